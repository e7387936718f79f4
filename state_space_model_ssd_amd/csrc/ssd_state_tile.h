// The bf16 chunk_state tile (internal): one (chunk, head) of the chunk_state
// stage, optionally with chunk_cumsum in front, as a device function shared
// by the chunk_state kernel, the fused front and the fused forward.
// ssd_chunk_state.hip describes the computation.
#pragma once

#include "ssd_device.h"

// Multiply-adds are fused into FMAs only inside one expression (not by the
// code generator across statements), so every kernel that inlines these
// bodies, whatever surrounds them, rounds exactly alike.
#pragma clang fp contract(on)

namespace ssd {
namespace {

// ------------------------------------------------------------- bf16 kernels
// Threads of the bf16 chunk_state and front workgroups (8 waves).
constexpr int kStateThreads = 512;

template <int P, int N, int L>
struct StateSmem {
  static constexpr int KS = 64;    // tokens per slice
  bf16 xs[KS * P];                 // weighted x slice, token-major, swizzled
  bf16 bs[KS * N];                 // B slice, token-major, swizzled
  float wl[L];
  float cum[L];
  float wave_tot[kStateThreads / 64];
};

// chunk_state for chunk j, head h (kStateThreads threads).  With CUMSUM the workgroup
// also runs chunk_cumsum for its (chunk, head) -- the step and its running
// sum come from dt here and are written to delta/dAcs for the later stages --
// otherwise it reads them from delta/dAcs.
//
// Each 64-token slice of x (scaled by w[l] in fp32 and rounded once to bf16)
// and of B is staged token-major in LDS; the MFMA operands come out through
// the transpose read.  The MFMAs produce the transposed tile S^T[n][p], so a
// lane holds four consecutive n of one p and S leaves in 16-byte stores.
// Loads and stores go through buffer resources bounded by the chunk: tokens
// past its end read as zeros.
//
// AUX: cache-policy bits of the stores of S, delta and dAcs (kSc1 when another
// workgroup of the same launch reads them).  OPQ: the body runs inside a
// persistent loop.
template <int P, int N, int L, bool CUMSUM, int AUX = 0, bool OPQ = false>
__device__ __forceinline__ void chunk_state_bf16_body(
    const ChunkDesc& d, int j, int h, const bf16* __restrict__ x, const bf16* __restrict__ B,
    float* __restrict__ delta, float* __restrict__ dAcs, const float* __restrict__ dt,
    const float* __restrict__ dt_bias, const float* __restrict__ A, float dt_min, float dt_max,
    int H, int G, float* __restrict__ S, StateSmem<P, N, L>& sm) {
  static_assert(L % 64 == 0 && L <= 256 && P % 16 == 0 && N % 16 == 0, "tile shape");
  using SM = StateSmem<P, N, L>;
  constexpr int KS = SM::KS;
  constexpr int XC = P / 8, BC = N / 8;   // 16-byte pieces per row
  constexpr int TH = kStateThreads, NWV = TH / 64;
  constexpr int XU = (KS * XC + TH - 1) / TH, BU = (KS * BC + TH - 1) / TH;
  constexpr int PT = P / 16, NT = N / 16;
  constexpr int WN = NT < 4 ? NT : 4;                       // waves along n
  constexpr int WP = (NWV / WN) < PT ? (NWV / WN) : PT;     // waves along p
  constexpr int TP = PT / WP, TN = NT / WN;
  static_assert(PT % WP == 0 && NT % WN == 0, "tile split");
  const int g = h / (H / G);
  const int tid = body_tid<OPQ, TH>(), w = wave_id(), lane = tid & 63;
  const int last = d.len - 1;
  const uint32_t HP = (uint32_t)H * P, GN = (uint32_t)G * N;
  const auto rx = buf_rsrc(x + ((int64_t)d.start * H + h) * P, ((uint32_t)last * HP + P) * 2u);
  const auto rb = buf_rsrc(B + ((int64_t)d.start * G + g) * N, ((uint32_t)last * GN + N) * 2u);

  uint4 xr[XU], br[BU];
  const int nsl = (d.len + KS - 1) / KS;
  // slice `sl` into registers (pieces past a thread's share, if any, read
  // out of range as zeros and are never staged)
#define SSD_STATE_FETCH(sl)                                                               \
  {                                                                                       \
    _Pragma("unroll") for (int u = 0; u < XU; ++u) {                                      \
      const int i = tid + TH * u, r = (sl) * KS + i / XC, c = i % XC;                     \
      xr[u] = buf_load16(rx, i < KS * XC ? ((uint32_t)r * HP + c * 8) * 2u : 0xFFFFFFF0u);  \
    }                                                                                     \
    _Pragma("unroll") for (int u = 0; u < BU; ++u) {                                      \
      const int i = tid + TH * u, r = (sl) * KS + i / BC, c = i % BC;                     \
      br[u] = buf_load16(rb, i < KS * BC ? ((uint32_t)r * GN + c * 8) * 2u : 0xFFFFFFF0u);  \
    }                                                                                     \
  }
  SSD_STATE_FETCH(0)                      // in flight while the weights are formed

  // w[l] = exp(a_last - a_l) * delta_l
  if constexpr (CUMSUM) {
    float step, cum;
    chunk_cumsum_block<L>(d, tid, dt, dt_bias, A, H, h, dt_min, dt_max, sm.wave_tot, step, cum);
    if (tid < L) {
      const int64_t o = ((int64_t)j * H + h) * L;
      buf_store4<AUX>(buf_rsrc(delta + o, L * 4), tid * 4, step);
      buf_store4<AUX>(buf_rsrc(dAcs + o, L * 4), tid * 4, cum);
      sm.cum[tid] = cum;
      sm.wl[tid] = step;
    }
    __syncthreads();
    if (tid < L) sm.wl[tid] = exp2_fast((sm.cum[last] - sm.cum[tid]) * kLog2e) * sm.wl[tid];
  } else {
    const float* dA = dAcs + ((int64_t)j * H + h) * L;
    const float* dl = delta + ((int64_t)j * H + h) * L;
    const float lastv = dA[last];
    for (int l = tid; l < L; l += TH)
      sm.wl[l] = (l < d.len) ? exp2_fast((lastv - dA[l]) * kLog2e) * dl[l] : 0.f;
  }

  const int wp = w / WN, wn = w - (w / WN) * WN;
  const bool active = w < WP * WN;
  f32x4 acc[TN][TP];                      // S^T tiles: rows n, columns p
#pragma unroll
  for (int b = 0; b < TN; ++b)
#pragma unroll
    for (int a = 0; a < TP; ++a) acc[b][a] = f32x4{0.f, 0.f, 0.f, 0.f};

  __syncthreads();                        // wl ready
  for (int sl = 0; sl < nsl; ++sl) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int i = tid + TH * u, r = i / XC, c = i % XC;
      if (i < KS * XC) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, xr[u]);
        const float wv = sm.wl[sl * KS + r];   // 0 past the chunk's end
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = static_cast<bf16>(static_cast<float>(v[e]) * wv);
        *reinterpret_cast<bf16x8*>(&sm.xs[tile_at<P>(r, c * 8)]) = o;
      }
    }
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int i = tid + TH * u, r = i / BC, c = i % BC;
      if (i < KS * BC) *reinterpret_cast<uint4*>(&sm.bs[tile_at<N>(r, c * 8)]) = br[u];
    }
    __syncthreads();
    if (sl + 1 < nsl) SSD_STATE_FETCH(sl + 1)   // in flight while this slice multiplies
    if (active) {
#pragma unroll
      for (int k0 = 0; k0 < KS; k0 += 32) {
        bf16x8 fa[TP], fb[TN];
#pragma unroll
        for (int a = 0; a < TP; ++a) fa[a] = lds_operand_sw<P>(sm.xs, k0, 16 * (wp * TP + a), lane);
#pragma unroll
        for (int b = 0; b < TN; ++b) fb[b] = lds_operand_sw<N>(sm.bs, k0, 16 * (wn * TN + b), lane);
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int a = 0; a < TP; ++a) acc[b][a] = Mfma<bf16>::mma(fb[b], fa[a], acc[b][a]);
      }
    }
    __syncthreads();
  }
#undef SSD_STATE_FETCH

  if (!active) return;
  const auto rs = buf_rsrc(S + ((int64_t)j * H + h) * P * N, P * N * 4);
  const int lr = lane & 15;
#pragma unroll
  for (int b = 0; b < TN; ++b)
#pragma unroll
    for (int a = 0; a < TP; ++a) {
      const int p = 16 * (wp * TP + a) + lr;
      const int n = 16 * (wn * TN + b) + (lane >> 4) * 4;
      buf_store16<AUX>(rs, ((uint32_t)p * N + n) * 4u, __builtin_bit_cast(uint4, acc[b][a]));
    }
}

}  // namespace
}  // namespace ssd

#pragma clang fp contract(fast)
