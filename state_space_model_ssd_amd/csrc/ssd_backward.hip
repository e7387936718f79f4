// The SSD backward: gradients of loss = sum(y * dy) + sum(final * dfinal)
// with respect to x, dt, dt_bias, A, B, C, D and the initial states (the
// layer's backward kernels listed next to the forward ones: clova.ai, table
// "Share of compute time by kernel": _chunk_scan_bwd_dx, _chunk_state_bwd_db,
// _state_passing_bwd, _chunk_scan_bwd_dstates, ...).
//
// The forward's stages 0-4 run first (delta, the running sums a, CB and the
// states entering each chunk, H).  Then, per chunk j, head h (tokens l, s of
// the chunk, a_last the running sum at its last token, E[l,s] = exp(a_l -
// a_s) for s <= l):
//   1. Q_j[p,n]  = sum_l exp(a_l) dy[l,p] C[l,n]          (dloss/dH via y)
//   2. reverse chain per sequence: G = dfinal; for j from the last chunk
//      down: dS_j = G; G = exp(a_last_j) G + Q_j; then dinit = G.  dS_j is
//      the gradient of the state leaving chunk j.
//   3. per token, with U[l,s] = dy_l . x_s and dCB[l,s] = E[l,s] delta_s U[l,s]:
//      dx_s     = delta_s sum_{l>=s} CB[l,s] E[l,s] dy_l
//                 + delta_s exp(a_last - a_s) dS_j B_s + D dy_s
//      ddelta_s = sum_{l>=s} CB[l,s] E[l,s] U[l,s] + exp(a_last - a_s) B_s.(x_s dS_j)
//      da_l     = sum_{s<=l} CB dCB[l,.] - sum_{l'>=l} CB dCB[.,l]   (intra)
//                 + exp(a_l) C_l . (dy_l H)                            (inter)
//                 - delta_l exp(a_last - a_l) B_l.(x_l dS_j)           (state)
//      plus, at the last token, sum_s delta_s exp(a_last - a_s) B_s.(x_s dS_j)
//      + exp(a_last) <dS_j, H>; then a = cumsum(delta A) gives
//      ddelta_k += A sum_{l>=k} da_l and dA += sum_k delta_k sum_{l>=k} da_l,
//      and ddt = ddelta softplus'(dt + dt_bias) where the clamp passes it.
//   4. per group g (B and C are shared by its heads, so the intra-chunk
//      parts contract dCB summed over the heads, once per group, and the
//      state terms are one contraction over (head, p)):
//      dC[l] = sum_{s<=l} (sum_h dCB_h[l,s]) B_s + sum_h exp(a_l) dy_l H,
//      dB[s] = sum_{l>=s} (sum_h dCB_h[l,s]) C_l
//              + sum_h delta_s exp(a_last - a_s) x_s dS_j;
//   5. dA, dD and dt_bias: sums over chunks.
// Everything accumulates in fp32; dx, dB and dC are rounded once to x's
// dtype.  Deterministic: fixed loop orders, no atomics.
//
// Launches: Q tiles (1, and each chunk's log-decay) -> reverse chain (2,
// and <dS_j, H_j> in pieces) -> V tiles (3's intra sums, dCB summed over
// head blocks) -> head-block sum of dCB -> dB/dC per group (4, and the inter
// and state row dots of da per head) -> per-token pass (3's da, ddelta,
// ddt) -> dx (with bf16 inputs it also does 5; with fp32 inputs a per-head
// sum launch follows).
//
// The contractions are 64 x 64 output tiles.  With bf16 inputs they run on
// the bf16 MFMA: a head's rows staged in LDS from whole-line loads, or
// k-major slices read with the gfx950 transpose read; an operand that is
// scaled or fp32 is rounded to bf16 once, and row factors are applied to
// the product where they can be.  Loops over heads or token slices load the
// next step's operands while the current one is multiplied, with buffer
// loads issued without branches (a branch around a load or store makes the
// compiler wait for every outstanding load at the loop's head).  The fp32
// path uses fp32 tiles on the vector ALUs, staged through LDS with 16-byte
// loads.
#include "ssd_kernels.h"
#include "ssd_scan_tile.h"

namespace ssd {

namespace {

constexpr int kBwdThreads = 256;
// Largest |a_last| log2(e) of a chunk for which dx factors its decay
// exp(a_l - a_s) into exp(a_l) exp(-a_s): both stay far inside fp32.
constexpr float kBwdFastMaxLog2 = 64.f;
// Most blocks a group's heads are split into for the summed dCB and the
// dB/dC state terms.  More blocks: more workgroups in 3a and 4a, but more
// partial sums written there and read in 3b' and 4b; the launcher takes the
// fewest that give kBwdMinWgPerCu workgroups per CU (three: V 30.7 -> 28.7
// us on the Mamba-2 layer shape against 0.9 us more in the dCB sum and dB/dC;
// four gain nothing in V).
constexpr int kBwdHeadBlocks = 8;
constexpr int kBwdMinWgPerCu = 3;

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return to_f32(*p); }

// 64 x 64 fp32 tiles on the vector ALUs (the fp32 path): operand slices
// staged in LDS as S[k * kGemmPitch + i], 4 x 4 outputs per thread of 256.
constexpr int kGemmPitch = 68;

template <typename T>
__device__ __forceinline__ void load16_f32(const T* p, bool ok, float* v);
template <>
__device__ __forceinline__ void load16_f32<float>(const float* p, bool ok, float* v) {
  const float4 t = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}

// One KS-long slice (k in [kb, kb + KS)) of a 64-wide GEMM operand staged in
// LDS as S[k * kGemmPitch + i], read from memory rows with 16-byte loads.
// KCONTIG: element (i, k) is at p[i * stride + k] (a row per i, k
// contiguous); otherwise at p[k * stride + i] (a row per k, i contiguous).
// Elements with i >= ni or k >= k1 are 0 (a piece that straddles either
// bound must still lie inside the buffer).  TRI keeps only k <= i + ioff
// (1) or k >= i + ioff (2).  scale (LDS, or null for 1): each stored row is
// multiplied by scale[row], row = i (KCONTIG) or k.
template <typename T, bool KCONTIG, int KS, int TRI = 0>
__device__ __forceinline__ void stage_slice(const T* p, int64_t stride, int ni, int kb, int k1,
                                            const float* scale, float* S, int ioff = 0) {
  constexpr int V = 16 / sizeof(T);
  static_assert(KS % V == 0 && 64 % V == 0, "piece size");
  auto keep = [&](int i, int k) {
    return i < ni && k < k1 && (TRI == 0 || (TRI == 1 ? k <= i + ioff : k >= i + ioff));
  };
  if constexpr (KCONTIG) {
    for (int t = threadIdx.x; t < 64 * (KS / V); t += kBwdThreads) {
      const int r = t & 63, c = (t >> 6) * V;   // consecutive threads: consecutive rows
      const bool ok = r < ni && kb + c < k1;
      float v[V];
      load16_f32<T>(p + r * stride + kb + c, ok, v);
      const float sc = (scale && ok) ? scale[r] : 1.f;
#pragma unroll
      for (int e = 0; e < V; ++e)
        S[(c + e) * kGemmPitch + r] = keep(r, kb + c + e) ? (scale ? sc * v[e] : v[e]) : 0.f;
    }
  } else {
    constexpr int PR = 64 / V;             // pieces per row
    for (int t = threadIdx.x; t < KS * PR; t += kBwdThreads) {
      const int kr = t / PR, c = (t - kr * PR) * V;
      const bool ok = kb + kr < k1 && c < ni;
      float v[V];
      load16_f32<T>(p + (int64_t)(kb + kr) * stride + c, ok, v);
      const float sc = (scale && ok) ? scale[kb + kr] : 1.f;
#pragma unroll
      for (int e = 0; e < V; ++e)
        S[kr * kGemmPitch + c + e] = keep(c + e, kb + kr) ? (scale ? sc * v[e] : v[e]) : 0.f;
    }
  }
}

// acc += A B over k in [k0, k1) for a 64 x 64 tile, both operands staged
// per slice by stage_slice (A's i = m, B's i = n; TRI and ioff mask A).
template <typename TA, bool AK, typename TB, bool BK, int KS = 32, int TRI = 0>
__device__ __forceinline__ void gemm_staged(const TA* pa, int64_t sa, int na, const float* scale_a,
                                            const TB* pb, int64_t sb, int nb, int k0, int k1,
                                            float (&acc)[4][4], float* As, float* Bs, int ioff = 0) {
  const int tid = threadIdx.x;
  const int tm = (tid >> 4) * 4, tn = (tid & 15) * 4;
  for (int kb = k0; kb < k1; kb += KS) {
    __syncthreads();                       // previous slice consumed (and the caller's staging done)
    stage_slice<TA, AK, KS, TRI>(pa, sa, na, kb, k1, scale_a, As, ioff);
    stage_slice<TB, BK, KS>(pb, sb, nb, kb, k1, nullptr, Bs);
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < KS; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&As[k * kGemmPitch + tm]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[k * kGemmPitch + tn]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[i][jn] += av[i] * bv[jn];
    }
  }
}

// bf16 MFMA tiles (16x16x32, fp32 sums) for 64 x 64 outputs: each of the 4
// waves computes a 32 x 32 quarter d[mi][ni] (rows wr + 16 mi + 4 (lane/16)
// + r, columns wc + 16 ni + lane%16); quarter_to_thread then moves the tile
// through LDS into the 4 x 4 block of the vector epilogues.
struct MfmaQuarter {
  int lane, wr, wc, lr, kq;
  __device__ __forceinline__ MfmaQuarter() {
    const int w = wave_id();
    lane = threadIdx.x & (kWave - 1);
    wr = (w >> 1) * 32;
    wc = (w & 1) * 32;
    lr = lane & 15;
    kq = (lane >> 4) * 8;
  }
  // row (column) of d[mi][ni][r] within the tile
  __device__ __forceinline__ int row(int mi, int r) const { return wr + mi * 16 + (lane >> 4) * 4 + r; }
  __device__ __forceinline__ int col(int ni) const { return wc + ni * 16 + lr; }
};

__device__ __forceinline__ void zero_quarter(f32x4 (&d)[2][2]) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) d[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// 16 bytes at byte offset off of a buffer resource, or zeros when !ok.  The
// load is issued whatever ok is (the offset of a lane without data lies
// past the resource's records, which reads zeros), so no branch surrounds
// it and the wait before its use counts only the loads issued after it:
// software-pipelined loops keep their prefetches in flight.  Resources of
// these loads are under 2 GiB.
constexpr uint32_t kPastRecords = 0x80000000u;

// A value every lane reads from the same address, loaded through the vector
// memory path.  As a scalar load it would be waited for with lgkmcnt, which
// the LDS accesses share and which scalar loads decrement out of order: the
// wait for any LDS store before a barrier would then wait for a prefetch of
// the next iteration's value too.  A vector load is counted in order with
// the other prefetches.
__device__ __forceinline__ float ld_vmem(const float* p) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(p, 4), 0u, 0, 0));
}
// A buffer resource whose base and size are the workgroup's (read from the
// first lane): the compiler cannot always prove a workgroup-wide address
// uniform, and a resource it takes for a per-lane value makes it loop over
// the distinct values around every access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_u(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return buf_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
}

// A store that every lane issues; lanes without !ok aim past the resource's
// records, where the store is dropped.  Stores count in the same wait as
// loads, so a store under a branch would also blur the waits of a
// software-pipelined loop.
__device__ __forceinline__ void store_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, float v, bool ok) {
  buf_store4(r, ok ? off : kPastRecords, v);
}
__device__ __forceinline__ bf16x8 frag_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok = true) {
  return __builtin_bit_cast(bf16x8, buf_load16(r, ok ? off : kPastRecords));
}

// The quarters of the waves into acc[i][jn] (tile row tm + i, column tn + jn)
// through LDS: rows 0-31 in lo, 32-63 in hi (32 x kGemmPitch floats each).
// Begins and ends with a barrier.
__device__ __forceinline__ void quarter_to_thread(const MfmaQuarter& q, const f32x4 (&d)[2][2],
                                                  float (&acc)[4][4], float* lo, float* hi) {
  __syncthreads();                         // lo and hi free
  float* dst = q.wr == 0 ? lo : hi;        // wave-uniform
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dst[(q.row(mi, r) & 31) * kGemmPitch + q.col(ni)] = d[mi][ni][r];
  __syncthreads();
  const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
  const float* src = tm < 32 ? lo : hi;    // wave-uniform
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(&src[((tm + i) & 31) * kGemmPitch + tn]);
    acc[i][0] = v.x; acc[i][1] = v.y; acc[i][2] = v.z; acc[i][3] = v.w;
  }
}

// d += A B over the 32-long k-slice held in LDS as k-major bf16 tiles
// at[k * kKtPitch + m] and bt[k * kKtPitch + n] (read by transpose reads).
constexpr int kKtPitch = 80;               // 160-byte rows: a transpose read's 16 lanes hit distinct banks
__device__ __forceinline__ void mfma_kmajor(const MfmaQuarter& q, const bf16* at, const bf16* bt,
                                            f32x4 (&d)[2][2]) {
  using M = Mfma<bf16>;
  bf16x8 a[2], b[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) a[mi] = lds_operand_kmajor(at, kKtPitch, 0, q.wr + mi * 16, q.lane);
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) b[ni] = lds_operand_kmajor(bt, kKtPitch, 0, q.wc + ni * 16, q.lane);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) d[mi][ni] = M::mma(a[mi], b[ni], d[mi][ni]);
}

// Lower-triangular tile index t -> (row tile, column tile <= row tile).
__device__ __forceinline__ int2 lower_tile(int t) {
  int r = 0;
  while (t > r) {
    t -= r + 1;
    ++r;
  }
  return make_int2(r, t);
}

// Sum of v over the 16 threads that share a row of the 4 x 4 blocks (lanes
// differing in their low 4 bits); every one of them gets it.
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Sums over lanes by DPP (a data-parallel move folded into the add: no LDS
// traffic).  dpp_add(v, CTRL, ROWS) adds to v the value that lane pattern
// CTRL reads, in the rows (16-lane groups) of mask ROWS; other rows add 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}
// The sum over each row of 16 lanes, in every lane of the row: neighbours
// in pairs (quad_perm 1,0,3,2), pairs of pairs (quad_perm 2,3,0,1), then the
// half-row and row mirrors.
__device__ __forceinline__ float row_sum16(float v) {
  v = dpp_add<0xb1>(v);
  v = dpp_add<0x4e>(v);
  v = dpp_add<0x141>(v);
  return dpp_add<0x140>(v);
}
// Eight sums over each row of 16 lanes at once: the v[i] (i < 8) of the
// row's lanes are added, and lane lr ends with the sum of v[4 (lr >> 3) +
// 2 ((lr >> 2) & 1) + ((lr >> 1) & 1)] (lanes lr and lr ^ 1 hold the same
// one).  Each step pairs the lanes (rotation by 8, half-row mirror, then
// quad_perm 2,3,0,1): a lane keeps half of its values and adds its
// partner's copy of that half.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16_x8(const float (&v)[8], int lr) {
  const bool u8 = lr & 8, u4 = lr & 4, u2 = lr & 2;
  float a[4], b[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = (u8 ? v[4 + k] : v[k]) + dpp_mov<0x128>(u8 ? v[k] : v[4 + k]);
#pragma unroll
  for (int k = 0; k < 2; ++k) b[k] = (u4 ? a[2 + k] : a[k]) + dpp_mov<0x141>(u4 ? a[k] : a[2 + k]);
  const float c = (u2 ? b[1] : b[0]) + dpp_mov<0x4e>(u2 ? b[0] : b[1]);
  return c + dpp_mov<0xb1>(c);
}

// The sum over the wave, in lane 63: the row sums, then row 15's and row
// 31's broadcasts into the rows after them.
__device__ __forceinline__ float wave_sum_last(float v) {
  v = row_sum16(v);
  v = dpp_add<0x142, 0xa>(v);
  return dpp_add<0x143, 0xc>(v);
}

// 1. Q_j[p,n] = sum_l exp(a_l) dy[l,p] C[l,n] as 64 x 64 tiles, and the
// chunk's log-decay a_last for the reverse chain (0 for an empty chunk:
// decay 1), dla[j][h]; grid: xcd_grid(chunk slots, ceil(P/64) * ceil(N/64)
// * H), every tile and head of a chunk on the XCD of that chunk.
template <typename T, int P, int N, int L>
__global__ __launch_bounds__(kBwdThreads) void bwd_q_tiled_kernel(
    ChunkMap cm, int nslots, const T* __restrict__ dy, const T* __restrict__ C,
    const float* __restrict__ dAcs, int H, int G, float* __restrict__ Q, float* __restrict__ dla) {
  __shared__ __align__(16) float As[32 * kGemmPitch], Bs[32 * kGemmPitch];
  __shared__ float sc[L];
  constexpr int NT = (N + 63) / 64;
  constexpr int NX = ((P + 63) / 64) * NT;
  const int2 ci = xcd_chunk_head(blockIdx.x, NX * H);
  if (ci.x >= nslots) return;
  const int bx = ci.y % NX;
  const int m0 = (bx / NT) * 64, n0 = (bx % NT) * 64;
  const int h = ci.y / NX, j = ci.x, g = h / (H / G);
  const ChunkDesc cd = cm.desc(j);
  const int64_t jh = (int64_t)j * H + h;
  for (int l = threadIdx.x; l < L; l += kBwdThreads) sc[l] = exp2_fast(dAcs[jh * L + l] * kLog2e);
  if (bx == 0 && threadIdx.x == 0) dla[jh] = cd.len > 0 ? dAcs[jh * L + cd.len - 1] : 0.f;
  __syncthreads();
  if constexpr (sizeof(T) == 2) {
    // bf16 MFMA over slices of 32 tokens l: exp(a_l) dy_l (rounded once) and
    // C_l staged k-major in LDS
    __shared__ __align__(16) bf16 yt[32 * kKtPitch], ct[32 * kKtPitch];
    static_assert(32 * 8 == kBwdThreads, "one 8-wide piece of each slice tile per thread");
    const MfmaQuarter q;
    f32x4 d[2][2];
    zero_quarter(d);
    const int len = max(cd.len, 0), kr = threadIdx.x >> 3, c = (threadIdx.x & 7) * 8;
    // the next slice's rows are loaded while the current one is multiplied
    // (buffer loads without a branch: tokens past the chunk read zeros)
    const __amdgpu_buffer_rsrc_t rdy =
        buf_rsrc_u(dy + (int64_t)cd.start * H * P, (uint32_t)((int64_t)len * H * P * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rc =
        buf_rsrc_u(C + (int64_t)cd.start * G * N, (uint32_t)((int64_t)len * G * N * sizeof(T)));
    bf16x8 yv, cv;
    auto fetch = [&](int kb) {
      const int l = kb + kr;
      yv = frag_buf(rdy, (uint32_t)(((l * H + h) * P + m0 + c) * sizeof(T)), m0 + c < P);
      cv = frag_buf(rc, (uint32_t)(((l * G + g) * N + n0 + c) * sizeof(T)), n0 + c < N);
    };
    if (len > 0) fetch(0);
    for (int kb = 0; kb < len; kb += 32) {
      const int l = kb + kr;
      const float f = l < len ? sc[l] : 0.f;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = f * static_cast<float>(yv[e]);
      const bf16x8 ccur = cv;
      fetch(kb + 32);                      // past the chunk: zeros
      __syncthreads();                     // previous slice consumed
      *reinterpret_cast<bf16x8*>(&yt[kr * kKtPitch + c]) = Mfma<bf16>::pack(v);
      *reinterpret_cast<bf16x8*>(&ct[kr * kKtPitch + c]) = ccur;
      __syncthreads();
      mfma_kmajor(q, yt, ct, d);
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = m0 + q.row(mi, r), n = n0 + q.col(ni);
          if (p < P && n < N) Q[(jh * P + p) * N + n] = d[mi][ni][r];
        }
  } else {
    float acc[4][4] = {};
    // rows l of dy (columns p, scaled by exp(a_l)) and of C (columns n)
    gemm_staged<T, false, T, false>(dy + ((int64_t)cd.start * H + h) * P + m0, (int64_t)H * P, P - m0, sc,
                                    C + ((int64_t)cd.start * G + g) * N + n0, (int64_t)G * N, N - n0, 0,
                                    max(cd.len, 0), acc, As, Bs);
    const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        const int p = m0 + tm + i, n = n0 + tn + jn;
        if (p < P && n < N) Q[(jh * P + p) * N + n] = acc[i][jn];
      }
  }
}

// 1, bf16 inputs: one workgroup per (chunk, head, 64 rows p) computes all
// N columns, so the chunk's dy rows are loaded and scaled once: wave w holds
// rows 32 (w / 2) .. of columns 64 (w % 2) .. (2 x 4 MFMA tiles).  Slices
// of 32 tokens l: exp(a_l) dy_l (rounded once) and C_l staged k-major in LDS,
// the next slice's rows loaded while the current one is multiplied.
template <int P, int N, int L>
__global__ __launch_bounds__(kBwdThreads) void bwd_q_mfma_kernel(
    ChunkMap cm, int nslots, const bf16* __restrict__ dy, const bf16* __restrict__ C,
    const float* __restrict__ dAcs, int H, int G, float* __restrict__ Q, float* __restrict__ dla) {
  constexpr int PT = (P + 63) / 64;
  constexpr int NT = (N + 63) / 64;
  static_assert(NT <= 2, "one or two 64-column halves");
  __shared__ float sc[L];
  __shared__ __align__(16) bf16 yt[32 * kKtPitch], ct[NT][32 * kKtPitch];
  const int2 ci = xcd_chunk_head(blockIdx.x, PT * H);
  if (ci.x >= nslots) return;
  const int pt = ci.y % PT, m0 = pt * 64;
  const int h = ci.y / PT, j = ci.x, g = h / (H / G);
  const ChunkDesc cd = cm.desc(j);
  const int64_t jh = (int64_t)j * H + h;
  for (int l = threadIdx.x; l < L; l += kBwdThreads) sc[l] = exp2_fast(dAcs[jh * L + l] * kLog2e);
  if (pt == 0 && threadIdx.x == 0) dla[jh] = cd.len > 0 ? dAcs[jh * L + cd.len - 1] : 0.f;
  __syncthreads();
  static_assert(32 * 8 == kBwdThreads, "one 8-wide piece of each slice tile per thread");
  const int lane = threadIdx.x & (kWave - 1), w = wave_id();
  const int wr = (w >> 1) * 32, half = w & 1;
  const int len = max(cd.len, 0), kr = threadIdx.x >> 3, c = (threadIdx.x & 7) * 8;
  const __amdgpu_buffer_rsrc_t rdy =
      buf_rsrc_u(dy + (int64_t)cd.start * H * P, (uint32_t)((int64_t)len * H * P * sizeof(bf16)));
  const __amdgpu_buffer_rsrc_t rc =
      buf_rsrc_u(C + (int64_t)cd.start * G * N, (uint32_t)((int64_t)len * G * N * sizeof(bf16)));
  f32x4 d[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) d[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 yv, cv[NT];
  auto fetch = [&](int kb) {
    const int l = kb + kr;
    yv = frag_buf(rdy, (uint32_t)(((l * H + h) * P + m0 + c) * sizeof(bf16)), m0 + c < P);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      cv[t] = frag_buf(rc, (uint32_t)(((l * G + g) * N + 64 * t + c) * sizeof(bf16)), 64 * t + c < N);
  };
  if (len > 0) fetch(0);
  for (int kb = 0; kb < len; kb += 32) {
    const int l = kb + kr;
    const float f = l < len ? sc[l] : 0.f;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f * static_cast<float>(yv[e]);
    bf16x8 ccur[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) ccur[t] = cv[t];
    fetch(kb + 32);                        // past the chunk: zeros
    __syncthreads();                       // previous slice consumed
    *reinterpret_cast<bf16x8*>(&yt[kr * kKtPitch + c]) = Mfma<bf16>::pack(v);
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<bf16x8*>(&ct[t][kr * kKtPitch + c]) = ccur[t];
    __syncthreads();
    if (half < NT) {                       // wave-uniform: N = 64 leaves the second half idle
      bf16x8 a[2], b[4];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) a[mi] = lds_operand_kmajor(yt, kKtPitch, 0, wr + mi * 16, lane);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) b[ni] = lds_operand_kmajor(ct[half], kKtPitch, 0, ni * 16, lane);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) d[mi][ni] = Mfma<bf16>::mma(a[mi], b[ni], d[mi][ni]);
    }
  }
  if (half >= NT) return;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = m0 + wr + mi * 16 + 4 * lg + r, n = 64 * half + ni * 16 + lr;
        if (p < P && n < N) Q[(jh * P + p) * N + n] = d[mi][ni][r];
      }
}

// Four consecutive values rounded once to T (8- or 16-byte store).
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)__builtin_bit_cast(unsigned short, static_cast<bf16>(a)) |
                      ((uint32_t)__builtin_bit_cast(unsigned short, static_cast<bf16>(b)) << 16);
  const uint32_t hi = (uint32_t)__builtin_bit_cast(unsigned short, static_cast<bf16>(c)) |
                      ((uint32_t)__builtin_bit_cast(unsigned short, static_cast<bf16>(d)) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

// Four consecutive values of T as fp32 (8- or 16-byte load).
__device__ __forceinline__ float4 load4_f32(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4_f32(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// 2. Reverse chain, four consecutive state elements per thread (16-byte
// loads and stores).  Alongside, the dot <dS_j, H_j> of the gradient leaving
// chunk j with the state entering it (the chunk's last token's da needs
// it), as one partial sum per wave (256 state elements): ghpart[j][h][PN /
// 256].  dS in fp32 is written only where dS32 is given (the fp32 path's
// operands).  A ring of D register sets holds the Q piece, entering state
// and log-decay of the next D chunks: every load is a vector load issued
// without a branch, so the wait before a set's use leaves the other sets'
// loads in flight.  grid (ceil(P*N / 1024), H, nstates).
template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_chain_kernel(
    ChunkMap cm, const float* __restrict__ Q, const float* __restrict__ dla,
    const float* __restrict__ dfinal, const T* __restrict__ states_in, int H, int PN,
    float* __restrict__ dS32, bf16* __restrict__ dS16, float* __restrict__ ghpart,
    float* __restrict__ dinit) {
  const int e = (blockIdx.x * kBwdThreads + threadIdx.x) * 4;
  if (e >= PN) return;                     // PN is a multiple of 256: whole waves
  const int h = blockIdx.y, s = blockIdx.z, wv = e / (4 * kWave), nw = PN / (4 * kWave);
  const int2 r = cm.seq_range(s);
  float4 g = dfinal ? *reinterpret_cast<const float4*>(dfinal + ((int64_t)s * H + h) * PN + e)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  if (r.y > r.x) {
    float4 q[D], hv[D];
    float la[D];
    auto loads = [&](int set, int j) {
      const int64_t jh = (int64_t)j * H + h;
      q[set] = *reinterpret_cast<const float4*>(Q + jh * PN + e);
      hv[set] = load4_f32(states_in + jh * PN + e);
      la[set] = ld_vmem(dla + jh);
    };
    // chunk j with set's values; then (REFILL) chunk j - D's loads into the set
    auto step = [&](int set, int j, auto refill) {
      const int64_t jh = (int64_t)j * H + h;
      const float4 qj = q[set], hj = hv[set];
      const float dec = expf(la[set]);
      if constexpr (decltype(refill)::value) loads(set, max(j - D, r.x));   // before the start: its first chunk
      if (dS32) *reinterpret_cast<float4*>(dS32 + jh * PN + e) = g;
      if (dS16) store4(dS16 + jh * PN + e, g.x, g.y, g.z, g.w);   // rounded once, for the MFMA operands
      const float gh = wave_sum_last(g.x * hj.x + g.y * hj.y + g.z * hj.z + g.w * hj.w);
      if ((threadIdx.x & (kWave - 1)) == kWave - 1) ghpart[jh * nw + wv] = gh;
      g = make_float4(dec * g.x + qj.x, dec * g.y + qj.y, dec * g.z + qj.z, dec * g.w + qj.w);
    };
#pragma unroll
    for (int u = 0; u < D; ++u) {          // chunks r.y - 1, r.y - 2, .. in sets 0, 1, ..
      loads(u, max(r.y - 1 - u, r.x));
      __builtin_amdgcn_sched_barrier(0);   // the sets' loads in the order they are used
    }
    int j = r.y - 1;
    for (; j - (D - 1) >= r.x; j -= D) {   // whole rounds of the ring: every path issues the same loads
#pragma unroll
      for (int u = 0; u < D; ++u) {
        step(u, j - u, std::true_type{});
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < D - 1; ++u)        // the last chunks (fewer than D): nothing left to load
      if (j - u >= r.x) step(u, j - u, std::false_type{});   // uniform over the workgroup
  }
  if (dinit) *reinterpret_cast<float4*>(dinit + ((int64_t)s * H + h) * PN + e) = g;
}

// dinit = dfinal (or 0) when there are no chunks.
__global__ __launch_bounds__(kBwdThreads) void bwd_pass_final_kernel(const float* __restrict__ dfinal,
                                                                     int64_t n, float* __restrict__ dinit) {
  const int64_t i = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  if (i < n) dinit[i] = dfinal ? dfinal[i] : 0.f;
}

// Three sums over the workgroup (L threads, L a multiple of 64) at once;
// every thread gets them.
template <int L>
__device__ __forceinline__ float3 block_sum3(float3 v, float* red) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    v.x += __shfl_xor(v.x, off);
    v.y += __shfl_xor(v.y, off);
    v.z += __shfl_xor(v.z, off);
  }
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[3 * (threadIdx.x / kWave)] = v.x;
    red[3 * (threadIdx.x / kWave) + 1] = v.y;
    red[3 * (threadIdx.x / kWave) + 2] = v.z;
  }
  __syncthreads();
  float3 t = make_float3(0.f, 0.f, 0.f);
#pragma unroll
  for (int w = 0; w < L / kWave; ++w) {
    t.x += red[3 * w];
    t.y += red[3 * w + 1];
    t.z += red[3 * w + 2];
  }
  return t;
}

// Inclusive suffix sum over the workgroup (L threads): thread k gets the sum
// of v over threads k .. L-1.  wred: L / kWave floats of LDS.
template <int L>
__device__ __forceinline__ float block_suffix_sum(float v, float* wred) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float u = __shfl_down(v, off);
    if (lane + off < kWave) v += u;
  }
  __syncthreads();
  if (lane == 0) wred[w] = v;              // the wave's total
  __syncthreads();
#pragma unroll
  for (int w2 = L / kWave - 1; w2 > 0; --w2)
    if (w2 > w) v += wred[w2];
  return v;
}

// 16 bytes of T as fp32 values.
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& u, float* v);
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& u, float* v) {
  v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
  v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
}

// 3a. For each head, V[l,s] = exp(a_l - a_s) (dy_l . x_s) for s <= l as
// 64 x 64 tiles on or below the diagonal, with each tile's partial sums
//   rowpart[st][l] = sum_s CB[l,s] delta_s V[l,s]   (s in column tile st)
//   colpart[lt][s] = sum_l CB[l,s] V[l,s]           (l in row tile lt),
// and dCB[l,s] = delta_s V[l,s] summed over a block of the group's heads:
// B and C are shared by the group, so dB and dC need dCB only summed over
// its heads.  Workgroup (lt, st, g, hb) walks the heads of block hb of group
// g (HB blocks per group) and writes that block's sum to dcbp[j][g][hb].
// grid: xcd_grid(chunk slots, (L/64)(L/64 + 1)/2 * G * HB), the tiles on or
// below the diagonal, every tile and head block of a chunk on its XCD.
template <typename T, int P, int N, int L>
__global__ __launch_bounds__(kBwdThreads) void bwd_v_tiled_kernel(
    ChunkMap cm, int nslots, const T* __restrict__ x, const T* __restrict__ dy, const T* __restrict__ cb,
    const float* __restrict__ delta, const float* __restrict__ dAcs, int H, int G, int HB,
    float* __restrict__ dcbp, float* __restrict__ rowpart, float* __restrict__ colpart,
    float* __restrict__ ddot) {
  __shared__ __align__(16) float As[32 * kGemmPitch], Bs[32 * kGemmPitch];
  __shared__ float cpart[16][64];
  // the head's running sums at the tile's rows and columns and its steps at
  // the columns (fac[3] repeats fac[2]: every thread loads one value)
  __shared__ __align__(16) float fac[4][64];
  float* al = fac[0];
  float* as = fac[1];
  float* dls = fac[2];
  constexpr int LT = L / 64;
  constexpr int NX = LT * (LT + 1) / 2;   // tiles on or below the diagonal
  const int2 ci = xcd_chunk_head(blockIdx.x, NX * G * HB);
  if (ci.x >= nslots) return;
  const int2 tt = lower_tile(ci.y % NX);
  // the tile is the workgroup's: read it as one value (buffer resources
  // built from it must be uniform)
  const int lt = __builtin_amdgcn_readfirstlane(tt.x), st = __builtin_amdgcn_readfirstlane(tt.y);
  const int by = ci.y / NX;
  const int g = by / HB, hb = by - (by / HB) * HB, j = ci.x;
  const int hpg = H / G, h0 = g * hpg + hb * hpg / HB, h1 = g * hpg + (hb + 1) * hpg / HB;
  const ChunkDesc cd = cm.desc(j);
  const int len = max(cd.len, 0);
  const int l0 = lt * 64, s0 = st * 64;
  if (l0 >= len) return;
  const int64_t t0 = cd.start;
  const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
  const T* cbj = cb + ((int64_t)j * G + g) * L * L;
  // this thread's 4 x 4 block of the CB tile, the same for every head (rows
  // past the chunk are read but never used)
  float cbr[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = load4_f32(cbj + (int64_t)(l0 + tm + i) * L + s0 + tn);
    cbr[i][0] = v.x; cbr[i][1] = v.y; cbr[i][2] = v.z; cbr[i][3] = v.w;
  }
  float w[4][4] = {};                      // this block's sum of delta_s V[l,s]
  // The next head's loads are issued before the current head's product and
  // wait in registers: its factor value (one per thread) and, for bf16, its
  // MFMA fragments of the dy and x rows (buffer loads: rows past the chunk
  // read zeros).  Every load and store in the loop is issued without a
  // branch, so the waits leave the prefetch in flight.
  const int fk = threadIdx.x >> 6, fi = threadIdx.x & 63;
  auto fac_src = [&](int h) -> const float* {
    const int64_t jh = (int64_t)j * H + h;
    return fk == 0 ? dAcs + jh * L + l0 + fi : fk == 1 ? dAcs + jh * L + s0 + fi : delta + jh * L + s0 + fi;
  };
  constexpr int KS = P / 32 > 0 ? P / 32 : 1;
  const MfmaQuarter q;
  const __amdgpu_buffer_rsrc_t rdy =
      buf_rsrc_u(dy + (t0 + l0) * H * P, (uint32_t)((int64_t)(len - l0) * H * P * sizeof(T)));
  const __amdgpu_buffer_rsrc_t rx =
      buf_rsrc_u(x + (t0 + s0) * H * P, (uint32_t)((int64_t)(len - s0) * H * P * sizeof(T)));
  bf16x8 fa[KS][2], fb[KS][2];
  float fv;
  auto fetch = [&](int h) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = q.wr + u * 16 + q.lr, c = q.wc + u * 16 + q.lr;
          fa[ks][u] = frag_buf(rdy, (uint32_t)(((r * H + h) * P + ks * 32 + q.kq) * sizeof(T)));
          fb[ks][u] = frag_buf(rx, (uint32_t)(((c * H + h) * P + ks * 32 + q.kq) * sizeof(T)));
        }
    }
    fv = *fac_src(h);
  };
  // a head's fragments and factor move from the prefetch registers at the
  // end of the previous head (a point the loop reaches only from its body,
  // so the wait there counts this head's loads exactly)
  bf16x8 a[KS][2], b[KS][2];
  auto take = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        a[ks][u] = fa[ks][u];
        b[ks][u] = fb[ks][u];
      }
    fac[fk][fi] = fv;                      // the previous head's reads ended at its last barrier
  };
  fetch(h0);
  take();
  for (int h = h0; h < h1; ++h) {
    const int64_t jh = (int64_t)j * H + h;
    float acc[4][4] = {};
    if constexpr (sizeof(T) == 2) {        // dy_l . x_s: bf16 rows, exact products on MFMA
      static_assert(P % 32 == 0, "k-steps of the rows");
      fetch(min(h + 1, h1 - 1));           // past the block's last head: that head again
      f32x4 d[2][2];
      zero_quarter(d);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) d[mi][ni] = Mfma<bf16>::mma(a[ks][mi], b[ks][ni], d[mi][ni]);
      quarter_to_thread(q, d, acc, As, Bs);  // its barriers also publish fac
    } else {
      fetch(min(h + 1, h1 - 1));
      gemm_staged<T, true, T, true>(dy + ((t0 + l0) * H + h) * P, (int64_t)H * P, len - l0, nullptr,
                                    x + ((t0 + s0) * H + h) * P, (int64_t)H * P, len - s0, 0, P, acc,
                                    As, Bs);
    }
    float rsum[4] = {0.f, 0.f, 0.f, 0.f}, csum[4] = {0.f, 0.f, 0.f, 0.f};
    const float4 al4 = *reinterpret_cast<const float4*>(&al[tm]);
    const float4 as4 = *reinterpret_cast<const float4*>(&as[tn]);
    const float4 dl4 = *reinterpret_cast<const float4*>(&dls[tn]);
    const float alv[4] = {al4.x, al4.y, al4.z, al4.w}, asv[4] = {as4.x, as4.y, as4.z, as4.w};
    const float dlv[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        const int l = l0 + tm + i, sx = s0 + tn + jn;
        if (l < len && sx <= l) {
          const float v = exp2_fast((alv[i] - asv[jn]) * kLog2e) * acc[i][jn];
          const float dv = dlv[jn] * v;
          w[i][jn] += dv;
          rsum[i] += cbr[i][jn] * dv;
          csum[jn] += cbr[i][jn] * v;
        }
      }
    const __amdgpu_buffer_rsrc_t rrow = buf_rsrc_u(rowpart + (jh * LT + st) * L + l0, 64 * sizeof(float));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = row_sum16(rsum[i]);
      store_buf(rrow, (tm + i) * sizeof(float), r, (threadIdx.x & 15) == 0);
    }
    // on the diagonal, V[l,l] before its decay (1) is dy_l . x_l: the
    // per-token dot of dD, taken here instead of re-reading dy and x
    const __amdgpu_buffer_rsrc_t rdd = buf_rsrc_u(ddot + jh * L + l0, (uint32_t)((len - l0) * sizeof(float)));
#pragma unroll
    for (int i = 0; i < 4; ++i) store_buf(rdd, (tm + i) * sizeof(float), acc[i][i], lt == st && tm == tn);
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) cpart[threadIdx.x >> 4][tn + jn] = csum[jn];
    __syncthreads();
    {                                      // every thread sums a column; the first 64 store it
      float c = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) c += cpart[r][fi];
      store_buf(buf_rsrc_u(colpart + (jh * LT + lt) * L + s0, 64 * sizeof(float)), fi * sizeof(float), c,
                threadIdx.x < 64);
    }
    __syncthreads();                       // cpart, al, as, dls read before the next head writes them
    take();
  }
  // whole 4-wide pieces of the rows in the chunk (w is 0 above the
  // diagonal; entries there and past the chunk are never read)
  float* W = dcbp + (((int64_t)j * G + g) * HB + hb) * L * L;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int l = l0 + tm + i;
    if (l < len) store4(W + (int64_t)l * L + s0 + tn, w[i][0], w[i][1], w[i][2], w[i][3]);
  }
}

// 3a, bf16 inputs: the same sums with the epilogue in the MFMA result
// layout (each wave's 32 x 32 quarter: a lane holds rows wr + 16 mi +
// 4 (lane / 16) + r of columns wc + 16 ni + lane % 16), so a head needs no
// pass of the tile through LDS.  The partial sums go to two slots per tile,
// one per half of its columns (rows) held by a wave:
//   rowpart[2 st + wc / 32][l],  colpart[2 lt + wr / 32][s].
// The head's dy and x rows of the tile and its running sums and steps are
// staged in LDS, alternating between two buffers: one barrier per head.
// The next head's rows (16-byte pieces, eight lanes per 128-byte row) and
// factor values are loaded during the current head (buffer loads without
// branches; rows past the chunk read zeros).
template <int P, int L>
__global__ __launch_bounds__(kBwdThreads) void bwd_v_mfma_kernel(
    ChunkMap cm, int nslots, const bf16* __restrict__ x, const bf16* __restrict__ dy,
    const bf16* __restrict__ cb, const float* __restrict__ delta, const float* __restrict__ dAcs, int H,
    int G, int HB, float* __restrict__ dcbp, float* __restrict__ rowpart, float* __restrict__ colpart,
    float* __restrict__ ddot, bf16* __restrict__ cbt, bf16* __restrict__ dcb16) {
  // per head: a at the tile's rows, a at its columns, delta at its columns
  __shared__ __align__(16) float fac[2][3][64];
  // per head: the tile's dy rows and x rows (P bf16 each, padded rows)
  constexpr int RP = P + 8;
  __shared__ __align__(16) bf16 ty[2][64 * RP], tx[2][64 * RP];
  constexpr int LT = L / 64;
  constexpr int NX = LT * (LT + 1) / 2;   // tiles on or below the diagonal
  constexpr int KS = P / 32;
  static_assert(P % 32 == 0, "k-steps of the rows");
  const int2 ci = xcd_chunk_head(blockIdx.x, NX * G * HB);
  if (ci.x >= nslots) return;
  const int2 tt = lower_tile(ci.y % NX);
  const int lt = __builtin_amdgcn_readfirstlane(tt.x), st = __builtin_amdgcn_readfirstlane(tt.y);
  const int by = ci.y / NX;
  const int g = by / HB, hb = by - (by / HB) * HB, j = ci.x;
  const int hpg = H / G, h0 = g * hpg + hb * hpg / HB, h1 = g * hpg + (hb + 1) * hpg / HB;
  const ChunkDesc cd = cm.desc(j);
  const int len = max(cd.len, 0);
  const int l0 = lt * 64, s0 = st * 64;
  if (l0 >= len) return;
  const int64_t t0 = cd.start;
  const MfmaQuarter q;
  const int lg = q.lane >> 4;
  // CB at this lane's 16 elements, 0 where V is not summed (s > l, rows past
  // the chunk): the same for every head.  Loaded together without a branch
  // (an element that is not summed aims past the records and reads 0).
  const __amdgpu_buffer_rsrc_t rcbj = buf_rsrc_u(cb + ((int64_t)j * G + g) * L * L, L * L * sizeof(bf16));
  float cbq[2][2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int l = l0 + q.row(mi, r), sx = s0 + q.col(ni);
        const uint32_t off = (l < len && sx <= l) ? (uint32_t)(l * L + sx) * sizeof(bf16) : kPastRecords;
        cbq[mi][ni][r] = static_cast<float>(
            __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(rcbj, off, 0, 0)));
      }
  // the first head block also writes these values transposed for dx: a
  // lane's four rows l of column s are four consecutive entries of row s
  {
    const __amdgpu_buffer_rsrc_t rt = buf_rsrc_u(cbt + ((int64_t)j * G + g) * L * L, L * L * sizeof(bf16));
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = static_cast<bf16>(cbq[mi][ni][r]);
        const uint32_t off = ((uint32_t)(s0 + q.col(ni)) * L + l0 + q.row(mi, 0)) * sizeof(bf16);
        buf_store8(rt, hb == 0 ? off : kPastRecords, __builtin_bit_cast(uint2, v));
      }
  }
  f32x4 w[2][2];                           // this block's sum of delta_s V[l,s]
  zero_quarter(w);
  const __amdgpu_buffer_rsrc_t rdy =
      buf_rsrc_u(dy + (t0 + l0) * H * P, (uint32_t)((int64_t)(len - l0) * H * P * sizeof(bf16)));
  const __amdgpu_buffer_rsrc_t rx =
      buf_rsrc_u(x + (t0 + s0) * H * P, (uint32_t)((int64_t)(len - s0) * H * P * sizeof(bf16)));
  const int fk = min(threadIdx.x >> 6, 2), fi = threadIdx.x & 63;   // threads 192-255 repeat delta
  constexpr int PR = P / 8;                // 16-byte pieces per row
  constexpr int NP = 64 * PR / kBwdThreads;   // pieces of each tile per thread
  static_assert(64 * PR % kBwdThreads == 0, "pieces of the row tiles");
  bf16x8 py[NP], px[NP];
  float fv;
  auto fetch = [&](int h) {
    const int64_t jh = (int64_t)j * H + h;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = threadIdx.x + kBwdThreads * u, r = i / PR, c = (i % PR) * 8;
      py[u] = frag_buf(rdy, (uint32_t)(((r * H + h) * P + c) * sizeof(bf16)));
      px[u] = frag_buf(rx, (uint32_t)(((r * H + h) * P + c) * sizeof(bf16)));
    }
    fv = fk == 0 ? dAcs[jh * L + l0 + fi] : fk == 1 ? dAcs[jh * L + s0 + fi] : delta[jh * L + s0 + fi];
  };
  auto take = [&](int set) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = threadIdx.x + kBwdThreads * u, r = i / PR, c = (i % PR) * 8;
      *reinterpret_cast<bf16x8*>(&ty[set][r * RP + c]) = py[u];
      *reinterpret_cast<bf16x8*>(&tx[set][r * RP + c]) = px[u];
    }
    fac[set][fk][fi] = fv;
  };
  const int RS = 2 * LT;                   // partial-sum slots per token
  fetch(h0);
  take(0);
  for (int h = h0; h < h1; ++h) {
    const int set = (h - h0) & 1;
    const int64_t jh = (int64_t)j * H + h;
    fetch(min(h + 1, h1 - 1));             // past the block's last head: that head again
    // fac[set] written; the previous head's reads of fac[set ^ 1] are done
    __syncthreads();
    f32x4 d[2][2];
    zero_quarter(d);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        a[u] = *reinterpret_cast<const bf16x8*>(&ty[set][(q.wr + u * 16 + q.lr) * RP + ks * 32 + q.kq]);
        b[u] = *reinterpret_cast<const bf16x8*>(&tx[set][(q.wc + u * 16 + q.lr) * RP + ks * 32 + q.kq]);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) d[mi][ni] = Mfma<bf16>::mma(a[mi], b[ni], d[mi][ni]);
    }
    float rs[8], cs[2] = {0.f, 0.f};
    float asv[2], dlv[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      asv[ni] = fac[set][1][q.col(ni)];
      dlv[ni] = fac[set][2][q.col(ni)];
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const float4 al4 = *reinterpret_cast<const float4*>(&fac[set][0][q.row(mi, 0)]);
      const float alv[4] = {al4.x, al4.y, al4.z, al4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int l = l0 + q.row(mi, r);
        float rsum = 0.f;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int sx = s0 + q.col(ni);
          // the mask selects the exponent (exp2 of -inf is 0): no branch,
          // and nothing undefined enters the sums
          const float arg = (l < len && sx <= l) ? (alv[r] - asv[ni]) * kLog2e : -INFINITY;
          const float v = exp2_fast(arg) * d[mi][ni][r];
          const float dv = dlv[ni] * v;
          w[mi][ni][r] += dv;
          rsum += cbq[mi][ni][r] * dv;
          cs[ni] += cbq[mi][ni][r] * v;
        }
        rs[4 * mi + r] = rsum;
      }
    }
    // row sums over the wave's 32 columns: lane lr ends with one row
    {
      const float sum = row_sum16_x8(rs, q.lr);
      const int rl = q.row(q.lr >> 3, 2 * ((q.lr >> 2) & 1) + ((q.lr >> 1) & 1));
      const __amdgpu_buffer_rsrc_t rp =
          buf_rsrc_u(rowpart + (jh * RS + 2 * st + (q.wc >> 5)) * L + l0, 64 * sizeof(float));
      store_buf(rp, rl * sizeof(float), sum, (q.lr & 1) == 0);
    }
    // column sums over the wave's 32 rows: the lane groups hold 8 rows
    // each; pairing across groups 0-1 / 2-3, lanes of group 2 lg' keep
    // column ni = lg' / 2 ... one column per lane pair of groups
    {
      const bool hi = lg & 2;
      float t = (hi ? cs[1] : cs[0]) + __shfl_xor(hi ? cs[0] : cs[1], 32);
      t += __shfl_xor(t, 16);
      const int cl = q.col(hi ? 1 : 0);
      const __amdgpu_buffer_rsrc_t rc =
          buf_rsrc_u(colpart + (jh * RS + 2 * lt + (q.wr >> 5)) * L + s0, 64 * sizeof(float));
      store_buf(rc, cl * sizeof(float), t, (lg & 1) == 0);
    }
    // on the diagonal, V[l,l] before its decay (1) is dy_l . x_l: the
    // per-token dot of dD (lanes whose column is one of their rows)
    {
      const __amdgpu_buffer_rsrc_t rdd = buf_rsrc_u(ddot + jh * L + l0, (uint32_t)((len - l0) * sizeof(float)));
      const int rr = q.lr & 3;
      const bool on = lt == st && q.wr == q.wc && (q.lr >> 2) == lg;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const f32x4 dd = d[mi][mi];
        const float v = rr == 0 ? dd[0] : rr == 1 ? dd[1] : rr == 2 ? dd[2] : dd[3];
        store_buf(rdd, q.row(mi, rr) * sizeof(float), v, on);
      }
    }
    take(set ^ 1);                         // the next head's rows and factors
  }
  // the block's sum, rows in the chunk (w is 0 above the diagonal; entries
  // there and past the chunk are never read): a partial sum in fp32, or,
  // with one block per group, the group's dCB rounded once to bf16
  if (HB > 1) {                            // uniform
    float* W = dcbp + (((int64_t)j * G + g) * HB + hb) * L * L;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int l = l0 + q.row(mi, r);
        if (l < len) {
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) W[(int64_t)l * L + s0 + q.col(ni)] = w[mi][ni][r];
        }
      }
  } else {
    bf16* W = dcb16 + ((int64_t)j * G + g) * L * L;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int l = l0 + q.row(mi, r);
        if (l < len) {
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) W[(int64_t)l * L + s0 + q.col(ni)] = static_cast<bf16>(w[mi][ni][r]);
        }
      }
  }
}

// 3b, fp32 inputs: dx as 64 x 64 tiles of (token s, p):
//   dx_s = delta_s [ sum_{l>=s} CB[l,s] exp(a_l - a_s) dy_l + exp(a_last - a_s) dS_j B_s ]
//          + D dy_s;
// grid: xcd_grid(chunk slots, L/64 * ceil(P/64) * H), a chunk's tiles on its XCD.
template <typename T, int P, int N, int L>
__global__ __launch_bounds__(kBwdThreads, 8) void bwd_dx_tiled_kernel(
    ChunkMap cm, int nslots, const T* __restrict__ B, const T* __restrict__ dy, const T* __restrict__ cb,
    const float* __restrict__ delta, const float* __restrict__ dAcs, const float* __restrict__ dS,
    const float* __restrict__ D, int H, int G, T* __restrict__ dx) {
  __shared__ __align__(16) float As[32 * kGemmPitch], Bs[32 * kGemmPitch];
  __shared__ float es[L], av[L];
  constexpr int PT = (P + 63) / 64;
  constexpr int NX = (L / 64) * PT;
  const int2 ci = xcd_chunk_head(blockIdx.x, NX * H);
  if (ci.x >= nslots) return;
  const int bx = ci.y % NX;
  const int s0 = (bx / PT) * 64, p0 = (bx % PT) * 64;
  const int h = ci.y / NX, j = ci.x, g = h / (H / G);
  const ChunkDesc cd = cm.desc(j);
  const int len = max(cd.len, 0);
  if (s0 >= len) return;
  const int64_t jh = (int64_t)j * H + h, t0 = cd.start;
  const float* a = dAcs + jh * L;
  const float alast = a[len - 1];
  for (int l = threadIdx.x; l < L; l += kBwdThreads) {
    es[l] = exp2_fast((alast - a[l]) * kLog2e);
    av[l] = a[l];
  }
  const T* cbj = cb + ((int64_t)j * G + g) * L * L;
  float acc[4][4] = {};
  // sum_{l >= s} CB[l,s] exp(a_l - a_s) dy_l: slices of 32 tokens l, each a
  // CB row (columns s) and a dy row (columns p) in 16-byte pieces
  {
    constexpr int V = 16 / sizeof(T), PC = 64 / V;   // pieces per 64-wide row
    const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
    for (int kb = s0; kb < len; kb += 32) {
      __syncthreads();                     // previous slice consumed (es, av staged)
      for (int i = threadIdx.x; i < 32 * PC; i += kBwdThreads) {
        const int kr = i / PC, c = (i - (i / PC) * PC) * V, l = kb + kr;
        const bool lok = l < len;
        float va[V], vb[V];
        load16_f32<T>(cbj + (int64_t)l * L + s0 + c, lok, va);
        load16_f32<T>(dy + ((t0 + l) * H + h) * P + p0 + c, lok && p0 + c < P, vb);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int sx = s0 + c + e;
          As[kr * kGemmPitch + c + e] =
              (lok && sx < len && l >= sx) ? va[e] * exp2_fast((av[l] - av[sx]) * kLog2e) : 0.f;
          Bs[kr * kGemmPitch + c + e] = vb[e];
        }
      }
      __syncthreads();
#pragma unroll 8
      for (int k = 0; k < 32; ++k) {
        const float4 a4 = *reinterpret_cast<const float4*>(&As[k * kGemmPitch + tm]);
        const float4 b4 = *reinterpret_cast<const float4*>(&Bs[k * kGemmPitch + tn]);
        const float avv[4] = {a4.x, a4.y, a4.z, a4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jn = 0; jn < 4; ++jn) acc[i][jn] += avv[i] * bv[jn];
      }
    }
  }
  // + exp(a_last - a_s) B_s . dS_j[p, :]: rows s of B (scaled), rows p of dS
  gemm_staged<T, true, float, true, (N < 32 ? N : 32)>(B + ((t0 + s0) * G + g) * N, (int64_t)G * N,
                                                       len - s0, es + s0, dS + (jh * P + p0) * N, N,
                                                       P - p0, 0, N, acc, As, Bs);
  const float Dh = D ? D[h] : 0.f;
  const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
  static_assert(P % 4 == 0, "4-wide pieces of a row");
  // the rows' loads first (rows past the chunk read its last row, columns
  // past P its first piece; neither is stored), then the stores
  float dsv[4];
  float4 yv4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sx = min(s0 + tm + i, len - 1), pc = p0 + tn < P ? p0 + tn : 0;
    dsv[i] = delta[jh * L + sx];
    yv4[i] = load4_f32(dy + ((t0 + sx) * H + h) * P + pc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sx = s0 + tm + i;
    if (sx >= len || p0 + tn >= P) continue;
    const int64_t o = ((t0 + sx) * H + h) * P + p0 + tn;
    const float4 y = yv4[i];
    store4(dx + o, dsv[i] * acc[i][0] + Dh * y.x, dsv[i] * acc[i][1] + Dh * y.y,
           dsv[i] * acc[i][2] + Dh * y.z, dsv[i] * acc[i][3] + Dh * y.w);
  }
}

// 3b, bf16 inputs: dx as one tile per (chunk, head), the adjoint of the
// forward's chunk_scan tile,
//   dx^T[p][s] = delta_s [ sum_{l >= s} dy^T[p][l] CBt[s][l] exp(a_l - a_s)
//                          + exp(a_last - a_s) sum_n dS[p][n] B[s][n] ] + D dy_s[p],
// with that tile's operand flow: dy rows staged XOR-swizzled in LDS give the
// dy^T operands by transpose read (x^T there); rows of CB's transposed copy,
// written by 3a, stream from memory through a register ring as the B
// operands (CB rows there); the dS term is its inter-chunk term with dS as
// the state and B rows as the C rows.  A lane holds four consecutive p of
// one token s.  Row group m (16 tokens s) meets the k-steps from m / 2 on;
// with 256-token chunks each wave owns a mirror pair of row groups, so every
// wave carries the same work, otherwise one row group.
// dy is staged as loaded, and each CBt piece is scaled before its MFMA.
// FAST (the chunk's whole decay within 2^kBwdFastMaxLog2): by exp(a_l) (0
// where l < s as CBt itself), the dS term by exp(a_last), and row s by
// delta_s exp(-a_s) at the end.  Otherwise by the decay exp(a_l - a_s) --
// below the diagonal split around the block's first token r as
// exp(a_l - a_r) exp(a_r - a_s), both <= 1, one exponential per piece; on
// it masked exponentials -- the dS term by exp(a_last - a_s), and row s by
// delta_s.  D dy_s joins in fp32, from the staged dy.

// Waves of a dx tile: eight from 128-token chunks on (one or two row groups
// each), four for 64-token chunks.
template <int L> constexpr int kDxWaves = L >= 128 ? 8 : 4;

// CBt piece at k-step q times exp(a_l) (el: exp(a) per token; factored path).
__device__ __forceinline__ bf16x8 dx_scaled_cbt(const bf16x8& v, int q, int kq, const float* el) {
  const float4 f0 = *reinterpret_cast<const float4*>(&el[32 * q + kq]);
  const float4 f1 = *reinterpret_cast<const float4*>(&el[32 * q + kq + 4]);
  const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
  float mv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mv[e] = static_cast<float>(v[e]) * f[e];
  return Mfma<bf16>::pack(mv);
}

// CBt piece of row s (row group m) at k-step q times its decay (exact path).
__device__ __forceinline__ bf16x8 dx_masked_cbt(const bf16x8& v, int m, int q, int s, int kq,
                                                const float* dal2, const float* cfr) {
  const int l0 = 32 * q;
  const float das = dal2[s];
  float mv[8];
  if (l0 >= 16 * m + 16) {               // the block lies after every row of the group
    const float rf = exp2_fast(dal2[l0] - das);
    const float4 f0 = *reinterpret_cast<const float4*>(&cfr[l0 + kq]);
    const float4 f1 = *reinterpret_cast<const float4*>(&cfr[l0 + kq + 4]);
    const float cf[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) mv[e] = static_cast<float>(v[e]) * (cf[e] * rf);
  } else {                               // on the diagonal
    const float4 a0 = *reinterpret_cast<const float4*>(&dal2[l0 + kq]);
    const float4 a1 = *reinterpret_cast<const float4*>(&dal2[l0 + kq + 4]);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // before the row the exponent is -inf, and exp2 gives exactly 0
      const float arg = l0 + kq + e >= s ? av[e] - das : -__builtin_inff();
      mv[e] = static_cast<float>(v[e]) * exp2_fast(arg);
    }
  }
  return Mfma<bf16>::pack(mv);
}

template <int P, int N, int L, bool FAST>
__device__ __forceinline__ void bwd_dx_tile(const ScanTile& T, float last2, const bf16* __restrict__ B,
                                            const bf16* __restrict__ dy, const bf16* __restrict__ cbt,
                                            const float* __restrict__ delta, const float* __restrict__ dAcs,
                                            const bf16* __restrict__ dS16, const float* __restrict__ D,
                                            int H, int G, bf16* __restrict__ dx, bf16* ys, bf16* hsm,
                                            float* dal2, float* dls, float* cfr) {
  using M = Mfma<bf16>;
  constexpr int NW = kDxWaves<L>, NT = 64 * NW;
  constexpr int HP = N + 8;              // dS tile pitch, as the forward's state tile
  constexpr int RG = L / 16, RGW = RG / NW, PT = P / 16, NK = N / 32, NQ = L / 32;
  constexpr int CPR = P / 8, XU = L * CPR / NT, HPR = N / 8, HU = (P * HPR + NT - 1) / NT;
  static_assert(RGW * NW == RG && (RGW == 1 || RGW == 2), "row-group split");
  static_assert((L * CPR) % NT == 0 && L <= NT, "dy staging");
  const int h = T.h, g = h / (H / G);
  const uint32_t HPx = (uint32_t)H * P, GN = (uint32_t)G * N;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63;
  const int lr = lane & 15, kg = lane >> 4, kq = kg * 8;
  const int64_t jh = (int64_t)T.j * H + h;
  int mg[RGW], srow[RGW], qs[RGW];
  mg[0] = w;
  if constexpr (RGW == 2) mg[1] = RG - 1 - w;
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    srow[i] = 16 * mg[i] + lr;
    qs[i] = mg[i] / 2;                     // first k-step that reaches the row group
  }
  const int nqv = (T.len + 31) / 32;       // k-steps inside the chunk

  // ---- global loads, in the order of use
  const auto rdy = rows_rsrc(dy, T, H, P, HPx);
  const auto rda = buf_rsrc(dAcs + jh * L, L * 4);
  uint4 yv[XU];
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tid + NT * u, r = i / CPR, c = i % CPR;
    yv[u] = buf_load16(rdy, ((uint32_t)r * HPx + c * 8) * 2u);
  }
  const auto rh = buf_rsrc(dS16 + jh * P * N, P * N * 2);
  uint4 hv[HU];
#pragma unroll
  for (int u = 0; u < HU; ++u) hv[u] = buf_load16(rh, (uint32_t)(tid + NT * u) * 16);
  const float dA_t = buf_load4(rda, tid * 4);
  const float dl_t = buf_load4(buf_rsrc(delta + jh * L, L * 4), tid * 4);
  const auto rb = buf_rsrc(B + ((int64_t)T.start * G + g) * N, ((uint32_t)(T.len - 1) * GN + N) * 2u);
  bf16x8 fb[RGW][NK];                      // B rows of this lane, all n-steps
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int k = 0; k < NK; ++k)
      fb[i][k] = __builtin_bit_cast(bf16x8, buf_load16(rb, ((uint32_t)srow[i] * GN + 32 * k + kq) * 2u));
  const auto rct = buf_rsrc(cbt + ((int64_t)T.j * G + g) * L * L, L * L * 2);

  // ---- stage dy as loaded (rows past the chunk arrived as zeros), the dS
  // tile and the per-token values
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tid + NT * u, r = i / CPR, c = i % CPR;
    *reinterpret_cast<uint4*>(&ys[r * P + ((c ^ tile_sw<CPR>(r)) << 3)]) = yv[u];
  }
#pragma unroll
  for (int u = 0; u < HU; ++u) {
    const int i = tid + NT * u, r = i / HPR, c = i % HPR;
    if ((P * HPR) % NT == 0 || i < P * HPR) *reinterpret_cast<uint4*>(&hsm[r * HP + c * 8]) = hv[u];
  }
  {
    // every thread stores its entry (one per thread; those past the chunk's
    // L tokens are read by none), so that the loads of a and delta stay at
    // the top
    const float a2 = dA_t * kLog2e;
    dal2[tid] = a2;
    dls[tid] = dl_t;
    if constexpr (FAST) {
      cfr[tid] = exp2_fast(a2);            // exp(a_l); past the chunk a is flat: finite
    } else {
      const float a2r = __shfl(a2, lane & ~31);   // the first token of the 32-token block
      cfr[tid] = exp2_fast(a2 - a2r);
    }
  }
  f32x4 acc[RGW][PT];
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int a = 0; a < PT; ++a) acc[i][a] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  scan_tile_inter<P, N, RGW, HP>(acc, fb, hsm, lr, kq);
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    const float f = FAST ? exp2_fast(last2) : exp2_fast(last2 - dal2[srow[i]]);
#pragma unroll
    for (int a = 0; a < PT; ++a) acc[i][a] *= f;
  }

  // ---- intra-chunk term: CBt pieces through a ring of RD per row group,
  // RD - 1 k-steps ahead; dy^T operands through a ring of XR over the
  // sequence (step, p-tile).  Every ring load is issued, without a branch:
  // one a row group does not need (before its first k-step, past the
  // chunk's last) aims past the records and reads zeros.  Steps before a
  // row group's first multiply nothing; the loop ends at the chunk's last
  // k-step.
  // (two operand slots from 128-token chunks on keep the tile within 128 VGPRs)
  constexpr int RD = 3, XR = L >= 128 ? 2 : 3, NOP = NQ * PT;
  const int xrow = 8 * kg + (lr >> 2);
  const int xsl = tile_sw<CPR>(xrow) >> 1;
  const int xcol = ((lr & 3) >> 1) * 8 + (lr & 1) * 4;
  const auto cbt_off = [&](int i, int q) {
    return (q >= qs[i] && q < nqv) ? ((uint32_t)srow[i] * L + 32 * q + kq) * 2u : kPastRecords;
  };
  bf16x8 ring[RGW][RD];
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int q = 0; q < RD - 1; ++q) ring[i][q] = __builtin_bit_cast(bf16x8, buf_load16(rct, cbt_off(i, q)));
  bf16x8 fxr[XR];
#pragma unroll
  for (int n = 0; n < XR; ++n) fxr[n] = scan_x_operand<P>(ys, n / PT, n % PT, xrow, xsl, xcol);
  bf16x8 fm[RGW];
#pragma unroll
  for (int n = 0; n < NOP; ++n) {
    const int q = n / PT, a = n % PT;
    if (a == 0) {
      if (q >= nqv) break;                 // wave-uniform
      if (q + RD - 1 < NQ) {
#pragma unroll
        for (int i = 0; i < RGW; ++i)
          ring[i][(q + RD - 1) % RD] = __builtin_bit_cast(bf16x8, buf_load16(rct, cbt_off(i, q + RD - 1)));
      }
#pragma unroll
      for (int i = 0; i < RGW; ++i) {
        if (q >= qs[i]) {                  // wave-uniform
          if constexpr (FAST) fm[i] = dx_scaled_cbt(ring[i][q % RD], q, kq, cfr);
          else fm[i] = dx_masked_cbt(ring[i][q % RD], mg[i], q, srow[i], kq, dal2, cfr);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RGW; ++i)
      if (q >= qs[i]) acc[i][a] = M::mma(fxr[n % XR], fm[i], acc[i][a]);   // wave-uniform
    if (n + XR < NOP) fxr[n % XR] = scan_x_operand<P>(ys, (n + XR) / PT, (n + XR) % PT, xrow, xsl, xcol);
  }

  // ---- epilogue: row factor and D dy in fp32 (dy from the staged tile, at
  // this lane's outputs), rounded once; the tile goes to LDS over dy (every
  // wave is done with it) in the out_sw layout, a lane's four p of one token
  // as one 8-byte piece, and leaves as whole rows
  uint2 dyr[RGW][PT];
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int a = 0; a < PT; ++a) {
      const int s = srow[i], c = 2 * a + (kg >> 1);   // p = 16 a + 4 kg: piece c, half kg & 1
      dyr[i][a] = *reinterpret_cast<const uint2*>(&ys[s * P + ((c ^ tile_sw<CPR>(s)) << 3) + 4 * (kg & 1)]);
    }
  const float Dh = D ? D[h] : 0.f;
  float rsc[RGW];
#pragma unroll
  for (int i = 0; i < RGW; ++i)
    rsc[i] = FAST ? dls[srow[i]] * exp2_fast(-dal2[srow[i]]) : dls[srow[i]];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int a = 0; a < PT; ++a) {
      const int s = srow[i];
      const bf16x4 raw = __builtin_bit_cast(bf16x4, dyr[i][a]);
      bf16x4 yo;
#pragma unroll
      for (int r = 0; r < 4; ++r) yo[r] = static_cast<bf16>(acc[i][a][r] * rsc[i] + Dh * static_cast<float>(raw[r]));
      *reinterpret_cast<bf16x4*>(&ys[s * P + ((4 * a + kg) ^ out_sw<P>(s)) * 4]) = yo;
    }
  __syncthreads();
  const auto rdx = rows_rsrc(dx, T, H, P, HPx);
  // the store rows from a fresh copy of the thread index: indices shared with
  // the staging loop would stay live across the tile
  const int tids = opaque_tid();
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tids + NT * u, r = i / CPR, c = i % CPR;
    const int sw = out_sw<P>(r);
    const uint2 v0 = *reinterpret_cast<const uint2*>(&ys[r * P + ((2 * c) ^ sw) * 4]);
    const uint2 v1 = *reinterpret_cast<const uint2*>(&ys[r * P + ((2 * c + 1) ^ sw) * 4]);
    buf_store16(rdx, ((uint32_t)r * HPx + c * 8) * 2u, make_uint4(v0.x, v0.y, v1.x, v1.y));
  }
}

// grid: xcd_grid(chunk slots, H), a chunk's heads on its XCD.
// dA, dD and dt_bias of head h: the per-token pass's parts summed over the
// chunk slots (lanes stride the slots, then a shuffle sum; one wave).
__device__ __forceinline__ void head_sums(const float* __restrict__ dA_part,
                                          const float* __restrict__ dD_part,
                                          const float* __restrict__ dbias_part, int h, int H,
                                          int nslots, int lane, float* __restrict__ dA,
                                          float* __restrict__ dD, float* __restrict__ dbias) {
  float sa = 0.f, sd = 0.f, sb = 0.f;
  for (int j = lane; j < nslots; j += kWave) {
    sa += dA_part[(int64_t)j * H + h];
    sd += dD_part[(int64_t)j * H + h];
    sb += dbias_part[(int64_t)j * H + h];
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    sa += __shfl_xor(sa, off);
    sd += __shfl_xor(sd, off);
    sb += __shfl_xor(sb, off);
  }
  if (lane == 0) {
    dA[h] = sa;
    if (dD) dD[h] = sd;
    if (dbias) dbias[h] = sb;
  }
}

// grid: xcd_grid(chunk slots, H), a chunk's heads on its XCD.  The first
// wave of chunk slot 0's workgroup for head h, once its tile is stored, also
// writes that head's dA, dD and dt_bias (the per-token pass runs before this
// launch).
template <int P, int N, int L>
__global__ __launch_bounds__(64 * kDxWaves<L>) __attribute__((amdgpu_waves_per_eu(
    kTileWavesPerEU<L, kDxWaves<L>>))) void bwd_dx_scan_kernel(ChunkMap cm, int nslots,
                                                              const bf16* __restrict__ B,
                                                              const bf16* __restrict__ dy,
                                                              const bf16* __restrict__ cbt,
                                                              const float* __restrict__ delta,
                                                              const float* __restrict__ dAcs,
                                                              const bf16* __restrict__ dS16,
                                                              const float* __restrict__ D, int H, int G,
                                                              bf16* __restrict__ dx,
                                                              const float* __restrict__ dA_part,
                                                              const float* __restrict__ dD_part,
                                                              const float* __restrict__ dbias_part,
                                                              float* __restrict__ dA, float* __restrict__ dD,
                                                              float* __restrict__ dbias) {
  __shared__ __align__(16) bf16 ys[L * P];
  __shared__ __align__(16) bf16 hsm[P * (N + 8)];
  // per-token vectors, one entry per thread (64 kDxWaves >= L)
  __shared__ __align__(16) float dal2[64 * kDxWaves<L>];  // running sum of delta*A, times log2(e)
  __shared__ __align__(16) float dls[64 * kDxWaves<L>];   // delta
  __shared__ __align__(16) float cfr[64 * kDxWaves<L>];   // exp(a_l) (factored) or exp(a_l - a_r), r = first of l's 32-block
  const int2 ci = xcd_chunk_head(blockIdx.x, H);
  if (ci.x >= nslots) return;
  // the running sum is monotone inside a chunk and flat past its end: its
  // value at the last position bounds every |a_s|
  const float last = dAcs[((int64_t)ci.x * H + ci.y) * L + L - 1];
  const ChunkDesc cd = cm.desc(ci.x);
  if (cd.len > 0) {
    const ScanTile T{ci.x, ci.y, cd.start, cd.len};
    if (fabsf(last) * kLog2e <= kBwdFastMaxLog2)   // uniform over the workgroup
      bwd_dx_tile<P, N, L, true>(T, last * kLog2e, B, dy, cbt, delta, dAcs, dS16, D, H, G, dx, ys, hsm,
                                 dal2, dls, cfr);
    else
      bwd_dx_tile<P, N, L, false>(T, last * kLog2e, B, dy, cbt, delta, dAcs, dS16, D, H, G, dx, ys, hsm,
                                  dal2, dls, cfr);
  }
  if (ci.x == 0 && threadIdx.x < kWave)
    head_sums(dA_part, dD_part, dbias_part, ci.y, H, nslots, threadIdx.x, dA, dD, dbias);
}

// 3b'. The group's dCB: the HB partial sums of 3a added, four entries per
// thread: into the first partial, or, given dcb16 (bf16 inputs), rounded
// once to bf16 there.  Only the 64 x 64 tiles on or below the diagonal,
// the ones 3a writes and 4 reads (entries above the diagonal inside them
// or past the chunk are summed too and never read): kDcbBlocksPerTile
// workgroups per tile, the tiles in row order, a wave on 4 rows x 64
// columns.  grid (L/64 (L/64 + 1) / 2 * kDcbBlocksPerTile, G, chunk slots).
constexpr int kDcbBlocksPerTile = 64 * 64 / 4 / kBwdThreads;
template <int L>
__global__ __launch_bounds__(kBwdThreads) void bwd_dcb_sum_kernel(int G, int HB, float* __restrict__ dcbp,
                                                                  bf16* __restrict__ dcb16) {
  const int t = blockIdx.x / kDcbBlocksPerTile;   // the t-th tile on or below the diagonal
  int ti = 0;
  while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
  const int tj = t - ti * (ti + 1) / 2;
  const int i = (blockIdx.x % kDcbBlocksPerTile) * kBwdThreads + threadIdx.x;   // 0 .. 1023 in the tile
  const int e = ((ti * 64 + i / 16) * L + tj * 64 + (i % 16) * 4) / 4;
  const int64_t LL4 = (int64_t)L * L / 4, jg = (int64_t)blockIdx.z * G + blockIdx.y;
  float4* W = reinterpret_cast<float4*>(dcbp) + jg * HB * LL4 + e;
  float4 v = W[0];
  for (int k = 1; k < HB; ++k) {
    const float4 u = W[k * LL4];
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  }
  if (dcb16) store4(dcb16 + (jg * LL4 + e) * 4, v.x, v.y, v.z, v.w);
  else W[0] = v;
}

// 4. dC and dB of a group as 64 x 64 tiles of rows x n, rounded once to the
// dtype: the group's summed dCB (3b') times B or C, plus the state terms
// summed over the group's heads h and their rows p:
//   dC[l] = sum_{s<=l} dCB[l,s] B_s + sum_h sum_p exp(a_l) dy_l[p] H_h[p, :],
//   dB[s] = sum_{l>=s} dCB[l,s] C_l + sum_h sum_p delta_s exp(a_last - a_s) x_s[p] dS_h[p, :]
// (a, delta, a_last those of head h).  The state terms are one contraction
// over (h, p) per tile: dy and x rows are laid out with a token's heads side
// by side, the entering states and dS with a chunk's heads side by side.
// Each head's product before the sum also gives the per-token pass two row
// dots over the tile's 64 columns n (slot 2 nt + half of the columns):
//   interpart[slot][l] = sum_n C[l,n] exp(a_l) (dy_l H_h)[n]          (dC tiles)
//   vxpart[slot][s]    = sum_n B[s,n] exp(a_last - a_s) (x_s dS_h)[n] (dB tiles)
// so the dB tiles scale each head's product by delta_s after the dot.
// grid: xcd_grid(chunk slots, L/64 * ceil(N/64) * 2 * G), a chunk's tiles
// on its XCD; even tiles: dC, odd: dB.
template <typename T, int P, int N, int L>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_bc_group_kernel(
    ChunkMap cm, int nslots, const T* __restrict__ x, const T* __restrict__ B, const T* __restrict__ C,
    const T* __restrict__ dy, const float* __restrict__ delta, const float* __restrict__ dAcs,
    const T* __restrict__ states_in, const float* __restrict__ dS, const bf16* __restrict__ dS16,
    const float* __restrict__ dcbp, const bf16* __restrict__ dcb16, int H, int G, int HB,
    T* __restrict__ dB, T* __restrict__ dC,
    float* __restrict__ interpart, float* __restrict__ vxpart) {
  __shared__ __align__(16) float As[32 * kGemmPitch], Bs[32 * kGemmPitch];
  constexpr int NT = (N + 63) / 64;
  constexpr int NX = (L / 64) * NT * 2;
  const int2 ci = xcd_chunk_head(blockIdx.x, NX * G);
  if (ci.x >= nslots) return;
  const int bx = ci.y % NX;
  const int which = bx & 1, t = bx >> 1;
  const int m0 = (t / NT) * 64, n0 = (t % NT) * 64;
  const int g = ci.y / NX, j = ci.x;
  const ChunkDesc cd = cm.desc(j);
  const int len = max(cd.len, 0);
  if (m0 >= len) return;                   // uniform: rows past the chunk
  const int64_t t0 = cd.start;
  const int hpg = H / G, h0 = g * hpg;
  const float* W = dcbp + ((int64_t)j * G + g) * HB * L * L;   // the summed slot
  const T* rows = which == 0 ? dy : x;     // the state term's scaled rows
  const T* M = which == 0 ? C : B;         // the row dots' group rows
  float* part = which == 0 ? interpart : vxpart;
  constexpr int SL = 2 * NT;               // row-dot slots per token
  const int nt = n0 / 64;
  float acc[4][4] = {};
  if constexpr (sizeof(T) == 2) {
    // bf16 MFMA over 32-long k-slices, the summed dCB as rounded once to
    // bf16 by 3a or 3b' (masked to s <= l); B (dC) or C (dB) rows staged
    // k-major in LDS
    // One LDS region serves the three phases in turn -- the slices' k-major
    // tiles (at, bt), the heads' operand and row tiles (kt, ta), the final
    // regrouping of the quarters -- with a barrier between phases, so that
    // three workgroups fit on a CU.
    constexpr int kKtBytes = 2 * P * kKtPitch * 2, kTaBytes = 2 * 64 * (P + 8) * 2;
    constexpr int kSliceBytes = 2 * 32 * kKtPitch * 2, kRegroupBytes = 2 * 32 * kGemmPitch * 4;
    constexpr int kRegion = kKtBytes + kTaBytes > kSliceBytes
                                ? (kKtBytes + kTaBytes > kRegroupBytes ? kKtBytes + kTaBytes : kRegroupBytes)
                                : (kSliceBytes > kRegroupBytes ? kSliceBytes : kRegroupBytes);
    __shared__ __align__(16) unsigned char region[kRegion];
    bf16* at = reinterpret_cast<bf16*>(region);
    bf16* bt = at + 32 * kKtPitch;
    static_assert(32 * 8 == kBwdThreads, "one 8-wide piece of each slice tile per thread");
    const int kr = threadIdx.x >> 3, c = (threadIdx.x & 7) * 8;
    const MfmaQuarter q;
    f32x4 d[2][2];
    zero_quarter(d);
    const int k0 = which == 0 ? 0 : m0, k1 = which == 0 ? min(len, m0 + 64) : len;
    const T* R = which == 0 ? B : C;       // rows k of the second operand
    // A slice's pieces are loaded two slices ahead, while the slice between
    // is multiplied: buffer loads issued without a branch whichever the tile
    // (a load a tile does not need aims past the records and reads zeros).
    // dC: rows l = m0 + row of W, columns s = kb + kq ..; dB: rows l = k of
    // W, columns s = m0 + c ..
    const __amdgpu_buffer_rsrc_t rR = buf_rsrc_u(R + t0 * G * N, (uint32_t)((int64_t)len * G * N * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rW =
        buf_rsrc_u(dcb16 + ((int64_t)j * G + g) * L * L, (uint32_t)(L * L * sizeof(bf16)));
    // Two register sets (set = the slice's parity) hold them, so the loop
    // carries no register copies and waits only for the older set.
    bf16x8 rvp[2], wv[2][2];
    auto fetch_intra = [&](int set, int kb) {
      const int k = kb + kr;
      rvp[set] = frag_buf(rR, (uint32_t)(((k * G + g) * N + n0 + c) * sizeof(T)), k < k1 && n0 + c < N);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int l = m0 + q.wr + mi * 16 + q.lr, s1 = kb + q.kq;
        const uint32_t off = which == 0 ? (uint32_t)((l * L + s1) * sizeof(bf16))
                                        : (uint32_t)((k * L + m0 + c) * sizeof(bf16));
        const bool ok = which == 0 ? (l < len && s1 < k1) : (mi == 0 && k < k1);
        wv[set][mi] = frag_buf(rW, off, ok);
      }
    };
    auto intra = [&](int set, int kb) {
      const int k = kb + kr;
      const bf16x8 rv = rvp[set];
      const bf16x8 wc[2] = {wv[set][0], wv[set][1]};
      bf16x8 av[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        bf16x8 v;
        if (which == 0) {
          // A rows l = m0 + row: dCB[l, kb + kq ..] for s <= l
          const int l = m0 + q.wr + mi * 16 + q.lr, s1 = kb + q.kq;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (s1 + e <= l && s1 + e < k1) ? wc[mi][e] : bf16(0.f);
        } else {
          // rows l = k: dCB[l, s] for s <= l, k-major
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (m0 + c + e <= k && m0 + c + e < len) ? wc[mi][e] : bf16(0.f);
        }
        av[mi] = v;
      }
      __syncthreads();                     // previous slice consumed
      *reinterpret_cast<bf16x8*>(&bt[kr * kKtPitch + c]) = rv;
      if (which != 0) *reinterpret_cast<bf16x8*>(&at[kr * kKtPitch + c]) = av[0];
      __syncthreads();
      if (which == 0) {
        bf16x8 b[2];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) b[ni] = lds_operand_kmajor(bt, kKtPitch, 0, q.wc + ni * 16, q.lane);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) d[mi][ni] = Mfma<bf16>::mma(av[mi], b[ni], d[mi][ni]);
      } else {
        mfma_kmajor(q, at, bt, d);
      }
      fetch_intra(set, kb + 64);           // past k1: zeros
      __builtin_amdgcn_sched_barrier(0);   // keep the sets' loads in issue order
    };
    fetch_intra(0, k0);
    __builtin_amdgcn_sched_barrier(0);
    fetch_intra(1, k0 + 32);
    __builtin_amdgcn_sched_barrier(0);
    int kb = k0;
    for (; kb + 32 < k1; kb += 64) {       // whole pairs of slices
      intra(0, kb);
      intra(1, kb + 32);
    }
    if (kb < k1) intra(0, kb);             // an odd count's last slice
    __syncthreads();                       // the slices' tiles read: the heads' tiles take their place
    // The state terms, head by head: the rows (dy or x, exact bf16, staged
    // in LDS from whole-line loads) times the head's P x 64 operand (the
    // entering state or dS in bf16, staged k-major); both alternate between
    // two LDS buffers, so one barrier per head; the row factor exp(a_l) or
    // exp(a_last - a_s) (and delta_s for dB) multiplies the product's rows.
    // Two register sets hold the rows, operand pieces and factors of the
    // next two heads, loaded while the current head is multiplied.
    constexpr int KS = P / 32;             // 32-long k-steps per head
    constexpr int PP = P * 8 / kBwdThreads;   // 16-byte operand pieces per thread
    static_assert(P % 32 == 0 && PP >= 1 && P * 8 % kBwdThreads == 0, "head operand pieces");
    bf16 (*kt)[P * kKtPitch] = reinterpret_cast<bf16 (*)[P * kKtPitch]>(region);
    // the head's rows (dy or x) of the tile, P bf16 each (padded rows)
    constexpr int RPA = P + 8, PRA = P / 8, NPA = 64 * PRA / kBwdThreads;
    static_assert(64 * PRA % kBwdThreads == 0, "pieces of the row tile");
    static_assert(2 * 64 * RPA * 2 == kTaBytes, "row tiles in the region");
    bf16 (*ta)[64 * RPA] = reinterpret_cast<bf16 (*)[64 * RPA]>(region + kKtBytes);
    const bf16* K16 = which == 0 ? reinterpret_cast<const bf16*>(states_in) : dS16;
    const int h1 = h0 + hpg;
    // the chunk's rows (tokens past its end read zeros) and its heads'
    // P x N operands as buffer resources
    const __amdgpu_buffer_rsrc_t rrow =
        buf_rsrc_u(rows + t0 * H * P, (uint32_t)((int64_t)len * H * P * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rk16 =
        buf_rsrc_u(K16 + (int64_t)j * H * P * N, (uint32_t)((int64_t)H * P * N * sizeof(bf16)));
    // the row dots' M[row, n] at this lane's 8 rows and 2 columns of the
    // product (rows past the chunk and columns past N read 0), loaded
    // together without a branch
    const __amdgpu_buffer_rsrc_t rM = buf_rsrc_u(M + t0 * G * N, (uint32_t)((int64_t)len * G * N * sizeof(T)));
    float mrow[2][2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + q.row(mi, r), col = n0 + q.col(ni);
          const uint32_t off = col < N ? (uint32_t)((row * G + g) * N + col) * sizeof(T) : kPastRecords;
          mrow[mi][ni][r] = static_cast<float>(
              __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(rM, off, 0, 0)));
        }
    bf16x8 ra[2][NPA], rk[2][PP];
    float fl[2];
    // the row factors: thread t loads a and delta of tile row t % 64 (rows
    // < L: inside the chunk's row of the workspace) and at each head writes
    // f (the product's row factor) or g (what the sum takes: f, times
    // delta for dB) of that row to LDS, beside the head's operand tile
    __shared__ __align__(16) float fac[2][2][64];
    const int fr_row = threadIdx.x & 63, fr_k = (threadIdx.x >> 6) & 1;
    float fa[2], fd[2];
    auto fetch = [&](int set, int h) {     // no branch: see frag_buf
      const int64_t jh = (int64_t)j * H + h;
#pragma unroll
      for (int u = 0; u < NPA; ++u) {      // 16-byte pieces, PRA lanes per row
        const int i = threadIdx.x + kBwdThreads * u, r = m0 + i / PRA, c = (i % PRA) * 8;
        ra[set][u] = frag_buf(rrow, (uint32_t)(((r * H + h) * P + c) * sizeof(T)));
      }
      fa[set] = dAcs[jh * L + m0 + fr_row];
      fd[set] = delta[jh * L + m0 + fr_row];
      fl[set] = ld_vmem(dAcs + jh * L + len - 1);
#pragma unroll
      for (int u = 0; u < PP; ++u) {
        const int i = threadIdx.x + kBwdThreads * u, r = i >> 3, cc = (i & 7) * 8;
        rk[set][u] = frag_buf(rk16, (uint32_t)(((h * P + r) * N + n0 + cc) * sizeof(bf16)), n0 + cc < N);
      }
    };
    auto step = [&](int set, int h) {      // set = (h - h0) & 1, also the LDS buffer
      bf16* kb = kt[set];
#pragma unroll
      for (int u = 0; u < PP; ++u) {
        const int i = threadIdx.x + kBwdThreads * u;
        *reinterpret_cast<bf16x8*>(&kb[(i >> 3) * kKtPitch + (i & 7) * 8]) = rk[set][u];
      }
      {
        // rows past the chunk: factor 0 (their a and delta are not defined)
        const bool ok = m0 + fr_row < len;
        const float f = ok ? exp2_fast((which == 0 ? fa[set] : fl[set] - fa[set]) * kLog2e) : 0.f;
        const float gsum = which == 0 ? f : (ok ? fd[set] : 0.f) * f;
        fac[set][fr_k][fr_row] = fr_k ? gsum : f;   // threads 128-255 repeat 0-127
      }
#pragma unroll
      for (int u = 0; u < NPA; ++u) {
        const int i = threadIdx.x + kBwdThreads * u;
        *reinterpret_cast<bf16x8*>(&ta[set][(i / PRA) * RPA + (i % PRA) * 8]) = ra[set][u];
      }
      fetch(set, min(h + 2, h1 - 1));      // past the group's last head: that head again
      __builtin_amdgcn_sched_barrier(0);   // keep the sets' loads in issue order
      __syncthreads();                     // this head's operand tile stored
      f32x4 dh[2][2];                      // this head's product
      zero_quarter(dh);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 aop[2], b[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          aop[mi] = *reinterpret_cast<const bf16x8*>(&ta[set][(q.wr + mi * 16 + q.lr) * RPA + ks * 32 + q.kq]);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) b[ni] = lds_operand_kmajor(kb, kKtPitch, ks * 32, q.wc + ni * 16, q.lane);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) dh[mi][ni] = Mfma<bf16>::mma(aop[mi], b[ni], dh[mi][ni]);
      }
      // the row dots (a row's 16 lanes hold its columns): lane lr ends with
      // row (mi, r) = (lr >> 3, 2 ((lr >> 2) & 1) + ((lr >> 1) & 1)), one
      // store per head for the wave's rows; then the sum, rows scaled by g
      const int64_t jh = (int64_t)j * H + h;
      float v[8];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[4 * mi + r] = mrow[mi][0][r] * dh[mi][0][r] + mrow[mi][1][r] * dh[mi][1][r];
      {
        const float sum = row_sum16_x8(v, q.lr);
        const int rl = q.row(q.lr >> 3, 2 * ((q.lr >> 2) & 1) + ((q.lr >> 1) & 1));
        const __amdgpu_buffer_rsrc_t rp =
            buf_rsrc_u(part + (jh * SL + 2 * nt + (q.wc >> 5)) * L + m0, (uint32_t)((len - m0) * sizeof(float)));
        store_buf(rp, rl * sizeof(float), fac[set][0][rl] * sum, (q.lr & 1) == 0);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const float4 g4 = *reinterpret_cast<const float4*>(&fac[set][1][q.row(mi, 0)]);
        const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) d[mi][ni][r] += gv[r] * dh[mi][ni][r];
      }
    };
    fetch(0, h0);
    __builtin_amdgcn_sched_barrier(0);     // set 0's loads first, as in the loop
    fetch(1, min(h0 + 1, h1 - 1));
    __builtin_amdgcn_sched_barrier(0);
    int h = h0;
    for (; h + 1 < h1; h += 2) {           // whole pairs: every path through the loop
      step(0, h);                          // issues the same loads in the same order
      step(1, h + 1);
    }
    if (h < h1) step(0, h);                // an odd group's last head
    quarter_to_thread(q, d, acc, reinterpret_cast<float*>(region),   // its first barrier ends the heads
                      reinterpret_cast<float*>(region) + 32 * kGemmPitch);
  } else {
    if (which == 0) {                      // dC rows m0..m0+63: s runs to the tile's last row
      // rows l of the summed dCB (columns s <= l), rows s of B
      gemm_staged<float, true, T, false, 32, 1>(W + (int64_t)m0 * L, L, len - m0, nullptr,
                                                B + (t0 * G + g) * N + n0, (int64_t)G * N, N - n0, 0,
                                                min(len, m0 + 64), acc, As, Bs, m0);
    } else {                               // dB rows m0..m0+63: l runs from the tile's first row
      // rows l of the summed dCB (columns s <= l), rows l of C
      gemm_staged<float, false, T, false, 32, 2>(W + m0, L, len - m0, nullptr,
                                                 C + (t0 * G + g) * N + n0, (int64_t)G * N, N - n0, m0,
                                                 len, acc, As, Bs, m0);
    }
    // the state terms, head by head: the rows scaled by their factor
    // (staged in LDS), times the head's entering state or dS rows p; the
    // row dots of each head's product (one slot per column tile: the
    // tile's second slot is 0), then its sum
    __shared__ float sc[64], dsr[64];
    const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
    float mv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        const int r = m0 + tm + i, nn = n0 + tn + jn;
        mv[i][jn] = (r < len && nn < N) ? ld(M + ((t0 + r) * G + g) * N + nn) : 0.f;
      }
    for (int h = h0; h < h0 + hpg; ++h) {
      const int64_t jh = (int64_t)j * H + h;
      __syncthreads();                     // the previous head's factors consumed
      if (threadIdx.x < 64) {
        const int m = m0 + threadIdx.x;
        const float* ah = dAcs + jh * L;
        sc[threadIdx.x] = m >= len ? 0.f : exp2_fast((which == 0 ? ah[m] : ah[len - 1] - ah[m]) * kLog2e);
        dsr[threadIdx.x] = delta[jh * L + m];
      }
      float ah[4][4] = {};
      if (which == 0)
        gemm_staged<T, true, T, false>(dy + ((t0 + m0) * H + h) * P, (int64_t)H * P, len - m0, sc,
                                       states_in + jh * P * N + n0, N, N - n0, 0, P, ah, As, Bs);
      else
        gemm_staged<T, true, float, false>(x + ((t0 + m0) * H + h) * P, (int64_t)H * P, len - m0, sc,
                                           dS + jh * P * N + n0, N, N - n0, 0, P, ah, As, Bs);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + tm + i;
        float v = 0.f;
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) v += mv[i][jn] * ah[i][jn];
        v = row16_sum(v);
        if ((threadIdx.x & 15) == 0 && r < len) {
          part[(jh * SL + 2 * nt) * L + r] = v;
          part[(jh * SL + 2 * nt + 1) * L + r] = 0.f;
        }
        const float fr = which == 0 ? 1.f : dsr[tm + i];
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[i][jn] += fr * ah[i][jn];
      }
    }
  }
  T* out = which == 0 ? dC : dB;
  const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
  static_assert(N % 4 == 0, "4-wide pieces of a row");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + tm + i;
    if (r < len && n0 + tn < N)
      store4(out + ((t0 + r) * G + g) * N + n0 + tn, acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  }
}

// 3c. Per (chunk, head), one thread per token: da from the partial sums,
// its suffix sums, ddelta and ddt, and the chunk's parts of dA, dD and
// dt_bias.  grid (H, chunk slots), L threads.
template <typename T, int P, int N, int L>
__global__ __launch_bounds__(L) void bwd_token_kernel(
    ChunkMap cm, const float* __restrict__ dt, const float* __restrict__ dt_bias,
    const float* __restrict__ A, const float* __restrict__ delta, const float* __restrict__ dAcs,
    const float* __restrict__ ghpart, const float* __restrict__ rowpart,
    const float* __restrict__ colpart, const float* __restrict__ vxpart,
    const float* __restrict__ interpart, const float* __restrict__ ddot, int H, float dt_min,
    float dt_max, float* __restrict__ ddt, float* __restrict__ dA_part,
    float* __restrict__ dD_part, float* __restrict__ dbias_part) {
  __shared__ float red[3 * (L / kWave)];
  constexpr int LT = L / 64, VX = 2 * ((N + 63) / 64);   // row-dot slots per token
  constexpr int RH = sizeof(T) == 2 ? 2 : 1;              // V partial-sum slots per tile
  const int h = blockIdx.x, j = blockIdx.y, k = threadIdx.x;
  const ChunkDesc cd = cm.desc(j);
  const int64_t jh = (int64_t)j * H + h;
  if (cd.len <= 0) {                       // uniform over the workgroup
    if (k == 0) {
      dA_part[jh] = 0.f;
      dD_part[jh] = 0.f;
      dbias_part[jh] = 0.f;
    }
    return;
  }
  const int len = cd.len;
  const bool valid = k < len;
  const float* a = dAcs + jh * L;
  const float alast = a[len - 1];
  const float dk = delta[jh * L + k];
  const int64_t tk = cd.start + k;
  // Every partial sum of the token is loaded at once, without a branch: a
  // slot the token does not take (every slot, past the chunk's end) aims
  // past the records and reads zero, and the sums run in slot order.
  const int kt = k / 64;
  const uint32_t ko = (uint32_t)k * 4u;
  const __amdgpu_buffer_rsrc_t rrow = buf_rsrc_u(rowpart + jh * LT * RH * L, LT * RH * L * 4u);
  const __amdgpu_buffer_rsrc_t rcol = buf_rsrc_u(colpart + jh * LT * RH * L, LT * RH * L * 4u);
  const __amdgpu_buffer_rsrc_t rvx = buf_rsrc_u(vxpart + jh * VX * L, VX * L * 4u);
  const __amdgpu_buffer_rsrc_t rin = buf_rsrc_u(interpart + jh * VX * L, VX * L * 4u);
  float rp[LT][RH], cp[LT][RH], vp[VX], ip[VX];
#pragma unroll
  for (int st = 0; st < LT; ++st)
#pragma unroll
    for (int u = 0; u < RH; ++u) {
      const uint32_t o = (uint32_t)((st * RH + u) * L) * 4u + ko;
      rp[st][u] = buf_load4(rrow, valid && st <= kt ? o : kPastRecords);
      cp[st][u] = buf_load4(rcol, valid && st >= kt && st * 64 < len ? o : kPastRecords);
    }
#pragma unroll
  for (int v = 0; v < VX; ++v) {
    vp[v] = buf_load4(rvx, valid ? (uint32_t)(v * L) * 4u + ko : kPastRecords);
    ip[v] = buf_load4(rin, valid ? (uint32_t)(v * L) * 4u + ko : kPastRecords);
  }
  const float dd = valid ? ddot[jh * L + k] : 0.f;    // dy_k . x_k, from the V tiles
  float rowsum = 0.f, sdir = 0.f, inter = 0.f, vxe = 0.f;
#pragma unroll
  for (int st = 0; st < LT; ++st)
#pragma unroll
    for (int u = 0; u < RH; ++u) {
      rowsum += rp[st][u];
      sdir += cp[st][u];
    }
#pragma unroll
  for (int v = 0; v < VX; ++v) {
    vxe += vp[v];
    inter += ip[v];
  }
  const float vs = dk * vxe;
  // <dS_j, H_j>: the chain's partial sums, one per 256 state elements
  constexpr int NW = P * N / (4 * kWave);
  static_assert(NW <= L && (P * N) % (4 * kWave) == 0, "partial sums of <dS, H>");
  const float gh = k < NW ? ghpart[jh * NW + k] : 0.f;
  const float3 gt = block_sum3<L>(make_float3(gh, valid ? vs : 0.f, 0.f), red);
  float da = valid ? rowsum - dk * sdir + inter - vs : 0.f;
  if (k == len - 1) da += gt.y + expf(alast) * gt.x;
  const float rc = block_suffix_sum<L>(da, red);
  const float ddelta = sdir + vxe + A[h] * rc;
  float dbias = 0.f;
  if (valid) {
    const float u = dt[tk * H + h] + (dt_bias ? dt_bias[h] : 0.f);
    const float sp = fmaxf(u, 0.f) + log1pf(expf(-fabsf(u)));
    const float pass = (sp >= dt_min && sp <= dt_max) ? 1.f : 0.f;
    const float sig = 1.f / (1.f + expf(-u));
    dbias = ddelta * sig * pass;
    ddt[tk * H + h] = dbias;
  }
  const float3 sums = block_sum3<L>(make_float3(valid ? dk * rc : 0.f, dd, dbias), red);
  if (k == 0) {
    dA_part[jh] = sums.x;
    dD_part[jh] = sums.y;
    dbias_part[jh] = sums.z;
  }
}

// 5, with fp32 inputs and for a problem without chunks (with bf16 inputs
// dx's launch does it): dA, dD, dt_bias as sums over the chunk slots; one
// wave per head (lanes stride the slots, then a shuffle sum).  grid (H),
// kWave threads.
__global__ __launch_bounds__(kWave) void bwd_head_reduce_kernel(
    const float* __restrict__ dA_part, const float* __restrict__ dD_part,
    const float* __restrict__ dbias_part, int H, int nslots, float* __restrict__ dA,
    float* __restrict__ dD, float* __restrict__ dbias) {
  const int h = blockIdx.x;
  float sa = 0.f, sd = 0.f, sb = 0.f;
  for (int j = threadIdx.x; j < nslots; j += kWave) {
    sa += dA_part[(int64_t)j * H + h];
    sd += dD_part[(int64_t)j * H + h];
    sb += dbias_part[(int64_t)j * H + h];
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    sa += __shfl_xor(sa, off);
    sd += __shfl_xor(sd, off);
    sb += __shfl_xor(sb, off);
  }
  if (threadIdx.x == 0) {
    dA[h] = sa;
    if (dD) dD[h] = sd;
    if (dbias) dbias[h] = sb;
  }
}

}  // namespace

// Head blocks per group: the fewest (at most hpg and kBwdHeadBlocks) for
// which `wg_per_block` workgroups per block give kBwdMinWgPerCu workgroups
// per CU of the current device (CU count cached per device).
static int bwd_head_blocks(int hpg, int64_t wg_per_block) {
  const int cus = device_cu_count();
  const int cap = hpg < kBwdHeadBlocks ? hpg : kBwdHeadBlocks;
  if (cus <= 0) return cap;
  int hb = 1;
  while (hb < cap && wg_per_block * hb < (int64_t)kBwdMinWgPerCu * cus) ++hb;
  return hb;
}

// Depth of the reverse chain's ring: each chunk in flight holds about 18
// VGPRs, so the ring gets shallower as the chain's waves fill the device
// (4 SIMDs per CU): 8 chunks up to one wave per SIMD (long chains over few
// heads), 4 up to four, else 2.
static int bwd_chain_depth(int64_t waves) {
  const int cus = device_cu_count();
  if (cus <= 0) return 2;
  const int64_t simds = 4LL * cus;
  return waves <= simds ? 8 : waves <= 4 * simds ? 4 : 2;
}

template <typename T, int P, int N, int L>
hipError_t launch_backward(const FwdArgs& a, const BwdArgs& b, hipStream_t s) {
  const int mc = a.max_chunks, H = a.H, G = a.G, PN = P * N;
  const ChunkMap cm = a.cmap();
  if (mc <= 0) {                           // no tokens: dinit = dfinal, zero parameter gradients
    const int64_t ne = (int64_t)a.nstates * H * PN;
    if (b.dinit && ne > 0)
      hipLaunchKernelGGL(bwd_pass_final_kernel, dim3((unsigned)((ne + kBwdThreads - 1) / kBwdThreads)),
                         dim3(kBwdThreads), 0, s, b.dfinal, ne, b.dinit);
    hipLaunchKernelGGL(bwd_head_reduce_kernel, dim3(H), dim3(kWave), 0, s, b.dA_part, b.dD_part,
                       b.dbias_part, H, 0, b.dA, b.dD, b.ddt_bias);
    return hipGetLastError();
  }
  const T* x = (const T*)a.x;
  const T* B = (const T*)a.B;
  const T* C = (const T*)a.C;
  const T* dy = (const T*)b.dy;
  const T* cb = (const T*)a.cb;
  const T* hin = (const T*)a.states_in;
  constexpr int NT = (N + 63) / 64;
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((bwd_q_mfma_kernel<P, N, L>), dim3(xcd_grid(mc, ((P + 63) / 64) * H)),
                       dim3(kBwdThreads), 0, s, cm, mc, (const bf16*)dy, (const bf16*)C, a.dAcs, H, G, b.Q,
                       b.dla);
  else
    hipLaunchKernelGGL((bwd_q_tiled_kernel<T, P, N, L>), dim3(xcd_grid(mc, ((P + 63) / 64) * NT * H)),
                       dim3(kBwdThreads), 0, s, cm, mc, dy, C, a.dAcs, H, G, b.Q, b.dla);
  static_assert((P * N) % 4 == 0, "four state elements per thread");
  static_assert(PN % (4 * kWave) == 0, "whole waves of the chain");
  {
    const dim3 cg((PN / 4 + kBwdThreads - 1) / kBwdThreads, H, a.nstates);
    auto chain = [&](auto kern) {
      hipLaunchKernelGGL(kern, cg, dim3(kBwdThreads), 0, s, cm, b.Q, b.dla, b.dfinal, hin, H, PN,
                         sizeof(T) == 4 ? b.dS : nullptr,
                         sizeof(T) == 2 ? static_cast<bf16*>(b.dS16) : nullptr, b.ghpart, b.dinit);
    };
    const int depth = bwd_chain_depth((int64_t)cg.x * cg.y * cg.z * (kBwdThreads / kWave));
    if (depth == 8) chain(bwd_chain_kernel<T, 8>);
    else if (depth == 4) chain(bwd_chain_kernel<T, 4>);
    else chain(bwd_chain_kernel<T, 2>);
  }
  constexpr int LT = L / 64;
  // head blocks per group for the summed dCB: the fewest that fill the GPU
  // with 3a's workgroups (their partial sums fit the workspace's H L^2
  // floats per chunk: G * HB <= H)
  const int hpg = H / G, HB = bwd_head_blocks(hpg, (int64_t)(LT * (LT + 1) / 2) * G * mc);
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((bwd_v_mfma_kernel<P, L>), dim3(xcd_grid(mc, LT * (LT + 1) / 2 * G * HB)),
                       dim3(kBwdThreads), 0, s, cm, mc, (const bf16*)x, (const bf16*)dy, (const bf16*)cb,
                       a.delta, a.dAcs, H, G, HB, b.dcb, b.rowpart, b.colpart, b.ddot, static_cast<bf16*>(b.cbt),
                       static_cast<bf16*>(b.dcb16));
  else
    hipLaunchKernelGGL((bwd_v_tiled_kernel<T, P, N, L>), dim3(xcd_grid(mc, LT * (LT + 1) / 2 * G * HB)),
                       dim3(kBwdThreads), 0, s, cm, mc, x, dy, cb, a.delta, a.dAcs, H, G, HB, b.dcb,
                       b.rowpart, b.colpart, b.ddot);
  if (HB > 1)
    hipLaunchKernelGGL((bwd_dcb_sum_kernel<L>), dim3(LT * (LT + 1) / 2 * kDcbBlocksPerTile, G, mc),
                       dim3(kBwdThreads), 0, s, G, HB, b.dcb, sizeof(T) == 2 ? static_cast<bf16*>(b.dcb16) : nullptr);
  hipLaunchKernelGGL((bwd_bc_group_kernel<T, P, N, L>), dim3(xcd_grid(mc, LT * NT * 2 * G)),
                     dim3(kBwdThreads), 0, s, cm, mc, x, B, C, dy, a.delta, a.dAcs, hin, b.dS,
                     static_cast<const bf16*>(b.dS16), b.dcb, static_cast<const bf16*>(b.dcb16), H, G, HB,
                     (T*)b.dB, (T*)b.dC, b.interpart, b.vxpart);
  // the per-token pass, then dx; with bf16 inputs dx's launch also sums the
  // per-token pass's parts of dA, dD and dt_bias per head
  hipLaunchKernelGGL((bwd_token_kernel<T, P, N, L>), dim3(H, mc), dim3(L), 0, s, cm, a.dt, a.dt_bias,
                     a.A, a.delta, a.dAcs, b.ghpart, b.rowpart, b.colpart, b.vxpart, b.interpart,
                     b.ddot, H, a.dt_min, a.dt_max, b.ddt, b.dA_part, b.dD_part, b.dbias_part);
  if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((bwd_dx_scan_kernel<P, N, L>), dim3(xcd_grid(mc, H)), dim3(64 * kDxWaves<L>), 0, s,
                       cm, mc, (const bf16*)B, (const bf16*)dy, static_cast<const bf16*>(b.cbt), a.delta,
                       a.dAcs, static_cast<const bf16*>(b.dS16), a.D, H, G, (bf16*)b.dx, b.dA_part,
                       b.dD_part, b.dbias_part, b.dA, b.dD, b.ddt_bias);
  } else {
    hipLaunchKernelGGL((bwd_dx_tiled_kernel<T, P, N, L>), dim3(xcd_grid(mc, LT * ((P + 63) / 64) * H)),
                       dim3(kBwdThreads), 0, s, cm, mc, B, dy, cb, a.delta, a.dAcs, b.dS, a.D, H, G,
                       (T*)b.dx);
    hipLaunchKernelGGL(bwd_head_reduce_kernel, dim3(H), dim3(kWave), 0, s, b.dA_part, b.dD_part,
                       b.dbias_part, H, mc, b.dA, b.dD, b.ddt_bias);
  }
  return hipGetLastError();
}

#define SSD_BWD_INST(T, P, N, L) \
  template hipError_t launch_backward<T, P, N, L>(const FwdArgs&, const BwdArgs&, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_BWD_INST)
#undef SSD_BWD_INST

}  // namespace ssd
