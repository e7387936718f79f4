// Device-side building blocks shared by more than one SSD kernel (internal).
#pragma once

#include "ssd_common.h"

namespace ssd {

// softplus(u) = log(1 + e^u) in its overflow-free form, then the clamp.
__device__ __forceinline__ float step_from_raw(float u, float dt_min, float dt_max) {
  const float sp = fmaxf(u, 0.f) + log1pf(expf(-fabsf(u)));
  return fminf(fmaxf(sp, dt_min), dt_max);
}

// Discretised step of token l of chunk d and the chunk-local inclusive
// running sum of step * A (the chunk_cumsum stage for one (chunk, head)).
// Every thread of the workgroup must call it (it holds a barrier); threads
// with l >= L contribute nothing.  Past the chunk's end the step is 0 and the
// running sum stays flat.  `wave_tot` is LDS scratch of blockDim / 64 floats.
template <int L>
__device__ __forceinline__ void chunk_cumsum_block(const ChunkDesc& d, int l,
                                                   const float* __restrict__ dt,
                                                   const float* __restrict__ dt_bias,
                                                   const float* __restrict__ A, int H, int h,
                                                   float dt_min, float dt_max, float* wave_tot,
                                                   float& step, float& cum) {
  float dl = 0.f;
  if (l < d.len) dl = step_from_raw(dt[(int64_t)(d.start + l) * H + h] + (dt_bias ? dt_bias[h] : 0.f),
                                    dt_min, dt_max);
  float v = l < L ? dl * A[h] : 0.f;
  const int lane = l & (kWave - 1), wv = l / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  constexpr int NW = L / kWave;
  if constexpr (NW > 1) {
    if (lane == kWave - 1 && wv < NW) wave_tot[wv] = v;
    __syncthreads();
    float add = 0.f;
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) add += (w < wv) ? wave_tot[w] : 0.f;
    v += add;
  }
  step = dl;
  cum = v;
}

// One lower-triangular 64x64 tile (ti >= tj) of CB = C B^T for chunk d and
// group g, accumulated in fp32 on MFMA and stored in T.  TH threads (4 or 8
// waves: each wave owns 4 or 2 of the 16 output 16x16 tiles); Cs and Bs are
// LDS tiles of 64 x (N + 16 bytes).  Rows past the chunk's end load as zeros,
// so their CB entries are exactly 0.  A diagonal tile (ti == tj) stores 0
// above the diagonal (s > l): the stored CB is causal, and a consumer may
// multiply whole 32- or 64-token blocks of a row without masking them.
//
// AUX: cache-policy bits of the CB stores (bf16 only; kSc1 when another
// workgroup of the same launch reads them).  OPQ: the tile runs inside a
// persistent loop.
template <typename T, int N, int L, int TH = 256, int AUX = 0, bool OPQ = false>
__device__ __forceinline__ void bmm_tile(const ChunkDesc& d, int j, int g, int ti, int tj,
                                         const T* __restrict__ C, const T* __restrict__ B, int G,
                                         T* __restrict__ cb, T* Cs, T* Bs) {
  using M = Mfma<T>;
  static_assert(TH == 256 || TH == 512, "4 or 8 waves");
  constexpr int V = 16 / sizeof(T);   // elements per 16-byte vector
  constexpr int LD = N + V;           // padded LDS row
  constexpr int VPR = N / V;
  constexpr int MI = TH == 256 ? 2 : 1;   // 16-row tiles per wave
  const int tid = body_tid<OPQ, TH>();
  for (int i = tid; i < 64 * VPR; i += TH) {
    const int r = i / VPR, cv = i - (i / VPR) * VPR;
    const int lc = ti * 64 + r, lb = tj * 64 + r;
    const uint4 vc = load16(C + ((int64_t)(d.start + lc) * G + g) * N + cv * V, lc < d.len);
    const uint4 vb = load16(B + ((int64_t)(d.start + lb) * G + g) * N + cv * V, lb < d.len);
    *reinterpret_cast<uint4*>(&Cs[r * LD + cv * V]) = vc;
    *reinterpret_cast<uint4*>(&Bs[r * LD + cv * V]) = vb;
  }
  __syncthreads();
  const int w = wave_id(), lane = tid & (kWave - 1);
  const int wr = TH == 256 ? (w >> 1) * 32 : (w >> 1) * 16, wc = (w & 1) * 32;
  const int lr = lane & 15, kq = (lane >> 4) * M::KPL;
  f32x4 acc[MI][2];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k0 = 0; k0 < N; k0 += M::K) {
    typename M::frag a[MI], b[2];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) a[mi] = M::load(&Cs[(wr + mi * 16 + lr) * LD + k0 + kq]);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) b[ni] = M::load(&Bs[(wc + ni * 16 + lr) * LD + k0 + kq]);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = M::mma(a[mi], b[ni], acc[mi][ni]);
  }
  T* out = cb + ((int64_t)j * G + g) * L * L;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = ti * 64 + wr + mi * 16 + (lane >> 4) * 4 + r;
        const int col = tj * 64 + wc + ni * 16 + lr;
        if constexpr (AUX == 0) {
          out[(int64_t)row * L + col] = from_f32<T>(col <= row ? acc[mi][ni][r] : 0.f);
        } else {
          static_assert(sizeof(T) == 2, "write-through CB stores are bf16");
          buf_store2<AUX>(buf_rsrc(out, L * L * 2), ((uint32_t)row * L + col) * 2u,
                          from_f32<T>(col <= row ? acc[mi][ni][r] : 0.f));
        }
      }
}

// Lower-triangular tile index t -> (ti, tj), tj <= ti.
__device__ __forceinline__ int2 tri_tile(int t) {
  int ti = 0;
  while (t > ti) { t -= ti + 1; ++ti; }
  return make_int2(ti, t);
}

}  // namespace ssd
