// Stage 3, chunk_state: the state each logical chunk j would produce from a
// zero start (clova.ai, table "Share of compute time by kernel":
// _chunk_state_fwd),
//   S[j,h,p,n] = sum_{l < len} w[l] * x[t0+l,h,p] * B[t0+l,g,n],
//   w[l]       = exp(dAcs[len-1] - dAcs[l]) * delta[l].
// A P x N result with a K = chunk-length contraction over tokens: MFMA.
//
// One workgroup (4 waves) per (chunk, head); the waves split the P x N
// output into rectangles of 16x16 tiles.  Tokens are the contraction index
// and both operands arrive token-major from HBM.
//  - bf16 kernel (production): each 64-token slice of x (scaled by w[l] and
//    rounded once to bf16) and of B is staged in LDS in its natural
//    token-major layout with coalesced 16-byte accesses, and the MFMA A and B
//    operands come out of it through the gfx950 LDS transpose read.  The next
//    slice is loaded into registers while the current one is multiplied.
//    Workgroups of one chunk share an XCD, so B stays in its L2.
//  - fp32 kernel (exactness path): each slice is transposed on its way into
//    LDS (k contiguous per row, 16-byte padded rows).
#include "ssd_device.h"
#include "ssd_kernels.h"
#include "ssd_state_tile.h"

namespace ssd {

namespace {

// Store a pair of consecutive-k values of one LDS row.
__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
__device__ __forceinline__ void store_pair(bf16* p, float a, float b) {
  bf16x2 v;
  v[0] = static_cast<bf16>(a);
  v[1] = static_cast<bf16>(b);
  *reinterpret_cast<bf16x2*>(p) = v;
}

template <typename T, int P, int N, int L>
__global__ __launch_bounds__(256) void chunk_state_kernel(
    ChunkMap cm, const T* __restrict__ x, const T* __restrict__ B,
    const float* __restrict__ delta, const float* __restrict__ dAcs, int H, int G,
    float* __restrict__ S) {
  using M = Mfma<T>;
  constexpr int KS = 64;                 // tokens per LDS slice
  constexpr int V = 16 / sizeof(T);      // elements per 16-byte vector
  constexpr int LDK = KS + V;            // padded LDS row (k = token)
  constexpr int PT = P / 16, NT = N / 16;
  constexpr int WN = NT < 4 ? NT : 4;                  // waves along n
  constexpr int WP = (4 / WN) < PT ? (4 / WN) : PT;    // waves along p
  constexpr int TP = PT / WP, TN = NT / WN;            // tiles per wave
  static_assert(PT % WP == 0 && NT % WN == 0, "tile split");

  __shared__ __align__(16) T xT[P * LDK];
  __shared__ __align__(16) T bT[N * LDK];
  __shared__ float wl[L];

  const int j = blockIdx.x, h = blockIdx.y, g = h / (H / G);
  const ChunkDesc d = cm.desc(j);
  if (d.len <= 0) return;
  const int tid = threadIdx.x;
  const float* dA = dAcs + ((int64_t)j * H + h) * L;
  const float* dl = delta + ((int64_t)j * H + h) * L;
  const float last = dA[d.len - 1];
  for (int l = tid; l < L; l += 256) wl[l] = (l < d.len) ? fexp<T>(last - dA[l]) * dl[l] : 0.f;

  const int w = wave_id(), lane = tid & (kWave - 1);
  const bool active = w < WP * WN;
  const int wp = w / WN, wn = w - (w / WN) * WN;
  const int lr = lane & 15, kq = (lane >> 4) * M::KPL;
  f32x4 acc[TP][TN];
#pragma unroll
  for (int a = 0; a < TP; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const int nslices = (d.len + KS - 1) / KS;
  for (int sl = 0; sl < nslices; ++sl) {
    const int l0 = sl * KS;
    // x: row pairs (l, l+1) x 16-byte segments, scaled and transposed
    for (int i = tid; i < (KS / 2) * (P / V); i += 256) {
      const int pr = i % (KS / 2), seg = i / (KS / 2);
      const int l = l0 + 2 * pr;
      float v0[V], v1[V];
      load16_as_f32(x + ((int64_t)(d.start + l) * H + h) * P + seg * V, l < d.len, v0);
      load16_as_f32(x + ((int64_t)(d.start + l + 1) * H + h) * P + seg * V, l + 1 < d.len, v1);
      const float w0 = wl[l], w1 = wl[l + 1];
#pragma unroll
      for (int e = 0; e < V; ++e) store_pair(&xT[(seg * V + e) * LDK + 2 * pr], v0[e] * w0, v1[e] * w1);
    }
    // B: same transposition, no scaling
    for (int i = tid; i < (KS / 2) * (N / V); i += 256) {
      const int pr = i % (KS / 2), seg = i / (KS / 2);
      const int l = l0 + 2 * pr;
      float v0[V], v1[V];
      load16_as_f32(B + ((int64_t)(d.start + l) * G + g) * N + seg * V, l < d.len, v0);
      load16_as_f32(B + ((int64_t)(d.start + l + 1) * G + g) * N + seg * V, l + 1 < d.len, v1);
#pragma unroll
      for (int e = 0; e < V; ++e) store_pair(&bT[(seg * V + e) * LDK + 2 * pr], v0[e], v1[e]);
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int kk = 0; kk < KS; kk += M::K) {
        typename M::frag fa[TP], fb[TN];
#pragma unroll
        for (int a = 0; a < TP; ++a) fa[a] = M::load(&xT[((wp * TP + a) * 16 + lr) * LDK + kk + kq]);
#pragma unroll
        for (int b = 0; b < TN; ++b) fb[b] = M::load(&bT[((wn * TN + b) * 16 + lr) * LDK + kk + kq]);
#pragma unroll
        for (int a = 0; a < TP; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b) acc[a][b] = M::mma(fa[a], fb[b], acc[a][b]);
      }
    }
    __syncthreads();
  }

  if (!active) return;
  float* out = S + ((int64_t)j * H + h) * P * N;
#pragma unroll
  for (int a = 0; a < TP; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = (wp * TP + a) * 16 + (lane >> 4) * 4 + r;
        const int n = (wn * TN + b) * 16 + lr;
        out[(int64_t)p * N + n] = acc[a][b][r];
      }
}


template <int P, int N, int L>
__global__ __launch_bounds__(kStateThreads) void chunk_state_bf16_kernel(
    ChunkMap cm, int nslots, const bf16* __restrict__ x, const bf16* __restrict__ B,
    float* __restrict__ delta, float* __restrict__ dAcs, int H, int G, float* __restrict__ S) {
  __shared__ __align__(16) StateSmem<P, N, L> sm;
  const int2 jh = xcd_chunk_head(blockIdx.x, H);
  if (jh.x >= nslots) return;
  const ChunkDesc d = cm.desc(jh.x);
  if (d.len <= 0) return;
  chunk_state_bf16_body<P, N, L, false>(d, jh.x, jh.y, x, B, delta, dAcs, nullptr, nullptr,
                                        nullptr, 0.f, 0.f, H, G, S, sm);
}

// The front of the bf16 forward in one launch: the first `nstate` workgroups
// run chunk_cumsum + chunk_state for one (chunk, head) each, the rest compute
// bmm_chunk tiles.  The three stages are independent of each other's outputs
// here, so they share the machine instead of running back to back; the short
// bmm workgroups come last and fill the CUs the chunk_state tail leaves idle.
//
// With nclear > 0 the last nclear workgroups set the `nzero` ints at `zero` to
// 0 (the counters the fused forward's next launch counts on).
template <int P, int N, int L>
__global__ __launch_bounds__(kStateThreads) void front_bf16_kernel(
    ChunkMap cm, int nslots, int nstate, int nbmm, int G, const bf16* __restrict__ x,
    const bf16* __restrict__ B, const bf16* __restrict__ C, const float* __restrict__ dt,
    const float* __restrict__ dt_bias, const float* __restrict__ A, float dt_min, float dt_max,
    int H, float* __restrict__ delta, float* __restrict__ dAcs, bf16* __restrict__ cb,
    float* __restrict__ S, int* __restrict__ zero, int64_t nzero) {
  constexpr int LDB = N + 8;
  constexpr int NTRI = (L / 64) * (L / 64 + 1) / 2;
  constexpr size_t kBmm = 2 * 64 * LDB * sizeof(bf16);
  constexpr size_t kState = sizeof(StateSmem<P, N, L>);
  __shared__ __align__(16) unsigned char smem[kBmm > kState ? kBmm : kState];
  const int b = blockIdx.x;
  if (b >= nstate + nbmm) {
    const int64_t i = (int64_t)(b - nstate - nbmm) * kStateThreads + threadIdx.x;
    if (i < nzero) zero[i] = 0;
    return;
  }
  if (b >= nstate) {
    // nstate is a multiple of 8, so the bmm tiles of chunk j run on the XCD
    // of its chunk_state workgroups, and one L2 fetches its B and C rows
    const int2 jt = xcd_chunk_head(b - nstate, G * NTRI);
    const int j = jt.x, g = jt.y / NTRI, tile = jt.y - (jt.y / NTRI) * NTRI;
    if (j >= nslots) return;
    const int2 t = tri_tile(tile);
    const ChunkDesc d = cm.desc(j);
    if (d.len <= 0 || t.x * 64 >= d.len) return;
    bf16* Cs = reinterpret_cast<bf16*>(smem);
    bmm_tile<bf16, N, L, kStateThreads>(d, j, g, t.x, t.y, C, B, G, cb, Cs, Cs + 64 * LDB);
    return;
  }
  const int2 jh = xcd_chunk_head(b, H);
  if (jh.x >= nslots) return;
  const ChunkDesc d = cm.desc(jh.x);
  if (d.len <= 0) return;
  chunk_state_bf16_body<P, N, L, true>(d, jh.x, jh.y, x, B, delta, dAcs, dt, dt_bias, A, dt_min,
                                       dt_max, H, G, S,
                                       *reinterpret_cast<StateSmem<P, N, L>*>(smem));
}
}  // namespace

template <typename T, int P, int N, int L>
hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t s) {
  if (a.max_chunks <= 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((chunk_state_bf16_kernel<P, N, L>), dim3(xcd_grid(a.max_chunks, a.H)),
                       dim3(kStateThreads), 0, s, a.cmap(), a.max_chunks, (const bf16*)a.x,
                       (const bf16*)a.B, a.delta, a.dAcs, a.H, a.G, a.chunk_states);
  } else {
    dim3 grid(a.max_chunks, a.H);
    hipLaunchKernelGGL((chunk_state_kernel<T, P, N, L>), grid, dim3(256), 0, s, a.cmap(),
                       (const T*)a.x, (const T*)a.B, a.delta, a.dAcs, a.H, a.G, a.chunk_states);
  }
  return hipGetLastError();
}

template <typename T, int P, int N, int L>
hipError_t launch_front(const FwdArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorInvalidValue;           // the fp32 path runs the stages one by one
  } else {
    if (a.max_chunks <= 0) return hipSuccess;
    constexpr int ntri = (L / 64) * (L / 64 + 1) / 2;
    const int nbmm = xcd_grid(a.max_chunks, a.G * ntri);
    const int nstate = xcd_grid(a.max_chunks, a.H);
    const int nclear = (int)((a.zero_ints + kStateThreads - 1) / kStateThreads);
    hipLaunchKernelGGL((front_bf16_kernel<P, N, L>), dim3(nstate + nbmm + nclear),
                       dim3(kStateThreads), 0, s, a.cmap(), a.max_chunks, nstate, nbmm, a.G,
                       (const bf16*)a.x, (const bf16*)a.B, (const bf16*)a.C, a.dt, a.dt_bias,
                       a.A, a.dt_min, a.dt_max, a.H, a.delta, a.dAcs, (bf16*)a.cb,
                       a.chunk_states, a.sync, a.zero_ints);
    return hipGetLastError();
  }
}

#define SSD_INST(T, P, N, L)                                                           \
  template hipError_t launch_chunk_state<T, P, N, L>(const FwdArgs&, hipStream_t); \
  template hipError_t launch_front<T, P, N, L>(const FwdArgs&, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_INST)
#undef SSD_INST

}  // namespace ssd
