// Stage 3, chunk_state: the state each logical chunk j would produce from a
// zero start (clova.ai, table "Share of compute time by kernel":
// _chunk_state_fwd),
//   S[j,h,p,n] = sum_{l < len} w[l] * x[t0+l,h,p] * B[t0+l,g,n],
//   w[l]       = exp(dAcs[len-1] - dAcs[l]) * delta[l].
// A P x N result with a K = chunk-length contraction over tokens: MFMA.
//
// One workgroup (4 waves) per (chunk, head).  Tokens are the contraction
// index, and both operands arrive token-major from HBM, so each 64-token
// slice is transposed on its way into LDS (k contiguous per row, 16-byte
// padded rows): x scaled by w[l] and rounded once to the operand type, B
// as is.  The waves split the P x N output into rectangles of 16x16 tiles.
#include "ssd_kernels.h"

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

  const int w = tid / kWave, lane = tid & (kWave - 1);
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

}  // namespace

template <typename T, int P, int N, int L>
hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t s) {
  if (a.max_chunks <= 0) return hipSuccess;
  dim3 grid(a.max_chunks, a.H);
  hipLaunchKernelGGL((chunk_state_kernel<T, P, N, L>), grid, dim3(256), 0, s, a.cmap(),
                     (const T*)a.x, (const T*)a.B, a.delta, a.dAcs, a.H, a.G, a.chunk_states);
  return hipGetLastError();
}

#define SSD_INST(T, P, N, L) template hipError_t launch_chunk_state<T, P, N, L>(const FwdArgs&, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_INST)
#undef SSD_INST

}  // namespace ssd
