// Stage 2, bmm_chunk: CB[j,g,l,s] = sum_n C[t0+l,g,n] * B[t0+s,g,n] inside
// each logical chunk j, accumulated in fp32 and stored in the input dtype (the intra-chunk C B^T that the output construction
// of the chunked scan consumes; aiproviderindex.com, "Mamba-2 offers a
// different scaling path").  Only 64x64 tiles on or below the diagonal are
// computed: the output stage never reads s > l.
//
// One workgroup (4 waves) per (chunk, group, lower-triangular 64x64 tile).
// C and B rows are staged in LDS as the MFMA operand type (rows padded by 16
// bytes); each wave computes a 32x32 quarter with 2x2 MFMA 16x16 tiles and
// K = dstate.  Rows past the chunk's valid length load as zeros.
#include "ssd_kernels.h"

namespace ssd {

namespace {

template <typename T, int N, int L>
__global__ __launch_bounds__(256) void bmm_chunk_kernel(ChunkMap cm, const T* __restrict__ C,
                                                        const T* __restrict__ B, int G,
                                                        T* __restrict__ cb) {
  using M = Mfma<T>;
  constexpr int V = 16 / sizeof(T);   // elements per 16-byte vector
  constexpr int LD = N + V;           // padded LDS row
  constexpr int VPR = N / V;
  __shared__ __align__(16) T Cs[64 * LD];
  __shared__ __align__(16) T Bs[64 * LD];

  const int j = blockIdx.x / G, g = blockIdx.x - (blockIdx.x / G) * G;
  int t = blockIdx.y, ti = 0;
  while (t > ti) { t -= ti + 1; ++ti; }
  const int tj = t;
  const ChunkDesc d = cm.desc(j);
  if (d.len <= 0 || ti * 64 >= d.len) return;   // rows the output stage never reads

  const int tid = threadIdx.x;
  for (int i = tid; i < 64 * VPR; i += 256) {
    const int r = i / VPR, cv = i - (i / VPR) * VPR;
    const int lc = ti * 64 + r, lb = tj * 64 + r;
    const uint4 vc = load16(C + ((int64_t)(d.start + lc) * G + g) * N + cv * V, lc < d.len);
    const uint4 vb = load16(B + ((int64_t)(d.start + lb) * G + g) * N + cv * V, lb < d.len);
    *reinterpret_cast<uint4*>(&Cs[r * LD + cv * V]) = vc;
    *reinterpret_cast<uint4*>(&Bs[r * LD + cv * V]) = vb;
  }
  __syncthreads();

  const int w = tid / kWave, lane = tid & (kWave - 1);
  const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
  const int lr = lane & 15, kq = (lane >> 4) * M::KPL;
  f32x4 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 4
  for (int k0 = 0; k0 < N; k0 += M::K) {
    typename M::frag a[2], b[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) a[mi] = M::load(&Cs[(wr + mi * 16 + lr) * LD + k0 + kq]);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) b[ni] = M::load(&Bs[(wc + ni * 16 + lr) * LD + k0 + kq]);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = M::mma(a[mi], b[ni], acc[mi][ni]);
  }

  T* out = cb + ((int64_t)j * G + g) * L * L;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = ti * 64 + wr + mi * 16 + (lane >> 4) * 4 + r;
        const int col = tj * 64 + wc + ni * 16 + lr;
        out[(int64_t)row * L + col] = from_f32<T>(acc[mi][ni][r]);
      }
}

}  // namespace

template <typename T, int N, int L>
hipError_t launch_bmm_chunk(const FwdArgs& a, hipStream_t s) {
  static_assert(L % 64 == 0, "chunk size must be a multiple of 64");
  static_assert(N % Mfma<T>::K == 0, "dstate must be a multiple of the MFMA K");
  if (a.max_chunks <= 0) return hipSuccess;
  constexpr int nt = L / 64;
  dim3 grid(a.max_chunks * a.G, nt * (nt + 1) / 2);
  hipLaunchKernelGGL((bmm_chunk_kernel<T, N, L>), grid, dim3(256), 0, s, a.cmap(),
                     (const T*)a.C, (const T*)a.B, a.G, (T*)a.cb);
  return hipGetLastError();
}

#define SSD_INST_BMM(T, P, N, L) template hipError_t launch_bmm_chunk<T, N, L>(const FwdArgs&, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_INST_BMM)
#undef SSD_INST_BMM

}  // namespace ssd
