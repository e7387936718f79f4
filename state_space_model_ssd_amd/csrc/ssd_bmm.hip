// Stage 2, bmm_chunk: CB[j,g,l,s] = sum_n C[t0+l,g,n] * B[t0+s,g,n] inside
// each logical chunk j, accumulated in fp32 and stored in the input dtype (the intra-chunk C B^T that the output construction
// of the chunked scan consumes; aiproviderindex.com, "Mamba-2 offers a
// different scaling path").  Only 64x64 tiles on or below the diagonal are
// computed, and diagonal tiles hold 0 above the diagonal: the output stage
// reads no tile with s > l and multiplies diagonal blocks unmasked.
//
// One workgroup (4 waves) per (chunk, group, lower-triangular 64x64 tile);
// every tile of chunk j runs on XCD j mod 8, so one L2 fetches its rows.
// C and B rows are staged in LDS as the MFMA operand type (rows padded by 16
// bytes); each wave computes a 32x32 quarter with 2x2 MFMA 16x16 tiles and
// K = dstate.  Rows past the chunk's valid length load as zeros.  The bf16
// forward runs the same tiles as extra workgroups of the chunk_state launch
// (ssd_chunk_state.hip); this standalone launch serves the stage-by-stage
// entry point and the fp32 path.
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {

template <typename T, int N, int L>
__global__ __launch_bounds__(256) void bmm_chunk_kernel(ChunkMap cm, int nslots,
                                                        const T* __restrict__ C,
                                                        const T* __restrict__ B, int G,
                                                        T* __restrict__ cb) {
  constexpr int LD = N + 16 / sizeof(T);
  __shared__ __align__(16) T Cs[64 * LD];
  __shared__ __align__(16) T Bs[64 * LD];
  constexpr int NTRI = (L / 64) * (L / 64 + 1) / 2;
  const int2 jt = xcd_chunk_head(blockIdx.x, G * NTRI);
  const int j = jt.x, g = jt.y / NTRI;
  if (j >= nslots) return;
  const int2 t = tri_tile(jt.y - g * NTRI);
  const ChunkDesc d = cm.desc(j);
  if (d.len <= 0 || t.x * 64 >= d.len) return;   // rows the output stage never reads
  bmm_tile<T, N, L>(d, j, g, t.x, t.y, C, B, G, cb, Cs, Bs);
}

}  // namespace

template <typename T, int N, int L>
hipError_t launch_bmm_chunk(const FwdArgs& a, hipStream_t s) {
  static_assert(L % 64 == 0, "chunk size must be a multiple of 64");
  static_assert(N % Mfma<T>::K == 0, "dstate must be a multiple of the MFMA K");
  if (a.max_chunks <= 0) return hipSuccess;
  constexpr int nt = L / 64;
  const int grid = xcd_grid(a.max_chunks, a.G * nt * (nt + 1) / 2);
  hipLaunchKernelGGL((bmm_chunk_kernel<T, N, L>), dim3(grid), dim3(256), 0, s, a.cmap(),
                     a.max_chunks, (const T*)a.C, (const T*)a.B, a.G, (T*)a.cb);
  return hipGetLastError();
}

#define SSD_INST_BMM(T, P, N, L) template hipError_t launch_bmm_chunk<T, N, L>(const FwdArgs&, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_INST_BMM)
#undef SSD_INST_BMM

}  // namespace ssd
