// Stage 5, chunk_scan: the output construction (clova.ai, table "Share of
// compute time by kernel": _chunk_scan_fwd; aiproviderindex.com, "Mamba-2
// offers a different scaling path": output construction).  For token l of
// logical chunk j, head h, group g:
//   y[l,p] = sum_{s <= l} CB[l,s] * exp(dAcs[l] - dAcs[s]) * delta[s] * x[s,p]
//          + exp(dAcs[l]) * sum_n C[l,n] * states_in[j,h,p,n]
//          + D[h] * x[l,p]
// accumulated in fp32 and rounded once to the output type.
//
// One workgroup (4 waves) per (chunk, 64-row tile, head); each wave owns 16
// output rows and all P columns (P/16 MFMA tiles).
//  - intra-chunk term: the A operand (decay-masked CB row) is built per lane
//    in registers; the mask is applied by selection before the exponential,
//    so the upper triangle never evaluates exp of a positive argument.  x is
//    the B operand, staged per 64-token slice in LDS transposed (k = token
//    contiguous).  Slices past the wave's last row are skipped.
//  - inter-chunk term: C rows and the entering state are read straight from
//    HBM in operand layout (n contiguous) and contracted over n; the row
//    scale exp(dAcs[l]) is applied to that partial sum.
//  - skip term: x of the diagonal slice is still in LDS.
#include "ssd_kernels.h"

namespace ssd {

namespace {

__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
__device__ __forceinline__ void store_pair(bf16* p, float a, float b) {
  bf16x2 v;
  v[0] = static_cast<bf16>(a);
  v[1] = static_cast<bf16>(b);
  *reinterpret_cast<bf16x2*>(p) = v;
}

// KPL consecutive fp32 values of a CB row (16- or 32-byte aligned).
template <int KPL>
__device__ __forceinline__ void load_cb(const float* p, float* v) {
  if constexpr (KPL == 1) {
    v[0] = *p;
  } else {
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q) {
      const float4 t = reinterpret_cast<const float4*>(p)[q];
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
  }
}

template <typename T> __device__ __forceinline__ typename Mfma<T>::frag zero_frag();
template <> __device__ __forceinline__ float zero_frag<float>() { return 0.f; }
template <> __device__ __forceinline__ bf16x8 zero_frag<bf16>() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<bf16>(0.f);
  return z;
}

template <typename T, int P, int N, int L>
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    ChunkMap cm, const T* __restrict__ x, const T* __restrict__ C, const float* __restrict__ cb,
    const float* __restrict__ delta, const float* __restrict__ dAcs,
    const T* __restrict__ states_in, const float* __restrict__ D, int H, int G,
    T* __restrict__ out) {
  using M = Mfma<T>;
  constexpr int RT = 64;                 // output rows per workgroup
  constexpr int NRT = L / RT;
  constexpr int KS = 64;                 // tokens per LDS slice
  constexpr int V = 16 / sizeof(T);
  constexpr int LDK = KS + V;
  constexpr int PT = P / 16;
  constexpr int KPL = M::KPL;

  __shared__ __align__(16) T xT[P * LDK];
  __shared__ float dAs[L];
  __shared__ float dls[L];

  const int j = blockIdx.x / NRT, rt = blockIdx.x - (blockIdx.x / NRT) * NRT;
  const int h = blockIdx.y, g = h / (H / G);
  const ChunkDesc d = cm.desc(j);
  if (d.len <= 0 || rt * RT >= d.len) return;

  const int tid = threadIdx.x;
  {
    const float* dA = dAcs + ((int64_t)j * H + h) * L;
    const float* dl = delta + ((int64_t)j * H + h) * L;
    for (int l = tid; l < L; l += 256) {
      dAs[l] = dA[l];
      dls[l] = dl[l];
    }
  }
  const int w = tid / kWave, lane = tid & (kWave - 1);
  const int lr = lane & 15, kq = (lane >> 4) * KPL;
  const int row0 = rt * RT + w * 16;     // first output row of this wave
  const int my_row = row0 + lr;          // A-operand row of this lane
  const bool row_ok = my_row < d.len;
  const float* cbrow = cb + (((int64_t)j * G + g) * L + my_row) * L;

  f32x4 acc[PT];
#pragma unroll
  for (int a = 0; a < PT; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const float dA_row = dAs[my_row];

  for (int sl = 0; sl <= rt; ++sl) {
    const int s0 = sl * KS;
    for (int i = tid; i < (KS / 2) * (P / V); i += 256) {
      const int pr = i % (KS / 2), seg = i / (KS / 2);
      const int l = s0 + 2 * pr;
      float v0[V], v1[V];
      load16_as_f32(x + ((int64_t)(d.start + l) * H + h) * P + seg * V, l < d.len, v0);
      load16_as_f32(x + ((int64_t)(d.start + l + 1) * H + h) * P + seg * V, l + 1 < d.len, v1);
#pragma unroll
      for (int e = 0; e < V; ++e) store_pair(&xT[(seg * V + e) * LDK + 2 * pr], v0[e], v1[e]);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; kk += M::K) {
      const int sb = s0 + kk;
      if (sb > row0 + 15) break;         // wave-uniform: past this wave's last row
      const int sf = sb + kq;            // first k of this lane
      float cbv[KPL], m[KPL];
      load_cb<KPL>(cbrow + sf, cbv);
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int s = sf + e;
        const bool ok = row_ok && s <= my_row && s < d.len;
        const float arg = ok ? dA_row - dAs[s] : 0.f;
        m[e] = ok ? cbv[e] * fexp<T>(arg) * dls[s] : 0.f;
      }
      const typename M::frag fa = M::pack(m);
#pragma unroll
      for (int a = 0; a < PT; ++a) {
        const typename M::frag fb = M::load(&xT[(a * 16 + lr) * LDK + kk + kq]);
        acc[a] = M::mma(fa, fb, acc[a]);
      }
    }
    if (sl < rt) __syncthreads();        // the diagonal slice stays for the skip term
  }

  // inter-chunk term over n
  f32x4 acc2[PT];
#pragma unroll
  for (int a = 0; a < PT; ++a) acc2[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  const T* crow = C + ((int64_t)(d.start + my_row) * G + g) * N;
  const T* hs = states_in + ((int64_t)j * H + h) * P * N;
#pragma unroll 4
  for (int k0 = 0; k0 < N; k0 += M::K) {
    const typename M::frag fa = row_ok ? M::load(crow + k0 + kq) : zero_frag<T>();
#pragma unroll
    for (int a = 0; a < PT; ++a) {
      const typename M::frag fb = M::load(hs + (a * 16 + lr) * N + k0 + kq);
      acc2[a] = M::mma(fa, fb, acc2[a]);
    }
  }

  const float Dh = D ? D[h] : 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + (lane >> 4) * 4 + r;
    if (row >= d.len) continue;
    const float sc = fexp<T>(dAs[row]);
    T* yrow = out + ((int64_t)(d.start + row) * H + h) * P;
#pragma unroll
    for (int a = 0; a < PT; ++a) {
      const int p = a * 16 + lr;
      const float xv = to_f32(xT[p * LDK + (row - rt * KS)]);
      yrow[p] = from_f32<T>(acc[a][r] + sc * acc2[a][r] + Dh * xv);
    }
  }
}

}  // namespace

template <typename T, int P, int N, int L>
hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t s) {
  static_assert(L % 64 == 0, "chunk size must be a multiple of 64");
  if (a.max_chunks <= 0) return hipSuccess;
  dim3 grid(a.max_chunks * (L / 64), a.H);
  hipLaunchKernelGGL((chunk_scan_kernel<T, P, N, L>), grid, dim3(256), 0, s, a.cmap(),
                     (const T*)a.x, (const T*)a.C, a.cb, a.delta, a.dAcs,
                     (const T*)a.states_in, a.D, a.H, a.G, (T*)a.out);
  return hipGetLastError();
}

#define SSD_INST(T, P, N, L) template hipError_t launch_chunk_scan<T, P, N, L>(const FwdArgs&, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_INST)
#undef SSD_INST

}  // namespace ssd
