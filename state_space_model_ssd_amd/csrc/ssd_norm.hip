// The gated RMS norm that follows the SSD in a Mamba-2 layer, forward and
// backward.  The pages name it only through its backward kernel,
// _layer_norm_bwd, the layer's largest single share of time and memory-bound
// (clova.ai, table "Share of compute time by kernel"; the case study "The
// highway got wider..." and "How we fixed it": at 8 TB/s a memory-bound
// kernel needs many more bytes in flight than its old launch heuristic gave
// it).  Per row (token) and per group of `group_size` consecutive channels:
//   g_c   = y_c * silu(z_c)
//   r     = 1 / sqrt(mean_{c in group} g_c^2 + eps)
//   out_c = g_c * r * w_c
// and the backward of sum(out * dout):
//   u_c = g_c r,  du_c = dout_c w_c,  dw_c = sum over rows of dout_c u_c
//   dg_c = r (du_c - u_c mean_{c' in group}(du_c' u_c'))
//   dy_c = dg_c silu(z_c),  dz_c = dg_c y_c sigma(z_c) (1 + z_c (1 - sigma(z_c)))
//
// One workgroup of TH threads (64 to 256: the row's 16-byte vectors rounded
// up to a wave, at most 256) per row at a time; thread t owns the row's
// vectors t, t + TH, ... (KT of them), so every access is a coalesced
// 16-byte load and a thread's channels never change from row to row.  A group spans NV = group_size / V consecutive vectors: for NV <= 64 (a
// power of two) a group is an aligned run of NV lanes of one wave and reduces
// with xor shuffles inside the run; for NV a multiple of 64 a group is NV / 64
// consecutive 64-vector chunks, each reduced over its wave, and the chunk
// sums are added in LDS in chunk order.  A thread sums its elements in order
// and the shuffles run from the smallest offset up, the same order as the
// fused chunk_scan epilogue, so both round alike.  Workgroups walk rows with a
// stride of the grid, about eight workgroups per CU, so several rows of loads
// are in flight on every CU.
//
// The weight gradient: each thread accumulates dout * u for its own channels
// over the rows its workgroup visits and writes one partial row per
// workgroup; a second kernel sums the partials in workgroup order.  No
// atomics: results are deterministic.
#include "ssd_gate.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kNormThreads = 256;  // most threads of a norm workgroup
constexpr int kNormMaxKT = 4;    // vectors per thread: channels <= 1024 V

template <typename T> struct NormVec;
template <> struct NormVec<bf16> {
  static constexpr int V = 8;
  __device__ static void unpack(const uint4& q, float* f) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = static_cast<float>(b[e]);
  }
  __device__ static uint4 pack(const float* f) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = static_cast<bf16>(f[e]);
    return __builtin_bit_cast(uint4, b);
  }
};
template <> struct NormVec<float> {
  static constexpr int V = 4;
  __device__ static void unpack(const uint4& q, float* f) {
    f[0] = __builtin_bit_cast(float, q.x);
    f[1] = __builtin_bit_cast(float, q.y);
    f[2] = __builtin_bit_cast(float, q.z);
    f[3] = __builtin_bit_cast(float, q.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(__builtin_bit_cast(uint32_t, f[0]), __builtin_bit_cast(uint32_t, f[1]),
                      __builtin_bit_cast(uint32_t, f[2]), __builtin_bit_cast(uint32_t, f[3]));
  }
};

// v plus the value of the lane that DPP control CTRL selects.
template <int CTRL>
__device__ __forceinline__ float dpp_xadd(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false);
  return v + __builtin_bit_cast(float, o);
}

// run_sum's butterfly (lane i adds lane i ^ off, off = 1, 2, 4, ... below n),
// the same additions in the same order and so the same result bit for bit,
// with the exchanges in registers instead of LDS permutes.  Lanes ^1 and ^2
// come by quad permutes; ^4 and ^8 by mirroring within 8 and 16 lanes, which
// reaches a lane holding the same value once the smaller runs agree.  Then
// every row of 16 lanes holds one value r0..r3, so the ^16 step gives
// r0 + r1 in the lower half and r2 + r3 in the upper one (a lane's own row
// plus its partner's, in either order the same sum) and the ^32 step their
// sum.  n: a power of two <= 64, the same in every lane.
__device__ __forceinline__ float run_sum_dpp(float v, int n) {
  if (n > 1) v = dpp_xadd<0xb1>(v);    // quad_perm [1,0,3,2]
  if (n > 2) v = dpp_xadd<0x4e>(v);    // quad_perm [2,3,0,1]
  if (n > 4) v = dpp_xadd<0x141>(v);   // row_half_mirror
  if (n > 8) v = dpp_xadd<0x140>(v);   // row_mirror
  if (n > 16) {
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    const float lo = r0 + r1, hi = r2 + r3;
    v = n > 32 ? lo + hi : ((threadIdx.x & 32) ? hi : lo);
  }
  return v;
}

// Group sums of s[k] (this thread's vector t + TH k), in place.  `chunk`
// is LDS scratch of KT * TH / 64 floats, nchunks (<= KT * TH / 64) the row's
// 64-vector chunks; every thread of the workgroup must call it (it holds a
// barrier when groups span waves).  Callers alternate between two scratch
// buffers, so the barrier of the next call also frees this one.
template <int KT, int TH>
__device__ __forceinline__ void group_sums(float (&s)[KT], int NV, int nchunks, float* chunk) {
  constexpr int NW = TH / 64;
  if (NV <= 64) {
#pragma unroll
    for (int k = 0; k < KT; ++k) s[k] = run_sum_dpp(s[k], NV);
    return;
  }
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const float c = run_sum_dpp(s[k], 64);  // chunk q = NW k + w
    if (lane == 0) chunk[NW * k + w] = c;
  }
  __syncthreads();
  const int cpg = NV / 64;                  // chunks per group
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    // chunks past the row's last (idle threads) stay as they are: the
    // group would reach past the chunks written
    const int q0 = (NW * k + w) / cpg * cpg;
    if (q0 + cpg > nchunks) continue;
    float g = 0.f;
    for (int q = q0; q < q0 + cpg; ++q) g += chunk[q];
    s[k] = g;
  }
}

// The value through an empty asm statement: the compiler cannot reuse what
// it computed from it before.
__device__ __forceinline__ void launder(uint4& q) {
  asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
}

// Offset for a lane with nothing to load or store: past every resource's
// records, so the load reads zeros and the store is dropped.
constexpr uint32_t kNormPast = 0x80000000u;

// Byte offset of thread t's vector k in a row, or kNormPast past the row's last.
template <int TH>
__device__ __forceinline__ uint32_t vec_off(int t, int k, int nvec) {
  const int v = t + TH * k;
  return v < nvec ? (uint32_t)v * 16u : kNormPast;
}

// Row r's vectors of y, z (and dout, with D) owned by thread t, through
// resources over the row: a row past the end has no records and a vector past
// the row's last is aimed past them, so both read as zeros without a branch
// around the loads (a branch would make the first use of any load in flight,
// the next row's included, wait for all of them).
template <int KT, int TH, bool D, typename T>
__device__ __forceinline__ void load_row(const T* y, const T* z, const T* d, int64_t r,
                                         int64_t rows, int C, int nvec, int t, uint4 (&yv)[KT],
                                         uint4 (&zv)[KT], uint4 (&dv)[KT]) {
  const bool in = r < rows;
  const int64_t o = in ? r * C : 0;
  const uint32_t bytes = in ? (uint32_t)C * (uint32_t)sizeof(T) : 0u;
  const auto ry = buf_rsrc(y + o, bytes), rz = buf_rsrc(z + o, bytes);
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const uint32_t off = vec_off<TH>(t, k, nvec);
    yv[k] = buf_load16(ry, off);
    zv[k] = buf_load16(rz, off);
    if constexpr (D) dv[k] = buf_load16(buf_rsrc(d + o, bytes), off);
  }
}

// The weights of thread t's vectors (zeros past the row's last).
template <int KT, int TH, int V>
__device__ __forceinline__ void load_w(const float* w, int C, int nvec, int t,
                                       float (&wv)[KT][V]) {
  const auto rw = buf_rsrc(w, (uint32_t)C * 4u);
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const uint32_t off = vec_off<TH>(t, k, nvec);
    // V floats per vector: V / 4 loads of 16 bytes (a vector's channels lie at
    // V * sizeof(T) = 16 bytes of T, V * 4 bytes of w)
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const uint4 u = buf_load16(rw, off == kNormPast ? kNormPast : off * (V / 4) + 16u * q);
      wv[k][4 * q + 0] = __builtin_bit_cast(float, u.x);
      wv[k][4 * q + 1] = __builtin_bit_cast(float, u.y);
      wv[k][4 * q + 2] = __builtin_bit_cast(float, u.z);
      wv[k][4 * q + 3] = __builtin_bit_cast(float, u.w);
    }
  }
}

template <typename T, int KT, int TH>
__global__ __launch_bounds__(TH) void gated_norm_fwd_kernel(
    const T* __restrict__ y, const T* __restrict__ z, const float* __restrict__ w, int64_t rows,
    int C, int GS, float eps, T* __restrict__ out, float* __restrict__ rstd) {
  using NVc = NormVec<T>;
  constexpr int V = NVc::V, NCH = KT * TH / 64;
  __shared__ float chunk[2 * NCH];      // two buffers, used alternately
  const int t = threadIdx.x;
  const int nvec = C / V, NV = GS / V, ng = C / GS;
  const float inv_gs = 1.f / (float)GS;
  float wr[KT][V];                          // the weights of this thread's channels
  load_w<KT, TH, V>(w, C, nvec, t, wr);
  // r per group, stored by the group's first vector (no records without rstd)
  uint32_t roff[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int v = t + TH * k;
    roff[k] = (v < nvec && v % NV == 0) ? (uint32_t)(v / NV) * 4u : kNormPast;
  }
  int par = 0;                              // LDS buffer of this row's group sums
#pragma unroll 1
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x, par ^= 1) {
    uint4 yv[KT], zv[KT], unused[KT];
    load_row<KT, TH, false>(y, z, y, r, rows, C, nvec, t, yv, zv, unused);
    float g[KT][V], s[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      float yf[V], zf[V];
      NVc::unpack(yv[k], yf);
      NVc::unpack(zv[k], zf);
      s[k] = gate_values<V>(yf, zf, g[k]);
    }
    group_sums<KT, TH>(s, NV, (nvec + 63) / 64, chunk + par * NCH);
    const auto ro = buf_rsrc(out + r * C, (uint32_t)C * (uint32_t)sizeof(T));
    const auto rr = rstd ? buf_rsrc(rstd + r * ng, (uint32_t)ng * 4u) : buf_rsrc(out, 0u);
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const float rs = gate_rstd(s[k], inv_gs, eps);
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = (g[k][e] * rs) * wr[k][e];
      buf_store16(ro, vec_off<TH>(t, k, nvec), NVc::pack(o));
      buf_store4(rr, roff[k], rs);
    }
  }
}

template <typename T, int KT, int TH>
__global__ __launch_bounds__(TH) void gated_norm_bwd_kernel(
    const T* __restrict__ y, const T* __restrict__ z, const float* __restrict__ w,
    const T* __restrict__ dout, int64_t rows, int C, int GS, float eps, T* __restrict__ dy,
    T* __restrict__ dz, float* __restrict__ dw_part) {
  using NVc = NormVec<T>;
  constexpr int V = NVc::V, NCH = KT * TH / 64;
  // With up to two vectors per thread the sigmoids of the first pass stay in
  // registers for the second; with more, they are computed again there (the
  // same values either way).
  constexpr bool KEEP = KT <= 2;
  __shared__ float chunk[2 * NCH];      // two buffers, used alternately
  const int t = threadIdx.x;
  const int nvec = C / V, NV = GS / V;
  const float inv_gs = 1.f / (float)GS;
  const uint32_t row_bytes = (uint32_t)C * (uint32_t)sizeof(T);
  float dwa[KT][V], wr[KT][V];             // dw sums and the weights of this thread's channels
  load_w<KT, TH, V>(w, C, nvec, t, wr);
#pragma unroll
  for (int k = 0; k < KT; ++k)
#pragma unroll
    for (int e = 0; e < V; ++e) dwa[k][e] = 0.f;
  // the next row's inputs are loaded while this row is processed
  uint4 yv[KT], zv[KT], dv[KT];
  load_row<KT, TH, true>(y, z, dout, (int64_t)blockIdx.x, rows, C, nvec, t, yv, zv, dv);
#pragma unroll 1
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    uint4 ny[KT], nz[KT], nd[KT];
    load_row<KT, TH, true>(y, z, dout, r + gridDim.x, rows, C, nvec, t, ny, nz, nd);
    // g = y silu(z) and the group sums of g^2
    float u[KT][V], s[KT], sg[KEEP ? KT : 1][V];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      float yf[V], zf[V];
      NVc::unpack(yv[k], yf);
      NVc::unpack(zv[k], zf);
      if constexpr (KEEP) s[k] = gate_values_sig<V>(yf, zf, u[k], sg[k]);
      else s[k] = gate_values<V>(yf, zf, u[k]);
    }
    group_sums<KT, TH>(s, NV, (nvec + 63) / 64, chunk);
    // u = g r; dw += dout u; the group sums of du u with du = dout w
    float p[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      s[k] = gate_rstd(s[k], inv_gs, eps);  // s now holds r
      float df[V];
      NVc::unpack(dv[k], df);
      p[k] = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        u[k][e] = u[k][e] * s[k];
        dwa[k][e] += df[e] * u[k][e];
        p[k] += (df[e] * wr[k][e]) * u[k][e];
      }
    }
    group_sums<KT, TH>(p, NV, (nvec + 63) / 64, chunk + NCH);
    // with several vectors per thread, unpacking again from the packed
    // registers (the laundering keeps the compiler from holding the unpacked
    // values across the sums); with one, the unpacked values fit
    if constexpr (KT > 1) {
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        launder(yv[k]);
        launder(zv[k]);
        launder(dv[k]);
      }
    }
    const auto rdy = buf_rsrc(dy + r * C, row_bytes), rdz = buf_rsrc(dz + r * C, row_bytes);
    // vectors past the row's last hold zeros, compute finite values and
    // store past the records
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      float yf[V], zf[V], df[V];
      NVc::unpack(yv[k], yf);
      NVc::unpack(zv[k], zf);
      NVc::unpack(dv[k], df);
      const float mp = p[k] * inv_gs;
      float ody[V], odz[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float dg = s[k] * (df[e] * wr[k][e] - u[k][e] * mp);
        float sig;
        float gate;
        if constexpr (KEEP) {
          sig = sg[k][e];
          gate = zf[e] * sig;                // gate_silu's product, from the kept sigmoid
        } else {
          gate = gate_silu(zf[e], sig);
        }
        ody[e] = dg * gate;
        odz[e] = dg * yf[e] * sig * (1.f + zf[e] * (1.f - sig));
      }
      const uint32_t off = vec_off<TH>(t, k, nvec);
      buf_store16(rdy, off, NVc::pack(ody));
      buf_store16(rdz, off, NVc::pack(odz));
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      yv[k] = ny[k];
      zv[k] = nz[k];
      dv[k] = nd[k];
    }
  }
  // this workgroup's partial dw: each channel belongs to one thread
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int v = t + TH * k;
    if (v >= nvec) continue;
#pragma unroll
    for (int e = 0; e < V; ++e) dw_part[(int64_t)blockIdx.x * C + v * V + e] = dwa[k][e];
  }
}

// Column sums of the partial rows [y R, min((y + 1) R, nparts)) of `part`
// ([nparts][C]) into row y of `out`, for the 256 channels of column block x
// (four per lane).  Wave w sums rows [y R + w R / 4, y R + (w + 1) R / 4) in
// row order, kDwBatch loads in flight at a time, then the four wave sums are
// added in wave order.  R is a multiple of 4; rows and channels past the
// ends read as zeros through the resource and leave every sum as it is.
constexpr int kDwBatch = 8;
__global__ __launch_bounds__(kNormThreads) void gated_norm_dw_kernel(
    const float* __restrict__ part, int nparts, int R, int C, float* __restrict__ out) {
  __shared__ float4 wsum[3][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = (blockIdx.x * 64 + lane) * 4;
  const auto rp = buf_rsrc(part, (uint32_t)nparts * (uint32_t)C * 4u);
  const int rw = R / 4, a = blockIdx.y * R + w * rw;
  const int b = min(a + rw, nparts);
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int pb = a; pb < b; pb += kDwBatch) {
    uint4 v[kDwBatch];
#pragma unroll
    for (int i = 0; i < kDwBatch; ++i) {
      const int row = pb + i;
      v[i] = buf_load16(rp, (row < b && c < C) ? ((uint32_t)row * (uint32_t)C + c) * 4u
                                                : kNormPast);
    }
#pragma unroll
    for (int i = 0; i < kDwBatch; ++i) {
      t.x += __builtin_bit_cast(float, v[i].x);
      t.y += __builtin_bit_cast(float, v[i].y);
      t.z += __builtin_bit_cast(float, v[i].z);
      t.w += __builtin_bit_cast(float, v[i].w);
    }
  }
  if (w > 0) wsum[w - 1][lane] = t;
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const float4 u = wsum[q][lane];
    t.x += u.x;
    t.y += u.y;
    t.z += u.z;
    t.w += u.w;
  }
  const auto ro = buf_rsrc(out + (int64_t)blockIdx.y * C, (uint32_t)C * 4u);
  buf_store16(ro, c < C ? (uint32_t)c * 4u : kNormPast,
              make_uint4(__builtin_bit_cast(uint32_t, t.x), __builtin_bit_cast(uint32_t, t.y),
                         __builtin_bit_cast(uint32_t, t.z), __builtin_bit_cast(uint32_t, t.w)));
}

// Workgroups of the norm kernels: `per_cu` per CU (several rows of loads in
// flight on each), never more than the rows or kNormMaxParts (the backward's
// workspace holds that many partial rows of dw).
constexpr int kNormMaxParts = 2048;
constexpr int kNormDwRows = 32;            // partial rows summed per block in the first pass
int norm_grid(int64_t rows, int per_cu) {
  const int cus = device_cu_count();
  int64_t want = (int64_t)(cus > 0 ? cus : 256) * per_cu;
  if (want > kNormMaxParts) want = kNormMaxParts;
  return (int)(rows < want ? (rows > 0 ? rows : 1) : want);
}

// dw from the backward's nparts partial rows: sums of kNormDwRows rows at a
// time into the scratch after them, then the sum of those (both in a fixed
// order).
hipError_t norm_dw(const NormArgs& a, int nparts, hipStream_t s) {
  const int gx = (a.C + 255) / 256;
  const int n1 = (nparts + kNormDwRows - 1) / kNormDwRows;
  float* mid = a.dw_part + (int64_t)kNormMaxParts * a.C;
  if (n1 > 1) {
    hipLaunchKernelGGL(gated_norm_dw_kernel, dim3(gx, n1), dim3(kNormThreads), 0, s,
                       (const float*)a.dw_part, nparts, kNormDwRows, a.C, mid);
    hipLaunchKernelGGL(gated_norm_dw_kernel, dim3(gx, 1), dim3(kNormThreads), 0, s,
                       (const float*)mid, n1, (n1 + 3) / 4 * 4, a.C, a.dw);
  } else {
    hipLaunchKernelGGL(gated_norm_dw_kernel, dim3(gx, 1), dim3(kNormThreads), 0, s,
                       (const float*)a.dw_part, nparts, (nparts + 3) / 4 * 4, a.C, a.dw);
  }
  return hipGetLastError();
}

template <typename T, int KT, int TH>
hipError_t norm_fwd_kt(const NormArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gated_norm_fwd_kernel<T, KT, TH>), dim3(norm_grid(a.rows, 8)), dim3(TH),
                     0, s, (const T*)a.y, (const T*)a.z, a.w, a.rows, a.C, a.GS, a.eps,
                     (T*)a.out, a.rstd);
  return hipGetLastError();
}

template <typename T, int KT, int TH>
hipError_t norm_bwd_kt(const NormArgs& a, hipStream_t s) {
  const int grid = norm_grid(a.rows, 4);
  hipLaunchKernelGGL((gated_norm_bwd_kernel<T, KT, TH>), dim3(grid), dim3(TH), 0, s,
                     (const T*)a.y, (const T*)a.z, a.w, (const T*)a.dout, a.rows, a.C, a.GS,
                     a.eps, (T*)a.dy, (T*)a.dz, a.dw_part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return norm_dw(a, grid, s);
}

// Threads per workgroup: the row's vectors rounded up to a wave, at most
// kNormThreads (rows of up to 192 vectors leave no wave idle); then the
// vectors per thread.
template <typename T, bool BWD>
hipError_t norm_dispatch(const NormArgs& a, hipStream_t s) {
  constexpr int V = NormVec<T>::V;
  const int nvec = a.C / V;
  const int th = nvec >= kNormThreads ? kNormThreads : (nvec + 63) / 64 * 64;
  if (th < kNormThreads) {
    switch (th) {
#define SSD_TH(n) \
      case n: return BWD ? norm_bwd_kt<T, 1, n>(a, s) : norm_fwd_kt<T, 1, n>(a, s);
      SSD_TH(64) SSD_TH(128) SSD_TH(192)
#undef SSD_TH
    }
    return hipErrorInvalidValue;
  }
  const int kt = (nvec + kNormThreads - 1) / kNormThreads;
  switch (kt) {
#define SSD_KT(n) \
    case n: return BWD ? norm_bwd_kt<T, n, kNormThreads>(a, s) : norm_fwd_kt<T, n, kNormThreads>(a, s);
    SSD_KT(1) SSD_KT(2) SSD_KT(3) SSD_KT(4)
#undef SSD_KT
  }
  return hipErrorInvalidValue;
}

}  // namespace

int norm_max_channels(int32_t dtype) { return kNormMaxKT * kNormThreads * (dtype == 1 ? 8 : 4); }

int64_t norm_workspace_floats(int64_t C) {
  return (int64_t)(kNormMaxParts + (kNormMaxParts + kNormDwRows - 1) / kNormDwRows) * C;
}

hipError_t launch_norm_fwd(const NormArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  return a.bf16 ? norm_dispatch<bf16, false>(a, s) : norm_dispatch<float, false>(a, s);
}

hipError_t launch_norm_bwd(const NormArgs& a, hipStream_t s) {
  if (a.rows <= 0) return norm_dw(a, 0, s);
  return a.bf16 ? norm_dispatch<bf16, true>(a, s) : norm_dispatch<float, true>(a, s);
}

}  // namespace ssd
