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
    for (int k = 0; k < KT; ++k) s[k] = run_sum(s[k], NV);
    return;
  }
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const float c = run_sum(s[k], 64);      // chunk q = NW k + w
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

// Row r's vectors of y, z (and d, if given) owned by thread t; zeros for a
// row past the end or a vector past the row's last.
template <int KT, int TH, int V, typename T>
__device__ __forceinline__ void load_row(const T* y, const T* z, const T* d, int64_t r,
                                         int64_t rows, int C, int nvec, int t, uint4 (&yv)[KT],
                                         uint4 (&zv)[KT], uint4* dv) {
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int v = t + TH * k;
    const bool ok = r < rows && v < nvec;
    const int64_t o = r * C + (int64_t)v * V;
    yv[k] = ok ? *reinterpret_cast<const uint4*>(y + o) : make_uint4(0, 0, 0, 0);
    zv[k] = ok ? *reinterpret_cast<const uint4*>(z + o) : make_uint4(0, 0, 0, 0);
    if (d) dv[k] = ok ? *reinterpret_cast<const uint4*>(d + o) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void load_w(const float* w, int v, int nvec, float* wv, int V) {
  for (int e = 0; e < V; ++e) wv[e] = v < nvec ? w[v * V + e] : 0.f;
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
  int par = 0;                              // LDS buffer of this row's group sums
#pragma unroll 1
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x, par ^= 1) {
    uint4 yv[KT], zv[KT];
    load_row<KT, TH, V>(y, z, static_cast<const T*>(nullptr), r, rows, C, nvec, t, yv, zv, nullptr);
    float g[KT][V], s[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      float yf[V], zf[V];
      NVc::unpack(yv[k], yf);
      NVc::unpack(zv[k], zf);
      s[k] = gate_values<V>(yf, zf, g[k]);
    }
    group_sums<KT, TH>(s, NV, (nvec + 63) / 64, chunk + par * NCH);
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int v = t + TH * k;
      if (v >= nvec) continue;
      const float rs = gate_rstd(s[k], inv_gs, eps);
      float wv[V], o[V];
      load_w(w, v, nvec, wv, V);
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = (g[k][e] * rs) * wv[e];
      *reinterpret_cast<uint4*>(out + r * C + v * V) = NVc::pack(o);
      if (rstd && (v % NV) == 0) rstd[r * ng + v / NV] = rs;
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
  float dwa[KT][V], wr[KT][V];             // dw sums and the weights of this thread's channels
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    load_w(w, t + TH * k, nvec, wr[k], V);
#pragma unroll
    for (int e = 0; e < V; ++e) dwa[k][e] = 0.f;
  }
  // the next row's inputs are loaded while this row is processed
  uint4 yv[KT], zv[KT], dv[KT];
  load_row<KT, TH, V>(y, z, dout, (int64_t)blockIdx.x, rows, C, nvec, t, yv, zv, dv);
#pragma unroll 1
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    uint4 ny[KT], nz[KT], nd[KT];
    load_row<KT, TH, V>(y, z, dout, r + gridDim.x, rows, C, nvec, t, ny, nz, nd);
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
    // unpacking again from the packed registers (the laundering keeps the
    // compiler from holding the unpacked values across the sums)
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      launder(yv[k]);
      launder(zv[k]);
      launder(dv[k]);
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int v = t + TH * k;
      if (v >= nvec) continue;
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
      *reinterpret_cast<uint4*>(dy + r * C + v * V) = NVc::pack(ody);
      *reinterpret_cast<uint4*>(dz + r * C + v * V) = NVc::pack(odz);
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

// Sums of the partial rows [y R, min((y + 1) R, nparts)) of `part`
// ([nparts][C]), in row order, four channels per thread: row y of `out`.
__global__ __launch_bounds__(kNormThreads) void gated_norm_dw_kernel(
    const float* __restrict__ part, int nparts, int R, int C, float* __restrict__ out) {
  const int c = (blockIdx.x * kNormThreads + threadIdx.x) * 4;
  if (c >= C) return;
  const int p0 = blockIdx.y * R, p1 = min(p0 + R, nparts);
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int kB = 8;                     // rows loaded together, then added in order
  for (int pb = p0; pb < p1; pb += kB) {
    float4 v[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i)
      v[i] = pb + i < p1 ? *reinterpret_cast<const float4*>(part + (int64_t)(pb + i) * C + c)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      if (pb + i < p1) {
        t.x += v[i].x;
        t.y += v[i].y;
        t.z += v[i].z;
        t.w += v[i].w;
      }
    }
  }
  *reinterpret_cast<float4*>(out + (int64_t)blockIdx.y * C + c) = t;
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
// time into the scratch after them, then the sum of those (both in row order).
hipError_t norm_dw(const NormArgs& a, int nparts, hipStream_t s) {
  const int gx = (a.C / 4 + kNormThreads - 1) / kNormThreads;
  const int n1 = (nparts + kNormDwRows - 1) / kNormDwRows;
  float* mid = a.dw_part + (int64_t)kNormMaxParts * a.C;
  if (n1 > 1) {
    hipLaunchKernelGGL(gated_norm_dw_kernel, dim3(gx, n1), dim3(kNormThreads), 0, s,
                       (const float*)a.dw_part, nparts, kNormDwRows, a.C, mid);
    hipLaunchKernelGGL(gated_norm_dw_kernel, dim3(gx, 1), dim3(kNormThreads), 0, s,
                       (const float*)mid, n1, n1, a.C, a.dw);
  } else {
    hipLaunchKernelGGL(gated_norm_dw_kernel, dim3(gx, 1), dim3(kNormThreads), 0, s,
                       (const float*)a.dw_part, nparts, nparts, a.C, a.dw);
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
