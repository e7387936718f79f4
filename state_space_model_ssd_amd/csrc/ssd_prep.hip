// Stage 0 (plan: logical chunks of a packed batch) and stage 1
// (chunk_cumsum: the discretised step and its chunk-local running sum).
//
// chunk_cumsum is the first of the forward stages the pages name
// (aiproviderindex.com, "Mamba-2 offers a different scaling path": the
// cumulative parameters inside each chunk).  Per logical chunk j, head h and
// position l < len:
//   delta[j,h,l] = clamp(softplus(dt[t,h] + dt_bias[h]), dt_min, dt_max)
//   dAcs[j,h,l]  = sum_{k <= l} delta[j,h,k] * A[h]
// with delta = 0 for l >= len (the running sum stays flat there).
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kPlanThreads = 256;

// First index i in [0, n) with a[i] >= v for a non-decreasing a, else n.
// For a malformed (decreasing) array the result is still in [0, n].
__device__ int lower_bound_i32(const int32_t* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Token range [x, y) of sequence s, clamped into [0, total] and non-empty
// or empty but never reversed.
__device__ int2 seq_bounds(int s, const int32_t* cu, const int32_t* sidx, int total) {
  int st, en;
  if (cu) {
    st = min(max(cu[s], 0), total);
    en = min(max(cu[s + 1], st), total);
  } else {
    st = lower_bound_i32(sidx, total, s);
    en = max(st, lower_bound_i32(sidx, total, s + 1));
  }
  return make_int2(st, en);
}

// One workgroup: chunk counts per sequence and their exclusive prefix sum.
__global__ __launch_bounds__(kPlanThreads) void plan_seq_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ sidx, int nstates, int total,
    int L, int max_chunks, int* __restrict__ seq_chunks) {
  __shared__ int wave_tot[kPlanThreads / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  int carry = 0;
  for (int base = 0; base < nstates; base += kPlanThreads) {
    const int s = base + tid;
    int cnt = 0;
    if (s < nstates) {
      int2 b = seq_bounds(s, cu, sidx, total);
      cnt = (b.y - b.x + L - 1) / L;
    }
    int v = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      int t = __shfl_up(v, off);
      if (lane >= off) v += t;
    }
    if (lane == kWave - 1) wave_tot[wv] = v;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / kWave; ++w) {
      before += (w < wv) ? wave_tot[w] : 0;
      all += wave_tot[w];
    }
    if (s < nstates) seq_chunks[s] = min(carry + before + v - cnt, max_chunks);
    carry += all;
    __syncthreads();
  }
  if (tid == 0) seq_chunks[nstates] = min(carry, max_chunks);
}

// One thread per table slot: which sequence owns slot j, and where it starts.
__global__ __launch_bounds__(kPlanThreads) void plan_chunk_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ sidx, int nstates, int total,
    int L, int max_chunks, const int* __restrict__ seq_chunks, int4* __restrict__ table) {
  const int j = blockIdx.x * kPlanThreads + threadIdx.x;
  if (j >= max_chunks) return;
  const int used = seq_chunks[nstates];
  if (j >= used || nstates <= 0) {
    table[j] = make_int4(0, 0, 0, 0);
    return;
  }
  int lo = 0, hi = nstates - 1;  // largest s with seq_chunks[s] <= j
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seq_chunks[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int k = j - seq_chunks[lo];
  const int2 b = seq_bounds(lo, cu, sidx, total);
  const int st = b.x + k * L;
  const int len = max(0, min(L, b.y - st));
  table[j] = make_int4(len > 0 ? st : 0, len, lo, k);
}

template <int L>
__global__ __launch_bounds__(L) void chunk_cumsum_kernel(
    ChunkMap cm, const float* __restrict__ dt, const float* __restrict__ dt_bias,
    const float* __restrict__ A, int H, float dt_min, float dt_max,
    float* __restrict__ delta, float* __restrict__ dAcs) {
  __shared__ float wave_tot[L / kWave];
  const int j = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const ChunkDesc d = cm.desc(j);
  if (d.len <= 0) return;  // unused slot: uniform over the workgroup
  float step, cum;
  chunk_cumsum_block<L>(d, l, dt, dt_bias, A, H, h, dt_min, dt_max, wave_tot, step, cum);
  const int64_t o = ((int64_t)j * H + h) * L + l;
  delta[o] = step;
  dAcs[o] = cum;
}

}  // namespace

hipError_t launch_plan(const FwdArgs& a, hipStream_t s) {
  if (!a.packed) return hipSuccess;
  const int total = a.batch * a.seqlen;
  hipLaunchKernelGGL(plan_seq_kernel, dim3(1), dim3(kPlanThreads), 0, s, a.cu_seqlens,
                     a.seq_idx, a.nstates, total, a.L, a.max_chunks, a.seq_chunks);
  if (a.max_chunks > 0) {
    hipLaunchKernelGGL(plan_chunk_kernel, dim3((a.max_chunks + kPlanThreads - 1) / kPlanThreads),
                       dim3(kPlanThreads), 0, s, a.cu_seqlens, a.seq_idx, a.nstates, total, a.L,
                       a.max_chunks, (const int*)a.seq_chunks, a.table);
  }
  return hipGetLastError();
}

hipError_t launch_chunk_cumsum(const FwdArgs& a, hipStream_t s) {
  if (a.max_chunks <= 0) return hipSuccess;
  dim3 grid(a.max_chunks, a.H);
  switch (a.L) {
    case 64:
      hipLaunchKernelGGL(chunk_cumsum_kernel<64>, grid, dim3(64), 0, s, a.cmap(), a.dt,
                         a.dt_bias, a.A, a.H, a.dt_min, a.dt_max, a.delta, a.dAcs);
      break;
    case 128:
      hipLaunchKernelGGL(chunk_cumsum_kernel<128>, grid, dim3(128), 0, s, a.cmap(), a.dt,
                         a.dt_bias, a.A, a.H, a.dt_min, a.dt_max, a.delta, a.dAcs);
      break;
    case 256:
      hipLaunchKernelGGL(chunk_cumsum_kernel<256>, grid, dim3(256), 0, s, a.cmap(), a.dt,
                         a.dt_bias, a.A, a.H, a.dt_min, a.dt_max, a.delta, a.dAcs);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ssd
