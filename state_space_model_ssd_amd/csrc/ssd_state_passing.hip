// Stage 4, state_passing: the sequential inter-chunk chain (clova.ai, table
// "Share of compute time by kernel": _state_passing_fwd; aiproviderindex.com,
// "Mamba-2 offers a different scaling path": state propagation).  For each
// sequence s and head h, over the sequence's chunks j in order:
//   states_in[j] = state                       (state entering chunk j)
//   state        = exp(dAcs[j, len_j - 1]) * state + S[j]
// starting from initial_states[s,h] (or 0); final_states[s,h] = state.
//
// Pure HBM streaming: each thread owns 4 consecutive state elements of one
// (sequence, head) and walks the chain.  The chunk-state loads do not depend
// on the chain, so a group of them is issued before the dependent FMAs
// consume it; more bytes in flight per CU is what keeps the 8 TB/s HBM busy
// (the same lesson as the clova.ai section "How we fixed it").
#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kSpThreads = 256;
constexpr int kSpDepth = 8;   // chunk loads in flight per thread

__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, float4 v) {
  bf16x4 q;
  q[0] = static_cast<bf16>(v.x);
  q[1] = static_cast<bf16>(v.y);
  q[2] = static_cast<bf16>(v.z);
  q[3] = static_cast<bf16>(v.w);
  *reinterpret_cast<bf16x4*>(p) = q;
}

__device__ __forceinline__ float chunk_decay(const ChunkMap& cm, const float* dAcs, int j, int h,
                                             int H, int L) {
  const int len = cm.desc(j).len;
  return len > 0 ? expf(dAcs[((int64_t)j * H + h) * L + len - 1]) : 1.f;
}

template <typename T>
__global__ __launch_bounds__(kSpThreads) void state_passing_kernel(
    ChunkMap cm, const float* __restrict__ S, const float* __restrict__ dAcs,
    const float* __restrict__ init, int H, int PN, int L, T* __restrict__ states_in,
    float* __restrict__ final_states) {
  const int s = blockIdx.z, h = blockIdx.y;
  const int e = (blockIdx.x * kSpThreads + threadIdx.x) * 4;
  if (e >= PN) return;
  const int2 r = cm.seq_range(s);
  float4 st = init ? *reinterpret_cast<const float4*>(init + ((int64_t)s * H + h) * PN + e)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  int j = r.x;
  for (; j + kSpDepth <= r.y; j += kSpDepth) {
    float4 sv[kSpDepth];
    float a[kSpDepth];
#pragma unroll
    for (int i = 0; i < kSpDepth; ++i) {
      sv[i] = *reinterpret_cast<const float4*>(S + ((int64_t)(j + i) * H + h) * PN + e);
      a[i] = chunk_decay(cm, dAcs, j + i, h, H, L);
    }
#pragma unroll
    for (int i = 0; i < kSpDepth; ++i) {
      store4(states_in + ((int64_t)(j + i) * H + h) * PN + e, st);
      st.x = a[i] * st.x + sv[i].x;
      st.y = a[i] * st.y + sv[i].y;
      st.z = a[i] * st.z + sv[i].z;
      st.w = a[i] * st.w + sv[i].w;
    }
  }
  for (; j < r.y; ++j) {
    const float4 sv = *reinterpret_cast<const float4*>(S + ((int64_t)j * H + h) * PN + e);
    const float a = chunk_decay(cm, dAcs, j, h, H, L);
    store4(states_in + ((int64_t)j * H + h) * PN + e, st);
    st.x = a * st.x + sv.x;
    st.y = a * st.y + sv.y;
    st.z = a * st.z + sv.z;
    st.w = a * st.w + sv.w;
  }
  if (final_states) store4(final_states + ((int64_t)s * H + h) * PN + e, st);
}

}  // namespace

template <typename T>
hipError_t launch_state_passing(const FwdArgs& a, hipStream_t s) {
  const int PN = a.P * a.N;
  if (a.nstates <= 0) return hipSuccess;
  dim3 grid((PN / 4 + kSpThreads - 1) / kSpThreads, a.H, a.nstates);
  hipLaunchKernelGGL(state_passing_kernel<T>, grid, dim3(kSpThreads), 0, s, a.cmap(),
                     a.chunk_states, a.dAcs, a.init, a.H, PN, a.L, (T*)a.states_in,
                     a.final_states);
  return hipGetLastError();
}

template hipError_t launch_state_passing<float>(const FwdArgs&, hipStream_t);
template hipError_t launch_state_passing<bf16>(const FwdArgs&, hipStream_t);

}  // namespace ssd
