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
// on the chain, so a ring of them stays in flight ahead of the dependent
// FMAs; more bytes in flight per CU is what keeps the 8 TB/s HBM busy (the
// same lesson as the clova.ai section "How we fixed it").
#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kSpThreads = 256;
constexpr int kSpDepth = 16;   // chunk loads in flight per thread
constexpr int kSpBatch = 1024;  // chunk decays staged in LDS at a time

// VEC consecutive fp32 state values per thread.
template <int VEC> struct VecF;
template <> struct VecF<1> { using type = float; };
template <> struct VecF<2> { using type = float2; };
template <> struct VecF<4> { using type = float4; };

template <int VEC>
__device__ __forceinline__ void fma_state(typename VecF<VEC>::type& st, float a,
                                          const typename VecF<VEC>::type& s) {
  if constexpr (VEC == 1) {
    st = a * st + s;
  } else if constexpr (VEC == 2) {
    st.x = a * st.x + s.x;
    st.y = a * st.y + s.y;
  } else {
    st.x = a * st.x + s.x;
    st.y = a * st.y + s.y;
    st.z = a * st.z + s.z;
    st.w = a * st.w + s.w;
  }
}

template <int VEC> __device__ __forceinline__ void store_state(float* p, const typename VecF<VEC>::type& v) {
  *reinterpret_cast<typename VecF<VEC>::type*>(p) = v;
}
template <int VEC> __device__ __forceinline__ void store_state(bf16* p, const typename VecF<VEC>::type& v);
template <> __device__ __forceinline__ void store_state<1>(bf16* p, const float& v) { *p = static_cast<bf16>(v); }
template <> __device__ __forceinline__ void store_state<2>(bf16* p, const float2& v) {
  bf16x2 q;
  q[0] = static_cast<bf16>(v.x);
  q[1] = static_cast<bf16>(v.y);
  *reinterpret_cast<bf16x2*>(p) = q;
}
template <> __device__ __forceinline__ void store_state<4>(bf16* p, const float4& v) {
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

template <typename T, int VEC>
__global__ __launch_bounds__(kSpThreads) void state_passing_kernel(
    ChunkMap cm, const float* __restrict__ S, const float* __restrict__ dAcs,
    const float* __restrict__ init, int H, int PN, int L, T* __restrict__ states_in,
    float* __restrict__ final_states) {
  using V = typename VecF<VEC>::type;
  __shared__ float decs[kSpBatch];      // chunk decays of the current batch of chunks
  const int s = blockIdx.z, h = blockIdx.y;
  const int e = (blockIdx.x * kSpThreads + threadIdx.x) * VEC;
  const bool live = e < PN;             // dead lanes still join the barriers
  const int2 r = cm.seq_range(s);
  V st{};
  if (init && live) st = *reinterpret_cast<const V*>(init + ((int64_t)s * H + h) * PN + e);
  for (int b0 = r.x; b0 < r.y; b0 += kSpBatch) {
    const int nb = min(kSpBatch, r.y - b0);
    __syncthreads();                    // previous batch's decays consumed
    for (int i = threadIdx.x; i < nb; i += kSpThreads) decs[i] = chunk_decay(cm, dAcs, b0 + i, h, H, L);
    __syncthreads();
    if (!live) continue;
    // Rolling ring of kSpDepth chunk loads: after chunk j is consumed, the
    // load of chunk j + kSpDepth takes its slot, so the ring stays full.  The
    // main loop has no branches (refills past the batch end re-read its last
    // chunk), so the compiler waits for one load at a time, not for all.
    V buf[kSpDepth];
#pragma unroll
    for (int i = 0; i < kSpDepth; ++i)
      buf[i] = *reinterpret_cast<const V*>(S + ((int64_t)(b0 + min(i, nb - 1)) * H + h) * PN + e);
    int base = 0;
    for (; base + kSpDepth <= nb; base += kSpDepth) {
#pragma unroll
      for (int i = 0; i < kSpDepth; ++i) {
        const int jj = base + i;
        store_state<VEC>(states_in + ((int64_t)(b0 + jj) * H + h) * PN + e, st);
        fma_state<VEC>(st, decs[jj], buf[i]);
        buf[i] = *reinterpret_cast<const V*>(
            S + ((int64_t)(b0 + min(jj + kSpDepth, nb - 1)) * H + h) * PN + e);
      }
    }
#pragma unroll
    for (int i = 0; i < kSpDepth; ++i) {  // tail: fewer than kSpDepth chunks
      const int jj = base + i;
      if (jj < nb) {                      // uniform over the workgroup
        store_state<VEC>(states_in + ((int64_t)(b0 + jj) * H + h) * PN + e, st);
        fma_state<VEC>(st, decs[jj], buf[i]);
      }
    }
  }
  if (final_states && live) *reinterpret_cast<V*>(final_states + ((int64_t)s * H + h) * PN + e) = st;
}

}  // namespace

template <typename T>
hipError_t launch_state_passing(const FwdArgs& a, hipStream_t s) {
  const int PN = a.P * a.N;
  if (a.nstates <= 0) return hipSuccess;
  // Widest vector per thread that still gives every SIMD a wave (1024 waves
  // of 64 lanes); each wave keeps kSpDepth chunk loads in flight, so the bytes
  // in flight do not depend on the width, only the instruction count does.
  const int64_t lanes = (int64_t)a.nstates * a.H * PN;
  int vec = (lanes / 4 >= (int64_t)1024 * 64) ? 4 : (lanes / 2 >= (int64_t)1024 * 64) ? 2 : 1;
  if (a.sp_vec == 1 || a.sp_vec == 2 || a.sp_vec == 4) vec = a.sp_vec;   // pinned by the caller
  if (PN % vec != 0) return hipErrorInvalidValue;
  auto go = [&](auto kern, int v) {
    dim3 grid((PN / v + kSpThreads - 1) / kSpThreads, a.H, a.nstates);
    hipLaunchKernelGGL(kern, grid, dim3(kSpThreads), 0, s, a.cmap(), a.chunk_states, a.dAcs,
                       a.init, a.H, PN, a.L, (T*)a.states_in, a.final_states);
  };
  if (vec == 4) go(state_passing_kernel<T, 4>, 4);
  else if (vec == 2) go(state_passing_kernel<T, 2>, 2);
  else go(state_passing_kernel<T, 1>, 1);
  return hipGetLastError();
}

template hipError_t launch_state_passing<float>(const FwdArgs&, hipStream_t);
template hipError_t launch_state_passing<bf16>(const FwdArgs&, hipStream_t);

}  // namespace ssd
