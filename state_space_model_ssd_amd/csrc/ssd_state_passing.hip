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
//
// Chunk-parallel form (clova.ai, "Stage 3. Logic and heuristic refinement":
// the state-passing loop rebuilt on an associative scan; Figure 3 contrasts
// the two).  A chunk acts on the state as the affine map h -> d h + S, and
// maps compose associatively: (d1, S1) then (d2, S2) = (d1 d2, d2 S1 + S2).
// When a problem has too few state elements to keep the HBM busy with one
// chain per element, each sequence's chunks are cut into KB consecutive
// blocks and scanned in two launches:
//   reduce: block b's composed map from a zero state: E_b (its end state)
//           and log d_b = sum of its chunks' dAcs at their last token;
//   scan:   block b's entering state is init composed with the maps of
//           blocks 0..b-1 (read back from the reduce), then the block walks
//           its chunks writing states_in; the last block writes the final
//           state.
// That reads the chunk states twice instead of once, for KB times the
// parallelism.
#include <type_traits>

#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kSpThreads = 256;
constexpr int kSpDepth = 16;   // chunk loads in flight per thread
constexpr int kSpBatch = 1024;  // chunk decays staged in LDS at a time
constexpr int kSpCarryGroup = 8;  // block end states in flight when composing a carry

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

// What a walk over a range of chunks does with the states it passes.
enum SpMode {
  kSpChain = 0,    // whole sequence: states_in written, end state -> final
  kSpReduce = 1,   // one block from a zero state: end state -> block_states
  kSpScan = 2,     // one block from its entering state: states_in written,
                   // the last block's end state -> final
};

// Chunk range [x, y) of block b of KB equal blocks of sequence s.
__device__ __forceinline__ int2 sp_block_range(const ChunkMap& cm, int s, int b, int KB) {
  const int2 r = cm.seq_range(s);
  const int n = r.y - r.x;
  return make_int2(r.x + (int)((int64_t)n * b / KB), r.x + (int)((int64_t)n * (b + 1) / KB));
}

// grid: (element vectors, H, nstates * KB); workgroup (., h, s * KB + b).
template <typename T, int VEC, int MODE>
__global__ __launch_bounds__(kSpThreads) void state_passing_kernel(
    ChunkMap cm, const float* __restrict__ S, const float* __restrict__ dAcs,
    const float* __restrict__ init, int H, int PN, int L, int KB, T* __restrict__ states_in,
    float* __restrict__ final_states, float* __restrict__ block_states,
    float* __restrict__ block_logdecay) {
  using V = typename VecF<VEC>::type;
  __shared__ float decs[kSpBatch];      // chunk decays of the current batch of chunks
  __shared__ float wsum[kSpThreads / kWave];
  const int s = blockIdx.z / KB, b = blockIdx.z - (blockIdx.z / KB) * KB, h = blockIdx.y;
  if (MODE == kSpReduce && b == KB - 1) return;   // the last block's map is never composed
  const int e = (blockIdx.x * kSpThreads + threadIdx.x) * VEC;
  const bool live = e < PN;             // dead lanes still join the barriers
  const int2 r = MODE == kSpChain ? cm.seq_range(s) : sp_block_range(cm, s, b, KB);
  const size_t bsh = (size_t)H * PN;    // one block's states, all heads
  V st{};
  if (MODE != kSpReduce && init && live) st = *reinterpret_cast<const V*>(init + ((int64_t)s * H + h) * PN + e);
  if (MODE == kSpScan && live) {
    // entering state of block b: the maps of blocks 0..b-1 applied in order,
    // their end states loaded kSpCarryGroup at a time (clamped to block b-1,
    // so every load is in bounds) ahead of the dependent FMAs
    for (int c0 = 0; c0 < b; c0 += kSpCarryGroup) {
      V eb[kSpCarryGroup];
      float ld[kSpCarryGroup];
#pragma unroll
      for (int u = 0; u < kSpCarryGroup; ++u) {
        const int c = min(c0 + u, b - 1);
        ld[u] = block_logdecay[((size_t)s * KB + c) * H + h];
        eb[u] = *reinterpret_cast<const V*>(block_states + ((size_t)s * KB + c) * bsh + (size_t)h * PN + e);
      }
#pragma unroll
      for (int u = 0; u < kSpCarryGroup; ++u)
        if (c0 + u < b) fma_state<VEC>(st, expf(ld[u]), eb[u]);   // uniform over the workgroup
    }
  }
  float logsum = 0.f;                   // kSpReduce: this thread's share of log d_b
  for (int b0 = r.x; b0 < r.y; b0 += kSpBatch) {
    const int nb = min(kSpBatch, r.y - b0);
    __syncthreads();                    // previous batch's decays consumed
    for (int i = threadIdx.x; i < nb; i += kSpThreads) {
      const int len = cm.desc(b0 + i).len;
      const float la = len > 0 ? dAcs[((int64_t)(b0 + i) * H + h) * L + len - 1] : 0.f;
      decs[i] = expf(la);
      logsum += la;
    }
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
        if constexpr (MODE != kSpReduce)
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
        if constexpr (MODE != kSpReduce)
          store_state<VEC>(states_in + ((int64_t)(b0 + jj) * H + h) * PN + e, st);
        fma_state<VEC>(st, decs[jj], buf[i]);
      }
    }
  }
  if constexpr (MODE == kSpReduce) {
    if (live) *reinterpret_cast<V*>(block_states + ((size_t)s * KB + b) * bsh + (size_t)h * PN + e) = st;
    if (blockIdx.x == 0) {                // one workgroup per (block, head) sums log d_b
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) logsum += __shfl_xor(logsum, off);
      if ((threadIdx.x & (kWave - 1)) == 0) wsum[threadIdx.x / kWave] = logsum;
      __syncthreads();
      if (threadIdx.x == 0) {
        float t = 0.f;
        for (int w = 0; w < kSpThreads / kWave; ++w) t += wsum[w];
        block_logdecay[((size_t)s * KB + b) * H + h] = t;
      }
    }
  } else {
    const bool last = MODE == kSpChain || b == KB - 1;
    if (last && final_states && live) *reinterpret_cast<V*>(final_states + ((int64_t)s * H + h) * PN + e) = st;
  }
}

}  // namespace

// Widest vector per thread that still gives every SIMD of the device a wave
// of 64 lanes (4 SIMDs per CU); each wave keeps kSpDepth chunk loads in
// flight, so the bytes in flight do not depend on the width, only the
// instruction count does.
int state_passing_vec(const FwdArgs& a) {
  const int KB = a.sp_blocks > 1 ? a.sp_blocks : 1;
  const int64_t lanes = (int64_t)a.nstates * KB * a.H * a.P * a.N;
  const int cus = device_cu_count();
  const int64_t wave_lanes = (int64_t)(cus > 0 ? cus : 256) * 4 * 64;
  return (lanes / 4 >= wave_lanes) ? 4 : (lanes / 2 >= wave_lanes) ? 2 : 1;
}

template <typename T>
hipError_t launch_state_passing(const FwdArgs& a, hipStream_t s) {
  const int PN = a.P * a.N;
  if (a.nstates <= 0) return hipSuccess;
  const int KB = a.sp_blocks > 1 ? a.sp_blocks : 1;
  if (KB > 1 && (!a.block_states || !a.block_logdecay)) return hipErrorInvalidValue;
  int vec = state_passing_vec(a);
  if (a.sp_vec == 1 || a.sp_vec == 2 || a.sp_vec == 4) vec = a.sp_vec;   // pinned by the caller
  if (PN % vec != 0) return hipErrorInvalidValue;
  auto go = [&](auto kern, int v) {
    dim3 grid((PN / v + kSpThreads - 1) / kSpThreads, a.H, a.nstates * KB);
    hipLaunchKernelGGL(kern, grid, dim3(kSpThreads), 0, s, a.cmap(), a.chunk_states, a.dAcs,
                       a.init, a.H, PN, a.L, KB, (T*)a.states_in, a.final_states, a.block_states,
                       a.block_logdecay);
  };
  auto mode = [&](auto m) {
    constexpr int M = decltype(m)::value;
    if (vec == 4) go(state_passing_kernel<T, 4, M>, 4);
    else if (vec == 2) go(state_passing_kernel<T, 2, M>, 2);
    else go(state_passing_kernel<T, 1, M>, 1);
  };
  if (KB == 1) {
    mode(std::integral_constant<int, kSpChain>{});
  } else {
    mode(std::integral_constant<int, kSpReduce>{});
    mode(std::integral_constant<int, kSpScan>{});
  }
  return hipGetLastError();
}

template hipError_t launch_state_passing<float>(const FwdArgs&, hipStream_t);
template hipError_t launch_state_passing<bf16>(const FwdArgs&, hipStream_t);

}  // namespace ssd
