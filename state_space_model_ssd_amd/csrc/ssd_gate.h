// The arithmetic of the gated RMS norm (internal), shared by the standalone
// norm kernels and the chunk_scan epilogue that fuses the norm, so both round
// exactly alike:
//   g = y silu(z), silu(z) = z sigma(z);  r = 1 / sqrt(sum(g^2) / group + eps)
#pragma once

#include "ssd_common.h"

// Multiply-adds are fused only inside one expression, the same in every
// kernel that includes this header.
#pragma clang fp contract(on)

namespace ssd {

// silu(z) = z sigma(z), with sigma through the hardware reciprocal (about one
// unit in the last place of fp32): sigma -> 0 for z -> -inf (exp overflows to
// inf, whose reciprocal is 0) and -> 1 for z -> +inf.
__device__ __forceinline__ float gate_silu(float z, float& sig) {
  sig = __builtin_amdgcn_rcpf(1.f + __expf(-z));
  return z * sig;
}

// g[e] = y[e] silu(z[e]) for V values; returns sum of g[e]^2 in order of e.
template <int V>
__device__ __forceinline__ float gate_values(const float* yf, const float* zf, float* g) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < V; ++e) {
    float sig;
    g[e] = yf[e] * gate_silu(zf[e], sig);
    s += g[e] * g[e];
  }
  return s;
}

// gate_values that also hands out each sigmoid (the same arithmetic).
template <int V>
__device__ __forceinline__ float gate_values_sig(const float* yf, const float* zf, float* g,
                                                 float* sg) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < V; ++e) {
    g[e] = yf[e] * gate_silu(zf[e], sg[e]);
    s += g[e] * g[e];
  }
  return s;
}

// 1 / sqrt(mean + eps) from a group's sum of squares.
__device__ __forceinline__ float gate_rstd(float sum, float inv_gs, float eps) {
  return rsqrtf(sum * inv_gs + eps);
}

// Sum of v over the lanes of an aligned run of n lanes (n a power of two
// <= 64), offsets from 1 up.
__device__ __forceinline__ float run_sum(float v, int n) {
  for (int off = 1; off < n; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

}  // namespace ssd

#pragma clang fp contract(fast)
