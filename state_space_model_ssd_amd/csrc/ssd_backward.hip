// The SSD backward: gradients of loss = sum(y * dy) + sum(final * dfinal)
// with respect to x, dt, dt_bias, A, B, C, D and the initial states (the
// layer's backward kernels listed next to the forward ones: clova.ai, table
// "Share of compute time by kernel": _chunk_scan_bwd_dx, _chunk_state_bwd_db,
// _state_passing_bwd, _chunk_scan_bwd_dstates, ...).
//
// The forward's stages 0-4 run first (delta, the running sums a, CB and the
// states entering each chunk, H).  Then, per chunk j, head h (tokens l, s of
// the chunk, a_last the running sum at its last token, E[l,s] = exp(a_l -
// a_s) for s <= l):
//   1. Q_j[p,n]  = sum_l exp(a_l) dy[l,p] C[l,n]          (dloss/dH via y)
//   2. reverse chain per sequence: G = dfinal; for j from the last chunk
//      down: dS_j = G; G = exp(a_last_j) G + Q_j; then dinit = G.  dS_j is
//      the gradient of the state leaving chunk j.
//   3. per token, with U[l,s] = dy_l . x_s and dCB[l,s] = E[l,s] delta_s U[l,s]:
//      dx_s     = delta_s sum_{l>=s} CB[l,s] E[l,s] dy_l
//                 + delta_s exp(a_last - a_s) dS_j B_s + D dy_s
//      ddelta_s = sum_{l>=s} CB[l,s] E[l,s] U[l,s] + exp(a_last - a_s) B_s.(x_s dS_j)
//      da_l     = sum_{s<=l} CB dCB[l,.] - sum_{l'>=l} CB dCB[.,l]   (intra)
//                 + exp(a_l) C_l . (dy_l H)                            (inter)
//                 - delta_l exp(a_last - a_l) B_l.(x_l dS_j)           (state)
//      plus, at the last token, sum_s delta_s exp(a_last - a_s) B_s.(x_s dS_j)
//      + exp(a_last) <dS_j, H>; then a = cumsum(delta A) gives
//      ddelta_k += A sum_{l>=k} da_l and dA += sum_k delta_k sum_{l>=k} da_l,
//      and ddt = ddelta softplus'(dt + dt_bias) where the clamp passes it.
//   4. per head: dC_h[l] = sum_{s<=l} dCB[l,s] B_s + exp(a_l) dy_l H,
//      dB_h[s] = sum_{l>=s} dCB[l,s] C_l + delta_s exp(a_last - a_s) x_s dS_j;
//   5. dB, dC: sums of dB_h, dC_h over the heads of each group; dA, dD and
//      dt_bias: sums over chunks.
// Everything accumulates in fp32; dx, dB and dC are rounded once to x's
// dtype.  Deterministic: fixed loop orders, no atomics.
//
// This first version is direct loops over global memory (the operands stay
// in L2) with the states in LDS: correctness first, MFMA tiling later.
#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kBwdThreads = 256;

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return to_f32(*p); }

// A 64 x 64 fp32 output tile of sum_k A(m, k) B(k, n) for k in [k0, k1),
// accumulated into acc (4 x 4 per thread of 256).  Operand tiles of 32
// k-values pass through LDS: As[k][m] and Bs[k][n] (row pitch 68 floats).
// A_KFAST: A(m, k) is contiguous in k (else in m); B(k, n) is read with n
// fastest.  The loaders return 0 outside the operands.
constexpr int kGemmPitch = 68;

template <bool A_KFAST, typename LA, typename LB>
__device__ __forceinline__ void gemm_tile(int k0, int k1, LA loadA, LB loadB, float (&acc)[4][4],
                                          float* As, float* Bs) {
  const int tid = threadIdx.x;
  const int tm = (tid >> 4) * 4, tn = (tid & 15) * 4;
  for (int kb = k0; kb < k1; kb += 32) {
    __syncthreads();                       // previous tile consumed
    for (int i = tid; i < 64 * 32; i += kBwdThreads) {
      int m, k;
      if constexpr (A_KFAST) { m = i >> 5; k = i & 31; } else { k = i >> 6; m = i & 63; }
      As[k * kGemmPitch + m] = kb + k < k1 ? loadA(m, kb + k) : 0.f;
      const int kk = i >> 6, n = i & 63;
      Bs[kk * kGemmPitch + n] = kb + kk < k1 ? loadB(kb + kk, n) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&As[k * kGemmPitch + tm]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[k * kGemmPitch + tn]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[i][jn] += av[i] * bv[jn];
    }
  }
}

// 1. Q_j[p,n] = sum_l exp(a_l) dy[l,p] C[l,n] as 64 x 64 tiles;
// grid (ceil(P/64) * ceil(N/64), H, chunk slots).
template <typename T, int P, int N, int L>
__global__ __launch_bounds__(kBwdThreads) void bwd_q_tiled_kernel(
    ChunkMap cm, const T* __restrict__ dy, const T* __restrict__ C,
    const float* __restrict__ dAcs, int H, int G, float* __restrict__ Q) {
  __shared__ __align__(16) float As[32 * kGemmPitch], Bs[32 * kGemmPitch];
  __shared__ float sc[L];
  constexpr int NT = (N + 63) / 64;
  const int m0 = (blockIdx.x / NT) * 64, n0 = (blockIdx.x % NT) * 64;
  const int h = blockIdx.y, j = blockIdx.z, g = h / (H / G);
  const ChunkDesc cd = cm.desc(j);
  const int64_t jh = (int64_t)j * H + h;
  for (int l = threadIdx.x; l < L; l += kBwdThreads) sc[l] = expf(dAcs[jh * L + l]);
  __syncthreads();
  float acc[4][4] = {};
  gemm_tile<false>(0, max(cd.len, 0),
      [&](int m, int l) { const int p = m0 + m;
        return p < P ? sc[l] * ld(dy + ((int64_t)(cd.start + l) * H + h) * P + p) : 0.f; },
      [&](int l, int n) { const int nn = n0 + n;
        return nn < N ? ld(C + ((int64_t)(cd.start + l) * G + g) * N + nn) : 0.f; },
      acc, As, Bs);
  const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int p = m0 + tm + i, n = n0 + tn + jn;
      if (p < P && n < N) Q[(jh * P + p) * N + n] = acc[i][jn];
    }
}

// 2. Reverse chain; grid (ceil(P*N / 256), H, nstates).
__global__ __launch_bounds__(kBwdThreads) void bwd_chain_kernel(
    ChunkMap cm, const float* __restrict__ Q, const float* __restrict__ dAcs,
    const float* __restrict__ dfinal, int H, int PN, int L, float* __restrict__ dS,
    float* __restrict__ dinit) {
  const int e = blockIdx.x * kBwdThreads + threadIdx.x;
  if (e >= PN) return;
  const int h = blockIdx.y, s = blockIdx.z;
  const int2 r = cm.seq_range(s);
  float g = dfinal ? dfinal[((int64_t)s * H + h) * PN + e] : 0.f;
  for (int j = r.y - 1; j >= r.x; --j) {
    const int64_t jh = (int64_t)j * H + h;
    dS[jh * PN + e] = g;
    const int len = cm.desc(j).len;
    const float dec = len > 0 ? expf(dAcs[jh * L + len - 1]) : 1.f;
    g = dec * g + Q[jh * PN + e];
  }
  if (dinit) dinit[((int64_t)s * H + h) * PN + e] = g;
}

// dinit = dfinal (or 0) when there are no chunks.
__global__ __launch_bounds__(kBwdThreads) void bwd_pass_final_kernel(const float* __restrict__ dfinal,
                                                                     int64_t n, float* __restrict__ dinit) {
  const int64_t i = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  if (i < n) dinit[i] = dfinal ? dfinal[i] : 0.f;
}

// Sum over the workgroup (L threads, L a multiple of 64); every thread gets it.
template <int L>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < L / kWave; ++w) t += red[w];
  return t;
}

// 3. Per (chunk, head), one thread per token: dx, ddt, the dCB rows, and the
// chunk's parts of dA, dD and dt_bias.  grid (H, chunk slots), L threads.
template <typename T, int P, int N, int L>
__global__ __launch_bounds__(L) void bwd_chunk_kernel(
    ChunkMap cm, const T* __restrict__ x, const float* __restrict__ dt,
    const float* __restrict__ dt_bias, const float* __restrict__ A, const T* __restrict__ B,
    const T* __restrict__ C, const float* __restrict__ D, const T* __restrict__ dy,
    const float* __restrict__ delta, const float* __restrict__ dAcs, const T* __restrict__ cb,
    const T* __restrict__ states_in, const float* __restrict__ dS, int H, int G, float dt_min,
    float dt_max, T* __restrict__ dx, float* __restrict__ ddt, float* __restrict__ dcb,
    float* __restrict__ dA_part, float* __restrict__ dD_part, float* __restrict__ dbias_part) {
  __shared__ float Gs[P * N];     // dS_j
  __shared__ float Hs[P * N];     // H entering chunk j
  __shared__ float as[L], ds[L], das[L];
  __shared__ float red[L / kWave];
  const int h = blockIdx.x, j = blockIdx.y, g = h / (H / G), k = threadIdx.x;
  const ChunkDesc cd = cm.desc(j);
  const int64_t jh = (int64_t)j * H + h;
  if (cd.len <= 0) {                       // uniform over the workgroup
    if (k == 0) {
      dA_part[jh] = 0.f;
      dD_part[jh] = 0.f;
      dbias_part[jh] = 0.f;
    }
    return;
  }
  const int len = cd.len;
  for (int i = k; i < P * N; i += L) {
    Gs[i] = dS[jh * P * N + i];
    Hs[i] = ld(states_in + jh * P * N + i);
  }
  as[k] = dAcs[jh * L + k];
  ds[k] = delta[jh * L + k];
  __syncthreads();
  const bool valid = k < len;
  const float ak = as[k], dk = ds[k], alast = as[len - 1];
  const T* cbj = cb + ((int64_t)j * G + g) * L * L;
  const int64_t tk = cd.start + k;
  const float Dh = D ? D[h] : 0.f;

  float ddir = 0.f, colsum = 0.f, vs = 0.f, dd = 0.f, rowsum = 0.f, inter = 0.f;
  if (valid) {
    // ---- with x_k held: dx_k, the column sums, the state term
    float xk[P], acc[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      xk[p] = ld(x + (tk * H + h) * P + p);
      acc[p] = 0.f;
    }
    float sdir = 0.f;
    for (int l = k; l < len; ++l) {
      const float c = ld(cbj + (int64_t)l * L + k) * expf(as[l] - ak);
      const T* dyl = dy + ((cd.start + l) * H + h) * P;
      float u = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const float v = ld(dyl + p);
        u += v * xk[p];
        acc[p] += c * v;
      }
      sdir += c * u;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) acc[p] *= dk;
    const float fs = dk * expf(alast - ak);
    float vx = 0.f;
    for (int n = 0; n < N; ++n) {
      const float b = ld(B + (tk * G + g) * N + n);
      const float fb = fs * b;
      float xg = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const float gv = Gs[p * N + n];
        xg += xk[p] * gv;
        acc[p] += fb * gv;
      }
      vx += b * xg;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float dyk = ld(dy + (tk * H + h) * P + p);
      dd += dyk * xk[p];
      dx[(tk * H + h) * P + p] = from_f32<T>(acc[p] + Dh * dyk);
    }
    ddir = sdir + expf(alast - ak) * vx;
    colsum = dk * sdir;
    vs = fs * vx;

    // ---- with dy_k held: the row sums (and the dCB row), the inter term
    float yk[P];
#pragma unroll
    for (int p = 0; p < P; ++p) yk[p] = ld(dy + (tk * H + h) * P + p);
    float* dcbk = dcb + (jh * L + k) * L;
    for (int s = 0; s <= k; ++s) {
      const T* xs = x + ((cd.start + s) * H + h) * P;
      float u = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) u += yk[p] * ld(xs + p);
      const float w = expf(ak - as[s]) * ds[s] * u;
      dcbk[s] = w;
      rowsum += ld(cbj + (int64_t)k * L + s) * w;
    }
    float it = 0.f;
    for (int n = 0; n < N; ++n) {
      float yh = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) yh += yk[p] * Hs[p * N + n];
      it += ld(C + (tk * G + g) * N + n) * yh;
    }
    inter = expf(ak) * it;
  }

  // ---- da, its suffix sums, and the parts reduced over the chunk
  float gh = 0.f;
  for (int i = k; i < P * N; i += L) gh += Gs[i] * Hs[i];
  gh = block_sum<L>(gh, red);
  const float t1 = block_sum<L>(valid ? vs : 0.f, red);
  float da = valid ? rowsum - colsum + inter - vs : 0.f;
  if (k == len - 1) da += t1 + expf(alast) * gh;
  das[k] = da;
  __syncthreads();
  float rc = 0.f;
  for (int l = L - 1; l >= k; --l) rc += das[l];
  const float ddelta = ddir + A[h] * rc;
  float dbias = 0.f;
  if (valid) {
    const float u = dt[tk * H + h] + (dt_bias ? dt_bias[h] : 0.f);
    const float sp = fmaxf(u, 0.f) + log1pf(expf(-fabsf(u)));
    const float pass = (sp >= dt_min && sp <= dt_max) ? 1.f : 0.f;
    const float sig = 1.f / (1.f + expf(-u));
    dbias = ddelta * sig * pass;
    ddt[tk * H + h] = dbias;
  }
  const float da_sum = block_sum<L>(valid ? dk * rc : 0.f, red);
  const float dd_sum = block_sum<L>(dd, red);
  const float db_sum = block_sum<L>(dbias, red);
  if (k == 0) {
    dA_part[jh] = da_sum;
    dD_part[jh] = dd_sum;
    dbias_part[jh] = db_sum;
  }
}

// 4. Per-head dC and dB rows as 64 x 64 tiles:
//   dC_h = dCB B (s <= l) + diag(exp(a)) dy H,
//   dB_h = dCB^T C (l >= s) + diag(delta exp(a_last - a)) x dS_j;
// grid (L/64 * ceil(N/64), H, chunk slots), blockIdx.x even: dC, odd: dB
// (the x index counts (row tile, column tile, which)).
template <typename T, int P, int N, int L>
__global__ __launch_bounds__(kBwdThreads) void bwd_bc_tiled_kernel(
    ChunkMap cm, const T* __restrict__ x, const T* __restrict__ B, const T* __restrict__ C,
    const T* __restrict__ dy, const float* __restrict__ delta, const float* __restrict__ dAcs,
    const T* __restrict__ states_in, const float* __restrict__ dS, const float* __restrict__ dcb,
    int H, int G, float* __restrict__ dBh, float* __restrict__ dCh) {
  __shared__ __align__(16) float As[32 * kGemmPitch], Bs[32 * kGemmPitch];
  __shared__ float sc[L];
  constexpr int NT = (N + 63) / 64;
  const int which = blockIdx.x & 1, t = blockIdx.x >> 1;
  const int m0 = (t / NT) * 64, n0 = (t % NT) * 64;
  const int h = blockIdx.y, j = blockIdx.z, g = h / (H / G);
  const ChunkDesc cd = cm.desc(j);
  const int len = max(cd.len, 0);
  if (m0 >= len) return;                   // uniform: rows past the chunk
  const int64_t jh = (int64_t)j * H + h;
  const float* a = dAcs + jh * L;
  const float alast = a[len - 1];
  for (int l = threadIdx.x; l < L; l += kBwdThreads)
    sc[l] = which == 0 ? expf(a[l]) : delta[jh * L + l] * expf(alast - a[l]);
  const float* dcbj = dcb + jh * L * L;
  const int64_t t0 = cd.start;
  float acc[4][4] = {};
  auto ldB = [&](int s, int n) { const int nn = n0 + n;
    return nn < N ? ld(B + ((t0 + s) * G + g) * N + nn) : 0.f; };
  auto ldC = [&](int l, int n) { const int nn = n0 + n;
    return nn < N ? ld(C + ((t0 + l) * G + g) * N + nn) : 0.f; };
  if (which == 0) {
    // dC rows m0..m0+63: s runs to the tile's last row
    gemm_tile<true>(0, min(len, m0 + 64),
        [&](int m, int s) { const int l = m0 + m;
          return (l < len && s <= l) ? dcbj[(int64_t)l * L + s] : 0.f; },
        ldB, acc, As, Bs);
    gemm_tile<true>(0, P,
        [&](int m, int p) { const int l = m0 + m;
          return l < len ? sc[l] * ld(dy + ((t0 + l) * H + h) * P + p) : 0.f; },
        [&](int p, int n) { const int nn = n0 + n;
          return nn < N ? ld(states_in + (jh * P + p) * N + nn) : 0.f; },
        acc, As, Bs);
  } else {
    // dB rows m0..m0+63: l runs from the tile's first row
    gemm_tile<false>(m0, len,
        [&](int m, int l) { const int s = m0 + m;
          return (s < len && l >= s) ? dcbj[(int64_t)l * L + s] : 0.f; },
        ldC, acc, As, Bs);
    gemm_tile<true>(0, P,
        [&](int m, int p) { const int s = m0 + m;
          return s < len ? sc[s] * ld(x + ((t0 + s) * H + h) * P + p) : 0.f; },
        [&](int p, int n) { const int nn = n0 + n;
          return nn < N ? dS[(jh * P + p) * N + nn] : 0.f; },
        acc, As, Bs);
  }
  float* out = which == 0 ? dCh : dBh;
  const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int r = m0 + tm + i, n = n0 + tn + jn;
      if (r < len && n < N) out[(jh * L + r) * N + n] = acc[i][jn];
    }
}

// 5a. dB, dC: sums over the heads of a group; grid (ceil(L*N / 256), G, chunk slots).
template <typename T, int N, int L>
__global__ __launch_bounds__(kBwdThreads) void bwd_bc_reduce_kernel(
    ChunkMap cm, const float* __restrict__ dBh, const float* __restrict__ dCh, int H, int G,
    T* __restrict__ dB, T* __restrict__ dC) {
  const int o = blockIdx.x * kBwdThreads + threadIdx.x;
  if (o >= L * N) return;
  const int g = blockIdx.y, j = blockIdx.z;
  const int k = o / N, n = o - (o / N) * N;
  const ChunkDesc cd = cm.desc(j);
  if (k >= cd.len) return;
  const int hpg = H / G;
  float sb = 0.f, sc = 0.f;
  for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
    const int64_t i = (((int64_t)j * H + h) * L + k) * N + n;
    sb += dBh[i];
    sc += dCh[i];
  }
  const int64_t t = cd.start + k;
  dB[(t * G + g) * N + n] = from_f32<T>(sb);
  dC[(t * G + g) * N + n] = from_f32<T>(sc);
}

// 5b. dA, dD, dt_bias: sums over the chunk slots; one thread per head.
__global__ __launch_bounds__(kBwdThreads) void bwd_head_reduce_kernel(
    const float* __restrict__ dA_part, const float* __restrict__ dD_part,
    const float* __restrict__ dbias_part, int H, int nslots, float* __restrict__ dA,
    float* __restrict__ dD, float* __restrict__ dbias) {
  const int h = blockIdx.x * kBwdThreads + threadIdx.x;
  if (h >= H) return;
  float sa = 0.f, sd = 0.f, sb = 0.f;
  for (int j = 0; j < nslots; ++j) {
    sa += dA_part[(int64_t)j * H + h];
    sd += dD_part[(int64_t)j * H + h];
    sb += dbias_part[(int64_t)j * H + h];
  }
  dA[h] = sa;
  if (dD) dD[h] = sd;
  if (dbias) dbias[h] = sb;
}

}  // namespace

template <typename T, int P, int N, int L>
hipError_t launch_backward(const FwdArgs& a, const BwdArgs& b, hipStream_t s) {
  const int mc = a.max_chunks, H = a.H, G = a.G, PN = P * N;
  const ChunkMap cm = a.cmap();
  if (mc <= 0) {                           // no tokens: dinit = dfinal, zero parameter gradients
    const int64_t ne = (int64_t)a.nstates * H * PN;
    if (b.dinit && ne > 0)
      hipLaunchKernelGGL(bwd_pass_final_kernel, dim3((unsigned)((ne + kBwdThreads - 1) / kBwdThreads)),
                         dim3(kBwdThreads), 0, s, b.dfinal, ne, b.dinit);
    hipLaunchKernelGGL(bwd_head_reduce_kernel, dim3((H + kBwdThreads - 1) / kBwdThreads),
                       dim3(kBwdThreads), 0, s, b.dA_part, b.dD_part, b.dbias_part, H, 0, b.dA,
                       b.dD, b.ddt_bias);
    return hipGetLastError();
  }
  const T* x = (const T*)a.x;
  const T* B = (const T*)a.B;
  const T* C = (const T*)a.C;
  const T* dy = (const T*)b.dy;
  const T* cb = (const T*)a.cb;
  const T* hin = (const T*)a.states_in;
  constexpr int NT = (N + 63) / 64;
  hipLaunchKernelGGL((bwd_q_tiled_kernel<T, P, N, L>), dim3(((P + 63) / 64) * NT, H, mc),
                     dim3(kBwdThreads), 0, s, cm, dy, C, a.dAcs, H, G, b.Q);
  hipLaunchKernelGGL(bwd_chain_kernel, dim3((PN + kBwdThreads - 1) / kBwdThreads, H, a.nstates),
                     dim3(kBwdThreads), 0, s, cm, b.Q, a.dAcs, b.dfinal, H, PN, L, b.dS, b.dinit);
  hipLaunchKernelGGL((bwd_chunk_kernel<T, P, N, L>), dim3(H, mc), dim3(L), 0, s, cm, x, a.dt,
                     a.dt_bias, a.A, B, C, a.D, dy, a.delta, a.dAcs, cb, hin, b.dS, H, G, a.dt_min,
                     a.dt_max, (T*)b.dx, b.ddt, b.dcb, b.dA_part, b.dD_part, b.dbias_part);
  hipLaunchKernelGGL((bwd_bc_tiled_kernel<T, P, N, L>), dim3((L / 64) * NT * 2, H, mc),
                     dim3(kBwdThreads), 0, s, cm, x, B, C, dy, a.delta, a.dAcs, hin, b.dS, b.dcb, H,
                     G, b.dBh, b.dCh);
  hipLaunchKernelGGL((bwd_bc_reduce_kernel<T, N, L>), dim3((L * N + kBwdThreads - 1) / kBwdThreads, G, mc),
                     dim3(kBwdThreads), 0, s, cm, b.dBh, b.dCh, H, G, (T*)b.dB, (T*)b.dC);
  hipLaunchKernelGGL(bwd_head_reduce_kernel, dim3((H + kBwdThreads - 1) / kBwdThreads), dim3(kBwdThreads),
                     0, s, b.dA_part, b.dD_part, b.dbias_part, H, mc, b.dA, b.dD, b.ddt_bias);
  return hipGetLastError();
}

#define SSD_BWD_INST(T, P, N, L) \
  template hipError_t launch_backward<T, P, N, L>(const FwdArgs&, const BwdArgs&, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_BWD_INST)
#undef SSD_BWD_INST

}  // namespace ssd
