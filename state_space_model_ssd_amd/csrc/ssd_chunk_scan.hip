// Stage 5, chunk_scan: the output construction (clova.ai, table "Share of
// compute time by kernel": _chunk_scan_fwd; aiproviderindex.com, "Mamba-2
// offers a different scaling path": output construction).  For token l of
// logical chunk j, head h, group g:
//   y[l,p] = sum_{s <= l} CB[l,s] * exp(dAcs[l] - dAcs[s]) * delta[s] * x[s,p]
//          + exp(dAcs[l]) * sum_n C[l,n] * states_in[j,h,p,n]
//          + D[h] * x[l,p]
// accumulated in fp32 and rounded once to the output type.
//
// bf16 kernel (the production path): one workgroup (4 waves) per (chunk,
// head), the whole chunk at once.
//  - x of the chunk is staged once in LDS in its natural token-major layout
//    (coalesced 16-byte loads and stores) and read as the MFMA B operand with
//    the gfx950 LDS transpose read.
//  - intra-chunk term: 16-row groups are dealt to the waves round-robin (the
//    causal work evens out).  Per 32-token k-step the lane builds its 8
//    A-operand values from the CB row.  Below the diagonal the decay splits
//    around the step's last token r:  exp(a_l - a_s) = exp(a_l - a_r) *
//    exp(a_r - a_s), both factors <= 1, the second (times delta_s) kept per
//    token in LDS, so a step costs one exp per lane instead of eight.  Steps
//    that touch the diagonal evaluate the masked exponential directly (mask
//    selected before the exp).
//  - inter-chunk term: the C row scaled by exp(a_l) is the A operand, the
//    entering state (n contiguous) the B operand, accumulated into the same
//    tile.
//  - epilogue: y = acc + D x is written over x in LDS by the lane that read
//    it, then the tile leaves in coalesced 16-byte rows.
//
// fp32 kernel (exactness path): one workgroup per (chunk, 64-row tile, head);
// each wave owns 16 output rows and all P columns (P/16 MFMA tiles).
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

// KPL consecutive values of a CB row as fp32.
__device__ __forceinline__ void load_cb1(const float* p, float* v) { v[0] = *p; }
__device__ __forceinline__ void load_cb8(const bf16* p, float* v) {
  const bf16x8 t = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(t[e]);
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
    ChunkMap cm, const T* __restrict__ x, const T* __restrict__ C, const T* __restrict__ cb,
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
  const int w = wave_id(), lane = tid & (kWave - 1);
  const int lr = lane & 15, kq = (lane >> 4) * KPL;
  const int row0 = rt * RT + w * 16;     // first output row of this wave
  const int my_row = row0 + lr;          // A-operand row of this lane
  const bool row_ok = my_row < d.len;
  const T* cbrow = cb + (((int64_t)j * G + g) * L + my_row) * L;

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
      if constexpr (KPL == 1) load_cb1(cbrow + sf, cbv); else load_cb8(cbrow + sf, cbv);
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


// ------------------------------------------------------------- bf16 kernel
// Waves per workgroup: two 16-row groups per wave for L >= 128 (8 waves for a
// 256-token chunk), one per wave for L = 64.
template <int L> constexpr int kScanWaves = (L / 16) / 2 < 4 ? 4 : (L / 16) / 2;

template <int P, int N, int L>
__global__ __launch_bounds__(64 * kScanWaves<L>) __attribute__((amdgpu_waves_per_eu(4))) void
chunk_scan_bf16_kernel(ChunkMap cm, int nslots, const bf16* __restrict__ x,
                       const bf16* __restrict__ C, const bf16* __restrict__ cb,
                       const float* __restrict__ delta, const float* __restrict__ dAcs,
                       const bf16* __restrict__ states_in, const float* __restrict__ D, int H,
                       int G, bf16* __restrict__ out) {
  static_assert(L % 64 == 0 && P % 16 == 0 && N % 32 == 0, "tile shape");
  constexpr int NW = kScanWaves<L>;
  constexpr int NT = 64 * NW;            // threads
  constexpr int XP = P + 8;              // x tile pitch (elements): conflict-free transpose reads
  constexpr int HP = N + 8;              // state tile pitch: conflict-free 16-byte row reads
  constexpr int RG = L / 16;             // 16-row groups of the chunk
  constexpr int RGW = RG / NW;           // row groups per wave: 1 or 2
  static_assert(RGW * NW == RG && (RGW == 1 || RGW == 2), "row-group split");
  constexpr int PT = P / 16;
  constexpr int NK = N / 32;             // k-steps of the inter-chunk term
  constexpr int NQ = L / 32;             // k-steps of the intra-chunk term
  constexpr int CPR = P / 8;             // 16-byte pieces per x row
  constexpr int XU = L * CPR / NT;       // x pieces per thread
  constexpr int HPR = N / 8;             // 16-byte pieces per state row
  constexpr int HU = (P * HPR + NT - 1) / NT;
  static_assert((L * CPR) % NT == 0 && L <= NT, "x staging");
  __shared__ __align__(16) bf16 xs[L * XP];
  __shared__ __align__(16) bf16 hsm[P * HP];
  __shared__ __align__(16) float dal2[L];   // running sum of delta*A, times log2(e)
  __shared__ __align__(16) float dls[L];    // delta
  __shared__ __align__(16) float cfs[L];    // delta_s * exp(a_r - a_s), r = last token of s's 32-block

  const int2 jh = xcd_chunk_head(blockIdx.x, H);
  const int j = jh.x, h = jh.y;
  if (j >= nslots) return;
  const ChunkDesc d = cm.desc(j);
  if (d.len <= 0) return;
  const int g = h / (H / G);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63;
  const int lr = lane & 15, kq = (lane >> 4) * 8;
  // Row groups of this wave; with two per wave they pair from both ends of
  // the chunk, so every wave carries the same causal work.
  int mg[RGW];
  mg[0] = w;
  if constexpr (RGW == 2) mg[1] = RG - 1 - w;
  int lrow[RGW], nq[RGW];
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    lrow[i] = 16 * mg[i] + lr;
    nq[i] = (16 * mg[i] + 15) / 32 + 1;    // k-steps that reach this row group
  }
  const int last = d.len - 1;

  // ---- global loads issued together.  Addresses are clamped into the chunk
  // and out-of-chunk values replaced after arrival, so nothing branches.
  uint4 xv[XU];
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tid + NT * u, r = i / CPR, c = i - (i / CPR) * CPR;
    xv[u] = *reinterpret_cast<const uint4*>(x + ((int64_t)(d.start + min(r, last)) * H + h) * P + c * 8);
  }
  const bf16* hs = states_in + ((int64_t)j * H + h) * P * N;
  uint4 hv[HU];
#pragma unroll
  for (int u = 0; u < HU; ++u) {
    const int i = min(tid + NT * u, P * HPR - 1);
    hv[u] = *reinterpret_cast<const uint4*>(hs + i * 8);
  }
  const int tl = tid < L ? tid : L - 1;
  const float dA_t = dAcs[((int64_t)j * H + h) * L + tl];
  const float dl_t = delta[((int64_t)j * H + h) * L + tl];
  bf16x8 fc[RGW][NK];                      // C rows of this lane, all n-steps
  const bf16* cbrow[RGW];
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    const bf16* crow = C + ((int64_t)(d.start + min(lrow[i], last)) * G + g) * N + kq;
#pragma unroll
    for (int k = 0; k < NK; ++k) fc[i][k] = *reinterpret_cast<const bf16x8*>(crow + 32 * k);
    cbrow[i] = cb + (((int64_t)j * G + g) * L + lrow[i]) * L + kq;
  }
  bf16x8 cur[RGW];                         // CB rows of the current k-step
#pragma unroll
  for (int i = 0; i < RGW; ++i) cur[i] = *reinterpret_cast<const bf16x8*>(cbrow[i]);

  // ---- stage x, the state, the running sums and the per-token factors
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tid + NT * u, r = i / CPR, c = i - (i / CPR) * CPR;
    *reinterpret_cast<uint4*>(&xs[r * XP + c * 8]) = r < d.len ? xv[u] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < HU; ++u) {
    const int i = tid + NT * u, r = i / HPR, c = i - (i / HPR) * HPR;
    if (i < P * HPR) *reinterpret_cast<uint4*>(&hsm[r * HP + c * 8]) = hv[u];
  }
  if (tid < L) {
    dal2[tid] = dA_t * kLog2e;
    dls[tid] = dl_t;
  }
  __syncthreads();
  if (tid < L) cfs[tid] = dls[tid] * exp2_fast(dal2[tid | 31] - dal2[tid]);

  // The MFMAs compute the transposed tile y^T[p][l]: A = x^T or the state
  // (rows p), B = the decay-masked CB row or the C row (columns l).  A lane
  // then holds four consecutive p of one token.
  f32x4 acc[RGW][PT];
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int a = 0; a < PT; ++a) acc[i][a] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- inter-chunk term: y^T[p][l] = exp(a_l) * sum_n state[p][n] C[l][n].
  // C enters the MFMA as loaded; exp(a_l) scales the accumulator afterwards
  // (a lane's column is one token).  Columns of tokens past the chunk end
  // hold junk that no store reads: an output column depends on its own
  // B-operand column only.
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    bf16x8 fh[PT];
#pragma unroll
    for (int a = 0; a < PT; ++a)
      fh[a] = *reinterpret_cast<const bf16x8*>(&hsm[(16 * a + lr) * HP + 32 * k + kq]);
#pragma unroll
    for (int i = 0; i < RGW; ++i)
#pragma unroll
      for (int a = 0; a < PT; ++a) acc[i][a] = Mfma<bf16>::mma(fh[a], fc[i][k], acc[i][a]);
  }
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    const float rsc = exp2_fast(dal2[lrow[i]]);
#pragma unroll
    for (int a = 0; a < PT; ++a) acc[i][a] *= rsc;
  }
  __syncthreads();                         // cfs ready

  // ---- intra-chunk term, k-steps outer: the x^T operands of a step serve
  // both row groups of the wave; the next step's CB rows are in flight.
  const int nq_wave = nq[RGW - 1];
  for (int q = 0; q < nq_wave; ++q) {
    const int s0 = 32 * q;
    const int sn = min(s0 + 32, L - 32);   // next step (clamped: always in the row)
    bf16x8 nxt[RGW];
#pragma unroll
    for (int i = 0; i < RGW; ++i) nxt[i] = *reinterpret_cast<const bf16x8*>(cbrow[i] + sn);
    bf16x8 fx[PT];
#pragma unroll
    for (int a = 0; a < PT; ++a) fx[a] = lds_operand_kmajor(xs, XP, s0, 16 * a, lane);
    const float dal_r = dal2[s0 + 31];
    const float4 f0 = *reinterpret_cast<const float4*>(&cfs[s0 + kq]);
    const float4 f1 = *reinterpret_cast<const float4*>(&cfs[s0 + kq + 4]);
    const float cf[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      const int m = mg[i];
      if (q >= nq[i]) continue;            // wave-uniform: above this row group
      float cbv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cbv[e] = static_cast<float>(cur[i][e]);
      const float dal = dal2[lrow[i]];
      float mv[8];
      if (s0 + 32 <= 16 * m) {             // below the diagonal: factored decay
        const float rf = exp2_fast(dal - dal_r);
#pragma unroll
        for (int e = 0; e < 8; ++e) mv[e] = cbv[e] * (rf * cf[e]);
      } else {                             // on the diagonal: masked exponential
        const float4 a0 = *reinterpret_cast<const float4*>(&dal2[s0 + kq]);
        const float4 a1 = *reinterpret_cast<const float4*>(&dal2[s0 + kq + 4]);
        const float4 d0 = *reinterpret_cast<const float4*>(&dls[s0 + kq]);
        const float4 d1 = *reinterpret_cast<const float4*>(&dls[s0 + kq + 4]);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = s0 + kq + e <= lrow[i];
          const float arg = ok ? dal - av[e] : 0.f;
          mv[e] = ok ? cbv[e] * exp2_fast(arg) * dv[e] : 0.f;
        }
      }
      const bf16x8 fm = Mfma<bf16>::pack(mv);
#pragma unroll
      for (int a = 0; a < PT; ++a) acc[i][a] = Mfma<bf16>::mma(fx[a], fm, acc[i][a]);
    }
#pragma unroll
    for (int i = 0; i < RGW; ++i) cur[i] = nxt[i];
  }

  // ---- epilogue: y = acc + D x, written over x in LDS (each element read
  // and written by one lane), then the rows leave coalesced
  __syncthreads();
  const float Dh = D ? D[h] : 0.f;
  const int p4 = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int a = 0; a < PT; ++a) {
      bf16x4* e = reinterpret_cast<bf16x4*>(&xs[lrow[i] * XP + 16 * a + p4]);
      const bf16x4 xo = *e;
      bf16x4 yo;
#pragma unroll
      for (int r = 0; r < 4; ++r) yo[r] = static_cast<bf16>(acc[i][a][r] + Dh * static_cast<float>(xo[r]));
      *e = yo;
    }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tid + NT * u, r = i / CPR, c = i - (i / CPR) * CPR;
    if (r < d.len)
      *reinterpret_cast<uint4*>(out + ((int64_t)(d.start + r) * H + h) * P + c * 8) =
          *reinterpret_cast<const uint4*>(&xs[r * XP + c * 8]);
  }
}

}  // namespace

template <typename T, int P, int N, int L>
hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t s) {
  static_assert(L % 64 == 0, "chunk size must be a multiple of 64");
  if (a.max_chunks <= 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((chunk_scan_bf16_kernel<P, N, L>), dim3(xcd_grid(a.max_chunks, a.H)),
                       dim3(64 * kScanWaves<L>), 0, s, a.cmap(), a.max_chunks, (const bf16*)a.x,
                       (const bf16*)a.C, (const bf16*)a.cb, a.delta, a.dAcs,
                       (const bf16*)a.states_in, a.D,
                       a.H, a.G, (bf16*)a.out);
  } else {
    dim3 grid(a.max_chunks * (L / 64), a.H);
    hipLaunchKernelGGL((chunk_scan_kernel<T, P, N, L>), grid, dim3(256), 0, s, a.cmap(),
                       (const T*)a.x, (const T*)a.C, (const T*)a.cb, a.delta, a.dAcs,
                       (const T*)a.states_in, a.D, a.H, a.G, (T*)a.out);
  }
  return hipGetLastError();
}

#define SSD_INST(T, P, N, L) template hipError_t launch_chunk_scan<T, P, N, L>(const FwdArgs&, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_INST)
#undef SSD_INST

}  // namespace ssd
