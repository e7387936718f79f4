// Stage 5, chunk_scan: the output construction (clova.ai, table "Share of
// compute time by kernel": _chunk_scan_fwd; aiproviderindex.com, "Mamba-2
// offers a different scaling path": output construction).  For token l of
// logical chunk j, head h, group g:
//   y[l,p] = sum_{s <= l} CB[l,s] * exp(dAcs[l] - dAcs[s]) * delta[s] * x[s,p]
//          + exp(dAcs[l]) * sum_n C[l,n] * states_in[j,h,p,n]
//          + D[h] * x[l,p]
// accumulated in fp32 and rounded once to the output type.
//
// bf16 kernels (the production path).  Common to both:
//  - the MFMAs compute the transposed tile y^T[p][l] (A = x^T by the gfx950
//    LDS transpose read from a token-major, XOR-swizzled x tile, or the
//    entering state; B = a CB row or a C row), so a lane holds four
//    consecutive p of one token;
//  - the masked intra-chunk term builds each lane's 8 B-operand values from
//    the CB row.  Below the diagonal the decay splits around the k-step's
//    last token r: exp(a_l - a_s) = exp(a_l - a_r) * exp(a_r - a_s), both
//    factors <= 1, the second (times delta_s) kept per token in LDS, so a
//    step costs one exp per lane instead of eight.  Diagonal steps use the
//    same factors while the block's own decay is within 2^64, else the
//    masked exponential (exp2(-inf) = 0 above the diagonal);
//  - the inter-chunk term is the entering state times the C rows on MFMA,
//    scaled by exp(a_l) per token;
//  - all global traffic goes through buffer resources bounded by the tile.
// Two kernels, the first in two sizes (a caller may pin any of them):
//  - one workgroup per (chunk, head) tile, of 8 waves (two 16-row groups per
//    wave; 4 waves for chunks of 128 tokens or fewer) or of 4 waves (four
//    row groups per wave, three workgroups per CU).  Each tile takes the
//    rescaled path when its whole decay is within 2^64 (x staged as
//    x delta 2^(-a), CB rows used as loaded, one row factor 2^(a_l) at the
//    end), else the masked path; the two are compiled as separate bodies;
//  - a persistent workgroup of 4 L threads per resident slot, walking the
//    tiles with the next tile's inputs in flight (masked path).
// The library runs the 8-wave tile for 256-token chunks, and for shorter
// chunks the one-tile-per-workgroup kernel on small grids and the persistent
// walk on large ones (chunk_scan_choice).
// The y = acc + D x epilogue stages y in LDS and stores coalesced rows.
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
#include <atomic>

#include "ssd_kernels.h"
#include "ssd_scan_tile.h"

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
template <int P, int N, int L>
struct ScanShape {
  static constexpr int RG = L / 16;        // 16-row groups of a chunk
  static constexpr int NPAIR = RG / 2;     // mirror pairs (16m.., 16(RG-1-m)..)
  static constexpr int NW = 2 * NPAIR;     // two waves per pair
  static constexpr int NT = 64 * NW;       // threads (= 4 L)
  static constexpr int PT = P / 16;        // 16-column MFMA tiles over p
  static constexpr int NK = N / 32;        // n-steps of the inter-chunk term
  static constexpr int CPR = P / 8;        // 16-byte pieces per x row
  static constexpr int XU = L * CPR / NT;  // x pieces per thread
  static constexpr int HPR = N / 8;        // 16-byte pieces per state row
  static constexpr int HN = P * HPR;
  static constexpr int HU = (HN + NT - 1) / NT;
  static constexpr int HP = N + 8;         // state LDS pitch: conflict-free row reads
  // The two row groups of a pair need RG/2 + 1 intra-chunk k-steps in all;
  // the first wave of the pair takes NS0 of them, the second NS1.
  static constexpr int NS0 = RG / 4 + 1;
  static constexpr int NS1 = RG / 2 + 1 - NS0;
  static_assert(L % 64 == 0 && P % 32 == 0 && N % 32 == 0, "tile shape");
  static_assert((L * CPR) % NT == 0 && XU >= 1, "x staging");
};


__device__ __forceinline__ ScanTile scan_tile(const ChunkMap& cm, int nslots, int ntiles, int t,
                                              int H) {
  ScanTile T{0, 0, 0, 0};
  if (t >= ntiles) return T;
  const int2 jh = xcd_chunk_head(t, H);
  T.j = jh.x;
  T.h = jh.y;
  if (T.j < nslots) {
    if (cm.table) {
      // read through the constant address space: scalar loads
      typedef const __attribute__((address_space(4))) int cint;
      const cint* e = (const cint*)cm.table + 4 * T.j;
      T.start = e[0];
      T.len = max(e[1], 0);
    } else {
      const ChunkDesc d = cm.desc(T.j);
      T.start = d.start;
      T.len = max(d.len, 0);
    }
  }
  return T;
}

// Registers that carry one tile's staged inputs from its prefetch to its
// staging in LDS.
template <int P, int N, int L>
struct ScanStage {
  uint4 xv[ScanShape<P, N, L>::XU];
  uint4 hv[ScanShape<P, N, L>::HU];
  float dA, dl;
};


// Issue the loads of a tile's x rows, entering state, running sums and steps.
template <int P, int N, int L>
__device__ __forceinline__ void scan_prefetch(const ScanTile& T, int tid, ScanStage<P, N, L>& st,
                                              const bf16* x, const bf16* states_in,
                                              const float* dAcs, const float* delta, int H,
                                              uint32_t HPx) {
  using S = ScanShape<P, N, L>;
  const auto rx = rows_rsrc(x, T, H, P, HPx);
#pragma unroll
  for (int u = 0; u < S::XU; ++u) {
    const int i = tid + S::NT * u, r = i / S::CPR, c = i % S::CPR;
    st.xv[u] = buf_load16(rx, ((uint32_t)r * HPx + c * 8) * 2u);
  }
  const int64_t jh = (int64_t)T.j * H + T.h;
  const auto rh = buf_rsrc(states_in + jh * P * N, T.len > 0 ? P * N * 2 : 0);
#pragma unroll
  for (int u = 0; u < S::HU; ++u) st.hv[u] = buf_load16(rh, (uint32_t)(tid + S::NT * u) * 16);
  const uint32_t lb = T.len > 0 ? L * 4 : 0;
  st.dA = buf_load4(buf_rsrc(dAcs + jh * L, lb), tid * 4);
  st.dl = buf_load4(buf_rsrc(delta + jh * L, lb), tid * 4);
}

// A wave's share of one mirror pair (all wave-uniform).
struct ScanSplit {
  int mg0, mg1;   // row groups of the pair
  int nq0;        // 32-token k-steps reaching mg0
  int xs1;        // k-steps of mg1 taken by the first wave
  int kap;        // 0: first wave (owns mg0), 1: second wave (owns mg1)
  int mown;       // row group this wave finishes
  int nslot;      // k-steps this wave takes
  // slots of the first wave: mg1's k-steps 0..xs1-1, then mg0's 0..nq0-1;
  // slots of the second wave: mg1's k-steps xs1..
  __device__ __forceinline__ int rg(int s) const { return kap ? 1 : (s < xs1 ? 1 : 0); }
  __device__ __forceinline__ int q(int s) const { return kap ? xs1 + s : (s < xs1 ? s : s - xs1); }
};

// Issue the loads of the own row group's C rows (all n-steps).
template <int N>
__device__ __forceinline__ void scan_load_c(const ScanTile& T, int lane, const ScanSplit& sp,
                                            bf16x8 (&fc)[N / 32], const bf16* C, int H, int G,
                                            uint32_t GN) {
  const int g = T.h / (H / G);
  const int lr = lane & 15, kq = (lane >> 4) * 8;
  const uint32_t cbytes = T.len > 0 ? ((uint32_t)(T.len - 1) * GN + N) * 2u : 0u;
  const auto rc = buf_rsrc(C + ((int64_t)T.start * G + g) * N, cbytes);
  const uint32_t co = ((uint32_t)(16 * sp.mown + lr) * GN + kq) * 2u;
#pragma unroll
  for (int k = 0; k < N / 32; ++k) fc[k] = __builtin_bit_cast(bf16x8, buf_load16(rc, co + 64 * k));
}

// Issue the loads of the CB rows of every k-step this wave takes.
template <int P, int N, int L>
__device__ __forceinline__ void scan_load_cb(const ScanTile& T, int lane, const ScanSplit& sp,
                                             bf16x8 (&cbs)[ScanShape<P, N, L>::NS0],
                                             const bf16* cb, int H, int G) {
  using S = ScanShape<P, N, L>;
  const int g = T.h / (H / G);
  const int lr = lane & 15, kq = (lane >> 4) * 8;
  const auto rcb = buf_rsrc(cb + ((int64_t)T.j * G + g) * L * L, T.len > 0 ? L * L * 2 : 0);
#pragma unroll
  for (int sl = 0; sl < S::NS0; ++sl) {
    if (sl < sp.nslot) {                   // wave-uniform
      const int m = sp.rg(sl) ? sp.mg1 : sp.mg0;
      const uint32_t o = ((uint32_t)(16 * m + lr) * L + kq + 32 * sp.q(sl)) * 2u;
      cbs[sl] = __builtin_bit_cast(bf16x8, buf_load16(rcb, o));
    }
  }
}


// One intra-chunk k-step of row group m (tokens 32q .. 32q+31):
// acc += x^T (decay-masked CB rows)^T.
template <int P>
__device__ __forceinline__ void scan_kstep(f32x4 (&acc)[P / 16], int m, int q, const bf16x8& cbr,
                                           int lr, int kq, int xrow, int xsl, int xcol,
                                           const float* dal2, const float* dls, const float* cfs,
                                           const bf16* xs) {
  const bf16x8 fm = scan_masked_cb(m, q, cbr, lr, kq, dal2, dls, cfs);
#pragma unroll
  for (int a = 0; a < P / 16; ++a)
    acc[a] = Mfma<bf16>::mma(scan_x_operand<P>(xs, q, a, xrow, xsl, xcol), fm, acc[a]);
}

// Persistent chunk_scan for bf16: workgroup b walks the tiles b, b + grid,
// b + 2 grid, ... (grid a multiple of 8, so each tile stays on the XCD of its
// chunk) and has the next tile's inputs in flight while it computes one.
//
// Waves w and w + NPAIR share the mirror pair of row groups m0 = pi and
// m1 = RG-1-pi, which together need RG/2 + 1 intra-chunk k-steps whatever pi
// is.  The first wave owns m0: its inter-chunk term, all of its k-steps, and
// the first k-steps of m1 (NS0 k-steps in all).  The second wave owns m1: its
// inter-chunk term and its remaining NS1 k-steps, which include the diagonal.
// The first wave hands its partial sums for m1 to the second through LDS.
//
// MFMAs compute the transposed tile y^T[p][l]: A = x^T (LDS transpose read)
// or the state (rows p), B = the decay-masked CB row or the C row (columns
// l); a lane holds four consecutive p of one token.
template <int P, int N, int L>
__global__ __launch_bounds__(4 * L) __attribute__((amdgpu_waves_per_eu(4))) void chunk_scan_bf16_kernel(
    ChunkMap cm, int nslots, int ntiles, const bf16* __restrict__ x, const bf16* __restrict__ C,
    const bf16* __restrict__ cb, const float* __restrict__ delta, const float* __restrict__ dAcs,
    const bf16* __restrict__ states_in, const float* __restrict__ D, int H, int G,
    bf16* __restrict__ out) {
  using S = ScanShape<P, N, L>;
  using M = Mfma<bf16>;
  __shared__ __align__(16) bf16 xs[L * P];
  __shared__ __align__(16) bf16 hsm[P * S::HP];
  __shared__ __align__(16) f32x4 red[S::NPAIR * S::PT * kWave];
  __shared__ __align__(16) float dal2[L];   // running sum of delta*A, times log2(e)
  __shared__ __align__(16) float dls[L];    // delta
  __shared__ __align__(16) float cfs[L];    // delta_s * exp(a_r - a_s), r = last token of s's 32-block

  const int w = wave_id();
  const int pi = w % S::NPAIR, kap = w / S::NPAIR;
  const int mg0 = pi, mg1 = S::RG - 1 - pi;          // this pair's row groups
  const int nq0 = mg0 / 2 + 1;                       // 32-token k-steps reaching m0
  const int xs1 = S::NS0 - nq0;                      // k-steps of m1 the first wave takes
  const int mown = kap ? mg1 : mg0;                  // row group this wave finishes
  const int nslot = kap ? S::NS1 : S::NS0;
  const uint32_t HPx = (uint32_t)H * P, GN = (uint32_t)G * N;
  const int grid = gridDim.x;

  ScanSplit sp;
  sp.mg0 = mg0;
  sp.mg1 = mg1;
  sp.nq0 = nq0;
  sp.xs1 = xs1;
  sp.kap = kap;
  sp.mown = mown;
  sp.nslot = nslot;

  int t = blockIdx.x;
  if (t >= ntiles) return;                 // uniform over the workgroup
  ScanTile T = scan_tile(cm, nslots, ntiles, t, H);
  ScanStage<P, N, L> st;
  bf16x8 fc[S::NK];
  bf16x8 cbs[S::NS0];
  {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    scan_prefetch<P, N, L>(T, tid, st, x, states_in, dAcs, delta, H, HPx);
    scan_load_c<N>(T, lane, sp, fc, C, H, G, GN);
    scan_load_cb<P, N, L>(T, lane, sp, cbs, cb, H, G);
  }

  for (; t < ntiles; t += grid) {
    // Lane indices come from an opaque copy of threadIdx.x each tile, so the
    // compiler rebuilds the lane's offsets here instead of holding them in
    // registers across the whole loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int lr = lane & 15, kg = lane >> 4, kq = kg * 8;

    // ---- stage this tile: x (swizzled), state, running sums, factors
#pragma unroll
    for (int u = 0; u < S::XU; ++u) {
      const int i = tid + S::NT * u, r = i / S::CPR, c = i % S::CPR;
      *reinterpret_cast<uint4*>(&xs[r * P + ((c ^ tile_sw<S::CPR>(r)) << 3)]) = st.xv[u];
    }
#pragma unroll
    for (int u = 0; u < S::HU; ++u) {
      const int i = tid + S::NT * u;
      if (i < S::HN) {
        const int r = i / S::HPR, c = i % S::HPR;
        *reinterpret_cast<uint4*>(&hsm[r * S::HP + c * 8]) = st.hv[u];
      }
    }
    {
      const float a2 = st.dA * kLog2e;
      const float a2r = __shfl(a2, lane | 31);   // token tid|31 is in this wave
      if (tid < L) {                             // whole waves
        dal2[tid] = a2;
        dls[tid] = st.dl;
        cfs[tid] = st.dl * exp2_fast(a2r - a2);
      }
    }
    const ScanTile TC = T;
    const float Dh = D ? D[TC.h] : 0.f;
    __syncthreads();

    // ---- the next tile's inputs go in flight (after this tile's operands:
    // the count of outstanding loads drains in issue order)
    T = scan_tile(cm, nslots, ntiles, t + grid, H);
    scan_prefetch<P, N, L>(T, tid, st, x, states_in, dAcs, delta, H, HPx);

    // ---- one intra-chunk k-step: acc += x^T (decay-masked CB row)^T for row
    // group m, tokens s0..s0+31
    f32x4 acc[S::PT];
#pragma unroll
    for (int a = 0; a < S::PT; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int xrow = 8 * kg + (lr >> 2);
    const int xsl = tile_sw<S::CPR>(xrow) >> 1;          // rows xrow + 32q (and +4) share it
    const int xcol = ((lr & 3) >> 1) * 8 + (lr & 1) * 4;
    // ---- phase A (first wave only): its k-steps of the partner's row group
#pragma unroll
    for (int sl = 0; sl < S::NS0; ++sl)
      if (kap == 0 && sl < xs1)             // wave-uniform
        scan_kstep<P>(acc, mg1, sl, cbs[sl], lr, kq, xrow, xsl, xcol, dal2, dls, cfs, xs);
    if (kap == 0) {
#pragma unroll
      for (int a = 0; a < S::PT; ++a) {
        red[(pi * S::PT + a) * kWave + lane] = acc[a];
        acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

    // ---- phase B: inter-chunk term of the own row group,
    //      y^T[p][l] = exp(a_l) * sum_n state[p][n] C[l][n]
#pragma unroll
    for (int k = 0; k < S::NK; ++k)
#pragma unroll
      for (int a = 0; a < S::PT; ++a) {
        const bf16x8 fh = *reinterpret_cast<const bf16x8*>(&hsm[(16 * a + lr) * S::HP + 32 * k + kq]);
        acc[a] = M::mma(fh, fc[k], acc[a]);
      }
    {
      const float rsc = exp2_fast(dal2[16 * mown + lr]);
#pragma unroll
      for (int a = 0; a < S::PT; ++a) acc[a] *= rsc;
    }
    // Loads for the next tile go out in the order they will be used: its C
    // rows now, its CB rows after this tile's last CB use, and only then this
    // tile's stores (the count of outstanding memory operations drains in
    // issue order, so a load queued behind a store waits for that store).
    scan_load_c<N>(T, lane, sp, fc, C, H, G, GN);

    // ---- phase C: the own row group's k-steps
    {
      const int lo = kap ? 0 : xs1;
#pragma unroll
      for (int sl = 0; sl < S::NS0; ++sl)
        if (sl >= lo && sl < nslot)           // wave-uniform
          scan_kstep<P>(acc, mown, kap ? xs1 + sl : sl - xs1, cbs[sl], lr, kq, xrow, xsl, xcol, dal2, dls, cfs, xs);
    }
    scan_load_cb<P, N, L>(T, lane, sp, cbs, cb, H, G);

    // ---- the second wave adds the first wave's part, then each wave
    // finishes its own row group: y = acc + D x, written over x in LDS (each
    // element read and written by the same lane)
    __syncthreads();
    {
      if (kap == 1) {
#pragma unroll
        for (int a = 0; a < S::PT; ++a) acc[a] += red[(pi * S::PT + a) * kWave + lane];
      }
      const int l = 16 * mown + lr;
      const int p4 = kg * 4;
#pragma unroll
      for (int a = 0; a < S::PT; ++a) {
        const int pc = 16 * a + p4;
        bf16x4* e = reinterpret_cast<bf16x4*>(&xs[l * P + (((pc >> 3) ^ tile_sw<S::CPR>(l)) << 3) + (pc & 7)]);
        const bf16x4 xo = *e;
        bf16x4 yo;
#pragma unroll
        for (int r = 0; r < 4; ++r) yo[r] = static_cast<bf16>(acc[a][r] + Dh * static_cast<float>(xo[r]));
        *e = yo;
      }
    }
    __syncthreads();
    {
      // the tile's rows leave as coalesced 16-byte pieces
      const auto ry = rows_rsrc(out, TC, H, P, HPx);
#pragma unroll
      for (int u = 0; u < S::XU; ++u) {
        const int i = tid + S::NT * u, r = i / S::CPR, c = i % S::CPR;
        buf_store16(ry, ((uint32_t)r * HPx + c * 8) * 2u,
                    *reinterpret_cast<const uint4*>(&xs[r * P + ((c ^ tile_sw<S::CPR>(r)) << 3)]));
      }
    }
    __syncthreads();                       // LDS free for the next tile
  }
}


template <int P, int N, int L, int NW, bool GATE = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kTileWavesPerEU<L, NW>))) void
chunk_scan_bf16_tile_kernel(ChunkMap cm, int nslots, const bf16* __restrict__ x,
                            const bf16* __restrict__ C, const bf16* __restrict__ cb,
                            const float* __restrict__ delta, const float* __restrict__ dAcs,
                            const bf16* __restrict__ states_in, const float* __restrict__ D, int H,
                            int G, bf16* __restrict__ out, ScanGate gate) {
  static_assert(L % 64 == 0 && P % 32 == 0 && N % 32 == 0, "tile shape");
  constexpr int HP = N + 8;
  __shared__ __align__(16) bf16 xs[L * P];
  __shared__ __align__(16) bf16 hsm[P * HP];
  __shared__ __align__(16) float dal2[L];   // running sum of delta*A, times log2(e)
  __shared__ __align__(16) float dls[L];    // delta
  __shared__ __align__(16) float cfs[L];    // delta_s * exp(a_r - a_s), r = last token of s's 32-block


  const int2 jh = xcd_chunk_head(blockIdx.x, H);
  if (jh.x >= nslots) return;
  // Whole-chunk decay.  The running sum is monotone inside a chunk (delta is
  // never negative and A is one number per head) and flat past its end, so
  // its value at the last position bounds every |a_s|; read together with
  // the chunk descriptor.
  const float last = dAcs[((int64_t)jh.x * H + jh.y) * L + L - 1];
  ScanTile T{jh.x, jh.y, 0, 0};
  {
    const ChunkDesc d = cm.desc(T.j);
    T.start = d.start;
    T.len = d.len;
  }
  if (T.len <= 0) return;
  if (fabsf(last) * kLog2e <= kScanFastMaxLog2)   // uniform over the workgroup
    scan_tile_body<P, N, L, NW, true, 0, 0, false, GATE>(T, x, C, cb, delta, dAcs, states_in, D, H, G,
                                                        out, xs, hsm, dal2, dls, cfs, gate);
  else
    scan_tile_body<P, N, L, NW, false, 0, 0, false, GATE>(T, x, C, cb, delta, dAcs, states_in, D, H, G,
                                                         out, xs, hsm, dal2, dls, cfs, gate);
}

}  // namespace

// With 256-token chunks one 8-wave workgroup per tile is fastest at every
// grid size measured (5-7% ahead of 4-wave tiles, three workgroups per CU,
// and of the persistent walk on the training batch, long and packed
// sequences).  With shorter chunks, below this many tiles per resident
// persistent workgroup one workgroup per tile is used, above it the
// persistent walk.
constexpr int kPersistentMinTiles = 6;

// Workgroups of the persistent kernel <P, N, L> that stay resident per CU,
// times the CU count, rounded down to a multiple of the 8 XCDs; queried once
// per (instantiation, device) and cached (0 if a query fails).
template <int P, int N, int L>
static int persistent_grid() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int c = cached[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  const int cus = device_cu_count();
  int per_cu = 0;
  if (cus <= 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(
                      &per_cu, chunk_scan_bf16_kernel<P, N, L>, 4 * L, 0) != hipSuccess)
    return 0;
  const int g = (cus * per_cu) / 8 * 8;
  cached[dev].store(g, std::memory_order_relaxed);
  return g;
}

template <typename T, int P, int N, int L>
int chunk_scan_choice(const FwdArgs& a) {
  if constexpr (sizeof(T) != 2) {
    return 0;
  } else {
    const int g = persistent_grid<P, N, L>();
    if (g <= 0) return -1;
    const int ntiles = xcd_grid(a.max_chunks, a.H);
    if constexpr (kTileWaves<L> == 8) return 1;
    return ntiles < kPersistentMinTiles * g ? 1 : 2;
  }
}

template <typename T, int P, int N, int L>
hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t s) {
  static_assert(L % 64 == 0, "chunk size must be a multiple of 64");
  if (a.max_chunks <= 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    auto kern = chunk_scan_bf16_kernel<P, N, L>;
    const int ntiles = xcd_grid(a.max_chunks, a.H);
    int choice = a.scan_kernel;
    if (choice == 0) choice = chunk_scan_choice<T, P, N, L>(a);
    if (choice < 0) return hipErrorInvalidDevice;
    if (choice == 2 && a.gate_z) return hipErrorInvalidValue;   // the caller picks a tile kernel
    if (choice == 2) {
      const int g = persistent_grid<P, N, L>();
      if (g <= 0) return hipErrorInvalidDevice;
      hipLaunchKernelGGL(kern, dim3(g), dim3(4 * L), 0, s, a.cmap(), a.max_chunks, ntiles,
                         (const bf16*)a.x, (const bf16*)a.C, (const bf16*)a.cb, a.delta, a.dAcs,
                         (const bf16*)a.states_in, a.D, a.H, a.G, (bf16*)a.out);
    } else {
      // one workgroup per tile: 4 waves (choice 3) or the chunk size's default;
      // with a gate the tile's store applies the gated RMS norm
      ScanGate gate{};
      if (a.gate_z) {
        gate.z = static_cast<const bf16*>(a.gate_z);
        gate.w = a.gate_w;
        gate.eps = a.gate_eps;
        gate.inv_gs = 1.f / (float)a.gate_gs;
        gate.gpl = a.gate_gs / 8;
      }
      auto go = [&](auto kern, int nw) {
        hipLaunchKernelGGL(kern, dim3(ntiles), dim3(64 * nw), 0, s, a.cmap(), a.max_chunks,
                           (const bf16*)a.x, (const bf16*)a.C, (const bf16*)a.cb, a.delta, a.dAcs,
                           (const bf16*)a.states_in, a.D, a.H, a.G, (bf16*)a.out, gate);
      };
      if (choice == 3) {
        if (a.gate_z) go(chunk_scan_bf16_tile_kernel<P, N, L, 4, true>, 4);
        else go(chunk_scan_bf16_tile_kernel<P, N, L, 4, false>, 4);
      } else {
        constexpr int NW = kTileWaves<L>;
        if (a.gate_z) go(chunk_scan_bf16_tile_kernel<P, N, L, NW, true>, NW);
        else go(chunk_scan_bf16_tile_kernel<P, N, L, NW, false>, NW);
      }
    }
  } else {
    dim3 grid(a.max_chunks * (L / 64), a.H);
    hipLaunchKernelGGL((chunk_scan_kernel<T, P, N, L>), grid, dim3(256), 0, s, a.cmap(),
                       (const T*)a.x, (const T*)a.C, (const T*)a.cb, a.delta, a.dAcs,
                       (const T*)a.states_in, a.D, a.H, a.G, (T*)a.out);
  }
  return hipGetLastError();
}

#define SSD_INST(T, P, N, L)                                                          \
  template hipError_t launch_chunk_scan<T, P, N, L>(const FwdArgs&, hipStream_t); \
  template int chunk_scan_choice<T, P, N, L>(const FwdArgs&);
SSD_FOR_EACH_CONFIG(SSD_INST)
#undef SSD_INST

}  // namespace ssd
