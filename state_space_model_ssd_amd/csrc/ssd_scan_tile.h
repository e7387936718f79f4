// The bf16 chunk_scan tile (internal): one (chunk, head) tile of the output
// construction as a device function, shared by the one-tile-per-workgroup
// kernel, the persistent kernel and the fused forward.  ssd_chunk_scan.hip
// describes the computation and its two paths (rescaled, masked).
#pragma once

#include "ssd_common.h"
#include "ssd_gate.h"

// Multiply-adds are fused into FMAs only inside one expression (not by the
// code generator across statements), so every kernel that inlines these
// bodies, whatever surrounds them, rounds exactly alike.
#pragma clang fp contract(on)

namespace ssd {
namespace {

// One (chunk slot, head) tile as the persistent loop sees it (wave-uniform).
struct ScanTile {
  int j, h, start, len;
};

// Buffer resource over a tile's x (or y) rows: token r of the chunk, head h.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* base, const ScanTile& T,
                                                            int H, int P, uint32_t HPx) {
  const uint32_t bytes = T.len > 0 ? ((uint32_t)(T.len - 1) * HPx + P) * 2u : 0u;
  return buf_rsrc(base + ((int64_t)T.start * H + T.h) * P, bytes);
}

// Largest decay, in powers of two, of a 32-token block for which its
// diagonal k-step uses the factored decay (factors up to 2^64 and down to
// delta 2^-64, far from fp32 over- and underflow).
constexpr float kDiagFactorMaxLog2 = 64.f;

// Decay-masked CB piece of row group m at k-step q (the MFMA B operand):
// M[l][s] = CB[l][s] exp(a_l - a_s) delta_s for s <= l, else 0.
__device__ __forceinline__ bf16x8 scan_masked_cb(int m, int q, const bf16x8& cbr, int lr, int kq,
                                                 const float* dal2, const float* dls,
                                                 const float* cfs) {
  const int s0 = 32 * q;
  const int lrow = 16 * m + lr;
  const float dal = dal2[lrow];
  float mv[8];
  if (s0 + 32 <= 16 * m) {               // below the diagonal: factored decay
    const float rf = exp2_fast(dal - dal2[s0 + 31]);
    const float4 f0 = *reinterpret_cast<const float4*>(&cfs[s0 + kq]);
    const float4 f1 = *reinterpret_cast<const float4*>(&cfs[s0 + kq + 4]);
    const float cf[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) mv[e] = static_cast<float>(cbr[e]) * (rf * cf[e]);
  } else if (dal2[s0] - dal2[s0 + 31] <= kDiagFactorMaxLog2) {
    // on the diagonal, a block whose own decay is within 2^kDiagFactorMaxLog2:
    // the same two factors, exp(a_l - a_r) now >= 1 but bounded by that
    // decay, and tokens after the lane's own masked to zero
    const float rf = exp2_fast(dal - dal2[s0 + 31]);
    const float4 f0 = *reinterpret_cast<const float4*>(&cfs[s0 + kq]);
    const float4 f1 = *reinterpret_cast<const float4*>(&cfs[s0 + kq + 4]);
    const float cf[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    const int t = lrow - s0 - kq;          // element e is token s0 + kq + e
#pragma unroll
    for (int e = 0; e < 8; ++e) mv[e] = e <= t ? static_cast<float>(cbr[e]) * (rf * cf[e]) : 0.f;
  } else {                               // on the diagonal: masked exponential
    const float4 a0 = *reinterpret_cast<const float4*>(&dal2[s0 + kq]);
    const float4 a1 = *reinterpret_cast<const float4*>(&dal2[s0 + kq + 4]);
    const float4 d0 = *reinterpret_cast<const float4*>(&dls[s0 + kq]);
    const float4 d1 = *reinterpret_cast<const float4*>(&dls[s0 + kq + 4]);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // above the diagonal the exponent is -inf, and exp2 gives exactly 0
      const float arg = s0 + kq + e <= lrow ? dal - av[e] : -__builtin_inff();
      mv[e] = static_cast<float>(cbr[e]) * dv[e] * exp2_fast(arg);
    }
  }
  return Mfma<bf16>::pack(mv);
}

// x^T operand (rows p of p-tile a, 8 consecutive tokens of k-step q per lane)
// by transpose read from the swizzled x tile.
template <int P>
__device__ __forceinline__ bf16x8 scan_x_operand(const bf16* xs, int q, int a, int xrow, int xsl,
                                                 int xcol) {
  const int off = ((32 * q + xrow) * P + (2 * (a ^ xsl)) * 8 + xcol) * 2;
  const bf16* p = reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(xs) + off);
  const i16x4 lo = lds_tr16_b64(p);
  const i16x4 hi = lds_tr16_b64(p + 4 * P);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// bf16, one workgroup per (chunk, head) tile: for small grids (a few tiles per
// CU), where two tiles resident per CU overlap each other's loads better than
// one persistent workgroup overlaps its own.  Waves own mirror pairs of row
// groups (two per wave for L >= 128); every load is issued up front in the
// order of use; x is staged XOR-swizzled and read with the transpose read;
// the next k-step's CB rows are in flight while one is multiplied.
// B operands of the MFMAs that add D x to y: column l of the k-step holds
// D at the row of token l itself and zeros elsewhere.  D is split into two
// bf16 parts (hi + lo) so that the products keep about 16 significant bits;
// the MFMA multiplies bf16 exactly and sums in fp32.  t = l - (first token of
// the lane's 8 k values); only 0 <= t < 8 puts a nonzero in this lane.
__device__ __forceinline__ void skip_operands(uint32_t hi, uint32_t lo, int t, bf16x8& fh,
                                              bf16x8& fl) {
  const int sh = (t & 1) * 16;
  const uint32_t vh = hi << sh, vl = lo << sh;
  u32x4 a, b;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const bool on = (t >> 1) == d;       // t < 0 shifts to a negative index
    a[d] = on ? vh : 0u;
    b[d] = on ? vl : 0u;
  }
  fh = __builtin_bit_cast(bf16x8, a);
  fl = __builtin_bit_cast(bf16x8, b);
}

// 8-byte piece of row l of the output tile (P bf16 per row, pieces of 4):
// piece k is stored at k ^ out_sw<P>(l).  Sixteen consecutive rows with one
// logical piece, and two half-rows of 16-byte reads, land on distinct banks.
template <int P>
__device__ __forceinline__ int out_sw(int l) {
  static_assert(P == 32 || P == 64, "output tile swizzle");
  if constexpr (P == 64) return l & 15;
  else return (l >> 1) & 7;
}

// Largest whole-chunk decay, in powers of two, for which chunk_scan stages x
// scaled by delta_s 2^(-a_s) and rescales rows by 2^(a_l): both factors stay
// inside [2^-64, 2^64], far from fp32 and bf16 overflow and underflow.
constexpr float kScanFastMaxLog2 = 64.f;

// Eight bf16 values times w, rounded once to bf16.
__device__ __forceinline__ bf16x8 scale_bf16x8(uint4 v, float w) {
  const bf16x8 b = __builtin_bit_cast(bf16x8, v);
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = static_cast<float>(b[e]) * w;
  return Mfma<bf16>::pack(f);
}


// Inter-chunk MFMAs of a wave: y^T[p][l] += sum_n state[p][n] C[l][n] for its
// row groups (the row factor 2^(a_l) is applied by the caller).
template <int P, int N, int RGW, int HP>
__device__ __forceinline__ void scan_tile_inter(f32x4 (&acc)[RGW][P / 16],
                                                const bf16x8 (&fc)[RGW][N / 32], const bf16* hsm,
                                                int lr, int kq) {
  using M = Mfma<bf16>;
#pragma unroll
  for (int k = 0; k < N / 32; ++k) {
    bf16x8 fh[P / 16];
#pragma unroll
    for (int a = 0; a < P / 16; ++a)
      fh[a] = *reinterpret_cast<const bf16x8*>(&hsm[(16 * a + lr) * HP + 32 * k + kq]);
#pragma unroll
    for (int i = 0; i < RGW; ++i)
#pragma unroll
      for (int a = 0; a < P / 16; ++a) acc[i][a] = M::mma(fh[a], fc[i][k], acc[i][a]);
  }
}

// The gated RMS norm fused into the tile's store: out = rmsnorm(y * silu(z))
// * w over groups of `gpl` 16-byte pieces (8 channels each) of one head's
// row, for norm groups that lie inside a head.  y is the tile's output as
// rounded to bf16 in LDS, so the result equals the standalone norm kernel
// run on the stored y (same arithmetic, same order of the group sum).
struct ScanGate {
  const bf16* z;       // like x and y
  const float* w;      // [H * P]
  float eps, inv_gs;
  int gpl;             // pieces per norm group: 1, 2, 4 or 8 (a power of two, <= P / 8)
};

// z piece u of this thread's rows (the rows the store loop writes).  The
// first min(XU, 4) pieces are loaded before the workgroup meets, the rest
// inside the store loop, four pieces ahead.
template <int P, int NT>
__device__ __forceinline__ uint4 gate_load_z(const ScanGate& gate, const ScanTile& T, int H,
                                             uint32_t HPx, int tid, int u) {
  constexpr int CPR = P / 8;
  const auto rz = rows_rsrc(gate.z, T, H, P, HPx);
  const int i = tid + NT * u, r = i / CPR, c = i % CPR;
  return buf_load16(rz, ((uint32_t)r * HPx + c * 8) * 2u);
}
template <int XU> constexpr int kGateRing = XU < 4 ? XU : 4;

// One 16-byte piece of the gated, normalised output from the y piece and the
// z piece of (row, piece c) of head h.  Every lane calls it (the group sum
// shuffles); the 8 pieces of a row are 8 consecutive lanes.
template <int P>
__device__ __forceinline__ uint4 gate_piece(uint4 yq, uint4 zq, const ScanGate& gate, int h,
                                            int c) {
  const bf16x8 yb = __builtin_bit_cast(bf16x8, yq), zb = __builtin_bit_cast(bf16x8, zq);
  float yf[8], zf[8], g[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    yf[e] = static_cast<float>(yb[e]);
    zf[e] = static_cast<float>(zb[e]);
  }
  const float sum = run_sum(gate_values<8>(yf, zf, g), gate.gpl);
  const float rs = gate_rstd(sum, gate.inv_gs, gate.eps);
  const float4 w0 = *reinterpret_cast<const float4*>(gate.w + h * P + c * 8);
  const float4 w1 = *reinterpret_cast<const float4*>(gate.w + h * P + c * 8 + 4);
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = static_cast<bf16>((g[e] * rs) * wv[e]);
  return __builtin_bit_cast(uint4, o);
}

template <int L> constexpr int kTileWaves = (L / 16) / 2 < 4 ? 4 : (L / 16) / 2;
// Waves per SIMD the tile kernel is compiled for: two workgroups per CU with
// 8-wave tiles; three with 4-wave tiles of four row groups per wave.
template <int L, int NW> constexpr int kTileWavesPerEU = (L / 16) / NW == 4 ? 3 : 4;

// One tile of the bf16 chunk_scan.  FAST: the chunk's whole decay is within
// 2^kScanFastMaxLog2, and the rescaled path runs; otherwise the masked one.
// The two paths share their loads and the inter-chunk term but are compiled
// as separate bodies, so that neither carries the other's registers.
//
// AUX: cache-policy bits of the loads of the entering state, the running sums
// and the steps; CBAUX: of the CB loads (kSc1 when another workgroup of the
// same launch wrote them).  OPQ: the body runs inside a persistent loop.
// GATE: the stored output is the gated RMS norm of y (`gate`).
template <int P, int N, int L, int NW, bool FAST, int AUX = 0, int CBAUX = 0, bool OPQ = false,
          bool GATE = false>
__device__ __forceinline__ void scan_tile_body(const ScanTile& T, const bf16* __restrict__ x,
                                               const bf16* __restrict__ C, const bf16* __restrict__ cb,
                                               const float* __restrict__ delta,
                                               const float* __restrict__ dAcs,
                                               const bf16* __restrict__ states_in,
                                               const float* __restrict__ D, int H, int G, bf16* __restrict__ out,
                                               bf16* xs, bf16* hsm, float* dal2, float* dls, float* cfs,
                                               const ScanGate& gate = ScanGate{}) {
  using M = Mfma<bf16>;
  constexpr int NT = 64 * NW;            // threads
  constexpr int HP = N + 8;              // state tile pitch: conflict-free 16-byte row reads
  constexpr int RG = L / 16;             // 16-row groups of the chunk
  constexpr int RGW = RG / NW;           // row groups per wave: 1, 2 or 4
  static_assert(RGW * NW == RG && (RGW == 1 || RGW == 2 || RGW == 4), "row-group split");
  constexpr int PT = P / 16;
  constexpr int NK = N / 32;             // k-steps of the inter-chunk term
  constexpr int NQ = RG / 2;             // most intra-chunk k-steps of one row group
  constexpr int CPR = P / 8;             // 16-byte pieces per x row
  constexpr int XU = L * CPR / NT;       // x pieces per thread
  constexpr int HPR = N / 8;             // 16-byte pieces per state row
  constexpr int HU = (P * HPR + NT - 1) / NT;
  static_assert((L * CPR) % NT == 0 && L <= NT, "x staging");
  const int h = T.h, g = h / (H / G);
  const uint32_t HPx = (uint32_t)H * P, GN = (uint32_t)G * N;
  const int tid = body_tid<OPQ, NT>(), w = wave_id(), lane = tid & 63;
  const int lr = lane & 15, kg = lane >> 4, kq = kg * 8;
  const bool has_d = D != nullptr;
  const float Dh = has_d ? D[h] : 0.f;
  // Row groups of this wave; with two per wave they pair from both ends of
  // the chunk, with four from both ends of each half, so every wave carries
  // the same causal work (the last one listed reaches furthest).
  int mg[RGW];
  mg[0] = w;
  if constexpr (RGW == 2) mg[1] = RG - 1 - w;
  if constexpr (RGW == 4) {
    mg[1] = 2 * NW - 1 - w;
    mg[2] = 2 * NW + w;
    mg[3] = RG - 1 - w;
  }
  int lrow[RGW], nq[RGW];
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    lrow[i] = 16 * mg[i] + lr;
    nq[i] = mg[i] / 2 + 1;               // k-steps that reach this row group
  }

  // ---- global loads issued together, in the order they are used
  const auto rx = rows_rsrc(x, T, H, P, HPx);
  uint4 xv[XU];
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tid + NT * u, r = i / CPR, c = i % CPR;
    xv[u] = buf_load16(rx, ((uint32_t)r * HPx + c * 8) * 2u);
  }
  const int64_t jhl = (int64_t)T.j * H + h;
  const auto rh = buf_rsrc(states_in + jhl * P * N, P * N * 2);
  uint4 hv[HU];
#pragma unroll
  for (int u = 0; u < HU; ++u) hv[u] = buf_load16<AUX>(rh, (uint32_t)(tid + NT * u) * 16);
  const float dA_t = buf_load4<AUX>(buf_rsrc(dAcs + jhl * L, L * 4), tid * 4);
  const float dl_t = buf_load4<AUX>(buf_rsrc(delta + jhl * L, L * 4), tid * 4);
  const auto rc = buf_rsrc(C + ((int64_t)T.start * G + g) * N, ((uint32_t)(T.len - 1) * GN + N) * 2u);
  // C rows of this lane, all n-steps.  With four row groups per wave the
  // last two groups' rows are issued once x and the state are staged, so
  // that they do not share registers with the staging loads.
  constexpr int RGE = RGW == 4 ? 2 : RGW;
  bf16x8 fc[RGW][NK];
#pragma unroll
  for (int i = 0; i < RGE; ++i)
#pragma unroll
    for (int k = 0; k < NK; ++k)
      fc[i][k] = __builtin_bit_cast(bf16x8, buf_load16(rc, ((uint32_t)lrow[i] * GN + 32 * k + kq) * 2u));
  const auto rcb = buf_rsrc(cb + ((int64_t)T.j * G + g) * L * L, L * L * 2);

  // ---- stage x as loaded (swizzled; rows past the end arrived as zeros),
  // the state, the running sums and the per-token factors
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tid + NT * u, r = i / CPR, c = i % CPR;
    *reinterpret_cast<uint4*>(&xs[r * P + ((c ^ tile_sw<CPR>(r)) << 3)]) = xv[u];
  }
#pragma unroll
  for (int u = 0; u < HU; ++u) {
    const int i = tid + NT * u, r = i / HPR, c = i % HPR;
    // the guard is a constant where the threads split the tile evenly: with
    // one that depends on the thread the compiler would move the second load
    // of the state down to this store and wait for it there
    if ((P * HPR) % NT == 0 || i < P * HPR) *reinterpret_cast<uint4*>(&hsm[r * HP + c * 8]) = hv[u];
  }
  {
    const float a2 = dA_t * kLog2e;
    const float a2r = __shfl(a2, lane | 31);   // token tid|31 is in this wave
    if (tid < L) {                             // whole waves
      dal2[tid] = a2;
      dls[tid] = dl_t;
      cfs[tid] = dl_t * exp2_fast(a2r - a2);
    }
  }
#pragma unroll
  for (int i = RGE; i < RGW; ++i)
#pragma unroll
    for (int k = 0; k < NK; ++k)
      fc[i][k] = __builtin_bit_cast(bf16x8, buf_load16(rc, ((uint32_t)lrow[i] * GN + 32 * k + kq) * 2u));
  // Masked path with one or two row groups per wave, one tile per
  // workgroup: CB pieces stream through a ring of RM registers per row
  // group, RM - 1 k-steps ahead of their use, the first RM - 1 issued once
  // the inter-chunk term has released the C rows' registers.  (Inside a
  // persistent loop the registers are not there: one step ahead.)  The order
  // of the MFMAs is the same either way.
  constexpr bool MRING = !FAST && RGW <= 2 && !OPQ;
  constexpr int RM = GATE ? 3 : 4;         // the gate's store loop needs registers too
  bf16x8 mring[RGW][MRING ? RM : 1];
  const int xrow = 8 * kg + (lr >> 2);
  const int xsl = tile_sw<CPR>(xrow) >> 1;
  const int xcol = ((lr & 3) >> 1) * 8 + (lr & 1) * 4;
  const int nq_wave = nq[RGW - 1];
  f32x4 acc[RGW][PT];
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int a = 0; a < PT; ++a) acc[i][a] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  scan_tile_inter<P, N, RGW, HP>(acc, fc, hsm, lr, kq);
  if constexpr (MRING) {
#pragma unroll
    for (int i = 0; i < RGW; ++i)
#pragma unroll
      for (int q = 0; q < RM - 1; ++q)
        if (q < nq[i])                     // wave-uniform
          mring[i][q] = __builtin_bit_cast(bf16x8, buf_load16<CBAUX>(rcb, ((uint32_t)lrow[i] * L + kq + 32 * q) * 2u));
  }

  if constexpr (FAST) {
    // Every term of the chunk is accumulated without its row factor 2^(a_l),
    // applied once at the end: D x enters divided by it (while x is still
    // staged as loaded), and x is then rescaled in place to x_s delta_s
    // 2^(-a_s), so that the intra-chunk terms carry their decay
    // 2^(a_l - a_s) and the CB rows enter the MFMAs as loaded.
    // |a| <= kScanFastMaxLog2 keeps every factor far from over- and underflow.
    if (has_d) {
#pragma unroll
      for (int i = 0; i < RGW; ++i) {
        const int q = nq[i] - 1;           // the row group's diagonal step
        const float dd = Dh * exp2_fast(-dal2[lrow[i]]);
        const bf16 d1 = static_cast<bf16>(dd);
        const bf16 d2 = static_cast<bf16>(dd - static_cast<float>(d1));
        bf16x8 fdh, fdl;
        skip_operands(__builtin_bit_cast(unsigned short, d1), __builtin_bit_cast(unsigned short, d2),
                      lrow[i] - 32 * q - kq, fdh, fdl);
#pragma unroll
        for (int a = 0; a < PT; ++a) {
          const bf16x8 fx = scan_x_operand<P>(xs, q, a, xrow, xsl, xcol);
          acc[i][a] = M::mma(fx, fdh, acc[i][a]);
          acc[i][a] = M::mma(fx, fdl, acc[i][a]);
        }
      }
    }
    // CB pieces stream through a ring of RD per row group, and enter the
    // MFMAs as loaded (the stored CB is 0 above the diagonal, so the diagonal
    // step needs no mask): the first RD - 1 steps' pieces are in flight while
    // x is rescaled, and each step issues the pieces RD - 1 steps ahead (the
    // loop is unrolled, so the slots are fixed registers).  Steps past a row
    // group's last load nothing.
    constexpr int RD = RGW == 4 ? 2 : 3;   // ring slots (registers) per row group
    bf16x8 ring[RGW][RD];
#pragma unroll
    for (int i = 0; i < RGW; ++i)
#pragma unroll
      for (int q = 0; q < RD - 1; ++q)
        if (q < nq[i])                     // wave-uniform
          ring[i][q] = __builtin_bit_cast(bf16x8, buf_load16<CBAUX>(rcb, ((uint32_t)lrow[i] * L + kq + 32 * q) * 2u));
    __syncthreads();                       // x as loaded is no longer read
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int i = tid + NT * u, r = i / CPR, c = i % CPR;
      uint4* e = reinterpret_cast<uint4*>(&xs[r * P + ((c ^ tile_sw<CPR>(r)) << 3)]);
      *e = __builtin_bit_cast(uint4, scale_bf16x8(*e, dls[r] * exp2_fast(-dal2[r])));
    }
    __syncthreads();
    // The x^T operands run through a ring of XR registers over the sequence
    // (step, p-tile): each is read XR operands before its MFMAs, so the LDS
    // latency overlaps the MFMAs of the ones before it.  Reads past the last
    // step stay inside the tile and go unused.
    constexpr int XR = 3;
    constexpr int NOP = NQ * PT;
    bf16x8 fxr[XR];
#pragma unroll
    for (int n = 0; n < XR; ++n) fxr[n] = scan_x_operand<P>(xs, n / PT, n % PT, xrow, xsl, xcol);
    bf16x8 fb[RGW];
#pragma unroll
    for (int n = 0; n < NOP; ++n) {
      const int q = n / PT, a = n % PT;
      if (a == 0) {
        if (q >= nq_wave) break;           // wave-uniform
#pragma unroll
        for (int i = 0; i < RGW; ++i)
          if (q + RD - 1 < nq[i])          // wave-uniform
            ring[i][(q + RD - 1) % RD] = __builtin_bit_cast(
                bf16x8, buf_load16<CBAUX>(rcb, ((uint32_t)lrow[i] * L + kq + 32 * (q + RD - 1)) * 2u));
#pragma unroll
        for (int i = 0; i < RGW; ++i)
          if (q < nq[i]) fb[i] = ring[i][q % RD];
      }
#pragma unroll
      for (int i = 0; i < RGW; ++i)
        if (q < nq[i]) acc[i][a] = M::mma(fxr[n % XR], fb[i], acc[i][a]);   // wave-uniform
      if (n + XR < NOP) fxr[n % XR] = scan_x_operand<P>(xs, (n + XR) / PT, (n + XR) % PT, xrow, xsl, xcol);
    }
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      const float rsc = exp2_fast(dal2[lrow[i]]);
#pragma unroll
      for (int a = 0; a < PT; ++a) acc[i][a] *= rsc;
    }
  } else {
    // ---- exact path: each CB piece is masked with its decay
    // exp(a_l - a_s) delta_s; the next step's CB rows are in flight while
    // one is multiplied.  With four row groups per wave, two passes over the
    // k-steps take two row groups each (the pairs mirror inside each half of
    // the chunk, so the second of a pass reaches furthest).
    constexpr int RP = RGW == 4 ? 2 : RGW;   // row groups per pass
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      const float rsc = exp2_fast(dal2[lrow[i]]);
#pragma unroll
      for (int a = 0; a < PT; ++a) acc[i][a] *= rsc;
    }
    if constexpr (MRING) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q >= nq_wave) break;           // wave-uniform
#pragma unroll
        for (int i = 0; i < RGW; ++i)
          if (q + RM - 1 < nq[i])          // wave-uniform
            mring[i][(q + RM - 1) % RM] = __builtin_bit_cast(
                bf16x8, buf_load16<CBAUX>(rcb, ((uint32_t)lrow[i] * L + kq + 32 * (q + RM - 1)) * 2u));
        bf16x8 fm[RGW];
#pragma unroll
        for (int i = 0; i < RGW; ++i)
          if (q < nq[i]) fm[i] = scan_masked_cb(mg[i], q, mring[i][q % RM], lr, kq, dal2, dls, cfs);
#pragma unroll
        for (int a = 0; a < PT; ++a) {
          const bf16x8 fx = scan_x_operand<P>(xs, q, a, xrow, xsl, xcol);
#pragma unroll
          for (int i = 0; i < RGW; ++i)
            if (q < nq[i]) acc[i][a] = M::mma(fx, fm[i], acc[i][a]);   // wave-uniform
        }
      }
    }
#pragma unroll
    for (int i0 = 0; i0 < (MRING ? 0 : RGW); i0 += RP) {
      uint32_t cbo[RP];
      bf16x8 cur[RP];                      // CB rows of the current k-step
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        cbo[r] = ((uint32_t)lrow[i0 + r] * L + kq) * 2u;
        cur[r] = __builtin_bit_cast(bf16x8, buf_load16<CBAUX>(rcb, cbo[r]));
      }
      const int nqp = nq[i0 + RP - 1];
      for (int q = 0; q < nqp; ++q) {
        const int sn = min(32 * q + 32, L - 32);   // next step (clamped: always in the row)
        bf16x8 nxt[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) nxt[r] = __builtin_bit_cast(bf16x8, buf_load16<CBAUX>(rcb, cbo[r] + sn * 2));
        bf16x8 fm[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r)
          if (q < nq[i0 + r]) fm[r] = scan_masked_cb(mg[i0 + r], q, cur[r], lr, kq, dal2, dls, cfs);
#pragma unroll
        for (int a = 0; a < PT; ++a) {
          const bf16x8 fx = scan_x_operand<P>(xs, q, a, xrow, xsl, xcol);
#pragma unroll
          for (int r = 0; r < RP; ++r)
            if (q < nq[i0 + r]) acc[i0 + r][a] = M::mma(fx, fm[r], acc[i0 + r][a]);   // wave-uniform
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) cur[r] = nxt[r];
      }
    }
    // y = acc + D x, written over x (each element read and written by one lane)
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RGW; ++i)
#pragma unroll
      for (int a = 0; a < PT; ++a) {
        const int l = lrow[i], pc = 16 * a + 4 * kg;
        bf16x4* e = reinterpret_cast<bf16x4*>(&xs[l * P + (((pc >> 3) ^ tile_sw<CPR>(l)) << 3) + (pc & 7)]);
        const bf16x4 xo = *e;
        bf16x4 yo;
#pragma unroll
        for (int r = 0; r < 4; ++r) yo[r] = static_cast<bf16>(acc[i][a][r] + Dh * static_cast<float>(xo[r]));
        *e = yo;
      }
    constexpr int ZR = GATE ? kGateRing<XU> : 1;
    uint4 zv[ZR];
    if constexpr (GATE) {
#pragma unroll
      for (int u = 0; u < ZR; ++u) zv[u] = gate_load_z<P, NT>(gate, T, H, HPx, tid, u);
    }
    __syncthreads();
    const auto ry = rows_rsrc(out, T, H, P, HPx);
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int i = tid + NT * u, r = i / CPR, c = i % CPR;
      uint4 yq = *reinterpret_cast<const uint4*>(&xs[r * P + ((c ^ tile_sw<CPR>(r)) << 3)]);
      if constexpr (GATE) {
        const uint4 zq = zv[u % ZR];
        if (u + ZR < XU) zv[u % ZR] = gate_load_z<P, NT>(gate, T, H, HPx, tid, u + ZR);
        yq = gate_piece<P>(yq, zq, gate, h, c);
      }
      buf_store16(ry, ((uint32_t)r * HPx + c * 8) * 2u, yq);
    }
    return;
  }

  // ---- fast path epilogue: y goes to LDS over x (every wave is done with
  // x) in the out_sw layout, a lane's four p of one token as one 8-byte
  // piece; then the rows leave coalesced
  __syncthreads();
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int a = 0; a < PT; ++a) {
      const int l = lrow[i];
      bf16x4 yo;
#pragma unroll
      for (int r = 0; r < 4; ++r) yo[r] = static_cast<bf16>(acc[i][a][r]);
      *reinterpret_cast<bf16x4*>(&xs[l * P + ((4 * a + kg) ^ out_sw<P>(l)) * 4]) = yo;
    }
  constexpr int ZR = GATE ? kGateRing<XU> : 1;
  uint4 zv[ZR];
  if constexpr (GATE) {
#pragma unroll
    for (int u = 0; u < ZR; ++u) zv[u] = gate_load_z<P, NT>(gate, T, H, HPx, tid, u);
  }
  __syncthreads();
  const auto ry = rows_rsrc(out, T, H, P, HPx);
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int i = tid + NT * u, r = i / CPR, c = i % CPR;
    const int sw = out_sw<P>(r);
    const uint2 v0 = *reinterpret_cast<const uint2*>(&xs[r * P + ((2 * c) ^ sw) * 4]);
    const uint2 v1 = *reinterpret_cast<const uint2*>(&xs[r * P + ((2 * c + 1) ^ sw) * 4]);
    uint4 yq = make_uint4(v0.x, v0.y, v1.x, v1.y);
    if constexpr (GATE) {
      const uint4 zq = zv[u % ZR];
      if (u + ZR < XU) zv[u % ZR] = gate_load_z<P, NT>(gate, T, H, HPx, tid, u + ZR);
      yq = gate_piece<P>(yq, zq, gate, h, c);
    }
    buf_store16(ry, ((uint32_t)r * HPx + c * 8) * 2u, yq);
  }
}

}  // namespace
}  // namespace ssd

#pragma clang fp contract(fast)
