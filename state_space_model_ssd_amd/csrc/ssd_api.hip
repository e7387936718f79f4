// C ABI of the SSD forward (declared in include/ssd.h): host-side argument
// checks, workspace layout, and the stage launches on the caller's stream.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "ssd.h"
#include "ssd_kernels.h"

namespace ssd {

int device_cu_count() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

typedef hipError_t (*launch_fn)(const FwdArgs&, hipStream_t);

typedef hipError_t (*launch_bwd_fn)(const FwdArgs&, const BwdArgs&, hipStream_t);
typedef int (*choice_fn)(const FwdArgs&);

typedef hipError_t (*launch_fused_fn)(const FwdArgs&, int, hipStream_t);

struct Kernels {
  int32_t dtype;
  int64_t P, N, L;
  launch_fn bmm, chunk_state, state_passing, chunk_scan, front;
  launch_bwd_fn backward;
  choice_fn scan_choice;
  launch_fused_fn fused;   // nullptr: no fused forward for this configuration
};

template <typename T> constexpr int32_t dtype_of();
template <> constexpr int32_t dtype_of<float>() { return SSD_F32; }
template <> constexpr int32_t dtype_of<bf16>() { return SSD_BF16; }

#define SSD_ROW(T, P, N, L)                                                              \
  {dtype_of<T>(), P, N, L, &launch_bmm_chunk<T, N, L>, &launch_chunk_state<T, P, N, L>, \
   &launch_state_passing<T>, &launch_chunk_scan<T, P, N, L>,                          \
   sizeof(T) == 2 ? &launch_front<T, P, N, L> : nullptr, &launch_backward<T, P, N, L>,   \
   &chunk_scan_choice<T, P, N, L>,                                                      \
   fused_supported<T, P, N, L>() ? &launch_fused<T, P, N, L> : nullptr},
const Kernels kKernels[] = {SSD_FOR_EACH_CONFIG(SSD_ROW)};
#undef SSD_ROW

const Kernels* find_kernels(int32_t dtype, int64_t P, int64_t N, int64_t L) {
  for (const Kernels& k : kKernels)
    if (k.dtype == dtype && k.P == P && k.N == N && k.L == L) return &k;
  return nullptr;
}

size_t elem_size(int32_t dtype) { return dtype == SSD_BF16 ? 2 : 4; }

// Shape checks that do not look at pointers.
ssd_status_t check_problem(const ssd_problem_t* p) {
  if (!p) return SSD_ERR_INVALID_ARG;
  if (p->batch < 1 || p->seqlen < 0 || p->nheads < 1 || p->headdim < 1 || p->dstate < 1 ||
      p->ngroups < 1 || p->chunk_size < 1 || p->nseq < 0)
    return SSD_ERR_INVALID_ARG;
  if (p->nheads % p->ngroups != 0) return SSD_ERR_INVALID_ARG;
  if (p->dtype != SSD_F32 && p->dtype != SSD_BF16) return SSD_ERR_INVALID_ARG;
  if (p->nseq > 0 && p->batch != 1) return SSD_ERR_INVALID_ARG;
  if (isnan(p->dt_min) || isnan(p->dt_max) || p->dt_min > p->dt_max) return SSD_ERR_INVALID_ARG;
  // int32 token and chunk indices on the device; grid limits
  if (p->batch * p->seqlen > (int64_t)INT32_MAX / 2) return SSD_ERR_UNSUPPORTED;
  if (p->nheads > 65535) return SSD_ERR_UNSUPPORTED;
  const int64_t nstates = p->nseq > 0 ? p->nseq : p->batch;
  if (nstates > 65535) return SSD_ERR_UNSUPPORTED;
  if (!find_kernels(p->dtype, p->headdim, p->dstate, p->chunk_size)) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

int64_t max_chunks_of(const ssd_problem_t* p) {
  const int64_t L = p->chunk_size;
  if (p->nseq > 0) {
    // sum_s ceil(len_s / L) <= (T + nseq (L - 1)) / L, and never more than
    // one chunk per token
    const int64_t bound = (p->seqlen + p->nseq * (L - 1)) / L;
    return bound < p->seqlen ? bound : p->seqlen;
  }
  return p->batch * ((p->seqlen + L - 1) / L);
}

// The blocked state_passing (associative scan over blocks of chunks) is
// for problems whose state elements, one chain each, cannot keep the HBM
// busy: fewer than one wave of 64 lanes, 4 elements each, per SIMD of the
// device.  The workspace reserves the blocks' storage for problems under
// kSpReserveElems state elements, a fixed bound (the reported workspace
// size never depends on the device); the threshold the library uses is the
// device's, capped at that bound.
constexpr int64_t kSpReserveElems = int64_t(1) << 18;
constexpr int kSpMaxBlocks = 16;

int64_t state_elems(const ssd_problem_t* p) {
  const int64_t nstates = p->nseq > 0 ? p->nseq : p->batch;
  return nstates * p->nheads * p->headdim * p->dstate;
}

// State elements below which the library blocks the chain on this device.
int64_t sp_block_threshold() {
  const int cus = device_cu_count();
  const int64_t t = cus > 0 ? (int64_t)cus * 4 * 64 * 4 : kSpReserveElems;
  return t < kSpReserveElems ? t : kSpReserveElems;
}

// The library's own block count.  Blocking costs a second launch and a
// second read of the chunk states, which measured slower for sequences of
// 32 and 64 chunks and up to 37% faster from 256 chunks on; so: sequences of
// at least 128 chunks on average, enough blocks to reach the device's
// threshold in chains, and blocks of at least 16 chunks.
int auto_sp_blocks(const ssd_problem_t* p, int64_t max_chunks) {
  const int64_t elems = state_elems(p);
  const int64_t nstates = p->nseq > 0 ? p->nseq : p->batch;
  const int64_t per_seq = max_chunks / (nstates > 0 ? nstates : 1);
  const int64_t thr = sp_block_threshold();
  if (elems <= 0 || elems >= thr || per_seq < 128) return 1;
  int kb = 1;
  while (kb < kSpMaxBlocks && elems * kb < thr && per_seq >= 16 * (2 * kb)) kb *= 2;
  return kb;
}

void layout_of(const ssd_problem_t* p, ssd_workspace_layout_t* w) {
  const int64_t mc = max_chunks_of(p);
  const int64_t nstates = p->nseq > 0 ? p->nseq : p->batch;
  const size_t H = p->nheads, L = p->chunk_size, PN = p->headdim * p->dstate;
  size_t off = 0;
  w->max_chunks = mc;
  w->chunk_table = off;  off = align_up(off + sizeof(int32_t) * 4 * (size_t)mc);
  w->seq_chunks = off;   off = align_up(off + sizeof(int32_t) * (size_t)(nstates + 1));
  w->delta = off;        off = align_up(off + sizeof(float) * (size_t)mc * H * L);
  w->dA_cumsum = off;    off = align_up(off + sizeof(float) * (size_t)mc * H * L);
  w->cb = off;           off = align_up(off + elem_size(p->dtype) * (size_t)mc * p->ngroups * L * L);
  w->chunk_states = off; off = align_up(off + sizeof(float) * (size_t)mc * H * PN);
  w->states_in = off;    off = align_up(off + elem_size(p->dtype) * (size_t)mc * H * PN);
  w->sp_blocks = state_elems(p) < kSpReserveElems ? kSpMaxBlocks : 1;
  const size_t kbw = w->sp_blocks > 1 ? (size_t)w->sp_blocks : 0;
  w->block_states = off;   off = align_up(off + sizeof(float) * (size_t)nstates * kbw * H * PN);
  w->block_logdecay = off; off = align_up(off + sizeof(float) * (size_t)nstates * kbw * H);
  w->sync = off;           off = align_up(off + fused_sync_bytes((int)nstates, (int)H, (int)p->ngroups, (int)mc));
  w->total_bytes = off;
}

// Ranges of the pinned kernel choices (0 keeps the library's choice).
ssd_status_t check_tuning(const ssd_problem_t* p, const ssd_tuning_t& t, int64_t ws_blocks) {
  const bool bf16 = p->dtype == SSD_BF16;
  if (t.sp_blocks != 0 && t.sp_blocks != 1 && t.sp_blocks != 2 && t.sp_blocks != 4 &&
      t.sp_blocks != 8 && t.sp_blocks != 16)
    return SSD_ERR_INVALID_ARG;
  if (t.sp_blocks > ws_blocks) return SSD_ERR_INVALID_ARG;
  if (t.scan_kernel < 0 || t.scan_kernel > 3 || (!bf16 && t.scan_kernel != 0)) return SSD_ERR_INVALID_ARG;
  if (t.sp_vec != 0 && t.sp_vec != 1 && t.sp_vec != 2 && t.sp_vec != 4) return SSD_ERR_INVALID_ARG;
  if (t.front < 0 || t.front > 2 || (!bf16 && t.front != 0)) return SSD_ERR_INVALID_ARG;
  if (t.fused < 0 || t.fused > 2) return SSD_ERR_INVALID_ARG;
  if (t.fused == 2) {
    const Kernels* k = find_kernels(p->dtype, p->headdim, p->dstate, p->chunk_size);
    // the fused launch has its own state passing and its own (8-wave) scan tile
    if (!k || !k->fused || t.sp_blocks > 1 || t.front == 2 || (t.sp_vec != 0 && t.sp_vec != 4) ||
        t.scan_kernel == 2)
      return SSD_ERR_INVALID_ARG;
  }
  return SSD_OK;
}

// The arguments common to the forward and the backward: pointer checks and
// the forward's part of the workspace.
ssd_status_t fill_args(const ssd_problem_t* p, const ssd_workspace_layout_t& w,
                       const ssd_tuning_t& tune, const void* x, const float* dt,
                       const float* dt_bias, const float* A, const void* B, const void* C,
                       const float* D, const float* initial_states, const int32_t* cu_seqlens,
                       const int32_t* seq_idx, void* out, float* final_states, void* workspace,
                       FwdArgs* out_args) {
  const bool packed = p->nseq > 0;
  const int64_t tokens = p->batch * p->seqlen;
  // a packed batch names its sequences by exactly one of the two arrays; with
  // no tokens (every sequence empty) it may pass neither
  if (packed && cu_seqlens && seq_idx) return SSD_ERR_INVALID_ARG;
  if (packed && !cu_seqlens && !seq_idx && tokens > 0) return SSD_ERR_INVALID_ARG;
  if (!packed && (cu_seqlens || seq_idx)) return SSD_ERR_INVALID_ARG;
  if (tokens > 0 && (!x || !dt || !A || !B || !C)) return SSD_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return SSD_ERR_WORKSPACE;

  FwdArgs& a = *out_args;
  a.batch = (int)p->batch;
  a.seqlen = (int)p->seqlen;
  a.H = (int)p->nheads;
  a.P = (int)p->headdim;
  a.N = (int)p->dstate;
  a.G = (int)p->ngroups;
  a.L = (int)p->chunk_size;
  a.nstates = (int)(packed ? p->nseq : p->batch);
  a.max_chunks = (int)w.max_chunks;
  a.nc_row = (int)((p->seqlen + p->chunk_size - 1) / p->chunk_size);
  a.packed = packed;
  a.dt_min = p->dt_min;
  a.dt_max = p->dt_max;
  a.scan_kernel = tune.scan_kernel;
  a.sp_vec = tune.sp_vec;
  a.sp_blocks = tune.sp_blocks > 0 ? tune.sp_blocks : auto_sp_blocks(p, w.max_chunks);
  a.fused = tune.fused;
  a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.D = D;
  a.init = initial_states;
  a.cu_seqlens = cu_seqlens;
  a.seq_idx = seq_idx;
  a.out = out;
  a.final_states = final_states;
  char* base = static_cast<char*>(workspace);
  a.table = reinterpret_cast<int4*>(base + w.chunk_table);
  a.seq_chunks = reinterpret_cast<int*>(base + w.seq_chunks);
  a.delta = reinterpret_cast<float*>(base + w.delta);
  a.dAcs = reinterpret_cast<float*>(base + w.dA_cumsum);
  a.cb = base + w.cb;
  a.chunk_states = reinterpret_cast<float*>(base + w.chunk_states);
  a.states_in = base + w.states_in;
  a.block_states = w.sp_blocks > 1 ? reinterpret_cast<float*>(base + w.block_states) : nullptr;
  a.block_logdecay = w.sp_blocks > 1 ? reinterpret_cast<float*>(base + w.block_logdecay) : nullptr;
  a.sync = reinterpret_cast<int*>(base + w.sync);
  a.zero_ints = 0;
  a.gate_z = nullptr;
  a.gate_w = nullptr;
  a.gate_eps = 0.f;
  a.gate_gs = 0;
  return SSD_OK;
}

// 2: the fused forward, 1: separate launches.  A pinned choice wins; the
// library's own keeps separate launches (the fused one uses the one-chain
// state passing, so it is never picked where the blocked one is).
int fused_choice(const ssd_problem_t* p, const FwdArgs& a, const ssd_tuning_t& tune) {
  (void)p;
  if (tune.fused != 0) return tune.fused;
  if (a.sp_blocks > 1 || tune.front == 2) return 1;
  return 1;
}

ssd_status_t launch_stages(const ssd_problem_t* p, const FwdArgs& a, uint32_t stages,
                           const ssd_tuning_t& tune, void* stream) {
  const Kernels* k = find_kernels(p->dtype, p->headdim, p->dstate, p->chunk_size);
  hipStream_t s = static_cast<hipStream_t>(stream);
  struct Step { uint32_t bit; launch_fn fn; };
  const Step steps[] = {
      {SSD_STAGE_PLAN, &launch_plan},
      {SSD_STAGE_CUMSUM, &launch_chunk_cumsum},
      {SSD_STAGE_BMM, k->bmm},
      {SSD_STAGE_CHUNK_STATE, k->chunk_state},
      {SSD_STAGE_STATE_PASSING, k->state_passing},
      {SSD_STAGE_CHUNK_SCAN, k->chunk_scan},
  };
  // Stages 1-5 as one fused launch: when all of them are asked for and the
  // caller pinned it (or the library picks it for the shape).
  constexpr uint32_t kAfterPlan = SSD_STAGE_ALL & ~(uint32_t)SSD_STAGE_PLAN;
  if (k->fused && (stages & kAfterPlan) == kAfterPlan && fused_choice(p, a, tune) == 2) {
    if ((stages & SSD_STAGE_PLAN) && launch_plan(a, s) != hipSuccess) return SSD_ERR_HIP;
    const int scan = tune.scan_kernel != 0 ? tune.scan_kernel : k->scan_choice(a);
    if (scan < 0) return SSD_ERR_HIP;
    if (k->fused(a, scan, s) != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
  }
  // The bf16 path runs stages 1-3 as one launch when all three are asked for.
  constexpr uint32_t kFront = SSD_STAGE_CUMSUM | SSD_STAGE_BMM | SSD_STAGE_CHUNK_STATE;
  const bool fuse_front = k->front && (stages & kFront) == kFront && tune.front != 2;
  for (const Step& stp : steps) {
    if (!(stages & stp.bit)) continue;
    if (fuse_front && (stp.bit & kFront)) {
      if (stp.bit == SSD_STAGE_CUMSUM && k->front(a, s) != hipSuccess) return SSD_ERR_HIP;
      continue;
    }
    if (stp.fn(a, s) != hipSuccess) return SSD_ERR_HIP;
  }
  return SSD_OK;
}

ssd_status_t check_norm(const ssd_norm_problem_t* p);
NormArgs norm_args(const ssd_norm_problem_t* p);

ssd_status_t run(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias,
                 const float* A, const void* B, const void* C, const float* D,
                 const float* initial_states, const int32_t* cu_seqlens, const int32_t* seq_idx,
                 void* out, float* final_states, void* workspace, size_t workspace_bytes,
                 uint32_t stages, const ssd_tuning_t* tuning, void* stream,
                 const ssd_gate_t* gate = nullptr) {
  ssd_status_t st = check_problem(p);
  if (st != SSD_OK) return st;
  if (stages & ~(uint32_t)SSD_STAGE_ALL) return SSD_ERR_INVALID_ARG;
  const ssd_tuning_t tune = tuning ? *tuning : ssd_tuning_t{0, 0, 0, 0, 0};
  ssd_workspace_layout_t w;
  layout_of(p, &w);
  st = check_tuning(p, tune, w.sp_blocks);
  if (st != SSD_OK) return st;
  const int64_t tokens = p->batch * p->seqlen;
  if (tokens > 0 && !out) return SSD_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < w.total_bytes) return SSD_ERR_WORKSPACE;
  FwdArgs a;
  st = fill_args(p, w, tune, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx, out,
                 final_states, workspace, &a);
  if (st != SSD_OK) return st;
  if (!gate) return launch_stages(p, a, stages, tune, stream);
  // the gated RMS norm after the forward: fused into chunk_scan's store when
  // its groups lie inside a head and a one-tile-per-workgroup scan kernel
  // runs, else a launch of its own over `out` in place
  const ssd_norm_problem_t np{tokens, p->nheads * p->headdim, gate->group_size, p->dtype, gate->eps};
  st = check_norm(&np);
  if (st != SSD_OK) return st;
  if (tokens > 0 && (!gate->z || !gate->weight)) return SSD_ERR_INVALID_ARG;
  const Kernels* k = find_kernels(p->dtype, p->headdim, p->dstate, p->chunk_size);
  const int scan = tune.scan_kernel != 0 ? tune.scan_kernel : k->scan_choice(a);
  if (scan < 0) return SSD_ERR_HIP;
  const bool fusable = p->dtype == SSD_BF16 && p->headdim % gate->group_size == 0 &&
                       (scan == 1 || scan == 3) && fused_choice(p, a, tune) != 2;
  if (fusable) {
    a.gate_z = gate->z;
    a.gate_w = gate->weight;
    a.gate_eps = gate->eps;
    a.gate_gs = (int)gate->group_size;
    return launch_stages(p, a, stages, tune, stream);
  }
  st = launch_stages(p, a, stages, tune, stream);
  if (st != SSD_OK || tokens == 0) return st;
  NormArgs na = norm_args(&np);
  na.y = out;
  na.z = gate->z;
  na.w = gate->weight;
  na.out = out;
  if (launch_norm_fwd(na, static_cast<hipStream_t>(stream)) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}


// The backward's regions follow the forward's in its workspace.
struct BwdLayout {
  size_t Q, dS, dS16, dcb, rowpart, colpart, vxpart, interpart, ghpart, dla, dA_part, dD_part, dbias_part,
      ddot, cbt, dcb16, total;
};

void bwd_layout_of(const ssd_problem_t* p, const ssd_workspace_layout_t& w, BwdLayout* b) {
  const size_t mc = (size_t)w.max_chunks, H = p->nheads, L = p->chunk_size, N = p->dstate;
  const size_t PN = (size_t)p->headdim * p->dstate;
  size_t off = w.total_bytes;
  b->Q = off;          off = align_up(off + sizeof(float) * mc * H * PN);
  b->dS = off;         off = align_up(off + sizeof(float) * mc * H * PN);
  b->dS16 = off;       off = align_up(off + sizeof(uint16_t) * mc * H * PN);
  b->dcb = off;        off = align_up(off + sizeof(float) * mc * H * L * L);
  const size_t LT = L / 64, VX = 2 * ((N + 63) / 64);
  b->rowpart = off;    off = align_up(off + sizeof(float) * mc * H * 2 * LT * L);
  b->colpart = off;    off = align_up(off + sizeof(float) * mc * H * 2 * LT * L);
  b->vxpart = off;     off = align_up(off + sizeof(float) * mc * H * VX * L);
  b->interpart = off;  off = align_up(off + sizeof(float) * mc * H * VX * L);
  b->ghpart = off;     off = align_up(off + sizeof(float) * mc * H * (PN / 256));
  b->dla = off;        off = align_up(off + sizeof(float) * mc * H);
  b->dA_part = off;    off = align_up(off + sizeof(float) * mc * H);
  b->dD_part = off;    off = align_up(off + sizeof(float) * mc * H);
  b->dbias_part = off; off = align_up(off + sizeof(float) * mc * H);
  b->ddot = off;       off = align_up(off + sizeof(float) * mc * H * L);
  b->cbt = off;        off = align_up(off + sizeof(uint16_t) * mc * p->ngroups * L * L);
  b->dcb16 = off;      off = align_up(off + sizeof(uint16_t) * mc * p->ngroups * L * L);
  b->total = off;
}

ssd_status_t run_bwd(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias,
                     const float* A, const void* B, const void* C, const float* D,
                     const float* initial_states, const int32_t* cu_seqlens,
                     const int32_t* seq_idx, const void* dout, const float* dfinal, void* dx,
                     float* ddt, float* dA, void* dB, void* dC, float* dD, float* ddt_bias,
                     float* dinit, void* workspace, size_t workspace_bytes, void* stream,
                     bool recompute_forward) {
  ssd_status_t st = check_problem(p);
  if (st != SSD_OK) return st;
  const int64_t tokens = p->batch * p->seqlen;
  if (!dA) return SSD_ERR_INVALID_ARG;
  if (tokens > 0 && (!dout || !dx || !ddt || !dB || !dC)) return SSD_ERR_INVALID_ARG;
  ssd_workspace_layout_t w;
  layout_of(p, &w);
  BwdLayout bl;
  bwd_layout_of(p, w, &bl);
  if (!workspace || workspace_bytes < bl.total) return SSD_ERR_WORKSPACE;
  const ssd_tuning_t tune{0, 0, 0, 0, 0};
  FwdArgs a;
  st = fill_args(p, w, tune, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx,
                 nullptr, nullptr, workspace, &a);
  if (st != SSD_OK) return st;
  // the forward's stages 0-4: delta, running sums, CB, the entering states
  // (already in the workspace when an ssd_fwd call on these inputs left them)
  if (recompute_forward) {
    st = launch_stages(p, a, SSD_STAGE_ALL & ~(uint32_t)SSD_STAGE_CHUNK_SCAN, tune, stream);
    if (st != SSD_OK) return st;
  }
  char* base = static_cast<char*>(workspace);
  BwdArgs b;
  b.dy = dout; b.dfinal = dfinal; b.dx = dx; b.ddt = ddt; b.dA = dA; b.dB = dB; b.dC = dC;
  b.dD = dD; b.ddt_bias = ddt_bias; b.dinit = dinit;
  b.Q = reinterpret_cast<float*>(base + bl.Q);
  b.dS = reinterpret_cast<float*>(base + bl.dS);
  b.dS16 = base + bl.dS16;
  b.dcb = reinterpret_cast<float*>(base + bl.dcb);
  b.rowpart = reinterpret_cast<float*>(base + bl.rowpart);
  b.colpart = reinterpret_cast<float*>(base + bl.colpart);
  b.vxpart = reinterpret_cast<float*>(base + bl.vxpart);
  b.interpart = reinterpret_cast<float*>(base + bl.interpart);
  b.ghpart = reinterpret_cast<float*>(base + bl.ghpart);
  b.dla = reinterpret_cast<float*>(base + bl.dla);
  b.dA_part = reinterpret_cast<float*>(base + bl.dA_part);
  b.dD_part = reinterpret_cast<float*>(base + bl.dD_part);
  b.dbias_part = reinterpret_cast<float*>(base + bl.dbias_part);
  b.ddot = reinterpret_cast<float*>(base + bl.ddot);
  b.cbt = base + bl.cbt;
  b.dcb16 = base + bl.dcb16;
  const Kernels* k = find_kernels(p->dtype, p->headdim, p->dstate, p->chunk_size);
  if (k->backward(a, b, static_cast<hipStream_t>(stream)) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

// The allocation-free forward's workspace: a static device array, one copy
// per device the library runs on, kept until the process ends.  Host code
// never passes the array's name to a kernel (in host code it is only a
// stand-in): each device's address comes from hipGetSymbolAddress, taken
// once per device with that device current.
static_assert(SSD_NOALLOC_SCRATCH_BYTES % kAlign == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];

// This device's scratch address, or nullptr if the query fails.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot]() {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) slot.ptr = ptr;
  });
  return slot.ptr;
}

}  // namespace
}  // namespace ssd

extern "C" {

size_t ssd_fwd_workspace_size(const ssd_problem_t* p) {
  if (ssd::check_problem(p) != SSD_OK) return 0;
  ssd_workspace_layout_t w;
  ssd::layout_of(p, &w);
  return w.total_bytes;
}

ssd_status_t ssd_workspace_layout(const ssd_problem_t* p, ssd_workspace_layout_t* layout) {
  if (!layout) return SSD_ERR_INVALID_ARG;
  ssd_status_t st = ssd::check_problem(p);
  if (st != SSD_OK) return st;
  ssd::layout_of(p, layout);
  return SSD_OK;
}

int ssd_config_supported(int32_t dtype, int64_t headdim, int64_t dstate, int64_t chunk_size) {
  return ssd::find_kernels(dtype, headdim, dstate, chunk_size) != nullptr;
}

ssd_status_t ssd_fwd(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias,
                     const float* A, const void* B, const void* C, const float* D,
                     const float* initial_states, const int32_t* cu_seqlens,
                     const int32_t* seq_idx, void* out, float* final_states, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return ssd::run(p, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx, out,
                  final_states, workspace, workspace_bytes, SSD_STAGE_ALL, nullptr, stream);
}

ssd_status_t ssd_fwd_stages(const ssd_problem_t* p, const void* x, const float* dt,
                            const float* dt_bias, const float* A, const void* B, const void* C,
                            const float* D, const float* initial_states,
                            const int32_t* cu_seqlens, const int32_t* seq_idx, void* out,
                            float* final_states, void* workspace, size_t workspace_bytes,
                            uint32_t stages, void* stream) {
  return ssd::run(p, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx, out,
                  final_states, workspace, workspace_bytes, stages, nullptr, stream);
}

ssd_status_t ssd_fwd_tuned(const ssd_problem_t* p, const void* x, const float* dt,
                           const float* dt_bias, const float* A, const void* B, const void* C,
                           const float* D, const float* initial_states,
                           const int32_t* cu_seqlens, const int32_t* seq_idx, void* out,
                           float* final_states, void* workspace, size_t workspace_bytes,
                           uint32_t stages, const ssd_tuning_t* tuning, void* stream) {
  return ssd::run(p, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx, out,
                  final_states, workspace, workspace_bytes, stages, tuning, stream);
}

size_t ssd_bwd_workspace_size(const ssd_problem_t* p) {
  if (ssd::check_problem(p) != SSD_OK) return 0;
  ssd_workspace_layout_t w;
  ssd::layout_of(p, &w);
  ssd::BwdLayout b;
  ssd::bwd_layout_of(p, w, &b);
  return b.total;
}

ssd_status_t ssd_bwd(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias,
                     const float* A, const void* B, const void* C, const float* D,
                     const float* initial_states, const int32_t* cu_seqlens,
                     const int32_t* seq_idx, const void* dout, const float* dfinal_states,
                     void* dx, float* ddt, float* dA, void* dB, void* dC, float* dD,
                     float* ddt_bias, float* dinitial_states, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return ssd::run_bwd(p, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx, dout,
                      dfinal_states, dx, ddt, dA, dB, dC, dD, ddt_bias, dinitial_states,
                      workspace, workspace_bytes, stream, true);
}

ssd_status_t ssd_bwd_after_fwd(const ssd_problem_t* p, const void* x, const float* dt,
                               const float* dt_bias, const float* A, const void* B, const void* C,
                               const float* D, const float* initial_states,
                               const int32_t* cu_seqlens, const int32_t* seq_idx, const void* dout,
                               const float* dfinal_states, void* dx, float* ddt, float* dA,
                               void* dB, void* dC, float* dD, float* ddt_bias,
                               float* dinitial_states, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return ssd::run_bwd(p, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx, dout,
                      dfinal_states, dx, ddt, dA, dB, dC, dD, ddt_bias, dinitial_states,
                      workspace, workspace_bytes, stream, false);
}

ssd_status_t ssd_fwd_noalloc(const ssd_problem_t* p, const void* x, const float* dt,
                             const float* dt_bias, const float* A, const void* B, const void* C,
                             const float* D, const float* initial_states,
                             const int32_t* cu_seqlens, const int32_t* seq_idx, void* out,
                             float* final_states, void* stream) {
  ssd_status_t st = ssd::check_problem(p);
  if (st != SSD_OK) return st;
  ssd_workspace_layout_t w;
  ssd::layout_of(p, &w);
  if (w.total_bytes > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_TOO_LARGE;
  void* ws = ssd::scratch_address();
  if (!ws) return SSD_ERR_HIP;
  return ssd::run(p, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx, out,
                  final_states, ws, SSD_NOALLOC_SCRATCH_BYTES, SSD_STAGE_ALL, nullptr, stream);
}

ssd_status_t ssd_fwd_gated(const ssd_problem_t* p, const void* x, const float* dt,
                           const float* dt_bias, const float* A, const void* B, const void* C,
                           const float* D, const float* initial_states,
                           const int32_t* cu_seqlens, const int32_t* seq_idx,
                           const ssd_gate_t* gate, void* out, float* final_states,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!gate) return SSD_ERR_INVALID_ARG;
  return ssd::run(p, x, dt, dt_bias, A, B, C, D, initial_states, cu_seqlens, seq_idx, out,
                  final_states, workspace, workspace_bytes, SSD_STAGE_ALL, nullptr, stream, gate);
}

ssd_status_t ssd_fwd_choices(const ssd_problem_t* p, ssd_tuning_t* choices) {
  if (!choices) return SSD_ERR_INVALID_ARG;
  ssd_status_t st = ssd::check_problem(p);
  if (st != SSD_OK) return st;
  ssd_workspace_layout_t w;
  ssd::layout_of(p, &w);
  ssd::FwdArgs a{};
  a.batch = (int)p->batch;
  a.seqlen = (int)p->seqlen;
  a.H = (int)p->nheads;
  a.P = (int)p->headdim;
  a.N = (int)p->dstate;
  a.G = (int)p->ngroups;
  a.L = (int)p->chunk_size;
  a.nstates = (int)(p->nseq > 0 ? p->nseq : p->batch);
  a.max_chunks = (int)w.max_chunks;
  a.packed = p->nseq > 0;
  a.sp_blocks = ssd::auto_sp_blocks(p, w.max_chunks);
  const ssd::Kernels* k = ssd::find_kernels(p->dtype, p->headdim, p->dstate, p->chunk_size);
  const int scan = k->scan_choice(a);
  if (scan < 0 || ssd::device_cu_count() <= 0) return SSD_ERR_HIP;
  choices->scan_kernel = scan;
  choices->sp_vec = ssd::state_passing_vec(a);
  choices->front = k->front ? 1 : 0;
  choices->sp_blocks = a.sp_blocks;
  choices->fused = k->fused ? ssd::fused_choice(p, a, ssd_tuning_t{0, 0, 0, 0, 0}) : 1;
  return SSD_OK;
}

}  // extern "C"

namespace ssd {
namespace {

ssd_status_t check_norm(const ssd_norm_problem_t* p) {
  if (!p) return SSD_ERR_INVALID_ARG;
  if (p->tokens < 0 || p->channels < 1 || p->group_size < 1) return SSD_ERR_INVALID_ARG;
  if (p->dtype != SSD_F32 && p->dtype != SSD_BF16) return SSD_ERR_INVALID_ARG;
  if (p->channels % p->group_size != 0) return SSD_ERR_INVALID_ARG;
  if (!(p->eps >= 0.f) || isinf(p->eps)) return SSD_ERR_INVALID_ARG;
  const int64_t V = p->dtype == SSD_BF16 ? 8 : 4;
  if (p->group_size % V != 0) return SSD_ERR_UNSUPPORTED;
  const int64_t nv = p->group_size / V;
  const bool pow2 = (nv & (nv - 1)) == 0;
  if (!((nv <= 64 && pow2) || nv % 64 == 0)) return SSD_ERR_UNSUPPORTED;
  if (p->channels > norm_max_channels(p->dtype)) return SSD_ERR_UNSUPPORTED;
  if (p->tokens * p->channels > (int64_t)1 << 40) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

NormArgs norm_args(const ssd_norm_problem_t* p) {
  NormArgs a{};
  a.rows = p->tokens;
  a.C = (int)p->channels;
  a.GS = (int)p->group_size;
  a.eps = p->eps;
  a.bf16 = p->dtype == SSD_BF16;
  return a;
}

}  // namespace
}  // namespace ssd

extern "C" {

ssd_status_t ssd_gated_norm_fwd(const ssd_norm_problem_t* p, const void* y, const void* z,
                                const float* w, void* out, float* rstd, void* stream) {
  ssd_status_t st = ssd::check_norm(p);
  if (st != SSD_OK) return st;
  if (p->tokens > 0 && (!y || !z || !w || !out)) return SSD_ERR_INVALID_ARG;
  ssd::NormArgs a = ssd::norm_args(p);
  a.y = y; a.z = z; a.w = w; a.out = out; a.rstd = rstd;
  if (ssd::launch_norm_fwd(a, static_cast<hipStream_t>(stream)) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

size_t ssd_gated_norm_bwd_workspace_size(const ssd_norm_problem_t* p) {
  if (ssd::check_norm(p) != SSD_OK) return 0;
  return ssd::align_up(sizeof(float) * (size_t)ssd::norm_workspace_floats(p->channels));
}

ssd_status_t ssd_gated_norm_bwd(const ssd_norm_problem_t* p, const void* y, const void* z,
                                const float* w, const void* dout, void* dy, void* dz, float* dw,
                                void* workspace, size_t workspace_bytes, void* stream) {
  ssd_status_t st = ssd::check_norm(p);
  if (st != SSD_OK) return st;
  if (!w || !dw) return SSD_ERR_INVALID_ARG;
  if (p->tokens > 0 && (!y || !z || !dout || !dy || !dz)) return SSD_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % ssd::kAlign) != 0 ||
      workspace_bytes < ssd_gated_norm_bwd_workspace_size(p))
    return SSD_ERR_WORKSPACE;
  ssd::NormArgs a = ssd::norm_args(p);
  a.y = y; a.z = z; a.w = w; a.dout = dout; a.dy = dy; a.dz = dz; a.dw = dw;
  a.dw_part = static_cast<float*>(workspace);
  if (ssd::launch_norm_bwd(a, static_cast<hipStream_t>(stream)) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

const char* ssd_status_string(ssd_status_t s) {
  switch (s) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported (dtype, headdim, dstate, chunk_size) or size";
    case SSD_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SSD_ERR_HIP: return "HIP launch failed";
    case SSD_ERR_TOO_LARGE:
      return "problem needs more workspace than ssd_fwd_noalloc's static scratch buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
