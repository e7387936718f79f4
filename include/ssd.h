/*
 * ssd.h: C ABI of the Mamba-2 SSD (state-space duality) chunked-scan
 * forward on one AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  A Mamba-2 layer updates a fixed-size hidden
 * state per head with every token, and the chunkwise form processes it
 * chunk by chunk (aiproviderindex.com, item on CUDA Tile Mamba-2 kernels,
 * "Mamba-2 offers a different scaling path").  The pages do not write the
 * update out; this library reads it as the plain Mamba-2 selective
 * state-space update.  For each sequence s, head h (B/C group g =
 * h / (nheads / ngroups)) and token t:
 *
 *   delta_t  = clamp(softplus(dt[t,h] + dt_bias[h]), dt_min, dt_max)
 *   h_t      = exp(delta_t * A[h]) * h_{t-1} + delta_t * x[t,h,:] (outer) B[t,g,:]
 *   y[t,h,:] = h_t . C[t,g,:]  +  D[h] * x[t,h,:]        (h_t is P x N)
 *   h_{-1}   = initial_states[s,h] (or 0);  final_states[s,h] = h after the
 *              sequence's last token.
 *
 * It does so with the chunked scan whose forward stages the pages name
 * (aiproviderindex.com, "Mamba-2 offers a different scaling path":
 * chunk_cumsum, state propagation and output construction; clova.ai, table
 * "Share of compute time by kernel": _chunk_state_fwd, _state_passing_fwd,
 * _chunk_scan_fwd), as hand-written HIP kernels:
 *
 *   stage 0  plan            logical chunk table (chunks never straddle a
 *                            sequence)
 *   stage 1  chunk_cumsum    delta and its chunk-local running sum of delta*A
 *   stage 2  bmm_chunk       C B^T inside each chunk (lower triangle)
 *   stage 3  chunk_state     per-chunk state from a zero start
 *   stage 4  state_passing   chain over chunks: states entering each chunk
 *                            and the final states; one sequential chain per
 *                            sequence, or, for problems with few state
 *                            elements, blocks of chunks composed as an
 *                            associative scan (clova.ai, "Stage 3. Logic and
 *                            heuristic refinement")
 *   stage 5  chunk_scan      decay-masked (C B^T) x  +  exp(cumsum) C . state
 *                            +  D x, accumulated in fp32
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates nothing and keeps no state between calls.  Inputs are
 *     only read; `out`, `final_states` and `workspace` are written.  No
 *     pointer may alias another.
 *   - Layouts are contiguous row-major:
 *       x, out  [batch, seqlen, nheads, headdim]        dtype
 *       dt      [batch, seqlen, nheads]                 fp32 (before softplus)
 *       dt_bias [nheads] fp32 (nullable: 0);  A [nheads] fp32
 *       B, C    [batch, seqlen, ngroups, dstate]        dtype
 *       D       [nheads] fp32 (nullable: no skip term)
 *       initial_states, final_states [nstates, nheads, headdim, dstate] fp32,
 *               nstates = nseq for a packed batch, else batch (nullable)
 *       cu_seqlens [nseq + 1] int32, seq_idx [seqlen] int32 (packed batch)
 *   - `stream` is a hipStream_t (NULL: the null stream).  Work is enqueued
 *     asynchronously; nothing synchronises with the host and nothing is
 *     allocated, so a call can be captured in a HIP graph.  Kernel faults
 *     surface at the caller's next synchronisation.
 *   - Errors: argument checks run on the host before anything is enqueued; a
 *     non-OK status means no work was enqueued, except SSD_ERR_HIP (a launch
 *     failed; earlier stages of that call may have been enqueued).
 *   - Results are deterministic: no atomics, fixed reduction orders.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1,  /* a size, pointer or combination is invalid   */
  SSD_ERR_UNSUPPORTED = 2,  /* valid, but (dtype, headdim, dstate, chunk)  */
                            /* has no compiled kernel                      */
  SSD_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than required     */
  SSD_ERR_HIP = 4,          /* a HIP launch or device query failed         */
  SSD_ERR_TOO_LARGE = 5     /* ssd_fwd_noalloc: the problem's workspace is */
                            /* larger than SSD_NOALLOC_SCRATCH_BYTES       */
} ssd_status_t;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype_t;

/* Stage bits for ssd_fwd_stages. */
enum {
  SSD_STAGE_PLAN = 1u << 0,
  SSD_STAGE_CUMSUM = 1u << 1,
  SSD_STAGE_BMM = 1u << 2,
  SSD_STAGE_CHUNK_STATE = 1u << 3,
  SSD_STAGE_STATE_PASSING = 1u << 4,
  SSD_STAGE_CHUNK_SCAN = 1u << 5,
  SSD_STAGE_ALL = 0x3Fu
};

typedef struct {
  int64_t batch;       /* rows; must be 1 for a packed batch               */
  int64_t seqlen;      /* tokens per row (packed batch: total tokens); >= 0 */
  int64_t nheads;      /* H >= 1                                            */
  int64_t headdim;     /* P                                                 */
  int64_t dstate;      /* N                                                 */
  int64_t ngroups;     /* G >= 1, H % G == 0                                */
  int64_t chunk_size;  /* L                                                 */
  int64_t nseq;        /* 0: rows are the sequences; > 0: packed batch of   */
                       /* nseq sequences given by cu_seqlens or seq_idx     */
  int32_t dtype;       /* ssd_dtype_t of x, B, C and out                    */
  float dt_min;        /* clamp of delta after softplus; use 0 and +inf for */
  float dt_max;        /* no clamp                                          */
} ssd_problem_t;

/* Byte offsets into the workspace of the stage intermediates (all 256-byte
 * aligned) and the bound on the number of logical chunks they are sized for.
 *   chunk_table  int32 [max_chunks][4]: first token on the flattened token
 *                axis, valid length (<= L), sequence, index within sequence
 *   seq_chunks   int32 [nstates + 1]: first logical chunk of each sequence;
 *                the last entry is the number of chunks in use
 *   delta, dA_cumsum  fp32 [max_chunks][nheads][L]
 *   cb           dtype [max_chunks][ngroups][L][L] (entries with s <= l of
 *                the valid rows hold C B^T, fp32 accumulation stored in the
 *                dtype of x; entries with s > l in the same 64-token block
 *                as l are 0; the rest are not written)
 *   chunk_states fp32 [max_chunks][nheads][headdim][dstate]
 *   states_in    dtype [max_chunks][nheads][headdim][dstate]: state entering
 *                each chunk
 *   block_states, block_logdecay  fp32 [nstates][sp_blocks][nheads][headdim *
 *                dstate] and [nstates][sp_blocks][nheads]: the blocked
 *                state_passing's per-block end states and log decays
 *                (present, with sp_blocks = 16, only when nstates * nheads *
 *                headdim * dstate < 2^18; else sp_blocks = 1 and both are
 *                empty)
 *   sync         int32 counters of the fused forward (ssd_tuning_t.fused):
 *                max_chunks * nheads + 1                                   */
typedef struct {
  int64_t max_chunks;
  size_t chunk_table, seq_chunks, delta, dA_cumsum, cb, chunk_states, states_in;
  size_t block_states, block_logdecay, sync;
  int64_t sp_blocks;
  size_t total_bytes;
} ssd_workspace_layout_t;

/* Workspace bytes ssd_fwd needs for this problem (0 if the problem is
 * invalid or unsupported): the intermediates the stages above hand to one
 * another, stored in the layout their consumer reads (aiproviderindex.com,
 * "Memory layout is part of the algorithm").  Library bookkeeping: no
 * passage of the pages defines it. */
size_t ssd_fwd_workspace_size(const ssd_problem_t* p);

/* Fills *layout for this problem.  SSD_ERR_INVALID_ARG / SSD_ERR_UNSUPPORTED
 * as for ssd_fwd. */
ssd_status_t ssd_workspace_layout(const ssd_problem_t* p, ssd_workspace_layout_t* layout);

/* 1 if (dtype, headdim, dstate, chunk_size) has compiled kernels, else 0
 * (library bookkeeping, not from the pages). */
int ssd_config_supported(int32_t dtype, int64_t headdim, int64_t dstate, int64_t chunk_size);

/*
 * The whole SSD forward: stages 0..5 above, enqueued on `stream`.
 *
 * x, dt, A, B, C, out are required (they may be NULL only when
 * batch * seqlen == 0).  dt_bias, D, initial_states, final_states are
 * optional.  A packed batch (p->nseq > 0, p->batch == 1) takes exactly one
 * of cu_seqlens (non-decreasing, from 0 to seqlen) or seq_idx (the sequence
 * id of each token, non-decreasing, in [0, nseq)); with seqlen == 0 it may
 * pass neither (every sequence is then empty).  An unpacked problem takes
 * neither.  Malformed packing arrays give unspecified outputs but never an
 * access outside the given buffers.  Tokens that belong to no sequence keep
 * whatever `out` held.
 *
 * The workspace (ssd_fwd_workspace_size bytes, 256-byte aligned) holds the
 * intermediates laid out as ssd_workspace_layout reports; its prior contents
 * do not matter.
 */
ssd_status_t ssd_fwd(const ssd_problem_t* p,
                     const void* x, const float* dt, const float* dt_bias,
                     const float* A, const void* B, const void* C, const float* D,
                     const float* initial_states,
                     const int32_t* cu_seqlens, const int32_t* seq_idx,
                     void* out, float* final_states,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * As ssd_fwd, but enqueues only the stages whose SSD_STAGE_* bit is set in
 * `stages`, in stage order, reading the intermediates earlier stages left in
 * the workspace.  Used to time and test stages one by one.
 */
ssd_status_t ssd_fwd_stages(const ssd_problem_t* p,
                            const void* x, const float* dt, const float* dt_bias,
                            const float* A, const void* B, const void* C, const float* D,
                            const float* initial_states,
                            const int32_t* cu_seqlens, const int32_t* seq_idx,
                            void* out, float* final_states,
                            void* workspace, size_t workspace_bytes,
                            uint32_t stages, void* stream);

/*
 * Kernel choices a caller may pin for one call.  0 in a field keeps the
 * library's own choice for the shape.  An offline tuner times the choices
 * per problem shape and records the fastest in a config file; the Python
 * binding reads that file and falls back to 0 (the built-in choice) for
 * shapes it does not list.  None of the choices changes what is computed;
 * they move rounding only where noted.
 *   scan_kernel  chunk_scan for bf16: 1 = one workgroup per (chunk, head)
 *                tile (its rescaled path rounds differently from the
 *                masked one), 2 = the persistent walk over tiles, 3 = one
 *                workgroup of four waves per tile (bitwise the same results
 *                as 1; with 256-token chunks each wave owns four 16-row
 *                groups instead of two, so three workgroups fit on a CU).
 *                Must be 0 for fp32.
 *   sp_vec       consecutive state elements per state_passing thread: 1, 2
 *                or 4 (identical results).
 *   front        bf16 stages 1-3: 1 = one fused launch, 2 = one launch per
 *                stage (identical results).  Must be 0 for fp32.
 *   sp_blocks    state_passing: 1 = one sequential chain per sequence; 2, 4,
 *                8 or 16 = that many blocks per sequence, scanned in two
 *                launches (rounds differently: the blocks' maps are
 *                composed in another order).  Above 1 only when the
 *                workspace layout's sp_blocks is 16.
 *   fused        bf16 with 128- or 256-token chunks: 1 = front,
 *                state_passing and chunk_scan as separate launches, 2 =
 *                the front's launch, then state_passing and chunk_scan in
 *                one persistent launch in which the scan tiles of a chunk
 *                start once the state chain has passed it; bitwise the same
 *                results as 1 with the one-chain state passing and the same
 *                scan tile (scan_kernel 1 or 3, or the library's choice).
 *                2 cannot be combined with sp_blocks > 1, front 2, sp_vec
 *                1 or 2, or scan_kernel 2; it applies when a call runs all
 *                of stages 1-5.
 * A field outside its range, or a choice the dtype does not have, is
 * rejected with SSD_ERR_INVALID_ARG before anything is enqueued.
 */
typedef struct {
  int32_t scan_kernel;
  int32_t sp_vec;
  int32_t front;
  int32_t sp_blocks;
  int32_t fused;
} ssd_tuning_t;

/*
 * As ssd_fwd_stages, with kernel choices pinned by `tuning` (NULL: all 0).
 * Meant for tuners and for callers replaying a tuned configuration.
 */
ssd_status_t ssd_fwd_tuned(const ssd_problem_t* p,
                           const void* x, const float* dt, const float* dt_bias,
                           const float* A, const void* B, const void* C, const float* D,
                           const float* initial_states,
                           const int32_t* cu_seqlens, const int32_t* seq_idx,
                           void* out, float* final_states,
                           void* workspace, size_t workspace_bytes,
                           uint32_t stages, const ssd_tuning_t* tuning, void* stream);

/*
 * The kernel choices ssd_fwd / ssd_fwd_stages (and ssd_fwd_tuned for its
 * fields left 0) make for this problem on the calling thread's current HIP
 * device, in the fields of ssd_tuning_t: scan_kernel 1-3 (0 for fp32),
 * sp_vec 1/2/4, front 1 (bf16) or 0 (fp32), sp_blocks 1-16, fused 1 or 2.  They depend on
 * the shape and on the device's compute-unit count and occupancy only, never
 * on earlier calls, so a tuner or test can pin exactly what the default
 * path runs (clova.ai page, section "Stage 3. Logic and heuristic
 * refinement": launch parameters tied to the GPU's unit count belong with
 * the device, not in the code).  Host only; enqueues nothing.  Errors:
 * SSD_ERR_INVALID_ARG / SSD_ERR_UNSUPPORTED as for ssd_fwd, SSD_ERR_HIP if
 * a device query fails (e.g. no device).
 */
ssd_status_t ssd_fwd_choices(const ssd_problem_t* p, ssd_tuning_t* choices);

/*
 * The backward: gradients of loss = sum(out * dout) + sum(final_states *
 * dfinal_states) with respect to every input of ssd_fwd (the layer's backward
 * kernels are listed next to the forward ones on the clova.ai page, table
 * "Share of compute time by kernel").  Same problem, inputs and conventions
 * as ssd_fwd; the forward's stages 0-4 are recomputed inside, so no forward
 * call needs to precede it.
 *
 *   dout           [batch, seqlen, nheads, headdim] dtype (required)
 *   dfinal_states  [nstates, nheads, headdim, dstate] fp32 (nullable: 0)
 *   dx             like x, dtype          ddt  like dt, fp32
 *   dB, dC         like B and C, dtype    dA   [nheads] fp32
 *   dD, ddt_bias   [nheads] fp32 (nullable: not computed)
 *   dinitial_states [nstates, nheads, headdim, dstate] fp32 (nullable)
 * dD and ddt_bias are the gradients at the given D and dt_bias (also when
 * those are NULL, i.e. 0); dinitial_states likewise for a NULL initial
 * state.  Gradients accumulate in fp32; dx, dB, dC are rounded once to the
 * dtype.  Entries of tokens that belong to no sequence are not written.
 * The workspace is ssd_bwd_workspace_size bytes (256-byte aligned); it
 * begins with the forward's layout (ssd_workspace_layout) followed by the
 * backward's own fp32 buffers.  Errors as for ssd_fwd.
 */
size_t ssd_bwd_workspace_size(const ssd_problem_t* p);

ssd_status_t ssd_bwd(const ssd_problem_t* p,
                     const void* x, const float* dt, const float* dt_bias,
                     const float* A, const void* B, const void* C, const float* D,
                     const float* initial_states,
                     const int32_t* cu_seqlens, const int32_t* seq_idx,
                     const void* dout, const float* dfinal_states,
                     void* dx, float* ddt, float* dA, void* dB, void* dC,
                     float* dD, float* ddt_bias, float* dinitial_states,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * As ssd_bwd, without recomputing the forward's stages 0-4: the workspace
 * (ssd_bwd_workspace_size bytes) must hold, unchanged, what a completed
 * ssd_fwd / ssd_fwd_stages / ssd_fwd_tuned call that ran stages 0-4 on the
 * same problem and the same inputs wrote into its leading
 * ssd_workspace_layout part (the steps, running sums, CB and entering
 * states), as in training, where the backward follows its forward.  The
 * gradients are those of that forward's intermediates; with the forward's
 * default kernel choices they equal ssd_bwd's bit for bit.  The library
 * cannot check that the workspace holds them: anything else in it gives
 * wrong gradients without an error.  Arguments and errors as for ssd_bwd.
 */
ssd_status_t ssd_bwd_after_fwd(const ssd_problem_t* p,
                               const void* x, const float* dt, const float* dt_bias,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* initial_states,
                               const int32_t* cu_seqlens, const int32_t* seq_idx,
                               const void* dout, const float* dfinal_states,
                               void* dx, float* ddt, float* dA, void* dB, void* dC,
                               float* dD, float* ddt_bias, float* dinitial_states,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The gated RMS norm that follows the SSD in a Mamba-2 layer, and its
 * backward.  The pages name the layer's norm only through its backward
 * kernel (clova.ai page, table "Share of compute time by kernel":
 * _layer_norm_bwd, the largest share, memory-bound; section "How we fixed
 * it"); the norm read here is the Mamba-2 gated RMS norm.  For every row t
 * (token) and every group of group_size consecutive channels:
 *
 *   g_c   = y[t,c] * silu(z[t,c]),        silu(v) = v / (1 + exp(-v))
 *   r     = 1 / sqrt(mean_{c in group} g_c^2 + eps)
 *   out[t,c] = g_c * r * w[c]
 *
 * y is the SSD output flattened to rows of channels = nheads * headdim
 * ([tokens][channels], the layout of ssd_fwd's out), z the gate of the same
 * layout and dtype, w [channels] fp32.  Accumulation in fp32, one rounding of
 * each output to the dtype.
 *   - group_size divides channels; group_size / (16 / dtype size) is a
 *     power of two up to 64 or a multiple of 64 (else SSD_ERR_UNSUPPORTED);
 *     channels <= 8192 (bf16) or 4096 (fp32); eps >= 0.
 *   - ssd_gated_norm_fwd: out (may be y itself: each element is read before
 *     it is written, by the same thread); rstd [tokens][channels /
 *     group_size] fp32 receives r (nullable).
 *   - ssd_gated_norm_bwd: the gradients of sum(out * dout): dy, dz like y,
 *     dw [channels] fp32 (required); the workspace is
 *     ssd_gated_norm_bwd_workspace_size bytes, 256-byte aligned.  No atomics:
 *     deterministic.
 * Device pointers, asynchronous on `stream`; errors as for ssd_fwd.
 */
typedef struct {
  int64_t tokens;      /* rows                                           */
  int64_t channels;    /* channels per row                               */
  int64_t group_size;  /* consecutive channels normalised together       */
  int32_t dtype;       /* ssd_dtype_t of y, z, out, dout, dy, dz         */
  float eps;
} ssd_norm_problem_t;

ssd_status_t ssd_gated_norm_fwd(const ssd_norm_problem_t* p, const void* y, const void* z,
                                const float* w, void* out, float* rstd, void* stream);

size_t ssd_gated_norm_bwd_workspace_size(const ssd_norm_problem_t* p);

ssd_status_t ssd_gated_norm_bwd(const ssd_norm_problem_t* p, const void* y, const void* z,
                                const float* w, const void* dout, void* dy, void* dz, float* dw,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward followed by the gated RMS norm of its output (the same norm as
 * ssd_gated_norm_fwd, over rows of nheads * headdim channels): `out`
 * receives rmsnorm(y * silu(z)) * weight, not y.  Where the norm's groups lie
 * inside a head (group_size divides headdim; bf16) and chunk_scan runs a
 * one-tile-per-workgroup kernel (the library's choice for most shapes), the
 * norm is applied in chunk_scan's store and y never reaches memory;
 * otherwise the forward writes y into `out` and the norm runs over it in
 * place.  Either way the result equals ssd_fwd followed by
 * ssd_gated_norm_fwd bit for bit.  final_states and the workspace are as
 * for ssd_fwd.
 */
typedef struct {
  const void* z;        /* gate, layout and dtype of x and out           */
  const float* weight;  /* [nheads * headdim]                            */
  float eps;
  int64_t group_size;   /* channels normalised together (see ssd_norm_problem_t) */
} ssd_gate_t;

ssd_status_t ssd_fwd_gated(const ssd_problem_t* p,
                           const void* x, const float* dt, const float* dt_bias,
                           const float* A, const void* B, const void* C, const float* D,
                           const float* initial_states,
                           const int32_t* cu_seqlens, const int32_t* seq_idx,
                           const ssd_gate_t* gate, void* out, float* final_states,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ssd_fwd
 * without a workspace argument.  The workspace is a static device array of
 * SSD_NOALLOC_SCRATCH_BYTES inside the library, one per device, allocated
 * when the library's code is loaded on that device and held until the
 * process ends; this call allocates nothing and calls no allocating routine.
 * The caller still passes every input and output, as for ssd_fwd.
 *   - Problems whose ssd_fwd_workspace_size exceeds SSD_NOALLOC_SCRATCH_BYTES
 *     are rejected with SSD_ERR_TOO_LARGE before anything is enqueued.
 *   - Every call on one device shares that device's array, whose contents
 *     persist between calls (nothing in it needs to start at zero).  Calls
 *     that overlap on one device, on different streams or from different
 *     threads, race on it and give wrong results: serialise them (e.g. on
 *     one stream).
 * Results are bit for bit those of ssd_fwd on the same problem and inputs.
 * Other errors as for ssd_fwd.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

ssd_status_t ssd_fwd_noalloc(const ssd_problem_t* p,
                             const void* x, const float* dt, const float* dt_bias,
                             const float* A, const void* B, const void* C, const float* D,
                             const float* initial_states,
                             const int32_t* cu_seqlens, const int32_t* seq_idx,
                             void* out, float* final_states, void* stream);

/* Static description of a status code (library bookkeeping, not from the
 * pages). */
const char* ssd_status_string(ssd_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
