// Host-side launch interface of the SSD forward stages (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_common.h"

namespace ssd {

// Everything one forward call needs: shapes, caller buffers, workspace.
struct FwdArgs {
  int batch, seqlen, H, P, N, G, L;
  int nstates;      // sequences: rows, or packed sequences
  int max_chunks;   // logical chunks the workspace is sized for
  int nc_row;       // chunks per row (rows mode)
  bool packed;
  float dt_min, dt_max;
  int scan_kernel;  // 0: by shape, 1: one workgroup per tile, 2: persistent (bf16)
  int sp_vec;       // 0: by shape, else state elements per state_passing thread
  int sp_blocks;    // state_passing: 1 = one chain per sequence, KB > 1 = KB blocks
  int fused;        // 1: front, state_passing, chunk_scan as separate launches; 2: one launch

  const void* x;
  const float* dt;
  const float* dt_bias;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const float* init;
  const int32_t* cu_seqlens;
  const int32_t* seq_idx;
  void* out;
  float* final_states;

  int4* table;
  int* seq_chunks;
  float* delta;
  float* dAcs;
  void* cb;             // dtype of x
  float* chunk_states;
  void* states_in;
  float* block_states;     // [nstates][KB][H][P*N] when sp_blocks > 1
  float* block_logdecay;   // [nstates][KB][H]
  // gated RMS norm fused into chunk_scan's store (gate_z nullptr: none)
  const void* gate_z;
  const float* gate_w;
  float gate_eps;
  int gate_gs;
  int* sync;               // counters of the fused forward
  int64_t zero_ints;       // the front also clears this many ints at `sync` (0: none)

  __host__ __device__ ChunkMap cmap() const {
    ChunkMap m;
    m.table = packed ? table : nullptr;
    m.seq_chunks = packed ? seq_chunks : nullptr;
    m.seqlen = seqlen;
    m.nc_row = nc_row;
    m.L = L;
    return m;
  }
};

// The backward's own buffers (gradients and its workspace regions).
struct BwdArgs {
  const void* dy;           // dtype of x, like the output
  const float* dfinal;      // nullable
  void* dx;                 // dtype of x
  float* ddt;
  float* dA;
  void* dB;                 // dtype of x
  void* dC;                 // dtype of x
  float* dD;                // nullable
  float* ddt_bias;          // nullable
  float* dinit;             // nullable
  float* Q;                 // [max_chunks][H][P*N]
  float* dS;                // [max_chunks][H][P*N] (fp32 inputs only)
  void* dS16;               // [max_chunks][H][P*N] bf16: dS rounded once (bf16 inputs)
  float* dcb;               // [max_chunks][H][L][L] floats; holds [max_chunks][G][HB][L][L]: sums
                            // of delta_s exp(a_l - a_s) dy_l . x_s (s <= l) over head blocks
  float* rowpart;           // [max_chunks][H][L/64][halves][L] (halves: 2 for bf16, 1 for fp32)
  float* colpart;           // [max_chunks][H][L/64][halves][L]
  float* vxpart;            // [max_chunks][H][2 ceil(N/64)][L]
  float* interpart;         // [max_chunks][H][2 ceil(N/64)][L]
  float* ghpart;            // [max_chunks][H][P*N / 256]: <dS_j, H_j> in pieces
  float* dla;               // [max_chunks][H]: the chunk's log-decay a_last (0 if empty)
  float* dA_part;           // [max_chunks][H]
  float* dD_part;           // [max_chunks][H]
  float* dbias_part;        // [max_chunks][H]
  float* ddot;              // [max_chunks][H][L]: dy_t . x_t per token
  void* cbt;                // [max_chunks][G][L][L] bf16 (bf16 inputs): CB transposed,
                            // cbt[s][l] = CB[l][s] for s <= l < len, else 0, in the 64 x 64
                            // tiles with l-tile >= s-tile and l-tile inside the chunk
  void* dcb16;              // [max_chunks][G][L][L] bf16 (bf16 inputs): the group's summed dCB,
                            // rounded once (rows past the chunk and tiles above the diagonal
                            // are not written)
};

// Devices whose per-device launch parameters the library caches.
constexpr int kMaxDevices = 64;

// Compute units of the calling thread's current HIP device, queried once per
// device and cached (0 if the query fails).  Launch heuristics size their
// grids and thresholds from it instead of assuming a CU count.
int device_cu_count();

// The library's own chunk_scan kernel for this problem on the current device
// (1, 2 or 3 as in ssd_tuning_t.scan_kernel; 0 for fp32, -1 if a device
// query fails).
template <typename T, int P, int N, int L>
int chunk_scan_choice(const FwdArgs& a);
// The library's own state_passing vector width (1, 2 or 4) for this problem.
int state_passing_vec(const FwdArgs& a);

// The gated RMS norm after the SSD (forward and backward).
struct NormArgs {
  int64_t rows;
  int C, GS;            // channels per row, channels per group
  float eps;
  bool bf16;            // dtype of y, z, out, dout, dy, dz
  const void* y;
  const void* z;
  const float* w;
  void* out;
  float* rstd;          // nullable
  const void* dout;
  void* dy;
  void* dz;
  float* dw;
  float* dw_part;       // norm_workspace_floats(C) floats
};
// Most channels per row the norm kernels take for a dtype.
int norm_max_channels(int32_t dtype);
// Floats of the backward's workspace (partial rows of dw and their first
// sums) for rows of C channels: a bound that does not depend on the device.
int64_t norm_workspace_floats(int64_t C);
hipError_t launch_norm_fwd(const NormArgs& a, hipStream_t s);
hipError_t launch_norm_bwd(const NormArgs& a, hipStream_t s);

// Stage 0: logical chunk table of a packed batch.
hipError_t launch_plan(const FwdArgs& a, hipStream_t s);
// Stage 1: delta and its chunk-local cumulative sum times A.
hipError_t launch_chunk_cumsum(const FwdArgs& a, hipStream_t s);
// Stage 2: C B^T per chunk and group.
template <typename T, int N, int L>
hipError_t launch_bmm_chunk(const FwdArgs& a, hipStream_t s);
// Stage 3: per-chunk states.
template <typename T, int P, int N, int L>
hipError_t launch_chunk_state(const FwdArgs& a, hipStream_t s);
// Stages 1-3 of the bf16 path in one launch (bmm tiles as extra workgroups,
// chunk_cumsum inside the chunk_state workgroups).
template <typename T, int P, int N, int L>
hipError_t launch_front(const FwdArgs& a, hipStream_t s);
// Stage 4: inter-chunk chain.
template <typename T>
hipError_t launch_state_passing(const FwdArgs& a, hipStream_t s);
// Stage 5: outputs.
template <typename T, int P, int N, int L>
hipError_t launch_chunk_scan(const FwdArgs& a, hipStream_t s);
// Stages 1-5 of the bf16 forward as the front's launch (which clears the
// counters at a.sync, fused_sync_bytes long) and one persistent launch of
// state_passing and chunk_scan; scan_choice as chunk_scan_choice.
size_t fused_sync_bytes(int nstates, int H, int G, int max_chunks);
template <typename T, int P, int N, int L>
bool fused_supported();
template <typename T, int P, int N, int L>
hipError_t launch_fused(const FwdArgs& a, int scan_choice, hipStream_t s);
// The backward, after stages 0-4 of the forward have filled `a`'s workspace.
template <typename T, int P, int N, int L>
hipError_t launch_backward(const FwdArgs& a, const BwdArgs& b, hipStream_t s);

}  // namespace ssd

// (dtype, headdim, dstate, chunk_size) combinations with compiled kernels.
#define SSD_FOR_EACH_CONFIG(X) \
  X(float, 32, 16, 64)         \
  X(float, 64, 128, 64)        \
  X(float, 64, 128, 256)       \
  X(bf16, 32, 32, 64)          \
  X(bf16, 64, 128, 64)         \
  X(bf16, 64, 128, 128)        \
  X(bf16, 64, 128, 256)
