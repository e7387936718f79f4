// Internal device-side definitions shared by the SSD forward kernels
// (gfx950 / CDNA4 only: 64-wide wavefronts, MFMA 16x16 tiles, LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// threadIdx.x through an empty asm statement: values computed from it cannot
// be hoisted out of an enclosing loop.  A persistent kernel that runs a tile
// body per loop iteration would otherwise keep every lane offset of every
// body in registers for the whole loop.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// threadIdx.x for a tile body of TH threads: laundered when the body runs
// inside a persistent loop (OPQ), with its range restated so the compiler
// keeps the code it makes for a known thread range; plain otherwise.
template <bool OPQ, int TH>
__device__ __forceinline__ int body_tid() {
  if constexpr (OPQ) {
    const int t = opaque_tid();
    __builtin_assume(t >= 0 && t < TH);
    return t;
  } else {
    return threadIdx.x;
  }
}

// Index of the calling wave within its workgroup, as a wave-uniform (scalar)
// value: branches and addresses derived from it stay on the scalar unit.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

// ---------------------------------------------------------------------------
// Logical chunks.  A chunk never straddles a sequence: sequence s owns
// ceil(len_s / L) chunks that start at its first token, so only its last
// chunk can be short.  For unpacked rows the map is arithmetic (row r owns
// chunks [r*nc_row, (r+1)*nc_row)); for a packed batch it is the table the
// plan kernels write into the workspace.
// ---------------------------------------------------------------------------
struct ChunkDesc {
  int start;  // first token on the flattened (batch * seqlen) token axis
  int len;    // valid tokens, 0 for an unused table slot
  int seq;    // sequence (row, or packed sequence)
  int idx;    // index of the chunk within its sequence
};

struct ChunkMap {
  const int4* table;       // packed batch: [max_chunks]; nullptr for rows
  const int* seq_chunks;   // packed batch: [nstates + 1]
  int seqlen;              // tokens per row (rows mode)
  int nc_row;              // chunks per row (rows mode)
  int L;

  __device__ __forceinline__ ChunkDesc desc(int j) const {
    ChunkDesc d;
    if (table) {
      int4 v = table[j];
      d.start = v.x; d.len = v.y; d.seq = v.z; d.idx = v.w;
    } else {
      int r = j / nc_row, c = j - r * nc_row;
      d.start = r * seqlen + c * L;
      d.len = min(L, seqlen - c * L);
      d.seq = r;
      d.idx = c;
    }
    return d;
  }
  // [first, last) logical chunks of sequence s
  __device__ __forceinline__ int2 seq_range(int s) const {
    if (table) return make_int2(seq_chunks[s], seq_chunks[s + 1]);
    return make_int2(s * nc_row, (s + 1) * nc_row);
  }
};

// ---------------------------------------------------------------------------
// Element types.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// exp on the fp32 path keeps the accurate library routine; the bf16 path uses
// the hardware exp2 (its relative error is far below bf16's 2^-9).
template <typename T> __device__ __forceinline__ float fexp(float v);
template <> __device__ __forceinline__ float fexp<float>(float v) { return expf(v); }
template <> __device__ __forceinline__ float fexp<bf16>(float v) { return __expf(v); }

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles, fp32 accumulation.
//   A operand: lane i holds A[i % 16][kb + KPL*(i/16) + e], e < KPL
//   B operand: lane i holds B[kb + KPL*(i/16) + e][i % 16]
//   C/D:       lane i holds D[4*(i/16) + r][i % 16], r < 4
// fp32 inputs use v_mfma_f32_16x16x4_f32 (K = 4, one value per lane),
// bf16 inputs the gfx950 v_mfma_f32_16x16x32_bf16 (K = 32, eight per lane).
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<float> {
  static constexpr int K = 4;
  static constexpr int KPL = 1;
  using frag = float;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
  __device__ __forceinline__ static frag pack(const float* v) { return v[0]; }
};

template <> struct Mfma<bf16> {
  static constexpr int K = 32;
  static constexpr int KPL = 8;
  using frag = bf16x8;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ __forceinline__ static frag pack(const float* v) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = static_cast<bf16>(v[e]);
    return f;
  }
};

// 16-byte global vector of T
template <typename T> struct Vec16 {
  static constexpr int n = 16 / sizeof(T);
};

__device__ __forceinline__ void load_f32(const float* p, float* v, int n) {
  for (int i = 0; i < n; ++i) v[i] = p[i];
}

// Load 16 bytes (4 fp32 or 8 bf16) as fp32 values; zeros when !valid.
__device__ __forceinline__ void load16_as_f32(const float* p, bool valid, float* v) {
  if (valid) {
    float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
    v[0] = v[1] = v[2] = v[3] = 0.f;
  }
}
__device__ __forceinline__ void load16_as_f32(const bf16* p, bool valid, float* v) {
  if (valid) {
    bf16x8 q = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(q[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
}

// Raw 16-byte copy helpers.
__device__ __forceinline__ uint4 load16(const void* p, bool valid) {
  if (valid) return *reinterpret_cast<const uint4*>(p);
  return make_uint4(0, 0, 0, 0);
}


// ---------------------------------------------------------------------------
// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j receives elements j, 16+j, 32+j, 48+j of the group's
// concatenated 8-byte reads.  So if lane m of the group reads 4 bf16 at
// row (k0 + m/4), columns (c0 + 4*(m%4)) of a row-major [k][c] LDS tile, lane
// j gets column c0 + j of rows k0..k0+3: four consecutive k for one column,
// which is how the MFMA operands hold their k values.  Two such reads (rows
// k0.. and k0+4..) fill one 8-value bf16 operand.
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 lds_tr16_b64(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((__attribute__((address_space(3))) char*)(p)));
}

// MFMA operand (8 consecutive k of column c0 + lane%16, k starting at
// k0 + 8*(lane/16)) from a row-major [k][c] bf16 LDS tile with row pitch
// `pitch` elements.
__device__ __forceinline__ bf16x8 lds_operand_kmajor(const bf16* tile, int pitch, int k0, int c0,
                                                     int lane) {
  const int m = lane & 15, kg = lane >> 4;
  const bf16* p = tile + (k0 + 8 * kg + (m >> 2)) * pitch + c0 + 4 * (m & 3);
  const i16x4 lo = lds_tr16_b64(p);
  const i16x4 hi = lds_tr16_b64(p + 4 * pitch);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Workgroup id -> (chunk slot, head) so that every head of one chunk runs on
// the same XCD (the hardware deals workgroups to the 8 XCDs round-robin), where
// the chunk's shared B, C and CB tiles stay in that XCD's L2.
__device__ __forceinline__ int2 xcd_chunk_head(int b, int H) {
  const int x8 = b & 7, rest = b >> 3;
  return make_int2(8 * (rest / H) + x8, rest % H);
}
inline int xcd_grid(int max_chunks, int H) { return ((max_chunks + 7) / 8) * 8 * H; }

// ---------------------------------------------------------------------------
// Buffer resources: 32-bit offsets from a per-tile base, range-checked by the
// hardware.  A load past num_records returns zeros (also into LDS) and a
// store past it is dropped, so rows past a chunk's end need neither clamps
// nor branches, and no access can leave the tile.
// ---------------------------------------------------------------------------
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// Cache-policy bits of a buffer access (the aux operand): 0 is the default;
// kSc1 makes the access coherent at device scope -- a load sees what another
// workgroup on any XCD stored with kSc1 and waited for, and a store is
// written through the L2 -- which is how one launch hands data from one
// workgroup to another.
constexpr int kSc1 = 16;

template <int AUX = 0>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ float buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store2(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16 v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, off, 0, AUX);
}

// ---------------------------------------------------------------------------
// Token-major bf16 tiles in LDS, unpadded, with the 16-byte pieces of row r
// permuted by XOR with tile_sw(r).  One transpose read instruction touches
// rows r0 + {0..3} and r0 + {8..11} (r0 a multiple of 8) at two adjacent
// pieces; the XOR spreads those 8 rows x 2 pieces over distinct bank groups
// whether the LDS serves 16 or 32 lanes of 8-byte reads per clock.  Rows of
// 16 or more pieces (256 bytes: every row starts on the same bank) need all
// 16 pieces distinct; narrower rows alternate bank halves by themselves.
// tile_sw(r + 4) == tile_sw(r) whenever r % 8 < 4.
// ---------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int tile_sw(int r) {
  if constexpr (CPR >= 16) return (2 * ((r & 3) | ((r >> 1) & 4))) & (CPR - 1);
  else return (2 * ((r & 3) ^ ((r >> 3) & 1))) & (CPR - 1);
}

// Element offset of (row r, column c) in a swizzled tile of COLS columns.
template <int COLS>
__device__ __forceinline__ int tile_at(int r, int c) {
  return r * COLS + ((((c >> 3) ^ tile_sw<COLS / 8>(r))) << 3) + (c & 7);
}

// MFMA operand (8 consecutive k of column c0 + lane%16, k starting at
// k0 + 8*(lane/16); k0 a multiple of 8) from a swizzled token-major tile,
// by two transpose reads.
template <int COLS>
__device__ __forceinline__ bf16x8 lds_operand_sw(const bf16* tile, int k0, int c0, int lane) {
  const int m = lane & 15, kg = lane >> 4;
  const int r = k0 + 8 * kg + (m >> 2);
  const bf16* p = tile + tile_at<COLS>(r, c0 + 4 * (m & 3));
  const i16x4 lo = lds_tr16_b64(p);
  const i16x4 hi = lds_tr16_b64(p + 4 * COLS);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

}  // namespace ssd
