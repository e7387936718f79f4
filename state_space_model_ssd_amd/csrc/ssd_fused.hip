// The fused bf16 forward: the front (chunk_cumsum, bmm_chunk, chunk_state)
// in one launch, then state_passing and chunk_scan in ONE persistent launch
// in which the chunk_scan tiles of a chunk start as soon as the state chain
// has passed it.  The pages run the forward's stages as one fused path
// (aiproviderindex.com, "Mamba-2 offers a different scaling path":
// cumulative parameters, state propagation, output construction) and rework
// the state passing for parallel hardware (clova.ai, "Stage 3. Logic and
// heuristic refinement").  The front keeps a launch of its own: it runs at
// four 8-wave workgroups per CU, which the scan tile's registers would not
// allow, and it clears this launch's counters.
//
// Work items of the persistent launch, in this order (item i is taken by
// workgroup i mod grid, and every workgroup takes its items in increasing
// order):
//   1. chain items: per (sequence, head, slice of 4 * threads state
//      elements), the state_passing walk over the sequence's chunks,
//      writing the entering states in segments of 1, 2, 4, 8, then 16
//      chunks, each segment counted as done for its chunks when its stores
//      are complete;
//   2. scan items: per (chunk, head), the chunk_scan tile, which waits until
//      every chain slice of its (chunk, head) is counted.
// Counting argument: the lowest unfinished item has all of its dependencies
// finished (chain items depend on nothing in the launch, scan items on chain
// items), and its workgroup has finished everything before it, so it runs;
// with every workgroup resident (the grid is sized from the occupancy) the
// launch always drains.  A wait also gives up after about a second, setting an
// error word instead of hanging.
//
// Hand-over: the chain writes the entering states with device-coherent
// (sc1) stores, waits until its stores are complete (s_waitcnt vmcnt(0)),
// meets the workgroup's barrier, and one thread adds to the counters (device
// scope atomics); the scan tile polls its counter with device-scope loads and
// reads the entering states with sc1 loads.  No L2 write-back or invalidate
// is needed.  Everything else the tiles read was written by the front's
// launch.
//
// The arithmetic is exactly the separate launches' (same device functions,
// same order), so results equal the three-launch forward bit for bit when it
// runs the one-chain state passing and the same scan tile.
#include <atomic>

#include "ssd_kernels.h"
#include "ssd_scan_tile.h"
#include "ssd_state_tile.h"

namespace ssd {

namespace {

constexpr int kChainVec = 4;           // state elements per chain thread
constexpr int kChainSeg = 16;          // longest chain segment (its loads are in flight together)
constexpr unsigned kSpinLimit = 1u << 22;   // polls of about 0.1 us or more before giving up

// Counters of one fused call, cleared by the front's launch.
struct FusedSync {
  int* pdone;    // [max_chunks][H]: chain slices that wrote the chunk's entering state
  int* err;      // [1]: a wait gave up
};

__host__ __device__ inline int64_t sync_ints(int mc, int H) { return (int64_t)mc * H + 1; }

__device__ __forceinline__ FusedSync sync_of(int* base, int mc, int H) {
  FusedSync f;
  f.pdone = base;
  f.err = base + (int64_t)mc * H;
  return f;
}

// Thread 0 waits until *p >= target (or gives up, raising *err), then the
// whole workgroup meets.
__device__ __forceinline__ void wait_count(const int* p, int target, int* err) {
  if (threadIdx.x == 0) {
    unsigned n = 0;
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if ((++n & 255u) == 0 &&
          (n >= kSpinLimit || __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Every thread of the workgroup waits until its earlier stores are complete,
// then the workgroup meets: after this, all of them are.
__device__ __forceinline__ void stores_done_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// The state_passing walk of one slice of (sequence s, head h), TH threads of
// kChainVec elements: segment k covers min(2^k, kChainSeg) chunks, whose
// states are loaded together; the entering states leave as sc1 stores in
// x's dtype, and the segment is counted in pdone for its chunks once they are
// complete.  Short first segments let the scan tiles of a sequence's first
// chunks start early; long later ones keep many loads in flight.  Same
// arithmetic as the one-chain state_passing kernel.
template <int TH>
__device__ __forceinline__ void chain_item(const FwdArgs& a, const FusedSync& f, int s, int h,
                                           int slice, float* decs) {
  const ChunkMap cm = a.cmap();
  const int H = a.H, PN = a.P * a.N, L = a.L;
  const int tid = opaque_tid();
  const int e = (slice * TH + tid) * kChainVec;
  const bool live = e < PN;
  const int2 r = cm.seq_range(s);
  float4 st = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.init && live) st = *reinterpret_cast<const float4*>(a.init + ((int64_t)s * H + h) * PN + e);
  bf16* hin = static_cast<bf16*>(a.states_in);
  int seg = 1;
  for (int c0 = r.x; c0 < r.y; c0 += seg, seg = min(2 * seg, kChainSeg)) {
    const int nb = min(seg, r.y - c0);
    if (tid < nb) {
      const int len = cm.desc(c0 + tid).len;
      const float la = len > 0 ? a.dAcs[((int64_t)(c0 + tid) * H + h) * L + len - 1] : 0.f;
      decs[tid] = expf(la);
    }
    __syncthreads();
    if (live) {
      float4 buf[kChainSeg];
#pragma unroll
      for (int i = 0; i < kChainSeg; ++i)
        if (i < nb)                         // uniform over the workgroup
          buf[i] = *reinterpret_cast<const float4*>(a.chunk_states + ((int64_t)(c0 + i) * H + h) * PN + e);
#pragma unroll
      for (int i = 0; i < kChainSeg; ++i) {
        if (i < nb) {
          bf16x4 q;
          q[0] = static_cast<bf16>(st.x);
          q[1] = static_cast<bf16>(st.y);
          q[2] = static_cast<bf16>(st.z);
          q[3] = static_cast<bf16>(st.w);
          buf_store8<kSc1>(buf_rsrc(hin + ((int64_t)(c0 + i) * H + h) * PN, PN * 2), e * 2,
                           __builtin_bit_cast(uint2, q));
          const float d = decs[i];
          st.x = d * st.x + buf[i].x;
          st.y = d * st.y + buf[i].y;
          st.z = d * st.z + buf[i].z;
          st.w = d * st.w + buf[i].w;
        }
      }
    }
    stores_done_barrier();                  // every entering state of the segment is stored
    if (tid < nb)
      __hip_atomic_fetch_add(f.pdone + (int64_t)(c0 + tid) * H + h, 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();                        // decs free for the next segment
  }
  if (live && a.final_states)
    *reinterpret_cast<float4*>(a.final_states + ((int64_t)s * H + h) * PN + e) = st;
}

template <int P, int N, int L>
struct FusedSmem {
  static constexpr int HP = N + 8;
  static constexpr size_t kScan = (size_t)L * P * 2 + (size_t)P * HP * 2 + 3 * L * 4;
  static constexpr size_t kChain = kChainSeg * 4;
  static constexpr size_t bytes = kScan > kChain ? kScan : kChain;
};

// Item counts of one call (host and device agree on them).
struct FusedPlan {
  int nchain, nchain8, nscan, nslices;
  __host__ __device__ int total() const { return nchain8 + nscan; }
};

__host__ __device__ inline FusedPlan fused_plan(int mc, int H, int nstates, int PN, int th) {
  FusedPlan p;
  p.nslices = (PN + th * kChainVec - 1) / (th * kChainVec);
  p.nchain = nstates * H * p.nslices;
  p.nchain8 = (p.nchain + 7) / 8 * 8;
  p.nscan = ((mc + 7) / 8) * 8 * H;
  return p;
}

typedef const __attribute__((address_space(4))) FwdArgs KernFwdArgs;

// The kernel's arguments as loaded for one item: the pointer to them is
// laundered every iteration, so the compiler loads each field (scalar loads
// from the kernel-argument segment) inside the branch that uses it instead of
// holding every field in registers across the whole loop.
__device__ __forceinline__ FwdArgs item_args() {
#if defined(__HIP_DEVICE_COMPILE__)
  KernFwdArgs* ka = (KernFwdArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ka));
  return *ka;
#else
  return FwdArgs{};                         // (host pass: never called)
#endif
}

// NW waves per workgroup: the scan tile of the separate launches the
// library would pick (8 waves, or 4 waves of four row groups each).
template <int P, int N, int L, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kTileWavesPerEU<L, NW>))) void
fused_scan_kernel(FwdArgs args) {
  using SM = FusedSmem<P, N, L>;
  constexpr int TH = 64 * NW;
  __shared__ __align__(16) unsigned char smem[SM::bytes];
  const FusedPlan pl = fused_plan(args.max_chunks, args.H, args.nstates, P * N, TH);
  const int total = pl.total();

  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    __syncthreads();                        // the previous item is done with the LDS
    const FwdArgs a = item_args();
    const int H = a.H, G = a.G, mc = a.max_chunks;
    const FusedSync f = sync_of(a.sync, mc, H);
    int k = it;
    if (k < pl.nchain8) {                   // ---- state_passing chain slice
      if (k >= pl.nchain) continue;
      const int sl = k % pl.nslices, sh = k / pl.nslices;
      chain_item<TH>(a, f, sh / H, sh % H, sl, reinterpret_cast<float*>(smem));
      continue;
    }
    k -= pl.nchain8;                        // ---- chunk_scan tile
    const int2 jh = xcd_chunk_head(k, H);
    if (jh.x >= mc) continue;
    const ChunkDesc d = a.cmap().desc(jh.x);
    if (d.len <= 0) continue;
    wait_count(f.pdone + (int64_t)jh.x * H + jh.y, pl.nslices, f.err);
    const float last = a.dAcs[((int64_t)jh.x * H + jh.y) * L + L - 1];
    const ScanTile T{jh.x, jh.y, d.start, d.len};
    bf16* xs = reinterpret_cast<bf16*>(smem);
    bf16* hsm = xs + L * P;
    float* dal2 = reinterpret_cast<float*>(hsm + P * SM::HP);
    float* dls = dal2 + L;
    float* cfs = dls + L;
    const bf16* x = static_cast<const bf16*>(a.x);
    const bf16* C = static_cast<const bf16*>(a.C);
    const bf16* cb = static_cast<const bf16*>(a.cb);
    const bf16* hin = static_cast<const bf16*>(a.states_in);
    bf16* out = static_cast<bf16*>(a.out);
    if (fabsf(last) * kLog2e <= kScanFastMaxLog2)   // uniform over the workgroup
      scan_tile_body<P, N, L, NW, true, kSc1, 0, true>(T, x, C, cb, a.delta, a.dAcs, hin, a.D, H,
                                                        G, out, xs, hsm, dal2, dls, cfs);
    else
      scan_tile_body<P, N, L, NW, false, kSc1, 0, true>(T, x, C, cb, a.delta, a.dAcs, hin, a.D, H,
                                                         G, out, xs, hsm, dal2, dls, cfs);
  }
}

// Resident workgroups of the fused kernel, a multiple of 8, cached per
// (instantiation, device); 0 if a query fails.
template <int P, int N, int L, int NW>
int fused_grid() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int c = cached[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  const int cus = device_cu_count();
  int per_cu = 0;
  if (cus <= 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(
                      &per_cu, fused_scan_kernel<P, N, L, NW>, 64 * NW, 0) != hipSuccess)
    return 0;
  const int g = (cus * per_cu) / 8 * 8;
  cached[dev].store(g, std::memory_order_relaxed);
  return g;
}

template <int P, int N, int L, int NW>
hipError_t launch_fused_scan(const FwdArgs& a, hipStream_t s) {
  const int g = fused_grid<P, N, L, NW>();
  if (g <= 0) return hipErrorInvalidDevice;
  const FusedPlan pl = fused_plan(a.max_chunks, a.H, a.nstates, P * N, 64 * NW);
  const int total = pl.total();
  if (total <= 0) return hipSuccess;
  const int grid = total < g ? (total + 7) / 8 * 8 : g;
  hipLaunchKernelGGL((fused_scan_kernel<P, N, L, NW>), dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t fused_sync_bytes(int nstates, int H, int G, int max_chunks) {
  (void)nstates;
  (void)G;
  return sizeof(int) * (size_t)sync_ints(max_chunks, H);
}

template <typename T, int P, int N, int L>
bool fused_supported() {
  return sizeof(T) == 2 && (L == 128 || L == 256);
}

// The front (which also clears the counters), then the chain and the scan
// tiles in one launch, with the scan tile the separate launches would run
// (choice 3: four waves; 1 or 2: eight waves).
template <typename T, int P, int N, int L>
hipError_t launch_fused(const FwdArgs& a, int scan_choice, hipStream_t s) {
  if constexpr (sizeof(T) != 2 || (L != 128 && L != 256)) {
    return hipErrorInvalidValue;
  } else {
    FwdArgs fa = a;
    fa.zero_ints = a.max_chunks > 0 ? sync_ints(a.max_chunks, a.H) : 0;
    hipError_t e = launch_front<T, P, N, L>(fa, s);
    if (e != hipSuccess) return e;
    if (scan_choice == 3 && kTileWaves<L> == 8) return launch_fused_scan<P, N, L, 4>(a, s);
    return launch_fused_scan<P, N, L, 8>(a, s);
  }
}

#define SSD_INST(T, P, N, L)                                                               \
  template bool fused_supported<T, P, N, L>();                                         \
  template hipError_t launch_fused<T, P, N, L>(const FwdArgs&, int, hipStream_t);
SSD_FOR_EACH_CONFIG(SSD_INST)
#undef SSD_INST

}  // namespace ssd
