// Device and host helpers shared by the kernels of libmsda.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

constexpr int kWave = 64;  // CDNA wavefront width
constexpr int kXcds = 8;   // MI355X: 8 accelerator dies, each with its own L2
constexpr int kDieBounds = kXcds + 1;  // entries of a per-die split of a list (DieShare)

// Compute units of the device current at the first call (256 when the
// runtime cannot say), read once per process; safe to call from several
// threads.  Grids sized from it assume every device the library runs on has
// as many.
int device_cu_count();

// Raw buffer resource over [base, base + bytes).  A load whose offset is at
// or beyond `bytes` returns zeros and makes no memory request, which is how
// corners outside the map are skipped without a branch.  Word 3 is the gfx9
// data-format word for untyped 32-bit accesses.
// The base must be the same in every lane; it is read from the first active
// lane so that the compiler keeps the descriptor in scalar registers (a
// descriptor it cannot prove uniform costs a readfirstlane loop per load).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Order LDS traffic between the lanes of one wavefront: everything written
// before is visible to reads after (LDS serves one wave in issue order; this
// also stops the compiler from moving accesses across).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ inline int64_t uniform(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Checked builds (compiled with -DMSDA_CHECKED into libmsda_checked.so):
// device-side bounds checks on the compaction's writes, on the work-list,
// plan and pair-list entries the kernels read, and on every corner row a
// gather stages.  A failed check adds one to a per-kind counter in device
// memory (a vector atomic; nothing traps and no result changes), which
// msda_check_counts reads back.  In the regular build MSDA_CHECK evaluates
// nothing.
constexpr int kCheckKinds = 4;
enum CheckKind {
  kCheckGatherRow = 0,    // a staged corner row outside its sample's level or image
  kCheckPairWrite = 1,    // a pair-list entry written outside its tile's range, or a query index outside [0, Nq)
  kCheckOrderWrite = 2,   // a work-list slot written outside [0, B*Nq) or its segment's range
  kCheckListEntry = 3,    // a work-list, plan, pair-list or segment-bound entry read that had to be clamped
};
// Adds a translation unit's counters to counts (and zeroes them when reset);
// the readers of every unit are registered at load time (abi.hip).
typedef hipError_t (*CheckReader)(unsigned long long* counts, bool reset);
bool register_check_reader(CheckReader reader);

#ifdef MSDA_CHECKED
static __device__ unsigned long long g_check_counts[kCheckKinds];
#define MSDA_CHECK(kind, cond)                                                 \
  do {                                                                         \
    if (!(cond)) atomicAdd(&::msda::g_check_counts[(kind)], 1ull);             \
  } while (0)
static hipError_t read_check_counts(unsigned long long* counts, bool reset) {
  unsigned long long h[kCheckKinds];
  hipError_t e = hipMemcpyFromSymbol(h, HIP_SYMBOL(g_check_counts), sizeof h, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  for (int k = 0; k < kCheckKinds; ++k) counts[k] += h[k];
  if (!reset) return hipSuccess;
  const unsigned long long zero[kCheckKinds] = {};
  return hipMemcpyToSymbol(HIP_SYMBOL(g_check_counts), zero, sizeof zero, 0, hipMemcpyHostToDevice);
}
[[maybe_unused]] static const bool g_check_reader_registered = register_check_reader(&read_check_counts);
#else
#define MSDA_CHECK(kind, cond) \
  do {                         \
    (void)sizeof(cond);        \
  } while (0)
#endif

// Work split for a grid whose size is a multiple of kXcds.  The hardware
// hands workgroups to the dies round-robin (block i -> die i % 8), so die x
// owns the contiguous item range [N*x/8, N*(x+1)/8) and walks it with all of
// its waves; neighbouring items (which read neighbouring value rows) then
// share one L2.
struct XcdSplit {
  int64_t begin, end, stride;
  __device__ XcdSplit(int64_t n_items, int waves_per_block) {
    const int xcd = blockIdx.x % kXcds;
    const int local = blockIdx.x / kXcds;
    const int nlocal = gridDim.x / kXcds;
    const int wave = uniform(threadIdx.x / kWave);
    const int64_t lo = n_items * xcd / kXcds;
    end = n_items * (xcd + 1) / kXcds;
    begin = lo + (int64_t)local * waves_per_block + wave;
    stride = (int64_t)nlocal * waves_per_block;
  }
};

// The same walk over a range given per die: die x takes the work-list
// entries [bounds[x], bounds[x+1]) (clamped to [0, n_items], so that bounds
// from another call never send a read out of bounds).
struct DieShare {
  int64_t begin, end, stride;
  __device__ DieShare(const int32_t* bounds, int64_t n_items, int waves_per_block) {
    const int xcd = blockIdx.x % kXcds;
    const int local = blockIdx.x / kXcds;
    const int nlocal = gridDim.x / kXcds;
    const int wave = uniform(threadIdx.x / kWave);
    int64_t lo = bounds[xcd], hi = bounds[xcd + 1];
    MSDA_CHECK(kCheckListEntry, lo >= 0 && lo <= hi && hi <= n_items);
    lo = lo < 0 ? 0 : (lo > n_items ? n_items : lo);
    hi = hi < lo ? lo : (hi > n_items ? n_items : hi);
    begin = lo + (int64_t)local * waves_per_block + wave;
    end = hi;
    stride = (int64_t)nlocal * waves_per_block;
  }
};

}  // namespace msda
