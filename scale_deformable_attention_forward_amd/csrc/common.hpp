// Device and host helpers shared by the kernels of libmsda.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

constexpr int kWave = 64;  // CDNA wavefront width
constexpr int kXcds = 8;   // MI355X: 8 accelerator dies, each with its own L2

// Raw buffer resource over [base, base + bytes).  A load whose offset is at
// or beyond `bytes` returns zeros and makes no memory request, which is how
// corners outside the map are skipped without a branch.  Word 3 is the gfx9
// data-format word for untyped 32-bit accesses.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
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

}  // namespace msda
