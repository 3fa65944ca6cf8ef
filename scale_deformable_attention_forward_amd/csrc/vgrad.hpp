// Value gradient of the backward pass without atomics (vgrad.hip): the
// backward kernels write one record per sample, these kernels sort the
// records by corner and sum, for every value row, the records of its four
// neighbouring corner keys in a fixed order.  Arguments are validated by the
// caller (abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sampling.hpp"

namespace msda {

constexpr uint32_t kDeadKey = 0xffffffffu;  // a sample with no corner inside its map
constexpr int kSortTile = 2048;             // records a block of a sort pass ranks and writes together
constexpr int kDigitBits = 8;               // key bits per sort pass
constexpr int kDigits = 1 << kDigitBits;
constexpr int kRowChunk = 128;              // records of a value row the first pass sums (one 8-lane group)

// Payload of a sample record: the upstream gradient row it scales (b*Nq + q)*nH + h,
// its attention weight (for SCA divided by the query's hit count) and its
// position inside the cell.
struct VgradRec {
  uint32_t src;
  float alpha, fx, fy;
};

// Set by the kernels; nonzero makes the row kernel write NaN rows.
constexpr int kVgradPairsOverflow = 1;  // more camera-query pairs than the workspace holds
constexpr int kVgradKeysOverflow = 2;   // the level table's corner grid exceeds the key range

struct VgradState {
  int64_t n_items;  // record slots written by the backward kernel
  int64_t n_live;   // records left after the first sort pass (dead ones dropped)
  int32_t status;
  int32_t pad;
};

// Workspace: two key and two payload buffers (sort ping-pong), per-tile digit
// counts, per-key ranges of the sorted records, the SCA pair index of each
// (camera, query) and the state.
struct VgradLayout {
  size_t keys[2], vals[2], counts, digit_totals, ranges, long_row, pair_of, state, total;
  int64_t slots;      // record capacity
  int64_t sort_tiles;  // ceil(slots / kSortTile)
  int64_t key_bound;  // keys are below this
  int passes;         // kDigitBits-bit digit passes covering key_bound - 1
};
// images: B (MSDA) or B*Ncam (SCA); pair_of_entries: Ncam*B*Nq (SCA) or 0
VgradLayout vgrad_layout(int64_t images, int64_t Nv, int L, int nH, int64_t slots, int64_t pair_of_entries);

struct VgradArgs {
  // records and sort buffers
  uint32_t* keys[2];
  VgradRec* vals[2];
  uint32_t* counts;        // [kDigits][sort_tiles]
  uint32_t* digit_totals;  // [kDigits]
  int2* ranges;            // [key_bound] (first, end) of each key's records
  uint8_t* long_row;       // [images*Nv*nH] rows with more than kRowChunk records at a level
  VgradState* state;
  int64_t slots, key_bound;
  int64_t sort_tiles;  // tiles of kSortTile slots the buffers hold
  int passes;
  // geometry
  const int64_t* shapes;
  const int64_t* starts;
  int L, nH, Nv;
  int64_t images;
  const float* grad_out;  // [B*Nq*nH][32]
  uint32_t grad_out_bytes;
  float* grad_value;      // [images][Nv][nH][32]
  // SCA: pairs (from the compaction) and where the records of each pair start
  int32_t* pair_of;  // [Ncam][B][Nq]
  const uint32_t* cammask;
  const int32_t* tile_offsets;
  const int32_t* tile_counts;
  int B, Ncam, Nq, tiles;
  int64_t max_pairs;
  int LP;
};

// Start of each level's corner keys: level l has (W + 1) x (H + 1) of them
// (corner (x0 + 1, y0 + 1) for x0 in [-1, W - 1], y0 in [-1, H - 1]); ext[L]
// is the number per image and head (saturated far above any key range).
__device__ inline void load_corner_starts(const Level* lv, int L, long long* ext) {
  if (threadIdx.x == 0) {
    long long s = 0;
    for (int l = 0; l < L; ++l) {
      ext[l] = s;
      s += (long long)(lv[l].W + 1) * (lv[l].H + 1);
      if (s > (1ll << 50)) s = 1ll << 50;
    }
    ext[L] = s;
  }
  __syncthreads();
}

// Key of corner (ex, ey) = (x0 + 1, y0 + 1) of level l, head h of an image.
__device__ inline uint64_t corner_key(int64_t image, long long next, long long ext_l, int W, int ex, int ey, int nH,
                                      int h) {
  return (uint64_t)((image * next + ext_l + (long long)ey * (W + 1) + ex) * (long long)nH + h);
}

// Before the backward kernel: the state, and for SCA the pair indices.
hipError_t launch_vgrad_setup(const VgradArgs& a, bool sca, hipStream_t stream);
// After the backward kernel: sort, key ranges, rows of grad_value.
hipError_t launch_vgrad_rows(const VgradArgs& a, hipStream_t stream);

}  // namespace msda
