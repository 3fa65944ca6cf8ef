// Value gradient of the backward pass without atomics (vgrad.hip): the
// backward kernels write one record per sample, these kernels sort the
// records by corner and sum, for every value row, the records of its four
// neighbouring corner keys in a fixed order.  Arguments are validated by the
// caller (abi.hip).
//
// Records are kept in segments, one per (image, head) s = image * nH + h,
// each starting on a sort tile: a sample's key is its corner's index in the
// image's corner grids (below 2^16 for maps of up to ~32 k pixels), so a
// segment sorts in kDigitBits-bit passes over that index alone; the
// segment-wide key of corner key k is s * (corner keys per image) + k.
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
constexpr int kHistTiles = 8;               // sort tiles one histogram block counts

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
  int64_t corner_keys;  // corner keys per image and head: the levels' (W + 1)(H + 1) summed
  int64_t tiles;        // sort tiles in use
  int32_t status;
  int32_t passes;       // digit passes the corner keys need (the launches past them return at once)
  int32_t sorted;       // the key / record buffer the last pass wrote
  int32_t pad;
};

// Workspace: two key and two payload buffers (sort ping-pong), per-tile digit
// counts, per-segment digit totals and tables, per-key ranges of the sorted
// records, the SCA pair index of each (camera, query) and the state.
struct VgradLayout {
  size_t keys[2], vals[2], counts, tile_seg, digit_totals, seg_tile, seg_items, seg_live, pair_start, ranges, long_row,
      pair_of, state, total;
  int64_t segments;    // images * nH
  int64_t sort_tiles;  // tile capacity of the record buffers (kSortTile slots each)
  int64_t slots;       // sort_tiles * kSortTile
  int64_t key_bound;   // segment-wide keys are below this
  int passes;          // kDigitBits-bit digit passes covering a corner key
};
// images: B (MSDA) or B*Ncam (SCA); records: the most samples the records
// hold (pairs * nH * L * P); pair_of_entries: Ncam*B*Nq (SCA) or 0;
// per_segment: the records of every (image, head) when all hold the same
// number (MSDA: Nq * L * P), else 0
VgradLayout vgrad_layout(int64_t images, int64_t Nv, int L, int nH, int64_t records, int64_t pair_of_entries,
                         int64_t per_segment);

struct VgradArgs {
  // records and sort buffers
  uint32_t* keys[2];
  VgradRec* vals[2];
  uint32_t* counts;        // [kDigits][sort_tiles] digit counts of each tile, then their offsets in the segment
  int32_t* tile_seg;       // [sort_tiles] the segment of each tile in use
  uint32_t* digit_totals;  // [segments][kDigits]
  int32_t* seg_tile;       // [segments + 1] first tile of each segment; the last entry is the tiles in use
  int32_t* seg_items;      // [segments] record slots the backward kernel writes in each segment
  int32_t* seg_live;       // [segments] records left after the first pass (dead ones dropped)
  int32_t* pair_start;     // [images] first pair of each image (SCA)
  int2* ranges;            // [key_bound] (first, end) of each key's records
  uint8_t* long_row;       // [images*Nv*nH] rows with more than kRowChunk records at a level
  VgradState* state;
  int64_t segments, sort_tiles, key_bound;
  int passes;
  // geometry
  const int64_t* shapes;
  const int64_t* starts;
  int L, nH, Nv;
  int64_t images;
  const float* grad_out;  // [B*Nq*nH][32]
  uint32_t grad_out_bytes;
  float* grad_value;      // [images][Nv][nH][32]
  // MSDA: an image's pairs are its Nq queries; SCA: the pairs of the
  // compaction (image b*Ncam + c holds the pair list of (b, c)) and the pair
  // index of each (camera, query)
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

// Key of corner (ex, ey) = (x0 + 1, y0 + 1) of level l within its image's
// corner grids (ext_l from load_corner_starts).
__device__ inline uint32_t corner_key(long long ext_l, int W, int ex, int ey) {
  return (uint32_t)(ext_l + (long long)ey * (W + 1) + ex);
}

// The segment-wide key: corner key k of segment s = image * nH + h, with
// next corner keys per image and head.
__device__ inline uint64_t segment_key(int64_t s, long long next, uint32_t k) {
  return (uint64_t)s * (uint64_t)next + k;  // wraps only for a level table the setup flags
}

// The segment of sort tile t: the last s with seg_tile[s] <= t (seg_tile
// ascending, segments + 1 entries).
__device__ inline int64_t segment_of_tile(const int32_t* seg_tile, int64_t segments, int64_t t) {
  int64_t lo = 0, hi = segments;  // seg_tile[lo] <= t < seg_tile[hi]
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if (seg_tile[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Before the backward kernel: the state, and for SCA the pair indices.
hipError_t launch_vgrad_setup(const VgradArgs& a, bool sca, hipStream_t stream);
// After the backward kernel: sort, key ranges, rows of grad_value.
hipError_t launch_vgrad_rows(const VgradArgs& a, hipStream_t stream);

}  // namespace msda
