// Internal launcher interface between the C ABI (abi.hip) and the kernels.
// Arguments are validated by the caller; launchers only size grids, enqueue
// on `stream` and return the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msda {

struct GatherArgs {
  // value images: image i starts at value + i * image_bytes
  const void* value;
  uint32_t image_bytes;
  int bf16;
  // level table (device, int64) and sizes
  const int64_t* shapes;
  const int64_t* starts;
  int L, P, LP, nH, Nv;
  float inv_P, inv_D;
  // MSDA / frames mode: image b*F + f; rows of locations and weights are
  // indexed by ((b*F + f)*Nq + q)
  const float* loc;
  const float* weights;
  int weight_logits;
  int F;
  // SCA mode: images b*Ncam + c; work list from the compaction
  const float* rp;        // [Ncam][B][Nq][D][2]
  const float* offsets;   // [B][Nq][nH][L][P][2]
  const float* logits;    // [B][Nq][nH][L*P]
  const uint32_t* cammask;  // [B][Nq] bit c = camera c sees the query
  const int32_t* order;     // seen queries b*Nq + q, in locality order
  const int32_t* order_at;  // device: batch item b's entries are [order_at[b*stride], order_at[(b+1)*stride])
  int order_stride;
  int Ncam, D;
  int64_t B, Nq;
  float* out;  // [B][Nq][nH*32]
};

hipError_t launch_msda_gather(const GatherArgs& a, hipStream_t stream);
hipError_t launch_sca_gather(const GatherArgs& a, hipStream_t stream);

// SCA compaction and work ordering: workspace layout and launch.
constexpr int kQueryTile = 256;  // queries per tile of the compaction (and its pair ranking)
// Image-tile grid used to order the gather work (per first camera).
constexpr int kOrderBinsX = 64, kOrderBinsY = 16, kOrderBins = kOrderBinsX * kOrderBinsY;

struct CompactLayout {
  // bin_hist, seg_seen and seg_pairs are adjacent: one clear covers them
  size_t cammask, qkey, tile_counts, tile_offsets, pair_offsets, pair_q, bin_hist, seg_seen, seg_pairs,
      bin_offsets, order, total;
  int tiles;  // tiles of the query axis per (b, c)
  int clear_ints;  // int32 entries from bin_hist on to zero before a compaction
};
CompactLayout compact_layout(int64_t B, int64_t Ncam, int64_t Nq);

struct CompactArgs {
  const uint8_t* bev_mask;
  const float* rp;  // [Ncam][B][Nq][D][2], only to order the work
  int B, Ncam, Nq, D;
  uint32_t* cammask;
  int32_t* qkey;       // [B][Nq] ordering bin of a seen query, -1 if unseen
  int32_t* hit_count;  // may be null
  int32_t* tile_counts;
  int32_t* tile_offsets;
  int32_t* pair_offsets;
  int32_t* pair_q;
  int32_t* bin_hist;     // [B*Ncam*kOrderBins]
  int32_t* seg_seen;     // [B*Ncam] seen queries whose first camera is c, per (b, c)
  int32_t* seg_pairs;    // [B*Ncam] pairs per (b, c)
  int32_t* bin_offsets;  // [B*Ncam*kOrderBins + 1]; the last entry counts the seen queries
  int32_t* order;        // [B*Nq]
  int clear_ints;
};
hipError_t launch_sca_compact(const CompactArgs& a, int tiles, hipStream_t stream);

}  // namespace msda
