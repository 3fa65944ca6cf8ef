// Internal launcher interface between the C ABI (abi.hip) and the kernels.
// Arguments are validated by the caller; launchers only size grids, enqueue
// on `stream` and return the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace msda {

struct GatherArgs {
  // value images: image i starts at value + i * image_bytes
  const void* value;
  uint32_t image_bytes;
  int bf16;
  int pairs;  // bf16 in the head-pair layout (SCA only): per image [nH][Nv][2][32]
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
  float inv_LP;
  // optional locality plan (msda_plan): entries [b*Nq, (b+1)*Nq) hold batch
  // item b's queries b*Nq + q in the order to visit them
  const int32_t* plan;
  // SCA mode: images b*Ncam + c; work list from the compaction
  const float* rp;        // [Ncam][B][Nq][D][2]
  const float* offsets;   // [B][Nq][nH][L][P][2]
  const float* logits;    // [B][Nq][nH][L*P]
  const uint32_t* cammask;  // [B][Nq] bit c = camera c sees the query
  const int32_t* order;       // seen queries b*Nq + q, in locality order
  const int32_t* die_bounds;  // [B][kDieBounds]: die x's entries of batch item b, cost-balanced
  int Ncam, D;
  int64_t B, Nq;
  float* out;  // [B][Nq][nH*32]
};

hipError_t launch_msda_gather(const GatherArgs& a, hipStream_t stream);

// msda_pack_pairs_bf16 (pairs.hip): bf16 value [n_images][Nv][nH][32] to the
// head-pair layout [n_images][nH][Nv][2][32]
hipError_t launch_pack_pairs(const void* value, void* pairs, int64_t n_images, int64_t Nv, int nH,
                             hipStream_t stream);

// Locality plan of the operator (plan.hip): point of query (b, q) at
// points[b*batch_stride + q*point_stride] (x, y normalised); the plan buffer
// holds the visiting order [B*Nq] and, 256-byte aligned after it, the tile
// histograms of each batch item's kPlanChunks chunks [B][kPlanChunks][kPlanBins].
constexpr int kPlanBins = 32 * 32;
constexpr int kPlanChunks = 16;
inline size_t plan_bins_offset(int64_t B, int64_t Nq) { return ((size_t)(B * Nq) * 4 + 255) / 256 * 256; }
inline size_t plan_bytes(int64_t B, int64_t Nq) {
  return plan_bins_offset(B, Nq) + (size_t)B * kPlanChunks * kPlanBins * 4;
}
struct PlanArgs {
  const float* points;
  int64_t batch_stride, point_stride;
  int B, Nq;
  int32_t* order;
  int32_t* bins;
};
hipError_t launch_msda_plan(const PlanArgs& a, hipStream_t stream);
hipError_t launch_sca_gather(const GatherArgs& a, hipStream_t stream);

// SCA compaction and work ordering: workspace layout and launch.
constexpr int kQueryTile = 256;  // queries per tile of the compaction (and its pair ranking)
// Image-tile grid used to order the gather work (per first camera).
constexpr int kOrderBinsX = 64, kOrderBinsY = 16, kOrderBins = kOrderBinsX * kOrderBinsY;

// Each seen query also carries a work estimate, its cost: over the cameras
// that see it, 1 + the camera's marked anchors (an unmarked anchor projects
// outside the image, so its samples cost nothing).  The gather's split of a
// batch item's work list over the dies follows the summed cost.
struct CompactLayout {
  // bin_hist, seg_seen, seg_pairs, bin_cost and seg_cost are adjacent: one
  // clear covers them
  size_t cammask, qkey, qrank, tile_counts, tile_offsets, pair_offsets, pair_q, bin_hist, seg_seen, seg_pairs,
      bin_cost, seg_cost, order, die_bounds, total;
  int tiles;  // tiles of the query axis per (b, c)
  int clear_ints;  // int32 words from bin_hist on to zero before a compaction
};
CompactLayout compact_layout(int64_t B, int64_t Ncam, int64_t Nq);

struct CompactArgs {
  const uint8_t* bev_mask;
  const float* rp;  // [Ncam][B][Nq][D][2], only to order the work
  int B, Ncam, Nq, D;
  uint32_t* cammask;
  int32_t* qkey;       // [B][Nq] ordering bin of a seen query, -1 if unseen
  int32_t* qrank;      // [B][Nq] a seen query's rank among its bin's queries
  int32_t* hit_count;  // may be null
  int32_t* tile_counts;
  int32_t* tile_offsets;
  int32_t* pair_offsets;
  int32_t* pair_q;
  int32_t* bin_hist;     // [B*Ncam*kOrderBins]
  int32_t* seg_seen;     // [B*Ncam] seen queries whose first camera is c, per (b, c)
  int32_t* seg_pairs;    // [B*Ncam] pairs per (b, c)
  int32_t* order;        // [B*Nq]
  uint64_t* bin_cost;    // [B*Ncam*kOrderBins] summed cost of each ordering bin
  uint64_t* seg_cost;    // [B*Ncam] summed cost of the seen queries whose first camera is c, per (b, c)
  int32_t* die_bounds;   // [B][kDieBounds]: die x takes work-list entries [x, x+1) of its batch item
  int clear_ints;
};
hipError_t launch_sca_compact(const CompactArgs& a, int tiles, hipStream_t stream);

}  // namespace msda
