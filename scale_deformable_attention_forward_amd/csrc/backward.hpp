// Launcher interface of the backward pass (backward.hip).  Arguments are
// validated by the caller (abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

struct BackwardArgs {
  // value images (image i starts at value + i * image_bytes) and their
  // gradient (float32, image i starts at grad_value + i * grad_image_bytes)
  const void* value;
  uint32_t image_bytes;
  int bf16;
  float* grad_value;
  uint32_t grad_image_bytes;
  int64_t images;  // number of images (B for MSDA, B * Ncam for SCA)
  const int64_t* shapes;
  const int64_t* starts;
  int L, P, LP, nH, Nv;
  float inv_P, inv_D;
  int64_t B, Nq;
  int F;                  // MSDA: frames per batch item (images b * F + f, B counting images), 1 otherwise
  const float* grad_out;  // [B / F][Nq][nH*32]
  // MSDA: weights and locations per (b, q); outputs per (b, q)
  const float* loc;
  const float* weights;
  int weight_logits;
  float* grad_loc;      // [B][Nq][nH][L][P][2]
  float* grad_weights;  // [B][Nq][nH][L*P]
  // SCA: anchors, offsets, logits, the compaction's camera masks and work list
  const float* rp;
  const float* offsets;
  const float* logits;
  const uint32_t* cammask;
  const int32_t* order;
  const int32_t* die_bounds;  // [B][kDieBounds], as sca_compact left them
  int Ncam, D;
  float* grad_offsets;  // [B][Nq][nH][L][P][2]
  float* grad_logits;   // [B][Nq][nH][L*P]
  // When rec_keys is set, the value gradient is not accumulated here: every
  // sample writes its record (vgrad.hpp) in the segment of its (image, head)
  // s = image * nH + h, at slot seg_tile[s] * kSortTile + local * LP + k,
  // local = q for MSDA and pair_of[c][b][q] - pair_start[image] for SCA
  // (pairs at or past max_pairs write nothing), and vgrad.hip builds
  // grad_value from them.
  uint32_t* rec_keys;
  void* rec_vals;
  uint32_t rec_slots;  // slots the record buffers hold (below 2^28)
  const int32_t* seg_tile;
  const int32_t* pair_start;
  const int32_t* pair_of;
  int64_t max_pairs;
};

hipError_t launch_msda_backward(const BackwardArgs& a, hipStream_t stream);
hipError_t launch_sca_backward(const BackwardArgs& a, hipStream_t stream);

}  // namespace msda
