// Launcher interface of the padded rebatch form of SCA (rebatch.hip).
// Arguments are validated by the caller (abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

struct RebatchArgs {
  const int32_t* pair_offsets;  // [B*Ncam + 1]
  const int32_t* pair_q;        // [pairs]
  const float* rp;              // [Ncam][B][Nq][D][2]
  const float* offsets;         // [B][Nq][nH][L][P][2]
  const float* logits;          // [B][Nq][nH][L*P]
  const int64_t* shapes;        // [L][2] as (H, W), device
  int64_t B, Ncam, Nq;
  int nH, L, P, D;
  int64_t max_len;
  float* loc_out;     // [B*Ncam][max_len][nH][L][P][2]
  float* logits_out;  // [B*Ncam][max_len][nH][L*P]
};

struct ScatterArgs {
  const float* rows;  // [B*Ncam][max_len][C]
  const int32_t* pair_offsets;
  const int32_t* pair_q;
  const int32_t* hit_count;  // [B][Nq]
  int64_t B, Ncam, Nq, C, max_len;
  float* slots;  // [B][Nq][C]
};

hipError_t launch_sca_rebatch(const RebatchArgs& a, hipStream_t stream);
hipError_t launch_sca_scatter_mean(const ScatterArgs& a, hipStream_t stream);

}  // namespace msda
