// Launcher interface of the bf16 projections on matrix cores (gemm.hip).
// Arguments are validated by the caller (abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

// Y = X W^T + bias over N output columns, split in two parts: columns
// [0, N1) use W1 / bias1 and go to Y1 [M][N1], columns [N1, N) use W2 /
// bias2 and go to Y2 [M][N - N1] (N1 == N: one output).  N1 % 32 == 0.
struct GemmArgs {
  const void* X;  // [M][K], bf16 bits or float32
  int x_f32;
  const float* X_add;  // float32 [M][K] added to float32 X before rounding, or null
  int64_t M;
  int N, K, N1;
  const uint16_t* W1;
  const float* bias1;
  void* Y1;
  const uint16_t* W2;
  const float* bias2;
  void* Y2;
  int y_f32;
  // single-output epilogue: + residual [M][N] (float32, may alias Y1), then,
  // with gamma, the layer norm of each row over its N == 256 columns
  const float* residual;
  const float* gamma;
  const float* beta;
  float eps;
  // > 0: Y1 is bf16 in the head-pair layout of images of pairs_Nv rows
  // ([M / pairs_Nv][N / 32][pairs_Nv][2][32]); single output, no epilogue
  int64_t pairs_Nv;
};

constexpr int kGemmNormCols = 256;  // row length the layer-norm epilogue handles

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream);

}  // namespace msda
