// Device helpers shared by the forward (gather.hip) and backward
// (backward.hip) sampling kernels: the level table, per-head attention
// weights, sample liveness and 8-lane group reductions.
#pragma once

#include <cmath>

#include "common.hpp"

namespace msda {

constexpr int kHeadSlots = 8;  // heads per wave pass: lane group g = lane / 8
constexpr size_t kMaxBlockLds = 64 * 1024;
constexpr int kMaxLevels = 64;
constexpr uint32_t kSkip = 0x80000000u;  // beyond every image (images < 2^31 bytes)
// samples per lane (template kSPL): 4 when L*P <= 32, 8 when L*P <= 64

struct Level {
  int W, H;
  long long start;
};

// k / n for 0 <= k < 2^16 and 1 <= n <= 64, with inv = 1/n in fp32: the
// quotient sits at least 0.5/n away from the next integer, far beyond the
// rounding error of (k + 1/2) * inv.
__device__ inline int small_div(int k, float inv) { return (int)((k + 0.5f) * inv); }

// Lane exchanges inside a group of 8 as DPP moves (VALU, no LDS traffic):
// quad_perm(1,0,3,2) swaps lanes i and i^1, quad_perm(2,3,0,1) lanes i and
// i^2, row_half_mirror lanes i and 7-i (which, once each quad holds one
// value, is the other quad's).  All 8 lanes of a group are active together.
template <int kCtrl>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1, kDppXor2 = 0x4e, kDppHalfMirror = 0x141;

__device__ inline float group_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  return fmaxf(v, dpp<kDppHalfMirror>(v));
}
__device__ inline float group_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  return v + dpp<kDppHalfMirror>(v);
}

// Weights of the samples k = j + 8i of one head: probabilities as given, or
// softmax over the head's L*P logits, reduced across the 8 lanes of a group.
template <int kSPL>
__device__ inline void head_weights(const float* __restrict__ w_row, bool head_ok, int LP, int j, bool logits,
                                    float (&alpha)[kSPL]) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    const int k = j + 8 * i;
    alpha[i] = (head_ok && k < LP) ? w_row[k] : 0.f;
    if (head_ok && k < LP) m = fmaxf(m, alpha[i]);
  }
  if (!logits) return;
  m = group_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    const int k = j + 8 * i;
    const float e = (head_ok && k < LP) ? expf(alpha[i] - m) : 0.f;
    alpha[i] = e;
    s += e;
  }
  s = group_sum(s);
  const float inv = head_ok ? 1.0f / s : 0.f;
#pragma unroll
  for (int i = 0; i < kSPL; ++i) alpha[i] *= inv;
}

// A sample is live when at least one of its corners can lie inside the map:
// -1 <= x < W and -1 <= y < H (a live sample may still contribute nothing;
// a dead one never does).
__device__ inline bool sample_live(double x, double y, const Level& lv) {
  return x >= -1.0 && x < (double)lv.W && y >= -1.0 && y < (double)lv.H;
}

// The level table (H, W, start of each level) into LDS, then a block barrier.
__device__ inline void load_levels(const int64_t* shapes, const int64_t* starts, int L, Level* lv) {
  for (int l = threadIdx.x; l < L; l += blockDim.x) {
    const long long H = shapes[2 * l], W = shapes[2 * l + 1], s = starts[l];
    Level v;
    const bool ok = H >= 1 && W >= 1 && H <= (1 << 30) && W <= (1 << 30);
    v.W = ok ? (int)W : 0;  // an unusable level samples nothing
    v.H = ok ? (int)H : 0;
    v.start = s < -(1ll << 40) ? -(1ll << 40) : (s > (1ll << 40) ? (1ll << 40) : s);
    lv[l] = v;
  }
  __syncthreads();
}

}  // namespace msda
