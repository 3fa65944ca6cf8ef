// Fused softmax + bilinear gather-accumulate: the hot loop of multi-scale
// deformable attention, for the plain operator, the frame-mean variant and
// BEVFormer's spatial cross-attention (SCA).
//
// Method ("BEV(三) BEVFormer：Query 参数如何与 Feature 的 8 个 Head 交互"):
//   4.2  per head, softmax over its L*P logits;
//   5    SCA location s = rho[anchor p mod D] + (dx / W_l, dy / H_l);
//   6    continuous level coordinate x = W_l*s_x - 1/2, y = H_l*s_y - 1/2 and
//        four-neighbour bilinear interpolation (corners outside read zero);
//   8, 9 weighted sum over the L*P samples, heads concatenated;
//   10   SCA: mean over the cameras that see the query.
//
// Mapping onto a gfx950 wavefront (64 lanes):
//   - one wave owns one output row (a query, or a (batch item, query) of the
//     SCA) and up to 8 heads at a time: lane group g = lane / 8 is head
//     hb + g, and lane j = lane % 8 of the group owns channels 4j..4j+3;
//   - staging: lane j of group g computes samples k = j, j+8, ... of its head
//     (softmax, location, the four corners) and writes one (row offset,
//     weight) pair per corner to LDS; corners outside the map get an offset
//     past the end of the image and weight 0;
//   - gather: the group walks its 4*L*P corner rows; per row its 8 lanes read
//     one 128-byte (fp32) or 64-byte (bf16) head row with one 16- or 8-byte
//     buffer load each (a skipped corner's load returns zeros and makes no
//     memory request) and accumulate weight * row into 4 fp32 registers.  A
//     wave-wide load instruction thus fetches one row for each of 8 heads; no
//     cross-lane reduction is needed, and the 8 groups' output chunks form
//     one contiguous 1 KB store per row;
//   - the sample geometry (x, y, floor, row index) is computed in fp64 so
//     that the interpolation fractions are exact to fp32 rounding;
//     interpolation weights, softmax and accumulation are fp32.
#include <climits>
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace msda {

constexpr int kHeadSlots = 8;      // heads per wave pass
constexpr int kSamplesPerLane = 8; // L*P <= 64 = 8 lanes x 8
constexpr int kUnroll = 8;         // corner rows in flight per lane
constexpr int kMaxWavesPerBlock = 4;
constexpr size_t kMaxBlockLds = 64 * 1024;
constexpr int kMaxLevels = 64;
constexpr uint32_t kSkip = 0x80000000u;  // beyond every image (images < 2^31 bytes)

struct Level {
  int W, H;
  long long start;
};

__host__ __device__ inline int rows_padded(int LP) { return (4 * LP + kUnroll - 1) / kUnroll * kUnroll; }
// per-head stride of the LDS staging area, in (offset, weight) pairs; odd, so
// that the 8 groups of a wave hit different LDS banks
__host__ __device__ inline int meta_stride(int LP) { return rows_padded(LP) + 1; }

__device__ inline float group_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 8));
  v = fmaxf(v, __shfl_xor(v, 2, 8));
  return fmaxf(v, __shfl_xor(v, 4, 8));
}
__device__ inline float group_sum(float v) {
  v += __shfl_xor(v, 1, 8);
  v += __shfl_xor(v, 2, 8);
  return v + __shfl_xor(v, 4, 8);
}

// Weights of the samples k = j + 8i of one head: probabilities as given, or
// softmax over the head's L*P logits, reduced across the 8 lanes of a group.
__device__ inline void head_weights(const float* __restrict__ w_row, bool head_ok, int LP, int j,
                                    bool logits, float (&alpha)[kSamplesPerLane]) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSamplesPerLane; ++i) {
    const int k = j + 8 * i;
    alpha[i] = (head_ok && k < LP) ? w_row[k] : 0.f;
    if (head_ok && k < LP) m = fmaxf(m, alpha[i]);
  }
  if (!logits) return;
  m = group_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kSamplesPerLane; ++i) {
    const int k = j + 8 * i;
    const float e = (head_ok && k < LP) ? expf(alpha[i] - m) : 0.f;
    alpha[i] = e;
    s += e;
  }
  s = group_sum(s);
  const float inv = head_ok ? 1.0f / s : 0.f;
#pragma unroll
  for (int i = 0; i < kSamplesPerLane; ++i) alpha[i] *= inv;
}

// The four corners of one sample at continuous level coordinate (x, y):
// (row offset in bytes within the image, alpha * bilinear weight), written
// to rows 4k .. 4k+3 of the group's staging area.
__device__ inline void stage_corners(uint2* __restrict__ rows, int k, double x, double y, float alpha,
                                     const Level& lv, bool live, int h, int nH, int Nv, uint32_t row_bytes) {
  // beyond [-2, size+1] every corner is outside anyway; clamping keeps the
  // integer conversions in range (and sends NaN to -2)
  x = fmin(fmax(x, -2.0), (double)lv.W + 1.0);
  y = fmin(fmax(y, -2.0), (double)lv.H + 1.0);
  const double xf = floor(x), yf = floor(y);
  const float fx = (float)(x - xf), fy = (float)(y - yf);
  const int ix = (int)xf, iy = (int)yf;
  const long long base = lv.start + (long long)iy * lv.W + ix;
  const float wx[2] = {1.f - fx, fx};
  const float wy[2] = {1.f - fy, fy};
#pragma unroll
  for (int dy = 0; dy < 2; ++dy) {
#pragma unroll
    for (int dx = 0; dx < 2; ++dx) {
      const int cx = ix + dx, cy = iy + dy;
      const long long pix = base + (long long)dy * lv.W + dx;
      const bool ok = live && cx >= 0 && cx < lv.W && cy >= 0 && cy < lv.H && pix >= 0 && pix < Nv;
      const uint32_t off = ok ? (uint32_t)((pix * nH + h) * (long long)row_bytes) : kSkip;
      const float w = ok ? alpha * wx[dx] * wy[dy] : 0.f;
      rows[4 * k + 2 * dy + dx] = make_uint2(off, __float_as_uint(w));
    }
  }
}

// Accumulate weight * value row over the group's staged corner rows.
template <bool kBF16>
__device__ inline void gather_rows(const uint2* __restrict__ rows, int R, __amdgpu_buffer_rsrc_t img, int j,
                                   float4& acc) {
  const uint32_t lane_off = (uint32_t)j * (kBF16 ? 8u : 16u);
  for (int r = 0; r < R; r += kUnroll) {
    uint2 m[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) m[u] = rows[r + u];
    if constexpr (!kBF16) {
      float4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const auto raw = __builtin_amdgcn_raw_buffer_load_b128(img, m[u].x + lane_off, 0, 0);
        v[u] = make_float4(__uint_as_float(raw[0]), __uint_as_float(raw[1]), __uint_as_float(raw[2]),
                           __uint_as_float(raw[3]));
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float w = __uint_as_float(m[u].y);
        acc.x = fmaf(w, v[u].x, acc.x);
        acc.y = fmaf(w, v[u].y, acc.y);
        acc.z = fmaf(w, v[u].z, acc.z);
        acc.w = fmaf(w, v[u].w, acc.w);
      }
    } else {
      uint32_t lo[kUnroll], hi[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const auto raw = __builtin_amdgcn_raw_buffer_load_b64(img, m[u].x + lane_off, 0, 0);
        lo[u] = raw[0];
        hi[u] = raw[1];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float w = __uint_as_float(m[u].y);
        acc.x = fmaf(w, __uint_as_float(lo[u] << 16), acc.x);
        acc.y = fmaf(w, __uint_as_float(lo[u] & 0xffff0000u), acc.y);
        acc.z = fmaf(w, __uint_as_float(hi[u] << 16), acc.z);
        acc.w = fmaf(w, __uint_as_float(hi[u] & 0xffff0000u), acc.w);
      }
    }
  }
}

__device__ inline void load_levels(const GatherArgs& a, Level* lv) {
  for (int l = threadIdx.x; l < a.L; l += blockDim.x) {
    const long long H = a.shapes[2 * l], W = a.shapes[2 * l + 1], s = a.starts[l];
    Level v;
    const bool ok = H >= 1 && W >= 1 && H <= (1 << 30) && W <= (1 << 30);
    v.W = ok ? (int)W : 0;  // an unusable level samples nothing
    v.H = ok ? (int)H : 0;
    v.start = s < -(1ll << 40) ? -(1ll << 40) : (s > (1ll << 40) ? (1ll << 40) : s);
    lv[l] = v;
  }
  __syncthreads();
}

__device__ inline int small_div(int k, float inv) { return (int)((k + 0.5f) * inv); }

// Padding rows past 4*L*P never change; write them as skipped rows.
__device__ inline void stage_padding(uint2* rows, int LP, int j) {
  const int r = 4 * LP + j;
  if (r < rows_padded(LP)) rows[r] = make_uint2(kSkip, 0u);
}

// ---------------------------------------------------------------------------
// plain operator and frame mean: item = (b, q); sources = frames f
// ---------------------------------------------------------------------------
template <bool kBF16>
__global__ __launch_bounds__(kMaxWavesPerBlock* kWave) void msda_gather_kernel(GatherArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Level* lv = reinterpret_cast<Level*>(smem);
  load_levels(a, lv);
  const int waves_per_block = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wave = uniform(threadIdx.x / kWave);
  const int g = lane / 8, j = lane % 8;
  const int RS = meta_stride(a.LP), R = rows_padded(a.LP);
  uint2* rows = reinterpret_cast<uint2*>(smem + sizeof(Level) * kMaxLevels) + ((size_t)wave * kHeadSlots + g) * RS;
  stage_padding(rows, a.LP, j);
  const uint32_t row_bytes = kBF16 ? 64u : 128u;

  XcdSplit split(a.B * a.Nq, waves_per_block);
  for (int64_t item = split.begin; item < split.end; item += split.stride) {
    const int64_t b = item / a.Nq, q = item % a.Nq;
    for (int hb = 0; hb < a.nH; hb += kHeadSlots) {
      const int h = hb + g;
      const bool head_ok = h < a.nH;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int f = 0; f < a.F; ++f) {
        const int64_t img_index = b * a.F + f;
        const int64_t src_row = (img_index * a.Nq + q) * a.nH + (head_ok ? h : 0);
        float alpha[kSamplesPerLane];
        head_weights(a.weights + src_row * a.LP, head_ok, a.LP, j, a.weight_logits != 0, alpha);
        const float2* loc = reinterpret_cast<const float2*>(a.loc) + src_row * a.LP;
#pragma unroll
        for (int i = 0; i < kSamplesPerLane; ++i) {
          const int k = j + 8 * i;
          if (k < a.LP) {
            const Level L = lv[small_div(k, a.inv_P)];
            const float2 s = head_ok ? loc[k] : make_float2(0.f, 0.f);
            stage_corners(rows, k, (double)s.x * L.W - 0.5, (double)s.y * L.H - 0.5, alpha[i], L, head_ok, h, a.nH,
                          a.Nv, row_bytes);
          }
        }
        wave_lds_sync();
        const auto img = make_rsrc(static_cast<const char*>(a.value) + img_index * (int64_t)a.image_bytes,
                                   a.image_bytes);
        gather_rows<kBF16>(rows, R, img, j, acc);
        wave_lds_sync();
      }
      if (head_ok) {
        if (a.F != 1) {
          const float n = (float)a.F;
          acc = make_float4(acc.x / n, acc.y / n, acc.z / n, acc.w / n);
        }
        float4* dst = reinterpret_cast<float4*>(a.out + ((item * a.nH + h) * 32)) + j;
        *dst = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// SCA: item = entry of the compacted (b, c, q) pair list; the pair of the
// first camera that sees q runs the whole query (all its cameras), so each
// query is written once, by one wave, and no atomics are needed.  Rows of
// queries that no camera sees are zeroed at the end.
// ---------------------------------------------------------------------------
template <bool kBF16>
__global__ __launch_bounds__(kMaxWavesPerBlock* kWave) void sca_gather_kernel(GatherArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Level* lv = reinterpret_cast<Level*>(smem);
  load_levels(a, lv);
  const int waves_per_block = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wave = uniform(threadIdx.x / kWave);
  const int g = lane / 8, j = lane % 8;
  const int RS = meta_stride(a.LP), R = rows_padded(a.LP);
  uint2* rows = reinterpret_cast<uint2*>(smem + sizeof(Level) * kMaxLevels) + ((size_t)wave * kHeadSlots + g) * RS;
  stage_padding(rows, a.LP, j);
  const uint32_t row_bytes = kBF16 ? 64u : 128u;
  const int nseg = (int)(a.B * a.Ncam);
  // the pair lists come from sca_compact; clamp so that a workspace that
  // never saw one cannot send a read out of bounds
  int64_t n_pairs = a.pair_offsets[nseg];
  n_pairs = n_pairs < 0 ? 0 : (n_pairs > a.B * a.Ncam * a.Nq ? a.B * a.Ncam * a.Nq : n_pairs);
  const uint32_t cam_bits = a.Ncam >= 32 ? 0xffffffffu : ((1u << a.Ncam) - 1u);

  XcdSplit split(n_pairs, waves_per_block);
  for (int64_t item = split.begin; item < split.end; item += split.stride) {
    // segment (b, c) of this pair: the last s with pair_offsets[s] <= item
    int lo = 0, hi = nseg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.pair_offsets[mid] <= item) lo = mid; else hi = mid;
    }
    const int64_t b = lo / a.Ncam;
    const int c_item = lo % a.Ncam;
    const int64_t q = a.pair_q[item];
    if (q < 0 || q >= a.Nq) continue;
    const int64_t bq = b * a.Nq + q;
    const uint32_t seen = a.cammask[bq] & cam_bits;
    if (seen == 0u || __builtin_ctz(seen) != c_item) continue;  // another pair of this query runs it
    const int hits = __popc(seen);

    for (int hb = 0; hb < a.nH; hb += kHeadSlots) {
      const int h = hb + g;
      const bool head_ok = h < a.nH;
      const int64_t src_row = bq * a.nH + (head_ok ? h : 0);
      // the query's weights and offsets serve every camera
      float alpha[kSamplesPerLane];
      head_weights(a.logits + src_row * a.LP, head_ok, a.LP, j, true, alpha);
      float2 off[kSamplesPerLane];
      const float2* off_row = reinterpret_cast<const float2*>(a.offsets) + src_row * a.LP;
#pragma unroll
      for (int i = 0; i < kSamplesPerLane; ++i) {
        const int k = j + 8 * i;
        off[i] = (head_ok && k < a.LP) ? off_row[k] : make_float2(0.f, 0.f);
      }
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (uint32_t rest = seen; rest != 0u; rest &= rest - 1u) {
        const int c = __builtin_ctz(rest);
        const float2* rho = reinterpret_cast<const float2*>(a.rp) + ((c * a.B + b) * a.Nq + q) * a.D;
#pragma unroll
        for (int i = 0; i < kSamplesPerLane; ++i) {
          const int k = j + 8 * i;
          if (k < a.LP) {
            const Level L = lv[small_div(k, a.inv_P)];
            const int m = k - a.D * small_div(k, a.inv_D);  // anchor k mod D (P is a multiple of D)
            const float2 r = rho[m];
            // x = W*(rho_x + dx/W) - 1/2 = W*rho_x + dx - 1/2, evaluated in fp64
            const double x = (double)r.x * L.W + (double)off[i].x - 0.5;
            const double y = (double)r.y * L.H + (double)off[i].y - 0.5;
            stage_corners(rows, k, x, y, alpha[i], L, head_ok, h, a.nH, a.Nv, row_bytes);
          }
        }
        wave_lds_sync();
        const auto img = make_rsrc(static_cast<const char*>(a.value) + (b * a.Ncam + c) * (int64_t)a.image_bytes,
                                   a.image_bytes);
        gather_rows<kBF16>(rows, R, img, j, acc);
        wave_lds_sync();
      }
      if (head_ok) {
        if (hits > 1) {
          const float n = (float)hits;
          acc = make_float4(acc.x / n, acc.y / n, acc.z / n, acc.w / n);
        }
        float4* dst = reinterpret_cast<float4*>(a.out + ((bq * a.nH + h) * 32)) + j;
        *dst = acc;
      }
    }
  }

  // queries no camera sees are on no pair list: their rows are zero
  const int64_t row4 = (int64_t)a.nH * 8;
  const int64_t waves = (int64_t)gridDim.x * waves_per_block;
  for (int64_t bq = (int64_t)blockIdx.x * waves_per_block + wave; bq < a.B * a.Nq; bq += waves) {
    if ((a.cammask[bq] & cam_bits) != 0u) continue;
    float4* dst = reinterpret_cast<float4*>(a.out + bq * a.nH * 32);
    for (int64_t e = lane; e < row4; e += kWave) dst[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

static size_t smem_bytes(int LP, int waves) {
  return sizeof(Level) * kMaxLevels + sizeof(uint2) * (size_t)waves * kHeadSlots * meta_stride(LP);
}

// Waves per block: as many as fit the 64 KB block LDS budget (4, or 2 for
// L*P above 32).
static int block_waves(int LP) {
  int w = kMaxWavesPerBlock;
  while (w > 1 && smem_bytes(LP, w) > kMaxBlockLds) w /= 2;
  return w;
}

// Blocks for n_items (an upper bound when the count lives on the device):
// at most blocks_per_cu per compute unit, a multiple of the die count.
static unsigned grid_for(int64_t n_items, int waves, int blocks_per_cu) {
  int64_t need = (n_items + waves - 1) / waves;
  const int64_t cap = (int64_t)device_cus() * blocks_per_cu;
  if (need > cap) need = cap;
  if (need < 1) need = 1;
  return (unsigned)((need + kXcds - 1) / kXcds * kXcds);
}

hipError_t launch_msda_gather(const GatherArgs& a, hipStream_t stream) {
  const int waves = block_waves(a.LP);
  const unsigned grid = grid_for(a.B * a.Nq, waves, 8 * kMaxWavesPerBlock / waves);
  const size_t smem = smem_bytes(a.LP, waves);
  if (a.bf16)
    msda_gather_kernel<true><<<grid, waves * kWave, smem, stream>>>(a);
  else
    msda_gather_kernel<false><<<grid, waves * kWave, smem, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_sca_gather(const GatherArgs& a, hipStream_t stream) {
  const int waves = block_waves(a.LP);
  const unsigned grid = grid_for(a.B * a.Ncam * a.Nq, waves, 8 * kMaxWavesPerBlock / waves);
  const size_t smem = smem_bytes(a.LP, waves);
  if (a.bf16)
    sca_gather_kernel<true><<<grid, waves * kWave, smem, stream>>>(a);
  else
    sca_gather_kernel<false><<<grid, waves * kWave, smem, stream>>>(a);
  return hipGetLastError();
}

}  // namespace msda
