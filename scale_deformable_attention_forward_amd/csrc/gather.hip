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
//     (softmax, location); samples with a corner that can lie inside the map
//     are live, and the four corners of each live sample become (row
//     offset, weight) pairs packed densely into the group's LDS area (prefix
//     sum over its 8 lanes), so samples entirely outside the map cost
//     nothing later;
//   - gather: all groups walk the same number of rows (the largest count in
//     the wave, rounded up to 8; short groups are padded with rows whose
//     offset lies past the image, which buffer loads turn into zeros without
//     a memory request).  Per row the group's 8 lanes read one 128-byte
//     (fp32) or 64-byte (bf16) head row with one 16- or 8-byte buffer load
//     each and accumulate weight * row into 4 fp32 registers.  A wave-wide
//     load thus fetches one row for each of 8 heads; no cross-lane reduction
//     is needed, and the 8 groups' output chunks form one contiguous store;
//   - the sample geometry (x, y, floor, row index) is computed in fp64 so
//     that the interpolation fractions are exact to fp32 rounding;
//     interpolation weights, softmax and accumulation are fp32.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"
#include "sampling.hpp"

namespace msda {

constexpr int kBatch = 8;  // corner rows per load batch
constexpr int kMaxWavesPerBlock = 4;

__host__ __device__ inline int rows_padded(int LP) { return (4 * LP + kBatch - 1) / kBatch * kBatch; }
// per-head stride of the LDS staging area, in (offset, weight) pairs; odd, so
// that the 8 groups of a wave hit different LDS banks
__host__ __device__ inline int meta_stride(int LP) { return rows_padded(LP) + 1; }

// The four corners of one sample at continuous level coordinate (x, y):
// (row offset in bytes within the image, alpha * bilinear weight), with
// offset kSkip for corners outside the level or outside [0, Nv).
__device__ inline void sample_corners(uint2 (&c)[4], double x, double y, float alpha, const Level& lv, bool live,
                                      int h, int nH, int Nv, uint32_t row_bytes) {
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
      c[2 * dy + dx] = ok ? make_uint2((uint32_t)((pix * nH + h) * (long long)row_bytes),
                                       __float_as_uint(alpha * wx[dx] * wy[dy]))
                          : make_uint2(kSkip, 0u);
    }
  }
}

// Write the four corner rows of the group's live samples densely into `rows`
// (lane order, then sample order; a prefix sum over the group's 8 lanes
// places each lane) and pad every group of the wave with skipped rows up to
// the wave's largest count rounded up to kBatch.  Returns that row count
// (the same in every lane).  Dead samples cost no row at all.
template <int kSPL>
__device__ inline int stage_rows(uint2* __restrict__ rows, const double (&xs)[kSPL], const double (&ys)[kSPL],
                                 const float (&alpha)[kSPL], uint32_t live, const Level* lv, float inv_P, int j,
                                 int h, int nH, int Nv, uint32_t row_bytes) {
  const int n = 4 * __popc(live);
  int incl = n;
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    const int v = __shfl_up(incl, d, 8);
    if (j >= d) incl += v;
  }
  const int group_total = __shfl(incl, 7, 8);
  int wave_max = group_total;
  wave_max = max(wave_max, __shfl_xor(wave_max, 8));
  wave_max = max(wave_max, __shfl_xor(wave_max, 16));
  wave_max = max(wave_max, __shfl_xor(wave_max, 32));
  const int R = (wave_max + kBatch - 1) / kBatch * kBatch;
  int pos = incl - n;
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    if ((live >> i) & 1u) {
      const Level L = lv[small_div(j + 8 * i, inv_P)];
      uint2 c[4];
      sample_corners(c, xs[i], ys[i], alpha[i], L, true, h, nH, Nv, row_bytes);
#pragma unroll
      for (int t = 0; t < 4; ++t) rows[pos + t] = c[t];
      pos += 4;
    }
  }
  for (int r = group_total + j; r < R; r += 8) rows[r] = make_uint2(kSkip, 0u);
  return uniform(R);
}

// Accumulate weight * value row over the group's R staged rows (R a
// multiple of kBatch), kBatch loads in flight per lane.
template <bool kBF16>
__device__ inline void gather_rows(const uint2* __restrict__ rows, int R, __amdgpu_buffer_rsrc_t img, int j,
                                   float4& acc) {
  const uint32_t lane_off = (uint32_t)j * (kBF16 ? 8u : 16u);
  for (int r = 0; r < R; r += kBatch) {
    uint2 m[kBatch];
    uint32_t d[kBatch][kBF16 ? 2 : 4];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) m[u] = rows[r + u];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if constexpr (kBF16) {
        const auto raw = __builtin_amdgcn_raw_buffer_load_b64(img, m[u].x + lane_off, 0, 0);
        d[u][0] = raw[0];
        d[u][1] = raw[1];
      } else {
        const auto raw = __builtin_amdgcn_raw_buffer_load_b128(img, m[u].x + lane_off, 0, 0);
        d[u][0] = raw[0];
        d[u][1] = raw[1];
        d[u][2] = raw[2];
        d[u][3] = raw[3];
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = __uint_as_float(m[u].y);
      if constexpr (kBF16) {
        acc.x = fmaf(w, __uint_as_float(d[u][0] << 16), acc.x);
        acc.y = fmaf(w, __uint_as_float(d[u][0] & 0xffff0000u), acc.y);
        acc.z = fmaf(w, __uint_as_float(d[u][1] << 16), acc.z);
        acc.w = fmaf(w, __uint_as_float(d[u][1] & 0xffff0000u), acc.w);
      } else {
        acc.x = fmaf(w, __uint_as_float(d[u][0]), acc.x);
        acc.y = fmaf(w, __uint_as_float(d[u][1]), acc.y);
        acc.z = fmaf(w, __uint_as_float(d[u][2]), acc.z);
        acc.w = fmaf(w, __uint_as_float(d[u][3]), acc.w);
      }
    }
  }
}

__device__ inline float4 scaled(float4 v, int n) {
  if (n <= 1) return v;
  const float f = (float)n;
  return make_float4(v.x / f, v.y / f, v.z / f, v.w / f);
}

// ---------------------------------------------------------------------------
// plain operator and frame mean: item = (b, q); sources = frames f
// ---------------------------------------------------------------------------
template <bool kBF16, int kSPL>
__global__ __launch_bounds__(kMaxWavesPerBlock* kWave) void msda_gather_kernel(GatherArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Level* lv = reinterpret_cast<Level*>(smem);
  load_levels(a.shapes, a.starts, a.L, lv);
  const int waves_per_block = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wave = uniform((int)(threadIdx.x / kWave));
  const int g = lane / 8, j = lane % 8;
  uint2* rows = reinterpret_cast<uint2*>(smem + sizeof(Level) * kMaxLevels) +
                ((size_t)wave * kHeadSlots + g) * meta_stride(a.LP);
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
        float alpha[kSPL];
        head_weights<kSPL>(a.weights + src_row * a.LP, head_ok, a.LP, j, a.weight_logits != 0, alpha);
        const float2* loc = reinterpret_cast<const float2*>(a.loc) + src_row * a.LP;
        double xs[kSPL], ys[kSPL];
        uint32_t live = 0u;
#pragma unroll
        for (int i = 0; i < kSPL; ++i) {
          const int k = j + 8 * i;
          const bool valid = head_ok && k < a.LP;
          const Level L = lv[valid ? small_div(k, a.inv_P) : 0];
          const float2 s = valid ? loc[k] : make_float2(0.f, 0.f);
          xs[i] = (double)s.x * L.W - 0.5;
          ys[i] = (double)s.y * L.H - 0.5;
          if (valid && sample_live(xs[i], ys[i], L)) live |= 1u << i;
        }
        const int R = stage_rows<kSPL>(rows, xs, ys, alpha, live, lv, a.inv_P, j, h, a.nH, a.Nv, row_bytes);
        wave_lds_sync();
        const auto img = make_rsrc(static_cast<const char*>(a.value) + img_index * (int64_t)a.image_bytes,
                                   a.image_bytes);
        gather_rows<kBF16>(rows, R, img, j, acc);
        wave_lds_sync();
      }
      if (head_ok) reinterpret_cast<float4*>(a.out + ((item * a.nH + h) * 32))[j] = scaled(acc, a.F);
    }
  }
}

// ---------------------------------------------------------------------------
// SCA: item = entry of the work list sca_compact builds (every seen query
// once, grouped by first camera and image tile); the wave runs all cameras
// of its query and averages them in registers, so each query is written
// once, by one wave, and no atomics are needed.  Rows of queries that no
// camera sees are zeroed at the end.
// ---------------------------------------------------------------------------
// For L*P <= 32 the kernel is held to 128 VGPRs, 4 waves per SIMD (the LDS
// allows 4): the fp32 variant then spills a few registers outside its load
// loop and still measures about 2% faster than at 133 VGPRs and 3 waves.
template <bool kBF16, int kSPL>
__global__ __launch_bounds__(kMaxWavesPerBlock* kWave, kSPL == 4 ? 4 : 1) void sca_gather_kernel(GatherArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Level* lv = reinterpret_cast<Level*>(smem);
  load_levels(a.shapes, a.starts, a.L, lv);
  const int waves_per_block = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wave = uniform((int)(threadIdx.x / kWave));
  const int g = lane / 8, j = lane % 8;
  uint2* rows = reinterpret_cast<uint2*>(smem + sizeof(Level) * kMaxLevels) +
                ((size_t)wave * kHeadSlots + g) * meta_stride(a.LP);
  const uint32_t row_bytes = kBF16 ? 64u : 128u;
  const int64_t n_queries = a.B * a.Nq;
  const uint32_t cam_bits = a.Ncam >= 32 ? 0xffffffffu : ((1u << a.Ncam) - 1u);

  // Batch item by batch item, each die takes an eighth of the item's work
  // list, so the dies share one item's value maps at a time.  The list comes
  // from sca_compact; clamping keeps a workspace that never saw one from
  // sending a read out of bounds.
  for (int64_t bi = 0; bi < a.B; ++bi) {
  int64_t lo = a.order_at[bi * a.order_stride], hi = a.order_at[(bi + 1) * a.order_stride];
  lo = lo < 0 ? 0 : (lo > n_queries ? n_queries : lo);
  hi = hi < lo ? lo : (hi > n_queries ? n_queries : hi);
  XcdSplit split(hi - lo, waves_per_block);
  for (int64_t item = lo + split.begin; item < lo + split.end; item += split.stride) {
    const int64_t bq = uniform((int64_t)a.order[item]);
    if (bq < 0 || bq >= n_queries) continue;
    const int64_t b = bq / a.Nq, q = bq % a.Nq;
    const uint32_t seen = uniform(a.cammask[bq] & cam_bits);
    if (seen == 0u) continue;

    for (int hb = 0; hb < a.nH; hb += kHeadSlots) {
      const int h = hb + g;
      const bool head_ok = h < a.nH;
      const int64_t src_row = bq * a.nH + (head_ok ? h : 0);
      // the query's weights and offsets serve every camera
      float alpha[kSPL];
      head_weights<kSPL>(a.logits + src_row * a.LP, head_ok, a.LP, j, true, alpha);
      float2 off[kSPL];
      const float2* off_row = reinterpret_cast<const float2*>(a.offsets) + src_row * a.LP;
#pragma unroll
      for (int i = 0; i < kSPL; ++i) {
        const int k = j + 8 * i;
        off[i] = (head_ok && k < a.LP) ? off_row[k] : make_float2(0.f, 0.f);
      }
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (uint32_t rest = seen; rest != 0u; rest &= rest - 1u) {
        const int c = __builtin_ctz(rest);
        const float2* rho = reinterpret_cast<const float2*>(a.rp) + ((c * a.B + b) * a.Nq + q) * a.D;
        double xs[kSPL], ys[kSPL];
        uint32_t live = 0u;
#pragma unroll
        for (int i = 0; i < kSPL; ++i) {
          const int k = j + 8 * i;
          const bool valid = head_ok && k < a.LP;
          const Level L = lv[valid ? small_div(k, a.inv_P) : 0];
          const int m = k - a.D * small_div(k, a.inv_D);  // anchor k mod D (P is a multiple of D)
          const float2 r = valid ? rho[m] : make_float2(0.f, 0.f);
          // x = W*(rho_x + dx/W) - 1/2 = W*rho_x + dx - 1/2, evaluated in fp64
          xs[i] = (double)r.x * L.W + (double)off[i].x - 0.5;
          ys[i] = (double)r.y * L.H + (double)off[i].y - 0.5;
          if (valid && sample_live(xs[i], ys[i], L)) live |= 1u << i;
        }
        const int R = stage_rows<kSPL>(rows, xs, ys, alpha, live, lv, a.inv_P, j, h, a.nH, a.Nv, row_bytes);
        wave_lds_sync();
        const auto img = make_rsrc(static_cast<const char*>(a.value) + (b * a.Ncam + c) * (int64_t)a.image_bytes,
                                   a.image_bytes);
        gather_rows<kBF16>(rows, R, img, j, acc);
        wave_lds_sync();
      }
      if (head_ok) reinterpret_cast<float4*>(a.out + ((bq * a.nH + h) * 32))[j] = scaled(acc, __popc(seen));
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

// Blocks for n_items (an upper bound when the count lives on the device),
// a multiple of the die count.
//   - SCA (resident_only): no more than the chip holds at once, so that every
//     block is resident from the start and all waves sweep the locality-
//     ordered work together.  A grid larger than that runs in rounds: a block
//     of the first round goes on to later batch items while the next round
//     starts on the first, and several items' value maps compete for L2.
//   - MSDA: up to 8 blocks of 4 waves per compute unit, more than are
//     resident: with few queries per wave, blocks that start late balance
//     the tail.
template <typename Kernel>
static unsigned grid_for(Kernel kernel, int64_t n_items, int waves, size_t smem, bool resident_only) {
  int per_cu = 8 * kMaxWavesPerBlock / waves;
  if (resident_only &&
      (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, waves * kWave, smem) != hipSuccess || per_cu < 1))
    per_cu = 1;
  int64_t need = (n_items + waves - 1) / waves;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  if (need > cap) need = cap;
  if (need < 1) need = 1;
  return (unsigned)((need + kXcds - 1) / kXcds * kXcds);
}

template <typename Kernel>
static void launch(Kernel kernel, int64_t n_items, int waves, size_t smem, bool resident_only, const GatherArgs& a,
                   hipStream_t stream) {
  kernel<<<grid_for(kernel, n_items, waves, smem, resident_only), waves * kWave, smem, stream>>>(a);
}

hipError_t launch_msda_gather(const GatherArgs& a, hipStream_t stream) {
  const int waves = block_waves(a.LP);
  const size_t smem = smem_bytes(a.LP, waves);
  const int64_t n = a.B * a.Nq;
  if (a.LP <= 32)
    launch(a.bf16 ? msda_gather_kernel<true, 4> : msda_gather_kernel<false, 4>, n, waves, smem, false, a, stream);
  else
    launch(a.bf16 ? msda_gather_kernel<true, 8> : msda_gather_kernel<false, 8>, n, waves, smem, false, a, stream);
  return hipGetLastError();
}

hipError_t launch_sca_gather(const GatherArgs& a, hipStream_t stream) {
  const int waves = block_waves(a.LP);
  const size_t smem = smem_bytes(a.LP, waves);
  const int64_t n = a.B * a.Nq;
  if (a.LP <= 32)
    launch(a.bf16 ? sca_gather_kernel<true, 4> : sca_gather_kernel<false, 4>, n, waves, smem, true, a, stream);
  else
    launch(a.bf16 ? sca_gather_kernel<true, 8> : sca_gather_kernel<false, 8>, n, waves, smem, true, a, stream);
  return hipGetLastError();
}

}  // namespace msda
