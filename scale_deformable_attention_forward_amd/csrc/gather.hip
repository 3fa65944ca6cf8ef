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

// staged (offset, weight) slots of one head: 4 per sample, the count
// rounded up to whole load batches (kBatch slots; 2 * kBatch in the
// head-pair layout, where a load takes two slots, one per corner of a pair)
__host__ __device__ inline int rows_padded(int LP, bool pairs = false) {
  const int q = pairs ? 2 * kBatch : kBatch;
  return (4 * LP + q - 1) / q * q;
}
// per-head stride of the LDS staging area, in (offset, weight) slots; odd, so
// that the 8 groups of a wave hit different LDS banks
__host__ __device__ inline int meta_stride(int LP, bool pairs = false) { return rows_padded(LP, pairs) + 1; }

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

// The same four corners for a value in the head-pair layout (per image
// [nH][Nv][2][32] bf16: line (h, p) of 128 bytes holds pixel p of head h in
// its left half and pixel p + 1 in its right half), as two x-adjacent pairs:
// c[2*dy] = corner A = (x0, y0 + dy), c[2*dy + 1] = corner B = (x0 + 1,
// y0 + dy), each (byte offset of the corner's 64 bytes, weight).  B is read
// from the right half of A's line when A is inside the map (one line for the
// pair), else from the left half of its own line.
__device__ inline void sample_pairs(uint2 (&c)[4], double x, double y, float alpha, const Level& lv, bool live,
                                    int h, int Nv) {
  x = fmin(fmax(x, -2.0), (double)lv.W + 1.0);
  y = fmin(fmax(y, -2.0), (double)lv.H + 1.0);
  const double xf = floor(x), yf = floor(y);
  const float fx = (float)(x - xf), fy = (float)(y - yf);
  const int ix = (int)xf, iy = (int)yf;
  const long long base = lv.start + (long long)iy * lv.W + ix;
  const float wx[2] = {1.f - fx, fx};
  const float wy[2] = {1.f - fy, fy};
  const long long head = (long long)h * Nv;
#pragma unroll
  for (int dy = 0; dy < 2; ++dy) {
    const int cy = iy + dy;
    const long long pa = base + (long long)dy * lv.W, pb = pa + 1;
    const bool row_ok = live && cy >= 0 && cy < lv.H;
    const bool ok_a = row_ok && ix >= 0 && ix < lv.W && pa >= 0 && pa < Nv;
    const bool ok_b = row_ok && ix + 1 >= 0 && ix + 1 < lv.W && pb >= 0 && pb < Nv;
    const uint32_t line_a = (uint32_t)((head + pa) * 128), line_b = (uint32_t)((head + pb) * 128);
    c[2 * dy] = ok_a ? make_uint2(line_a, __float_as_uint(alpha * wx[0] * wy[dy])) : make_uint2(kSkip, 0u);
    c[2 * dy + 1] = ok_b ? make_uint2(ok_a ? line_a + 64u : line_b, __float_as_uint(alpha * wx[1] * wy[dy]))
                         : make_uint2(kSkip, 0u);
  }
}

// Checked builds: a staged corner (byte offset within its image) names a
// pixel of its sample's level, in head h's row (or, in the head-pair layout,
// head h's line of pixel p, whose right half holds pixel p + 1).
template <bool kPairs>
__device__ inline bool corner_in_level(uint32_t off, const Level& lv, int h, int nH, int Nv, uint32_t row_bytes) {
  long long pix;
  if constexpr (kPairs) {
    const uint32_t part = off % 128u;
    if (part != 0u && part != 64u) return false;
    pix = (long long)(off / 128u) - (long long)h * Nv + (part != 0u ? 1 : 0);
  } else {
    const long long row = off / row_bytes;
    if (off % row_bytes != 0u || row % nH != h) return false;
    pix = row / nH;
  }
  return pix >= lv.start && pix < lv.start + (long long)lv.W * lv.H && pix < Nv;
}

// Write the four corner rows of the group's live samples densely into `rows`
// (sample order, then lane order: a ballot per sample places each lane) and
// pad every group of the wave with skipped rows up to
// the wave's largest count rounded up to kBatch.  Returns that row count
// (the same in every lane).  Dead samples cost no row at all.  where(i)
// gives sample i's level index and the byte offset of its image within the
// buffer the gather reads (non-zero when one buffer holds several frames).
// With kPairs, the slots are sample_pairs' (A, B) per pair and the count
// is rounded up to 2 * kBatch.
template <int kSPL, typename Where, bool kPairs = false>
__device__ inline int stage_rows(uint2* __restrict__ rows, const double (&xs)[kSPL], const double (&ys)[kSPL],
                                 const float (&alpha)[kSPL], uint32_t live, const Level* lv, Where where, int j,
                                 int h, int nH, int Nv, uint32_t row_bytes) {
  // per sample, the group's lanes that hold it live
  const int gbase = (int)(threadIdx.x % kWave) & ~7;  // the group's first lane
  uint32_t group_live[kSPL];
  int group_total = 0;
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    group_live[i] = (uint32_t)(__ballot((live >> i) & 1u) >> gbase) & 0xffu;
    group_total += 4 * __popc(group_live[i]);
  }
  int wave_max = group_total;
  wave_max = max(wave_max, __shfl_xor(wave_max, 8));
  wave_max = max(wave_max, __shfl_xor(wave_max, 16));
  wave_max = max(wave_max, __shfl_xor(wave_max, 32));
  constexpr int q = kPairs ? 2 * kBatch : kBatch;
  const int R = (wave_max + q - 1) / q * q;
  // rows in sample order, then lane order: all lanes' live sample 0, then
  // sample 1, ... (for the SCA's and the DETR encoder's L*P = 32 and 16,
  // level by level).  With the group totals from the same ballots instead
  // of a shuffle prefix sum: 4% faster than lane order on the DETR encoder
  // and on the batch-4 SCA with a head-pair value, the same elsewhere.
  int base = 0;
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    const int pos = base + 4 * __popc(group_live[i] & ((1u << j) - 1u));
    base += 4 * __popc(group_live[i]);
    if ((live >> i) & 1u) {
      const int2 at = where(i);
      uint2 c[4];
      if constexpr (kPairs)
        sample_pairs(c, xs[i], ys[i], alpha[i], lv[at.x], true, h, Nv);
      else
        sample_corners(c, xs[i], ys[i], alpha[i], lv[at.x], true, h, nH, Nv, row_bytes);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        MSDA_CHECK(kCheckGatherRow, c[t].x == kSkip || corner_in_level<kPairs>(c[t].x, lv[at.x], h, nH, Nv, row_bytes));
        // skipped corners keep their offset past every image
        if (c[t].x != kSkip) c[t].x += (uint32_t)at.y;
        rows[pos + t] = c[t];
      }
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
  // one batch per iteration: unrolled further, the loads in flight take
  // registers that the occupancy needs
#pragma nounroll
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

// The head-pair layout's gather: R staged slots (a multiple of 2 * kBatch)
// hold R / 2 corner pairs (A, B).  Lanes j < 4 read corner A's channels
// 8j..8j+7, lanes j >= 4 corner B's channels 8(7-j)..8(7-j)+7, 16 bytes
// each, so that one wave-wide load fetches both corners of a pair for 8
// heads, mostly from one 128-byte line per head.  Lanes j and 7 - j
// accumulate the same 8 channels (from the two corners); pair_total() adds
// them up.  The wave raises its issue priority for the loop: the head-pair
// kernels keep the vector ALUs busier than the row layouts do (their staging
// writes two entries per sample and packs corner pairs), and a wave that
// holds loads to issue then goes first (2.5% on the batch-4 bf16 layer's
// gather; the row layouts measured no better with it).
__device__ inline void gather_pairs(const uint2* __restrict__ rows, int R, __amdgpu_buffer_rsrc_t img, int j,
                                    float (&acc)[8]) {
  const bool left = j < 4;
  const uint32_t lane_off = (uint32_t)(left ? j : 7 - j) * 16u;
  const int half = left ? 0 : 1;
  __builtin_amdgcn_s_setprio(1);
#pragma nounroll
  for (int r = 0; r < R; r += 2 * kBatch) {
    uint2 m[kBatch];
    uint32_t d[kBatch][4];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) m[u] = rows[r + 2 * u + half];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const auto raw = __builtin_amdgcn_raw_buffer_load_b128(img, m[u].x + lane_off, 0, 0);
      d[u][0] = raw[0];
      d[u][1] = raw[1];
      d[u][2] = raw[2];
      d[u][3] = raw[3];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = __uint_as_float(m[u].y);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = fmaf(w, __uint_as_float(d[u][k] << 16), acc[2 * k]);
        acc[2 * k + 1] = fmaf(w, __uint_as_float(d[u][k] & 0xffff0000u), acc[2 * k + 1]);
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// Sum of lanes j and 7 - j (the two corners' shares of the same channels),
// in both; returns this lane's 4 output channels and their float4 index in
// the head's row: lane j < 4 channels 8j..8j+3, lane j >= 4 channels
// 8(7-j)+4..8(7-j)+7.
__device__ inline float4 pair_total(float (&acc)[8], int j, int& at) {
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] += dpp<kDppHalfMirror>(acc[k]);
  const bool left = j < 4;
  at = left ? 2 * j : 2 * (7 - j) + 1;
  return left ? make_float4(acc[0], acc[1], acc[2], acc[3]) : make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// v / n: a multiplication by the exact reciprocal when n is a power of two
// (the same result, without the division's instruction sequence)
__device__ inline float4 scaled(float4 v, int n) {
  if (n <= 1) return v;
  if ((n & (n - 1)) == 0) {
    const float r = 1.0f / (float)n;
    return make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
  }
  const float f = (float)n;
  return make_float4(v.x / f, v.y / f, v.z / f, v.w / f);
}

// ---------------------------------------------------------------------------
// plain operator and frame mean: item = (b, q); sources = frames f
// ---------------------------------------------------------------------------
// The operator's work items (b, q) for one wave, in order: the queries in
// index order, or, with a plan from msda_plan, batch item by batch item in
// the plan's locality order.  Each die takes a contiguous eighth of a batch
// item's items.  next() returns the next item, or -1 after the last; plan
// entries outside [0, B*Nq) are skipped, so a foreign plan never sends a
// read out of bounds (its queries' rows are then left unwritten).
struct MsdaWalk {
  const int32_t* plan;
  int64_t n, Nq, B;
  int64_t i, end, stride, lo, bi;
  int waves_per_block;
  __device__ MsdaWalk(const GatherArgs& a, int wpb)
      : plan(a.plan), n(a.B * a.Nq), Nq(a.Nq), B(a.B), lo(0), bi(0), waves_per_block(wpb) {
    const XcdSplit s(plan ? Nq : n, wpb);
    i = s.begin - s.stride;
    end = s.end;
    stride = s.stride;
  }
  __device__ int64_t next() {
    for (;;) {
      i += stride;
      if (i < end) {
        if (!plan) return i;
        const int64_t item = uniform((int64_t)plan[lo + i]);
        MSDA_CHECK(kCheckListEntry, item >= lo && item < lo + Nq);  // batch item bi's entries name its queries
        if (item >= 0 && item < n) return item;
        continue;
      }
      if (!plan || ++bi >= B) return -1;
      const XcdSplit s(Nq, waves_per_block);
      lo = bi * Nq;
      i = s.begin - s.stride;
      end = s.end;
      stride = s.stride;
    }
  }
};

// item = b * Nq + q (a 32-bit division when both fit, as they do in practice)
__device__ inline void split_item(int64_t item, int64_t Nq, int64_t& b, int64_t& q) {
  if (item <= 0x7fffffff && Nq <= 0x7fffffff) {
    const uint32_t bb = (uint32_t)item / (uint32_t)Nq;
    b = bb;
    q = item - (int64_t)bb * Nq;
  } else {
    b = item / Nq;
    q = item - b * Nq;
  }
}

// One unit of the all-frames-in-one-pass operator, (item, head pass hb), as
// one lane reads it: the raw weight (or logit) and the location of its
// samples t = j + 8i of head hb + g (zero for none).
template <int kSPL>
struct FlatUnit {
  float w[kSPL];
  float2 s[kSPL];
};

// Frame of the lane's samples: frame f = t / LP holds samples
// [f*LP, (f+1)*LP) of a head; -1 for no sample.
template <int kSPL>
__device__ inline void flat_frames(bool head_ok, int FLP, float inv_LP, int j, int (&fr)[kSPL]) {
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    const int t = j + 8 * i;
    fr[i] = head_ok && t < FLP ? small_div(t, inv_LP) : -1;
  }
}

// Issue the loads of a unit's inputs (consumed one unit later, so that they
// arrive while the wave gathers).
template <int kSPL>
__device__ inline void load_flat_unit(FlatUnit<kSPL>& u, const GatherArgs& a, int64_t b, int64_t q, int hb, int g,
                                      int j) {
  const int h = hb + g;
  const bool head_ok = h < a.nH;
  const int64_t src_row = (b * a.F * a.Nq + q) * a.nH + (head_ok ? h : 0);  // frame 0
  const int64_t stride = a.Nq * a.nH * a.LP;                                // elements per frame
  const float* w0 = a.weights + src_row * a.LP;
  const float2* s0 = reinterpret_cast<const float2*>(a.loc) + src_row * a.LP;
  int fr[kSPL];
  flat_frames<kSPL>(head_ok, a.F * a.LP, a.inv_LP, j, fr);
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    const int f = fr[i];
    const int64_t at = f >= 0 ? f * stride + (j + 8 * i - f * a.LP) : 0;
    u.w[i] = f >= 0 ? w0[at] : 0.f;
    u.s[i] = f >= 0 ? s0[at] : make_float2(0.f, 0.f);
  }
}

// The unit's sample weights: probabilities as given, or a softmax per frame
// over that frame's L*P logits, reduced over the lanes of the group that
// hold its samples.
template <int kSPL>
__device__ inline void flat_weights(const FlatUnit<kSPL>& u, const int (&fr)[kSPL], int F, bool logits,
                                    float (&alpha)[kSPL]) {
#pragma unroll
  for (int i = 0; i < kSPL; ++i) alpha[i] = u.w[i];
  if (!logits) return;
  for (int f = 0; f < F; ++f) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kSPL; ++i)
      if (fr[i] == f) m = fmaxf(m, alpha[i]);
    m = group_max(m);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kSPL; ++i)
      if (fr[i] == f) {
        alpha[i] = expf(alpha[i] - m);
        sum += alpha[i];
      }
    const float inv = 1.0f / group_sum(sum);
#pragma unroll
    for (int i = 0; i < kSPL; ++i)
      if (fr[i] == f) alpha[i] *= inv;
  }
}

// kFlat: all F frames' samples of a head are staged together and gathered
// in one pass through one buffer descriptor spanning the batch item's F
// images (needs F*L*P <= 8*kSPL and F images under 2^31 bytes); the wave
// loads the next unit's inputs before it stages and gathers the current
// one.  Otherwise frame by frame.  kPairs: bf16 value in the head-pair
// layout, as in the SCA kernel.
template <bool kBF16, int kSPL, bool kFlat, bool kPairs>
__global__ __launch_bounds__(kMaxWavesPerBlock* kWave) void msda_gather_kernel(GatherArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Level* lv = reinterpret_cast<Level*>(smem);
  load_levels(a.shapes, a.starts, a.L, lv);
  const int waves_per_block = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wave = uniform((int)(threadIdx.x / kWave));
  const int g = lane / 8, j = lane % 8;
  uint2* rows = reinterpret_cast<uint2*>(smem + sizeof(Level) * kMaxLevels) +
                ((size_t)wave * kHeadSlots + g) * meta_stride(kFlat ? a.F * a.LP : a.LP, kPairs);
  const uint32_t row_bytes = kBF16 ? 64u : 128u;
  MsdaWalk walk(a, waves_per_block);

  if constexpr (kFlat) {
    int64_t item = walk.next(), b = 0, q = 0;
    int hb = 0;
    FlatUnit<kSPL> cur;
    if (item >= 0) {
      split_item(item, a.Nq, b, q);
      load_flat_unit<kSPL>(cur, a, b, q, hb, g, j);
    }
    while (item >= 0) {
      // the lane's group and channel slot, re-derived in every unit so that
      // the compiler does not hold their loop-invariant consequences in
      // registers across the gather (which the occupancy needs)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int g = ln / 8, j = ln % 8;
      // the next unit: its inputs are in flight while this one runs
      int64_t n_item = item, nb = b, nq = q;
      int n_hb = hb + kHeadSlots;
      if (n_hb >= a.nH) {
        n_hb = 0;
        n_item = walk.next();
        if (n_item >= 0) split_item(n_item, a.Nq, nb, nq);
      }
      FlatUnit<kSPL> nxt;
      if (n_item >= 0) load_flat_unit<kSPL>(nxt, a, nb, nq, n_hb, g, j);

      const int h = hb + g;
      int fr[kSPL];
      flat_frames<kSPL>(h < a.nH, a.F * a.LP, a.inv_LP, j, fr);
      float alpha[kSPL];
      flat_weights<kSPL>(cur, fr, a.F, a.weight_logits != 0, alpha);
      double xs[kSPL], ys[kSPL];
      uint32_t live = 0u;
#pragma unroll
      for (int i = 0; i < kSPL; ++i) {
        const int f = fr[i] < 0 ? 0 : fr[i];
        const int k = j + 8 * i - f * a.LP;
        const Level L = lv[fr[i] < 0 ? 0 : small_div(k, a.inv_P)];
        xs[i] = (double)cur.s[i].x * L.W - 0.5;
        ys[i] = (double)cur.s[i].y * L.H - 0.5;
        if (fr[i] >= 0 && sample_live(xs[i], ys[i], L)) live |= 1u << i;
      }
      const int LP = a.LP;
      const float inv_LP = a.inv_LP, inv_P = a.inv_P;
      const uint32_t image_bytes = a.image_bytes;
      auto where = [&](int i) {
        const int t = j + 8 * i;
        const int f = small_div(t, inv_LP);
        return make_int2(small_div(t - f * LP, inv_P), (int)(f * image_bytes));
      };
      const int R = stage_rows<kSPL, decltype(where), kPairs>(rows, xs, ys, alpha, live, lv, where, j, h, a.nH,
                                                                a.Nv, row_bytes);
      wave_lds_sync();
      const auto img = make_rsrc(static_cast<const char*>(a.value) + b * a.F * (int64_t)a.image_bytes,
                                 (uint32_t)(a.F * (int64_t)a.image_bytes));
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      int at = j;
      if constexpr (kPairs) {
        float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        gather_pairs(rows, R, img, j, acc8);
        acc = pair_total(acc8, j, at);
      } else {
        gather_rows<kBF16>(rows, R, img, j, acc);
      }
      wave_lds_sync();
      if (h < a.nH) reinterpret_cast<float4*>(a.out + ((item * a.nH + h) * 32))[at] = scaled(acc, a.F);
      item = n_item;
      hb = n_hb;
      b = nb;
      q = nq;
      cur = nxt;
    }
  } else {
    for (int64_t item = walk.next(); item >= 0; item = walk.next()) {
      int64_t b, q;
      split_item(item, a.Nq, b, q);
      for (int hb = 0; hb < a.nH; hb += kHeadSlots) {
        const int h = hb + g;
        const bool head_ok = h < a.nH;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // head-pair layout
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
          const float inv_P = a.inv_P;
          auto where = [&](int i) { return make_int2(small_div(j + 8 * i, inv_P), 0); };
          const int R = stage_rows<kSPL, decltype(where), kPairs>(rows, xs, ys, alpha, live, lv, where, j, h, a.nH,
                                                                    a.Nv, row_bytes);
          wave_lds_sync();
          const auto img = make_rsrc(static_cast<const char*>(a.value) + img_index * (int64_t)a.image_bytes,
                                     a.image_bytes);
          if constexpr (kPairs)
            gather_pairs(rows, R, img, j, acc8);
          else
            gather_rows<kBF16>(rows, R, img, j, acc);
          wave_lds_sync();
        }
        int at = j;
        if constexpr (kPairs) acc = pair_total(acc8, j, at);
        if (head_ok) reinterpret_cast<float4*>(a.out + ((item * a.nH + h) * 32))[at] = scaled(acc, a.F);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// SCA: item = entry of the work list sca_compact builds (every seen query
// once, grouped by first camera and image tile); the wave runs all cameras
// of its query and averages them in registers, so each query is written
// once, by one wave, and no atomics are needed.  Rows of queries that no
// camera sees are zeroed first.
// ---------------------------------------------------------------------------
// For L*P <= 32 the kernel is held to 128 VGPRs, 4 waves per SIMD (the LDS
// allows 4): the fp32, bf16 and head-pair variants fit (126, 116, 128).
// kPairs: bf16 value in the head-pair layout (sample_pairs, gather_pairs).
template <bool kBF16, int kSPL, bool kPairs>
__global__ __launch_bounds__(kMaxWavesPerBlock* kWave, kSPL == 4 ? 4 : 1) void sca_gather_kernel(GatherArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Level* lv = reinterpret_cast<Level*>(smem);
  load_levels(a.shapes, a.starts, a.L, lv);
  const int waves_per_block = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wave = uniform((int)(threadIdx.x / kWave));
  const int g = lane / 8, j = lane % 8;
  uint2* rows = reinterpret_cast<uint2*>(smem + sizeof(Level) * kMaxLevels) +
                ((size_t)wave * kHeadSlots + g) * meta_stride(a.LP, kPairs);
  const uint32_t row_bytes = kBF16 ? 64u : 128u;
  const int64_t n_queries = a.B * a.Nq;
  const uint32_t cam_bits = a.Ncam >= 32 ? 0xffffffffu : ((1u << a.Ncam) - 1u);

  // Queries no camera sees are on no work list: their rows are zero.  One
  // wave-wide mask load covers 64 queries, before the wave's gathers (a loop
  // of one query per wave after them waited for each load in turn, on the
  // kernel's tail).
  {
    const int64_t row4 = (int64_t)a.nH * 8;  // float4s per output row
    const int64_t n_waves = (int64_t)gridDim.x * waves_per_block;
    for (int64_t q0 = ((int64_t)blockIdx.x * waves_per_block + wave) * kWave; q0 < n_queries; q0 += n_waves * kWave) {
      const bool unseen = q0 + lane < n_queries && (a.cammask[q0 + lane] & cam_bits) == 0u;
      for (uint64_t m = __ballot(unseen); m != 0ull; m &= m - 1ull) {
        float4* dst = reinterpret_cast<float4*>(a.out + (q0 + __builtin_ctzll(m)) * a.nH * 32);
        for (int64_t e = lane; e < row4; e += kWave) dst[e] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }

  // Batch item by batch item, each die takes its share of the item's work
  // list (contiguous, of equal estimated cost), so the dies share one item's
  // value maps at a time.  The list and the shares come from sca_compact;
  // clamping keeps a workspace that never saw one from sending a read out
  // of bounds.
  for (int64_t bi = 0; bi < a.B; ++bi) {
  const DieShare split(a.die_bounds + bi * kDieBounds, n_queries, waves_per_block);
  for (int64_t item = split.begin; item < split.end; item += split.stride) {
    const int64_t bq = uniform((int64_t)a.order[item]);
    MSDA_CHECK(kCheckListEntry, bq >= bi * a.Nq && bq < (bi + 1) * a.Nq);
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
      float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // head-pair layout
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
        const float inv_P = a.inv_P;
        auto level_of = [&](int i) { return make_int2(small_div(j + 8 * i, inv_P), 0); };
        const int R = stage_rows<kSPL, decltype(level_of), kPairs>(rows, xs, ys, alpha, live, lv, level_of, j, h,
                                                                     a.nH, a.Nv, row_bytes);
        wave_lds_sync();
        const auto img = make_rsrc(static_cast<const char*>(a.value) + (b * a.Ncam + c) * (int64_t)a.image_bytes,
                                   a.image_bytes);
        if constexpr (kPairs)
          gather_pairs(rows, R, img, j, acc8);
        else
          gather_rows<kBF16>(rows, R, img, j, acc);
        wave_lds_sync();
      }
      int at = j;
      if constexpr (kPairs) acc = pair_total(acc8, j, at);
      if (head_ok) reinterpret_cast<float4*>(a.out + ((bq * a.nH + h) * 32))[at] = scaled(acc, __popc(seen));
    }
  }
  }

}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static size_t smem_bytes(int LP, int waves, bool pairs = false) {
  return sizeof(Level) * kMaxLevels + sizeof(uint2) * (size_t)waves * kHeadSlots * meta_stride(LP, pairs);
}

// Waves per block: as many as fit the 64 KB block LDS budget (4, or 2 for
// L*P above 32).
static int block_waves(int LP, bool pairs = false) {
  int w = kMaxWavesPerBlock;
  while (w > 1 && smem_bytes(LP, w, pairs) > kMaxBlockLds) w /= 2;
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

// The operator's kernel for kSPL samples per lane (8 * kSPL per head and pass).
template <int kSPL, bool kFlat>
static void launch_msda_spl(const GatherArgs& a, int waves, size_t smem, bool resident, hipStream_t stream) {
  if (a.pairs)
    launch(msda_gather_kernel<true, kSPL, kFlat, true>, a.B * a.Nq, waves, smem, resident, a, stream);
  else if (a.bf16)
    launch(msda_gather_kernel<true, kSPL, kFlat, false>, a.B * a.Nq, waves, smem, resident, a, stream);
  else
    launch(msda_gather_kernel<false, kSPL, kFlat, false>, a.B * a.Nq, waves, smem, resident, a, stream);
}

template <bool kFlat>
static void launch_msda_staged(const GatherArgs& a, int staged, int waves, size_t smem, bool resident,
                               hipStream_t stream) {
  // as few samples per lane as the head's staged samples need: unused
  // sample slots still cost their (masked) staging instructions
  if (staged <= 8)
    launch_msda_spl<1, kFlat>(a, waves, smem, resident, stream);
  else if (staged <= 16)
    launch_msda_spl<2, kFlat>(a, waves, smem, resident, stream);
  else if (staged <= 32)
    launch_msda_spl<4, kFlat>(a, waves, smem, resident, stream);
  else
    launch_msda_spl<8, kFlat>(a, waves, smem, resident, stream);
}

hipError_t launch_msda_gather(const GatherArgs& a, hipStream_t stream) {
  // all frames in one pass when their samples fit one staging area and
  // their images one buffer descriptor (offset kSkip must lie beyond them)
  const bool flat = (int64_t)a.F * a.LP <= 64 && (int64_t)a.F * a.image_bytes < (int64_t)kSkip;
  const int staged = flat ? a.F * a.LP : a.LP;
  const bool pairs = a.pairs != 0;
  const int waves = block_waves(staged, pairs);
  const size_t smem = smem_bytes(staged, waves, pairs);
  // all waves resident, so that they sweep the (planned or given) order of
  // the queries together: measured against 8 blocks per compute unit (late
  // blocks balancing the tail), 0.0748 against 0.0782 ms on the temporal
  // workload, whose BEV-grid queries come in raster order, and 0.0873
  // against 0.0853 ms on the DETR encoder's randomly placed queries, which
  // are meant to go through a plan (0.065 ms)
  const bool resident = true;
  if (flat)
    launch_msda_staged<true>(a, staged, waves, smem, resident, stream);
  else
    launch_msda_staged<false>(a, staged, waves, smem, resident, stream);
  return hipGetLastError();
}

template <int kSPL>
static void launch_sca_spl(const GatherArgs& a, int waves, size_t smem, hipStream_t stream) {
  const int64_t n = a.B * a.Nq;
  if (a.pairs)
    launch(sca_gather_kernel<true, kSPL, true>, n, waves, smem, true, a, stream);
  else if (a.bf16)
    launch(sca_gather_kernel<true, kSPL, false>, n, waves, smem, true, a, stream);
  else
    launch(sca_gather_kernel<false, kSPL, false>, n, waves, smem, true, a, stream);
}

hipError_t launch_sca_gather(const GatherArgs& a, hipStream_t stream) {
  const bool pairs = a.pairs != 0;
  const int waves = block_waves(a.LP, pairs);
  const size_t smem = smem_bytes(a.LP, waves, pairs);
  if (a.LP <= 32)
    launch_sca_spl<4>(a, waves, smem, stream);
  else
    launch_sca_spl<8>(a, waves, smem, stream);
  return hipGetLastError();
}

}  // namespace msda
