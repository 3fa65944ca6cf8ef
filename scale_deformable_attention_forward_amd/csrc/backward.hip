// Backward pass of multi-scale deformable attention and of BEVFormer's
// spatial cross-attention: gradients with respect to the value maps, the
// sampling locations (for SCA, the offsets in cells) and the attention
// weights (probabilities, or logits through each head's softmax).
//
// "BEV(三) BEVFormer：Query 参数如何与 Feature 的 8 个 Head 交互" says only
// that offsets and weights are learned by back-propagation (section 4.3);
// the gradients are the derivatives of the forward definitions (sections
// 4.2, 5, 6, 8, 10).  For one head of one query, with g = d loss / d out:
//   d/d alpha_k = <S_k, g>,  S_k = sum_c w_c V_c the bilinear sample;
//   d/d V_c    += alpha_k w_c g;
//   d/d x       = alpha_k sum_c <V_c, g> dw_c/dx, dw_c/dx = (i ? 1 : -1)(j ? fy : 1-fy),
//                 and alike for y; d x / d s_x = W (MSDA locations), d x / d dx = 1
//                 (SCA offsets in cells);
//   softmax: d/d a_i = alpha_i (d/d alpha_i - sum_k alpha_k d/d alpha_k).
// SCA: each seeing camera's share is divided by the hit count, and offsets
// and logits, shared by the cameras, sum their gradients over them.
//
// Mapping (as the forward): one wave per query, up to 8 heads per pass; lane
// group g = lane / 8 is a head and lane j = lane % 8 holds channels
// 4j..4j+3 of the upstream gradient and of every corner row.  Staging packs
// the group's live samples (corner rows, cell fractions, weight) densely into
// LDS; the group walks them two at a time (8 corner loads in flight), forms
// <V_c, g> for the four corners and turns them into <S, g>, <dS/dx, g>,
// <dS/dy, g> with an 8-lane reduction.  Each lane then turns its own
// samples' results into location / offset and weight / logit gradients and
// writes them once, in a fixed order.
//
// The value gradient is a scatter: samples of different queries hit the same
// rows.  By default (kEmit) these kernels only write, per sample, a corner
// key and a record (source row, weight, cell fractions) for the transpose
// gather of vgrad.hip, which sums every value row in a fixed order, so
// grad_value is the same bit for bit on every run.  Without a records buffer
// (the A/B variant) the walk adds alpha * w_c * g into the value gradient
// with float32 buffer atomics, each instruction covering two whole 128-byte
// rows (the 8 heads' rows are exchanged across the wave with shuffles; a
// corner outside the map has an offset past the image, and the hardware
// drops that add); their order, and so the last bits of grad_value, varies
// from run to run.
#include "backward.hpp"
#include "common.hpp"
#include "sampling.hpp"
#include "vgrad.hpp"

namespace msda {

constexpr int kBwdMaxWaves = 4;
constexpr uint32_t kNoRow = 0xffffffffu;

// One live sample of a head, staged for the group's 8 lanes (32 bytes).
struct SampleRec {
  uint32_t row[4];  // head row (pixel * nH + h) of corner (dx, dy) = (c & 1, c >> 1), kNoRow outside
  float fx, fy;     // position inside the cell
  float alpha;      // attention weight
  float pad;
};

// records per head area: samples rounded up to the pair the walk takes, plus
// one so that the 8 groups' areas start on different LDS banks
__host__ __device__ inline int rec_stride(int LP) { return (LP + 1) / 2 * 2 + 1; }

__device__ inline void sample_rows_of(SampleRec& r, double x, double y, float alpha, const Level& lv, int h, int nH,
                                      int Nv) {
  x = fmin(fmax(x, -2.0), (double)lv.W + 1.0);  // as the forward: keeps the conversions in range
  y = fmin(fmax(y, -2.0), (double)lv.H + 1.0);
  const double xf = floor(x), yf = floor(y);
  r.fx = (float)(x - xf);
  r.fy = (float)(y - yf);
  r.alpha = alpha;
  r.pad = 0.f;
  const int ix = (int)xf, iy = (int)yf;
  const long long base = lv.start + (long long)iy * lv.W + ix;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int dx = c & 1, dy = c >> 1;
    const long long pix = base + (long long)dy * lv.W + dx;
    const bool ok = ix + dx >= 0 && ix + dx < lv.W && iy + dy >= 0 && iy + dy < lv.H && pix >= 0 && pix < Nv;
    r.row[c] = ok ? (uint32_t)(pix * nH + h) : kNoRow;
    // checked builds: the row is pixel p's row of head h, p inside the level
    MSDA_CHECK(kCheckGatherRow, r.row[c] == kNoRow ||
                                    ((long long)r.row[c] % nH == h && (long long)r.row[c] / nH >= lv.start &&
                                     (long long)r.row[c] / nH < lv.start + (long long)lv.W * lv.H &&
                                     (long long)r.row[c] / nH < Nv));
  }
}

// Pack the group's live samples into `recs` (prefix sum over its 8 lanes)
// and pad every group up to the wave's largest count rounded up to 2.  pos[i]
// is the record of this lane's sample i (-1 if dead).  Returns the padded
// count (the same in every lane).
template <int kSPL>
__device__ inline int stage_samples(SampleRec* __restrict__ recs, const double (&xs)[kSPL],
                                    const double (&ys)[kSPL], const float (&alpha)[kSPL], uint32_t live,
                                    const Level* lv, float inv_P, int j, int h, int nH, int Nv, int (&pos)[kSPL]) {
  const int n = __popc(live);
  int incl = n;
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    const int v = __shfl_up(incl, d, 8);
    if (j >= d) incl += v;
  }
  const int total = __shfl(incl, 7, 8);
  int wmax = total;
  wmax = max(wmax, __shfl_xor(wmax, 8));
  wmax = max(wmax, __shfl_xor(wmax, 16));
  wmax = max(wmax, __shfl_xor(wmax, 32));
  const int S = (wmax + 1) / 2 * 2;
  int p = incl - n;
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    pos[i] = -1;
    if ((live >> i) & 1u) {
      SampleRec r;
      sample_rows_of(r, xs[i], ys[i], alpha[i], lv[small_div(j + 8 * i, inv_P)], h, nH, Nv);
      recs[p] = r;
      pos[i] = p++;
    }
  }
  for (int r = total + j; r < S; r += 8) {
    SampleRec d;
    d.row[0] = d.row[1] = d.row[2] = d.row[3] = kNoRow;
    d.fx = d.fy = d.alpha = d.pad = 0.f;
    recs[r] = d;
  }
  return uniform(S);
}

__device__ inline float4 load_row4(__amdgpu_buffer_rsrc_t img, uint32_t row, uint32_t row_bytes, uint32_t lane_off,
                                   bool bf16) {
  const uint32_t off = row == kNoRow ? kSkip : row * row_bytes + lane_off;
  if (bf16) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(img, off, 0, 0);
    return make_float4(__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                       __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u));
  }
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(img, off, 0, 0);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

__device__ inline float dot4(float4 a, float4 b) { return (a.x * b.x + a.y * b.y) + (a.z * b.z + a.w * b.w); }

// The upstream gradient laid out for whole-row atomics: in atomic step e
// (0..3), half-wave hw = lane / 32 adds the row of head group 2e + hw, lane
// lane % 32 its channel lane % 32.  gt[e] is that channel of that group's g.
// (An atomic instruction that covers two whole 128-byte rows runs about four
// times as fast as one that covers 8 dwords at a 16-byte stride in each of 8
// rows, which is how the gather layout would issue them.)
__device__ inline void transpose_grad(float4 g4, int lane, float (&gt)[4]) {
  const int ch = lane & 31;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int src = (2 * e + (lane >> 5)) * 8 + (ch >> 2);
    const float x = __shfl(g4.x, src), y = __shfl(g4.y, src), z = __shfl(g4.z, src), w = __shfl(g4.w, src);
    const int c = ch & 3;
    gt[e] = c == 0 ? x : (c == 1 ? y : (c == 2 ? z : w));
  }
}

// Walk the group's S staged samples (two at a time).  res[s] receives
// (<S, g>, <dS/dx, g>, <dS/dy, g>) of record s; with kAtomics the value
// gradient of every corner gets alpha * w_c * g, as whole-row atomics
// (transpose_grad).
template <bool kBF16, bool kAtomics>
__device__ inline void walk_samples(const SampleRec* __restrict__ recs, float4* __restrict__ res, int S, float4 g4,
                                    const float (&gt)[4], __amdgpu_buffer_rsrc_t img, __amdgpu_buffer_rsrc_t gimg,
                                    int lane) {
  const int j = lane % 8;
  const uint32_t row_bytes = kBF16 ? 64u : 128u;
  const uint32_t lane_off = (uint32_t)j * (kBF16 ? 8u : 16u);
  const uint32_t glane = (uint32_t)(lane & 31) * 4u;  // float32 gradient rows: 128 bytes
  for (int s = 0; s < S; s += 2) {
    SampleRec r[2] = {recs[s], recs[s + 1]};
    float4 v[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) v[u][c] = load_row4(img, r[u].row[c], row_bytes, lane_off, kBF16);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float fx = r[u].fx, fy = r[u].fy;
      const float wxs[2] = {1.f - fx, fx}, wys[2] = {1.f - fy, fy};
      float ds = 0.f, dx = 0.f, dy = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ix = c & 1, iy = c >> 1;
        const float p = dot4(v[u][c], g4);
        ds = fmaf(wxs[ix] * wys[iy], p, ds);
        dx = fmaf((ix ? 1.f : -1.f) * wys[iy], p, dx);
        dy = fmaf(wxs[ix] * (iy ? 1.f : -1.f), p, dy);
      }
      ds = group_sum(ds);
      dx = group_sum(dx);
      dy = group_sum(dy);
      if (j == 0) res[s + u] = make_float4(ds, dx, dy, 0.f);
      if (!kAtomics) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float coef = r[u].alpha * wxs[c & 1] * wys[c >> 1];
        const uint32_t row = r[u].row[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int src = (2 * e + (lane >> 5)) * 8;  // a lane of the group whose row this half-wave adds
          const float ce = __shfl(coef, src);
          const uint32_t re = (uint32_t)__shfl((int)row, src);
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(ce * gt[e], gimg, re == kNoRow ? kSkip : re * 128u + glane,
                                                          0, 0);
        }
      }
    }
  }
}

// The records of one head's samples for the transpose gather of the value
// gradient (vgrad.hip): slot slot0 + k for sample k, key kDeadKey when no
// corner is inside the map.  The cell and fractions are those of
// sample_rows_of; alpha is divided by the query's hit count (SCA).
template <int kSPL>
__device__ inline void emit_records(const BackwardArgs& a, const Level* lv, const long long* ext, uint32_t slot0,
                                    uint32_t src, int hits, const double (&xs)[kSPL], const double (&ys)[kSPL],
                                    const float (&alpha)[kSPL], uint32_t live, int j) {
  VgradRec* vals = static_cast<VgradRec*>(a.rec_vals);
#pragma unroll
  for (int i = 0; i < kSPL; ++i) {
    const int k = j + 8 * i;
    if (k >= a.LP || slot0 + k >= a.rec_slots) continue;
    uint32_t key = kDeadKey;
    if ((live >> i) & 1u) {
      const int l = small_div(k, a.inv_P);
      const Level L = lv[l];
      const double x = fmin(fmax(xs[i], -2.0), (double)L.W + 1.0);
      const double y = fmin(fmax(ys[i], -2.0), (double)L.H + 1.0);
      const double xf = floor(x), yf = floor(y);
      VgradRec r;
      r.src = src;
      r.alpha = hits > 1 ? alpha[i] / (float)hits : alpha[i];
      r.fx = (float)(x - xf);
      r.fy = (float)(y - yf);
      // (a level table whose corner keys pass 2^32 is flagged by the setup:
      // the value gradient is NaN then, whatever the keys)
      key = corner_key(ext[l], L.W, (int)xf + 1, (int)yf + 1);
      vals[slot0 + k] = r;
    }
    a.rec_keys[slot0 + k] = key;
  }
}

// First record slot of pair `local` (its index among the image's pairs) and
// head h of an image: every head of an image has as many records, so its
// segments take equally many tiles from the image's first one on.
__device__ inline uint32_t record_slot(const BackwardArgs& a, int64_t image, int h, int64_t local) {
  const int64_t s = image * a.nH;
  const uint32_t first = (uint32_t)uniform(a.seg_tile[s]);
  const uint32_t tiles = (uint32_t)uniform(a.seg_tile[s + 1]) - first;
  return (first + (uint32_t)h * tiles) * (uint32_t)kSortTile + (uint32_t)local * (uint32_t)a.LP;
}

// LDS: the level table, then per wave and head group its sample records and
// their results.
struct BwdLds {
  Level* lv;
  SampleRec* recs;
  float4* res;
  __device__ BwdLds(unsigned char* smem, int LP, int wave, int g, int waves) {
    const int st = rec_stride(LP);
    lv = reinterpret_cast<Level*>(smem);
    SampleRec* r0 = reinterpret_cast<SampleRec*>(smem + sizeof(Level) * kMaxLevels);
    recs = r0 + ((size_t)wave * kHeadSlots + g) * st;
    res = reinterpret_cast<float4*>(r0 + (size_t)waves * kHeadSlots * st) + ((size_t)wave * kHeadSlots + g) * st;
  }
};

static size_t bwd_smem(int LP, int waves) {
  return sizeof(Level) * kMaxLevels + (sizeof(SampleRec) + sizeof(float4)) * (size_t)waves * kHeadSlots * rec_stride(LP);
}

// weights gradient of one head from the per-sample <S, g> (group-wide softmax backward for logits)
template <int kSPL>
__device__ inline void weights_grad(const float (&alpha)[kSPL], const float (&ds)[kSPL], bool logits,
                                    float (&gw)[kSPL]) {
  if (!logits) {
#pragma unroll
    for (int i = 0; i < kSPL; ++i) gw[i] = ds[i];
    return;
  }
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < kSPL; ++i) dot = fmaf(alpha[i], ds[i], dot);
  dot = group_sum(dot);
#pragma unroll
  for (int i = 0; i < kSPL; ++i) gw[i] = alpha[i] * (ds[i] - dot);
}

// ---------------------------------------------------------------------------
// MSDA operator: item = (image, q), image = b * F + f; the frame-mean variant
// (F > 1) takes frame f's share grad_out[b][q] / F of the upstream gradient
// ---------------------------------------------------------------------------
template <bool kBF16, int kSPL, bool kEmit>
__global__ __launch_bounds__(kBwdMaxWaves* kWave) void msda_backward_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ long long ext[kMaxLevels + 1];
  const int waves_per_block = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wave = uniform((int)(threadIdx.x / kWave));
  const int g = lane / 8, j = lane % 8;
  BwdLds m(smem, a.LP, wave, g, waves_per_block);
  load_levels(a.shapes, a.starts, a.L, m.lv);
  if (kEmit) load_corner_starts(m.lv, a.L, ext);

  XcdSplit split(a.B * a.Nq, waves_per_block);
  for (int64_t item = split.begin; item < split.end; item += split.stride) {
    const int64_t b = item / a.Nq;
    const auto img = make_rsrc(static_cast<const char*>(a.value) + b * (int64_t)a.image_bytes, a.image_bytes);
    const auto gimg = make_rsrc(reinterpret_cast<char*>(a.grad_value) + b * (int64_t)a.grad_image_bytes,
                                a.grad_image_bytes);
    for (int hb = 0; hb < a.nH; hb += kHeadSlots) {
      const int h = hb + g;
      const bool head_ok = h < a.nH;
      const int64_t src_row = item * a.nH + (head_ok ? h : 0);
      // the upstream-gradient row (b, q) of this image's batch item
      const int64_t grad_row = a.F > 1 ? ((b / a.F) * a.Nq + (item - b * a.Nq)) * a.nH + (head_ok ? h : 0) : src_row;
      float alpha[kSPL];
      head_weights<kSPL>(a.weights + src_row * a.LP, head_ok, a.LP, j, a.weight_logits != 0, alpha);
      float4 g4 = head_ok ? reinterpret_cast<const float4*>(a.grad_out + grad_row * 32)[j]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      if (a.F > 1) {
        const float n = (float)a.F;
        g4 = make_float4(g4.x / n, g4.y / n, g4.z / n, g4.w / n);
      }
      float gt[4];
      transpose_grad(g4, lane, gt);
      const float2* loc = reinterpret_cast<const float2*>(a.loc) + src_row * a.LP;
      double xs[kSPL], ys[kSPL];
      uint32_t live = 0u;
#pragma unroll
      for (int i = 0; i < kSPL; ++i) {
        const int k = j + 8 * i;
        const bool valid = head_ok && k < a.LP;
        const Level L = m.lv[valid ? small_div(k, a.inv_P) : 0];
        const float2 s = valid ? loc[k] : make_float2(0.f, 0.f);
        xs[i] = (double)s.x * L.W - 0.5;
        ys[i] = (double)s.y * L.H - 0.5;
        if (valid && sample_live(xs[i], ys[i], L)) live |= 1u << i;
      }
      int pos[kSPL];
      const int S = stage_samples<kSPL>(m.recs, xs, ys, alpha, live, m.lv, a.inv_P, j, h, a.nH, a.Nv, pos);
      if (kEmit && head_ok)
        emit_records<kSPL>(a, m.lv, ext,
                           record_slot(a, b, h, item - b * a.Nq),
                           (uint32_t)grad_row, a.F, xs, ys, alpha, live, j);
      wave_lds_sync();
      walk_samples<kBF16, !kEmit>(m.recs, m.res, S, g4, gt, img, gimg, lane);
      wave_lds_sync();
      float ds[kSPL], gw[kSPL];
#pragma unroll
      for (int i = 0; i < kSPL; ++i) {
        const int k = j + 8 * i;
        const float4 r = pos[i] >= 0 ? m.res[pos[i]] : make_float4(0.f, 0.f, 0.f, 0.f);
        ds[i] = r.x;
        if (head_ok && k < a.LP) {
          const Level L = m.lv[small_div(k, a.inv_P)];
          reinterpret_cast<float2*>(a.grad_loc)[src_row * a.LP + k] =
              make_float2(alpha[i] * (float)L.W * r.y, alpha[i] * (float)L.H * r.z);
        }
      }
      weights_grad<kSPL>(alpha, ds, a.weight_logits != 0, gw);
#pragma unroll
      for (int i = 0; i < kSPL; ++i) {
        const int k = j + 8 * i;
        if (head_ok && k < a.LP) a.grad_weights[src_row * a.LP + k] = gw[i];
      }
      wave_lds_sync();  // the next pass restages the records
    }
  }
}

// ---------------------------------------------------------------------------
// SCA: item = entry of the compaction's work list; the wave runs all cameras
// of its query, sums the offset and logit gradients over them, and writes
// them once.  Queries no camera sees get zero gradients first.
// ---------------------------------------------------------------------------
// For L*P > 32 the kernel is held to 2 waves per SIMD (256 registers).
template <bool kBF16, int kSPL, bool kEmit>
__global__ __launch_bounds__(kBwdMaxWaves* kWave, kSPL == 8 ? 2 : 1) void sca_backward_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ long long ext[kMaxLevels + 1];
  const int waves_per_block = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wave = uniform((int)(threadIdx.x / kWave));
  const int g = lane / 8, j = lane % 8;
  BwdLds m(smem, a.LP, wave, g, waves_per_block);
  load_levels(a.shapes, a.starts, a.L, m.lv);
  if (kEmit) load_corner_starts(m.lv, a.L, ext);
  const int64_t n_queries = a.B * a.Nq;
  const uint32_t cam_bits = a.Ncam >= 32 ? 0xffffffffu : ((1u << a.Ncam) - 1u);

  // Queries no camera sees are on no work list: their gradients are zero.
  // One wave-wide mask load covers 64 queries, before the wave's work.
  {
    const int64_t per_q = (int64_t)a.nH * a.LP;
    const int64_t n_waves = (int64_t)gridDim.x * waves_per_block;
    for (int64_t q0 = ((int64_t)blockIdx.x * waves_per_block + wave) * kWave; q0 < n_queries; q0 += n_waves * kWave) {
      const bool unseen = q0 + lane < n_queries && (a.cammask[q0 + lane] & cam_bits) == 0u;
      for (uint64_t u = __ballot(unseen); u != 0ull; u &= u - 1ull) {
        const int64_t bq = q0 + __builtin_ctzll(u);
        for (int64_t e = lane; e < per_q; e += kWave) {
          reinterpret_cast<float2*>(a.grad_offsets)[bq * per_q + e] = make_float2(0.f, 0.f);
          a.grad_logits[bq * per_q + e] = 0.f;
        }
      }
    }
  }

  for (int64_t bi = 0; bi < a.B; ++bi) {
    const DieShare split(a.die_bounds + bi * kDieBounds, n_queries, waves_per_block);
    for (int64_t item = split.begin; item < split.end; item += split.stride) {
      const int64_t bq = uniform((int64_t)a.order[item]);
      if (bq < 0 || bq >= n_queries) continue;
      const int64_t b = bq / a.Nq, q = bq % a.Nq;
      const uint32_t seen = uniform(a.cammask[bq] & cam_bits);
      if (seen == 0u) continue;
      const int hits = __popc(seen);

      for (int hb = 0; hb < a.nH; hb += kHeadSlots) {
        const int h = hb + g;
        const bool head_ok = h < a.nH;
        const int64_t src_row = bq * a.nH + (head_ok ? h : 0);
        float alpha[kSPL];
        head_weights<kSPL>(a.logits + src_row * a.LP, head_ok, a.LP, j, true, alpha);
        float2 off[kSPL];
        const float2* off_row = reinterpret_cast<const float2*>(a.offsets) + src_row * a.LP;
#pragma unroll
        for (int i = 0; i < kSPL; ++i) {
          const int k = j + 8 * i;
          off[i] = (head_ok && k < a.LP) ? off_row[k] : make_float2(0.f, 0.f);
        }
        // each seeing camera's share of the slot gradient is 1 / hits of it
        float4 g4 = head_ok ? reinterpret_cast<const float4*>(a.grad_out + src_row * 32)[j]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        if (hits > 1) {
          const float n = (float)hits;
          g4 = make_float4(g4.x / n, g4.y / n, g4.z / n, g4.w / n);
        }
        float gt[4];
        transpose_grad(g4, lane, gt);
        float ds[kSPL], dx[kSPL], dy[kSPL];
#pragma unroll
        for (int i = 0; i < kSPL; ++i) ds[i] = dx[i] = dy[i] = 0.f;
        for (uint32_t rest = seen; rest != 0u; rest &= rest - 1u) {
          const int c = __builtin_ctz(rest);
          const float2* rho = reinterpret_cast<const float2*>(a.rp) + ((c * a.B + b) * a.Nq + q) * a.D;
          double xs[kSPL], ys[kSPL];
          uint32_t live = 0u;
#pragma unroll
          for (int i = 0; i < kSPL; ++i) {
            const int k = j + 8 * i;
            const bool valid = head_ok && k < a.LP;
            const Level L = m.lv[valid ? small_div(k, a.inv_P) : 0];
            const int mm = k - a.D * small_div(k, a.inv_D);  // anchor k mod D
            const float2 r = valid ? rho[mm] : make_float2(0.f, 0.f);
            xs[i] = (double)r.x * L.W + (double)off[i].x - 0.5;
            ys[i] = (double)r.y * L.H + (double)off[i].y - 0.5;
            if (valid && sample_live(xs[i], ys[i], L)) live |= 1u << i;
          }
          int pos[kSPL];
          const int S = stage_samples<kSPL>(m.recs, xs, ys, alpha, live, m.lv, a.inv_P, j, h, a.nH, a.Nv, pos);
          const int64_t image = b * a.Ncam + c;
          if (kEmit) {
            const int64_t pair = uniform((int64_t)a.pair_of[(c * a.B + b) * a.Nq + q]);
            if (head_ok && pair >= 0 && pair < a.max_pairs)
              emit_records<kSPL>(a, m.lv, ext,
                                 record_slot(a, image, h, pair - uniform(a.pair_start[image])),
                                 (uint32_t)src_row, hits, xs, ys, alpha, live, j);
          }
          wave_lds_sync();
          const auto img = make_rsrc(static_cast<const char*>(a.value) + image * (int64_t)a.image_bytes,
                                     a.image_bytes);
          const auto gimg = make_rsrc(reinterpret_cast<char*>(a.grad_value) + image * (int64_t)a.grad_image_bytes,
                                      a.grad_image_bytes);
          walk_samples<kBF16, !kEmit>(m.recs, m.res, S, g4, gt, img, gimg, lane);
          wave_lds_sync();
#pragma unroll
          for (int i = 0; i < kSPL; ++i) {
            if (pos[i] >= 0) {
              const float4 r = m.res[pos[i]];
              ds[i] += r.x;
              dx[i] += r.y;
              dy[i] += r.z;
            }
          }
          wave_lds_sync();  // the next camera restages the records
        }
        float gw[kSPL];
        weights_grad<kSPL>(alpha, ds, true, gw);
#pragma unroll
        for (int i = 0; i < kSPL; ++i) {
          const int k = j + 8 * i;
          if (head_ok && k < a.LP) {
            reinterpret_cast<float2*>(a.grad_offsets)[src_row * a.LP + k] =
                make_float2(alpha[i] * dx[i], alpha[i] * dy[i]);
            a.grad_logits[src_row * a.LP + k] = gw[i];
          }
        }
      }
    }
  }

}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_kernel(float4* p, int64_t n4) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += (int64_t)gridDim.x * blockDim.x)
    p[e] = make_float4(0.f, 0.f, 0.f, 0.f);
}


static int bwd_waves(int LP) {
  int w = kBwdMaxWaves;
  while (w > 1 && bwd_smem(LP, w) > kMaxBlockLds) w /= 2;
  return w;
}

// a grid the chip holds at once (as the SCA forward), a multiple of the die count
template <typename Kernel>
static hipError_t launch(Kernel kernel, int64_t n_items, int LP, const BackwardArgs& a, hipStream_t stream) {
  const int waves = bwd_waves(LP);
  const size_t smem = bwd_smem(LP, waves);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, waves * kWave, smem) != hipSuccess || per_cu < 1)
    per_cu = 1;
  int64_t need = (n_items + waves - 1) / waves;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  if (need > cap) need = cap;
  if (need < 1) need = 1;
  const unsigned grid = (unsigned)((need + kXcds - 1) / kXcds * kXcds);
  kernel<<<grid, waves * kWave, smem, stream>>>(a);
  return hipGetLastError();
}

static void zero_grad_value(const BackwardArgs& a, hipStream_t stream) {
  const int64_t n4 = a.images * (int64_t)a.grad_image_bytes / 16;
  if (n4 == 0) return;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  zero_kernel<<<(unsigned)blocks, 256, 0, stream>>>(reinterpret_cast<float4*>(a.grad_value), n4);
}

hipError_t launch_msda_backward(const BackwardArgs& a, hipStream_t stream) {
  const int64_t n = a.B * a.Nq;
  if (a.rec_keys) {  // records for the transpose gather: grad_value is written later, whole
    if (a.LP <= 32)
      return launch(a.bf16 ? msda_backward_kernel<true, 4, true> : msda_backward_kernel<false, 4, true>, n, a.LP, a,
                    stream);
    return launch(a.bf16 ? msda_backward_kernel<true, 8, true> : msda_backward_kernel<false, 8, true>, n, a.LP, a,
                  stream);
  }
  zero_grad_value(a, stream);
  if (a.LP <= 32)
    return launch(a.bf16 ? msda_backward_kernel<true, 4, false> : msda_backward_kernel<false, 4, false>, n, a.LP, a,
                  stream);
  return launch(a.bf16 ? msda_backward_kernel<true, 8, false> : msda_backward_kernel<false, 8, false>, n, a.LP, a,
                stream);
}

hipError_t launch_sca_backward(const BackwardArgs& a, hipStream_t stream) {
  const int64_t n = a.B * a.Nq;
  if (a.rec_keys) {
    if (a.LP <= 32)
      return launch(a.bf16 ? sca_backward_kernel<true, 4, true> : sca_backward_kernel<false, 4, true>, n, a.LP, a,
                    stream);
    return launch(a.bf16 ? sca_backward_kernel<true, 8, true> : sca_backward_kernel<false, 8, true>, n, a.LP, a,
                  stream);
  }
  zero_grad_value(a, stream);
  if (a.LP <= 32)
    return launch(a.bf16 ? sca_backward_kernel<true, 4, false> : sca_backward_kernel<false, 4, false>, n, a.LP, a,
                  stream);
  return launch(a.bf16 ? sca_backward_kernel<true, 8, false> : sca_backward_kernel<false, 8, false>, n, a.LP, a,
                stream);
}

}  // namespace msda
