// The padded "rebatch" form of spatial cross-attention, kept as an A/B
// baseline for the fused path (Tencent Cloud developer article 2321140, a
// note on BEVFormer's Spatial Cross-Attention: its rebatch code and its
// scatter / count / divide code; locations as in "BEV(三) BEVFormer：Query
// 参数如何与 Feature 的 8 个 Head 交互", sections 5 and 18.4).
//
// The note copies every (batch item, camera) segment of seen queries into
// buffers padded to the longest segment, max_len, runs the deformable
// attention operator over all B * Ncam segments at once, adds each camera's
// rows back into the queries' slots and divides by the hit count.  Here:
//   - sca_rebatch_kernel writes, for every padded row, the row's sampling
//     locations s = rho + delta / (W_l, H_l) as a float32 tensor (the operator
//     takes them materialised) and its attention logits; padded rows get zero
//     locations and logits (their results are discarded, as in the note);
//   - the MSDA operator (gather.hip) then treats the B * Ncam segments as a
//     batch over the value images b * Ncam + c;
//   - sca_zero_kernel, one sca_scatter_kernel launch per camera in ascending
//     order (rows of one camera never collide: a query appears once per
//     segment) and sca_divide_kernel form the camera mean.
#include "common.hpp"
#include "rebatch.hpp"

namespace msda {

// Start and length of segment bc of the pair lists, clamped to the n_pairs
// entries pair_q can hold: a malformed pair_offsets array then reads and
// writes nothing out of bounds (the rows it names are simply not added).
__device__ inline void segment_bounds(const int32_t* pair_offsets, int64_t bc, int64_t n_pairs, int64_t* lo,
                                      int64_t* len) {
  int64_t s = pair_offsets[bc], e = pair_offsets[bc + 1];
  MSDA_CHECK(kCheckListEntry, s >= 0 && s <= e && e <= n_pairs);
  s = s < 0 ? 0 : (s > n_pairs ? n_pairs : s);
  e = e < s ? s : (e > n_pairs ? n_pairs : e);
  *lo = s;
  *len = e - s;
}

// one wavefront per padded row (segment bc, position i)
__global__ __launch_bounds__(256) void sca_rebatch_kernel(RebatchArgs a) {
  const int lane = threadIdx.x % kWave;
  const int64_t rows = a.B * a.Ncam * a.max_len;
  const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int S = a.nH * a.L * a.P;  // samples per row
  for (int64_t r = wave0; r < rows; r += nwaves) {
    const int64_t bc = r / a.max_len, i = r % a.max_len;
    const int64_t b = bc / a.Ncam, c = bc % a.Ncam;
    int64_t lo, len;
    segment_bounds(a.pair_offsets, bc, a.B * a.Ncam * a.Nq, &lo, &len);
    int64_t q = i < len ? a.pair_q[lo + i] : -1;
    MSDA_CHECK(kCheckListEntry, i >= len || (q >= 0 && q < a.Nq));
    const bool live = q >= 0 && q < a.Nq;  // an entry outside [0, Nq) is a padded row
    q = live ? q : 0;
    float2* loc = reinterpret_cast<float2*>(a.loc_out) + r * S;
    float* w = a.logits_out + r * S;
    for (int s = lane; s < S; s += kWave) {
      float2 v = make_float2(0.f, 0.f);
      float lg = 0.f;
      if (live) {
        const int p = s % a.P, l = (s / a.P) % a.L;
        const float2 rho = reinterpret_cast<const float2*>(a.rp)[((c * a.B + b) * a.Nq + q) * a.D + p % a.D];
        const float2 d = reinterpret_cast<const float2*>(a.offsets)[(b * a.Nq + q) * S + s];
        const float Wl = (float)a.shapes[2 * l + 1], Hl = (float)a.shapes[2 * l];
        v = make_float2(rho.x + d.x / Wl, rho.y + d.y / Hl);
        lg = a.logits[(b * a.Nq + q) * S + s];
      }
      loc[s] = v;
      w[s] = lg;
    }
  }
}

// slots = 0 (queries no camera sees stay zero)
__global__ __launch_bounds__(256) void sca_zero_kernel(float4* slots, int64_t n4) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += (int64_t)gridDim.x * blockDim.x)
    slots[e] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// slots[b][q] += rows[b * Ncam + c][i] for the segment of camera c: one
// wavefront per row, 16 bytes per lane
__global__ __launch_bounds__(256) void sca_scatter_kernel(ScatterArgs a, int c) {
  const int lane = threadIdx.x % kWave;
  const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int64_t C4 = a.C / 4;
  const int64_t n = a.B * a.max_len;
  for (int64_t t = wave0; t < n; t += nwaves) {
    const int64_t b = t / a.max_len, i = t % a.max_len;
    const int64_t bc = b * a.Ncam + c;
    int64_t lo, len;
    segment_bounds(a.pair_offsets, bc, a.B * a.Ncam * a.Nq, &lo, &len);
    if (i >= len) continue;  // uniform over the wavefront
    const int64_t q = a.pair_q[lo + i];
    MSDA_CHECK(kCheckListEntry, q >= 0 && q < a.Nq);
    if (q < 0 || q >= a.Nq) continue;
    const float4* src = reinterpret_cast<const float4*>(a.rows + (bc * a.max_len + i) * a.C);
    float4* dst = reinterpret_cast<float4*>(a.slots + (b * a.Nq + q) * a.C);
    for (int64_t e = lane; e < C4; e += kWave) {
      const float4 u = dst[e], v = src[e];
      dst[e] = make_float4(u.x + v.x, u.y + v.y, u.z + v.z, u.w + v.w);
    }
  }
}

// slots[b][q] /= max(1, hits[b][q])
__global__ __launch_bounds__(256) void sca_divide_kernel(ScatterArgs a) {
  const int64_t C4 = a.C / 4, n4 = a.B * a.Nq * C4;
  float4* s = reinterpret_cast<float4*>(a.slots);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += (int64_t)gridDim.x * blockDim.x) {
    const int hits = a.hit_count[e / C4];
    if (hits > 1) {
      const float n = (float)hits;
      const float4 v = s[e];
      s[e] = make_float4(v.x / n, v.y / n, v.z / n, v.w / n);
    }
  }
}

static unsigned blocks_for(int64_t items, int per_block) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

hipError_t launch_sca_rebatch(const RebatchArgs& a, hipStream_t stream) {
  const int64_t rows = a.B * a.Ncam * a.max_len;
  if (rows == 0) return hipSuccess;
  sca_rebatch_kernel<<<blocks_for(rows, 4), 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_sca_scatter_mean(const ScatterArgs& a, hipStream_t stream) {
  const int64_t n4 = a.B * a.Nq * (a.C / 4);
  if (n4 == 0) return hipSuccess;
  sca_zero_kernel<<<blocks_for(n4, 256), 256, 0, stream>>>(reinterpret_cast<float4*>(a.slots), n4);
  if (a.max_len > 0)
    for (int c = 0; c < a.Ncam; ++c) sca_scatter_kernel<<<blocks_for(a.B * a.max_len, 4), 256, 0, stream>>>(a, c);
  sca_divide_kernel<<<blocks_for(n4, 256), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace msda
