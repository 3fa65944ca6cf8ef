// SCA visibility and compaction (the bev_mask rebatch of the Tencent Cloud
// SCA note, article 2321140: per camera, the ascending indices of the BEV
// queries the camera sees; and its hit count per query), plus the order in
// which the gather kernel visits the seen queries.
//
// Four small stream-ordered kernels:
//   0. clear: zero the ordering histogram and the per-segment totals;
//   1. visibility: per (b, q) the bit set of cameras that see q (any of the D
//      anchors marked), the hit count, per (b, c, tile of 256 queries) the
//      number of seen queries, and for a seen query its ordering bin: the
//      image tile (kOrderBinsX columns x kOrderBinsY rows, column-major) of
//      the first marked anchor of its first camera, within the segment
//      (b, first camera);
//   2. scan: one workgroup per segment (b, c) turns the segment's tile counts
//      and bin counts into exclusive offsets, starting from the sums of the
//      earlier segments' totals (which the visibility kernel accumulated):
//      pair_offsets[b*Ncam + c] is the offset of the first tile of (b, c)
//      and pair_offsets[B*Ncam] the total; and it places the boundaries of
//      the dies' shares of the batch item's work list where the summed cost
//      of the bins crosses each eighth of the item's total (interpolating
//      inside the bin), so that every die gets the same estimated work;
//   3. compact: each query writes its index at tile offset + (seen queries
//      before it in the tile) for every camera that sees it, so each (b, c)
//      list comes out in ascending order (deterministic, no atomics); and a
//      seen query takes a slot of its bin in the work order (atomic slot
//      claims: the order inside a bin varies from run to run, which changes
//      only which wave computes which query, never a result).
// Queries that share a bin project to the same image tile of the same
// camera, so consecutive work items read neighbouring value rows and one
// die's L2 holds their working set.  Bins run column-major: the anchors of
// one query differ mostly in image row (pillar height), so a column band is
// finished before the next one starts.
#include "common.hpp"
#include "internal.hpp"

namespace msda {

constexpr int kTile = kQueryTile;  // queries per tile = threads per block
constexpr int kTileWaves = kTile / kWave;
constexpr int kScanThreads = kOrderBins;  // one bin per thread
static_assert(kScanThreads == 1024, "the scan block holds one segment's bins");

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

CompactLayout compact_layout(int64_t B, int64_t Ncam, int64_t Nq) {
  CompactLayout l;
  l.tiles = (int)((Nq + kTile - 1) / kTile);
  const size_t segs = (size_t)(B * Ncam);
  const size_t nq = (size_t)(B * Nq);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  l.cammask = take(sizeof(uint32_t) * nq);
  l.qkey = take(sizeof(int32_t) * nq);
  l.tile_counts = take(sizeof(int32_t) * segs * (size_t)l.tiles);
  l.tile_offsets = take(sizeof(int32_t) * segs * (size_t)l.tiles);
  l.pair_offsets = take(sizeof(int32_t) * (segs + 1));
  l.pair_q = take(sizeof(int32_t) * segs * (size_t)Nq);
  // bin_hist, seg_seen, seg_pairs, bin_cost and seg_cost back to back (only
  // the 8-byte alignment of the costs between), cleared as one range
  l.bin_hist = o;
  l.seg_seen = l.bin_hist + sizeof(int32_t) * segs * kOrderBins;
  l.seg_pairs = l.seg_seen + sizeof(int32_t) * segs;
  l.bin_cost = align_up(l.seg_pairs + sizeof(int32_t) * segs, 8);
  l.seg_cost = l.bin_cost + sizeof(uint64_t) * segs * kOrderBins;
  l.clear_ints = (int)((l.seg_cost + sizeof(uint64_t) * segs - l.bin_hist) / sizeof(int32_t));
  o = align_up(l.seg_cost + sizeof(uint64_t) * segs, 256);
  l.bin_offsets = take(sizeof(int32_t) * (segs * kOrderBins + 1));
  l.order = take(sizeof(int32_t) * nq);
  l.die_bounds = take(sizeof(int32_t) * (size_t)B * kDieBounds);
  l.total = o;
  return l;
}

__global__ __launch_bounds__(kTile) void sca_clear_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * kTile + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Nonzero bytes of a 32-bit word (marked anchors among four).
__device__ inline int nonzero_bytes(uint32_t w) {
  return __popc((((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u);
}

// Work estimate of one seeing camera: its marked anchors (capped) + 1.
__device__ inline uint32_t camera_cost(int marked) { return 1u + (uint32_t)min(marked, 1023); }

__device__ inline int tile_bin(float v, int n) {
  const float t = fminf(fmaxf(v, 0.f), 1.f) * (float)n;  // NaN -> 0
  return min((int)t, n - 1);
}

template <bool kWordMask>
__global__ __launch_bounds__(kTile) void sca_visibility_kernel(CompactArgs a, int tiles) {
  __shared__ int wave_counts[kTileWaves][32];
  __shared__ int first_counts[kTileWaves][32];
  __shared__ unsigned long long first_cost[32];  // cost of the block's queries by first camera
  const int tile = blockIdx.x, b = blockIdx.y;
  const int q = tile * kTile + (int)threadIdx.x;
  const bool in_range = q < a.Nq;
  if (threadIdx.x < 32) first_cost[threadIdx.x] = 0ull;
  __syncthreads();
  uint32_t seen = 0, cost = 0;
  int first_anchor = 0, key = -1;
  if (in_range) {
    const int64_t cam_stride = (int64_t)a.B * a.Nq * a.D;  // mask bytes between cameras
    const uint8_t* mq = a.bev_mask + ((int64_t)b * a.Nq + q) * a.D;
    // first: the camera's first marked anchor (-1: none); n_marked: its marked anchors
    auto note = [&](int c, int first, int n_marked) {
      if (first >= 0) {
        if (seen == 0u) first_anchor = first;
        seen |= 1u << c;
        cost += camera_cost(n_marked);
      }
    };
    if (kWordMask) {  // D % 4 == 0 and the mask is 4-byte aligned
      // the first word (4 anchors) of 8 cameras at a time: the loads go out together
      constexpr int kCams = 8;
      const int words = a.D / 4;
      for (int c0 = 0; c0 < a.Ncam; c0 += kCams) {
        uint32_t w0[kCams];
#pragma unroll
        for (int u = 0; u < kCams; ++u)
          w0[u] = c0 + u < a.Ncam ? *reinterpret_cast<const uint32_t*>(mq + (c0 + u) * cam_stride) : 0u;
#pragma unroll
        for (int u = 0; u < kCams; ++u) {
          if (c0 + u >= a.Ncam) break;
          const uint32_t* m = reinterpret_cast<const uint32_t*>(mq + (c0 + u) * cam_stride);
          int marked = w0[u] != 0u ? __builtin_ctz(w0[u]) / 8 : -1;
          int n_marked = nonzero_bytes(w0[u]);
          for (int k = 1; k < words; ++k) {
            const uint32_t wk = m[k];
            if (wk != 0u && marked < 0) marked = 4 * k + __builtin_ctz(wk) / 8;
            n_marked += nonzero_bytes(wk);
          }
          note(c0 + u, marked, n_marked);
        }
      }
    } else {
      for (int c = 0; c < a.Ncam; ++c) {
        const uint8_t* m = mq + c * cam_stride;
        int marked = -1, n_marked = 0;  // first marked anchor of this camera, and their number
        for (int k = 0; k < a.D; ++k)
          if (m[k] != 0) {
            if (marked < 0) marked = k;
            ++n_marked;
          }
        note(c, marked, n_marked);
      }
    }
    const int64_t bq = (int64_t)b * a.Nq + q;
    a.cammask[bq] = seen;
    if (a.hit_count) a.hit_count[bq] = __popc(seen);
    if (seen != 0u) {
      const int c0 = __builtin_ctz(seen);
      const float2 r = reinterpret_cast<const float2*>(a.rp)[(((int64_t)c0 * a.B + b) * a.Nq + q) * a.D + first_anchor];
      const int bin = tile_bin(r.x, kOrderBinsX) * kOrderBinsY + tile_bin(r.y, kOrderBinsY);
      key = (b * a.Ncam + c0) * kOrderBins + bin;
      atomicAdd(&a.bin_hist[key], 1);
      atomicAdd(&a.bin_cost[key], (unsigned long long)cost);
      atomicAdd(&first_cost[c0], (unsigned long long)cost);
    }
    a.qkey[bq] = key;
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int first = seen != 0u ? __builtin_ctz(seen) : -1;
  for (int c = 0; c < a.Ncam; ++c) {
    const uint64_t bits = __ballot((seen >> c) & 1u);
    const uint64_t firsts = __ballot(first == c);
    if (lane == 0) {
      wave_counts[wave][c] = __popcll(bits);
      first_counts[wave][c] = __popcll(firsts);
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < a.Ncam) {
    const int c = threadIdx.x;
    int s = 0, f = 0;
    for (int w = 0; w < kTileWaves; ++w) {
      s += wave_counts[w][c];
      f += first_counts[w][c];
    }
    a.tile_counts[((int64_t)b * a.Ncam + c) * tiles + tile] = s;
    if (s) atomicAdd(&a.seg_pairs[b * a.Ncam + c], s);
    if (f) atomicAdd(&a.seg_seen[b * a.Ncam + c], f);
    if (f) atomicAdd(&a.seg_cost[b * a.Ncam + c], first_cost[c]);
  }
}

// Exclusive scan of one value per thread over the block (kScanThreads);
// also returns the block total.
__device__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wave_sums[kScanThreads / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  __syncthreads();  // wave_sums may still be read by a previous scan
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kScanThreads / kWave; ++w) {
    const int ws = wave_sums[w];
    before += w < wave ? ws : 0;
    all += ws;
  }
  *total = all;
  return before + incl - v;
}

// Sum of x[0, n) over the block.
__device__ int block_sum(const int32_t* __restrict__ x, int n) {
  __shared__ int partial[kScanThreads / kWave];
  int s = 0;
  for (int i = threadIdx.x; i < n; i += kScanThreads) s += x[i];
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) s += __shfl_xor(s, d);
  __syncthreads();
  if (threadIdx.x % kWave == 0) partial[threadIdx.x / kWave] = s;
  __syncthreads();
  int all = 0;
  for (int w = 0; w < kScanThreads / kWave; ++w) all += partial[w];
  return all;
}

// Inclusive scan of one 64-bit value per thread over the block.
__device__ uint64_t block_inclusive_scan64(uint64_t v) {
  __shared__ uint64_t wave_sums64[kScanThreads / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint64_t incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint64_t u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  __syncthreads();
  if (lane == kWave - 1) wave_sums64[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wave_sums64[w];
  return incl;
}

// One block per segment s = b*Ncam + c.
__global__ __launch_bounds__(kScanThreads) void sca_scan_kernel(CompactArgs a, int tiles) {
  const int s = blockIdx.x, segs = a.B * a.Ncam;
  const int t = threadIdx.x;
  const int b = s / a.Ncam, c = s % a.Ncam;
  const int base_seen = block_sum(a.seg_seen, s);
  const int base_pairs = block_sum(a.seg_pairs, s);
  int total = 0;
  const int64_t bin = (int64_t)s * kOrderBins + t;
  const int count = a.bin_hist[bin];
  const int first_item = base_seen + block_exclusive_scan(count, &total);
  a.bin_offsets[bin] = first_item;

  // Boundaries of the dies' shares of batch item b's work list: share x
  // starts where the summed cost, in work-list order, reaches x/8 of the
  // item's total (inside a bin, by linear interpolation over its entries).
  // The bin holding a target writes it; the item's first and last segments
  // write its ends (and, with no cost at all, every boundary).
  uint64_t item_cost = 0, seg_base = 0;  // uniform: the item's total, and its cost before this segment
  for (int k = 0; k < a.Ncam; ++k) {
    const uint64_t v = a.seg_cost[(int64_t)b * a.Ncam + k];
    item_cost += v;
    seg_base += k < c ? v : 0ull;
  }
  const uint64_t bin_cost = a.bin_cost[bin];
  const uint64_t bin_end = seg_base + block_inclusive_scan64(bin_cost);  // relative to the item
  const uint64_t bin_begin = bin_end - bin_cost;
  int32_t* bounds = a.die_bounds + (int64_t)b * kDieBounds;
  for (int x = 1; x < kXcds; ++x) {
    const uint64_t target = item_cost * (uint64_t)x / kXcds;
    if (bin_cost != 0 && target >= bin_begin && target < bin_end) {
      // entry of the bin at that fraction of its cost (double: no overflow
      // of cost x count; the clamp keeps it inside the bin)
      const int k = (int)((double)(target - bin_begin) / (double)bin_cost * (double)count);
      bounds[x] = first_item + min(max(k, 0), count - 1);
    }
  }
  if (t == 0 && c == 0) {
    bounds[0] = base_seen;
    if (item_cost == 0)
      for (int x = 1; x < kXcds; ++x) bounds[x] = base_seen;
  }
  if (t == 0 && c == a.Ncam - 1) bounds[kXcds] = base_seen + a.seg_seen[s];
  int run = base_pairs;
  for (int t0 = 0; t0 < tiles; t0 += kScanThreads) {
    const int64_t i = (int64_t)s * tiles + t0 + t;
    const int v = t0 + t < tiles ? a.tile_counts[i] : 0;
    const int excl = block_exclusive_scan(v, &total);
    if (t0 + t < tiles) a.tile_offsets[i] = run + excl;
    run += total;
  }
  if (t == 0) {
    a.pair_offsets[s] = base_pairs;
    if (s == segs - 1) {
      a.pair_offsets[segs] = base_pairs + a.seg_pairs[s];
      a.bin_offsets[(int64_t)segs * kOrderBins] = base_seen + a.seg_seen[s];
    }
  }
}

__global__ __launch_bounds__(kTile) void sca_compact_kernel(CompactArgs a, int tiles) {
  __shared__ int wave_counts[kTileWaves][32];
  __shared__ int tile_start[32];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int q = tile * kTile + (int)threadIdx.x;
  const int64_t bq = (int64_t)b * a.Nq + q;
  if ((int)threadIdx.x < a.Ncam)  // loaded alongside the masks, used after the ballots
    tile_start[threadIdx.x] = a.tile_offsets[((int64_t)b * a.Ncam + threadIdx.x) * tiles + tile];
  const uint32_t seen = q < a.Nq ? a.cammask[bq] : 0u;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int c = 0; c < a.Ncam; ++c) {
    const uint64_t bits = __ballot((seen >> c) & 1u);
    if (lane == 0) wave_counts[wave][c] = __popcll(bits);
  }
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int c = 0; c < a.Ncam; ++c) {
    const uint64_t bits = __ballot((seen >> c) & 1u);
    if ((seen >> c) & 1u) {
      int rank = __popcll(bits & below);
      for (int w = 0; w < wave; ++w) rank += wave_counts[w][c];
      a.pair_q[tile_start[c] + rank] = q;
    }
  }
  if (seen != 0u) {
    const int key = a.qkey[bq];
    // count the bin down: the slot is unique, and the histogram ends at zero
    const int slot = a.bin_offsets[key] + atomicSub(&a.bin_hist[key], 1) - 1;
    a.order[slot] = (int32_t)bq;
  }
}

hipError_t launch_sca_compact(const CompactArgs& a, int tiles, hipStream_t stream) {
  sca_clear_kernel<<<(a.clear_ints + kTile - 1) / kTile, kTile, 0, stream>>>(a.bin_hist, a.clear_ints);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(tiles, a.B);
  const bool word = (a.D % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.bev_mask) & 3u) == 0);
  if (word)
    sca_visibility_kernel<true><<<grid, kTile, 0, stream>>>(a, tiles);
  else
    sca_visibility_kernel<false><<<grid, kTile, 0, stream>>>(a, tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  sca_scan_kernel<<<a.B * a.Ncam, kScanThreads, 0, stream>>>(a, tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  sca_compact_kernel<<<grid, kTile, 0, stream>>>(a, tiles);
  return hipGetLastError();
}

}  // namespace msda
