// SCA visibility and compaction (the bev_mask rebatch of the Tencent Cloud
// SCA note, article 2321140: per camera, the ascending indices of the BEV
// queries the camera sees; and its hit count per query), plus the order in
// which the gather kernel visits the seen queries.
//
// Three small stream-ordered kernels:
//   0. clear: zero the ordering histogram and the per-segment totals;
//   1. visibility: per (b, q) the bit set of cameras that see q (any of the D
//      anchors marked), the hit count, per (b, c, tile of 256 queries) the
//      number of seen queries, and for a seen query its ordering bin: the
//      image tile (kOrderBinsX columns x kOrderBinsY rows, column-major) of
//      the first marked anchor of its first camera, within the segment
//      (b, first camera), and its rank among the bin's queries (the count
//      its histogram add returns: unique, in no fixed order);
//   2. compact, two kinds of blocks in one grid:
//      - one per (b, tile): each query writes its index at tile offset +
//        (seen queries before it in the tile) for every camera that sees it,
//        so each (b, c) list comes out in ascending order (deterministic, no
//        atomics); the tile offset is the pairs of the earlier segments and
//        of the earlier tiles of (b, c), summed from the visibility counts.
//        A seen query takes the slot (its bin's first entry + its rank) of
//        the work order, the bins' first entries scanned in LDS for the
//        segments the tile's queries start in.  The rank's order varies from
//        run to run, which changes only which wave computes which query,
//        never a result;
//      - one per segment (b, c): its pair offset, and the boundaries of the
//        dies' shares of the batch item's work list where the summed cost of
//        the bins crosses each eighth of the item's total (interpolating
//        inside the bin), so that every die gets the same estimated work.
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
constexpr int kBinsPerThread = kOrderBins / kTile;
static_assert(kBinsPerThread == 4, "a block scans one segment's bins, four (one int4) per thread");

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
  l.qrank = take(sizeof(int32_t) * nq);
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
      a.qrank[bq] = atomicAdd(&a.bin_hist[key], 1);
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

// Sum of x[lo, hi) over the lanes of a wave (every lane gets it).
template <typename T>
__device__ T wave_sum(const T* __restrict__ x, int64_t lo, int64_t hi) {
  const int lane = threadIdx.x % kWave;
  T v = 0;
  for (int64_t i = lo + lane; i < hi; i += kWave) v += x[i];
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// Exclusive scan of one value per thread over the block (kTile threads);
// also returns the block total.  wsum: kTileWaves entries of LDS.
template <typename T>
__device__ T block_exclusive_scan(T v, T* total, T* wsum) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  T incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const T u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTileWaves; ++w) {
    const T ws = wsum[w];
    before += w < wave ? ws : T(0);
    all += ws;
  }
  *total = all;
  return before + incl - v;
}

// Segment s = (b, c): its pair offset, and where its bins hold the targets
// of the dies' shares of batch item b's work list: share x starts where the
// summed cost, in work-list order, reaches x/8 of the item's total (inside a
// bin, by linear interpolation over its entries).  The item's first and last
// segments write its ends (and, with no cost at all, every boundary).
__device__ void segment_bounds(const CompactArgs& a, int b, int c) {
  __shared__ int wsum[kTileWaves];
  __shared__ unsigned long long wsum64[kTileWaves];
  const int t = threadIdx.x;
  const int s = b * a.Ncam + c, segs = a.B * a.Ncam;
  const int64_t item0 = (int64_t)b * a.Ncam;
  // uniform: seen queries and pairs of the segments before s (all items),
  // the item's cost before s and in all
  const int base_seen = wave_sum(a.seg_seen, 0, s);
  const int base_pairs = wave_sum(a.seg_pairs, 0, s);
  const uint64_t seg_base = wave_sum<unsigned long long>(
      reinterpret_cast<const unsigned long long*>(a.seg_cost), item0, s);
  const uint64_t item_cost = wave_sum<unsigned long long>(
      reinterpret_cast<const unsigned long long*>(a.seg_cost), item0, item0 + a.Ncam);
  const int64_t bin0 = (int64_t)s * kOrderBins + kBinsPerThread * t;
  const int4 n4 = reinterpret_cast<const int4*>(a.bin_hist + bin0)[0];
  const int count[kBinsPerThread] = {n4.x, n4.y, n4.z, n4.w};
  unsigned long long cost[kBinsPerThread];
  unsigned long long cost_sum = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    cost[i] = a.bin_cost[bin0 + i];
    cost_sum += cost[i];
  }
  int seg_total = 0;
  unsigned long long seg_cost_total = 0;
  int first = base_seen + block_exclusive_scan(n4.x + n4.y + n4.z + n4.w, &seg_total, wsum);
  uint64_t begin = seg_base + block_exclusive_scan(cost_sum, &seg_cost_total, wsum64);
  int32_t* bounds = a.die_bounds + (int64_t)b * kDieBounds;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    const uint64_t end = begin + cost[i];
    for (int x = 1; x < kXcds; ++x) {
      const uint64_t target = item_cost * (uint64_t)x / kXcds;
      if (cost[i] != 0 && target >= begin && target < end) {
        // entry of the bin at that fraction of its cost (double: no overflow
        // of cost x count; the clamp keeps it inside the bin)
        const int k = (int)((double)(target - begin) / (double)cost[i] * (double)count[i]);
        bounds[x] = first + min(max(k, 0), count[i] - 1);
      }
    }
    begin = end;
    first += count[i];
  }
  if (t == 0) {
    if (c == 0) {
      bounds[0] = base_seen;
      if (item_cost == 0)
        for (int x = 1; x < kXcds; ++x) bounds[x] = base_seen;
    }
    if (c == a.Ncam - 1) bounds[kXcds] = base_seen + seg_total;
    a.pair_offsets[s] = base_pairs;
    if (s == segs - 1) a.pair_offsets[segs] = base_pairs + a.seg_pairs[s];
  }
}

// Tile `tile` of batch item b: the pair lists' entries of its queries, its
// offsets in them (tile_offsets), and its seen queries' work-order slots.
__device__ void tile_compact(const CompactArgs& a, int b, int tile, int tiles) {
  __shared__ int wave_counts[kTileWaves][32];
  __shared__ int tile_start[32];
  __shared__ int seen_before[32];  // seen queries of the segments before (b, c), all items
  __shared__ uint32_t wave_firsts[kTileWaves];
  __shared__ int wsum[kTileWaves];
  __shared__ int bin_first[kOrderBins];
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int q = tile * kTile + t;
  const int64_t bq = (int64_t)b * a.Nq + q;
  const uint32_t seen = q < a.Nq ? a.cammask[bq] : 0u;
  int key = 0, rank = 0;
  if (seen != 0u) {
    key = a.qkey[bq];
    rank = a.qrank[bq];
  }
  // per camera (one wave each): the tile's first pair in the lists, after
  // the pairs of the earlier segments and of the earlier tiles of (b, c)
  for (int c = wave; c < a.Ncam; c += kTileWaves) {
    const int s = b * a.Ncam + c;
    const int before = wave_sum(a.seg_pairs, 0, s) + wave_sum(a.tile_counts, (int64_t)s * tiles,
                                                              (int64_t)s * tiles + tile);
    const int seen_b = wave_sum(a.seg_seen, 0, s);
    if (lane == 0) {
      tile_start[c] = before;
      seen_before[c] = seen_b;
      a.tile_offsets[(int64_t)s * tiles + tile] = before;
    }
  }
  const int first = seen != 0u ? __builtin_ctz(seen) : -1;
  uint32_t firsts = 0u;  // first cameras of the wave's seen queries
  for (int c = 0; c < a.Ncam; ++c) {
    const uint64_t bits = __ballot((seen >> c) & 1u);
    if (__ballot(first == c) != 0ull) firsts |= 1u << c;
    if (lane == 0) wave_counts[wave][c] = __popcll(bits);
  }
  if (lane == 0) wave_firsts[wave] = firsts;
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int c = 0; c < a.Ncam; ++c) {
    const uint64_t bits = __ballot((seen >> c) & 1u);
    if ((seen >> c) & 1u) {
      int r = __popcll(bits & below);
      for (int w = 0; w < wave; ++w) r += wave_counts[w][c];
      // the tile's count from the visibility kernel bounds its run of (b, c)'s list
      MSDA_CHECK(kCheckPairWrite, q < a.Nq && r < a.tile_counts[(int64_t)(b * a.Ncam + c) * tiles + tile] &&
                                      (int64_t)tile_start[c] + r < (int64_t)a.B * a.Ncam * a.Nq);
      a.pair_q[tile_start[c] + r] = q;
    }
  }
  // work-order slots, segment by segment of the tile's first cameras: the
  // bin's first entry (seen queries before it) + the query's rank in the bin
  uint32_t need = 0u;
#pragma unroll
  for (int w = 0; w < kTileWaves; ++w) need |= wave_firsts[w];
  for (; need != 0u; need &= need - 1u) {
    const int c = __builtin_ctz(need);
    const int s = b * a.Ncam + c;
    const int4 n4 = reinterpret_cast<const int4*>(a.bin_hist + (int64_t)s * kOrderBins)[t];
    int total = 0;
    const int at = seen_before[c] + block_exclusive_scan(n4.x + n4.y + n4.z + n4.w, &total, wsum);
    bin_first[kBinsPerThread * t] = at;
    bin_first[kBinsPerThread * t + 1] = at + n4.x;
    bin_first[kBinsPerThread * t + 2] = at + n4.x + n4.y;
    bin_first[kBinsPerThread * t + 3] = at + n4.x + n4.y + n4.z;
    __syncthreads();
    if (first == c) {
      const int bin = key - s * kOrderBins;
      MSDA_CHECK(kCheckOrderWrite, bin >= 0 && bin < kOrderBins);
      const int slot = bin_first[bin < 0 ? 0 : (bin < kOrderBins ? bin : kOrderBins - 1)] + rank;
      // the segment's seen queries fill [seen_before, seen_before + total) of the list
      MSDA_CHECK(kCheckOrderWrite, slot >= seen_before[c] && slot < seen_before[c] + total &&
                                       (int64_t)slot < (int64_t)a.B * a.Nq);
      a.order[slot] = (int32_t)bq;
    }
    __syncthreads();  // bin_first is rewritten for the next segment
  }
}

// Grid (tiles + Ncam, B): blocks x < tiles are tiles, the rest segments.
__global__ __launch_bounds__(kTile) void sca_compact_kernel(CompactArgs a, int tiles) {
  const int b = blockIdx.y;
  if ((int)blockIdx.x < tiles)
    tile_compact(a, b, blockIdx.x, tiles);
  else
    segment_bounds(a, b, (int)blockIdx.x - tiles);
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
  sca_compact_kernel<<<dim3(tiles + a.Ncam, a.B), kTile, 0, stream>>>(a, tiles);
  return hipGetLastError();
}

}  // namespace msda
