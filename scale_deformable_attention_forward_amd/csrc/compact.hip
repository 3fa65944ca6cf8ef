// SCA visibility and compaction (the bev_mask rebatch of the Tencent Cloud
// SCA note, article 2321140: per camera, the ascending indices of the BEV
// queries the camera sees; and its hit count per query), plus the order in
// which the gather kernel visits the seen queries.
//
// Four small stream-ordered kernels:
//   0. clear: zero the ordering histogram;
//   1. visibility: per (b, q) the bit set of cameras that see q (any of the D
//      anchors marked), the hit count, per (b, c, tile of 256 queries) the
//      number of seen queries, and for a seen query its ordering bin: the
//      image tile (kOrderBinsX columns x kOrderBinsY rows, column-major) of
//      the first marked anchor of its first camera, within the segment
//      (b, first camera);
//   2. scan: one workgroup turns the tile counts (in b, c, tile order) into
//      exclusive offsets -- pair_offsets[b*Ncam + c] is the offset of the
//      first tile of (b, c) and pair_offsets[B*Ncam] the total -- and the
//      bin histogram into bin offsets;
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

constexpr int kTile = 256;  // queries per tile = threads per block
constexpr int kTileWaves = kTile / kWave;
constexpr int kScanThreads = 1024;

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
  l.bin_hist = take(sizeof(int32_t) * segs * kOrderBins);
  l.bin_offsets = take(sizeof(int32_t) * (segs * kOrderBins + 1));
  l.order = take(sizeof(int32_t) * nq);
  l.total = o;
  return l;
}

__global__ __launch_bounds__(kTile) void sca_clear_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * kTile + threadIdx.x;
  if (i < n) p[i] = 0;
}

__device__ inline int tile_bin(float v, int n) {
  const float t = fminf(fmaxf(v, 0.f), 1.f) * (float)n;  // NaN -> 0
  return min((int)t, n - 1);
}

template <bool kWordMask>
__global__ __launch_bounds__(kTile) void sca_visibility_kernel(CompactArgs a, int tiles) {
  __shared__ int wave_counts[kTileWaves][32];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int q = tile * kTile + (int)threadIdx.x;
  const bool in_range = q < a.Nq;
  uint32_t seen = 0;
  int first_anchor = 0;
  if (in_range) {
    for (int c = 0; c < a.Ncam; ++c) {
      const int64_t at = (((int64_t)c * a.B + b) * a.Nq + q) * a.D;
      int marked = -1;  // first marked anchor of this camera
      if (kWordMask) {  // D % 4 == 0 and the mask is 4-byte aligned
        const uint32_t* m = reinterpret_cast<const uint32_t*>(a.bev_mask + at);
        for (int k = 0; k < a.D / 4 && marked < 0; ++k)
          if (m[k] != 0u) marked = 4 * k + __builtin_ctz(m[k]) / 8;
      } else {
        for (int k = 0; k < a.D && marked < 0; ++k)
          if (a.bev_mask[at + k] != 0) marked = k;
      }
      if (marked >= 0) {
        if (seen == 0u) first_anchor = marked;
        seen |= 1u << c;
      }
    }
    const int64_t bq = (int64_t)b * a.Nq + q;
    a.cammask[bq] = seen;
    if (a.hit_count) a.hit_count[bq] = __popc(seen);
    int key = -1;
    if (seen != 0u) {
      const int c0 = __builtin_ctz(seen);
      const float2 r = reinterpret_cast<const float2*>(a.rp)[(((int64_t)c0 * a.B + b) * a.Nq + q) * a.D + first_anchor];
      const int bin = tile_bin(r.x, kOrderBinsX) * kOrderBinsY + tile_bin(r.y, kOrderBinsY);
      key = (b * a.Ncam + c0) * kOrderBins + bin;
      atomicAdd(&a.bin_hist[key], 1);
    }
    a.qkey[bq] = key;
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int c = 0; c < a.Ncam; ++c) {
    const uint64_t bits = __ballot((seen >> c) & 1u);
    if (lane == 0) wave_counts[wave][c] = __popcll(bits);
  }
  __syncthreads();
  if ((int)threadIdx.x < a.Ncam) {
    const int c = threadIdx.x;
    int s = 0;
    for (int w = 0; w < kTileWaves; ++w) s += wave_counts[w][c];
    a.tile_counts[((int64_t)b * a.Ncam + c) * tiles + tile] = s;
  }
}

// Exclusive scan of in[0, n) into out[0, n) by one block of kScanThreads;
// returns the total in every thread.  `every`/`firsts`: out[i] is also
// written to firsts[i / every] when i % every == 0 (may be null).
__device__ int block_exclusive_scan(const int32_t* __restrict__ in, int32_t* __restrict__ out, int n, int every,
                                    int32_t* __restrict__ firsts, int* part) {
  const int t = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += in[i];
  __syncthreads();  // part[] may still be read by a previous scan
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {  // inclusive scan of the partial sums
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - s;
  for (int i = lo; i < hi; ++i) {
    if (firsts && i % every == 0) firsts[i / every] = run;
    out[i] = run;
    run += in[i];
  }
  return part[kScanThreads - 1];
}

__global__ __launch_bounds__(kScanThreads) void sca_scan_kernel(CompactArgs a, int tiles) {
  __shared__ int part[kScanThreads];
  const int segs = a.B * a.Ncam;
  const int pairs = block_exclusive_scan(a.tile_counts, a.tile_offsets, segs * tiles, tiles, a.pair_offsets, part);
  if (threadIdx.x == 0) a.pair_offsets[segs] = pairs;
  const int nbins = segs * kOrderBins;
  const int seen = block_exclusive_scan(a.bin_hist, a.bin_offsets, nbins, 1, nullptr, part);
  if (threadIdx.x == 0) a.bin_offsets[nbins] = seen;
}

__global__ __launch_bounds__(kTile) void sca_compact_kernel(CompactArgs a, int tiles) {
  __shared__ int wave_counts[kTileWaves][32];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int q = tile * kTile + (int)threadIdx.x;
  const int64_t bq = (int64_t)b * a.Nq + q;
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
      a.pair_q[a.tile_offsets[((int64_t)b * a.Ncam + c) * tiles + tile] + rank] = q;
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
  const int nbins = a.B * a.Ncam * kOrderBins;
  sca_clear_kernel<<<(nbins + kTile - 1) / kTile, kTile, 0, stream>>>(a.bin_hist, nbins);
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
  sca_scan_kernel<<<1, kScanThreads, 0, stream>>>(a, tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  sca_compact_kernel<<<grid, kTile, 0, stream>>>(a, tiles);
  return hipGetLastError();
}

}  // namespace msda
