// SCA visibility and compaction (the bev_mask rebatch of the Tencent Cloud
// SCA note, article 2321140: per camera, the ascending indices of the BEV
// queries the camera sees; and its hit count per query).
//
// Three small stream-ordered kernels, deterministic and atomic-free:
//   1. visibility: per (b, q) the bit set of cameras that see q (any of the D
//      anchors marked), the hit count, and per (b, c, tile of 256 queries)
//      the number of seen queries;
//   2. scan: one workgroup turns the tile counts (in b, c, tile order) into
//      exclusive offsets; pair_offsets[b*Ncam + c] is the offset of the
//      first tile of (b, c) and pair_offsets[B*Ncam] the total;
//   3. compact: each query writes its index at
//      tile offset + (seen queries before it in the tile) for every camera
//      that sees it, so each (b, c) segment comes out in ascending order.
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
  size_t o = 0;
  l.cammask = o;
  o = align_up(o + sizeof(uint32_t) * (size_t)(B * Nq), 256);
  l.tile_counts = o;
  o = align_up(o + sizeof(int32_t) * segs * (size_t)l.tiles, 256);
  l.tile_offsets = o;
  o = align_up(o + sizeof(int32_t) * segs * (size_t)l.tiles, 256);
  l.pair_offsets = o;
  o = align_up(o + sizeof(int32_t) * (segs + 1), 256);
  l.pair_q = o;
  o = align_up(o + sizeof(int32_t) * segs * (size_t)Nq, 256);
  l.total = o;
  return l;
}

template <bool kWordMask>
__global__ __launch_bounds__(kTile) void sca_visibility_kernel(CompactArgs a, int tiles) {
  __shared__ int wave_counts[kTileWaves][32];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int q = tile * kTile + (int)threadIdx.x;
  const bool in_range = q < a.Nq;
  uint32_t seen = 0;
  if (in_range) {
    for (int c = 0; c < a.Ncam; ++c) {
      const int64_t at = (((int64_t)c * a.B + b) * a.Nq + q) * a.D;
      uint32_t any = 0;
      if (kWordMask) {  // D % 4 == 0 and the mask is 4-byte aligned
        const uint32_t* m = reinterpret_cast<const uint32_t*>(a.bev_mask + at);
        for (int k = 0; k < a.D / 4; ++k) any |= m[k];
      } else {
        for (int k = 0; k < a.D; ++k) any |= a.bev_mask[at + k];
      }
      seen |= (any != 0u ? 1u : 0u) << c;
    }
    a.cammask[(int64_t)b * a.Nq + q] = seen;
    if (a.hit_count) a.hit_count[(int64_t)b * a.Nq + q] = __popc(seen);
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

__global__ __launch_bounds__(kScanThreads) void sca_scan_kernel(CompactArgs a, int tiles) {
  __shared__ int part[kScanThreads];
  const int n = a.B * a.Ncam * tiles;
  const int t = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += a.tile_counts[i];
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
    if (i % tiles == 0) a.pair_offsets[i / tiles] = run;
    a.tile_offsets[i] = run;
    run += a.tile_counts[i];
  }
  if (t == kScanThreads - 1) a.pair_offsets[a.B * a.Ncam] = part[t];
}

__global__ __launch_bounds__(kTile) void sca_compact_kernel(CompactArgs a, int tiles) {
  __shared__ int wave_counts[kTileWaves][32];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int q = tile * kTile + (int)threadIdx.x;
  const uint32_t seen = q < a.Nq ? a.cammask[(int64_t)b * a.Nq + q] : 0u;
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
}

hipError_t launch_sca_compact(const CompactArgs& a, int tiles, hipStream_t stream) {
  const dim3 grid(tiles, a.B);
  const bool word = (a.D % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.bev_mask) & 3u) == 0);
  if (word)
    sca_visibility_kernel<true><<<grid, kTile, 0, stream>>>(a, tiles);
  else
    sca_visibility_kernel<false><<<grid, kTile, 0, stream>>>(a, tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  sca_scan_kernel<<<1, kScanThreads, 0, stream>>>(a, tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  sca_compact_kernel<<<grid, kTile, 0, stream>>>(a, tiles);
  return hipGetLastError();
}

}  // namespace msda
