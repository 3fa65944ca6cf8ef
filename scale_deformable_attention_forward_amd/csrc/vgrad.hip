// Value gradient of the backward pass as a transpose gather, with no atomics
// and a fixed summation order.
//
// "BEV(三) BEVFormer：Query 参数如何与 Feature 的 8 个 Head 交互" (sections 4.2,
// 6, 8) defines the forward as sums of alpha_k * w_c * V_c over the samples k
// of a query-head and the four corners c of each; so the gradient of a value
// row is the sum, over every (sample, corner) that reads the row, of
// alpha_k * w_c * g, g the upstream gradient of that query-head (for SCA
// divided by the query's hit count, section 10 of the same page and the
// Tencent Cloud SCA note, article 2321140).  Instead of scattering these
// terms with atomics:
//   1. the backward kernel writes one record per sample, at a slot fixed by
//      (image, head, pair, sample): records of one (image, head) form a
//      segment that starts on a sort tile.  A record holds the key of the
//      sample's corner (x0 + 1, y0 + 1) in the image's corner grids of
//      (W + 1) x (H + 1) keys per level (every sample with a corner inside
//      its map has such a key) and (source row, alpha, fx, fy);
//   2. a stable LSD radix sort of every segment at once (8-bit digits, two
//      passes for corner grids below 2^16 keys; a block ranks a tile of
//      kSortTile records in slot order with ballots, stages them in LDS in
//      digit order and writes each digit's run after the segment's records
//      of lower digits and the same digit's records of the segment's earlier
//      tiles, consecutive lanes to consecutive addresses) orders each
//      segment by key, dead samples dropped in the first pass (the host
//      launches the passes the bound 2 Nv + 2 L on the key count needs; the
//      setup kernel, which reads the level table, lets only the passes the
//      real count needs do work, and the others return at once);
//   3. the (first, end) range of every (segment, key) is recorded;
//   4. one 8-lane group per value row (pixel (x, y) of level l, head h)
//      sums, for the corners (dx, dy) = (0,0), (1,0), (0,1), (1,1) in turn,
//      the records of key (x + 1 - dx, y + 1 - dy) in sorted order (the four
//      lists walked as one sequence, 8 records per step, the next step's
//      records loading with this step's gradient rows), and writes the row
//      once.
// The order of every sum is fixed by the slots, so grad_value is the same
// bit for bit from run to run.
#include "common.hpp"
#include "internal.hpp"
#include "sampling.hpp"
#include "vgrad.hpp"

namespace msda {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

VgradLayout vgrad_layout(int64_t images, int64_t Nv, int L, int nH, int64_t records, int64_t pair_of_entries,
                         int64_t per_segment) {
  VgradLayout l = {};
  l.segments = images * nH;
  // every segment starts on a tile: with per_segment records each, exactly
  // that many tiles; otherwise at most one partly used tile each
  l.sort_tiles = per_segment > 0 ? l.segments * ((per_segment + kSortTile - 1) / kSortTile)
                                 : (records + kSortTile - 1) / kSortTile + l.segments;
  // a multiple of kHistTiles, so that each digit's counts of a histogram
  // block's tiles are one aligned run
  l.sort_tiles = (l.sort_tiles + kHistTiles - 1) / kHistTiles * kHistTiles;
  l.slots = l.sort_tiles * kSortTile;
  // (W + 1)(H + 1) <= 2 W H + 2 for W, H >= 1, so a level table whose maps fit
  // in Nv rows has at most 2 Nv + 2 L corner keys per image and head
  const int64_t corners = 2 * Nv + 2 * (int64_t)L;
  l.key_bound = l.segments * corners;
  int bits = 1;
  while (bits < 62 && ((int64_t)1 << bits) < corners) ++bits;
  l.passes = (bits + kDigitBits - 1) / kDigitBits;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  l.keys[0] = take(sizeof(uint32_t) * (size_t)l.slots);
  l.keys[1] = take(sizeof(uint32_t) * (size_t)l.slots);
  l.vals[0] = take(sizeof(VgradRec) * (size_t)l.slots);
  l.vals[1] = take(sizeof(VgradRec) * (size_t)l.slots);
  l.counts = take(sizeof(uint32_t) * (size_t)kDigits * (size_t)l.sort_tiles);
  l.tile_seg = take(sizeof(int32_t) * (size_t)l.sort_tiles);
  l.digit_totals = take(sizeof(uint32_t) * kDigits * (size_t)l.segments);
  l.seg_tile = take(sizeof(int32_t) * (size_t)(l.segments + 1));
  l.seg_items = take(sizeof(int32_t) * (size_t)l.segments);
  l.seg_live = take(sizeof(int32_t) * (size_t)l.segments);
  l.pair_start = take(sizeof(int32_t) * (size_t)images);
  l.ranges = take(sizeof(int2) * (size_t)l.key_bound);
  l.long_row = take((size_t)images * (size_t)Nv * (size_t)nH);
  l.pair_of = take(sizeof(int32_t) * (size_t)pair_of_entries);
  l.state = take(sizeof(VgradState));
  l.total = o;
  return l;
}

// ---------------------------------------------------------------------------
// block scan used by setup and the sort passes
// ---------------------------------------------------------------------------
constexpr int kSortBlock = 256;                   // threads per tile, one per digit
constexpr int kSortPer = kSortTile / kSortBlock;  // records per thread
static_assert(kSortBlock == kDigits, "one thread per digit");

// Exclusive scan of one value per thread over a kSortBlock block; *total is
// the block's sum.  Synchronises.
__device__ inline uint32_t sort_block_scan(uint32_t v, uint32_t* total) {
  __shared__ uint32_t wave_sums[kSortBlock / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  __syncthreads();  // wave_sums may still be read by a previous scan
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSortBlock / kWave; ++w) {
    before += w < wave ? wave_sums[w] : 0u;
    all += wave_sums[w];
  }
  *total = all;
  return before + incl - v;
}

// ---------------------------------------------------------------------------
// setup: state, SCA pair indices
// ---------------------------------------------------------------------------
// One block of kSortBlock threads: the state, and the segments: the pairs of
// each image (MSDA: its Nq queries; SCA: its (b, c) pair list, cut at
// max_pairs), each segment's record slots and first tile, and the segment of
// every tile (each thread writes its segment's).
__global__ __launch_bounds__(kSortBlock) void vgrad_setup_kernel(VgradArgs a, int sca) {
  __shared__ Level lv[kMaxLevels];
  __shared__ long long ext[kMaxLevels + 1];
  load_levels(a.shapes, a.starts, a.L, lv);
  load_corner_starts(lv, a.L, ext);
  const int t = threadIdx.x;
  int status = 0;
  const long long per_image = ext[a.L];  // corner keys per image and head
  if (per_image >= (long long)kDeadKey || per_image > a.key_bound / a.segments) status |= kVgradKeysOverflow;
  // SCA: the pair lists end where the last tile of the last (b, c) segment ends
  const int64_t last = (int64_t)a.B * a.Ncam * a.tiles - 1;
  const int64_t all_pairs = sca ? (last >= 0 ? (int64_t)a.tile_offsets[last] + a.tile_counts[last] : 0) : 0;
  if (sca && all_pairs > a.max_pairs) status |= kVgradPairsOverflow;
  int64_t run = 0;  // tiles of the segments before the current chunk
  for (int64_t s0 = 0; s0 < a.segments; s0 += kSortBlock) {
    const int64_t s = s0 + t;
    int64_t tiles = 0;
    if (s < a.segments) {
      const int64_t image = s / a.nH;
      int64_t first = image * a.Nq, n = a.Nq;
      if (sca) {
        first = 0;
        n = 0;
        if (a.tiles > 0) {
          first = a.tile_offsets[image * a.tiles];
          const int64_t end = image + 1 < a.images ? (int64_t)a.tile_offsets[(image + 1) * a.tiles] : all_pairs;
          const int64_t f = first < a.max_pairs ? first : a.max_pairs, e = end < a.max_pairs ? end : a.max_pairs;
          n = e > f ? e - f : 0;
        }
      }
      if (s % a.nH == 0) a.pair_start[image] = (int32_t)first;
      const int64_t items = n * a.LP;
      a.seg_items[s] = (int32_t)items;
      tiles = (items + kSortTile - 1) / kSortTile;
    }
    uint32_t chunk = 0;
    const uint32_t before = sort_block_scan((uint32_t)tiles, &chunk);
    if (s < a.segments) {
      // never past the capacity (the caller sized it), clamped regardless
      const int64_t at = run + before < a.sort_tiles ? run + before : a.sort_tiles;
      const int64_t end = at + tiles < a.sort_tiles ? at + tiles : a.sort_tiles;
      a.seg_tile[s] = (int32_t)at;
      for (int64_t tile = at; tile < end; ++tile) a.tile_seg[tile] = (int32_t)s;  // the segment of its tiles
    }
    run += chunk;
  }
  if (run > a.sort_tiles) status |= kVgradPairsOverflow;
  if (t == 0) {
    a.seg_tile[a.segments] = (int32_t)(run < a.sort_tiles ? run : a.sort_tiles);
    a.state->corner_keys = per_image;
    // digit passes the keys below per_image need (the host launches enough
    // for the bound 2 Nv + 2 L; the launches past these return at once)
    int bits = 1;
    while (bits < 62 && (1ll << bits) < per_image) ++bits;
    const int need = (bits + kDigitBits - 1) / kDigitBits;
    a.state->passes = need < a.passes ? need : a.passes;
    a.state->sorted = 0;
    a.state->tiles = run < a.sort_tiles ? run : a.sort_tiles;
    a.state->status = status;
  }
}

// pair_of[c][b][q] = index of (b, c, q) in the compaction's pair lists: the
// tile's offset in the (b, c) list plus the seen queries before q in the tile
// (the ranking of sca_compact_kernel)
__global__ __launch_bounds__(kQueryTile) void vgrad_pair_of_kernel(VgradArgs a) {
  constexpr int kTileWaves = kQueryTile / kWave;
  __shared__ int wave_counts[kTileWaves][32];
  __shared__ int tile_start[32];
  const int tile = blockIdx.x, b = blockIdx.y;
  const int q = tile * kQueryTile + (int)threadIdx.x;
  const int64_t bq = (int64_t)b * a.Nq + q;
  if ((int)threadIdx.x < a.Ncam)
    tile_start[threadIdx.x] = a.tile_offsets[((int64_t)b * a.Ncam + threadIdx.x) * a.tiles + tile];
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
      a.pair_of[((int64_t)c * a.B + b) * a.Nq + q] = tile_start[c] + rank;
    }
  }
}

// ---------------------------------------------------------------------------
// radix sort passes: block b ranks and writes tile b (slots b * kSortTile ..)
// of the segment the tile belongs to
// ---------------------------------------------------------------------------
__device__ inline uint32_t digit_of(uint32_t key, int shift) { return (key >> shift) & (kDigits - 1); }

// Where tile `tile` lies: its segment s, the segment's first slot and the
// records of the segment from the tile's first slot on (the backward
// kernel's slots before the first pass, the live records after it).
struct TileInSegment {
  int64_t s, seg0, n;
};
template <bool kFirst>
__device__ inline TileInSegment tile_in_segment(const VgradArgs& a, int64_t tile) {
  TileInSegment r;
  r.s = a.tile_seg[tile];
  r.seg0 = (int64_t)a.seg_tile[r.s] * kSortTile;
  r.n = (int64_t)(kFirst ? a.seg_items[r.s] : a.seg_live[r.s]) - (tile * kSortTile - r.seg0);
  return r;
}

// digit counts of each tile in use -> counts[digit][tile]; block b counts
// the tiles b * kHistTiles .. + kHistTiles - 1 and writes each digit's counts
// of them as one run
template <bool kFirst>
__global__ __launch_bounds__(kSortBlock) void vgrad_hist_kernel(VgradArgs a, int src, int shift) {
  __shared__ uint32_t h[kHistTiles][kDigits];
  __shared__ int64_t tile_n[kHistTiles];
  const int64_t used = uniform(a.seg_tile[a.segments]);
  const int64_t tile0 = (int64_t)blockIdx.x * kHistTiles;
  if (tile0 >= used || shift >= kDigitBits * uniform(a.state->passes)) return;
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kHistTiles; ++u) h[u][t] = 0u;
  // records of each tile (0 past the tiles in use)
  if (t < kHistTiles) tile_n[t] = tile0 + t < used ? tile_in_segment<kFirst>(a, tile0 + t).n : 0;
  __syncthreads();
  const uint32_t* keys = a.keys[src];
  uint32_t k[kHistTiles][kSortPer];
#pragma unroll
  for (int u = 0; u < kHistTiles; ++u) {
    const int64_t n = tile_n[u];
#pragma unroll
    for (int e = 0; e < kSortPer; ++e) {
      const int i = e * kSortBlock + t;
      k[u][e] = i < n ? keys[(tile0 + u) * kSortTile + i] : kDeadKey;
    }
  }
#pragma unroll
  for (int u = 0; u < kHistTiles; ++u)
#pragma unroll
    for (int e = 0; e < kSortPer; ++e)
      if (k[u][e] != kDeadKey) atomicAdd(&h[u][digit_of(k[u][e], shift)], 1u);
  __syncthreads();
  uint32_t* row = a.counts + (int64_t)t * a.sort_tiles + tile0;  // kHistTiles-aligned: sort_tiles is a multiple
#pragma unroll
  for (int u = 0; u < kHistTiles; ++u) row[u] = h[u][t];
}

// Block (s, g), 4 waves: wave w scans digit d = 4 g + w over segment s's
// tiles, counts[d][tile] -> the exclusive offset of the tile's d-records in
// the segment's d-records; digit_totals[s][d] = the segment's d-records.
__global__ __launch_bounds__(kSortBlock) void vgrad_scan_kernel(VgradArgs a, int shift) {
  if (shift >= kDigitBits * uniform(a.state->passes)) return;
  const int64_t s = blockIdx.x;
  const int d = (int)blockIdx.y * (kSortBlock / kWave) + (int)threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t0 = a.seg_tile[s], tiles = a.seg_tile[s + 1] - t0;
  uint32_t* row = a.counts + (int64_t)d * a.sort_tiles + t0;
  const int64_t per = (tiles + kWave - 1) / kWave;  // tiles per lane, contiguous
  const int64_t c0 = lane * per, c1 = c0 + per < tiles ? c0 + per : tiles;
  uint32_t sum = 0;
  for (int64_t c = c0; c < c1; ++c) sum += row[c];
  uint32_t incl = sum;
#pragma unroll
  for (int k = 1; k < kWave; k <<= 1) {
    const uint32_t y = __shfl_up(incl, k);
    if (lane >= k) incl += y;
  }
  uint32_t run = incl - sum;
  for (int64_t c = c0; c < c1; ++c) {
    const uint32_t v = row[c];
    row[c] = run;
    run += v;
  }
  if (lane == kWave - 1) a.digit_totals[s * kDigits + d] = incl;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Stable scatter of a tile.  Wave w ranks the tile's records w * 512 ..
// w * 512 + 511 in slot order, 64 at a time (ballots give the lanes with the
// same digit; the wave's own digit counts in LDS the records before), the
// waves' counts give each wave's offset within a digit, and the records are
// placed in LDS in (digit, rank) order and written out in that order: the tile's
// records of digit d go to consecutive addresses after every record of the
// segment with a lower digit and after digit d's records of the segment's
// earlier tiles.  Blocks are persistent (tiles blockIdx.x, + gridDim.x, ...):
// the next tile's keys load while this tile is ranked, its records while
// this tile is written.
template <bool kFirst>
__global__ __launch_bounds__(kSortBlock) void vgrad_scatter_kernel(VgradArgs a, int src, int shift) {
  constexpr int kWaves = kSortBlock / kWave;
  __shared__ uint32_t skeys[kSortTile];
  __shared__ VgradRec svals[kSortTile];
  __shared__ uint32_t cnt[kWaves][kDigits];
  __shared__ uint32_t local_off[kDigits];
  __shared__ uint32_t base[kDigits];
  const int64_t used = uniform(a.seg_tile[a.segments]);
  int64_t tile = blockIdx.x;
  if (tile >= used || shift >= kDigitBits * uniform(a.state->passes)) return;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  if (tile == 0 && t == 0) a.state->sorted = src ^ 1;  // read by the kernels after the sort
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  const uint32_t* keys = a.keys[src];
  const VgradRec* vals = a.vals[src];
  // stores through descriptors sized to the buffers: a position past the end
  // is dropped by the hardware
  const int dst = src ^ 1;
  const auto okeys = make_rsrc(a.keys[dst], (uint32_t)(a.sort_tiles * kSortTile * sizeof(uint32_t)));
  const auto ovals = make_rsrc(a.vals[dst], (uint32_t)(a.sort_tiles * kSortTile * sizeof(VgradRec)));

  // the next tile's keys (dead past its segment's records) and records
  uint32_t k[kSortPer];
  VgradRec v[kSortPer];
  TileInSegment ts = tile_in_segment<kFirst>(a, tile);
  // wave w holds the tile's records w * kWavePer + u * kWave + lane, u < kSortPer
  constexpr int kWavePer = kSortTile / kWaves;
  const int mine = wave * kWavePer + lane;
  auto fetch_keys = [&](int64_t tl, const TileInSegment& x, uint32_t (&kk)[kSortPer]) {
    const int64_t n = uniform(x.n);
#pragma unroll
    for (int u = 0; u < kSortPer; ++u) {
      const int i = mine + u * kWave;
      kk[u] = i < n ? keys[tl * kSortTile + i] : kDeadKey;
    }
  };
  auto fetch_vals = [&](int64_t tl, const uint32_t (&kk)[kSortPer], VgradRec (&vv)[kSortPer]) {
#pragma unroll
    for (int u = 0; u < kSortPer; ++u)
      vv[u] = kk[u] != kDeadKey ? vals[tl * kSortTile + mine + u * kWave] : VgradRec{0u, 0.f, 0.f, 0.f};
  };
  fetch_keys(tile, ts, k);
  fetch_vals(tile, k, v);

  for (;;) {
    const int64_t next = tile + gridDim.x;
    const bool more = next < used;
    TileInSegment tn = ts;
    uint32_t kn[kSortPer];
    if (more) {
      tn = tile_in_segment<kFirst>(a, next);
      fetch_keys(next, tn, kn);
    }

    // where digit t's records of this tile start: after the segment's records
    // of lower digits and the digit's records of the segment's earlier tiles
    uint32_t all = 0;
    const uint32_t lower = sort_block_scan(a.digit_totals[ts.s * kDigits + t], &all);
    base[t] = (uint32_t)ts.seg0 + lower + a.counts[(int64_t)t * a.sort_tiles + tile];
    if (kFirst && tile * kSortTile == ts.seg0 && t == 0) a.seg_live[ts.s] = (int32_t)all;  // survivors of pass 1
    // each wave ranks its own records against its own digit counts
    // (cnt[wave][d]: its records of digit d so far); the waves' counts are
    // then turned into each wave's offset within the digit
    uint32_t rank[kSortPer];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) cnt[w][t] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSortPer; ++u) {
      const bool live = k[u] != kDeadKey;
      const uint32_t d = digit_of(k[u], shift);
      uint64_t peers = __ballot(live);  // live lanes of this wave with the same digit
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool set = (d >> bit) & 1u;
        const uint64_t m = __ballot(set);
        peers &= set ? m : ~m;
      }
      const uint32_t before_me = live ? cnt[wave][d] : 0u;  // read by every peer before the leader adds
      wave_lds_sync();
      if (live) rank[u] = before_me + (uint32_t)__popcll(peers & below);
      if (live && (peers & below) == 0ull) cnt[wave][d] = before_me + (uint32_t)__popcll(peers);
      wave_lds_sync();
    }
    __syncthreads();
    uint32_t digit_all = 0;  // digit t's records in the tile; cnt[w][t] becomes wave w's offset in the digit
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = cnt[w][t];
      cnt[w][t] = digit_all;
      digit_all += c;
    }
    uint32_t tile_live = 0;
    local_off[t] = sort_block_scan(digit_all, &tile_live);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSortPer; ++u) {
      if (k[u] == kDeadKey) continue;
      const uint32_t d = digit_of(k[u], shift);
      const uint32_t lp = local_off[d] + cnt[wave][d] + rank[u];
      skeys[lp] = k[u];
      svals[lp] = v[u];
    }
    __syncthreads();
    VgradRec vn[kSortPer];
    if (more) fetch_vals(next, kn, vn);
    for (uint32_t j = t; j < tile_live; j += kSortBlock) {
      const uint32_t key = skeys[j];
      const uint32_t d = digit_of(key, shift);
      const uint32_t pos = base[d] + (j - local_off[d]);
      const VgradRec r = svals[j];
      __builtin_amdgcn_raw_buffer_store_b32(key, okeys, pos * (uint32_t)sizeof(uint32_t), 0, 0);
      const u32x4 pv = {r.src, __float_as_uint(r.alpha), __float_as_uint(r.fx), __float_as_uint(r.fy)};
      __builtin_amdgcn_raw_buffer_store_b128(pv, ovals, pos * (uint32_t)sizeof(VgradRec), 0, 0);
    }
    if (!more) break;
    __syncthreads();  // the next tile rewrites the staging area and the digit tables
    tile = next;
    ts = tn;
#pragma unroll
    for (int u = 0; u < kSortPer; ++u) {
      k[u] = kn[u];
      v[u] = vn[u];
    }
  }
}

// ---------------------------------------------------------------------------
// key ranges and value rows
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void vgrad_clear_ranges_kernel(VgradArgs a) {
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < a.key_bound;
       k += (int64_t)gridDim.x * blockDim.x)
    a.ranges[k] = make_int2(0, 0);
}

// Block per tile: the (first, end) slots of each (segment, key) run of the
// sorted records.
__global__ __launch_bounds__(256) void vgrad_ranges_kernel(VgradArgs a) {
  const uint32_t* keys = a.keys[uniform(a.state->sorted) & 1];
  const int64_t tile = blockIdx.x;
  const long long next = a.state->corner_keys;
  if (tile < uniform(a.seg_tile[a.segments])) {
    const TileInSegment ts = tile_in_segment<false>(a, tile);
    const int64_t t0 = tile * kSortTile, end = t0 + (ts.n < kSortTile ? ts.n : kSortTile);
    const int64_t seg_end = t0 + ts.n;  // one past the segment's last record
    for (int64_t i = t0 + threadIdx.x; i < end; i += blockDim.x) {
      const uint32_t k = keys[i];
      const uint64_t key = segment_key(ts.s, next, k);
      if (key >= (uint64_t)a.key_bound) continue;
      if (i == ts.seg0 || keys[i - 1] != k) a.ranges[key].x = (int)i;
      if (i == seg_end - 1 || keys[i + 1] != k) a.ranges[key].y = (int)(i + 1);
    }
  }
}

// The four corner lists of a value row at one level, walked as one sequence:
// record i is list c's (i - p[c])-th, p[0] = 0.
struct RowLists {
  int2 r[4];
  int p1, p2, p3, T;
};

__device__ inline RowLists row_lists(const VgradArgs& a, const long long* ext, int l, int W, int64_t image, int x,
                                     int y, int h) {
  RowLists s;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint64_t key =
        segment_key(image * a.nH + h, ext[a.L], corner_key(ext[l], W, x + 1 - (c & 1), y + 1 - (c >> 1)));
    s.r[c] = key < (uint64_t)a.key_bound ? a.ranges[key] : make_int2(0, 0);
  }
  s.p1 = s.r[0].y - s.r[0].x;
  s.p2 = s.p1 + s.r[1].y - s.r[1].x;
  s.p3 = s.p2 + s.r[2].y - s.r[2].x;
  s.T = s.p3 + s.r[3].y - s.r[3].x;
  return s;
}

// Sum of alpha * w_c * g over the records [b, min(b + 8, i1)) of the
// sequence for b = i0, i0 + step, ... < i1, for the 8-lane group (lane j:
// channels 4j..4j+3): lane j loads record b + j (the next step's records
// load while this step's gradient rows do), the group shares (source row,
// coefficient), and every lane adds its 4 channels of the rows in record
// order.
__device__ inline float4 sum_records(const RowLists& s, int i0, int i1, int step, const VgradRec* __restrict__ vals,
                                     __amdgpu_buffer_rsrc_t grad, int j) {
  auto fetch = [&](int i, VgradRec& rec, int& c) {
    c = (i >= s.p1) + (i >= s.p2) + (i >= s.p3);
    const int at = c == 0 ? s.r[0].x + i : (c == 1 ? s.r[1].x + i - s.p1 : (c == 2 ? s.r[2].x + i - s.p2 : s.r[3].x + i - s.p3));
    rec = i < i1 ? vals[at] : VgradRec{0u, 0.f, 0.f, 0.f};  // (a step never reaches past b + 8)
  };
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  VgradRec cur;
  int ccur;
  fetch(i0 + j, cur, ccur);
  for (int b = i0; b < i1; b += step) {
    // the coefficient of corner c: alpha * (dx ? fx : 1 - fx) * (dy ? fy : 1 - fy)
    const float wx = (ccur & 1) ? cur.fx : 1.f - cur.fx, wy = (ccur >> 1) ? cur.fy : 1.f - cur.fy;
    const float coef_mine = b + j < i1 ? cur.alpha * wx * wy : 0.f;
    const uint32_t src_mine = cur.src;
    VgradRec nxt;
    int cn;
    fetch(b + step + j, nxt, cn);
    float coef[8];
    float4 g[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t src = (uint32_t)__shfl((int)src_mine, t, 8);
      coef[t] = __shfl(coef_mine, t, 8);
      const uint32_t at = b + t < i1 ? src * 128u + (uint32_t)j * 16u : kSkip;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(grad, at, 0, 0);
      g[t] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc.x = fmaf(coef[t], g[t].x, acc.x);
      acc.y = fmaf(coef[t], g[t].y, acc.y);
      acc.z = fmaf(coef[t], g[t].z, acc.z);
      acc.w = fmaf(coef[t], g[t].w, acc.w);
    }
    cur = nxt;
    ccur = cn;
  }
  return acc;
}

// The row passes visit value rows head-major: visit index r is (image, head,
// pixel) = (r / (nH Nv), r / Nv % nH, r % Nv), the gradient row
// (image * Nv + pixel) * nH + head.  Rows of one head read only that head's
// upstream-gradient rows, so the rows a die works on at a time need about
// (queries seeing one camera) x 128 bytes of them: they stay in its L2.
struct RowPlace {
  int64_t image, row;
  int pix, h;
};
__device__ inline RowPlace row_place(int64_t r, int Nv, int nH) {
  RowPlace p;
  const int64_t per_image = (int64_t)Nv * nH;
  p.image = r / per_image;
  const int rem = (int)(r - p.image * per_image);
  p.h = rem / Nv;
  p.pix = rem - p.h * Nv;
  p.row = (p.image * Nv + p.pix) * nH + p.h;
  return p;
}

// One 8-lane group per row: the first kRowChunk records of each of its level
// sequences; a row with more (at some level) is flagged for the long-row pass,
// which adds the rest.  Rows are split by die (block i runs on die i % 8): die
// x takes the contiguous eighth x of the visit order, so the upstream-gradient
// rows its records read share its L2.
__global__ __launch_bounds__(256) void vgrad_rows_kernel(VgradArgs a) {
  __shared__ Level lv[kMaxLevels];
  __shared__ long long ext[kMaxLevels + 1];
  load_levels(a.shapes, a.starts, a.L, lv);
  load_corner_starts(lv, a.L, ext);
  const int j = threadIdx.x % 8;
  const int64_t rows = a.images * (int64_t)a.Nv * a.nH;
  const int die = blockIdx.x % kXcds, local = blockIdx.x / kXcds, nlocal = gridDim.x / kXcds;
  const int64_t lo = rows * die / kXcds, hi = rows * (die + 1) / kXcds;
  const int64_t stride = (int64_t)nlocal * (blockDim.x / 8);
  const bool poisoned = uniform(a.state->status) != 0;
  const VgradRec* vals = a.vals[uniform(a.state->sorted) & 1];
  const auto grad = make_rsrc(a.grad_out, a.grad_out_bytes);
  for (int64_t r = lo + (int64_t)local * (blockDim.x / 8) + threadIdx.x / 8; r < hi; r += stride) {
    const RowPlace pl = row_place(r, a.Nv, a.nH);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    bool more = false;
    for (int l = 0; l < a.L; ++l) {
      const Level L = lv[l];
      const long long off = (long long)pl.pix - L.start;
      if (L.W <= 0 || off < 0 || off >= (long long)L.W * L.H) continue;
      const int y = (int)(off / L.W), x = (int)(off - (long long)y * L.W);
      const RowLists s = row_lists(a, ext, l, L.W, pl.image, x, y, pl.h);
      const float4 part = sum_records(s, 0, min(s.T, kRowChunk), 8, vals, grad, j);
      acc = make_float4(acc.x + part.x, acc.y + part.y, acc.z + part.z, acc.w + part.w);
      more |= s.T > kRowChunk;
    }
    if (poisoned) acc = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    reinterpret_cast<float4*>(a.grad_value)[pl.row * 8 + j] = acc;
    if (j == 0) a.long_row[r] = more ? 1 : 0;
  }
}

// Rows flagged by vgrad_rows_kernel: one wave per row at a time, its 8 groups
// taking the 8-record steps after the first kRowChunk records in turn (group
// g the steps g, g + 8, ...), summed across the groups in a fixed pairwise
// order and added to the first kRowChunk records' sum.  Rows are split by
// die as in vgrad_rows_kernel; inside a die, wave w looks at the rows
// w, w + waves, ... of its eighth (64 flags per look), so the consecutive
// long rows of a coarse level spread over the die's waves.
__global__ __launch_bounds__(256) void vgrad_long_rows_kernel(VgradArgs a) {
  __shared__ Level lv[kMaxLevels];
  __shared__ long long ext[kMaxLevels + 1];
  load_levels(a.shapes, a.starts, a.L, lv);
  load_corner_starts(lv, a.L, ext);
  if (uniform(a.state->status) != 0) return;  // every row is NaN already
  const int lane = threadIdx.x % kWave, g = lane / 8, j = lane % 8;
  const int64_t rows = a.images * (int64_t)a.Nv * a.nH;
  const int die = blockIdx.x % kXcds, local = blockIdx.x / kXcds, nlocal = gridDim.x / kXcds;
  const int64_t lo = rows * die / kXcds, hi = rows * (die + 1) / kXcds;
  const int64_t waves = (int64_t)nlocal * (blockDim.x / kWave);
  const int64_t w = (int64_t)local * (blockDim.x / kWave) + threadIdx.x / kWave;
  const VgradRec* vals = a.vals[uniform(a.state->sorted) & 1];
  const auto grad = make_rsrc(a.grad_out, a.grad_out_bytes);
  for (int64_t base = lo + w; base < hi; base += waves * kWave) {
    const int64_t mine = base + (int64_t)lane * waves;
    uint64_t todo = __ballot(mine < hi && a.long_row[mine] != 0);
    while (todo) {
      const int who = __builtin_ctzll(todo);
      todo &= todo - 1;
      const RowPlace pl = row_place(base + (int64_t)who * waves, a.Nv, a.nH);
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int l = 0; l < a.L; ++l) {
        const Level L = lv[l];
        const long long off = (long long)pl.pix - L.start;
        if (L.W <= 0 || off < 0 || off >= (long long)L.W * L.H) continue;
        const int y = (int)(off / L.W), x = (int)(off - (long long)y * L.W);
        const RowLists s = row_lists(a, ext, l, L.W, pl.image, x, y, pl.h);
        const float4 part = sum_records(s, kRowChunk + 8 * g, s.T, 64, vals, grad, j);
        acc = make_float4(acc.x + part.x, acc.y + part.y, acc.z + part.z, acc.w + part.w);
      }
#pragma unroll
      for (int d = 8; d < kWave; d <<= 1) {  // groups (0+1), (2+3), ..., then pairs of those
        acc.x += __shfl_xor(acc.x, d);
        acc.y += __shfl_xor(acc.y, d);
        acc.z += __shfl_xor(acc.z, d);
        acc.w += __shfl_xor(acc.w, d);
      }
      if (g == 0) {
        float4* out = reinterpret_cast<float4*>(a.grad_value) + pl.row * 8 + j;
        const float4 first = *out;
        *out = make_float4(first.x + acc.x, first.y + acc.y, first.z + acc.z, first.w + acc.w);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_vgrad_setup(const VgradArgs& a, bool sca, hipStream_t stream) {
  vgrad_setup_kernel<<<1, kSortBlock, 0, stream>>>(a, sca ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !sca || a.tiles == 0) return e;
  vgrad_pair_of_kernel<<<dim3(a.tiles, a.B), kQueryTile, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_vgrad_rows(const VgradArgs& a, hipStream_t stream) {
  // blocks past the tiles in use return at once; the scatter's blocks are
  // persistent: as many as are resident at once
  const unsigned hist_blocks = (unsigned)(a.sort_tiles / kHistTiles);
  static const int scatter_per_cu = [] {  // initialised once, by one thread
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, vgrad_scatter_kernel<false>, kSortBlock, 0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  const int64_t resident = (int64_t)device_cu_count() * scatter_per_cu;
  const unsigned scatter_blocks = (unsigned)(a.sort_tiles < resident ? a.sort_tiles : resident);
  int src = 0;
  for (int p = 0; p < a.passes; ++p) {
    const int shift = kDigitBits * p;
    if (p == 0)
      vgrad_hist_kernel<true><<<hist_blocks, kSortBlock, 0, stream>>>(a, src, shift);
    else
      vgrad_hist_kernel<false><<<hist_blocks, kSortBlock, 0, stream>>>(a, src, shift);
    vgrad_scan_kernel<<<dim3((unsigned)a.segments, kDigits / (kSortBlock / kWave)), kSortBlock, 0, stream>>>(a,
                                                                                                        shift);
    if (p == 0)
      vgrad_scatter_kernel<true><<<scatter_blocks, kSortBlock, 0, stream>>>(a, src, shift);
    else
      vgrad_scatter_kernel<false><<<scatter_blocks, kSortBlock, 0, stream>>>(a, src, shift);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    src ^= 1;
  }
  const int64_t cap = (int64_t)device_cu_count() * 8;
  int64_t blocks = (a.key_bound + 255) / 256;
  vgrad_clear_ranges_kernel<<<(unsigned)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap), 256, 0, stream>>>(a);
  vgrad_ranges_kernel<<<(unsigned)a.sort_tiles, 256, 0, stream>>>(a);
  const int64_t rows = a.images * (int64_t)a.Nv * a.nH;
  blocks = (rows + 31) / 32;  // 32 rows per block of 256 threads
  const int64_t row_cap = (int64_t)device_cu_count() * 16;
  blocks = blocks < row_cap ? blocks : row_cap;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;  // a multiple of the die count
  vgrad_rows_kernel<<<(unsigned)blocks, 256, 0, stream>>>(a);
  vgrad_long_rows_kernel<<<(unsigned)((device_cu_count() * 8 + kXcds - 1) / kXcds * kXcds), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace msda
