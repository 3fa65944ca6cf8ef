// Locality plan of the multi-scale deformable attention operator: the
// order in which the gather visits the queries of a batch item.
//
// The operator's sampling locations cluster around each query's reference
// point on every level ("BEV(三) BEVFormer：Query 参数如何与 Feature 的 8 个
// Head 交互", sections 4.3 and 5: offsets of a few cells around the
// reference point).  Queries that arrive in an order unrelated to position
// (random reference points, or any other caller order) make consecutive
// work items read unrelated value rows, and every die's L2 then holds the
// whole map in turn.  The plan sorts each batch item's queries by the
// image tile (kPlanSide x kPlanSide tiles of the normalised square) of one
// point standing for the query, tiles taken in Morton order: the gather's
// split of a batch item's list into eight contiguous shares then gives each
// die a compact region of the maps.
//
// A counting sort in two stream-ordered kernels over kPlanChunks chunks of
// each batch item's queries (kernel launches, not the sort's work, are what
// a small plan costs: four kernels took ~18 us for 20,000 queries, one
// workgroup per batch item ~50 us, its points' cache lines all fetched
// through one compute unit):
//   1. count: each chunk's workgroup builds its tile histogram in LDS and
//      writes all of it (no clearing needed);
//   2. place: each chunk's workgroup reads every chunk's histogram, forms in
//      LDS the first slot of each tile for its own chunk (the queries of
//      earlier tiles, then those of the same tile in earlier chunks), and
//      each of its queries takes the next slot of its tile (LDS atomics: the
//      order inside a tile and chunk varies from run to run, which changes
//      only which wave computes a query, never a result).
#include "common.hpp"
#include "internal.hpp"

namespace msda {

constexpr int kPlanSide = 32;  // tiles per side of the unit square
constexpr int kPlanThreads = 1024;
constexpr int kPlanBits = 5;   // bits of a tile coordinate
static_assert(kPlanBins == kPlanSide * kPlanSide && kPlanBins == kPlanThreads && kPlanSide == 1 << kPlanBits,
              "one tile per thread");

__device__ inline int plan_tile(float v) {
  const float t = fminf(fmaxf(v, 0.f), 1.f) * (float)kPlanSide;  // NaN -> 0
  return min((int)t, kPlanSide - 1);
}

// Morton (Z-order) index of the tile of p: the bits of the row tile and the
// column tile interleaved, the row's above the column's at each level.
__device__ inline int plan_bin(const float* points, int64_t at) {
  const float2 p = *reinterpret_cast<const float2*>(points + at);
  const int tx = plan_tile(p.x), ty = plan_tile(p.y);
  int code = 0;
#pragma unroll
  for (int bit = 0; bit < kPlanBits; ++bit)
    code |= (((tx >> bit) & 1) << (2 * bit)) | (((ty >> bit) & 1) << (2 * bit + 1));
  return code;
}

// queries [lo, hi) of chunk c of a batch item
__device__ inline void chunk_range(int Nq, int c, int* lo, int* hi) {
  *lo = (int)((int64_t)Nq * c / kPlanChunks);
  *hi = (int)((int64_t)Nq * (c + 1) / kPlanChunks);
}

__global__ __launch_bounds__(kPlanThreads) void msda_plan_count_kernel(PlanArgs a) {
  __shared__ int hist[kPlanBins];
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  hist[t] = 0;
  __syncthreads();
  int lo, hi;
  chunk_range(a.Nq, c, &lo, &hi);
  for (int q = lo + t; q < hi; q += kPlanThreads)
    atomicAdd(&hist[plan_bin(a.points, b * a.batch_stride + q * a.point_stride)], 1);
  __syncthreads();
  a.bins[((int64_t)b * kPlanChunks + c) * kPlanBins + t] = hist[t];
}

__global__ __launch_bounds__(kPlanThreads) void msda_plan_place_kernel(PlanArgs a) {
  __shared__ int start[kPlanBins];
  __shared__ int wave_sums[kPlanThreads / kWave];
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  // thread t owns tile t: its total over all chunks and the count of the
  // chunks before this one
  const int32_t* hist = a.bins + (int64_t)b * kPlanChunks * kPlanBins + t;
  int n[kPlanChunks];
#pragma unroll
  for (int k = 0; k < kPlanChunks; ++k) n[k] = hist[(int64_t)k * kPlanBins];
  int total = 0, before = 0;
#pragma unroll
  for (int k = 0; k < kPlanChunks; ++k) {
    total += n[k];
    before += k < c ? n[k] : 0;
  }
  const int lane = t % kWave, wave = t / kWave;
  int incl = total;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  int first = incl - total;
  for (int w = 0; w < wave; ++w) first += wave_sums[w];
  start[t] = first + before;
  __syncthreads();
  int lo, hi;
  chunk_range(a.Nq, c, &lo, &hi);
  int32_t* order = a.order + (int64_t)b * a.Nq;
  for (int q = lo + t; q < hi; q += kPlanThreads) {
    const int bin = plan_bin(a.points, b * a.batch_stride + q * a.point_stride);
    order[atomicAdd(&start[bin], 1)] = (int32_t)((int64_t)b * a.Nq + q);
  }
}

hipError_t launch_msda_plan(const PlanArgs& a, hipStream_t stream) {
  const dim3 grid(kPlanChunks, a.B);
  msda_plan_count_kernel<<<grid, kPlanThreads, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  msda_plan_place_kernel<<<grid, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace msda
