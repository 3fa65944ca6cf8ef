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
// A counting sort in four small stream-ordered kernels, spread over the
// chip (a single workgroup per batch item spent ~50 us fetching the points'
// cache lines through one compute unit):
//   0. clear the tile counters of every batch item;
//   1. count: one thread per query adds one to its tile's counter;
//   2. scan: one workgroup per batch item turns the counters into the first
//      slot of each tile;
//   3. place: every query takes the next slot of its tile (the order inside
//      a tile varies from run to run, which changes only which wave computes
//      a query, never a result).
#include "common.hpp"
#include "internal.hpp"

namespace msda {

constexpr int kPlanSide = 64;                     // tiles per side of the unit square
constexpr int kPlanThreads = 256;                 // count / place kernels
constexpr int kPlanScanThreads = kPlanBins / 4;   // 4 tiles per scan thread
static_assert(kPlanBins == kPlanSide * kPlanSide, "tile count");

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
  for (int bit = 0; bit < 6; ++bit) code |= (((tx >> bit) & 1) << (2 * bit)) | (((ty >> bit) & 1) << (2 * bit + 1));
  return code;
}

__global__ __launch_bounds__(kPlanThreads) void msda_plan_clear_kernel(int32_t* __restrict__ bins, int n) {
  const int i = blockIdx.x * kPlanThreads + threadIdx.x;
  if (i < n) bins[i] = 0;
}

__global__ __launch_bounds__(kPlanThreads) void msda_plan_count_kernel(PlanArgs a) {
  const int q = blockIdx.x * kPlanThreads + threadIdx.x, b = blockIdx.y;
  if (q >= a.Nq) return;
  atomicAdd(&a.bins[(int64_t)b * kPlanBins + plan_bin(a.points, b * a.batch_stride + q * a.point_stride)], 1);
}

__global__ __launch_bounds__(kPlanScanThreads) void msda_plan_scan_kernel(PlanArgs a) {
  __shared__ int wave_sums[kPlanScanThreads / kWave];
  int32_t* bins = a.bins + (int64_t)blockIdx.x * kPlanBins;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  int own[4], sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    own[u] = bins[4 * t + u];
    sum += own[u];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  int start = incl - sum;
  for (int w = 0; w < wave; ++w) start += wave_sums[w];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    bins[4 * t + u] = start;
    start += own[u];
  }
}

__global__ __launch_bounds__(kPlanThreads) void msda_plan_place_kernel(PlanArgs a) {
  const int q = blockIdx.x * kPlanThreads + threadIdx.x, b = blockIdx.y;
  if (q >= a.Nq) return;
  const int bin = plan_bin(a.points, b * a.batch_stride + q * a.point_stride);
  const int slot = atomicAdd(&a.bins[(int64_t)b * kPlanBins + bin], 1);
  a.order[(int64_t)b * a.Nq + slot] = (int32_t)((int64_t)b * a.Nq + q);
}

hipError_t launch_msda_plan(const PlanArgs& a, hipStream_t stream) {
  const int n = a.B * kPlanBins;
  msda_plan_clear_kernel<<<(n + kPlanThreads - 1) / kPlanThreads, kPlanThreads, 0, stream>>>(a.bins, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((a.Nq + kPlanThreads - 1) / kPlanThreads, a.B);
  msda_plan_count_kernel<<<grid, kPlanThreads, 0, stream>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  msda_plan_scan_kernel<<<a.B, kPlanScanThreads, 0, stream>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  msda_plan_place_kernel<<<grid, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace msda
