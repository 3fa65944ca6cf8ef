// C ABI of libmsda.so (declared in include/msda.h): argument checks on the
// host, then stream-ordered launches.  Nothing here allocates device memory
// or synchronises the host, except msda_check_counts in the checked build
// (a debugging call that waits for the device before reading its counters).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <vector>

#include "backward.hpp"
#include "gemm.hpp"
#include "internal.hpp"
#include "rebatch.hpp"
#include "vgrad.hpp"
#include "msda.h"

int msda::device_cu_count() {
  // initialised once (C++ guarantees one thread runs the initialiser)
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      return n;
    return 256;
  }();
  return cus;
}

namespace {

// the counter readers of the translation units (checked builds; see
// common.hpp), registered by their static initialisers at load time
std::mutex& check_mutex() {
  static std::mutex m;
  return m;
}
std::vector<msda::CheckReader>& check_readers() {
  static std::vector<msda::CheckReader> r;
  return r;
}

}  // namespace

bool msda::register_check_reader(CheckReader reader) {
  std::lock_guard<std::mutex> lock(check_mutex());
  check_readers().push_back(reader);
  return true;
}

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSDA_OK;
  return fail(MSDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kI31 = (int64_t)1 << 31;

// Checks shared by the MSDA-style entry points; pairs_ok: the entry point
// takes MSDA_BF16_PAIRS (the forward ones).
int check_common(const void* value, int value_dtype, const int64_t* shapes, const int64_t* starts, int64_t Nv,
                 int64_t Nq, int nH, int Dh, int L, int P, const void* out, uint32_t* image_bytes,
                 bool pairs_ok = false) {
  // with no queries nothing per query is read or written: those buffers may be null
  if (!value || !shapes || !starts || (!out && Nq != 0)) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (value_dtype == MSDA_BF16_PAIRS && !pairs_ok)
    return fail(MSDA_ERR_INVALID_ARG, "MSDA_BF16_PAIRS is taken by the forward entry points only");
  if (value_dtype != MSDA_F32 && value_dtype != MSDA_BF16 && value_dtype != MSDA_BF16_PAIRS)
    return fail(MSDA_ERR_INVALID_ARG, "value_dtype %d is not MSDA_F32, MSDA_BF16 or MSDA_BF16_PAIRS", value_dtype);
  if (Nv < 1 || Nq < 0 || nH < 1 || Dh < 1 || L < 1 || P < 1)
    return fail(MSDA_ERR_INVALID_ARG, "sizes must be positive (Nv=%lld Nq=%lld nH=%d Dh=%d L=%d P=%d)",
                (long long)Nv, (long long)Nq, nH, Dh, L, P);
  if (Dh != 32) return fail(MSDA_ERR_UNSUPPORTED, "head width Dh=%d: only 32 is supported", Dh);
  if (nH > 64) return fail(MSDA_ERR_UNSUPPORTED, "nH=%d: at most 64 heads", nH);
  if ((int64_t)L * P > 64) return fail(MSDA_ERR_UNSUPPORTED, "L*P=%lld: at most 64 points per head", (long long)L * P);
  if (Nv >= kI31 || Nq >= kI31) return fail(MSDA_ERR_UNSUPPORTED, "Nv and Nq must be below 2^31");
  // the head-pair layout stores every pixel twice
  const int64_t elem = value_dtype == MSDA_BF16 ? 2 : 4;
  const int64_t bytes = Nv * nH * Dh * elem;
  if (bytes >= kI31) return fail(MSDA_ERR_UNSUPPORTED, "one value image is %lld bytes; the limit is 2^31", (long long)bytes);
  if (!aligned(value, 16) || (Nq != 0 && !aligned(out, 16)))
    return fail(MSDA_ERR_INVALID_ARG, "value and output must be 16-byte aligned");
  *image_bytes = (uint32_t)bytes;
  return MSDA_OK;
}

int check_gemm_sizes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 1 || K < 1) return fail(MSDA_ERR_INVALID_ARG, "M >= 0, N >= 1 and K >= 1 required");
  if (K % 32 != 0 || K > 256 || N % 16 != 0 || N > 65536 || M >= kI31)
    return fail(MSDA_ERR_UNSUPPORTED, "needs K %% 32 == 0, K <= 256, N %% 16 == 0, N <= 65536, M < 2^31 "
                "(got M=%lld N=%lld K=%lld)", (long long)M, (long long)N, (long long)K);
  return MSDA_OK;
}

// one output of N columns; callers fill in W, bias, Y and the epilogue
msda::GemmArgs gemm_args(const void* X, bool x_f32, int64_t M, int64_t N, int64_t K) {
  msda::GemmArgs g = {};
  g.X = X;
  g.x_f32 = x_f32;
  g.M = M;
  g.N = (int)N;
  g.K = (int)K;
  g.N1 = (int)N;
  return g;
}

}  // namespace

extern "C" {

const char* msda_status_string(int status) {
  switch (status) {
    case MSDA_OK: return "MSDA_OK";
    case MSDA_ERR_INVALID_ARG: return "MSDA_ERR_INVALID_ARG";
    case MSDA_ERR_UNSUPPORTED: return "MSDA_ERR_UNSUPPORTED";
    case MSDA_ERR_SHAPE: return "MSDA_ERR_SHAPE";
    case MSDA_ERR_WORKSPACE: return "MSDA_ERR_WORKSPACE";
    case MSDA_ERR_HIP: return "MSDA_ERR_HIP";
    default: return "MSDA_ERR_UNKNOWN";
  }
}

const char* msda_last_error(void) { return g_last_error; }

int msda_check_counts(unsigned long long* counts, int n, int reset) {
#ifndef MSDA_CHECKED
  (void)counts;
  (void)n;
  (void)reset;
  return fail(MSDA_ERR_UNSUPPORTED, "msda_check_counts: this library is built without device-side checks "
              "(libmsda_checked.so has them)");
#else
  if (!counts || n < msda::kCheckKinds)
    return fail(MSDA_ERR_INVALID_ARG, "counts must hold MSDA_CHECK_KINDS (%d) entries", msda::kCheckKinds);
  for (int k = 0; k < n; ++k) counts[k] = 0;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_status(e, "hipDeviceSynchronize");
  std::lock_guard<std::mutex> lock(check_mutex());
  for (msda::CheckReader r : check_readers()) {
    e = r(counts, reset != 0);
    if (e != hipSuccess) return hip_status(e, "reading the check counters");
  }
  return MSDA_OK;
#endif
}

static int msda_frames_impl(const void* value, int value_dtype, const int64_t* spatial_shapes,
                            const int64_t* level_start_index, const float* sampling_locations,
                            const float* attention_weights, int weight_mode, int64_t B, int64_t F, int64_t Nv,
                            int64_t Nq, int nH, int Dh, int L, int P, float* out, const int32_t* plan,
                            void* stream) {
  uint32_t image_bytes = 0;
  int rc = check_common(value, value_dtype, spatial_shapes, level_start_index, Nv, Nq, nH, Dh, L, P, out,
                        &image_bytes, true);
  if (rc != MSDA_OK) return rc;
  if ((!sampling_locations || !attention_weights) && Nq != 0)
    return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (B < 1 || F < 1) return fail(MSDA_ERR_INVALID_ARG, "B and F must be positive");
  if (weight_mode != MSDA_WEIGHTS_PROB && weight_mode != MSDA_WEIGHTS_LOGITS)
    return fail(MSDA_ERR_INVALID_ARG, "weight_mode %d is neither PROB nor LOGITS", weight_mode);
  if (Nq != 0 && (!aligned(sampling_locations, 8) || !aligned(attention_weights, 4)))
    return fail(MSDA_ERR_INVALID_ARG, "sampling_locations must be 8-byte aligned");
  if (B * F >= kI31 || B * Nq >= kI31 || B * F * Nq * nH >= kI31 / 64)
    return fail(MSDA_ERR_UNSUPPORTED, "B*F*Nq*nH too large");
  g_last_error[0] = '\0';
  if (Nq == 0) return MSDA_OK;
  msda::GatherArgs a = {};
  a.value = value;
  a.image_bytes = image_bytes;
  a.bf16 = value_dtype != MSDA_F32;
  a.pairs = value_dtype == MSDA_BF16_PAIRS;
  a.shapes = spatial_shapes;
  a.starts = level_start_index;
  a.L = L;
  a.P = P;
  a.LP = L * P;
  a.nH = nH;
  a.Nv = (int)Nv;
  a.inv_P = 1.0f / (float)P;
  a.inv_D = 1.0f;
  a.loc = sampling_locations;
  a.weights = attention_weights;
  a.weight_logits = weight_mode == MSDA_WEIGHTS_LOGITS;
  a.F = (int)F;
  a.inv_LP = 1.0f / (float)(L * P);
  a.plan = plan;
  a.B = B;
  a.Nq = Nq;
  a.out = out;
  return hip_status(msda::launch_msda_gather(a, static_cast<hipStream_t>(stream)), "msda gather launch");
}

int msda_forward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                 const int64_t* level_start_index, const float* sampling_locations,
                 const float* attention_weights, int weight_mode, int64_t B, int64_t Nv, int64_t Nq, int nH,
                 int Dh, int L, int P, float* out, void* stream) {
  return msda_frames_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_locations,
                          attention_weights, weight_mode, B, 1, Nv, Nq, nH, Dh, L, P, out, nullptr, stream);
}

int msda_forward_frames(const void* value, int value_dtype, const int64_t* spatial_shapes,
                        const int64_t* level_start_index, const float* sampling_locations,
                        const float* attention_weights, int weight_mode, int64_t B, int64_t F, int64_t Nv,
                        int64_t Nq, int nH, int Dh, int L, int P, float* out, void* stream) {
  return msda_frames_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_locations,
                          attention_weights, weight_mode, B, F, Nv, Nq, nH, Dh, L, P, out, nullptr, stream);
}

int msda_plan_size(int64_t B, int64_t Nq, size_t* bytes) {
  if (!bytes) return fail(MSDA_ERR_INVALID_ARG, "bytes is null");
  if (B < 1 || Nq < 0) return fail(MSDA_ERR_INVALID_ARG, "B >= 1 and Nq >= 0 required");
  if (B * Nq >= kI31 || B >= 65536) return fail(MSDA_ERR_UNSUPPORTED, "B*Nq must be below 2^31 and B below 65536");
  *bytes = msda::plan_bytes(B, Nq);
  return MSDA_OK;
}

int msda_plan(const float* points, int64_t batch_stride, int64_t point_stride, int64_t B, int64_t Nq, void* plan,
              size_t plan_bytes, void* stream) {
  size_t need = 0;
  int rc = msda_plan_size(B, Nq, &need);
  if (rc != MSDA_OK) return rc;
  if (Nq != 0 && !points) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (batch_stride < 0 || point_stride < 0 || ((batch_stride | point_stride) & 1))
    return fail(MSDA_ERR_INVALID_ARG, "strides must be even and >= 0 (float elements; points are float pairs)");
  if (Nq != 0 && !aligned(points, 8)) return fail(MSDA_ERR_INVALID_ARG, "points must be 8-byte aligned");
  if (!plan || plan_bytes < need || !aligned(plan, 256))
    return fail(MSDA_ERR_WORKSPACE, "plan must be >= %zu bytes and 256-byte aligned (got %zu)", need, plan_bytes);
  g_last_error[0] = '\0';
  if (Nq == 0) return MSDA_OK;
  msda::PlanArgs a = {points, batch_stride, point_stride, (int)B, (int)Nq, static_cast<int32_t*>(plan),
                      reinterpret_cast<int32_t*>(static_cast<char*>(plan) + msda::plan_bins_offset(B, Nq))};
  return hip_status(msda::launch_msda_plan(a, static_cast<hipStream_t>(stream)), "msda plan launch");
}

int msda_gather(const void* value, int value_dtype, const int64_t* spatial_shapes, const int64_t* level_start_index,
                const float* sampling_locations, const float* attention_weights, int weight_mode, int64_t B,
                int64_t F, int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, float* out, const void* plan,
                size_t plan_bytes, void* stream) {
  size_t need = 0;
  if (Nq != 0 && B >= 1 && Nq > 0 && msda_plan_size(B, Nq, &need) == MSDA_OK &&
      (!plan || plan_bytes < need || !aligned(plan, 256)))
    return fail(MSDA_ERR_WORKSPACE, "plan must be >= %zu bytes and 256-byte aligned (got %zu)", need, plan_bytes);
  return msda_frames_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_locations,
                          attention_weights, weight_mode, B, F, Nv, Nq, nH, Dh, L, P, out,
                          static_cast<const int32_t*>(plan), stream);
}

int sca_workspace_size(int64_t B, int64_t Ncam, int64_t Nq, size_t* bytes) {
  if (!bytes) return fail(MSDA_ERR_INVALID_ARG, "bytes is null");
  if (B < 1 || Ncam < 1 || Nq < 0) return fail(MSDA_ERR_INVALID_ARG, "B and Ncam must be positive, Nq >= 0");
  if (B * Ncam * Nq >= kI31 || B * Ncam >= (1 << 20))
    return fail(MSDA_ERR_UNSUPPORTED, "B*Ncam*Nq must be below 2^31");
  *bytes = msda::compact_layout(B, Ncam, Nq).total;
  return MSDA_OK;
}

int sca_plan_workspace(int64_t B, int64_t Ncam, int64_t Nq, size_t* bytes) {
  return sca_workspace_size(B, Ncam, Nq, bytes);
}

static int check_workspace(int64_t B, int64_t Ncam, int64_t Nq, const void* workspace, size_t workspace_bytes) {
  size_t need = 0;
  const int rc = sca_workspace_size(B, Ncam, Nq, &need);
  if (rc != MSDA_OK) return rc;
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(MSDA_ERR_WORKSPACE, "workspace must be >= %zu bytes and 256-byte aligned (got %zu)", need,
                workspace_bytes);
  return MSDA_OK;
}

static msda::CompactArgs compact_args(const uint8_t* bev_mask, const float* reference_points_cam, int64_t B,
                                      int64_t Ncam, int64_t Nq, int D, int32_t* hit_count, int32_t* pair_offsets,
                                      int32_t* pair_q, void* workspace) {
  const msda::CompactLayout lay = msda::compact_layout(B, Ncam, Nq);
  char* ws = static_cast<char*>(workspace);
  msda::CompactArgs c = {};
  c.bev_mask = bev_mask;
  c.rp = reference_points_cam;
  c.B = (int)B;
  c.Ncam = (int)Ncam;
  c.Nq = (int)Nq;
  c.D = D;
  c.cammask = reinterpret_cast<uint32_t*>(ws + lay.cammask);
  c.qkey = reinterpret_cast<int32_t*>(ws + lay.qkey);
  c.qrank = reinterpret_cast<int32_t*>(ws + lay.qrank);
  c.hit_count = hit_count;
  c.tile_counts = reinterpret_cast<int32_t*>(ws + lay.tile_counts);
  c.tile_offsets = reinterpret_cast<int32_t*>(ws + lay.tile_offsets);
  c.pair_offsets = pair_offsets ? pair_offsets : reinterpret_cast<int32_t*>(ws + lay.pair_offsets);
  c.pair_q = pair_q ? pair_q : reinterpret_cast<int32_t*>(ws + lay.pair_q);
  c.bin_hist = reinterpret_cast<int32_t*>(ws + lay.bin_hist);
  c.seg_seen = reinterpret_cast<int32_t*>(ws + lay.seg_seen);
  c.seg_pairs = reinterpret_cast<int32_t*>(ws + lay.seg_pairs);
  c.order = reinterpret_cast<int32_t*>(ws + lay.order);
  c.bin_cost = reinterpret_cast<uint64_t*>(ws + lay.bin_cost);
  c.seg_cost = reinterpret_cast<uint64_t*>(ws + lay.seg_cost);
  c.die_bounds = reinterpret_cast<int32_t*>(ws + lay.die_bounds);
  c.clear_ints = lay.clear_ints;
  return c;
}

int sca_compact(const uint8_t* bev_mask, const float* reference_points_cam, int64_t B, int64_t Ncam, int64_t Nq,
                int D, int32_t* hit_count, int32_t* pair_offsets, int32_t* pair_q, void* workspace,
                size_t workspace_bytes, void* stream) {
  if ((!bev_mask || !reference_points_cam) && Nq != 0) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (Nq != 0 && !aligned(reference_points_cam, 8))
    return fail(MSDA_ERR_INVALID_ARG, "reference_points_cam must be 8-byte aligned");
  if (B < 1 || Ncam < 1 || D < 1 || Nq < 0) return fail(MSDA_ERR_INVALID_ARG, "B, Ncam and D must be positive");
  if (Ncam > 32) return fail(MSDA_ERR_UNSUPPORTED, "Ncam=%lld: at most 32 cameras", (long long)Ncam);
  if ((int64_t)D * Nq * Ncam * B >= ((int64_t)1 << 40)) return fail(MSDA_ERR_UNSUPPORTED, "bev_mask too large");
  int rc = check_workspace(B, Ncam, Nq, workspace, workspace_bytes);
  if (rc != MSDA_OK) return rc;
  g_last_error[0] = '\0';
  if (Nq == 0) return MSDA_OK;
  const msda::CompactArgs c =
      compact_args(bev_mask, reference_points_cam, B, Ncam, Nq, D, hit_count, pair_offsets, pair_q, workspace);
  return hip_status(msda::launch_sca_compact(c, msda::compact_layout(B, Ncam, Nq).tiles,
                                             static_cast<hipStream_t>(stream)),
                    "sca compaction launch");
}

int sca_gather(const void* value, int value_dtype, const int64_t* spatial_shapes, const int64_t* level_start_index,
               const float* reference_points_cam, const float* sampling_offsets, const float* attention_logits,
               int64_t B, int64_t Ncam, int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, int D, float* slots,
               void* workspace, size_t workspace_bytes, void* stream) {
  uint32_t image_bytes = 0;
  int rc = check_common(value, value_dtype, spatial_shapes, level_start_index, Nv, Nq, nH, Dh, L, P, slots,
                        &image_bytes, true);
  if (rc != MSDA_OK) return rc;
  if ((!reference_points_cam || !sampling_offsets || !attention_logits) && Nq != 0)
    return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (B < 1 || Ncam < 1 || D < 1) return fail(MSDA_ERR_INVALID_ARG, "B, Ncam and D must be positive");
  if (Ncam > 32) return fail(MSDA_ERR_UNSUPPORTED, "Ncam=%lld: at most 32 cameras", (long long)Ncam);
  if (P % D != 0) return fail(MSDA_ERR_SHAPE, "P=%d is not a multiple of D=%d", P, D);
  if (Nq != 0 && (!aligned(reference_points_cam, 8) || !aligned(sampling_offsets, 8)))
    return fail(MSDA_ERR_INVALID_ARG, "reference_points_cam and sampling_offsets must be 8-byte aligned");
  if (B * Nq * nH >= kI31 / 64) return fail(MSDA_ERR_UNSUPPORTED, "B*Nq*nH too large");
  rc = check_workspace(B, Ncam, Nq, workspace, workspace_bytes);
  if (rc != MSDA_OK) return rc;
  g_last_error[0] = '\0';
  if (Nq == 0) return MSDA_OK;
  const msda::CompactArgs c = compact_args(nullptr, nullptr, B, Ncam, Nq, D, nullptr, nullptr, nullptr, workspace);
  msda::GatherArgs a = {};
  a.value = value;
  a.image_bytes = image_bytes;
  a.bf16 = value_dtype != MSDA_F32;
  a.pairs = value_dtype == MSDA_BF16_PAIRS;
  a.shapes = spatial_shapes;
  a.starts = level_start_index;
  a.L = L;
  a.P = P;
  a.LP = L * P;
  a.nH = nH;
  a.Nv = (int)Nv;
  a.inv_P = 1.0f / (float)P;
  a.inv_D = 1.0f / (float)D;
  a.rp = reference_points_cam;
  a.offsets = sampling_offsets;
  a.logits = attention_logits;
  a.cammask = c.cammask;
  a.order = c.order;
  a.die_bounds = c.die_bounds;
  a.Ncam = (int)Ncam;
  a.D = D;
  a.B = B;
  a.Nq = Nq;
  a.out = slots;
  return hip_status(msda::launch_sca_gather(a, static_cast<hipStream_t>(stream)), "sca gather launch");
}

int sca_forward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                const int64_t* level_start_index, const float* reference_points_cam, const uint8_t* bev_mask,
                const float* sampling_offsets, const float* attention_logits, int64_t B, int64_t Ncam, int64_t Nv,
                int64_t Nq, int nH, int Dh, int L, int P, int D, float* slots, int32_t* hit_count,
                int32_t* pair_offsets, int32_t* pair_q, void* workspace, size_t workspace_bytes, void* stream) {
  // check everything both stages check before enqueuing either
  uint32_t image_bytes = 0;
  int rc = check_common(value, value_dtype, spatial_shapes, level_start_index, Nv, Nq, nH, Dh, L, P, slots,
                        &image_bytes, true);
  if (rc != MSDA_OK) return rc;
  if ((!reference_points_cam || !bev_mask || !sampling_offsets || !attention_logits) && Nq != 0)
    return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (B < 1 || Ncam < 1 || D < 1) return fail(MSDA_ERR_INVALID_ARG, "B, Ncam and D must be positive");
  if (Ncam > 32) return fail(MSDA_ERR_UNSUPPORTED, "Ncam=%lld: at most 32 cameras", (long long)Ncam);
  if (P % D != 0) return fail(MSDA_ERR_SHAPE, "P=%d is not a multiple of D=%d", P, D);
  if (Nq != 0 && (!aligned(reference_points_cam, 8) || !aligned(sampling_offsets, 8)))
    return fail(MSDA_ERR_INVALID_ARG, "reference_points_cam and sampling_offsets must be 8-byte aligned");
  rc = check_workspace(B, Ncam, Nq, workspace, workspace_bytes);
  if (rc != MSDA_OK) return rc;
  if (B * Nq * nH >= kI31 / 64) return fail(MSDA_ERR_UNSUPPORTED, "B*Nq*nH too large");
  rc = sca_compact(bev_mask, reference_points_cam, B, Ncam, Nq, D, hit_count, pair_offsets, pair_q, workspace,
                   workspace_bytes, stream);
  if (rc != MSDA_OK) return rc;
  return sca_gather(value, value_dtype, spatial_shapes, level_start_index, reference_points_cam, sampling_offsets,
                    attention_logits, B, Ncam, Nv, Nq, nH, Dh, L, P, D, slots, workspace, workspace_bytes, stream);
}

int msda_gemm_bf16(const void* X, int x_dtype, const uint16_t* W, const float* bias, void* Y, int y_dtype,
                   int64_t M, int64_t N, int64_t K, void* stream) {
  if (!X || !W || !Y) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if ((x_dtype != MSDA_F32 && x_dtype != MSDA_BF16) || (y_dtype != MSDA_F32 && y_dtype != MSDA_BF16))
    return fail(MSDA_ERR_INVALID_ARG, "x_dtype and y_dtype must be MSDA_F32 or MSDA_BF16");
  int rc = check_gemm_sizes(M, N, K);
  if (rc != MSDA_OK) return rc;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(Y, 16) || (bias && !aligned(bias, 4)))
    return fail(MSDA_ERR_INVALID_ARG, "X, W and Y must be 16-byte aligned");
  g_last_error[0] = '\0';
  if (M == 0) return MSDA_OK;
  msda::GemmArgs g = gemm_args(X, x_dtype == MSDA_F32, M, N, K);
  g.W1 = W;
  g.bias1 = bias;
  g.Y1 = Y;
  g.y_f32 = y_dtype == MSDA_F32;
  return hip_status(msda::launch_gemm_bf16(g, static_cast<hipStream_t>(stream)), "gemm launch");
}

int msda_value_proj_pairs_bf16(const void* X, int x_dtype, const uint16_t* W, const float* bias, uint16_t* pairs,
                               int64_t M, int64_t N, int64_t K, int64_t Nv, void* stream) {
  if (!X || !W || !pairs) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (x_dtype != MSDA_F32 && x_dtype != MSDA_BF16)
    return fail(MSDA_ERR_INVALID_ARG, "x_dtype must be MSDA_F32 or MSDA_BF16");
  int rc = check_gemm_sizes(M, N, K);
  if (rc != MSDA_OK) return rc;
  if (Nv < 1) return fail(MSDA_ERR_INVALID_ARG, "Nv >= 1 required");
  if (N % 32 != 0) return fail(MSDA_ERR_UNSUPPORTED, "N %% 32 == 0 required (heads of 32 channels), got %lld",
                               (long long)N);
  if (M % Nv != 0) return fail(MSDA_ERR_SHAPE, "M=%lld is not a whole number of images of Nv=%lld rows",
                               (long long)M, (long long)Nv);
  if (Nv * (N / 32) * 128 >= kI31)
    return fail(MSDA_ERR_UNSUPPORTED, "one image in the head-pair layout is %lld bytes; the limit is 2^31",
                (long long)(Nv * (N / 32) * 128));
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(pairs, 16) || (bias && !aligned(bias, 4)))
    return fail(MSDA_ERR_INVALID_ARG, "X, W and pairs must be 16-byte aligned");
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(X), p0 = reinterpret_cast<uintptr_t>(pairs);
  const uintptr_t xb = (uintptr_t)(M * K * (x_dtype == MSDA_F32 ? 4 : 2)), pb = (uintptr_t)(M * N * 4);
  if (M != 0 && x0 < p0 + pb && p0 < x0 + xb) return fail(MSDA_ERR_INVALID_ARG, "pairs must not overlap X");
  g_last_error[0] = '\0';
  if (M == 0) return MSDA_OK;
  msda::GemmArgs g = gemm_args(X, x_dtype == MSDA_F32, M, N, K);
  g.W1 = W;
  g.bias1 = bias;
  g.Y1 = pairs;
  g.y_f32 = 0;
  g.pairs_Nv = Nv;
  return hip_status(msda::launch_gemm_bf16(g, static_cast<hipStream_t>(stream)), "value projection launch");
}

int msda_pack_pairs_bf16(const uint16_t* value, uint16_t* pairs, int64_t n_images, int64_t Nv, int nH,
                         void* stream) {
  // with no images nothing is read or written: the buffers may be null
  if ((!value || !pairs) && n_images != 0) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (n_images < 0 || Nv < 1 || nH < 1)
    return fail(MSDA_ERR_INVALID_ARG, "n_images >= 0, Nv >= 1 and nH >= 1 required");
  if (nH > 64) return fail(MSDA_ERR_UNSUPPORTED, "nH=%d: at most 64 heads", nH);
  if (Nv >= kI31 || Nv * nH * 128 >= kI31)
    return fail(MSDA_ERR_UNSUPPORTED, "one image in the head-pair layout is %lld bytes; the limit is 2^31",
                (long long)(Nv * nH * 128));
  if (n_images > ((int64_t)1 << 40) / (Nv * nH * 128))
    return fail(MSDA_ERR_UNSUPPORTED, "n_images=%lld too large", (long long)n_images);
  if (!aligned(value, 16) || !aligned(pairs, 16)) return fail(MSDA_ERR_INVALID_ARG, "value and pairs must be 16-byte aligned");
  const uintptr_t v0 = reinterpret_cast<uintptr_t>(value), p0 = reinterpret_cast<uintptr_t>(pairs);
  const uintptr_t vb = (uintptr_t)(n_images * Nv * nH * 64), pb = 2 * vb;
  if (vb != 0 && v0 < p0 + pb && p0 < v0 + vb) return fail(MSDA_ERR_INVALID_ARG, "pairs must not overlap value");
  g_last_error[0] = '\0';
  if (n_images == 0) return MSDA_OK;
  return hip_status(msda::launch_pack_pairs(value, pairs, n_images, Nv, nH, static_cast<hipStream_t>(stream)),
                    "pair packing launch");
}

int msda_query_proj_bf16(const float* query, const float* query_pos, const uint16_t* W_off, const float* b_off,
                         const uint16_t* W_att, const float* b_att, float* offsets, float* logits, int64_t M,
                         int64_t K, int64_t N_off, int64_t N_att, void* stream) {
  if (!query || !W_off || !W_att || !offsets || !logits) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (N_off < 1 || N_att < 1) return fail(MSDA_ERR_INVALID_ARG, "N_off >= 1 and N_att >= 1 required");
  if (N_off % 32 != 0)
    return fail(MSDA_ERR_UNSUPPORTED, "N_off %% 32 == 0 required (got %lld)", (long long)N_off);
  int rc = check_gemm_sizes(M, N_off + N_att, K);
  if (rc != MSDA_OK) return rc;
  if (!aligned(query, 16) || (query_pos && !aligned(query_pos, 16)) || !aligned(W_off, 16) ||
      !aligned(W_att, 16) || !aligned(offsets, 16) || !aligned(logits, 16) || (b_off && !aligned(b_off, 4)) ||
      (b_att && !aligned(b_att, 4)))
    return fail(MSDA_ERR_INVALID_ARG, "query, query_pos, weights and outputs must be 16-byte aligned");
  g_last_error[0] = '\0';
  if (M == 0) return MSDA_OK;
  msda::GemmArgs g = gemm_args(query, true, M, N_off + N_att, K);
  g.X_add = query_pos;
  g.N1 = (int)N_off;
  g.W1 = W_off;
  g.bias1 = b_off;
  g.Y1 = offsets;
  g.W2 = W_att;
  g.bias2 = b_att;
  g.Y2 = logits;
  g.y_f32 = 1;
  return hip_status(msda::launch_gemm_bf16(g, static_cast<hipStream_t>(stream)), "query projection launch");
}

int msda_output_proj_bf16(const void* X, int x_dtype, const uint16_t* W, const float* bias, const float* residual,
                          const float* gamma, const float* beta, float eps, float* Y, int64_t M, int64_t N,
                          int64_t K, void* stream) {
  if (!X || !W || !Y) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (x_dtype != MSDA_F32 && x_dtype != MSDA_BF16)
    return fail(MSDA_ERR_INVALID_ARG, "x_dtype must be MSDA_F32 or MSDA_BF16");
  if (beta && !gamma) return fail(MSDA_ERR_INVALID_ARG, "beta given without gamma");
  int rc = check_gemm_sizes(M, N, K);
  if (rc != MSDA_OK) return rc;
  if (gamma && N != msda::kGemmNormCols)
    return fail(MSDA_ERR_UNSUPPORTED, "the layer norm needs N == %d (got %lld)", msda::kGemmNormCols, (long long)N);
  if (gamma && !(eps >= 0.0f && eps < INFINITY)) return fail(MSDA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(Y, 16) || (residual && !aligned(residual, 16)) ||
      (bias && !aligned(bias, 4)) || (gamma && !aligned(gamma, 4)) || (beta && !aligned(beta, 4)))
    return fail(MSDA_ERR_INVALID_ARG, "X, W, Y and residual must be 16-byte aligned");
  g_last_error[0] = '\0';
  if (M == 0) return MSDA_OK;
  msda::GemmArgs g = gemm_args(X, x_dtype == MSDA_F32, M, N, K);
  g.W1 = W;
  g.bias1 = bias;
  g.Y1 = Y;
  g.y_f32 = 1;
  g.residual = residual;
  g.gamma = gamma;
  g.beta = beta;
  g.eps = eps;
  return hip_status(msda::launch_gemm_bf16(g, static_cast<hipStream_t>(stream)), "output projection launch");
}

int sca_rebatch(const int32_t* pair_offsets, const int32_t* pair_q, const float* reference_points_cam,
                const float* sampling_offsets, const float* attention_logits, const int64_t* spatial_shapes,
                int64_t B, int64_t Ncam, int64_t Nq, int nH, int L, int P, int D, int64_t max_len,
                float* sampling_locations, float* logits_out, void* stream) {
  if (B < 0 || Ncam < 1 || Nq < 0 || nH < 1 || L < 1 || P < 1 || D < 1 || max_len < 0)
    return fail(MSDA_ERR_INVALID_ARG, "B, Nq, max_len >= 0 and Ncam, nH, L, P, D >= 1 required");
  if (P % D != 0) return fail(MSDA_ERR_SHAPE, "P=%d is not a multiple of D=%d", P, D);
  if (Ncam > 32 || B * Ncam >= kI31 || Nq >= kI31 || B * Ncam * max_len >= kI31)
    return fail(MSDA_ERR_UNSUPPORTED, "sizes beyond the supported range");
  const bool rows = B * Ncam * max_len > 0;
  if (!pair_offsets || !spatial_shapes || (rows && (!pair_q || !reference_points_cam || !sampling_offsets ||
                                                    !attention_logits || !sampling_locations || !logits_out)))
    return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(reference_points_cam, 8) || !aligned(sampling_offsets, 8) || !aligned(sampling_locations, 8))
    return fail(MSDA_ERR_INVALID_ARG, "(x, y) arrays must be 8-byte aligned");
  g_last_error[0] = '\0';
  msda::RebatchArgs r = {pair_offsets, pair_q, reference_points_cam, sampling_offsets, attention_logits,
                         spatial_shapes, B, Ncam, Nq, nH, L, P, D, max_len, sampling_locations, logits_out};
  return hip_status(msda::launch_sca_rebatch(r, static_cast<hipStream_t>(stream)), "rebatch launch");
}

int sca_scatter_mean(const float* rows, const int32_t* pair_offsets, const int32_t* pair_q,
                     const int32_t* hit_count, int64_t B, int64_t Ncam, int64_t Nq, int64_t C, int64_t max_len,
                     float* slots, void* stream) {
  if (B < 0 || Ncam < 1 || Nq < 0 || C < 4 || max_len < 0)
    return fail(MSDA_ERR_INVALID_ARG, "B, Nq, max_len >= 0, Ncam >= 1 and C >= 4 required");
  if (C % 4 != 0) return fail(MSDA_ERR_UNSUPPORTED, "C %% 4 == 0 required (got %lld)", (long long)C);
  if (B * Ncam >= kI31 || B * Nq >= kI31 || B * Ncam * max_len >= kI31)
    return fail(MSDA_ERR_UNSUPPORTED, "sizes beyond the supported range");
  const bool any = B * Nq > 0;
  if (any && (!slots || !hit_count || !pair_offsets || (max_len > 0 && (!rows || !pair_q))))
    return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if ((rows && !aligned(rows, 16)) || (slots && !aligned(slots, 16)))
    return fail(MSDA_ERR_INVALID_ARG, "rows and slots must be 16-byte aligned");
  g_last_error[0] = '\0';
  msda::ScatterArgs a = {rows, pair_offsets, pair_q, hit_count, B, Ncam, Nq, C, max_len, slots};
  return hip_status(msda::launch_sca_scatter_mean(a, static_cast<hipStream_t>(stream)), "scatter launch");
}

// Checks of the gradient image shared by the backward entry points: float32
// [images][Nv][nH][Dh], each image addressed through one descriptor.
static int check_grad_value(const float* grad_value, int64_t Nv, int nH, int Dh, uint32_t* grad_image_bytes) {
  if (!grad_value) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  const int64_t bytes = Nv * nH * Dh * 4;
  if (bytes >= kI31) return fail(MSDA_ERR_UNSUPPORTED, "one gradient image is %lld bytes; the limit is 2^31",
                                 (long long)bytes);
  if (!aligned(grad_value, 16)) return fail(MSDA_ERR_INVALID_ARG, "grad_value must be 16-byte aligned");
  *grad_image_bytes = (uint32_t)bytes;
  return MSDA_OK;
}

// Layout of the workspace of the deterministic value gradient, after the
// size checks shared by the size queries and the entry points.
static int vgrad_plan(int64_t images, int64_t Nv, int64_t L, int64_t nH, int64_t records, int64_t pair_of_entries,
                      int64_t per_segment, msda::VgradLayout* lay) {
  constexpr int64_t kMaxSlots = (int64_t)1 << 28;
  if (records < 0 || records >= kMaxSlots)
    return fail(MSDA_ERR_UNSUPPORTED, "%lld sample records: at most 2^28 fit one workspace", (long long)records);
  const int64_t per_image = (2 * Nv + 2 * L) * nH;  // corner keys per image, bounded
  if (per_image >= kI31 || images > (kI31 - 1) / per_image)
    return fail(MSDA_ERR_UNSUPPORTED, "corner keys of the value gradient exceed 2^31");
  *lay = msda::vgrad_layout(images, Nv, (int)L, (int)nH, records, pair_of_entries, per_segment);
  if (lay->slots >= kMaxSlots)
    return fail(MSDA_ERR_UNSUPPORTED, "%lld record slots (each image and head starts a tile of %d): at most 2^28",
                (long long)lay->slots, msda::kSortTile);
  return MSDA_OK;
}

static int vgrad_sizes_ok(int64_t B, int64_t Nv, int64_t Nq, int nH, int L, int P) {
  if (B < 1 || Nv < 1 || Nq < 0 || nH < 1 || L < 1 || P < 1)
    return fail(MSDA_ERR_INVALID_ARG, "sizes must be positive");
  if (nH > 64 || (int64_t)L * P > 64 || Nv >= kI31 || Nq >= kI31 || B >= kI31)
    return fail(MSDA_ERR_UNSUPPORTED, "sizes beyond the supported range");
  return MSDA_OK;
}

int msda_backward_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int nH, int L, int P, size_t* bytes) {
  if (!bytes) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  int rc = vgrad_sizes_ok(B, Nv, Nq, nH, L, P);
  if (rc != MSDA_OK) return rc;
  msda::VgradLayout lay;
  rc = vgrad_plan(B, Nv, L, nH, B * Nq * nH * L * P, 0, Nq * L * P, &lay);
  if (rc != MSDA_OK) return rc;
  *bytes = lay.total;
  return MSDA_OK;
}

static int64_t sca_pair_capacity(int64_t B, int64_t Ncam, int64_t Nq, int64_t max_pairs) {
  const int64_t all = B * Nq * Ncam;
  return max_pairs > 0 && max_pairs < all ? max_pairs : all;
}

int sca_backward_workspace_size(int64_t B, int64_t Ncam, int64_t Nv, int64_t Nq, int nH, int L, int P,
                                int64_t max_pairs, size_t* bytes) {
  if (!bytes) return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  int rc = vgrad_sizes_ok(B, Nv, Nq, nH, L, P);
  if (rc != MSDA_OK) return rc;
  if (Ncam < 1 || Ncam > 32) return fail(MSDA_ERR_UNSUPPORTED, "Ncam=%lld: 1 to 32 cameras", (long long)Ncam);
  msda::VgradLayout lay;
  rc = vgrad_plan(B * Ncam, Nv, L, nH, sca_pair_capacity(B, Ncam, Nq, max_pairs) * nH * L * P, Ncam * B * Nq, 0, &lay);
  if (rc != MSDA_OK) return rc;
  *bytes = lay.total;
  return MSDA_OK;
}

// The state, sort buffers and geometry of the transpose gather.
static msda::VgradArgs vgrad_args(const msda::VgradLayout& lay, void* workspace, const int64_t* shapes,
                                  const int64_t* starts, int L, int nH, int64_t Nv, int64_t images,
                                  const float* grad_out, int64_t grad_rows, float* grad_value) {
  char* ws = static_cast<char*>(workspace);
  msda::VgradArgs v = {};
  for (int i = 0; i < 2; ++i) {
    v.keys[i] = reinterpret_cast<uint32_t*>(ws + lay.keys[i]);
    v.vals[i] = reinterpret_cast<msda::VgradRec*>(ws + lay.vals[i]);
  }
  v.counts = reinterpret_cast<uint32_t*>(ws + lay.counts);
  v.tile_seg = reinterpret_cast<int32_t*>(ws + lay.tile_seg);
  v.digit_totals = reinterpret_cast<uint32_t*>(ws + lay.digit_totals);
  v.seg_tile = reinterpret_cast<int32_t*>(ws + lay.seg_tile);
  v.seg_items = reinterpret_cast<int32_t*>(ws + lay.seg_items);
  v.seg_live = reinterpret_cast<int32_t*>(ws + lay.seg_live);
  v.pair_start = reinterpret_cast<int32_t*>(ws + lay.pair_start);
  v.ranges = reinterpret_cast<int2*>(ws + lay.ranges);
  v.long_row = reinterpret_cast<uint8_t*>(ws + lay.long_row);
  v.state = reinterpret_cast<msda::VgradState*>(ws + lay.state);
  v.pair_of = reinterpret_cast<int32_t*>(ws + lay.pair_of);
  v.segments = lay.segments;
  v.sort_tiles = lay.sort_tiles;
  v.key_bound = lay.key_bound;
  v.passes = lay.passes;
  v.shapes = shapes;
  v.starts = starts;
  v.L = L;
  v.nH = nH;
  v.Nv = (int)Nv;
  v.images = images;
  v.grad_out = grad_out;
  v.grad_out_bytes = (uint32_t)(grad_rows * 128);
  v.grad_value = grad_value;
  return v;
}

static int check_grad_workspace(const msda::VgradLayout& lay, const void* ws, size_t bytes) {
  if (bytes < lay.total || !aligned(ws, 256))
    return fail(MSDA_ERR_WORKSPACE, "gradient workspace must be >= %zu bytes and 256-byte aligned (got %zu)",
                lay.total, bytes);
  return MSDA_OK;
}

static void set_records(msda::BackwardArgs& a, const msda::VgradArgs& v, int64_t max_pairs) {
  a.rec_keys = v.keys[0];
  a.rec_vals = v.vals[0];
  a.rec_slots = (uint32_t)(v.sort_tiles * msda::kSortTile);
  a.seg_tile = v.seg_tile;
  a.pair_start = v.pair_start;
  a.pair_of = v.pair_of;
  a.max_pairs = max_pairs;
}

// The operator's backward over B batch items of F frames each (images
// b * F + f; F = 1 is the plain operator): frame f's gradients are the
// operator's for the upstream gradient grad_out[b] / F.
static int msda_backward_impl(const void* value, int value_dtype, const int64_t* spatial_shapes,
                              const int64_t* level_start_index, const float* sampling_locations,
                              const float* attention_weights, int weight_mode, const float* grad_out, int64_t B,
                              int64_t F, int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, float* grad_value,
                              float* grad_sampling_locations, float* grad_attention_weights, void* grad_workspace,
                              size_t grad_workspace_bytes, void* stream) {
  uint32_t image_bytes = 0, grad_bytes = 0;
  int rc = check_common(value, value_dtype, spatial_shapes, level_start_index, Nv, Nq, nH, Dh, L, P, grad_out,
                        &image_bytes);
  if (rc != MSDA_OK) return rc;
  if (B < 1 || F < 1) return fail(MSDA_ERR_INVALID_ARG, "B and F must be positive");
  rc = check_grad_value(grad_value, Nv, nH, Dh, &grad_bytes);
  if (rc != MSDA_OK) return rc;
  if (Nq != 0 && (!sampling_locations || !attention_weights || !grad_sampling_locations || !grad_attention_weights))
    return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (weight_mode != MSDA_WEIGHTS_PROB && weight_mode != MSDA_WEIGHTS_LOGITS)
    return fail(MSDA_ERR_INVALID_ARG, "weight_mode %d is neither PROB nor LOGITS", weight_mode);
  if (Nq != 0 && (!aligned(sampling_locations, 8) || !aligned(grad_sampling_locations, 8) ||
                  !aligned(attention_weights, 4) || !aligned(grad_attention_weights, 4)))
    return fail(MSDA_ERR_INVALID_ARG, "(x, y) arrays must be 8-byte aligned");
  if (B >= kI31 || F >= kI31 || B * F >= kI31 || B * F * Nq * nH >= kI31 / 64)
    return fail(MSDA_ERR_UNSUPPORTED, "B*F*Nq*nH too large");
  const int64_t I = B * F;  // images
  msda::VgradLayout lay = {};
  if (grad_workspace) {
    rc = vgrad_plan(I, Nv, L, nH, I * Nq * nH * L * P, 0, Nq * L * P, &lay);
    if (rc == MSDA_OK) rc = check_grad_workspace(lay, grad_workspace, grad_workspace_bytes);
    if (rc != MSDA_OK) return rc;
  }
  g_last_error[0] = '\0';
  msda::BackwardArgs a = {};
  a.value = value;
  a.image_bytes = image_bytes;
  a.bf16 = value_dtype == MSDA_BF16;
  a.grad_value = grad_value;
  a.grad_image_bytes = grad_bytes;
  a.images = I;
  a.shapes = spatial_shapes;
  a.starts = level_start_index;
  a.L = L;
  a.P = P;
  a.LP = L * P;
  a.nH = nH;
  a.Nv = (int)Nv;
  a.inv_P = 1.0f / (float)P;
  a.inv_D = 1.0f;
  a.B = I;
  a.Nq = Nq;
  a.F = (int)F;
  a.grad_out = grad_out;
  a.loc = sampling_locations;
  a.weights = attention_weights;
  a.weight_logits = weight_mode == MSDA_WEIGHTS_LOGITS;
  a.grad_loc = grad_sampling_locations;
  a.grad_weights = grad_attention_weights;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (!grad_workspace) return hip_status(msda::launch_msda_backward(a, st), "msda backward launch");
  msda::VgradArgs v = vgrad_args(lay, grad_workspace, spatial_shapes, level_start_index, L, nH, Nv, I, grad_out,
                                 B * Nq * nH, grad_value);
  v.LP = L * P;
  v.B = (int)I;
  v.Nq = (int)Nq;
  set_records(a, v, I * Nq);
  rc = hip_status(msda::launch_vgrad_setup(v, false, st), "value gradient setup");
  if (rc == MSDA_OK) rc = hip_status(msda::launch_msda_backward(a, st), "msda backward launch");
  if (rc == MSDA_OK) rc = hip_status(msda::launch_vgrad_rows(v, st), "value gradient rows");
  return rc;
}

int msda_backward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                  const int64_t* level_start_index, const float* sampling_locations, const float* attention_weights,
                  int weight_mode, const float* grad_out, int64_t B, int64_t Nv, int64_t Nq, int nH, int Dh, int L,
                  int P, float* grad_value, float* grad_sampling_locations, float* grad_attention_weights,
                  void* grad_workspace, size_t grad_workspace_bytes, void* stream) {
  return msda_backward_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_locations,
                            attention_weights, weight_mode, grad_out, B, 1, Nv, Nq, nH, Dh, L, P, grad_value,
                            grad_sampling_locations, grad_attention_weights, grad_workspace, grad_workspace_bytes,
                            stream);
}

int msda_backward_frames(const void* value, int value_dtype, const int64_t* spatial_shapes,
                         const int64_t* level_start_index, const float* sampling_locations,
                         const float* attention_weights, int weight_mode, const float* grad_out, int64_t B, int64_t F,
                         int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, float* grad_value,
                         float* grad_sampling_locations, float* grad_attention_weights, void* grad_workspace,
                         size_t grad_workspace_bytes, void* stream) {
  return msda_backward_impl(value, value_dtype, spatial_shapes, level_start_index, sampling_locations,
                            attention_weights, weight_mode, grad_out, B, F, Nv, Nq, nH, Dh, L, P, grad_value,
                            grad_sampling_locations, grad_attention_weights, grad_workspace, grad_workspace_bytes,
                            stream);
}

int sca_backward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                 const int64_t* level_start_index, const float* reference_points_cam, const float* sampling_offsets,
                 const float* attention_logits, const float* grad_slots, int64_t B, int64_t Ncam, int64_t Nv,
                 int64_t Nq, int nH, int Dh, int L, int P, int D, float* grad_value, float* grad_offsets,
                 float* grad_logits, void* workspace, size_t workspace_bytes, int64_t max_pairs,
                 void* grad_workspace, size_t grad_workspace_bytes, void* stream) {
  uint32_t image_bytes = 0, grad_bytes = 0;
  int rc = check_common(value, value_dtype, spatial_shapes, level_start_index, Nv, Nq, nH, Dh, L, P, grad_slots,
                        &image_bytes);
  if (rc != MSDA_OK) return rc;
  if (B < 1 || Ncam < 1 || D < 1) return fail(MSDA_ERR_INVALID_ARG, "B, Ncam and D must be positive");
  rc = check_grad_value(grad_value, Nv, nH, Dh, &grad_bytes);
  if (rc != MSDA_OK) return rc;
  if (Nq != 0 && (!reference_points_cam || !sampling_offsets || !attention_logits || !grad_offsets || !grad_logits))
    return fail(MSDA_ERR_INVALID_ARG, "null pointer argument");
  if (Ncam > 32) return fail(MSDA_ERR_UNSUPPORTED, "Ncam=%lld: at most 32 cameras", (long long)Ncam);
  if (P % D != 0) return fail(MSDA_ERR_SHAPE, "P=%d is not a multiple of D=%d", P, D);
  if (Nq != 0 && (!aligned(reference_points_cam, 8) || !aligned(sampling_offsets, 8) || !aligned(grad_offsets, 8) ||
                  !aligned(grad_logits, 4)))
    return fail(MSDA_ERR_INVALID_ARG, "(x, y) arrays must be 8-byte aligned");
  if (B * Ncam >= kI31 || B * Nq * nH >= kI31 / 64) return fail(MSDA_ERR_UNSUPPORTED, "B*Nq*nH too large");
  rc = check_workspace(B, Ncam, Nq, workspace, workspace_bytes);
  if (rc != MSDA_OK) return rc;
  const int64_t pairs_cap = sca_pair_capacity(B, Ncam, Nq, max_pairs);
  msda::VgradLayout lay = {};
  if (grad_workspace) {
    rc = vgrad_plan(B * Ncam, Nv, L, nH, pairs_cap * nH * L * P, Ncam * B * Nq, 0, &lay);
    if (rc == MSDA_OK) rc = check_grad_workspace(lay, grad_workspace, grad_workspace_bytes);
    if (rc != MSDA_OK) return rc;
  }
  g_last_error[0] = '\0';
  const msda::CompactArgs c = compact_args(nullptr, nullptr, B, Ncam, Nq, D, nullptr, nullptr, nullptr, workspace);
  msda::BackwardArgs a = {};
  a.value = value;
  a.image_bytes = image_bytes;
  a.bf16 = value_dtype == MSDA_BF16;
  a.grad_value = grad_value;
  a.grad_image_bytes = grad_bytes;
  a.images = B * Ncam;
  a.shapes = spatial_shapes;
  a.starts = level_start_index;
  a.L = L;
  a.P = P;
  a.LP = L * P;
  a.nH = nH;
  a.Nv = (int)Nv;
  a.inv_P = 1.0f / (float)P;
  a.inv_D = 1.0f / (float)D;
  a.B = B;
  a.Nq = Nq;
  a.grad_out = grad_slots;
  a.rp = reference_points_cam;
  a.offsets = sampling_offsets;
  a.logits = attention_logits;
  a.cammask = c.cammask;
  a.order = c.order;
  a.die_bounds = c.die_bounds;
  a.Ncam = (int)Ncam;
  a.D = D;
  a.grad_offsets = grad_offsets;
  a.grad_logits = grad_logits;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (!grad_workspace) return hip_status(msda::launch_sca_backward(a, st), "sca backward launch");
  msda::VgradArgs v = vgrad_args(lay, grad_workspace, spatial_shapes, level_start_index, L, nH, Nv, B * Ncam,
                                 grad_slots, B * Nq * nH, grad_value);
  v.LP = L * P;
  v.cammask = c.cammask;
  v.tile_offsets = c.tile_offsets;
  v.tile_counts = c.tile_counts;
  v.B = (int)B;
  v.Ncam = (int)Ncam;
  v.Nq = (int)Nq;
  v.tiles = msda::compact_layout(B, Ncam, Nq).tiles;
  v.max_pairs = pairs_cap;
  set_records(a, v, pairs_cap);
  rc = hip_status(msda::launch_vgrad_setup(v, true, st), "value gradient setup");
  if (rc == MSDA_OK) rc = hip_status(msda::launch_sca_backward(a, st), "sca backward launch");
  if (rc == MSDA_OK) rc = hip_status(msda::launch_vgrad_rows(v, st), "value gradient rows");
  return rc;
}

// ---------------------------------------------------------------------------
// sca_forward_noalloc: the SCA workspace in a static device array
// ---------------------------------------------------------------------------
// Each device the library runs on holds its own copy of this array from the
// first call on it until the process ends.  In host code `scratch` names a
// host-side stand-in: its device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[MSDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on its
// first use on that device).
int scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MSDA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MSDA_ERR_HIP, "hipGetSymbolAddress(scratch) returned no address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MSDA_OK;
}

}  // namespace

int sca_forward_noalloc(const void* value, int value_dtype, const int64_t* spatial_shapes,
                        const int64_t* level_start_index, const float* reference_points_cam, const uint8_t* bev_mask,
                        const float* sampling_offsets, const float* attention_logits, int64_t B, int64_t Ncam,
                        int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, int D, float* slots, int32_t* hit_count,
                        int32_t* pair_offsets, int32_t* pair_q, void* stream) {
  size_t need = 0;
  int rc = sca_workspace_size(B, Ncam, Nq, &need);
  if (rc != MSDA_OK) return rc;
  if (need > (size_t)MSDA_NOALLOC_SCRATCH_BYTES)
    return fail(MSDA_ERR_UNSUPPORTED,
                "B=%lld Ncam=%lld Nq=%lld needs %zu bytes of SCA scratch; sca_forward_noalloc holds %zu "
                "(use sca_forward with a workspace)", (long long)B, (long long)Ncam, (long long)Nq, need,
                (size_t)MSDA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc != MSDA_OK) return rc;
  return sca_forward(value, value_dtype, spatial_shapes, level_start_index, reference_points_cam, bev_mask,
                     sampling_offsets, attention_logits, B, Ncam, Nv, Nq, nH, Dh, L, P, D, slots, hit_count,
                     pair_offsets, pair_q, ws, (size_t)MSDA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
