/*
 * msda.h -- C ABI of libmsda.so: multi-scale deformable attention (MSDA) and
 * BEVFormer spatial cross-attention (SCA) on AMD Instinct MI355X (gfx950):
 *   msda_forward, msda_forward_frames        the MSDA operator (and a mean over frames)
 *   msda_plan_size, msda_plan, msda_gather   the operator in a locality order
 *   sca_workspace_size (sca_plan_workspace),
 *   sca_compact, sca_gather, sca_forward     SCA: visibility, compaction, sampling, camera mean
 *   sca_forward_noalloc                      sca_forward with its workspace in a static device array
 *   msda_gemm_bf16, msda_query_proj_bf16,
 *   msda_output_proj_bf16                    the layer's bf16 projections on matrix cores
 *   sca_rebatch, sca_scatter_mean            the padded rebatch form of SCA (an A/B baseline)
 *   msda_backward, sca_backward,
 *   msda_backward_workspace_size,
 *   msda_backward_frames,
 *   sca_backward_workspace_size              gradients of the MSDA operator (also of its
 *                                            frame mean) and of SCA
 *   msda_status_string, msda_last_error      status reporting
 *   msda_check_counts                        bounds-check counters (checked build)
 *
 * Sources, cited by page title and section:
 *   [8-heads]  "BEV(三) BEVFormer：Query 参数如何与 Feature 的 8 个 Head 交互"
 *              (leheavengame.com, reprint of a CSDN post).
 *   [SCA-note] Tencent Cloud developer article 2321140 on BEVFormer's Spatial
 *              Cross-Attention (bev_mask rebatch code; scatter / count /
 *              divide code).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked "device" point to GPU memory of the current HIP device;
 *    "host" pointers to ordinary CPU memory.  Every buffer is owned by the
 *    caller, dense and row-major in the shape given.  The library never
 *    allocates or frees memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it asynchronously; no entry point synchronises the
 *    host (the one exception is the debugging call msda_check_counts, which
 *    waits for the device).  Buffers must stay valid until the stream has
 *    finished the work.
 *    Every entry point enqueues kernels only (no memset or copy nodes), so
 *    it can be captured into a HIP graph and replayed.
 *  - Entry points may be called from several host threads at once.  Calls
 *    that share a workspace must be ordered (the same stream, or events):
 *    concurrent ones would overwrite each other's scratch.  The library
 *    reads the compute-unit count of the device current at its first call
 *    and sizes grids from it for every device.
 *  - Arguments are checked on the host before anything is enqueued.  A
 *    non-zero return means nothing was enqueued, except MSDA_ERR_HIP, which
 *    reports a failed launch (the stream may then hold part of the work).
 *    msda_status_string() names a code; msda_last_error() gives the message
 *    of the calling thread's last failure.
 *  - With Nq = 0 nothing is enqueued (the backward entry points still fill
 *    their value gradient with zeros) and the per-query buffers (locations,
 *    weights, offsets, logits, masks, anchors, outputs) may be NULL.
 *  - Floating-point inputs must be finite.  Sample locations may lie
 *    anywhere (outside the map they read zeros).
 *  - Shared limits: head width Dh = 32; L*P <= 64 sampling points per head;
 *    1 <= nH <= 64; one value image (Nv * nH * Dh elements of one batch
 *    item, camera or frame) under 2^31 bytes; Nq, Nv < 2^31.
 *  - Level table: spatial_shapes[l] = (H_l, W_l) and level_start_index[l] =
 *    first pixel of level l in the flattened value axis; pixel (x, y) of
 *    level l is value row level_start_index[l] + y*W_l + x.  Corners that
 *    fall outside the level, or whose row falls outside [0, Nv), read zero.
 *  - Channel layout: channel d of head h is element h*Dh + d of a pixel's
 *    value row and of an output row ([8-heads] 18.2 and 9).
 */
#ifndef MSDA_H
#define MSDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MSDA_OK 0
#define MSDA_ERR_INVALID_ARG 1 /* null pointer, bad size or enum, misaligned buffer */
#define MSDA_ERR_UNSUPPORTED 2 /* outside the shared limits above */
#define MSDA_ERR_SHAPE 3       /* inconsistent shapes (e.g. P not a multiple of D) */
#define MSDA_ERR_WORKSPACE 4   /* workspace missing, too small or misaligned */
#define MSDA_ERR_HIP 5         /* the HIP runtime reported an error */

/* element types */
#define MSDA_F32 0  /* IEEE binary32 */
#define MSDA_BF16 1 /* bfloat16 (upper half of a binary32), stored as uint16 */
/* bfloat16 value of the forward entry points in the head-pair layout: per
 * value image [nH][Nv][2][Dh] with Dh == 32, element [h][p][s][d] = channel d of
 * head h at flattened pixel p + s (s = 0, 1).  Each 128-byte line (h, p) thus
 * holds pixel p and its right-hand neighbour p + 1, the two corners a
 * bilinear sample reads in one row of a level, so that the gather fetches
 * both from one cache line.  [h][Nv-1][1] is never read (msda_pack_pairs_bf16
 * and msda_value_proj_pairs_bf16 write zeros there).  Twice the bytes of
 * MSDA_BF16 (as many as MSDA_F32).  The backward entry points refuse it. */
#define MSDA_BF16_PAIRS 2

/* meaning of attention_weights */
#define MSDA_WEIGHTS_PROB 0   /* already softmaxed over the L*P points of each head */
#define MSDA_WEIGHTS_LOGITS 1 /* logits: softmax over each head's L*P points is fused */

/*
 * MSDA operator ([8-heads] 18.5: the operator receives value, spatial_shapes,
 * level_start_index, sampling_locations and attention_weights; 4.2 softmax,
 * 6 bilinear sampling at x = W_l*s_x - 1/2, y = H_l*s_y - 1/2, 8 weighted sum
 * over levels and points, 9 concatenation of heads).
 *
 *   value               device [B][Nv][nH][Dh], MSDA_F32 or MSDA_BF16, or [B][nH][Nv][2][Dh]
 *                       in MSDA_BF16_PAIRS; 16-byte aligned
 *   spatial_shapes      device int64 [L][2], (H_l, W_l)
 *   level_start_index   device int64 [L]
 *   sampling_locations  device float [B][Nq][nH][L][P][2], normalised (x, y), 8-byte aligned
 *   attention_weights   device float [B][Nq][nH][L*P], per weight_mode
 *   out                 device float [B][Nq][nH*Dh], 16-byte aligned; fully overwritten
 *
 * out[b][q][h*Dh + d] = sum over l, p of alpha[b][q][h][l*P + p] *
 *                       bilinear(value[b][level l][.][h][d], sampling_locations[b][q][h][l][p])
 * Accumulation is in float32; bf16 values are widened exactly.
 */
int msda_forward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                 const int64_t* level_start_index, const float* sampling_locations,
                 const float* attention_weights, int weight_mode, int64_t B, int64_t Nv, int64_t Nq,
                 int nH, int Dh, int L, int P, float* out, void* stream);

/*
 * MSDA over F stacked value maps (the temporal workload: a BEV query attends
 * to the previous, aligned BEV map and the current one), with the frame as
 * an inner batch axis; each frame has its own locations and its own softmax,
 * and the output is the arithmetic mean over frames.  The pages only give
 * the operator ([8-heads] 18.5); the frame mean is this library's reading of
 * the two-map workload.
 *
 *   value               device [B][F][Nv][nH][Dh] (MSDA_BF16_PAIRS: [B][F][nH][Nv][2][Dh])
 *   sampling_locations  device float [B][F][Nq][nH][L][P][2]
 *   attention_weights   device float [B][F][Nq][nH][L*P]
 *   out                 device float [B][Nq][nH*Dh] = (1/F) * sum over f of MSDA(frame f)
 * Other arguments as msda_forward.  F >= 1.
 */
int msda_forward_frames(const void* value, int value_dtype, const int64_t* spatial_shapes,
                        const int64_t* level_start_index, const float* sampling_locations,
                        const float* attention_weights, int weight_mode, int64_t B, int64_t F,
                        int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, float* out, void* stream);

/*
 * Locality plan of the operator: the order in which msda_gather visits the
 * queries of each batch item.  The sampling locations of a query cluster
 * around its reference point on every level ([8-heads] 4.3 and 5: offsets of
 * a few cells around it), so queries visited in order of position read
 * neighbouring value rows one after the other.  Each batch item's queries
 * are sorted by the tile (32 x 32 tiles of the normalised square, taken in
 * Morton order) of the point standing for the query:
 *   point of (b, q) = points[b*batch_stride + q*point_stride + {0, 1}]
 * (normalised (x, y), clamped to [0, 1]; strides in float elements, even).
 * For the operator's own sampling_locations [B][Nq][nH][L][P][2] that is the
 * first sample of head 0: batch_stride = Nq*nH*L*P*2, point_stride =
 * nH*L*P*2; for frames [B][F][Nq]..., batch_stride = F*Nq*nH*L*P*2; for
 * reference points [B][Nq][2], 2*Nq and 2.  A plan built from the reference
 * points serves every layer that shares them.
 *
 * msda_plan_size: bytes of the plan buffer for (B, Nq) (host; no device
 *   work): the visiting order, B*Nq int32, then 64 KiB of tile counts per
 *   batch item (16 chunks of its queries x 1024 tiles).
 * msda_plan: fills the plan buffer (device, >= msda_plan_size() bytes,
 *   256-byte aligned; contents on entry irrelevant).  Its first B*Nq int32
 *   are the visiting order: entries [b*Nq, (b+1)*Nq) are batch item b's flat
 *   query indices b*Nq + q, each once (within a tile the order varies from
 *   run to run; results do not depend on it).  points: device float, 8-byte
 *   aligned.  Two small kernels.  B < 65536, B*Nq < 2^31.
 */
int msda_plan_size(int64_t B, int64_t Nq, size_t* bytes);
int msda_plan(const float* points, int64_t batch_stride, int64_t point_stride, int64_t B, int64_t Nq, void* plan,
              size_t plan_bytes, void* stream);

/*
 * msda_forward_frames (F = 1: msda_forward) visiting the queries in the
 * order of the plan that msda_plan wrote for the same B and Nq, enqueued
 * before on the same stream (or otherwise ordered before this call); plan
 * and plan_bytes as for msda_plan.  Every output row is written by exactly
 * the arithmetic of msda_forward_frames, so the result is the same bit for
 * bit; only the order of the work, and so the cache reuse, changes.  Order
 * entries outside [0, B*Nq) are skipped (their queries' rows are then not
 * written).  Other arguments as msda_forward_frames.
 */
int msda_gather(const void* value, int value_dtype, const int64_t* spatial_shapes,
                const int64_t* level_start_index, const float* sampling_locations,
                const float* attention_weights, int weight_mode, int64_t B, int64_t F, int64_t Nv, int64_t Nq,
                int nH, int Dh, int L, int P, float* out, const void* plan, size_t plan_bytes, void* stream);

/*
 * Workspace bytes sca_forward needs for (B, Ncam, Nq).  Host only; touches no
 * device.  Returns MSDA_OK and writes *bytes, or MSDA_ERR_INVALID_ARG.
 */
int sca_workspace_size(int64_t B, int64_t Ncam, int64_t Nq, size_t* bytes);

/*
 * The same query under the name of the planning step: the bytes of SCA
 * scratch (camera masks, pair lists, work order) that sca_forward,
 * sca_compact and sca_gather need for (B, Ncam, Nq).  Identical results and
 * status codes to sca_workspace_size.
 */
int sca_plan_workspace(int64_t B, int64_t Ncam, int64_t Nq, size_t* bytes);

/*
 * Spatial cross-attention forward, from the camera masks to the camera mean
 * (before the output projection).
 *
 * Steps:
 *  1. Visibility and compaction ([SCA-note] rebatch): camera c sees query q
 *     of batch item b when any of its D anchors is marked in bev_mask.  For
 *     each (b, c) in b-major order the ascending list of the queries c sees;
 *     pair_offsets[b*Ncam + c] is the start of that list in pair_q and
 *     pair_offsets[B*Ncam] the number of pairs.  hit_count[b][q] is the number
 *     of cameras that see the query ([SCA-note] count).  These are exact
 *     integers.
 *  2. For each seen (b, c, q): one softmax per head over the query's L*P
 *     logits ([8-heads] 4.2; the same for every camera, [8-heads] 10),
 *     sampling location of point p of level l at anchor p mod D:
 *     s = reference_points_cam[c][b][q][p mod D] + (dx / W_l, dy / H_l)
 *     ([8-heads] 5), bilinear sampling and the weighted sum ([8-heads] 6-9).
 *  3. slots[b][q] = (sum over the seeing cameras, in ascending order, of
 *     step 2) / max(1, hit_count[b][q]) ([8-heads] 10; [SCA-note] clamp and
 *     divide).  A query no camera sees gets zeros.
 *
 *   value                 device [B][Ncam][Nv][nH][Dh], MSDA_F32 or MSDA_BF16, or
 *                         [B][Ncam][nH][Nv][2][Dh] in MSDA_BF16_PAIRS; 16-byte aligned
 *   spatial_shapes        device int64 [L][2]; level_start_index device int64 [L]
 *   reference_points_cam  device float [Ncam][B][Nq][D][2], normalised (x, y), 8-byte aligned
 *   bev_mask              device uint8 [Ncam][B][Nq][D], nonzero = anchor marked
 *   sampling_offsets      device float [B][Nq][nH][L][P][2], in cells of level l, 8-byte aligned
 *   attention_logits      device float [B][Nq][nH][L*P]
 *   slots                 device float [B][Nq][nH*Dh], 16-byte aligned; fully overwritten
 *   hit_count             device int32 [B][Nq], or NULL
 *   pair_offsets          device int32 [B*Ncam + 1], or NULL (then kept in the workspace)
 *   pair_q                device int32 [B*Ncam*Nq] (only the first pair_offsets[B*Ncam]
 *                         entries are written), or NULL (then kept in the workspace)
 *   workspace             device, >= sca_workspace_size() bytes, 256-byte aligned; its
 *                         contents on entry do not matter and are clobbered
 * Limits: 1 <= Ncam <= 32; 1 <= D; P % D == 0 (else MSDA_ERR_SHAPE);
 * B*Ncam*Nq < 2^31; the shared limits above.
 * Equivalent to sca_compact followed by sca_gather (all arguments of both
 * are checked before either is enqueued).
 */
int sca_forward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                const int64_t* level_start_index, const float* reference_points_cam,
                const uint8_t* bev_mask, const float* sampling_offsets, const float* attention_logits,
                int64_t B, int64_t Ncam, int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, int D,
                float* slots, int32_t* hit_count, int32_t* pair_offsets, int32_t* pair_q,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 1 of sca_forward on its own: visibility, hit counts and the pair
 * lists ([SCA-note] rebatch and count), written to hit_count / pair_offsets /
 * pair_q when given, and the work list of stage 2, always in the workspace:
 * every seen query once, grouped by its first camera and by the image tile
 * of that camera's first marked anchor, so that neighbouring work items read
 * neighbouring value rows (reference_points_cam is read for this only).
 * Since the camera masks and anchors do not change between the encoder
 * layers of one frame, one sca_compact can serve several sca_gather calls.
 *   bev_mask, reference_points_cam, hit_count, pair_offsets, pair_q,
 *   workspace: as sca_forward.
 * Limits: 1 <= Ncam <= 32, D >= 1, B*Ncam*Nq < 2^31.
 */
int sca_compact(const uint8_t* bev_mask, const float* reference_points_cam, int64_t B, int64_t Ncam, int64_t Nq,
                int D, int32_t* hit_count, int32_t* pair_offsets, int32_t* pair_q, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * Stage 2 of sca_forward on its own: steps 2 and 3 for every query on the
 * work list of the workspace.  The workspace must hold what sca_compact
 * wrote for the same (B, Ncam, Nq) and the same masks and anchors, enqueued
 * before on the same stream (or otherwise ordered before this call).  slots
 * is fully overwritten.  Other arguments as sca_forward.  One kernel launch.
 */
int sca_gather(const void* value, int value_dtype, const int64_t* spatial_shapes, const int64_t* level_start_index,
               const float* reference_points_cam, const float* sampling_offsets, const float* attention_logits,
               int64_t B, int64_t Ncam, int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, int D, float* slots,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense projection on matrix cores, bf16 operands and float32 accumulation:
 *   Y[M][N] = X[M][K] * W[N][K]^T + bias[N]
 * The value projection V = W_v F + b_v ([8-heads] 3) and the output
 * projection o = W_o g + b_o ([8-heads] 11) of the bf16 configuration.
 *
 *   X     device [M][K]; MSDA_BF16, or MSDA_F32 (each element rounded to the
 *         nearest bf16, ties to even, as it is read); 16-byte aligned
 *   W     device bf16 [N][K], 16-byte aligned
 *   bias  device float [N], or NULL for zero
 *   Y     device [M][N]; MSDA_BF16 (rounded to nearest, ties to even) or MSDA_F32
 * Limits: K % 32 == 0 and 32 <= K <= 256; N % 16 == 0 and N <= 65536; M < 2^31.
 */
int msda_gemm_bf16(const void* X, int x_dtype, const uint16_t* W, const float* bias, void* Y,
                   int y_dtype, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The value projection of msda_gemm_bf16 ([8-heads] 3) with its bf16 output
 * written in the head-pair layout (MSDA_BF16_PAIRS) for the forward entry
 * points: the M = n_images * Nv rows of X are the pixels of n_images
 * value images of Nv pixels each, and the N = nH * 32 columns head h's
 * channels h*32 .. h*32+31.  Each output row is stored twice, as the left
 * half of its own line and the right half of its left-hand neighbour's
 * line; [h][Nv-1][1] of every image is set to zero.  The same products,
 * rounding and bias as msda_gemm_bf16 with y_dtype MSDA_BF16.
 *
 *   X      device [M][K]; MSDA_BF16 or MSDA_F32 (rounded to bf16 as read); 16-byte aligned
 *   W      device bf16 [N][K]; bias device float [N] or NULL; W 16-byte aligned
 *   pairs  device bf16 [n_images][nH][Nv][2][32], 16-byte aligned; must not overlap X
 * Limits: as msda_gemm_bf16, and N % 32 == 0, M % Nv == 0, Nv * nH * 128 < 2^31.
 */
int msda_value_proj_pairs_bf16(const void* X, int x_dtype, const uint16_t* W, const float* bias, uint16_t* pairs,
                               int64_t M, int64_t N, int64_t K, int64_t Nv, void* stream);

/*
 * A bf16 value in the usual layout [n_images][Nv][nH][32] rewritten in the
 * head-pair layout [n_images][nH][Nv][2][32] (MSDA_BF16_PAIRS), for callers
 * whose value comes from elsewhere than msda_value_proj_pairs_bf16.  A pure
 * copy: every element keeps its bits; [h][Nv-1][1] is set to zero.
 *
 *   value  device bf16 [n_images][Nv][nH][32], 16-byte aligned
 *   pairs  device bf16 [n_images][nH][Nv][2][32], 16-byte aligned; must not overlap value
 * (both may be NULL when n_images == 0).
 * Limits: 1 <= nH <= 64; Nv >= 1; Nv * nH * 128 < 2^31; n_images >= 0.
 */
int msda_pack_pairs_bf16(const uint16_t* value, uint16_t* pairs, int64_t n_images, int64_t Nv, int nH,
                         void* stream);

/*
 * Sampling offsets and attention logits from the query, in one launch on
 * matrix cores ([8-heads] 4.1, 4.2 and 18.3):
 *   q~              = query + query_pos            (float32 addition)
 *   offsets[M][N_off] = bf16(q~) W_off^T + b_off
 *   logits [M][N_att] = bf16(q~) W_att^T + b_att
 * bf16(.) rounds to the nearest bf16, ties to even; products accumulate in
 * float32.  For BEVFormer-base N_off = 8 heads x 4 levels x 8 points x 2 =
 * 512 and N_att = 256, laid out as sca_forward's sampling_offsets
 * [..][nH][L][P][2] and attention_logits [..][nH][L*P].
 *
 *   query      device float [M][K], 16-byte aligned
 *   query_pos  device float [M][K], 16-byte aligned, or NULL (no embedding)
 *   W_off      device bf16 [N_off][K]; W_att device bf16 [N_att][K]; 16-byte aligned
 *   b_off, b_att  device float [N_off] / [N_att], or NULL for zero
 *   offsets, logits  device float [M][N_off] / [M][N_att], 16-byte aligned
 * Limits: K % 32 == 0 and 32 <= K <= 256; N_off % 32 == 0; N_att % 16 == 0;
 * N_off + N_att <= 65536; M < 2^31.  The outputs must not overlap the inputs.
 */
int msda_query_proj_bf16(const float* query, const float* query_pos, const uint16_t* W_off, const float* b_off,
                         const uint16_t* W_att, const float* b_att, float* offsets, float* logits, int64_t M,
                         int64_t K, int64_t N_off, int64_t N_att, void* stream);

/*
 * Output projection with the residual and the encoder layer's norm
 * ([8-heads] 11, 18.6 and 18.7; dropout is the identity at inference):
 *   Y = residual + (bf16(X) W^T + bias)
 *   with gamma: each row of Y becomes (Y - mean) / sqrt(var + eps) * gamma + beta,
 *               mean and var (divisor N) taken over the row's N columns.
 *
 *   X         device [M][K]; MSDA_F32 (rounded to the nearest bf16, ties to
 *             even) or MSDA_BF16; 16-byte aligned
 *   W         device bf16 [N][K], 16-byte aligned
 *   bias      device float [N], or NULL for zero
 *   residual  device float [M][N], 16-byte aligned, or NULL (no residual);
 *             may be the same buffer as Y (each element is read before the
 *             same thread writes it)
 *   gamma, beta  device float [N], or NULL: no norm (beta needs gamma; NULL
 *             beta with gamma is a zero shift)
 *   eps       finite, >= 0 (the usual choice is 1e-5)
 *   Y         device float [M][N], 16-byte aligned
 * Limits: as msda_gemm_bf16; the norm needs N == 256.
 */
int msda_output_proj_bf16(const void* X, int x_dtype, const uint16_t* W, const float* bias, const float* residual,
                          const float* gamma, const float* beta, float eps, float* Y, int64_t M, int64_t N,
                          int64_t K, void* stream);

/*
 * Padded "rebatch" form of SCA, an A/B baseline for sca_gather ([SCA-note]
 * rebatch, scatter, count and divide code; locations as in [8-heads] 5 and
 * 18.4).  With the pair lists of sca_compact and max_len >= the longest
 * (batch item, camera) segment (the note takes the maximum on the host):
 *
 *   sca_rebatch      for every padded row (segment bc = b*Ncam + c, position
 *                    i < max_len): sampling_locations[bc][i][h][l][p] =
 *                    rho[c][b][q][p mod D] + (dx / W_l, dy / H_l) in float32
 *                    and logits_out[bc][i][h][l*P+p] = attention_logits[b][q][..],
 *                    q = pair_q[pair_offsets[bc] + i]; rows i >= segment
 *                    length get zeros.  Then msda_forward over the B*Ncam
 *                    segments (value [B][Ncam][Nv][nH][Dh] viewed as B*Ncam
 *                    images, Nq = max_len, weights as logits) gives rows
 *                    [B*Ncam][max_len][nH*Dh].
 *   sca_scatter_mean slots = 0; for each camera c in ascending order, slots[b][q]
 *                    += rows[b*Ncam + c][i] over its segment; then slots[b][q]
 *                    /= max(1, hit_count[b][q]).
 *
 *   pair_offsets, pair_q, hit_count  device int32, as written by sca_compact;
 *                    pair_q holds B*Ncam*Nq entries.  Segment bounds are
 *                    clamped to them and entries outside [0, Nq) are
 *                    skipped, so a malformed list reads and writes nothing
 *                    out of bounds (its result is then meaningless)
 *   reference_points_cam, sampling_offsets, attention_logits, spatial_shapes
 *                    as for sca_forward (device)
 *   sampling_locations device float [B*Ncam][max_len][nH][L][P][2]; logits_out
 *                    device float [B*Ncam][max_len][nH][L*P]; rows device float
 *                    [B*Ncam][max_len][C]; slots device float [B][Nq][C]
 * Alignment: (x, y) arrays 8 bytes; rows and slots 16 bytes.  C % 4 == 0.
 * A segment longer than max_len is cut at max_len (rows past it are neither
 * written nor added): pass the true maximum.
 */
int sca_rebatch(const int32_t* pair_offsets, const int32_t* pair_q, const float* reference_points_cam,
                const float* sampling_offsets, const float* attention_logits, const int64_t* spatial_shapes,
                int64_t B, int64_t Ncam, int64_t Nq, int nH, int L, int P, int D, int64_t max_len,
                float* sampling_locations, float* logits_out, void* stream);
int sca_scatter_mean(const float* rows, const int32_t* pair_offsets, const int32_t* pair_q,
                     const int32_t* hit_count, int64_t B, int64_t Ncam, int64_t Nq, int64_t C, int64_t max_len,
                     float* slots, void* stream);

/*
 * Backward pass of the MSDA operator.  The pages say only that the offsets
 * and weights are learned by back-propagation ([8-heads] 4.3); these are the
 * derivatives of msda_forward's definition ([8-heads] 4.2, 6, 8) for the
 * upstream gradient grad_out = d loss / d out:
 *   grad_value              d loss / d value, float32 [B][Nv][nH][Dh] whatever
 *                           value's type; every element written
 *   grad_sampling_locations d loss / d sampling_locations, [B][Nq][nH][L][P][2]
 *   grad_attention_weights  d loss / d attention_weights as given:
 *                           probabilities (MSDA_WEIGHTS_PROB) or logits through
 *                           each head's softmax (MSDA_WEIGHTS_LOGITS), [B][Nq][nH][L*P]
 * At an integer continuous coordinate, where bilinear sampling has a kink,
 * the derivative of the cell floor(x), floor(y) is used.
 *   grad_out   device float [B][Nq][nH*Dh], 16-byte aligned
 *   grad_value device, 16-byte aligned; one image (Nv*nH*Dh*4 bytes) < 2 GiB
 *   the gradients of locations and weights: device float, 8- and 4-byte aligned
 *   grad_workspace  device, >= msda_backward_workspace_size() bytes, 256-byte
 *              aligned, contents on entry irrelevant; or NULL.
 * The value gradient of a row is a sum over the samples of many queries.
 * With grad_workspace it is computed as a transpose gather: every sample
 * writes a record keyed by its cell, the records of each (image, head) are
 * sorted by key (a stable radix sort) and each row sums the records of its
 * four neighbouring cells in a fixed order and is written once -- no
 * atomics, and grad_value is the same bit for bit from run to run.  This needs the level table to fit its maps in
 * Nv rows (sum over levels of W*H <= Nv, as in any consistent table);
 * otherwise grad_value is filled with NaN.  With grad_workspace NULL,
 * grad_value is zeroed and accumulated with float32 atomics (its last bits
 * then vary from run to run).  The other outputs are each written once.
 * Other arguments and limits as msda_forward; with a gradient workspace, at
 * most 2^28 record slots: B*nH*ceil(Nq*L*P / 2048)*2048 < 2^28.
 */
int msda_backward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                  const int64_t* level_start_index, const float* sampling_locations, const float* attention_weights,
                  int weight_mode, const float* grad_out, int64_t B, int64_t Nv, int64_t Nq, int nH, int Dh, int L,
                  int P, float* grad_value, float* grad_sampling_locations, float* grad_attention_weights,
                  void* grad_workspace, size_t grad_workspace_bytes, void* stream);

/* Bytes of msda_backward's gradient workspace (host; no device work).  About
 * 40 bytes per record slot -- each (image, head) holds its Nq*L*P samples
 * rounded up to a multiple of 2048 -- plus 8 per cell key
 * (B*(2*Nv + 2*L)*nH), 1 KiB of digit counts per 2048 slots, 1 KiB per
 * (image, head), and a byte per value row. */
int msda_backward_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int nH, int L, int P, size_t* bytes);

/*
 * Backward pass of msda_forward_frames (the mean over F stacked value maps,
 * each frame with its own softmax): out[b][q] is the mean of the F per-frame
 * operators, so frame f's gradients are msda_backward's for the upstream
 * gradient grad_out[b] / F:
 *   grad_value              float32 [B][F][Nv][nH][Dh], every element written
 *   grad_sampling_locations [B][F][Nq][nH][L][P][2]
 *   grad_attention_weights  [B][F][Nq][nH][L*P], as given (probabilities or logits)
 *   grad_out                device float [B][Nq][nH*Dh], 16-byte aligned
 *   grad_workspace          >= msda_backward_workspace_size(B*F, Nv, Nq, nH, L, P)
 *                           bytes, or NULL (float32 atomics)
 * Other arguments, the value gradient's determinism and the limits as
 * msda_backward with B*F images.
 */
int msda_backward_frames(const void* value, int value_dtype, const int64_t* spatial_shapes,
                         const int64_t* level_start_index, const float* sampling_locations,
                         const float* attention_weights, int weight_mode, const float* grad_out, int64_t B, int64_t F,
                         int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, float* grad_value,
                         float* grad_sampling_locations, float* grad_attention_weights, void* grad_workspace,
                         size_t grad_workspace_bytes, void* stream);

/*
 * Backward pass of spatial cross-attention (sca_gather's definition,
 * [8-heads] 4.2, 5, 6, 8, 10), for grad_slots = d loss / d slots.  Each
 * seeing camera's share is divided by the hit count; offsets and logits serve
 * every camera of a query, so their gradients sum over the cameras:
 *   grad_value    float32 [B][Ncam][Nv][nH][Dh], every element written
 *   grad_offsets  d loss / d sampling_offsets (in cells), [B][Nq][nH][L][P][2]
 *   grad_logits   d loss / d attention_logits, [B][Nq][nH][L*P]
 * Queries no camera sees get zero offset and logit gradients.  The workspace
 * must hold the result of sca_compact for the same bev_mask and
 * reference_points_cam (as for sca_gather).
 *   max_pairs       capacity of grad_workspace in camera-query pairs; <= 0
 *                   means every camera seeing every query (B*Nq*Ncam).  If
 *                   the compaction found more pairs, grad_value is filled
 *                   with NaN.
 *   grad_workspace  device, >= sca_backward_workspace_size() bytes for the
 *                   same max_pairs, 256-byte aligned; or NULL (atomics).
 * The value gradient is built as for msda_backward (deterministic with a
 * gradient workspace, float32 atomics without); alignment and limits as
 * msda_backward, with at most 2^28 record slots (see
 * sca_backward_workspace_size).
 */
int sca_backward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                 const int64_t* level_start_index, const float* reference_points_cam, const float* sampling_offsets,
                 const float* attention_logits, const float* grad_slots, int64_t B, int64_t Ncam, int64_t Nv,
                 int64_t Nq, int nH, int Dh, int L, int P, int D, float* grad_value, float* grad_offsets,
                 float* grad_logits, void* workspace, size_t workspace_bytes, int64_t max_pairs,
                 void* grad_workspace, size_t grad_workspace_bytes, void* stream);

/* Bytes of sca_backward's gradient workspace for up to max_pairs camera-query
 * pairs (<= 0: B*Nq*Ncam) (host; no device work): about 40 bytes per record
 * slot -- pairs*nH*L*P samples plus up to 2048 per (image, head), since each
 * (b, c, head) starts a new block of 2048 (at most 2^28 slots) -- 8 per cell
 * key (B*Ncam*(2*Nv + 2*L)*nH), 4 per camera-query entry (Ncam*B*Nq), 1 KiB
 * of digit counts per 2048 slots, 1 KiB per (image, head), and a byte per
 * value row. */
int sca_backward_workspace_size(int64_t B, int64_t Ncam, int64_t Nv, int64_t Nq, int nH, int L, int P,
                                int64_t max_pairs, size_t* bytes);

/*
 * sca_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, results and checks as sca_forward, with the SCA
 * workspace taken from a static device array of MSDA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) instead of a caller's buffer.  Nothing is allocated, by this call
 * or by the library: each device the library runs on holds its own copy of
 * the array from the first call on it until the process ends (that first
 * call looks up the array's address, with the device current).
 *   Arguments: as sca_forward, without workspace and workspace_bytes; the
 *   caller still provides every input and output.
 *   Limit: sca_workspace_size(B, Ncam, Nq) <= MSDA_NOALLOC_SCRATCH_BYTES
 *   (6 cameras x 40000 queries need 1.48 MiB per batch item: up to B = 10);
 *   beyond it MSDA_ERR_UNSUPPORTED, with nothing enqueued.
 *   Every call on one device shares that device's array, which keeps the
 *   last call's contents (each call clears what it needs cleared): calls
 *   that can overlap on one device -- other streams, other host threads --
 *   race and give wrong results; order them (one stream, or events).
 *   One sca_forward_noalloc and later sca_gather calls cannot share the
 *   array: use sca_forward with a workspace for a compaction that serves
 *   several layers.
 */
#define MSDA_NOALLOC_SCRATCH_BYTES (16u << 20)
int sca_forward_noalloc(const void* value, int value_dtype, const int64_t* spatial_shapes,
                        const int64_t* level_start_index, const float* reference_points_cam,
                        const uint8_t* bev_mask, const float* sampling_offsets, const float* attention_logits,
                        int64_t B, int64_t Ncam, int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, int D,
                        float* slots, int32_t* hit_count, int32_t* pair_offsets, int32_t* pair_q, void* stream);

/* Name of a status code (host; static string). */
const char* msda_status_string(int status);

/* Message of the calling thread's last non-OK return (host; valid until the
 * thread's next call into the library). */
const char* msda_last_error(void);

/* Device-side bounds checks (host; a debugging aid for every caller, not a
 * passage of the pages).  libmsda_checked.so is the same library built with
 * MSDA_CHECKED: its kernels check the compaction's pair-list and work-list
 * writes against their segments, every work-list, plan and pair-list entry
 * they read against the range it must lie in, and every corner row a gather
 * stages against its sample's level and head.  A failed check adds one to a
 * counter of its kind (MSDA_CHECK_*) on the device for each lane that sees
 * it (a count of lanes, not of distinct entries: zero is the only value
 * with a fixed meaning); nothing traps and no result changes.  msda_check_counts waits for the current device
 * (hipDeviceSynchronize, unlike every other entry point), writes the
 * counters summed over the library to counts[0 .. MSDA_CHECK_KINDS), and
 * zeroes them when reset != 0.  counts must hold MSDA_CHECK_KINDS entries
 * (else MSDA_ERR_INVALID_ARG).  In the regular libmsda.so it returns
 * MSDA_ERR_UNSUPPORTED and touches nothing.  Counters are per device and
 * shared by every call on it. */
#define MSDA_CHECK_KINDS 4
#define MSDA_CHECK_GATHER_ROW 0  /* staged corner row outside its sample's level or head */
#define MSDA_CHECK_PAIR_WRITE 1  /* pair-list entry written outside its run, or a query outside [0, Nq) */
#define MSDA_CHECK_ORDER_WRITE 2 /* work-list slot written outside its segment's range */
#define MSDA_CHECK_LIST_ENTRY 3  /* work-list, plan, pair-list or segment-bound entry read out of its range */
int msda_check_counts(unsigned long long* counts, int n, int reset);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H */
