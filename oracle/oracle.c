/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for multi-scale
 * deformable attention (MSDA) and the spatial cross-attention (SCA) built on it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this code.  The HIP library never
 * calls it, links it or shares a line of source with it.
 *
 * Sources, cited by page title and section:
 *   [8-heads]  "BEV(三) BEVFormer：Query 参数如何与 Feature 的 8 个 Head 交互"
 *              (leheavengame.com, reprint of a CSDN post), sections 1-18.
 *   [SCA-note] Tencent Cloud developer article 2321140, a note on BEVFormer's
 *              Spatial Cross-Attention: its bev_mask rebatch code and its
 *              scatter / count / divide code.
 *
 * Everything is computed in IEEE double with plain nested loops in the order
 * the pages describe.  float32 inputs and bfloat16 bit patterns convert to
 * double exactly, so the only rounding is double rounding (about 1e-16).
 *
 * Readings where the pages are silent or garbled (each is also listed in the
 * design notes):
 *   - softmax denominator: sum over all L*P logits of one head ([8-heads] 4.2;
 *     the printed summation limits are garbled; the same section says each
 *     head normalises its own 32 = 4 levels x 8 points logits and that the
 *     weights of a head add up to one, which fixes the range);
 *   - bilinear boundary: every corner outside the map contributes zero and the
 *     remaining weights are not renormalised (the pages only say "four
 *     neighbour bilinear"; zero padding is the plainest reading);
 *   - corner index: floor toward minus infinity;
 *   - level table: spatial_shapes rows are (H_l, W_l); level l occupies pixels
 *     [start_l, start_l + H_l*W_l) of the flattened value axis, row-major, so
 *     pixel (x, y) of level l sits at start_l + y*W_l + x;
 *   - value layout [.., Nv, nH, Dh] so channel d of head h sits at h*Dh + d
 *     ([8-heads] 18.2 view(bs, num_value, heads, -1)); output likewise
 *     ([8-heads] 9, concatenation of heads);
 *   - point -> height anchor: m(k) = k mod D for the point index k inside a
 *     level ([8-heads] 5: k = 4j + m with D = 4);
 *   - offsets are divided by the level's (W_l, H_l), x by W and y by H
 *     ([8-heads] 5 and 18.4; the [SCA-note] omits the normaliser, [8-heads]
 *     is followed);
 *   - compaction is per (batch item, camera) ([SCA-note] builds its index
 *     list from batch item 0's mask but counts hits per batch item; the two
 *     agree when masks do not vary over the batch, and per-item compaction is
 *     the only reading in which scatter and count agree otherwise);
 *   - frames (two stacked BEV maps, temporal workload): two independent MSDAs,
 *     each with its own softmax, then the arithmetic mean over frames.  The
 *     pages do not describe this variant; parity of the frame mean rests on
 *     the invariants in the tests (identical frames, zero frame, symmetry);
 *   - bf16 projections: operands rounded to the nearest bf16 (ties to even),
 *     products summed exactly enough in double; the query-side input is the
 *     float32 sum query + position embedding ([8-heads] 4);
 *   - the encoder layer's norm after the residual ([8-heads] 18.7) is the
 *     plain layer norm over the row (variance with divisor N, eps inside the
 *     square root, then gamma and beta); the pages name it only;
 *   - backward pass ([8-heads] 4.3 says only that offsets and weights are
 *     learned by back-propagation): the derivatives of the forward
 *     definitions; at an integer x or y, where bilinear sampling has a kink,
 *     the derivative of the cell floor(x), floor(y) is taken.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> double                                                       */
/* ------------------------------------------------------------------------ */

/* A bfloat16 is the upper half of a float32 bit pattern, so widening is exact. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Nearest bfloat16 to x, ties to the even significand.  A bfloat16 has an
 * 8-bit significand (7 stored bits), exponent range as float32.  Write
 * x = m * 2^e with 0.5 <= |m| < 1; the bf16 spacing there is 2^(e-8), and
 * below the smallest normal (2^-126) the spacing stays 2^-133.  rint() rounds
 * half to even in the default rounding mode.
 */
uint16_t oracle_double_to_bf16(double x)
{
    if (isnan(x)) return (uint16_t)0x7FC0;
    if (x == 0.0) return signbit(x) ? (uint16_t)0x8000 : (uint16_t)0x0000;
    int e;
    (void)frexp(x, &e);
    if (e < -125) e = -125;
    double quantum = ldexp(1.0, e - 8);
    double y = rint(x / quantum) * quantum;
    const double bf16_max = 3.3895313892515355e38; /* (2 - 2^-7) * 2^127 */
    if (y > bf16_max) return (uint16_t)0x7F80;
    if (y < -bf16_max) return (uint16_t)0xFF80;
    float f = (float)y; /* exact: y is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_round_to_bf16(const double* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_double_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* value access                                                              */
/* ------------------------------------------------------------------------ */

/* One value image: [Nv][nH][Dh], float32 or bfloat16 bit patterns. */
typedef struct {
    const void* data;
    int is_bf16;
    int64_t nH, Dh;
} ValueImage;

static double value_at(const ValueImage* v, int64_t pixel, int64_t h, int64_t d)
{
    int64_t i = (pixel * v->nH + h) * v->Dh + d;
    if (v->is_bf16) return oracle_bf16_to_double(((const uint16_t*)v->data)[i]);
    return (double)((const float*)v->data)[i];
}

/* ------------------------------------------------------------------------ */
/* the method's steps                                                        */
/* ------------------------------------------------------------------------ */

/* [8-heads] 4.2: alpha_i = exp(a_i) / sum_j exp(a_j) over one head's logits. */
static void softmax(const float* logits, int n, double* alpha)
{
    double denom = 0.0;
    for (int i = 0; i < n; ++i) denom += exp((double)logits[i]);
    for (int i = 0; i < n; ++i) alpha[i] = exp((double)logits[i]) / denom;
}

/*
 * [8-heads] 6 and 7: sample head h of level (H, W, start) at the normalised
 * location (sx, sy) with four-neighbour bilinear interpolation and add
 * weight * sample to acc[0..Dh).  The continuous coordinate on the level is
 * x = W*sx - 1/2, y = H*sy - 1/2.  Corners outside the map add nothing.
 */
static void bilinear_accumulate(const ValueImage* v, int64_t H, int64_t W, int64_t start,
                                int64_t h, double sx, double sy, double weight, double* acc)
{
    double x = (double)W * sx - 0.5;
    double y = (double)H * sy - 0.5;
    double x0 = floor(x), y0 = floor(y);
    double fx = x - x0, fy = y - y0;
    for (int j = 0; j < 2; ++j) {
        for (int i = 0; i < 2; ++i) {
            double cx = x0 + i, cy = y0 + j;
            if (cx < 0.0 || cx >= (double)W || cy < 0.0 || cy >= (double)H) continue;
            double w = (i ? fx : 1.0 - fx) * (j ? fy : 1.0 - fy);
            int64_t pixel = start + (int64_t)cy * W + (int64_t)cx;
            for (int64_t d = 0; d < v->Dh; ++d) acc[d] += weight * w * value_at(v, pixel, h, d);
        }
    }
}

static int levels_ok(const int64_t* shapes, const int64_t* starts, int L, int64_t Nv)
{
    for (int l = 0; l < L; ++l) {
        int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
        if (H <= 0 || W <= 0 || starts[l] < 0 || starts[l] + H * W > Nv) return 0;
    }
    return 1;
}

/*
 * [8-heads] 8 and 9: one query against one value image.  For each head h,
 * g^(h) = sum over levels l and points k of alpha[h][l][k] * B(V^(h)_l, s[h][l][k]),
 * and the output row is the concatenation of the heads (channel h*Dh + d).
 *   loc   [nH][L][P][2]  normalised (x, y)
 *   alpha [nH][L*P]
 *   out   [nH*Dh]        overwritten
 */
static void msda_query(const ValueImage* img, const int64_t* shapes, const int64_t* starts,
                       int nH, int Dh, int L, int P, const float* loc, const double* alpha, double* out)
{
    for (int h = 0; h < nH; ++h) {
        double* acc = out + (int64_t)h * Dh;
        for (int d = 0; d < Dh; ++d) acc[d] = 0.0;
        for (int l = 0; l < L; ++l) {
            for (int k = 0; k < P; ++k) {
                const float* s = loc + (((int64_t)h * L + l) * P + k) * 2;
                bilinear_accumulate(img, shapes[2 * l], shapes[2 * l + 1], starts[l], h,
                                    (double)s[0], (double)s[1], alpha[(int64_t)h * L * P + l * P + k], acc);
            }
        }
    }
}

/* Head weights of one query: logits -> softmax per head ([8-heads] 4.2), or the
 * probabilities as given (the operator in [8-heads] 18.5 receives weights that
 * were already softmaxed in 18.3). */
static void head_weights(const float* w, int nH, int LP, int are_logits, double* alpha)
{
    for (int h = 0; h < nH; ++h) {
        if (are_logits) softmax(w + (int64_t)h * LP, LP, alpha + (int64_t)h * LP);
        else for (int i = 0; i < LP; ++i) alpha[(int64_t)h * LP + i] = (double)w[(int64_t)h * LP + i];
    }
}

/*
 * MSDA operator ([8-heads] 18.5: value, spatial_shapes, level_start_index,
 * sampling_locations, attention_weights).
 *   value               [B][Nv][nH][Dh]    float32, or bf16 bits if value_bf16
 *   spatial_shapes      [L][2]             (H_l, W_l)
 *   level_start_index   [L]
 *   sampling_locations  [B][Nq][nH][L][P][2]
 *   attention_weights   [B][Nq][nH][L*P]   logits if weights_are_logits, else probabilities
 *   rows                list of b*Nq + q to evaluate (NULL: all B*Nq rows in order)
 *   out                 [n_rows][nH*Dh]
 */
int oracle_msda(const void* value, int value_bf16, const int64_t* spatial_shapes,
                const int64_t* level_start_index, const float* sampling_locations,
                const float* attention_weights, int weights_are_logits, int64_t B, int64_t Nv,
                int64_t Nq, int nH, int Dh, int L, int P, const int64_t* rows, int64_t n_rows,
                double* out)
{
    if (!value || !spatial_shapes || !level_start_index || !sampling_locations || !attention_weights || !out)
        return ORACLE_BAD_ARG;
    if (B < 1 || Nv < 1 || Nq < 0 || nH < 1 || Dh < 1 || L < 1 || P < 1) return ORACLE_BAD_ARG;
    if (!levels_ok(spatial_shapes, level_start_index, L, Nv)) return ORACLE_BAD_ARG;
    if (!rows) n_rows = B * Nq;
    const int LP = L * P;
    double* alpha = (double*)malloc(sizeof(double) * (size_t)nH * LP);
    if (!alpha) return ORACLE_BAD_ARG;
    const size_t elem = value_bf16 ? 2 : 4;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t bq = rows ? rows[r] : r;
        if (bq < 0 || bq >= B * Nq) { free(alpha); return ORACLE_BAD_ARG; }
        int64_t b = bq / Nq;
        ValueImage img = {(const char*)value + (size_t)(b * Nv * nH * Dh) * elem, value_bf16, nH, Dh};
        head_weights(attention_weights + bq * nH * LP, nH, LP, weights_are_logits, alpha);
        msda_query(&img, spatial_shapes, level_start_index, nH, Dh, L, P,
                   sampling_locations + bq * nH * LP * 2, alpha, out + r * nH * Dh);
    }
    free(alpha);
    return ORACLE_OK;
}

/*
 * Temporal workload: F stacked value maps, one MSDA per frame (own locations,
 * own softmax), then the arithmetic mean over frames.
 *   value               [B][F][Nv][nH][Dh]
 *   sampling_locations  [B][F][Nq][nH][L][P][2]
 *   attention_weights   [B][F][Nq][nH][L*P]
 *   rows                list of b*Nq + q (NULL: all)
 *   out                 [n_rows][nH*Dh]
 */
int oracle_msda_frames(const void* value, int value_bf16, const int64_t* spatial_shapes,
                       const int64_t* level_start_index, const float* sampling_locations,
                       const float* attention_weights, int weights_are_logits, int64_t B, int64_t F,
                       int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, const int64_t* rows,
                       int64_t n_rows, double* out)
{
    if (!value || !spatial_shapes || !level_start_index || !sampling_locations || !attention_weights || !out)
        return ORACLE_BAD_ARG;
    if (B < 1 || F < 1 || Nv < 1 || Nq < 0 || nH < 1 || Dh < 1 || L < 1 || P < 1) return ORACLE_BAD_ARG;
    if (!levels_ok(spatial_shapes, level_start_index, L, Nv)) return ORACLE_BAD_ARG;
    if (!rows) n_rows = B * Nq;
    const int LP = L * P;
    const int64_t C = (int64_t)nH * Dh;
    double* alpha = (double*)malloc(sizeof(double) * (size_t)nH * LP);
    double* one = (double*)malloc(sizeof(double) * (size_t)C);
    if (!alpha || !one) { free(alpha); free(one); return ORACLE_BAD_ARG; }
    const size_t elem = value_bf16 ? 2 : 4;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t bq = rows ? rows[r] : r;
        if (bq < 0 || bq >= B * Nq) { free(alpha); free(one); return ORACLE_BAD_ARG; }
        int64_t b = bq / Nq, q = bq % Nq;
        double* o = out + r * C;
        for (int64_t i = 0; i < C; ++i) o[i] = 0.0;
        for (int64_t f = 0; f < F; ++f) {
            int64_t bf = b * F + f;
            ValueImage img = {(const char*)value + (size_t)(bf * Nv * C) * elem, value_bf16, nH, Dh};
            head_weights(attention_weights + (bf * Nq + q) * nH * LP, nH, LP, weights_are_logits, alpha);
            msda_query(&img, spatial_shapes, level_start_index, nH, Dh, L, P,
                       sampling_locations + (bf * Nq + q) * nH * LP * 2, alpha, one);
            for (int64_t i = 0; i < C; ++i) o[i] += one[i];
        }
        for (int64_t i = 0; i < C; ++i) o[i] /= (double)F;
    }
    free(alpha);
    free(one);
    return ORACLE_OK;
}

/*
 * Spatial cross-attention.
 *   value                 [B][Ncam][Nv][nH][Dh]   (batch-major, camera-minor)
 *   reference_points_cam  [Ncam][B][Nq][D][2]     projected pillar anchors, normalised (x, y)
 *   bev_mask              [Ncam][B][Nq][D]        nonzero = anchor lands in the image
 *   sampling_offsets      [B][Nq][nH][L][P][2]    in cells of level l ([8-heads] 4.3)
 *   attention_logits      [B][Nq][nH][L*P]
 *   rows                  list of b*Nq + q for slots (NULL: all)
 * Outputs (each may be NULL):
 *   slots         [n_rows][nH*Dh]
 *   hit_count     [B*Nq]          number of cameras that see each query
 *   pair_offsets  [B*Ncam + 1]    start of segment (b, c) in pair_q, b-major
 *   pair_q        [<= B*Ncam*Nq]  ascending query indices of each segment
 */
int oracle_sca(const void* value, int value_bf16, const int64_t* spatial_shapes,
               const int64_t* level_start_index, const float* reference_points_cam,
               const uint8_t* bev_mask, const float* sampling_offsets, const float* attention_logits,
               int64_t B, int64_t Ncam, int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P, int D,
               const int64_t* rows, int64_t n_rows, double* slots, int32_t* hit_count,
               int32_t* pair_offsets, int32_t* pair_q)
{
    if (!value || !spatial_shapes || !level_start_index || !reference_points_cam || !bev_mask ||
        !sampling_offsets || !attention_logits)
        return ORACLE_BAD_ARG;
    if (B < 1 || Ncam < 1 || Nv < 1 || Nq < 0 || nH < 1 || Dh < 1 || L < 1 || P < 1 || D < 1 || P % D != 0)
        return ORACLE_BAD_ARG;
    if (!levels_ok(spatial_shapes, level_start_index, L, Nv)) return ORACLE_BAD_ARG;
    const int LP = L * P;
    const int64_t C = (int64_t)nH * Dh;

    /* Step 1 ([SCA-note] rebatch and count): camera c sees query q of batch
     * item b when any of the query's D anchors is marked in bev_mask. */
    uint8_t* vis = (uint8_t*)malloc((size_t)(Ncam * B * Nq) + 1);
    if (!vis) return ORACLE_BAD_ARG;
    for (int64_t c = 0; c < Ncam; ++c)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t q = 0; q < Nq; ++q) {
                int any = 0;
                for (int m = 0; m < D; ++m) any |= bev_mask[((c * B + b) * Nq + q) * D + m] != 0;
                vis[(c * B + b) * Nq + q] = (uint8_t)any;
            }

    /* Step 2 ([SCA-note] rebatch): for each batch item and camera, the
     * ascending list of the queries that camera sees. */
    if (pair_offsets || pair_q) {
        int64_t n = 0;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t c = 0; c < Ncam; ++c) {
                if (pair_offsets) pair_offsets[b * Ncam + c] = (int32_t)n;
                for (int64_t q = 0; q < Nq; ++q)
                    if (vis[(c * B + b) * Nq + q]) {
                        if (pair_q) pair_q[n] = (int32_t)q;
                        ++n;
                    }
            }
        if (pair_offsets) pair_offsets[B * Ncam] = (int32_t)n;
    }

    /* Step 3 ([SCA-note] count; [8-heads] 10): number of cameras seeing each query. */
    if (hit_count)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t q = 0; q < Nq; ++q) {
                int32_t hits = 0;
                for (int64_t c = 0; c < Ncam; ++c) hits += vis[(c * B + b) * Nq + q];
                hit_count[b * Nq + q] = hits;
            }

    if (slots) {
        if (!rows) n_rows = B * Nq;
        double* alpha = (double*)malloc(sizeof(double) * (size_t)nH * LP);
        double* g = (double*)malloc(sizeof(double) * (size_t)C);
        if (!alpha || !g) {
            free(alpha); free(g); free(vis);
            return ORACLE_BAD_ARG;
        }
        const size_t elem = value_bf16 ? 2 : 4;
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t bq = rows ? rows[r] : r;
            if (bq < 0 || bq >= B * Nq) {
                free(alpha); free(g); free(vis);
                return ORACLE_BAD_ARG;
            }
            int64_t b = bq / Nq, q = bq % Nq;
            double* out = slots + r * C;
            for (int64_t i = 0; i < C; ++i) out[i] = 0.0;

            /* Step 4 ([8-heads] 4.2 and 10): one softmax per head; the offsets and
             * weights come from the query alone, so every camera uses the same ones. */
            head_weights(attention_logits + bq * nH * LP, nH, LP, 1, alpha);

            int hits = 0;
            for (int64_t c = 0; c < Ncam; ++c) {
                if (!vis[(c * B + b) * Nq + q]) continue;
                ++hits;
                ValueImage img = {(const char*)value + (size_t)((b * Ncam + c) * Nv * C) * elem,
                                  value_bf16, nH, Dh};
                const float* rho = reference_points_cam + ((c * B + b) * Nq + q) * D * 2;
                for (int h = 0; h < nH; ++h) {
                    double* acc = g + (int64_t)h * Dh;
                    for (int d = 0; d < Dh; ++d) acc[d] = 0.0;
                    for (int l = 0; l < L; ++l) {
                        int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1];
                        for (int k = 0; k < P; ++k) {
                            /* Step 5 ([8-heads] 5): point k uses height anchor k mod D and
                             * s = rho + (dx / W_l, dy / H_l). */
                            int m = k % D;
                            const float* off = sampling_offsets + ((bq * nH + h) * L + l) * P * 2 + (int64_t)k * 2;
                            double sx = (double)rho[m * 2 + 0] + (double)off[0] / (double)W;
                            double sy = (double)rho[m * 2 + 1] + (double)off[1] / (double)H;
                            bilinear_accumulate(&img, H, W, level_start_index[l], h, sx, sy,
                                                alpha[(int64_t)h * LP + l * P + k], acc);
                        }
                    }
                }
                /* Step 6 ([SCA-note] scatter): add this camera's result to the query's slot. */
                for (int64_t i = 0; i < C; ++i) out[i] += g[i];
            }
            /* Step 7 ([8-heads] 10; [SCA-note] clamp and divide): mean over the
             * cameras that see the query; a query no camera sees keeps zeros. */
            double n = hits > 1 ? (double)hits : 1.0;
            for (int64_t i = 0; i < C; ++i) out[i] /= n;
        }
        free(alpha); free(g);
    }
    free(vis);
    return ORACLE_OK;
}

/*
 * Linear layer from bf16 operands, accumulated in double:
 *   Y[M][N] = X[M][K] * W[N][K]^T + bias[N]
 * ([8-heads] 3: value projection V = W_v F + b_v; [8-heads] 11: output
 * projection o = W_o g + b_o).  X is bf16 bits, or float32 that is first
 * rounded to the nearest bf16 (the bf16 configuration stores the camera-mean
 * slots in bf16 before the output projection).  bias may be NULL.
 */
int oracle_linear_bf16(const void* X, int x_is_f32, const uint16_t* W, const float* bias,
                       int64_t M, int64_t N, int64_t K, double* Y)
{
    if (!X || !W || !Y || M < 0 || N < 1 || K < 1) return ORACLE_BAD_ARG;
    double* xrow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!xrow) return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t k = 0; k < K; ++k) {
            if (x_is_f32)
                xrow[k] = oracle_bf16_to_double(oracle_double_to_bf16((double)((const float*)X)[i * K + k]));
            else
                xrow[k] = oracle_bf16_to_double(((const uint16_t*)X)[i * K + k]);
        }
        for (int64_t n = 0; n < N; ++n) {
            double acc = bias ? (double)bias[n] : 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xrow[k] * oracle_bf16_to_double(W[n * K + k]);
            Y[i * N + n] = acc;
        }
    }
    free(xrow);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Query projections ([8-heads] 4.1, 4.2 and 18.3)                          */
/* ------------------------------------------------------------------------ */

/*
 * The vector that predicts the sampling parameters is the query plus its
 * position embedding ([8-heads] 4).  In the model both are float32 tensors,
 * so their sum is a float32 tensor: it is formed here with one float32
 * addition (the file is compiled without contraction or excess precision).
 * Then offsets = W_off q~ + b_off ([8-heads] 4.1, N_off = heads x levels x
 * points x 2) and logits = W_att q~ + b_att ([8-heads] 4.2, N_att = heads x
 * levels x points), each a bf16-operand linear map as in oracle_linear_bf16
 * (q~ rounded to the nearest bf16).  query_pos may be NULL (no embedding).
 */
int oracle_query_proj(const float* query, const float* query_pos, int64_t M, int64_t K,
                      const uint16_t* W_off, const float* b_off, int64_t N_off,
                      const uint16_t* W_att, const float* b_att, int64_t N_att,
                      double* offsets, double* logits)
{
    if (!query || !W_off || !W_att || !offsets || !logits || M < 0 || K < 1 || N_off < 1 || N_att < 1)
        return ORACLE_BAD_ARG;
    float* qt = (float*)malloc(sizeof(float) * (size_t)K);
    if (!qt) return ORACLE_BAD_ARG;
    int rc = ORACLE_OK;
    for (int64_t i = 0; i < M && rc == ORACLE_OK; ++i) {
        for (int64_t k = 0; k < K; ++k) {
            float s = query[i * K + k];
            if (query_pos) s = s + query_pos[i * K + k];
            qt[k] = s;
        }
        rc = oracle_linear_bf16(qt, 1, W_off, b_off, 1, N_off, K, offsets + i * N_off);
        if (rc == ORACLE_OK) rc = oracle_linear_bf16(qt, 1, W_att, b_att, 1, N_att, K, logits + i * N_att);
    }
    free(qt);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Output projection, residual and the layer's norm ([8-heads] 11, 18.6-7)  */
/* ------------------------------------------------------------------------ */

/*
 * o = W_o bf16(slots) + b_o (oracle_linear_bf16 with the float32 slots
 * rounded to the nearest bf16); q^ = residual + o, the dropout on the update
 * branch being the identity at inference ([8-heads] 18.6; residual may be
 * NULL: no residual).  With gamma given, the encoder layer's norm that
 * follows ([8-heads] 18.7): each row of q^ is centred on its mean, divided by
 * sqrt(variance + eps) with the variance taken over the row's N entries
 * (divisor N), then multiplied by gamma and shifted by beta (NULL beta: 0).
 * The pages name the norm but not its formula; this is the plain layer norm.
 */
int oracle_output_proj(const float* slots, const uint16_t* W, const float* bias, const float* residual,
                       const float* gamma, const float* beta, double eps, int64_t M, int64_t N, int64_t K,
                       double* Y)
{
    if (!slots || !W || !Y || M < 0 || N < 1 || K < 1) return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < M; ++i) {
        double* y = Y + i * N;
        int rc = oracle_linear_bf16(slots + i * K, 1, W, bias, 1, N, K, y);
        if (rc != ORACLE_OK) return rc;
        if (residual)
            for (int64_t n = 0; n < N; ++n) y[n] += (double)residual[i * N + n];
        if (gamma) {
            double mean = 0.0;
            for (int64_t n = 0; n < N; ++n) mean += y[n];
            mean /= (double)N;
            double var = 0.0;
            for (int64_t n = 0; n < N; ++n) var += (y[n] - mean) * (y[n] - mean);
            var /= (double)N;
            double inv = 1.0 / sqrt(var + eps);
            for (int64_t n = 0; n < N; ++n)
                y[n] = (y[n] - mean) * inv * (double)gamma[n] + (beta ? (double)beta[n] : 0.0);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward pass                                                             */
/* ------------------------------------------------------------------------ */

/*
 * The pages say only that the offsets and the weights are learned by back-
 * propagation ([8-heads] 4.3).  The gradients here are the derivatives of the
 * forward definitions above, by the chain rule.  For one head of one query,
 *   out = sum_k alpha_k * S_k,   S_k = sum over corners c of w_c * V[c],
 *   x = W*sx - 1/2, y = H*sy - 1/2, fx = x - floor(x), fy = y - floor(y),
 *   w_c = (i ? fx : 1-fx) * (j ? fy : 1-fy)  for corner (floor(x)+i, floor(y)+j);
 * so, with g = d loss / d out,
 *   d loss / d alpha_k = <S_k, g>,
 *   d loss / d V[c]   += alpha_k * w_c * g,
 *   d loss / d x       = alpha_k * sum_c <V[c], g> * d w_c / d x,
 *       d w_c / d x = (i ? 1 : -1) * (j ? fy : 1-fy),  d w_c / d y = (i ? fx : 1-fx) * (j ? 1 : -1),
 *   d x / d sx = W,  d y / d sy = H;
 * through the softmax, d loss / d a_i = alpha_i * (d loss / d alpha_i - sum_k alpha_k d loss / d alpha_k).
 * Corners outside the map hold no value (zero padding) and contribute to none
 * of these.  Where x or y is an integer the sampled function has a kink; the
 * derivative taken is the one of the cell floor(x), floor(y) (its right-hand
 * derivative), the plainest reading.
 */

/* One sample's backward: adds alpha * w_c * g to the value gradient of each
 * corner (grad_img laid out as the value image, may be NULL) and returns
 * <S, g>, <dS/dx, g> and <dS/dy, g>. */
static void bilinear_backward(const ValueImage* v, double* grad_img, int64_t H, int64_t W, int64_t start,
                              int64_t h, double sx, double sy, double weight, const double* g,
                              double* dot_s, double* dot_x, double* dot_y)
{
    double x = (double)W * sx - 0.5;
    double y = (double)H * sy - 0.5;
    double x0 = floor(x), y0 = floor(y);
    double fx = x - x0, fy = y - y0;
    *dot_s = *dot_x = *dot_y = 0.0;
    for (int j = 0; j < 2; ++j) {
        for (int i = 0; i < 2; ++i) {
            double cx = x0 + i, cy = y0 + j;
            if (cx < 0.0 || cx >= (double)W || cy < 0.0 || cy >= (double)H) continue;
            double w = (i ? fx : 1.0 - fx) * (j ? fy : 1.0 - fy);
            double wx = (i ? 1.0 : -1.0) * (j ? fy : 1.0 - fy);
            double wy = (i ? fx : 1.0 - fx) * (j ? 1.0 : -1.0);
            int64_t pixel = start + (int64_t)cy * W + (int64_t)cx;
            for (int64_t d = 0; d < v->Dh; ++d) {
                double vg = value_at(v, pixel, h, d) * g[d];
                *dot_s += w * vg;
                *dot_x += wx * vg;
                *dot_y += wy * vg;
                if (grad_img) grad_img[(pixel * v->nH + h) * v->Dh + d] += weight * w * g[d];
            }
        }
    }
}

/* d loss / d weights of one query: through the softmax of each head for
 * logits, as is for probabilities. */
static void weights_backward(const double* alpha, const double* dalpha, int nH, int LP, int are_logits,
                             double* grad_w)
{
    for (int h = 0; h < nH; ++h) {
        const double* a = alpha + (int64_t)h * LP;
        const double* da = dalpha + (int64_t)h * LP;
        double* gw = grad_w + (int64_t)h * LP;
        if (!are_logits) {
            for (int i = 0; i < LP; ++i) gw[i] = da[i];
            continue;
        }
        double dot = 0.0;
        for (int i = 0; i < LP; ++i) dot += a[i] * da[i];
        for (int i = 0; i < LP; ++i) gw[i] = a[i] * (da[i] - dot);
    }
}

/*
 * Gradients of the MSDA operator (oracle_msda) for d loss / d out = grad_out.
 *   grad_out        [B][Nq][nH*Dh]
 *   grad_value      [B][Nv][nH][Dh]        overwritten
 *   grad_locations  [B][Nq][nH][L][P][2]   with respect to the normalised (x, y)
 *   grad_weights    [B][Nq][nH][L*P]       with respect to attention_weights as given
 *                                          (logits or probabilities)
 */
int oracle_msda_backward(const void* value, int value_bf16, const int64_t* spatial_shapes,
                         const int64_t* level_start_index, const float* sampling_locations,
                         const float* attention_weights, int weights_are_logits, const float* grad_out,
                         int64_t B, int64_t Nv, int64_t Nq, int nH, int Dh, int L, int P,
                         double* grad_value, double* grad_locations, double* grad_weights)
{
    if (!value || !spatial_shapes || !level_start_index || !sampling_locations || !attention_weights ||
        !grad_out || !grad_value || !grad_locations || !grad_weights)
        return ORACLE_BAD_ARG;
    if (B < 1 || Nv < 1 || Nq < 0 || nH < 1 || Dh < 1 || L < 1 || P < 1) return ORACLE_BAD_ARG;
    if (!levels_ok(spatial_shapes, level_start_index, L, Nv)) return ORACLE_BAD_ARG;
    const int LP = L * P;
    const int64_t C = (int64_t)nH * Dh;
    for (int64_t i = 0; i < B * Nv * C; ++i) grad_value[i] = 0.0;
    double* alpha = (double*)malloc(sizeof(double) * (size_t)nH * LP);
    double* dalpha = (double*)malloc(sizeof(double) * (size_t)nH * LP);
    double* g = (double*)malloc(sizeof(double) * (size_t)Dh);
    if (!alpha || !dalpha || !g) { free(alpha); free(dalpha); free(g); return ORACLE_BAD_ARG; }
    const size_t elem = value_bf16 ? 2 : 4;
    for (int64_t bq = 0; bq < B * Nq; ++bq) {
        int64_t b = bq / Nq;
        ValueImage img = {(const char*)value + (size_t)(b * Nv * C) * elem, value_bf16, nH, Dh};
        double* grad_img = grad_value + b * Nv * C;
        head_weights(attention_weights + bq * nH * LP, nH, LP, weights_are_logits, alpha);
        for (int h = 0; h < nH; ++h) {
            for (int d = 0; d < Dh; ++d) g[d] = (double)grad_out[bq * C + (int64_t)h * Dh + d];
            for (int l = 0; l < L; ++l) {
                int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1];
                for (int k = 0; k < P; ++k) {
                    int64_t at = ((bq * nH + h) * L + l) * P + k;
                    const float* s = sampling_locations + at * 2;
                    double a = alpha[(int64_t)h * LP + l * P + k];
                    double ds, dx, dy;
                    bilinear_backward(&img, grad_img, H, W, level_start_index[l], h, (double)s[0], (double)s[1],
                                      a, g, &ds, &dx, &dy);
                    dalpha[(int64_t)h * LP + l * P + k] = ds;
                    grad_locations[at * 2 + 0] = a * (double)W * dx;
                    grad_locations[at * 2 + 1] = a * (double)H * dy;
                }
            }
        }
        weights_backward(alpha, dalpha, nH, LP, weights_are_logits, grad_weights + bq * nH * LP);
    }
    free(alpha); free(dalpha); free(g);
    return ORACLE_OK;
}

/*
 * Gradients of spatial cross-attention (oracle_sca) for d loss / d slots =
 * grad_slots.  The camera mean divides each seeing camera's contribution by
 * the hit count; a location is s = rho + (dx / W, dy / H), so an offset in
 * cells moves x and y one for one (d x / d dx = W * (1/W) = 1).  Offsets and
 * logits serve every camera, so their gradients sum over the cameras.
 *   grad_slots    [B][Nq][nH*Dh]
 *   grad_value    [B][Ncam][Nv][nH][Dh]   overwritten
 *   grad_offsets  [B][Nq][nH][L][P][2]    in cells; zero for queries no camera sees
 *   grad_logits   [B][Nq][nH][L*P]        likewise
 */
int oracle_sca_backward(const void* value, int value_bf16, const int64_t* spatial_shapes,
                        const int64_t* level_start_index, const float* reference_points_cam,
                        const uint8_t* bev_mask, const float* sampling_offsets, const float* attention_logits,
                        const float* grad_slots, int64_t B, int64_t Ncam, int64_t Nv, int64_t Nq, int nH, int Dh,
                        int L, int P, int D, double* grad_value, double* grad_offsets, double* grad_logits)
{
    if (!value || !spatial_shapes || !level_start_index || !reference_points_cam || !bev_mask ||
        !sampling_offsets || !attention_logits || !grad_slots || !grad_value || !grad_offsets || !grad_logits)
        return ORACLE_BAD_ARG;
    if (B < 1 || Ncam < 1 || Nv < 1 || Nq < 0 || nH < 1 || Dh < 1 || L < 1 || P < 1 || D < 1 || P % D != 0)
        return ORACLE_BAD_ARG;
    if (!levels_ok(spatial_shapes, level_start_index, L, Nv)) return ORACLE_BAD_ARG;
    const int LP = L * P;
    const int64_t C = (int64_t)nH * Dh;
    for (int64_t i = 0; i < B * Ncam * Nv * C; ++i) grad_value[i] = 0.0;
    double* alpha = (double*)malloc(sizeof(double) * (size_t)nH * LP);
    double* dalpha = (double*)malloc(sizeof(double) * (size_t)nH * LP);
    double* g = (double*)malloc(sizeof(double) * (size_t)Dh);
    if (!alpha || !dalpha || !g) { free(alpha); free(dalpha); free(g); return ORACLE_BAD_ARG; }
    const size_t elem = value_bf16 ? 2 : 4;
    for (int64_t bq = 0; bq < B * Nq; ++bq) {
        int64_t b = bq / Nq, q = bq % Nq;
        double* goff = grad_offsets + bq * nH * LP * 2;
        double* glog = grad_logits + bq * nH * LP;
        for (int64_t i = 0; i < (int64_t)nH * LP * 2; ++i) goff[i] = 0.0;
        for (int64_t i = 0; i < (int64_t)nH * LP; ++i) dalpha[i] = 0.0;
        /* the cameras that see the query (step 1 of the forward) */
        int hits = 0;
        for (int64_t c = 0; c < Ncam; ++c) {
            int any = 0;
            for (int m = 0; m < D; ++m) any |= bev_mask[((c * B + b) * Nq + q) * D + m] != 0;
            hits += any;
        }
        head_weights(attention_logits + bq * nH * LP, nH, LP, 1, alpha);
        double n = hits > 1 ? (double)hits : 1.0;
        for (int64_t c = 0; c < Ncam && hits > 0; ++c) {
            int any = 0;
            for (int m = 0; m < D; ++m) any |= bev_mask[((c * B + b) * Nq + q) * D + m] != 0;
            if (!any) continue;
            ValueImage img = {(const char*)value + (size_t)((b * Ncam + c) * Nv * C) * elem, value_bf16, nH, Dh};
            double* grad_img = grad_value + (b * Ncam + c) * Nv * C;
            const float* rho = reference_points_cam + ((c * B + b) * Nq + q) * D * 2;
            for (int h = 0; h < nH; ++h) {
                /* d slots / d (camera c's sum) = 1 / n */
                for (int d = 0; d < Dh; ++d) g[d] = (double)grad_slots[bq * C + (int64_t)h * Dh + d] / n;
                for (int l = 0; l < L; ++l) {
                    int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1];
                    for (int k = 0; k < P; ++k) {
                        int m = k % D;
                        int64_t at = ((int64_t)h * L + l) * P + k;
                        const float* off = sampling_offsets + (bq * nH * LP + at) * 2;
                        double sx = (double)rho[m * 2 + 0] + (double)off[0] / (double)W;
                        double sy = (double)rho[m * 2 + 1] + (double)off[1] / (double)H;
                        double a = alpha[(int64_t)h * LP + l * P + k];
                        double ds, dx, dy;
                        bilinear_backward(&img, grad_img, H, W, level_start_index[l], h, sx, sy, a, g, &ds, &dx,
                                          &dy);
                        dalpha[(int64_t)h * LP + l * P + k] += ds;
                        goff[at * 2 + 0] += a * dx;
                        goff[at * 2 + 1] += a * dy;
                    }
                }
            }
        }
        weights_backward(alpha, dalpha, nH, LP, 1, glog);
    }
    free(alpha); free(dalpha); free(g);
    return ORACLE_OK;
}
