/*
 * qmv_oracle.c -- plain, slow, obviously-correct CPU reference ("the oracle")
 * for the quantized matrix-vector path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; the two meet only through the seeded input generators.
 *
 * Every function below follows a definition stated on the source pages:
 *
 *   [T]  "Gemma 3 1B at 114 tokens per second on a laptop CPU"
 *        (sections "Step 1: a kernel for 1.6-bit weights",
 *         "Step 2: making a ternary Gemma",
 *         "Step 3: the output layer became the bottleneck",
 *         "Many users at once")
 *   [C]  cpp20gemma README (section "Architecture & implementation")
 *   [L]  "llama2.c -- Llama-2 Inference in One C File"
 *        (sections "matmul -- the one function that eats all the FLOPs",
 *         "Sampling -- turning logits into a token", "Key ideas & tradeoffs")
 *   [G]  the gemma.cpp tour (section "Weights, Blobs, and the .sbs Format")
 *
 * Arithmetic rules: fp32 where the pages fix fp32 (the quantisation scale and
 * the quantised value), otherwise exact integers (int64) or fp64.  Build with
 * -O2 -ffp-contract=off and never with -ffast-math.
 *
 * Parity status: every function here is pinned by the CPU tests (closed forms,
 * exhaustive enumeration, brute force on tiny inputs, planted answers).
 */
#include <assert.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* O1 -- symmetric absmax int8 quantisation.                                */
/*                                                                          */
/* [C] "Architecture & implementation": scale = max(|w|, 1e-9)/127 and      */
/* w8 = clip(round(w/scale), -128, 127), the scale multiplied in once after */
/* the dot product.  [T] "Step 2": the inputs of each layer are rounded to  */
/* int8.  [L] "Key ideas & tradeoffs": activations quantised dynamically at */
/* run time.  Readings (the pages are silent): the scale is computed in     */
/* fp32 with one correctly rounded division; w/scale is one IEEE fp32       */
/* division; round() is round-half-to-even (the IEEE default, which is what */
/* a NumPy conversion script gets from np.round / np.rint).                 */
/* ------------------------------------------------------------------------ */

/* The scale of one group of `count` values. */
static float oracle_scale_of(const float* v, int64_t count)
{
    float m = 0.0f;
    for (int64_t i = 0; i < count; ++i) {
        assert(isfinite(v[i]));
        float a = fabsf(v[i]);
        if (a > m) m = a;
    }
    if (m < 1e-9f) m = 1e-9f;
    return m / 127.0f;
}

/* One value: IEEE division, round half to even, clip to int8. */
static int8_t oracle_quantize_one(float v, float s)
{
    float q = v / s;
    float r = nearbyintf(q);          /* default rounding mode: half to even */
    if (r > 127.0f) r = 127.0f;
    if (r < -128.0f) r = -128.0f;
    return (int8_t)r;
}

/* Per-row (per-token) quantisation: x is [m][k]; q is [m][k]; s is [m]. */
void oracle_quantize_rows(const float* x, int64_t m, int64_t k, int8_t* q, float* s)
{
    for (int64_t r = 0; r < m; ++r) {
        const float* row = x + r * k;
        float sr = oracle_scale_of(row, k);
        s[r] = sr;
        for (int64_t c = 0; c < k; ++c) q[r * k + c] = oracle_quantize_one(row[c], sr);
    }
}

/* Per-tensor quantisation: one scale for the whole [n][k] matrix. */
void oracle_quantize_tensor(const float* w, int64_t n, int64_t k, int8_t* q, float* s)
{
    float st = oracle_scale_of(w, n * k);
    *s = st;
    for (int64_t i = 0; i < n * k; ++i) q[i] = oracle_quantize_one(w[i], st);
}

/* ------------------------------------------------------------------------ */
/* Device byte layout shared by both weight types (a layout of this library,*/
/* not of the pages).  A row's bytes are cut into 16-byte chunks; chunk c of*/
/* every row is stored before chunk c+1 of any row:                         */
/*     offset(row r, byte j) = ((j / 16) * n + r) * 16 + (j % 16)           */
/* Row byte counts are padded up to a multiple of 16.                       */
/* ------------------------------------------------------------------------ */

static int64_t oracle_offset(int64_t n, int64_t r, int64_t j)
{
    return ((j / 16) * n + r) * 16 + (j % 16);
}

/* Row bytes before padding and after padding, per weight type. */
int64_t oracle_trit5_row_bytes(int64_t k) { return (k + 4) / 5; }
int64_t oracle_trit5_row_stride(int64_t k) { return ((oracle_trit5_row_bytes(k) + 15) / 16) * 16; }
int64_t oracle_int8_row_stride(int64_t k) { return ((k + 15) / 16) * 16; }

/* ------------------------------------------------------------------------ */
/* O2 -- five trits per byte.                                               */
/*                                                                          */
/* [T] "Step 1": five ternary weights go in one byte because 3^5 = 243 fits */
/* in 256 values.  Reading: the byte is the base-3 number whose digit i     */
/* (weight 3^i) is t+1 for the trit of column 5j+i (the lowest column is    */
/* the least significant digit), so the byte runs over 0..242.  Columns at  */
/* or beyond k count as trit 0 (digit 1), so whole padding bytes hold 121.  */
/* A value outside {-1,0,1} is counted in *bad and packed as 0.             */
/* ------------------------------------------------------------------------ */

void oracle_pack_trit5(const int8_t* t, int64_t n, int64_t k, uint8_t* out, int64_t* bad)
{
    int64_t stride = oracle_trit5_row_stride(k);
    int64_t nbad = 0;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < stride; ++j) {
            int value = 0;
            int place = 1;
            for (int i = 0; i < 5; ++i) {
                int64_t col = 5 * j + i;
                int trit = 0;
                if (col < k) {
                    trit = t[r * k + col];
                    if (trit < -1 || trit > 1) { ++nbad; trit = 0; }
                }
                value += (trit + 1) * place;
                place *= 3;
            }
            out[oracle_offset(n, r, j)] = (uint8_t)value;
        }
    }
    if (bad) *bad = nbad;
}

/* Inverse of the above for columns < k.  Returns the number of bytes that
 * are not valid base-3 codes (>= 243); their trits are reported as 0. */
int64_t oracle_unpack_trit5(const uint8_t* in, int64_t n, int64_t k, int8_t* t)
{
    int64_t invalid = 0;
    int64_t nbytes = oracle_trit5_row_bytes(k);
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < nbytes; ++j) {
            int value = in[oracle_offset(n, r, j)];
            int ok = value < 243;
            if (!ok) ++invalid;
            for (int i = 0; i < 5; ++i) {
                int digit = value % 3;
                value /= 3;
                int64_t col = 5 * j + i;
                if (col < k) t[r * k + col] = (int8_t)(ok ? digit - 1 : 0);
            }
        }
    }
    return invalid;
}

/* ------------------------------------------------------------------------ */
/* O3 -- int8 weights with one scale per tensor, in the device layout.      */
/* [C] "Architecture & implementation": per-tensor symmetric scale, weights */
/* stored row-major [out][in].  Bytes past column k are 0.                  */
/* ------------------------------------------------------------------------ */

void oracle_layout_int8(const int8_t* q, int64_t n, int64_t k, int8_t* out)
{
    int64_t stride = oracle_int8_row_stride(k);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < stride; ++j)
            out[oracle_offset(n, r, j)] = (j < k) ? q[r * k + j] : 0;
}

/* ------------------------------------------------------------------------ */
/* O4 -- the exact integer core.                                            */
/*                                                                          */
/* [L] "matmul": out[i] = sum_j W[i][j] * x[j] over output rows i, with an  */
/* OpenMP split over rows.  [T] "Step 1": the dot product is exact integer  */
/* arithmetic on int8 inputs and weights, so its result does not depend on  */
/* thread count or batch size.  acc[mi][r] = sum_c x8[mi][c] * w[r][c],     */
/* summed in int64 and checked to fit int32.  w is [n][k] int8: trits in    */
/* {-1,0,1} for ternary weights, int8 codes for int8 weights.               */
/* ------------------------------------------------------------------------ */

int oracle_matmul_int(const int8_t* x8, const int8_t* w, int64_t m, int64_t n, int64_t k,
                      int32_t* acc, int threads)
{
    int overflow = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1) reduction(|:overflow)
#endif
    for (int64_t r = 0; r < n; ++r) {
        const int8_t* wr = w + r * k;
        for (int64_t mi = 0; mi < m; ++mi) {
            const int8_t* xr = x8 + mi * k;
            int64_t sum = 0;
            for (int64_t c = 0; c < k; ++c) sum += (int64_t)xr[c] * (int64_t)wr[c];
            if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
            acc[mi * n + r] = (int32_t)sum;
        }
    }
    (void)threads;
    return overflow;
}

/* ------------------------------------------------------------------------ */
/* O5 -- dequantisation after the dot product.                              */
/* [C] "Architecture & implementation": (x . w8) * scale, the scale applied */
/* once after the dot.  With a per-token activation scale sx[mi] and a      */
/* per-matrix weight scale sw, y = acc * sx * sw, formed in fp64 and        */
/* rounded once to fp32.                                                    */
/* ------------------------------------------------------------------------ */

void oracle_dequant(const int32_t* acc, int64_t m, int64_t n, const float* sx, float sw, float* y)
{
    for (int64_t mi = 0; mi < m; ++mi)
        for (int64_t r = 0; r < n; ++r)
            y[mi * n + r] = (float)((double)acc[mi * n + r] * (double)sx[mi] * (double)sw);
}

/* ------------------------------------------------------------------------ */
/* O6 -- output layer with greedy choice.                                   */
/*                                                                          */
/* [T] "Step 3": the output layer scores every vocabulary row against the   */
/* final hidden state; the next word is the best-scoring one.  [L]          */
/* "Sampling": greedy argmax keeps the first maximum (strict >).  Reading:  */
/* weights are bf16 (widened exactly to fp32), x stays fp32; each logit is  */
/* summed in fp64 from exact products; the choice is the first index whose  */
/* logit, rounded to fp32, is largest.                                      */
/* ------------------------------------------------------------------------ */

static double oracle_bf16_to_double(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

void oracle_lmhead(const uint16_t* w, const float* x, int64_t v, int64_t k, double* logits,
                   int32_t* idx, int threads)
{
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
#endif
    for (int64_t r = 0; r < v; ++r) {
        double sum = 0.0;
        for (int64_t c = 0; c < k; ++c) sum += oracle_bf16_to_double(w[r * k + c]) * (double)x[c];
        logits[r] = sum;
    }
    (void)threads;
    int64_t best = 0;
    for (int64_t r = 1; r < v; ++r)
        if ((float)logits[r] > (float)logits[best]) best = r;
    *idx = (int32_t)best;
}

/* ------------------------------------------------------------------------ */
/* O7 -- the sketch head: candidates first, exact scores for those only.    */
/*                                                                          */
/* [T] "Step 3", the sketch head, in the page's three steps:                */
/*  1. the 32 hidden dimensions with the largest values are scored exactly  */
/*     for every word;                                                      */
/*  2. the other dimensions are scored with a 1-bit (sign) copy of the      */
/*     table, the dimensions grouped by size and each group weighted;       */
/*  3. about 1,000 words with the best approximate scores are rescored      */
/*     exactly; every other word scores minus infinity.                     */
/* Readings (the page gives no more detail):                                */
/*  - "largest values" is largest |x|; ranks are by |x| descending, ties to */
/*    the lower dimension; T = min(32, k) dimensions are exact.             */
/*  - a sign bit is 1 for a value below zero (so 0 and -0 count as          */
/*    positive); a dimension adds +1 where the signs of w and x agree and   */
/*    -1 where they differ.                                                 */
/*  - "grouped by size": the remaining k - T dimensions in rank order are   */
/*    cut into 4 consecutive groups, floor((k - T) / 4) each, the last      */
/*    taking the rest.  Group weight = c * mean |x| of the group, with c    */
/*    the mean |w| of the whole table, so a group's sign agreement is       */
/*    turned into the size of the products it stands for.                   */
/*  - every quantity above is the plain definition, summed in fp64: c, the  */
/*    group means, and the score                                            */
/*        s = sum_(exact j) w_j x_j + sum_g weight_g * agreement_g.         */
/*  - "about 1,000 words": the N = min(1024, v) best approximate scores,    */
/*    ties to the lower word index.                                         */
/*  - the exact scores are O6's logits; the pick is O6's first maximum,     */
/*    over the candidates only.                                             */
/* ------------------------------------------------------------------------ */

#define ORACLE_SKETCH_TOP 32
#define ORACLE_SKETCH_GROUPS 4
#define ORACLE_SKETCH_CAND 1024

/* Sign bits of the table, word-major: bit (c % 32) of word (c / 32) * v + r */
/* is 1 when w[r][c] < 0; bits past k are 0.                                 */
void oracle_sketch_signs(const uint16_t* w, int64_t v, int64_t k, uint32_t* out, int threads)
{
    int64_t words = (k + 31) / 32;
    memset(out, 0, (size_t)(words * v) * sizeof(uint32_t));
    (void)threads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
#endif
    for (int64_t r = 0; r < v; ++r)
        for (int64_t c = 0; c < k; ++c)
            if (oracle_bf16_to_double(w[r * k + c]) < 0.0) out[(c / 32) * v + r] |= 1u << (c % 32);
}

/* c = mean |w| of the table: every |w| summed in fp64, divided by v * k. */
double oracle_sketch_scale(const uint16_t* w, int64_t v, int64_t k, int threads)
{
    double total = 0.0;
    (void)threads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1) reduction(+:total)
#endif
    for (int64_t r = 0; r < v; ++r)
        for (int64_t c = 0; c < k; ++c) total += fabs(oracle_bf16_to_double(w[r * k + c]));
    return total / ((double)v * (double)k);
}

/* The per-token plan: the exact dimensions in rank order (top_idx, *ntop), */
/* the group of every dimension (-1 for an exact one), the group sizes and  */
/* weights c * mean |x| (fp64).                                             */
void oracle_sketch_plan(const float* x, int64_t k, double c, int32_t* top_idx, int32_t* ntop, int32_t* group_of,
                        int32_t* group_n, double* group_w)
{
    /* rank by |x| descending, lower index first on ties: selection by repeated scans */
    int64_t* order = (int64_t*)malloc((size_t)k * sizeof(int64_t));
    uint8_t* used = (uint8_t*)calloc((size_t)k, 1);
    assert(order && used);
    for (int64_t r = 0; r < k; ++r) {
        int64_t best = -1;
        for (int64_t i = 0; i < k; ++i) {
            if (used[i]) continue;
            assert(isfinite(x[i]));
            if (best < 0 || fabsf(x[i]) > fabsf(x[best])) best = i;
        }
        used[best] = 1;
        order[r] = best;
    }
    int64_t t = k < ORACLE_SKETCH_TOP ? k : ORACLE_SKETCH_TOP;
    *ntop = (int32_t)t;
    for (int64_t j = 0; j < t; ++j) {
        top_idx[j] = (int32_t)order[j];
        group_of[order[j]] = -1;
    }
    int64_t rest = k - t, base = rest / ORACLE_SKETCH_GROUPS;
    for (int g = 0; g < ORACLE_SKETCH_GROUPS; ++g) {
        int64_t lo = t + g * base;
        int64_t hi = g == ORACLE_SKETCH_GROUPS - 1 ? k : lo + base;
        group_n[g] = (int32_t)(hi - lo);
        double sum = 0.0;
        for (int64_t r = lo; r < hi; ++r) {
            group_of[order[r]] = g;
            sum += fabs((double)x[order[r]]);
        }
        group_w[g] = hi > lo ? c * (sum / (double)(hi - lo)) : 0.0;
    }
    free(order);
    free(used);
}

/* Approximate scores (steps 1 and 2) in fp64, and for each word the sum of */
/* the magnitudes of its terms, sum_j |w_j x_j| + sum_g weight_g |agreement_g| */
/* (the scale any fp32 evaluation error of the score is proportional to).   */
void oracle_sketch_scores(const uint16_t* w, const float* x, int64_t v, int64_t k, double c, double* scores,
                          double* magnitude, int threads)
{
    int32_t top_idx[ORACLE_SKETCH_TOP], ntop, group_n[ORACLE_SKETCH_GROUPS];
    double group_w[ORACLE_SKETCH_GROUPS];
    int32_t* group_of = (int32_t*)malloc((size_t)k * sizeof(int32_t));
    assert(group_of);
    oracle_sketch_plan(x, k, c, top_idx, &ntop, group_of, group_n, group_w);
    (void)threads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
#endif
    for (int64_t r = 0; r < v; ++r) {
        double s = 0.0, mag = 0.0;
        for (int j = 0; j < ntop; ++j) {
            double p = oracle_bf16_to_double(w[r * k + top_idx[j]]) * (double)x[top_idx[j]];
            s += p;
            mag += fabs(p);
        }
        int64_t agree[ORACLE_SKETCH_GROUPS] = {0, 0, 0, 0};
        for (int64_t col = 0; col < k; ++col) {
            int g = group_of[col];
            if (g < 0) continue;
            int sw = oracle_bf16_to_double(w[r * k + col]) < 0.0, sx = x[col] < 0.0f;
            agree[g] += sw == sx ? 1 : -1;
        }
        for (int g = 0; g < ORACLE_SKETCH_GROUPS; ++g) {
            s += group_w[g] * (double)agree[g];
            mag += group_w[g] * fabs((double)agree[g]);
        }
        scores[r] = s;
        if (magnitude) magnitude[r] = mag;
    }
    free(group_of);
}

/* Step 3: the candidates (is_cand[r] = 1: the N best scores, ties to the   */
/* lower index, found by N scans for the best word not yet taken), the      */
/* exact logits of the candidates (logits[r], fp64; 0 elsewhere) and the    */
/* pick.  Returns the number of candidates.                                 */
int64_t oracle_sketch_pick(const uint16_t* w, const float* x, int64_t v, int64_t k, const double* scores,
                           uint8_t* is_cand, double* logits, int32_t* idx)
{
    int64_t need = v < ORACLE_SKETCH_CAND ? v : ORACLE_SKETCH_CAND;
    memset(is_cand, 0, (size_t)v);
    for (int64_t n = 0; n < need; ++n) {
        int64_t best = -1;
        for (int64_t r = 0; r < v; ++r)
            if (!is_cand[r] && (best < 0 || scores[r] > scores[best])) best = r;
        is_cand[best] = 1;
    }
    int64_t best = -1;
    for (int64_t r = 0; r < v; ++r) {
        logits[r] = 0.0;
        if (!is_cand[r]) continue;
        double sum = 0.0;
        for (int64_t col = 0; col < k; ++col) sum += oracle_bf16_to_double(w[r * k + col]) * (double)x[col];
        logits[r] = sum;
        if (best < 0 || (float)sum > (float)logits[best]) best = r;
    }
    *idx = (int32_t)best;
    return need;
}

/* ------------------------------------------------------------------------ */
/* O8 -- the steps either side of a GEMV: RMSNorm, gated activation.        */
/*                                                                          */
/* [L] "Step 1" and "Step 6": RMSNorm divides each value by the root mean   */
/* square of the row (plus eps under the root) and multiplies by a          */
/* per-dimension weight: o = weight * x / sqrt(sum(x^2) / k + eps).         */
/* [L] "Step 5": the gated feed-forward multiplies act(gate) by up, act =   */
/* SiLU(v) = v / (1 + exp(-v)); cpp20gemma and gemma.cpp use a GeLU gate   */
/* instead (GeGLU).  [T] "Step 2": the result is then rounded to int8 per  */
/* token (O1).                                                              */
/* Readings: both are evaluated here in fp64 straight from the definition   */
/* (the pages fix no precision for them); GeLU is the tanh form Gemma uses: */
/* 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).  The GPU evaluates them */
/* in fp32, so its int8 codes are checked as valid roundings of these       */
/* values (see the tests).                                                  */
/* ------------------------------------------------------------------------ */

void oracle_rmsnorm(const float* x, const float* weight, int64_t m, int64_t k, double eps, double* o)
{
    for (int64_t mi = 0; mi < m; ++mi) {
        const float* xr = x + mi * k;
        double ss = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            assert(isfinite(xr[j]));
            ss += (double)xr[j] * (double)xr[j];
        }
        double rms = sqrt(ss / (double)k + eps);
        for (int64_t j = 0; j < k; ++j) o[mi * k + j] = (double)weight[j] * (double)xr[j] / rms;
    }
}

/* act: 1 = GeLU (tanh form), 2 = SiLU.  h = act(gate) * up in fp64. */
void oracle_glu(const float* gate, const float* up, int64_t m, int64_t n, int act, double* h)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    for (int64_t i = 0; i < m * n; ++i) {
        double g = gate[i];
        double a = act == 1 ? 0.5 * g * (1.0 + tanh(c * (g + 0.044715 * g * g * g))) : g / (1.0 + exp(-g));
        h[i] = a * (double)up[i];
    }
}

/* ------------------------------------------------------------------------ */
/* O9 -- group-wise scales.                                                 */
/*                                                                          */
/* [G] "Weights, Blobs, and the .sbs Format": int8 weights stored in groups */
/* of 128 values that share one scale.  [T] "A side finding: Gemma 4 E4B in */
/* 4-bit": one activation scale per 32 values instead of one per token.     */
/* Readings: a group is that many consecutive columns of one row (the last  */
/* group of a row may be shorter; groups never span rows); each group is    */
/* quantised by O1's rule (absmax scale with the 1e-9 floor, one fp32       */
/* division, half-to-even, clip).  Activation group h (columns 32h..32h+31) */
/* lies inside weight group h/4, so each activation group's dot product is  */
/* exact in integers and its two scales are applied after that exact sum:   */
/*     y[m][n] = sum_h  sw[n][h/4] * sx[m][h] * D_h,                        */
/*     D_h = sum over the group's columns of x8 * w8,                       */
/* summed in fp64 (`bound` gets sum_h |term|, the scale of fp32 summation   */
/* error).                                                                  */
/* ------------------------------------------------------------------------ */

/* Quantise every row of x [m][k] in groups of `group` columns: q [m][k],
 * s [m][ceil(k/group)]. */
void oracle_quantize_groups(const float* x, int64_t m, int64_t k, int64_t group, int8_t* q, float* s)
{
    const int64_t ng = (k + group - 1) / group;
    for (int64_t r = 0; r < m; ++r)
        for (int64_t g = 0; g < ng; ++g) {
            const int64_t c0 = g * group, c1 = c0 + group < k ? c0 + group : k;
            const float sg = oracle_scale_of(x + r * k + c0, c1 - c0);
            s[r * ng + g] = sg;
            for (int64_t c = c0; c < c1; ++c) q[r * k + c] = oracle_quantize_one(x[r * k + c], sg);
        }
}

/* y and bound are [m][n] fp64; w8 [n][k] with sw [n][ceil(k/128)]; x8 [m][k]
 * with sx [m][ceil(k/32)]. */
void oracle_gemv_grouped(const int8_t* w8, const float* sw, const int8_t* x8, const float* sx, int64_t m,
                         int64_t n, int64_t k, double* y, double* bound, int threads)
{
    const int64_t gw = (k + 127) / 128, gx = (k + 31) / 32;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
#endif
    for (int64_t r = 0; r < n; ++r)
        for (int64_t mi = 0; mi < m; ++mi) {
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t h = 0; h < gx; ++h) {
                int64_t d = 0;
                const int64_t c1 = 32 * h + 32 < k ? 32 * h + 32 : k;
                for (int64_t c = 32 * h; c < c1; ++c) d += (int64_t)x8[mi * k + c] * (int64_t)w8[r * k + c];
                const double t = (double)sw[r * gw + h / 4] * (double)sx[mi * gx + h] * (double)d;
                sum += t;
                abs_sum += fabs(t);
            }
            y[mi * n + r] = sum;
            bound[mi * n + r] = abs_sum;
        }
    (void)threads;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
