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
