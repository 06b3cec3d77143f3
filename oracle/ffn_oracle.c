/*
 * ffn_oracle.c -- CPU oracle for the NVFP4 W4A16 gated FFN.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition of what the GPU library computes; only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load it. It shares no code, header,
 * table or constant with the GPU library.
 *
 * Everything is computed in double precision, element by element, with sums
 * taken in ascending index order. OpenMP, when enabled, only spreads
 * independent output elements over threads: each element is still one
 * sequential sum, so results do not depend on the thread count.
 *
 * Sources (web pages of the Atlas inference engine API docs):
 *  - dense_ffn.rs page, module doc comment: the gated FFN dataflow
 *    gate = gate_proj(x), up = up_proj(x), out = down_proj(act(gate) * up).
 *  - dense_ffn.rs page, FfnActivation enum: SiLU (Qwen/Llama) or GELU (Gemma).
 *  - dense_ffn.rs page, DenseFfnLayer::ensure_int8_weight doc comment: an NVFP4
 *    weight is packed E2M1 codes [N, K/2], one E4M3 scale per 16 elements
 *    [N, K/16], and one per-tensor F32 weight_scale_2.
 *  - dense_ffn.rs page, DenseFfnLayer::forward_prefill_inner, FP4-MMQ branch:
 *    weight_scale_2 multiplies each projection's output and, for gate and up,
 *    is applied before the nonlinearity.
 *  - qwen35_dense.rs page, load of the SSM FP8 prefill copies: E4M3 magnitudes
 *    are bounded by 448, i.e. the OCP "E4M3FN" variant (no infinities).
 *  - The E2M1 and E4M3 bit layouts follow the OCP Microscaling Formats (MX)
 *    v1.0 specification.
 *  - qwen35_dense.rs page, weight loader: a dense BF16 weight is turned into
 *    NVFP4 on the GPU by a global-absmax pass followed by a quantise pass
 *    (the quantiser below; its scale rule is a reading, the pages give none).
 *  - dense_ffn.rs page, the W4A4 native-FP4 prefill (w4a4_gemm and
 *    quantize_nvfp4 handles, and the NVFP4 W4A4 MMQ arm of forward_prefill):
 *    NVFP4 weights against activations quantised to 4 bits on every call,
 *    gate and up only, the down projection kept on the W4A16 path, scale2
 *    applied to the products (the W4A4 functions below; the scale format is
 *    a reading for gfx950, see there).
 *  - qwen35_dense.rs page, proj_is_fp8_any_scale doc comment: a native FP8
 *    weight [N, K] is E4M3 bytes with an FP32 block-scale grid
 *    [ceil(N/128), ceil(K/128)] that the kernels index as
 *    block_scale[n/128, k/128] (the FP8 functions below).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): the even column of a byte is its low nibble; GELU is the tanh form;
 * there is no clamp on the SwiGLU product; scale bytes may be negative and
 * NaN scale bytes propagate as NaN.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ACT_SILU 0
#define ORACLE_ACT_GELU_TANH 1

/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 encodes the subnormal m * 0.5; otherwise the value is
 * 2^(e-1) * (1 + m/2). */
double oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
 * Exponent field 0 is subnormal: (m/8) * 2^-6. The all-ones magnitude
 * S.1111.111 is NaN; there are no infinities, so 1111.110 = 448 is the max. */
double oracle_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1;
    int e = (byte >> 3) & 15;
    int m = byte & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp(m / 8.0, -6);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* bf16 is the upper half of an IEEE fp32; widening to double is exact. */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The bf16 nearest to v (ties to even), as its bit pattern: bf16 keeps 8
 * significant bits of an fp32, so v is rounded once, directly from double,
 * at the bf16 spacing of its binade (2^-133 below the smallest normal);
 * magnitudes that round past the largest finite bf16 give infinity. */
uint16_t oracle_bf16_round_bits(double v)
{
    const double mag = fabs(v);
    double r;
    if (mag == 0.0) {
        r = 0.0;
    } else {
        int e;
        frexp(mag, &e); /* mag in [2^(e-1), 2^e) */
        int q = e - 8;  /* spacing of 8 significant bits */
        if (q < -133)
            q = -133;
        const double scaled = ldexp(mag, -q);
        double n = floor(scaled);
        const double frac = scaled - n;
        if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0))
            n += 1.0;
        r = ldexp(n, q);
    }
    const float f = (float)r; /* exact: at most 8 significant bits, or infinity */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (v < 0.0 || (v == 0.0 && signbit(v)))
        u |= 0x80000000u;
    return (uint16_t)(u >> 16);
}

/* SiLU(g) = g * sigmoid(g) = g / (1 + e^-g). */
double oracle_silu(double g)
{
    return g / (1.0 + exp(-g));
}

/* GELU, tanh form: 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))). */
double oracle_gelu_tanh(double g)
{
    const double k = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * g * (1.0 + tanh(k * (g + 0.044715 * g * g * g)));
}

double oracle_act(int act, double g)
{
    return act == ORACLE_ACT_GELU_TANH ? oracle_gelu_tanh(g) : oracle_silu(g);
}

/* Lookup tables built from the two definitions above. */
static void build_tables(double e2m1[16], double e4m3[256])
{
    for (int i = 0; i < 16; ++i)
        e2m1[i] = oracle_e2m1_value(i);
    for (int i = 0; i < 256; ++i)
        e4m3[i] = oracle_e4m3_value(i);
}

/* Element (r, c) of a dequantised NVFP4 weight of logical shape [rows, cols]:
 * code(r, c) * scale(r, c/16) * scale2. Codes are packed two per byte along a
 * row, column 2j in the low nibble of byte j and column 2j+1 in the high one. */
static double weight_at(const double e2m1[16], const double e4m3[256],
                        const uint8_t *codes, const uint8_t *scales, double scale2,
                        int cols, int r, int c)
{
    uint8_t byte = codes[(size_t)r * (size_t)(cols / 2) + (size_t)(c / 2)];
    int code = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    uint8_t sb = scales[(size_t)r * (size_t)(cols / 16) + (size_t)(c / 16)];
    return e2m1[code] * e4m3[sb] * scale2;
}

void oracle_dequant(const uint8_t *codes, const uint8_t *scales, float scale2,
                    int rows, int cols, double *w_out)
{
    double e2m1[16], e4m3[256];
    build_tables(e2m1, e4m3);
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            w_out[(size_t)r * cols + c] = weight_at(e2m1, e4m3, codes, scales, scale2, cols, r, c);
}

/* y[m, r] = sum_c W[r, c] * a[m, c] over a [rows, cols] NVFP4 weight and a
 * double-precision input a[M, cols]; y is [M, rows]. */
void oracle_linear_f64(const double *a, int M, int cols, int rows,
                       const uint8_t *codes, const uint8_t *scales, float scale2,
                       double *y)
{
    double e2m1[16], e4m3[256];
    build_tables(e2m1, e4m3);
    long total = (long)M * rows;
#pragma omp parallel for schedule(static)
    for (long idx = 0; idx < total; ++idx) {
        int m = (int)(idx / rows);
        int r = (int)(idx % rows);
        double acc = 0.0;
        for (int c = 0; c < cols; ++c)
            acc += weight_at(e2m1, e4m3, codes, scales, scale2, cols, r, c) * a[(size_t)m * cols + c];
        y[idx] = acc;
    }
}

/* gate = W_g x and up = W_u x for bf16 x[M, K]; W_g, W_u are [N, K];
 * gate and up are [M, N]. Returns 0, or -1 if memory runs out. */
int oracle_dual(const uint16_t *x_bits, int M, int K, int N,
                const uint8_t *g_codes, const uint8_t *g_scales, float g_scale2,
                const uint8_t *u_codes, const uint8_t *u_scales, float u_scale2,
                double *gate, double *up)
{
    double *x = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    if (!x)
        return -1;
    for (size_t i = 0; i < (size_t)M * (size_t)K; ++i)
        x[i] = oracle_bf16_value(x_bits[i]);
    oracle_linear_f64(x, M, K, N, g_codes, g_scales, g_scale2, gate);
    oracle_linear_f64(x, M, K, N, u_codes, u_scales, u_scale2, up);
    free(x);
    return 0;
}

/* h[m, n] = act(gate[m, n]) * up[m, n]. */
void oracle_gated_act(int act, const double *gate, const double *up, size_t count, double *h)
{
    for (size_t i = 0; i < count; ++i)
        h[i] = oracle_act(act, gate[i]) * up[i];
}

/* out[m, j] = sum_n W_d[j, n] * h[m, n] with W_d of shape [K, N]. */
void oracle_down(const double *h, int M, int N, int K,
                 const uint8_t *d_codes, const uint8_t *d_scales, float d_scale2,
                 double *out)
{
    oracle_linear_f64(h, M, N, K, d_codes, d_scales, d_scale2, out);
}

/* The whole gated FFN: out = W_d (act(W_g x) * (W_u x)), all in double.
 * out is [M, K]. Returns 0, or -1 if memory runs out. */
int oracle_ffn(const uint16_t *x_bits, int M, int K, int N, int act,
               const uint8_t *g_codes, const uint8_t *g_scales, float g_scale2,
               const uint8_t *u_codes, const uint8_t *u_scales, float u_scale2,
               const uint8_t *d_codes, const uint8_t *d_scales, float d_scale2,
               double *out)
{
    size_t mn = (size_t)M * (size_t)N;
    double *gate = (double *)malloc(sizeof(double) * mn);
    double *up = (double *)malloc(sizeof(double) * mn);
    int rc = -1;
    if (gate && up &&
        oracle_dual(x_bits, M, K, N, g_codes, g_scales, g_scale2,
                    u_codes, u_scales, u_scale2, gate, up) == 0) {
        oracle_gated_act(act, gate, up, mn, gate); /* h overwrites gate */
        oracle_down(gate, M, N, K, d_codes, d_scales, d_scale2, out);
        rc = 0;
    }
    free(gate);
    free(up);
    return rc;
}

/* Number of threads an OpenMP region would use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    return 1;
#endif
}

/* Threads for later parallel regions (n >= 1); a no-op without OpenMP. The
 * sums are per output element, so results do not depend on n. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------ quantiser
 * BF16 -> NVFP4 (qwen35_dense.rs page, weight loader: a global absmax pass,
 * then a pass writing packed E2M1 codes [rows, cols/2], per-16 E4M3 scales
 * [rows, cols/16] and the per-tensor weight_scale_2). The pages give no scale
 * rule; the reading taken is the plainest one that fills both formats:
 *   scale2 = amax / (6 * 448)       (largest E2M1 value x largest E4M3 value),
 *   block scale byte = E4M3(bmax / (6 * scale2)), nearest, ties to even, at most 448,
 *   code = E2M1(w * (1 / (block scale * scale2))), nearest, ties to even, at most 6,
 *          with the sign of w (negative values that round to zero give -0),
 * with everything zero when amax = 0 and code 0 where block scale * scale2 is
 * zero. These steps decide integers, so they are taken in fp32 with the same
 * operations as the GPU: one correctly rounded division or multiplication
 * each, no fused multiply-add. Inputs must be finite.
 *
 * The two encoders are brute-force nearest-value searches over the decoders
 * above (no bit tricks), so they are correct by inspection. */

/* The E2M1 code nearest to q (ties to the code with mantissa bit 0),
 * saturating at 6; the sign bit is q's (so -0 and small negatives give code
 * 8, negative zero). */
int oracle_e2m1_encode(float q)
{
    const double a = fabs((double)q);
    int best = 0;
    double bd = INFINITY;
    if (a >= 6.0)  /* saturation (for huge a every distance would round alike) */
        return signbit(q) ? 15 : 7;
    for (int k = 0; k < 8; ++k) {
        const double d = fabs(a - oracle_e2m1_value(k));
        if (d < bd || (d == bd && (k & 1) == 0 && (best & 1) == 1)) {
            best = k;
            bd = d;
        }
    }
    return signbit(q) ? (best | 8) : best;
}

/* The E4M3FN byte nearest to s >= 0 (ties to the byte with mantissa bit 0),
 * saturating at 448 (byte 0x7E). */
int oracle_e4m3_encode(float s)
{
    const double a = (double)s;
    int best = 0;
    double bd = INFINITY;
    if (a >= 448.0)  /* saturation */
        return 0x7E;
    for (int b = 0; b < 127; ++b) {  /* 0x00 .. 0x7E: the non-negative finite values */
        const double d = fabs(a - oracle_e4m3_value(b));
        if (d < bd || (d == bd && (b & 1) == 0 && (best & 1) == 1)) {
            best = b;
            bd = d;
        }
    }
    return best;
}

static float bf16_to_float(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

void oracle_quantize(const uint16_t *w_bits, int rows, int cols, uint8_t *codes, uint8_t *scales,
                     float *scale2_out)
{
    const size_t n = (size_t)rows * (size_t)cols;
    float amax = 0.0f;
    for (size_t i = 0; i < n; ++i) {
        const float v = fabsf(bf16_to_float(w_bits[i]));
        if (v > amax)
            amax = v;
    }
    memset(codes, 0, n / 2);
    memset(scales, 0, n / 16);
    if (amax == 0.0f) {
        *scale2_out = 0.0f;
        return;
    }
    const float scale2 = amax / 2688.0f;  /* 6 * 448 */
    const float d = scale2 * 6.0f;
    const int nb = cols / 16;
    for (int r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t *blk = w_bits + (size_t)r * cols + (size_t)b * 16;
            float bmax = 0.0f;
            for (int j = 0; j < 16; ++j) {
                const float v = fabsf(bf16_to_float(blk[j]));
                if (v > bmax)
                    bmax = v;
            }
            const float sv = bmax / d;
            const int sb = oracle_e4m3_encode(sv);
            const float denom = (float)oracle_e4m3_value(sb) * scale2;
            const float inv = denom == 0.0f ? 0.0f : 1.0f / denom;
            scales[(size_t)r * nb + b] = (uint8_t)sb;
            for (int j = 0; j < 16; ++j) {
                const int c = b * 16 + j;
                const int code = denom == 0.0f ? 0 : oracle_e2m1_encode(bf16_to_float(blk[j]) * inv);
                uint8_t *byte = codes + (size_t)r * (cols / 2) + c / 2;
                *byte |= (uint8_t)((c % 2 == 0) ? code : (code << 4));
            }
        }
    }
    *scale2_out = scale2;
}

/* ------------------------------------------------------------------ FP8
 * An FP8 weight of logical shape [rows, cols]: E4M3FN bytes, row-major
 * [rows, cols], and an fp32 block-scale grid [ceil(rows/128), ceil(cols/128)],
 * row-major; element (r, c) = e4m3(w[r, c]) * block_scale[r/128, c/128]
 * (qwen35_dense.rs page, proj_is_fp8_any_scale doc comment). There is no
 * per-tensor multiplier. NaN bytes propagate. */
static double fp8_weight_at(const double e4m3[256], const uint8_t *w, const float *bs,
                            int cols, int r, int c)
{
    int bcols = (cols + 127) / 128;
    return e4m3[w[(size_t)r * (size_t)cols + (size_t)c]] * (double)bs[(size_t)(r / 128) * (size_t)bcols + (size_t)(c / 128)];
}

void oracle_fp8_dequant(const uint8_t *w, const float *bs, int rows, int cols, double *w_out)
{
    double e2m1[16], e4m3[256];
    build_tables(e2m1, e4m3);
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            w_out[(size_t)r * cols + c] = fp8_weight_at(e4m3, w, bs, cols, r, c);
}

/* y[m, r] = sum_c W[r, c] * a[m, c] over a [rows, cols] FP8 weight. */
void oracle_fp8_linear_f64(const double *a, int M, int cols, int rows,
                           const uint8_t *w, const float *bs, double *y)
{
    double e2m1[16], e4m3[256];
    build_tables(e2m1, e4m3);
    long total = (long)M * rows;
#pragma omp parallel for schedule(static)
    for (long idx = 0; idx < total; ++idx) {
        int m = (int)(idx / rows);
        int r = (int)(idx % rows);
        double acc = 0.0;
        for (int c = 0; c < cols; ++c)
            acc += fp8_weight_at(e4m3, w, bs, cols, r, c) * a[(size_t)m * cols + c];
        y[idx] = acc;
    }
}

/* gate = W_g x, up = W_u x with FP8 W_g, W_u [N, K] and bf16 x [M, K]. */
int oracle_fp8_dual(const uint16_t *x_bits, int M, int K, int N,
                    const uint8_t *gw, const float *gbs, const uint8_t *uw, const float *ubs,
                    double *gate, double *up)
{
    double *x = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    if (!x)
        return -1;
    for (size_t i = 0; i < (size_t)M * (size_t)K; ++i)
        x[i] = oracle_bf16_value(x_bits[i]);
    oracle_fp8_linear_f64(x, M, K, N, gw, gbs, gate);
    oracle_fp8_linear_f64(x, M, K, N, uw, ubs, up);
    free(x);
    return 0;
}

/* The whole gated FFN with FP8 weights (W_d of shape [K, N]), in double. */
int oracle_fp8_ffn(const uint16_t *x_bits, int M, int K, int N, int act,
                   const uint8_t *gw, const float *gbs, const uint8_t *uw, const float *ubs,
                   const uint8_t *dw, const float *dbs, double *out)
{
    size_t mn = (size_t)M * (size_t)N;
    double *gate = (double *)malloc(sizeof(double) * mn);
    double *up = (double *)malloc(sizeof(double) * mn);
    int rc = -1;
    if (gate && up && oracle_fp8_dual(x_bits, M, K, N, gw, gbs, uw, ubs, gate, up) == 0) {
        oracle_gated_act(act, gate, up, mn, gate); /* h overwrites gate */
        oracle_fp8_linear_f64(gate, M, N, K, dw, dbs, out);
        rc = 0;
    }
    free(gate);
    free(up);
    return rc;
}

/* ------------------------------------------------------------ W4A4 (MXFP4)
 * The matrix instructions of gfx950 that multiply 4-bit operands take one
 * power-of-two (E8M0) scale per 32 consecutive elements of a row, not an
 * E4M3 scale per 16, so the reading taken for the W4A4 arm is that both
 * operands are MXFP4 as the OCP MX v1.0 specification defines it:
 *   - per row and 32-element block, the shared exponent is
 *     se = floor(log2(amax)) - 2 (2 being the largest E2M1 exponent), clamped
 *     to [-127, 127], stored as the E8M0 byte se + 127; a block of zeros
 *     gets se = 0;
 *   - each element is E2M1(v / 2^se), nearest with ties to even, saturating
 *     at 6, keeping its sign (oracle_e2m1_encode); v / 2^se is taken in fp32,
 *     as the hardware conversion takes it (exact for the inputs here);
 *   - activations: v = the bf16 value, quantised on every call;
 *   - weights: requantised once from NVFP4, v = e2m1(code) * e4m3(scale)
 *     (exact); scale2 is not folded in: it multiplies the projection's sum;
 *   - products of two MXFP4 values are exact; sums are taken in double.
 * The hybrid FFN keeps the down projection on the W4A16 path (oracle_down);
 * the all-W4A4 FFN rounds h to bf16 and quantises it like the activations
 * (oracle_w4a4_down). Inputs and scales must be finite. */

double oracle_mx_value(int code, int e8m0)
{
    return oracle_e2m1_value(code & 15) * ldexp(1.0, e8m0 - 127);
}

int oracle_mx_block_exponent(double amax)
{
    int e;
    if (amax == 0.0)
        return 0;
    frexp(amax, &e);  /* amax = f 2^e with f in [0.5, 1): floor(log2(amax)) = e - 1 */
    int se = (e - 1) - 2;
    if (se < -127)
        se = -127;
    if (se > 127)
        se = 127;
    return se;
}

/* v [rows, cols] (cols a multiple of 32) -> codes [rows, cols/2] (element 2j
 * in the low nibble of byte j) and E8M0 bytes [rows, cols/32]. */
void oracle_mx_quantize(const double *v, int rows, int cols, uint8_t *codes, uint8_t *e8m0)
{
    const int nb = cols / 32;
    for (int r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const double *blk = v + (size_t)r * cols + (size_t)b * 32;
            double amax = 0.0;
            for (int j = 0; j < 32; ++j)
                if (fabs(blk[j]) > amax)
                    amax = fabs(blk[j]);
            const int se = oracle_mx_block_exponent(amax);
            e8m0[(size_t)r * nb + b] = (uint8_t)(se + 127);
            for (int j = 0; j < 32; ++j) {
                const float q = (float)(blk[j] / ldexp(1.0, se));
                const int code = oracle_e2m1_encode(q);
                const int c = b * 32 + j;
                uint8_t *byte = &codes[(size_t)r * (cols / 2) + (size_t)(c / 2)];
                if (c % 2 == 0)
                    *byte = (uint8_t)code;
                else
                    *byte = (uint8_t)(*byte | (code << 4));
            }
        }
    }
}

int oracle_mx_quantize_bf16(const uint16_t *x_bits, int M, int K, uint8_t *codes, uint8_t *e8m0)
{
    double *v = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    if (!v)
        return -1;
    for (size_t i = 0; i < (size_t)M * (size_t)K; ++i)
        v[i] = oracle_bf16_value(x_bits[i]);
    oracle_mx_quantize(v, M, K, codes, e8m0);
    free(v);
    return 0;
}

/* NVFP4 [rows, cols] (codes, scales; scale2 left out) -> MXFP4. */
int oracle_mx_requant_nvfp4(const uint8_t *codes, const uint8_t *scales, int rows, int cols, uint8_t *mx_codes,
                            uint8_t *mx_e8m0)
{
    double *v = (double *)malloc(sizeof(double) * (size_t)rows * (size_t)cols);
    if (!v)
        return -1;
    oracle_dequant(codes, scales, 1.0f, rows, cols, v);
    oracle_mx_quantize(v, rows, cols, mx_codes, mx_e8m0);
    free(v);
    return 0;
}

/* y[m, r] = sum_c mx(a)[m, c] * mx(w)[r, c]. */
void oracle_mx_linear_f64(const uint8_t *a_codes, const uint8_t *a_e8m0, int M, int cols, const uint8_t *w_codes,
                          const uint8_t *w_e8m0, int rows, double *y)
{
    long total = (long)M * rows;
#pragma omp parallel for schedule(static)
    for (long idx = 0; idx < total; ++idx) {
        const int m = (int)(idx / rows);
        const int r = (int)(idx % rows);
        double acc = 0.0;
        for (int c = 0; c < cols; ++c) {
            const uint8_t ab = a_codes[(size_t)m * (cols / 2) + (size_t)(c / 2)];
            const uint8_t wb = w_codes[(size_t)r * (cols / 2) + (size_t)(c / 2)];
            const int ac = (c % 2 == 0) ? (ab & 0x0F) : (ab >> 4);
            const int wc = (c % 2 == 0) ? (wb & 0x0F) : (wb >> 4);
            acc += oracle_mx_value(ac, a_e8m0[(size_t)m * (cols / 32) + (size_t)(c / 32)]) *
                   oracle_mx_value(wc, w_e8m0[(size_t)r * (cols / 32) + (size_t)(c / 32)]);
        }
        y[idx] = acc;
    }
}

/* gate = scale2_g * (mx(x) . mx(W_g)), up likewise, over MXFP4 weights. */
int oracle_w4a4_dual(const uint16_t *x_bits, int M, int K, int N, const uint8_t *g_codes, const uint8_t *g_e8m0,
                     float g_scale2, const uint8_t *u_codes, const uint8_t *u_e8m0, float u_scale2, double *gate,
                     double *up)
{
    uint8_t *xc = (uint8_t *)malloc((size_t)M * (size_t)(K / 2));
    uint8_t *xs = (uint8_t *)malloc((size_t)M * (size_t)(K / 32));
    int rc = -1;
    if (xc && xs && oracle_mx_quantize_bf16(x_bits, M, K, xc, xs) == 0) {
        oracle_mx_linear_f64(xc, xs, M, K, g_codes, g_e8m0, N, gate);
        oracle_mx_linear_f64(xc, xs, M, K, u_codes, u_e8m0, N, up);
        for (size_t i = 0; i < (size_t)M * (size_t)N; ++i) {
            gate[i] *= (double)g_scale2;
            up[i] *= (double)u_scale2;
        }
        rc = 0;
    }
    free(xc);
    free(xs);
    return rc;
}

/* The down projection on 4 bits: out = scale2_d * (mx(h) . mx(W_d)) for bf16
 * h [M, N] (quantised as the activations are) and an MXFP4 W_d [K, N]. */
int oracle_w4a4_down(const uint16_t *h_bits, int M, int N, int K, const uint8_t *d_codes, const uint8_t *d_e8m0,
                     float d_scale2, double *out)
{
    uint8_t *hc = (uint8_t *)malloc((size_t)M * (size_t)(N / 2));
    uint8_t *hs = (uint8_t *)malloc((size_t)M * (size_t)(N / 32));
    int rc = -1;
    if (hc && hs && oracle_mx_quantize_bf16(h_bits, M, N, hc, hs) == 0) {
        oracle_mx_linear_f64(hc, hs, M, N, d_codes, d_e8m0, K, out);
        for (size_t i = 0; i < (size_t)M * (size_t)K; ++i)
            out[i] *= (double)d_scale2;
        rc = 0;
    }
    free(hc);
    free(hs);
    return rc;
}

/* The all-W4A4 FFN: W4A4 gate and up, h = bf16(act(gate) * up) (the down
 * input is a bf16 tensor, quantised to 4 bits like the activations), then
 * the down projection on 4 bits. */
int oracle_w4a4_ffn_fp4(const uint16_t *x_bits, int M, int K, int N, int act, const uint8_t *g_codes,
                        const uint8_t *g_e8m0, float g_scale2, const uint8_t *u_codes, const uint8_t *u_e8m0,
                        float u_scale2, const uint8_t *d_codes, const uint8_t *d_e8m0, float d_scale2, double *out)
{
    size_t mn = (size_t)M * (size_t)N;
    double *gate = (double *)malloc(sizeof(double) * mn);
    double *up = (double *)malloc(sizeof(double) * mn);
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * mn);
    int rc = -1;
    if (gate && up && h &&
        oracle_w4a4_dual(x_bits, M, K, N, g_codes, g_e8m0, g_scale2, u_codes, u_e8m0, u_scale2, gate, up) == 0) {
        oracle_gated_act(act, gate, up, mn, gate);
        for (size_t i = 0; i < mn; ++i)
            h[i] = oracle_bf16_round_bits(gate[i]);
        rc = oracle_w4a4_down(h, M, N, K, d_codes, d_e8m0, d_scale2, out);
    }
    free(gate);
    free(up);
    free(h);
    return rc;
}

/* The hybrid FFN: W4A4 gate and up, h = act(gate) * up, W4A16 down (NVFP4). */
int oracle_w4a4_ffn(const uint16_t *x_bits, int M, int K, int N, int act, const uint8_t *g_codes,
                    const uint8_t *g_e8m0, float g_scale2, const uint8_t *u_codes, const uint8_t *u_e8m0,
                    float u_scale2, const uint8_t *d_codes, const uint8_t *d_scales, float d_scale2, double *out)
{
    size_t mn = (size_t)M * (size_t)N;
    double *gate = (double *)malloc(sizeof(double) * mn);
    double *up = (double *)malloc(sizeof(double) * mn);
    int rc = -1;
    if (gate && up &&
        oracle_w4a4_dual(x_bits, M, K, N, g_codes, g_e8m0, g_scale2, u_codes, u_e8m0, u_scale2, gate, up) == 0) {
        oracle_gated_act(act, gate, up, mn, gate);
        oracle_down(gate, M, N, K, d_codes, d_scales, d_scale2, out);
        rc = 0;
    }
    free(gate);
    free(up);
    return rc;
}
