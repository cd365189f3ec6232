/*
 * fos_oracle.c: CPU oracle for the four-over-six ("4over6") NVFP4 quantizer.
 *
 * TEST INFRASTRUCTURE. This is a plain, slow, obviously correct CPU
 * implementation of what the GPU path computes. Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg may load it. It
 * shares no code with the HIP library, and nothing in the library calls it.
 *
 * Sources (web pages on the method):
 *  [AO-GEMM] pytorch/ao PR "Add the four-over-six grouped GEMM and dispatcher
 *            wiring": the quoted commits "recipe + pure-PyTorch reference",
 *            "CuTe DSL fast-path kernel" and "MoE grouped wiring".
 *  [AO-KERN] wolfcomos/ao PR "Add a CuTe DSL fast-path kernel for four-over-six
 *            quantize": the PR description.
 *  [MLM-QDQ] radixark/Megatron-LM PR "Fuse NVFP4 fake-QAT quantize-dequantize
 *            with CuTe DSL": section "What does this PR do?".
 * The pages name the element formats but print neither their grids nor any
 * formula. Format facts follow the OCP Microscaling Formats spec v1.0 (E2M1,
 * E4M3) and IEEE 754 (binary16, binary32). The order of operations inside a
 * block is the reading written down with each step below.
 *
 * Precision: the pages fix FP32 arithmetic (correctly rounded FP32 division,
 * FP32 error pairs, FP32 amax), so every arithmetic step here is one IEEE
 * binary32 operation rounded to nearest even. Build with -ffp-contract=off
 * -fno-fast-math on x86-64 (SSE arithmetic, FLT_EVAL_METHOD == 0).
 *
 * Parity pins: tests/test_oracle_*.py check this file against the OCP grids,
 * library casts (torch float8_e4m3fn, numpy float16, torch bfloat16), hand-worked
 * blocks under tests/golden/, an exact-rational brute force on tiny blocks, and
 * invariants (scale invariance, negation symmetry, candidate selection,
 * standard NVFP4 == the map-to-6 candidate, grouped == per-group).
 */
#include "fos_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if FLT_EVAL_METHOD != 0
#error "the oracle needs binary32 expression evaluation (FLT_EVAL_METHOD == 0)"
#endif

/* ------------------------------------------------------------------ */
/* Element formats                                                     */
/* ------------------------------------------------------------------ */

/* E2M1 (OCP MX v1.0): sign bit 3, exponent bits 2..1 with bias 1, one
 * mantissa bit; exponent 0 is subnormal (0.5 * m). No inf, no NaN. */
float oracle_e2m1_value(int code) {
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    float mag = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return s ? -mag : mag;
}

/* E4M3, the "fn" variant (OCP MX v1.0): sign bit 7, exponent bits 6..3 with
 * bias 7, three mantissa bits; exponent 0 is subnormal (m * 2^-9); S.1111.111
 * is NaN; there is no infinity. */
float oracle_e4m3_value(int code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 15 && m == 7) return NAN;
    float mag = (e == 0) ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

/* Nearest E2M1 code to v, ties to the even code, magnitudes above 6 saturate
 * to 6 (code 7); NaN gives +6 (code 0x7), the NaN rule the quantize kernel of
 * [AO-KERN] documents. The sign bit is v's sign bit, so -0 encodes to 0x8.
 * Linear search over the eight magnitudes; the distances are exact in double
 * wherever two of them can tie (at a midpoint between two grid values). */
int oracle_e2m1_rne_sat(float v) {
    if (isnan(v)) return 0x7;
    int sign = signbit(v) ? 8 : 0;
    double mag = fabs((double)v);
    if (mag > 6.0) mag = 6.0;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs(mag - (double)oracle_e2m1_value(c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | best;
}

/* Nearest E4M3 code to t >= 0, ties to the even code, saturating to the
 * largest finite value 448 (code 0x7E) for t >= 448 and for +inf. Linear
 * search over the 127 finite non-negative codes. Block scales are never
 * negative or NaN; a NaN t returns the NaN code 0x7F so that a caller bug
 * cannot hide. */
int oracle_e4m3_rne_sat(float t) {
    if (isnan(t)) return 0x7F;
    if (t >= 448.0f) return 0x7E;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs((double)t - (double)oracle_e4m3_value(c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* binary16 -> binary32 from the IEEE 754 definition: 5 exponent bits (bias
 * 15), 10 fraction bits, subnormals m * 2^-24. Exact. */
float oracle_f16_bits_to_f32(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    float mag;
    if (e == 31)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexpf((float)m, -24);
    else
        mag = ldexpf((float)(1024 + m), e - 25);
    return s ? -mag : mag;
}

float oracle_bf16_bits_to_f32(uint16_t h) {
    /* bfloat16 is the upper half of a binary32 encoding */
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round |x| to the grid of a binary format with `mant` fraction bits and
 * minimum normal exponent `emin`, ties to even, in double (exact: x is a
 * binary32 value and the quantum is a power of two). */
static double round_to_format(double a, int mant, int emin) {
    if (a == 0.0) return 0.0;
    int e;
    frexp(a, &e);  /* a = f * 2^e with f in [0.5, 1): binade exponent e - 1 */
    int be = e - 1;
    if (be < emin) be = emin;
    double q = ldexp(1.0, be - mant);
    return nearbyint(a / q) * q; /* default rounding mode: ties to even */
}

/* binary32 -> binary16, round to nearest even, overflow to +-inf, gradual
 * underflow; NaN becomes the canonical 0x7E00. */
uint16_t oracle_f32_to_f16_rne(float x) {
    if (isnan(x)) return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isinf(x)) return sign | 0x7C00;
    double r = round_to_format(fabs((double)x), 10, -14);
    if (r > 65504.0) return sign | 0x7C00;
    if (r == 0.0) return sign;
    int e;
    frexp(r, &e);
    int be = e - 1;
    if (be < -14) return sign | (uint16_t)(r / ldexp(1.0, -24)); /* subnormal */
    uint16_t mant = (uint16_t)(r / ldexp(1.0, be - 10) - 1024.0);
    return sign | (uint16_t)((be + 15) << 10) | mant;
}

/* binary32 -> bfloat16, round to nearest even, overflow to +-inf, gradual
 * underflow; NaN becomes the canonical 0x7FC0. */
uint16_t oracle_f32_to_bf16_rne(float x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isinf(x)) return sign | 0x7F80;
    double r = round_to_format(fabs((double)x), 7, -126);
    if (r > ldexp(255.0, 120)) return sign | 0x7F80; /* max finite (2 - 2^-7) * 2^127 */
    if (r == 0.0) return sign;
    int e;
    frexp(r, &e);
    int be = e - 1;
    if (be < -126) return sign | (uint16_t)(r / ldexp(1.0, -133));
    uint16_t mant = (uint16_t)(r / ldexp(1.0, be - 7) - 128.0);
    return sign | (uint16_t)((be + 127) << 7) | mant;
}

void oracle_e2m1_rne_sat_array(const float* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)oracle_e2m1_rne_sat(v[i]);
}

void oracle_e4m3_rne_sat_array(const float* t, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)oracle_e4m3_rne_sat(t[i]);
}

void oracle_f32_to_f16_rne_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = oracle_f32_to_f16_rne(x[i]);
}

void oracle_f32_to_bf16_rne_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = oracle_f32_to_bf16_rne(x[i]);
}

/* ------------------------------------------------------------------ */
/* Global scales                                                       */
/* ------------------------------------------------------------------ */

/* Global encode scale. The pages name the E4M3 bound (448 or 256) and the
 * map-to-6 encoding ([MLM-QDQ] numerical contract; [AO-GEMM] recipe commit)
 * but print no formula. Reading: the tensor (or row, or group) amax maps to
 * 6 * bound, the largest value a map-to-6 block can reach:
 *     S_enc = RN(6 * bound / A)   for 0 < A < inf, clamped to FLT_MAX;
 *     S_enc = 1                   for A = 0, A = inf, A = NaN (or A < 0). */
float oracle_global_encode_scale(float A, int bound) {
    if (!(A > 0.0f) || isinf(A)) return 1.0f;
    float s = (6.0f * (float)bound) / A;
    if (s > FLT_MAX) s = FLT_MAX;
    return s;
}

/* Global decode scale: S_dec = RN(1 / S_enc). */
float oracle_global_decode_scale(float A, int bound) {
    return 1.0f / oracle_global_encode_scale(A, bound);
}

/* array forms of the two global scales (for exhaustive pins) */
void oracle_global_scales_array(const float* amax, int64_t n, int e4m3_bound, float* s_enc, float* s_dec) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        s_enc[i] = oracle_global_encode_scale(amax[i], e4m3_bound);
        s_dec[i] = oracle_global_decode_scale(amax[i], e4m3_bound);
    }
}

/* ------------------------------------------------------------------ */
/* Reductions                                                          */
/* ------------------------------------------------------------------ */

/* The pinned width-16 error-reduction order of [AO-KERN] (a clamped
 * shuffle-down tree): strides 8, 4, 2, 1, where position i adds position
 * i + stride. Position 0 ends with
 *   ((u0+u8)+(u4+u12)) + ((u2+u10)+(u6+u14))
 *     + ( ((u1+u9)+(u5+u13)) + ((u3+u11)+(u7+u15)) ).
 * Every + is one binary32 addition. */
float oracle_tree16(const float* u) {
    float w[16];
    memcpy(w, u, sizeof w);
    for (int stride = 8; stride >= 1; stride /= 2)
        for (int i = 0; i < stride; i++) w[i] = w[i] + w[i + stride];
    return w[0];
}

/* Transformer Engine's sequential order, which the Megatron-LM PR keeps for
 * its candidate errors ([MLM-QDQ] "What does this PR do?", FP16 error
 * contract): the sixteen terms added left to right in element order,
 * ((u0 + u1) + u2) + ... + u15, each + one binary32 addition. */
float oracle_seq16(const float* u) {
    float s = u[0];
    for (int i = 1; i < 16; i++) s = s + u[i];
    return s;
}

/* NaN-dropping max |x| with start value +0 ([AO-KERN]: NaN inputs take
 * NaN-dropping amaxes). |-0| = +0; an all-NaN set gives +0. */
static float nan_dropping_absmax(float acc, float x) {
    if (isnan(x)) return acc;
    float m = fabsf(x);
    return (m > acc) ? m : acc;
}

/* ------------------------------------------------------------------ */
/* Inputs                                                              */
/* ------------------------------------------------------------------ */

static int dtype_ok(int dtype) { return dtype == ORC_BF16 || dtype == ORC_FP16 || dtype == ORC_FP32; }

/* exact upcast of element idx to binary32 */
static float load_elem(const void* x, int dtype, int64_t idx) {
    if (dtype == ORC_BF16) return oracle_bf16_bits_to_f32(((const uint16_t*)x)[idx]);
    if (dtype == ORC_FP16) return oracle_f16_bits_to_f32(((const uint16_t*)x)[idx]);
    return ((const float*)x)[idx];
}

static void store_elem(void* y, int dtype, int64_t idx, float v) {
    if (dtype == ORC_BF16)
        ((uint16_t*)y)[idx] = oracle_f32_to_bf16_rne(v);
    else if (dtype == ORC_FP16)
        ((uint16_t*)y)[idx] = oracle_f32_to_f16_rne(v);
    else
        ((float*)y)[idx] = v;
}

int oracle_amax(const void* x, int dtype, int64_t M, int64_t K, int mode, float* out) {
    if (!dtype_ok(dtype) || M < 0 || K < 0) return -1;
    if (mode == ORC_AMAX_TENSOR) {
        float a = 0.0f;
        for (int64_t i = 0; i < M * K; i++) a = nan_dropping_absmax(a, load_elem(x, dtype, i));
        out[0] = a;
        return 0;
    }
    if (mode == ORC_AMAX_ROW) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < M; r++) {
            float a = 0.0f;
            for (int64_t c = 0; c < K; c++) a = nan_dropping_absmax(a, load_elem(x, dtype, r * K + c));
            out[r] = a;
        }
        return 0;
    }
    if (mode == ORC_AMAX_BAND16) {
        /* max over each 16-row band, written to every row of the band (the
         * tile-uniform per-row amax that 16x16 blocks accept, [AO-GEMM]) */
        if (M % 16) return -1;
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < M / 16; b++) {
            float a = 0.0f;
            for (int64_t i = b * 16 * K; i < (b + 1) * 16 * K; i++) a = nan_dropping_absmax(a, load_elem(x, dtype, i));
            for (int r = 0; r < 16; r++) out[b * 16 + r] = a;
        }
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------------ */
/* One block                                                           */
/* ------------------------------------------------------------------ */

typedef struct cand {
    uint8_t q[256];    /* E2M1 codes */
    float xhat[256];   /* decoded values in the real domain */
    int scale;         /* E4M3 code */
    float err;         /* summed error terms */
} cand;

/* Encode one block of n = 16 * nrows elements (row-major, 16 per row) with
 * candidate divisor c: 6 for the map-to-6 (standard NVFP4) encoding, 4 for
 * the map-to-4 candidate whose block scale is 1.5x larger ([AO-GEMM] recipe
 * commit: the block amax lands on E2M1 value 6 or 4). */
static void encode_candidate(const float* xb, int nrows, float a, float c, float S_enc, float S_dec,
                             const orc_cfg* cfg, int want_err, cand* out) {
    int n = 16 * nrows;
    /* block scale: t = RN(RN(a / c) * S_enc), cast to E4M3 with RNE and
     * saturation ([AO-KERN]: correctly rounded FP32 division and the E4M3
     * cast are the rounding-critical steps) */
    float t = (a / c) * S_enc;
    int s = oracle_e4m3_rne_sat(t);
    float sigma = oracle_e4m3_value(s);
    /* per-block multipliers: encode E = RN(S_enc / sigma) (0 when sigma = 0,
     * FLT_MAX when it overflows); decode D = RN(sigma * S_dec). Every element
     * is multiplied by one common scale ([MLM-QDQ] "packed pair arithmetic") */
    float E = 0.0f;
    if (sigma != 0.0f) {
        E = S_enc / sigma;
        if (E > FLT_MAX) E = FLT_MAX;
    }
    float D = sigma * S_dec;
    float terms[256];
    for (int i = 0; i < n; i++) {
        float v = xb[i] * E;
        int q = oracle_e2m1_rne_sat(v);
        float xhat = oracle_e2m1_value(q) * D;
        out->q[i] = (uint8_t)q;
        out->xhat[i] = xhat;
        if (want_err) {
            /* error in the real domain against the value the dequantizer
             * would emit; FP16-error mode first rounds that value to binary16
             * ([MLM-QDQ]: FP16 candidate-error contract, FP32 error pairs) */
            float ref = xhat;
            if (cfg->err_prec == ORC_ERR_FP16) ref = oracle_f16_bits_to_f32(oracle_f32_to_f16_rne(xhat));
            float e = xb[i] - ref;
            terms[i] = (cfg->err_metric == ORC_MAE) ? fabsf(e) : e * e;
        }
    }
    out->scale = s;
    out->err = 0.0f;
    if (want_err) {
        if (nrows == 1) {
            out->err = (cfg->err_order == ORC_ORDER_SEQ) ? oracle_seq16(terms) : oracle_tree16(terms);
        } else {
            /* 16x16 tile: one pinned tree per row, then the same tree over
             * the sixteen row sums (row index order) */
            float rows[16];
            for (int r = 0; r < 16; r++) rows[r] = oracle_tree16(terms + 16 * r);
            out->err = oracle_tree16(rows);
        }
    }
}

/* Quantize one block. Writes the kept candidate's codes, scale and decoded
 * values; returns the kept candidate's divisor (6 or 4). */
static int quantize_block(const float* xb, int nrows, float S_enc, float S_dec, const orc_cfg* cfg,
                          uint8_t* q_out, int* scale_out, float* xhat_out, float* err6, float* err4) {
    int n = 16 * nrows;
    float a = 0.0f;
    for (int i = 0; i < n; i++) a = nan_dropping_absmax(a, xb[i]);

    cand c6, c4;
    const cand* keep;
    int kept;
    if (cfg->recipe == ORC_RECIPE_NVFP4) {
        encode_candidate(xb, nrows, a, 6.0f, S_enc, S_dec, cfg, 0, &c6);
        keep = &c6;
        kept = 6;
        *err6 = NAN;
        *err4 = NAN;
    } else if (cfg->recipe == ORC_RECIPE_MAP4_ONLY) {
        encode_candidate(xb, nrows, a, 4.0f, S_enc, S_dec, cfg, 1, &c4);
        keep = &c4;
        kept = 4;
        *err6 = NAN;
        *err4 = c4.err;
    } else {
        encode_candidate(xb, nrows, a, 6.0f, S_enc, S_dec, cfg, 1, &c6);
        encode_candidate(xb, nrows, a, 4.0f, S_enc, S_dec, cfg, 1, &c4);
        /* keep the lower-error candidate ([AO-GEMM] recipe commit); a tie or a
         * NaN error keeps map-to-6 */
        if (c4.err < c6.err) {
            keep = &c4;
            kept = 4;
        } else {
            keep = &c6;
            kept = 6;
        }
        *err6 = c6.err;
        *err4 = c4.err;
    }
    memcpy(q_out, keep->q, (size_t)n);
    memcpy(xhat_out, keep->xhat, sizeof(float) * (size_t)n);
    *scale_out = keep->scale;
    return kept;
}

/* ------------------------------------------------------------------ */
/* Tensors                                                             */
/* ------------------------------------------------------------------ */

static int cfg_ok(const orc_cfg* cfg) {
    if (!cfg) return 0;
    if (cfg->recipe != ORC_RECIPE_NVFP4 && cfg->recipe != ORC_RECIPE_4OVER6 && cfg->recipe != ORC_RECIPE_MAP4_ONLY)
        return 0;
    if (cfg->block != ORC_BLOCK_1X16 && cfg->block != ORC_BLOCK_16X16) return 0;
    if (cfg->scale_gran != ORC_PER_TENSOR && cfg->scale_gran != ORC_PER_ROW) return 0;
    if (cfg->err_metric != ORC_MAE && cfg->err_metric != ORC_MSE) return 0;
    if (cfg->err_prec != ORC_ERR_EXACT && cfg->err_prec != ORC_ERR_FP16) return 0;
    if (cfg->e4m3_bound != 448 && cfg->e4m3_bound != 256) return 0;
    if (cfg->err_order != ORC_ORDER_TREE && cfg->err_order != ORC_ORDER_SEQ) return 0;
    /* the sequential order is defined for 1x16 blocks only */
    if (cfg->err_order == ORC_ORDER_SEQ && cfg->block != ORC_BLOCK_1X16) return 0;
    return 1;
}

/* Quantize X[M, K] (row-major). Outputs:
 *   codes[M, K/2]  element 2j in the low nibble of byte j of its row
 *   scales[M, K/16] row-major; a 16x16 tile's scale is written to all 16 rows
 *   sdec_out       S_dec per tensor ([1]) or per row ([M]), nullable
 *   xhat_out       float [M, K], the kept candidate's decoded values, nullable
 *   choice_out     [nblocks] the kept divisor (6 or 4), nullable
 *   err_out        [nblocks][2] (Err_6, Err_4), nullable
 *   status         OR of ORC_STATUS_* bits, nullable
 * Blocks are enumerated row-block-major: block (rb, cb) has index
 * rb * (K / 16) + cb with rb the row (1x16) or the 16-row band (16x16). */
int oracle_quantize(const void* x, int dtype, int64_t M, int64_t K, const float* amax,
                    const orc_cfg* cfg, uint8_t* codes, uint8_t* scales, float* sdec_out,
                    float* xhat_out, uint8_t* choice_out, float* err_out, int32_t* status) {
    if (!dtype_ok(dtype) || !cfg_ok(cfg) || M < 0 || K < 0 || K % 16) return -1;
    int nrows = (cfg->block == ORC_BLOCK_16X16) ? 16 : 1;
    if (M % nrows) return -1;
    const int64_t nbk = K / 16;
    const int64_t nrb = M / nrows;
    int32_t st = 0;

    if (sdec_out) {
        if (cfg->scale_gran == ORC_PER_TENSOR)
            sdec_out[0] = oracle_global_decode_scale(amax[0], cfg->e4m3_bound);
        else
            for (int64_t r = 0; r < M; r++) sdec_out[r] = oracle_global_decode_scale(amax[r], cfg->e4m3_bound);
    }

#pragma omp parallel for schedule(dynamic, 1) reduction(| : st)
    for (int64_t rb = 0; rb < nrb; rb++) {
        int64_t r0 = rb * nrows;
        /* the global amax of this block row: the tensor's, or the row's; a
         * 16x16 tile uses its first row's amax and flags a non-uniform band */
        float A = (cfg->scale_gran == ORC_PER_TENSOR) ? amax[0] : amax[r0];
        if (cfg->scale_gran == ORC_PER_ROW && nrows == 16) {
            for (int i = 1; i < 16; i++) {
                float Ai = amax[r0 + i];
                if (memcmp(&Ai, &A, sizeof A) != 0) st |= ORC_STATUS_TILE_NONUNIFORM;
            }
        }
        float S_enc = oracle_global_encode_scale(A, cfg->e4m3_bound);
        float S_dec = 1.0f / S_enc;

        float xb[256], xhat[256];
        uint8_t q[256];
        for (int64_t cb = 0; cb < nbk; cb++) {
            for (int i = 0; i < nrows; i++)
                for (int j = 0; j < 16; j++) xb[16 * i + j] = load_elem(x, dtype, (r0 + i) * K + cb * 16 + j);
            int s;
            float e6, e4;
            int kept = quantize_block(xb, nrows, S_enc, S_dec, cfg, q, &s, xhat, &e6, &e4);
            int64_t bidx = rb * nbk + cb;
            if (choice_out) choice_out[bidx] = (uint8_t)kept;
            if (err_out) {
                err_out[2 * bidx] = e6;
                err_out[2 * bidx + 1] = e4;
            }
            for (int i = 0; i < nrows; i++) {
                int64_t r = r0 + i;
                for (int j = 0; j < 8; j++)
                    codes[r * (K / 2) + cb * 8 + j] =
                        (uint8_t)((q[16 * i + 2 * j] & 0xF) | ((q[16 * i + 2 * j + 1] & 0xF) << 4));
                scales[r * nbk + cb] = (uint8_t)s;
                if (xhat_out)
                    for (int j = 0; j < 16; j++) xhat_out[r * K + cb * 16 + j] = xhat[16 * i + j];
            }
        }
    }
    if (status) *status |= st;
    return 0;
}

/* Fused fake-quantization ([MLM-QDQ] "fused data path"): the kept candidate's
 * decoded values rounded once to the input dtype (RNE); no codes or scales
 * leave the call. Same arithmetic as quantize followed by dequantize. */
int oracle_qdq(const void* x, int dtype, int64_t M, int64_t K, const float* amax, const orc_cfg* cfg, void* y) {
    if (!dtype_ok(dtype) || !cfg_ok(cfg) || M < 0 || K < 0 || K % 16) return -1;
    int nrows = (cfg->block == ORC_BLOCK_16X16) ? 16 : 1;
    if (M % nrows) return -1;
    size_t n = (size_t)(M * K);
    uint8_t* codes = (uint8_t*)malloc(n / 2 + 1);
    uint8_t* scales = (uint8_t*)malloc(n / 16 + 1);
    float* xhat = (float*)malloc(sizeof(float) * n + 1);
    if (!codes || !scales || !xhat) {
        free(codes);
        free(scales);
        free(xhat);
        return -2;
    }
    int rc = oracle_quantize(x, dtype, M, K, amax, cfg, codes, scales, NULL, xhat, NULL, NULL, NULL);
    if (rc == 0) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < (int64_t)n; i++) store_elem(y, dtype, i, xhat[i]);
    }
    free(codes);
    free(scales);
    free(xhat);
    return rc;
}

/* Standard NVFP4 decode, recipe-agnostic ([AO-GEMM] recipe commit,
 * nvfp4_dequantize): y = dtype(RN(val(q) * RN(sigma * S_dec))) with S_dec per
 * tensor or per row. */
int oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t M, int64_t K, const float* sdec,
                      int scale_gran, int out_dtype, void* y) {
    if (!dtype_ok(out_dtype) || M < 0 || K < 0 || K % 16) return -1;
    if (scale_gran != ORC_PER_TENSOR && scale_gran != ORC_PER_ROW) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; r++) {
        float S_dec = (scale_gran == ORC_PER_TENSOR) ? sdec[0] : sdec[r];
        for (int64_t c = 0; c < K; c++) {
            uint8_t byte = codes[r * (K / 2) + c / 2];
            int q = (c % 2) ? (byte >> 4) : (byte & 0xF);
            float sigma = oracle_e4m3_value(scales[r * (K / 16) + c / 16]);
            float D = sigma * S_dec;
            store_elem(y, out_dtype, r * K + c, oracle_e2m1_value(q) * D);
        }
    }
    return 0;
}

/* Grouped activations ([AO-GEMM] MoE commit): each token group's amax is
 * expanded to a per-row vector and the packed tensor quantizes as one
 * per-row-scaled 1x16 tensor. offs holds cumulative end rows (group g owns
 * rows [offs[g-1], offs[g]) with offs[-1] = 0); rows at or past offs[G-1] are
 * the over-allocated tail, which is not read and gets zero codes and scales.
 * group_sdec (nullable) receives S_dec of each group. */
int oracle_quantize_grouped(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                            const float* group_amax, const orc_cfg* cfg, uint8_t* codes, uint8_t* scales,
                            float* group_sdec, int32_t* status) {
    if (!dtype_ok(dtype) || !cfg_ok(cfg) || G <= 0 || M_alloc < 0 || K < 0 || K % 16) return -1;
    if (cfg->block != ORC_BLOCK_1X16) return -1;
    int32_t prev = 0;
    int bad = 0;
    for (int g = 0; g < G; g++) {
        if (offs[g] < prev || offs[g] % 16) bad = 1;
        prev = offs[g];
    }
    if (offs[G - 1] > M_alloc) bad = 1;
    if (bad) {
        if (status) *status |= ORC_STATUS_BAD_OFFS;
        return 0; /* nothing written: the offsets break the contract */
    }
    int64_t M = offs[G - 1];
    float* row_amax = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    if (!row_amax) return -2;
    int g = 0;
    for (int64_t r = 0; r < M; r++) {
        while (r >= offs[g]) g++;
        row_amax[r] = group_amax[g];
    }
    orc_cfg rc_cfg = *cfg;
    rc_cfg.scale_gran = ORC_PER_ROW;
    int rc = oracle_quantize(x, dtype, M, K, row_amax, &rc_cfg, codes, scales, NULL, NULL, NULL, NULL, status);
    free(row_amax);
    if (rc) return rc;
    memset(codes + M * (K / 2), 0, (size_t)((M_alloc - M) * (K / 2)));
    memset(scales + M * (K / 16), 0, (size_t)((M_alloc - M) * (K / 16)));
    if (group_sdec)
        for (int gg = 0; gg < G; gg++) group_sdec[gg] = oracle_global_decode_scale(group_amax[gg], cfg->e4m3_bound);
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
