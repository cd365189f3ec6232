/*
 * fos_oracle.h: CPU oracle for the four-over-six NVFP4 quantizer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header,
 * table or constant generator with the HIP library; the knob numbers below are
 * the values the library's C ABI documents, restated here.
 */
#ifndef FOS_ORACLE_H
#define FOS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of the high-precision tensors */
#define ORC_BF16 0
#define ORC_FP16 1
#define ORC_FP32 2

/* recipes: standard NVFP4 (map-to-6 only) or four-over-six (map-to-6 and
 * map-to-4, keep the lower error). ORC_RECIPE_MAP4_ONLY is an oracle-only
 * diagnostic that always keeps the map-to-4 candidate; the tests use it to
 * look at the candidate four-over-six did not keep. */
#define ORC_RECIPE_NVFP4 0
#define ORC_RECIPE_4OVER6 1
#define ORC_RECIPE_MAP4_ONLY 2

#define ORC_BLOCK_1X16 0
#define ORC_BLOCK_16X16 1

#define ORC_PER_TENSOR 0
#define ORC_PER_ROW 1

#define ORC_MAE 0
#define ORC_MSE 1

#define ORC_ERR_EXACT 0
#define ORC_ERR_FP16 1

/* amax reductions */
#define ORC_AMAX_TENSOR 0
#define ORC_AMAX_ROW 1
#define ORC_AMAX_BAND16 2

/* status bits reported for data-dependent contract violations */
#define ORC_STATUS_TILE_NONUNIFORM 1
#define ORC_STATUS_BAD_OFFS 2

/* error-sum orders: the pinned width-16 tree, or a left-to-right sum over
 * the block's sixteen terms (1x16 blocks only) */
#define ORC_ORDER_TREE 0
#define ORC_ORDER_SEQ 1

typedef struct orc_cfg {
    int32_t recipe;
    int32_t block;
    int32_t scale_gran;
    int32_t err_metric;
    int32_t err_prec;
    int32_t e4m3_bound; /* 448 or 256 */
    int32_t err_order;  /* ORC_ORDER_TREE or ORC_ORDER_SEQ */
} orc_cfg;

/* element formats */
float oracle_e2m1_value(int code);
float oracle_e4m3_value(int code);
int oracle_e2m1_rne_sat(float v);
int oracle_e4m3_rne_sat(float t);
float oracle_f16_bits_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16_rne(float x);
uint16_t oracle_f32_to_bf16_rne(float x);
float oracle_bf16_bits_to_f32(uint16_t h);

/* array forms of the element conversions (for exhaustive pins) */
void oracle_e2m1_rne_sat_array(const float* v, int64_t n, uint8_t* out);
void oracle_e4m3_rne_sat_array(const float* t, int64_t n, uint8_t* out);
void oracle_f32_to_f16_rne_array(const float* x, int64_t n, uint16_t* out);
void oracle_f32_to_bf16_rne_array(const float* x, int64_t n, uint16_t* out);

/* global scales */
float oracle_global_encode_scale(float amax, int e4m3_bound);
float oracle_global_decode_scale(float amax, int e4m3_bound);
void oracle_global_scales_array(const float* amax, int64_t n, int e4m3_bound, float* s_enc, float* s_dec);

/* T16 reduction of 16 terms in the pinned order */
float oracle_tree16(const float* u);
float oracle_seq16(const float* u);

int oracle_amax(const void* x, int dtype, int64_t M, int64_t K, int mode, float* out);

/* Returns 0 on success, a negative value for an invalid argument. */
int oracle_quantize(const void* x, int dtype, int64_t M, int64_t K, const float* amax,
                    const orc_cfg* cfg, uint8_t* codes, uint8_t* scales, float* sdec_out,
                    float* xhat_out, uint8_t* choice_out, float* err_out, int32_t* status);

int oracle_qdq(const void* x, int dtype, int64_t M, int64_t K, const float* amax,
               const orc_cfg* cfg, void* y);

int oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t M, int64_t K,
                      const float* sdec, int scale_gran, int out_dtype, void* y);

int oracle_quantize_grouped(const void* x, int dtype, int64_t M_alloc, int64_t K,
                            const int32_t* offs, int G, const float* group_amax,
                            const orc_cfg* cfg, uint8_t* codes, uint8_t* scales,
                            float* group_sdec, int32_t* status);

int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif

#endif
