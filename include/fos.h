/*
 * fos.h: C ABI of the four-over-six NVFP4 quantizer for AMD MI355X (gfx950).
 *
 * Four-over-six is an adaptive NVFP4 block-scaling recipe: every 16-element
 * block (1x16 along a row, or a 16x16 tile) is encoded twice, once with the
 * standard map-to-6 scaling (the block amax lands on E2M1 value 6) and once
 * with a 1.5x larger block scale (map-to-4, the amax lands on 4), and the
 * candidate with the lower error is stored as packed E2M1 codes plus an E4M3
 * block scale under an FP32 global scale (pytorch/ao PR "Add the four-over-six
 * grouped GEMM and dispatcher wiring", recipe commit). The error metric is MAE
 * or MSE, computed exactly in FP32 or against FP16-rounded decoded values, and
 * the E4M3 bound is 448 or 256 (radixark/Megatron-LM PR "Fuse NVFP4 fake-QAT
 * quantize-dequantize with CuTe DSL", "What does this PR do?", numerical
 * contract).
 *
 * Conventions for every call:
 *  - Tensor pointers are device pointers on the current HIP device. `stream`
 *    is a hipStream_t on that device (NULL: the null stream). Calls are
 *    asynchronous: a zero return means the work is enqueued on `stream`.
 *  - High-precision tensors are row-major [M, K], contiguous, with K a
 *    multiple of 16; element type bf16, fp16 or fp32 (FOS_BF16 ...); the base
 *    pointer is 16-byte aligned.
 *  - Codes: uint8 [M, K/2], element 2j of a row in the low nibble of byte j
 *    (E2M1: sign bit 3, magnitude codes 0..7 = {0, 0.5, 1, 1.5, 2, 3, 4, 6}).
 *  - Scales: uint8 [M, K/16] row-major E4M3 (the "fn" variant, max 448). A
 *    16x16 tile's scale is written to each of its 16 rows, so one decode
 *    serves both block shapes.
 *  - Global scales. From an amax A (per tensor, per row or per group) and the
 *    E4M3 bound B: S_enc = RN(6B / A), clamped to FLT_MAX, or 1 when A is 0,
 *    inf, NaN or negative; S_dec = RN(1 / S_enc).
 *  - The library allocates nothing and keeps no state between calls; the
 *    caller owns every buffer. Outputs are fully written by every successful
 *    call (padding rows of the grouped call included).
 *  - Errors: a nonzero return is an FOS_ERR_* code, nothing is enqueued, and
 *    fos_last_error() returns a description (thread-local). Conditions that
 *    only the data can reveal (a 16x16 tile whose per-row amax differs, bad
 *    group offsets) are OR-ed as FOS_STATUS_* bits into the optional device
 *    word `d_status` (the caller zeroes it; read it after the stream syncs).
 *  - NaN inputs follow the rule the kernel page (wolfcomos/ao PR "Add a CuTe
 *    DSL fast-path kernel for four-over-six quantize", description) states:
 *    block and global amaxes drop NaN, and a NaN element encodes to +6.
 *  - Every result is bitwise defined: one binary32 operation per step,
 *    round-to-nearest-even, E4M3/E2M1 casts RNE with saturation, the error
 *    terms of a block summed in one pinned order (the shuffle-down tree with
 *    strides 8, 4, 2, 1 by default, or a left-to-right sum), the map-to-4
 *    candidate kept only on a strictly lower error.
 */
#ifndef FOS_H
#define FOS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FOS_ABI_VERSION 6

/* element types */
#define FOS_BF16 0
#define FOS_FP16 1
#define FOS_FP32 2

/* fos_config.recipe */
#define FOS_RECIPE_NVFP4 0  /* standard NVFP4: the map-to-6 candidate only */
#define FOS_RECIPE_4OVER6 1 /* keep the lower-error of map-to-6 and map-to-4 */

/* fos_config.block */
#define FOS_BLOCK_1X16 0
#define FOS_BLOCK_16X16 1

/* fos_config.scale_gran: one amax per tensor or one per row */
#define FOS_PER_TENSOR 0
#define FOS_PER_ROW 1

/* fos_config.err_metric (four-over-six only) */
#define FOS_ERR_MAE 0
#define FOS_ERR_MSE 1

/* fos_config.err_prec (four-over-six only): error against the FP32 decoded
 * value, or against that value rounded to binary16 */
#define FOS_ERR_EXACT 0
#define FOS_ERR_FP16 1

/* fos_config.err_order (four-over-six only): the order in which a block's
 * sixteen error terms are summed. The tree is the width-16 shuffle-down order
 * the kernel page pins (wolfcomos/ao PR, description); the sequential order,
 * ((u0 + u1) + u2) + ... + u15, is Transformer Engine's term order that the
 * Megatron-LM PR keeps ("What does this PR do?", FP16 error contract). The
 * sequential order is defined for 1x16 blocks only. */
#define FOS_ORDER_TREE 0
#define FOS_ORDER_SEQ 1

/* fos_amax granularity */
#define FOS_AMAX_TENSOR 0
#define FOS_AMAX_ROW 1
#define FOS_AMAX_BAND16 2 /* max over each 16-row band, written to its 16 rows */

/* return codes */
#define FOS_OK 0
#define FOS_ERR_INVALID_ARG 1 /* null pointer, bad enum value, negative size */
#define FOS_ERR_DTYPE 2       /* element type not supported by this call */
#define FOS_ERR_SHAPE 3       /* K % 16, M % 16 for 16x16, size limits */
#define FOS_ERR_ALIGN 4       /* base pointer not 16-byte aligned */
#define FOS_ERR_CONFIG 5      /* knob combination not supported by this call */
#define FOS_ERR_DEVICE 6      /* no HIP device, or not a gfx950 device */
#define FOS_ERR_LAUNCH 7      /* the kernel launch failed (see fos_last_error) */

/* device status bits */
#define FOS_STATUS_TILE_NONUNIFORM 1 /* 16x16 with a per-row amax that differs within a 16-row band */
#define FOS_STATUS_BAD_OFFS 2        /* group offsets not monotone, not multiples of 16, or past M_alloc */
#define FOS_STATUS_BARRIER_TIMEOUT 4 /* fused calls: the grid barrier did not complete in time (fos_set_barrier_poll_limit) */

/* Bytes of the device workspace the fused calls (fos_quantize_fused,
 * fos_quantize_grouped_fused, fos_qdq_fused) need; the most groups the fused
 * grouped call takes (added in ABI version 3). */
#define FOS_FUSED_WORKSPACE_BYTES 16384
#define FOS_FUSED_MAX_GROUPS 256

typedef struct fos_config {
    int32_t recipe;     /* FOS_RECIPE_* */
    int32_t block;      /* FOS_BLOCK_* */
    int32_t scale_gran; /* FOS_PER_TENSOR | FOS_PER_ROW */
    int32_t err_metric; /* FOS_ERR_MAE | FOS_ERR_MSE */
    int32_t err_prec;   /* FOS_ERR_EXACT | FOS_ERR_FP16 */
    int32_t e4m3_bound; /* 448 or 256 */
    int32_t err_order;  /* FOS_ORDER_TREE | FOS_ORDER_SEQ (added in ABI version 2) */
} fos_config;

/* One tensor of a weight list (fos_qdq_list). */
typedef struct fos_tensor_desc {
    const void* x;      /* [M, K] input */
    void* y;            /* [M, K] output, same element type */
    const float* amax;  /* device FP32 amax: [1] per tensor, or [M] per row */
    int64_t M;
    int64_t K;
} fos_tensor_desc;

int fos_abi_version(void);
const char* fos_status_string(int status);
const char* fos_last_error(void);

/* The fused calls' grid barrier waits a bounded number of polls (each at
 * least 128 GPU cycles of sleep) before a workgroup gives up, sets
 * FOS_STATUS_BARRIER_TIMEOUT and leaves its part of the outputs unwritten.
 * The default, 2^20 polls, is about a second. This sets the limit for fused
 * calls enqueued from now on, process-wide, and returns the previous one
 * (-1 and no change for a negative value). A limit of 0 makes every
 * workgroup that is not the barrier's last arrival give up at once, which
 * lets a caller exercise its timeout handling (added in ABI version 5).
 * A workgroup that gives up has still arrived at the barrier, so the
 * barrier completes when the rest of the grid arrives: the workspace is
 * left consistent and the next call on it is correct. */
int fos_set_barrier_poll_limit(int polls);

/* Diagnostics (added in ABI version 6). With d_buf non-NULL, every
 * one-read fused launch (fos_quantize_fused or fos_qdq_fused on a tensor
 * that fits on chip) enqueued from now on, process-wide, writes for each of
 * its waves w < max_waves four values of the device's real-time counter to
 * d_buf[4w .. 4w + 3]: the wave's start, the moment its phase-1 loads have
 * landed, the moment the grid barrier releases it, and its end (a wave
 * whose barrier gave up writes nothing). d_buf is a device buffer of
 * 4 * max_waves uint64 values, owned by the caller and written by every
 * such launch until this is called again with d_buf = NULL. *clock_khz
 * (if non-NULL) receives the counter's rate in kHz. Calls whose launches
 * overlap overwrite each other's values. */
int fos_set_phase_timestamps(unsigned long long* d_buf, int64_t max_waves, int* clock_khz);

/* Global amax: NaN-dropping max |x| with start value +0, per tensor
 * (out[1]), per row (out[M]) or per 16-row band (out[M], M % 16 == 0).
 * Max is exact and order-free, so the result does not depend on the launch.
 * The pages compute this with one FP32 torch reduction per tensor before
 * the quantizer (Megatron-LM PR, "What does this PR do?", fused data path). */
int fos_amax(const void* x, int dtype, int64_t M, int64_t K, int gran, float* amax_out, void* stream);

/* Quantize x[M, K] to codes[M, K/2] and scales[M, K/16] under `cfg`
 * (pytorch/ao PR, recipe commit: four_over_six_quantize with per-tensor or
 * row-scaled global scales and 1x16 or 16x16 blocks).
 *   amax:     FP32 [1] (FOS_PER_TENSOR) or [M] (FOS_PER_ROW). With 16x16
 *             blocks a per-row amax must be equal within each 16-row band
 *             (the tile-uniform contract of the MoE commit); a band that is
 *             not is flagged in d_status and quantized with its first row's
 *             amax.
 *   sdec_out: nullable; receives S_dec per tensor [1] or per row [M].
 *   d_status: nullable device int32. */
int fos_quantize(const void* x, int dtype, int64_t M, int64_t K, const float* amax, const fos_config* cfg,
                 uint8_t* codes, uint8_t* scales, float* sdec_out, int32_t* d_status, void* stream);

/* Fused fake quantization: y[M, K] = the kept candidate's decoded values,
 * rounded once to the input type (RNE); no codes or scales are written
 * (Megatron-LM PR, "What does this PR do?": fused data path with a caller-
 * provided FP32 per-tensor amax, 1x16 blocks, bf16/fp16). Bitwise equal to
 * nvfp4_dequantize(fos_quantize(x)) for every config fos_quantize takes:
 * bf16, fp16 or fp32; 1x16 or 16x16 blocks; amax per tensor [1] or per row
 * [M] (16x16: equal within each 16-row band). */
int fos_qdq(const void* x, int dtype, int64_t M, int64_t K, const float* amax, const fos_config* cfg, void* y,
            void* stream);

/* fos_qdq over a list of n independently stored rank-2 tensors of one
 * element type (the list API of the Megatron-LM PR maps any number of
 * discrete weights): 1x16 blocks take one launch per 48 tensors, 16x16 tiles
 * one launch per tensor. Each descriptor's amax is [1] (per tensor) or [M]
 * (per row). `descs` is a HOST array; it is copied into the launch
 * arguments, so the caller may reuse it on return. */
int fos_qdq_list(int n, const fos_tensor_desc* descs, int dtype, const fos_config* cfg, void* stream);

/* Standard NVFP4 decode, recipe-agnostic (pytorch/ao PR, recipe commit:
 * nvfp4_dequantize): y = out_dtype(RN(val(q) * RN(sigma * S_dec))) with sdec
 * per tensor [1] or per row [M]. */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t M, int64_t K, const float* sdec,
                     int scale_gran, int out_dtype, void* y, void* stream);

/* Grouped (MoE) activation quantize in one launch (pytorch/ao PR, MoE
 * commit): x[M_alloc, K] holds G token groups back to back; group g owns
 * rows [offs[g-1], offs[g]) (offs[-1] = 0, cumulative end offsets, multiples
 * of 16, empty groups allowed) and its rows quantize with the per-row global
 * scale from group_amax[g]. Rows at or past offs[G-1] are an over-allocated
 * tail: they are not read, and their codes and scales are written as zero.
 * The result equals fos_quantize of each group slice with its own per-tensor
 * amax. cfg must be 1x16; cfg->scale_gran is ignored.
 *   offs, group_amax: device int32[G], float[G].
 *   group_sdec_out:   nullable device float[G].
 * Offsets that break the contract set FOS_STATUS_BAD_OFFS; the outputs are
 * then unspecified. */
int fos_quantize_grouped(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                         const float* group_amax, const fos_config* cfg, uint8_t* codes, uint8_t* scales,
                         float* group_sdec_out, int32_t* d_status, void* stream);

/* Columnwise quantize: the quantize of X^T (the [K, M] transpose of x,
 * the operand of the backward GEMM; pytorch/ao PR, recipe commit, and the
 * Megatron-LM PR's "Limitations and pending work" name the columnwise
 * output), without materialising X^T. 1x16 blocks run down the columns of
 * x: block (c, b) holds x[16b .. 16b+15, c]. Outputs are laid out as
 * fos_quantize of X^T would write them:
 *   codes_t:  [K, M/2]   (row c: the column c of x, element 2j in the low nibble)
 *   scales_t: [K, M/16]
 * Bitwise equal to fos_quantize(transpose(x)) with the same config. Needs
 * M % 16 == 0, K % 16 == 0, K <= 2^24 and M <= 2^23; cfg must be 1x16 with a
 * per-tensor amax [1] (the same global scale as the row-wise operand).
 *   sdec_out: nullable device float[1]. */
int fos_quantize_columnwise(const void* x, int dtype, int64_t M, int64_t K, const float* amax,
                            const fos_config* cfg, uint8_t* codes_t, uint8_t* scales_t, float* sdec_out,
                            void* stream);

/* Per-tensor amax and quantize in one launch: the amax pre-pass that the
 * Megatron-LM PR runs as a separate FP32 torch reduction ("What does this PR
 * do?", fused data path) folded into the quantizer of the pytorch/ao PR
 * (recipe commit). The result equals fos_amax(..., FOS_AMAX_TENSOR) followed
 * by fos_quantize with that amax, bit for bit. cfg must be 1x16.
 * With cfg->scale_gran FOS_PER_ROW (added in ABI version 4) the amax is per
 * row: the result equals fos_amax(..., FOS_AMAX_ROW) followed by
 * fos_quantize with those amaxes; that form has no grid-wide step and does
 * not use the workspace (which must still be passed).
 *   amax_out:  nullable device float[1] (per row: [M]), receives the
 *              NaN-dropping max |x|.
 *   sdec_out:  nullable device float[1] (per row: [M]), receives S_dec.
 *   workspace: device memory of FOS_FUSED_WORKSPACE_BYTES, 8-byte aligned,
 *              all zero before its first use (e.g. cleared once at
 *              allocation). Every completed call leaves its counters zero
 *              again (only the first 256 bytes, a call counter and the last
 *              amax, keep changing), so one workspace serves any number of
 *              calls made one after another; calls that may run at the same time (different
 *              streams) need workspaces of their own.
 *   d_status:  nullable device int32; FOS_STATUS_BARRIER_TIMEOUT is set if
 *              the launch's grid-wide barrier does not complete within the
 *              poll limit (fos_set_barrier_poll_limit; about a second by
 *              default), in which case the codes and scales are incomplete.
 *              That happens only with a workspace that was not zero, or when
 *              other long-running work keeps part of the launch from
 *              becoming resident: the launch holds exactly as many
 *              workgroups as fit on the device at once, so it needs the
 *              whole device to itself (co-residency), and two fused calls
 *              running at the same time on different streams can starve
 *              each other. Pass d_status and check it to detect this; the
 *              Python binding always passes one. */
int fos_quantize_fused(const void* x, int dtype, int64_t M, int64_t K, const fos_config* cfg, uint8_t* codes,
                       uint8_t* scales, float* amax_out, float* sdec_out, void* workspace, int32_t* d_status,
                       void* stream);

/* Per-tensor amax and fused fake quantization in one launch (added in ABI
 * version 4): the amax pre-pass of the Megatron-LM PR's fake-quantization
 * loop ("What does this PR do?": a separate FP32 reduction per weight before
 * the fused data path) folded into fos_qdq. The result equals
 * fos_amax(..., FOS_AMAX_TENSOR) followed by fos_qdq with that amax, bit for
 * bit. cfg must be 1x16 with FOS_PER_TENSOR; x and y are bf16, fp16 or fp32.
 * A tensor that fits on chip (up to 32 M elements of a 16-bit type or 16 M
 * fp32 on a 256-CU device) takes one launch that reads x from memory once;
 * a larger one takes the amax launch and the QDQ launch.
 *   y:         device [M, K] of x's type, 16-byte aligned.
 *   amax_out:  device float[1] (not NULL), receives the NaN-dropping max |x|.
 *   workspace, d_status: as for fos_quantize_fused. */
int fos_qdq_fused(const void* x, int dtype, int64_t M, int64_t K, const fos_config* cfg, void* y, float* amax_out,
                  void* workspace, int32_t* d_status, void* stream);

/* Every tensor's amax and fos_qdq_list in one launch (added in ABI version
 * 5): the Megatron-LM PR's fake-quantization loop computes one FP32 amax per
 * weight before its fused data path ("What does this PR do?"; its
 * "Performance" section times that amax as part of the fused primary); here
 * the amaxes come from the first phase of the list launch itself. The
 * result equals fos_amax(..., FOS_AMAX_TENSOR) of each tensor followed by
 * fos_qdq_list with those amaxes, bit for bit. cfg must be 1x16 with
 * FOS_PER_TENSOR; each descs[i].amax is ignored (may be NULL).
 *   amax_out:  device float[n] (not NULL): amax_out[i] receives tensor i's
 *              NaN-dropping max |x| (+0 for a tensor with no elements).
 *   workspace, d_status: as for fos_quantize_fused. The call shares the
 *              grouped fused call's slots and call counter, so the two may
 *              use one workspace one after the other.
 * One launch takes up to 48 tensors (longer lists take one launch per 48).
 * The launch reads every input twice (amax phase, QDQ phase); the second
 * read comes from the Infinity Cache when the list fits there (256 MB). */
int fos_qdq_list_fused(int n, const fos_tensor_desc* descs, int dtype, const fos_config* cfg, float* amax_out,
                       void* workspace, int32_t* d_status, void* stream);

/* Grouped (MoE) amax and quantize in one launch: the group amaxes that
 * fos_quantize_grouped takes as input (pytorch/ao PR, MoE commit; the
 * Megatron-LM PR's separate amax pre-pass, "What does this PR do?") are
 * computed in the same launch. Group g's amax is the NaN-dropping max |x|
 * over rows [offs[g-1], offs[g]) (0 for an empty group); padding rows at or
 * past offs[G-1] are neither read nor counted. The result equals fos_amax of
 * each group slice followed by fos_quantize_grouped with those amaxes, bit
 * for bit. cfg must be 1x16; cfg->scale_gran is ignored. 1 <= G <=
 * FOS_FUSED_MAX_GROUPS.
 *   offs:           device int32[G], as for fos_quantize_grouped.
 *   group_amax_out: nullable device float[G], receives the group amaxes.
 *   group_sdec_out: nullable device float[G], receives each group's S_dec.
 *   workspace:      as for fos_quantize_fused: FOS_FUSED_WORKSPACE_BYTES,
 *                   zero before its first use, one per stream that may
 *                   overlap. Fused per-tensor and fused grouped calls may
 *                   share it. Grouped calls also keep a call counter and
 *                   two banks of group maxima in it (they alternate; each
 *                   call clears the bank the next one uses).
 *   d_status:       nullable device int32: FOS_STATUS_BAD_OFFS as for
 *                   fos_quantize_grouped, FOS_STATUS_BARRIER_TIMEOUT as for
 *                   fos_quantize_fused.
 * A workspace stays consistent after FOS_STATUS_BARRIER_TIMEOUT: the
 * barrier's last arrival resets its counters and moves the grouped call
 * counter on whether or not other workgroups gave up waiting. */
int fos_quantize_grouped_fused(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                               const fos_config* cfg, uint8_t* codes, uint8_t* scales, float* group_amax_out,
                               float* group_sdec_out, void* workspace, int32_t* d_status, void* stream);

/* fos_quantize_grouped_fused without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The call allocates
 * nothing; the caller still passes every input and output.
 * The workspace is a library-held device array of FOS_FUSED_WORKSPACE_BYTES
 * (16 KiB), one copy per device, held until the process ends. Its address
 * is looked up on the first call on each device (that call, unless its
 * stream is being captured, also clears the array with a fill kernel on
 * `stream`). It holds the grid barrier's counters and the per-group maxima
 * of at most FOS_FUSED_MAX_GROUPS groups: G beyond that returns
 * FOS_ERR_INVALID_ARG and enqueues nothing. Every call on a device shares
 * that device's array and leaves it ready for the next call, so calls that
 * may overlap on one device (different streams) race and must not be made;
 * calls on one stream, or synchronized with each other, are safe.
 * Arguments, results and errors are otherwise those of
 * fos_quantize_grouped_fused (added in ABI version 5). */
int fos_quantize_grouped_fused_noalloc(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs,
                                       int G, const fos_config* cfg, uint8_t* codes, uint8_t* scales,
                                       float* group_amax_out, float* group_sdec_out, int32_t* d_status,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif
