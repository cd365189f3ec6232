// fos_kernels.h: launch interface between the C ABI (fos_api.hip) and the
// gfx950 kernels (fos_kernels.hip). Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fos {

// numbering matches include/fos.h
enum { kBF16 = 0, kFP16 = 1, kFP32 = 2 };
enum { kNVFP4 = 0, k4over6 = 1 };
enum { kMAE = 0, kMSE = 1 };
enum { kErrExact = 0, kErrFP16 = 1 };
enum { kOrderTree = 0, kOrderSeq = 1 };
enum { kGranTensor = 0, kGranRow = 1, kGranGroup = 2 };
enum { kOutQuant = 0, kOutQdq = 1 };
enum { kAmaxTensor = 0, kAmaxRow = 1, kAmaxBand16 = 2 };
enum { kStatusTileNonuniform = 1, kStatusBadOffs = 2, kStatusBarrier = 4 };

// Polls of the fused kernels' grid barrier before a workgroup gives up
// (each poll sleeps at least 128 cycles first): about a second.
constexpr int kDefaultSpinLimit = 1 << 20;

// Bytes of the fused kernels' workspace (the grid barrier's counters and
// the grouped kernel's per-group maxima), and the most groups the fused
// grouped kernel takes.
constexpr int kFusedWorkspaceBytes = 16384;
constexpr int kMaxFusedGroups = 256;

// Tensors per launch of the list kernel (the descriptors travel in the
// kernel arguments, 48 B each).
constexpr int kMaxList = 48;

// 16-element blocks per lane in one unit of the 1x16 kernels: a unit is
// 64 * NB consecutive blocks of a row (per-row and grouped scales) or of the
// flattened tensor (per-tensor scale). Quantizing 16-bit inputs keeps two
// blocks per lane in flight; fp32 inputs (twice the registers per block) and
// the fused QDQ (which holds decoded values too) keep one.
__host__ __device__ constexpr int unit_blocks(int out, int dt) {
  return 64 * ((out == kOutQuant && dt != kFP32) ? 2 : 1);
}

// Units of a grouped launch. A 16-row band holds K blocks and group offsets
// are multiples of 16 rows, so when K is a multiple of the unit size every
// group (and the padding tail) is a whole number of units: units then run
// flat over the tensor, crossing rows but never groups, and no lane idles at
// a row's end. Otherwise a unit is a segment of one row.
__host__ __device__ constexpr bool grouped_flat(int64_t K, int64_t ub) { return K % ub == 0; }
__host__ __device__ constexpr int64_t grouped_units(int64_t M, int64_t K, int64_t ub) {
  return grouped_flat(K, ub) ? (M * (K / 16) + ub - 1) / ub : M * ((K / 16 + ub - 1) / ub);
}

// One tensor of a 1x16 launch. unit_begin: index of its first 64-block unit
// in the launch's unit space.
struct TensorRef {
  const void* x;
  void* y;
  const float* amax;
  int64_t M, K;
  int64_t unit_begin;
  float* amax_out;  // fused list: receives the tensor's amax (nullable)
};

template <int NT>
struct Args1x16 {
  TensorRef t[NT];
  int n;            // tensors in t
  int G;            // groups (grouped launch)
  int64_t total_units;
  float six_b;      // 6 * E4M3 bound
  uint8_t* codes;   // quantize outputs (single tensor)
  uint8_t* scales;
  float* sdec_out;  // nullable: S_dec per tensor [1], row [M] or group [G]
  int32_t* status;  // nullable device status word
  const int32_t* offs;       // grouped: cumulative end offsets [G]
  const float* group_amax;   // grouped: [G]
  int spin_limit;            // fused calls: polls before the grid barrier gives up
  // nullable: the one-read fused kernel's per-wave phase timestamps (4 per
  // wave, for waves below phase_cap)
  unsigned long long* phase_ts;
  int64_t phase_cap;
};

struct Args16x16 {
  const void* x;
  void* y;
  const float* amax;
  int64_t M, K;
  float six_b;
  uint8_t* codes;
  uint8_t* scales;
  float* sdec_out;  // nullable: S_dec per tensor [1] or row [M]
  int32_t* status;
};

hipError_t launch_quant_1x16(int dt, int recipe, int metric, int prec, int order, int gran, const Args1x16<1>& a,
                             hipStream_t s);
hipError_t launch_fused(int dt, int recipe, int metric, int prec, int order, const Args1x16<1>& a, uint32_t* ws,
                        float* amax_out, hipStream_t s);
hipError_t launch_fused_row(int dt, int recipe, int metric, int prec, int order, const Args1x16<1>& a,
                            float* amax_out, hipStream_t s);
hipError_t launch_fused_qdq(int dt, int recipe, int metric, int prec, int order, const Args1x16<1>& a, uint32_t* ws,
                            float* amax_out, bool* done, hipStream_t s);
hipError_t launch_fused_grouped(int dt, int recipe, int metric, int prec, int order, const Args1x16<1>& a,
                                uint32_t* ws, float* amax_out, hipStream_t s);
hipError_t launch_qdq_1x16(int dt, int recipe, int metric, int prec, int order, int gran,
                           const Args1x16<kMaxList>& a, hipStream_t s);
hipError_t launch_fused_list(int dt, int recipe, int metric, int prec, int order, const Args1x16<kMaxList>& a,
                             uint32_t* ws, hipStream_t s);
hipError_t launch_colwise(int dt, int recipe, int metric, int prec, int order, const Args16x16& a, hipStream_t s);
hipError_t launch_16x16(int dt, int recipe, int metric, int prec, int gran, int out, const Args16x16& a,
                        hipStream_t s);
hipError_t launch_dequant(int dt, int gran, const uint8_t* codes, const uint8_t* scales, const float* sdec,
                          int64_t M, int64_t K, void* y, hipStream_t s);
hipError_t launch_amax(int dt, int gran, const void* x, int64_t M, int64_t K, float* out, int grid, hipStream_t s);
hipError_t launch_zero_u32(void* p, int64_t n, hipStream_t s);

}  // namespace fos
