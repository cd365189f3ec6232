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
enum { kGranTensor = 0, kGranRow = 1, kGranGroup = 2 };
enum { kOutQuant = 0, kOutQdq = 1 };
enum { kAmaxTensor = 0, kAmaxRow = 1, kAmaxBand16 = 2 };
enum { kStatusTileNonuniform = 1, kStatusBadOffs = 2 };

// Tensors per launch of the list kernel (the descriptors travel in the
// kernel arguments, 48 B each).
constexpr int kMaxList = 48;

// One tensor of a 1x16 launch. unit_begin: index of its first 64-block unit
// in the launch's unit space.
struct TensorRef {
  const void* x;
  void* y;
  const float* amax;
  int64_t M, K;
  int64_t unit_begin;
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
  const int32_t* offs;       // grouped: cumulative end offsets [G]
  const float* group_amax;   // grouped: [G]
};

struct Args16x16 {
  const void* x;
  void* y;
  const float* amax;
  int64_t M, K;
  float six_b;
  uint8_t* codes;
  uint8_t* scales;
  int32_t* status;
};

hipError_t launch_quant_1x16(int dt, int recipe, int metric, int prec, int gran, const Args1x16<1>& a, int grid,
                             hipStream_t s);
hipError_t launch_qdq_1x16(int dt, int recipe, int metric, int prec, const Args1x16<kMaxList>& a, int grid,
                           hipStream_t s);
hipError_t launch_quant_16x16(int dt, int recipe, int metric, int prec, int gran, const Args16x16& a, int grid,
                              hipStream_t s);
hipError_t launch_dequant(int dt, int gran, const uint8_t* codes, const uint8_t* scales, const float* sdec,
                          int64_t M, int64_t K, void* y, int grid, hipStream_t s);
hipError_t launch_amax(int dt, int gran, const void* x, int64_t M, int64_t K, float* out, int grid, hipStream_t s);
hipError_t launch_sdec(const float* amax, int64_t n, float six_b, float* out, hipStream_t s);
hipError_t launch_zero_u32(void* p, int64_t n, hipStream_t s);
hipError_t launch_check_offs(const int32_t* offs, int G, int64_t M_alloc, int32_t* status, hipStream_t s);

}  // namespace fos
