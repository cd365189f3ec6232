// fos_api.hip: the C ABI of include/fos.h: argument validation, template
// dispatch and launch on the caller's stream. Nothing here allocates memory
// or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <algorithm>

#include "fos.h"
#include "fos_kernels.h"

namespace {

thread_local std::string g_last_error;

// Polls a fused call's grid barrier makes before giving up (process-wide).
std::atomic<int> g_poll_limit{fos::kDefaultSpinLimit};
// the one-read fused kernel's phase timestamps (diagnostics): buffer, waves
std::atomic<unsigned long long*> g_phase_ts{nullptr};
std::atomic<int64_t> g_phase_cap{0};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Largest element count a launch accepts (2^40: far beyond one GPU's HBM,
// and small enough that every index fits int64 with room).
constexpr int64_t kMaxElems = int64_t(1) << 40;

// Grid size: enough workgroups (4 waves each) to cover the work, capped at
// a few per CU so each wave walks a contiguous range.
int grid_for(int64_t waves_wanted) {
  int64_t g = (waves_wanted + 3) / 4;
  const int64_t cap = 256 * 8;  // 256 CUs x 8 workgroups
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

// The current device must be a gfx950 (cached per device ordinal).
int check_device() {
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 ok, 2 bad
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(FOS_ERR_DEVICE, "no current HIP device");
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    if (known[dev] == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(FOS_ERR_DEVICE, "hipGetDeviceProperties failed");
      known[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
      if (known[dev] == 2) return fail(FOS_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    }
    if (known[dev] == 2) return fail(FOS_ERR_DEVICE, "device %d is not gfx950", dev);
  }
  return FOS_OK;
}

int launch_status(hipError_t e) {
  if (e != hipSuccess) return fail(FOS_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return FOS_OK;
}

int check_dtype(int dtype) {
  if (dtype != FOS_BF16 && dtype != FOS_FP16 && dtype != FOS_FP32) return fail(FOS_ERR_DTYPE, "unknown dtype %d", dtype);
  return FOS_OK;
}

int check_cfg(const fos_config* c) {
  if (!c) return fail(FOS_ERR_INVALID_ARG, "cfg is NULL");
  if (c->recipe != FOS_RECIPE_NVFP4 && c->recipe != FOS_RECIPE_4OVER6) return fail(FOS_ERR_INVALID_ARG, "bad recipe %d", c->recipe);
  if (c->block != FOS_BLOCK_1X16 && c->block != FOS_BLOCK_16X16) return fail(FOS_ERR_INVALID_ARG, "bad block %d", c->block);
  if (c->scale_gran != FOS_PER_TENSOR && c->scale_gran != FOS_PER_ROW)
    return fail(FOS_ERR_INVALID_ARG, "bad scale_gran %d", c->scale_gran);
  if (c->err_metric != FOS_ERR_MAE && c->err_metric != FOS_ERR_MSE)
    return fail(FOS_ERR_INVALID_ARG, "bad err_metric %d", c->err_metric);
  if (c->err_prec != FOS_ERR_EXACT && c->err_prec != FOS_ERR_FP16) return fail(FOS_ERR_INVALID_ARG, "bad err_prec %d", c->err_prec);
  if (c->e4m3_bound != 448 && c->e4m3_bound != 256) return fail(FOS_ERR_CONFIG, "e4m3_bound must be 448 or 256, got %d", c->e4m3_bound);
  if (c->err_order != FOS_ORDER_TREE && c->err_order != FOS_ORDER_SEQ)
    return fail(FOS_ERR_INVALID_ARG, "bad err_order %d", c->err_order);
  if (c->err_order == FOS_ORDER_SEQ && c->block != FOS_BLOCK_1X16 && c->recipe == FOS_RECIPE_4OVER6)
    return fail(FOS_ERR_CONFIG, "the sequential error order is defined for 1x16 blocks only");
  return FOS_OK;
}

int check_shape(int64_t M, int64_t K, int block) {
  if (M < 0 || K < 0) return fail(FOS_ERR_INVALID_ARG, "negative size M=%lld K=%lld", (long long)M, (long long)K);
  if (K % 16) return fail(FOS_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (block == FOS_BLOCK_16X16 && M % 16) return fail(FOS_ERR_SHAPE, "16x16 blocks need M %% 16 == 0, M=%lld", (long long)M);
  // a 16x16 unit addresses 16 rows from one base with 32-bit lane offsets
  if (block == FOS_BLOCK_16X16 && K > (int64_t(1) << 24))
    return fail(FOS_ERR_SHAPE, "16x16 blocks need K <= 2^24, K=%lld", (long long)K);
  if (K > 0 && M > kMaxElems / K) return fail(FOS_ERR_SHAPE, "M*K exceeds 2^40 elements");
  return FOS_OK;
}

float six_b(const fos_config* c) { return 6.0f * (float)c->e4m3_bound; }

// the error knobs are ignored by the standard recipe: normalize them so the
// dispatch picks its one instance
void mode_of(const fos_config* c, int& metric, int& prec, int& order) {
  const bool std = c->recipe == FOS_RECIPE_NVFP4;
  metric = std ? FOS_ERR_MSE : c->err_metric;
  prec = std ? FOS_ERR_EXACT : c->err_prec;
  order = std ? FOS_ORDER_TREE : c->err_order;
}

}  // namespace

// The workspace of fos_quantize_grouped_fused_noalloc, held by the library:
// one copy per device (each GPU keeps its own until the process ends), zero
// when the code object loads. Host code never passes this name to a kernel:
// in host code it is a stand-in, not a device address. The device address of
// each GPU's copy comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[FOS_FUSED_WORKSPACE_BYTES];

namespace {

int check_grouped_fused(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                        const fos_config* cfg, uint8_t* codes, uint8_t* scales, float* group_amax_out,
                        float* group_sdec_out, int32_t* d_status);
int launch_grouped_fused(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                         const fos_config* cfg, uint8_t* codes, uint8_t* scales, float* group_amax_out,
                         float* group_sdec_out, void* workspace, int32_t* d_status, void* stream);

// The current device's address of `scratch`, looked up once per device with
// that device current. The first call on a device that is not under stream
// capture also clears it with a fill kernel on `s` (ordered before the call's
// own launch); under capture the load-time zeros stand, since no call has
// used this device's copy yet.
int scratch_address(hipStream_t s, void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(FOS_ERR_DEVICE, "no current HIP device (or ordinal %d >= 64)", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FOS_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) cs = hipStreamCaptureStatusNone;
    if (cs == hipStreamCaptureStatusNone) {
      const hipError_t z = fos::launch_zero_u32(p, FOS_FUSED_WORKSPACE_BYTES / 4, s);
      if (z != hipSuccess) return fail(FOS_ERR_LAUNCH, "clearing the scratch failed: %s", hipGetErrorString(z));
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return FOS_OK;
}

}  // namespace

static_assert(FOS_FUSED_WORKSPACE_BYTES == fos::kFusedWorkspaceBytes, "workspace size mismatch");
static_assert(FOS_FUSED_MAX_GROUPS == fos::kMaxFusedGroups, "group limit mismatch");

extern "C" {

int fos_abi_version(void) { return FOS_ABI_VERSION; }

const char* fos_status_string(int status) {
  switch (status) {
    case FOS_OK: return "ok";
    case FOS_ERR_INVALID_ARG: return "invalid argument";
    case FOS_ERR_DTYPE: return "unsupported element type";
    case FOS_ERR_SHAPE: return "unsupported shape";
    case FOS_ERR_ALIGN: return "misaligned pointer";
    case FOS_ERR_CONFIG: return "unsupported configuration";
    case FOS_ERR_DEVICE: return "device error";
    case FOS_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* fos_last_error(void) { return g_last_error.c_str(); }

int fos_set_barrier_poll_limit(int polls) {
  if (polls < 0) return -1;
  return g_poll_limit.exchange(polls, std::memory_order_relaxed);
}

int fos_set_phase_timestamps(unsigned long long* d_buf, int64_t max_waves, int* clock_khz) {
  if (d_buf && (max_waves < 0 || !aligned(d_buf, 8))) return fail(FOS_ERR_INVALID_ARG, "bad timestamp buffer");
  if (clock_khz) {
    int dev = 0, khz = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) khz = 0;
    *clock_khz = khz;
  }
  g_phase_cap.store(d_buf ? max_waves : 0, std::memory_order_relaxed);
  g_phase_ts.store(d_buf, std::memory_order_relaxed);
  return FOS_OK;
}

int fos_amax(const void* x, int dtype, int64_t M, int64_t K, int gran, float* amax_out, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if (gran != FOS_AMAX_TENSOR && gran != FOS_AMAX_ROW && gran != FOS_AMAX_BAND16)
    return fail(FOS_ERR_INVALID_ARG, "bad amax granularity %d", gran);
  if ((rc = check_shape(M, K, gran == FOS_AMAX_BAND16 ? FOS_BLOCK_16X16 : FOS_BLOCK_1X16))) return rc;
  if (!amax_out) return fail(FOS_ERR_INVALID_ARG, "amax_out is NULL");
  if (!aligned(amax_out, 4)) return fail(FOS_ERR_ALIGN, "amax_out not 4-byte aligned");
  if (M * K > 0 && !x) return fail(FOS_ERR_INVALID_ARG, "x is NULL");
  if (x && !aligned(x, 16)) return fail(FOS_ERR_ALIGN, "x not 16-byte aligned");
  if ((rc = check_device())) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (gran != FOS_AMAX_TENSOR && M == 0) return FOS_OK;
  if (M * K == 0)  // no elements: every amax is +0
    return launch_status(fos::launch_zero_u32(amax_out, gran == FOS_AMAX_TENSOR ? 1 : M, s));
  const int64_t n16 = M * K / 16;
  // per tensor: at most 256 workgroups, so that their same-address atomics
  // (which serialize at the memory side) stay few
  int grid = gran == FOS_AMAX_TENSOR ? (int)std::max<int64_t>(1, std::min<int64_t>(256, (n16 + 1023) / 1024))
                                     : grid_for(M);
  return launch_status(fos::launch_amax(dtype, gran, x, M, K, amax_out, grid, s));
}

int fos_quantize(const void* x, int dtype, int64_t M, int64_t K, const float* amax, const fos_config* cfg,
                 uint8_t* codes, uint8_t* scales, float* sdec_out, int32_t* d_status, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_cfg(cfg))) return rc;
  if ((rc = check_shape(M, K, cfg->block))) return rc;
  if (!amax) return fail(FOS_ERR_INVALID_ARG, "amax is NULL");
  if (M * K > 0 && (!x || !codes || !scales)) return fail(FOS_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if (!aligned(x, 16)) return fail(FOS_ERR_ALIGN, "x not 16-byte aligned");
  if (!aligned(codes, 8)) return fail(FOS_ERR_ALIGN, "codes not 8-byte aligned");
  if (!aligned(amax, 4) || !aligned(sdec_out, 4) || !aligned(d_status, 4)) return fail(FOS_ERR_ALIGN, "amax/sdec/status misaligned");
  if ((rc = check_device())) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int metric, prec, order;
  mode_of(cfg, metric, prec, order);
  const bool per_row = cfg->scale_gran == FOS_PER_ROW;
  // the kernels also write S_dec; with no elements only S_dec remains
  if (M * K == 0 && !(sdec_out && (per_row ? M : 1) > 0)) return FOS_OK;
  if (cfg->block == FOS_BLOCK_1X16) {
    fos::Args1x16<1> a;
    memset(&a, 0, sizeof a);
    a.t[0] = fos::TensorRef{x, nullptr, amax, M, K > 0 ? K : 16, 0};
    a.n = 1;
    // units: 64 blocks of the flattened tensor, or per-row segments of up to
    // 64 blocks (one global scale per unit)
    const int64_t ub = fos::unit_blocks(fos::kOutQuant, dtype);
    a.total_units = per_row ? M * ((K / 16 + ub - 1) / ub) : (M * (K / 16) + ub - 1) / ub;
    a.six_b = six_b(cfg);
    a.codes = codes;
    a.scales = scales;
    a.sdec_out = sdec_out;
    return launch_status(fos::launch_quant_1x16(dtype, cfg->recipe, metric, prec, order,
                                                per_row ? fos::kGranRow : fos::kGranTensor, a, s));
  }
  fos::Args16x16 a;
  a.x = x;
  a.y = nullptr;
  a.amax = amax;
  a.M = M;
  a.K = K;
  a.six_b = six_b(cfg);
  a.codes = codes;
  a.scales = scales;
  a.sdec_out = sdec_out;
  a.status = d_status;
  return launch_status(fos::launch_16x16(dtype, cfg->recipe, metric, prec,
                                         per_row ? fos::kGranRow : fos::kGranTensor, fos::kOutQuant, a, s));
}

int fos_qdq_list(int n, const fos_tensor_desc* descs, int dtype, const fos_config* cfg, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (n < 0) return fail(FOS_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && !descs) return fail(FOS_ERR_INVALID_ARG, "descs is NULL");
  for (int i = 0; i < n; i++) {
    const fos_tensor_desc& d = descs[i];
    if ((rc = check_shape(d.M, d.K, cfg->block))) return fail(rc, "tensor %d: %s", i, g_last_error.c_str());
    if (!d.amax) return fail(FOS_ERR_INVALID_ARG, "tensor %d: amax is NULL", i);
    if (d.M * d.K > 0 && (!d.x || !d.y)) return fail(FOS_ERR_INVALID_ARG, "tensor %d: x/y is NULL", i);
    if (!aligned(d.x, 16) || !aligned(d.y, 16)) return fail(FOS_ERR_ALIGN, "tensor %d: x/y not 16-byte aligned", i);
    if (!aligned(d.amax, 4)) return fail(FOS_ERR_ALIGN, "tensor %d: amax misaligned", i);
  }
  if ((rc = check_device())) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int metric, prec, order;
  mode_of(cfg, metric, prec, order);
  const bool per_row = cfg->scale_gran == FOS_PER_ROW;
  const int gran = per_row ? fos::kGranRow : fos::kGranTensor;
  if (cfg->block == FOS_BLOCK_16X16) {
    // one 16x16 launch per tensor
    for (int i = 0; i < n; i++) {
      const fos_tensor_desc& d = descs[i];
      if (d.M * d.K == 0) continue;
      fos::Args16x16 a;
      memset(&a, 0, sizeof a);
      a.x = d.x;
      a.y = d.y;
      a.amax = d.amax;
      a.M = d.M;
      a.K = d.K;
      a.six_b = six_b(cfg);
      if ((rc = launch_status(fos::launch_16x16(dtype, cfg->recipe, metric, prec, gran, fos::kOutQdq, a, s))))
        return rc;
    }
    return FOS_OK;
  }
  const int64_t ub = fos::unit_blocks(fos::kOutQdq, dtype);
  int i = 0;
  while (i < n) {
    fos::Args1x16<fos::kMaxList> a;
    memset(&a, 0, sizeof a);
    int64_t units = 0;
    for (; i < n && a.n < fos::kMaxList; i++) {
      const fos_tensor_desc& d = descs[i];
      if (d.M * d.K == 0) continue;
      a.t[a.n++] = fos::TensorRef{d.x, d.y, d.amax, d.M, d.K, units};
      // units: 64 blocks of the flattened tensor, or per-row segments
      units += per_row ? d.M * ((d.K / 16 + ub - 1) / ub) : (d.M * (d.K / 16) + ub - 1) / ub;
    }
    if (a.n == 0) continue;
    a.total_units = units;
    a.six_b = six_b(cfg);
    if ((rc = launch_status(fos::launch_qdq_1x16(dtype, cfg->recipe, metric, prec, order, gran, a, s)))) return rc;
  }
  return FOS_OK;
}

int fos_qdq_list_fused(int n, const fos_tensor_desc* descs, int dtype, const fos_config* cfg, float* amax_out,
                       void* workspace, int32_t* d_status, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (cfg->block != FOS_BLOCK_1X16 || cfg->scale_gran != FOS_PER_TENSOR)
    return fail(FOS_ERR_CONFIG, "fused amaxes + QDQ list supports 1x16 blocks with a per-tensor scale");
  if (n < 0) return fail(FOS_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && !descs) return fail(FOS_ERR_INVALID_ARG, "descs is NULL");
  if (n > 0 && !amax_out) return fail(FOS_ERR_INVALID_ARG, "amax_out must be non-NULL");
  if (!workspace) return fail(FOS_ERR_INVALID_ARG, "workspace must be non-NULL");
  if (!aligned(amax_out, 4) || !aligned(workspace, 8) || !aligned(d_status, 4))
    return fail(FOS_ERR_ALIGN, "amax_out/workspace/status misaligned");
  for (int i = 0; i < n; i++) {
    const fos_tensor_desc& d = descs[i];
    if ((rc = check_shape(d.M, d.K, FOS_BLOCK_1X16))) return fail(rc, "tensor %d: %s", i, g_last_error.c_str());
    if (d.M * d.K > 0 && (!d.x || !d.y)) return fail(FOS_ERR_INVALID_ARG, "tensor %d: x/y is NULL", i);
    if (!aligned(d.x, 16) || !aligned(d.y, 16)) return fail(FOS_ERR_ALIGN, "tensor %d: x/y not 16-byte aligned", i);
  }
  if ((rc = check_device())) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int metric, prec, order;
  mode_of(cfg, metric, prec, order);
  const int64_t ub = fos::unit_blocks(fos::kOutQdq, dtype);
  int i = 0;
  while (i < n) {
    fos::Args1x16<fos::kMaxList> a;
    memset(&a, 0, sizeof a);
    int64_t units = 0;
    for (; i < n && a.n < fos::kMaxList; i++) {
      const fos_tensor_desc& d = descs[i];
      if (d.M * d.K == 0) {  // no elements: the amax is +0
        if ((rc = launch_status(fos::launch_zero_u32(amax_out + i, 1, s)))) return rc;
        continue;
      }
      a.t[a.n++] = fos::TensorRef{d.x, d.y, nullptr, d.M, d.K, units, amax_out + i};
      units += (d.M * (d.K / 16) + ub - 1) / ub;  // 64 blocks of the flattened tensor
    }
    if (a.n == 0) continue;
    a.total_units = units;
    a.six_b = six_b(cfg);
    a.status = d_status;
    a.spin_limit = g_poll_limit.load(std::memory_order_relaxed);
    if ((rc = launch_status(fos::launch_fused_list(dtype, cfg->recipe, metric, prec, order, a,
                                                   static_cast<uint32_t*>(workspace), s))))
      return rc;
  }
  return FOS_OK;
}

int fos_qdq(const void* x, int dtype, int64_t M, int64_t K, const float* amax, const fos_config* cfg, void* y,
            void* stream) {
  fos_tensor_desc d{x, y, amax, M, K};
  return fos_qdq_list(1, &d, dtype, cfg, stream);
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t M, int64_t K, const float* sdec,
                     int scale_gran, int out_dtype, void* y, void* stream) {
  int rc;
  if ((rc = check_dtype(out_dtype))) return rc;
  if (scale_gran != FOS_PER_TENSOR && scale_gran != FOS_PER_ROW) return fail(FOS_ERR_INVALID_ARG, "bad scale_gran %d", scale_gran);
  if ((rc = check_shape(M, K, FOS_BLOCK_1X16))) return rc;
  if (M * K > 0 && (!codes || !scales || !sdec || !y)) return fail(FOS_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(codes, 8) || !aligned(y, 16) || !aligned(sdec, 4)) return fail(FOS_ERR_ALIGN, "misaligned pointer");
  if ((rc = check_device())) return rc;
  if (M * K == 0) return FOS_OK;
  return launch_status(fos::launch_dequant(out_dtype, scale_gran == FOS_PER_ROW ? fos::kGranRow : fos::kGranTensor,
                                           codes, scales, sdec, M, K, y, static_cast<hipStream_t>(stream)));
}

int fos_quantize_grouped(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                         const float* group_amax, const fos_config* cfg, uint8_t* codes, uint8_t* scales,
                         float* group_sdec_out, int32_t* d_status, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (cfg->block != FOS_BLOCK_1X16) return fail(FOS_ERR_CONFIG, "grouped quantize supports 1x16 blocks");
  if ((rc = check_shape(M_alloc, K, FOS_BLOCK_1X16))) return rc;
  if (G <= 0) return fail(FOS_ERR_INVALID_ARG, "G must be positive, got %d", G);
  if (!offs || !group_amax) return fail(FOS_ERR_INVALID_ARG, "offs and group_amax must be non-NULL");
  if (M_alloc * K > 0 && (!x || !codes || !scales)) return fail(FOS_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if (!aligned(x, 16) || !aligned(codes, 8)) return fail(FOS_ERR_ALIGN, "x or codes misaligned");
  if (!aligned(offs, 4) || !aligned(group_amax, 4) || !aligned(group_sdec_out, 4) || !aligned(d_status, 4))
    return fail(FOS_ERR_ALIGN, "offs/amax/sdec/status misaligned");
  if ((rc = check_device())) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int metric, prec, order;
  mode_of(cfg, metric, prec, order);
  fos::Args1x16<1> a;
  memset(&a, 0, sizeof a);
  a.t[0] = fos::TensorRef{x, nullptr, nullptr, M_alloc, K > 0 ? K : 16, 0};
  a.n = 1;
  a.G = G;
  const int64_t ub = fos::unit_blocks(fos::kOutQuant, dtype);
  a.total_units = fos::grouped_units(M_alloc, a.t[0].K, ub);
  a.six_b = six_b(cfg);
  a.codes = codes;
  a.scales = scales;
  a.sdec_out = group_sdec_out;
  a.status = d_status;
  a.offs = offs;
  a.group_amax = group_amax;
  return launch_status(fos::launch_quant_1x16(dtype, cfg->recipe, metric, prec, order, fos::kGranGroup, a, s));
}

int fos_quantize_columnwise(const void* x, int dtype, int64_t M, int64_t K, const float* amax,
                            const fos_config* cfg, uint8_t* codes_t, uint8_t* scales_t, float* sdec_out,
                            void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (cfg->block != FOS_BLOCK_1X16 || cfg->scale_gran != FOS_PER_TENSOR)
    return fail(FOS_ERR_CONFIG, "columnwise quantize supports 1x16 blocks with a per-tensor amax");
  if ((rc = check_shape(M, K, FOS_BLOCK_16X16))) return rc;  // M % 16, K % 16, K <= 2^24
  if (M > (int64_t(1) << 23)) return fail(FOS_ERR_SHAPE, "columnwise quantize needs M <= 2^23, M=%lld", (long long)M);
  if (!amax) return fail(FOS_ERR_INVALID_ARG, "amax is NULL");
  if (M * K > 0 && (!x || !codes_t || !scales_t)) return fail(FOS_ERR_INVALID_ARG, "x, codes_t and scales_t must be non-NULL");
  if (!aligned(x, 16) || !aligned(codes_t, 8)) return fail(FOS_ERR_ALIGN, "x or codes_t misaligned");
  if (!aligned(amax, 4) || !aligned(sdec_out, 4)) return fail(FOS_ERR_ALIGN, "amax/sdec misaligned");
  if ((rc = check_device())) return rc;
  if (M * K == 0 && !sdec_out) return FOS_OK;
  int metric, prec, order;
  mode_of(cfg, metric, prec, order);
  fos::Args16x16 a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.amax = amax;
  a.M = M;
  a.K = K;
  a.six_b = six_b(cfg);
  a.codes = codes_t;
  a.scales = scales_t;
  a.sdec_out = sdec_out;
  return launch_status(fos::launch_colwise(dtype, cfg->recipe, metric, prec, order, a, static_cast<hipStream_t>(stream)));
}

int fos_quantize_fused(const void* x, int dtype, int64_t M, int64_t K, const fos_config* cfg, uint8_t* codes,
                       uint8_t* scales, float* amax_out, float* sdec_out, void* workspace, int32_t* d_status,
                       void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (cfg->block != FOS_BLOCK_1X16)
    return fail(FOS_ERR_CONFIG, "fused amax + quantize supports 1x16 blocks");
  if ((rc = check_shape(M, K, FOS_BLOCK_1X16))) return rc;
  if (M * K > 0 && (!x || !codes || !scales)) return fail(FOS_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if (!workspace) return fail(FOS_ERR_INVALID_ARG, "workspace must be non-NULL");
  if (!aligned(x, 16) || !aligned(codes, 8)) return fail(FOS_ERR_ALIGN, "x or codes misaligned");
  if (!aligned(workspace, 8) || !aligned(amax_out, 4) || !aligned(sdec_out, 4) || !aligned(d_status, 4))
    return fail(FOS_ERR_ALIGN, "workspace/amax/sdec/status misaligned");
  if ((rc = check_device())) return rc;
  int metric, prec, order;
  mode_of(cfg, metric, prec, order);
  fos::Args1x16<1> a;
  memset(&a, 0, sizeof a);
  a.t[0] = fos::TensorRef{x, nullptr, nullptr, M, K > 0 ? K : 16, 0};
  a.n = 1;
  const int64_t ub = fos::unit_blocks(fos::kOutQuant, dtype);
  a.six_b = six_b(cfg);
  a.codes = codes;
  a.scales = scales;
  a.sdec_out = sdec_out;
  a.status = d_status;
  a.spin_limit = g_poll_limit.load(std::memory_order_relaxed);
  a.phase_ts = g_phase_ts.load(std::memory_order_relaxed);
  a.phase_cap = g_phase_cap.load(std::memory_order_relaxed);
  if (cfg->scale_gran == FOS_PER_ROW) {  // per-row segments, one wave per row at a time
    a.total_units = M * ((a.t[0].K / 16 + ub - 1) / ub);
    return launch_status(fos::launch_fused_row(dtype, cfg->recipe, metric, prec, order, a, amax_out,
                                               static_cast<hipStream_t>(stream)));
  }
  a.total_units = (M * (K / 16) + ub - 1) / ub;
  return launch_status(fos::launch_fused(dtype, cfg->recipe, metric, prec, order, a, static_cast<uint32_t*>(workspace),
                                         amax_out, static_cast<hipStream_t>(stream)));
}

int fos_qdq_fused(const void* x, int dtype, int64_t M, int64_t K, const fos_config* cfg, void* y, float* amax_out,
                  void* workspace, int32_t* d_status, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (cfg->block != FOS_BLOCK_1X16 || cfg->scale_gran != FOS_PER_TENSOR)
    return fail(FOS_ERR_CONFIG, "fused amax + QDQ supports 1x16 blocks with a per-tensor scale");
  if ((rc = check_shape(M, K, FOS_BLOCK_1X16))) return rc;
  if (M * K > 0 && (!x || !y)) return fail(FOS_ERR_INVALID_ARG, "x and y must be non-NULL");
  if (!amax_out) return fail(FOS_ERR_INVALID_ARG, "amax_out must be non-NULL");
  if (!workspace) return fail(FOS_ERR_INVALID_ARG, "workspace must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(FOS_ERR_ALIGN, "x or y misaligned");
  if (!aligned(workspace, 8) || !aligned(amax_out, 4) || !aligned(d_status, 4))
    return fail(FOS_ERR_ALIGN, "workspace/amax/status misaligned");
  if ((rc = check_device())) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int metric, prec, order;
  mode_of(cfg, metric, prec, order);
  fos::Args1x16<1> a;
  memset(&a, 0, sizeof a);
  a.t[0] = fos::TensorRef{x, y, nullptr, M, K > 0 ? K : 16, 0};
  a.n = 1;
  const int64_t ub = fos::unit_blocks(fos::kOutQdq, dtype);
  a.total_units = (M * (K / 16) + ub - 1) / ub;
  a.six_b = six_b(cfg);
  a.status = d_status;
  a.spin_limit = g_poll_limit.load(std::memory_order_relaxed);
  a.phase_ts = g_phase_ts.load(std::memory_order_relaxed);
  a.phase_cap = g_phase_cap.load(std::memory_order_relaxed);
  bool done = false;
  if ((rc = launch_status(fos::launch_fused_qdq(dtype, cfg->recipe, metric, prec, order, a,
                                                static_cast<uint32_t*>(workspace), amax_out, &done, s))))
    return rc;
  if (done) return FOS_OK;
  // too large for one read: the amax, then the QDQ with it
  if ((rc = fos_amax(x, dtype, M, K, FOS_AMAX_TENSOR, amax_out, stream))) return rc;
  return fos_qdq(x, dtype, M, K, amax_out, cfg, y, stream);
}

int fos_quantize_grouped_fused(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                               const fos_config* cfg, uint8_t* codes, uint8_t* scales, float* group_amax_out,
                               float* group_sdec_out, void* workspace, int32_t* d_status, void* stream) {
  int rc;
  if ((rc = check_grouped_fused(x, dtype, M_alloc, K, offs, G, cfg, codes, scales, group_amax_out, group_sdec_out,
                                d_status)))
    return rc;
  if (!workspace) return fail(FOS_ERR_INVALID_ARG, "workspace must be non-NULL");
  if (!aligned(workspace, 8)) return fail(FOS_ERR_ALIGN, "workspace misaligned");
  if ((rc = check_device())) return rc;
  return launch_grouped_fused(x, dtype, M_alloc, K, offs, G, cfg, codes, scales, group_amax_out, group_sdec_out,
                              workspace, d_status, stream);
}

int fos_quantize_grouped_fused_noalloc(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs,
                                       int G, const fos_config* cfg, uint8_t* codes, uint8_t* scales,
                                       float* group_amax_out, float* group_sdec_out, int32_t* d_status,
                                       void* stream) {
  if (G > FOS_FUSED_MAX_GROUPS)
    return fail(FOS_ERR_INVALID_ARG, "G=%d exceeds the %d groups the library-held scratch holds", G,
                FOS_FUSED_MAX_GROUPS);
  // argument checks first, so that a rejected call touches no device state
  int rc;
  if ((rc = check_grouped_fused(x, dtype, M_alloc, K, offs, G, cfg, codes, scales, group_amax_out, group_sdec_out,
                                d_status)))
    return rc;
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(static_cast<hipStream_t>(stream), &ws))) return rc;
  return launch_grouped_fused(x, dtype, M_alloc, K, offs, G, cfg, codes, scales, group_amax_out, group_sdec_out, ws,
                              d_status, stream);
}

}  // extern "C"

namespace {

int check_grouped_fused(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                        const fos_config* cfg, uint8_t* codes, uint8_t* scales, float* group_amax_out,
                        float* group_sdec_out, int32_t* d_status) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (cfg->block != FOS_BLOCK_1X16) return fail(FOS_ERR_CONFIG, "grouped quantize supports 1x16 blocks");
  if ((rc = check_shape(M_alloc, K, FOS_BLOCK_1X16))) return rc;
  if (G <= 0 || G > FOS_FUSED_MAX_GROUPS)
    return fail(FOS_ERR_INVALID_ARG, "G must be in [1, %d], got %d", FOS_FUSED_MAX_GROUPS, G);
  if (!offs) return fail(FOS_ERR_INVALID_ARG, "offs must be non-NULL");
  if (M_alloc * K > 0 && (!x || !codes || !scales)) return fail(FOS_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if (!aligned(x, 16) || !aligned(codes, 8)) return fail(FOS_ERR_ALIGN, "x or codes misaligned");
  if (!aligned(offs, 4) || !aligned(group_amax_out, 4) || !aligned(group_sdec_out, 4) || !aligned(d_status, 4))
    return fail(FOS_ERR_ALIGN, "offs/amax/sdec/status misaligned");
  return FOS_OK;
}

int launch_grouped_fused(const void* x, int dtype, int64_t M_alloc, int64_t K, const int32_t* offs, int G,
                         const fos_config* cfg, uint8_t* codes, uint8_t* scales, float* group_amax_out,
                         float* group_sdec_out, void* workspace, int32_t* d_status, void* stream) {
  int metric, prec, order;
  mode_of(cfg, metric, prec, order);
  fos::Args1x16<1> a;
  memset(&a, 0, sizeof a);
  a.t[0] = fos::TensorRef{x, nullptr, nullptr, M_alloc, K > 0 ? K : 16, 0};
  a.n = 1;
  a.G = G;
  const int64_t ub = fos::unit_blocks(fos::kOutQuant, dtype);
  a.total_units = fos::grouped_units(M_alloc, a.t[0].K, ub);
  a.six_b = six_b(cfg);
  a.codes = codes;
  a.scales = scales;
  a.sdec_out = group_sdec_out;
  a.status = d_status;
  a.spin_limit = g_poll_limit.load(std::memory_order_relaxed);
  a.offs = offs;
  return launch_status(fos::launch_fused_grouped(dtype, cfg->recipe, metric, prec, order, a,
                                                 static_cast<uint32_t*>(workspace), group_amax_out,
                                                 static_cast<hipStream_t>(stream)));
}

}  // namespace
