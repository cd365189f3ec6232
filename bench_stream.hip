// bench_stream.hip: streaming kernels that measure the HBM ceiling of the
// quantizer's memory mixes on the device the benchmark runs on. Built into
// libbench_stream.so by __graft_entry__.build(); only bench.py loads it.
//
// They move bytes the way the 1x16 quantizer does, with nothing computed:
// each wave walks its units with 128-bit raw buffer loads (lane l reads
// 16-byte pieces l, l + 64, ... of the unit), two units in flight, and
// writes its share of the output with 128-bit stores. Per unit and lane: R
// loads, W stores, and one more store on the first T lanes. A wave's units
// are either one contiguous range (the quantizer's order) or pairs of
// consecutive units dealt out round robin (wave w takes pairs w, w + nwaves,
// ...), which keeps every wave inside one moving window of the buffers; the
// benchmark takes the faster as the ceiling.
// The mixes:
//   read only              R = 4, W = 0
//   write only             R = 0, W = 4
//   quantize (bf16 / fp16) R = 4, W = 1, T = 8: 4096 B read, 1152 B written
//                          per unit, 2 : 0.5625 as codes and scales are
//   QDQ (bf16 / fp16)      R = 2, W = 2: 1 : 1
// The loaded data feed the stored values (and an XOR kept per lane), so no
// load can be dropped. Stores are non-temporal (the quantizer's outputs are)
// or default-policy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace {

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Rsrc rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

template <int R, int W, int T, int POLICY>
__global__ void __launch_bounds__(256) k_stream(const char* src, char* dst, int64_t units, uint32_t* sink,
                                                int interleave) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t per = (units + nwaves - 1) / nwaves;
  // contiguous: [wave * per, + per) in steps of 2; interleaved: pairs from
  // 2 * wave in steps of 2 * nwaves. A pair is units u and u + 1 < u1.
  const int64_t u0 = interleave ? 2 * wave : wave * per;
  const int64_t u1 = interleave ? units : min(units, u0 + per);
  const int64_t step = interleave ? 2 * nwaves : 2;
  constexpr int64_t kRB = R * 1024, kWB = W * 1024 + T * 16;  // bytes per unit
  v4i acc = {0, 0, 0, 0};
  for (int64_t u = u0; u < u1; u += step) {
    v4i a[R > 0 ? R : 1], b[R > 0 ? R : 1];
    const Rsrc ra = rsrc(src + u * kRB, kRB), rb = rsrc(src + (u + 1) * kRB, u + 1 < u1 ? kRB : 0);
#pragma unroll
    for (int k = 0; k < R; k++) a[k] = __builtin_amdgcn_raw_buffer_load_b128(ra, (k * 64 + lane) * 16, 0, 0);
#pragma unroll
    for (int k = 0; k < R; k++) b[k] = __builtin_amdgcn_raw_buffer_load_b128(rb, (k * 64 + lane) * 16, 0, 0);
    v4i va = {lane, (int)u, 1, 2}, vb = {lane, (int)u + 1, 3, 4};
#pragma unroll
    for (int k = 0; k < R; k++) { va ^= a[k]; vb ^= b[k]; }
    acc ^= va ^ vb;
    if (W + T > 0) {
      const Rsrc wa = rsrc(dst + u * kWB, kWB), wb = rsrc(dst + (u + 1) * kWB, u + 1 < u1 ? kWB : 0);
#pragma unroll
      for (int k = 0; k < W; k++) __builtin_amdgcn_raw_buffer_store_b128(va, wa, (k * 64 + lane) * 16, 0, POLICY);
      if (T) __builtin_amdgcn_raw_buffer_store_b128(va, wa, lane < T ? (W * 64 + lane) * 16 : 0x80000000u, 0, POLICY);
#pragma unroll
      for (int k = 0; k < W; k++) __builtin_amdgcn_raw_buffer_store_b128(vb, wb, (k * 64 + lane) * 16, 0, POLICY);
      if (T) __builtin_amdgcn_raw_buffer_store_b128(vb, wb, lane < T ? (W * 64 + lane) * 16 : 0x80000000u, 0, POLICY);
    }
  }
  const uint32_t x = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (x == 0x9E3779B9u) sink[0] = x;  // keeps the loads; practically never stores
}

template <int R, int W, int T, int POLICY>
int launch(const void* src, void* dst, int64_t units, uint32_t* sink, int interleave, hipStream_t s) {
  auto* fn = &k_stream<R, W, T, POLICY>;
  int dev = 0, cus = 256, per_cu = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || per_cu <= 0) per_cu = 2;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((int64_t)cus * per_cu, (units + 3) / 4));
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const char*>(src), static_cast<char*>(dst),
                     units, sink, interleave);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

extern "C" {

// mix: 0 read only, 1 write only, 2 quantize, 3 QDQ; nt: non-temporal stores;
// interleave: units dealt in pairs round robin rather than as contiguous
// ranges. Bytes per unit: read 4096 / 0 / 4096 / 2048, written 0 / 4096 /
// 1152 / 2048. src and dst must hold units times those bytes.
int stream_bytes_per_unit(int mix, int64_t* read, int64_t* write) {
  static const int64_t r[4] = {4096, 0, 4096, 2048}, w[4] = {0, 4096, 1152, 2048};
  if (mix < 0 || mix > 3) return 1;
  *read = r[mix];
  *write = w[mix];
  return 0;
}

int stream_run(int mix, int nt, int interleave, const void* src, void* dst, int64_t units, uint32_t* sink,
               void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (mix * 2 + (nt ? 1 : 0)) {
    case 0: case 1: return launch<4, 0, 0, 0>(src, dst, units, sink, interleave, s);
    case 2: return launch<0, 4, 0, 0>(src, dst, units, sink, interleave, s);
    case 3: return launch<0, 4, 0, 2>(src, dst, units, sink, interleave, s);
    case 4: return launch<4, 1, 8, 0>(src, dst, units, sink, interleave, s);
    case 5: return launch<4, 1, 8, 2>(src, dst, units, sink, interleave, s);
    case 6: return launch<2, 2, 0, 0>(src, dst, units, sink, interleave, s);
    case 7: return launch<2, 2, 0, 2>(src, dst, units, sink, interleave, s);
    default: return 1;
  }
}

}  // extern "C"
