// gpu_primitives.hip: test kernels that run the quantizer's own device
// helpers (nvfp4_adaptive_block_amd/csrc/fos_device.h, built with the
// library's flags) over every input they can be fed, so that the test suite
// can compare each result bitwise with the CPU's IEEE arithmetic and the
// oracle's format conversions. This is what admits the gfx950 convert
// instructions and the FMA-corrected division by 6 into the kernels: the
// rounding-critical steps the wolfcomos/ao PR "Add a CuTe DSL fast-path
// kernel for four-over-six quantize" names (correctly rounded FP32 division,
// the FP4/E4M3 casts and their decodes).
//
// Inputs are enumerated from an index (binary32 patterns base + i, or pairs
// of 16-bit patterns), so nothing but the outputs crosses to the host. Every
// launcher takes device pointers, sizes and a stream; each grid covers
// exactly n items, with a bounds check per thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fos_device.h"

namespace {

constexpr int kBlock = 256;

unsigned grid_for(int64_t items) { return (unsigned)((items + kBlock - 1) / kBlock); }

// E2M1 encode of the 8 binary32 patterns base + 8 t .. base + 8 t + 7
__global__ void k_e2m1_encode(uint32_t base, int64_t nwords, uint32_t* out) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= nwords) return;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; k++) v[k] = __uint_as_float(base + (uint32_t)(8 * t + k));
  out[t] = fos::e2m1_pack8(v);
}

// E2M1 decode of code words
__global__ void k_e2m1_decode(const uint32_t* in, int64_t nwords, float* out) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= nwords) return;
  float q[8];
  fos::e2m1_unpack8(in[t], q);
#pragma unroll
  for (int k = 0; k < 8; k++) out[8 * t + k] = q[k];
}

// E4M3 code of the binary32 pattern base + i (low byte), and the OR of the
// word's upper bytes over the grid (the kernels use the word unmasked)
__global__ void k_e4m3_encode(uint32_t base, int64_t n, uint8_t* out, uint32_t* upper_or) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = fos::e4m3_code(__uint_as_float(base + (uint32_t)i));
  out[i] = (uint8_t)(w & 0xFFu);
  if (w >> 8) atomicOr(upper_or, w >> 8);
}

__global__ void k_e4m3_decode(int n, float* out) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i < n) out[i] = fos::e4m3_value((uint32_t)i);
}

// RN(a / 6) as the kernels take it, a = the binary32 pattern base + i
__global__ void k_div6(uint32_t base, int64_t n, float* out) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const float a = __uint_as_float(base + (uint32_t)(i < n ? i : 0));
  const float q = fos::div6(a);  // every lane of the wave takes part (the helper votes)
  if (i < n) out[i] = q;
}

// Global scales of A = the binary32 pattern base + i: S_enc and S_dec
__global__ void k_global_scales(uint32_t base, int64_t n, float six_b, float* enc, float* dec) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const float s = fos::global_encode_scale(__uint_as_float(base + (uint32_t)i), six_b);
  enc[i] = s;
  dec[i] = 1.0f / fos::opaque(s);
}

// Quotients and products of operand pairs (the per-block multiplier table)
__global__ void k_div_mul(const float* a, const float* b, int64_t n, float* q, float* p) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  q[i] = fos::opaque(a[i]) / fos::opaque(b[i]);
  p[i] = fos::opaque(a[i]) * fos::opaque(b[i]);
}

// bf16 / f16 packing of the binary32 patterns base + 2 t, base + 2 t + 1;
// the pair is also packed swapped, and any difference between a value's
// rounding in the low and in the high half sets *mismatch
__global__ void k_pack16(int f16, uint32_t base, int64_t npairs, uint32_t* out, uint32_t* mismatch) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= npairs) return;
  const float lo = __uint_as_float(base + (uint32_t)(2 * t)), hi = __uint_as_float(base + (uint32_t)(2 * t + 1));
  const uint32_t r = f16 ? fos::pack_f16(lo, hi) : fos::pack_bf16(lo, hi);
  const uint32_t q = f16 ? fos::pack_f16(hi, lo) : fos::pack_bf16(hi, lo);
  out[t] = r;
  if (((q >> 16) | (q << 16)) != r) atomicOr(mismatch, 1u);
}

// exact upcasts of every 16-bit pattern pair (w = 2 t | (2 t + 1) << 16)
__global__ void k_upcast16(int f16, float* out) {
  const int t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= 32768) return;
  const uint32_t w = (uint32_t)(2 * t) | ((uint32_t)(2 * t + 1) << 16);
  out[2 * t] = f16 ? fos::f16_lo(w) : fos::bf16_lo(w);
  out[2 * t + 1] = f16 ? fos::f16_hi(w) : fos::bf16_hi(w);
}

// Two items of the FP16-error difference through sub_f16x2, first in the
// order (a, b), then swapped: out gets the first results, and a value that
// differs between the low and the high half sets *mismatch (NaN agrees with
// any NaN).
__device__ void sub_pair(float xa, float xb, float ha, float hb, float* out, int64_t i, uint32_t* mismatch) {
  float ea, eb, fb, fa;
  fos::sub_f16x2(xa, xb, ha, hb, ea, eb);
  fos::sub_f16x2(xb, xa, hb, ha, fb, fa);
  out[i] = ea;
  out[i + 1] = eb;
  const bool same_a = __float_as_uint(ea) == __float_as_uint(fa) || (ea != ea && fa != fa);
  const bool same_b = __float_as_uint(eb) == __float_as_uint(fb) || (eb != eb && fb != fb);
  if (!(same_a && same_b)) atomicOr(mismatch, 1u);
}

// FP16-error difference x - f32(RN16(xh)) over items p = base + i (n even):
// x is the 16-bit pattern p >> 16 of the input type (bf16 or f16), xh the
// f16 value of the pattern p & 0xFFFF; thread t takes items 2t and 2t + 1
__global__ void k_sub_f16_pairs(int x_f16, uint32_t base, int64_t n, float* out, uint32_t* mismatch) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (2 * t >= n) return;
  float x[2], xh[2];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const uint32_t p = base + (uint32_t)(2 * t + k);
    const uint32_t xw = p >> 16;
    x[k] = x_f16 ? fos::f16_lo(xw) : fos::bf16_lo(xw);
    xh[k] = fos::f16_lo(p & 0xFFFFu);
  }
  sub_pair(x[0], x[1], xh[0], xh[1], out, 2 * t, mismatch);
}

// The same on given binary32 operands (fp32 inputs, xh not a binary16 value)
__global__ void k_sub_f16(const float* x, const float* xh, int64_t n, float* out, uint32_t* mismatch) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (2 * t < n) sub_pair(x[2 * t], x[2 * t + 1], xh[2 * t], xh[2 * t + 1], out, 2 * t, mismatch);
}

int done(void) { return hipGetLastError() == hipSuccess ? 0 : 1; }

}  // namespace

extern "C" {

int prim_e2m1_encode(uint32_t base, int64_t nwords, uint32_t* out, void* s) {
  hipLaunchKernelGGL(k_e2m1_encode, dim3(grid_for(nwords)), dim3(kBlock), 0, (hipStream_t)s, base, nwords, out);
  return done();
}
int prim_e2m1_decode(const uint32_t* in, int64_t nwords, float* out, void* s) {
  hipLaunchKernelGGL(k_e2m1_decode, dim3(grid_for(nwords)), dim3(kBlock), 0, (hipStream_t)s, in, nwords, out);
  return done();
}
int prim_e4m3_encode(uint32_t base, int64_t n, uint8_t* out, uint32_t* upper_or, void* s) {
  hipLaunchKernelGGL(k_e4m3_encode, dim3(grid_for(n)), dim3(kBlock), 0, (hipStream_t)s, base, n, out, upper_or);
  return done();
}
int prim_e4m3_decode(float* out256, void* s) {
  hipLaunchKernelGGL(k_e4m3_decode, dim3(1), dim3(kBlock), 0, (hipStream_t)s, 256, out256);
  return done();
}
int prim_div6(uint32_t base, int64_t n, float* out, void* s) {
  hipLaunchKernelGGL(k_div6, dim3(grid_for(n)), dim3(kBlock), 0, (hipStream_t)s, base, n, out);
  return done();
}
int prim_global_scales(uint32_t base, int64_t n, float six_b, float* enc, float* dec, void* s) {
  hipLaunchKernelGGL(k_global_scales, dim3(grid_for(n)), dim3(kBlock), 0, (hipStream_t)s, base, n, six_b, enc, dec);
  return done();
}
int prim_div_mul(const float* a, const float* b, int64_t n, float* q, float* p, void* s) {
  hipLaunchKernelGGL(k_div_mul, dim3(grid_for(n)), dim3(kBlock), 0, (hipStream_t)s, a, b, n, q, p);
  return done();
}
int prim_pack16(int f16, uint32_t base, int64_t npairs, uint32_t* out, uint32_t* mismatch, void* s) {
  hipLaunchKernelGGL(k_pack16, dim3(grid_for(npairs)), dim3(kBlock), 0, (hipStream_t)s, f16, base, npairs, out,
                     mismatch);
  return done();
}
int prim_upcast16(int f16, float* out65536, void* s) {
  hipLaunchKernelGGL(k_upcast16, dim3(grid_for(32768)), dim3(kBlock), 0, (hipStream_t)s, f16, out65536);
  return done();
}
// n must be even (items are taken in pairs)
int prim_sub_f16_pairs(int x_f16, uint32_t base, int64_t n, float* out, uint32_t* mismatch, void* s) {
  if (n & 1) return 1;
  hipLaunchKernelGGL(k_sub_f16_pairs, dim3(grid_for(n / 2)), dim3(kBlock), 0, (hipStream_t)s, x_f16, base, n, out,
                     mismatch);
  return done();
}
int prim_sub_f16(const float* x, const float* xh, int64_t n, float* out, uint32_t* mismatch, void* s) {
  if (n & 1) return 1;
  hipLaunchKernelGGL(k_sub_f16, dim3(grid_for(n / 2)), dim3(kBlock), 0, (hipStream_t)s, x, xh, n, out, mismatch);
  return done();
}

}  // extern "C"
