// fos_device.h: device-side building blocks of the four-over-six NVFP4
// quantizer for gfx950 (MI355X).
//
// Every function here computes one step of the quantizer bit-exactly: one
// binary32 operation per step, round to nearest even. Conversions use
// gfx950's convert instructions where those are checked exhaustively against
// the format definitions (tests/test_gpu_primitives.py runs these helpers on
// the device over every input the kernels can feed them and compares each
// result bitwise with the CPU), and plain integer/float code elsewhere:
//   - f32 -> E2M1 pair (v_cvt_scalef32_pk_fp4_f32, scale 1.0): RNE with
//     saturation to +-6 for every non-NaN input, -0 kept; a NaN becomes
//     (sign | 7), i.e. +-6, so blocks holding a NaN take the careful path, which encodes
//     NaN as +6 (the NaN rule the kernel page, wolfcomos/ao PR "Add a CuTe DSL
//     fast-path kernel for four-over-six quantize", states).
//   - E2M1 pair -> f32 (v_cvt_scalef32_pk_f32_fp4, scale 1.0): exact.
//   - f32 -> E4M3 (v_cvt_pk_fp8_f32) on inputs clamped to [0, 448]: RNE.
//   - E4M3 -> f32 (v_cvt_f32_fp8): exact.
//   - f32 pair -> f16 pair and f32 pair -> bf16 pair (v_cvt_pk_f16_f32,
//     v_cvt_pk_bf16_f32): RNE, overflow to inf, gradual underflow, in
//     either half.
// The build uses -ffp-contract=off and HIP's correctly rounded f32 division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fos {

constexpr float kFltMax = 3.40282346638528859812e+38f;

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Hide a value from the optimizer so that a following conversion is not
// fused with the operation that produced it (a fused multiply-and-round to
// f16 would round once instead of twice).
__device__ __forceinline__ float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ---------------------------------------------------------------- inputs

// bf16 pair in one dword -> two exact binary32 values
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// f16 pair -> two exact binary32 values
__device__ __forceinline__ float f16_lo(uint32_t w) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  return (float)h;
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  return (float)h;
}

// two binary32 -> packed bf16 pair / f16 pair (RNE), one packed convert
// each (written out: from two scalar casts the compiler emits two converts,
// a shift and an OR). Both halves round as the scalar casts do, checked on
// every binary32 input in either position.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  uint32_t r;
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}

// ---------------------------------------------------------------- scales

// Global encode scale: S_enc = RN(6B / A) clamped to FLT_MAX, or 1 when A is
// 0, inf, NaN or negative. six_b = 6 * bound (2688 or 1536, exact).
__device__ __forceinline__ float global_encode_scale(float A, float six_b) {
  bool ok = (A > 0.0f) && (A < __builtin_huge_valf());
  float s = six_b / (ok ? A : 1.0f);
  s = __builtin_fminf(s, kFltMax);
  return ok ? s : 1.0f;
}

// E4M3 code (RNE, saturating at 448) of t >= 0, t not NaN. The pair
// convert writes code(t) to byte 0 and code(+0) = 0 to byte 1 of a zero
// word, so the result needs no mask.
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  float tc = __builtin_fminf(t, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(tc, 0.0f, 0, false);
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// ---------------------------------------------------------------- E2M1

// Eight E2M1 codes (two per byte lane, element 2j in the low nibble) of
// v[0..7] into one dword. NaN inputs give (sign | 7); see the header note.
__device__ __forceinline__ uint32_t e2m1_pack8(const float* v) {
  // each convert writes one byte of w, so its starting value never shows:
  // starting from v[0]'s bits lets the first convert write over v[0] in place
  uint32_t w = __float_as_uint(v[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// Decode eight E2M1 codes of a dword into their values.
__device__ __forceinline__ void e2m1_unpack8(uint32_t w, float* out) {
  f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  out[0] = a.x; out[1] = a.y; out[2] = b.x; out[3] = b.y;
  out[4] = c.x; out[5] = c.y; out[6] = d.x; out[7] = d.y;
}

// ---------------------------------------------------------------- division

// RN(a / 6) for a >= 0 (a NaN gives a NaN): a product with RN(1/6)
// corrected by one fused multiply-add of the exact remainder. That formula is
// correctly rounded for every finite a >= 2^-125 (tests/test_div6_formula.py
// runs it on every binary32 on the CPU). Below, some quotients are subnormal
// and it is not; at +inf the remainder is inf - inf. Those inputs take the
// division instead, so the helper is RN(a / 6) on every a from +0 to +inf
// (tests/test_gpu_primitives.py runs it on each of them on the device).
__device__ __forceinline__ float div6(float a) {
  constexpr float r6 = 0x1.555556p-3f;  // RN(1/6)
  const float q0 = a * r6;
  const float r = __builtin_fmaf(-q0, 6.0f, a);
  float q = __builtin_fmaf(r, r6, q0);
  const bool slow = (a < 0x1p-125f) || (a > kFltMax);
  if (__ballot(slow)) q = slow ? a / 6.0f : q;
  return q;
}

// RN(x - f32(RN16(xh))) for two elements: the error of x against the
// decoded value rounded to binary16 (FP16-error mode). One packed convert
// rounds both decoded values to binary16; each difference is then one
// mixed-precision FMA, h * -1 + x, whose product is exact and which rounds
// once, so it is RN(x - f32(h)) with the same signed zeros (op_sel picks the
// high half for the second element).
__device__ __forceinline__ void sub_f16x2(float x0, float x1, float xh0, float xh1, float& e0, float& e1) {
  const uint32_t h = pack_f16(xh0, xh1);
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(e0) : "v"(h), "v"(x0));
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(e1) : "v"(h), "v"(x1));
}

// ---------------------------------------------------------------- reductions

// The pinned width-16 order: strides 8, 4, 2, 1 where position i adds
// position i + stride (the clamped shuffle-down tree of the kernel page).
// Overwrites u.
__device__ __forceinline__ float tree16(float* u) {
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) {
#pragma unroll
    for (int i = 0; i < s; i++) u[i] = u[i] + u[i + s];
  }
  return u[0];
}

// Cross-lane moves (register-to-register, no LDS): CTRL is a DPP control,
// e.g. quad_perm [a,b,c,d] = a | b << 2 | c << 4 | d << 6 (each lane of a
// group of four reads the lane the pattern names) or row_shl:n = 0x100 + n
// (lane i reads lane i + n of its 16-lane row; past the row's end: 0).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowShl = 0x100;

// The sequential order: the sixteen terms added left to right in element
// order (Transformer Engine's order, kept by the Megatron-LM page).
__device__ __forceinline__ float seq16(const float* u) {
  float s = u[0];
#pragma unroll
  for (int i = 1; i < 16; i++) s = s + u[i];
  return s;
}

}  // namespace fos
