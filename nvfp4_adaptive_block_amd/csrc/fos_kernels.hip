// fos_kernels.hip: gfx950 kernels of the four-over-six NVFP4 quantizer.
//
// Sources (web pages on the method): pytorch/ao PR "Add the four-over-six
// grouped GEMM and dispatcher wiring" (recipe commit: two candidates per
// block, lower error kept; per-tensor or row-scaled global scales; 1x16 or
// 16x16 blocks; MoE commit: per-group amax expanded per row, one launch, the
// offs[-1] tail), wolfcomos/ao PR "Add a CuTe DSL fast-path kernel for
// four-over-six quantize" (rounding-critical steps, pinned width-16 tree,
// NaN rule) and radixark/Megatron-LM PR "Fuse NVFP4 fake-QAT quantize-
// dequantize with CuTe DSL" ("What does this PR do?": fused data path that
// writes only BF16/FP16, list API, E4M3 bound 448/256, MAE/MSE, exact or
// FP16 candidate error; static dispatch of every mode).
//
// Work mapping, 1x16 blocks: one lane owns one 16-element block, so the
// block amax, both candidates, the 16-term error tree and the selection stay
// in that lane's registers. A wave covers a unit of 64 consecutive blocks
// (2 KiB of bf16 read with 128-bit loads) and walks its units two at a time,
// loading the next unit while it computes the current one. A single
// tensor's units go out in pairs dealt round robin over the waves (the waves
// in flight share one window moving through the tensor); list and per-row
// launches give each wave a contiguous range. The grid holds as many
// workgroups as are resident at once (four times as many for large
// round-robin launches, whose later workgroups start as the first finish).
//
// Per-block division is replaced by a table: the block scale sigma is one of
// 127 E4M3 values, so for each global scale the wave keeps, in LDS, the
// encode multipliers RN(S_enc / sigma) and decode multipliers
// RN(sigma * S_dec) of all 127 codes, rebuilt when the wave's tensor (or
// row, or group) changes. Every unit has one global scale: per-row units
// are segments of one row, and flat grouped units never cross a group.
//
// 16x16 tiles: four consecutive lanes own a tile (lane j of the four holds
// the tile's rows j, j + 4, j + 8, j + 12), and the tile amax and error sums
// cross those lanes. A unit is one 16-row band times 16 tiles.
#include "fos_device.h"
#include "fos_kernels.h"

namespace fos {

// ------------------------------------------------------------ memory

// Raw buffer loads and stores. A lane whose offset lies past the resource's
// range reads zeros and its stores are dropped by the hardware, so ragged
// tails and idle lanes need no branch around memory operations (which would
// make the compiler wait for every outstanding load, prefetches included).
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// A block's raw bits, loaded ahead of use.
template <int DT> struct Raw;

template <> struct Raw<kBF16> {
  static constexpr int kBytes = 32;  // bytes of one 16-element block
  v4i a, b;
  __device__ void load(Rsrc r, uint32_t off) {
    a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
  }
  __device__ void unpack(float* x) const {
    const uint32_t w[8] = {(uint32_t)a.x, (uint32_t)a.y, (uint32_t)a.z, (uint32_t)a.w,
                           (uint32_t)b.x, (uint32_t)b.y, (uint32_t)b.z, (uint32_t)b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
  }
};

template <> struct Raw<kFP16> {
  static constexpr int kBytes = 32;
  v4i a, b;
  __device__ void load(Rsrc r, uint32_t off) {
    a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
  }
  __device__ void unpack(float* x) const {
    const uint32_t w[8] = {(uint32_t)a.x, (uint32_t)a.y, (uint32_t)a.z, (uint32_t)a.w,
                           (uint32_t)b.x, (uint32_t)b.y, (uint32_t)b.z, (uint32_t)b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) { x[2 * i] = f16_lo(w[i]); x[2 * i + 1] = f16_hi(w[i]); }
  }
};

template <> struct Raw<kFP32> {
  static constexpr int kBytes = 64;
  v4i v[4];
  __device__ void load(Rsrc r, uint32_t off) {
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
  }
  __device__ void unpack(float* x) const {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x[4 * i] = __int_as_float(v[i].x); x[4 * i + 1] = __int_as_float(v[i].y);
      x[4 * i + 2] = __int_as_float(v[i].z); x[4 * i + 3] = __int_as_float(v[i].w);
    }
  }
};

// Cache policy of the output stores: non-temporal. No kernel reads its
// outputs back, and streaming them past the caches measured 4-11 % faster
// (quantize, fused amax + quantize, fused QDQ) than default stores. The
// columnwise kernel's whole-line stores keep the default policy: its scale
// lines are assembled from eight tiles in one L2, and non-temporal stores
// there measured slower.
constexpr int kStoreNT = 2;

// Store 16 decoded values as the tensor's element type.
template <int DT> __device__ __forceinline__ void store16(Rsrc r, uint32_t off, const float* y);

template <> __device__ __forceinline__ void store16<kBF16>(Rsrc r, uint32_t off, const float* y) {
  const v4i a = {(int)pack_bf16(y[0], y[1]), (int)pack_bf16(y[2], y[3]), (int)pack_bf16(y[4], y[5]),
                 (int)pack_bf16(y[6], y[7])};
  const v4i b = {(int)pack_bf16(y[8], y[9]), (int)pack_bf16(y[10], y[11]), (int)pack_bf16(y[12], y[13]),
                 (int)pack_bf16(y[14], y[15])};
  __builtin_amdgcn_raw_buffer_store_b128(a, r, off, 0, kStoreNT);
  __builtin_amdgcn_raw_buffer_store_b128(b, r, off + 16, 0, kStoreNT);
}
template <> __device__ __forceinline__ void store16<kFP16>(Rsrc r, uint32_t off, const float* y) {
  const v4i a = {(int)pack_f16(y[0], y[1]), (int)pack_f16(y[2], y[3]), (int)pack_f16(y[4], y[5]),
                 (int)pack_f16(y[6], y[7])};
  const v4i b = {(int)pack_f16(y[8], y[9]), (int)pack_f16(y[10], y[11]), (int)pack_f16(y[12], y[13]),
                 (int)pack_f16(y[14], y[15])};
  __builtin_amdgcn_raw_buffer_store_b128(a, r, off, 0, kStoreNT);
  __builtin_amdgcn_raw_buffer_store_b128(b, r, off + 16, 0, kStoreNT);
}
template <> __device__ __forceinline__ void store16<kFP32>(Rsrc r, uint32_t off, const float* y) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const v4i a = {__float_as_int(y[4 * i]), __float_as_int(y[4 * i + 1]), __float_as_int(y[4 * i + 2]),
                   __float_as_int(y[4 * i + 3])};
    __builtin_amdgcn_raw_buffer_store_b128(a, r, off + 16 * i, 0, kStoreNT);
  }
}

// Store 8 decoded values as the output type.
template <int DT> __device__ __forceinline__ void store8(Rsrc r, uint32_t off, const float* y);
template <> __device__ __forceinline__ void store8<kBF16>(Rsrc r, uint32_t off, const float* y) {
  const v4i a = {(int)pack_bf16(y[0], y[1]), (int)pack_bf16(y[2], y[3]), (int)pack_bf16(y[4], y[5]),
                 (int)pack_bf16(y[6], y[7])};
  __builtin_amdgcn_raw_buffer_store_b128(a, r, off, 0, kStoreNT);
}
template <> __device__ __forceinline__ void store8<kFP16>(Rsrc r, uint32_t off, const float* y) {
  const v4i a = {(int)pack_f16(y[0], y[1]), (int)pack_f16(y[2], y[3]), (int)pack_f16(y[4], y[5]),
                 (int)pack_f16(y[6], y[7])};
  __builtin_amdgcn_raw_buffer_store_b128(a, r, off, 0, kStoreNT);
}
template <> __device__ __forceinline__ void store8<kFP32>(Rsrc r, uint32_t off, const float* y) {
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const v4i a = {__float_as_int(y[4 * i]), __float_as_int(y[4 * i + 1]), __float_as_int(y[4 * i + 2]),
                   __float_as_int(y[4 * i + 3])};
    __builtin_amdgcn_raw_buffer_store_b128(a, r, off + 16 * i, 0, kStoreNT);
  }
}

// The block a lane holds in a unit of 64 blocks, and the byte offset of that
// block. Quantize units and fp32 QDQ units: lane l holds block l. QDQ units
// of 16-bit types: lane 2i holds block i and lane 2i + 1 block 32 + i, so
// that store_qdq16 can write the unit's outputs with two stores that each
// cover 1 KiB contiguously (16-byte pieces from every lane, in lane order).
// With each lane writing its own block's 32 bytes instead, every store
// instruction covers half of each line in a 2 KiB span; a stream of the
// QDQ's bytes with non-temporal stores in that pattern ran 1.7x slower.
template <int DT, int OUT>
__device__ __forceinline__ int unit_block_of_lane(int lane) {
  if (OUT == kOutQdq && DT != kFP32) return (lane >> 1) + (lane & 1) * 32;
  return lane;
}

// Store the decoded block of a 16-bit QDQ unit laid out by
// unit_block_of_lane: the lane pairs swap one 16-byte half (a DPP exchange
// within each pair), then the first store writes blocks 0-31 and the second
// blocks 32-63, each lane one 16-byte piece at 16 * lane.
template <int DT>
__device__ __forceinline__ void store_qdq16(Rsrc r, uint32_t unit_off, const float* y, int lane) {
  const bool even = (lane & 1) == 0;
  uint32_t lo[4], hi[4], out0[4], out1[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    lo[k] = DT == kBF16 ? pack_bf16(y[2 * k], y[2 * k + 1]) : pack_f16(y[2 * k], y[2 * k + 1]);
    hi[k] = DT == kBF16 ? pack_bf16(y[8 + 2 * k], y[9 + 2 * k]) : pack_f16(y[8 + 2 * k], y[9 + 2 * k]);
    // the even lane sends its high half, the odd lane its low half
    const uint32_t send = even ? hi[k] : lo[k];
    const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    out0[k] = even ? lo[k] : got;  // block i: low half (even lane), high half (odd lane)
    out1[k] = even ? got : hi[k];  // block 32 + i
  }
  const v4i a = {(int)out0[0], (int)out0[1], (int)out0[2], (int)out0[3]};
  const v4i b = {(int)out1[0], (int)out1[1], (int)out1[2], (int)out1[3]};
  __builtin_amdgcn_raw_buffer_store_b128(a, r, unit_off + 16 * lane, 0, kStoreNT);
  __builtin_amdgcn_raw_buffer_store_b128(b, r, unit_off + 1024 + 16 * lane, 0, kStoreNT);
}

__device__ __forceinline__ void store_codes(Rsrc r, uint32_t off, uint32_t c0, uint32_t c1) {
  const v2i v = {(int)c0, (int)c1};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStoreNT);
}

__device__ __forceinline__ void store_scale(Rsrc r, uint32_t off, uint32_t s) {
  __builtin_amdgcn_raw_buffer_store_b8((unsigned char)s, r, off, 0, kStoreNT);
}

// Stores that touch nothing (zero-range resource), fenced against
// reordering: between the first unit's loads and the second unit's, they
// stand in for the stores a loop iteration issues there (two per block), so that the
// compiler's memory wait before the first use equals the loop's.
template <int NB>
__device__ __forceinline__ void dummy_stores() {
  __builtin_amdgcn_sched_barrier(0);
  const Rsrc none = make_rsrc(nullptr, 0);
#pragma unroll
  for (int j = 0; j < NB; j++) {
    store_codes(none, 0, 0u, 0u);
    store_scale(none, 0, 0u);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Loads of values no kernel writes (amaxes, offsets), from the constant
// address space so that wave-uniform addresses become scalar loads.
typedef __attribute__((address_space(4))) const float* ConstF32;
typedef __attribute__((address_space(4))) const int32_t* ConstI32;
__device__ __forceinline__ float ld_const(const float* p, int64_t i) {
  return ((ConstF32)(const void*)p)[i];
}
__device__ __forceinline__ int32_t ld_const(const int32_t* p, int64_t i) {
  return ((ConstI32)(const void*)p)[i];
}

// ------------------------------------------------------------ scales

// Per-wave LDS table of the multipliers of all E4M3 codes for one global
// scale: E[c] = RN(S_enc / sigma_c) (0 for sigma = 0, FLT_MAX on overflow),
// D[c] = RN(sigma_c * S_dec). Codes never exceed 0x7E (scales saturate).
// One code's entries (c < 128; code 0x7F, the E4M3 NaN, gets zeros).
__device__ __forceinline__ void table_entry(int c, float S_enc, float S_dec, float* E, float* D) {
  const float sigma = e4m3_value((uint32_t)c);
  const bool zero = sigma == 0.0f || c >= 0x7F;
  const float e = S_enc / (zero ? 1.0f : sigma);
  E[c] = zero ? 0.0f : __builtin_fminf(e, kFltMax);
  D[c] = (c >= 0x7F) ? 0.0f : sigma * S_dec;
}

struct Table {
  float* E;
  float* D;
  __device__ void build(float S_enc, float S_dec, int lane) const {
#pragma unroll
    for (int k = 0; k < 2; k++) table_entry(lane + 64 * k, S_enc, S_dec, E, D);
    // the lanes of this wave read what other lanes wrote
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
};

// One candidate's block scale and multipliers: t = RN(q * S_enc) with q the
// already divided block amax (RN(a/6) or RN(a/4)); scale = E4M3(t); the
// multipliers E = RN(S_enc / sigma) and D = RN(sigma * S_dec) come from the
// wave's table.
struct Cand {
  uint32_t scale;
  float E, D;
};

__device__ __forceinline__ Cand make_cand(float q, float S_enc, const Table& tab) {
  Cand c;
  c.scale = e4m3_code(q * S_enc);
  c.E = tab.E[c.scale];
  c.D = tab.D[c.scale];
  return c;
}

// ------------------------------------------------------------ block pieces

// NaN-dropping max |x| over 16 values. The fast form (v_max3_f32) is exact
// whenever no element is NaN; a block holding a NaN is always recomputed by
// the careful form (integer max over the magnitude bits, NaN patterns -> +0).
template <bool CAREFUL>
__device__ __forceinline__ float amax16(const float* x) {
  if (CAREFUL) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const uint32_t m = __float_as_uint(x[i]) & 0x7FFFFFFFu;
      a = max(a, m <= 0x7F800000u ? m : 0u);
    }
    return __uint_as_float(a);
  } else {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) a = __builtin_fmaxf(a, __builtin_fabsf(x[i]));
    return a;
  }
}

// True when any of the 16 values is NaN (v_maximum3_f32 propagates NaN).
__device__ __forceinline__ bool any_nan16(const float* x) {
  float m = x[0];
#pragma unroll
  for (int i = 1; i < 16; i++) m = __builtin_elementwise_maximum(m, x[i]);
  return m != m;
}

// E2M1 codes of x * E. The careful form encodes NaN elements as +6.
template <bool CAREFUL>
__device__ __forceinline__ void encode16(const float* x, float E, uint32_t& c0, uint32_t& c1) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    v[i] = x[i] * E;
    if (CAREFUL) v[i] = (x[i] != x[i]) ? 6.0f : v[i];
  }
  c0 = e2m1_pack8(v);
  c1 = e2m1_pack8(v + 8);
}

// Decoded values x_hat = RN(val(q) * D).
__device__ __forceinline__ void decode16(uint32_t c0, uint32_t c1, float D, float* xh) {
  float q[16];
  e2m1_unpack8(c0, q);
  e2m1_unpack8(c1, q + 8);
#pragma unroll
  for (int i = 0; i < 16; i++) xh[i] = q[i] * D;
}

// Error terms of one row segment (16 elements) and their sum in the pinned
// order (the tree, or the sequential order for 1x16 blocks).
template <int METRIC, int PREC, int ORDER>
__device__ __forceinline__ float err16(const float* x, const float* xh) {
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    float e0, e1;
    if (PREC == kErrFP16) {
      sub_f16x2(x[i], x[i + 1], xh[i], xh[i + 1], e0, e1);
    } else {
      e0 = x[i] - xh[i];
      e1 = x[i + 1] - xh[i + 1];
    }
    u[i] = (METRIC == kMAE) ? __builtin_fabsf(e0) : e0 * e0;
    u[i + 1] = (METRIC == kMAE) ? __builtin_fabsf(e1) : e1 * e1;
  }
  return ORDER == kOrderSeq ? seq16(u) : tree16(u);
}

struct BlockOut {
  uint32_t c0, c1;  // 16 E2M1 codes
  uint32_t scale;   // E4M3 code
};

// Quantize one 1x16 block held in x. When NEED_XHAT, xh receives the kept
// candidate's decoded values. Returns false when the fast form cannot be
// trusted (the block holds a NaN); the caller then reruns with CAREFUL.
template <int RECIPE, int METRIC, int PREC, int ORDER, bool CAREFUL, bool NEED_XHAT>
__device__ __forceinline__ bool block_1x16(const float* x, float S_enc, float S_dec, const Table& tab, BlockOut& o,
                                           float* xh) {
  const float a = amax16<CAREFUL>(x);
  const Cand k6 = make_cand(div6(a), S_enc, tab);
  uint32_t c60, c61;
  encode16<CAREFUL>(x, k6.E, c60, c61);
  if (RECIPE == kNVFP4) {
    o.c0 = c60; o.c1 = c61; o.scale = k6.scale;
    if (NEED_XHAT) decode16(c60, c61, k6.D, xh);
    return CAREFUL || !any_nan16(x);
  } else {
    float e6;
    {
      float t[16];
      decode16(c60, c61, k6.D, t);
      e6 = err16<METRIC, PREC, ORDER>(x, t);
    }
    __builtin_amdgcn_sched_barrier(0);
    const Cand k4 = make_cand(a * 0.25f, S_enc, tab);
    uint32_t c40, c41;
    encode16<CAREFUL>(x, k4.E, c40, c41);
    float e4;
    {
      float t[16];
      decode16(c40, c41, k4.D, t);
      e4 = err16<METRIC, PREC, ORDER>(x, t);
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool four = e4 < e6;
    o.c0 = four ? c40 : c60;
    o.c1 = four ? c41 : c61;
    o.scale = four ? k4.scale : k6.scale;
    if (NEED_XHAT) decode16(o.c0, o.c1, four ? k4.D : k6.D, xh);
    return CAREFUL || (e6 == e6 && e4 == e4);
  }
}

// Quantize a 1x16 block with the fast form, falling back to the careful form
// when the block holds a NaN.
template <int RECIPE, int METRIC, int PREC, int ORDER, bool NEED_XHAT>
__device__ __forceinline__ void quantize_block(const float* x, float S_enc, float S_dec, const Table& tab,
                                               BlockOut& o, float* xh) {
  if (!block_1x16<RECIPE, METRIC, PREC, ORDER, false, NEED_XHAT>(x, S_enc, S_dec, tab, o, xh))
    block_1x16<RECIPE, METRIC, PREC, ORDER, true, NEED_XHAT>(x, S_enc, S_dec, tab, o, xh);
}

// ------------------------------------------------------------ 1x16 kernel

// Row -> group through the cumulative end offsets (binary search: the first
// g with r < offs[g]; rows past offs[G-1] map to G-1). Wave-uniform.
__device__ __forceinline__ int group_of(const int32_t* offs, int G, int64_t r) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (r < (int64_t)ld_const(offs, mid)) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// S_dec side outputs and the offsets check, spread over the grid.
template <int GRAN, int NT>
__device__ void side_outputs(const Args1x16<NT>& args) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gsz = (int64_t)gridDim.x * blockDim.x;
  if (args.sdec_out) {
    if (GRAN == kGranTensor) {
      if (gid == 0) args.sdec_out[0] = 1.0f / global_encode_scale(args.t[0].amax[0], args.six_b);
    } else if (GRAN == kGranRow) {
      for (int64_t r = gid; r < args.t[0].M; r += gsz)
        args.sdec_out[r] = 1.0f / global_encode_scale(args.t[0].amax[r], args.six_b);
    } else {
      for (int64_t g = gid; g < args.G; g += gsz)
        args.sdec_out[g] = 1.0f / global_encode_scale(args.group_amax[g], args.six_b);
    }
  }
  if (GRAN == kGranGroup && args.status) {
    for (int64_t g = gid; g < args.G; g += gsz) {
      const int32_t prev = g ? args.offs[g - 1] : 0;
      const int32_t o = args.offs[g];
      const bool bad = o < prev || (o & 15) || (g == args.G - 1 && (int64_t)o > args.t[0].M);
      if (bad) atomicOr(args.status, kStatusBadOffs);
    }
  }
}

// The buffer resources of one unit of a 1x16 launch.
struct Unit {
  Rsrc x, out, scl;  // input, codes (or QDQ output), scales
};

// Units of a 1x16 launch. Per-tensor scales: a unit is 64·NB consecutive
// blocks of the flattened tensor. Per-row scales: a unit is a segment of up
// to 64·NB blocks of one row, so each unit has one global scale. Grouped
// scales: flat units when every group is a whole number of units
// (grouped_flat), else per-row segments.
// Position of a unit: its index in the tensor and, for per-row units, its
// row and segment (flat grouped units: the row of their first block and
// that block's index in the row), kept up to date incrementally.
struct UPos {
  int64_t v, row, seg;
};

template <int DT, int GRAN, int OUT>
struct Walk {
  static constexpr int kB = Raw<DT>::kBytes;
  static constexpr int kUnitBlocks = unit_blocks(OUT, DT);
  const TensorRef& T;
  uint8_t* codes;
  uint8_t* scales;
  int64_t nbk, nblk, spr;
  bool flat;  // units over the flattened tensor (per tensor, or grouped_flat)
  __device__ Walk(const TensorRef& t, uint8_t* c, uint8_t* s) : T(t), codes(c), scales(s) {
    nbk = T.K >> 4;
    nblk = T.M * nbk;
    spr = (nbk + kUnitBlocks - 1) / kUnitBlocks;
    flat = GRAN == kGranTensor || (GRAN == kGranGroup && grouped_flat(T.K, kUnitBlocks));
  }
  __device__ UPos at(int64_t v) const {
    if (GRAN == kGranTensor) return UPos{v, 0, 0};
    if (flat) {
      const int64_t b0 = v * kUnitBlocks, row = b0 / nbk;
      return UPos{v, row, b0 - row * nbk};
    }
    const int64_t row = v / spr;
    return UPos{v, row, v - row * spr};
  }
  __device__ UPos next(UPos p) const {
    p.v += 1;
    if (GRAN != kGranTensor) {
      if (flat) {  // nbk >= kUnitBlocks / 16 here, so at most 16 steps
        p.seg += kUnitBlocks;
        while (p.seg >= nbk) { p.seg -= nbk; p.row += 1; }
      } else {
        p.seg += 1;
        if (p.seg == spr) { p.seg = 0; p.row += 1; }
      }
    }
    return p;
  }
  // Moving a position n units ahead: the row and segment steps of n units,
  // taken once, then one carry per move (segments stay below their limit).
  struct Step {
    int64_t n, drow, dseg;
  };
  __device__ Step step_of(int64_t n) const {
    if (GRAN == kGranTensor) return Step{n, 0, 0};
    const int64_t b = flat ? n * kUnitBlocks : n, lim = flat ? nbk : spr;
    return Step{n, b / lim, b - (b / lim) * lim};
  }
  __device__ UPos advance(UPos p, const Step& st) const {
    p.v += st.n;
    if (GRAN != kGranTensor) {
      const int64_t lim = flat ? nbk : spr;
      p.row += st.drow;
      p.seg += st.dseg;
      if (p.seg >= lim) { p.seg -= lim; p.row += 1; }
    }
    return p;
  }
  // resources for the unit at p (valid: the unit exists; rows_read: rows of
  // the tensor that hold data, later rows read as zeros)
  __device__ Unit unit(const UPos& p, bool valid, int64_t rows_read) const {
    int64_t b0, nvalid;
    if (flat) {
      b0 = p.v * kUnitBlocks;
      nvalid = min((int64_t)kUnitBlocks, nblk - b0);
    } else {
      b0 = p.row * nbk + p.seg * kUnitBlocks;
      nvalid = min((int64_t)kUnitBlocks, nbk - p.seg * kUnitBlocks);
    }
    if (!valid) nvalid = 0;
    const int64_t nread = (GRAN == kGranGroup && p.row >= rows_read) ? 0 : nvalid;
    Unit u;
    u.x = make_rsrc(static_cast<const char*>(T.x) + b0 * kB, nread * kB);
    if (OUT == kOutQuant) {
      u.out = make_rsrc(codes + b0 * 8, nvalid * 8);
      u.scl = make_rsrc(scales + b0, nvalid);
    } else {
      u.out = make_rsrc(static_cast<char*>(T.y) + b0 * kB, nvalid * kB);
      u.scl = u.out;
    }
    return u;
  }
};

// Quantize (or quantize-dequantize) the lane's blocks of one unit, held in
// raw, and store the outputs to the unit's resources.
template <int DT, int RECIPE, int METRIC, int PREC, int ORDER, int OUT>
__device__ __forceinline__ void unit_1x16(const Raw<DT>* raw, float S_enc, float S_dec, const Table& tab,
                                          const Unit& U, int lane) {
  constexpr bool kXhat = OUT == kOutQdq;
  constexpr int kB = Raw<DT>::kBytes;
  constexpr int kNB = unit_blocks(OUT, DT) / 64;
  const uint32_t off_x = lane * kB, off_c = lane * 8, off_s = lane;
  if constexpr (OUT == kOutQuant && kNB > 1) {
    // the lane's blocks of the unit go through the fast form together,
    // in one basic block (their serial parts interleave), and all are
    // redone in the careful form if any holds a NaN (the careful form
    // gives the same result on blocks without NaN)
    float x[kNB][16], xh[kNB][16];
    BlockOut o[kNB];
    bool fast_ok = true;
#pragma unroll
    for (int j = 0; j < kNB; j++) {
      raw[j].unpack(x[j]);
      fast_ok &= block_1x16<RECIPE, METRIC, PREC, ORDER, false, false>(x[j], S_enc, S_dec, tab, o[j], xh[j]);
    }
    if (!fast_ok) {
#pragma unroll
      for (int j = 0; j < kNB; j++)
        block_1x16<RECIPE, METRIC, PREC, ORDER, true, false>(x[j], S_enc, S_dec, tab, o[j], xh[j]);
    }
#pragma unroll
    for (int j = 0; j < kNB; j++) {
      store_codes(U.out, off_c + j * 64 * 8, o[j].c0, o[j].c1);
      store_scale(U.scl, off_s + j * 64, o[j].scale);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kNB; j++) {
      float x[16], xh[16];
      raw[j].unpack(x);
      BlockOut o;
      quantize_block<RECIPE, METRIC, PREC, ORDER, kXhat>(x, S_enc, S_dec, tab, o, xh);
      if (OUT == kOutQuant) {
        store_codes(U.out, off_c + j * 64 * 8, o.c0, o.c1);
        store_scale(U.scl, off_s + j * 64, o.scale);
      } else if (DT != kFP32) {
        store_qdq16<DT>(U.out, j * 64 * kB, xh, lane);
      } else {
        store16<DT>(U.out, off_x + j * 64 * kB, xh);
      }
    }
  }
}

// Zero codes and scales for the lane's blocks of a quantize unit.
template <int DT>
__device__ __forceinline__ void zero_unit_1x16(const Unit& U, int lane) {
  constexpr int kNB = unit_blocks(kOutQuant, DT) / 64;
#pragma unroll
  for (int j = 0; j < kNB; j++) {
    store_codes(U.out, lane * 8 + j * 64 * 8, 0u, 0u);
    store_scale(U.scl, lane + j * 64, 0u);
  }
}

// The units of one wave of a 1x16 launch: pairs u, u + 1, then u + stride,
// u + stride + 1, and so on, below u_end. stride 2 walks a contiguous range
// [u, u_end) (over the tensors of a list); a larger stride deals pairs out
// round robin over a single tensor's units. With FUSED the amaxes come from
// `fused_amax` (LDS, as float bits) rather than from memory: per-tensor
// scales [n], one per tensor of the launch; grouped scales [G]; per-row
// scales [1], the amax of the one row the range covers.
template <int NT, int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT, bool FUSED>
__device__ __forceinline__ void walk_1x16(const Args1x16<NT>& args, const Table& tab, int lane, int64_t u,
                                          int64_t u_end, const uint32_t* fused_amax, int64_t stride = 2) {
  constexpr int kB = Raw<DT>::kBytes;
  constexpr int kNB = unit_blocks(OUT, DT) / 64;
  const int64_t total = args.total_units;
  int ti = 0;
  while (ti + 1 < args.n && args.t[ti + 1].unit_begin <= u) ti++;
  const float six_b = args.six_b;
  const uint32_t off_x = unit_block_of_lane<DT, OUT>(lane) * kB;

  for (;;) {
    const TensorRef T = args.t[ti];
    const Walk<DT, GRAN, OUT> W(T, args.codes, args.scales);
    const int64_t stop = min(u_end, (ti + 1 < args.n) ? args.t[ti + 1].unit_begin : total);
    int64_t rows_read = T.M;  // grouped: rows before offs[G-1] hold data
    if (GRAN == kGranGroup) rows_read = min(max((int64_t)ld_const(args.offs, args.G - 1), (int64_t)0), T.M);

    float S_enc = 1.0f, S_dec = 1.0f;
    if (GRAN == kGranTensor) {
      S_enc = global_encode_scale(FUSED ? __uint_as_float(fused_amax[ti]) : ld_const(T.amax, 0), six_b);
      S_dec = 1.0f / S_enc;
      tab.build(S_enc, S_dec, lane);
    }
    // per-row scales: the row whose global scale is current, its amax bits
    // (rows of equal amax share the table) and, grouped, the current group's
    // row range
    int64_t tab_row = -1;
    int64_t tab_amax = -1;  // amax bits of the current table; -1: none built yet
    int64_t g_lo = 0, g_hi = 0;
    int g_cur = -1;
    // up to 64 groups: lane g holds offs[g] (and the group's amax bits), so
    // a row's group is a count of lanes rather than a chain of loads
    const bool lane_groups = GRAN == kGranGroup && args.G <= 64;
    int32_t offs_l = INT32_MAX;
    uint32_t gam_l = 0;
    if (GRAN == kGranGroup && lane_groups && lane < args.G) {
      offs_l = args.offs[lane];
      if (!FUSED) gam_l = __float_as_uint(args.group_amax[lane]);
    }

    // one unit: quantize the lane's block held in `raw`, store its outputs
    // (two stores). Units past the range compute on zeros and their stores
    // fall outside their resources.
    auto process = [&](const Raw<DT>* raw, const UPos& pos, bool valid, const Unit& U) {
      if (GRAN == kGranGroup && pos.row >= rows_read) {
        // a padding unit (wave-uniform: group offsets are multiples of 16
        // rows, so a flat unit never straddles offs[G-1], and a per-row unit
        // lies in one row): its outputs are zero, which is what quantizing
        // its zeros would give, so nothing is computed
        zero_unit_1x16<DT>(U, lane);
        return;
      }
      if (GRAN != kGranTensor) {
        const int64_t row = pos.row;  // wave-uniform
        if (valid && row != tab_row) {
          float A;
          if (GRAN == kGranRow) {
            A = FUSED ? __uint_as_float(fused_amax[0]) : ld_const(T.amax, row);
          } else {
            if (lane_groups) {
              // the groups that end at or before the row precede it (a data
              // row lies below offs[G-1] <= INT32_MAX)
              g_cur = min((int)__builtin_popcountll(__ballot(offs_l <= (int32_t)row)), args.G - 1);
            } else if (row < g_lo || row >= g_hi) {
              g_cur = group_of(args.offs, args.G, row);
              g_lo = g_cur ? (int64_t)ld_const(args.offs, g_cur - 1) : 0;
              g_hi = (g_cur == args.G - 1) ? INT64_MAX : (int64_t)ld_const(args.offs, g_cur);
            }
            A = FUSED ? __uint_as_float(fused_amax[g_cur])
                      : lane_groups ? __uint_as_float(__builtin_amdgcn_readlane(gam_l, g_cur))
                                    : ld_const(args.group_amax, g_cur);
          }
          if ((int64_t)__float_as_uint(A) != tab_amax) {
            S_enc = global_encode_scale(A, six_b);
            S_dec = 1.0f / S_enc;
            tab.build(S_enc, S_dec, lane);
            tab_amax = __float_as_uint(A);
          }
          tab_row = row;
        }
      }
      unit_1x16<DT, RECIPE, METRIC, PREC, ORDER, OUT>(raw, S_enc, S_dec, tab, U, lane);
    };

    auto load_unit = [&](Raw<DT>* r, const Unit& U) {
#pragma unroll
      for (int j = 0; j < kNB; j++) r[j].load(U.x, off_x + j * 64 * kB);
    };

    // Two units in flight, A and B: each is reloaded right after its stores,
    // so between a load and its use the same memory operations issue on
    // every path (the two dummy stores below stand in for the stores of a
    // unit before the first), and the compiler's wait counts only the loads
    // issued since.
    const int64_t v_stop = stop - T.unit_begin;
    const auto st = W.step_of(stride);
    UPos pa = W.at(u - T.unit_begin);
    UPos pb = W.next(pa);
    Unit UA = W.unit(pa, true, rows_read);
    Unit UB = W.unit(pb, pb.v < v_stop, rows_read);
    Raw<DT> A[kNB], B[kNB];
    load_unit(A, UA);
    dummy_stores<kNB>();
    load_unit(B, UB);
    for (; pa.v < v_stop;) {
      process(A, pa, true, UA);
      pa = W.advance(pa, st);
      UA = W.unit(pa, pa.v < v_stop, rows_read);
      load_unit(A, UA);
      process(B, pb, pb.v < v_stop, UB);
      pb = W.advance(pb, st);
      UB = W.unit(pb, pb.v < v_stop, rows_read);
      load_unit(B, UB);
    }
    u = stop;
    if (u >= u_end) break;
    ti++;
  }
}

// Lists of up to kListTables tensors with per-tensor scales: every tensor's
// table is built once per workgroup, in LDS, so that the units of the whole
// list can go out in pairs dealt round robin over the waves (the waves in
// flight then share one window moving through the list) without a table
// rebuilt per pair. tabs[i] holds tensor i's E (first 128) and D entries,
// scl[i] its S_enc and S_dec.
constexpr int kListTables = 16;

template <int NT, int DT, int RECIPE, int METRIC, int PREC, int ORDER, int OUT>
__device__ __forceinline__ void walk_list_rr(const Args1x16<NT>& args, float (*tabs)[256], const float (*scl)[2],
                                             int lane, int64_t u, int64_t stride) {
  static_assert(OUT == kOutQdq, "lists are quantize-dequantize launches");
  constexpr int kB = Raw<DT>::kBytes;
  constexpr int kNB = unit_blocks(OUT, DT) / 64;
  constexpr int64_t kUB = unit_blocks(OUT, DT);
  const int64_t total = args.total_units;
  const uint32_t off_x = unit_block_of_lane<DT, OUT>(lane) * kB;
  struct LPos {
    int64_t g;  // unit of the launch
    int ti;     // its tensor (the last one past the end)
  };
  auto locate = [&](int64_t g, int ti) {  // units only move forward
    while (ti + 1 < args.n && args.t[ti + 1].unit_begin <= g) ti++;
    return LPos{g, ti};
  };
  auto unit = [&](const LPos& p) {
    const TensorRef& T = args.t[p.ti];
    const int64_t b0 = (p.g - T.unit_begin) * kUB;
    const int64_t nvalid = p.g < total ? min(kUB, T.M * (T.K >> 4) - b0) : 0;
    Unit U;
    U.x = make_rsrc(static_cast<const char*>(T.x) + b0 * kB, nvalid * kB);
    U.out = make_rsrc(static_cast<char*>(T.y) + b0 * kB, nvalid * kB);
    U.scl = U.out;
    return U;
  };
  auto load_unit = [&](Raw<DT>* r, const Unit& U) {
#pragma unroll
    for (int j = 0; j < kNB; j++) r[j].load(U.x, off_x + j * 64 * kB);
  };
  // a unit past the end computes on zeros; its stores fall outside its
  // resources
  auto process = [&](const Raw<DT>* raw, const LPos& p, const Unit& U) {
    const Table tab{tabs[p.ti], tabs[p.ti] + 128};
    unit_1x16<DT, RECIPE, METRIC, PREC, ORDER, OUT>(raw, scl[p.ti][0], scl[p.ti][1], tab, U, lane);
  };
  // two units in flight, as in walk_1x16
  LPos pa = locate(u, 0);
  LPos pb = locate(u + 1, pa.ti);
  Unit UA = unit(pa), UB = unit(pb);
  Raw<DT> A[kNB], B[kNB];
  load_unit(A, UA);
  dummy_stores<kNB>();
  load_unit(B, UB);
  while (pa.g < total) {
    process(A, pa, UA);
    pa = locate(pa.g + stride, pa.ti);
    UA = unit(pa);
    load_unit(A, UA);
    process(B, pb, UB);
    pb = locate(pb.g + stride, pb.ti);
    UB = unit(pb);
    load_unit(B, UB);
  }
}

// The wave's share [u, u_end) of units [begin, end): contiguous ranges in
// wave order, of n / nwaves units and one more for the first n % nwaves
// waves. Waves are numbered round by round (workgroup b holds waves 4b ..
// 4b + 3, and the dispatcher deals workgroups out over the CUs in turn), so
// the longer ranges spread evenly over the SIMDs: each SIMD's total differs
// by at most a unit per round. (Ranges of ceil(n / nwaves) units would leave
// the last waves idle and load the SIMDs that hold none of them with up to
// a unit per wave more.)
__device__ __forceinline__ void wave_range(int64_t begin, int64_t end, int64_t wave, int64_t nwaves, int64_t& u,
                                           int64_t& u_end) {
  const int64_t n = max(end - begin, (int64_t)0);
  const int64_t base = n / nwaves, extra = n - base * nwaves;
  u = begin + wave * base + min(wave, extra);
  u_end = u + base + (wave < extra ? 1 : 0);
}

// Units of a grouped launch that hold data rows (rows before offs[G-1]);
// the units after them are padding. Group offsets are multiples of 16 rows,
// so with flat units the boundary falls between two units.
template <int DT, int NT>
__device__ __forceinline__ int64_t grouped_data_units(const Args1x16<NT>& args) {
  constexpr int64_t kUB = unit_blocks(kOutQuant, DT);
  const TensorRef& T = args.t[0];
  const int64_t rows = min(max((int64_t)ld_const(args.offs, args.G - 1), (int64_t)0), T.M);
  const int64_t nbk = T.K >> 4;
  const int64_t d = grouped_flat(T.K, kUB) ? (rows * nbk + kUB - 1) / kUB : rows * ((nbk + kUB - 1) / kUB);
  return min(d, args.total_units);
}

template <int NT, int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT>
__global__ void __launch_bounds__(256) k_1x16(const Args1x16<NT> args) {
  constexpr bool kList = NT > 1 && OUT == kOutQdq && GRAN == kGranTensor;
  __shared__ float lds[kList ? kListTables : 4][256];  // a table per wave, or per tensor of a list
  __shared__ float lscl[kList ? kListTables : 1][2];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const Table tab{lds[wv], lds[wv] + 128};

  if (OUT == kOutQuant) side_outputs<GRAN>(args);

  const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  if constexpr (kList) {
    if (args.n > 1 && args.n <= kListTables) {
      // every tensor's scales, then its table, shared by the workgroup
      if (threadIdx.x < args.n) {
        const float S_enc = global_encode_scale(ld_const(args.t[threadIdx.x].amax, 0), args.six_b);
        lscl[threadIdx.x][0] = S_enc;
        lscl[threadIdx.x][1] = 1.0f / S_enc;
      }
      __syncthreads();
      for (int i = threadIdx.x; i < args.n * 128; i += blockDim.x)
        table_entry(i & 127, lscl[i >> 7][0], lscl[i >> 7][1], lds[i >> 7], lds[i >> 7] + 128);
      __syncthreads();
      const int64_t u = 2 * wave;
      if (u < args.total_units)
        walk_list_rr<NT, DT, RECIPE, METRIC, PREC, ORDER, OUT>(args, lds, lscl, lane, u, 2 * nwaves);
      return;
    }
  }
  // A single tensor's units go out in pairs dealt round robin, so that the
  // waves in flight work inside one window that moves through the tensor;
  // the tensors of a list, and per-row units (a table per row), go out as
  // contiguous ranges.
  const bool rr = args.n == 1 && GRAN != kGranRow;
  const int64_t stride = rr ? 2 * nwaves : 2;
  int64_t u, u_end;
  auto share = [&](int64_t begin, int64_t end) {
    if (rr) {
      u = begin + 2 * wave;
      u_end = end;
    } else {
      wave_range(begin, end, wave, nwaves, u, u_end);
    }
  };
  if (GRAN == kGranGroup) {
    // the data units, then the padding units (zero outputs, nothing
    // computed), each dealt out evenly, so that no wave holds only padding
    const int64_t D = grouped_data_units<DT>(args);
    share(0, D);
    if (u < u_end)
      walk_1x16<NT, DT, RECIPE, METRIC, PREC, ORDER, GRAN, OUT, false>(args, tab, lane, u, u_end, nullptr, stride);
    share(D, args.total_units);
  } else {
    share(0, args.total_units);
  }
  if (u < u_end)
    walk_1x16<NT, DT, RECIPE, METRIC, PREC, ORDER, GRAN, OUT, false>(args, tab, lane, u, u_end, nullptr, stride);
}

// NaN-dropping magnitude max over packed 16-bit pairs: with m = |h| bits,
// adding `bias` (0x7F for bf16, 0x3FF for f16) sends exactly the NaN patterns
// past 0x7FFF, where a signed 16-bit max ignores them.
typedef short s16x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ s16x2 pair_key(uint32_t w) {
  const uint32_t bias = (DT == kBF16) ? 0x007F007Fu : 0x03FF03FFu;
  return __builtin_bit_cast(s16x2, w & 0x7FFF7FFFu) + __builtin_bit_cast(s16x2, bias);
}

template <int DT>
__device__ __forceinline__ uint32_t pair_key_to_f32_bits(s16x2 k) {
  const int bias = (DT == kBF16) ? 0x7F : 0x3FF;
  const int m = max((int)k.x, (int)k.y) - bias;  // magnitude bits of the max
  if (DT == kBF16) return (uint32_t)m << 16;
  const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)m);
  return __float_as_uint((float)h);
}

// ------------------------------------------------------------ 16x16 kernel

// A 16x16 tile belongs to LPT = 4 consecutive lanes: lane j of the group
// holds the tile's rows j, j + 4, j + 8, j + 12 (RPL = 4 rows of 16
// elements each). A wave's unit is one 16-row band times 16 consecutive
// tiles, so each load instruction covers 4 rows, each over 512 (bf16) or
// 1024 (fp32) contiguous bytes, instead of 16 rows.
//
// The pinned error order over a tile is the width-16 tree applied to the
// sixteen row sums in row order. Its levels of stride 8, 4 (and 2 when
// LPT = 2) pair rows of the same residue mod LPT, so they run inside a lane
// over the lane's own row sums (local strides 8 / LPT, ...); the remaining
// levels (stride LPT / 2, ..., 1) pair lanes of the group and run as DPP row
// shifts; the group's first lane then holds the pinned sum and a quad
// permute broadcasts it. The tile amax is the lane's max over its rows, then
// over the group.
template <int DT> struct Tile16 {
  // lanes per tile: 4 (2 for 16-bit inputs halves the rows per load
  // instruction but needs twice the registers for a tile's raw rows, which
  // costs more occupancy than the access pattern gains)
  static constexpr int kLPT = 4;
  static constexpr int kRPL = 16 / kLPT;              // rows per lane
  static constexpr int kTiles = 64 / kLPT;            // tiles per unit
};

// max over the lanes of a tile group
template <int LPT>
__device__ __forceinline__ float group_max(float v) {
  v = __builtin_fmaxf(v, dpp<0xB1>(v));                      // quad_perm [1,0,3,2]
  if (LPT == 4) v = __builtin_fmaxf(v, dpp<0x4E>(v));        // quad_perm [2,3,0,1]
  return v;
}

// The pinned tree's remaining levels across the group, then the group's
// first lane broadcast to the group.
template <int LPT>
__device__ __forceinline__ float group_tree(float v) {
  if (LPT == 4) v = v + dpp<kDppRowShl + 2>(v);
  v = v + dpp<kDppRowShl + 1>(v);
  return LPT == 4 ? dpp<0x00>(v) : dpp<0xA0>(v);             // quad_perm [0,0,0,0] / [0,0,2,2]
}

// The in-lane levels of the pinned tree over N local row sums (strides N/2,
// ..., 1: position i adds position i + stride). Overwrites w.
template <int N>
__device__ __forceinline__ float lane_tree(float* w) {
#pragma unroll
  for (int s = N / 2; s >= 1; s >>= 1)
#pragma unroll
    for (int i = 0; i < s; i++) w[i] = w[i] + w[i + s];
  return w[0];
}

// Quantize the lane's rows of one tile. raw[i] holds row j + LPT i; done(i)
// runs as soon as raw[i] is no longer needed (the caller refills it with the
// next unit's row). Returns false when the fast form cannot be trusted (a
// NaN in the tile); the caller then reruns with CAREFUL on the same rows. The
// kept candidate is the same on all lanes of the group.
template <int DT, int RECIPE, int METRIC, int PREC, bool CAREFUL, bool NEED_XHAT, class Done>
__device__ __forceinline__ bool tile_rows(Raw<DT>* raw, float S_enc, float S_dec, const Table& tab,
                                          uint32_t (*codes)[2], uint32_t& scale, float (*xh)[16], Done done) {
  constexpr int kLPT = Tile16<DT>::kLPT, kRPL = Tile16<DT>::kRPL;
  // NaN-dropping tile amax; 16-bit inputs straight from their bits (no
  // unpacked row stays live for the encode loop)
  float a = 0.0f;
  if constexpr (DT == kFP32) {
#pragma unroll
    for (int i = 0; i < kRPL; i++) {
      float x[16];
      raw[i].unpack(x);
      a = __builtin_fmaxf(a, amax16<true>(x));
    }
  } else {
    s16x2 k = pair_key<DT>(0u);
#pragma unroll
    for (int i = 0; i < kRPL; i++) {
      const uint32_t w[8] = {(uint32_t)raw[i].a.x, (uint32_t)raw[i].a.y, (uint32_t)raw[i].a.z, (uint32_t)raw[i].a.w,
                             (uint32_t)raw[i].b.x, (uint32_t)raw[i].b.y, (uint32_t)raw[i].b.z, (uint32_t)raw[i].b.w};
#pragma unroll
      for (int t = 0; t < 8; t++) k = __builtin_elementwise_max(k, pair_key<DT>(w[t]));
    }
    a = __uint_as_float(pair_key_to_f32_bits<DT>(k));
  }
  a = group_max<kLPT>(a);
  const Cand k6 = make_cand(div6(a), S_enc, tab);
  if (RECIPE == kNVFP4) {
    float nan = 0.0f;
#pragma unroll
    for (int i = 0; i < kRPL; i++) {
      float x[16];
      raw[i].unpack(x);
      encode16<CAREFUL>(x, k6.E, codes[i][0], codes[i][1]);
      if (NEED_XHAT) decode16(codes[i][0], codes[i][1], k6.D, xh[i]);
      if (!CAREFUL && any_nan16(x)) nan = 1.0f;
      done(i);
    }
    scale = k6.scale;
    return CAREFUL || group_max<kLPT>(nan) == 0.0f;
  } else {
    const Cand k4 = make_cand(a * 0.25f, S_enc, tab);
    float r6[kRPL], r4[kRPL];
    uint32_t c4[kRPL][2];
#pragma unroll
    for (int i = 0; i < kRPL; i++) {
      float x[16], t[16];
      raw[i].unpack(x);
      encode16<CAREFUL>(x, k6.E, codes[i][0], codes[i][1]);
      decode16(codes[i][0], codes[i][1], k6.D, t);
      r6[i] = err16<METRIC, PREC, kOrderTree>(x, t);
      encode16<CAREFUL>(x, k4.E, c4[i][0], c4[i][1]);
      decode16(c4[i][0], c4[i][1], k4.D, t);
      r4[i] = err16<METRIC, PREC, kOrderTree>(x, t);
      done(i);
      __builtin_amdgcn_sched_barrier(0);  // one row at a time (register pressure)
    }
    const float e6 = group_tree<kLPT>(lane_tree<kRPL>(r6));
    const float e4 = group_tree<kLPT>(lane_tree<kRPL>(r4));
    const bool four = e4 < e6;
#pragma unroll
    for (int i = 0; i < kRPL; i++) {
      codes[i][0] = four ? c4[i][0] : codes[i][0];
      codes[i][1] = four ? c4[i][1] : codes[i][1];
      if (NEED_XHAT) decode16(codes[i][0], codes[i][1], four ? k4.D : k6.D, xh[i]);
    }
    scale = four ? k4.scale : k6.scale;
    return CAREFUL || (e6 == e6 && e4 == e4);
  }
}

template <int DT, int RECIPE, int METRIC, int PREC, int GRAN, int OUT>
__global__ void __launch_bounds__(256) k_16x16(const Args16x16 args) {
  __shared__ float lds[4][256];
  constexpr int kB = Raw<DT>::kBytes;
  constexpr int kEB = kB / 16;  // bytes per element
  constexpr bool kXhat = OUT == kOutQdq;
  constexpr int kLPT = Tile16<DT>::kLPT, kRPL = Tile16<DT>::kRPL, kT = Tile16<DT>::kTiles;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const Table tab{lds[wv], lds[wv] + 128};
  const int jr = lane % kLPT, tl = lane / kLPT;  // first row in the tile, tile in the unit
  const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t K = args.K, nbk = K >> 4;
  const int64_t gpb = (nbk + kT - 1) / kT;  // units per band
  const int64_t total = (args.M >> 4) * gpb;
  // per-tensor scales: units dealt round robin over the waves (the waves in
  // flight share one window of the tensor); per-row scales (a table per
  // band): contiguous ranges
  const int64_t stride = GRAN == kGranTensor ? nwaves : 1;
  int64_t u = wave, u_end = total;
  if (GRAN != kGranTensor) wave_range(0, total, wave, nwaves, u, u_end);
  const float six_b = args.six_b;

  if (OUT == kOutQuant && args.sdec_out) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t gsz = (int64_t)gridDim.x * blockDim.x;
    if (GRAN == kGranTensor) {
      if (gid == 0) args.sdec_out[0] = 1.0f / global_encode_scale(args.amax[0], six_b);
    } else {
      for (int64_t r = gid; r < args.M; r += gsz) args.sdec_out[r] = 1.0f / global_encode_scale(args.amax[r], six_b);
    }
  }
  if (u >= u_end) return;

  float S_enc = 1.0f, S_dec = 1.0f;
  if (GRAN == kGranTensor) {
    S_enc = global_encode_scale(ld_const(args.amax, 0), six_b);
    S_dec = 1.0f / S_enc;
    tab.build(S_enc, S_dec, lane);
  }
  int64_t cur_band = -1;
  int64_t cur_amax = -1;  // amax bits of the current table; -1: none built yet
  const int64_t x_bytes = args.M * K * kEB;
  const int64_t c_bytes = args.M * K / 2;
  const int64_t s_bytes = args.M * nbk;
  // the lane's offsets within a unit: row jr + LPT i of tile tl
  const uint32_t ox0 = ((uint32_t)jr * (uint32_t)K + (uint32_t)tl * 16) * kEB;
  const uint32_t ox_step = (uint32_t)(kLPT * K * kEB);
  const uint32_t oc0 = (uint32_t)jr * (uint32_t)(K / 2) + (uint32_t)tl * 8, oc_step = (uint32_t)(kLPT * K / 2);
  const uint32_t os0 = (uint32_t)jr * (uint32_t)nbk + (uint32_t)tl, os_step = (uint32_t)(kLPT * nbk);

  struct U16 {
    Rsrc x, out, scl;
    bool active;
  };
  struct P16 {
    int64_t band, tg;
  };
  const int64_t sb = stride / gpb, st = stride - sb * gpb;  // bands and unit groups per step
  auto advance = [&](P16 p) {
    p.tg += st;
    p.band += sb;
    if (p.tg >= gpb) { p.tg -= gpb; ++p.band; }
    return p;
  };
  auto unit = [&](const P16& p, bool valid) {
    const int64_t t0 = p.tg * kT;                      // first tile of the unit
    const int64_t ex = p.band * 16 * K + t0 * 16;      // its first element
    const int64_t es = p.band * 16 * nbk + t0;         // its first scale
    U16 r;
    r.active = valid && (t0 + tl < nbk);
    r.x = make_rsrc(static_cast<const char*>(args.x) + ex * kEB, valid ? x_bytes - ex * kEB : 0);
    if (OUT == kOutQuant) {
      r.out = make_rsrc(args.codes + ex / 2, valid ? c_bytes - ex / 2 : 0);
      r.scl = make_rsrc(args.scales + es, valid ? s_bytes - es : 0);
    } else {
      r.out = make_rsrc(static_cast<char*>(args.y) + ex * kEB, valid ? x_bytes - ex * kEB : 0);
      r.scl = r.out;
    }
    return r;
  };
  auto load = [&](Raw<DT>* raw, const U16& U) {
#pragma unroll
    for (int i = 0; i < kRPL; i++) raw[i].load(U.x, U.active ? ox0 + i * ox_step : kOOB);
  };

  // The next unit's rows load while this unit is quantized, each into the
  // registers of a row as soon as the row is done (no registers beyond the
  // one unit's rows). A tile that needs the careful form reloads its rows.
  P16 p{u / gpb, u % gpb};
  U16 U = unit(p, true);
  Raw<DT> raw[kRPL];
  load(raw, U);
  for (; u < u_end; u += stride) {
    const P16 pn = advance(p);
    const U16 Un = unit(pn, u + stride < u_end);
    if (GRAN == kGranRow && p.band != cur_band) {
      // tile-uniform contract: the band uses its first row's amax, and a band
      // whose rows differ is flagged
      const float A = ld_const(args.amax, p.band * 16);
      bool uniform = true;
#pragma unroll
      for (int i = 1; i < 16; i++) uniform &= __float_as_uint(ld_const(args.amax, p.band * 16 + i)) == __float_as_uint(A);
      if (!uniform && args.status && lane == 0) atomicOr(args.status, kStatusTileNonuniform);
      if ((int64_t)__float_as_uint(A) != cur_amax) {
        S_enc = global_encode_scale(A, six_b);
        S_dec = 1.0f / S_enc;
        tab.build(S_enc, S_dec, lane);
        cur_amax = __float_as_uint(A);
      }
      cur_band = p.band;
    }
    uint32_t codes[kRPL][2], scale;
    float xh[kXhat ? kRPL : 1][16];
    auto refill = [&](int i) { raw[i].load(Un.x, Un.active ? ox0 + i * ox_step : kOOB); };
    if (!tile_rows<DT, RECIPE, METRIC, PREC, false, kXhat>(raw, S_enc, S_dec, tab, codes, scale, xh, refill)) {
      load(raw, U);
      tile_rows<DT, RECIPE, METRIC, PREC, true, kXhat>(raw, S_enc, S_dec, tab, codes, scale, xh, [](int) {});
      load(raw, Un);
    }
#pragma unroll
    for (int i = 0; i < kRPL; i++) {
      if (OUT == kOutQuant) {
        store_codes(U.out, U.active ? oc0 + i * oc_step : kOOB, codes[i][0], codes[i][1]);
        store_scale(U.scl, U.active ? os0 + i * os_step : kOOB, scale);
      } else {
        store16<DT>(U.out, U.active ? ox0 + i * ox_step : kOOB, xh[i]);
      }
    }
    p = pn;
    U = Un;
  }
}

// ------------------------------------------------------------ columnwise

// Columnwise quantize: the 1x16 quantize of X^T ([K, M]), whose blocks are
// 16 consecutive rows of one column of X (the transposed operand of the
// backward GEMM).
//
// A wave's unit is a tile of 16 bands (256 rows) by 64 columns, and lane j
// owns column j of it: for each band the lane loads its column's 16 values
// (one 2- or 4-byte load per row, so one load instruction is 128 or 256
// contiguous bytes of one row), quantizes that block, and keeps its codes in
// a wave-private LDS area and its scales in a four-register shift queue. The
// next band's rows load while the current band is quantized. When the tile
// is done the lane holds its column's whole 128-byte run of X^T codes and
// 16 scale bytes; the wave writes the runs eight columns per store
// instruction (16 bytes per lane, whole 128-byte lines), so no X^T line is
// assembled from pieces written by different waves. Waves never wait for
// one another.
//
// The scale runs (16 bytes per column per tile) fill an X^T scale line
// together with the seven neighbouring tiles of the same column strip. The
// tile order is arranged so that those eight tiles run on one XCD (whose
// L2 then merges the pieces): workgroup b runs on XCD b % 8, and the tiles
// are dealt out as if the workgroups of one XCD were consecutive.
constexpr int kColTW = 64;  // columns per wave tile

template <int DT>
__device__ __forceinline__ float col_value(uint32_t w) {
  if (DT == kFP32) return __uint_as_float(w);
  if (DT == kBF16) return __uint_as_float(w << 16);
  return f16_lo(w);
}

template <int DT, int RECIPE, int METRIC, int PREC, int ORDER>
__global__ void __launch_bounds__(256) k_colwise(const Args16x16 args) {
  __shared__ float lds_tab[4][256];
  __shared__ uint64_t lds_codes[4][kColTW][17];  // [wave][column][band], padded
  constexpr int kEB = Raw<DT>::kBytes / 16;      // bytes per element
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const Table tab{lds_tab[wv], lds_tab[wv] + 128};
  uint64_t (&cl)[kColTW][17] = lds_codes[wv];
  const int64_t M = args.M, K = args.K;
  const int64_t nbands = M >> 4;
  const int64_t ngroups = (nbands + 15) >> 4, nstrips = (K + kColTW - 1) / kColTW;
  const int64_t total = ngroups * nstrips;
  // XCD-aware order: the grid is a multiple of 8 workgroups
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int64_t wave = ((b & 7) * (G >> 3) + (b >> 3)) * 4 + wv, nwaves = G * 4;
  if (blockIdx.x == 0 && threadIdx.x == 0 && args.sdec_out)
    args.sdec_out[0] = 1.0f / global_encode_scale(args.amax[0], args.six_b);
  if (wave >= total) return;

  const float S_enc = global_encode_scale(ld_const(args.amax, 0), args.six_b);
  const float S_dec = 1.0f / S_enc;
  tab.build(S_enc, S_dec, lane);
  const int64_t x_bytes = M * K * kEB, c_bytes = K * (M >> 1), s_bytes = K * (M >> 4);
  const uint32_t row_bytes = (uint32_t)(K * kEB);

  // Load the lane's 16 values of band bg of tile t (zeros past the tensor).
  auto load_band = [&](int64_t t, int bg, uint32_t (&w)[16]) {
    const int64_t strip = t / ngroups, group = t - strip * ngroups;
    const int64_t band = group * 16 + bg;
    const bool band_ok = t < total && band < nbands;  // wave-uniform
    const int64_t ex = band * 16 * K + strip * kColTW;  // first element of the band's rows in the tile
    const Rsrc rx = make_rsrc(static_cast<const char*>(args.x) + (band_ok ? ex : 0) * kEB,
                              band_ok ? x_bytes - ex * kEB : 0);
    // columns past K: an offset past the resource (kOOB + 15 rows < 2^32)
    const uint32_t lo = strip * kColTW + lane < K ? (uint32_t)(lane * kEB) : kOOB;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      if (DT == kFP32) w[r] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rx, lo + r * row_bytes, 0, 0);
      else w[r] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rx, lo + r * row_bytes, 0, 0);
    }
  };

  uint32_t cur[16], nxt[16];
  load_band(wave, 0, cur);
  for (int64_t t = wave; t < total; t += nwaves) {
    const int64_t strip = t / ngroups, group = t - strip * ngroups;
    uint32_t sq[4] = {0u, 0u, 0u, 0u};  // scale bytes, band 0 ends in the low byte of sq[0]
#pragma unroll 1
    for (int bg = 0; bg < 16; bg++) {
      if (bg < 15) load_band(t, bg + 1, nxt);
      else load_band(t + nwaves, 0, nxt);
      float x[16], xh[16];
#pragma unroll
      for (int r = 0; r < 16; r++) x[r] = col_value<DT>(cur[r]);
      BlockOut o;
      quantize_block<RECIPE, METRIC, PREC, ORDER, false>(x, S_enc, S_dec, tab, o, xh);
      cl[lane][bg] = (uint64_t)o.c0 | ((uint64_t)o.c1 << 32);
      sq[0] = __builtin_amdgcn_alignbit(sq[1], sq[0], 8);
      sq[1] = __builtin_amdgcn_alignbit(sq[2], sq[1], 8);
      sq[2] = __builtin_amdgcn_alignbit(sq[3], sq[2], 8);
      sq[3] = __builtin_amdgcn_alignbit(o.scale, sq[3], 8);
#pragma unroll
      for (int r = 0; r < 16; r++) cur[r] = nxt[r];
    }
    // the lanes of this wave read what other lanes wrote
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int64_t col0 = strip * kColTW;
    const int nvalid = (int)min((int64_t)16, nbands - group * 16);  // bands of this tile in the tensor
    // 16-byte stores where every band is in the tensor and the runs are
    // 16-byte aligned, else 8-byte code and 1-byte scale stores
    const bool wide_c = nvalid == 16 && ((M >> 1) & 15) == 0 && ((uintptr_t)args.codes & 15) == 0;
    const bool wide_s = nvalid == 16 && ((M >> 4) & 15) == 0 && ((uintptr_t)args.scales & 15) == 0;
    const int64_t ec = col0 * (M >> 1) + group * 128, es = col0 * (M >> 4) + group * 16;
    const Rsrc rc = make_rsrc(args.codes + ec, c_bytes - ec);
    const Rsrc rs = make_rsrc(args.scales + es, s_bytes - es);
    // codes: lane L writes bytes 16 (L % 8) .. +15 of column 8 i + L / 8
    const int piece = lane & 7;
#pragma unroll
    for (int i = 0; i < kColTW / 8; i++) {
      const int col = 8 * i + (lane >> 3);
      const bool col_ok = col0 + col < K;
      const uint64_t c0 = cl[col][2 * piece], c1 = cl[col][2 * piece + 1];
      const uint32_t off = (uint32_t)(col * (M >> 1) + 16 * piece);
      if (wide_c) {
        const v4i v = {(int)(uint32_t)c0, (int)(uint32_t)(c0 >> 32), (int)(uint32_t)c1, (int)(uint32_t)(c1 >> 32)};
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, col_ok ? off : kOOB, 0, 0);
      } else {
        store_codes(rc, col_ok && 2 * piece < nvalid ? off : kOOB, (uint32_t)c0, (uint32_t)(c0 >> 32));
        store_codes(rc, col_ok && 2 * piece + 1 < nvalid ? off + 8 : kOOB, (uint32_t)c1, (uint32_t)(c1 >> 32));
      }
    }
    // scales: lane j writes its column's 16 bytes
    {
      const bool col_ok = col0 + lane < K;
      const uint32_t off = (uint32_t)(lane * (M >> 4));
      if (wide_s) {
        const v4i v = {(int)sq[0], (int)sq[1], (int)sq[2], (int)sq[3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, col_ok ? off : kOOB, 0, 0);
      } else {
#pragma unroll
        for (int k = 0; k < 16; k++)
          store_scale(rs, col_ok && k < nvalid ? off + k : kOOB, (sq[k >> 2] >> (8 * (k & 3))) & 0xFFu);
      }
    }
    // the next tile's LDS writes come after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ------------------------------------------------------------ dequantize

// Plain global stores of 16 decoded values as the output type.
template <int DT> __device__ __forceinline__ void put16(void* base, int64_t idx, const float* y);
template <> __device__ __forceinline__ void put16<kBF16>(void* base, int64_t idx, const float* y) {
  uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx);
  p[0] = make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7]));
  p[1] = make_uint4(pack_bf16(y[8], y[9]), pack_bf16(y[10], y[11]), pack_bf16(y[12], y[13]), pack_bf16(y[14], y[15]));
}
template <> __device__ __forceinline__ void put16<kFP16>(void* base, int64_t idx, const float* y) {
  uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx);
  p[0] = make_uint4(pack_f16(y[0], y[1]), pack_f16(y[2], y[3]), pack_f16(y[4], y[5]), pack_f16(y[6], y[7]));
  p[1] = make_uint4(pack_f16(y[8], y[9]), pack_f16(y[10], y[11]), pack_f16(y[12], y[13]), pack_f16(y[14], y[15]));
}
template <> __device__ __forceinline__ void put16<kFP32>(void* base, int64_t idx, const float* y) {
  float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
#pragma unroll
  for (int i = 0; i < 4; i++) p[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
}


// Decode: one lane per half block (8 elements), so that a wave's output
// store is 1 KiB contiguous (16-bit types) and its code load 256 B. A unit
// is 32 blocks of the flattened tensor, or of one row for per-row S_dec;
// waves take units grid-stride, kDqU units per step with all their loads
// issued first. Loads and stores are raw buffer operations (past the end:
// zeros read, stores dropped).
constexpr int kDqU = 4;

template <int DT, int GRAN>
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ sdec, int64_t M, int64_t K, void* y,
                                                 int64_t total_units) {
  constexpr int kOH = Raw<DT>::kBytes / 2;  // output bytes per half block
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t nbk = K >> 4, nblk = M * nbk;
  const int64_t spr = (nbk + 31) / 32;  // units per row (per-row S_dec)
  const uint32_t off_c = lane * 4, off_s = lane >> 1, off_y = lane * kOH;
  // per-row units: (row, segment) of the first unit, advanced by whole steps
  // of nwaves units without dividing per unit
  const int64_t q1 = nwaves / spr, r1 = nwaves - q1 * spr;
  const int64_t first = (int64_t)blockIdx.x * 4 + wv;
  int64_t row0 = (GRAN == kGranTensor) ? 0 : first / spr;
  int64_t seg0 = (GRAN == kGranTensor) ? 0 : first - row0 * spr;
  for (int64_t u0 = first; u0 < total_units; u0 += nwaves * kDqU) {
    Rsrc rc[kDqU], ry[kDqU];
    uint32_t c[kDqU], sc[kDqU];
    float S_dec[kDqU];
    int64_t row = row0, seg = seg0;
#pragma unroll
    for (int j = 0; j < kDqU; j++) {
      const int64_t u = u0 + j * nwaves;
      const bool valid = u < total_units;
      int64_t b0, nvalid;
      if (GRAN == kGranTensor) {
        b0 = u * 32;
        nvalid = min((int64_t)32, nblk - b0);
      } else {
        b0 = row * nbk + seg * 32;
        nvalid = min((int64_t)32, nbk - seg * 32);
      }
      if (!valid) nvalid = 0;
      rc[j] = make_rsrc(codes + b0 * 8, nvalid * 8);
      const Rsrc rs = make_rsrc(scales + b0, nvalid);
      ry[j] = make_rsrc(static_cast<char*>(y) + b0 * 2 * kOH, nvalid * 2 * kOH);
      c[j] = __builtin_amdgcn_raw_buffer_load_b32(rc[j], off_c, 0, 0);
      sc[j] = __builtin_amdgcn_raw_buffer_load_b8(rs, off_s, 0, 0);
      S_dec[j] = (GRAN == kGranTensor) ? ld_const(sdec, 0) : (valid ? ld_const(sdec, row) : 1.0f);
      if (GRAN != kGranTensor) {  // to the unit nwaves further on
        row += q1;
        seg += r1;
        if (seg >= spr) { seg -= spr; ++row; }
      }
    }
    row0 = row;
    seg0 = seg;
#pragma unroll
    for (int j = 0; j < kDqU; j++) {
      float q[8];
      e2m1_unpack8(c[j], q);
      const float D = e4m3_value(sc[j]) * S_dec[j];
#pragma unroll
      for (int i = 0; i < 8; i++) q[i] = q[i] * D;
      store8<DT>(ry[j], off_y, q);
    }
  }
}

// ------------------------------------------------------------ amax

// NaN-dropping |x| max as unsigned bits (NaN patterns count as +0); the
// order of non-negative binary32 values equals the order of their bits.
__device__ __forceinline__ uint32_t mag_bits(float v) {
  const uint32_t m = __float_as_uint(v) & 0x7FFFFFFFu;
  return m <= 0x7F800000u ? m : 0u;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, s, 64));
  return v;
}

// max |x| (as binary32 bits) over 16-element blocks b, b + stride, ... < n16
// of x; four blocks in flight per lane.
template <int DT>
__device__ __forceinline__ uint32_t absmax_blocks(const void* x, int64_t b, int64_t n16, int64_t stride) {
  if constexpr (DT == kFP32) {
    const float4* p = static_cast<const float4*>(x);
    uint32_t m = 0;
    for (; b < n16; b += stride) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float4 v = p[b * 4 + i];
        m = max(max(m, mag_bits(v.x)), max(mag_bits(v.y), max(mag_bits(v.z), mag_bits(v.w))));
      }
    }
    return m;
  } else {
    const uint4* p = static_cast<const uint4*>(x);
    s16x2 k = pair_key<DT>(0u);
    for (; b + 3 * stride < n16; b += 4 * stride) {
      uint4 r[8];
#pragma unroll
      for (int j = 0; j < 4; j++) { r[2 * j] = p[(b + j * stride) * 2]; r[2 * j + 1] = p[(b + j * stride) * 2 + 1]; }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        k = __builtin_elementwise_max(k, pair_key<DT>(r[j].x));
        k = __builtin_elementwise_max(k, pair_key<DT>(r[j].y));
        k = __builtin_elementwise_max(k, pair_key<DT>(r[j].z));
        k = __builtin_elementwise_max(k, pair_key<DT>(r[j].w));
      }
    }
    for (; b < n16; b += stride) {
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const uint4 r = p[b * 2 + j];
        k = __builtin_elementwise_max(k, pair_key<DT>(r.x));
        k = __builtin_elementwise_max(k, pair_key<DT>(r.y));
        k = __builtin_elementwise_max(k, pair_key<DT>(r.z));
        k = __builtin_elementwise_max(k, pair_key<DT>(r.w));
      }
    }
    return pair_key_to_f32_bits<DT>(k);
  }
}

__global__ void k_zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// Per-tensor amax: many small workgroups, so that their completions (and
// their one atomic each) spread over the launch; a workgroup whose maximum
// does not exceed the value already stored skips its atomic. Same-address
// atomics serialize at the memory side, so they are kept few.
template <int DT>
__global__ void __launch_bounds__(256) k_amax_tensor(const void* x, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t m = absmax_blocks<DT>(x, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, n16, stride);
  m = wave_max_u32(m);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t r = max(max(part[0], part[1]), max(part[2], part[3]));
    if (r > __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(out, r);
  }
}

// one wave per row
template <int DT>
__global__ void __launch_bounds__(256) k_amax_row(const void* x, int64_t M, int64_t K, float* out) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t nbk = K >> 4;
  for (int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < M; r += nwaves) {
    uint32_t m = absmax_blocks<DT>(static_cast<const char*>(x) + r * K * (DT == kFP32 ? 4 : 2), lane, nbk, 64);
    m = wave_max_u32(m);
    if (lane == 0) out[r] = __uint_as_float(m);
  }
}

__global__ void k_band16(float* out, int64_t nbands) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nbands; b += (int64_t)gridDim.x * blockDim.x) {
    uint32_t m = 0;
    for (int i = 0; i < 16; i++) m = max(m, __float_as_uint(out[b * 16 + i]));
    for (int i = 0; i < 16; i++) out[b * 16 + i] = __uint_as_float(m);
  }
}

// ------------------------------------------------------------ fused amax + quantize

// One launch for the per-tensor amax and the quantize (the amax pre-pass the
// Megatron-LM page runs as a separate torch reduction, "What does this PR
// do?"). Phase 1: each wave takes the NaN-dropping max |x| over exactly the
// unit range it quantizes later. A grid-wide max barrier combines the
// workgroups' maxima. Phase 2: the 1x16 walk with the combined amax, over
// data the wave just read (largely still in the Infinity Cache).
//
// The barrier is two-level so that same-address atomics stay few (they
// serialize at the memory side): workgroup b arrives at group b % ng with
// an atomic max and a count; the last arrival of a group forwards the group
// max to the top level; the last top arrival publishes the amax and bumps
// the generation word that every workgroup polls (each compares it with the
// value it read before arriving, so the word never needs a reset). Each
// level's counters and maxima are reset by its last arrival, so they are
// zero again when the launch ends.
//
// The grid holds only as many workgroups as fit on the device at once, so
// they all become resident unless other long-running work holds CUs (for
// example a second fused launch on another stream). The poll is bounded
// either way: after args.spin_limit polls a workgroup sets kStatusBarrier
// and returns without quantizing rather than wait forever.

// max |x| bits over blocks [b0, b1) of a flattened tensor: lane l takes
// blocks b0 + l + 64 k, four in flight.
template <int DT>
__device__ __forceinline__ uint32_t range_absmax(const void* x, int64_t b0, int64_t b1, int lane) {
  constexpr int kB = Raw<DT>::kBytes;
  if (b1 <= b0) return 0u;
  const Rsrc r = make_rsrc(static_cast<const char*>(x) + b0 * kB, (b1 - b0) * kB);
  const uint32_t n = (uint32_t)(b1 - b0);
  uint32_t m = 0;                  // fp32: magnitude bits
  s16x2 k = pair_key<DT>(0u);      // 16-bit inputs: packed keys, starting at +0
  for (uint32_t i = 0; i < n; i += 256) {
    Raw<DT> q[4];
#pragma unroll
    for (int j = 0; j < 4; j++) q[j].load(r, (i + 64 * j + lane) * kB);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if constexpr (DT == kFP32) {
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const v4i v = q[j].v[t];
          m = max(max(m, mag_bits(__int_as_float(v.x))), max(mag_bits(__int_as_float(v.y)),
                  max(mag_bits(__int_as_float(v.z)), mag_bits(__int_as_float(v.w)))));
        }
      } else {
        const uint32_t w[8] = {(uint32_t)q[j].a.x, (uint32_t)q[j].a.y, (uint32_t)q[j].a.z, (uint32_t)q[j].a.w,
                               (uint32_t)q[j].b.x, (uint32_t)q[j].b.y, (uint32_t)q[j].b.z, (uint32_t)q[j].b.w};
#pragma unroll
        for (int t = 0; t < 8; t++) k = __builtin_elementwise_max(k, pair_key<DT>(w[t]));
      }
    }
  }
  if constexpr (DT == kFP32) return m;
  else return pair_key_to_f32_bits<DT>(k);
}

constexpr int kBarGroups = 32;  // first-level arrival groups

// Word offsets in the workspace; every counter and maximum sits on a
// 128-byte line of its own. The published word (8-byte aligned) holds the
// barrier's generation in its low half and the launch's combined maximum in
// its high half, so one 64-bit store publishes both and one load reads both.
struct BarWs {
  uint32_t* w;
  __device__ uint64_t* pub() const { return reinterpret_cast<uint64_t*>(w); }
  __device__ uint32_t* gcount(uint32_t g) const { return w + 64 + 32 * g; }
  __device__ uint32_t* gmax(uint32_t g) const { return w + 64 + 32 * (kBarGroups + g); }
  __device__ uint32_t* tcount() const { return w + 64 + 32 * (2 * kBarGroups); }
  __device__ uint32_t* tmax() const { return w + 64 + 32 * (2 * kBarGroups + 1); }
  // grouped calls: their own call counter, and two banks of per-group
  // maxima (8 bytes apart) used by alternate grouped calls
  __device__ uint32_t* ggen() const { return w + 64 + 32 * (2 * kBarGroups + 2); }
  __device__ uint32_t* gslot(uint32_t bank, uint32_t g) const { return w + kSlotBase + 2 * (bank * kMaxFusedGroups + g); }
  static constexpr int kSlotBase = 64 + 32 * (2 * kBarGroups + 4);
};
static_assert((BarWs::kSlotBase + 4 * kMaxFusedGroups) * 4 <= kFusedWorkspaceBytes, "workspace too small");

// Wait until this wave's vector memory operations (atomics included) have
// completed; also a compiler barrier for memory operations.
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Called by one thread per workgroup with the workgroup's max; returns false
// when `spin_limit` polls passed without the barrier completing. The last
// arrival (which runs exactly once per barrier, after every workgroup has
// arrived) also adds 1 to *bump when bump is not null, before publishing.
//
// A workgroup that gives up has still arrived, so the barrier completes once
// the rest of the grid arrives: its counters end at zero and *bump is bumped
// whether or not any workgroup waited for it.
//
// Every value that crosses workgroups travels through an atomic read-modify-
// write or an agent-scope atomic load or store (which the compiler issues
// coherent across the XCDs' L2 caches); the order between two of them is
// kept by waiting for the first to complete before issuing the second. No
// acquire or release fence is used: at agent scope each one writes back or
// invalidates the L2, which, issued by every workgroup, costs far more than
// the barrier itself. Nothing else needs ordering: phase 2 reads only the
// input, which the launch already sees.
//
// g0 is the generation word as read (barrier_generation) before this
// workgroup's arrival; every workgroup of a launch reads the same value,
// since the word changes only after all of them have arrived.
__device__ __forceinline__ uint32_t barrier_generation(const BarWs& ws) {
  const uint64_t p = __hip_atomic_load(ws.pub(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  vm_wait();
  return (uint32_t)p;
}

__device__ bool grid_max_barrier(const BarWs& ws, uint32_t g0, uint32_t m, uint32_t& result, uint32_t* bump,
                                 int spin_limit) {
  constexpr int kA = __HIP_MEMORY_SCOPE_AGENT;
  constexpr int kR = __ATOMIC_RELAXED;
  const uint32_t G = gridDim.x;
  const uint32_t ng = G < (uint32_t)kBarGroups ? G : (uint32_t)kBarGroups;
  const uint32_t g = blockIdx.x % ng;
  const uint32_t gsize = G / ng + (g < G % ng ? 1u : 0u);
  __hip_atomic_fetch_max(ws.gmax(g), m, kR, kA);
  vm_wait();
  if (__hip_atomic_fetch_add(ws.gcount(g), 1u, kR, kA) == gsize - 1) {
    // last of its group: every member's max is in; forward it, reset the group
    const uint32_t gm = __hip_atomic_exchange(ws.gmax(g), 0u, kR, kA);
    __hip_atomic_store(ws.gcount(g), 0u, kR, kA);
    __hip_atomic_fetch_max(ws.tmax(), gm, kR, kA);
    vm_wait();
    if (__hip_atomic_fetch_add(ws.tcount(), 1u, kR, kA) == ng - 1) {
      const uint32_t a = __hip_atomic_exchange(ws.tmax(), 0u, kR, kA);
      __hip_atomic_store(ws.tcount(), 0u, kR, kA);
      if (bump) {
        __hip_atomic_fetch_add(bump, 1u, kR, kA);
        vm_wait();
      }
      __hip_atomic_store(ws.pub(), ((uint64_t)a << 32) | (uint64_t)(g0 + 1u), kR, kA);
    }
  }
  uint64_t p = __hip_atomic_load(ws.pub(), kR, kA);
  for (int it = 0; (uint32_t)p == g0; it++) {
    if (it >= spin_limit) return false;
    __builtin_amdgcn_s_sleep(2);
    p = __hip_atomic_load(ws.pub(), kR, kA);
  }
  result = (uint32_t)(p >> 32);
  return true;
}

template <int DT, int RECIPE, int METRIC, int PREC, int ORDER>
__global__ void __launch_bounds__(256) k_fused(const Args1x16<1> args, uint32_t* workspace, float* amax_out) {
  __shared__ float lds[4][256];
  __shared__ uint32_t part[4];
  __shared__ uint32_t amax_bits;
  __shared__ int ok;
  constexpr int kUB = unit_blocks(kOutQuant, DT);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const Table tab{lds[wv], lds[wv] + 128};
  const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  int64_t u, u_end;  // at most ceil(total_units / nwaves) units
  wave_range(0, args.total_units, wave, nwaves, u, u_end);
  const TensorRef& T = args.t[0];
  const int64_t nblk = T.M * (T.K >> 4);

  // phase 1
  uint32_t m = range_absmax<DT>(T.x, min(nblk, u * kUB), min(nblk, u_end * kUB), lane);
  m = wave_max_u32(m);
  if (lane == 0) part[wv] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    const BarWs ws{workspace};
    const uint32_t g0 = barrier_generation(ws);
    ok = grid_max_barrier(ws, g0, max(max(part[0], part[1]), max(part[2], part[3])), a, nullptr,
                          args.spin_limit) ? 1 : 0;
    amax_bits = a;
    if (!ok && args.status) atomicOr(args.status, kStatusBarrier);
  }
  __syncthreads();
  if (!ok) return;
  const float A = __uint_as_float(amax_bits);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (amax_out) amax_out[0] = A;
    if (args.sdec_out) args.sdec_out[0] = 1.0f / global_encode_scale(A, args.six_b);
  }

  // phase 2: pairs of units dealt round robin, as the quantize takes them
  if (2 * wave >= args.total_units) return;
  walk_1x16<1, DT, RECIPE, METRIC, PREC, ORDER, kGranTensor, kOutQuant, true>(args, tab, lane, 2 * wave,
                                                                              args.total_units, &amax_bits, 2 * nwaves);
}

// ------------------------------------------------------------ on-chip fused amax + quantize

// The fused amax and quantize (or quantize-dequantize) for a tensor that
// fits on chip: when no wave has more than onchip_units() units, each wave
// reads its units once, the first half of them straight into a wave-private
// LDS stage (direct buffer loads: lane l's 16-byte piece k of the stage
// lands at stage + 1024 k + 16 l) and the rest into registers, takes their
// NaN-dropping max, passes the grid barrier of k_fused, and quantizes from
// the stage and the registers. Phase 2 reads nothing from memory, so the
// launch moves each input byte once (k_fused reads it twice).
//
// A lane holds 128 bytes of input on chip: 8 pieces of 16 bytes in the
// stage (8 KiB per wave, 32 KiB per workgroup) and 8 in registers.
constexpr int kOnchipPieces = 8;  // 16-byte pieces per lane, in LDS and again in registers

// 16-byte pieces of a lane's part of one unit
__host__ __device__ constexpr int unit_pieces(int out, int dt) {
  return unit_blocks(out, dt) / 64 * (dt == kFP32 ? 4 : 2);
}
// units a wave holds on chip (half staged in LDS, half in registers)
__host__ __device__ constexpr int onchip_units(int out, int dt) { return 2 * kOnchipPieces / unit_pieces(out, dt); }

// Piece k (16 bytes) of a lane's part of a quantize unit: its byte offset in
// the unit, and the register it is held in (16-bit types: two blocks of two
// pieces; fp32: one block of four).
template <int DT, int OUT = kOutQuant>
__device__ __forceinline__ uint32_t piece_offset(int lane, int k) {
  if (DT == kFP32) return lane * 64 + k * 16;
  return (k >> 1) * 64 * 32 + unit_block_of_lane<DT, OUT>(lane) * 32 + (k & 1) * 16;
}
// Direct load to LDS: each lane reads 16 bytes at voffset of r and the
// hardware writes lane l's bytes to dst + 16 l (64 lanes: 1 KiB).
__device__ __forceinline__ void load_lds16(Rsrc r, v4i* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voffset, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ v4i& piece(Raw<DT>* r, int k) {
  if constexpr (DT == kFP32) return r[0].v[k];
  else return (k & 1) ? r[k >> 1].b : r[k >> 1].a;
}

// Running NaN-dropping max |x| of raw pieces: magnitude bits for fp32,
// packed 16-bit keys for the 16-bit types.
template <int DT>
struct PieceMax {
  uint32_t m = 0;
  s16x2 k = pair_key<DT>(0u);
  __device__ void add(const v4i p) {
    if constexpr (DT == kFP32) {
      m = max(max(m, mag_bits(__int_as_float(p.x))), max(mag_bits(__int_as_float(p.y)),
              max(mag_bits(__int_as_float(p.z)), mag_bits(__int_as_float(p.w)))));
    } else {
      k = __builtin_elementwise_max(k, pair_key<DT>((uint32_t)p.x));
      k = __builtin_elementwise_max(k, pair_key<DT>((uint32_t)p.y));
      k = __builtin_elementwise_max(k, pair_key<DT>((uint32_t)p.z));
      k = __builtin_elementwise_max(k, pair_key<DT>((uint32_t)p.w));
    }
  }
  __device__ uint32_t bits() const {
    if constexpr (DT == kFP32) return m;
    else return pair_key_to_f32_bits<DT>(k);
  }
};

template <int DT, int RECIPE, int METRIC, int PREC, int ORDER, int OUT>
__global__ void __launch_bounds__(256) k_fused_onchip(const Args1x16<1> args, uint32_t* workspace, float* amax_out) {
  constexpr int kUB = unit_blocks(OUT, DT);
  constexpr int kNB = kUB / 64;
  constexpr int kB = Raw<DT>::kBytes;
  constexpr int kPieces = unit_pieces(OUT, DT);
  constexpr int kOnchipLds = kOnchipPieces / kPieces;  // units per wave staged in LDS
  constexpr int kOnchipReg = kOnchipLds;               // units per wave held in registers
  static_assert(sizeof(Raw<DT>) * kNB == 16 * kPieces, "a lane's unit is kPieces 16-byte pieces");
  static_assert(kOnchipLds * kPieces == kOnchipPieces, "whole units in the stage");
  __shared__ float lds[4][256];
  __shared__ v4i stage[4][kOnchipLds][kPieces][64];
  __shared__ uint32_t part[4];
  __shared__ uint32_t amax_bits;
  __shared__ int ok;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const Table tab{lds[wv], lds[wv] + 128};
  const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  int64_t u, u_end;  // at most ceil(total_units / nwaves) units
  wave_range(0, args.total_units, wave, nwaves, u, u_end);
  const TensorRef& T = args.t[0];
  const int64_t nblk = T.M * (T.K >> 4);
  const Walk<DT, kGranTensor, OUT> W(T, args.codes, args.scales);
  // diagnostics: the wave's real-time clock at its start, when its loads
  // have landed, when the barrier releases it and at its end
  const bool stamp = args.phase_ts != nullptr && wave < args.phase_cap;  // wave-uniform
  uint64_t ts[3] = {0, 0, 0};
  if (stamp) ts[0] = __builtin_amdgcn_s_memrealtime();
  auto finish = [&]() {
    if (stamp && lane == 0) {
      const uint64_t t3 = __builtin_amdgcn_s_memrealtime();
      unsigned long long* o = args.phase_ts + 4 * wave;
      o[0] = ts[0];
      o[1] = ts[1];
      o[2] = ts[2];
      o[3] = t3;
    }
  };

  // phase 1: read every unit once; units past the wave's range have empty
  // resources (their loads read zeros and are never used)
  Raw<DT> R[kOnchipReg][kNB];
#pragma unroll
  for (int t = 0; t < kOnchipLds; t++) {
    const Unit U = W.unit(W.at(u + t), u + t < u_end, T.M);
#pragma unroll
    for (int k = 0; k < kPieces; k++) load_lds16(U.x, &stage[wv][t][k][0], piece_offset<DT, OUT>(lane, k));
  }
#pragma unroll
  for (int r = 0; r < kOnchipReg; r++) {
    const Unit U = W.unit(W.at(u + kOnchipLds + r), u + kOnchipLds + r < u_end, T.M);
#pragma unroll
    for (int j = 0; j < kNB; j++) R[r][j].load(U.x, unit_block_of_lane<DT, OUT>(lane) * kB + j * 64 * kB);
  }
  vm_wait();  // the loads, the LDS-bound ones included, have landed
  if (stamp) ts[1] = __builtin_amdgcn_s_memrealtime();
  PieceMax<DT> pm;
#pragma unroll
  for (int t = 0; t < kOnchipLds; t++) {
    // only blocks of the tensor count: a stage lane past its end holds
    // whatever an earlier launch left there
    const int64_t nvalid = (u + t < u_end) ? min((int64_t)kUB, nblk - (u + t) * kUB) : 0;
#pragma unroll
    for (int k = 0; k < kPieces; k++) {
      const int64_t blk = (DT == kFP32 ? 0 : (k >> 1) * 64) + unit_block_of_lane<DT, OUT>(lane);
      if (blk < nvalid) pm.add(stage[wv][t][k][lane]);
    }
  }
#pragma unroll
  for (int r = 0; r < kOnchipReg; r++)
#pragma unroll
    for (int k = 0; k < kPieces; k++) pm.add(piece<DT>(R[r], k));
  const uint32_t m = wave_max_u32(pm.bits());
  if (lane == 0) part[wv] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    const BarWs ws{workspace};
    const uint32_t g0 = barrier_generation(ws);
    ok = grid_max_barrier(ws, g0, max(max(part[0], part[1]), max(part[2], part[3])), a, nullptr,
                          args.spin_limit) ? 1 : 0;
    amax_bits = a;
    if (!ok && args.status) atomicOr(args.status, kStatusBarrier);
  }
  __syncthreads();
  if (!ok) return;
  if (stamp) ts[2] = __builtin_amdgcn_s_memrealtime();
  const float A = __uint_as_float(amax_bits);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (amax_out) amax_out[0] = A;
    if (args.sdec_out) args.sdec_out[0] = 1.0f / global_encode_scale(A, args.six_b);
  }

  // phase 2: the register units, then the staged ones
  if (u >= u_end) {
    finish();
    return;
  }
  const float S_enc = global_encode_scale(A, args.six_b);
  const float S_dec = 1.0f / S_enc;
  tab.build(S_enc, S_dec, lane);
#pragma unroll
  for (int r = 0; r < kOnchipReg; r++) {
    const int64_t v = u + kOnchipLds + r;
    if (v < u_end)
      unit_1x16<DT, RECIPE, METRIC, PREC, ORDER, OUT>(R[r], S_enc, S_dec, tab, W.unit(W.at(v), true, T.M), lane);
  }
#pragma unroll
  for (int t = 0; t < kOnchipLds; t++) {
    const int64_t v = u + t;
    if (v < u_end) {
      Raw<DT> q[kNB];
#pragma unroll
      for (int k = 0; k < kPieces; k++) piece<DT>(q, k) = stage[wv][t][k][lane];
      unit_1x16<DT, RECIPE, METRIC, PREC, ORDER, OUT>(q, S_enc, S_dec, tab, W.unit(W.at(v), true, T.M), lane);
    }
  }
  finish();
}

// ------------------------------------------------------------ fused per-row amax + quantize

// Per-row global scales need no grid-wide step: each wave takes whole rows
// (row w, w + nwaves, ...), takes a row's NaN-dropping max, writes the row's
// amax and S_dec, and quantizes the row.
//
// A row of at most kRowStage units (8 KiB: bf16 and fp16 up to K = 4096,
// fp32 up to 2048) is read once, into a wave-private LDS stage with direct
// buffer loads; the wave copies it to registers, starts the next row's loads
// into the stage, and takes the amax and the quantize from the registers, so
// the next row's read overlaps this row's compute. A longer row is read for
// its max and then quantized with the 1x16 walk, whose loads find the row
// in the L2 cache.
template <int DT, int RECIPE, int METRIC, int PREC, int ORDER>
__global__ void __launch_bounds__(256) k_fused_row(const Args1x16<1> args, float* amax_out) {
  constexpr int kUB = unit_blocks(kOutQuant, DT);
  constexpr int kNB = kUB / 64;
  constexpr int kPieces = unit_pieces(kOutQuant, DT);
  constexpr int kRowStage = kOnchipPieces / kPieces;  // units of a row the stage holds
  __shared__ float lds[4][256];
  __shared__ uint32_t row_amax[4];
  __shared__ v4i stage[4][kRowStage][kPieces][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const Table tab{lds[wv], lds[wv] + 128};
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const TensorRef& T = args.t[0];
  const int64_t nbk = T.K >> 4, spr = (nbk + kUB - 1) / kUB;
  const float six_b = args.six_b;
  const int64_t r0 = (int64_t)blockIdx.x * 4 + wv;

  auto publish = [&](int64_t r, uint32_t m) {
    const float A = __uint_as_float(m);
    if (lane == 0) {
      if (amax_out) amax_out[r] = A;
      if (args.sdec_out) args.sdec_out[r] = 1.0f / global_encode_scale(A, six_b);
    }
  };

  if (spr > kRowStage) {
    for (int64_t r = r0; r < T.M; r += nwaves) {
      const uint32_t m = wave_max_u32(range_absmax<DT>(T.x, r * nbk, (r + 1) * nbk, lane));
      publish(r, m);
      if (lane == 0) row_amax[wv] = m;
      // the lanes read the word lane 0 wrote
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      walk_1x16<1, DT, RECIPE, METRIC, PREC, ORDER, kGranRow, kOutQuant, true>(args, tab, lane, r * spr,
                                                                              (r + 1) * spr, &row_amax[wv]);
    }
    return;
  }

  const Walk<DT, kGranRow, kOutQuant> W(T, args.codes, args.scales);
  auto stage_row = [&](int64_t r) {  // the row's units into the stage (rows past the end: nothing read)
#pragma unroll
    for (int t = 0; t < kRowStage; t++) {
      const Unit U = W.unit(UPos{r * spr + t, r, t}, r < T.M && t < spr, T.M);
#pragma unroll
      for (int k = 0; k < kPieces; k++) load_lds16(U.x, &stage[wv][t][k][0], piece_offset<DT>(lane, k));
    }
  };
  stage_row(r0);
  for (int64_t r = r0; r < T.M; r += nwaves) {
    Raw<DT> R[kRowStage][kNB];
    vm_wait();  // the row has landed in the stage
#pragma unroll
    for (int t = 0; t < kRowStage; t++)
#pragma unroll
      for (int k = 0; k < kPieces; k++) piece<DT>(R[t], k) = stage[wv][t][k][lane];
    // the copies have left the stage before the next row's loads overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    stage_row(r + nwaves);
    // NaN-dropping max over the row's blocks: a lane past the row's end
    // holds whatever an earlier row or launch left in the stage
    PieceMax<DT> pm;
    const v4i zero = {0, 0, 0, 0};  // +0: leaves the max unchanged
#pragma unroll
    for (int t = 0; t < kRowStage; t++) {
      const int64_t nvalid = t < spr ? min((int64_t)kUB, nbk - t * kUB) : 0;
#pragma unroll
      for (int k = 0; k < kPieces; k++) {
        const int64_t blk = (DT == kFP32) ? lane : (k >> 1) * 64 + lane;
        pm.add(blk < nvalid ? piece<DT>(R[t], k) : zero);
      }
    }
    const uint32_t m = wave_max_u32(pm.bits());
    publish(r, m);
    const float S_enc = global_encode_scale(__uint_as_float(m), six_b);
    const float S_dec = 1.0f / S_enc;
    tab.build(S_enc, S_dec, lane);
#pragma unroll
    for (int t = 0; t < kRowStage; t++)
      if (t < spr)
        unit_1x16<DT, RECIPE, METRIC, PREC, ORDER, kOutQuant>(R[t], S_enc, S_dec, tab,
                                                             W.unit(UPos{r * spr + t, r, t}, true, T.M), lane);
  }
  vm_wait();  // no stage load outlives the wave
}

// Grouped (MoE) amax and quantize in one launch: the per-group amaxes the
// grouped quantize takes as input (pytorch/ao PR, MoE commit) computed in
// phase 1 of the same launch. Each wave takes the NaN-dropping max over the
// part of its unit range in each group it touches (rows at or past
// offs[G-1] are padding and are skipped); the workgroup combines its waves'
// maxima in LDS and adds them to the group slots of the workspace with
// atomic maxima; the grid barrier then orders every addition before any
// read. Phase 2 is the grouped 1x16 walk with the group amaxes held in LDS.
//
// Slots are banked: a grouped call accumulates in bank ggen % 2 (ggen counts
// grouped calls and is read before arriving, so every workgroup sees the
// same value), and workgroup 0 clears all of the other bank, which the next
// grouped call uses. The barrier's last arrival bumps ggen, so the next call
// moves to the cleared bank even when some workgroups (workgroup 0
// included) gave up waiting.
template <int DT, int RECIPE, int METRIC, int PREC, int ORDER>
__global__ void __launch_bounds__(256) k_fused_grouped(const Args1x16<1> args, uint32_t* workspace, float* amax_out) {
  constexpr int kA = __HIP_MEMORY_SCOPE_AGENT;
  constexpr int kR = __ATOMIC_RELAXED;
  __shared__ float lds[4][256];
  __shared__ uint32_t gm[kMaxFusedGroups];
  __shared__ uint32_t gen0, bank;
  __shared__ int ok;
  constexpr int kUB = unit_blocks(kOutQuant, DT);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const Table tab{lds[wv], lds[wv] + 128};
  const BarWs ws{workspace};
  const int G = args.G;
  const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  // phase 1 reads the data rows, each wave a contiguous range of the data
  // units; phase 2 takes the data units, then the padding units (zeros
  // written), in pairs dealt round robin as in the grouped quantize
  const int64_t D = grouped_data_units<DT>(args);
  int64_t u, u_end;
  wave_range(0, D, wave, nwaves, u, u_end);
  const TensorRef& T = args.t[0];
  const int64_t nbk = T.K >> 4, spr = (nbk + kUB - 1) / kUB;
  const bool flat = grouped_flat(T.K, kUB);

  for (int g = threadIdx.x; g < G; g += blockDim.x) gm[g] = 0u;
  if (threadIdx.x == 0) {
    gen0 = barrier_generation(ws);
    bank = __hip_atomic_load(ws.ggen(), kR, kA) & 1u;
  }
  if (args.status) {  // the offsets contract, as the grouped quantize checks it
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t g = gid; g < G; g += (int64_t)gridDim.x * blockDim.x) {
      const int32_t prev = g ? args.offs[g - 1] : 0;
      const int32_t o = args.offs[g];
      if (o < prev || (o & 15) || (g == G - 1 && (int64_t)o > T.M)) atomicOr(args.status, kStatusBadOffs);
    }
  }
  __syncthreads();
  if (blockIdx.x == 0)  // every slot: the next grouped call may have more groups
    for (int g = threadIdx.x; g < kMaxFusedGroups; g += blockDim.x) __hip_atomic_store(ws.gslot(bank ^ 1u, g), 0u, kR, kA);

  // phase 1: the wave's units are the blocks [b0, b1) of the flattened
  // tensor (flat units, or per-row segments in order), clipped to the rows
  // that hold data
  const int64_t rows_read = min(max((int64_t)ld_const(args.offs, G - 1), (int64_t)0), T.M);
  if (u < u_end) {
    int64_t r0, b0, b1;
    if (flat) {
      b0 = u * kUB;
      b1 = min(min(u_end * kUB, T.M * nbk), rows_read * nbk);
      r0 = b0 / nbk;
    } else {
      r0 = u / spr;
      const int64_t r1 = (u_end - 1) / spr;
      b0 = r0 * nbk + (u - r0 * spr) * kUB;
      b1 = min(r1 * nbk + min(nbk, ((u_end - 1) - r1 * spr + 1) * kUB), rows_read * nbk);
    }
    if (b0 < b1) {
      for (int g = group_of(args.offs, G, r0); g < G; g++) {
        const int64_t g_end = (int64_t)ld_const(args.offs, g) * nbk;
        const int64_t lo = max(b0, g ? (int64_t)ld_const(args.offs, g - 1) * nbk : (int64_t)0);
        const int64_t hi = min(b1, g_end);
        if (lo < hi) {
          const uint32_t m = wave_max_u32(range_absmax<DT>(T.x, lo, hi, lane));
          if (lane == 0 && m) atomicMax(&gm[g], m);
        }
        if (g_end >= b1) break;
      }
    }
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x)
    if (gm[g]) __hip_atomic_fetch_max(ws.gslot(bank, g), gm[g], kR, kA);
  vm_wait();  // this wave's additions are done before the workgroup arrives
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t unused = 0;
    ok = grid_max_barrier(ws, gen0, 0u, unused, ws.ggen(), args.spin_limit) ? 1 : 0;
    if (!ok && args.status) atomicOr(args.status, kStatusBarrier);
  }
  __syncthreads();
  if (!ok) return;
  for (int g = threadIdx.x; g < G; g += blockDim.x) gm[g] = __hip_atomic_load(ws.gslot(bank, g), kR, kA);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
      const float A = __uint_as_float(gm[g]);
      if (amax_out) amax_out[g] = A;
      if (args.sdec_out) args.sdec_out[g] = 1.0f / global_encode_scale(A, args.six_b);
    }
  }

  // phase 2 (the pairs dealt round robin: no better for phase 1's reads)
  const int64_t stride = 2 * nwaves;
  u = 2 * wave;
  if (u < D) walk_1x16<1, DT, RECIPE, METRIC, PREC, ORDER, kGranGroup, kOutQuant, true>(args, tab, lane, u, D, gm, stride);
  u = D + 2 * wave;
  if (u < args.total_units)
    walk_1x16<1, DT, RECIPE, METRIC, PREC, ORDER, kGranGroup, kOutQuant, true>(args, tab, lane, u, args.total_units, gm,
                                                                               stride);
}

// ------------------------------------------------------------ fused amaxes + QDQ list

// Every tensor's amax and the fused QDQ of a list of tensors in one launch:
// the per-weight FP32 amax pre-pass of the Megatron-LM page's fake-
// quantization loop ("What does this PR do?", "Performance": the fused
// primary includes one amax per weight) folded into the list launch. Phase
// 1: each wave takes the NaN-dropping max |x| over the part of its unit
// range in each tensor it touches; the workgroup combines its waves' maxima
// per tensor in LDS and adds them to the workspace's slots (banked as for
// the grouped kernel, whose slots and call counter it shares). After the
// grid barrier, phase 2 is the list walk of the QDQ with the tensor amaxes
// held in LDS; it reads the inputs a second time, from the Infinity Cache
// when the list fits there.
template <int DT, int RECIPE, int METRIC, int PREC, int ORDER>
__global__ void __launch_bounds__(256) k_fused_list(const Args1x16<kMaxList> args, uint32_t* workspace) {
  constexpr int kA = __HIP_MEMORY_SCOPE_AGENT;
  constexpr int kR = __ATOMIC_RELAXED;
  constexpr int kUB = unit_blocks(kOutQdq, DT);
  __shared__ float lds[kListTables][256];  // a table per wave, or per tensor (phase 2 of short lists)
  __shared__ float lscl[kListTables][2];
  __shared__ uint32_t gm[kMaxList];
  __shared__ uint32_t gen0, bank;
  __shared__ int ok;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const Table tab{lds[wv], lds[wv] + 128};
  const BarWs ws{workspace};
  const int n = args.n;
  const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  int64_t u, u_end;  // at most ceil(total_units / nwaves) units
  wave_range(0, args.total_units, wave, nwaves, u, u_end);

  for (int t = threadIdx.x; t < n; t += blockDim.x) gm[t] = 0u;
  if (threadIdx.x == 0) {
    gen0 = barrier_generation(ws);
    bank = __hip_atomic_load(ws.ggen(), kR, kA) & 1u;
  }
  __syncthreads();
  if (blockIdx.x == 0)  // every slot: the next banked call may have more groups or tensors
    for (int g = threadIdx.x; g < kMaxFusedGroups; g += blockDim.x) __hip_atomic_store(ws.gslot(bank ^ 1u, g), 0u, kR, kA);

  // phase 1: the wave's units [u, u_end) intersected with each tensor's
  // units; a tensor's units are 64 consecutive blocks of its flattened data
  if (u < u_end) {
    int ti = 0;
    while (ti + 1 < n && args.t[ti + 1].unit_begin <= u) ti++;
    for (; ti < n; ti++) {
      const TensorRef& T = args.t[ti];
      const int64_t tb = T.unit_begin;
      const int64_t te = (ti + 1 < n) ? args.t[ti + 1].unit_begin : args.total_units;
      const int64_t lo = max(u, tb), hi = min(u_end, te);
      if (lo < hi) {
        const int64_t nblk = T.M * (T.K >> 4);
        const uint32_t m = wave_max_u32(range_absmax<DT>(T.x, (lo - tb) * kUB, min(nblk, (hi - tb) * kUB), lane));
        if (lane == 0 && m) atomicMax(&gm[ti], m);
      }
      if (te >= u_end) break;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += blockDim.x)
    if (gm[t]) __hip_atomic_fetch_max(ws.gslot(bank, t), gm[t], kR, kA);
  vm_wait();  // this wave's additions are done before the workgroup arrives
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t unused = 0;
    ok = grid_max_barrier(ws, gen0, 0u, unused, ws.ggen(), args.spin_limit) ? 1 : 0;
    if (!ok && args.status) atomicOr(args.status, kStatusBarrier);
  }
  __syncthreads();
  if (!ok) return;
  for (int t = threadIdx.x; t < n; t += blockDim.x) gm[t] = __hip_atomic_load(ws.gslot(bank, t), kR, kA);
  __syncthreads();
  if (blockIdx.x == 0)
    for (int t = threadIdx.x; t < n; t += blockDim.x)
      if (args.t[t].amax_out) args.t[t].amax_out[0] = __uint_as_float(gm[t]);

  // phase 2: up to kListTables tensors, the units of the list in pairs dealt
  // round robin with every tensor's table in LDS, as the QDQ list takes them;
  // longer lists, the wave's contiguous range
  if (n <= kListTables) {
    if (threadIdx.x < n) {
      const float S_enc = global_encode_scale(__uint_as_float(gm[threadIdx.x]), args.six_b);
      lscl[threadIdx.x][0] = S_enc;
      lscl[threadIdx.x][1] = 1.0f / S_enc;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n * 128; i += blockDim.x)
      table_entry(i & 127, lscl[i >> 7][0], lscl[i >> 7][1], lds[i >> 7], lds[i >> 7] + 128);
    __syncthreads();
    if (2 * wave < args.total_units)
      walk_list_rr<kMaxList, DT, RECIPE, METRIC, PREC, ORDER, kOutQdq>(args, lds, lscl, lane, 2 * wave, 2 * nwaves);
    return;
  }
  if (u >= u_end) return;
  walk_1x16<kMaxList, DT, RECIPE, METRIC, PREC, ORDER, kGranTensor, kOutQdq, true>(args, tab, lane, u, u_end, gm);
}

// ------------------------------------------------------------ dispatch

// workgroups of 256 threads for an n-item elementwise helper (capped)
static unsigned small_grid(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 1024 ? 1024 : g));
}

// compute units of the current device
static int64_t num_cus() {
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  return cus;
}

// Workgroups of 256 threads resident at once for kernel fn: the grid of the
// unit-walking kernels (each wave then walks its share of the units).
static int64_t resident_grid(const void* fn) {
  int dev = 0, cus = 0, per_cu = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || per_cu <= 0) per_cu = 2;
  return (int64_t)cus * per_cu;
}

template <int NT, int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT>
static hipError_t launch_1x16_t(const Args1x16<NT>& a, hipStream_t s) {
  auto* fn = &k_1x16<NT, DT, RECIPE, METRIC, PREC, ORDER, GRAN, OUT>;
  static const int64_t resident = resident_grid(reinterpret_cast<const void*>(fn));
  static const int64_t cap = OUT == kOutQuant ? min(resident, 4 * num_cus()) : resident;
  // Launches whose units go out round robin and give each wave of that grid
  // at least 16 units run with 4 times as many workgroups: the later ones
  // start as the first ones finish, which evens out the end of the launch
  // (grouped step 242.5 -> 231.6 us; 2 times: 233.7, 8 times: 235.8).
  const bool rr = (a.n == 1 && GRAN != kGranRow) || (NT > 1 && a.n <= kListTables && OUT == kOutQdq);
  const int64_t c = rr && a.total_units >= 16 * 4 * cap ? 4 * cap : cap;
  const int64_t grid = max((int64_t)1, min(c, (a.total_units + 3) / 4));
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT>
static hipError_t launch_fused_t(const Args1x16<1>& a, uint32_t* ws, float* amax_out, hipStream_t s) {
  static_assert(GRAN == kGranTensor && OUT == kOutQuant, "fused: per-tensor quantize only");
  auto* fn = &k_fused<DT, RECIPE, METRIC, PREC, ORDER>;
  auto* fn_chip = &k_fused_onchip<DT, RECIPE, METRIC, PREC, ORDER, kOutQuant>;
  static const int64_t resident = resident_grid(reinterpret_cast<const void*>(fn));
  static const int64_t resident_chip = resident_grid(reinterpret_cast<const void*>(fn_chip));
  // the on-chip form when its resident grid leaves each wave at most
  // onchip_units units (the tensor then fits in the waves' registers and
  // LDS stages), else the two-read form
  const int64_t grid_chip = max((int64_t)1, min(resident_chip, (a.total_units + 3) / 4));
  const bool chip = a.total_units <= grid_chip * 4 * onchip_units(kOutQuant, DT);
  const int64_t grid = chip ? grid_chip : max((int64_t)1, min(resident, (a.total_units + 3) / 4));
  Args1x16<1> args = a;
  void* params[] = {&args, &ws, &amax_out};
  if (chip) return hipLaunchKernel(reinterpret_cast<const void*>(fn_chip), dim3((unsigned)grid), dim3(256), params, 0, s);
  // A plain launch: a cooperative one costs about 16 us more per call on
  // this device. The grid holds only the workgroups that fit at once, so on
  // a GPU without other long-running work all of them are resident.
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid), dim3(256), params, 0, s);
}

template <int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT>
static hipError_t launch_fused_row_t(const Args1x16<1>& a, float* amax_out, hipStream_t s) {
  static_assert(GRAN == kGranRow && OUT == kOutQuant, "fused per-row: quantize");
  auto* fn = &k_fused_row<DT, RECIPE, METRIC, PREC, ORDER>;
  static const int64_t resident = resident_grid(reinterpret_cast<const void*>(fn));
  const int64_t grid = max((int64_t)1, min(resident, (a.t[0].M + 3) / 4));
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, s, a, amax_out);
  return hipGetLastError();
}

// Fused amax + QDQ: the on-chip form only; *done is false (and nothing is
// launched) when the tensor does not fit, and the caller then runs the amax
// and the QDQ as two launches.
template <int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT>
static hipError_t launch_fused_qdq_t(const Args1x16<1>& a, uint32_t* ws, float* amax_out, bool* done, hipStream_t s) {
  static_assert(GRAN == kGranTensor && OUT == kOutQdq, "fused QDQ: per-tensor scale");
  auto* fn = &k_fused_onchip<DT, RECIPE, METRIC, PREC, ORDER, kOutQdq>;
  static const int64_t resident = resident_grid(reinterpret_cast<const void*>(fn));
  const int64_t grid = max((int64_t)1, min(resident, (a.total_units + 3) / 4));
  *done = a.total_units <= grid * 4 * onchip_units(kOutQdq, DT);
  if (!*done) return hipSuccess;
  Args1x16<1> args = a;
  void* params[] = {&args, &ws, &amax_out};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid), dim3(256), params, 0, s);
}

template <int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT>
static hipError_t launch_fused_grouped_t(const Args1x16<1>& a, uint32_t* ws, float* amax_out, hipStream_t s) {
  static_assert(GRAN == kGranGroup && OUT == kOutQuant, "fused grouped: grouped quantize only");
  auto* fn = &k_fused_grouped<DT, RECIPE, METRIC, PREC, ORDER>;
  static const int64_t resident = resident_grid(reinterpret_cast<const void*>(fn));
  const int64_t grid = max((int64_t)1, min(resident, (a.total_units + 3) / 4));
  Args1x16<1> args = a;
  void* params[] = {&args, &ws, &amax_out};
  // a plain launch of the resident grid, as for the per-tensor fused kernel
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid), dim3(256), params, 0, s);
}

template <int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT>
static hipError_t launch_fused_list_t(const Args1x16<kMaxList>& a, uint32_t* ws, hipStream_t s) {
  static_assert(GRAN == kGranTensor && OUT == kOutQdq, "fused list: per-tensor QDQ only");
  auto* fn = &k_fused_list<DT, RECIPE, METRIC, PREC, ORDER>;
  static const int64_t resident = resident_grid(reinterpret_cast<const void*>(fn));
  const int64_t grid = max((int64_t)1, min(resident, (a.total_units + 3) / 4));
  Args1x16<kMaxList> args = a;
  void* params[] = {&args, &ws};
  // a plain launch of the resident grid, as for the other fused kernels
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid), dim3(256), params, 0, s);
}

template <int DT, int RECIPE, int METRIC, int PREC, int ORDER, int GRAN, int OUT>
static hipError_t launch_colwise_t(const Args16x16& a, hipStream_t s) {
  static_assert(GRAN == kGranTensor && OUT == kOutQuant, "columnwise: per-tensor quantize only");
  auto* fn = &k_colwise<DT, RECIPE, METRIC, PREC, ORDER>;
  static const int64_t resident = resident_grid(reinterpret_cast<const void*>(fn));
  // one wave per tile up to the resident grid, in whole groups of 8
  // workgroups (the kernel's XCD-aware tile order needs a multiple of 8)
  const int64_t tiles = ((a.M / 16 + 15) / 16) * ((a.K + kColTW - 1) / kColTW);
  const int64_t grid = 8 * max((int64_t)1, min(resident / 8, (tiles + 31) / 32));
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int RECIPE, int METRIC, int PREC, int GRAN, int OUT>
static hipError_t launch_16x16_t(const Args16x16& a, hipStream_t s) {
  auto* fn = &k_16x16<DT, RECIPE, METRIC, PREC, GRAN, OUT>;
  static const int64_t resident = resident_grid(reinterpret_cast<const void*>(fn));
  constexpr int kT = Tile16<DT>::kTiles;
  const int64_t units = (a.M / 16) * ((a.K / 16 + kT - 1) / kT);
  const int64_t grid = max((int64_t)1, min(resident, (units + 3) / 4));
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Expand the runtime knobs into template instances. Every mode is a compiled
// specialization; the kernels never branch on a mode. FOS_MODES covers the
// 1x16 kernels (with the error order), FOS_MODES_T the 16x16 kernel (tree
// order only).
#define FOS_MODES(DT, GRAN, OUT, CALL)                                                                      \
  if (recipe == kNVFP4) return CALL(DT, kNVFP4, kMSE, kErrExact, kOrderTree, GRAN, OUT);                     \
  if (order == kOrderSeq) {                                                                                  \
    if (metric == kMAE && prec == kErrExact) return CALL(DT, k4over6, kMAE, kErrExact, kOrderSeq, GRAN, OUT); \
    if (metric == kMAE && prec == kErrFP16) return CALL(DT, k4over6, kMAE, kErrFP16, kOrderSeq, GRAN, OUT);   \
    if (metric == kMSE && prec == kErrExact) return CALL(DT, k4over6, kMSE, kErrExact, kOrderSeq, GRAN, OUT); \
    return CALL(DT, k4over6, kMSE, kErrFP16, kOrderSeq, GRAN, OUT);                                          \
  }                                                                                                          \
  if (metric == kMAE && prec == kErrExact) return CALL(DT, k4over6, kMAE, kErrExact, kOrderTree, GRAN, OUT);  \
  if (metric == kMAE && prec == kErrFP16) return CALL(DT, k4over6, kMAE, kErrFP16, kOrderTree, GRAN, OUT);    \
  if (metric == kMSE && prec == kErrExact) return CALL(DT, k4over6, kMSE, kErrExact, kOrderTree, GRAN, OUT);  \
  return CALL(DT, k4over6, kMSE, kErrFP16, kOrderTree, GRAN, OUT);

#define FOS_MODES_T(DT, GRAN, OUT, CALL)                                                          \
  if (recipe == kNVFP4) return CALL(DT, kNVFP4, kMSE, kErrExact, GRAN, OUT);                     \
  if (metric == kMAE && prec == kErrExact) return CALL(DT, k4over6, kMAE, kErrExact, GRAN, OUT); \
  if (metric == kMAE && prec == kErrFP16) return CALL(DT, k4over6, kMAE, kErrFP16, GRAN, OUT);   \
  if (metric == kMSE && prec == kErrExact) return CALL(DT, k4over6, kMSE, kErrExact, GRAN, OUT); \
  return CALL(DT, k4over6, kMSE, kErrFP16, GRAN, OUT);

#define FOS_DTYPES(MODES, GRAN, OUT, CALL)           \
  if (dt == kBF16) { MODES(kBF16, GRAN, OUT, CALL) } \
  if (dt == kFP16) { MODES(kFP16, GRAN, OUT, CALL) } \
  { MODES(kFP32, GRAN, OUT, CALL) }

#define CALL_Q1(DT, R, M, P, O, G, OUT) launch_1x16_t<1, DT, R, M, P, O, G, OUT>(a, s)
#define CALL_QL(DT, R, M, P, O, G, OUT) launch_1x16_t<kMaxList, DT, R, M, P, O, G, OUT>(a, s)
#define CALL_F(DT, R, M, P, O, G, OUT) launch_fused_t<DT, R, M, P, O, G, OUT>(a, ws, amax_out, s)
#define CALL_T(DT, R, M, P, G, OUT) launch_16x16_t<DT, R, M, P, G, OUT>(a, s)

hipError_t launch_quant_1x16(int dt, int recipe, int metric, int prec, int order, int gran, const Args1x16<1>& a,
                             hipStream_t s) {
  if (gran == kGranTensor) { FOS_DTYPES(FOS_MODES, kGranTensor, kOutQuant, CALL_Q1) }
  if (gran == kGranRow) { FOS_DTYPES(FOS_MODES, kGranRow, kOutQuant, CALL_Q1) }
  FOS_DTYPES(FOS_MODES, kGranGroup, kOutQuant, CALL_Q1)
}

hipError_t launch_fused(int dt, int recipe, int metric, int prec, int order, const Args1x16<1>& a, uint32_t* ws,
                        float* amax_out, hipStream_t s) {
  FOS_DTYPES(FOS_MODES, kGranTensor, kOutQuant, CALL_F)
}

#define CALL_FQ(DT, R, M, P, O, G, OUT) launch_fused_qdq_t<DT, R, M, P, O, G, OUT>(a, ws, amax_out, done, s)
#define CALL_FR(DT, R, M, P, O, G, OUT) launch_fused_row_t<DT, R, M, P, O, G, OUT>(a, amax_out, s)

hipError_t launch_fused_row(int dt, int recipe, int metric, int prec, int order, const Args1x16<1>& a,
                            float* amax_out, hipStream_t s) {
  FOS_DTYPES(FOS_MODES, kGranRow, kOutQuant, CALL_FR)
}

hipError_t launch_fused_qdq(int dt, int recipe, int metric, int prec, int order, const Args1x16<1>& a, uint32_t* ws,
                            float* amax_out, bool* done, hipStream_t s) {
  FOS_DTYPES(FOS_MODES, kGranTensor, kOutQdq, CALL_FQ)
}

#define CALL_FG(DT, R, M, P, O, G, OUT) launch_fused_grouped_t<DT, R, M, P, O, G, OUT>(a, ws, amax_out, s)

hipError_t launch_fused_grouped(int dt, int recipe, int metric, int prec, int order, const Args1x16<1>& a,
                                uint32_t* ws, float* amax_out, hipStream_t s) {
  FOS_DTYPES(FOS_MODES, kGranGroup, kOutQuant, CALL_FG)
}

hipError_t launch_qdq_1x16(int dt, int recipe, int metric, int prec, int order, int gran,
                           const Args1x16<kMaxList>& a, hipStream_t s) {
  if (gran == kGranTensor) { FOS_DTYPES(FOS_MODES, kGranTensor, kOutQdq, CALL_QL) }
  FOS_DTYPES(FOS_MODES, kGranRow, kOutQdq, CALL_QL)
}

#define CALL_FL(DT, R, M, P, O, G, OUT) launch_fused_list_t<DT, R, M, P, O, G, OUT>(a, ws, s)

hipError_t launch_fused_list(int dt, int recipe, int metric, int prec, int order, const Args1x16<kMaxList>& a,
                             uint32_t* ws, hipStream_t s) {
  FOS_DTYPES(FOS_MODES, kGranTensor, kOutQdq, CALL_FL)
}

#define CALL_C(DT, R, M, P, O, G, OUT) launch_colwise_t<DT, R, M, P, O, G, OUT>(a, s)

hipError_t launch_colwise(int dt, int recipe, int metric, int prec, int order, const Args16x16& a, hipStream_t s) {
  FOS_DTYPES(FOS_MODES, kGranTensor, kOutQuant, CALL_C)
}

hipError_t launch_16x16(int dt, int recipe, int metric, int prec, int gran, int out, const Args16x16& a,
                        hipStream_t s) {
  if (out == kOutQuant) {
    if (gran == kGranTensor) { FOS_DTYPES(FOS_MODES_T, kGranTensor, kOutQuant, CALL_T) }
    FOS_DTYPES(FOS_MODES_T, kGranRow, kOutQuant, CALL_T)
  }
  if (gran == kGranTensor) { FOS_DTYPES(FOS_MODES_T, kGranTensor, kOutQdq, CALL_T) }
  FOS_DTYPES(FOS_MODES_T, kGranRow, kOutQdq, CALL_T)
}

template <int DT, int GRAN>
static hipError_t launch_dequant_t(const uint8_t* codes, const uint8_t* scales, const float* sdec, int64_t M,
                                   int64_t K, void* y, hipStream_t s) {
  const int64_t nbk = K / 16;
  const int64_t units = (GRAN == kGranTensor) ? (M * nbk + 31) / 32 : M * ((nbk + 31) / 32);
  // many workgroups: a write-heavy stream keeps more stores in flight that way
  const int64_t grid = max((int64_t)1, min((int64_t)8192, (units + 4 * kDqU - 1) / (4 * kDqU)));
  hipLaunchKernelGGL((k_dequant<DT, GRAN>), dim3((unsigned)grid), dim3(256), 0, s, codes, scales, sdec, M, K, y,
                     units);
  return hipGetLastError();
}

hipError_t launch_dequant(int dt, int gran, const uint8_t* codes, const uint8_t* scales, const float* sdec,
                          int64_t M, int64_t K, void* y, hipStream_t s) {
#define FOS_DQ(DT, G) return launch_dequant_t<DT, G>(codes, scales, sdec, M, K, y, s)
  if (dt == kBF16) { if (gran == kGranTensor) FOS_DQ(kBF16, kGranTensor); else FOS_DQ(kBF16, kGranRow); }
  else if (dt == kFP16) { if (gran == kGranTensor) FOS_DQ(kFP16, kGranTensor); else FOS_DQ(kFP16, kGranRow); }
  else { if (gran == kGranTensor) FOS_DQ(kFP32, kGranTensor); else FOS_DQ(kFP32, kGranRow); }
#undef FOS_DQ
  return hipGetLastError();
}

hipError_t launch_amax(int dt, int gran, const void* x, int64_t M, int64_t K, float* out, int grid, hipStream_t s) {
  if (gran == kAmaxTensor) {
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, s, reinterpret_cast<uint32_t*>(out), (int64_t)1);
    const int64_t n16 = M * K / 16;
    uint32_t* o = reinterpret_cast<uint32_t*>(out);
    if (dt == kBF16) hipLaunchKernelGGL(k_amax_tensor<kBF16>, dim3(grid), dim3(256), 0, s, x, n16, o);
    else if (dt == kFP16) hipLaunchKernelGGL(k_amax_tensor<kFP16>, dim3(grid), dim3(256), 0, s, x, n16, o);
    else hipLaunchKernelGGL(k_amax_tensor<kFP32>, dim3(grid), dim3(256), 0, s, x, n16, o);
    return hipGetLastError();
  }
  if (dt == kBF16) hipLaunchKernelGGL(k_amax_row<kBF16>, dim3(grid), dim3(256), 0, s, x, M, K, out);
  else if (dt == kFP16) hipLaunchKernelGGL(k_amax_row<kFP16>, dim3(grid), dim3(256), 0, s, x, M, K, out);
  else hipLaunchKernelGGL(k_amax_row<kFP32>, dim3(grid), dim3(256), 0, s, x, M, K, out);
  if (gran == kAmaxBand16) {
    const int64_t nb = M / 16;
    hipLaunchKernelGGL(k_band16, dim3(small_grid(nb)), dim3(256), 0, s, out, nb);
  }
  return hipGetLastError();
}

hipError_t launch_zero_u32(void* p, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_u32, dim3(small_grid(n)), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace fos
