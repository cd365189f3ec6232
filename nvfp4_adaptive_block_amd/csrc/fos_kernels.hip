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
// Work mapping (1x16 blocks): one lane owns one 16-element block, so the
// block amax, both candidates, the 16-term error tree and the selection stay
// in that lane's registers; a wave covers 64 consecutive blocks (2 KiB of
// bf16, read with 128-bit loads) and walks a contiguous range of such units,
// so per-row global scales are recomputed only when a lane's row changes.
// 16x16 tiles: a lane owns one 16-element row segment of a tile, 16 lanes
// (one DPP row) hold a tile, and the tile amax and error sums cross lanes.
#include "fos_device.h"
#include "fos_kernels.h"

namespace fos {

// ------------------------------------------------------------ loads/stores

template <int DT> struct Io;

template <> struct Io<kBF16> {
  static constexpr int kBytes = 2;
  __device__ static void load16(const void* base, int64_t idx, float* x) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
  }
  __device__ static void store16(void* base, int64_t idx, const float* y) {
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx);
    uint4 a, b;
    a.x = pack_bf16(y[0], y[1]); a.y = pack_bf16(y[2], y[3]); a.z = pack_bf16(y[4], y[5]); a.w = pack_bf16(y[6], y[7]);
    b.x = pack_bf16(y[8], y[9]); b.y = pack_bf16(y[10], y[11]); b.z = pack_bf16(y[12], y[13]); b.w = pack_bf16(y[14], y[15]);
    p[0] = a;
    p[1] = b;
  }
};

template <> struct Io<kFP16> {
  static constexpr int kBytes = 2;
  __device__ static void load16(const void* base, int64_t idx, float* x) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) { x[2 * i] = f16_lo(w[i]); x[2 * i + 1] = f16_hi(w[i]); }
  }
  __device__ static void store16(void* base, int64_t idx, const float* y) {
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx);
    uint4 a, b;
    a.x = pack_f16(y[0], y[1]); a.y = pack_f16(y[2], y[3]); a.z = pack_f16(y[4], y[5]); a.w = pack_f16(y[6], y[7]);
    b.x = pack_f16(y[8], y[9]); b.y = pack_f16(y[10], y[11]); b.z = pack_f16(y[12], y[13]); b.w = pack_f16(y[14], y[15]);
    p[0] = a;
    p[1] = b;
  }
};

template <> struct Io<kFP32> {
  static constexpr int kBytes = 4;
  __device__ static void load16(const void* base, int64_t idx, float* x) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float4 v = p[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
  }
  __device__ static void store16(void* base, int64_t idx, const float* y) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; i++) p[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
  }
};

// ------------------------------------------------------------ block pieces

// NaN-dropping max |x| over 16 values. The fast form uses v_max3_f32, which
// is exact whenever no element is NaN; a block holding a NaN is always
// recomputed by the careful form (integer max over the magnitude bits with
// NaN patterns mapped to +0).
template <bool CAREFUL>
__device__ __forceinline__ float amax16(const float* x) {
  if (CAREFUL) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      uint32_t m = __float_as_uint(x[i]) & 0x7FFFFFFFu;
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

// One candidate's block scale and multipliers: t = RN(q * S_enc) with q the
// already divided amax (RN(a/6) or RN(a/4)); scale = E4M3(t); encode
// multiplier E = RN(S_enc / sigma) (0 for sigma = 0, FLT_MAX on overflow);
// decode multiplier D = RN(sigma * S_dec).
struct Cand {
  uint32_t scale;
  float E, D;
};

__device__ __forceinline__ Cand make_cand(float q, float S_enc, float S_dec) {
  Cand c;
  float t = q * S_enc;
  c.scale = e4m3_code(t);
  float sigma = e4m3_value(c.scale);
  bool zero = sigma == 0.0f;
  float e = S_enc / (zero ? 1.0f : sigma);
  c.E = zero ? 0.0f : __builtin_fminf(e, kFltMax);
  c.D = sigma * S_dec;
  return c;
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

// Error terms of one row segment (16 elements) and their pinned tree sum.
template <int METRIC, int PREC>
__device__ __forceinline__ float err16(const float* x, const float* xh) {
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    float r = (PREC == kErrFP16) ? round_f16(xh[i]) : xh[i];
    float e = x[i] - r;
    u[i] = (METRIC == kMAE) ? __builtin_fabsf(e) : e * e;
  }
  return tree16(u);
}

// Everything a kernel needs to store for one block (or one tile row).
struct BlockOut {
  uint32_t c0, c1;  // 16 E2M1 codes
  uint32_t scale;   // E4M3 code
  float D;          // decode multiplier of the kept candidate
};

// Quantize one 1x16 block held in x. When NEED_XHAT, xh receives the kept
// candidate's decoded values. Returns false when the fast form cannot be
// trusted (the block holds a NaN); the caller then reruns with CAREFUL.
template <int RECIPE, int METRIC, int PREC, bool CAREFUL, bool NEED_XHAT>
__device__ __forceinline__ bool block_1x16(const float* x, float S_enc, float S_dec, BlockOut& o, float* xh) {
  const float a = amax16<CAREFUL>(x);
  const Cand k6 = make_cand(a / 6.0f, S_enc, S_dec);
  uint32_t c60, c61;
  encode16<CAREFUL>(x, k6.E, c60, c61);
  if (RECIPE == kNVFP4) {
    o.c0 = c60; o.c1 = c61; o.scale = k6.scale; o.D = k6.D;
    if (NEED_XHAT) decode16(c60, c61, k6.D, xh);
    return CAREFUL || !any_nan16(x);
  } else {
    const Cand k4 = make_cand(a * 0.25f, S_enc, S_dec);
    uint32_t c40, c41;
    encode16<CAREFUL>(x, k4.E, c40, c41);
    float xh6[16], xh4[16];
    decode16(c60, c61, k6.D, xh6);
    decode16(c40, c41, k4.D, xh4);
    const float e6 = err16<METRIC, PREC>(x, xh6);
    const float e4 = err16<METRIC, PREC>(x, xh4);
    const bool four = e4 < e6;
    o.c0 = four ? c40 : c60;
    o.c1 = four ? c41 : c61;
    o.scale = four ? k4.scale : k6.scale;
    o.D = four ? k4.D : k6.D;
    if (NEED_XHAT) {
#pragma unroll
      for (int i = 0; i < 16; i++) xh[i] = four ? xh4[i] : xh6[i];
    }
    return CAREFUL || (e6 == e6 && e4 == e4);
  }
}

// Quantize one 16x16 tile: this lane holds one 16-element row segment, the
// 16 lanes of its DPP row hold the tile's rows 0..15 in lane order. The tile
// amax is the max over the lanes; each lane sums its row's error terms with
// the pinned tree, and the lane sums are combined with the same tree in row
// order. The result (kept candidate) is the same on all 16 lanes.
template <int RECIPE, int METRIC, int PREC, bool CAREFUL, bool NEED_XHAT>
__device__ __forceinline__ bool tile_16x16(const float* x, float S_enc, float S_dec, BlockOut& o, float* xh) {
  const float a = max16_lanes(amax16<CAREFUL>(x));
  const Cand k6 = make_cand(a / 6.0f, S_enc, S_dec);
  uint32_t c60, c61;
  encode16<CAREFUL>(x, k6.E, c60, c61);
  if (RECIPE == kNVFP4) {
    o.c0 = c60; o.c1 = c61; o.scale = k6.scale; o.D = k6.D;
    if (NEED_XHAT) decode16(c60, c61, k6.D, xh);
    if (CAREFUL) return true;
    float n = any_nan16(x) ? 1.0f : 0.0f;
    return max16_lanes(n) == 0.0f;
  } else {
    const Cand k4 = make_cand(a * 0.25f, S_enc, S_dec);
    uint32_t c40, c41;
    encode16<CAREFUL>(x, k4.E, c40, c41);
    float xh6[16], xh4[16];
    decode16(c60, c61, k6.D, xh6);
    decode16(c40, c41, k4.D, xh4);
    float e6 = tree16_lanes(err16<METRIC, PREC>(x, xh6));
    float e4 = tree16_lanes(err16<METRIC, PREC>(x, xh4));
    e6 = __shfl(e6, 0, 16);
    e4 = __shfl(e4, 0, 16);
    const bool four = e4 < e6;
    o.c0 = four ? c40 : c60;
    o.c1 = four ? c41 : c61;
    o.scale = four ? k4.scale : k6.scale;
    o.D = four ? k4.D : k6.D;
    if (NEED_XHAT) {
#pragma unroll
      for (int i = 0; i < 16; i++) xh[i] = four ? xh4[i] : xh6[i];
    }
    return CAREFUL || (e6 == e6 && e4 == e4);
  }
}

__device__ __forceinline__ void store_codes(uint8_t* codes, int64_t byte_idx, uint32_t c0, uint32_t c1) {
  *reinterpret_cast<uint2*>(codes + byte_idx) = make_uint2(c0, c1);
}

// ------------------------------------------------------------ 1x16 kernel

// Lane position inside a tensor: (row, column block), advanced by 64 blocks
// per unit.
struct Pos {
  int64_t row, cb;
};

__device__ __forceinline__ Pos pos_of(int64_t b, int64_t nbk) { return Pos{b / nbk, b % nbk}; }

__device__ __forceinline__ void advance(Pos& p, int64_t nbk, int64_t dr, int64_t dc) {
  p.row += dr;
  p.cb += dc;
  if (p.cb >= nbk) { p.cb -= nbk; p.row += 1; }
}

// Row -> group through the cumulative end offsets (binary search: the first
// g with r < offs[g]); G >= 1 and r < offs[G-1].
__device__ __forceinline__ int group_of(const int32_t* offs, int G, int64_t r) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (r < (int64_t)offs[mid]) hi = mid; else lo = mid + 1;
  }
  return lo;
}

template <int NT, int DT, int RECIPE, int METRIC, int PREC, int GRAN, int OUT>
__global__ void __launch_bounds__(256) k_1x16(const Args1x16<NT> args) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t total = args.total_units;
  const int64_t per = (total + nwaves - 1) / nwaves;
  int64_t u = wave * per;
  const int64_t u_end = min(total, u + per);
  if (u >= u_end) return;

  // locate the tensor holding unit u
  int ti = 0;
  while (ti + 1 < args.n && args.t[ti + 1].unit_begin <= u) ti++;

  const float six_b = args.six_b;
  for (;;) {
    const TensorRef T = args.t[ti];
    const int64_t nbk = T.K >> 4;
    const int64_t unit_end_t = (ti + 1 < args.n) ? args.t[ti + 1].unit_begin : total;
    const int64_t dr = 64 / nbk, dc = 64 % nbk;
    Pos p = pos_of((u - T.unit_begin) * 64 + lane, nbk);
    const int64_t M_rows = T.M;            // rows to write
    // rows holding data: all of them, or for a grouped launch the rows
    // before offs[G-1] (clamped to the allocation)
    int64_t M_read = T.M;
    if (GRAN == kGranGroup) M_read = min(max((int64_t)args.offs[args.G - 1], (int64_t)0), T.M);

    float S_enc = 1.0f, S_dec = 1.0f;
    int64_t cur_row = -1;
    if (GRAN == kGranTensor) {
      S_enc = global_encode_scale(T.amax[0], six_b);
      S_dec = 1.0f / S_enc;
    }
    const int64_t stop = min(u_end, unit_end_t);
    for (; u < stop; ++u, advance(p, nbk, dr, dc)) {
      if (p.row >= M_rows) continue;
      const int64_t elem = p.row * T.K + p.cb * 16;
      if (GRAN == kGranGroup && p.row >= M_read) {
        // over-allocated tail: not read, zero codes and scale
        store_codes(args.codes, elem >> 1, 0u, 0u);
        args.scales[p.row * nbk + p.cb] = 0;
        continue;
      }
      if (GRAN != kGranTensor && p.row != cur_row) {
        float A;
        if (GRAN == kGranRow) A = T.amax[p.row];
        else A = args.group_amax[group_of(args.offs, args.G, p.row)];
        S_enc = global_encode_scale(A, six_b);
        S_dec = 1.0f / S_enc;
        cur_row = p.row;
      }
      float x[16];
      Io<DT>::load16(T.x, elem, x);
      BlockOut o;
      float xh[16];
      constexpr bool kXhat = OUT == kOutQdq;
      if (!block_1x16<RECIPE, METRIC, PREC, false, kXhat>(x, S_enc, S_dec, o, xh))
        block_1x16<RECIPE, METRIC, PREC, true, kXhat>(x, S_enc, S_dec, o, xh);
      if (OUT == kOutQuant) {
        store_codes(args.codes, elem >> 1, o.c0, o.c1);
        args.scales[p.row * nbk + p.cb] = (uint8_t)o.scale;
      } else {
        Io<DT>::store16(T.y, elem, xh);
      }
    }
    if (u >= u_end) break;
    ti++;
  }
}

// ------------------------------------------------------------ 16x16 kernel

// A unit is one 16-row band times four consecutive tiles: lane = 16 * tile +
// row in tile, so a wave reads 16 rows x 64 columns.
template <int DT, int RECIPE, int METRIC, int PREC, int GRAN, int OUT>
__global__ void __launch_bounds__(256) k_16x16(const Args16x16 args) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, tq = lane >> 4;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t nbk = args.K >> 4;
  const int64_t groups_per_band = (nbk + 3) >> 2;
  const int64_t total = (args.M >> 4) * groups_per_band;
  const int64_t per = (total + nwaves - 1) / nwaves;
  int64_t u = wave * per;
  const int64_t u_end = min(total, u + per);
  const float six_b = args.six_b;

  float S_enc = 1.0f, S_dec = 1.0f;
  if (GRAN == kGranTensor) {
    S_enc = global_encode_scale(args.amax[0], six_b);
    S_dec = 1.0f / S_enc;
  }
  int64_t cur_band = -1;
  for (; u < u_end; ++u) {
    const int64_t band = u / groups_per_band;
    const int64_t cb = (u % groups_per_band) * 4 + tq;
    const int64_t row = band * 16 + r16;
    if (GRAN == kGranRow && band != cur_band) {
      // tile-uniform contract: the tile uses its first row's amax
      const float A_mine = args.amax[row];
      const float A = __shfl(A_mine, 0, 16);
      if (__float_as_uint(A_mine) != __float_as_uint(A) && args.status) atomicOr(args.status, kStatusTileNonuniform);
      S_enc = global_encode_scale(A, six_b);
      S_dec = 1.0f / S_enc;
      cur_band = band;
    }
    if (cb >= nbk) continue;  // whole 16-lane group idles together
    const int64_t elem = row * args.K + cb * 16;
    float x[16];
    Io<DT>::load16(args.x, elem, x);
    BlockOut o;
    float xh[16];
    constexpr bool kXhat = OUT == kOutQdq;
    if (!tile_16x16<RECIPE, METRIC, PREC, false, kXhat>(x, S_enc, S_dec, o, xh))
      tile_16x16<RECIPE, METRIC, PREC, true, kXhat>(x, S_enc, S_dec, o, xh);
    if (OUT == kOutQuant) {
      store_codes(args.codes, elem >> 1, o.c0, o.c1);
      args.scales[row * nbk + cb] = (uint8_t)o.scale;
    } else {
      Io<DT>::store16(args.y, elem, xh);
    }
  }
}

// ------------------------------------------------------------ dequantize

template <int DT, int GRAN>
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ sdec, int64_t M, int64_t K, void* y) {
  const int64_t nbk = K >> 4;
  const int64_t nblk = M * nbk;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
    const int64_t row = b / nbk;
    const float S_dec = (GRAN == kGranTensor) ? sdec[0] : sdec[row];
    const uint2 c = *reinterpret_cast<const uint2*>(codes + b * 8);
    const float D = e4m3_value(scales[b]) * S_dec;
    float xh[16];
    decode16(c.x, c.y, D, xh);
    Io<DT>::store16(y, b * 16, xh);
  }
}

// ------------------------------------------------------------ amax

// NaN-dropping |x| max as unsigned bits (NaN patterns count as +0); the
// order of non-negative binary32 values equals the order of their bits.
__device__ __forceinline__ uint32_t mag_bits(float v) {
  uint32_t m = __float_as_uint(v) & 0x7FFFFFFFu;
  return m <= 0x7F800000u ? m : 0u;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, s, 64));
  return v;
}

__global__ void k_zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

template <int DT>
__global__ void __launch_bounds__(256) k_amax_tensor(const void* x, int64_t n16, uint32_t* out) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n16; b += stride) {
    float v[16];
    Io<DT>::load16(x, b * 16, v);
#pragma unroll
    for (int i = 0; i < 16; i++) m = max(m, mag_bits(v[i]));
  }
  m = wave_max_u32(m);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = max(max(part[0], part[1]), max(part[2], part[3]));
    atomicMax(out, r);
  }
}

// one wave per row
template <int DT>
__global__ void __launch_bounds__(256) k_amax_row(const void* x, int64_t M, int64_t K, float* out) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t nbk = K >> 4;
  for (int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < M; r += nwaves) {
    uint32_t m = 0;
    for (int64_t cb = lane; cb < nbk; cb += 64) {
      float v[16];
      Io<DT>::load16(x, r * K + cb * 16, v);
#pragma unroll
      for (int i = 0; i < 16; i++) m = max(m, mag_bits(v[i]));
    }
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

// S_dec outputs: per tensor [1], per row [M] or per group [G]
__global__ void k_sdec(const float* amax, int64_t n, float six_b, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = 1.0f / global_encode_scale(amax[i], six_b);
}

// offs contract check: monotone, multiples of 16, last <= M_alloc
__global__ void k_check_offs(const int32_t* offs, int G, int64_t M_alloc, int32_t* status) {
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int32_t prev = g ? offs[g - 1] : 0;
    const bool bad = offs[g] < prev || (offs[g] & 15) || (g == G - 1 && (int64_t)offs[g] > M_alloc);
    if (bad && status) atomicOr(status, kStatusBadOffs);
  }
}

// ------------------------------------------------------------ dispatch

// workgroups of 256 threads for an n-item elementwise helper (capped)
static unsigned small_grid(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 1024 ? 1024 : g));
}

template <int DT, int RECIPE, int METRIC, int PREC, int GRAN, int OUT>
static hipError_t launch_1x16_t(const Args1x16<1>& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_1x16<1, DT, RECIPE, METRIC, PREC, GRAN, OUT>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int RECIPE, int METRIC, int PREC, int GRAN, int OUT>
static hipError_t launch_list_t(const Args1x16<kMaxList>& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_1x16<kMaxList, DT, RECIPE, METRIC, PREC, GRAN, OUT>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int RECIPE, int METRIC, int PREC, int GRAN, int OUT>
static hipError_t launch_16x16_t(const Args16x16& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_16x16<DT, RECIPE, METRIC, PREC, GRAN, OUT>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Expand the runtime knobs into template instances. Every mode is a compiled
// specialization; the kernels never branch on a mode.
#define FOS_MODES(DT, GRAN, OUT, FN)                                                         \
  if (recipe == kNVFP4) return FN<DT, kNVFP4, kMSE, kErrExact, GRAN, OUT>(a, grid, s);      \
  if (metric == kMAE && prec == kErrExact) return FN<DT, k4over6, kMAE, kErrExact, GRAN, OUT>(a, grid, s); \
  if (metric == kMAE && prec == kErrFP16) return FN<DT, k4over6, kMAE, kErrFP16, GRAN, OUT>(a, grid, s);   \
  if (metric == kMSE && prec == kErrExact) return FN<DT, k4over6, kMSE, kErrExact, GRAN, OUT>(a, grid, s); \
  return FN<DT, k4over6, kMSE, kErrFP16, GRAN, OUT>(a, grid, s);

#define FOS_DTYPES(GRAN, OUT, FN)                       \
  if (dt == kBF16) { FOS_MODES(kBF16, GRAN, OUT, FN) } \
  if (dt == kFP16) { FOS_MODES(kFP16, GRAN, OUT, FN) } \
  { FOS_MODES(kFP32, GRAN, OUT, FN) }

hipError_t launch_quant_1x16(int dt, int recipe, int metric, int prec, int gran, const Args1x16<1>& a, int grid,
                             hipStream_t s) {
  if (gran == kGranTensor) { FOS_DTYPES(kGranTensor, kOutQuant, launch_1x16_t) }
  if (gran == kGranRow) { FOS_DTYPES(kGranRow, kOutQuant, launch_1x16_t) }
  FOS_DTYPES(kGranGroup, kOutQuant, launch_1x16_t)
}

hipError_t launch_qdq_1x16(int dt, int recipe, int metric, int prec, const Args1x16<kMaxList>& a, int grid,
                           hipStream_t s) {
  if (dt == kBF16) { FOS_MODES(kBF16, kGranTensor, kOutQdq, launch_list_t) }
  FOS_MODES(kFP16, kGranTensor, kOutQdq, launch_list_t)
}

hipError_t launch_quant_16x16(int dt, int recipe, int metric, int prec, int gran, const Args16x16& a, int grid,
                              hipStream_t s) {
  if (gran == kGranTensor) { FOS_DTYPES(kGranTensor, kOutQuant, launch_16x16_t) }
  FOS_DTYPES(kGranRow, kOutQuant, launch_16x16_t)
}

hipError_t launch_dequant(int dt, int gran, const uint8_t* codes, const uint8_t* scales, const float* sdec,
                          int64_t M, int64_t K, void* y, int grid, hipStream_t s) {
#define FOS_DQ(DT, G) hipLaunchKernelGGL((k_dequant<DT, G>), dim3(grid), dim3(256), 0, s, codes, scales, sdec, M, K, y)
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

hipError_t launch_sdec(const float* amax, int64_t n, float six_b, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_sdec, dim3(small_grid(n)), dim3(256), 0, s, amax, n, six_b, out);
  return hipGetLastError();
}

hipError_t launch_zero_u32(void* p, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_u32, dim3(small_grid(n)), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_check_offs(const int32_t* offs, int G, int64_t M_alloc, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_check_offs, dim3(1), dim3(256), 0, s, offs, G, M_alloc, status);
  return hipGetLastError();
}

}  // namespace fos
