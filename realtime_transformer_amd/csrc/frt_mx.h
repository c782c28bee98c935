// frt_mx.h -- MXFP4 element and block-scale conversions on the device.
//
// OCP Microscaling MXFP4 (the 4-bit FFN variant modelled on the NVFP4 encoder
// FFN of the itsolotime article, section 7.2): blocks of 32 values along the
// reduction dimension share one E8M0 exponent e (scale 2^(e-127)); elements
// are FP4 E2M1 codes (sign bit 3; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
//   e = floor(log2(amax)) - 2 + 127 clamped to [0, 254] (0 for amax == 0)
//   code = E2M1(v * 2^(127-e)), round to nearest with ties to the even
//   mantissa, saturating at 6; the sign bit follows v
// Packing: element 2i in the low nibble of byte i.
#pragma once
#include "frt_device.h"

namespace frt {

// Packed MXFP4 weights (k_mx.hip): codes 1 KiB per (16-row group, 128-K
// block), lane l's 16 bytes = row l%16, K sub-block l/16; exponents 64 lanes
// x 4 bytes per (group, four K blocks), byte j = K block 4*kb4 + j.
__host__ __device__ __forceinline__ size_t mx_code_off(uint32_t prow, uint32_t kb, uint32_t lane, uint32_t KB) {
  return (((size_t)(prow >> 4) * KB + kb) * 64 + lane) * 16;
}
__host__ __device__ __forceinline__ size_t mx_scale_off(uint32_t prow, uint32_t kb, uint32_t lane, uint32_t KB) {
  return (((size_t)(prow >> 4) * (KB >> 2) + (kb >> 2)) * 64 + lane) * 4 + (kb & 3);
}

// MXFP4 down matrix in the column-quad order of the whole-column decode
// down GEMV (K % 512 == 0): quad n / 4 owns K / 512 steps of 512 values;
// in step t lane l holds column 4 (n / 4) + (l & 3), the 32 values at
// 512 t + 128 p + 32 (l >> 4) with part p = (l & 15) >> 2 -- 16 code bytes
// (1 KiB per step) and one exponent byte (64 per step).  b: 32-block index.
__host__ __device__ __forceinline__ uint32_t mx_quad_lane(uint32_t n, uint32_t b) {
  const uint32_t w = b & 15u;  // 32-block within the step: part w / 4, sub-block w % 4
  return (w & 3u) * 16u + (w >> 2) * 4u + (n & 3u);
}
__host__ __device__ __forceinline__ size_t mx_quad_code_off(uint32_t n, uint32_t b, uint32_t K) {
  return (((size_t)(n >> 2) * (K >> 9) + (b >> 4)) * 64 + mx_quad_lane(n, b)) * 16;
}
__host__ __device__ __forceinline__ size_t mx_quad_scale_off(uint32_t n, uint32_t b, uint32_t K) {
  return ((size_t)(n >> 2) * (K >> 9) + (b >> 4)) * 64 + mx_quad_lane(n, b);
}

// floor(log2(amax)) from the exponent field (frexp: amax = f * 2^x, f in
// [0.5, 1)); amax below 2^-126 (zero, subnormal) gives e = 0 either way.
__device__ __forceinline__ int mx_block_exp(float amax) {
  if (!(amax >= 0x1p-126f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 2 + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

// maximum over each aligned group of 4 lanes, and of 16 lanes
__device__ __forceinline__ float quad_max(float v) {
  v = __builtin_fmaxf(v, dpp_f32<DPP_QUAD_X1>(v));
  return __builtin_fmaxf(v, dpp_f32<DPP_QUAD_X2>(v));
}
__device__ __forceinline__ float row16_max(float v) {
  v = quad_max(v);
  v = __builtin_fmaxf(v, dpp_f32<DPP_ROW_HALF_MIRROR>(v));
  return __builtin_fmaxf(v, dpp_f32<DPP_ROW_MIRROR>(v));
}

// E2M1 codes of two values already divided by the block scale, packed into
// byte SEL of w (x0 low nibble, x1 high): gfx950's v_cvt_scalef32_pk_fp4_f32
// with unit scale.  It rounds to nearest with ties to the even mantissa,
// saturates at 6 and keeps the sign (including -0); NaN takes the largest
// magnitude -- the encoding the format defines, checked value by value over
// [-10, 10] in steps of 2^-8, each midpoint and its neighbouring floats,
// zeros, subnormals, infinities and NaN.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t w, float x0, float x1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x0, x1, 1.0f, SEL);
}

// eight values of one 32-block (scale exponent e) -> one dword of codes
__device__ __forceinline__ uint32_t mx_pack8(const float x[8], int e) {
  const int s = 127 - e;
  uint32_t w = 0;
  w = e2m1_pack2<0>(w, ldexpf(x[0], s), ldexpf(x[1], s));
  w = e2m1_pack2<1>(w, ldexpf(x[2], s), ldexpf(x[3], s));
  w = e2m1_pack2<2>(w, ldexpf(x[4], s), ldexpf(x[5], s));
  w = e2m1_pack2<3>(w, ldexpf(x[6], s), ldexpf(x[7], s));
  return w;
}

// Gated combine of the MXFP4 FFN (act(g) * u, or gelu_tanh(u) without gate).
enum { MX_GEGLU = 0, MX_SWIGLU = 1, MX_GELU = 2 };
template <int ACT>
__device__ __forceinline__ float mx_gated(float g, float u) {
  if (ACT == MX_GELU) return gelu_tanh_f32(u);
  const float a = (ACT == MX_SWIGLU) ? silu_f32(g) : gelu_tanh_f32(g);
  return a * u;
}

// One 32-column block of h for one row, held by the 16 lanes of a lane row
// group (lane row `row` = column row and 16 + row): block exponent from the
// 16-lane maximum, E2M1 codes, two per byte written by the even lane, the
// exponent by lane row 0.  Every lane of the wave must call it (lane moves);
// `store` says whether this row exists.  codes points at the block's 16
// bytes of the row, scale at its exponent byte.
// The two halves: mx_h32_codes returns the block exponent in bits 16..23
// and the lane pair's two code bytes in bits 0..15 (valid in the even lane);
// mx_h32_store writes them.  Callers with many blocks form every block's
// codes first and store afterwards, so the lane moves and transcendentals of
// independent blocks share one basic block (the stores' row guards would
// otherwise split it and leave each lane move waiting on its own hazard).
// 16-lane maximum of non-negative values through their bit patterns (for
// finite values >= 0 the integer order is the float order), so no float
// maximum needs its inputs canonicalised
__device__ __forceinline__ uint32_t row16_max_u(uint32_t v) {
  v = max(v, dpp_u32<DPP_QUAD_X1>(v));
  v = max(v, dpp_u32<DPP_QUAD_X2>(v));
  v = max(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
  return max(v, dpp_u32<DPP_ROW_MIRROR>(v));
}
__device__ __forceinline__ uint32_t mx_h32_pack(float h0, float h1, float am) {
  const int e = mx_block_exp(am);
  const float x0 = ldexpf(h0, 127 - e), x1 = ldexpf(h1, 127 - e);
  // the odd lane's values reach its even neighbour, which packs the byte
  const uint32_t b = e2m1_pack2<1>(e2m1_pack2<0>(0u, x0, dpp_f32<DPP_QUAD_X1>(x0)), x1, dpp_f32<DPP_QUAD_X1>(x1));
  return (b & 0xffffu) | ((uint32_t)e << 16);
}
__device__ __forceinline__ uint32_t mx_h32_codes(float h0, float h1) {
  const uint32_t am = row16_max_u(__float_as_uint(__builtin_fmaxf(__builtin_fabsf(h0), __builtin_fabsf(h1))));
  return mx_h32_pack(h0, h1, __uint_as_float(am));
}
// two blocks at once, their lane-move chains interleaved (each lane move
// waits on the previous step of its own chain only)
__device__ __forceinline__ void mx_h32_codes2(float a0, float a1, float b0, float b1, uint32_t& ra, uint32_t& rb) {
  uint32_t va = __float_as_uint(__builtin_fmaxf(__builtin_fabsf(a0), __builtin_fabsf(a1)));
  uint32_t vb = __float_as_uint(__builtin_fmaxf(__builtin_fabsf(b0), __builtin_fabsf(b1)));
  va = max(va, dpp_u32<DPP_QUAD_X1>(va));
  vb = max(vb, dpp_u32<DPP_QUAD_X1>(vb));
  va = max(va, dpp_u32<DPP_QUAD_X2>(va));
  vb = max(vb, dpp_u32<DPP_QUAD_X2>(vb));
  va = max(va, dpp_u32<DPP_ROW_HALF_MIRROR>(va));
  vb = max(vb, dpp_u32<DPP_ROW_HALF_MIRROR>(vb));
  va = max(va, dpp_u32<DPP_ROW_MIRROR>(va));
  vb = max(vb, dpp_u32<DPP_ROW_MIRROR>(vb));
  ra = mx_h32_pack(a0, a1, __uint_as_float(va));
  rb = mx_h32_pack(b0, b1, __uint_as_float(vb));
}
__device__ __forceinline__ void mx_h32_store(uint32_t be, bool store, int row, uint8_t* codes, uint8_t* scale) {
  if (store && (row & 1) == 0) {
    codes[row >> 1] = (uint8_t)be;
    codes[8 + (row >> 1)] = (uint8_t)(be >> 8);
    if (row == 0) *scale = (uint8_t)(be >> 16);
  }
}
__device__ __forceinline__ void mx_store_h32(float h0, float h1, bool store, int row, uint8_t* codes,
                                             uint8_t* scale) {
  mx_h32_store(mx_h32_codes(h0, h1), store, row, codes, scale);
}

__device__ __forceinline__ v4f mx_mfma(v8i a, int sa, v8i b, int sb, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

// GEMV-layout activation exponents (M <= 64, rows padded to 16): per (16-row
// tile, four 128-K blocks) 64 lanes x 4 bytes; lane = 32-sub-block * 16 +
// row % 16 (the MFMA operand's lane), byte = K block % 4 -- the weights'
// layout with the row tile in place of the group, so one dword per lane
// carries four K blocks of either operand.  Row m, 32-block b.
__host__ __device__ __forceinline__ size_t mx_act_scale_off_gemv(uint32_t m, uint32_t b, uint32_t KB) {
  return (((size_t)(m >> 4) * (KB >> 2) + (b >> 4)) * 64 + ((b & 3u) * 16u + (m & 15u))) * 4 + ((b >> 2) & 3u);
}

// Block-scaled FP4 product whose exponents are byte U of each operand's
// exponent dword (op_sel)
template <int U>
__device__ __forceinline__ v4f mx_mfma_u(v8i a, int sa, v8i b, int sb, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, U, sa, U, sb);
}

// Prefill-layout exponents (k_mxmm), arranged so that one 32-bit LDS read
// gives a lane the exponents of four MFMA operands and the instruction picks
// the byte (op_sel).  Weights: per (quad of 16-row groups, 128-K block) 64
// lanes x 4 bytes, byte j = group 4 * quad + j.
__host__ __device__ __forceinline__ size_t mx_scale_off_mm(uint32_t prow, uint32_t kb, uint32_t lane, uint32_t KB) {
  return ((size_t)(prow >> 6) * KB + kb) * 256 + lane * 4 + ((prow >> 4) & 3u);
}
// Activations (rows padded to a multiple of 128): per (64-row group, 128-K
// block) 64 lanes x 4 bytes; lane = 32-sub-block * 16 + row % 16 (the
// operand's lane), byte i = 16-row block i of the group.  Row m, 32-block b.
__host__ __device__ __forceinline__ size_t mx_act_scale_off_mm(uint32_t m, uint32_t b, uint32_t KB) {
  return ((size_t)(m >> 6) * KB + (b >> 2)) * 256 + (((b & 3u) * 16u + (m & 15u)) * 4u) + ((m >> 4) & 3u);
}

}  // namespace frt
