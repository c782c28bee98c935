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

__device__ __forceinline__ int mx_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = ilogbf(amax) - 2 + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

// E2M1 code of v (already divided by the block scale): the magnitude code is
// the number of decision points passed -- the midpoints 0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5 between neighbouring magnitudes, each a strict or
// non-strict comparison so that a value on a midpoint goes to the neighbour
// with mantissa bit 0 (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
// 3.5 -> 4, 5 -> 4); NaN takes the largest magnitude.  No branches.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
               (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  c = (a == a) ? c : 7u;
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// eight values of one 32-block (scale exponent e) -> one dword of codes
__device__ __forceinline__ uint32_t mx_pack8(const float x[8], int e) {
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= e2m1_code(ldexpf(x[j], 127 - e)) << (4 * j);
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
// exponent by lane row 0.  Every lane of the wave must call it (shuffles);
// `store` says whether this row exists.  codes points at the block's 16
// bytes of the row, scale at its exponent byte.
__device__ __forceinline__ void mx_store_h32(float h0, float h1, bool store, int row, uint8_t* codes,
                                             uint8_t* scale) {
  float am = __builtin_fmaxf(__builtin_fabsf(h0), __builtin_fabsf(h1));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) am = __builtin_fmaxf(am, __shfl_xor(am, o, 64));
  const int e = mx_block_exp(am);
  const uint32_t c0 = e2m1_code(ldexpf(h0, 127 - e)), c1 = e2m1_code(ldexpf(h1, 127 - e));
  const uint32_t p0 = (uint32_t)__shfl_xor((int)c0, 1, 64), p1 = (uint32_t)__shfl_xor((int)c1, 1, 64);
  if (store && (row & 1) == 0) {
    codes[row >> 1] = (uint8_t)(c0 | (p0 << 4));
    codes[8 + (row >> 1)] = (uint8_t)(c1 | (p1 << 4));
    if (row == 0) *scale = (uint8_t)e;
  }
}

__device__ __forceinline__ v4f mx_mfma(v8i a, int sa, v8i b, int sb, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

// Prefill-layout weight exponents (k_mxmm): one byte per lane per (16-row
// group, 128-K block): ((g * KB + kb) * 64 + lane).
__host__ __device__ __forceinline__ size_t mx_scale_off_mm(uint32_t prow, uint32_t kb, uint32_t lane, uint32_t KB) {
  return ((size_t)(prow >> 4) * KB + kb) * 64 + lane;
}

}  // namespace frt
