// frt_device.h -- device-side helpers shared by the gfx950 kernels of libfrt.
//
// Number formats (FlashRT pages: itsolotime article, section 7.1, FP8 E4M3;
// section 7.2, high-precision residual stream):
//   bf16  : uint16 bit pattern, widened exactly to fp32, narrowed by
//           round-to-nearest-even (inputs are never NaN on this path).
//   E4M3  : OCP E4M3FN byte.  The quantiser clamps to +-448 first and then
//           uses the hardware converter, which rounds to nearest even; on
//           gfx950 the converter alone turns |v| > 464 into NaN, so the clamp
//           is what makes it saturate.
//
// Packed weight layout (written by the weight quantiser, read by the GEMV,
// GEMM and calibration kernels).  A weight matrix W[N][K] (nn.Linear
// [out, in]) is cut into blocks of 16 rows x 128 columns; block (g, kb) is
// 2048 contiguous bytes at ((g * K/128) + kb) * 2048.  Inside a block, lane
// l (0..63) of a wave owns row g*16 + l%16 and columns kb*128 + (l/16)*32 +
// [0, 32); its 32 bytes sit as two 16-byte halves at offsets l*16 (columns
// +0..15) and 1024 + l*16 (columns +16..31).  This is the operand fragment
// of a 16-row MFMA tile, so one 16-byte load per lane reads 1 KiB
// contiguously.  For the gated activations the packed matrix is [2I][K] with
// 16-row groups alternating gate (even group) and up (odd group):
// packed row 32*(i/16) + i%16 is gate row i, 32*(i/16) + 16 + i%16 is up
// row i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace frt {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float clamp_e4m3(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -kE4M3Max), kE4M3Max);
}

// four fp32 -> four E4M3 bytes (byte i = value i), saturating, RNE
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), p, true);
  return (uint32_t)p;
}
__device__ __forceinline__ uint32_t e4m3x1(float a) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), 0.0f, 0, false) & 0xffu;
}

// E4M3 bytes -> fp32 (exact)
template <bool HI>
__device__ __forceinline__ v2f e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)byte, false)[0];
}

// E4M3 bytes -> f16 (exact: every E4M3 value is an f16 value)
template <bool HI>
__device__ __forceinline__ v2h e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI);
}
// 8 E4M3 bytes (two dwords) -> 8 f16
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
  v2h a = e4m3x2_to_f16<false>(w0), b = e4m3x2_to_f16<true>(w0);
  v2h c = e4m3x2_to_f16<false>(w1), d = e4m3x2_to_f16<true>(w1);
  v8h r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Byte offset of element (n, k) of a packed [N][K] weight (K % 128 == 0).
__host__ __device__ __forceinline__ size_t packed_offset(uint32_t n, uint32_t k, uint32_t K) {
  uint32_t g = n >> 4, kb = k >> 7, lane = (n & 15u) + 16u * ((k & 127u) >> 5);
  uint32_t half = (k & 31u) >> 4;
  return ((size_t)g * (K >> 7) + kb) * 2048u + half * 1024u + lane * 16u + (k & 15u);
}

// Byte offset of element (n, k) of a [N][K] down matrix in the column-quad
// layout of the whole-column decode down GEMV (K % 256 == 0, N % 4 == 0):
// quad n / 4 owns K / 256 blocks of 1 KiB, block t covering elements
// 256 t .. 256 t + 255 of its four columns as four 64-element parts; lane
// l's 16 bytes are column 4 (n / 4) + (l & 3), elements 256 t + 64 p +
// (l >> 4) * 16 .. + 15 with part p = (l & 15) >> 2.
__host__ __device__ __forceinline__ size_t quad_offset(uint32_t n, uint32_t k, uint32_t K) {
  const uint32_t w = k & 255u, p = w >> 6;
  const uint32_t lane = ((w & 63u) >> 4) * 16u + p * 4u + (n & 3u);
  return (((size_t)(n >> 2) * (K >> 8) + (k >> 8)) * 64u + lane) * 16u + (k & 15u);
}

// Packed row of gate row i / up row i in the gated [2I][K] matrix.
__host__ __device__ __forceinline__ uint32_t gate_row(uint32_t i) { return 32u * (i >> 4) + (i & 15u); }
__host__ __device__ __forceinline__ uint32_t up_row_gated(uint32_t i) {
  return 32u * (i >> 4) + 16u + (i & 15u);
}
// ... in the octet order of the decode gate/up GEMV's eight-column
// workgroups: one 16-row group holds gate rows 8j .. 8j+7, then up rows
// 8j .. 8j+7, so a workgroup streams one group for both matrices.
__host__ __device__ __forceinline__ uint32_t gate_row_oct(uint32_t i) { return 16u * (i >> 3) + (i & 7u); }
__host__ __device__ __forceinline__ uint32_t up_row_oct(uint32_t i) { return 16u * (i >> 3) + 8u + (i & 7u); }

// Activations in fp32, written from their definitions:
//   tanh-GELU(z) = 0.5 z (1 + tanh(c (z + 0.044715 z^3))), c = sqrt(2/pi),
//                = z * sigmoid(2 c (z + 0.044715 z^3))
//   SiLU(z)      = z * sigmoid(z)
// sigmoid(t) = 1 / (1 + exp(-t)), with exp(-t) = 2^(-t * log2 e) on the
// hardware exp2 (v_exp_f32) and the hardware reciprocal (v_rcp_f32): two
// transcendental instructions instead of the library expf and an IEEE
// division (some twenty instructions per element in the GEMM epilogues).
// Relative error: the product -t * log2 e is rounded once (2^-24 |t| log2 e
// relative in exp), plus about one ulp from each instruction; for |t| < 16
// that is under 1e-6, which moves a re-quantised E4M3 code only when the
// value sits that close to a rounding boundary.  Limits: for t < -88 exp2
// overflows to +inf and the reciprocal is 0; for t > 88 exp2 underflows to 0
// and the result is 1; where the reciprocal would be an fp32 denormal it may
// flush to 0, which every consumer quantises to E4M3 zero anyway.
__device__ __forceinline__ float sigmoid_f32(float t) {
  const float e = __builtin_amdgcn_exp2f(t * -1.4426950408889634f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float gelu_tanh_f32(float z) {
  const float c2 = 1.5957691216057308f;  // 2 * sqrt(2/pi)
  float inner = z * (1.0f + 0.044715f * z * z);
  return z * sigmoid_f32(c2 * inner);
}
__device__ __forceinline__ float silu_f32(float z) { return z * sigmoid_f32(z); }

// y of 8 consecutive elements from S fp32 partial tiles (split order).  The
// first four splits' loads are issued together before the adds.
__device__ __forceinline__ uint4 y_from_partials(const float* __restrict__ part, size_t split_stride,
                                                 size_t off, int S, float alpha_d) {
  float4 lo[4], hi[4];
#pragma unroll
  for (int sp = 0; sp < 4; ++sp) {
    if (sp < S) {
      lo[sp] = *reinterpret_cast<const float4*>(part + sp * split_stride + off);
      hi[sp] = *reinterpret_cast<const float4*>(part + sp * split_stride + off + 4);
    }
  }
  float a[8] = {lo[0].x, lo[0].y, lo[0].z, lo[0].w, hi[0].x, hi[0].y, hi[0].z, hi[0].w};
#pragma unroll
  for (int sp = 1; sp < 4; ++sp) {
    if (sp < S) {
      a[0] += lo[sp].x; a[1] += lo[sp].y; a[2] += lo[sp].z; a[3] += lo[sp].w;
      a[4] += hi[sp].x; a[5] += hi[sp].y; a[6] += hi[sp].z; a[7] += hi[sp].w;
    }
  }
  for (int sp = 4; sp < S; ++sp) {
    const float4 p0 = *reinterpret_cast<const float4*>(part + sp * split_stride + off);
    const float4 p1 = *reinterpret_cast<const float4*>(part + sp * split_stride + off + 4);
    a[0] += p0.x; a[1] += p0.y; a[2] += p0.z; a[3] += p0.w;
    a[4] += p1.x; a[5] += p1.y; a[6] += p1.z; a[7] += p1.w;
  }
  return make_uint4(pack_bf16x2(a[0] * alpha_d, a[1] * alpha_d), pack_bf16x2(a[2] * alpha_d, a[3] * alpha_d),
                    pack_bf16x2(a[4] * alpha_d, a[5] * alpha_d), pack_bf16x2(a[6] * alpha_d, a[7] * alpha_d));
}

// Lane moves inside a 16-lane row (DPP, no LDS round trip): quad_perm
// [1,0,3,2] and [2,3,0,1] exchange lane pairs and pairs of pairs,
// row_half_mirror reverses each 8 lanes, row_mirror the 16.
enum { DPP_QUAD_X1 = 0xB1, DPP_QUAD_X2 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140 };
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
// maximum over each aligned group of 4 lanes, and of 16 lanes

// wave64 reductions.  The fp64 sum adds within 16-lane rows by DPP lane
// moves and then the four row sums read from lanes 0, 16, 32, 48 (scalar
// reads), so no step is an LDS round trip; every lane returns the total.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<DPP_QUAD_X1>(v);
  v += dpp_f64<DPP_QUAD_X2>(v);
  v += dpp_f64<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f64<DPP_ROW_MIRROR>(v);
  return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// max of non-negative floats through their bit patterns (monotone for >= 0)
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

}  // namespace frt
