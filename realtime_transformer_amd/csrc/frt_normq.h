// frt_normq.h -- the second half of the split decode norm, shared by the
// GEMVs that quantise their own activations (k_gemv_gateup_nq, k_gemv_qkv_nq).
//
// itsolotime article, section 7.2 (RMSNorm of the high-precision residual
// feeding the FP8 GEMMs); FlashRT architecture doc, component "Kernel
// library" (residual + norm + quant fusions).
//
// After k_add_sumsq has stored r' = bf16(R + Y) and fp64 sums of r'^2 over
// 512-element slices of each row, a GEMV wave that multiplies K blocks
// [kb0, kb1) forms exactly those activations itself:
//   inv_m = f32(1 / sqrt(S_m / K + eps))  (fp64; S_m = slice sums in order)
//   XQ[m][k] = e4m3(f32(f32(f32(r'[m][k] * inv_m) * w_norm[k]) * inv_x))
// (the arithmetic of the one-kernel k_add_rmsnorm_quant) into a wave-private
// part of an LDS row buffer [M][K].  Loads come first (no load behind a
// branch: indices are clamped), so the caller can issue its first weight
// loads between load() and quant() and the compiler's wait before the
// quantisation counts only these.
#pragma once

#include "frt_device.h"

namespace frt {

struct NormQ {
  const uint16_t* r;       // r' = R[l+1], bf16 [M][K]
  const uint16_t* w_norm;  // RMSNorm weight, bf16 [K]
  const double* sq;        // slice sums of r'^2, fp64 [M][G]
  int G;
  float eps, inv_x;
  uint8_t* xq_out;         // XQ, E4M3 [M][K] (the caller's workgroup 0 stores it)
};
constexpr int kNqLdsBytes = 16384;  // row buffer M * K
constexpr int kNqMaxSlices = 16;    // slice sums per row (H <= 8192)

// Whether a GEMV can take the split norm at this shape: the row buffer fits
// its LDS budget and every slice sum has a lane (M * G <= 64).
__host__ __device__ inline bool normq_shape_ok(int M, int K, int G) {
  return M >= 1 && M <= 16 && K % 128 == 0 && (long)M * K <= kNqLdsBytes && G >= 1 && G <= kNqMaxSlices &&
         M * G <= 64;
}

// NCH: 8-element chunks per lane whose loads are issued together.
template <int NCH>
struct NormQWave {
  int M, K, kc0, nkc, nch;
  float rcp_nkc;
  double part_v;
  int cm[NCH], ck[NCH];
  uint4 rv[NCH], wv[NCH];

  // K blocks [kb0, kb1) of rows [0, M), kb1 > kb0
  __device__ __forceinline__ void init(const NormQ& nq, int M_, int K_, int kb0, int kb1, int lane) {
    M = M_;
    K = K_;
    kc0 = kb0 * 16;
    nkc = (kb1 - kb0) * 16;
    nch = M * nkc;
    rcp_nkc = __builtin_amdgcn_rcpf((float)nkc);
    part_v = nq.sq[lane < M * nq.G ? lane : M * nq.G - 1];
  }
  // chunk c of the range is (row c / nkc, K chunk kc0 + c % nkc)
  __device__ __forceinline__ void load(const NormQ& nq, int c0, int lane) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      int c = c0 + j * 64 + lane;
      c = c < nch ? c : nch - 1;  // lanes past the end redo the last chunk (same bytes)
      int m = (int)(((float)c + 0.5f) * rcp_nkc);
      m -= (m * nkc > c) ? 1 : 0;
      m += ((m + 1) * nkc <= c) ? 1 : 0;
      cm[j] = m;
      ck[j] = (kc0 + (c - m * nkc)) * 8;
      rv[j] = *reinterpret_cast<const uint4*>(nq.r + (size_t)m * K + ck[j]);
      wv[j] = *reinterpret_cast<const uint4*>(nq.w_norm + ck[j]);
    }
  }
  // 1/rms of row `lane` (lanes < M; the others compute row 0's)
  __device__ __forceinline__ float inv_rms(const NormQ& nq, int lane) const {
    const int G = nq.G;
    const double part = lane < M * G ? part_v : 0.0;
    const int base = lane < M ? lane * G : 0;
    const unsigned long long b = (unsigned long long)__double_as_longlong(part);
    double ssum = 0.0;
#pragma unroll
    for (int g = 0; g < kNqMaxSlices; ++g) {
      const int src = base + (g < G ? g : 0);
      const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)b, src, 64);
      const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(b >> 32), src, 64);
      const double v = __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
      ssum += g < G ? v : 0.0;
    }
    return (float)(1.0 / sqrt(ssum / (double)K + (double)nq.eps));
  }
  // codes of the loaded chunks into the row buffer (and XQ when store)
  __device__ __forceinline__ void quant(const NormQ& nq, int c0, int lane, float inv_rms_lane, uint8_t* xrow,
                                        bool store) const {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const float inv = __shfl(inv_rms_lane, cm[j], 64);
      const uint32_t rr[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
      const uint32_t ww[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
      float x[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        x[2 * t] = (bf16_lo(rr[t]) * inv) * bf16_lo(ww[t]);
        x[2 * t + 1] = (bf16_hi(rr[t]) * inv) * bf16_hi(ww[t]);
      }
      const float ix = nq.inv_x;
      uint2 code;
      code.x = e4m3x4(x[0] * ix, x[1] * ix, x[2] * ix, x[3] * ix);
      code.y = e4m3x4(x[4] * ix, x[5] * ix, x[6] * ix, x[7] * ix);
      if (c0 + j * 64 + lane < nch) {
        const size_t o = (size_t)cm[j] * K + ck[j];
        *reinterpret_cast<uint2*>(xrow + o) = code;
        if (store) *reinterpret_cast<uint2*>(nq.xq_out + o) = code;
      }
    }
  }
};

// LDS written by one lane of a wave and read by another lane of the same
// wave: the LDS serves a wave's operations in order; the fences keep the
// compiler from moving the accesses across.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace frt
