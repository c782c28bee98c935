// k_gemm.hip -- the two FP8 GEMMs of the FFN block with fused epilogues.
//
// itsolotime article, section 7.2 (the encoder FFN loop): gate and up
// projections, a fused kernel for the GEGLU/SiLU-style gating that
// re-quantises its output, then the down projection back to the residual
// path; FlashRT architecture doc, component "Calibration": dequantisation by
// alpha = act_scale * weight_scale baked as host scalars.
//
//   gate/up : HQ[m][i] = e4m3(h * inv_h),  h = act(Ag*a_g) * (Au*a_u)
//             (non-gated: h = gelu_tanh(Au*a_u)),  A* = XQ[m] . W*[i]
//   down    : Y[m][n]  = bf16(Ad * a_d),   Ad = HQ[m] . Wd[n]
//
// Arithmetic.  The dot products run on the f16 matrix cores: every E4M3
// value converts exactly to f16 and those MFMAs accumulate at fp32 accuracy,
// which is what the fp32-accumulated GEMM of the method asks for.  The gfx950
// FP8 matrix instructions align the products of one instruction to the
// largest and drop bits below about 2^-13 of it (relative errors of
// 1e-5..1e-3 on FFN data, measured); fed into the re-quantiser that flips a
// few 1e-4 of the HQ codes, and through a deep chain it multiplies the drift
// between two correct implementations by ~20.  The down projection can opt
// into the full-rate FP8 matrix cores (plan flag), whose bf16 block output
// still meets the per-block tolerance.
//
// Two shapes:
//   GEMV (M <= 16): one workgroup per 16 output columns, its waves split K;
//     weights stream from HBM through registers in the packed fragment
//     layout, the activation rows come from L2; partials meet in LDS.
//   GEMM (M > 16): 128x128 output tile per workgroup, K step 128, operand
//     tiles staged through LDS in fragment order (double buffered), 2x2 waves
//     of 64x64.  The down GEMM may split K across workgroups with the same
//     last-arrival fixed-order reduction.
#include "frt_device.h"

namespace frt {

enum { GU_GEGLU = 0, GU_SWIGLU = 1, GU_GELU = 2 };

template <int ACT>
__device__ __forceinline__ float gated_h(float g, float u) {
  if (ACT == GU_GELU) return gelu_tanh_f32(u);
  float a = (ACT == GU_SWIGLU) ? silu_f32(g) : gelu_tanh_f32(g);
  return a * u;
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ v4f mfma_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v8i as_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}
// 16x16x128 step as four f16 16x16x32 MFMAs over the lane's 32 bytes
__device__ __forceinline__ v4f mfma_f16_x4(const uint32_t a[8], const uint32_t b[8], v4f c) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
    c = mfma_f16(e4m3x8_to_f16(a[2 * t], a[2 * t + 1]), e4m3x8_to_f16(b[2 * t], b[2 * t + 1]), c);
  return c;
}
__device__ __forceinline__ void unpack8(uint4 lo, uint4 hi, uint32_t o[8]) {
  o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
  o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
}
// one 16 x 16 x 128 step: FP8 matrix cores, or four f16 steps (fp32-accurate)
template <bool FP8>
__device__ __forceinline__ v4f mfma_step(const uint32_t a[8], const uint32_t b[8], v4f c) {
  if (FP8) {
    v8i av, bv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      av[i] = (int)a[i];
      bv[i] = (int)b[i];
    }
    return mfma_fp8(av, bv, c);
  }
  return mfma_f16_x4(a, b, c);
}

// ===========================================================================
// GEMV path (M <= 16)
// ===========================================================================
//
// One workgroup of W waves owns 16 output columns (for the gated forms: 16
// intermediate columns, i.e. the gate group and the up group of the packed
// matrix).  Wave w streams K blocks [w*KB/W, (w+1)*KB/W) of those rows with
// nontemporal 16-byte loads, two K blocks in flight per step; the W partial
// accumulators meet in LDS and wave 0 adds them in wave order (fixed order:
// the result does not depend on timing) and runs the epilogue.  Keeping the
// split inside the workgroup needs no cross-workgroup handshake, so no
// device-scope fence (which on this multi-XCD part writes back the L2).

typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const uint8_t* p) {
  v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// activation fragment of K block kb: lane's 32 bytes of row (lane & 15) or zeros
__device__ __forceinline__ void load_x32(const uint8_t* xr, bool has_row, int kb, uint32_t o[8]) {
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (has_row) {
    a = ld16(xr + kb * 128);
    b = ld16(xr + kb * 128 + 16);
  }
  unpack8(a, b, o);
}
__device__ __forceinline__ void load_w32(const uint8_t* wp, int kb, uint32_t o[8]) {
  unpack8(ld16_nt(wp + (size_t)kb * 2048), ld16_nt(wp + (size_t)kb * 2048 + 1024), o);
}

template <int ACT, int W>
__global__ __launch_bounds__(W * 64) void k_gemv_gateup(const uint8_t* __restrict__ xq,
                                                        const uint8_t* __restrict__ w,
                                                        uint8_t* __restrict__ hq, int M, int K,
                                                        int I, float alpha_g, float alpha_u,
                                                        float inv_h) {
  constexpr bool GATED = ACT != GU_GELU;
  constexpr int NACC = GATED ? 2 : 1;
  __shared__ v4f red[W][NACC][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = blockIdx.x;  // column group
  const int KB = K >> 7;
  const int kb0 = wave * KB / W, kb1 = (wave + 1) * KB / W;
  const int row = lane & 15, q = lane >> 4;
  const bool has_row = row < M;
  const uint8_t* wg = w + (size_t)(GATED ? 2 * p : 0) * KB * 2048 + lane * 16;
  const uint8_t* wu = w + (size_t)(GATED ? 2 * p + 1 : p) * KB * 2048 + lane * 16;
  const uint8_t* xr = xq + (size_t)(has_row ? row : 0) * K + q * 32;

  v4f accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
  int kb = kb0;
  for (; kb + 1 < kb1; kb += 2) {
    uint32_t x0[8], x1[8], u0[8], u1[8], g0[8], g1[8];
    load_w32(wu, kb, u0);
    load_w32(wu, kb + 1, u1);
    if (GATED) {
      load_w32(wg, kb, g0);
      load_w32(wg, kb + 1, g1);
    }
    load_x32(xr, has_row, kb, x0);
    load_x32(xr, has_row, kb + 1, x1);
    accu = mfma_f16_x4(x0, u0, accu);
    if (GATED) accg = mfma_f16_x4(x0, g0, accg);
    accu = mfma_f16_x4(x1, u1, accu);
    if (GATED) accg = mfma_f16_x4(x1, g1, accg);
  }
  if (kb < kb1) {
    uint32_t x0[8], u0[8], g0[8];
    load_w32(wu, kb, u0);
    if (GATED) load_w32(wg, kb, g0);
    load_x32(xr, has_row, kb, x0);
    accu = mfma_f16_x4(x0, u0, accu);
    if (GATED) accg = mfma_f16_x4(x0, g0, accg);
  }
  if (W > 1) {
    red[wave][0][lane] = accu;
    if (GATED) red[wave][NACC - 1][lane] = accg;
    __syncthreads();
    if (wave != 0) return;
    accu = red[0][0][lane];
    if (GATED) accg = red[0][NACC - 1][lane];
#pragma unroll
    for (int v = 1; v < W; ++v) {
      accu += red[v][0][lane];
      if (GATED) accg += red[v][NACC - 1][lane];
    }
  }
  // lane holds rows m = 4q + r of column 16p + row
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * q + r;
    if (m < M) {
      const float h = gated_h<ACT>(accg[r] * alpha_g, accu[r] * alpha_u);
      hq[(size_t)m * I + p * 16 + row] = (uint8_t)e4m3x1(h * inv_h);
    }
  }
}

template <int W, bool FP8>
__global__ __launch_bounds__(W * 64) void k_gemv_down(const uint8_t* __restrict__ hq,
                                                      const uint8_t* __restrict__ w,
                                                      uint16_t* __restrict__ y, int M, int K, int N,
                                                      float alpha_d) {
  __shared__ v4f red[W][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = blockIdx.x;
  const int KB = K >> 7;
  const int kb0 = wave * KB / W, kb1 = (wave + 1) * KB / W;
  const int row = lane & 15, q = lane >> 4;
  const bool has_row = row < M;
  const uint8_t* wp = w + (size_t)p * KB * 2048 + lane * 16;
  const uint8_t* xr = hq + (size_t)(has_row ? row : 0) * K + q * 32;

  v4f acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  int kb = kb0;
  for (; kb + 1 < kb1; kb += 2) {
    uint32_t x0[8], x1[8], w0[8], w1[8];
    load_w32(wp, kb, w0);
    load_w32(wp, kb + 1, w1);
    load_x32(xr, has_row, kb, x0);
    load_x32(xr, has_row, kb + 1, x1);
    acc0 = mfma_step<FP8>(x0, w0, acc0);
    acc1 = mfma_step<FP8>(x1, w1, acc1);
  }
  if (kb < kb1) {
    uint32_t x0[8], w0[8];
    load_w32(wp, kb, w0);
    load_x32(xr, has_row, kb, x0);
    acc0 = mfma_step<FP8>(x0, w0, acc0);
  }
  v4f acc = acc0 + acc1;
  if (W > 1) {
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    acc = red[0][lane];
#pragma unroll
    for (int v = 1; v < W; ++v) acc += red[v][lane];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * q + r;
    if (m < M) y[(size_t)m * N + p * 16 + row] = (uint16_t)f32_to_bf16(acc[r] * alpha_d);
  }
}

// ===========================================================================
// GEMM path (M > 16)
// ===========================================================================

constexpr int BM = 128, BN = 128, BKB = 128;  // tile rows, packed tile columns, K step (bytes)
constexpr int TILE_BYTES = 8 * 2048;            // 8 fragment blocks of 16 x 128

// Stage one K step: A (activations, row-major [M][K]) into fragment order,
// B (packed weights) verbatim.  Thread t moves 4 + 4 16-byte pieces.
struct StageRegs {
  uint4 a[4], b[4];
};

__device__ __forceinline__ void stage_load(StageRegs& st, const uint8_t* __restrict__ act, int M,
                                           int K, int m0, const uint8_t* __restrict__ wt,
                                           int g0, int KB, int kb) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;  // 0..1023
    const int r = c >> 3, kc = c & 7;
    const int m = m0 + r;
    st.a[j] = make_uint4(0, 0, 0, 0);
    if (m < M) st.a[j] = ld16(act + (size_t)m * K + kb * 128 + kc * 16);
    const int grp = c >> 7, off = (c & 127) * 16;
    st.b[j] = ld16(wt + ((size_t)(g0 + grp) * KB + kb) * 2048 + off);
  }
}
__device__ __forceinline__ void stage_store(const StageRegs& st, uint8_t* lds_a, uint8_t* lds_b) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    const int r = c >> 3, kc = c & 7;
    const int mg = r >> 4, ln = (r & 15) + 16 * (kc >> 1), half = kc & 1;
    *reinterpret_cast<uint4*>(lds_a + mg * 2048 + half * 1024 + ln * 16) = st.a[j];
    *reinterpret_cast<uint4*>(lds_b + c * 16) = st.b[j];
  }
}

// MODE: GU_GEGLU / GU_SWIGLU / GU_GELU for gate/up, 3 for down (f16 matrix
// cores), 4 for down on the FP8 matrix cores.
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ act,
                                              const uint8_t* __restrict__ wt,
                                              void* __restrict__ out, float* __restrict__ part,
                                              uint32_t* __restrict__ cnt, int M, int K,
                                              int Npk, int S, float alpha_a, float alpha_b,
                                              float inv_out) {
  constexpr bool DOWN = MODE >= 3;
  constexpr bool FP8 = MODE == 4;
  constexpr bool GATED = MODE == GU_GEGLU || MODE == GU_SWIGLU;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][TILE_BYTES];  // [buf][A/B]
  int* s_last = reinterpret_cast<int*>(&lds[0][0][0]);  // reused after the main loop

  const int tn = blockIdx.x, tm = blockIdx.y, s = blockIdx.z;
  const int m0 = tm * BM, g0 = tn * (BN / 16);
  const int KB = K >> 7;
  const int kb0 = s * KB / S, kb1 = (s + 1) * KB / S;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0, 0, 0, 0};

  StageRegs st;
  stage_load(st, act, M, K, m0, wt, g0, KB, kb0);
  stage_store(st, lds[0][0], lds[0][1]);
  __syncthreads();
  int cur = 0;
  for (int kb = kb0; kb < kb1; ++kb) {
    const bool more = kb + 1 < kb1;
    if (more) stage_load(st, act, M, K, m0, wt, g0, KB, kb + 1);
    const uint8_t* la = lds[cur][0] + (wm * 4) * 2048 + lane * 16;
    const uint8_t* lb = lds[cur][1] + (wn * 4) * 2048 + lane * 16;
    uint32_t af[4][8], bf[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      unpack8(*reinterpret_cast<const uint4*>(la + i * 2048),
              *reinterpret_cast<const uint4*>(la + i * 2048 + 1024), af[i]);
      unpack8(*reinterpret_cast<const uint4*>(lb + i * 2048),
              *reinterpret_cast<const uint4*>(lb + i * 2048 + 1024), bf[i]);
    }
    if (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma_fp8(as_v8i(make_uint4(af[i][0], af[i][1], af[i][2], af[i][3]),
                                      make_uint4(af[i][4], af[i][5], af[i][6], af[i][7])),
                               as_v8i(make_uint4(bf[j][0], bf[j][1], bf[j][2], bf[j][3]),
                                      make_uint4(bf[j][4], bf[j][5], bf[j][6], bf[j][7])),
                               acc[i][j]);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v8h ah[4], bh[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ah[i] = e4m3x8_to_f16(af[i][2 * t], af[i][2 * t + 1]);
          bh[i] = e4m3x8_to_f16(bf[i][2 * t], bf[i][2 * t + 1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f16(ah[i], bh[j], acc[i][j]);
      }
    }
    if (more) stage_store(st, lds[cur ^ 1][0], lds[cur ^ 1][1]);
    __syncthreads();
    cur ^= 1;
  }

  const int q = lane >> 4, col = lane & 15;
  if (!DOWN) {
    // packed groups of this wave: g0 + wn*4 + j; pairs for the gated form
    uint8_t* hq = reinterpret_cast<uint8_t*>(out);
    const int I = GATED ? Npk / 2 : Npk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (wm * 4 + i) * 16 + 4 * q + r;
        if (m >= M) continue;
        if (GATED) {
#pragma unroll
          for (int jp = 0; jp < 2; ++jp) {
            const int pair = (g0 + wn * 4) / 2 + jp;
            const float h = gated_h<MODE>(acc[i][2 * jp][r] * alpha_a, acc[i][2 * jp + 1][r] * alpha_b);
            hq[(size_t)m * I + pair * 16 + col] = (uint8_t)e4m3x1(h * inv_out);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int grp = g0 + wn * 4 + j;
            const float h = gated_h<MODE>(0.0f, acc[i][j][r] * alpha_b);
            hq[(size_t)m * I + grp * 16 + col] = (uint8_t)e4m3x1(h * inv_out);
          }
        }
      }
    }
    return;
  }

  // down: optional split-K reduction, then bf16 output
  uint16_t* y = reinterpret_cast<uint16_t*>(out);
  const int N = Npk;
  if (S > 1) {
    float* ps = part + (size_t)s * M * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (wm * 4 + i) * 16 + 4 * q + r;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) ps[(size_t)m * N + (g0 + wn * 4 + j) * 16 + col] = acc[i][j][r];
      }
    __threadfence();
    __syncthreads();
    const int tile = tm * gridDim.x + tn;
    if (threadIdx.x == 0) *s_last = atomicAdd(&cnt[tile], 1u) == (unsigned)(S - 1);
    __syncthreads();
    if (!*s_last) return;
    __threadfence();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0, 0, 0, 0};
    for (int t = 0; t < S; ++t) {
      const float* pt = part + (size_t)t * M * N;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + (wm * 4 + i) * 16 + 4 * q + r;
          if (m >= M) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j][r] += pt[(size_t)m * N + (g0 + wn * 4 + j) * 16 + col];
        }
    }
    if (threadIdx.x == 0) cnt[tile] = 0u;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + (wm * 4 + i) * 16 + 4 * q + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        y[(size_t)m * N + (g0 + wn * 4 + j) * 16 + col] = (uint16_t)f32_to_bf16(acc[i][j][r] * alpha_a);
    }
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------

template <int W>
static void gemv_gateup_w(int act, const uint8_t* xq, const uint8_t* w, uint8_t* hq, int M, int K,
                          int I, float a_g, float a_u, float inv_h, hipStream_t s) {
  dim3 grid(I / 16), block(W * 64);
  if (act == GU_GEGLU)
    hipLaunchKernelGGL((k_gemv_gateup<GU_GEGLU, W>), grid, block, 0, s, xq, w, hq, M, K, I, a_g, a_u, inv_h);
  else if (act == GU_SWIGLU)
    hipLaunchKernelGGL((k_gemv_gateup<GU_SWIGLU, W>), grid, block, 0, s, xq, w, hq, M, K, I, a_g, a_u, inv_h);
  else
    hipLaunchKernelGGL((k_gemv_gateup<GU_GELU, W>), grid, block, 0, s, xq, w, hq, M, K, I, a_g, a_u, inv_h);
}

// waves per workgroup W: 1, 2, 4, 8 or 16 (at most the number of K blocks)
hipError_t launch_gemv_gateup(int act, const uint8_t* xq, const uint8_t* w, uint8_t* hq, int M,
                              int K, int I, int W, float alpha_g, float alpha_u, float inv_h,
                              hipStream_t s) {
  switch (W) {
    case 1: gemv_gateup_w<1>(act, xq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s); break;
    case 2: gemv_gateup_w<2>(act, xq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s); break;
    case 4: gemv_gateup_w<4>(act, xq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s); break;
    case 8: gemv_gateup_w<8>(act, xq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s); break;
    case 16: gemv_gateup_w<16>(act, xq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool FP8>
static hipError_t gemv_down_t(const uint8_t* hq, const uint8_t* w, uint16_t* y, int M, int K,
                              int N, int W, float alpha_d, hipStream_t s) {
  dim3 grid(N / 16), block(W * 64);
  switch (W) {
    case 1: hipLaunchKernelGGL((k_gemv_down<1, FP8>), grid, block, 0, s, hq, w, y, M, K, N, alpha_d); break;
    case 2: hipLaunchKernelGGL((k_gemv_down<2, FP8>), grid, block, 0, s, hq, w, y, M, K, N, alpha_d); break;
    case 4: hipLaunchKernelGGL((k_gemv_down<4, FP8>), grid, block, 0, s, hq, w, y, M, K, N, alpha_d); break;
    case 8: hipLaunchKernelGGL((k_gemv_down<8, FP8>), grid, block, 0, s, hq, w, y, M, K, N, alpha_d); break;
    case 16: hipLaunchKernelGGL((k_gemv_down<16, FP8>), grid, block, 0, s, hq, w, y, M, K, N, alpha_d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_down(const uint8_t* hq, const uint8_t* w, uint16_t* y, int M, int K, int N,
                            int W, bool fp8, float alpha_d, hipStream_t s) {
  return fp8 ? gemv_down_t<true>(hq, w, y, M, K, N, W, alpha_d, s)
             : gemv_down_t<false>(hq, w, y, M, K, N, W, alpha_d, s);
}

hipError_t launch_gemm_gateup(int act, const uint8_t* xq, const uint8_t* w, uint8_t* hq, int M,
                              int K, int Npk, float alpha_g, float alpha_u, float inv_h,
                              hipStream_t s) {
  dim3 grid(Npk / BN, (M + BM - 1) / BM, 1);
  if (act == GU_GEGLU)
    hipLaunchKernelGGL(k_gemm<GU_GEGLU>, grid, dim3(256), 0, s, xq, w, hq, nullptr, nullptr, M, K,
                       Npk, 1, alpha_g, alpha_u, inv_h);
  else if (act == GU_SWIGLU)
    hipLaunchKernelGGL(k_gemm<GU_SWIGLU>, grid, dim3(256), 0, s, xq, w, hq, nullptr, nullptr, M,
                       K, Npk, 1, alpha_g, alpha_u, inv_h);
  else
    hipLaunchKernelGGL(k_gemm<GU_GELU>, grid, dim3(256), 0, s, xq, w, hq, nullptr, nullptr, M, K,
                       Npk, 1, alpha_g, alpha_u, inv_h);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const uint8_t* hq, const uint8_t* w, uint16_t* y, float* part,
                            uint32_t* cnt, int M, int K, int N, int S, bool fp8, float alpha_d,
                            hipStream_t s) {
  dim3 grid(N / BN, (M + BM - 1) / BM, S);
  if (fp8)
    hipLaunchKernelGGL(k_gemm<4>, grid, dim3(256), 0, s, hq, w, y, part, cnt, M, K, N, S, alpha_d,
                       0.0f, 0.0f);
  else
    hipLaunchKernelGGL(k_gemm<3>, grid, dim3(256), 0, s, hq, w, y, part, cnt, M, K, N, S, alpha_d,
                       0.0f, 0.0f);
  return hipGetLastError();
}

}  // namespace frt
