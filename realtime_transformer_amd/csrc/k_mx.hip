// k_mx.hip -- the MXFP4 form of the FFN block's two GEMMs (M <= 64) and the
// packing of its weights.
//
// itsolotime article, section 7.2 (the NVFP4 encoder FFN: AWQ pre-scaled
// activations, 4-bit gate/up and down GEMMs, a gated combine that
// re-quantises to 4 bits, a high-precision residual); the format here is OCP
// MXFP4 (frt_mx.h) on gfx950's block-scaled FP4 matrix instructions.
//
// Packed weights.  Codes: 1 KiB per (16-row group, 128-K block), lane l's 16
// bytes at l*16 hold row l%16, K values (l/16)*32 .. +32 (two per byte, low
// nibble first) -- exactly the operand of v_mfma_scale_f32_16x16x128_f8f6f4
// with FP4 inputs.  Scales: per (group, four K blocks) 64 lanes x 4 bytes,
// byte j of lane l = exponent of row l%16, K block 4*kb4 + j, sub-block l/16
// (mx_code_off / mx_scale_off in frt_mx.h).  Gate and up groups interleave as
// in the FP8 layout (group 2i gate, 2i + 1 up).
//
// Products: one scaled MFMA multiplies 16 activation rows by 16 weight rows
// over 128 K values with each lane's E8M0 scales applied per 32-block; within
// an instruction the FP4 products are exact and the sum is accurate to an
// fp32 rounding (measured), across instructions the accumulator is fp32.
#include <type_traits>

#include "frt_mx.h"

namespace frt {

// One thread per (row n, 32-block b) of src [N][K] bf16 (times colw[k] when
// given, an exact product): block exponent, 32 codes into the packed layout.
// mode 0: packed row n, 1: gate row, 2: up row (gated layout).
__global__ __launch_bounds__(256) void k_quant_mx(const uint16_t* __restrict__ src, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales, int N, int K, int mode,
                                                  const uint16_t* __restrict__ colw, int mm_layout) {
  const size_t nb = (size_t)K / 32;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)N * nb) return;
  const int n = (int)(idx / nb), b = (int)(idx % nb);
  const uint4* sp = reinterpret_cast<const uint4*>(src + (size_t)n * K + (size_t)b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 a = sp[q];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = bf16_lo(w[j]);
      v[8 * q + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
  if (colw) {
    const uint4* cp = reinterpret_cast<const uint4*>(colw + (size_t)b * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 a = cp[q];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * q + 2 * j] = v[8 * q + 2 * j] * bf16_lo(w[j]);
        v[8 * q + 2 * j + 1] = v[8 * q + 2 * j + 1] * bf16_hi(w[j]);
      }
    }
  }
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) am = __builtin_fmaxf(am, __builtin_fabsf(v[j]));
  const int e = mx_block_exp(am);
  uint32_t out[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = mx_pack8(v + 8 * q, e);
  const uint32_t prow = mode == 0 ? (uint32_t)n : (mode == 1 ? gate_row((uint32_t)n) : up_row_gated((uint32_t)n));
  if (mm_layout == 2) {  // the column-quad order (down matrix, mode 0)
    *reinterpret_cast<uint4*>(codes + mx_quad_code_off(prow, (uint32_t)b, (uint32_t)K)) =
        make_uint4(out[0], out[1], out[2], out[3]);
    scales[mx_quad_scale_off(prow, (uint32_t)b, (uint32_t)K)] = (uint8_t)e;
    return;
  }
  const uint32_t KB = (uint32_t)K / 128, kb = (uint32_t)b >> 2, lane = (prow & 15u) + 16u * ((uint32_t)b & 3u);
  *reinterpret_cast<uint4*>(codes + mx_code_off(prow, kb, lane, KB)) = make_uint4(out[0], out[1], out[2], out[3]);
  scales[mm_layout ? mx_scale_off_mm(prow, kb, lane, KB) : mx_scale_off(prow, kb, lane, KB)] = (uint8_t)e;
}

// mm_layout: 1 exponents in the prefill GEMM's layout (mx_scale_off_mm); 2
// codes and exponents in the column-quad order (mx_quad_code_off)
hipError_t launch_quant_mx(const uint16_t* src, uint8_t* codes, uint8_t* scales, int N, int K, int mode,
                           const uint16_t* colw, hipStream_t s, int mm_layout) {
  if (K % 512) return hipErrorInvalidValue;
  if (mm_layout == 2 && (mode != 0 || N % 4)) return hipErrorInvalidValue;  // column quads of a plain matrix
  const size_t n = (size_t)N * (K / 32);
  hipLaunchKernelGGL(k_quant_mx, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, codes, scales, N, K, mode,
                     colw, mm_layout);
  return hipGetLastError();
}

typedef unsigned v4u_mx __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i mx_w16(const uint8_t* p) {
  const v4u_mx a = __builtin_nontemporal_load(reinterpret_cast<const v4u_mx*>(p));
  v8i r;
  r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}
__device__ __forceinline__ v8i mx_x16(const uint8_t* p, bool has) {
  uint4 a = make_uint4(0, 0, 0, 0);
  if (has) a = *reinterpret_cast<const uint4*>(p);
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// Activation row pointers of tile t: codes [M][K/2]; the lane's exponent
// dword of quad 0 in the GEMV layout (mx_act_scale_off_gemv).
struct MxRows {
  const uint8_t* c;
  const uint8_t* s;
  bool has;
};

// Gate/up: one workgroup per 32 intermediate columns (packed groups 4P..4P+3
// = gate 2P, up 2P, gate 2P+1, up 2P+1), W waves splitting the K blocks, MT
// activation tiles of 16 rows.  Epilogue (wave t < MT, tile t): h for 32
// columns of each row, the block exponent from the 16 lanes of that row, two
// codes per byte (the even lane writes), exponent from lane 0 of the row.
template <int ACT, int W, int MT>
__global__ __launch_bounds__(W * 64) void k_gemv_gateup_mx(const uint8_t* __restrict__ xc,
                                                           const uint8_t* __restrict__ xs,
                                                           const uint8_t* __restrict__ wc,
                                                           const uint8_t* __restrict__ ws, uint8_t* __restrict__ hc,
                                                           uint8_t* __restrict__ hs, int M, int K, int I) {
  constexpr bool GATED = ACT != MX_GELU;
  constexpr int NA = GATED ? 4 : 2;  // accumulators per tile
  static_assert(W >= MT, "one wave per tile finishes the epilogue");
  __shared__ v4f red[W][MT][NA][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = blockIdx.x;
  const int KB = K >> 7, KQ = KB >> 2;  // K blocks, quads of four
  const int kq0 = wave * KQ / W, kq1 = (wave + 1) * KQ / W;
  const int row = lane & 15, q = lane >> 4;
  // packed groups of this workgroup (gated: g0 u0 g1 u1; plain: u0 u1)
  uint32_t grp[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) grp[a] = (uint32_t)(NA * P + a);
  MxRows xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + row;
    xr[t].has = m < M;
    const int mm = xr[t].has ? m : 0;
    xr[t].c = xc + (size_t)mm * (K / 2) + q * 16;
    xr[t].s = xs + ((size_t)t * KQ * 64 + lane) * 4;  // this lane's exponent dword of quad 0
  }
  v4f acc[MT][NA];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[t][a] = v4f{0, 0, 0, 0};

  // one quad of K blocks per step: every load of the step (four code runs
  // per operand and one exponent dword per operand) is issued before its
  // MFMAs, which take exponent byte u of each dword through op_sel
  for (int kq = kq0; kq < kq1; ++kq) {
    v8i wv[4][NA], xv[4][MT];
    int wsd[NA], xsd[MT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
      wsd[a] = *reinterpret_cast<const int*>(ws + mx_scale_off(grp[a] * 16, 4 * kq, lane, KB));
#pragma unroll
    for (int t = 0; t < MT; ++t) xsd[t] = xr[t].has ? *reinterpret_cast<const int*>(xr[t].s + (size_t)kq * 256) : 0x7f7f7f7f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int a = 0; a < NA; ++a) wv[u][a] = mx_w16(wc + mx_code_off(grp[a] * 16, 4 * kq + u, lane, KB));
#pragma unroll
      for (int t = 0; t < MT; ++t) xv[u][t] = mx_x16(xr[t].c + (size_t)(4 * kq + u) * 64, xr[t].has);
    }
    auto step = [&](auto U) {
      constexpr int u = decltype(U)::value;
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int a = 0; a < NA; ++a) acc[t][a] = mx_mfma_u<u>(xv[u][t], xsd[t], wv[u][a], wsd[a], acc[t][a]);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int a = 0; a < NA; ++a) red[wave][t][a][lane] = acc[t][a];
  __syncthreads();
  if (wave >= MT) return;
  const int t = wave;
  v4f f[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    f[a] = red[0][t][a][lane];
#pragma unroll
    for (int v = 1; v < W; ++v) f[a] += red[v][t][a][lane];
  }
  // lane holds rows m = 16t + 4q + r, columns 32P + row and 32P + 16 + row
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 16 * t + 4 * q + r;
    const float h0 = GATED ? mx_gated<ACT>(f[0][r], f[1][r]) : mx_gated<ACT>(0.0f, f[0][r]);
    const float h1 = GATED ? mx_gated<ACT>(f[2][r], f[3][r]) : mx_gated<ACT>(0.0f, f[1][r]);
    const int mm = m < M ? m : 0;
    mx_store_h32(h0, h1, m < M, row, hc + (size_t)mm * (I / 2) + (size_t)P * 16,
                 hs + mx_act_scale_off_gemv((uint32_t)mm, (uint32_t)P, (uint32_t)I / 128));
  }
}

// Decode gate/up (M <= 16) that finishes the norm itself, as the E4M3
// k_gemv_gateup_nq: after k_add_sumsq has formed r' and the slice sums of
// r'^2, each wave forms the MXFP4 activation of its own K quads,
// x = f32(f32(f32(r' * inv_rms) * w_norm) * inv_awq) with inv_rms =
// f32(1 / sqrt(S / K + eps)) in fp64 from the row's slice sums in slice
// order (the arithmetic of the MXFP4 k_add_rmsnorm_quant), each 32-block's
// exponent from the 4-lane maximum of its chunks, the codes and exponents
// into a wave-private LDS copy of the activation slot (codes [M][K/2],
// exponents in the GEMV layout), and multiplies from there.  Workgroup 0
// also stores them to the slot.  Loads are issued as: slice sums, the
// r' / w_norm / inv_awq chunks, then the first quad's weights.
struct MxNormQ {
  const uint16_t* r;       // r' bf16 [M][K]
  const uint16_t* w_norm;  // RMSNorm weight bf16 [K]
  const float* inv_awq;    // AWQ reciprocal fp32 [K]
  const double* sq;        // slice sums fp64 [M][G]
  int G;
  float eps;
  uint8_t* xc_out;         // codes [M][K/2]
  uint8_t* xs_out;         // exponents, GEMV layout (rows padded to 16)
};
constexpr int kMxNqChunks = 2;      // 8-element chunks per lane whose loads are issued together
constexpr int kMxNqLdsBytes = 16384;  // codes M*K/2 + exponents K/2
constexpr int kMxNqMaxSlices = 16;
constexpr int kMxNqWidePairs = 4;  // WIDE: 16-byte slice-sum loads per thread, M * G <= 8 * 64 * W

// WIDE (M <= 4): the slice sums are those of the whole-column down GEMV, one
// per four columns (G = K / 4): the workgroup's threads load them as
// 16-byte pairs, add their pairs per row in index order, and the waves'
// totals meet in LDS, added in wave order (fp64 throughout; the terms are
// squares of bf16 values, so the total does not depend on the order).
template <int ACT, int W, bool WIDE = false, int NP = kMxNqWidePairs>
__global__ __launch_bounds__(W * 64) void k_gemv_gateup_mx_nq(const MxNormQ nq, const uint8_t* __restrict__ wc,
                                                              const uint8_t* __restrict__ ws,
                                                              uint8_t* __restrict__ hc, uint8_t* __restrict__ hs,
                                                              int M, int K, int I) {
  constexpr bool GATED = ACT != MX_GELU;
  constexpr int NA = GATED ? 4 : 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];  // codes [M][K/2], then exponents [K/2]
  __shared__ v4f red[W][NA][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int P = blockIdx.x;
  const int KB = K >> 7, KQ = KB >> 2;
  const int kq0 = wave * KQ / W, kq1 = (wave + 1) * KQ / W;  // empty when W > KQ
  const int row = lane & 15, q = lane >> 4;
  const bool has = row < M;
  // a wave without quads loads the last quad's activations and weights (in
  // bounds, unused) so that no load sits behind a branch, and writes nothing
  const bool work = kq1 > kq0;
  const int kqa = work ? kq0 : KQ - 1, nqw = work ? kq1 - kq0 : 1;
  uint8_t* lds_c = xlds;
  uint8_t* lds_s = xlds + (size_t)M * (K / 2);
  uint32_t grp[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) grp[a] = (uint32_t)(NA * P + a);

  // (1) activation-side loads: 64-chunk groups (512 elements, one row each)
  const int G = nq.G;
  double part_v = 0.0;
  double2 sqp[WIDE ? NP : 1];
  if (WIDE) {
    const int npairs = (M * G) >> 1;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int i = (int)threadIdx.x + j * W * 64;
      sqp[j] = reinterpret_cast<const double2*>(nq.sq)[i < npairs ? i : npairs - 1];
    }
  } else {
    part_v = nq.sq[lane < M * G ? lane : M * G - 1];
  }
  const int ngrp = M * nqw;
  int gm[kMxNqChunks], gk[kMxNqChunks];
  uint4 rv[kMxNqChunks], wv[kMxNqChunks];
  float4 av[kMxNqChunks][2];
  auto load_group = [&](int g0) {
#pragma unroll
    for (int j = 0; j < kMxNqChunks; ++j) {
      int g = g0 + j;
      g = g < ngrp ? g : ngrp - 1;  // a missing group redoes the last (same bytes)
      const int m = g / nqw;
      gm[j] = m;
      gk[j] = (kqa * 64 + (g - m * nqw) * 64 + lane) * 8;  // first element of the lane's chunk
      rv[j] = *reinterpret_cast<const uint4*>(nq.r + (size_t)m * K + gk[j]);
      wv[j] = *reinterpret_cast<const uint4*>(nq.w_norm + gk[j]);
      av[j][0] = *reinterpret_cast<const float4*>(nq.inv_awq + gk[j]);
      av[j][1] = *reinterpret_cast<const float4*>(nq.inv_awq + gk[j] + 4);
    }
  };
  load_group(0);
  __builtin_amdgcn_sched_barrier(0);

  // (2) the first quad's weights
  v8i wq[4][NA];
  int wsd[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) wsd[a] = *reinterpret_cast<const int*>(ws + mx_scale_off(grp[a] * 16, 4 * kqa, lane, KB));
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int a = 0; a < NA; ++a) wq[u][a] = mx_w16(wc + mx_code_off(grp[a] * 16, 4 * kqa + u, lane, KB));
  __builtin_amdgcn_sched_barrier(0);

  // (3) 1/rms of row `lane` (lanes < M), then this wave's codes and exponents
  double ssum = 0.0;
  if (WIDE) {
    __shared__ double wsum[W][4];
    const int npairs = (M * G) >> 1;
    double rs[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int i = (int)threadIdx.x + j * W * 64;
      const int m = (2 * i) / G;  // a pair never straddles rows (G even)
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
        if (i < npairs && m == mm) {
          rs[mm] += sqp[j].x;
          rs[mm] += sqp[j].y;
        }
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      if (mm >= M) break;  // uniform
      const double t = wave_sum_f64(rs[mm]);
      if (lane == 0) wsum[wave][mm] = t;
    }
    __syncthreads();
    const int mrow = lane < M ? lane : 0;
#pragma unroll
    for (int v = 0; v < W; ++v) ssum += wsum[v][mrow & 3];
  } else {
    const double part = lane < M * G ? part_v : 0.0;
    const int base = lane < M ? lane * G : 0;
    const unsigned long long b = (unsigned long long)__double_as_longlong(part);
#pragma unroll
    for (int g = 0; g < kMxNqMaxSlices; ++g) {
      const int src = base + (g < G ? g : 0);
      const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)b, src, 64);
      const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(b >> 32), src, 64);
      const double v = __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
      ssum += g < G ? v : 0.0;
    }
  }
  const float inv_rms = (float)(1.0 / sqrt(ssum / (double)K + (double)nq.eps));
  const bool store_x = blockIdx.x == 0;
  auto quant_group = [&](int g0) {
#pragma unroll
    for (int j = 0; j < kMxNqChunks; ++j) {
      if (!work || g0 + j >= ngrp) continue;  // uniform
      const float inv = __shfl(inv_rms, gm[j], 64);
      const uint32_t rr[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
      const uint32_t ww[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
      const float aw[8] = {av[j][0].x, av[j][0].y, av[j][0].z, av[j][0].w,
                           av[j][1].x, av[j][1].y, av[j][1].z, av[j][1].w};
      float x[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        x[2 * t] = (bf16_lo(rr[t]) * inv) * bf16_lo(ww[t]);
        x[2 * t + 1] = (bf16_hi(rr[t]) * inv) * bf16_hi(ww[t]);
      }
      float am = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        x[t] = x[t] * aw[t];
        am = __builtin_fmaxf(am, __builtin_fabsf(x[t]));
      }
      am = quad_max(am);
      const int e = mx_block_exp(am);
      const uint32_t codes = mx_pack8(x, e);
      const uint32_t m = (uint32_t)gm[j], ch = (uint32_t)gk[j] >> 3;
      const size_t co = (size_t)m * (K / 2) + (size_t)ch * 4;
      const size_t so = mx_act_scale_off_gemv(m, ch >> 2, (uint32_t)KB);
      *reinterpret_cast<uint32_t*>(lds_c + co) = codes;
      if ((ch & 3) == 0) lds_s[so] = (uint8_t)e;
      if (store_x) {
        *reinterpret_cast<uint32_t*>(nq.xc_out + co) = codes;
        if ((ch & 3) == 0) nq.xs_out[so] = (uint8_t)e;
      }
    }
  };
  quant_group(0);
  for (int g0 = kMxNqChunks; g0 < ngrp; g0 += kMxNqChunks) {
    load_group(g0);
    quant_group(g0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // (4) the GEMV over this wave's quads, activations from LDS
  v4f acc[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) acc[a] = v4f{0, 0, 0, 0};
  const uint8_t* xcl = lds_c + (size_t)(has ? row : 0) * (K / 2) + q * 16;
  for (int kq = kq0; kq < kq1; ++kq) {
    if (kq != kq0) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
        wsd[a] = *reinterpret_cast<const int*>(ws + mx_scale_off(grp[a] * 16, 4 * kq, lane, KB));
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int a = 0; a < NA; ++a) wq[u][a] = mx_w16(wc + mx_code_off(grp[a] * 16, 4 * kq + u, lane, KB));
    }
    const int xsd = has ? *reinterpret_cast<const int*>(lds_s + ((size_t)kq * 64 + lane) * 4) : 0x7f7f7f7f;
    v8i xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint4 c = make_uint4(0, 0, 0, 0);
      if (has) c = *reinterpret_cast<const uint4*>(xcl + (size_t)(4 * kq + u) * 64);
      xv[u][0] = (int)c.x; xv[u][1] = (int)c.y; xv[u][2] = (int)c.z; xv[u][3] = (int)c.w;
      xv[u][4] = 0; xv[u][5] = 0; xv[u][6] = 0; xv[u][7] = 0;
    }
    auto step = [&](auto U) {
      constexpr int u = decltype(U)::value;
#pragma unroll
      for (int a = 0; a < NA; ++a) acc[a] = mx_mfma_u<u>(xv[u], xsd, wq[u][a], wsd[a], acc[a]);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
  }
#pragma unroll
  for (int a = 0; a < NA; ++a) red[wave][a][lane] = acc[a];
  __syncthreads();
  if (wave != 0) return;
  v4f f[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    f[a] = red[0][a][lane];
#pragma unroll
    for (int v = 1; v < W; ++v) f[a] += red[v][a][lane];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * q + r;
    const float h0 = GATED ? mx_gated<ACT>(f[0][r], f[1][r]) : mx_gated<ACT>(0.0f, f[0][r]);
    const float h1 = GATED ? mx_gated<ACT>(f[2][r], f[3][r]) : mx_gated<ACT>(0.0f, f[1][r]);
    const int mm = m < M ? m : 0;
    mx_store_h32(h0, h1, m < M, row, hc + (size_t)mm * (I / 2) + (size_t)P * 16,
                 hs + mx_act_scale_off_gemv((uint32_t)mm, (uint32_t)P, (uint32_t)I / 128));
  }
}

// Down: one workgroup per 16 output columns and K split (gridDim.y), W waves
// splitting the split's K blocks, MT tiles.  One split: bf16 Y; several:
// fp32 partials [split][M][N] for the consumer (as the FP8 form).
template <int W, int MT>
__global__ __launch_bounds__(W * 64) void k_gemv_down_mx(const uint8_t* __restrict__ hc,
                                                         const uint8_t* __restrict__ hs,
                                                         const uint8_t* __restrict__ wc,
                                                         const uint8_t* __restrict__ ws, uint16_t* __restrict__ y,
                                                         float* __restrict__ part, int M, int K, int N) {
  static_assert(W >= MT, "one wave per tile finishes the epilogue");
  __shared__ v4f red[W][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = blockIdx.x;
  const int KB = K >> 7, KQ = KB >> 2;  // K blocks, quads of four
  const int S = gridDim.y, sp = blockIdx.y;
  const int ks0 = sp * KQ / S, ks1 = (sp + 1) * KQ / S;
  const int kq0 = ks0 + wave * (ks1 - ks0) / W, kq1 = ks0 + (wave + 1) * (ks1 - ks0) / W;
  const int row = lane & 15, q = lane >> 4;
  MxRows xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + row;
    xr[t].has = m < M;
    const int mm = xr[t].has ? m : 0;
    xr[t].c = hc + (size_t)mm * (K / 2) + q * 16;
    xr[t].s = hs + ((size_t)t * KQ * 64 + lane) * 4;  // this lane's exponent dword of quad 0
  }
  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4f{0, 0, 0, 0};
  // one quad of K blocks per step, as in the gate/up GEMV
  for (int kq = kq0; kq < kq1; ++kq) {
    v8i wv[4], xv[4][MT];
    const int wsd = *reinterpret_cast<const int*>(ws + mx_scale_off((uint32_t)p * 16, 4 * kq, lane, KB));
    int xsd[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xsd[t] = xr[t].has ? *reinterpret_cast<const int*>(xr[t].s + (size_t)kq * 256) : 0x7f7f7f7f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wv[u] = mx_w16(wc + mx_code_off((uint32_t)p * 16, 4 * kq + u, lane, KB));
#pragma unroll
      for (int t = 0; t < MT; ++t) xv[u][t] = mx_x16(xr[t].c + (size_t)(4 * kq + u) * 64, xr[t].has);
    }
    auto step = [&](auto U) {
      constexpr int u = decltype(U)::value;
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mx_mfma_u<u>(xv[u][t], xsd[t], wv[u], wsd, acc[t]);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave >= MT) return;
  const int t = wave;
  v4f a = red[0][t][lane];
#pragma unroll
  for (int v = 1; v < W; ++v) a += red[v][t][lane];
  float* ps = part + (size_t)sp * M * N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 16 * t + 4 * q + r;
    if (m < M) {
      if (S == 1)
        y[(size_t)m * N + p * 16 + row] = (uint16_t)f32_to_bf16(a[r]);
      else
        ps[(size_t)m * N + p * 16 + row] = a[r];
    }
  }
}

// Whole-column down GEMV (M <= 4), MXFP4 down matrix in the column-quad
// order (mx_quad_code_off): one workgroup per four output columns reads
// them over all of K, so it owns their sums and neither split-K partials
// nor a norm kernel follow it.  Step t covers K values 512 t .. 512 t + 511
// dealt to four parts of 128 (part p: 512 t + 128 p ..), and one scaled
// MFMA takes the four parts side by side: operand row 4 p' + m' is
// activation row m' over part p', operand column 4 p + c weight column c
// over part p, each lane's exponent byte scaling its own 32 values; the
// products with p' == p are the parts' partial dot products, the others
// are discarded (lanes 20 p + c hold part p of column c, row m in element
// m).  Per step a lane loads 16 weight code bytes and one exponent byte
// (1 KiB + 64 bytes per step) and the 16 code bytes and exponent byte
// of its activation row and part.  The epilogue forms, for its columns,
//   Y = bf16(sum),  R' = bf16(R + Y)  (R' and Z alike: r_out),
//   and the fp64 sum of R'^2 over the four columns, slice c4 of row m of
//   sq [M][N / 4] (the next layer's split norm reads these slices);
// r_out == nullptr stores Y only.  Steps are pipelined over two register
// sets (the loads of step i + 1 issued before the MFMA of step i); rows
// m' >= M read row 0, whose products reach only discarded rows.
template <int W>
__global__ __launch_bounds__(W * 64) void k_gemv_down_mx_quad(const uint8_t* __restrict__ hc,
                                                              const uint8_t* __restrict__ hs,
                                                              const uint8_t* __restrict__ wc,
                                                              const uint8_t* __restrict__ ws,
                                                              const uint16_t* __restrict__ r_in,
                                                              uint16_t* __restrict__ y, uint16_t* __restrict__ r_out,
                                                              double* __restrict__ sq, int M, int K, int N) {
  __shared__ v4f red[W][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c4 = blockIdx.x;
  const int T = K >> 9;
  const int t0 = wave * T / W, t1 = (wave + 1) * T / W;
  const int part = (lane & 15) >> 2, mr = lane & 3, sb = lane >> 4;
  const int mx = mr < M ? mr : 0;
  const uint8_t* wp = wc + ((size_t)c4 * T * 64 + lane) * 16;
  const uint8_t* wsp = ws + (size_t)c4 * T * 64 + lane;
  const uint8_t* xp = hc + (size_t)mx * (K / 2) + part * 64 + sb * 16;
  const uint8_t* xsp = hs + (size_t)(sb * 16 + mx) * 4 + part;  // + 256 t: mx_act_scale_off_gemv, tile 0
  const int nstep = t1 - t0;
  struct Step {
    v4u_mx w, x;
    uint32_t we, xe;
  };
  // step i (clamped to the range: a clamped step is loaded, not used)
  auto load_step = [&](Step& st, int i) {
    const int t = t0 + (i < nstep ? i : nstep - 1);
    st.w = __builtin_nontemporal_load(reinterpret_cast<const v4u_mx*>(wp + (size_t)t * 1024));
    st.we = wsp[(size_t)t * 64];
    st.x = *reinterpret_cast<const v4u_mx*>(xp + (size_t)t * 256);
    st.xe = xsp[(size_t)t * 256];
  };
  v4f acc = {0, 0, 0, 0};
  auto mma_step = [&](Step& st, int i) {
    asm volatile("" : "+v"(st.w[0]), "+v"(st.w[1]), "+v"(st.w[2]), "+v"(st.w[3]));
    asm volatile("" : "+v"(st.x[0]), "+v"(st.x[1]), "+v"(st.x[2]), "+v"(st.x[3]), "+v"(st.we), "+v"(st.xe));
    if (i < nstep) {  // wave-uniform
      v8i a, b;
      a[0] = (int)st.x[0]; a[1] = (int)st.x[1]; a[2] = (int)st.x[2]; a[3] = (int)st.x[3];
      a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
      b[0] = (int)st.w[0]; b[1] = (int)st.w[1]; b[2] = (int)st.w[2]; b[3] = (int)st.w[3];
      b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
      acc = mx_mfma_u<0>(a, (int)st.xe, b, (int)st.we, acc);
    }
  };
  // wave 0 (which runs the epilogue) requests its columns' R values right
  // after its first weights, so that they arrive during the stream (rows
  // clamped to M - 1; any valid address when R is not needed)
  uint16_t rv[4] = {0, 0, 0, 0};
  if (nstep > 0) {
    Step A, B;
    load_step(A, 0);
    if (wave == 0) {
      const uint16_t* rp = r_in ? r_in : y;
#pragma unroll
      for (int m = 0; m < 4; ++m) rv[m] = rp[(size_t)(m < M ? m : M - 1) * N + (size_t)c4 * 4 + (lane & 3)];
    }
    int i = 0;
    for (; i + 2 < nstep; i += 2) {
      load_step(B, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(A, i);
      load_step(A, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(B, i + 1);
    }
    if (i + 1 < nstep) {
      load_step(B, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(A, i);
      mma_step(B, i + 1);
    } else {
      mma_step(A, i);
    }
  }
  if (W > 1) {
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    acc = red[0][lane];
#pragma unroll
    for (int v = 1; v < W; ++v) acc += red[v][lane];
  }
  // column c = lane & 3 of lanes 0..3: its parts in order, then the epilogue
  const int c = lane & 3;
  float tot[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float q0 = __shfl(acc[m], c, 64), q1 = __shfl(acc[m], 20 + c, 64);
    const float q2 = __shfl(acc[m], 40 + c, 64), q3 = __shfl(acc[m], 60 + c, 64);
    tot[m] = ((q0 + q1) + q2) + q3;
  }
  const size_t col = (size_t)c4 * 4 + c;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m >= M) break;  // uniform
    const uint32_t yb = f32_to_bf16(tot[m]);
    double d = 0.0;
    if (lane < 4) {
      y[(size_t)m * N + col] = (uint16_t)yb;
      if (r_out) {
        const float rf = __uint_as_float((uint32_t)rv[m] << 16);
        const uint32_t rb = f32_to_bf16(rf + __uint_as_float(yb << 16));
        r_out[(size_t)m * N + col] = (uint16_t)rb;
        const double rd = (double)__uint_as_float(rb << 16);
        d = rd * rd;
      }
    }
    if (r_out) {
      const double d1 = __shfl(d, 1, 64), d2 = __shfl(d, 2, 64), d3 = __shfl(d, 3, 64);
      if (lane == 0) sq[(size_t)m * (N >> 2) + c4] = ((d + d1) + d2) + d3;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers: W in {4, 5, 8, 10, 16} (gate/up; {4, 8, 16} down), MT = ceil(M / 16) <= 4, W * MT <= 16 (the
// reduction buffer: W * MT * NA KiB of LDS)
// ---------------------------------------------------------------------------

template <int ACT, int W, int MT>
static hipError_t gateup_mx_t(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws,
                              uint8_t* hc, uint8_t* hs, int M, int K, int I, hipStream_t s) {
  if constexpr (W >= MT && W * MT <= 16) {
    hipLaunchKernelGGL((k_gemv_gateup_mx<ACT, W, MT>), dim3(I / 32), dim3(W * 64), 0, s, xc, xs, wc, ws, hc, hs, M,
                       K, I);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <int ACT, int W>
static hipError_t gateup_mx_w(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws,
                              uint8_t* hc, uint8_t* hs, int M, int K, int I, hipStream_t s) {
  switch ((M + 15) / 16) {
    case 1: return gateup_mx_t<ACT, W, 1>(xc, xs, wc, ws, hc, hs, M, K, I, s);
    case 2: return gateup_mx_t<ACT, W, 2>(xc, xs, wc, ws, hc, hs, M, K, I, s);
    case 3: return gateup_mx_t<ACT, W, 3>(xc, xs, wc, ws, hc, hs, M, K, I, s);
    case 4: return gateup_mx_t<ACT, W, 4>(xc, xs, wc, ws, hc, hs, M, K, I, s);
    default: return hipErrorInvalidValue;
  }
}

template <int ACT>
static hipError_t gateup_mx_act(int W, const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws,
                                uint8_t* hc, uint8_t* hs, int M, int K, int I, hipStream_t s) {
  if (W == 4) return gateup_mx_w<ACT, 4>(xc, xs, wc, ws, hc, hs, M, K, I, s);
  if (W == 5) return gateup_mx_w<ACT, 5>(xc, xs, wc, ws, hc, hs, M, K, I, s);
  if (W == 8) return gateup_mx_w<ACT, 8>(xc, xs, wc, ws, hc, hs, M, K, I, s);
  if (W == 10) return gateup_mx_w<ACT, 10>(xc, xs, wc, ws, hc, hs, M, K, I, s);
  if (W == 16) return gateup_mx_w<ACT, 16>(xc, xs, wc, ws, hc, hs, M, K, I, s);
  return hipErrorInvalidValue;
}

int gemv_mx_max_waves(int M) { return M <= 16 ? 16 : (M <= 32 ? 8 : 4); }

template <int ACT, int W>
static void gateup_mx_nq_t(const MxNormQ& nq, const uint8_t* wc, const uint8_t* ws, uint8_t* hc, uint8_t* hs, int M,
                           int K, int I, bool wide, hipStream_t s) {
  const size_t lds = (size_t)M * (K / 2) + (size_t)K / 2;
  // two slice-sum pairs per thread where they cover the rows, else four
  if (wide && M * (K / 4) / 2 <= 2 * W * 64)
    hipLaunchKernelGGL((k_gemv_gateup_mx_nq<ACT, W, true, 2>), dim3(I / 32), dim3(W * 64), lds, s, nq, wc, ws, hc, hs,
                       M, K, I);
  else if (wide)
    hipLaunchKernelGGL((k_gemv_gateup_mx_nq<ACT, W, true, 4>), dim3(I / 32), dim3(W * 64), lds, s, nq, wc, ws, hc, hs,
                       M, K, I);
  else
    hipLaunchKernelGGL((k_gemv_gateup_mx_nq<ACT, W, false>), dim3(I / 32), dim3(W * 64), lds, s, nq, wc, ws, hc, hs,
                       M, K, I);
}

template <int ACT>
static hipError_t gateup_mx_nq_act(int W, const MxNormQ& nq, const uint8_t* wc, const uint8_t* ws, uint8_t* hc,
                                   uint8_t* hs, int M, int K, int I, bool wide, hipStream_t s) {
  switch (W) {
    case 4: gateup_mx_nq_t<ACT, 4>(nq, wc, ws, hc, hs, M, K, I, wide, s); break;
    case 5: gateup_mx_nq_t<ACT, 5>(nq, wc, ws, hc, hs, M, K, I, wide, s); break;
    case 8: gateup_mx_nq_t<ACT, 8>(nq, wc, ws, hc, hs, M, K, I, wide, s); break;
    case 10: gateup_mx_nq_t<ACT, 10>(nq, wc, ws, hc, hs, M, K, I, wide, s); break;
    case 16: gateup_mx_nq_t<ACT, 16>(nq, wc, ws, hc, hs, M, K, I, wide, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Whether k_gemv_gateup_mx_nq takes the shape (the LDS copy of the slot fits,
// every slice sum has a lane).
bool gemv_mx_nq_supported(int M, int K, int G) {
  return M >= 1 && M <= 16 && K % 512 == 0 && (long)M * (K / 2) + K / 2 <= kMxNqLdsBytes && G >= 1 &&
         G <= kMxNqMaxSlices && M * G <= 64;
}

// ... with the whole-column down GEMV's slice sums (G = K / 4) on W waves
bool gemv_mx_nq_wide_supported(int M, int K, int W) {
  const int G = K / 4;
  return M >= 1 && M <= 4 && K % 512 == 0 && (long)M * (K / 2) + K / 2 <= kMxNqLdsBytes &&
         M * G <= 2 * kMxNqWidePairs * 64 * W;
}

// G == K / 4 selects the whole-column down GEMV's slice sums (WIDE)
hipError_t launch_gemv_gateup_mx_nq(int act, const uint16_t* r, const uint16_t* w_norm, const float* inv_awq,
                                    const double* sq, int G, float eps, uint8_t* xc_out, uint8_t* xs_out,
                                    const uint8_t* wc, const uint8_t* ws, uint8_t* hc, uint8_t* hs, int M, int K,
                                    int I, int W, hipStream_t s) {
  const bool wide = K >= 64 && G == K / 4;
  if (!(wide ? gemv_mx_nq_wide_supported(M, K, W) : gemv_mx_nq_supported(M, K, G)) || I % 32 || !inv_awq)
    return hipErrorInvalidValue;
  const MxNormQ nq{r, w_norm, inv_awq, sq, G, eps, xc_out, xs_out};
  if (act == MX_GEGLU) return gateup_mx_nq_act<MX_GEGLU>(W, nq, wc, ws, hc, hs, M, K, I, wide, s);
  if (act == MX_SWIGLU) return gateup_mx_nq_act<MX_SWIGLU>(W, nq, wc, ws, hc, hs, M, K, I, wide, s);
  return gateup_mx_nq_act<MX_GELU>(W, nq, wc, ws, hc, hs, M, K, I, wide, s);
}

hipError_t launch_gemv_gateup_mx(int act, const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws,
                                 uint8_t* hc, uint8_t* hs, int M, int K, int I, int W, hipStream_t s) {
  if (M < 1 || M > 64 || K % 512 || I % 32) return hipErrorInvalidValue;
  if (act == MX_GEGLU) return gateup_mx_act<MX_GEGLU>(W, xc, xs, wc, ws, hc, hs, M, K, I, s);
  if (act == MX_SWIGLU) return gateup_mx_act<MX_SWIGLU>(W, xc, xs, wc, ws, hc, hs, M, K, I, s);
  return gateup_mx_act<MX_GELU>(W, xc, xs, wc, ws, hc, hs, M, K, I, s);
}

template <int W, int MT>
static hipError_t down_mx_t(const uint8_t* hc, const uint8_t* hs, const uint8_t* wc, const uint8_t* ws, uint16_t* y,
                            float* part, int M, int K, int N, int S, hipStream_t s) {
  if constexpr (W >= MT && W * MT <= 32) {
    hipLaunchKernelGGL((k_gemv_down_mx<W, MT>), dim3(N / 16, S), dim3(W * 64), 0, s, hc, hs, wc, ws, y, part, M, K,
                       N);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <int W>
static hipError_t down_mx_w(const uint8_t* hc, const uint8_t* hs, const uint8_t* wc, const uint8_t* ws, uint16_t* y,
                            float* part, int M, int K, int N, int S, hipStream_t s) {
  switch ((M + 15) / 16) {
    case 1: return down_mx_t<W, 1>(hc, hs, wc, ws, y, part, M, K, N, S, s);
    case 2: return down_mx_t<W, 2>(hc, hs, wc, ws, y, part, M, K, N, S, s);
    case 3: return down_mx_t<W, 3>(hc, hs, wc, ws, y, part, M, K, N, S, s);
    case 4: return down_mx_t<W, 4>(hc, hs, wc, ws, y, part, M, K, N, S, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_down_mx(const uint8_t* hc, const uint8_t* hs, const uint8_t* wc, const uint8_t* ws, uint16_t* y,
                               float* part, int M, int K, int N, int W, int S, hipStream_t s) {
  if (M < 1 || M > 64 || K % 512 || N % 16 || S < 1 || S > K / 512) return hipErrorInvalidValue;
  if (W == 4) return down_mx_w<4>(hc, hs, wc, ws, y, part, M, K, N, S, s);
  if (W == 8) return down_mx_w<8>(hc, hs, wc, ws, y, part, M, K, N, S, s);
  if (W == 16) return down_mx_w<16>(hc, hs, wc, ws, y, part, M, K, N, S, s);
  return hipErrorInvalidValue;
}

// Whether the whole-column MXFP4 down GEMV takes the shape
bool gemv_down_mx_quad_supported(int M, int K, int N) { return M >= 1 && M <= 4 && K % 512 == 0 && N % 4 == 0; }

// W waves per workgroup (1, 2, 4, 8, 16; at most one per 512-value step)
hipError_t launch_gemv_down_mx_quad(const uint8_t* hc, const uint8_t* hs, const uint8_t* wc, const uint8_t* ws,
                                    const uint16_t* r_in, uint16_t* y, uint16_t* r_out, double* sq, int M, int K,
                                    int N, int W, hipStream_t s) {
  if (!gemv_down_mx_quad_supported(M, K, N) || W < 1 || W > (K >> 9) || (r_out && (!r_in || !sq)))
    return hipErrorInvalidValue;
  const dim3 grid(N / 4), block(W * 64);
#define FRT_DMQ(WV) \
  hipLaunchKernelGGL((k_gemv_down_mx_quad<WV>), grid, block, 0, s, hc, hs, wc, ws, r_in, y, r_out, sq, M, K, N)
  switch (W) {
    case 1: FRT_DMQ(1); break;
    case 2: FRT_DMQ(2); break;
    case 4: FRT_DMQ(4); break;
    case 8: FRT_DMQ(8); break;
    case 16: FRT_DMQ(16); break;
    default: return hipErrorInvalidValue;
  }
#undef FRT_DMQ
  return hipGetLastError();
}

}  // namespace frt
