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
#include "frt_normq.h"

namespace frt {

enum { GU_GEGLU = 0, GU_SWIGLU = 1, GU_GELU = 2, EPI_DOWN = 3 };

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
// nontemporal 16-byte loads (the decode gate/up and down kernels keep the
// next K block's loads in flight while a block computes); the W partial
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

// Decode gate/up that finishes the norm itself (three kernels per layer
// still, but the norm kernel before it is the short k_add_sumsq).  The
// quantised row is needed by every workgroup, but each wave only needs its
// own K range of it: wave w forms XQ[m][k] = e4m3(f32(f32(r'[m][k] * inv_m) *
// w_norm[k]) * inv_x) for its K blocks [kb0, kb1) and all M rows, with
// inv_m = f32(1 / sqrt(S_m / K + eps)) in fp64 and S_m the sum of the row's
// slice sums in slice order (the arithmetic of k_add_rmsnorm_quant), writes
// the codes to its own part of an LDS row buffer [M][K] and reads its
// activation fragments from there.  Workgroup 0 also stores them to the XQ
// slot.  Loads are issued in the order: slice sums and r' / w_norm chunks,
// then the first step's weights, so the HBM stream starts before the
// quantisation runs and only the activation loads (completed first) are
// waited for.  LDS writes and reads stay inside one wave, which the LDS
// serves in order.
// NQC: 8-element chunks per lane whose loads are issued together (2, or 3
// where a wave's range has up to 192 chunks, so that it is quantised after
// one round trip)

// The weight stream runs in steps of NB K blocks.  PIPE: two register sets
// alternate, and the loads of step i + 1 are issued before the MFMAs of step
// i, so every wave keeps a step in flight while it computes (the register
// cost of 2 NB blocks); otherwise each step's loads are issued right before
// its MFMAs.
// WIDE: the slice sums are the whole-column down GEMV's, one per four
// columns (G = K / 4, more than a lane each): the workgroup's threads load
// them as 16-byte pairs, add their pairs per row in index order, the waves'
// totals meet in LDS and are added in wave order (fp64 throughout).
// OCT (gated): the gate/up matrix in octet order (gate_row_oct / up_row_oct):
// workgroup p streams the one 16-row group holding gate and up columns
// 8p .. 8p+7, one weight fragment per K block; MFMA column j < 8 is gate
// column 8p + j and j + 8 its up column, which the epilogue pairs by a lane
// swap.  Twice the workgroups of half the bytes each.
constexpr int kNqWidePairs = 4;  // 16-byte slice-sum loads per thread: M * G <= 8 * 64 * W
template <int ACT, int W, int NB, bool PIPE, int NQC, bool WIDE = false, int NP = kNqWidePairs, bool OCT = false>
__global__ __launch_bounds__(W * 64) void k_gemv_gateup_nq(const NormQ nq, const uint8_t* __restrict__ w,
                                                           uint8_t* __restrict__ hq, int M, int K, int I,
                                                           float alpha_g, float alpha_u, float inv_h) {
  constexpr bool GATED = ACT != GU_GELU && !OCT;  // two weight streams
  static_assert(!OCT || ACT != GU_GELU, "octet order is for the gated activations");
  constexpr int NACC = GATED ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t xrow[];  // [M][K] E4M3
  __shared__ v4f red[W][NACC][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const int KB = K >> 7;
  const int kb0 = wave * KB / W, kb1 = (wave + 1) * KB / W;
  const int row = lane & 15, q = lane >> 4;
  const bool has_row = row < M;
  const uint8_t* wg = w + (size_t)(GATED ? 2 * p : 0) * KB * 2048 + lane * 16;
  const uint8_t* wu = w + (size_t)(GATED ? 2 * p + 1 : p) * KB * 2048 + lane * 16;

  // (1) activation-side loads: the row's slice sums (lane i < M*G holds
  // sum i; WIDE: this thread's pairs) and the r' / w_norm chunks of this
  // wave's K blocks
  double2 sqp[WIDE ? NP : 1];
  if (WIDE) {
    const int npairs = (M * nq.G) >> 1;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int i = (int)threadIdx.x + j * W * 64;
      sqp[j] = reinterpret_cast<const double2*>(nq.sq)[i < npairs ? i : npairs - 1];
    }
  }
  NormQWave<NQC> nqw;
  nqw.init(nq, M, K, kb0, kb1, lane);  // kb1 > kb0: W <= K / 128
  nqw.load(nq, 0, lane);
  __builtin_amdgcn_sched_barrier(0);

  // (2) the first step's weights: blocks kb0 + i0 .. + NB - 1 (indices
  // clamped to the range, so no load of a step sits behind a branch; a
  // clamped block is loaded, not used)
  const int nblk = kb1 - kb0;
  typedef uint32_t Frag[NB][8];
  Frag uA, gA, uB, gB;
  auto load_step = [&](Frag& uu, Frag& gg, int i0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int k = kb0 + (i0 + j < nblk ? i0 + j : nblk - 1);
      load_w32(wu, k, uu[j]);
      if (GATED) load_w32(wg, k, gg[j]);
    }
  };
  load_step(uA, gA, 0);
  __builtin_amdgcn_sched_barrier(0);

  // (3) 1/rms of row `lane` (lanes < M), then the codes of this wave's range
  float inv_rms;
  if (WIDE) {
    __shared__ double wsum[W][4];
    const int npairs = (M * nq.G) >> 1;
    double rs[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int i = (int)threadIdx.x + j * W * 64;
      const int m = (2 * i) / nq.G;  // a pair never straddles rows (G even)
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
    double tot = 0.0;
#pragma unroll
    for (int v = 0; v < W; ++v) tot += wsum[v][mrow & 3];
    inv_rms = (float)(1.0 / sqrt(tot / (double)K + (double)nq.eps));
  } else {
    inv_rms = nqw.inv_rms(nq, lane);
  }
  const bool store_xq = blockIdx.x == 0;
  nqw.quant(nq, 0, lane, inv_rms, xrow, store_xq);
  for (int c0 = NQC * 64; c0 < nqw.nch; c0 += NQC * 64) {
    nqw.load(nq, c0, lane);
    nqw.quant(nq, c0, lane, inv_rms, xrow, store_xq);
  }
  wave_lds_sync();

  // (4) the GEMV over this wave's K range, activations from LDS
  auto lds_x32 = [&](int kb, uint32_t o[8]) {
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (has_row) {
      const uint8_t* xp = xrow + (size_t)row * K + kb * 128 + q * 32;
      a = *reinterpret_cast<const uint4*>(xp);
      b = *reinterpret_cast<const uint4*>(xp + 16);
    }
    unpack8(a, b, o);
  };
  v4f accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
  auto mma_step = [&](Frag& uu, Frag& gg, int i0) {
    if (PIPE) {
      // the step's weights count as written here: the compiler may not
      // convert them earlier, which would wait for them (and for every load
      // issued after them) before the previous step's MFMAs
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          asm volatile("" : "+v"(uu[j][t]));
          if (GATED) asm volatile("" : "+v"(gg[j][t]));
        }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (i0 + j < nblk) {  // wave-uniform
        uint32_t x0[8];
        lds_x32(kb0 + i0 + j, x0);
        accu = mfma_f16_x4(x0, uu[j], accu);
        if (GATED) accg = mfma_f16_x4(x0, gg[j], accg);
      }
    }
  };
  if (PIPE) {
    // Both loads of an iteration are unconditional (a load behind a branch
    // makes the join wait for every load in flight); the last one or two
    // steps are peeled.  The scheduling barriers keep the compiler from
    // sinking the loads below the MFMAs of the step before them.
    int i = 0;
    for (; i + 2 * NB < nblk; i += 2 * NB) {
      load_step(uB, gB, i + NB);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(uA, gA, i);
      load_step(uA, gA, i + 2 * NB);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(uB, gB, i + NB);
    }
    if (i + NB < nblk) {
      load_step(uB, gB, i + NB);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(uA, gA, i);
      mma_step(uB, gB, i + NB);
    } else {
      mma_step(uA, gA, i);
    }
  } else {
    for (int i = 0; i < nblk; i += NB) {
      if (i != 0) load_step(uA, gA, i);
      mma_step(uA, gA, i);
    }
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
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * q + r;
    if (OCT) {
      // lane row < 8 holds gate column 8p + row, lane row + 8 its up column
      const float up = __shfl(accu[r], lane ^ 8, 64);
      if (m < M && row < 8) {
        const float h = gated_h<ACT>(accu[r] * alpha_g, up * alpha_u);
        hq[(size_t)m * I + p * 8 + row] = (uint8_t)e4m3x1(h * inv_h);
      }
    } else if (m < M) {
      const float h = gated_h<ACT>(accg[r] * alpha_g, accu[r] * alpha_u);
      hq[(size_t)m * I + p * 16 + row] = (uint8_t)e4m3x1(h * inv_h);
    }
  }
}

// Decode form of gate/up with the norm fused in front (two kernels per
// layer instead of three; batch-1 time goes to kernel boundaries).  Every
// workgroup forms y (from the previous down projection's split-K partials,
// summed in split order and dequantised, or from the Y slot), R' = bf16(R +
// y), the fp64 mean square and the E4M3 row XQ of its M <= 16 rows into LDS
// (the inputs are a few KiB, L2-resident after the first workgroup), then
// streams its 16 columns of gate/up weights exactly as k_gemv_gateup does
// with the activation fragments read from LDS.  Workgroup 0 also stores y,
// R' and XQ to their slots.  The first two K blocks of weights are requested
// before the prologue so the HBM stream starts at once.  Row layout of the
// prologue: for M == 1 the whole workgroup shares the row (chunks of 8
// elements, at most NCH per thread kept in registers); for M > 1 each wave
// takes rows wave, wave + W, ...
constexpr int kFusedXqBytes = 32768;  // LDS for the quantised rows: M * H <= this

struct FusedArgs {
  const uint16_t* r_prev;  // R[l] bf16 [M][K]
  const uint16_t* y_prev;  // Y[l] bf16 [M][K] (when y_part is null)
  const float* y_part;     // previous down projection's fp32 partials [S][M][K], or null
  int S;                   // their split count
  float a_prev;            // their dequantisation scale
  uint16_t* y_store;       // Y[l] slot, written from the partials by workgroup 0
  const uint16_t* w_norm;  // RMSNorm weight [K]
  uint16_t* r_out;         // R[l+1]
  uint8_t* xq_out;         // XQ[l]
  const uint8_t* w;        // packed gate/up weights
  uint8_t* hq;             // HQ[l]
  int M, K, I;
  float eps, inv_x, alpha_g, alpha_u, inv_h;
};

template <int ACT, int W, int NCH, int G>
__global__ __launch_bounds__(W * 64, 4) void k_gemv_gateup_fused(const FusedArgs a) {
  constexpr bool GATED = ACT != GU_GELU;
  constexpr int NACC = GATED ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t xs[kFusedXqBytes];
  __shared__ v4f red[W * NACC * 64];
  __shared__ double dred[W];
  const int M = a.M, K = a.K, I = a.I;
  const uint8_t* __restrict__ w = a.w;
  uint8_t* __restrict__ hq = a.hq;
  const float alpha_g = a.alpha_g, alpha_u = a.alpha_u, inv_h = a.inv_h, inv_x = a.inv_x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool writer = blockIdx.x == 0;
  const int KB = K >> 7;
  const int kb0 = wave * KB / W, kb1 = (wave + 1) * KB / W;
  const int P = I >> 4;
  // this workgroup's column groups: blockIdx.x + g * gridDim.x, g < G
  const int p0 = blockIdx.x;
  const uint8_t* wg0 = w + (size_t)(GATED ? 2 * p0 : 0) * KB * 2048 + lane * 16;
  const uint8_t* wu0 = w + (size_t)(GATED ? 2 * p0 + 1 : p0) * KB * 2048 + lane * 16;

  // request the first two weight blocks of the first group before the prologue
  uint32_t u0[8] = {}, u1[8] = {}, g0[8] = {}, g1[8] = {};
  if (kb0 < kb1) {
    load_w32(wu0, kb0, u0);
    if (GATED) load_w32(wg0, kb0, g0);
  }
  if (kb0 + 1 < kb1) {
    load_w32(wu0, kb0 + 1, u1);
    if (GATED) load_w32(wg0, kb0 + 1, g1);
  }

  // ---- prologue: R' = bf16(R + Y), RMSNorm, E4M3 -> xs (once per workgroup) ----
  const int nchunk = K >> 3;
  const int group_threads = (M == 1) ? W * 64 : 64;
  const int t_in = (M == 1) ? tid : lane;
  for (int m = (M == 1) ? 0 : wave; m < M; m += (M == 1) ? 1 : W) {
    const size_t base = (size_t)m * K;
    uint4 rn[NCH], wn[NCH];
    double sq = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = t_in + c * group_threads;
      rn[c] = make_uint4(0, 0, 0, 0);
      wn[c] = rn[c];
      if (ch < nchunk) {
        const uint4 rv = *reinterpret_cast<const uint4*>(a.r_prev + base + (size_t)ch * 8);
        uint4 yv;
        if (a.y_part) {
          yv = y_from_partials(a.y_part, (size_t)M * K, base + (size_t)ch * 8, a.S, a.a_prev);
          if (writer) *reinterpret_cast<uint4*>(a.y_store + base + (size_t)ch * 8) = yv;
        } else {
          yv = *reinterpret_cast<const uint4*>(a.y_prev + base + (size_t)ch * 8);
        }
        wn[c] = *reinterpret_cast<const uint4*>(a.w_norm + (size_t)ch * 8);
        const uint32_t rr[4] = {rv.x, rv.y, rv.z, rv.w}, yy[4] = {yv.x, yv.y, yv.z, yv.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[j] = pack_bf16x2(bf16_lo(rr[j]) + bf16_lo(yy[j]), bf16_hi(rr[j]) + bf16_hi(yy[j]));
          const double dlo = (double)bf16_lo(o[j]), dhi = (double)bf16_hi(o[j]);
          sq += dlo * dlo;
          sq += dhi * dhi;
        }
        rn[c] = make_uint4(o[0], o[1], o[2], o[3]);
        if (writer) *reinterpret_cast<uint4*>(a.r_out + base + (size_t)ch * 8) = rn[c];
      }
    }
    sq = wave_sum_f64(sq);
    if (M == 1) {
      if (lane == 0) dred[wave] = sq;
      __syncthreads();
      sq = 0.0;
#pragma unroll
      for (int v = 0; v < W; ++v) sq += dred[v];
    }
    const float inv_rms = (float)(1.0 / sqrt(sq / (double)K + (double)a.eps));
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = t_in + c * group_threads;
      if (ch < nchunk) {
        const uint32_t ww[4] = {wn[c].x, wn[c].y, wn[c].z, wn[c].w};
        const uint32_t rr[4] = {rn[c].x, rn[c].y, rn[c].z, rn[c].w};
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = (bf16_lo(rr[j]) * inv_rms) * bf16_lo(ww[j]);
          x[2 * j + 1] = (bf16_hi(rr[j]) * inv_rms) * bf16_hi(ww[j]);
        }
        uint2 q;
        q.x = e4m3x4(x[0] * inv_x, x[1] * inv_x, x[2] * inv_x, x[3] * inv_x);
        q.y = e4m3x4(x[4] * inv_x, x[5] * inv_x, x[6] * inv_x, x[7] * inv_x);
        *reinterpret_cast<uint2*>(xs + base + (size_t)ch * 8) = q;
        if (writer) *reinterpret_cast<uint2*>(a.xq_out + base + (size_t)ch * 8) = q;
      }
    }
  }
  __syncthreads();

  const int row = lane & 15, q = lane >> 4;
  const bool has_row = row < M;
  const uint8_t* xr = xs + (has_row ? row : 0) * K + q * 32;
#pragma unroll 1
  for (int gi = 0; gi < G; ++gi) {
    const int p = p0 + gi * (int)gridDim.x;
    if (p >= P) break;  // uniform across the workgroup
    const uint8_t* wg = w + (size_t)(GATED ? 2 * p : 0) * KB * 2048 + lane * 16;
    const uint8_t* wu = w + (size_t)(GATED ? 2 * p + 1 : p) * KB * 2048 + lane * 16;
    v4f accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    int kb = kb0;
    if (gi > 0) {
      if (kb0 < kb1) {
        load_w32(wu, kb0, u0);
        if (GATED) load_w32(wg, kb0, g0);
      }
      if (kb0 + 1 < kb1) {
        load_w32(wu, kb0 + 1, u1);
        if (GATED) load_w32(wg, kb0 + 1, g1);
      }
    }
    if (kb + 1 < kb1) {
      uint32_t x0[8], x1[8];
      load_x32(xr, has_row, kb, x0);
      load_x32(xr, has_row, kb + 1, x1);
      accu = mfma_f16_x4(x0, u0, accu);
      if (GATED) accg = mfma_f16_x4(x0, g0, accg);
      accu = mfma_f16_x4(x1, u1, accu);
      if (GATED) accg = mfma_f16_x4(x1, g1, accg);
      kb += 2;
    } else if (kb < kb1) {
      uint32_t x0[8];
      load_x32(xr, has_row, kb, x0);
      accu = mfma_f16_x4(x0, u0, accu);
      if (GATED) accg = mfma_f16_x4(x0, g0, accg);
      kb += 1;
    }
    for (; kb + 1 < kb1; kb += 2) {
      uint32_t x0[8], x1[8], a0[8], a1[8], b0[8], b1[8];
      load_w32(wu, kb, a0);
      load_w32(wu, kb + 1, a1);
      if (GATED) {
        load_w32(wg, kb, b0);
        load_w32(wg, kb + 1, b1);
      }
      load_x32(xr, has_row, kb, x0);
      load_x32(xr, has_row, kb + 1, x1);
      accu = mfma_f16_x4(x0, a0, accu);
      if (GATED) accg = mfma_f16_x4(x0, b0, accg);
      accu = mfma_f16_x4(x1, a1, accu);
      if (GATED) accg = mfma_f16_x4(x1, b1, accg);
    }
    if (kb < kb1) {
      uint32_t x0[8], a0[8], b0[8];
      load_w32(wu, kb, a0);
      if (GATED) load_w32(wg, kb, b0);
      load_x32(xr, has_row, kb, x0);
      accu = mfma_f16_x4(x0, a0, accu);
      if (GATED) accg = mfma_f16_x4(x0, b0, accg);
    }
    red[(wave * NACC + 0) * 64 + lane] = accu;
    if (GATED) red[(wave * NACC + NACC - 1) * 64 + lane] = accg;
    __syncthreads();
    if (wave == 0) {
      accu = red[0 * 64 + lane];
      if (GATED) accg = red[(NACC - 1) * 64 + lane];
#pragma unroll
      for (int v = 1; v < W; ++v) {
        accu += red[(v * NACC + 0) * 64 + lane];
        if (GATED) accg += red[(v * NACC + NACC - 1) * 64 + lane];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * q + r;
        if (m < M) {
          const float h = gated_h<ACT>(accg[r] * alpha_g, accu[r] * alpha_u);
          hq[(size_t)m * I + p * 16 + row] = (uint8_t)e4m3x1(h * inv_h);
        }
      }
    }
    __syncthreads();  // red is reused by the next group
  }
}

// Down GEMV.  COLS = 16: a workgroup owns one 16-row group of Wd; COLS = 8:
// it owns half a group (lanes of the other half load nothing and their
// accumulator columns are discarded), doubling the workgroups so that every
// CU gets the same share when the group count is small (H/16 = 320 for
// H = 5120 on 256 CUs).  Half-group loads still read whole 128-byte lines.
template <int W, bool FP8, int COLS, int NB, bool PIPE>
__global__ __launch_bounds__(W * 64) void k_gemv_down(const uint8_t* __restrict__ hq,
                                                      const uint8_t* __restrict__ w,
                                                      uint16_t* __restrict__ y, float* __restrict__ part,
                                                      int M, int K, int N, float alpha_d, int order) {
  __shared__ v4f red[W][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // order 1: consecutive workgroups take consecutive K splits of one column
  // group (one group's bytes are read by neighbouring workgroups)
  const int S = gridDim.y;
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int bx = order ? lin / S : (int)blockIdx.x, sp = order ? lin % S : (int)blockIdx.y;
  const int p = (COLS == 16) ? bx : (bx >> 1);
  const int half = (COLS == 16) ? 0 : (bx & 1);
  const int KB = K >> 7;
  // K split sp of S, then this wave's share of it
  const int ks0 = sp * KB / S, ks1 = (sp + 1) * KB / S;
  const int kb0 = ks0 + wave * (ks1 - ks0) / W, kb1 = ks0 + (wave + 1) * (ks1 - ks0) / W;
  const int row = lane & 15, q = lane >> 4;
  const bool has_row = row < M;
  const bool my_col = (COLS == 16) || ((row >> 3) == half);
  const uint8_t* wp = w + (size_t)p * KB * 2048 + lane * 16;
  const uint8_t* xr = hq + (size_t)(has_row ? row : 0) * K + q * 32;

  // steps of NB K blocks, each step's weight and activation loads issued
  // together (block indices clamped to the range: a clamped block is loaded,
  // not used); PIPE as in k_gemv_gateup_nq (two register sets, the next
  // step's loads in flight while the current one computes).  Blocks
  // alternate between two accumulators by their index's parity.
  const int nblk = kb1 - kb0;
  typedef uint32_t Frag[NB][8];
  Frag xA, wA, xB, wB;
  auto load_step = [&](Frag& xs, Frag& ws, int i0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int k = kb0 + (i0 + j < nblk ? i0 + j : nblk - 1);
      if (my_col) {
        load_w32(wp, k, ws[j]);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) ws[j][t] = 0u;
      }
    }
    // every lane loads its activations (a load behind a lane branch would
    // make the join wait for all loads in flight): lanes of rows past M read
    // row 0's bytes, which reach only output rows past M, never stored
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int k = kb0 + (i0 + j < nblk ? i0 + j : nblk - 1);
      unpack8(ld16(xr + k * 128), ld16(xr + k * 128 + 16), xs[j]);
    }
  };
  v4f acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  auto mma_step = [&](Frag& xs, Frag& ws, int i0) {
    if (PIPE) {
      // the step's operands count as written here (as in k_gemv_gateup_nq)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          asm volatile("" : "+v"(xs[j][t]));
          asm volatile("" : "+v"(ws[j][t]));
        }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (i0 + j < nblk) {  // wave-uniform
        if ((i0 + j) & 1) acc1 = mfma_step<FP8>(xs[j], ws[j], acc1);
        else acc0 = mfma_step<FP8>(xs[j], ws[j], acc0);
      }
    }
  };
  if (nblk > 0) load_step(xA, wA, 0);
  if (PIPE && nblk > 0) {
    // (loop shape as in k_gemv_gateup_nq)
    int i = 0;
    for (; i + 2 * NB < nblk; i += 2 * NB) {
      load_step(xB, wB, i + NB);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(xA, wA, i);
      load_step(xA, wA, i + 2 * NB);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(xB, wB, i + NB);
    }
    if (i + NB < nblk) {
      load_step(xB, wB, i + NB);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(xA, wA, i);
      mma_step(xB, wB, i + NB);
    } else {
      mma_step(xA, wA, i);
    }
  } else if (!PIPE) {
    for (int i = 0; i < nblk; i += NB) {
      if (i != 0) load_step(xA, wA, i);
      mma_step(xA, wA, i);
    }
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
  if (!my_col) return;
  // one split: bf16 Y; several: fp32 partial [split][M][N] (the consumer adds
  // the splits in split order and dequantises)
  float* ps = part + (size_t)sp * M * N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * q + r;
    if (m < M) {
      if (S == 1)
        y[(size_t)m * N + p * 16 + row] = (uint16_t)f32_to_bf16(acc[r] * alpha_d);
      else
        ps[(size_t)m * N + p * 16 + row] = acc[r];
    }
  }
}

// Whole-column decode down GEMV (M <= 4), down matrix in the column-quad
// layout (quad_offset): one workgroup per four output columns reads those
// columns over all of K, so it owns their sums and no split-K partials or
// norm kernel follow it.  K is cut into 64-element stripes dealt to four
// parts in turn (part p: stripes 4t + p), and each MFMA takes the four
// parts side by side: operand row 4 p' + m' is activation row m' over part
// p', operand column 4 p + c is weight column c over part p, so the
// products with p' == p are the parts' partial dot products and the others
// are discarded (lanes 20 p + c hold part p of column c, row m in element
// m).  The epilogue forms, for its columns,
//   Y = bf16(alpha_d * sum),  R' = bf16(R + Y)  (R' and Z alike: r_out),
//   and the fp64 sum of R'^2 over the four columns, slice c4 of row m of
//   sq [M][N / 4] (the next layer's split norm reads these slices);
// r_out == nullptr stores Y only.  Step t covers elements 256 t .. 256 t +
// 255 (1 KiB of weights, 16 bytes per lane, and the 256 activation bytes
// of each row read as one contiguous run), two MFMAs each,
// NB steps per load stage, stages pipelined over two register sets as in
// k_gemv_gateup_nq; rows m' >= M read row 0, whose products reach only
// discarded rows.
template <int W, int NB, bool PIPE>
__global__ __launch_bounds__(W * 64) void k_gemv_down_quad(const uint8_t* __restrict__ hq,
                                                           const uint8_t* __restrict__ w,
                                                           const uint16_t* __restrict__ r_in,
                                                           uint16_t* __restrict__ y, uint16_t* __restrict__ r_out,
                                                           double* __restrict__ sq, int M, int K, int N,
                                                           float alpha_d) {
  __shared__ v4f red[W][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c4 = blockIdx.x;
  const int T = K >> 8;
  const int t0 = wave * T / W, t1 = (wave + 1) * T / W;
  const int part = (lane & 15) >> 2, mr = lane & 3;
  const uint8_t* wp = w + (size_t)c4 * T * 1024 + lane * 16;
  const uint8_t* xr = hq + (size_t)(mr < M ? mr : 0) * K + part * 64 + (lane >> 4) * 16;
  const int nstep = t1 - t0;
  uint4 wA[NB], xA[NB], wB[NB], xB[NB];
  // steps i0 .. i0 + NB - 1 (indices clamped to the range: a clamped step is
  // loaded, not used)
  auto load_step = [&](uint4 (&ww)[NB], uint4 (&xx)[NB], int i0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = t0 + (i0 + j < nstep ? i0 + j : nstep - 1);
      ww[j] = ld16_nt(wp + (size_t)t * 1024);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = t0 + (i0 + j < nstep ? i0 + j : nstep - 1);
      xx[j] = ld16(xr + t * 256);
    }
  };
  v4f acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  auto mma_step = [&](uint4 (&ww)[NB], uint4 (&xx)[NB], int i0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (PIPE) {
        asm volatile("" : "+v"(ww[j].x), "+v"(ww[j].y), "+v"(ww[j].z), "+v"(ww[j].w));
        asm volatile("" : "+v"(xx[j].x), "+v"(xx[j].y), "+v"(xx[j].z), "+v"(xx[j].w));
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (i0 + j < nstep) {  // wave-uniform
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(xx[j].x, xx[j].y), e4m3x8_to_f16(ww[j].x, ww[j].y),
                                                      acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(xx[j].z, xx[j].w), e4m3x8_to_f16(ww[j].z, ww[j].w),
                                                      acc1, 0, 0, 0);
      }
    }
  };
  // wave 0 (which runs the epilogue) requests its columns' R values right
  // after its first weights, so that they arrive during the stream (rows
  // clamped to M - 1; any valid address when R is not needed): 15.92-15.98
  // against 16.00-16.05 us loading them in the epilogue, and 18.1 when every
  // wave requested them ahead of its weights
  uint16_t rv[4] = {0, 0, 0, 0};
  if (nstep > 0) {
    load_step(wA, xA, 0);
    if (wave == 0) {
      const uint16_t* rp = r_in ? r_in : y;
#pragma unroll
      for (int m = 0; m < 4; ++m) rv[m] = rp[(size_t)(m < M ? m : M - 1) * N + (size_t)c4 * 4 + (lane & 3)];
    }
    if (PIPE) {
      int i = 0;
      for (; i + 2 * NB < nstep; i += 2 * NB) {
        load_step(wB, xB, i + NB);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(wA, xA, i);
        load_step(wA, xA, i + 2 * NB);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(wB, xB, i + NB);
      }
      if (i + NB < nstep) {
        load_step(wB, xB, i + NB);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(wA, xA, i);
        mma_step(wB, xB, i + NB);
      } else {
        mma_step(wA, xA, i);
      }
    } else {
      for (int i = 0; i < nstep; i += NB) {
        if (i != 0) load_step(wA, xA, i);
        mma_step(wA, xA, i);
      }
    }
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
    const uint32_t yb = f32_to_bf16(tot[m] * alpha_d);
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

// ===========================================================================
// GEMM path (M > 16)
// ===========================================================================
//
// Workgroup tile BM rows x BN packed columns, K step 128, WGM x WGN waves of
// (BM/WGM) x (BN/WGN).  Both operand tiles are staged through LDS in
// fragment order (16-row blocks of 2 KiB, lane l's 16-byte halves at l*16 and
// 1024 + l*16: every ds_read_b128 reads 1 KiB contiguously), double
// buffered: the next step's global loads are in flight while the current
// step computes.  The down GEMM may split K over gridDim.z; each split then
// writes its fp32 partial tile and the consumer (the next layer's norm
// kernel, or the final residual add) sums the splits in split order, so no
// workgroup waits for another and no device-scope fence is needed.

template <int BM, int BN, int NT>
struct Stage {
  static constexpr int AP = BM * 8 / NT;  // 16-byte pieces per thread
  static constexpr int BP = BN * 8 / NT;
  uint4 a[AP], b[BP];
};

template <int BM, int BN, int NT>
__device__ __forceinline__ void stage_load(Stage<BM, BN, NT>& st, const uint8_t* __restrict__ act,
                                           int M, int K, int m0, const uint8_t* __restrict__ wt,
                                           int g0, int KB, int kb) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < Stage<BM, BN, NT>::AP; ++j) {
    const int c = tid + NT * j;  // piece: row c / 8, 16-byte column c % 8
    const int m = m0 + (c >> 3);
    st.a[j] = make_uint4(0, 0, 0, 0);
    if (m < M) st.a[j] = ld16(act + (size_t)m * K + kb * 128 + (c & 7) * 16);
  }
#pragma unroll
  for (int j = 0; j < Stage<BM, BN, NT>::BP; ++j) {
    const int c = tid + NT * j;  // piece: group c / 128, byte (c % 128) * 16
    st.b[j] = ld16(wt + ((size_t)(g0 + (c >> 7)) * KB + kb) * 2048 + (c & 127) * 16);
  }
}

// Both operands go to LDS as E4M3 bytes in the 2 KiB fragment order of the
// packed weights (16-row block mg: half h of lane ln at mg*2048 + h*1024 +
// ln*16, lane ln = row + 16 * (k-chunk / 2)), so one 1 KiB contiguous
// ds_read_b128 per wave serves each half fragment.
template <int BM, int BN, int NT>
__device__ __forceinline__ void stage_store(const Stage<BM, BN, NT>& st, uint8_t* lds_a, uint8_t* lds_b) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < Stage<BM, BN, NT>::AP; ++j) {
    const int c = tid + NT * j;
    const int r = c >> 3, kc = c & 7;
    *reinterpret_cast<uint4*>(lds_a + (r >> 4) * 2048 + (kc & 1) * 1024 + ((r & 15) + 16 * (kc >> 1)) * 16) =
        st.a[j];
  }
#pragma unroll
  for (int j = 0; j < Stage<BM, BN, NT>::BP; ++j) {
    const int c = tid + NT * j;
    *reinterpret_cast<uint4*>(lds_b + c * 16) = st.b[j];
  }
}

// EPI: GU_GEGLU / GU_SWIGLU / GU_GELU for gate/up (E4M3 output), EPI_DOWN for
// down (bf16 output or fp32 split partials).  FP8: the products run on the
// FP8 matrix cores (one 16x16x128 instruction per tile and K step), else on
// the f16 matrix cores from exactly converted operands (four 16x16x32 steps).
template <int EPI, bool FP8, int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm(const uint8_t* __restrict__ act,
                                                         const uint8_t* __restrict__ wt,
                                                         void* __restrict__ out, float* __restrict__ part,
                                                         int M, int K, int Npk, int S, float alpha_a,
                                                         float alpha_b, float inv_out) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int MTM = BM / WGM / 16, MTN = BN / WGN / 16;  // 16x16 tiles per wave
  constexpr bool DOWN = EPI == EPI_DOWN;
  constexpr bool GATED = EPI == GU_GEGLU || EPI == GU_SWIGLU;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static_assert(!GATED || (MTN % 2) == 0, "gated tiles hold whole gate/up pairs");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][A_BYTES + B_BYTES];

  const int tn = blockIdx.x, tm = blockIdx.y, s = blockIdx.z;
  const int m0 = tm * BM, g0 = tn * (BN / 16);
  const int KB = K >> 7;
  const int kb0 = s * KB / S, kb1 = (s + 1) * KB / S;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / WGN, wn = wave % WGN;

  v4f acc[MTM][MTN];
#pragma unroll
  for (int i = 0; i < MTM; ++i)
#pragma unroll
    for (int j = 0; j < MTN; ++j) acc[i][j] = v4f{0, 0, 0, 0};

  Stage<BM, BN, NT> st;
  stage_load<BM, BN, NT>(st, act, M, K, m0, wt, g0, KB, kb0);
  stage_store<BM, BN, NT>(st, lds[0], lds[0] + A_BYTES);
  __syncthreads();
  int cur = 0;
  for (int kb = kb0; kb < kb1; ++kb) {
    const bool more = kb + 1 < kb1;
    if (more) stage_load<BM, BN, NT>(st, act, M, K, m0, wt, g0, KB, kb + 1);
    const uint8_t* la = lds[cur] + (wm * MTM) * 2048 + lane * 16;
    const uint8_t* lb = lds[cur] + A_BYTES + (wn * MTN) * 2048 + lane * 16;
    if (FP8) {
      v8i af[MTM], bf[MTN];
#pragma unroll
      for (int i = 0; i < MTM; ++i)
        af[i] = as_v8i(*reinterpret_cast<const uint4*>(la + i * 2048),
                       *reinterpret_cast<const uint4*>(la + i * 2048 + 1024));
#pragma unroll
      for (int j = 0; j < MTN; ++j)
        bf[j] = as_v8i(*reinterpret_cast<const uint4*>(lb + j * 2048),
                       *reinterpret_cast<const uint4*>(lb + j * 2048 + 1024));
#pragma unroll
      for (int i = 0; i < MTM; ++i)
#pragma unroll
        for (int j = 0; j < MTN; ++j) acc[i][j] = mfma_fp8(af[i], bf[j], acc[i][j]);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // 16-byte half of each lane's 32 bytes
        uint4 ar[MTM], br[MTN];
#pragma unroll
        for (int i = 0; i < MTM; ++i) ar[i] = *reinterpret_cast<const uint4*>(la + i * 2048 + h * 1024);
#pragma unroll
        for (int j = 0; j < MTN; ++j) br[j] = *reinterpret_cast<const uint4*>(lb + j * 2048 + h * 1024);
#pragma unroll
        for (int t = 0; t < 2; ++t) {  // 8-value k-substeps
          v8h ah[MTM], bh[MTN];
#pragma unroll
          for (int i = 0; i < MTM; ++i) ah[i] = t ? e4m3x8_to_f16(ar[i].z, ar[i].w) : e4m3x8_to_f16(ar[i].x, ar[i].y);
#pragma unroll
          for (int j = 0; j < MTN; ++j) bh[j] = t ? e4m3x8_to_f16(br[j].z, br[j].w) : e4m3x8_to_f16(br[j].x, br[j].y);
#pragma unroll
          for (int i = 0; i < MTM; ++i)
#pragma unroll
            for (int j = 0; j < MTN; ++j) acc[i][j] = mfma_f16(ah[i], bh[j], acc[i][j]);
        }
      }
    }
    if (more) stage_store<BM, BN, NT>(st, lds[cur ^ 1], lds[cur ^ 1] + A_BYTES);
    __syncthreads();
    cur ^= 1;
  }

  const int q = lane >> 4, col = lane & 15;
  const int gw = g0 + wn * MTN;  // first packed group of this wave
  if (!DOWN) {
    uint8_t* hq = reinterpret_cast<uint8_t*>(out);
    const int I = GATED ? Npk / 2 : Npk;
#pragma unroll
    for (int i = 0; i < MTM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (wm * MTM + i) * 16 + 4 * q + r;
        if (m >= M) continue;
        if (GATED) {
#pragma unroll
          for (int jp = 0; jp < MTN / 2; ++jp) {
            const int pair = gw / 2 + jp;
            const float h = gated_h<EPI>(acc[i][2 * jp][r] * alpha_a, acc[i][2 * jp + 1][r] * alpha_b);
            hq[(size_t)m * I + pair * 16 + col] = (uint8_t)e4m3x1(h * inv_out);
          }
        } else {
#pragma unroll
          for (int j = 0; j < MTN; ++j) {
            const float h = gated_h<EPI>(0.0f, acc[i][j][r] * alpha_b);
            hq[(size_t)m * I + (gw + j) * 16 + col] = (uint8_t)e4m3x1(h * inv_out);
          }
        }
      }
    }
    return;
  }
  // down: one split writes bf16 Y; several write fp32 partials for the consumer
  const int N = Npk;
  uint16_t* y = reinterpret_cast<uint16_t*>(out);
  float* ps = part + (size_t)s * M * N;
#pragma unroll
  for (int i = 0; i < MTM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + (wm * MTM + i) * 16 + 4 * q + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < MTN; ++j) {
        const size_t o = (size_t)m * N + (gw + j) * 16 + col;
        if (S == 1)
          y[o] = (uint16_t)f32_to_bf16(acc[i][j][r] * alpha_a);
        else
          ps[o] = acc[i][j][r];
      }
    }
}

// Workgroup tile configurations (index): {BM, BN, WGM, WGN}
//   0: 128 x 128, 2 x 2 waves     1: 128 x 256, 2 x 2     2: 256 x 128, 2 x 2
//   3: 128 x 256, 2 x 4           4: 128 x 256, 1 x 4     5:  64 x 256, 1 x 4
//   6: 256 x 256, 2 x 2 (FP8 only: the f16 form runs out of registers)
constexpr int kGemmConfigs = 7;
__host__ __device__ constexpr int cfg_bm(int c) { return c == 2 || c == 6 ? 256 : (c == 5 ? 64 : 128); }
__host__ __device__ constexpr int cfg_bn(int c) { return c == 0 || c == 2 ? 128 : 256; }
__host__ __device__ constexpr int cfg_wgm(int c) { return c == 4 || c == 5 ? 1 : 2; }
__host__ __device__ constexpr int cfg_wgn(int c) { return c >= 3 && c <= 5 ? 4 : 2; }

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

// ===========================================================================
// Multi-tile GEMV (16 < M <= 64)
// ===========================================================================
//
// The same weight stream as the GEMV above (one workgroup per 16 output
// columns, waves splitting K, partials meeting in LDS in wave order), with
// the M rows taken as MT = ceil(M / 16) activation tiles of 16: each weight
// fragment is loaded and converted to f16 once and multiplied into all MT
// tiles.  At these M the weights are still read exactly once per launch (a
// 128-row GEMM tile would waste most of its rows and leave most CUs idle);
// the activation rows (M x K bytes) come from L2.  After the reduction,
// wave t finishes tile t (t < MT).

// lane's 32 bytes of K block kb of weight rows as four f16 operands
__device__ __forceinline__ void cvt_w32(const uint32_t w[8], v8h o[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = e4m3x8_to_f16(w[2 * t], w[2 * t + 1]);
}

template <int ACT, int W, int MT>
__global__ __launch_bounds__(W * 64) void k_gemv_gateup_mt(const uint8_t* __restrict__ xq,
                                                           const uint8_t* __restrict__ w,
                                                           uint8_t* __restrict__ hq, int M, int K,
                                                           int I, float alpha_g, float alpha_u,
                                                           float inv_h) {
  constexpr bool GATED = ACT != GU_GELU;
  constexpr int NACC = GATED ? 2 : 1;
  static_assert(W >= MT, "one wave per tile finishes the epilogue");
  __shared__ v4f red[W][MT][NACC][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = blockIdx.x;  // column group
  const int KB = K >> 7;
  const int kb0 = wave * KB / W, kb1 = (wave + 1) * KB / W;
  const int row = lane & 15, q = lane >> 4;
  const uint8_t* wg = w + (size_t)(GATED ? 2 * p : 0) * KB * 2048 + lane * 16;
  const uint8_t* wu = w + (size_t)(GATED ? 2 * p + 1 : p) * KB * 2048 + lane * 16;
  const uint8_t* xr[MT];
  bool has[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    has[t] = 16 * t + row < M;
    xr[t] = xq + (size_t)(has[t] ? 16 * t + row : 0) * K + q * 32;
  }

  v4f accg[MT], accu[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) accg[t] = accu[t] = v4f{0, 0, 0, 0};

  for (int kb = kb0; kb < kb1; kb += 2) {
    const bool two = kb + 1 < kb1;
    uint32_t u0[8], u1[8], g0[8], g1[8], x0[MT][8], x1[MT][8];
    load_w32(wu, kb, u0);
    if (GATED) load_w32(wg, kb, g0);
    if (two) {
      load_w32(wu, kb + 1, u1);
      if (GATED) load_w32(wg, kb + 1, g1);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      load_x32(xr[t], has[t], kb, x0[t]);
      load_x32(xr[t], has[t] && two, kb + (two ? 1 : 0), x1[t]);
    }
    v8h uh[4], gh[4];
    cvt_w32(u0, uh);
    if (GATED) cvt_w32(g0, gh);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const v8h xh = e4m3x8_to_f16(x0[t][2 * s4], x0[t][2 * s4 + 1]);
        accu[t] = mfma_f16(xh, uh[s4], accu[t]);
        if (GATED) accg[t] = mfma_f16(xh, gh[s4], accg[t]);
      }
    if (two) {
      cvt_w32(u1, uh);
      if (GATED) cvt_w32(g1, gh);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const v8h xh = e4m3x8_to_f16(x1[t][2 * s4], x1[t][2 * s4 + 1]);
          accu[t] = mfma_f16(xh, uh[s4], accu[t]);
          if (GATED) accg[t] = mfma_f16(xh, gh[s4], accg[t]);
        }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    red[wave][t][0][lane] = accu[t];
    if (GATED) red[wave][t][NACC - 1][lane] = accg[t];
  }
  __syncthreads();
  if (wave >= MT) return;
  const int t = wave;
  v4f au = red[0][t][0][lane], ag = red[0][t][NACC - 1][lane];
#pragma unroll
  for (int v = 1; v < W; ++v) {
    au += red[v][t][0][lane];
    if (GATED) ag += red[v][t][NACC - 1][lane];
  }
  // lane holds rows m = 16t + 4q + r of column 16p + row
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 16 * t + 4 * q + r;
    if (m < M) {
      const float h = gated_h<ACT>(ag[r] * alpha_g, au[r] * alpha_u);
      hq[(size_t)m * I + p * 16 + row] = (uint8_t)e4m3x1(h * inv_h);
    }
  }
}

// Down projection, multi-tile form: K split over gridDim.y workgroups per 16
// output columns (fp32 partials [split][M][N] when > 1, as k_gemv_down).
template <int W, bool FP8, int MT>
__global__ __launch_bounds__(W * 64) void k_gemv_down_mt(const uint8_t* __restrict__ hq,
                                                         const uint8_t* __restrict__ w,
                                                         uint16_t* __restrict__ y, float* __restrict__ part,
                                                         int M, int K, int N, float alpha_d) {
  static_assert(W >= MT, "one wave per tile finishes the epilogue");
  __shared__ v4f red[W][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = blockIdx.x;
  const int KB = K >> 7;
  const int S = gridDim.y, sp = blockIdx.y;
  const int ks0 = sp * KB / S, ks1 = (sp + 1) * KB / S;
  const int kb0 = ks0 + wave * (ks1 - ks0) / W, kb1 = ks0 + (wave + 1) * (ks1 - ks0) / W;
  const int row = lane & 15, q = lane >> 4;
  const uint8_t* wp = w + (size_t)p * KB * 2048 + lane * 16;
  const uint8_t* xr[MT];
  bool has[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    has[t] = 16 * t + row < M;
    xr[t] = hq + (size_t)(has[t] ? 16 * t + row : 0) * K + q * 32;
  }
  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4f{0, 0, 0, 0};

  for (int kb = kb0; kb < kb1; kb += 2) {
    const bool two = kb + 1 < kb1;
    uint32_t w0[8], w1[8], x0[MT][8], x1[MT][8];
    load_w32(wp, kb, w0);
    if (two) load_w32(wp, kb + 1, w1);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      load_x32(xr[t], has[t], kb, x0[t]);
      load_x32(xr[t], has[t] && two, kb + (two ? 1 : 0), x1[t]);
    }
    if (FP8) {
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mfma_step<true>(x0[t], w0, acc[t]);
      if (two) {
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = mfma_step<true>(x1[t], w1, acc[t]);
      }
    } else {
      v8h wh[4];
      cvt_w32(w0, wh);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          acc[t] = mfma_f16(e4m3x8_to_f16(x0[t][2 * s4], x0[t][2 * s4 + 1]), wh[s4], acc[t]);
      if (two) {
        cvt_w32(w1, wh);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            acc[t] = mfma_f16(e4m3x8_to_f16(x1[t][2 * s4], x1[t][2 * s4 + 1]), wh[s4], acc[t]);
      }
    }
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
        y[(size_t)m * N + p * 16 + row] = (uint16_t)f32_to_bf16(a[r] * alpha_d);
      else
        ps[(size_t)m * N + p * 16 + row] = a[r];
    }
  }
}

// K blocks per load step of the decode GEMVs and whether the steps are
// pipelined (FRT_GEMV_NB_GATEUP / FRT_GEMV_NB_DOWN: 1 or 2;
// FRT_GEMV_PIPE_GATEUP / FRT_GEMV_PIPE_DOWN: 0 or 1).
static int gemv_nb(const char* env, int dflt) {
  const char* e = getenv(env);
  const int v = (e && *e) ? atoi(e) : dflt;
  return v >= 2 ? 2 : 1;
}
static bool gemv_pipe(const char* env, bool dflt) {
  const char* e = getenv(env);
  return (e && *e) ? atoi(e) != 0 : dflt;
}

template <int W, int NB, bool PIPE, int NQC, bool WIDE, int NP = kNqWidePairs, bool OCT = false>
static void gemv_gateup_nq_wnpc(int act, const NormQ& nq, const uint8_t* w, uint8_t* hq, int M, int K, int I,
                                float a_g, float a_u, float inv_h, hipStream_t s) {
  dim3 grid(OCT ? I / 8 : I / 16), block(W * 64);
  const size_t lds = (size_t)M * K;
  if (act == GU_GEGLU) {
    hipLaunchKernelGGL((k_gemv_gateup_nq<GU_GEGLU, W, NB, PIPE, NQC, WIDE, NP, OCT>), grid, block, lds, s, nq, w, hq,
                       M, K, I, a_g, a_u, inv_h);
  } else if (act == GU_SWIGLU) {
    hipLaunchKernelGGL((k_gemv_gateup_nq<GU_SWIGLU, W, NB, PIPE, NQC, WIDE, NP, OCT>), grid, block, lds, s, nq, w,
                       hq, M, K, I, a_g, a_u, inv_h);
  } else {
    if constexpr (!OCT)
      hipLaunchKernelGGL((k_gemv_gateup_nq<GU_GELU, W, NB, PIPE, NQC, WIDE, NP>), grid, block, lds, s, nq, w, hq, M,
                         K, I, a_g, a_u, inv_h);
  }
}

template <int W, int NB, bool PIPE, bool WIDE = false, bool OCT = false>
static void gemv_gateup_nq_wnp(int act, const NormQ& nq, const uint8_t* w, uint8_t* hq, int M, int K, int I,
                               float a_g, float a_u, float inv_h, hipStream_t s) {
  // chunks of the largest wave range: M x ceil(K blocks / W) x 16
  const int chunks = M * (((K >> 7) + W - 1) / W) * 16;
  // WIDE: two slice-sum pairs per thread where they cover the rows, else four
  if constexpr (WIDE) {
    const bool np2 = (M * nq.G) / 2 <= 2 * W * 64;
    if (chunks > 128 && chunks <= 192) {
      if (np2) gemv_gateup_nq_wnpc<W, NB, PIPE, 3, true, 2, OCT>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
      else gemv_gateup_nq_wnpc<W, NB, PIPE, 3, true, kNqWidePairs, OCT>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
    } else {
      if (np2) gemv_gateup_nq_wnpc<W, NB, PIPE, 2, true, 2, OCT>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
      else gemv_gateup_nq_wnpc<W, NB, PIPE, 2, true, kNqWidePairs, OCT>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
    }
  } else {
    if (chunks > 128 && chunks <= 192)
      gemv_gateup_nq_wnpc<W, NB, PIPE, 3, false, kNqWidePairs, OCT>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
    else
      gemv_gateup_nq_wnpc<W, NB, PIPE, 2, false, kNqWidePairs, OCT>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
  }
}

template <int W>
static void gemv_gateup_nq_w(int act, const NormQ& nq, const uint8_t* w, uint8_t* hq, int M, int K, int I,
                             float a_g, float a_u, float inv_h, hipStream_t s, bool oct) {
  if (oct) {
    // octet order (gated): one step per K block, pipelined
    if (nq.G > kNqMaxSlices) gemv_gateup_nq_wnp<W, 1, true, true, true>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
    else gemv_gateup_nq_wnp<W, 1, true, false, true>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
    return;
  }
  if (nq.G > kNqMaxSlices) {
    // the whole-column down GEMV's slice sums (one step per K block, pipelined)
    gemv_gateup_nq_wnp<W, 1, true, true>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
    return;
  }
  const bool pipe = gemv_pipe("FRT_GEMV_PIPE_GATEUP", true);
  if (gemv_nb("FRT_GEMV_NB_GATEUP", 1) == 2) {
    if (pipe) gemv_gateup_nq_wnp<W, 2, true>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
    else gemv_gateup_nq_wnp<W, 2, false>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
  } else {
    if (pipe) gemv_gateup_nq_wnp<W, 1, true>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
    else gemv_gateup_nq_wnp<W, 1, false>(act, nq, w, hq, M, K, I, a_g, a_u, inv_h, s);
  }
}

// Whether k_gemv_gateup_nq takes the shape (frt_normq.h), and with slice sums
// per four columns (G = K / 4) at W waves.
bool gemv_nq_supported(int M, int K, int G) { return normq_shape_ok(M, K, G); }
bool gemv_nq_wide_supported(int M, int K, int W) {
  const int G = K / 4;
  return normq_shape_ok(M, K, 1) && M <= 4 && G > kNqMaxSlices && G % 2 == 0 &&
         M * G <= 2 * kNqWidePairs * 64 * W;
}

// gate/up GEMV from r' and the slice sums (k_add_sumsq) instead of XQ; the
// codes it forms are stored to xq_out.
// oct: the gate/up matrix in octet order (gated activations only).
hipError_t launch_gemv_gateup_nq(int act, const uint16_t* r, const uint16_t* w_norm, const double* sq, int G,
                                 float eps, float inv_x, uint8_t* xq_out, const uint8_t* w, uint8_t* hq, int M, int K,
                                 int I, int W, float alpha_g, float alpha_u, float inv_h, hipStream_t s, int oct) {
  const bool wide = G > kNqMaxSlices;
  if ((wide ? !(G == K / 4 && gemv_nq_wide_supported(M, K, W)) : !gemv_nq_supported(M, K, G)) || G < 1 || I % 16 ||
      W > K / 128 || (oct && act == GU_GELU))
    return hipErrorInvalidValue;
  const NormQ nq{r, w_norm, sq, G, eps, inv_x, xq_out};
  const bool o = oct != 0;
  switch (W) {
    case 1: gemv_gateup_nq_w<1>(act, nq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s, o); break;
    case 2: gemv_gateup_nq_w<2>(act, nq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s, o); break;
    case 4: gemv_gateup_nq_w<4>(act, nq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s, o); break;
    case 8: gemv_gateup_nq_w<8>(act, nq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s, o); break;
    case 16: gemv_gateup_nq_w<16>(act, nq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s, o); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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

// Column groups per workgroup of the fused kernel: FRT_GEMV_FUSED_GROUPS
// (1, 2 or 4; default 2).
static int fused_groups() {
  const char* e = getenv("FRT_GEMV_FUSED_GROUPS");
  int g = (e && *e) ? atoi(e) : 2;
  return (g == 1 || g == 2 || g == 4) ? g : 2;
}

template <int ACT, int W, int NCH>
static hipError_t gateup_fused_nch(const FusedArgs& a, hipStream_t s) {
  const int G = fused_groups();
  const int P = a.I / 16;
  dim3 grid((P + G - 1) / G), block(W * 64);
  if (G == 1)
    hipLaunchKernelGGL((k_gemv_gateup_fused<ACT, W, NCH, 1>), grid, block, 0, s, a);
  else if (G == 2)
    hipLaunchKernelGGL((k_gemv_gateup_fused<ACT, W, NCH, 2>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_gemv_gateup_fused<ACT, W, NCH, 4>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int ACT, int W>
static hipError_t gateup_fused_w(const FusedArgs& a, hipStream_t s) {
  const int nchunk = a.K / 8;
  const int gt = (a.M == 1) ? W * 64 : 64;
  const int nch = (nchunk + gt - 1) / gt;
  if (nch <= 1) return gateup_fused_nch<ACT, W, 1>(a, s);
  if (nch <= 2) return gateup_fused_nch<ACT, W, 2>(a, s);
  if (nch <= 4) return gateup_fused_nch<ACT, W, 4>(a, s);
  if (nch <= 8) return gateup_fused_nch<ACT, W, 8>(a, s);
  return hipErrorInvalidValue;
}

template <int ACT>
static hipError_t gateup_fused_act(int W, const FusedArgs& a, hipStream_t s) {
  switch (W) {
    case 2: return gateup_fused_w<ACT, 2>(a, s);
    case 4: return gateup_fused_w<ACT, 4>(a, s);
    case 8: return gateup_fused_w<ACT, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Whether the fused decode kernel can take this shape (LDS for the rows,
// register chunks of the prologue, at least two waves to share a row).
bool gemv_fused_supported(int M, int K, int W) {
  if (M < 1 || M > 16 || W < 2 || W > 8 || (long)M * K > kFusedXqBytes) return false;
  const int gt = (M == 1) ? W * 64 : 64;
  return (K / 8 + gt - 1) / gt <= 8;
}

// y_part null: Y comes from y_prev; else from S fp32 partials (dequantised by
// a_prev) and workgroup 0 stores it to y_store.
hipError_t launch_gemv_gateup_fused(int act, const uint16_t* r_prev, const uint16_t* y_prev, const float* y_part,
                                    int S, float a_prev, uint16_t* y_store, const uint16_t* w_norm,
                                    uint16_t* r_out, uint8_t* xq_out, const uint8_t* w, uint8_t* hq, int M, int K,
                                    int I, int W, float eps, float inv_x, float a_g, float a_u, float inv_h,
                                    hipStream_t s) {
  const FusedArgs a{r_prev, y_prev, y_part, S, a_prev, y_store, w_norm, r_out, xq_out, w, hq, M, K, I,
                    eps, inv_x, a_g, a_u, inv_h};
  if (act == GU_GEGLU) return gateup_fused_act<GU_GEGLU>(W, a, s);
  if (act == GU_SWIGLU) return gateup_fused_act<GU_SWIGLU>(W, a, s);
  return gateup_fused_act<GU_GELU>(W, a, s);
}

template <bool FP8, int COLS, int NB, bool PIPE>
static hipError_t gemv_down_tnp(const uint8_t* hq, const uint8_t* w, uint16_t* y, float* part, int M, int K,
                                int N, int W, int S, float alpha_d, hipStream_t s) {
  dim3 grid((N / 16) * (16 / COLS), S), block(W * 64);
  // split-major workgroup order by default (M=1 decode down GEMV: 15.41
  // against 15.58 us); FRT_GEMV_DOWN_ORDER=0 restores column-major
  const char* oe = getenv("FRT_GEMV_DOWN_ORDER");
  const int order = (oe && *oe) ? atoi(oe) != 0 : 1;
#define FRT_DOWN(WV) \
  hipLaunchKernelGGL((k_gemv_down<WV, FP8, COLS, NB, PIPE>), grid, block, 0, s, hq, w, y, part, M, K, N, alpha_d, \
                     order)
  switch (W) {
    case 1: FRT_DOWN(1); break;
    case 2: FRT_DOWN(2); break;
    case 4: FRT_DOWN(4); break;
    case 8: FRT_DOWN(8); break;
    case 16: FRT_DOWN(16); break;
    default: return hipErrorInvalidValue;
  }
#undef FRT_DOWN
  return hipGetLastError();
}

template <bool FP8, int COLS>
static hipError_t gemv_down_t(const uint8_t* hq, const uint8_t* w, uint16_t* y, float* part, int M, int K,
                              int N, int W, int S, float alpha_d, hipStream_t s) {
  const bool pipe = gemv_pipe("FRT_GEMV_PIPE_DOWN", true);
  if (gemv_nb("FRT_GEMV_NB_DOWN", 1) == 2)
    return pipe ? gemv_down_tnp<FP8, COLS, 2, true>(hq, w, y, part, M, K, N, W, S, alpha_d, s)
                : gemv_down_tnp<FP8, COLS, 2, false>(hq, w, y, part, M, K, N, W, S, alpha_d, s);
  return pipe ? gemv_down_tnp<FP8, COLS, 1, true>(hq, w, y, part, M, K, N, W, S, alpha_d, s)
              : gemv_down_tnp<FP8, COLS, 1, false>(hq, w, y, part, M, K, N, W, S, alpha_d, s);
}

// Columns per down-GEMV workgroup (FRT_GEMV_DOWN_COLS = 8 or 16).
static int down_cols(int N) {
  (void)N;
  const char* e = getenv("FRT_GEMV_DOWN_COLS");
  if (e && *e) return atoi(e) == 8 ? 8 : 16;
  return 16;  // measured: half-group workgroups stream slower at H = 5120
}

// S > 1: K split over S workgroups per column group, fp32 partials [S][M][N]
// into part (summed by the consumer), else bf16 Y.
hipError_t launch_gemv_down(const uint8_t* hq, const uint8_t* w, uint16_t* y, float* part, int M, int K,
                            int N, int W, int S, bool fp8, float alpha_d, hipStream_t s) {
  const int cols = down_cols(N);
  if (S < 1 || S > (K >> 7)) return hipErrorInvalidValue;
  if (fp8)
    return cols == 8 ? gemv_down_t<true, 8>(hq, w, y, part, M, K, N, W, S, alpha_d, s)
                     : gemv_down_t<true, 16>(hq, w, y, part, M, K, N, W, S, alpha_d, s);
  return cols == 8 ? gemv_down_t<false, 8>(hq, w, y, part, M, K, N, W, S, alpha_d, s)
                   : gemv_down_t<false, 16>(hq, w, y, part, M, K, N, W, S, alpha_d, s);
}

// Whole-column down GEMV (M <= 4, K % 256 == 0, N % 4 == 0, W at most
// K / 256): Y, and with r_out R' = bf16(R + Y) and the quad slice sums.
// FRT_GEMV_PIPE_DOWN=0 runs it unpipelined.
bool gemv_down_quad_supported(int M, int K, int N) {
  return M >= 1 && M <= 4 && K >= 256 && K % 256 == 0 && N >= 4 && N % 4 == 0;
}

hipError_t launch_gemv_down_quad(const uint8_t* hq, const uint8_t* w, const uint16_t* r_in, uint16_t* y,
                                 uint16_t* r_out, double* sq, int M, int K, int N, int W, float alpha_d,
                                 hipStream_t s) {
  if (!gemv_down_quad_supported(M, K, N) || W < 1 || W > (K >> 8) || (r_out && (!r_in || !sq)))
    return hipErrorInvalidValue;
  const bool pipe = gemv_pipe("FRT_GEMV_PIPE_DOWN", true);
  // one 1 KiB step per stage by default (measured at M=1, N=5120, K=17408 on
  // eight waves: 16.0 us against 16.4 with two steps and 18.0 with four)
  const int nb = gemv_nb("FRT_GEMV_NB_DOWN_QUAD", 1);
  const dim3 grid(N / 4), block(W * 64);
#define FRT_DQ(WV, B, P) \
  hipLaunchKernelGGL((k_gemv_down_quad<WV, B, P>), grid, block, 0, s, hq, w, r_in, y, r_out, sq, M, K, N, alpha_d)
#define FRT_DQW(WV)                   \
  if (nb == 2) {                      \
    if (pipe) FRT_DQ(WV, 2, true);    \
    else FRT_DQ(WV, 2, false);        \
  } else {                            \
    if (pipe) FRT_DQ(WV, 1, true);    \
    else FRT_DQ(WV, 1, false);        \
  }
  switch (W) {
    case 1: FRT_DQW(1); break;
    case 2: FRT_DQW(2); break;
    case 4: FRT_DQW(4); break;
    case 8: FRT_DQW(8); break;
    case 16: FRT_DQW(16); break;
    default: return hipErrorInvalidValue;
  }
#undef FRT_DQW
#undef FRT_DQ
  return hipGetLastError();
}

// Multi-tile GEMV launchers (16 < M <= 64): W in {4, 8} waves (at least MT).
template <int ACT, int W, int MT>
static void gemv_gateup_mt_t(const uint8_t* xq, const uint8_t* w, uint8_t* hq, int M, int K, int I, float a_g,
                             float a_u, float inv_h, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv_gateup_mt<ACT, W, MT>), dim3(I / 16), dim3(W * 64), 0, s, xq, w, hq, M, K, I, a_g,
                     a_u, inv_h);
}

template <int ACT, int W>
static hipError_t gemv_gateup_mt_w(const uint8_t* xq, const uint8_t* w, uint8_t* hq, int M, int K, int I,
                                   float a_g, float a_u, float inv_h, hipStream_t s) {
  switch ((M + 15) / 16) {
    case 2: gemv_gateup_mt_t<ACT, W, 2>(xq, w, hq, M, K, I, a_g, a_u, inv_h, s); break;
    case 3: gemv_gateup_mt_t<ACT, W, 3>(xq, w, hq, M, K, I, a_g, a_u, inv_h, s); break;
    case 4: gemv_gateup_mt_t<ACT, W, 4>(xq, w, hq, M, K, I, a_g, a_u, inv_h, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int ACT>
static hipError_t gemv_gateup_mt_act(int W, const uint8_t* xq, const uint8_t* w, uint8_t* hq, int M, int K,
                                     int I, float a_g, float a_u, float inv_h, hipStream_t s) {
  if (W == 4) return gemv_gateup_mt_w<ACT, 4>(xq, w, hq, M, K, I, a_g, a_u, inv_h, s);
  if (W == 8) return gemv_gateup_mt_w<ACT, 8>(xq, w, hq, M, K, I, a_g, a_u, inv_h, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_gateup_mt(int act, const uint8_t* xq, const uint8_t* w, uint8_t* hq, int M, int K, int I,
                                 int W, float alpha_g, float alpha_u, float inv_h, hipStream_t s) {
  if (M <= 16 || M > 64 || (K >> 7) < 1) return hipErrorInvalidValue;
  if (act == GU_GEGLU) return gemv_gateup_mt_act<GU_GEGLU>(W, xq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s);
  if (act == GU_SWIGLU) return gemv_gateup_mt_act<GU_SWIGLU>(W, xq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s);
  return gemv_gateup_mt_act<GU_GELU>(W, xq, w, hq, M, K, I, alpha_g, alpha_u, inv_h, s);
}

template <int W, bool FP8>
static hipError_t gemv_down_mt_w(const uint8_t* hq, const uint8_t* w, uint16_t* y, float* part, int M, int K,
                                 int N, int S, float alpha_d, hipStream_t s) {
  dim3 grid(N / 16, S), block(W * 64);
  switch ((M + 15) / 16) {
    case 2: hipLaunchKernelGGL((k_gemv_down_mt<W, FP8, 2>), grid, block, 0, s, hq, w, y, part, M, K, N, alpha_d); break;
    case 3: hipLaunchKernelGGL((k_gemv_down_mt<W, FP8, 3>), grid, block, 0, s, hq, w, y, part, M, K, N, alpha_d); break;
    case 4: hipLaunchKernelGGL((k_gemv_down_mt<W, FP8, 4>), grid, block, 0, s, hq, w, y, part, M, K, N, alpha_d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_down_mt(const uint8_t* hq, const uint8_t* w, uint16_t* y, float* part, int M, int K,
                               int N, int W, int S, bool fp8, float alpha_d, hipStream_t s) {
  if (M <= 16 || M > 64 || S < 1 || S > (K >> 7)) return hipErrorInvalidValue;
  if (W == 4) return fp8 ? gemv_down_mt_w<4, true>(hq, w, y, part, M, K, N, S, alpha_d, s)
                         : gemv_down_mt_w<4, false>(hq, w, y, part, M, K, N, S, alpha_d, s);
  if (W == 8) return fp8 ? gemv_down_mt_w<8, true>(hq, w, y, part, M, K, N, S, alpha_d, s)
                         : gemv_down_mt_w<8, false>(hq, w, y, part, M, K, N, S, alpha_d, s);
  return hipErrorInvalidValue;
}

bool gemm_config_ok(int cfg, bool fp8) { return cfg >= 0 && cfg < kGemmConfigs && (fp8 || cfg != 6); }

template <int EPI, bool FP8, int C>
static void gemm_cfg(dim3 grid, hipStream_t s, const uint8_t* act, const uint8_t* w, void* out, float* part,
                     int M, int K, int Npk, int S, float a, float b, float inv) {
  constexpr int WGM = cfg_wgm(C), WGN = cfg_wgn(C);
  hipLaunchKernelGGL((k_gemm<EPI, FP8, cfg_bm(C), cfg_bn(C), WGM, WGN>), grid, dim3(WGM * WGN * 64), 0, s,
                     act, w, out, part, M, K, Npk, S, a, b, inv);
}

template <int EPI, bool FP8>
static hipError_t gemm_mode(int cfg, const uint8_t* act, const uint8_t* w, void* out, float* part, int M,
                            int K, int Npk, int S, float a, float b, float inv, hipStream_t s) {
  if (!gemm_config_ok(cfg, FP8)) return hipErrorInvalidValue;
  const int BM = cfg_bm(cfg), BN = cfg_bn(cfg);
  if (Npk % BN) return hipErrorInvalidValue;
  dim3 grid(Npk / BN, (M + BM - 1) / BM, S);
  switch (cfg) {
    case 0: gemm_cfg<EPI, FP8, 0>(grid, s, act, w, out, part, M, K, Npk, S, a, b, inv); break;
    case 1: gemm_cfg<EPI, FP8, 1>(grid, s, act, w, out, part, M, K, Npk, S, a, b, inv); break;
    case 2: gemm_cfg<EPI, FP8, 2>(grid, s, act, w, out, part, M, K, Npk, S, a, b, inv); break;
    case 3: gemm_cfg<EPI, FP8, 3>(grid, s, act, w, out, part, M, K, Npk, S, a, b, inv); break;
    case 4: gemm_cfg<EPI, FP8, 4>(grid, s, act, w, out, part, M, K, Npk, S, a, b, inv); break;
    case 5: gemm_cfg<EPI, FP8, 5>(grid, s, act, w, out, part, M, K, Npk, S, a, b, inv); break;
    default:
      if constexpr (FP8) gemm_cfg<EPI, FP8, 6>(grid, s, act, w, out, part, M, K, Npk, S, a, b, inv);
      break;
  }
  return hipGetLastError();
}

int gemm_config_bm(int cfg) { return cfg_bm(cfg); }
int gemm_config_bn(int cfg) { return cfg_bn(cfg); }

hipError_t launch_gemm_gateup(int act, int cfg, bool fp8, const uint8_t* xq, const uint8_t* w, uint8_t* hq,
                              int M, int K, int Npk, float alpha_g, float alpha_u, float inv_h, hipStream_t s) {
  const float a = alpha_g, b = alpha_u;
  if (fp8) {
    if (act == GU_GEGLU) return gemm_mode<GU_GEGLU, true>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
    if (act == GU_SWIGLU) return gemm_mode<GU_SWIGLU, true>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
    return gemm_mode<GU_GELU, true>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
  }
  if (act == GU_GEGLU) return gemm_mode<GU_GEGLU, false>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
  if (act == GU_SWIGLU) return gemm_mode<GU_SWIGLU, false>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
  return gemm_mode<GU_GELU, false>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
}

// S > 1: fp32 partials [S][M][N] into part (summed by the consumer), else bf16 Y.
hipError_t launch_gemm_down(int cfg, const uint8_t* hq, const uint8_t* w, uint16_t* y, float* part, int M,
                            int K, int N, int S, bool fp8, float alpha_d, hipStream_t s) {
  if (fp8) return gemm_mode<EPI_DOWN, true>(cfg, hq, w, y, part, M, K, N, S, alpha_d, 0.0f, 0.0f, s);
  return gemm_mode<EPI_DOWN, false>(cfg, hq, w, y, part, M, K, N, S, alpha_d, 0.0f, 0.0f, s);
}

}  // namespace frt
