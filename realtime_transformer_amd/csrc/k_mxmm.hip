// k_mxmm.hip -- the prefill-sized (M > 64) MXFP4 GEMMs of the FFN block.
//
// itsolotime article, section 7.2 (the 4-bit encoder FFN: 4-bit gate/up and
// down GEMMs over a few hundred prefix tokens, a gated combine that
// re-quantises to 4 bits); the format is OCP MXFP4 (frt_mx.h).
//
// Tile: 128 activation rows x 128 packed weight rows per workgroup, four
// waves of 64 x 64 (4 x 4 blocks of 16 x 16).  K advances in stages of 128
// values (64 bytes of codes per row).  Per stage each 16-row block of either
// operand is one 1 KiB run in LDS in the operand order of the block-scaled
// FP4 instruction (lane l: row l % 16, values (l / 16) * 32 .. + 32), so one
// ds_read_b128 per block feeds one v_mfma_scale_f32_16x16x128_f8f6f4; the
// exponents of the stage are staged beside the codes (activations: 4 bytes
// per row; weights: 64 bytes per 16-row group in the prefill layout, one per
// lane).  All staging is direct-to-LDS (global_load_lds_dwordx4 / _dword):
// each wave issues exactly five such loads per stage (two activation runs,
// two weight runs, one exponent run), into a ring of four stage buffers, so
// its wait counts are static.
//
// Epilogues: gate/up -- a wave's 64 packed rows are gate 2P, up 2P, gate
// 2P + 1, up 2P + 1 of intermediate block P (32 columns), so the gated
// combine and the 4-bit re-quantisation of that block run in registers as in
// the GEMV (mx_store_h32).  Down -- bf16 Y, or fp32 partials [split][M][N]
// when K is split over workgroups (summed by the consumer).
#include "frt_mx.h"

namespace frt {

enum { MXM_GEGLU = MX_GEGLU, MXM_SWIGLU = MX_SWIGLU, MXM_GELU = MX_GELU, MXM_DOWN = 3 };

// direct-to-LDS loads (as in k_mm.hip: issued from inline assembly so that
// the compiler does not make later LDS reads wait for them; the kernel
// orders them with its own s_waitcnt vmcnt and barriers)
__device__ __forceinline__ void mx_dma16(const uint8_t* g, const uint8_t* l) {
  const uint32_t m0 = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)l);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void mx_dma4(const uint8_t* g, const uint8_t* l) {
  const uint32_t m0 = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)l);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
constexpr int mx_waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
__device__ __forceinline__ void mx_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int XBM = 128, XBN = 128, XNS = 4, XOPS = 5;
constexpr int XA = XBM * 64;               // activation codes
constexpr int XB = XBN * 64;               // weight codes
constexpr int XAS = XBM * 4;               // activation exponents: [row][4]
constexpr int XBS = (XBN / 16) * 64;       // weight exponents: [group][lane]
constexpr int XSTAGE = XA + XB + XAS + XBS;

typedef int v4i_mx __attribute__((ext_vector_type(4)));

template <int EPI>
__global__ __launch_bounds__(256) void k_mxmm(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                              const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                                              uint8_t* __restrict__ hc, uint8_t* __restrict__ hs,
                                              uint16_t* __restrict__ y, float* __restrict__ part, int M, int K,
                                              int Npk, int tiles_n, int tiles_m, int S) {
  __shared__ __attribute__((aligned(1024))) uint8_t l0[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t l1[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t l2[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t l3[XSTAGE];
  constexpr bool DOWN = EPI == MXM_DOWN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wa = wave >> 1, wn = wave & 1;

  // Work item: split-major, then column tile, then row tile.  Consecutive
  // workgroups go to different XCDs (round robin over 8); workgroup b runs
  // item (b % 8) * q + min(b % 8, r) + b / 8 (T = 8 q + r items), so XCD x
  // holds one contiguous range of items: all row tiles of a column tile
  // share that XCD's L2, which fetches the weight panel once.
  int sp, tn, tm;
  {
    const int T = tiles_n * tiles_m * S, q = T >> 3, r = T & 7;
    const int x = blockIdx.x & 7;
    const int idx = x * q + (x < r ? x : r) + (blockIdx.x >> 3);
    sp = idx / (tiles_n * tiles_m);
    const int rem = idx - sp * tiles_n * tiles_m;
    tn = rem / tiles_m;
    tm = rem - tn * tiles_m;
  }
  const int m0 = tm * XBM, n0 = tn * XBN;
  const int KB = K >> 7;  // stages (128-value blocks)
  const int kb0 = sp * KB / S, kb1 = (sp + 1) * KB / S, nk = kb1 - kb0;
  const int g0 = n0 >> 4;  // first 16-row weight group of the tile

  // This wave's five loads per stage: activation runs r = wave, wave + 4;
  // weight runs g = wave, wave + 4; one exponent run (waves 0, 1: activation
  // rows 64 t .. 64 t + 63; waves 2, 3: weight groups 4 t .. 4 t + 3).
  // Source addresses at stage 0, the stage stride, LDS destinations.
  const uint8_t* src[XOPS];
  uint32_t step[XOPS], dst[XOPS];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = i * 4 + wave;
    int m = m0 + 16 * r + (lane & 15);
    m = m < M ? m : M - 1;  // rows past M load row M - 1; their outputs are not stored
    src[i] = xc + (size_t)m * (K / 2) + (lane >> 4) * 16;
    step[i] = 64;
    dst[i] = (uint32_t)(r * 1024);
    const int g = g0 + i * 4 + wave;
    src[2 + i] = wc + (size_t)g * KB * 1024 + lane * 16;
    step[2 + i] = 1024;
    dst[2 + i] = (uint32_t)(XA + (i * 4 + wave) * 1024);
  }
  if (wave < 2) {
    int m = m0 + wave * 64 + lane;
    m = m < M ? m : M - 1;
    src[4] = xs + (size_t)m * (K / 32);
    step[4] = 4;
    dst[4] = (uint32_t)(XA + XB + wave * 256);
  } else {
    const int t = wave - 2;
    const int g = g0 + t * 4 + (lane >> 4);
    src[4] = ws + (size_t)g * KB * 64 + (lane & 15) * 4;
    step[4] = 64;
    dst[4] = (uint32_t)(XA + XB + XAS + t * 256);
  }
  auto issue = [&](int kb, uint8_t* base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) mx_dma16(src[i] + (size_t)kb * step[i], base + dst[i]);
    mx_dma4(src[4] + (size_t)kb * step[4], base + dst[4]);
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0, 0, 0, 0};

  // per-lane LDS read offsets inside a stage
  const int a_rd = (wa * 4) * 1024 + lane * 16;
  const int b_rd = XA + (wn * 4) * 1024 + lane * 16;
  const int as_rd = XA + XB + ((wa * 4) * 16 + (lane & 15)) * 4 + (lane >> 4);
  const int bs_rd = XA + XB + XAS + (wn * 4) * 64 + lane;

  auto mma_stage = [&](const uint8_t* base) {
    v8i a[4], b[4];
    int sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4i_mx t = *reinterpret_cast<const v4i_mx*>(base + a_rd + i * 1024);
      a[i] = v8i{t[0], t[1], t[2], t[3], 0, 0, 0, 0};
      sa[i] = base[as_rd + i * 16 * 4];
      const v4i_mx u = *reinterpret_cast<const v4i_mx*>(base + b_rd + i * 1024);
      b[i] = v8i{u[0], u[1], u[2], u[3], 0, 0, 0, 0};
      sb[i] = base[bs_rd + i * 64];
    }
    // the fragments are in registers: the buffer may be refilled after the
    // next barrier
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    mx_lds_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mx_mfma(a[i], sa[i], b[j], sb[j], acc[i][j]);
  };
  // stage t complete for this wave once at most `after` later stages of its
  // loads are outstanding
  auto wait_stage = [&](int t) {
    const int after = (nk - 1 - t) < (XNS - 1) ? (nk - 1 - t) : (XNS - 1);
    if (after >= 3) __builtin_amdgcn_s_waitcnt(mx_waitcnt_vm(3 * XOPS));
    else if (after == 2) __builtin_amdgcn_s_waitcnt(mx_waitcnt_vm(2 * XOPS));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(mx_waitcnt_vm(XOPS));
    else __builtin_amdgcn_s_waitcnt(mx_waitcnt_vm(0));
    mx_lds_barrier();
  };
  // step t: refill the buffer freed at step t - 1 with stage t + 3, wait for
  // stage t, read its fragments, release its buffer, multiply
#define FRT_MXMM_STEP(t, FILL, CUR)                     \
  do {                                                  \
    if ((t) + XNS - 1 < nk) issue(kb0 + (t) + XNS - 1, FILL); \
    wait_stage(t);                                      \
    mma_stage(CUR);                                     \
  } while (0)
  if (nk > 0) issue(kb0, l0);
  if (nk > 1) issue(kb0 + 1, l1);
  if (nk > 2) issue(kb0 + 2, l2);
  int t = 0;
  for (; t + 3 < nk; t += 4) {
    FRT_MXMM_STEP(t, l3, l0);
    FRT_MXMM_STEP(t + 1, l0, l1);
    FRT_MXMM_STEP(t + 2, l1, l2);
    FRT_MXMM_STEP(t + 3, l2, l3);
  }
  if (t < nk) FRT_MXMM_STEP(t, l3, l0);
  if (t + 1 < nk) FRT_MXMM_STEP(t + 1, l0, l1);
  if (t + 2 < nk) FRT_MXMM_STEP(t + 2, l1, l2);
#undef FRT_MXMM_STEP

  // ---- epilogue ----
  const int row = lane & 15, q = lane >> 4;
  if (!DOWN) {
    const int I = (EPI == MXM_GELU) ? Npk : Npk / 2;
    // packed groups g0 + 4 wn .. + 3 -> intermediate 32-column block P
    const int P = (g0 + 4 * wn) >> 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (wa * 4 + i) * 16 + 4 * q + r;
        float h0, h1;
        if (EPI == MXM_GELU) {
          // plain layout: groups 4P' .. 4P' + 3 are two 32-column blocks
          h0 = mx_gated<MX_GELU>(0.0f, acc[i][0][r]);
          h1 = mx_gated<MX_GELU>(0.0f, acc[i][1][r]);
        } else {
          h0 = mx_gated<EPI>(acc[i][0][r], acc[i][1][r]);
          h1 = mx_gated<EPI>(acc[i][2][r], acc[i][3][r]);
        }
        const int mm = m < M ? m : 0;
        const int Pb = (EPI == MXM_GELU) ? 2 * P : P;
        mx_store_h32(h0, h1, m < M, row, hc + (size_t)mm * (I / 2) + (size_t)Pb * 16, hs + (size_t)mm * (I / 32) + Pb);
        if (EPI == MXM_GELU) {
          const float h2 = mx_gated<MX_GELU>(0.0f, acc[i][2][r]);
          const float h3 = mx_gated<MX_GELU>(0.0f, acc[i][3][r]);
          mx_store_h32(h2, h3, m < M, row, hc + (size_t)mm * (I / 2) + (size_t)(Pb + 1) * 16,
                       hs + (size_t)mm * (I / 32) + Pb + 1);
        }
      }
    }
    return;
  }
  const int N = Npk;
  float* ps = part + (size_t)sp * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + (wa * 4 + i) * 16 + 4 * q + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t o = (size_t)m * N + (size_t)(g0 + wn * 4 + j) * 16 + row;
        if (S == 1)
          y[o] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        else
          ps[o] = acc[i][j][r];
      }
    }
  }
}

// Gate/up: Npk packed rows (2I gated, I plain), K = H; E4M3-free 4-bit out.
hipError_t launch_mxmm_gateup(int act, const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws,
                              uint8_t* hc, uint8_t* hs, int M, int K, int Npk, hipStream_t s) {
  if (M < 1 || K % 512 || Npk % XBN) return hipErrorInvalidValue;
  const int tn = Npk / XBN, tm = (M + XBM - 1) / XBM;
  const dim3 grid(tn * tm), block(256);
  if (act == MX_GEGLU)
    hipLaunchKernelGGL((k_mxmm<MXM_GEGLU>), grid, block, 0, s, xc, xs, wc, ws, hc, hs, nullptr, nullptr, M, K, Npk, tn,
                       tm, 1);
  else if (act == MX_SWIGLU)
    hipLaunchKernelGGL((k_mxmm<MXM_SWIGLU>), grid, block, 0, s, xc, xs, wc, ws, hc, hs, nullptr, nullptr, M, K, Npk,
                       tn, tm, 1);
  else
    hipLaunchKernelGGL((k_mxmm<MXM_GELU>), grid, block, 0, s, xc, xs, wc, ws, hc, hs, nullptr, nullptr, M, K, Npk, tn,
                       tm, 1);
  return hipGetLastError();
}

// Down: N = H output columns, K = I; S splits (> 1: fp32 partials).
hipError_t launch_mxmm_down(const uint8_t* hc, const uint8_t* hs, const uint8_t* wc, const uint8_t* ws, uint16_t* y,
                            float* part, int M, int K, int N, int S, hipStream_t s) {
  if (M < 1 || K % 512 || N % XBN || S < 1 || S > K / 128) return hipErrorInvalidValue;
  const int tn = N / XBN, tm = (M + XBM - 1) / XBM;
  hipLaunchKernelGGL((k_mxmm<MXM_DOWN>), dim3(tn * tm * S), dim3(256), 0, s, hc, hs, wc, ws, nullptr, nullptr, y, part,
                     M, K, N, tn, tm, S);
  return hipGetLastError();
}

}  // namespace frt
