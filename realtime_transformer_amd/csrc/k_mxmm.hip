// k_mxmm.hip -- the prefill-sized (M > 64) MXFP4 GEMMs of the FFN block.
//
// itsolotime article, section 7.2 (the 4-bit encoder FFN: 4-bit gate/up and
// down GEMMs over a few hundred prefix tokens, a gated combine that
// re-quantises to 4 bits); the format is OCP MXFP4 (frt_mx.h).
//
// Tile: 128 activation rows x 32*NB packed weight rows per workgroup, four
// waves of 64 x 16*NB (4 x NB blocks of 16 x 16).  K advances in stages of
// 128 values (64 bytes of codes per row).  Per stage each 16-row block of
// either operand is one 1 KiB run in LDS in the operand order of the
// block-scaled FP4 instruction (lane l: row l % 16, values (l / 16) * 32 ..
// + 32), so one ds_read_b128 per block feeds one
// v_mfma_scale_f32_16x16x128_f8f6f4; the exponents of the stage are staged
// beside the codes in the prefill layouts (frt_mx.h), where one 32-bit read
// gives a lane the exponents of four blocks and op_sel picks the byte.  All
// staging is direct-to-LDS (global_load_lds_dwordx4 / _dword) into a ring of
// NS stage buffers; every wave issues the same number of loads per stage, so
// its wait counts are static, and one barrier per stage both publishes the
// stage and frees the buffer read one stage earlier.
//
// Why wide tiles: the staging path is the bound (measured with the MFMAs,
// LDS reads and epilogue switched off: ~12 TB/s from L2 for 128 x 128 tiles
// at M = 788, K = 2048), so the bytes staged per flop set the time; 128 x 256
// tiles stage 27% fewer bytes than 128 x 128 for the gate/up GEMM.
//
// Epilogues: gate/up -- a wave's packed rows are, per intermediate block P
// (32 columns), gate 2P, up 2P, gate 2P + 1, up 2P + 1, so the gated combine
// and the 4-bit re-quantisation of that block run in registers as in the
// GEMV (mx_store_h32); its exponents go out in the prefill layout for the
// down GEMM.  Down -- bf16 Y, or fp32 partials [split][M][N] when K is split
// over workgroups (summed by the consumer).
#include <utility>

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

typedef int v4i_mx __attribute__((ext_vector_type(4)));

// Tile geometry for NB weight blocks per wave (4: 128 x 128 tiles, 4-stage
// ring; 8: 128 x 256 tiles, 3-stage ring -- both leave room for two
// workgroups per CU).
template <int NB>
struct MxTile {
  static constexpr int BM = 128, BN = 32 * NB, NS = NB == 8 ? 3 : 4;
  static constexpr int XA = BM * 64;          // activation codes: 8 runs of 1 KiB
  static constexpr int XB = BN * 64;          // weight codes: 2 NB runs
  static constexpr int XAS = 2 * 256;         // activation exponents: 2 row groups x 64 lanes x 4
  static constexpr int XBS = (BN / 64) * 256; // weight exponents: NB / 2 group quads x 64 lanes x 4
  static constexpr int STAGE = XA + XB + XAS + XBS;
  static constexpr int CRUNS = 2 + NB / 2;       // code runs per wave per stage
  static constexpr int ERUNS = NB == 8 ? 2 : 1;  // exponent runs per wave per stage
  static constexpr int OPS = CRUNS + ERUNS;
};

template <int OA, int OB>
__device__ __forceinline__ v4f mx_mfma_sel(v8i a, int sa, v8i b, int sb, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OA, sa, OB, sb);
}
// all 4 x NB products of one stage; the exponent bytes are op_sel immediates
template <int NB, int... IJ>
__device__ __forceinline__ void mx_mma_all(v4f (&acc)[4][NB], const v8i (&a)[4], const v8i (&b)[NB], int sa,
                                           const int (&sb)[NB / 4], std::integer_sequence<int, IJ...>) {
  ((acc[IJ / NB][IJ % NB] = mx_mfma_sel<IJ / NB, (IJ % NB) & 3>(a[IJ / NB], sa, b[IJ % NB], sb[(IJ % NB) >> 2],
                                                               acc[IJ / NB][IJ % NB])),
   ...);
}

template <int EPI, int NB>
__global__ __launch_bounds__(256, 2) void k_mxmm(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                 const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                                                 uint8_t* __restrict__ hc, uint8_t* __restrict__ hs,
                                                 uint16_t* __restrict__ y, float* __restrict__ part, int M, int K,
                                                 int Npk, int tiles_n, int tiles_m, int S) {
  using T = MxTile<NB>;
  constexpr int NS = T::NS;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * T::STAGE];
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
    const int Ti = tiles_n * tiles_m * S, q = Ti >> 3, r = Ti & 7;
    const int x = blockIdx.x & 7;
    const int idx = x * q + (x < r ? x : r) + (blockIdx.x >> 3);
    sp = idx / (tiles_n * tiles_m);
    const int rem = idx - sp * tiles_n * tiles_m;
    tn = rem / tiles_m;
    tm = rem - tn * tiles_m;
  }
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int KB = K >> 7;  // stages (128-value blocks)
  const int kb0 = sp * KB / S, kb1 = (sp + 1) * KB / S, nk = kb1 - kb0;
  const int g0 = n0 >> 4;  // first 16-row weight group of the tile

  // This wave's loads per stage: code runs (activation runs wave, wave + 4;
  // weight runs wave + 4 i), then exponent runs e = wave (+ 4): e < 2 the
  // activation row group e, else the weight group quad e - 2; a wave whose
  // second exponent run index passes the end repeats its first (same bytes
  // to the same place).  Source at stage 0, stage stride, LDS offset.
  const uint8_t* src[T::OPS];
  uint32_t step[T::OPS], dst[T::OPS];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = i * 4 + wave;
    int m = m0 + 16 * r + (lane & 15);
    m = m < M ? m : M - 1;  // rows past M load row M - 1; their outputs are not stored
    src[i] = xc + (size_t)m * (K / 2) + (lane >> 4) * 16;
    step[i] = 64;
    dst[i] = (uint32_t)(r * 1024);
  }
#pragma unroll
  for (int i = 0; i < NB / 2; ++i) {
    const int r = i * 4 + wave;
    src[2 + i] = wc + (size_t)(g0 + r) * KB * 1024 + lane * 16;
    step[2 + i] = 1024;
    dst[2 + i] = (uint32_t)(T::XA + r * 1024);
  }
#pragma unroll
  for (int j = 0; j < T::ERUNS; ++j) {
    int e = wave + 4 * j;
    if (e >= 2 + NB / 2) e = wave;
    if (e < 2) {
      src[T::CRUNS + j] = xs + ((size_t)((m0 >> 6) + e) * KB) * 256 + lane * 4;
      dst[T::CRUNS + j] = (uint32_t)(T::XA + T::XB + e * 256);
    } else {
      src[T::CRUNS + j] = ws + ((size_t)((g0 >> 2) + e - 2) * KB) * 256 + lane * 4;
      dst[T::CRUNS + j] = (uint32_t)(T::XA + T::XB + T::XAS + (e - 2) * 256);
    }
    step[T::CRUNS + j] = 256;
  }
  auto issue = [&](int kb, int buf) {
    uint8_t* base = lds + buf * T::STAGE;
#pragma unroll
    for (int i = 0; i < T::CRUNS; ++i) mx_dma16(src[i] + (size_t)kb * step[i], base + dst[i]);
#pragma unroll
    for (int j = 0; j < T::ERUNS; ++j)
      mx_dma4(src[T::CRUNS + j] + (size_t)kb * step[T::CRUNS + j], base + dst[T::CRUNS + j]);
  };

  v4f acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0, 0, 0, 0};

  // per-lane LDS read offsets inside a stage
  const int a_rd = (wa * 4) * 1024 + lane * 16;
  const int b_rd = T::XA + (wn * NB) * 1024 + lane * 16;
  const int as_rd = T::XA + T::XB + wa * 256 + lane * 4;
  const int bs_rd = T::XA + T::XB + T::XAS + (wn * (NB / 4)) * 256 + lane * 4;

  auto mma_stage = [&](int buf) {
    const uint8_t* base = lds + buf * T::STAGE;
    v8i a[4], b[NB];
    int sb[NB / 4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4i_mx t = *reinterpret_cast<const v4i_mx*>(base + a_rd + i * 1024);
      a[i] = v8i{t[0], t[1], t[2], t[3], 0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const v4i_mx u = *reinterpret_cast<const v4i_mx*>(base + b_rd + j * 1024);
      b[j] = v8i{u[0], u[1], u[2], u[3], 0, 0, 0, 0};
    }
    const int sa = *reinterpret_cast<const int*>(base + as_rd);
#pragma unroll
    for (int q = 0; q < NB / 4; ++q) sb[q] = *reinterpret_cast<const int*>(base + bs_rd + q * 256);
    mx_mma_all<NB>(acc, a, b, sa, sb, std::make_integer_sequence<int, 4 * NB>{});
  };

  // Step t: wait until this wave's loads of stage t have landed (at most
  // min(NS - 2, nk - 1 - t) later stages outstanding) and its reads of stage
  // t - 1 are done; the barrier then publishes stage t and frees buffer
  // (t - 1) % NS, which receives stage t + NS - 1; read stage t, multiply.
  for (int t = 0; t < NS - 1 && t < nk; ++t) issue(kb0 + t, t);
  int buf = 0;
  for (int t = 0; t < nk; ++t) {
    const int ahead = (nk - 1 - t) < (NS - 2) ? (nk - 1 - t) : (NS - 2);
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(mx_waitcnt_vm(2 * T::OPS));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(mx_waitcnt_vm(T::OPS));
    else __builtin_amdgcn_s_waitcnt(mx_waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    mx_lds_barrier();
    if (t + NS - 1 < nk) issue(kb0 + t + NS - 1, buf == 0 ? NS - 1 : buf - 1);
    mma_stage(buf);
    buf = buf == NS - 1 ? 0 : buf + 1;
  }

  // ---- epilogue ----
  const int row = lane & 15, q = lane >> 4;
  if (!DOWN) {
    const int I = (EPI == MXM_GELU) ? Npk : Npk / 2;
    const uint32_t KBh = (uint32_t)I / 128;
    // this wave's packed groups g0 + NB wn .. + NB - 1: NB / 4 gated 32-column
    // blocks starting at P, or NB / 2 plain ones starting at 2 P
    const int P = (g0 + NB * wn) >> 2;
    // every block's codes first (one basic block), then the stores
    constexpr int NBLK = (EPI == MXM_GELU) ? NB / 2 : NB / 4;  // 32-column blocks per row
    uint32_t be[4][4][NBLK];
    // (two rows r, r + 1 at a time, their lane-move chains interleaved)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; r += 2)
#pragma unroll
        for (int c = 0; c < NB / 4; ++c) {
          // groups 4c .. 4c + 3 of the wave: one gated block, or two plain
          if (EPI == MXM_GELU) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
              mx_h32_codes2(mx_gated<MX_GELU>(0.0f, acc[i][4 * c + 2 * h][r]),
                            mx_gated<MX_GELU>(0.0f, acc[i][4 * c + 2 * h + 1][r]),
                            mx_gated<MX_GELU>(0.0f, acc[i][4 * c + 2 * h][r + 1]),
                            mx_gated<MX_GELU>(0.0f, acc[i][4 * c + 2 * h + 1][r + 1]), be[i][r][2 * c + h],
                            be[i][r + 1][2 * c + h]);
          } else {
            mx_h32_codes2(mx_gated<EPI>(acc[i][4 * c][r], acc[i][4 * c + 1][r]),
                          mx_gated<EPI>(acc[i][4 * c + 2][r], acc[i][4 * c + 3][r]),
                          mx_gated<EPI>(acc[i][4 * c][r + 1], acc[i][4 * c + 1][r + 1]),
                          mx_gated<EPI>(acc[i][4 * c + 2][r + 1], acc[i][4 * c + 3][r + 1]), be[i][r][c],
                          be[i][r + 1][c]);
          }
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (wa * 4 + i) * 16 + 4 * q + r;
        const int mm = m < M ? m : 0;
        uint8_t* hrow = hc + (size_t)mm * (I / 2);
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
          const int Pb = (EPI == MXM_GELU) ? 2 * P + b : P + b;
          mx_h32_store(be[i][r][b], m < M, row, hrow + (size_t)Pb * 16, hs + mx_act_scale_off_mm(mm, Pb, KBh));
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
      for (int j = 0; j < NB; ++j) {
        const size_t o = (size_t)m * N + (size_t)(g0 + wn * NB + j) * 16 + row;
        if (S == 1)
          y[o] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        else
          ps[o] = acc[i][j][r];
      }
    }
  }
}

template <int EPI, int NB>
static void mxmm_launch(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws, uint8_t* hc,
                        uint8_t* hs, uint16_t* y, float* part, int M, int K, int Npk, int S, hipStream_t s) {
  const int tn = Npk / MxTile<NB>::BN, tm = (M + 127) / 128;
  hipLaunchKernelGGL((k_mxmm<EPI, NB>), dim3(tn * tm * S), dim3(256), 0, s, xc, xs, wc, ws, hc, hs, y, part, M, K,
                     Npk, tn, tm, S);
}

// Gate/up: Npk packed rows (2I gated, I plain), K = H; 4-bit h out (codes
// row-major [M][I/2], exponents in the prefill layout).  128 x 256 tiles.
hipError_t launch_mxmm_gateup(int act, const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws,
                              uint8_t* hc, uint8_t* hs, int M, int K, int Npk, hipStream_t s) {
  if (M < 1 || K % 512 || Npk % 256) return hipErrorInvalidValue;
  if (act == MX_GEGLU)
    mxmm_launch<MXM_GEGLU, 8>(xc, xs, wc, ws, hc, hs, nullptr, nullptr, M, K, Npk, 1, s);
  else if (act == MX_SWIGLU)
    mxmm_launch<MXM_SWIGLU, 8>(xc, xs, wc, ws, hc, hs, nullptr, nullptr, M, K, Npk, 1, s);
  else
    mxmm_launch<MXM_GELU, 8>(xc, xs, wc, ws, hc, hs, nullptr, nullptr, M, K, Npk, 1, s);
  return hipGetLastError();
}

// Down: N = H output columns, K = I; S splits (> 1: fp32 partials); column
// tiles of 32 * nb (nb 4 or 8).
hipError_t launch_mxmm_down(const uint8_t* hc, const uint8_t* hs, const uint8_t* wc, const uint8_t* ws, uint16_t* y,
                            float* part, int M, int K, int N, int S, int nb, hipStream_t s) {
  if (M < 1 || K % 512 || S < 1 || S > K / 128 || (nb != 4 && nb != 8) || N % (32 * nb)) return hipErrorInvalidValue;
  if (nb == 8)
    mxmm_launch<MXM_DOWN, 8>(hc, hs, wc, ws, nullptr, nullptr, y, part, M, K, N, S, s);
  else
    mxmm_launch<MXM_DOWN, 4>(hc, hs, wc, ws, nullptr, nullptr, y, part, M, K, N, S, s);
  return hipGetLastError();
}

}  // namespace frt
