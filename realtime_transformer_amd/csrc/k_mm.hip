// k_mm.hip -- the prefill-sized (M >= 128) FP8 GEMMs of the FFN block with
// fused epilogues, on the gfx950 f16 matrix cores.
//
// itsolotime article, section 7.2 (the encoder FFN loop): gate and up
// projections, a fused gating kernel that re-quantises its output, then the
// down projection back to the residual path; FlashRT architecture doc,
// component "Calibration": dequantisation by alpha = act_scale *
// weight_scale applied as host scalars.
//
//   gate/up : HQ[m][i] = e4m3(h * inv_h),  h = act(Ag*a_g) * (Au*a_u)
//             (non-gated: h = gelu_tanh(Au*a_u)),  A* = XQ[m] . W*[i]
//   down    : Y[m][n]  = bf16(Ad * a_d),   Ad = HQ[m] . Wd[n]
//             (or, split over K, fp32 partial sums that the consumer adds)
//
// Arithmetic: operands stay E4M3 bytes in HBM and LDS; each wave converts
// its fragments exactly to f16 (every E4M3 value is an f16 value) and runs
// v_mfma_f32_32x32x16_f16, which accumulates at fp32 accuracy.
//
// Data movement.  A workgroup owns BM activation rows x BN packed weight
// rows.  Per K stage (KS bytes of K) both operand tiles go HBM -> LDS with
// direct-to-LDS loads (global_load_lds_dwordx4: each lane's 16 bytes land at
// lane * 16 of a 1 KiB run), so staging costs no registers and no VALU.  The
// gather into those runs builds the 32-row fragment order of the 32x32x16
// MFMA: in a 32-row block, 1 KiB slice q holds for lane p the 16 bytes of
// row p % 32 at K offset (p / 32) * KS/2 + q * 16, so every ds_read_b128 of
// a wave reads one contiguous KiB (conflict-free) and each 16 bytes feed two
// MFMA steps.  Activations are gathered from row-major XQ/HQ, weights from
// the 16-row packed blocks (frt_device.h).  Stages form a ring of NS
// buffers; a wave waits only for its own loads of the stage it is about to
// read (s_waitcnt vmcnt(n)), then a barrier makes everyone's loads visible.
//
// Output fragment of the 32x32x16 MFMA (A operand = weight rows, B operand
// = activation rows): lane l, register r holds weight row
// 8*(r/4) + 4*(l/32) + r%4 and activation row l%32 of the tile.  A 32-row
// packed weight tile of the gated forms is one gate group and the matching
// up group, so gate (r < 8) and up (r + 8) of the same intermediate index sit
// in the same lane, and four consecutive indices (r%4) form one 32-bit store.
//
// Workgroup order: consecutive workgroups go to different XCDs (round
// robin over 8); work items are numbered so that the workgroups of one XCD
// share operands (all row tiles of a column tile, and one K split, run on one
// XCD, whose L2 then serves the weight tile and the activation rows to each
// of them).
#include "frt_device.h"
#include "frt_qkv_dev.h"

namespace frt {

// MM_QKV: the attention input's fused QKV projection with the split + rotary
// epilogue (frt_qkv_dev.h); its packed pairs hold rotation partners.
enum { MM_GEGLU = 0, MM_SWIGLU = 1, MM_GELU = 2, MM_DOWN = 3, MM_QKV = 4 };

template <int EPI>
__device__ __forceinline__ float mm_act(float g, float u) {
  if (EPI == MM_GELU) return gelu_tanh_f32(u);
  const float a = (EPI == MM_SWIGLU) ? silu_f32(g) : gelu_tanh_f32(g);
  return a * u;
}

// Direct-to-LDS 16-byte load: lane i's 16 bytes from g land at LDS byte
// m0 + 16 * i.  Issued from inline assembly so that the compiler does not
// track it as an LDS write: it would otherwise make every later LDS read
// wait for all outstanding loads (s_waitcnt vmcnt(0)), serialising the
// stage ring.  The kernel orders these loads itself: s_waitcnt vmcnt(n) on
// its own loads, then a workgroup barrier, before any wave reads the stage.
// (The s_nop covers the M0 write -> LDS-DMA read hazard.)
__device__ __forceinline__ void dma16(const uint8_t* g, const uint8_t* l) {
  const uint32_t m0 = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)l);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}

// s_waitcnt immediate for "vmcnt <= n" (other counters unconstrained); gfx9
// encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Barrier without the memory fence of __syncthreads: LDS written by this
// wave's direct loads is complete once vmcnt says so; the compiler-level
// memory clobbers keep LDS accesses on their side of the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ v8h cvt8_f16(uint32_t w0, uint32_t w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, true);
  v8h r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

template <int BM_, int BN_, int WA_, int WW_, int NS_, int MINB_ = 1>
struct MMCfg {
  static constexpr int BM = BM_, BN = BN_;   // activation rows, packed weight rows per workgroup
  static constexpr int WA = WA_, WW = WW_;   // waves along activations, along weights
  static constexpr int KS = 64;              // K bytes per stage
  static constexpr int NS = NS_;             // LDS stages (ring)
  static constexpr int MINB = MINB_;         // workgroups per CU the registers and LDS are sized for
  static constexpr int NW = WA * WW, NT = 64 * NW;
  static constexpr int TA = BM / 32 / WA;    // 32-row activation tiles per wave
  static constexpr int TW = BN / 32 / WW;    // 32-row weight tiles per wave
  static constexpr int A_CH = BM / 16;       // 1 KiB loads per stage: 16 activation rows each
  static constexpr int W_CH = BN / 16;       // ... and 16 weight rows each (two 1 KiB slices per 32 rows)
  static constexpr int ACPW = (A_CH + NW - 1) / NW;  // per wave (the last ones may repeat a load)
  static constexpr int WCPW = (W_CH + NW - 1) / NW;
  static constexpr int CPW = ACPW + WCPW;
  static constexpr int A_BYTES = BM * KS, STAGE_BYTES = (BM + BN) * KS;
  static_assert(BM % (32 * WA) == 0 && BN % (32 * WW) == 0, "whole 32-row tiles per wave");
  static_assert(NS >= 2 && NS <= 4 && MINB * NS * STAGE_BYTES <= 160 * 1024, "LDS");
  static_assert((NS - 2) * CPW < 64, "vmcnt range");
};

// One workgroup: tile (tn, tm) of the output, K stages [kb0, kb1) of 64 bytes.
//
// LDS per stage: activations row-major [BM][64] with the four 16-byte chunks
// of row R stored at chunk position c ^ ((R >> 2) & 3), then the weights in
// 32-row fragment order (1 KiB slice q of a 32-row block holds, for lane p,
// row p % 32 at stage K byte (p / 32) * 32 + q * 16).  A direct load of 16
// activation rows reads four whole 64-byte row segments per row group (the
// swizzle only permutes which lane fetches which chunk); the fragment read
// of lane l (row l % 32, chunk (l / 32) * 2 + q) then hits 16 distinct
// 16-byte bank groups per 16 lanes, i.e. it is conflict-free.
template <int EPI, class C, bool FP8>
__global__ __launch_bounds__(C::NT, C::MINB) void k_mm(const uint8_t* __restrict__ act, const uint8_t* __restrict__ wt,
                                              void* __restrict__ out, float* __restrict__ part, int M, int K,
                                              int Npk, int tiles_n, int tiles_m, int num_splits, float alpha_a,
                                              float alpha_b, float inv_out, const QkvOut qo) {
  constexpr int BM = C::BM, BN = C::BN, KS = C::KS, NS = C::NS, CPW = C::CPW;
  constexpr int TA = C::TA, TW = C::TW, NW = C::NW;
  constexpr bool GATED = EPI == MM_GEGLU || EPI == MM_SWIGLU;
  // one statically allocated array per stage: the compiler then knows that
  // reads of one stage do not alias the direct loads still filling another
  // and adds no wait for them
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[NS > 2 ? C::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[NS > 3 ? C::STAGE_BYTES : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wa = wave / C::WW, ww = wave % C::WW;

  // Work item of this workgroup: (split, column tile, row tile) numbered
  // split-major, then column, then row.  Consecutive workgroups go to
  // different XCDs (round robin over 8), so when the items divide evenly the
  // numbering gives XCD x the contiguous range [x * T/8, (x+1) * T/8): one
  // split, a few column tiles and all their row tiles share that XCD's L2
  // (the weight tile once per column tile, the activation rows once per
  // split).
  const int S = num_splits, T = tiles_n * tiles_m * S;
  int sp, tn, tm;
  {
    const int bid = blockIdx.x;
    const int idx = (T & 7) == 0 ? (bid & 7) * (T >> 3) + (bid >> 3) : bid;
    sp = idx / (tiles_n * tiles_m);
    const int rem = idx - sp * (tiles_n * tiles_m);
    tn = rem / tiles_m;
    tm = rem - tn * tiles_m;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int nst = K / KS;
  const int kb0 = sp * nst / S, kb1 = (sp + 1) * nst / S;
  const int KB = K >> 7;  // 128-byte K blocks of the packed weights

  // This wave's direct loads: activation run a = i * NW + wave (16 rows),
  // weight run w = i * NW + wave (one 1 KiB slice of a 32-row block); a
  // wave whose last run index passes the end repeats its previous run (same
  // bytes to the same place).  Per lane: 32-bit source offset at stage 0
  // and the wave-uniform LDS offset.
  uint32_t src[CPW], dst[CPW];
#pragma unroll
  for (int i = 0; i < C::ACPW; ++i) {
    int a = i * NW + wave;
    if (a >= C::A_CH) a -= NW;
    const int R = a * 16 + (lane >> 2);               // row inside the tile
    const int pos = lane & 3, c = pos ^ ((R >> 2) & 3);  // chunk this lane fetches
    int m = m0 + R;
    m = m < M ? m : M - 1;  // rows past M load row M-1; their outputs are not stored
    src[i] = (uint32_t)m * (uint32_t)K + (uint32_t)(c * 16);
    dst[i] = (uint32_t)(a * 1024);
  }
#pragma unroll
  for (int i = 0; i < C::WCPW; ++i) {
    int w = i * NW + wave;
    if (w >= C::W_CH) w -= NW;
    const int blk = w >> 1, q = w & 1;
    const int r = lane & 31;
    const int g = (n0 + blk * 32) / 16 + (r >> 4);
    const int kk = (lane >> 5) * 32 + q * 16;  // K byte inside the stage (stage 0: packed block 0)
    src[C::ACPW + i] = (uint32_t)g * (uint32_t)KB * 2048u +
                       (uint32_t)(((kk & 31) >> 4) * 1024 + ((r & 15) + 16 * (kk >> 5)) * 16);
    dst[C::ACPW + i] = (uint32_t)(C::A_BYTES + w * 1024);
  }

  // stage kb: activations advance by 64 bytes; weights by (kb/2) packed
  // blocks plus (kb%2) * 64 bytes (two 32-byte chunks of 256 bytes each)
  auto issue = [&](int kb, uint8_t* base) {
    const uint32_t a_off = (uint32_t)kb * KS;
    const uint32_t w_off = (uint32_t)(kb >> 1) * 2048u + (uint32_t)(kb & 1) * 512u;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      if (i < C::ACPW) dma16(act + (src[i] + a_off), base + dst[i]);
      else dma16(wt + (src[i] + w_off), base + dst[i]);
    }
  };

  v16f acc[TW][TA];
#pragma unroll
  for (int j = 0; j < TW; ++j)
#pragma unroll
    for (int i = 0; i < TA; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  // per-lane LDS read offsets: activation row l % 32 of each tile, chunk
  // (l / 32) * 2 + q at its swizzled position; weights in fragment order
  const int rr = lane & 31;
  const int a_rd0 = (wa * TA * 32 + rr) * 64 + 16 * ((((lane >> 5) * 2) + 0) ^ ((rr >> 2) & 3));
  const int a_rd1 = (wa * TA * 32 + rr) * 64 + 16 * ((((lane >> 5) * 2) + 1) ^ ((rr >> 2) & 3));
  const int w_rd = C::A_BYTES + (ww * TW) * 2048 + lane * 16;

  // a stage's fragments of this wave, both 16-byte K slices, in registers
  typedef int v4i __attribute__((ext_vector_type(4)));
  struct Frag {
    v4i a[2][TA], w[2][TW];
  };
  auto read_stage = [&](const uint8_t* base, Frag& f) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int i = 0; i < TA; ++i)
        f.a[q][i] = *reinterpret_cast<const v4i*>(base + (q ? a_rd1 : a_rd0) + i * 32 * 64);
#pragma unroll
      for (int j = 0; j < TW; ++j) f.w[q][j] = *reinterpret_cast<const v4i*>(base + w_rd + j * 2048 + q * 1024);
    }
  };
  auto mma_stage = [&](const Frag& f) {
    if (FP8) {
      // one 32x32x64 FP8 step per tile pair: the lane's 32 bytes (both
      // slices) are exactly the operand of v_mfma_scale_f32_32x32x64_f8f6f4
      // (row l % 32, K bytes (l / 32) * 32 + [0, 32)); unit scales
      v8i xa[TA], xw[TW];
#pragma unroll
      for (int i = 0; i < TA; ++i) xa[i] = __builtin_shufflevector(f.a[0][i], f.a[1][i], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int j = 0; j < TW; ++j) xw[j] = __builtin_shufflevector(f.w[0][j], f.w[1][j], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int j = 0; j < TW; ++j)
#pragma unroll
        for (int i = 0; i < TA; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xw[j], xa[i], acc[j][i], 0, 0, 0, 0, 0, 0);
      return;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v8h xa[TA], xw[TW];
#pragma unroll
        for (int i = 0; i < TA; ++i)
          xa[i] = h ? cvt8_f16(f.a[q][i][2], f.a[q][i][3]) : cvt8_f16(f.a[q][i][0], f.a[q][i][1]);
#pragma unroll
        for (int j = 0; j < TW; ++j)
          xw[j] = h ? cvt8_f16(f.w[q][j][2], f.w[q][j][3]) : cvt8_f16(f.w[q][j][0], f.w[q][j][1]);
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
          for (int i = 0; i < TA; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xw[j], xa[i], acc[j][i], 0, 0, 0);
      }
    }
  };

  // Ring of NS stages.  Each wave holds the fragments of the stage it is
  // multiplying in registers, so a buffer is free as soon as every wave has
  // read it: at step t the wave waits for its loads of stage t + 1, meets the
  // others at the barrier (after which stage t + 1 is complete and buffer
  // t % NS is free), refills buffer t % NS with stage t + NS, reads stage
  // t + 1 into registers and multiplies stage t meanwhile, so the LDS latency
  // and the barrier overlap the MFMAs.  The loop is unrolled by NS so every
  // buffer is named statically, with a straight-line body (a conditional
  // step inside it makes the compiler shuttle accumulators between register
  // files); the tail follows it.
  const int nk = kb1 - kb0;
  issue(kb0, lds0);
  if (nk > 1) issue(kb0 + 1, lds1);
  if (NS > 2 && nk > 2) issue(kb0 + 2, lds2);
  if (NS > 3 && nk > 3) issue(kb0 + 3, lds3);
  Frag fa, fb;  // stage fragments, alternating between two register sets
  {
    // stage 0 complete: at most min(nk - 1, NS - 1) later stages outstanding
    const int after = (nk - 1) < (NS - 1) ? (nk - 1) : (NS - 1);
    if (NS > 3 && after >= 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * CPW));
    else if (NS > 2 && after >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * CPW));
    else if (after >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(CPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    read_stage(lds0, fa);
  }
  // before step t: this wave's loads of stage t + 1 are complete once at most
  // min(nk - 2 - t, NS - 2) later stages of its loads are outstanding, and
  // its reads of stage t must have returned before anyone refills buffer t
  auto sync_next = [&](int t) {
    const int after = (nk - 2 - t) < (NS - 2) ? (nk - 2 - t) : (NS - 2);
    if (NS > 3 && after >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * CPW));
    else if (NS > 2 && after >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(CPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    lds_barrier();
  };
  // step t: FC holds stage t (reads issued); NEXT is the buffer of stage
  // t + 1, read into FN while FC is multiplied (the scheduling barrier keeps
  // those reads ahead of the MFMAs, so their latency overlaps them).  A
  // macro rather than a lambda: fragment sets passed by reference end up in
  // scratch memory.
#define FRT_MM_STEP(t, CUR, NEXT, FC, FN)            \
  do {                                               \
    if ((t) + 1 < nk) {                              \
      sync_next(t);                                  \
      if ((t) + NS < nk) issue(kb0 + (t) + NS, CUR); \
      read_stage(NEXT, FN);                          \
      __builtin_amdgcn_sched_barrier(0);             \
    }                                                \
    mma_stage(FC);                                   \
  } while (0)
  int t = 0;
  if (NS == 2) {
    for (; t + 1 < nk; t += 2) {
      FRT_MM_STEP(t, lds0, lds1, fa, fb);
      FRT_MM_STEP(t + 1, lds1, lds0, fb, fa);
    }
    if (t < nk) FRT_MM_STEP(t, lds0, lds1, fa, fb);
  } else if (NS == 3) {
    // period 6: three buffers x two register sets
    for (; t + 5 < nk; t += 6) {
      FRT_MM_STEP(t, lds0, lds1, fa, fb);
      FRT_MM_STEP(t + 1, lds1, lds2, fb, fa);
      FRT_MM_STEP(t + 2, lds2, lds0, fa, fb);
      FRT_MM_STEP(t + 3, lds0, lds1, fb, fa);
      FRT_MM_STEP(t + 4, lds1, lds2, fa, fb);
      FRT_MM_STEP(t + 5, lds2, lds0, fb, fa);
    }
    if (t < nk) FRT_MM_STEP(t, lds0, lds1, fa, fb);
    if (t + 1 < nk) FRT_MM_STEP(t + 1, lds1, lds2, fb, fa);
    if (t + 2 < nk) FRT_MM_STEP(t + 2, lds2, lds0, fa, fb);
    if (t + 3 < nk) FRT_MM_STEP(t + 3, lds0, lds1, fb, fa);
    if (t + 4 < nk) FRT_MM_STEP(t + 4, lds1, lds2, fa, fb);
  } else {
    for (; t + 3 < nk; t += 4) {
      FRT_MM_STEP(t, lds0, lds1, fa, fb);
      FRT_MM_STEP(t + 1, lds1, lds2, fb, fa);
      FRT_MM_STEP(t + 2, lds2, lds3, fa, fb);
      FRT_MM_STEP(t + 3, lds3, lds0, fb, fa);
    }
    if (t < nk) FRT_MM_STEP(t, lds0, lds1, fa, fb);
    if (t + 1 < nk) FRT_MM_STEP(t + 1, lds1, lds2, fb, fa);
    if (t + 2 < nk) FRT_MM_STEP(t + 2, lds2, lds3, fa, fb);
  }
#undef FRT_MM_STEP

  // ---- epilogue ----
  const int col = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < TA; ++i) {
    const int m = m0 + (wa * TA + i) * 32 + col;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int nt = n0 + (ww * TW + j) * 32;  // first packed row of the tile
      if (EPI == MM_DOWN) {
        const int N = Npk;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int n = nt + 8 * g4 + 4 * hi;
          const float a0 = acc[j][i][4 * g4], a1 = acc[j][i][4 * g4 + 1];
          const float a2 = acc[j][i][4 * g4 + 2], a3 = acc[j][i][4 * g4 + 3];
          if (S == 1) {
            uint16_t* y = reinterpret_cast<uint16_t*>(out);
            const uint2 v = make_uint2(pack_bf16x2(a0 * alpha_a, a1 * alpha_a), pack_bf16x2(a2 * alpha_a, a3 * alpha_a));
            *reinterpret_cast<uint2*>(y + (size_t)m * N + n) = v;
          } else {
            float* ps = part + (size_t)sp * M * N;
            *reinterpret_cast<float4*>(ps + (size_t)m * N + n) = make_float4(a0, a1, a2, a3);
          }
        }
      } else if (EPI == MM_QKV) {
        // the tile is one pair: lane row rho = 8 g4 + 4 hi + r of both groups
#pragma unroll
        for (int g4 = 0; g4 < 2; ++g4) {
          float f[4], g[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            f[r] = acc[j][i][4 * g4 + r];
            g[r] = acc[j][i][8 + 4 * g4 + r];
          }
          qkv_store4(qo, m, nt / 32, 8 * g4 + 4 * hi, f, g);
        }
      } else if (GATED) {
        const int I = Npk / 2;
        const int i0 = nt / 2;  // intermediate index of the tile's gate group
        uint8_t* hq = reinterpret_cast<uint8_t*>(out) + (size_t)m * I + i0;
#pragma unroll
        for (int g4 = 0; g4 < 2; ++g4) {
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            h[r] = mm_act<EPI>(acc[j][i][4 * g4 + r] * alpha_a, acc[j][i][8 + 4 * g4 + r] * alpha_b);
          *reinterpret_cast<uint32_t*>(hq + 8 * g4 + 4 * hi) =
              e4m3x4(h[0] * inv_out, h[1] * inv_out, h[2] * inv_out, h[3] * inv_out);
        }
      } else {
        const int I = Npk;
        uint8_t* hq = reinterpret_cast<uint8_t*>(out) + (size_t)m * I + nt;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = mm_act<EPI>(0.0f, acc[j][i][4 * g4 + r] * alpha_b);
          *reinterpret_cast<uint32_t*>(hq + 8 * g4 + 4 * hi) =
              e4m3x4(h[0] * inv_out, h[1] * inv_out, h[2] * inv_out, h[3] * inv_out);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// configurations and launchers
// ---------------------------------------------------------------------------
//   0: BM 224 x BN 256, waves 1 x 4 (wave tile 224 x 64), 4 stages   M ~ 800 gate/up
//   1: BM 256 x BN 224, waves 4 x 1 (wave tile  64 x 224), 4 stages  large M, N % 224 == 0
//   2: BM 256 x BN 192, waves 2 x 2 (wave tile 128 x 96), 4 stages   large M, N % 192 == 0
//   3: BM 128 x BN 256, waves 2 x 2 (wave tile  64 x 128), 4 stages  generic
//   4: BM 256 x BN 256, waves 2 x 2 (wave tile 128 x 128), 4 stages  generic, large
//   5: BM 128 x BN 128, waves 2 x 2 (wave tile  64 x 64), 4 stages   small grids
//   6: BM  64 x BN 128, waves 2 x 2 (wave tile  32 x 64), 4 stages   QKV only
//   7: BM 128 x BN  64, waves 2 x 2 (wave tile  64 x 32), 4 stages   QKV only
//   8: BM 128 x BN 256, waves 2 x 2 (wave tile  64 x 128), 3 stages, two workgroups per CU
//   9: BM 256 x BN 192, waves 4 x 2 (wave tile  64 x  96), 4 stages, eight waves (f16 cores only)
using MMC0 = MMCfg<224, 256, 1, 4, 4>;
using MMC1 = MMCfg<256, 224, 4, 1, 4>;
using MMC2 = MMCfg<256, 192, 2, 2, 4>;
using MMC3 = MMCfg<128, 256, 2, 2, 4>;
using MMC4 = MMCfg<256, 256, 2, 2, 4>;
using MMC5 = MMCfg<128, 128, 2, 2, 4>;
// small tiles for short outputs (the attention input's fused QKV): more
// workgroups than CUs where 128 x 128 tiles would leave part of the chip idle
using MMC6 = MMCfg<64, 128, 2, 2, 4>;
using MMC7 = MMCfg<128, 64, 2, 2, 4>;
// 128 x 256 on a 3-stage ring, registers and LDS sized for two workgroups
// per CU (two waves per SIMD, so one wave's LDS reads, conversions and
// barrier waits overlap the other's matrix instructions)
using MMC8 = MMCfg<128, 256, 2, 2, 3, 2>;
// 256 x 192 with eight waves (two per SIMD, so one wave's conversions and
// LDS reads run while the other's matrix instructions do; wave tiles 64 x
// 96): on the f16 cores it replaces configuration 2 (measured on the M=4096
// down GEMM: 271-273 against 280-283 us; 256 x 256 eight-wave tiles were
// level or slower where their grid leaves CUs idle)
using MMC9 = MMCfg<256, 192, 4, 2, 4>;
constexpr int kMMConfigs = 10;

static const int kMM_BM[kMMConfigs] = {MMC0::BM, MMC1::BM, MMC2::BM, MMC3::BM, MMC4::BM,
                                       MMC5::BM, MMC6::BM, MMC7::BM, MMC8::BM, MMC9::BM};
static const int kMM_BN[kMMConfigs] = {MMC0::BN, MMC1::BN, MMC2::BN, MMC3::BN, MMC4::BN,
                                       MMC5::BN, MMC6::BN, MMC7::BN, MMC8::BN, MMC9::BN};
static const int kMM_KS[kMMConfigs] = {MMC0::KS, MMC1::KS, MMC2::KS, MMC3::KS, MMC4::KS,
                                       MMC5::KS, MMC6::KS, MMC7::KS, MMC8::KS, MMC9::KS};

int mm_config_bm(int c) { return (c >= 0 && c < kMMConfigs) ? kMM_BM[c] : 0; }
int mm_config_bn(int c) { return (c >= 0 && c < kMMConfigs) ? kMM_BN[c] : 0; }
int mm_config_ks(int c) { return (c >= 0 && c < kMMConfigs) ? kMM_KS[c] : 0; }

template <int EPI, class C, bool FP8>
static hipError_t mm_launch(const uint8_t* act, const uint8_t* w, void* out, float* part, int M, int K, int Npk,
                            int S, float a, float b, float inv, hipStream_t s, const QkvOut& qo) {
  if (Npk % C::BN || K % C::KS || S < 1 || S > K / C::KS) return hipErrorInvalidValue;
  const int tiles_n = Npk / C::BN, tiles_m = (M + C::BM - 1) / C::BM;
  hipLaunchKernelGGL((k_mm<EPI, C, FP8>), dim3(tiles_n * tiles_m * S), dim3(C::NT), 0, s, act, w, out, part, M, K,
                     Npk, tiles_n, tiles_m, S, a, b, inv, qo);
  return hipGetLastError();
}

template <int EPI, bool FP8>
static hipError_t mm_cfg(int cfg, const uint8_t* act, const uint8_t* w, void* out, float* part, int M, int K,
                         int Npk, int S, float a, float b, float inv, hipStream_t s, const QkvOut& qo = QkvOut{}) {
  switch (cfg) {
    case 0: return mm_launch<EPI, MMC0, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
    case 1: return mm_launch<EPI, MMC1, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
    case 2: return mm_launch<EPI, MMC2, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
    case 3: return mm_launch<EPI, MMC3, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
    case 4: return mm_launch<EPI, MMC4, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
    case 5: return mm_launch<EPI, MMC5, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
    case 6:
      if constexpr (EPI == MM_QKV) return mm_launch<EPI, MMC6, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
      return hipErrorInvalidValue;
    case 7:
      if constexpr (EPI == MM_QKV) return mm_launch<EPI, MMC7, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
      return hipErrorInvalidValue;
    case 8:
      if constexpr (EPI != MM_QKV) return mm_launch<EPI, MMC8, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
      return hipErrorInvalidValue;
    case 9:
      if constexpr (EPI != MM_QKV && !FP8)
        return mm_launch<EPI, MMC9, FP8>(act, w, out, part, M, K, Npk, S, a, b, inv, s, qo);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// Gate/up GEMM (act: 0 GeGLU, 1 SwiGLU, 2 non-gated GELU), E4M3 output.
// fp8: the products run on the FP8 matrix cores instead of the f16 ones.
hipError_t launch_mm_gateup(int act, int cfg, bool fp8, const uint8_t* xq, const uint8_t* w, uint8_t* hq, int M,
                            int K, int Npk, float alpha_g, float alpha_u, float inv_h, hipStream_t s) {
  const float a = alpha_g, b = alpha_u;
  if (fp8) {
    if (act == MM_GEGLU) return mm_cfg<MM_GEGLU, true>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
    if (act == MM_SWIGLU) return mm_cfg<MM_SWIGLU, true>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
    return mm_cfg<MM_GELU, true>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
  }
  if (act == MM_GEGLU) return mm_cfg<MM_GEGLU, false>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
  if (act == MM_SWIGLU) return mm_cfg<MM_SWIGLU, false>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
  return mm_cfg<MM_GELU, false>(cfg, xq, w, hq, nullptr, M, K, Npk, 1, a, b, inv_h, s);
}

// Down GEMM: S == 1 writes bf16 Y; S > 1 writes fp32 partials [S][M][N] to
// part (summed in split order by the consumer).
hipError_t launch_mm_down(int cfg, bool fp8, const uint8_t* hq, const uint8_t* w, uint16_t* y, float* part, int M,
                          int K, int N, int S, float alpha_d, hipStream_t s) {
  if (fp8) return mm_cfg<MM_DOWN, true>(cfg, hq, w, y, part, M, K, N, S, alpha_d, 0.0f, 0.0f, s);
  return mm_cfg<MM_DOWN, false>(cfg, hq, w, y, part, M, K, N, S, alpha_d, 0.0f, 0.0f, s);
}

// Fused QKV projection (attention input) with the split + rotary epilogue:
// Npk = (nq + 2 nkv) hd packed rows, no K split (the rotation needs whole sums).
hipError_t launch_mm_qkv(int cfg, const uint8_t* xq, const uint8_t* w, const QkvOut& o, int M, int K, int Npk,
                         hipStream_t s) {
  return mm_cfg<MM_QKV, false>(cfg, xq, w, nullptr, nullptr, M, K, Npk, 1, 0.0f, 0.0f, 0.0f, s, o);
}

}  // namespace frt
