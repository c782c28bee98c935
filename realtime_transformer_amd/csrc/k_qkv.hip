// k_qkv.hip -- attention-input kernels: the rotary table, the packing of the
// fused QKV weight, and the fused QKV GEMV (M <= 64) with the split + rotary
// epilogue.
//
// FlashRT architecture doc, "Kernel library" (the "qkv split + RoPE" fusion
// after the QKV projection); itsolotime article section 5.2 (the FusedQKV
// weight: q, k, v rows fused, quantised with one scale, head interleave).
//
// The GEMV streams the packed weight exactly as the FFN's gate/up GEMV does
// (one workgroup per pair of 16-row groups, waves splitting K, each weight
// fragment converted to f16 once and multiplied into ceil(M/16) activation
// tiles, partials meeting in LDS in wave order); only the epilogue differs.
// Bound: HBM (N*H weight bytes per launch), latency at small N.
#include "frt_qkv_dev.h"
#include "frt_normq.h"

namespace frt {

// Rotary table entry (p, i) = (f32(cos(p * theta_i)), f32(sin(p * theta_i))),
// theta_i = base^(-2i/hd), all in fp64 and rounded once.
__global__ __launch_bounds__(256) void k_rope_table(float2* __restrict__ out, int P, int half, int hd,
                                                    double base) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)P * half) return;
  const int i = (int)(idx % (size_t)half);
  const int p = (int)(idx / (size_t)half);
  const double theta = pow(base, -(2.0 * (double)i) / (double)hd);
  const double a = (double)p * theta;
  out[idx] = make_float2((float)cos(a), (float)sin(a));
}

hipError_t launch_rope_table(float2* out, int P, int hd, double base, hipStream_t s) {
  const size_t n = (size_t)P * (hd / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, out, P, hd / 2, hd, base);
  return hipGetLastError();
}

// Quantise one of the three source matrices (rows [row_base, row_base +
// nrows) of the fused weight, [nrows][K] bf16, times colw[k] when given) with
// factor inv into the packed layout (frt_qkv_dev.h).  One thread per 16
// consecutive K values of a row.
__global__ __launch_bounds__(256) void k_quant_pack_qkv(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                        int nrows, int K, float inv, int row_base, int hd, int n_rope,
                                                        const uint16_t* __restrict__ colw, int oct) {
  const size_t pieces_per_row = (size_t)K / 16;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)nrows * pieces_per_row) return;
  const int n = (int)(idx / pieces_per_row);
  const int k0 = (int)(idx % pieces_per_row) * 16;
  const uint4* sp = reinterpret_cast<const uint4*>(src + (size_t)n * K + k0);
  const uint4 a = sp[0], b = sp[1];
  const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = 0x3F803F80u;  // bf16 1.0 pairs
  if (colw) {
    const uint4* cp = reinterpret_cast<const uint4*>(colw + k0);
    const uint4 c0 = cp[0], c1 = cp[1];
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
  }
  uint32_t q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    q[j] = e4m3x4((bf16_lo(v[2 * j]) * bf16_lo(c[2 * j])) * inv, (bf16_hi(v[2 * j]) * bf16_hi(c[2 * j])) * inv,
                  (bf16_lo(v[2 * j + 1]) * bf16_lo(c[2 * j + 1])) * inv,
                  (bf16_hi(v[2 * j + 1]) * bf16_hi(c[2 * j + 1])) * inv);
  const uint32_t prow = oct ? qkv_packed_row_oct((uint32_t)(row_base + n), (uint32_t)hd, (uint32_t)n_rope)
                            : qkv_packed_row((uint32_t)(row_base + n), (uint32_t)hd, (uint32_t)n_rope);
  *reinterpret_cast<uint4*>(dst + packed_offset(prow, (uint32_t)k0, (uint32_t)K)) = make_uint4(q[0], q[1], q[2], q[3]);
}

hipError_t launch_quant_pack_qkv(const uint16_t* src, uint8_t* dst, int nrows, int K, float inv, int row_base,
                                 int hd, int n_rope, const uint16_t* colw, hipStream_t s, int oct) {
  const size_t pieces = (size_t)nrows * (K / 16);
  if (pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_pack_qkv, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, src, dst, nrows, K,
                     inv, row_base, hd, n_rope, colw, oct);
  return hipGetLastError();
}

typedef unsigned v4u_q __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void qkv_load_w32(const uint8_t* wp, int kb, uint32_t o[8]) {
  const v4u_q a = __builtin_nontemporal_load(reinterpret_cast<const v4u_q*>(wp + (size_t)kb * 2048));
  const v4u_q b = __builtin_nontemporal_load(reinterpret_cast<const v4u_q*>(wp + (size_t)kb * 2048 + 1024));
  o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
  o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
}
__device__ __forceinline__ void qkv_load_x32(const uint8_t* xr, bool has_row, int kb, uint32_t o[8]) {
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (has_row) {
    a = *reinterpret_cast<const uint4*>(xr + kb * 128);
    b = *reinterpret_cast<const uint4*>(xr + kb * 128 + 16);
  }
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// One workgroup of W waves per pair p of 16-row groups; MT activation tiles.
// PIPE: one K block per step over two register sets, the next block's
// weight and activation loads issued before the current block's MFMAs (as
// the FFN decode GEMVs do), every load unconditional (rows past M read row
// 0, whose products reach only output rows past M, never stored).
template <int W, int MT, bool PIPE, bool OCT = false>
__global__ __launch_bounds__(W * 64) void k_gemv_qkv(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ w,
                                                     const QkvOut o, int M, int K) {
  static_assert(W >= MT, "one wave per tile finishes the epilogue");
  __shared__ v4f red[W][MT][2][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = blockIdx.x;
  const int KB = K >> 7;
  const int kb0 = wave * KB / W, kb1 = (wave + 1) * KB / W;
  const int row = lane & 15, q = lane >> 4;
  const uint8_t* w1 = w + (size_t)(OCT ? p : 2 * p) * KB * 2048 + lane * 16;
  const uint8_t* w2 = w + (size_t)(OCT ? p : 2 * p + 1) * KB * 2048 + lane * 16;
  const uint8_t* xr[MT];
  bool has[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    has[t] = 16 * t + row < M;
    xr[t] = xq + (size_t)(has[t] ? 16 * t + row : 0) * K + q * 32;
  }
  v4f acc1[MT], acc2[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc1[t] = acc2[t] = v4f{0, 0, 0, 0};

  if (PIPE) {
    const int nblk = kb1 - kb0;
    typedef uint32_t Frag[8];
    Frag aA, bA, aB, bB, xA[MT], xB[MT];
    auto load_step = [&](Frag& a, Frag& b, Frag (&x)[MT], int i) {
      const int kb = kb0 + (i < nblk ? i : nblk - 1);
      qkv_load_w32(w1, kb, a);
      if (!OCT) qkv_load_w32(w2, kb, b);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint4 lo = *reinterpret_cast<const uint4*>(xr[t] + kb * 128);
        const uint4 hi = *reinterpret_cast<const uint4*>(xr[t] + kb * 128 + 16);
        x[t][0] = lo.x; x[t][1] = lo.y; x[t][2] = lo.z; x[t][3] = lo.w;
        x[t][4] = hi.x; x[t][5] = hi.y; x[t][6] = hi.z; x[t][7] = hi.w;
      }
    };
    auto mma_step = [&](Frag& a, Frag& b, Frag (&x)[MT]) {
      // the step's operands count as written here, so the compiler cannot
      // convert them early (which would wait for every later load as well)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        asm volatile("" : "+v"(a[j]));
        if (!OCT) asm volatile("" : "+v"(b[j]));
#pragma unroll
        for (int t = 0; t < MT; ++t) asm volatile("" : "+v"(x[t][j]));
      }
      v8h ah[4], bh[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        ah[s4] = e4m3x8_to_f16(a[2 * s4], a[2 * s4 + 1]);
        if (!OCT) bh[s4] = e4m3x8_to_f16(b[2 * s4], b[2 * s4 + 1]);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const v8h xh = e4m3x8_to_f16(x[t][2 * s4], x[t][2 * s4 + 1]);
          acc1[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, ah[s4], acc1[t], 0, 0, 0);
          if (!OCT) acc2[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, bh[s4], acc2[t], 0, 0, 0);
        }
    };
    if (nblk > 0) {
      load_step(aA, bA, xA, 0);
      int i = 0;
      for (; i + 2 < nblk; i += 2) {
        load_step(aB, bB, xB, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(aA, bA, xA);
        load_step(aA, bA, xA, i + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(aB, bB, xB);
      }
      if (i + 1 < nblk) {
        load_step(aB, bB, xB, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_step(aA, bA, xA);
        mma_step(aB, bB, xB);
      } else {
        mma_step(aA, bA, xA);
      }
    }
  }
  for (int kb = kb0; !PIPE && kb < kb1; kb += 2) {
    const bool two = kb + 1 < kb1;
    uint32_t a0[8], a1[8], b0[8], b1[8], x0[MT][8], x1[MT][8];
    qkv_load_w32(w1, kb, a0);
    qkv_load_w32(w2, kb, b0);
    if (two) {
      qkv_load_w32(w1, kb + 1, a1);
      qkv_load_w32(w2, kb + 1, b1);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      qkv_load_x32(xr[t], has[t], kb, x0[t]);
      qkv_load_x32(xr[t], has[t] && two, kb + (two ? 1 : 0), x1[t]);
    }
    v8h ah[4], bh[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      ah[s4] = e4m3x8_to_f16(a0[2 * s4], a0[2 * s4 + 1]);
      bh[s4] = e4m3x8_to_f16(b0[2 * s4], b0[2 * s4 + 1]);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const v8h xh = e4m3x8_to_f16(x0[t][2 * s4], x0[t][2 * s4 + 1]);
        acc1[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, ah[s4], acc1[t], 0, 0, 0);
        acc2[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, bh[s4], acc2[t], 0, 0, 0);
      }
    if (two) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        ah[s4] = e4m3x8_to_f16(a1[2 * s4], a1[2 * s4 + 1]);
        bh[s4] = e4m3x8_to_f16(b1[2 * s4], b1[2 * s4 + 1]);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const v8h xh = e4m3x8_to_f16(x1[t][2 * s4], x1[t][2 * s4 + 1]);
          acc1[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, ah[s4], acc1[t], 0, 0, 0);
          acc2[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, bh[s4], acc2[t], 0, 0, 0);
        }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    red[wave][t][0][lane] = acc1[t];
    red[wave][t][1][lane] = acc2[t];
  }
  __syncthreads();
  if (wave >= MT) return;
  const int t = wave;
  v4f f = red[0][t][0][lane], g = red[0][t][1][lane];
#pragma unroll
  for (int v = 1; v < W; ++v) {
    f += red[v][t][0][lane];
    g += red[v][t][1][lane];
  }
  // lane holds rows m = 16t + 4q + r of lane row `row` in both groups (OCT:
  // of the one group, its rotation partner in lane row `row` ^ 8)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 16 * t + 4 * q + r;
    if (OCT) {
      const float partner = __shfl(f[r], lane ^ 8, 64);
      if (m < M) qkv_store_oct(o, m, p, row, f[r], partner);
    } else if (m < M) {
      qkv_store(o, m, p, row, f[r], g[r]);
    }
  }
}

// Decode form (M <= 16) after the split norm's slice-sum kernel: each wave
// quantises the activations of its own K blocks into a wave-private LDS row
// buffer (frt_normq.h) between issuing its first weight loads and using
// them, then multiplies as k_gemv_qkv with one activation tile; workgroup 0
// stores XQ.
constexpr int kQkvNqChunks = 3;  // 8-element chunks per lane loaded together (a 10-block range: 160 chunks)

template <int W>
__global__ __launch_bounds__(W * 64) void k_gemv_qkv_nq(const NormQ nq, const uint8_t* __restrict__ w, const QkvOut o,
                                                        int M, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xrow[];  // [M][K] E4M3
  __shared__ v4f red[W][2][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const int KB = K >> 7;
  const int kb0 = wave * KB / W, kb1 = (wave + 1) * KB / W;  // kb1 > kb0: W <= K / 128
  const int row = lane & 15, q = lane >> 4;
  const bool has = row < M;
  const uint8_t* w1 = w + (size_t)(2 * p) * KB * 2048 + lane * 16;
  const uint8_t* w2 = w + (size_t)(2 * p + 1) * KB * 2048 + lane * 16;

  NormQWave<kQkvNqChunks> nqw;
  nqw.init(nq, M, K, kb0, kb1, lane);
  nqw.load(nq, 0, lane);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t a0[8], a1[8], b0[8], b1[8];
  {
    const int kb_b = kb0 + 1 < kb1 ? kb0 + 1 : kb0;  // a one-block range loads its block twice
    qkv_load_w32(w1, kb0, a0);
    qkv_load_w32(w2, kb0, b0);
    qkv_load_w32(w1, kb_b, a1);
    qkv_load_w32(w2, kb_b, b1);
  }
  __builtin_amdgcn_sched_barrier(0);
  const float inv_rms = nqw.inv_rms(nq, lane);
  const bool store_xq = blockIdx.x == 0;
  nqw.quant(nq, 0, lane, inv_rms, xrow, store_xq);
  for (int c0 = kQkvNqChunks * 64; c0 < nqw.nch; c0 += kQkvNqChunks * 64) {
    nqw.load(nq, c0, lane);
    nqw.quant(nq, c0, lane, inv_rms, xrow, store_xq);
  }
  wave_lds_sync();

  auto lds_x32 = [&](int kb, uint32_t x[8]) {
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (has) {
      const uint8_t* xp = xrow + (size_t)row * K + kb * 128 + q * 32;
      a = *reinterpret_cast<const uint4*>(xp);
      b = *reinterpret_cast<const uint4*>(xp + 16);
    }
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  };
  v4f acc1 = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
  auto mma = [&](const uint32_t x[8], const uint32_t wa[8], const uint32_t wb[8]) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const v8h xh = e4m3x8_to_f16(x[2 * s4], x[2 * s4 + 1]);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, e4m3x8_to_f16(wa[2 * s4], wa[2 * s4 + 1]), acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, e4m3x8_to_f16(wb[2 * s4], wb[2 * s4 + 1]), acc2, 0, 0, 0);
    }
  };
  for (int kb = kb0; kb < kb1; kb += 2) {
    const bool two = kb + 1 < kb1;
    if (kb != kb0) {
      qkv_load_w32(w1, kb, a0);
      qkv_load_w32(w2, kb, b0);
      if (two) {
        qkv_load_w32(w1, kb + 1, a1);
        qkv_load_w32(w2, kb + 1, b1);
      }
    }
    uint32_t x0[8], x1[8];
    lds_x32(kb, x0);
    mma(x0, a0, b0);
    if (two) {
      lds_x32(kb + 1, x1);
      mma(x1, a1, b1);
    }
  }
  red[wave][0][lane] = acc1;
  red[wave][1][lane] = acc2;
  __syncthreads();
  if (wave != 0) return;
  v4f f = red[0][0][lane], g = red[0][1][lane];
#pragma unroll
  for (int v = 1; v < W; ++v) {
    f += red[v][0][lane];
    g += red[v][1][lane];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * q + r;
    if (m < M) qkv_store(o, m, p, row, f[r], g[r]);
  }
}

bool gemv_qkv_nq_supported(int M, int K, int G) { return normq_shape_ok(M, K, G); }

// M <= 16 after k_add_sumsq; W in {4, 8, 16}, at most K / 128.
hipError_t launch_gemv_qkv_nq(const uint16_t* r, const uint16_t* w_norm, const double* sq, int G, float eps,
                              float inv_x, uint8_t* xq_out, const uint8_t* w, const QkvOut& o, int M, int K, int W,
                              hipStream_t s) {
  if (!normq_shape_ok(M, K, G) || W > K / 128) return hipErrorInvalidValue;
  const NormQ nq{r, w_norm, sq, G, eps, inv_x, xq_out};
  const int pairs = (o.nq + 2 * o.nkv) * o.hd / 32;
  const size_t lds = (size_t)M * K;
  switch (W) {
    case 4: hipLaunchKernelGGL((k_gemv_qkv_nq<4>), dim3(pairs), dim3(256), lds, s, nq, w, o, M, K); break;
    case 8: hipLaunchKernelGGL((k_gemv_qkv_nq<8>), dim3(pairs), dim3(512), lds, s, nq, w, o, M, K); break;
    case 16: hipLaunchKernelGGL((k_gemv_qkv_nq<16>), dim3(pairs), dim3(1024), lds, s, nq, w, o, M, K); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// (W = 16 only with MT <= 2: the reduction buffer is W * MT * 2 KiB of LDS)
// FRT_QKV_GEMV_PIPE=0 keeps the unpipelined stream
template <int W, int MT>
static hipError_t gemv_qkv_t(const uint8_t* xq, const uint8_t* w, const QkvOut& o, int M, int K, int pairs,
                             hipStream_t s, bool oct) {
  const char* e = getenv("FRT_QKV_GEMV_PIPE");
  if (oct)
    hipLaunchKernelGGL((k_gemv_qkv<W, MT, true, true>), dim3(2 * pairs), dim3(W * 64), 0, s, xq, w, o, M, K);
  else if (e && *e && atoi(e) == 0)
    hipLaunchKernelGGL((k_gemv_qkv<W, MT, false>), dim3(pairs), dim3(W * 64), 0, s, xq, w, o, M, K);
  else
    hipLaunchKernelGGL((k_gemv_qkv<W, MT, true>), dim3(pairs), dim3(W * 64), 0, s, xq, w, o, M, K);
  return hipGetLastError();
}

// M <= 64; W in {4, 8, 16} (16 taken as 8 above M = 32); pairs = (nq + 2 nkv) * hd / 32;
// oct: the weight in octet order, one group (half a pair) per workgroup.
hipError_t launch_gemv_qkv(const uint8_t* xq, const uint8_t* w, const QkvOut& o, int M, int K, int W,
                           hipStream_t s, int oct) {
  if (M < 1 || M > 64 || K < 128 || (K & 127)) return hipErrorInvalidValue;
  const int pairs = (o.nq + 2 * o.nkv) * o.hd / 32;
  const int mt = (M + 15) / 16;
  if (W == 16 && mt > 2) W = 8;
  if (W == 16)
    return mt == 1 ? gemv_qkv_t<16, 1>(xq, w, o, M, K, pairs, s, oct != 0)
                   : gemv_qkv_t<16, 2>(xq, w, o, M, K, pairs, s, oct != 0);
  if (W == 8) {
    switch (mt) {
      case 1: return gemv_qkv_t<8, 1>(xq, w, o, M, K, pairs, s, oct != 0);
      case 2: return gemv_qkv_t<8, 2>(xq, w, o, M, K, pairs, s, oct != 0);
      case 3: return gemv_qkv_t<8, 3>(xq, w, o, M, K, pairs, s, oct != 0);
      default: return gemv_qkv_t<8, 4>(xq, w, o, M, K, pairs, s, oct != 0);
    }
  }
  if (W == 4) {
    switch (mt) {
      case 1: return gemv_qkv_t<4, 1>(xq, w, o, M, K, pairs, s, oct != 0);
      case 2: return gemv_qkv_t<4, 2>(xq, w, o, M, K, pairs, s, oct != 0);
      case 3: return gemv_qkv_t<4, 3>(xq, w, o, M, K, pairs, s, oct != 0);
      default: return gemv_qkv_t<4, 4>(xq, w, o, M, K, pairs, s, oct != 0);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace frt
