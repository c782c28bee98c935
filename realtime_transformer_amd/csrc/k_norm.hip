// k_norm.hip -- fused residual add + RMSNorm + per-tensor E4M3 quantise.
//
// FlashRT architecture doc, component "Kernel library": hand-written kernels
// for the memory-bound ops, including residual + norm + quant fusions;
// itsolotime article, section 3.3: rms_norm(x, w, out, S, D, eps, stream)
// calling convention; section 7.2: the residual stream stays high precision
// and the norm output feeds the low-precision GEMMs.
//
// Per row (rows are independent):
//   r'  = bf16(r + y)                       stored as the new residual
//   S   = sum r'^2 in fp64 (each square is exact in fp64)
//   inv = f32(1 / sqrt(S / H + eps)) in fp64, rounded once
//   x   = f32(f32(r' * inv) * w), or with AdaRMSNorm modulation (per-channel
//         scale and shift, itsolotime article section 5.2: Pi0.5)
//         x = f32(f32(f32(r' * inv) * f32(1 + scale)) + shift)
//   xq  = e4m3(f32(x * inv_x))              (measure mode: store x, amax|x|)
//
// Bound: HBM.  Algorithmic bytes per row: 2H (r) + 2H (y) + 2H (r') + H (xq),
// plus 2H once for w.
//
// When the previous down GEMM split K, its output arrives as S fp32 partial
// tiles [S][M][H]; the kernel then forms y = bf16(f32(sum_s part[s]) * a_d),
// adding the splits in split order, stores it to the Y slot and continues
// with that y.  Layout: TPR threads own one row; each thread holds
// NC chunks of 8 bf16 (16-byte loads) in registers between the two passes,
// so r' is read from HBM once.  The fp64 sum of squares is reduced across
// the wave with shuffles and across the row's waves through LDS.
#include "frt_device.h"
#include "frt_mx.h"

namespace frt {

// MX: the MXFP4 form (frt_mx.h): x is multiplied by inv_awq[k] (the AWQ
// pre-scale, itsolotime article section 7.2), each 32-block of a row (four
// consecutive chunks, i.e. four neighbouring lanes) takes its E8M0 exponent
// from the 4-lane maximum, and xq_out receives [M][H/2] E2M1 codes, xs_out
// [M][H/32] exponents.
// UPW: the one-wave-per-row form also issues every load of its row (and of
// the first four split-K partials) before using any, as the one-workgroup
// form does: one memory round trip per row instead of one per chunk, for
// the workloads whose rows are too few for occupancy to hide the per-chunk
// round trips.
template <int TPR, int NC, bool MEASURE, bool MX = false, bool UPW = false>
__global__ __launch_bounds__(256) void k_add_rmsnorm_quant(
    const uint16_t* __restrict__ r_prev, const uint16_t* __restrict__ y_prev,
    const uint16_t* __restrict__ w_norm, const uint16_t* __restrict__ mod, uint16_t* __restrict__ r_out,
    uint8_t* __restrict__ xq_out, float* __restrict__ x_out, float* __restrict__ amax_out,
    int M, int H, float eps, float inv_x, const float* __restrict__ y_part, int S, float alpha_d,
    uint16_t* __restrict__ y_store, const float* __restrict__ inv_awq = nullptr, uint8_t* __restrict__ xs_out = nullptr,
    int xs_mm = 0) {
  constexpr int RPW = 256 / TPR;  // rows per workgroup
  constexpr int WPR = TPR / 64;   // waves per row
  __shared__ double red[256 / 64];
  const int tid = threadIdx.x;
  const int row_in_wg = tid / TPR;
  const int t = tid % TPR;
  const int row = blockIdx.x * RPW + row_in_wg;
  const bool active = row < M;
  const int nchunk = H >> 3;
  const size_t base = (size_t)(active ? row : 0) * (size_t)H;

  // Every load of the row is issued before any is used, so a row costs one
  // memory round trip rather than one per chunk: chunk indices are clamped
  // into the row (threads past the end re-read the last chunk and discard
  // it) and the uniform choices select pointers, so no load waits behind a
  // per-chunk branch.  wn: the norm weight, or with modulation the
  // per-channel scale (mh: shift); aw: the MXFP4 form's AWQ reciprocals;
  // pp: the first four split-K partial tiles (further splits are read
  // after these, in split order).  This is for the one-workgroup-per-row
  // form (small M, where the row's latency is the kernel's time: the M = 1,
  // H = 5120 decode chain gains 0.4 us per layer); the many-row form (one
  // wave per row) reads chunk by chunk in the second loop instead, where
  // occupancy hides the latency and the up-front registers would halve it.
  constexpr bool UP = TPR == 256 || UPW;
  constexpr bool PF = UP && NC <= 4;
  uint4 rn[NC], wn[NC], mh[NC], yv[NC];
  float4 aw[MX ? NC : 1][2];
  // the first four split-K partial tiles (split index clamped to S - 1;
  // splits past the fourth are read one at a time after these)
  constexpr int SP = 4;
  float4 pp[SP][PF ? NC : 1][2];
  const uint16_t* wsrc = mod ? mod : w_norm;
  const uint16_t* hsrc = mod ? mod + H : w_norm;
  const size_t pstride = (size_t)M * H;
  // loads of chunk c (clamped into the row)
  auto load_chunk = [&](int c) {
    const int chc = min(t + c * TPR, nchunk - 1);
    const size_t o = base + (size_t)chc * 8;
    rn[c] = *reinterpret_cast<const uint4*>(r_prev + o);
    wn[c] = *reinterpret_cast<const uint4*>(wsrc + (size_t)chc * 8);
    mh[c] = *reinterpret_cast<const uint4*>(hsrc + (size_t)chc * 8);
    if (MX) {
      const float4* ap = reinterpret_cast<const float4*>(inv_awq + (size_t)chc * 8);
      aw[MX ? c : 0][0] = ap[0];
      aw[MX ? c : 0][1] = ap[1];
    }
    if (!y_part && y_prev) yv[c] = *reinterpret_cast<const uint4*>(y_prev + o);
  };
  if (UP) {
#pragma unroll
    for (int c = 0; c < NC; ++c) load_chunk(c);
  }
  if (y_part) {
    if (PF) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const size_t o = base + (size_t)min(t + c * TPR, nchunk - 1) * 8;
#pragma unroll
        for (int sp = 0; sp < SP; ++sp) {
          const size_t so = (size_t)(sp < S ? sp : S - 1) * pstride + o;
          pp[sp][PF ? c : 0][0] = *reinterpret_cast<const float4*>(y_part + so);
          pp[sp][PF ? c : 0][1] = *reinterpret_cast<const float4*>(y_part + so + 4);
        }
      }
    }
  }
  double sq = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = t + c * TPR;
    const bool ok = active && ch < nchunk;
    if (!UP) {
      if (!ok) {
        rn[c] = wn[c] = mh[c] = make_uint4(0, 0, 0, 0);
        if (MX) aw[MX ? c : 0][0] = aw[MX ? c : 0][1] = make_float4(0, 0, 0, 0);
        continue;
      }
      load_chunk(c);
    }
    if (!mod) mh[c] = make_uint4(0, 0, 0, 0);
    if (y_part) {
      // y = bf16(f32(sum of the splits in split order) * alpha_d)
      const size_t o = base + (size_t)min(ch, nchunk - 1) * 8;
      const int pc = PF ? c : 0;
      if (!PF) {
#pragma unroll
        for (int sp = 0; sp < SP; ++sp) {
          const size_t so = (size_t)(sp < S ? sp : S - 1) * pstride + o;
          pp[sp][0][0] = *reinterpret_cast<const float4*>(y_part + so);
          pp[sp][0][1] = *reinterpret_cast<const float4*>(y_part + so + 4);
        }
      }
      float a[8] = {pp[0][pc][0].x, pp[0][pc][0].y, pp[0][pc][0].z, pp[0][pc][0].w,
                    pp[0][pc][1].x, pp[0][pc][1].y, pp[0][pc][1].z, pp[0][pc][1].w};
      if (S > 1) {
#pragma unroll
        for (int sp = 1; sp < SP; ++sp) {
          if (sp < S) {
            a[0] += pp[sp][pc][0].x; a[1] += pp[sp][pc][0].y; a[2] += pp[sp][pc][0].z; a[3] += pp[sp][pc][0].w;
            a[4] += pp[sp][pc][1].x; a[5] += pp[sp][pc][1].y; a[6] += pp[sp][pc][1].z; a[7] += pp[sp][pc][1].w;
          }
        }
      }
      for (int sp = SP; sp < S; ++sp) {
        const float4 q0 = *reinterpret_cast<const float4*>(y_part + sp * pstride + o);
        const float4 q1 = *reinterpret_cast<const float4*>(y_part + sp * pstride + o + 4);
        a[0] += q0.x; a[1] += q0.y; a[2] += q0.z; a[3] += q0.w;
        a[4] += q1.x; a[5] += q1.y; a[6] += q1.z; a[7] += q1.w;
      }
      yv[c] = make_uint4(pack_bf16x2(a[0] * alpha_d, a[1] * alpha_d), pack_bf16x2(a[2] * alpha_d, a[3] * alpha_d),
                         pack_bf16x2(a[4] * alpha_d, a[5] * alpha_d), pack_bf16x2(a[6] * alpha_d, a[7] * alpha_d));
      if (ok) *reinterpret_cast<uint4*>(y_store + base + (size_t)ch * 8) = yv[c];
    } else if (!y_prev) {
      yv[c] = make_uint4(0, 0, 0, 0);
    }
    if (!ok) {
      rn[c] = make_uint4(0, 0, 0, 0);
      wn[c] = rn[c];
      mh[c] = rn[c];
      if (MX) aw[MX ? c : 0][0] = aw[MX ? c : 0][1] = make_float4(0, 0, 0, 0);
      continue;
    }
    const uint32_t rr[4] = {rn[c].x, rn[c].y, rn[c].z, rn[c].w};
    const uint32_t yy[4] = {yv[c].x, yv[c].y, yv[c].z, yv[c].w};
    uint32_t o4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_lo(rr[j]) + bf16_lo(yy[j]);
      const float hi = bf16_hi(rr[j]) + bf16_hi(yy[j]);
      o4[j] = pack_bf16x2(lo, hi);
      const double dlo = (double)bf16_lo(o4[j]), dhi = (double)bf16_hi(o4[j]);
      sq += dlo * dlo;
      sq += dhi * dhi;
    }
    rn[c] = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    *reinterpret_cast<uint4*>(r_out + base + (size_t)ch * 8) = rn[c];
  }
  sq = wave_sum_f64(sq);
  if (WPR > 1) {
    const int wave = tid >> 6;
    if ((tid & 63) == 0) red[wave] = sq;
    __syncthreads();
    sq = 0.0;
    const int w0 = row_in_wg * WPR;
    for (int w = 0; w < WPR; ++w) sq += red[w0 + w];
  }
  const float inv_rms = (float)(1.0 / sqrt(sq / (double)H + (double)eps));

  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = t + c * TPR;
    if (MX) {
      // every lane takes part in the block maximum; rows and chunks outside
      // the tensor contribute zeros and store nothing
      const bool ok = active && ch < nchunk;
      float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (ok) {
        const uint4 wv = wn[c];
        uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
        uint32_t rr[4] = {rn[c].x, rn[c].y, rn[c].z, rn[c].w};
        uint32_t hh[4] = {mh[c].x, mh[c].y, mh[c].z, mh[c].w};
        if (mod) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[2 * j] = ((bf16_lo(rr[j]) * inv_rms) * (1.0f + bf16_lo(ww[j]))) + bf16_lo(hh[j]);
            x[2 * j + 1] = ((bf16_hi(rr[j]) * inv_rms) * (1.0f + bf16_hi(ww[j]))) + bf16_hi(hh[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[2 * j] = (bf16_lo(rr[j]) * inv_rms) * bf16_lo(ww[j]);
            x[2 * j + 1] = (bf16_hi(rr[j]) * inv_rms) * bf16_hi(ww[j]);
          }
        }
        const float4 a0 = aw[MX ? c : 0][0], a1 = aw[MX ? c : 0][1];
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = x[j] * av[j];
      }
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = __builtin_fmaxf(am, __builtin_fabsf(x[j]));
      am = quad_max(am);
      const int e = mx_block_exp(am);
      const uint32_t codes = mx_pack8(x, e);
      if (ok) {
        *reinterpret_cast<uint32_t*>(xq_out + (size_t)row * (H / 2) + (size_t)ch * 4) = codes;
        if ((ch & 3) == 0)
          xs_out[xs_mm ? mx_act_scale_off_mm((uint32_t)row, (uint32_t)(ch >> 2), (uint32_t)H / 128)
                       : mx_act_scale_off_gemv((uint32_t)row, (uint32_t)(ch >> 2), (uint32_t)H / 128)] = (uint8_t)e;
      }
      continue;
    }
    if (active && ch < nchunk) {
      const uint4 wv = wn[c];
      uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
      uint32_t rr[4] = {rn[c].x, rn[c].y, rn[c].z, rn[c].w};
      uint32_t hh[4] = {mh[c].x, mh[c].y, mh[c].z, mh[c].w};
      float x[8];
      if (mod) {
        // AdaRMSNorm: f32(f32(t * f32(1 + scale)) + shift)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = ((bf16_lo(rr[j]) * inv_rms) * (1.0f + bf16_lo(ww[j]))) + bf16_lo(hh[j]);
          x[2 * j + 1] = ((bf16_hi(rr[j]) * inv_rms) * (1.0f + bf16_hi(ww[j]))) + bf16_hi(hh[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = (bf16_lo(rr[j]) * inv_rms) * bf16_lo(ww[j]);
          x[2 * j + 1] = (bf16_hi(rr[j]) * inv_rms) * bf16_hi(ww[j]);
        }
      }
      if (MEASURE) {
        float4* dst = reinterpret_cast<float4*>(x_out + base + (size_t)ch * 8);
        dst[0] = make_float4(x[0], x[1], x[2], x[3]);
        dst[1] = make_float4(x[4], x[5], x[6], x[7]);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[j]));
      } else {
        uint2 q;
        q.x = e4m3x4(x[0] * inv_x, x[1] * inv_x, x[2] * inv_x, x[3] * inv_x);
        q.y = e4m3x4(x[4] * inv_x, x[5] * inv_x, x[6] * inv_x, x[7] * inv_x);
        *reinterpret_cast<uint2*>(xq_out + base + (size_t)ch * 8) = q;
      }
    }
  }
  if (MEASURE) {
    amax = wave_max_f32(amax);
    if ((tid & 63) == 0) atomic_max_nonneg(amax_out, amax);
  }
}

// First half of the decode norm, for the gate/up GEMV that quantises its own
// activations (k_gemv_gateup_nq): r' = bf16(r + y) as above (y from the Y
// slot, or formed from the split-K partials and stored there) and the fp64
// sum of r'^2 over each 512-element slice of a row.  Workgroup (g, m) owns
// slice g of row m, one 8-element chunk per lane, and stores its sum to
// sq_out[m * gridDim.x + g]; the consumer adds the slices in slice order.
// Every square of a bf16 value is exact in fp64, so these slice sums and
// the one-pass sum of the whole row differ only where the row's squares span
// more than fp64's 53 bits.  Spread over H/512 workgroups, the row's loads
// are issued by as many CUs (one CU's request queue was the latency of the
// one-workgroup form).  quad != 0: the sums are over 4-element slices
// instead (sq_out[m * H/4 + k/4], the slices of the whole-column down GEMV).
template <int SMAX>
__global__ __launch_bounds__(64) void k_add_sumsq(const uint16_t* __restrict__ r_prev,
                                                  const uint16_t* __restrict__ y_prev,
                                                  const float* __restrict__ y_part, int S, float alpha_d,
                                                  uint16_t* __restrict__ y_store, uint16_t* __restrict__ r_out,
                                                  double* __restrict__ sq_out, int M, int H, int quad) {
  const int m = blockIdx.y, g = blockIdx.x;
  const int ch = g * 64 + (int)threadIdx.x;
  double sq = 0.0, sq4[2] = {0.0, 0.0};
  if (ch < H / 8) {
    const size_t o = (size_t)m * H + (size_t)ch * 8;
    const uint4 rv = *reinterpret_cast<const uint4*>(r_prev + o);
    uint4 yv = make_uint4(0, 0, 0, 0);
    if (y_part && SMAX > 0) {
      // every split's loads first (split index clamped, extra ones unused),
      // then the sum in split order: one memory round trip for any S <= SMAX
      const size_t stride = (size_t)M * H;
      float4 lo[SMAX > 0 ? SMAX : 1], hi[SMAX > 0 ? SMAX : 1];
#pragma unroll
      for (int sp = 0; sp < SMAX; ++sp) {
        const size_t so = (size_t)(sp < S ? sp : S - 1) * stride + o;
        lo[sp] = *reinterpret_cast<const float4*>(y_part + so);
        hi[sp] = *reinterpret_cast<const float4*>(y_part + so + 4);
      }
      float a[8] = {lo[0].x, lo[0].y, lo[0].z, lo[0].w, hi[0].x, hi[0].y, hi[0].z, hi[0].w};
#pragma unroll
      for (int sp = 1; sp < SMAX; ++sp) {
        if (sp < S) {
          a[0] += lo[sp].x; a[1] += lo[sp].y; a[2] += lo[sp].z; a[3] += lo[sp].w;
          a[4] += hi[sp].x; a[5] += hi[sp].y; a[6] += hi[sp].z; a[7] += hi[sp].w;
        }
      }
      yv = make_uint4(pack_bf16x2(a[0] * alpha_d, a[1] * alpha_d), pack_bf16x2(a[2] * alpha_d, a[3] * alpha_d),
                      pack_bf16x2(a[4] * alpha_d, a[5] * alpha_d), pack_bf16x2(a[6] * alpha_d, a[7] * alpha_d));
      *reinterpret_cast<uint4*>(y_store + o) = yv;
    } else if (y_part) {
      yv = y_from_partials(y_part, (size_t)M * H, o, S, alpha_d);
      *reinterpret_cast<uint4*>(y_store + o) = yv;
    } else if (y_prev) {
      yv = *reinterpret_cast<const uint4*>(y_prev + o);
    }
    const uint32_t rr[4] = {rv.x, rv.y, rv.z, rv.w}, yy[4] = {yv.x, yv.y, yv.z, yv.w};
    uint32_t o4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o4[j] = pack_bf16x2(bf16_lo(rr[j]) + bf16_lo(yy[j]), bf16_hi(rr[j]) + bf16_hi(yy[j]));
      const double dlo = (double)bf16_lo(o4[j]), dhi = (double)bf16_hi(o4[j]);
      sq += dlo * dlo;
      sq += dhi * dhi;
      sq4[j >> 1] += dlo * dlo;
      sq4[j >> 1] += dhi * dhi;
    }
    *reinterpret_cast<uint4*>(r_out + o) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    if (quad) {
      // slices of four elements (those of the whole-column down GEMV)
      double* qo = sq_out + (size_t)m * (H / 4) + 2 * ch;
      qo[0] = sq4[0];
      qo[1] = sq4[1];
    }
  }
  if (quad) return;  // (uniform)
  sq = wave_sum_f64(sq);
  if (threadIdx.x == 0) sq_out[(size_t)m * gridDim.x + g] = sq;
}

// Z = bf16(R + Y), the residual add after the last block.  With partials
// (S > 1 splits of the last down GEMM) Y is formed first and stored to its
// slot; with z == nullptr only that Y is written (a forward range that ends
// before the last layer).
__global__ __launch_bounds__(256) void k_residual_add(const uint16_t* __restrict__ r,
                                                      uint16_t* __restrict__ y,
                                                      uint16_t* __restrict__ z, size_t n8,
                                                      const float* __restrict__ y_part, int S,
                                                      float alpha_d) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  uint4 b;
  if (y_part) {
    b = y_from_partials(y_part, n8 * 8, i * 8, S, alpha_d);
    reinterpret_cast<uint4*>(y)[i] = b;
  } else {
    b = reinterpret_cast<const uint4*>(y)[i];
  }
  if (!z) return;
  uint4 a = reinterpret_cast<const uint4*>(r)[i];
  uint32_t aa[4] = {a.x, a.y, a.z, a.w}, bb[4] = {b.x, b.y, b.z, b.w}, o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = pack_bf16x2(bf16_lo(aa[j]) + bf16_lo(bb[j]), bf16_hi(aa[j]) + bf16_hi(bb[j]));
  reinterpret_cast<uint4*>(z)[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

// Device E4M3 quantiser over an fp32 array (the same conversion every kernel uses).
__global__ __launch_bounds__(256) void k_e4m3_encode(const float* __restrict__ in,
                                                     uint8_t* __restrict__ out, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = (uint8_t)e4m3x1(in[i]);
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------

// Whether the one-wave-per-row form issues its row's loads up front (UPW):
// where the rows are few enough (M <= 1024, at most four per CU) that the
// per-chunk round trips are the kernel's time; with more rows the extra
// registers cost the occupancy that hides them.  Measured: M=788 (H=2048,
// four split-K partials) 9.05 -> 7.04 us; M=4096 (H=3072) 17.3 -> 19.8 us.
// FRT_NORM_UPFRONT=0 / 1 forces it off / on.
static bool norm_upfront(int M) {
  const char* e = getenv("FRT_NORM_UPFRONT");
  if (e && *e) return atoi(e) != 0;
  return M <= 1024;
}

template <bool MEASURE>
static hipError_t launch_norm_t(const uint16_t* r_prev, const uint16_t* y_prev,
                                const uint16_t* w, const uint16_t* mod, uint16_t* r_out, uint8_t* xq, float* x_out,
                                float* amax, int M, int H, float eps, float inv_x,
                                hipStream_t s, const float* y_part = nullptr, int S = 1,
                                float alpha_d = 0.0f, uint16_t* y_store = nullptr) {
  const int nchunk = H / 8;
  // one wave per row when the row fits 8 chunks per lane, else a whole
  // workgroup per row
  if (nchunk <= 64 * 8) {
    const int nc = (nchunk + 63) / 64;
    dim3 grid((M + 3) / 4);
    const bool upw = !MEASURE && norm_upfront(M);
#define FRT_NORM64(NCV)                                                                                         \
  do {                                                                                                          \
    if (upw)                                                                                                    \
      hipLaunchKernelGGL((k_add_rmsnorm_quant<64, NCV, MEASURE, false, true>), grid, dim3(256), 0, s, r_prev,  \
                         y_prev, w, mod, r_out, xq, x_out, amax, M, H, eps, inv_x, y_part, S, alpha_d, y_store); \
    else                                                                                                        \
      hipLaunchKernelGGL((k_add_rmsnorm_quant<64, NCV, MEASURE>), grid, dim3(256), 0, s, r_prev, y_prev, w,    \
                         mod, r_out, xq, x_out, amax, M, H, eps, inv_x, y_part, S, alpha_d, y_store);           \
  } while (0)
    if (nc <= 2) FRT_NORM64(2);
    else if (nc <= 4) FRT_NORM64(4);
    else if (nc <= 6) FRT_NORM64(6);
    else FRT_NORM64(8);
#undef FRT_NORM64
  } else {
    const int nc = (nchunk + 255) / 256;
    dim3 grid(M);
    if (nc <= 4)
      hipLaunchKernelGGL((k_add_rmsnorm_quant<256, 4, MEASURE>), grid, dim3(256), 0, s, r_prev,
                         y_prev, w, mod, r_out, xq, x_out, amax, M, H, eps, inv_x, y_part, S, alpha_d,
                         y_store);
    else
      hipLaunchKernelGGL((k_add_rmsnorm_quant<256, 8, MEASURE>), grid, dim3(256), 0, s, r_prev,
                         y_prev, w, mod, r_out, xq, x_out, amax, M, H, eps, inv_x, y_part, S, alpha_d,
                         y_store);
  }
  return hipGetLastError();
}

// Small M: spread one row over a whole workgroup so the row's loads are
// issued by many waves at once (latency, not bandwidth, bounds M <= 64).
hipError_t launch_add_rmsnorm_quant(const uint16_t* r_prev, const uint16_t* y_prev,
                                    const uint16_t* w, const uint16_t* mod, uint16_t* r_out, uint8_t* xq, int M,
                                    int H, float eps, float inv_x, hipStream_t s,
                                    const float* y_part, int S, float alpha_d, uint16_t* y_store) {
  const int nchunk = H / 8;
  if (M <= 64 && nchunk > 64 && nchunk <= 256 * 8) {
    const int nc = (nchunk + 255) / 256;
    dim3 grid(M);
    if (nc <= 1)
      hipLaunchKernelGGL((k_add_rmsnorm_quant<256, 1, false>), grid, dim3(256), 0, s, r_prev,
                         y_prev, w, mod, r_out, xq, nullptr, nullptr, M, H, eps, inv_x, y_part, S, alpha_d, y_store);
    else if (nc <= 2)
      hipLaunchKernelGGL((k_add_rmsnorm_quant<256, 2, false>), grid, dim3(256), 0, s, r_prev,
                         y_prev, w, mod, r_out, xq, nullptr, nullptr, M, H, eps, inv_x, y_part, S, alpha_d, y_store);
    else if (nc <= 4)
      hipLaunchKernelGGL((k_add_rmsnorm_quant<256, 4, false>), grid, dim3(256), 0, s, r_prev,
                         y_prev, w, mod, r_out, xq, nullptr, nullptr, M, H, eps, inv_x, y_part, S, alpha_d, y_store);
    else
      hipLaunchKernelGGL((k_add_rmsnorm_quant<256, 8, false>), grid, dim3(256), 0, s, r_prev,
                         y_prev, w, mod, r_out, xq, nullptr, nullptr, M, H, eps, inv_x, y_part, S, alpha_d, y_store);
    return hipGetLastError();
  }
  return launch_norm_t<false>(r_prev, y_prev, w, mod, r_out, xq, nullptr, nullptr, M, H, eps, inv_x,
                              s, y_part, S, alpha_d, y_store);
}

// MXFP4 form of K1: xq_codes [M][H/2], the exponents in the GEMV layout
// (rows padded to 16) or with xs_mm the prefill GEMM's (rows padded to 128);
// inv_awq [H].  H % 512 == 0.
hipError_t launch_add_rmsnorm_mx(const uint16_t* r_prev, const uint16_t* y_prev, const uint16_t* w,
                                 const uint16_t* mod, const float* inv_awq, uint16_t* r_out, uint8_t* xq_codes,
                                 uint8_t* xq_scales, int M, int H, float eps, hipStream_t s, const float* y_part,
                                 int S, float alpha_d, uint16_t* y_store, int xs_mm) {
  if (H % 512 || !inv_awq) return hipErrorInvalidValue;
  const int nchunk = H / 8;
  const int nc = (nchunk + 255) / 256;
#define FRT_MX_NORM(NCV)                                                                                          \
  hipLaunchKernelGGL((k_add_rmsnorm_quant<256, NCV, false, true>), dim3(M), dim3(256), 0, s, r_prev, y_prev, w,   \
                     mod, r_out, xq_codes, nullptr, nullptr, M, H, eps, 1.0f, y_part, S, alpha_d, y_store, inv_awq, \
                     xq_scales, xs_mm)
  if (nc <= 1)
    FRT_MX_NORM(1);
  else if (nc <= 2)
    FRT_MX_NORM(2);
  else if (nc <= 4)
    FRT_MX_NORM(4);
  else
    FRT_MX_NORM(8);
#undef FRT_MX_NORM
  return hipGetLastError();
}

// Slices per row of k_add_sumsq (the consumer's G).
int add_sumsq_slices(int H) { return (H / 8 + 63) / 64; }

hipError_t launch_add_sumsq(const uint16_t* r_prev, const uint16_t* y_prev, const float* y_part, int S,
                            float alpha_d, uint16_t* y_store, uint16_t* r_out, double* sq_out, int M, int H,
                            hipStream_t s, int quad) {
  if (M < 1 || H % 8 || (y_part && (S < 1 || !y_store))) return hipErrorInvalidValue;
  const dim3 grid(add_sumsq_slices(H), M);
#define FRT_SUMSQ(SM)                                                                                        \
  hipLaunchKernelGGL((k_add_sumsq<SM>), grid, dim3(64), 0, s, r_prev, y_prev, y_part, S, alpha_d, y_store, r_out, \
                     sq_out, M, H, quad)
  if (!y_part || S <= 4)
    FRT_SUMSQ(4);
  else if (S <= 8)
    FRT_SUMSQ(8);
  else if (S <= 17)
    FRT_SUMSQ(17);
  else if (S <= 32)
    FRT_SUMSQ(32);
  else
    FRT_SUMSQ(0);  // splits summed by the loop of y_from_partials
#undef FRT_SUMSQ
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm_measure(const uint16_t* r_prev, const uint16_t* y_prev,
                                      const uint16_t* w, const uint16_t* mod, uint16_t* r_out, float* x_out,
                                      float* amax, int M, int H, float eps, hipStream_t s) {
  return launch_norm_t<true>(r_prev, y_prev, w, mod, r_out, nullptr, x_out, amax, M, H, eps, 1.0f, s);
}

hipError_t launch_residual_add(const uint16_t* r, uint16_t* y, uint16_t* z, size_t n, hipStream_t s,
                               const float* y_part, int S, float alpha_d) {
  size_t n8 = n / 8;
  hipLaunchKernelGGL(k_residual_add, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, r, y, z,
                     n8, y_part, S, alpha_d);
  return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_e4m3_encode, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

}  // namespace frt
