// frt_ffn.hip -- host side of the C ABI declared in include/frt_ffn.h.
//
// FlashRT architecture doc: the layer diagram's "C ABI execution contract:
// Buffer / Graph / Plan, replay-time mechanism for native hosts";
// component "CUDA Graph": the captured forward takes only device pointers,
// allocates nothing during replay and lives for the process lifetime;
// itsolotime article, section 4.1: capture in relaxed mode (only this
// stream), every runtime call checked by name, replay without a captured
// graph is an error; section 4.2: all intermediates preallocated, the
// forward passes raw pointers, shapes are stable.
//
// The plan never allocates device memory: every buffer is carved out of the
// caller's workspace at plan creation.  The only host allocations are the
// plan object and the temporary host buffer of frt_export_weight_codes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/frt_ffn.h"
#include "frt_device.h"
#include "frt_host.h"
#include "frt_mx.h"

namespace frt {
hipError_t launch_add_rmsnorm_quant(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*,
                                    uint8_t*, int, int, float, float, hipStream_t, const float*, int,
                                    float, uint16_t*);
hipError_t launch_add_rmsnorm_measure(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                                      uint16_t*, float*, float*, int, int, float, hipStream_t);
hipError_t launch_residual_add(const uint16_t*, uint16_t*, uint16_t*, size_t, hipStream_t, const float*,
                               int, float);
hipError_t launch_e4m3_encode(const float*, uint8_t*, int64_t, hipStream_t);
hipError_t launch_amax_bf16(const uint16_t*, size_t, float*, hipStream_t, const uint16_t*, size_t);
hipError_t launch_quant_pack(const uint16_t*, uint8_t*, int, int, float, int, hipStream_t, const uint16_t*);
hipError_t launch_gemv_gateup(int, const uint8_t*, const uint8_t*, uint8_t*, int, int, int, int,
                              float, float, float, hipStream_t);
hipError_t launch_gemv_down(const uint8_t*, const uint8_t*, uint16_t*, float*, int, int, int, int, int,
                            bool, float, hipStream_t);
hipError_t launch_gemv_gateup_mt(int, const uint8_t*, const uint8_t*, uint8_t*, int, int, int, int, float, float,
                                 float, hipStream_t);
hipError_t launch_gemv_down_mt(const uint8_t*, const uint8_t*, uint16_t*, float*, int, int, int, int, int, bool,
                               float, hipStream_t);
bool gemv_fused_supported(int, int, int);
hipError_t launch_add_sumsq(const uint16_t*, const uint16_t*, const float*, int, float, uint16_t*, uint16_t*, double*,
                            int, int, hipStream_t, int = 0);
int add_sumsq_slices(int);
bool gemv_nq_supported(int, int, int);
bool gemv_nq_wide_supported(int, int, int);
bool gemv_down_quad_supported(int, int, int);
hipError_t launch_gemv_down_quad(const uint8_t*, const uint8_t*, const uint16_t*, uint16_t*, uint16_t*, double*, int,
                                 int, int, int, float, hipStream_t);
bool gemv_mx_nq_supported(int, int, int);
hipError_t launch_gemv_gateup_mx_nq(int, const uint16_t*, const uint16_t*, const float*, const double*, int, float,
                                    uint8_t*, uint8_t*, const uint8_t*, const uint8_t*, uint8_t*, uint8_t*, int, int,
                                    int, int, hipStream_t);
hipError_t launch_gemv_gateup_nq(int, const uint16_t*, const uint16_t*, const double*, int, float, float, uint8_t*,
                                 const uint8_t*, uint8_t*, int, int, int, int, float, float, float, hipStream_t, int);
hipError_t launch_add_rmsnorm_mx(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, const float*,
                                 uint16_t*, uint8_t*, uint8_t*, int, int, float, hipStream_t, const float*, int, float,
                                 uint16_t*, int);
hipError_t launch_quant_mx(const uint16_t*, uint8_t*, uint8_t*, int, int, int, const uint16_t*, hipStream_t, int);
hipError_t launch_mxmm_gateup(int, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, uint8_t*, uint8_t*,
                              int, int, int, hipStream_t);
hipError_t launch_mxmm_down(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, uint16_t*, float*, int, int,
                            int, int, int, hipStream_t);
hipError_t launch_gemv_gateup_mx(int, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, uint8_t*,
                                 uint8_t*, int, int, int, int, hipStream_t);
hipError_t launch_gemv_down_mx(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, uint16_t*, float*, int,
                               int, int, int, int, hipStream_t);
int gemv_mx_max_waves(int M);
bool gemv_mx_nq_wide_supported(int M, int K, int W);
bool gemv_down_mx_quad_supported(int M, int K, int N);
hipError_t launch_gemv_down_mx_quad(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const uint16_t*,
                                    uint16_t*, uint16_t*, double*, int, int, int, int, hipStream_t);
hipError_t launch_gemv_gateup_fused(int, const uint16_t*, const uint16_t*, const float*, int, float, uint16_t*,
                                    const uint16_t*, uint16_t*, uint8_t*, const uint8_t*, uint8_t*, int, int, int, int,
                                    float, float, float, float, float, hipStream_t);
hipError_t launch_gemm_gateup(int, int, bool, const uint8_t*, const uint8_t*, uint8_t*, int, int, int,
                              float, float, float, hipStream_t);
hipError_t launch_gemm_down(int, const uint8_t*, const uint8_t*, uint16_t*, float*, int, int, int, int,
                            bool, float, hipStream_t);
bool gemm_config_ok(int, bool);
hipError_t launch_mm_gateup(int, int, bool, const uint8_t*, const uint8_t*, uint8_t*, int, int, int, float, float,
                            float, hipStream_t);
hipError_t launch_mm_down(int, bool, const uint8_t*, const uint8_t*, uint16_t*, float*, int, int, int, int, float,
                          hipStream_t);
int gemm_config_bm(int);
int gemm_config_bn(int);
hipError_t launch_calib_gateup(int, const float*, const uint8_t*, float*, float*, int, int, int,
                               float, float, hipStream_t, int);
hipError_t launch_calib_down(const float*, const uint8_t*, uint16_t*, int, int, int, float,
                             hipStream_t, int);
}  // namespace frt

using namespace frt;

// ---------------------------------------------------------------------------
// plan and workspace layout
// ---------------------------------------------------------------------------

namespace {

constexpr int kGemvMaxM = 16;
constexpr int kGemvMtMaxM = 64;  // multi-tile GEMV up to here (FRT_GEMV_MT_MAX_M lowers it)
constexpr int kMMMinM = 128;  // from here on the LDS-DMA GEMM takes the f16 path
constexpr int kCUs = 256;  // MI355X compute units (workgroup rounds are counted against them)

}  // namespace

int frt::env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return (e && *e) ? atoi(e) : dflt;
}

namespace {

// Waves per GEMV workgroup: the smallest power of two (<= 16, <= K blocks)
// that brings workgroups * W to `target` waves across the chip (measured best:
// ~6 per SIMD for gate/up, ~4 for the K-split down GEMV).
// FRT_GEMV_WAVES_GATEUP / FRT_GEMV_WAVES_DOWN override it (tuning sweeps).
int gemv_waves(int groups, int kblocks, const char* env, int target) {
  const char* e = getenv(env);
  int w = 1;
  if (e && *e) {
    w = atoi(e);
  } else {
    while (w < 16 && groups * w < target) w *= 2;
  }
  if (w != 1 && w != 2 && w != 4 && w != 8 && w != 16) w = 4;
  while (w > 1 && w > kblocks) w /= 2;
  return w;
}

// K splits of the decode down GEMV: at least `per_cu` workgroups per CU (a
// grid of a few hundred workgroups leaves CUs with one and others with two,
// and the per-CU load rate then sets the time), each split at least 8 K
// blocks.  Measured at H = 5120, I = 17408: 2 splits x 8 waves stream 5.1
// TB/s against 3.9 TB/s unsplit; 4 splits x 4 waves gain another 0.6 us
// (MXFP4: 0.4 us) when the consumer is the many-workgroup slice-sum kernel
// (per_cu 4), but cost more than they gain in the one-workgroup norm kernel
// (per_cu 2).
// FRT_GEMV_DOWN_SPLIT overrides.
int gemv_down_splits(int groups, int kblocks, int per_cu) {
  int s = 1;
  while (groups * s < per_cu * kCUs && kblocks / (2 * s) >= 8) s *= 2;
  s = env_int("FRT_GEMV_DOWN_SPLIT", s);
  return std::max(1, std::min(s, kblocks));
}

struct Layout {
  size_t wgu, wgu_layer;  // packed gate/up (or up) weights, per-layer stride
  size_t wd, wd_layer;    // packed down weights
  size_t wn;              // norm weights [L][H] bf16
  size_t r, y, xq, hq, z; // activation slots
  size_t mod;             // AdaRMSNorm modulation [L][2][H] bf16
  size_t part, part_bytes;
  size_t cnt, cnt_words;  // 2 regions of cnt_words uint32
  size_t amax;            // [2 + 2L] floats
  size_t cal_x, cal_h, cal_r, cal_y;
  size_t total;
  int s_gu, s_dn;  // GEMV: waves per workgroup; GEMM: K splits of the down GEMM
  int k_dn;        // GEMV: K splits of the down GEMV (workgroups per 16 output columns)
  int split_dn;    // K splits of the down projection, either path (> 1: fp32 partials)
  bool gemv_mt;    // 16 < M <= 64 on the multi-tile GEMVs
  bool mx;         // MXFP4 plan
  bool mx_mm;      // MXFP4 with M > 64: the prefill GEMMs (k_mxmm), their exponent layouts
  int mx_dn_nb;    // prefill down GEMM: weight blocks per wave (column tile 32 * nb)
  size_t wgu_sc, wd_sc;        // MXFP4: offset of the exponents inside a layer's weights
  size_t xq_stride, hq_stride; // bytes per XQ / HQ slot
  size_t awq, inv_awq;         // MXFP4: AWQ scale bf16 [L][H], its reciprocal fp32 [L][H]
  int cfg_gu, cfg_dn;  // GEMM tile configurations
  bool mm_gu, mm_dn;   // GEMM runs on the LDS-DMA f16 kernel (k_mm) rather than k_gemm
  bool norm_split;     // decode GEMV path: k_add_sumsq, then the gate/up GEMV quantises (k_gemv_gateup_nq)
  bool gu_oct;         // ... with the gated gate/up matrix in octet order (eight-column workgroups)
  bool dn_quad;        // ... with the whole-column down GEMV (k_gemv_down_quad, k_gemv_down_mx_quad), which forms the next
                       // layer's R' and 4-column slice sums itself: no norm kernel between layers
  size_t sqp;          // its slice sums of squares, fp64 [M][G]
  size_t sqp_bytes;    // bytes of that region
};


bool desc_ok(const frt_ffn_desc* d) {
  if (!d) return false;
  if (d->M < 1 || d->L < 1 || d->H < 128 || d->I < 128) return false;
  if (d->H % 128 || d->I % 128) return false;
  if (d->H > 16384 || d->I > 32768) return false;
  if (d->act < FRT_ACT_GEGLU_TANH || d->act > FRT_ACT_GELU_TANH) return false;
  if (!(d->eps > 0.0f) || !std::isfinite(d->eps)) return false;
  if ((d->flags & ~(uint32_t)(FRT_FLAG_FP8_MFMA_DOWN | FRT_FLAG_FUSED_NORM | FRT_FLAG_FP8_MFMA_GATEUP |
                              FRT_FLAG_NORM_FUSE | FRT_FLAG_ADA_NORM | FRT_FLAG_MXFP4)) != 0u ||
      d->device < 0)
    return false;
  // MXFP4: K dimensions in whole groups of four 128-blocks (one exponent
  // dword per lane in the GEMV layout), no FP8 or fused-norm options
  if ((d->flags & FRT_FLAG_MXFP4) &&
      (d->H % 512 || d->I % 512 ||
       (d->flags & (FRT_FLAG_FP8_MFMA_DOWN | FRT_FLAG_FP8_MFMA_GATEUP | FRT_FLAG_FUSED_NORM | FRT_FLAG_NORM_FUSE))))
    return false;
  // AdaRMSNorm replaces the norm weight: no folding of it, and no fused
  // decode prologue (which applies the weight)
  if ((d->flags & FRT_FLAG_ADA_NORM) && (d->flags & (FRT_FLAG_NORM_FUSE | FRT_FLAG_FUSED_NORM))) return false;
  // activation offsets inside the kernels are 32-bit: M*I and M*H bytes
  // (and the fp32 split-K partials, 4*M*H per split, addressed per split)
  if ((int64_t)d->M * d->I > (int64_t)1 << 31) return false;
  if ((int64_t)d->M * d->H > (int64_t)1 << 31) return false;
  return true;
}




// GEMM tile configurations for M > 16 (see k_gemm.hip): the gate/up GEMM
// takes the largest tile whose workgroups fill the chip; the down GEMM (few
// output columns) takes 128 x 256 tiles and splits K until about two
// workgroups per CU, its splits summed by the consumer.
// FRT_GEMM_GATEUP_CFG / FRT_GEMM_DOWN_CFG / FRT_GEMM_DOWN_SPLIT override.
// LDS-DMA GEMM (k_mm) configuration for an [M] x [N] output over K: the
// tile that minimises workgroup rounds x tile work, and for the down GEMM the
// K split that fills the chip against the cost of its fp32 partials (written
// once, read once by the consumer).  Rates are rough per-CU figures; the
// choice only has to rank the candidates.
}  // namespace

void frt::choose_mm(int M, int N, int K, bool allow_split, int& cfg, int& split, int ncfg) {
  const double cu_flops = 1.5e15 / kCUs, hbm = 5.0e12;
  double best = 1e30;
  cfg = -1;
  split = 1;
  for (int c = 0; c < ncfg; ++c) {
    const int bm = mm_config_bm(c), bn = mm_config_bn(c), ks = mm_config_ks(c);
    if (N % bn || K % ks) continue;
    const int tiles = (N / bn) * ceil_div(M, bm);
    for (int sp = 1; sp <= (allow_split ? 8 : 1); sp *= 2) {
      if (K / ks < 4 * sp) break;
      const int rounds = ceil_div(tiles * sp, kCUs);
      double t = rounds * (double)bm * bn * (K / sp) * 2.0 / cu_flops;
      if (sp > 1) t += (double)sp * M * N * 8.0 / hbm;
      if (t < best * 0.999) {
        best = t;
        cfg = c;
        split = sp;
      }
    }
  }
}

namespace {

void choose_gemm(const frt_ffn_desc& d, Layout& lo) {
  const int npk = d.act != FRT_ACT_GELU_TANH ? 2 * d.I : d.I;
  const bool fp8_gu = (d.flags & FRT_FLAG_FP8_MFMA_GATEUP) != 0u;
  const bool fp8_dn = (d.flags & FRT_FLAG_FP8_MFMA_DOWN) != 0u;
  int gu = env_int("FRT_GEMM_GATEUP_CFG", 1);
  if (!gemm_config_ok(gu, fp8_gu) || npk % gemm_config_bn(gu)) gu = 0;
  int dn = env_int("FRT_GEMM_DOWN_CFG", 1);
  if (!gemm_config_ok(dn, fp8_dn) || d.H % gemm_config_bn(dn)) dn = 0;
  const int tiles = (d.H / gemm_config_bn(dn)) * ceil_div(d.M, gemm_config_bm(dn));
  const int kb = d.I / 128;
  int split = std::max(1, std::min(16, ceil_div(2 * kCUs, tiles)));
  split = std::min(split, std::max(1, kb / 4));
  split = env_int("FRT_GEMM_DOWN_SPLIT", split);
  split = std::max(1, std::min(split, kb));
  lo.cfg_gu = gu;
  lo.cfg_dn = dn;
  lo.s_gu = 1;
  lo.s_dn = split;
  // prefill-sized M: the LDS-DMA kernel, on the f16 or (plan flags) the FP8
  // matrix cores (FRT_MM_GATEUP_CFG / FRT_MM_DOWN_CFG / FRT_MM_DOWN_SPLIT override)
  lo.mm_gu = lo.mm_dn = false;
  if (d.M >= kMMMinM) {
    int c, sp;
    {
      choose_mm(d.M, npk, d.H, false, c, sp);
      // on the FP8 matrix cores (no conversions in the loop) the 128 x 256
      // tile at two workgroups per CU wins (18-layer M = 788 chain with both
      // GEMMs on the FP8 cores: 110.7-112.5 against 113.3-114.0 us/layer);
      // on the f16 cores it is level with the model's choice
      if (fp8_gu && npk % mm_config_bn(kMMConfigTwoPerCU) == 0 && d.H % mm_config_ks(kMMConfigTwoPerCU) == 0)
        c = kMMConfigTwoPerCU;
      c = env_int("FRT_MM_GATEUP_CFG", c);
      if (mm_config_ffn(c) && npk % mm_config_bn(c) == 0 && d.H % mm_config_ks(c) == 0) {
        lo.mm_gu = true;
        lo.cfg_gu = c;
      }
    }
    {
      choose_mm(d.M, d.H, d.I, true, c, sp);
      // On the f16 cores, when the down GEMM's tile grid is small enough to
      // need a K split, the 128 x 256 two-per-CU tile splits K until its
      // workgroups cover 7/8 of the CUs: per wave 64 x 128 (three
      // conversions per MFMA against four for 64 x 64).  Measured on the
      // M = 788 chain: 167.3-168.8 against 171.1-173.0 us/layer (128 x 128,
      // 2 splits); on the FP8 matrix cores level, so unchanged there.
      const int c8 = kMMConfigTwoPerCU;
      if (!fp8_dn && sp > 1 && d.H % mm_config_bn(c8) == 0 && d.I % mm_config_ks(c8) == 0) {
        const int tiles8 = (d.H / mm_config_bn(c8)) * ceil_div(d.M, mm_config_bm(c8));
        int sp8 = 1;
        while (tiles8 * sp8 < kCUs * 7 / 8 && d.I / (mm_config_ks(c8) * sp8 * 2) >= 4) sp8 *= 2;
        c = c8;
        sp = sp8;
      }
      // the 256 x 192 tile with eight waves on the f16 cores (M = 4096 down
      // GEMM: 271-273 against 280-283 us with four waves)
      if (!fp8_dn && c == 2) c = kMMConfigEightWaves;
      c = env_int("FRT_MM_DOWN_CFG", c);
      sp = env_int("FRT_MM_DOWN_SPLIT", sp);
      if (mm_config_ffn(c) && d.H % mm_config_bn(c) == 0 && d.I % mm_config_ks(c) == 0 && sp >= 1 &&
          sp <= d.I / mm_config_ks(c)) {
        lo.mm_dn = true;
        lo.cfg_dn = c;
        lo.s_dn = sp;
      }
    }
  }
}

Layout make_layout(const frt_ffn_desc& d) {
  Layout lo{};
  const size_t M = d.M, H = d.H, I = d.I, L = d.L;
  const bool gated = d.act != FRT_ACT_GELU_TANH;
  const size_t npk = gated ? 2 * I : I;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  lo.mx = (d.flags & FRT_FLAG_MXFP4) != 0u;
  lo.mx_mm = lo.mx && d.M > kGemvMtMaxM;
  if (lo.mx) {
    // codes (half a byte per weight) then one exponent per 32 weights; the
    // activation exponents cover rows padded to 16 (GEMV layout) or to 128
    // (the prefill GEMM's)
    const size_t Mx = (size_t)ceil_div(d.M, lo.mx_mm ? 128 : 16) * (lo.mx_mm ? 128 : 16);
    lo.wgu_sc = align256(npk * H / 2);
    lo.wgu_layer = lo.wgu_sc + align256(npk * H / 32);
    lo.wd_sc = align256(H * I / 2);
    lo.wd_layer = lo.wd_sc + align256(H * I / 32);
    lo.xq_stride = align256(M * H / 2 + Mx * H / 32);
    lo.hq_stride = align256(M * I / 2 + Mx * I / 32);
  } else {
    lo.wgu_layer = align256(npk * H);
    lo.wd_layer = align256(H * I);
    lo.xq_stride = M * H;
    lo.hq_stride = M * I;
  }
  lo.wgu = take(lo.wgu_layer * L);
  lo.wd = take(lo.wd_layer * L);
  lo.wn = take(L * H * 2);
  lo.r = take((L + 1) * M * H * 2);
  lo.y = take((L + 1) * M * H * 2);
  lo.xq = take(L * lo.xq_stride);
  lo.hq = take(L * lo.hq_stride);
  lo.awq = take(lo.mx ? L * H * 2 : 256);
  lo.inv_awq = take(lo.mx ? L * H * 4 : 256);
  lo.z = take(M * H * 2);
  lo.mod = take((d.flags & FRT_FLAG_ADA_NORM) ? L * 2 * H * 2 : 256);

  size_t part = 0, words = 1;
  lo.gemv_mt = d.M > kGemvMaxM && d.M <= std::min(kGemvMtMaxM, env_int("FRT_GEMV_MT_MAX_M", kGemvMtMaxM));
  // The decode GEMV path splits the norm: a short kernel forms r' and slice
  // sums of squares, the gate/up GEMV quantises its own K range (measured
  // at M = 1, H = 5120: the one-workgroup norm kernel's latency was its
  // single CU's load queue).  FRT_NORM_SPLIT=0 keeps the one-kernel norm.
  // The MXFP4 decode GEMV path does the same (k_gemv_gateup_mx_nq).
  {
    const int G = add_sumsq_slices((int)H);
    const bool shape_ok = lo.mx ? (!lo.mx_mm && gemv_mx_nq_supported((int)M, (int)H, G))
                                : (!lo.gemv_mt && gemv_nq_supported((int)M, (int)H, G));
    lo.norm_split = shape_ok && d.M <= kGemvMaxM && (d.flags & (FRT_FLAG_FUSED_NORM | FRT_FLAG_ADA_NORM)) == 0u &&
                    env_int("FRT_NORM_SPLIT", 1) != 0;
  }
  if (lo.mx_mm) {
    // K split of the MXFP4 down GEMM until its 128 x (32 nb) tiles give at
    // least one workgroup per CU (each split at least 8 stages)
    lo.mx_dn_nb = env_int("FRT_MXMM_DOWN_NB", 4) == 8 && H % 256 == 0 ? 8 : 4;
    const int tiles = (int)(H / (32 * lo.mx_dn_nb)) * ceil_div(d.M, 128);
    int sp = 1;
    while (tiles * sp < kCUs && (int)(I / 128) / (2 * sp) >= 8 && sp < 8) sp *= 2;
    sp = std::max(1, std::min(env_int("FRT_MXMM_DOWN_SPLIT", sp), (int)(I / 128)));
    lo.s_gu = lo.s_dn = 0;
    lo.k_dn = lo.split_dn = sp;
    part = sp > 1 ? (size_t)sp * M * H * 4 : 4;
    words = 1;
  } else if (d.M <= kGemvMaxM || lo.gemv_mt || lo.mx) {
    lo.s_gu = gemv_waves((int)(I / 16), (int)(H / 128), "FRT_GEMV_WAVES_GATEUP", 6144);
    lo.k_dn = gemv_down_splits((int)(H / 16), (int)(I / 128), lo.norm_split ? 4 : 2);
    lo.s_dn = gemv_waves((int)(H / 16) * lo.k_dn, (int)(I / 128) / lo.k_dn, "FRT_GEMV_WAVES_DOWN", 4096);
    if (lo.mx) {
      // the MXFP4 down GEMV splits K in whole 512-value quads (an override
      // beyond them is clamped)
      lo.k_dn = std::max(1, std::min(lo.k_dn, (int)(I / 512)));
      // MXFP4 GEMVs: 4, 8 or 16 waves, fewer for more row tiles (LDS); the
      // gate/up workgroups own 32 columns.  Target ~2 waves per SIMD
      // (measured at the decode shape: 4 waves per workgroup for both GEMVs,
      // 38.1 us/layer against 39.8 with 8)
      lo.s_gu = gemv_waves((int)(I / 32), (int)(H / 128), "FRT_GEMV_WAVES_GATEUP", 2048);
      lo.s_dn = gemv_waves((int)(H / 16) * lo.k_dn, (int)(I / 128) / lo.k_dn, "FRT_GEMV_WAVES_DOWN", 2048);
      const int wmax = gemv_mx_max_waves(d.M);
      lo.s_gu = std::min(wmax, std::max(4, lo.s_gu));
      lo.s_dn = std::min(wmax, std::max(4, lo.s_dn));
      lo.s_gu = lo.s_gu >= 16 ? 16 : (lo.s_gu >= 8 ? 8 : 4);
      // the gate/up waves split K in quads of blocks: where four waves would
      // get uneven shares (H = 5120: 2, 3, 2, 3 quads) and five divide them,
      // take five (measured at the decode shape: 18.7 against 19.3 us)
      const int kq = (int)(H / 512), mt = ceil_div(d.M, 16);
      if (lo.s_gu == 4 && kq % 4 != 0 && kq % 5 == 0 && 5 * mt <= 16) lo.s_gu = 5;
      {
        // an override is taken only where the kernel has it: 4, 5, 8, 10 or
        // 16 waves, at least one per row tile, W * row tiles <= 16
        const int w = env_int("FRT_GEMV_WAVES_GATEUP_MX", lo.s_gu);
        if ((w == 4 || w == 5 || w == 8 || w == 10 || w == 16) && w >= mt && w * mt <= 16) lo.s_gu = w;
      }
      lo.s_dn = lo.s_dn >= 16 ? 16 : (lo.s_dn >= 8 ? 8 : 4);
      // M <= 4 on the split norm: the whole-column MXFP4 down GEMV (down
      // matrix in the column-quad order), FRT_DOWN_QUAD=0 keeps the split-K
      // GEMV and the slice-sum kernel
      lo.dn_quad = lo.norm_split && gemv_down_mx_quad_supported((int)M, (int)I, (int)H) &&
                   gemv_mx_nq_wide_supported((int)M, (int)H, lo.s_gu) && env_int("FRT_DOWN_QUAD", 1) != 0;
      if (lo.dn_quad) {
        // 512-value steps per workgroup: I / 512, over eight waves (at M=1,
        // H=5120, I=17408: 30.7 us/layer against 30.9 with four), fewer
        // where the steps do not reach one per wave
        const int steps = (int)(I / 512);
        int w = env_int("FRT_GEMV_WAVES_DOWN_QUAD_MX", 8);
        if (w != 1 && w != 2 && w != 4 && w != 8 && w != 16) w = 8;
        while (w > 1 && w > steps) w /= 2;
        lo.k_dn = 1;
        lo.s_dn = w;
      }
    } else if (lo.gemv_mt) {
      // the multi-tile kernels take 4 or 8 waves (at least one per row tile)
      lo.s_gu = lo.s_gu >= 8 ? 8 : 4;
      lo.s_dn = lo.s_dn >= 8 ? 8 : 4;
    }
    // gated activations on the split norm: the gate/up matrix in octet order,
    // one 16-row group per workgroup holding eight gate and eight up columns
    // (twice the workgroups of half the bytes); FRT_GATEUP_OCT=0 keeps the
    // 16 + 16 column workgroups
    lo.gu_oct = lo.norm_split && !lo.mx && !lo.gemv_mt && d.act != FRT_ACT_GELU_TANH && I % 8 == 0 &&
                env_int("FRT_GATEUP_OCT", 1) != 0;
    if (lo.gu_oct) {
      int w = env_int("FRT_GEMV_WAVES_GATEUP_OCT", 8);
      if (w != 1 && w != 2 && w != 4 && w != 8 && w != 16) w = 8;
      while (w > 1 && w > (int)(H / 128)) w /= 2;
      lo.s_gu = w;
    }
    // M <= 4 on the split norm: the whole-column down GEMV (down matrix in
    // the column-quad layout), FRT_DOWN_QUAD=0 keeps the split-K GEMV and
    // the slice-sum kernel
    if (!lo.mx)
      lo.dn_quad = lo.norm_split && !lo.gemv_mt && (d.flags & FRT_FLAG_FP8_MFMA_DOWN) == 0u &&
                   gemv_down_quad_supported((int)M, (int)I, (int)H) &&
                   gemv_nq_wide_supported((int)M, (int)H, lo.s_gu) && env_int("FRT_DOWN_QUAD", 1) != 0;
    if (lo.dn_quad && !lo.mx) {
      // 1 KiB steps per workgroup: I / 256, over eight waves (at M=1,
      // H=5120, I=17408: 16.0 us against 17.5 with sixteen and 18.2 with
      // four), fewer where the steps do not reach one per wave
      const int steps = (int)(I / 256);
      int w = env_int("FRT_GEMV_WAVES_DOWN_QUAD", 8);
      if (w != 1 && w != 2 && w != 4 && w != 8 && w != 16) w = 8;
      while (w > 1 && w > steps) w /= 2;
      lo.k_dn = 1;
      lo.s_dn = w;
    }
    lo.split_dn = lo.k_dn;
    part = lo.k_dn > 1 ? (size_t)lo.k_dn * M * H * 4 : 4;
    words = 1;
  } else {
    choose_gemm(d, lo);
    lo.k_dn = 1;
    lo.split_dn = lo.s_dn;
    part = lo.s_dn > 1 ? (size_t)lo.s_dn * M * H * 4 : 4;
    words = 1;
  }
  lo.sqp_bytes = lo.norm_split ? M * (size_t)(lo.dn_quad ? H / 4 : add_sumsq_slices((int)H)) * 8 : 256;
  lo.sqp = take(lo.sqp_bytes);
  lo.part = take(part);
  lo.part_bytes = part;
  lo.cnt_words = words;
  lo.cnt = take(2 * words * 4);
  lo.amax = take((2 + 2 * L) * 4);
  lo.cal_x = take(M * H * 4);
  lo.cal_h = take(M * I * 4);
  lo.cal_r = take(2 * M * H * 2);
  lo.cal_y = take(2 * M * H * 2);
  lo.total = off;
  return lo;
}

}  // namespace

struct frt_plan {
  frt_ffn_desc d{};
  Layout lo{};
  uint8_t* ws = nullptr;
  bool gated = true;
  std::vector<uint8_t> w_set;
  std::vector<float> s_x, s_g, s_u, s_h, s_d;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  bool captured = false, stale = false;
  std::vector<hipEvent_t> prof_events;  // created on the first profiled forward

  uint8_t* wgu(int l) const { return ws + lo.wgu + (size_t)l * lo.wgu_layer; }
  uint8_t* wd(int l) const { return ws + lo.wd + (size_t)l * lo.wd_layer; }
  uint16_t* wn(int l) const { return reinterpret_cast<uint16_t*>(ws + lo.wn) + (size_t)l * d.H; }
  size_t mh() const { return (size_t)d.M * d.H; }
  uint16_t* r(int l) const { return reinterpret_cast<uint16_t*>(ws + lo.r) + (size_t)l * mh(); }
  uint16_t* y(int l) const { return reinterpret_cast<uint16_t*>(ws + lo.y) + (size_t)l * mh(); }
  uint8_t* xq(int l) const { return ws + lo.xq + (size_t)l * lo.xq_stride; }
  uint8_t* hq(int l) const { return ws + lo.hq + (size_t)l * lo.hq_stride; }
  // MXFP4: exponents after the codes of a slot / a layer's weights
  uint8_t* xs(int l) const { return xq(l) + mh() / 2; }
  uint8_t* hs(int l) const { return hq(l) + (size_t)d.M * d.I / 2; }
  uint8_t* wgu_s(int l) const { return wgu(l) + lo.wgu_sc; }
  uint8_t* wd_s(int l) const { return wd(l) + lo.wd_sc; }
  uint16_t* awq(int l) const { return reinterpret_cast<uint16_t*>(ws + lo.awq) + (size_t)l * d.H; }
  float* inv_awq(int l) const { return reinterpret_cast<float*>(ws + lo.inv_awq) + (size_t)l * d.H; }
  bool mx() const { return lo.mx; }
  uint16_t* z() const { return reinterpret_cast<uint16_t*>(ws + lo.z); }
  bool ada() const { return (d.flags & FRT_FLAG_ADA_NORM) != 0u; }
  bool norm_fuse() const { return (d.flags & FRT_FLAG_NORM_FUSE) != 0u; }
  // layer l's modulation [2][H] (scale, shift), or null when the plan has none
  const uint16_t* mod(int l) const {
    return ada() ? reinterpret_cast<const uint16_t*>(ws + lo.mod) + (size_t)l * 2 * d.H : nullptr;
  }
  // the forward's scratch (split-K partials, slice sums): in the workspace,
  // or, during frt_ffn_forward_range_static_scratch, in the library's static
  // device array (scratch_base set for the duration of that call)
  uint8_t* scratch_base = nullptr;
  size_t scratch_part_off() const { return align256(lo.sqp_bytes); }
  size_t scratch_bytes() const { return scratch_part_off() + lo.part_bytes; }
  float* part() const {
    return reinterpret_cast<float*>(scratch_base ? scratch_base + scratch_part_off() : ws + lo.part);
  }
  double* sqp() const { return reinterpret_cast<double*>(scratch_base ? scratch_base : ws + lo.sqp); }
  uint32_t* cnt(int region) const {
    return reinterpret_cast<uint32_t*>(ws + lo.cnt) + (size_t)region * lo.cnt_words;
  }
  float* amax() const { return reinterpret_cast<float*>(ws + lo.amax); }
  bool fp8_down() const { return (d.flags & FRT_FLAG_FP8_MFMA_DOWN) != 0u; }
  bool fp8_gateup() const { return (d.flags & FRT_FLAG_FP8_MFMA_GATEUP) != 0u; }
  // optionally, decode shapes run the norm inside the gate/up GEMV
  bool fused_norm() const {
    return d.M <= kGemvMaxM && (d.flags & FRT_FLAG_FUSED_NORM) != 0u && gemv_fused_supported(d.M, d.H, lo.s_gu);
  }
  bool act_scales_set() const {
    if (mx()) return true;  // MXFP4 takes its block scales from the data
    for (int l = 0; l < d.L; ++l)
      if (!(s_x[l] > 0.0f) || !(s_h[l] > 0.0f)) return false;
    return true;
  }
  bool all_weights() const {
    for (auto v : w_set)
      if (!v) return false;
    return true;
  }
  void drop_events() {
    for (auto e : prof_events) (void)hipEventDestroy(e);
    prof_events.clear();
  }
  void drop_graph() {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    exec = nullptr;
    graph = nullptr;
    captured = false;
    stale = false;
  }
  void mark_stale() {
    if (captured) stale = true;
  }
};

// ---------------------------------------------------------------------------
// exported entry points
// ---------------------------------------------------------------------------

extern "C" {

const char* frt_last_error(void) { return frt::last_error_text().c_str(); }

frt_status frt_ffn_workspace_size(const frt_ffn_desc* desc, size_t* bytes) {
  if (!bytes) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_workspace_size: bytes is NULL");
  if (!desc_ok(desc)) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_workspace_size: invalid descriptor");
  *bytes = make_layout(*desc).total;
  return FRT_OK;
}

frt_status frt_ffn_plan_create(const frt_ffn_desc* desc, void* d_workspace, size_t bytes,
                               frt_plan** out) {
  if (!out) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_plan_create: out is NULL");
  *out = nullptr;
  if (!desc_ok(desc)) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_plan_create: invalid descriptor");
  if (!d_workspace) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_plan_create: workspace is NULL");
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256)
    return fail(FRT_ERR_WORKSPACE, "frt_ffn_plan_create: workspace not 256-byte aligned");
  Layout lo = make_layout(*desc);
  if (bytes < lo.total)
    return fail(FRT_ERR_WORKSPACE, "frt_ffn_plan_create: workspace %zu bytes < %zu needed", bytes,
                lo.total);
  int ndev = 0;
  HIP_CHECK(hipGetDeviceCount(&ndev));
  if (desc->device >= ndev)
    return fail(FRT_ERR_INVALID_ARG, "frt_ffn_plan_create: device %d of %d", desc->device, ndev);
  DeviceGuard g(desc->device);
  HIP_CHECK(g.err);
  hipDeviceProp_t prop;
  HIP_CHECK(hipGetDeviceProperties(&prop, desc->device));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(FRT_ERR_UNSUPPORTED, "frt_ffn_plan_create: device is %s, need gfx950",
                prop.gcnArchName);
  hipPointerAttribute_t attr;
  HIP_CHECK(hipPointerGetAttributes(&attr, d_workspace));
  if (attr.type != hipMemoryTypeDevice || attr.device != desc->device)
    return fail(FRT_ERR_INVALID_ARG, "frt_ffn_plan_create: workspace is not device memory of device %d",
                desc->device);

  frt_plan* p = new (std::nothrow) frt_plan();
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_plan_create: out of host memory");
  p->d = *desc;
  p->lo = lo;
  p->ws = static_cast<uint8_t*>(d_workspace);
  p->gated = desc->act != FRT_ACT_GELU_TANH;
  p->w_set.assign(desc->L, 0);  // (GEMM tiles chosen in make_layout)
  p->s_x.assign(desc->L, 0.0f);
  p->s_h.assign(desc->L, 0.0f);
  p->s_g.assign(desc->L, 1.0f);
  p->s_u.assign(desc->L, 1.0f);
  p->s_d.assign(desc->L, 1.0f);
  hipError_t e = hipMemset(p->ws + lo.cnt, 0, 2 * lo.cnt_words * 4);
  if (e == hipSuccess) e = hipMemset(p->y(0), 0, p->mh() * 2);
  if (e == hipSuccess && p->ada()) e = hipMemset(p->ws + lo.mod, 0, (size_t)desc->L * 2 * desc->H * 2);
  if (e == hipSuccess && lo.mx)  // AWQ scale 1 and reciprocal 1 until set
    e = hipMemsetD16(reinterpret_cast<hipDeviceptr_t>(p->ws + lo.awq), 0x3F80u, (size_t)desc->L * desc->H);
  if (e == hipSuccess && lo.mx)
    e = hipMemsetD32(reinterpret_cast<hipDeviceptr_t>(p->ws + lo.inv_awq), 0x3F800000, (size_t)desc->L * desc->H);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    delete p;
    return fail(FRT_ERR_HIP, "frt_ffn_plan_create: clearing counters failed: %s", hipGetErrorString(e));
  }
  *out = p;
  return FRT_OK;
}

frt_status frt_ffn_plan_destroy(frt_plan* plan) {
  if (!plan) return FRT_OK;
  {
    DeviceGuard g(plan->d.device);
    plan->drop_graph();
    plan->drop_events();
  }
  delete plan;
  return FRT_OK;
}

static frt_status quant_one(frt_plan* p, const void* src, int N, int K, uint8_t* dst, int mode,
                            float* scale_out, hipStream_t s, const void* colw = nullptr) {
  const uint16_t* cw = static_cast<const uint16_t*>(colw);
  float* am = p->amax();
  float amax_h = 0.0f;
  HIP_CHECK(hipMemsetAsync(am, 0, sizeof(float), s));
  KERNEL_CHECK(launch_amax_bf16(static_cast<const uint16_t*>(src), (size_t)N * K, am, s, cw, (size_t)K), "amax_bf16");
  HIP_CHECK(hipMemcpyAsync(&amax_h, am, sizeof(float), hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  if (!std::isfinite(amax_h))
    return fail(FRT_ERR_INVALID_ARG, "frt_quant_weights: weight tensor holds a non-finite value");
  const float sc = amax_h > 0.0f ? amax_h / 448.0f : 1.0f;
  const float inv = 1.0f / sc;
  KERNEL_CHECK(launch_quant_pack(static_cast<const uint16_t*>(src), dst, N, K, inv, mode, s, cw),
               "quant_pack");
  *scale_out = sc;
  return FRT_OK;
}

frt_status frt_quant_weights(frt_plan* p, int32_t layer, const void* d_w_gate, const void* d_w_up,
                             const void* d_w_down, const void* d_norm_w, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_quant_weights: plan is NULL");
  if (layer < 0 || layer >= p->d.L) return fail(FRT_ERR_INVALID_ARG, "frt_quant_weights: layer %d out of range", layer);
  if (!d_w_up || !d_w_down || !d_norm_w)
    return fail(FRT_ERR_INVALID_ARG, "frt_quant_weights: NULL weight pointer");
  if (p->gated != (d_w_gate != nullptr))
    return fail(FRT_ERR_INVALID_ARG, "frt_quant_weights: gate weight must be %s for this activation",
                p->gated ? "given" : "NULL");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = p->d.H, I = p->d.I;
  float sg = 1.0f, su = 1.0f, sd = 1.0f;
  frt_status st;
  if (p->mx()) {
    // MXFP4: gate/up times the layer's AWQ scale per input column, then 32-blocks
    const uint16_t* aw = p->awq(layer);
    const int mml = p->lo.mx_mm ? 1 : 0;
    if (p->gated) {
      KERNEL_CHECK(launch_quant_mx(static_cast<const uint16_t*>(d_w_gate), p->wgu(layer), p->wgu_s(layer), I, H, 1, aw, s,
                                   mml),
                   "quant_mx");
      KERNEL_CHECK(launch_quant_mx(static_cast<const uint16_t*>(d_w_up), p->wgu(layer), p->wgu_s(layer), I, H, 2, aw, s,
                                   mml),
                   "quant_mx");
    } else {
      KERNEL_CHECK(launch_quant_mx(static_cast<const uint16_t*>(d_w_up), p->wgu(layer), p->wgu_s(layer), I, H, 0, aw, s,
                                   mml),
                   "quant_mx");
    }
    KERNEL_CHECK(launch_quant_mx(static_cast<const uint16_t*>(d_w_down), p->wd(layer), p->wd_s(layer), H, I, 0, nullptr,
                                 s, p->lo.dn_quad ? 2 : mml),
                 "quant_mx");
    HIP_CHECK(hipMemcpyAsync(p->wn(layer), d_norm_w, (size_t)H * 2, hipMemcpyDeviceToDevice, s));
    HIP_CHECK(hipStreamSynchronize(s));
    p->w_set[layer] = 1;
    p->mark_stale();
    return FRT_OK;
  }
  // norm fusion folds the RMSNorm weight into the gate/up matrices per input
  // column and normalises with a unit weight
  const void* fold = p->norm_fuse() ? d_norm_w : nullptr;
  if (p->gated) {
    const bool oct = p->lo.gu_oct;
    if ((st = quant_one(p, d_w_gate, I, H, p->wgu(layer), oct ? 4 : 1, &sg, s, fold)) != FRT_OK) return st;
    if ((st = quant_one(p, d_w_up, I, H, p->wgu(layer), oct ? 5 : 2, &su, s, fold)) != FRT_OK) return st;
  } else {
    if ((st = quant_one(p, d_w_up, I, H, p->wgu(layer), 0, &su, s, fold)) != FRT_OK) return st;
  }
  if ((st = quant_one(p, d_w_down, H, I, p->wd(layer), p->lo.dn_quad ? 3 : 0, &sd, s)) != FRT_OK) return st;
  if (p->norm_fuse())
    HIP_CHECK(hipMemsetD16Async(reinterpret_cast<hipDeviceptr_t>(p->wn(layer)), 0x3F80u, (size_t)H, s));
  else
    HIP_CHECK(hipMemcpyAsync(p->wn(layer), d_norm_w, (size_t)H * 2, hipMemcpyDeviceToDevice, s));
  HIP_CHECK(hipStreamSynchronize(s));
  p->s_g[layer] = sg;
  p->s_u[layer] = su;
  p->s_d[layer] = sd;
  p->w_set[layer] = 1;
  p->mark_stale();
  return FRT_OK;
}

frt_status frt_export_weight_codes(const frt_plan* p, int32_t layer, int32_t which, void* host_dst) {
  if (!p || !host_dst) return fail(FRT_ERR_INVALID_ARG, "frt_export_weight_codes: NULL argument");
  if (layer < 0 || layer >= p->d.L) return fail(FRT_ERR_INVALID_ARG, "frt_export_weight_codes: layer out of range");
  if (which < 0 || which > 2 || (which == 0 && !p->gated))
    return fail(FRT_ERR_INVALID_ARG, "frt_export_weight_codes: bad tensor index %d", which);
  if (!p->w_set[layer]) return fail(FRT_ERR_STATE, "frt_export_weight_codes: layer %d not quantised", layer);
  if (p->mx()) return fail(FRT_ERR_STATE, "frt_export_weight_codes: MXFP4 plan (use frt_export_mxfp4_weights)");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  const uint32_t H = p->d.H, I = p->d.I;
  const bool down = which == 2;
  const uint32_t N = down ? H : I, K = down ? I : H;
  const uint32_t rows_packed = down ? H : (p->gated ? 2 * I : I);
  const size_t bytes = (size_t)rows_packed * K;
  std::vector<uint8_t> tmp;
  try {
    tmp.resize(bytes);
  } catch (...) {
    return fail(FRT_ERR_INVALID_ARG, "frt_export_weight_codes: out of host memory");
  }
  HIP_CHECK(hipMemcpy(tmp.data(), down ? p->wd(layer) : p->wgu(layer), bytes, hipMemcpyDeviceToHost));
  uint8_t* dst = static_cast<uint8_t*>(host_dst);
  for (uint32_t n = 0; n < N; ++n) {
    uint32_t prow = n;
    if (!down && p->gated && p->lo.gu_oct) prow = which == 0 ? gate_row_oct(n) : up_row_oct(n);
    else if (!down && p->gated) prow = which == 0 ? gate_row(n) : up_row_gated(n);
    for (uint32_t k = 0; k < K; k += 16)
      memcpy(dst + (size_t)n * K + k,
             tmp.data() + (down && p->lo.dn_quad ? quad_offset(n, k, K) : packed_offset(prow, k, K)), 16);
  }
  return FRT_OK;
}

frt_status frt_export_mxfp4_weights(const frt_plan* p, int32_t layer, int32_t which, void* host_codes,
                                    void* host_exponents) {
  if (!p || !host_codes || !host_exponents) return fail(FRT_ERR_INVALID_ARG, "frt_export_mxfp4_weights: NULL argument");
  if (!p->mx()) return fail(FRT_ERR_STATE, "frt_export_mxfp4_weights: not an MXFP4 plan");
  if (layer < 0 || layer >= p->d.L) return fail(FRT_ERR_INVALID_ARG, "frt_export_mxfp4_weights: layer out of range");
  if (which < 0 || which > 2 || (which == 0 && !p->gated))
    return fail(FRT_ERR_INVALID_ARG, "frt_export_mxfp4_weights: bad tensor index %d", which);
  if (!p->w_set[layer]) return fail(FRT_ERR_STATE, "frt_export_mxfp4_weights: layer %d not quantised", layer);
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  const uint32_t H = p->d.H, I = p->d.I;
  const bool down = which == 2;
  const uint32_t N = down ? H : I, K = down ? I : H, KB = K / 128;
  const uint32_t rows_packed = down ? H : (p->gated ? 2 * I : I);
  const size_t code_bytes = (size_t)rows_packed * K / 2, sc_bytes = (size_t)rows_packed * K / 32;
  std::vector<uint8_t> tc, ts;
  try {
    tc.resize(code_bytes);
    ts.resize(sc_bytes);
  } catch (...) {
    return fail(FRT_ERR_INVALID_ARG, "frt_export_mxfp4_weights: out of host memory");
  }
  HIP_CHECK(hipMemcpy(tc.data(), down ? p->wd(layer) : p->wgu(layer), code_bytes, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(ts.data(), down ? p->wd_s(layer) : p->wgu_s(layer), sc_bytes, hipMemcpyDeviceToHost));
  uint8_t* dc = static_cast<uint8_t*>(host_codes);
  uint8_t* dsc = static_cast<uint8_t*>(host_exponents);
  for (uint32_t n = 0; n < N; ++n) {
    const uint32_t pr = down || !p->gated ? n : (which == 0 ? gate_row(n) : up_row_gated(n));
    for (uint32_t b = 0; b < K / 32; ++b) {
      if (down && p->lo.dn_quad) {
        memcpy(dc + (size_t)n * (K / 2) + (size_t)b * 16, tc.data() + mx_quad_code_off(n, b, K), 16);
        dsc[(size_t)n * (K / 32) + b] = ts[mx_quad_scale_off(n, b, K)];
        continue;
      }
      const uint32_t kb = b >> 2, lane = (pr & 15u) + 16u * (b & 3u);
      memcpy(dc + (size_t)n * (K / 2) + (size_t)b * 16, tc.data() + mx_code_off(pr, kb, lane, KB), 16);
      dsc[(size_t)n * (K / 32) + b] = ts[p->lo.mx_mm ? mx_scale_off_mm(pr, kb, lane, KB) : mx_scale_off(pr, kb, lane, KB)];
    }
  }
  return FRT_OK;
}

frt_status frt_set_awq(frt_plan* p, int32_t layer, const void* d_awq, void* stream) {
  if (!p || !d_awq) return fail(FRT_ERR_INVALID_ARG, "frt_set_awq: NULL argument");
  if (!p->mx()) return fail(FRT_ERR_UNSUPPORTED, "frt_set_awq: AWQ pre-scale needs an MXFP4 plan");
  if (layer < 0 || layer >= p->d.L) return fail(FRT_ERR_INVALID_ARG, "frt_set_awq: layer %d out of range", layer);
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = p->d.H;
  std::vector<uint16_t> sb(H);
  std::vector<float> inv(H);
  HIP_CHECK(hipMemcpyAsync(sb.data(), d_awq, (size_t)H * 2, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  for (int k = 0; k < H; ++k) {
    uint32_t u = (uint32_t)sb[k] << 16;
    float v;
    memcpy(&v, &u, 4);
    if (!std::isfinite(v) || !(v > 0.0f))
      return fail(FRT_ERR_INVALID_ARG, "frt_set_awq: scale %d is not finite and positive", k);
    inv[k] = 1.0f / v;  // f32(1 / s), rounded once
  }
  HIP_CHECK(hipMemcpyAsync(p->awq(layer), sb.data(), (size_t)H * 2, hipMemcpyHostToDevice, s));
  HIP_CHECK(hipMemcpyAsync(p->inv_awq(layer), inv.data(), (size_t)H * 4, hipMemcpyHostToDevice, s));
  HIP_CHECK(hipStreamSynchronize(s));
  p->w_set[layer] = 0;  // the layer's weights must be quantised (again) with this scale
  p->mark_stale();
  return FRT_OK;
}

frt_status frt_calibrate(frt_plan* p, const void* const* d_r_batches, const void* const* d_y_batches,
                         int32_t nbatch, int32_t rows, int32_t layer_begin, int32_t layer_end,
                         void* stream) {
  if (!p || !d_r_batches) return fail(FRT_ERR_INVALID_ARG, "frt_calibrate: NULL argument");
  if (p->mx()) return fail(FRT_ERR_UNSUPPORTED, "frt_calibrate: an MXFP4 plan takes its block scales from the data");
  if (nbatch < 1 || rows < 1 || rows > p->d.M)
    return fail(FRT_ERR_INVALID_ARG, "frt_calibrate: nbatch %d rows %d (1..%d)", nbatch, rows, p->d.M);
  if (layer_begin < 0 || layer_end > p->d.L || layer_begin >= layer_end)
    return fail(FRT_ERR_INVALID_ARG, "frt_calibrate: bad layer range [%d, %d)", layer_begin, layer_end);
  for (int b = 0; b < nbatch; ++b)
    if (!d_r_batches[b]) return fail(FRT_ERR_INVALID_ARG, "frt_calibrate: batch %d residual is NULL", b);
  for (int l = layer_begin; l < layer_end; ++l)
    if (!p->w_set[l]) return fail(FRT_ERR_STATE, "frt_calibrate: weights of layer %d not set", l);
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int L = p->d.L, H = p->d.H, I = p->d.I;
  float* am = p->amax() + 2;  // [L] x, then [L] h
  HIP_CHECK(hipMemsetAsync(am, 0, sizeof(float) * 2 * L, s));
  float* x = reinterpret_cast<float*>(p->ws + p->lo.cal_x);
  float* h = reinterpret_cast<float*>(p->ws + p->lo.cal_h);
  uint16_t* cr = reinterpret_cast<uint16_t*>(p->ws + p->lo.cal_r);
  uint16_t* cy = reinterpret_cast<uint16_t*>(p->ws + p->lo.cal_y);
  const size_t rh = (size_t)rows * H;
  for (int b = 0; b < nbatch; ++b) {
    const uint16_t* r_cur = static_cast<const uint16_t*>(d_r_batches[b]);
    const uint16_t* y_cur = d_y_batches ? static_cast<const uint16_t*>(d_y_batches[b]) : nullptr;
    for (int l = layer_begin; l < layer_end; ++l) {
      uint16_t* r_next = cr + (size_t)(l & 1) * rh;
      uint16_t* y_next = cy + (size_t)(l & 1) * rh;
      KERNEL_CHECK(launch_add_rmsnorm_measure(r_cur, y_cur, p->wn(l), p->mod(l), r_next, x, am + l, rows, H,
                                              p->d.eps, s), "add_rmsnorm_measure");
      KERNEL_CHECK(launch_calib_gateup(p->d.act, x, p->wgu(l), h, am + L + l, rows, H, I,
                                       p->gated ? p->s_g[l] : p->s_u[l], p->s_u[l], s, p->lo.gu_oct ? 1 : 0),
                   "calib_gateup");
      KERNEL_CHECK(launch_calib_down(h, p->wd(l), y_next, rows, I, H, p->s_d[l], s, p->lo.dn_quad ? 1 : 0),
                   "calib_down");
      r_cur = r_next;
      y_cur = y_next;
    }
  }
  std::vector<float> hm(2 * L);
  HIP_CHECK(hipMemcpyAsync(hm.data(), am, sizeof(float) * 2 * L, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  for (int l = layer_begin; l < layer_end; ++l) {
    if (!std::isfinite(hm[l]) || !std::isfinite(hm[L + l]))
      return fail(FRT_ERR_INVALID_ARG, "frt_calibrate: non-finite activation at layer %d", l);
  }
  for (int l = layer_begin; l < layer_end; ++l) {
    p->s_x[l] = hm[l] > 0.0f ? hm[l] / 448.0f : 1.0f;
    p->s_h[l] = hm[L + l] > 0.0f ? hm[L + l] / 448.0f : 1.0f;
  }
  p->mark_stale();
  return FRT_OK;
}

frt_status frt_get_scales(const frt_plan* p, float* host_out) {
  if (!p || !host_out) return fail(FRT_ERR_INVALID_ARG, "frt_get_scales: NULL argument");
  for (int l = 0; l < p->d.L; ++l) {
    host_out[5 * l + 0] = p->s_x[l];
    host_out[5 * l + 1] = p->s_g[l];
    host_out[5 * l + 2] = p->s_u[l];
    host_out[5 * l + 3] = p->s_h[l];
    host_out[5 * l + 4] = p->s_d[l];
  }
  return FRT_OK;
}

frt_status frt_set_act_scales(frt_plan* p, const float* host_in) {
  if (!p || !host_in) return fail(FRT_ERR_INVALID_ARG, "frt_set_act_scales: NULL argument");
  for (int l = 0; l < 2 * p->d.L; ++l)
    if (!std::isfinite(host_in[l]) || !(host_in[l] > 0.0f))
      return fail(FRT_ERR_INVALID_ARG, "frt_set_act_scales: scale %d is not finite and positive", l);
  for (int l = 0; l < p->d.L; ++l) {
    p->s_x[l] = host_in[2 * l];
    p->s_h[l] = host_in[2 * l + 1];
  }
  p->mark_stale();
  return FRT_OK;
}

static uint32_t path_bits_of(const frt_ffn_desc& d, const Layout& lo) {
  uint32_t b = 0;
  if (d.M <= kGemvMaxM && !lo.mx_mm) b |= FRT_PATH_GEMV;
  if (lo.norm_split) b |= FRT_PATH_NORM_SPLIT;
  if (lo.dn_quad) b |= FRT_PATH_DOWN_WHOLE_COLUMN;
  if (lo.split_dn > 1) b |= FRT_PATH_DOWN_SPLIT_K;
  if (lo.gu_oct) b |= FRT_PATH_GATEUP_OCTETS;
  return b;
}

frt_status frt_ffn_plan_path(const frt_plan* p, uint32_t* path_bits) {
  if (!p || !path_bits) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_plan_path: NULL argument");
  *path_bits = path_bits_of(p->d, p->lo);
  return FRT_OK;
}

frt_status frt_ffn_desc_path(const frt_ffn_desc* desc, uint32_t* path_bits) {
  if (!path_bits) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_desc_path: path_bits is NULL");
  if (!desc_ok(desc)) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_desc_path: invalid descriptor");
  *path_bits = path_bits_of(*desc, make_layout(*desc));
  return FRT_OK;
}

frt_status frt_ffn_io_get(const frt_plan* p, frt_ffn_io* out) {
  if (!p || !out) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_io_get: NULL argument");
  out->r_slots = p->r(0);
  out->y_slots = p->y(0);
  out->xq_slots = p->xq(0);
  out->hq_slots = p->hq(0);
  out->z_out = p->z();
  out->stride_rh = p->mh() * 2;
  out->stride_xq = p->lo.xq_stride;
  out->stride_hq = p->lo.hq_stride;
  out->mod_slots = p->ada() ? p->ws + p->lo.mod : nullptr;
  out->stride_mod = (size_t)2 * p->d.H * 2;
  return FRT_OK;
}

// Launch kernel `which` (0: add+RMSNorm+quantise, 1: gate/up GEMM, 2: down
// GEMM) of layer l on stream s.  When the norm is fused into the gate/up
// kernel, `which` 0 launches nothing and 1 runs both steps.
// Down output of layer l-1 still in split-K partials (GEMM path, split > 1)?
static bool down_split(const frt_plan* p) { return p->lo.split_dn > 1; }

// after_down: layer l - 1's down GEMM ran before this launch in the same
// sequence (with the whole-column down GEMV, layer l's norm step is then
// already done and launches nothing).
static frt_status launch_layer_kernel(frt_plan* p, int l, int which, hipStream_t s,
                                      bool y_in_partials = false, bool after_down = false) {
  const int M = p->d.M, H = p->d.H, I = p->d.I;
  const int npk = p->gated ? 2 * I : I;
  const float s_x = p->s_x[l], s_h = p->s_h[l];
  const float inv_x = 1.0f / s_x, inv_h = 1.0f / s_h;
  const float a_g = s_x * p->s_g[l], a_u = s_x * p->s_u[l], a_d = s_h * p->s_d[l];
  const bool fused = p->fused_norm();
  if (p->mx()) {
    if (which == 0 && p->lo.dn_quad && after_down) {
      // R' and the slice sums came from layer l - 1's down GEMV
    } else if (which == 0 && p->lo.norm_split) {
      const float* yp = (y_in_partials && l > 0) ? p->part() : nullptr;
      KERNEL_CHECK(launch_add_sumsq(p->r(l), p->y(l), yp, p->lo.split_dn, 1.0f, p->y(l), p->r(l + 1), p->sqp(), M, H,
                                    s, p->lo.dn_quad ? 1 : 0),
                   "add_sumsq");
    } else if (which == 0) {
      const float* yp = (y_in_partials && l > 0) ? p->part() : nullptr;
      KERNEL_CHECK(launch_add_rmsnorm_mx(p->r(l), p->y(l), p->wn(l), p->mod(l), p->inv_awq(l), p->r(l + 1), p->xq(l),
                                         p->xs(l), M, H, p->d.eps, s, yp, p->lo.split_dn, 1.0f, p->y(l),
                                         p->lo.mx_mm ? 1 : 0),
                   "add_rmsnorm_mx");
    } else if (which == 1 && p->lo.mx_mm) {
      KERNEL_CHECK(launch_mxmm_gateup(p->d.act, p->xq(l), p->xs(l), p->wgu(l), p->wgu_s(l), p->hq(l), p->hs(l), M, H,
                                      npk, s),
                   "mxmm_gateup");
    } else if (which == 1 && p->lo.norm_split) {
      KERNEL_CHECK(launch_gemv_gateup_mx_nq(p->d.act, p->r(l + 1), p->wn(l), p->inv_awq(l), p->sqp(),
                                            p->lo.dn_quad ? H / 4 : add_sumsq_slices(H), p->d.eps, p->xq(l), p->xs(l), p->wgu(l), p->wgu_s(l),
                                            p->hq(l), p->hs(l), M, H, I, p->lo.s_gu, s),
                   "gemv_gateup_mx_nq");
    } else if (which == 1) {
      KERNEL_CHECK(launch_gemv_gateup_mx(p->d.act, p->xq(l), p->xs(l), p->wgu(l), p->wgu_s(l), p->hq(l), p->hs(l), M,
                                         H, I, p->lo.s_gu, s),
                   "gemv_gateup_mx");
    } else if (p->lo.mx_mm) {
      KERNEL_CHECK(launch_mxmm_down(p->hq(l), p->hs(l), p->wd(l), p->wd_s(l), p->y(l + 1), p->part(), M, I, H,
                                    p->lo.split_dn, p->lo.mx_dn_nb, s),
                   "mxmm_down");
    } else if (p->lo.dn_quad) {
      KERNEL_CHECK(launch_gemv_down_mx_quad(p->hq(l), p->hs(l), p->wd(l), p->wd_s(l), p->r(l + 1), p->y(l + 1),
                                            l + 1 < p->d.L ? p->r(l + 2) : p->z(), p->sqp(), M, I, H, p->lo.s_dn, s),
                   "gemv_down_mx_quad");
    } else {
      KERNEL_CHECK(launch_gemv_down_mx(p->hq(l), p->hs(l), p->wd(l), p->wd_s(l), p->y(l + 1), p->part(), M, I, H,
                                       p->lo.s_dn, p->lo.k_dn, s),
                   "gemv_down_mx");
    }
    return FRT_OK;
  }
  if (which == 0) {
    if (p->lo.dn_quad && after_down) {
      // R' and the slice sums came from layer l - 1's down GEMV
    } else if (p->lo.norm_split) {
      const float* yp = nullptr;
      float a_prev = 0.0f;
      if (y_in_partials && l > 0) {
        yp = p->part();
        a_prev = p->s_h[l - 1] * p->s_d[l - 1];
      }
      KERNEL_CHECK(launch_add_sumsq(p->r(l), p->y(l), yp, p->lo.split_dn, a_prev, p->y(l), p->r(l + 1), p->sqp(), M,
                                    H, s, p->lo.dn_quad ? 1 : 0),
                   "add_sumsq");
    } else if (!fused) {
      const float* yp = nullptr;
      float a_prev = 0.0f;
      if (y_in_partials && l > 0) {
        yp = p->part();
        a_prev = p->s_h[l - 1] * p->s_d[l - 1];
      }
      KERNEL_CHECK(launch_add_rmsnorm_quant(p->r(l), p->y(l), p->wn(l), p->mod(l), p->r(l + 1), p->xq(l), M, H,
                                            p->d.eps, inv_x, s, yp, p->lo.split_dn, a_prev, p->y(l)),
                   "add_rmsnorm_quant");
    }
  } else if (which == 1) {
    if (fused) {
      const float* yp = nullptr;
      float a_prev = 0.0f;
      if (y_in_partials && l > 0) {
        yp = p->part();
        a_prev = p->s_h[l - 1] * p->s_d[l - 1];
      }
      KERNEL_CHECK(launch_gemv_gateup_fused(p->d.act, p->r(l), p->y(l), yp, p->lo.split_dn, a_prev, p->y(l), p->wn(l),
                                            p->r(l + 1), p->xq(l), p->wgu(l), p->hq(l), M, H, I, p->lo.s_gu,
                                            p->d.eps, inv_x, a_g, a_u, inv_h, s), "gemv_gateup_fused");
    }
    else if (p->lo.norm_split)
      KERNEL_CHECK(launch_gemv_gateup_nq(p->d.act, p->r(l + 1), p->wn(l), p->sqp(),
                                         p->lo.dn_quad ? H / 4 : add_sumsq_slices(H), p->d.eps,
                                         inv_x, p->xq(l), p->wgu(l), p->hq(l), M, H, I, p->lo.s_gu, a_g, a_u, inv_h,
                                         s, p->lo.gu_oct ? 1 : 0),
                   "gemv_gateup_nq");
    else if (M <= kGemvMaxM)
      KERNEL_CHECK(launch_gemv_gateup(p->d.act, p->xq(l), p->wgu(l), p->hq(l), M, H, I, p->lo.s_gu,
                                      a_g, a_u, inv_h, s), "gemv_gateup");
    else if (p->lo.gemv_mt)
      KERNEL_CHECK(launch_gemv_gateup_mt(p->d.act, p->xq(l), p->wgu(l), p->hq(l), M, H, I, p->lo.s_gu,
                                         a_g, a_u, inv_h, s), "gemv_gateup_mt");
    else if (p->lo.mm_gu)
      KERNEL_CHECK(launch_mm_gateup(p->d.act, p->lo.cfg_gu, p->fp8_gateup(), p->xq(l), p->wgu(l), p->hq(l), M, H,
                                    npk, a_g, a_u, inv_h, s), "mm_gateup");
    else
      KERNEL_CHECK(launch_gemm_gateup(p->d.act, p->lo.cfg_gu, p->fp8_gateup(), p->xq(l), p->wgu(l),
                                      p->hq(l), M, H, npk, a_g, a_u, inv_h, s), "gemm_gateup");
  } else {
    if (p->lo.dn_quad)
      KERNEL_CHECK(launch_gemv_down_quad(p->hq(l), p->wd(l), p->r(l + 1), p->y(l + 1),
                                         l + 1 < p->d.L ? p->r(l + 2) : p->z(), p->sqp(), M, I, H, p->lo.s_dn, a_d,
                                         s),
                   "gemv_down_quad");
    else if (M <= kGemvMaxM)
      KERNEL_CHECK(launch_gemv_down(p->hq(l), p->wd(l), p->y(l + 1), p->part(), M, I, H, p->lo.s_dn,
                                    p->lo.k_dn, p->fp8_down(),
                                    a_d, s), "gemv_down");
    else if (p->lo.gemv_mt)
      KERNEL_CHECK(launch_gemv_down_mt(p->hq(l), p->wd(l), p->y(l + 1), p->part(), M, I, H, p->lo.s_dn,
                                       p->lo.k_dn, p->fp8_down(), a_d, s), "gemv_down_mt");
    else if (p->lo.mm_dn)
      KERNEL_CHECK(launch_mm_down(p->lo.cfg_dn, p->fp8_down(), p->hq(l), p->wd(l), p->y(l + 1), p->part(), M, I, H,
                                  p->lo.s_dn, a_d, s), "mm_down");
    else
      KERNEL_CHECK(launch_gemm_down(p->lo.cfg_dn, p->hq(l), p->wd(l), p->y(l + 1), p->part(), M, I, H,
                                    p->lo.s_dn, p->fp8_down(), a_d, s), "gemm_down");
  }
  return FRT_OK;
}

// Layers [lb, le): layer lb reads its Y slot; later layers take Y from the
// previous down GEMM's split-K partials when it split.  After the last layer
// of the range the Y slot is materialised (and Z formed after layer L-1).
static frt_status forward_range(frt_plan* p, int lb, int le, hipStream_t s,
                                const hipEvent_t* ev = nullptr) {
  const int L = p->d.L;
  const bool split = down_split(p);
  for (int l = lb; l < le; ++l) {
    const hipEvent_t* e = ev ? ev + 4 * (l - lb) : nullptr;
    for (int k = 0; k < 3; ++k) {
      if (e) HIP_CHECK(hipEventRecord(e[k], s));
      frt_status st = launch_layer_kernel(p, l, k, s, split && l > lb, l > lb);
      if (st != FRT_OK) return st;
    }
    if (e) HIP_CHECK(hipEventRecord(e[3], s));
  }
  const float a_last = p->mx() ? 1.0f : p->s_h[le - 1] * p->s_d[le - 1];
  if (le == L && p->lo.dn_quad) {
    // Z = bf16(R + Y) came from the last down GEMV
  } else if (le == L)
    KERNEL_CHECK(launch_residual_add(p->r(L), p->y(L), p->z(), p->mh(), s, split ? p->part() : nullptr,
                                     p->lo.split_dn, a_last), "residual_add");
  else if (split)
    KERNEL_CHECK(launch_residual_add(p->r(le), p->y(le), nullptr, p->mh(), s, p->part(), p->lo.split_dn, a_last),
                 "finalize_y");
  return FRT_OK;
}

// ---------------------------------------------------------------------------
// The forward with its scratch in a static device array, for callers that
// cannot allocate (the workspace's scratch region is not touched).
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
// One copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// kernels get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (which must be current),
// looked up on the first call per device and kept.
frt_status static_scratch(int dev, uint8_t** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(FRT_ERR_UNSUPPORTED, "static scratch: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FRT_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return FRT_OK;
}

}  // namespace

frt_status frt_ffn_forward_range_static_scratch(frt_plan* p, int32_t layer_begin, int32_t layer_end, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_forward_range_static_scratch: plan is NULL");
  if (layer_begin < 0 || layer_end > p->d.L || layer_begin >= layer_end)
    return fail(FRT_ERR_INVALID_ARG, "frt_ffn_forward_range_static_scratch: bad range [%d, %d)", layer_begin,
                layer_end);
  if (p->scratch_bytes() > kStaticScratchBytes)
    return fail(FRT_ERR_UNSUPPORTED,
                "frt_ffn_forward_range_static_scratch: the plan needs %zu bytes of scratch, the static array "
                "holds %zu (use frt_ffn_forward_range)",
                p->scratch_bytes(), kStaticScratchBytes);
  for (int l = layer_begin; l < layer_end; ++l)
    if (!p->w_set[l]) return fail(FRT_ERR_STATE, "frt_ffn_forward_range_static_scratch: weights of layer %d not set", l);
  if (!p->act_scales_set()) return fail(FRT_ERR_STATE, "frt_ffn_forward_range_static_scratch: activation scales not set");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  uint8_t* base = nullptr;
  frt_status st = static_scratch(p->d.device, &base);
  if (st != FRT_OK) return st;
  p->scratch_base = base;
  st = forward_range(p, layer_begin, layer_end, static_cast<hipStream_t>(stream));
  p->scratch_base = nullptr;
  return st;
}

frt_status frt_ffn_forward_range(frt_plan* p, int32_t layer_begin, int32_t layer_end, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_forward_range: plan is NULL");
  if (layer_begin < 0 || layer_end > p->d.L || layer_begin >= layer_end)
    return fail(FRT_ERR_INVALID_ARG, "frt_ffn_forward_range: bad range [%d, %d)", layer_begin, layer_end);
  for (int l = layer_begin; l < layer_end; ++l)
    if (!p->w_set[l]) return fail(FRT_ERR_STATE, "frt_ffn_forward_range: weights of layer %d not set", l);
  if (!p->act_scales_set()) return fail(FRT_ERR_STATE, "frt_ffn_forward_range: activation scales not set");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  return forward_range(p, layer_begin, layer_end, static_cast<hipStream_t>(stream));
}

frt_status frt_ffn_forward(frt_plan* p, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_forward: plan is NULL");
  return frt_ffn_forward_range(p, 0, p->d.L, stream);
}

frt_status frt_ffn_forward_profiled(frt_plan* p, void* stream, float* host_ms) {
  if (!p || !host_ms) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_forward_profiled: NULL argument");
  if (!p->all_weights() || !p->act_scales_set())
    return fail(FRT_ERR_STATE, "frt_ffn_forward_profiled: weights and activation scales must be set first");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  const int L = p->d.L;
  if (p->prof_events.empty()) {
    p->prof_events.resize((size_t)4 * L, nullptr);
    for (auto& e : p->prof_events) {
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) {
        p->drop_events();
        return fail(FRT_ERR_HIP, "hipEventCreate failed: %s", hipGetErrorString(err));
      }
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  frt_status st = forward_range(p, 0, L, s, p->prof_events.data());
  if (st != FRT_OK) return st;
  HIP_CHECK(hipStreamSynchronize(s));
  for (int l = 0; l < L; ++l)
    for (int k = 0; k < 3; ++k)
      HIP_CHECK(hipEventElapsedTime(&host_ms[3 * l + k], p->prof_events[4 * l + k], p->prof_events[4 * l + k + 1]));
  return FRT_OK;
}

frt_status frt_ffn_time_kernel(frt_plan* p, int32_t which, int32_t reps, void* stream, float* avg_us) {
  if (!p || !avg_us) return fail(FRT_ERR_INVALID_ARG, "frt_ffn_time_kernel: NULL argument");
  if (which < 0 || which > 2 || reps < 1)
    return fail(FRT_ERR_INVALID_ARG, "frt_ffn_time_kernel: which %d reps %d", which, reps);
  if (!p->all_weights() || !p->act_scales_set())
    return fail(FRT_ERR_STATE, "frt_ffn_time_kernel: weights and activation scales must be set first");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  HIP_CHECK(hipEventCreate(&e0));
  hipError_t err = hipEventCreate(&e1);
  if (err != hipSuccess) {
    (void)hipEventDestroy(e0);
    return fail(FRT_ERR_HIP, "hipEventCreate failed: %s", hipGetErrorString(err));
  }
  frt_status st = FRT_OK;
  float ms = 0.0f;
  err = hipEventRecord(e0, s);
  for (int r = 0; r < reps && st == FRT_OK && err == hipSuccess; ++r)
    for (int l = 0; l < p->d.L && st == FRT_OK; ++l)
      st = launch_layer_kernel(p, l, which, s, down_split(p) && l > 0, l > 0);
  if (err == hipSuccess && st == FRT_OK) err = hipEventRecord(e1, s);
  if (err == hipSuccess && st == FRT_OK) err = hipEventSynchronize(e1);
  if (err == hipSuccess && st == FRT_OK) err = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != FRT_OK) return st;
  if (err != hipSuccess) return fail(FRT_ERR_HIP, "frt_ffn_time_kernel: event timing failed: %s", hipGetErrorString(err));
  *avg_us = ms * 1000.0f / (float)((int64_t)reps * p->d.L);
  return FRT_OK;
}

frt_status frt_graph_capture(frt_plan* p, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_graph_capture: plan is NULL");
  if (!stream) return fail(FRT_ERR_INVALID_ARG, "frt_graph_capture: the null stream cannot be captured");
  if (!p->all_weights() || !p->act_scales_set())
    return fail(FRT_ERR_STATE, "frt_graph_capture: weights and activation scales must be set first");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  p->drop_graph();
  HIP_CHECK(hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed));
  frt_status st = forward_range(p, 0, p->d.L, s);
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(s, &graph);
  if (st != FRT_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (e != hipSuccess) return fail(FRT_ERR_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(FRT_ERR_HIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
  }
  p->graph = graph;
  p->exec = exec;
  p->captured = true;
  p->stale = false;
  return FRT_OK;
}

frt_status frt_graph_replay(frt_plan* p, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_graph_replay: plan is NULL");
  if (!p->captured) return fail(FRT_ERR_STATE, "frt_graph_replay: No graph captured");
  if (p->stale)
    return fail(FRT_ERR_STATE, "frt_graph_replay: graph is stale (weights or scales changed); capture again");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  HIP_CHECK(hipGraphLaunch(p->exec, static_cast<hipStream_t>(stream)));
  return FRT_OK;
}

frt_status frt_e4m3_encode_f32(const void* d_in, void* d_out, int64_t n, void* stream) {
  if ((!d_in || !d_out) && n > 0) return fail(FRT_ERR_INVALID_ARG, "frt_e4m3_encode_f32: NULL pointer");
  if (n < 0) return fail(FRT_ERR_INVALID_ARG, "frt_e4m3_encode_f32: negative length");
  KERNEL_CHECK(launch_e4m3_encode(static_cast<const float*>(d_in), static_cast<uint8_t*>(d_out), n,
                                  static_cast<hipStream_t>(stream)), "e4m3_encode");
  return FRT_OK;
}

}  // extern "C"
