// frt_qkv.hip -- host side of the attention-input C ABI (include/frt_qkv.h):
// K1 (residual add + RMSNorm + E4M3) followed by the fused QKV projection
// with the split + rotary epilogue.
//
// FlashRT architecture doc, "Kernel library" (the "qkv split + RoPE"
// fusion) and "CUDA Graph" (pointer-only forward, no allocation at replay);
// itsolotime article section 5.2 (FusedQKV weight, norm fold for Pi0,
// AdaRMSNorm for Pi0.5).
//
// Like the FFN plan, this plan never allocates device memory: every buffer
// is carved out of the caller's workspace.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <new>
#include <vector>

#include "../../include/frt_qkv.h"
#include "frt_host.h"
#include "frt_qkv_dev.h"

namespace frt {
hipError_t launch_add_rmsnorm_quant(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*,
                                    uint8_t*, int, int, float, float, hipStream_t, const float*, int, float,
                                    uint16_t*);
hipError_t launch_add_rmsnorm_measure(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                                      uint16_t*, float*, float*, int, int, float, hipStream_t);
hipError_t launch_amax_bf16(const uint16_t*, size_t, float*, hipStream_t, const uint16_t*, size_t);
hipError_t launch_rope_table(float2*, int, int, double, hipStream_t);
hipError_t launch_quant_pack_qkv(const uint16_t*, uint8_t*, int, int, float, int, int, int, const uint16_t*,
                                 hipStream_t, int);
hipError_t launch_gemv_qkv(const uint8_t*, const uint8_t*, const QkvOut&, int, int, int, hipStream_t, int);
hipError_t launch_mm_qkv(int, const uint8_t*, const uint8_t*, const QkvOut&, int, int, int, hipStream_t);
hipError_t launch_add_sumsq(const uint16_t*, const uint16_t*, const float*, int, float, uint16_t*, uint16_t*, double*,
                            int, int, hipStream_t, int = 0);
int add_sumsq_slices(int);
bool gemv_qkv_nq_supported(int, int, int);
hipError_t launch_gemv_qkv_nq(const uint16_t*, const uint16_t*, const double*, int, float, float, uint8_t*,
                              const uint8_t*, const QkvOut&, int, int, int, hipStream_t);
}  // namespace frt

using namespace frt;

namespace {

constexpr int kQkvGemvMaxM = 64;  // the multi-tile GEMV up to here, the LDS-DMA GEMM above

bool qkv_desc_ok(const frt_qkv_desc* d) {
  if (!d) return false;
  if (d->M < 1 || d->H < 128 || d->H % 128 || d->H > 16384) return false;
  if (d->nq < 1 || d->nkv < 1 || d->nq > 1024 || d->nkv > 1024) return false;
  if (d->hd < 32 || d->hd % 32 || d->hd > 512) return false;
  if (d->max_pos < 1 || d->max_pos > (1 << 24)) return false;
  if (!(d->eps > 0.0f) || !std::isfinite(d->eps)) return false;
  if (!(d->rope_base > 1.0f) || !std::isfinite(d->rope_base)) return false;
  if (d->device < 0) return false;
  if (d->flags & ~(uint32_t)(FRT_FLAG_NORM_FUSE | FRT_FLAG_ADA_NORM)) return false;
  if ((d->flags & FRT_FLAG_NORM_FUSE) && (d->flags & FRT_FLAG_ADA_NORM)) return false;
  const int64_t N = (int64_t)(d->nq + 2 * d->nkv) * d->hd;
  if (N > 65536 || (int64_t)d->M * N > ((int64_t)1 << 31)) return false;
  // activation offsets inside the kernels are 32-bit
  if ((int64_t)d->M * d->H > ((int64_t)1 << 31)) return false;
  return true;
}

struct QkvLayout {
  size_t w, wn, mod, rope, r_in, y_in, pos, r_out, xq, q, k, v, amax, cal_x, cal_r, sqp, total;
  bool norm_split;  // M <= 16: k_add_sumsq, then the QKV GEMV quantises its own K blocks (k_gemv_qkv_nq)
  int gemv_w;  // GEMV waves per workgroup (M <= 64)
  bool oct;    // the GEMV (M <= 64, no split norm) over the octet-ordered weight, one group per workgroup
  int mm_cfg;  // LDS-DMA GEMM configuration (M > 64)
};

// GEMV waves: the smallest of 4, 8, 16 that gives about `target` waves
// across the workgroups (pairs: 1280, measured: 4 waves on the 320 pairs of
// the decode shape beat 16 by 12%, 8 on the 80 pairs of the action-expert
// shape; octet groups: 4096, 8 waves on the 640 groups of the decode shape
// 9.68-9.78 us against 9.89-9.91 with 4), at most the K blocks, 8 above
// M = 32.
int qkv_gemv_waves(int pairs, int kblocks, int M, int target = 1280) {
  int w = env_int("FRT_QKV_GEMV_WAVES", 0);
  if (w != 4 && w != 8 && w != 16) {
    w = 4;
    while (w < 16 && pairs * w < target) w *= 2;
    while (w > 4 && w > kblocks) w /= 2;
  }
  if (w == 16 && M > 32) w = 8;
  return w;
}

QkvLayout qkv_layout(const frt_qkv_desc& d) {
  QkvLayout lo{};
  const size_t M = d.M, H = d.H, N = (size_t)(d.nq + 2 * d.nkv) * d.hd;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + (bytes ? bytes : 1));
    return at;
  };
  lo.w = take(N * H);
  lo.wn = take(H * 2);
  lo.mod = take(2 * H * 2);
  lo.rope = take((size_t)d.max_pos * (d.hd / 2) * 8);
  lo.r_in = take(M * H * 2);
  lo.y_in = take(M * H * 2);
  lo.pos = take(M * 4);
  lo.r_out = take(M * H * 2);
  lo.xq = take(M * H);
  lo.q = take(M * d.nq * d.hd * 2);
  lo.k = take(M * d.nkv * d.hd * 2);
  lo.v = take(M * d.nkv * d.hd * 2);
  lo.amax = take(256);
  lo.cal_x = take(M * H * 4);
  lo.cal_r = take(M * H * 2);
  lo.sqp = take(M * (size_t)add_sumsq_slices(d.H) * 8);
  lo.total = off;
  lo.gemv_w = qkv_gemv_waves((int)(N / 32), d.H / 128, d.M);
  // Opt-in (FRT_QKV_NORM_SPLIT=1): the decode norm in two parts, as on the
  // FFN plan.  The per-block graph replay that the benchmark times is bound
  // by the host's graph launch (about 27 us against 14 us of kernels), so
  // the gain the FFN chain shows (2 us per layer) could not be measured here
  // and the one-kernel norm stays the default.
  lo.norm_split = d.M <= 16 && (d.flags & FRT_FLAG_ADA_NORM) == 0u &&
                  gemv_qkv_nq_supported(d.M, d.H, add_sumsq_slices(d.H)) && lo.gemv_w <= d.H / 128 &&
                  env_int("FRT_QKV_NORM_SPLIT", 0) != 0;
  // the plain decode GEMV over the octet-ordered weight: one 16-row group
  // (eight rotation pairs, or sixteen v rows) per workgroup, twice the
  // workgroups of the pair order; FRT_QKV_OCT=0 keeps pairs
  lo.oct = d.M <= kQkvGemvMaxM && !lo.norm_split && env_int("FRT_QKV_OCT", 1) != 0;
  if (lo.oct) lo.gemv_w = qkv_gemv_waves((int)(N / 16), d.H / 128, d.M, 4096);
  lo.mm_cfg = -1;
  if (d.M > kQkvGemvMaxM) {
    int c = -1, sp = 1;
    choose_mm(d.M, (int)N, d.H, false, c, sp, kMMConfigCountAll);
    // a short output leaves CUs idle under the chosen tiles: take 64 x 128
    // tiles (measured at M=788, N=2560: 20.3 us against 23.3 us for 128 x 128)
    if (c >= 0 && (int)(N / mm_config_bn(c)) * ceil_div(d.M, mm_config_bm(c)) < 256 && N % mm_config_bn(6) == 0)
      c = 6;
    c = env_int("FRT_MM_QKV_CFG", c);
    if (c >= 0 && c < kMMConfigCountAll && N % mm_config_bn(c) == 0 && d.H % mm_config_ks(c) == 0) lo.mm_cfg = c;
  }
  return lo;
}

}  // namespace

struct frt_qkv_plan {
  frt_qkv_desc d{};
  QkvLayout lo{};
  uint8_t* ws = nullptr;
  float s_x = 0.0f, s_w = 0.0f;
  bool w_set = false;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  bool captured = false, stale = false;

  int N() const { return (d.nq + 2 * d.nkv) * d.hd; }
  bool ada() const { return (d.flags & FRT_FLAG_ADA_NORM) != 0u; }
  bool norm_fuse() const { return (d.flags & FRT_FLAG_NORM_FUSE) != 0u; }
  template <class T>
  T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  QkvOut out() const {
    QkvOut o;
    o.pos = at<const int32_t>(lo.pos);
    o.rope = at<const float2>(lo.rope);
    o.q = at<uint16_t>(lo.q);
    o.k = at<uint16_t>(lo.k);
    o.v = at<uint16_t>(lo.v);
    o.max_pos = d.max_pos;
    o.nq = d.nq;
    o.nkv = d.nkv;
    o.hd = d.hd;
    o.alpha = s_x * s_w;
    return o;
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

static frt_status qkv_launch(frt_qkv_plan* p, int which, hipStream_t s) {
  const int M = p->d.M, H = p->d.H;
  if (which == 0 && p->lo.norm_split) {
    KERNEL_CHECK(launch_add_sumsq(p->at<uint16_t>(p->lo.r_in), p->at<uint16_t>(p->lo.y_in), nullptr, 1, 0.0f, nullptr,
                                  p->at<uint16_t>(p->lo.r_out), p->at<double>(p->lo.sqp), M, H, s),
                 "add_sumsq");
  } else if (which == 0) {
    const float inv_x = 1.0f / p->s_x;
    KERNEL_CHECK(launch_add_rmsnorm_quant(p->at<uint16_t>(p->lo.r_in), p->at<uint16_t>(p->lo.y_in),
                                          p->at<uint16_t>(p->lo.wn), p->ada() ? p->at<uint16_t>(p->lo.mod) : nullptr,
                                          p->at<uint16_t>(p->lo.r_out), p->at<uint8_t>(p->lo.xq), M, H, p->d.eps,
                                          inv_x, s, nullptr, 1, 0.0f, nullptr),
                 "add_rmsnorm_quant");
  } else if (p->lo.norm_split) {
    KERNEL_CHECK(launch_gemv_qkv_nq(p->at<uint16_t>(p->lo.r_out), p->at<uint16_t>(p->lo.wn), p->at<double>(p->lo.sqp),
                                    add_sumsq_slices(H), p->d.eps, 1.0f / p->s_x, p->at<uint8_t>(p->lo.xq),
                                    p->at<uint8_t>(p->lo.w), p->out(), M, H, p->lo.gemv_w, s),
                 "gemv_qkv_nq");
  } else if (M <= kQkvGemvMaxM) {
    KERNEL_CHECK(launch_gemv_qkv(p->at<uint8_t>(p->lo.xq), p->at<uint8_t>(p->lo.w), p->out(), M, H, p->lo.gemv_w, s,
                                 p->lo.oct ? 1 : 0),
                 "gemv_qkv");
  } else {
    KERNEL_CHECK(launch_mm_qkv(p->lo.mm_cfg, p->at<uint8_t>(p->lo.xq), p->at<uint8_t>(p->lo.w), p->out(), M, H,
                               p->N(), s),
                 "mm_qkv");
  }
  return FRT_OK;
}

static frt_status qkv_ready(const frt_qkv_plan* p, const char* who) {
  if (!p->w_set || !(p->s_x > 0.0f))
    return fail(FRT_ERR_STATE, "%s: weights and the activation scale must be set first", who);
  return FRT_OK;
}

extern "C" {

frt_status frt_qkv_workspace_size(const frt_qkv_desc* desc, size_t* bytes) {
  if (!bytes) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_workspace_size: bytes is NULL");
  if (!qkv_desc_ok(desc)) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_workspace_size: invalid descriptor");
  *bytes = qkv_layout(*desc).total;
  return FRT_OK;
}

frt_status frt_qkv_plan_create(const frt_qkv_desc* desc, void* d_workspace, size_t bytes, frt_qkv_plan** out) {
  if (!out) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_plan_create: out is NULL");
  *out = nullptr;
  if (!qkv_desc_ok(desc)) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_plan_create: invalid descriptor");
  if (!d_workspace) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_plan_create: workspace is NULL");
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256)
    return fail(FRT_ERR_WORKSPACE, "frt_qkv_plan_create: workspace not 256-byte aligned");
  const QkvLayout lo = qkv_layout(*desc);
  if (bytes < lo.total)
    return fail(FRT_ERR_WORKSPACE, "frt_qkv_plan_create: workspace %zu bytes, need %zu", bytes, lo.total);
  if (lo.mm_cfg < 0 && desc->M > kQkvGemvMaxM)
    return fail(FRT_ERR_UNSUPPORTED, "frt_qkv_plan_create: no GEMM tile divides N = %d",
                (desc->nq + 2 * desc->nkv) * desc->hd);
  DeviceGuard g(desc->device);
  HIP_CHECK(g.err);
  frt_qkv_plan* p = new (std::nothrow) frt_qkv_plan();
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_plan_create: out of host memory");
  p->d = *desc;
  p->lo = lo;
  p->ws = static_cast<uint8_t*>(d_workspace);
  hipError_t e = hipMemset(p->ws, 0, lo.total);
  if (e == hipSuccess) e = launch_rope_table(p->at<float2>(lo.rope), desc->max_pos, desc->hd, (double)desc->rope_base,
                                             nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    delete p;
    return fail(FRT_ERR_HIP, "frt_qkv_plan_create: %s", hipGetErrorString(e));
  }
  *out = p;
  return FRT_OK;
}

frt_status frt_qkv_plan_destroy(frt_qkv_plan* p) {
  if (!p) return FRT_OK;
  {
    DeviceGuard g(p->d.device);
    p->drop_graph();
  }
  delete p;
  return FRT_OK;
}

frt_status frt_qkv_quant_weights(frt_qkv_plan* p, const void* d_wq, const void* d_wk, const void* d_wv,
                                 const void* d_norm_w, void* stream) {
  if (!p || !d_wq || !d_wk || !d_wv || !d_norm_w) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_quant_weights: NULL argument");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = p->d.H, hd = p->d.hd;
  const int rows[3] = {p->d.nq * hd, p->d.nkv * hd, p->d.nkv * hd};
  const uint16_t* src[3] = {static_cast<const uint16_t*>(d_wq), static_cast<const uint16_t*>(d_wk),
                            static_cast<const uint16_t*>(d_wv)};
  const uint16_t* fold = p->norm_fuse() ? static_cast<const uint16_t*>(d_norm_w) : nullptr;
  float* am = p->at<float>(p->lo.amax);
  HIP_CHECK(hipMemsetAsync(am, 0, sizeof(float), s));
  for (int t = 0; t < 3; ++t)
    KERNEL_CHECK(launch_amax_bf16(src[t], (size_t)rows[t] * H, am, s, fold, (size_t)H), "amax_bf16");
  float amax = 0.0f;
  HIP_CHECK(hipMemcpyAsync(&amax, am, sizeof(float), hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  if (!std::isfinite(amax)) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_quant_weights: non-finite weight");
  const float sw = amax > 0.0f ? amax / 448.0f : 1.0f;
  const float inv = 1.0f / sw;
  const int n_rope = (p->d.nq + p->d.nkv) * hd;
  int base = 0;
  for (int t = 0; t < 3; ++t) {
    KERNEL_CHECK(launch_quant_pack_qkv(src[t], p->at<uint8_t>(p->lo.w), rows[t], H, inv, base, hd, n_rope, fold, s,
                                       p->lo.oct ? 1 : 0),
                 "quant_pack_qkv");
    base += rows[t];
  }
  if (p->norm_fuse())
    HIP_CHECK(hipMemsetD16Async(reinterpret_cast<hipDeviceptr_t>(p->at<uint16_t>(p->lo.wn)), 0x3F80u, (size_t)H, s));
  else
    HIP_CHECK(hipMemcpyAsync(p->at<uint16_t>(p->lo.wn), d_norm_w, (size_t)H * 2, hipMemcpyDeviceToDevice, s));
  HIP_CHECK(hipStreamSynchronize(s));
  p->s_w = sw;
  p->w_set = true;
  p->mark_stale();
  return FRT_OK;
}

frt_status frt_qkv_export_weight_codes(const frt_qkv_plan* p, void* host_dst) {
  if (!p || !host_dst) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_export_weight_codes: NULL argument");
  if (!p->w_set) return fail(FRT_ERR_STATE, "frt_qkv_export_weight_codes: weights not quantised");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  const uint32_t N = (uint32_t)p->N(), H = (uint32_t)p->d.H, hd = (uint32_t)p->d.hd;
  const uint32_t n_rope = (uint32_t)(p->d.nq + p->d.nkv) * hd;
  std::vector<uint8_t> tmp;
  try {
    tmp.resize((size_t)N * H);
  } catch (...) {
    return fail(FRT_ERR_INVALID_ARG, "frt_qkv_export_weight_codes: out of host memory");
  }
  HIP_CHECK(hipMemcpy(tmp.data(), p->at<uint8_t>(p->lo.w), tmp.size(), hipMemcpyDeviceToHost));
  uint8_t* dst = static_cast<uint8_t*>(host_dst);
  for (uint32_t n = 0; n < N; ++n) {
    const uint32_t pr = p->lo.oct ? qkv_packed_row_oct(n, hd, n_rope) : qkv_packed_row(n, hd, n_rope);
    for (uint32_t k = 0; k < H; ++k) dst[(size_t)n * H + k] = tmp[packed_offset(pr, k, H)];
  }
  return FRT_OK;
}

frt_status frt_qkv_calibrate(frt_qkv_plan* p, const void* const* d_r_batches, const void* const* d_y_batches,
                             int32_t nbatch, int32_t rows, void* stream) {
  if (!p || !d_r_batches) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_calibrate: NULL argument");
  if (nbatch < 1 || rows < 1 || rows > p->d.M)
    return fail(FRT_ERR_INVALID_ARG, "frt_qkv_calibrate: nbatch %d rows %d (1..%d)", nbatch, rows, p->d.M);
  for (int b = 0; b < nbatch; ++b)
    if (!d_r_batches[b]) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_calibrate: batch %d residual is NULL", b);
  if (!p->w_set) return fail(FRT_ERR_STATE, "frt_qkv_calibrate: weights not set");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* am = p->at<float>(p->lo.amax) + 1;
  HIP_CHECK(hipMemsetAsync(am, 0, sizeof(float), s));
  for (int b = 0; b < nbatch; ++b) {
    const uint16_t* y = d_y_batches ? static_cast<const uint16_t*>(d_y_batches[b]) : nullptr;
    KERNEL_CHECK(launch_add_rmsnorm_measure(static_cast<const uint16_t*>(d_r_batches[b]), y,
                                            p->at<uint16_t>(p->lo.wn), p->ada() ? p->at<uint16_t>(p->lo.mod) : nullptr,
                                            p->at<uint16_t>(p->lo.cal_r), p->at<float>(p->lo.cal_x), am, rows,
                                            p->d.H, p->d.eps, s),
                 "add_rmsnorm_measure");
  }
  float amax = 0.0f;
  HIP_CHECK(hipMemcpyAsync(&amax, am, sizeof(float), hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  if (!std::isfinite(amax)) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_calibrate: non-finite activation");
  p->s_x = amax > 0.0f ? amax / 448.0f : 1.0f;
  p->mark_stale();
  return FRT_OK;
}

frt_status frt_qkv_get_scales(const frt_qkv_plan* p, float* host_out) {
  if (!p || !host_out) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_get_scales: NULL argument");
  host_out[0] = p->s_x;
  host_out[1] = p->s_w;
  return FRT_OK;
}

frt_status frt_qkv_set_act_scale(frt_qkv_plan* p, float s_x) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_set_act_scale: plan is NULL");
  if (!std::isfinite(s_x) || !(s_x > 0.0f))
    return fail(FRT_ERR_INVALID_ARG, "frt_qkv_set_act_scale: scale must be finite and positive");
  p->s_x = s_x;
  p->mark_stale();
  return FRT_OK;
}

frt_status frt_qkv_set_positions(frt_qkv_plan* p, const int32_t* host_pos, void* stream) {
  if (!p || !host_pos) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_set_positions: NULL argument");
  for (int m = 0; m < p->d.M; ++m)
    if (host_pos[m] < 0 || host_pos[m] >= p->d.max_pos)
      return fail(FRT_ERR_INVALID_ARG, "frt_qkv_set_positions: position %d of row %d outside [0, %d)", host_pos[m], m,
                  p->d.max_pos);
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_CHECK(hipMemcpyAsync(p->at<int32_t>(p->lo.pos), host_pos, sizeof(int32_t) * p->d.M, hipMemcpyHostToDevice, s));
  HIP_CHECK(hipStreamSynchronize(s));
  return FRT_OK;
}

frt_status frt_qkv_io_get(const frt_qkv_plan* p, frt_qkv_io* out) {
  if (!p || !out) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_io_get: NULL argument");
  out->r_in = p->ws + p->lo.r_in;
  out->y_in = p->ws + p->lo.y_in;
  out->pos = p->ws + p->lo.pos;
  out->mod = p->ada() ? p->ws + p->lo.mod : nullptr;
  out->r_out = p->ws + p->lo.r_out;
  out->xq = p->ws + p->lo.xq;
  out->q = p->ws + p->lo.q;
  out->k = p->ws + p->lo.k;
  out->v = p->ws + p->lo.v;
  out->rope = p->ws + p->lo.rope;
  return FRT_OK;
}

frt_status frt_qkv_forward(frt_qkv_plan* p, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_forward: plan is NULL");
  frt_status st = qkv_ready(p, "frt_qkv_forward");
  if (st != FRT_OK) return st;
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = qkv_launch(p, 0, s)) != FRT_OK) return st;
  return qkv_launch(p, 1, s);
}

frt_status frt_qkv_time_kernel(frt_qkv_plan* p, int32_t which, int32_t reps, void* stream, float* avg_us) {
  if (!p || !avg_us) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_time_kernel: NULL argument");
  if (which < 0 || which > 1 || reps < 1)
    return fail(FRT_ERR_INVALID_ARG, "frt_qkv_time_kernel: which %d reps %d", which, reps);
  frt_status st = qkv_ready(p, "frt_qkv_time_kernel");
  if (st != FRT_OK) return st;
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
  float ms = 0.0f;
  err = hipEventRecord(e0, s);
  for (int r = 0; r < reps && st == FRT_OK && err == hipSuccess; ++r) st = qkv_launch(p, which, s);
  if (err == hipSuccess && st == FRT_OK) err = hipEventRecord(e1, s);
  if (err == hipSuccess && st == FRT_OK) err = hipEventSynchronize(e1);
  if (err == hipSuccess && st == FRT_OK) err = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != FRT_OK) return st;
  if (err != hipSuccess) return fail(FRT_ERR_HIP, "frt_qkv_time_kernel: event timing failed: %s", hipGetErrorString(err));
  *avg_us = ms * 1000.0f / (float)reps;
  return FRT_OK;
}

frt_status frt_qkv_graph_capture(frt_qkv_plan* p, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_graph_capture: plan is NULL");
  if (!stream) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_graph_capture: the null stream cannot be captured");
  frt_status st = qkv_ready(p, "frt_qkv_graph_capture");
  if (st != FRT_OK) return st;
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  p->drop_graph();
  HIP_CHECK(hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed));
  st = qkv_launch(p, 0, s);
  if (st == FRT_OK) st = qkv_launch(p, 1, s);
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

frt_status frt_qkv_graph_replay(frt_qkv_plan* p, void* stream) {
  if (!p) return fail(FRT_ERR_INVALID_ARG, "frt_qkv_graph_replay: plan is NULL");
  if (!p->captured) return fail(FRT_ERR_STATE, "frt_qkv_graph_replay: No graph captured");
  if (p->stale)
    return fail(FRT_ERR_STATE, "frt_qkv_graph_replay: graph is stale (weights or scale changed); capture again");
  DeviceGuard g(p->d.device);
  HIP_CHECK(g.err);
  HIP_CHECK(hipGraphLaunch(p->exec, static_cast<hipStream_t>(stream)));
  return FRT_OK;
}

}  // extern "C"
