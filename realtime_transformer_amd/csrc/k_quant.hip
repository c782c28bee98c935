// k_quant.hip -- per-tensor E4M3 weight quantisation into the packed layout.
//
// FlashRT architecture doc, component "Weights" (declarative transforms:
// transpose and Quant() per tensor, per-tensor scales collected into one
// table); itsolotime article, section 5.2 (FusedGateUp: gate and up fused
// into one FP8 operand per layer).  Per tensor T (bf16, [N][K]):
//   amax = max |T|                  (exact: a max of bf16 values)
//   s    = amax > 0 ? f32(amax / 448) : 1,  inv = f32(1 / s)   (host scalars)
//   code = e4m3(f32(T * inv))
// (with norm fusion T[n][k] is f32(W[n][k] * w_norm[k]), see below)
// The codes are written straight into the MFMA fragment layout described in
// frt_device.h; gate and up rows interleave in 16-row groups.
#include "frt_device.h"

namespace frt {

// Norm fusion (itsolotime article, section 5.2: the Pi0 decoder spec folds
// the RMSNorm weight into the gate/up matrices before Quant()): element
// (n, k) of the tensor is f32(T[n][k] * colw[k]), an exact product of two
// bf16 values; colw == nullptr means the tensor itself.

// amax over n bf16 values (n % 8 == 0, cols % 8 == 0), max-accumulated into
// *out (>= 0).
__global__ __launch_bounds__(256) void k_amax_bf16(const uint16_t* __restrict__ w, size_t n8,
                                                   float* __restrict__ out, const uint16_t* __restrict__ colw,
                                                   size_t cols8) {
  float m = 0.0f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    uint4 v = reinterpret_cast<const uint4*>(w)[i];
    uint32_t a[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[4] = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
    if (colw) {
      const uint4 cv = reinterpret_cast<const uint4*>(colw)[i % cols8];
      c[0] = cv.x; c[1] = cv.y; c[2] = cv.z; c[3] = cv.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_lo(a[j]) * bf16_lo(c[j])));
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_hi(a[j]) * bf16_hi(c[j])));
    }
  }
  m = wave_max_f32(m);
  if ((threadIdx.x & 63) == 0) atomic_max_nonneg(out, m);
}

// Quantise src [N][K] bf16 (times colw[k] when given) with factor inv and
// scatter 16-column pieces into the packed matrix; source row n lands on
// packed row
//   mode 0: n (plain), 1: gate_row(n), 2: up_row_gated(n), 4: gate_row_oct(n),
//   5: up_row_oct(n); mode 3 scatters row n into the column-quad layout.
__global__ __launch_bounds__(256) void k_quant_pack(const uint16_t* __restrict__ src,
                                                    uint8_t* __restrict__ dst, int N, int K,
                                                    float inv, int mode, const uint16_t* __restrict__ colw) {
  const size_t pieces_per_row = (size_t)K / 16;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)N * pieces_per_row) return;
  const uint32_t n = (uint32_t)(idx / pieces_per_row);
  const uint32_t k0 = (uint32_t)(idx % pieces_per_row) * 16u;
  const uint4* s = reinterpret_cast<const uint4*>(src + (size_t)n * K + k0);
  uint4 a = s[0], b = s[1];
  uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = 0x3F803F80u;
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
  // mode 3: the column-quad layout of the whole-column down GEMV
  const uint32_t prow = mode == 0 || mode == 3 ? n
                        : mode == 1            ? gate_row(n)
                        : mode == 2            ? up_row_gated(n)
                        : mode == 4            ? gate_row_oct(n)
                                               : up_row_oct(n);
  const size_t off = mode == 3 ? quad_offset(n, k0, (uint32_t)K) : packed_offset(prow, k0, (uint32_t)K);
  *reinterpret_cast<uint4*>(dst + off) = make_uint4(q[0], q[1], q[2], q[3]);
}

hipError_t launch_amax_bf16(const uint16_t* w, size_t n, float* out, hipStream_t s, const uint16_t* colw,
                            size_t cols) {
  size_t n8 = n / 8;
  if (colw && (cols % 8 || n % cols)) return hipErrorInvalidValue;
  unsigned blocks = (unsigned)((n8 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_amax_bf16, dim3(blocks), dim3(256), 0, s, w, n8, out, colw, colw ? cols / 8 : 1);
  return hipGetLastError();
}

hipError_t launch_quant_pack(const uint16_t* src, uint8_t* dst, int N, int K, float inv, int mode,
                             hipStream_t s, const uint16_t* colw) {
  size_t pieces = (size_t)N * (K / 16);
  hipLaunchKernelGGL(k_quant_pack, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, src,
                     dst, N, K, inv, mode, colw);
  return hipGetLastError();
}

}  // namespace frt
