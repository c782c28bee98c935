// k_quant.hip -- per-tensor E4M3 weight quantisation into the packed layout.
//
// FlashRT architecture doc, component "Weights" (declarative transforms:
// transpose and Quant() per tensor, per-tensor scales collected into one
// table); itsolotime article, section 5.2 (FusedGateUp: gate and up fused
// into one FP8 operand per layer).  Per tensor T (bf16, [N][K]):
//   amax = max |T|                  (exact: a max of bf16 values)
//   s    = amax > 0 ? f32(amax / 448) : 1,  inv = f32(1 / s)   (host scalars)
//   code = e4m3(f32(T * inv))
// The codes are written straight into the MFMA fragment layout described in
// frt_device.h; gate and up rows interleave in 16-row groups.
#include "frt_device.h"

namespace frt {

// amax over n bf16 values (n % 8 == 0), max-accumulated into *out (>= 0).
__global__ __launch_bounds__(256) void k_amax_bf16(const uint16_t* __restrict__ w, size_t n8,
                                                   float* __restrict__ out) {
  float m = 0.0f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    uint4 v = reinterpret_cast<const uint4*>(w)[i];
    uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_lo(a[j])));
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_hi(a[j])));
    }
  }
  m = wave_max_f32(m);
  if ((threadIdx.x & 63) == 0) atomic_max_nonneg(out, m);
}

// Quantise src [N][K] bf16 with factor inv and scatter 16-column pieces into
// the packed matrix; source row n lands on packed row
//   mode 0: n (plain), 1: gate_row(n), 2: up_row_gated(n).
__global__ __launch_bounds__(256) void k_quant_pack(const uint16_t* __restrict__ src,
                                                    uint8_t* __restrict__ dst, int N, int K,
                                                    float inv, int mode) {
  const size_t pieces_per_row = (size_t)K / 16;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)N * pieces_per_row) return;
  const uint32_t n = (uint32_t)(idx / pieces_per_row);
  const uint32_t k0 = (uint32_t)(idx % pieces_per_row) * 16u;
  const uint4* s = reinterpret_cast<const uint4*>(src + (size_t)n * K + k0);
  uint4 a = s[0], b = s[1];
  uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    q[j] = e4m3x4(bf16_lo(v[2 * j]) * inv, bf16_hi(v[2 * j]) * inv, bf16_lo(v[2 * j + 1]) * inv,
                  bf16_hi(v[2 * j + 1]) * inv);
  const uint32_t prow = mode == 0 ? n : (mode == 1 ? gate_row(n) : up_row_gated(n));
  *reinterpret_cast<uint4*>(dst + packed_offset(prow, k0, (uint32_t)K)) =
      make_uint4(q[0], q[1], q[2], q[3]);
}

hipError_t launch_amax_bf16(const uint16_t* w, size_t n, float* out, hipStream_t s) {
  size_t n8 = n / 8;
  unsigned blocks = (unsigned)((n8 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_amax_bf16, dim3(blocks), dim3(256), 0, s, w, n8, out);
  return hipGetLastError();
}

hipError_t launch_quant_pack(const uint16_t* src, uint8_t* dst, int N, int K, float inv, int mode,
                             hipStream_t s) {
  size_t pieces = (size_t)N * (K / 16);
  hipLaunchKernelGGL(k_quant_pack, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, src,
                     dst, N, K, inv, mode);
  return hipGetLastError();
}

}  // namespace frt
