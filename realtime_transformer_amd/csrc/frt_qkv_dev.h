// frt_qkv_dev.h -- device pieces of the attention-input path shared by its
// GEMV (k_qkv.hip) and the prefill GEMM's epilogue (k_mm.hip): the packed
// row order of the fused QKV weight and the split + rotary epilogue.
//
// FlashRT architecture doc, "Kernel library": the "qkv split + RoPE" fusion;
// itsolotime article section 5.2: the FusedQKV weight with head interleave.
//
// Packed order.  The fused rows [q heads; k heads; v heads] go into 16-row
// groups taken in pairs: pair p of a q or k head h holds, in its first group,
// dimensions 16j .. 16j+15 of head h and, in its second group, dimensions
// hd/2 + 16j .. hd/2 + 16j+15 (j = p mod hd/32), so each rotation pair
// (d, d + hd/2) lands in the same lane of the matrix-core output (as gate and
// up do in the FFN).  v rows follow in plain order, 32 per pair.
#pragma once
#include "frt_device.h"

namespace frt {

struct QkvOut {
  const int32_t* pos;   // [M] rotary positions
  const float2* rope;   // [max_pos][hd/2] (cos, sin)
  uint16_t* q;          // [M][nq][hd]
  uint16_t* k;          // [M][nkv][hd]
  uint16_t* v;          // [M][nkv][hd]
  int max_pos, nq, nkv, hd;
  float alpha;          // s_x * s_w
};

// packed row of fused row n ((nq + nkv) * hd = n_rope rows are rotated)
__host__ __device__ __forceinline__ uint32_t qkv_packed_row(uint32_t n, uint32_t hd, uint32_t n_rope) {
  if (n < n_rope) {
    const uint32_t head = n / hd, d = n - head * hd, half = hd >> 1;
    const uint32_t hb = d >= half ? 1u : 0u, dd = d - hb * half;
    const uint32_t pair = head * (hd >> 5) + (dd >> 4);
    return (2u * pair + hb) * 16u + (dd & 15u);
  }
  const uint32_t nv = n - n_rope;
  const uint32_t pair = (n_rope >> 5) + (nv >> 5);
  return (2u * pair + ((nv >> 4) & 1u)) * 16u + (nv & 15u);
}

// ... in the octet order of the decode GEMV's one-group workgroups: group g
// of a q or k head holds dimensions 8j .. 8j+7 (j = g mod hd/16) in its first
// eight rows and their partners hd/2 + 8j .. hd/2 + 8j+7 in the last eight;
// v rows follow in plain order, 16 per group.
__host__ __device__ __forceinline__ uint32_t qkv_packed_row_oct(uint32_t n, uint32_t hd, uint32_t n_rope) {
  if (n < n_rope) {
    const uint32_t head = n / hd, d = n - head * hd, half = hd >> 1;
    const uint32_t hb = d >= half ? 1u : 0u, dd = d - hb * half;
    const uint32_t g = head * (hd >> 4) + (dd >> 3);
    return g * 16u + hb * 8u + (dd & 7u);
  }
  return n;  // (n_rope is a multiple of 16: v rows keep their places)
}

__device__ __forceinline__ int qkv_clamp_pos(const QkvOut& o, int m) {
  const int ps = o.pos[m];
  return ps < 0 ? 0 : (ps >= o.max_pos ? o.max_pos - 1 : ps);
}

// Row m, pair p, lane row rho (0..15) of the pair's groups: the two fp32
// accumulators of that lane (first group, second group).
//   q/k: out[d] = bf16(x1 c - x2 s), out[d + hd/2] = bf16(x2 c + x1 s)
//   v:   out[n] = bf16(x1), out[n + 16] = bf16(x2)
// with x = f32(acc * alpha) and every product rounded on its own.
__device__ __forceinline__ void qkv_store(const QkvOut& o, int m, int p, int rho, float first, float second) {
  const int pph = o.hd >> 5;
  const int nrp = (o.nq + o.nkv) * pph;
  const float x1 = first * o.alpha, x2 = second * o.alpha;
  if (p < nrp) {
    const int head = p / pph, j = p - head * pph, half = o.hd >> 1;
    const int d = 16 * j + rho;
    const float2 cs = o.rope[(size_t)qkv_clamp_pos(o, m) * half + d];
    const float x1c = x1 * cs.x, x2s = x2 * cs.y, x2c = x2 * cs.x, x1s = x1 * cs.y;
    uint16_t* dst = head < o.nq ? o.q + ((size_t)m * o.nq + head) * o.hd
                                : o.k + ((size_t)m * o.nkv + (head - o.nq)) * o.hd;
    dst[d] = (uint16_t)f32_to_bf16(x1c - x2s);
    dst[d + half] = (uint16_t)f32_to_bf16(x2c + x1s);
  } else {
    const int nv = 32 * (p - nrp) + rho;
    uint16_t* dst = o.v + (size_t)m * o.nkv * o.hd;
    dst[nv] = (uint16_t)f32_to_bf16(x1);
    dst[nv + 16] = (uint16_t)f32_to_bf16(x2);
  }
}

// Octet order: row m, group g, lane row rho of the group's accumulator,
// with `partner` the accumulator of lane row rho ^ 8.  q/k groups: rows
// rho < 8 store dimension 8j + rho and its partner (the rotation as in
// qkv_store); v groups: every row stores its own value.
__device__ __forceinline__ void qkv_store_oct(const QkvOut& o, int m, int g, int rho, float acc, float partner) {
  const int gph = o.hd >> 4;
  const int nrg = (o.nq + o.nkv) * gph;
  if (g < nrg) {
    if (rho >= 8) return;
    const int head = g / gph, j = g - head * gph, half = o.hd >> 1;
    const int d = 8 * j + rho;
    const float x1 = acc * o.alpha, x2 = partner * o.alpha;
    const float2 cs = o.rope[(size_t)qkv_clamp_pos(o, m) * half + d];
    const float x1c = x1 * cs.x, x2s = x2 * cs.y, x2c = x2 * cs.x, x1s = x1 * cs.y;
    uint16_t* dst = head < o.nq ? o.q + ((size_t)m * o.nq + head) * o.hd
                                : o.k + ((size_t)m * o.nkv + (head - o.nq)) * o.hd;
    dst[d] = (uint16_t)f32_to_bf16(x1c - x2s);
    dst[d + half] = (uint16_t)f32_to_bf16(x2c + x1s);
  } else {
    const int nv = 16 * (g - nrg) + rho;
    o.v[(size_t)m * o.nkv * o.hd + nv] = (uint16_t)f32_to_bf16(acc * o.alpha);
  }
}

// Four consecutive lane rows rho0 .. rho0+3 (rho0 % 4 == 0) of one row m:
// the same values as four qkv_store calls, stored 8 bytes at a time.
__device__ __forceinline__ void qkv_store4(const QkvOut& o, int m, int p, int rho0, const float first[4],
                                           const float second[4]) {
  const int pph = o.hd >> 5;
  const int nrp = (o.nq + o.nkv) * pph;
  float x1[4], x2[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x1[r] = first[r] * o.alpha;
    x2[r] = second[r] * o.alpha;
  }
  if (p < nrp) {
    const int head = p / pph, j = p - head * pph, half = o.hd >> 1;
    const int d = 16 * j + rho0;
    const float4* t = reinterpret_cast<const float4*>(o.rope + (size_t)qkv_clamp_pos(o, m) * half + d);
    const float4 t0 = t[0], t1 = t[1];
    const float c[4] = {t0.x, t0.z, t1.x, t1.z}, s[4] = {t0.y, t0.w, t1.y, t1.w};
    float lo[4], hi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x1c = x1[r] * c[r], x2s = x2[r] * s[r], x2c = x2[r] * c[r], x1s = x1[r] * s[r];
      lo[r] = x1c - x2s;
      hi[r] = x2c + x1s;
    }
    uint16_t* dst = head < o.nq ? o.q + ((size_t)m * o.nq + head) * o.hd
                                : o.k + ((size_t)m * o.nkv + (head - o.nq)) * o.hd;
    *reinterpret_cast<uint2*>(dst + d) = make_uint2(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]));
    *reinterpret_cast<uint2*>(dst + d + half) = make_uint2(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));
  } else {
    const int nv = 32 * (p - nrp) + rho0;
    uint16_t* dst = o.v + (size_t)m * o.nkv * o.hd;
    *reinterpret_cast<uint2*>(dst + nv) = make_uint2(pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3]));
    *reinterpret_cast<uint2*>(dst + nv + 16) = make_uint2(pack_bf16x2(x2[0], x2[1]), pack_bf16x2(x2[2], x2[3]));
  }
}

}  // namespace frt
