// k_calib.hip -- the calibration measurement pass (not on the timed path).
//
// FlashRT architecture doc, component "Calibration", phase (a): a
// measurement pass records amax per FP8 GEMM input; the predict() flow's
// cache-miss path runs one forward and records amax.  The measurement
// forward keeps activations unquantised (fp32) and uses the quantised
// weights times their per-tensor scale:
//   g = f32(s_g * (x . dec(Qg))), u = f32(s_u * (x . dec(Qu)))
//   h = act(g) * u  (non-gated: gelu_tanh(u)),  amax_h = max |h|
//   y = bf16(f32(s_d * (h . dec(Qd))))
// amax_x (gate/up input) comes from the measure form of the norm kernel.
//
// The dot products run on the fp32 vector ALUs (FMA, K-sequential per
// output): 64x64 output tile per workgroup, K step 32 staged through LDS, 4x4
// outputs per thread.  Weights are read from the packed fragment layout and
// decoded exactly to fp32.
#include "frt_device.h"

namespace frt {

enum { CAL_GEGLU = 0, CAL_SWIGLU = 1, CAL_GELU = 2, CAL_DOWN = 3 };

template <int MODE>
__device__ __forceinline__ float cal_h(float g, float u) {
  if (MODE == CAL_GELU) return gelu_tanh_f32(u);
  float a = (MODE == CAL_SWIGLU) ? silu_f32(g) : gelu_tanh_f32(g);
  return a * u;
}

// Decode the 16 packed codes of row prow, columns [k0, k0+16) into dst[kk*LD + col]
// (quad: the column-quad layout of the whole-column down GEMV).
__device__ __forceinline__ void load_w16(const uint8_t* __restrict__ w, uint32_t prow, uint32_t k0,
                                         uint32_t K, float* dst, int ld, bool quad) {
  const uint4 v = *reinterpret_cast<const uint4*>(w + (quad ? quad_offset(prow, k0, K) : packed_offset(prow, k0, K)));
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v2f a = e4m3x2_to_f32<false>(d[j]), b = e4m3x2_to_f32<true>(d[j]);
    dst[(4 * j + 0) * ld] = a[0];
    dst[(4 * j + 1) * ld] = a[1];
    dst[(4 * j + 2) * ld] = b[0];
    dst[(4 * j + 3) * ld] = b[1];
  }
}

// X [rows][K] fp32.  Gate/up modes write h [rows][Nout] fp32 and amax|h|;
// CAL_DOWN writes y [rows][Nout] bf16.  Nout is I or H; Nout % 64 == 0.
// layout != 0: the decode plans' orders (gated gate/up: octet rows; down:
// column quads).
template <int MODE>
__global__ __launch_bounds__(256) void k_calib_gemm(const float* __restrict__ X,
                                                    const uint8_t* __restrict__ W, void* out,
                                                    float* __restrict__ amax, int rows, int K,
                                                    int Nout, float s_a, float s_b, int layout) {
  constexpr bool TWO = MODE == CAL_GEGLU || MODE == CAL_SWIGLU;
  constexpr int LD = 64 + 1;
  __shared__ float xs[32][LD];
  __shared__ float wa[32][LD];
  __shared__ float wb[TWO ? 32 : 1][LD];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  float acc_a[4][4] = {}, acc_b[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 32) {
    // X tile: 64 rows x 32 columns, transposed into xs[k][m]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + 256 * j;  // 512 float4 pieces
      const int r = c >> 3, kc = (c & 7) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m0 + r < rows) v = *reinterpret_cast<const float4*>(X + (size_t)(m0 + r) * K + k0 + kc);
      xs[kc + 0][r] = v.x;
      xs[kc + 1][r] = v.y;
      xs[kc + 2][r] = v.z;
      xs[kc + 3][r] = v.w;
    }
    // weight tile: 64 output rows x 32 columns (two 16-column pieces each)
    if (tid < 128) {
      const int n = n0 + (tid >> 1), kk = (tid & 1) * 16;
      uint32_t prow_a, prow_b = 0;
      if (MODE == CAL_GEGLU || MODE == CAL_SWIGLU) {
        prow_a = layout ? gate_row_oct((uint32_t)n) : gate_row((uint32_t)n);
        prow_b = layout ? up_row_oct((uint32_t)n) : up_row_gated((uint32_t)n);
      } else {
        prow_a = (uint32_t)n;
      }
      load_w16(W, prow_a, (uint32_t)(k0 + kk), (uint32_t)K, &wa[kk][tid >> 1], LD, MODE == CAL_DOWN && layout != 0);
      if (TWO) load_w16(W, prow_b, (uint32_t)(k0 + kk), (uint32_t)K, &wb[kk][tid >> 1], LD, false);
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4], c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = wa[kk][tx * 4 + j];
        if (TWO) c[j] = wb[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc_a[i][j] = __builtin_fmaf(a[i], b[j], acc_a[i][j]);
          if (TWO) acc_b[i][j] = __builtin_fmaf(a[i], c[j], acc_b[i][j]);
        }
    }
    __syncthreads();
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + ty * 4 + i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (MODE == CAL_DOWN) {
        reinterpret_cast<uint16_t*>(out)[(size_t)r * Nout + n] =
            (uint16_t)f32_to_bf16(acc_a[i][j] * s_a);
      } else {
        float h;
        if (TWO)
          h = cal_h<MODE>(acc_a[i][j] * s_a, acc_b[i][j] * s_b);  // a: gate, b: up
        else
          h = cal_h<MODE>(0.0f, acc_a[i][j] * s_a);
        reinterpret_cast<float*>(out)[(size_t)r * Nout + n] = h;
        m = __builtin_fmaxf(m, __builtin_fabsf(h));
      }
    }
  }
  if (MODE != CAL_DOWN) {
    m = wave_max_f32(m);
    if ((tid & 63) == 0) atomic_max_nonneg(amax, m);
  }
}

hipError_t launch_calib_gateup(int act, const float* x, const uint8_t* w, float* h, float* amax,
                               int rows, int K, int I, float s_g, float s_u, hipStream_t s, int oct) {
  dim3 grid(I / 64, (rows + 63) / 64);
  if (act == CAL_GEGLU)
    hipLaunchKernelGGL(k_calib_gemm<CAL_GEGLU>, grid, dim3(256), 0, s, x, w, (void*)h, amax, rows,
                       K, I, s_g, s_u, oct);
  else if (act == CAL_SWIGLU)
    hipLaunchKernelGGL(k_calib_gemm<CAL_SWIGLU>, grid, dim3(256), 0, s, x, w, (void*)h, amax,
                       rows, K, I, s_g, s_u, oct);
  else
    hipLaunchKernelGGL(k_calib_gemm<CAL_GELU>, grid, dim3(256), 0, s, x, w, (void*)h, amax, rows,
                       K, I, s_u, 0.0f, 0);
  return hipGetLastError();
}

hipError_t launch_calib_down(const float* h, const uint8_t* w, uint16_t* y, int rows, int K, int H,
                             float s_d, hipStream_t s, int quad) {
  dim3 grid(H / 64, (rows + 63) / 64);
  hipLaunchKernelGGL(k_calib_gemm<CAL_DOWN>, grid, dim3(256), 0, s, h, w, (void*)y, nullptr, rows,
                     K, H, s_d, 0.0f, quad);
  return hipGetLastError();
}

}  // namespace frt
