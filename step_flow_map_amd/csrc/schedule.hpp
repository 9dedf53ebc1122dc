// Schedule precompute: the adaLN vectors of each flow-map jump (s, t).
//
//   feat(tau) = [cos(tau w_i), sin(tau w_i)], w_i = exp(-ln(1e4) i / 128)
//   c         = TE_s(s) + TE_t(t),  TE(tau) = W2 silu(W1 feat(tau) + b1) + b2
//   block l   : W_ada^l silu(c) + b_ada^l  -> shift1, scale1, gate1, shift2, scale2, gate2
//   final     : W_fa silu(c) + b_fa        -> shift_f, scale_f
//
// Everything here is float32 (weights are widened exactly); it runs once per
// schedule, so a plain one-wave-per-output GEMV is enough.
#pragma once
#include "common.hpp"

namespace fm {

// f[0..255] = feat(tau): cos(tau w_i) then sin(tau w_i), i < 128
__global__ void time_features_kernel(float tau, float* f) {
  const int i = threadIdx.x;  // 128 threads
  const float w = expf(-9.210340371976184f * (float)i / 128.f);
  f[i] = cosf(tau * w);
  f[128 + i] = sinf(tau * w);
}

// out[r][n] (+)= act( sum_k in_act(in[r][k]) * W[n][k] + b[n] ), r < R <= 4.
// One wave per output column; in is float32 [R][ldi], W storage [N][K].
template <typename T>
__global__ __launch_bounds__(256) void gemv_kernel(const float* in, int ldi, int R, const T* W, const T* b, int N,
                                                   int K, float* out, int ldo, int in_silu, int out_silu,
                                                   int accumulate) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const T* w = W + (size_t)n * K;
  for (int k = lane; k < K; k += 64) {
    const float wv = to_f32<T>(w[k]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < R) {
        float x = in[(size_t)r * ldi + k];
        if (in_silu) x = silu(x);
        acc[r] += x * wv;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r >= R) break;
    float v = warp_sum(acc[r]);
    if (lane == 0) {
      if (b) v += to_f32<T>(b[n]);
      if (out_silu) v = silu(v);
      float* o = out + (size_t)r * ldo + n;
      *o = accumulate ? *o + v : v;
    }
  }
}

}  // namespace fm
