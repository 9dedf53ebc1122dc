// LayerNorm (no affine, biased variance, eps) with adaLN modulation, written
// in storage type as the operand of the next contraction:
//
//   out[r][c] = T( LN(x[r])[c] * (1 + scale[c]) + shift[c] )
//
// shift/scale may be null (plain LayerNorm, used for the context fusion).
// One workgroup per row; the row stays in registers for the two-pass mean and
// variance.
#pragma once
#include "common.hpp"

namespace fm {

template <typename T, int NT>
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = warp_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += sh[w];
  return t;
}

template <typename T, int PER>
__global__ __launch_bounds__(256) void ln_mod_kernel(const float* x, int ldx, int d, const float* shift,
                                                     const float* scale, T* out, int ldo, float eps) {
  __shared__ float red[4];
  const float* row = x + (size_t)blockIdx.x * ldx;
  float v[PER], sc[PER], sh[PER];
  float s = 0.f;
  // the modulation is loaded together with the row, not after the reductions
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int c = threadIdx.x + p * 256;
    const int cc = c < d ? c : 0;
    v[p] = c < d ? row[cc] : 0.f;
    sc[p] = scale ? scale[cc] : 0.f;
    sh[p] = scale ? shift[cc] : 0.f;
    s += v[p];
  }
  const float mean = block_sum<T, 256>(s, red) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int c = threadIdx.x + p * 256;
    const float dv = c < d ? v[p] - mean : 0.f;
    q += dv * dv;
  }
  const float var = block_sum<T, 256>(q, red) / (float)d;
  const float rstd = 1.f / sqrtf(var + eps);
  T* o = out + (size_t)blockIdx.x * ldo;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int c = threadIdx.x + p * 256;
    if (c < d) {
      float y = (v[p] - mean) * rstd;
      if (scale) y = y * (1.f + sc[p]) + sh[p];
      o[c] = from_f32<T>(y);
    }
  }
}

// dst[i] = src[i] (float32), for the optional hidden-state trace
__global__ void copy_f32_kernel(const float* src, float* dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// p[i] = 0 for i < n (32-bit words); used instead of memset so the clear can
// sit inside a captured graph
__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace fm
