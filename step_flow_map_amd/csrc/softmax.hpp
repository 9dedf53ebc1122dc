// Row softmax over the vocabulary for a flow-map jump that ends before t = 1:
// D[m][v] = exp(l[m][v] - max_m) / sum_v exp(l[m][v] - max_m), stored in the
// storage type as the operand of the next embedding contraction.
// Two launches over (row, chunk) workgroups: per-chunk (max, sum) partials,
// then every chunk merges its row's partials in chunk order and writes D.
#pragma once
#include "common.hpp"

namespace fm {

struct SoftmaxArgs {
  const float* logits;  // [M][V]
  int V, n_chunks;
  float* part;          // [M][n_chunks][2]
  uint32_t* counters;   // unused
  void* out;            // [M][V] storage type
};

template <int CH>
__device__ __forceinline__ void block_max_sum(float& mx, float& sm, float* sh) {
  // inputs: per-thread (mx, sm) with sm relative to mx; output: block-wide
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m = warp_max(mx);
  float s = warp_sum(sm * expf(mx - m));
  if (lane == 0) {
    sh[2 * wave] = m;
    sh[2 * wave + 1] = s;
  }
  __syncthreads();
  float M = sh[0];
  for (int w = 1; w < 4; ++w) M = fmaxf(M, sh[2 * w]);
  float S = 0.f;
  for (int w = 0; w < 4; ++w) S += sh[2 * w + 1] * expf(sh[2 * w] - M);
  mx = M;
  sm = S;
}

template <int CH>
__global__ __launch_bounds__(256) void softmax_stats_kernel(SoftmaxArgs a) {
  __shared__ float sh[8];
  const int row = blockIdx.x / a.n_chunks, ch = blockIdx.x % a.n_chunks;
  const float* x = a.logits + (size_t)row * a.V;
  const int v0 = ch * CH, v1 = min(a.V, v0 + CH);
  float mx = -INFINITY;
  for (int v = v0 + threadIdx.x; v < v1; v += 256) mx = fmaxf(mx, x[v]);
  float sm = 0.f;
  if (mx > -INFINITY)
    for (int v = v0 + threadIdx.x; v < v1; v += 256) sm += expf(x[v] - mx);
  else
    mx = 0.f;  // thread saw no element: contributes sum 0
  block_max_sum<CH>(mx, sm, sh);
  if (threadIdx.x == 0) {
    a.part[((size_t)row * a.n_chunks + ch) * 2 + 0] = mx;
    a.part[((size_t)row * a.n_chunks + ch) * 2 + 1] = sm;
  }
}

template <typename T, int CH>
__global__ __launch_bounds__(256) void softmax_write_kernel(SoftmaxArgs a) {
  const int row = blockIdx.x / a.n_chunks, ch = blockIdx.x % a.n_chunks;
  const float* p = a.part + (size_t)row * a.n_chunks * 2;
  float M = -INFINITY;
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, p[2 * c]);
  float Z = 0.f;
  for (int c = 0; c < a.n_chunks; ++c) Z += p[2 * c + 1] * expf(p[2 * c] - M);
  const float inv = 1.f / Z;
  const float* x = a.logits + (size_t)row * a.V;
  T* o = reinterpret_cast<T*>(a.out) + (size_t)row * a.V;
  const int v0 = ch * CH, v1 = min(a.V, v0 + CH);
  for (int v = v0 + threadIdx.x; v < v1; v += 256) o[v] = from_f32<T>(expf(x[v] - M) * inv);
}

}  // namespace fm
