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

// A workgroup's chunk is CH = 4096 columns: thread t holds the float4s
// t + 256 i (i < 4), all loads in flight at once.  V and CH are multiples of
// 4, so a float4 lies wholly inside or outside the row.
template <int CH>
__device__ __forceinline__ void load_chunk(const float* x, int v0, int v1, float4 (&q)[CH / 1024], bool (&ok)[CH / 1024]) {
#pragma unroll
  for (int i = 0; i < CH / 1024; ++i) {
    const int v = v0 + 4 * (threadIdx.x + 256 * i);
    ok[i] = v < v1;
    q[i] = *reinterpret_cast<const float4*>(x + (ok[i] ? v : v0));
  }
}

template <int CH>
__global__ __launch_bounds__(256) void softmax_stats_kernel(SoftmaxArgs a) {
  static_assert(CH % 1024 == 0, "four floats a thread per 1024 columns");
  __shared__ float sh[8];
  const int row = blockIdx.x / a.n_chunks, ch = blockIdx.x % a.n_chunks;
  const float* x = a.logits + (size_t)row * a.V;
  const int v0 = ch * CH, v1 = min(a.V, v0 + CH);
  float4 q[CH / 1024];
  bool ok[CH / 1024];
  load_chunk<CH>(x, v0, v1, q, ok);
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < CH / 1024; ++i)
    if (ok[i]) mx = fmaxf(mx, fmaxf(fmaxf(q[i].x, q[i].y), fmaxf(q[i].z, q[i].w)));
  float sm = 0.f;
  if (mx > -INFINITY) {
#pragma unroll
    for (int i = 0; i < CH / 1024; ++i)
      if (ok[i]) sm += (expf(q[i].x - mx) + expf(q[i].y - mx)) + (expf(q[i].z - mx) + expf(q[i].w - mx));
  } else {
    mx = 0.f;  // thread saw no element: contributes sum 0
  }
  block_max_sum<CH>(mx, sm, sh);
  if (threadIdx.x == 0) {
    a.part[((size_t)row * a.n_chunks + ch) * 2 + 0] = mx;
    a.part[((size_t)row * a.n_chunks + ch) * 2 + 1] = sm;
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* o, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* o, float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
  *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
}
template <>
__device__ __forceinline__ void store4<float>(float* o, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(o) = make_float4(a, b, c, d);
}

// the row's chunk partials are staged in LDS (one load per thread) and
// merged in chunk order by every thread; n_chunks <= 128
template <typename T, int CH>
__global__ __launch_bounds__(256) void softmax_write_kernel(SoftmaxArgs a) {
  __shared__ float sp[256];
  const int row = blockIdx.x / a.n_chunks, ch = blockIdx.x % a.n_chunks;
  const float* x = a.logits + (size_t)row * a.V;
  const int v0 = ch * CH, v1 = min(a.V, v0 + CH);
  float4 q[CH / 1024];
  bool ok[CH / 1024];
  load_chunk<CH>(x, v0, v1, q, ok);
  const float* p = a.part + (size_t)row * a.n_chunks * 2;
  if ((int)threadIdx.x < 2 * a.n_chunks) sp[threadIdx.x] = p[threadIdx.x];
  __syncthreads();
  float M = -INFINITY;
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, sp[2 * c]);
  float Z = 0.f;
  for (int c = 0; c < a.n_chunks; ++c) Z += sp[2 * c + 1] * expf(sp[2 * c] - M);
  const float inv = 1.f / Z;
  T* o = reinterpret_cast<T*>(a.out) + (size_t)row * a.V;
#pragma unroll
  for (int i = 0; i < CH / 1024; ++i) {
    if (!ok[i]) continue;
    const int v = v0 + 4 * (threadIdx.x + 256 * i);
    store4<T>(o + v, expf(q[i].x - M) * inv, expf(q[i].y - M) * inv, expf(q[i].z - M) * inv,
              expf(q[i].w - M) * inv);
  }
}

}  // namespace fm
