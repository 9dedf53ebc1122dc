// Greedy verification of drafted blocks against the target's logits.
//
//   y[b][j]   = lowest-index argmax of target_logits[b][j][:], j = 0..K
//   accept[b] = largest n <= K with draft[b][i] == y[b][i] for all i < n
//   emitted   = draft[b][0..n-1], y[b][n], then -1
//   best      = lowest b with the largest accept[b]
//
// Two launches and no scratch memory: the first writes y into the emitted
// buffer (it has exactly B*(K+1) slots), the second turns it into the result.
#pragma once
#include "common.hpp"

namespace fm {

template <typename T>
__global__ __launch_bounds__(1024) void verify_argmax_kernel(const T* logits, int V, int32_t* y) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = Vec<T>::N;
  __shared__ uint64_t wk[16];
  const T* row = logits + (size_t)blockIdx.x * V;
  const int tid = threadIdx.x;
  // head elements up to 16-byte alignment, vector body, tail.  Each thread
  // visits its elements in increasing index order and keeps the first maximum
  // (strict >, and -0 == +0 compare equal); the order-preserving key is built
  // once per thread for the cross-thread reduction.
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = (int)(((16 - (addr & 15)) & 15) / sizeof(T));
  if (head > V) head = V;
  const int nvec = (V - head) / VE;
  const int tail0 = head + nvec * VE;
  float bv = -INFINITY;
  int bi = -1;
  auto visit = [&](float v, int idx) {
    if (bi < 0 || v > bv) {
      bv = v;
      bi = idx;
    }
  };
  if (tid < head) visit(to_f32<T>(row[tid]), tid);
  const VT* body = reinterpret_cast<const VT*>(row + head);
  constexpr int U = 8;  // eight 16-byte loads in flight per thread
  int i = tid;
  for (; i + (U - 1) * 1024 < nvec; i += U * 1024) {
    VT v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = body[i + u * 1024];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = head + (i + u * 1024) * VE;
#pragma unroll
      for (int e = 0; e < VE; ++e) visit(velem(v[u], e), base + e);
    }
  }
  for (; i < nvec; i += 1024) {
    const VT v = body[i];
    const int base = head + i * VE;
#pragma unroll
    for (int e = 0; e < VE; ++e) visit(velem(v, e), base + e);
  }
  if (tail0 + tid < V) visit(to_f32<T>(row[tail0 + tid]), tail0 + tid);
  uint64_t best = bi >= 0 ? argmax_key(bv, (uint32_t)bi) : 0ull;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = umax64(best, shfl_xor_u64(best, o));
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) wk[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t k = 0ull;
    for (int w = 0; w < 16; ++w) k = umax64(k, wk[w]);
    y[blockIdx.x] = (int32_t)argmax_key_index(k);
  }
}

// one thread per branch (B <= 64)
__global__ __launch_bounds__(64) void verify_prefix_kernel(const int32_t* draft, int B, int K, int32_t* emitted,
                                                           int32_t* accept, int32_t* best) {
  __shared__ int ns[64];
  const int b = threadIdx.x;
  int n = -1;
  if (b < B) {
    int32_t* row = emitted + (size_t)b * (K + 1);
    const int32_t* dr = draft + (size_t)b * K;
    n = 0;
    while (n < K && dr[n] == row[n]) ++n;
    const int32_t bonus = row[n];
    for (int i = 0; i <= K; ++i) row[i] = i < n ? dr[i] : (i == n ? bonus : -1);
    accept[b] = n;
  }
  ns[b] = n;
  __syncthreads();
  if (b == 0) {
    int bi = 0;
    for (int i = 1; i < B; ++i)
      if (ns[i] > ns[bi]) bi = i;
    best[0] = bi;
  }
}

}  // namespace fm
