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
#include "lmhead.hpp"
#include "philox.hpp"

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


// ------------------------------------------------- greedy, several workgroups per row
// The same verification with each target row split into S contiguous slices
// of `slice` elements (a multiple of the vector width; the caller guarantees
// 16-byte aligned rows and V a multiple of the vector width): workgroup
// (s, row) writes the slice's best 64-bit key to keys[row][s]; then one
// workgroup merges each row's keys (max of the keys: independent of order)
// and runs the prefix, emitted tokens, accept and best branch.  Each thread
// keeps its first maximum as the one-workgroup argmax does, so both agree on
// every input without NaN.
constexpr int VSL_THREADS = 256;
constexpr int VSL_SLICES = 16;
template <typename T>
__global__ __launch_bounds__(VSL_THREADS) void verify_slice_kernel(const T* logits, int V, int slice,
                                                                   uint64_t* keys) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = Vec<T>::N;
  constexpr int U = 4;  // 16-byte loads in flight per thread
  __shared__ uint64_t wk[VSL_THREADS / 64];
  const int s = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const T* row = logits + (size_t)r * V;
  const int v0 = s * slice, v1 = min(V, v0 + slice);
  const int nvec = v1 > v0 ? (v1 - v0) / VE : 0;
  const VT* body = reinterpret_cast<const VT*>(row + v0);
  float bv = -INFINITY;
  int bi = -1;
  auto visit = [&](float v, int idx) {
    if (bi < 0 || v > bv) {
      bv = v;
      bi = idx;
    }
  };
  int i = tid;
  for (; i + (U - 1) * VSL_THREADS < nvec; i += U * VSL_THREADS) {
    VT v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = body[i + u * VSL_THREADS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = v0 + (i + u * VSL_THREADS) * VE;
#pragma unroll
      for (int e = 0; e < VE; ++e) visit(velem(v[u], e), base + e);
    }
  }
  for (; i < nvec; i += VSL_THREADS) {
    const VT v = body[i];
    const int base = v0 + i * VE;
#pragma unroll
    for (int e = 0; e < VE; ++e) visit(velem(v, e), base + e);
  }
  uint64_t best = bi >= 0 ? argmax_key(bv, (uint32_t)bi) : 0ull;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = umax64(best, shfl_xor_u64(best, o));
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) wk[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t k = 0ull;
    for (int w = 0; w < VSL_THREADS / 64; ++w) k = umax64(k, wk[w]);
    keys[(size_t)r * VSL_SLICES + s] = k;
  }
}

// One workgroup: lane group of 16 per target row merges that row's slice keys
// (rows r, r + 64, ...), then one thread per branch runs the prefix.
__global__ __launch_bounds__(1024) void verify_merge_kernel(const uint64_t* keys, int S, const int32_t* draft, int B,
                                                            int K, int32_t* emitted, int32_t* accept, int32_t* best) {
  __shared__ int32_t y[64 * 65];
  __shared__ int ns[64];
  const int t = threadIdx.x, rows = B * (K + 1);
  for (int r = t / 16; r < rows; r += 1024 / 16) {
    uint64_t k = (t % 16) < S ? keys[(size_t)r * VSL_SLICES + (t % 16)] : 0ull;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) k = umax64(k, shfl_xor_u64(k, o));
    if (t % 16 == 0) y[r] = (int32_t)argmax_key_index(k);
  }
  __syncthreads();
  if (t < 64) {
    int n = -1;
    if (t < B) {
      const int32_t* yr = y + t * (K + 1);
      const int32_t* dr = draft + (size_t)t * K;
      n = 0;
      while (n < K && dr[n] == yr[n]) ++n;
      int32_t* row = emitted + (size_t)t * (K + 1);
      for (int i = 0; i <= K; ++i) row[i] = i < n ? dr[i] : (i == n ? yr[n] : -1);
      accept[t] = n;
    }
    ns[t] = n;
  }
  __syncthreads();
  if (t == 0) {
    int bi = 0;
    for (int i = 1; i < B; ++i)
      if (ns[i] > ns[bi]) bi = i;
    best[0] = bi;
  }
}


// ------------------------------------------------------------ temperature > 0
// Probabilistic verification (speculative sampling) of B branches:
//   p_j = softmax(T_j / tau) for target rows j = 0..K, q_i = softmax(Q_i / tau)
//   the drafter's distribution of row i (its log-normaliser lseQ_i comes with
//   the draft).  Draft i is accepted while u_i * q_i(d_i) < p_i(d_i), u_i the
//   uniform of Philox counter (0, i, b, stream 2); n = accepted prefix.  Row n
//   emits the Gumbel-max sample (counters (v, n, b, stream 1)) of the residual
//   max(0, p_n - q_n) when n < K, of p_K when n = K; a residual that is zero
//   everywhere (p = q in float32) falls back to p_n.
// Four launches: the target rows' (max, sum of exp) per vocabulary slice
// ([B*(K+1)] x S workgroups); per branch the rows' log-normalisers and the
// accepted prefix n; row n's residual and fallback keys per slice (B x S);
// per branch the merge of row n's keys into the emitted tokens.  Merge orders
// are fixed, so results are reproducible.
struct VsArgs {
  const void* T;          // [B][K+1][V] target logits
  const float* Q;         // [B][K][V] drafter logits of the last jump
  const float* lseQ;      // [B][K] log sum_v exp(Q / tau)
  const int32_t* draft;   // [B][K]
  int B, K, V, S, slice;  // S vocabulary slices of `slice` tokens
  float tau;
  BlockRng rng;           // key and branch word of each branch
  float2* stats;          // [B*(K+1)][S]
  float* lse_rows;        // [B*(K+1)] log sum_v exp(T / tau) of every target row
  int32_t* n_acc;         // [B] accepted prefix
  uint64_t* keys;         // [B][S][2]: row n's residual (or bonus) key, fallback key
  int32_t* emitted;       // [B][K+1]
  int32_t* accept;        // [B]
};

constexpr int VS_THREADS = 256;
constexpr int VS_UNROLL = 4;  // loads in flight per thread

template <typename T>
__global__ __launch_bounds__(VS_THREADS) void vs_stats_kernel(VsArgs g) {
  __shared__ float2 sw[VS_THREADS / 64];
  const int s = blockIdx.x, r = blockIdx.y;
  const T* row = reinterpret_cast<const T*>(g.T) + (size_t)r * g.V;
  const int v0 = s * g.slice, v1 = min(g.V, v0 + g.slice);
  float m = -INFINITY, sum = 0.f;
  for (int base = v0 + (int)threadIdx.x; base < v1; base += VS_UNROLL * VS_THREADS) {
    float x[VS_UNROLL];
#pragma unroll
    for (int u = 0; u < VS_UNROLL; ++u) {
      const int v = base + u * VS_THREADS;
      x[u] = to_f32<T>(row[v < v1 ? v : v0]);
    }
#pragma unroll
    for (int u = 0; u < VS_UNROLL; ++u)
      if (base + u * VS_THREADS < v1) lse_add(m, sum, x[u] / g.tau);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lse_shfl_merge(m, sum, o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sw[wave] = make_float2(m, sum);
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < VS_THREADS / 64; ++w) lse_merge(m, sum, sw[w].x, sw[w].y);
    g.stats[(size_t)r * g.S + s] = make_float2(m, sum);
  }
}

// One workgroup of 16 waves per branch: wave w merges the slice states of
// rows w, w + 16, ... (S <= 256 slices, four per lane, all loads in flight).
// A row's log-normaliser is M + log(sum_t s_t exp(m_t - M)) with M the
// largest slice maximum: a max reduction, one exponential per slice and a
// sum, each over a fixed tree.  Lane i of wave 0 then tests draft i.
constexpr int VS_ACCEPT_THREADS = 1024;
template <typename T, int R>
__global__ __launch_bounds__(VS_ACCEPT_THREADS) void vs_accept_kernel(VsArgs g) {
  static_assert(R <= 65, "K <= 64");
  constexpr int NWV = VS_ACCEPT_THREADS / 64;
  __shared__ float slse[R];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // the drafted token's target and drafter logits, loaded up front
  const bool tester = wave == 0 && lane < g.K;
  float t_d = 0.f, q_d = 0.f, lseq = 0.f;
  if (tester) {
    const int d = min(max(g.draft[b * g.K + lane], 0), g.V - 1);  // memory safety only
    const T* Tb = reinterpret_cast<const T*>(g.T) + (size_t)b * R * g.V;
    t_d = to_f32<T>(Tb[(size_t)lane * g.V + d]);
    q_d = g.Q[((size_t)b * g.K + lane) * g.V + d];
    lseq = g.lseQ[b * g.K + lane];
  }
  for (int j = wave; j < R; j += NWV) {
    float2 e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = lane + 64 * u;
      e[u] = i < g.S ? g.stats[((size_t)b * R + j) * g.S + i] : make_float2(-INFINITY, 0.f);
    }
    float M = fmaxf(fmaxf(e[0].x, e[1].x), fmaxf(e[2].x, e[3].x));
    M = warp_max(M);
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) v += lane + 64 * u < g.S ? e[u].y * expf(e[u].x - M) : 0.f;
    const float sum = warp_sum(v);
    if (lane == 0) {
      slse[j] = M + logf(sum);
      g.lse_rows[b * R + j] = slse[j];
    }
  }
  __syncthreads();
  if (wave == 0) {
    bool reject = false;
    if (tester) {
      const float lp = t_d / g.tau - slse[lane];
      const float lq = q_d / g.tau - lseq;
      uint32_t k0, k1, bw;
      block_rng(g.rng, b, k0, k1, bw);
      const float u = uniform_of(philox_x0(0u, (uint32_t)lane, bw, RNG_ACCEPT, k0, k1));
      reject = !(u * expf(lq) < expf(lp));
    }
    const uint64_t rej = __ballot(reject);
    if (lane == 0) g.n_acc[b] = rej ? (int)__builtin_ctzll(rej) : g.K;
  }
}

// Block-wide max of two keys; thread 0 ends with the results.
__device__ __forceinline__ void block_max2(uint64_t& a, uint64_t& b) {
  __shared__ uint64_t sk[2][VS_THREADS / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a = umax64(a, shfl_xor_u64(a, o));
    b = umax64(b, shfl_xor_u64(b, o));
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sk[0][wave] = a;
    sk[1][wave] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < VS_THREADS / 64; ++w) {
      a = umax64(a, sk[0][w]);
      b = umax64(b, sk[1][w]);
    }
}

// Row n of branch b, slice s: the residual (bonus) key and the fallback key.
template <typename T>
__global__ __launch_bounds__(VS_THREADS) void vs_keys_kernel(VsArgs g) {
  const int s = blockIdx.x, b = blockIdx.y;
  uint32_t rk0, rk1, bw;  // this branch's Philox key and branch word
  block_rng(g.rng, b, rk0, rk1, bw);
  const int n = g.n_acc[b];
  const int r = b * (g.K + 1) + n;
  const float lseP = g.lse_rows[r];
  const T* row = reinterpret_cast<const T*>(g.T) + (size_t)r * g.V;
  const bool bonus = n == g.K;
  const float* qrow = g.Q + ((size_t)b * g.K + (bonus ? 0 : n)) * g.V;
  const float lseQ = bonus ? 0.f : g.lseQ[b * g.K + n];
  const int v0 = s * g.slice, v1 = min(g.V, v0 + g.slice);
  uint64_t k1 = 0ull, k2 = 0ull;
  for (int base = v0 + (int)threadIdx.x; base < v1; base += VS_UNROLL * VS_THREADS) {
    float x[VS_UNROLL], q[VS_UNROLL];
#pragma unroll
    for (int u = 0; u < VS_UNROLL; ++u) {
      const int v = base + u * VS_THREADS < v1 ? base + u * VS_THREADS : v0;
      x[u] = to_f32<T>(row[v]);
      q[u] = qrow[v];
    }
#pragma unroll
    for (int u = 0; u < VS_UNROLL; ++u) {
      const int v = base + u * VS_THREADS;
      if (v >= v1) continue;
      const float lp = x[u] / g.tau - lseP;
      const float G = gumbel_of(philox_x0((uint32_t)v, (uint32_t)n, bw, RNG_CORRECT, rk0, rk1));
      k2 = umax64(k2, argmax_key(lp + G, (uint32_t)v));
      if (bonus) {
        k1 = umax64(k1, argmax_key(lp + G, (uint32_t)v));
      } else {
        const float w = expf(lp) - expf(q[u] / g.tau - lseQ);
        if (w > 0.f) k1 = umax64(k1, argmax_key(logf(w) + G, (uint32_t)v));
      }
    }
  }
  block_max2(k1, k2);
  if (threadIdx.x == 0) {
    g.keys[((size_t)b * g.S + s) * 2 + 0] = k1;
    g.keys[((size_t)b * g.S + s) * 2 + 1] = k2;
  }
}

// one wave per branch: merge row n's slice keys (S <= VS_THREADS), write the
// emitted tokens
__global__ __launch_bounds__(64) void vs_final_kernel(VsArgs g) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = g.n_acc[b];
  uint64_t k1 = 0ull, k2 = 0ull;
  for (int t = lane; t < g.S; t += 64) {
    k1 = umax64(k1, g.keys[((size_t)b * g.S + t) * 2 + 0]);
    k2 = umax64(k2, g.keys[((size_t)b * g.S + t) * 2 + 1]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    k1 = umax64(k1, shfl_xor_u64(k1, o));
    k2 = umax64(k2, shfl_xor_u64(k2, o));
  }
  const int y = (int)argmax_key_index(k1 ? k1 : k2);
  for (int i = lane; i <= g.K; i += 64)
    g.emitted[(size_t)b * (g.K + 1) + i] = i < n ? g.draft[b * g.K + i] : (i == n ? y : -1);
  if (lane == 0) g.accept[b] = n;
}

}  // namespace fm
