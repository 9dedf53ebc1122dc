// Frozen LM head with the draft decision fused in:
//
//   logits[m][v] = sum_c z[m][c] * W_lm[v][c]      (float32, no bias)
//   tokens[m]    = lowest v among the maxima of logits[m][:]
//
// Each wave owns NT 16-column (vocabulary) tiles at a time and walks the full
// width d; the workgroups stride over all tiles of the vocabulary.  The
// running best of each row is an order-preserving 64-bit key (value, then
// lower index), so the reduction across lanes, waves and workgroups is a plain
// max in any order.  The last workgroup to finish reduces the per-workgroup
// keys and writes the tokens.  Optionally the float32 logits are written out.
#pragma once
#include "common.hpp"

namespace fm {

struct LmArgs {
  const void* z;      // [M][d]
  int M, d;
  const void* W;      // [V][d]
  int V;
  float* logits;      // [M][V] or null
  uint64_t* partial;  // [gridDim.x][M]
  uint32_t* counter;
  int32_t* tokens;    // [M] or null
};

template <typename T, int MT, int NT, int U, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void lmhead_kernel(LmArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = Vec<T>::N;
  constexpr int CHUNK = 4 * U * VE;
  constexpr int MROWS = MT * 16;
  __shared__ uint64_t wbest[WAVES][MROWS];
  __shared__ int flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const T* Z = reinterpret_cast<const T*>(g.z);
  const T* W = reinterpret_cast<const T*>(g.W);
  const int n_groups = (g.V + 16 * NT - 1) / (16 * NT);

  const T* zrow[MT];
  bool zok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + j;
    zok[mt] = m < g.M;
    zrow[mt] = Z + (size_t)(zok[mt] ? m : 0) * g.d;
  }
  uint64_t best[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) best[mt][i] = 0ull;

  for (int tg = blockIdx.x * WAVES + wave; tg < n_groups; tg += gridDim.x * WAVES) {
    const int n0 = tg * 16 * NT;
    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const T* wrow[NT];
    bool wok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + nt * 16 + j;
      wok[nt] = n < g.V;
      wrow[nt] = W + (size_t)(wok[nt] ? n : 0) * g.d;
    }
    for (int kc = 0; kc < g.d; kc += CHUNK) {
      const int kl = kc + grp * U * VE;
      VT b[NT][U], a[MT][U];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k = kl + u * VE;
          b[nt][u] = (wok[nt] && k < g.d) ? vload<T>(wrow[nt] + k) : vzero<VT>();
        }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k = kl + u * VE;
          a[mt][u] = (zok[mt] && k < g.d) ? vload<T>(zrow[mt] + k) : vzero<VT>();
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma(acc[mt][nt], a[mt][u], b[nt][u]);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * grp + i;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = n0 + nt * 16 + j;
          if (n < g.V && m < g.M) {
            const float v = acc[mt][nt][i];
            best[mt][i] = umax64(best[mt][i], argmax_key(v, (uint32_t)n));
            if (g.logits) g.logits[(size_t)m * g.V + n] = v;
          }
        }
      }
  }

  // reduce over the 16 lanes that share a row group, then over waves
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint64_t k = best[mt][i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) k = umax64(k, shfl_xor_u64(k, o));
      if (j == 0) wbest[wave][mt * 16 + 4 * grp + i] = k;
    }
  __syncthreads();
  for (int m = threadIdx.x; m < g.M; m += WAVES * 64) {
    uint64_t k = 0ull;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) k = umax64(k, wbest[w][m]);
    g.partial[(size_t)blockIdx.x * g.M + m] = k;
  }
  if (!arrive_last(g.counter, gridDim.x, &flag)) return;

  // final reduction: TPR threads per row, consecutive lanes of one wave
  int mp = WAVES;  // at most 64 threads per row, so one wave holds a row
  while (mp < g.M) mp <<= 1;
  const int tpr = (WAVES * 64) / mp;  // host guarantees M <= WAVES * 64
  const int m = threadIdx.x / tpr, sub = threadIdx.x % tpr;
  uint64_t k = 0ull;
  if (m < g.M)
    for (int blk = sub; blk < (int)gridDim.x; blk += tpr) k = umax64(k, g.partial[(size_t)blk * g.M + m]);
  for (int o = 1; o < tpr; o <<= 1) k = umax64(k, shfl_xor_u64(k, o));
  if (m < g.M && sub == 0 && g.tokens) g.tokens[m] = (int32_t)argmax_key_index(k);
}

}  // namespace fm
