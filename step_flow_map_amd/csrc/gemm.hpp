// Skinny "activation x weight^T" contraction for the drafter's linear layers.
//
//   out[m][n] = sum_k A[m][k] * W[n][k]        (W row-major [N][K], k contiguous)
//
// M is small (block rows of every branch, plus the context rows appended in the
// step: at most 80), so each 16-byte weight vector loaded from HBM feeds M/16
// MFMAs and the layer is bound by streaming W.  A workgroup owns NT 16-column
// tiles and one K range of a deterministic split-K; its waves take interleaved
// k chunks (so the four waves of a workgroup read adjacent bytes of every
// weight row), reduce through LDS in a fixed order, and either run the
// epilogue (one split) or publish a float32 partial.  The last workgroup to
// arrive on a column tile sums the partials in split order and runs the
// epilogue, so results never depend on scheduling.
#pragma once
#include "common.hpp"

namespace fm {

enum EpiKind {
  EPI_F32 = 0,    // out_f32[m][n] = v + bias[n]
  EPI_ACT = 1,    // out_act[m][n] = T(v + bias[n])
  EPI_GELU = 2,   // out_act[m][n] = T(gelu(v + bias[n]))
  EPI_RESID = 3,  // out_f32[m][n] += gate[n] * (v + bias[n])   (residual stream)
  EPI_QKV = 4     // block rows: out_act[m][n] = T(v + b); context rows: K/V to cache
};

struct EpiParams {
  const void* bias;     // [N] storage type, or null
  float* out_f32;       // EPI_F32 / EPI_RESID
  int ld_f32;
  void* out_act;        // EPI_ACT / EPI_GELU / EPI_QKV
  int ld_act;
  const float* gate;    // EPI_RESID, [N]
  int rows_block;       // EPI_QKV: rows >= rows_block are context rows
  void* cache;          // EPI_QKV: this block's cache base, [C_max][2][d]
  int cache_pos0;       // EPI_QKV: context position of row rows_block
  int d;                // EPI_QKV: width
  int col_offset;       // EPI_QKV: logical qkv column of n = 0 (d for a K/V-only call)
};

struct GemmArgs {
  const void* A;
  int lda, M;
  const void* W;
  int ldw, N, K;
  int S;          // k splits
  int k_split;    // k elements per split (multiple of the chunk)
  float* partial; // [S][M][N] float32 when S > 1
  uint32_t* counters;  // one per column group, zero on entry, zero on exit
};

template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const EpiParams& e, int m, int n, float v) {
  if (e.bias) v += to_f32<T>(reinterpret_cast<const T*>(e.bias)[n]);
  if (EPI == EPI_F32) {
    e.out_f32[(size_t)m * e.ld_f32 + n] = v;
  } else if (EPI == EPI_ACT) {
    reinterpret_cast<T*>(e.out_act)[(size_t)m * e.ld_act + n] = from_f32<T>(v);
  } else if (EPI == EPI_GELU) {
    reinterpret_cast<T*>(e.out_act)[(size_t)m * e.ld_act + n] = from_f32<T>(gelu_tanh(v));
  } else if (EPI == EPI_RESID) {
    float* p = e.out_f32 + (size_t)m * e.ld_f32 + n;
    *p = *p + e.gate[n] * v;
  } else {  // EPI_QKV
    const int nn = n + e.col_offset;
    if (m < e.rows_block) {
      reinterpret_cast<T*>(e.out_act)[(size_t)m * e.ld_act + n] = from_f32<T>(v);
    } else if (nn >= e.d) {
      const int p = e.cache_pos0 + (m - e.rows_block);
      const int which = nn >= 2 * e.d;  // 0: key, 1: value
      reinterpret_cast<T*>(e.cache)[((size_t)p * 2 + which) * e.d + (nn - (1 + which) * e.d)] =
          from_f32<T>(v);
    }
  }
}

template <typename T, int MT, int NT, int U, int WAVES, int EPI>
__global__ __launch_bounds__(WAVES * 64) void gemm_nt_kernel(GemmArgs g, EpiParams e) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = Vec<T>::N;
  constexpr int CHUNK = 4 * U * VE;  // k elements per wave iteration
  constexpr int ELEMS = MT * NT * 4 * 64;
  __shared__ float red[WAVES > 1 ? WAVES * ELEMS : 1];
  __shared__ int flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int group = blockIdx.x / g.S, s = blockIdx.x % g.S;
  const int n0 = group * 16 * NT;
  const int k_begin = s * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);
  const T* A = reinterpret_cast<const T*>(g.A);
  const T* W = reinterpret_cast<const T*>(g.W);

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
    wok[nt] = n < g.N;
    wrow[nt] = W + (size_t)(wok[nt] ? n : 0) * g.ldw;
  }
  const T* arow[MT];
  bool aok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + j;
    aok[mt] = m < g.M;
    arow[mt] = A + (size_t)(aok[mt] ? m : 0) * g.lda;
  }

  for (int kc = k_begin + wave * CHUNK; kc < k_end; kc += WAVES * CHUNK) {
    const int kl = kc + grp * U * VE;
    VT b[NT][U], a[MT][U];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = kl + u * VE;
        b[nt][u] = (wok[nt] && k < k_end) ? vload<T>(wrow[nt] + k) : vzero<VT>();
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = kl + u * VE;
        a[mt][u] = (aok[mt] && k < k_end) ? vload<T>(arow[mt] + k) : vzero<VT>();
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) mma(acc[mt][nt], a[mt][u], b[nt][u]);
  }

  // ---- fixed-order reduction over the waves of the workgroup
  float val[MT * NT];  // this thread's elements e = threadIdx.x + r * WAVES * 64
  if (WAVES > 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[wave * ELEMS + ((mt * NT + nt) * 4 + i) * 64 + lane] = acc[mt][nt][i];
    __syncthreads();
  }
  constexpr int PER_THREAD = ELEMS / (WAVES * 64);
  static_assert(ELEMS % (WAVES * 64) == 0, "elements must split evenly over threads");
  int em[PER_THREAD], en[PER_THREAD];
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    const int el = threadIdx.x + r * WAVES * 64;
    const int ln = el & 63, q = el >> 6;  // q = (mt*NT + nt)*4 + i
    const int i = q & 3, tile = q >> 2;
    const int mt = tile / NT, nt = tile % NT;
    em[r] = mt * 16 + 4 * (ln >> 4) + i;
    en[r] = n0 + nt * 16 + (ln & 15);
    float v;
    if (WAVES > 1) {
      v = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += red[w * ELEMS + el];
    } else {
      v = acc[mt][nt][i];
    }
    val[r] = v;
  }

  if (g.S == 1) {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r)
      if (em[r] < g.M && en[r] < g.N) epilogue<T, EPI>(e, em[r], en[r], val[r]);
    return;
  }
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r)
    if (em[r] < g.M && en[r] < g.N)
      g.partial[((size_t)s * g.M + em[r]) * g.N + en[r]] = val[r];
  if (!arrive_last(&g.counters[group], (uint32_t)g.S, &flag)) return;
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    if (em[r] < g.M && en[r] < g.N) {
      float v = 0.f;
      for (int ss = 0; ss < g.S; ++ss) v += g.partial[((size_t)ss * g.M + em[r]) * g.N + en[r]];
      epilogue<T, EPI>(e, em[r], en[r], v);
    }
  }
}

}  // namespace fm
