// Noise-block embedding contraction of the flow-map jump:
//
//   e[m][c] = alpha * e[m][c] + beta * sum_v x[m][v] * E[v][c]
//   h[m][c] = e[m][c] + P[m % K][c]
//
// x is the block state over the vocabulary ([M][V]: Gaussian noise at s = 0,
// the denoiser's softmax before a later jump), E the frozen embedding [V][d]
// stored one row per token.  The reduction runs over E's rows, which are
// contiguous along c, so a lane loads a VE x VE block (VE rows, VE adjacent
// columns, one 16-byte load per row) and transposes it in registers into VE
// MFMA B operands, one per column; E is read exactly once with fully used
// 16-byte loads and no LDS round trip.
//
// Work split: a wave covers 16*VE columns; a workgroup's waves take
// interleaved 4*VE-row chunks of one row range (a deterministic split of V);
// partials are reduced in fixed order by the last workgroup of each column
// block.  Workgroups that read the same x rows (same split) are placed on the
// same XCD (the hardware deals workgroups round-robin over the 8 XCDs), so x
// is fetched once per XCD.
#pragma once
#include "common.hpp"

namespace fm {

struct EmbedArgs {
  const void* x;      // [M][ldx]
  int ldx, M, V;
  const void* E;      // [V][d]
  int d;
  int S;              // splits of V (multiple of 8)
  int rows_split;     // rows of V per split (multiple of 4*VE)
  float* partial;     // [S][M][d]
  uint32_t* counters; // one per column block
  float* e_state;     // [M][d] in/out
  float* h;           // [M][d] out
  float alpha, beta;  // alpha == 0: e_state is not read
  int K;              // positions per branch (rows m use position m % K)
  int use_pos;
};

// P[k][c] = sin(k w_c) for c < d/2, cos(k w_{c-d/2}) otherwise,
// w_i = 10000^(-i/(d/2))
__device__ __forceinline__ float pos_table(int k, int c, int d) {
  const int half = d >> 1;
  const int i = c < half ? c : c - half;
  const float w = expf(-9.210340371976184f * (float)i / (float)half);  // ln(1e4)
  const float a = (float)k * w;
  return c < half ? sinf(a) : cosf(a);
}

template <typename T, int MT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void embed_kernel(EmbedArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = Vec<T>::N;
  constexpr int RCH = 4 * VE;   // rows per wave iteration
  constexpr int COLS = 16 * VE; // columns per wave
  constexpr int ELEMS = MT * VE * 4 * 64;
  __shared__ float red[ELEMS];
  __shared__ int flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int n_cb = g.d / COLS;
  // XCD-aware placement: blocks bid, bid+8, ... run on one XCD
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int cb = slot % n_cb;
  const int s = (slot / n_cb) * 8 + xcd;
  const int c0 = cb * COLS;
  const int v_begin = s * g.rows_split;
  const int v_end = min(g.V, v_begin + g.rows_split);
  const T* X = reinterpret_cast<const T*>(g.x);
  const T* E = reinterpret_cast<const T*>(g.E);

  f32x4 acc[MT][VE];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < VE; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const T* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + j;
    xok[mt] = m < g.M;
    xrow[mt] = X + (size_t)(xok[mt] ? m : 0) * g.ldx;
  }
  const T* ecol = E + c0 + j * VE;

  for (int v0 = v_begin + wave * RCH; v0 < v_end; v0 += WAVES * RCH) {
    const int vr = v0 + grp * VE;  // first of this lane's VE rows
    const bool ok = vr < v_end;    // V and the split are multiples of VE
    VT in[VE], bt[VE], a[MT];
#pragma unroll
    for (int r = 0; r < VE; ++r) in[r] = ok ? vload<T>(ecol + (size_t)(vr + r) * g.d) : vzero<VT>();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = (ok && xok[mt]) ? vload<T>(xrow[mt] + vr) : vzero<VT>();
    transpose_block(in, bt);
#pragma unroll
    for (int t = 0; t < VE; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) mma(acc[mt][t], a[mt], bt[t]);
  }

  // ---- fixed-order reduction over waves (wave 0 stores, others add in turn)
  for (int w = 0; w < WAVES; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < VE; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float& dst = red[((mt * VE + t) * 4 + i) * 64 + lane];
            dst = (w == 0) ? acc[mt][t][i] : dst + acc[mt][t][i];
          }
    }
    __syncthreads();
  }
  constexpr int PER_THREAD = ELEMS / (WAVES * 64);
  int em[PER_THREAD], ec[PER_THREAD];
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    const int el = threadIdx.x + r * WAVES * 64;
    const int ln = el & 63, q = el >> 6;  // q = (mt*VE + t)*4 + i
    const int i = q & 3, t = (q >> 2) % VE, mt = (q >> 2) / VE;
    em[r] = mt * 16 + 4 * (ln >> 4) + i;
    ec[r] = c0 + (ln & 15) * VE + t;
    if (em[r] < g.M) g.partial[((size_t)s * g.M + em[r]) * g.d + ec[r]] = red[el];
  }
  if (!arrive_last(&g.counters[cb], (uint32_t)g.S, &flag)) return;
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    const int m = em[r], c = ec[r];
    if (m >= g.M) continue;
    float v = 0.f;
    for (int ss = 0; ss < g.S; ++ss) v += g.partial[((size_t)ss * g.M + m) * g.d + c];
    const size_t o = (size_t)m * g.d + c;
    float e = g.beta * v;
    if (g.alpha != 0.f) e += g.alpha * g.e_state[o];
    g.e_state[o] = e;
    g.h[o] = e + (g.use_pos ? pos_table(m % g.K, c, g.d) : 0.f);
  }
}

}  // namespace fm
