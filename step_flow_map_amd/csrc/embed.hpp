// Noise-block embedding contraction of the flow-map jump:
//
//   e[m][c] = alpha * e[m][c] + beta * sum_v x[m][v] * E[v][c]
//   h[m][c] = e[m][c] + P[m % K][c]        (float32)
//
// x is the block state over the vocabulary ([M][V]: Gaussian noise at s = 0,
// the denoiser's softmax before a later jump), E the frozen embedding [V][d]
// stored one row per token.  The reduction runs over E's rows, which are
// contiguous along c, so a lane loads a VE x VE block (VE rows, VE adjacent
// columns, one 16-byte load per row; every load instruction covers four rows x
// 256 contiguous bytes) and transposes it in registers into VE MFMA B
// operands, one per column; E is read exactly once.
//
// Work split: a wave covers 16*VE columns; a workgroup's waves take
// interleaved 4*VE-row chunks (next chunk in flight) of one row range (a
// "split" of V), sum their accumulators through LDS in wave order and store
// the split's float32 partial with plain stores.  embed_reduce_kernel,
// launched next, sums a column block's splits in split order and writes e
// and h, so the result never depends on scheduling; it also writes h's
// per-16-column row statistics for the LayerNorm fused into the first QKV,
// and further workgroups of it apply the context fusion's LayerNorm to the
// rows the call appends.  Column blocks get Sf
// row splits, or Ss for the blocks with cb % 4 == 1: with 16 blocks of 256
// bytes those stream about 20% slower (their offset in each 4 KB row of E),
// so they get shorter row ranges and every workgroup finishes at about the
// same time.  Workgroups that read the same x rows are placed on the same XCD
// (the hardware deals workgroups round-robin over the 8 XCDs), so x is
// fetched about once per XCD.
#pragma once
#include "common.hpp"
#include "stream.hpp"

namespace fm {

constexpr int EMB_SPLITS_MAX = 19; // row splits of a column block

struct EmbedArgs {
  const void* x;      // [M][ldx]
  int ldx, M, V;
  const void* E;      // [V][d]
  int d;
  int Sf, Ss;         // row splits of a column block (Ss for cb % 4 == 1, Ss >= Sf)
  int rows_split;     // rows of V per split with Sf splits (multiple of 4*VE)
  int rows_split_s;   // the same with Ss splits
  float* partial;     // [Ss][M][d]
  float* e_state;     // [M][d] in/out
  float* h;           // [M][d] out
  float alpha, beta;  // alpha == 0: e_state is not read
  int K;              // positions per branch (rows m use position m % K)
  int use_pos;
  float2* ln_part;    // or null: per-16-column (mean, M2) of h for the LayerNorm
  int ln_part_ld;     // fused into the next contraction, at [m * ln_part_ld + c / 16]
  // context rows fused in this call, normalised by the reduce (the plain
  // LayerNorm of the fusion) instead of a launch of their own: n_u rows of
  // u_pre [n_u][d] (float32) with their per-16-column statistics u_part, written
  // in the storage type to u_out [n_u][d]; n_u = 0: none
  const float* u_pre;
  const float2* u_part;
  int u_part_ld;
  void* u_out;
  int n_u;
  float eps;
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

template <typename T, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void embed_kernel(EmbedArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = Vec<T>::N;
  constexpr int RCH = 4 * VE;   // rows per wave iteration
  constexpr int COLS = 16 * VE; // columns per wave
  constexpr int ELEMS = MT * VE * 4 * 64;
  __shared__ float red[ELEMS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int n_cb = g.d / COLS;
  // XCD-aware placement: blocks bid, bid+8, ... run on one XCD, which takes
  // consecutive entries e of the list (split 0 of every column block, split 1,
  // ..., then the slow blocks' further splits); the grid is a multiple of 8
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int e = xcd * (int)(gridDim.x >> 3) + slot;
  int cb, s;
  if (e < g.Sf * n_cb) {
    s = e / n_cb;
    cb = e % n_cb;
  } else {
    const int e2 = e - g.Sf * n_cb, n_slow = n_cb / 4;
    s = g.Sf + e2 / n_slow;
    cb = 4 * (e2 % n_slow) + 1;
  }
  const bool slow = g.Ss > g.Sf && (cb & 3) == 1;
  const int rows = slow ? g.rows_split_s : g.rows_split;
  const int c0 = cb * COLS;
  const int v_begin = s * rows;
  const int v_end = min(g.V, v_begin + rows);
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

  // this lane's VE rows of chunk v0 start at v0 + grp*VE; V and the split are
  // multiples of VE, so a lane's rows are all in range or all out.  Loads use
  // clamped addresses; the range check is applied to x at use (an out-of-range
  // chunk contributes x = 0), so no loaded value is selected before the MFMA.
  // x comes with the E rows of its chunk, one chunk ahead; from 64 rows on it
  // is loaded at use instead (x is an L2 hit: every column block reads it),
  // which keeps the accumulators and both E buffers in registers without spills.
  constexpr bool X_AHEAD = MT < 4;
  auto load = [&](VT (&in)[VE], VT (&a)[MT], int v0) {
    const int vr = v0 + grp * VE;
    const int vs = vr < v_end ? vr : 0;
#pragma unroll
    for (int r = 0; r < VE; ++r) in[r] = as_vec<T>(ldg_stream(ecol + (size_t)(vs + r) * g.d));
    if constexpr (X_AHEAD) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[mt] = vload<T>(xrow[mt] + vs);
    }
  };
  auto compute = [&](const VT (&in)[VE], const VT (&a)[MT], int v0) {
    const bool ok = v0 + grp * VE < v_end;
    VT bt[VE], am[MT];
    transpose_block(in, bt);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const VT xv = X_AHEAD ? a[mt] : vload<T>(xrow[mt] + (ok ? v0 + grp * VE : 0));
      am[mt] = vkeep(xv, ok && xok[mt]);
    }
#pragma unroll
    for (int t = 0; t < VE; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) mma(acc[mt][t], am[mt], bt[t]);
  };

  VT in0[VE], in1[VE], a0[MT], a1[MT];
  const int first = v_begin + wave * RCH, step = NW * RCH;
  if (first < v_end) load(in0, a0, first);
  for (int v0 = first; v0 < v_end; v0 += 2 * step) {
    if (v0 + step < v_end) load(in1, a1, v0 + step);
    compute(in0, a0, v0);
    if (v0 + step < v_end) {
      if (v0 + 2 * step < v_end) load(in0, a0, v0 + 2 * step);
      compute(in1, a1, v0 + step);
    }
  }

  // ---- fixed-order reduction over waves (wave 0 stores, others add in turn)
  for (int w = 0; w < NW; ++w) {
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
  // thread element el = row el / COLS, column el % COLS: consecutive lanes
  // take consecutive columns, so the partial stores coalesce into whole row
  // segments (lane-strided 4-byte stores each made a transaction of their own)
  constexpr int PER_THREAD = (ELEMS + NW * 64 - 1) / (NW * 64);
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    const int el = threadIdx.x + r * NW * 64;
    const int cl = el % COLS, m = el / COLS;
    // the MFMA output acc[mt][t][i] of lane (grp, j) is row mt*16 + 4*grp + i, column j*VE + t
    const int j = cl / VE, t = cl % VE, mt = m >> 4, grp = (m & 15) >> 2, i = m & 3;
    if (el < ELEMS && m < g.M)
      g.partial[((size_t)s * g.M + m) * g.d + c0 + cl] = red[((mt * VE + t) * 4 + i) * 64 + grp * 16 + j];
  }
}

// Workgroups past the M x d outputs of the reduce each normalise one fused
// context row (plain LayerNorm, biased variance): wave 0 merges the row's
// per-16-column statistics (two a lane in column order, then a fixed tree
// over the lanes), and every thread writes its columns.
template <typename T>
__device__ __forceinline__ void norm_context_row(const EmbedArgs& g, int r) {
  __shared__ float mr[2];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    const int np = g.d >> 4;
    float n = 0.f, mean = 0.f, M2 = 0.f;
    auto merge = [&](float nb, float mb, float m2b) {
      const float nn = n + nb, delta = mb - mean;
      const float f = nb > 0.f ? nb / nn : 0.f;
      mean += delta * f;
      M2 += nb > 0.f ? m2b + delta * delta * (n * f) : 0.f;
      n = nn;
    };
    const float2* pr = g.u_part + (size_t)r * g.u_part_ld;
    const float2 a = pr[min(lane, np - 1)], b = pr[min(lane + 64, np - 1)];
    merge(lane < np ? 16.f : 0.f, a.x, a.y);
    merge(lane + 64 < np ? 16.f : 0.f, b.x, b.y);
    float on = dpp_mov<0xB1>(n), om = dpp_mov<0xB1>(mean), o2 = dpp_mov<0xB1>(M2);
    merge(on, om, o2);
    on = dpp_mov<0x4E>(n), om = dpp_mov<0x4E>(mean), o2 = dpp_mov<0x4E>(M2);
    merge(on, om, o2);
    on = dpp_mov<0x141>(n), om = dpp_mov<0x141>(mean), o2 = dpp_mov<0x141>(M2);
    merge(on, om, o2);
    on = dpp_mov<0x140>(n), om = dpp_mov<0x140>(mean), o2 = dpp_mov<0x140>(M2);
    merge(on, om, o2);
    on = __shfl_xor(n, 16, 64), om = __shfl_xor(mean, 16, 64), o2 = __shfl_xor(M2, 16, 64);
    merge(on, om, o2);
    on = __shfl_xor(n, 32, 64), om = __shfl_xor(mean, 32, 64), o2 = __shfl_xor(M2, 32, 64);
    merge(on, om, o2);
    if (lane == 0) {
      mr[0] = mean;
      mr[1] = 1.f / sqrtf(M2 / (float)g.d + g.eps);  // biased variance
    }
  }
  __syncthreads();
  const float mean = mr[0], rstd = mr[1];
  const float* u = g.u_pre + (size_t)r * g.d;
  T* o = reinterpret_cast<T*>(g.u_out) + (size_t)r * g.d;
  for (int c = tid; c < g.d; c += 256) o[c] = from_f32<T>((u[c] - mean) * rstd);
}

// The sum over a column block's row splits, in split order, and the state
// update: e = alpha e + beta sum, h = e + P, one thread per output; launched
// after embed_kernel (the kernel boundary orders the partials' plain stores
// before these loads).  n_u further workgroups normalise the fused context rows.
template <typename T>
__global__ __launch_bounds__(256) void embed_reduce_kernel(EmbedArgs g) {
  constexpr int COLS = 16 * Vec<T>::N;
  const int n_main = (g.M * g.d + 255) / 256;
  if ((int)blockIdx.x >= n_main) {
    norm_context_row<T>(g, (int)blockIdx.x - n_main);
    return;
  }
  const int q0 = blockIdx.x * 256 + threadIdx.x;
  const bool ok = q0 < g.M * g.d;  // uniform over 16 lanes: M * d is a multiple of 16
  const int q = ok ? q0 : 0;
  const int m = q / g.d, c = q % g.d, cb = c / COLS;
  const int S_cb = (g.Ss > g.Sf && (cb & 3) == 1) ? g.Ss : g.Sf;
  // every split's load in flight at once, then the sum in split order
  float pv[EMB_SPLITS_MAX];
#pragma unroll
  for (int s = 0; s < EMB_SPLITS_MAX; ++s) pv[s] = s < S_cb ? g.partial[((size_t)s * g.M + m) * g.d + c] : 0.f;
  float v = 0.f;
#pragma unroll
  for (int s = 0; s < EMB_SPLITS_MAX; ++s) v += pv[s];
  float e = g.beta * v;
  if (g.alpha != 0.f) e += g.alpha * g.e_state[q];
  const float hv = e + (g.use_pos ? pos_table(m % g.K, c, g.d) : 0.f);
  if (ok) {
    g.e_state[q] = e;
    g.h[q] = hv;
  }
  // 16 consecutive lanes hold 16 consecutive columns of one row (d % 16 == 0)
  if (g.ln_part) row16_stats(hv, ok, g.ln_part + (size_t)m * g.ln_part_ld + (c >> 4));
}

}  // namespace fm
