// Frozen LM head with the draft decision fused in:
//
//   logits[m][v] = sum_c z[m][c] * W_lm[v][c]      (float32, no bias)
//   tokens[m]    = lowest v among the maxima of logits[m][:]
//
// W_lm is streamed once from HBM in 16-row vocabulary tiles, each row read in
// 512-byte chunks through a per-wave LDS tile into MFMA operands with the next
// chunk in flight.  lmhead_ks_kernel (the usual plan) splits every tile's k
// range over the waves of a workgroup so that z stays in registers;
// lmhead_kernel (when z would not fit there) gives each wave whole tiles and
// reads z at use.  The running best of each row is an order-preserving 64-bit
// key (value, then lower index), so lanes, waves and workgroups combine with a
// plain max in any order; each workgroup writes its keys and
// argmax_finalize_kernel reduces them.
//
// Temperature tau > 0 (draft sampling): the key of logit l at (row m, token
// v) is l / tau + G, G the Gumbel noise of Philox counter (v, m % K, branch
// word of block m / K, stream 0) under that block's key, so the row's winner
// is a sample of softmax(l / tau); each
// workgroup also writes the row's (max, sum of exp(l / tau - max)) and the
// finalize kernel merges them into log sum_v exp(l_v / tau).
#pragma once
#include "common.hpp"
#include "philox.hpp"
#include "stream.hpp"

namespace fm {

struct LmArgs {
  const void* z;      // [M][d]
  int M, d;
  const void* W;      // [V][d]
  int V;
  float* logits;      // [M][V] or null
  uint64_t* partial;  // [M][gridDim.x]
  float tau;          // 0: greedy argmax; > 0: sampling at this temperature
  BlockRng rng;       // key and branch word of each row block (tau > 0)
  int K;              // rows per branch
  float2* lse_part;   // [M][gridDim.x] (tau > 0)
};

// Online log-sum-exp state (m, s): sum of exp(x - m) over the values seen.
__device__ __forceinline__ void lse_add(float& m, float& s, float x) {
  if (x > m) {
    s = s * expf(m - x) + 1.f;  // m = -inf at the start: s = 0 * 0 + 1
    m = x;
  } else {
    s += expf(x - m);
  }
}
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  const float mm = fmaxf(m, m2);
  s = s * expf(m - mm) + s2 * expf(m2 - mm);
  m = mm;
}
__device__ __forceinline__ void lse_shfl_merge(float& m, float& s, int o) {
  const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
  lse_merge(m, s, m2, s2);
}

// One finished logit v at (row m, token n): running key, log-sum-exp state,
// optional dump.
__device__ __forceinline__ void lm_visit(const LmArgs& g, float v, int m, int n, uint64_t& best, float& lm,
                                         float& ls, bool write = true) {
  float key = v;
  if (g.tau > 0.f) {
    const float x = v / g.tau;
    lse_add(lm, ls, x);
    uint32_t k0, k1, bw;
    block_rng(g.rng, m / g.K, k0, k1, bw);
    key = x + gumbel_of(philox_x0((uint32_t)n, (uint32_t)(m % g.K), bw, RNG_DRAFT, k0, k1));
  }
  best = umax64(best, argmax_key(key, (uint32_t)n));
  if (write && g.logits) g.logits[(size_t)m * g.V + n] = v;
}

template <typename T, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void lmhead_kernel(LmArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = ChunkT<T>::VE;
  constexpr int KC = ChunkT<T>::KC;
  __shared__ uint4 wtiles[NW * 512];
  __shared__ uint64_t wbest[NW][MT * 16];
  __shared__ float2 wlse[NW][MT * 16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const T* Z = reinterpret_cast<const T*>(g.z);
  const T* W = reinterpret_cast<const T*>(g.W);

  const T* zrow[MT];
  bool zok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + j;
    zok[mt] = m < g.M;
    zrow[mt] = Z + (size_t)(zok[mt] ? m : 0) * g.d;
  }
  uint64_t best[MT][4];
  float lm[MT][4], ls[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      best[mt][i] = 0ull;
      lm[mt][i] = -INFINITY;
      ls[mt][i] = 0.f;
    }

  const int ntiles = (g.V + 15) / 16, nch = (g.d + KC - 1) / KC;
  const int gw = blockIdx.x * NW + wave, nw = gridDim.x * NW;
  const int total = gw < ntiles ? ((ntiles - 1 - gw) / nw + 1) * nch : 0;
  uint4* wt = wtiles + wave * 512;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](uint4 (&r)[8], int q) {
    const int t = gw + (q / nch) * nw, c = q % nch;
    chunk_load<T>(r, W, g.d, t * 16, g.V, c * KC, g.d);
  };
  auto process = [&](const uint4 (&r)[8], int q) {
    const int t = gw + (q / nch) * nw, c = q % nch;
    const int k0 = c * KC;
    chunk_to_lds(r, wt);
    wave_lds_sync();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const VT b = as_vec<T>(chunk_frag(wt, st));
      const int k = k0 + (4 * st + grp) * VE;
      const bool kok = k < g.d;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bool ok = kok && zok[mt];
        VT av = vload<T>(zrow[mt] + (ok ? k : 0));
        av = ok ? av : vzero<VT>();
        mma(acc[mt], av, b);
      }
    }
    wave_lds_sync();
    if (c == nch - 1) {
      const int n = t * 16 + j;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + 4 * grp + i;
          if (n < g.V && m < g.M) lm_visit(g, acc[mt][i], m, n, best[mt][i], lm[mt][i], ls[mt][i]);
        }
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  uint4 r0[8], r1[8];
  if (total > 0) load(r0, 0);
  for (int q = 0; q < total; q += 2) {
    if (q + 1 < total) load(r1, q + 1);
    process(r0, q);
    if (q + 1 < total) {
      if (q + 2 < total) load(r0, q + 2);
      process(r1, q + 1);
    }
  }

  // reduce over the 16 lanes that share a row group, then over the waves
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint64_t k = best[mt][i];
      float a = lm[mt][i], b = ls[mt][i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        k = umax64(k, shfl_xor_u64(k, o));
        lse_shfl_merge(a, b, o);
      }
      if (j == 0) {
        wbest[wave][mt * 16 + 4 * grp + i] = k;
        wlse[wave][mt * 16 + 4 * grp + i] = make_float2(a, b);
      }
    }
  __syncthreads();
  for (int m = threadIdx.x; m < g.M; m += NW * 64) {
    uint64_t k = 0ull;
    float a = -INFINITY, b = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      k = umax64(k, wbest[w][m]);
      lse_merge(a, b, wlse[w][m].x, wlse[w][m].y);
    }
    g.partial[(size_t)m * gridDim.x + blockIdx.x] = k;
    if (g.tau > 0.f) g.lse_part[(size_t)m * gridDim.x + blockIdx.x] = make_float2(a, b);
  }
}

// Variant with the k range split over the waves: wave w owns chunks w, w+NW,
// ... of every vocabulary tile, so its z fragments for those chunks stay in
// registers for the whole kernel (any number of rows up to 64, no z traffic in
// the loop).  A workgroup takes tiles blockIdx, blockIdx+G, ... (a tile is 16
// vocabulary rows, one contiguous stretch of W_lm); its waves stream their
// chunks of the tile (each next chunk in flight), multiply, and put
// their partial tile into LDS (two buffers by tile parity, so one LDS barrier
// per tile suffices); every thread then sums the waves in order for its fixed
// output elements, updates its running key and writes the logit if asked.
// The keys of a row are combined over 16 lanes and written per workgroup for
// argmax_finalize_kernel.  With 16 rows, logits that are asked for wait in LDS
// (one 1 KB tile per vocabulary tile, up to LM_STAGE_TILES) and are written
// after the last tile: written tile by tile, their 64-byte row pieces slowed
// the weight stream by about 10%.
constexpr int LM_STAGE_TILES = 20;
template <typename T, int MT, int NW, int CPW>
__global__ __launch_bounds__(NW * 64) void lmhead_ks_kernel(LmArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = ChunkT<T>::VE;
  constexpr int KC = ChunkT<T>::KC;
  constexpr int ELEMS = MT * 256;                        // outputs of one tile
  constexpr int PER = (ELEMS + NW * 64 - 1) / (NW * 64);  // outputs per thread
  __shared__ uint4 wtiles[NW * 512];
  __shared__ float red[2][NW * ELEMS];
  constexpr int NT_STAGE = MT == 1 ? LM_STAGE_TILES : 0;
  __shared__ __align__(16) float slog[NT_STAGE ? NT_STAGE * ELEMS : 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const T* Z = reinterpret_cast<const T*>(g.z);
  const T* W = reinterpret_cast<const T*>(g.W);
  uint4* wt = wtiles + wave * 512;
  const int nch = (g.d + KC - 1) / KC;
  const int ntiles = (g.V + 15) / 16;
  const int G = gridDim.x;
  const int nt = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / G + 1 : 0;
  const bool stage = NT_STAGE > 0 && g.logits != nullptr && nt <= NT_STAGE;

  // z fragments of this wave's chunks: rows >= M and columns >= d are zeroed
  VT zf[CPW][MT][8];
#pragma unroll
  for (int u = 0; u < CPW; ++u)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int c = wave + u * NW;
        const int m = mt * 16 + j, k = c * KC + (4 * st + grp) * VE;
        const bool ok = m < g.M && c < nch && k < g.d;
        zf[u][mt][st] = vkeep(vload<T>(Z + (size_t)(ok ? m : 0) * g.d + (ok ? k : 0)), ok);
      }
  uint64_t best[PER];
  float lm[PER], ls[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    best[r] = 0ull;
    lm[r] = -INFINITY;
    ls[r] = 0.f;
  }

  // this wave's chunk u of tile it (of this workgroup); tiles past the end read row 0
  auto load_chunk = [&](uint4 (&rb)[8], int it, int u) {
    const int t = (int)blockIdx.x + it * G;
    const int c = min(wave + u * NW, nch - 1);
    chunk_load<T>(rb, W, g.d, t * 16, g.V, c * KC, g.d);
  };
  // the waves' partial tile through LDS, then each thread's fixed outputs
  auto finish = [&](f32x4 (&acc)[MT], int it) {
    float* rd = red[it & 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rd[wave * ELEMS + (mt * 4 + i) * 64 + lane] = acc[mt][i];
    lds_barrier();
    const int n0 = ((int)blockIdx.x + it * G) * 16;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int el = tid + r * NW * 64;
      if (el < ELEMS) {
        const int ln = el & 63, q = el >> 6;  // q = mt*4 + i
        const int m = (q >> 2) * 16 + 4 * (ln >> 4) + (q & 3), n = n0 + (ln & 15);
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += rd[w * ELEMS + el];
        if (stage) slog[it * ELEMS + el] = v;
        if (n < g.V && m < g.M) lm_visit(g, v, m, n, best[r], lm[r], ls[r], !stage);
      }
    }
  };
  // One register buffer: each chunk of the tile goes to the wave's LDS tile,
  // the next tile's same chunk is issued into the freed registers, and the
  // MFMAs read LDS meanwhile.  Two buffers made 64 rows spill (107.6 against
  // 103.7 us) and were no faster at 16 rows.
  auto process = [&](uint4 (&rb)[CPW][8], int it) {
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      chunk_to_lds(rb[u], wt);
      load_chunk(rb[u], it + 1, u);
      wave_lds_sync();
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const VT b = as_vec<T>(chunk_frag(wt, st));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mma(acc[mt], zf[u][mt][st], b);
      }
      wave_lds_sync();
    }
    finish(acc, it);
  };

  uint4 r0[CPW][8];
#pragma unroll
  for (int u = 0; u < CPW; ++u) load_chunk(r0[u], 0, u);
  for (int it = 0; it < nt; ++it) process(r0, it);

  if (stage) {
    // tile it's logit (row m, column c) sits at slog[it*ELEMS + (m&3)*64 + (m>>2)*16 + c]
    __syncthreads();
    const bool v4 = (g.V & 3) == 0;
    for (int idx = tid; idx < nt * 64; idx += NW * 64) {
      const int it = idx >> 6, m = (idx >> 2) & 15, c = (idx & 3) * 4;
      const int n = ((int)blockIdx.x + it * G) * 16 + c;
      if (m >= g.M) continue;
      const float4 v = *reinterpret_cast<const float4*>(&slog[it * ELEMS + (m & 3) * 64 + (m >> 2) * 16 + c]);
      float* dst = g.logits + (size_t)m * g.V + n;
      if (v4 && n + 3 < g.V) {
        *reinterpret_cast<float4*>(dst) = v;
      } else {
        if (n < g.V) dst[0] = v.x;
        if (n + 1 < g.V) dst[1] = v.y;
        if (n + 2 < g.V) dst[2] = v.z;
        if (n + 3 < g.V) dst[3] = v.w;
      }
    }
  }
  // a row's keys: 16 lanes (the tile's columns) of one wave
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int el = tid + r * NW * 64;
    uint64_t k = best[r];
    float a = lm[r], b = ls[r];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      k = umax64(k, shfl_xor_u64(k, o));
      lse_shfl_merge(a, b, o);
    }
    const int ln = el & 63, q = el >> 6;
    const int m = (q >> 2) * 16 + 4 * (ln >> 4) + (q & 3);
    if (el < ELEMS && (ln & 15) == 0 && m < g.M) {
      g.partial[(size_t)m * gridDim.x + blockIdx.x] = k;
      if (g.tau > 0.f) g.lse_part[(size_t)m * gridDim.x + blockIdx.x] = make_float2(a, b);
    }
  }
}

// Context lengths on the device (in the handle's workspace): len[r] for each
// request, then at len[FM_MAX_REQ] a sticky flag set when an append would pass
// the capacity (the length then stops at the capacity and the rows past it are
// not written).  A call that appends rows advances the lengths in its last
// kernel, after every kernel that reads them, so a captured graph advances the
// context on every replay.
struct CtxUpdate {
  int* len;              // null: no update
  int first, count;      // requests first .. first + count - 1
  int val[FM_MAX_REQ];   // rows appended (set == 0), or the new length (set == 1)
  int set;
  int cap;
};
__device__ __forceinline__ void ctx_update(const CtxUpdate& u) {
  if (!u.len) return;
  for (int i = 0; i < u.count; ++i) {
    const int r = u.first + i;
    int v = u.set ? u.val[i] : u.len[r] + u.val[i];
    if (v > u.cap) {
      v = u.cap;
      u.len[FM_MAX_REQ] = 1;
    }
    u.len[r] = v;
  }
}
__global__ __launch_bounds__(64) void ctx_update_kernel(CtxUpdate u) {
  if (threadIdx.x == 0) ctx_update(u);
}

// tokens[m] = index of max over the G workgroup keys of row m, and with
// lse_part given lse[m] = log sum_g s_g exp(m_g) over the row's G workgroup
// (max, sum) states.
// One workgroup per row: the row's G workgroup keys (and states) are
// contiguous; every thread folds its strided share, then waves and the
// workgroup combine in a fixed order (keys by max, states by log-sum-exp).
constexpr int FIN_THREADS = 256;
// The first workgroup also applies the context update `cu` of the draft.
__global__ __launch_bounds__(FIN_THREADS) void argmax_finalize_kernel(const uint64_t* partial, int G,
                                                                     int32_t* tokens, const float2* lse_part,
                                                                     float* lse, CtxUpdate cu) {
  __shared__ uint64_t sk[FIN_THREADS / 64];
  __shared__ float2 ss[FIN_THREADS / 64];
  const int m = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (m == 0 && t == 0) ctx_update(cu);
  const uint64_t* pk = partial + (size_t)m * G;
  const float2* pe = lse_part ? lse_part + (size_t)m * G : nullptr;
  uint64_t k = 0ull;
  float mx = -INFINITY, sum = 0.f;
  for (int g0 = t; g0 < G; g0 += 4 * FIN_THREADS) {
    uint64_t v[4];
    float2 e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gi = g0 + u * FIN_THREADS;
      v[u] = gi < G ? pk[gi] : 0ull;
      if (pe) e[u] = gi < G ? pe[gi] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      k = umax64(k, v[u]);
      if (pe) lse_merge(mx, sum, e[u].x, e[u].y);
    }
  }
  for (int o = 1; o < 64; o <<= 1) {
    k = umax64(k, shfl_xor_u64(k, o));
    if (pe) lse_shfl_merge(mx, sum, o);
  }
  if (lane == 0) {
    sk[wave] = k;
    ss[wave] = make_float2(mx, sum);
  }
  __syncthreads();
  if (t == 0) {
    uint64_t kk = sk[0];
    float a = ss[0].x, b = ss[0].y;
    for (int w = 1; w < FIN_THREADS / 64; ++w) {
      kk = umax64(kk, sk[w]);
      lse_merge(a, b, ss[w].x, ss[w].y);
    }
    tokens[m] = (int32_t)argmax_key_index(kk);
    if (pe) lse[m] = a + logf(b);
  }
}

}  // namespace fm
