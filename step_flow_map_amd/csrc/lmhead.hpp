// Frozen LM head with the draft decision fused in:
//
//   logits[m][v] = sum_c z[m][c] * W_lm[v][c]      (float32, no bias)
//   tokens[m]    = lowest v among the maxima of logits[m][:]
//
// Persistent grid: every wave walks a fixed set of 16-row vocabulary tiles
// (tile t, t + waves, ...), streaming each tile's d-wide rows chunk by chunk
// through its LDS tile into MFMA operands with the next chunk in flight.  z is
// staged once per workgroup in LDS (XOR-swizzled rows) when it fits.  The
// running best of each row is an order-preserving 64-bit key (value, then lower
// index), so lanes, waves and workgroups combine with a plain max in any order;
// each workgroup writes its keys and argmax_finalize_kernel reduces them.
#pragma once
#include "common.hpp"
#include "stream.hpp"

namespace fm {

struct LmArgs {
  const void* z;      // [M][d]
  int M, d;
  const void* W;      // [V][d]
  int V;
  float* logits;      // [M][V] or null
  uint64_t* partial;  // [gridDim.x][M]
};

constexpr int LM_ZLDS_U4 = 4096;  // 64 KB of z in LDS

template <typename T, int MT, int NW, bool ZLDS>
__global__ __launch_bounds__(NW * 64) void lmhead_kernel(LmArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = ChunkT<T>::VE;
  constexpr int KC = ChunkT<T>::KC;
  static_assert(!ZLDS || MT == 1, "z in LDS holds one 16-row tile");
  __shared__ uint4 wtiles[NW * 512];
  __shared__ uint4 zs[ZLDS ? LM_ZLDS_U4 : 1];
  __shared__ uint64_t wbest[NW][MT * 16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const T* Z = reinterpret_cast<const T*>(g.z);
  const T* W = reinterpret_cast<const T*>(g.W);
  const int pieces = g.d / VE;  // 16-byte pieces per z row

  if (ZLDS) {  // rows m < M, piece p at m*pieces + (p ^ (m & 15))
    const uint4* zg = reinterpret_cast<const uint4*>(Z);
    for (int i = threadIdx.x; i < 16 * pieces; i += NW * 64) {
      const int m = i / pieces, p = i % pieces;
      zs[m * pieces + (p ^ (m & 15))] = m < g.M ? zg[(size_t)m * pieces + p] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
  }

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
        VT av;
        if (ZLDS) {
          const int p = kok ? k / VE : 0;
          av = as_vec<T>(zs[j * pieces + (p ^ j)]);
          av = kok ? av : vzero<VT>();
        } else {
          const bool ok = kok && zok[mt];
          av = vload<T>(zrow[mt] + (ok ? k : 0));
          av = ok ? av : vzero<VT>();
        }
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
          if (n < g.V && m < g.M) {
            const float v = acc[mt][i];
            best[mt][i] = umax64(best[mt][i], argmax_key(v, (uint32_t)n));
            if (g.logits) g.logits[(size_t)m * g.V + n] = v;
          }
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
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) k = umax64(k, shfl_xor_u64(k, o));
      if (j == 0) wbest[wave][mt * 16 + 4 * grp + i] = k;
    }
  __syncthreads();
  for (int m = threadIdx.x; m < g.M; m += NW * 64) {
    uint64_t k = 0ull;
#pragma unroll
    for (int w = 0; w < NW; ++w) k = umax64(k, wbest[w][m]);
    g.partial[(size_t)blockIdx.x * g.M + m] = k;
  }
}

// tokens[m] = index of max over G workgroup keys; 256 threads, tpr threads per
// row on consecutive lanes (M <= 64)
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const uint64_t* partial, int G, int M, int32_t* tokens) {
  int mp = 4;
  while (mp < M) mp <<= 1;
  const int tpr = 256 / mp;
  const int m = threadIdx.x / tpr, sub = threadIdx.x % tpr;
  uint64_t k = 0ull;
  if (m < M)
    for (int b = sub; b < G; b += tpr) k = umax64(k, partial[(size_t)b * M + m]);
  for (int o = 1; o < tpr; o <<= 1) k = umax64(k, shfl_xor_u64(k, o));
  if (m < M && sub == 0) tokens[m] = (int32_t)argmax_key_index(k);
}

}  // namespace fm
