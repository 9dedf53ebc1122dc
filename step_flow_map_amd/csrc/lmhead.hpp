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

template <typename T, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void lmhead_kernel(LmArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = ChunkT<T>::VE;
  constexpr int KC = ChunkT<T>::KC;
  __shared__ uint4 wtiles[NW * 512];
  __shared__ uint64_t wbest[NW][MT * 16];

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

// Variant with the k range split over the waves: wave w owns chunks w, w+NW,
// ... of every vocabulary tile, so its z fragments for those chunks stay in
// registers for the whole kernel (any number of rows up to 64, no z traffic in
// the loop).  A workgroup takes tiles blockIdx, blockIdx+G, ... (a tile is 16
// vocabulary rows, one contiguous stretch of W_lm); its waves stream their
// chunks of the tile (the next tile's chunks in flight), multiply, and put
// their partial tile into LDS (two buffers by tile parity, so one LDS barrier
// per tile suffices); every thread then sums the waves in order for its fixed
// output elements, updates its running key and writes the logit if asked.
// The keys of a row are combined over 16 lanes and written per workgroup for
// argmax_finalize_kernel.
template <typename T, int MT, int NW, int CPW>
__global__ __launch_bounds__(NW * 64) void lmhead_ks_kernel(LmArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = ChunkT<T>::VE;
  constexpr int KC = ChunkT<T>::KC;
  constexpr int ELEMS = MT * 256;                        // outputs of one tile
  constexpr int PER = (ELEMS + NW * 64 - 1) / (NW * 64);  // outputs per thread
  __shared__ uint4 wtiles[NW * 512];
  __shared__ float red[2][NW * ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const T* Z = reinterpret_cast<const T*>(g.z);
  const T* W = reinterpret_cast<const T*>(g.W);
  uint4* wt = wtiles + wave * 512;
  const int nch = (g.d + KC - 1) / KC;
  const int ntiles = (g.V + 15) / 16;
  const int G = gridDim.x;
  const int nt = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / G + 1 : 0;

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
#pragma unroll
  for (int r = 0; r < PER; ++r) best[r] = 0ull;

  // chunks of tile it (of this workgroup); tiles past the end read row 0
  auto load = [&](uint4 (&rb)[CPW][8], int it) {
    const int t = (int)blockIdx.x + it * G;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int c = min(wave + u * NW, nch - 1);
      chunk_load<T>(rb[u], W, g.d, t * 16, g.V, c * KC, g.d);
    }
  };
  auto process = [&](const uint4 (&rb)[CPW][8], int it) {
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      chunk_to_lds(rb[u], wt);
      wave_lds_sync();
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const VT b = as_vec<T>(chunk_frag(wt, st));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mma(acc[mt], zf[u][mt][st], b);
      }
      wave_lds_sync();
    }
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
        if (n < g.V && m < g.M) {
          best[r] = umax64(best[r], argmax_key(v, (uint32_t)n));
          if (g.logits) g.logits[(size_t)m * g.V + n] = v;
        }
      }
    }
  };

  uint4 r0[CPW][8], r1[CPW][8];
  load(r0, 0);
  for (int it = 0; it < nt; it += 2) {
    load(r1, it + 1);
    process(r0, it);
    if (it + 1 < nt) {
      load(r0, it + 2);
      process(r1, it + 1);
    }
  }

  // a row's keys: 16 lanes (the tile's columns) of one wave
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int el = tid + r * NW * 64;
    uint64_t k = best[r];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) k = umax64(k, shfl_xor_u64(k, o));
    const int ln = el & 63, q = el >> 6;
    const int m = (q >> 2) * 16 + 4 * (ln >> 4) + (q & 3);
    if (el < ELEMS && (ln & 15) == 0 && m < g.M) g.partial[(size_t)blockIdx.x * g.M + m] = k;
  }
}

// tokens[m] = index of max over G workgroup keys.  1024 threads, tpr threads
// per row on consecutive lanes of one wave (M <= 64); each thread keeps eight loads in
// flight at once, so G = 512 costs one memory latency for up to 16 rows.
constexpr int FIN_THREADS = 1024;
__global__ __launch_bounds__(FIN_THREADS) void argmax_finalize_kernel(const uint64_t* partial, int G, int M,
                                                                     int32_t* tokens) {
  int mp = 16;
  while (mp < M) mp <<= 1;
  const int tpr = FIN_THREADS / mp;
  const int m = threadIdx.x / tpr, sub = threadIdx.x % tpr;
  const int mr = m < M ? m : 0;
  uint64_t k = 0ull;
  for (int b0 = sub; b0 < G; b0 += 8 * tpr) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = b0 + u * tpr;
      v[u] = partial[(size_t)(b < G ? b : 0) * M + mr];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) k = umax64(k, b0 + u * tpr < G ? v[u] : 0ull);
  }
  for (int o = 1; o < tpr; o <<= 1) k = umax64(k, shfl_xor_u64(k, o));  // tpr <= 64
  if (m < M && sub == 0) tokens[m] = (int32_t)argmax_key_index(k);
}

}  // namespace fm
