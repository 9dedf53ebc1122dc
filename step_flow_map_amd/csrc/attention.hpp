// Attention of the K block rows of one branch over [context; own block] keys.
//
// Every query sees every key (no mask).  Keys/values of context rows come from
// the cache ([C_max][2][d] per block, written by the QKV epilogue); those of
// block rows from this branch's rows of the QKV buffer, so branches of a draft
// tree share the context but never see each other's rows.  Scores, softmax
// and P.V run in float32 on the VALU (P is not rounded).
//
// Work split: one workgroup per (branch, head, chunk of CH keys).  It stages
// q, K and V of its chunk in LDS as float32, writes a partial (row max, row
// sum, unnormalised output) and the last chunk to finish merges all chunks of
// the (branch, head) in chunk order and writes the output in storage type.
#pragma once
#include "common.hpp"

namespace fm {

struct AttnArgs {
  const void* qkv;    // [B*K][3d]: query at column 0, key at d, value at 2d
  int ld_qkv;
  const void* cache;  // this block's [C_max][2][d]
  int C;              // context rows visible to the block
  int K, d, nh;
  int n_chunks;       // ceil((C + K) / CH)
  float* part_o;      // [B*nh][n_chunks][K][HD]
  float* part_ml;     // [B*nh][n_chunks][K][2]
  uint32_t* counters; // [B*nh]
  void* out;          // [B*K][d]
  float scale;        // 1/sqrt(hd)
};

template <typename T, int HD, int CH>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs g) {
  constexpr int KB = 16;           // block rows per branch
  constexpr int NT = 256;
  static_assert(CH == 64, "one key per lane of a wave");
  __shared__ float sq[KB][HD];
  __shared__ float sk[CH][HD + 1];
  __shared__ float sv[CH][HD];
  __shared__ float sp[KB][CH];
  __shared__ int flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x % g.n_chunks;
  const int bh = blockIdx.x / g.n_chunks;
  const int head = bh % g.nh, b = bh / g.nh;
  const int total = g.C + g.K;
  const int key0 = chunk * CH;
  const T* qkv = reinterpret_cast<const T*>(g.qkv);
  const T* cache = reinterpret_cast<const T*>(g.cache);
  const int hoff = head * HD;

  // stage q (K rows), keys and values of the chunk
  for (int idx = tid; idx < KB * HD; idx += NT) {
    const int i = idx / HD, c = idx % HD;
    sq[i][c] = to_f32<T>(qkv[(size_t)(b * g.K + i) * g.ld_qkv + hoff + c]);
  }
  for (int idx = tid; idx < CH * HD; idx += NT) {
    const int kk = idx / HD, c = idx % HD;
    const int key = key0 + kk;
    float kv = 0.f, vv = 0.f;
    if (key < g.C) {
      const T* p = cache + (size_t)key * 2 * g.d + hoff + c;
      kv = to_f32<T>(p[0]);
      vv = to_f32<T>(p[g.d]);
    } else if (key < total) {
      const T* p = qkv + (size_t)(b * g.K + (key - g.C)) * g.ld_qkv + hoff + c;
      kv = to_f32<T>(p[g.d]);
      vv = to_f32<T>(p[2 * g.d]);
    }
    sk[kk][c] = kv;
    sv[kk][c] = vv;
  }
  __syncthreads();

  // scores: lane = key, rows wave, wave+4, wave+8, wave+12
  const int key = key0 + lane;
  const bool valid = key < total;
  float mrow[4], lrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = wave + 4 * r;
    float sc = 0.f;
#pragma unroll 8
    for (int c = 0; c < HD; ++c) sc += sq[i][c] * sk[lane][c];
    sc = valid ? sc * g.scale : -INFINITY;
    const float mx = warp_max(sc);  // every chunk holds at least one valid key
    const float p = valid ? expf(sc - mx) : 0.f;
    const float l = warp_sum(p);
    sp[i][lane] = p;
    mrow[r] = mx;
    lrow[r] = l;
  }
  const size_t pbase = (size_t)bh * g.n_chunks + chunk;
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = wave + 4 * r;
      g.part_ml[(pbase * KB + i) * 2 + 0] = mrow[r];
      g.part_ml[(pbase * KB + i) * 2 + 1] = lrow[r];
    }
  }
  __syncthreads();

  // unnormalised P.V: thread owns column c for rows i0, i0 + RS, ...
  constexpr int RS = NT / HD;        // rows handled in parallel
  const int c = tid % HD, i0 = tid / HD;
  const int lim = min(CH, total - key0);
  for (int i = i0; i < KB; i += RS) {
    float o = 0.f;
    for (int kk = 0; kk < lim; ++kk) o += sp[i][kk] * sv[kk][c];
    g.part_o[(pbase * KB + i) * HD + c] = o;
  }

  if (!arrive_last(&g.counters[bh], (uint32_t)g.n_chunks, &flag)) return;

  // merge chunks in order
  T* out = reinterpret_cast<T*>(g.out);
  const size_t cbase = (size_t)bh * g.n_chunks;
  for (int i = i0; i < KB; i += RS) {
    float M = -INFINITY;
    for (int ch = 0; ch < g.n_chunks; ++ch) M = fmaxf(M, g.part_ml[((cbase + ch) * KB + i) * 2]);
    float den = 0.f, num = 0.f;
    for (int ch = 0; ch < g.n_chunks; ++ch) {
      const float w = expf(g.part_ml[((cbase + ch) * KB + i) * 2] - M);
      den += w * g.part_ml[((cbase + ch) * KB + i) * 2 + 1];
      num += w * g.part_o[((cbase + ch) * KB + i) * HD + c];
    }
    out[(size_t)(b * g.K + i) * g.d + hoff + c] = from_f32<T>(num / den);
  }
}

}  // namespace fm
