// LayerNorm fused into the A operand of a contraction: 16 rows
//
//   a[r][k] = LN(h[r])[k] * (1 + scale[k]) + shift[k],  rounded to the storage type,
//
// computed inside every workgroup of 8 waves from the float32 residual rows h
// (never rounded before the statistics and the normalisation, which are
// float32).  The row statistics come from the kernel that produced h: it
// wrote (mean, M2) of every 16 columns of every row, and each workgroup merges
// them in a fixed order.  Wave w holds chunk w of the rows (KC columns), so
// the k range is at most 8 chunks.  Used by the tile-group contraction for the
// two adaLN-modulated LayerNorms of a DiT block (before QKV and before the
// first MLP layer).
#pragma once
#include "common.hpp"
#include "stream.hpp"

namespace fm {

struct LnArgs {
  const float* h;      // [16][ldh] float32 residual stream
  int ldh;
  const float* shift;  // [K]
  const float* scale;  // [K]
  float eps;
  // per-16-column (mean, M2) of every row of h, written by the kernel that
  // produced h: [16][part_ld], K / 16 entries per row
  const float2* part;
  int part_ld;
};
constexpr int LN_PART_MAX = 128;  // K / 16 for K up to 2048, the fused LayerNorm's longest row

// What one thread loads: float4 element i of the lane covers row hrow(i),
// columns k0 + hcol .. + 3 of the wave's chunk (the same columns in every row
// it holds), one float4 each of the modulation, and the statistics partials
// (t % 32) + 32u of row t / 32 (thread t of the 512).
template <typename T>
struct LnChunk {
  static constexpr int KC = ChunkT<T>::KC;
  static constexpr int HN = KC / 16;  // 16 rows x KC floats / (64 lanes x 4)
  static constexpr int PU = LN_PART_MAX / 32;
  float4 hv[HN];
  float4 msc, msh;
  float2 pp[PU];
  __device__ __forceinline__ static int hcol() { return ((threadIdx.x & 63) * 4) % KC; }
  __device__ __forceinline__ static int hrow(int i) { return (i * 256 + (threadIdx.x & 63) * 4) / KC; }
};

// Issue the loads of the wave's chunk at k0 (has = false: the wave has no
// chunk, but its threads still take part in the statistics), partials first
// so that the statistics are ready before the rows.  Every load is
// unconditional with a clamped address: a masked load would make the wave
// wait for all of them at once.  K: the row length (a multiple of 16).
template <typename T>
__device__ __forceinline__ void ln_issue(LnChunk<T>& c, const LnArgs& ln, int K, int k0, int k_end, bool has) {
  const int tid = threadIdx.x, prow = tid >> 5, psub = tid & 31, np = K >> 4;
#pragma unroll
  for (int u = 0; u < LnChunk<T>::PU; ++u)  // the count masks the unused ones
    c.pp[u] = ln.part[(size_t)prow * ln.part_ld + min(psub + 32 * u, np - 1)];
  const int hc = LnChunk<T>::hcol();
  const int kc = has && k0 + hc < k_end ? k0 + hc : 0;
#pragma unroll
  for (int i = 0; i < LnChunk<T>::HN; ++i)
    c.hv[i] = *reinterpret_cast<const float4*>(ln.h + (size_t)LnChunk<T>::hrow(i) * ln.ldh + kc);
  c.msc = *reinterpret_cast<const float4*>(ln.scale + kc);
  c.msh = *reinterpret_cast<const float4*>(ln.shift + kc);
}

// Row statistics, normalisation and the MFMA fragments of the wave's chunk.
// Thread t merges its partials of row t / 32 in order (pairwise update of
// Chan, Golub and LeVeque; every partial covers 16 columns), the 32 threads
// of the row merge in a fixed tree (a DPP row, then its two halves), and
// thread 32r publishes row r's mean and 1 / std through sstat.  After one LDS
// barrier (loads in flight stay in flight) every wave normalises, modulates
// and rounds its values into its LDS tile wt in the weights' chunk layout
// (piece p of row r at r * 32 + (p ^ r)) and reads its fragments back.  All
// 512 threads of the workgroup must call it.
template <typename T>
__device__ __forceinline__ void ln_finish(const LnChunk<T>& c, const LnArgs& ln, int K, uint4* wt,
                                          float (*sstat)[2], typename Vec<T>::type (&af)[8]) {
  const int tid = threadIdx.x, lane = tid & 63, prow = tid >> 5, psub = tid & 31, np = K >> 4;
  float n = 0.f, mean = 0.f, M2 = 0.f;
  auto merge = [&](float nb, float mb, float m2b) {
    const float nn = n + nb, delta = mb - mean;
    const float f = nb > 0.f ? nb / nn : 0.f;
    mean += delta * f;
    M2 += nb > 0.f ? m2b + delta * delta * (n * f) : 0.f;
    n = nn;
  };
#pragma unroll
  for (int u = 0; u < LnChunk<T>::PU; ++u) merge(psub + 32 * u < np ? 16.f : 0.f, c.pp[u].x, c.pp[u].y);
  {
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
  }
  if (psub == 0) {
    sstat[prow][0] = mean;
    sstat[prow][1] = 1.f / sqrtf(M2 / (float)K + ln.eps);
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < LnChunk<T>::HN; ++i) {
    const int rr = LnChunk<T>::hrow(i);
    const float m_r = sstat[rr][0], s_r = sstat[rr][1];
    const float4 hv = c.hv[i], sc = c.msc, sh = c.msh;
    const float y0 = ((hv.x - m_r) * s_r) * (1.f + sc.x) + sh.x;
    const float y1 = ((hv.y - m_r) * s_r) * (1.f + sc.y) + sh.y;
    const float y2 = ((hv.z - m_r) * s_r) * (1.f + sc.z) + sh.z;
    const float y3 = ((hv.w - m_r) * s_r) * (1.f + sc.w) + sh.w;
    if constexpr (sizeof(T) == 2) {
      const int pc = lane >> 1;  // 16-byte piece of 8 columns; this lane holds half of it
      uint2 u;
      u.x = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
      u.y = (uint32_t)f32_to_bf16(y2) | ((uint32_t)f32_to_bf16(y3) << 16);
      reinterpret_cast<uint2*>(wt + rr * 32 + (pc ^ rr))[lane & 1] = u;
    } else {
      const int pc = lane & 31;
      wt[rr * 32 + (pc ^ rr)] =
          make_uint4(__float_as_uint(y0), __float_as_uint(y1), __float_as_uint(y2), __float_as_uint(y3));
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int st = 0; st < 8; ++st) af[st] = as_vec<T>(chunk_frag(wt, st));
  wave_lds_sync();
}

}  // namespace fm
