// Attention of the K = 16 block rows of one branch over [context; own block]
// keys.
//
// Every query sees every key (no mask).  Keys/values of context rows come from
// the cache ([C_max][2][d] per block, written by the QKV epilogue); those of
// block rows from this branch's rows of the QKV buffer, so branches of a draft
// tree share the context but never see each other's rows.
//
// Work split: one workgroup (4 waves) per (branch, head, key range).  It walks
// its range in 64-key sub-chunks, 16 keys per wave:
//   scores  S = q k^T * scale   MFMA over storage-type operands (exact products,
//                               float32 accumulation), wave w -> keys 16w..16w+15
//   softmax running row max / row sum across sub-chunks (online softmax)
//   P.V     float32 MFMA (P is not rounded), wave w -> output columns
//           w*HD/4 .. (w+1)*HD/4 - 1, V staged in LDS as float32
// It publishes (max, sum, unnormalised output) with coherent stores; the last of
// the (at most 8) ranges of a (branch, head) merges them in range order and
// writes the output in storage type.
#pragma once
#include "common.hpp"

namespace fm {

constexpr int ATT_RANGES_MAX = 8;  // key ranges per (branch, head) = arrivals per counter

struct AttnArgs {
  const void* qkv;    // [B*K][3d]: query at column 0, key at d, value at 2d
  int ld_qkv;
  const void* cache;  // this block's [C_max][2][d]
  int C;              // context rows visible to the block
  int K, d, nh;
  int n_ranges;       // key ranges per (branch, head), <= 8
  int range_keys;     // keys per range (multiple of 64)
  float* part_o;      // [B*nh][n_ranges][K][HD]
  float* part_ml;     // [B*nh][n_ranges][K][2]
  uint32_t* counters; // [B*nh], COUNTER_STRIDE apart
  void* out;          // [B*K][d]
  float scale;        // 1/sqrt(hd)
};

template <typename T, int HD>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int KB = 16;            // block rows per branch
  constexpr int CH = 64;            // keys per sub-chunk
  constexpr int VE = Vec<T>::N;
  constexpr int QSTEPS = HD / (4 * VE);  // MFMA k-steps over the head width
  constexpr int OT = HD / 64;            // 16-column output tiles per wave
  __shared__ float sv[CH][HD + 4];       // values of the sub-chunk, float32
  __shared__ float sp[KB][CH + 4];       // probabilities of the sub-chunk
  __shared__ float swmax[4][KB], swsum[4][KB];
  __shared__ float scorr[KB], srow_m[KB], srow_l[KB];
  __shared__ int flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int range = blockIdx.x % g.n_ranges;
  const int bh = blockIdx.x / g.n_ranges;
  const int head = bh % g.nh, b = bh / g.nh;
  const int total = g.C + g.K;
  const int key_lo = range * g.range_keys;
  const int key_hi = min(total, key_lo + g.range_keys);
  const T* qkv = reinterpret_cast<const T*>(g.qkv);
  const T* cache = reinterpret_cast<const T*>(g.cache);
  const int hoff = head * HD;

  // q fragments: lane (row j, group grp) holds piece 4s+grp of query row j
  VT qf[QSTEPS];
  {
    const T* qrow = qkv + (size_t)(b * g.K + j) * g.ld_qkv + hoff;
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) qf[s] = vload<T>(qrow + (4 * s + grp) * VE);
  }
  if (tid < KB) {
    srow_m[tid] = -INFINITY;
    srow_l[tid] = 0.f;
  }
  f32x4 o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto key_ptr = [&](int key) -> const T* {  // start of the key row (value at +d)
    return key < g.C ? cache + (size_t)key * 2 * g.d + hoff
                     : qkv + (size_t)(b * g.K + (key - g.C)) * g.ld_qkv + g.d + hoff;
  };

  for (int key0 = key_lo; key0 < key_hi; key0 += CH) {
    __syncthreads();  // previous sub-chunk's sv / sp fully consumed
    // stage values (float32) of the 64 keys
    for (int idx = tid; idx < CH * HD / VE; idx += 256) {
      const int kk = idx / (HD / VE), cc = (idx % (HD / VE)) * VE;
      const int key = key0 + kk;
      VT vv = vzero<VT>();
      if (key < key_hi) vv = vload<T>(key_ptr(key) + g.d + cc);
#pragma unroll
      for (int e = 0; e < VE; ++e) sv[kk][cc + e] = velem(vv, e);
    }
    // scores of this wave's 16 keys: lane (j, grp) -> rows 4*grp+i, key 16*wave+j
    const int key = key0 + 16 * wave + j;
    const bool valid = key < key_hi;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    {
      const T* kr = key_ptr(valid ? key : key0);
#pragma unroll
      for (int s = 0; s < QSTEPS; ++s) {
        const VT kv = vload<T>(kr + (4 * s + grp) * VE);
        mma(sc, qf[s], valid ? kv : vzero<VT>());
      }
    }
    float rmax[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = valid ? sc[i] * g.scale : -INFINITY;
      float m = sc[i];
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) m = fmaxf(m, __shfl_xor(m, o2, 64));
      rmax[i] = m;
    }
    if (j == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) swmax[wave][4 * grp + i] = rmax[i];
    }
    __syncthreads();
    float mnew[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * grp + i;
      float m = srow_m[row];
#pragma unroll
      for (int w = 0; w < 4; ++w) m = fmaxf(m, swmax[w][row]);
      mnew[i] = m;  // finite: key0 (wave 0, lane 0) is always valid
      const float p = valid ? expf(sc[i] - m) : 0.f;
      sp[row][16 * wave + j] = p;
      float ssum = p;
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) ssum += __shfl_xor(ssum, o2, 64);
      if (j == 0) swsum[wave][row] = ssum;
    }
    __syncthreads();
    if (tid < KB) {
      float m = srow_m[tid];
#pragma unroll
      for (int w = 0; w < 4; ++w) m = fmaxf(m, swmax[w][tid]);
      const float corr = expf(srow_m[tid] - m);  // 0 on the first sub-chunk
      float l = srow_l[tid] * corr;
#pragma unroll
      for (int w = 0; w < 4; ++w) l += swsum[w][tid];
      scorr[tid] = corr;
      srow_m[tid] = m;
      srow_l[tid] = l;
    }
    __syncthreads();
    // rescale the running output, then add P.V for this wave's column tiles
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] *= scorr[4 * grp + i];
#pragma unroll
    for (int s = 0; s < CH / 4; ++s) {
      const float pa = sp[j][4 * s + grp];
#pragma unroll
      for (int t = 0; t < OT; ++t) {
        const float vb = sv[4 * s + grp][wave * (HD / 4) + 16 * t + j];
        o[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vb, o[t], 0, 0, 0);
      }
    }
    (void)mnew;
  }

  // publish: output rows 4*grp+i, columns wave*HD/4 + 16t + j
  const size_t pbase = (size_t)bh * g.n_ranges + range;
#pragma unroll
  for (int t = 0; t < OT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st_coh(&g.part_o[(pbase * KB + 4 * grp + i) * HD + wave * (HD / 4) + 16 * t + j], o[t][i]);
  if (tid < KB) {
    st_coh(&g.part_ml[(pbase * KB + tid) * 2 + 0], srow_m[tid]);
    st_coh(&g.part_ml[(pbase * KB + tid) * 2 + 1], srow_l[tid]);
  }
  if (!arrive(&g.counters[bh * COUNTER_STRIDE], (uint32_t)g.n_ranges, &flag)) return;

  // merge ranges in order; every coherent load is issued before any is used
  T* out = reinterpret_cast<T*>(g.out);
  const size_t cbase = (size_t)bh * g.n_ranges;
  constexpr int RS = 256 / HD;  // rows handled in parallel
  const int c = tid % HD, i0 = tid / HD;
#pragma unroll
  for (int r = 0; r < KB / RS; ++r) {
    const int i = i0 + r * RS;
    float mv[ATT_RANGES_MAX], lv[ATT_RANGES_MAX], ov[ATT_RANGES_MAX];
#pragma unroll
    for (int ch = 0; ch < ATT_RANGES_MAX; ++ch) {
      const bool ok = ch < g.n_ranges;
      const size_t pi = (cbase + (ok ? ch : 0)) * KB + i;
      mv[ch] = ok ? ld_coh(&g.part_ml[pi * 2]) : -INFINITY;
      lv[ch] = ok ? ld_coh(&g.part_ml[pi * 2 + 1]) : 0.f;
      ov[ch] = ok ? ld_coh(&g.part_o[pi * HD + c]) : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int ch = 0; ch < ATT_RANGES_MAX; ++ch) M = fmaxf(M, mv[ch]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int ch = 0; ch < ATT_RANGES_MAX; ++ch) {
      const float w = ch < g.n_ranges ? expf(mv[ch] - M) : 0.f;
      den += w * lv[ch];
      num += w * ov[ch];
    }
    out[(size_t)(b * g.K + i) * g.d + hoff + c] = from_f32<T>(num / den);
  }
}

}  // namespace fm
