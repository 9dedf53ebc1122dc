// Attention of the K = 16 block rows of one branch over [context; own block]
// keys (every query sees every key, no mask).
//
// Cache layout, per DiT block and head, P positions (context rows, then one
// 32-position scratch block per branch that holds that branch's 16 block rows):
//   keys    kc[head][pos][hd]                         row-major
//   values  vt[head][pos / 32][hd][32]                transposed in 32-key blocks,
//           key kk of a block at slot vt_slot<T>(kk)
// so that every MFMA operand of the kernel is one contiguous 16-byte load.
//
// One wave handles whole 32-key blocks.  For a block it computes the
// transposed scores S^T = K Q^T (MFMA, A = 16 keys, B = the 16 queries), which
// leaves lane (query j, group g) holding the 8 scores of query j for keys
// 4g..4g+3 and 16+4g..16+4g+3: exactly the B operand of O^T += V^T P^T for
// that key order, so probabilities never leave registers.  The value cache
// stores the keys of a block in the same order, so the A operand (V^T) is a
// single load as well.  Softmax runs online per wave and query row (running
// max and sum, rescaling the accumulator).  In bf16 storage P is split into
// hi + lo bf16 parts, two MFMAs per tile, which keeps P to 16 significant bits
// (float32 accumulation throughout); float storage multiplies in float32.
//
// Work split: a workgroup (NW waves) per (branch, head, block range); waves
// take the range's blocks round-robin with the next block's loads in flight
// while the current one is computed, then merge their (max, sum, output)
// through LDS.  Short contexts use a single range, so no merge crosses
// workgroups.
// With several ranges per (branch, head) each publishes its merged state with
// coherent stores and the last to arrive (at most 8) merges them in range order.
// Results never depend on scheduling.
#pragma once
#include "common.hpp"

namespace fm {

constexpr int ATT_RANGES_MAX = 8;  // ranges per (branch, head) = arrivals per counter
constexpr int FM_MAX_REQ = 4;      // requests with their own context in one launch
constexpr int ATT_BLK = 32;        // keys per block

// slot of key kk (0..31) inside a 32-key block of the value cache
template <typename T> __host__ __device__ __forceinline__ int vt_slot(int kk);
template <> __host__ __device__ __forceinline__ int vt_slot<bf16_t>(int kk) {
  return 8 * ((kk & 15) >> 2) + 4 * (kk >> 4) + (kk & 3);
}
template <> __host__ __device__ __forceinline__ int vt_slot<float>(int kk) { return kk; }

struct AttnArgs {
  const void* q;       // [B*K][ldq] queries of the block rows
  int ldq;
  const void* kc;      // this DiT block's key cache   [nh][P][hd] (request 0)
  const void* vt;      // this DiT block's value cache [nh][P/32][hd][32] (request 0)
  size_t req_stride;   // elements between consecutive requests' caches
  int P;               // positions per head (multiple of 32)
  int C[FM_MAX_REQ];   // context rows visible to branch b
  int scratch_blk;     // block index of the first block rows
  int scratch_step;    // 1: branches share request 0's cache (branch b at scratch_blk + b);
                       // 0: branch b is request b (its rows at scratch_blk of its own cache)
  int K, d, nh;
  int n_ranges;        // ranges per (branch, head), <= 8
  int blocks_per_range;
  float* part_o;       // [B*nh][n_ranges][K][HD]
  float* part_ml;      // [B*nh][n_ranges][K][2]
  uint32_t* counters;  // [B*nh], COUNTER_STRIDE apart
  void* out;           // [B*K][d]
  float scale;         // 1/sqrt(hd)
};

template <typename T, int HD, int NW>
__global__ __launch_bounds__(NW * 64) void attention_kernel(AttnArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int KB = 16;              // block rows (queries) per branch
  constexpr int VE = Vec<T>::N;
  constexpr int QS = HD / (4 * VE);   // score MFMA steps over the head width
  constexpr int OT = HD / 16;         // 16-dim output tiles
  constexpr int PS = 32 / (4 * VE);   // P.V steps per block: bf16 1, float 2
  constexpr bool BF = sizeof(T) == 2;
  __shared__ float so[NW][KB][HD + 4];
  __shared__ float sm[NW][KB], sl[NW][KB];
  __shared__ int flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int range = blockIdx.x % g.n_ranges;
  const int bh = blockIdx.x / g.n_ranges;
  const int head = bh % g.nh, b = bh / g.nh;
  const int C = g.C[b];
  const int ctx_blocks = (C + ATT_BLK - 1) / ATT_BLK;
  const int nblk = ctx_blocks + 1;
  const int blo = range * g.blocks_per_range;
  const int bhi = min(nblk, blo + g.blocks_per_range);  // empty for ranges past a short context
  const size_t rb = g.scratch_step ? 0 : (size_t)b * g.req_stride;
  const T* kbase = reinterpret_cast<const T*>(g.kc) + rb + (size_t)head * g.P * HD;
  const T* vbase = reinterpret_cast<const T*>(g.vt) + rb + (size_t)head * (g.P / ATT_BLK) * HD * ATT_BLK;

  // queries (B operand): lane (row j, group grp) holds piece 4s+grp of query j
  VT qf[QS];
  {
    const T* qrow = reinterpret_cast<const T*>(g.q) + (size_t)(b * g.K + j) * g.ldq + head * HD;
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[s] = vload<T>(qrow + (4 * s + grp) * VE);
  }

  struct Tile {
    VT k[2][QS];     // keys 16*tb + j, pieces 4s+grp
    VT v[PS][OT];    // value dims 16t + j, slots ps*4*VE + grp*VE ..
  };
  // physical block and number of valid keys of logical block bi
  auto phys = [&](int bi) { return bi < ctx_blocks ? bi : g.scratch_blk + g.scratch_step * b; };
  auto nvalid = [&](int bi) { return bi < ctx_blocks ? min(ATT_BLK, C - ATT_BLK * bi) : KB; };
  auto load = [&](Tile& t, int bi) {
    const int pb = phys(bi);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const T* kr = kbase + (size_t)(pb * ATT_BLK + 16 * tb + j) * HD;
#pragma unroll
      for (int s = 0; s < QS; ++s) t.k[tb][s] = vload<T>(kr + (4 * s + grp) * VE);
    }
    const T* vb = vbase + (size_t)pb * HD * ATT_BLK;
#pragma unroll
    for (int ps = 0; ps < PS; ++ps)
#pragma unroll
      for (int ot = 0; ot < OT; ++ot)
        t.v[ps][ot] = vload<T>(vb + (size_t)(16 * ot + j) * ATT_BLK + ps * 4 * VE + grp * VE);
  };

  float m_run = -INFINITY, l_run = 0.f;  // of query row j (same in all four groups)
  f32x4 o[OT];                           // o[t][i] = O[row j][16t + 4grp + i]
#pragma unroll
  for (int t = 0; t < OT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](Tile& t, int bi) {
    const int nv = nvalid(bi);
    // transposed scores: sc[tb][i] = S[query j][key 16tb + 4grp + i]
    f32x4 sc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < QS; ++s) mma(sc[tb], t.k[tb][s], qf[s]);
    }
    float mb = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 16 * tb + 4 * grp + i;
        sc[tb][i] = kk < nv ? sc[tb][i] * g.scale : -INFINITY;
        mb = fmaxf(mb, sc[tb][i]);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float m_new = fmaxf(m_run, mb);  // finite: key 0 of every block is valid
    const float corr = expf(m_run - m_new);
    float p[2][4], ps_sum = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[tb][i] = expf(sc[tb][i] - m_new);  // 0 for masked keys
        ps_sum += p[tb][i];
      }
    ps_sum += __shfl_xor(ps_sum, 16, 64);
    ps_sum += __shfl_xor(ps_sum, 32, 64);
    l_run = l_run * corr + ps_sum;
    m_run = m_new;
#pragma unroll
    for (int ot = 0; ot < OT; ++ot)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[ot][i] *= corr;
    // values of masked keys are zeroed (the cache there may hold anything)
    const bool partial = nv < ATT_BLK;
    if constexpr (BF) {
      // P^T fragment: element e <- key (e < 4 ? 4grp+e : 16+4grp+e-4) = sc layout
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = p[w >> 1][(2 * w) & 3], c = p[w >> 1][(2 * w + 1) & 3];
        const bf16_t ah = f32_to_bf16(a), ch = f32_to_bf16(c);
        const bf16_t al = f32_to_bf16(a - bf16_to_f32(ah)), cl = f32_to_bf16(c - bf16_to_f32(ch));
        hi[w] = (uint32_t)ah | ((uint32_t)ch << 16);
        lo[w] = (uint32_t)al | ((uint32_t)cl << 16);
      }
      const uint4 phi = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      const uint4 plo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      uint4 vmask = make_uint4(~0u, ~0u, ~0u, ~0u);
      if (partial) {
        uint32_t mw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int e0 = 2 * w, e1 = 2 * w + 1;
          const int k0 = e0 < 4 ? 4 * grp + e0 : 16 + 4 * grp + e0 - 4;
          const int k1 = e1 < 4 ? 4 * grp + e1 : 16 + 4 * grp + e1 - 4;
          mw[w] = (k0 < nv ? 0xFFFFu : 0u) | (k1 < nv ? 0xFFFF0000u : 0u);
        }
        vmask = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      }
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) {
        uint4 v = t.v[0][ot];
        v.x &= vmask.x; v.y &= vmask.y; v.z &= vmask.z; v.w &= vmask.w;
        mma(o[ot], v, phi);
        mma(o[ot], v, plo);
      }
    } else {
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        // step ps covers keys 16ps + 4grp + i: lane's p[ps][i]
        const float4 pf = make_float4(p[ps][0], p[ps][1], p[ps][2], p[ps][3]);
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) {
          float4 v = t.v[ps][ot];
          if (partial) {
            const int k0 = 16 * ps + 4 * grp;
            v.x = k0 + 0 < nv ? v.x : 0.f;
            v.y = k0 + 1 < nv ? v.y : 0.f;
            v.z = k0 + 2 < nv ? v.z : 0.f;
            v.w = k0 + 3 < nv ? v.w : 0.f;
          }
          mma(o[ot], v, pf);
        }
      }
    }
  };

  // blocks blo + wave, +NW, ... with the next block's loads in flight
  Tile t0, t1;
  int bi = blo + wave;
  if (bi < bhi) load(t0, bi);
  for (; bi < bhi; bi += 2 * NW) {
    if (bi + NW < bhi) load(t1, bi + NW);
    process(t0, bi);
    if (bi + NW < bhi) {
      if (bi + 2 * NW < bhi) load(t0, bi + 2 * NW);
      process(t1, bi + NW);
    }
  }

  // ---- merge the waves (fixed order) through LDS
#pragma unroll
  for (int ot = 0; ot < OT; ++ot)
    *reinterpret_cast<float4*>(&so[wave][j][16 * ot + 4 * grp]) = make_float4(o[ot][0], o[ot][1], o[ot][2], o[ot][3]);
  if (grp == 0) {
    sm[wave][j] = m_run;
    sl[wave][j] = l_run;
  }
  __syncthreads();
  constexpr int CPT = KB * HD / (NW * 64);  // output columns per thread
  const int row = tid / (HD / CPT), c0 = (tid % (HD / CPT)) * CPT;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w][row]);
  float Lsum = 0.f, acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    // 0 for waves without blocks (and for a range without blocks, where M = -inf)
    const float wt = M == -INFINITY ? 0.f : expf(sm[w][row] - M);
    Lsum += wt * sl[w][row];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] += wt * so[w][row][c0 + c];
  }
  T* out = reinterpret_cast<T*>(g.out) + (size_t)(b * g.K + row) * g.d + head * HD + c0;
  if (g.n_ranges == 1) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) out[c] = from_f32<T>(acc[c] / Lsum);
    return;
  }
  // ---- publish this range, the last range of the (branch, head) merges
  const size_t pbase = ((size_t)bh * g.n_ranges + range) * KB + row;
#pragma unroll
  for (int c = 0; c < CPT; ++c) st_coh(&g.part_o[pbase * HD + c0 + c], acc[c]);
  if (c0 == 0) {
    st_coh(&g.part_ml[pbase * 2 + 0], M);
    st_coh(&g.part_ml[pbase * 2 + 1], Lsum);
  }
  if (!arrive(&g.counters[bh * COUNTER_STRIDE], (uint32_t)g.n_ranges, &flag)) return;
  float mv[ATT_RANGES_MAX], lv[ATT_RANGES_MAX], ov[ATT_RANGES_MAX][CPT];
#pragma unroll
  for (int r = 0; r < ATT_RANGES_MAX; ++r) {
    const bool ok = r < g.n_ranges;
    const size_t pi = ((size_t)bh * g.n_ranges + (ok ? r : 0)) * KB + row;
    mv[r] = ok ? ld_coh(&g.part_ml[pi * 2]) : -INFINITY;
    lv[r] = ok ? ld_coh(&g.part_ml[pi * 2 + 1]) : 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) ov[r][c] = ok ? ld_coh(&g.part_o[pi * HD + c0 + c]) : 0.f;
  }
  float MM = -INFINITY;
#pragma unroll
  for (int r = 0; r < ATT_RANGES_MAX; ++r) MM = fmaxf(MM, mv[r]);
  float den = 0.f, num[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) num[c] = 0.f;
#pragma unroll
  for (int r = 0; r < ATT_RANGES_MAX; ++r) {
    const float wt = r < g.n_ranges ? expf(mv[r] - MM) : 0.f;
    den += wt * lv[r];
#pragma unroll
    for (int c = 0; c < CPT; ++c) num[c] += wt * ov[r][c];
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) out[c] = from_f32<T>(num[c] / den);
}

}  // namespace fm
