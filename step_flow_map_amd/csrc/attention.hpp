// Attention of the K = 16 block rows of one branch over [context; own block]
// keys (every query sees every key, no mask).
//
// Cache layout, per DiT block and head, P positions (context rows, then one
// 32-position scratch block per branch that holds that branch's 16 block rows)
// in 32-key blocks of 32 x hd keys (key cache) and 32 x hd values (value
// cache).  Inside a block both are stored in the order of the MFMA operands
// that read them (kt_off, vt_off): every operand is one 16-byte piece per
// lane, and the 64 lanes of a wave read 1 KB in lane order.
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
#include "l2warm.hpp"
#include "stream.hpp"

namespace fm {

constexpr int ATT_RANGES_MAX = 8;  // ranges per (branch, head) = arrivals per counter
constexpr int ATT_TREE_RANGES = 16;  // ranges per head of attention_tree_kernel (no counter)
constexpr int ATT_BLK = 32;        // keys per block
constexpr int KB_ROWS = 16;        // block rows (queries) per branch

// slot of key kk (0..31) inside a 32-key block of the value cache
template <typename T> __host__ __device__ __forceinline__ int vt_slot(int kk);
template <> __host__ __device__ __forceinline__ int vt_slot<bf16_t>(int kk) {
  return 8 * ((kk & 15) >> 2) + 4 * (kk >> 4) + (kk & 3);
}
template <> __host__ __device__ __forceinline__ int vt_slot<float>(int kk) { return kk; }

// Offset of key kk (0..31), dimension dd of a 32-key block, in elements from
// the block's start, for pieces of VE = 16 / sizeof(T) elements:
//   keys:   operand (tile kk / 16, piece dd / VE), lane (kk % 16) + 16 (piece % 4),
//           where the scores' MFMA step s takes pieces 4s .. 4s + 3 of each key;
//   values: slot q = vt_slot(kk), operand (step q / (4 VE), dims 16 (dd / 16) ..),
//           lane (dd % 16) + 16 ((q / VE) % 4).
// Operand o of a block is its 16-byte words 64 o .. 64 o + 63 (word = lane).
template <typename T> __host__ __device__ __forceinline__ int kt_off(int kk, int dd, int hd) {
  constexpr int VE = 16 / (int)sizeof(T);
  return (((kk >> 4) * (hd / VE) + dd / VE) * 16 + (kk & 15)) * VE + dd % VE;
}
template <typename T> __host__ __device__ __forceinline__ int vt_off(int kk, int dd, int hd) {
  constexpr int VE = 16 / (int)sizeof(T);
  const int q = vt_slot<T>(kk);
  return ((((q / (4 * VE)) * (hd / 16) + (dd >> 4)) * 4 + (q / VE) % 4) * 16 + (dd & 15)) * VE + q % VE;
}

struct AttnArgs {
  const void* q;       // [B*K][ldq] queries of the block rows
  int ldq;
  const void* kc;      // this DiT block's key cache   [nh][P/32][32 hd] (request 0)
  const void* vt;      // this DiT block's value cache [nh][P/32][32 hd] (request 0)
  size_t req_stride;   // elements between consecutive requests' caches
  int P;               // positions per head (multiple of 32)
  const int* ctx_len;  // device: context length of each request before this call
  int n_new[FM_MAX_REQ];  // rows this call appends for branch b's request
  int ctx_cap;         // cache capacity (C_max): visible rows never exceed it
  int scratch_blk;     // block index of the first block rows
  int scratch_step;    // 1: branches share request 0's cache (branch b at scratch_blk + b);
                       // 0: branch b is request b (its rows at scratch_blk of its own cache)
  int K, d, nh;
  int n_ranges;        // range slots per (branch, head) in the grid (at most ATT_RANGES_MAX,
                       // or ATT_TREE_RANGES for the tree kernel); the ranges in use are
                       // planned on the device from the visible context
  float* part_o;       // [B*nh][n_ranges][K][HD]
  float* part_ml;      // [B*nh][n_ranges][K][2]
  uint32_t* counters;  // [B*nh], COUNTER_STRIDE apart
  void* out;           // [B*K][d]
  float scale;         // 1/sqrt(hd)
  L2Warm warm;         // attention_kernel: workgroups from warm.first_wg on warm the L2s
};

// Context rows branch b sees: its request's length when the stream reaches the
// call (device-resident, so one captured graph stays valid as the context
// grows) plus the rows the call appends, clipped to the cache capacity.
__device__ __forceinline__ int visible_ctx(const AttnArgs& g, int b) {
  const int req = g.scratch_step ? 0 : b;
  return min(g.ctx_len[req] + g.n_new[b], g.ctx_cap);
}

// Key ranges of attention_kernel for n_blocks 32-key blocks of one (branch,
// head) over workgroups of nw waves: about one block a wave (all of a wave's
// loads in flight at once), but at most 6 ranges, since every further arrival
// at the merge costs more than a second block per wave (measured at 18 and 66
// blocks).  The same plan runs on the host (grid size, for the capacity) and
// on the device (the ranges in use, for the current length).
__host__ __device__ inline int attn_max_ranges(int n_blocks, int nw) {
  const int r = (n_blocks + nw - 1) / nw;
  return r < 6 ? (r < 1 ? 1 : r) : (6 < ATT_RANGES_MAX ? 6 : ATT_RANGES_MAX);
}
__host__ __device__ inline void attn_plan(int n_blocks, int nw, int& n_ranges, int& per_range) {
  const int r = attn_max_ranges(n_blocks, nw);
  per_range = (n_blocks + r - 1) / r;
  n_ranges = (n_blocks + per_range - 1) / per_range;
}
// the same for attention_tree_kernel over ctx_blocks context blocks (at least
// one range, which also serves the branches' own rows)
__host__ __device__ inline int tree_max_ranges(int ctx_blocks) {
  const int r = (ctx_blocks + 3) / 4;
  return r < 1 ? 1 : (r < ATT_TREE_RANGES ? r : ATT_TREE_RANGES);
}
__host__ __device__ inline void tree_plan(int ctx_blocks, int& n_ranges, int& per_range) {
  const int r = tree_max_ranges(ctx_blocks);
  per_range = (ctx_blocks + r - 1) / r;
  if (per_range < 1) per_range = 1;
  n_ranges = (ctx_blocks + per_range - 1) / per_range;
  if (n_ranges < 1) n_ranges = 1;
}

// One wave's 16 queries against one 32-key block (nv valid keys): transposed
// scores by MFMA, online softmax per query row (running max and sum, the
// accumulator rescaled), then O^T += V^T P^T with P kept in registers.
template <typename T, int HD>
struct AttnTile {
  typedef typename Vec<T>::type VT;
  static constexpr int VE = Vec<T>::N;
  static constexpr int QS = HD / (4 * VE);  // score MFMA steps over the head width
  static constexpr int OT = HD / 16;        // 16-dim output tiles
  static constexpr int PS = 32 / (4 * VE);  // P.V steps per block: bf16 1, float 2
  VT k[2][QS];                              // keys 16*tb + j, pieces 4s+grp
  VT v[PS][OT];                             // value dims 16t + j, slots ps*4*VE + grp*VE ..
};

// The operands of one 32-key block (keys at kb, values at vb, both in the
// caches' block order): word lane of operands tb * QS + s and ps * OT + t.
template <typename T, int HD>
__device__ __forceinline__ void attn_tile_load(AttnTile<T, HD>& t, const T* kb, const T* vb, int lane) {
  typedef AttnTile<T, HD> Tile;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int s = 0; s < Tile::QS; ++s) t.k[tb][s] = vload<T>(kb + (size_t)((tb * Tile::QS + s) * 64 + lane) * Tile::VE);
#pragma unroll
  for (int ps = 0; ps < Tile::PS; ++ps)
#pragma unroll
    for (int ot = 0; ot < Tile::OT; ++ot)
      t.v[ps][ot] = vload<T>(vb + (size_t)((ps * Tile::OT + ot) * 64 + lane) * Tile::VE);
}

template <typename T, int HD>
__device__ __forceinline__ void attn_block(const AttnTile<T, HD>& t, const typename Vec<T>::type (&qf)[AttnTile<T, HD>::QS],
                                           int nv, float scale, float& m_run, float& l_run,
                                           f32x4 (&o)[AttnTile<T, HD>::OT]) {
  constexpr int QS = AttnTile<T, HD>::QS, OT = AttnTile<T, HD>::OT, PS = AttnTile<T, HD>::PS;
  constexpr bool BF = sizeof(T) == 2;
  const int grp = (threadIdx.x & 63) >> 4;
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
      sc[tb][i] = kk < nv ? sc[tb][i] * scale : -INFINITY;
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
}

// WARM: the kind of the L2 warming its extra workgroups do (L2W_NONE: none)
template <typename T, int HD, int NW, int WARM>
__global__ __launch_bounds__(NW * 64) void attention_kernel(AttnArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int KB = 16;              // block rows (queries) per branch
  constexpr int VE = Vec<T>::N;
  constexpr int QS = HD / (4 * VE);   // score MFMA steps over the head width
  constexpr int OT = HD / 16;         // 16-dim output tiles
  constexpr int PS = 32 / (4 * VE);   // P.V steps per block: bf16 1, float 2
  __shared__ float so[NW][KB][HD + 4];
  __shared__ float sm[NW][KB], sl[NW][KB];
  __shared__ int flag;

  if constexpr (WARM != L2W_NONE) {
    if ((int)blockIdx.x >= g.warm.first_wg) {  // the next contractions' weights
      l2_warm<WARM>(g.warm, blockIdx.x, NW * 64);
      return;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int range = blockIdx.x % g.n_ranges;
  const int bh = blockIdx.x / g.n_ranges;
  const int head = bh % g.nh, b = bh / g.nh;
  const int C = visible_ctx(g, b);
  const int ctx_blocks = (C + ATT_BLK - 1) / ATT_BLK;
  const int nblk = ctx_blocks + 1;
  int n_ranges, per_range;
  attn_plan(nblk, NW, n_ranges, per_range);
  if (range >= n_ranges) return;  // a slot the current length does not use
  const int blo = range * per_range;
  const int bhi = min(nblk, blo + per_range);
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

  typedef AttnTile<T, HD> Tile;
  // physical block and number of valid keys of logical block bi
  auto phys = [&](int bi) { return bi < ctx_blocks ? bi : g.scratch_blk + g.scratch_step * b; };
  auto nvalid = [&](int bi) { return bi < ctx_blocks ? min(ATT_BLK, C - ATT_BLK * bi) : KB; };
  auto load = [&](Tile& t, int bi) {
    const size_t off = (size_t)phys(bi) * ATT_BLK * HD;
    attn_tile_load<T, HD>(t, kbase + off, vbase + off, lane);
  };

  float m_run = -INFINITY, l_run = 0.f;  // of query row j (same in all four groups)
  f32x4 o[OT];                           // o[t][i] = O[row j][16t + 4grp + i]
#pragma unroll
  for (int t = 0; t < OT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // blocks blo + wave, +NW, ... with the next block's loads in flight
  Tile t0, t1;
  int bi = blo + wave;
  if (bi < bhi) load(t0, bi);
  for (; bi < bhi; bi += 2 * NW) {
    if (bi + NW < bhi) load(t1, bi + NW);
    attn_block<T, HD>(t0, qf, nvalid(bi), g.scale, m_run, l_run, o);
    if (bi + NW < bhi) {
      if (bi + 2 * NW < bhi) load(t0, bi + 2 * NW);
      attn_block<T, HD>(t1, qf, nvalid(bi + NW), g.scale, m_run, l_run, o);
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
  // thread: row tid / TPR, columns c0 + c*TPR (c < CPT), so that each store
  // and load below covers TPR consecutive floats of a row
  constexpr int CPT = KB * HD / (NW * 64);  // output columns per thread
  constexpr int TPR = HD / CPT;             // threads per row
  const int row = tid / TPR, c0 = tid % TPR;
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
    for (int c = 0; c < CPT; ++c) acc[c] += wt * so[w][row][c0 + c * TPR];
  }
  T* out = reinterpret_cast<T*>(g.out) + (size_t)(b * g.K + row) * g.d + head * HD + c0;
  if (n_ranges == 1) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) out[c * TPR] = from_f32<T>(acc[c] / Lsum);
    return;
  }
  // ---- publish this range, the last range of the (branch, head) merges
  const size_t pbase = ((size_t)bh * g.n_ranges + range) * KB + row;
#pragma unroll
  for (int c = 0; c < CPT; ++c) st_coh(&g.part_o[pbase * HD + c0 + c * TPR], acc[c]);
  if (c0 == 0) {
    st_coh(&g.part_ml[pbase * 2 + 0], M);
    st_coh(&g.part_ml[pbase * 2 + 1], Lsum);
  }
  if (!arrive(&g.counters[bh * COUNTER_STRIDE], (uint32_t)n_ranges, &flag)) return;
  float mv[ATT_RANGES_MAX], lv[ATT_RANGES_MAX], ov[ATT_RANGES_MAX][CPT];
#pragma unroll
  for (int r = 0; r < ATT_RANGES_MAX; ++r) {
    const bool ok = r < n_ranges;
    const size_t pi = ((size_t)bh * g.n_ranges + (ok ? r : 0)) * KB + row;
    mv[r] = ok ? ld_coh(&g.part_ml[pi * 2]) : -INFINITY;
    lv[r] = ok ? ld_coh(&g.part_ml[pi * 2 + 1]) : 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) ov[r][c] = ok ? ld_coh(&g.part_o[pi * HD + c0 + c * TPR]) : 0.f;
  }
  float MM = -INFINITY;
#pragma unroll
  for (int r = 0; r < ATT_RANGES_MAX; ++r) MM = fmaxf(MM, mv[r]);
  float den = 0.f, num[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) num[c] = 0.f;
#pragma unroll
  for (int r = 0; r < ATT_RANGES_MAX; ++r) {
    const float wt = r < n_ranges ? expf(mv[r] - MM) : 0.f;
    den += wt * lv[r];
#pragma unroll
    for (int c = 0; c < CPT; ++c) num[c] += wt * ov[r][c];
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) out[c * TPR] = from_f32<T>(num[c] / den);
}


// Attention of the BR (2..4) branches of one tree over their shared context
// (bf16 storage).  A workgroup of 8 waves takes a (head, range of context
// blocks); wave w serves branch w / 2 (if below BR) and stream w % 2, and the
// two streams take the range's blocks alternately.  A block's keys and values (32 x HD each) are
// read from HBM once per workgroup: every wave loads a part of the next two
// blocks into registers while the current two are computed, writes it into
// the other half of a double-buffered LDS stage, and one barrier per step
// hands the stage over.  The stage keeps the caches' block order, in which
// each MFMA operand is 1 KB read in lane order (no bank conflicts).  Each
// branch's own 16 block rows (its scratch
// block) are read by the branch's stream-0 wave of the last range straight
// from HBM.  The waves of a branch merge through LDS; with several ranges the
// ranges' partial states go to memory and attention_merge_kernel combines
// them (spread over many workgroups: one workgroup merging all the
// branches of a head would be bound by the bytes one CU can take in).
// All branches see the same context length (that of request 0).
template <int HD, int BR>
__global__ __launch_bounds__(512) void attention_tree_kernel(AttnArgs g) {
  typedef bf16_t T;
  typedef AttnTile<T, HD> Tile;
  // 8 waves load every step; waves 2b and 2b + 1 compute branch b < BR (the
  // others only load), so one read of a key/value block serves every branch
  constexpr int NW = 8, WPB = 2;
  static_assert(BR >= 1 && BR * WPB <= NW, "at most four branches");
  constexpr int QS = Tile::QS, OT = Tile::OT, VE = Tile::VE;
  constexpr int KP = HD / VE;                          // 16-byte pieces per key row
  constexpr int PART_U4 = 32 * KP;                     // a block's keys (= its values) in uint4
  constexpr int BLOCK_U4 = 2 * PART_U4;
  constexpr int STEP_U4 = WPB * BLOCK_U4;              // blocks of one step (one per stream)
  constexpr int PER_LANE = STEP_U4 / (NW * 64);
  static_assert(PER_LANE * NW * 64 == STEP_U4, "a step's blocks split evenly over the lanes");
  constexpr int STAGE_BYTES = 2 * STEP_U4 * 16;        // two steps
  constexpr int MERGE_BYTES = NW * KB_ROWS * (HD + 4) * 4;
  constexpr int SMEM_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
  __shared__ __align__(16) unsigned char smem[SMEM_BYTES];
  __shared__ float sm[NW][KB_ROWS], sl[NW][KB_ROWS];
  uint4* stage = reinterpret_cast<uint4*>(smem);
  u32x4_t* stagev = reinterpret_cast<u32x4_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int range = blockIdx.x % g.n_ranges, head = blockIdx.x / g.n_ranges;
  const int b = wave / WPB, stream = wave % WPB;
  const bool computes = b < BR;
  const int C = visible_ctx(g, 0);
  const int ctx_blocks = (C + ATT_BLK - 1) / ATT_BLK;
  int n_ranges, per_range;
  tree_plan(ctx_blocks, n_ranges, per_range);
  if (range >= n_ranges) return;  // a slot the current length does not use
  const int blo = min(ctx_blocks, range * per_range);
  const int bhi = min(ctx_blocks, blo + per_range);
  const int n_steps = (bhi - blo + WPB - 1) / WPB;
  const T* kbase = reinterpret_cast<const T*>(g.kc) + (size_t)head * g.P * HD;
  const T* vbase = reinterpret_cast<const T*>(g.vt) + (size_t)head * (g.P / ATT_BLK) * HD * ATT_BLK;

  uint4 qf[QS];
  {
    const T* qrow = reinterpret_cast<const T*>(g.q) + (size_t)((computes ? b : 0) * g.K + j) * g.ldq + head * HD;
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[s] = vload<T>(qrow + (4 * s + grp) * VE);
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMA fragments of this wave's block of a step from the stage half (the
  // block's words in the caches' order: a wave reads 1 KB in lane order)
  auto frags = [&](Tile& t, int half) {
    const uint4* kb = stage + half * STEP_U4 + stream * BLOCK_U4 + lane;
    const uint4* vb = kb + PART_U4;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int s = 0; s < QS; ++s) t.k[tb][s] = kb[(tb * QS + s) * 64];
#pragma unroll
    for (int ot = 0; ot < OT; ++ot) t.v[0][ot] = vb[ot * 64];
  };

  // lane's share of a step: word e = u*512 + tid of the step's (stream,
  // keys/values, word), copied in the caches' order.  Blocks past the range
  // load block blo instead (never used).  Both addresses are formed and one
  // selected, so no branch surrounds the load.
  const uint4* src[PER_LANE];
  int src_blk[PER_LANE];
#pragma unroll
  for (int u = 0; u < PER_LANE; ++u) {
    const int e = u * NW * 64 + tid;
    const int sb = e / BLOCK_U4, w = e % BLOCK_U4;
    const uint4* ks = reinterpret_cast<const uint4*>(kbase) + w;
    const uint4* vs = reinterpret_cast<const uint4*>(vbase) + (w - PART_U4);
    src[u] = w < PART_U4 ? ks : vs;
    src_blk[u] = sb;
  }
  // uint4 offset of block bi from block 0: keys ATT_BLK*HD elements, values HD*ATT_BLK
  constexpr int BLK_STRIDE_U4 = ATT_BLK * HD / VE;
  // D steps of prefetch in flight in registers: step st's share goes to
  // pf[st % D], is written to LDS half st & 1 at the end of step st - 1, and
  // the barrier between steps orders LDS only, so the later steps' loads stay
  // in flight.  The steps are padded to a multiple of D; steps past the range
  // compute nothing and fetch block blo (clamped, never used), so no branch
  // surrounds a prefetch.
  constexpr int D = 2;
  if (n_steps > 0) {
    u32x4_t pf[D][PER_LANE];  // native vectors: kept in registers
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int u = 0; u < PER_LANE; ++u) {
        const int bi0 = blo + k * WPB + src_blk[u];
        pf[k][u] = *reinterpret_cast<const u32x4_t*>(src[u] + (size_t)(bi0 < bhi ? bi0 : blo) * BLK_STRIDE_U4);
      }
#pragma unroll
    for (int u = 0; u < PER_LANE; ++u) stagev[u * NW * 64 + tid] = pf[0][u];
    lds_barrier();
    for (int st0 = 0; st0 < n_steps; st0 += D) {
#pragma unroll
      for (int k = 0; k < D; ++k) {
        const int st = st0 + k;
        const int half = k & 1;  // D is even: st & 1 == k & 1
        // pf[k] (step st) is already in LDS: refill it with step st + D
#pragma unroll
        for (int u = 0; u < PER_LANE; ++u) {
          const int bi0 = blo + (st + D) * WPB + src_blk[u];
          pf[k][u] = *reinterpret_cast<const u32x4_t*>(src[u] + (size_t)(bi0 < bhi ? bi0 : blo) * BLK_STRIDE_U4);
        }
        const int bi = blo + st * WPB + stream;
        if (computes && bi < bhi) {
          Tile t;
          frags(t, half);
          attn_block<T, HD>(t, qf, min(ATT_BLK, C - ATT_BLK * bi), g.scale, m_run, l_run, o);
        }
#pragma unroll
        for (int u = 0; u < PER_LANE; ++u) stagev[(half ^ 1) * STEP_U4 + u * NW * 64 + tid] = pf[(k + 1) % D][u];
        lds_barrier();
      }
    }
  }
  // the branch's own block rows: the last range, the branch's stream-0 wave
  if (computes && range == n_ranges - 1 && stream == 0) {
    Tile t;
    const size_t off = (size_t)(g.scratch_blk + b) * ATT_BLK * HD;
    attn_tile_load<T, HD>(t, kbase + off, vbase + off, lane);
    attn_block<T, HD>(t, qf, KB_ROWS, g.scale, m_run, l_run, o);
  }

  // ---- merge each branch's waves (fixed order) through LDS (the stage is free)
  typedef float MergeRow[KB_ROWS][HD + 4];
  MergeRow* so = reinterpret_cast<MergeRow*>(smem);
#pragma unroll
  for (int ot = 0; ot < OT; ++ot)
    *reinterpret_cast<float4*>(&so[wave][j][16 * ot + 4 * grp]) = make_float4(o[ot][0], o[ot][1], o[ot][2], o[ot][3]);
  if (grp == 0) {
    sm[wave][j] = m_run;
    sl[wave][j] = l_run;
  }
  __syncthreads();
  // thread lt of branch mb's 128 handles column lt of all 16 rows, so every
  // row's stores and loads below are contiguous across the lanes
  constexpr int TPB = 128;  // threads per branch (= HD at HD 128); those of branches >= BR idle
  static_assert(TPB % HD == 0 || HD % TPB == 0, "columns split evenly");
  constexpr int CPT = HD / TPB > 0 ? HD / TPB : 1;  // columns per thread
  const int mb = tid / TPB, lt = tid % TPB, w0 = mb * WPB;
  const int bh = mb * g.nh + head;
  const bool col_ok = lt < HD && mb < BR;  // HD < TPB: the surplus threads idle
  float acc[KB_ROWS][CPT], Mr[KB_ROWS], Lr[KB_ROWS];
#pragma unroll
  for (int row = 0; row < KB_ROWS; ++row) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPB; ++w) M = fmaxf(M, sm[min(w0 + w, NW - 1)][row]);
    float Lsum = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[row][c] = 0.f;
#pragma unroll
    for (int w = 0; w < WPB; ++w) {
      const int ww = min(w0 + w, NW - 1);
      const float wt = M == -INFINITY ? 0.f : expf(sm[ww][row] - M);
      Lsum += wt * sl[ww][row];
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[row][c] += wt * (col_ok ? so[ww][row][c * TPB + lt] : 0.f);
    }
    Mr[row] = M;
    Lr[row] = Lsum;
  }
  if (n_ranges == 1) {
    if (col_ok) {
#pragma unroll
      for (int row = 0; row < KB_ROWS; ++row) {
        T* out = reinterpret_cast<T*>(g.out) + (size_t)(mb * g.K + row) * g.d + head * HD;
#pragma unroll
        for (int c = 0; c < CPT; ++c) out[c * TPB + lt] = from_f32<T>(acc[row][c] / Lr[row]);
      }
    }
    return;
  }
  // ---- publish this range (row by row, contiguous); attention_merge_kernel,
  // launched next, combines the ranges
  if (col_ok) {
#pragma unroll
    for (int row = 0; row < KB_ROWS; ++row) {
      const size_t pr = ((size_t)bh * g.n_ranges + range) * KB_ROWS + row;
#pragma unroll
      for (int c = 0; c < CPT; ++c) g.part_o[pr * HD + c * TPB + lt] = acc[row][c];
    }
  }
  if (lt < KB_ROWS && mb < BR) {
    const size_t pr = ((size_t)bh * g.n_ranges + range) * KB_ROWS + lt;
    float m = 0.f, l = 0.f;
#pragma unroll
    for (int row = 0; row < KB_ROWS; ++row) {
      m = row == lt ? Mr[row] : m;
      l = row == lt ? Lr[row] : l;
    }
    g.part_ml[pr * 2 + 0] = m;
    g.part_ml[pr * 2 + 1] = l;
  }
}

// Combination of the ranges' (max, sum, output) of attention_tree_kernel for
// B branches x nh heads x 16 rows: workgroup (branch, head, 2-row group),
// thread = column; ranges in order, so results never depend on scheduling.
template <typename T, int HD>
__global__ __launch_bounds__(HD) void attention_merge_kernel(AttnArgs g) {
  constexpr int RG = 2;  // rows per workgroup
  static_assert(HD >= RG * ATT_TREE_RANGES, "one (row, range) pair per thread");
  __shared__ float2 sml[RG][ATT_TREE_RANGES];
  const int col = threadIdx.x;
  const int bh = blockIdx.x / (KB_ROWS / RG), row0 = (blockIdx.x % (KB_ROWS / RG)) * RG;
  const int b = bh / g.nh, head = bh % g.nh;
  int n_ranges, per_range;
  tree_plan((visible_ctx(g, 0) + ATT_BLK - 1) / ATT_BLK, n_ranges, per_range);
  if (n_ranges == 1) return;  // attention_tree_kernel wrote the output itself
  // the rows' (max, sum) of every range: one pair per thread, through LDS
  {
    const int i = col / ATT_TREE_RANGES, r = col % ATT_TREE_RANGES;
    if (i < RG) {
      const size_t pr = ((size_t)bh * g.n_ranges + (r < n_ranges ? r : 0)) * KB_ROWS + row0 + i;
      const float2 ml = reinterpret_cast<const float2*>(g.part_ml)[pr];
      // a range past n_ranges (or one without blocks, M = -inf) gets weight 0
      sml[i][r] = make_float2(r < n_ranges ? ml.x : -INFINITY, ml.y);
    }
  }
  float ov[RG][ATT_TREE_RANGES];
#pragma unroll
  for (int i = 0; i < RG; ++i)
#pragma unroll
    for (int r = 0; r < ATT_TREE_RANGES; ++r) {
      const size_t pr = ((size_t)bh * g.n_ranges + (r < n_ranges ? r : 0)) * KB_ROWS + row0 + i;
      ov[i][r] = g.part_o[pr * HD + col];
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    float MM = -INFINITY;
#pragma unroll
    for (int r = 0; r < ATT_TREE_RANGES; ++r) MM = fmaxf(MM, sml[i][r].x);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int r = 0; r < ATT_TREE_RANGES; ++r) {
      const float2 ml = sml[i][r];
      const float wt = ml.x == -INFINITY ? 0.f : expf(ml.x - MM);
      den += wt * ml.y;
      num += wt * ov[i][r];
    }
    reinterpret_cast<T*>(g.out)[(size_t)(b * g.K + row0 + i) * g.d + head * HD + col] = from_f32<T>(num / den);
  }
}

}  // namespace fm
