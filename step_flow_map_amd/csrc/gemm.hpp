// Skinny "activation x weight^T" contraction for the drafter's linear layers.
//
//   out[m][n] = sum_k A[m][k] * W[n][k]        (W row-major [N][K], k contiguous)
//
// M is small (block rows of every branch, plus the context rows appended in the
// step: at most 80), so the layer is bound by streaming W once from HBM.
// A workgroup owns one 16-row tile of W and one k range of a deterministic
// split-K; its waves take interleaved 8 KB chunks of that range, stream them
// through their LDS tile into MFMA operands (stream.hpp) with the next chunk
// already in flight, and reduce across waves through LDS in wave order.  With
// one split the workgroup runs the epilogue; otherwise it publishes a float32
// partial with coherent stores and the last of the (few) splits of the tile
// sums them in split order and runs the epilogue.  Results never depend on
// scheduling.
#pragma once
#include "common.hpp"
#include "stream.hpp"
#include "lnfuse.hpp"
#include "attention.hpp"
#include "norm.hpp"

namespace fm {

enum EpiKind {
  EPI_F32 = 0,    // out_f32[m][n] = v + bias[n]
  EPI_ACT = 1,    // out_act[m][n] = T(v + bias[n])
  EPI_GELU = 2,   // out_act[m][n] = T(gelu(v + bias[n]))
  EPI_RESID = 3,  // out_f32[m][n] += gate[n] * (v + bias[n])   (residual stream);
                  // with out_act, also the new value in the storage type there
  EPI_QKV = 4     // block rows: queries to out_act, keys/values to the branch's
                  // scratch block of the cache; context rows: keys/values to the cache
};

struct EpiParams {
  const void* bias;     // [N] storage type, or null
  float* out_f32;       // EPI_F32 / EPI_RESID
  int ld_f32;
  void* out_act;        // EPI_ACT / EPI_GELU / EPI_QKV; EPI_RESID: copy of the residual, or null
  int ld_act;
  const float* gate;    // EPI_RESID, [N]
  // EPI_QKV (cache layout: attention.hpp)
  int rows_block;       // rows < rows_block are block rows (branch m / 16), the rest context rows
  void* kcache;         // this DiT block's key cache   [nh][P/32][32 hd] of request 0
  void* vcache;         // this DiT block's value cache [nh][P/32][32 hd] of request 0
  size_t req_stride;    // elements from one request's key (value) cache to the next one's
  int P, hd, d;         // positions per head, head width, model width
  int scratch_pos0;     // position of the first block row
  int scratch_step;     // 32: branches share request 0's cache, branch b's rows at +32b;
                        // 0: branch b is request b, its rows in its own cache
  int n_req;            // context row c belongs to request r with ctx_first[r] <= c <
  int ctx_first[FM_MAX_REQ + 1];  // ctx_first[r + 1], and goes to position
                        // ctx_len[r] + ctx_off + c - ctx_first[r] of that request's cache
  const int* ctx_len;   // device: each request's context length before the call
  int ctx_off;          // rows the call has already appended ahead of these
  int ctx_cap;          // positions >= ctx_cap are not written (the cache is full)
  int col_offset;       // logical qkv column of n = 0 (d for a K/V-only call)
  // EPI_RESID through gemm_reduce_ln_kernel: the LayerNorm + modulation of the
  // updated rows, written in the storage type (the next contraction's operand)
  const float* ln_shift;
  const float* ln_scale;
  void* ln_out;
  int ln_ldo;
  // EPI_RESID / EPI_F32: per-16-column statistics (mean, M2) of the stored rows
  // for a LayerNorm applied later, at ln_part[m * ln_part_ld + n / 16]
  float2* ln_part;
  int ln_part_ld;
};

constexpr int GEMM_SPLIT_MAX = 8;  // k splits per tile (= arrivals per counter)

struct GemmArgs {
  const void* A;
  int lda, M;
  const void* W;
  int ldw, N, K;
  int S;          // k splits (<= 8: arrivals per counter)
  int k_split;    // k elements per split (multiple of the chunk)
  float* partial; // [S][M][N] float32 when S > 1
  uint32_t* counters;  // one per 16-row tile, COUNTER_STRIDE apart; zero on entry and exit
};

// returns the stored float32 value for EPI_F32 and EPI_RESID (0 otherwise)
template <typename T, int EPI>
__device__ __forceinline__ float epilogue(const EpiParams& e, int m, int n, float v) {
  if (e.bias) v += to_f32<T>(reinterpret_cast<const T*>(e.bias)[n]);
  if (EPI == EPI_F32) {
    e.out_f32[(size_t)m * e.ld_f32 + n] = v;
    return v;
  } else if (EPI == EPI_ACT) {
    reinterpret_cast<T*>(e.out_act)[(size_t)m * e.ld_act + n] = from_f32<T>(v);
  } else if (EPI == EPI_GELU) {
    reinterpret_cast<T*>(e.out_act)[(size_t)m * e.ld_act + n] = from_f32<T>(gelu_tanh(v));
  } else if (EPI == EPI_RESID) {
    float* p = e.out_f32 + (size_t)m * e.ld_f32 + n;
    const float r = *p + e.gate[n] * v;
    *p = r;
    if (e.out_act) reinterpret_cast<T*>(e.out_act)[(size_t)m * e.ld_act + n] = from_f32<T>(r);
    return r;
  } else {  // EPI_QKV
    const int nn = n + e.col_offset;
    int pos, req;
    if (m < e.rows_block) {
      if (nn < e.d) {
        reinterpret_cast<T*>(e.out_act)[(size_t)m * e.ld_act + nn] = from_f32<T>(v);
        return 0.f;
      }
      pos = e.scratch_pos0 + e.scratch_step * (m >> 4) + (m & 15);
      req = e.scratch_step ? 0 : (m >> 4);
    } else {
      if (nn < e.d) return 0.f;  // queries of context rows are not needed
      const int c = m - e.rows_block;
      req = 0;
#pragma unroll
      for (int r = 1; r < FM_MAX_REQ; ++r) req += (r < e.n_req && c >= e.ctx_first[r]) ? 1 : 0;
      pos = e.ctx_len[req] + e.ctx_off + c - e.ctx_first[req];
      if (pos >= e.ctx_cap) return 0.f;  // past the capacity: nothing is written
    }
    const int which = nn >= 2 * e.d;  // 0: key, 1: value
    const int col = nn - (1 + which) * e.d;
    const int head = col / e.hd, c = col - head * e.hd;
    // the position's 32-key block, then the element's place in it
    const size_t blk0 = (size_t)req * e.req_stride + ((size_t)head * e.P + (pos & ~31)) * e.hd;
    if (!which)
      reinterpret_cast<T*>(e.kcache)[blk0 + kt_off<T>(pos & 31, c, e.hd)] = from_f32<T>(v);
    else
      reinterpret_cast<T*>(e.vcache)[blk0 + vt_off<T>(pos & 31, c, e.hd)] = from_f32<T>(v);
  }
  return 0.f;
}

// The epilogue of output (m, n) when ok, then (EPI_F32 or EPI_RESID with
// ln_part) the statistics of the stored row over the tile's 16 columns, which
// the 16 lanes of a DPP row hold (row m, columns 16 (n / 16) ..): every lane
// calls it.
template <typename T, int EPI>
__device__ __forceinline__ void epilogue_out(const EpiParams& e, int m, int n, float v, bool ok) {
  float r = 0.f;
  if (ok) r = epilogue<T, EPI>(e, m, n, v);
  if constexpr (EPI == EPI_RESID || EPI == EPI_F32) {
    if (e.ln_part) row16_stats(r, ok, e.ln_part + (size_t)(ok ? m : 0) * e.ln_part_ld + (n >> 4));
  }
}

template <typename T, int MT, int NW, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(GemmArgs g, EpiParams e) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = ChunkT<T>::VE;
  constexpr int KC = ChunkT<T>::KC;
  constexpr int ELEMS = MT * 256;  // outputs of the tile: MT*16 rows x 16 columns
  constexpr int RED_U4 = (NW * ELEMS + 3) / 4;
  constexpr int TILE_U4 = NW * 512;
  __shared__ uint4 smem[TILE_U4 > RED_U4 ? TILE_U4 : RED_U4];
  __shared__ int flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int tile = blockIdx.x / g.S, s = blockIdx.x % g.S;
  const int n0 = tile * 16;
  const int k_begin = s * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);
  const int nch = k_end > k_begin ? (k_end - k_begin + KC - 1) / KC : 0;
  const T* A = reinterpret_cast<const T*>(g.A);
  const T* W = reinterpret_cast<const T*>(g.W);
  uint4* wt = smem + wave * 512;

  const T* arow[MT];
  bool aok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + j;
    aok[mt] = m < g.M;
    arow[mt] = A + (size_t)(aok[mt] ? m : 0) * g.lda;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // With one row tile a chunk's weights and the matching A rows are loaded
  // together (both coalesced), one chunk ahead of the MFMAs, so neither
  // latency is exposed; the A rows reach their fragment layout through the
  // wave's tile before the weights do.  More row tiles load A fragments at
  // use, which keeps the register count low enough for two workgroups per CU.
  constexpr bool PRE_A = MT == 1;
  constexpr int AF = PRE_A ? 8 : 1;
  // A values outside [k_begin, k_end) or rows >= M are zeroed at use (this also
  // neutralises the clamped weight columns beyond the k range)
  auto a_ok = [&](int mt, int k0, int st) { return (k0 + (4 * st + grp) * VE) < k_end && aok[mt]; };
  auto a_load = [&](int mt, int k0, int st) -> VT {
    const int k = k0 + (4 * st + grp) * VE;
    return vload<T>(arow[mt] + (a_ok(mt, k0, st) ? k : 0));
  };
  auto load = [&](uint4 (&r)[8], uint4 (&ra)[AF], int c) {
    const int k0 = k_begin + c * KC;
    if constexpr (PRE_A) chunk_load_act<T>(ra, A, g.lda, 0, g.M, k0, k_end);
    chunk_load<T>(r, W, g.ldw, n0, g.N, k0, k_end);
  };
  auto process = [&](const uint4 (&r)[8], const uint4 (&ra)[AF], int c) {
    const int k0 = k_begin + c * KC;
    VT af[PRE_A ? 8 : 1];
    if constexpr (PRE_A) {
      chunk_to_lds(ra, wt);
      wave_lds_sync();
#pragma unroll
      for (int st = 0; st < 8; ++st) af[st] = as_vec<T>(chunk_frag(wt, st));
      wave_lds_sync();
    }
    chunk_to_lds(r, wt);
    wave_lds_sync();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const VT b = as_vec<T>(chunk_frag(wt, st));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const VT av = PRE_A ? af[PRE_A ? st : 0] : a_load(mt, k0, st);
        mma(acc[mt], a_ok(mt, k0, st) ? av : vzero<VT>(), b);
      }
    }
    wave_lds_sync();
  };

  uint4 r0[8], r1[8];
  uint4 a0[AF], a1[AF];
  if (wave < nch) load(r0, a0, wave);
  for (int c = wave; c < nch; c += 2 * NW) {
    if (c + NW < nch) load(r1, a1, c + NW);
    process(r0, a0, c);
    if (c + NW < nch) {
      if (c + 2 * NW < nch) load(r0, a0, c + 2 * NW);
      process(r1, a1, c + NW);
    }
  }

  // ---- fixed-order reduction over the waves of the workgroup
  __syncthreads();  // every wave is done with its LDS tile
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave * ELEMS + (mt * 4 + i) * 64 + lane] = acc[mt][i];
  __syncthreads();
  constexpr int PER_THREAD = (ELEMS + NW * 64 - 1) / (NW * 64);
  float val[PER_THREAD];
  int em[PER_THREAD], en[PER_THREAD];
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    const int el = threadIdx.x + r * NW * 64;
    const int ln = el & 63, q = el >> 6;  // q = mt*4 + i
    const int i = q & 3, mt = q >> 2;
    em[r] = el < ELEMS ? mt * 16 + 4 * (ln >> 4) + i : g.M;
    en[r] = n0 + (ln & 15);
    float v = 0.f;
    if (el < ELEMS) {
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w * ELEMS + el];
    }
    val[r] = v;
  }

  if (g.S == 1) {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) epilogue_out<T, EPI>(e, em[r], en[r], val[r], em[r] < g.M && en[r] < g.N);
    return;
  }
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r)
    if (em[r] < g.M && en[r] < g.N) st_coh(&g.partial[((size_t)s * g.M + em[r]) * g.N + en[r]], val[r]);
  if (!arrive(&g.counters[tile * COUNTER_STRIDE], (uint32_t)g.S, &flag)) return;
  // all coherent loads in flight together, then summed in split order
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    const bool ok = em[r] < g.M && en[r] < g.N;
    float pv[GEMM_SPLIT_MAX];
#pragma unroll
    for (int ss = 0; ss < GEMM_SPLIT_MAX; ++ss)
      pv[ss] = (ok && ss < g.S) ? ld_coh(&g.partial[((size_t)ss * g.M + em[r]) * g.N + en[r]]) : 0.f;
    float v = 0.f;
#pragma unroll
    for (int ss = 0; ss < GEMM_SPLIT_MAX; ++ss) v += pv[ss];
    epilogue_out<T, EPI>(e, em[r], en[r], v, ok);
  }
}

// Tile-group variant for wide layers (many 16-row tiles, a k range of at most
// NW chunks): a workgroup owns TT adjacent tiles and wave w takes chunks w,
// w+NW, ...  For a chunk it loads the A operand first (it is consumed first,
// and loads complete in issue order), then the TT weight chunks, and applies
// the A fragments to all TT tiles, so A is fetched once per TT tiles.  PIPE
// (one row tile, several chunks a wave): a wave's next chunk is in flight
// while it consumes the current one.  The waves then reduce through LDS in
// wave order and run the epilogue.
//
// With LN (the k range is at most NW = 8 chunks) row tile 0 is the LayerNorm
// of the 16 residual rows (ln_issue / ln_finish): each wave loads its chunk of
// the rows coalesced (every lane holds 4 consecutive columns of one row) and
// the row statistics from the producer's per-16-column partials, all before
// its weights, and normalises into MFMA fragments while the weights stream.
template <typename T, int MT, int NW, int TT, int EPI, bool LN, bool PIPE = false>
__global__ __launch_bounds__(NW * 64) void gemm_tg_kernel(GemmArgs g, EpiParams e, LnArgs ln) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = ChunkT<T>::VE;
  constexpr int KC = ChunkT<T>::KC;
  constexpr int ELEMS = TT * MT * 256;  // outputs: TT tiles x MT*16 rows x 16 columns
  constexpr int RED_U4 = NW * ELEMS / 4;
  constexpr int TILE_U4 = NW * 512;
  __shared__ uint4 smem[TILE_U4 > RED_U4 ? TILE_U4 : RED_U4];
  __shared__ float sstat[16][2];                           // LN: per row mean, 1 / std
  // LN with context rows: their chunk waits in LDS (a wave-private tile in
  // the weights' layout) rather than as fragments in registers
  static_assert(!LN || MT <= 2, "fused LayerNorm supports at most 16 further rows");
  static_assert(!LN || NW == 8, "fused LayerNorm: 32 threads per row of statistics");
  static_assert(!PIPE || (!LN && MT == 1), "two register sets of chunks fit one row tile only");
  constexpr bool CTX_LDS = LN && MT == 2;
  __shared__ uint4 sctx[CTX_LDS ? NW : 1][CTX_LDS ? 512 : 1];
  __shared__ uint4 sa[PIPE ? NW : 1][PIPE ? 512 : 1];  // PIPE: the A chunk of each wave

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int group = blockIdx.x / g.S, split = blockIdx.x % g.S;
  const int n0 = group * 16 * TT;
  const int k_begin = split * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);
  const int nch = k_end > k_begin ? (k_end - k_begin + KC - 1) / KC : 0;
  const T* A = reinterpret_cast<const T*>(g.A);
  const T* W = reinterpret_cast<const T*>(g.W);
  uint4* wt = smem + wave * 512;

  // rows of A: with LN, row tile 0 is computed and tiles 1.. read A rows 0..
  constexpr int MT0 = LN ? 1 : 0;
  bool aok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) aok[mt] = mt * 16 + j < g.M;
  f32x4 acc[TT][MT];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (LN) {
    const int c = wave;
    const bool has = c < nch;  // every wave takes part in the statistics
    const int k0 = k_begin + c * KC;
    bool kok[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) kok[st] = has && k0 + (4 * st + grp) * VE < k_end;
    // ---- issue: residual rows, modulation, A rows, weights.  Addresses are
    // clamped in range and nothing here is conditional, so no load waits for
    // another one before the statistics need the residual rows.
    LnChunk<T> lc;
    ln_issue<T>(lc, ln, g.K, k0, k_end, has);
    // A rows of the chunk in the weights' pattern; their fragments come back
    // through LDS below
    uint4 ra[MT][8];
#pragma unroll
    for (int mt = MT0; mt < MT; ++mt) chunk_load_act<T>(ra[mt], A, g.lda, (mt - MT0) * 16, g.M - 16 * MT0, k0, k_end);
    VT af[MT][8];
    uint4 r[TT][8];
#pragma unroll
    for (int t = 0; t < TT; ++t) chunk_load<T>(r[t], W, g.ldw, n0 + 16 * t, g.N, k0, k_end);
    {
      // every load above is issued before the statistics consume the first one
      __builtin_amdgcn_sched_barrier(0);
      ln_finish<T>(lc, ln, g.K, wt, sstat, af[0]);
      // the context rows (issued after the residual rows) wait in their tile
      if constexpr (CTX_LDS) chunk_to_lds(ra[1], sctx[wave]);
    }
#pragma unroll
    for (int t = 0; t < TT && has; ++t) {
      chunk_to_lds(r[t], wt);
      wave_lds_sync();
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const VT b = as_vec<T>(chunk_frag(wt, st));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const VT a = (CTX_LDS && mt == 1) ? as_vec<T>(chunk_frag(sctx[wave], st)) : af[mt][st];
          mma(acc[t][mt], (kok[st] && aok[mt]) ? a : vzero<VT>(), b);
        }
      }
      wave_lds_sync();
    }
  } else if constexpr (!PIPE) {
    for (int c = wave; c < nch; c += NW) {
      const int k0 = k_begin + c * KC;
      bool kok[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) kok[st] = k0 + (4 * st + grp) * VE < k_end;
      // A rows of the chunk in the weights' pattern; their fragments come
      // back through LDS
      uint4 ra[MT][8];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) chunk_load_act<T>(ra[mt], A, g.lda, mt * 16, g.M, k0, k_end);
      VT af[MT][8];
      uint4 r[TT][8];
#pragma unroll
      for (int t = 0; t < TT; ++t) chunk_load<T>(r[t], W, g.ldw, n0 + 16 * t, g.N, k0, k_end);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        chunk_to_lds(ra[mt], wt);
        wave_lds_sync();
#pragma unroll
        for (int st = 0; st < 8; ++st) af[mt][st] = as_vec<T>(chunk_frag(wt, st));
        wave_lds_sync();
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        chunk_to_lds(r[t], wt);
        wave_lds_sync();
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const VT b = as_vec<T>(chunk_frag(wt, st));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) mma(acc[t][mt], (kok[st] && aok[mt]) ? af[mt][st] : vzero<VT>(), b);
        }
        wave_lds_sync();
      }
    }
  } else {
    // One row tile, several chunks a wave: two register sets in turn, the
    // next chunk's loads in flight while the current chunk is consumed (a
    // wave without a next chunk issues placeholder loads of one line).  The A
    // chunk waits in a second wave-private tile, read at each MFMA step.
    uint4* at = sa[wave];
    auto issue = [&](int c, uint4 (&xa)[8], uint4 (&xr)[TT][8]) {
      const bool live = c < nch;
      const int k0 = k_begin + c * KC;
      chunk_load_act<T>(xa, A, g.lda, 0, g.M, k0, k_end, live);
#pragma unroll
      for (int t = 0; t < TT; ++t) chunk_load<T>(xr[t], W, g.ldw, n0 + 16 * t, g.N, k0, k_end, live);
    };
    auto consume = [&](int c, const uint4 (&xa)[8], const uint4 (&xr)[TT][8]) {
      const int k0 = k_begin + c * KC;
      bool kok[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) kok[st] = aok[0] && k0 + (4 * st + grp) * VE < k_end;
      chunk_to_lds(xa, at);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        chunk_to_lds(xr[t], wt);
        wave_lds_sync();
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const VT a = as_vec<T>(chunk_frag(at, st));
          mma(acc[t][0], kok[st] ? a : vzero<VT>(), as_vec<T>(chunk_frag(wt, st)));
        }
        wave_lds_sync();
      }
    };
    uint4 a0[8], r0[TT][8], a1[8], r1[TT][8];
    issue(wave, a0, r0);
    for (int c = wave; c < nch; c += 2 * NW) {
      issue(c + NW, a1, r1);
      consume(c, a0, r0);
      if (c + NW >= nch) break;
      issue(c + 2 * NW, a0, r0);
      consume(c + NW, a1, r1);
    }
  }

  // ---- fixed-order reduction over the waves
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * ELEMS + ((t * MT + mt) * 4 + i) * 64 + lane] = acc[t][mt][i];
  __syncthreads();
  constexpr int PER_THREAD = (ELEMS + NW * 64 - 1) / (NW * 64);
  float val[PER_THREAD];
  int em[PER_THREAD], en[PER_THREAD];
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    const int el = tid + r * NW * 64;
    const int ln_ = el & 63, q = el >> 6;  // q = (t*MT + mt)*4 + i
    const int i = q & 3, tm = q >> 2;
    const int mt = tm % MT, t = tm / MT;
    em[r] = el < ELEMS ? mt * 16 + 4 * (ln_ >> 4) + i : g.M;
    en[r] = n0 + 16 * t + (ln_ & 15);
    float v = 0.f;
    if (el < ELEMS) {
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w * ELEMS + el];
    }
    val[r] = v;
  }
  if (g.S == 1) {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) epilogue_out<T, EPI>(e, em[r], en[r], val[r], em[r] < g.M && en[r] < g.N);
    return;
  }
  // ---- split k: publish, the last split of the tile group sums in split order
  __shared__ int flag;
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r)
    if (em[r] < g.M && en[r] < g.N) st_coh(&g.partial[((size_t)split * g.M + em[r]) * g.N + en[r]], val[r]);
  if (!arrive(&g.counters[group * COUNTER_STRIDE], (uint32_t)g.S, &flag)) return;
#pragma unroll
  for (int r = 0; r < PER_THREAD; ++r) {
    const bool ok = em[r] < g.M && en[r] < g.N;
    float pv[GEMM_SPLIT_MAX];
#pragma unroll
    for (int ss = 0; ss < GEMM_SPLIT_MAX; ++ss)
      pv[ss] = (ok && ss < g.S) ? ld_coh(&g.partial[((size_t)ss * g.M + em[r]) * g.N + en[r]]) : 0.f;
    float v = 0.f;
#pragma unroll
    for (int ss = 0; ss < GEMM_SPLIT_MAX; ++ss) v += pv[ss];
    epilogue_out<T, EPI>(e, em[r], en[r], v, ok);
  }
}


// Many rows (48..80) against a wide weight: the rows' A slice would dominate
// what every 16-column tile reads, so a workgroup keeps it in LDS.  A
// workgroup owns 8 column tiles and a 512-wide k slice: wave w issues tile w's
// two weight chunks, the workgroup copies the slice's A rows into LDS once
// (direct global-to-LDS loads, one row's 1 KB per copy), and every wave then
// reads its A fragments from LDS.  Each k slice writes its float32 partial with
// plain stores; gemm_reduce_kernel, launched next, sums the slices in order
// and runs the epilogue.  Rows >= M read row 0 (valid memory) and produce
// outputs that are never stored.
constexpr int AS_TILES = 8;    // column tiles per workgroup (one a wave)
template <typename T, int MT, int KS>  // KS: k per workgroup, 256 or 512 (one or two bf16 chunks)
__global__ __launch_bounds__(512) void gemm_as_kernel(GemmArgs g) {
  typedef typename Vec<T>::type VT;
  constexpr int VE = ChunkT<T>::VE;
  constexpr int KC = ChunkT<T>::KC;
  constexpr int NCH = KS / KC;                     // chunks per slice
  constexpr int PIECES = KS / VE;                  // 16-byte pieces of a row's slice
  static_assert(PIECES == 32 || PIECES == 64, "one row's slice is one copy of up to 64 lanes");
  __shared__ uint4 sA[MT * 16 * PIECES];
  __shared__ uint4 wtile[AS_TILES * 512];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int group = blockIdx.x / g.S, s = blockIdx.x % g.S;
  const int n0 = group * 16 * AS_TILES + 16 * wave;
  const int k0 = s * KS;
  const T* A = reinterpret_cast<const T*>(g.A);
  const T* W = reinterpret_cast<const T*>(g.W);
  // this wave's tile's weight chunks first (the long HBM stream)
  uint4 r[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) chunk_load<T>(r[c], W, g.ldw, n0, g.N, k0 + c * KC, g.K);
  // row rr of the slice: one copy of its KS elements, lane i fetching piece
  // i ^ (rr & 15) into slot rr*PIECES + i, so that the fragment reads below (16
  // rows, one piece group each) hit 16 distinct banks.  With 32 pieces a row
  // the upper half-wave copies row rr + 1.
  constexpr int ROWS_PER_COPY = 64 / PIECES;
#pragma unroll
  for (int i = 0; i < MT * 16 / (8 * ROWS_PER_COPY); ++i) {
    const int rr = (i * 8 + wave) * ROWS_PER_COPY + lane / PIECES;
    const int pc = lane % PIECES;
    const T* src = A + (size_t)(rr < g.M ? rr : 0) * g.lda + k0 + (pc ^ (rr & 15)) * VE;
    lds_dma16(src, sA + (rr - lane / PIECES) * PIECES);
  }
  __syncthreads();  // the copies have landed (the compiler waits for all loads first)
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4* wt = wtile + wave * 512;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    chunk_to_lds(r[c], wt);
    wave_lds_sync();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const VT b = as_vec<T>(chunk_frag(wt, st));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        mma(acc[mt], as_vec<T>(sA[(mt * 16 + j) * PIECES + ((c * 32 + 4 * st + grp) ^ j)]), b);
    }
    wave_lds_sync();
  }
  // D element (row 4grp + i, column j) of each row tile
  const int n = n0 + j;
  if (n < g.N) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * grp + i;
        if (m < g.M) g.partial[((size_t)s * g.M + m) * g.N + n] = acc[mt][i];
      }
  }
}

// out[m][n] = epilogue(sum over the S k slices of partial[s][m][n], in order).
// A thread takes VW adjacent outputs (N % VW == 0) with every slice's values in
// flight at once (S <= AS_SMAX).  The QKV epilogue scatters into the caches, so
// it runs one output per thread (more threads in flight).
constexpr int AS_SMAX = 16;
template <typename T, int EPI, int VW>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs g, EpiParams e) {
  static_assert(VW == 1 || VW == 4, "one or four outputs per thread");
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;  // VW-element index of [M][N]
  const size_t mn = (size_t)g.M * g.N;
  if (q * VW >= mn) return;
  float v[VW];
#pragma unroll
  for (int c = 0; c < VW; ++c) v[c] = 0.f;
  if constexpr (VW == 4) {
    float4 pv[AS_SMAX];
#pragma unroll
    for (int s = 0; s < AS_SMAX; ++s)
      pv[s] = s < g.S ? reinterpret_cast<const float4*>(g.partial + s * mn)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < AS_SMAX; ++s) {
      v[0] += pv[s].x;
      v[1] += pv[s].y;
      v[2] += pv[s].z;
      v[3] += pv[s].w;
    }
  } else {
    float pv[AS_SMAX];
#pragma unroll
    for (int s = 0; s < AS_SMAX; ++s) pv[s] = s < g.S ? g.partial[s * mn + q] : 0.f;
#pragma unroll
    for (int s = 0; s < AS_SMAX; ++s) v[0] += pv[s];
  }
  const int m = (int)(q * VW / g.N), n = (int)(q * VW % g.N);
#pragma unroll
  for (int c = 0; c < VW; ++c) epilogue<T, EPI>(e, m, n + c, v[c]);
}


// EPI_RESID reduce fused with the LayerNorm that follows it: one workgroup of
// 1024 threads per row m sums the S k slices of its N = 1024 * PER columns (in
// order, all slices in flight), applies the gated residual update to h, and
// writes LN(h[m]) * (1 + ln_scale) + ln_shift in the storage type (two-pass
// mean and variance, as ln_mod_kernel).
template <typename T, int PER>
__global__ __launch_bounds__(1024) void gemm_reduce_ln_kernel(GemmArgs g, EpiParams e, float eps) {
  constexpr int NT = 1024;
  constexpr int SM = AS_SMAX;  // slices in flight (S <= SM)
  __shared__ float red[NT / 64];
  const int m = blockIdx.x, t = threadIdx.x;
  const size_t mn = (size_t)g.M * g.N;
  float pv[SM][PER];
#pragma unroll
  for (int s = 0; s < SM; ++s)
#pragma unroll
    for (int p = 0; p < PER; ++p)
      pv[s][p] = s < g.S ? g.partial[s * mn + (size_t)m * g.N + t + p * NT] : 0.f;
  float v[PER], sc[PER], sh[PER], sum = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int c = t + p * NT;
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < SM; ++s) a += pv[s][p];
    if (e.bias) a += to_f32<T>(reinterpret_cast<const T*>(e.bias)[c]);
    float* hp = e.out_f32 + (size_t)m * e.ld_f32 + c;
    const float r = *hp + e.gate[c] * a;
    *hp = r;
    if (e.out_act) reinterpret_cast<T*>(e.out_act)[(size_t)m * e.ld_act + c] = from_f32<T>(r);
    v[p] = r;
    sc[p] = e.ln_scale[c];
    sh[p] = e.ln_shift[c];
    sum += r;
  }
  const float mean = block_sum<T, NT>(sum, red) / (float)g.N;
  float q = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const float dv = v[p] - mean;
    q += dv * dv;
  }
  const float var = block_sum<T, NT>(q, red) / (float)g.N;
  const float rstd = 1.f / sqrtf(var + eps);
  T* o = reinterpret_cast<T*>(e.ln_out) + (size_t)m * e.ln_ldo;
#pragma unroll
  for (int p = 0; p < PER; ++p) o[t + p * NT] = from_f32<T>((v[p] - mean) * rstd * (1.f + sc[p]) + sh[p]);
}

}  // namespace fm
