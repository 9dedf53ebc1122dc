// Host side of the FlashMap drafting library: argument checks, workspace
// layout, launch planning and the launch sequences behind the C ABI declared
// in include/flashmap.h.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <string>
#include <vector>

#include "../../include/flashmap.h"
#include "attention.hpp"
#include "common.hpp"
#include "embed.hpp"
#include "gemm.hpp"
#include "lmhead.hpp"
#include "norm.hpp"
#include "schedule.hpp"
#include "softmax.hpp"
#include "stream.hpp"
#include "verify.hpp"

using namespace fm;

// Scratch of fm_verify_sample_noalloc, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops): one copy per GPU,
// held until the process ends.  Host code must not pass the array's name to a
// kernel (on the host it is a stand-in, not a device address): the address of
// each device's copy comes from hipGetSymbolAddress, once per device.
constexpr int NOALLOC_MAX_B = 4;  // branches (of K = 16 rows) one call may verify
static __device__ __align__(256) unsigned char scratch[160 * 1024];

namespace {

thread_local std::string g_err;

fm_status fail(fm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

// this device's copy of `scratch`, looked up once per device (device current)
fm_status scratch_ptr(char** out) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static char* ptr[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEV) return fail(FM_EINVAL, "device %d outside 0..%d", dev, MAX_DEV - 1);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(FM_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    ptr[dev] = static_cast<char*>(p);
  }
  *out = ptr[dev];
  return FM_OK;
}

#define FM_HIP(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return fail(FM_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define FM_LAUNCHED(what)                                                                       \
  do {                                                                                          \
    hipError_t e_ = hipGetLastError();                                                          \
    if (e_ != hipSuccess) return fail(FM_EHIP, "launch of %s: %s", what, hipGetErrorString(e_)); \
  } while (0)

#define FM_TRY(expr)                 \
  do {                               \
    fm_status s_ = (expr);           \
    if (s_ != FM_OK) return s_;      \
  } while (0)

constexpr int KB = 16;             // block rows per branch (K)
constexpr int ATT_MAX_RANGES = ATT_RANGES_MAX;
constexpr int ATT_WAVES = 8;  // waves per attention workgroup
constexpr int GEMM_MAX_SPLIT = GEMM_SPLIT_MAX;
constexpr int LM_WAVES = 8;
constexpr int LM_GRID = 512;  // most LM head workgroups (keys per row)
constexpr int VS_MAX_SLICES = VS_THREADS;  // vocabulary slices of the probabilistic verifier
constexpr int VS_SLICE = 1024;             // tokens per slice (at least)
constexpr int EMB_WAVES = 8;
constexpr int MAX_PREFILL_ROWS = 16;
constexpr int N_COUNTER_SLOTS = 1024;  // counters, COUNTER_STRIDE words apart
constexpr int SOFTMAX_CHUNK = 4096;

size_t esize(fm_dtype t) { return t == FM_BF16 ? 2 : 4; }
int vec_elems(fm_dtype t) { return t == FM_BF16 ? 8 : 4; }
int gemm_chunk(fm_dtype t) { return 32 * vec_elems(t); }  // k elements per streamed chunk
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

// scratch of the probabilistic verifier: slice states, row normalisers, the
// accepted prefixes and row n's slice keys
struct VsScratch {
  float2* stats;     // [B*(K+1)][VS_MAX_SLICES]
  float* lse_rows;   // [B*(K+1)]
  int32_t* n_acc;    // [B]
  uint64_t* keys;    // [B][VS_MAX_SLICES][2]
};

// bytes of VsScratch for B branches of K rows, carved from one 256-byte-aligned base
size_t vs_scratch_bytes(int B, int K) {
  return align256((size_t)B * (K + 1) * VS_MAX_SLICES * 8) + align256((size_t)B * (K + 1) * 4) +
         align256((size_t)B * 4) + align256((size_t)B * VS_MAX_SLICES * 16);
}
VsScratch vs_scratch_at(char* base, int B, int K) {
  VsScratch s;
  s.stats = reinterpret_cast<float2*>(base);
  base += align256((size_t)B * (K + 1) * VS_MAX_SLICES * 8);
  s.lse_rows = reinterpret_cast<float*>(base);
  base += align256((size_t)B * (K + 1) * 4);
  s.n_acc = reinterpret_cast<int32_t*>(base);
  base += align256((size_t)B * 4);
  s.keys = reinterpret_cast<uint64_t*>(base);
  return s;
}


struct GemmPlan {
  int S, k_split, n_groups, grid, waves;
  int tg;  // > 0: tile-group kernel with tg tiles per workgroup
};

// One workgroup per (16-row tile, k split).  Without a split there is no
// cross-workgroup reduction at all; a split is used only when the tiles alone
// cannot cover the CUs and the k range is long (a device-scope arrival costs a
// memory round trip).  Workgroups of 8 waves when tiles are few, else 4.
//
// A workgroup's bytes are its weight share plus the A rows of its k range, so
// with many rows (M > 32) A dominates: tiles are grouped two to a workgroup
// to share it, except at 80 rows, where the two tiles' A and weight fragments
// would not fit in registers.  Measured at 64 rows, a finer k split at the
// same grouping moves the same bytes per CU and only adds arrivals.
GemmPlan plan_gemm(int M, int N, int K, fm_dtype t) {
  const int chunk = gemm_chunk(t);
  const int MT = cdiv(M, 16);
  GemmPlan p;
  p.n_groups = cdiv(N, 16);
  const int nch = std::max(1, cdiv(K, chunk));
  p.tg = 0;
  if (p.n_groups >= 256 && nch <= 8) {
    // wide layer, short k: tiles per workgroup of 8 waves, one chunk per wave
    p.tg = MT >= 5 ? 1 : 2;
    p.waves = 8;
    p.S = 1;
    p.k_split = nch * chunk;
    p.grid = cdiv(p.n_groups, p.tg);
    return p;
  }
  if (p.n_groups < 256 && nch >= 16 && nch <= 4 * GEMM_MAX_SPLIT && MT >= 3) {
    // narrow layer, long k, many rows: two tiles and eight chunks (one a wave)
    // per workgroup of 8 waves, k split at most four ways
    p.tg = 2;
    p.waves = 8;
    p.k_split = 8 * chunk;
    p.S = cdiv(K, p.k_split);
    p.grid = cdiv(p.n_groups, 2) * p.S;
    return p;
  }
  if (p.n_groups < 256 && nch >= 16 && nch <= 4 * GEMM_MAX_SPLIT) {
    // narrow layer, long k: one tile and four chunks (one a wave) per workgroup
    // of 4 waves, up to 8 splits of k summed by the last split to arrive.  With
    // 16 rows and the weights streaming from HBM this beats two tiles per
    // 8-wave workgroup split four ways (582 against 590 us per step), which
    // moves fewer bytes per CU but hides less latency with half the waves
    p.tg = 1;
    p.waves = 4;
    p.S = cdiv(nch, 4);
    p.k_split = 4 * chunk;
    p.grid = p.n_groups * p.S;
    return p;
  }
  if (p.n_groups < 256 && nch > 4 * GEMM_MAX_SPLIT && p.n_groups % 2 == 0) {
    // narrow layer, very long k (the context fusion, k = 5H): two tiles per
    // workgroup of 8 waves share each activation chunk, k split so that the
    // launch has about 256 workgroups, waves loop over their chunks
    p.tg = 2;
    p.waves = 8;
    p.S = std::min(GEMM_MAX_SPLIT, std::max(1, 256 / (p.n_groups / 2)));
    p.k_split = cdiv(nch, p.S) * chunk;
    p.S = cdiv(K, p.k_split);
    p.grid = (p.n_groups / 2) * p.S;
    return p;
  }
  p.waves = p.n_groups < 256 ? 8 : 4;
  int S = 1;
  if (p.n_groups < 256 && nch > 4 * p.waves) S = std::min(GEMM_MAX_SPLIT, cdiv(256, p.n_groups));
  p.k_split = cdiv(nch, S) * chunk;
  p.S = cdiv(K, p.k_split);
  p.grid = p.n_groups * p.S;
  return p;
}

// 48..80 rows (bf16) and enough (column group, k slice) workgroups to cover
// half the CUs: the A slice is kept in LDS per workgroup (gemm_as_kernel) and
// the slices are summed by gemm_reduce_kernel.  Slices of 512 (two chunks)
// where they give enough workgroups, else of 256.  S = k slices.
bool use_as(int M, int N, int K, fm_dtype t, int* S, int* KS) {
  if (t != FM_BF16 || cdiv(M, 16) < 3 || cdiv(M, 16) > 5 || N % 4 != 0) return false;
  const int groups = cdiv(N, 16 * AS_TILES);
  for (int ks : {512, 256}) {
    if (K % ks != 0 || K / ks > AS_SMAX || groups * (K / ks) < 128) continue;
    *S = K / ks;
    *KS = ks;
    return true;
  }
  return false;
}

// a gated residual contraction on that path whose row-wise reduce can also
// apply the LayerNorm that follows (widths 2048 and 4096)
bool resid_ln_fused(int M, int N, int K, fm_dtype t) {
  int S, KS;
  return use_as(M, N, K, t, &S, &KS) && (N == 2048 || N == 4096);
}

struct EmbedPlan {
  int MT, n_cb, Sf, Ss, grid;
};

// Column blocks of 16*VE columns, each over Sf row splits of V (Ss for the
// slower blocks; the grid is a multiple of 8 for the XCD placement).
EmbedPlan plan_embed(int d, fm_dtype t, int M) {
  EmbedPlan p;
  p.MT = cdiv(M, 16);
  p.n_cb = d / (16 * vec_elems(t));
  if (p.n_cb == 16 && t == FM_BF16) {
    // the four column blocks at 256-byte offsets 4i+1 of each 4 KB row of E
    // stream about 20% slower: 19 row splits for them, 15 for the others
    // (256 workgroups, finishing together; 100 against 94 us streaming alone)
    p.Sf = 15;
    p.Ss = 19;
  } else {
    p.Sf = p.Ss = 16;
  }
  p.grid = p.n_cb * p.Sf + (p.Ss - p.Sf) * (p.n_cb / 4);
  return p;
}

// positions per head of one request's cache: the context capacity rounded up to
// whole 32-key blocks, then one 32-position scratch block per branch for that
// branch's block rows
int cache_positions(const fm_config& c) { return cdiv(c.C_max, ATT_BLK) * ATT_BLK + ATT_BLK * c.max_branches; }
// row blocks of one draft: branches of one request, or requests of one batch
int max_blocks(const fm_config& c) { return std::max(c.max_branches, c.max_requests); }

struct Layout {
  size_t cache, mods, sched, ctx, h, e_state, u_pre, act_qkv, act_d, attn_o, act_f, qkv;
  size_t att_po, att_ml, partial, lm_part, lm_lse, counters, dsoft, logits_tmp, sm_part, vs, lnpart, lnpart_u, total;
};

int max_rows(const fm_config& c) { return max_blocks(c) * KB; }

size_t partial_bytes(const fm_config& c) {
  const int Mb = max_rows(c), F = c.mlp_mult * c.d, d = c.d;
  struct S3 { int M, N, K; };
  const S3 shapes[] = {{Mb + c.max_new, 3 * d, d}, {Mb, d, d}, {Mb, F, d}, {Mb, d, F},
                       {MAX_PREFILL_ROWS, d, c.n_ctx_layers * c.H}, {MAX_PREFILL_ROWS, 2 * d, d}};
  size_t mx = 0;
  // the plan depends on the 16-row tiles of M: the largest M of each count
  for (const S3& s : shapes)
    for (int M = std::min(16, s.M);; M = std::min(s.M, M + 16)) {
      GemmPlan p = plan_gemm(M, s.N, s.K, c.dtype);
      if (p.S > 1) mx = std::max(mx, (size_t)p.S * M * s.N * 4);
      int S_as, KS_as;
      if (use_as(M, s.N, s.K, c.dtype, &S_as, &KS_as)) mx = std::max(mx, (size_t)S_as * M * s.N * 4);
      if (M == s.M) break;
    }
  for (int M = 16; M <= Mb; M += 16) {
    EmbedPlan e = plan_embed(c.d, c.dtype, M);
    mx = std::max(mx, (size_t)e.Ss * M * d * 4);
  }
  return mx;
}

Layout make_layout(const fm_config& c) {
  Layout L{};
  const size_t es = esize(c.dtype);
  const size_t d = c.d, F = (size_t)c.mlp_mult * c.d, Mb = max_rows(c), hd = c.d / c.n_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  // per DiT block: the keys of every request, then their values
  L.cache = take((size_t)c.L * 2 * c.max_requests * cache_positions(c) * d * es);
  L.mods = take((size_t)c.max_steps * (6 * c.L + 2) * d * 4);
  L.sched = take(((size_t)2 * c.max_steps * 256 + 3 * (size_t)c.max_steps * d) * 4);
  L.ctx = take((FM_MAX_REQ + 1) * 4);  // context length of each request, then the overflow flag
  L.h = take(Mb * d * 4);
  L.e_state = take(Mb * d * 4);
  L.u_pre = take((size_t)std::max(MAX_PREFILL_ROWS, c.max_new) * d * 4);
  L.act_qkv = take((Mb + std::max(MAX_PREFILL_ROWS, c.max_new)) * d * es);
  L.act_d = take(Mb * d * es);
  L.attn_o = take(Mb * d * es);
  L.act_f = take(Mb * F * es);
  L.qkv = take(Mb * d * es);  // queries of the block rows
  const int att_ranges = std::max(ATT_MAX_RANGES, ATT_TREE_RANGES);
  L.att_po = take((size_t)max_blocks(c) * c.n_heads * att_ranges * KB * hd * 4);
  L.att_ml = take((size_t)max_blocks(c) * c.n_heads * att_ranges * KB * 2 * 4);
  L.partial = take(partial_bytes(c));
  L.lm_part = take((size_t)LM_GRID * Mb * 8);
  L.lm_lse = take((size_t)LM_GRID * Mb * 8);
  L.vs = take(vs_scratch_bytes(max_blocks(c), KB));  // branches of one request, or requests
  L.lnpart = take((size_t)KB * LN_PART_MAX * sizeof(float2));  // row statistics for the fused LayerNorms
  L.lnpart_u = take((size_t)16 * LN_PART_MAX * sizeof(float2));  // and for the new context rows (max_new <= 16)
  L.counters = take((size_t)N_COUNTER_SLOTS * COUNTER_STRIDE * 4);
  if (c.max_steps > 1) {
    L.dsoft = take(Mb * (size_t)c.V * es);
    L.logits_tmp = take(Mb * (size_t)c.V * 4);
    L.sm_part = take(Mb * (size_t)cdiv(c.V, SOFTMAX_CHUNK) * 2 * 4);
  }
  L.total = off;
  return L;
}

fm_status check_config(const fm_config* c) {
  if (!c) return fail(FM_EINVAL, "config is NULL");
  if (c->dtype != FM_BF16 && c->dtype != FM_F32) return fail(FM_EINVAL, "dtype must be FM_BF16 or FM_F32");
  const int ve = vec_elems(c->dtype);
  if (c->K != KB) return fail(FM_EINVAL, "K must be 16 (got %d)", c->K);
  if (c->d < 16 * ve || c->d % (16 * ve))
    return fail(FM_EINVAL, "d must be a positive multiple of %d (got %d)", 16 * ve, c->d);
  if (c->n_heads < 1 || c->d % c->n_heads) return fail(FM_EINVAL, "n_heads must divide d");
  const int hd = c->d / c->n_heads;
  if (hd != 64 && hd != 128) return fail(FM_EINVAL, "head width d/n_heads must be 64 or 128 (got %d)", hd);
  if (c->d > 4096) return fail(FM_EINVAL, "d above 4096 is not supported (got %d)", c->d);
  if (c->L < 1) return fail(FM_EINVAL, "L must be >= 1");
  if (c->mlp_mult < 1) return fail(FM_EINVAL, "mlp_mult must be >= 1");
  if (c->n_ctx_layers != 5) return fail(FM_EINVAL, "n_ctx_layers must be 5 (layers 1, 9, 17, 25, 33)");
  if (c->V < 16 || c->V % ve) return fail(FM_EINVAL, "V must be >= 16 and a multiple of %d (got %d)", ve, c->V);
  if (c->H < 1 || c->H % ve) return fail(FM_EINVAL, "H must be a positive multiple of %d (got %d)", ve, c->H);
  if (c->C_max < 0) return fail(FM_EINVAL, "C_max must be >= 0");
  if (c->max_branches < 1 || c->max_branches > 4) return fail(FM_EINVAL, "max_branches must be in 1..4");
  if (c->max_new < 0 || c->max_new > 16) return fail(FM_EINVAL, "max_new must be in 0..16");
  if (c->max_steps < 1 || c->max_steps > 4) return fail(FM_EINVAL, "max_steps must be in 1..4");
  if (c->max_steps > 1 && cdiv(c->V, SOFTMAX_CHUNK) > 128)
    return fail(FM_EINVAL, "schedules of several jumps take V <= %d (got %d)", 128 * SOFTMAX_CHUNK, c->V);
  if (c->max_requests < 1 || c->max_requests > FM_MAX_REQ)
    return fail(FM_EINVAL, "max_requests must be in 1..%d", FM_MAX_REQ);
  if (c->max_requests > 1 && c->max_branches > 1)
    return fail(FM_EINVAL, "a handle holds either branches of one request or several requests, not both");
  return FM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

struct fm_handle {
  fm_config cfg;
  int device;
  char* ws;
  Layout lay;
  fm_weights w;
  std::vector<fm_block_weights> blocks;
  bool has_weights = false;
  int n_steps = 0;
  float times[8];
  // Host mirror of the device-resident context lengths, advanced by the calls
  // made on the host (not by graph replays; fm_context_sync reloads it).  It
  // serves the argument checks only: kernels read the lengths on the device.
  int ctx_len[FM_MAX_REQ] = {};
  int ctx_high[FM_MAX_REQ] = {};  // rows [0, ctx_high) have been written at least once
  int probe = FM_PROBE_NONE;
  hipEvent_t probe_start = nullptr, probe_stop = nullptr;

  template <typename P> P* at(size_t off) { return reinterpret_cast<P*>(ws + off); }
  // device-resident context lengths (and the overflow flag after them)
  int* ctx_dev() { return at<int>(lay.ctx); }
  int n_cu = 256;  // compute units of the device (sizes the L2 warming)
  // key / value cache of DiT block l, request 0 (request r at + r * req_stride())
  size_t req_stride() const { return (size_t)cache_positions(cfg) * cfg.d; }
  template <typename T> T* kcache(int l) { return at<T>(lay.cache) + (size_t)l * 2 * cfg.max_requests * req_stride(); }
  template <typename T> T* vcache(int l) { return kcache<T>(l) + (size_t)cfg.max_requests * req_stride(); }
};

namespace {

// ------------------------------------------------------------------ launchers
template <typename T, int MT, int EPI>
void launch_gemm_mt(const GemmArgs& a, const EpiParams& e, int grid, int waves, int tg, hipStream_t st) {
  if (tg == 2 && MT == 1 && a.k_split > 8 * ChunkT<T>::KC)  // several chunks a wave
    hipLaunchKernelGGL((gemm_tg_kernel<T, 1, 8, 2, EPI, false, true>), dim3(grid), dim3(8 * 64), 0, st, a, e,
                       LnArgs{});
  else if (tg == 2)
    hipLaunchKernelGGL((gemm_tg_kernel<T, MT, 8, 2, EPI, false>), dim3(grid), dim3(8 * 64), 0, st, a, e, LnArgs{});
  else if (tg == 1 && waves == 8)
    hipLaunchKernelGGL((gemm_tg_kernel<T, MT, 8, 1, EPI, false>), dim3(grid), dim3(8 * 64), 0, st, a, e, LnArgs{});
  else if (tg == 1)
    hipLaunchKernelGGL((gemm_tg_kernel<T, MT, 4, 1, EPI, false>), dim3(grid), dim3(4 * 64), 0, st, a, e, LnArgs{});
  else if (waves == 8)
    hipLaunchKernelGGL((gemm_kernel<T, MT, 8, EPI>), dim3(grid), dim3(8 * 64), 0, st, a, e);
  else
    hipLaunchKernelGGL((gemm_kernel<T, MT, 4, EPI>), dim3(grid), dim3(4 * 64), 0, st, a, e);
}

template <typename T, int EPI>
fm_status launch_gemm_epi(const GemmArgs& a, const EpiParams& e, const GemmPlan& p, hipStream_t st) {
  switch (cdiv(a.M, 16)) {
    case 1: launch_gemm_mt<T, 1, EPI>(a, e, p.grid, p.waves, p.tg, st); break;
    case 2: launch_gemm_mt<T, 2, EPI>(a, e, p.grid, p.waves, p.tg, st); break;
    case 3: launch_gemm_mt<T, 3, EPI>(a, e, p.grid, p.waves, p.tg, st); break;
    case 4: launch_gemm_mt<T, 4, EPI>(a, e, p.grid, p.waves, p.tg, st); break;
    case 5: launch_gemm_mt<T, 5, EPI>(a, e, p.grid, p.waves, p.tg, st); break;
    default: return fail(FM_EINVAL, "contraction with %d rows exceeds 80", a.M);
  }
  FM_LAUNCHED("gemm_kernel");
  return FM_OK;
}

// The L2 region of the contraction gemm() runs for (M, N, K) on weights W:
// on the tile paths without a k split (gemm_kernel, or gemm_tg_kernel with its
// tiles per workgroup) workgroup b reads tile group b alone, on the LDS-slice
// path k slice b % S of row group b / S; N a whole number of groups.  False:
// no such mapping.
bool l2_region(const fm_handle* h, int M, int N, int K, const void* W, L2Region* r) {
  const fm_dtype t = h->cfg.dtype;
  int S_as, KS_as;
  *r = L2Region{};
  if (t == FM_BF16 && use_as(M, N, K, t, &S_as, &KS_as)) {
    // the LDS-slice path: workgroup b = g * S + s reads rows 128 g .. + 128
    // (AS_TILES tiles), k slice s of KS_as elements
    const int rows = 16 * AS_TILES;
    if (N % rows || (size_t)KS_as * esize(t) % 16 || (size_t)K * esize(t) % 16) return false;
    r->base = reinterpret_cast<const uint4*>(W);
    r->n_groups = N / rows;
    r->slices = S_as;
    r->rows = rows;
    r->row_u4 = (size_t)K * esize(t) / 16;
    r->take_u4 = (size_t)KS_as * esize(t) / 16;
    return true;
  }
  const GemmPlan p = plan_gemm(M, N, K, t);
  const int tiles = p.tg == 2 ? 2 : 1;
  if (p.S != 1 || N % (16 * tiles) || p.grid != N / (16 * tiles)) return false;
  r->base = reinterpret_cast<const uint4*>(W);
  r->group_u4 = (size_t)16 * tiles * K * esize(t) / 16;
  r->off_u4 = 0;
  r->take_u4 = r->group_u4;
  r->n_groups = N / (16 * tiles);
  return true;
}

// The same for a fused-LayerNorm contraction (gemm_ln: workgroup b reads
// tiles 2b and 2b + 1)
bool l2_region_ln(const fm_handle* h, int N, int K, const void* W, L2Region* r) {
  *r = L2Region{};
  if (N % 32) return false;
  r->base = reinterpret_cast<const uint4*>(W);
  r->group_u4 = (size_t)32 * K * esize(h->cfg.dtype) / 16;
  r->off_u4 = 0;
  r->take_u4 = r->group_u4;
  r->n_groups = N / 32;
  return true;
}

// Warming workgroups for a launch of grid workgroups on the CUs it leaves
// idle: fills w's workgroup range and returns the grid with them (w.n_reg = 0
// or no idle CUs: grid unchanged, w disabled).
int l2_warm_attach(const fm_handle* h, int grid, L2Warm& w) {
  if (w.n_reg <= 0 || grid + 8 > h->n_cu) {
    w.n_reg = 0;
    return grid;
  }
  w.first_wg = grid;
  w.n_wg = (h->n_cu - grid) / 8 * 8;
  return grid + w.n_wg;
}

// out[m][n] = epilogue( sum_k A[m][k] W[n][k] )
template <typename T>
fm_status gemm(fm_handle* h, int epi, const void* A, int lda, int M, const void* W, int N, int K,
               const EpiParams& e, hipStream_t st) {
  if (M <= 0) return FM_OK;
  if constexpr (std::is_same<T, bf16_t>::value) {
    int S_as, KS_as;
    if (use_as(M, N, K, h->cfg.dtype, &S_as, &KS_as)) {
      GemmArgs a{};
      a.A = A;
      a.lda = lda;
      a.M = M;
      a.W = W;
      a.ldw = K;
      a.N = N;
      a.K = K;
      a.S = S_as;
      a.k_split = KS_as;
      a.partial = h->at<float>(h->lay.partial);
      const int grid = cdiv(N, 16 * AS_TILES) * S_as;
      const int mt = cdiv(M, 16);
      const bool ln_after = epi == EPI_RESID && e.ln_out;
      if (e.ln_part) return fail(FM_EINVAL, "no row statistics from the LDS-slice contraction");
      if (ln_after && !resid_ln_fused(M, N, K, h->cfg.dtype))
        return fail(FM_EINVAL, "no LayerNorm-fused reduce for this contraction");
      if (KS_as == 512) {
        if (mt == 3) hipLaunchKernelGGL((gemm_as_kernel<T, 3, 512>), dim3(grid), dim3(512), 0, st, a);
        else if (mt == 4) hipLaunchKernelGGL((gemm_as_kernel<T, 4, 512>), dim3(grid), dim3(512), 0, st, a);
        else hipLaunchKernelGGL((gemm_as_kernel<T, 5, 512>), dim3(grid), dim3(512), 0, st, a);
      } else {
        if (mt == 3) hipLaunchKernelGGL((gemm_as_kernel<T, 3, 256>), dim3(grid), dim3(512), 0, st, a);
        else if (mt == 4) hipLaunchKernelGGL((gemm_as_kernel<T, 4, 256>), dim3(grid), dim3(512), 0, st, a);
        else hipLaunchKernelGGL((gemm_as_kernel<T, 5, 256>), dim3(grid), dim3(512), 0, st, a);
      }
      FM_LAUNCHED("gemm_as_kernel");
      if (ln_after) {
        if (N == 2048)
          hipLaunchKernelGGL((gemm_reduce_ln_kernel<T, 2>), dim3(M), dim3(1024), 0, st, a, e, 1e-6f);
        else
          hipLaunchKernelGGL((gemm_reduce_ln_kernel<T, 4>), dim3(M), dim3(1024), 0, st, a, e, 1e-6f);
        FM_LAUNCHED("gemm_reduce_ln_kernel");
        return FM_OK;
      }
      const dim3 rgrid4((unsigned)(((size_t)M * N / 4 + 255) / 256));
      const dim3 rgrid1((unsigned)(((size_t)M * N + 255) / 256));
      switch (epi) {
        case EPI_F32: hipLaunchKernelGGL((gemm_reduce_kernel<T, EPI_F32, 4>), rgrid4, dim3(256), 0, st, a, e); break;
        case EPI_ACT: hipLaunchKernelGGL((gemm_reduce_kernel<T, EPI_ACT, 4>), rgrid4, dim3(256), 0, st, a, e); break;
        case EPI_GELU: hipLaunchKernelGGL((gemm_reduce_kernel<T, EPI_GELU, 4>), rgrid4, dim3(256), 0, st, a, e); break;
        case EPI_RESID: hipLaunchKernelGGL((gemm_reduce_kernel<T, EPI_RESID, 4>), rgrid4, dim3(256), 0, st, a, e); break;
        default: hipLaunchKernelGGL((gemm_reduce_kernel<T, EPI_QKV, 1>), rgrid1, dim3(256), 0, st, a, e); break;
      }
      FM_LAUNCHED("gemm_reduce_kernel");
      return FM_OK;
    }
  }
  GemmPlan p = plan_gemm(M, N, K, h->cfg.dtype);
  if (p.S > 1 && p.n_groups > N_COUNTER_SLOTS) return fail(FM_EINVAL, "too many column tiles for split-K");
  GemmArgs a;
  a.A = A;
  a.lda = lda;
  a.M = M;
  a.W = W;
  a.ldw = K;
  a.N = N;
  a.K = K;
  a.S = p.S;
  a.k_split = p.k_split;
  a.partial = h->at<float>(h->lay.partial);
  a.counters = h->at<uint32_t>(h->lay.counters);
  switch (epi) {
    case EPI_F32: return launch_gemm_epi<T, EPI_F32>(a, e, p, st);
    case EPI_ACT: return launch_gemm_epi<T, EPI_ACT>(a, e, p, st);
    case EPI_GELU: return launch_gemm_epi<T, EPI_GELU>(a, e, p, st);
    case EPI_RESID: return launch_gemm_epi<T, EPI_RESID>(a, e, p, st);
    default: return launch_gemm_epi<T, EPI_QKV>(a, e, p, st);
  }
}

// LayerNorm + modulation of the 16 residual rows x fused into the contraction's
// A operand; A_ctx supplies M_ctx further rows (already normalised) below them.
bool ln_fusable(const fm_config& c, int B) { return B == 1 && cdiv(c.d, gemm_chunk(c.dtype)) <= 8; }

template <typename T>
fm_status gemm_ln(fm_handle* h, int epi, const float* x, const float* shift, const float* scale, const void* A_ctx,
                  int M_ctx, const void* W, int N, int K, const EpiParams& e, hipStream_t st) {
  if (cdiv(K, gemm_chunk(h->cfg.dtype)) > 8) return fail(FM_EINVAL, "fused LayerNorm needs k <= 8 chunks");
  if (K % 16 || K / 16 > LN_PART_MAX) return fail(FM_EINVAL, "fused LayerNorm row of %d columns", K);
  GemmArgs a;
  a.A = A_ctx;
  a.lda = K;
  a.M = KB + M_ctx;
  a.W = W;
  a.ldw = K;
  a.N = N;
  a.K = K;
  a.S = 1;
  a.k_split = K;
  a.partial = nullptr;
  a.counters = nullptr;
  LnArgs l;
  l.h = x;
  l.ldh = K;
  l.shift = shift;
  l.scale = scale;
  l.eps = 1e-6f;
  l.part = h->at<float2>(h->lay.lnpart);  // written by the kernel that produced x
  l.part_ld = LN_PART_MAX;
  const dim3 grid(cdiv(cdiv(N, 16), 2)), block(8 * 64);
  const bool two = a.M > 16;
  if (epi == EPI_QKV && two)
    hipLaunchKernelGGL((gemm_tg_kernel<T, 2, 8, 2, EPI_QKV, true>), grid, block, 0, st, a, e, l);
  else if (epi == EPI_QKV)
    hipLaunchKernelGGL((gemm_tg_kernel<T, 1, 8, 2, EPI_QKV, true>), grid, block, 0, st, a, e, l);
  else if (epi == EPI_GELU && !two)
    hipLaunchKernelGGL((gemm_tg_kernel<T, 1, 8, 2, EPI_GELU, true>), grid, block, 0, st, a, e, l);
  else
    return fail(FM_EINVAL, "no fused LayerNorm variant for this contraction");
  FM_LAUNCHED("gemm_tg_kernel");
  return FM_OK;
}

template <typename T>
fm_status ln_mod(fm_handle* h, const float* x, int rows, const float* shift, const float* scale, T* out, int ldo,
                 hipStream_t st) {
  if (rows <= 0) return FM_OK;
  const int d = h->cfg.d;
  if (d <= 1024)
    hipLaunchKernelGGL((ln_mod_kernel<T, 4>), dim3(rows), dim3(256), 0, st, x, d, d, shift, scale, out, ldo, 1e-6f);
  else if (d <= 2048)
    hipLaunchKernelGGL((ln_mod_kernel<T, 8>), dim3(rows), dim3(256), 0, st, x, d, d, shift, scale, out, ldo, 1e-6f);
  else
    hipLaunchKernelGGL((ln_mod_kernel<T, 16>), dim3(rows), dim3(256), 0, st, x, d, d, shift, scale, out, ldo,
                       1e-6f);
  FM_LAUNCHED("ln_mod_kernel");
  return FM_OK;
}

fm_status probe_begin(fm_handle* h, int kernel, hipStream_t st);
fm_status probe_end(fm_handle* h, int kernel, hipStream_t st);

// probe: FM_PROBE_EMBED brackets embed_kernel alone (the contraction the
// counters and the roofline describe, without its split-sum kernel); -1
// records nothing
// ln_part: where the reduce also writes h's per-16-column row statistics for
// a fused LayerNorm that follows, or null.  n_u > 0: the reduce also applies
// the context fusion's LayerNorm to the n_u rows that fuse_rows left in u_pre
// (with their statistics), writing them to u_out.
template <typename T>
fm_status embed(fm_handle* h, const void* x, int ldx, int M, float alpha, float beta, hipStream_t st,
                int probe = -1, float2* ln_part = nullptr, int n_u = 0, T* u_out = nullptr) {
  const fm_config& c = h->cfg;
  if (M > 64) return fail(FM_EINVAL, "embedding contraction with %d rows exceeds 64", M);
  EmbedPlan p = plan_embed(c.d, c.dtype, M);
  EmbedArgs a;
  a.x = x;
  a.ldx = ldx;
  a.M = M;
  a.V = c.V;
  a.E = h->w.E;
  a.d = c.d;
  a.Sf = p.Sf;
  a.Ss = p.Ss;
  a.rows_split = cdiv(cdiv(c.V, p.Sf), 4 * vec_elems(c.dtype)) * 4 * vec_elems(c.dtype);
  a.rows_split_s = cdiv(cdiv(c.V, p.Ss), 4 * vec_elems(c.dtype)) * 4 * vec_elems(c.dtype);
  a.partial = h->at<float>(h->lay.partial);
  a.e_state = h->at<float>(h->lay.e_state);
  a.h = h->at<float>(h->lay.h);
  a.alpha = alpha;
  a.beta = beta;
  a.K = KB;
  a.use_pos = 1;
  a.ln_part = ln_part;
  a.ln_part_ld = LN_PART_MAX;
  a.u_pre = h->at<float>(h->lay.u_pre);
  a.u_part = h->at<float2>(h->lay.lnpart_u);
  a.u_part_ld = LN_PART_MAX;
  a.u_out = u_out;
  a.n_u = n_u;
  a.eps = 1e-6f;
  if (n_u < 0 || n_u > 16 || (n_u > 0 && (!u_out || c.d / 16 > LN_PART_MAX)))
    return fail(FM_EINVAL, "%d context rows for the embedding's reduce to normalise", n_u);
  if (p.Ss > EMB_SPLITS_MAX) return fail(FM_EINVAL, "embedding with %d row splits (at most %d)", p.Ss, EMB_SPLITS_MAX);
  const dim3 grid(p.grid), block(EMB_WAVES * 64);
  FM_TRY(probe_begin(h, probe, st));
  switch (p.MT) {
    case 1: hipLaunchKernelGGL((embed_kernel<T, 1, EMB_WAVES>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((embed_kernel<T, 2, EMB_WAVES>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((embed_kernel<T, 3, EMB_WAVES>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((embed_kernel<T, 4, EMB_WAVES>), grid, block, 0, st, a); break;
  }
  FM_LAUNCHED("embed_kernel");
  FM_TRY(probe_end(h, probe, st));
  hipLaunchKernelGGL((embed_reduce_kernel<T>), dim3(cdiv(M * c.d, 256) + n_u), dim3(256), 0, st, a);
  FM_LAUNCHED("embed_reduce_kernel");
  return FM_OK;
}

// attention of B row blocks in DiT block l; n_new[b]: rows the call appends to
// branch b's request (its visible context is that request's device-resident
// length plus n_new[b]).  Grids are sized for the cache capacity; the ranges
// in use follow the current length on the device.
template <typename T, int HD>
void launch_attention(const AttnArgs& a, int grid, int warm_kind, hipStream_t st) {
  const dim3 g(grid), b(ATT_WAVES * 64);
  if (warm_kind == L2W_TILES)
    hipLaunchKernelGGL((attention_kernel<T, HD, ATT_WAVES, L2W_TILES>), g, b, 0, st, a);
  else if (warm_kind == L2W_SLICES)
    hipLaunchKernelGGL((attention_kernel<T, HD, ATT_WAVES, L2W_SLICES>), g, b, 0, st, a);
  else
    hipLaunchKernelGGL((attention_kernel<T, HD, ATT_WAVES, L2W_NONE>), g, b, 0, st, a);
}

// warm: L2 warming for the next contractions, carried by extra workgroups of
// attention_kernel on the CUs it leaves idle
template <typename T>
fm_status attention(fm_handle* h, int l, int B, const int* n_new, bool own_ctx, hipStream_t st,
                    const L2Warm& warm = L2Warm{}) {
  const fm_config& c = h->cfg;
  const int hd = c.d / c.n_heads;
  AttnArgs a{};
  a.q = h->at<T>(h->lay.qkv);
  a.ldq = c.d;
  a.kc = h->kcache<T>(l);
  a.vt = h->vcache<T>(l);
  a.req_stride = h->req_stride();
  a.P = cache_positions(c);
  a.ctx_len = h->ctx_dev();
  for (int b = 0; b < B; ++b) a.n_new[b] = n_new[b];
  a.ctx_cap = c.C_max;
  a.scratch_blk = cdiv(c.C_max, ATT_BLK);
  a.scratch_step = own_ctx ? 0 : 1;
  a.K = KB;
  a.d = c.d;
  a.nh = c.n_heads;
  a.part_o = h->at<float>(h->lay.att_po);
  a.part_ml = h->at<float>(h->lay.att_ml);
  a.counters = h->at<uint32_t>(h->lay.counters);
  a.out = h->at<T>(h->lay.attn_o);
  a.scale = 1.0f / std::sqrt((float)hd);
  const int cap_blocks = cdiv(c.C_max, ATT_BLK);
  if constexpr (std::is_same<T, bf16_t>::value) {
    // 2..4 branches over one shared context: each key/value block is read
    // once per (head, range) and served to every branch from LDS
    if (!own_ctx && B >= 2 && B <= 4 && (hd == 128 || hd == 64)) {
      a.n_ranges = tree_max_ranges(cap_blocks);
      const dim3 tgrid(c.n_heads * a.n_ranges), tblock(512);
      if (hd == 128) {
        if (B == 2) hipLaunchKernelGGL((attention_tree_kernel<128, 2>), tgrid, tblock, 0, st, a);
        else if (B == 3) hipLaunchKernelGGL((attention_tree_kernel<128, 3>), tgrid, tblock, 0, st, a);
        else hipLaunchKernelGGL((attention_tree_kernel<128, 4>), tgrid, tblock, 0, st, a);
      } else {
        if (B == 2) hipLaunchKernelGGL((attention_tree_kernel<64, 2>), tgrid, tblock, 0, st, a);
        else if (B == 3) hipLaunchKernelGGL((attention_tree_kernel<64, 3>), tgrid, tblock, 0, st, a);
        else hipLaunchKernelGGL((attention_tree_kernel<64, 4>), tgrid, tblock, 0, st, a);
      }
      FM_LAUNCHED("attention_tree_kernel");
      if (a.n_ranges > 1) {
        const int mgrid = B * c.n_heads * (KB / 2);
        if (hd == 128)
          hipLaunchKernelGGL((attention_merge_kernel<T, 128>), dim3(mgrid), dim3(128), 0, st, a);
        else
          hipLaunchKernelGGL((attention_merge_kernel<T, 64>), dim3(mgrid), dim3(64), 0, st, a);
        FM_LAUNCHED("attention_merge_kernel");
      }
      return FM_OK;
    }
  }
  a.n_ranges = attn_max_ranges(cap_blocks + 1, ATT_WAVES);
  a.warm = warm;
  // the warming's regions are of one kind: those of the first region's kind
  const int kind = a.warm.n_reg <= 0 ? L2W_NONE : a.warm.reg[0].slices > 0 ? L2W_SLICES : L2W_TILES;
  int n_same = 0;
  while (n_same < a.warm.n_reg && (a.warm.reg[n_same].slices > 0) == (kind == L2W_SLICES)) ++n_same;
  a.warm.n_reg = n_same;
  const int grid = l2_warm_attach(h, B * c.n_heads * a.n_ranges, a.warm);
  const int wk = a.warm.n_reg > 0 ? kind : L2W_NONE;
  if (hd == 128) launch_attention<T, 128>(a, grid, wk, st);
  else launch_attention<T, 64>(a, grid, wk, st);
  FM_LAUNCHED("attention_kernel");
  return FM_OK;
}

// A draft over several requests: row block r is request r, with its own
// context, to which n_new[r] rows are appended first.
struct Batch {
  int R;
  int n_new[FM_MAX_REQ];
};

// Temperature > 0 drafting: tokens are sampled from softmax(logits / tau) and
// the per-row log-normalisers are written to lse.
struct Sampling {
  float tau;
  uint64_t seed;
  float* lse;                           // [M]
  const uint64_t* req_seeds = nullptr;  // host [R]: one seed per request of a batch
  int R = 0;
};

// the Philox keys of a draft's row blocks, or of a batch's requests
BlockRng rng_shared(uint64_t seed) {
  BlockRng r{};
  r.lo[0] = (uint32_t)(seed & 0xFFFFFFFFu);
  r.hi[0] = (uint32_t)(seed >> 32);
  r.per_request = 0;
  return r;
}
BlockRng rng_per_request(const uint64_t* seeds, int R) {
  BlockRng r{};
  for (int i = 0; i < R && i < 4; ++i) {
    r.lo[i] = (uint32_t)(seeds[i] & 0xFFFFFFFFu);
    r.hi[i] = (uint32_t)(seeds[i] >> 32);
  }
  r.per_request = 1;
  return r;
}
BlockRng rng_of(const Sampling& smp) {
  return smp.req_seeds ? rng_per_request(smp.req_seeds, smp.R) : rng_shared(smp.seed);
}

// probe: FM_PROBE_LM_HEAD brackets the LM head kernel alone (not the argmax
// merge); -1 records nothing
// cu: the draft's context update, applied by the argmax merge (the draft's
// last kernel)
template <typename T>
fm_status lm_head(fm_handle* h, const void* z, int M, float* logits, int32_t* tokens, hipStream_t st,
                  const Sampling* smp = nullptr, int probe = -1, const CtxUpdate& cu = CtxUpdate{}) {
  const fm_config& c = h->cfg;
  LmArgs a{};
  a.tau = smp ? smp->tau : 0.f;
  a.rng = smp ? rng_of(*smp) : BlockRng{};
  a.K = KB;
  a.lse_part = smp ? h->at<float2>(h->lay.lm_lse) : nullptr;
  a.z = z;
  a.M = M;
  a.d = c.d;
  a.W = h->w.W_lm;
  a.V = c.V;
  a.logits = logits;
  a.partial = h->at<uint64_t>(h->lay.lm_part);
  // k split over the waves with z held in registers (at most four 16-row x
  // 512-byte fragment sets per lane); with 16 rows, 512 workgroups (a second
  // dispatch round fills the CUs that finish first) even out the finish times
  const int mt = cdiv(M, 16), cpw = cdiv(cdiv(c.d, 32 * vec_elems(c.dtype)), LM_WAVES);
  if (mt < 1 || mt > 4) return fail(FM_EINVAL, "LM head with %d rows (1..64)", M);
  const bool ks = mt * cpw <= 4;
  const int grid = ks ? std::min(mt == 1 ? LM_GRID : LM_GRID / 2, cdiv(c.V, 16))
                      : std::min(LM_GRID / 2, cdiv(cdiv(c.V, 16), LM_WAVES));
  const dim3 block(LM_WAVES * 64);
  FM_TRY(probe_begin(h, probe, st));
  if (ks) {
    switch (mt * 8 + cpw) {
      case 9: hipLaunchKernelGGL((lmhead_ks_kernel<T, 1, LM_WAVES, 1>), dim3(grid), block, 0, st, a); break;
      case 10: hipLaunchKernelGGL((lmhead_ks_kernel<T, 1, LM_WAVES, 2>), dim3(grid), block, 0, st, a); break;
      case 11: hipLaunchKernelGGL((lmhead_ks_kernel<T, 1, LM_WAVES, 3>), dim3(grid), block, 0, st, a); break;
      case 12: hipLaunchKernelGGL((lmhead_ks_kernel<T, 1, LM_WAVES, 4>), dim3(grid), block, 0, st, a); break;
      case 17: hipLaunchKernelGGL((lmhead_ks_kernel<T, 2, LM_WAVES, 1>), dim3(grid), block, 0, st, a); break;
      case 18: hipLaunchKernelGGL((lmhead_ks_kernel<T, 2, LM_WAVES, 2>), dim3(grid), block, 0, st, a); break;
      case 25: hipLaunchKernelGGL((lmhead_ks_kernel<T, 3, LM_WAVES, 1>), dim3(grid), block, 0, st, a); break;
      case 33: hipLaunchKernelGGL((lmhead_ks_kernel<T, 4, LM_WAVES, 1>), dim3(grid), block, 0, st, a); break;
      default: return fail(FM_EINVAL, "LM head plan: %d row tiles x %d chunks per wave", mt, cpw);
    }
    FM_LAUNCHED("lmhead_ks_kernel");
  } else {
    switch (mt) {
      case 1: hipLaunchKernelGGL((lmhead_kernel<T, 1, LM_WAVES>), dim3(grid), block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((lmhead_kernel<T, 2, LM_WAVES>), dim3(grid), block, 0, st, a); break;
      case 3: hipLaunchKernelGGL((lmhead_kernel<T, 3, LM_WAVES>), dim3(grid), block, 0, st, a); break;
      default: hipLaunchKernelGGL((lmhead_kernel<T, 4, LM_WAVES>), dim3(grid), block, 0, st, a); break;
    }
    FM_LAUNCHED("lmhead_kernel");
  }
  FM_TRY(probe_end(h, probe, st));
  if (tokens) {
    hipLaunchKernelGGL(argmax_finalize_kernel, dim3(M), dim3(FIN_THREADS), 0, st, a.partial, grid, tokens,
                       a.lse_part, smp ? smp->lse : nullptr, cu);
    FM_LAUNCHED("argmax_finalize_kernel");
  }
  return FM_OK;
}

template <typename T>
fm_status softmax_rows(fm_handle* h, int M, hipStream_t st) {
  const fm_config& c = h->cfg;
  SoftmaxArgs a;
  a.logits = h->at<float>(h->lay.logits_tmp);
  a.V = c.V;
  a.n_chunks = cdiv(c.V, SOFTMAX_CHUNK);  // <= 128 (checked with the configuration)
  a.part = h->at<float>(h->lay.sm_part);
  a.counters = nullptr;
  a.out = h->at<T>(h->lay.dsoft);
  hipLaunchKernelGGL((softmax_stats_kernel<SOFTMAX_CHUNK>), dim3(M * a.n_chunks), dim3(256), 0, st, a);
  FM_LAUNCHED("softmax_stats_kernel");
  hipLaunchKernelGGL((softmax_write_kernel<T, SOFTMAX_CHUNK>), dim3(M * a.n_chunks), dim3(256), 0, st, a);
  FM_LAUNCHED("softmax_write_kernel");
  return FM_OK;
}

fm_status trace_copy(const float* src, float* dst, size_t n, hipStream_t st) {
  hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)std::min<size_t>(1024, (n + 255) / 256)), dim3(256), 0, st, src,
                     dst, n);
  FM_LAUNCHED("copy_f32_kernel");
  return FM_OK;
}

fm_status probe_begin(fm_handle* h, int kernel, hipStream_t st) {
  if (h->probe == kernel) FM_HIP(hipEventRecord(h->probe_start, st));
  return FM_OK;
}
fm_status probe_end(fm_handle* h, int kernel, hipStream_t st) {
  if (h->probe == kernel) FM_HIP(hipEventRecord(h->probe_stop, st));
  return FM_OK;
}

const void* blk(const fm_handle* h, int l, int which) {
  const fm_block_weights& b = h->blocks[l];
  const void* const p[] = {b.W_ada, b.b_ada, b.W_qkv, b.b_qkv, b.W_o, b.b_o, b.W_1, b.b_1, b.W_2, b.b_2};
  return p[which];
}
enum { B_WADA, B_BADA, B_WQKV, B_BQKV, B_WO, B_BO, B_W1, B_B1, B_W2, B_B2 };

template <typename T>
const void* offset_rows(const void* p, size_t elems) {
  return reinterpret_cast<const T*>(p) + elems;
}

// whether the embedding's reduce can apply the context fusion's LayerNorm to
// n new rows (their statistics fit its per-16-column buffer)
bool ln_u_in_reduce(const fm_config& c, int n) { return n > 0 && n <= 16 && c.d / 16 <= LN_PART_MAX; }

// u rows (fusion + LN) for n context rows, written to out (storage type).
// ln_later: the contraction writes the rows' per-16-column statistics and the
// LayerNorm is left to the embedding's reduce (out is then unused here).
template <typename T>
fm_status fuse_rows(fm_handle* h, const void* feats, int n, T* out, hipStream_t st, bool ln_later = false) {
  const fm_config& c = h->cfg;
  const int K5 = c.n_ctx_layers * c.H;
  EpiParams e{};
  e.bias = h->w.b_f;
  e.out_f32 = h->at<float>(h->lay.u_pre);
  e.ld_f32 = c.d;
  if (ln_later) {
    e.ln_part = h->at<float2>(h->lay.lnpart_u);
    e.ln_part_ld = LN_PART_MAX;
  }
  FM_TRY(gemm<T>(h, EPI_F32, feats, K5, n, h->w.W_f, c.d, K5, e, st));
  if (ln_later) return FM_OK;
  return ln_mod<T>(h, h->at<float>(h->lay.u_pre), n, nullptr, nullptr, out, c.d, st);
}

// cache fields of the QKV epilogue for DiT block l
template <typename T>
void qkv_cache_params(fm_handle* h, int l, EpiParams& e) {
  const fm_config& c = h->cfg;
  e.kcache = h->kcache<T>(l);
  e.vcache = h->vcache<T>(l);
  e.req_stride = h->req_stride();
  e.P = cache_positions(c);
  e.hd = c.d / c.n_heads;
  e.d = c.d;
  e.scratch_pos0 = cdiv(c.C_max, ATT_BLK) * ATT_BLK;
  e.scratch_step = ATT_BLK;
  e.n_req = 1;
  e.ctx_len = h->ctx_dev();
  e.ctx_off = 0;
  e.ctx_cap = c.C_max;
}

fm_status ctx_update_launch(const CtxUpdate& u, hipStream_t st) {
  hipLaunchKernelGGL(ctx_update_kernel, dim3(1), dim3(64), 0, st, u);
  FM_LAUNCHED("ctx_update_kernel");
  return FM_OK;
}

template <typename T>
fm_status context_append_impl(fm_handle* h, int req, const void* feats, int n, hipStream_t st) {
  const fm_config& c = h->cfg;
  const int K5 = c.n_ctx_layers * c.H;
  T* stage = h->at<T>(h->lay.act_qkv);
  for (int r0 = 0; r0 < n; r0 += MAX_PREFILL_ROWS) {
    const int rows = std::min(MAX_PREFILL_ROWS, n - r0);
    const void* f = reinterpret_cast<const T*>(feats) + (size_t)r0 * K5;
    FM_TRY(fuse_rows<T>(h, f, rows, stage, st));
    for (int l = 0; l < c.L; ++l) {
      EpiParams e{};
      e.bias = offset_rows<T>(blk(h, l, B_BQKV), c.d);
      e.rows_block = 0;
      qkv_cache_params<T>(h, l, e);
      e.kcache = h->kcache<T>(l) + (size_t)req * h->req_stride();
      e.vcache = h->vcache<T>(l) + (size_t)req * h->req_stride();
      e.ctx_first[0] = 0;
      e.ctx_first[1] = rows;
      e.ctx_len = h->ctx_dev() + req;
      e.ctx_off = r0;
      e.col_offset = c.d;
      FM_TRY(gemm<T>(h, EPI_QKV, stage, c.d, rows, offset_rows<T>(blk(h, l, B_WQKV), (size_t)c.d * c.d), 2 * c.d,
                     c.d, e, st));
    }
  }
  CtxUpdate u{};
  u.len = h->ctx_dev();
  u.first = req;
  u.count = 1;
  u.val[0] = n;
  u.cap = c.C_max;
  return ctx_update_launch(u, st);
}

template <typename T>
fm_status draft_impl(fm_handle* h, const void* noise, int B, const void* new_feats, int n_new, int32_t* tokens,
                     float* logits, float* hidden, hipStream_t st, const Sampling* smp = nullptr,
                     const Batch* bt = nullptr) {
  const fm_config& c = h->cfg;
  const int d = c.d, F = c.mlp_mult * c.d, Mb = B * KB, L = c.L;
  // rows appended to each row block's request, and where the new context rows
  // of each request sit below the block rows
  int nb_new[FM_MAX_REQ];
  EpiParams ctx{};
  ctx.n_req = bt ? bt->R : 1;
  ctx.ctx_first[0] = 0;
  for (int b = 0; b < B; ++b) nb_new[b] = bt ? bt->n_new[b] : n_new;
  for (int r = 0; r < ctx.n_req; ++r) ctx.ctx_first[r + 1] = ctx.ctx_first[r] + (bt ? bt->n_new[r] : n_new);
  // the lengths advance in the draft's last kernel
  CtxUpdate adv{};
  adv.len = h->ctx_dev();
  adv.first = 0;
  adv.count = ctx.n_req;
  for (int r = 0; r < ctx.n_req; ++r) adv.val[r] = bt ? bt->n_new[r] : n_new;
  adv.cap = c.C_max;
  const bool fuse_ln = ln_fusable(c, B);
  // with fused LayerNorms, the producers of h (the embedding's reduce, W_o and
  // fc2) also write its per-16-column row statistics
  float2* lnp = fuse_ln ? h->at<float2>(h->lay.lnpart) : nullptr;
  // many rows: the reduces of W_o and fc2 also write the LayerNorm that follows
  const bool ln_in_reduce = !fuse_ln && resid_ln_fused(Mb, d, d, c.dtype) && resid_ln_fused(Mb, d, F, c.dtype);
  T* act_qkv = h->at<T>(h->lay.act_qkv);
  T* act_d = h->at<T>(h->lay.act_d);
  T* act_f = h->at<T>(h->lay.act_f);
  T* attn_o = h->at<T>(h->lay.attn_o);
  T* qkv = h->at<T>(h->lay.qkv);
  float* hres = h->at<float>(h->lay.h);
  const float* mods_all = h->at<float>(h->lay.mods);

  // context rows appended in this step: u goes below the block rows of act_qkv,
  // normalised by the first embedding's reduce where it can
  const bool u_in_reduce = ln_u_in_reduce(c, n_new);
  if (n_new > 0) FM_TRY(fuse_rows<T>(h, new_feats, n_new, act_qkv + (size_t)Mb * d, st, u_in_reduce));

  for (int j = 0; j < h->n_steps; ++j) {
    const float s = h->times[j], t = h->times[j + 1];
    const float* mods = mods_all + (size_t)j * (6 * L + 2) * d;
    if (j == 0) {
      FM_TRY(embed<T>(h, noise, c.V, Mb, 0.f, 1.f, st, FM_PROBE_EMBED, lnp, u_in_reduce ? n_new : 0,
                      act_qkv + (size_t)Mb * d));
    } else {
      const float sp = h->times[j - 1];
      FM_TRY(embed<T>(h, h->at<T>(h->lay.dsoft), c.V, Mb, (1.f - s) / (1.f - sp), (s - sp) / (1.f - sp), st, -1,
                      lnp));
    }
    if (hidden) FM_TRY(trace_copy(hres, hidden + ((size_t)j * (L + 1)) * Mb * d, (size_t)Mb * d, st));
    const int m_qkv = Mb + (j == 0 ? n_new : 0);
    for (int l = 0; l < L; ++l) {
      const float* mv = mods + (size_t)6 * l * d;  // shift1 scale1 gate1 shift2 scale2 gate2
      {
        EpiParams e{};
        e.bias = blk(h, l, B_BQKV);
        e.out_act = qkv;
        e.ld_act = d;
        e.rows_block = Mb;
        qkv_cache_params<T>(h, l, e);
        e.scratch_step = bt ? 0 : ATT_BLK;
        e.n_req = ctx.n_req;
        std::memcpy(e.ctx_first, ctx.ctx_first, sizeof e.ctx_first);
        e.col_offset = 0;
        if (fuse_ln) {
          FM_TRY(gemm_ln<T>(h, EPI_QKV, hres, mv + 0 * d, mv + 1 * d, act_qkv + (size_t)Mb * d, m_qkv - Mb,
                            blk(h, l, B_WQKV), 3 * d, d, e, st));
        } else {
          // block 0's rows come from the embedding; later ones were normalised by fc2's reduce
          if (!ln_in_reduce || l == 0) FM_TRY(ln_mod<T>(h, hres, Mb, mv + 0 * d, mv + 1 * d, act_qkv, d, st));
          FM_TRY(gemm<T>(h, EPI_QKV, act_qkv, d, m_qkv, blk(h, l, B_WQKV), 3 * d, d, e, st));
        }
      }
      {
        // the CUs attention leaves idle warm the L2s with W_o's tiles and
        // the first three quarters of each of fc1's groups (all of fc1
        // besides W_o would overflow a 4 MB L2 at d = 2048)
        L2Warm w{};
        if (l2_region(h, Mb, d, d, blk(h, l, B_WO), &w.reg[w.n_reg])) ++w.n_reg;
        if (fuse_ln && l2_region_ln(h, F, d, blk(h, l, B_W1), &w.reg[w.n_reg])) {
          w.reg[w.n_reg].take_u4 = w.reg[w.n_reg].group_u4 * 3 / 4;
          ++w.n_reg;
        }
        FM_TRY(attention<T>(h, l, B, nb_new, bt != nullptr, st, w));
      }
      {
        EpiParams e{};
        e.bias = blk(h, l, B_BO);
        e.out_f32 = hres;
        e.ld_f32 = d;
        e.gate = mv + 2 * d;
        e.ln_part = lnp;  // LN2, fused into fc1
        e.ln_part_ld = LN_PART_MAX;
        if (ln_in_reduce) {  // LN2 for fc1
          e.ln_shift = mv + 3 * d;
          e.ln_scale = mv + 4 * d;
          e.ln_out = act_d;
          e.ln_ldo = d;
        }
        FM_TRY(gemm<T>(h, EPI_RESID, attn_o, d, Mb, blk(h, l, B_WO), d, d, e, st));
      }
      {
        EpiParams e{};
        e.bias = blk(h, l, B_B1);
        e.out_act = act_f;
        e.ld_act = F;
        const int pk = (j == 0 && l == 0) ? FM_PROBE_FC1 : -1;
        if (fuse_ln) {
          FM_TRY(probe_begin(h, pk, st));
          FM_TRY(gemm_ln<T>(h, EPI_GELU, hres, mv + 3 * d, mv + 4 * d, nullptr, 0, blk(h, l, B_W1), F, d, e, st));
          FM_TRY(probe_end(h, pk, st));
        } else {
          if (!ln_in_reduce) FM_TRY(ln_mod<T>(h, hres, Mb, mv + 3 * d, mv + 4 * d, act_d, d, st));
          FM_TRY(probe_begin(h, pk, st));
          FM_TRY(gemm<T>(h, EPI_GELU, act_d, d, Mb, blk(h, l, B_W1), F, d, e, st));
          FM_TRY(probe_end(h, pk, st));
        }
      }
      {
        EpiParams e{};
        e.bias = blk(h, l, B_B2);
        e.out_f32 = hres;
        e.ld_f32 = d;
        e.gate = mv + 5 * d;
        e.ln_part = l + 1 < L ? lnp : nullptr;  // the next block's LN1, fused into its QKV
        e.ln_part_ld = LN_PART_MAX;
        if (ln_in_reduce) {  // the next block's LN1, or the final LN before the LM head
          const float* nm = mods + (size_t)6 * (l + 1) * d;
          e.ln_shift = nm;
          e.ln_scale = nm + d;
          e.ln_out = l + 1 < L ? act_qkv : act_d;
          e.ln_ldo = d;
        }
        FM_TRY(gemm<T>(h, EPI_RESID, act_f, F, Mb, blk(h, l, B_W2), d, F, e, st));
      }
      if (hidden) FM_TRY(trace_copy(hres, hidden + ((size_t)j * (L + 1) + l + 1) * Mb * d, (size_t)Mb * d, st));
    }
    const float* fin = mods + (size_t)6 * L * d;  // shift_f, scale_f
    if (!ln_in_reduce) FM_TRY(ln_mod<T>(h, hres, Mb, fin, fin + d, act_d, d, st));
    if (t == 1.f) {
      FM_TRY(lm_head<T>(h, act_d, Mb, logits, tokens, st, smp, FM_PROBE_LM_HEAD, adv));
    } else {
      FM_TRY(lm_head<T>(h, act_d, Mb, h->at<float>(h->lay.logits_tmp), nullptr, st));
      FM_TRY(softmax_rows<T>(h, Mb, st));
    }
  }
  return FM_OK;
}

template <typename T>
fm_status schedule_impl(fm_handle* h, int n_jumps, hipStream_t st) {
  const fm_config& c = h->cfg;
  const int d = c.d, L = c.L;
  float* feats = h->at<float>(h->lay.sched);             // [2*n][256]: feat(s_j), feat(t_j)
  float* hid_s = feats + (size_t)2 * c.max_steps * 256;  // [n][d]
  float* hid_t = hid_s + (size_t)c.max_steps * d;        // [n][d]
  float* cvec = hid_t + (size_t)c.max_steps * d;         // [n][d]
  float* mods = h->at<float>(h->lay.mods);               // [n][6L+2][d]
  for (int j = 0; j < n_jumps; ++j)
    for (int which = 0; which < 2; ++which) {
      hipLaunchKernelGGL(time_features_kernel, dim3(1), dim3(128), 0, st, h->times[j + which],
                         feats + (size_t)(2 * j + which) * 256);
      FM_LAUNCHED("time_features_kernel");
    }
  auto gv = [&](const float* in, int ldi, const void* Wp, const void* bp, int N, int K, float* out, int ldo,
                int in_silu, int out_silu, int acc) -> fm_status {
    hipLaunchKernelGGL((gemv_kernel<T>), dim3(cdiv(N, 4)), dim3(256), 0, st, in, ldi, n_jumps,
                       reinterpret_cast<const T*>(Wp), reinterpret_cast<const T*>(bp), N, K, out, ldo, in_silu,
                       out_silu, acc);
    FM_LAUNCHED("gemv_kernel");
    return FM_OK;
  };
  FM_TRY(gv(feats, 512, h->w.te_s_W1, h->w.te_s_b1, d, 256, hid_s, d, 0, 1, 0));
  FM_TRY(gv(feats + 256, 512, h->w.te_t_W1, h->w.te_t_b1, d, 256, hid_t, d, 0, 1, 0));
  FM_TRY(gv(hid_s, d, h->w.te_s_W2, h->w.te_s_b2, d, d, cvec, d, 0, 0, 0));
  FM_TRY(gv(hid_t, d, h->w.te_t_W2, h->w.te_t_b2, d, d, cvec, d, 0, 0, 1));
  const int per_jump = (6 * L + 2) * d;
  for (int l = 0; l < L; ++l)
    FM_TRY(gv(cvec, d, blk(h, l, B_WADA), blk(h, l, B_BADA), 6 * d, d, mods + (size_t)6 * l * d, per_jump, 1, 0, 0));
  FM_TRY(gv(cvec, d, h->w.W_fa, h->w.b_fa, 2 * d, d, mods + (size_t)6 * L * d, per_jump, 1, 0, 0));
  return FM_OK;
}

template <typename T>
fm_status verify_impl(const void* tl, int B, int K, int V, const int32_t* draft, int32_t* emitted, int32_t* accept,
                      int32_t* best, hipStream_t st) {
  hipLaunchKernelGGL((verify_argmax_kernel<T>), dim3(B * (K + 1)), dim3(1024), 0, st,
                     reinterpret_cast<const T*>(tl), V, emitted);
  FM_LAUNCHED("verify_argmax_kernel");
  hipLaunchKernelGGL(verify_prefix_kernel, dim3(1), dim3(64), 0, st, draft, B, K, emitted, accept, best);
  FM_LAUNCHED("verify_prefix_kernel");
  return FM_OK;
}

// greedy verification with VSL_SLICES workgroups per target row; the slice
// keys live in the handle's verifier scratch (its slice-state area, which
// holds at least VSL_SLICES 8-byte words per row)
template <typename T>
fm_status verify_sliced_impl(uint64_t* keys, const void* tl, int B, int K, int V, const int32_t* draft,
                             int32_t* emitted, int32_t* accept, int32_t* best, hipStream_t st) {
  static_assert(VS_MAX_SLICES >= VSL_SLICES, "slice keys overflow the verifier scratch");
  const int VE = (int)(16 / sizeof(T));
  const int slice = cdiv(cdiv(V, VSL_SLICES), VE) * VE;
  hipLaunchKernelGGL((verify_slice_kernel<T>), dim3(VSL_SLICES, B * (K + 1)), dim3(VSL_THREADS), 0, st,
                     reinterpret_cast<const T*>(tl), V, slice, keys);
  FM_LAUNCHED("verify_slice_kernel");
  hipLaunchKernelGGL(verify_merge_kernel, dim3(1), dim3(1024), 0, st, keys, VSL_SLICES, draft, B, K, emitted, accept,
                     best);
  FM_LAUNCHED("verify_merge_kernel");
  return FM_OK;
}

template <typename T>
fm_status verify_sample_impl(const VsScratch& sc, int V, const void* tl, int B, const float* Q, const float* lseQ,
                             const int32_t* draft, float tau, const BlockRng& rng, int32_t* emitted,
                             int32_t* accept, hipStream_t st) {
  VsArgs a{};
  a.T = tl;
  a.Q = Q;
  a.lseQ = lseQ;
  a.draft = draft;
  a.B = B;
  a.K = KB;
  a.V = V;
  a.S = std::min(VS_MAX_SLICES, cdiv(V, VS_SLICE));
  a.slice = cdiv(V, a.S);
  a.tau = tau;
  a.rng = rng;
  a.stats = sc.stats;
  a.lse_rows = sc.lse_rows;
  a.n_acc = sc.n_acc;
  a.keys = sc.keys;
  a.emitted = emitted;
  a.accept = accept;
  hipLaunchKernelGGL((vs_stats_kernel<T>), dim3(a.S, B * (KB + 1)), dim3(VS_THREADS), 0, st, a);
  FM_LAUNCHED("vs_stats_kernel");
  hipLaunchKernelGGL((vs_accept_kernel<T, KB + 1>), dim3(B), dim3(VS_ACCEPT_THREADS), 0, st, a);
  FM_LAUNCHED("vs_accept_kernel");
  hipLaunchKernelGGL((vs_keys_kernel<T>), dim3(a.S, B), dim3(VS_THREADS), 0, st, a);
  FM_LAUNCHED("vs_keys_kernel");
  hipLaunchKernelGGL(vs_final_kernel, dim3(B), dim3(64), 0, st, a);
  FM_LAUNCHED("vs_final_kernel");
  return FM_OK;
}

// argument checks shared by the two probabilistic verifiers
fm_status check_verify_sample(const void* target_logits, fm_dtype dtype, int B, const float* draft_logits,
                              const float* draft_lse, const int32_t* draft, float temperature, int32_t* emitted,
                              int32_t* accept) {
  if (!target_logits || !draft_logits || !draft_lse || !draft || !emitted || !accept)
    return fail(FM_EINVAL, "a pointer argument is NULL");
  if (dtype != FM_BF16 && dtype != FM_F32) return fail(FM_EINVAL, "dtype must be FM_BF16 or FM_F32");
  if (B < 1) return fail(FM_EINVAL, "B must be >= 1");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(FM_EINVAL, "temperature must be finite and > 0");
  if (reinterpret_cast<uintptr_t>(target_logits) % esize(dtype) || reinterpret_cast<uintptr_t>(draft_logits) % 4 ||
      reinterpret_cast<uintptr_t>(draft_lse) % 4)
    return fail(FM_EINVAL, "a logits array is not aligned to its element size");
  return FM_OK;
}

fm_status check_weights(const fm_config& c, const fm_weights* w) {
  if (!w) return fail(FM_EINVAL, "weights struct is NULL");
  const void* top[] = {w->E, w->W_lm, w->W_f, w->b_f, w->te_s_W1, w->te_s_b1, w->te_s_W2, w->te_s_b2,
                       w->te_t_W1, w->te_t_b1, w->te_t_W2, w->te_t_b2, w->W_fa, w->b_fa};
  const char* names[] = {"E", "W_lm", "W_f", "b_f", "te_s_W1", "te_s_b1", "te_s_W2", "te_s_b2",
                         "te_t_W1", "te_t_b1", "te_t_W2", "te_t_b2", "W_fa", "b_fa"};
  for (int i = 0; i < 14; ++i) {
    if (!top[i]) return fail(FM_EINVAL, "weight %s is NULL", names[i]);
    if (!aligned16(top[i])) return fail(FM_EINVAL, "weight %s is not 16-byte aligned", names[i]);
  }
  if (!w->blocks) return fail(FM_EINVAL, "blocks array is NULL");
  for (int l = 0; l < c.L; ++l) {
    const fm_block_weights& b = w->blocks[l];
    const void* p[] = {b.W_ada, b.b_ada, b.W_qkv, b.b_qkv, b.W_o, b.b_o, b.W_1, b.b_1, b.W_2, b.b_2};
    for (int i = 0; i < 10; ++i) {
      if (!p[i]) return fail(FM_EINVAL, "block %d weight %d is NULL", l, i);
      if (!aligned16(p[i])) return fail(FM_EINVAL, "block %d weight %d is not 16-byte aligned", l, i);
    }
  }
  return FM_OK;
}

}  // namespace

// =================================================================== C ABI
extern "C" {

size_t fm_workspace_bytes(const fm_config* cfg) {
  if (check_config(cfg) != FM_OK) return 0;
  return make_layout(*cfg).total;
}

fm_status fm_create(const fm_config* cfg, void* workspace, size_t ws_bytes, int device, fm_handle** out) {
  g_err.clear();
  FM_TRY(check_config(cfg));
  if (!out) return fail(FM_EINVAL, "out is NULL");
  if (!workspace) return fail(FM_EINVAL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(FM_EINVAL, "workspace is not 256-byte aligned");
  if (device < 0) return fail(FM_EINVAL, "device must be >= 0");
  Layout lay = make_layout(*cfg);
  if (ws_bytes < lay.total)
    return fail(FM_ECAPACITY, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, lay.total);
  fm_handle* h = new fm_handle();
  h->cfg = *cfg;
  h->device = device;
  h->ws = reinterpret_cast<char*>(workspace);
  h->lay = lay;
  int n_cu = 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && n_cu > 0)
    h->n_cu = n_cu;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(64), dim3(256), 0, 0, h->at<uint32_t>(lay.counters),
                     (size_t)N_COUNTER_SLOTS * COUNTER_STRIDE);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {  // empty contexts, overflow flag clear
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, 0, h->at<uint32_t>(lay.ctx), (size_t)FM_MAX_REQ + 1);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(0);
  if (e != hipSuccess) {
    delete h;
    return fail(FM_EHIP, "clearing the workspace counters: %s", hipGetErrorString(e));
  }
  *out = h;
  return FM_OK;
}

void fm_destroy(fm_handle* h) { delete h; }

fm_status fm_set_weights(fm_handle* h, const fm_weights* w) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  FM_TRY(check_weights(h->cfg, w));
  h->w = *w;
  h->blocks.assign(w->blocks, w->blocks + h->cfg.L);
  h->w.blocks = h->blocks.data();
  h->has_weights = true;
  return FM_OK;
}

fm_status fm_set_schedule(fm_handle* h, const float* times, int num_steps, void* stream) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  if (!times) return fail(FM_EINVAL, "times is NULL");
  if (num_steps < 1 || num_steps > h->cfg.max_steps)
    return fail(FM_EINVAL, "num_steps %d outside 1..%d", num_steps, h->cfg.max_steps);
  if (times[0] != 0.f || times[num_steps] != 1.f) return fail(FM_EINVAL, "schedule must start at 0 and end at 1");
  for (int j = 0; j < num_steps; ++j)
    if (!(times[j + 1] > times[j])) return fail(FM_EINVAL, "schedule must rise strictly");
  if (!h->has_weights) return fail(FM_ESTATE, "fm_set_schedule before fm_set_weights");
  for (int j = 0; j <= num_steps; ++j) h->times[j] = times[j];
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  fm_status s = h->cfg.dtype == FM_BF16 ? schedule_impl<bf16_t>(h, num_steps, st) : schedule_impl<float>(h, num_steps, st);
  if (s == FM_OK) h->n_steps = num_steps;
  return s;
}

fm_status fm_context_append_req(fm_handle* h, int req, const void* feats, int n, void* stream) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  if (req < 0 || req >= h->cfg.max_requests)
    return fail(FM_EINVAL, "request %d outside 0..%d", req, h->cfg.max_requests - 1);
  if (n < 0) return fail(FM_EINVAL, "n must be >= 0");
  if (n == 0) return FM_OK;
  if (!feats) return fail(FM_EINVAL, "feats is NULL");
  if (!aligned16(feats)) return fail(FM_EINVAL, "feats is not 16-byte aligned");
  if (!h->has_weights) return fail(FM_ESTATE, "fm_context_append before fm_set_weights");
  if (h->ctx_len[req] + n > h->cfg.C_max)
    return fail(FM_ECAPACITY, "context of %d rows + %d exceeds C_max %d", h->ctx_len[req], n, h->cfg.C_max);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  fm_status s = h->cfg.dtype == FM_BF16 ? context_append_impl<bf16_t>(h, req, feats, n, st)
                                        : context_append_impl<float>(h, req, feats, n, st);
  if (s == FM_OK) {
    h->ctx_len[req] += n;
    h->ctx_high[req] = std::max(h->ctx_high[req], h->ctx_len[req]);
  }
  return s;
}

fm_status fm_context_append(fm_handle* h, const void* feats, int n, void* stream) {
  return fm_context_append_req(h, 0, feats, n, stream);
}

fm_status fm_context_truncate_req(fm_handle* h, int req, int new_len, void* stream) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  if (req < 0 || req >= h->cfg.max_requests)
    return fail(FM_EINVAL, "request %d outside 0..%d", req, h->cfg.max_requests - 1);
  if (new_len < 0 || new_len > h->ctx_high[req])
    return fail(FM_EINVAL, "new length %d outside 0..%d (rows written so far)", new_len, h->ctx_high[req]);
  CtxUpdate u{};
  u.len = h->ctx_dev();
  u.first = req;
  u.count = 1;
  u.val[0] = new_len;
  u.set = 1;
  u.cap = h->cfg.C_max;
  FM_TRY(ctx_update_launch(u, reinterpret_cast<hipStream_t>(stream)));
  h->ctx_len[req] = new_len;
  return FM_OK;
}

fm_status fm_context_truncate(fm_handle* h, int new_len, void* stream) {
  return fm_context_truncate_req(h, 0, new_len, stream);
}

fm_status fm_context_sync(fm_handle* h, void* stream) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int dev[FM_MAX_REQ + 1];
  FM_HIP(hipMemcpyAsync(dev, h->ctx_dev(), sizeof dev, hipMemcpyDeviceToHost, st));
  FM_HIP(hipStreamSynchronize(st));
  for (int r = 0; r < h->cfg.max_requests; ++r) {
    h->ctx_len[r] = dev[r];
    h->ctx_high[r] = std::max(h->ctx_high[r], dev[r]);
  }
  if (dev[FM_MAX_REQ]) {
    CtxUpdate u{};  // clear the flag (the lengths stay at the capacity)
    u.len = h->ctx_dev() + FM_MAX_REQ;
    u.first = 0;
    u.count = 1;
    u.set = 1;
    u.cap = 0;
    FM_TRY(ctx_update_launch(u, st));
    return fail(FM_ECAPACITY, "an append on the device passed C_max %d: the rows past it were dropped",
                h->cfg.C_max);
  }
  return FM_OK;
}

int fm_context_length_req(const fm_handle* h, int req) {
  return h && req >= 0 && req < h->cfg.max_requests ? h->ctx_len[req] : -1;
}

int fm_context_length(const fm_handle* h) { return fm_context_length_req(h, 0); }

static fm_status draft_checked(fm_handle* h, const void* noise, int B, const void* new_feats, int n_new,
                               int32_t* tokens, float* logits, float* hidden, void* stream, const Sampling* smp) {
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  const fm_config& c = h->cfg;
  if (!noise || !tokens) return fail(FM_EINVAL, "noise and tokens must not be NULL");
  if (!aligned16(noise)) return fail(FM_EINVAL, "noise is not 16-byte aligned");
  if (B < 1) return fail(FM_EINVAL, "B must be >= 1");
  if (B > c.max_branches) return fail(FM_ECAPACITY, "B %d exceeds max_branches %d", B, c.max_branches);
  if (n_new < 0) return fail(FM_EINVAL, "n_new must be >= 0");
  if (n_new > c.max_new) return fail(FM_ECAPACITY, "n_new %d exceeds max_new %d", n_new, c.max_new);
  if (n_new > 0 && !new_feats) return fail(FM_EINVAL, "new_feats is NULL with n_new > 0");
  if (n_new > 0 && !aligned16(new_feats)) return fail(FM_EINVAL, "new_feats is not 16-byte aligned");
  if (h->ctx_len[0] + n_new > c.C_max)
    return fail(FM_ECAPACITY, "context of %d rows + %d exceeds C_max %d", h->ctx_len[0], n_new, c.C_max);
  if (!h->has_weights) return fail(FM_ESTATE, "fm_draft before fm_set_weights");
  if (h->n_steps < 1) return fail(FM_ESTATE, "fm_draft before fm_set_schedule");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  fm_status s = c.dtype == FM_BF16 ? draft_impl<bf16_t>(h, noise, B, new_feats, n_new, tokens, logits, hidden, st, smp)
                                   : draft_impl<float>(h, noise, B, new_feats, n_new, tokens, logits, hidden, st, smp);
  if (s == FM_OK) {
    h->ctx_len[0] += n_new;
    h->ctx_high[0] = std::max(h->ctx_high[0], h->ctx_len[0]);
  }
  return s;
}

static fm_status draft_batch_checked(fm_handle* h, const void* noise, int R, const void* new_feats,
                                     const int* n_new, int32_t* tokens, float* logits, void* stream,
                                     const Sampling* smp) {
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  const fm_config& c = h->cfg;
  if (!noise || !tokens) return fail(FM_EINVAL, "noise and tokens must not be NULL");
  if (!aligned16(noise)) return fail(FM_EINVAL, "noise is not 16-byte aligned");
  if (R < 1) return fail(FM_EINVAL, "R must be >= 1");
  if (R > c.max_requests) return fail(FM_ECAPACITY, "R %d exceeds max_requests %d", R, c.max_requests);
  Batch bt{};
  bt.R = R;
  int total = 0;
  for (int r = 0; r < R; ++r) {
    const int n = n_new ? n_new[r] : 0;
    if (n < 0) return fail(FM_EINVAL, "n_new[%d] must be >= 0", r);
    if (h->ctx_len[r] + n > c.C_max)
      return fail(FM_ECAPACITY, "request %d: context of %d rows + %d exceeds C_max %d", r, h->ctx_len[r], n,
                  c.C_max);
    bt.n_new[r] = n;
    total += n;
  }
  if (total > c.max_new) return fail(FM_ECAPACITY, "%d new context rows exceed max_new %d", total, c.max_new);
  if (total > 0 && !new_feats) return fail(FM_EINVAL, "new_feats is NULL with new rows");
  if (total > 0 && !aligned16(new_feats)) return fail(FM_EINVAL, "new_feats is not 16-byte aligned");
  if (!h->has_weights) return fail(FM_ESTATE, "fm_draft_batch before fm_set_weights");
  if (h->n_steps < 1) return fail(FM_ESTATE, "fm_draft_batch before fm_set_schedule");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  fm_status s = c.dtype == FM_BF16
                    ? draft_impl<bf16_t>(h, noise, R, new_feats, total, tokens, logits, nullptr, st, smp, &bt)
                    : draft_impl<float>(h, noise, R, new_feats, total, tokens, logits, nullptr, st, smp, &bt);
  if (s == FM_OK)
    for (int r = 0; r < R; ++r) {
      h->ctx_len[r] += bt.n_new[r];
      h->ctx_high[r] = std::max(h->ctx_high[r], h->ctx_len[r]);
    }
  return s;
}

fm_status fm_draft_batch(fm_handle* h, const void* noise, int R, const void* new_feats, const int* n_new,
                         int32_t* tokens, float* logits, void* stream) {
  g_err.clear();
  return draft_batch_checked(h, noise, R, new_feats, n_new, tokens, logits, stream, nullptr);
}

fm_status fm_draft_batch_sample(fm_handle* h, const void* noise, int R, const void* new_feats, const int* n_new,
                                float temperature, const uint64_t* seeds, int32_t* tokens, float* logits, float* lse,
                                void* stream) {
  g_err.clear();
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(FM_EINVAL, "temperature must be finite and > 0");
  if (!logits || !lse) return fail(FM_EINVAL, "logits and lse must not be NULL when sampling");
  if (!seeds) return fail(FM_EINVAL, "seeds is NULL");
  Sampling smp{temperature, 0, lse};
  smp.req_seeds = seeds;
  smp.R = R;
  return draft_batch_checked(h, noise, R, new_feats, n_new, tokens, logits, stream, &smp);
}

fm_status fm_draft(fm_handle* h, const void* noise, int B, const void* new_feats, int n_new, int32_t* tokens,
                   float* logits, float* hidden, void* stream) {
  g_err.clear();
  return draft_checked(h, noise, B, new_feats, n_new, tokens, logits, hidden, stream, nullptr);
}

fm_status fm_draft_sample(fm_handle* h, const void* noise, int B, const void* new_feats, int n_new,
                          float temperature, uint64_t seed, int32_t* tokens, float* logits, float* lse,
                          void* stream) {
  g_err.clear();
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(FM_EINVAL, "temperature must be finite and > 0");
  if (!logits || !lse) return fail(FM_EINVAL, "logits and lse must not be NULL when sampling");
  const Sampling smp{temperature, seed, lse};
  return draft_checked(h, noise, B, new_feats, n_new, tokens, logits, nullptr, stream, &smp);
}

fm_status fm_verify(const void* target_logits, fm_dtype dtype, int B, int K, int V, const int32_t* draft,
                    int32_t* emitted, int32_t* accept, int32_t* best, void* stream) {
  g_err.clear();
  if (!target_logits || !draft || !emitted || !accept || !best)
    return fail(FM_EINVAL, "a pointer argument is NULL");
  if (dtype != FM_BF16 && dtype != FM_F32) return fail(FM_EINVAL, "dtype must be FM_BF16 or FM_F32");
  if (B < 1 || B > 64) return fail(FM_EINVAL, "B must be in 1..64 (got %d)", B);
  if (K < 1 || K > 64) return fail(FM_EINVAL, "K must be in 1..64 (got %d)", K);
  if (V < 1) return fail(FM_EINVAL, "V must be >= 1");
  if (reinterpret_cast<uintptr_t>(target_logits) % esize(dtype))
    return fail(FM_EINVAL, "target_logits is not aligned to its element size");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return dtype == FM_BF16 ? verify_impl<bf16_t>(target_logits, B, K, V, draft, emitted, accept, best, st)
                          : verify_impl<float>(target_logits, B, K, V, draft, emitted, accept, best, st);
}

fm_status fm_verify_greedy(fm_handle* h, const void* target_logits, fm_dtype dtype, int B, const int32_t* draft,
                           int32_t* emitted, int32_t* accept, int32_t* best, void* stream) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  if (!target_logits || !draft || !emitted || !accept || !best)
    return fail(FM_EINVAL, "a pointer argument is NULL");
  if (dtype != FM_BF16 && dtype != FM_F32) return fail(FM_EINVAL, "dtype must be FM_BF16 or FM_F32");
  if (B < 1 || B > 64) return fail(FM_EINVAL, "B must be in 1..64 (got %d)", B);
  if (B > max_blocks(h->cfg))
    return fail(FM_ECAPACITY, "B %d exceeds the handle's %d row blocks", B, max_blocks(h->cfg));
  const int V = h->cfg.V;
  if (reinterpret_cast<uintptr_t>(target_logits) % esize(dtype))
    return fail(FM_EINVAL, "target_logits is not aligned to its element size");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the sliced kernels read whole 16-byte vectors: every row must start on a
  // 16-byte boundary; otherwise the one-workgroup-per-row path gives the same result
  const bool vec_ok = reinterpret_cast<uintptr_t>(target_logits) % 16 == 0 && ((size_t)V * esize(dtype)) % 16 == 0;
  if (!vec_ok)
    return dtype == FM_BF16 ? verify_impl<bf16_t>(target_logits, B, KB, V, draft, emitted, accept, best, st)
                            : verify_impl<float>(target_logits, B, KB, V, draft, emitted, accept, best, st);
  uint64_t* keys = reinterpret_cast<uint64_t*>(vs_scratch_at(h->at<char>(h->lay.vs), max_blocks(h->cfg), KB).stats);
  return dtype == FM_BF16 ? verify_sliced_impl<bf16_t>(keys, target_logits, B, KB, V, draft, emitted, accept, best, st)
                          : verify_sliced_impl<float>(keys, target_logits, B, KB, V, draft, emitted, accept, best, st);
}

fm_status fm_verify_sample(fm_handle* h, const void* target_logits, fm_dtype dtype, int B, const float* draft_logits,
                           const float* draft_lse, const int32_t* draft, float temperature, uint64_t seed,
                           int32_t* emitted, int32_t* accept, void* stream) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  FM_TRY(check_verify_sample(target_logits, dtype, B, draft_logits, draft_lse, draft, temperature, emitted, accept));
  if (B > max_blocks(h->cfg))
    return fail(FM_ECAPACITY, "B %d exceeds the handle's %d row blocks", B, max_blocks(h->cfg));
  const VsScratch sc = vs_scratch_at(h->at<char>(h->lay.vs), max_blocks(h->cfg), KB);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return dtype == FM_BF16 ? verify_sample_impl<bf16_t>(sc, h->cfg.V, target_logits, B, draft_logits, draft_lse,
                                                       draft, temperature, rng_shared(seed), emitted, accept, st)
                          : verify_sample_impl<float>(sc, h->cfg.V, target_logits, B, draft_logits, draft_lse,
                                                      draft, temperature, rng_shared(seed), emitted, accept, st);
}

fm_status fm_verify_sample_batch(fm_handle* h, const void* target_logits, fm_dtype dtype, int R,
                                 const float* draft_logits, const float* draft_lse, const int32_t* draft,
                                 float temperature, const uint64_t* seeds, int32_t* emitted, int32_t* accept,
                                 void* stream) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  if (!seeds) return fail(FM_EINVAL, "seeds is NULL");
  FM_TRY(check_verify_sample(target_logits, dtype, R, draft_logits, draft_lse, draft, temperature, emitted, accept));
  if (R > h->cfg.max_requests)
    return fail(FM_ECAPACITY, "R %d exceeds max_requests %d", R, h->cfg.max_requests);
  const VsScratch sc = vs_scratch_at(h->at<char>(h->lay.vs), max_blocks(h->cfg), KB);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const BlockRng rng = rng_per_request(seeds, R);
  return dtype == FM_BF16 ? verify_sample_impl<bf16_t>(sc, h->cfg.V, target_logits, R, draft_logits, draft_lse,
                                                       draft, temperature, rng, emitted, accept, st)
                          : verify_sample_impl<float>(sc, h->cfg.V, target_logits, R, draft_logits, draft_lse,
                                                      draft, temperature, rng, emitted, accept, st);
}

fm_status fm_verify_sample_noalloc(const void* target_logits, fm_dtype dtype, int B, int K, int V,
                                   const float* draft_logits, const float* draft_lse, const int32_t* draft,
                                   float temperature, uint64_t seed, int32_t* emitted, int32_t* accept,
                                   void* stream) {
  g_err.clear();
  FM_TRY(check_verify_sample(target_logits, dtype, B, draft_logits, draft_lse, draft, temperature, emitted, accept));
  if (K != KB) return fail(FM_EINVAL, "K must be 16 (got %d)", K);
  if (V < 1) return fail(FM_EINVAL, "V must be >= 1");
  if (B > NOALLOC_MAX_B || vs_scratch_bytes(B, K) > sizeof(scratch))
    return fail(FM_ECAPACITY, "B %d exceeds the %d branches the static scratch (%zu bytes) holds", B, NOALLOC_MAX_B,
                sizeof(scratch));
  char* base = nullptr;
  FM_TRY(scratch_ptr(&base));
  const VsScratch sc = vs_scratch_at(base, B, K);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return dtype == FM_BF16 ? verify_sample_impl<bf16_t>(sc, V, target_logits, B, draft_logits, draft_lse, draft,
                                                       temperature, rng_shared(seed), emitted, accept, st)
                          : verify_sample_impl<float>(sc, V, target_logits, B, draft_logits, draft_lse, draft,
                                                      temperature, rng_shared(seed), emitted, accept, st);
}

fm_status fm_set_probe(fm_handle* h, fm_probe_kernel kernel, void* ev_start, void* ev_stop) {
  g_err.clear();
  if (!h) return fail(FM_EINVAL, "handle is NULL");
  if (kernel < FM_PROBE_NONE || kernel > FM_PROBE_VERIFY) return fail(FM_EINVAL, "unknown probe kernel %d", (int)kernel);
  if (kernel != FM_PROBE_NONE && (!ev_start || !ev_stop)) return fail(FM_EINVAL, "probe events are NULL");
  h->probe = kernel;
  h->probe_start = reinterpret_cast<hipEvent_t>(ev_start);
  h->probe_stop = reinterpret_cast<hipEvent_t>(ev_stop);
  return FM_OK;
}

const char* fm_last_error(void) { return g_err.c_str(); }

}  // extern "C"
