// Warming each XCD's L2 with the weights the next contractions will read there.
//
// Workgroups of a launch are dispatched round robin over the chip's 8 XCDs
// (workgroup i on XCD i % 8), and each XCD has its own L2.  A contraction
// whose workgroup b reads one contiguous tile group b of its weight matrix
// (no k split) therefore reads, on XCD x, exactly the groups b = x, x + 8, ...
// A launch that leaves most CUs idle (attention: a few dozen workgroups) can
// carry extra workgroups that read those groups on the same XCDs first, so
// that the next launch finds its weights in L2 rather than in HBM.  The reads
// change no memory; their values are folded and discarded.
#pragma once
#include "common.hpp"

namespace fm {

// the tile groups of one later launch: group b (read by its workgroup b) at
// base + b * group_u4, of which the 16-byte words off_u4 .. off_u4 + take_u4
// are warmed.  slices > 0: workgroup b = g * slices + s instead reads rows
// g * rows .. + rows of a matrix with rows of row_u4 words, words s * take_u4
// .. + take_u4 of each (a k slice of a row group; n_groups = row groups).
struct L2Region {
  const uint4* base;
  size_t group_u4, off_u4, take_u4;
  int n_groups;
  int slices, rows;
  size_t row_u4;
};
constexpr int L2W_REGIONS = 2;

struct L2Warm {
  L2Region reg[L2W_REGIONS];
  int n_reg;     // 0: no warming workgroups
  int first_wg;  // blockIdx of this launch's first warming workgroup
  int n_wg;      // warming workgroups, a multiple of 8 (n_wg / 8 per XCD)
};

constexpr int L2W_UNROLL = 8;  // loads in flight per thread and round
enum { L2W_NONE = 0, L2W_TILES = 1, L2W_SLICES = 2 };  // region kinds (compiled separately)

// words lo .. hi of one region on XCD x, word i at addr(i); folded into acc
template <typename Addr>
__device__ __forceinline__ void l2_warm_range(size_t lo, size_t hi, int nthreads, uint32_t& acc, Addr addr) {
  for (size_t i0 = lo + threadIdx.x; i0 < hi; i0 += (size_t)L2W_UNROLL * nthreads) {
    uint4 v[L2W_UNROLL];
#pragma unroll
    for (int u = 0; u < L2W_UNROLL; ++u) v[u] = *addr(min(i0 + (size_t)u * nthreads, hi - 1));  // clamped
#pragma unroll
    for (int u = 0; u < L2W_UNROLL; ++u) acc ^= v[u].x;
  }
}

// Warming workgroup blk (first_wg <= blk < first_wg + n_wg): its share of
// every region's words on its own XCD, read by all nthreads threads.  KIND:
// the regions' kind (L2W_TILES: tile groups, slices = 0; L2W_SLICES: k slices).
template <int KIND>
__device__ __forceinline__ void l2_warm(const L2Warm& w, int blk, int nthreads) {
  const int x = blk & 7;                                   // this workgroup's XCD
  const int r = (blk - w.first_wg) >> 3, R = w.n_wg >> 3;  // rank among the XCD's warmers
  uint32_t acc = 0;
  for (int q = 0; q < w.n_reg && q < L2W_REGIONS; ++q) {
    const L2Region& g = w.reg[q];
    const int nb = KIND == L2W_SLICES ? g.n_groups * g.slices : g.n_groups;  // workgroups of the later launch
    if (x >= nb) continue;
    const size_t per_b = KIND == L2W_SLICES ? (size_t)g.rows * g.take_u4 : g.take_u4;  // words of one
    const size_t total = (size_t)((nb - 1 - x) / 8 + 1) * per_b;                    // words of this XCD
    const size_t per = (total + R - 1) / R;
    const size_t lo = (size_t)r * per, hi = min(total, lo + per);
    if constexpr (KIND == L2W_SLICES) {
      l2_warm_range(lo, hi, nthreads, acc, [&](size_t i) {
        const size_t bj = i / per_b, rem = i % per_b;
        const int b = x + 8 * (int)bj, gg = b / g.slices, ss = b % g.slices;
        const size_t row = (size_t)gg * g.rows + rem / g.take_u4, col = ss * g.take_u4 + rem % g.take_u4;
        return g.base + row * g.row_u4 + col;
      });
    } else {
      l2_warm_range(lo, hi, nthreads, acc, [&](size_t i) {
        const size_t gi = i / g.take_u4, o = i % g.take_u4;
        return g.base + (x + 8 * gi) * g.group_u4 + g.off_u4 + o;
      });
    }
  }
  // keep the loads: the folded value is an operand of an empty asm statement
  asm volatile("" ::"v"(acc));
}

}  // namespace fm
