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
// are warmed
struct L2Region {
  const uint4* base;
  size_t group_u4, off_u4, take_u4;
  int n_groups;
};
constexpr int L2W_REGIONS = 2;

struct L2Warm {
  L2Region reg[L2W_REGIONS];
  int n_reg;     // 0: no warming workgroups
  int first_wg;  // blockIdx of this launch's first warming workgroup
  int n_wg;      // warming workgroups, a multiple of 8 (n_wg / 8 per XCD)
};

constexpr int L2W_UNROLL = 8;  // loads in flight per thread and round

// Warming workgroup blk (first_wg <= blk < first_wg + n_wg): its share of
// every region's groups on its own XCD, read by all nthreads threads.
__device__ __forceinline__ void l2_warm(const L2Warm& w, int blk, int nthreads) {
  const int x = blk & 7;                                   // this workgroup's XCD
  const int r = (blk - w.first_wg) >> 3, R = w.n_wg >> 3;  // rank among the XCD's warmers
  uint32_t acc = 0;
  for (int q = 0; q < w.n_reg && q < L2W_REGIONS; ++q) {
    const L2Region& g = w.reg[q];
    if (x >= g.n_groups) continue;
    const size_t total = (size_t)((g.n_groups - 1 - x) / 8 + 1) * g.take_u4;  // words of this XCD
    const size_t per = (total + R - 1) / R;
    const size_t lo = (size_t)r * per, hi = min(total, lo + per);
    for (size_t i0 = lo + threadIdx.x; i0 < hi; i0 += (size_t)L2W_UNROLL * nthreads) {
      uint4 v[L2W_UNROLL];
#pragma unroll
      for (int u = 0; u < L2W_UNROLL; ++u) {
        const size_t i = min(i0 + (size_t)u * nthreads, hi - 1);  // clamped: the last word again
        const size_t gi = i / g.take_u4, o = i % g.take_u4;
        v[u] = g.base[(x + 8 * gi) * g.group_u4 + g.off_u4 + o];
      }
#pragma unroll
      for (int u = 0; u < L2W_UNROLL; ++u) acc ^= v[u].x;
    }
  }
  // keep the loads: the folded value is an operand of an empty asm statement
  asm volatile("" ::"v"(acc));
}

}  // namespace fm
