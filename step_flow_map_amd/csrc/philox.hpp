// Counter-based random numbers for temperature > 0 drafting and verification.
//
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds over a 128-bit counter (c0..c3) under
// a 64-bit key (k0, k1).  A round multiplies c0 and c2 by two fixed odd
// constants; the new state is (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1),
// hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)), and the key advances by two Weyl constants
// before every round after the first.
//
// Counter convention: (v, row, branch, stream), key = the caller's 64-bit
// seed; word 0 of the output is the draw.  Streams: 0 Gumbel noise of draft
// sampling, 1 Gumbel noise of the residual / bonus sample, 2 acceptance
// uniforms.  A draw x stands for U = (x + 0.5) / 2^32 in (0, 1).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

constexpr uint32_t PHILOX_M0 = 0xD2511F53u, PHILOX_M1 = 0xCD9E8D57u;
constexpr uint32_t PHILOX_W0 = 0x9E3779B9u, PHILOX_W1 = 0xBB67AE85u;
constexpr uint32_t RNG_DRAFT = 0, RNG_CORRECT = 1, RNG_ACCEPT = 2;

__device__ __forceinline__ uint32_t philox_x0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    const uint32_t lo0 = c0 * PHILOX_M0, hi0 = __umulhi(c0, PHILOX_M0);
    const uint32_t lo1 = c2 * PHILOX_M1, hi1 = __umulhi(c2, PHILOX_M1);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

// Gumbel noise -log(-log U) for the draw x, with E = -log U evaluated on the
// side where it keeps its relative precision in float32: log of (x + 0.5)
// scaled by 2^-32 for the lower half of the range, log1p of -(1 - U) for the
// upper half (where 1 - U is small and U itself would round to 1).
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  float e;
  if (x < 0x80000000u) {
    e = 22.18070977791825f - logf((float)x + 0.5f);  // 32 ln 2 - ln(x + 0.5)
  } else {
    const float one_minus_u = ((float)(0xFFFFFFFFu - x) + 0.5f) * 2.3283064365386963e-10f;  // 2^-32
    e = -log1pf(-one_minus_u);
  }
  return -logf(e);
}

// Key and branch word of row block b.  The branches of one draft share the
// caller's seed and differ in the branch word (the block index); the requests
// of a batch each bring their own seed and draw with branch word 0, exactly
// as each would drafted or verified alone.
struct BlockRng {
  uint32_t lo[4], hi[4];  // per request (per_request), else entry 0 for every block
  int per_request;
};
__device__ __forceinline__ void block_rng(const BlockRng& r, int b, uint32_t& k0, uint32_t& k1, uint32_t& bw) {
  if (!r.per_request) {
    k0 = r.lo[0];
    k1 = r.hi[0];
    bw = (uint32_t)b;
    return;
  }
  // selects, not a runtime index into the argument block
  k0 = b == 0 ? r.lo[0] : b == 1 ? r.lo[1] : b == 2 ? r.lo[2] : r.lo[3];
  k1 = b == 0 ? r.hi[0] : b == 1 ? r.hi[1] : b == 2 ? r.hi[2] : r.hi[3];
  bw = 0u;
}

// Uniform in (0, 1) from the top 24 bits of the draw (exact in float32).
__device__ __forceinline__ float uniform_of(uint32_t x) { return ((float)(x >> 8) + 0.5f) * 5.9604644775390625e-8f; }

}  // namespace fm
