// Streaming weight chunks into MFMA B operands.
//
// A chunk is 16 weight rows x KC = 32*VE elements (512 bytes per row, 8 KB).
// MFMA wants lanes 0..15 on 16 different rows, which would make every global
// load touch 16 rows at once; instead each load instruction covers two rows x
// 512 contiguous bytes (lanes 0-31 row 2i, lanes 32-63 row 2i+1, 16-byte piece
// p = lane & 31), the wave writes the chunk into its own LDS tile with piece p
// of row r at slot r*32 + (p ^ r) (the XOR keeps the fragment reads free of
// bank conflicts), and reads MFMA fragments back: step s (0..7) gives lane
// (j, g) piece 4s+g of row j, i.e. k = (4s+g)*VE .. +VE-1 of weight row j.
// The A operand of step s must use the same k.
#pragma once
#include "common.hpp"

namespace fm {

template <typename T>
struct ChunkT {
  static constexpr int VE = Vec<T>::N;
  static constexpr int KC = 32 * VE;  // k elements per chunk
};

// Load the chunk of rows n0..n0+15 (rows >= N read as zero) and columns
// k0..k0+KC-1 (columns >= K read as zero; K is a multiple of VE).  Loads are
// unconditional from clamped, valid addresses; the value is then selected.
template <typename T>
__device__ __forceinline__ void chunk_load(uint4 (&r)[8], const T* W, size_t ldw, int n0, int N, int k0, int K) {
  constexpr int VE = ChunkT<T>::VE;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, p = lane & 31;
  const int kk = k0 + p * VE;
  const bool kok = kk < K;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = n0 + 2 * i + half;
    const bool ok = kok && row < N;
    const T* ptr = W + (size_t)(ok ? row : 0) * ldw + (ok ? kk : 0);
    const uint4 v = *reinterpret_cast<const uint4*>(ptr);
    r[i] = ok ? v : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void chunk_to_lds(const uint4 (&r)[8], uint4* tile) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, p = lane & 31;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 2 * i + half;
    tile[row * 32 + (p ^ row)] = r[i];
  }
}

// fragment of MFMA step s for this lane: row (lane & 15), piece 4s + (lane >> 4)
__device__ __forceinline__ uint4 chunk_frag(const uint4* tile, int s) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  return tile[j * 32 + ((4 * s + g) ^ j)];
}

template <typename T> __device__ __forceinline__ typename Vec<T>::type as_vec(uint4 v);
template <> __device__ __forceinline__ uint4 as_vec<bf16_t>(uint4 v) { return v; }
template <> __device__ __forceinline__ float4 as_vec<float>(uint4 v) {
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

}  // namespace fm
