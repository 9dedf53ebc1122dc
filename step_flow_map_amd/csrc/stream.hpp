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
// The A operand of step s must use the same k; activation rows are staged
// through the same tile layout (chunk_load_act), so both operands come from
// coalesced loads.
#pragma once
#include "common.hpp"

namespace fm {

// 16-byte load of data read exactly once (weights): nontemporal hint
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <typename T>
struct ChunkT {
  static constexpr int VE = Vec<T>::N;
  static constexpr int KC = 32 * VE;  // k elements per chunk
};

// Load the chunk of rows n0..n0+15 and columns k0..k0+KC-1.  Addresses are
// clamped into the matrix (rows >= N read row 0, columns >= K read column 0),
// never masked here: a select on a loaded value would make the wave wait for
// that load right away and defeat the prefetch.  Rows >= N only feed output
// columns that are never stored, and columns >= K meet A values that the
// consumer zeroes, so the clamped data never reaches a result.
// live = false: every lane reads the matrix's first 16 bytes (one line per
// instruction), a placeholder for a chunk that does not exist.
template <typename T>
__device__ __forceinline__ void chunk_load(uint4 (&r)[8], const T* W, size_t ldw, int n0, int N, int k0, int K,
                                           bool live = true) {
  constexpr int VE = ChunkT<T>::VE;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, p = lane & 31;
  const int kk = k0 + p * VE;
  const int kc = live && kk < K ? kk : 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = n0 + 2 * i + half;
    r[i] = ldg_stream(W + (size_t)(live && row < N ? row : 0) * ldw + kc);
  }
}

// The same pattern for activation rows r0.. of A (R rows, row stride lda),
// with ordinary cached loads: every workgroup reads the same A.  Rows >= R
// read row 0 and columns >= K read column 0 (both masked by the consumer).
template <typename T>
__device__ __forceinline__ void chunk_load_act(uint4 (&r)[8], const T* A, size_t lda, int r0, int R, int k0, int K,
                                               bool live = true) {
  constexpr int VE = ChunkT<T>::VE;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, p = lane & 31;
  const int kk = k0 + p * VE;
  const int kc = live && kk < K ? kk : 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r0 + 2 * i + half;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(A + (size_t)(live && row < R ? row : 0) * lda + kc);
    r[i] = make_uint4(v[0], v[1], v[2], v[3]);
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
