// Device helpers shared by the FlashMap kernels (gfx950 / CDNA4).
//
// Storage types: bf16 (uint16_t bit patterns) or float.  Every contraction
// accumulates in float32.  Operands travel as 16-byte vectors ("vec"): 8 bf16
// or 4 floats per lane; one vec pair feeds one v_mfma_f32_16x16x32_bf16, or
// four v_mfma_f32_16x16x4_f32.
//
// MFMA 16x16 layouts used throughout (wave64, lane l, group g = l / 16):
//   A operand: row (l % 16), a run of k values owned by group g
//   B operand: column (l % 16), the same run of k values
//   D (f32x4): rows 4*g + i (i = 0..3), column (l % 16)
// Any assignment of k values to (group, element) is valid as long as A and B
// use the same one, so loaders give each lane contiguous k runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

constexpr int FM_MAX_REQ = 4;  // requests with their own context in one launch

typedef uint16_t bf16_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct Vec;
template <> struct Vec<bf16_t> {
  typedef uint4 type;
  static constexpr int N = 8;
};
template <> struct Vec<float> {
  typedef float4 type;
  static constexpr int N = 4;
};

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

template <typename V> __device__ __forceinline__ V vzero();
template <> __device__ __forceinline__ uint4 vzero<uint4>() { return make_uint4(0, 0, 0, 0); }
template <> __device__ __forceinline__ float4 vzero<float4>() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// VE floats rounded to the storage type and packed into a vec
template <typename T> __device__ __forceinline__ typename Vec<T>::type pack_vec(const float (&y)[Vec<T>::N]);
template <> __device__ __forceinline__ uint4 pack_vec<bf16_t>(const float (&y)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(y[2 * i]) | ((uint32_t)f32_to_bf16(y[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
template <> __device__ __forceinline__ float4 pack_vec<float>(const float (&y)[4]) {
  return make_float4(y[0], y[1], y[2], y[3]);
}

// the VE values of a vec as floats
__device__ __forceinline__ void unpack_vec(uint4 v, float (&y)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = __uint_as_float(w[i] << 16);
    y[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack_vec(float4 v, float (&y)[4]) {
  y[0] = v.x;
  y[1] = v.y;
  y[2] = v.z;
  y[3] = v.w;
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes go to
// lds_base + 16 i (lds_base must be the same for the whole wave).  Completion
// is counted like a vector load, and the compiler waits for all outstanding
// vector loads before any LDS read that follows, so this pays where nothing
// else needs to stay in flight.  For data already in L2 it moves several times
// more bytes per CU than loads into registers.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

// v if keep, else zero, without a branch or a select on the vector
__device__ __forceinline__ uint4 vkeep(uint4 v, bool keep) {
  const uint32_t m = keep ? ~0u : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}
__device__ __forceinline__ float4 vkeep(float4 v, bool keep) {
  const uint32_t m = keep ? ~0u : 0u;
  return make_float4(__uint_as_float(__float_as_uint(v.x) & m), __uint_as_float(__float_as_uint(v.y) & m),
                     __uint_as_float(__float_as_uint(v.z) & m), __uint_as_float(__float_as_uint(v.w) & m));
}

template <typename T>
__device__ __forceinline__ typename Vec<T>::type vload(const T* p) {
  return *reinterpret_cast<const typename Vec<T>::type*>(p);
}

// acc += A_run . B_run over the k values held by this lane's group
__device__ __forceinline__ void mma(f32x4& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, float4 a, float4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
}

// element e of a vec as float
__device__ __forceinline__ float velem(uint4 v, int e) {
  uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return bf16_to_f32((bf16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu)));
}
__device__ __forceinline__ float velem(float4 v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// Transpose a VxV block held as V row vectors in[r] (r = k index, element t =
// column) into V column vectors out[t] (element r = k index).
// Each output word takes one bf16 from each of two input words: one byte
// permute (v_perm_b32: bytes 0-3 of the second operand, 4-7 of the first).
__device__ __forceinline__ void transpose_block(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4& a = in[2 * p];
      const uint4& b = in[2 * p + 1];
      uint32_t wa = (t >> 1) == 0 ? a.x : (t >> 1) == 1 ? a.y : (t >> 1) == 2 ? a.z : a.w;
      uint32_t wb = (t >> 1) == 0 ? b.x : (t >> 1) == 1 ? b.y : (t >> 1) == 2 ? b.z : b.w;
      // even t: low halves (wa.lo, wb.lo); odd t: high halves (wa.hi, wb.hi)
      w[p] = __builtin_amdgcn_perm(wb, wa, (t & 1) ? 0x07060302u : 0x05040100u);
    }
    out[t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}
__device__ __forceinline__ void transpose_block(const float4 (&in)[4], float4 (&out)[4]) {
  out[0] = make_float4(in[0].x, in[1].x, in[2].x, in[3].x);
  out[1] = make_float4(in[0].y, in[1].y, in[2].y, in[3].y);
  out[2] = make_float4(in[0].z, in[1].z, in[2].z, in[3].z);
  out[3] = make_float4(in[0].w, in[1].w, in[2].w, in[3].w);
}

// ---------------------------------------------------------------- argmax keys
// Order-preserving 64-bit key: larger value wins, then the lower index.
// -0 and +0 map to the same key (they compare equal).
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t argmax_key_index(uint64_t key) {
  return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, mask, 64);
  hi = __shfl_xor(hi, mask, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ------------------------------------------------------- cross-workgroup sync
// Data one workgroup hands to another inside a launch is written with
// device-coherent stores and read with device-coherent loads (agent-scope
// relaxed atomics: they write through / bypass the XCD-local L2), so no L2
// writeback or invalidate is needed.  arrive() waits until this workgroup's
// coherent stores are acknowledged, then bumps `counter`; the workgroup that
// brings it to `expected` gets true and resets it to zero for the next launch.
// A device-scope atomic on one address costs a few hundred ns and serialises,
// so every counter is given only a handful of arrivals.
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coh(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool arrive(uint32_t* counter, uint32_t expected, int* lds_flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): coherent stores acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == expected - 1;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// ------------------------------------------------ row statistics of 16 lanes
// DPP move within a row of 16 lanes (no LDS traffic)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row: neighbours 1 and 2 (quad permutes), then
// the mirrored half and the mirrored row.  Every step adds two equal-order
// partial sums of symmetric partners, so all 16 lanes end with the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}
// A row's statistics over 16 consecutive columns, held one per lane by the 16
// lanes of a DPP row (every lane of the wave calls this): mean and sum of
// squared deviations, two passes; the row's first lane stores them when ok.
__device__ __forceinline__ void row16_stats(float x, bool ok, float2* dst) {
  const float mean = row16_sum(x) * 0.0625f;
  const float dv = x - mean;
  const float m2 = row16_sum(dv * dv);
  if (ok && (threadIdx.x & 15) == 0) *dst = make_float2(mean, m2);
}

// counters live 32 words (128 bytes) apart so contended lines never share
constexpr int COUNTER_STRIDE = 32;

// Ordering point between a wave's LDS writes and its reads of other lanes'
// data.  The LDS executes one wave's accesses in order, so the hardware needs
// no wait; the wavefront-scope fence keeps the compiler from moving LDS
// accesses across this point (it emits no instruction and, unlike a
// workgroup-scope fence, waits for no outstanding global load), and the wave
// barrier keeps the scheduler from doing so.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also waits
// for every outstanding global load of the wave, which would drain loads that
// are meant to stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.f + tanhf(k0 * (x + 0.044715f * x * x * x)));
}
__device__ __forceinline__ float silu(float x) { return x / (1.f + expf(-x)); }

}  // namespace fm
