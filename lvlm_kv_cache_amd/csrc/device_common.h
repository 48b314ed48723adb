// Device helpers shared by the gfx950 kernels of the AirCache pass: MFMA
// operand fragments, wave reductions and agent-coherent loads/stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aircache {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) unsigned short u16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

constexpr int kWave = 64;

// Element tags: the kernels are templated on the storage type of Q/K/V.
struct Bf16Tag {
  using store_t = uint16_t;
  static constexpr int kBytes = 2;
};
struct F32Tag {
  using store_t = float;
  static constexpr int kBytes = 4;
};

// One MFMA operand fragment: 8 consecutive elements of a row (a 32-wide slice
// of the contraction dimension is split over the 4 lane groups of 16 lanes).
template <typename Tag> struct Frag;

template <> struct Frag<Bf16Tag> {
  u16x8_t v;
  __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const u16x8_t *>(p); }
  __device__ __forceinline__ void zero() { v = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0}; }
};

template <> struct Frag<F32Tag> {
  f32x4_t lo, hi;
  __device__ __forceinline__ void load(const float *p) {
    lo = *reinterpret_cast<const f32x4_t *>(p);
    hi = *reinterpret_cast<const f32x4_t *>(p + 4);
  }
  __device__ __forceinline__ void zero() {
    lo = f32x4_t{0.f, 0.f, 0.f, 0.f};
    hi = lo;
  }
};

// acc[i] += sum over the 32-wide slice of A[m][k] * B[k][n] with m the A row
// held by lane group (lane / 16) * 4 + i and n = lane % 16 (gfx950 layout of
// the 16x16 f32 result).
__device__ __forceinline__ void mfma_slice(f32x4_t &acc, const Frag<Bf16Tag> &a, const Frag<Bf16Tag> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                __builtin_bit_cast(bf16x8_t, b.v), acc, 0, 0, 0);
}

__device__ __forceinline__ void mfma_slice(f32x4_t &acc, const Frag<F32Tag> &a, const Frag<F32Tag> &b) {
  // The same 32-wide slice as eight K=4 steps: step s contracts element s of
  // every lane's 8-element run, identically in A and B.
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Agent-coherent scalar accesses for values exchanged between workgroups of
// one launch: relaxed device-scope atomics compile to sc1 loads/stores, which
// the MI355X memory model makes coherent across XCDs without a full L2
// write-back. Ordering is obtained by waiting for completion (s_waitcnt)
// before the counter update that publishes them.
template <typename T> __device__ __forceinline__ void store_coherent(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T> __device__ __forceinline__ T load_coherent(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned counter_add(unsigned *p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ void store_nt(u32x4_t *p, u32x4_t v) { __builtin_nontemporal_store(v, p); }

}  // namespace aircache
