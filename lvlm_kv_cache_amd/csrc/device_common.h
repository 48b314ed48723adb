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

// Cross-lane moves by DPP (no LDS round trip). CTRL: 0xB1 quad_perm
// [1,0,3,2] (lane ^ 1), 0x4E quad_perm [2,3,0,1] (lane ^ 2), 0x141 row half
// mirror (lane i of each 8-lane half from lane 7 - i), 0x140 row mirror (lane
// i of each 16-lane row from lane 15 - i).
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL> __device__ __forceinline__ double dpp_d(double v) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(x >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Reductions over the 16 lanes of a DPP row; every lane of the row receives
// the same bits (each step combines a lane with its mirror partner, and the
// operations are commutative).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return fmaxf(v, dpp_f<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}
__device__ __forceinline__ double row16_sum_d(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x141>(v);
  return v + dpp_d<0x140>(v);
}

// Sum over the four 16-lane rows (lanes n, n + 16, n + 32, n + 48) with the
// gfx950 row-swap permutes; every lane receives (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float sum_across_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)x, l), hi = __builtin_amdgcn_readlane((int)(x >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Whole-wave reductions: rows first, then the four row results in a fixed
// order; the result is wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ double wave_sum_d(double v) {
  v = row16_sum_d(v);
  return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
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
// Agent-coherent loads that the compiler may batch like ordinary loads: buffer
// loads with the sc1 cache policy through a raw buffer resource (gfx9 family
// resource word 3; out-of-range offsets read as 0). They observe values
// published with store_coherent without invalidating the L2.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float load_sc1_f(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 16));
}
__device__ __forceinline__ int load_sc1_i(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 16);
}
__device__ __forceinline__ double load_sc1_d(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 16));
}

// Acquire at device scope: after it, ordinary loads observe every value that
// another workgroup published with store_coherent before its counter update
// (invalidates this CU's L1 and the XCD's non-coherent L2 lines). Used once
// per elected finisher, so its reads can be ordinary, batched loads instead
// of one atomic load at a time.
__device__ __forceinline__ void acquire_device() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ void store_nt(u32x4_t *p, u32x4_t v) { __builtin_nontemporal_store(v, p); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (vector memory operations complete in issue order). Also a compiler memory
// fence, so no LDS access is moved across it.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Wait until every LDS access of this wave has completed (before an LDS-DMA
// load overwrites a region the wave just read); also a compiler memory fence.
__device__ __forceinline__ void wait_lds_reads() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt, expcnt at maximum; lgkmcnt 0
  asm volatile("" ::: "memory");
}

// wait_vmcnt<t * PER>() for a count t in 0..3 known after unrolling.
template <int PER> __device__ __forceinline__ void wait_tiles(int t) {
  switch (t) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PER>(); break;
    case 2: wait_vmcnt<2 * PER>(); break;
    case 3: wait_vmcnt<3 * PER>(); break;
    case 4: wait_vmcnt<(4 * PER < 63 ? 4 * PER : 63)>(); break;
    case 5: wait_vmcnt<(5 * PER < 63 ? 5 * PER : 63)>(); break;
    case 6: wait_vmcnt<(6 * PER < 63 ? 6 * PER : 63)>(); break;
    default: wait_vmcnt<(7 * PER < 63 ? 7 * PER : 63)>(); break;
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS-DMA: every lane copies 16 bytes from its own global address to
// lds + 16 * lane (gfx950 global_load_lds_dwordx4). lds must be wave-uniform.
__device__ __forceinline__ void load_lds16(const void *gsrc, void *lds) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t *)lds, 16, 0, 0);
}

// Staging of one 16-key tile in LDS for MFMA B operands. DMA instruction j
// (j < 16 * row_bytes / 1024) moves, for lane i, bytes [16 (i / 16) + 64 j,
// +16) of key row i % 16 to tile + 1024 j + 16 i. The fragment of lane
// (n = lane % 16, grp = lane / 16) for 32-element slice c is then read back as
// whole 16-byte pieces.
template <typename Tag> struct LdsTile;

template <> struct LdsTile<Bf16Tag> {
  // slice c of row n is bytes [64 c + 16 grp, +16): DMA j = c, lane group grp
  __device__ static __forceinline__ void read(Frag<Bf16Tag> &f, const unsigned char *tile, int c, int lane) {
    f.v = *reinterpret_cast<const u16x8_t *>(tile + 1024 * c + 16 * lane);
  }
};

template <> struct LdsTile<F32Tag> {
  // slice c of row n is bytes [128 c + 32 grp, +32): DMA j = 2c + grp / 2,
  // lane groups 2 (grp % 2) and 2 (grp % 2) + 1
  __device__ static __forceinline__ void read(Frag<F32Tag> &f, const unsigned char *tile, int c, int lane) {
    const int n = lane & 15, grp = lane >> 4;
    const unsigned char *b = tile + 1024 * (2 * c + (grp >> 1)) + 16 * (32 * (grp & 1) + n);
    f.lo = *reinterpret_cast<const f32x4_t *>(b);
    f.hi = *reinterpret_cast<const f32x4_t *>(b + 256);
  }
};

}  // namespace aircache
