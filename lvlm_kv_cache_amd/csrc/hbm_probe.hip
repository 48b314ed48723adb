// Bandwidth ceilings of one MI355X (gfx950) for the benchmark: a read-only
// stream, a device-to-device copy and an empty kernel (the gap between two
// back-to-back launches on one stream). Measurement tools, not part of the
// compression pass: the benchmark compares the pass with what these plain
// kernels reach on the same device.
//
// Both streaming kernels move 16-byte pieces, eight per thread in flight, over
// a grid-stride loop; the grid is a fixed multiple of the compute units so
// every CU keeps many loads outstanding.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// Reads n16 16-byte pieces; every thread folds what it read into one word,
// and a workgroup's words are written out so the loads cannot be dropped.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4_t *src, size_t n16, unsigned *sink) {
  const size_t stride = (size_t)gridDim.x * kThreads * kUnroll;
  unsigned acc = 0;
  for (size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16; base += stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4_t *src, u32x4_t *dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads * kUnroll;
  for (size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16; base += stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// Workgroups the streaming kernels launch: grid_per_cu per compute unit.
// sink must hold grid * 256 unsigned words (hbm_probe_sink_words).
int hbm_probe_grid(int grid_per_cu) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus * (grid_per_cu > 0 ? grid_per_cu : 1);
}

size_t hbm_probe_sink_words(int grid) { return (size_t)grid * kThreads; }

// Read `bytes` (a multiple of 16, 16-byte aligned) from device memory src.
int hbm_probe_read(const void *src, size_t bytes, unsigned *sink, int grid, void *stream) {
  if (!src || !sink || grid < 1 || (bytes & 15u) || ((uintptr_t)src & 15u)) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t *>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned, no overlap).
int hbm_probe_copy(const void *src, void *dst, size_t bytes, int grid, void *stream) {
  if (!src || !dst || grid < 1 || (bytes & 15u) || (((uintptr_t)src | (uintptr_t)dst) & 15u)) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t *>(src), static_cast<u32x4_t *>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// One launch of a kernel that does nothing (one workgroup of one wave).
int hbm_probe_empty(void *stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
