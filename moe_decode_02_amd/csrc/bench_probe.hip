// bench_probe.hip - measurement helpers for the benchmark (not part of the
// decode path and not declared in the library's C ABI).
//
//   moe_probe_stream_read: a read-only streaming kernel over a device buffer,
//     16-byte loads, grid-strided, eight loads in flight per lane; its time
//     gives the HBM read rate this GPU sustains, the practical ceiling of a
//     weight-streaming decode step.
//   moe_probe_stream_read_u: the same with 1, 2, 4 or 8 loads in flight per
//     lane, so that the bytes in flight per CU can be set (the read rate
//     falls when far more than ~32 KB per CU are in flight).
//   moe_probe_copy: a plain 16-byte copy kernel of known size; its hardware
//     counters (bytes fetched and written) calibrate the counters read on the
//     decode kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                          unsigned *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // keeps the loads alive; the value is never 0x9E3779B9 in practice, so the store is skipped
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ void __launch_bounds__(256) copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                   size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// bytes must be a multiple of 16 and p 16-byte aligned; sink: one device word.
// Returns a hipError_t.
int moe_probe_stream_read_u(const void *p, size_t bytes, void *sink, int grid, int loads, void *stream) {
  if (!p || !sink || (bytes & 15u) || ((uintptr_t)p & 15u) || grid < 1) return (int)hipErrorInvalidValue;
  const hipStream_t s = (hipStream_t)stream;
  const size_t n16 = bytes / 16;
  switch (loads) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(grid), dim3(256), 0, s, (const u32x4 *)p, n16, (unsigned *)sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(grid), dim3(256), 0, s, (const u32x4 *)p, n16, (unsigned *)sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(256), 0, s, (const u32x4 *)p, n16, (unsigned *)sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, s, (const u32x4 *)p, n16, (unsigned *)sink); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int moe_probe_stream_read(const void *p, size_t bytes, void *sink, int grid, void *stream) {
  return moe_probe_stream_read_u(p, bytes, sink, grid, 8, stream);
}

int moe_probe_copy(const void *src, void *dst, size_t bytes, int grid, void *stream) {
  if (!src || !dst || (bytes & 15u) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || grid < 1)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint4 *)src, (uint4 *)dst,
                     bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
