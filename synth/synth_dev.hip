/*
 * synth_dev.hip - device side of the seeded synthetic-input generator.
 *
 * Fills large device tensors (expert weights of all 896 experts) with exactly
 * the bytes synth_host.c would write: the same counter-based index
 * (synth_core.h, integer arithmetic only) into the same host-built value
 * table, which the caller uploads. Holds no arithmetic of the MoE layer.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYNTH_FN __host__ __device__ static inline
#include "synth_core.h"

namespace {

template <typename T>
__global__ void __launch_bounds__(256) fill_kernel(T *__restrict__ dst, uint64_t n, uint64_t key,
                                                   const T *__restrict__ table) {
  __shared__ T lut[SYNTH_TABLE_SIZE];
  for (uint32_t i = threadIdx.x; i < SYNTH_TABLE_SIZE; i += blockDim.x) lut[i] = table[i];
  __syncthreads();
  const uint64_t quads = (n + 3u) / 4u;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += stride) {
    const uint64_t h = synth_bits(key, q);
    const uint64_t base = q * 4u;
#pragma unroll
    for (uint32_t s = 0; s < 4u; ++s) {
      if (base + s < n) dst[base + s] = lut[(uint32_t)(h >> (16u * s)) & (SYNTH_TABLE_SIZE - 1u)];
    }
  }
}

/* fp8 codes [rows][cols]; row group g (128 rows) reads the code table of its
 * scale class, the top two bits of draw g of class_key. */
__global__ void __launch_bounds__(256) fill_fp8_kernel(uint8_t *__restrict__ dst, uint64_t rows,
                                                       uint64_t cols, uint64_t key, uint64_t class_key,
                                                       const uint8_t *__restrict__ codes) {
  __shared__ uint8_t lut[4 * SYNTH_TABLE_SIZE];
  for (uint32_t i = threadIdx.x; i < 4 * SYNTH_TABLE_SIZE; i += blockDim.x) lut[i] = codes[i];
  __syncthreads();
  const uint64_t n = rows * cols;
  const uint64_t group_elems = 128u * cols;
  const uint64_t quads = (n + 3u) / 4u;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += stride) {
    const uint64_t h = synth_bits(key, q);
    const uint64_t base = q * 4u;
#pragma unroll
    for (uint32_t s = 0; s < 4u; ++s) {
      const uint64_t i = base + s;
      if (i < n) {
        const uint32_t c = (uint32_t)(synth_bits(class_key, i / group_elems) >> 62);
        dst[i] = lut[c * SYNTH_TABLE_SIZE + ((uint32_t)(h >> (16u * s)) & (SYNTH_TABLE_SIZE - 1u))];
      }
    }
  }
}

unsigned grid_for(uint64_t n) {
  uint64_t quads = (n + 3u) / 4u;
  uint64_t blocks = (quads + 255u) / 256u;
  if (blocks > 8192u) blocks = 8192u;
  if (blocks < 1u) blocks = 1u;
  return (unsigned)blocks;
}

}  // namespace

extern "C" {

/* dst[i] = table[index(key, i)], i < n; table has 2^14 entries of elem_bytes
 * (1, 2 or 4). All pointers are device pointers. Returns a hipError_t. */
int synth_dev_fill(void *dst, uint64_t n, uint64_t key, const void *table, int elem_bytes,
                   void *stream) {
  if (n == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  unsigned g = grid_for(n);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(fill_kernel<uint32_t>, dim3(g), dim3(256), 0, s, (uint32_t *)dst, n, key,
                       (const uint32_t *)table);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(fill_kernel<uint16_t>, dim3(g), dim3(256), 0, s, (uint16_t *)dst, n, key,
                       (const uint16_t *)table);
  else if (elem_bytes == 1)
    hipLaunchKernelGGL(fill_kernel<uint8_t>, dim3(g), dim3(256), 0, s, (uint8_t *)dst, n, key,
                       (const uint8_t *)table);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

/* fp8 weight [rows][cols], rows a multiple of 128; codes = 4 device tables of
 * 2^14 codes (one per scale class). */
int synth_dev_fill_fp8(uint8_t *dst, uint64_t rows, uint64_t cols, uint64_t key, uint64_t class_key,
                       const uint8_t *codes, void *stream) {
  if (rows == 0 || cols == 0) return 0;
  if (rows % 128u) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_fp8_kernel, dim3(grid_for(rows * cols)), dim3(256), 0,
                     (hipStream_t)stream, dst, rows, cols, key, class_key, codes);
  return (int)hipGetLastError();
}

}  // extern "C"
