// Device side of the layer pool's aliasing audit: a 64-bit checksum of a slot and the poison
// fill of a released slot. The checksum is a sum modulo 2^64 of mixed 8-byte words, so the
// integer atomics that combine the per-workgroup partial sums give the same value in any
// order; the host computes the same function over the pinned image (pool.cpp).

#include "pool_checksum.h"

namespace lsn {
namespace {

__global__ __launch_bounds__(256) void k_checksum(const uint64_t *__restrict__ p, uint64_t n_words,
                                                  unsigned long long *__restrict__ out) {
  uint64_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride)
    acc += checksum_word(p[i], i);
  // wave reduction, then one integer atomic per wave (order-independent: addition mod 2^64)
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)acc, off);
    const uint32_t hi = __shfl_xor((uint32_t)(acc >> 32), off);
    acc += ((uint64_t)hi << 32) | lo;
  }
  if ((threadIdx.x & 63) == 0) atomicAdd(out, (unsigned long long)acc);
}

__global__ __launch_bounds__(256) void k_poison(uint4 *__restrict__ p, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint4 ones = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = ones;
}

}  // namespace

hipError_t launch_checksum(const void *p, size_t bytes, unsigned long long *out, hipStream_t s) {
  const uint64_t n_words = bytes / 8;
  hipLaunchKernelGGL(k_checksum, dim3(1024), dim3(256), 0, s, (const uint64_t *)p, n_words, out);
  return hipGetLastError();
}

hipError_t launch_poison(void *p, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(k_poison, dim3(1024), dim3(256), 0, s, (uint4 *)p, (uint64_t)(bytes / 16));
  return hipGetLastError();
}

}  // namespace lsn
