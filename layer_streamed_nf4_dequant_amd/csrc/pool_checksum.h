// The layer pool's slot checksum, shared by its host and device halves.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace lsn {

// splitmix64's finaliser applied to (word + index * golden ratio): position-sensitive, so a
// slot holding another layer's bytes, or the right bytes at the wrong offsets, changes it.
__host__ __device__ inline uint64_t checksum_word(uint64_t w, uint64_t i) {
  uint64_t z = w + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline uint64_t checksum_host(const void *p, size_t bytes) {
  const uint64_t *w = static_cast<const uint64_t *>(p);
  uint64_t acc = 0;
  for (size_t i = 0; i < bytes / 8; ++i) acc += checksum_word(w[i], i);
  return acc;
}

hipError_t launch_checksum(const void *p, size_t bytes, unsigned long long *out, hipStream_t s);
hipError_t launch_poison(void *p, size_t bytes, hipStream_t s);

}  // namespace lsn
