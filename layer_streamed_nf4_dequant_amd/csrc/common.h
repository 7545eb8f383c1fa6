// Internal helpers shared by the HIP sources of liblsnf4 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/lsnf4.h"

namespace lsn {

// ---- error reporting (thread-local message, see lsn_last_error) ---------------------------
lsn_status fail(lsn_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
lsn_status check_hip(hipError_t e, const char *what);

// ---- the NF4 tables the kernels use, computed on the host at first use -------------------
struct Nf4Table {
  float q[16];   // levels, ascending
  float m[15];   // midpoints between consecutive levels
};
const Nf4Table &nf4_table();

// ---- small device helpers ------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Round fp32 to bf16 (nearest even) with the gfx950 conversion; returns the 16-bit pattern.
// two fp32 -> bf16 (round to nearest even) in one packed conversion
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __builtin_bit_cast(float, h16 << 16);
}

// c'_b = fl32( fl32(code8[v] * s2) + mu ), two separately rounded operations (no contraction).
__device__ __forceinline__ float decode_absmax(float code8, float s2, float mu) {
  return __fadd_rn(__fmul_rn(code8, s2), mu);
}

// code8[v] = fl32(v / 127), correctly rounded division.
__device__ __forceinline__ float int8_level(int v) { return __fdiv_rn((float)v, 127.0f); }

// ---- launchers (host side), defined in the .hip files --------------------------------------
lsn_status launch_pack_codes(const float *w, int64_t n, uint8_t *codes, float *absmax,
                             int *nonfinite_flag, hipStream_t s);
lsn_status launch_pack_second(const float *absmax, int64_t n_blocks, float mu, int8_t *qabsmax,
                              float *absmax2, hipStream_t s);
// dequantise n (<= kMaxDqJobs) tensors into out[g] in one launch (all in the same layout)
constexpr int kMaxDqJobs = 8;
lsn_status launch_dequant(int n, const lsn_nf4 *w, void *const *out, int out_dtype, hipStream_t s);
// rotary embedding in place from a (cos, sin) table [n_pos][head_dim / 2] (rope_table), on
// n_heads heads at the start of each of T rows (row stride ld); sign -1: the inverse rotation.
// head_dim / 2 a multiple of 8, ld a multiple of 8, x and cs 16-byte aligned.
lsn_status launch_rope_tab(int64_t T, int n_heads, int head_dim, uint16_t *x, int64_t ld, const int32_t *positions,
                           const float *cs, int n_pos, float sign, hipStream_t s);

}  // namespace lsn
