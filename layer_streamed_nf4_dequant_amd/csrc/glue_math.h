// Elementwise arithmetic of the decoder-layer glue (rotary embedding, SwiGLU), shared by the
// standalone glue kernels and the GEMM / attention epilogues that apply the same operations to
// their own outputs. One definition, so a fused epilogue and the standalone kernel produce the
// same bits from the same bf16 inputs: fp32 arithmetic, every product and sum separately rounded
// (the sources are built without contraction), one bf16 rounding per stored value.
#pragma once

#include "common.h"

namespace lsn {

__device__ __forceinline__ float bf16f(uint16_t h) { return bf16_bits_to_f32(h); }
__device__ __forceinline__ uint16_t f2bf(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu); }

// ---- rotary position embedding -------------------------------------------------------------
// Pair (x1, x2) = (element i, element i + d/2) of a head turns by the angle a = fl32(p * f_i),
// f_i = theta^(-2 i / d) (fp32, from the host): y1 = x1 cos a - x2 sin a, y2 = x2 cos a + x1 sin a.
// The inverse (the backward) turns by -a, i.e. uses -sin a.
__device__ __forceinline__ void rope_pair(float x1, float x2, float c, float s, float &y1, float &y2) {
  y1 = __fsub_rn(__fmul_rn(x1, c), __fmul_rn(x2, s));
  y2 = __fadd_rn(__fmul_rn(x2, c), __fmul_rn(x1, s));
}

// cosine and sine of the angle of position p at frequency f (the one place they are computed)
__device__ __forceinline__ void rope_cos_sin(float p, float f, float &c, float &s) {
  sincosf(__fmul_rn(p, f), &s, &c);
}

// eight consecutive pairs of one head: x1 holds elements i .. i+7, x2 elements i+d/2 .. i+d/2+7
// (bf16, packed two per word); c, s the pairs' cosines and (signed) sines
__device__ __forceinline__ void rope_chunk8(u32x4_t x1, u32x4_t x2, const float (&c)[8], const float (&s)[8],
                                            u32x4_t &y1, u32x4_t &y2) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float a[2], b[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * q + h;
      rope_pair(bf16f((uint16_t)(x1[q] >> (16 * h))), bf16f((uint16_t)(x2[q] >> (16 * h))), c[e], s[e], a[h], b[h]);
    }
    y1[q] = pack_bf16x2(a[0], a[1]);
    y2[q] = pack_bf16x2(b[0], b[1]);
  }
}

// the (cos, sin) of eight consecutive pairs from a table row (16 floats, 16-byte aligned); the
// sines multiplied by sign (-1: the inverse rotation)
__device__ __forceinline__ void rope_load8(const float *__restrict__ cs, float sign, float (&c)[8], float (&s)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const floatx4_t v = *reinterpret_cast<const floatx4_t *>(cs + 4 * q);
    c[2 * q] = v[0];
    s[2 * q] = __fmul_rn(sign, v[1]);
    c[2 * q + 1] = v[2];
    s[2 * q + 1] = __fmul_rn(sign, v[3]);
  }
}

// bf16( r + v ) on packed bf16 words (the residual stream's addition)
__device__ __forceinline__ uint32_t add_bf16_word(uint32_t r, uint32_t v) {
  return pack_bf16x2(__fadd_rn(bf16f((uint16_t)r), bf16f((uint16_t)v)),
                     __fadd_rn(bf16f((uint16_t)(r >> 16)), bf16f((uint16_t)(v >> 16))));
}

// ---- SwiGLU --------------------------------------------------------------------------------
// sigma(z) = 1 / (1 + e^-z) from the hardware's base-2 exponential and reciprocal (v_exp_f32,
// v_rcp_f32, each within 1 ulp): e^-z = 2^(-z log2 e), whose argument rounding adds a relative
// error of about |z| 2^-24, so sigma is within (|z| + 4) 2^-24 relative of its exact value - far
// inside the bf16 rounding of every output (a sigma below the fp32 normal range, z < -87, may come
// out as 0). Five instructions against about thirty for the correctly rounded exp and division,
// which matters where the SwiGLU runs in a GEMM's epilogue.
__device__ __forceinline__ float sigmoid_f32(float z) {
  const float e = __builtin_amdgcn_exp2f(__fmul_rn(z, -1.44269504088896340736f));
  return __builtin_amdgcn_rcpf(__fadd_rn(1.0f, e));
}

// m = bf16( silu(g) u ) on eight bf16 pairs
__device__ __forceinline__ u32x4_t swiglu8(u32x4_t gv, u32x4_t uv) {
  u32x4_t o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float t[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float z = bf16f((uint16_t)(gv[q] >> (16 * h)));
      t[h] = __fmul_rn(__fmul_rn(z, sigmoid_f32(z)), bf16f((uint16_t)(uv[q] >> (16 * h))));
    }
    o[q] = pack_bf16x2(t[0], t[1]);
  }
  return o;
}

// dg = bf16( dm u sigma (1 + g (1 - sigma)) ), du = bf16( dm silu(g) ) on one packed word (two
// bf16 triples)
__device__ __forceinline__ void swiglu_bwd_word(uint32_t gw, uint32_t uw, uint32_t dw, uint32_t &og, uint32_t &ou) {
  float tg[2], tu[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float z = bf16f((uint16_t)(gw >> (16 * h)));
    const float uu = bf16f((uint16_t)(uw >> (16 * h)));
    const float d = bf16f((uint16_t)(dw >> (16 * h)));
    const float sg = sigmoid_f32(z);
    const float dsilu = __fmul_rn(sg, __fadd_rn(1.0f, __fmul_rn(z, __fsub_rn(1.0f, sg))));
    tg[h] = __fmul_rn(__fmul_rn(d, uu), dsilu);
    tu[h] = __fmul_rn(d, __fmul_rn(z, sg));
  }
  og = pack_bf16x2(tg[0], tg[1]);
  ou = pack_bf16x2(tu[0], tu[1]);
}

__device__ __forceinline__ void swiglu8_bwd(u32x4_t gv, u32x4_t uv, u32x4_t dv, u32x4_t &og, u32x4_t &ou) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t a, b;
    swiglu_bwd_word(gv[q], uv[q], dv[q], a, b);
    og[q] = a;
    ou[q] = b;
  }
}

}  // namespace lsn
