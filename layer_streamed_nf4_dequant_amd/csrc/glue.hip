// The decoder-layer glue around the seven projections: RMSNorm, rotary position embedding and the
// SwiGLU gate, forward and backward. The pages train Llama-3.1 and Qwen2.5 decoder layers
// ("Exact Layer Streaming", Abstract; "An 8B Fine-Tune Now Fits in 4 GB of VRAM": the decoder
// layer is the streamed unit) and print none of these formulas; these are those models' published
// layer definitions. All of them are bandwidth-bound elementwise or row work: fp32 arithmetic on
// bf16 tensors, every product and sum separately rounded (no contraction), and every row
// reduction in a fixed order, so the bits depend only on the inputs.

#include <algorithm>
#include <cmath>
#include <vector>

#include "common.h"
#include "glue_math.h"

namespace lsn {
lsn_status require_gfx950();
bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb);

namespace {

constexpr int kGlueThreads = 256;
constexpr int kMaxRopePairs = 256;   // head_dim <= 512


// sum over the NT threads of a workgroup: a fixed butterfly in each wave (every lane of a wave
// ends with the same bits: each level adds the same two values on both lanes of a pair), then
// the waves' sums in wave order
template <int NT>
__device__ __forceinline__ float team_sum(float v, float *scratch) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __fadd_rn(v, __shfl_xor(v, off));
  if constexpr (NT == 64) {
    return v;
  } else {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    float s = scratch[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) s = __fadd_rn(s, scratch[w]);
    return s;
  }
}

// y = bf16( (x * rstd) * g ), rstd = 1 / sqrt(mean x^2 + eps). One workgroup of NT threads per
// row (NT sized to the row: 8 values per thread step). A row of at most kRmsChunks chunks per
// thread is held in registers, with the gain requested beside it before the reduction, so the
// second pass reads nothing; a longer row is re-read (L2) in the second pass. Both forms sum in
// the same order.
constexpr int kRmsChunks = 2;
template <int NT>
__global__ __launch_bounds__(NT) void k_rmsnorm_fwd(int64_t H, const uint16_t *__restrict__ x,
                                                    const uint16_t *__restrict__ g, float eps,
                                                    uint16_t *__restrict__ y, float *__restrict__ rstd) {
  __shared__ float scratch[NT / 64];
  const int64_t row = blockIdx.x;
  const int64_t nc = H / 8;
  const u32x4_t *xr = reinterpret_cast<const u32x4_t *>(x + row * H);
  const u32x4_t *gr = reinterpret_cast<const u32x4_t *>(g);
  u32x4_t *yr = reinterpret_cast<u32x4_t *>(y + row * H);
  auto sq8 = [](float ss, const u32x4_t &v) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = bf16f((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
      ss = __fadd_rn(ss, __fmul_rn(f, f));
    }
    return ss;
  };
  auto out8 = [](const u32x4_t &v, const u32x4_t &gv, float r) {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float t[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float f = bf16f((uint16_t)(v[q] >> (16 * h)));
        const float w = bf16f((uint16_t)(gv[q] >> (16 * h)));
        t[h] = __fmul_rn(__fmul_rn(f, r), w);
      }
      o[q] = pack_bf16x2(t[0], t[1]);
    }
    return o;
  };
  auto rstd_of = [&](float ss) { return __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(ss, (float)H), eps))); };
  if (nc <= (int64_t)NT * kRmsChunks) {
    u32x4_t xv[kRmsChunks], gv[kRmsChunks];
#pragma unroll
    for (int i = 0; i < kRmsChunks; ++i) {
      const int64_t c = threadIdx.x + (int64_t)i * NT;
      if (c < nc) {
        xv[i] = xr[c];
        gv[i] = gr[c];
      }
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kRmsChunks; ++i)
      if (threadIdx.x + (int64_t)i * NT < nc) ss = sq8(ss, xv[i]);
    ss = team_sum<NT>(ss, scratch);
    const float r = rstd_of(ss);
    if (threadIdx.x == 0) rstd[row] = r;
#pragma unroll
    for (int i = 0; i < kRmsChunks; ++i) {
      const int64_t c = threadIdx.x + (int64_t)i * NT;
      if (c < nc) yr[c] = out8(xv[i], gv[i], r);
    }
    return;
  }
  float ss = 0.0f;
  for (int64_t c = threadIdx.x; c < nc; c += NT) ss = sq8(ss, xr[c]);
  ss = team_sum<NT>(ss, scratch);
  const float r = rstd_of(ss);
  if (threadIdx.x == 0) rstd[row] = r;
  for (int64_t c = threadIdx.x; c < nc; c += NT) yr[c] = out8(xr[c], gr[c], r);
}

// dx = rstd (g dy) - x rstd^3 (sum_j g_j dy_j x_j) / H; dy and dx fp32, dx stored or added to.
// One workgroup of NT threads per row; a row of at most kRmsChunks chunks per thread is held in
// registers (x, g, dy, and the dx being added to, all requested before the reduction), a longer
// one re-read in the second pass. Both forms sum in the same order.
template <int NT>
__global__ __launch_bounds__(NT) void k_rmsnorm_bwd(int64_t H, const uint16_t *__restrict__ x,
                                                    const uint16_t *__restrict__ g, const float *__restrict__ rstd,
                                                    const float *__restrict__ dy, float *__restrict__ dx,
                                                    int accumulate, uint16_t *__restrict__ dx16) {
  __shared__ float scratch[NT / 64];
  const int64_t row = blockIdx.x;
  const int64_t nc = H / 8;
  const u32x4_t *xr = reinterpret_cast<const u32x4_t *>(x + row * H);
  const floatx4_t *dr = reinterpret_cast<const floatx4_t *>(dy + row * H);
  const u32x4_t *gr = reinterpret_cast<const u32x4_t *>(g);
  floatx4_t *o = reinterpret_cast<floatx4_t *>(dx + row * H);
  auto dot8 = [](float dot, const u32x4_t &v, const u32x4_t &gv, const floatx4_t &d0, const floatx4_t &d1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = e >> 1, h = 16 * (e & 1);
      const float gd = __fmul_rn(bf16f((uint16_t)(gv[q] >> h)), e < 4 ? d0[e & 3] : d1[e & 3]);
      dot = __fadd_rn(dot, __fmul_rn(gd, bf16f((uint16_t)(v[q] >> h))));
    }
    return dot;
  };
  // chunk c's gradient, added to `prev` (the stored values) when accumulating, stored (and its
  // bf16 copy, for the operand that reads it next)
  auto store8 = [&](int64_t c, const u32x4_t &v, const u32x4_t &gv, const floatx4_t &d0, const floatx4_t &d1,
                    float r, float k, const floatx4_t (&prev)[2]) {
    float res[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = e >> 1, h = 16 * (e & 1);
      const float gd = __fmul_rn(bf16f((uint16_t)(gv[q] >> h)), e < 4 ? d0[e & 3] : d1[e & 3]);
      res[e] = __fsub_rn(__fmul_rn(r, gd), __fmul_rn(bf16f((uint16_t)(v[q] >> h)), k));
    }
    floatx4_t cur[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        cur[half][e] = accumulate ? __fadd_rn(prev[half][e], res[4 * half + e]) : res[4 * half + e];
      o[2 * c + half] = cur[half];
    }
    if (dx16)
      reinterpret_cast<u32x4_t *>(dx16 + row * H)[c] =
          u32x4_t{pack_bf16x2(cur[0][0], cur[0][1]), pack_bf16x2(cur[0][2], cur[0][3]),
                  pack_bf16x2(cur[1][0], cur[1][1]), pack_bf16x2(cur[1][2], cur[1][3])};
  };
  const float r = rstd[row];
  auto k_of = [&](float dot) { return __fdiv_rn(__fmul_rn(__fmul_rn(__fmul_rn(r, r), r), dot), (float)H); };
  if (nc <= (int64_t)NT * kRmsChunks) {
    u32x4_t xv[kRmsChunks], gv[kRmsChunks];
    floatx4_t dv[kRmsChunks][2], pv[kRmsChunks][2];
#pragma unroll
    for (int i = 0; i < kRmsChunks; ++i) {
      const int64_t c = threadIdx.x + (int64_t)i * NT;
      if (c < nc) {
        xv[i] = xr[c];
        gv[i] = gr[c];
        dv[i][0] = dr[2 * c];
        dv[i][1] = dr[2 * c + 1];
        if (accumulate) {
          pv[i][0] = o[2 * c];
          pv[i][1] = o[2 * c + 1];
        }
      }
    }
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < kRmsChunks; ++i)
      if (threadIdx.x + (int64_t)i * NT < nc) dot = dot8(dot, xv[i], gv[i], dv[i][0], dv[i][1]);
    dot = team_sum<NT>(dot, scratch);
    const float k = k_of(dot);
#pragma unroll
    for (int i = 0; i < kRmsChunks; ++i) {
      const int64_t c = threadIdx.x + (int64_t)i * NT;
      if (c < nc) store8(c, xv[i], gv[i], dv[i][0], dv[i][1], r, k, pv[i]);
    }
    return;
  }
  float dot = 0.0f;
  for (int64_t c = threadIdx.x; c < nc; c += NT) dot = dot8(dot, xr[c], gr[c], dr[2 * c], dr[2 * c + 1]);
  dot = team_sum<NT>(dot, scratch);
  const float k = k_of(dot);
  for (int64_t c = threadIdx.x; c < nc; c += NT) {
    floatx4_t prev[2] = {floatx4_t{0.0f, 0.0f, 0.0f, 0.0f}, floatx4_t{0.0f, 0.0f, 0.0f, 0.0f}};
    if (accumulate) {
      prev[0] = o[2 * c];
      prev[1] = o[2 * c + 1];
    }
    store8(c, xr[c], gr[c], dr[2 * c], dr[2 * c + 1], r, k, prev);
  }
}

// threads per row: the row's 16-byte chunks rounded up to whole waves, at most 256
int rms_team(int64_t H) {
  const int64_t chunks = H / 8;
  return chunks > 128 ? 256 : chunks > 64 ? 128 : 64;
}

struct RopeTable {
  float inv_freq[kMaxRopePairs];
};

// In place on n_heads heads of width 2 half in each row (row stride ld elements): pair
// (i, i + half) of a head turns by pos * inv_freq[i] (minus that for the backward).
// Vector form (half % 8 == 0, 16-byte aligned rows): a workgroup takes `rows` consecutive rows
// (rows x half <= kRopeRowPairs), computes the sine and cosine of each of those rows' pairs once
// into LDS (one pair per thread), then rotates 8 consecutive pairs of one head per thread and
// round with 16-byte loads and stores, threads ordered pair-block fastest so that neighbouring
// lanes cover a head's two contiguous halves. Every head of a row reuses the row's angles.
constexpr int kRopeRowPairs = 1024;
__global__ __launch_bounds__(kGlueThreads) void k_rope_rows(int64_t T, int n_heads, int half, int rows, int64_t ld,
                                                            uint16_t *__restrict__ x,
                                                            const int32_t *__restrict__ positions, RopeTable tab,
                                                            float sign) {
  __shared__ float2 cs[kRopeRowPairs];
  const int64_t r0 = (int64_t)blockIdx.x * rows;
  const int nr = (int)min((int64_t)rows, T - r0);
  for (int i = threadIdx.x; i < nr * half; i += kGlueThreads) {
    const int r = i / half, j = i - r * half;
    float c, s;
    rope_cos_sin((float)positions[r0 + r], tab.inv_freq[j], c, s);
    cs[i] = float2{c, __fmul_rn(sign, s)};
  }
  __syncthreads();
  const int nblk = half / 8, per_row = n_heads * nblk;
  for (int it = threadIdx.x; it < nr * per_row; it += kGlueThreads) {
    const int r = it / per_row, rem = it - r * per_row;
    const int h = rem / nblk, blk = rem - h * nblk;
    uint16_t *base = x + (r0 + r) * ld + (int64_t)h * 2 * half + blk * 8;
    u32x4_t *p1 = reinterpret_cast<u32x4_t *>(base);
    u32x4_t *p2 = reinterpret_cast<u32x4_t *>(base + half);
    float c[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 t = cs[r * half + blk * 8 + e];
      c[e] = t.x;
      sn[e] = t.y;
    }
    u32x4_t o1, o2;
    rope_chunk8(*p1, *p2, c, sn, o1, o2);
    *p1 = o1;
    *p2 = o2;
  }
}

// (cos, sin) of every position's angles: cs[p][i] = (cos a, sin a), a = fl32(p f_i), for
// p < n_pos, i < half; the same arithmetic as the kernels above, so rotations driven by the table
// give their bits
__global__ __launch_bounds__(kGlueThreads) void k_rope_table(int64_t n, int half, RopeTable tab,
                                                             float *__restrict__ cs) {
  const int64_t item = (int64_t)blockIdx.x * kGlueThreads + threadIdx.x;
  if (item >= n) return;
  const int64_t p = item / half;
  const int i = (int)(item - p * half);
  float c, sv;
  rope_cos_sin((float)p, tab.inv_freq[i], c, sv);
  cs[2 * item] = c;
  cs[2 * item + 1] = sv;
}

// In place, driven by a (cos, sin) table [n_pos][half]: a thread takes 8 consecutive pairs of one
// head of one row (half % 8 == 0, 16-byte aligned rows); positions outside the table are clamped
// to it (they only guard the table read).
__global__ __launch_bounds__(kGlueThreads) void k_rope_tab(int64_t T, int n_heads, int half, int64_t ld,
                                                           uint16_t *__restrict__ x,
                                                           const int32_t *__restrict__ positions,
                                                           const float *__restrict__ cs, int n_pos, float sign) {
  const int nblk = half / 8;
  const int64_t per_row = (int64_t)n_heads * nblk;
  const int64_t item = (int64_t)blockIdx.x * kGlueThreads + threadIdx.x;
  if (item >= T * per_row) return;
  const int64_t row = item / per_row;
  const int rem = (int)(item - row * per_row);
  const int h = rem / nblk, blk = rem - h * nblk;
  const int pos = min(max(positions[row], 0), n_pos - 1);
  float c[8], sn[8];
  rope_load8(cs + ((int64_t)pos * half + blk * 8) * 2, sign, c, sn);
  uint16_t *base = x + row * ld + (int64_t)h * 2 * half + blk * 8;
  u32x4_t *p1 = reinterpret_cast<u32x4_t *>(base);
  u32x4_t *p2 = reinterpret_cast<u32x4_t *>(base + half);
  u32x4_t o1, o2;
  rope_chunk8(*p1, *p2, c, sn, o1, o2);
  *p1 = o1;
  *p2 = o2;
}

// Scalar form for any even head width: one thread per pair.
__global__ __launch_bounds__(kGlueThreads) void k_rope_s(int64_t T, int n_heads, int half, int64_t ld,
                                                         uint16_t *__restrict__ x,
                                                         const int32_t *__restrict__ positions, RopeTable tab,
                                                         float sign) {
  const int64_t per_row = (int64_t)n_heads * half;
  const int64_t item = (int64_t)blockIdx.x * kGlueThreads + threadIdx.x;
  if (item >= T * per_row) return;
  const int64_t row = item / per_row;
  const int p = (int)(item - row * per_row);
  const int head = p / half, i = p - head * half;
  float sv, cv;
  rope_cos_sin((float)positions[row], tab.inv_freq[i], cv, sv);
  uint16_t *xr = x + row * ld + (int64_t)head * 2 * half;
  float y1, y2;
  rope_pair(bf16f(xr[i]), bf16f(xr[i + half]), cv, __fmul_rn(sign, sv), y1, y2);
  xr[i] = f2bf(y1);
  xr[i + half] = f2bf(y2);
}

constexpr int kEltChunks = 2;   // SwiGLU: 16-byte chunks (8 values) per thread, loads issued together

// m = bf16( silu(g) u ); thread chunks c0 and c0 + kGlueThreads of its workgroup's range
__global__ __launch_bounds__(kGlueThreads) void k_swiglu_fwd(int64_t n8, const uint16_t *__restrict__ g,
                                                             const uint16_t *__restrict__ u, uint16_t *__restrict__ m) {
  const int64_t c0 = (int64_t)blockIdx.x * kGlueThreads * kEltChunks + threadIdx.x;
  const u32x4_t *gp = reinterpret_cast<const u32x4_t *>(g), *up = reinterpret_cast<const u32x4_t *>(u);
  u32x4_t gv[kEltChunks], uv[kEltChunks];
#pragma unroll
  for (int k = 0; k < kEltChunks; ++k) {
    const int64_t c = c0 + k * kGlueThreads;
    if (c < n8) {
      gv[k] = gp[c];
      uv[k] = up[c];
    }
  }
#pragma unroll
  for (int k = 0; k < kEltChunks; ++k) {
    const int64_t c = c0 + k * kGlueThreads;
    if (c < n8) reinterpret_cast<u32x4_t *>(m)[c] = swiglu8(gv[k], uv[k]);
  }
}

// dg = bf16( dm u sigma (1 + g (1 - sigma)) ), du = bf16( dm silu(g) )
__global__ __launch_bounds__(kGlueThreads) void k_swiglu_bwd(int64_t n8, const uint16_t *__restrict__ g,
                                                             const uint16_t *__restrict__ u,
                                                             const uint16_t *__restrict__ dm, uint16_t *__restrict__ dg,
                                                             uint16_t *__restrict__ du) {
  const int64_t c0 = (int64_t)blockIdx.x * kGlueThreads * kEltChunks + threadIdx.x;
  const u32x4_t *gp = reinterpret_cast<const u32x4_t *>(g), *up = reinterpret_cast<const u32x4_t *>(u),
                *dp = reinterpret_cast<const u32x4_t *>(dm);
  u32x4_t gv[kEltChunks], uv[kEltChunks], dv[kEltChunks];
#pragma unroll
  for (int k = 0; k < kEltChunks; ++k) {
    const int64_t c = c0 + k * kGlueThreads;
    if (c < n8) {
      gv[k] = gp[c];
      uv[k] = up[c];
      dv[k] = dp[c];
    }
  }
#pragma unroll
  for (int k = 0; k < kEltChunks; ++k) {
    const int64_t c = c0 + k * kGlueThreads;
    if (c < n8) {
      u32x4_t og, ou;
      swiglu8_bwd(gv[k], uv[k], dv[k], og, ou);
      reinterpret_cast<u32x4_t *>(dg)[c] = og;
      reinterpret_cast<u32x4_t *>(du)[c] = ou;
    }
  }
}

// out = bf16( a + b ) for bf16 a, b (the residual stream's additions), 8 values per thread
__global__ __launch_bounds__(kGlueThreads) void k_add_bf16(int64_t n8, const uint16_t *__restrict__ a,
                                                           const uint16_t *__restrict__ b, uint16_t *__restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * kGlueThreads + threadIdx.x;
  if (c >= n8) return;
  const u32x4_t x = reinterpret_cast<const u32x4_t *>(a)[c], y = reinterpret_cast<const u32x4_t *>(b)[c];
  u32x4_t o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = add_bf16_word(x[q], y[q]);
  reinterpret_cast<u32x4_t *>(out)[c] = o;
}

// fp32 -> bf16 (round to nearest even), 8 values per thread
__global__ __launch_bounds__(kGlueThreads) void k_f32_to_bf16(int64_t n8, const float *__restrict__ in,
                                                              uint16_t *__restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * kGlueThreads + threadIdx.x;
  if (c >= n8) return;
  const floatx4_t x0 = reinterpret_cast<const floatx4_t *>(in)[2 * c], x1 = reinterpret_cast<const floatx4_t *>(in)[2 * c + 1];
  reinterpret_cast<u32x4_t *>(out)[c] =
      u32x4_t{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]), pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
}

// bf16 -> fp32 (exact), 8 values per thread
__global__ __launch_bounds__(kGlueThreads) void k_bf16_to_f32(int64_t n8, const uint16_t *__restrict__ in,
                                                              float *__restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * kGlueThreads + threadIdx.x;
  if (c >= n8) return;
  const u32x4_t x = reinterpret_cast<const u32x4_t *>(in)[c];
  floatx4_t lo, hi;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = bf16f((uint16_t)(x[e >> 1] >> (16 * (e & 1))));
    hi[e] = bf16f((uint16_t)(x[2 + (e >> 1)] >> (16 * (e & 1))));
  }
  reinterpret_cast<floatx4_t *>(out)[2 * c] = lo;
  reinterpret_cast<floatx4_t *>(out)[2 * c + 1] = hi;
}

bool a16(const void *p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace
}  // namespace lsn

using namespace lsn;

extern "C" {

lsn_status rmsnorm_fwd(int64_t T, int64_t H, const uint16_t *x, const uint16_t *gain, float eps, uint16_t *y,
                       float *rstd, void *stream) {
  if (T < 1 || T > 0x7fffffff || H < 8 || H % 8)
    return fail(LSN_E_ARG, "rmsnorm_fwd: need 1 <= T < 2^31 and H a positive multiple of 8");
  if (!x || !gain || !y || !rstd || !a16(x) || !a16(gain) || !a16(y))
    return fail(LSN_E_ARG, "rmsnorm_fwd: null or misaligned pointer");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(LSN_E_ARG, "rmsnorm_fwd: eps must be finite and >= 0");
  const size_t xb = (size_t)(T * H * 2), rb = (size_t)T * 4;
  if (ranges_overlap(y, xb, x, xb) || ranges_overlap(y, xb, gain, (size_t)H * 2) ||
      ranges_overlap(rstd, rb, x, xb) || ranges_overlap(rstd, rb, gain, (size_t)H * 2) ||
      ranges_overlap(rstd, rb, y, xb))
    return fail(LSN_E_ARG, "rmsnorm_fwd: an output overlaps an input or the other output");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const hipStream_t hs = (hipStream_t)stream;
  switch (rms_team(H)) {
    case 64: hipLaunchKernelGGL(k_rmsnorm_fwd<64>, dim3((unsigned)T), dim3(64), 0, hs, H, x, gain, eps, y, rstd); break;
    case 128: hipLaunchKernelGGL(k_rmsnorm_fwd<128>, dim3((unsigned)T), dim3(128), 0, hs, H, x, gain, eps, y, rstd); break;
    default: hipLaunchKernelGGL(k_rmsnorm_fwd<256>, dim3((unsigned)T), dim3(256), 0, hs, H, x, gain, eps, y, rstd);
  }
  return check_hip(hipGetLastError(), "k_rmsnorm_fwd launch");
}

lsn_status rmsnorm_bwd(int64_t T, int64_t H, const uint16_t *x, const uint16_t *gain, const float *rstd,
                       const float *dy, float *dx, int32_t accumulate, uint16_t *dx_bf16, void *stream) {
  if (T < 1 || T > 0x7fffffff || H < 8 || H % 8)
    return fail(LSN_E_ARG, "rmsnorm_bwd: need 1 <= T < 2^31 and H a positive multiple of 8");
  if (!x || !gain || !rstd || !dy || !dx || !a16(x) || !a16(gain) || !a16(dy) || !a16(dx))
    return fail(LSN_E_ARG, "rmsnorm_bwd: null or misaligned pointer");
  const size_t fb = (size_t)(T * H * 4);
  if (ranges_overlap(dx, fb, x, (size_t)(T * H * 2)) || ranges_overlap(dx, fb, dy, fb) ||
      ranges_overlap(dx, fb, rstd, (size_t)T * 4))
    return fail(LSN_E_ARG, "rmsnorm_bwd: dx overlaps an input");
  if (dx_bf16) {
    const size_t hb = (size_t)(T * H * 2);
    if (!a16(dx_bf16) || ranges_overlap(dx_bf16, hb, x, hb) || ranges_overlap(dx_bf16, hb, dy, fb) ||
        ranges_overlap(dx_bf16, hb, dx, fb) || ranges_overlap(dx_bf16, hb, rstd, (size_t)T * 4) ||
        ranges_overlap(dx_bf16, hb, gain, (size_t)H * 2))
      return fail(LSN_E_ARG, "rmsnorm_bwd: dx_bf16 misaligned or overlapping");
  }
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const hipStream_t hs = (hipStream_t)stream;
  const int acc = accumulate ? 1 : 0;
  switch (rms_team(H)) {
    case 64:
      hipLaunchKernelGGL(k_rmsnorm_bwd<64>, dim3((unsigned)T), dim3(64), 0, hs, H, x, gain, rstd, dy, dx, acc, dx_bf16);
      break;
    case 128:
      hipLaunchKernelGGL(k_rmsnorm_bwd<128>, dim3((unsigned)T), dim3(128), 0, hs, H, x, gain, rstd, dy, dx, acc, dx_bf16);
      break;
    default:
      hipLaunchKernelGGL(k_rmsnorm_bwd<256>, dim3((unsigned)T), dim3(256), 0, hs, H, x, gain, rstd, dy, dx, acc, dx_bf16);
  }
  return check_hip(hipGetLastError(), "k_rmsnorm_bwd launch");
}

}  // extern "C"

namespace lsn {
namespace {
// f_i = theta^(-2i/d) in fp64, rounded to fp32 (the frequencies every rotation uses)
RopeTable rope_freqs(float theta, int head_dim) {
  RopeTable tab{};
  for (int i = 0; i < head_dim / 2; ++i) tab.inv_freq[i] = (float)std::pow((double)theta, -2.0 * i / head_dim);
  return tab;
}
}  // namespace

lsn_status launch_rope_tab(int64_t T, int n_heads, int head_dim, uint16_t *x, int64_t ld, const int32_t *positions,
                           const float *cs, int n_pos, float sign, hipStream_t s) {
  const int half = head_dim / 2;
  if (half % 8 || ld % 8 || ((uintptr_t)x & 15) || ((uintptr_t)cs & 15) || n_pos < 1) return LSN_E_ARG;
  const int64_t items = T * n_heads * (half / 8);
  hipLaunchKernelGGL(k_rope_tab, dim3((unsigned)((items + kGlueThreads - 1) / kGlueThreads)), dim3(kGlueThreads), 0, s,
                     T, n_heads, half, ld, x, positions, cs, n_pos, sign);
  return check_hip(hipGetLastError(), "k_rope_tab launch");
}
}  // namespace lsn

extern "C" {

lsn_status rope_table(int32_t n_pos, int32_t head_dim, float theta, float *cs, void *stream) {
  if (n_pos < 1 || n_pos > (1 << 24) || head_dim < 2 || head_dim % 2 || head_dim / 2 > kMaxRopePairs)
    return fail(LSN_E_ARG, "rope_table: need 1 <= n_pos <= 2^24 and an even head_dim <= %d", 2 * kMaxRopePairs);
  if (!cs || ((uintptr_t)cs & 15)) return fail(LSN_E_ARG, "rope_table: cs null or not 16-byte aligned");
  if (!(theta > 1.0f) || !std::isfinite(theta)) return fail(LSN_E_ARG, "rope_table: theta must be finite and > 1");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const int half = head_dim / 2;
  const int64_t n = (int64_t)n_pos * half;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + kGlueThreads - 1) / kGlueThreads)), dim3(kGlueThreads), 0,
                     (hipStream_t)stream, n, half, rope_freqs(theta, head_dim), cs);
  return check_hip(hipGetLastError(), "k_rope_table launch");
}

lsn_status rope_apply(int64_t T, int32_t n_heads, int32_t head_dim, uint16_t *x, int64_t ld, const int32_t *positions,
                      float theta, int32_t inverse, void *stream) {
  if (T < 1 || n_heads < 1 || head_dim < 2 || head_dim % 2 || head_dim / 2 > kMaxRopePairs)
    return fail(LSN_E_ARG, "rope_apply: need T >= 1, n_heads >= 1 and an even head_dim <= %d", 2 * kMaxRopePairs);
  if (ld < (int64_t)n_heads * head_dim) return fail(LSN_E_ARG, "rope_apply: ld smaller than n_heads x head_dim");
  if (!x || !positions) return fail(LSN_E_ARG, "rope_apply: null pointer");
  if (!(theta > 1.0f) || !std::isfinite(theta)) return fail(LSN_E_ARG, "rope_apply: theta must be finite and > 1");
  if (T > ((int64_t)1 << 38) / ((int64_t)n_heads * head_dim))
    return fail(LSN_E_ARG, "rope_apply: more than 2^37 pairs in one call");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const RopeTable tab = rope_freqs(theta, head_dim);
  const int half = head_dim / 2;
  const bool vec = half % 8 == 0 && ld % 8 == 0 && ((uintptr_t)x & 15) == 0;
  if (vec) {
    // rows per workgroup: about one head chunk per thread, within the LDS for the rows' angles
    const int64_t per_row = (int64_t)n_heads * (half / 8);
    const int rows = (int)std::min<int64_t>(std::max<int64_t>(1, kGlueThreads / per_row), kRopeRowPairs / half);
    hipLaunchKernelGGL(k_rope_rows, dim3((unsigned)((T + rows - 1) / rows)), dim3(kGlueThreads), 0,
                       (hipStream_t)stream, T, (int)n_heads, half, rows, ld, x, positions, tab,
                       inverse ? -1.0f : 1.0f);
  } else {
    const int64_t items = T * n_heads * half;
    hipLaunchKernelGGL(k_rope_s, dim3((unsigned)((items + kGlueThreads - 1) / kGlueThreads)), dim3(kGlueThreads), 0,
                       (hipStream_t)stream, T, (int)n_heads, half, ld, x, positions, tab, inverse ? -1.0f : 1.0f);
  }
  return check_hip(hipGetLastError(), "k_rope launch");
}

lsn_status swiglu_fwd(int64_t n, const uint16_t *g, const uint16_t *u, uint16_t *m, void *stream) {
  if (n < 8 || n % 8 || n > ((int64_t)1 << 40)) return fail(LSN_E_ARG, "swiglu_fwd: need n a positive multiple of 8, at most 2^40");
  if (!g || !u || !m || !a16(g) || !a16(u) || !a16(m)) return fail(LSN_E_ARG, "swiglu_fwd: null or misaligned pointer");
  if (ranges_overlap(m, (size_t)n * 2, g, (size_t)n * 2) || ranges_overlap(m, (size_t)n * 2, u, (size_t)n * 2))
    return fail(LSN_E_ARG, "swiglu_fwd: m overlaps an input");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const int64_t n8 = n / 8;
  const int64_t per_block = (int64_t)kGlueThreads * kEltChunks;
  hipLaunchKernelGGL(k_swiglu_fwd, dim3((unsigned)((n8 + per_block - 1) / per_block)), dim3(kGlueThreads), 0,
                     (hipStream_t)stream, n8, g, u, m);
  return check_hip(hipGetLastError(), "k_swiglu_fwd launch");
}

lsn_status swiglu_bwd(int64_t n, const uint16_t *g, const uint16_t *u, const uint16_t *dm, uint16_t *dg, uint16_t *du,
                      void *stream) {
  if (n < 8 || n % 8 || n > ((int64_t)1 << 40)) return fail(LSN_E_ARG, "swiglu_bwd: need n a positive multiple of 8, at most 2^40");
  if (!g || !u || !dm || !dg || !du || !a16(g) || !a16(u) || !a16(dm) || !a16(dg) || !a16(du))
    return fail(LSN_E_ARG, "swiglu_bwd: null or misaligned pointer");
  const size_t b = (size_t)n * 2;
  const void *ins[] = {g, u, dm};
  for (const void *in : ins)
    if (ranges_overlap(dg, b, in, b) || ranges_overlap(du, b, in, b))
      return fail(LSN_E_ARG, "swiglu_bwd: an output overlaps an input");
  if (ranges_overlap(dg, b, du, b)) return fail(LSN_E_ARG, "swiglu_bwd: dg overlaps du");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const int64_t n8 = n / 8;
  const int64_t per_block = (int64_t)kGlueThreads * kEltChunks;
  hipLaunchKernelGGL(k_swiglu_bwd, dim3((unsigned)((n8 + per_block - 1) / per_block)), dim3(kGlueThreads), 0,
                     (hipStream_t)stream, n8, g, u, dm, dg, du);
  return check_hip(hipGetLastError(), "k_swiglu_bwd launch");
}

lsn_status add_bf16(int64_t n, const uint16_t *a, const uint16_t *b, uint16_t *out, void *stream) {
  if (n < 8 || n % 8 || n > ((int64_t)1 << 40)) return fail(LSN_E_ARG, "add_bf16: need n a positive multiple of 8, at most 2^40");
  if (!a || !b || !out || !a16(a) || !a16(b) || !a16(out)) return fail(LSN_E_ARG, "add_bf16: null or misaligned pointer");
  // out may be a or b exactly (in place); a partial overlap is refused
  const size_t nb = (size_t)n * 2;
  if ((out != a && ranges_overlap(out, nb, a, nb)) || (out != b && ranges_overlap(out, nb, b, nb)))
    return fail(LSN_E_ARG, "add_bf16: out partially overlaps an input");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_add_bf16, dim3((unsigned)((n8 + kGlueThreads - 1) / kGlueThreads)), dim3(kGlueThreads), 0,
                     (hipStream_t)stream, n8, a, b, out);
  return check_hip(hipGetLastError(), "k_add_bf16 launch");
}

lsn_status convert_f32_bf16(int64_t n, const float *in, uint16_t *out, void *stream) {
  if (n < 8 || n % 8 || n > ((int64_t)1 << 40)) return fail(LSN_E_ARG, "convert_f32_bf16: need n a positive multiple of 8, at most 2^40");
  if (!in || !out || !a16(in) || !a16(out)) return fail(LSN_E_ARG, "convert_f32_bf16: null or misaligned pointer");
  if (ranges_overlap(out, (size_t)n * 2, in, (size_t)n * 4)) return fail(LSN_E_ARG, "convert_f32_bf16: out overlaps in");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_f32_to_bf16, dim3((unsigned)((n8 + kGlueThreads - 1) / kGlueThreads)), dim3(kGlueThreads), 0,
                     (hipStream_t)stream, n8, in, out);
  return check_hip(hipGetLastError(), "k_f32_to_bf16 launch");
}

lsn_status convert_bf16_f32(int64_t n, const uint16_t *in, float *out, void *stream) {
  if (n < 8 || n % 8 || n > ((int64_t)1 << 40)) return fail(LSN_E_ARG, "convert_bf16_f32: need n a positive multiple of 8, at most 2^40");
  if (!in || !out || !a16(in) || !a16(out)) return fail(LSN_E_ARG, "convert_bf16_f32: null or misaligned pointer");
  if (ranges_overlap(out, (size_t)n * 4, in, (size_t)n * 2)) return fail(LSN_E_ARG, "convert_bf16_f32: out overlaps in");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_bf16_to_f32, dim3((unsigned)((n8 + kGlueThreads - 1) / kGlueThreads)), dim3(kGlueThreads), 0,
                     (hipStream_t)stream, n8, in, out);
  return check_hip(hipGetLastError(), "k_bf16_to_f32 launch");
}

}  // extern "C"
