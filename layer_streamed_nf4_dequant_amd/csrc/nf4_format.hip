// NF4 storage format kernels for gfx950: pack (first and second quantisation pass) and the
// standalone dequantisation.
//
// Format ("Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript
// @2:19-2:29: 4-bit codes on normal-quantile levels, then a second quantisation pass over the
// per-block constants): blocks of 64 consecutive row-major weights share an absmax c_b; the
// c_b, minus their mean mu, are stored as int8 codes v/127 scaled per group of 256 blocks by
// an fp32 s2_g. Byte j of the codes holds element 2j in its high nibble.
//
// Every fp32 step uses an explicitly rounded intrinsic (__fdiv_rn, __fmul_rn, __fadd_rn,
// __fsub_rn), so the results do not depend on FMA contraction.

#include "common.h"

namespace lsn {
namespace {

struct Nf4KernelTable {
  float q[16];
  float m[15];
};

Nf4KernelTable kernel_table() {
  Nf4KernelTable t;
  const Nf4Table &h = nf4_table();
  for (int i = 0; i < 16; ++i) t.q[i] = h.q[i];
  for (int i = 0; i < 15; ++i) t.m[i] = h.m[i];
  return t;
}

// ---------------------------------------------------------------------------------------------
// pack, first pass: one thread per 8 consecutive weights, 8 threads per 64-weight block.
// c_b = max|w| (exact), x = fl32(w / c_b), code = #{i : x > m_i}.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pack_codes(const float4 *__restrict__ w, int64_t n8,
                                                    uint32_t *__restrict__ codes,
                                                    float *__restrict__ absmax,
                                                    int *__restrict__ nonfinite,
                                                    Nf4KernelTable tab) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // group of 8 weights
  // n8 is a multiple of 8 (whole blocks) and the grid covers it exactly in multiples of 256,
  // so whole 8-lane groups are either all in range or all out of range.
  const bool live = g < n8;
  float v[8];
  if (live) {
    const float4 a = w[2 * g], b = w[2 * g + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    finite = finite && __builtin_isfinite(v[i]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  // max over the 8 lanes of this block (lanes 8k .. 8k+7 of the wave)
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  if (!live) return;
  if (!finite) atomicOr(nonfinite, 1);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = amax > 0.0f ? __fdiv_rn(v[i], amax) : 0.0f;
    uint32_t code = 0;
#pragma unroll
    for (int k = 0; k < 15; ++k) code += (x > tab.m[k]) ? 1u : 0u;
    // element 2j -> high nibble of byte j; byte j of the little-endian word is bits 8j..8j+7
    const int byte = i >> 1;
    const int shift = 8 * byte + ((i & 1) ? 0 : 4);
    word |= code << shift;
  }
  codes[g] = word;
  if ((threadIdx.x & 7) == 0) absmax[g >> 3] = amax;
}

// ---------------------------------------------------------------------------------------------
// pack, second pass: one 256-thread workgroup per group of 256 blocks.
// d_b = fl32(c_b - mu); s2 = max|d_b|; y = fl32(d_b / s2); v_b = -127 + #{t_v < y}.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float int8_midpoint(int v) {
  // t_v = fl32((code8[v] + code8[v+1]) / 2); the fp64 sum of two fp32 values in [-1, 1] is
  // exact, and halving is exact, so one rounding to fp32 remains.
  const double lo = (double)int8_level(v), hi = (double)int8_level(v + 1);
  return (float)((lo + hi) * 0.5);
}

__device__ __forceinline__ int quantise_int8(float y) {
  int v = (int)rintf(y * 127.0f);
  v = v < -127 ? -127 : (v > 127 ? 127 : v);
  // settle on v = -127 + #{u in [-127, 126] : y > t_u}; the midpoints are increasing
  while (v > -127 && !(y > int8_midpoint(v - 1))) --v;
  while (v < 127 && y > int8_midpoint(v)) ++v;
  return v;
}

__global__ __launch_bounds__(256) void k_pack_second(const float *__restrict__ absmax, float mu,
                                                     int8_t *__restrict__ qabsmax,
                                                     float *__restrict__ absmax2) {
  __shared__ float wave_max[4];
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float d = __fsub_rn(absmax[b], mu);
  float m = fabsf(d);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  const float s2 = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float y = s2 > 0.0f ? __fdiv_rn(d, s2) : 0.0f;
  qabsmax[b] = (int8_t)quantise_int8(y);
  if (threadIdx.x == 0) absmax2[blockIdx.x] = s2;
}

// ---------------------------------------------------------------------------------------------
// standalone dequantisation of up to kMaxDqJobs tensors in one launch (a decoder layer's seven
// projections: one ramp and one tail instead of seven). Each job owns a contiguous range of
// workgroups starting at wg0; a workgroup finds its job by comparing blockIdx.x with the wg0.
// ---------------------------------------------------------------------------------------------
struct DqJob {
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *absmax2;
  float mu;
  int64_t rows, cols;
  void *out;
  int64_t wg0;
};
struct DqJobs {
  int n;
  DqJob job[kMaxDqJobs];
};

__device__ __forceinline__ int find_job(const DqJobs &jobs, int64_t b) {
  int g = 0;
#pragma unroll
  for (int q = 1; q < kMaxDqJobs; ++q)
    if (q < jobs.n && b >= jobs.job[q].wg0) g = q;
  return g;
}

// Row-major: a 256-thread workgroup covers 8192 weights; thread t handles the 8-weight groups
// t, t+256, t+512, t+768 of its chunk, so every load and store of a wave is contiguous (4 B of
// codes in, 16 B of bf16 or 32 B of fp32 out per lane).
template <int OUT>
__global__ __launch_bounds__(256) void k_dequant(DqJobs jobs, Nf4KernelTable tab) {
  __shared__ float sq[16];
  __shared__ float scode8[256];
  const int t = threadIdx.x;
  if (t < 16) sq[t] = tab.q[t];
  if (t < 255) scode8[t] = int8_level(t - 127);
  const DqJob &J = jobs.job[find_job(jobs, blockIdx.x)];
  const uint32_t *codes = reinterpret_cast<const uint32_t *>(J.codes);
  const int64_t g0 = ((int64_t)blockIdx.x - J.wg0) * 1024 + t;
  uint32_t word[4];
  int v[4];
  float s2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t g = g0 + 256 * i;
    word[i] = __builtin_nontemporal_load(&codes[g]);
    v[i] = J.qabsmax[g >> 3];
    s2[i] = J.absmax2[g >> 11];
  }
  __syncthreads();
  const float mu = J.mu;
  void *out = J.out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t g = g0 + 256 * i;
    const float c = decode_absmax(scode8[v[i] + 127], s2[i], mu);
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int shift = 8 * (e >> 1) + ((e & 1) ? 0 : 4);
      f[e] = __fmul_rn(sq[(word[i] >> shift) & 15u], c);
    }
    if (OUT == LSN_OUT_BF16) {
      u32x4_t o;
      o.x = pack_bf16x2(f[0], f[1]);
      o.y = pack_bf16x2(f[2], f[3]);
      o.z = pack_bf16x2(f[4], f[5]);
      o.w = pack_bf16x2(f[6], f[7]);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t *>(out) + g);
    } else {
      floatx4_t *o = reinterpret_cast<floatx4_t *>(out) + 2 * g;
      const floatx4_t lo = {f[0], f[1], f[2], f[3]}, hi = {f[4], f[5], f[6], f[7]};
      __builtin_nontemporal_store(lo, o);
      __builtin_nontemporal_store(hi, o + 1);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dequantise into the transposed layout: out[k][n] = w_hat[n][k] (bf16), for a backward GEMM
// that reduces over n with both operands n-contiguous. Same arithmetic as k_dequant, so the
// values are bit-identical. Workgroup tile: 64 rows n x 512 columns k, one pass: thread t decodes
// rows n0 + 8 (t % 8) .. +7 at columns k0 + 16 (t / 8) .. +15 (8 code bytes per row, inside one
// 64-weight block), then stores each of its 16 columns as 8 consecutive n (16 bytes), so 8 lanes
// write one whole 128-byte line of an out row and a wave instruction covers 8 out rows. Tiles
// walk n fastest. Measured against wider tiles (512-byte and longer row runs per tile) after a
// layer's row-major dequant, as the backward visit runs them, this shape writes fastest: the
// output lines in flight spread over many rows instead of long runs of few.
// Requires rows % 8 == 0 (checked by the caller); cols % 64 == 0 by the format.
// ---------------------------------------------------------------------------------------------
constexpr int kDqtRows = 64, kDqtCols = 512;
__host__ __device__ inline int64_t dqt_tiles(int64_t rows, int64_t cols) {
  return ((rows + kDqtRows - 1) / kDqtRows) * ((cols + kDqtCols - 1) / kDqtCols);
}

__global__ __launch_bounds__(256) void k_dequant_t(DqJobs jobs, Nf4KernelTable tab) {
  __shared__ float sq[16];
  __shared__ float scode8[256];
  const int t = threadIdx.x;
  if (t < 16) sq[t] = tab.q[t];
  if (t < 255) scode8[t] = int8_level(t - 127);
  const DqJob &J = jobs.job[find_job(jobs, blockIdx.x)];
  const int64_t tile = (int64_t)blockIdx.x - J.wg0;
  const int64_t rows = J.rows, cols = J.cols;
  // threads: kDqtRows / 8 along n (8 rows each), the rest along k (16 columns per pass)
  constexpr int NG = kDqtRows / 8, KG = 256 / NG, KSTRIDE = 16 * KG;
  const int64_t ntn = (rows + kDqtRows - 1) / kDqtRows;
  const int64_t n = (tile % ntn) * kDqtRows + 8 * (t % NG);
  const int64_t kbase = (tile / ntn) * kDqtCols + 16 * (t / NG);
  const bool row_ok = n < rows;
  constexpr int NP = kDqtCols / KSTRIDE;
  uint2 word[NP][8];
  int v[NP][8];
  float s2[NP][8];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int64_t k = kbase + KSTRIDE * ps;
    const bool ok = row_ok && k < cols;              // whole 64-column blocks: cols % 64 == 0
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t e = (n + i) * cols + k;          // element index of the thread's first weight in row n+i
      word[ps][i] = ok ? *reinterpret_cast<const uint2 *>(J.codes + (e >> 1)) : make_uint2(0u, 0u);
      v[ps][i] = ok ? J.qabsmax[e >> 6] : 0;
      s2[ps][i] = ok ? J.absmax2[e >> 14] : 0.0f;
    }
  }
  __syncthreads();
  const float mu = J.mu;
  uint16_t *out = reinterpret_cast<uint16_t *>(J.out);
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int64_t k = kbase + KSTRIDE * ps;
    if (!row_ok || k >= cols) continue;
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = decode_absmax(scode8[v[ps][i] + 127], s2[ps][i], mu);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int shift = 8 * ((e >> 1) & 3) + ((e & 1) ? 0 : 4);
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = (e < 8) ? word[ps][i].x : word[ps][i].y;
        f[i] = __fmul_rn(sq[(w >> shift) & 15u], c[i]);
      }
      u32x4_t o;
      o.x = pack_bf16x2(f[0], f[1]);
      o.y = pack_bf16x2(f[2], f[3]);
      o.z = pack_bf16x2(f[4], f[5]);
      o.w = pack_bf16x2(f[6], f[7]);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t *>(out + (k + e) * rows + n));
    }
  }
}

}  // namespace

lsn_status launch_pack_codes(const float *w, int64_t n, uint8_t *codes, float *absmax,
                             int *nonfinite_flag, hipStream_t s) {
  const int64_t n8 = n / 8;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(k_pack_codes, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const float4 *>(w), n8, reinterpret_cast<uint32_t *>(codes),
                     absmax, nonfinite_flag, kernel_table());
  return check_hip(hipGetLastError(), "k_pack_codes launch");
}

lsn_status launch_pack_second(const float *absmax, int64_t n_blocks, float mu, int8_t *qabsmax,
                              float *absmax2, hipStream_t s) {
  hipLaunchKernelGGL(k_pack_second, dim3((unsigned)(n_blocks / 256)), dim3(256), 0, s, absmax, mu,
                     qabsmax, absmax2);
  return check_hip(hipGetLastError(), "k_pack_second launch");
}

lsn_status launch_dequant(int n, const lsn_nf4 *w, void *const *out, int out_dtype, hipStream_t s) {
  DqJobs jobs{};
  jobs.n = n;
  int64_t wg = 0;
  for (int g = 0; g < n; ++g) {
    DqJob &J = jobs.job[g];
    J.codes = w[g].codes;
    J.qabsmax = w[g].qabsmax;
    J.absmax2 = w[g].absmax2;
    J.mu = w[g].mean;
    J.rows = w[g].rows;
    J.cols = w[g].cols;
    J.out = out[g];
    J.wg0 = wg;
    if (out_dtype == LSN_OUT_BF16_T)
      wg += dqt_tiles(w[g].rows, w[g].cols);
    else
      wg += w[g].rows * w[g].cols / 8192;
  }
  const dim3 grid((unsigned)wg);
  if (out_dtype == LSN_OUT_BF16_T)
    hipLaunchKernelGGL(k_dequant_t, grid, dim3(256), 0, s, jobs, kernel_table());
  else if (out_dtype == LSN_OUT_BF16)
    hipLaunchKernelGGL(k_dequant<LSN_OUT_BF16>, grid, dim3(256), 0, s, jobs, kernel_table());
  else
    hipLaunchKernelGGL(k_dequant<LSN_OUT_F32>, grid, dim3(256), 0, s, jobs, kernel_table());
  return check_hip(hipGetLastError(), "k_dequant launch");
}

}  // namespace lsn
