// The rank-r LoRA side products on gfx950 MFMA (16x16x32 bf16, fp32 accumulate):
//   U = bf16(X A^T), G = bf16(dY B)                      (row projections, reduce over K or N)
//   dB = s dY^T U,   dA = s G^T X                        (reduce over the T token rows)
// ("Can You Fine-Tune a 27B Model on a Laptop?", transcript @1:25-1:58: only the thin adapter
// matrices are trained; the frozen base gets no gradient.)
//
// The reductions over T are split into fixed chunks of 256 rows whose partial sums go to a
// workspace, then a second kernel adds the chunks in index order: no atomics, so the bits
// depend only on the shapes and the inputs.

#include "common.h"
#include "gemm.h"

namespace lsn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------------------------
// row projections sharing one activation: out_g[m][j] = bf16( sum_k act[m][k] P_g[j][k] ), j < r_g,
// for up to 8 low-rank matrices P_g (ranks multiples of 8, total <= 128), so act is read once.
// One 256-thread workgroup per 16 rows; wave w takes the 32-wide K-steps w, w+4, w+8, ...; the
// four partial results are added in wave order through LDS. Column block cb (16 columns of the
// concatenated P) is one MFMA 16x16x32 accumulator.
// The work per K-step is tiny (one activation fragment, NBMAX weight fragments, NBMAX MFMAs), so
// the loop is latency-bound unless many loads are in flight: each wave keeps the operands of
// DEPTH K-steps in registers and issues the loads of step i + DEPTH as it consumes step i.
// ---------------------------------------------------------------------------------------------
template <int NBMAX, int DEPTH>
__global__ __launch_bounds__(256) void k_rowproj(const uint16_t *__restrict__ act, int64_t M, int64_t K,
                                                 RowProjSet set) {
  __shared__ floatx4_t part[4][NBMAX][64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int64_t m = min(m0 + (lane & 15), M - 1);      // clamped rows are never stored
  const int kq = 8 * (lane >> 4);
  const int nks = (int)(K / 32);
  const int nblk = (set.total + 15) / 16;
  // the concatenated row c of P: group g, local row c - start[g]
  const uint16_t *prow[NBMAX];
  bool pok[NBMAX];
#pragma unroll
  for (int cb = 0; cb < NBMAX; ++cb) {
    const int c = 16 * cb + (lane & 15);
    int g = 0;
#pragma unroll
    for (int q = 1; q < 8; ++q) g += (q < set.n && c >= set.start[q]) ? 1 : 0;
    pok[cb] = cb < nblk && c < set.total;
    prow[cb] = set.P[g] + (int64_t)(pok[cb] ? c - set.start[g] : 0) * K;
  }
  const uint16_t *arow = act + m * K + kq;
  floatx4_t acc[NBMAX];
#pragma unroll
  for (int cb = 0; cb < NBMAX; ++cb) acc[cb] = floatx4_t{0, 0, 0, 0};
  u32x4_t va[DEPTH], vb[DEPTH][NBMAX];
  // K-step of this wave's i-th iteration, clamped (a clamped step is loaded but not used)
  auto load = [&](int i, u32x4_t &a_, u32x4_t (&b_)[NBMAX]) {
    const int64_t k = (int64_t)min(wave + 4 * i, nks - 1) * 32;
    a_ = *reinterpret_cast<const u32x4_t *>(arow + k);
#pragma unroll
    for (int cb = 0; cb < NBMAX; ++cb) {
      b_[cb] = u32x4_t{0, 0, 0, 0};
      if (pok[cb]) b_[cb] = *reinterpret_cast<const u32x4_t *>(prow[cb] + k + kq);
    }
  };
  const int iters = (nks - wave + 3) / 4;                // K-steps of this wave
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load(d, va[d], vb[d]);
  for (int i0 = 0; i0 < iters; i0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (i0 + d < iters) {
#pragma unroll
        for (int cb = 0; cb < NBMAX; ++cb)
          if (cb < nblk)
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[d]), as_bf16x8(vb[d][cb]), acc[cb], 0, 0, 0);
      }
      load(i0 + d + DEPTH, va[d], vb[d]);
    }
  }
#pragma unroll
  for (int cb = 0; cb < NBMAX; ++cb) part[wave][cb][lane] = acc[cb];
  __syncthreads();
  // 4 waves finish 4 column blocks at a time; lane holds column c = 16 cb + lane % 16 and rows
  // 4 (lane / 16) + e
  for (int cb = wave; cb < nblk; cb += 4) {
    floatx4_t sum = part[0][cb][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const floatx4_t p = part[w][cb][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] = __fadd_rn(sum[e], p[e]);
    }
    const int c = 16 * cb + (lane & 15);
    if (c >= set.total) continue;
    int g = 0;
    for (int q = 1; q < set.n; ++q) g += c >= set.start[q] ? 1 : 0;
    const int j = c - set.start[g], r = set.r[g];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = m0 + 4 * (lane >> 4) + e;
      if (row < M) {
        const __bf16 b = (__bf16)sum[e];
        set.out[g][row * r + j] = __builtin_bit_cast(uint16_t, b);
      }
    }
  }
}

// dst[c][r] = src[r][c] for a small bf16 matrix (a LoRA factor): one element per thread
__global__ __launch_bounds__(256) void k_transpose(const uint16_t *__restrict__ src, int64_t rows, int64_t cols,
                                                   uint16_t *__restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols, c = i % cols;
  dst[c * rows + r] = src[i];
}

// ---------------------------------------------------------------------------------------------
// split-T partial products: partial[c][p][j] = sum_{t in chunk c} Z[t][p] V[t][j].
// Workgroup = (64 columns p, one chunk of 256 rows t). Both operands are t-major in memory,
// so each is loaded in 8 x 8 blocks and transposed in registers into LDS as [p][t] and [j][t]
// (rows padded to 528 B so the 16-row fragment reads hit distinct banks).
// ---------------------------------------------------------------------------------------------
constexpr int TPITCH = 256 * 2 + 16;   // bytes per LDS row of 256 bf16 (+16 B pad)

__device__ __forceinline__ void transpose8(const uint32_t (&in)[8][4], u32x4_t (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[e][q] = __builtin_amdgcn_perm(in[2 * q + 1][e >> 1], in[2 * q][e >> 1], sel);
  }
}

__global__ __launch_bounds__(256) void k_tn_partial(const uint16_t *__restrict__ Z, int64_t T, int64_t P,
                                                    const uint16_t *__restrict__ V, int r,
                                                    float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) char zt[64 * TPITCH];
  __shared__ __attribute__((aligned(16))) char vt[32 * TPITCH];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t p0 = (int64_t)blockIdx.x * 64;
  const int64_t c = blockIdx.y;
  const int64_t t0 = c * TN_CHUNK;

  {  // Z block: rows t0 + 8 tb + i, columns p0 + 8 pb + e
    const int tb = t & 31, pb = t >> 5;
    uint32_t in[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = t0 + 8 * tb + i;
      u32x4_t v = {0, 0, 0, 0};
      if (row < T) v = *reinterpret_cast<const u32x4_t *>(Z + row * P + p0 + 8 * pb);
#pragma unroll
      for (int q = 0; q < 4; ++q) in[i][q] = v[q];
    }
    u32x4_t o[8];
    transpose8(in, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4_t *>(zt + (8 * pb + e) * TPITCH + 16 * tb) = o[e];
  }
  if (t < 128) {  // V block: rows t0 + 8 tb + i, columns 8 jb + e (zero beyond r)
    const int tb = t & 31, jb = t >> 5;
    uint32_t in[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = t0 + 8 * tb + i;
      u32x4_t v = {0, 0, 0, 0};
      if (row < T && 8 * jb < r) v = *reinterpret_cast<const u32x4_t *>(V + row * r + 8 * jb);
#pragma unroll
      for (int q = 0; q < 4; ++q) in[i][q] = v[q];
    }
    u32x4_t o[8];
    transpose8(in, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4_t *>(vt + (8 * jb + e) * TPITCH + 16 * tb) = o[e];
  }
  __syncthreads();

  floatx4_t acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  const int prow = 16 * wave + (lane & 15);
  const int tq = 16 * (lane >> 4);       // byte offset of this lane's 8 t values inside a step
#pragma unroll
  for (int ts = 0; ts < TN_CHUNK / 32; ++ts) {
    const bf16x8 fa = *reinterpret_cast<const bf16x8 *>(zt + prow * TPITCH + 64 * ts + tq);
    const bf16x8 fb0 = *reinterpret_cast<const bf16x8 *>(vt + (lane & 15) * TPITCH + 64 * ts + tq);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb0, acc0, 0, 0, 0);
    if (r > 16) {
      const bf16x8 fb1 = *reinterpret_cast<const bf16x8 *>(vt + (16 + (lane & 15)) * TPITCH + 64 * ts + tq);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb1, acc1, 0, 0, 0);
    }
  }
  // lane holds column j = lane % 16 (+16) and rows p = 4 (lane / 16) + e of this wave's 16
  float *out = partial + c * P * r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t p = p0 + 16 * wave + 4 * (lane >> 4) + e;
    const int j = lane & 15;
    if (j < r) out[p * r + j] = acc0[e];
    if (r > 16 && 16 + j < r) out[p * r + 16 + j] = acc1[e];
  }
}

__global__ __launch_bounds__(256) void k_tn_reduce(const float *__restrict__ partial, int64_t n_chunks,
                                                   int64_t P, int r, float scale, int accumulate,
                                                   int transposed, float *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // index p * r + j
  if (i >= P * r) return;
  float s = partial[i];
  for (int64_t c = 1; c < n_chunks; ++c) s = __fadd_rn(s, partial[c * P * r + i]);
  const float v = __fmul_rn(scale, s);
  const int64_t p = i / r, j = i % r;
  float *o = transposed ? out + j * P + p : out + i;
  *o = accumulate ? __fadd_rn(*o, v) : v;
}

}  // namespace

lsn_status launch_rowproj(const uint16_t *act, int64_t M, int64_t K, const RowProjSet &set, hipStream_t s) {
  const dim3 grid((unsigned)((M + 15) / 16));
  const int nblk = (set.total + 15) / 16;
  if (nblk <= 2)
    hipLaunchKernelGGL((k_rowproj<2, 8>), grid, dim3(256), 0, s, act, M, K, set);
  else if (nblk <= 5)
    hipLaunchKernelGGL((k_rowproj<5, 4>), grid, dim3(256), 0, s, act, M, K, set);
  else
    hipLaunchKernelGGL((k_rowproj<8, 3>), grid, dim3(256), 0, s, act, M, K, set);
  return check_hip(hipGetLastError(), "k_rowproj launch");
}

lsn_status launch_rowproj(const uint16_t *act, int64_t M, int64_t K, const uint16_t *P, int r, uint16_t *out,
                          hipStream_t s) {
  RowProjSet set{};
  set.n = 1;
  set.total = r;
  set.P[0] = P;
  set.out[0] = out;
  set.r[0] = r;
  set.start[0] = 0;
  return launch_rowproj(act, M, K, set, s);
}

lsn_status launch_transpose(const uint16_t *src, int64_t rows, int64_t cols, uint16_t *dst, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose, dim3((unsigned)((rows * cols + 255) / 256)), dim3(256), 0, s, src, rows, cols,
                     dst);
  return check_hip(hipGetLastError(), "k_transpose launch");
}

lsn_status launch_tn_partial(const uint16_t *Z, int64_t T, int64_t P, const uint16_t *V, int r, float *partial,
                             hipStream_t s) {
  const int64_t n_chunks = (T + TN_CHUNK - 1) / TN_CHUNK;
  hipLaunchKernelGGL(k_tn_partial, dim3((unsigned)(P / 64), (unsigned)n_chunks), dim3(256), 0, s, Z, T, P, V,
                     r, partial);
  return check_hip(hipGetLastError(), "k_tn_partial launch");
}

lsn_status launch_tn_reduce(const float *partial, int64_t n_chunks, int64_t P, int r, float scale,
                            int accumulate, int transposed, float *out, hipStream_t s) {
  hipLaunchKernelGGL(k_tn_reduce, dim3((unsigned)((P * r + 255) / 256)), dim3(256), 0, s, partial, n_chunks, P,
                     r, scale, accumulate, transposed, out);
  return check_hip(hipGetLastError(), "k_tn_reduce launch");
}

}  // namespace lsn
