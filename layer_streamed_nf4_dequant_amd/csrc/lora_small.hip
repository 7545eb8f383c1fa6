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
// Several jobs (activations of their own, the same M) run as grid rows of one launch.
// One workgroup of RP_WAVES waves per 16 rows; wave w takes the 64-wide K-steps w, w + RP_WAVES,
// ...; the partial results are added in wave order through LDS. Column block cb (16 columns of the
// concatenated P) is one MFMA 16x16x32 accumulator; NB is the exact number of column blocks.
// The activation is read in whole 128-byte lines (a lane loads 16 bytes of row lane / 8 and its
// twin 8 rows down, eight lanes per line): an MFMA fragment spans only 64 bytes of each of 16
// rows, and half-line loads ran the stream about 30% slower. The wave turns its 16 x 64 block
// into fragments through its own 2 KB of LDS (chunk c of row r at slot c ^ ((r ^ r >> 3) & 7), so
// neither the row writes nor the 16-row fragment reads conflict). P is small and read from L2 in
// fragment layout.
// The work per K-step is tiny (two activation fragments, 2 NB weight fragments, 2 NB MFMAs), so
// the loads run ahead: each wave keeps the operands of DEPTH K-steps in registers and issues the
// loads of step i + DEPTH as it consumes step i (1-2 steps measured fastest; deeper queues ran
// 10-20% slower). Every
// load is unconditional (columns past the total read a valid row and are never stored; steps
// past the wave's last re-read its last step), so the load counter waits stay exact.
// ---------------------------------------------------------------------------------------------
constexpr int RP_WAVES = 8;
__device__ __forceinline__ int rp_xoff(int r, int c) { return r * 128 + 16 * (c ^ ((r ^ (r >> 3)) & 7)); }

template <int NB, int DEPTH>
__global__ __launch_bounds__(64 * RP_WAVES) void k_rowproj(int64_t M, RowProjJobs jobs) {
  __shared__ floatx4_t part[RP_WAVES][NB][64];
  __shared__ __attribute__((aligned(16))) char xs[RP_WAVES][16 * 128];
  // job blockIdx.y: its own activation [M][K] and matrices
  const RowProjJob &J = jobs.job[blockIdx.y];
  const uint16_t *__restrict__ act = J.act;
  const int64_t K = J.K;
  const RowProjSet &set = J.set;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int kq = 8 * (lane >> 4);
  const int nks = (int)(K / 64);
  // the concatenated row c of P: group g, local row c - start[g] (c clamped to the last row)
  const uint16_t *prow[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int c = min(16 * cb + (lane & 15), set.total - 1);
    int g = 0;
#pragma unroll
    for (int q = 1; q < 8; ++q) g += (q < set.n && c >= set.start[q]) ? 1 : 0;
    prow[cb] = set.P[g] + (int64_t)(c - set.start[g]) * K + kq;
  }
  // activation lines: rows xr and 8 + xr of the block (clamped rows are never stored), chunk xc
  const int xr = lane >> 3, xc = lane & 7;
  const uint16_t *xa0 = act + min(m0 + xr, M - 1) * K + 8 * xc;
  const uint16_t *xa1 = act + min(m0 + 8 + xr, M - 1) * K + 8 * xc;
  char *xw = xs[wave];
  const int wo0 = rp_xoff(xr, xc), wo1 = rp_xoff(8 + xr, xc);
  const int ro0 = rp_xoff(lane & 15, lane >> 4), ro1 = rp_xoff(lane & 15, 4 + (lane >> 4));
  floatx4_t acc[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) acc[cb] = floatx4_t{0, 0, 0, 0};
  u32x4_t va[DEPTH][2], vb[DEPTH][NB][2];
  // K-step of this wave's i-th iteration, clamped (a clamped step is loaded but not used)
  auto load = [&](int i, u32x4_t (&a_)[2], u32x4_t (&b_)[NB][2]) {
    const int64_t k = (int64_t)min(wave + RP_WAVES * i, nks - 1) * 64;
    a_[0] = *reinterpret_cast<const u32x4_t *>(xa0 + k);
    a_[1] = *reinterpret_cast<const u32x4_t *>(xa1 + k);
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      b_[cb][0] = *reinterpret_cast<const u32x4_t *>(prow[cb] + k);
      b_[cb][1] = *reinterpret_cast<const u32x4_t *>(prow[cb] + k + 32);
    }
  };
  const int iters = (nks - wave + RP_WAVES - 1) / RP_WAVES;   // K-steps of this wave (may be 0)
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    load(d, va[d], vb[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // at least one pass, with no guard between the loads above and the loop: a guard lets the
  // compiler sink some of those loads past it, and the load waits inside the loop then merge two
  // different load orders and come out too strict
  int i0 = 0;
  do {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      // the wave's 16 x 64 block into fragment layout (LDS operations of a wave run in order, so
      // the reads see these writes, and the next step's writes follow these reads)
      *reinterpret_cast<u32x4_t *>(xw + wo0) = va[d][0];
      *reinterpret_cast<u32x4_t *>(xw + wo1) = va[d][1];
      u32x4_t a0 = *reinterpret_cast<const u32x4_t *>(xw + ro0);
      u32x4_t a1 = *reinterpret_cast<const u32x4_t *>(xw + ro1);
      // a step past the wave's last contributes zero (a select, not a branch, so the loop body
      // is straight-line code and its load waits are exact)
      const uint32_t keep = i0 + d < iters ? 0xffffffffu : 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0[e] &= keep;
        a1[e] &= keep;
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(vb[d][cb][0]), acc[cb], 0, 0, 0);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(vb[d][cb][1]), acc[cb], 0, 0, 0);
      }
      load(i0 + d + DEPTH, va[d], vb[d]);
      // keep the loads in program order: the scheduler would otherwise sink them to their uses
      // and undo the pipelining
      __builtin_amdgcn_sched_barrier(0);
    }
    i0 += DEPTH;
  } while (i0 < iters);
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) part[wave][cb][lane] = acc[cb];
  __syncthreads();
  // the waves finish the column blocks; lane holds column c = 16 cb + lane % 16 and rows
  // 4 (lane / 16) + e
  for (int cb = wave; cb < NB; cb += RP_WAVES) {
    floatx4_t sum = part[0][cb][lane];
#pragma unroll
    for (int w = 1; w < RP_WAVES; ++w) {
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

// several small transposes in one launch (a layer's B -> B^T and A -> A^T): job g owns the
// elements [first[g], first[g] + rows[g] * cols[g]) of the flattened index space
__global__ __launch_bounds__(256) void k_transpose_many(TransposeSet set) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int g = 0;
#pragma unroll
  for (int q = 1; q < kMaxTransposes; ++q)
    if (q < set.n && i >= set.first[q]) g = q;
  const int64_t li = i - set.first[g];
  if (li >= set.rows[g] * set.cols[g]) return;
  const int64_t r = li / set.cols[g], c = li % set.cols[g];
  set.dst[g][c * set.rows[g] + r] = set.src[g][li];
}


// ---------------------------------------------------------------------------------------------
// split-T partial products: partial[c][p][j] = sum over t in chunk c (TN_CHUNK = 256 rows) of
// Z[t][p] V[t][j]. Workgroup = (256 columns p, one chunk), walked in 4 blocks of 64 rows. Both
// operands are t-major in memory, so each thread loads an 8 x 8 block (8 rows, 16 bytes each;
// 32 lanes cover 512 contiguous bytes of a row) and transposes it in registers into LDS as
// [p][t] rows (128 bytes; 16-byte chunk ch of row w sits at slot ch ^ ((w ^ w >> 3) & 7), which
// keeps both the transposed writes and the fragment reads free of bank conflicts), V likewise
// as [j][t]; then each
// wave runs its 64 columns against V on 16x16x32 MFMAs. The next block's loads are issued
// before the current block's MFMAs. The t order of the sums (steps of 32 in increasing t) is
// the same as a single pass over the chunk.
// ---------------------------------------------------------------------------------------------
constexpr int TN_COLS = 256;          // columns p per workgroup
constexpr int TN_ROWS = 64;           // rows t per LDS block
constexpr int TPITCH = TN_ROWS * 2;       // bytes per LDS row of 64 bf16

__device__ __forceinline__ int tn_off(int row, int ch) { return row * TPITCH + 16 * (ch ^ ((row ^ (row >> 3)) & 7)); }

__device__ __forceinline__ void transpose8(const uint32_t (&in)[8][4], u32x4_t (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[e][q] = __builtin_amdgcn_perm(in[2 * q + 1][e >> 1], in[2 * q][e >> 1], sel);
  }
}

// Several jobs in one launch: job g owns workgroups wg0 .. wg0 + (its column blocks x chunks) - 1,
// column block fastest.
template <bool WIDE>   // r > 16: two 16-column blocks of V
__global__ __launch_bounds__(256) void k_tn_partial(int64_t T, TnJobs jobs) {
  __shared__ __attribute__((aligned(16))) char zt[TN_COLS * TPITCH];
  __shared__ __attribute__((aligned(16))) char vt[32 * TPITCH];
  int g = 0;
#pragma unroll
  for (int q = 1; q < kMaxTn; ++q)
    if (q < jobs.n && (int64_t)blockIdx.x >= jobs.job[q].wg0) g = q;
  const TnJob &J = jobs.job[g];
  const uint16_t *__restrict__ Z = J.Z;
  const uint16_t *__restrict__ V = J.V;
  const int64_t P = J.P;
  const int r = J.r;
  float *__restrict__ partial = J.partial;
  const int64_t npb = (P + TN_COLS - 1) / TN_COLS;
  const int64_t local = (int64_t)blockIdx.x - J.wg0;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t p0 = (local % npb) * TN_COLS;
  const int64_t c = local / npb;
  const int64_t t0 = c * TN_CHUNK;
  const int cg = t & 31, rg = t >> 5;         // Z: columns p0 + 8 cg .. +7, rows 8 rg .. +7 of a block
  const bool col_ok = p0 + 8 * cg < P;
  const int vjg = t & 3, vrg = (t >> 2) & 7;  // V (threads < 32): columns 8 vjg .. +7, rows 8 vrg .. +7
  uint32_t zin[8][4], vin[8][4];
  auto load = [&](int rb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = t0 + TN_ROWS * rb + 8 * rg + i;
      u32x4_t v = {0, 0, 0, 0};
      if (row < T && col_ok) v = *reinterpret_cast<const u32x4_t *>(Z + row * P + p0 + 8 * cg);
#pragma unroll
      for (int q = 0; q < 4; ++q) zin[i][q] = v[q];
    }
    if (t < 32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t row = t0 + TN_ROWS * rb + 8 * vrg + i;
        u32x4_t v = {0, 0, 0, 0};
        if (row < T && 8 * vjg < r) v = *reinterpret_cast<const u32x4_t *>(V + row * r + 8 * vjg);
#pragma unroll
        for (int q = 0; q < 4; ++q) vin[i][q] = v[q];
      }
    }
  };
  floatx4_t acc[4][WIDE ? 2 : 1];
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
#pragma unroll
    for (int jb = 0; jb < (WIDE ? 2 : 1); ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[pb][jb][e] = 0.0f;
  load(0);
  for (int rb = 0; rb < TN_CHUNK / TN_ROWS; ++rb) {
    {
      u32x4_t o[8];
      transpose8(zin, o);
#pragma unroll
      for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4_t *>(zt + tn_off(8 * cg + e, rg)) = o[e];
      if (t < 32) {
        transpose8(vin, o);
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4_t *>(vt + tn_off(8 * vjg + e, vrg)) = o[e];
      }
    }
    __syncthreads();
    if (rb + 1 < TN_CHUNK / TN_ROWS) load(rb + 1);
    // All fragments of the block are read first and stay live until after the closing barrier:
    // with the reads interleaved, the compiler reused an MFMA's source registers for address
    // arithmetic right after issuing it, and rows i % 4 in {2, 3} of that MFMA came out wrong
    // (no wait states were inserted between the MFMA and the overwrite).
    bf16x8 fa[TN_ROWS / 32][4], fb[TN_ROWS / 32][WIDE ? 2 : 1];
#pragma unroll
    for (int ks = 0; ks < TN_ROWS / 32; ++ks) {
      const int ch = 4 * ks + (lane >> 4);    // chunk of this lane's 8 t values
#pragma unroll
      for (int jb = 0; jb < (WIDE ? 2 : 1); ++jb)
        fb[ks][jb] = *reinterpret_cast<const bf16x8 *>(vt + tn_off(16 * jb + (lane & 15), ch));
#pragma unroll
      for (int pb = 0; pb < 4; ++pb)
        fa[ks][pb] = *reinterpret_cast<const bf16x8 *>(zt + tn_off(64 * wave + 16 * pb + (lane & 15), ch));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < TN_ROWS / 32; ++ks)
#pragma unroll
      for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int jb = 0; jb < (WIDE ? 2 : 1); ++jb)
          acc[pb][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks][pb], fb[ks][jb], acc[pb][jb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7");   // 16 wait states before anything may overwrite them
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < TN_ROWS / 32; ++ks) {
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) asm volatile("" ::"v"(fa[ks][pb]));
#pragma unroll
      for (int jb = 0; jb < (WIDE ? 2 : 1); ++jb) asm volatile("" ::"v"(fb[ks][jb]));
    }
  }
  // lane holds column j = lane % 16 (+16) and rows p = 4 (lane / 16) + e of each 16-row block
  float *out = partial + c * P * r;
  const int j = lane & 15;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t p = p0 + 64 * wave + 16 * pb + 4 * (lane >> 4) + e;
      if (p < P) {
        if (j < r) out[p * r + j] = acc[pb][0][e];
        if constexpr (WIDE)
          if (16 + j < r) out[p * r + 16 + j] = acc[pb][WIDE ? 1 : 0][e];
      }
    }
}

// job g owns the elements i0 .. i0 + P r - 1 of the flattened index space (whole workgroups)
__global__ __launch_bounds__(256) void k_tn_reduce(int64_t n_chunks, TnRedJobs jobs) {
  const int64_t b = (int64_t)blockIdx.x * 256;
  int g = 0;
#pragma unroll
  for (int q = 1; q < kMaxTn; ++q)
    if (q < jobs.n && b >= jobs.job[q].i0) g = q;
  const TnRedJob &J = jobs.job[g];
  const float *__restrict__ partial = J.partial;
  const int64_t P = J.P;
  const int r = J.r;
  const float scale = J.scale;
  float *__restrict__ out = J.out;
  const int accumulate = J.accumulate, transposed = J.transposed;
  const int64_t i = b - J.i0 + threadIdx.x;   // index p * r + j
  if (i >= P * r) return;
  float s = partial[i];
  for (int64_t c = 1; c < n_chunks; ++c) s = __fadd_rn(s, partial[c * P * r + i]);
  const float v = __fmul_rn(scale, s);
  const int64_t p = i / r, j = i % r;
  float *o = transposed ? out + j * P + p : out + i;
  *o = accumulate ? __fadd_rn(*o, v) : v;
}

}  // namespace

lsn_status launch_rowproj_jobs(int64_t M, const RowProjJobs &jobs, hipStream_t s) {
  if (jobs.n < 1 || jobs.n > 8) return LSN_E_ARG;
  const int nb = (jobs.job[0].set.total + 15) / 16;
  for (int g = 1; g < jobs.n; ++g)
    if ((jobs.job[g].set.total + 15) / 16 != nb) return LSN_E_ARG;
  const dim3 grid((unsigned)((M + 15) / 16), (unsigned)jobs.n), block(64 * RP_WAVES);
  switch (nb) {
    case 1: hipLaunchKernelGGL((k_rowproj<1, 2>), grid, block, 0, s, M, jobs); break;
    case 2: hipLaunchKernelGGL((k_rowproj<2, 2>), grid, block, 0, s, M, jobs); break;
    case 3: hipLaunchKernelGGL((k_rowproj<3, 1>), grid, block, 0, s, M, jobs); break;
    case 4: hipLaunchKernelGGL((k_rowproj<4, 1>), grid, block, 0, s, M, jobs); break;
    case 5: hipLaunchKernelGGL((k_rowproj<5, 1>), grid, block, 0, s, M, jobs); break;
    case 6: hipLaunchKernelGGL((k_rowproj<6, 1>), grid, block, 0, s, M, jobs); break;
    case 7: hipLaunchKernelGGL((k_rowproj<7, 1>), grid, block, 0, s, M, jobs); break;
    case 8: hipLaunchKernelGGL((k_rowproj<8, 1>), grid, block, 0, s, M, jobs); break;
    default: return LSN_E_ARG;
  }
  return check_hip(hipGetLastError(), "k_rowproj launch");
}

lsn_status launch_rowproj(const uint16_t *act, int64_t M, int64_t K, const RowProjSet &set, hipStream_t s) {
  RowProjJobs jobs{};
  jobs.n = 1;
  jobs.job[0].act = act;
  jobs.job[0].K = K;
  jobs.job[0].set = set;
  return launch_rowproj_jobs(M, jobs, s);
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


lsn_status launch_transpose_many(TransposeSet set, hipStream_t s) {
  int64_t total = 0;
  for (int g = 0; g < set.n; ++g) {
    set.first[g] = total;
    total += set.rows[g] * set.cols[g];
  }
  if (total == 0) return LSN_OK;
  hipLaunchKernelGGL(k_transpose_many, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, set);
  return check_hip(hipGetLastError(), "k_transpose_many launch");
}

lsn_status launch_tn_partial_jobs(int64_t T, TnJobs jobs, hipStream_t s) {
  if (jobs.n < 1 || jobs.n > kMaxTn) return LSN_E_ARG;
  const int64_t n_chunks = (T + TN_CHUNK - 1) / TN_CHUNK;
  int64_t wg = 0;
  bool wide = false;
  for (int g = 0; g < jobs.n; ++g) {
    jobs.job[g].wg0 = wg;
    wg += ((jobs.job[g].P + TN_COLS - 1) / TN_COLS) * n_chunks;
    wide = wide || jobs.job[g].r > 16;
  }
  if (wide)
    hipLaunchKernelGGL(k_tn_partial<true>, dim3((unsigned)wg), dim3(256), 0, s, T, jobs);
  else
    hipLaunchKernelGGL(k_tn_partial<false>, dim3((unsigned)wg), dim3(256), 0, s, T, jobs);
  return check_hip(hipGetLastError(), "k_tn_partial launch");
}

lsn_status launch_tn_partial(const uint16_t *Z, int64_t T, int64_t P, const uint16_t *V, int r, float *partial,
                             hipStream_t s) {
  TnJobs jobs{};
  jobs.n = 1;
  jobs.job[0] = TnJob{Z, P, V, r, partial, 0};
  return launch_tn_partial_jobs(T, jobs, s);
}

lsn_status launch_tn_reduce_jobs(int64_t n_chunks, TnRedJobs jobs, hipStream_t s) {
  if (jobs.n < 1 || jobs.n > kMaxTn) return LSN_E_ARG;
  int64_t i0 = 0;
  for (int g = 0; g < jobs.n; ++g) {
    jobs.job[g].i0 = i0;
    i0 += (jobs.job[g].P * jobs.job[g].r + 255) / 256 * 256;     // whole workgroups per job
  }
  hipLaunchKernelGGL(k_tn_reduce, dim3((unsigned)(i0 / 256)), dim3(256), 0, s, n_chunks, jobs);
  return check_hip(hipGetLastError(), "k_tn_reduce launch");
}

lsn_status launch_tn_reduce(const float *partial, int64_t n_chunks, int64_t P, int r, float scale,
                            int accumulate, int transposed, float *out, hipStream_t s) {
  TnRedJobs jobs{};
  jobs.n = 1;
  jobs.job[0] = TnRedJob{partial, P, r, scale, accumulate, transposed, out, 0};
  return launch_tn_reduce_jobs(n_chunks, jobs, s);
}

}  // namespace lsn
