// Causal scaled dot-product attention with grouped key/value heads, forward and backward, on
// gfx950 MFMA (16x16x32 bf16, fp32 accumulate). The pages train Llama-3.1 and Qwen2.5 decoder
// layers ("Exact Layer Streaming", Abstract; "An 8B Fine-Tune Now Fits in 4 GB of VRAM": the
// decoder layer is the streamed unit) and print no attention formula; this is the definition
// those models use: query head h reads key/value head h / (n_q / n_kv), on packed sequences of
// S rows each,
//   s_ij = scale q_i.k_j (j <= i),  lse_i = log sum_j exp s_ij,  O_i = sum_j exp(s_ij - lse_i) v_j
// and the backward dV = P^T dO, dS = P (dO V^T - D), D_i = dO_i.O_i, dQ = scale dS K,
// dK = scale dS^T Q (dK, dV of a shared head summed over its query heads).
//
// Layout of the work (all kernels 4 waves; a wave owns 16 rows of its block):
//  * one MFMA lane column = one query (forward, dQ) or one key (dK/dV), so the softmax row
//    statistics and the rescaling stay inside a lane; the row max and sum need two shuffles;
//  * scores are computed transposed where that keeps the probabilities in registers as the
//    next product's operand: the MFMA reduction index k = 8 g + i (lane group g = lane / 16)
//    is mapped to rows 4 g + i (i < 4) and 16 + 4 g + i - 4 (i >= 4) of a 32-row step on both
//    operands, which is the register layout of two accumulator tiles;
//  * the operand that has to be read along the other dimension (V in the forward, Q, dO and K
//    in the backward) is staged in LDS transposed as well, by 8x8 register transposes.
// Every sum runs in a fixed order and no kernel uses atomics: the results depend only on the
// inputs. Keys and queries at or past S read as zeros and are never stored.

#include <cmath>

#include "common.h"

namespace lsn {
lsn_status require_gfx950();
bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kB = 64;                       // rows per block (queries or keys)
constexpr int kTP = kB * 2 + 16;             // pitch (bytes) of a transposed tile: [D][64] + pad
constexpr int kFwdThreads = 512;             // forward: 8 waves of 16 queries share each K/V tile
constexpr int kFwdQ = 128;                   // queries per forward workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Tile {
  static constexpr int RP = D * 2 + 16;      // pitch (bytes) of a row-major tile [64][D] + pad
  static constexpr int RM_BYTES = kB * RP;
  static constexpr int TR_BYTES = D * kTP;
  static constexpr int NBLK = 8 * (D / 8);   // 8x8 blocks of a 64 x D tile
};

__device__ __forceinline__ bf16x8 as_bf(u32x4_t v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 rows x 8 bf16 -> 8 columns x 8 rows (out[e] = column e of rows 0..7)
__device__ __forceinline__ void transpose8(const u32x4_t (&in)[8], u32x4_t (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[e][q] = __builtin_amdgcn_perm(in[2 * q + 1][e >> 1], in[2 * q][e >> 1], sel);
  }
}

// The 64 x D block of rows row0.. (rows >= nvalid read as zeros) of a bf16 matrix (row stride ld
// elements, head columns from `base`) is staged into LDS in two halves so that the global loads
// of the next block are in flight while the current one is computed: load_block fetches this
// thread's 8x8 block (`blk` in [0, NBLK): 8 rows of one 16-byte column chunk) into registers,
// store_block writes it row-major into `rm` and/or transposed into `tr`.
template <int D>
__device__ __forceinline__ void load_block(const uint16_t *__restrict__ base, int64_t ld, int64_t row0, int nvalid,
                                           int blk, u32x4_t (&in)[8]) {
  const int rb = blk & 7, cb = blk >> 3;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int row = 8 * rb + r;
    in[r] = row < nvalid ? *reinterpret_cast<const u32x4_t *>(base + (row0 + row) * ld + 8 * cb)
                         : u32x4_t{0u, 0u, 0u, 0u};
  }
}

template <int D>
__device__ __forceinline__ void store_block(const u32x4_t (&in)[8], int blk, char *rm, char *tr) {
  const int rb = blk & 7, cb = blk >> 3;
  if (rm) {
#pragma unroll
    for (int r = 0; r < 8; ++r) *reinterpret_cast<u32x4_t *>(rm + (8 * rb + r) * Tile<D>::RP + 16 * cb) = in[r];
  }
  if (tr) {
    u32x4_t out[8];
    transpose8(in, out);
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4_t *>(tr + (8 * cb + e) * kTP + 16 * rb) = out[e];
  }
}

__device__ __forceinline__ int rows_left(int64_t S, int64_t blk) {
  return (int)(S - blk * kB < kB ? S - blk * kB : kB);
}

// A/B fragment of a row-major tile: row `row`, reduction chunk `ch` (8 consecutive columns)
template <int D>
__device__ __forceinline__ bf16x8 rm_frag(const char *rm, int row, int ch) {
  return as_bf(*reinterpret_cast<const u32x4_t *>(rm + row * Tile<D>::RP + 16 * ch));
}

// A fragment of a transposed tile for reduction step c (32 rows of the original): original rows
// 32 c + 4 g + i (i < 4) and 32 c + 16 + 4 g + i - 4 (i >= 4), matching the accumulator layout
__device__ __forceinline__ bf16x8 tr_frag(const char *tr, int row, int c, int g) {
  const u32x2 lo = *reinterpret_cast<const u32x2 *>(tr + row * kTP + (32 * c + 4 * g) * 2);
  const u32x2 hi = *reinterpret_cast<const u32x2 *>(tr + row * kTP + (32 * c + 16 + 4 * g) * 2);
  return as_bf(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

// B fragment from two accumulator tiles (rows 4 g + e of tile t0 and of tile t1), to bf16
__device__ __forceinline__ bf16x8 acc_frag(floatx4 t0, floatx4 t1) {
  return as_bf(u32x4_t{pack_bf16x2(t0[0], t0[1]), pack_bf16x2(t0[2], t0[3]), pack_bf16x2(t1[0], t1[1]),
                       pack_bf16x2(t1[2], t1[3])});
}

// 2^x on the hardware exponential (v_exp_f32). Softmax weights below 2^-126 are of no
// consequence next to the row's largest (weight 1), so the library's denormal range handling
// is not needed; -inf gives 0.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Keep MFMA source registers from being reused before the MFMAs have read them.
#define AT_MFMA_FENCE()                    \
  do {                                     \
    __builtin_amdgcn_sched_barrier(0);     \
    asm volatile("s_nop 7\n\ts_nop 7");    \
  } while (0)

struct AttnArgs {
  int64_t n_seq, S;
  int n_q, n_kv;
  float scale;
  const uint16_t *q, *k, *v, *o, *dO;
  int64_t ldq, ldk, ldv, ldo, lddo;
  float *lse;        // [T][n_q]
  const float *dot;  // [T][n_q]  D_i = dO_i . O_i
  uint16_t *out_o, *dq, *dk, *dv;
  int64_t ld_out_o, lddq, lddk, lddv;
};

// ------------------------------------------------------------------------------------------
// Forward: one workgroup of 8 waves per (128-query block, sequence, query head), heaviest blocks
// first; a wave skips the key blocks that lie entirely after its 16 queries.
template <int D>
__global__ __launch_bounds__(kFwdThreads) void k_attn_fwd(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char k_rm[Tile<D>::RM_BYTES];
  __shared__ __attribute__((aligned(16))) char v_tr[Tile<D>::TR_BYTES];
  const int64_t nqb = (a.S + kFwdQ - 1) / kFwdQ, nkb = (a.S + kB - 1) / kB;
  const int64_t per = a.n_seq * a.n_q;
  const int64_t qb = nqb - 1 - blockIdx.x / per;
  const int64_t rest = blockIdx.x % per;
  const int64_t b = rest / a.n_q;
  const int h = (int)(rest % a.n_q), hk = h / (a.n_q / a.n_kv);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, col = lane & 15;
  const int64_t wq0 = qb * kFwdQ + 16 * wave;   // this wave's first query
  const int64_t q_in_seq = wq0 + col;
  const int64_t seq0 = b * a.S;
  const uint16_t *Kb = a.k + hk * D, *Vb = a.v + hk * D;

  bf16x8 qf[D / 32];   // B operand of S^T = K Q^T: query `col`, dims 32 c + 8 g ..
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    qf[c] = q_in_seq < a.S
                ? as_bf(*reinterpret_cast<const u32x4_t *>(a.q + (seq0 + q_in_seq) * a.ldq + h * D + 32 * c + 8 * g))
                : as_bf(u32x4_t{0u, 0u, 0u, 0u});
  floatx4 acc[D / 16];   // O^T: dims 16 j + 4 g + e of query `col`
#pragma unroll
  for (int j = 0; j < D / 16; ++j) acc[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f;
  const float c2 = a.scale * kLog2e;

  // threads 0..127 stage K (row-major), threads 128..255 stage V (transposed); the key blocks
  // run up to the one holding the workgroup's last query
  const int t = threadIdx.x;
  const bool stK = t < Tile<D>::NBLK, stV = t >= 128 && t - 128 < Tile<D>::NBLK;
  const int64_t kb_end = ((qb + 1) * kFwdQ < a.S ? (qb + 1) * kFwdQ : a.S);   // one past the last query
  const int64_t kb_last = (kb_end - 1) / kB < nkb - 1 ? (kb_end - 1) / kB : nkb - 1;
  u32x4_t pre[8];
  auto fetch = [&](int64_t kb) {
    if (stK) load_block<D>(Kb, a.ldk, seq0 + kb * kB, rows_left(a.S, kb), t, pre);
    else if (stV) load_block<D>(Vb, a.ldv, seq0 + kb * kB, rows_left(a.S, kb), t - 128, pre);
  };
  fetch(0);
  for (int64_t kb = 0; kb <= kb_last; ++kb) {
    __syncthreads();
    if (stK) store_block<D>(pre, t, k_rm, nullptr);
    else if (stV) store_block<D>(pre, t - 128, nullptr, v_tr);
    __syncthreads();
    if (kb < kb_last) fetch(kb + 1);   // in flight while this block is computed
    if (kb * kB > wq0 + 15) continue;  // every key of the block is after this wave's queries
    const bool diag = kb * kB + kB - 1 > wq0;   // some key of the block is after some query here

    // S^T tile tt: keys 16 tt + 4 g + e (rows) x query `col`; two tiles per half
    floatx4 s[4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      bf16x8 kf[2][D / 32];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kf[u][c] = rm_frag<D>(k_rm, 16 * (2 * hf + u) + col, 4 * c + g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s[2 * hf + u] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) s[2 * hf + u] = mfma(kf[u][c], qf[c], s[2 * hf + u]);
      }
      AT_MFMA_FENCE();
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) asm volatile("" ::"v"(kf[u][c]));
    }
    // online softmax in the exp2 domain
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = s[tt][e] * c2;
        if (diag && kb * kB + 16 * tt + 4 * g + e > q_in_seq) x = -INFINITY;
        s[tt][e] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = ex2(m - m_new);
    float rs = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[tt][e] = ex2(s[tt][e] - m_new);
        rs += s[tt][e];
      }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = m_new;
    // rescale only when some lane's running max moved (multiplying by exactly 1 changes nothing)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int j = 0; j < D / 16; ++j) acc[j] *= alpha;
    }
    // O^T += V^T P^T over the block's 64 keys (two reduction steps of 32)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 pf = acc_frag(s[2 * c], s[2 * c + 1]);
      bf16x8 vf[D / 16];
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) vf[jj] = tr_frag(v_tr, 16 * jj + col, c, g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) acc[jj] = mfma(vf[jj], pf, acc[jj]);
      AT_MFMA_FENCE();
      asm volatile("" ::"v"(pf));
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) asm volatile("" ::"v"(vf[jj]));
    }
  }
  if (q_in_seq < a.S) {
    const float inv = 1.0f / l;
    uint16_t *orow = a.out_o + (seq0 + q_in_seq) * a.ld_out_o + h * D;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const u32x2 w = {pack_bf16x2(acc[j][0] * inv, acc[j][1] * inv), pack_bf16x2(acc[j][2] * inv, acc[j][3] * inv)};
      *reinterpret_cast<u32x2 *>(orow + 16 * j + 4 * g) = w;
    }
    if (g == 0) a.lse[(seq0 + q_in_seq) * a.n_q + h] = (m + log2f(l)) * 0.69314718055994531f;
  }
}

// ------------------------------------------------------------------------------------------
// D_i = dO_i . O_i per (row, query head): D / 8 lanes per (row, head), 8 values per lane.
template <int D>
__global__ __launch_bounds__(kThreads) void k_attn_dot(AttnArgs a, float *__restrict__ dot) {
  constexpr int L = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t item = gid / L;   // (row, head)
  const int ch = (int)(gid % L);
  const int64_t T = a.n_seq * a.S;
  const bool ok = item < T * a.n_q;
  float sum = 0.0f;
  if (ok) {
    const int64_t row = item / a.n_q;
    const int h = (int)(item % a.n_q);
    const u32x4_t x = *reinterpret_cast<const u32x4_t *>(a.dO + row * a.lddo + h * D + 8 * ch);
    const u32x4_t y = *reinterpret_cast<const u32x4_t *>(a.o + row * a.ldo + h * D + 8 * ch);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = e >> 1, sh = 16 * (e & 1);
      sum += bf16_bits_to_f32((x[q] >> sh) & 0xffffu) * bf16_bits_to_f32((y[q] >> sh) & 0xffffu);
    }
  }
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (ok && ch == 0) dot[item] = sum;
}

// ------------------------------------------------------------------------------------------
// dK, dV: one workgroup per (key block, sequence, key/value head), heaviest (first) blocks
// first; a wave owns 16 keys (lane column = key) and loops over the group's query heads and the
// query blocks at or after its key block.
template <int D>
__global__ __launch_bounds__(kThreads) void k_attn_bwd_kv(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char q_rm[Tile<D>::RM_BYTES];
  __shared__ __attribute__((aligned(16))) char q_tr[Tile<D>::TR_BYTES];
  __shared__ __attribute__((aligned(16))) char d_rm[Tile<D>::RM_BYTES];
  __shared__ __attribute__((aligned(16))) char d_tr[Tile<D>::TR_BYTES];
  __shared__ float lse2_s[kB], dot_s[kB];
  const int64_t nb = (a.S + kB - 1) / kB;
  const int64_t per = a.n_seq * a.n_kv;
  const int64_t kb = blockIdx.x / per;
  const int64_t rest = blockIdx.x % per;
  const int64_t b = rest / a.n_kv;
  const int hk = (int)(rest % a.n_kv), grp = a.n_q / a.n_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, col = lane & 15;
  const int64_t k_in_seq = kb * kB + 16 * wave + col;
  const int64_t seq0 = b * a.S;
  const bool kvalid = k_in_seq < a.S;
  bf16x8 kf[D / 32], vf[D / 32];   // B operands: key `col`, dims 32 c + 8 g ..
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    kf[c] = kvalid ? as_bf(*reinterpret_cast<const u32x4_t *>(a.k + (seq0 + k_in_seq) * a.ldk + hk * D + 32 * c + 8 * g))
                   : as_bf(u32x4_t{0u, 0u, 0u, 0u});
    vf[c] = kvalid ? as_bf(*reinterpret_cast<const u32x4_t *>(a.v + (seq0 + k_in_seq) * a.ldv + hk * D + 32 * c + 8 * g))
                   : as_bf(u32x4_t{0u, 0u, 0u, 0u});
  }
  floatx4 dk[D / 16], dv[D / 16];   // dK^T, dV^T: dims 16 j + 4 g + e of key `col`
#pragma unroll
  for (int j = 0; j < D / 16; ++j) dk[j] = dv[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  const float c2 = a.scale * kLog2e;

  // threads 0..127 stage Q, threads 128..255 stage dO (both row-major and transposed), threads
  // 0..63 the rows' lse and D; the next (head, query block)'s tiles are fetched while the current
  // one is computed
  const int t = threadIdx.x;
  const bool stQ = t < Tile<D>::NBLK, stD = t >= 128 && t - 128 < Tile<D>::NBLK;
  u32x4_t pre[8];
  float pre_lse = INFINITY, pre_dot = 0.0f;
  auto fetch = [&](int hh, int64_t qb) {
    const int h = hk * grp + hh;
    const int nvalid = rows_left(a.S, qb);
    if (stQ) load_block<D>(a.q + h * D, a.ldq, seq0 + qb * kB, nvalid, t, pre);
    else if (stD) load_block<D>(a.dO + h * D, a.lddo, seq0 + qb * kB, nvalid, t - 128, pre);
    if (t < kB) {
      const bool ok = t < nvalid;
      pre_lse = ok ? a.lse[(seq0 + qb * kB + t) * a.n_q + h] * kLog2e : INFINITY;
      pre_dot = ok ? a.dot[(seq0 + qb * kB + t) * a.n_q + h] : 0.0f;
    }
  };
  fetch(0, kb);
  for (int hh = 0; hh < grp; ++hh) {
    for (int64_t qb = kb; qb < nb; ++qb) {
      __syncthreads();
      if (stQ) store_block<D>(pre, t, q_rm, q_tr);
      else if (stD) store_block<D>(pre, t - 128, d_rm, d_tr);
      if (t < kB) {
        lse2_s[t] = pre_lse;
        dot_s[t] = pre_dot;
      }
      __syncthreads();
      if (qb + 1 < nb) fetch(hh, qb + 1);
      else if (hh + 1 < grp) fetch(hh + 1, kb);

      // S and dP tiles tt: queries 16 tt + 4 g + e (rows) x key `col`; two tiles per half
      floatx4 s[4], dp[4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 qa[2][D / 32], da[2][D / 32];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            qa[u][c] = rm_frag<D>(q_rm, 16 * (2 * hf + u) + col, 4 * c + g);
            da[u][c] = rm_frag<D>(d_rm, 16 * (2 * hf + u) + col, 4 * c + g);
          }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int tt = 2 * hf + u;
          s[tt] = dp[tt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            s[tt] = mfma(qa[u][c], kf[c], s[tt]);
            dp[tt] = mfma(da[u][c], vf[c], dp[tt]);
          }
        }
        AT_MFMA_FENCE();
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            asm volatile("" ::"v"(qa[u][c]));
            asm volatile("" ::"v"(da[u][c]));
          }
      }
      // P and dS = P (dP - D)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qi = 16 * tt + 4 * g + e;
          float p = ex2(s[tt][e] * c2 - lse2_s[qi]);
          if (qb == kb && qb * kB + qi < k_in_seq) p = 0.0f;
          s[tt][e] = p;
          dp[tt][e] = p * (dp[tt][e] - dot_s[qi]);
        }
      // dV^T += dO^T P,  dK^T += Q^T dS  (reduction over the block's 64 queries, in two steps)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
          const bf16x8 bf = which == 0 ? acc_frag(s[2 * c], s[2 * c + 1]) : acc_frag(dp[2 * c], dp[2 * c + 1]);
          bf16x8 af[D / 16];
#pragma unroll
          for (int jj = 0; jj < D / 16; ++jj) af[jj] = tr_frag(which == 0 ? d_tr : q_tr, 16 * jj + col, c, g);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int jj = 0; jj < D / 16; ++jj) {
            if (which == 0) dv[jj] = mfma(af[jj], bf, dv[jj]);
            else dk[jj] = mfma(af[jj], bf, dk[jj]);
          }
          AT_MFMA_FENCE();
          asm volatile("" ::"v"(bf));
#pragma unroll
          for (int jj = 0; jj < D / 16; ++jj) asm volatile("" ::"v"(af[jj]));
        }
      }
    }
  }
  if (kvalid) {
    uint16_t *krow = a.dk + (seq0 + k_in_seq) * a.lddk + hk * D;
    uint16_t *vrow = a.dv + (seq0 + k_in_seq) * a.lddv + hk * D;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const u32x2 wk = {pack_bf16x2(dk[j][0] * a.scale, dk[j][1] * a.scale),
                        pack_bf16x2(dk[j][2] * a.scale, dk[j][3] * a.scale)};
      const u32x2 wv = {pack_bf16x2(dv[j][0], dv[j][1]), pack_bf16x2(dv[j][2], dv[j][3])};
      *reinterpret_cast<u32x2 *>(krow + 16 * j + 4 * g) = wk;
      *reinterpret_cast<u32x2 *>(vrow + 16 * j + 4 * g) = wv;
    }
  }
}

// ------------------------------------------------------------------------------------------
// dQ: one workgroup per (query block, sequence, query head), heaviest blocks first; a wave owns
// 16 queries (lane column = query) and loops over the key blocks up to its own.
template <int D>
__global__ __launch_bounds__(kFwdThreads) void k_attn_bwd_q(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char k_rm[Tile<D>::RM_BYTES];
  __shared__ __attribute__((aligned(16))) char k_tr[Tile<D>::TR_BYTES];
  __shared__ __attribute__((aligned(16))) char v_rm[Tile<D>::RM_BYTES];
  const int64_t nqb = (a.S + kFwdQ - 1) / kFwdQ, nkb = (a.S + kB - 1) / kB;
  const int64_t per = a.n_seq * a.n_q;
  const int64_t qb = nqb - 1 - blockIdx.x / per;
  const int64_t rest = blockIdx.x % per;
  const int64_t b = rest / a.n_q;
  const int h = (int)(rest % a.n_q), hk = h / (a.n_q / a.n_kv);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, col = lane & 15;
  const int64_t wq0 = qb * kFwdQ + 16 * wave;   // this wave's first query
  const int64_t q_in_seq = wq0 + col;
  const int64_t seq0 = b * a.S;
  const bool qvalid = q_in_seq < a.S;
  bf16x8 qf[D / 32], df[D / 32];   // B operands: query `col`, dims 32 c + 8 g ..
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    qf[c] = qvalid ? as_bf(*reinterpret_cast<const u32x4_t *>(a.q + (seq0 + q_in_seq) * a.ldq + h * D + 32 * c + 8 * g))
                   : as_bf(u32x4_t{0u, 0u, 0u, 0u});
    df[c] = qvalid ? as_bf(*reinterpret_cast<const u32x4_t *>(a.dO + (seq0 + q_in_seq) * a.lddo + h * D + 32 * c + 8 * g))
                   : as_bf(u32x4_t{0u, 0u, 0u, 0u});
  }
  const float lse2 = qvalid ? a.lse[(seq0 + q_in_seq) * a.n_q + h] * kLog2e : INFINITY;
  const float dq_dot = qvalid ? a.dot[(seq0 + q_in_seq) * a.n_q + h] : 0.0f;
  floatx4 acc[D / 16];   // dQ^T: dims 16 j + 4 g + e of query `col`
#pragma unroll
  for (int j = 0; j < D / 16; ++j) acc[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  const float c2 = a.scale * kLog2e;

  // threads 0..127 stage K (row-major and transposed), threads 128..255 stage V (row-major)
  const int t = threadIdx.x;
  const bool stK = t < Tile<D>::NBLK, stV = t >= 128 && t - 128 < Tile<D>::NBLK;
  u32x4_t pre[8];
  auto fetch = [&](int64_t kb) {
    if (stK) load_block<D>(a.k + hk * D, a.ldk, seq0 + kb * kB, rows_left(a.S, kb), t, pre);
    else if (stV) load_block<D>(a.v + hk * D, a.ldv, seq0 + kb * kB, rows_left(a.S, kb), t - 128, pre);
  };
  const int64_t kb_end = ((qb + 1) * kFwdQ < a.S ? (qb + 1) * kFwdQ : a.S);   // one past the last query
  const int64_t kb_last = (kb_end - 1) / kB < nkb - 1 ? (kb_end - 1) / kB : nkb - 1;
  fetch(0);
  for (int64_t kb = 0; kb <= kb_last; ++kb) {
    __syncthreads();
    if (stK) store_block<D>(pre, t, k_rm, k_tr);
    else if (stV) store_block<D>(pre, t - 128, v_rm, nullptr);
    __syncthreads();
    if (kb < kb_last) fetch(kb + 1);
    if (kb * kB > wq0 + 15) continue;  // every key of the block is after this wave's queries
    const bool diag = kb * kB + kB - 1 > wq0;

    // S^T and dP^T tiles tt: keys 16 tt + 4 g + e (rows) x query `col`; two tiles per half
    floatx4 s[4], dp[4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      bf16x8 ka[2][D / 32], va[2][D / 32];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          ka[u][c] = rm_frag<D>(k_rm, 16 * (2 * hf + u) + col, 4 * c + g);
          va[u][c] = rm_frag<D>(v_rm, 16 * (2 * hf + u) + col, 4 * c + g);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tt = 2 * hf + u;
        s[tt] = dp[tt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          s[tt] = mfma(ka[u][c], qf[c], s[tt]);
          dp[tt] = mfma(va[u][c], df[c], dp[tt]);
        }
      }
      AT_MFMA_FENCE();
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          asm volatile("" ::"v"(ka[u][c]));
          asm volatile("" ::"v"(va[u][c]));
        }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = ex2(s[tt][e] * c2 - lse2);
        if (diag && kb * kB + 16 * tt + 4 * g + e > q_in_seq) p = 0.0f;
        dp[tt][e] = p * (dp[tt][e] - dq_dot);
      }
    // dQ^T += K^T dS^T over the block's 64 keys (two steps of 32)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 sf = acc_frag(dp[2 * c], dp[2 * c + 1]);
      bf16x8 ka[D / 16];
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) ka[jj] = tr_frag(k_tr, 16 * jj + col, c, g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) acc[jj] = mfma(ka[jj], sf, acc[jj]);
      AT_MFMA_FENCE();
      asm volatile("" ::"v"(sf));
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) asm volatile("" ::"v"(ka[jj]));
    }
  }
  if (qvalid) {
    uint16_t *row = a.dq + (seq0 + q_in_seq) * a.lddq + h * D;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const u32x2 w = {pack_bf16x2(acc[j][0] * a.scale, acc[j][1] * a.scale),
                       pack_bf16x2(acc[j][2] * a.scale, acc[j][3] * a.scale)};
      *reinterpret_cast<u32x2 *>(row + 16 * j + 4 * g) = w;
    }
  }
}

bool al16(const void *p, int64_t ld) { return ((uintptr_t)p & 15) == 0 && ld % 8 == 0; }

lsn_status check_common(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim, float scale,
                        const char *who) {
  if (n_seq < 1 || S < 1 || n_q < 1 || n_kv < 1 || n_q % n_kv)
    return fail(LSN_E_ARG, "%s: need n_seq, S, n_q, n_kv >= 1 and n_kv dividing n_q", who);
  if (head_dim != 64 && head_dim != 128) return fail(LSN_E_ARG, "%s: head_dim must be 64 or 128", who);
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(LSN_E_ARG, "%s: scale must be finite and > 0", who);
  const int64_t nb = (S + kB - 1) / kB;
  if (nb * n_seq * (int64_t)n_q > 0x7fffffffLL) return fail(LSN_E_ARG, "%s: too many blocks for one launch", who);
  return LSN_OK;
}

size_t span(int64_t T, int64_t ld, int64_t width, int64_t elt) { return (size_t)(((T - 1) * ld + width) * elt); }

// A strided operand: T rows of `width` elements of `elt` bytes, row stride ld elements.
struct Strided {
  const void *p;
  int64_t ld, width, elt;
};

// Do two strided operands share a byte? Exact when the row strides (in bytes) are equal (column
// ranges of one matrix, e.g. q, k and v of a fused projection output); otherwise the address
// spans decide (conservative).
bool overlap(const Strided &a, const Strided &b, int64_t T) {
  if (!ranges_overlap(a.p, span(T, a.ld, a.width, a.elt), b.p, span(T, b.ld, b.width, b.elt))) return false;
  const int64_t row = a.ld * a.elt;
  if (row != b.ld * b.elt) return true;
  const int64_t diff = (int64_t)((uintptr_t)b.p - (uintptr_t)a.p);
  const int64_t r = ((diff % row) + row) % row;   // b's first byte within a's row period
  if (r + b.width * b.elt > row) return true;     // b wraps into the next row period
  return r < a.width * a.elt;                     // a holds bytes [0, width) of each period
}

}  // namespace
}  // namespace lsn

using namespace lsn;

extern "C" {

lsn_status attention_fwd(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim, const uint16_t *q,
                         int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v, int64_t ldv, float scale,
                         uint16_t *o, int64_t ldo, float *lse, void *stream) {
  lsn_status st = check_common(n_seq, S, n_q, n_kv, head_dim, scale, "attention_fwd");
  if (st != LSN_OK) return st;
  const int64_t D = head_dim, T = n_seq * S;
  if (!q || !k || !v || !o || !lse) return fail(LSN_E_ARG, "attention_fwd: null pointer");
  if (!al16(q, ldq) || !al16(k, ldk) || !al16(v, ldv) || !al16(o, ldo))
    return fail(LSN_E_ARG, "attention_fwd: q, k, v, o need 16-byte aligned rows (ld a multiple of 8)");
  if (ldq < n_q * D || ldk < n_kv * D || ldv < n_kv * D || ldo < n_q * D)
    return fail(LSN_E_ARG, "attention_fwd: a row stride is smaller than its heads");
  const Strided ins[] = {{q, ldq, n_q * D, 2}, {k, ldk, n_kv * D, 2}, {v, ldv, n_kv * D, 2}};
  const Strided outs[] = {{o, ldo, n_q * D, 2}, {lse, n_q, n_q, 4}};
  for (const Strided &out : outs)
    for (const Strided &in : ins)
      if (overlap(out, in, T)) return fail(LSN_E_ARG, "attention_fwd: an output overlaps an input");
  if (overlap(outs[0], outs[1], T)) return fail(LSN_E_ARG, "attention_fwd: o overlaps lse");
  st = require_gfx950();
  if (st != LSN_OK) return st;
  AttnArgs a{};
  a.n_seq = n_seq;
  a.S = S;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.scale = scale;
  a.q = q;
  a.k = k;
  a.v = v;
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldv = ldv;
  a.lse = lse;
  a.out_o = o;
  a.ld_out_o = ldo;
  const unsigned grid = (unsigned)(((S + kFwdQ - 1) / kFwdQ) * n_seq * n_q);
  if (head_dim == 128)
    hipLaunchKernelGGL(k_attn_fwd<128>, dim3(grid), dim3(kFwdThreads), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(k_attn_fwd<64>, dim3(grid), dim3(kFwdThreads), 0, (hipStream_t)stream, a);
  return check_hip(hipGetLastError(), "k_attn_fwd launch");
}

size_t attention_bwd_ws_bytes(int64_t n_seq, int64_t S, int32_t n_q) {
  if (n_seq < 1 || S < 1 || n_q < 1) return 0;
  return (size_t)(n_seq * S * n_q) * 4;
}

lsn_status attention_bwd(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim, const uint16_t *q,
                         int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v, int64_t ldv,
                         const uint16_t *o, int64_t ldo, const float *lse, const uint16_t *dO, int64_t lddo,
                         float scale, uint16_t *dq, int64_t lddq, uint16_t *dk, int64_t lddk, uint16_t *dv,
                         int64_t lddv, void *ws, size_t ws_bytes, void *stream) {
  lsn_status st = check_common(n_seq, S, n_q, n_kv, head_dim, scale, "attention_bwd");
  if (st != LSN_OK) return st;
  const int64_t D = head_dim, T = n_seq * S;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !ws)
    return fail(LSN_E_ARG, "attention_bwd: null pointer");
  if (!al16(q, ldq) || !al16(k, ldk) || !al16(v, ldv) || !al16(o, ldo) || !al16(dO, lddo) || !al16(dq, lddq) ||
      !al16(dk, lddk) || !al16(dv, lddv) || ((uintptr_t)ws & 15))
    return fail(LSN_E_ARG, "attention_bwd: tensors need 16-byte aligned rows (ld a multiple of 8)");
  if (ldq < n_q * D || ldk < n_kv * D || ldv < n_kv * D || ldo < n_q * D || lddo < n_q * D || lddq < n_q * D ||
      lddk < n_kv * D || lddv < n_kv * D)
    return fail(LSN_E_ARG, "attention_bwd: a row stride is smaller than its heads");
  if (ws_bytes < attention_bwd_ws_bytes(n_seq, S, n_q))
    return fail(LSN_E_ARG, "attention_bwd: workspace smaller than attention_bwd_ws_bytes");
  const Strided ins[] = {{q, ldq, n_q * D, 2}, {k, ldk, n_kv * D, 2}, {v, ldv, n_kv * D, 2},
                         {o, ldo, n_q * D, 2}, {lse, n_q, n_q, 4},       {dO, lddo, n_q * D, 2}};
  const Strided outs[] = {{dq, lddq, n_q * D, 2}, {dk, lddk, n_kv * D, 2}, {dv, lddv, n_kv * D, 2},
                          {ws, n_q, n_q, 4}};
  for (int i = 0; i < 4; ++i) {
    for (const Strided &in : ins)
      if (overlap(outs[i], in, T)) return fail(LSN_E_ARG, "attention_bwd: an output or the workspace overlaps an input");
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j], T)) return fail(LSN_E_ARG, "attention_bwd: outputs overlap");
  }
  st = require_gfx950();
  if (st != LSN_OK) return st;
  AttnArgs a{};
  a.n_seq = n_seq;
  a.S = S;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.scale = scale;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dO = dO;
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldv = ldv;
  a.ldo = ldo;
  a.lddo = lddo;
  a.lse = const_cast<float *>(lse);
  a.dot = static_cast<const float *>(ws);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.lddq = lddq;
  a.lddk = lddk;
  a.lddv = lddv;
  const hipStream_t hs = (hipStream_t)stream;
  const int64_t nb = (S + kB - 1) / kB;
  const unsigned dot_grid = (unsigned)((T * n_q * (D / 8) + kThreads - 1) / kThreads);
  const unsigned kv_grid = (unsigned)(nb * n_seq * n_kv);
  const unsigned q_grid = (unsigned)(((S + kFwdQ - 1) / kFwdQ) * n_seq * n_q);
  if (head_dim == 128) {
    hipLaunchKernelGGL(k_attn_dot<128>, dim3(dot_grid), dim3(kThreads), 0, hs, a, static_cast<float *>(ws));
    hipLaunchKernelGGL(k_attn_bwd_kv<128>, dim3(kv_grid), dim3(kThreads), 0, hs, a);
    hipLaunchKernelGGL(k_attn_bwd_q<128>, dim3(q_grid), dim3(kFwdThreads), 0, hs, a);
  } else {
    hipLaunchKernelGGL(k_attn_dot<64>, dim3(dot_grid), dim3(kThreads), 0, hs, a, static_cast<float *>(ws));
    hipLaunchKernelGGL(k_attn_bwd_kv<64>, dim3(kv_grid), dim3(kThreads), 0, hs, a);
    hipLaunchKernelGGL(k_attn_bwd_q<64>, dim3(q_grid), dim3(kFwdThreads), 0, hs, a);
  }
  return check_hip(hipGetLastError(), "attention backward launch");
}

}  // extern "C"
