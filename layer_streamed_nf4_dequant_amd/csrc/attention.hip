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
// Layout of the work (forward: 4 waves of 32 queries as two groups of 16; dK/dV: 4 waves of 16
// keys; dQ: 8 waves of 16 queries):
//  * one MFMA lane column = one query (forward, dQ) or one key (dK/dV), so the softmax row
//    statistics and the rescaling stay inside a lane; the row max and sum need two shuffles;
//  * scores are computed transposed where that keeps the probabilities in registers as the
//    next product's operand: the MFMA reduction index k = 8 g + i (lane group g = lane / 16)
//    is mapped to rows 4 g + i (i < 4) and 16 + 4 g + i - 4 (i >= 4) of a 32-row step on both
//    operands, which is the register layout of two accumulator tiles;
//  * K, V, Q and dO blocks are staged row-major in LDS by direct-to-LDS loads, and the operand
//    that has to be read along the other dimension (V in the forward, Q, dO and K in the
//    backward) comes from the same tile by the gfx950 LDS transpose read.
// Every sum runs in a fixed order and no kernel uses atomics: the results depend only on the
// inputs. Keys and queries at or past S read as zeros and are never stored.

#include <cmath>

#include <type_traits>

#include "common.h"
#include "glue_math.h"

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
constexpr int kFwdQ = 128;                   // queries per forward / dQ workgroup
constexpr int kFwd2Threads = 256;            // forward: 4 waves of 32 queries (two groups of 16)
// dQ: groups of 16 queries per wave. Two groups (4 waves of 32 queries) need 327 registers per
// lane without spilling, so one wave per SIMD, and the whole backward ran 13% slower at the 8B
// shape than with one group (8 waves of 16, two per SIMD); squeezed into two waves per SIMD they
// spill 64 bytes per lane and the backward ran 2.5% faster. One group, without spills.
constexpr int kDqGroups = 1;
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
  // rope != 0: dq and dk are rotated back (the inverse rotary embedding) before they are stored
  int rope, rope_n_pos;
  const float *rope_cs;        // (cos, sin) table [rope_n_pos][D / 2]
  const int32_t *rope_pos;     // [T] table row of each token row
  // dK, dV pass split over the group's query heads (kv_split workgroups per key block, 1 or 2);
  // with 2, each writes fp32 partial sums [part][dK, dV][T][n_kv][D] to kv_part
  int kv_split;
  float *kv_part;
};

// Store one row's gradient (dims 16 j + 4 g + e of the row held by the lane, g = lane / 16):
// bf16( acc * mul ); with rot, each pair (i, i + D/2) of the rounded values is then turned back
// by its angle (rope_apply's inverse rotation, the same arithmetic), and rounded again. Pair
// partners sit in the same lane: dims 16 j + .. and 16 (j + D/32) + ..
template <int D>
__device__ __forceinline__ void store_grad_row(uint16_t *dst, const floatx4 (&acc)[D / 16], float mul, bool rot,
                                               const AttnArgs &a, int64_t row, int g) {
  float v[D / 16][4];
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) v[j][e] = acc[j][e] * mul;
  if (rot) {
    const int pos = min(max(a.rope_pos[row], 0), a.rope_n_pos - 1);
    const float *cs = a.rope_cs + (int64_t)pos * D;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const int f0 = 16 * j + 4 * g;   // pair index of v[j][0]
      const floatx4 c01 = *reinterpret_cast<const floatx4 *>(cs + 2 * f0);
      const floatx4 c23 = *reinterpret_cast<const floatx4 *>(cs + 2 * f0 + 4);
      const float cv[4] = {c01[0], c01[2], c23[0], c23[2]};
      const float sv[4] = {c01[1], c01[3], c23[1], c23[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = bf16f(f2bf(v[j][e])), x2 = bf16f(f2bf(v[j + D / 32][e]));
        rope_pair(x1, x2, cv[e], __fmul_rn(-1.0f, sv[e]), v[j][e], v[j + D / 32][e]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const u32x2 w = {pack_bf16x2(v[j][0], v[j][1]), pack_bf16x2(v[j][2], v[j][3])};
    *reinterpret_cast<u32x2 *>(dst + 16 * j + 4 * g) = w;
  }
}

// ------------------------------------------------------------------------------------------
// Row-major tiles staged by direct-to-LDS loads. A 64-row tile of D bf16 columns is 64 rows of
// 2D bytes; 16-byte chunk c of row r sits at physical chunk c ^ swz(r), so that a fragment read
// (16 consecutive rows, one chunk each) and a transpose read (4 consecutive rows, 32 bytes each)
// both touch every bank at most once. A direct load (one wave instruction) fills one 1 KB LDS
// segment, lane l writing bytes 16 l .. 16 l + 15: lane l loads the global chunk that belongs at
// its slot. Rows past the block's valid rows load the last valid row (finite values: the keys
// they stand for are masked, and their P is exactly 0).
// ------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);   // 16 chunks per row
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);                // 8 chunks; two rows per bank line
}

template <int D>
struct DTile {
  static constexpr int ROW = 2 * D;              // bytes per row
  static constexpr int BYTES = kB * ROW;          // one 64-row tile
  static constexpr int SEGS = BYTES / 1024;       // direct loads per tile
  static constexpr int CH = D / 8;                // 16-byte chunks per row
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base, int64_t bytes) {
  // raw buffer, no stride; loads past num_records return 0 (never fault)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Byte offset (from the tile's first row in global memory) of the chunk lane `lane` loads for
// segment `seg`; rows at or past `nvalid` read row nvalid - 1.
template <int D>
__device__ __forceinline__ uint32_t seg_voff(int seg, int lane, int64_t ld, int nvalid) {
  constexpr int RPS = 1024 / DTile<D>::ROW;      // rows per segment
  const int row = seg * RPS + lane / DTile<D>::CH;
  const int c = (lane % DTile<D>::CH) ^ swz<D>(row);
  const int grow = row < nvalid ? row : nvalid - 1;
  return (uint32_t)((grow * ld + 8 * c) * 2);
}

__device__ __forceinline__ void direct_load(__amdgpu_buffer_rsrc_t rs, char *lds_seg, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)lds_seg, 16, voff, soff, 0, 0);
}

// the wave's loads of this block must have landed and its reads of the stage about to be
// refilled must have returned; then all waves meet
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0070);            // vmcnt(0), lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// A/B fragment of a row-major tile: row `row`, 8 columns of chunk `ch`
template <int D>
__device__ __forceinline__ bf16x8 sw_frag(const char *tile, int row, int ch) {
  return as_bf(*reinterpret_cast<const u32x4_t *>(tile + row * DTile<D>::ROW + ((ch ^ swz<D>(row)) << 4)));
}

// Transposed fragment from a row-major tile: this lane's column 16 j + (lane % 16) at the rows
// of reduction step c that the accumulator layout pairs with lane group g: rows 32 c + 4 g + i
// (i < 4) and 32 c + 16 + 4 g + i - 4 (i >= 4), read with the gfx950 LDS transpose read (each
// 16-lane group reads a 4-row x 16-column block; lane l points at row l / 4, columns 4 (l % 4)
// .. + 3, and receives column l of the 4 rows).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag_rm(const char *tile, int j, int c, int g, int lane) {
  const int sl = lane & 15;
  const int ch = 2 * j + ((sl & 3) >> 1);
  const int r0 = 32 * c + 4 * g + (sl >> 2), r1 = r0 + 16;
  lds_char *p0 = (lds_char *)(tile + r0 * DTile<D>::ROW + ((ch ^ swz<D>(r0)) << 4) + 8 * (sl & 1));
  lds_char *p1 = (lds_char *)(tile + r1 * DTile<D>::ROW + ((ch ^ swz<D>(r1)) << 4) + 8 * (sl & 1));
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One row's fp32 partial sum (dims 16 j + 4 g + e of the row held by the lane), unscaled.
template <int D>
__device__ __forceinline__ void store_part_row(float *dst, const floatx4 (&acc)[D / 16], int g) {
#pragma unroll
  for (int j = 0; j < D / 16; ++j) *reinterpret_cast<floatx4 *>(dst + 16 * j + 4 * g) = acc[j];
}

// ------------------------------------------------------------------------------------------
// Forward: one workgroup of 4 waves per (128-query block, sequence, query head), heaviest blocks
// first. A wave owns 32 queries as two groups of 16 (one query of each group per MFMA lane
// column), so every K and V fragment it reads from LDS feeds the MFMAs of both groups: half the
// LDS reads per MFMA of 16-query waves. A wave skips the key blocks that lie entirely after its
// queries. K and V blocks of 64 keys stream through two LDS stages by direct-to-LDS loads (each
// wave issues its share of the next block right after the barrier that frees its stage), so the
// workgroup meets once per block and no thread spends instructions on staging.
constexpr float kLazy = 8.0f;   // log2 of the largest probability between rescales
template <int D>
__global__ __launch_bounds__(kFwd2Threads, 2) void k_attn_fwd(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * DTile<D>::BYTES];   // [stage][K, V]
  constexpr int NG = 2;                            // query groups of 16 per wave
  const int nqb = (int)((a.S + kFwdQ - 1) / kFwdQ);
  const int64_t per = a.n_seq * a.n_q;
  const int qb = nqb - 1 - (int)(blockIdx.x / per);
  const int64_t rest = blockIdx.x % per;
  const int64_t b = rest / a.n_q;
  const int h = (int)(rest % a.n_q), hk = h / (a.n_q / a.n_kv);
  // (the wave index in a scalar register, so that the direct loads' LDS destinations are scalar)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g = lane >> 4,
            col = lane & 15;
  const int S = (int)a.S;
  const int wq0 = qb * kFwdQ + 16 * NG * wave;     // this wave's first query
  const int64_t seq0 = b * a.S;
  int qis[NG];                                     // the lane's query of each group
#pragma unroll
  for (int u = 0; u < NG; ++u) qis[u] = wq0 + 16 * u + col;

  bf16x8 qf[NG][D / 32];   // B operands of S^T = K Q^T: query qis[u], dims 32 c + 8 g ..
#pragma unroll
  for (int u = 0; u < NG; ++u)
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      qf[u][c] = qis[u] < S ? as_bf(*reinterpret_cast<const u32x4_t *>(a.q + (seq0 + qis[u]) * a.ldq + h * D + 32 * c + 8 * g))
                            : as_bf(u32x4_t{0u, 0u, 0u, 0u});
  floatx4 acc[NG][D / 16];   // O^T: dims 16 j + 4 g + e of query qis[u]
#pragma unroll
  for (int u = 0; u < NG; ++u)
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[u][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float m[NG], l[NG];
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    m[u] = -INFINITY;
    l[u] = 0.0f;
  }
  const float c2 = a.scale * kLog2e;

  // the key blocks run up to the one holding the workgroup's last query
  const int q_end = (qb + 1) * kFwdQ < S ? (qb + 1) * kFwdQ : S;   // one past the last query
  const int kb_last = (q_end - 1) / kB;
  const __amdgpu_buffer_rsrc_t rk = rsrc_of(a.k + seq0 * a.ldk + hk * D, a.S * a.ldk * 2);
  const __amdgpu_buffer_rsrc_t rv = rsrc_of(a.v + seq0 * a.ldv + hk * D, a.S * a.ldv * 2);
  constexpr int NW = kFwd2Threads / 64;
  constexpr int SEGW = DTile<D>::SEGS / NW;       // segments of each tile per wave
  // the wave's share of block kb: segments wave * SEGW .. of the K tile and of the V tile (the
  // lanes' offsets of a whole block computed once; the last, partial block clamps its rows)
  uint32_t vk_full[SEGW], vv_full[SEGW];
#pragma unroll
  for (int i = 0; i < SEGW; ++i) {
    vk_full[i] = seg_voff<D>(wave * SEGW + i, lane, a.ldk, kB);
    vv_full[i] = seg_voff<D>(wave * SEGW + i, lane, a.ldv, kB);
  }
  auto issue = [&](int kb) {
    const int nvalid = S - kb * kB < kB ? S - kb * kB : kB;
    char *st = smem + (kb & 1) * 2 * DTile<D>::BYTES;
    const uint32_t sk = (uint32_t)(kb * kB * a.ldk * 2), sv = (uint32_t)(kb * kB * a.ldv * 2);
#pragma unroll
    for (int i = 0; i < SEGW; ++i) {
      const int sg = wave * SEGW + i;
      const bool full = nvalid == kB;
      direct_load(rk, st + sg * 1024, full ? vk_full[i] : seg_voff<D>(sg, lane, a.ldk, nvalid), sk);
      direct_load(rv, st + DTile<D>::BYTES + sg * 1024, full ? vv_full[i] : seg_voff<D>(sg, lane, a.ldv, nvalid), sv);
    }
  };
  issue(0);
  for (int kb = 0; kb <= kb_last; ++kb) {
    tile_barrier();                                // block kb has landed; stage (kb+1)&1 is free
    if (kb < kb_last) issue(kb + 1);
    if (kb * kB > wq0 + 16 * NG - 1) continue;     // every key of the block is after this wave's queries
    const bool diag = kb * kB + kB - 1 > wq0;      // some key of the block is after some query here
    const char *k_t = smem + (kb & 1) * 2 * DTile<D>::BYTES;
    const char *v_t = k_t + DTile<D>::BYTES;

    // S^T tile tt of group u: keys 16 tt + 4 g + e (rows) x query qis[u]; two key tiles per half
    floatx4 s[NG][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      bf16x8 kf[2][D / 32];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kf[t][c] = sw_frag<D>(k_t, 16 * (2 * hf + t) + col, 4 * c + g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < NG; ++u) {
          s[u][2 * hf + t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int c = 0; c < D / 32; ++c) s[u][2 * hf + t] = mfma(kf[t][c], qf[u][c], s[u][2 * hf + t]);
        }
      AT_MFMA_FENCE();
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) asm volatile("" ::"v"(kf[t][c]));
    }
    // online softmax in the exp2 domain, per group; the causal mask only on blocks that reach past
    // a query (a uniform branch: the other blocks skip its compares and selects). The block's
    // maximum is taken over the raw scores (x -> fl32(x c2) is monotone for c2 > 0, so it scales
    // to the maximum of the scaled ones exactly), and p = 2^fma(s, c2, -m). m is the row's
    // reference maximum: it moves, and the output and sum are rescaled, only when some row's
    // maximum exceeds its reference by more than kLazy (so p <= 2^kLazy in between).
    const int key0 = kb * kB + 4 * g;
    float mxs[NG];
    auto block_max = [&](auto masked) {
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (decltype(masked)::value) {
              if (key0 + 16 * tt + e > qis[u]) s[u][tt][e] = -INFINITY;
            }
            mx = fmaxf(mx, s[u][tt][e]);
          }
        mxs[u] = mx;
      }
    };
    if (diag)
      block_max(std::true_type{});
    else
      block_max(std::false_type{});
    bool grow = false;
    float m_cand[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      float mx = mxs[u];
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_cand[u] = fmaxf(m[u], mx * c2);
      grow = grow || m_cand[u] > m[u] + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const float alpha = ex2(m[u] - m_cand[u]);
        l[u] *= alpha;
        m[u] = m_cand[u];
#pragma unroll
        for (int j = 0; j < D / 16; ++j) acc[u][j] *= alpha;
      }
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const float nm = -m[u];
      float rs = 0.0f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[u][tt][e] = ex2(__builtin_fmaf(s[u][tt][e], c2, nm));
          rs += s[u][tt][e];
        }
      rs += __shfl_xor(rs, 16);
      rs += __shfl_xor(rs, 32);
      l[u] += rs;
    }
    // O^T += V^T P^T over the block's 64 keys (two reduction steps of 32); V^T fragments come
    // from the row-major V tile by transpose reads and serve both groups
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 pf[NG];
#pragma unroll
      for (int u = 0; u < NG; ++u) pf[u] = acc_frag(s[u][2 * c], s[u][2 * c + 1]);
      bf16x8 vf[D / 16];
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) vf[jj] = tr_frag_rm<D>(v_t, jj, c, g, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj)
#pragma unroll
        for (int u = 0; u < NG; ++u) acc[u][jj] = mfma(vf[jj], pf[u], acc[u][jj]);
      AT_MFMA_FENCE();
#pragma unroll
      for (int u = 0; u < NG; ++u) asm volatile("" ::"v"(pf[u]));
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) asm volatile("" ::"v"(vf[jj]));
    }
  }
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    if (qis[u] < S) {
      const float inv = 1.0f / l[u];
      uint16_t *orow = a.out_o + (seq0 + qis[u]) * a.ld_out_o + h * D;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const u32x2 w = {pack_bf16x2(acc[u][j][0] * inv, acc[u][j][1] * inv),
                         pack_bf16x2(acc[u][j][2] * inv, acc[u][j][3] * inv)};
        *reinterpret_cast<u32x2 *>(orow + 16 * j + 4 * g) = w;
      }
      if (g == 0) a.lse[(seq0 + qis[u]) * a.n_q + h] = (m[u] + log2f(l[u])) * 0.69314718055994531f;
    }
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
// dK, dV: one workgroup per (key block, sequence, key/value head, part), heaviest (first) blocks
// first; a wave owns 16 keys (lane column = key) and loops over its part of the group's query
// heads (all of them, or one half with a.kv_split = 2) and the query blocks at or after its key
// block. Each (head, query block)'s Q and dO tiles and the rows' log-sum-exp and D stream through
// two LDS stages by direct-to-LDS loads (Q^T and dO^T fragments by transpose reads of the
// row-major tiles). A key block's work falls from 2 n_blocks (head, query block) pairs for the
// first block to 2 for the last: unsplit, the first blocks' workgroups set the pass's time while
// the last ones finish early (all of them fit on the device at once); split in two, twice as many
// workgroups of half the work queue up heaviest first and the light ones fill in behind. The
// split pass stores fp32 partial sums, which k_attn_kv_reduce adds in a fixed order.
template <int D>
__global__ __launch_bounds__(kThreads) void k_attn_bwd_kv(AttnArgs a) {
  constexpr int STAGE = 2 * DTile<D>::BYTES + 2 * kB * 4;                      // Q, dO, lse, D
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  const int nb = (int)((a.S + kB - 1) / kB);
  const int nsplit = a.kv_split;
  const int64_t per = a.n_seq * a.n_kv * nsplit;
  const int kb = (int)(blockIdx.x / per);
  const int64_t rest = blockIdx.x % per;
  const int part = (int)(rest % nsplit);
  const int64_t b = rest / nsplit / a.n_kv;
  const int hk = (int)(rest / nsplit % a.n_kv), grp = a.n_q / a.n_kv, hpw = grp / nsplit;
  // (the wave index in a scalar register, so that the direct loads' LDS destinations are scalar)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g = lane >> 4,
            col = lane & 15;
  const int S = (int)a.S;
  const int k_in_seq = kb * kB + 16 * wave + col;
  const int64_t seq0 = b * a.S;
  const bool kvalid = k_in_seq < S;
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

  const __amdgpu_buffer_rsrc_t rq = rsrc_of(a.q + seq0 * a.ldq, a.S * a.ldq * 2);
  const __amdgpu_buffer_rsrc_t rd = rsrc_of(a.dO + seq0 * a.lddo, a.S * a.lddo * 2);
  const __amdgpu_buffer_rsrc_t rl = rsrc_of(a.lse + seq0 * a.n_q, a.S * a.n_q * 4);
  const __amdgpu_buffer_rsrc_t rt = rsrc_of(a.dot + seq0 * a.n_q, a.S * a.n_q * 4);
  constexpr int SEGW = DTile<D>::SEGS / 4;        // segments of each tile per wave (4 waves)
  // iteration it = hh * (nb - kb) + (qb - kb) visits query head hk * grp + part * hpw + hh, query
  // block qb
  const int nqb = nb - kb, n_it = hpw * nqb;
  uint32_t vq_full[SEGW], vd_full[SEGW];     // the lanes' offsets within a whole block
#pragma unroll
  for (int i = 0; i < SEGW; ++i) {
    vq_full[i] = seg_voff<D>(wave * SEGW + i, lane, a.ldq, kB);
    vd_full[i] = seg_voff<D>(wave * SEGW + i, lane, a.lddo, kB);
  }
  auto issue = [&](int it) {
    const int hh = it / nqb, qb = kb + it % nqb, h = hk * grp + part * hpw + hh;
    const int nvalid = S - qb * kB < kB ? S - qb * kB : kB;
    const bool full = nvalid == kB;
    char *st = smem + (it & 1) * STAGE;
#pragma unroll
    for (int i = 0; i < SEGW; ++i) {
      const int sg = wave * SEGW + i;
      direct_load(rq, st + sg * 1024, (full ? vq_full[i] : seg_voff<D>(sg, lane, a.ldq, nvalid)) + h * D * 2,
                  (uint32_t)(qb * kB * a.ldq * 2));
      direct_load(rd, st + DTile<D>::BYTES + sg * 1024,
                  (full ? vd_full[i] : seg_voff<D>(sg, lane, a.lddo, nvalid)) + h * D * 2,
                  (uint32_t)(qb * kB * a.lddo * 2));
    }
    if (wave < 2) {   // the rows' lse (wave 0) and D (wave 1), 4 bytes per lane
      const int row = lane < nvalid ? lane : nvalid - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wave == 0 ? rl : rt,
                                               (lds_void *)(st + 2 * DTile<D>::BYTES + wave * kB * 4), 4,
                                               (uint32_t)((row * a.n_q + h) * 4), (uint32_t)(qb * kB * a.n_q * 4),
                                               0, 0);
    }
  };
  issue(0);
  for (int it = 0; it < n_it; ++it) {
    tile_barrier();
    if (it + 1 < n_it) issue(it + 1);
    const int qb = kb + it % nqb;
    const char *q_t = smem + (it & 1) * STAGE;
    const char *d_t = q_t + DTile<D>::BYTES;
    const float *lse_s = reinterpret_cast<const float *>(q_t + 2 * DTile<D>::BYTES);
    const float *dot_s = lse_s + kB;

    // S and dP tiles tt: queries 16 tt + 4 g + e (rows) x key `col`; two tiles per half
    floatx4 s[4], dp[4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      bf16x8 qa[2][D / 32], da[2][D / 32];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          qa[u][c] = sw_frag<D>(q_t, 16 * (2 * hf + u) + col, 4 * c + g);
          da[u][c] = sw_frag<D>(d_t, 16 * (2 * hf + u) + col, 4 * c + g);
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
    // P and dS = P (dP - D); queries before the key (first block) or past S (padding rows of the
    // last block, which hold copies of row S - 1) contribute nothing
    // (the masked form only on those blocks: a uniform branch)
    const int q0 = qb * kB + 4 * g;
    const bool edge = qb == kb || qb * kB + kB > S;
    auto probs = [&](auto masked) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qi = 16 * tt + 4 * g + e;
          float p = ex2(s[tt][e] * c2 - lse_s[qi] * kLog2e);
          if constexpr (decltype(masked)::value) {
            if (q0 + 16 * tt + e < k_in_seq || q0 + 16 * tt + e >= S) p = 0.0f;
          }
          s[tt][e] = p;
          dp[tt][e] = p * (dp[tt][e] - dot_s[qi]);
        }
    };
    if (edge)
      probs(std::true_type{});
    else
      probs(std::false_type{});
    // dV^T += dO^T P,  dK^T += Q^T dS  (reduction over the block's 64 queries, in two steps)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const bf16x8 bf = which == 0 ? acc_frag(s[2 * c], s[2 * c + 1]) : acc_frag(dp[2 * c], dp[2 * c + 1]);
        bf16x8 af[D / 16];
#pragma unroll
        for (int jj = 0; jj < D / 16; ++jj) af[jj] = tr_frag_rm<D>(which == 0 ? d_t : q_t, jj, c, g, lane);
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
  if (kvalid) {
    const int64_t row = seq0 + k_in_seq;
    if (nsplit == 1) {
      store_grad_row<D>(a.dk + row * a.lddk + hk * D, dk, a.scale, a.rope != 0, a, row, g);
      store_grad_row<D>(a.dv + row * a.lddv + hk * D, dv, 1.0f, false, a, row, g);
    } else {
      const int64_t T = a.n_seq * a.S;
      store_part_row<D>(a.kv_part + ((2 * part * T + row) * a.n_kv + hk) * D, dk, g);
      store_part_row<D>(a.kv_part + (((2 * part + 1) * T + row) * a.n_kv + hk) * D, dv, g);
    }
  }
}

// dK and dV from the split pass's partial sums, added in a fixed order (part 0, then part 1), and
// stored as the unsplit pass stores its sums: dk = bf16(scale (p0 + p1)), with rope each pair
// (i, i + D/2) of the rounded values then turned back by its angle (the same arithmetic as
// store_grad_row), dv = bf16(p0 + p1). A thread takes pairs f0 .. f0+3 of one row and head.
template <int D>
__global__ __launch_bounds__(kThreads) void k_attn_kv_reduce(AttnArgs a) {
  constexpr int TPR = D / 8;
  const int64_t T = a.n_seq * a.S;
  const int64_t item = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t rh = item / TPR;
  if (rh >= T * a.n_kv) return;
  const int f0 = (int)(item % TPR) * 4;
  const int64_t row = rh / a.n_kv;
  const int hk = (int)(rh % a.n_kv);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const float *p0 = a.kv_part + ((which * T + row) * a.n_kv + hk) * D;
    const float *p1 = a.kv_part + (((2 + which) * T + row) * a.n_kv + hk) * D;
    const floatx4 l0 = *reinterpret_cast<const floatx4 *>(p0 + f0);
    const floatx4 h0 = *reinterpret_cast<const floatx4 *>(p0 + f0 + D / 2);
    const floatx4 l1 = *reinterpret_cast<const floatx4 *>(p1 + f0);
    const floatx4 h1 = *reinterpret_cast<const floatx4 *>(p1 + f0 + D / 2);
    const float mul = which == 0 ? a.scale : 1.0f;
    float v1[4], v2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v1[e] = __fmul_rn(__fadd_rn(l0[e], l1[e]), mul);
      v2[e] = __fmul_rn(__fadd_rn(h0[e], h1[e]), mul);
    }
    if (which == 0 && a.rope) {
      const int pos = min(max(a.rope_pos[row], 0), a.rope_n_pos - 1);
      const float *cs = a.rope_cs + (int64_t)pos * D;
      const floatx4 c01 = *reinterpret_cast<const floatx4 *>(cs + 2 * f0);
      const floatx4 c23 = *reinterpret_cast<const floatx4 *>(cs + 2 * f0 + 4);
      const float cv[4] = {c01[0], c01[2], c23[0], c23[2]};
      const float sv[4] = {c01[1], c01[3], c23[1], c23[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = bf16f(f2bf(v1[e])), x2 = bf16f(f2bf(v2[e]));
        rope_pair(x1, x2, cv[e], __fmul_rn(-1.0f, sv[e]), v1[e], v2[e]);
      }
    }
    uint16_t *dst = (which == 0 ? a.dk + row * a.lddk : a.dv + row * a.lddv) + hk * D;
    *reinterpret_cast<u32x2 *>(dst + f0) = u32x2{pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
    *reinterpret_cast<u32x2 *>(dst + f0 + D / 2) = u32x2{pack_bf16x2(v2[0], v2[1]), pack_bf16x2(v2[2], v2[3])};
  }
}

// ------------------------------------------------------------------------------------------
// dQ: one workgroup per (query block, sequence, query head), heaviest blocks first; a wave owns
// 16 NG queries as NG groups of 16 (lane column = one query of each group) and loops over the key
// blocks up to its own; every K and V fragment it reads serves all its groups. K and V blocks
// stream through two LDS stages by direct-to-LDS loads (row-major; K^T fragments by transpose
// reads), as in the forward.
template <int D, int NG>
__global__ __launch_bounds__(kFwdQ / NG * 4) void k_attn_bwd_q(AttnArgs a) {
  constexpr int NT = kFwdQ / NG * 4;               // 8 waves of 16 queries, or 4 of 32
  __shared__ __attribute__((aligned(1024))) char smem[4 * DTile<D>::BYTES];   // [stage][K, V]
  const int nqb = (int)((a.S + kFwdQ - 1) / kFwdQ);
  const int64_t per = a.n_seq * a.n_q;
  const int qb = nqb - 1 - (int)(blockIdx.x / per);
  const int64_t rest = blockIdx.x % per;
  const int64_t b = rest / a.n_q;
  const int h = (int)(rest % a.n_q), hk = h / (a.n_q / a.n_kv);
  // (the wave index in a scalar register, so that the direct loads' LDS destinations are scalar)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g = lane >> 4,
            col = lane & 15;
  const int S = (int)a.S;
  const int wq0 = qb * kFwdQ + 16 * NG * wave;     // this wave's first query
  const int64_t seq0 = b * a.S;
  int qis[NG];
  bf16x8 qf[NG][D / 32], df[NG][D / 32];   // B operands: query qis[u], dims 32 c + 8 g ..
  float lse2[NG], dq_dot[NG];
  floatx4 acc[NG][D / 16];   // dQ^T: dims 16 j + 4 g + e of query qis[u]
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    qis[u] = wq0 + 16 * u + col;
    const bool qvalid = qis[u] < S;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      qf[u][c] = qvalid ? as_bf(*reinterpret_cast<const u32x4_t *>(a.q + (seq0 + qis[u]) * a.ldq + h * D + 32 * c + 8 * g))
                        : as_bf(u32x4_t{0u, 0u, 0u, 0u});
      df[u][c] = qvalid ? as_bf(*reinterpret_cast<const u32x4_t *>(a.dO + (seq0 + qis[u]) * a.lddo + h * D + 32 * c + 8 * g))
                        : as_bf(u32x4_t{0u, 0u, 0u, 0u});
    }
    lse2[u] = qvalid ? a.lse[(seq0 + qis[u]) * a.n_q + h] * kLog2e : INFINITY;
    dq_dot[u] = qvalid ? a.dot[(seq0 + qis[u]) * a.n_q + h] : 0.0f;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[u][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float c2 = a.scale * kLog2e;

  const int q_end = (qb + 1) * kFwdQ < S ? (qb + 1) * kFwdQ : S;   // one past the last query
  const int kb_last = (q_end - 1) / kB;
  const __amdgpu_buffer_rsrc_t rk = rsrc_of(a.k + seq0 * a.ldk + hk * D, a.S * a.ldk * 2);
  const __amdgpu_buffer_rsrc_t rv = rsrc_of(a.v + seq0 * a.ldv + hk * D, a.S * a.ldv * 2);
  constexpr int SEGW = DTile<D>::SEGS / (NT / 64);
  auto issue = [&](int kb) {
    const int nvalid = S - kb * kB < kB ? S - kb * kB : kB;
    char *st = smem + (kb & 1) * 2 * DTile<D>::BYTES;
#pragma unroll
    for (int i = 0; i < SEGW; ++i) {
      const int sg = wave * SEGW + i;
      direct_load(rk, st + sg * 1024, seg_voff<D>(sg, lane, a.ldk, nvalid), (uint32_t)(kb * kB * a.ldk * 2));
      direct_load(rv, st + DTile<D>::BYTES + sg * 1024, seg_voff<D>(sg, lane, a.ldv, nvalid),
                  (uint32_t)(kb * kB * a.ldv * 2));
    }
  };
  issue(0);
  for (int kb = 0; kb <= kb_last; ++kb) {
    tile_barrier();
    if (kb < kb_last) issue(kb + 1);
    if (kb * kB > wq0 + 16 * NG - 1) continue;  // every key of the block is after this wave's queries
    const bool diag = kb * kB + kB - 1 > wq0;
    const char *k_t = smem + (kb & 1) * 2 * DTile<D>::BYTES;
    const char *v_t = k_t + DTile<D>::BYTES;

    // S^T and dP^T tiles tt of group u: keys 16 tt + 4 g + e (rows) x query qis[u]; one key tile
    // at a time
    floatx4 s[NG][4], dp[NG][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      bf16x8 ka[D / 32], va[D / 32];
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        ka[c] = sw_frag<D>(k_t, 16 * tt + col, 4 * c + g);
        va[c] = sw_frag<D>(v_t, 16 * tt + col, 4 * c + g);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        s[u][tt] = dp[u][tt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          s[u][tt] = mfma(ka[c], qf[u][c], s[u][tt]);
          dp[u][tt] = mfma(va[c], df[u][c], dp[u][tt]);
        }
      }
      AT_MFMA_FENCE();
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        asm volatile("" ::"v"(ka[c]));
        asm volatile("" ::"v"(va[c]));
      }
    }
    // (the causal mask only on blocks that reach past a query: a uniform branch)
    const int key0 = kb * kB + 4 * g;
    auto dscores = [&](auto masked) {
#pragma unroll
      for (int u = 0; u < NG; ++u)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float p = ex2(s[u][tt][e] * c2 - lse2[u]);
            if constexpr (decltype(masked)::value) {
              if (key0 + 16 * tt + e > qis[u]) p = 0.0f;
            }
            dp[u][tt][e] = p * (dp[u][tt][e] - dq_dot[u]);
          }
    };
    if (diag)
      dscores(std::true_type{});
    else
      dscores(std::false_type{});
    // dQ^T += K^T dS^T over the block's 64 keys (two steps of 32); K^T fragments by transpose
    // reads of the row-major K tile, serving every group
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 sf[NG];
#pragma unroll
      for (int u = 0; u < NG; ++u) sf[u] = acc_frag(dp[u][2 * c], dp[u][2 * c + 1]);
      bf16x8 ka[D / 16];
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) ka[jj] = tr_frag_rm<D>(k_t, jj, c, g, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj)
#pragma unroll
        for (int u = 0; u < NG; ++u) acc[u][jj] = mfma(ka[jj], sf[u], acc[u][jj]);
      AT_MFMA_FENCE();
#pragma unroll
      for (int u = 0; u < NG; ++u) asm volatile("" ::"v"(sf[u]));
#pragma unroll
      for (int jj = 0; jj < D / 16; ++jj) asm volatile("" ::"v"(ka[jj]));
    }
  }
#pragma unroll
  for (int u = 0; u < NG; ++u)
    if (qis[u] < S)
      store_grad_row<D>(a.dq + (seq0 + qis[u]) * a.lddq + h * D, acc[u], a.scale, a.rope != 0, a, seq0 + qis[u], g);
}

// workgroups per key block of the dK/dV pass: the group's query heads in two halves when their
// number is even (the partial sums then go through the workspace), else all in one
int kv_split(int32_t n_q, int32_t n_kv) { return (n_q / n_kv) % 2 == 0 ? 2 : 1; }

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
  if (S * ldk * 2 >= ((int64_t)1 << 31) || S * ldv * 2 >= ((int64_t)1 << 31))
    return fail(LSN_E_ARG, "attention_fwd: one sequence of k or v spans 2 GiB or more");
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
    hipLaunchKernelGGL(k_attn_fwd<128>, dim3(grid), dim3(kFwd2Threads), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(k_attn_fwd<64>, dim3(grid), dim3(kFwd2Threads), 0, (hipStream_t)stream, a);
  return check_hip(hipGetLastError(), "k_attn_fwd launch");
}

size_t attention_bwd_ws_bytes(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim) {
  if (n_seq < 1 || S < 1 || n_q < 1 || n_kv < 1 || n_q % n_kv || head_dim < 1) return 0;
  const size_t dots = ((size_t)(n_seq * S * n_q) * 4 + 255) / 256 * 256;
  return dots + (kv_split(n_q, n_kv) == 2 ? (size_t)4 * n_seq * S * n_kv * head_dim * 4 : 0);
}

}  // extern "C"

namespace {

// attention_bwd, and with rope (may be null) attention_bwd_rope; `who` names the entry point
lsn_status attn_bwd_impl(const char *who, int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim,
                         const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v,
                         int64_t ldv, const uint16_t *o, int64_t ldo, const float *lse, const uint16_t *dO,
                         int64_t lddo, float scale, uint16_t *dq, int64_t lddq, uint16_t *dk, int64_t lddk,
                         uint16_t *dv, int64_t lddv, void *ws, size_t ws_bytes, const lsn_rope *rope, void *stream) {
  lsn_status st = check_common(n_seq, S, n_q, n_kv, head_dim, scale, who);
  if (st != LSN_OK) return st;
  const int64_t D = head_dim, T = n_seq * S;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !ws)
    return fail(LSN_E_ARG, "%s: null pointer", who);
  if (rope && (!rope->cs || ((uintptr_t)rope->cs & 15) || !rope->positions || rope->n_pos < 1 ||
               rope->head_dim != head_dim))
    return fail(LSN_E_ARG, "%s: the rotation needs a 16-byte aligned table of this head width, positions and "
                           "n_pos >= 1", who);
  if (!al16(q, ldq) || !al16(k, ldk) || !al16(v, ldv) || !al16(o, ldo) || !al16(dO, lddo) || !al16(dq, lddq) ||
      !al16(dk, lddk) || !al16(dv, lddv) || ((uintptr_t)ws & 15))
    return fail(LSN_E_ARG, "%s: tensors need 16-byte aligned rows (ld a multiple of 8)", who);
  if (ldq < n_q * D || ldk < n_kv * D || ldv < n_kv * D || ldo < n_q * D || lddo < n_q * D || lddq < n_q * D ||
      lddk < n_kv * D || lddv < n_kv * D)
    return fail(LSN_E_ARG, "%s: a row stride is smaller than its heads", who);
  const size_t ws_need = attention_bwd_ws_bytes(n_seq, S, n_q, n_kv, head_dim);
  if (ws_bytes < ws_need) return fail(LSN_E_ARG, "%s: workspace smaller than attention_bwd_ws_bytes", who);
  if (S * ldq * 2 >= ((int64_t)1 << 31) || S * ldk * 2 >= ((int64_t)1 << 31) || S * ldv * 2 >= ((int64_t)1 << 31) ||
      S * lddo * 2 >= ((int64_t)1 << 31))
    return fail(LSN_E_ARG, "%s: one sequence of q, k, v or dO spans 2 GiB or more", who);
  const Strided ins[] = {{q, ldq, n_q * D, 2}, {k, ldk, n_kv * D, 2}, {v, ldv, n_kv * D, 2},
                         {o, ldo, n_q * D, 2}, {lse, n_q, n_q, 4},       {dO, lddo, n_q * D, 2}};
  const Strided outs[] = {{dq, lddq, n_q * D, 2}, {dk, lddk, n_kv * D, 2}, {dv, lddv, n_kv * D, 2}};
  if (rope) {
    for (int i = 0; i < 3; ++i) {
      const size_t ob = span(T, outs[i].ld, outs[i].width, outs[i].elt);
      if (ranges_overlap(outs[i].p, ob, rope->cs, (size_t)rope->n_pos * D * 4) ||
          ranges_overlap(outs[i].p, ob, rope->positions, (size_t)T * 4))
        return fail(LSN_E_ARG, "%s: an output overlaps the rotation inputs", who);
    }
    if (ranges_overlap(ws, ws_need, rope->cs, (size_t)rope->n_pos * D * 4) ||
        ranges_overlap(ws, ws_need, rope->positions, (size_t)T * 4))
      return fail(LSN_E_ARG, "%s: the workspace overlaps the rotation inputs", who);
  }
  for (int i = 0; i < 3; ++i) {
    for (const Strided &in : ins)
      if (overlap(outs[i], in, T)) return fail(LSN_E_ARG, "%s: an output overlaps an input", who);
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j], T)) return fail(LSN_E_ARG, "%s: outputs overlap", who);
    if (ranges_overlap(ws, ws_need, outs[i].p, span(T, outs[i].ld, outs[i].width, outs[i].elt)))
      return fail(LSN_E_ARG, "%s: the workspace overlaps an output", who);
  }
  for (const Strided &in : ins)
    if (ranges_overlap(ws, ws_need, in.p, span(T, in.ld, in.width, in.elt)))
      return fail(LSN_E_ARG, "%s: the workspace overlaps an input", who);
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
  a.kv_split = kv_split(n_q, n_kv);
  a.kv_part = a.kv_split == 2
                  ? reinterpret_cast<float *>(static_cast<char *>(ws) + ((size_t)(T * n_q) * 4 + 255) / 256 * 256)
                  : nullptr;
  if (rope) {
    a.rope = 1;
    a.rope_n_pos = rope->n_pos;
    a.rope_cs = rope->cs;
    a.rope_pos = rope->positions;
  }
  const hipStream_t hs = (hipStream_t)stream;
  const int64_t nb = (S + kB - 1) / kB;
  const unsigned dot_grid = (unsigned)((T * n_q * (D / 8) + kThreads - 1) / kThreads);
  const unsigned kv_grid = (unsigned)(nb * n_seq * n_kv * a.kv_split);
  const unsigned q_grid = (unsigned)(((S + kFwdQ - 1) / kFwdQ) * n_seq * n_q);
  const unsigned red_grid = (unsigned)((T * n_kv * (D / 8) + kThreads - 1) / kThreads);
  if (head_dim == 128) {
    hipLaunchKernelGGL(k_attn_dot<128>, dim3(dot_grid), dim3(kThreads), 0, hs, a, static_cast<float *>(ws));
    hipLaunchKernelGGL(k_attn_bwd_kv<128>, dim3(kv_grid), dim3(kThreads), 0, hs, a);
    if (a.kv_split == 2) hipLaunchKernelGGL(k_attn_kv_reduce<128>, dim3(red_grid), dim3(kThreads), 0, hs, a);
    hipLaunchKernelGGL((k_attn_bwd_q<128, kDqGroups>), dim3(q_grid), dim3(kFwdQ / kDqGroups * 4), 0, hs, a);
  } else {
    hipLaunchKernelGGL(k_attn_dot<64>, dim3(dot_grid), dim3(kThreads), 0, hs, a, static_cast<float *>(ws));
    hipLaunchKernelGGL(k_attn_bwd_kv<64>, dim3(kv_grid), dim3(kThreads), 0, hs, a);
    if (a.kv_split == 2) hipLaunchKernelGGL(k_attn_kv_reduce<64>, dim3(red_grid), dim3(kThreads), 0, hs, a);
    hipLaunchKernelGGL((k_attn_bwd_q<64, kDqGroups>), dim3(q_grid), dim3(kFwdQ / kDqGroups * 4), 0, hs, a);
  }
  return check_hip(hipGetLastError(), "attention backward launch");
}

}  // namespace

extern "C" {

lsn_status attention_bwd(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim, const uint16_t *q,
                         int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v, int64_t ldv,
                         const uint16_t *o, int64_t ldo, const float *lse, const uint16_t *dO, int64_t lddo,
                         float scale, uint16_t *dq, int64_t lddq, uint16_t *dk, int64_t lddk, uint16_t *dv,
                         int64_t lddv, void *ws, size_t ws_bytes, void *stream) {
  return attn_bwd_impl("attention_bwd", n_seq, S, n_q, n_kv, head_dim, q, ldq, k, ldk, v, ldv, o, ldo, lse, dO, lddo,
                       scale, dq, lddq, dk, lddk, dv, lddv, ws, ws_bytes, nullptr, stream);
}

lsn_status attention_bwd_rope(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim,
                              const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v,
                              int64_t ldv, const uint16_t *o, int64_t ldo, const float *lse, const uint16_t *dO,
                              int64_t lddo, float scale, uint16_t *dq, int64_t lddq, uint16_t *dk, int64_t lddk,
                              uint16_t *dv, int64_t lddv, void *ws, size_t ws_bytes, const lsn_rope *rope,
                              void *stream) {
  if (!rope) return fail(LSN_E_ARG, "attention_bwd_rope: null rotation");
  return attn_bwd_impl("attention_bwd_rope", n_seq, S, n_q, n_kv, head_dim, q, ldq, k, ldk, v, ldv, o, ldo, lse, dO,
                       lddo, scale, dq, lddq, dk, lddk, dv, lddv, ws, ws_bytes, rope, stream);
}

}  // extern "C"
