// Fused frozen-base GEMMs with the LoRA term, on gfx950 MFMA (bf16 operands, fp32 accumulate).
//
//   forward  (NT):  Y  = bf16( X  W^T + s U B^T )      X [M][K], W [N][K], U [M][r], B [N][r]
//   backward (NN):  dX = dY W + s G A   (bf16 store or fp32 accumulate)
//                                       dY [M][N], W [N][K], G [M][r], A [r][K]
// ("Can You Fine-Tune a 27B Model on a Laptop?", transcript @1:25-1:58: frozen base plus a
// thin pair of trainable matrices; "Exact Layer Streaming", Abstract: the step is dominated by
// these GEMMs, and per-layer NF4 dequantisation is the largest streaming-specific cost.)
//
// W is either bf16 or NF4. For NF4 the tile of W a K-step needs is dequantised straight into
// LDS (never to HBM), bit-identical to the standalone dequantisation:
//   w = bf16_RNE( fl32( q[code] * fl32( fl32(v/127 * s2) + mu ) ) ).
// Every visit re-dequantises from the bytes the descriptor points at; nothing is cached.
//
// Two kernels: k_gemm_direct (further down: every bf16-weight product, and the forward of NF4
// weights whose arrays are aligned for direct loads, decoded in the kernel) and k_gemm, the
// register-staged kernel described here, which serves NF4 weights in the input-gradient product
// (the NN layout) and in the forward when their arrays are not aligned for direct loads.
// Tiling: one 256-thread workgroup (4 waves, 2 x 2) computes a 256 x 256 output tile; each
// wave owns 128 x 128 (4 x 4 MFMA 32x32x16 tiles, 256 fp32 accumulators per lane). K-steps of
// 64 (one NF4 block per W row) are double-buffered in LDS: the global loads of step k+1 are in
// flight while step k runs on the matrix cores, then they are dequantised / written to the
// other buffer. LDS rows are 128 B (64 bf16) split into eight 16-byte chunks placed at
// chunk ^ ((row ^ row >> 3) & 7), so both the row-wise writes and the 32-row fragment reads
// hit distinct banks.
//
// The LoRA term runs first: the accumulators start as (s U) B^T (forward) or (s G) A
// (backward), from r-wide MFMA steps whose operands come straight from global memory, with the
// scale applied to the bf16 U (or G) fragments, bf16(s u): exact for a power-of-two s, so the
// result is then s (U B^T) in the fp32 sum's own rounding; any other s rounds s u to bf16 once.
// The base product accumulates on top. With adapters off the accumulators start at +0, which is
// also what B = 0 gives, so adapters-off and B = 0 produce identical bits.
//
// Determinism: the reduction order is fixed by the tiling (which depends only on shapes);
// there are no atomics.

#include <cmath>
#include <type_traits>

#include "common.h"
#include "gemm.h"
#include "glue_math.h"

namespace lsn {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NT = 256;                       // threads per workgroup
constexpr int TILE_BYTES = 256 * BK * 2;      // one 256 x 64 bf16 LDS tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

__device__ __forceinline__ int lds_off(int row, int chunk) { return (row * 8 + swz(row, chunk)) * 16; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------------------------
// operand tile loaders
// ---------------------------------------------------------------------------------------------

// Forward, NF4 W[N][K]: rows n0 .. n0+255, columns k0 .. k0+63 (exactly one NF4 block per
// row). Thread t handles half (t%2) of row (t/2) and of row 128 + t/2: 32 codes each.
struct Nf4RowTile {
  u32x4_t codes[2];
  int v[2];
  float s2[2];
};

__device__ __forceinline__ void load_nf4_rows(Nf4RowTile &st, const GemmArgs &a, int64_t n0, int64_t k0,
                                              int t) {
  const int half = t & 1;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int64_t n = min(n0 + p * 128 + (t >> 1), a.Nout - 1);   // clamped: unstored columns
    const int64_t e = n * a.Kred + k0;                               // element index of the block
    st.codes[p] = *reinterpret_cast<const u32x4_t *>(a.codes + e / 2 + 16 * half);
    const int64_t b = e >> 6;
    st.v[p] = a.qabsmax[b];
    st.s2[p] = a.absmax2[b >> 8];
  }
}

// 8 codes of one 32-bit word (element 2j in the high nibble of byte j) -> 4 words of bf16 pairs
__device__ __forceinline__ u32x4_t dequant8(uint32_t w, float c, const float *__restrict__ sq) {
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int shift = 8 * (e >> 1) + ((e & 1) ? 0 : 4);
    f[e] = __fmul_rn(sq[(w >> shift) & 15u], c);
  }
  return u32x4_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
}

// Backward (dX), W[N][K] read transposed: the tile covers W rows (reduction) n0 .. n0+63 and
// columns (output) k0 .. k0+255, and is stored in LDS as [256 output columns][64 reductions].
// Thread t handles the 8 x 8 block rows n0 + 8 (t/32) + i, columns k0 + 8 (t%32) + e.
struct Bf16ColTile {
  u32x4_t v[8];
};

__device__ __forceinline__ void load_bf16_cols(Bf16ColTile &st, const GemmArgs &a, int64_t n0, int64_t k0,
                                               int t) {
  const int rg = t >> 5, cg = t & 31;
  const int64_t col = min(k0 + 8 * cg, a.Nout - 8);     // clamped: unstored output columns
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = n0 + 8 * rg + i;
    st.v[i] = *reinterpret_cast<const u32x4_t *>(a.w16 + n * a.ldw + col);
  }
}

struct Nf4ColTile {
  uint32_t codes[8];
  int v[8];
  float s2[8];
};

__device__ __forceinline__ void load_nf4_cols(Nf4ColTile &st, const GemmArgs &a, int64_t n0, int64_t k0,
                                              int t) {
  const int rg = t >> 5, cg = t & 31;
  const int64_t col = min(k0 + 8 * cg, a.Nout - 8);     // clamped: unstored output columns
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = n0 + 8 * rg + i;
    const int64_t e = n * a.ldw + col;
    st.codes[i] = *reinterpret_cast<const uint32_t *>(a.codes + e / 2);
    const int64_t b = e >> 6;
    st.v[i] = a.qabsmax[b];
    st.s2[i] = a.absmax2[b >> 8];
  }
}

// ---------------------------------------------------------------------------------------------
// direct-to-LDS loads (gfx950 global_load_lds_dwordx4): lane l of one wave instruction writes the
// 16 bytes at (wave-uniform LDS base) + 16 l, so each instruction fills one 1 KB LDS segment =
// 8 rows of 128 B. Lane l loads the global chunk that belongs at its slot: row 8 sg + l/8,
// physical chunk l%8, i.e. logical chunk (l%8) ^ f(row).
// ---------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// Per-lane byte offsets of the 8 chunks a lane loads for one 256 x 64 tile; they do not depend on
// the K-step (the step's byte offset goes in the scalar offset), so they stay in 8 VGPRs.
struct DirectRows {
  uint32_t voff[8];
};

__device__ __forceinline__ void make_direct_rows(DirectRows &d, int64_t rows, int64_t ld, int64_t r0, int wave,
                                                 int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sg = wave * 8 + i;
    const int row = sg * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    const int64_t grow = min(r0 + row, rows - 1);     // clamped rows feed only unstored outputs
    d.voff[i] = (uint32_t)((grow * ld + 8 * c) * 2);
  }
}

__device__ __forceinline__ void issue_rows_direct(char *lds_tile, __amdgpu_buffer_rsrc_t rsrc, const DirectRows &d,
                                                  uint32_t k_bytes, int wave) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(lds_tile + (wave * 8 + i) * 1024), 16, d.voff[i],
                                             k_bytes, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  // raw buffer, no stride; loads past num_records return 0 (never fault)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// wait until every vector-memory operation of this wave has completed (incl. direct-to-LDS)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------------------------
// register path for W (NF4, or transposed bf16 in the backward): the staged codes or values are
// turned into eight 16-byte chunks of bf16, produced two at a time during the MFMA sub-steps.
// ---------------------------------------------------------------------------------------------
struct NoStage {};

template <int LAYOUT, int WKIND>
struct BStage;
template <> struct BStage<GEMM_NT, W_IS_BF16> { typedef NoStage type; };
template <> struct BStage<GEMM_NT, W_IS_NF4> { typedef Nf4RowTile type; };
template <> struct BStage<GEMM_NN, W_IS_BF16> { typedef Bf16ColTile type; };
template <> struct BStage<GEMM_NN, W_IS_NF4> { typedef Nf4ColTile type; };

// decoded block constants of a staged NF4 tile (2 rows forward, 8 rows backward)
template <int LAYOUT> struct Decoded;
template <> struct Decoded<GEMM_NT> { float c[2]; };
template <> struct Decoded<GEMM_NN> { float c[8]; };

template <int LAYOUT, int WKIND>
__device__ __forceinline__ void load_b(typename BStage<LAYOUT, WKIND>::type &st, const GemmArgs &a, int64_t n0,
                                       int64_t kstep0, int t) {
  if constexpr (LAYOUT == GEMM_NT && WKIND == W_IS_NF4) load_nf4_rows(st, a, n0, kstep0, t);
  else if constexpr (LAYOUT == GEMM_NN && WKIND == W_IS_BF16) load_bf16_cols(st, a, kstep0, n0, t);
  else if constexpr (LAYOUT == GEMM_NN && WKIND == W_IS_NF4) load_nf4_cols(st, a, kstep0, n0, t);
}

template <int LAYOUT, int WKIND>
__device__ __forceinline__ Decoded<LAYOUT> decode_b(const typename BStage<LAYOUT, WKIND>::type &st, float mu,
                                                    const float *__restrict__ scode8) {
  Decoded<LAYOUT> d;
  if constexpr (WKIND == W_IS_NF4) {
    constexpr int R = (LAYOUT == GEMM_NT) ? 2 : 8;
#pragma unroll
    for (int i = 0; i < R; ++i) d.c[i] = decode_absmax(scode8[st.v[i] + 127], st.s2[i], mu);
  }
  return d;
}

__device__ __forceinline__ float deq1(uint32_t w, int e, float c, const float *__restrict__ sq) {
  const int shift = 8 * (e >> 1) + ((e & 1) ? 0 : 4);
  return __fmul_rn(sq[(w >> shift) & 15u], c);
}

// chunk idx of the staged tile, and its LDS offset
template <int LAYOUT, int WKIND>
__device__ __forceinline__ u32x4_t make_chunk(const typename BStage<LAYOUT, WKIND>::type &st,
                                              const Decoded<LAYOUT> &d, int idx, const float *__restrict__ sq) {
  if constexpr (LAYOUT == GEMM_NT && WKIND == W_IS_NF4) {
    return dequant8(st.codes[idx >> 2][idx & 3], d.c[idx >> 2], sq);
  } else if constexpr (LAYOUT == GEMM_NN && WKIND == W_IS_NF4) {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16x2(deq1(st.codes[2 * q], idx, d.c[2 * q], sq), deq1(st.codes[2 * q + 1], idx, d.c[2 * q + 1], sq));
    return o;
  } else if constexpr (LAYOUT == GEMM_NN && WKIND == W_IS_BF16) {
    const uint32_t sel = (idx & 1) ? 0x07060302u : 0x05040100u;
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(st.v[2 * q + 1][idx >> 1], st.v[2 * q][idx >> 1], sel);
    return o;
  } else {
    return u32x4_t{0, 0, 0, 0};
  }
}

template <int LAYOUT>
__device__ __forceinline__ int chunk_off(int idx, int t) {
  if constexpr (LAYOUT == GEMM_NT) {
    const int row = (idx >> 2) * 128 + (t >> 1);
    return lds_off(row, 4 * (t & 1) + (idx & 3));
  } else {
    return lds_off(8 * (t & 31) + idx, t >> 5);
  }
}

// LoRA operand fragments for one 32x32x16 step over r-columns j0 .. j0+15.
// Activation side (U or G, [M][r]): lane reads row m, columns j0 + 8 (lane/32) .. +7.
__device__ __forceinline__ bf16x8 lora_act_frag(const GemmArgs &a, int64_t m, int j0, int lane) {
  const int j = j0 + 8 * (lane >> 5);
  u32x4_t v = {0, 0, 0, 0};
  if (m < a.M && j < a.r) v = *reinterpret_cast<const u32x4_t *>(a.lr_act + m * a.r + j);
  return as_bf16x8(v);
}

// Weight side. Forward: B [N][r], row n. Backward: A [r][K], column n (8 strided loads).
template <int LAYOUT>
__device__ __forceinline__ bf16x8 lora_w_frag(const GemmArgs &a, int64_t n, int j0, int lane) {
  const int j = j0 + 8 * (lane >> 5);
  if constexpr (LAYOUT == GEMM_NT) {
    u32x4_t v = {0, 0, 0, 0};
    if (n < a.Nout && j < a.r) v = *reinterpret_cast<const u32x4_t *>(a.lr_w + n * a.r + j);
    return as_bf16x8(v);
  } else {
    uint16_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (n < a.Nout && j + i < a.r) ? a.lr_w[(int64_t)(j + i) * a.Nout + n] : 0;
    u32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (uint32_t)h[2 * q] | ((uint32_t)h[2 * q + 1] << 16);
    return as_bf16x8(v);
  }
}

// ---------------------------------------------------------------------------------------------
// the kernel. MFMA operands are (W fragment, activation fragment), so the accumulator holds
// out^T: lane l has output row m = 32 i + l%32 and columns n = 32 j + 8 (e/4) + 4 (l/32) + e%4,
// four consecutive columns per group e/4, stored 8 (bf16) or 16 (fp32) bytes at a time.
// ---------------------------------------------------------------------------------------------
template <int LAYOUT, int WKIND, int EPI>
__global__ __launch_bounds__(NT, 1) void k_gemm(GemmArgs a) {
  constexpr bool B_DIRECT = (LAYOUT == GEMM_NT && WKIND == W_IS_BF16);
  typedef typename BStage<LAYOUT, WKIND>::type Stage;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *lds_a = smem;                              // 2 buffers
  char *lds_b = smem + 2 * TILE_BYTES;             // 2 buffers
  float *sq = reinterpret_cast<float *>(smem + 4 * TILE_BYTES);
  float *scode8 = sq + 16;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // tile coordinates: consecutive workgroups walk down M for one N tile, so the workgroups
  // resident at a time share W tiles
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t m0 = (int64_t)(blockIdx.x % tiles_m) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x / tiles_m) * BN;

  if constexpr (WKIND == W_IS_NF4) {
    if (t < 16) sq[t] = a.q[t];
    if (t < 255) scode8[t] = int8_level(t - 127);
  }

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  // ---- LoRA prologue: acc = s * (lr_w . lr_act^T) over r, or +0 with adapters off ----
  if (a.adapters) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j0 = 16 * h;
      if (j0 >= a.r) break;
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lora_act_frag(a, m0 + wm * 128 + 32 * i + (lane & 31), j0, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = lora_w_frag<LAYOUT>(a, n0 + wn * 128 + 32 * j + (lane & 31), j0, lane);
      // the scale on the activation-side fragments: bf16(s u), as the direct-load GEMM does
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) fa[i][e] = (__bf16)((float)fa[i][e] * a.scale);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
  }

  const int nk = (int)(a.Kred / BK);
  Stage S0, S1;
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(a.act, a.M * a.Kred * 2);
  DirectRows da;
  make_direct_rows(da, a.M, a.Kred, m0, wave, lane);
  __amdgpu_buffer_rsrc_t rs_b;
  DirectRows db;
  if constexpr (B_DIRECT) {
    rs_b = make_rsrc(a.w16, a.Nout * a.ldw * 2);
    make_direct_rows(db, a.Nout, a.ldw, n0, wave, lane);
  }

  // ---- prologue: step 0 into buffer 0; W of step 1 into registers ----
  // Prefetches past the last K-step are clamped to it: they re-load valid memory into the buffer
  // or staging set that is never read again, which keeps the loop free of tail code.
  const int k_last = nk - 1;
  issue_rows_direct(lds_a, rs_a, da, 0, wave);
  if constexpr (B_DIRECT) {
    issue_rows_direct(lds_b, rs_b, db, 0, wave);
  } else {
    load_b<LAYOUT, WKIND>(S0, a, n0, 0, t);
    load_b<LAYOUT, WKIND>(S1, a, n0, (int64_t)min(1, k_last) * BK, t);
  }
  __syncthreads();   // codebook tables visible
  if constexpr (!B_DIRECT) {
    const Decoded<LAYOUT> d = decode_b<LAYOUT, WKIND>(S0, a.mean, scode8);
#pragma unroll
    for (int idx = 0; idx < 8; ++idx)
      *reinterpret_cast<u32x4_t *>(lds_b + chunk_off<LAYOUT>(idx, t)) = make_chunk<LAYOUT, WKIND>(S0, d, idx, sq);
  }
  wait_vm_all();
  __syncthreads();

  // one K-step on buffer kt%2 while step kt+1 lands in the other buffer and (register path)
  // the W of step kt+2 is loaded into the free staging set
  auto step = [&](int kt, Stage &s_next, Stage &s_free) {
    const int cur = kt & 1;
    const char *la = lds_a + cur * TILE_BYTES;
    const char *lb = lds_b + cur * TILE_BYTES;
    char *lb_next = lds_b + (cur ^ 1) * TILE_BYTES;
    if constexpr (!B_DIRECT) load_b<LAYOUT, WKIND>(s_free, a, n0, (int64_t)min(kt + 2, k_last) * BK, t);
    const uint32_t kb = (uint32_t)min(kt + 1, k_last) * BK * 2;
    issue_rows_direct(lds_a + (cur ^ 1) * TILE_BYTES, rs_a, da, kb, wave);
    if constexpr (B_DIRECT) issue_rows_direct(lb_next, rs_b, db, kb, wave);
    Decoded<LAYOUT> d;
    if constexpr (!B_DIRECT) d = decode_b<LAYOUT, WKIND>(s_next, a.mean, scode8);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int chunk = 2 * s + (lane >> 5);
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8 *>(la + lds_off(wm * 128 + 32 * i + (lane & 31), chunk));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const bf16x8 *>(lb + lds_off(wn * 128 + 32 * j + (lane & 31), chunk));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
      if constexpr (!B_DIRECT) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<u32x4_t *>(lb_next + chunk_off<LAYOUT>(2 * s + h, t)) =
              make_chunk<LAYOUT, WKIND>(s_next, d, 2 * s + h, sq);
      }
    }
    wait_vm_all();
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, S1, S0);
    if (kt + 1 < nk) step(kt + 1, S0, S1);
  }

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * 128 + 32 * j + 8 * g + 4 * (lane >> 5);
        if (m < a.M && n < a.Nout) {
          const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1], v2 = acc[i][j][4 * g + 2],
                      v3 = acc[i][j][4 * g + 3];
          if constexpr (EPI == EPI_BF16 || EPI == EPI_BF16_RES) {
            uint2 o;
            o.x = pack_bf16x2(v0, v1);
            o.y = pack_bf16x2(v2, v3);
            if constexpr (EPI == EPI_BF16_RES) {
              const uint2 r = *reinterpret_cast<const uint2 *>(a.res + m * a.Nout + n);
              o.x = add_bf16_word(r.x, o.x);
              o.y = add_bf16_word(r.y, o.y);
            }
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + m * a.Nout + n) = o;
          } else if constexpr (EPI == EPI_SWIGLU_BWD) {
            const uint2 dm = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
            const uint2 gv = *reinterpret_cast<const uint2 *>(a.x.gate + m * a.Nout + n);
            const uint2 uv = *reinterpret_cast<const uint2 *>(a.x.up + m * a.Nout + n);
            uint2 dg, du;
            swiglu_bwd_word(gv.x, uv.x, dm.x, dg.x, du.x);
            swiglu_bwd_word(gv.y, uv.y, dm.y, dg.y, du.y);
            *reinterpret_cast<uint2 *>(a.x.dgate + m * a.Nout + n) = dg;
            *reinterpret_cast<uint2 *>(a.x.dup + m * a.Nout + n) = du;
          } else {
            floatx4_t *o = reinterpret_cast<floatx4_t *>(reinterpret_cast<float *>(a.out) + m * a.Nout + n);
            floatx4_t cur = *o;
            cur[0] = __fadd_rn(cur[0], v0);
            cur[1] = __fadd_rn(cur[1], v1);
            cur[2] = __fadd_rn(cur[2], v2);
            cur[3] = __fadd_rn(cur[3], v3);
            *o = cur;
          }
        }
      }
    }
  }
}

// =============================================================================================
// Direct-load NT GEMM (both operands K-contiguous; W bf16, or NF4 decoded into the stage as
// described further down): out_seg = act W_seg^T (+ LoRA term)
// for up to kMaxSegs output segments that share the activation (e.g. q, k, v, gate and up of a
// layer read the same input). K-steps of 64 stream through two LDS stages (64 KB each:
// 256 rows x 128 B per operand); buffer_load...lds fills the next stage while the matrix cores
// work on the current one.
// Each direct load moves 8 whole rows of 128 B, i.e. whole 128-byte lines: the CU's address
// unit processes a load per cache line, so half-line segments (a 32-wide K-step) would double
// its work per byte and its queue would stall the waves.
// LDS rows are 128 B (64 bf16, eight 16-byte chunks); chunk p of row r sits at slot
// 8 r + (p ^ ((r ^ (r >> 3)) & 7)): a 16-lane group of a fragment read (16 consecutive rows,
// one logical chunk) then covers all 64 four-byte banks once, and the direct writes are
// contiguous 1 KB segments.
// Reduction-major B (template flag BT): W is given as [K][N] (N contiguous), as a weight W[N'][K']
// is for the input-gradient product dY W, whose reduction runs over W's rows. A stage then holds
// 64 K-rows of 512 B (the tile's 256 N); each direct load moves two of them, and the fragment
// reads use the gfx950 LDS transpose read (ds_read_b64_tr_b16), which hands each lane four
// K-consecutive values of one column, so the matrix cores see the same fragments as from a
// [N][K] operand and the result is bit-identical. 16-byte chunk c of K-row k sits at slot
// c ^ 4 (k % 4): the four K-rows one transpose read spans then fall on different banks.
// =============================================================================================
constexpr int DBK = 64;
constexpr int DTILE = 256 * DBK * 2;           // 32 KB: one operand, one stage
constexpr int kEpiPitch = 256 * 2 + 16;        // bytes per LDS row of the bf16 output tile
constexpr int kPosOffset = 256 * kEpiPitch;     // the rotary epilogue: the tile rows' positions (1 KB)

__device__ __forceinline__ int dlds_off(int row, int chunk) {
  return (row * 8 + (chunk ^ ((row ^ (row >> 3)) & 7))) * 16;
}

struct DirectRows8 {
  uint32_t voff[8];
};

// wave w fills the LDS segments 8w .. 8w+7 (1 KB = 8 rows each) of a 256 x 64 tile
__device__ __forceinline__ void make_direct_rows8(DirectRows8 &d, int64_t rows, int64_t ld, int64_t r0, int wave,
                                                  int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    const int64_t grow = min(r0 + row, rows - 1);     // clamped rows feed only unstored outputs
    d.voff[i] = (uint32_t)((grow * ld + 8 * c) * 2);
  }
}

// reduction-major B: wave w fills K-rows 16w .. 16w+15 of a 64 x 256 tile, two per load
// (lanes 0-31 the first row, 32-63 the second; chunk slot = lane % 32). Columns past N (a ragged
// last tile) read the next row's start, or zeros past the end of the buffer: they feed only
// unstored outputs.
__device__ __forceinline__ void make_direct_rows8_t(DirectRows8 &d, int64_t ld, int64_t c0, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (wave * 8 + i) * 2 + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (row & 3));
    d.voff[i] = (uint32_t)((row * ld + c0 + 8 * c) * 2);
  }
}

__device__ __forceinline__ int dlds_off_t(int row, int chunk) { return row * 512 + ((chunk ^ (4 * (row & 3))) << 4); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// The restrict-qualified parameter gives the inlined read alias-scope metadata. Without it the
// compiler cannot tell the read from the direct loads still landing in the other stage and waits
// for all of them before every read; the reads of a stage are ordered after that stage's loads
// by the explicit waits of the ring barrier, as the plain LDS reads are.
__device__ __forceinline__ bf16x4 tr_read(lds_char_t *__restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)p);
}

__device__ __forceinline__ void issue_direct1(char *lds_tile, __amdgpu_buffer_rsrc_t rsrc, const DirectRows8 &d,
                                              uint32_t k_bytes, int wave, int i) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(lds_tile + (wave * 8 + i) * 1024), 16, d.voff[i],
                                           k_bytes, 0, 0);
}

// gfx9 s_waitcnt immediate: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
template <int N>
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14)); }

// Workgroup barrier for LDS traffic only: orders the waves' LDS accesses across it (each wave
// waits for its own LDS operations) but, unlike __syncthreads(), leaves the wave's global loads in
// flight, so operands an epilogue has requested keep arriving while the tile goes through LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier of the double buffer: each wave waits for its own direct loads (the stage
// about to be read) and its own LDS reads (of the stage about to be refilled), then meets the
// others. __syncthreads() is not used because its memory fence is not needed here; the
// scheduling barriers keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD b % 8) and each
// XCD has its own L2. Tile order: groups of GROUP_M m-tiles walk across all n-tiles, m fastest,
// and each XCD takes a contiguous run of that order, so the ~32 tiles an XCD holds at once span
// 4 m-tiles x 8 n-tiles and share their operand slices in that XCD's L2.
constexpr int GROUP_M = 4;
constexpr bool kXcdRemap = true;
__device__ __forceinline__ void tile_coords(int64_t b, int64_t ntiles, int64_t tiles_m, int64_t &mt, int64_t &nt) {
  int64_t id = b;
  if (kXcdRemap) {
    const int64_t n8 = ntiles / 8 * 8;
    if (b < n8) id = (b % 8) * (n8 / 8) + b / 8;
  }
  const int64_t tiles_n = ntiles / tiles_m;
  const int64_t per_group = GROUP_M * tiles_n;
  const int64_t g = id / per_group;
  const int64_t gm = min((int64_t)GROUP_M, tiles_m - g * GROUP_M);
  const int64_t in = id - g * per_group;
  mt = g * GROUP_M + in % gm;
  nt = in / gm;
}

// NF4 W in the direct kernel (template flag NF4W, forward layout): the B stage of a K-step is
// decoded from the packed weight instead of loaded. A K-step of 64 columns is exactly one NF4 block
// per W row; thread t owns half t % 2 (32 codes, 16 bytes) of the block of tile rows t / 2 and
// 128 + t / 2. Its codes, the word holding each block's quantised constant and the block's
// second-level scale come by direct-to-LDS loads (each lane lands its own data) into one of two
// staging buffers, two K-steps ahead, and the thread writes its rows as four 16-byte chunks of
// bf16 into the stage, at the slots the fragment reads expect. Per row it first forms the 16
// products bf16(q_i c) of its block constant c (the values the staging dequantisation would store
// for the 16 codes), as byte planes, so that each code then costs a byte permute instead of a table
// read and a multiply: w = bf16_RNE(fl32(q[code] c)), bit for bit the staged operand.
constexpr int kNf4TabOffset = 256 * kEpiPitch + 1024;   // 255 floats: fl32(v / 127), v = -127 .. 127
constexpr int kNf4StageOffset = kNf4TabOffset + 1024;   // two staging buffers
constexpr int kNf4Buf = 12288;   // codes [2][256][16 B], constant words [2][256][4 B], scales [2][256][4 B]
// products bf16(q_i c), i = 0 .. 15, as byte planes: lo[j] / hi[j] hold the low / high bytes of
// entries 4j .. 4j+3
struct Nf4Planes {
  uint32_t lo[4], hi[4];
};
__device__ __forceinline__ void nf4_planes_half(Nf4Planes &pl, const float *q, float c, int h) {
#pragma unroll
  for (int j = 2 * h; j < 2 * h + 2; ++j) {
    const uint32_t p0 = pack_bf16x2(__fmul_rn(q[4 * j], c), __fmul_rn(q[4 * j + 1], c));
    const uint32_t p1 = pack_bf16x2(__fmul_rn(q[4 * j + 2], c), __fmul_rn(q[4 * j + 3], c));
    pl.lo[j] = __builtin_amdgcn_perm(p1, p0, 0x06040200u);
    pl.hi[j] = __builtin_amdgcn_perm(p1, p0, 0x07050301u);
  }
}
// (m & x) | (~m & y), one v_bfi_b32
__device__ __forceinline__ uint32_t nf4_sel(uint32_t m, uint32_t x, uint32_t y) { return (m & x) | (~m & y); }
// four codes at once: byte j of c7 = code_j & 7, byte j of m = 0xff where code_j >= 8; returns the
// low bytes (lo) and high bytes (hi) of the four products
__device__ __forceinline__ void nf4_look4(const Nf4Planes &pl, uint32_t c7, uint32_t m, uint32_t &lo, uint32_t &hi) {
  lo = nf4_sel(m, __builtin_amdgcn_perm(pl.lo[3], pl.lo[2], c7), __builtin_amdgcn_perm(pl.lo[1], pl.lo[0], c7));
  hi = nf4_sel(m, __builtin_amdgcn_perm(pl.hi[3], pl.hi[2], c7), __builtin_amdgcn_perm(pl.hi[1], pl.hi[0], c7));
}
// The eight codes of word w in two halves (for the scheduling of the K-step): the even elements
// (high nibbles) give their bf16 values as (e0, e2) and (e4, e6) ...
__device__ __forceinline__ void nf4_even(const Nf4Planes &pl, uint32_t w, uint32_t &e01, uint32_t &e23) {
  const uint32_t c7 = (w >> 4) & 0x07070707u;
  // byte j's bit 7 (code 2j's bit 3) replicated over byte j: permute selectors 8 - 11 copy the
  // sign bits of bytes 1 and 3 of either source
  const uint32_t m = __builtin_amdgcn_perm(w, w << 8, 0x0b090a08u);
  uint32_t lo, hi;
  nf4_look4(pl, c7, m, lo, hi);
  e01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  e23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}
// ... the odd ones (low nibbles) give their low and high bytes ...
__device__ __forceinline__ void nf4_odd(const Nf4Planes &pl, uint32_t w, uint32_t &lo, uint32_t &hi) {
  const uint32_t c7 = w & 0x07070707u;
  const uint32_t m = __builtin_amdgcn_perm(w << 4, w << 12, 0x0b090a08u);
  nf4_look4(pl, c7, m, lo, hi);
}
// ... and the two complete the chunk: bf16 elements 0 .. 7 in order
__device__ __forceinline__ u32x4_t nf4_chunk(uint32_t e01, uint32_t e23, uint32_t lo, uint32_t hi) {
  const uint32_t o01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  const uint32_t o23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  return u32x4_t{__builtin_amdgcn_perm(o01, e01, 0x05040100u), __builtin_amdgcn_perm(o01, e01, 0x07060302u),
                 __builtin_amdgcn_perm(o23, e23, 0x05040100u), __builtin_amdgcn_perm(o23, e23, 0x07060302u)};
}

// SPLIT (split-K): the grid holds a.ksplit copies of the tile grid; copy s reduces over K-steps
// [s nk / S, (s+1) nk / S) and stores its fp32 partial product to out + s M N (the caller adds
// the partials in split order). Used where a product has few output tiles and a long reduction.
template <int EPI, bool KSEG, bool BT, bool SPLIT, bool NF4W>
__global__ __launch_bounds__(NT, 1) void k_gemm_direct(DirectArgs a) {
  static_assert(!NF4W || (!KSEG && !BT && !SPLIT && EPI != EPI_SWIGLU && EPI != EPI_SWIGLU_BWD),
                "NF4 W: plain forward products");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *lds_a = smem;                               // 2 stages
  char *lds_b = smem + 2 * DTILE;                   // 2 stages
  const int t = threadIdx.x;
  const int lane = t & 63;
  // the wave index is uniform: keep it in a scalar register so that the LDS destinations of the
  // direct loads (the M0 operand) are scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // tile -> (m tile, segment, n tile within the segment)
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  int64_t mt, nt;
  int64_t tiles_here = gridDim.x, split = 0;
  if constexpr (SPLIT) {
    tiles_here = gridDim.x / a.ksplit;
    split = blockIdx.x / tiles_here;
  }
  tile_coords(SPLIT ? blockIdx.x % tiles_here : blockIdx.x, tiles_here, tiles_m, mt, nt);
  int sidx = 0;
#pragma unroll
  for (int q = 1; q < kMaxSegs; ++q)
    if (q < a.nseg && nt >= a.seg[q].ntile0) sidx = q;
  const GemmSeg sg = a.seg[sidx];
  nt -= sg.ntile0;
  // a gate/up pair: the tile's B rows 0..127 are gate rows n0.., rows 128..255 the same up rows
  constexpr bool PAIR = EPI == EPI_SWIGLU;
  static_assert(!PAIR || (!KSEG && !BT && !SPLIT), "the gate/up pair is a plain forward product");
  const int64_t m0 = mt * BM;
  const int64_t n0 = nt * (PAIR ? BN / 2 : BN);

  floatx16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  int nk = (int)(a.K / DBK);
  int64_t kt0 = 0;                                  // first K-step of this split
  if constexpr (SPLIT) {
    const int nk_all = nk;
    kt0 = split * nk_all / a.ksplit;
    nk = (int)((split + 1) * nk_all / a.ksplit - kt0);
  }
  const int k_last = nk - 1;
  // Operand sources. In reduction-segment mode the A loads (one step ahead of the B loads)
  // and the B loads each follow their own segment, switched when their step crosses into it.
  __amdgpu_buffer_rsrc_t rs_a, rs_b;
  DirectRows8 da, db;
  int pa = 0, pb = 0;                               // segment of the next A / B load step
  if constexpr (KSEG) {
    rs_a = make_rsrc(a.kseg[0].act, a.M * a.kseg[0].K * 2);
    rs_b = make_rsrc(a.kseg[0].w, sg.N * a.kseg[0].K * 2);
    make_direct_rows8(da, a.M, a.kseg[0].K, m0, wave, lane);
  } else {
    // (pair: waves 0-1 fill the gate half of the B tile, waves 2-3 the up half)
    const uint16_t *wb = PAIR && wave >= 2 ? a.x.w2 : sg.w;
    rs_a = make_rsrc(a.act + kt0 * DBK, a.M * a.K * 2 - kt0 * DBK * 2);
    if constexpr (NF4W)
      rs_b = rs_a;   // (no B loads: the B stage is decoded from the packed weight)
    else
      rs_b = BT ? make_rsrc(wb + kt0 * DBK * sg.N, (a.K - kt0 * DBK) * sg.N * 2)
                : make_rsrc(wb + kt0 * DBK, sg.N * a.K * 2 - kt0 * DBK * 2);
    make_direct_rows8(da, a.M, a.K, m0, wave, lane);
  }
  if constexpr (BT)
    make_direct_rows8_t(db, sg.N, n0, wave, lane);   // the same for every reduction segment
  else if constexpr (!NF4W)   // (pair: the up half's LDS rows 128.. hold up rows n0..)
    make_direct_rows8(db, sg.N, KSEG ? a.kseg[0].K : a.K, PAIR && wave >= 2 ? n0 - 128 : n0, wave, lane);

  // NF4 W: this thread's two half-rows of every K-step's block (rows past N read row N - 1: they
  // feed only unstored outputs), staged in buffer k % 2 from two K-steps before the decode of
  // K-step k until the barrier after it; the row's product planes and the decode's intermediates
  __amdgpu_buffer_rsrc_t rs_codes, rs_qa, rs_s2;
  uint32_t nf_voff[2], nf_brow[2];
  Nf4Planes nfp;
  u32x4_t nf_codes[2];
  uint32_t nf_qw[2];
  float nf_s2[2], nf_c8[2], nf_c = 0.0f;
  uint32_t nf_e01 = 0, nf_e23 = 0, nf_lo = 0, nf_hi = 0;
  char *const nf_lds = smem + kNf4StageOffset;
  const float *nf_tab = reinterpret_cast<const float *>(smem + kNf4TabOffset);
  if constexpr (NF4W) {
    const int64_t kb = a.K / DBK;                       // blocks per row
    rs_codes = make_rsrc(sg.codes, sg.N * a.K / 2);
    rs_qa = make_rsrc(sg.qabsmax, sg.N * kb);
    rs_s2 = make_rsrc(sg.absmax2, (sg.N * kb + 255) / 256 * 4);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int64_t row = min(n0 + p * 128 + (t >> 1), sg.N - 1);
      nf_voff[p] = (uint32_t)(row * a.K / 2 + 16 * (t & 1));
      nf_brow[p] = (uint32_t)(row * kb);
    }
    if (t < 255) reinterpret_cast<float *>(smem + kNf4TabOffset)[t] = int8_level(t - 127);
  }
  // K-step k's codes, constant words and scales of this wave's lanes into staging buffer `buf`
  // (lane l of wave w lands at 16 (64 w + l) or 4 (64 w + l) of its array: its own thread's slots).
  // The constant is read as the aligned word holding its byte (N K / 64 is a multiple of 4, so the
  // word never reaches past the array).
  auto nf4_issue = [&](int buf, int k) {
    char *b = nf_lds + buf * kNf4Buf;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t blk = nf_brow[p] + (uint32_t)k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_codes, (lds_void_t *)(b + p * 4096 + wave * 1024), 16, nf_voff[p],
                                               (uint32_t)k * 32, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_qa, (lds_void_t *)(b + 8192 + p * 1024 + wave * 256), 4, blk & ~3u,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s2, (lds_void_t *)(b + 10240 + p * 1024 + wave * 256), 4,
                                               (blk >> 8) * 4, 0, 0, 0);
    }
  };
  // Piece p (0 .. 31) of decoding K-step k from staging buffer `buf` into the B area of stage
  // `buf`: the staged words (0, 1) and the level table (1), per row the block constant and product
  // planes (two pieces), then per word of codes three pieces: the even elements, the odd ones, the
  // chunk's assembly and store. The pieces go one per fragment group: 0 - 7 in the sub-step after
  // the ring barrier that frees the stage, 8 - 31 in the three sub-steps before the next one.
  auto nf4_piece = [&](int p, int buf, int k) {
    const char *b = nf_lds + buf * kNf4Buf;
    if (p == 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        nf_qw[r] = *reinterpret_cast<const uint32_t *>(b + 8192 + r * 1024 + 4 * t);
        nf_s2[r] = *reinterpret_cast<const float *>(b + 10240 + r * 1024 + 4 * t);
      }
    } else if (p == 1) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int v = (int)(int8_t)(nf_qw[r] >> (8 * ((nf_brow[r] + (uint32_t)k) & 3u)));
        nf_c8[r] = nf_tab[v + 127];
        nf_codes[r] = *reinterpret_cast<const u32x4_t *>(b + r * 4096 + 16 * t);
      }
    } else if (p == 2 || p == 16) {
      const int r = p == 2 ? 0 : 1;
      nf_c = decode_absmax(nf_c8[r], nf_s2[r], sg.mean);
      nf4_planes_half(nfp, a.nf4_q, nf_c, 0);
    } else if (p == 3 || p == 17) {
      nf4_planes_half(nfp, a.nf4_q, nf_c, 1);
    } else if ((p >= 4 && p <= 15) || (p >= 18 && p <= 29)) {
      const int r = p <= 15 ? 0 : 1, i = p - (r ? 18 : 4), d = i / 3, part = i % 3;
      const uint32_t w = nf_codes[r][d];
      if (part == 0) {
        nf4_even(nfp, w, nf_e01, nf_e23);
      } else if (part == 1) {
        nf4_odd(nfp, w, nf_lo, nf_hi);
      } else {
        char *dst = lds_b + buf * DTILE + dlds_off(r * 128 + (t >> 1), 4 * (t & 1) + d);
        *reinterpret_cast<u32x4_t *>(dst) = nf4_chunk(nf_e01, nf_e23, nf_lo, nf_hi);
      }
    }
  };
  // bytes from one K-step of B to the next
  const int64_t b_step_bytes = BT ? (int64_t)DBK * sg.N * 2 : (int64_t)DBK * 2;
  // byte offset along K of global step `step` inside its segment (moving pa / pb forward)
  auto a_kb = [&](int step) -> uint32_t {
    if constexpr (KSEG) {
      while (pa + 1 < a.nkseg && step >= a.kseg[pa + 1].step0) {
        ++pa;
        rs_a = make_rsrc(a.kseg[pa].act, a.M * a.kseg[pa].K * 2);
        make_direct_rows8(da, a.M, a.kseg[pa].K, m0, wave, lane);
      }
      return (uint32_t)(step - a.kseg[pa].step0) * DBK * 2;
    } else {
      return (uint32_t)step * DBK * 2;
    }
  };
  auto b_kb = [&](int step) -> uint32_t {
    if constexpr (KSEG) {
      while (pb + 1 < a.nkseg && step >= a.kseg[pb + 1].step0) {
        ++pb;
        rs_b = make_rsrc(a.kseg[pb].w, sg.N * a.kseg[pb].K * 2);
        if constexpr (!BT) make_direct_rows8(db, sg.N, a.kseg[pb].K, n0, wave, lane);
      }
      return (uint32_t)((step - a.kseg[pb].step0) * b_step_bytes);
    } else {
      return (uint32_t)(step * b_step_bytes);
    }
  };

  if constexpr (EPI == EPI_BF16_ROPE) {
    // the tile rows' table rows, for the epilogue (an LDS area of their own, past the tile)
    if (sg.rope) {
      const int64_t m = min(m0 + t, a.M - 1);
      reinterpret_cast<int *>(smem + kPosOffset)[t] = min(max(a.x.positions[m], 0), a.x.n_pos - 1);
    }
  }
  // stage 0 <- step 0 (first, so that its latency overlaps the LoRA prologue)
  if constexpr (NF4W) {
    nf4_issue(0, 0);
    nf4_issue(1, min(1, k_last));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    issue_direct1(lds_a, rs_a, da, 0, wave, i);
    if constexpr (!NF4W) issue_direct1(lds_b, rs_b, db, 0, wave, i);
  }
  // ---- LoRA prologue: acc = s * (B_seg . U_seg^T) over r (B_seg [N][r], U_seg [M][r]) ----
  // (reduction-segment mode: the sum of the segments' terms, in segment order)
  if (a.adapters) {
#pragma unroll 1
   for (int p = 0; p < (KSEG ? a.nkseg : 1); ++p) {
    // (pair: the waves of the up half (wn = 1) take the up member's U and B)
    const uint16_t *lr_act = KSEG ? a.kseg[p].lr_act : PAIR && wn ? a.x.lr_act2 : sg.lr_act;
    const uint16_t *lr_w = KSEG ? a.kseg[p].lr_w : PAIR && wn ? a.x.lr_w2 : sg.lr_w;
    const int64_t nw0 = PAIR ? n0 : n0 + wn * 128;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (16 * h >= a.r) break;
      const int jl = 16 * h + 8 * (lane >> 5);
      bf16x8 la[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + 32 * i + (lane & 31);
        u32x4_t v = {0, 0, 0, 0};
        if (m < a.M && jl < a.r) v = *reinterpret_cast<const u32x4_t *>(lr_act + m * a.r + jl);
        la[i] = as_bf16x8(v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = nw0 + 32 * j + (lane & 31);
        u32x4_t v = {0, 0, 0, 0};
        if (n < sg.N && jl < a.r) v = *reinterpret_cast<const u32x4_t *>(lr_w + n * a.r + jl);
        lb[j] = as_bf16x8(v);
      }
      // the scale on the U fragments, bf16(s u): for s a power of two (alpha / r with both powers
      // of two, the usual case) exact, as are then all the fp32 partial sums, so the result is
      // bit-identical to scaling the fp32 sum; any other s rounds s u to bf16 once
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) la[i][e] = (__bf16)((float)la[i][e] * a.scale);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[j], la[i], acc[i][j], 0, 0, 0);
    }
   }
  }

  // fragment q of sub-step s2 (16 K-columns) of a stage, in consumption order: 0 -> fa0,
  // 1..4 -> fb0..fb3, 5..7 -> fa1..fa3 (the first MFMAs of a batch walk j fastest)
  auto read_frag = [&](int stage, int s2, int q, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
    const int chunk = 2 * s2 + (lane >> 5);
    if (q == 0 || q >= 5) {
      const int i = q == 0 ? 0 : q - 4;
      fa[i] = *reinterpret_cast<const bf16x8 *>(lds_a + stage * DTILE + dlds_off(wm * 128 + 32 * i + (lane & 31), chunk));
    } else {
      const int j = q - 1;
      if constexpr (BT) {
        // 16-lane group g: columns 16 (g % 2) .. +15 of fragment j, K-rows 8 (g / 2) + 0..3 and
        // + 4..7 of the sub-step; source lane l of a group points at K-row l / 4, columns
        // 4 (l % 4) .. +3, and receives column l, K-rows 0..3 of the group's block
        const int g = lane >> 4, sl = lane & 15;
        const int row = 16 * s2 + 8 * (g >> 1) + (sl >> 2);
        const int c = wn * 16 + 4 * j + 2 * (g & 1) + ((sl & 3) >> 1);
        lds_char_t *p = (lds_char_t *)(lds_b + stage * DTILE) + dlds_off_t(row, c) + 8 * (sl & 1);
        const bf16x4 lo = tr_read(p);
        const bf16x4 hi = tr_read(p + 4 * 512);
        fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        fb[j] = *reinterpret_cast<const bf16x8 *>(lds_b + stage * DTILE + dlds_off(wn * 128 + 32 * j + (lane & 31), chunk));
      }
    }
  };
  // One sub-step: its 16 MFMAs on (cA, cB) in pairs; before each pair, one fragment of the
  // sub-step that follows is read into (nA, nB) from stage `rstage` at K-slice `rs2`, and, when
  // `lhalf` >= 0, one of the 8 direct loads of half `lhalf` (0: operand A, 1: operand B) of a
  // K-step goes out to stage `lstage`; each group is fenced so the interleaving holds.
  // (NF4 W: with np0 >= 0, pieces np0 .. np0+7 of decoding staging buffer nset, K-step nk_dec, go
  // one per group)
  auto substep = [&](int rstage, int rs2, int lhalf, int lstage, uint32_t kb, bf16x8 (&cA)[4], bf16x8 (&cB)[4],
                     bf16x8 (&nA)[4], bf16x8 (&nB)[4], int np0 = -1, int nset = 0, int nk_dec = 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      read_frag(rstage, rs2, q, nA, nB);
      const int i = q >> 1, j0 = 2 * (q & 1);
      acc[i][j0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cB[j0], cA[i], acc[i][j0], 0, 0, 0);
      acc[i][j0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cB[j0 + 1], cA[i], acc[i][j0 + 1], 0, 0, 0);
      if (lhalf == 0) issue_direct1(lds_a + lstage * DTILE, rs_a, da, kb, wave, q);
      if (lhalf == 1) issue_direct1(lds_b + lstage * DTILE, rs_b, db, kb, wave, q);
      if constexpr (NF4W) {
        if (np0 >= 0) {
          nf4_piece(np0 + q, nset, nk_dec);
          // the group's order: LDS reads, an MFMA, half of the decode's VALU work, the other MFMA,
          // the rest, then the direct load and the chunk store, so that the VALU work runs beside
          // the matrix cores instead of after them
          __builtin_amdgcn_sched_group_barrier(0x0100, 8, 0);    // DS read
          __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);    // MFMA
          __builtin_amdgcn_sched_group_barrier(0x0002, 8, 0);    // VALU
          __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);    // MFMA
          __builtin_amdgcn_sched_group_barrier(0x0002, 32, 0);   // VALU
          __builtin_amdgcn_sched_group_barrier(0x0010, 1, 0);    // VMEM
          __builtin_amdgcn_sched_group_barrier(0x0200, 1, 0);    // DS write
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (NF4W) {
    wait_vm_all();   // this thread's staged K-steps 0 and 1
    lds_barrier();   // the level table is written
#pragma unroll
    for (int p = 0; p < 32; ++p) nf4_piece(p, 0, 0);
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // buffer 0 read: refill it
    nf4_issue(0, min(2, k_last));
    // the first pieces of K-step 1's decode, as the sub-step after a ring barrier does in the loop
#pragma unroll
    for (int p = 0; p < 8; ++p) nf4_piece(p, 1, min(1, k_last));
  }
  // operand A of step 1 to stage 1 (free); then wait for step 0 only, and read its first fragments
  {
    const uint32_t kb = a_kb(min(1, k_last));
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_direct1(lds_a + DTILE, rs_a, da, kb, wave, i);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NF4W) {
    wait_vm<14>();   // all but K-step 2's staging (6) and operand A of step 1 (8)
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0): stage 0's W written
  } else {
    wait_vm<8>();
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 ca[4], cb[4], na[4], nb[4];
#pragma unroll
  for (int q = 0; q < 8; ++q) read_frag(0, 0, q, ca, cb);
  // Step kt (stage st, its sub-step 0 fragments in (ca, cb); operand A of step kt+1 already on
  // its way to stage st^1):
  //   sub-step 0 sends operand B of step kt+1 to stage st^1;
  //   after sub-step 2 each wave waits for its own loads and LDS reads, and all meet: step
  //   kt+1 is visible, and no wave reads stage st any more;
  //   sub-step 3 reads the first fragments of step kt+1 while its MFMAs run (the matrix cores
  //   never wait on LDS after the barrier) and sends operand A of step kt+2 to stage st.
  // Every load has at least two sub-steps to land. The last steps re-load the last K-step into
  // stages that are never read again, so the loop needs no branch.
  // (unrolled by two so that the stage of each step is a constant)
  // NF4 W: the three sub-steps before the barrier finish decoding step kt+1 (staging buffer nx) into
  // stage nx in place of its B loads; after the barrier, buffer nx is free and takes step kt+3's
  // data (which the barrier of step kt+1 waits for, a step before its decode starts), and the
  // sub-step after it starts decoding step kt+2 (buffer st, landed) into stage st, which the
  // barrier has just freed.
  auto step = [&](int kt, int st) {
    const int nx = st ^ 1;
    const uint32_t kb1 = NF4W ? 0u : b_kb(min(kt + 1, k_last));
    const uint32_t kb2 = a_kb(min(kt + 2, k_last));
    const int kd = min(kt + 1, k_last);
    substep(st, 1, NF4W ? -1 : 1, nx, kb1, ca, cb, na, nb, NF4W ? 8 : -1, nx, kd);
    substep(st, 2, -1, 0, 0, na, nb, ca, cb, NF4W ? 16 : -1, nx, kd);
    substep(st, 3, -1, 0, 0, ca, cb, na, nb, NF4W ? 24 : -1, nx, kd);
    ring_barrier();
    if constexpr (NF4W) nf4_issue(nx, min(kt + 3, k_last));
    substep(nx, 0, 0, st, kb2, na, nb, ca, cb, NF4W ? 0 : -1, st, min(kt + 2, k_last));
  };
  if constexpr (NF4W) {
    // (the loop is re-entered only after its second step: a path from the first step back to the
    // top would make the compiler wait there for the codes that step has just requested)
    for (int kt = 0;; kt += 2) {
      step(kt, 0);
      if (kt + 1 >= nk) break;
      step(kt + 1, 1);
      if (kt + 2 >= nk) break;
    }
  } else {
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, 0);
      if (kt + 1 < nk) step(kt + 1, 1);
    }
  }
  wait_vm_all();

  // ---- epilogue: lane holds row m = 32 i + lane%32, columns 32 j + 8 g + 4 (lane/32) .. +3 ----
  if constexpr (EPI == EPI_BF16 || EPI == EPI_BF16_RES || EPI == EPI_BF16_ROPE || EPI == EPI_SWIGLU ||
                EPI == EPI_SWIGLU_BWD) {
    // Through LDS (free once every wave is past the loop): the 256 x 256 bf16 tile is written
    // with 8-byte stores at a 528-byte row pitch (2-way bank conflicts at most), then read back
    // as 16-byte row chunks so that every global store is a 16-byte piece of a 512-byte row run
    // (non-temporal: the tile is not read again by this kernel; measured 1-2% faster).
    // The glue operands the epilogue reads from global memory (the residual, the rows'
    // positions, the SwiGLU's inputs) are requested before the tile goes through LDS, or a batch
    // ahead of their use, so that one wave per SIMD does not wait out their latency row by row.
    constexpr int RPP = NT / 32;                  // rows per pass of a 32-chunk row loop
    constexpr int NP = BM / RPP;                  // its passes
    const int chunk = t & 31;
    const int64_t n = n0 + 8 * chunk;
    const bool n_ok = n < sg.N;
    auto row_of = [&](int p) { return m0 + p * RPP + (t >> 5); };
    u32x4_t pre[NP];                              // the residual's chunks of this thread's rows
    int posv[BM / (NT / 16)];                     // the rotation's table rows (16-chunk loop)
    if constexpr (EPI == EPI_BF16_ROPE) {
      if (sg.rope) {
#pragma unroll
        for (int p = 0; p < BM / (NT / 16); ++p)
          posv[p] = reinterpret_cast<const int *>(smem + kPosOffset)[p * (NT / 16) + (t >> 4)];
      }
    }
    if constexpr (EPI == EPI_BF16_RES) {
      if (sg.res) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int64_t m = row_of(p);
          pre[p] = m < a.M && n_ok ? *reinterpret_cast<const u32x4_t *>(sg.res + m * sg.N + n) : u32x4_t{0, 0, 0, 0};
        }
      }
    }
    // rotary embedding (EPI_BF16_ROPE): thread k = t % 16 of a row takes 8 pairs of one head, the
    // chunk at column c1 and its partner D/2 to the right, 16 rows per pass; the (cos, sin) table
    // rows of a batch of 4 passes are loaded a batch ahead, the first batch before the LDS pass
    const int D = EPI == EPI_BF16_ROPE ? a.x.rope_dim : 128, half = D / 2, cph = half / 8, k = t & 15;
    const int c1 = (k / cph) * D + 8 * (k % cph), c2 = c1 + half;
    const int64_t n1 = n0 + c1;
    const float *cs = a.x.rope_cs + 16 * (k % cph);
    constexpr int PB = 4, NPR = BM / (NT / 16);
    floatx4_t tb[2][PB][4];
    auto fetch_cs = [&](int buf, int b) {
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          tb[buf][q][w] = *reinterpret_cast<const floatx4_t *>(cs + (int64_t)posv[b * PB + q] * D + 4 * w);
    };
    if constexpr (EPI == EPI_BF16_ROPE) {
      if (sg.rope) fetch_cs(0, 0);
    }
    constexpr int SB = 8;                         // SwiGLU backward: rows per batch
    u32x4_t gbuf[2][SB], ubuf[2][SB];
    auto fetch_gu = [&](int buf, int b) {
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        const int64_t m = row_of(b * SB + q);
        const bool ok = m < a.M && n_ok;
        gbuf[buf][q] = ok ? *reinterpret_cast<const u32x4_t *>(a.x.gate + m * sg.N + n) : u32x4_t{0, 0, 0, 0};
        ubuf[buf][q] = ok ? *reinterpret_cast<const u32x4_t *>(a.x.up + m * sg.N + n) : u32x4_t{0, 0, 0, 0};
      }
    };
    if constexpr (EPI == EPI_SWIGLU_BWD) fetch_gu(0, 0);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = wn * 128 + 32 * j + 8 * g + 4 * (lane >> 5);
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
          o.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<uint2 *>(smem + r * kEpiPitch + c * 2) = o;
        }
    }
    lds_barrier();
    if constexpr (EPI == EPI_SWIGLU) {
      // row r of the tile: gate columns n0 .. n0+127 in chunks 0-15, the same up columns in
      // chunks 16-31; a thread takes chunk c of both halves, 16 rows per pass
      const int c = t & 15;
      const int64_t nc = n0 + 8 * c;
#pragma unroll 4
      for (int p = 0; p < BM / (NT / 16); ++p) {
        const int r = p * (NT / 16) + (t >> 4);
        const int64_t m = m0 + r;
        const u32x4_t gv = *reinterpret_cast<const u32x4_t *>(smem + r * kEpiPitch + c * 16);
        const u32x4_t uv = *reinterpret_cast<const u32x4_t *>(smem + r * kEpiPitch + (c + 16) * 16);
        if (m < a.M && nc < sg.N) {
          const int64_t o = m * sg.N + nc;
          if (sg.out) __builtin_nontemporal_store(gv, reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(sg.out) + o));
          if (a.x.out2) __builtin_nontemporal_store(uv, reinterpret_cast<u32x4_t *>(a.x.out2 + o));
          __builtin_nontemporal_store(swiglu8(gv, uv), reinterpret_cast<u32x4_t *>(a.x.mout + o));
        }
      }
      return;
    }
    if constexpr (EPI == EPI_SWIGLU_BWD) {
      // the tile is dm; the gradients of the SwiGLU's inputs at the same elements, a batch of
      // rows' gate and up in flight while the previous batch is computed
#pragma unroll
      for (int b = 0; b < NP / SB; ++b) {
        if (b + 1 < NP / SB) fetch_gu((b + 1) & 1, b + 1);
#pragma unroll
        for (int q = 0; q < SB; ++q) {
          const int p = b * SB + q;
          const int r = p * RPP + (t >> 5);
          const int64_t m = m0 + r;
          const u32x4_t v = *reinterpret_cast<const u32x4_t *>(smem + r * kEpiPitch + chunk * 16);
          if (m < a.M && n_ok) {
            const int64_t o = m * sg.N + n;
            u32x4_t dg, du;
            swiglu8_bwd(gbuf[b & 1][q], ubuf[b & 1][q], v, dg, du);
            __builtin_nontemporal_store(dg, reinterpret_cast<u32x4_t *>(a.x.dgate + o));
            __builtin_nontemporal_store(du, reinterpret_cast<u32x4_t *>(a.x.dup + o));
          }
        }
      }
      return;
    }
    if (EPI == EPI_BF16_ROPE && sg.rope) {   // (a constant false in the other kernels)
      // the rotary embedding of the rounded tile (columns = whole heads of D)
#pragma unroll
      for (int b = 0; b < NPR / PB; ++b) {
        if (b + 1 < NPR / PB) fetch_cs((b + 1) & 1, b + 1);
#pragma unroll
        for (int q = 0; q < PB; ++q) {
          const int r = (b * PB + q) * (NT / 16) + (t >> 4);
          const int64_t m = m0 + r;
          const u32x4_t x1 = *reinterpret_cast<const u32x4_t *>(smem + r * kEpiPitch + c1 * 2);
          const u32x4_t x2 = *reinterpret_cast<const u32x4_t *>(smem + r * kEpiPitch + c2 * 2);
          if (m < a.M && n1 < sg.N) {
            float cv[8], sv[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              cv[2 * w] = tb[b & 1][q][w][0];
              sv[2 * w] = tb[b & 1][q][w][1];
              cv[2 * w + 1] = tb[b & 1][q][w][2];
              sv[2 * w + 1] = tb[b & 1][q][w][3];
            }
            u32x4_t y1, y2;
            rope_chunk8(x1, x2, cv, sv, y1, y2);
            uint16_t *o = reinterpret_cast<uint16_t *>(sg.out) + m * sg.N + n1;
            __builtin_nontemporal_store(y1, reinterpret_cast<u32x4_t *>(o));
            __builtin_nontemporal_store(y2, reinterpret_cast<u32x4_t *>(o + half));
          }
        }
      }
      return;
    }
    if constexpr (EPI == EPI_BF16_RES) {
      if (sg.res) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int r = p * RPP + (t >> 5);
          const int64_t m = m0 + r;
          u32x4_t v = *reinterpret_cast<const u32x4_t *>(smem + r * kEpiPitch + chunk * 16);
          if (m < a.M && n_ok) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = add_bf16_word(pre[p][q], v[q]);
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(sg.out) + m * sg.N + n));
          }
        }
        return;
      }
    }
#pragma unroll 4
    for (int p = 0; p < NP; ++p) {
      const int r = p * RPP + (t >> 5);
      const int64_t m = m0 + r;
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(smem + r * kEpiPitch + chunk * 16);
      if (m < a.M && n_ok)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(reinterpret_cast<uint16_t *>(sg.out) + m * sg.N + n));
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * 128 + 32 * j + 8 * g + 4 * (lane >> 5);
        if (m < a.M && n < sg.N) {
          const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1], v2 = acc[i][j][4 * g + 2],
                      v3 = acc[i][j][4 * g + 3];
          floatx4_t *o = reinterpret_cast<floatx4_t *>(reinterpret_cast<float *>(sg.out) + split * a.M * sg.N +
                                                      m * sg.N + n);
          if constexpr (EPI == EPI_F32_SET) {
            const floatx4_t v = {v0, v1, v2, v3};
            __builtin_nontemporal_store(v, o);
          } else {
            floatx4_t cur = *o;
            cur[0] = __fadd_rn(cur[0], v0);
            cur[1] = __fadd_rn(cur[1], v1);
            cur[2] = __fadd_rn(cur[2], v2);
            cur[3] = __fadd_rn(cur[3], v3);
            *o = cur;
          }
        }
      }
    }
  }
}

constexpr size_t kDirectSmemBytes = 256 * kEpiPitch > 4 * DTILE ? 256 * kEpiPitch : 4 * DTILE;
static_assert(256 * kEpiPitch <= kDirectSmemBytes, "the epilogue tile must fit in the ring's LDS");

// N tiles of a segment (a gate/up pair: 128 columns of each member per tile)
int64_t seg_ntiles(int64_t N, int epi) {
  const int64_t w = epi == EPI_SWIGLU ? BN / 2 : BN;
  return (N + w - 1) / w;
}

template <int EPI, bool KSEG, bool BT, bool SPLIT = false, bool NF4W = false>
lsn_status launch_direct_one(const DirectArgs &a, hipStream_t s) {
  // (past the tile: the rotary epilogue's positions, 1 KB; then the NF4 level table, 1 KB, and the
  // NF4 staging buffers)
  constexpr size_t smem_bytes =
      kDirectSmemBytes + (NF4W ? 2048 + 2 * kNf4Buf : EPI == EPI_BF16_ROPE ? 256 * sizeof(int) : 0);
  static_assert(EPI != EPI_BF16_ROPE || kPosOffset == (int)kDirectSmemBytes, "positions past the tile");
  static_assert(!NF4W || kNf4StageOffset + 2 * kNf4Buf == (int)smem_bytes, "the NF4 areas past the positions");
  static_assert(smem_bytes <= 160 * 1024, "LDS of one workgroup");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_direct<EPI, KSEG, BT, SPLIT, NF4W>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_bytes);
    if (e != hipSuccess) return check_hip(e, "gemm_direct smem attribute");
    attr_set = true;
  }
  int64_t ntiles_n = 0;
  for (int q = 0; q < a.nseg; ++q) ntiles_n += seg_ntiles(a.seg[q].N, EPI);
  const int64_t tiles = ((a.M + BM - 1) / BM) * ntiles_n * (SPLIT ? a.ksplit : 1);
  hipLaunchKernelGGL((k_gemm_direct<EPI, KSEG, BT, SPLIT, NF4W>), dim3((unsigned)tiles), dim3(NT), smem_bytes, s, a);
  return check_hip(hipGetLastError(), "k_gemm_direct launch");
}

constexpr size_t kSmemBytes = 4 * TILE_BYTES + (16 + 256) * sizeof(float);

template <int LAYOUT, int WKIND, int EPI>
lsn_status launch_one(const GemmArgs &a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm<LAYOUT, WKIND, EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
    if (e != hipSuccess) return check_hip(e, "gemm smem attribute");
    attr_set = true;
  }
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.Nout + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm<LAYOUT, WKIND, EPI>), dim3((unsigned)tiles), dim3(NT), kSmemBytes, s, a);
  return check_hip(hipGetLastError(), "k_gemm launch");
}

}  // namespace

namespace {
template <bool KSEG, bool BT>
lsn_status launch_direct_epi(const DirectArgs &a, int epi, hipStream_t s) {
  if constexpr (!KSEG && !BT) {
    if (a.nf4) {
      if (epi != EPI_BF16) return fail(LSN_E_ARG, "gemm_direct: NF4 W takes the bf16 epilogues");
      bool res = false, rope = false;
      for (int q = 0; q < a.nseg; ++q) {
        res = res || a.seg[q].res;
        rope = rope || a.seg[q].rope;
      }
      if (rope) return launch_direct_one<EPI_BF16_ROPE, false, false, false, true>(a, s);
      if (res) return launch_direct_one<EPI_BF16_RES, false, false, false, true>(a, s);
      return launch_direct_one<EPI_BF16, false, false, false, true>(a, s);
    }
  }
  if (a.nf4) return fail(LSN_E_ARG, "gemm_direct: NF4 W is for the plain forward layout");
  if (epi == EPI_BF16) {
    bool res = false, rope = false;
    for (int q = 0; q < a.nseg; ++q) {
      res = res || a.seg[q].res;
      rope = rope || a.seg[q].rope;
    }
    if constexpr (!KSEG && !BT) {
      if (rope) return launch_direct_one<EPI_BF16_ROPE, false, false>(a, s);
      if (res) return launch_direct_one<EPI_BF16_RES, false, false>(a, s);
    }
    if (res || rope) return fail(LSN_E_ARG, "gemm_direct: the residual and rotary epilogues are forward-only");
    return launch_direct_one<EPI_BF16, KSEG, BT>(a, s);
  }
  if (epi == EPI_F32_ADD) return launch_direct_one<EPI_F32_ADD, KSEG, BT>(a, s);
  if constexpr (!KSEG) {
    if (epi == EPI_SWIGLU_BWD) return launch_direct_one<EPI_SWIGLU_BWD, false, BT>(a, s);
    if constexpr (!BT) {
      if (epi == EPI_SWIGLU) return launch_direct_one<EPI_SWIGLU, false, false>(a, s);
    }
  }
  if (epi != EPI_F32_SET) return fail(LSN_E_ARG, "gemm_direct: epilogue %d not available for this operand layout", epi);
  return launch_direct_one<EPI_F32_SET, KSEG, BT>(a, s);
}
}  // namespace

lsn_status launch_gemm_direct(DirectArgs a, int epi, hipStream_t s) {
  if (a.nf4) {
    const Nf4Table &tab = nf4_table();
    for (int i = 0; i < 16; ++i) a.nf4_q[i] = tab.q[i];
    if (a.nkseg > 0 || a.ksplit > 1 || a.b_red_major || a.K % DBK)
      return fail(LSN_E_ARG, "gemm_direct: NF4 W needs a plain forward product with K %% 64 == 0");
  }
  int64_t t0 = 0;
  for (int q = 0; q < a.nseg; ++q) {
    a.seg[q].ntile0 = t0;
    t0 += seg_ntiles(a.seg[q].N, epi);
  }
  // the glue epilogues: SwiGLU on one plain forward segment, its backward on one segment
  if ((epi == EPI_SWIGLU || epi == EPI_SWIGLU_BWD) && (a.nseg != 1 || a.nkseg > 0 || a.ksplit > 1))
    return fail(LSN_E_ARG, "gemm_direct: the SwiGLU epilogues take one plain segment");
  if (epi == EPI_SWIGLU && a.b_red_major)
    return fail(LSN_E_ARG, "gemm_direct: the SwiGLU forward epilogue needs W as [N][K]");
  if (a.nkseg > 0) {
    int64_t step = 0;
    for (int p = 0; p < a.nkseg; ++p) {
      a.kseg[p].step0 = (int)step;
      step += a.kseg[p].K / DBK;
    }
    a.K = step * DBK;
    return a.b_red_major ? launch_direct_epi<true, true>(a, epi, s) : launch_direct_epi<true, false>(a, epi, s);
  }
  if (a.ksplit > 1) {
    // split-K: fp32 partials of a reduction-major product (the caller adds them)
    if (!a.b_red_major || epi != EPI_F32_SET || a.nseg != 1 || a.adapters || a.ksplit > a.K / DBK)
      return LSN_E_ARG;
    return launch_direct_one<EPI_F32_SET, false, true, true>(a, s);
  }
  return a.b_red_major ? launch_direct_epi<false, true>(a, epi, s) : launch_direct_epi<false, false>(a, epi, s);
}

namespace {
// out[i] = bf16(partial[0][i] + partial[1][i] + ... ), four elements per thread, fixed order
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ partial, int S, int64_t n,
                                                       uint16_t *__restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  floatx4_t acc = __builtin_nontemporal_load(reinterpret_cast<const floatx4_t *>(partial + i));
  for (int sp = 1; sp < S; ++sp) {
    const floatx4_t v = __builtin_nontemporal_load(reinterpret_cast<const floatx4_t *>(partial + sp * n + i));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __fadd_rn(acc[e], v[e]);
  }
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  *reinterpret_cast<u32x2_t *>(out + i) = o;
}
}  // namespace

namespace {
__global__ __launch_bounds__(256) void k_fill_zero(u32x4_t *p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = u32x4_t{0, 0, 0, 0};
}
}  // namespace

lsn_status launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
  if (bytes % 16) return LSN_E_ARG;
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return LSN_OK;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, static_cast<u32x4_t *>(p), n16);
  return check_hip(hipGetLastError(), "k_fill_zero launch");
}

lsn_status launch_splitk_reduce(const float *partial, int S, int64_t n, uint16_t *out, hipStream_t s) {
  if (S < 1 || n < 1 || n % 4) return LSN_E_ARG;
  const int64_t blocks = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, s, partial, S, n, out);
  return check_hip(hipGetLastError(), "k_splitk_reduce launch");
}

lsn_status launch_gemm(int layout, int wkind, int epi, GemmArgs a, hipStream_t s) {
  const Nf4Table &tab = nf4_table();
  for (int i = 0; i < 16; ++i) a.q[i] = tab.q[i];
  if (layout == GEMM_NT) {
    if (wkind == W_IS_NF4)
      return a.res ? launch_one<GEMM_NT, W_IS_NF4, EPI_BF16_RES>(a, s) : launch_one<GEMM_NT, W_IS_NF4, EPI_BF16>(a, s);
    return launch_one<GEMM_NT, W_IS_BF16, EPI_BF16>(a, s);
  }
  if (epi == EPI_SWIGLU_BWD)
    return wkind == W_IS_NF4 ? launch_one<GEMM_NN, W_IS_NF4, EPI_SWIGLU_BWD>(a, s)
                             : launch_one<GEMM_NN, W_IS_BF16, EPI_SWIGLU_BWD>(a, s);
  if (wkind == W_IS_NF4)
    return epi == EPI_BF16 ? launch_one<GEMM_NN, W_IS_NF4, EPI_BF16>(a, s) : launch_one<GEMM_NN, W_IS_NF4, EPI_F32_ADD>(a, s);
  return epi == EPI_BF16 ? launch_one<GEMM_NN, W_IS_BF16, EPI_BF16>(a, s) : launch_one<GEMM_NN, W_IS_BF16, EPI_F32_ADD>(a, s);
}

}  // namespace lsn
