/*
 * lsnf4.h - C ABI of liblsnf4.so: exact layer-streamed NF4 LoRA on MI355X (gfx950).
 *
 * The library computes, for one adapted projection of a decoder layer, the per-visit NF4
 * dequantisation of the frozen base, the frozen-base linear and the rank-r LoRA adapter,
 * forward and backward, and streams decoder layers through a small pool of device slots
 * filled from pinned host memory on a separate stream.
 *
 * Sources (the pages this library implements):
 *  - "Exact Layer Streaming: LoRA Fine-Tuning of an 8B Model on a 4 GB Laptop GPU",
 *    Abstract: layer streaming holds a small pool of decoder layers in GPU memory and fetches
 *    the rest from host RAM on demand; the streamed run must be bit-identical to a resident
 *    run of the same numerics; per-layer NF4 dequantisation is the largest streaming-specific
 *    cost.
 *  - "Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript @1:25-1:58
 *    (frozen base plus a thin pair of trainable matrices), @2:19-2:29 (NF4 and the second
 *    quantisation pass over the block constants), @7:11-7:32 (one layer at a time is copied
 *    into a small on-card buffer on a separate stream while the previous layer computes;
 *    every layer crosses the host link two times in a step: forward and backward recompute).
 *  - "An 8B Fine-Tune Now Fits in 4 GB of VRAM": layers stream through pre-allocated device
 *    buffers; only the adapters and their gradients stay resident.
 *  - Soup v0.73.0 benchmarks README, reading conventions: the fit decision refuses instead
 *    of warning; forward and backward exactness are separate claims.
 *
 * Conventions for every entry point
 *  - Status: every call returns lsn_status. On a non-OK status, lsn_last_error() returns a
 *    thread-local message. Validation is synchronous; no exception crosses the ABI.
 *  - Memory: the caller allocates every device buffer (weights, slots, activations,
 *    outputs, workspaces) and keeps ownership. The library allocates only its pool object
 *    (host struct and HIP events) and, in audit mode, a small device array of checksums.
 *    Hot-path calls (nf4_dequant, lora_linear_*, layer_pool_prefetch/acquire/release)
 *    neither allocate nor synchronise: they enqueue work on the given stream and return.
 *  - Pointers marked "device" must be device memory of the current HIP device; "host" ones
 *    host memory. Streams are hipStream_t passed as void* (NULL = the null stream).
 *  - bf16 tensors are passed as uint16_t bit patterns; all matrices are dense row-major.
 *  - No output may overlap any input of the same call (LSN_E_ARG).
 *  - Determinism: results depend only on shapes and input bytes, never on addresses,
 *    streams, pool slots or timing. No floating-point atomics are used.
 *  - Asynchronous device faults surface at the caller's next synchronisation; the next
 *    library call then returns LSN_E_HIP.
 *  - The library runs only on gfx950; on any other device calls return LSN_E_STATE.
 */
#ifndef LSNF4_H
#define LSNF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LSN_OK = 0,
  LSN_E_ARG = 1,    /* invalid argument: null pointer, bad shape, overlap, non-finite input */
  LSN_E_NOFIT = 2,  /* does not fit: refused rather than spilled (pool slots, device memory) */
  LSN_E_STATE = 3,  /* call not valid in the current state (pool misuse, wrong device) */
  LSN_E_HIP = 4,    /* the HIP runtime reported an error */
  LSN_E_AUDIT = 5   /* the pool's aliasing audit found a mismatch */
} lsn_status;

/* Thread-local text of the last non-OK status returned on this thread ("" if none). */
const char *lsn_last_error(void);

/* ABI version of this header (incremented on any incompatible change). */
#define LSN_ABI_VERSION 1
int32_t lsn_abi_version(void);

/*
 * The NF4 codebook the kernels use, computed by the library on the host: 16 ascending levels
 * (levels[0] = -1, levels[7] = 0, levels[15] = +1) at standard-normal quantiles of evenly
 * spaced probabilities between P = ((1 - 1/30) + (1 - 1/32)) / 2 and 1/2, normalised by the
 * quantile at P, rounded to fp32; midpoints[i] = fl32((levels[i] + levels[i+1]) / 2).
 * ("Can You Fine-Tune a 27B Model on a Laptop?", transcript @2:19: levels placed where
 * normally distributed weights fall; construction of QLoRA, arXiv 2305.14314.)
 * Host-only; needs no GPU. Either pointer may be NULL.
 */
void lsn_nf4_codebook(float levels[16], float midpoints[15]);

/* ------------------------------------------------------------------------------------------
 * NF4 weight storage (transcript @2:19-2:29: 4-bit codes plus per-block constants, and a
 * second quantisation pass over those constants).
 *
 * W[rows][cols] (rows = output features N, cols = input features K), n = rows*cols,
 * blocks of 64 consecutive row-major elements, groups of 256 consecutive blocks:
 *   codes    u8[n/2]      byte j = code[2j] << 4 | code[2j+1]          (device)
 *   qabsmax  i8[n/64]     int8 code v_b in [-127, 127] of block b      (device)
 *   absmax2  f32[n/16384] fp32 scale s2_g of group g                   (device)
 *   mean     f32          per-tensor offset mu                          (host value)
 * Decoded block constant:  c'_b = fl32( fl32( fl32(v_b / 127) * s2_g ) + mu )
 * Dequantised weight:      w = fl32( q[code] * c'_b ), then bf16 round-to-nearest-even.
 * Requirements: cols % 64 == 0 and n % 16384 == 0 (LSN_E_ARG otherwise).
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int64_t rows;
  int64_t cols;
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *absmax2;
  float mean;
} lsn_nf4;

enum { LSN_W_NF4 = 0, LSN_W_BF16 = 1, LSN_W_BF16_T = 2 };

/*
 * A frozen base weight W[N][K]: NF4-packed, un-quantised (or already dequantised) bf16, or
 * bf16 in the transposed layout W^T[K][N] (what nf4_dequant writes with LSN_OUT_BF16_T). The
 * transposed layout serves the backward only: there the product dY W reduces over N, which is
 * then the contiguous dimension of both operands; lora_linear_fwd rejects it (LSN_E_ARG).
 * The backward reads a bf16 W[N][K] as it is (the GEMM turns its tiles in LDS), with results
 * bit-identical to the transposed layout's, so one row-major copy serves a whole visit.
 */
typedef struct {
  int32_t kind;           /* LSN_W_NF4, LSN_W_BF16 or LSN_W_BF16_T */
  lsn_nf4 nf4;            /* used when kind == LSN_W_NF4 (rows = N, cols = K) */
  const uint16_t *bf16;   /* LSN_W_BF16: device bf16 W[N][K]; LSN_W_BF16_T: device bf16 W^T[K][N] */
} lsn_weight;

/* Device workspace bytes nf4_pack needs for a rows x cols weight. */
size_t nf4_pack_ws_bytes(int64_t rows, int64_t cols);

/*
 * nf4_pack - quantise fp32 W[rows][cols] (device) into the NF4 storage above.
 * First pass per block b: c_b = max|w| (exact), x = fl32(w / c_b) (x = 0 if c_b = 0),
 * code = number of midpoints m_i with x > m_i (an exact tie takes the lower level).
 * Second pass: mu = fl32(S / n_b) with S the left-to-right fp64 sum of the c_b (computed on
 * the host); d_b = fl32(c_b - mu); s2_g = max|d_b| over the group; y = fl32(d_b / s2_g)
 * (0 if s2_g = 0); v_b = -127 + number of midpoints between consecutive fl32(v/127) that y
 * exceeds.
 * Outputs codes/qabsmax/absmax2 are device buffers; *mean_out is a host float.
 * ws: device, at least nf4_pack_ws_bytes(rows, cols). Non-finite input gives LSN_E_ARG.
 * Set-up time only: SYNCHRONISES the stream (it reads the block constants back).
 */
lsn_status nf4_pack(const float *w, int64_t rows, int64_t cols, uint8_t *codes,
                    int8_t *qabsmax, float *absmax2, float *mean_out, void *ws,
                    size_t ws_bytes, void *stream);

enum { LSN_OUT_BF16 = 0, LSN_OUT_F32 = 1, LSN_OUT_BF16_T = 2 };

/*
 * nf4_dequant - standalone dequantisation of a whole NF4 tensor into a dense device buffer
 * `out` (16-byte aligned) of rows*cols elements: row-major bf16 (LSN_OUT_BF16, the GEMM
 * operand), the row-major fp32 product before rounding (LSN_OUT_F32), or bf16 transposed,
 * out[c][r] = w_hat[r][c] (LSN_OUT_BF16_T, the backward's operand; needs rows % 8 == 0).
 * Bit-exact with the definition above in every layout. `out` must not overlap the NF4 arrays.
 * ("Exact Layer Streaming", Abstract: per-layer NF4 dequantisation.) Async on `stream`.
 */
lsn_status nf4_dequant(const lsn_nf4 *w, void *out, int32_t out_dtype, void *stream);

/*
 * nf4_dequant_batch - nf4_dequant of n (1 <= n <= 8) tensors, all into the same layout, as one
 * launch (a decoder layer's seven projections per visit: "Exact Layer Streaming", Abstract,
 * per-layer dequantisation). w is a host array of n descriptors, out a host array of n device
 * pointers. Bit-identical to n nf4_dequant calls; the same rules per tensor; no output may
 * overlap any input or another output (LSN_E_ARG). Async on `stream`.
 */
lsn_status nf4_dequant_batch(int32_t n, const lsn_nf4 *w, void *const *out, int32_t out_dtype, void *stream);

/* ------------------------------------------------------------------------------------------
 * LoRA linear on a frozen base (transcript @1:25-1:58), rank r, scale s (= alpha / r):
 *   forward   U = bf16(X A^T);  Y = bf16( X W^T + s U B^T )   (fp32 accumulation)
 *             adapters off:     Y = bf16( X W^T )
 *   backward  G = bf16(dY B);   dX = dY W + s G A;  dB = s dY^T U;  dA = s G^T X
 * Shapes: X [T][K], W [N][K] (or W^T [K][N], backward only), A [r][K], B [N][r], Y and dY [T][N], U and G [T][r],
 * dX [T][K], dA [r][K] fp32, dB [N][r] fp32. W is re-dequantised on every call from the
 * bytes the descriptor points at (a pool slot or a resident buffer): nothing is cached.
 * Requirements: T >= 1, K % 64 == 0, N % 64 == 0, r in {8, 16, 24, 32}, and the NF4 rules for W.
 * The scale enters the GEMMs' LoRA terms on the bf16 operand, as (bf16(s U)) B^T and
 * (bf16(s G)) A: exact, i.e. s (U B^T) and s (G A) with their fp32 sums' rounding, when s is a
 * power of two (alpha and r powers of two, as in every configuration here); another s rounds
 * s u to bf16 once per element. dA and dB scale their fp32 sums.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int64_t T, K, N, r;
  float scale;
  lsn_weight W;
  const uint16_t *A;   /* device bf16 [r][K] */
  const uint16_t *B;   /* device bf16 [N][r] */
} lsn_lora_linear;

/* Device workspace bytes lora_linear_fwd / lora_linear_bwd need for these shapes. */
size_t lora_linear_ws_bytes(int64_t T, int64_t K, int64_t N, int64_t r);

enum { LSN_ADAPTERS_OFF = 0, LSN_ADAPTERS_ON = 1, LSN_ADAPTERS_U_READY = 2 };

/*
 * lora_down - the adapters' down-projections of up to 8 linears that share one input X [T][K]
 * (device bf16): U_g = bf16(X A_g^T) for g < n, with A_g device bf16 [r_g][K] and U_g device
 * bf16 [T][r_g]; r_g in {8, 16, 24, 32}, sum of r_g <= 128, K % 64 == 0. X is read once for all
 * of them (in a decoder layer, q, k, v, gate and up all read the same input). A, r and U are
 * host arrays of n entries. Async on `stream`.
 */
lsn_status lora_down(int64_t T, int64_t K, const uint16_t *X, int32_t n, const uint16_t *const *A,
                     const int32_t *r, uint16_t *const *U, void *stream);

/*
 * lora_linear_fwd - Y = bf16(X W^T + s U B^T).
 *   adapters == LSN_ADAPTERS_ON:      computes U = bf16(X A^T) into U (device [T][r]) first;
 *   adapters == LSN_ADAPTERS_U_READY: U already holds bf16(X A^T) (from lora_down): one GEMM;
 *   adapters == LSN_ADAPTERS_OFF:     the adapter is skipped and Y = bf16(X W^T), bit-identical
 *                                     to the adapters-on result with B = 0; U is ignored.
 * An NF4 W is decoded tile by tile inside the GEMM (never to HBM), bit for bit the bf16 operand
 * nf4_dequant writes, so the result equals the forward on that dequantised W.
 * ws: device, at least lora_linear_ws_bytes(T, K, N, r) (may be NULL for the forward).
 * Async on `stream`.
 */
lsn_status lora_linear_fwd(const lsn_lora_linear *L, int32_t adapters, const uint16_t *X,
                           uint16_t *Y, uint16_t *U, void *ws, size_t ws_bytes, void *stream);

/*
 * lora_linear_fwd_group - the forwards of n (1 <= n <= 8) linears that read the same input
 * X [T][K] (in a decoder layer q, k, v, gate and up all read the attention input; transcript
 * @1:25-1:58 puts an adapter on each): Y_g = bf16(X W_g^T + s U_g B_g^T) for g < n, bit-identical
 * to n calls of lora_linear_fwd. L is an array of n descriptors that share T, K, r and the scale
 * (their N and weights differ); Y and U are host arrays of n device pointers (U ignored with
 * adapters off). With bf16 weights, or with NF4 weights whose codes are 16-byte and whose constant
 * arrays are 4-byte aligned (each K-step's blocks then decoded into the GEMM's LDS stage), the n
 * products run as one GEMM launch over the concatenated output columns (fewer, fuller waves of
 * tiles); with a mix, or other NF4 alignments, each runs on its own. Output/input overlaps give
 * LSN_E_ARG. Async on `stream`.
 */
lsn_status lora_linear_fwd_group(int32_t n, const lsn_lora_linear *L, int32_t adapters, const uint16_t *X,
                                 uint16_t *const *Y, uint16_t *const *U, void *ws, size_t ws_bytes,
                                 void *stream);

enum { LSN_DX_BF16_SET = 0, LSN_DX_F32_ADD = 1, LSN_DX_F32_SET = 2 };
enum { LSN_GRAD_SET = 0, LSN_GRAD_ADD = 1 };

/*
 * lora_linear_bwd - given X, dY and U = bf16(X A^T) from the (recomputed) forward:
 *   dX: LSN_DX_BF16_SET writes bf16(dY W + s G A) to a bf16 [T][K] buffer;
 *       LSN_DX_F32_SET writes fp32 (dY W + s G A) to an fp32 [T][K] buffer;
 *       LSN_DX_F32_ADD adds fp32 (dY W + s G A) into an fp32 [T][K] buffer (for inputs shared
 *       by several projections; the sum order is the caller's call order).
 *   dA, dB (fp32): LSN_GRAD_SET overwrites, LSN_GRAD_ADD accumulates. The reductions over T
 *       run as fixed-order partial sums in `ws`; no atomics, so results are deterministic.
 * ws: device, at least lora_linear_ws_bytes(T, K, N, r). Async on `stream`.
 */
lsn_status lora_linear_bwd(const lsn_lora_linear *L, const uint16_t *X, const uint16_t *dY,
                           const uint16_t *U, void *dX, int32_t dx_mode, float *dA, float *dB,
                           int32_t grad_mode, void *ws, size_t ws_bytes, void *stream);

/*
 * lora_linear_bwd_noalloc - lora_linear_bwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, modes, kernels and results (bit-identical to
 * lora_linear_bwd) as above; the workspace is the library's own static device array of
 * lora_linear_bwd_noalloc_max_ws_bytes() bytes (32 MiB), one per GPU, created with the
 * library's code object on each device it runs on and held until the process ends. Shapes whose
 * lora_linear_ws_bytes exceeds it give LSN_E_ARG. Calls no allocator. Every call on a GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (on different streams, or from
 * different threads) race on it; calls in one stream order are safe. Async on `stream`.
 */
lsn_status lora_linear_bwd_noalloc(const lsn_lora_linear *L, const uint16_t *X, const uint16_t *dY,
                                   const uint16_t *U, void *dX, int32_t dx_mode, float *dA, float *dB,
                                   int32_t grad_mode, void *stream);
/* The size of lora_linear_bwd_noalloc's static workspace, in bytes. */
size_t lora_linear_bwd_noalloc_max_ws_bytes(void);

/* Device workspace bytes lora_linear_bwd_group needs for these n linears. */
size_t lora_linear_group_ws_bytes(int32_t n, const lsn_lora_linear *L);

/*
 * lora_linear_bwd_group - the backwards of n (1 <= n <= 8) linears that read the same input X
 * [T][K] (a decoder layer's q, k, v, gate and up), whose input gradients add up in one dX:
 *   dX:  LSN_DX_BF16_SET writes bf16( sum_g (dY_g W_g + s G_g A_g) );
 *        LSN_DX_F32_ADD adds the fp32 sum into dX; LSN_DX_F32_SET writes it (fp32);
 *   dA_g, dB_g as lora_linear_bwd (LSN_GRAD_SET / LSN_GRAD_ADD), bit-identical to it.
 * L: host array of n descriptors sharing T, K, r and the scale; dY, U, dA, dB: host arrays of
 * n device pointers. With every W in bf16, all in the same layout (LSN_W_BF16 or
 * LSN_W_BF16_T), the n dX products run as one GEMM whose reduction walks the members' N in
 * turn (one fp32 accumulator, member order; the two layouts give identical bits); otherwise the
 * members run one after another (fp32 dX only when n > 1).
 * ws: device, at least lora_linear_group_ws_bytes(n, L). Overlaps give LSN_E_ARG. Async.
 */
lsn_status lora_linear_bwd_group(int32_t n, const lsn_lora_linear *L, const uint16_t *X,
                                 const uint16_t *const *dY, const uint16_t *const *U, void *dX,
                                 int32_t dx_mode, float *const *dA, float *const *dB, int32_t grad_mode,
                                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------------------------
 * Projections with the decoder-layer glue in their GEMM's epilogue. Each result is bit-identical
 * to the projection entry point followed by the glue entry point named (the same fp32 arithmetic
 * on the same rounded bf16 product), and costs no separate pass over HBM: the epilogue applies
 * the glue to the output tile it has just computed. Used in every forward and recomputed
 * forward of a decoder layer ("Exact Layer Streaming", Abstract: the recompute is part of the
 * step). All pointers are device pointers unless said otherwise; overlaps give LSN_E_ARG.
 * ---------------------------------------------------------------------------------------- */

/* The rotary embedding a fused epilogue applies: a table written by rope_table (below). */
typedef struct {
  const float *cs;           /* table from rope_table (device, 16-byte aligned) */
  int32_t n_pos;             /* its rows */
  int32_t head_dim;          /* its head width: 64 or 128 */
  const int32_t *positions;  /* device int32 [T]: the position (table row) of each token row;
                                values outside [0, n_pos) are clamped into it (a wrong rotation,
                                never an out-of-bounds read) */
} lsn_rope;

/*
 * lora_linear_fwd_group_epi - lora_linear_fwd_group with, per member g:
 *   residual != NULL and residual[g] != NULL: Y_g = bf16( residual[g] + P_g ), P_g the plain
 *     output bf16(X W_g^T + s U_g B_g^T): add_bf16(P_g, residual[g]) (the residual stream's
 *     addition after the o and down projections). Y_g may be residual[g] itself.
 *   bit g of rope_mask: Y_g = rope_apply(P_g) with the table, head width and positions of *rope
 *     (q and k); N_g a multiple of rope->head_dim. Not together with a residual.
 * residual: NULL or a host array of n device pointers (entries may be NULL); rope: host pointer,
 * may be NULL when rope_mask is 0. NF4 members run as lora_linear_fwd (the residual added in its
 * epilogue, the rotation by a table-driven pass after it). Async on `stream`.
 */
lsn_status lora_linear_fwd_group_epi(int32_t n, const lsn_lora_linear *L, int32_t adapters, const uint16_t *X,
                                     uint16_t *const *Y, uint16_t *const *U, const uint16_t *const *residual,
                                     uint32_t rope_mask, const lsn_rope *rope, void *ws, size_t ws_bytes,
                                     void *stream);

/*
 * lora_linear_fwd_swiglu - the gate and up projections of a gated MLP and the SwiGLU between
 * them, for descriptors Lg and Lu sharing T, K, N, r and the scale:
 *   gate = bf16(X Wg^T + s Ug Bg^T), up = bf16(X Wu^T + s Uu Bu^T), M = swiglu_fwd(gate, up).
 * Adapters as lora_linear_fwd (Ug, Uu device [T][r]). gate and up (device [T][N]) may be NULL
 * when both weights are bf16: then they are not stored (a forward whose backward recomputes
 * them). With bf16 weights one GEMM launch computes 128 gate and the same 128 up columns per
 * tile and the SwiGLU in its epilogue; with NF4 weights gate and up are required and the call
 * runs lora_linear_fwd_group, then swiglu_fwd. N a multiple of 8. Async on `stream`.
 */
lsn_status lora_linear_fwd_swiglu(const lsn_lora_linear *Lg, const lsn_lora_linear *Lu, int32_t adapters,
                                  const uint16_t *X, uint16_t *gate, uint16_t *up, uint16_t *M, uint16_t *Ug,
                                  uint16_t *Uu, void *ws, size_t ws_bytes, void *stream);

/*
 * lora_linear_bwd_swiglu - lora_linear_bwd of the down projection (input X = M, the SwiGLU's
 * output) followed by swiglu_bwd: dM = bf16(dY W + s G A) is not stored; the epilogue writes
 * dgate = bf16( dM up sigma(gate) (1 + gate (1 - sigma(gate))) ) and dup = bf16( dM silu(gate) )
 * (gate, up, dgate, dup: device bf16 [T][K]). dA, dB and grad_mode, ws as lora_linear_bwd.
 * Bit-identical to lora_linear_bwd (LSN_DX_BF16_SET) then swiglu_bwd. Async on `stream`.
 */
lsn_status lora_linear_bwd_swiglu(const lsn_lora_linear *L, const uint16_t *X, const uint16_t *dY,
                                  const uint16_t *U, const uint16_t *gate, const uint16_t *up, uint16_t *dgate,
                                  uint16_t *dup, float *dA, float *dB, int32_t grad_mode, void *ws, size_t ws_bytes,
                                  void *stream);

/* ------------------------------------------------------------------------------------------
 * The resident ends of the stack ("Can You Fine-Tune a 27B Model on a Laptop? (I Did the
 * Math)", transcript @7:42-7:55: the embedding table and the output head stay resident and
 * unquantised; "Exact Layer Streaming", Abstract: the cross-entropy logits term, 14 bytes per
 * logit element measured against 6 by first principles).
 * ---------------------------------------------------------------------------------------- */

/* Device workspace bytes lm_head_ce needs: 6 bytes per logit element of one chunk
 * (fp32 logits and bf16 logit gradients of min(chunk_rows, T) rows x V), plus the fp32 partial
 * products of the chunk's hidden-state gradient (up to 8 x chunk_rows x H x 4 bytes). */
size_t lm_head_ce_ws_bytes(int64_t chunk_rows, int64_t H, int64_t V);

/*
 * lm_head_ce - cross-entropy through a frozen LM head W [V][H] (bf16, device) for the final
 * hidden states h [T][H] (bf16, device) and labels [T] (int32, device; a label outside [0, V)
 * marks an ignored row), chunked over rows so that only chunk_rows x V logits exist at a time:
 *   z = h W^T (fp32 accumulate), lse_t = log sum_j exp z_tj,
 *   loss[t] = lse_t - z_t,label_t (fp32, device; 0 for ignored rows),
 *   dh = bf16( (softmax(z) - onehot(label)) * grad_scale ) W, rounded to bf16 (device [T][H];
 *        zero rows for ignored rows). grad_scale is typically 1 / (number of counted rows).
 * Rows are independent, so the results do not depend on chunk_rows. H, V: multiples of 64.
 * ws: device, 256-byte aligned, at least lm_head_ce_ws_bytes(chunk_rows, H, V). Overlaps between
 * outputs and inputs give LSN_E_ARG. Async on `stream`.
 */
lsn_status lm_head_ce(int64_t T, int64_t H, int64_t V, const uint16_t *h, const uint16_t *W,
                      const int32_t *labels, float grad_scale, float *loss, uint16_t *dh,
                      int64_t chunk_rows, void *ws, size_t ws_bytes, void *stream);

/*
 * embedding_gather - X[t] = E[ids[t]] for a frozen embedding table E [V][H] (bf16, device) and
 * ids [T] (int32, device); X [T][H] bf16 (device). An id outside [0, V) gives a zero row and
 * adds 1 to *bad_ids (device int32; may be null). H: a multiple of 8. Async on `stream`.
 */
lsn_status embedding_gather(int64_t T, int64_t H, int64_t V, const int32_t *ids, const uint16_t *E,
                            uint16_t *X, int32_t *bad_ids, void *stream);

/* ------------------------------------------------------------------------------------------
 * Decoder-layer glue around the seven projections. The pages train Llama-3.1 and Qwen2.5
 * decoder layers ("Exact Layer Streaming", Abstract; "An 8B Fine-Tune Now Fits in 4 GB of
 * VRAM": the decoder layer is the streamed unit) but print none of these formulas; these are
 * those models' published layer definitions. fp32 arithmetic on bf16 tensors, every product and
 * sum separately rounded, every row reduction in a fixed order (bitwise reproducible).
 * All pointers are device pointers; bf16 tensors are row-major and 16-byte aligned. Bad sizes,
 * null or misaligned pointers and output/input overlaps give LSN_E_ARG. Async on `stream`.
 * ---------------------------------------------------------------------------------------- */

/*
 * rmsnorm_fwd - y[t] = bf16( x[t] * rstd[t] * gain ), rstd[t] = 1 / sqrt(mean_j x_tj^2 + eps)
 * (RMSNorm with a frozen gain). x, y [T][H] bf16; gain [H] bf16; rstd [T] fp32 (kept for the
 * backward). H: a multiple of 8; eps >= 0.
 */
lsn_status rmsnorm_fwd(int64_t T, int64_t H, const uint16_t *x, const uint16_t *gain, float eps,
                       uint16_t *y, float *rstd, void *stream);

/*
 * rmsnorm_bwd - gradient of rmsnorm_fwd with respect to x (the gain is frozen):
 *   dx[t] = rstd_t (gain dy[t]) - x[t] rstd_t^3 sum_j (gain dy x)_tj / H
 * x [T][H] bf16; gain [H] bf16; rstd [T] fp32 from rmsnorm_fwd; dy [T][H] fp32 (the normalised
 * input's gradient as the projections' fp32 dX modes leave it); dx [T][H] fp32, stored
 * (accumulate = 0) or added to what it holds (accumulate != 0: the residual stream's gradient).
 * dx_bf16 (device, may be NULL): also receives bf16(dx) as stored (round to nearest even), the
 * operand the next projection backward reads, so no separate conversion pass is needed.
 */
lsn_status rmsnorm_bwd(int64_t T, int64_t H, const uint16_t *x, const uint16_t *gain, const float *rstd,
                       const float *dy, float *dx, int32_t accumulate, uint16_t *dx_bf16, void *stream);

/*
 * rope_apply - rotary position embedding, in place, on n_heads heads of width head_dim at the
 * start of each row of x (bf16, row stride ld elements, so q and k of a fused projection output
 * are rotated by two calls on offsets into it). In head h of row t, pair (i, i + head_dim/2)
 * turns by a = positions[t] * theta^(-2i/head_dim) (the frequencies are computed on the host
 * in fp64 and rounded to fp32; the angle is an fp32 product); inverse != 0 turns by -a, which
 * is the backward. positions [T] int32. head_dim even and <= 512.
 */
lsn_status rope_apply(int64_t T, int32_t n_heads, int32_t head_dim, uint16_t *x, int64_t ld,
                      const int32_t *positions, float theta, int32_t inverse, void *stream);

/*
 * swiglu_fwd - m = bf16( silu(g) u ), silu(z) = z / (1 + e^-z), elementwise over n values;
 * the sigmoid from the hardware's base-2 exponential and reciprocal (within (|z| + 4) 2^-24
 * relative; it may come out as 0 for z < -87, where its exact value is below 1e-38)
 * (the gated MLP's gate and up projections in, the down projection's input out).
 * g, u, m: bf16 [n], n a multiple of 8.
 */
lsn_status swiglu_fwd(int64_t n, const uint16_t *g, const uint16_t *u, uint16_t *m, void *stream);

/*
 * swiglu_bwd - dg = bf16( dm u sigma(g) (1 + g (1 - sigma(g))) ), du = bf16( dm silu(g) ),
 * sigma as in swiglu_fwd. g, u, dm, dg, du: bf16 [n], n a multiple of 8.
 */
lsn_status swiglu_bwd(int64_t n, const uint16_t *g, const uint16_t *u, const uint16_t *dm, uint16_t *dg,
                      uint16_t *du, void *stream);

/* add_bf16 - out = bf16(a + b) elementwise over n bf16 values (the residual stream's additions);
 * out may be a or b itself. n a multiple of 8. */
lsn_status add_bf16(int64_t n, const uint16_t *a, const uint16_t *b, uint16_t *out, void *stream);

/* convert_f32_bf16 - out = bf16(in) (round to nearest even); convert_bf16_f32 - out = in
 * (exact). n values, a multiple of 8. Used where an fp32 gradient feeds a bf16 operand and back. */
lsn_status convert_f32_bf16(int64_t n, const float *in, uint16_t *out, void *stream);
lsn_status convert_bf16_f32(int64_t n, const uint16_t *in, float *out, void *stream);

/*
 * rope_table - the cosines and sines every rotation of rope_apply uses, as a table:
 * cs[p][i] = (cos a, sin a), a = fl32(p * f_i), f_i = fl32(theta^(-2i/head_dim)), for
 * p < n_pos, i < head_dim/2, with rope_apply's arithmetic, so a rotation driven by the table has
 * rope_apply's bits. cs: device fp32 [n_pos][head_dim/2][2], 16-byte aligned. head_dim even and
 * <= 512; 1 <= n_pos <= 2^24; theta finite and > 1.
 */
lsn_status rope_table(int32_t n_pos, int32_t head_dim, float theta, float *cs, void *stream);


/*
 * attention_fwd - causal scaled dot-product attention with grouped key/value heads (the
 * attention of the Llama-3.1 and Qwen2.5 layers the pages train; they print no formula):
 * n_seq packed sequences of S rows each (T = n_seq x S rows; sequence b is rows b S .. b S + S - 1);
 * query head h (of n_q) reads key/value head h / (n_q / n_kv). For row i and key rows j <= i of
 * its sequence:
 *   s_ij = scale (q_i . k_j),  lse_i = log sum_j exp s_ij,  o_i = sum_j exp(s_ij - lse_i) v_j.
 * q [T][>= n_q head_dim] (row stride ldq elements), k and v [T][>= n_kv head_dim] (ldk, ldv):
 * head h in columns h head_dim .. ; they may be column ranges of one fused projection output.
 * o (bf16, ldo) like q; lse [T][n_q] fp32 (natural log; kept for the backward). head_dim 64
 * or 128; rows 16-byte aligned (ld a multiple of 8); scale > 0 (1/sqrt(head_dim) for these
 * models). Products on bf16 MFMA with fp32 accumulation; the probabilities enter the value
 * product as bf16. Deterministic (no atomics).
 */
lsn_status attention_fwd(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim,
                         const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk,
                         const uint16_t *v, int64_t ldv, float scale, uint16_t *o, int64_t ldo,
                         float *lse, void *stream);

/* Device workspace bytes attention_bwd needs: T x n_q fp32 (the row dots D_i = dO_i . o_i), and,
 * when a key/value head serves an even number of query heads (its dk, dv then summed from two
 * halves of them in a fixed order), 4 x T x n_kv x head_dim fp32 of partial sums. 0 for invalid
 * arguments (n_kv not dividing n_q). */
size_t attention_bwd_ws_bytes(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim);

/*
 * attention_bwd - gradients of attention_fwd for an upstream gradient dO (bf16, like o):
 *   P_ij = exp(s_ij - lse_i), dv_j = sum_i P_ij dO_i, dS_ij = P_ij (dO_i . v_j - dO_i . o_i),
 *   dq_i = scale sum_j dS_ij k_j, dk_j = scale sum_i dS_ij q_i,
 * with dk and dv of a shared key/value head summed over its query heads (bf16 outputs dq like
 * q, dk and dv like k and v, each with its own row stride; stored, not accumulated). o and lse
 * are attention_fwd's outputs. ws: device, 16-byte aligned, at least attention_bwd_ws_bytes.
 * Deterministic: dk and dv have one writer per row (or two fp32 partial sums over fixed halves of
 * the query heads, added in a fixed order), dq is computed by a separate pass.
 */
lsn_status attention_bwd(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim,
                         const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk,
                         const uint16_t *v, int64_t ldv, const uint16_t *o, int64_t ldo,
                         const float *lse, const uint16_t *dO, int64_t lddo, float scale,
                         uint16_t *dq, int64_t lddq, uint16_t *dk, int64_t lddk, uint16_t *dv,
                         int64_t lddv, void *ws, size_t ws_bytes, void *stream);

/*
 * attention_bwd_rope - attention_bwd for a q and k that the forward received rotated by the rotary
 * embedding (rope_apply, or lora_linear_fwd_group_epi's rotation): dq and dk come out rotated
 * back, i.e. as the gradients of the unrotated projection outputs, bit-identical to attention_bwd
 * followed by rope_apply(inverse) on dq and dk with the same table (rope->head_dim equal to
 * head_dim; rope->positions [n_seq S]). The rotation is applied to each gradient row as it is
 * stored: no extra pass over dq or dk. rope: host pointer. Async on `stream`.
 */
lsn_status attention_bwd_rope(int64_t n_seq, int64_t S, int32_t n_q, int32_t n_kv, int32_t head_dim,
                              const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk,
                              const uint16_t *v, int64_t ldv, const uint16_t *o, int64_t ldo,
                              const float *lse, const uint16_t *dO, int64_t lddo, float scale,
                              uint16_t *dq, int64_t lddq, uint16_t *dk, int64_t lddk, uint16_t *dv,
                              int64_t lddv, void *ws, size_t ws_bytes, const lsn_rope *rope, void *stream);

/* ------------------------------------------------------------------------------------------
 * Layer pool ("Exact Layer Streaming", Abstract; transcript @7:11-7:32; "An 8B Fine-Tune
 * Now Fits in 4 GB of VRAM"): n_slots caller-owned device slots hold decoder-layer images;
 * each layer's image lives in pinned host memory; copies run on the pool's copy stream and
 * are ordered against compute by events:
 *   prefetch(l)  picks a free slot (never one acquired or holding a pending prefetch), makes
 *                the copy stream wait for that slot's release event, copies the image,
 *                records the slot's ready event. If every slot is busy: LSN_E_STATE.
 *   acquire(l)   makes the compute stream wait for the ready event and returns the slot's
 *                device address; a layer not prefetched is prefetched first (a miss).
 *   release(l)   records the slot's release event on the compute stream; the slot may be
 *                refilled only after that event. Releasing a layer not held: LSN_E_STATE.
 * Every visit copies the layer again (two host reads of every layer per step) unless
 * LSN_POOL_KEEP_AT_TURN is set, in which case a layer still in a free slot is reused.
 * Refusal (Soup benchmarks README, reading conventions: a run that does not fit is stopped): the slots are
 * caller memory, so whether n_slots x slot_bytes fits in free device memory is decided (and
 * refused) by the caller before it allocates them; register returns LSN_E_NOFIT for an image
 * larger than slot_bytes. Nothing ever spills to host-mapped memory.
 * Aliasing audit (LSN_POOL_AUDIT; the pages' silent wrong-gradient defect was aliasing): a
 * 64-bit checksum of the slot is taken on the compute stream at every acquire and release
 * and compared with the host image's checksum by layer_pool_audit; released slots are
 * poisoned (0xFF bytes, which decode to NaN) so a stale read cannot go unnoticed.
 * LSN_FAULT_* flags plant deterministic defects for the gate's same-process controls.
 * LSN_POOL_HOST_SIM runs the same state machine on host memory (memcpy, no GPU).
 * File tier (LSN_POOL_FILE_TIER; "Soup v0.73.0 benchmarks README", record index, the disk tier;
 * "An 8B Fine-Tune Now Fits in 4 GB of VRAM": the base stays in host RAM, or on NVMe when RAM is
 * short): the caller then also hands layer_pool_create two pinned bounce buffers of slot_bytes,
 * and the pool starts an I/O thread. Layers registered with layer_pool_register_file are read by that thread
 * (8 reader threads per image) into the bounce buffers, alternately, and copied from there on
 * the copy stream; prefetch() posts the read and returns, and acquire() blocks the calling
 * host thread until the layer's copy has been enqueued. An I/O failure is reported by the
 * acquire that needs it (LSN_E_HIP, with the reason). Planted faults and the audit behave as
 * for host images. With LSN_POOL_FILE_DIRECT as well, the tier reads with O_DIRECT, bypassing
 * the page cache (each fill is a read of the storage device) into the caller's plain staging
 * buffers (lsn_pool_buffers.direct_stage), which the readers copy on to the bounce buffers:
 * slot_bytes and the staging buffers must be 4096-byte aligned, each image's offset too, and
 * the file must hold the image's bytes rounded up to a whole 4096 (the padding is read and not
 * copied to the slot).
 * ---------------------------------------------------------------------------------------- */
typedef struct lsn_pool lsn_pool;

enum {
  LSN_POOL_AUDIT = 1u << 0,
  LSN_POOL_KEEP_AT_TURN = 1u << 1,
  LSN_POOL_HOST_SIM = 1u << 2,
  LSN_POOL_FILE_TIER = 1u << 3,
  LSN_POOL_FILE_DIRECT = 1u << 4,      /* file tier reads bypass the page cache (O_DIRECT) */
  LSN_FAULT_STALE_REFETCH = 1u << 8,   /* a layer's second visit skips its copy (stale slot) */
  LSN_FAULT_WRONG_SLOT = 1u << 9       /* a layer's second visit returns another slot */
};

typedef struct {
  uint64_t copies;          /* host->device copies enqueued */
  uint64_t bytes_copied;
  uint64_t hits;            /* acquires served by KEEP_AT_TURN reuse */
  uint64_t misses;          /* acquires without a prior prefetch */
  uint64_t acquires;
  uint64_t releases;
  uint64_t audit_checks;    /* checksums compared by layer_pool_audit */
  uint64_t audit_failures;
} lsn_pool_stats;

/* Caller-owned memory the pool uses besides its slots (the pool allocates no device or pinned
 * memory; it owns only its host-side state, its events and, with the file tier, its I/O thread):
 *   audit_sums      LSN_POOL_AUDIT: an 8-byte aligned device array (host array under
 *                   LSN_POOL_HOST_SIM) of audit_capacity checksums, not overlapping a slot;
 *                   layer_pool_create and layer_pool_audit zero it; 2 checksums per layer
 *                   visit are recorded between two layer_pool_audit calls, more: LSN_E_STATE.
 *   bounce[0..1]    LSN_POOL_FILE_TIER: two non-overlapping buffers of slot_bytes each, in
 *                   pinned host memory (hipHostMalloc; plain host memory under HOST_SIM).
 *   direct_stage[0..1]  LSN_POOL_FILE_DIRECT: two non-overlapping buffers of slot_bytes each in
 *                   plain (pageable) host memory, 4096-byte aligned: the O_DIRECT reads land
 *                   there (direct I/O cannot target pinned driver memory) and are copied on to
 *                   the bounce buffers by the reader threads.
 * Unused fields may be NULL / 0; the whole struct may be NULL when neither flag is set. The
 * memory must outlive the pool (until layer_pool_destroy returns). */
typedef struct {
  unsigned long long *audit_sums;
  size_t audit_capacity;
  void *bounce[2];
  void *direct_stage[2];
} lsn_pool_buffers;

/* slots: n_slots device pointers of slot_bytes each (caller-owned, 256-byte aligned);
 * n_layers: the layer indices the pool serves are 0 .. n_layers-1 (each registered once
 * before its first prefetch); copy_stream: the stream the copies run on (must differ from the
 * compute streams); bufs: see lsn_pool_buffers. LSN_E_ARG on a missing, misaligned, overlapping
 * or (file tier) unpinned buffer. Synchronises (zeroing the checksum array). */
lsn_status layer_pool_create(int32_t n_slots, size_t slot_bytes, void *const *slots,
                             int32_t n_layers, void *copy_stream, uint32_t flags,
                             const lsn_pool_buffers *bufs, lsn_pool **out);
/* host_image: pinned host memory (hipHostMalloc), bytes <= slot_bytes; not modified after.
 * Registering a layer again replaces its image: refused (LSN_E_STATE) while the layer is
 * prefetched or acquired; a free slot still holding the old bytes is never reused for it. */
lsn_status layer_pool_register(lsn_pool *pool, int32_t layer, const void *host_image,
                               size_t bytes);
/* File tier only: the layer's image is `bytes` at `offset` of the file at `path` (opened
 * read-only and kept open until layer_pool_destroy; the file must not change meanwhile).
 * LSN_E_ARG if it cannot be opened or is too short; LSN_E_NOFIT if bytes > slot_bytes;
 * LSN_E_STATE on a pool without LSN_POOL_FILE_TIER or while the layer is in flight. On any
 * error the layer keeps its previous registration. */
lsn_status layer_pool_register_file(lsn_pool *pool, int32_t layer, const char *path,
                                    uint64_t offset, size_t bytes);
lsn_status layer_pool_prefetch(lsn_pool *pool, int32_t layer);
lsn_status layer_pool_acquire(lsn_pool *pool, int32_t layer, void *compute_stream,
                              const void **dev_image);
lsn_status layer_pool_release(lsn_pool *pool, int32_t layer, void *compute_stream);
lsn_status layer_pool_stats(const lsn_pool *pool, lsn_pool_stats *out);
/* Synchronises; compares every recorded slot checksum with its layer's host checksum.
 * LSN_E_AUDIT (with the first mismatching layer and visit in the message) on any mismatch. */
lsn_status layer_pool_audit(lsn_pool *pool);
/* Finishes the posted reads, waits for in-flight copies, destroys events and closes the files;
 * never frees caller memory (slots, checksum array, bounce buffers). */
lsn_status layer_pool_destroy(lsn_pool *pool);

#ifdef __cplusplus
}
#endif
#endif /* LSNF4_H */
