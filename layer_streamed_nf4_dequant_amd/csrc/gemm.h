// Internal interface of the fused GEMM kernels (gemm.hip) and the skinny LoRA kernels
// (lora_small.hip).
#pragma once

#include "common.h"

namespace lsn {

enum { GEMM_NT = 0, GEMM_NN = 1 };        // forward Y = act W^T ; backward dX = act W
enum { W_IS_NF4 = 0, W_IS_BF16 = 1 };
// output epilogues: bf16 store, fp32 add into, fp32 store; and the decoder glue on a bf16 result
// (see EpiOps): the SwiGLU forward on a gate/up pair, its backward, the residual add and the
// rotary embedding (the launchers pick the last two from EPI_BF16 when a segment asks for them,
// so the plain bf16 kernel carries none of their code)
enum { EPI_BF16 = 0, EPI_F32_ADD = 1, EPI_F32_SET = 2, EPI_SWIGLU = 3, EPI_SWIGLU_BWD = 4, EPI_BF16_RES = 5,
       EPI_BF16_ROPE = 6 };

// Operands of the decoder-glue epilogues (bf16 outputs only). Every one of them applies to the
// rounded bf16 product exactly what the standalone glue kernel would apply to the stored product,
// with the same arithmetic (glue_math.h), so fused and unfused results have the same bits.
struct EpiOps {
  // rotary embedding of the rounded output, on segments flagged `rope` (columns = whole heads)
  const float *rope_cs;        // (cos, sin) table [n_pos][rope_dim / 2], 16-byte aligned
  const int32_t *positions;    // [M]: table row of each output row (clamped to [0, n_pos))
  int n_pos, rope_dim;         // rope_dim 64 or 128
  // EPI_SWIGLU: the one segment is the gate member of a gate/up pair sharing the activation; a
  // tile computes 128 gate and the same 128 up columns; out (gate) and out2 (up) may be null
  const uint16_t *w2, *lr_w2, *lr_act2;   // the up member's W [N][K], B [N][r], U [M][r]
  uint16_t *out2;              // up [M][N] or null
  uint16_t *mout;              // bf16( silu(gate) up ) [M][N]
  // EPI_SWIGLU_BWD: the product is dm (the gradient of the SwiGLU output, rounded to bf16, not
  // stored); the epilogue stores the gradients of its inputs
  const uint16_t *gate, *up;   // [M][N]
  uint16_t *dgate, *dup;       // [M][N]
};

struct GemmArgs {
  int64_t M;            // rows of act and out (tokens)
  int64_t Nout;         // columns of out
  int64_t Kred;         // reduction length (columns of act)
  const uint16_t *act;  // bf16 [M][Kred]: X (forward) or dY (backward)
  // frozen base W: forward [Nout][Kred], backward [Kred][Nout]; ldw = elements per W row
  int64_t ldw;
  const uint16_t *w16;  // bf16 W
  const uint8_t *codes; // NF4 W
  const int8_t *qabsmax;
  const float *absmax2;
  float mean;
  float q[16];          // NF4 levels (filled by launch_gemm)
  // LoRA term: forward s * U B^T (lr_act = U [M][r], lr_w = B [Nout][r]);
  //            backward s * G A  (lr_act = G [M][r], lr_w = A [r][Nout])
  const uint16_t *lr_act;
  const uint16_t *lr_w;
  int r;
  float scale;
  int adapters;
  void *out;            // bf16 or fp32 [M][Nout]
  const uint16_t *res;  // EPI_BF16: null, or bf16 [M][Nout] added to the rounded product
  EpiOps x;             // EPI_SWIGLU_BWD operands (the rotary and SwiGLU-forward ones are unused)
};

lsn_status launch_gemm(int layout, int wkind, int epi, GemmArgs a, hipStream_t s);

// direct-load NT GEMM on bf16 W: out_seg = bf16/f32+= ( act W_seg^T + s U_seg B_seg^T ) for up to
// kMaxSegs segments sharing act [M][K] (K % 32 == 0)
constexpr int kMaxSegs = 8;
struct GemmSeg {
  int64_t ntile0;          // first N tile of the segment (filled by launch_gemm_direct)
  int64_t N;
  const uint16_t *w;       // bf16 W [N][K] (reduction-major B: [K][N])
  const uint16_t *lr_w;    // LoRA B [N][r]
  const uint16_t *lr_act;  // U [M][r]
  void *out;               // [M][N]
  const uint16_t *res;     // EPI_BF16: null, or bf16 [M][N] added to the rounded product
  int rope;                // EPI_BF16: rotary embedding of the rounded product (DirectArgs x)
  // NF4 W (DirectArgs nf4 != 0; w unused): the packed weight [N][K] of the segment
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *absmax2;
  float mean;
};
// reduction segments: out = sum_p ( act_p W_p^T + s lr_act_p lr_w_p^T ), one output, the K-steps
// of the segments run back to back (each K_p % 64 == 0)
struct KSeg {
  const uint16_t *act;     // [M][K_p]
  const uint16_t *w;       // [N][K_p] (reduction-major B: [K_p][N])
  int64_t K;
  const uint16_t *lr_act;  // [M][r]
  const uint16_t *lr_w;    // [N][r]
  int step0;               // first K-step of the segment (filled by launch_gemm_direct)
};
struct DirectArgs {
  int64_t M, K;            // K: total reduction length (the sum of the K_p in reduction-segment mode)
  const uint16_t *act;
  int nseg;
  GemmSeg seg[kMaxSegs];
  int nkseg;               // > 0: reduction-segment mode (nseg must be 1; act, seg[0].w/lr_* unused)
  KSeg kseg[kMaxSegs];
  int r;
  float scale;
  int adapters;
  int b_red_major;       // B operand stored [K][N] (N contiguous) instead of [N][K]
  int ksplit;            // > 1: split-K into fp32 partials out + s M N (reduction-major B, fp32 store)
  EpiOps x;
  int nf4;               // W of every segment is NF4 (GemmSeg codes ..), decoded into LDS per K-step
  float nf4_q[16];       // the NF4 levels (filled by launch_gemm_direct)
};
lsn_status launch_gemm_direct(DirectArgs a, int epi, hipStream_t s);
// zero bytes (a multiple of 16) at p, with a kernel (no memset node in captured graphs)
lsn_status launch_fill_zero(void *p, size_t bytes, hipStream_t s);
// out[i] = bf16( sum_{s < S} partial[s][i] ), in split order, for i < n (n % 4 == 0)
lsn_status launch_splitk_reduce(const float *partial, int S, int64_t n, uint16_t *out, hipStream_t s);

// up to 8 low-rank row projections sharing one activation: out_g = bf16(act P_g^T)
struct RowProjSet {
  int n;                  // number of matrices
  int total;              // sum of ranks (<= 128)
  const uint16_t *P[8];   // P_g [r_g][K]
  uint16_t *out[8];       // out_g [M][r_g]
  int r[8];
  int start[8];           // first concatenated column of matrix g
};
lsn_status launch_rowproj(const uint16_t *act, int64_t M, int64_t K, const RowProjSet &set, hipStream_t s);
// up to 8 row-projection jobs with activations of their own, one launch (all jobs: the same M and
// the same number of 16-column blocks)
struct RowProjJob {
  const uint16_t *act;    // [M][K]
  int64_t K;
  RowProjSet set;
};
struct RowProjJobs {
  int n;
  RowProjJob job[8];
};
lsn_status launch_rowproj_jobs(int64_t M, const RowProjJobs &jobs, hipStream_t s);
// out[m][j] = bf16( sum_k act[m][k] * P[j][k] ), j < r   (U = X A^T, or G = dY B with P = B^T)
lsn_status launch_rowproj(const uint16_t *act, int64_t M, int64_t K, const uint16_t *P, int r,
                          uint16_t *out, hipStream_t s);
// up to kMaxTransposes small transposes in one launch, dst_g [cols][rows] = src_g [rows][cols]^T
// (LoRA factors: B -> B^T, A -> A^T; first[] filled by the launcher)
constexpr int kMaxTransposes = 16;
struct TransposeSet {
  int n;
  const uint16_t *src[kMaxTransposes];
  uint16_t *dst[kMaxTransposes];
  int64_t rows[kMaxTransposes], cols[kMaxTransposes], first[kMaxTransposes];
};
lsn_status launch_transpose_many(TransposeSet set, hipStream_t s);
// partial[c][p][j] = sum over t in chunk c of Z[t][p] * V[t][j]   (chunks of TN_CHUNK rows)
constexpr int TN_CHUNK = 256;
lsn_status launch_tn_partial(const uint16_t *Z, int64_t T, int64_t P, const uint16_t *V, int r,
                             float *partial, hipStream_t s);
// out = s * sum_c partial[c] (fixed order), set or accumulate; transposed: out[j][p], else out[p][j]
lsn_status launch_tn_reduce(const float *partial, int64_t n_chunks, int64_t P, int r, float scale,
                            int accumulate, int transposed, float *out, hipStream_t s);
// several split-T partial products (all with the same T), then several reductions, one launch
// each; every job computes exactly what the single-job launch computes
constexpr int kMaxTn = 2 * kMaxSegs;
struct TnJob {
  const uint16_t *Z;      // [T][P]
  int64_t P;
  const uint16_t *V;      // [T][r]
  int r;
  float *partial;         // [T / TN_CHUNK][P][r]
  int64_t wg0;            // first workgroup (filled by the launcher)
};
struct TnJobs {
  int n;
  TnJob job[kMaxTn];
};
lsn_status launch_tn_partial_jobs(int64_t T, TnJobs jobs, hipStream_t s);
struct TnRedJob {
  const float *partial;
  int64_t P;
  int r;
  float scale;
  int accumulate, transposed;
  float *out;
  int64_t i0;             // first element of the flattened index space (filled by the launcher)
};
struct TnRedJobs {
  int n;
  TnRedJob job[kMaxTn];
};
lsn_status launch_tn_reduce_jobs(int64_t n_chunks, TnRedJobs jobs, hipStream_t s);

}  // namespace lsn
