// C ABI of the LoRA linear on a frozen (NF4 or bf16) base: validation, workspace layout and
// the kernel sequence. Contracts in include/lsnf4.h.
//
// forward:  U = bf16(X A^T)                                  k_rowproj
//           Y = bf16(s U B^T + X W^T)                        k_gemm NT (NF4 dequantised in LDS)
// backward: Bt = B^T (and A^T) ; G = bf16(dY B)             k_transpose_many, k_rowproj
//           dX = s G A + dY W                                k_gemm NN (NF4 or bf16 W[N][K]), or
//                                                            k_gemm_direct NT on W^T[K][N] with A^T
//                                                            (bf16 store or fp32 add)
//           dB = s sum_t dY^T U ; dA = s sum_t G^T X         k_tn_partial + k_tn_reduce

#include <mutex>
#include <utility>

#include "common.h"
#include "gemm.h"

namespace lsn {
lsn_status require_gfx950();
bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb);
lsn_status check_nf4(const lsn_nf4 *w, const char *what);
}  // namespace lsn

using namespace lsn;

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct BwdWs {
  uint16_t *G;
  uint16_t *Bt;
  uint16_t *At;
  float *part_dB;
  float *part_dA;
  size_t bytes;
};

BwdWs bwd_layout(void *ws, int64_t T, int64_t K, int64_t N, int64_t r) {
  const int64_t nc = (T + TN_CHUNK - 1) / TN_CHUNK;
  char *p = static_cast<char *>(ws);
  BwdWs w;
  size_t off = 0;
  w.G = reinterpret_cast<uint16_t *>(p + off);
  off += align256((size_t)(T * r * 2));
  w.Bt = reinterpret_cast<uint16_t *>(p + off);
  off += align256((size_t)(r * N * 2));
  w.At = reinterpret_cast<uint16_t *>(p + off);
  off += align256((size_t)(K * r * 2));
  w.part_dB = reinterpret_cast<float *>(p + off);
  off += align256((size_t)(nc * N * r * 4));
  w.part_dA = reinterpret_cast<float *>(p + off);
  off += align256((size_t)(nc * K * r * 4));
  w.bytes = off;
  return w;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

lsn_status check_linear(const lsn_lora_linear *L, const char *what) {
  if (!L) return fail(LSN_E_ARG, "%s: null linear descriptor", what);
  if (L->T < 1 || L->K < 64 || L->N < 64 || L->K % 64 || L->N % 64)
    return fail(LSN_E_ARG, "%s: need T >= 1 and K, N positive multiples of 64 (got T=%lld K=%lld N=%lld)", what,
                (long long)L->T, (long long)L->K, (long long)L->N);
  if (L->r < 8 || L->r > 32 || L->r % 8)
    return fail(LSN_E_ARG, "%s: rank r must be 8, 16, 24 or 32 (got %lld)", what, (long long)L->r);
  if (L->W.kind == LSN_W_NF4) {
    lsn_status st = check_nf4(&L->W.nf4, what);
    if (st != LSN_OK) return st;
    if (L->W.nf4.rows != L->N || L->W.nf4.cols != L->K)
      return fail(LSN_E_ARG, "%s: NF4 W is %lld x %lld, expected N x K = %lld x %lld", what,
                  (long long)L->W.nf4.rows, (long long)L->W.nf4.cols, (long long)L->N, (long long)L->K);
  } else if (L->W.kind == LSN_W_BF16 || L->W.kind == LSN_W_BF16_T) {
    if (!L->W.bf16 || !aligned16(L->W.bf16)) return fail(LSN_E_ARG, "%s: bf16 W null or not 16-byte aligned", what);
  } else {
    return fail(LSN_E_ARG, "%s: unknown weight kind %d", what, L->W.kind);
  }
  if (!L->A || !L->B || !aligned16(L->A) || !aligned16(L->B))
    return fail(LSN_E_ARG, "%s: A and B must be non-null and 16-byte aligned", what);
  return LSN_OK;
}

// The input byte ranges of a linear's frozen weight (three arrays for NF4, one for bf16).
int w_ranges(const lsn_lora_linear *L, const void **p, size_t *n) {
  if (L->W.kind == LSN_W_NF4) {
    const size_t e = (size_t)(L->N * L->K);
    p[0] = L->W.nf4.codes;   n[0] = e / 2;
    p[1] = L->W.nf4.qabsmax; n[1] = e / 64;
    p[2] = L->W.nf4.absmax2; n[2] = e / 16384 * 4;
    return 3;
  }
  p[0] = L->W.bf16;
  n[0] = (size_t)(L->N * L->K * 2);
  return 1;
}

GemmArgs base_args(const lsn_lora_linear *L) {
  GemmArgs a{};
  a.r = (int)L->r;
  a.scale = L->scale;
  if (L->W.kind == LSN_W_NF4) {
    a.codes = L->W.nf4.codes;
    a.qabsmax = L->W.nf4.qabsmax;
    a.absmax2 = L->W.nf4.absmax2;
    a.mean = L->W.nf4.mean;
  } else {
    a.w16 = L->W.bf16;
  }
  return a;
}

}  // namespace

extern "C" {

lsn_status lora_down(int64_t T, int64_t K, const uint16_t *X, int32_t n, const uint16_t *const *A, const int32_t *r,
                     uint16_t *const *U, void *stream) {
  if (T < 1 || K < 64 || K % 64) return fail(LSN_E_ARG, "lora_down: need T >= 1 and K a positive multiple of 64");
  if (n < 1 || n > 8 || !A || !r || !U) return fail(LSN_E_ARG, "lora_down: need 1 <= n <= 8 and non-null arrays");
  if (!X || !aligned16(X)) return fail(LSN_E_ARG, "lora_down: X null or not 16-byte aligned");
  RowProjSet set{};
  set.n = n;
  int total = 0;
  for (int g = 0; g < n; ++g) {
    if (r[g] < 8 || r[g] > 32 || r[g] % 8) return fail(LSN_E_ARG, "lora_down: rank %d must be 8, 16, 24 or 32", r[g]);
    if (!A[g] || !U[g] || !aligned16(A[g]) || !aligned16(U[g]))
      return fail(LSN_E_ARG, "lora_down: A[%d] / U[%d] null or not 16-byte aligned", g, g);
    set.P[g] = A[g];
    set.out[g] = U[g];
    set.r[g] = r[g];
    set.start[g] = total;
    total += r[g];
  }
  if (total > 128) return fail(LSN_E_ARG, "lora_down: total rank %d exceeds 128", total);
  set.total = total;
  for (int g = 0; g < n; ++g) {
    const size_t ub = (size_t)(T * r[g] * 2);
    if (ranges_overlap(U[g], ub, X, (size_t)(T * K * 2))) return fail(LSN_E_ARG, "lora_down: U overlaps X");
    for (int h = 0; h < n; ++h) {
      if (ranges_overlap(U[g], ub, A[h], (size_t)(r[h] * K * 2)))
        return fail(LSN_E_ARG, "lora_down: U overlaps an A");
      if (h < g && ranges_overlap(U[g], ub, U[h], (size_t)(T * r[h] * 2)))
        return fail(LSN_E_ARG, "lora_down: two outputs overlap");
    }
  }
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  return launch_rowproj(X, T, K, set, (hipStream_t)stream);
}

size_t lora_linear_ws_bytes(int64_t T, int64_t K, int64_t N, int64_t r) {
  if (T < 1 || K < 1 || N < 1 || r < 1) return 0;
  return bwd_layout(nullptr, T, K, N, r).bytes;
}

}  // extern "C"

namespace {

// NF4 W decoded inside the direct-load GEMM: its codes 16-byte and its constant arrays 4-byte
// aligned (the kernel stages them by 16- and 4-byte direct loads)
bool nf4_direct_ok(const lsn_weight &w) {
  return w.kind == LSN_W_NF4 && ((uintptr_t)w.nf4.codes & 15) == 0 && ((uintptr_t)w.nf4.qabsmax & 3) == 0 &&
         ((uintptr_t)w.nf4.absmax2 & 3) == 0;
}

void set_nf4_seg(GemmSeg &g, const lsn_weight &w) {
  g.codes = w.nf4.codes;
  g.qabsmax = w.nf4.qabsmax;
  g.absmax2 = w.nf4.absmax2;
  g.mean = w.nf4.mean;
}

// The forward of one linear; res (may be null): the residual added to the rounded product in the
// epilogue (res == Y allowed, in place).
lsn_status fwd_impl(const char *what, const lsn_lora_linear *L, int32_t adapters, const uint16_t *X, uint16_t *Y,
                    uint16_t *U, const uint16_t *res, hipStream_t s) {
  lsn_status st = check_linear(L, what);
  if (st != LSN_OK) return st;
  if (L->W.kind == LSN_W_BF16_T)
    return fail(LSN_E_ARG, "%s: the transposed bf16 layout is for the backward only", what);
  const int64_t T = L->T, K = L->K, N = L->N, r = L->r;
  if (!X || !Y || !aligned16(X) || !aligned16(Y))
    return fail(LSN_E_ARG, "%s: X and Y must be non-null and 16-byte aligned", what);
  if (adapters != LSN_ADAPTERS_OFF && adapters != LSN_ADAPTERS_ON && adapters != LSN_ADAPTERS_U_READY)
    return fail(LSN_E_ARG, "%s: unknown adapters mode %d", what, adapters);
  if (adapters && (!U || !aligned16(U)))
    return fail(LSN_E_ARG, "%s: U must be non-null and 16-byte aligned when adapters are on", what);
  if (res && !aligned16(res)) return fail(LSN_E_ARG, "%s: residual not 16-byte aligned", what);
  const size_t yb = (size_t)(T * N * 2), ub = (size_t)(T * r * 2);
  const void *ins[6] = {X, L->A, L->B};
  size_t inb[6] = {(size_t)(T * K * 2), (size_t)(r * K * 2), (size_t)(N * r * 2)};
  const int n_in = 3 + w_ranges(L, ins + 3, inb + 3);
  for (int i = 0; i < n_in; ++i) {
    if (ranges_overlap(Y, yb, ins[i], inb[i]) ||
        (adapters == LSN_ADAPTERS_ON && ranges_overlap(U, ub, ins[i], inb[i])))
      return fail(LSN_E_ARG, "%s: an output overlaps an input", what);
  }
  if (adapters && ranges_overlap(Y, yb, U, ub)) return fail(LSN_E_ARG, "%s: Y overlaps U", what);
  if (res && ((res != Y && ranges_overlap(res, yb, Y, yb)) ||
              (adapters == LSN_ADAPTERS_ON && ranges_overlap(res, yb, U, ub))))
    return fail(LSN_E_ARG, "%s: the residual overlaps an output (other than being Y itself)", what);
  if ((st = require_gfx950()) != LSN_OK) return st;
  if (adapters == LSN_ADAPTERS_ON && (st = launch_rowproj(X, T, K, L->A, (int)r, U, s)) != LSN_OK) return st;
  if (L->W.kind == LSN_W_BF16 || nf4_direct_ok(L->W)) {
    DirectArgs d{};
    d.M = T;
    d.K = K;
    d.act = X;
    d.nseg = 1;
    d.seg[0].N = N;
    d.seg[0].w = L->W.bf16;
    if (L->W.kind == LSN_W_NF4) {
      d.nf4 = 1;
      set_nf4_seg(d.seg[0], L->W);
    }
    d.seg[0].lr_w = L->B;
    d.seg[0].lr_act = U;
    d.seg[0].out = Y;
    d.seg[0].res = res;
    d.r = (int)r;
    d.scale = L->scale;
    d.adapters = adapters ? 1 : 0;
    return launch_gemm_direct(d, EPI_BF16, s);
  }
  GemmArgs a = base_args(L);
  a.M = T;
  a.Nout = N;
  a.Kred = K;
  a.act = X;
  a.ldw = K;
  a.lr_act = U;
  a.lr_w = L->B;
  a.adapters = adapters ? 1 : 0;
  a.out = Y;
  a.res = res;
  return launch_gemm(GEMM_NT, W_IS_NF4, EPI_BF16, a, s);
}

bool valid_rope(const lsn_rope *rope) {
  return rope && rope->cs && aligned16(rope->cs) && rope->positions && rope->n_pos >= 1 &&
         (rope->head_dim == 64 || rope->head_dim == 128);
}

// The forwards of n linears sharing X; residual (may be null, entries may be null) and rope_mask
// as lora_linear_fwd_group_epi.
lsn_status fwd_group_impl(const char *what, int32_t n, const lsn_lora_linear *L, int32_t adapters, const uint16_t *X,
                          uint16_t *const *Y, uint16_t *const *U, const uint16_t *const *residual,
                          uint32_t rope_mask, const lsn_rope *rope, void *ws, size_t ws_bytes, hipStream_t s) {
  (void)ws;
  (void)ws_bytes;
  if (n < 1 || n > kMaxSegs || !L || !Y || (adapters && !U))
    return fail(LSN_E_ARG, "%s: need 1 <= n <= %d and non-null arrays", what, kMaxSegs);
  if (rope_mask >> n) return fail(LSN_E_ARG, "%s: rope_mask names members past n", what);
  if (rope_mask && !valid_rope(rope))
    return fail(LSN_E_ARG, "%s: the rotation needs a 16-byte aligned table, positions, n_pos >= 1 and a head width "
                           "of 64 or 128", what);
  bool all_bf16 = true, all_nf4 = true;
  for (int g = 0; g < n; ++g) {
    lsn_status st = check_linear(&L[g], what);
    if (st != LSN_OK) return st;
    if (L[g].T != L[0].T || L[g].K != L[0].K || L[g].r != L[0].r || L[g].scale != L[0].scale)
      return fail(LSN_E_ARG, "%s: members must share T, K, r and the scale", what);
    if (L[g].W.kind == LSN_W_BF16_T)
      return fail(LSN_E_ARG, "%s: the transposed bf16 layout is for the backward only", what);
    all_bf16 = all_bf16 && L[g].W.kind == LSN_W_BF16;
    all_nf4 = all_nf4 && nf4_direct_ok(L[g].W);
    const uint16_t *res = residual ? residual[g] : nullptr;
    if (res && !aligned16(res)) return fail(LSN_E_ARG, "%s: residual[%d] not 16-byte aligned", what, g);
    if ((rope_mask >> g) & 1) {
      if (res) return fail(LSN_E_ARG, "%s: member %d has both a residual and a rotation", what, g);
      if (L[g].N % rope->head_dim)
        return fail(LSN_E_ARG, "%s: member %d's width %lld is not whole heads of %d", what, g, (long long)L[g].N,
                    rope->head_dim);
    }
  }
  if (adapters != LSN_ADAPTERS_OFF && adapters != LSN_ADAPTERS_ON && adapters != LSN_ADAPTERS_U_READY)
    return fail(LSN_E_ARG, "%s: unknown adapters mode %d", what, adapters);
  const int64_t T = L[0].T, K = L[0].K, r = L[0].r;
  if (!X || !aligned16(X)) return fail(LSN_E_ARG, "%s: X null or not 16-byte aligned", what);
  // every output against every input, and the outputs pairwise
  const void *outs[2 * kMaxSegs];
  size_t outb[2 * kMaxSegs];
  int n_out = 0;
  for (int g = 0; g < n; ++g) {
    if (!Y[g] || !aligned16(Y[g])) return fail(LSN_E_ARG, "%s: Y[%d] null or not 16-byte aligned", what, g);
    outs[n_out] = Y[g];
    outb[n_out++] = (size_t)(T * L[g].N * 2);
    if (adapters) {
      if (!U[g] || !aligned16(U[g]))
        return fail(LSN_E_ARG, "%s: U[%d] null or not 16-byte aligned", what, g);
      if (adapters == LSN_ADAPTERS_ON) {
        outs[n_out] = U[g];
        outb[n_out++] = (size_t)(T * r * 2);
      }
    }
  }
  const size_t tab_b = rope_mask ? (size_t)rope->n_pos * rope->head_dim * 4 : 0;
  for (int o = 0; o < n_out; ++o) {
    if (ranges_overlap(outs[o], outb[o], X, (size_t)(T * K * 2)))
      return fail(LSN_E_ARG, "%s: an output overlaps X", what);
    if (rope_mask && (ranges_overlap(outs[o], outb[o], rope->cs, tab_b) ||
                      ranges_overlap(outs[o], outb[o], rope->positions, (size_t)T * 4)))
      return fail(LSN_E_ARG, "%s: an output overlaps the rotation table or the positions", what);
    for (int p = 0; p < o; ++p)
      if (ranges_overlap(outs[o], outb[o], outs[p], outb[p]))
        return fail(LSN_E_ARG, "%s: two outputs overlap", what);
    for (int g = 0; g < n; ++g) {
      const void *ins[5] = {L[g].A, L[g].B};
      size_t inb[5] = {(size_t)(r * K * 2), (size_t)(L[g].N * r * 2)};
      const int n_in = 2 + w_ranges(&L[g], ins + 2, inb + 2);
      for (int i = 0; i < n_in; ++i)
        if (ranges_overlap(outs[o], outb[o], ins[i], inb[i]))
          return fail(LSN_E_ARG, "%s: an output overlaps an input", what);
      // a residual may be its own member's output, nothing else
      const uint16_t *res = residual ? residual[g] : nullptr;
      if (res && outs[o] != (const void *)Y[g] && ranges_overlap(outs[o], outb[o], res, (size_t)(T * L[g].N * 2)))
        return fail(LSN_E_ARG, "%s: residual[%d] overlaps an output other than Y[%d]", what, g, g);
      if (res && outs[o] == (const void *)Y[g] && res != Y[g] && ranges_overlap(Y[g], outb[o], res, outb[o]))
        return fail(LSN_E_ARG, "%s: residual[%d] partially overlaps Y[%d]", what, g, g);
    }
  }
  if (adapters == LSN_ADAPTERS_U_READY)
    for (int g = 0; g < n; ++g)
      for (int h = 0; h < n; ++h)
        if (ranges_overlap(Y[g], (size_t)(T * L[g].N * 2), U[h], (size_t)(T * r * 2)))
          return fail(LSN_E_ARG, "%s: a Y overlaps a U", what);
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  if (adapters == LSN_ADAPTERS_ON) {
    // the down-projections in as few passes over X as the 128-column limit of one pass allows
    for (int g0 = 0; g0 < n;) {
      RowProjSet set{};
      while (g0 < n && set.total + r <= 128) {
        set.P[set.n] = L[g0].A;
        set.out[set.n] = U[g0];
        set.r[set.n] = (int)r;
        set.start[set.n] = set.total;
        set.total += (int)r;
        ++set.n;
        ++g0;
      }
      if ((st = launch_rowproj(X, T, K, set, s)) != LSN_OK) return st;
    }
  }
  const int mode = adapters ? LSN_ADAPTERS_U_READY : LSN_ADAPTERS_OFF;
  if (!all_bf16 && !all_nf4) {
    for (int g = 0; g < n; ++g) {
      if ((st = fwd_impl(what, &L[g], mode, X, Y[g], adapters ? U[g] : nullptr, residual ? residual[g] : nullptr,
                         s)) != LSN_OK)
        return st;
      if ((rope_mask >> g) & 1) {
        st = launch_rope_tab(T, (int)(L[g].N / rope->head_dim), rope->head_dim, Y[g], L[g].N, rope->positions,
                             rope->cs, rope->n_pos, 1.0f, s);
        if (st != LSN_OK) return st;
      }
    }
    return LSN_OK;
  }
  DirectArgs d{};
  d.M = T;
  d.K = K;
  d.act = X;
  d.nseg = n;
  for (int g = 0; g < n; ++g) {
    d.seg[g].N = L[g].N;
    d.seg[g].w = L[g].W.bf16;
    if (all_nf4) set_nf4_seg(d.seg[g], L[g].W);
    d.seg[g].lr_w = L[g].B;
    d.seg[g].lr_act = adapters ? U[g] : nullptr;
    d.seg[g].out = Y[g];
    d.seg[g].res = residual ? residual[g] : nullptr;
    d.seg[g].rope = (int)((rope_mask >> g) & 1);
  }
  if (rope_mask) {
    d.x.rope_cs = rope->cs;
    d.x.positions = rope->positions;
    d.x.n_pos = rope->n_pos;
    d.x.rope_dim = rope->head_dim;
  }
  d.r = (int)r;
  d.scale = L[0].scale;
  d.adapters = adapters ? 1 : 0;
  d.nf4 = all_nf4 ? 1 : 0;
  return launch_gemm_direct(d, EPI_BF16, s);
}

}  // namespace

extern "C" {

lsn_status lora_linear_fwd(const lsn_lora_linear *L, int32_t adapters, const uint16_t *X, uint16_t *Y,
                           uint16_t *U, void *ws, size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  return fwd_impl("lora_linear_fwd", L, adapters, X, Y, U, nullptr, (hipStream_t)stream);
}

lsn_status lora_linear_fwd_group(int32_t n, const lsn_lora_linear *L, int32_t adapters, const uint16_t *X,
                                 uint16_t *const *Y, uint16_t *const *U, void *ws, size_t ws_bytes, void *stream) {
  return fwd_group_impl("lora_linear_fwd_group", n, L, adapters, X, Y, U, nullptr, 0u, nullptr, ws, ws_bytes,
                        (hipStream_t)stream);
}

lsn_status lora_linear_fwd_group_epi(int32_t n, const lsn_lora_linear *L, int32_t adapters, const uint16_t *X,
                                     uint16_t *const *Y, uint16_t *const *U, const uint16_t *const *residual,
                                     uint32_t rope_mask, const lsn_rope *rope, void *ws, size_t ws_bytes,
                                     void *stream) {
  return fwd_group_impl("lora_linear_fwd_group_epi", n, L, adapters, X, Y, U, residual, rope_mask, rope, ws,
                        ws_bytes, (hipStream_t)stream);
}

lsn_status lora_linear_fwd_swiglu(const lsn_lora_linear *Lg, const lsn_lora_linear *Lu, int32_t adapters,
                                  const uint16_t *X, uint16_t *gate, uint16_t *up, uint16_t *M, uint16_t *Ug,
                                  uint16_t *Uu, void *ws, size_t ws_bytes, void *stream) {
  const char *what = "lora_linear_fwd_swiglu";
  lsn_status st;
  if ((st = check_linear(Lg, what)) != LSN_OK || (st = check_linear(Lu, what)) != LSN_OK) return st;
  if (Lg->T != Lu->T || Lg->K != Lu->K || Lg->N != Lu->N || Lg->r != Lu->r || Lg->scale != Lu->scale)
    return fail(LSN_E_ARG, "%s: gate and up must share T, K, N, r and the scale", what);
  if (Lg->W.kind == LSN_W_BF16_T || Lu->W.kind == LSN_W_BF16_T)
    return fail(LSN_E_ARG, "%s: the transposed bf16 layout is for the backward only", what);
  const bool bf16 = Lg->W.kind == LSN_W_BF16 && Lu->W.kind == LSN_W_BF16;
  if (!bf16 && (!gate || !up))
    return fail(LSN_E_ARG, "%s: with NF4 weights gate and up must be given", what);
  if (adapters != LSN_ADAPTERS_OFF && adapters != LSN_ADAPTERS_ON && adapters != LSN_ADAPTERS_U_READY)
    return fail(LSN_E_ARG, "%s: unknown adapters mode %d", what, adapters);
  const int64_t T = Lg->T, K = Lg->K, N = Lg->N, r = Lg->r;
  if (!X || !M || !aligned16(X) || !aligned16(M) || (gate && !aligned16(gate)) || (up && !aligned16(up)))
    return fail(LSN_E_ARG, "%s: X and M must be non-null, and X, M, gate, up 16-byte aligned", what);
  if (adapters && (!Ug || !Uu || !aligned16(Ug) || !aligned16(Uu)))
    return fail(LSN_E_ARG, "%s: Ug and Uu must be non-null and 16-byte aligned when adapters are on", what);
  const size_t yb = (size_t)(T * N * 2), ub = (size_t)(T * r * 2);
  const void *outs[5] = {M, gate, up};
  size_t outb[5] = {yb, yb, yb};
  int n_out = 3;
  if (adapters == LSN_ADAPTERS_ON) {
    outs[n_out] = Ug;
    outb[n_out++] = ub;
    outs[n_out] = Uu;
    outb[n_out++] = ub;
  }
  const void *ins[12] = {X, Lg->A, Lg->B, Lu->A, Lu->B};
  size_t inb[12] = {(size_t)(T * K * 2), (size_t)(r * K * 2), (size_t)(N * r * 2), (size_t)(r * K * 2),
                    (size_t)(N * r * 2)};
  int n_in = 5;
  n_in += w_ranges(Lg, ins + n_in, inb + n_in);
  n_in += w_ranges(Lu, ins + n_in, inb + n_in);
  if (adapters == LSN_ADAPTERS_U_READY) {
    ins[n_in] = Ug;
    inb[n_in++] = ub;
    ins[n_in] = Uu;
    inb[n_in++] = ub;
  }
  for (int o = 0; o < n_out; ++o) {
    if (!outs[o]) continue;
    for (int i = 0; i < n_in; ++i)
      if (ranges_overlap(outs[o], outb[o], ins[i], inb[i]))
        return fail(LSN_E_ARG, "%s: an output overlaps an input", what);
    for (int p = 0; p < o; ++p)
      if (outs[p] && ranges_overlap(outs[o], outb[o], outs[p], outb[p]))
        return fail(LSN_E_ARG, "%s: two outputs overlap", what);
  }
  if ((st = require_gfx950()) != LSN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (!bf16) {
    const lsn_lora_linear Ls[2] = {*Lg, *Lu};
    uint16_t *Ys[2] = {gate, up};
    uint16_t *Us[2] = {Ug, Uu};
    if ((st = fwd_group_impl(what, 2, Ls, adapters, X, Ys, Us, nullptr, 0u, nullptr, ws, ws_bytes, s)) != LSN_OK)
      return st;
    return swiglu_fwd(T * N, gate, up, M, stream);
  }
  if (adapters == LSN_ADAPTERS_ON) {
    RowProjSet set{};
    set.n = 2;
    set.P[0] = Lg->A;
    set.P[1] = Lu->A;
    set.out[0] = Ug;
    set.out[1] = Uu;
    set.r[0] = set.r[1] = (int)r;
    set.start[1] = (int)r;
    set.total = (int)(2 * r);
    if ((st = launch_rowproj(X, T, K, set, s)) != LSN_OK) return st;
  }
  DirectArgs d{};
  d.M = T;
  d.K = K;
  d.act = X;
  d.nseg = 1;
  d.seg[0].N = N;
  d.seg[0].w = Lg->W.bf16;
  d.seg[0].lr_w = Lg->B;
  d.seg[0].lr_act = adapters ? Ug : nullptr;
  d.seg[0].out = gate;
  d.x.w2 = Lu->W.bf16;
  d.x.lr_w2 = Lu->B;
  d.x.lr_act2 = adapters ? Uu : nullptr;
  d.x.out2 = up;
  d.x.mout = M;
  d.r = (int)r;
  d.scale = Lg->scale;
  d.adapters = adapters ? 1 : 0;
  return launch_gemm_direct(d, EPI_SWIGLU, s);
}

}  // extern "C"

namespace {

// The backward of one linear on the workspace `ws` (ws_bytes long); `what` names the entry point
// in error messages. sw (may be null): the SwiGLU's inputs (gate, up) and gradient outputs
// (dgate, dup) when the linear is the down projection after a SwiGLU: dX is then dm, not stored
// (dX unused, dx_mode LSN_DX_BF16_SET), and the epilogue writes dgate and dup.
lsn_status bwd_impl(const char *what, const lsn_lora_linear *L, const uint16_t *X, const uint16_t *dY,
                    const uint16_t *U, void *dX, int32_t dx_mode, float *dA, float *dB, int32_t grad_mode,
                    void *ws, size_t ws_bytes, void *stream, const EpiOps *sw = nullptr) {
  lsn_status st = check_linear(L, what);
  if (st != LSN_OK) return st;
  const int64_t T = L->T, K = L->K, N = L->N, r = L->r;
  if (sw) {
    if (!sw->gate || !sw->up || !sw->dgate || !sw->dup || !aligned16(sw->gate) || !aligned16(sw->up) ||
        !aligned16(sw->dgate) || !aligned16(sw->dup))
      return fail(LSN_E_ARG, "%s: gate, up, dgate, dup must be non-null and 16-byte aligned", what);
    dx_mode = LSN_DX_BF16_SET;
  }
  if (!X || !dY || !U || (!dX && !sw) || !dA || !dB || !ws)
    return fail(LSN_E_ARG, "%s: null pointer argument", what);
  if (!aligned16(X) || !aligned16(dY) || !aligned16(U) || (dX && !aligned16(dX)) || ((uintptr_t)ws & 255))
    return fail(LSN_E_ARG, "%s: X, dY, U, dX must be 16-byte and ws 256-byte aligned", what);
  if (dx_mode != LSN_DX_BF16_SET && dx_mode != LSN_DX_F32_ADD && dx_mode != LSN_DX_F32_SET)
    return fail(LSN_E_ARG, "%s: unknown dX mode %d", what, dx_mode);
  if (grad_mode != LSN_GRAD_SET && grad_mode != LSN_GRAD_ADD)
    return fail(LSN_E_ARG, "%s: unknown gradient mode %d", what, grad_mode);
  const BwdWs need = bwd_layout(ws, T, K, N, r);
  if (ws_bytes < need.bytes)
    return fail(LSN_E_ARG, "%s: workspace too small (%zu < %zu)", what, ws_bytes, need.bytes);
  const size_t dxb = (size_t)(T * K * (dx_mode == LSN_DX_BF16_SET ? 2 : 4));
  const void *outs[5] = {dA, dB, ws, sw ? (const void *)sw->dgate : dX, sw ? (const void *)sw->dup : nullptr};
  const size_t outb[5] = {(size_t)(r * K * 4), (size_t)(N * r * 4), need.bytes, dxb, dxb};
  const int n_out = sw ? 5 : 4;
  const void *ins[10] = {X, dY, U, L->A, L->B};
  size_t inb[10] = {(size_t)(T * K * 2), (size_t)(T * N * 2), (size_t)(T * r * 2), (size_t)(r * K * 2),
                    (size_t)(N * r * 2)};
  int n_in = 5 + w_ranges(L, ins + 5, inb + 5);
  if (sw) {
    ins[n_in] = sw->gate;
    inb[n_in++] = dxb;
    ins[n_in] = sw->up;
    inb[n_in++] = dxb;
  }
  for (int o = 0; o < n_out; ++o) {
    for (int i = 0; i < n_in; ++i)
      if (ranges_overlap(outs[o], outb[o], ins[i], inb[i]))
        return fail(LSN_E_ARG, "%s: an output overlaps an input", what);
    for (int p = 0; p < o; ++p)
      if (ranges_overlap(outs[o], outb[o], outs[p], outb[p]))
        return fail(LSN_E_ARG, "%s: two outputs overlap", what);
  }
  if ((st = require_gfx950()) != LSN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nc = (T + TN_CHUNK - 1) / TN_CHUNK;
  {
    TransposeSet ts{};
    ts.src[0] = L->B;
    ts.dst[0] = need.Bt;
    ts.rows[0] = N;
    ts.cols[0] = r;
    ts.n = 1;
    if (L->W.kind != LSN_W_NF4) {
      ts.src[1] = L->A;
      ts.dst[1] = need.At;
      ts.rows[1] = r;
      ts.cols[1] = K;
      ts.n = 2;
    }
    if ((st = launch_transpose_many(ts, s)) != LSN_OK) return st;
  }
  if ((st = launch_rowproj(dY, T, N, need.Bt, (int)r, need.G, s)) != LSN_OK) return st;
  const int epi = sw ? EPI_SWIGLU_BWD
                     : dx_mode == LSN_DX_F32_ADD ? EPI_F32_ADD : dx_mode == LSN_DX_F32_SET ? EPI_F32_SET : EPI_BF16;
  if (L->W.kind != LSN_W_NF4) {
    // dX = dY W + s G (A^T)^T, a product over N: from W^T [K][N] both operands are N-contiguous;
    // from W [N][K] the GEMM reads its B operand reduction-major (same fragments, same bits)
    DirectArgs d{};
    d.M = T;
    d.K = N;
    d.act = dY;
    d.nseg = 1;
    d.seg[0].N = K;
    d.seg[0].w = L->W.bf16;
    d.seg[0].lr_w = need.At;
    d.seg[0].lr_act = need.G;
    d.seg[0].out = dX;
    d.r = (int)r;
    d.scale = L->scale;
    d.adapters = 1;
    d.b_red_major = L->W.kind == LSN_W_BF16;
    if (sw) d.x = *sw;
    if ((st = launch_gemm_direct(d, epi, s)) != LSN_OK) return st;
  } else {
    GemmArgs a = base_args(L);
    a.M = T;
    a.Nout = K;
    a.Kred = N;
    a.act = dY;
    a.ldw = K;
    a.lr_act = need.G;
    a.lr_w = L->A;
    a.adapters = 1;
    a.out = dX;
    if (sw) a.x = *sw;
    // (this kernel adds or stores bf16: an fp32 store is a zero fill and an add)
    if (epi == EPI_F32_SET && (st = launch_fill_zero(dX, dxb, s)) != LSN_OK) return st;
    if ((st = launch_gemm(GEMM_NN, L->W.kind == LSN_W_NF4 ? W_IS_NF4 : W_IS_BF16,
                          epi == EPI_F32_SET ? EPI_F32_ADD : epi, a, s)) != LSN_OK)
      return st;
  }
  // dB = s dY^T U and dA = s G^T X (stored as A's [r][K]): both partials in one launch, then both
  // reductions in one launch
  const int acc = grad_mode == LSN_GRAD_ADD;
  TnJobs tj{};
  tj.n = 2;
  tj.job[0] = TnJob{dY, N, U, (int)r, need.part_dB, 0};
  tj.job[1] = TnJob{X, K, need.G, (int)r, need.part_dA, 0};
  if ((st = launch_tn_partial_jobs(T, tj, s)) != LSN_OK) return st;
  TnRedJobs rj{};
  rj.n = 2;
  rj.job[0] = TnRedJob{need.part_dB, N, (int)r, L->scale, acc, 0, dB, 0};
  rj.job[1] = TnRedJob{need.part_dA, K, (int)r, L->scale, acc, 1, dA, 0};
  return launch_tn_reduce_jobs(nc, rj, s);
}

}  // namespace

extern "C" {

lsn_status lora_linear_bwd(const lsn_lora_linear *L, const uint16_t *X, const uint16_t *dY, const uint16_t *U,
                           void *dX, int32_t dx_mode, float *dA, float *dB, int32_t grad_mode, void *ws,
                           size_t ws_bytes, void *stream) {
  return bwd_impl("lora_linear_bwd", L, X, dY, U, dX, dx_mode, dA, dB, grad_mode, ws, ws_bytes, stream);
}

lsn_status lora_linear_bwd_swiglu(const lsn_lora_linear *L, const uint16_t *X, const uint16_t *dY,
                                  const uint16_t *U, const uint16_t *gate, const uint16_t *up, uint16_t *dgate,
                                  uint16_t *dup, float *dA, float *dB, int32_t grad_mode, void *ws, size_t ws_bytes,
                                  void *stream) {
  EpiOps sw{};
  sw.gate = gate;
  sw.up = up;
  sw.dgate = dgate;
  sw.dup = dup;
  return bwd_impl("lora_linear_bwd_swiglu", L, X, dY, U, nullptr, LSN_DX_BF16_SET, dA, dB, grad_mode, ws, ws_bytes,
                  stream, &sw);
}

}  // extern "C"

// ---- the backward without a caller workspace, for callers that cannot allocate ----
// One file-scope device array per GPU (created with the library's code object on each device
// it runs on, held until the process ends). In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is handed to kernels.
static constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// the current device's address of `scratch`
lsn_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return check_hip(e, "lora_linear_bwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LSN_E_ARG, "lora_linear_bwd_noalloc: device %d outside the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return check_hip(e, "lora_linear_bwd_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LSN_OK;
}

}  // namespace

extern "C" {

size_t lora_linear_bwd_noalloc_max_ws_bytes(void) { return kNoAllocScratchBytes; }

lsn_status lora_linear_bwd_noalloc(const lsn_lora_linear *L, const uint16_t *X, const uint16_t *dY,
                                   const uint16_t *U, void *dX, int32_t dx_mode, float *dA, float *dB,
                                   int32_t grad_mode, void *stream) {
  lsn_status st = check_linear(L, "lora_linear_bwd_noalloc");
  if (st != LSN_OK) return st;
  const size_t need = bwd_layout(nullptr, L->T, L->K, L->N, L->r).bytes;
  if (need > kNoAllocScratchBytes)
    return fail(LSN_E_ARG, "lora_linear_bwd_noalloc: T=%lld K=%lld N=%lld r=%lld needs %zu B of workspace, more "
                "than the library's static %zu B: use lora_linear_bwd with a caller workspace",
                (long long)L->T, (long long)L->K, (long long)L->N, (long long)L->r, need, kNoAllocScratchBytes);
  if ((st = require_gfx950()) != LSN_OK) return st;
  void *ws = nullptr;
  if ((st = scratch_address(&ws)) != LSN_OK) return st;
  // every buffer the kernels use in the workspace (G, B^T, A^T, the partial sums) is written in
  // full before it is read: nothing has to start at zero
  return bwd_impl("lora_linear_bwd_noalloc", L, X, dY, U, dX, dx_mode, dA, dB, grad_mode, ws,
                  kNoAllocScratchBytes, stream);
}

size_t lora_linear_group_ws_bytes(int32_t n, const lsn_lora_linear *L) {
  if (n < 1 || n > kMaxSegs || !L) return 0;
  size_t total = 0;
  for (int g = 0; g < n; ++g) {
    if (L[g].T < 1 || L[g].K < 1 || L[g].N < 1 || L[g].r < 1) return 0;
    total += bwd_layout(nullptr, L[g].T, L[g].K, L[g].N, L[g].r).bytes;
  }
  return total;
}

lsn_status lora_linear_bwd_group(int32_t n, const lsn_lora_linear *L, const uint16_t *X, const uint16_t *const *dY,
                                 const uint16_t *const *U, void *dX, int32_t dx_mode, float *const *dA,
                                 float *const *dB, int32_t grad_mode, void *ws, size_t ws_bytes, void *stream) {
  if (n < 1 || n > kMaxSegs || !L || !dY || !U || !dA || !dB)
    return fail(LSN_E_ARG, "lora_linear_bwd_group: need 1 <= n <= %d and non-null arrays", kMaxSegs);
  // one GEMM over the members' concatenated N when every W is bf16 in the same layout
  bool fused = L && L[0].W.kind != LSN_W_NF4;
  for (int g = 0; g < n; ++g) {
    lsn_status st = check_linear(&L[g], "lora_linear_bwd_group");
    if (st != LSN_OK) return st;
    if (L[g].T != L[0].T || L[g].K != L[0].K || L[g].r != L[0].r || L[g].scale != L[0].scale)
      return fail(LSN_E_ARG, "lora_linear_bwd_group: members must share T, K, r and the scale");
    fused = fused && L[g].W.kind == L[0].W.kind;
  }
  if (dx_mode != LSN_DX_BF16_SET && dx_mode != LSN_DX_F32_ADD && dx_mode != LSN_DX_F32_SET)
    return fail(LSN_E_ARG, "lora_linear_bwd_group: unknown dX mode %d", dx_mode);
  if (grad_mode != LSN_GRAD_SET && grad_mode != LSN_GRAD_ADD)
    return fail(LSN_E_ARG, "lora_linear_bwd_group: unknown gradient mode %d", grad_mode);
  if (!fused && dx_mode == LSN_DX_BF16_SET && n > 1)
    return fail(LSN_E_ARG, "lora_linear_bwd_group: a bf16 dX summed over several members needs their weights "
                           "in bf16, all in the same layout");
  const int64_t T = L[0].T, K = L[0].K, r = L[0].r;
  if (!X || !dX || !ws || !aligned16(X) || !aligned16(dX) || ((uintptr_t)ws & 255))
    return fail(LSN_E_ARG, "lora_linear_bwd_group: X, dX must be non-null and 16-byte, ws 256-byte aligned");
  const size_t need = lora_linear_group_ws_bytes(n, L);
  if (ws_bytes < need)
    return fail(LSN_E_ARG, "lora_linear_bwd_group: workspace too small (%zu < %zu)", ws_bytes, need);
  // every output against every input, and the outputs pairwise
  const void *outs[2 + 2 * kMaxSegs];
  size_t outb[2 + 2 * kMaxSegs];
  int n_out = 0;
  outs[n_out] = dX;
  outb[n_out++] = (size_t)(T * K * (dx_mode == LSN_DX_BF16_SET ? 2 : 4));
  outs[n_out] = ws;
  outb[n_out++] = need;
  for (int g = 0; g < n; ++g) {
    if (!dY[g] || !U[g] || !dA[g] || !dB[g] || !aligned16(dY[g]) || !aligned16(U[g]))
      return fail(LSN_E_ARG, "lora_linear_bwd_group: member %d: null or misaligned dY, U, dA or dB", g);
    outs[n_out] = dA[g];
    outb[n_out++] = (size_t)(r * K * 4);
    outs[n_out] = dB[g];
    outb[n_out++] = (size_t)(L[g].N * r * 4);
  }
  for (int o = 0; o < n_out; ++o) {
    for (int p = 0; p < o; ++p)
      if (ranges_overlap(outs[o], outb[o], outs[p], outb[p]))
        return fail(LSN_E_ARG, "lora_linear_bwd_group: two outputs overlap");
    if (ranges_overlap(outs[o], outb[o], X, (size_t)(T * K * 2)))
      return fail(LSN_E_ARG, "lora_linear_bwd_group: an output overlaps X");
    for (int g = 0; g < n; ++g) {
      const void *ins[8] = {dY[g], U[g], L[g].A, L[g].B};
      size_t inb[8] = {(size_t)(T * L[g].N * 2), (size_t)(T * r * 2), (size_t)(r * K * 2), (size_t)(L[g].N * r * 2)};
      const int n_in = 4 + w_ranges(&L[g], ins + 4, inb + 4);
      for (int i = 0; i < n_in; ++i)
        if (ranges_overlap(outs[o], outb[o], ins[i], inb[i]))
          return fail(LSN_E_ARG, "lora_linear_bwd_group: an output overlaps an input of member %d", g);
    }
  }
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (!fused) {
    // one member at a time (fp32 accumulation into dX in member order)
    char *w = static_cast<char *>(ws);
    for (int g = 0; g < n; ++g) {
      const size_t b = bwd_layout(nullptr, T, K, L[g].N, r).bytes;
      // an fp32 store: the first member stores, the others add
      const int32_t mode = (dx_mode == LSN_DX_F32_SET && g > 0) ? LSN_DX_F32_ADD : dx_mode;
      if ((st = lora_linear_bwd(&L[g], X, dY[g], U[g], dX, mode, dA[g], dB[g], grad_mode, w, b, stream)) != LSN_OK)
        return st;
      w += b;
    }
    return LSN_OK;
  }
  // G_g = bf16(dY_g B_g) and A_g^T for every member, then the n dX products as one GEMM whose
  // reduction runs over the members' N in turn, then dA_g, dB_g
  BwdWs part[kMaxSegs];
  char *w = static_cast<char *>(ws);
  DirectArgs d{};
  d.M = T;
  d.nseg = 1;
  d.seg[0].N = K;
  d.seg[0].out = dX;
  d.nkseg = n;
  d.r = (int)r;
  d.scale = L[0].scale;
  d.adapters = 1;
  d.b_red_major = L[0].W.kind == LSN_W_BF16;
  TransposeSet ts{};
  for (int g = 0; g < n; ++g) {
    part[g] = bwd_layout(w, T, K, L[g].N, r);
    w += part[g].bytes;
    ts.src[ts.n] = L[g].B;
    ts.dst[ts.n] = part[g].Bt;
    ts.rows[ts.n] = L[g].N;
    ts.cols[ts.n++] = r;
    ts.src[ts.n] = L[g].A;
    ts.dst[ts.n] = part[g].At;
    ts.rows[ts.n] = r;
    ts.cols[ts.n++] = K;
  }
  if ((st = launch_transpose_many(ts, s)) != LSN_OK) return st;
  // the G jobs run longest first (a workgroup's work grows with N), so that the short ones fill
  // the end of the launch
  int order[kMaxSegs];
  for (int g = 0; g < n; ++g) order[g] = g;
  for (int i = 1; i < n; ++i)
    for (int j = i; j > 0 && L[order[j]].N > L[order[j - 1]].N; --j) std::swap(order[j], order[j - 1]);
  int slot[kMaxSegs];
  for (int i = 0; i < n; ++i) slot[order[i]] = i;
  RowProjJobs gj{};
  gj.n = n;
  for (int g = 0; g < n; ++g) {
    const int64_t N = L[g].N;
    RowProjJob &J = gj.job[slot[g]];
    J.act = dY[g];
    J.K = N;
    J.set.n = 1;
    J.set.total = (int)r;
    J.set.P[0] = part[g].Bt;
    J.set.out[0] = part[g].G;
    J.set.r[0] = (int)r;
    d.kseg[g].act = dY[g];
    d.kseg[g].w = L[g].W.bf16;
    d.kseg[g].K = N;
    d.kseg[g].lr_act = part[g].G;
    d.kseg[g].lr_w = part[g].At;
  }
  // every member's G in one launch
  if ((st = launch_rowproj_jobs(T, gj, s)) != LSN_OK) return st;
  const int epi = dx_mode == LSN_DX_F32_ADD ? EPI_F32_ADD : dx_mode == LSN_DX_F32_SET ? EPI_F32_SET : EPI_BF16;
  if ((st = launch_gemm_direct(d, epi, s)) != LSN_OK) return st;
  // every member's dB and dA partials in one launch, then every reduction in one launch
  const int64_t nc = (T + TN_CHUNK - 1) / TN_CHUNK;
  const int acc = grad_mode == LSN_GRAD_ADD;
  TnJobs tj{};
  TnRedJobs rj{};
  for (int g = 0; g < n; ++g) {
    const int64_t N = L[g].N;
    tj.job[tj.n++] = TnJob{dY[g], N, U[g], (int)r, part[g].part_dB, 0};
    tj.job[tj.n++] = TnJob{X, K, part[g].G, (int)r, part[g].part_dA, 0};
    rj.job[rj.n++] = TnRedJob{part[g].part_dB, N, (int)r, L[g].scale, acc, 0, dB[g], 0};
    rj.job[rj.n++] = TnRedJob{part[g].part_dA, K, (int)r, L[g].scale, acc, 1, dA[g], 0};
  }
  if ((st = launch_tn_partial_jobs(T, tj, s)) != LSN_OK) return st;
  return launch_tn_reduce_jobs(nc, rj, s);
}

}  // extern "C"
