// The resident ends of the stack: the frozen embedding lookup, and cross-entropy through the
// frozen LM head, chunked over token rows.
//
// "Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript @7:42-7:55: the
// embedding table and the output head stay resident and unquantised beside the streamed layers.
// "Exact Layer Streaming", Abstract: the cross-entropy logits term is the memory cost to watch
// (14 bytes per logit element measured, 6 by first principles); transcript @4:01-4:15: at a
// 150k vocabulary the logits of one batch outgrow the whole layer pool. Here the logits of a
// chunk of rows exist only in the caller's workspace, 6 bytes per element (fp32 logits and bf16
// logit gradients), and the two products run on the direct-load GEMM:
//   z  = h_c W^T          (fp32, [rows][V])
//   lse_t = max_j z_tj + log sum_j exp(z_tj - max_j z_tj),  loss_t = lse_t - z_t,label_t
//   dz = bf16( (softmax(z)_tj - [j == label_t]) * scale )
//   dh_c = bf16( dz W )   (a reduction over the vocabulary: W read reduction-major, split over
//                          kCeSplit ranges of the vocabulary whose fp32 partials are then added
//                          in order: a chunk has few output tiles and a very long reduction)
// A row whose label is negative is ignored: loss 0, dz 0.

#include <cmath>

#include "common.h"
#include "gemm.h"

namespace lsn {
lsn_status require_gfx950();
bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb);

namespace {

constexpr int kCeThreads = 256;
constexpr int kCeSplit = 8;   // vocabulary ranges of the dh product (fixed: results do not depend on the chunk)

int ce_splits(int64_t V) { return (int)(V / 64 < kCeSplit ? V / 64 : kCeSplit); }

// (max, sum of exp(x - max)) pairs combined in a fixed order: the result depends only on the row
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  const float a = m == -INFINITY ? 0.0f : s * expf(m - mm);
  const float b = m2 == -INFINITY ? 0.0f : s2 * expf(m2 - mm);
  m = mm;
  s = a + b;
}

// One workgroup per row of the chunk. Pass 1: each thread folds its elements (columns
// 4 t + 1024 i .. +3, in increasing i) into a running (max, sum) pair; the 256 pairs are merged by
// a fixed butterfly inside each wave and then wave 0..3 in order. Pass 2 writes the gradients.
__global__ __launch_bounds__(kCeThreads) void k_ce_rows(const float *__restrict__ z, int64_t V,
                                                        const int32_t *__restrict__ labels, float scale,
                                                        float *__restrict__ loss, uint16_t *__restrict__ dz) {
  __shared__ float wm[kCeThreads / 64], wsum[kCeThreads / 64];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float *zr = z + row * V;
  const int lab = labels[row];
  float m = -INFINITY, s = 0.0f;
  for (int64_t j = 4 * t; j < V; j += 4 * kCeThreads) {
    const floatx4_t v = *reinterpret_cast<const floatx4_t *>(zr + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v[e] > m) {
        s = s * expf(m - v[e]) + 1.0f;
        m = v[e];
      } else {
        s += expf(v[e] - m);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    // both lanes of a pair compute the same merge (operands in lane order), so they stay equal
    if ((lane & off) == 0) {
      lse_merge(m, s, m2, s2);
    } else {
      float mo = m2, so = s2;
      lse_merge(mo, so, m, s);
      m = mo;
      s = so;
    }
  }
  if (lane == 0) {
    wm[wave] = m;
    wsum[wave] = s;
  }
  __syncthreads();
  m = wm[0];
  s = wsum[0];
#pragma unroll
  for (int w = 1; w < kCeThreads / 64; ++w) lse_merge(m, s, wm[w], wsum[w]);
  const float lse = m + logf(s);
  const bool ignored = lab < 0 || lab >= V;
  if (t == 0) loss[row] = ignored ? 0.0f : lse - zr[lab];
  uint16_t *dr = dz + row * V;
  for (int64_t j = 4 * t; j < V; j += 4 * kCeThreads) {
    const floatx4_t v = *reinterpret_cast<const floatx4_t *>(zr + j);
    float g[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = expf(v[e] - lse);
      g[e] = ignored ? 0.0f : (p - ((j + e) == lab ? 1.0f : 0.0f)) * scale;
    }
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t o = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2_t *>(dr + j));
  }
}

// X[t] = E[ids[t]] (bf16 rows of H); an id outside [0, V) gives a zero row and is counted in *bad
__global__ __launch_bounds__(256) void k_embed(const int32_t *__restrict__ ids, const uint16_t *__restrict__ E,
                                               int64_t H, int64_t V, uint16_t *__restrict__ X, int *bad) {
  const int64_t row = blockIdx.x;
  const int id = ids[row];
  const bool ok = id >= 0 && id < V;
  if (!ok && threadIdx.x == 0 && bad) atomicAdd(bad, 1);
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(E + (int64_t)(ok ? id : 0) * H);
  u32x4_t *dst = reinterpret_cast<u32x4_t *>(X + row * H);
  for (int64_t c = threadIdx.x; c < H / 8; c += 256) dst[c] = ok ? src[c] : u32x4_t{0, 0, 0, 0};
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace
}  // namespace lsn

using namespace lsn;

extern "C" {

size_t lm_head_ce_ws_bytes(int64_t chunk_rows, int64_t H, int64_t V) {
  if (chunk_rows < 1 || H < 1 || V < 64) return 0;
  return align256((size_t)(chunk_rows * V * 4)) + align256((size_t)(chunk_rows * V * 2)) +
         align256((size_t)(ce_splits(V) * chunk_rows * H * 4));
}

lsn_status lm_head_ce(int64_t T, int64_t H, int64_t V, const uint16_t *h, const uint16_t *W, const int32_t *labels,
                      float grad_scale, float *loss, uint16_t *dh, int64_t chunk_rows, void *ws, size_t ws_bytes,
                      void *stream) {
  if (T < 1 || H < 64 || H % 64 || V < 64 || V % 64)
    return fail(LSN_E_ARG, "lm_head_ce: need T >= 1 and H, V positive multiples of 64 (got T=%lld H=%lld V=%lld)",
                (long long)T, (long long)H, (long long)V);
  if (chunk_rows < 1) return fail(LSN_E_ARG, "lm_head_ce: chunk_rows must be >= 1");
  if (!h || !W || !labels || !loss || !dh || !ws)
    return fail(LSN_E_ARG, "lm_head_ce: null pointer argument");
  if (((uintptr_t)h | (uintptr_t)W | (uintptr_t)dh) & 15 || (uintptr_t)ws & 255)
    return fail(LSN_E_ARG, "lm_head_ce: h, W, dh must be 16-byte and ws 256-byte aligned");
  if (!std::isfinite(grad_scale)) return fail(LSN_E_ARG, "lm_head_ce: grad_scale must be finite");
  const int64_t rows_max = chunk_rows < T ? chunk_rows : T;
  const size_t need = lm_head_ce_ws_bytes(rows_max, H, V);
  if (ws_bytes < need)
    return fail(LSN_E_ARG, "lm_head_ce: workspace too small (%zu < %zu)", ws_bytes, need);
  const size_t hb = (size_t)(T * H * 2), wb = (size_t)(V * H * 2);
  const void *ins[] = {h, W, labels};
  const size_t inb[] = {hb, wb, (size_t)(T * 4)};
  const void *outs[] = {loss, dh, ws};
  const size_t outb[] = {(size_t)(T * 4), hb, need};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 3; ++i)
      if (ranges_overlap(outs[o], outb[o], ins[i], inb[i]))
        return fail(LSN_E_ARG, "lm_head_ce: an output overlaps an input");
    for (int p = 0; p < o; ++p)
      if (ranges_overlap(outs[o], outb[o], outs[p], outb[p])) return fail(LSN_E_ARG, "lm_head_ce: outputs overlap");
  }
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  float *z = static_cast<float *>(ws);
  uint16_t *dz = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + align256((size_t)(rows_max * V * 4)));
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(dz) + align256((size_t)(rows_max * V * 2)));
  const int S = ce_splits(V);
  for (int64_t c0 = 0; c0 < T; c0 += rows_max) {
    const int64_t rows = T - c0 < rows_max ? T - c0 : rows_max;
    DirectArgs d{};                                   // z = h_c W^T, fp32
    d.M = rows;
    d.K = H;
    d.act = h + c0 * H;
    d.nseg = 1;
    d.seg[0].N = V;
    d.seg[0].w = W;
    d.seg[0].out = z;
    if ((st = launch_gemm_direct(d, EPI_F32_SET, s)) != LSN_OK) return st;
    hipLaunchKernelGGL(k_ce_rows, dim3((unsigned)rows), dim3(kCeThreads), 0, s, z, V, labels + c0, grad_scale,
                       loss + c0, dz);
    if ((st = check_hip(hipGetLastError(), "k_ce_rows launch")) != LSN_OK) return st;
    DirectArgs e{};                                   // dh_c = dz W, a reduction over V, split
    e.M = rows;
    e.K = V;
    e.act = dz;
    e.nseg = 1;
    e.seg[0].N = H;
    e.seg[0].w = W;
    e.seg[0].out = part;
    e.b_red_major = 1;
    e.ksplit = S;
    if (S > 1) {
      if ((st = launch_gemm_direct(e, EPI_F32_SET, s)) != LSN_OK) return st;
      if ((st = launch_splitk_reduce(part, S, rows * H, dh + c0 * H, s)) != LSN_OK) return st;
    } else {
      e.ksplit = 0;
      e.seg[0].out = dh + c0 * H;
      if ((st = launch_gemm_direct(e, EPI_BF16, s)) != LSN_OK) return st;
    }
  }
  return LSN_OK;
}

lsn_status embedding_gather(int64_t T, int64_t H, int64_t V, const int32_t *ids, const uint16_t *E, uint16_t *X,
                            int32_t *bad_ids, void *stream) {
  if (T < 1 || H < 8 || H % 8 || V < 1)
    return fail(LSN_E_ARG, "embedding_gather: need T >= 1, H a positive multiple of 8, V >= 1");
  if (!ids || !E || !X || ((uintptr_t)E | (uintptr_t)X) & 15)
    return fail(LSN_E_ARG, "embedding_gather: null or misaligned pointer");
  if (ranges_overlap(X, (size_t)(T * H * 2), E, (size_t)(V * H * 2)) ||
      ranges_overlap(X, (size_t)(T * H * 2), ids, (size_t)(T * 4)))
    return fail(LSN_E_ARG, "embedding_gather: X overlaps an input");
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  hipLaunchKernelGGL(k_embed, dim3((unsigned)T), dim3(256), 0, (hipStream_t)stream, ids, E, H, V, X,
                     reinterpret_cast<int *>(bad_ids));
  return check_hip(hipGetLastError(), "k_embed launch");
}

}  // extern "C"
