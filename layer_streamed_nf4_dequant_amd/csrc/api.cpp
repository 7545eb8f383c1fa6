// C ABI of liblsnf4: validation, error reporting and dispatch to the gfx950 kernels.
// The entry points and their contracts are declared and documented in include/lsnf4.h.

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"

namespace lsn {

namespace {
thread_local std::string g_err;
}

lsn_status fail(lsn_status st, const char *fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

lsn_status check_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return LSN_OK;
  return fail(LSN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The library runs on gfx950 only: anything else is refused, never emulated.
lsn_status require_gfx950() {
  static std::atomic<int> verdict[64];   // 0 unknown, 1 ok, 2 refused
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LSN_E_HIP, "hipGetDevice failed: no GPU?");
  if (dev < 0 || dev >= 64) return fail(LSN_E_STATE, "device index %d out of range", dev);
  int v = verdict[dev].load();
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(LSN_E_HIP, "hipGetDeviceProperties failed");
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    verdict[dev].store(v);
  }
  if (v != 1) return fail(LSN_E_STATE, "liblsnf4 runs only on gfx950 (MI355X)");
  // surface an asynchronous error left by earlier work before enqueueing more
  const hipError_t pending = hipGetLastError();
  if (pending != hipSuccess)
    return fail(LSN_E_HIP, "pending HIP error from earlier work: %s", hipGetErrorString(pending));
  return LSN_OK;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

lsn_status check_nf4_shape(int64_t rows, int64_t cols, const char *what) {
  if (rows <= 0 || cols <= 0 || cols % 64 != 0 || (rows * cols) % 16384 != 0)
    return fail(LSN_E_ARG, "%s: NF4 needs cols %% 64 == 0 and rows*cols %% 16384 == 0 (got %lld x %lld)",
                what, (long long)rows, (long long)cols);
  return LSN_OK;
}

lsn_status check_nf4(const lsn_nf4 *w, const char *what) {
  if (!w) return fail(LSN_E_ARG, "%s: null NF4 descriptor", what);
  lsn_status st = check_nf4_shape(w->rows, w->cols, what);
  if (st != LSN_OK) return st;
  if (!w->codes || !w->qabsmax || !w->absmax2)
    return fail(LSN_E_ARG, "%s: null NF4 codes/qabsmax/absmax2", what);
  if (((uintptr_t)w->codes & 15) != 0)
    return fail(LSN_E_ARG, "%s: NF4 codes must be 16-byte aligned", what);
  if (((uintptr_t)w->absmax2 & 3) != 0)
    return fail(LSN_E_ARG, "%s: absmax2 must be 4-byte aligned", what);
  if (!std::isfinite(w->mean)) return fail(LSN_E_ARG, "%s: non-finite NF4 mean", what);
  return LSN_OK;
}

size_t nf4_bytes(const lsn_nf4 &w) {
  const size_t n = (size_t)(w.rows * w.cols);
  return n / 2 + n / 64 + 4 * (n / 16384);
}

}  // namespace lsn

using namespace lsn;

extern "C" {

const char *lsn_last_error(void) { return g_err.c_str(); }

int32_t lsn_abi_version(void) { return LSN_ABI_VERSION; }

void lsn_nf4_codebook(float levels[16], float midpoints[15]) {
  const Nf4Table &t = nf4_table();
  if (levels) std::memcpy(levels, t.q, sizeof(t.q));
  if (midpoints) std::memcpy(midpoints, t.m, sizeof(t.m));
}

size_t nf4_pack_ws_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  const size_t nb = (size_t)(rows * cols) / 64;
  return ((nb * 4 + 255) / 256) * 256 + 256;
}

lsn_status nf4_pack(const float *w, int64_t rows, int64_t cols, uint8_t *codes, int8_t *qabsmax,
                    float *absmax2, float *mean_out, void *ws, size_t ws_bytes, void *stream) {
  lsn_status st = check_nf4_shape(rows, cols, "nf4_pack");
  if (st != LSN_OK) return st;
  if (!w || !codes || !qabsmax || !absmax2 || !mean_out || !ws)
    return fail(LSN_E_ARG, "nf4_pack: null pointer argument");
  if (((uintptr_t)w & 15) || ((uintptr_t)codes & 3) || ((uintptr_t)absmax2 & 3) || ((uintptr_t)ws & 255))
    return fail(LSN_E_ARG, "nf4_pack: w must be 16-byte, codes/absmax2 4-byte, ws 256-byte aligned");
  const int64_t n = rows * cols;
  const int64_t nb = n / 64;
  if (ws_bytes < nf4_pack_ws_bytes(rows, cols))
    return fail(LSN_E_ARG, "nf4_pack: workspace too small (%zu < %zu)", ws_bytes,
                nf4_pack_ws_bytes(rows, cols));
  const size_t in_bytes = (size_t)n * 4;
  if (ranges_overlap(codes, n / 2, w, in_bytes) || ranges_overlap(qabsmax, nb, w, in_bytes) ||
      ranges_overlap(absmax2, nb / 256 * 4, w, in_bytes) || ranges_overlap(ws, ws_bytes, w, in_bytes))
    return fail(LSN_E_ARG, "nf4_pack: an output overlaps the input");
  if ((st = require_gfx950()) != LSN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  float *absmax = (float *)ws;
  int *flag = (int *)((char *)ws + ((nb * 4 + 255) / 256) * 256);
  if ((st = check_hip(hipMemsetAsync(flag, 0, sizeof(int), s), "nf4_pack memset")) != LSN_OK) return st;
  if ((st = launch_pack_codes(w, n, codes, absmax, flag, s)) != LSN_OK) return st;
  std::vector<float> host(nb);
  int host_flag = 0;
  if ((st = check_hip(hipMemcpyAsync(host.data(), absmax, nb * 4, hipMemcpyDeviceToHost, s),
                      "nf4_pack D2H absmax")) != LSN_OK)
    return st;
  if ((st = check_hip(hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, s),
                      "nf4_pack D2H flag")) != LSN_OK)
    return st;
  if ((st = check_hip(hipStreamSynchronize(s), "nf4_pack sync")) != LSN_OK) return st;
  if (host_flag) return fail(LSN_E_ARG, "nf4_pack: non-finite weight");
  // mu = fl32(S / n_b), S the left-to-right fp64 sum of the block absmax values
  double S = 0.0;
  for (int64_t i = 0; i < nb; ++i) S += (double)host[i];
  const float mu = (float)(S / (double)nb);
  if ((st = launch_pack_second(absmax, nb, mu, qabsmax, absmax2, s)) != LSN_OK) return st;
  *mean_out = mu;
  return LSN_OK;
}

lsn_status nf4_dequant_batch(int32_t n, const lsn_nf4 *w, void *const *out, int32_t out_dtype, void *stream) {
  if (n < 1 || n > kMaxDqJobs || !w || !out)
    return fail(LSN_E_ARG, "nf4_dequant: need 1 <= n <= %d tensors and non-null arrays", kMaxDqJobs);
  if (out_dtype != LSN_OUT_BF16 && out_dtype != LSN_OUT_F32 && out_dtype != LSN_OUT_BF16_T)
    return fail(LSN_E_ARG, "nf4_dequant: unknown output dtype %d", out_dtype);
  for (int g = 0; g < n; ++g) {
    lsn_status st = check_nf4(&w[g], "nf4_dequant");
    if (st != LSN_OK) return st;
    if (!out[g]) return fail(LSN_E_ARG, "nf4_dequant: null output %d", g);
    if ((uintptr_t)out[g] & 15) return fail(LSN_E_ARG, "nf4_dequant: output %d must be 16-byte aligned", g);
    if (out_dtype == LSN_OUT_BF16_T && w[g].rows % 8)
      return fail(LSN_E_ARG, "nf4_dequant: the transposed output needs rows %% 8 == 0 (got %lld)",
                  (long long)w[g].rows);
  }
  for (int g = 0; g < n; ++g) {
    const size_t ne = (size_t)(w[g].rows * w[g].cols);
    const size_t ob = ne * (out_dtype == LSN_OUT_F32 ? 4 : 2);
    for (int h = 0; h < n; ++h) {
      const size_t nh = (size_t)(w[h].rows * w[h].cols);
      if (ranges_overlap(out[g], ob, w[h].codes, nh / 2) || ranges_overlap(out[g], ob, w[h].qabsmax, nh / 64) ||
          ranges_overlap(out[g], ob, w[h].absmax2, nh / 16384 * 4))
        return fail(LSN_E_ARG, "nf4_dequant: an output overlaps an NF4 input");
      if (h < g && ranges_overlap(out[g], ob, out[h], nh * (out_dtype == LSN_OUT_F32 ? 4 : 2)))
        return fail(LSN_E_ARG, "nf4_dequant: two outputs overlap");
    }
  }
  lsn_status st = require_gfx950();
  if (st != LSN_OK) return st;
  return launch_dequant(n, w, out, out_dtype, (hipStream_t)stream);
}

lsn_status nf4_dequant(const lsn_nf4 *w, void *out, int32_t out_dtype, void *stream) {
  void *outs[1] = {out};
  return nf4_dequant_batch(1, w, outs, out_dtype, stream);
}

}  // extern "C"
