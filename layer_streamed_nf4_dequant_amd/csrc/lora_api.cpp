// C ABI of the LoRA linear (forward and backward). Contracts in include/lsnf4.h.
#include "common.h"

using namespace lsn;

extern "C" {

size_t lora_linear_ws_bytes(int64_t T, int64_t K, int64_t N, int64_t r) {
  (void)T; (void)K; (void)N; (void)r;
  return 0;
}

lsn_status lora_linear_fwd(const lsn_lora_linear *L, int32_t adapters, const uint16_t *X,
                           uint16_t *Y, uint16_t *U, void *ws, size_t ws_bytes, void *stream) {
  (void)L; (void)adapters; (void)X; (void)Y; (void)U; (void)ws; (void)ws_bytes; (void)stream;
  return fail(LSN_E_STATE, "lora_linear_fwd: not built yet");
}

lsn_status lora_linear_bwd(const lsn_lora_linear *L, const uint16_t *X, const uint16_t *dY,
                           const uint16_t *U, void *dX, int32_t dx_mode, float *dA, float *dB,
                           int32_t grad_mode, void *ws, size_t ws_bytes, void *stream) {
  (void)L; (void)X; (void)dY; (void)U; (void)dX; (void)dx_mode; (void)dA; (void)dB;
  (void)grad_mode; (void)ws; (void)ws_bytes; (void)stream;
  return fail(LSN_E_STATE, "lora_linear_bwd: not built yet");
}

}  // extern "C"
