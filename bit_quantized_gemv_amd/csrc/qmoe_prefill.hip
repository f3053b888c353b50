// qmoe_prefill.hip -- chunked prefill (grouped dequantizing GEMMs on MFMA).
#include "qmoe_common.h"

namespace qmoe {
size_t prefill_ws_bytes(const qmoe_moe_layer& L, int T) {
  (void)L; (void)T;
  return 0;
}
qmoe_status launch_prefill(const qmoe_moe_layer& L, const uint16_t* X, int T, const int32_t* idx,
                           const float* w, const uint16_t* residual, uint16_t* out, uint8_t* ws,
                           void* stream) {
  (void)L; (void)X; (void)T; (void)idx; (void)w; (void)residual; (void)out; (void)ws; (void)stream;
  return QMOE_ERR_UNSUPPORTED;
}
}  // namespace qmoe
