// Library-level entry points of libmoefp8: workspace sizing, the debug
// read-back of the sticky device-error word, status strings and version.
#include "common.hpp"

namespace moe {
size_t quantize_rows_ws_bytes(int64_t R, int64_t C, int mode);
size_t sort_ws_bytes(int64_t M, int E);
size_t gmm_ws_bytes();
size_t tgmm_ws_bytes(int64_t M, int64_t K, int64_t N, int E);
}  // namespace moe

extern "C" int moe_workspace_bytes(int op, int64_t d0, int64_t d1, int64_t d2, int32_t E, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  switch (op) {
    case MOE_OP_QUANTIZE_ROWS:
      if (d0 < 0 || d1 < 0) return MOE_ERR_SHAPE;
      *bytes = moe::quantize_rows_ws_bytes(d0, d1, static_cast<int>(d2));
      return MOE_OK;
    case MOE_OP_SORT_BY_EXPERT:
      if (d0 < 0 || E <= 0 || E > 1024) return MOE_ERR_SHAPE;
      *bytes = moe::sort_ws_bytes(d0, E);
      return MOE_OK;
    case MOE_OP_GMM:
      if (d0 < 0 || d1 < 0 || d2 < 0) return MOE_ERR_SHAPE;
      *bytes = moe::gmm_ws_bytes();
      return MOE_OK;
    case MOE_OP_TGMM:
      if (d0 < 0 || d1 < 0 || d2 < 0 || E <= 0 || E > 1024) return MOE_ERR_SHAPE;
      *bytes = moe::tgmm_ws_bytes(d0, d1, d2, E);
      return MOE_OK;
    case MOE_OP_GATHER_REDUCE:
    case MOE_OP_QUANTIZE_WEIGHTS:
      *bytes = 256;
      return MOE_OK;
    default:
      return MOE_ERR_UNSUPPORTED;
  }
}

extern "C" int moe_debug_check(const void* ws, void* stream, int32_t* device_error) {
  if (!ws || !device_error) return MOE_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_HIP;
  if (hipMemcpy(device_error, ws, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "sizes inconsistent or outside the supported range";
    case MOE_ERR_UNSUPPORTED: return "unsupported combination of arguments";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" int moe_version(void) { return 100; }
