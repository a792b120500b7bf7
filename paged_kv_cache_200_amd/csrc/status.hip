// Diagnostics: version, status strings and the device error word.

#include "common.h"

extern "C" int pkv_version(void) { return 100; }

extern "C" const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_DTYPE: return "unknown dtype";
    case PKV_ERR_SHAPE: return "unsupported size or shape";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_DEVICE: return "HIP runtime call failed";
    case PKV_ERR_OUT_OF_BLOCKS: return "block pool exhausted";
    case PKV_ERR_ARG: return "bad argument value";
    case PKV_ERR_SCRATCH: return "the call needs more than the static scratch buffer holds";
    default: return "unknown status";
  }
}

extern "C" int pkv_device_error(pkv_stream_t stream, int32_t* flags) {
  if (!flags) return PKV_ERR_NULL;
  *flags = 0;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_DEVICE;
  int st = pkv_internal_take_error_decode(flags);
  if (st == PKV_OK) st = pkv_internal_take_error_append(flags);
  if (st == PKV_OK) st = pkv_internal_take_error_copy(flags);
  if (st == PKV_OK) st = pkv_internal_take_error_prefill(flags);
  return st;
}
