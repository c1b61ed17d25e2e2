// Library-wide C-ABI pieces: status strings, the device status word and a
// few host helpers used by every entry point.

#include <hip/hip_runtime.h>

#include "nvq.h"
#include "nvq_internal.h"

namespace nvq {

namespace {
__global__ void k_status_clear(uint32_t* status) { *status = 0u; }
}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

int clear_status(uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_status_clear, dim3(1), dim3(1), 0, s, status);
  return last_launch();
}

}  // namespace nvq

extern "C" const char* nvq_status_string(int status) {
  switch (status) {
    case NVQ_OK: return "ok";
    case NVQ_EINVAL: return "invalid argument (null pointer or bad enum)";
    case NVQ_ESHAPE: return "unsupported shape";
    case NVQ_EALIGN: return "misaligned pointer";
    case NVQ_EWORKSPACE: return "workspace missing or too small";
    case NVQ_EHIP: return "HIP runtime error";
    case NVQ_EUNSUPPORTED: return "not supported by this build";
    default: return "unknown status";
  }
}

extern "C" int nvq_device_status(const void* ws, void* stream, uint32_t* flags) {
  if (!ws || !flags) return NVQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return NVQ_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return NVQ_EHIP;
  *flags = v;
  return NVQ_OK;
}
