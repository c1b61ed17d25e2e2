// Asymmetric W4A16 QAT grouped GEMMs (placeholder until the MFMA kernels land).
#include <hip/hip_runtime.h>

#include "nvq.h"
#include "nvq_internal.h"

extern "C" size_t qat_gemm_workspace_bytes(int64_t rows, int64_t E) {
  (void)rows;
  (void)E;
  return nvq::kAlign;
}

extern "C" int qat_fakequant_gemm_w4a16(const nvq_qat_gemm_args* a, void* stream) {
  (void)a;
  (void)stream;
  return NVQ_EUNSUPPORTED;
}
