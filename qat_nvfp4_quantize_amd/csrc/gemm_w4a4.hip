// W4A4 MoE grouped GEMM with residual compensation (placeholder until the
// MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "nvq.h"
#include "nvq_internal.h"

extern "C" size_t moe_gemm_workspace_bytes(int64_t rows, int64_t E) {
  (void)rows;
  (void)E;
  return nvq::kAlign;
}

extern "C" int moe_grouped_gemm_w4a4_comp(const nvq_moe_gemm_args* a, void* stream) {
  (void)a;
  (void)stream;
  return NVQ_EUNSUPPORTED;
}
