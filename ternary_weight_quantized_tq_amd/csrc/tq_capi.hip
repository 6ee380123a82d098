// Workspace sizing and error reporting for the C entry points.
#include "tq_internal.h"

#include <stdio.h>

namespace {
thread_local char g_last_error[256] = "";
}

void tq_set_hip_error(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
}

extern "C" const char* tq_last_error(void) { return g_last_error; }

extern "C" size_t tq_workspace_bytes(int op, const tq_weights* w, int m_or_t, int topk) {
  if (tq_check_weights(w, 0) != TQ_OK || m_or_t < 1) return SIZE_MAX;
  switch (op) {
    case TQ_OP_GEMV:
      if (w->num_experts != 1 || m_or_t > 8) return SIZE_MAX;
      return tq_gemv_workspace(w->n, w->k, m_or_t);
    case TQ_OP_MOE:
      if (topk < 1 || topk > 32) return SIZE_MAX;
      return tq_moe_workspace(w, m_or_t, topk);
    case TQ_OP_GEMM:
      if (w->num_experts != 1) return SIZE_MAX;
      return tq_gemm_workspace(w->n, w->k, m_or_t);
    default:
      return SIZE_MAX;
  }
}
