// Workspace sizing and error reporting for the C entry points.
#include "tq_internal.h"

#include <limits.h>
#include <stdio.h>

namespace {
thread_local char g_last_error[256] = "";
}

void tq_set_hip_error(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
}

extern "C" const char* tq_last_error(void) { return g_last_error; }

extern "C" size_t tq_workspace_bytes(int op, const tq_weights* w, int m_or_t, int topk) {
  if (tq_check_weights(w, 0) != TQ_OK || !tq::tq_dim_ok(m_or_t)) return SIZE_MAX;
  switch (op) {
    case TQ_OP_GEMV:
      if (w->num_experts != 1 || m_or_t > 8) return SIZE_MAX;
      return tq_gemv_workspace(w->n, w->k, m_or_t);
    case TQ_OP_MOE:
      if (topk < 1 || topk > 32 || static_cast<long long>(m_or_t) * topk > INT_MAX / 4) return SIZE_MAX;
      return tq_moe_workspace(w, m_or_t, topk);
    case TQ_OP_GEMM:
      if (w->num_experts != 1) return SIZE_MAX;
      return tq_gemm_workspace(w->n, w->k, m_or_t);
    default:
      return SIZE_MAX;
  }
}

// ------------------------------------------- memory-read reference ---
// tq_read_bytes: a plain one-pass read of a buffer with the decode GEMV's
// load form (16-byte non-temporal loads), four loads in flight per lane,
// folded into one word per lane; the word is stored only if it is zero
// (so the loads cannot be dropped and almost nothing is written).  It is
// the memory-read ceiling the GEMV is measured against, not a step of the
// computation.
namespace {
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kReadLoads = 4;

__global__ __launch_bounds__(256) void read_bytes_kernel(const uint4* __restrict__ src, size_t quads,
                                                         uint32_t* __restrict__ sink) {
  const size_t base = (static_cast<size_t>(blockIdx.x) * kReadLoads) * 256 + threadIdx.x;
  u32x4_t v[kReadLoads];
#pragma unroll
  for (int i = 0; i < kReadLoads; ++i) {
    const size_t q = base + static_cast<size_t>(i) * 256;
    v[i] = q < quads ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + q)) : u32x4_t{1, 0, 0, 0};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kReadLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (acc == 0u) sink[0] = 1u;
}
}  // namespace

extern "C" int tq_read_bytes(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return TQ_EINVAL;
  if (!tq::tq_aligned(src, 16) || !tq::tq_aligned(sink, 4) || bytes % 16) return TQ_EINVAL;
  const size_t quads = bytes / 16;
  if (quads == 0) return TQ_OK;
  const size_t grid = (quads + 256 * kReadLoads - 1) / (256 * kReadLoads);
  if (grid > 0x7fffffffu) return TQ_ESHAPE;
  hipLaunchKernelGGL(read_bytes_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), quads, sink);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}
