// Prefill GEMM on packed ternary weights:
//   Y[m][n] = sum_k fp32(s[n][k/128]) t[n][k] x'[m][k],  x' = H_128 x.
//
// Two launches on the caller's stream:
//   1. prep: block-128 transform of every activation row (FP32), split into
//      hi = fp16(x') and lo = fp16(x' - hi), written to the workspace padded
//      to whole tiles (zeros outside M x K).  hi + lo carries ~22 bits of x'.
//   2. gemm: each workgroup computes a 64 x 256 tile of Y on the matrix cores
//      (v_mfma_f32_32x32x16_f16).  Per 160-trit K step (2 quads of packed
//      words per weight row) the workgroup decodes its 256 weight rows into
//      fp16 values s*t, which are exact in fp16 because t is in {-1, 0, 1},
//      so the per-group scale is applied before the product and no separate
//      FP32 scale pass is needed; the activation tile (hi and lo) is staged
//      next to it in LDS.  Both parts are multiplied and accumulated in FP32.
//      The next step's words, scales and activations are loaded into
//      registers while the current step's MFMAs run.
// Weights stream once per 64-row M tile; tiles are ordered so that all N
// tiles of one M tile run on one XCD, keeping that activation tile (64 x K x
// 4 bytes) in the XCD's L2.
#include "tq_internal.h"

#include <limits.h>

using namespace tq;

namespace {

constexpr int BM = 64;          // rows of Y per workgroup
constexpr int BN = 256;         // columns of Y per workgroup (4 wavefronts x 64)
constexpr int BK = 160;         // trits per K step = 2 quads = 8 words
constexpr int LDA = BK + 8;     // padded LDS row stride (halves) against bank conflicts
constexpr int kThreads = 256;

typedef float float16_t __attribute__((ext_vector_type(16)));

#define TQ_LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// ------------------------------------------------------------------ prep ---
// One wavefront per (row, block of 128) of the padded [mpad][kpad] output.
__global__ __launch_bounds__(256) void gemm_prep_kernel(const void* __restrict__ x, int dtype, int m, int k,
                                                        int mpad, int kpad, int fused, _Float16* __restrict__ xh,
                                                        _Float16* __restrict__ xl) {
  const int bpr = kpad / 128;
  const long long job = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (job >= static_cast<long long>(mpad) * bpr) return;
  const int lane = threadIdx.x & 63;
  const int row = static_cast<int>(job / bpr);
  const int kb = static_cast<int>(job % bpr) * 128;
  float v0 = 0.0f, v1 = 0.0f;
  if (row < m && kb < k) {
    load_act2(x, dtype, static_cast<size_t>(row) * k + kb + 2 * lane, v0, v1);
    if (fused) wave_fwht128<float>(v0, v1, lane, kInvSqrt128);
  }
  const _Float16 h0 = static_cast<_Float16>(v0), h1 = static_cast<_Float16>(v1);
  const _Float16 l0 = static_cast<_Float16>(v0 - static_cast<float>(h0));
  const _Float16 l1 = static_cast<_Float16>(v1 - static_cast<float>(h1));
  const size_t o = static_cast<size_t>(row) * kpad + kb + 2 * lane;
  half2_t hh = {h0, h1}, ll = {l0, l1};
  *reinterpret_cast<half2_t*>(xh + o) = hh;
  *reinterpret_cast<half2_t*>(xl + o) = ll;
}

struct GemmArgs {
  const uint4* words;
  const uint16_t* scales;
  const _Float16* xh;
  const _Float16* xl;
  float* y;
  int m, n, k, kpad, nb, groups, mtiles, ntiles, steps, xcd_map;
};

// Tile of this workgroup: all N tiles of an M tile on one XCD (workgroups
// are dispatched to the 8 XCDs round-robin by id) when M tiles divide by 8.
__device__ __forceinline__ void tile_of(const GemmArgs& a, int& mt, int& nt) {
  const int b = blockIdx.x;
  if (a.xcd_map) {
    const int xcd = b & 7, j = b >> 3;
    mt = xcd + 8 * (j / a.ntiles);
    nt = j % a.ntiles;
  } else {
    mt = b / a.ntiles;
    nt = b % a.ntiles;
  }
}

struct Prefetch {
  uint4 w[2];       // two quads of this thread's weight row
  float s[2];       // scales of the (at most two) groups the step touches
  uint4 ah[5];      // activation hi: 64 rows x 160 halves = 1280 uint4 / 256 threads
  uint4 al[5];
};

__device__ __forceinline__ void prefetch(const GemmArgs& a, int mt, int nt, int step, Prefetch& p) {
  const int tid = threadIdx.x;
  // weights: row n of the tile = tid
  int row = nt * BN + tid;
  if (row > a.nb * 64 - 1) row = a.nb * 64 - 1;
  const int k0 = step * BK;
  const int slice = k0 / kSliceTrits;
  const int q0 = (k0 % kSliceTrits) / 80;  // 0, 2, 4, 6
  const uint4* wp = a.words + row64_quad_base(slice, row >> 6, a.nb) + (row & 63);
  p.w[0] = wp[q0 * 64];
  p.w[1] = wp[(q0 + 1) * 64];
  const int g0 = k0 / TQ_GROUP;
  const int g1 = min(g0 + 1, (a.groups + kSliceGroups - 1) / kSliceGroups * kSliceGroups - 1);
  p.s[0] = f16_to_f32(a.scales[row64_scale_index(row, g0, a.nb)]);
  p.s[1] = f16_to_f32(a.scales[row64_scale_index(row, g1, a.nb)]);
  // activations: 64 rows x 160 halves = 64 x 20 uint4; thread covers 5 of them
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int idx = tid + i * kThreads;  // 0..1279
    const int r = idx / 20, c = idx % 20;
    const size_t off = static_cast<size_t>(mt * BM + r) * a.kpad + k0 + c * 8;
    p.ah[i] = *reinterpret_cast<const uint4*>(a.xh + off);
    p.al[i] = *reinterpret_cast<const uint4*>(a.xl + off);
  }
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As_h[BM * LDA];
  __shared__ __attribute__((aligned(16))) _Float16 As_l[BM * LDA];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[BN * LDA];
  __shared__ uint32_t codes_lo[81], codes_hi[81];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int mt, nt;
  tile_of(a, mt, nt);
  if (tid < 81) {
    uint16_t h[4];
    int c = tid;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(static_cast<float>(c % 3) - 1.0f));
      c /= 3;
    }
    codes_lo[tid] = h[0] | (static_cast<uint32_t>(h[1]) << 16);
    codes_hi[tid] = h[2] | (static_cast<uint32_t>(h[3]) << 16);
  }
  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  Prefetch p;
  prefetch(a, mt, nt, 0, p);
  for (int step = 0; step < a.steps; ++step) {
    TQ_LDS_BARRIER();  // previous step's fragments have been read
    // activations -> LDS
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / 20, c = idx % 20;
      *reinterpret_cast<uint4*>(&As_h[r * LDA + c * 8]) = p.ah[i];
      *reinterpret_cast<uint4*>(&As_l[r * LDA + c * 8]) = p.al[i];
    }
    // weights -> fp16 s*t in LDS (row tid, 160 trits)
    {
      const int k0 = step * BK;
      const int gsplit = (k0 / TQ_GROUP + 1) * TQ_GROUP - k0;  // first K offset in the second group
      const _Float16 sa = static_cast<_Float16>(p.s[0]), sb = static_cast<_Float16>(p.s[1]);
      _Float16* brow = &Bs[tid * LDA];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t wv[4] = {p.w[q].x, p.w[q].y, p.w[q].z, p.w[q].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t o[5];
          word_offsets_s<2, false>(wv[j], o);  // no inline asm next to MFMAs
#pragma unroll
          for (int h = 0; h < 5; ++h) {
            const int kk = 4 * row64_chunk(4 * q + j, h);  // trit offset in the 160-trit unit
            const _Float16 sc = kk < gsplit ? sa : sb;
            const half2_t s2 = {sc, sc};
            const half2_t lo = __builtin_bit_cast(
                half2_t, *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(codes_lo) + o[h]));
            const half2_t hi = __builtin_bit_cast(
                half2_t, *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(codes_hi) + o[h]));
            const half2_t vlo = lo * s2, vhi = hi * s2;
            uint2 pk;
            pk.x = __builtin_bit_cast(uint32_t, vlo);
            pk.y = __builtin_bit_cast(uint32_t, vhi);
            *reinterpret_cast<uint2*>(&brow[kk]) = pk;
          }
        }
      }
    }
    if (step + 1 < a.steps) prefetch(a, mt, nt, step + 1, p);
    TQ_LDS_BARRIER();
    // MFMA: wavefront w covers columns [64w, 64w+64) of the tile, all 64 rows.
    const int li = lane & 31, lk = (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      half8_t ah[2], al[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = *reinterpret_cast<const half8_t*>(&As_h[(i * 32 + li) * LDA + kk + lk]);
        al[i] = *reinterpret_cast<const half8_t*>(&As_l[(i * 32 + li) * LDA + kk + lk]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const half8_t*>(&Bs[(wave * 64 + j * 32 + li) * LDA + kk + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bf[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
  }
  // store: acc[i][j][v] is row 8*(v/4) + 4*(lane/32) + v%4 of the 32x32 block
  // (i, j), column lane%32.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = nt * BN + wave * 64 + j * 32 + (lane & 31);
      if (col >= a.n) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = mt * BM + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
        if (row < a.m) a.y[static_cast<size_t>(row) * a.n + col] = acc[i][j][v];
      }
    }
}

struct GemmPlan {
  int mpad, kpad, mtiles, ntiles, steps;
  size_t xh_bytes, total;
};

GemmPlan plan_gemm(int n, int k, int m) {
  GemmPlan p;
  p.mtiles = (m + BM - 1) / BM;
  p.ntiles = (n + BN - 1) / BN;
  p.mpad = p.mtiles * BM;
  p.steps = (k + BK - 1) / BK;
  p.kpad = p.steps * BK;
  if (p.kpad % 128) p.kpad = (p.kpad + 127) / 128 * 128;  // prep works in blocks of 128
  p.xh_bytes = (static_cast<size_t>(p.mpad) * p.kpad * 2 + 255) & ~static_cast<size_t>(255);
  p.total = 2 * p.xh_bytes;
  return p;
}

}  // namespace

size_t tq_gemm_workspace(int n, int k, int m) { return plan_gemm(n, k, m).total; }

extern "C" int tq_gemm(const tq_weights* w, const void* x, int x_dtype, int m, float* y, unsigned flags,
                       void* workspace, size_t ws_bytes, void* stream) {
  int st = tq_check_weights(w, 1);
  if (st != TQ_OK) return st;
  if (!x || !y || !workspace) return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16 && x_dtype != TQ_F16) return TQ_EINVAL;
  if (flags & ~static_cast<unsigned>(TQ_FWHT_FUSED)) return TQ_EINVAL;
  if (m < 1) return TQ_ESHAPE;
  const GemmPlan p = plan_gemm(w->n, w->k, m);
  if (ws_bytes < p.total) return TQ_ENOSPACE;
  if (static_cast<long long>(p.mtiles) * p.ntiles > INT_MAX) return TQ_ESHAPE;
  _Float16* xh = static_cast<_Float16*>(workspace);
  _Float16* xl = reinterpret_cast<_Float16*>(static_cast<char*>(workspace) + p.xh_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long jobs = static_cast<long long>(p.mpad) * (p.kpad / 128);
  hipLaunchKernelGGL(gemm_prep_kernel, dim3(static_cast<unsigned>((jobs + 3) / 4)), dim3(256), 0, s, x, x_dtype, m,
                     w->k, p.mpad, p.kpad, (flags & TQ_FWHT_FUSED) ? 1 : 0, xh, xl);
  TQ_LAUNCH_CHECK();
  GemmArgs a;
  a.words = reinterpret_cast<const uint4*>(w->words);
  a.scales = w->scales;
  a.xh = xh;
  a.xl = xl;
  a.y = y;
  a.m = m;
  a.n = w->n;
  a.k = w->k;
  a.kpad = p.kpad;
  a.nb = row_blocks(w->n);
  a.groups = w->k / TQ_GROUP;
  a.mtiles = p.mtiles;
  a.ntiles = p.ntiles;
  a.steps = p.steps;
  a.xcd_map = (p.mtiles % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(gemm_kernel, dim3(p.mtiles * p.ntiles), dim3(kThreads), 0, s, a);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}
