/*
 * tq.h -- C ABI of the ternary-weight (1.58-bit) packed GEMV/GEMM library
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are web pages, cited by title and section):
 *
 *   * Weights take one of three values -c, 0, +c ("TurboQuant-MLX 1.58-bit
 *     build" page, tantan.ink, introduction).  Every 128 consecutive weights
 *     of a row share one FP16 scale that restores the magnitude ("27B model
 *     in 5.9 GB: ternary quantization" page, cosmocat.dev, section 2 (2)).
 *   * Ternary values are coded base 3, 20 per 32-bit integer, about 1.6 bits
 *     per weight (TurboQuant-MLX page, section "Why 1.58 bit did not turn into
 *     gibberish", point 3).  Here digit d = t + 1, and trit k of a row is digit
 *     (k mod 20) of word floor(k / 20), least significant digit first; rows are
 *     packed back to back, so a word may straddle two scale groups; trits past
 *     K are 0 (digit 1).
 *   * The weights were Hadamard-rotated along K before ternarisation and the
 *     activation receives the matching fast transform at inference, at
 *     O(n log n) cost (27B ternary page, section 2 (1)).  Here: Sylvester
 *     Hadamard of order 128 in natural order, scaled by 1/sqrt(128), applied
 *     on every aligned block of 128 (the same blocks as the scale groups).
 *   * y[m][n] = sum_k fp32(s[n][k/128]) * t[n][k] * x'[m][k], x' = H_128 x;
 *     kernels work on the packed format directly and never expand the
 *     weights in memory (27B ternary page, section 2 (3)); with ternary
 *     weights the product reduces to sign tests and adds/subtracts
 *     ("Ternary-Bonsai2-27B vs Qwen3.8-27B-GSQ-RCO" page, nxmr.cn, §1.1).
 *   * MoE: only the routed experts are ternary (256 experts, 8 active per
 *     token); the router gate stays at full precision (TurboQuant-MLX page,
 *     section "Why 1.58 bit...", point 1).
 *
 * Conventions for every entry point:
 *   * Array pointers are DEVICE pointers owned by the caller; no call
 *     allocates, frees or synchronises.  Work is enqueued on `stream`, a
 *     hipStream_t passed as void* (NULL = the default stream), and runs
 *     asynchronously after the call returns.
 *   * Arguments, shapes and descriptors are checked synchronously; a bad one
 *     returns a negative tq_status and enqueues nothing (a corrupted
 *     descriptor is an error, never silent garbage).  A failed kernel
 *     launch returns TQ_EHIP.  No exception crosses the ABI.
 *   * The library keeps no mutable global state beyond a per-thread
 *     message for tq_last_error() and a per-device cache of the compute-unit
 *     count; calls on different streams with different workspaces may run
 *     concurrently.
 *   * Workspaces are caller-owned device memory of tq_workspace_bytes()
 *     bytes; their contents need no initialisation.  Two calls in flight at
 *     the same time must not share a workspace.
 *   * Alignment (checked; TQ_EINVAL otherwise): packed words, scales and
 *     workspaces 16 bytes; activations two elements (8 bytes for TQ_F32, 4
 *     for 16-bit types); FP32 outputs 4 bytes (tq_fwht's 8).  Allocations
 *     from hipMalloc or PyTorch are 256-byte aligned.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_MAGIC 0x30325154u /* "TQ20" */
#define TQ_VERSION 1u
#define TQ_TRITS_PER_WORD 20
#define TQ_GROUP 128

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,       /* null pointer, bad enum, bad flag                    */
  TQ_ESHAPE = -2,       /* size out of range or K not a multiple of 128        */
  TQ_EFORMAT = -3,      /* descriptor magic/version/layout/expert count wrong  */
  TQ_ENOSPACE = -4,     /* workspace too small                                 */
  TQ_EHIP = -5,         /* a HIP launch failed                                 */
  TQ_EUNSUPPORTED = -6  /* valid request the library does not implement        */
} tq_status;

/* Element types of activations / inputs. */
enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2, TQ_F64 = 3 };

/* Word / scale layouts.
 * TQ_LAYOUT_ROWMAJOR: the canonical interchange layout. words[n][ceil(K/20)],
 *   scales[n][K/128] (IEEE fp16 bits), rows contiguous.
 * TQ_LAYOUT_ROW64: the compute layout consumed by tq_gemv / tq_moe_gemv /
 *   tq_gemm.  K is cut into slices of 640 trits (32 words = 8 quads of 4
 *   words = 5 scale groups; 640 is the least common multiple of 20 and 128),
 *   rows into blocks of 64.  Word 32s + 4q + j of row 64b + r is stored at
 *   words[(((s*nb + b)*8 + q)*64 + r)*4 + j], nb = ceil(n/64), and the scale
 *   of group 5s + g of that row at scales[((s*nb + b)*5 + g)*64 + r].  One
 *   16-byte load per lane reads a quad of its row, a 64-lane wavefront reads
 *   1 KiB contiguously, and the 8 KiB of one slice of one row block are
 *   contiguous.
 *   Each word is a base-3 number of 20 trits as in ROWMAJOR, but within
 *   each unit of 160 trits (quads 2u and 2u + 1 of a slice: unit words
 *   wl = 0..7) the trits are grouped into 40 chunks of 4 and reordered:
 *   digits 4j .. 4j + 3 of unit word wl are unit trits 4c .. 4c + 3 with
 *     q = 5 (wl % 2) + j,   c = 8 (q / 2) + 2 (wl / 2) + q % 2,
 *   so that words 2kb and 2kb + 1 hold, in digit order, the trit runs
 *   32i + 8kb .. 32i + 8kb + 7 for i = 0..4 (a 32-trit run of the unit is
 *   spread over the four word pairs and never crosses a scale group).
 *   Rows past n, trits past K and groups past K/128 are padding (zero
 *   trits, so a word of padding only is the all-zero word 1743392200;
 *   scale 0).  tq_unpack inverts the layout exactly. */
enum { TQ_LAYOUT_ROWMAJOR = 0, TQ_LAYOUT_ROW64 = 1 };

/* Flags.
 * TQ_FWHT_FUSED: apply the block-128 transform to the activations inside the
 *   call (the online half of the rotation).  Without it the activations are
 *   taken as already transformed.
 * TQ_ACCUMULATE (tq_gemv): y += W x' instead of y = W x', in a single
 *   launch with device-scope float atomics and no workspace (for example to
 *   add a projection straight into a residual stream); the order in which
 *   the K slices are added is not fixed, so results may differ from run to
 *   run in the last bits.  Without it the call is deterministic.
 *   (tq_moe_gemv): y += the layer's output; deterministic except with at
 *   most 64 (token, slot) pairs and fewer than four tokens, where each
 *   slot's row is added with device atomics (and the slots' combine step is
 *   skipped).  (tq_gemm): Y += ..., deterministic (one workgroup writes
 *   each output). */
enum { TQ_FWHT_FUSED = 1u, TQ_ACCUMULATE = 2u };

/* Operation ids for tq_workspace_bytes. */
enum { TQ_OP_GEMV = 0, TQ_OP_MOE = 1, TQ_OP_GEMM = 2 };

/* Self-describing weight descriptor.  For MoE, num_experts > 1 and expert e's
 * words start at words + e * tq_layout_words(n, k, layout) (likewise scales). */
typedef struct {
  uint32_t magic;       /* TQ_MAGIC   */
  uint32_t version;     /* TQ_VERSION */
  int32_t n;            /* rows = outputs                         */
  int32_t k;            /* columns = inputs, a multiple of 128    */
  int32_t num_experts;  /* 1 for a dense layer                    */
  int32_t layout;       /* TQ_LAYOUT_*                            */
  const uint32_t *words;
  const uint16_t *scales;
} tq_weights;

/* ---- sizes (host only, no GPU work) ------------------------------------ */
/* ceil(k / 20). */
size_t tq_words_per_row(int k);
/* Algorithmic packed bytes of one n x k matrix: 4*n*ceil(k/20) + 2*n*(k/128)
 * (the canonical layout's size; ROW64 adds only padding). */
size_t tq_packed_bytes(int n, int k);
/* Number of uint32 words / uint16 scales a buffer of the given layout holds
 * for one n x k matrix (padding included).  0 for an invalid request. */
size_t tq_layout_words(int n, int k, int layout);
size_t tq_layout_scales(int n, int k, int layout);

/* ---- offline conversion ------------------------------------------------ */
/* Rotate and ternarise W (TurboQuant-MLX introduction; 27B ternary page,
 * sections 2 (1) and 2 (2)).  w: [n][k] row-major, w_dtype TQ_F64 or TQ_F32.
 * For every row and group of 128: w' = H_128 applied along K, computed in
 * FP64; gamma = mean |w'|; t = sign(w') where |w'| > gamma/2, else 0 (an
 * exact tie gives 0); s = fp16(gamma) rounded to nearest-even once from FP64
 * (gamma == 0 gives t = 0, s = 0).  Outputs trits int8 [n][k] and scales
 * uint16 (fp16 bits) [n][k/128], both row-major.  k % 128 == 0. */
int tq_quantize(const void *w, int w_dtype, int n, int k, int8_t *trits,
                uint16_t *scales, void *stream);

/* Base-3 pack (TurboQuant-MLX, "Why 1.58 bit...", point 3): trits int8
 * [n][k] row-major, values in {-1,0,1} (a precondition: other values give
 * unspecified words), into `words` of tq_layout_words(n,k,layout) uint32 in
 * the requested layout, pads included.  Any k >= 1 for ROWMAJOR; ROW64
 * needs k % 128 == 0. */
int tq_pack(const int8_t *trits, int n, int k, int layout, uint32_t *words,
            void *stream);

/* Re-lay a row-major scale array [n][k/128] into `layout` (ROWMAJOR copies,
 * ROW64 interleaves as described above and zero-fills padded rows). */
int tq_pack_scales(const uint16_t *scales, int n, int k, int layout,
                   uint16_t *scales_out, void *stream);

/* Inverse of tq_pack (test export): words in `layout` -> trits int8 [n][k]
 * row-major, t = digit - 1. */
int tq_unpack(const uint32_t *words, int n, int k, int layout, int8_t *trits,
              void *stream);

/* ---- online path ------------------------------------------------------- */
/* x_rot[m][k] = H_128 x[m][k] on every aligned block of 128 (27B ternary
 * page, section 2 (1)); x: [m][k] row-major of x_dtype (F32/BF16/F16),
 * x_rot FP32.  k % 128 == 0. */
int tq_fwht(const void *x, int x_dtype, int m, int k, float *x_rot,
            void *stream);

/* Decode GEMV, 1 <= m <= 8 activation rows:
 * y[m][n] = sum_k fp32(s[n][k/128]) t[n][k] x'[m][k], x' = H_128 x if flags
 * has TQ_FWHT_FUSED else x (with TQ_ACCUMULATE: y += ...).  w: ROW64
 * layout, num_experts == 1.  x: [m][k] of x_dtype (F32/BF16/F16); y: FP32
 * [m][n].  m == 1 accumulates in FP32 throughout; m >= 2 multiplies fp16
 * trit codes by x' split into two fp16 parts (about 22 significant bits,
 * after a power-of-two scaling per activation row and 640-trit slice) with
 * FP32 accumulation.  Unless
 * TQ_ACCUMULATE is set, needs a workspace of tq_workspace_bytes(TQ_OP_GEMV,
 * w, m, 0) bytes (0 when K <= 640).  One launch, plus a short reduction
 * launch when K > 640 and TQ_ACCUMULATE is not set. */
int tq_gemv(const tq_weights *w, const void *x, int x_dtype, int m, float *y,
            unsigned flags, void *workspace, size_t ws_bytes, void *stream);

/* Full-precision router (TurboQuant-MLX, point 1): per token, p = softmax of
 * logits[t][0..e) in FP32, the topk largest p (ties to the lower id), and
 * weights p / (sum of the chosen p).  ids int32 [t][topk], weights FP32
 * [t][topk], in decreasing p.  1 <= topk <= 32, e <= 1024. */
int tq_moe_route(const float *logits, int t, int e, int topk, int32_t *ids,
                 float *weights, void *stream);

/* Routed ternary expert MLP (TurboQuant-MLX, point 1):
 *   for every token i and slot j with e = expert_ids[i][j]:
 *     g||u = W_gu[e] . H x_i    (W_gu rows [0, I) gate, [I, 2I) up)
 *     h    = silu(g) * u        (silu(z) = z / (1 + exp(-z)))
 *     o    = W_dn[e] . H h
 *   y[i] = sum_j route_w[i][j] * o   (TQ_ACCUMULATE: y[i] += ...).
 * w_gate_up: E experts of n = 2I, k = Hd; w_down: E experts of n = Hd,
 * k = I; both ROW64 (I % 64 == 0, Hd and I multiples of 128).  x: [t][Hd]
 * of x_dtype; y FP32 [t][Hd].  The expert products use the m >= 2 decode
 * GEMV arithmetic (fp16 codes, x' and H h as two fp16 parts, FP32
 * accumulation).  With t * topk <= 64 every (token, slot) pair is its own
 * one-row product (two launches; below four tokens the last slot of a token
 * to finish adds the slots in slot order, from four tokens on one
 * workgroup per token and row block adds them); otherwise the pairs are
 * grouped by expert and an expert's tokens go 8 at a time (four launches;
 * E <= 1024, else TQ_EUNSUPPORTED).  y is deterministic either way.  Only the experts that receive tokens are read.  Ids outside
 * [0, E) are an error detected on the device: such slots contribute
 * nothing.  Needs tq_workspace_bytes(TQ_OP_MOE, w_gate_up, t, topk) bytes of
 * workspace, which calls that overlap in time must not share. */
int tq_moe_gemv(const tq_weights *w_gate_up, const tq_weights *w_down,
                const void *x, int x_dtype, int t, int topk,
                const int32_t *expert_ids, const float *route_w, float *y,
                unsigned flags, void *workspace, size_t ws_bytes, void *stream);

/* Prefill GEMM: Y[m][n] = sum_k fp32(s[n][k/128]) t[n][k] x'[m][k] for any
 * m >= 1 on the matrix cores.  x' (FP32 after the optional transform) is
 * split into an fp16 high part and an fp16 remainder, and each is
 * multiplied by the exact fp16 weights s*t decoded from the packed words
 * (into registers), accumulating in FP32.  w: ROW64, num_experts == 1.  Needs
 * tq_workspace_bytes(TQ_OP_GEMM, w, m, 0) bytes of workspace. */
int tq_gemm(const tq_weights *w, const void *x, int x_dtype, int m, float *y,
            unsigned flags, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes an operation needs (0 when it needs none; SIZE_MAX for an
 * invalid request).  m_or_t: activation rows (GEMV/GEMM) or tokens (MoE). */
size_t tq_workspace_bytes(int op, const tq_weights *w, int m_or_t, int topk);

/* Static message for a tq_status value. */
const char *tq_strerror(int status);

/* Description of the last HIP failure (TQ_EHIP) seen by a tq_* call on the
 * calling host thread: the entry point and HIP's error name and text; ""
 * if there was none.  Valid until the next failing call on that thread. */
const char *tq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
