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
 *   * Array pointers are DEVICE pointers owned by the caller (except the
 *     host count of tq_moe_bad_ids); no call allocates or frees, and none
 *     synchronises except tq_moe_bad_ids.  Work is enqueued on `stream`, a
 *     hipStream_t passed as void* (NULL = the default stream), and runs
 *     asynchronously after the call returns.
 *   * Arguments, shapes and descriptors are checked synchronously; a bad one
 *     returns a negative tq_status and enqueues nothing (a corrupted
 *     descriptor is an error, never silent garbage).  A failed kernel
 *     launch returns TQ_EHIP.  No exception crosses the ABI.
 *   * The library keeps no mutable global state beyond a per-thread
 *     message for tq_last_error(), a per-device cache of the compute-unit
 *     count, and tq_gemv_noalloc's per-device scratch array and its address;
 *     calls on different streams with different workspaces may run
 *     concurrently.
 *   * Workspaces are caller-owned device memory of tq_workspace_bytes()
 *     bytes; their contents need no initialisation.  Two calls in flight at
 *     the same time must not share a workspace.
 *   * Alignment (checked; TQ_EINVAL otherwise): packed words, scales and
 *     workspaces 16 bytes; activations two elements (8 bytes for TQ_F32, 4
 *     for 16-bit types); FP32 outputs 4 bytes (tq_fwht's 8); offline
 *     inputs and outputs to their element size (tq_quantize's trits 2
 *     bytes).  Allocations from hipMalloc or PyTorch are 256-byte aligned.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_MAGIC 0x30325154u /* "TQ20" */
#define TQ_VERSION 2u
#define TQ_TRITS_PER_WORD 20
#define TQ_GROUP 128      /* default weights per scale; 64 is the other group size */
#define TQ_BITS_PER_WORD 32 /* binary variant: one sign bit per weight */
/* Largest n, k or activation row count m that any call takes (2^30): every
 * row, slice and word index the kernels form then fits an int.  Larger
 * sizes are TQ_ESHAPE, and the size queries return 0 for them. */
#define TQ_MAX_DIM (1 << 30)

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,       /* null pointer, bad enum, bad flag                    */
  TQ_ESHAPE = -2,       /* size out of range (above TQ_MAX_DIM, or not
                           positive) or K not a multiple of 128              */
  TQ_EFORMAT = -3,      /* descriptor magic/version/layout/expert count wrong  */
  TQ_ENOSPACE = -4,     /* workspace too small                                 */
  TQ_EHIP = -5,         /* a HIP launch failed                                 */
  TQ_EUNSUPPORTED = -6, /* valid request the library does not implement        */
  TQ_EDATA = -7         /* input values out of range (reported by the checking
                           calls: trits outside {-1,0,1}, expert ids outside
                           [0, E))                                             */
} tq_status;

/* Element types of activations / inputs. */
enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2, TQ_F64 = 3 };

/* Formats.  Two parameters describe the weights:
 *   levels 3 (ternary {-c,0,+c}, the path's format): base-3 words, 20 per
 *     uint32, as above;
 *   levels 2 (binary {-c,+c}, the pure 1-bit variant the TurboQuant-MLX page
 *     compares against, point 3): one sign bit per weight, 32 per uint32,
 *     bit i of word w is weight 32w + i, 1 for +c;
 *   group 128 (27B ternary page, section 2 (2)) or 64 (the "-g64" model id
 *     on the TurboQuant-MLX page): weights per FP16 scale.  The rotation is
 *     block-128 either way; K stays a multiple of 128.
 *
 * Word / scale layouts.
 * TQ_LAYOUT_ROWMAJOR: the canonical interchange layout. words[n][ceil(K/20)]
 *   (binary: ceil(K/32)), scales[n][K/group] (IEEE fp16 bits), rows
 *   contiguous.
 * TQ_LAYOUT_ROW64: the compute layout consumed by tq_gemv / tq_moe_gemv /
 *   tq_gemm.  K is cut into slices of 640 trits (32 words = 8 quads of 4
 *   words; 640 is the least common multiple of 20 and 128), rows into
 *   blocks of 64.  Word 32s + 4q + j of row 64b + r is stored at
 *   words[(((s*nb + b)*8 + q)*64 + r)*4 + j], nb = ceil(n/64).  A slice has
 *   G = 640/group scale groups (5 at group 128, 10 at group 64); the scale
 *   of group Gs + g of that row is at scales[((s*nb + b)*G + g)*64 + r].
 *   One 16-byte load per lane reads a quad of its row, a 64-lane wavefront
 *   reads 1 KiB contiguously, and the 8 KiB of one slice of one row block
 *   are contiguous.
 *   Binary words (levels 2): a slice is 640 weights = 20 words = 5 quads;
 *   word 20s + 4q + j of row 64b + r is at words[(((s*nb + b)*5 + q)*64 + r)*4
 *   + j], bits in ROWMAJOR order (no reordering); scales as above.
 *   Each word is a base-3 number of 20 trits as in ROWMAJOR, but within
 *   each unit of 160 trits (quads 2u and 2u + 1 of a slice: unit words
 *   wl = 0..7) the trits are grouped into 40 chunks of 4 and reordered:
 *   digits 4j .. 4j + 3 of unit word wl are unit trits 4c .. 4c + 3 with
 *     q = 5 (wl % 2) + j,   c = 8 (q / 2) + 2 (wl / 2) + q % 2,
 *   so that words 2kb and 2kb + 1 hold, in digit order, the trit runs
 *   32i + 8kb .. 32i + 8kb + 7 for i = 0..4 (a 32-trit run of the unit is
 *   spread over the four word pairs and never crosses a scale group).
 *   Rows past n, trits past K and groups past K/group are padding (zero
 *   trits, so a word of padding only is the all-zero word 1743392200;
 *   binary padding bits are 0; scale 0).  tq_unpack inverts the layout
 *   exactly. */
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
 *   each output).
 * TQ_MOE_ONE_LAUNCH (tq_moe_gemv, at most 64 (token, slot) pairs and an
 *   intermediate size of at most 2560): the whole expert MLP in a single
 *   launch.  The last workgroup of each (token, slot) pair to finish its
 *   gate/up share runs that pair's down projection, and the last slot of a
 *   token combines the slots in slot order (no workgroup waits for
 *   another).  Its arrival counters reset themselves, so a workspace used
 *   with this flag must be zero-filled before its first use (each call
 *   leaves the counters zero).  TQ_EUNSUPPORTED for larger requests.
 * TQ_FAST_F16 (tq_gemm): x' (after its power-of-two scaling per row) as a
 *   single fp16 part instead of hi + lo: about 2^-12 relative rounding per
 *   activation, a relative L2 error near 3e-4 on Gaussian activations
 *   (within the path's 1e-3 bound, against about 1e-7 for the default),
 *   for half the matrix-core work and weight re-reads (128 tokens per
 *   workgroup instead of 64). */
enum { TQ_FWHT_FUSED = 1u, TQ_ACCUMULATE = 2u, TQ_MOE_ONE_LAUNCH = 4u, TQ_FAST_F16 = 8u };

/* Operation ids for tq_workspace_bytes. */
enum { TQ_OP_GEMV = 0, TQ_OP_MOE = 1, TQ_OP_GEMM = 2 };

/* Self-describing weight descriptor.  For MoE, num_experts > 1 and expert e's
 * words start at words + e * tq_layout_words(n, k, layout, levels) (likewise
 * scales with tq_layout_scales(n, k, layout, group)). */
typedef struct {
  uint32_t magic;       /* TQ_MAGIC   */
  uint32_t version;     /* TQ_VERSION */
  int32_t n;            /* rows = outputs                         */
  int32_t k;            /* columns = inputs, a multiple of 128    */
  int32_t num_experts;  /* 1 for a dense layer                    */
  int32_t layout;       /* TQ_LAYOUT_*                            */
  int32_t group;        /* weights per scale: 128 or 64           */
  int32_t levels;       /* 3: ternary; 2: binary                  */
  const uint32_t *words;
  const uint16_t *scales;
} tq_weights;

/* ---- sizes (host only, no GPU work) ------------------------------------ */
/* ceil(k / 20): words per row at 20 trits per 32-bit word (TurboQuant-MLX
 * page, "Why 1.58 bit did not turn into gibberish", point 3). */
size_t tq_words_per_row(int k);
/* Algorithmic packed bytes of one n x k matrix: 4*n*ceil(k/20) + 2*n*(k/128),
 * the base-3 words (TurboQuant-MLX page, point 3) plus one FP16 scale per
 * 128 weights (27B ternary page, section 2 (2)); the canonical layout's
 * size (ROW64 adds only padding).  0 for n <= 0 or k <= 0. */
size_t tq_packed_bytes(int n, int k);
/* Algorithmic bytes of one n x k matrix in any format: words (levels 3:
 * 4*n*ceil(k/20); levels 2: 4*n*ceil(k/32)) plus 2*n*(k/group).  0 for an
 * invalid request (k not a multiple of group, group not 64 or 128, levels
 * not 2 or 3). */
size_t tq_format_bytes(int n, int k, int group, int levels);
/* Number of uint32 words a buffer of the given layout holds for one n x k
 * matrix of `levels` (padding included), and of uint16 scales for `group`.
 * 0 for an invalid request. */
size_t tq_layout_words(int n, int k, int layout, int levels);
size_t tq_layout_scales(int n, int k, int layout, int group);

/* ---- offline conversion ------------------------------------------------ */
/* Rotate and ternarise W (TurboQuant-MLX introduction; 27B ternary page,
 * sections 2 (1) and 2 (2)).  w: [n][k] row-major, w_dtype TQ_F64 or TQ_F32.
 * w' = H_128 applied along K on every block of 128, computed in FP64; then
 * for every row and group of `group` (128 or 64) weights: gamma = mean |w'|,
 * s = fp16(gamma) rounded to nearest-even once from FP64, and
 *   levels 3: t = sign(w') where |w'| > gamma/2, else 0 (an exact tie gives
 *             0; gamma == 0 gives t = 0, s = 0);
 *   levels 2: t = +1 where w' >= 0, else -1 (the binary variant).
 * Outputs t int8 [n][k] and scales uint16 (fp16 bits) [n][k/group], both
 * row-major.  k % 128 == 0. */
int tq_quantize(const void *w, int w_dtype, int n, int k, int group, int levels,
                int8_t *trits, uint16_t *scales, void *stream);

/* Pack (TurboQuant-MLX, "Why 1.58 bit...", point 3): t int8 [n][k]
 * row-major into `words` of tq_layout_words(n,k,layout,levels) uint32 in the
 * requested layout, pads included.
 *   levels 3: base-3 words of 20 trits, values in {-1,0,1}; a value outside
 *     is a caller error and is packed as 0, so every word stays a valid
 *     base-3 number below 3^20;
 *   levels 2: 32 sign bits per word, values in {-1,+1}; any other value is
 *     a caller error and is packed as +1 (the sign rule's side for 0).
 * tq_pack_checked also counts such values.  Any k >= 1 for ROWMAJOR; ROW64
 * needs k % 128 == 0.  Alignment: words 4 bytes. */
int tq_pack(const int8_t *trits, int n, int k, int layout, int levels,
            uint32_t *words, void *stream);

/* tq_pack plus a count of the input values outside the format's set: `bad`
 * is one device int32 that the call overwrites (two launches: it is
 * cleared, then every bad value adds one).  For offline conversion that must
 * not pack garbage silently (27B ternary page, section 2 (3): a runtime
 * that loads a format it does not understand outputs garbage without a
 * word).  Read *bad after the stream reaches this work. */
int tq_pack_checked(const int8_t *trits, int n, int k, int layout, int levels,
                    uint32_t *words, int32_t *bad, void *stream);

/* Re-lay a row-major scale array [n][k/group] into `layout` (ROWMAJOR
 * copies, ROW64 interleaves as described above and zero-fills padded rows
 * and groups). */
int tq_pack_scales(const uint16_t *scales, int n, int k, int layout, int group,
                   uint16_t *scales_out, void *stream);

/* Inverse of tq_pack (test export; the base-3 digits of TurboQuant-MLX,
 * point 3, or the sign bits of the binary variant, read back): words in
 * `layout` -> t int8 [n][k] row-major (t = digit - 1, or 2 bit - 1).
 * Alignment: words 4 bytes. */
int tq_unpack(const uint32_t *words, int n, int k, int layout, int levels,
              int8_t *trits, void *stream);

/* ---- online path ------------------------------------------------------- */
/* x_rot[m][k] = H_128 x[m][k] on every aligned block of 128 (27B ternary
 * page, section 2 (1)); x: [m][k] row-major of x_dtype (F32/BF16/F16),
 * x_rot FP32.  k % 128 == 0. */
int tq_fwht(const void *x, int x_dtype, int m, int k, float *x_rot,
            void *stream);

/* Decode GEMV, 1 <= m <= 8 activation rows (the decode-time product of the
 * 27B ternary page, sections 2 (1)-(3): the packed weights, their FP16
 * group scales and the matching transform of the activation; adds and
 * subtracts only, "Ternary-Bonsai2-27B vs ..." page, section 1.1):
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

/* tq_gemv for callers that cannot allocate device memory, not even a
 * workspace: code under HIP graph capture where allocation is forbidden,
 * tight serving loops, harnesses that forbid it.  Same arguments, result and
 * flags as tq_gemv without the workspace: the slice partial sums of the
 * default (deterministic) mode go to a library-owned device array of
 * 16 MiB per GPU (held from the library's loading until the process ends),
 * so the call allocates nothing.  Returns TQ_ENOSPACE, before any GPU work,
 * when the partial sums (4 * ceil(k/640) * m * 64 * ceil(n/64) bytes) exceed
 * 16 MiB; TQ_ACCUMULATE needs no array.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU race (for example on
 * two streams); serialise them.  Nothing in the array needs to start at
 * zero (each call writes every element it reads). */
int tq_gemv_noalloc(const tq_weights *w, const void *x, int x_dtype, int m,
                    float *y, unsigned flags, void *stream);

/* Full-precision router (TurboQuant-MLX, point 1): per token, p = softmax of
 * logits[t][0..e) in FP32, the topk largest p (ties to the lower id), and
 * weights p / (sum of the chosen p).  ids int32 [t][topk], weights FP32
 * [t][topk], in decreasing p.  1 <= topk <= 32, e <= 1024.  Alignment:
 * logits, ids and weights 4 bytes. */
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
 * E <= 1024, else TQ_EUNSUPPORTED).  y is deterministic either way.  Only
 * the experts that receive tokens are read.  Ids outside [0, E) are a caller
 * error detected on the device: such slots contribute nothing, and the
 * number of them is left in the workspace for tq_moe_bad_ids.  Needs
 * tq_workspace_bytes(TQ_OP_MOE, w_gate_up, t, topk) bytes of workspace,
 * which calls that overlap in time must not share. */
int tq_moe_gemv(const tq_weights *w_gate_up, const tq_weights *w_down,
                const void *x, int x_dtype, int t, int topk,
                const int32_t *expert_ids, const float *route_w, float *y,
                unsigned flags, void *workspace, size_t ws_bytes, void *stream);

/* Number of (token, slot) entries whose expert id was outside [0, E) in the
 * last tq_moe_gemv that used this workspace (the router's choice is taken
 * as input; a bad id must not vanish silently, 27B ternary page, section
 * 2 (3)).  Copies the count to *count (host memory) and WAITS for `stream`
 * (the one call in the library that synchronises).  Returns TQ_EDATA if the
 * count is nonzero, TQ_OK if it is zero. */
int tq_moe_bad_ids(const void *workspace, size_t ws_bytes, int32_t *count,
                   void *stream);

/* Prefill GEMM (the same product as tq_gemv for a whole prompt at once;
 * kernels that work on the packed format directly, 27B ternary page,
 * section 2 (3)): Y[m][n] = sum_k fp32(s[n][k/128]) t[n][k] x'[m][k] for any
 * m >= 1 on the matrix cores.  x' (FP32 after the optional transform) is
 * scaled by a power of two per row (max |x'| 2^e in [2^13, 2^14), so any
 * activation scale stays in fp16's normal range; undone on the output),
 * split into an fp16 high part and an fp16 remainder, and each is
 * multiplied by the exact fp16 weights s*t decoded from the packed words
 * (into registers), accumulating in FP32.  w: ROW64, num_experts == 1.  Needs
 * tq_workspace_bytes(TQ_OP_GEMM, w, m, 0) bytes of workspace. */
int tq_gemm(const tq_weights *w, const void *x, int x_dtype, int m, float *y,
            unsigned flags, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes an operation needs (0 when it needs none; SIZE_MAX for an
 * invalid request).  m_or_t: activation rows (GEMV/GEMM) or tokens (MoE). */
size_t tq_workspace_bytes(int op, const tq_weights *w, int m_or_t, int topk);

/* Memory-read reference (a measurement aid, not a step of the product):
 * reads `bytes` bytes of `src` once with the decode GEMV's load form
 * (16-byte non-temporal loads, one launch) and writes at most one word to
 * *sink (device memory).  Timing it on the same bytes as one GEMV launch
 * gives the read ceiling that launch size allows.  src 16-byte aligned,
 * bytes a multiple of 16. */
int tq_read_bytes(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* ---- KV-cache quantiser (TurboQuant) ----------------------------------- *
 * A second workload beside the ternary weights: compressing the attention
 * KV cache ("Mac users can use TurboQuant in oMLX, with Gemma-4-31B" page,
 * aitntnews, section "What TurboQuant is and what problem it solves"): each
 * K or V vector is rotated by a random orthogonal matrix and kept in polar
 * form, a high-precision radius and a quantised direction (PolarQuant); a
 * 1-bit Johnson-Lindenstrauss projection of the direction's residual (QJL)
 * removes the bias of key inner products; no per-block scale is stored.
 * Decoding costs a rotation and table lookups (section "Why these results").
 * Readings where the page is silent:
 *   * vectors have TQ_KV_DIM = 128 coordinates; Pi = H diag(sigma), H the
 *     Sylvester Hadamard of order 128 scaled by 1/sqrt(128), sigma = signs;
 *   * r = |x| stored as fp16 (one rounding); u = Pi x / r (0 if r = 0);
 *   * each coordinate of u takes the nearest level of the m-bit codebook
 *     (tq_kv_codebook, a value on a boundary takes the lower level);
 *   * keys (bits b): m = b - 1 codebook bits, then z = sign(S e) for the
 *     residual e = u - u~, S = jl (128 x 128, row-major fp32), sign(0) = +1,
 *     and gamma = |e| as fp16;
 *     score(q, k) = r (<Pi q, u~> + gamma sqrt(pi/2)/128 <S Pi q, z>);
 *   * values (bits b): m = b codebook bits; v^ = r Pi^T u~;
 *   * record of a vector (16 b bytes, uint32 words): code j in record bits
 *     m j .. m j + m - 1, little-endian (word w holds bits 32 w .. 32 w + 31),
 *     then for keys 128 bits with bit j set where z_j = +1.
 * Arithmetic: quantisation in FP64 (the codes and signs are the ones an FP64
 * evaluation gives); scores and value sums in FP32. */
#define TQ_KV_DIM 128
#define TQ_KV_MAX_BITS 8
enum { TQ_KV_OP_SCORES = 0, TQ_KV_OP_VALUES = 1, TQ_KV_OP_ATTEND = 2 };

/* The 2^bits levels, ascending, of the Lloyd-Max quantiser of N(0, 1/128)
 * (the distribution of one coordinate of a random unit vector in R^128):
 * each level is the mean of the values nearest to it.  Host function, no
 * GPU work; `levels` is host memory of 2^bits doubles.  bits 1..8. Upload
 * the result for tq_kv_quantize, tq_kv_scores and tq_kv_values (keys use
 * the bits - 1 codebook).  TQ_EUNSUPPORTED if the solve did not converge. */
int tq_kv_codebook(int bits, double *levels);

/* Bytes of one record: 16 * bits (0 for bits outside 1..8). */
size_t tq_kv_record_bytes(int bits);

/* Quantise n vectors x [n][128] (TQ_F32, TQ_BF16 or TQ_F16) as keys
 * (keys != 0, bits 2..8) or values (bits 1..8).  Vector i is written to
 * record i * stride (records uint32 [..][4 bits], 16-byte aligned), its
 * radius to radius[i * stride] and, for keys, gamma to gamma[i * stride]
 * (fp16 bits).  A stride > 1 writes one token of several heads into a
 * head-major cache.  signs: 128 floats +-1; jl: 128 x 128 floats (keys
 * only, NULL for values); levels: the codebook of the code bits (device,
 * 2^m doubles).  n = 0 is a no-op. */
int tq_kv_quantize(const void *x, int x_dtype, int64_t n, const float *signs,
                   const float *jl, const double *levels, int bits, int keys,
                   int64_t stride, uint32_t *records, uint16_t *radius,
                   uint16_t *gamma, void *stream);

/* Workspace bytes of tq_kv_scores (op TQ_KV_OP_SCORES), tq_kv_values
 * (TQ_KV_OP_VALUES) or tq_kv_attend (TQ_KV_OP_ATTEND) for n cached vectors
 * per head, `heads` heads and nq queries per head; SIZE_MAX for an invalid
 * request. */
size_t tq_kv_workspace(int op, int64_t n, int heads, int nq);

/* Scores of queries against quantised keys: for head h and query j,
 * scores[h][j][i] = score(q[h][j], key i of head h), the estimator above.
 * q fp32 [heads][nq][128]; keys records [heads][n][4 bits]; radius, gamma
 * fp16 bits [heads][n]; scores fp32 [heads][nq][n]; levels the bits - 1
 * codebook; jl 16-byte aligned.  heads * nq <= 65535.  Two launches (the
 * rotated query and S Pi q into the workspace, then one lane per key over
 * table lookups). */
int tq_kv_scores(const float *q, int heads, int nq, const uint32_t *keys,
                 const uint16_t *radius, const uint16_t *gamma, int64_t n,
                 int bits, const float *signs, const float *jl,
                 const double *levels, float *scores, void *workspace,
                 size_t ws_bytes, void *stream);

/* Probability-weighted sums of quantised values: for head h and query j,
 * out[h][j] = sum_i p[h][j][i] v^_i over the n values of head h, with
 * v^ = r Pi^T u~ (the sum is taken in the rotated frame and rotated back
 * once).  p fp32 [heads][nq][n] (any weights; softmax of the scores in
 * attention); values records [heads][n][4 bits]; radius fp16 bits
 * [heads][n]; out fp32 [heads][nq][128] (8-byte aligned); levels the
 * bits codebook.  heads * nq <= 65535.  Deterministic: the partial sums
 * of the key chunks are added in a fixed order. */
int tq_kv_values(const float *p, int heads, int nq, const uint32_t *values,
                 const uint16_t *radius, int64_t n, int bits,
                 const float *signs, const double *levels, float *out,
                 void *workspace, size_t ws_bytes, void *stream);

/* Decode attention over quantised values with the softmax folded in
 * ("Mac users can use TurboQuant in oMLX, with Gemma-4-31B", the section on
 * enabling TurboQuant in oMLX: its fused decode kernel; the softmax is the
 * attention the cache serves, not a step of the quantiser): for head h and
 * query j, out[h][j] = sum_i w_i v^_i / sum_i w_i with
 * w_i = exp(scale * scores[h][j][i] - max_i scale * scores[h][j][i]),
 * v^ as for tq_kv_values.  Equal to tq_kv_values with p the softmax of
 * scale * scores, without writing p: each key chunk keeps its own maximum
 * and weight sum and the finishing launch rescales the chunks to the
 * common maximum (the online-softmax merge).  scores fp32
 * [heads][nq][n], finite or -inf (masked); scale finite; a query whose
 * scores are all -inf, and n = 0, give zeros.  Other arguments, layout
 * and limits as for tq_kv_values; deterministic. */
int tq_kv_attend(const float *scores, float scale, int heads, int nq,
                 const uint32_t *values, const uint16_t *radius, int64_t n,
                 int bits, const float *signs, const double *levels,
                 float *out, void *workspace, size_t ws_bytes, void *stream);

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
