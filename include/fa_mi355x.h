/*
 * fa_mi355x.h -- C ABI of libfa_mi355x.so: exact tiled softmax attention
 * (FlashAttention-style forward) on AMD MI355X (gfx950).
 *
 * The operation (Transformers & Math, Module 16, sections 16.1-16.2; the
 * notebook "Online Softmax Without the Attention Matrix"):
 *
 *     O = softmax(s) V,   s_ij = scale * <q_i, k_j>  (optionally soft-capped),
 *
 * computed by streaming tiles of K and V through on-chip memory while each
 * query row keeps a running maximum m, normaliser l and unnormalised output,
 * rescaling both by exp(m_old - m_new) when the maximum grows, so the
 * Nq x Nk score matrix is never written to memory.  The result equals the
 * direct softmax up to rounding.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: device pointers (HBM), caller-allocated and caller-owned.  The
 *   library never allocates, frees or synchronises, keeps no state between
 *   calls and is safe to call from several host threads.
 * Alignment: every tensor base pointer must be a multiple of 16 bytes (the
 *   kernels move 16 bytes per lane to and from q, k, v, o, o_part and the
 *   caches), except the fp32 row arrays lse, m_part and l_part (4 bytes) and
 *   the arguments of fa_combine (natural alignment of their element type).
 *   A misaligned pointer returns FA_ERR_INVALID_ARG.  Allocations from
 *   hipMalloc (and torch) are aligned; a view that starts at an element
 *   offset may not be.
 * Layouts: row-major, contiguous, no padding:
 *   q, o       [B, H,   Nq, d]
 *   k, v       [B, Hkv, Nk, d]
 *   lse        [B, H,   Nq]           fp32, natural log of sum_j e^(s_ij)
 *   o_part     [B, H,   Nq, S, d]     fp32 (split-KV partial outputs)
 *   m_part,
 *   l_part     [B, H,   Nq, S]        fp32
 * Heads: query head h reads key/value head g = h / (H / Hkv) (consecutive
 *   groups of H/Hkv query heads share one K/V head); H % Hkv must be 0.
 * Positions: query row i sits at absolute position p = i + (Nk - Nq), i.e.
 *   the last query is aligned with the last key.  causal != 0 keeps keys
 *   j <= p.  window > 0 (only with causal) also drops keys j <= p - window,
 *   leaving exactly the `window` most recent keys including position p
 *   (Transformers & Math section 16.3, sliding-window attention; the causal
 *   mask uses each token's position in the full sequence, section 16.2).
 * Soft-cap: softcap > 0 replaces every score z by softcap * tanh(z/softcap)
 *   (Transformers & Math section 16.5) before masking; softcap == 0 turns it
 *   off.
 * Degenerate inputs: B, H or Nq == 0 is a no-op returning FA_OK.  A query
 *   row with no visible key (Nk == 0, or more queries than keys under a
 *   causal mask) gets O = 0 and lse = -inf, as a zero normaliser leaves the
 *   output at zero (oxios_kernel flash_attention.rs, attention).
 * Streams: every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *   null stream).  Errors found before launch return a negative status and
 *   launch nothing; FA_ERR_HIP reports a failed launch (hipGetLastError).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same underlying type as hipStream_t, without pulling in HIP headers. */
typedef struct ihipStream_t *fa_stream_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1, /* bad size, null pointer, bad flag combination */
    FA_ERR_UNSUPPORTED = -2, /* valid request with no kernel (d, dtype)       */
    FA_ERR_HIP = -3,         /* the HIP runtime reported a launch failure     */
    FA_ERR_SCRATCH_LIMIT = -4 /* fa_splitkv_attention_static: partials exceed
                                 FA_STATIC_SCRATCH_BYTES                      */
} fa_status;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_FP32 = 1 } fa_dtype;

/* Head sizes with kernels: d in {32, 64, 128}.  Per head, Nq*d and Nk*d
 * must be below 2^31, and so must B*H and the grid's workgroup count
 * (FA_ERR_UNSUPPORTED otherwise). */
#define FA_MAX_HEAD_WINDOWS 256 /* largest H accepted with per-head windows */

/*
 * fa_fwd -- bf16 forward attention, fp32 accumulation, bf16 output.
 *
 * q, k, v: bf16 device tensors in the layouts above.  o: bf16 [B,H,Nq,d],
 * written with round-to-nearest-even.  lse: fp32 [B,H,Nq] or NULL (not
 * written).  scale multiplies q.k before the soft-cap (use 1/sqrt(d) for the
 * usual scaled dot product, nx_flashattn_scale.nx and Transformers & Math
 * section 16.5).  causal: 0/1.  window: 0 = none, > 0 needs causal.
 * softcap: 0 = none, > 0 = cap value.
 * Numerics: scores, the running maximum, the normaliser and O accumulate in
 * fp32; each tile's weights are rounded to bf16 for the P.V product, while
 * the normaliser, and so lse, sums the fp32 weights.  (With a soft-cap up to
 * 60 the reference maximum stays 0; O is then divided by the sum of the
 * bf16 weights P.V used, lse still takes the fp32 sum.)
 * Range with 0 < softcap <= 60: every weight is then e^z with |z| <= softcap
 * instead of at most 1, so the fp32 output accumulator of a row reaches up
 * to e^softcap * sum_j |v_j| over its visible keys.  That sum must stay
 * below the fp32 maximum (3.4e38), i.e. max|v| * Nk < 3.4e38 / e^softcap:
 * at 16384 keys, |v| below about 4e12 for softcap 50 and 1.8e8 for softcap
 * 60.  Beyond that the result overflows to inf/NaN; a softcap above 60 takes
 * the running maximum, whose weights never exceed 1.
 * Errors: FA_ERR_INVALID_ARG for negative sizes, Hkv < 1, H % Hkv != 0, a
 * NULL q/k/v/o when the tensor is non-empty, window < 0, window > 0 without
 * causal, softcap < 0 or non-finite, non-finite scale; FA_ERR_UNSUPPORTED
 * for d not in {32, 64, 128} or Nq*d, Nk*d or B*H >= 2^31.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
           float scale, int causal, int window, float softcap, fa_stream_t stream);

/*
 * fa_fwd_f32 -- the same operation on fp32 tensors (q, k, v, o fp32), with
 * fp32 arithmetic throughout.  Arguments and errors as fa_fwd.
 */
int fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
               int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
               float scale, int causal, int window, float softcap, fa_stream_t stream);

/*
 * fa_fwd_ex -- fa_fwd / fa_fwd_f32 with a window per query head, as when
 * local (sliding-window) and global heads alternate (Transformers & Math
 * section 16.3, alternating local and global attention).
 *
 * dtype selects bf16 (FA_DTYPE_BF16) or fp32 (FA_DTYPE_FP32) tensors.
 * head_window: NULL (every head uses `window`) or a HOST array of exactly H
 * int32 values (entry h for query head h; the library reads all H of them),
 * each 0 (no window) or > 0; read during the call only.  H may be at
 * most FA_MAX_HEAD_WINDOWS when head_window is given (else
 * FA_ERR_UNSUPPORTED).  A positive entry needs causal.
 */
typedef struct fa_fwd_args {
    int dtype;
    const void *q, *k, *v;
    void *o;
    float *lse;
    int64_t B, H, Hkv, Nq, Nk, d;
    float scale;
    int causal;
    int window;
    float softcap;
    const int32_t *head_window;
    fa_stream_t stream;
} fa_fwd_args;

int fa_fwd_ex(const fa_fwd_args *args);

/*
 * fa_fwd_fp8 -- forward attention on fp8 q, k, v: both products on the fp8
 * matrix cores, the online-softmax state (maximum, normaliser, output) in
 * fp32, bf16 output.  A low-precision variant of the same operation: the
 * two matrix products of the loop run in a narrow format while the softmax
 * bookkeeping stays wide (HiFA4 abstract, there with 4-bit operands on
 * Ascend NPUs).
 *
 * q, k, v: bytes in the OCP 8-bit E4M3 format (1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits; no infinities, 0x7f and 0xff are NaN), one
 * byte per element, in the layouts above.  Element values are
 * q_descale * E4M3(q byte), k_descale * E4M3(k byte), v_descale *
 * E4M3(v byte); each descale must be finite and > 0.  The scores are
 * scale * <q_i, k_j> of those values, computed exactly from the products of
 * the bytes and one fp32 factor.  The weights e^(s_ij - m) of each key tile
 * are rounded to E4M3 (after a fixed power-of-two shift, relative error at
 * most 2^-4 for weights above 2^-13 of the running maximum) for the P.V
 * product; the normaliser and lse use the fp32 weights.  O is therefore
 * exact attention of the dequantised inputs up to that rounding of P.
 * o: bf16 [B,H,Nq,d].  lse: fp32 [B,H,Nq] or NULL.  causal and window as
 * fa_fwd.  No soft-cap.  d in {64, 128}.
 * Errors: as fa_fwd, plus FA_ERR_INVALID_ARG for a descale that is not
 * finite and > 0 or a score factor scale*q_descale*k_descale beyond fp32
 * range, FA_ERR_UNSUPPORTED for d not in {64, 128}.
 */
int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
               int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
               float scale, float q_descale, float k_descale, float v_descale,
               int causal, int window, fa_stream_t stream);

/*
 * fa_fwd_splitkv -- split-KV attention, first pass (bf16 q, k, v).
 *
 * The keys are cut into num_splits chunks of C = ceil(Nk / num_splits) keys;
 * split s covers keys [s*C, min(Nk, (s+1)*C)).  For every query row and split
 * it writes the split's own result, the per-block state of the merge rule
 * in Transformers & Math section 16.2:
 *   m_part[.., s] = max of the row's visible scores in the chunk (-inf if none),
 *   l_part[.., s] = sum over those keys of exp(score - m_part) (0 if none),
 *   o_part[.., s, :] = that chunk's normalised output (0 if none),
 * all fp32, scores in natural-log units (after scale and soft-cap).
 * fa_combine merges them.  Masks, soft-cap and GQA as fa_fwd; num_splits >= 1.
 * Errors as fa_fwd, plus FA_ERR_INVALID_ARG for num_splits < 1 or NULL
 * partial pointers when B*H*Nq > 0.
 */
int fa_fwd_splitkv(const void *q, const void *k, const void *v,
                   float *o_part, float *m_part, float *l_part,
                   int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int causal, int window, float softcap, int num_splits,
                   fa_stream_t stream);

/*
 * fa_combine -- merge per-split results into the final output.
 *
 * For each row: m = max_s m_s, l = sum_s e^(m_s - m) l_s,
 * O = sum_s (e^(m_s - m) l_s / l) O_s, lse = m + ln l: the two-block merge
 * equations of Transformers & Math section 16.2 applied to all splits at
 * once (splits with l_s = 0 carry no weight).  o: [B,H,Nq,d] in out_dtype
 * (FA_DTYPE_BF16, round-to-nearest-even, or FA_DTYPE_FP32).  lse: fp32
 * [B,H,Nq] or NULL.  A row whose splits are all empty gets O = 0,
 * lse = -inf.  Errors: FA_ERR_INVALID_ARG for negative sizes, num_splits < 1,
 * NULL inputs/o when non-empty, unknown out_dtype; FA_ERR_UNSUPPORTED for d
 * not in {32, 64, 128}.
 */
int fa_combine(const float *o_part, const float *m_part, const float *l_part,
               void *o, float *lse, int64_t B, int64_t H, int64_t Nq, int64_t d,
               int num_splits, int out_dtype, fa_stream_t stream);

/*
 * Rolling KV cache with attention sinks, for streaming decode.
 *
 * Transformers & Math section 16.3: a local (sliding-window) layer attends
 * to the last W positions only, so its cache never needs more than W
 * entries; section 16.6: streaming keeps the first few tokens (attention
 * sinks, 4 in the setup it describes) alongside the window.  A cache of one
 * such layer is two bf16 tensors k_cache, v_cache [B, Hkv, sinks + window, d]
 * (row-major, caller-owned, device memory): rows [0, sinks) hold tokens
 * 0 .. sinks-1 for good, rows [sinks, sinks + window) are a ring in which
 * token t >= sinks lives in row sinks + (t - sinks) % window until token
 * t + window replaces it.  After tokens 0 .. pos were written, the filled
 * rows are the prefix [0, min(pos + 1, sinks + window)) and hold exactly the
 * sink tokens and the window of the last W positions.
 */

/*
 * fa_kv_append -- write the K and V rows of tokens pos .. pos+T-1 into a
 * rolling cache.  k_new, v_new: bf16 [B, Hkv, T, d] (device); k_cache,
 * v_cache as above.  Token t goes to row t if t < sinks, else to row
 * sinks + (t - sinks) % window; when two of the T tokens map to one row the
 * later one is written.  Asynchronous on stream.
 * Errors: FA_ERR_INVALID_ARG for negative sizes, pos < 0, window < 1,
 * sinks < 0, NULL pointers when B*Hkv*T*d > 0; FA_ERR_UNSUPPORTED for d not
 * in {32, 64, 128} or B*Hkv*T >= 2^31.
 */
int fa_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                 int64_t B, int64_t Hkv, int64_t T, int64_t d,
                 int64_t pos, int64_t window, int64_t sinks, fa_stream_t stream);

/*
 * fa_decode_rolling -- split-KV first pass for the query of the token at
 * position pos against a rolling cache that holds tokens 0 .. pos (its own
 * K/V included: append first).  q: bf16 [B, H, 1, d]; query head h reads
 * cache head h / (H / Hkv).  The filled rows [0, n) with
 * n = min(pos + 1, sinks + window) are cut into num_splits chunks of
 * ceil(n / num_splits) rows, and the partials are written exactly as by
 * fa_fwd_splitkv with Nq = 1 (o_part [B,H,1,S,d], m_part and l_part
 * [B,H,1,S], fp32); fa_combine(..., Nq = 1, ...) then gives the output and
 * lse.  The result is attention of that query over the sink tokens and the
 * window of the last W positions, each once.  scale and softcap as
 * fa_fwd.  Errors as fa_kv_append, plus FA_ERR_INVALID_ARG for
 * num_splits < 1, H % Hkv != 0, non-finite scale or softcap < 0.
 */
int fa_decode_rolling(const void *q, const void *k_cache, const void *v_cache,
                      float *o_part, float *m_part, float *l_part,
                      int64_t B, int64_t H, int64_t Hkv, int64_t d,
                      int64_t pos, int64_t window, int64_t sinks,
                      float scale, float softcap, int num_splits, fa_stream_t stream);

/*
 * Row softmax with the online normaliser ("Online normalizer calculation
 * for softmax", abstract: the classical softmax with fewer memory passes;
 * the notebook "Online Softmax Without the Attention Matrix": the running
 * maximum and denominator recurrence).
 *
 * fa_softmax -- y[r, j] = exp(x[r, j] - max_j x[r, :]) / sum_j exp(...) for
 * each of `rows` rows of n values; lse[r] = max + ln sum (fp32, or NULL).
 * x, y: device, row-major [rows, n], both fp32 (FA_DTYPE_FP32) or both bf16
 * (FA_DTYPE_BF16, y rounded to nearest even); fp32 arithmetic.  The maximum
 * and the normaliser come from one read of each row; a second read writes y.
 * Rows need at least one finite value (NaN or +inf inputs are undefined).
 * Errors: FA_ERR_INVALID_ARG for negative sizes, an unknown dtype or NULL
 * x / y when rows*n > 0; FA_ERR_UNSUPPORTED for rows >= 2^31.
 */
int fa_softmax(const void *x, void *y, float *lse, int64_t rows, int64_t n, int dtype,
               fa_stream_t stream);

/* Largest k supported by fa_softmax_topk. */
#define FA_MAX_TOPK 64

/*
 * fa_softmax_topk -- the k largest softmax probabilities of each row and
 * their column indices, from ONE read of x: the online normaliser and a
 * running top-k are kept together.  probs: fp32 [rows, k] in descending
 * order; indices: int32 [rows, k]; equal values come lower column first.
 * lse as fa_softmax (or NULL).  1 <= k <= min(n, FA_MAX_TOPK).
 * Errors: FA_ERR_INVALID_ARG for negative sizes, k out of range, an unknown
 * dtype or NULL x / probs / indices when rows > 0; FA_ERR_UNSUPPORTED for
 * rows or n >= 2^31.
 */
int fa_softmax_topk(const void *x, float *probs, int32_t *indices, float *lse, int64_t rows,
                    int64_t n, int k, int dtype, fa_stream_t stream);

/*
 * fa_splitkv_attention_static -- split-KV attention (fa_fwd_splitkv followed
 * by fa_combine) that allocates nothing and takes no workspace: the
 * per-split partials live in a fixed device array inside the library, one
 * per GPU, of FA_STATIC_SCRATCH_BYTES.  For callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).
 *
 * Arguments as fa_fwd_splitkv, plus o ([B,H,Nq,d] in out_dtype,
 * FA_DTYPE_BF16 or FA_DTYPE_FP32) and lse (fp32 [B,H,Nq] or NULL) as
 * fa_combine writes them; q, k, v bf16.  The partials need
 * B*H*Nq*num_splits*(d+2)*4 bytes; a larger request returns
 * FA_ERR_SCRATCH_LIMIT and launches nothing.  The first call on a device
 * looks up that device's array (hipGetSymbolAddress) and keeps its address;
 * the array itself is held until the process ends.  Every call on one GPU
 * uses the same array: calls that overlap on one GPU (on different streams,
 * or from several host threads without ordering) race and give wrong
 * results.  Calls ordered on one stream are fine; every partial is written
 * before it is read, so nothing needs clearing between calls.
 * Errors: as fa_fwd_splitkv and fa_combine, plus FA_ERR_SCRATCH_LIMIT, and
 * FA_ERR_HIP if the device array cannot be looked up.
 */
#define FA_STATIC_SCRATCH_BYTES (8u << 20) /* 8 MiB per GPU */

int fa_splitkv_attention_static(const void *q, const void *k, const void *v, void *o, float *lse,
                                int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                                float scale, int causal, int window, float softcap, int num_splits,
                                int out_dtype, fa_stream_t stream);

/* Human-readable name of a status code (static storage). */
const char *fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
