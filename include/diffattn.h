/*
 * diffattn.h - C ABI of the MI355X (gfx950) causal differential-attention
 * forward library, libdiffattn.so.
 *
 * The operation (Motif 2.6B explainer, section "Differential attention" and
 * the figure 1 caption of section "The block"): per batch row b and head h,
 *
 *     o = [ softmax(Q1 K1^T * scale) - lambda_h * softmax(Q2 K2^T * scale) ] V
 *     y = GroupNorm(o)   (one group per head over its d_v channels:
 *                         y = (o - mean) / sqrt(var + eps) * gain[h, c],
 *                         biased variance, no bias)
 *
 * with a causal mask (the model is decoder-only, per the edgentiq article on
 * Motif-2.6B): query i attends to keys j <= i.  Decode attends a single query
 * to every cached position of its sequence.  scale defaults to 1/sqrt(d_qk).
 *
 * Supported head sizes: d_qk = 64, d_v = 128 (Motif 2.6B: 16 heads, hidden
 * 2048, no grouped-query sharing; explainer section "The block").
 *
 * Conventions shared by every entry point
 *   - Tensors are device memory owned by the caller.  The library allocates
 *     nothing, keeps no pointer after it returns, and has no global mutable
 *     state; calls are thread-safe.  Keep buffers alive until the stream work
 *     has finished.
 *   - Inputs Q1, Q2, K1, K2, V are bf16 (raw 16-bit patterns).  V is converted
 *     exactly to fp16 on chip, so its magnitudes must stay below 65504;
 *     values below 2^-14 lose precision as fp16 subnormals (below 2^-24 they
 *     flush to zero).
 *   - Layout [B, T, H, D] with element strides given per tensor by
 *     diffattn_strides {b, t, h}; the innermost dimension D is contiguous.  A
 *     NULL strides pointer means C-contiguous [B, T, H, D].  Base pointers
 *     must be 16-byte aligned, every stride a non-negative multiple of 8
 *     elements, and the t stride below 2^25 elements (DIFFATTN_ERR_LAYOUT
 *     otherwise).
 *   - Outputs are C-contiguous.  out: bf16 (round to nearest even) or fp32,
 *     chosen by out_dtype.  o_pre: optional fp32 copy of o before the norm
 *     (NULL to skip).
 *   - lambda: one finite value for all heads, or lambda_per_head (device fp32
 *     [H]) when non-NULL.  No clamping.  gain: device fp32 [H, d_v].
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     returns immediately.  Arguments are validated on the host before any
 *     HIP call: on an invalid argument the call returns a nonzero status and
 *     touches no memory.  DIFFATTN_ERR_HIP reports the failure of one of this
 *     call's own launches (an error left by an earlier, unrelated HIP call is
 *     neither reported nor cleared).  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Results are bitwise reproducible run to run (no atomics).
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DIFFATTN_API __attribute__((visibility("default")))
#else
#define DIFFATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum diffattn_status {
    DIFFATTN_OK = 0,
    DIFFATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    DIFFATTN_ERR_SHAPE = 2,       /* a size is non-positive or too large */
    DIFFATTN_ERR_UNSUPPORTED = 3, /* head sizes other than d_qk=64, d_v=128 */
    DIFFATTN_ERR_LAYOUT = 4,      /* misaligned pointer or stride */
    DIFFATTN_ERR_WORKSPACE = 5,   /* workspace missing, misaligned or too small */
    DIFFATTN_ERR_HIP = 6,         /* the HIP runtime refused a launch */
    DIFFATTN_ERR_VALUE = 7        /* non-finite lambda/eps/scale, eps < 0, bad dtype, split count or option */
};

enum diffattn_out_dtype { DIFFATTN_OUT_BF16 = 0, DIFFATTN_OUT_F32 = 1 };

/* Rotary position embedding on Q1, Q2, K1, K2 (diffattn_options.rope). */
enum diffattn_rope {
    DIFFATTN_ROPE_NONE = 0,
    DIFFATTN_ROPE_HALF = 1,        /* pairs (i, i + 32) of each 64-dim vector */
    DIFFATTN_ROPE_INTERLEAVED = 2  /* pairs (2i, 2i + 1) */
};

/*
 * Variants of the operation, for the *_ex entry points.  Zero-initialise and
 * set what is needed: all fields zero is exactly the plain causal operation.
 *   window     : > 0 gives a sliding window: query i attends keys
 *                i-window+1 .. i (decode: the last `window` positions of the
 *                sequence); 0 attends every key <= i.  Motif 3 alternates one
 *                full causal layer with three sliding-window layers (picx.dev
 *                summary of the Motif 3 report, section 2.1).
 *   kv_ring    : decode only (prefill requires 0).  Nonzero: each sequence's
 *                cache of L slots is a ring buffer, position p in slot p % L,
 *                so seqlens may exceed L; the query attends the last
 *                min(seqlen, window) positions, and window = 0 means window =
 *                L.  A window larger than L is an error (the ring no longer
 *                holds those positions).  Zero: slot p holds position p and
 *                seqlens above L count as L.
 *   rope       : rotary position embedding applied to Q1, Q2, K1, K2 inside
 *                the kernels before the score products (Motif 2.6B explainer,
 *                section "The block": RoPE with base 500,000).  Each 64-wide
 *                vector is rotated on its own: pair c turns by the angle
 *                pos * rope_theta^(-c/32), pairing dims (c, c + 32) for
 *                DIFFATTN_ROPE_HALF or (2c, 2c + 1) for
 *                DIFFATTN_ROPE_INTERLEAVED, computed in fp32.  Prefill: token
 *                t sits at position rope_pos0 + t; the rotated Q and K are
 *                rounded to fp16 for the score products (eight times finer
 *                than bf16), so their magnitudes must stay below 65504.
 *                Decode: only the query is rotated (kept in fp32), at position
 *                rope_pos0 + n - 1 for a sequence of n cached tokens (n as
 *                counted after the clamp to L of a linear cache); the cache
 *                must hold keys already rotated (diffattn_rope_apply).
 *   rope_theta : base, finite and > 0 when rope is on.
 *   rope_pos0  : >= 0; positions must stay below 2^32.
 *   ws_prepared: diffattn_fwd_prefill_ws only (0 or 1; must be 0 for every
 *                other entry point).  1: the workspace already holds what
 *                diffattn_prefill_prepare wrote for the same K1, K2, V,
 *                strides, sizes and options, so the call skips its pre-pass
 *                and runs the prefill kernel alone.
 *   reserved   : must be zero.
 */
typedef struct {
    int32_t window;
    int32_t kv_ring;
    int32_t rope;
    int32_t rope_pos0;
    float rope_theta;
    int32_t ws_prepared;
    int32_t reserved[2];
} diffattn_options;

/* Element strides of the three outer dimensions of a [B, T, H, D] tensor. */
typedef struct {
    int64_t b, t, h;
} diffattn_strides;

/*
 * Causal prefill over T tokens (a square causal map per (b, h)).
 *   q1, q2, k1, k2 : bf16 [B, T, H, d_qk]
 *   v              : bf16 [B, T, H, d_v]
 *   strides        : 5 entries, for q1, q2, k1, k2, v in that order; or NULL
 *   lambda, lambda_per_head, gain, gn_eps : as above (gn_eps >= 0)
 *   scale          : score factor; <= 0 selects 1/sqrt(d_qk)
 *   out            : [B, T, H, d_v], bf16 or fp32 per out_dtype
 *   o_pre          : fp32 [B, T, H, d_v] or NULL
 * Limits: B*H <= 2^24, T <= 2^22, ceil(T/128)*B*H <= 2^23.
 */
DIFFATTN_API int diffattn_fwd_prefill(const void* q1, const void* q2, const void* k1, const void* k2,
                         const void* v, const diffattn_strides* strides, int B, int T, int H,
                         int d_qk, int d_v, float lambda, const float* lambda_per_head,
                         const float* gain, float gn_eps, float scale, void* out, int out_dtype,
                         float* o_pre, void* stream);

/*
 * Bytes of device workspace that diffattn_fwd_decode needs for these sizes:
 * per (b, h, split) and per map, the split's running max, sum and d_v
 * unnormalised outputs, in fp32.  num_splits <= 0 means the default (8).
 * Returns 0 for invalid sizes.
 */
DIFFATTN_API size_t diffattn_decode_workspace_bytes(int B, int H, int d_v, int num_splits);

/*
 * Single-query decode against a KV cache, split over the cached positions
 * (each split keeps both maps' softmax states; a second kernel merges the
 * splits, keeping the two maps apart until o = O1/L1 - lambda O2/L2, then
 * applies the GroupNorm).
 *   q1, q2         : bf16 [B, H, d_qk], C-contiguous
 *   k1, k2         : bf16 cache [B, L, H, d_qk]
 *   v              : bf16 cache [B, L, H, d_v]
 *   cache_strides  : 3 entries, for k1, k2, v (t = cache position); or NULL
 *   seqlens        : device int32 [B] cached lengths, or NULL for L.  Values
 *                    above L count as L; values <= 0 give all-zero output.
 *   num_splits     : 1..64, or <= 0 for the default (8)
 *   workspace      : device buffer of >= diffattn_decode_workspace_bytes()
 *                    bytes, 16-byte aligned; contents need no initialisation
 *   out            : [B, H, d_v], bf16 or fp32 per out_dtype
 *   o_pre          : fp32 [B, H, d_v] or NULL
 * Limits: B*H <= 2^24, L <= 2^26, B*H*num_splits <= 2^23.
 */
DIFFATTN_API int diffattn_fwd_decode(const void* q1, const void* q2, const void* k1, const void* k2,
                        const void* v, const diffattn_strides* cache_strides,
                        const int32_t* seqlens, int B, int L, int H, int d_qk, int d_v,
                        float lambda, const float* lambda_per_head, const float* gain,
                        float gn_eps, float scale, int num_splits, void* workspace,
                        size_t workspace_bytes, void* out, int out_dtype, float* o_pre,
                        void* stream);

/* diffattn_fwd_prefill with variants (opt may be NULL: plain causal).  A
 * negative window, a nonzero kv_ring or reserved field, an unknown rope mode,
 * or with rope on a non-finite or non-positive rope_theta or a negative
 * rope_pos0 returns DIFFATTN_ERR_VALUE. */
DIFFATTN_API int diffattn_fwd_prefill_ex(const diffattn_options* opt, const void* q1, const void* q2,
                                         const void* k1, const void* k2, const void* v,
                                         const diffattn_strides* strides, int B, int T, int H, int d_qk,
                                         int d_v, float lambda, const float* lambda_per_head,
                                         const float* gain, float gn_eps, float scale, void* out,
                                         int out_dtype, float* o_pre, void* stream);

/*
 * Bytes of device workspace diffattn_fwd_prefill_ws needs for these options
 * and sizes: with rope on, one fp16 copy of each of K1 and K2, rotated once
 * (2 * B * T * H * 64 * 2 bytes, rounded up to 256-byte slices); then V as
 * fp16 V^T tiles, B * H * ceil(T / 32) * 8192 bytes.  0 for invalid sizes.
 */
DIFFATTN_API size_t diffattn_prefill_workspace_bytes(const diffattn_options* opt, int B, int T, int H);

/*
 * diffattn_fwd_prefill_ex with a workspace, the fast path.  With rope on, K1
 * and K2 are first rotated into the workspace, each key once (the same fp32
 * rotation and fp16 rounding the kernels of diffattn_fwd_prefill_ex apply to
 * every key tile they stage), and the prefill then reads those copies: the
 * query blocks no longer repeat the rotation of the keys they share.  V is
 * converted once to fp16 (the same exact conversion the kernels otherwise
 * apply while staging each tile) into transposed 32-key tiles that the
 * prefill kernels move into LDS by DMA; with rope, one launch does both
 * pre-passes.  Where the grid of 128-query blocks fits the chip in one round
 * (two per compute unit) both entry points run the same kernel and the
 * results equal those of diffattn_fwd_prefill_ex bit for bit (same products,
 * same order); on larger grids whose long/short query-block pairs fill
 * their rounds of the chip the workspace path keeps the persistent two-group
 * kernel, whose per-group reference maxima round P to fp16 differently, so
 * the two differ within that rounding (other grids run the four-wave kernel
 * on both paths).  A sliding window of
 * at most 129 keys uses the workspace only for the rotated keys.  Without
 * rope the workspace may be NULL (then it is the plain entry point).
 *   workspace : >= diffattn_prefill_workspace_bytes(opt, B, T, H) bytes,
 *               256-byte aligned; contents need no initialisation
 * Errors as for diffattn_fwd_prefill_ex, plus DIFFATTN_ERR_WORKSPACE (a
 * missing workspace with rope on, or a misaligned or too small one) and
 * DIFFATTN_ERR_SHAPE when the pre-pass launch would exceed 2^32 work-items
 * (256 per V^T tile and per 32 rotated key vectors).  The
 * workspace is overwritten on the stream: calls that share one must not
 * overlap.
 */
DIFFATTN_API int diffattn_fwd_prefill_ws(const diffattn_options* opt, const void* q1, const void* q2,
                                         const void* k1, const void* k2, const void* v,
                                         const diffattn_strides* strides, int B, int T, int H, int d_qk,
                                         int d_v, float lambda, const float* lambda_per_head,
                                         const float* gain, float gn_eps, float scale, void* out,
                                         int out_dtype, float* o_pre, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * The pre-pass of diffattn_fwd_prefill_ws alone: the rotated key copies
 * (rope on) and the fp16 V^T tiles, written to the workspace exactly as that
 * call writes them.  A caller that runs several prefills over the same keys
 * and values (query chunks against one cache, repeated calls) prepares once
 * and passes opt->ws_prepared = 1 to each diffattn_fwd_prefill_ws, which then
 * launches the prefill kernel alone.  Arguments as for diffattn_fwd_prefill_ws
 * (strides: the five entries, of which those of K1, K2 and V are used; opt
 * with ws_prepared 0).  Results of the prepared calls equal those of
 * unprepared ones bit for bit.  Errors as for diffattn_fwd_prefill_ws.
 */
DIFFATTN_API int diffattn_prefill_prepare(const diffattn_options* opt, const void* k1, const void* k2,
                                          const void* v, const diffattn_strides* strides, int B, int T, int H,
                                          int d_qk, int d_v, void* workspace, size_t workspace_bytes,
                                          void* stream);

/* diffattn_fwd_decode with variants (opt may be NULL: every cached position).
 * Errors as for diffattn_fwd_prefill_ex, and DIFFATTN_ERR_VALUE for a ring
 * cache with window > L.  With a ring cache, seqlens may exceed L (up to
 * 2^31 - 1). */
DIFFATTN_API int diffattn_fwd_decode_ex(const diffattn_options* opt, const void* q1, const void* q2,
                                        const void* k1, const void* k2, const void* v,
                                        const diffattn_strides* cache_strides, const int32_t* seqlens,
                                        int B, int L, int H, int d_qk, int d_v, float lambda,
                                        const float* lambda_per_head, const float* gain, float gn_eps,
                                        float scale, int num_splits, void* workspace,
                                        size_t workspace_bytes, void* out, int out_dtype, float* o_pre,
                                        void* stream);

/*
 * diffattn_fwd_decode_ex without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  It makes no allocation of any
 * kind.  The split partials live in a buffer the library holds on each device
 * (a file-scope device array of DIFFATTN_DECODE_SCRATCH_BYTES, kept until the
 * process ends), so B * H * num_splits * 2 * (d_v + 2) * 4 bytes (the value
 * of diffattn_decode_workspace_bytes) must not exceed it:
 * DIFFATTN_ERR_WORKSPACE otherwise, before any HIP call.  The first call on a
 * device looks the buffer's address up there (DIFFATTN_ERR_HIP if that fails).
 * Every call on one device shares that device's buffer and the buffer keeps
 * the last call's contents; each call writes every record it reads, so none
 * needs clearing.  Calls that overlap on one device (different streams, or
 * threads with no ordering between them) race on the buffer and give wrong
 * results; calls in order on one stream are safe.  Otherwise as
 * diffattn_fwd_decode_ex, with the same arguments, results and errors.
 */
#define DIFFATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
DIFFATTN_API int diffattn_fwd_decode_noalloc(const diffattn_options* opt, const void* q1, const void* q2,
                                             const void* k1, const void* k2, const void* v,
                                             const diffattn_strides* cache_strides, const int32_t* seqlens,
                                             int B, int L, int H, int d_qk, int d_v, float lambda,
                                             const float* lambda_per_head, const float* gain, float gn_eps,
                                             float scale, int num_splits, void* out, int out_dtype,
                                             float* o_pre, void* stream);

/*
 * Rotary embedding of a bf16 [B, T, H, 64] tensor, the same rotation the *_ex
 * entry points apply (see diffattn_options.rope), for writing rotated keys
 * into a decode cache.  Token t of batch row b sits at position
 * pos0 + pos_start[b] + t (pos_start: device int32 [B], values >= 0, or NULL
 * for 0).  out may be x itself (in place, same strides).  Strides and
 * alignment as for the other entry points (NULL = C-contiguous).
 *   mode  : DIFFATTN_ROPE_HALF or DIFFATTN_ROPE_INTERLEAVED
 *   theta : finite, > 0;  pos0 >= 0
 * Limits: B*T*H <= 2^34.
 */
DIFFATTN_API int diffattn_rope_apply(const void* x, const diffattn_strides* x_strides, void* out,
                                     const diffattn_strides* out_strides, int B, int T, int H, int d, int mode,
                                     float theta, int pos0, const int32_t* pos_start, void* stream);

/*
 * Training forward: diffattn_fwd_prefill (plain causal; for windows and RoPE
 * see diffattn_fwd_prefill_train_ex) that also saves what the backward pass
 * needs.
 *   o1, o2 : fp32 [B, T, H, d_v], each map's normalised output
 *            softmax(Q_m K_m^T * scale) V (so o = o1 - lambda o2)
 *   lse    : fp32 [B, T, H, 2], each map's log-sum-exp of its scaled scores
 *            in base 2: log2 sum_j 2^(scale * log2(e) * q_i . k_j)
 * All three are required, C-contiguous and 16-byte aligned; other arguments
 * and errors as for diffattn_fwd_prefill.
 */
DIFFATTN_API int diffattn_fwd_prefill_train(const void* q1, const void* q2, const void* k1, const void* k2,
                                            const void* v, const diffattn_strides* strides, int B, int T, int H,
                                            int d_qk, int d_v, float lambda, const float* lambda_per_head,
                                            const float* gain, float gn_eps, float scale, void* out, int out_dtype,
                                            float* o_pre, float* o1, float* o2, float* lse, void* stream);

/*
 * diffattn_fwd_prefill_train with variants: opt->window (a sliding window)
 * and opt->rope, rope_theta, rope_pos0 (the rotary embedding of Q1, Q2, K1,
 * K2, rotated inside the kernels as diffattn_fwd_prefill_ex does), the
 * training outputs then being those of the rotated, windowed operation (lse
 * over each query's visible keys).  kv_ring and ws_prepared must be 0
 * (DIFFATTN_ERR_VALUE).  opt may be NULL.  Pass the same options to
 * diffattn_bwd_prefill_ex.
 */
DIFFATTN_API int diffattn_fwd_prefill_train_ex(const diffattn_options* opt, const void* q1, const void* q2,
                                               const void* k1, const void* k2, const void* v,
                                               const diffattn_strides* strides, int B, int T, int H, int d_qk,
                                               int d_v, float lambda, const float* lambda_per_head,
                                               const float* gain, float gn_eps, float scale, void* out,
                                               int out_dtype, float* o_pre, float* o1, float* o2, float* lse,
                                               void* stream);

/*
 * Bytes of device workspace diffattn_bwd_prefill needs (256-byte aligned
 * buffer): fp16 copies of q1, q2, k1, k2 and v, the pre-norm output gradient
 * in fp16, two row statistics and the gain/lambda partial sums (about
 * B * T * H * (4 d_qk + 2 d_v) * 2 bytes).  Returns 0 for invalid sizes.
 */
DIFFATTN_API size_t diffattn_bwd_workspace_bytes(int B, int T, int H, int d_v);

/*
 * Backward pass of the causal prefill: the gradients of sum(y * dy) for the
 * operation above (the calculus of the definition on the Motif 2.6B
 * explainer, section "Differential attention"; plain causal, and see
 * diffattn_bwd_prefill_ex for windows and RoPE).
 *   q1 .. v, strides, B, T, H, d_qk, d_v, lambda, lambda_per_head, gain,
 *   gn_eps, scale : the forward's arguments
 *   o1, o2, lse   : the forward's training outputs (diffattn_fwd_prefill_train)
 *   dy            : [B, T, H, d_v] bf16 or fp32 per dy_dtype, C-contiguous
 *   dq1, dq2, dk1, dk2 : fp32 [B, T, H, d_qk] out, C-contiguous
 *   dv            : fp32 [B, T, H, d_v] out
 *   dlambda       : fp32 [H] out, per head (for one shared lambda, sum it)
 *   dgain         : fp32 [H, d_v] out
 *   workspace     : >= diffattn_bwd_workspace_bytes() bytes, 256-byte aligned
 * Every output is written (not accumulated).  Errors as for the forward,
 * plus DIFFATTN_ERR_WORKSPACE.  Deterministic (no atomics).
 */
DIFFATTN_API int diffattn_bwd_prefill(const void* q1, const void* q2, const void* k1, const void* k2,
                                      const void* v, const diffattn_strides* strides, int B, int T, int H,
                                      int d_qk, int d_v, float lambda, const float* lambda_per_head,
                                      const float* gain, float gn_eps, float scale, const float* o1,
                                      const float* o2, const float* lse, const void* dy, int dy_dtype, float* dq1,
                                      float* dq2, float* dk1, float* dk2, float* dv, float* dlambda,
                                      float* dgain, void* workspace, size_t workspace_bytes, void* stream);

/*
 * diffattn_bwd_prefill with variants, for the forward diffattn_fwd_prefill_train_ex
 * ran with the same options (its o1, o2, lse):
 *   opt->window > 0: the sliding window (picx.dev summary of the Motif 3
 *     report, section 2.1); the gradients flow through the visible pairs only.
 *   opt->rope: the rotary embedding (Motif 2.6B explainer, section "The
 *     block"); dq1, dq2, dk1, dk2 are the gradients of the unrotated inputs:
 *     the rotated copies' gradients turned back by the inverse rotation of
 *     their position (the rotation is orthogonal), in fp32.
 * kv_ring and ws_prepared must be 0 (DIFFATTN_ERR_VALUE).  opt may be NULL
 * (then it is diffattn_bwd_prefill).  Other arguments, outputs and errors as
 * for diffattn_bwd_prefill.
 */
DIFFATTN_API int diffattn_bwd_prefill_ex(const diffattn_options* opt, const void* q1, const void* q2,
                                         const void* k1, const void* k2, const void* v,
                                         const diffattn_strides* strides, int B, int T, int H, int d_qk, int d_v,
                                         float lambda, const float* lambda_per_head, const float* gain,
                                         float gn_eps, float scale, const float* o1, const float* o2,
                                         const float* lse, const void* dy, int dy_dtype, float* dq1, float* dq2,
                                         float* dk1, float* dk2, float* dv, float* dlambda, float* dgain,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped differential attention with a token-wise lambda and an output gate
 * (picx.dev summary of the Motif 3 report, section 2.2, "Grouped
 * Differential Attention" and "Output Gating"), causal prefill:
 *   n_heads = n_S + n_N heads with n_N = n_heads / (group + 1) noise heads
 *   and n_S = group * n_N signal heads; heads 0 .. n_S-1 are the signal heads,
 *   n_S .. n_heads-1 the noise heads, and signal head s is paired with noise
 *   head n_S + s / group (each noise head repeated group times in place).
 *   Every head is ordinary causal softmax attention with its own values,
 *   H_h = softmax(Q_h K_h^T * scale) V_h, and
 *     out_s = sigmoid(G_s) * (H_s - lambda_t[s] * H_(n_S + s / group))
 *   with no GroupNorm (the formula applies only the gate).
 *   q, k        : bf16 [B, T, n_heads, d_qk];  v : bf16 [B, T, n_heads, d_v]
 *   strides     : 3 entries for q, k, v, or NULL (C-contiguous)
 *   lambda_t    : device fp32 [B, T, n_S], C-contiguous (any finite values;
 *                 the model's sigmoid output lies in (0, 1))
 *   gate        : device bf16 [B, T, n_S, d_v] gate logits G, C-contiguous
 *                 and 8-byte aligned, or NULL for no gate
 *   scale       : score factor; <= 0 selects 1/sqrt(d_qk)
 *   out         : [B, T, n_S, d_v] bf16 or fp32 per out_dtype
 *   workspace   : >= diffattn_grouped_workspace_bytes() bytes, 16-byte
 *                 aligned, contents need no initialisation: every head's
 *                 normalised output (fp32, B * T * n_heads * d_v * 4 bytes),
 *                 each noise head's computed once, then V converted once into
 *                 fp16 transposed 32-key tiles that the attention kernel
 *                 moves into LDS by DMA (B * n_heads * ceil(T / 32) * 8192
 *                 bytes)
 * Errors: DIFFATTN_ERR_SHAPE also when n_heads is not a multiple of group + 1.
 */
DIFFATTN_API size_t diffattn_grouped_workspace_bytes(int B, int T, int n_heads, int group, int d_v);
DIFFATTN_API int diffattn_fwd_grouped(const void* q, const void* k, const void* v,
                                      const diffattn_strides* strides, int B, int T, int n_heads, int group,
                                      int d_qk, int d_v, const float* lambda_t, const void* gate, float scale,
                                      void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Single-query decode of the grouped form above (picx.dev summary of the
 * Motif 3 report, section 2.2, and its note on KV-cache reduction for
 * long-context inference): the query of each sequence's newest token against
 * its cache, per head H_h = softmax(q_h K_h^T * scale) V_h over the cached
 * positions, and
 *   out_s = sigmoid(G_s) * (H_s - lambda_t[s] * H_(n_S + s / group)),
 * no GroupNorm.  Each noise head is computed once per sequence.
 *   opt         : window (the last `window` positions) and kv_ring as for
 *                 diffattn_fwd_decode_ex; rope and ws_prepared must be 0
 *                 (DIFFATTN_ERR_VALUE); may be NULL
 *   q           : bf16 [B, n_heads, d_qk], C-contiguous
 *   k, v        : bf16 caches [B, L, n_heads, d_qk] and [B, L, n_heads, d_v]
 *   strides     : 2 entries (k, v) or NULL (C-contiguous)
 *   seqlens     : device int32 [B] cached positions per sequence (as
 *                 diffattn_fwd_decode), or NULL for L each; 0 gives 0 output
 *   lambda_t    : device fp32 [B, n_S], the newest token's lambda per signal head
 *   gate        : device bf16 [B, n_S, d_v] gate logits, 8-byte aligned, or NULL
 *   num_splits  : key ranges per (b, head), 1 .. 64; <= 0 selects 8
 *   workspace   : >= diffattn_grouped_decode_workspace_bytes() bytes, 16-byte
 *                 aligned: each (b, head, split)'s softmax state
 *   out         : [B, n_S, d_v] bf16 or fp32 per out_dtype
 * Errors as for diffattn_fwd_decode_ex, and DIFFATTN_ERR_SHAPE when n_heads
 * is not a multiple of group + 1.
 */
DIFFATTN_API size_t diffattn_grouped_decode_workspace_bytes(int B, int n_heads, int d_v, int num_splits);
DIFFATTN_API int diffattn_fwd_grouped_decode(const diffattn_options* opt, const void* q, const void* k,
                                             const void* v, const diffattn_strides* strides,
                                             const int32_t* seqlens, int B, int L, int n_heads, int group,
                                             int d_qk, int d_v, const float* lambda_t, const void* gate,
                                             float scale, int num_splits, void* workspace,
                                             size_t workspace_bytes, void* out, int out_dtype, void* stream);

/* Static text for a status code (never NULL). */
DIFFATTN_API const char* diffattn_status_string(int status);

/* Library ABI version (major * 100 + minor): 101 adds the *_ex entry points,
 * 102 the rotary embedding (diffattn_options.rope, diffattn_rope_apply), 103
 * the training forward and the backward pass, 104 grouped attention, 105 the
 * prefill workspace entry points (keys rotated once), 106 a larger backward
 * workspace (fp16 input copies; query diffattn_bwd_workspace_bytes again),
 * 107 diffattn_fwd_decode_noalloc, 108 V^T tiles in the prefill workspace,
 * 109 diffattn_prefill_prepare and diffattn_options.ws_prepared, 110 the
 * training forward and backward with windows and RoPE (_train_ex, _bwd_prefill_ex),
 * 111 the grouped decode (diffattn_fwd_grouped_decode), 112 V^T tiles in the
 * grouped prefill's workspace (query diffattn_grouped_workspace_bytes again)
 * (query diffattn_prefill_workspace_bytes again). */
DIFFATTN_API int diffattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
