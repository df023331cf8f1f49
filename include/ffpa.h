/*
 * ffpa.h -- C ABI of the MI355X (gfx950) exact large-head-dim attention forward.
 *
 * The operation is the one the ffpa-attn "API Reference" (readthedocs) page
 * defines for ffpa_attn_func, restated here:
 *
 *   O[b,h,r,:] = sum_k softmax_k( scale * <Q[b,h,r,:], K[b,g(h),k,:]> + mask[b,h,r,k] ) * V[b,g(h),k,:]
 *   LSE[b,h,r] = log( sum_k exp( scale * <Q[b,h,r,:], K[b,g(h),k,:]> + mask[b,h,r,k] ) )
 *
 * with g(h) = h / (Hq / Hkv) (grouped-query and multi-query heads: page
 * parameter "key", group_size = Nh_q / Nh_kv), the tail-aligned causal rule
 * of parameter "is_causal" (row r sees key k only when k <= r + Nkv - Nq,
 * which needs Nkv >= Nq), the mask of parameter "attn_mask" (a boolean entry
 * that is true takes part, a false one is excluded; a floating entry is an
 * additive bias, added after scaling), and scale = 1/sqrt(D) when not given
 * (parameter "scale").  The natural-log LSE follows the fp32 log-sum-exp that
 * the page's varlen entry returns.  A row whose keys are all excluded gets
 * O = 0 and LSE = -inf.
 *
 * Every step of every entry runs in hand-written HIP kernels on the caller's
 * stream; no entry allocates, and none keeps a pointer after a call returns.
 * The forward entries and the dropout keep-bit generator need no workspace;
 * the backward entries take a small caller-provided one (one float per query
 * row).  The only state is a thread-local error message, so calls from
 * several host threads are safe.
 */
#ifndef FFPA_H_
#define FFPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum { FFPA_BF16 = 0, FFPA_FP16 = 1 } ffpa_dtype;

/* Mask element types.  BOOL_U8: one byte per entry, nonzero = takes part.
 * ADD_*: additive bias in the named floating type. */
typedef enum {
  FFPA_MASK_NONE = 0,
  FFPA_MASK_BOOL_U8 = 1,
  FFPA_MASK_ADD_F32 = 2,
  FFPA_MASK_ADD_BF16 = 3,
  FFPA_MASK_ADD_FP16 = 4
} ffpa_mask_kind;

/* A mask broadcastable to [B, Hq, Nq, Nkv] (page parameter "attn_mask").
 * Entry (b, h, r, k) lives at data + b*stride_b + h*stride_h + r*stride_q
 * + k*stride_k, in elements of the mask type.  A zero stride broadcasts that
 * dimension.  stride_k must be 1.  `data` is a device pointer owned by the
 * caller. */
typedef struct {
  const void* data;
  int32_t kind; /* ffpa_mask_kind */
  int64_t stride_b, stride_h, stride_q, stride_k;
} ffpa_mask_t;

/* Status codes.  The Python layer maps 1/2/3/4 to TypeError / ValueError /
 * NotImplementedError / RuntimeError, the error classes the API page lists. */
enum {
  FFPA_OK = 0,
  FFPA_ERR_TYPE = 1,        /* dtype not bf16/fp16, or unknown mask kind */
  FFPA_ERR_VALUE = 2,       /* inconsistent shapes, causal with Nkv < Nq, bad scale, bad pointers */
  FFPA_ERR_UNSUPPORTED = 3, /* a valid request outside what the kernels cover (e.g. D % 8 != 0) */
  FFPA_ERR_HIP = 4          /* the HIP runtime refused the launch */
};

/*
 * ffpa_fwd -- enqueue the attention forward on `stream`.
 *
 *   q    device, [B, Hq, Nq, D], contiguous row-major, dtype elements
 *   k, v device, [B, Hkv, Nkv, D], contiguous row-major, dtype elements
 *   mask NULL for none, else a host pointer to a descriptor of a device mask
 *        (read during this call only); with is_causal, a key takes part only
 *        where both the mask and the causal rule admit it
 *   o    device, [B, Hq, Nq, D], contiguous, dtype elements; written
 *   lse  device, [B, Hq, Nq] float32, natural log; written; NULL skips it
 *   B, Hq, Hkv, Nq, Nkv >= 1; Hq % Hkv == 0; 8 <= D <= 1024 with D % 8 == 0
 *        (head dims divisible by 8, as the README's "End-to-End Inference"
 *        section allows; a D other than 64, 128, 192, 256, 320, 384, 448,
 *        512, 640, 768, 896 and 1024 runs the next of these up, see
 *        ffpa_kernel_head_dim; K and V must then hold finite values, since
 *        the padding columns of one key row read the next row's first ones,
 *        multiplied by zero)
 *   scale   finite, or NaN for the default 1/sqrt(D)
 *   is_causal  0 or 1; 1 requires Nkv >= Nq
 *   dtype   ffpa_dtype
 *   stream  hipStream_t, NULL for the null stream
 *
 * q, k, v and o must be 16-byte aligned and o must not overlap q, k, v, mask
 * or lse.  Arguments are checked on the host before any HIP call, so an
 * error return means nothing was enqueued.  The call returns once the kernel
 * is enqueued; faults during execution surface at the caller's next
 * synchronisation.
 */
int ffpa_fwd(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, void* o, float* lse,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale,
             int is_causal, int dtype, void* stream);

/* Element strides of the tensors of ffpa_fwd_strided: {batch, head, row} for
 * each of Q, K, V and O (the head-dim stride is 1).  Element (b, h, n, d) of
 * Q is at q + b*q[0] + h*q[1] + n*q[2] + d, and likewise for the others. */
typedef struct {
  int64_t q[3], k[3], v[3], o[3];
} ffpa_layout_t;

/*
 * ffpa_fwd_strided -- ffpa_fwd over tensors laid out by `layout` (a host
 * pointer, read during this call only) instead of contiguously: views such
 * as a [B, N, H, D] tensor seen as [B, H, N, D], or heads sliced out of a
 * fused projection, are read and written in place (the "zero-copy" layouts
 * of the ffpa-attn pages).  The operation, the other arguments and the
 * errors are those of ffpa_fwd, plus:
 *   - every stride is >= 0 and a multiple of 8 elements (16-byte rows), and
 *     every row stride is at least D (FFPA_ERR_UNSUPPORTED otherwise; a
 *     dimension of size 1 may take any such stride);
 *   - K and V share their row stride (their batch and head strides may
 *     differ);
 *   - the strides of O give every element its own address;
 *   - (Nq + 256) x the Q row stride and (Nkv + 256) x the K/V row stride,
 *     in bytes, stay below 2 GiB (FFPA_ERR_UNSUPPORTED otherwise).
 * LSE stays contiguous [B, Hq, Nq].  O must not overlap q, k, v, mask or lse
 * (checked on the address ranges from each tensor's first to its last
 * element).
 */
int ffpa_fwd_strided(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                     const ffpa_layout_t* layout, float scale, int is_causal, int dtype, void* stream);

/* The host-side argument check ffpa_fwd_strided performs, without enqueuing
 * anything. */
int ffpa_check_strided_args(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, const void* o,
                            const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                            const ffpa_layout_t* layout, float scale, int is_causal, int dtype);

/*
 * ffpa_dropout_keep -- enqueue the drawing of attention-dropout keep
 * decisions on `stream` (the ffpa-attn "API Reference" page, parameter
 * "dropout_p" of ffpa_attn_func: SDPA-style dropout keeps each attention
 * weight independently with probability 1 - p).
 *
 *   keep    device, [B, Hq, Nq, W] uint32, W = ceil(Nkv / 32), contiguous,
 *           4-byte aligned; written.  Bit i of word w set keeps key 32 w + i
 *           for that query row; bits of keys >= Nkv are 0.
 *   B, Hq, Nq, Nkv >= 1
 *   p       drop probability, 0 <= p < 1
 *   seed, offset  select the stream: the decisions are a pure function of
 *           (seed, offset, p, b, h, r, key) and of Hq, Nq (the row index
 *           (b Hq + h) Nq + r); they come from Philox4x32-10 (Salmon et al.,
 *           SC 2011) with key (seed mod 2^32, seed div 2^32) and, for word w of
 *           row index R and block j < 8, counter (8 w + j, R mod 2^32,
 *           R div 2^32, offset); output i of block j decides key 32 w + 4 j + i,
 *           kept when it is at least floor(p 2^32).
 *   stream  hipStream_t, NULL for the null stream
 *
 * Errors: FFPA_ERR_VALUE for sizes < 1, p outside [0, 1) or a null or
 * misaligned keep; FFPA_ERR_UNSUPPORTED for a mask beyond 2^40 words;
 * FFPA_ERR_HIP if the launch fails.  Allocates nothing.
 */
int ffpa_dropout_keep(uint32_t* keep, int64_t B, int64_t Hq, int64_t Nq, int64_t Nkv, float p, uint64_t seed,
                      uint32_t offset, void* stream);

/*
 * ffpa_fwd_dropout -- ffpa_fwd with SDPA-style attention dropout on the
 * softmax weights (same page, parameter "dropout_p"):
 *
 *   O[b,h,r,:] = sum_k P[r,k] * keep[r,k] / (1 - dropout_p) * V[b,g(h),k,:]
 *
 * with P the softmax weights of ffpa_fwd and keep[r,k] the bit of `keep`
 * (device, [B, Hq, Nq, ceil(Nkv / 32)] uint32 in the layout of
 * ffpa_dropout_keep, read only; any bits may be given).  The LSE is that of
 * the logits, as in ffpa_fwd: dropout does not change it.  Tensors are
 * contiguous as in ffpa_fwd; every other argument, rule and error is that of
 * ffpa_fwd (every head dim of ffpa_fwd included), plus FFPA_ERR_VALUE for
 * dropout_p outside [0, 1), a null or misaligned keep, or o / lse
 * overlapping keep.
 */
int ffpa_fwd_dropout(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale,
                     int is_causal, int dtype, const uint32_t* keep, float dropout_p, void* stream);

/* The host-side argument check ffpa_fwd_dropout performs, without enqueuing
 * anything. */
int ffpa_check_dropout_args(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, const void* o,
                            const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                            float scale, int is_causal, int dtype, const uint32_t* keep, float dropout_p);

/*
 * ffpa_bwd -- enqueue the backward of ffpa_fwd on `stream`: the gradients of
 * O with respect to Q, K and V, given dout = dL/dO (the ffpa-attn "API
 * Reference" page supports the backward of ffpa_attn_func; here the mask is a
 * constant - ffpa_bwd_mask_grad also returns its gradient).  With P the
 * softmax of the forward's logits and Delta[r] = <dout[r], o[r]>:
 *   dV = sum over a KV head's group of P^T dout
 *   dS = P * (dout V^T - Delta),  dQ = scale dS K,
 *   dK = scale * sum over the group of dS^T Q.
 *
 *   q, k, v, mask, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype: as given
 *        to ffpa_fwd (same layouts and rules)
 *   o    device, [B, Hq, Nq, D]: the forward's output
 *   dout device, [B, Hq, Nq, D]: the gradient of the output
 *   lse  device, [B, Hq, Nq] float32: the forward's LSE (required)
 *   dq   device, [B, Hq, Nq, D]; dk, dv device, [B, Hkv, Nkv, D]; written,
 *        in the input dtype
 *   workspace  device, 256-byte aligned, at least ffpa_bwd_workspace_size()
 *        bytes, owned by the caller; it receives Delta (scratch)
 *
 * Three kernels on `stream`: Delta; a KV-stationary pass forming dK and dV
 * (each workgroup loops over the query rows of every head of its KV group);
 * a Q-stationary pass forming dQ.  Both passes recompute P from q, k, the
 * mask and the LSE, so no score matrix is stored.  Head dims: 8 <= D <=
 * 1024 with D % 8 == 0 (as for the forward, kernels exist for multiples of
 * 64 and other head dims run the next one up; the inputs must then hold
 * finite values).  Products take bf16/fp16 operands (P and dS rounded
 * once to the input type) with fp32 accumulation.  Errors as for ffpa_fwd;
 * FFPA_ERR_VALUE also for a missing or short workspace.
 */
int ffpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             const ffpa_mask_t* mask, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
             int64_t Nkv, int64_t D, float scale, int is_causal, int dtype, void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * ffpa_bwd_noalloc -- ffpa_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and results.  Its Delta buffer is a device array built into the
 * library, at most 4,194,304 (2^22) query rows (B * Hq * Nq); larger sizes
 * return FFPA_ERR_UNSUPPORTED.  It calls no allocating routine; the first
 * call on a device looks up that device's copy of the array.  Every call on
 * one GPU shares that array: calls that overlap on one GPU (two streams, two
 * host threads) race and must be serialised by the caller.
 */
int ffpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     const ffpa_mask_t* mask, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype, void* stream);

/*
 * ffpa_bwd_dropout -- the backward of ffpa_fwd_dropout: as ffpa_bwd, with
 * the forward's keep words `keep` (device, [B, Hq, Nq, ceil(Nkv / 32)]
 * uint32, read only) and dropout_p.  With M = keep / (1 - dropout_p) a
 * constant, the output was O = (P * M) V, so
 *   dV = sum over the group of (P * M)^T dout,
 *   dS = P * (dout V^T * M - Delta) with Delta[r] = <dout[r], o[r]>,
 * and dQ, dK as in ffpa_bwd.  `o` is the dropout forward's output.  Errors
 * as for ffpa_bwd, plus FFPA_ERR_VALUE for dropout_p outside [0, 1) or a
 * null or misaligned keep.  The workspace is ffpa_bwd_workspace_size().
 */
int ffpa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     const ffpa_mask_t* mask, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype, const uint32_t* keep,
                     float dropout_p, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ffpa_bwd_mask_grad -- ffpa_bwd (keep == NULL, dropout_p 0) or
 * ffpa_bwd_dropout (keep, dropout_p as there), plus the gradient of the
 * additive mask (ffpa-attn "API Reference": the attn_mask of the SDPA-style
 * call; SDPA differentiates a floating mask as a bias added to the logits).
 * The logits are scale * q.k + mask, so the mask's gradient is the logits'
 * gradient P * (dout V^T [* M] - Delta), summed over every dimension along
 * which the mask broadcasts (its stride 0: stride_b, stride_h or stride_q).
 *   mask   additive (FFPA_MASK_ADD_F32 / _BF16 / _FP16); required.  Keys
 *          contiguous (stride_k 1), as everywhere.
 *   dmask  device, float32, written: dense [B', H', Nq', Nkv] with B' = 1 if
 *          mask->stride_b is 0 and B otherwise, H' = 1 if stride_h is 0 and
 *          Hq otherwise, Nq' = 1 if stride_q is 0 and Nq otherwise.
 *          Entries the mask excludes (-inf, causal) get 0.  Without
 *          broadcast dimensions (B' = B, H' = Hq, Nq' = Nq, or those of size
 *          1) each element is written once and repeated calls give identical
 *          bits; the sums over broadcast dimensions use float atomic adds,
 *          whose order may vary from call to call.
 * dq, dk, dv as ffpa_bwd.  Errors as ffpa_bwd / ffpa_bwd_dropout, plus
 * FFPA_ERR_VALUE for a missing or boolean mask, a null or misaligned dmask,
 * or dropout_p != 0 without keep words.  Workspace: ffpa_bwd_workspace_size().
 */
int ffpa_bwd_mask_grad(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                       const ffpa_mask_t* mask, void* dq, void* dk, void* dv, float* dmask, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype,
                       const uint32_t* keep, float dropout_p, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace ffpa_bwd, ffpa_bwd_dropout and ffpa_bwd_mask_grad need for these sizes:
 * 4 * B * Hq * Nq (Delta), rounded up to 256.  0 for invalid sizes.  Host-only. */
size_t ffpa_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D);

/* The host-side argument check ffpa_fwd performs, without enqueuing anything
 * and without touching the memory the pointers refer to. */
int ffpa_check_args(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, const void* o,
                    const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                    float scale, int is_causal, int dtype);

/* A static, human-readable name of a status code.  Never NULL. */
const char* ffpa_status_string(int status);

/* The most specific description of the problem found by the calling
 * thread's last failing ffpa_fwd / ffpa_check_args call ("" if none).  The
 * text lives in thread-local storage and stays valid until that thread's
 * next call into the library. */
const char* ffpa_last_error_detail(void);

/* Rows of Q handled by one workgroup for head dim D (the tiling the kernels
 * use), or 0 for an unsupported D.  Host-only; for schedulers and tests. */
int ffpa_rows_per_block(int64_t D);

/* Head dim of the kernel that serves tensors of head dim D in ffpa_fwd,
 * ffpa_fwd_strided and ffpa_fwd_varlen: the smallest of 64, 128, 192, 256,
 * 320, 384, 448, 512, 640, 768, 896 and 1024 at or above D (its columns past
 * D are padding: zeros in Q, never stored in O).  576, 704, 832 and 960 thus
 * run 640, 768, 896 and 1024.  0 for an unsupported D.  Host-only. */
int64_t ffpa_kernel_head_dim(int64_t D);

/* Name of the GPU kernel that serves head dim D (as profilers list it, without
 * template arguments), or NULL for an unsupported D.  Which variant of that
 * kernel runs also depends on the mask and causal arguments.  Host-only; a
 * static string. */
const char* ffpa_kernel_name(int64_t D);

/*
 * ffpa_fwd_fp8 -- enqueue the FP8 attention forward (the ffpa-attn README,
 * "Latest News": FP8 attention for head dims 64..1024, and "End-to-End
 * Inference": masks, causal, GQA/MQA) on the gfx950 fp8 matrix core.  q, k and v hold OCP e4m3 ("e4m3fn") codes, one byte per
 * element, laid out as the 16-bit tensors of ffpa_fwd; the per-head
 * dequantisation factors make the tensors that take part
 *
 *   Q' = q_descale[b, hq] * Q,  K' = k_descale[b, hk] * K,  V' = v_descale[b, hk] * V,
 *
 * and the result is ffpa_fwd's over them: O = softmax(scale Q' K'^T + mask) V'
 * in out_dtype (bf16 or fp16) and the natural-log LSE in fp32.  The factors
 * are folded into the kernels' arithmetic (the "scale folding" named on the
 * skills page), never applied to the tensors.
 *
 *   q            device, [B, Hq, Nq, D] e4m3 bytes, contiguous
 *   k, v         device, [B, Hkv, Nkv, D] e4m3 bytes, contiguous
 *   q_descale    device, [B, Hq] float32, positive and finite; NULL = all 1
 *   k_descale, v_descale  device, [B, Hkv] float32, positive and finite;
 *                NULL = all 1 (other values give unspecified results: the
 *                kernels cannot check device memory)
 *   mask, o, lse, B, Hq, Hkv, Nq, Nkv, scale, is_causal, stream: as for ffpa_fwd
 *   D            16 <= D <= 1024, D % 16 == 0 (FFPA_ERR_UNSUPPORTED otherwise);
 *                a D other than 128, 256, 384, 512, 768 or 1024 runs the next
 *                of those up with padding columns (zeros in Q, never stored
 *                in O; K and V must then hold finite codes)
 *   out_dtype    ffpa_dtype of o (FFPA_ERR_TYPE otherwise)
 *
 * Both products run on e4m3 operands with fp32 accumulation: the
 * probabilities are rounded to e4m3 (round to nearest even) for the P V
 * product, so O carries a relative error of about 2^-4 / sqrt(3) per weight
 * (the tolerance the tests derive); the LSE is exact up to fp32 rounding.
 * q, k, v and o must be 16-byte aligned, the factors 4-byte aligned; o must
 * not overlap q, k, v, lse, the mask or the factors.  Errors as ffpa_fwd.
 * Allocates nothing.
 */
int ffpa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                 const float* v_descale, const ffpa_mask_t* mask, void* o, float* lse, int64_t B, int64_t Hq,
                 int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int out_dtype,
                 void* stream);

/* The host-side argument check ffpa_fwd_fp8 performs, without enqueuing
 * anything. */
int ffpa_check_fp8_args(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                        const float* v_descale, const ffpa_mask_t* mask, const void* o, const float* lse, int64_t B,
                        int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal,
                        int out_dtype);

/* Head dim of the fp8 kernel serving D (the next of 128, 256, 384, 512, 768
 * and 1024), 0 for an unsupported D.  Host-only. */
int64_t ffpa_fp8_kernel_head_dim(int64_t D);

/*
 * ffpa_clock_stamps -- measurement aid.  While `stamps` is non-NULL, every
 * forward launch (ffpa_fwd, ffpa_fwd_strided, ffpa_fwd_dropout,
 * ffpa_fwd_varlen, ffpa_fwd_fp8) enqueued by the calling thread makes the
 * first wave of its workgroup 0 write the GPU's shader-clock counter and its
 * 100 MHz real-time counter at that wave's start (stamps[0], stamps[1]) and
 * end (stamps[2], stamps[3]); the shader clock over that span is
 * (stamps[2] - stamps[0]) * 100 / (stamps[3] - stamps[1]) MHz.  `stamps` is
 * a device pointer to 4 uint64 owned by the caller (8-byte aligned, else
 * FFPA_ERR_VALUE); NULL turns the aid off.  The setting is the calling
 * thread's own; nothing is allocated.  Host-only.
 */
int ffpa_clock_stamps(unsigned long long* stamps);

/*
 * ffpa_fwd_varlen -- enqueue the attention forward over a packed batch of
 * sequences of different lengths (ffpa-attn "API Reference" page,
 * ffpa_attn_varlen_func: packed THD layout, cumulative sequence offsets,
 * longest lengths, and an [H_q, T_q] fp32 LSE).  Sequence b takes query
 * tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key tokens
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1, and each sequence is one dense
 * problem of the form above (GQA heads, tail-aligned causal rule with its own
 * Nq_b and Nkv_b; no mask).
 *
 *   q, o  device, [Tq, Hq, D], contiguous, dtype elements (o written)
 *   k, v  device, [Tk, Hkv, D], contiguous, dtype elements
 *   cu_seqlens_q, cu_seqlens_k  device, B+1 int32 each: 0 = c[0] <= c[1] <= ...
 *         <= c[B] = Tq (resp. Tk).  May be the same array.
 *   lse   device, [Hq, Tq] float32, natural log; written; NULL skips it
 *   B >= 1, Hq >= 1, Hkv >= 1 with Hq % Hkv == 0, Tq >= 0, Tk >= 0
 *   max_seqlen_q, max_seqlen_k  at least every sequence's query (key) length;
 *         they size the grid and the kernels' 32-bit offsets
 *   D, scale, dtype, stream  as for ffpa_fwd
 *   is_causal  0 or 1.  A sequence with fewer keys than queries is allowed:
 *         its first Nq_b - Nkv_b rows see no key, and every row that sees no
 *         key (also any row of a sequence with no keys) gets O = 0 and
 *         LSE = -inf.
 *
 * The offsets live in device memory, so the host cannot read them: offsets
 * that break the rules above give unspecified values in o and lse (the
 * kernels clamp every sequence to [0, Tq) and [0, Tk) and to the longest
 * lengths, so no access leaves the tensors), and rows past max_seqlen_q of a
 * longer sequence are not written.  ffpa_check_cu_seqlens checks a host copy.
 * q, k, v and o must be 16-byte aligned (pointers of empty tensors may be
 * NULL); o must not overlap q, k, v, lse or the offsets.  Tq == 0 or
 * max_seqlen_q == 0 enqueues nothing.  Other rules as for ffpa_fwd.
 */
int ffpa_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t Tq, int64_t Tk, int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D, float scale,
                    int is_causal, int dtype, void* stream);

/* The host-side argument check ffpa_fwd_varlen performs (the offsets are not
 * read), without enqueuing anything. */
int ffpa_check_varlen_args(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, const void* o, const float* lse, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t Tq, int64_t Tk, int64_t max_seqlen_q, int64_t max_seqlen_k,
                           int64_t D, float scale, int is_causal, int dtype);

/* Checks a HOST copy of B+1 cumulative offsets against the rules of
 * ffpa_fwd_varlen: c[0] == 0, non-decreasing, c[B] == T, and every length
 * c[b+1] - c[b] <= max_seqlen.  FFPA_ERR_VALUE (with a detail) if not.
 * Host-only; reads cu_host[0..B]. */
int ffpa_check_cu_seqlens(const int32_t* cu_host, int64_t B, int64_t T, int64_t max_seqlen);

#ifdef __cplusplus
}
#endif

#endif /* FFPA_H_ */
