/*
 * fa_gfx950.h -- C ABI of the exact tiled attention library for MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention in BF16 as described on
 * the FlashAttention-4 pages:
 *   - forward (lecompute.fr FA4 article, section "Between the matrix products the
 *     kernel must produce weights"; fdeinterviews.com FA4 summary, opening
 *     paragraph): S = scale * Q K^T, a row softmax P (positive, rows summing to one),
 *     O = P V, computed tile by tile with an online softmax so that the score matrix
 *     never exists in device memory; the natural-log log-sum-exp of each row,
 *     LSE_i = ln sum_j exp(S_ij), is written beside O for the backward;
 *   - backward (fdeinterviews.com FA4 summary, "Paired-CTA backward pass" bullet and
 *     features paragraph): dQ, dK, dV from the saved LSE, with dQ accumulated by
 *     atomic adds or, in deterministic mode, by a fixed-order reduction whose result
 *     is bit-identical from run to run;
 *   - causal masks and packed variable-length batches, with work ordered longest
 *     first (fdeinterviews.com FA4 summary, features paragraph).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP global memory) owned by the caller.
 *     The library allocates no device memory, keeps no state between calls beyond
 *     its loaded code object, never synchronizes the host, and is reentrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream); all
 *     device work of a call is enqueued on it, in order.
 *   - Every argument is validated before any HIP call.  On a non-FA_OK return no
 *     device work has been enqueued (except FA_ERR_HIP, reported when a launch
 *     fails).  Faults inside kernels surface asynchronously on the stream.
 *   - Tensor layouts: fixed length Q/K/V/O/dO are [B, S, H, D] with arbitrary
 *     element strides for B, S and H (given per tensor) and D contiguous.  Variable
 *     length tensors are packed [T, H, D] (the batch stride is ignored) with
 *     sequence b occupying rows cu_seqlens[b] .. cu_seqlens[b+1]-1.
 *     Base pointers must be 16-byte aligned and the S and H strides multiples of 8
 *     elements.  bf16 is the IEEE binary32 upper half (bfloat16).
 *   - LSE is fp32, natural log, with the softmax scale included: [B, H, S_q]
 *     contiguous for fixed length, [H, total_q] for variable length.
 *   - cu_seqlens arrays live in device memory, hold batch+1 non-decreasing int32
 *     entries starting at 0 and ending at total_q (total_k).  Their contents are
 *     trusted (not validated).
 *   - Causal masking hides key j from query i (both counted from the start of
 *     their sequence) when j > i + L_k - L_q: the mask's diagonal ends at the last
 *     query and the last key (bottom-right alignment), which is the usual j > i
 *     for equal lengths and puts L_q < L_k queries at the end of the key sequence,
 *     as in generation with a cache.  Per sequence for variable length.
 *   - A query row that sees no key gets O = 0 and LSE = -inf.
 *   - NaN/Inf in the data are propagated, not checked.
 */
#ifndef FA_GFX950_H
#define FA_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad stride, ... */
  FA_ERR_UNSUPPORTED = 2,        /* valid request the library does not implement  */
  FA_ERR_WORKSPACE_TOO_SMALL = 3,
  FA_ERR_HIP = 4                 /* a HIP launch or runtime call failed */
} fa_status;

typedef enum fa_dtype { FA_DTYPE_BF16 = 0, FA_DTYPE_F32 = 1 } fa_dtype;

/* Arguments of the forward pass. */
typedef struct fa_fwd_args {
  const void* q;         /* bf16 [B,S_q,H,D] or [T_q,H,D]                          */
  const void* k;         /* bf16 [B,S_k,H,D] or [T_k,H,D]                          */
  const void* v;         /* bf16, same shape as k                                  */
  void* o;               /* out: bf16, same shape as q                             */
  float* lse;            /* out: fp32 [B,H,S_q] or [H,T_q]                         */
  int64_t q_stride[3];   /* element strides {batch, seq, head}                     */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int32_t batch;         /* B (number of sequences for variable length)            */
  int32_t seqlen_q;      /* S_q (fixed length; ignored when cu_seqlens_q != NULL)  */
  int32_t seqlen_k;      /* S_k (fixed length)                                     */
  int32_t num_heads;     /* H (same for Q, K and V)                                */
  int32_t head_dim;      /* D: 64 or 128                                           */
  const int32_t* cu_seqlens_q;  /* device, batch+1 entries, or NULL (fixed length) */
  const int32_t* cu_seqlens_k;  /* device, or NULL (then equal to cu_seqlens_q)    */
  int32_t max_seqlen_q;  /* variable length: upper bound of any query length      */
  int32_t max_seqlen_k;
  int32_t total_q;       /* variable length: T_q = cu_seqlens_q[batch]             */
  int32_t total_k;
  float softmax_scale;   /* finite and > 0, e.g. 1/sqrt(D); else see fa_fwd       */
  int32_t causal;        /* 0 or 1                                                 */
  int32_t o_dtype;       /* FA_DTYPE_BF16 (0, the default) or FA_DTYPE_F32: O in fp32,
                            the normalised output before its bf16 rounding (a
                            diagnostic; o_stride then counts fp32 elements)          */
} fa_fwd_args;

/* Optional forward variant selection (NULL = defaults).  The knobs select among
 * compiled kernel instances; values without an instance give FA_ERR_UNSUPPORTED.
 * The defaults (hardware exponential only, threshold 8, two query tiles, key split
 * chosen from the shape) are the fast path; the other values exist so that each
 * of the method's choices can be measured against its alternative, and the
 * exp2-share and threshold alternatives are compiled for head_dim 128 with fixed
 * length only. */
typedef struct fa_fwd_tuning {
  /* Of every 16 score registers of a lane, how many take the FMA-only exp2
   * (integer/fraction split, cubic on the fraction, integer added to the exponent
   * field; fdeinterviews.com FA4 summary, "Software exponentials" bullet) instead of
   * the hardware v_exp_f32.  Compiled: 0, 2, 4.  -1 = default (0, the measured
   * fastest). */
  int32_t exp2_poly_per16;
  /* Lazy rescale threshold in log2 units (fdeinterviews.com FA4 summary, "Lazy
   * rescaling" bullet): the output is rescaled only when a row's maximum grows by
   * more than this.  Compiled: 8 (the method) and 0 (eager).  -1 = default (8). */
  int32_t rescale_threshold_log2;
  /* Query tiles of 128 rows interleaved per workgroup (two wave sets sharing each
   * K/V stage; fdeinterviews.com FA4 summary, "Pipeline for asynchronous tensor
   * cores" bullet).  Compiled: 1, 2.  -1 = default (2). */
  int32_t q_tiles_per_workgroup;
  /* Split of each sequence's keys into this many contiguous chunks, each handled
   * by its own workgroups (128-row query tiles); every chunk writes a partial O
   * (fp32) and LSE to the workspace and a merge pass combines them:
   * LSE = ln sum_c e^LSE_c, O = sum_c e^(LSE_c - LSE) O_c.  For short query
   * sequences against long key sequences (generation with a cache; fdeinterviews.com
   * FA4 summary, paragraph on long-context inference and training), where the query
   * tiles alone cannot fill the GPU.  1 = no split; 2..64 = that many; 0 or negative =
   * chosen from the shape. */
  int32_t key_splits;
} fa_fwd_tuning;

/* Bytes of device workspace fa_fwd needs for `a` and `tuning` (NULL = defaults):
 * room for the longest-first work list of variable-length batches (fdeinterviews.com
 * FA4 summary, features paragraph), and either for the partial results of a key
 * split (fp32 O and LSE per chunk) or, without a split, for an fp16 copy of V with
 * one power-of-two exponent per 64-key tile (2 bytes per V element plus 4 bytes per
 * key row and head): the unsplit PV product runs in fp16, so that the weights keep
 * 11 significant bits under the lazy reference.  0 only for an empty problem.  Validates `a` and `tuning` exactly as fa_fwd does and
 * returns the same status; `bytes` must not be NULL (FA_ERR_INVALID_ARGUMENT).  No
 * HIP call is made. */
fa_status fa_fwd_workspace_size(const fa_fwd_args* a, const fa_fwd_tuning* tuning, size_t* bytes);

/* Forward pass (lecompute.fr FA4 article, section "Between the matrix products the
 * kernel must produce weights"; fdeinterviews.com FA4 summary, opening paragraph,
 * "Lazy rescaling" and "Software exponentials" bullets): writes O (bf16, layout of
 * q) and LSE (fp32, natural log, scale included) for every query row, tiling Q
 * against K/V with an online softmax so that no score reaches device memory.
 * `workspace` (device, 256-byte aligned, at least fa_fwd_workspace_size bytes,
 * contents ignored on entry and clobbered) may be NULL when that size is 0.
 * Errors, all reported before any device work is enqueued:
 *   FA_ERR_INVALID_ARGUMENT  NULL or misaligned pointer, negative size, stride
 *                            smaller than head_dim or not a multiple of 16
 *                            bytes, causal not 0/1, o_dtype not BF16/F32,
 *                            non-finite scale;
 *   FA_ERR_UNSUPPORTED       head_dim not 64/128, scale <= 0 (the kernels fold
 *                            the scale into the exponent after taking row maxima
 *                            of the raw scores, which needs a positive scale),
 *                            offsets beyond 2^31 bytes per sequence, sequences
 *                            longer than 524,288, a tuning without an instance;
 *   FA_ERR_WORKSPACE_TOO_SMALL  workspace NULL or smaller than required;
 *   FA_ERR_HIP               a kernel launch failed.
 * An empty batch (batch = 0 or no query rows) returns FA_OK with no work.
 * V elements must be below 2^31 in magnitude (the fp16 copy's exponent range);
 * max_seqlen_k must bound every key length (it sizes the copy's grid). */
fa_status fa_fwd(const fa_fwd_args* a, const fa_fwd_tuning* tuning, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Builds only the longest-first work list of a variable-length forward into
 * `workspace` (the first step of fa_fwd for variable length; fdeinterviews.com FA4
 * summary, features paragraph: tiles are dispatched most expensive first), so that
 * it can be inspected.  Layout: int32 count n, then n pairs {sequence, query tile},
 * tiles of `fa_fwd_tile_rows` rows, in dispatch order.  Longest first by cost
 * bucket: with cost = key tiles visited (64 keys each) and bucket = cost / w,
 * w = 16 * tile_rows / 64, the bucket never increases along the list; inside a
 * bucket each sequence's items form one run of non-increasing cost (the runs of
 * different sequences may come in any order), so that neighbouring tiles of one
 * sequence run together and share its K/V in L2.  Errors as fa_fwd, plus
 * FA_ERR_INVALID_ARGUMENT for a fixed-length `a`. */
fa_status fa_fwd_build_schedule(const fa_fwd_args* a, const fa_fwd_tuning* tuning,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Query rows per forward work item for the given tuning (NULL = defaults): the
 * tile size of the work list above.  0 for a tuning without an instance. */
int32_t fa_fwd_tile_rows(const fa_fwd_tuning* tuning);

/* Diagnostic: evaluates, for n fp32 values x (device), the two ways the forward
 * forms the softmax weights 2^x -- the software exponential that splits x into an
 * integer and a fraction, evaluates a cubic on the fraction with multiply-adds and
 * adds the integer to the exponent bits (FA4 summary page, "Software exponentials"
 * bullet; lecompute.fr article, section "Move some exponential work to different
 * units"), into y_poly, and the hardware v_exp_f32 into y_hw -- exactly as the
 * forward kernel evaluates them.  The software path is valid for x <= 8 (the lazy
 * rescale bound) and returns 0 for x < -126.  All three arrays are caller-owned
 * device memory of n floats; n = 0 does nothing; n < 0 or a NULL array with n > 0
 * is FA_ERR_INVALID_ARGUMENT.  Enqueued on `stream`. */
fa_status fa_exp2_probe(const float* x, float* y_poly, float* y_hw, int64_t n, void* stream);

/* Arguments of the backward pass. */
typedef struct fa_bwd_args {
  const void* q;         /* bf16, as in the forward                                */
  const void* k;
  const void* v;
  const void* o;         /* bf16 forward output                                    */
  const void* dout;      /* bf16 gradient of the loss w.r.t. O, shape of o         */
  const float* lse;      /* fp32 LSE written by fa_fwd (same layout)               */
  void* dq;              /* out: grad_dtype, shape of q                            */
  void* dk;              /* out: grad_dtype, shape of k                            */
  void* dv;              /* out: grad_dtype, shape of v                            */
  int64_t q_stride[3];   /* element strides {batch, seq, head} of each tensor      */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int64_t do_stride[3];
  int64_t dq_stride[3];
  int64_t dk_stride[3];
  int64_t dv_stride[3];
  int32_t batch;
  int32_t seqlen_q;
  int32_t seqlen_k;
  int32_t num_heads;
  int32_t head_dim;      /* 64 or 128 */
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int32_t total_q;
  int32_t total_k;
  float softmax_scale;
  int32_t causal;
  int32_t deterministic; /* 0: dQ by atomic adds; 1: fixed-order, bit-reproducible */
  int32_t grad_dtype;    /* FA_DTYPE_F32 (default) or FA_DTYPE_BF16                */
} fa_bwd_args;

/* Bytes of device workspace fa_bwd needs for `a`: the fp32 dQ accumulator (atomic
 * mode only), the row terms D_i = sum_d dO_id O_id, the fp16 copies of Q and K that
 * the dS products use (2 * head_dim bytes per query row and per key row, per head),
 * the pre pass's magnitude maxima (128 KiB) and the work lists of variable-length
 * batches.  Validates `a` exactly as fa_bwd does and returns the
 * same status; `bytes` must not be NULL.  No HIP call is made. */
fa_status fa_bwd_workspace_size(const fa_bwd_args* a, size_t* bytes);

/* Backward pass (fdeinterviews.com FA4 summary, "Paired-CTA backward pass" bullet
 * and features paragraph: a backward from the saved log-sum-exp whose dQ is added
 * with atomics, with a deterministic mode): writes dQ, dK, dV (grad_dtype, layouts
 * of q, k, v) of the loss whose gradient with respect to O is dout, recomputing the
 * softmax weights from q, k and lse; the equations are the textbook gradient of
 * softmax attention (dV = P^T dO, dS = P o (dO V^T - D), dQ = scale dS K,
 * dK = scale dS^T Q).  deterministic = 1 reduces dQ in a fixed order (bit-identical
 * results from run to run on one GPU); 0 adds it with fp32 atomics.  `workspace` as
 * for fa_fwd (required: the row terms always live there).  Errors as for fa_fwd,
 * plus FA_ERR_INVALID_ARGUMENT for deterministic or grad_dtype out of range. */
fa_status fa_bwd(const fa_bwd_args* a, void* workspace, size_t workspace_bytes, void* stream);

/* The backward of fa_bwd (same passages, arguments and errors) split into its three
 * phases, enqueued in this order by fa_bwd:
 *   FA_BWD_PHASE_PRE:  row terms D_i = sum_d dO_id O_id into the workspace (and, in
 *                      atomic mode, zeroing of the fp32 dQ accumulator);
 *   FA_BWD_PHASE_MAIN: the key-block kernel: dK and dV (and, in atomic mode, dQ
 *                      added by fp32 atomics into the accumulator);
 *   FA_BWD_PHASE_POST: dQ in dQ's layout and dtype: atomic mode converts the
 *                      accumulator; deterministic mode runs the query-block kernel
 *                      that reduces dQ in a fixed order.
 * fa_bwd_phases runs the selected subset (a bitwise OR) on the same arguments and
 * workspace, so callers can time or interleave them; a phase reads what the earlier
 * phases left in the workspace, so running MAIN without a preceding PRE on that
 * workspace gives undefined gradients.  `phases` outside 1..7 is
 * FA_ERR_INVALID_ARGUMENT. */
enum { FA_BWD_PHASE_PRE = 1, FA_BWD_PHASE_MAIN = 2, FA_BWD_PHASE_POST = 4, FA_BWD_PHASE_ALL = 7 };
fa_status fa_bwd_phases(const fa_bwd_args* a, int32_t phases, void* workspace, size_t workspace_bytes,
                        void* stream);

/* The backward of fa_bwd (same arguments, results and errors) for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Its workspace is a static device
 * array inside the library (fa_bwd_noalloc_scratch_bytes() bytes, 64 MiB, one copy
 * per GPU, held until the process ends); the call allocates nothing.  A request whose
 * workspace (fa_bwd_workspace_size) exceeds that size returns
 * FA_ERR_WORKSPACE_TOO_SMALL before any device work: per head the deterministic
 * mode needs 4 + 2 * head_dim bytes per query row and 2 * head_dim bytes per key row,
 * plus 128 KiB and the work lists of variable-length batches; the atomic mode adds
 * 4 * head_dim bytes per query row and head (e.g. B=1 S=4096 H=16 d=128 fits
 * deterministically, B=2 S=8192 does not).  Every call on a
 * GPU uses that GPU's one array, whose contents carry over from the last call (each
 * call writes everything it reads): calls that overlap in time on one GPU -- on
 * different streams, or from different threads -- race and give undefined
 * gradients.  FA_ERR_HIP if the array's address cannot be obtained. */
fa_status fa_bwd_noalloc(const fa_bwd_args* a, void* stream);

/* Size in bytes of the static workspace fa_bwd_noalloc uses. */
size_t fa_bwd_noalloc_scratch_bytes(void);

/* Static name of a status code, e.g. "FA_ERR_UNSUPPORTED" ("FA_ERR_UNKNOWN" for a
 * value outside the enum; never NULL).  The codes are this library's own; the
 * pages define no interface (the argument set follows the operation: Q, K, V, the
 * softmax scale, the causal flag and packed lengths). */
const char* fa_status_str(fa_status s);

/* Library version string (static, never NULL). */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_GFX950_H */
