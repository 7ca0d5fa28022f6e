/*
 * liblce -- cross-entropy over a tokens x vocab logit matrix, for AMD Instinct
 * MI355X (gfx950).  C ABI: plain pointers, sizes and a HIP stream; no C++ or
 * framework types cross this boundary.
 *
 * Operations (KernelIndex pages; the loss formula itself is not printed there
 * and is read as textbook softmax cross-entropy in natural log):
 *
 *   per token i:   loss_i = ln( sum_j exp(z_ij) ) - z_{i, t_i}
 *   mean:          (1 / tokens) * sum_i loss_i
 *
 * on a stored logit matrix or on logits z = x * W^T formed on the fly from
 * bf16 activations and an LM head; with its gradients, the two local halves
 * of a vocab split across devices, per-sequence sums of target
 * log-probabilities, and a generalized Jensen-Shannon divergence between a
 * student's and a teacher's projections.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     row-major and contiguous.  The caller owns every buffer; liblce never
 *     frees or retains a caller pointer after the call returns.
 *   - Inputs are never written.  `out` must not overlap any input
 *     (each page's Semantics block rules out mutating or aliasing inputs).
 *   - Calls are asynchronous: work is enqueued on `stream` (0 = the null
 *     stream) and the call returns without synchronising.  Argument errors are
 *     reported synchronously, before anything is enqueued; a failed launch is
 *     reported as LCE_ERR_HIP.  Faults during execution surface at the
 *     caller's next synchronisation, as for any HIP kernel.
 *   - Targets are int64 class indices.  A target outside [0, vocab) is a
 *     contract violation: that token's loss is NaN (so is the mean), and no
 *     out-of-bounds read happens.  There is no ignore_index: no page
 *     mentions one.
 *   - Losses are always fp32; accumulation is fp32.
 *   - Results are bitwise reproducible run to run for the same inputs, shape
 *     and device: every reduction has a fixed order and no float atomics are
 *     used (the pages do not specify determinism).  The fused backward's two
 *     GEMMs run the algorithm hipBLASLt's heuristic picks for the shape.
 *   - liblce keeps a device scratch buffer per (device, stream), grown on
 *     demand with hipMalloc to 1.25x the need.  It is small (per-token and
 *     per-workgroup partials) except for lce_fused_linear_jsd_fwd and
 *     lce_fused_linear_xent_bwd, which keep up to LCE_JSD_STORE_BYTES and
 *     LCE_FUSED_BWD_STORE_BYTES (default 2 GiB each) of logits there (the
 *     backward also 128 MiB of GEMM workspace).  An
 *     outgrown buffer is retired, never freed: every scratch buffer is kept
 *     until the process ends, so the retired ones add up to at most 4x the
 *     live one.  Calls on one stream are ordered by the stream; calls on
 *     different streams use different scratch buffers.
 *   - HIP graph capture: a call may be captured if an earlier, uncaptured
 *     call on the same stream and device already grew its scratch far enough
 *     (the largest shape to be captured is enough); otherwise the call fails
 *     with LCE_ERR_UNSUPPORTED before anything is enqueued.  A captured call
 *     keeps using the scratch of the stream it was captured on, so replays
 *     must not run concurrently with other liblce work on that stream.
 *   - No call throws; every error is a status code plus a thread-local
 *     message (lce_last_error).
 */
#ifndef LCE_H
#define LCE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; only these entry points are exported. */
#define LCE_API __attribute__((visibility("default")))

#define LCE_VERSION_MAJOR 0
#define LCE_VERSION_MINOR 6
#define LCE_VERSION_PATCH 0

/* The enums are passed as int.  A caller may pass any int value (a bad one is
 * rejected with LCE_ERR_INVALID_ARG), so C++ gives them int as a fixed
 * underlying type: every int is then a valid value of the enum type, and the
 * library reads such an argument without undefined behaviour.  In C an enum
 * with these constants is int-sized too, so the ABI is the same. */
#ifdef __cplusplus
#define LCE_ENUM enum : int
#else
#define LCE_ENUM enum
#endif

typedef LCE_ENUM {
    LCE_F32 = 0,  /* IEEE binary32 logits */
    LCE_BF16 = 1  /* bfloat16 logits (upper 16 bits of a binary32) */
} lce_dtype;

typedef LCE_ENUM {
    LCE_REDUCTION_MEAN = 0, /* out[0] = mean of the per-token losses */
    LCE_REDUCTION_NONE = 1  /* out[i] = loss of token i */
} lce_reduction;

typedef LCE_ENUM {
    LCE_OK = 0,
    LCE_ERR_INVALID_ARG = 1, /* NULL pointer, negative or zero size, bad enum */
    LCE_ERR_UNSUPPORTED = 2, /* valid but not handled (see each call) */
    LCE_ERR_ALIAS = 3,       /* out overlaps an input */
    LCE_ERR_OOM = 4,         /* scratch allocation failed */
    LCE_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} lce_status;

/*
 * Row-wise softmax cross-entropy over a logit matrix.
 *
 * Defines: KernelIndex "Cross-entropy loss" (description; Semantics: logits
 * float [tokens, vocab], target int64 [tokens], loss float [1]) and
 * "Vocab-parallel cross-entropy, Megatron layout" (description; Semantics:
 * logits float [seq, batch, vocab], target int64 [seq, batch], loss fp32
 * [seq, batch]; only the TP=1 case, where each device holds the whole vocab).
 *
 *   logits    device, `tokens * vocab` elements of `dtype`, row-major: row i
 *             holds token i's vocab logits.  A [seq, batch, vocab] tensor is
 *             passed as tokens = seq * batch (row = s * batch + b).  Must be
 *             aligned to its element size; any vocab >= 1 is accepted (rows
 *             need not be 16-byte aligned).
 *   dtype     LCE_F32 or LCE_BF16.
 *   tokens    number of rows, >= 0.
 *   vocab     number of classes, 1 <= vocab < 2^31.
 *   target    device, `tokens` int64 class indices (same row order).  May be
 *             NULL only when tokens == 0.
 *   reduction LCE_REDUCTION_MEAN: out[0] = mean loss (NaN when tokens == 0).
 *             LCE_REDUCTION_NONE: out[i] = loss_i, i < tokens (nothing is
 *             written when tokens == 0).
 *   out       device fp32, 1 or `tokens` elements; 4-byte aligned; must not
 *             overlap logits or target.
 *   stream    HIP stream the work is enqueued on.
 *
 * Returns LCE_OK, LCE_ERR_INVALID_ARG (NULL pointer, tokens < 0, vocab < 1,
 * bad enum, misaligned pointer), LCE_ERR_UNSUPPORTED (vocab >= 2^31, or
 * scratch that would have to grow under graph capture), LCE_ERR_ALIAS,
 * LCE_ERR_OOM or LCE_ERR_HIP.
 */
LCE_API lce_status lce_xent_fwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                        const int64_t* target, lce_reduction reduction, float* out,
                        hipStream_t stream);

/*
 * lce_xent_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels, path selection, results (bitwise) and errors as
 * lce_xent_fwd, but the call makes no hipMalloc or hipFree and uses no
 * allocating library routine: its scratch (the mean's epoch word and
 * per-workgroup slots, the split path's partials) lives in one static 8 MiB
 * device array per GPU, held until the process ends.
 *
 * Limits: with LCE_REDUCTION_MEAN at most 2^19 workgroup slots (a mean over
 * at most 2^23 rows of 2 to 32 KiB, 16 rows per workgroup, or of rows with
 * scalar edges; rows of at most 2 KiB without edges take 32, 16 or 8 rows per
 * workgroup for rows of at most 512 B, 1 KiB or 2 KiB, so at most 2^24, 2^23
 * or 2^22 rows), and the split path's partials (8 bytes per row and slice)
 * within 4 MiB; a call beyond them returns LCE_ERR_UNSUPPORTED before
 * anything but the first call's clear is enqueued.
 *
 * Every call on a GPU shares that GPU's array, and the array keeps the last
 * call's contents between calls: calls that overlap on one GPU (concurrent
 * streams, threads or graph replays) race and must be serialised by the
 * caller.  The first call on a GPU also clears the array's mean state with a
 * kernel on `stream` (when that call is being captured into a HIP graph, the
 * clear is captured too and the next uncaptured call clears again).
 */
LCE_API lce_status lce_xent_fwd_noalloc(const void* logits, lce_dtype dtype, int64_t tokens,
                                        int64_t vocab, const int64_t* target,
                                        lce_reduction reduction, float* out, hipStream_t stream);

/*
 * Gradient of the cross-entropy with respect to the logits (the backward
 * step of lce_xent_fwd).  The pages give the forward only; this is its
 * derivative, softmax minus the one-hot target:
 *
 *     dlogits_ij = g_i * (e^(z_ij - lse_i) - [j == t_i]),  lse_i = ln sum_k e^(z_ik)
 *
 *   logits, dtype, tokens, vocab, target: as lce_xent_fwd.
 *   reduction  the reduction of the forward call whose gradient this is.
 *   grad       device fp32 gradient of the forward's output: 1 element for
 *              LCE_REDUCTION_MEAN (then g_i = grad[0] / tokens), `tokens`
 *              elements for LCE_REDUCTION_NONE (g_i = grad[i]).
 *   dlogits    device, same dtype and layout as logits (bf16 results are
 *              rounded to nearest even), starting at the same byte offset
 *              modulo 16 as logits (else LCE_ERR_UNSUPPORTED).  May be the
 *              logits buffer itself (computed in place); must not otherwise
 *              overlap logits, and must not overlap target or grad.
 *   stream     HIP stream.
 *
 * A row whose target is outside [0, vocab) gets a NaN gradient row.  Rows of
 * up to 32 KiB are read once and written once; longer rows are read twice.
 * Nothing is written when tokens == 0.  Returns as lce_xent_fwd.
 */
LCE_API lce_status lce_xent_bwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                        const int64_t* target, lce_reduction reduction, const float* grad,
                        void* dlogits, hipStream_t stream);

/*
 * The forward and the backward of the row cross-entropy in one call: the
 * losses (or their mean) of lce_xent_fwd and the logit gradient of
 * lce_xent_bwd, for a training step whose output gradient `grad` is known
 * before the loss (for a mean loss, usually 1).  Rows of up to 32 KiB are read
 * once and the gradient written once, against one read for lce_xent_fwd and
 * a read and a write for lce_xent_bwd; the loss comes from the same row state
 * as the gradient.
 *
 *   logits, dtype, tokens, vocab, target, reduction: as lce_xent_fwd.
 *   grad, dlogits: as lce_xent_bwd (dlogits may be the logits buffer).
 *   out        device fp32, as lce_xent_fwd's; must not overlap logits,
 *              target, grad or dlogits.
 *   stream     HIP stream.
 *
 * dlogits is bitwise what lce_xent_bwd writes.  The losses agree with
 * lce_xent_fwd's within the forward's tolerance but not always bitwise: for
 * rows of up to 32 KiB they come from the gradient kernel's own fold of the
 * row (the running-maximum fold rather than the forward kernels' fixed
 * reference).  A row whose target is outside [0, vocab) has a NaN loss (and
 * a NaN mean) and a NaN gradient row.  tokens == 0 writes NaN for a mean and
 * nothing else.  Returns as lce_xent_fwd.
 */
LCE_API lce_status lce_xent_fwd_bwd(const void* logits, lce_dtype dtype, int64_t tokens, int64_t vocab,
                                    const int64_t* target, lce_reduction reduction, const float* grad,
                                    float* out, void* dlogits, hipStream_t stream);

/*
 * Vocab-shard statistics: the per-row quantities one device contributes when
 * the vocab axis is split across devices.
 *
 * Defines: KernelIndex "Vocab-parallel cross-entropy, Megatron layout"
 * (description: cross-entropy with the vocab axis split across devices; the
 * page measures only the one-device case).  Each device holds the logits of a
 * contiguous vocab range [vocab_start, vocab_start + shard_vocab) for every
 * token and calls this on them; gathering the 12 bytes per token from all
 * devices and calling lce_xent_merge gives every device the full loss.
 *
 *   logits       device, `tokens * shard_vocab` elements of `dtype`,
 *                row-major: row i holds token i's logits of this vocab range
 *                (alignment and layout as for lce_xent_fwd).
 *   shard_vocab  columns held, 1 <= shard_vocab < 2^31.
 *   vocab_start  full-vocab index of column 0, >= 0.
 *   target       device int64 [tokens], indices into the FULL vocab.
 *   partial      device fp32 [tokens][3], 4-byte aligned, must not overlap
 *                the inputs; row i receives
 *                  m  = max_j z_ij over this range,
 *                  s  = sum_j e^(z_ij - m)   (m + ln s is the range's
 *                       log-sum-exp; a row of -inf only gives (-inf, 0)),
 *                  zt = z_{i, t_i} if vocab_start <= t_i < vocab_start +
 *                       shard_vocab, else NaN (another device holds it).
 *   stream       HIP stream.
 *
 * Nothing is written when tokens == 0.  Returns as lce_xent_fwd.
 */
LCE_API lce_status lce_xent_partial_fwd(const void* logits, lce_dtype dtype, int64_t tokens,
                                int64_t shard_vocab, int64_t vocab_start, const int64_t* target,
                                float* partial, hipStream_t stream);

/*
 * Loss from the vocab-shard statistics of all devices (same page and section
 * as lce_xent_partial_fwd).  For each token the shards' (m, s) are folded in
 * shard order into M = max m and S = sum s e^(m - M), the target logit is the
 * one a shard reported, and loss = (M - zt) + ln S.
 *
 *   partials  device fp32 [shards][tokens][3]: lce_xent_partial_fwd's output
 *             of each shard, in a fixed shard order (the result depends on the
 *             order only through fp32 rounding; one order gives one result).
 *   shards    >= 1;  tokens >= 0.
 *   target    device int64 [tokens] (full-vocab indices).
 *   vocab     full vocab size, >= 1: a target outside [0, vocab), or one no
 *             shard reported, gives NaN.
 *   reduction, out, stream: as lce_xent_fwd (out must not overlap partials
 *             or target).
 *
 * Returns LCE_OK, LCE_ERR_INVALID_ARG (NULL pointer, shards < 1, tokens < 0,
 * vocab < 1, bad enum, misaligned pointer), LCE_ERR_UNSUPPORTED
 * (shards >= 2^31, or scratch that would have to grow under graph capture),
 * LCE_ERR_ALIAS, LCE_ERR_OOM or LCE_ERR_HIP.
 */
LCE_API lce_status lce_xent_merge(const float* partials, int64_t shards, int64_t tokens,
                          const int64_t* target, int64_t vocab, lce_reduction reduction,
                          float* out, hipStream_t stream);

/*
 * Fused LM-head projection + cross-entropy; the logits are never stored.
 *
 * Defines: KernelIndex "Fused linear + CPO loss" (description: activations
 * projected through a vocab x hidden LM head against integer targets,
 * reduced chunk by chunk so the logits are never stored; Semantics: x float
 * [batch, seq, hidden], weight float [vocab, hidden], target int64
 * [batch, seq], loss float [1]).  The loss applied to the projected logits
 * is the same per-token cross-entropy as lce_xent_fwd (the CPO preference
 * term is not part of this call).
 *
 *   x         device bf16 [tokens, hidden], row-major ([batch, seq, hidden]
 *             passed as tokens = batch * seq, row = b * seq + s).
 *   weight    device bf16 [vocab, hidden], row-major (one row per class).
 *   tokens    >= 0;  1 <= hidden < 2^22, a multiple of 8;  1 <= vocab < 2^31.
 *   target    device int64 [tokens].
 *   reduction LCE_REDUCTION_MEAN or LCE_REDUCTION_NONE, as for lce_xent_fwd.
 *   out       device fp32, 1 or `tokens` elements; must not overlap inputs.
 *   stream    HIP stream.
 *
 * logits z = x * weight^T are accumulated in fp32 from exact bf16 products
 * and reduced on the fly into a per-token running (max, sum-exp) and the
 * target logit.
 *
 * Returns as lce_xent_fwd; LCE_ERR_UNSUPPORTED when hidden is not a multiple
 * of 8 or x / weight are not 16-byte aligned.
 */
LCE_API lce_status lce_fused_linear_xent_fwd(const void* x, const void* weight, int64_t tokens,
                                     int64_t hidden, int64_t vocab, const int64_t* target,
                                     lce_reduction reduction, float* out, hipStream_t stream);

/*
 * Per-sequence sums of target log-probabilities under the fused projection:
 * the quantity the "Fused linear + CPO loss" page's preference loss is built
 * from (the page gives the loss only by name; its formula is not on the page,
 * so the preference term itself is not computed here).
 *
 *     out[b] = sum_{s < seq} log softmax(x_{b*seq+s} * weight^T)[t_{b*seq+s}]
 *            = -(sum of the per-token losses of sequence b)
 *
 *   x        device bf16 [batch, seq, hidden] (row b*seq + s), as
 *            lce_fused_linear_xent_fwd with tokens = batch * seq.
 *   weight, hidden, vocab: as lce_fused_linear_xent_fwd.
 *   target   device int64 [batch, seq]; an out-of-range target makes its
 *            sequence's sum NaN.
 *   out      device fp32 [batch]; must not overlap the inputs.  seq == 0
 *            writes zeros; batch == 0 writes nothing.
 *
 * The sum over a sequence is a fixed-order reduction (bitwise reproducible).
 * Returns as lce_fused_linear_xent_fwd.
 */
LCE_API lce_status lce_fused_linear_logprob_sums(const void* x, const void* weight, int64_t batch,
                                         int64_t seq, int64_t hidden, int64_t vocab,
                                         const int64_t* target, float* out, hipStream_t stream);

/*
 * Gradients of the fused projection + cross-entropy (lce_fused_linear_xent_fwd)
 * with respect to the activations and the head.  The pages give only the
 * forward ("Fused linear + CPO loss": description, Semantics); this is its
 * derivative written out.  With z = x * weight^T and per-token output
 * gradient g_i (grad[0] / tokens for a mean, grad[i] per token),
 *
 *     dZ_ij  = g_i (softmax(z_i)_j - [j == t_i])
 *     dx     = dZ * weight        [tokens, hidden]
 *     dweight = dZ^T * x          [vocab, hidden]
 *
 * Per chunk of tokens, the fused kernel forms the logits with their per-token
 * log-sum-exp and keeps them in scratch as fp32, a streaming kernel turns them
 * into dZ as bf16 (round to nearest even), and two hipBLASLt GEMMs (bf16
 * operands, fp32 accumulation) consume it.  The chunk is the largest multiple
 * of 256 tokens whose logits and dZ (6 * tokens * vocab bytes, vocab rounded
 * up to 256) fit in LCE_FUSED_BWD_STORE_BYTES (environment, default 2 GiB).
 * When not even 256 tokens fit, no fp32 logits are kept: the log-sum-exp of
 * every token is taken first and the fused kernel recomputes the logits of
 * each 256-token chunk to write dZ (2 bytes per logit; one more GEMM pass).
 *
 *   x, weight, tokens, hidden, target: as lce_fused_linear_xent_fwd; also
 *             vocab < 2^23 - 256.
 *   reduction LCE_REDUCTION_MEAN or LCE_REDUCTION_NONE: the forward's.
 *   grad      device fp32: 1 element (mean) or `tokens` elements (none).
 *   dx        device fp32 [tokens, hidden], overwritten; NULL skips it.
 *   dweight   device fp32 [vocab, hidden], overwritten (zeros for tokens == 0);
 *             NULL skips it.  At least one of dx, dweight is non-NULL.
 *   stream    HIP stream.
 *
 * A token whose target is outside [0, vocab) gets a NaN row of dx and makes
 * all of dweight NaN (its loss is NaN).  dweight sums over the tokens of each
 * chunk inside the GEMM and over chunks in chunk order (deterministic).
 * Outputs must not overlap the inputs or each other.  The first call of a
 * shape plans its GEMMs (hipBLASLt handle and heuristic); a call inside a graph
 * capture whose shape was never planned, or whose scratch would have to grow,
 * fails with LCE_ERR_UNSUPPORTED.  Returns as lce_fused_linear_xent_fwd,
 * LCE_ERR_HIP also for a failing hipBLASLt call.
 */
LCE_API lce_status lce_fused_linear_xent_bwd(const void* x, const void* weight, int64_t tokens,
                                     int64_t hidden, int64_t vocab, const int64_t* target,
                                     lce_reduction reduction, const float* grad, float* dx,
                                     float* dweight, hipStream_t stream);

/*
 * The forward and the backward of the fused projection + cross-entropy in
 * one call: the losses (or their mean) of lce_fused_linear_xent_fwd together
 * with dx and dweight of lce_fused_linear_xent_bwd, for a training step whose
 * output gradient `grad` is known before the loss.  The backward's first
 * pass over the head already forms every token's log-sum-exp; it also
 * finishes the losses, so the separate forward pass is not needed.
 *
 *   x, weight, tokens, hidden, vocab, target, reduction, grad, dx, dweight,
 *             stream: as lce_fused_linear_xent_bwd.
 *   out       device fp32, as lce_fused_linear_xent_fwd's; must not overlap
 *             x, weight, target, grad, dx or dweight.
 *
 * dx and dweight are bitwise what lce_fused_linear_xent_bwd writes.  The
 * losses are bitwise those of lce_fused_linear_xent_fwd when one chunk of
 * the backward's plan holds every token or the logits are recomputed.  With
 * several chunks of stored logits, each chunk's losses come from its own
 * vocab segmentation and a mean is the fixed-order mean of the per-token
 * losses: both agree with the forward's within its tolerance, and are
 * deterministic.  tokens == 0 writes NaN for a mean and zeros into dweight.
 * Returns as lce_fused_linear_xent_bwd.
 */
LCE_API lce_status lce_fused_linear_xent_fwd_bwd(const void* x, const void* weight, int64_t tokens,
                                                 int64_t hidden, int64_t vocab, const int64_t* target,
                                                 lce_reduction reduction, const float* grad, float* out,
                                                 float* dx, float* dweight, hipStream_t stream);

/*
 * Generalized Jensen-Shannon divergence between a student and a teacher
 * distribution, each from its own fused projection (KernelIndex "Fused linear +
 * JSD": description and Semantics block; beta 0.5 and "batchmean" there).
 * With P = softmax(student_x * student_weight^T), Q = softmax(teacher_x *
 * teacher_weight^T) and M = beta P + (1 - beta) Q, per token
 *
 *     jsd = beta KL(P || M) + (1 - beta) KL(Q || M),   KL(A || B) = sum_j A_j ln(A_j / B_j)
 *
 * (the page names the divergence without printing it; this is the usual
 * generalized form, symmetric at beta = 0.5).  Each head's logits are formed
 * once by the fused projection, which also takes the head's per-token
 * log-sum-exp and writes the fp32 logits of a chunk of tokens to scratch; a
 * streaming pass then sums the divergence terms.  The chunk is the largest
 * multiple of 256 tokens whose two heads' logits (8 * tokens * vocab bytes,
 * vocab rounded up to 256) fit in LCE_JSD_STORE_BYTES (environment, default
 * 2 GiB).  With LCE_JSD_STORE_BYTES=0, or too large a vocab, no logits are
 * stored: a second pass recomputes both heads' logits tile by tile (about
 * twice the time).
 *
 *   student_x, teacher_x            device bf16 [tokens, hidden], row-major.
 *   student_weight, teacher_weight  device bf16 [vocab, hidden], row-major.
 *   tokens >= 0;  1 <= hidden < 2^22, a multiple of 8;  1 <= vocab < 2^31.
 *   beta       in (0, 1); 0.5 is the page's setting.
 *   reduction  LCE_REDUCTION_MEAN: out[0] = sum of jsd over tokens / tokens
 *              ("batchmean"; NaN for tokens == 0), a fixed-order reduction
 *              (bitwise reproducible).  LCE_REDUCTION_NONE: out[i] = jsd of
 *              token i (nothing written for tokens == 0).
 *   out        device fp32, 1 or `tokens` elements; must not overlap inputs.
 *   stream     HIP stream.
 *
 * Returns LCE_ERR_INVALID_ARG for a NULL pointer, a bad size, reduction or
 * beta; LCE_ERR_UNSUPPORTED as lce_fused_linear_xent_fwd; LCE_ERR_ALIAS when
 * out overlaps an input; LCE_ERR_HIP / LCE_ERR_OOM as lce_xent_fwd.
 */
LCE_API lce_status lce_fused_linear_jsd_fwd(const void* student_x, const void* student_weight,
                                    const void* teacher_x, const void* teacher_weight,
                                    int64_t tokens, int64_t hidden, int64_t vocab, float beta,
                                    lce_reduction reduction, float* out, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
LCE_API const char* lce_status_string(lce_status status);

/* Detail message of the last failing call on this thread ("" if none).
 * The pointer stays valid until the next liblce call on this thread. */
LCE_API const char* lce_last_error(void);

/* MAJOR * 10000 + MINOR * 100 + PATCH. */
LCE_API int lce_version(void);

/* What the last call on this thread enqueued, for profilers and benchmarks:
 * the kernels in launch order, joined by " + ", each as its name with the
 * template arguments that select it (as a demangler prints them) and its grid,
 * e.g. "xent_wave_rows_kernel<float, 8, 16> grid 1024 x 1024", and
 * "hipBLASLt GEMM m .. n .. k .." for a library product.  "" after a call that
 * failed before launching anything or had nothing to do.  Not an operation of
 * the pages; it describes this library's own dispatch.  The pointer stays
 * valid until the next liblce call on this thread. */
LCE_API const char* lce_last_launch(void);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H */
