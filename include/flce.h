/*
 * flce.h -- C ABI of the fused linear cross-entropy engine for AMD MI355X
 * (gfx950).
 *
 * The engine computes, for hidden states X [N, H] (N = B*T rows), an output
 * weight W [V, H] and integer labels [B, T]:
 *
 *   loss = CE(X . W^T, y)      without ever holding the [N, V] logits,
 *   dX   = G . W,  dW = G^T . X,  G = c * (softmax(X . W^T) - onehot(y))
 *
 * with c = grad_scale / n_valid for the mean and c = grad_scale for the sum.
 * The identities Z = X.W^T, dX = dZ.W, dW = dZ^T.X are the ones of the ms-swift
 * PR "feat(sft): Add optional fused linear ce for qwen2/qwen3 on npu", section
 * "Mathematical Equivalence".  The argument set (hidden, weight, labels,
 * ignore_index = -100, shift, reduction = "mean") is that of the
 * linear_cross_entropy call in the LoRA-SFT blog post's CCE patch, where W is
 * stored (vocab_size, hidden_dim).  dX is accumulated in FP32 over the whole
 * vocabulary and rounded to the input type once, as item 2 of Megatron-LM PR
 * "[Dev] Fix Linear-Cross-Entropy Convergence Issue" prescribes.
 *
 * Conventions
 *   - Targets: with shift != 0, row (b, t) is scored against labels[b, t+1] and
 *     the last row of every sequence has no target; with shift == 0 row i is
 *     scored against labels[i].  A target equal to ignore_index (compared as an
 *     int64, before any range check) marks the row as ignored.
 *   - n_valid counts the rows that have a target; the mean divides by it.  With
 *     n_valid == 0 the loss is 0 and all gradients are 0.
 *   - Layouts are row-major and dense: X is [B*T, H] with H contiguous, W is
 *     [V, H] with H contiguous, labels are [B, T] int64.
 *   - dtype FLCE_DTYPE_BF16: X, W are bfloat16; products run on bf16 MFMA with
 *     FP32 accumulation.  FLCE_DTYPE_F32: X, W are float32 on fp32 MFMA.
 *   - All pointers except the workspace-size query are DEVICE pointers on the
 *     current HIP device, 16-byte aligned, owned by the caller.  The library
 *     allocates nothing and keeps no state between calls; the only scratch it
 *     uses is the caller's workspace.  Calls are asynchronous on `stream`
 *     (a hipStream_t; NULL = the null stream) and never synchronise the host.
 *   - Two calls may run concurrently only with separate workspaces.
 *
 * Errors
 *   Host-side checks run before anything is launched; on failure the function
 *   returns a nonzero FLCE_ERR_* code and touches no output.  A label that is
 *   neither ignore_index nor in [0, V) is found on the device: it sets
 *   *status = FLCE_ERR_LABEL_RANGE (when status is non-NULL), the forward loss
 *   becomes NaN and the backward gradients become NaN.  Launch failures return
 *   FLCE_ERR_HIP.
 */
#ifndef FLCE_H_
#define FLCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FLCE_OK 0
#define FLCE_ERR_NULL 1        /* a required pointer is NULL               */
#define FLCE_ERR_SHAPE 2       /* B, T, H or V out of range, or N too large */
#define FLCE_ERR_ALIGN 3       /* H % 8 != 0 or a pointer not 16B aligned   */
#define FLCE_ERR_DTYPE 4       /* unknown dtype / grad dtype                */
#define FLCE_ERR_REDUCTION 5   /* unknown reduction                         */
#define FLCE_ERR_WORKSPACE 6   /* workspace NULL or smaller than required   */
#define FLCE_ERR_HIP 7         /* a HIP launch or query failed              */
#define FLCE_ERR_LABEL_RANGE 8 /* device: a valid label outside [0, V)      */
#define FLCE_ERR_ALIAS 9       /* an output overlaps an input, another
                                  output or the workspace                   */
#define FLCE_ERR_TOO_LARGE 10  /* beyond the allocation-free scratch        */

/* bytes of the device array flce_forward_noalloc uses as its scratch */
#define FLCE_NOALLOC_SCRATCH_BYTES (160ll << 20)

/* element types */
#define FLCE_DTYPE_F32 0
#define FLCE_DTYPE_BF16 1

/* reductions.  NONE returns the per-row losses l_i = lse_i - z_{i,y_i} (their
 * negatives are the target log-probs) and takes a per-row upstream gradient:
 * the per-token outputs that RL objectives need (the ms-swift PR lists
 * GRPO/PPO under "Limitations" because mean cross-entropy is not enough). */
#define FLCE_REDUCTION_MEAN 0
#define FLCE_REDUCTION_SUM 1
#define FLCE_REDUCTION_NONE 2

/*
 * flce_workspace_size -- bytes of device scratch that flce_forward and
 * flce_backward need for this shape and dtype (one buffer serves both).
 * Host-only arithmetic, no HIP call.  The figure is the engine's whole extra
 * device memory: it grows linearly in N (per-row indices, a compacted copy of
 * the valid rows of X, FP32 dX accumulators -- one, or up to eight vocabulary
 * parts when few hidden x row tiles would leave compute units idle -- FP32
 * per-target row sums for the one-hot part of dW, and two bounded slabs of
 * softmax gradients, each covering a fixed vocabulary block), plus 4 bytes
 * per vocabulary entry; never with N*V.
 *   B, T, H, V : problem sizes (B*T = N rows)
 *   dtype      : FLCE_DTYPE_*
 *   bytes      : out, host pointer
 */
int flce_workspace_size(int64_t B, int64_t T, int64_t H, int64_t V, int dtype,
                        size_t* bytes);

/*
 * flce_forward -- loss and per-row log-sum-exp.
 *   X [B*T, H], W [V, H] : dtype elements, device
 *   labels [B, T]        : int64, device
 *   ignore_index         : label value that marks a row as ignored (e.g. -100)
 *   reduction            : FLCE_REDUCTION_MEAN, _SUM or _NONE
 *   shift                : nonzero = next-token targets inside each sequence
 *   loss                 : out, float32, device: a scalar (MEAN, SUM), or
 *                          [B*T] per-row losses (NONE: 0.0 on ignored rows,
 *                          NaN everywhere after a bad label)
 *   lse [B*T]            : out, float32, device; log sum_v exp(z_iv) of every
 *                          row with a target, 0.0 for ignored rows.  Keep it
 *                          for flce_backward.
 *   n_valid              : out, int64 scalar, device, may be NULL
 *   status               : out, int32 scalar, device, may be NULL; 0 or
 *                          FLCE_ERR_LABEL_RANGE
 *   workspace, workspace_bytes : device scratch of flce_workspace_size bytes
 *   stream               : hipStream_t
 */
int flce_forward(const void* X, const void* W, const int64_t* labels,
                 int64_t B, int64_t T, int64_t H, int64_t V, int dtype,
                 int64_t ignore_index, int reduction, int shift,
                 float* loss, float* lse, int64_t* n_valid, int32_t* status,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * flce_forward_noalloc -- flce_forward without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Arguments, outputs
 * and errors as flce_forward.  The scratch is a fixed device array inside
 * the library, FLCE_NOALLOC_SCRATCH_BYTES (160 MiB), one copy per device,
 * held until the process ends; its address is looked up on a device's first
 * call.  The call allocates nothing.  A problem whose forward needs more
 * scratch than that returns FLCE_ERR_TOO_LARGE before anything is launched.
 * The forward needs about N * (H * es + 24) + 4 MiB bytes (es = 2 for bf16,
 * 4 for fp32; the compacted copy of the valid rows of X dominates), so every
 * bf16 problem with N * H <= 64M elements and N <= 2^20 fits.  All calls on
 * one device share the array: two such calls that overlap in time on one
 * device (two streams, or two host threads) race and must be serialised by
 * the caller.
 */
int flce_forward_noalloc(const void* X, const void* W, const int64_t* labels,
                         int64_t B, int64_t T, int64_t H, int64_t V, int dtype,
                         int64_t ignore_index, int reduction, int shift,
                         float* loss, float* lse, int64_t* n_valid, int32_t* status,
                         void* stream);

/*
 * flce_backward -- gradients of grad_scale * loss with respect to X and W.
 *   X, W, labels, sizes, dtype, ignore_index, reduction, shift : as forward
 *   lse [B*T]     : float32, device, the forward's output for the same inputs
 *   grad_scale    : float32, device: the upstream dL/dloss, a scalar (MEAN,
 *                   SUM) or [B*T] per-row values (NONE); NULL = 1
 *   dX [B*T, H]   : out, device, fully overwritten (ignored rows are 0)
 *   dW [V, H]     : out, device, fully overwritten
 *   grad_dtype    : element type of dX and dW: the input dtype, or
 *                   FLCE_DTYPE_F32 to receive the FP32 accumulators unrounded
 *   dW_accumulate : 0 = dW is overwritten; 1 = the gradient is added to the
 *                   dW already there (beta = 1: gradient accumulation over
 *                   micro-batches, or the gradient buffer of a weight tied to
 *                   the input embedding), summed in FP32 and rounded once
 *   status, workspace, workspace_bytes, stream : as forward
 * dX must not overlap X, dW must not overlap W, and neither may overlap the
 * other or the workspace's first flce_workspace_size bytes (else
 * FLCE_ERR_ALIAS, before anything is launched).  The FP32 accumulation and the
 * single final rounding follow Megatron-LM PR "[Dev] Fix Linear-Cross-Entropy
 * Convergence Issue", item 2.
 */
int flce_backward(const void* X, const void* W, const int64_t* labels,
                  int64_t B, int64_t T, int64_t H, int64_t V, int dtype,
                  int64_t ignore_index, int reduction, int shift,
                  const float* lse, const float* grad_scale,
                  void* dX, void* dW, int grad_dtype, int dW_accumulate, int32_t* status,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Vocabulary shards: the output layer split along V across devices, as the
 * column-parallel output layer of Megatron-LM PR "[Dev] Fix Linear-Cross-
 * Entropy Convergence Issue" (item 1; its item 2 is why the dX partials stay
 * FP32 until they are summed).  A device holding W rows [v_begin, v_begin + V)
 * of a V_total vocabulary runs flce_shard_forward; the per-row (lse, target
 * logit) pairs of all shards are then gathered (the one exchange of the
 * forward; [N] floats twice per shard) and merged by flce_shard_merge into the
 * loss and the global lse; flce_shard_backward with that lse gives the shard's
 * dW rows (complete) and its FP32 share of dX, to be summed over the shards
 * (an all-reduce) and rounded once.  The calls are the same on one device;
 * moving the partials between devices is the caller's (RCCL) business.
 *
 * flce_shard_forward -- per-row lse over this shard and target logits.
 *   X, labels, B, T, H, dtype, ignore_index, shift, status, stream : as
 *                  flce_forward (labels index the whole vocabulary)
 *   W [V, H]     : this shard's rows of the output weight
 *   V, v_begin, V_total : shard rows, first row's vocabulary index, vocabulary
 *                  size; 0 <= v_begin, v_begin + V <= V_total
 *   lse [B*T]    : out, float32, device: log sum over the shard's entries (0 on
 *                  ignored rows)
 *   zt [B*T]     : out, float32, device: z_{i,y_i} when y_i lies in this shard,
 *                  else 0
 *   workspace    : flce_workspace_size(B, T, H, V, dtype) bytes
 */
int flce_shard_forward(const void* X, const void* W, const int64_t* labels,
                       int64_t B, int64_t T, int64_t H, int64_t V, int64_t v_begin,
                       int64_t V_total, int dtype, int64_t ignore_index, int shift,
                       float* lse, float* zt, int32_t* status, void* workspace,
                       size_t workspace_bytes, void* stream);

/* flce_shard_merge_workspace_size -- device scratch bytes of flce_shard_merge. */
int flce_shard_merge_workspace_size(int64_t B, int64_t T, size_t* bytes);

/*
 * flce_shard_merge -- loss and global lse from the shards' partials.
 *   lse_shards, zt_shards [shards][B*T] : float32, device: the shards' outputs
 *   labels, B, T, ignore_index, shift, reduction, loss, lse, n_valid, status :
 *                  as flce_forward (V_total: the vocabulary size, for the
 *                  label check)
 */
int flce_shard_merge(const float* lse_shards, const float* zt_shards, int shards,
                     const int64_t* labels, int64_t B, int64_t T, int64_t V_total,
                     int64_t ignore_index, int shift, int reduction, float* loss, float* lse,
                     int64_t* n_valid, int32_t* status, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * flce_shard_backward -- this shard's dW rows and its share of dX.
 *   arguments as flce_backward, with W, V, v_begin, V_total as in
 *   flce_shard_forward and lse the merged (global) lse;
 *   dX_partial [B*T, H] : out, float32, device: sum over the shard's
 *                  vocabulary of G_iv W_v (ignored rows 0); sum over the
 *                  shards, then round once
 *   dW [V, H]    : out, grad_dtype, this shard's rows (dW_accumulate as in
 *                  flce_backward)
 * dX_partial and dW follow flce_backward's rules on overlapping buffers.
 */
int flce_shard_backward(const void* X, const void* W, const int64_t* labels,
                        int64_t B, int64_t T, int64_t H, int64_t V, int64_t v_begin,
                        int64_t V_total, int dtype, int64_t ignore_index, int reduction,
                        int shift, const float* lse, const float* grad_scale,
                        float* dX_partial, void* dW, int grad_dtype, int dW_accumulate,
                        int32_t* status, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Chunked mode: the row-chunk recipe of the ms-swift PR "feat(sft): Add
 * optional fused linear ce for qwen2/qwen3 on npu" ("What this PR does": the
 * sequence cut into chunks, each chunk's logits, loss and both gradients
 * computed at once; "Mathematical Equivalence": grad_weight summed over the
 * chunks).  One call returns loss, lse, dX and dW.  A chunk of C valid rows
 * keeps its softmax gradient over the whole vocabulary in a [C, V] slab of
 * the workspace, so the logits are computed once (three contractions,
 * 6 n H V flop, instead of the forward + backward pair's four) at the price
 * of memory proportional to the chunk.
 *
 * chunk_rows (both calls, which must agree): rows per chunk, rounded up to a
 * multiple of 256 (the pages' CHUNK_SIZE); 0 = as many as a 2 GiB slab holds
 * (6912 rows at V = 152064 bf16).  Capped at the padded row count.  A 256-row
 * tile of the slab must stay below 2^31 bytes (V <= 4194048 for bf16,
 * 2096896 for fp32), and a chunk's 256 x 256 logits tiles, like a vocabulary
 * block's dX and dW tiles, must fit one dispatch (fewer than 2^24
 * workgroups of 256 threads); else FLCE_ERR_SHAPE.
 *
 * flce_chunked_workspace_size -- bytes of device scratch flce_chunked needs
 * (host-only arithmetic).  Other arguments as flce_workspace_size.
 */
int flce_chunked_workspace_size(int64_t B, int64_t T, int64_t H, int64_t V, int dtype,
                                int64_t chunk_rows, size_t* bytes);

/*
 * flce_chunked -- loss, per-row lse and the gradients of grad_scale * loss.
 *   X, W, labels, sizes, dtype, ignore_index, reduction, shift : as forward
 *   chunk_rows    : as flce_chunked_workspace_size
 *   grad_scale    : as flce_backward (scalar, or per row under NONE); NULL = 1
 *   loss, lse, n_valid : as flce_forward's outputs
 *   dX, dW, grad_dtype, dW_accumulate : as flce_backward's (the same rules
 *                   on overlapping buffers, with this call's workspace size)
 *   status        : as forward (a bad label also makes the gradients NaN)
 *   workspace, workspace_bytes : device scratch of flce_chunked_workspace_size
 *   stream        : hipStream_t
 * dW is summed over the row chunks: with grad_dtype = FLCE_DTYPE_F32 in FP32;
 * with bf16 it is rounded once per chunk (ceil(n / C) roundings; one when all
 * valid rows fit one chunk).  dX is accumulated in FP32 and rounded once.
 */
int flce_chunked(const void* X, const void* W, const int64_t* labels,
                 int64_t B, int64_t T, int64_t H, int64_t V, int dtype,
                 int64_t ignore_index, int reduction, int shift, int64_t chunk_rows,
                 const float* grad_scale,
                 float* loss, float* lse, int64_t* n_valid, void* dX, void* dW,
                 int grad_dtype, int dW_accumulate, int32_t* status, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * flce_scale_grads -- dX = *scale * dX_in and dW = *scale * dW_in (the
 * upstream gradient applied to gradients computed with grad_scale = 1, e.g.
 * by flce_chunked during an autograd forward).  Each output may be its own
 * input (in place) or must not overlap it (else FLCE_ERR_ALIAS); out of
 * place, the inputs stay as they are, so the same saved gradients can be
 * scaled again (a second backward through a retained graph).  nx, nw: element
 * counts, multiples of 8 (bf16) or 4 (fp32); grad_dtype FLCE_DTYPE_BF16 or
 * _F32; scale: float32 scalar, device.  Buffers 16-byte aligned.
 */
int flce_scale_grads(const void* dX_in, void* dX, int64_t nx, const void* dW_in, void* dW,
                     int64_t nw, int grad_dtype, const float* scale, void* stream);

/*
 * flce_convert_grads -- dst = round(*scale * src (+ dst)) for FP32 gradient
 * sums src [n] (flce_chunked's or flce_backward's with grad_dtype =
 * FLCE_DTYPE_F32), with exactly one rounding to dst_dtype (FLCE_DTYPE_BF16,
 * round-to-nearest-even; FLCE_DTYPE_F32: none).  This is how a bf16 caller
 * of the chunked mode gets dW summed over all row chunks in FP32 and rounded
 * once, as item 2 of Megatron-LM PR "[Dev] Fix Linear-Cross-Entropy
 * Convergence Issue" prescribes for the gradient sums, and how an upstream
 * gradient is applied to FP32 sums before that one rounding.
 *   src [n]      : float32, device
 *   dst [n]      : dst_dtype, device; must not overlap src
 *   n            : element count, a multiple of 4
 *   scale        : float32 scalar, device, or NULL (= 1)
 *   accumulate   : 1 = the values dst already holds are added (in FP32,
 *                  before the rounding); 0 = dst is overwritten
 *   stream       : hipStream_t
 * Buffers 16-byte aligned.
 */
int flce_convert_grads(const float* src, void* dst, int64_t n, int dst_dtype,
                       const float* scale, int accumulate, void* stream);

/* flce_status_string -- static, NUL-terminated description of a status code. */
const char* flce_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H_ */
