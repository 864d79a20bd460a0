/*
 * ce.h - C ABI of the MI355X (gfx950) fused softmax cross-entropy library
 *        (libce_mi355x.so).
 *
 * The operation is the fused cross-entropy of the rumus project page,
 * milestone M7a "Loss Functions & GPU Optimizers" (log-sum-exp with a
 * per-row max and sum of exponentials, the gradient formed in the forward
 * pass, the loss reduced to a scalar that stays on the device), whose kernel
 * is shown in the rumus 0.1.1 source view of cross_entropy.wgsl: pass 1
 * (steps 1-4: row max, sum of exp(z - max), per-row loss scaled by 1/B,
 * gradient softmax - one-hot scaled by 1/B) and pass 2 (sum of the per-row
 * losses).  For a [B, C] logit matrix z and int32 targets t:
 *
 *     loss_rows[b] = (log(sum_c exp(z[b,c])) - z[b, t_b]) / B
 *     grad[b, c]   = (softmax(z[b,:])[c] - [c == t_b]) / B
 *     loss         = sum_b loss_rows[b]                     (the batch mean)
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller.  The
 *    library allocates nothing and keeps no mutable state (apart from the
 *    test-only hooks at the end, and the 4 KB per GPU that
 *    ce_reduce_loss_noalloc holds).
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *    void*; NULL means the default stream).  No call synchronises the
 *    device or copies data to the host.
 *  - Arguments are validated on the host before any HIP call; a negative
 *    ce_status is returned and nothing is launched.  A failed launch returns
 *    CE_ERR_LAUNCH.  Faults of earlier asynchronous work surface at the
 *    caller's next synchronisation, as for any HIP call.
 *  - Outputs are overwritten, never accumulated.
 *  - The calls are thread-safe.
 */
#ifndef CE_MI355X_H
#define CE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the logits and of the gradient (they always match).
 * Accumulation is float32 in every case; per-row losses are float32. */
typedef enum {
    CE_F32 = 0,  /* IEEE binary32 */
    CE_BF16 = 1, /* bfloat16; the gradient is rounded to nearest, ties to even */
    CE_F16 = 2   /* IEEE binary16 (the pages' F16 data type, rumus project page
                    milestone M11); widened exactly, the gradient rounded to
                    nearest, ties to even, with binary16 subnormals */
} ce_dtype;

typedef enum {
    CE_OK = 0,
    CE_ERR_NULL = -1,      /* a required pointer is NULL */
    CE_ERR_SHAPE = -2,     /* B <= 0, C <= 0, or a size beyond the limits below */
    CE_ERR_DTYPE = -3,     /* dtype is not a ce_dtype */
    CE_ERR_WORKSPACE = -4, /* workspace NULL or smaller than ce_reduce_workspace_bytes(B) */
    CE_ERR_LAUNCH = -5,    /* the HIP runtime rejected a kernel launch */
    CE_ERR_ALIGN = -6,     /* a pointer is not aligned as required */
    CE_ERR_ALIAS = -7,     /* an output overlaps an input in a way the call refuses */
    CE_ERR_PATH = -8       /* the forced path (ce_debug_force_path) cannot take this shape */
} ce_status;

/* Largest number of classes accepted: a row must stay below 2^31 bytes. */
#define CE_MAX_C ((int64_t)1 << 28)

/* ignore_index value of ce_fwd_grad_ex that ignores no row. */
#define CE_NO_IGNORE ((int32_t)(-2147483647 - 1))

/*
 * ce_fwd_grad - per-row loss and gradient of softmax cross-entropy, one pass.
 *
 * Defined by: rumus 0.1.1 cross_entropy.wgsl, pass 1, steps 1-4; rumus
 * project page, milestone M7a (gradient pre-computed during the forward).
 *
 *   logits    [B, C] row-major, contiguous, dtype elements.  Read once.
 *             Must be aligned to the element size.
 *   targets   [B] int32 class indices.  A target outside [0, C) is not an
 *             error: that row's loss and its whole gradient row are NaN.
 *   B, C      1 <= B <= 2^31 - 1, 1 <= C <= CE_MAX_C.
 *   dtype     CE_F32, CE_BF16 or CE_F16.
 *   grad_out  [B, C] dtype, fully overwritten with (softmax - onehot) / B.
 *             Contents on entry are ignored; on path 4 with several
 *             parts per row the call also uses 16 bytes per other part of
 *             each part's own gradient as a mailbox before the gradient is
 *             written there.
 *             grad_out == logits computes the gradient in place of the
 *             logits (every kernel holds a row's data on chip, or reads it
 *             again from the same thread, before writing it; rows that
 *             path 4 would cut into several parts run on path 2 or 3
 *             instead; with ce_fwd_grad_ex and an in-place workspace,
 *             they run on path 4).
 *             Any other overlap with logits is refused.  Must be aligned
 *             to the element size, and (grad_out - logits) must be a
 *             multiple of 16 bytes (true for any two allocations from the
 *             HIP or torch allocators).
 *   loss_out  [B] float32, overwritten with the per-row losses, already
 *             scaled by 1/B; ce_reduce_loss sums them to the batch mean.
 *   stream    hipStream_t or NULL.
 *
 * Returns CE_OK or a negative ce_status.  Results are bitwise reproducible
 * for the same inputs, shape and dtype on the same device.
 */
int ce_fwd_grad(const void* logits, const int32_t* targets, int64_t B, int64_t C,
                int dtype, void* grad_out, float* loss_out, void* stream);

/*
 * ce_fwd_loss - per-row losses only, for evaluation: the logits are read
 * once and only loss_out is written.  Arguments, layout and errors as
 * ce_fwd_grad without grad_out; runs on paths 1, 2, 3 and 5 (no row parts
 * are needed when nothing has to stay on chip for a gradient), so forcing
 * path 4 returns CE_ERR_PATH.
 *
 * Defined by: rumus 0.1.1 cross_entropy.wgsl, pass 1 steps 1-3 (row max,
 * sum of exponentials, per-row loss scaled by 1/B).
 */
int ce_fwd_loss(const void* logits, const int32_t* targets, int64_t B, int64_t C, int dtype,
                float* loss_out, void* stream);

/*
 * ce_fwd_grad_scaled - ce_fwd_grad with the gradient multiplied by an
 * upstream gradient of the loss that is known before the forward pass
 * (for example a loss-scaling factor): grad_out = (softmax - onehot) / B *
 * (*grad_scale), at no extra memory traffic.  loss_out is not scaled.
 *
 * Defined by: rumus project page, milestone M7a (the backward of the fused
 * loss is a broadcast scale of the gradient formed in the forward).
 *
 *   grad_scale  DEVICE pointer to one float32, read by the kernels in
 *               stream order; 4-byte aligned; must not be NULL.
 *   other arguments, layout and errors as ce_fwd_grad.
 */
int ce_fwd_grad_scaled(const void* logits, const int32_t* targets, int64_t B, int64_t C,
                       int dtype, void* grad_out, float* loss_out, const float* grad_scale,
                       void* stream);

/*
 * ce_fwd_grad_ex - ce_fwd_grad with row strides, an optional device
 * gradient scale, the loss-only mode and ignore_index in one call.
 *
 * Defined by: as ce_fwd_grad.  Row strides: a tensor's Layout holds its
 * shape, strides and offset, and views share storage with other layouts
 * (rumus project page, core-types table); ignore_index is not on the pages
 * and follows the common mean-reduction convention.
 *
 *   logits        row b starts at logits + b * ld_logits elements;
 *                 ld_logits >= C.
 *   grad_out      NULL for the per-row losses only (ld_grad is then
 *                 unused), else row b starts at grad_out + b * ld_grad,
 *                 ld_grad >= C.  In place when grad_out == logits and
 *                 ld_grad == ld_logits; otherwise the two spans (first
 *                 element of row 0 to the last of row B-1) must not
 *                 overlap.  Every row of grad must start at the same
 *                 address modulo 16 as its row of logits: (grad_out -
 *                 logits) and (ld_grad - ld_logits) * element size are
 *                 multiples of 16 bytes.
 *   grad_scale    DEVICE float32 scalar multiplying the gradient, or NULL.
 *   ignore_index  CE_NO_IGNORE, or a class value: rows whose target equals
 *                 it get loss 0 and a zero gradient row, and the other rows
 *                 are scaled by 1/N instead of 1/B, N the number of rows
 *                 not ignored, counted on the device (no host
 *                 synchronisation).  Other targets outside [0, C) still
 *                 give NaN rows (and count in N).
 *   workspace     device scratch of ce_fwd_workspace_bytes(ignore_index)
 *                 bytes (4-byte aligned), or NULL when that is 0; it holds
 *                 the count N while the call's kernels run.  In place, rows
 *                 that path 4 cuts into several parts run as parts when the
 *                 workspace also has ce_fwd_inplace_workspace_bytes(B)
 *                 bytes, is 8-byte aligned and was zero-filled before its
 *                 first use (each call leaves those bytes zero again, so a
 *                 workspace serves any number of calls ordered on one
 *                 stream; calls that may overlap need workspaces of their
 *                 own); otherwise they run on path 2 or 3.
 *   other arguments and errors as ce_fwd_grad; CE_ERR_WORKSPACE when the
 *   workspace is missing or too small.
 */
size_t ce_fwd_workspace_bytes(int32_t ignore_index);

/*
 * ce_fwd_inplace_workspace_bytes - the ce_fwd_grad_ex workspace with which
 * the gradient in place of rows that path 4 cuts into several parts (bf16
 * and fp16 C of 81921 to 524288 in two, four or eight parts, fp32 C of
 * 40961 to 262144, for rows starting on a 16-byte boundary) runs on path
 * 4: 256 bytes (the ignore_index count in the first 4), then 18 64-bit
 * words a row, 256 + 144 B in all (0 for B outside [1, 2^31 - 1]).
 *
 * Defined by: as ce_fwd_grad (the gradient formed in the forward pass,
 * here over the logits' own storage).
 *
 * The parts of a row cannot trade their partial results through the
 * gradient (it is the logits), and a part that stops waiting for its
 * partners cannot read their logits again (they may be gradient already).
 * So each row's parts meet at its words.  Two parts: the first to arrive
 * claims the first word with its pair; the second reads that pair,
 * publishes its own in the second word and writes its half; the first
 * polls the second word a bounded number of times and then either writes
 * its half or marks the word and ends without writing, leaving its half
 * as logits for the second part to write as well (the second finds the
 * mark when it publishes).  Four or eight parts: each part publishes its
 * pair in a word of its own and counts its arrival; the last to arrive
 * reads every pair and claims each other part's flag word, writing the
 * gradient of any part whose flag it finds marked; any other part polls
 * for the pairs a bounded number of times, then writes its own part, or
 * marks its flag and ends without writing, or (when the last part has
 * already claimed its flag, so every pair is on its way) reads the pairs
 * and writes its own part.  No wait is on a part that has not published,
 * and each element's value does not depend on which part wrote it.
 */
size_t ce_fwd_inplace_workspace_bytes(int64_t B);

int ce_fwd_grad_ex(const void* logits, int64_t ld_logits, const int32_t* targets, int64_t B,
                   int64_t C, int dtype, void* grad_out, int64_t ld_grad, float* loss_out,
                   const float* grad_scale, int32_t ignore_index, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * ce_scale_grad - the backward of the fused loss: grad *= *scale in place,
 * for the n elements of a gradient that ce_fwd_grad produced and the
 * upstream gradient `scale` of the loss (a DEVICE float32 scalar, read in
 * stream order, so the host never reads it).  When *scale is exactly 1 the
 * kernel returns without touching grad (the broadcast scale of the common
 * `loss.backward()` moves no gradient bytes).  bf16 values are scaled in
 * float32 and rounded to nearest even.
 *
 * Defined by: rumus project page, milestone M7a (the backward of the fused
 * loss is a zero-copy broadcast scale of the gradient formed in the
 * forward).
 *
 *   grad   [n] dtype, element-aligned, DEVICE pointer, scaled in place.
 *   n      >= 1 elements.
 *   scale  DEVICE pointer to one float32, 4-byte aligned, not inside grad.
 */
int ce_scale_grad(void* grad, int64_t n, int dtype, const float* scale, void* stream);

/*
 * ce_reduce_workspace_bytes - device scratch that ce_reduce_loss needs for
 * B per-row losses (0 when one workgroup sums them directly).
 */
size_t ce_reduce_workspace_bytes(int64_t B);

/*
 * ce_reduce_loss - the batch-mean loss as one float32 on the device.
 *
 * Defined by: rumus 0.1.1 cross_entropy.wgsl, pass 2 (the per-row losses
 * summed into one scalar); rumus project page, milestone M7b (the loss is
 * read back as 4 bytes only when the caller wants it).
 *
 *   loss_rows        [B] float32 (the loss_out of ce_fwd_grad).
 *   B                number of rows, 1 <= B <= 2^39 (CE_ERR_SHAPE above:
 *                    a first-level chunk's bytes must fit 32 bits).
 *   loss_scalar_out  [1] float32, overwritten with sum_b loss_rows[b].
 *   workspace        device scratch of at least ce_reduce_workspace_bytes(B)
 *                    bytes (may be NULL when that is 0); contents on entry
 *                    are ignored.
 *
 * The sum uses a fixed two-level tree whose shape depends only on B, with
 * no atomics, so the result is bitwise reproducible.
 */
int ce_reduce_loss(const float* loss_rows, int64_t B, float* loss_scalar_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * ce_fwd_grad_loss - the whole training step of the loss in one call:
 * ce_fwd_grad, then ce_reduce_loss of its per-row losses, on the same
 * stream (two kernel launches, one host call).
 *
 * Defined by: rumus 0.1.1 cross_entropy.wgsl, pass 1 (per-row loss and
 * gradient) and pass 2 (the per-row losses summed into one scalar).
 *
 *   logits, targets, B, C, dtype, grad_out, stream  as ce_fwd_grad.
 *   loss_rows_out    [B] float32, the per-row losses (loss_out of
 *                    ce_fwd_grad), kept for the caller.
 *   loss_scalar_out  [1] float32, the batch-mean loss (as ce_reduce_loss).
 *   workspace        device scratch of ce_reduce_workspace_bytes(B) bytes
 *                    (NULL when that is 0).
 *
 * Every argument, the reduction's included, is checked before anything is
 * launched, so an error leaves all outputs untouched.  The results are
 * bitwise those of the two calls made one after the other.
 */
int ce_fwd_grad_loss(const void* logits, const int32_t* targets, int64_t B, int64_t C, int dtype,
                     void* grad_out, float* loss_rows_out, float* loss_scalar_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Largest B that ce_reduce_loss_noalloc accepts. */
#define CE_NOALLOC_MAX_ROWS ((int64_t)2147483647)

/*
 * ce_reduce_loss_noalloc - ce_reduce_loss without a workspace argument, for
 * callers that cannot allocate device memory: code recorded under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 *   loss_rows, B, loss_scalar_out, stream   as ce_reduce_loss;
 *                                            1 <= B <= CE_NOALLOC_MAX_ROWS.
 *
 * The first level's partial sums go to a scratch array of 1024 floats
 * (4 KB) that the library holds in device memory, one copy per GPU, from
 * its first use on that GPU until the process ends.  The call allocates
 * nothing: the array's device address is looked up once per device (on
 * the first call made with that device current) and cached.  The kernels
 * and the tree are those of ce_reduce_loss, so the scalar is bitwise the
 * same.  Every call on a GPU shares that GPU's array: calls whose
 * executions overlap on one GPU (other streams, other host threads) race
 * and may return wrong sums; calls ordered on one stream are safe.
 *
 * Returns CE_OK, CE_ERR_NULL, CE_ERR_SHAPE (B out of range), CE_ERR_ALIGN,
 * or CE_ERR_LAUNCH (a failed launch, or the runtime could not give the
 * scratch array's address).
 */
int ce_reduce_loss_noalloc(const float* loss_rows, int64_t B, float* loss_scalar_out,
                           void* stream);

/*
 * ce_softmax_fwd - row-wise softmax and log-sum-exp.
 *
 * Defined by: rumus project page, milestone M8c (row-wise softmax kept
 * stable with the log-sum-exp trick) and its feature table's Softmax row.
 * For each row of x:
 *
 *     y[b, c]  = exp(x[b,c] - m_b) / sum_j exp(x[b,j] - m_b),  m_b = max_j x[b,j]
 *     lse[b]   = m_b + ln(sum_j exp(x[b,j] - m_b))
 *
 * computed by the kernels of ce_fwd_grad (same paths, same single read of
 * x and single write of y), in float32, the log-sum-exp in the log2
 * domain as ln2 * (round(m log2 e) + log2 s).
 *
 *   x        [B, C] dtype, row-major, contiguous, element-aligned.
 *   B, C     as ce_fwd_grad.
 *   y_out    [B, C] dtype, overwritten; y_out == x computes the softmax in
 *            place (rows that path 4 would cut into several parts then run
 *            on path 2 or 3).  Other overlaps are refused; (y_out - x) must
 *            be a multiple of 16 bytes.  Path 4's rows of several parts use
 *            16 bytes per other part of each part of y_out as a mailbox
 *            before writing it.
 *   lse_out  [B] float32 (4-byte aligned), or NULL for none.
 * Returns CE_OK or a negative ce_status.
 */
int ce_softmax_fwd(const void* x, int64_t B, int64_t C, int dtype, void* y_out, float* lse_out,
                   void* stream);

/*
 * ce_softmax_bwd - backward of the row-wise softmax.
 *
 * Defined by: rumus project page, milestone M8c (softmax backward kernel).
 * The pages give no formula; this is the vector-Jacobian product of the
 * forward, from its output y and the upstream gradient dy:
 *
 *     dx[b, c] = y[b,c] * (dy[b,c] - sum_j dy[b,j] * y[b,j])
 *
 * in float32 with a fixed summation order (bitwise reproducible).
 *
 *   y, dy    [B, C] dtype, row-major, contiguous, element-aligned; y is the
 *            softmax (for example ce_softmax_fwd's y_out).
 *   dx_out   [B, C] dtype, overwritten.  May be y or dy themselves; any
 *            other overlap is refused.  (dy - y) and (dx_out - y) must be
 *            multiples of 16 bytes.
 * Rows of C <= 256 run many to a wave (path 1); rows of up to 8 KB whose
 * length and alignment allow 4-byte or wider vectors run whole in one
 * wavefront's registers, one to four rows per wave (path 5); other rows of
 * up to 8192 16-byte vectors run one workgroup per row with y and dy held
 * in registers (path 2); longer rows of up to 32768 body vectors, out of
 * place, run in four parts (up to 16384 vectors) or eight that trade their
 * partial dot products (path 4), and beyond that, or in place, stream the
 * rest of the row a second time (path 3).  ce_debug_force_path applies.
 */
int ce_softmax_bwd(const void* y, const void* dy, int64_t B, int64_t C, int dtype, void* dx_out,
                   void* stream);

/*
 * Cross-entropy over a vocabulary split into column shards.
 *
 * Defined by: rumus project page, milestone M24 (a column-parallel linear
 * layer splits its weight along the output features, so each rank holds
 * the logits of a contiguous range of classes), with the cross-entropy of
 * rumus 0.1.1 cross_entropy.wgsl pass 1 taken over such ranges: the max and
 * the sum of exponentials of the whole row are the max of the shards' maxes
 * and the rescaled sum of their sums.
 *
 * Shard k holds columns [col0_k, col0_k + C_k) of every row as its own
 * [B, C_k] row-major array.  The calls:
 *   1. ce_shard_stats on every shard writes B records of 4 float32 (c, sx,
 *      zt, own): c = max_c z * log2(e) rounded to float32; sx = the sum over
 *      the shard's columns other than the target of 2^(z log2e - c); zt =
 *      the target logit, and own = 1, where the shard holds the target
 *      (else zt = own = 0).
 *   2. The caller gathers the records of all N shards into one array of
 *      N x B records, shard-major, in shard order (one all-gather of
 *      16 B bytes per shard on several GPUs).
 *   3. ce_shard_grad on every shard combines each row's N records in shard
 *      order (c = max c_k, sx = sum sx_k 2^(c_k - c), zt from the owning
 *      shard) and writes that shard's columns of (softmax - onehot) / B,
 *      times *grad_scale when grad_scale is not NULL, and, when loss_out is
 *      not NULL, the per-row losses (lse - z_t) / B.
 * A row whose target lies outside [0, C_total), or whose records do not
 * name exactly one owner, gets a NaN loss and NaN gradient.  All shards
 * compute identical per-row values, so any one may write the losses.
 *
 * ce_shard_stats:
 *   logits       [B, C] dtype, the shard (C = C_k columns), element-aligned.
 *   targets      [B] int32, the global class indices.
 *   col0         the shard's first column, 0 <= col0 <= 2^31 - 1.
 *   records_out  [B][4] float32, 16-byte aligned, overwritten.
 * It reads the shard once on paths 1, 2, 3 and 5 (path 4 is refused).
 *
 * ce_shard_grad:
 *   logits, targets, B, C, col0, dtype as ce_shard_stats.
 *   C_total      the whole row's length: col0 + C <= C_total <= 2^31 - 1.
 *   records      [n_shards][B][4] float32, 16-byte aligned (step 2).
 *   n_shards     1 to 1024.
 *   grad_out     [B, C] dtype, overwritten; may be logits itself (each
 *                thread reads its elements before writing them); no other
 *                overlap with logits or records.
 *   loss_out     [B] float32 or NULL.
 *   grad_scale   DEVICE float32 scalar or NULL (as ce_fwd_grad_scaled).
 */
int ce_shard_stats(const void* logits, const int32_t* targets, int64_t B, int64_t C, int64_t col0,
                   int dtype, float* records_out, void* stream);

int ce_shard_grad(const void* logits, const int32_t* targets, int64_t B, int64_t C, int64_t col0,
                  int64_t C_total, int dtype, const float* records, int n_shards, void* grad_out,
                  float* loss_out, const float* grad_scale, void* stream);

/* Static text for a ce_status value. */
const char* ce_status_string(int status);

/* Library version string. */
const char* ce_version(void);

/*
 * ce_stream_copy - measurement reference, not part of the method: copies
 * `bytes` bytes from src to dst (device pointers, 16-byte aligned, bytes a
 * positive multiple of 16, no overlap) with the memory pattern of the
 * row-part kernel (1024-thread workgroups, 128 KiB each as 8 slots of
 * 16-byte non-temporal loads issued before the stores).  The benchmark
 * reports the cross-entropy kernel's bandwidth as a share of this copy's.
 * Stream-ordered; returns CE_OK or a negative ce_status.
 */
int ce_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * Kernel paths:
 *   1 short rows  - many rows per 64-lane wavefront, cross-lane DPP
 *                   reductions (C <= 256); contiguous rows in 16-byte
 *                   aligned arrays of at most 64 bytes, or whose byte
 *                   length is not a multiple of 16, move through LDS in
 *                   chunks of whole 16-byte vectors;
 *   2 resident    - one workgroup per row, the row held on chip in
 *                   registers between the reduction and the gradient write,
 *                   so it is read from HBM once and written once;
 *   3 long rows   - as 2, with the part of the row beyond the on-chip
 *                   capacity streamed with online max/sum-exp partials and
 *                   re-read for the gradient;
 *   4 row parts   - the row cut into one, two, four or eight parts (one
 *                   256-thread workgroup for rows up to 32 KB, else
 *                   1024-thread workgroups of up to 12 x 16 KB, two per
 *                   CU); each part is read once into registers and LDS and
 *                   reduced to a max/sum-exp pair, the parts trade
 *                   their pairs and combine them in a fixed order, and each
 *                   writes its share of the gradient from on chip.  A part
 *                   that does not receive a partner's pair in time
 *                   recomputes it with the same code, so the bits do not
 *                   depend on timing.  Automatic above 8 KB of 16-bit or
 *                   4 KB of fp32 elements (above 4 KB for 16-bit rows of
 *                   odd length), up to 1 MB (16-bit C up to 524288, fp32 C
 *                   up to 262144).
 *   5 wave rows   - rows of up to 16 KB (automatic above 256 elements)
 *                   whose starts, lengths and strides allow 16-, 8- or
 *                   4-byte vectors (4-byte ones up to 8 KB; 16-bit rows of
 *                   odd length have none): each 64-lane wavefront holds one
 *                   to eight whole rows in registers, reduces them with DPP
 *                   and writes their outputs from there.  Automatic
 *                   selection runs other such rows on path 2 up to 256
 *                   16-byte vectors (16-bit rows of odd length up to 1024
 *                   elements through the LDS-staged kernel) and as one row
 *                   part (path 4) above.
 *
 * ce_select_path returns the path ce_fwd_grad takes for (C, dtype) with
 * contiguous rows and 16-byte aligned base pointers, or a negative
 * ce_status.
 */
int ce_select_path(int64_t C, int dtype);

/*
 * Test hook: force every later call of ce_fwd_grad, ce_fwd_grad_scaled,
 * ce_fwd_loss, ce_softmax_fwd, ce_softmax_bwd and ce_shard_stats onto one
 * path (0 = automatic, 1 to 5 as above; path 3 is then run with a small
 * on-chip part so that the streamed part is exercised).  A shape the forced path cannot take
 * returns CE_ERR_PATH.  Returns the previous setting, or CE_ERR_PATH for an
 * unknown value.  Process-wide; not meant for production use.
 */
int ce_debug_force_path(int path);

/*
 * Test hook: how many times a path-4 row part polls for its partners'
 * max/sum-exp pairs before it recomputes the missing ones itself (default
 * 64; 0 makes every part of a row of several parts recompute every other
 * part's pair), and likewise for the parts of the softmax backward.
 * Results are bitwise the same for any value.  Returns the previous value, or CE_ERR_PATH if polls < 0.
 * Process-wide; not meant for production use.
 */
int ce_debug_part_polls(int polls);

/*
 * Test hook: a DEVICE pointer to a uint32 to which every path-4 part adds
 * the number of partner pairs it recomputed, atomically (NULL turns the
 * count off, the default).  The caller owns the counter and must keep it alive
 * while calls that were made with it set can still run.  Returns CE_OK.
 * Process-wide; not meant for production use.
 */
int ce_debug_part_counter(uint32_t* device_counter);

/*
 * Measurement hook: the next kernel launch that the library makes on the
 * calling thread records start_event when that kernel starts and
 * stop_event when it ends (hipExtLaunchKernel; either may be NULL), with
 * no event packets of the caller's own between kernels on the stream.
 * Both are hipEvent_t created by the caller (for example
 * torch.cuda.Event(enable_timing=True).event_id... or hipEventCreate).
 * One launch takes them: the first kernel of the next call (an entry point
 * that launches several kernels times only its first).  Returns CE_OK.
 * Per thread; not meant for production use.
 */
int ce_debug_time_next_launch(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* CE_MI355X_H */
