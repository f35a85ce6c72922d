/* sma.h -- C ABI of the scaled masked attention forward library (libsma.so, gfx950).
 *
 * The operation (oxicuda ComputeBackend page, documentation of `attention`):
 * for every batch b and head h,
 *
 *     O = softmax(scale * Q K^T + mask) V
 *
 * with the scale a multiplier of QK^T (its usual value is 1/sqrt(head_dim)) and
 * an optional causal mask that keeps the lower triangle. The pieces fixed by
 * the other pages:
 *   - scale, mask and softmax fuse into one pass over the scores, in that order
 *     (MicroGPT CuBLASBackend page, `fused_attn_softmax`);
 *   - the softmax is the max-subtracted row softmax, and the optional per-row
 *     output is the log-sum-exp log(sum_j exp(s_ij)) of the same scores
 *     (pulsatrix HIPBackend page, `softmax_rows` and `logsumexp_rows`);
 *   - masked scores take no part in the row max or the denominator, and a row
 *     in which the mask admits no key is all zeros (TorchLean Kernels page,
 *     hard-masked softmax); its log-sum-exp is -infinity, the log of an empty sum;
 *   - bf16 operands are multiplied with fp32 accumulation and an fp32 result
 *     (oxicuda ComputeBackend page, `gemm_mixed_precision`).
 *
 * Causal alignment. With seq_q != seq_kv the mask is bottom-right aligned:
 * query i may attend key j iff j <= i + seq_kv - seq_q. For seq_q == seq_kv
 * this is j <= i. When seq_q > seq_kv the first seq_q - seq_kv query rows see
 * no key and are written as +0.0 (LSE -inf).
 *
 * Layout (contiguous, row-major, no strides):
 *   q, o  [batch][heads][seq_q][head_dim]
 *   k, v  [batch][heads][seq_kv][head_dim]
 *   lse   [batch][heads][seq_q]     fp32, natural log
 *
 * Ownership and threading. The caller owns every buffer (device memory on
 * the current HIP device) and the stream. The library never allocates, frees
 * or synchronizes; it keeps only a per-device property cache filled on first
 * use. Calls are reentrant and may come from several host threads. Kernels
 * run asynchronously on `stream`; a fault inside a kernel surfaces at the
 * caller's next synchronization. Results are deterministic: the same inputs
 * and sizes give bitwise-identical outputs (no atomics).
 *
 * Errors are returned as sma_status codes; nothing is thrown across the ABI.
 * Host-side argument errors launch nothing.
 */
#ifndef SMA_H
#define SMA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMA_ABI_VERSION 3

/* Element types. Accumulation is always fp32. */
typedef enum {
  SMA_DTYPE_F32 = 0,  /* IEEE binary32 */
  SMA_DTYPE_BF16 = 1, /* bfloat16 (binary32 with the low 16 fraction bits dropped) */
  SMA_DTYPE_F16 = 2   /* IEEE binary16 */
} sma_dtype;

typedef enum {
  SMA_OK = 0,
  SMA_ERR_NULL_POINTER = 1,  /* a required pointer is NULL */
  SMA_ERR_INVALID_VALUE = 2, /* bad size, dtype code, non-finite scale, size overflow */
  SMA_ERR_UNSUPPORTED = 3,   /* valid request the kernels do not implement: head_dim, dtype pair,
                                seq_q or seq_kv above 2^30, bf16 K/V of one (batch, head) of 2 GiB
                                or more, grid limit */
  SMA_ERR_MISALIGNED = 4,    /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
  SMA_ERR_ALIASING = 5,      /* o or lse overlaps q, k, v, the workspace, or each other */
  SMA_ERR_HIP = 6,           /* the HIP runtime reported an error (device query or launch) */
  SMA_ERR_SCRATCH = 7        /* sma_attention_fwd_noalloc: the requested key split needs more
                                than its device scratch (SMA_NOALLOC_SCRATCH_BYTES) */
} sma_status;

/* Memory layout of q, k, v and o (lse is always [B,H,Sq]). Both are dense and
 * row-major with the head dim contiguous. */
typedef enum {
  SMA_LAYOUT_BHSD = 0, /* [batch, heads, seq, head_dim] (what sma_attention_fwd takes) */
  SMA_LAYOUT_BSHD = 1  /* [batch, seq, heads, head_dim]: the heads of one position adjacent, as
                          a fused projection writes them; no transposition is needed */
} sma_layout;

/* Kernels the library can run for one call. Each computes the whole operation;
 * they differ only in how the work is spread over workgroups. */
typedef enum {
  SMA_KERNEL_AUTO = -1,         /* let the library choose (what sma_attention_fwd does) */
  SMA_KERNEL_F32_QBLOCK = 0,    /* fp32: 128 query rows per workgroup; keys optionally split
                                   across workgroups, merged by a second kernel */
  SMA_KERNEL_F32_KSPLIT = 1,    /* fp32: 32 query rows per workgroup, keys split over its four
                                   waves and merged in-workgroup; never needs a workspace (the
                                   automatic fp32 choice unless its grid is small and rows long) */
  SMA_KERNEL_BF16_QBLOCK = 2    /* bf16 or fp16: 256 query rows per workgroup (512 at head dim
                                   128, 192 at 256); keys optionally split across workgroups,
                                   merged by a second kernel */
} sma_kernel;

/* How a call is carried out: filled by sma_attention_fwd_plan, read by
 * sma_attention_fwd_ex. */
typedef struct sma_plan {
  int kernel;              /* an sma_kernel other than SMA_KERNEL_AUTO */
  int nsplit;              /* key splits per query row across workgroups, 1..32 (1 = none) */
  size_t workgroups;       /* workgroups of the main kernel */
  size_t workspace_bytes;  /* workspace this plan needs (0 when nsplit == 1) */
} sma_plan;

/* Attention forward.
 *
 *   q, k, v    device pointers, element type in_dtype, layout above. k and v may
 *              be NULL only when seq_kv == 0; q and o only when batch*heads*seq_q == 0.
 *   o          device pointer, element type o_dtype, fully overwritten.
 *   lse        device pointer to batch*heads*seq_q floats, or NULL for no LSE output.
 *   in_dtype   SMA_DTYPE_F32, SMA_DTYPE_BF16 or SMA_DTYPE_F16 (16-bit inputs run on 16-bit
 *              MFMA with fp32 accumulation; P is rounded to the input type for P V).
 *   o_dtype    SMA_DTYPE_F32, or SMA_DTYPE_BF16 / SMA_DTYPE_F16: the fp32 result rounded
 *              to that type (nearest even; beyond fp16's range, infinity) as it is stored.
 *              Any with any input type. LSE is always fp32.
 *   head_dim   32, 64, 128 or 256 with every input type; SMA_KERNEL_F32_KSPLIT runs
 *              32, 64 and 128 only (0 -> INVALID_VALUE; other values, and 256 forced
 *              onto that kernel -> UNSUPPORTED).
 *   scale      finite multiplier of QK^T (zero and negative values are allowed).
 *   causal     0: no mask; nonzero: bottom-right causal mask.
 *   workspace  optional device scratch for splitting the keys of a row across
 *              workgroups (used when there are too few query blocks to fill the
 *              GPU); NULL or too small just disables splitting, which stays correct.
 *              sma_attention_fwd_workspace_bytes gives the size that enables it.
 *              It must not overlap any other argument. Contents on entry do not matter.
 *   stream     hipStream_t to launch on; NULL means the null stream.
 *
 * batch*heads*seq_q == 0 returns SMA_OK and launches nothing. seq_kv == 0 writes
 * o = +0.0 and lse = -inf for every row.
 */
int sma_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                      size_t seq_kv, size_t head_dim, double scale, int causal, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Measurement hook: exactly sma_attention_fwd, and in addition records the
 * caller's HIP events (hipEvent_t handles, either may be NULL) on `stream`
 * immediately before and after the main attention kernel, so that its
 * duration can be read with hipEventElapsedTime apart from the split-combine
 * kernel that may follow it. The events are recorded only when the call
 * launches (status SMA_OK with work to do). */
int sma_attention_fwd_timed(const void* q, const void* k, const void* v, void* o, float* lse,
                            int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                            size_t seq_kv, size_t head_dim, double scale, int causal,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* event_before, void* event_after);

/* The same checks as sma_attention_fwd, on the host only: no HIP call, nothing
 * launched, pointers are not dereferenced. Returns the status sma_attention_fwd
 * would return before launching. This is the validating no-op backend of the
 * oxicuda ComputeBackend page (its `NullBackend` implementor, which checks a call's
 * arguments and computes nothing), for the attention call alone. */
int sma_attention_fwd_validate(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, int in_dtype, int o_dtype, size_t batch,
                               size_t heads, size_t seq_q, size_t seq_kv, size_t head_dim,
                               double scale, int causal, const void* workspace,
                               size_t workspace_bytes);

/* Workspace bytes that let sma_attention_fwd split keys across workgroups for
 * this shape ([B,H,S,d]) on the current HIP device (if its compute units
 * cannot be queried, as on a host without a GPU, 256 are assumed). 0 means
 * splitting is never used for this shape. Invalid arguments also give 0.
 * sma_attention_fwd_plan gives the same figure for another layout or CU count. */
size_t sma_attention_fwd_workspace_bytes(int in_dtype, size_t batch, size_t heads, size_t seq_q,
                                         size_t seq_kv, size_t head_dim, int causal);

/* The plan for a shape in `layout` (an sma_layout: the row stride it implies
 * enters the size limits and the kernel choice), on the host only (no launch).
 * kernel: SMA_KERNEL_AUTO for the library's own choice, else the kernel to plan
 * for (one that does not run in_dtype or head_dim -> UNSUPPORTED). nsplit: 0
 * lets the library choose the key split; 1..32 asks for that many (the plan may
 * merge splits so that each keeps a whole number of key tiles, and
 * SMA_KERNEL_F32_KSPLIT accepts only 0 or 1, and only (seq_q + 32) and
 * (seq_kv + 32) rows of head_dim floats of at most 2 GiB; otherwise
 * UNSUPPORTED). num_cus: compute units to plan for; 0 for the current HIP
 * device (256 if it cannot be queried). The plan of SMA_KERNEL_AUTO with
 * num_cus = 0 is the one sma_attention_fwd_layout follows when it is given at
 * least plan.workspace_bytes of workspace. Shape errors as
 * sma_attention_fwd_layout; out NULL -> NULL_POINTER. */
int sma_attention_fwd_plan(int in_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                           size_t head_dim, int causal, int layout, int kernel, int nsplit,
                           int num_cus, sma_plan* out);

/* sma_attention_fwd with the memory layout of sma_attention_fwd_layout, the
 * kernel and key split taken from `plan` (NULL: the library's choice, exactly
 * sma_attention_fwd for SMA_LAYOUT_BHSD) and the measurement events of
 * sma_attention_fwd_timed. Only plan->kernel and plan->nsplit are
 * read; the plan is rebuilt from them for this shape and the current device,
 * so plan->workgroups and plan->workspace_bytes are informative. Unlike the
 * automatic choice, an explicit split is never dropped: a workspace smaller
 * than the rebuilt plan needs -> INVALID_VALUE. Results are the same for every
 * plan up to floating-point rounding order. */
int sma_attention_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                         int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                         size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                         void* workspace, size_t workspace_bytes, const sma_plan* plan,
                         void* stream, void* event_before, void* event_after);

/* sma_attention_fwd on tensors in `layout` (an sma_layout; other values ->
 * INVALID_VALUE), with the library's plan. The result is bitwise the same as
 * for the same data in [B,H,S,d]. The size checks apply to the layout's row
 * stride: with SMA_LAYOUT_BSHD one row of a head is heads*head_dim elements
 * from the next, so the 2 GiB limits on (seq + tile) rows are reached at
 * 1/heads the sequence length. sma_attention_fwd_plan with the same layout
 * gives the plan and the workspace that enables its key split; a workspace too
 * small for that plan only disables the key split. */
int sma_attention_fwd_layout(const void* q, const void* k, const void* v, void* o, float* lse,
                             int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                             size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ no allocation
 *
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): sma_attention_fwd_layout
 * with an optional explicit plan (as sma_attention_fwd_ex), whose key-split
 * partials go to a device array of SMA_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends, instead of a caller
 * workspace. It allocates nothing: no hipMalloc, no hipFree, no allocating
 * library call.
 *
 *   plan   NULL: the library's plan (every automatic plan on a 256-CU GPU fits
 *          the scratch; one that would not runs without a key split, which stays
 *          correct). An explicit plan whose split needs more than the scratch ->
 *          SMA_ERR_SCRATCH, before anything is launched.
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * partials (nothing in it needs to start at zero: each call writes every
 * partial it reads). Calls on one stream are ordered; calls that may overlap on
 * one GPU (other streams, other host threads) race on the scratch and must be
 * serialised by the caller. Results are bitwise those of sma_attention_fwd_ex
 * with the same plan. Other arguments, errors and asynchrony as for
 * sma_attention_fwd_ex. */
#define SMA_NOALLOC_SCRATCH_BYTES (72u * 1024u * 1024u)

int sma_attention_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                              size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                              const sma_plan* plan, void* stream);

/* ------------------------------------------------------------------ hard mask
 *
 * sma_attention_fwd_ex with an explicit hard mask, as the TorchLean page's
 * stable row-wise hard-masked softmax defines it: key j takes part in query
 * row i's max and sum only if mask byte (b, h, i, j) is nonzero (and, with
 * `causal`, j <= i + seq_kv - seq_q as well); blocked keys weigh exactly zero
 * and are never read into the arithmetic; a row that admits nothing is +0.0
 * with LSE -inf.
 *
 *   mask           device bytes [mask_batches][mask_heads][seq_q][seq_kv],
 *                  contiguous; mask_batches is 1 or batch and mask_heads 1 or
 *                  heads (1 broadcasts the mask over that dimension). Must not
 *                  overlap o, lse or the workspace (ALIASING).
 *   workspace      required: the mask packed to one bit per pair comes first,
 *                  else INVALID_VALUE: for fp32 inputs 4 bytes per 32 keys of a
 *                  row; for 16-bit inputs 4 bytes per key of each 32-row block
 *                  (keys rounded up to 64) plus 4 bytes per 64-key tile of each
 *                  block, which class the tile as admitting nothing (skipped),
 *                  everything (run unmasked) or a mix; each part 256-byte
 *                  aligned. A key split across workgroups uses the bytes after
 *                  it (too few of them only disables the library's split, as for
 *                  sma_attention_fwd). sma_attention_fwd_masked_workspace_bytes
 *                  gives both.
 *   plan           as for sma_attention_fwd_ex: every kernel applies the mask.
 * Everything else as for sma_attention_fwd_ex. mask NULL with nonzero
 * mask_batches or mask_heads -> NULL_POINTER (when there is work); a mask
 * with mask_batches = mask_heads = 0 is INVALID_VALUE. */
int sma_attention_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                             const void* mask, size_t mask_batches, size_t mask_heads, int in_dtype,
                             int o_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                             size_t head_dim, double scale, int causal, int layout, void* workspace,
                             size_t workspace_bytes, const sma_plan* plan, void* stream,
                             void* event_before, void* event_after);

/* Workspace bytes sma_attention_fwd_masked needs: the packed mask plus the
 * library's key split on the current HIP device (256 CUs assumed if it cannot
 * be queried); 0 for invalid arguments. */
size_t sma_attention_fwd_masked_workspace_bytes(int in_dtype, size_t batch, size_t heads,
                                                size_t seq_q, size_t seq_kv, size_t head_dim,
                                                int causal, int layout, size_t mask_batches,
                                                size_t mask_heads);

/* ------------------------------------------------------------------ backward
 *
 * Gradients of the forward above with respect to q, k and v, given the
 * upstream gradient dout = dL/dO, the forward's output o and its log-sum-exp
 * lse (the composition of the forward's two products with the softmax
 * vector-Jacobian product dx = y (dy - sum y dy): pulsatrix HIPBackend page,
 * `softmax_rows_backward`; MicroGPT page, the fused attention-softmax
 * backward). Per (batch, head), over the admitted pairs (i, j):
 *   P_ij = exp(scale q_i.k_j - lse_i),  dP_ij = dout_i . v_j,
 *   D_i = dout_i . o_i,  dS_ij = P_ij (dP_ij - D_i),
 *   dv_j = sum_i P_ij dout_i,  dk_j = scale sum_i dS_ij q_i,  dq_i = scale sum_j dS_ij k_j.
 * P is recomputed from q, k and lse; o enters only through D. Both must be
 * what sma_attention_fwd returned for these q, k, v, scale and causal (a row
 * with no admitted key has lse = -inf and gets dq = 0; it adds nothing to dk
 * and dv). Results are bitwise reproducible: no atomics.
 *
 *   q, o, dout, dq   [B,H,Sq,d];  k, v, dk, dv  [B,H,Skv,d];  lse [B,H,Sq].
 *   in_dtype         element type of q, k and v: SMA_DTYPE_F32 (fp32 MFMA), or
 *                    SMA_DTYPE_BF16 or SMA_DTYPE_F16 (16-bit MFMA with fp32
 *                    accumulation, under the forward's mixed-precision contract:
 *                    dout is rounded once to the input type for the products, and
 *                    P and dS are rounded to it for the products that take them;
 *                    D = dout . o stays fp32). fp16 is not rescaled: the caller keeps
 *                    dout, and with it dS = P (dout . v - D), inside fp16's range
 *                    (beyond 65504 the results are not finite; under 2^-14 bits are
 *                    lost), as loss scaling does. o, dout, lse and the three
 *                    gradients are always fp32 (o as sma_attention_fwd returns it).
 *   head_dim         32, 64 or 128; 256 with bf16 or fp16 inputs (others, and 256 with
 *                    fp32 inputs, -> UNSUPPORTED).
 *   scale, causal, stream   as for sma_attention_fwd.
 *   workspace        required device scratch of at least
 *                    sma_attention_bwd_workspace_bytes bytes (smaller or NULL
 *                    when that is nonzero -> INVALID_VALUE); contents on entry
 *                    do not matter; it must not overlap any other argument.
 *
 * Pointers are device memory on the current HIP device, 16-byte aligned (lse
 * 4-byte). q, o, lse, dout and dq may be NULL only when batch*heads*seq_q == 0,
 * k, v, dk and dv only when batch*heads*seq_kv == 0. The gradients and the
 * workspace must not overlap the inputs or each other (ALIASING). Every
 * element of dq, dk and dv is written: seq_kv == 0 gives dq = 0, seq_q == 0
 * gives dk = dv = 0. Per (batch, head), (seq_q + 32) and (seq_kv + 32) rows of
 * head_dim floats must stay within 2 GiB (else UNSUPPORTED). Other errors as
 * for sma_attention_fwd. Asynchronous on `stream`; nothing is allocated. */
int sma_attention_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv,
                      int in_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                      size_t head_dim, double scale, int causal, void* workspace,
                      size_t workspace_bytes, void* stream);

/* sma_attention_bwd with the memory layout of sma_attention_fwd_layout: with
 * SMA_LAYOUT_BSHD, q, o, dout and dq are [B,Sq,H,d] and k, v, dk and dv
 * [B,Skv,H,d] (lse stays [B,H,Sq]); SMA_LAYOUT_BHSD is sma_attention_bwd. The
 * workspace is the same size for both layouts. The 2 GiB limit counts rows of
 * heads*head_dim elements under SMA_LAYOUT_BSHD. Gradients are bitwise those of
 * SMA_LAYOUT_BHSD on the transposed tensors. Other arguments and errors as for
 * sma_attention_bwd; a layout code other than the two -> INVALID_VALUE. */
int sma_attention_bwd_layout(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, float* dq, float* dk, float* dv,
                             int in_dtype, size_t batch, size_t heads, size_t seq_q,
                             size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                             void* workspace, size_t workspace_bytes, void* stream);

/* sma_attention_bwd_layout with the hard mask of sma_attention_fwd_masked:
 * the gradients of that forward (TorchLean page, hard-masked softmax: a pair
 * whose mask byte is zero has no probability, so it adds nothing to any
 * gradient; a row that admits nothing gets dq = 0). o and lse must be what
 * sma_attention_fwd_masked returned for the same mask. mask, mask_batches and
 * mask_heads as for sma_attention_fwd_masked (device bytes, nonzero admits, a
 * size of 1 broadcasts; combined with the causal bound when causal). The
 * workspace (sma_attention_bwd_masked_workspace_bytes) holds the packed mask
 * after what sma_attention_bwd needs. The mask must not overlap dq, dk, dv or
 * the workspace (ALIASING). Other arguments and errors as for
 * sma_attention_bwd_layout. */
int sma_attention_bwd_masked(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, float* dq, float* dk, float* dv,
                             const void* mask, size_t mask_batches, size_t mask_heads,
                             int in_dtype, size_t batch, size_t heads, size_t seq_q,
                             size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sma_attention_bwd_masked needs: those of sma_attention_bwd,
 * then the packed mask (one 32-bit word per 32 keys of each row of each
 * (mask batch, mask head), rounded up to 256). 0 for invalid arguments. */
size_t sma_attention_bwd_masked_workspace_bytes(int in_dtype, size_t batch, size_t heads,
                                                size_t seq_q, size_t seq_kv, size_t head_dim,
                                                int causal, int layout, size_t mask_batches,
                                                size_t mask_heads);

/* Workspace bytes sma_attention_bwd needs for this shape: 256 per 32-row query
 * block of every (batch, head), rounded up to 256; with 16-bit inputs also
 * batch*heads*seq_q*head_dim*2 bytes (dout in 16 bits), rounded up to 256. 0 for
 * invalid arguments. */
size_t sma_attention_bwd_workspace_bytes(int in_dtype, size_t batch, size_t heads, size_t seq_q,
                                         size_t seq_kv, size_t head_dim, int causal);

/* Measurement hook: exactly sma_attention_bwd, and in addition records the
 * caller's HIP events (either may be NULL) on `stream` after the preprocess
 * kernel and after the dK/dV kernel; the dQ kernel follows. */
int sma_attention_bwd_timed(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, float* dq, float* dk, float* dv,
                            int in_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                            size_t head_dim, double scale, int causal, void* workspace,
                            size_t workspace_bytes, void* stream, void* event_after_pre,
                            void* event_after_dkdv);

/* ------------------------------------------------------------------ row primitives
 *
 * Softmax-family operations on a materialised fp32 score matrix, row-major
 * [rows][cols] (contiguous, row i at in + i*cols). Per row, over the admitted
 * entries j:  m = max s_j,  p_j = exp(s_j - m) / sum_k exp(s_k - m),
 * lse = m + log(sum_k exp(s_k - m)) (natural log), with s_j = x_j, or
 * scale * x_j for sma_scaled_causal_softmax. Entries not admitted are written
 * as exactly 0 and their input is never used (it may be NaN). An input of
 * -infinity at an admitted position weighs zero (also under any scale); a row
 * whose admitted inputs are all -infinity, or that admits nothing, is all
 * zeros and its log-sum-exp is -infinity. Admitted inputs of +infinity or NaN
 * are undefined.
 *
 * Pointers are device memory on the current HIP device, 4-byte aligned (16-
 * byte alignment with cols a multiple of 4 selects vector loads). `out` may be
 * the same buffer as `in` (in-place) but must not overlap it otherwise, nor
 * the mask. rows and cols up to 2^31 - 1. Asynchronous on `stream`; nothing
 * is allocated. rows*cols = 0 launches nothing, except that
 * sma_logsumexp_rows with cols = 0 writes -infinity for every row.
 * Errors as for the attention calls (NULL_POINTER, MISALIGNED, ALIASING,
 * INVALID_VALUE for size overflow or a non-finite scale, UNSUPPORTED past the
 * size limits, HIP). */

/* Row softmax, max-subtracted (pulsatrix HIPBackend page, `softmax_rows`). */
int sma_softmax_rows(const float* in, float* out, size_t rows, size_t cols, void* stream);

/* Per-row log-sum-exp, max-subtracted (pulsatrix HIPBackend page,
 * `logsumexp_rows`): out[i] for i < rows. */
int sma_logsumexp_rows(const float* in, float* out, size_t rows, size_t cols, void* stream);

/* Hard-masked row softmax (TorchLean "CUDA Buffer Kernels FFI" page, stable
 * row-wise hard-masked softmax): entry j of row i is admitted iff
 * mask[i][j] != 0 (mask fp32, same layout as in). */
int sma_masked_softmax_rows(const float* in, const float* mask, float* out, size_t rows,
                            size_t cols, void* stream);

/* Scale, causal mask and softmax in one pass (MicroGPT CuBLASBackend page,
 * `fused_attn_softmax`) over `batch` matrices of [rows][cols]: s = scale * x,
 * and with causal nonzero row r of each matrix admits j <= r + cols - rows
 * (bottom-right, as in the attention call). scale must be finite. */
int sma_scaled_causal_softmax(const float* in, float* out, size_t batch, size_t rows, size_t cols,
                              double scale, int causal, void* stream);

/* Softmax backward from the forward's output (pulsatrix HIPBackend page,
 * `softmax_rows_backward`; with scale, the backward of the MicroGPT
 * CuBLASBackend page's fused scale + mask + softmax, `fused_attn_softmax_backward`):
 * for each of `rows` rows of `cols` fp32 entries,
 *     dx_j = scale * y_j * (dy_j - sum_k y_k * dy_k),
 * with y the softmax output and dy the gradient with respect to it, both
 * row-major [rows][cols]. Entries the forward blocked have y = 0 and get
 * dx = 0. scale = 1 is the plain softmax backward; the fused op's scale
 * gives the gradient with respect to its unscaled input. The dot product is
 * accumulated in fp32 (fused multiply-adds, then a tree over the lanes).
 * dx may be the same buffer as y or dy (in place) but must not overlap them
 * otherwise; y and dy may overlap each other. Alignment, sizes, errors and
 * asynchrony as for the row primitives above; scale must be finite;
 * rows*cols = 0 launches nothing. */
int sma_softmax_rows_backward(const float* y, const float* dy, float* dx, size_t rows, size_t cols,
                              double scale, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* sma_status_string(int status);

/* SMA_ABI_VERSION of the built library. */
int sma_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMA_H */
