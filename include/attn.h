/*
 * attn.h - C ABI of the exact blockwise attention forward library (libattn.so).
 *
 * The operation.  For every batch b, head h and query row i, with N queries and
 * N keys per head:
 *
 *     s_ij   = scale * <q_i, k_j>             for keys j allowed by the mask
 *     O_i    = sum_j softmax_j(s_ij) v_j      (masked keys get probability 0)
 *     LSE_i  = ln sum_j exp(s_ij)             (natural log, allowed keys only)
 *
 * This is softmax(Q K^T / sqrt(d_k)) V ("Transformer多头注意力8头并行计算PyTorch实现与
 * CUDA核函数优化", §1), with masked scores set to -inf before the softmax (same page,
 * §2.2).  It is computed blockwise: every block of queries walks the keys tile by
 * tile with a running maximum and sum, so the N x N score matrix never exists
 * ("Blockwise Parallel Transformer in PyTorch", the blockwise_attention example;
 * Mosaic long-sequence attention page, §2.2 and §3.2).  LSE is the log-space
 * statistic that keeps the softmax free of overflow (Mosaic page, §5.1).
 *
 * Masks (mask_kind):
 *     ATTN_MASK_NONE    every key
 *     ATTN_MASK_CAUSAL  key j allowed iff j <= i (square, top-left aligned)
 *     ATTN_MASK_WINDOW  key j allowed iff |i - j| <= window, the inclusive band of
 *                       the sliding-window section ("长序列推理中的注意力机制优化策略与实践",
 *                       §2.1); clipped at both ends of the sequence.
 *     ATTN_MASK_CAUSAL_WINDOW  key j allowed iff i - window <= j <= i: the band's
 *                       causal half (a token sees itself and the window tokens
 *                       before it, as an autoregressive model with a bounded KV
 *                       cache does).
 * Every row has at least one allowed key (its own), so O and LSE are always finite
 * for finite inputs.
 */
#ifndef ATTN_H
#define ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

enum attn_mask_kind { ATTN_MASK_NONE = 0, ATTN_MASK_CAUSAL = 1, ATTN_MASK_WINDOW = 2, ATTN_MASK_CAUSAL_WINDOW = 3 };

enum attn_dtype { ATTN_DTYPE_F32 = 0, ATTN_DTYPE_BF16 = 1 };

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_PTR = -1,              /* a tensor pointer is NULL                        */
    ATTN_ERR_BAD_SHAPE = -2,             /* B, H or N <= 0, or a size overflows the limits  */
    ATTN_ERR_UNSUPPORTED_HEAD_DIM = -3,  /* d not in {64, 128}                              */
    ATTN_ERR_BAD_MASK = -4,              /* unknown mask_kind, or window < 0 for WINDOW     */
    ATTN_ERR_BAD_DTYPE = -5,             /* dtype not an attn_dtype                         */
    ATTN_ERR_ALIAS = -6,                 /* an output overlaps an input or another output   */
    ATTN_ERR_BAD_SCALE = -7,             /* scale is NaN or infinite                        */
    ATTN_ERR_MISALIGNED = -8,            /* a tensor pointer is not 16-byte aligned         */
    ATTN_ERR_HIP = -9,                   /* the HIP runtime reported an error at launch     */
    ATTN_ERR_WORKSPACE = -10,            /* workspace NULL or smaller than required         */
    ATTN_ERR_SCRATCH_LIMIT = -11         /* attn_fwd_kv_noalloc: the shape needs more than
                                            ATTN_NOALLOC_SCRATCH_BYTES of scratch           */
};

/*
 * attn_fwd - exact attention forward, O and LSE.
 *
 *   q, k, v   device pointers, each a contiguous row-major [B, H, N, d] tensor of
 *             `dtype` (fp32 or bf16); read only.
 *   out       device pointer, contiguous [B, H, N, d] of `dtype`; fully overwritten.
 *   lse       device pointer, contiguous [B, H, N] of fp32; fully overwritten.
 *   B, H, N   batch, heads, sequence length; each >= 1.  Limits: N * d < 2^31,
 *             B * H * N < 2^31.
 *   d         head dimension: 64 or 128.
 *   scale     softmax scale applied to q.k (1/sqrt(d) for standard attention); finite.
 *   mask_kind an attn_mask_kind.
 *   window    band half-width w >= 0; read only for ATTN_MASK_WINDOW and
 *             ATTN_MASK_CAUSAL_WINDOW.
 *   dtype     an attn_dtype: the element type of q, k, v and out.  bf16 inputs are
 *             multiplied on bf16 matrix cores with fp32 accumulation; the
 *             probabilities are rounded to bf16 for the P.V product; O is rounded
 *             to bf16 (nearest-even) from fp32.  fp32 inputs are computed in fp32.
 *   stream    a hipStream_t (NULL = the default stream) on the current device.
 *
 * Ownership: the caller allocates and frees all five buffers on the current
 * device.  The library allocates nothing, frees nothing and never synchronises:
 * the call enqueues the work on `stream` and returns.  It keeps no state between
 * calls and may be called concurrently from several host threads.
 *
 * Tile shape: bf16 calls pick 64 or 32 query rows per wave from the shape (32 for a
 * grid too small to fill the device twice, a window w < 2048 or a causal window w < 4096), and
 * run workgroups in groups of heads whose K and V fit in half the device's 256 MB
 * Infinity Cache.  attn_set_schedule forces either choice; neither changes a result
 * beyond the rounding of the bf16 probabilities.  When the query blocks alone
 * would leave the device short of work (no mask or causal, at most one or two
 * workgroups per compute unit), the waves of a workgroup also split its keys into
 * 2 or 4 key groups whose softmax states are merged exactly at the end (the merge
 * of local attention results of the Mosaic long-sequence page, §2.1, applied inside
 * the workgroup); attn_set_key_groups forces that choice.
 *
 * Errors: returns ATTN_OK (0) or a negative attn_status.  Argument errors are
 * detected on the host before anything is enqueued, so nothing is written on such
 * an error.  ATTN_ERR_HIP means the launch itself failed (hipGetLastError); the
 * outputs are then undefined.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int H, int N, int d, float scale, int mask_kind, int window,
             int dtype, void* stream);

/*
 * attn_check_args - the host-side argument check attn_fwd performs, on its own.
 * Same arguments as attn_fwd minus the stream; touches no device and no pointer
 * target (pointers are compared, never dereferenced).  Returns what attn_fwd
 * would return before launching.
 */
int attn_check_args(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    int B, int H, int N, int d, float scale, int mask_kind, int window, int dtype);

/*
 * attn_bwd - gradients of the attention forward: dq, dk, dv for an upstream dout.
 *
 * For O = softmax(scale Q K^T) V with the mask of attn_fwd, and L any scalar with
 * dL/dO = dout, computes dq = dL/dq, dk = dL/dk, dv = dL/dv:
 *     dV = P^T dO,  dP = dO V^T,  D_i = <dO_i, O_i>,  dS = P o (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q,
 * the derivative of the forward map (masked keys excluded).  P is recomputed from
 * q, k and the forward's lse rather than stored: the recomputation in the backward
 * pass that the "长序列推理中的注意力机制优化策略与实践" page describes for FlashAttention
 * (§3.1), which keeps memory O(N) like the gradient checkpointing of the Mosaic
 * long-sequence attention page (§2.2).
 *
 *   q, k, v, out, dout  device pointers, contiguous [B, H, N, d] bf16; read only.
 *             out and lse must be what attn_fwd returned for these q, k, v, scale
 *             and mask (they define P and D).
 *   lse       device pointer, contiguous [B, H, N] fp32 (attn_fwd's output); read only.
 *   dq, dk, dv  device pointers, contiguous [B, H, N, d] bf16; fully overwritten.
 *             dq also serves as the scratch for D between the three kernels the
 *             call enqueues, so its contents are undefined until the stream
 *             reaches the end of the call.
 *   B, H, N, d, scale, mask_kind, window  as for attn_fwd.
 *   dtype     ATTN_DTYPE_BF16 (fp32 inputs are not supported by the backward:
 *             ATTN_ERR_BAD_DTYPE).  Products on bf16 matrix cores with fp32
 *             accumulation; P and dS are rounded to bf16 for the products that
 *             consume them; the outputs are rounded to bf16 (nearest-even).
 *   stream    a hipStream_t (NULL = the default stream) on the current device.
 *
 * Ownership and errors as for attn_fwd: the library allocates nothing; argument
 * errors (including any of dq, dk, dv overlapping an input or each other) are
 * reported before anything is enqueued.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int mask_kind, int window,
             int dtype, void* stream);

/*
 * attn_bwd_check_args - the host-side argument check attn_bwd performs, on its own
 * (same arguments minus the stream; pointers are compared, never dereferenced).
 */
int attn_bwd_check_args(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, const void* dq, const void* dk, const void* dv, int B, int H, int N,
                        int d, float scale, int mask_kind, int window, int dtype);

/*
 * attn_fwd_kv - attention forward for Nq new queries against Nk >= Nq cached keys.
 *
 * Query row i of every (b, h) sits at position p_i = q_offset + i of the key
 * sequence (a chunk of new tokens after q_offset cached ones; decode is Nq = 1,
 * q_offset = Nk - 1), and the masks of attn_fwd apply to positions: causal allows
 * keys j <= p_i, the window |p_i - j| <= window, the causal window
 * p_i - window <= j <= p_i.  The output is that of attn_fwd on the full sequence,
 * restricted to rows q_offset .. q_offset + Nq - 1.  This is the KV-cache reading
 * of the long-sequence inference page ("长序列推理中的注意力机制优化策略与实践", §4.1:
 * the keys and values of earlier tokens are kept and reused); its decode case is
 * bound by memory bandwidth, not by arithmetic ("万亿参数大模型Day-0适配实践与稀疏
 * 注意力优化", §二, item 2).  When the query blocks alone would leave the device
 * idle, the keys of each head are cut into ranges processed by separate
 * workgroups, each producing a partial O and LSE, which are merged exactly:
 * LSE = ln sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r (the blockwise
 * combination of the Mosaic long-sequence attention page, §2.2, over key ranges).
 *
 *   q         device pointer, contiguous [B, H, Nq, d] bf16; read only.
 *   k, v      device pointers, contiguous [B, H, Nk, d] bf16; read only.
 *   out       device pointer, contiguous [B, H, Nq, d] bf16; fully overwritten.
 *   lse       device pointer, contiguous [B, H, Nq] fp32; fully overwritten.
 *   B, H      batch and heads, >= 1.
 *   Nq, Nk    query rows and keys per head: 1 <= Nq, q_offset + Nq <= Nk.
 *             Limits: Nk * d < 2^31, B * H * Nk < 2^31.
 *   d         64 or 128.
 *   scale, mask_kind, window  as for attn_fwd (window clamped to Nk - 1).
 *   q_offset  position of query row 0, >= 0.
 *   dtype     ATTN_DTYPE_BF16 (ATTN_DTYPE_F32: ATTN_ERR_BAD_DTYPE).  Arithmetic as
 *             for attn_fwd's bf16 path; the partials are fp32.
 *   workspace device pointer to at least attn_fwd_kv_workspace_size(B, H, Nq, Nk, d)
 *             bytes, 16-byte aligned, owned by the caller and overlapping no
 *             tensor argument; may be NULL when that size is 0.  Its contents
 *             are undefined after the call; it must not be reused by other work
 *             until the stream reaches the end of the call.
 *   workspace_bytes  its size in bytes.
 *   stream    a hipStream_t (NULL = the default stream) on the current device.
 *
 * Ownership and errors as for attn_fwd: the library allocates nothing; argument
 * errors are reported before anything is enqueued (ATTN_ERR_WORKSPACE for a
 * missing or short workspace).
 */
int attn_fwd_kv(const void* q, const void* k, const void* v, void* out, float* lse,
                int B, int H, int Nq, int Nk, int d, float scale, int mask_kind, int window, int q_offset,
                int dtype, void* workspace, unsigned long long workspace_bytes, void* stream);

/*
 * attn_fwd_kv_workspace_size - bytes of workspace attn_fwd_kv needs for this shape
 * (0 when the keys are not split).  A function of the arguments alone; returns 0
 * for arguments attn_fwd_kv would reject as a bad shape.
 */
unsigned long long attn_fwd_kv_workspace_size(int B, int H, int Nq, int Nk, int d);

/*
 * attn_fwd_kv_check_args - the host-side argument check attn_fwd_kv performs, on
 * its own (same arguments minus the stream; pointers are compared, never
 * dereferenced).
 */
int attn_fwd_kv_check_args(const void* q, const void* k, const void* v, const void* out, const float* lse,
                           int B, int H, int Nq, int Nk, int d, float scale, int mask_kind, int window,
                           int q_offset, int dtype, const void* workspace, unsigned long long workspace_bytes);

/*
 * attn_fwd_kv_noalloc - attn_fwd_kv for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, kernels and result, with the split-KV
 * partials kept in a static device array of the library instead of a caller
 * workspace.  The call allocates and frees nothing.
 *
 *   q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset, dtype,
 *   stream    as for attn_fwd_kv.
 *
 * Limit: shapes whose attn_fwd_kv_workspace_size exceeds ATTN_NOALLOC_SCRATCH_BYTES
 * (64 MiB) are rejected with ATTN_ERR_SCRATCH_LIMIT before anything is enqueued
 * (decode fits for any cache size; chunks of Nq queries fit while B * H * splits *
 * Nq * (d + 1) * 4 bytes does; call attn_fwd_kv with a workspace otherwise).
 * Each device holds its own copy of the array until the process ends, and every
 * call on that device shares it: calls whose work may overlap on one device (two
 * streams, or two host threads) race on it and must be ordered by the caller.  A
 * call on one stream is safe after any earlier call on the same stream.  Other
 * errors as for attn_fwd_kv.
 */
enum { ATTN_NOALLOC_SCRATCH_BYTES = 67108864 };

int attn_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int H, int Nq, int Nk, int d, float scale, int mask_kind, int window,
                        int q_offset, int dtype, void* stream);

/*
 * attn_fwd_block_sparse - exact attention restricted to a block layout.
 *
 * The keys are cut into blocks of ATTN_BLOCK_SPARSE_BLOCK (128) tokens and so are
 * the queries; layout[h][qb][kb] != 0 allows every key of block kb for every query
 * of block qb in head h (the same layout for every batch entry).  With causal = 1
 * the layout is intersected with j <= i.  For every allowed set A(i) the result is
 * exact attention over A(i), as attn_fwd computes it for its masks; a row with no
 * allowed key gets O = 0 and LSE = -inf.  Blocks the layout excludes are never
 * read: the block-sparse attention that the long-sequence inference page
 * ("长序列推理中的注意力机制优化策略与实践", §2.1 sparse attention, §7 block-sparse as
 * the configuration for AMD parts) and the Mosaic long-sequence attention page
 * (§6, block sparsity beyond 100K tokens) describe, as a whole-tile skip.
 *
 *   q, k, v, out, lse, B, H, N, d, scale  as for attn_fwd (bf16 only).
 *   causal    0 or 1.
 *   layout    device pointer to H x nb x nb bytes, nb = ceil(N / 128), row-major
 *             [H, nb, nb]; read only.  nb <= ATTN_BLOCK_SPARSE_MAX_BLOCKS.
 *   dtype     ATTN_DTYPE_BF16 (ATTN_DTYPE_F32: ATTN_ERR_BAD_DTYPE).
 *   stream    a hipStream_t (NULL = the default stream) on the current device.
 *
 * Ownership and errors as for attn_fwd; out or lse overlapping the layout is
 * ATTN_ERR_ALIAS, a missing layout ATTN_ERR_NULL_PTR, causal outside {0, 1}
 * ATTN_ERR_BAD_MASK.
 */
enum { ATTN_BLOCK_SPARSE_BLOCK = 128, ATTN_BLOCK_SPARSE_MAX_BLOCKS = 8192 };

int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int H, int N, int d, float scale, int causal,
                          const unsigned char* layout, int dtype, void* stream);

/* attn_fwd_block_sparse_check_args - its host-side argument check, on its own. */
int attn_fwd_block_sparse_check_args(const void* q, const void* k, const void* v, const void* out,
                                     const float* lse, int B, int H, int N, int d, float scale, int causal,
                                     const unsigned char* layout, int dtype);

/*
 * attn_set_schedule - force the schedule choices the library otherwise makes from
 * the shape, process-wide, for every later call (a tuning and test switch, not part
 * of the operation: every setting computes the same result, bit for bit for a
 * given tile shape).
 *
 *   rows_per_wave  query rows per wave of the bf16 forward kernels: 32 or 64, or 0
 *                  for the library's own choice.
 *   head_group     heads per workgroup group of the bf16 forward and backward
 *                  kernels (groups run one after another so that their K and V stay
 *                  in the Infinity Cache): n >= 1 heads, 0 for a single group of
 *                  every head, or -1 for the library's own choice.
 *
 * Returns ATTN_OK, or ATTN_ERR_BAD_SHAPE for a value outside those sets (then
 * nothing changes).  Safe to call from any thread; calls already enqueued keep the
 * schedule they were launched with.
 */
int attn_set_schedule(int rows_per_wave, int head_group);

/*
 * attn_set_key_groups - force the number of key groups of the bf16 forward with no
 * mask or the causal mask, process-wide, for every later attn_fwd call (a tuning
 * and test switch like attn_set_schedule).  With g key groups the four waves of a
 * workgroup form 4 / g sets of query rows times g sets of key tiles (tile t_lo +
 * g u + j for group j at step u); each group keeps its own running maximum and sums,
 * and the groups are merged at the end with weights 2^(m_j - max m).  The result is
 * the same attention up to the rounding of the bf16 probabilities, which are
 * taken against each group's own maximum.
 *
 *   key_groups  1 (never split the keys), 2 or 4, or -1 for the library's own
 *               choice (the default).  Rows per wave come from attn_set_schedule
 *               when it forces them, else 32 for 2 groups at d = 64 and 64
 *               otherwise.  The band masks always use one group.  With -1 and a
 *               forced rows_per_wave, keys are split only where the library's own
 *               choice has those rows per wave.
 *
 * Returns ATTN_OK, or ATTN_ERR_BAD_SHAPE for another value (then nothing changes).
 * Safe to call from any thread; calls already enqueued keep their setting.
 */
int attn_set_key_groups(int key_groups);

/*
 * attn_set_work_queue - how the bf16 forward deals its (query block, head) items to
 * workgroups, process-wide, for every later attn_fwd call (a tuning and test switch
 * like attn_set_schedule: every setting computes the same result, bit for bit).
 *
 * Without the queue, workgroup i computes item i, and the dispatcher deals the
 * workgroups to the device's 8 XCDs round robin, an equal share each, however fast
 * each XCD runs.  With it, the first three quarters of every XCD's items stay fixed
 * that way; the rest are claimed at run time (one atomic counter per XCD in a slot
 * of a device array the library owns), first from the claiming workgroup's own XCD,
 * then from the others, and the grid carries a few extra workgroups per XCD, so an
 * XCD that runs ahead takes over the tail of a slower one (the balance of the
 * multi-die schedule; the Mosaic long-sequence page, §3.1, asks for balanced work
 * across devices).  A launch leaves its slot at zero when its last claiming
 * workgroup has claimed; the library rotates over 64 slots per device, so launches
 * share a slot only if 64 of them run at once on one device.  A call made while its
 * stream is being captured into a graph runs without the queue (the captured
 * launch would keep one slot for every replay).
 *
 *   mode  1 (use the queue for every launch it serves: the unmasked and causal
 *         forward at 64 query rows per wave and one key group), 0 (never), or -1
 *         for the library's own choice (the default: those launches when they have
 *         at least 8192 workgroups).
 *
 * Returns ATTN_OK, or ATTN_ERR_BAD_SHAPE for another value (then nothing changes).
 * Safe to call from any thread; calls already enqueued keep their setting.
 */
int attn_set_work_queue(int mode);

/* attn_strerror - static, NUL-terminated text for a status code (never NULL). */
const char* attn_strerror(int status);

/* attn_version - static, NUL-terminated library version and target string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
