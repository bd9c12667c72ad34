/*
 * fa.h -- C ABI of the MI355X (gfx950) fused attention forward library (libfa.so).
 *
 * The operation is exact masked softmax attention with grouped-query KV heads,
 * computed without materialising the M x N score matrix:
 *
 *     O[b,h,i,:] = sum_{j visible to i} softmax_j( scale * q[b,h,i,:] . k[b,hk,j,:] ) * v[b,hk,j,:]
 *     hk = h / (Hq / Hkv)
 *     lse[b,h,i] = ln sum_{j visible to i} exp( scale * q[b,h,i,:] . k[b,hk,j,:] )
 *
 * Sources (web pages, cited by title and section):
 *   - "从零开始写Qwen3" (FlashAttention derivation article), sections "在线softmax" and
 *     "FlashAttention": the online-softmax recurrence, the FlashAttention-2 tiling with
 *     the KV sequence as the inner loop, the grouped KV head mapping (query head // groups)
 *     and the causal mask (query index >= key index) of its kernel listing.
 *   - "从零开始写Qwen3" (FlashAttention speed-up article), sections "改进1-使用正确的grid",
 *     "改进2-KV只读取下三角", "改进3-两阶段计算", "优化点6-使用exp2而不是exp" and
 *     "改进点7-把stride当成常量": Q tiles fastest in the grid, KV tiles above the diagonal
 *     never visited, unmasked tiles separated from the masked diagonal band, exp2 with
 *     log2(e) folded into the scale, unit stride along the head dimension.
 *   - "Flash Attention CUDA Kernel 优化: 从 56 到 986 TFLOPS on B300 — G2", section
 *     "V6: 算术指令优化" ("第一处：推迟 scale 乘法"): scale and max subtraction fused in one
 *     FMA feeding exp2, valid because scale > 0.
 *
 * Readings taken where those pages are silent:
 *   - causal alignment for M != N is bottom-right: key j is visible to query i iff
 *     j <= i + (N - M) (the pages' "i >= j" when M == N);
 *   - a query row that sees no key (causal, M > N) gets O = 0 and lse = -inf;
 *   - lse is the natural log over the *scaled* logits.
 *
 * Every entry point below (and those of gdn.h) validates its arguments on the host, then only
 * enqueues kernels on the caller's stream: it never allocates, frees, memsets or
 * synchronises, and keeps no state between calls.  Calls are therefore safe from several host
 * threads at once and can be captured into a HIP graph (stream capture); outputs and
 * workspaces keep the addresses the captured call was given.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* input/output element type */
typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

/* Element strides of the batch, head and row axes of a [B, H, S, D] tensor; the D axis always
 * has unit stride.  Contiguous row-major is {H*S*D, S*D, D}; a [B, S, H, D] buffer viewed as
 * [B, H, S, D] is {S*H*D, D, H*D}. */
typedef struct {
    long long batch, head, row;
} fa_strides;

/* return codes */
enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, Hq % Hkv != 0, scale not finite or <= 0,
                                unknown dtype, sizes whose element counts overflow int64 */
    FA_ERR_UNSUPPORTED = -2, /* D not in {64, 128}, a pointer or row not 16-byte aligned, a K/V row stride
                                over 17 043 456 elements, or a grid beyond 2^31 - 1 workgroups */
    FA_ERR_LAUNCH = -3,      /* the kernel launch reported an error (hipGetLastError) */
    FA_ERR_SCRATCH_TOO_SMALL = -4 /* fa_fwd_splitkv_noalloc: the plan's partial results exceed its scratch */
};

/*
 * fa_fwd -- fused attention forward on one GPU.
 *
 * Arguments (all tensors contiguous, row-major, DEVICE memory owned by the caller):
 *   q    [B, Hq,  M, D]  fp16 or bf16 (dtype)
 *   k    [B, Hkv, N, D]  same dtype
 *   v    [B, Hkv, N, D]  same dtype
 *   o    [B, Hq,  M, D]  same dtype, written (rounded to nearest even); must not alias q, k, v
 *   lse  [B, Hq,  M]     fp32, written: natural-log logsumexp of each row's scaled logits
 *   B, Hq, Hkv, M, N, D  sizes; Hq must be a multiple of Hkv (query head h reads KV head
 *                        h / (Hq / Hkv)); D must be 64 or 128
 *   scale                > 0 and finite (usually 1/sqrt(D))
 *   causal               0: every key visible; nonzero: key j visible to query i iff j <= i + N - M
 *   dtype                FA_F16 or FA_BF16
 *   stream               a hipStream_t, or NULL for the default stream
 *
 * All pointers must be 16-byte aligned.  Indexing is 64-bit (K and V rows inside one 64-key tile
 * use 32-bit buffer offsets).
 *
 * Behaviour: validates every argument before any HIP call and returns a negative code
 * without touching the GPU if one is bad.  Otherwise enqueues one kernel on `stream`
 * and returns FA_OK without synchronising; the library allocates nothing, frees nothing
 * and keeps no global mutable state, so concurrent calls on different streams are safe.
 * Device faults surface at the caller's next synchronisation, as for any HIP kernel.
 * The result is deterministic: the same inputs give the same bits on every call.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int M, int N,
           int D, float scale, int causal, int dtype, void *stream);

/*
 * fa_fwd_strided -- fa_fwd on tensors with arbitrary batch / head / row strides ("从零开始写Qwen3"
 * (derivation article), section "FlashAttention": the kernel listing takes a stride for every
 * axis of q, k, v and o).  A NULL stride pointer means that tensor is contiguous, so
 * fa_fwd(...) == fa_fwd_strided(..., NULL, NULL, NULL, NULL, ...).  lse stays contiguous
 * [B, Hq, M].  Strides must be non-negative multiples of 8 elements (every row 16-byte aligned);
 * zero strides may broadcast q, k or v, but o's rows must not overlap each other or q, k, v.
 * K and V row strides are at most 17 043 456 elements.  Results are bitwise those of fa_fwd on
 * the same values stored contiguously.  Errors as fa_fwd (FA_ERR_INVALID_ARG for a negative
 * stride or offsets past int64, FA_ERR_UNSUPPORTED for a stride not a multiple of 8 or a K/V row
 * stride over the limit).
 */
int fa_fwd_strided(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int M,
                   int N, int D, const fa_strides *q_strides, const fa_strides *k_strides,
                   const fa_strides *v_strides, const fa_strides *o_strides, float scale, int causal, int dtype,
                   void *stream);

/*
 * fa_bwd -- backward pass: gradients of O with respect to q, k and v on one GPU.
 *
 * Not on the pages (they treat the forward only); the chain rule of the definition above, with
 * P recomputed from the forward's lse and the softmax Jacobian's row term taken as
 * Delta_i = dO_i . O_i (equal to sum_j P_ij dP_ij):
 *     dv_j  = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . v_j - Delta_i),
 *     dq_i  = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
 * where dk and dv of a KV head sum over the Hq / Hkv query heads that read it.  lse is not
 * differentiated.
 *
 * Arguments (contiguous row-major DEVICE tensors owned by the caller, dtype as for fa_fwd):
 *   q, k, v       the forward's inputs
 *   o, lse        the forward's outputs (fa_fwd's O and lse for the same q, k, v, scale, causal)
 *   dout          [B, Hq, M, D] upstream gradient of O
 *   dq            [B, Hq, M, D] written;  dk, dv [B, Hkv, N, D] written (rounded to dtype)
 *   workspace     at least fa_bwd_workspace_size(B, Hq, M) bytes of device memory, 16-byte
 *                 aligned; overwritten (per-row Delta and lse statistics)
 * Every pointer 16-byte aligned; outputs must not alias inputs.  Enqueues three kernels on
 * `stream` and returns without synchronising; allocates nothing.  Rows that see no key get
 * dq = 0; keys no row sees get dk = dv = 0.  Deterministic (no atomics).  Errors as fa_fwd,
 * plus FA_ERR_INVALID_ARG for a missing or too small workspace.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int M);
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse, void *dq,
           void *dk, void *dv, int B, int Hq, int Hkv, int M, int N, int D, float scale, int causal, int dtype,
           void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable text for a return code (static storage; never NULL). */
const char *fa_strerror(int code);

/*
 * Key-split forward, for grids too small to fill the GPU (few heads or query tiles, decode-like M).
 *
 * The key tiles a 128-row query tile visits are divided into even shares of at most
 * `tiles_per_split` tiles, one workgroup per share.  Each share's workgroup runs the same online
 * softmax over its keys and leaves its normalised partial output O_s and natural-log partial
 * lse_s in the workspace; a merge kernel then forms, per row,
 *     lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s,
 * which is the online-softmax combination step of "从零开始写Qwen3" (FlashAttention derivation
 * article), section "在线softmax", applied to two or more disjoint key sets at once: the result
 * equals fa_fwd's up to fp32 rounding order.  A share whose keys a row cannot see has
 * lse_s = -inf and weight 0.  Query tiles with a single share write O and lse directly.
 * Choosing the share count from the grid size follows the small-grid rule of
 * "lab3：GDN Prefill 前向优化", sections "TMA, DV 分块" and "GVA 感知的 block_DV" (a finer
 * work split only when the plain grid leaves CUs idle).
 *
 * fa_splitkv_plan: host-only.  tiles_per_split > 0 is used as given; <= 0 asks for the automatic
 *   choice (no split when the 4-wave grid already has 512 workgroups or no query tile visits 32
 *   key tiles, else shares of the key-tile work spread over about 512 workgroups, at least 8
 *   tiles each, and at least a quarter of the rows a share's partial output holds as long as
 *   the grid keeps 256 workgroups).  Writes the key tiles per share
 *   actually used (*tiles_used), the workgroup count of the split kernel (*workgroups) and the
 *   workspace size in bytes (*workspace_bytes; 0 when no query tile is split).  Returns FA_OK,
 *   FA_ERR_INVALID_ARG (null pointer, non-positive size, Hq % Hkv != 0) or FA_ERR_UNSUPPORTED
 *   (D not 64 or 128, more than 128 query tiles per head, i.e. M > 16384, or split query tiles
 *   whose merge would need more than 2^31 - 1 rows per query-tile rank, i.e. B * Hq * min(128, M)
 *   beyond that when the query heads are not stacked).
 *
 * fa_fwd_splitkv: arguments, layouts, determinism and error codes as fa_fwd, plus
 *   tiles_per_split   as for fa_splitkv_plan (the plan is recomputed from the same arguments)
 *   workspace         DEVICE memory owned by the caller, 256-byte aligned, at least the size
 *                     fa_splitkv_plan reports (may be NULL when that size is 0); overwritten
 *   workspace_bytes   its size
 * Enqueues the split kernel and, when some query tile is split, the merge kernel, both on
 * `stream`; returns without synchronising.  The workspace must not be used by another call
 * until the merge has run (calls on one stream are ordered).  Returns FA_ERR_INVALID_ARG also
 * for a missing or too small workspace, FA_ERR_UNSUPPORTED also for a workspace not 256-byte
 * aligned or M > 16384.
 */
int fa_splitkv_plan(int B, int Hq, int Hkv, int M, int N, int D, int causal, int tiles_per_split, int *tiles_used,
                    long long *workgroups, size_t *workspace_bytes);
int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int M,
                   int N, int D, float scale, int causal, int dtype, int tiles_per_split, void *workspace,
                   size_t workspace_bytes, void *stream);
/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same arguments,
 * layouts, plan, kernels, results (bit for bit) and error codes as fa_fwd_splitkv, without the
 * workspace: the partial results go to a scratch array of FA_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds in device memory, one per GPU, from the first call on that GPU until the process
 * ends.  The call allocates nothing and frees nothing (no hipMalloc, no allocating library
 * routine); the first call on a device looks up that device's scratch address.  The stream must
 * belong to the current device (NULL: the current device's default stream); otherwise the call
 * returns FA_ERR_INVALID_ARG without launching.
 * Returns FA_ERR_SCRATCH_TOO_SMALL, before touching the GPU, when the plan's workspace (the size
 * fa_splitkv_plan reports for the same arguments) exceeds FA_NOALLOC_SCRATCH_BYTES; plans that use
 * no workspace never touch the scratch.
 * All calls on one GPU share its scratch, which keeps the last call's contents (nothing in it needs
 * to start at zero): two calls whose kernels may overlap on one GPU -- on different streams, or
 * from different host threads without ordering -- race on it and give wrong results.  Calls on
 * one stream are ordered and safe.
 */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)
int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv,
                           int M, int N, int D, float scale, int causal, int dtype, int tiles_per_split,
                           void *stream);
/* fa_fwd_splitkv on strided tensors (strides as for fa_fwd_strided; NULL = contiguous). */
int fa_fwd_splitkv_strided(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv,
                           int M, int N, int D, const fa_strides *q_strides, const fa_strides *k_strides,
                           const fa_strides *v_strides, const fa_strides *o_strides, float scale, int causal,
                           int dtype, int tiles_per_split, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Introspection of the launch plan (host-only, no GPU needed).  These report the tiling
 * fa_fwd uses, so that tests can check the tile classification against the pages' worked
 * counts and benchmarks can count the work actually issued.
 *
 * fa_tile_shape: the query-tile and key-tile heights fa_fwd uses for a problem with B batches,
 *   Hq query heads, M queries per head and head dimension D (query tiles of 256 rows when
 *   D = 128 and the grid still fills the GPU, 128 rows otherwise; key tiles of 64 rows).
 *   Returns FA_OK,
 *   FA_ERR_INVALID_ARG for a null pointer or non-positive size, FA_ERR_UNSUPPORTED for an
 *   unsupported D.
 *
 * fa_tile_counts: for one (b, h), with query tiles of BM rows and key tiles of BN rows,
 *   counts the key tiles visited without a mask (*full), with a mask (*masked: the
 *   diagonal band of the causal mask and a ragged last key tile), and skipped (*skipped:
 *   tiles that no row of the query tile can see, never loaded).
 *   Follows "从零开始写Qwen3" (FlashAttention speed-up article), sections "改进2-KV只读取下三角"
 *   and "改进3-两阶段计算".  Returns FA_OK or FA_ERR_INVALID_ARG.
 *
 * fa_schedule: the (b, h, query-tile) that workgroup `wg` of fa_fwd's grid computes,
 *   for a launch of B * Hq * ceil(M / BM) workgroups (BM as fa_tile_shape reports).  Returns
 *   FA_OK or FA_ERR_INVALID_ARG.
 */
int fa_tile_shape(int B, int Hq, int M, int D, int *BM, int *BN);
int fa_tile_counts(int M, int N, int BM, int BN, int causal, long long *full, long long *masked,
                   long long *skipped);
int fa_schedule(int B, int Hq, int Hkv, int M, int D, int causal, long long wg, int *b, int *h, int *q_tile);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
