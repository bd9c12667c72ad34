/*
 * gdn.h -- C ABI of the Gated DeltaNet chunked prefill in libfa.so (MI355X, gfx950).
 *
 * Source: the page "lab3：GDN Prefill 前向优化", section "算法与数据依赖": chunks of 64 tokens,
 * head dim 128, the framework-side inputs g (the gate's cumulative log inside each chunk) and
 * A (the "KKT" triangular-solve result), and the chunk recurrence, per value head h reading
 * query/key head h / (Hv / Hqk) (the page's GVA mapping):
 *     U' = K S_c;  W' = beta (V - exp(g) U');  V_new = A W';
 *     O  = scale (exp(g) (Q S_c) + scores V_new),  scores_ts = (q_t . k_s) exp(g_t - g_s) for s <= t;
 *     S_{c+1} = exp(g_last) S_c + (K exp(g_last - g))^T V_new.
 * Reading taken (the page names A but does not print it): A = (I + L)^-1 per chunk with
 * L_ts = beta_t (k_t . k_s) exp(g_t - g_s) for s < t and 0 otherwise -- beta and the gate decay
 * folded in, as the page's note on its rejected FlashQLA port says its inputs have -- which makes
 * the chunk recurrence equal to the token-by-token gated delta rule
 *     S <- a_t S;  u_t = beta_t (v_t - S^T k_t);  S <- S + k_t u_t^T;  o_t = scale S^T q_t,
 * with a_t = exp(g_t - g_{t-1}) inside a chunk (g_{-1} = 0 at a chunk start).
 *
 * Layouts (contiguous, DEVICE memory owned by the caller):
 *   q, k   [B, T, Hqk, DK]  fp16 or bf16 (dtype as in fa.h)     DK must be 128
 *   v      [B, T, Hv, DV]   same dtype                            DV a multiple of 64
 *   g      [B, T, Hv]  fp32: cumulative log-gate inside each chunk [64 c, 64 c + 64) (T need not
 *          be a multiple of 64: the last chunk is shorter)
 *   beta   [B, T, Hv]  fp32
 *   A      [B, T, Hv, 64]  dtype: row t holds row (t mod 64) of its chunk's 64 x 64 matrix; columns
 *          past the chunk's end are ignored
 *   s0     [B, Hv, DK, DV] fp32 initial state, or NULL for zeros
 *   o      [B, T, Hv, DV]  dtype, written;  s_final [B, Hv, DK, DV] fp32, written
 * All pointers 16-byte aligned.  Hv must be a multiple of Hqk.
 *
 * gdn_kkt: computes A from k, g, beta (K K^T in fp32 on MFMA, the inverse by forward
 *   substitution in fp32, rounded to dtype once).  One kernel on `stream`.
 * gdn_chunk_fwd: the chunk recurrence.  Operands of the products are rounded to dtype (the
 *   state's operand copy included); accumulation and the state itself are fp32.  Two modes,
 *   with bit-identical results:
 *   - workspace == NULL: one kernel, one workgroup per (b, value head, 64 state columns)
 *     walking the chunks in order and forming each chunk's output on the way;
 *   - workspace != NULL: the page's own split of the work into a sequential state path and an
 *     output path that only reads the state, taken further: one kernel walks the chunks doing
 *     only U', W', V_new and the state update, storing each chunk's starting state and V_new
 *     (dtype) in the workspace; a second kernel then forms all chunks' outputs in parallel.
 *     `workspace` is DEVICE memory owned by the caller, 256-byte aligned, at least
 *     gdn_chunk_workspace_size(B, T, Hv, DV) bytes (`workspace_bytes` its size), and must not
 *     be in use by another call at the same time; its contents on entry do not matter.
 *   gdn_chunk_workspace_size returns that size (0 for a non-positive argument).
 * gdn_chunk_plan: the sequential mode this library would pick for the shape: *workspace_bytes =
 *   the workspace size when the two-kernel mode is expected to be faster (its state walk then
 *   occupies at most a quarter of the 256 CUs), else 0 (one kernel).  FA_ERR_INVALID_ARG for a null
 *   pointer or a non-positive size, FA_ERR_UNSUPPORTED for DV not a multiple of 64.
 * gdn_chunk_fwd_segmented: the same recurrence with the chunks cut into runs that are walked in
 *   parallel.  The recurrence is affine in the state, S_end = M S_start + Z for a run (M the run's
 *   linear map of the state, Z its end state from zero), and each state column evolves on its own.
 *   Three kernels on `stream`: (1) every run but the last is walked from [I | 0] with its values
 *   seen only by the last DV columns, giving [M | Z] (fp32; the same operand rounding as the
 *   sequential walk); (2) the runs' start states S_{r+1} = M_r S_r + Z_r, S_0 = s0, in fp32;
 *   (3) every run is walked again from its start state as in the one-kernel mode, forming the
 *   outputs, the last run writing s_final.  `segments` >= 1 asks for that many runs: runs of
 *   ceil(chunks / segments) chunks (at most one run per chunk, none empty).  The result equals the
 *   sequential modes' up to rounding (the products are re-associated), not bit for bit, and is
 *   deterministic.  One run (segments == 1, or a one-chunk sequence) runs the one-kernel mode,
 *   with its bits, and needs no workspace.  Otherwise `workspace` is caller-owned DEVICE memory,
 *   256-byte aligned, at least gdn_segmented_workspace_size(B, T, Hv, DV, segments) bytes (M,
 *   then Z, then the start states: 4 * 128 * (128 + 2 DV) bytes per (b, value head) and run but
 *   one, each part rounded up to 256 bytes), not in use by another call at the same time; its
 *   contents on entry do not matter.  FA_ERR_INVALID_ARG also for segments <= 0 or a missing or
 *   too small workspace, FA_ERR_UNSUPPORTED for a misaligned one.
 *   gdn_segmented_workspace_size returns that size (0 for one run or a non-positive argument).
 * gdn_segment_plan: *segments = the run count this library would pick for the shape, or 1 when it
 *   picks a sequential mode (gdn_chunk_plan) instead: only for grids of at most 128 state walkers
 *   (B * Hv * DV / 64), from a cost model of the three kernels.  Errors as gdn_chunk_plan.
 * gdn_kkt, gdn_chunk_fwd and gdn_chunk_fwd_segmented validate every argument before any HIP call
 * (FA_ERR_INVALID_ARG: null pointer, bad size, Hv % Hqk, scale not finite or <= 0, unknown dtype,
 * a workspace smaller than needed; FA_ERR_UNSUPPORTED: DK != 128, DV not a multiple of 64, misaligned pointer or workspace,
 * strides beyond 32-bit tile offsets, a grid beyond 2^31 - 1 workgroups), return FA_ERR_LAUNCH if
 * the launch fails, allocate nothing and do not synchronise.  Deterministic.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int gdn_kkt(const void *k, const float *g, const float *beta, void *A, int B, int T, int Hqk, int Hv, int DK,
            int dtype, void *stream);
size_t gdn_chunk_workspace_size(int B, int T, int Hv, int DV);
int gdn_chunk_plan(int B, int T, int Hv, int DV, size_t *workspace_bytes);
int gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta, const void *A,
                  const float *s0, void *o, float *s_final, int B, int T, int Hqk, int Hv, int DK, int DV, float scale,
                  int dtype, void *workspace, size_t workspace_bytes, void *stream);
size_t gdn_segmented_workspace_size(int B, int T, int Hv, int DV, int segments);
int gdn_segment_plan(int B, int T, int Hv, int DV, int *segments);
int gdn_chunk_fwd_segmented(const void *q, const void *k, const void *v, const float *g, const float *beta,
                            const void *A, const float *s0, void *o, float *s_final, int B, int T, int Hqk, int Hv,
                            int DK, int DV, float scale, int dtype, int segments, void *workspace,
                            size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
