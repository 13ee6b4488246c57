/*
 * hstu.h -- C ABI of the HSTU pointwise aggregated attention / layer forward
 * library for AMD MI355X (gfx950).
 *
 * What is computed (page title, section):
 *  - "Actions Speak Louder than Words" reading notes, §3.1 eqs. (1)-(3):
 *      U, V, Q, K = Split(SiLU(f1(X)))                                  (1)
 *      A V        = SiLU(Q K^T + rab^{p,t}) V   (no softmax, §3.2)      (2)
 *      Y          = f2(LayerNorm(A V) * U)                              (3)
 *    with f1, f2 single linear layers W x + b, and layers stacked with
 *    residual connections.
 *  - "4.4 推荐模型的 Scaling", section "HSTU 层" and its toy layer: chunk order
 *    U, V, Q, K; head h owns columns [h d, (h+1) d) of each chunk; causal mask
 *    j <= i including the diagonal; an optional normalising constant.
 *  - rab^{p,t}: bias from the relative position and the timestamp difference
 *    (§3.1 of the first page).  Bucketed form used here:
 *      rab(i, j) = w_pos[min(i - j, P - 1)] + w_time[min(floor(log2(1 + max(t_i - t_j, 0))), NT - 1)]
 *  - GenRank article (joto.ai), part (2): ALiBi in place of the learned bias,
 *      rab(i, j) = -slope_h * (i - j).
 *
 * The attention computes, for every user b, head h and local row i < n_b,
 *      O[i] = out_scale * sum_{j <= i} SiLU(alpha * <q_i, k_j> + rab_h(i, j)) * v_j .
 *
 * Conventions shared by all entry points:
 *  - Every pointer argument named as "device" must be a device allocation on
 *    the current HIP device; the caller owns all memory.  The library never
 *    allocates, frees or synchronises: every call only enqueues kernels on
 *    `stream` and returns.
 *  - Jagged batches: `offsets` is a device int32 array [B + 1], offsets[0] = 0,
 *    non-decreasing, offsets[B] = total_tokens; user b owns tokens
 *    [offsets[b], offsets[b+1]).  Empty users are allowed.  Every user length
 *    must be <= max_seqlen (the scheduler sizes its work list from it).
 *  - Row strides are in elements and must keep every row 16-byte aligned.
 *  - Errors detectable on the host return a negative hstu_status and enqueue
 *    nothing; a failed launch returns HSTU_ERR_HIP.  A thread-local message is
 *    available from hstu_last_error().  Device-side contract violations
 *    (non-monotone offsets, lengths above max_seqlen) are not checked by the
 *    fast path; hstu_validate_offsets() detects them.
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = -1,
  HSTU_ERR_UNSUPPORTED = -2,
  HSTU_ERR_WORKSPACE = -3,
  HSTU_ERR_HIP = -4
} hstu_status;

/* HSTU_DTYPE_BF16_OUT_F32: bf16 q, k, v with the attention output written in fp32 (before its
 * bf16 rounding); accepted by the attention entry points, which otherwise treat it as BF16. */
typedef enum { HSTU_DTYPE_F32 = 0, HSTU_DTYPE_BF16 = 1, HSTU_DTYPE_BF16_OUT_F32 = 2 } hstu_dtype;

typedef enum { HSTU_BIAS_NONE = 0, HSTU_BIAS_RAB_PT = 1, HSTU_BIAS_ALIBI = 2 } hstu_bias_kind;

/* Relative attention bias.  Host struct; the arrays it points to are device memory.
 *  RAB_PT: timestamps [T] int64 (any unit; only differences are used; may be NULL when T = 0);
 *          w_pos [H_tab][pos_head_stride] and w_time [H_tab][time_head_stride] fp32,
 *          with num_pos_buckets in [1, 1024] and num_time_buckets in [1, 64];
 *          a head stride of 0 shares one table across heads.
 *  ALIBI:  alibi_slopes [H] fp32, or NULL for slope_h = 2^(-8 (h+1) / H).
 *  NONE:   rab = 0. */
typedef struct {
  int32_t kind;
  const int64_t* timestamps;
  const float* w_pos;
  const float* w_time;
  int32_t num_pos_buckets;
  int32_t num_time_buckets;
  int32_t pos_head_stride;
  int32_t time_head_stride;
  const float* alibi_slopes;
} hstu_bias;

/* Bytes of device workspace hstu_attn_fwd needs for B users, H heads, lengths up to
 * max_seqlen and total_tokens tokens (work list of the jagged scheduler, per-token
 * timestamp statistics and tile classes of the relative bias, and the bf16 path's
 * per (32-key block, head) key norm bounds). */
size_t hstu_attn_workspace_bytes(int32_t B, int32_t H, int32_t max_seqlen, int64_t total_tokens);

/* Jagged causal pointwise attention, eq. (2) above.
 *  dt          HSTU_DTYPE_BF16 (bf16 in/out, fp32 accumulation), HSTU_DTYPE_BF16_OUT_F32
 *              (bf16 in, fp32 out) or HSTU_DTYPE_F32.
 *  B, H        users and heads; d_qk == d_v in {32, 64} (BF16_OUT_F32 included).
 *  offsets     device int32 [B+1]; max_seqlen >= every user length, <= 65536.
 *  q, k, v     device [T, H, d] rows with row strides q_row_stride etc.
 *              (elements between consecutive tokens; >= H*d).
 *  bias        host pointer to the bias description (may be NULL = NONE).
 *  alpha       multiplies Q K^T inside the SiLU; out_scale multiplies the sum.
 *  o           device [T, H, d_v] contiguous output (fp32 for BF16_OUT_F32).
 *  workspace   device, >= hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens),
 *              256-B aligned.
 * Layout of the workspace after the call: int32 item_count at byte 0, then
 * from byte 256 the scheduler's work list, one 32-byte entry per item
 * {int32 b, h, q_tile, n_b (the user's length); int64 first token of user b;
 * int64 0}, in launch order (cost = q_tile + 1 descending, then b, h ascending);
 * after it (256-aligned) per-token timestamp statistics of the bias, the tile
 * classes and the key norm bounds. */
hstu_status hstu_attn_fwd(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                          const int32_t* offsets, int32_t max_seqlen, int64_t total_tokens,
                          const void* q, int64_t q_row_stride, const void* k,
                          int64_t k_row_stride, const void* v, int64_t v_row_stride,
                          const hstu_bias* bias, float alpha, float out_scale, void* o,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* hstu_attn_fwd for callers that cannot allocate or pass device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation with
 * the same arguments minus the workspace, which is instead a 32 MiB static device array that
 * the library holds on each device it runs on until the process ends.  Batches whose
 * hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens) exceeds 32 MiB are rejected with
 * HSTU_ERR_UNSUPPORTED before anything is enqueued.  Allocates nothing (no hipMalloc, no
 * library allocation); the first call on a device looks up that device's array address.
 * Every call on one device uses the same array, so calls that overlap on one device (two
 * streams, two host threads) race; calls on one stream are ordered and safe. */
hstu_status hstu_attn_fwd_noalloc(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                  const int32_t* offsets, int32_t max_seqlen,
                                  int64_t total_tokens, const void* q, int64_t q_row_stride,
                                  const void* k, int64_t k_row_stride, const void* v,
                                  int64_t v_row_stride, const hstu_bias* bias, float alpha,
                                  float out_scale, void* o, hipStream_t stream);

/* The two halves of hstu_attn_fwd, for callers that run several attentions over one
 * jagged batch (a layer stack) or time the kernels apart.
 * hstu_attn_plan runs the jagged scheduler only: it writes the work list for
 * (dt, B, H, d, offsets, max_seqlen) into `workspace` (layout as above).
 * hstu_attn_fwd_planned runs the attention only, on a workspace that a completed
 * or earlier-enqueued hstu_attn_plan call with the same dt, B, H, d, offsets and
 * max_seqlen filled (it rewrites only the regions after the work list: timestamp
 * statistics, tile classes, key norm bounds); all other arguments as for hstu_attn_fwd. */
hstu_status hstu_attn_plan(int32_t dt, int32_t B, int32_t H, int32_t d, const int32_t* offsets,
                           int32_t max_seqlen, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);
hstu_status hstu_attn_fwd_planned(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                  const int32_t* offsets, int32_t max_seqlen,
                                  int64_t total_tokens, const void* q, int64_t q_row_stride,
                                  const void* k, int64_t k_row_stride, const void* v,
                                  int64_t v_row_stride, const hstu_bias* bias, float alpha,
                                  float out_scale, void* o, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* hstu_attn_fwd_planned in two parts, for callers that time or schedule them apart.
 * hstu_attn_prepare enqueues only the per-batch prepasses the bf16 kernel reads: key norm
 * bounds (max |k|^2 per 32-key block and head) and, for the position + time bias, the
 * per-block timestamp statistics and the tile classes; it reads k (rows as for
 * hstu_attn_fwd), offsets, the bias timestamps and nothing else, writes only the workspace
 * regions after the work list, and is a no-op for HSTU_DTYPE_F32.
 * hstu_attn_fwd_prepared enqueues only the attention kernel, on a workspace that
 * hstu_attn_plan and then hstu_attn_prepare (same dt, B, H, d, offsets, max_seqlen,
 * total_tokens, k and bias) filled; arguments as for hstu_attn_fwd_planned, whose result it
 * reproduces bit for bit.  Errors as for hstu_attn_fwd; neither call allocates. */
hstu_status hstu_attn_prepare(int32_t dt, int32_t B, int32_t H, int32_t d,
                              const int32_t* offsets, int32_t max_seqlen, int64_t total_tokens,
                              const void* k, int64_t k_row_stride, const hstu_bias* bias,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
hstu_status hstu_attn_fwd_prepared(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                   const int32_t* offsets, int32_t max_seqlen,
                                   int64_t total_tokens, const void* q, int64_t q_row_stride,
                                   const void* k, int64_t k_row_stride, const void* v,
                                   int64_t v_row_stride, const hstu_bias* bias, float alpha,
                                   float out_scale, void* o, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Query rows per work item (q_tile granularity) of the attention kernel for a dtype/d. */
int32_t hstu_attn_block_rows(int32_t dt, int32_t d);

/* Bytes of device workspace hstu_layer_fwd needs. */
size_t hstu_layer_workspace_bytes(int32_t B, int64_t total_tokens, int32_t d_model, int32_t H,
                                  int32_t d_qk, int32_t d_v, int32_t max_seqlen);

/* Gradients of the attention ("Actions Speak Louder than Words" reading notes §3.1 eq. (2),
 * §3.2) for an upstream gradient dO of O:
 *   dV_j = out_scale sum_{i >= j} SiLU(x_ij) dO_i,   g_ij = <dO_i, v_j> SiLU'(x_ij),
 *   dQ_i = alpha out_scale sum_{j <= i} g_ij k_j,    dK_j = alpha out_scale sum_{i >= j} g_ij q_i,
 *   dw_pos[pos bucket(i, j)] += out_scale g_ij,  dw_time[time bucket(i, j)] += out_scale g_ij
 * with x_ij = alpha <q_i, k_j> + rab(i, j) and SiLU'(x) = s (1 + x (1 - s)), s = 1/(1+e^-x).
 *  dt        HSTU_DTYPE_BF16 only; d_qk = d_v = 64
 *  q, k, v, d_o  device bf16 rows [T, H, 64] with the given row strides (as for hstu_attn_fwd)
 *  dq, dk, dv    device bf16 [T, H, 64] contiguous, overwritten
 *  dw_pos, dw_time  rab_pt bias only (else may be NULL): device fp32 shaped like w_pos / w_time
 *            (H x head stride, or one table when the stride is 0: then it sums over heads),
 *            overwritten (zeros for an empty batch: B, T or max_seqlen 0); added to with
 *            atomics, so their last bits vary between runs
 *  workspace as for hstu_attn_fwd (same size); other arguments as for hstu_attn_fwd. */
hstu_status hstu_attn_bwd(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                          const int32_t* offsets, int32_t max_seqlen, int64_t total_tokens,
                          const void* q, int64_t q_row_stride, const void* k,
                          int64_t k_row_stride, const void* v, int64_t v_row_stride,
                          const void* d_o, int64_t do_row_stride, const hstu_bias* bias,
                          float alpha, float out_scale, void* dq, void* dk, void* dv,
                          float* dw_pos, float* dw_time, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* One HSTU layer forward, eqs. (1)-(3), bf16 storage with fp32 accumulation.
 *  x        device bf16 [T, d_model]
 *  w1       device bf16 [2H(d_qk+d_v), d_model] (row n = output feature n), b1 fp32 [2H(d_qk+d_v)] or NULL
 *  ln_gamma, ln_beta  device fp32 [H d_v] (NULL = 1 / 0), ln_eps > 0
 *  w2       device bf16 [d_model, H d_v], b2 fp32 [d_model] or NULL
 *  residual nonzero: y = x + f2(...)
 *  y        device bf16 [T, d_model]; may not alias x.
 *  The workspace holds Z = SiLU(x W1^T + b1) as bf16 [T, 2H(d_qk+d_v)] (column blocks
 *  U | V | Q | K) at byte 0, then the attention output O as bf16 [T, H d_v] stored relative to
 *  a per (token, head) offset m (O[t, h, :] = m + stored value), then per (token, head) four
 *  fp32 values {m, mean of the head's d_v values of O, their sum of squared deviations, 0}
 *  (the LayerNorm statistics are combined from these), then the attention workspace; offsets
 *  of each are returned by hstu_layer_workspace_offsets(). */
hstu_status hstu_layer_fwd(int32_t dt, int32_t B, int32_t d_model, int32_t H, int32_t d_qk,
                           int32_t d_v, const int32_t* offsets, int32_t max_seqlen,
                           int64_t total_tokens, const void* x, const void* w1, const float* b1,
                           const float* ln_gamma, const float* ln_beta, float ln_eps,
                           const void* w2, const float* b2, const hstu_bias* bias, float alpha,
                           int32_t residual, void* y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* A stack of n_layers HSTU layers (each as hstu_layer_fwd, layer l + 1 taking layer l's y as
 * its x), the single-operator form of the reading notes' §3.5 available between layers: with
 * fuse_boundaries nonzero, layer l's LayerNorm, gate, f2 (and residual) and layer l + 1's
 * f1 + SiLU + split run as one kernel per 64-token tile, the tile's y kept on chip between the
 * two products (d_model = 512 only; otherwise HSTU_ERR_UNSUPPORTED).  Both forms give identical
 * bits: the fused kernel takes f1's products in f1's order.  The attention stays a kernel of its
 * own (it needs every key of a user).  The jagged work list is made once per call, and the
 * attention's tile classes once per distinct (timestamps, bucket counts) of the layers'
 * position + time biases; the output equals hstu_layer_fwd applied layer by layer.
 *  w1, b1, ln_gamma, ln_beta, w2, b2, bias  host arrays of n_layers per-layer arguments, each
 *            as for hstu_layer_fwd (device pointers; NULL entries allowed where hstu_layer_fwd
 *            allows them)
 *  x, y      device bf16 [T, d_model]; y may not alias x
 *  workspace >= hstu_stack_workspace_bytes(...), 256-byte aligned: the layer workspace, then two
 *            bf16 [T, d_model] buffers for the layers in between.
 *  Errors as for hstu_layer_fwd; n_layers >= 1. */
size_t hstu_stack_workspace_bytes(int32_t B, int64_t total_tokens, int32_t d_model, int32_t H,
                                  int32_t d_qk, int32_t d_v, int32_t max_seqlen);
hstu_status hstu_stack_fwd(int32_t dt, int32_t B, int32_t n_layers, int32_t d_model, int32_t H,
                           int32_t d_qk, int32_t d_v, const int32_t* offsets, int32_t max_seqlen,
                           int64_t total_tokens, const void* x, const void* const* w1,
                           const float* const* b1, const float* const* ln_gamma,
                           const float* const* ln_beta, float ln_eps, const void* const* w2,
                           const float* const* b2, const hstu_bias* const* bias, float alpha,
                           int32_t residual, int32_t fuse_boundaries, void* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Gradients of one HSTU layer ("Actions Speak Louder than Words" reading notes §3.1 eqs. (1)-(3))
 * for an upstream gradient dY, after hstu_layer_fwd on the same inputs: fwd_workspace is that
 * call's workspace, whose Z and O it reads (Zpre = X W1^T + b1 is recomputed).  By the chain
 * rule through eq. (3) (dG = dY W2, dW2 = dY^T G, db2 = sum dY, the gate and LayerNorm),
 * eq. (2) (hstu_attn_bwd, out_scale 1) and eq. (1) (dZpre = dZ SiLU'(Zpre), dX = dZpre W1,
 * dW1 = dZpre^T X, db1 = sum dZpre), plus dY for the residual.
 *  dt HSTU_DTYPE_BF16; d_qk = d_v = 64; d_model % 32 == 0; H d_v <= 2048
 *  dy, dx    device bf16 [T, d_model]
 *  dw1 fp32 [2H(d_qk+d_v), d_model], db1 [2H(d_qk+d_v)], dgamma / dbeta [H d_v],
 *  dw2 fp32 [d_model, H d_v], db2 [d_model]; dw_pos / dw_time as for hstu_attn_bwd: all
 *            overwritten (sums over tokens, added with atomics: last bits vary between runs)
 *  workspace >= hstu_layer_bwd_workspace_bytes(...), 256-byte aligned. */
hstu_status hstu_layer_bwd(int32_t dt, int32_t B, int32_t d_model, int32_t H, int32_t d_qk,
                           int32_t d_v, const int32_t* offsets, int32_t max_seqlen,
                           int64_t total_tokens, const void* x, const void* w1, const float* b1,
                           const float* ln_gamma, const float* ln_beta, float ln_eps,
                           const void* w2, const hstu_bias* bias, float alpha, int32_t residual,
                           const void* fwd_workspace, const void* dy, void* dx, float* dw1,
                           float* db1, float* dgamma, float* dbeta, float* dw2, float* db2,
                           float* dw_pos, float* dw_time, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);
size_t hstu_layer_bwd_workspace_bytes(int32_t B, int64_t total_tokens, int32_t H, int32_t d_qk,
                                      int32_t d_v, int32_t max_seqlen);

/* Byte offsets of Z, O, the O statistics and the attention workspace inside the layer
 * workspace (any pointer may be NULL). */
void hstu_layer_workspace_offsets(int64_t total_tokens, int32_t H, int32_t d_qk, int32_t d_v,
                                  size_t* z_offset, size_t* o_offset, size_t* stats_offset,
                                  size_t* attn_offset);

/* Candidate scoring over a cached user history (M-FALCON, "Actions Speak Louder than Words"
 * reading notes §3.6; candidates of one request share one position, GenRank article part (2)).
 * User b has n_b history tokens (rows [hist_offsets[b], hist_offsets[b+1]) of k_hist, v_hist and
 * the bias timestamps) and m_b candidates (rows [cand_offsets[b], cand_offsets[b+1]) of q_cand,
 * k_cand, v_cand and cand_timestamps).  Every candidate c sits at position n_b and sees the
 * whole history and itself, no other candidate:
 *   O[c] = out_scale * ( sum_{j < n_b} SiLU(alpha <q_c, k_j> + rab(n_b - j, t_c - t_j)) v_j
 *                        + SiLU(alpha <q_c, k_c> + rab(0, 0)) v_c )
 * which is the row eq. (2) gives c appended alone after the history.  The history's K, V are
 * the cache: score candidates in micro-batches by calling once per batch.
 *  dt        HSTU_DTYPE_BF16 only; d_qk = d_v = 64
 *  hist_offsets, cand_offsets  device int32 [B + 1] (jagged, as for the attention); every
 *            n_b <= max_hist and m_b <= max_cand; total_hist = hist_offsets[B],
 *            total_cand = cand_offsets[B]
 *  q_cand, k_cand, v_cand  device bf16 [total_cand, H, 64] rows with the given strides
 *  k_hist, v_hist          device bf16 [total_hist, H, 64] rows with the given strides
 *  bias      as for hstu_attn_fwd; bias->timestamps are the history's [total_hist]
 *  cand_timestamps  device int64 [total_cand] (RAB_PT only, else may be NULL)
 *  o         device bf16 [total_cand, H, 64]
 *  workspace device, >= hstu_attn_candidates_workspace_bytes(B, H, max_hist, total_hist,
 *            total_cand) bytes, 256-byte aligned.  Histories longer than 1024 keys are scored
 *            in chunks of 1024 whose fp32 sums it holds; they are added in chunk order.  It
 *            also holds the list of (user, head, chunk) work units and per-32-key timestamp
 *            extremes of the history (position + time bias).  Contents need no initialisation
 *            and are scratch after the call; calls sharing a workspace must not overlap.
 * Errors as for hstu_attn_fwd. */
hstu_status hstu_attn_candidates_fwd(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                     const int32_t* hist_offsets, int32_t max_hist,
                                     int64_t total_hist, const int32_t* cand_offsets,
                                     int32_t max_cand, int64_t total_cand, const void* q_cand,
                                     int64_t q_stride,
                                     const void* k_cand, int64_t k_cand_stride,
                                     const void* v_cand, int64_t v_cand_stride,
                                     const void* k_hist, int64_t k_hist_stride,
                                     const void* v_hist, int64_t v_hist_stride,
                                     const hstu_bias* bias, const int64_t* cand_timestamps,
                                     float alpha, float out_scale, void* o, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace hstu_attn_candidates_fwd needs: each part rounded up to 256,
 * 4 x 64 x H x total_cand x ceil(max_hist / 1024) when max_hist > 1024 (else 0),
 * + 16 x total_hist + 4 x total_hist, + 256 + 4 x B x H x max(ceil(max_hist / 1024), 1). */
size_t hstu_attn_candidates_workspace_bytes(int32_t B, int32_t H, int32_t max_hist,
                                            int64_t total_hist, int64_t total_cand);

/* Stochastic Length ("Actions Speak Louder than Words" reading notes §3.3) of a jagged batch.
 * With L = floor(N_c^(alpha/2)): a user with n_b <= L events keeps them all; with n_b > L it is
 * subsampled to L events iff u_user[b] < 1 - N_c^alpha / n_b^2 (in double: probability
 * 1 - N_c^alpha / n_b^2 for uniform draws), else kept whole.  A subsampled user keeps the L
 * events with the smallest key_tok (ties by lower index) in their original order (a uniform
 * random subset for i.i.d. keys; keys must not be NaN).
 *  offsets   device int32 [B + 1]; lengths <= max_seqlen; total_tokens = offsets[B]
 *  N_c >= 1, 0 < alpha <= 2 (the pages use alpha in (1, 2]; 2 keeps every sequence)
 *  u_user    device float [B];  key_tok device float [total_tokens]
 *  x, row_bytes  optional rows [total_tokens][row_bytes] (row_bytes % 16 == 0) to gather into
 *            x_out; ts optional int64 [total_tokens] to gather into ts_out
 *  out_offsets  device int32 [B + 1]: the subsampled batch; out_offsets[B] <= total_tokens and
 *            every new length <= the old one, so input-sized outputs and max_seqlen bound it
 *  src_index device int32 [total_tokens]: the input token of each output token
 *  workspace >= hstu_stochastic_length_workspace_bytes(B, total_tokens), 256-byte aligned. */
hstu_status hstu_stochastic_length(int32_t B, const int32_t* offsets, int32_t max_seqlen,
                                   int64_t total_tokens, int32_t N_c, double alpha,
                                   const float* u_user, const float* key_tok, const void* x,
                                   int64_t row_bytes, const int64_t* ts, int32_t* out_offsets,
                                   int32_t* src_index, void* x_out, int64_t* ts_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t hstu_stochastic_length_workspace_bytes(int32_t B, int64_t total_tokens);

/* GenRank action-oriented tokens (GenRank article, part (1)): x[t] = item_table[item_ids[t]]
 * + action_table[action_ids[t]], bf16 in and out, fp32 add.  ids are device int32 [T];
 * an id outside [0, num_items) or [0, num_actions) contributes a zero row.  dim % 8 == 0. */
hstu_status hstu_embed_sum_fwd(int64_t total_tokens, int32_t dim, const void* item_table,
                               int64_t num_items, const void* action_table, int32_t num_actions,
                               const int32_t* item_ids, const int32_t* action_ids, void* x,
                               hipStream_t stream);

/* Checks a jagged offsets array on the device: writes int32 flags to device `flags_out`
 * (bit 0: offsets[0] != 0, bit 1: decreasing, bit 2: offsets[B] != total_tokens,
 * bit 3: a length above max_seqlen).  0 means valid. */
hstu_status hstu_validate_offsets(int32_t B, const int32_t* offsets, int64_t total_tokens,
                                  int32_t max_seqlen, int32_t* flags_out, hipStream_t stream);

/* Test hook: the bias bucket indices the attention kernel uses, for R (token_i, token_j)
 * pairs of the same user (local positions from `offsets`).  Writes device int32
 * pos_bucket[R], time_bucket[R]. */
hstu_status hstu_debug_buckets(int32_t B, const int32_t* offsets, const int64_t* timestamps,
                               int32_t num_pos_buckets, int32_t num_time_buckets, int64_t R,
                               const int64_t* token_i, const int64_t* token_j,
                               int32_t* pos_bucket, int32_t* time_bucket, hipStream_t stream);

const char* hstu_status_string(int32_t status);
const char* hstu_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HSTU_H_ */
