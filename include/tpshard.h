/*
 * tpshard.h — C ABI of libtpshard.so: one tensor-parallel rank's shard of a Megatron Transformer
 * layer on one AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources cited by page title and section):
 *  - The QKV ColumnParallelLinear split by head, then each rank's heads computed independently
 *    ("Megatron-LM 深度解读报告", table of §2.2, attention row; "Megatron-LM（英伟达超大模型训练框架）
 *    完整介绍", §二.2 张量并行).
 *  - The MLP: fc1 split by columns, fc2 split by rows, no synchronisation between them; the row-split
 *    output is a partial sum that an all-reduce would complete ("Megatron-LM — 架构与原理", §4 巧妙之处,
 *    the Column->Row pairing; same table of "Megatron-LM 深度解读报告" §2.2, MLP row).
 *  - The column split itself, Y = X·W with W = [W1 W2] computed as X·W1 and X·W2 on different devices
 *    ("Megatron-LM技术演进与大规模模型训练实践", §2.1).
 *  - Backward: copy is the identity forward and an all-reduce backward, reduce the reverse
 *    ("Megatron-LM — 架构与原理", §4): every rank receives the full dZ and returns a partial dX.
 * The pages leave the activation, the attention formula and the bias placement open; this library
 * takes: exact GeLU x·Φ(x); scores q·k/√d with a causal mask (key j visible to query i iff j <= i)
 * and a max-subtracted softmax; bqkv and b1 split with their columns; b2 added by rank 0 only.
 *
 * Conventions for every entry point:
 *  - Shard geometry: a rank owns cnt(n,t,r) = floor(n/t) + (r < n mod t) of n heads (or MLP
 *    columns), starting at off(n,t,r) = r*floor(n/t) + min(r, n mod t).  d = H / n_heads.
 *  - Layout: row-major, contiguous.  Activations [B, S, ·] flattened to token b*S + s (T = B*S rows).
 *    Weights [in, out], so Y = X·W.  QKV columns are head-interleaved: column h*3d + s*d + j holds
 *    part s (0 = q, 1 = k, 2 = v), element j, of local head h.  ctx column h*d + j is head h.
 *  - Pointers are device pointers (hipMalloc'd or torch CUDA storage), 16-byte aligned.  The caller
 *    owns every buffer; the library never allocates, frees or keeps a pointer after returning.
 *  - `dtype`: TP_BF16 (bf16 in/out, fp32 accumulation and fp32 softmax/GeLU) or TP_F32 (fp32
 *    throughout: the check mode).  Every output has that type except LSE and workspace, fp32.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is ordered on it; calls return
 *    without synchronising.  Outputs are overwritten (never accumulated into).  The calls
 *    with independent GEMMs (tp_mlp_shard_bwd, tp_qkv_shard_bwd, tp_attn_out_shard_bwd,
 *    tp_moe_shard_bwd; tp_mlp_grouped_shard_fwd and tp_moe_shard_fwd, which run the second half
 *    of the experts there) may
 *    run some of them on a library-owned side stream (one per caller stream and device, created on
 *    first use outside graph capture, default priority; for up to 64 such pairs, after which calls
 *    from further streams run serially on `stream`), forked from and joined back into `stream` with
 *    events before they return: to the caller the effect is the same as if everything ran on
 *    `stream`, independent caller streams stay independent, and a captured graph simply gets two
 *    branches.  While per-launch timing is on, or when the environment variable TP_SERIAL is
 *    set to a non-zero value, everything runs on `stream`.
 *  - Errors: arguments are validated on the host before any launch; a negative tp_status is
 *    returned and nothing is enqueued.  A failed launch returns TP_EHIP; tp_last_error() then holds
 *    the HIP message for the calling thread.  Faults inside kernels surface at the caller's next
 *    synchronisation.  Calls are thread-safe; calls that share output buffers on one stream order
 *    themselves by the stream.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TP_BF16 = 0, TP_F32 = 1 } tp_dtype;

/* The MLP's activation: the exact GeLU x·Φ(x), or its tanh form ½x(1 + tanh(√(2/π)(x + 0.044715x³))). */
typedef enum { TP_GELU = 0, TP_GELU_TANH = 1 } tp_activation;

typedef enum {
  TP_OK = 0,
  TP_EINVAL = -1,        /* a size, rank or dtype out of range, or a shape the split does not allow */
  TP_ENULL = -2,         /* a required pointer is NULL                                             */
  TP_EALIGN = -3,        /* a pointer is not 16-byte aligned                                       */
  TP_EUNSUPPORTED = -4,  /* valid request this build does not implement (e.g. head_dim > 128)      */
  TP_EWORKSPACE = -5,    /* workspace missing or smaller than tp_workspace_bytes() asks            */
  TP_EHIP = -6           /* a HIP call failed; see tp_last_error()                                 */
} tp_status;

/* A0 — shard geometry (host only, no device work).  The rank's [offset, offset+count) of n items:
 * balanced, lower ranks take the remainder (25 heads over 2 ranks: 13 then 12).  Returns TP_EINVAL
 * for n < 0, tp_size < 1 or rank outside [0, tp_size); TP_ENULL for NULL outputs. */
int tp_shard_range(int n, int tp_size, int rank, int* offset, int* count);

/* A1 — QKV ColumnParallelLinear of one rank, split by head, output not gathered.
 *   QKV_r[T, 3*nh_r*d] = X[T, H] · Wqkv_r[H, 3*nh_r*d] + bqkv_r[3*nh_r*d]
 * Wqkv_r / bqkv_r are the columns [3d*h0, 3d*(h0+nh_r)) of the full head-interleaved weight / bias.
 * Requires H % n_heads == 0, n_heads >= tp_size; bqkv_r may not be NULL. */
int tp_qkv_shard_fwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                     const void* X, const void* Wqkv_r, const void* bqkv_r, void* QKV_r,
                     void* stream);

/* A2 — causal softmax attention over the rank's nh_r heads, each independent.
 *   per (b, h): P = softmax_j(Q·Kᵀ/√d, key j visible to query i iff j <= i); ctx = P·V
 *   ctx_r[T, nh_r*d];  lse_r[B, nh_r, S] (fp32, nullable) = m_i + log Σ_j exp(score_ij - m_i).
 * Supports d in {16, 32, 64, 96, 128}. */
int tp_attn_heads_fwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                      const void* QKV_r, void* ctx_r, float* lse_r, void* stream);

/* A3 + A4 — MLP shard: fc1 column block with the bias and GeLU fused into its epilogue, then the
 * fc2 row block producing the partial sum Z_r that an all-reduce over ranks would complete.
 *   A1_r[T, F_r] = X·W1_r + b1_r ;  Y_r = GeLU(A1_r) = A1_r·Φ(A1_r)
 *   Z_r[T, H]    = Y_r·W2_r  (+ b2 iff rank == 0 and b2 != NULL)
 * W1_r[H, F_r], b1_r[F_r] are columns [f0, f0+F_r) of W1, b1; W2_r[F_r, H] rows [f0, f0+F_r) of W2.
 * Y_r is required (fc2 reads it); A1_r is nullable (not stored; the backward needs it). */
int tp_mlp_shard_fwd(int tp_size, int rank, int T, int H, int F, int dtype,
                     const void* X, const void* W1_r, const void* b1_r, const void* W2_r,
                     const void* b2, void* Z_r, void* A1_r, void* Y_r, void* stream);

/* A5 — MLP shard backward.  dZ[T, H] is the full upstream gradient (reduce's backward is the
 * identity), the same on every rank.
 *   dW2_r = Y_rᵀ·dZ ;  db2 = Σ_t dZ (iff rank == 0 and db2 != NULL)
 *   dA1   = (dZ·W2_rᵀ) ∘ GeLU'(A1_r),  GeLU'(x) = Φ(x) + x·φ(x)
 *   db1_r = Σ_t dA1 ;  dW1_r = Xᵀ·dA1 ;  dX_r = dA1·W1_rᵀ (a partial: Σ_r dX_r = dX)
 * workspace: device memory of at least tp_workspace_bytes("tp_mlp_shard_bwd", ...) bytes. */
int tp_mlp_shard_bwd(int tp_size, int rank, int T, int H, int F, int dtype,
                     const void* X, const void* W1_r, const void* W2_r, const void* A1_r,
                     const void* Y_r, const void* dZ, void* dX_r, void* dW1_r, void* db1_r,
                     void* dW2_r, void* db2, void* workspace, size_t workspace_bytes,
                     void* stream);

/* tp_mlp_shard_fwd and tp_mlp_shard_bwd with the activation chosen (TP_GELU, as the plain calls
 * use, or TP_GELU_TANH; its derivative in the backward).  TP_EINVAL for another value.  The tanh
 * form is GeLU's usual approximation; the pages name no activation, so it is an option beside the
 * exact form the library takes by default. */
int tp_mlp_shard_fwd_act(int tp_size, int rank, int T, int H, int F, int dtype,
                         const void* X, const void* W1_r, const void* b1_r, const void* W2_r,
                         const void* b2, void* Z_r, void* A1_r, void* Y_r, int activation, void* stream);
int tp_mlp_shard_bwd_act(int tp_size, int rank, int T, int H, int F, int dtype,
                         const void* X, const void* W1_r, const void* W2_r, const void* A1_r,
                         const void* Y_r, const void* dZ, void* dX_r, void* dW1_r, void* db1_r,
                         void* dW2_r, void* db2, void* workspace, size_t workspace_bytes, int activation,
                         void* stream);

/* A6 — QKV shard backward: dWqkv_r = Xᵀ·dQKV_r ; dbqkv_r = Σ_t dQKV_r ; dX_r = dQKV_r·Wqkv_rᵀ
 * (a partial).  workspace: tp_workspace_bytes("tp_qkv_shard_bwd", ...). */
int tp_qkv_shard_bwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                     const void* X, const void* Wqkv_r, const void* dQKV_r, void* dX_r,
                     void* dWqkv_r, void* dbqkv_r, void* workspace, size_t workspace_bytes,
                     void* stream);

/* tp_qkv_shard_bwd for callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and errors as tp_qkv_shard_bwd,
 * without the workspace: the bias gradient's column-sum partials (ceil(B*S/64) * 3*nh_r*d fp32
 * values) go to a scratch array inside the library, tp_qkv_shard_bwd_noalloc_max_scratch() bytes
 * (16 MiB) per device, held from the first call on a device until the process ends.  A shard whose
 * partials do not fit returns TP_EWORKSPACE before anything is enqueued.  The call allocates
 * nothing (no hipMalloc / hipFree, no stream or event; per-launch timing off) and runs every launch
 * on `stream`.  Every call on one device shares that device's scratch: calls that overlap on one
 * GPU (on different streams, or from different threads without ordering between them) race, so
 * order them.  The scratch needs no clearing between calls: each call writes every partial it
 * reads. */
int tp_qkv_shard_bwd_noalloc(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                             const void* X, const void* Wqkv_r, const void* dQKV_r, void* dX_r,
                             void* dWqkv_r, void* dbqkv_r, void* stream);
size_t tp_qkv_shard_bwd_noalloc_max_scratch(void);

/* A7 — attention backward over the rank's heads, P recomputed from Q, K and the saved LSE:
 *   D_i = Σ_c dO_ic·O_ic ; dV = Pᵀ·dO ; dP = dO·Vᵀ ; dS = P∘(dP − D) ; dQ = dS·K/√d ; dK = dSᵀ·Q/√d
 * ctx_r and lse_r must be this call's forward outputs for QKV_r.  dQKV_r has QKV_r's layout.
 * workspace: tp_workspace_bytes("tp_attn_heads_bwd", ...). Deterministic (no atomics). */
int tp_attn_heads_bwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                      const void* QKV_r, const void* ctx_r, const float* lse_r,
                      const void* dctx_r, void* dQKV_r, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Attention output projection, a RowParallelLinear over the rank's heads.  The pages have the
 * heads' outputs aggregated after each card's attention ("Megatron-LM（英伟达超大模型训练框架）完整介绍",
 * §二.2); the row-split linear layer and the column->row pairing that needs one all-reduce at its exit
 * are in "Megatron-LM — 架构与原理", §2.3 and §4.  The rank holds the d*nh_r rows of the full
 * Wo[H, H] that multiply its own heads' context columns, and produces a partial sum:
 *   O_r[T, H] = ctx_r[T, nh_r*d] · Wo_r[nh_r*d, H]  (+ bo[H] iff rank == 0 and bo != NULL)
 * so Σ_r O_r = ctx·Wo + bo.  Wo_r is rows [d*h0, d*(h0+nh_r)) of Wo; ctx_r is the output of
 * tp_attn_heads_fwd.  Same geometry checks as tp_qkv_shard_fwd. */
int tp_attn_out_shard_fwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                          const void* ctx_r, const void* Wo_r, const void* bo, void* O_r,
                          void* stream);

/* Backward of tp_attn_out_shard_fwd.  dO[T, H] is the full upstream gradient, the same on every
 * rank (the all-reduce's backward is the identity):
 *   dWo_r = ctx_rᵀ·dO ;  dbo = Σ_t dO (iff rank == 0 and dbo != NULL) ;  dctx_r = dO·Wo_rᵀ
 * dctx_r is the rank's own column block of dctx (no sum over ranks), ready for tp_attn_heads_bwd.
 * workspace: tp_workspace_bytes("tp_attn_out_shard_bwd", ...): the bias gradient's fp32 partials and,
 * in bf16 when dctx_r has few output tiles (the GPT-3 shard's [2048, 1536]), fp32 partials of dctx_r
 * over up to four slices of H, summed in slice order into dctx_r (deterministic). */
int tp_attn_out_shard_bwd(int tp_size, int rank, int B, int S, int H, int n_heads, int dtype,
                          const void* ctx_r, const void* Wo_r, const void* dO, void* dctx_r,
                          void* dWo_r, void* dbo, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Residual add with dropout, then LayerNorm: the ops outside the tensor split, which every rank
 * holds whole ("Megatron-LM 深度解读报告", §2.2 table, LayerNorm / Dropout row) or, under sequence
 * parallelism, splits along the sequence ("NVIDIA Megatron-LM：大规模Transformer模型分布式训练框架",
 * the five-strategies section; "Megatron-LM — 架构与原理", capability table).  Per row:
 *   h = x + o∘keep/(1 − p_drop)           (o nullable: h = x;  keep nullable: no dropout)
 *   y = (h − mean)·rstd·γ + β,  mean and the biased variance over the H features,
 *   rstd = 1/√(var + eps)
 * o is the sublayer's output after its all-reduce (bias included).  A pre-norm block carries h on
 * as its residual stream, a post-norm block y; the op is the same.  Rows: all T = B·S tokens when
 * sequence_parallel == 0; else the rank's block [off(T,t,r), off+cnt) of them (the sequence itself
 * when B = 1), and every pointer then addresses that block, [cnt, H].  keep: uint8 [rows, H],
 * non-zero = kept (the caller draws the mask).  h: required when o != NULL (nullable otherwise);
 * y, mean [rows], rstd [rows] (fp32) required.  In bf16 mode the statistics are those of h as
 * stored (rounded to bf16).  Requires 0 <= p_drop < 1, eps >= 0 (finite), H <= 24576
 * (TP_EUNSUPPORTED above). */
int tp_residual_ln_fwd(int tp_size, int rank, int sequence_parallel, int T, int H, int dtype,
                       const void* x, const void* o, const unsigned char* keep, float p_drop,
                       const void* gamma, const void* beta, float eps, void* h, void* y, float* mean,
                       float* rstd, void* stream);

/* Backward of tp_residual_ln_fwd on the same rows, with g = dy∘γ and x̂ = (h − mean)·rstd:
 *   dh = dh_in + rstd·(g − mean_H(g) − x̂·mean_H(g·x̂))   (dh_in nullable: the gradient reaching h
 *        along the residual stream; dh is also the gradient of x)
 *   d_o = dh∘keep/(1 − p_drop)                             (nullable)
 *   dγ = Σ_rows dy∘x̂ ;  dβ = Σ_rows dy                    (partials under sequence parallelism:
 *        Σ_r over ranks is the full gradient; deterministic)
 * mean and rstd are the forward's.  workspace: tp_workspace_bytes("tp_residual_ln_bwd", ...) (sized
 * for all T rows, so it also serves the sequence-parallel call). */
int tp_residual_ln_bwd(int tp_size, int rank, int sequence_parallel, int T, int H, int dtype,
                       const void* dy, const void* dh_in, const void* h, const float* mean,
                       const float* rstd, const void* gamma, const unsigned char* keep, float p_drop,
                       void* dh, void* d_o, void* dgamma, void* dbeta, void* workspace,
                       size_t workspace_bytes, void* stream);

/* A9 — grouped expert MLP shard (MoE experts as grouped GEMMs: "Megatron-LM — 架构与原理", §6, TE
 * GroupedLinear).  Rows [off[e], off[e+1]) of the expert-sorted token matrix X_perm[rows, H] belong to
 * expert e (e < n_groups); each goes through expert e's column shard of fc1 with bias and GeLU and
 * its row shard of fc2:
 *   A1_r[row] = X_perm[row]·W1_r[e] + b1_r[e] ;  Y_r[row] = GeLU(A1_r[row]) ;  Z_r[row] = Y_r[row]·W2_r[e]
 * W1_r [n_groups, H, F_r], b1_r [n_groups, F_r], W2_r [n_groups, F_r, H]; F_r = cnt(F_group, t, r).
 * group_offsets: n_groups+1 ints in device memory (the routing produced them there), expected
 * non-decreasing from 0; the library clamps each to [previous, rows] before use, so malformed offsets
 * cannot cause out-of-range accesses.  Rows outside [off[0], off[n_groups]) of Z_r, Y_r, A1_r are
 * left untouched.  No bias on the experts' fc2 partial.  Y_r required (fc2 reads it), A1_r nullable.
 * workspace: tp_workspace_bytes("tp_mlp_grouped_shard_fwd", ...) with n_heads = n_groups. */
int tp_mlp_grouped_shard_fwd(int tp_size, int rank, int n_groups, const int* group_offsets, int rows,
                             int H, int F_group, int dtype, const void* X_perm, const void* W1_r,
                             const void* b1_r, const void* W2_r, void* Z_r, void* A1_r, void* Y_r,
                             void* workspace, size_t workspace_bytes, void* stream);

/* MoE routing, the first of the four beats route -> dispatch (permute) -> experts -> combine
 * (unpermute) of "Megatron-LM — 架构与原理", §4, for one device's tokens.  logits: fp32 [tokens, E].
 * Each token takes its top_k experts by logit — the same choice as the top_k of the softmax, made
 * on the fp32 logits themselves; equal logits go to the lower expert id — in descending order:
 *   expert_idx[t, j], gates[t, j] = softmax(logits[t])[expert_idx[t, j]]  (fp32, not renormalised)
 * and the dispatch order, rows sorted by (expert, token):
 *   group_offsets[E+1] (expert e owns rows [off[e], off[e+1])), row_token[tokens·k] (the token of
 *   each row), token_row[tokens, k] (the row of (t, j)).
 * Integer outputs are deterministic and exact.  Logits must be finite.  E <= 1024, top_k <= 32.
 * All arrays int32 / fp32 in device memory, 4-byte aligned.  workspace:
 * tp_workspace_bytes("tp_moe_route", ...) with B·S = tokens and n_heads = E. */
int tp_moe_route(int tokens, int n_experts, int top_k, const float* logits, float* gates, int* expert_idx,
                 int* group_offsets, int* row_token, int* token_row, void* workspace, size_t workspace_bytes,
                 void* stream);

/* The MoE expert block of one tensor-parallel rank, on tp_moe_route's outputs: the dispatch is fused
 * into fc1's operand loads (row r of the expert-sorted matrix is read straight from X[row_token[r]],
 * no permuted copy of X is made), each expert's fc1 column shard with bias and GeLU, its fc2 row
 * shard, and the gate-weighted combine of the rank's partials:
 *   Y_r[r] = GeLU(X[row_token[r]]·W1_r[e] + b1_r[e]),  Z_r[r] = Y_r[r]·W2_r[e]   (r in expert e's rows)
 *   out_r[t] = Σ_j gates[t, j]·Z_r[token_row[t, j]]   (fp32 sum, j in order)
 * The combine is linear, so combining before the all-reduce gives the same sum over ranks with a
 * message k times smaller ([tokens, H] instead of [tokens·k, H]).  X [tokens, H]; W1_r [E, H, F_r],
 * b1_r [E, F_r], W2_r [E, F_r, H] with F_r = cnt(F_expert, t, r); Z_r [tokens·k, H] and Y_r
 * [tokens·k, F_r] required (written), A1_r nullable; out_r [tokens, H].  Offsets are clamped on the
 * device as in tp_mlp_grouped_shard_fwd; gathered and combined row indices outside their ranges read
 * as zero.  The fused gather needs X under 2 GiB for the bf16 tiled kernels (larger X runs the
 * generic kernels).  workspace: tp_workspace_bytes("tp_moe_shard_fwd", ...) with n_heads = E. */
int tp_moe_shard_fwd(int tp_size, int rank, int tokens, int H, int n_experts, int top_k, int F_expert, int dtype,
                     const void* X, const float* gates, const int* group_offsets, const int* row_token,
                     const int* token_row, const void* W1_r, const void* b1_r, const void* W2_r, void* out_r,
                     void* Z_r, void* A1_r, void* Y_r, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of tp_mlp_grouped_shard_fwd (the experts as grouped GEMMs: "Megatron-LM — 架构与原理", §6,
 * TE GroupedLinear), expert by expert on the same expert-sorted rows — the dense MLP shard's chain
 * rule (tp_mlp_shard_bwd) applied to each expert's rows and weights:
 *   dA1 = (dZ_perm·W2_r[e]ᵀ) ∘ GeLU'(A1_r)     dX_perm = dA1·W1_r[e]ᵀ   (rows of expert e)
 *   dW1_r[e] = X_eᵀ·dA1_e ;  db1_r[e] = Σ_rows dA1_e ;  dW2_r[e] = Y_eᵀ·dZ_e
 * An expert without rows gets zero weight and bias gradients.  Shapes as the forward's; dX_perm and
 * dZ_perm [rows, H], dW1_r like W1_r, db1_r like b1_r, dW2_r like W2_r.  dX_perm may be the same
 * buffer as dZ_perm (every read of dZ_perm comes first).  The experts' weight gradients are grouped
 * GEMMs whose k dimension is the expert's rows.  workspace: tp_workspace_bytes(
 * "tp_mlp_grouped_shard_bwd", ...) with B·S = rows, n_heads = n_groups, F = F_group (the offsets'
 * plan and dA1). */
int tp_mlp_grouped_shard_bwd(int tp_size, int rank, int n_groups, const int* group_offsets, int rows, int H,
                             int F_group, int dtype, const void* X_perm, const void* W1_r, const void* W2_r,
                             const void* A1_r, const void* Y_r, const void* dZ_perm, void* dX_perm, void* dW1_r,
                             void* db1_r, void* dW2_r, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of tp_moe_shard_fwd on rank r — the four beats route -> dispatch -> experts -> combine of
 * "Megatron-LM — 架构与原理", §4, taken in reverse — given d_out [tokens, H], the gradient of the whole
 * MoE output (every rank receives it, as the copy / all-reduce pair of the same section gives the
 * dense MLP its dZ), with row (t, j) = token_row[t, j]:
 *   dZ[row] = gates[t, j]·d_out[t]            the combine's backward
 *   dgates_r[t, j] = ⟨d_out[t], Y_r[row]·W2_r[e]⟩   (fp32; e the row's expert; Y_r[row]·W2_r[e] is
 *                                              the row's Z before rounding; a partial: Σ_r over ranks
 *                                              is the gate gradient, the combine being linear in them)
 *   the experts' backward as tp_mlp_grouped_shard_bwd, on X's rows in dispatch order
 *   dX_r[t] = Σ_j dX_perm[row]                 the dispatch's backward (a partial over ranks)
 * dZ is never stored: d_out's rows are gathered (row_token) and scaled by their gates inside the
 * GEMMs that use them, and the gate gradients are taken in the dA1 GEMM's epilogue as per-tile row
 * dots of its accumulators with Y_r, summed in a fixed order.  Inputs are the forward's: X, gates,
 * group_offsets, row_token, token_row from tp_moe_route, A1_r and Y_r from tp_moe_shard_fwd (A1_r now
 * required); Z_r is not read and may be NULL.  As in the forward, X's rows are gathered in dispatch
 * order (row_token) inside the dW1 GEMM's operand loads; indices outside X read as zero rows.
 * token_row must be a permutation of [0, tokens·k) and group_offsets cover all tokens·k rows, as
 * tp_moe_route writes them; token_row entries outside that range are skipped.  Outputs dW1_r, db1_r,
 * dW2_r as in tp_mlp_grouped_shard_bwd.  workspace: tp_workspace_bytes("tp_moe_shard_bwd", ...) with
 * B·S = tokens·top_k, n_heads = E, F = F_expert (the plan, dA1, the gates per row, the gate-scaled Y,
 * the row dots, dX_perm). */
int tp_moe_shard_bwd(int tp_size, int rank, int tokens, int H, int n_experts, int top_k, int F_expert, int dtype,
                     const void* X, const float* gates, const int* group_offsets, const int* row_token,
                     const int* token_row, const void* W1_r, const void* W2_r, const void* A1_r, const void* Y_r,
                     const void* Z_r, const void* d_out, void* dX_r, float* dgates_r, void* dW1_r, void* db1_r,
                     void* dW2_r, void* workspace, size_t workspace_bytes, void* stream);

/* The router's logit gradient from the (complete) gate gradient, the top-k choice held fixed (the
 * backward of tp_moe_route's gates, the route beat of "Megatron-LM — 架构与原理", §4):
 * with p = softmax(logits[t]) and gates[t, j] = p[expert_idx[t, j]],
 *   d_logits[t, e] = Σ_j dgates[t, j]·p[i_j]·(δ(i_j, e) − p[e]),  i_j = expert_idx[t, j]
 * fp32 [tokens, E]; the softmax is recomputed from the fp32 logits.  E <= 1024, top_k <= 32. */
int tp_moe_route_bwd(int tokens, int n_experts, int top_k, const float* logits, const int* expert_idx,
                     const float* dgates, float* d_logits, void* stream);

/* FP8: the OCP 8-bit floats E4M3 (1 sign, 4 exponent bits, bias 7, 3 mantissa bits, max 448) for
 * weights and activations and E5M2 (5 exponent bits, bias 15, 2 mantissa bits, max 57344) for
 * gradients.  Forward and backward GEMMs in FP8 beside FP32 master weights
 * ("Megatron-LM技术演进与大规模模型训练实践", §2.3); FP8 among the stack's mixed precisions ("NVIDIA
 * Megatron-LM：大规模Transformer模型分布式训练框架", §技术栈; "Megatron-LM — 架构与原理", capability
 * table). */
typedef enum { TP_FP8_E4M3 = 0, TP_FP8_E5M2 = 1 } tp_fp8_format;
typedef enum {
  TP_FP8_EPI_NONE = 0,        /* C = pre                                     */
  TP_FP8_EPI_GELU = 1,        /* C = GeLU(pre), C_pre = pre (nullable)       */
  TP_FP8_EPI_GELU_TANH = 2,   /* C = tanh-form GeLU(pre), C_pre = pre        */
  TP_FP8_EPI_DGELU = 3,       /* C = pre ∘ GeLU'(aux)   (fc1's backward)     */
  TP_FP8_EPI_DGELU_TANH = 4   /* C = pre ∘ tanh-form GeLU'(aux)              */
} tp_fp8_epilogue;

/* Per-tensor quantisation of x [rows, cols] (bf16 or fp32) to `format`:
 *   amax = max |x|;  s = vmax / amax and descale = amax / vmax in fp32 (1 and 1 when amax = 0)
 *   q = nearest code of fp32(x·s), ties to the even mantissa, saturating at ±vmax
 * vmax = 448 (E4M3) or 57344 (E5M2).  q [rows, cols] receives the codes as they lie, q_t [cols, rows]
 * the transposed copy (the K-major operand tp_fp8_gemm_nt takes for a matrix used along its rows);
 * either may be NULL, not both (TP_ENULL).  Asking for both reads x twice in all (amax, then one
 * pass writing both layouts when rows and cols are multiples of 16).  descale: one fp32 in device
 * memory (written).  x must be finite.  workspace: tp_workspace_bytes("tp_fp8_quantize", ...). */
int tp_fp8_quantize(int rows, int cols, int dtype, const void* x, int format, unsigned char* q, unsigned char* q_t,
                    float* descale, void* workspace, size_t workspace_bytes, void* stream);

/* GEMM on 8-bit codes, both operands K-major:
 *   pre = (A·Bᵀ)·a_descale·b_descale (+ bias[n]),  A [M, K], B [N, K] codes in their formats
 *   C per `epilogue` (tp_fp8_epilogue); aux [M, N] bf16 for the GeLU' epilogues
 * C, C_pre, aux, bias bf16; descales fp32 scalars in device memory (as tp_fp8_quantize writes them);
 * fp32 accumulation.  Requires K % 16 == 0, N % 8 == 0, operands below 2 GiB, not both operands
 * E5M2 (TP_EUNSUPPORTED otherwise). */
int tp_fp8_gemm_nt(int M, int N, int K, const unsigned char* A, int a_format, const float* a_descale,
                   const unsigned char* B, int b_format, const float* b_descale, const void* bias, int epilogue,
                   const void* aux, void* C, void* C_pre, void* stream);

/* Bias gradient of a linear layer: db[c] = Σ_{r < rows} dy[r, c], dy [rows, cols] row-major and db
 * [cols] in dtype, fp32 accumulation in a fixed order (repeatable bit for bit).  The backward
 * composed from the FP8 entry points takes db1 = Σ_t dA1 from it (the chain rule of the linear layer
 * Y = X·W + b of "Megatron-LM技术演进与大规模模型训练实践", §2.1).  workspace: tp_workspace_bytes("tp_bias_grad", ...) with B·S = rows
 * and H = cols. */
int tp_bias_grad(int rows, int cols, int dtype, const void* dy, void* db, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Workspace bytes an entry point needs for these sizes ("tp_mlp_shard_bwd", "tp_qkv_shard_bwd",
 * "tp_attn_heads_bwd", "tp_attn_out_shard_bwd", "tp_residual_ln_bwd", "tp_mlp_grouped_shard_fwd",
 * "tp_mlp_grouped_shard_bwd", "tp_moe_route", "tp_moe_shard_fwd", "tp_moe_shard_bwd", "tp_fp8_quantize",
 * "tp_bias_grad"; 0 for the others).  T = B*S; F is used by the
 * MLPs only, n_heads by the others (for "tp_mlp_grouped_shard_fwd" it carries n_groups).  Returns 0
 * for an unknown name or invalid sizes. */
size_t tp_workspace_bytes(const char* fn, int tp_size, int rank, int B, int S, int H,
                          int n_heads, int F, int dtype);

/* Kernel timing for benchmarks.  While enabled, every kernel this library launches is bracketed by
 * two hipEvents recorded on that launch's own stream and tagged with the kernel's name and the
 * launch's algorithmic FLOPs and bytes.  Off by default; the cost is two event records per launch. */
int tp_prof_enable(int enable);

/* Waits for the recorded events, aggregates them per kernel tag (first-seen order) and clears the
 * record.  Writes up to max_entries rows: tag (NUL-terminated, in names + i*name_len, at most
 * name_len bytes), launches, total milliseconds, total FLOPs, total bytes.  Returns the number of
 * distinct tags (possibly more than max_entries), or a negative tp_status. */
int tp_prof_collect(int max_entries, char* names, int name_len, int* launches, double* total_ms,
                    double* total_flop, double* total_bytes);

/* Static description of a status code. */
const char* tp_status_str(int status);

/* Message of the last TP_EHIP (or TP_EUNSUPPORTED detail) on the calling thread; "" if none. */
const char* tp_last_error(void);

/* Library version string, e.g. "tpshard 0.1 gfx950". */
const char* tp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
