"""Plain float64 CPU oracle for one tensor-parallel rank's shard of a Megatron Transformer layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP path: it imports numpy and scipy's erf
and nothing from the package.

Sources (the pages this follows; each is cited by title and section):
  [TP-essay]  "Megatron-LM技术演进与大规模模型训练实践", §2.1 并行范式奠基期: Y = X·W with W split by
              columns W = [W1 W2]; each device computes X·W1 or X·W2.
  [Digest]    "Megatron-LM 深度解读报告", §2.1 (column blocks computed independently, then joined)
              and the table of §2.2 (Q/K/V projections column-split by head; MLP first matmul
              column-split, second row-split; LayerNorm / Dropout replicated, not split).
  [Arch]      "Megatron-LM — 架构与原理", §4 巧妙之处: copy (identity forward, all-reduce backward)
              and reduce (all-reduce forward, identity backward) are duals; the column->row pairing
              leaves the MLP with one all-reduce at the RowParallelLinear exit.
  [Intro]     "Megatron-LM（英伟达超大模型训练框架）完整介绍", §二.2 张量并行: QKV split by column,
              heads computed independently on each card; MLP fc1 by column, fc2 by row.
  [Overview]  "NVIDIA Megatron-LM：大规模Transformer模型分布式训练框架", §核心架构：五大并行策略的协同艺术,
              sequence parallelism: LayerNorm and dropout activations, replicated under plain TP,
              are split along the sequence.

Readings where the pages are silent (numbered as in the design notes):
  R1 activation  = exact GeLU, x·Φ(x) = ½x(1 + erf(x/√2)); the pages name no activation.  Option:
                   the tanh form ½x(1 + tanh(√(2/π)(x + 0.044715x³))), GeLU's standard approximation.
  R2 attention   = scaled dot-product, scores·1/√d, causal (key j visible to query i iff j <= i),
                   softmax over keys; LSE_i = log Σ_j exp(score_ij) over visible keys.
  R3 QKV columns = head-interleaved: column h·3d + s·d + j holds part s∈{q,k,v}, element j of head h,
                   so a contiguous column block is a set of whole heads ("split by column, by head").
  R4 uneven split = balanced, lower ranks take the remainder (25 heads over 2 ranks -> 13 / 12).
  R5 biases      = bqkv and b1 split with their weight columns; b2 (row-split layer) added once, by
                   rank 0, so the partials sum to the unsharded output; db2 produced by rank 0 only.
  R6 the heads' outputs are combined by the attention output projection O = ctx·Wo + bo, taken as a
                   RowParallelLinear: rank r holds the rows of Wo that multiply its own heads' ctx
                   columns and yields a partial that the all-reduce completes, the same column->row
                   pairing as the MLP ([Intro] §二.2 says the heads' outputs are aggregated after
                   the per-card attention; [Arch] §2.3 lists RowParallelLinear, §4 the pairing).
                   bo is added once, by rank 0, as b2 (R5); dO is the full tensor on every rank (R9).
  R9 upstream gradient dZ of the row-split output is the full [T, H] tensor on every rank
                   (backward of reduce is the identity, [Arch] §4).
  R10 layout     = row-major; activations [B, S, ·] flattened to token b·S + s; weights [in, out].
  R11 LayerNorm, residual, dropout = replicated outside the split ([Digest] §2.2 table): the shard's
                   GEMMs take the already-normalised input.  As an op of its own: h = x + dropout(o)
                   (o the sublayer's summed output, bias included), y = LayerNorm(h)·γ + β per token
                   over the H features, biased variance, eps inside the square root; inverted dropout
                   (kept values scaled by 1/(1-p)) with the keep mask an input (the method's random
                   draws are passed in).  Pre-norm blocks carry h on as the residual stream, post-norm
                   blocks carry y; the op is the same.
  R14 MoE routing = each token's top-k experts by router logit (softmax is monotone, so the same
                   choice as the top-k of the softmax probabilities); equal logits go to the lower
                   expert id; the choice is made on the fp32 logits, as the device makes it.  Gate =
                   that expert's softmax probability over all experts (no renormalisation over the
                   k).  Dispatch order: rows sorted by (expert, token), stable.  No capacity limit.
                   Combine = Σ_j gate_j · expert output, j in the token's top-k order; it is linear,
                   so a rank may combine its fc2 partials before the all-reduce ([Arch] §4: route ->
                   dispatch (permute) -> experts -> combine (unpermute)).
  R15 FP8 = the OCP 8-bit floats: E4M3 (bias 7, 3 mantissa bits, no infinities, S.1111.111 NaN,
                   largest 448) for weights and activations, E5M2 (bias 15, 2 mantissa bits, IEEE-like
                   infinities and NaNs, largest 57344) for gradients.  One scale per tensor:
                   s = vmax / amax (fp32), the code of x is the value nearest to fp32(x·s), ties to
                   the even mantissa, saturating at ±vmax; descale = amax / vmax (1 when amax = 0).
                   The scale and the product are taken in fp32 because that is where the device
                   makes the decision.  A GEMM on codes: C = (Σ_k dec(a)·dec(b))·descale_a·descale_b.
  R13 sequence parallelism = LayerNorm and dropout split along the sequence ([Overview]; [Arch], the
                   table under 它能做什么): rank r owns rows [off(T,t,r), off+cnt) of the flattened
                   tokens (the sequence itself when B = 1) and its dγ, dβ are partial sums over its
                   rows; without it every rank holds all T rows and the full dγ, dβ.

Every function takes and returns float64 numpy arrays; nothing is rounded to the device's types.
"""

import math

import numpy as np
from scipy.special import erf as _erf

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ---- A0: shard geometry ----------------------------------------------------------------------

def shard_range(n: int, tp_size: int, rank: int):
    """Offset and count of the items (heads, MLP columns) rank `rank` owns out of n.

    Column blocks of one split ([TP-essay] §2.1; [Digest] §2.1).  Uneven split: reading R4.
    """
    if tp_size < 1 or not 0 <= rank < tp_size or n < 0:
        raise ValueError("bad shard request")
    base, rem = divmod(n, tp_size)
    count = base + (1 if rank < rem else 0)
    offset = rank * base + min(rank, rem)
    return offset, count


def qkv_column_range(n_heads: int, head_dim: int, tp_size: int, rank: int):
    """Columns [c0, c1) of the full QKV weight owned by `rank`: its heads, whole (reading R3)."""
    h0, nh = shard_range(n_heads, tp_size, rank)
    return 3 * head_dim * h0, 3 * head_dim * (h0 + nh)


# ---- explicit slicing of the unsharded weights ------------------------------------------------

def slice_qkv(Wqkv, bqkv, n_heads: int, tp_size: int, rank: int):
    """Column block of the QKV ColumnParallelLinear ([Digest] §2.2 table, attention row)."""
    d = Wqkv.shape[0] // n_heads
    c0, c1 = qkv_column_range(n_heads, d, tp_size, rank)
    return Wqkv[:, c0:c1], bqkv[c0:c1]


def slice_fc1(W1, b1, tp_size: int, rank: int):
    """Column block of fc1 ([Digest] §2.2 table, MLP row: first matmul column-split)."""
    f0, fr = shard_range(W1.shape[1], tp_size, rank)
    return W1[:, f0:f0 + fr], b1[f0:f0 + fr]


def slice_fc2(W2, tp_size: int, rank: int):
    """Row block of fc2 ([Digest] §2.2 table, MLP row: second matmul row-split)."""
    f0, fr = shard_range(W2.shape[0], tp_size, rank)
    return W2[f0:f0 + fr, :]


def slice_attn_out(Wo, n_heads: int, tp_size: int, rank: int):
    """Row block of the attention output projection: the d·nh_r rows that multiply the rank's own
    heads' context columns (reading R6)."""
    d = Wo.shape[0] // n_heads
    h0, nh = shard_range(n_heads, tp_size, rank)
    return Wo[d * h0:d * (h0 + nh), :]


# ---- element-wise activation (reading R1) ------------------------------------------------------

def gelu(x):
    """GeLU(x) = x·Φ(x), Φ the standard normal CDF = ½(1 + erf(x/√2))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / _SQRT2))


def gelu_grad(x):
    """d/dx [x·Φ(x)] = Φ(x) + x·φ(x), φ the standard normal density."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + _erf(x / _SQRT2)) + x * _INV_SQRT_2PI * np.exp(-0.5 * x * x)


_C_TANH = math.sqrt(2.0 / math.pi)


def gelu_tanh(x):
    """The tanh approximation of GeLU: ½x(1 + tanh(√(2/π)(x + 0.044715x³)))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(_C_TANH * (x + 0.044715 * x ** 3)))


def gelu_tanh_grad(x):
    """Its derivative: ½(1 + t) + ½x(1 − t²)·√(2/π)(1 + 3·0.044715x²), t = tanh(√(2/π)(x + 0.044715x³))."""
    x = np.asarray(x, dtype=np.float64)
    t = np.tanh(_C_TANH * (x + 0.044715 * x ** 3))
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * _C_TANH * (1.0 + 3 * 0.044715 * x * x)


def _activation(a):
    """(function, derivative) of activation a: 0 the exact GeLU, 1 its tanh form."""
    if a == 0:
        return gelu, gelu_grad
    if a == 1:
        return gelu_tanh, gelu_tanh_grad
    raise ValueError(f"unknown activation {a}")


# ---- attention (readings R2, R3) ---------------------------------------------------------------

def _heads(QKV, B: int, S: int, n_heads: int, d: int):
    """q, k, v of every head, each [B, n_heads, S, d], from the head-interleaved columns."""
    t = np.asarray(QKV).reshape(B, S, n_heads, 3, d)
    return (t[:, :, :, 0, :].transpose(0, 2, 1, 3),
            t[:, :, :, 1, :].transpose(0, 2, 1, 3),
            t[:, :, :, 2, :].transpose(0, 2, 1, 3))


def _softmax_causal(q, k, d: int):
    """P = softmax_j(q·kᵀ/√d) over visible keys j <= i, and LSE_i (reading R2)."""
    S = q.shape[0]
    sc = (q @ k.T) / math.sqrt(d)
    visible = np.tril(np.ones((S, S), dtype=bool))
    sc = np.where(visible, sc, -np.inf)
    m = sc.max(axis=1, keepdims=True)
    e = np.exp(sc - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def attention_fwd(QKV, B: int, S: int, n_heads: int, d: int):
    """Per-head causal attention; heads are independent ([Intro] §二.2; [Digest] §2.2 table).

    Returns ctx [B·S, n_heads·d] (head h in columns h·d .. h·d+d-1) and LSE [B, n_heads, S].
    """
    q, k, v = _heads(QKV, B, S, n_heads, d)
    ctx = np.zeros((B, S, n_heads, d))
    lse = np.zeros((B, n_heads, S))
    for b in range(B):
        for h in range(n_heads):
            p, lse[b, h] = _softmax_causal(q[b, h], k[b, h], d)
            ctx[b, :, h, :] = p @ v[b, h]
    return ctx.reshape(B * S, n_heads * d), lse


def attention_bwd(QKV, dctx, B: int, S: int, n_heads: int, d: int):
    """Gradient of the causal attention w.r.t. its QKV input, from the definitions.

    P is recomputed from q, k (recomputation instead of storing it: [Intro] 三.2).
    dV = Pᵀ·dO;  dP = dO·Vᵀ;  softmax Jacobian dS_ij = P_ij·(dP_ij − Σ_k P_ik·dP_ik);
    dQ = dS·K/√d;  dK = dSᵀ·Q/√d.  Returned in the same interleaved [B·S, 3·n_heads·d] layout.
    """
    q, k, v = _heads(QKV, B, S, n_heads, d)
    do = np.asarray(dctx).reshape(B, S, n_heads, d)
    dqkv = np.zeros((B, S, n_heads, 3, d))
    for b in range(B):
        for h in range(n_heads):
            p, _ = _softmax_causal(q[b, h], k[b, h], d)
            dO = do[b, :, h, :]
            dP = dO @ v[b, h].T
            dS = p * (dP - (p * dP).sum(axis=1, keepdims=True))
            dqkv[b, :, h, 0, :] = dS @ k[b, h] / math.sqrt(d)
            dqkv[b, :, h, 1, :] = dS.T @ q[b, h] / math.sqrt(d)
            dqkv[b, :, h, 2, :] = p.T @ dO
    return dqkv.reshape(B * S, n_heads * 3 * d)


# ---- linear parts ------------------------------------------------------------------------------

def qkv_fwd(X, Wqkv, bqkv):
    """QKV = X·Wqkv + bqkv ([TP-essay] §2.1: Y = X·W)."""
    return X @ Wqkv + bqkv


def qkv_bwd(X, Wqkv, dQKV):
    """dW = Xᵀ·dQKV, db = Σ_t dQKV, dX = dQKV·Wᵀ (input gradient; a partial sum on a shard)."""
    return {"dX": dQKV @ Wqkv.T, "dW": X.T @ dQKV, "db": dQKV.sum(axis=0)}


def mlp_fwd(X, W1, b1, W2, b2, activation=0):
    """A1 = X·W1 + b1;  Y = GeLU(A1) (activation 1: the tanh form);  Z = Y·W2 (+ b2 when b2 is not None)."""
    A1 = X @ W1 + b1
    Y = _activation(activation)[0](A1)
    Z = Y @ W2
    if b2 is not None:
        Z = Z + b2
    return {"A1": A1, "Y": Y, "Z": Z}


def mlp_bwd(X, W1, W2, A1, Y, dZ, with_db2: bool, activation=0):
    """Backward of mlp_fwd, from the chain rule written out:

    dW2 = Yᵀ·dZ;  db2 = Σ_t dZ;  dA1 = (dZ·W2ᵀ) ∘ GeLU'(A1);  db1 = Σ_t dA1;
    dW1 = Xᵀ·dA1;  dX = dA1·W1ᵀ.
    """
    dA1 = (dZ @ W2.T) * _activation(activation)[1](A1)
    return {"dX": dA1 @ W1.T, "dW1": X.T @ dA1, "db1": dA1.sum(axis=0),
            "dW2": Y.T @ dZ, "db2": dZ.sum(axis=0) if with_db2 else None, "dA1": dA1}


def attn_out_fwd(ctx, Wo, bo):
    """O = ctx·Wo (+ bo when bo is not None): the heads' outputs combined (reading R6)."""
    O = ctx @ Wo
    if bo is not None:
        O = O + bo
    return O


def attn_out_bwd(ctx, Wo, dO, with_db: bool):
    """Backward of attn_out_fwd from the chain rule: dWo = ctxᵀ·dO; dbo = Σ_t dO; dctx = dO·Woᵀ."""
    return {"dctx": dO @ Wo.T, "dW": ctx.T @ dO, "db": dO.sum(axis=0) if with_db else None}


# ---- replicated-side ops: residual add with dropout, LayerNorm (readings R11, R13) ------------

def dropout_add(x, o, keep, p_drop):
    """h = x + o ∘ keep / (1 − p): inverted dropout of the sublayer output o, then the residual add.
    o None: h = x.  keep None: no dropout."""
    x = np.asarray(x, dtype=np.float64)
    if o is None:
        return x.copy()
    if keep is None:
        return x + o
    return x + o * np.asarray(keep, dtype=np.float64) / (1.0 - p_drop)


def layernorm(h, gamma, beta, eps):
    """Per row over the features: mean, biased variance, y = (h − mean)/√(var + eps)·γ + β.
    Returns y, mean, rstd = 1/√(var + eps)."""
    mean = h.mean(axis=1)
    c = h - mean[:, None]
    var = (c * c).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    return c * rstd[:, None] * gamma + beta, mean, rstd


def layernorm_bwd(h, gamma, dy, eps):
    """Gradients of layernorm by the chain rule through the row mean and variance.  With
    x̂ = (h − mean)·rstd and g = dy·γ:  dβ = Σ_t dy;  dγ = Σ_t dy·x̂;
    dh = rstd·(g − mean_H(g) − x̂·mean_H(g·x̂))."""
    mean = h.mean(axis=1)
    c = h - mean[:, None]
    rstd = 1.0 / np.sqrt((c * c).mean(axis=1) + eps)
    xhat = c * rstd[:, None]
    g = dy * gamma
    dh = rstd[:, None] * (g - g.mean(axis=1, keepdims=True) - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dh, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def sp_rows(T: int, tp_size: int, rank: int, sequence_parallel: bool):
    """Rows [r0, r0 + n) of the T tokens a rank normalises (reading R13)."""
    if sequence_parallel:
        return shard_range(T, tp_size, rank)
    if tp_size < 1 or not 0 <= rank < tp_size:
        raise ValueError("bad rank")
    return 0, T


# ---- the unsharded layer ------------------------------------------------------------------------

def layer_fwd(X, Wqkv, bqkv, W1, b1, W2, b2, B: int, S: int, n_heads: int, Wo=None, bo=None):
    """QKV projection + per-head causal attention (+ the output projection O when Wo is given), and
    the MLP, on one device, unsplit.

    LayerNorm, dropout and residuals are replicated outside the split ([Digest] §2.2 table) and
    are not part of the shard; X is the already-normalised input of both blocks.
    """
    d = X.shape[1] // n_heads
    QKV = qkv_fwd(X, Wqkv, bqkv)
    ctx, lse = attention_fwd(QKV, B, S, n_heads, d)
    out = mlp_fwd(X, W1, b1, W2, b2)
    out.update(QKV=QKV, ctx=ctx, lse=lse)
    if Wo is not None:
        out["O"] = attn_out_fwd(ctx, Wo, bo)
    return out


# ---- one rank's shard: the same names and arguments as the C ABI ---------------------------------

def _check_heads(H, n_heads, tp_size, rank):
    if H % n_heads:
        raise ValueError("H must be a multiple of n_heads")
    h0, nh = shard_range(n_heads, tp_size, rank)
    return h0, nh, H // n_heads


def tp_qkv_shard_fwd(tp_size, rank, B, S, H, n_heads, X, Wqkv_r, bqkv_r):
    """QKV ColumnParallelLinear of rank r: X·Wqkv_r + bqkv_r, no gather ([Arch] §4; [Digest] §2.2)."""
    _, nh, d = _check_heads(H, n_heads, tp_size, rank)
    assert X.shape == (B * S, H) and Wqkv_r.shape == (H, 3 * nh * d)
    return qkv_fwd(X, Wqkv_r, bqkv_r)


def tp_attn_heads_fwd(tp_size, rank, B, S, H, n_heads, QKV_r):
    """Causal attention over the rank's own heads ([Intro] §二.2: each card computes its heads)."""
    _, nh, d = _check_heads(H, n_heads, tp_size, rank)
    assert QKV_r.shape == (B * S, 3 * nh * d)
    return attention_fwd(QKV_r, B, S, nh, d)


def tp_mlp_shard_fwd(tp_size, rank, T, H, F, X, W1_r, b1_r, W2_r, b2, activation=0):
    """fc1 column shard + GeLU, fc2 row shard -> partial Z_r; b2 added iff rank == 0 (R5).

    Σ_r Z_r is the unsharded Z: the all-reduce at the RowParallelLinear exit ([Arch] §4).
    """
    _, fr = shard_range(F, tp_size, rank)
    assert X.shape == (T, H) and W1_r.shape == (H, fr) and W2_r.shape == (fr, H)
    return mlp_fwd(X, W1_r, b1_r, W2_r, b2 if rank == 0 else None, activation)


def tp_mlp_shard_bwd(tp_size, rank, T, H, F, X, W1_r, W2_r, A1_r, Y_r, dZ, activation=0):
    """Backward of the rank's MLP shard.  dZ is the full upstream gradient (R9); dX_r is a partial
    whose sum over ranks is dX (copy's backward all-reduce, [Arch] §4); db2 iff rank == 0 (R5)."""
    _, fr = shard_range(F, tp_size, rank)
    assert dZ.shape == (T, H) and A1_r.shape == (T, fr) and Y_r.shape == (T, fr)
    return mlp_bwd(X, W1_r, W2_r, A1_r, Y_r, dZ, with_db2=(rank == 0), activation=activation)


def tp_qkv_shard_bwd(tp_size, rank, B, S, H, n_heads, X, Wqkv_r, dQKV_r):
    """Backward of the QKV column shard; dX_r is a partial summed over ranks ([Arch] §4)."""
    _, nh, d = _check_heads(H, n_heads, tp_size, rank)
    assert dQKV_r.shape == (B * S, 3 * nh * d)
    return qkv_bwd(X, Wqkv_r, dQKV_r)


def tp_attn_heads_bwd(tp_size, rank, B, S, H, n_heads, QKV_r, dctx_r):
    """Backward of the rank's heads.  The definition needs only QKV_r and dctx_r: P is recomputed."""
    _, nh, d = _check_heads(H, n_heads, tp_size, rank)
    assert dctx_r.shape == (B * S, nh * d)
    return attention_bwd(QKV_r, dctx_r, B, S, nh, d)


def tp_attn_out_shard_fwd(tp_size, rank, B, S, H, n_heads, ctx_r, Wo_r, bo):
    """Output projection of the rank's heads, a RowParallelLinear: O_r = ctx_r·Wo_r (+ bo iff
    rank == 0).  Σ_r O_r is the unsharded ctx·Wo + bo (reading R6)."""
    _, nh, d = _check_heads(H, n_heads, tp_size, rank)
    assert ctx_r.shape == (B * S, nh * d) and Wo_r.shape == (nh * d, H)
    return attn_out_fwd(ctx_r, Wo_r, bo if rank == 0 else None)


def tp_attn_out_shard_bwd(tp_size, rank, B, S, H, n_heads, ctx_r, Wo_r, dO):
    """Backward of the rank's output projection.  dO is the full upstream gradient (R9); dctx_r is
    the rank's own column block of dctx (no sum needed); dbo iff rank == 0 (R6)."""
    _, nh, d = _check_heads(H, n_heads, tp_size, rank)
    assert dO.shape == (B * S, H) and ctx_r.shape == (B * S, nh * d)
    return attn_out_bwd(ctx_r, Wo_r, dO, with_db=(rank == 0))


def tp_residual_ln_fwd(tp_size, rank, sequence_parallel, T, H, x, o, keep, p_drop, gamma, beta, eps):
    """Residual add with dropout, then LayerNorm, on the rank's rows (all T, or its block of the
    sequence under sequence parallelism): h = x + dropout(o); y = LayerNorm(h)·γ + β (R11, R13)."""
    _, n = sp_rows(T, tp_size, rank, sequence_parallel)
    assert np.shape(x) == (n, H)
    h = dropout_add(x, o, keep, p_drop)
    y, mean, rstd = layernorm(h, gamma, beta, eps)
    return {"h": h, "y": y, "mean": mean, "rstd": rstd}


def tp_residual_ln_bwd(tp_size, rank, sequence_parallel, T, H, dy, dh_in, h, gamma, keep, p_drop, eps):
    """Backward of tp_residual_ln_fwd on the rank's rows.  dh_in is the gradient reaching h along
    the residual stream (None: none); dh is the gradient of h, which is also that of x (the
    residual passes it through); do = dh ∘ keep/(1 − p).  dγ, dβ sum over the rank's rows: partials
    under sequence parallelism, whose sum over ranks is the full gradient (R13)."""
    _, n = sp_rows(T, tp_size, rank, sequence_parallel)
    assert np.shape(dy) == (n, H)
    dh, dgamma, dbeta = layernorm_bwd(h, gamma, dy, eps)
    if dh_in is not None:
        dh = dh + dh_in
    do = dh * np.asarray(keep, dtype=np.float64) / (1.0 - p_drop) if keep is not None else dh.copy()
    return {"dh": dh, "do": do, "dgamma": dgamma, "dbeta": dbeta}


def moe_route(logits32, top_k: int):
    """Top-k routing (reading R14).  logits32: float32 [tokens, E].  Returns gates [tokens, k]
    (float64 softmax probabilities of the chosen experts), experts [tokens, k] (descending logit,
    ties to the lower id), group_offsets [E+1], row_token [tokens·k] (the token of each
    expert-sorted row) and token_row [tokens, k] (the row of each (token, j))."""
    lg = np.asarray(logits32, dtype=np.float32)
    n, E = lg.shape
    experts = np.zeros((n, top_k), dtype=np.int64)
    for t in range(n):
        # sort by (−logit, id): compare the float32 values exactly, lower id first on ties
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))
        experts[t] = order[:top_k]
    l64 = lg.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    gates = np.take_along_axis(p, experts, axis=1)
    counts = np.bincount(experts.reshape(-1), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    row_token = np.zeros(n * top_k, dtype=np.int64)
    token_row = np.zeros((n, top_k), dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(n):                      # token order within each expert: stable
        for j in range(top_k):
            e = experts[t, j]
            row_token[fill[e]] = t
            token_row[t, j] = fill[e]
            fill[e] += 1
    return {"gates": gates, "experts": experts, "group_offsets": offsets, "row_token": row_token,
            "token_row": token_row}


def moe_combine(Z_rows, gates, token_row):
    """out[t] = Σ_j gates[t, j] · Z_rows[token_row[t, j]] (reading R14)."""
    out = np.zeros((gates.shape[0], Z_rows.shape[1]))
    for j in range(gates.shape[1]):
        out += gates[:, j:j + 1] * Z_rows[token_row[:, j]]
    return out


def tp_moe_shard_fwd(tp_size, rank, X, route, W1_r, b1_r, W2_r):
    """The MoE expert block on rank r: dispatch (the rows of X in expert-sorted order), each
    expert's fc1 column shard with bias and GeLU and its fc2 row shard, then the gate-weighted
    combine of the rank's partials.  Σ_r over ranks is the full MoE output ([Arch] §4, §6).
    Also returns the expert-sorted A1, Y and Z rows the backward takes."""
    Xp = np.asarray(X)[route["row_token"]]
    off = route["group_offsets"]
    A1 = np.zeros((Xp.shape[0], W1_r.shape[2]))
    for e in range(W1_r.shape[0]):
        lo, hi = int(off[e]), int(off[e + 1])
        A1[lo:hi] = Xp[lo:hi] @ W1_r[e] + b1_r[e]
    Y = gelu(A1)
    Z = tp_mlp_grouped_shard_fwd(tp_size, rank, off, Xp, W1_r, b1_r, W2_r)
    return {"out": moe_combine(Z, route["gates"], route["token_row"]), "Z": Z, "A1": A1, "Y": Y}


def moe_combine_bwd(d_out, Z_rows, gates, token_row):
    """Backward of moe_combine (out[t] = Σ_j g[t, j]·Z[token_row[t, j]]), from the chain rule:
    dZ[token_row[t, j]] = g[t, j]·d_out[t]  (each row is one (t, j): the dispatch is a permutation)
    dg[t, j] = ⟨d_out[t], Z[token_row[t, j]]⟩."""
    n, k = gates.shape
    dZ = np.zeros(Z_rows.shape)
    dg = np.zeros((n, k))
    for j in range(k):
        rows = token_row[:, j]
        dZ[rows] = gates[:, j:j + 1] * d_out
        dg[:, j] = np.sum(d_out * Z_rows[rows], axis=1)
    return {"dZ": dZ, "dgates": dg}


def tp_mlp_grouped_shard_bwd(group_offsets, X_perm, W1_r, W2_r, A1, Y, dZ):
    """Backward of tp_mlp_grouped_shard_fwd: for each expert e, mlp_bwd on its rows with its own
    weights (dW1[e], db1[e], dW2[e] from its rows only; zero for an expert without rows); the rows'
    input gradients dX_perm in the same expert-sorted order."""
    G, H, Fr = W1_r.shape
    dXp = np.zeros(X_perm.shape)
    dA1 = np.zeros(A1.shape)
    dW1, db1, dW2 = np.zeros((G, H, Fr)), np.zeros((G, Fr)), np.zeros((G, Fr, H))
    for e in range(G):
        lo, hi = int(group_offsets[e]), int(group_offsets[e + 1])
        if hi > lo:
            g = mlp_bwd(X_perm[lo:hi], W1_r[e], W2_r[e], A1[lo:hi], Y[lo:hi], dZ[lo:hi], False)
            dXp[lo:hi], dA1[lo:hi] = g["dX"], g["dA1"]
            dW1[e], db1[e], dW2[e] = g["dW1"], g["db1"], g["dW2"]
    return {"dX_perm": dXp, "dA1": dA1, "dW1": dW1, "db1": db1, "dW2": dW2}


def tp_moe_shard_bwd(tp_size, rank, X, route, W1_r, W2_r, fwd, d_out):
    """Backward of tp_moe_shard_fwd on rank r, given the gradient d_out of the full MoE output (every
    rank receives it, as the copy / all-reduce pair makes it for the dense MLP): the combine's
    backward (dZ rows, the rank's partial gate gradient — Σ over ranks is the full one, since the
    combine is linear in the partials), the experts' grouped backward, and the dispatch's backward
    dX[t] = Σ_j dX_perm[token_row[t, j]] (the rank's partial input gradient).  The combine's
    backward takes each row's expert output Z[r] = Y[r]·W2_r[e] as the grouped fc2 defines it, from
    the saved Y (not a Z the forward may have rounded to storage)."""
    Y = np.asarray(fwd["Y"], dtype=np.float64)
    off = route["group_offsets"]
    Z = np.zeros((Y.shape[0], W2_r.shape[2]))
    for e in range(W2_r.shape[0]):
        lo, hi = int(off[e]), int(off[e + 1])
        Z[lo:hi] = Y[lo:hi] @ W2_r[e]
    cb = moe_combine_bwd(d_out, Z, route["gates"], route["token_row"])
    Xp = np.asarray(X)[route["row_token"]]
    g = tp_mlp_grouped_shard_bwd(route["group_offsets"], Xp, W1_r, W2_r, fwd["A1"], fwd["Y"], cb["dZ"])
    tr = route["token_row"]
    dX = np.zeros(np.shape(X))
    for j in range(tr.shape[1]):
        dX += g["dX_perm"][tr[:, j]]
    return {"dX": dX, "dgates": cb["dgates"], "dW1": g["dW1"], "db1": g["db1"], "dW2": g["dW2"],
            "dA1": g["dA1"], "dZ": cb["dZ"]}


def moe_route_bwd(logits32, experts, dgates):
    """Gradient of the router logits from the gates' gradient (reading R14: gate = p_e, the softmax
    probability over all experts, for the chosen e).  With the choice held fixed, ∂p_i/∂l_e =
    p_i(δ_ie − p_e), so d_logits[t, e] = Σ_j dg[t, j]·p_{i_j}·(δ_{i_j e} − p_e)."""
    l64 = np.asarray(logits32, dtype=np.float32).astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    n, E = p.shape
    dl = np.zeros((n, E))
    for t in range(n):
        s = 0.0
        for j in range(experts.shape[1]):
            i = int(experts[t, j])
            dl[t, i] += dgates[t, j] * p[t, i]
            s += dgates[t, j] * p[t, i]
        dl[t] -= s * p[t]
    return dl


# ---- FP8 (reading R15) -------------------------------------------------------------------------

def _fp8_format(fmt):
    """(exponent bits, mantissa bits, bias, largest finite value) of an OCP 8-bit float."""
    if fmt == "e4m3":
        return 4, 3, 7, 448.0
    if fmt == "e5m2":
        return 5, 2, 15, 57344.0
    raise ValueError(f"unknown fp8 format {fmt!r}")


def fp8_decode(codes, fmt="e4m3"):
    """Values of 8-bit float codes from the format's definition.  E4M3: no infinities, S.1111.111
    is NaN.  E5M2: exponent 31 holds ±inf (mantissa 0) and NaN."""
    eb, mb, bias, _ = _fp8_format(fmt)
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> mb) & ((1 << eb) - 1)
    m = c & ((1 << mb) - 1)
    frac = m / float(1 << mb)
    mag = np.where(e == 0, frac * 2.0 ** (1 - bias), (1.0 + frac) * 2.0 ** (e.astype(np.float64) - bias))
    if fmt == "e4m3":
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
    else:
        mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def e4m3_decode(codes):
    return fp8_decode(codes, "e4m3")


_FP8_POS = {f: fp8_decode(np.arange(0x80), f) for f in ("e4m3", "e5m2")}


def fp8_encode(y, fmt="e4m3"):
    """Nearest finite code to each value (ties to the even mantissa), saturating at ± the largest
    finite value of the format."""
    _, _, _, vmax = _fp8_format(fmt)
    pos = _FP8_POS[fmt]
    n = int(np.searchsorted(pos, vmax, side="right"))      # the finite non-negative codes: 0 .. n-1
    fin = pos[:n]
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), vmax)
    hi = np.clip(np.searchsorted(fin, a, side="left"), 0, n - 1)    # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_hi, d_lo = fin[hi] - a, a - fin[lo]
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == fin[hi], hi, pick)
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def e4m3_encode(y):
    return fp8_encode(y, "e4m3")


def fp8_quantize(x, transpose=False, fmt="e4m3"):
    """Per-tensor quantisation (reading R15): s = vmax / amax in fp32, codes = nearest of fp32(x·s),
    descale = amax / vmax (1 and 1 when amax = 0); vmax = 448 (E4M3) or 57344 (E5M2).  Returns the
    codes (transposed when asked: the [cols, rows] copy a K-major GEMM operand needs) and the fp32
    descale."""
    vmax = np.float32(_fp8_format(fmt)[3])
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if amax == 0:
        s, descale = np.float32(1), np.float32(1)
    else:
        s = vmax / amax
        descale = amax / vmax
    q = fp8_encode((x32 * s).astype(np.float32), fmt)
    return (np.ascontiguousarray(q.T) if transpose else q), descale


FP8_EPI_NONE, FP8_EPI_GELU, FP8_EPI_GELU_TANH, FP8_EPI_DGELU, FP8_EPI_DGELU_TANH = 0, 1, 2, 3, 4


def fp8_gemm_nt(A_codes, a_descale, B_codes, b_descale, bias=None, epi=FP8_EPI_NONE, aux=None,
                fmt_a="e4m3", fmt_b="e4m3"):
    """pre = (dec(A)·dec(B)ᵀ)·descale_a·descale_b (+ bias);  C = pre, GeLU(pre) (exact or tanh form),
    or pre ∘ GeLU'(aux) (the fc1 backward's product with the activation's derivative at A1 = aux).
    A [M, K] and B [N, K] codes in their formats."""
    pre = (fp8_decode(A_codes, fmt_a) @ fp8_decode(B_codes, fmt_b).T) * float(a_descale) * float(b_descale)
    if bias is not None:
        pre = pre + bias
    if epi == FP8_EPI_NONE:
        C = pre
    elif epi in (FP8_EPI_GELU, FP8_EPI_GELU_TANH):
        C = _activation(epi - 1)[0](pre)
    else:
        C = pre * _activation(epi - 3)[1](np.asarray(aux, dtype=np.float64))
    return {"pre": pre, "C": C}


def tp_mlp_grouped_shard_fwd(tp_size, rank, group_offsets, X_perm, W1_r, b1_r, W2_r):
    """Expert MLP shards applied to the rows each expert owns.

    Rows [o_e, o_{e+1}) of the expert-sorted token matrix go through expert e's column shard of fc1,
    GeLU, and its row shard of fc2 (expert FFNs as grouped GEMMs: "Megatron-LM — 架构与原理", §6,
    TE GroupedLinear).  No bias on the expert's fc2 partial.
    """
    G = W1_r.shape[0]
    Z = np.zeros((X_perm.shape[0], W2_r.shape[2]))
    for e in range(G):
        lo, hi = int(group_offsets[e]), int(group_offsets[e + 1])
        if hi > lo:
            Z[lo:hi] = gelu(X_perm[lo:hi] @ W1_r[e] + b1_r[e]) @ W2_r[e]
    return Z


def normwise_error(got, ref):
    """‖got − ref‖_F / ‖ref‖_F in float64 (absolute ‖got − ref‖_F when ‖ref‖_F = 0).

    The per-tensor parity measure: a normwise relative error, the bar being 2e-2 for bf16 operands
    with fp32 accumulation and 1e-5 in fp32 mode.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return num / den if den > 0 else num


def _as_rows(a):
    """A tensor viewed as a matrix: one row per index of the leading dimensions (a vector is one row)."""
    a = np.asarray(a, dtype=np.float64)
    if a.ndim == 0:
        return a.reshape(1, 1)
    if a.ndim == 1:
        return a.reshape(1, -1)
    return a.reshape(-1, a.shape[-1])


def blockwise_error(got, ref, block=64):
    """The largest local error over the block x block tiles of a tensor (viewed as a matrix).

    For each tile b:  ‖got_b − ref_b‖_F / max(‖ref_b‖_F, ‖ref‖_F·√(n_b/n)),  n_b the tile's element
    count and n the tensor's.  So a tile is held to the normwise bar relative to its own values, or,
    where its values are smaller than the tensor's average, relative to its share of the whole
    tensor's norm.  A defect confined to one tile (a dropped k-slice, a wrong tile offset) counts at
    its local size instead of being diluted by the rest of the tensor.  Absolute per-tile error
    ‖got_b − ref_b‖_F when ‖ref‖_F = 0.
    """
    g, r = _as_rows(got), _as_rows(ref)
    assert g.shape == r.shape, f"shape {g.shape} vs {r.shape}"
    R, C = r.shape
    if R * C == 0:
        return 0.0
    br, bc = min(block, R), min(block, C)
    nR, nC = -(-R // br), -(-C // bc)

    def tile_sums(x):
        pad = np.zeros((nR * br, nC * bc))
        pad[:R, :C] = x
        return pad.reshape(nR, br, nC, bc).sum(axis=(1, 3))

    diff2 = tile_sums((g - r) ** 2)
    ref2 = tile_sums(r * r)
    count = tile_sums(np.ones_like(r))
    total = np.linalg.norm(r)
    if total == 0:
        return float(np.sqrt(diff2.max()))
    den = np.maximum(np.sqrt(ref2), total * np.sqrt(count / (R * C)))
    return float((np.sqrt(diff2) / den).max())
