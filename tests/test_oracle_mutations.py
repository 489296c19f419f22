"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin catches each one."""

import math

import numpy as np
import pytest

import oracle.tp_shard as T
import oracle_pins as P

_erf = T._erf


def _softmax_variant(mask_k=0, scale=None, lse_without_max=False, no_mask=False):
    def f(q, k, d):
        S = q.shape[0]
        sc = (q @ k.T) / (scale(d) if scale else math.sqrt(d))
        if not no_mask:
            sc = np.where(np.tril(np.ones((S, S), dtype=bool), k=mask_k), sc, -np.inf)
        m = sc.max(axis=1, keepdims=True)
        e = np.exp(sc - m)
        l = e.sum(axis=1, keepdims=True)
        lse = np.log(l)[:, 0] if lse_without_max else (m + np.log(l))[:, 0]
        return e / l, lse
    return f


def _heads_blocked(QKV, B, S, n_heads, d):
    t = np.asarray(QKV).reshape(B, S, 3, n_heads, d)      # [Q_all | K_all | V_all]
    return tuple(t[:, :, s].transpose(0, 2, 1, 3) for s in range(3))


def _gelu_tanh(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def _gelu_grad_no_density(x):
    return 0.5 * (1.0 + _erf(np.asarray(x) / math.sqrt(2.0)))


def _shard_range_last_takes_rest(n, t, r):
    base, rem = divmod(n, t)
    return r * base, base + (rem if r == t - 1 else 0)


def _mlp_fwd_b2_everywhere(tp_size, rank, Tt, H, F, X, W1_r, b1_r, W2_r, b2):
    return T.mlp_fwd(X, W1_r, b1_r, W2_r, b2)


def _mlp_fwd_no_b1(X, W1, b1, W2, b2):
    A1 = X @ W1
    Y = T.gelu(A1)
    Z = Y @ W2 + (b2 if b2 is not None else 0)
    return {"A1": A1, "Y": Y, "Z": Z}


def _attn_bwd_variant(drop_D=False, dK_untransposed=False, dQ_unscaled=False, dV_wrong=False):
    def f(QKV, dctx, B, S, n_heads, d):
        q, k, v = T._heads(QKV, B, S, n_heads, d)
        do = np.asarray(dctx).reshape(B, S, n_heads, d)
        out = np.zeros((B, S, n_heads, 3, d))
        for b in range(B):
            for h in range(n_heads):
                p, _ = T._softmax_causal(q[b, h], k[b, h], d)
                dO = do[b, :, h, :]
                dP = dO @ v[b, h].T
                dS = p * dP if drop_D else p * (dP - (p * dP).sum(axis=1, keepdims=True))
                out[b, :, h, 0, :] = dS @ k[b, h] / (1.0 if dQ_unscaled else math.sqrt(d))
                out[b, :, h, 1, :] = (dS if dK_untransposed else dS.T) @ q[b, h] / math.sqrt(d)
                out[b, :, h, 2, :] = (p @ dO) if dV_wrong else (p.T @ dO)
        return out.reshape(B * S, n_heads * 3 * d)
    return f


def _mlp_bwd_variant(gelu_not_grad=False, db1_before_gelu=False, dW2_from_A1=False):
    def f(X, W1, W2, A1, Y, dZ, with_db2):
        dY = dZ @ W2.T
        dA1 = dY * (T.gelu(A1) if gelu_not_grad else T.gelu_grad(A1))
        return {"dX": dA1 @ W1.T, "dW1": X.T @ dA1,
                "db1": dY.sum(axis=0) if db1_before_gelu else dA1.sum(axis=0),
                "dW2": (A1 if dW2_from_A1 else Y).T @ dZ,
                "db2": dZ.sum(axis=0) if with_db2 else None, "dA1": dA1}
    return f


def _qkv_bwd_db_wrong_axis(X, Wqkv, dQKV):
    return {"dX": dQKV @ Wqkv.T, "dW": X.T @ dQKV, "db": dQKV.mean(axis=0)}


def _grouped_off_by_one(tp_size, rank, group_offsets, X_perm, W1_r, b1_r, W2_r):
    Z = np.zeros((X_perm.shape[0], W2_r.shape[2]))
    for e in range(W1_r.shape[0]):
        lo, hi = int(group_offsets[e]), int(group_offsets[e + 1])
        if hi > lo + 1:
            Z[lo:hi - 1] = T.gelu(X_perm[lo:hi - 1] @ W1_r[e] + b1_r[e]) @ W2_r[e]
    return Z


def _attn_out_rows_at_qkv_offset(Wo, n_heads, tp_size, rank):
    d = Wo.shape[0] // n_heads
    h0, nh = T.shard_range(n_heads, tp_size, rank)
    return Wo[3 * d * h0:3 * d * h0 + d * nh, :]


def _attn_out_fwd_bo_everywhere(tp_size, rank, B, S, H, n_heads, ctx_r, Wo_r, bo):
    return T.attn_out_fwd(ctx_r, Wo_r, bo)


def _attn_out_bwd_dbo_everywhere(tp_size, rank, B, S, H, n_heads, ctx_r, Wo_r, dO):
    return T.attn_out_bwd(ctx_r, Wo_r, dO, with_db=True)


def _attn_out_bwd_untransposed(ctx, Wo, dO, with_db):
    return {"dctx": dO @ Wo[:, :Wo.shape[0]], "dW": ctx.T @ dO, "db": dO.sum(axis=0) if with_db else None}


def _ln_variant(ddof=0, eps_outside=False, over_tokens=False):
    def f(h, gamma, beta, eps):
        ax = 0 if over_tokens else 1
        mean = h.mean(axis=ax, keepdims=True)
        c = h - mean
        var = (c * c).sum(axis=ax, keepdims=True) / (h.shape[ax] - ddof)
        rstd = 1.0 / (np.sqrt(var) + eps) if eps_outside else 1.0 / np.sqrt(var + eps)
        y = c * rstd * gamma + beta
        if over_tokens:
            return y, np.broadcast_to(mean, h.shape)[:, 0], np.broadcast_to(rstd, h.shape)[:, 0]
        return y, mean[:, 0], rstd[:, 0]
    return f


def _ln_bwd_variant(drop_mean=False, drop_proj=False, dgamma_plain=False):
    def f(h, gamma, dy, eps):
        mean = h.mean(axis=1)
        c = h - mean[:, None]
        rstd = 1.0 / np.sqrt((c * c).mean(axis=1) + eps)
        xhat = c * rstd[:, None]
        g = dy * gamma
        t = g.copy()
        if not drop_mean:
            t = t - g.mean(axis=1, keepdims=True)
        if not drop_proj:
            t = t - xhat * (g * xhat).mean(axis=1, keepdims=True)
        return rstd[:, None] * t, (dy if dgamma_plain else dy * xhat).sum(axis=0), dy.sum(axis=0)
    return f


def _dropout_add_unscaled(x, o, keep, p_drop):
    x = np.asarray(x, dtype=np.float64)
    if o is None:
        return x.copy()
    return x + (o if keep is None else o * keep)


def _ln_bwd_ignores_dh_in(tp_size, rank, sp, Tt, H, dy, dh_in, h, gamma, keep, p_drop, eps):
    return _ORIG_LN_BWD(tp_size, rank, sp, Tt, H, dy, None, h, gamma, keep, p_drop, eps)


_ORIG_LN_BWD = T.tp_residual_ln_bwd


def _route_variant(ties_high=False, renorm=False, by_token=False):
    orig = _ORIG_ROUTE

    def f(logits32, top_k):
        lg = np.asarray(logits32, dtype=np.float32)
        if ties_high:
            lg2 = lg[:, ::-1]
            r = orig(lg2, top_k)
            E = lg.shape[1]
            ex = E - 1 - r["experts"]
            # rebuild the rest from the flipped choice with the same bookkeeping
            return _rebuild(lg, ex)
        r = orig(lg, top_k)
        if renorm:
            r["gates"] = r["gates"] / r["gates"].sum(axis=1, keepdims=True)
        if by_token:
            n, k = r["experts"].shape
            r["row_token"] = np.repeat(np.arange(n), k)
            r["token_row"] = np.arange(n * k).reshape(n, k)
        return r
    return f


def _rebuild(lg, experts):
    n, k = experts.shape
    E = lg.shape[1]
    l64 = lg.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    counts = np.bincount(experts.reshape(-1), minlength=E)
    off = np.concatenate([[0], np.cumsum(counts)])
    fill, rt, tr = off[:-1].copy(), np.zeros(n * k, dtype=np.int64), np.zeros((n, k), dtype=np.int64)
    for t in range(n):
        for j in range(k):
            e = experts[t, j]
            rt[fill[e]] = t
            tr[t, j] = fill[e]
            fill[e] += 1
    return {"gates": np.take_along_axis(p, experts, axis=1), "experts": experts, "group_offsets": off,
            "row_token": rt, "token_row": tr}


def _combine_first_choice_only(Z_rows, gates, token_row):
    return gates[:, :1] * Z_rows[token_row[:, 0]]


_ORIG_ROUTE = T.moe_route


def _fp8_decode_bias8(codes, fmt="e4m3"):
    v = _ORIG_DECODE(codes, fmt)
    return v / 2.0 if fmt == "e4m3" else v


def _fp8_encode_ties_up(y, fmt="e4m3"):
    vmax = T._fp8_format(fmt)[3]
    pos = T._FP8_POS[fmt]
    fin = pos[:int(np.searchsorted(pos, vmax, side="right"))]
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), vmax)
    hi = np.clip(np.searchsorted(fin, a, side="left"), 0, len(fin) - 1)
    lo = np.maximum(hi - 1, 0)
    pick = np.where(fin[hi] - a <= a - fin[lo], hi, lo)
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def _fp8_quantize_descale_inverted(x, transpose=False, fmt="e4m3"):
    q, d = _ORIG_QUANT(x, transpose, fmt)
    return q, np.float32(1) / d


def _fp8_gemm_dgelu_uses_gelu(A_codes, a_descale, B_codes, b_descale, bias=None, epi=0, aux=None, fmt_a="e4m3",
                              fmt_b="e4m3"):
    r = _ORIG_GEMM(A_codes, a_descale, B_codes, b_descale, bias, epi, aux, fmt_a, fmt_b)
    if epi == T.FP8_EPI_DGELU:
        r["C"] = r["pre"] * T.gelu(np.asarray(aux))
    return r


_ORIG_DECODE = T.fp8_decode
_ORIG_QUANT = T.fp8_quantize
_ORIG_GEMM = T.fp8_gemm_nt


def _gelu_tanh_cubic_dropped(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * x))


def _combine_bwd_ungated(d_out, Z_rows, gates, token_row):
    r = _ORIG_COMBINE_BWD(d_out, Z_rows, gates, token_row)
    for j in range(gates.shape[1]):
        r["dZ"][token_row[:, j]] = d_out
    return r


def _route_bwd_no_softmax_coupling(logits32, experts, dgates):
    l64 = np.asarray(logits32, dtype=np.float32).astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dl = np.zeros(p.shape)
    for j in range(experts.shape[1]):
        np.put_along_axis(dl, experts[:, j:j + 1], (dgates[:, j] * np.take_along_axis(p, experts[:, j:j + 1], 1)[:, 0])[:, None], 1)
    return dl


def _moe_bwd_dX_first_choice(tp_size, rank, X, route, W1_r, W2_r, fwd, d_out):
    r = _ORIG_MOE_BWD(tp_size, rank, X, route, W1_r, W2_r, fwd, d_out)
    Xp = np.asarray(X)[route["row_token"]]
    gb = T.tp_mlp_grouped_shard_bwd(route["group_offsets"], Xp, W1_r, W2_r, fwd["A1"], fwd["Y"], r["dZ"])
    r["dX"] = gb["dX_perm"][route["token_row"][:, 0]]
    return r


_ORIG_COMBINE_BWD = T.moe_combine_bwd
_ORIG_MOE_BWD = T.tp_moe_shard_bwd


def _normwise_den_from_got(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(got)
    return np.linalg.norm(got - ref) / den if den > 0 else np.linalg.norm(got - ref)


def _normwise_max_norm(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    return np.abs(got - ref).max() / den if den > 0 else np.abs(got - ref).max()


def _blockwise_is_normwise(got, ref, block=64):
    return T.normwise_error(got, ref)


def _blockwise_own_norm_only(got, ref, block=64):
    g, r = T._as_rows(got), T._as_rows(ref)
    worst = 0.0
    for i in range(0, r.shape[0], block):
        for j in range(0, r.shape[1], block):
            rb, gb = r[i:i + block, j:j + block], g[i:i + block, j:j + block]
            den = np.linalg.norm(rb)
            worst = max(worst, np.linalg.norm(gb - rb) / den if den > 0 else np.linalg.norm(gb - rb))
    return worst


MUTANTS = {
    "gelu_tanh_approx": {"gelu": _gelu_tanh},
    "gelu_grad_drops_x_phi": {"gelu_grad": _gelu_grad_no_density},
    "scale_1_over_d": {"_softmax_causal": _softmax_variant(scale=lambda d: d)},
    "mask_sees_next_key": {"_softmax_causal": _softmax_variant(mask_k=1)},
    "mask_strict": {"_softmax_causal": _softmax_variant(mask_k=-1)},
    "no_causal_mask": {"_softmax_causal": _softmax_variant(no_mask=True)},
    "lse_without_max": {"_softmax_causal": _softmax_variant(lse_without_max=True)},
    "qkv_blocked_layout": {"_heads": _heads_blocked},
    "remainder_to_last_rank": {"shard_range": _shard_range_last_takes_rest},
    "b2_on_every_rank": {"tp_mlp_shard_fwd": _mlp_fwd_b2_everywhere},
    "fc1_bias_dropped": {"mlp_fwd": _mlp_fwd_no_b1},
    "attn_bwd_drops_D": {"attention_bwd": _attn_bwd_variant(drop_D=True)},
    "attn_bwd_dK_untransposed": {"attention_bwd": _attn_bwd_variant(dK_untransposed=True)},
    "attn_bwd_dQ_unscaled": {"attention_bwd": _attn_bwd_variant(dQ_unscaled=True)},
    "attn_bwd_dV_untransposed": {"attention_bwd": _attn_bwd_variant(dV_wrong=True)},
    "mlp_bwd_gelu_for_grad": {"mlp_bwd": _mlp_bwd_variant(gelu_not_grad=True)},
    "mlp_bwd_db1_before_gelu": {"mlp_bwd": _mlp_bwd_variant(db1_before_gelu=True)},
    "mlp_bwd_dW2_from_A1": {"mlp_bwd": _mlp_bwd_variant(dW2_from_A1=True)},
    "qkv_bwd_db_mean": {"qkv_bwd": _qkv_bwd_db_wrong_axis},
    "grouped_drops_last_row": {"tp_mlp_grouped_shard_fwd": _grouped_off_by_one},
    "attn_out_rows_at_qkv_offset": {"slice_attn_out": _attn_out_rows_at_qkv_offset},
    "attn_out_bo_on_every_rank": {"tp_attn_out_shard_fwd": _attn_out_fwd_bo_everywhere},
    "attn_out_dbo_on_every_rank": {"tp_attn_out_shard_bwd": _attn_out_bwd_dbo_everywhere},
    "attn_out_bwd_untransposed": {"attn_out_bwd": _attn_out_bwd_untransposed},
    "ln_unbiased_variance": {"layernorm": _ln_variant(ddof=1)},
    "ln_eps_outside_sqrt": {"layernorm": _ln_variant(eps_outside=True)},
    "ln_stats_over_tokens": {"layernorm": _ln_variant(over_tokens=True)},
    "ln_bwd_drops_mean_term": {"layernorm_bwd": _ln_bwd_variant(drop_mean=True)},
    "ln_bwd_drops_projection": {"layernorm_bwd": _ln_bwd_variant(drop_proj=True)},
    "ln_bwd_dgamma_without_xhat": {"layernorm_bwd": _ln_bwd_variant(dgamma_plain=True)},
    "dropout_without_rescale": {"dropout_add": _dropout_add_unscaled},
    "ln_bwd_ignores_residual_grad": {"tp_residual_ln_bwd": _ln_bwd_ignores_dh_in},
    "moe_ties_to_higher_id": {"moe_route": _route_variant(ties_high=True)},
    "moe_gates_renormalised": {"moe_route": _route_variant(renorm=True)},
    "moe_rows_in_token_order": {"moe_route": _route_variant(by_token=True)},
    "moe_combine_first_choice_only": {"moe_combine": _combine_first_choice_only},
    "e4m3_exponent_bias_8": {"fp8_decode": _fp8_decode_bias8},
    "fp8_ties_away": {"fp8_encode": _fp8_encode_ties_up},
    "fp8_descale_inverted": {"fp8_quantize": _fp8_quantize_descale_inverted},
    "fp8_dgelu_uses_gelu": {"fp8_gemm_nt": _fp8_gemm_dgelu_uses_gelu},
    "gelu_tanh_cubic_dropped": {"gelu_tanh": _gelu_tanh_cubic_dropped},
    "moe_combine_bwd_ungated": {"moe_combine_bwd": _combine_bwd_ungated},
    "moe_route_bwd_no_softmax_coupling": {"moe_route_bwd": _route_bwd_no_softmax_coupling},
    "moe_bwd_dX_first_choice_only": {"tp_moe_shard_bwd": _moe_bwd_dX_first_choice},
    "normwise_denominator_from_got": {"normwise_error": _normwise_den_from_got},
    "normwise_max_norm": {"normwise_error": _normwise_max_norm},
    "blockwise_is_normwise": {"blockwise_error": _blockwise_is_normwise},
    "blockwise_own_norm_only": {"blockwise_error": _blockwise_own_norm_only},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name].items():
        assert hasattr(T, attr), attr
        monkeypatch.setattr(T, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in P.ALL_PINS:
            try:
                pin()
            except Exception as e:          # an assertion or a crash both reveal the mistake
                caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutant {name} passed every pin"
