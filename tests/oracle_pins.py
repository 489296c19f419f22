"""Pins of the fp64 oracle against things other than itself.

Each pin raises AssertionError on failure.  Pins look the oracle's functions up on the module at call
time, so tests/test_oracle_mutations.py can plant a mistake in the oracle and check that some pin
fails.  What pins what:

  geometry    golden fixture (the workloads' stated splits) + invariants (cover, contiguous, balanced)
  gelu        textbook normal-CDF values; odd-part identity; derivative by central differences
  brute       pure-Python scalar loops (tests/bruteforce.py) on the tiny layer, both ranks
  identities  column split X·[W1 W2] = [X·W1, X·W2]; row split Σ_r Z_r = Z and Σ_r O_r = O (the
              attention output projection); Σ_r dX_r = dX; dctx and weight-gradient blocks; tp=1
              equals the unsharded layer
  closed      attention closed forms: S=1, query 0, Q=0 (prefix mean, LSE = log(i+1)), constant keys
              (LSE = q·k/√d + log(i+1)), one dominant key, dV for Q=0
  fd          central finite differences in fp64 for every gradient output
  moe         routing against numpy's stable argsort, exact ties to the lower id, permutation and
              inverse invariants, gates summing to 1 when k = E; the whole MoE block against scalar
              per-token loops; E = k = 1 equals the dense MLP shard; Σ over TP ranks = unsharded
  fp8         E4M3 anchors from the format's definition; every finite code against torch's
              float8_e4m3fn; encode(decode(c)) = c; midpoints to the even code; saturation; the
              amax element quantises to ±448; the GEMM on codes against scalar loops
  checkers    normwise_error and blockwise_error (the parity measures) against hand-worked values;
              a planted one-tile GEMM defect that the normwise measure misses and the tile-wise one
              catches
  layernorm   scalar loops; a textbook row; zero mean / unit mean square (eps = 0); shift and scale
              invariance; constant rows; dropout-add cases by hand; finite differences through the
              fused residual + dropout + LayerNorm op; the sequence-parallel split (row blocks
              concatenate, dγ / dβ partials sum)
"""

import math
import os

import numpy as np

import oracle.tp_shard as T
import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    den = max(np.linalg.norm(b), 1e-300)
    err = np.linalg.norm(a - b) / den
    assert err <= tol, f"{what}: normwise error {err:.3e} > {tol:.1e}"


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append([float(x) for x in line.split()])
    return rows


def _rng(seed):
    return np.random.default_rng(seed)


# ---- geometry ---------------------------------------------------------------------------------

def pin_geometry():
    for n, t, r, off, cnt in _read_table("shard_geometry.txt"):
        got = T.shard_range(int(n), int(t), int(r))
        assert got == (int(off), int(cnt)), f"shard_range({n},{t},{r}) = {got}"
    for n in range(0, 40):
        for t in range(1, 10):
            parts = [T.shard_range(n, t, r) for r in range(t)]
            assert sum(c for _, c in parts) == n
            assert parts[0][0] == 0
            for (o0, c0), (o1, _) in zip(parts, parts[1:]):
                assert o1 == o0 + c0, "blocks must be contiguous"
            counts = [c for _, c in parts]
            assert max(counts) - min(counts) <= 1
            assert counts == sorted(counts, reverse=True), "lower ranks take the remainder"
    assert T.qkv_column_range(25, 64, 2, 1) == (13 * 192, 25 * 192)


# ---- GeLU ---------------------------------------------------------------------------------------

def pin_gelu():
    for x, phi_cdf in _read_table("normal_cdf.txt"):
        assert abs(float(T.gelu(x)) - x * phi_cdf) <= 1e-13, f"GeLU({x})"
        dens = math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
        assert abs(float(T.gelu_grad(x)) - (phi_cdf + x * dens)) <= 1e-13, f"GeLU'({x})"
    xs = np.linspace(-6, 6, 241)
    assert np.allclose(T.gelu(xs) - T.gelu(-xs), xs, rtol=0, atol=1e-13), "odd-part identity"
    assert float(T.gelu(0.0)) == 0.0 and abs(float(T.gelu_grad(0.0)) - 0.5) < 1e-15
    eps = 1e-5
    fd = (T.gelu(xs + eps) - T.gelu(xs - eps)) / (2 * eps)
    assert np.max(np.abs(fd - T.gelu_grad(xs))) < 1e-9, "GeLU' vs central differences"
    assert abs(float(T.gelu(12.0)) - 12.0) < 1e-12 and abs(float(T.gelu(-12.0))) < 1e-12
    # the tanh form: its defining value at 1 (tanh(√(2/π)·1.044715) from the standard library),
    # the odd-part identity (tanh is odd), closeness to the exact GeLU, its derivative by differences
    t1 = 0.5 * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * 1.044715))
    assert abs(float(T.gelu_tanh(1.0)) - t1) < 1e-15 and abs(t1 - 0.8411919906082768) < 1e-13
    assert np.allclose(T.gelu_tanh(xs) - T.gelu_tanh(-xs), xs, rtol=0, atol=1e-13), "tanh form: odd part"
    assert np.max(np.abs(T.gelu_tanh(xs) - T.gelu(xs))) < 1e-3, "tanh form within 1e-3 of the exact GeLU"
    assert np.max(np.abs(T.gelu_tanh(xs) - T.gelu(xs))) > 1e-5, "and not equal to it"
    fdt = (T.gelu_tanh(xs + eps) - T.gelu_tanh(xs - eps)) / (2 * eps)
    assert np.max(np.abs(fdt - T.gelu_tanh_grad(xs))) < 1e-9, "tanh form derivative vs central differences"
    # the MLP with the tanh form uses it in both directions
    g = _rng(81)
    X, W1, b1, W2 = g.standard_normal((3, 4)), g.standard_normal((4, 5)), g.standard_normal(5), g.standard_normal((5, 2))
    fw = T.mlp_fwd(X, W1, b1, W2, None, activation=1)
    _close(fw["Y"], T.gelu_tanh(X @ W1 + b1), 1e-15, "tanh-form MLP forward")
    dZ = g.standard_normal((3, 2))
    bw = T.mlp_bwd(X, W1, W2, fw["A1"], fw["Y"], dZ, False, activation=1)
    want = _fd_dir(lambda z: float((T.mlp_fwd(X, z, b1, W2, None, activation=1)["Z"] * dZ).sum()), W1,
                   np.ones_like(W1))
    assert abs(float(bw["dW1"].sum()) - want) < 1e-7 * max(1, abs(want)), "tanh-form backward by differences"


# ---- tiny layer --------------------------------------------------------------------------------

TINY = dict(B=2, S=32, H=64, nh=4, F=256, t=2)


def _tiny_full(seed=7, wstd=0.02, bstd=0.02, xstd=1.0, H=None, nh=None, F=None, B=None, S=None):
    cfg = dict(TINY)
    for k, v in dict(H=H, nh=nh, F=F, B=B, S=S).items():
        if v is not None:
            cfg[k] = v
    g = _rng(seed)
    Tt, H, F = cfg["B"] * cfg["S"], cfg["H"], cfg["F"]
    p = dict(
        X=g.standard_normal((Tt, H)) * xstd,
        Wqkv=g.standard_normal((H, 3 * H)) * wstd, bqkv=g.standard_normal(3 * H) * bstd,
        W1=g.standard_normal((H, F)) * wstd, b1=g.standard_normal(F) * bstd,
        W2=g.standard_normal((F, H)) * wstd, b2=g.standard_normal(H) * bstd)
    p.update(Wo=g.standard_normal((H, H)) * wstd, bo=g.standard_normal(H) * bstd)
    return cfg, p


def pin_brute_forward():
    cfg, p = _tiny_full()
    B, S, H, nh, F, t = (cfg[k] for k in ("B", "S", "H", "nh", "F", "t"))
    d = H // nh
    for r in range(t):
        Wq, bq = T.slice_qkv(p["Wqkv"], p["bqkv"], nh, t, r)
        qkv = T.tp_qkv_shard_fwd(t, r, B, S, H, nh, p["X"], Wq, bq)
        _close(qkv, bf.matmul_bias(p["X"], Wq, bq), 1e-13, f"QKV r{r}")
        # sharper scores than the layer's own weights give, so the softmax is far from flat
        sharp = qkv * 12.0
        ctx, lse = T.tp_attn_heads_fwd(t, r, B, S, H, nh, sharp)
        _, nh_r = T.shard_range(nh, t, r)
        bctx, blse = bf.attention(sharp, B, S, nh_r, d)
        _close(ctx, bctx, 1e-13, f"ctx r{r}")
        _close(lse, blse, 1e-13, f"lse r{r}")
        Wo = T.slice_attn_out(p["Wo"], nh, t, r)
        O = T.tp_attn_out_shard_fwd(t, r, B, S, H, nh, ctx, Wo, p["bo"])
        _close(O, bf.matmul_bias(ctx, Wo, p["bo"] if r == 0 else None), 1e-13, f"O r{r}")
        W1, b1 = T.slice_fc1(p["W1"], p["b1"], t, r)
        W2 = T.slice_fc2(p["W2"], t, r)
        out = T.tp_mlp_shard_fwd(t, r, B * S, H, F, p["X"] * 20.0, W1, b1, W2, p["b2"])
        A1, Y, Z = bf.mlp_forward(p["X"] * 20.0, W1, b1, W2, p["b2"] if r == 0 else None)
        _close(out["A1"], A1, 1e-13, f"A1 r{r}")
        _close(out["Y"], Y, 1e-13, f"Y r{r}")
        _close(out["Z"], Z, 1e-13, f"Z r{r}")


def pin_brute_backward():
    g = _rng(11)
    Tt, H, F, t = 8, 16, 32, 2
    X = g.standard_normal((Tt, H))
    W1, b1 = g.standard_normal((H, F)) * 0.3, g.standard_normal(F) * 0.3
    W2 = g.standard_normal((F, H)) * 0.3
    dZ = g.standard_normal((Tt, H))
    for r in range(t):
        W1r, b1r = T.slice_fc1(W1, b1, t, r)
        W2r = T.slice_fc2(W2, t, r)
        fw = T.tp_mlp_shard_fwd(t, r, Tt, H, F, X, W1r, b1r, W2r, None)
        got = T.tp_mlp_shard_bwd(t, r, Tt, H, F, X, W1r, W2r, fw["A1"], fw["Y"], dZ)
        ref = bf.mlp_backward(X, W1r, W2r, fw["A1"], fw["Y"], dZ)
        for k in ("dX", "dW1", "db1", "dW2"):
            _close(got[k], ref[k], 1e-13, f"MLP {k} r{r}")
        if r == 0:
            _close(got["db2"], ref["db2"], 1e-13, "db2 r0")
        else:
            assert got["db2"] is None, "db2 belongs to rank 0 only"
    B, S, nh = 1, 8, 4
    d = H // nh
    Wqkv = g.standard_normal((H, 3 * H)) * 0.3
    for r in range(t):
        Wq, _ = T.slice_qkv(Wqkv, np.zeros(3 * H), nh, t, r)
        dQKV = g.standard_normal((B * S, Wq.shape[1]))
        got = T.tp_qkv_shard_bwd(t, r, B, S, H, nh, X, Wq, dQKV)
        ref = bf.linear_backward(X, Wq, dQKV)
        for k in ("dX", "dW", "db"):
            _close(got[k], ref[k], 1e-13, f"QKV {k} r{r}")
    Wo = g.standard_normal((H, H)) * 0.3
    dO = g.standard_normal((B * S, H))
    for r in range(t):
        Wor = T.slice_attn_out(Wo, nh, t, r)
        ctx = g.standard_normal((B * S, Wor.shape[0]))
        got = T.tp_attn_out_shard_bwd(t, r, B, S, H, nh, ctx, Wor, dO)
        ref = bf.linear_backward(ctx, Wor, dO)
        _close(got["dctx"], ref["dX"], 1e-13, f"out-proj dctx r{r}")
        _close(got["dW"], ref["dW"], 1e-13, f"out-proj dWo r{r}")
        if r == 0:
            _close(got["db"], ref["db"], 1e-13, "out-proj dbo r0")
        else:
            assert got["db"] is None, "dbo belongs to rank 0 only"


# ---- identities -------------------------------------------------------------------------------

def _run_ranks(cfg, p, t):
    B, S, H, nh, F = (cfg[k] for k in ("B", "S", "H", "nh", "F"))
    outs = []
    for r in range(t):
        Wq, bq = T.slice_qkv(p["Wqkv"], p["bqkv"], nh, t, r)
        qkv = T.tp_qkv_shard_fwd(t, r, B, S, H, nh, p["X"], Wq, bq)
        ctx, lse = T.tp_attn_heads_fwd(t, r, B, S, H, nh, qkv)
        W1, b1 = T.slice_fc1(p["W1"], p["b1"], t, r)
        W2 = T.slice_fc2(p["W2"], t, r)
        mlp = T.tp_mlp_shard_fwd(t, r, B * S, H, F, p["X"], W1, b1, W2, p["b2"])
        Wo = T.slice_attn_out(p["Wo"], nh, t, r)
        O = T.tp_attn_out_shard_fwd(t, r, B, S, H, nh, ctx, Wo, p["bo"])
        outs.append(dict(qkv=qkv, ctx=ctx, lse=lse, **mlp, W1=W1, W2=W2, Wq=Wq, Wo=Wo, O=O))
    return outs


def pin_identities():
    for (H, nh, F, t) in ((64, 4, 256, 2), (48, 6, 100, 4), (50, 5, 90, 3), (64, 4, 256, 1)):
        cfg, p = _tiny_full(seed=3, H=H, nh=nh, F=F, B=2, S=12, wstd=0.2, bstd=0.1)
        B, S = cfg["B"], cfg["S"]
        d = H // nh
        full = T.layer_fwd(p["X"], p["Wqkv"], p["bqkv"], p["W1"], p["b1"], p["W2"], p["b2"], B, S, nh,
                           p["Wo"], p["bo"])
        outs = _run_ranks(cfg, p, t)
        # column identity: QKV, ctx, lse, A1, Y are column blocks of the unsharded results
        _close(np.concatenate([o["qkv"] for o in outs], 1), full["QKV"], 1e-13, "QKV concat")
        _close(np.concatenate([o["ctx"] for o in outs], 1), full["ctx"], 1e-13, "ctx concat")
        _close(np.concatenate([o["lse"] for o in outs], 1), full["lse"], 1e-13, "lse concat")
        _close(np.concatenate([o["A1"] for o in outs], 1), full["A1"], 1e-13, "A1 concat")
        _close(np.concatenate([o["Y"] for o in outs], 1), full["Y"], 1e-13, "Y concat")
        # row identity: the partials sum to the unsharded output
        _close(sum(o["Z"] for o in outs), full["Z"], 1e-13, f"sum Z_r (t={t})")
        _close(sum(o["O"] for o in outs), full["O"], 1e-13, f"sum O_r (t={t})")
        # the unsharded output projection, from its definition written out per head: the heads'
        # contexts each times their own d rows of Wo, summed, plus the bias once
        per_head = sum(full["ctx"][:, h * d:(h + 1) * d] @ p["Wo"][h * d:(h + 1) * d] for h in range(nh))
        _close(full["O"], per_head + p["bo"], 1e-13, "O as a sum over heads")
        # backward: weight-gradient blocks and input-gradient partials
        g = _rng(5)
        dZ = g.standard_normal((B * S, H))
        dctx = g.standard_normal((B * S, H))
        fullm = T.mlp_bwd(p["X"], p["W1"], p["W2"], full["A1"], full["Y"], dZ, True)
        d_full_attn = T.attention_bwd(full["QKV"], dctx, B, S, nh, d)
        fullq = T.qkv_bwd(p["X"], p["Wqkv"], d_full_attn)
        dXm = np.zeros_like(p["X"])
        dXq = np.zeros_like(p["X"])
        dW1s, dW2s, db1s, dWqs, dbqs, dqkvs = [], [], [], [], [], []
        for r, o in enumerate(outs):
            m = T.tp_mlp_shard_bwd(t, r, B * S, H, F, p["X"], o["W1"], o["W2"], o["A1"], o["Y"], dZ)
            h0, nhr = T.shard_range(nh, t, r)
            dq = T.tp_attn_heads_bwd(t, r, B, S, H, nh, o["qkv"], dctx[:, h0 * d:(h0 + nhr) * d])
            q = T.tp_qkv_shard_bwd(t, r, B, S, H, nh, p["X"], o["Wq"], dq)
            dXm += m["dX"]
            dXq += q["dX"]
            dW1s.append(m["dW1"]); dW2s.append(m["dW2"]); db1s.append(m["db1"])
            dWqs.append(q["dW"]); dbqs.append(q["db"]); dqkvs.append(dq)
            if r == 0:
                _close(m["db2"], fullm["db2"], 1e-13, "db2")
        _close(dXm, fullm["dX"], 1e-13, "sum dX_r (MLP)")
        _close(dXq, fullq["dX"], 1e-13, "sum dX_r (QKV)")
        _close(np.concatenate(dW1s, 1), fullm["dW1"], 1e-13, "dW1 blocks")
        _close(np.concatenate(db1s), fullm["db1"], 1e-13, "db1 blocks")
        _close(np.concatenate(dW2s, 0), fullm["dW2"], 1e-13, "dW2 blocks")
        _close(np.concatenate(dqkvs, 1), d_full_attn, 1e-13, "dQKV blocks")
        _close(np.concatenate(dWqs, 1), fullq["dW"], 1e-13, "dWqkv blocks")
        _close(np.concatenate(dbqs), fullq["db"], 1e-13, "dbqkv blocks")
        # output projection backward: dctx_r is the rank's column block of dctx (no sum), dWo_r its
        # row block of dWo, dbo from rank 0 only
        dO = g.standard_normal((B * S, H))
        fullo = T.attn_out_bwd(full["ctx"], p["Wo"], dO, True)
        ob = [T.tp_attn_out_shard_bwd(t, r, B, S, H, nh, o["ctx"], o["Wo"], dO) for r, o in enumerate(outs)]
        _close(np.concatenate([b["dctx"] for b in ob], 1), fullo["dctx"], 1e-13, "dctx blocks")
        _close(np.concatenate([b["dW"] for b in ob], 0), fullo["dW"], 1e-13, "dWo blocks")
        _close(ob[0]["db"], fullo["db"], 1e-13, "dbo")
        assert all(b["db"] is None for b in ob[1:]), "dbo belongs to rank 0 only"


# ---- attention closed forms --------------------------------------------------------------------

def _qkv_from(q, k, v):
    """Assemble the interleaved [B*S, 3*nh*d] matrix from per-head q, k, v [B, nh, S, d]."""
    B, nh, S, d = q.shape
    t = np.stack([q, k, v], axis=3)              # [B, nh, S, 3, d]
    return t.transpose(0, 2, 1, 3, 4).reshape(B * S, nh * 3 * d)


def pin_attention_closed_forms():
    g = _rng(21)
    B, nh, S, d = 2, 3, 9, 8
    q, k, v = (g.standard_normal((B, nh, S, d)) for _ in range(3))
    # S = 1: ctx = v, LSE = q·k/√d
    ctx, lse = T.attention_fwd(_qkv_from(q[:, :, :1], k[:, :, :1], v[:, :, :1]), B, 1, nh, d)
    _close(ctx.reshape(B, 1, nh, d).transpose(0, 2, 1, 3), v[:, :, :1], 1e-15, "S=1 ctx")
    _close(lse[:, :, 0], (q[:, :, 0] * k[:, :, 0]).sum(-1) / math.sqrt(d), 1e-15, "S=1 lse")
    # query 0 sees only key 0
    ctx, lse = T.attention_fwd(_qkv_from(q, k, v), B, S, nh, d)
    c = ctx.reshape(B, S, nh, d).transpose(0, 2, 1, 3)
    _close(c[:, :, 0], v[:, :, 0], 1e-15, "row 0 ctx")
    # Q = 0: uniform weights over the visible prefix, LSE = log(i+1)
    ctx, lse = T.attention_fwd(_qkv_from(np.zeros_like(q), k, v), B, S, nh, d)
    c = ctx.reshape(B, S, nh, d).transpose(0, 2, 1, 3)
    prefix = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    _close(c, prefix, 1e-14, "Q=0 prefix mean")
    _close(lse, np.broadcast_to(np.log(np.arange(1, S + 1)), lse.shape), 1e-14, "Q=0 LSE")
    # all keys equal: uniform weights, LSE_i = q_i·k/√d + log(i+1)  (pins the 1/√d scale)
    kc = np.broadcast_to(k[:, :, :1], k.shape).copy()
    ctx, lse = T.attention_fwd(_qkv_from(q, kc, v), B, S, nh, d)
    c = ctx.reshape(B, S, nh, d).transpose(0, 2, 1, 3)
    _close(c, prefix, 1e-13, "constant-key prefix mean")
    want = (q * kc).sum(-1) / math.sqrt(d) + np.log(np.arange(1, S + 1))[None, None, :]
    _close(lse, want, 1e-13, "constant-key LSE")
    # one dominant visible key: ctx_i -> v_j* for i >= j*, while queries before j* cannot see it
    jstar = 4
    kd = k.copy() * 0.01
    kd[:, :, jstar] = 0.0
    kd[:, :, jstar, 0] = 1.0
    qd = np.zeros_like(q)
    qd[..., 0] = 400.0
    ctx, _ = T.attention_fwd(_qkv_from(qd, kd, v), B, S, nh, d)
    c = ctx.reshape(B, S, nh, d).transpose(0, 2, 1, 3)
    _close(c[:, :, jstar:], np.broadcast_to(v[:, :, jstar:jstar + 1], c[:, :, jstar:].shape), 1e-12,
           "dominant key")
    assert np.max(np.abs(c[:, :, :jstar] - v[:, :, jstar:jstar + 1])) > 0.1, "future key leaked"
    # backward with Q = 0: dV_j = Σ_{i>=j} dO_i / (i+1)
    dO = g.standard_normal((B, S, nh, d))
    dqkv = T.attention_bwd(_qkv_from(np.zeros_like(q), k, v), dO.reshape(B * S, nh * d), B, S, nh, d)
    dv = dqkv.reshape(B, S, nh, 3, d)[:, :, :, 2, :]
    w = dO / np.arange(1, S + 1)[None, :, None, None]
    want_dv = np.flip(np.cumsum(np.flip(w, axis=1), axis=1), axis=1)
    _close(dv, want_dv, 1e-13, "Q=0 dV")


# ---- finite differences -----------------------------------------------------------------------

def _fd_dir(f, x, v, eps=1e-6):
    return (f(x + eps * v) - f(x - eps * v)) / (2 * eps)


def pin_finite_differences():
    g = _rng(31)
    Tt, H, F, t = 6, 8, 12, 2
    X = g.standard_normal((Tt, H))
    W1, b1 = g.standard_normal((H, F)) * 0.5, g.standard_normal(F) * 0.5
    W2, b2 = g.standard_normal((F, H)) * 0.5, g.standard_normal(H) * 0.5
    dZ = g.standard_normal((Tt, H))
    for r in range(t):
        W1r, b1r = T.slice_fc1(W1, b1, t, r)
        W2r = T.slice_fc2(W2, t, r)

        def loss(X_=X, W1_=W1r, b1_=b1r, W2_=W2r, b2_=b2):
            return float((T.tp_mlp_shard_fwd(t, r, Tt, H, F, X_, W1_, b1_, W2_, b2_)["Z"] * dZ).sum())

        fw = T.tp_mlp_shard_fwd(t, r, Tt, H, F, X, W1r, b1r, W2r, b2)
        gr = T.tp_mlp_shard_bwd(t, r, Tt, H, F, X, W1r, W2r, fw["A1"], fw["Y"], dZ)
        for name, x0, grad, call in (
                ("dX", X, gr["dX"], lambda z: loss(X_=z)),
                ("dW1", W1r, gr["dW1"], lambda z: loss(W1_=z)),
                ("db1", b1r, gr["db1"], lambda z: loss(b1_=z)),
                ("dW2", W2r, gr["dW2"], lambda z: loss(W2_=z))):
            for _ in range(3):
                vdir = g.standard_normal(x0.shape)
                want = _fd_dir(call, x0, vdir)
                got = float((grad * vdir).sum())
                assert abs(got - want) <= 1e-7 * max(1.0, abs(want)), f"FD {name} r{r}: {got} vs {want}"
        vdir = g.standard_normal(b2.shape)
        want = _fd_dir(lambda z: loss(b2_=z), b2, vdir)
        if r == 0:
            assert abs(float((gr["db2"] * vdir).sum()) - want) <= 1e-7 * max(1, abs(want)), "FD db2"
        else:
            assert abs(want) < 1e-9, "b2 must not enter a rank other than 0"
    # QKV projection
    B, S, nh = 1, 6, 2
    Wq, bq = g.standard_normal((H, 3 * H)) * 0.5, g.standard_normal(3 * H) * 0.5
    dQ = g.standard_normal((B * S, 3 * H))
    gq = T.tp_qkv_shard_bwd(1, 0, B, S, H, nh, X, Wq, dQ)
    for name, x0, grad, call in (
            ("dX", X, gq["dX"], lambda z: float((T.tp_qkv_shard_fwd(1, 0, B, S, H, nh, z, Wq, bq) * dQ).sum())),
            ("dW", Wq, gq["dW"], lambda z: float((T.tp_qkv_shard_fwd(1, 0, B, S, H, nh, X, z, bq) * dQ).sum())),
            ("db", bq, gq["db"], lambda z: float((T.tp_qkv_shard_fwd(1, 0, B, S, H, nh, X, Wq, z) * dQ).sum()))):
        vdir = g.standard_normal(x0.shape)
        want = _fd_dir(call, x0, vdir)
        got = float((grad * vdir).sum())
        assert abs(got - want) <= 1e-7 * max(1.0, abs(want)), f"FD QKV {name}"
    # attention output projection, each rank of a 2-way split
    B, S, nh, Ho = 1, 5, 4, 8
    Wo, bo = g.standard_normal((Ho, Ho)) * 0.5, g.standard_normal(Ho) * 0.5
    dO = g.standard_normal((B * S, Ho))
    for r in range(2):
        Wor = T.slice_attn_out(Wo, nh, 2, r)
        ctx = g.standard_normal((B * S, Wor.shape[0]))
        go = T.tp_attn_out_shard_bwd(2, r, B, S, Ho, nh, ctx, Wor, dO)

        def oloss(c=ctx, w=Wor, b=bo):
            return float((T.tp_attn_out_shard_fwd(2, r, B, S, Ho, nh, c, w, b) * dO).sum())

        for name, x0, grad, call in (("dctx", ctx, go["dctx"], lambda z: oloss(c=z)),
                                     ("dWo", Wor, go["dW"], lambda z: oloss(w=z))):
            vdir = g.standard_normal(x0.shape)
            want = _fd_dir(call, x0, vdir)
            got = float((grad * vdir).sum())
            assert abs(got - want) <= 1e-7 * max(1.0, abs(want)), f"FD out-proj {name} r{r}"
        vdir = g.standard_normal(bo.shape)
        want = _fd_dir(lambda z: oloss(b=z), bo, vdir)
        if r == 0:
            assert abs(float((go["db"] * vdir).sum()) - want) <= 1e-7 * max(1, abs(want)), "FD dbo"
        else:
            assert abs(want) < 1e-9, "bo must not enter a rank other than 0"
    # attention, a mild and a sharp case, every component checked through random directions
    for scale in (1.0, 3.0):
        B, S, nh, d = 2, 7, 2, 4
        qkv = g.standard_normal((B * S, 3 * nh * d)) * scale
        dctx = g.standard_normal((B * S, nh * d))
        H2 = nh * d
        grad = T.tp_attn_heads_bwd(1, 0, B, S, H2, nh, qkv, dctx)

        def aloss(z):
            return float((T.tp_attn_heads_fwd(1, 0, B, S, H2, nh, z)[0] * dctx).sum())

        for part in range(3):          # q, k, v columns separately
            mask = np.zeros((B * S, nh, 3, d))
            mask[:, :, part, :] = 1.0
            vdir = g.standard_normal(qkv.shape) * mask.reshape(qkv.shape)
            want = _fd_dir(aloss, qkv, vdir)
            got = float((grad * vdir).sum())
            assert abs(got - want) <= 1e-7 * max(1.0, abs(want)), f"FD attention part {part} x{scale}"


def pin_grouped():
    """Grouped expert shards = the dense MLP shard applied per expert to its rows (no bias on fc2)."""
    g = _rng(41)
    G, H, Fr = 4, 8, 6
    offsets = np.array([0, 3, 3, 10, 12])
    Xp = g.standard_normal((12, H))
    W1 = g.standard_normal((G, H, Fr)) * 0.4
    b1 = g.standard_normal((G, Fr)) * 0.4
    W2 = g.standard_normal((G, Fr, H)) * 0.4
    Z = T.tp_mlp_grouped_shard_fwd(8, 0, offsets, Xp, W1, b1, W2)
    for e in range(G):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            _, _, ref = bf.mlp_forward(Xp[lo:hi], W1[e], b1[e], W2[e], None)
            _close(Z[lo:hi], ref, 1e-13, f"expert {e}")


def pin_layernorm():
    g = _rng(51)
    # scalar loops
    h = g.standard_normal((5, 7)) * 3.0 + 1.5
    gam, bet = g.standard_normal(7), g.standard_normal(7)
    y, mean, rstd = T.layernorm(h, gam, bet, 1e-5)
    by, bm, br = bf.layernorm(h, gam, bet, 1e-5)
    _close(y, by, 1e-13, "LN y brute")
    _close(mean, bm, 1e-13, "LN mean brute")
    _close(rstd, br, 1e-13, "LN rstd brute")
    # a textbook row: [1, 2, 3, 4] has mean 2.5 and variance 1.25
    y, mean, rstd = T.layernorm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), np.zeros(4), 0.0)
    _close(y, np.array([[-1.5, -0.5, 0.5, 1.5]]) / math.sqrt(1.25), 1e-15, "LN textbook row")
    assert abs(mean[0] - 2.5) < 1e-15 and abs(rstd[0] - 1 / math.sqrt(1.25)) < 1e-15
    # eps = 0, γ = 1, β = 0: every row has mean 0 and mean square 1; shift and scale invariance
    h = g.standard_normal((6, 33)) * 2.0 - 3.0
    y, _, _ = T.layernorm(h, np.ones(33), np.zeros(33), 0.0)
    assert np.abs(y.mean(axis=1)).max() < 1e-14 and np.abs((y * y).mean(axis=1) - 1).max() < 1e-13
    a, c = np.abs(g.standard_normal((6, 1))) + 0.5, g.standard_normal((6, 1)) * 10
    _close(T.layernorm(a * h + c, np.ones(33), np.zeros(33), 0.0)[0], y, 1e-12, "LN shift/scale invariance")
    # a constant row normalises to β; x̂ = 0 there, so its input gradient is (g − mean(g))/√eps
    hc = np.vstack([np.full(9, 2.75), g.standard_normal(9)])
    bet, gam, dyc = g.standard_normal(9), g.standard_normal(9), g.standard_normal((2, 9))
    assert np.abs(T.layernorm(hc, gam, bet, 1e-5)[0][0] - bet).max() < 1e-15
    dh, _, _ = T.layernorm_bwd(hc, gam, dyc, 1e-5)
    gc = dyc[0] * gam
    _close(dh[0], (gc - gc.mean()) / math.sqrt(1e-5), 1e-12, "constant row input gradient")
    # dropout + residual add, by hand
    x, o = np.array([[1.0, 2.0]]), np.array([[4.0, 8.0]])
    _close(T.dropout_add(x, o, np.array([[1, 0]], np.uint8), 0.5), np.array([[9.0, 2.0]]), 1e-15, "dropout-add")
    _close(T.dropout_add(x, o, None, 0.5), x + o, 1e-15, "add without dropout")
    _close(T.dropout_add(x, None, None, 0.0), x, 1e-15, "no sublayer output")
    _close(T.dropout_add(x, o, np.ones((1, 2), np.uint8), 0.2), x + o / 0.8, 1e-15, "all kept")
    # finite differences through h = x + dropout(o), y = LN(h)·γ + β, loss = Σ y·dy + Σ h·dh_in
    n, H, p, eps = 4, 10, 0.3, 1e-5
    x, o = g.standard_normal((n, H)), g.standard_normal((n, H)) * 2
    keep = (g.random((n, H)) > p).astype(np.uint8)
    gam, bet = g.standard_normal(H), g.standard_normal(H)
    dy, dh_in = g.standard_normal((n, H)), g.standard_normal((n, H))
    for sp, t, r in ((False, 2, 1), (True, 1, 0)):
        def loss(x_=x, o_=o, gm=gam, bt=bet):
            f = T.tp_residual_ln_fwd(t, r, sp, n, H, x_, o_, keep, p, gm, bt, eps)
            return float((f["y"] * dy).sum() + (f["h"] * dh_in).sum())
        fw = T.tp_residual_ln_fwd(t, r, sp, n, H, x, o, keep, p, gam, bet, eps)
        gr = T.tp_residual_ln_bwd(t, r, sp, n, H, dy, dh_in, fw["h"], gam, keep, p, eps)
        for name, x0, grad, call in (("dx", x, gr["dh"], lambda z: loss(x_=z)),
                                     ("do", o, gr["do"], lambda z: loss(o_=z)),
                                     ("dgamma", gam, gr["dgamma"], lambda z: loss(gm=z)),
                                     ("dbeta", bet, gr["dbeta"], lambda z: loss(bt=z))):
            for _ in range(3):
                vdir = g.standard_normal(x0.shape)
                want = _fd_dir(call, x0, vdir)
                got = float((grad * vdir).sum())
                assert abs(got - want) <= 1e-7 * max(1.0, abs(want)), f"FD LN {name}: {got} vs {want}"
    # sequence parallelism: rank row blocks concatenate to the replicated result; dγ, dβ partials sum
    Tt, H, t = 11, 6, 3
    x, o = g.standard_normal((Tt, H)), g.standard_normal((Tt, H))
    keep = (g.random((Tt, H)) > 0.1).astype(np.uint8)
    gam, bet, dy = g.standard_normal(H), g.standard_normal(H), g.standard_normal((Tt, H))
    full = T.tp_residual_ln_fwd(t, 1, False, Tt, H, x, o, keep, 0.1, gam, bet, 1e-5)
    fullb = T.tp_residual_ln_bwd(t, 1, False, Tt, H, dy, None, full["h"], gam, keep, 0.1, 1e-5)
    parts, bparts = [], []
    for r in range(t):
        r0, nr = T.sp_rows(Tt, t, r, True)
        sl = slice(r0, r0 + nr)
        f = T.tp_residual_ln_fwd(t, r, True, Tt, H, x[sl], o[sl], keep[sl], 0.1, gam, bet, 1e-5)
        parts.append(f)
        bparts.append(T.tp_residual_ln_bwd(t, r, True, Tt, H, dy[sl], None, f["h"], gam, keep[sl], 0.1, 1e-5))
    for k in ("h", "y", "mean", "rstd"):
        _close(np.concatenate([f[k] for f in parts]), full[k], 1e-15, f"SP concat {k}")
    for k in ("dh", "do"):
        _close(np.concatenate([b[k] for b in bparts]), fullb[k], 1e-15, f"SP concat {k}")
    for k in ("dgamma", "dbeta"):
        _close(sum(b[k] for b in bparts), fullb[k], 1e-13, f"SP sum of {k} partials")
    assert [T.sp_rows(Tt, t, r, True) for r in range(t)] == [(0, 4), (4, 4), (8, 3)]
    assert T.sp_rows(Tt, t, 2, False) == (0, Tt)


def pin_moe():
    g = _rng(61)
    n, E, k = 23, 7, 3
    lg = g.standard_normal((n, E)).astype(np.float32)
    lg[4, :] = 0.5                         # all equal: experts 0, 1, 2 in that order
    lg[9, 5] = lg[9, 2] = lg[9].max() + 1  # a tie at the top between experts 2 and 5
    r = T.moe_route(lg, k)
    want = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    assert (r["experts"] == want).all(), "top-k differs from a stable argsort of -logits"
    assert list(r["experts"][4]) == [0, 1, 2] and list(r["experts"][9][:2]) == [2, 5], "ties to the lower id"
    p = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    _close(r["gates"], np.take_along_axis(p, want, axis=1), 1e-15, "gates = softmax probabilities")
    assert (r["gates"].sum(axis=1) <= 1 + 1e-12).all()
    off, rt, tr = r["group_offsets"], r["row_token"], r["token_row"]
    assert off[0] == 0 and off[-1] == n * k and (np.diff(off) == np.bincount(want.reshape(-1), minlength=E)).all()
    for e in range(E):
        blk = rt[off[e]:off[e + 1]]
        assert (np.diff(blk) > 0).all(), "rows of an expert in token order"
        assert all(e in want[t] for t in blk)
    assert sorted(tr.reshape(-1).tolist()) == list(range(n * k)), "token_row is a permutation"
    for t in range(n):
        for j in range(k):
            row = tr[t, j]
            assert rt[row] == t and off[want[t, j]] <= row < off[want[t, j] + 1]
    # k = E: the gates are the whole softmax; combining equal rows returns the row itself
    rr = T.moe_route(lg, E)
    _close(rr["gates"].sum(axis=1), np.ones(n), 1e-14, "k = E gates sum to 1")
    c = g.standard_normal(5)
    _close(T.moe_combine(np.tile(c, (n * E, 1)), rr["gates"], rr["token_row"]), np.tile(c, (n, 1)), 1e-14,
           "combine of equal rows")
    # the whole block against per-token scalar loops, on a 2-way split of each expert's ffn columns
    n, E, k, H, Fe, t = 6, 4, 2, 5, 6, 2
    X = g.standard_normal((n, H))
    lg = g.standard_normal((n, E)).astype(np.float32)
    W1, b1 = g.standard_normal((E, H, Fe)) * 0.5, g.standard_normal((E, Fe)) * 0.5
    W2 = g.standard_normal((E, Fe, H)) * 0.5
    r = T.moe_route(lg, k)
    total = np.zeros((n, H))
    for rank in range(t):
        f0, fr = T.shard_range(Fe, t, rank)
        out = T.tp_moe_shard_fwd(t, rank, X, r, W1[:, :, f0:f0 + fr], b1[:, f0:f0 + fr], W2[:, f0:f0 + fr])["out"]
        ref = np.zeros((n, H))
        for tok in range(n):
            for j in range(k):
                e = r["experts"][tok, j]
                _, _, z = bf.mlp_forward(X[tok:tok + 1], W1[e][:, f0:f0 + fr], b1[e][f0:f0 + fr],
                                         W2[e][f0:f0 + fr], None)
                ref[tok] += r["gates"][tok, j] * np.array(z[0])
        _close(out, ref, 1e-13, f"MoE block r{rank} vs scalar loops")
        total += out
    full = T.tp_moe_shard_fwd(1, 0, X, r, W1, b1, W2)["out"]
    _close(total, full, 1e-13, "MoE: sum over TP ranks = unsharded")
    # one expert, top-1: the gate is 1 and the block is the dense MLP shard (no fc2 bias)
    r1 = T.moe_route(g.standard_normal((n, 1)).astype(np.float32), 1)
    d = T.tp_moe_shard_fwd(1, 0, X, r1, W1[:1], b1[:1], W2[:1])["out"]
    _close(d, T.tp_mlp_shard_fwd(1, 0, n, H, Fe, X, W1[0], b1[0], W2[0], None)["Z"], 1e-14, "E = k = 1")


def pin_fp8():
    import torch
    d = T.e4m3_decode(np.arange(256))
    for code, val in ((0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
                      (0x3C, 1.5), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0)):
        assert d[code] == val, f"decode 0x{code:02x} = {d[code]} != {val}"
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and np.signbit(d[0x80]) and d[0x80] == 0
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    fin = ~np.isnan(t)
    assert np.array_equal(d[fin], t[fin]) and np.array_equal(np.isnan(d), np.isnan(t)), "decode vs torch"
    codes = np.arange(256)[fin]
    assert np.array_equal(T.e4m3_encode(d[codes]), codes.astype(np.uint8)), "encode(decode(c)) = c"
    pos = np.sort(d[(np.arange(256) < 0x7F)])
    mid = (pos[1:] + pos[:-1]) / 2                 # exact midpoints: ties
    want = torch.from_numpy(mid.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = T.e4m3_encode(mid)
    assert np.array_equal(got, want) and (got % 2 == 0).all(), "midpoints round to the even code"
    g = _rng(71)
    x = (g.standard_normal(20000) * 60).astype(np.float32).clip(-448, 448)
    assert np.array_equal(T.e4m3_encode(x), torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert list(T.e4m3_encode([449.0, 1e6, -1e6, 464.0])) == [0x7E, 0x7E, 0xFE, 0x7E], "saturation"
    # per-tensor quantisation: the largest magnitude maps to 448, the descale undoes the scale
    X = g.standard_normal((7, 5)).astype(np.float32)
    X[3, 2] = -4.0 * np.abs(X).max()
    q, ds = T.fp8_quantize(X)
    assert q[3, 2] == 0xFE, "the largest magnitude quantises to -448"
    assert abs(float(ds) - float(np.abs(X).max()) / 448) <= 1e-7 * float(np.abs(X).max())
    qt, dst = T.fp8_quantize(X, transpose=True)
    assert np.array_equal(qt, q.T) and dst == ds
    qz, dz = T.fp8_quantize(np.zeros((3, 4), np.float32))
    assert dz == 1 and not qz.any()
    err = np.abs(T.e4m3_decode(q) * float(ds) - X) / np.abs(X).max()
    assert err.max() <= 2.0 ** -4 * 1.001, "relative rounding error within half an E4M3 step"
    # the GEMM on codes against scalar loops
    A = g.integers(0, 256, (5, 9)).astype(np.uint8)
    B = g.integers(0, 256, (4, 9)).astype(np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x38                   # no NaN codes
    B[(B & 0x7F) == 0x7F] = 0xB8
    bias = g.standard_normal(4)
    da, db = np.float32(0.25), np.float32(3.0)
    r = T.fp8_gemm_nt(A, da, B, db, bias, epi=T.FP8_EPI_GELU)
    dA, dB = T.e4m3_decode(A).tolist(), T.e4m3_decode(B).tolist()
    for i in range(5):
        for j in range(4):
            acc = 0.0
            for k in range(9):
                acc += dA[i][k] * dB[j][k]
            pre = acc * 0.25 * 3.0 + bias[j]
            assert abs(r["pre"][i, j] - pre) <= 1e-12 * max(1.0, abs(pre))
            assert abs(r["C"][i, j] - bf.gelu(pre)) <= 1e-12 * max(1.0, abs(pre))
    # E5M2 (gradients): anchors, every finite code against torch's float8_e5m2, round trip, ties,
    # saturation; a mixed-format GEMM with the GeLU' epilogue against scalar loops
    d5 = T.fp8_decode(np.arange(256), "e5m2")
    for code, val in ((0x3C, 1.0), (0x7B, 57344.0), (0x01, 2.0 ** -16), (0x04, 2.0 ** -14), (0xBC, -1.0)):
        assert d5[code] == val, f"e5m2 decode 0x{code:02x} = {d5[code]}"
    assert d5[0x7C] == np.inf and d5[0xFC] == -np.inf and np.isnan(d5[0x7D]) and np.isnan(d5[0xFF])
    t5 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).float().numpy().astype(np.float64)
    fin5 = np.isfinite(t5)
    assert np.array_equal(d5[fin5], t5[fin5]) and np.array_equal(np.isfinite(d5), fin5), "e5m2 decode vs torch"
    c5 = np.arange(256)[fin5]
    assert np.array_equal(T.fp8_encode(d5[c5], "e5m2"), c5.astype(np.uint8)), "e5m2 encode(decode(c)) = c"
    pos5 = np.sort(d5[np.arange(256) < 0x7C])
    mid5 = (pos5[1:] + pos5[:-1]) / 2
    got5 = T.fp8_encode(mid5, "e5m2")
    assert np.array_equal(got5, torch.from_numpy(mid5.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy())
    assert (got5 % 2 == 0).all(), "e5m2 midpoints to the even code"
    x5 = (g.standard_normal(20000) * 3000).astype(np.float32).clip(-57344, 57344)
    assert np.array_equal(T.fp8_encode(x5, "e5m2"),
                          torch.from_numpy(x5).to(torch.float8_e5m2).view(torch.uint8).numpy())
    assert list(T.fp8_encode([60000.0, -1e9], "e5m2")) == [0x7B, 0xFB], "e5m2 saturation"
    q5, ds5 = T.fp8_quantize(X, fmt="e5m2")
    assert q5[3, 2] == 0xFB and abs(float(ds5) - float(np.abs(X).max()) / 57344) <= 1e-7 * float(np.abs(X).max())
    A5 = g.integers(0, 256, (4, 6)).astype(np.uint8)
    A5[(A5 & 0x7F) >= 0x7C] = 0x3C                    # finite E5M2 codes only
    B4 = g.integers(0, 256, (3, 6)).astype(np.uint8)
    B4[(B4 & 0x7F) == 0x7F] = 0x38
    aux = g.standard_normal((4, 3))
    r = T.fp8_gemm_nt(A5, np.float32(0.5), B4, np.float32(2.0), epi=T.FP8_EPI_DGELU, aux=aux,
                      fmt_a="e5m2", fmt_b="e4m3")
    dA, dB = T.fp8_decode(A5, "e5m2").tolist(), T.fp8_decode(B4, "e4m3").tolist()
    for i in range(4):
        for j in range(3):
            pre = sum(dA[i][k] * dB[j][k] for k in range(6)) * 0.5 * 2.0
            assert abs(r["C"][i, j] - pre * bf.gelu_prime(aux[i, j])) <= 1e-12 * max(1.0, abs(pre))


def pin_moe_backward():
    """The MoE block's backward against fp64 central differences of Σ out_r ∘ d_out in X, each
    expert's weight shards and the gates (held as inputs), on both ranks of a split; the router's
    logit gradient against differences of the routed gates (logits far enough apart that the
    choice stays fixed); rank sums and shard blocks against the unsharded block; E = k = 1 against
    the dense MLP backward; k = E with equal gate gradients gives zero logit gradient (Σ_e p_e = 1)."""
    g = _rng(67)
    n, E, k, H, Fe, t = 7, 5, 2, 4, 6, 2
    X = g.standard_normal((n, H))
    lg = (g.permutation(n * E).reshape(n, E) * 0.375).astype(np.float32)    # distinct, gaps >= 3/8
    W1, b1 = g.standard_normal((E, H, Fe)) * 0.5, g.standard_normal((E, Fe)) * 0.5
    W2 = g.standard_normal((E, Fe, H)) * 0.5
    d_out = g.standard_normal((n, H))
    r = T.moe_route(lg, k)
    full_fwd = T.tp_moe_shard_fwd(1, 0, X, r, W1, b1, W2)
    full = T.tp_moe_shard_bwd(1, 0, X, r, W1, W2, full_fwd, d_out)
    sum_dX, sum_dg = np.zeros((n, H)), np.zeros((n, k))
    for rank in range(t):
        f0, fr = T.shard_range(Fe, t, rank)
        W1r, b1r, W2r = W1[:, :, f0:f0 + fr], b1[:, f0:f0 + fr], W2[:, f0:f0 + fr]
        fwd = T.tp_moe_shard_fwd(t, rank, X, r, W1r, b1r, W2r)
        b = T.tp_moe_shard_bwd(t, rank, X, r, W1r, W2r, fwd, d_out)

        def loss(X_=X, W1_=W1r, b1_=b1r, W2_=W2r, gates_=r["gates"]):
            rt = dict(r, gates=gates_)
            return float((T.tp_moe_shard_fwd(t, rank, X_, rt, W1_, b1_, W2_)["out"] * d_out).sum())
        for name, x, grad, kw in (("X", X, b["dX"], "X_"), ("W1", W1r, b["dW1"], "W1_"), ("b1", b1r, b["db1"], "b1_"),
                                  ("W2", W2r, b["dW2"], "W2_"), ("gates", r["gates"], b["dgates"], "gates_")):
            for _ in range(2):
                v = g.standard_normal(x.shape)
                fd = _fd_dir(lambda y: loss(**{kw: y}), x, v)
                _close(np.array([(grad * v).sum()]), np.array([fd]), 1e-7, f"MoE bwd r{rank} d{name} vs differences")
        sum_dX += b["dX"]
        sum_dg += b["dgates"]
        _close(b["dW1"], full["dW1"][:, :, f0:f0 + fr], 1e-12, "dW1 rank block = columns of the unsharded")
        _close(b["db1"], full["db1"][:, f0:f0 + fr], 1e-12, "db1 rank block")
        _close(b["dW2"], full["dW2"][:, f0:f0 + fr], 1e-12, "dW2 rank block = rows of the unsharded")
    _close(sum_dX, full["dX"], 1e-12, "MoE bwd: sum of dX over ranks = unsharded")
    _close(sum_dg, full["dgates"], 1e-12, "MoE bwd: sum of gate gradients over ranks = unsharded")
    # router: differences of Σ gates(l)·dg with the choice fixed
    dg = full["dgates"]
    dl = T.moe_route_bwd(lg, r["experts"], dg)
    # directions of small integers and a step of 2⁻¹⁰ keep l ± h·v exact in float32 (the logits are
    # multiples of 3/8 below 16), so the difference quotient carries no rounding of its inputs
    for _ in range(3):
        v = g.integers(-3, 4, lg.shape).astype(np.float64)

        def gsum(l):
            rr = T.moe_route(l.astype(np.float32), k)
            assert (rr["experts"] == r["experts"]).all()
            return float((rr["gates"] * dg).sum())
        h = 2.0 ** -10
        fd = (gsum(lg.astype(np.float64) + h * v) - gsum(lg.astype(np.float64) - h * v)) / (2 * h)
        _close(np.array([(dl * v).sum()]), np.array([fd]), 1e-5, "router logit gradient vs differences")
    rE = T.moe_route(lg, E)
    assert np.abs(T.moe_route_bwd(lg, rE["experts"], np.full((n, E), 0.7))).max() < 1e-15, "k = E, equal dg"
    # one expert, top-1: gate 1, the dense MLP backward; dgate = <d_out, Z>
    r1 = T.moe_route(np.zeros((n, 1), np.float32), 1)
    f1 = T.tp_moe_shard_fwd(1, 0, X, r1, W1[:1], b1[:1], W2[:1])
    b1_ = T.tp_moe_shard_bwd(1, 0, X, r1, W1[:1], W2[:1], f1, d_out)
    dense = T.mlp_fwd(X, W1[0], b1[0], W2[0], None)
    db = T.mlp_bwd(X, W1[0], W2[0], dense["A1"], dense["Y"], d_out, False)
    for a, bb in (("dX", "dX"), ("dW1", "dW1"), ("db1", "db1"), ("dW2", "dW2")):
        got = b1_[a][0] if a != "dX" else b1_[a]
        _close(got, db[bb], 1e-13, f"E = k = 1 {a} = dense")
    _close(b1_["dgates"][:, 0], (d_out * dense["Z"]).sum(axis=1), 1e-13, "E = k = 1 dgate = <d_out, Z>")


def pin_error_metrics():
    """The parity checkers themselves, against values worked out by hand.

    normwise_error is ‖got − ref‖_F / ‖ref‖_F: the denominator from ref (swapping got and ref
    changes the value), the Frobenius norm (not the largest element), the absolute form for a zero
    reference.  blockwise_error is the largest 64 x 64 tile error, each tile's difference over the
    larger of its own norm and its share ‖ref‖_F·√(n_b/n) of the whole: the hand values below fix
    the tiling, the share, ragged edge tiles and the view of vectors and 3-D tensors as matrices.
    Last, a planted localised defect — one 256 x 192 output tile of a GEMM that skipped one 16-deep
    k-step of its 2048 — is below the 2e-2 bar normwise (≈0.6%) and far above it tile-wise.
    """
    ne, be = T.normwise_error, T.blockwise_error
    assert abs(ne([[3.3, 3.6]], [[3.0, 4.0]]) - 0.1) <= 1e-15, "0.5 / 5"
    assert abs(ne([6.0, 8.0], [3.0, 4.0]) - 1.0) <= 1e-15, "‖(3, 4)‖ / ‖(3, 4)‖"
    assert abs(ne([3.0, 4.0], [6.0, 8.0]) - 0.5) <= 1e-15, "‖(3, 4)‖ / ‖(6, 8)‖: denominator from ref"
    assert ne([0.0, 0.0], [3.0, 4.0]) == 1.0, "zero output: error 1"
    assert abs(ne([[2.0, 1.0], [1.0, 1.0]], np.ones((2, 2))) - 0.5) <= 1e-15, "Frobenius: 1 / 2, not max 1 / 1"
    assert ne([3.0, 4.0], [0.0, 0.0]) == 5.0, "zero reference: absolute ‖got‖"
    assert ne(np.ones(7), np.ones(7)) == 0.0

    ones = np.ones((128, 128))
    g = ones.copy()
    g[:64, :64] += 0.1                  # tile (0, 0): ‖diff‖ = 6.4, own norm 64, share 128·½ = 64
    assert abs(be(g, ones) - 0.1) <= 1e-14, f"one tile +10%: {be(g, ones)}"
    assert abs(ne(g, ones) - 0.05) <= 1e-14
    r = ones.copy()
    r[64:, 64:] = 0.01                  # a tile of small values: held to its share of the whole
    g = r.copy()
    g[64:, 64:] += 0.001
    want = 0.064 / (0.5 * math.sqrt(3 * 4096 + 4096 * 1e-4))
    assert abs(be(g, r) - want) <= 1e-14 * want, f"small tile: {be(g, r)} vs {want}"
    r = np.ones((3, 100))               # ragged: tiles 3 x 64 and 3 x 36
    g = r.copy()
    g[0, 70] += 1.0
    assert abs(be(g, r) - 1.0 / math.sqrt(108)) <= 1e-14, "ragged edge tile of 108 elements"
    v = np.ones(130)                    # a vector is one row: tiles of 64, 64 and 2 elements
    w = v.copy()
    w[129] = 2.0
    assert abs(be(w, v) - 1.0 / math.sqrt(2)) <= 1e-14, "vector edge tile of 2 elements"
    t3 = np.ones((2, 3, 64))            # leading dimensions become rows: one 6 x 64 tile
    u3 = t3.copy()
    u3[1, 2, 5] = 0.0
    assert abs(be(u3, t3) - 1.0 / math.sqrt(384)) <= 1e-14, "3-D tensor as a 6 x 64 matrix"
    assert be([0.0, 0.0, 3.0, 4.0], np.zeros(4)) == 5.0, "zero reference: absolute"
    assert be(ones, ones) == 0.0

    rng = _rng(71)
    A = rng.standard_normal((2048, 2048))
    B = rng.standard_normal((2048, 4608)) * 0.02
    C = A @ B
    bad = C.copy()
    bad[256:512, 384:576] -= A[256:512, 1024:1040] @ B[1024:1040, 384:576]
    assert 3e-3 <= ne(bad, C) <= 1e-2, f"planted defect normwise {ne(bad, C):.2e}"
    assert be(bad, C) >= 5e-2, f"planted defect tile-wise {be(bad, C):.2e}"


ALL_PINS = [pin_geometry, pin_gelu, pin_brute_forward, pin_brute_backward, pin_identities,
            pin_attention_closed_forms, pin_finite_differences, pin_grouped, pin_layernorm, pin_moe, pin_moe_backward,
            pin_fp8, pin_error_metrics]
