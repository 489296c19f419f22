"""GPU parity of the residual add with dropout + LayerNorm (the layer's replicated-side ops, or the
same ops on a rank's row block under sequence parallelism), forward and backward, against the fp64
oracle on the same seeded inputs: vector and scalar paths (H a multiple of 8 or not, up to the
24576-feature maximum), with and without the sublayer output, the dropout mask and the residual
gradient; the sequence-parallel split against the replicated call; empty input, guard bands,
determinism and graph replay.  Expected values come from the oracle only.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import TORCH_DT, assert_close, empty, host
from test_gpu_graph import _capture
from test_gpu_parity import _guarded
from tensor_transformer_layer_mlp_amd import binding as bd, synth

pytestmark = pytest.mark.gpu

EPS, P = 1e-5, 0.1

# (T, H): ragged rows on the vector path, GPT-2 / GPT-3 hidden sizes, H not a multiple of 8 (bf16
# scalar path; fp32 vector path when H % 4 == 0), odd H, the largest register class, the maximum H
SHAPES = [(201, 192), (64, 1600), (37, 12288), (50, 100), (9, 7), (6, 20000), (3, 24576), (4, 20001)]
VARIANTS = {"full": (True, True, True), "no_dropout": (True, False, True), "plain_ln": (False, False, False)}


def _inputs(T, H, dtype, with_o, with_keep, tag=""):
    f = lambda name, shape, std=1.0: synth.normal(f"ln_{name}{tag}", shape, std, dtype)  # noqa: E731
    ops = {"x": f("x", (T, H)), "gamma": synth.make_operand(1.0 + f("g", (H,), 0.1).f64, dtype),
           "beta": f("b", (H,), 0.1), "dy": f("dy", (T, H)), "dh_in": f("dhin", (T, H))}
    if with_o:
        ops["o"] = f("o", (T, H), 2.0)
    keep = synth.keep_mask(f"ln_keep{tag}", (T, H), P) if with_keep else None
    return ops, keep


def _dev(op):
    from gpu_harness import dev
    return dev(op)


def _run(T, H, dtype, ops, keep, with_dh_in, tp=1, rank=0, sp=False, rows=None, outs=None):
    rows = T if rows is None else rows
    tdt = TORCH_DT[dtype]
    D = {k: _dev(v) for k, v in ops.items()}
    K = torch.from_numpy(keep).cuda() if keep is not None else None
    o = outs or {}
    h = o.get("h", empty((rows, H), dtype)) if "o" in D else None
    y = o.get("y", empty((rows, H), dtype))
    mean, rstd = o.get("mean", empty((rows,), torch.float32)), o.get("rstd", empty((rows,), torch.float32))
    bd.tp_residual_ln_fwd(tp, rank, sp, T, H, D["x"], D.get("o"), K, P, D["gamma"], D["beta"], EPS, h, y, mean, rstd)
    dh, d_o = o.get("dh", empty((rows, H), dtype)), o.get("d_o", empty((rows, H), dtype))
    dg, db = o.get("dg", empty((H,), dtype)), o.get("db", empty((H,), dtype))
    ws = bd.workspace("tp_residual_ln_bwd", tp, rank, 1, T, H, 1, 1, tdt)
    bd.tp_residual_ln_bwd(tp, rank, sp, T, H, D["dy"], D["dh_in"] if with_dh_in else None,
                          h if h is not None else D["x"], mean, rstd, D["gamma"], K, P, dh, d_o, dg, db, ws)
    torch.cuda.synchronize()
    return dict(h=h, y=y, mean=mean, rstd=rstd, dh=dh, d_o=d_o, dg=dg, db=db)


def _oracle(T, H, ops, keep, with_dh_in, tp=1, rank=0, sp=False):
    f = {k: v.f64 for k, v in ops.items()}
    fw = oracle.tp_residual_ln_fwd(tp, rank, sp, T, H, f["x"], f.get("o"), keep, P, f["gamma"], f["beta"], EPS)
    bw = oracle.tp_residual_ln_bwd(tp, rank, sp, T, H, f["dy"], f["dh_in"] if with_dh_in else None, fw["h"],
                                   f["gamma"], keep, P, EPS)
    return fw, bw


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,H", SHAPES, ids=[f"t{t}_h{h}" for t, h in SHAPES])
def test_residual_ln(T, H, dtype, variant):
    with_o, with_keep, with_dh_in = VARIANTS[variant]
    ops, keep = _inputs(T, H, dtype, with_o, with_keep)
    print(f"ln T={T} H={H} {dtype} {variant}", flush=True)
    g = _run(T, H, dtype, ops, keep, with_dh_in)
    fw, bw = _oracle(T, H, ops, keep, with_dh_in)
    if with_o:
        assert_close(g["h"], fw["h"], dtype, "h")
    assert_close(g["y"], fw["y"], dtype, "y")
    assert_close(g["mean"], fw["mean"], dtype, "mean")
    assert_close(g["rstd"], fw["rstd"], dtype, "rstd")
    assert_close(g["dh"], bw["dh"], dtype, "dh")
    assert_close(g["d_o"], bw["do"], dtype, "d_o")
    assert_close(g["dg"], bw["dgamma"], dtype, "dgamma")
    assert_close(g["db"], bw["dbeta"], dtype, "dbeta")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_residual_ln_many_wide_rows(dtype):
    """Enough rows for the 256-thread workgroups with the widest register class (H > 16384)."""
    T, H = 1030, 16392
    ops, keep = _inputs(T, H, dtype, True, True, tag="_wide")
    g = _run(T, H, dtype, ops, keep, True)
    fw, bw = _oracle(T, H, ops, keep, True)
    for k, rk in (("h", "h"), ("y", "y"), ("mean", "mean"), ("rstd", "rstd")):
        assert_close(g[k], fw[rk], dtype, k)
    for k, rk in (("dh", "dh"), ("d_o", "do"), ("dg", "dgamma"), ("db", "dbeta")):
        assert_close(g[k], bw[rk], dtype, k)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sequence_parallel_split(dtype):
    """Each of 4 ranks normalises its block of 203 rows: the blocks equal the replicated call's rows
    bitwise (rows are independent), and the dγ, dβ partials sum to the full gradient."""
    T, H, t = 203, 384, 4
    ops, keep = _inputs(T, H, dtype, True, True)
    full = _run(T, H, dtype, ops, keep, True)
    parts = []
    for r in range(t):
        r0, n = oracle.shard_range(T, t, r)
        sl = slice(r0, r0 + n)
        sub = {k: (synth.make_operand(v.f64[sl], dtype) if v.f64.ndim == 2 else v) for k, v in ops.items()}
        parts.append(_run(T, H, dtype, sub, keep[sl], True, tp=t, rank=r, sp=True, rows=n))
    for k in ("h", "y", "mean", "rstd", "dh", "d_o"):
        assert torch.equal(torch.cat([p[k] for p in parts]), full[k]), f"SP rows of {k} differ from the replicated call"
    fw, bw = _oracle(T, H, ops, keep, True)
    for k, ref in (("dg", bw["dgamma"]), ("db", bw["dbeta"])):
        assert_close(sum(p[k].double() for p in parts), ref, dtype, f"sum of SP {k} partials")
        e = oracle.normwise_error(host(sum(p[k].float() for p in parts)), host(full[k]))
        assert e <= (2e-2 if dtype == "bf16" else 1e-5), f"SP {k} sum vs replicated: {e:.2e}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_empty(dtype):
    """No rows (T = 0, or a sequence-parallel rank with none): dγ and dβ are exact zeros."""
    H = 64
    tdt = TORCH_DT[dtype]
    z = torch.empty(0, H, dtype=tdt, device="cuda")
    zf = torch.empty(0, dtype=torch.float32, device="cuda")
    g = torch.ones(H, dtype=tdt, device="cuda")
    bd.tp_residual_ln_fwd(1, 0, False, 0, H, z, z, None, 0.0, g, g, EPS, z, z, zf, zf)
    for tp, rank, sp, T in ((1, 0, False, 0), (4, 3, True, 3)):
        dg, db = empty((H,), dtype), empty((H,), dtype)
        ws = bd.workspace("tp_residual_ln_bwd", tp, rank, 1, T, H, 1, 1, tdt)
        bd.tp_residual_ln_bwd(tp, rank, sp, T, H, z, None, z, zf, zf, g, None, 0.0, z, None, dg, db, ws)
        torch.cuda.synchronize()
        assert (dg == 0).all() and (db == 0).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_no_out_of_bounds_writes(dtype):
    T, H = 67, 200
    ops, keep = _inputs(T, H, dtype, True, True)
    outs, guards = {}, []
    for k, shape, dt in (("h", (T, H), dtype), ("y", (T, H), dtype), ("mean", (T,), torch.float32),
                         ("rstd", (T,), torch.float32), ("dh", (T, H), dtype), ("d_o", (T, H), dtype),
                         ("dg", (H,), dtype), ("db", (H,), dtype)):
        outs[k], g = _guarded(shape, dt)
        guards.append((k, g))
    _run(T, H, dtype, ops, keep, True, outs=outs)
    for k, g in guards:
        assert (g.float() == -7776.0).all(), f"guard band after {k} overwritten"


def test_ln_deterministic_and_graph_replay():
    T, H, dtype = 130, 1024, "bf16"
    ops, keep = _inputs(T, H, dtype, True, True)
    a = _run(T, H, dtype, ops, keep, True)
    b = _run(T, H, dtype, ops, keep, True)
    for k in a:
        assert torch.equal(a[k], b[k]), f"{k} differs between two runs"
    D = {k: _dev(v) for k, v in ops.items()}
    K = torch.from_numpy(keep).cuda()
    o = {k: torch.empty_like(v) for k, v in a.items()}
    ws = bd.workspace("tp_residual_ln_bwd", 1, 0, 1, T, H, 1, 1, torch.bfloat16)

    def call():
        bd.tp_residual_ln_fwd(1, 0, False, T, H, D["x"], D["o"], K, P, D["gamma"], D["beta"], EPS, o["h"], o["y"],
                              o["mean"], o["rstd"])
        bd.tp_residual_ln_bwd(1, 0, False, T, H, D["dy"], D["dh_in"], o["h"], o["mean"], o["rstd"], D["gamma"], K,
                              P, o["dh"], o["d_o"], o["dg"], o["db"], ws)
    g = _capture(call)
    for rep in range(3):
        for v in o.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in o:
            assert torch.equal(o[k], a[k]), f"replay {rep}: {k} differs from the eager call"
        call()
        torch.cuda.synchronize()
    assert np.isfinite(host(o["y"])).all()


def test_ln_gpt3_full_size():
    """The GPT-3 175B hidden size at the full 2048 tokens, replicated, and rank 0's 256-row block
    under sequence parallelism over 8 ranks (bf16, dropout 0.1, residual gradient)."""
    T, H, dtype = 2048, 12288, "bf16"
    ops, keep = _inputs(T, H, dtype, True, True, tag="_gpt3")
    g = _run(T, H, dtype, ops, keep, True)
    fw, bw = _oracle(T, H, ops, keep, True)
    for k, rk in (("h", "h"), ("y", "y"), ("mean", "mean"), ("rstd", "rstd")):
        assert_close(g[k], fw[rk], dtype, f"{k} full size")
    for k, rk in (("dh", "dh"), ("d_o", "do"), ("dg", "dgamma"), ("db", "dbeta")):
        assert_close(g[k], bw[rk], dtype, f"{k} full size")
    r0, n = oracle.shard_range(T, 8, 0)
    sub = {k: (synth.make_operand(v.f64[r0:r0 + n], dtype) if v.f64.ndim == 2 else v) for k, v in ops.items()}
    s = _run(T, H, dtype, sub, keep[r0:r0 + n], True, tp=8, rank=0, sp=True, rows=n)
    fs, bs = _oracle(T, H, sub, keep[r0:r0 + n], True, tp=8, rank=0, sp=True)
    assert_close(s["y"], fs["y"], dtype, "SP rank 0 y")
    assert_close(s["dg"], bs["dgamma"], dtype, "SP rank 0 dgamma partial")
