"""The entry points under HIP graph capture.

They allocate nothing, synchronise nothing and enqueue only kernels on the caller's stream, so a
whole step can be captured once and replayed.  Each test captures the step, replays the graph
several times with eager work and synchronisations in between, and checks every replay bitwise
against the eager step on the same inputs (and, once, against the oracle).
"""

import pytest
import torch

import oracle
from gpu_harness import Shard, assert_close, dev
from test_gpu_parity import RAGGED8, TILES, _grouped_inputs, ws
from tensor_transformer_layer_mlp_amd import binding as bd

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _step_buffers(sh):
    wl, dt = sh.wl, sh.dtype
    T, H, d = wl.T, wl.H, sh.d
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    e = lambda *s, t=tdt: torch.empty(*s, dtype=t, device="cuda")  # noqa: E731
    return {"QKV": e(T, sh.Nq), "ctx": e(T, sh.nh * d), "lse": e(wl.B, sh.nh, wl.S, t=torch.float32),
            "Z": e(T, H), "A1": e(T, sh.Fr), "Y": e(T, sh.Fr), "dXm": e(T, H), "dW1": e(H, sh.Fr),
            "db1": e(sh.Fr), "dW2": e(sh.Fr, H), "db2": e(H), "dQKV": e(T, sh.Nq), "dXq": e(T, H),
            "dWq": e(H, sh.Nq), "dbq": e(sh.Nq)}


def _make_step(sh, o):
    wl, r = sh.wl, sh.rank
    db2 = o["db2"]
    t, B, S, H, nh, F, T = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F, wl.T
    X, Wq, bq = sh.d_("X"), sh.d_("Wqkv"), sh.d_("bqkv")
    W1, b1, W2, b2 = sh.d_("W1"), sh.d_("b1"), sh.d_("W2"), sh.d_("b2")
    dZ, dctx = sh.d_("dZ"), sh.d_("dctx")
    ws_m, ws_q, ws_a = ws("tp_mlp_shard_bwd", sh), ws("tp_qkv_shard_bwd", sh), ws("tp_attn_heads_bwd", sh)

    def step():
        bd.tp_qkv_shard_fwd(t, r, B, S, H, nh, X, Wq, bq, o["QKV"])
        bd.tp_attn_heads_fwd(t, r, B, S, H, nh, o["QKV"], o["ctx"], o["lse"])
        bd.tp_mlp_shard_fwd(t, r, T, H, F, X, W1, b1, W2, b2, o["Z"], o["A1"], o["Y"])
        bd.tp_mlp_shard_bwd(t, r, T, H, F, X, W1, W2, o["A1"], o["Y"], dZ, o["dXm"], o["dW1"], o["db1"],
                            o["dW2"], db2, ws_m)
        bd.tp_attn_heads_bwd(t, r, B, S, H, nh, o["QKV"], o["ctx"], o["lse"], dctx, o["dQKV"], ws_a)
        bd.tp_qkv_shard_bwd(t, r, B, S, H, nh, X, Wq, o["dQKV"], o["dXq"], o["dWq"], o["dbq"], ws_q)
    return step


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                 # warm-up on a side stream, as capture requires
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("wl,dtype,rank", [(TILES, "bf16", 1), (RAGGED8, "bf16", 2), (RAGGED8, "f32", 0)],
                         ids=["tiles-bf16", "ragged8-bf16", "ragged8-f32"])
def test_step_graph_replay(wl, dtype, rank):
    sh = Shard(wl, rank, dtype)
    o = _step_buffers(sh)
    step = _make_step(sh, o)
    if rank != 0:
        del o["db2"]                         # written by rank 0 only
    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in o.items()}
    g = _capture(step)
    for rep in range(REPLAYS):
        for v in o.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in o:
            assert torch.equal(o[k], eager[k]), f"replay {rep}: {k} differs from the eager step"
        step()                               # eager work between replays
        torch.cuda.synchronize()
    t, B, S, H, nh, F = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F
    R = oracle.tp_mlp_shard_fwd(t, rank, B * S, H, F, sh.f64("X"), sh.f64("W1"), sh.f64("b1"),
                                sh.f64("W2"), sh.f64("b2"))
    assert_close(o["Z"], R["Z"], dtype, "Z_r after replays")
    R_qkv = oracle.tp_qkv_shard_fwd(t, rank, B, S, H, nh, sh.f64("X"), sh.f64("Wqkv"), sh.f64("bqkv"))
    R_dqkv = oracle.tp_attn_heads_bwd(t, rank, B, S, H, nh, R_qkv, sh.f64("dctx"))
    assert_close(o["dQKV"], R_dqkv, dtype, "dQKV_r after replays")


def test_grouped_graph_replay():
    """The grouped expert MLP (device-side offsets, plan kernel + two grouped GEMMs) in a graph."""
    sizes, H, Fg, tp, rank = [0, 5, 300, 1, 257, 77], 192, 128, 2, 1
    off, rows, Fr, ops = _grouped_inputs(sizes, 0, "bf16", H, Fg, tp, rank)
    G = len(sizes)
    bf = torch.bfloat16
    X, W1, b1, W2 = (dev(ops[k]) for k in ("X", "W1", "b1", "W2"))
    Z, A1, Y = (torch.empty(rows, c, dtype=bf, device="cuda") for c in (H, Fr, Fr))
    offs = torch.from_numpy(off).cuda()
    wsb = bd.workspace("tp_mlp_grouped_shard_fwd", tp, rank, 1, rows, H, G, Fg, bf)

    def call():
        bd.tp_mlp_grouped_shard_fwd(tp, rank, G, offs, rows, H, Fg, X, W1, b1, W2, Z, A1, Y, wsb)
    call()
    torch.cuda.synchronize()
    eager = [Z.clone(), A1.clone(), Y.clone()]
    g = _capture(call)
    for rep in range(REPLAYS):
        for v in (Z, A1, Y):
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref, k in zip((Z, A1, Y), eager, ("Z", "A1", "Y")):
            assert torch.equal(got, ref), f"replay {rep}: {k} differs from the eager call"
        call()
        torch.cuda.synchronize()
    f = {k: v.f64 for k, v in ops.items()}
    ref = oracle.tp_mlp_grouped_shard_fwd(tp, rank, off, f["X"], f["W1"], f["b1"], f["W2"])
    assert_close(Z, ref, "bf16", "Z_r grouped after replays")
