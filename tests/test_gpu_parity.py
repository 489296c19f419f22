"""GPU parity: every entry point against the fp64 oracle on the same seeded inputs.

Sizes here let the oracle finish in seconds while spanning several tiles and ragged tails; the
full-size workloads are in test_gpu_fullsize.py.  Tolerance: normwise relative error <= 2e-2 with
bf16 inputs / fp32 accumulation, <= 1e-5 in the fp32 check mode.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import Shard, assert_close, dev, empty, host, TORCH_DT
from tensor_transformer_layer_mlp_amd import binding as bd, synth
from tensor_transformer_layer_mlp_amd.configs import LayerWorkload, TINY

pytestmark = pytest.mark.gpu

RAGGED = LayerWorkload("ragged_b3_s67_h192_nh3_f500_tp2", 3, 67, 192, 3, 500, 2, (0, 1), 0.05)
UNEVEN = LayerWorkload("uneven_b2_s40_h400_nh25_f130_tp2", 2, 40, 400, 25, 130, 2, (0, 1), 0.05)
D96 = LayerWorkload("d96_b2_s100_h384_nh4_f776_tp2", 2, 100, 384, 4, 776, 2, (0, 1), 0.05)
D128 = LayerWorkload("d128_b1_s130_h256_nh2_f520_tp1", 1, 130, 256, 2, 520, 1, (0,), 0.05)
D32 = LayerWorkload("d32_b2_s80_h128_nh4_f256_tp4", 2, 80, 128, 4, 256, 4, (0, 3), 0.05)
TILES = LayerWorkload("tiles_b2_s320_h512_nh8_f2560_tp2", 2, 320, 512, 8, 2560, 2, (1,), 0.03)
# dimensions multiples of 8 but ragged against every tile: M = 264, N = 336, K = 328 / 264
RAGGED8 = LayerWorkload("ragged8_b3_s88_h320_nh20_f984_tp3", 3, 88, 320, 20, 984, 3, (0, 2), 0.05)
SMALL = [TINY, RAGGED, UNEVEN, D96, D128, D32, TILES, RAGGED8]
DTYPES = ["bf16", "f32"]


def cases():
    for wl in SMALL:
        for dt in DTYPES:
            for r in wl.ranks:
                yield pytest.param(wl, dt, r, id=f"{wl.name}-{dt}-r{r}")


def ws(fn, sh):
    wl = sh.wl
    return bd.workspace(fn, wl.tp_size, sh.rank, wl.B, wl.S, wl.H, wl.n_heads, wl.F, TORCH_DT[sh.dtype])


def run_qkv_fwd(sh, X=None):
    wl = sh.wl
    out = empty((wl.T, sh.Nq), sh.dtype)
    bd.tp_qkv_shard_fwd(wl.tp_size, sh.rank, wl.B, wl.S, wl.H, wl.n_heads,
                        sh.d_("X") if X is None else X, sh.d_("Wqkv"), sh.d_("bqkv"), out)
    return out


def run_attn_fwd(sh, qkv):
    wl = sh.wl
    ctx = empty((wl.T, sh.nh * sh.d), sh.dtype)
    lse = empty((wl.B, sh.nh, wl.S), torch.float32)
    bd.tp_attn_heads_fwd(wl.tp_size, sh.rank, wl.B, wl.S, wl.H, wl.n_heads, qkv, ctx, lse)
    return ctx, lse


def run_mlp_fwd(sh, with_b2=True):
    wl = sh.wl
    Z = empty((wl.T, wl.H), sh.dtype)
    A1 = empty((wl.T, sh.Fr), sh.dtype)
    Y = empty((wl.T, sh.Fr), sh.dtype)
    bd.tp_mlp_shard_fwd(wl.tp_size, sh.rank, wl.T, wl.H, wl.F, sh.d_("X"), sh.d_("W1"), sh.d_("b1"),
                        sh.d_("W2"), sh.d_("b2") if with_b2 else None, Z, A1, Y)
    return Z, A1, Y


def run_mlp_bwd(sh, A1, Y):
    wl = sh.wl
    o = dict(dX=empty((wl.T, wl.H), sh.dtype), dW1=empty((wl.H, sh.Fr), sh.dtype),
             db1=empty((sh.Fr,), sh.dtype), dW2=empty((sh.Fr, wl.H), sh.dtype),
             db2=empty((wl.H,), sh.dtype))
    bd.tp_mlp_shard_bwd(wl.tp_size, sh.rank, wl.T, wl.H, wl.F, sh.d_("X"), sh.d_("W1"), sh.d_("W2"),
                        A1, Y, sh.d_("dZ"), o["dX"], o["dW1"], o["db1"], o["dW2"], o["db2"],
                        ws("tp_mlp_shard_bwd", sh))
    return o


def run_qkv_bwd(sh, dqkv):
    wl = sh.wl
    o = dict(dX=empty((wl.T, wl.H), sh.dtype), dW=empty((wl.H, sh.Nq), sh.dtype),
             db=empty((sh.Nq,), sh.dtype))
    bd.tp_qkv_shard_bwd(wl.tp_size, sh.rank, wl.B, wl.S, wl.H, wl.n_heads, sh.d_("X"), sh.d_("Wqkv"),
                        dqkv, o["dX"], o["dW"], o["db"], ws("tp_qkv_shard_bwd", sh))
    return o


def run_attn_bwd(sh, qkv, ctx, lse, dctx):
    wl = sh.wl
    out = empty((wl.T, sh.Nq), sh.dtype)
    bd.tp_attn_heads_bwd(wl.tp_size, sh.rank, wl.B, wl.S, wl.H, wl.n_heads, qkv, ctx, lse, dctx, out,
                         ws("tp_attn_heads_bwd", sh))
    return out


# ---- stage-wise ---------------------------------------------------------------------------------

@pytest.mark.parametrize("wl,dtype,rank", list(cases()))
def test_qkv_fwd(wl, dtype, rank):
    sh = Shard(wl, rank, dtype)
    got = run_qkv_fwd(sh)
    ref = oracle.tp_qkv_shard_fwd(wl.tp_size, rank, wl.B, wl.S, wl.H, wl.n_heads, sh.f64("X"),
                                  sh.f64("Wqkv"), sh.f64("bqkv"))
    assert_close(got, ref, dtype, "QKV_r")


@pytest.mark.parametrize("qkv_std", [0.5, 2.0], ids=["mild", "sharp"])
@pytest.mark.parametrize("wl,dtype,rank", list(cases()))
def test_attn_fwd(wl, dtype, rank, qkv_std):
    sh = Shard(wl, rank, dtype, qkv_std=qkv_std)
    ctx, lse = run_attn_fwd(sh, sh.d_("QKV"))
    rctx, rlse = oracle.tp_attn_heads_fwd(wl.tp_size, rank, wl.B, wl.S, wl.H, wl.n_heads, sh.f64("QKV"))
    assert_close(ctx, rctx, dtype, "ctx_r")
    assert_close(lse, rlse, dtype, "lse_r", tol=1e-5 if dtype == "f32" else 1e-3)


@pytest.mark.parametrize("wl,dtype,rank", list(cases()))
def test_mlp_fwd(wl, dtype, rank):
    sh = Shard(wl, rank, dtype)
    Z, A1, Y = run_mlp_fwd(sh)
    ref = oracle.tp_mlp_shard_fwd(wl.tp_size, rank, wl.T, wl.H, wl.F, sh.f64("X"), sh.f64("W1"),
                                  sh.f64("b1"), sh.f64("W2"), sh.f64("b2"))
    assert_close(A1, ref["A1"], dtype, "A1_r")
    assert_close(Y, ref["Y"], dtype, "Y_r")
    assert_close(Z, ref["Z"], dtype, "Z_r")


@pytest.mark.parametrize("wl,dtype,rank", list(cases()))
def test_mlp_bwd(wl, dtype, rank):
    sh = Shard(wl, rank, dtype)
    o = run_mlp_bwd(sh, sh.d_("A1"), sh.d_("Y"))
    ref = oracle.tp_mlp_shard_bwd(wl.tp_size, rank, wl.T, wl.H, wl.F, sh.f64("X"), sh.f64("W1"),
                                  sh.f64("W2"), sh.f64("A1"), sh.f64("Y"), sh.f64("dZ"))
    for k in ("dX", "dW1", "db1", "dW2"):
        assert_close(o[k], ref[k], dtype, k)
    if rank == 0:
        assert_close(o["db2"], ref["db2"], dtype, "db2")
    else:
        assert torch.isnan(o["db2"]).all(), "db2 is written by rank 0 only"


@pytest.mark.parametrize("wl,dtype,rank", list(cases()))
def test_qkv_bwd(wl, dtype, rank):
    sh = Shard(wl, rank, dtype)
    o = run_qkv_bwd(sh, sh.d_("dQKV"))
    ref = oracle.tp_qkv_shard_bwd(wl.tp_size, rank, wl.B, wl.S, wl.H, wl.n_heads, sh.f64("X"),
                                  sh.f64("Wqkv"), sh.f64("dQKV"))
    assert_close(o["dX"], ref["dX"], dtype, "dX_r")
    assert_close(o["dW"], ref["dW"], dtype, "dWqkv_r")
    assert_close(o["db"], ref["db"], dtype, "dbqkv_r")


@pytest.mark.parametrize("qkv_std", [0.5, 2.0], ids=["mild", "sharp"])
@pytest.mark.parametrize("wl,dtype,rank", list(cases()))
def test_attn_bwd(wl, dtype, rank, qkv_std):
    sh = Shard(wl, rank, dtype, qkv_std=qkv_std)
    qkv = sh.d_("QKV")
    ctx, lse = run_attn_fwd(sh, qkv)
    got = run_attn_bwd(sh, qkv, ctx, lse, sh.d_("dctx"))
    ref = oracle.tp_attn_heads_bwd(wl.tp_size, rank, wl.B, wl.S, wl.H, wl.n_heads, sh.f64("QKV"),
                                   sh.f64("dctx"))
    assert_close(got, ref, dtype, "dQKV_r")
    # the q, k and v parts separately, so a small part cannot hide behind a large one
    g = host(got).reshape(wl.T, sh.nh, 3, sh.d)
    r = ref.reshape(wl.T, sh.nh, 3, sh.d)
    for part, name in enumerate("qkv"):
        assert_close(g[:, :, part], r[:, :, part], dtype, f"d{name}")


# ---- the whole shard, chained --------------------------------------------------------------------

@pytest.mark.parametrize("wl,dtype,rank", list(cases()))
def test_chain(wl, dtype, rank, lse_tol=None):
    """QKV -> attention -> MLP forward, then MLP, attention and QKV backward, all on the GPU, each
    stage fed the previous stage's device output; the oracle runs the same chain in fp64.
    lse_tol overrides the LSE bound (see the single-token case)."""
    sh = Shard(wl, rank, dtype)
    t, B, S, H, nh, F = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F
    qkv = run_qkv_fwd(sh)
    ctx, lse = run_attn_fwd(sh, qkv)
    Z, A1, Y = run_mlp_fwd(sh)
    m = run_mlp_bwd(sh, A1, Y)
    dqkv = run_attn_bwd(sh, qkv, ctx, lse, sh.d_("dctx"))
    q = run_qkv_bwd(sh, dqkv)
    torch.cuda.synchronize()
    R_qkv = oracle.tp_qkv_shard_fwd(t, rank, B, S, H, nh, sh.f64("X"), sh.f64("Wqkv"), sh.f64("bqkv"))
    R_ctx, R_lse = oracle.tp_attn_heads_fwd(t, rank, B, S, H, nh, R_qkv)
    R = oracle.tp_mlp_shard_fwd(t, rank, B * S, H, F, sh.f64("X"), sh.f64("W1"), sh.f64("b1"),
                                sh.f64("W2"), sh.f64("b2"))
    Rm = oracle.tp_mlp_shard_bwd(t, rank, B * S, H, F, sh.f64("X"), sh.f64("W1"), sh.f64("W2"),
                                 R["A1"], R["Y"], sh.f64("dZ"))
    R_dqkv = oracle.tp_attn_heads_bwd(t, rank, B, S, H, nh, R_qkv, sh.f64("dctx"))
    Rq = oracle.tp_qkv_shard_bwd(t, rank, B, S, H, nh, sh.f64("X"), sh.f64("Wqkv"), R_dqkv)
    pairs = [(qkv, R_qkv, "QKV"), (ctx, R_ctx, "ctx"), (Z, R["Z"], "Z"), (Y, R["Y"], "Y"),
             (A1, R["A1"], "A1"), (m["dX"], Rm["dX"], "mlp dX"), (m["dW1"], Rm["dW1"], "dW1"),
             (m["db1"], Rm["db1"], "db1"), (m["dW2"], Rm["dW2"], "dW2"), (dqkv, R_dqkv, "dQKV"),
             (q["dX"], Rq["dX"], "qkv dX"), (q["dW"], Rq["dW"], "dWqkv"), (q["db"], Rq["db"], "dbqkv")]
    for got, ref, what in pairs:
        assert_close(got, ref, dtype, what)
    if lse_tol is None:
        lse_tol = 1e-5 if dtype == "f32" else 2e-3
    assert_close(lse, R_lse, dtype, "lse", tol=lse_tol)


# ---- sharding identity on the GPU ---------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("wl", [TINY, RAGGED, UNEVEN, D32, RAGGED8], ids=lambda w: w.name)
def test_sharding_identity(wl, dtype):
    """Run every rank's shard in sequence on the one GPU; the fp32 sum of the partials Z_r and dX_r
    and the concatenation of the column outputs equal the unsharded layer (oracle) and the GPU's
    own tp=1 run."""
    t = wl.tp_size
    Zsum = torch.zeros(wl.T, wl.H, dtype=torch.float32, device="cuda")
    dXsum = torch.zeros_like(Zsum)
    qkv_cols, ctx_cols = [], []
    for r in range(t):
        sh = Shard(wl, r, dtype)
        Z, A1, Y = run_mlp_fwd(sh)
        Zsum += Z.float()
        dXsum += run_mlp_bwd(sh, A1, Y)["dX"].float()
        qkv = run_qkv_fwd(sh)
        qkv_cols.append(qkv)
        ctx_cols.append(run_attn_fwd(sh, qkv)[0])
    # oracle: the unsharded layer from the full tensors
    full = Shard(LayerWorkload(wl.name + "_tp1", wl.B, wl.S, wl.H, wl.n_heads, wl.F, 1, (0,), wl.w_std),
                 0, dtype)
    ref = oracle.layer_fwd(full.f64("X"), full.f64("Wqkv"), full.f64("bqkv"), full.f64("W1"),
                           full.f64("b1"), full.f64("W2"), full.f64("b2"), wl.B, wl.S, wl.n_heads)
    refb = oracle.mlp_bwd(full.f64("X"), full.f64("W1"), full.f64("W2"), ref["A1"], ref["Y"],
                          full.f64("dZ"), True)
    assert_close(Zsum, ref["Z"], dtype, "sum_r Z_r vs unsharded Z")
    assert_close(dXsum, refb["dX"], dtype, "sum_r dX_r vs unsharded dX")
    assert_close(torch.cat(qkv_cols, 1), ref["QKV"], dtype, "concat QKV_r")
    assert_close(torch.cat(ctx_cols, 1), ref["ctx"], dtype, "concat ctx_r")
    # the GPU's own unsharded run
    Z1, _, _ = run_mlp_fwd(full)
    e = oracle.normwise_error(host(Zsum), host(Z1))
    assert e <= (2e-2 if dtype == "bf16" else 1e-5), f"GPU sum of partials vs GPU tp=1: {e:.2e}"


# ---- robustness ---------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_deterministic(dtype):
    sh = Shard(RAGGED, 0, dtype, qkv_std=1.5)
    runs = []
    for _ in range(2):
        qkv = run_qkv_fwd(sh)
        ctx, lse = run_attn_fwd(sh, sh.d_("QKV"))
        Z, A1, Y = run_mlp_fwd(sh)
        m = run_mlp_bwd(sh, A1, Y)
        da = run_attn_bwd(sh, sh.d_("QKV"), ctx, lse, sh.d_("dctx"))
        q = run_qkv_bwd(sh, da)
        runs.append([qkv, ctx, lse, Z, A1, Y, da] + list(m.values()) + list(q.values()))
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                           b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))


def _guarded(shape, dtype, n_guard=4096):
    """A contiguous view followed by a guard band of sentinel values in the same allocation."""
    n = int(np.prod(shape))
    buf = torch.empty(n + n_guard, dtype=TORCH_DT[dtype] if isinstance(dtype, str) else dtype,
                      device="cuda")
    buf.fill_(-7776.0)   # exactly representable in bf16 and fp32
    return buf[:n].view(shape), buf[n:]


@pytest.mark.parametrize("dtype", DTYPES)
def test_no_out_of_bounds_writes(dtype):
    wl = RAGGED
    sh = Shard(wl, 1, dtype, qkv_std=1.0)
    guards = []

    def out(shape, dt=None):
        v, g = _guarded(shape, dt or dtype)
        guards.append(g)
        return v

    t, B, S, H, nh, F = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F
    qkv = out((wl.T, sh.Nq))
    bd.tp_qkv_shard_fwd(t, 1, B, S, H, nh, sh.d_("X"), sh.d_("Wqkv"), sh.d_("bqkv"), qkv)
    ctx, lse = out((wl.T, sh.nh * sh.d)), out((B, sh.nh, S), torch.float32)
    bd.tp_attn_heads_fwd(t, 1, B, S, H, nh, sh.d_("QKV"), ctx, lse)
    Z, A1, Y = out((wl.T, H)), out((wl.T, sh.Fr)), out((wl.T, sh.Fr))
    bd.tp_mlp_shard_fwd(t, 1, wl.T, H, F, sh.d_("X"), sh.d_("W1"), sh.d_("b1"), sh.d_("W2"), sh.d_("b2"),
                        Z, A1, Y)
    dX, dW1, db1, dW2 = out((wl.T, H)), out((H, sh.Fr)), out((sh.Fr,)), out((sh.Fr, H))
    bd.tp_mlp_shard_bwd(t, 1, wl.T, H, F, sh.d_("X"), sh.d_("W1"), sh.d_("W2"), A1, Y, sh.d_("dZ"),
                        dX, dW1, db1, dW2, None, ws("tp_mlp_shard_bwd", sh))
    dq = out((wl.T, sh.Nq))
    bd.tp_attn_heads_bwd(t, 1, B, S, H, nh, sh.d_("QKV"), ctx, lse, sh.d_("dctx"), dq,
                         ws("tp_attn_heads_bwd", sh))
    dXq, dWq, dbq = out((wl.T, H)), out((H, sh.Nq)), out((sh.Nq,))
    bd.tp_qkv_shard_bwd(t, 1, B, S, H, nh, sh.d_("X"), sh.d_("Wqkv"), dq, dXq, dWq, dbq,
                        ws("tp_qkv_shard_bwd", sh))
    torch.cuda.synchronize()
    for i, g in enumerate(guards):
        assert (g.float() == -7776.0).all(), f"guard band {i} overwritten"


@pytest.mark.parametrize("dtype", DTYPES)
def test_empty_batch(dtype):
    """T = 0: forward calls do nothing; weight and bias gradients are exact zeros."""
    wl = LayerWorkload("empty", 0, 16, 64, 4, 256, 2, (0,), 0.02)
    sh = Shard(TINY, 0, dtype)
    e = torch.empty(0, 64, dtype=TORCH_DT[dtype], device="cuda")
    dW1, db1 = empty((64, 128), dtype), empty((128,), dtype)
    dW2, db2 = empty((128, 64), dtype), empty((64,), dtype)
    a = torch.empty(0, 128, dtype=TORCH_DT[dtype], device="cuda")
    wsz = bd.workspace("tp_mlp_shard_bwd", 2, 0, 0, 16, 64, 4, 256, TORCH_DT[dtype])
    bd.tp_mlp_shard_bwd(2, 0, 0, 64, 256, e, sh.d_("W1"), sh.d_("W2"), a, a, e, e, dW1, db1, dW2, db2, wsz)
    dWq, dbq = empty((64, 96), dtype), empty((96,), dtype)
    q = torch.empty(0, 96, dtype=TORCH_DT[dtype], device="cuda")
    wsq = bd.workspace("tp_qkv_shard_bwd", 2, 0, 0, 16, 64, 4, 256, TORCH_DT[dtype])
    bd.tp_qkv_shard_bwd(2, 0, 0, 16, 64, 4, e, sh.d_("Wqkv"), q, e, dWq, dbq, wsq)
    torch.cuda.synchronize()
    for t_ in (dW1, db1, dW2, db2, dWq, dbq):
        assert (t_ == 0).all()
    assert wl.T == 0


# ---- grouped expert MLP shard -----------------------------------------------------------------

GROUP_CASES = {
    "tiled_ragged": ([0, 5, 300, 1, 257, 77], 0),        # 640 rows: tiled path, ragged and empty groups
    "tiled_aligned": ([256, 512, 0, 256], 0),
    "generic_ragged": ([3, 0, 200, 131, 300], 7),         # 634 + 7 rows: generic path, untouched tail
}


def _grouped_inputs(sizes, extra, dtype, H=192, F_group=128, tp=2, rank=1, std=0.05):
    G = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(off[-1]) + extra
    _, Fr = oracle.shard_range(F_group, tp, rank)
    ops = dict(X=synth.normal("Xperm", (rows, H), 1.0, dtype),
               W1=synth.normal("W1g", (G, H, Fr), std, dtype),
               b1=synth.normal("b1g", (G, Fr), std, dtype),
               W2=synth.normal("W2g", (G, Fr, H), std, dtype))
    return off, rows, Fr, ops


def _run_grouped(off, rows, H, F_group, tp, rank, ops, dtype, Fr):
    G = len(off) - 1
    Z, A1, Y = empty((rows, H), dtype), empty((rows, Fr), dtype), empty((rows, Fr), dtype)
    ws = bd.workspace("tp_mlp_grouped_shard_fwd", tp, rank, 1, rows, H, G, F_group, TORCH_DT[dtype])
    bd.tp_mlp_grouped_shard_fwd(tp, rank, G, torch.from_numpy(off).to("cuda"), rows, H, F_group,
                                dev(ops["X"]), dev(ops["W1"]), dev(ops["b1"]), dev(ops["W2"]), Z, A1, Y, ws)
    torch.cuda.synchronize()
    return Z, A1, Y


@pytest.mark.parametrize("dtype", DTYPES)
def test_grouped_mlp_long_k(dtype):
    """fc1 with k = H = 2056 (>= 2048: the ping-pong 256 x 256 tile for the bf16 path, with a ragged
    k tail) over ragged and empty groups."""
    H, F_group, tp, rank = 2056, 512, 2, 0
    off, rows, Fr, ops = _grouped_inputs([300, 0, 513, 1], 0, dtype, H, F_group, tp, rank, std=0.02)
    Z, A1, Y = _run_grouped(off, rows, H, F_group, tp, rank, ops, dtype, Fr)
    f = {k: v.f64 for k, v in ops.items()}
    ref = oracle.tp_mlp_grouped_shard_fwd(tp, rank, off, f["X"], f["W1"], f["b1"], f["W2"])
    a1 = np.zeros((rows, Fr))
    for e in range(len(off) - 1):
        a1[off[e]:off[e + 1]] = f["X"][off[e]:off[e + 1]] @ f["W1"][e] + f["b1"][e]
    assert_close(A1, a1, dtype, "A1 (long k)")
    assert_close(Y, oracle.gelu(a1), dtype, "Y (long k)")
    assert_close(Z, ref, dtype, "Z (long k)")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("case", sorted(GROUP_CASES))
def test_grouped_mlp(case, dtype):
    sizes, extra = GROUP_CASES[case]
    H, F_group, tp, rank = 192, 128, 2, 1
    off, rows, Fr, ops = _grouped_inputs(sizes, extra, dtype, H, F_group, tp, rank)
    Z, A1, Y = _run_grouped(off, rows, H, F_group, tp, rank, ops, dtype, Fr)
    f = {k: v.f64 for k, v in ops.items()}
    ref = oracle.tp_mlp_grouped_shard_fwd(tp, rank, off, f["X"], f["W1"], f["b1"], f["W2"])
    n = int(off[-1])
    assert_close(host(Z)[:n], ref[:n], dtype, "Z_r grouped")
    for e in range(len(sizes)):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            r = oracle.mlp_fwd(f["X"][lo:hi], f["W1"][e], f["b1"][e], f["W2"][e], None)
            assert_close(host(Y)[lo:hi], r["Y"], dtype, f"Y expert {e}")
            assert_close(host(A1)[lo:hi], r["A1"], dtype, f"A1 expert {e}")
    if extra:
        assert torch.isnan(Z[n:]).all() and torch.isnan(Y[n:]).all(), "rows past the last group untouched"


@pytest.mark.parametrize("dtype", DTYPES)
def test_grouped_mlp_malformed_offsets(dtype):
    """Decreasing offsets and offsets past the end are clamped (prev <= off[e] <= rows) before use."""
    H, F_group, tp, rank = 192, 128, 2, 0
    raw_off = np.array([0, 300, 100, 500, 900], dtype=np.int32)      # 900 > rows = 640
    _, rows, Fr, ops = _grouped_inputs([300, 0, 200, 140], 0, dtype, H, F_group, tp, rank)
    Z, A1, Y = _run_grouped(raw_off, rows, H, F_group, tp, rank, ops, dtype, Fr)
    clamped = np.array([0, 300, 300, 500, 640])
    f = {k: v.f64 for k, v in ops.items()}
    ref = oracle.tp_mlp_grouped_shard_fwd(tp, rank, clamped, f["X"], f["W1"], f["b1"], f["W2"])
    assert_close(Z, ref, dtype, "Z_r with clamped offsets")


def test_grouped_mlp_many_groups():
    """More groups than the plan kernel's threads (its passes carry the running offset and tile
    counts), with empty groups and a decreasing offset that the running maximum clamps."""
    sizes = [int(v) for v in np.random.default_rng(17).integers(0, 4, 1500)]
    H, F_group, tp, rank, dtype = 64, 32, 2, 0, "bf16"
    off, rows, Fr, ops = _grouped_inputs(sizes, 0, dtype, H, F_group, tp, rank)
    raw = off.copy()
    raw[700] = raw[650]                      # decreasing: clamped up to off[699]
    Z, A1, Y = _run_grouped(raw, rows, H, F_group, tp, rank, ops, dtype, Fr)
    clamped = np.maximum.accumulate(np.minimum(raw, rows))
    f = {k: v.f64 for k, v in ops.items()}
    ref = oracle.tp_mlp_grouped_shard_fwd(tp, rank, clamped, f["X"], f["W1"], f["b1"], f["W2"])
    assert_close(Z, ref, dtype, "Z_r over 1500 groups")


def test_grouped_mlp_deterministic():
    off, rows, Fr, ops = _grouped_inputs([0, 5, 300, 1, 257, 77], 0, "bf16")
    a = _run_grouped(off, rows, 192, 128, 2, 1, ops, "bf16", Fr)[0]
    b = _run_grouped(off, rows, 192, 128, 2, 1, ops, "bf16", Fr)[0]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
