"""GPU parity of the MoE backward against the oracle: tp_mlp_grouped_shard_bwd on expert-sorted rows
(ragged and empty experts, tiled and generic GEMM paths, dX_perm sharing dZ_perm's buffer),
tp_moe_shard_bwd (the combine's backward folded into the experts' grouped backward with the k
dimension split by expert, the gate gradients from the dA1 GEMM's row dots, the dispatch's backward)
on the GPU forward's own A1 / Y (stage-wise), its
determinism, and tp_moe_route_bwd (the router's logit gradient); the 128-expert rank-0 shard at full
size on sampled experts and tokens.  Expected values come from the oracle only.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import TORCH_DT, assert_close, dev, empty, host
from test_gpu_moe import _expert_weights, _logits, _route_gpu, _run_block
from tensor_transformer_layer_mlp_amd import binding as bd, synth

pytestmark = pytest.mark.gpu


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


# (rows per group, H, F_group, tp, rank): ragged groups, an empty group at each end and inside, a
# group of one row; H = 100 and F_r = 30 take the generic kernels; H = 2056 the long-k tile
GCASES = [([300, 0, 17, 512, 1], 256, 256, 2, 0), ([0, 64, 0, 200, 0], 128, 96, 1, 0),
          ([5, 1, 40], 100, 60, 2, 1), ([1000, 24], 512, 1024, 4, 3),
          ([300, 0, 513, 1], 2056, 512, 2, 1)]      # k = H >= 2048: the ping-pong tile, a ragged k tail


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,H,Fg,tp,rank", GCASES, ids=[f"g{len(c[0])}_h{c[1]}_f{c[2]}_tp{c[3]}r{c[4]}"
                                                            for c in GCASES])
def test_grouped_mlp_bwd(counts, H, Fg, tp, rank, dtype):
    print(f"grouped bwd counts={counts} H={H} F={Fg} tp={tp} r={rank} {dtype}", flush=True)
    G, rows = len(counts), int(sum(counts))
    off = _offsets(counts)
    f0, Fr = oracle.shard_range(Fg, tp, rank)
    X = synth.normal(f"gbX_{rows}_{H}", (rows, H), 1.0, dtype)
    W1 = synth.normal(f"gbW1_{G}_{H}_{Fr}", (G, H, Fr), 0.05, dtype)
    b1 = synth.normal(f"gbb1_{G}_{Fr}", (G, Fr), 0.05, dtype)
    W2 = synth.normal(f"gbW2_{G}_{Fr}_{H}", (G, Fr, H), 0.05, dtype)
    dZ = synth.normal(f"gbdZ_{rows}_{H}", (rows, H), 1.0, dtype)
    # the forward's A1 and Y as stored (rounded to the storage type once)
    A1 = np.zeros((rows, Fr))
    for e in range(G):
        A1[off[e]:off[e + 1]] = X.f64[off[e]:off[e + 1]] @ W1.f64[e] + b1.f64[e]
    A1op = synth.make_operand(A1, dtype)
    Yop = synth.make_operand(oracle.gelu(A1op.f64), dtype)
    dX, dW1, db1, dW2 = (empty(s, dtype) for s in ((rows, H), (G, H, Fr), (G, Fr), (G, Fr, H)))
    ws = bd.workspace("tp_mlp_grouped_shard_bwd", tp, rank, 1, rows, H, G, Fg, TORCH_DT[dtype])
    offs = torch.from_numpy(off.astype(np.int32)).cuda()
    bd.tp_mlp_grouped_shard_bwd(tp, rank, offs, H, Fg, dev(X), dev(W1), dev(W2), dev(A1op), dev(Yop), dev(dZ),
                                dX, dW1, db1, dW2, ws)
    torch.cuda.synchronize()
    ref = oracle.tp_mlp_grouped_shard_bwd(off, X.f64, W1.f64, W2.f64, A1op.f64, Yop.f64, dZ.f64)
    assert_close(dX, ref["dX_perm"], dtype, "dX_perm")
    for k in ("dW1", "db1", "dW2"):
        got = host({"dW1": dW1, "db1": db1, "dW2": dW2}[k])
        for e in range(G):
            if counts[e] == 0:
                assert np.all(got[e] == 0), f"{k}[{e}] of an empty expert is not zero"
            else:
                assert_close(got[e], ref[k][e], dtype, f"{k}[{e}]")
    # the same call with dX_perm in dZ_perm's buffer
    dZd = dev(dZ)
    bd.tp_mlp_grouped_shard_bwd(tp, rank, offs, H, Fg, dev(X), dev(W1), dev(W2), dev(A1op), dev(Yop), dZd,
                                dZd, dW1, db1, dW2, ws)
    torch.cuda.synchronize()
    assert torch.equal(dZd, dX), "dX_perm aliasing dZ_perm changed the result"


BWD_CASES = [(300, 192, 6, 2, 128, 2, 1), (518, 256, 16, 4, 512, 4, 0), (64, 100, 5, 3, 60, 2, 1),
             (8, 64, 6, 1, 16, 1, 0), (300, 2056, 6, 2, 512, 2, 1)]   # the last: k = H on the long-k tile


def _moe_bwd(tp, rank, tokens, H, E, k, F_expert, dtype, X, route, W, fwd, d_out, z_none=False):
    n = tokens * k
    z = None if z_none else fwd["Z"]        # the backward does not read Z_r
    Fr = fwd["Y"].shape[1]
    o = dict(dX=empty((tokens, H), dtype), dgates=empty((tokens, k), "f32"), dW1=empty((E, H, Fr), dtype),
             db1=empty((E, Fr), dtype), dW2=empty((E, Fr, H), dtype))
    ws = bd.workspace("tp_moe_shard_bwd", tp, rank, 1, n, H, E, F_expert, TORCH_DT[dtype])
    bd.tp_moe_shard_bwd(tp, rank, tokens, H, E, k, F_expert, X, route["gates"], route["offsets"], route["row_token"],
                        route["token_row"],
                        dev(W["W1"]), dev(W["W2"]), fwd["A1"], fwd["Y"], z, d_out, o["dX"], o["dgates"],
                        o["dW1"], o["db1"], o["dW2"], ws)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("tokens,H,E,k,F_expert,tp,rank", BWD_CASES,
                         ids=[f"t{c[0]}_h{c[1]}_e{c[2]}_k{c[3]}_f{c[4]}_tp{c[5]}r{c[6]}" for c in BWD_CASES])
def test_moe_shard_bwd(tokens, H, E, k, F_expert, tp, rank, dtype):
    print(f"moe bwd tokens={tokens} H={H} E={E} k={k} F={F_expert} tp={tp} r={rank} {dtype}", flush=True)
    lg = _logits(tokens, E, f"bwd_{tokens}_{E}")
    route = _route_gpu(lg, k)
    Xop = synth.normal("moeXbw", (tokens, H), 1.0, dtype)
    Fr, W = _expert_weights(E, H, F_expert, tp, rank, dtype)
    X = dev(Xop)
    fwd = _run_block(tp, rank, tokens, H, E, k, F_expert, dtype, X, route, W, Fr)
    dop = synth.normal("moedout", (tokens, H), 1.0, dtype)
    g = _moe_bwd(tp, rank, tokens, H, E, k, F_expert, dtype, X, route, W, fwd, dev(dop))
    r = oracle.moe_route(lg, k)
    ref = oracle.tp_moe_shard_bwd(tp, rank, Xop.f64, r, W["W1"].f64, W["W2"].f64,
                                  {key: host(fwd[key]) for key in ("A1", "Y", "Z")}, dop.f64)
    assert_close(g["dX"], ref["dX"], dtype, "dX_r")
    assert_close(g["dgates"], ref["dgates"], dtype, "dgates_r", tol=1e-4)
    counts = np.diff(r["group_offsets"])
    for key in ("dW1", "db1", "dW2"):
        got = host(g[key])
        for e in range(E):
            if counts[e] == 0:
                assert np.all(got[e] == 0), f"{key}[{e}] of an expert without tokens is not zero"
            else:
                assert_close(got[e], ref[key][e], dtype, f"{key}[{e}]")
    # deterministic: a second call gives the same bits (this one without Z_r)
    g2 = _moe_bwd(tp, rank, tokens, H, E, k, F_expert, dtype, X, route, W, fwd, dev(dop), z_none=True)
    for key in g:
        assert torch.equal(g[key], g2[key]), f"{key} differs between two calls"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_moe_shard_bwd_skewed_routing(dtype):
    """Router logits biased so that three experts take nearly every token's three choices: expert
    groups of several m-tiles next to a one-row group and eight empty ones in the gathered, gated
    dA1 GEMM, its row dots over several n-tiles (F_r = 640: three 256-wide tiles, the last ragged) and
    the weight gradients' k ranges; against the oracle, and repeatable bit for bit."""
    tokens, H, E, k, F_expert, tp, rank = 700, 256, 12, 3, 1280, 2, 1
    lg = _logits(tokens, E, "bwd_skew")
    lg[:, 0] += 7.0
    lg[:, 7] += 6.0
    lg[:, 3] += 5.0
    route = _route_gpu(lg, k)
    r = oracle.moe_route(lg, k)
    counts = np.diff(r["group_offsets"])
    # (the seeded draw gives 700, 700, 699 rows, one expert with a single row, eight without any)
    assert counts.max() == tokens and (counts == 0).sum() == 8 and (counts == 1).sum() == 1, counts
    Xop = synth.normal("moeXskew", (tokens, H), 1.0, dtype)
    Fr, W = _expert_weights(E, H, F_expert, tp, rank, dtype)
    X = dev(Xop)
    fwd = _run_block(tp, rank, tokens, H, E, k, F_expert, dtype, X, route, W, Fr)
    dop = synth.normal("moedskew", (tokens, H), 1.0, dtype)
    g = _moe_bwd(tp, rank, tokens, H, E, k, F_expert, dtype, X, route, W, fwd, dev(dop))
    ref = oracle.tp_moe_shard_bwd(tp, rank, Xop.f64, r, W["W1"].f64, W["W2"].f64,
                                  {key: host(fwd[key]) for key in ("A1", "Y", "Z")}, dop.f64)
    assert_close(g["dX"], ref["dX"], dtype, "dX_r")
    assert_close(g["dgates"], ref["dgates"], dtype, "dgates_r", tol=1e-4)
    for key in ("dW1", "db1", "dW2"):
        got = host(g[key])
        for e in range(E):
            if counts[e] == 0:
                assert np.all(got[e] == 0), f"{key}[{e}] of an expert without tokens is not zero"
            else:
                assert_close(got[e], ref[key][e], dtype, f"{key}[{e}]")
    g2 = _moe_bwd(tp, rank, tokens, H, E, k, F_expert, dtype, X, route, W, fwd, dev(dop), z_none=True)
    for key in g:
        assert torch.equal(g[key], g2[key]), f"{key} differs between two calls"


RB_CASES = [(37, 8, 2), (500, 64, 8), (300, 128, 8), (77, 200, 5), (16, 1024, 32), (5, 3, 3), (1, 1, 1)]


@pytest.mark.parametrize("tokens,E,k", RB_CASES, ids=[f"t{t}_e{e}_k{k}" for t, e, k in RB_CASES])
def test_moe_route_bwd(tokens, E, k):
    lg = _logits(tokens, E, f"rbwd_{tokens}_{E}")
    r = oracle.moe_route(lg, k)
    dg = synth._rng(f"rbwd_dg_{tokens}", 0).standard_normal((tokens, k), dtype=np.float32)
    out = torch.full((tokens, E), float("nan"), device="cuda")
    bd.tp_moe_route_bwd(torch.from_numpy(lg).cuda(), torch.from_numpy(r["experts"].astype(np.int32)).cuda(),
                        torch.from_numpy(dg).cuda(), out)
    torch.cuda.synchronize()
    ref = oracle.moe_route_bwd(lg, r["experts"], dg.astype(np.float64))
    if np.linalg.norm(ref) == 0:        # E = k = 1: the gate is 1 whatever the logit
        assert np.all(host(out) == 0)
    else:
        assert_close(out, ref, "f32", "d_logits")


def test_moe_bwd_full_size_rank0():
    """The 128-expert MoE FFN shard's backward at full size (hidden 8192, 16384 tokens, top-8, expert
    ffn 2048 -> 256 columns on rank 0 of 8): the weight gradients of three experts whole, the gate
    and input gradients of sampled tokens, against the oracle on the GPU forward's A1 / Y."""
    from tensor_transformer_layer_mlp_amd.configs import MOE_E128 as mw
    tokens, H, E, k, tp, rank, dtype = mw.tokens, mw.H, mw.n_experts, mw.top_k, mw.tp_size, 0, "bf16"
    lg = _logits(tokens, E, "moe_full")
    route = _route_gpu(lg, k)
    r = oracle.moe_route(lg, k)
    f0, Fr = oracle.shard_range(mw.F_expert, tp, rank)
    bf = torch.bfloat16
    g = torch.Generator(device="cuda")
    g.manual_seed(515)
    W1 = (torch.randn(E, H, Fr, generator=g, device="cuda") * mw.w_std).to(bf)
    b1 = (torch.randn(E, Fr, generator=g, device="cuda") * mw.w_std).to(bf)
    W2 = (torch.randn(E, Fr, H, generator=g, device="cuda") * mw.w_std).to(bf)
    X = torch.randn(tokens, H, generator=g, device="cuda").to(bf)
    d_out = torch.randn(tokens, H, generator=g, device="cuda").to(bf)
    n = tokens * k
    out, Z = torch.empty(tokens, H, dtype=bf, device="cuda"), torch.empty(n, H, dtype=bf, device="cuda")
    A1, Y = torch.empty(n, Fr, dtype=bf, device="cuda"), torch.empty(n, Fr, dtype=bf, device="cuda")
    ws = bd.workspace("tp_moe_shard_fwd", tp, rank, 1, n, H, E, mw.F_expert, bf)
    bd.tp_moe_shard_fwd(tp, rank, tokens, H, E, k, mw.F_expert, X, route["gates"], route["offsets"],
                        route["row_token"], route["token_row"], W1, b1, W2, out, Z, A1, Y, ws)
    del ws
    dX, dg = torch.empty(tokens, H, dtype=bf, device="cuda"), torch.empty(tokens, k, device="cuda")
    dW1, db1, dW2 = torch.empty_like(W1), torch.empty_like(b1), torch.empty_like(W2)
    wsb = bd.workspace("tp_moe_shard_bwd", tp, rank, 1, n, H, E, mw.F_expert, bf)
    bd.tp_moe_shard_bwd(tp, rank, tokens, H, E, k, mw.F_expert, X, route["gates"], route["offsets"],
                        route["row_token"], route["token_row"], W1, W2, A1, Y, Z, d_out, dX, dg, dW1, db1, dW2, wsb)
    torch.cuda.synchronize()
    del wsb
    off, rt, tr, gates = r["group_offsets"], r["row_token"], r["token_row"], r["gates"]
    h = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    Xh, Dh = h(X), h(d_out)
    for e in (0, 57, E - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.arange(lo, hi)
        t_of = rt[rows]
        j_of = np.array([int(np.nonzero(tr[t] == rr)[0][0]) for t, rr in zip(t_of, rows)])
        dZe = gates[t_of, j_of][:, None] * Dh[t_of]
        A1e, Ye = h(A1[lo:hi]), h(Y[lo:hi])
        w1, w2 = h(W1[e]), h(W2[e])
        dA1 = (dZe @ w2.T) * oracle.gelu_grad(A1e)
        assert_close(dW2[e], Ye.T @ dZe, dtype, f"dW2[{e}]")
        assert_close(dW1[e], Xh[t_of].T @ dA1, dtype, f"dW1[{e}]")
        assert_close(db1[e], dA1.sum(axis=0), dtype, f"db1[{e}]")
    pick = np.unique(np.concatenate([[0, tokens - 1], np.random.default_rng(5).integers(0, tokens, 16)]))
    ref_dx, ref_dg = np.zeros((len(pick), H)), np.zeros((len(pick), k))
    for i, t in enumerate(pick):
        for j in range(k):
            e, row = int(r["experts"][t, j]), int(tr[t, j])
            ref_dg[i, j] = float(Dh[t] @ (h(Y[row]) @ h(W2[e])))     # Z[row] = Y[row]·W2[e], not rounded
            dz = gates[t, j] * Dh[t]
            da1 = (dz @ h(W2[e]).T) * oracle.gelu_grad(h(A1[row]))
            ref_dx[i] += da1 @ h(W1[e]).T
    assert_close(host(dX)[pick], ref_dx, dtype, "dX_r sampled tokens")
    assert_close(host(dg)[pick], ref_dg, dtype, "dgates_r sampled tokens", tol=1e-4)


def test_moe_fwd_bwd_graph_replay():
    """Route, block forward, block backward and router backward captured in one HIP graph: three
    replays (buffers scrambled before each, eager calls in between) each equal the eager result."""
    from test_gpu_graph import _capture
    tokens, H, E, k, F_expert, tp, rank, dtype = 256, 256, 8, 2, 256, 2, 1, "bf16"
    n = tokens * k
    lg = torch.from_numpy(_logits(tokens, E, "bwd_graph")).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    gates, ex, off = torch.empty(tokens, k, device="cuda"), torch.empty(tokens, k, **i32), torch.empty(E + 1, **i32)
    rt, tr = torch.empty(n, **i32), torch.empty(tokens, k, **i32)
    X = dev(synth.normal("moeXgb", (tokens, H), 1.0, dtype))
    d_out = dev(synth.normal("moedgb", (tokens, H), 1.0, dtype))
    Fr, W = _expert_weights(E, H, F_expert, tp, rank, dtype)
    W1, b1, W2 = dev(W["W1"]), dev(W["b1"]), dev(W["W2"])
    bf = torch.bfloat16
    e = lambda *s: torch.empty(*s, dtype=bf, device="cuda")  # noqa: E731
    out, Z, Y, A1 = e(tokens, H), e(n, H), e(n, Fr), e(n, Fr)
    dX, dW1, db1, dW2 = e(tokens, H), e(E, H, Fr), e(E, Fr), e(E, Fr, H)
    dg, dlog = torch.empty(tokens, k, device="cuda"), torch.empty(tokens, E, device="cuda")
    wsr = bd.workspace("tp_moe_route", 1, 0, 1, tokens, 1, E, 1, torch.float32)
    wsf = bd.workspace("tp_moe_shard_fwd", tp, rank, 1, n, H, E, F_expert, bf)
    wsb = bd.workspace("tp_moe_shard_bwd", tp, rank, 1, n, H, E, F_expert, bf)

    def call():
        bd.tp_moe_route(tokens, E, k, lg, gates, ex, off, rt, tr, wsr)
        bd.tp_moe_shard_fwd(tp, rank, tokens, H, E, k, F_expert, X, gates, off, rt, tr, W1, b1, W2, out, Z, A1, Y, wsf)
        bd.tp_moe_shard_bwd(tp, rank, tokens, H, E, k, F_expert, X, gates, off, rt, tr, W1, W2, A1, Y, Z, d_out, dX, dg,
                            dW1, db1, dW2, wsb)
        bd.tp_moe_route_bwd(lg, ex, dg, dlog)
    call()
    torch.cuda.synchronize()
    bufs = dict(out=out, Z=Z, Y=Y, A1=A1, dX=dX, dW1=dW1, db1=db1, dW2=dW2, dg=dg, dlog=dlog)
    eager = {key: v.clone() for key, v in bufs.items()}
    g = _capture(call)
    for rep in range(3):
        for v in bufs.values():
            v.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in bufs:
            assert torch.equal(bufs[key], eager[key]), f"replay {rep}: {key} differs from the eager call"
        call()
        torch.cuda.synchronize()
