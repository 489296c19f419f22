"""GPU parity of the MoE route -> dispatch -> experts -> combine path: tp_moe_route against the
oracle's routing (the integer outputs bit for bit — expert choice, offsets, row order and its
inverse — and the gates to the fp32 bar), and tp_moe_shard_fwd (fc1 with the dispatch gathered in
its operand loads, GeLU, fc2, gate-weighted combine) against the oracle's block on the same routing.
Expected values come from the oracle only.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import TORCH_DT, assert_close, dev, empty, host
from test_gpu_graph import _capture
from tensor_transformer_layer_mlp_amd import binding as bd, synth

pytestmark = pytest.mark.gpu


def _logits(tokens, E, tag, ties=False):
    lg = synth._rng(tag, 0).standard_normal((tokens, E), dtype=np.float32)
    if ties:                      # few distinct values: many exact ties between experts
        lg = np.round(lg * 2.0).astype(np.float32) / np.float32(2.0)
    return lg


def _route_gpu(lg, k):
    tokens, E = lg.shape
    i32 = dict(dtype=torch.int32, device="cuda")
    L = torch.from_numpy(np.ascontiguousarray(lg)).cuda()
    o = dict(gates=torch.full((tokens, k), float("nan"), device="cuda"), experts=torch.full((tokens, k), -7, **i32),
             offsets=torch.full((E + 1,), -7, **i32), row_token=torch.full((tokens * k,), -7, **i32),
             token_row=torch.full((tokens, k), -7, **i32))
    ws = bd.workspace("tp_moe_route", 1, 0, 1, tokens, 1, E, 1, torch.float32)
    bd.tp_moe_route(tokens, E, k, L, o["gates"], o["experts"], o["offsets"], o["row_token"], o["token_row"], ws)
    torch.cuda.synchronize()
    return o


ROUTE_CASES = [(37, 8, 2, False), (1000, 64, 8, False), (1000, 128, 8, True), (301, 200, 5, True),
               (64, 1024, 32, False), (5, 3, 3, True), (1, 1, 1, False), (0, 16, 4, False)]


@pytest.mark.parametrize("tokens,E,k,ties", ROUTE_CASES, ids=[f"t{t}_e{e}_k{k}{'_ties' if ti else ''}"
                                                            for t, e, k, ti in ROUTE_CASES])
def test_moe_route(tokens, E, k, ties):
    lg = _logits(tokens, E, f"route_{tokens}_{E}", ties)
    g = _route_gpu(lg, k)
    r = oracle.moe_route(lg, k)
    assert np.array_equal(host(g["experts"]).astype(np.int64), r["experts"]), "expert choice"
    assert np.array_equal(host(g["offsets"]).astype(np.int64), r["group_offsets"]), "group offsets"
    assert np.array_equal(host(g["row_token"]).astype(np.int64), r["row_token"]), "row -> token"
    assert np.array_equal(host(g["token_row"]).astype(np.int64), r["token_row"]), "(token, j) -> row"
    if tokens:
        assert_close(g["gates"], r["gates"], "f32", "gates")


@pytest.mark.parametrize("E", [16, 128, 300])
def test_moe_route_signed_zeros(E):
    """Logits of +0.0 and -0.0 compare equal (the fp32 comparison the routing is defined by), so the
    lower expert id wins between them whichever sign each has: rows mixing both signs of zero with
    negative values, per expert count that takes each kernel form (rows of 16 lanes, whole waves)."""
    tokens, k = 70, 6
    lg = -np.abs(synth._rng(f"zeros_{E}", 0).standard_normal((tokens, E), dtype=np.float32)) - np.float32(1)
    sel = synth._rng(f"zeros_{E}", 1).integers(0, 3, size=(tokens, E))
    lg[sel == 0] = np.float32(0.0)
    lg[sel == 1] = np.float32(-0.0)
    g = _route_gpu(lg, k)
    r = oracle.moe_route(lg, k)
    assert np.array_equal(host(g["experts"]).astype(np.int64), r["experts"]), "expert choice"
    assert np.array_equal(host(g["offsets"]).astype(np.int64), r["group_offsets"]), "group offsets"
    assert_close(g["gates"], r["gates"], "f32", "gates")


def _expert_weights(E, H, F_expert, tp, rank, dtype, std=0.05):
    f0, Fr = oracle.shard_range(F_expert, tp, rank)
    return Fr, dict(W1=synth.normal("moeW1", (E, H, Fr), std, dtype), b1=synth.normal("moeb1", (E, Fr), std, dtype),
                    W2=synth.normal("moeW2", (E, Fr, H), std, dtype))


def _run_block(tp, rank, tokens, H, E, k, F_expert, dtype, X, route, W, Fr):
    n = tokens * k
    out, Z, Y, A1 = empty((tokens, H), dtype), empty((n, H), dtype), empty((n, Fr), dtype), empty((n, Fr), dtype)
    ws = bd.workspace("tp_moe_shard_fwd", tp, rank, 1, n, H, E, F_expert, TORCH_DT[dtype])
    bd.tp_moe_shard_fwd(tp, rank, tokens, H, E, k, F_expert, X, route["gates"], route["offsets"], route["row_token"],
                        route["token_row"], dev(W["W1"]), dev(W["b1"]), dev(W["W2"]), out, Z, A1, Y, ws)
    torch.cuda.synchronize()
    return dict(out=out, Z=Z, Y=Y, A1=A1)


# H = 2048 takes the ping-pong 256 x 256 tile for fc1's long k loop
BLOCK_CASES = [(300, 192, 6, 2, 128, 2, 1), (518, 256, 16, 4, 512, 4, 0), (64, 100, 5, 3, 60, 2, 1),
               (8, 64, 3, 3, 16, 1, 0), (200, 2048, 8, 2, 256, 2, 0)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("tokens,H,E,k,F_expert,tp,rank", BLOCK_CASES,
                         ids=[f"t{c[0]}_h{c[1]}_e{c[2]}_k{c[3]}_f{c[4]}_tp{c[5]}r{c[6]}" for c in BLOCK_CASES])
def test_moe_shard_fwd(tokens, H, E, k, F_expert, tp, rank, dtype):
    print(f"moe block tokens={tokens} H={H} E={E} k={k} F={F_expert} tp={tp} r={rank} {dtype}", flush=True)
    lg = _logits(tokens, E, f"block_{tokens}_{E}")
    route = _route_gpu(lg, k)
    Xop = synth.normal("moeXb", (tokens, H), 1.0, dtype)
    Fr, W = _expert_weights(E, H, F_expert, tp, rank, dtype)
    g = _run_block(tp, rank, tokens, H, E, k, F_expert, dtype, dev(Xop), route, W, Fr)
    r = oracle.moe_route(lg, k)
    ref = oracle.tp_moe_shard_fwd(tp, rank, Xop.f64, r, W["W1"].f64, W["b1"].f64, W["W2"].f64)
    assert_close(g["out"], ref["out"], dtype, "out_r")
    assert_close(g["Z"], ref["Z"], dtype, "Z_r (expert-sorted rows)")
    Xp = Xop.f64[r["row_token"]]
    for e in range(E):
        lo, hi = int(r["group_offsets"][e]), int(r["group_offsets"][e + 1])
        if hi > lo:
            m = oracle.mlp_fwd(Xp[lo:hi], W["W1"].f64[e], W["b1"].f64[e], W["W2"].f64[e], None)
            assert_close(host(g["Y"])[lo:hi], m["Y"], dtype, f"Y expert {e}")
            assert_close(host(g["A1"])[lo:hi], m["A1"], dtype, f"A1 expert {e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_moe_sum_over_ranks(dtype):
    """Every TP rank's block in sequence: the fp32 sum of the out_r partials is the unsharded MoE block."""
    tokens, H, E, k, F_expert, tp = 200, 128, 8, 2, 256, 4
    lg = _logits(tokens, E, "ranks")
    route = _route_gpu(lg, k)
    Xop = synth.normal("moeXr", (tokens, H), 1.0, dtype)
    full_W = dict(W1=synth.normal("moeW1r", (E, H, F_expert), 0.05, dtype),
                  b1=synth.normal("moeb1r", (E, F_expert), 0.05, dtype),
                  W2=synth.normal("moeW2r", (E, F_expert, H), 0.05, dtype))
    total = torch.zeros(tokens, H, dtype=torch.float32, device="cuda")
    for rank in range(tp):
        f0, Fr = oracle.shard_range(F_expert, tp, rank)
        W = {"W1": synth.make_operand(full_W["W1"].f64[:, :, f0:f0 + Fr], dtype),
             "b1": synth.make_operand(full_W["b1"].f64[:, f0:f0 + Fr], dtype),
             "W2": synth.make_operand(full_W["W2"].f64[:, f0:f0 + Fr], dtype)}
        total += _run_block(tp, rank, tokens, H, E, k, F_expert, dtype, dev(Xop), route, W, Fr)["out"].float()
    ref = oracle.tp_moe_shard_fwd(1, 0, Xop.f64, oracle.moe_route(lg, k), full_W["W1"].f64, full_W["b1"].f64,
                                  full_W["W2"].f64)
    assert_close(total, ref["out"], dtype, "sum over ranks of out_r vs unsharded")


def test_moe_malformed_indices_read_zero():
    """Out-of-range gather and combine indices are dropped on the device (zero rows), not followed."""
    tokens, H, E, k, F_expert, dtype = 64, 128, 4, 2, 64, "bf16"
    lg = _logits(tokens, E, "bad")
    route = _route_gpu(lg, k)
    r = oracle.moe_route(lg, k)
    route["row_token"][0] = -3
    route["row_token"][5] = tokens + 1000
    route["token_row"][2, 1] = tokens * k + 7
    Xop = synth.normal("moeXbad", (tokens, H), 1.0, dtype)
    Fr, W = _expert_weights(E, H, F_expert, 1, 0, dtype)
    g = _run_block(1, 0, tokens, H, E, k, F_expert, dtype, dev(Xop), route, W, Fr)
    Xp = Xop.f64[r["row_token"]]
    Xp[0] = 0.0
    Xp[5] = 0.0
    Z = oracle.tp_mlp_grouped_shard_fwd(1, 0, r["group_offsets"], Xp, W["W1"].f64, W["b1"].f64, W["W2"].f64)
    tr = r["token_row"].copy()
    gates = r["gates"].copy()
    gates[2, 1] = 0.0
    assert_close(g["Z"], Z, dtype, "Z_r with zeroed gathered rows")
    assert_close(g["out"], oracle.moe_combine(Z, gates, tr), dtype, "out_r with a dropped combine row")


def test_moe_graph_replay_and_determinism():
    tokens, H, E, k, F_expert, dtype = 256, 256, 8, 2, 128, "bf16"
    lg = torch.from_numpy(_logits(tokens, E, "graph")).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    gates = torch.empty(tokens, k, device="cuda")
    ex, off = torch.empty(tokens, k, **i32), torch.empty(E + 1, **i32)
    rt, tr = torch.empty(tokens * k, **i32), torch.empty(tokens, k, **i32)
    Xop = synth.normal("moeXg", (tokens, H), 1.0, dtype)
    X = dev(Xop)
    Fr, W = _expert_weights(E, H, F_expert, 2, 0, dtype)
    W1, b1, W2 = dev(W["W1"]), dev(W["b1"]), dev(W["W2"])
    n = tokens * k
    out, Z, Y = (torch.empty(*s, dtype=torch.bfloat16, device="cuda") for s in ((tokens, H), (n, H), (n, Fr)))
    ws = bd.workspace("tp_moe_shard_fwd", 2, 0, 1, n, H, E, F_expert, torch.bfloat16)
    wsr = bd.workspace("tp_moe_route", 1, 0, 1, tokens, 1, E, 1, torch.float32)

    def call():
        bd.tp_moe_route(tokens, E, k, lg, gates, ex, off, rt, tr, wsr)
        bd.tp_moe_shard_fwd(2, 0, tokens, H, E, k, F_expert, X, gates, off, rt, tr, W1, b1, W2, out, Z, None, Y, ws)
    call()
    torch.cuda.synchronize()
    bufs = dict(gates=gates, ex=ex, off=off, rt=rt, tr=tr, out=out, Z=Z, Y=Y)
    eager = {k_: v.clone() for k_, v in bufs.items()}
    call()
    torch.cuda.synchronize()
    for k_ in bufs:
        assert torch.equal(bufs[k_], eager[k_]), f"{k_} differs between two eager calls"
    g = _capture(call)
    for rep in range(3):
        for v in bufs.values():
            v.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k_ in bufs:
            assert torch.equal(bufs[k_], eager[k_]), f"replay {rep}: {k_} differs from the eager call"
        call()
        torch.cuda.synchronize()


def test_moe_full_size_rank0():
    """The 128-expert MoE FFN shard at full size (hidden 8192, 16384 tokens, top-8, expert ffn 2048
    -> 256 columns on rank 0 of 8): routing compared whole and bit for bit, out_r on sampled tokens."""
    from tensor_transformer_layer_mlp_amd.configs import MOE_E128 as mw
    tokens, H, E, k, tp, rank, dtype = mw.tokens, mw.H, mw.n_experts, mw.top_k, mw.tp_size, 0, "bf16"
    lg = _logits(tokens, E, "moe_full")
    route = _route_gpu(lg, k)
    r = oracle.moe_route(lg, k)
    for key, rk in (("experts", "experts"), ("offsets", "group_offsets"), ("row_token", "row_token"),
                    ("token_row", "token_row")):
        assert np.array_equal(host(route[key]).astype(np.int64), r[rk]), key
    f0, Fr = oracle.shard_range(mw.F_expert, tp, rank)
    Xop = synth.normal("moeX", (tokens, H), 1.0, dtype)
    W1 = torch.empty(E, H, Fr, dtype=torch.bfloat16, device="cuda")
    b1 = torch.empty(E, Fr, dtype=torch.bfloat16, device="cuda")
    W2 = torch.empty(E, Fr, H, dtype=torch.bfloat16, device="cuda")
    host_w = {}
    for e in range(E):
        w1 = synth.column_blocks(f"W1_e{e}", H, f0, f0 + Fr, mw.w_std, dtype)
        bb = synth.vector_blocks(f"b1_e{e}", f0, f0 + Fr, mw.w_std, dtype)
        w2 = synth.row_blocks(f"W2_e{e}", H, f0, f0 + Fr, mw.w_std, dtype)
        W1[e], b1[e], W2[e] = dev(w1), dev(bb), dev(w2)
        host_w[e] = (w1.f64, bb.f64, w2.f64)
    n = tokens * k
    out = torch.empty(tokens, H, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(n, H, dtype=torch.bfloat16, device="cuda")
    Y = torch.empty(n, Fr, dtype=torch.bfloat16, device="cuda")
    ws = bd.workspace("tp_moe_shard_fwd", tp, rank, 1, n, H, E, mw.F_expert, torch.bfloat16)
    bd.tp_moe_shard_fwd(tp, rank, tokens, H, E, k, mw.F_expert, dev(Xop), route["gates"], route["offsets"],
                        route["row_token"], route["token_row"], W1, b1, W2, out, Z, None, Y, ws)
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([[0, tokens - 1], np.random.default_rng(3).integers(0, tokens, 24)]))
    ref = np.zeros((len(pick), H))
    for i, t in enumerate(pick):
        for j in range(k):
            e = int(r["experts"][t, j])
            w1, bb, w2 = host_w[e]
            ref[i] += r["gates"][t, j] * oracle.mlp_fwd(Xop.f64[t:t + 1], w1, bb, w2, None)["Z"][0]
    assert_close(host(out)[pick], ref, dtype, "out_r sampled tokens")
