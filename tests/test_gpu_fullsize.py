"""GPU parity at the full GPT-shaped shard sizes, in the launch configuration the benchmark times.

The GPU runs each entry point on the whole shard.  The oracle checks sampled outputs: rows of
row-separable results (QKV, Z, O, dX, dctx), columns of column-separable ones (dW1, db1, dW2,
dWqkv, dWo, dbo), and whole heads of the attention.  Each sample is the oracle's own function
applied to a row or column block of the inputs, which the column and row split identities make
exact.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import Shard, assert_close, dev, host
from test_gpu_attn_out import run_out_bwd, run_out_fwd
from test_gpu_parity import (run_attn_bwd, run_attn_fwd, run_mlp_bwd, run_mlp_fwd, run_qkv_bwd,
                             run_qkv_fwd)
from tensor_transformer_layer_mlp_amd import binding as bd, synth
from tensor_transformer_layer_mlp_amd.configs import GPT2_1P5B, GPT3_175B, GPT_8P3B  # noqa: F401

pytestmark = pytest.mark.gpu


def sample(n, k, seed):
    g = np.random.default_rng(seed)
    idx = set([0, n - 1]) | set(g.choice(n, size=min(k, n), replace=False).tolist())
    return np.array(sorted(idx))


def check_shard(wl, rank):
    dt = "bf16"
    sh = Shard(wl, rank, dt, qkv_std=1.0)
    t, B, S, H, nh, F = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F
    rows = sample(wl.T, 40, 1 + rank)
    cols_f = sample(sh.Fr, 48, 2 + rank)
    cols_q = sample(sh.Nq, 48, 3 + rank)
    X, W, bq = sh.f64("X"), sh.f64("Wqkv"), sh.f64("bqkv")

    qkv = run_qkv_fwd(sh)
    ref = oracle.tp_qkv_shard_fwd(t, rank, 1, len(rows), H, nh, X[rows], W, bq)
    assert_close(host(qkv)[rows], ref, dt, "QKV_r rows")

    Z, A1, Y = run_mlp_fwd(sh)
    r = oracle.tp_mlp_shard_fwd(t, rank, len(rows), H, F, X[rows], sh.f64("W1"), sh.f64("b1"),
                                sh.f64("W2"), sh.f64("b2"))
    for got, key in ((Z, "Z"), (A1, "A1"), (Y, "Y")):
        assert_close(host(got)[rows], r[key], dt, f"{key} rows")

    m = run_mlp_bwd(sh, sh.d_("A1"), sh.d_("Y"))
    A1h, Yh, dZ = sh.f64("A1"), sh.f64("Y"), sh.f64("dZ")
    rr = oracle.mlp_bwd(X[rows], sh.f64("W1"), sh.f64("W2"), A1h[rows], Yh[rows], dZ[rows], False)
    assert_close(host(m["dX"])[rows], rr["dX"], dt, "dX_r rows")
    rc = oracle.mlp_bwd(X, sh.f64("W1")[:, cols_f], sh.f64("W2")[cols_f], A1h[:, cols_f],
                        Yh[:, cols_f], dZ, rank == 0)
    assert_close(host(m["dW1"])[:, cols_f], rc["dW1"], dt, "dW1_r cols")
    assert_close(host(m["db1"])[cols_f], rc["db1"], dt, "db1_r cols")
    assert_close(host(m["dW2"])[cols_f], rc["dW2"], dt, "dW2_r rows")
    if rank == 0:
        assert_close(m["db2"], rc["db2"], dt, "db2")

    q = run_qkv_bwd(sh, sh.d_("dQKV"))
    dQ = sh.f64("dQKV")
    assert_close(host(q["dX"])[rows], dQ[rows] @ W.T, dt, "qkv dX_r rows")
    rq = oracle.qkv_bwd(X, W[:, cols_q], dQ[:, cols_q])
    assert_close(host(q["dW"])[:, cols_q], rq["dW"], dt, "dWqkv_r cols")
    assert_close(q["db"], dQ.sum(axis=0), dt, "dbqkv_r")

    # attention output projection: rows of O_r and dctx_r, columns of dWo_r, all of dbo
    cols_h = sample(H, 48, 4 + rank)
    C, Wo, dO = sh.f64("ctx"), sh.f64("Wo"), sh.f64("dO")
    O = run_out_fwd(sh, sh.d_("ctx"))
    ro = oracle.tp_attn_out_shard_fwd(t, rank, 1, len(rows), H, nh, C[rows], Wo, sh.f64("bo"))
    assert_close(host(O)[rows], ro, dt, "O_r rows")
    ob = run_out_bwd(sh, sh.d_("ctx"), sh.d_("dO"))
    rd = oracle.attn_out_bwd(C[rows], Wo, dO[rows], False)
    assert_close(host(ob["dctx"])[rows], rd["dctx"], dt, "dctx_r rows")
    rb = oracle.attn_out_bwd(C, Wo[:, cols_h], dO[:, cols_h], rank == 0)
    assert_close(host(ob["dW"])[:, cols_h], rb["dW"], dt, "dWo_r cols")
    if rank == 0:
        assert_close(host(ob["db"])[cols_h], rb["db"], dt, "dbo cols")

    QKV = sh.d_("QKV")
    ctx, lse = run_attn_fwd(sh, QKV)
    dqkv = run_attn_bwd(sh, QKV, ctx, lse, sh.d_("dctx"))
    d = sh.d
    Qh, dctx = sh.f64("QKV"), sh.f64("dctx")
    ctx_h, lse_h, dqkv_h = host(ctx), host(lse), host(dqkv)
    for h in sorted({0, sh.nh - 1}):
        for b in sorted({0, B - 1}):
            tok = slice(b * S, (b + 1) * S)
            qh = Qh[tok, 3 * d * h: 3 * d * (h + 1)]
            rctx, rlse = oracle.attention_fwd(qh, 1, S, 1, d)
            assert_close(ctx_h[tok, d * h: d * (h + 1)], rctx, dt, f"ctx head {h} batch {b}")
            assert_close(lse_h[b, h], rlse[0, 0], dt, f"lse head {h} batch {b}", tol=2e-3)
            rd = oracle.attention_bwd(qh, dctx[tok, d * h: d * (h + 1)], 1, S, 1, d)
            assert_close(dqkv_h[tok, 3 * d * h: 3 * d * (h + 1)], rd, dt, f"dQKV head {h} batch {b}")


@pytest.mark.parametrize("rank", [0, 1])
def test_gpt2_1p5b_tp2(rank):
    check_shard(GPT2_1P5B, rank)


def test_gpt3_175b_tp8_rank0():
    check_shard(GPT3_175B, 0)


def all_ranks_identities(wl):
    """Every rank of a layer in sequence on the one GPU, then the collectives replaced by their
    definitions: the column-split outputs (QKV_r, ctx_r, LSE_r) concatenated over ranks equal the
    unsharded layer's, and the row-split and input-gradient partials (Z_r, the MLP's dX_r, the QKV
    projection's dX_r) summed in fp32 over ranks equal the unsharded ones — the column identity
    X·[W1 W2] = [X·W1, X·W2] and the row-split exit whose partials the all-reduce adds
    ("Megatron-LM技术演进与大规模模型训练实践", §2.1; "Megatron-LM — 架构与原理", §4).  The unsharded
    results come from the oracle on sampled rows (and whole sampled heads for the attention)."""
    dt = "bf16"
    t, B, S, H, nh_all, F, T, d = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F, wl.T, wl.head_dim
    rows = sample(T, 32, 9)
    f32 = dict(dtype=torch.float32, device="cuda")
    Zsum, dXm, dXq = torch.zeros(T, H, **f32), torch.zeros(T, H, **f32), torch.zeros(T, H, **f32)
    QKVcat = torch.full((T, 3 * H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ctxcat = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    lsecat = torch.full((B, nh_all, S), float("nan"), **f32)
    for r in range(t):
        print(f"{wl.name}: rank {r} of {t}", flush=True)
        sh = Shard(wl, r, dt, qkv_std=1.0)
        c0, c1 = 3 * d * sh.h0, 3 * d * (sh.h0 + sh.nh)
        QKVcat[:, c0:c1] = run_qkv_fwd(sh)
        ctx, lse = run_attn_fwd(sh, sh.d_("QKV"))
        ctxcat[:, d * sh.h0:d * (sh.h0 + sh.nh)] = ctx
        lsecat[:, sh.h0:sh.h0 + sh.nh] = lse
        Z, _, _ = run_mlp_fwd(sh)
        Zsum += Z.float()
        dXm += run_mlp_bwd(sh, sh.d_("A1"), sh.d_("Y"))["dX"].float()
        dXq += run_qkv_bwd(sh, sh.d_("dQKV"))["dX"].float()
        torch.cuda.synchronize()
        del sh
    X = synth.X(wl, dt).f64[rows]
    Wq = synth.qkv_weight(wl, 0, 3 * H, dt).f64
    bq = synth.qkv_bias(wl, 0, 3 * H, dt).f64
    assert_close(host(QKVcat)[rows], oracle.qkv_fwd(X, Wq, bq), dt, "concat_r QKV_r rows vs unsharded")
    dQ = synth.column_blocks("dQKV", T, 0, 3 * H, 1.0, dt).f64[rows]
    assert_close(host(dXq)[rows], oracle.qkv_bwd(X, Wq, dQ)["dX"], dt, "sum_r qkv dX_r rows vs unsharded")
    W1 = synth.fc1_weight(wl, 0, F, dt).f64
    b1 = synth.fc1_bias(wl, 0, F, dt).f64
    W2 = synth.fc2_weight(wl, 0, F, dt).f64
    b2 = synth.fc2_bias(wl, dt).f64
    assert_close(host(Zsum)[rows], oracle.mlp_fwd(X, W1, b1, W2, b2)["Z"], dt, "sum_r Z_r rows vs unsharded")
    A1 = synth.column_blocks("A1", T, 0, F, 1.0, dt).f64[rows]
    Y = synth.column_blocks("Y", T, 0, F, 1.0, dt).f64[rows]
    dZ = synth.upstream(wl, H, dt, "dZ").f64[rows]
    fb = oracle.mlp_bwd(X, W1, W2, A1, Y, dZ, True)
    assert_close(host(dXm)[rows], fb["dX"], dt, "sum_r mlp dX_r rows vs unsharded")
    # whole heads of the concatenated attention output: the first and last head of every rank
    ctx_h, lse_h = host(ctxcat), host(lsecat)
    heads = sorted({h for r in range(t) for h in (oracle.shard_range(nh_all, t, r)[0],
                                                 sum(oracle.shard_range(nh_all, t, r)) - 1)})
    for h in heads:
        qh_all = synth.column_blocks("QKVin", T, 3 * d * h, 3 * d * (h + 1), 1.0, dt).f64
        for b in sorted({0, B - 1}):
            tok = slice(b * S, (b + 1) * S)
            rctx, rlse = oracle.attention_fwd(qh_all[tok], 1, S, 1, d)
            assert_close(ctx_h[tok, d * h:d * (h + 1)], rctx, dt, f"concat ctx head {h} batch {b}")
            assert_close(lse_h[b, h], rlse[0, 0], dt, f"concat lse head {h} batch {b}", tol=2e-3)


def test_gpt2_1p5b_tp2_all_ranks_identities():
    """GPT-2 1.5B at tp = 2: the uneven 13 / 12-head split (and 3200 MLP columns each)."""
    all_ranks_identities(GPT2_1P5B)


def test_gpt_8p3b_tp8_all_ranks_identities():
    """The 8.3B layer at tp = 8: all eight ranks (4 heads of 96 and 1536 MLP columns each)."""
    all_ranks_identities(GPT_8P3B)


@pytest.mark.parametrize("rank", [3, 7])
def test_gpt_8p3b_tp8_rank(rank):
    check_shard(GPT_8P3B, rank)


def test_moe_expert_shard_tp8_rank0():
    """The 128-expert MoE FFN shard (hidden 8192, expert ffn 2048 -> 256 columns on rank 0 of 8,
    16384 tokens routed top-8 -> 131072 rows) at full size; sampled experts and rows checked."""
    from tensor_transformer_layer_mlp_amd.configs import MOE_E128 as mw
    dt, tp, rank = "bf16", mw.tp_size, 0
    f0, Fr = oracle.shard_range(mw.F_expert, tp, rank)
    off, tok = synth.moe_assignments(mw.tokens, mw.n_experts, mw.top_k)
    rows, H, G = int(off[-1]), mw.H, mw.n_experts
    print(f"moe: rows {rows} experts {G} H {H} Fr {Fr}", flush=True)
    Xop = synth.normal("moeX", (mw.tokens, H), 1.0, dt)
    X = dev(Xop)
    Xperm = X.index_select(0, torch.from_numpy(tok).to("cuda")).contiguous()
    keep = {0, G // 2, G - 1}
    W1 = torch.empty(G, H, Fr, dtype=torch.bfloat16, device="cuda")
    b1 = torch.empty(G, Fr, dtype=torch.bfloat16, device="cuda")
    W2 = torch.empty(G, Fr, H, dtype=torch.bfloat16, device="cuda")
    host_w = {}
    for e in range(G):
        w1 = synth.column_blocks(f"W1_e{e}", H, f0, f0 + Fr, mw.w_std, dt)
        bb = synth.vector_blocks(f"b1_e{e}", f0, f0 + Fr, mw.w_std, dt)
        w2 = synth.row_blocks(f"W2_e{e}", H, f0, f0 + Fr, mw.w_std, dt)
        W1[e], b1[e], W2[e] = dev(w1), dev(bb), dev(w2)
        if e in keep:
            host_w[e] = (w1.f64, bb.f64, w2.f64)
    print("moe: inputs ready", flush=True)
    Z = torch.empty(rows, H, dtype=torch.bfloat16, device="cuda")
    Y = torch.empty(rows, Fr, dtype=torch.bfloat16, device="cuda")
    ws = bd.workspace("tp_mlp_grouped_shard_fwd", tp, rank, 1, rows, H, G, mw.F_expert, torch.bfloat16)
    bd.tp_mlp_grouped_shard_fwd(tp, rank, G, torch.from_numpy(off).to("cuda"), rows, H, mw.F_expert,
                                Xperm, W1, b1, W2, Z, None, Y, ws)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    for e in sorted(keep):
        lo, hi = int(off[e]), int(off[e + 1])
        pick = np.unique(np.concatenate([[lo, hi - 1], g.integers(lo, hi, 8)]))
        xs = Xop.f64[tok[pick]]
        w1, bb, w2 = host_w[e]
        r = oracle.mlp_fwd(xs, w1, bb, w2, None)
        assert_close(host(Z[torch.from_numpy(pick).to("cuda")]), r["Z"], dt, f"Z rows of expert {e}")
        assert_close(host(Y[torch.from_numpy(pick).to("cuda")]), r["Y"], dt, f"Y rows of expert {e}")
