"""GPU parity of the FP8 (OCP E4M3 and E5M2) path against the oracle: the per-tensor quantiser's
codes bit for bit (the code is a decision made in fp32 on both sides) and its descale exactly, plain
and transposed, in both formats; the GEMM on codes against the oracle's product of the decoded codes,
with bias, GeLU and GeLU' epilogues and mixed operand formats, over ragged and full-size shapes; and
the FP8 MLP forward and backward composed from those calls.  Expected values come from the oracle only.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import assert_close, dev, host
from tensor_transformer_layer_mlp_amd import binding as bd, synth

pytestmark = pytest.mark.gpu


def _ws():
    return bd.workspace("tp_fp8_quantize", 1, 0, 1, 1, 1, 1, 1, torch.bfloat16)


FMT = {"e4m3": bd.TP_FP8_E4M3, "e5m2": bd.TP_FP8_E5M2}


def _quantize(x, transpose=False, fmt="e4m3"):
    rows, cols = x.shape
    q = torch.full((cols, rows) if transpose else (rows, cols), 0xAA, dtype=torch.uint8, device="cuda")
    d = torch.full((1,), float("nan"), device="cuda")
    if transpose:
        bd.tp_fp8_quantize(x, None, d, _ws(), q_t=q, fmt=FMT[fmt])
    else:
        bd.tp_fp8_quantize(x, q, d, _ws(), fmt=FMT[fmt])
    torch.cuda.synchronize()
    return q, d


# (64, 64), (80, 144) and (1024, 512) take the one-pass kernel (rows and cols multiples of 16), the
# others the separate plain and transposed kernels
QCASES = [(1, 1, 1.0), (7, 13, 1.0), (64, 64, 30.0), (130, 70, 1e-3), (257, 1000, 5.0), (3, 8, 0.0),
          (80, 144, 2.0), (1024, 512, 1.0)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("transpose", [False, True], ids=["plain", "transposed"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,std", QCASES, ids=[f"{r}x{c}_s{s}" for r, c, s in QCASES])
def test_fp8_quantize(rows, cols, std, dtype, transpose, fmt):
    op = synth.normal(f"f8q_{rows}_{cols}", (rows, cols), std, dtype)
    q, d = _quantize(dev(op), transpose, fmt)
    rq, rd = oracle.fp8_quantize(op.f64.astype(np.float32), transpose, fmt)
    assert np.array_equal(host(q).astype(np.uint8), rq), "codes differ from the oracle's"
    assert np.float32(host(d)[0]) == rd, f"descale {host(d)[0]} != {rd}"


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(80, 144), (1024, 512), (130, 70), (16, 32)])
def test_fp8_quantize_both_layouts(rows, cols, dtype, fmt):
    """One call writing the plain and the transposed codes: each bit for bit as the oracle's."""
    op = synth.normal(f"f8q2_{rows}_{cols}", (rows, cols), 3.0, dtype)
    q = torch.full((rows, cols), 0xAA, dtype=torch.uint8, device="cuda")
    qt = torch.full((cols, rows), 0xAA, dtype=torch.uint8, device="cuda")
    d = torch.full((1,), float("nan"), device="cuda")
    bd.tp_fp8_quantize(dev(op), q, d, _ws(), q_t=qt, fmt=FMT[fmt])
    torch.cuda.synchronize()
    rq, rd = oracle.fp8_quantize(op.f64.astype(np.float32), False, fmt)
    assert np.array_equal(host(q).astype(np.uint8), rq), "plain codes differ from the oracle's"
    assert np.array_equal(host(qt).astype(np.uint8), np.ascontiguousarray(rq.T)), "transposed codes differ"
    assert np.float32(host(d)[0]) == rd


@pytest.mark.parametrize("fmt,vmax", [("e4m3", 448.0), ("e5m2", 57344.0)])
def test_fp8_quantize_edge_values(fmt, vmax):
    """Values at code midpoints (ties), at the subnormal boundary, and the amax element at ±vmax."""
    pos = oracle.fp8_decode(np.arange(0x80), fmt)
    pos = pos[np.isfinite(pos)]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([mids, -mids, pos.astype(np.float32), [vmax, -vmax, 0.0]]).astype(np.float32)
    x = np.pad(x, (0, (-len(x)) % 8)).reshape(-1, 8)          # amax = vmax -> s = 1: x itself is encoded
    xd = torch.from_numpy(x).cuda()
    q, d = _quantize(xd, fmt=fmt)
    rq, rd = oracle.fp8_quantize(x, fmt=fmt)
    assert rd == 1.0 and host(d)[0] == 1.0
    assert np.array_equal(host(q).astype(np.uint8), rq)


def _codes(shape, tag, std=1.0, fmt="e4m3"):
    x = synth.normal(tag, shape, std, "f32").f64.astype(np.float32)
    q, d = oracle.fp8_quantize(x, fmt=fmt)
    return q, d


E = oracle
# small shapes take the 256 x 128 tile; (2048, 6144) and the ragged (2000, 9000) the 256 x 192 one;
# (2048, 16384) the 256 x 256 one.  E5M2 operands are the backward's gradients.
GCASES = [(256, 256, 128, E.FP8_EPI_NONE, "e4m3", "e4m3"), (300, 200, 176, E.FP8_EPI_GELU, "e4m3", "e4m3"),
          (17, 8, 16, E.FP8_EPI_NONE, "e4m3", "e4m3"), (2048, 6144, 1024, E.FP8_EPI_GELU, "e4m3", "e4m3"),
          (513, 1032, 2064, E.FP8_EPI_NONE, "e4m3", "e4m3"), (2000, 9000, 64, E.FP8_EPI_GELU, "e4m3", "e4m3"),
          (2048, 16384, 256, E.FP8_EPI_NONE, "e4m3", "e4m3"),
          (300, 200, 176, E.FP8_EPI_NONE, "e5m2", "e4m3"), (513, 1032, 2064, E.FP8_EPI_NONE, "e4m3", "e5m2"),
          (130, 264, 2048, E.FP8_EPI_NONE, "e4m3", "e5m2"), (2000, 9000, 64, E.FP8_EPI_DGELU, "e5m2", "e4m3"),
          (256, 256, 128, E.FP8_EPI_DGELU_TANH, "e5m2", "e4m3"), (2048, 6144, 1024, E.FP8_EPI_DGELU, "e5m2", "e4m3"),
          (77, 40, 32, E.FP8_EPI_GELU_TANH, "e4m3", "e5m2")]


@pytest.mark.parametrize("M,N,K,epi,fa,fb", GCASES, ids=[f"m{m}_n{n}_k{k}_epi{e}_{a}x{b}" for m, n, k, e, a, b in GCASES])
def test_fp8_gemm(M, N, K, epi, fa, fb):
    print(f"fp8 gemm M={M} N={N} K={K} epilogue={epi} {fa} x {fb}", flush=True)
    A, da = _codes((M, K), f"f8A_{M}_{K}", 1.0 if fa == "e4m3" else 1e-3, fa)
    B, db = _codes((N, K), f"f8B_{N}_{K}", 0.05 if fb == "e4m3" else 1e-3, fb)
    bias = synth.normal(f"f8bias_{N}", (N,), 0.1, "bf16") if epi < E.FP8_EPI_DGELU else None
    aux = synth.normal(f"f8aux_{M}_{N}", (M, N), 1.0, "bf16") if epi >= E.FP8_EPI_DGELU else None
    gelu = epi in (E.FP8_EPI_GELU, E.FP8_EPI_GELU_TANH)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    Cp = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda") if gelu else None
    tA, tB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    tda, tdb = torch.tensor([da], device="cuda"), torch.tensor([db], device="cuda")
    bd.tp_fp8_gemm_nt(tA, tda, tB, tdb, C, bias=dev(bias) if bias is not None else None, epilogue=epi,
                      aux=dev(aux) if aux is not None else None, C_pre=Cp, a_fmt=FMT[fa], b_fmt=FMT[fb])
    torch.cuda.synchronize()
    ref = oracle.fp8_gemm_nt(A, da, B, db, bias.f64 if bias is not None else None, epi=epi,
                             aux=aux.f64 if aux is not None else None, fmt_a=fa, fmt_b=fb)
    assert_close(C, ref["C"], "bf16", "C")
    if gelu:
        assert_close(Cp, ref["pre"], "bf16", "C_pre")


def test_fp8_mlp_forward_against_bf16_definition():
    """The FP8 path end to end on a GPT-shaped MLP shard forward: quantise X and the transposed
    weights, fc1 with bias + GeLU, quantise Y, fc2.  Checked two ways: against the same recipe run by
    the oracle (X and the weights quantised by the oracle, Y quantised from the GPU's own bf16 Y — the
    value the GPU quantised — so every code is the same on both sides and each GEMM is held to the
    bf16 bar), and against the oracle's exact-precision MLP, within the error FP8 rounding of four
    operands allows (a looser bar: 8e-2 normwise)."""
    T, H, Fr = 512, 1024, 768
    X = synth.normal("f8mlpX", (T, H), 1.0, "bf16")
    W1 = synth.normal("f8mlpW1", (H, Fr), 0.02, "bf16")
    b1 = synth.normal("f8mlpb1", (Fr,), 0.02, "bf16")
    W2 = synth.normal("f8mlpW2", (Fr, H), 0.02, "bf16")
    u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")  # noqa: E731
    f1 = lambda: torch.empty(1, device="cuda")  # noqa: E731
    qX, qW1t, qW2t, qY = u8(T, H), u8(Fr, H), u8(H, Fr), u8(T, Fr)
    dX, dW1, dW2, dY = f1(), f1(), f1(), f1()
    ws = _ws()
    bd.tp_fp8_quantize(dev(X), qX, dX, ws)
    bd.tp_fp8_quantize(dev(W1), None, dW1, ws, q_t=qW1t)
    bd.tp_fp8_quantize(dev(W2), None, dW2, ws, q_t=qW2t)
    Y = torch.empty(T, Fr, dtype=torch.bfloat16, device="cuda")
    bd.tp_fp8_gemm_nt(qX, dX, qW1t, dW1, Y, bias=dev(b1), epilogue=bd.TP_FP8_EPI_GELU)
    bd.tp_fp8_quantize(Y, qY, dY, ws)
    Z = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    bd.tp_fp8_gemm_nt(qY, dY, qW2t, dW2, Z)
    torch.cuda.synchronize()
    f32 = lambda a: a.f64.astype(np.float32)  # noqa: E731
    oq, g = oracle.fp8_quantize, oracle.fp8_gemm_nt
    cX, oX = oq(f32(X))
    cW1t, oW1 = oq(f32(W1), True)
    cW2t, oW2 = oq(f32(W2), True)
    for name, got, codes, gs, os_ in (("X", qX, cX, dX, oX), ("W1ᵀ", qW1t, cW1t, dW1, oW1), ("W2ᵀ", qW2t, cW2t, dW2, oW2)):
        assert np.array_equal(got.cpu().numpy(), codes), f"codes of {name} differ from the oracle's"
        assert np.float32(gs.item()) == np.float32(os_), f"descale of {name}"
    emu_Y = g(cX, oX, cW1t, oW1, b1.f64, epi=oracle.FP8_EPI_GELU)["C"]
    assert_close(Y, emu_Y, "bf16", "Y (the FP8 recipe on the oracle)")
    cY, oY = oq(host(Y).astype(np.float32))
    assert np.array_equal(qY.cpu().numpy(), cY), "codes of Y differ from the oracle's"
    assert_close(Z, g(cY, oY, cW2t, oW2)["C"], "bf16", "Z (the FP8 recipe on the oracle)")
    ref = oracle.mlp_fwd(X.f64, W1.f64, b1.f64, W2.f64, None)
    assert_close(Y, ref["Y"], "bf16", "Y (fp8 fc1)", tol=8e-2)
    assert_close(Z, ref["Z"], "bf16", "Z (fp8 fc2)", tol=8e-2)


def test_fp8_mlp_backward():
    """The FP8 MLP-shard backward composed from the entry points, the usual FP8 training recipe:
    gradients in E5M2, weights and activations in E4M3, each GEMM with K-major code operands —
    dA1 = (dZ·W2ᵀ) ∘ GeLU'(A1) (the GeLU' epilogue), dW2 = Yᵀ·dZ, dX = dA1·W1ᵀ, dW1 = Xᵀ·dA1 — and
    db1 = Σ_t dA1.  Checked two ways: against the same recipe run by the oracle from the GPU's own
    bf16 intermediates (A1, Y, dA1: the values the GPU quantised, so every code is the same on both
    sides and each GEMM is held to the bf16 bar), and against the oracle's
    exact-precision backward (E5M2 keeps 2 mantissa bits: 1.5e-1 normwise, where the errors the
    recipe itself makes sit near 9e-2 for these shapes)."""
    T, H, Fr = 512, 1024, 768
    X = synth.normal("f8mlpX", (T, H), 1.0, "bf16")
    W1 = synth.normal("f8mlpW1", (H, Fr), 0.02, "bf16")
    b1 = synth.normal("f8mlpb1", (Fr,), 0.02, "bf16")
    W2 = synth.normal("f8mlpW2", (Fr, H), 0.02, "bf16")
    dZ = synth.normal("f8mlpdZ", (T, H), 1.0, "bf16")
    u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")  # noqa: E731
    f1 = lambda: torch.empty(1, device="cuda")  # noqa: E731
    bf = lambda *s: torch.full(s, float("nan"), dtype=torch.bfloat16, device="cuda")  # noqa: E731
    ws = _ws()
    e4, e5 = bd.TP_FP8_E4M3, bd.TP_FP8_E5M2
    # forward (keeps A1 for the backward)
    qX, qXt, qW1t, qW1, qW2t, qW2 = u8(T, H), u8(H, T), u8(Fr, H), u8(H, Fr), u8(H, Fr), u8(Fr, H)
    sX, sW1, sW2, sY, sdZ, sdA1 = f1(), f1(), f1(), f1(), f1(), f1()
    bd.tp_fp8_quantize(dev(X), qX, sX, ws, q_t=qXt)
    bd.tp_fp8_quantize(dev(W1), qW1, sW1, ws, q_t=qW1t)
    bd.tp_fp8_quantize(dev(W2), qW2, sW2, ws, q_t=qW2t)
    A1, Y = bf(T, Fr), bf(T, Fr)
    bd.tp_fp8_gemm_nt(qX, sX, qW1t, sW1, Y, bias=dev(b1), epilogue=bd.TP_FP8_EPI_GELU, C_pre=A1)
    qYt = u8(Fr, T)
    bd.tp_fp8_quantize(Y, None, sY, ws, q_t=qYt)
    # backward
    qdZ, qdZt, qdA1, qdA1t = u8(T, H), u8(H, T), u8(T, Fr), u8(Fr, T)
    bd.tp_fp8_quantize(dev(dZ), qdZ, sdZ, ws, q_t=qdZt, fmt=e5)
    dA1, dW2, dX, dW1 = bf(T, Fr), bf(Fr, H), bf(T, H), bf(H, Fr)
    db1 = bf(Fr)
    bd.tp_fp8_gemm_nt(qdZ, sdZ, qW2, sW2, dA1, epilogue=bd.TP_FP8_EPI_DGELU, aux=A1, a_fmt=e5, b_fmt=e4)
    bd.tp_fp8_gemm_nt(qYt, sY, qdZt, sdZ, dW2, a_fmt=e4, b_fmt=e5)
    bd.tp_fp8_quantize(dA1, qdA1, sdA1, ws, q_t=qdA1t, fmt=e5)
    bd.tp_fp8_gemm_nt(qdA1, sdA1, qW1, sW1, dX, a_fmt=e5, b_fmt=e4)
    bd.tp_fp8_gemm_nt(qXt, sX, qdA1t, sdA1, dW1, a_fmt=e4, b_fmt=e5)
    wsb = bd.workspace("tp_bias_grad", 1, 0, T, 1, Fr, 1, 1, torch.bfloat16)
    bd.tp_bias_grad(dA1, db1, wsb)
    torch.cuda.synchronize()

    # the recipe on the oracle, from the GPU's bf16 A1 / Y / dA1 (the values the GPU quantised)
    A1h, Yh, dA1h = host(A1).astype(np.float32), host(Y).astype(np.float32), host(dA1).astype(np.float32)
    f32 = lambda a: a.f64.astype(np.float32)  # noqa: E731
    oq = oracle.fp8_quantize
    cdZ, odZ = oq(f32(dZ), fmt="e5m2")
    cdZt, _ = oq(f32(dZ), True, "e5m2")
    cW2, oW2 = oq(f32(W2))
    cW1, oW1 = oq(f32(W1))
    cXt, oX = oq(f32(X), True)
    cYt, oY = oq(Yh, True)
    cA, oA = oq(dA1h, fmt="e5m2")
    cAt, _ = oq(dA1h, True, "e5m2")
    g = oracle.fp8_gemm_nt
    emu = {"dA1": g(cdZ, odZ, cW2, oW2, epi=oracle.FP8_EPI_DGELU, aux=A1h, fmt_a="e5m2")["C"],
           "dW2": g(cYt, oY, cdZt, odZ, fmt_b="e5m2")["C"],
           "dX": g(cA, oA, cW1, oW1, fmt_a="e5m2")["C"],
           "dW1": g(cXt, oX, cAt, oA, fmt_b="e5m2")["C"],
           "db1": dA1h.astype(np.float64).sum(axis=0)}
    got = {"dA1": dA1, "dW2": dW2, "dX": dX, "dW1": dW1, "db1": db1}
    for k in emu:
        assert_close(got[k], emu[k], "bf16", f"{k} (the FP8 recipe on the oracle)")
    ref = oracle.mlp_bwd(X.f64, W1.f64, W2.f64, *[oracle.mlp_fwd(X.f64, W1.f64, b1.f64, W2.f64, None)[k]
                                                 for k in ("A1", "Y")], dZ.f64, False)
    for k in ("dX", "dW1", "db1", "dW2"):
        assert_close(got[k], ref[k], "bf16", f"{k} (exact precision)", tol=1.5e-1)


def test_fp8_mlp_graph_replay():
    """The FP8 MLP forward and backward (quantisations, GEMMs, bias gradient) captured in one HIP
    graph: three replays each equal the eager result bit for bit."""
    from test_gpu_graph import _capture
    T, H, Fr = 256, 512, 384
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    bf = torch.bfloat16
    r = lambda *s, std=1.0: (torch.randn(*s, generator=g, device="cuda") * std).to(bf)  # noqa: E731
    X, W1, b1, W2, dZ = r(T, H), r(H, Fr, std=0.02), r(Fr, std=0.02), r(Fr, H, std=0.02), r(T, H)
    u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")  # noqa: E731
    e = lambda *s: torch.empty(*s, dtype=bf, device="cuda")  # noqa: E731
    qX, qXt, qW1, qW1t, qW2, qW2t, qY, qYt = u8(T, H), u8(H, T), u8(H, Fr), u8(Fr, H), u8(Fr, H), u8(H, Fr), \
        u8(T, Fr), u8(Fr, T)
    qdZ, qdZt, qdA1, qdA1t = u8(T, H), u8(H, T), u8(T, Fr), u8(Fr, T)
    sc = [torch.empty(1, device="cuda") for _ in range(6)]
    A1, Y, Z, dA1, dW2, dX, dW1, db1 = e(T, Fr), e(T, Fr), e(T, H), e(T, Fr), e(Fr, H), e(T, H), e(H, Fr), e(Fr)
    ws = _ws()
    wsb = bd.workspace("tp_bias_grad", 1, 0, T, 1, Fr, 1, 1, bf)
    e4, e5 = bd.TP_FP8_E4M3, bd.TP_FP8_E5M2

    def call():
        bd.tp_fp8_quantize(X, qX, sc[0], ws, q_t=qXt)
        bd.tp_fp8_quantize(W1, qW1, sc[1], ws, q_t=qW1t)
        bd.tp_fp8_quantize(W2, qW2, sc[2], ws, q_t=qW2t)
        bd.tp_fp8_gemm_nt(qX, sc[0], qW1t, sc[1], Y, bias=b1, epilogue=bd.TP_FP8_EPI_GELU, C_pre=A1)
        bd.tp_fp8_quantize(Y, qY, sc[3], ws, q_t=qYt)
        bd.tp_fp8_gemm_nt(qY, sc[3], qW2t, sc[2], Z)
        bd.tp_fp8_quantize(dZ, qdZ, sc[4], ws, q_t=qdZt, fmt=e5)
        bd.tp_fp8_gemm_nt(qdZ, sc[4], qW2, sc[2], dA1, epilogue=bd.TP_FP8_EPI_DGELU, aux=A1, a_fmt=e5, b_fmt=e4)
        bd.tp_fp8_gemm_nt(qYt, sc[3], qdZt, sc[4], dW2, a_fmt=e4, b_fmt=e5)
        bd.tp_fp8_quantize(dA1, qdA1, sc[5], ws, q_t=qdA1t, fmt=e5)
        bd.tp_fp8_gemm_nt(qdA1, sc[5], qW1, sc[1], dX, a_fmt=e5, b_fmt=e4)
        bd.tp_fp8_gemm_nt(qXt, sc[0], qdA1t, sc[5], dW1, a_fmt=e4, b_fmt=e5)
        bd.tp_bias_grad(dA1, db1, wsb)
    call()
    torch.cuda.synchronize()
    bufs = dict(A1=A1, Y=Y, Z=Z, dA1=dA1, dW2=dW2, dX=dX, dW1=dW1, db1=db1, qXt=qXt, qdA1t=qdA1t)
    eager = {key: v.clone() for key, v in bufs.items()}
    gr = _capture(call)
    for rep in range(3):
        for v in bufs.values():
            v.fill_(0 if v.dtype == torch.uint8 else -1)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for key in bufs:
            assert torch.equal(bufs[key], eager[key]), f"replay {rep}: {key} differs from the eager call"
        call()
        torch.cuda.synchronize()
