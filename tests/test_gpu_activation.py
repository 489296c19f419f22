"""The tanh form of GeLU as the MLP's activation (tp_mlp_shard_fwd_act / _bwd_act with TP_GELU_TANH,
and gelu = 2 in the FP8 GEMM) against the oracle; and the _act entry points with TP_GELU equal to
the plain ones bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import Shard, assert_close, dev, empty, host
from test_gpu_parity import RAGGED, RAGGED8, TILES, TINY, ws
from tensor_transformer_layer_mlp_amd import binding as bd, synth

pytestmark = pytest.mark.gpu

CASES = [(wl, dt, r) for wl in (TINY, RAGGED, TILES, RAGGED8) for dt in ("bf16", "f32") for r in wl.ranks[:1]]


def _run(sh, activation):
    wl = sh.wl
    Z, A1, Y = empty((wl.T, wl.H), sh.dtype), empty((wl.T, sh.Fr), sh.dtype), empty((wl.T, sh.Fr), sh.dtype)
    bd.tp_mlp_shard_fwd(wl.tp_size, sh.rank, wl.T, wl.H, wl.F, sh.d_("X"), sh.d_("W1"), sh.d_("b1"), sh.d_("W2"),
                        sh.d_("b2"), Z, A1, Y, activation=activation)
    o = dict(dX=empty((wl.T, wl.H), sh.dtype), dW1=empty((wl.H, sh.Fr), sh.dtype), db1=empty((sh.Fr,), sh.dtype),
             dW2=empty((sh.Fr, wl.H), sh.dtype), db2=empty((wl.H,), sh.dtype))
    bd.tp_mlp_shard_bwd(wl.tp_size, sh.rank, wl.T, wl.H, wl.F, sh.d_("X"), sh.d_("W1"), sh.d_("W2"), sh.d_("A1"),
                        sh.d_("Y"), sh.d_("dZ"), o["dX"], o["dW1"], o["db1"], o["dW2"], o["db2"],
                        ws("tp_mlp_shard_bwd", sh), activation=activation)
    torch.cuda.synchronize()
    return Z, A1, Y, o


@pytest.mark.parametrize("wl,dtype,rank", CASES, ids=[f"{w.name}-{d}-r{r}" for w, d, r in CASES])
def test_mlp_tanh_gelu(wl, dtype, rank):
    sh = Shard(wl, rank, dtype)
    Z, A1, Y, o = _run(sh, bd.TP_GELU_TANH)
    ref = oracle.tp_mlp_shard_fwd(wl.tp_size, rank, wl.T, wl.H, wl.F, sh.f64("X"), sh.f64("W1"), sh.f64("b1"),
                                  sh.f64("W2"), sh.f64("b2"), activation=1)
    for got, k in ((A1, "A1"), (Y, "Y"), (Z, "Z")):
        assert_close(got, ref[k], dtype, f"{k} (tanh form)")
    rb = oracle.tp_mlp_shard_bwd(wl.tp_size, rank, wl.T, wl.H, wl.F, sh.f64("X"), sh.f64("W1"), sh.f64("W2"),
                                 sh.f64("A1"), sh.f64("Y"), sh.f64("dZ"), activation=1)
    for k in ("dX", "dW1", "db1", "dW2"):
        assert_close(o[k], rb[k], dtype, f"{k} (tanh form)")
    # and it is a different function: the exact-GeLU oracle is measurably off at the fp32 bar
    if dtype == "f32":
        exact = oracle.tp_mlp_shard_fwd(wl.tp_size, rank, wl.T, wl.H, wl.F, sh.f64("X"), sh.f64("W1"),
                                        sh.f64("b1"), sh.f64("W2"), sh.f64("b2"))
        assert oracle.normwise_error(host(Y), exact["Y"]) > 1e-5


def test_act_entry_points_with_exact_gelu_match_plain_ones():
    sh = Shard(RAGGED8, 2, "bf16")
    a = _run(sh, bd.TP_GELU)
    b = _run(sh, None)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    for k in a[3]:
        if sh.rank != 0 and k == "db2":
            continue
        assert torch.equal(a[3][k], b[3][k]), k


def test_fp8_gemm_tanh_gelu():
    M, N, K = 300, 256, 512
    x = synth.normal("f8tA", (M, K), 1.0, "f32").f64.astype(np.float32)
    w = synth.normal("f8tB", (N, K), 0.05, "f32").f64.astype(np.float32)
    A, da = oracle.fp8_quantize(x)
    B, db = oracle.fp8_quantize(w)
    bias = synth.normal("f8tbias", (N,), 0.1, "bf16")
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    Cp = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    bd.tp_fp8_gemm_nt(torch.from_numpy(A).cuda(), torch.tensor([da], device="cuda"), torch.from_numpy(B).cuda(),
                      torch.tensor([db], device="cuda"), C, bias=dev(bias), epilogue=bd.TP_FP8_EPI_GELU_TANH,
                      C_pre=Cp)
    torch.cuda.synchronize()
    ref = oracle.fp8_gemm_nt(A, da, B, db, bias.f64)
    assert_close(Cp, ref["pre"], "bf16", "pre-activation")
    assert_close(C, oracle.gelu_tanh(ref["pre"]), "bf16", "tanh-form GeLU")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_gelu_elementwise(dtype):
    """The device's exact GeLU and GeLU' elementwise, through the MLP shard at tp = 1 with identity
    weights, zero bias and an all-ones dZ: A1 = X (one product per output, exact), Y = GeLU(X), and
    db1 = Σ_t (dZ·W2ᵀ)∘GeLU'(A1) = Σ_t GeLU'(X_t).  X holds 8 rows of 4096 points spanning [−9, 9]
    (bf16-representable, so both modes see the same values).  Bound: the evaluation's own error
    (2.1e-7 for GeLU and 7e-8 for GeLU' absolute) plus the output's rounding (fp32; bf16 for Y in bf16
    mode), against the oracle's erf-based values."""
    T, H = 8, 4096
    xs = np.linspace(-9.0, 9.0, T * H).reshape(T, H)
    X = synth.make_operand(xs, "bf16").f64                      # bf16-exact points
    op = synth.make_operand(X, dtype)
    eye = synth.make_operand(np.eye(H), dtype)
    zero = synth.make_operand(np.zeros(H), dtype)
    ones = synth.make_operand(np.ones((T, H)), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Xd, I, z, dZ = dev(op), dev(eye), dev(zero), dev(ones)
    Z, A1, Y = empty((T, H), dtype), empty((T, H), dtype), empty((T, H), dtype)
    bd.tp_mlp_shard_fwd(1, 0, T, H, H, Xd, I, z, I, z, Z, A1, Y)
    o = dict(dX=empty((T, H), dtype), dW1=empty((H, H), dtype), db1=empty((H,), dtype), dW2=empty((H, H), dtype),
             db2=empty((H,), dtype))
    wsb = bd.workspace("tp_mlp_shard_bwd", 1, 0, 1, T, H, 1, H, tdt)
    bd.tp_mlp_shard_bwd(1, 0, T, H, H, Xd, I, I, A1, Y, dZ, o["dX"], o["dW1"], o["db1"], o["dW2"], o["db2"], wsb)
    torch.cuda.synchronize()
    assert np.array_equal(host(A1), X), "A1 = X·I must be exact"
    g, gg = oracle.gelu(X), oracle.gelu_grad(X)
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    err = np.abs(host(Y) - g)
    assert (err <= 2.2e-7 + rel * np.abs(g)).all(), f"GeLU: worst excess {(err - rel * np.abs(g)).max():.3e}"
    # db1 sums the stored dA1 = GeLU'(X_t) (rounded to the storage type) over the 8 rows in fp32,
    # then rounds the sum to the storage type
    want = gg.sum(axis=0)
    e1 = np.abs(host(o["db1"]) - want)
    r_elem = (2.0 ** -9 if dtype == "bf16" else 0.0) + 8 * 2.0 ** -23
    tol1 = 8 * 7.5e-8 + r_elem * np.abs(gg).sum(axis=0) + rel * np.abs(want)
    assert (e1 <= tol1).all(), f"GeLU': worst excess {(e1 - tol1).max():.3e}"
