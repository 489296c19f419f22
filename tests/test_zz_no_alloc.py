"""tp_qkv_shard_bwd_noalloc, the QKV shard backward on the library's own scratch array, against
tp_qkv_shard_bwd (the same call with a caller workspace) through the C ABI: two calls in a row, the
second on a smaller shard, each bitwise equal to the workspace call's results (the same kernels in
the same order) and within the bf16 / fp32 bar of the oracle."""

import pytest
import torch

import oracle
from gpu_harness import Shard, TORCH_DT, assert_close, empty
from tensor_transformer_layer_mlp_amd import binding as bd
from tensor_transformer_layer_mlp_amd.configs import LayerWorkload

pytestmark = pytest.mark.gpu

BIG = LayerWorkload("noalloc_b2_s320_h512_nh8_f1024_tp2", 2, 320, 512, 8, 1024, 2, (1,), 0.03)
SMALL = LayerWorkload("noalloc_b2_s100_h384_nh4_f512_tp2", 2, 100, 384, 4, 512, 2, (0,), 0.05)


def _outputs(sh):
    wl = sh.wl
    return dict(dX=empty((wl.T, wl.H), sh.dtype), dW=empty((wl.H, sh.Nq), sh.dtype), db=empty((sh.Nq,), sh.dtype))


def _run_pair(wl, dt):
    r = wl.ranks[0]
    sh = Shard(wl, r, dt)
    print(f"noalloc: {wl.name} rank {r} {dt}", flush=True)
    args = (wl.tp_size, r, wl.B, wl.S, wl.H, wl.n_heads, sh.d_("X"), sh.d_("Wqkv"), sh.d_("dQKV"))
    ref = _outputs(sh)
    ws = bd.workspace("tp_qkv_shard_bwd", wl.tp_size, r, wl.B, wl.S, wl.H, wl.n_heads, wl.F, TORCH_DT[dt])
    bd.tp_qkv_shard_bwd(*args, ref["dX"], ref["dW"], ref["db"], ws)
    got = _outputs(sh)
    bd.tp_qkv_shard_bwd_noalloc(*args, got["dX"], got["dW"], got["db"])
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), f"{wl.name} {dt}: {k} differs from tp_qkv_shard_bwd's"
    o = oracle.tp_qkv_shard_bwd(wl.tp_size, r, wl.B, wl.S, wl.H, wl.n_heads, sh.f64("X"), sh.f64("Wqkv"),
                                sh.f64("dQKV"))
    assert_close(got["dX"], o["dX"], dt, "dX_r")
    assert_close(got["dW"], o["dW"], dt, "dWqkv_r")
    assert_close(got["db"], o["db"], dt, "dbqkv_r")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_workspace_call_twice(dt):
    _run_pair(BIG, dt)
    _run_pair(SMALL, dt)


def test_noalloc_rejects_oversize_before_launch():
    """A shard whose column-sum partials exceed the scratch is refused before anything is enqueued."""
    cap = bd.tp_qkv_shard_bwd_noalloc_max_scratch()
    assert cap == 16 << 20
    lib, P = bd.raw(), 0x100000
    # T = 65536 tokens, 12 heads of 128 -> 1024 chunks x 4608 columns x 4 bytes = 18 MiB > 16 MiB
    rc = lib.tp_qkv_shard_bwd_noalloc(8, 0, 1, 65536, 12288, 96, 0, P, P, P, P, P, P, None)
    assert rc == -5 and "scratch" in lib.tp_last_error().decode()
