"""Helpers for the GPU tests: seeded operands to device tensors, shard inputs, error metrics.

Nothing here computes any part of the layer.  Expected values come from the oracle, fed the same
seeded synthetic operands the device receives (never anything the device produced).
"""

import numpy as np
import torch

import oracle
from tensor_transformer_layer_mlp_amd import synth

TOL = {"bf16": 2e-2, "f32": 1e-5}
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def dev(op: synth.Operand) -> torch.Tensor:
    """Device copy of an operand, bit-exact."""
    if op.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(op.dev).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(op.dev))
    return t.to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def empty(shape, dtype, fill=float("nan")):
    """Output buffer pre-filled with NaN so an element the kernel never writes is caught."""
    t = torch.empty(shape, dtype=TORCH_DT[dtype] if isinstance(dtype, str) else dtype, device="cuda")
    t.fill_(fill)
    return t


def err(got, ref):
    g = host(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    return oracle.normwise_error(g, ref)


def assert_close(got, ref, dtype, what, tol=None):
    """Parity of a device result with the oracle's: every element finite, the normwise relative error
    within the bar, and the same bar on every 64 x 64 tile of the result viewed as a matrix (each
    tile against its own norm or its share of the whole, whichever is larger), so that a defect
    confined to a few tiles is not diluted by the rest of the tensor."""
    tol = TOL[dtype] if tol is None else tol
    g = host(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    assert g.shape == np.shape(ref), f"{what}: shape {g.shape} vs {np.shape(ref)}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output (unwritten or overflow)"
    e = oracle.normwise_error(g, ref)
    assert e <= tol, f"{what}: normwise error {e:.3e} > {tol:.0e}"
    b = oracle.blockwise_error(g, ref)
    assert b <= tol, f"{what}: 64x64 tile error {b:.3e} > {tol:.0e} (normwise {e:.3e})"
    return e


class Shard:
    """Seeded operands of one rank's shard of a layer workload, on host (fp64) and device."""

    def __init__(self, wl, rank, dtype, qkv_std=None):
        self.wl, self.rank, self.dtype = wl, rank, dtype
        t = wl.tp_size
        self.h0, self.nh = oracle.shard_range(wl.n_heads, t, rank)
        self.f0, self.Fr = oracle.shard_range(wl.F, t, rank)
        d = self.d = wl.head_dim
        c0, c1 = 3 * d * self.h0, 3 * d * (self.h0 + self.nh)
        self.Nq = c1 - c0
        self.ops = {
            "X": synth.X(wl, dtype),
            "Wqkv": synth.qkv_weight(wl, c0, c1, dtype),
            "bqkv": synth.qkv_bias(wl, c0, c1, dtype),
            "W1": synth.fc1_weight(wl, self.f0, self.f0 + self.Fr, dtype),
            "b1": synth.fc1_bias(wl, self.f0, self.f0 + self.Fr, dtype),
            "W2": synth.fc2_weight(wl, self.f0, self.f0 + self.Fr, dtype),
            "b2": synth.fc2_bias(wl, dtype),
            "dZ": synth.upstream(wl, wl.H, dtype, "dZ"),
            "dctx": synth.column_blocks("dctx", wl.T, self.h0 * d, (self.h0 + self.nh) * d, 1.0, dtype),
            "dQKV": synth.column_blocks("dQKV", wl.T, c0, c1, 1.0, dtype),
            "A1": synth.column_blocks("A1", wl.T, self.f0, self.f0 + self.Fr, 1.0, dtype),
            "Y": synth.column_blocks("Y", wl.T, self.f0, self.f0 + self.Fr, 1.0, dtype),
            "Wo": synth.attn_out_weight(wl, self.h0 * d, (self.h0 + self.nh) * d, dtype),
            "bo": synth.attn_out_bias(wl, dtype),
            "dO": synth.upstream(wl, wl.H, dtype, "dO"),
            "ctx": synth.column_blocks("ctxin", wl.T, self.h0 * d, (self.h0 + self.nh) * d, 1.0, dtype),
        }
        if qkv_std is not None:   # a free-standing QKV input for the attention stage tests
            self.ops["QKV"] = synth.column_blocks("QKVin", wl.T, c0, c1, qkv_std, dtype)
        self._dev = {}

    def f64(self, name):
        return self.ops[name].f64

    def d_(self, name):
        if name not in self._dev:
            self._dev[name] = dev(self.ops[name])
        return self._dev[name]
