"""The seeded input generators: rounding and block-slicing invariants (CPU only)."""

import numpy as np
import torch

from tensor_transformer_layer_mlp_amd import synth
from tensor_transformer_layer_mlp_amd.configs import TINY, GPT2_1P5B


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000) * s for s in (1e-3, 0.02, 1.0, 300.0)])
    x = np.concatenate([x, [0.0, -0.0, 1.0, -1.0, 1.00390625, 1.005859375]])  # exact ties
    bits = synth.to_bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bits, ref.view(np.uint16))
    back = synth.bf16_bits_to_f64(bits)
    ref_back = torch.from_numpy(ref).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, ref_back)


def test_shards_are_slices_of_one_full_tensor():
    wl = TINY
    full = synth.fc1_weight(wl, 0, wl.F, "bf16")
    for lo, hi in ((0, 128), (128, 256), (37, 201), (0, 1)):
        part = synth.fc1_weight(wl, lo, hi, "bf16")
        assert np.array_equal(part.dev, full.dev[:, lo:hi])
        w2 = synth.fc2_weight(wl, lo, hi, "f32")
        assert np.array_equal(w2.dev, synth.fc2_weight(wl, 0, wl.F, "f32").dev[lo:hi])
        b = synth.fc1_bias(wl, lo, hi, "f32")
        assert np.array_equal(b.dev, synth.fc1_bias(wl, 0, wl.F, "f32").dev[lo:hi])


def test_operand_dtypes_and_distribution():
    wl = GPT2_1P5B
    x = synth.normal("probe", (4096, 64), 0.02, "bf16")
    assert x.dev.dtype == np.uint16 and x.f64.dtype == np.float64
    assert abs(x.f64.std() - 0.02) < 0.001
    y = synth.qkv_weight(wl, 0, 192, "f32")
    assert y.dev.dtype == np.float32 and y.shape == (wl.H, 192)
    assert np.array_equal(y.dev.astype(np.float64), y.f64)


def test_moe_assignments_structure():
    off, tok = synth.moe_assignments(512, 16, 4)
    assert off[0] == 0 and off[-1] == 512 * 4 and np.all(np.diff(off) >= 0)
    for e in range(16):
        rows = tok[off[e]:off[e + 1]]
        assert np.all(np.diff(rows) > 0), "tokens of one expert are sorted and distinct"
    counts = np.bincount(tok, minlength=512)
    assert np.all(counts == 4), "every token goes to top_k experts"
