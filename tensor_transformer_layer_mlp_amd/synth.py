"""Seeded synthetic inputs shared by the HIP path's tests and the oracle's.

This module only draws random numbers and rounds them to the storage type.  It holds none of the
layer's arithmetic: no slicing rule, no GEMM, no activation, no softmax.  Callers pass explicit
column / row / head ranges.

Every full weight is drawn in fixed blocks, each from its own counter-seeded PCG64 stream
(seed = (1234, crc32(tensor name), block index)).  Any rank's shard is therefore the exact slice of
one fixed full tensor, whatever tp_size is, and costs only the blocks it covers.

Values are drawn in float64, rounded to float32 (round-to-nearest-even), and for bf16 once more to
bf16 (round-to-nearest-even on the top 16 bits).  `Operand.f64` is the exact value the device sees.
"""

from dataclasses import dataclass
import zlib

import numpy as np

BASE_SEED = 1234
BLOCK = 64          # width of a column block (row block for the row-split weight)


def _rng(tag: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence([BASE_SEED, zlib.crc32(tag.encode()), int(block)])
    return np.random.Generator(np.random.PCG64(ss))


def to_bf16_bits(x) -> np.ndarray:
    """float64/float32 values -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


@dataclass
class Operand:
    """One input tensor: `dev` is what the device receives, `f64` the same values exactly."""
    dev: np.ndarray     # uint16 bf16 bit patterns, or float32
    f64: np.ndarray     # float64
    dtype: str          # "bf16" or "f32"

    @property
    def shape(self):
        return self.f64.shape


def make_operand(values, dtype: str) -> Operand:
    v = np.asarray(values, dtype=np.float64)
    if dtype == "bf16":
        bits = to_bf16_bits(v)
        return Operand(bits, bf16_bits_to_f64(bits), dtype)
    if dtype == "f32":
        f = v.astype(np.float32)
        return Operand(f, f.astype(np.float64), dtype)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(tag: str, shape, std: float, dtype: str) -> Operand:
    """A whole tensor from one stream (activations, upstream gradients, small biases)."""
    v = _rng(tag, 0).standard_normal(shape) * std
    return make_operand(v, dtype)


def column_blocks(tag: str, rows: int, col_lo: int, col_hi: int, std: float, dtype: str,
                  block: int = BLOCK) -> Operand:
    """Columns [col_lo, col_hi) of a [rows, *] tensor drawn in `block`-wide column blocks."""
    parts = []
    for b in range(col_lo // block, (col_hi + block - 1) // block):
        blk = _rng(tag, b).standard_normal((rows, block)) * std
        lo = max(col_lo, b * block) - b * block
        hi = min(col_hi, (b + 1) * block) - b * block
        parts.append(blk[:, lo:hi])
    v = np.concatenate(parts, axis=1) if parts else np.zeros((rows, 0))
    return make_operand(v, dtype)


def row_blocks(tag: str, cols: int, row_lo: int, row_hi: int, std: float, dtype: str,
               block: int = BLOCK) -> Operand:
    """Rows [row_lo, row_hi) of a [*, cols] tensor drawn in `block`-high row blocks."""
    parts = []
    for b in range(row_lo // block, (row_hi + block - 1) // block):
        blk = _rng(tag, b).standard_normal((block, cols)) * std
        lo = max(row_lo, b * block) - b * block
        hi = min(row_hi, (b + 1) * block) - b * block
        parts.append(blk[lo:hi, :])
    v = np.concatenate(parts, axis=0) if parts else np.zeros((0, cols))
    return make_operand(v, dtype)


def vector_blocks(tag: str, lo: int, hi: int, std: float, dtype: str,
                  block: int = BLOCK) -> Operand:
    """Entries [lo, hi) of a bias vector drawn in `block`-long pieces."""
    parts = []
    for b in range(lo // block, (hi + block - 1) // block):
        blk = _rng(tag, b).standard_normal(block) * std
        parts.append(blk[max(lo, b * block) - b * block: min(hi, (b + 1) * block) - b * block])
    v = np.concatenate(parts) if parts else np.zeros(0)
    return make_operand(v, dtype)


# ---- the layer's tensors, by name --------------------------------------------------------------

def X(wl, dtype, tag="X") -> Operand:
    return normal(tag, (wl.T, wl.H), wl.x_std, dtype)


def upstream(wl, cols: int, dtype, tag) -> Operand:
    """An upstream gradient (dZ, dctx, dQKV) of shape [T, cols], ~ N(0, 1)."""
    return normal(tag, (wl.T, cols), 1.0, dtype)


def qkv_weight(wl, col_lo: int, col_hi: int, dtype) -> Operand:
    """Columns [col_lo, col_hi) of the full [H, 3H] QKV weight (head-interleaved columns)."""
    return column_blocks("Wqkv", wl.H, col_lo, col_hi, wl.w_std, dtype)


def qkv_bias(wl, col_lo: int, col_hi: int, dtype) -> Operand:
    return vector_blocks("bqkv", col_lo, col_hi, wl.w_std, dtype)


def fc1_weight(wl, col_lo: int, col_hi: int, dtype) -> Operand:
    return column_blocks("W1", wl.H, col_lo, col_hi, wl.w_std, dtype)


def fc1_bias(wl, col_lo: int, col_hi: int, dtype) -> Operand:
    return vector_blocks("b1", col_lo, col_hi, wl.w_std, dtype)


def fc2_weight(wl, row_lo: int, row_hi: int, dtype) -> Operand:
    return row_blocks("W2", wl.H, row_lo, row_hi, wl.w_std, dtype)


def fc2_bias(wl, dtype) -> Operand:
    return vector_blocks("b2", 0, wl.H, wl.w_std, dtype)


# ---- MoE routing (input construction only) -----------------------------------------------------

def moe_assignments(tokens: int, n_experts: int, top_k: int, seed_tag="router_logits"):
    """Token -> expert assignments, sorted by (expert, token).

    Router logits ~ N(0, 1) [tokens, n_experts] (float32).  Each token takes the top_k largest
    logits; equal logits go to the lower expert id.  Because softmax is monotone this is the same
    selection as top_k of the softmax.  No capacity limit.  Returns (group_offsets[n_experts+1],
    token_of_row[tokens*top_k]).
    """
    logits = _rng(seed_tag, 0).standard_normal((tokens, n_experts)).astype(np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    tok = np.repeat(np.arange(tokens), top_k)
    exp = order.reshape(-1)
    perm = np.lexsort((tok, exp))
    tok, exp = tok[perm], exp[perm]
    counts = np.bincount(exp, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    return offsets.astype(np.int32), tok.astype(np.int64)
