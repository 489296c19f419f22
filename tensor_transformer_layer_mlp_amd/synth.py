"""Seeded synthetic inputs shared by the HIP path's tests and the oracle's.

This module only draws random numbers and rounds them to the storage type.  It holds none of the
layer's arithmetic: no slicing rule, no GEMM, no activation, no softmax.  Callers pass explicit
column / row / head ranges.

Every full weight is drawn in fixed blocks, each from its own counter-seeded PCG64 stream
(seed = (1234, crc32(tensor name), block index)).  Any rank's shard is therefore the exact slice of
one fixed full tensor, whatever tp_size is, and costs only the blocks it covers.

Values are standard normals drawn in float32 (numpy's ziggurat), scaled by the tensor's standard
deviation in float32, and for bf16 rounded once more to bf16 (round-to-nearest-even on the top 16
bits).  `Operand.f64` is the exact value the device sees.
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
    u = np.array(x, dtype=np.float32, copy=True, order="C").view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    u += r
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32)
    b <<= np.uint32(16)
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
    """Operand from float32 (or float64) values: fp32 kept as is, bf16 rounded once (RNE)."""
    if dtype == "bf16":
        bits = to_bf16_bits(values)
        return Operand(bits, bf16_bits_to_f64(bits), dtype)
    if dtype == "f32":
        f = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
        return Operand(f, f.astype(np.float64), dtype)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal32(tag, block, shape, std):
    v = _rng(tag, block).standard_normal(shape, dtype=np.float32)
    v *= np.float32(std)
    return v


def normal(tag: str, shape, std: float, dtype: str) -> Operand:
    """A whole tensor from one stream (activations, upstream gradients, small biases)."""
    return make_operand(_normal32(tag, 0, shape, std), dtype)


def column_blocks(tag: str, rows: int, col_lo: int, col_hi: int, std: float, dtype: str,
                  block: int = BLOCK) -> Operand:
    """Columns [col_lo, col_hi) of a [rows, *] tensor drawn in `block`-wide column blocks."""
    out = np.empty((rows, max(col_hi - col_lo, 0)), dtype=np.float32)
    for b in range(col_lo // block, (col_hi + block - 1) // block):
        blk = _normal32(tag, b, (rows, block), std)
        lo, hi = max(col_lo, b * block), min(col_hi, (b + 1) * block)
        out[:, lo - col_lo:hi - col_lo] = blk[:, lo - b * block:hi - b * block]
    return make_operand(out, dtype)


def row_blocks(tag: str, cols: int, row_lo: int, row_hi: int, std: float, dtype: str,
               block: int = BLOCK) -> Operand:
    """Rows [row_lo, row_hi) of a [*, cols] tensor drawn in `block`-high row blocks."""
    out = np.empty((max(row_hi - row_lo, 0), cols), dtype=np.float32)
    for b in range(row_lo // block, (row_hi + block - 1) // block):
        blk = _normal32(tag, b, (block, cols), std)
        lo, hi = max(row_lo, b * block), min(row_hi, (b + 1) * block)
        out[lo - row_lo:hi - row_lo] = blk[lo - b * block:hi - b * block]
    return make_operand(out, dtype)


def vector_blocks(tag: str, lo: int, hi: int, std: float, dtype: str,
                  block: int = BLOCK) -> Operand:
    """Entries [lo, hi) of a bias vector drawn in `block`-long pieces."""
    out = np.empty(max(hi - lo, 0), dtype=np.float32)
    for b in range(lo // block, (hi + block - 1) // block):
        blk = _normal32(tag, b, block, std)
        a, z = max(lo, b * block), min(hi, (b + 1) * block)
        out[a - lo:z - lo] = blk[a - b * block:z - b * block]
    return make_operand(out, dtype)


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


def attn_out_weight(wl, row_lo: int, row_hi: int, dtype) -> Operand:
    """Rows [row_lo, row_hi) of the full [H, H] attention output-projection weight."""
    return row_blocks("Wo", wl.H, row_lo, row_hi, wl.w_std, dtype)


def attn_out_bias(wl, dtype) -> Operand:
    return vector_blocks("bo", 0, wl.H, wl.w_std, dtype)


def keep_mask(tag: str, shape, p_drop: float) -> np.ndarray:
    """A dropout keep mask (uint8, 1 = kept): uniform draws in [0, 1) above p_drop.  The draws are
    an input of the residual-dropout op, made here like every other random input."""
    u = _rng(tag, 0).random(shape, dtype=np.float32)
    return (u >= np.float32(p_drop)).astype(np.uint8)


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
