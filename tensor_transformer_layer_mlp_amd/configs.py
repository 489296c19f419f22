"""Workload presets: the shard shapes and value distributions of the five GPT-shaped layers.

Pure data.  Nothing here computes any part of the layer; the sizes are those of the GPT-shaped
workloads the shard is exercised on (a tiny layer, GPT-2 1.5B at tp=2, an 8.3B GPT at tp=8,
GPT-3 175B at tp=8, and a 128-expert MoE FFN at tp=8).
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class LayerWorkload:
    name: str
    B: int            # batch
    S: int            # sequence length
    H: int            # hidden size
    n_heads: int      # attention heads of the unsharded layer
    F: int            # MLP inner size of the unsharded layer
    tp_size: int
    ranks: tuple      # ranks the tests run (all of them unless stated)
    w_std: float      # weights and biases ~ N(0, w_std)
    x_std: float = 1.0

    @property
    def T(self) -> int:
        return self.B * self.S

    @property
    def head_dim(self) -> int:
        return self.H // self.n_heads


@dataclass(frozen=True)
class MoEWorkload:
    name: str
    H: int
    n_experts: int
    F_expert: int
    tp_size: int
    tokens: int
    top_k: int
    w_std: float
    ranks: tuple = field(default=(0,))


TINY = LayerWorkload("tiny_b2_s32_h64_nh4_f256_tp2", B=2, S=32, H=64, n_heads=4, F=256,
                     tp_size=2, ranks=(0, 1), w_std=0.02)
GPT2_1P5B = LayerWorkload("gpt2_1.5b_b8_s1024_h1600_nh25_f6400_tp2", B=8, S=1024, H=1600,
                          n_heads=25, F=6400, tp_size=2, ranks=(0, 1), w_std=0.02)
GPT_8P3B = LayerWorkload("gpt_8.3b_b8_s1024_h3072_nh32_f12288_tp8", B=8, S=1024, H=3072,
                         n_heads=32, F=12288, tp_size=8, ranks=tuple(range(8)), w_std=0.02)
GPT3_175B = LayerWorkload("gpt3_175b_b1_s2048_h12288_nh96_f49152_tp8", B=1, S=2048, H=12288,
                          n_heads=96, F=49152, tp_size=8, ranks=(0,), w_std=0.006)
MOE_E128 = MoEWorkload("moe_h8192_e128_fe2048_tp8_tok16384_top8", H=8192, n_experts=128,
                       F_expert=2048, tp_size=8, tokens=16384, top_k=8, w_std=0.02)

LAYER_WORKLOADS = {w.name: w for w in (TINY, GPT2_1P5B, GPT_8P3B, GPT3_175B)}
