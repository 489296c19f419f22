#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's shard of a Megatron Transformer layer, on one MI355X.

Workload: the GPT-3 175B layer at tp_size=8, rank 0 — B=1, S=2048, H=12288, 96 heads (12 per rank,
head_dim 128), ffn 49152 (6144 columns per rank) — bf16 inputs with fp32 accumulation.  One step is
the whole hot path, forward and backward, through the C ABI of libtpshard.so:
    tp_qkv_shard_fwd -> tp_attn_heads_fwd -> tp_mlp_shard_fwd ->
    tp_mlp_shard_bwd -> tp_attn_heads_bwd -> tp_qkv_shard_bwd
Inputs are synthetic and seeded (X, dZ, dctx ~ N(0, 1); weights and biases ~ N(0, 0.006)) and
resident in HBM before the timed region.  The metric is algorithmic TFLOP/s of the step (GEMM flops
2·M·N·K; causal attention 4·d per visible (query, key) pair forward and 8·d backward) and its
fraction of the bf16 dense MFMA peak, 2516.6 TFLOP/s (256 CU x 2.4 GHz x 4096 flop/clk).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--cpu-seq S | --no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM traffic of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of `--pmc-pass`
# scaled by the same counters on a copy of known size; valid only while the kernel's sources hash the
# same as when the counters were taken.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_bf16_tn_gpt3_175b_tp8_rank0_traffic.txt")
GEMM_SOURCES = ["gemm_bf16.hip", "common.h", "kernels.h"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seq", type=int, default=2048,
                    help="tokens of the oracle's CPU sample (the first S of the sequence)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-moe", action="store_true", help="skip the MoE measurements")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--no-attn-out", action="store_true",
                    help="skip the attention output-projection measurement")
    ap.add_argument("--no-ln", action="store_true", help="skip the residual + LayerNorm measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 MLP measurement")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="for rocprofv3 --pmc runs: a 1 GiB fp32 negation (the copy the counters are "
                         "calibrated on), then --warmup + --steps steps, and nothing else")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time without the per-kernel events (the roofline object is then null)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache step timing")
    ap.add_argument("--no-other-shards", action="store_true",
                    help="skip the GPT-2 1.5B (tp=2, both ranks) and 8.3B (tp=8) shard steps")
    ap.add_argument("--pmc-ln", action="store_true",
                    help="with --pmc-pass: also one residual + LayerNorm forward and backward")
    ap.add_argument("--blas-compare", action="store_true",
                    help="also time torch.matmul on the nine GEMM shapes of the GPT-3 shard")
    ap.add_argument("--summarize", choices=["stats", "traffic", "mfma", "hbm", "lds", "blas"],
                    help="print a profile summary from rocprofv3 CSV output under --prof-dir, and exit")
    ap.add_argument("--prof-dir", default="rocprof_out",
                    help="rocprofv3 output directory (stats: one kernel-trace run; traffic / hbm: the "
                         "directory holding pmc_fetch/ and pmc_write/; mfma: pmc_clk/ and pmc_mfma/)")
    ap.add_argument("--kernel", default="gemm_bf16_kernel<Tile<256, 256, 4, 2, 2, 64, 0>, false, false, 0>",
                    help="with --summarize traffic: the kernel (as named in the trace, template arguments "
                         "included) whose per-launch traffic is summarised")
    ap.add_argument("--tag", default="gemm_bf16_kernel<256x256, tn, epi0>",
                    help="with --summarize traffic: that kernel's tag in the library's per-launch timing")
    return ap.parse_args()


def gemm_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "tensor_transformer_layer_mlp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """Bytes per launch recorded for `kernel`, or None when absent or taken on other kernel sources."""
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel") != kernel or kv.get("sources_sha256") != gemm_sources_sha256():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def kernel_roofline(n, ms, flop, byts, steps):
    """Per-kernel figures from the library's per-launch events: the bound is MFMA when the kernel's
    algorithmic flop per byte is above the ridge (2516.6 TFLOP/s / 8 TB/s), else HBM."""
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    s = ms * 1e-3
    out = {"launches_per_step": n / steps, "ms_per_step": round(ms / steps, 4),
           "avg_launch_us": round(1e3 * ms / n, 2) if n else None}
    if s <= 0:
        return out
    if flop / max(byts, 1.0) > ridge:
        a = flop / s / 1e12
        out.update(bound="mfma", achieved=round(a, 2), unit="TFLOP/s", frac=round(a / PEAK_BF16_TFLOPS, 4))
    else:
        a = byts / s / 1e9
        out.update(bound="hbm", achieved=round(a, 1), unit="GB/s", frac=round(a / PEAK_HBM_GBS, 4))
    out["tflops"] = round(flop / s / 1e12, 2)
    return out


def step_flops(T, S, B, H, Nq, nh, d, Fr):
    gemm_fwd = 2.0 * T * H * Nq + 2.0 * T * H * Fr + 2.0 * T * Fr * H
    pairs = B * nh * S * (S + 1) / 2.0
    return {"gemm": 3.0 * gemm_fwd, "attn_fwd": 4.0 * d * pairs, "attn_bwd": 8.0 * d * pairs}


def cpu_baseline(wl, rank, seq, min_seconds=10.0, max_reps=4, one_seq=128):
    """The fp64 oracle, as it stands, on the first `seq` tokens of the same shard (same weights)."""
    import numpy as np
    import oracle
    from tensor_transformer_layer_mlp_amd import synth
    from tensor_transformer_layer_mlp_amd.configs import LayerWorkload
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    sw = LayerWorkload(wl.name + f"_first{seq}", 1, seq, wl.H, wl.n_heads, wl.F, wl.tp_size, (rank,), wl.w_std)
    h0, nh = oracle.shard_range(wl.n_heads, wl.tp_size, rank)
    f0, Fr = oracle.shard_range(wl.F, wl.tp_size, rank)
    d = wl.head_dim
    c0, c1 = 3 * d * h0, 3 * d * (h0 + nh)
    dt = "bf16"
    X = synth.X(sw, dt).f64
    W = synth.qkv_weight(sw, c0, c1, dt).f64
    bq = synth.qkv_bias(sw, c0, c1, dt).f64
    W1 = synth.fc1_weight(sw, f0, f0 + Fr, dt).f64
    b1 = synth.fc1_bias(sw, f0, f0 + Fr, dt).f64
    W2 = synth.fc2_weight(sw, f0, f0 + Fr, dt).f64
    b2 = synth.fc2_bias(sw, dt).f64
    dZ = synth.upstream(sw, wl.H, dt, "dZ").f64
    dctx = synth.column_blocks("dctx", sw.T, h0 * d, (h0 + nh) * d, 1.0, dt).f64
    t, T, H, F = wl.tp_size, sw.T, wl.H, wl.F
    reps, secs = 0, 0.0
    while reps < max_reps and (reps == 0 or secs < min_seconds):
        t0 = time.perf_counter()
        qkv = oracle.tp_qkv_shard_fwd(t, rank, 1, seq, H, wl.n_heads, X, W, bq)
        oracle.tp_attn_heads_fwd(t, rank, 1, seq, H, wl.n_heads, qkv)
        fw = oracle.tp_mlp_shard_fwd(t, rank, T, H, F, X, W1, b1, W2, b2)
        oracle.tp_mlp_shard_bwd(t, rank, T, H, F, X, W1, W2, fw["A1"], fw["Y"], dZ)
        dq = oracle.tp_attn_heads_bwd(t, rank, 1, seq, H, wl.n_heads, qkv, dctx)
        oracle.tp_qkv_shard_bwd(t, rank, 1, seq, H, wl.n_heads, X, W, dq)
        secs += time.perf_counter() - t0
        reps += 1
    fl = step_flops(T, seq, 1, H, c1 - c0, nh, d, Fr)
    total = sum(fl.values()) * reps
    res = {"value": total / secs / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"the fp64 numpy oracle, fwd+bwd of the same rank-0 shard (same shapes and "
                     f"weights) on {seq} of the 2048 tokens, {reps} pass(es): "
                     f"{total / 1e9:.1f} GFLOP in {secs:.1f} s",
           "seconds": round(secs, 2), "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    # the same oracle on one BLAS thread, over the first `one_seq` tokens (bounded CPU time)
    try:
        from threadpoolctl import threadpool_limits
        n1 = one_seq
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            qkv = oracle.tp_qkv_shard_fwd(t, rank, 1, n1, H, wl.n_heads, X[:n1], W, bq)
            oracle.tp_attn_heads_fwd(t, rank, 1, n1, H, wl.n_heads, qkv)
            fw = oracle.tp_mlp_shard_fwd(t, rank, n1, H, F, X[:n1], W1, b1, W2, b2)
            oracle.tp_mlp_shard_bwd(t, rank, n1, H, F, X[:n1], W1, W2, fw["A1"], fw["Y"], dZ[:n1])
            dq = oracle.tp_attn_heads_bwd(t, rank, 1, n1, H, wl.n_heads, qkv, dctx[:n1])
            oracle.tp_qkv_shard_bwd(t, rank, 1, n1, H, wl.n_heads, X[:n1], W, dq)
            s1 = time.perf_counter() - t0
        f1 = sum(step_flops(n1, n1, 1, H, c1 - c0, nh, d, Fr).values())
        res["single_thread"] = {"value": f1 / s1 / 1e12, "unit": "TFLOP/s", "cores": 1, "seconds": round(s1, 2),
                                "sample": f"fwd+bwd of the same shard on the first {n1} tokens, one BLAS thread"}
    except ImportError:
        res["single_thread"] = None
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


def moe_grouped(bd, torch, steps, warmup):
    """The 128-expert MoE FFN shard (row A9) on its own workload: rank 0 of tp=8, 16384 tokens routed
    top-8 -> 131072 expert-sorted rows, hidden 8192, 256 expert-ffn columns per rank.  HBM-bound:
    bytes = X_perm read + expert weights + Y written and read back + Z written."""
    from tensor_transformer_layer_mlp_amd import synth
    from tensor_transformer_layer_mlp_amd.configs import MOE_E128 as mw
    tp, rank = mw.tp_size, 0
    _, Fr = bd.tp_shard_range(mw.F_expert, tp, rank)
    off, _ = synth.moe_assignments(mw.tokens, mw.n_experts, mw.top_k)
    rows, H, G = int(off[-1]), mw.H, mw.n_experts
    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    bf = torch.bfloat16
    r = lambda *sh, std=1.0: (torch.randn(*sh, generator=g, device="cuda") * std).to(bf)  # noqa: E731
    Xp = r(rows, H)
    W1, b1, W2 = r(G, H, Fr, std=mw.w_std), r(G, Fr, std=mw.w_std), r(G, Fr, H, std=mw.w_std)
    Z, Y = torch.empty(rows, H, dtype=bf, device="cuda"), torch.empty(rows, Fr, dtype=bf, device="cuda")
    offs = torch.from_numpy(off).to("cuda")
    ws = bd.workspace("tp_mlp_grouped_shard_fwd", tp, rank, 1, rows, H, G, mw.F_expert, bf)
    call = lambda: bd.tp_mlp_grouped_shard_fwd(tp, rank, G, offs, rows, H, mw.F_expert, Xp, W1, b1,  # noqa: E731
                                               W2, Z, None, Y, ws)
    for _ in range(warmup):
        call()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    bd.tp_prof_collect()
    bd.tp_prof_enable(True)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    bd.tp_prof_enable(False)
    kernels = {tag: kernel_roofline(n, kms, fl, by, steps) for tag, (n, kms, fl, by) in bd.tp_prof_collect().items()}
    flop = 4.0 * rows * H * Fr
    byts = 2.0 * (2 * rows * H + 2 * G * H * Fr + G * Fr + 2 * rows * Fr)
    out = {"workload": mw.name + "_rank0", "rows": rows, "ms": round(ms, 4),
           "tflops": round(flop / ms / 1e9, 2), "gb_per_s": round(byts / ms / 1e6, 1),
           "hbm_frac": round(byts / ms / 1e6 / PEAK_HBM_GBS, 4), "gbyte_per_call": round(byts / 1e9, 3),
           "kernels": kernels}
    del Xp, W1, W2, Z, Y
    torch.cuda.empty_cache()
    return out


def moe_layer(bd, torch, steps, warmup):
    """The whole MoE expert block of rank 0 on the 128-expert workload, forward and backward timed
    apart.  Forward, from router logits to the combined partial: tp_moe_route (top-8 of 128,
    dispatch order) then tp_moe_shard_fwd (fc1 with the dispatch gathered from X inside its operand
    loads, GeLU, fc2, gate-weighted combine; A1 kept for the backward).  Backward, from the output
    gradient: tp_moe_shard_bwd (the experts' grouped backward with the combine's backward folded in:
    d_out's rows gathered and gate-scaled inside the GEMMs, the gate gradients from the dA1 GEMM's
    row dots; then the dispatch's backward) then tp_moe_route_bwd (router logit gradient).
    Algorithmic bytes, forward: logits, X, the expert weights, A1 and Y written, Y read, Z written
    and read back by the combine, out written.  Backward: d_out, X, A1, Y and the weights read, dA1
    written and read twice, dX, the weight gradients and the small gate / logit arrays."""
    from tensor_transformer_layer_mlp_amd.configs import MOE_E128 as mw
    tp, rank, E, k, H, tokens = mw.tp_size, 0, mw.n_experts, mw.top_k, mw.H, mw.tokens
    _, Fr = bd.tp_shard_range(mw.F_expert, tp, rank)
    n = tokens * k
    g = torch.Generator(device="cuda")
    g.manual_seed(97531)
    bf = torch.bfloat16
    r = lambda *sh, std=1.0: (torch.randn(*sh, generator=g, device="cuda") * std).to(bf)  # noqa: E731
    logits = torch.randn(tokens, E, generator=g, device="cuda")
    X = r(tokens, H)
    W1, b1, W2 = r(E, H, Fr, std=mw.w_std), r(E, Fr, std=mw.w_std), r(E, Fr, H, std=mw.w_std)
    d_out = r(tokens, H, std=1e-2)
    i32 = dict(dtype=torch.int32, device="cuda")
    gates, ex, off = torch.empty(tokens, k, device="cuda"), torch.empty(tokens, k, **i32), torch.empty(E + 1, **i32)
    rt, tr = torch.empty(n, **i32), torch.empty(tokens, k, **i32)
    e = lambda *sh: torch.empty(*sh, dtype=bf, device="cuda")  # noqa: E731
    out, Z, Y, A1 = e(tokens, H), e(n, H), e(n, Fr), e(n, Fr)
    dX, dW1, db1, dW2 = e(tokens, H), e(E, H, Fr), e(E, Fr), e(E, Fr, H)
    dg, dlog = torch.empty(tokens, k, device="cuda"), torch.empty(tokens, E, device="cuda")
    ws = bd.workspace("tp_moe_shard_fwd", tp, rank, 1, n, H, E, mw.F_expert, bf)
    wsr = bd.workspace("tp_moe_route", tp, rank, 1, tokens, H, E, mw.F_expert, bf)
    wsb = bd.workspace("tp_moe_shard_bwd", tp, rank, 1, n, H, E, mw.F_expert, bf)

    def fwd():
        bd.tp_moe_route(tokens, E, k, logits, gates, ex, off, rt, tr, wsr)
        bd.tp_moe_shard_fwd(tp, rank, tokens, H, E, k, mw.F_expert, X, gates, off, rt, tr, W1, b1, W2, out, Z, A1,
                            Y, ws)

    def bwd():
        bd.tp_moe_shard_bwd(tp, rank, tokens, H, E, k, mw.F_expert, X, gates, off, rt, tr, W1, W2, A1, Y, None, d_out,
                            dX, dg, dW1, db1, dW2, wsb)
        bd.tp_moe_route_bwd(logits, ex, dg, dlog)

    def timed(call):
        for _ in range(warmup):
            call()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            call()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        bd.tp_prof_collect()
        bd.tp_prof_enable(True)
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        bd.tp_prof_enable(False)
        return ms, {tag: kernel_roofline(c, kms, fl, by, steps) for tag, (c, kms, fl, by) in bd.tp_prof_collect().items()}

    fwd()
    ms, kernels = timed(fwd)
    byts = 4.0 * tokens * E + 2.0 * tokens * H + 2.0 * (2 * E * H * Fr + E * Fr) + 2.0 * 3 * n * Fr + \
        2.0 * 2 * n * H + 2.0 * tokens * H
    flop = 4.0 * n * H * Fr + 2.0 * n * H
    res = {"workload": mw.name + "_rank0_route_experts_combine", "tokens": tokens, "rows": n, "ms": round(ms, 4),
           "tflops": round(flop / ms / 1e9, 2), "gb_per_s": round(byts / ms / 1e6, 1),
           "hbm_frac": round(byts / ms / 1e6 / PEAK_HBM_GBS, 4), "gbyte_per_call": round(byts / 1e9, 3),
           "kernels": kernels}
    ms_b, kernels_b = timed(bwd)
    byts_b = 2.0 * (2 * tokens * H + 2 * n * Fr + 2 * E * H * Fr) + 2.0 * 3 * n * Fr + \
        2.0 * (tokens * H + 2 * E * H * Fr + E * Fr) + 4.0 * (2 * tokens * k + 2 * tokens * E)
    flop_b = 8.0 * n * H * Fr + 2.0 * n * H
    res["bwd"] = {"ms": round(ms_b, 4), "tflops": round(flop_b / ms_b / 1e9, 2),
                  "gb_per_s": round(byts_b / ms_b / 1e6, 1), "hbm_frac": round(byts_b / ms_b / 1e6 / PEAK_HBM_GBS, 4),
                  "gbyte_per_call": round(byts_b / 1e9, 3), "kernels": kernels_b}
    del X, W1, W2, Z, Y, A1, out, dX, dW1, dW2, d_out, ws, wsb
    torch.cuda.empty_cache()
    return res


PEAK_FP8_TFLOPS = 5033.2   # dense E4M3 MFMA: twice the bf16 rate


def fp8_mlp(bd, torch, wl, steps, warmup):
    """The MLP shard in FP8 on the GPT-3 rank-0 shapes (T 2048, H 12288, F_r 6144), forward and
    backward timed apart.  Forward: quantise X (E4M3), X·W1 (2048 x 6144 x 12288) with bias + GeLU
    (A1 kept), quantise Y, Y·W2 (2048 x 12288 x 6144).  Backward: dZ in E5M2 (plain and the
    transposed copy), dA1 = (dZ·W2ᵀ) ∘ GeLU'(A1), dW2 = Yᵀ·dZ, dA1 in E5M2 (both copies),
    dX = dA1·W1ᵀ, dW1 = Xᵀ·dA1, db1 = Σ_t dA1; dZ and dA1 are quantised once into both layouts, and
    the K-major copies of X and Y the weight gradients take are quantised inside the backward.  Weights are quantised once, outside the timed region
    (both copies; they change once per optimizer step).  A precision variant beside the bf16 step,
    against the FP8 peak."""
    T, H = wl.T, wl.H
    _, Fr = bd.tp_shard_range(wl.F, wl.tp_size, 0)
    g = torch.Generator(device="cuda")
    g.manual_seed(8642)
    bf = torch.bfloat16
    r = lambda *sh, std=1.0: (torch.randn(*sh, generator=g, device="cuda") * std).to(bf)  # noqa: E731
    X, W1, b1, W2 = r(T, H), r(H, Fr, std=wl.w_std), r(Fr, std=wl.w_std), r(Fr, H, std=wl.w_std)
    dZ = r(T, H, std=1e-3)
    u8 = lambda *sh: torch.empty(*sh, dtype=torch.uint8, device="cuda")  # noqa: E731
    qX, qXt, qW1t, qW1, qW2t, qW2, qY, qYt = u8(T, H), u8(H, T), u8(Fr, H), u8(H, Fr), u8(H, Fr), u8(Fr, H), \
        u8(T, Fr), u8(Fr, T)
    qdZ, qdZt, qdA1, qdA1t = u8(T, H), u8(H, T), u8(T, Fr), u8(Fr, T)
    sX, sW1, sW2, sY, sdZ, sdA1 = (torch.empty(1, device="cuda") for _ in range(6))
    e = lambda *sh: torch.empty(*sh, dtype=bf, device="cuda")  # noqa: E731
    A1, Y, Z = e(T, Fr), e(T, Fr), e(T, H)
    dA1, dW2, dX, dW1, db1 = e(T, Fr), e(Fr, H), e(T, H), e(H, Fr), e(Fr)
    ws = bd.workspace("tp_fp8_quantize", 1, 0, 1, 1, 1, 1, 1, bf)
    wsb = bd.workspace("tp_bias_grad", 1, 0, T, 1, Fr, 1, 1, bf)
    e4, e5 = bd.TP_FP8_E4M3, bd.TP_FP8_E5M2
    bd.tp_fp8_quantize(W1, qW1, sW1, ws, q_t=qW1t)
    bd.tp_fp8_quantize(W2, qW2, sW2, ws, q_t=qW2t)

    def fwd():
        bd.tp_fp8_quantize(X, qX, sX, ws)
        bd.tp_fp8_gemm_nt(qX, sX, qW1t, sW1, Y, bias=b1, epilogue=bd.TP_FP8_EPI_GELU, C_pre=A1)
        bd.tp_fp8_quantize(Y, qY, sY, ws)
        bd.tp_fp8_gemm_nt(qY, sY, qW2t, sW2, Z)

    def bwd():
        bd.tp_fp8_quantize(dZ, qdZ, sdZ, ws, q_t=qdZt, fmt=e5)
        bd.tp_fp8_gemm_nt(qdZ, sdZ, qW2, sW2, dA1, epilogue=bd.TP_FP8_EPI_DGELU, aux=A1, a_fmt=e5, b_fmt=e4)
        bd.tp_fp8_quantize(Y, None, sY, ws, q_t=qYt)
        bd.tp_fp8_gemm_nt(qYt, sY, qdZt, sdZ, dW2, a_fmt=e4, b_fmt=e5)
        bd.tp_fp8_quantize(dA1, qdA1, sdA1, ws, q_t=qdA1t, fmt=e5)
        bd.tp_fp8_gemm_nt(qdA1, sdA1, qW1, sW1, dX, a_fmt=e5, b_fmt=e4)
        bd.tp_fp8_quantize(X, None, sX, ws, q_t=qXt)
        bd.tp_fp8_gemm_nt(qXt, sX, qdA1t, sdA1, dW1, a_fmt=e4, b_fmt=e5)
        bd.tp_bias_grad(dA1, db1, wsb)

    def timed(call, flop):
        for _ in range(warmup):
            call()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            call()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        bd.tp_prof_collect()
        bd.tp_prof_enable(True)
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        bd.tp_prof_enable(False)
        kernels = {}
        for tag, (n, kms, fl, by) in bd.tp_prof_collect().items():
            us = 1e3 * kms / n
            k = {"launches_per_step": n / steps, "avg_launch_us": round(us, 2)}
            if tag.startswith("gemm_fp8"):
                tf = fl / n / us / 1e6
                k.update(tflops=round(tf, 1), frac_of_fp8_peak=round(tf / PEAK_FP8_TFLOPS, 4))
            else:
                k.update(gb_per_s=round(by / n / us / 1e3, 1))
            kernels[tag] = k
        return {"ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
                "pct_of_fp8_peak": round(100 * flop / ms / 1e9 / PEAK_FP8_TFLOPS, 2), "kernels": kernels}

    fwd()
    res = {"workload": "gpt3_175b_tp8_rank0_mlp_fp8_e4m3_fwd_e5m2_grads",
           "fwd": timed(fwd, 2 * 2.0 * T * H * Fr), "bwd": timed(bwd, 4 * 2.0 * T * H * Fr)}
    del X, W1, W2, dZ, qX, qXt, qW1t, qW1, qW2t, qW2, qY, qYt, qdZ, qdZt, qdA1, qdA1t, A1, Y, Z, dA1, dW2, dX, dW1
    torch.cuda.empty_cache()
    return res


def attn_out_proj(bd, torch, wl, rank, steps, warmup):
    """The attention output projection of the same shard (a RowParallelLinear over the rank's 12
    heads: O_r = ctx_r·Wo_r + bo, then dWo_r, dbo, dctx_r), forward + backward, timed on its own
    beside the step: 3 GEMMs of 2·T·(nh_r·d)·H flop each."""
    t, B, S, H, nh_all = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads
    T, d = wl.T, wl.head_dim
    _, nh = bd.tp_shard_range(nh_all, t, rank)
    Kr = nh * d
    g = torch.Generator(device="cuda")
    g.manual_seed(5678)
    bf = torch.bfloat16
    r = lambda *sh, std=1.0: (torch.randn(*sh, generator=g, device="cuda") * std).to(bf)  # noqa: E731
    ctx, dO = r(T, Kr), r(T, H)
    Wo, bo = r(Kr, H, std=wl.w_std), r(H, std=wl.w_std)
    e = lambda *sh: torch.empty(*sh, dtype=bf, device="cuda")  # noqa: E731
    O, dctx, dWo, dbo = e(T, H), e(T, Kr), e(Kr, H), e(H)
    ws = bd.workspace("tp_attn_out_shard_bwd", t, rank, B, S, H, nh_all, wl.F, bf)

    def call():
        bd.tp_attn_out_shard_fwd(t, rank, B, S, H, nh_all, ctx, Wo, bo, O)
        bd.tp_attn_out_shard_bwd(t, rank, B, S, H, nh_all, ctx, Wo, dO, dctx, dWo, dbo, ws)
    for _ in range(warmup):
        call()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    bd.tp_prof_collect()
    bd.tp_prof_enable(True)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    bd.tp_prof_enable(False)
    kernels = {tag: kernel_roofline(n, kms, fl, by, steps) for tag, (n, kms, fl, by) in bd.tp_prof_collect().items()}
    flop = 3 * 2.0 * T * Kr * H
    out = {"workload": "gpt3_175b_tp8_rank0_attn_out_proj_fwd_bwd", "ms": round(ms, 4),
           "gflop": round(flop / 1e9, 1), "tflops": round(flop / ms / 1e9, 2),
           "pct_of_peak": round(100.0 * flop / ms / 1e9 / PEAK_BF16_TFLOPS, 2), "kernels": kernels}
    del ctx, dO, Wo, O, dctx, dWo
    torch.cuda.empty_cache()
    return out, flop


def residual_ln(bd, torch, wl, steps, warmup):
    """The residual add with dropout + LayerNorm of the same layer, forward + backward, on its own:
    replicated (all 2048 tokens of H = 12288, as plain tensor parallelism holds it) and sequence-
    parallel (rank 0's 256-token block of 8).  HBM-bound: algorithmic bytes = x, o read, keep read,
    h, y written (9 B per element in bf16) forward; dy, h, dh_in, keep read, dh, d_o written (11 B)
    backward, then dy and h read again for dγ, dβ (4 B)."""
    T, H, p = wl.T, wl.H, 0.1
    g = torch.Generator(device="cuda")
    g.manual_seed(2468)
    bf = torch.bfloat16
    r = lambda *sh, std=1.0: (torch.randn(*sh, generator=g, device="cuda") * std).to(bf)  # noqa: E731
    out = {}
    for name, sp, rows in (("replicated", False, T), ("sequence_parallel_rank0", True, bd.tp_shard_range(T, 8, 0)[1])):
        x, o, dy, dh_in = r(rows, H), r(rows, H), r(rows, H), r(rows, H)
        gamma, beta = 1.0 + r(H, std=0.1).float(), r(H, std=0.1)
        gamma = gamma.to(bf)
        keep = (torch.rand(rows, H, generator=g, device="cuda") >= p).to(torch.uint8)
        e = lambda *sh, dt=bf: torch.empty(*sh, dtype=dt, device="cuda")  # noqa: E731
        h, y, dh, d_o, dg, db = e(rows, H), e(rows, H), e(rows, H), e(rows, H), e(H), e(H)
        mean, rstd = e(rows, dt=torch.float32), e(rows, dt=torch.float32)
        ws = bd.workspace("tp_residual_ln_bwd", 8, 0, 1, T, H, 1, 1, bf)

        def call():
            bd.tp_residual_ln_fwd(8, 0, sp, T, H, x, o, keep, p, gamma, beta, 1e-5, h, y, mean, rstd)
            bd.tp_residual_ln_bwd(8, 0, sp, T, H, dy, dh_in, h, mean, rstd, gamma, keep, p, dh, d_o, dg, db, ws)
        for _ in range(warmup):
            call()
        bd.tp_prof_collect()
        bd.tp_prof_enable(True)
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        bd.tp_prof_enable(False)
        k = bd.tp_prof_collect()
        n = rows * H
        res = {"rows": rows, "H": H}
        for tag, alg in (("ln_fwd", 9.0 * n), ("ln_bwd", 11.0 * n)):
            if tag in k:
                cnt, ms, _, _ = k[tag]
                us = 1e3 * ms / cnt
                res[tag] = {"avg_launch_us": round(us, 2), "algorithmic_bytes": alg,
                            "gb_per_s": round(alg / us / 1e3, 1), "hbm_frac": round(alg / us / 1e3 / PEAK_HBM_GBS, 4)}
        if "ln_bwd_params" in k:           # dγ, dβ: dy and h read again (4 B per element), two sums
            cnt, ms, _, _ = k["ln_bwd_params"]
            us = 1e3 * ms / cnt
            res["ln_bwd_params"] = {"avg_launch_us": round(us, 2), "algorithmic_bytes": 4.0 * n,
                                    "gb_per_s": round(4.0 * n / us / 1e3, 1)}
        out[name] = res
        del x, o, dy, dh_in, keep, h, y, dh, d_o
    torch.cuda.empty_cache()
    return out


# ---- profile summaries (rocprofv3 CSV output -> the tables under profiles/) -----------------------

# the GPT-3 shard step's library dispatches in launch order with every launch on one stream
# (TP_SERIAL=1): the labels of the per-dispatch counter tables
STEP_LABELS = ["QKV fwd (NN+bias) 2048x4608x12288", "attn fwd", "fc1 (NN+bias+GeLU) 2048x6144x12288",
               "fc2 (NN+bias) 2048x12288x6144", "dA1 (NT+GeLU') 2048x6144x12288", "dW2 (TN) 6144x12288x2048",
               "db2 colsum partial", "db2 colsum final", "dX mlp (NT) 2048x12288x6144", "db1 colsum partial",
               "db1 colsum final", "dW1 (TN) 12288x6144x2048", "attn bwd dQ (+ row dots)", "attn bwd dK/dV",
               "dWqkv (TN) 12288x4608x2048", "dbqkv colsum partial", "dbqkv colsum final",
               "dX qkv (NT) 2048x12288x4608"]


def _csv_files(d, suffix):
    found = []
    for root, _, files in os.walk(d):
        found += [os.path.join(root, f) for f in files if f.endswith(suffix)]
    if not found:
        raise SystemExit(f"no *{suffix} under {d}")
    return sorted(found)


def short_kernel(name):
    import re
    name = name.replace("tp::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    m = re.match(r"void (gemm_\w+)<(.*)>\([\w:, ]*\)$", name)
    if m:
        return f"{m.group(1)}<{m.group(2)}>"
    m = re.match(r"_ZN2tp12_GLOBAL__N_1(\d+)(\w+)", name)
    if m:
        n = int(m.group(1))
        return m.group(2)[:n]
    m = re.match(r"(?:void )?([\w:]+)", name)
    return (m.group(1) if m else name)[:150]


def _is_library(name):
    return any(k in name for k in ("tp::", "_ZN2tp", "gemm_", "attn_", "colsum", "ln_", "moe_", "fp8_", "grouped"))


def _trace_rows(d):
    import csv
    rows = []
    for f in _csv_files(d, "kernel_trace.csv"):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return rows


def _pmc_dispatches(d):
    """Per dispatch, in dispatch order: name, grid, duration (us) and each counter summed over its
    instances (XCDs, SEs)."""
    import csv
    disp = {}
    for f in _csv_files(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            k = (f, int(r["Dispatch_Id"]))
            e = disp.setdefault(k, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                    "dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def _calibration(dispatches, counter, true_kib):
    """Factor turning `counter` (KiB) into bytes, from the 1 GiB fp32 negation the pmc pass starts with."""
    cal = [e for e in dispatches if "neg" in e["name"].lower() and e["grid"] >= (1 << 26)]
    if not cal:
        raise SystemExit("calibration copy (the 1 GiB negation) not found in the counter run")
    return true_kib / cal[0][counter] * 1024.0


def summarize(what, d, kernel, tag):
    if what == "stats":
        rows = _trace_rows(d)
        per = {}
        for r in rows:
            key = short_kernel(r["Kernel_Name"])
            per.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        total = sum(sum(v) for v in per.values())
        print("# columns: calls, average us, min us, max us, median us, share of kernel time, kernel")
        for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            srt = sorted(v)
            print("%5d %10.2f %10.2f %10.2f %10.2f %6.2f%%  %s" % (len(v), sum(v) / len(v), srt[0], srt[-1],
                                                                   srt[len(v) // 2], 100 * sum(v) / total, k))
    elif what in ("traffic", "hbm"):
        f = _pmc_dispatches(os.path.join(d, "pmc_fetch"))
        w = _pmc_dispatches(os.path.join(d, "pmc_write"))
        ff = _calibration(f, "FETCH_SIZE", 1 << 20)
        fw = _calibration(w, "WRITE_SIZE", 1 << 20)
        print(f"# calibration: fp32 negation of 1 GiB (reads 1 GiB, writes 1 GiB): factors {ff / 1024:.4f} "
              f"(FETCH_SIZE), {fw / 1024:.4f} (WRITE_SIZE)")
        lib = lambda ds: [e for e in ds if _is_library(e["name"])]  # noqa: E731
        f, w = lib(f), lib(w)
        if what == "traffic":
            fl = [e for e in f if short_kernel(e["name"]) == kernel][-3:]
            wl_ = [e for e in w if short_kernel(e["name"]) == kernel][-3:]
            if not fl:
                raise SystemExit(f"kernel {kernel} not in the counter runs")
            for a, b in zip(fl, wl_):
                print("# grid %d: fetch %.1f MB, write %.1f MB" % (a["grid"], a["FETCH_SIZE"] * ff / 1e6,
                                                                   b["WRITE_SIZE"] * fw / 1e6))
            fb = sum(a["FETCH_SIZE"] for a in fl) / len(fl) * ff
            wb = sum(b["WRITE_SIZE"] for b in wl_) / len(wl_) * fw
            # every GEMM of the last step, in launch order (the pass runs the GPT-3 tp=8 rank-0 step; its
            # nine GEMMs are the last nine GEMM dispatches): HBM-side bytes against the operands' unique bytes
            gf = [e for e in f if "gemm" in short_kernel(e["name"])][-9:]
            gw = [e for e in w if "gemm" in short_kernel(e["name"])][-9:]
            if len(gf) == 9 and len(gw) == 9:
                sh = gemm_site_shapes(2048, 12288, 4608, 6144)
                print("# every GEMM of the last step: HBM-side fetch / write per dispatch, and the fetch over the")
                print("# unique bytes of the operands it reads (A, B, and A1 for dA1's GeLU')")
                print("# %-8s %6s %6s %6s %9s %9s %10s %8s" % ("site", "M", "N", "K", "fetch MB", "write MB",
                                                               "unique MB", "refetch"))
                for site, a, b in zip(sh, gf, gw):
                    M, N, K = sh[site]
                    uniq = 2.0 * (M * K + K * N + (M * N if site == "dA1" else 0))
                    fm = a["FETCH_SIZE"] * ff
                    print("# %-8s %6d %6d %6d %9.1f %9.1f %10.1f %7.2fx" % (site, M, N, K, fm / 1e6,
                                                                           b["WRITE_SIZE"] * fw / 1e6, uniq / 1e6,
                                                                           fm / uniq))
            print(f"trace_kernel: {kernel}")
            print(f"kernel: {tag}")
            print(f"sources_sha256: {gemm_sources_sha256()}")
            print(f"fetch_bytes_per_launch: {int(fb)}")
            print(f"write_bytes_per_launch: {int(wb)}")
            print(f"traffic_bytes_per_launch: {int(fb + wb)}")
        else:
            trace = _trace_rows(os.path.join(d, "trace"))
            dur = {}
            for r in trace:
                key = (short_kernel(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
                dur.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            print("# HBM-side bytes per dispatch (counters x calibration) over the median duration of the same")
            print("# kernel and grid in the kernel-trace run; every bandwidth-bound library dispatch of the last")
            print("# pass (GEMMs and attention excluded)")
            print("%-34s %9s %10s %10s %9s %9s %8s" % ("kernel", "grid", "fetch MB", "write MB", "dur us",
                                                       "GB/s", "of 8 TB/s"))
            seen = set()
            for a, b in reversed(list(zip(f, w))):
                name = short_kernel(a["name"])
                if "gemm" in name or "attn_fwd" in name or "attn_bwd" in name:
                    continue
                key = (name, a["grid"])
                if key in seen:
                    continue
                seen.add(key)
                ds = sorted(dur.get(key, [a["dur"]]))
                us = ds[len(ds) // 2]
                byts = a["FETCH_SIZE"] * ff + b["WRITE_SIZE"] * fw
                print("%-34s %9d %10.2f %10.2f %9.2f %9.1f %7.1f%%" % (name[:34], a["grid"], a["FETCH_SIZE"] * ff / 1e6,
                                                                       b["WRITE_SIZE"] * fw / 1e6, us, byts / us / 1e3,
                                                                       100 * byts / us / 1e3 / PEAK_HBM_GBS))
    elif what == "lds":
        L = [e for e in _pmc_dispatches(os.path.join(d, "pmc_lds")) if _is_library(e["name"])]
        T = [e for e in _pmc_dispatches(os.path.join(d, "pmc_ta")) if _is_library(e["name"])]
        n = len(STEP_LABELS)
        print("# per dispatch of the last step; cycles = GRBM_GUI_ACTIVE / 8, utilisations over 256 CUs")
        print("# LdsUtil = SQ_LDS_IDX_ACTIVE / (cycles x 256) (indexed LDS operations only: ds_read / ds_write,")
        print("#   not the direct global -> LDS loads); bank = SQ_LDS_BANK_CONFLICT / (cycles x 256);")
        print("# TA, TD = TA_TA_BUSY, TD_TD_BUSY / (cycles x 256); wait LDS, wait any = SQ_WAIT_INST_LDS,")
        print("#   SQ_WAIT_ANY / SQ_WAVE_CYCLES (shares of the waves' resident cycles)")
        print("%-36s %7s %8s %6s %6s %6s %9s %9s" % ("dispatch", "dur us", "LdsUtil", "bank", "TA", "TD", "wait LDS",
                                                     "wait any"))
        labels = STEP_LABELS if len(L) % n == 0 else [short_kernel(e["name"])[:36] for e in L[-n:]]
        for lab, a, b in zip(labels, L[-n:], T[-n:]):
            g = a["GRBM_GUI_ACTIVE"] / 8 * 256
            wc = max(b["SQ_WAVE_CYCLES"], 1.0)
            print("%-36s %7.1f %7.1f%% %5.1f%% %5.1f%% %5.1f%% %8.1f%% %8.1f%%" % (
                lab[:36], a["dur"], 100 * a["SQ_LDS_IDX_ACTIVE"] / g, 100 * a["SQ_LDS_BANK_CONFLICT"] / g,
                100 * b["TA_TA_BUSY"] / g, 100 * b["TD_TD_BUSY"] / g, 100 * a["SQ_WAIT_INST_LDS"] / wc,
                100 * b["SQ_WAIT_ANY"] / wc))
    elif what == "blas":
        # the JSON line of a --blas-compare run, saved as <prof-dir>/blas.log
        line = [x for x in open(os.path.join(d, "blas.log")) if x.startswith("{")][-1]
        j = json.loads(line)
        bc, sites = j["blas_compare"], j["gemm_call_sites"]
        print(f"# library: {bc['library']}, torch {bc['torch']}")
        print("%-8s %6s %6s %6s %12s %12s %12s %12s" % ("gemm", "M", "N", "K", "BLAS us", "BLAS TF/s", "here us",
                                                        "here TF/s"))
        tb = th = fl = 0.0
        for site in GEMM_SITES:
            b, h = bc["gemms"][site], sites[site]
            f = 2.0 * b["M"] * b["N"] * b["K"]
            tb, th, fl = tb + b["avg_us"], th + h["avg_launch_us"], fl + f
            print("%-8s %6d %6d %6d %12.1f %12.1f %12.1f %12.1f" % (site, b["M"], b["N"], b["K"], b["avg_us"],
                                                                    f / b["avg_us"] / 1e6, h["avg_launch_us"],
                                                                    f / h["avg_launch_us"] / 1e6))
        print("%-8s %20s %12.1f %12.1f %12.1f %12.1f" % ("total", "", tb, fl / tb / 1e6, th, fl / th / 1e6))
    elif what == "mfma":
        import numpy as np
        clk = [e for e in _pmc_dispatches(os.path.join(d, "pmc_clk")) if _is_library(e["name"])]
        mf = [e for e in _pmc_dispatches(os.path.join(d, "pmc_mfma")) if _is_library(e["name"])]
        x = np.array([c["dur"] * 1e3 for c in clk])
        y = np.array([c["GRBM_GUI_ACTIVE"] / 8 for c in clk])
        A = np.vstack([np.ones_like(x), x]).T
        (c0, c1), *_ = np.linalg.lstsq(A, y, rcond=None)
        print("# clock fit over %d dispatches: GRBM_GUI_ACTIVE/8 = %.0f cycles + %.3f GHz x duration (ns)" %
              (len(clk), c0, c1))
        print("%-38s %7s %7s %9s %11s %10s %7s" % ("dispatch", "grid", "dur us", "clock GHz", "MFMA busy %",
                                                   "MFMA TF/s", "frac"))
        n = len(STEP_LABELS)
        labels = STEP_LABELS if len(clk) % n == 0 else [short_kernel(e["name"])[:38] for e in clk[-n:]]
        for lab, a, b in zip(labels, clk[-n:], mf[-n:]):
            ghz = (a["GRBM_GUI_ACTIVE"] / 8 - c0) / (a["dur"] * 1e3)
            busy = 100 * b.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (b["GRBM_GUI_ACTIVE"] / 8 * 1024)
            tf = b.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) * 512 / (b["dur"] * 1e-6) / 1e12
            print("%-38s %7d %7.1f %9.2f %11.1f %10.1f %7.3f" % (lab, a["grid"], a["dur"], ghz, busy, tf,
                                                                 tf / PEAK_BF16_TFLOPS))


# the nine GEMMs of a layer shard's step: call site -> (M, N, K) in terms of T, H, Nq, F_r
GEMM_SITES = ("qkv_fwd", "fc1", "fc2", "dA1", "dW2", "dX_mlp", "dW1", "dWqkv", "dX_qkv")
GEMM_TARGET_FRAC = 0.70


def gemm_site_shapes(T, H, Nq, Fr):
    return {"qkv_fwd": (T, Nq, H), "fc1": (T, Fr, H), "fc2": (T, H, Fr), "dA1": (T, Fr, H), "dW2": (Fr, H, T),
            "dX_mlp": (T, H, Fr), "dW1": (H, Fr, T), "dWqkv": (H, Nq, T), "dX_qkv": (T, H, Nq)}


def split_sites(k):
    """Per-launch records keyed "site|tag" (or a bare tag) -> (by kernel tag, by call site)."""
    by_tag, by_site = {}, {}
    for key, v in k.items():
        site, tag = key.split("|", 1) if "|" in key else (None, key)
        for d, name in ((by_tag, tag), (by_site, site)):
            if name is None:
                continue
            a = d.get(name, (0, 0.0, 0.0, 0.0))
            d[name] = tuple(x + y for x, y in zip(a, v))
        if site is not None:
            by_site.setdefault(site + "#tags", set()).add(tag)
    return by_tag, by_site


class LayerShard:
    """One rank's shard of a layer workload on the GPU: seeded inputs resident in HBM, and one step =
    the whole hot path forward and backward through the C ABI:
        tp_qkv_shard_fwd -> tp_attn_heads_fwd -> tp_mlp_shard_fwd ->
        tp_mlp_shard_bwd -> tp_attn_heads_bwd -> tp_qkv_shard_bwd"""

    def __init__(self, bd, torch, wl, rank, seed=1234):
        self.bd, self.torch, self.wl, self.rank = bd, torch, wl, rank
        t, B, S, H, nh_all, F = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F
        T, d = wl.T, wl.head_dim
        _, nh = bd.tp_shard_range(nh_all, t, rank)
        _, Fr = bd.tp_shard_range(F, t, rank)
        Nq = 3 * nh * d
        self.T, self.H, self.Nq, self.Fr, self.nh, self.d = T, H, Nq, Fr, nh, d
        dev, bf = "cuda", torch.bfloat16
        g = torch.Generator(device=dev)
        g.manual_seed(seed)

        def randn(shape, std):
            return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(bf)

        self.X, self.dZ, self.dctx = randn((T, H), 1.0), randn((T, H), 1.0), randn((T, nh * d), 1.0)
        self.Wq, self.bq = randn((H, Nq), wl.w_std), randn((Nq,), wl.w_std)
        self.W1, self.b1 = randn((H, Fr), wl.w_std), randn((Fr,), wl.w_std)
        self.W2, self.b2 = randn((Fr, H), wl.w_std), randn((H,), wl.w_std)
        e = lambda *s, dt=bf: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        self.QKV, self.ctx, self.lse = e(T, Nq), e(T, nh * d), e(B, nh, S, dt=torch.float32)
        self.Z, self.A1, self.Y = e(T, H), e(T, Fr), e(T, Fr)
        self.dXm, self.dW1, self.db1, self.dW2, self.db2 = e(T, H), e(H, Fr), e(Fr), e(Fr, H), e(H)
        self.dQKV, self.dXq, self.dWq, self.dbq = e(T, Nq), e(T, H), e(H, Nq), e(Nq)
        self.ws_m = bd.workspace("tp_mlp_shard_bwd", t, rank, B, S, H, nh_all, F, bf)
        self.ws_q = bd.workspace("tp_qkv_shard_bwd", t, rank, B, S, H, nh_all, F, bf)
        self.ws_a = bd.workspace("tp_attn_heads_bwd", t, rank, B, S, H, nh_all, F, bf)
        self.flops = step_flops(T, S, B, H, Nq, nh, d, Fr)
        self.flop_step = sum(self.flops.values())

    def step(self):
        bd, wl, r = self.bd, self.wl, self.rank
        t, B, S, H, nh_all, F, T = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F, self.T
        bd.tp_qkv_shard_fwd(t, r, B, S, H, nh_all, self.X, self.Wq, self.bq, self.QKV)
        bd.tp_attn_heads_fwd(t, r, B, S, H, nh_all, self.QKV, self.ctx, self.lse)
        bd.tp_mlp_shard_fwd(t, r, T, H, F, self.X, self.W1, self.b1, self.W2, self.b2, self.Z, self.A1, self.Y)
        bd.tp_mlp_shard_bwd(t, r, T, H, F, self.X, self.W1, self.W2, self.A1, self.Y, self.dZ, self.dXm, self.dW1,
                            self.db1, self.dW2, self.db2, self.ws_m)
        bd.tp_attn_heads_bwd(t, r, B, S, H, nh_all, self.QKV, self.ctx, self.lse, self.dctx, self.dQKV, self.ws_a)
        bd.tp_qkv_shard_bwd(t, r, B, S, H, nh_all, self.X, self.Wq, self.dQKV, self.dXq, self.dWq, self.dbq,
                            self.ws_q)

    def timed(self, steps, with_events=False):
        """Mean step time over `steps` steps between two events on the stream (nothing else enqueued
        in between); with_events: the library's per-launch events on (their per-site/tag totals)."""
        torch, bd = self.torch, self.bd
        stream = torch.cuda.current_stream()
        if with_events:
            bd.tp_prof_collect()          # drop anything recorded before
            bd.tp_prof_enable(True)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        t0.record(stream)
        for _ in range(steps):
            self.step()
        t1.record(stream)
        torch.cuda.synchronize()
        w = time.perf_counter() - w0
        k = None
        if with_events:
            bd.tp_prof_enable(False)
            k = bd.tp_prof_collect()
        return t0.elapsed_time(t1) / steps, w, k

    def per_step(self, steps, cold=False):
        """Each step timed alone between two events; cold: a 1 GiB buffer (4x the 256 MB last-level
        cache) is written before each step, outside its events, so the step starts with none of its
        operands cached."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        flush = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda") if cold else None
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(ev):
            if cold:
                flush.fill_(float(i))
            a.record(stream)
            self.step()
            b.record(stream)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)
        del flush
        return ms

    def gemm_sites(self, by_site, steps):
        shapes = gemm_site_shapes(self.T, self.H, self.Nq, self.Fr)
        out = {}
        for site in GEMM_SITES:
            if site not in by_site:
                continue
            n, ms, flop, byts = by_site[site]
            M, N, K = shapes[site]
            us = 1e3 * ms / n
            tf = flop / n / (us * 1e-6) / 1e12
            out[site] = {"M": M, "N": N, "K": K, "kernel": sorted(by_site[site + "#tags"])[0],
                         "avg_launch_us": round(us, 2), "tflops": round(tf, 1),
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "target_frac": GEMM_TARGET_FRAC,
                         "meets_target": bool(tf / PEAK_BF16_TFLOPS >= GEMM_TARGET_FRAC)}
        return out

    def measure(self, steps, warmup, events=True, cold=True):
        for _ in range(warmup):
            self.step()
        ms, wall, _ = self.timed(steps)
        res = {"ms_per_step": round(ms, 4), "tflops": round(self.flop_step / (ms * 1e-3) / 1e12, 2),
               "pct_of_peak": round(100.0 * self.flop_step / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
               "gflop_per_step": round(self.flop_step / 1e9, 1), "wall_s_timed_region": round(wall, 3)}
        each = self.per_step(steps)
        res["ms_per_step_median"] = round(each[len(each) // 2], 4)
        res["ms_per_step_min"] = round(each[0], 4)
        if cold:
            c = self.per_step(steps, cold=True)
            res["ms_per_step_cold_median"] = round(c[len(c) // 2], 4)
            res["ms_per_step_cold_min"] = round(c[0], 4)
            res["tflops_cold_median"] = round(self.flop_step / (c[len(c) // 2] * 1e-3) / 1e12, 2)
        if events:
            ms_ev, _, k = self.timed(steps, with_events=True)
            by_tag, by_site = split_sites(k)
            res["ms_per_step_with_kernel_events"] = round(ms_ev, 4)
            res["kernels"] = {tag: kernel_roofline(n, kms, fl, by, steps) for tag, (n, kms, fl, by) in by_tag.items()}
            res["gemm_call_sites"] = self.gemm_sites(by_site, steps)
            res["_by_tag_raw"] = by_tag
        return res

    def free(self):
        for k in list(vars(self)):
            if k not in ("bd", "torch", "wl", "rank"):
                setattr(self, k, None)
        self.torch.cuda.empty_cache()


def blas_compare(torch, wl, rank, steps, warmup):
    """The vendor BLAS (torch.matmul, bf16 in, fp32 accumulation) on the nine GEMM shapes of the same
    shard, each timed alone in the same operand layouts (weights [in, out], the weight gradients as
    Xᵀ·dY on the stored X): a reference point, not part of the step."""
    from tensor_transformer_layer_mlp_amd import binding as bd
    T, H, d = wl.T, wl.H, wl.head_dim
    _, nh = bd.tp_shard_range(wl.n_heads, wl.tp_size, rank)
    _, Fr = bd.tp_shard_range(wl.F, wl.tp_size, rank)
    Nq = 3 * nh * d
    bf = torch.bfloat16
    r = lambda *s: torch.randn(*s, device="cuda").to(bf)  # noqa: E731
    X, dZ, dQ, A, Yv = r(T, H), r(T, H), r(T, Nq), r(T, Fr), r(T, Fr)
    Wq, W1, W2 = r(H, Nq) * 0.006, r(H, Fr) * 0.006, r(Fr, H) * 0.006
    calls = {"qkv_fwd": lambda: torch.matmul(X, Wq), "fc1": lambda: torch.matmul(X, W1),
             "fc2": lambda: torch.matmul(Yv, W2), "dA1": lambda: torch.matmul(dZ, W2.t()),
             "dW2": lambda: torch.matmul(Yv.t(), dZ), "dX_mlp": lambda: torch.matmul(A, W1.t()),
             "dW1": lambda: torch.matmul(X.t(), A), "dWqkv": lambda: torch.matmul(X.t(), dQ),
             "dX_qkv": lambda: torch.matmul(dQ, Wq.t())}
    shapes = gemm_site_shapes(T, H, Nq, Fr)
    out, total_us, total_flop = {}, 0.0, 0.0
    for site, f in calls.items():
        for _ in range(warmup):
            f()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            f()
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / steps
        M, N, K = shapes[site]
        fl = 2.0 * M * N * K
        out[site] = {"M": M, "N": N, "K": K, "avg_us": round(us, 2), "tflops": round(fl / us / 1e6, 1)}
        total_us += us
        total_flop += fl
    return {"library": "torch.matmul (rocBLAS / hipBLASLt)", "torch": torch.__version__, "gemms": out,
            "total_us": round(total_us, 1), "tflops": round(total_flop / total_us / 1e6, 1)}


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.prof_dir, args.kernel, args.tag)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the shard of one rank runs on one MI355X, and no "
              f"collective is part of this build (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from tensor_transformer_layer_mlp_amd import binding as bd
    from tensor_transformer_layer_mlp_amd.configs import GPT2_1P5B, GPT3_175B, GPT_8P3B

    wl, rank = GPT3_175B, 0
    sh = LayerShard(bd, torch, wl, rank)

    if args.pmc_pass:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        c = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=c)                     # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del a, c
        for _ in range(args.warmup + args.steps):
            sh.step()
        torch.cuda.synchronize()
        if args.pmc_ln:
            sh.free()
            residual_ln(bd, torch, wl, 1, 0)
        print(json.dumps({"pmc_pass": True, "calibration_bytes": 1 << 30, "steps": args.warmup + args.steps,
                          "gemm_sources_sha256": gemm_sources_sha256()}), flush=True)
        return

    events = not args.no_kernel_events
    head = sh.measure(args.steps, args.warmup, events=events, cold=not args.no_cold)
    ms_step = head["ms_per_step"]
    # the same step captured once in a HIP graph and replayed (the entry points allocate and
    # synchronise nothing, so capture is legal); reported beside the eager figure
    ms_graph = None
    if not args.no_graph:
        stream = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            sh.step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sh.step()
        for _ in range(args.warmup):
            graph.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        ms_graph = g0.elapsed_time(g1) / args.steps
        del graph
    flop_step = sh.flop_step
    tflops = flop_step / (ms_step * 1e-3) / 1e12

    roofline = None
    if events:
        kernels = head.pop("_by_tag_raw")
        dom = max(kernels, key=lambda k: kernels[k][1])
        n, ms, flop, byts = kernels[dom]
        ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)      # flop per byte
        avg_s = ms * 1e-3 / n
        if flop / max(byts, 1.0) > ridge:
            ach = flop / n / avg_s / 1e12
            roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                        "traffic": recorded_traffic(dom), "launches_per_step": n / args.steps,
                        "avg_launch_us": round(avg_s * 1e6, 2), "flop_per_launch": flop / n,
                        "algorithmic_bytes_per_launch": byts / n}
        else:
            ach = byts / n / avg_s / 1e9
            roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": recorded_traffic(dom),
                        "launches_per_step": n / args.steps, "avg_launch_us": round(avg_s * 1e6, 2),
                        "bytes_per_launch": byts / n}
    sh.free()
    del sh

    # the other GPT-shaped shards: GPT-2 1.5B at tp=2 (both ranks: 13 and 12 heads) and the 8.3B
    # layer at tp=8 (rank 0; every rank has the same shapes)
    other = {}
    if not args.no_other_shards:
        for key, w, r in (("gpt2_1p5b_tp2_rank0", GPT2_1P5B, 0), ("gpt2_1p5b_tp2_rank1", GPT2_1P5B, 1),
                          ("gpt_8p3b_tp8_rank0", GPT_8P3B, 0)):
            o = LayerShard(bd, torch, w, r)
            m = o.measure(args.steps, args.warmup, events=events, cold=False)
            m.pop("_by_tag_raw", None)
            m.update(workload=w.name + f"_rank{r}", heads_per_rank=o.nh, head_dim=o.d, ffn_cols_per_rank=o.Fr)
            other[key] = m
            o.free()

    moe = None if args.no_moe else moe_grouped(bd, torch, args.steps, args.warmup)
    moe_l = None if args.no_moe else moe_layer(bd, torch, args.steps, args.warmup)
    oproj, oproj_flop = (None, 0.0) if args.no_attn_out else attn_out_proj(bd, torch, wl, rank, args.steps,
                                                                           args.warmup)

    ln = None if args.no_ln else residual_ln(bd, torch, wl, args.steps, args.warmup)
    f8 = None if args.no_fp8 else fp8_mlp(bd, torch, wl, args.steps, args.warmup)
    blas = blas_compare(torch, wl, rank, args.steps, args.warmup) if args.blas_compare else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, rank, args.cpu_seq)

    t, B, S, H, nh_all, F = wl.tp_size, wl.B, wl.S, wl.H, wl.n_heads, wl.F
    _, nh = bd.tp_shard_range(nh_all, t, rank)
    _, Fr = bd.tp_shard_range(F, t, rank)
    sites = head.get("gemm_call_sites") or {}
    out = {
        "metric": "TFLOPs/s and % of bf16 MFMA peak per TP-rank layer shard (fwd+bwd)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gpt3_175b_tp8_rank0_layer_shard_fwd_bwd", "B": B, "S": S, "H": H,
                   "n_heads": nh_all, "head_dim": wl.head_dim, "F": F, "tp_size": t, "rank": rank,
                   "heads_per_rank": nh, "ffn_cols_per_rank": Fr, "global_batch": B, "seq_len": S,
                   "parallelism": "tp8, rank 0's shard on one GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "gflop_per_step": round(flop_step / 1e9, 1),
        "ms_per_step_median": head["ms_per_step_median"], "ms_per_step_min": head["ms_per_step_min"],
        "ms_per_step_cold_median": head.get("ms_per_step_cold_median"),
        "ms_per_step_cold_min": head.get("ms_per_step_cold_min"),
        "tflops_cold_median": head.get("tflops_cold_median"),
        "wall_s_timed_region": head["wall_s_timed_region"],
        "ms_per_step_with_kernel_events": head.get("ms_per_step_with_kernel_events"),
        "ms_per_step_graph_replay": round(ms_graph, 4) if ms_graph else None,
        "tflops_graph_replay": round(flop_step / (ms_graph * 1e-3) / 1e12, 2) if ms_graph else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "gemm_call_sites": sites,
        "gemms_meeting_target": f"{sum(v['meets_target'] for v in sites.values())} of {len(sites)} at >= "
                                f"{GEMM_TARGET_FRAC:.2f} of peak" if sites else None,
        "kernels": head.get("kernels"),
        "other_shards": other or None,
        "moe_grouped_shard": moe,
        "moe_layer_shard": moe_l,
        "attn_out_proj_shard": oproj,
        "residual_layernorm": ln,
        "fp8_mlp": f8,
        "blas_compare": blas,
        # the step plus the attention output projection: the whole Megatron layer shard's GEMMs
        "tflops_layer_with_out_proj": round((flop_step + oproj_flop) / ((ms_step + oproj["ms"]) * 1e-3) / 1e12, 2)
        if oproj else None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
