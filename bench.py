#!/usr/bin/env python3
"""Benchmark of the GPTQ per-layer solve on one MI355X.

One step = one whole layer solve of the Llama-2-7B-shaped q_proj layer:
W 4096 x 4096 bf16, N = 262144 calibration tokens (128 x 2048) of bf16
activations, 4-bit, group 128, symmetric, no act-order, damp 0.01:

    S = 0; S += X^T X (all N tokens, one call); H, damping, U; column sweep
    over 32 lazy blocks; pack.

Inputs are synthetic (seeded generators with the layer's distributions) and
resident in HBM before timing starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GPTQ layer-solve ms & weight cols/s (4096×4096, N=262144); MFMA % peak"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hessian_bf16_4096x4096_N262144_counters.md")
HESSIAN_SRC = os.path.join(ROOT, "post_weight_quantization_07_amd", "csrc", "hessian.hip")
HESSIAN_KERNEL = "hessian_bf16_pipe_kernel+hessian_reduce_kernel"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="launch one device copy of this many MiB first (HBM counter calibration)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="time the oracle on this many tokens only (0: all N; the default is the whole layer)")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="time the oracle's sweep on this many rows only (0: all d_out)")
    ap.add_argument("--all-configs", metavar="PATH", default=None,
                    help="instead of the one-line result: time every layer of the five configurations and write "
                         "a markdown table to PATH")
    ap.add_argument("--all-configs-steps", type=int, default=3)
    ap.add_argument("--block", metavar="PATH", default=None,
                    help="quantize a Llama-7B-shaped transformer block layer by layer (true-sequential) and "
                         "write the per-stage times to PATH")
    ap.add_argument("--dequant", metavar="PATH", default=None,
                    help="time gptq_dequant_matmul on the layer shapes of configurations 3 and 5 and write a "
                         "markdown table to PATH")
    ap.add_argument("--shared", metavar="PATH", default=None,
                    help="time the layers that read one input (q/k/v, gate/up of configurations 2-3) solved "
                         "against one H and one U against separate solves; write a markdown table to PATH")
    return ap.parse_args()


def source_hash() -> str:
    with open(HESSIAN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the Hessian kernel from the committed counter
    summary, or None when it is missing or was taken on other kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    txt = open(COUNTERS_FILE).read()
    m = re.search(r"traffic_json:\s*(\{.*\})", txt)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != source_hash() or rec.get("kernel") != HESSIAN_KERNEL:
        return None
    return rec


def cpu_baseline(layer, W_host, args, x_chunks=None):
    """The oracle, untuned, on the same workload: by default the whole layer
    solve (all N tokens, all d_out rows); --cpu-sample-tokens / -rows bound it
    and scale the measured times up.  x_chunks: the activations as stored on
    the device (bf16 bit patterns, token chunks in order), or None to draw
    them again from the seeded generator."""
    import numpy as np

    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in info if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        blas = []
    threads = max([t for _, t in blas if t] or [os.cpu_count() or 1])
    n_s = layer.n_tokens if args.cpu_sample_tokens <= 0 else min(args.cpu_sample_tokens, layer.n_tokens)
    rows = layer.d_out if args.cpu_sample_rows <= 0 else min(args.cpu_sample_rows, layer.d_out)
    n_chunks = (n_s + synth.CHUNK_TOKENS - 1) // synth.CHUNK_TOKENS

    def chunks():
        # the stored bf16 values (exact in fp32), or the same values drawn again
        if x_chunks is not None:
            for c in range(n_chunks):
                yield synth.bf16_to_f32(x_chunks[c])
        else:
            sig = synth.channel_sigma(layer)
            for c in range(n_chunks):
                yield synth.activation_chunk(layer, c, sig)

    t0 = time.perf_counter()
    S, n = O.hessian_sum(chunks())
    t_h = time.perf_counter() - t0
    t0 = time.perf_counter()
    H = O.finalize_hessian(S, n)
    prep = O.prepare(H, layer.damp_percent, layer.desc_act)
    t_p = time.perf_counter() - t0
    t0 = time.perf_counter()
    sw = O.quantize_layer(W_host, prep.U, prep.perm, layer.bits, layer.group_size, layer.sym, layer.static_groups,
                          rows=np.arange(rows))
    t_q = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.pack(sw.codes, layer.bits)
    t_k = time.perf_counter() - t0
    total = t_h * (layer.n_tokens / n) + t_p + (t_q + t_k) * (layer.d_out / rows)
    full = n == layer.n_tokens and rows == layer.d_out
    if full:
        sample = (f"full N: the whole layer solve, X^T X over all {n} tokens, damping + order + explicit inverse + "
                  f"Cholesky of the {layer.d_in}x{layer.d_in} H, the blocked sweep of all {rows} rows, pack")
    else:
        sample = (f"X^T X on {n} of {layer.n_tokens} tokens (scaled x{layer.n_tokens / n:g}); full {layer.d_in}x"
                  f"{layer.d_in} damping+order+inverse+Cholesky; sweep and pack on {rows} of {layer.d_out} rows "
                  f"(scaled x{layer.d_out / rows:g})")
    return {
        "value": layer.d_in / total,
        "unit": "weight cols/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{sample}; numpy {np.__version__} fp64, BLAS {blas}",
        "est_total_s": total,
        "measured_s": t_h + t_p + t_q + t_k,
        "stages_s": {"hessian": t_h, "prepare": t_p, "quantize": t_q, "pack": t_k},
    }


def fp32_planes(d_in, n_tokens):
    """Whether the library accumulates an fp32 X of this shape as three bf16
    planes on the bf16 matrix cores (its rule: N d^2 >= 4e9 and d <= 8192)."""
    return d_in <= 8192 and float(n_tokens) * d_in * d_in >= 4e9


def stage_metrics(layer, st):
    """Algorithmic rates of the four stages and their fraction of the bound
    that applies: MFMA peak (bf16 or fp32) for the contractions, HBM for the
    sweep (approximated on the whole quantize stage) and the pack."""
    d_out, d_in, N = layer.d_out, layer.d_in, layer.n_tokens
    G = layer.group_size if layer.group_size > 0 else d_in
    f_h = float(N) * d_in * (d_in + 1)
    f_inv = 2.0 / 3.0 * d_in ** 3
    f_upd = float(d_out) * d_in * (d_in - 1)
    b_sweep = float(d_out) * d_in * (9 + 8.0 / G)
    b_pack = float(d_out) * d_in * (1 + layer.bits / 8.0)
    # fp32 X on the plane path: six bf16 part products per fp32-equivalent flop
    peak_h = (PEAK_BF16_TFLOPS if layer.x_dtype == "bf16" else
              PEAK_BF16_TFLOPS / 6.0 if fp32_planes(d_in, N) else PEAK_FP32_TFLOPS)

    def rate(work, ms, scale):
        return work / (ms * 1e-3) / scale
    h = rate(f_h, st["hessian"], 1e12)
    p_ = rate(f_inv, st["prepare"], 1e12)
    q = rate(f_upd, st["quantize"], 1e12)
    qb = rate(b_sweep, st["quantize"], 1e9)
    k = rate(b_pack, st["pack"], 1e9)
    return {
        "hessian": {"ms": st["hessian"], "TFLOP/s": h, "peak": peak_h, "frac": h / peak_h, "flops": f_h},
        "prepare": {"ms": st["prepare"], "TFLOP/s": p_, "peak": PEAK_FP32_TFLOPS, "frac": p_ / PEAK_FP32_TFLOPS,
                    "flops": f_inv},
        "quantize": {"ms": st["quantize"], "update TFLOP/s": q, "peak": PEAK_FP32_TFLOPS, "frac": q / PEAK_FP32_TFLOPS,
                     "flops": f_upd, "sweep GB/s": qb, "sweep frac of HBM": qb / PEAK_HBM_GBS, "sweep bytes": b_sweep},
        "pack": {"ms": st["pack"], "GB/s": k, "frac of HBM": k / PEAK_HBM_GBS, "bytes": b_pack},
    }


class LayerSolve:
    """Inputs resident in HBM, outputs and workspaces allocated once; step()
    runs one whole layer solve (zero S, accumulate all tokens in one call,
    prepare, quantize, pack) on the current stream.  With `members` (layers
    that read `layer`'s input), their weights are stacked and solved against
    one H and one U, as solve_layers_shared does."""

    def __init__(self, layer, copy_calib_mib=0, members=None, keep_host_x=False):
        import numpy as np
        import torch

        import post_weight_quantization_07_amd as G
        import synth
        self.G, self.layer, self.torch = G, layer, torch
        dev = torch.device("cuda:0")
        members = members or [layer]
        d_out, d_in, N = sum(L.d_out for L in members), layer.d_in, layer.n_tokens
        self.cfg = cfg = G.QuantizeConfig(**layer.quant_kwargs())
        self.W_host = np.vstack([synth.weight(L) for L in members]) if len(members) > 1 else synth.weight(layer)
        if layer.w_dtype == "bf16":
            self.W = torch.from_numpy(synth.bf16_bits(self.W_host).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            self.W = torch.from_numpy(self.W_host).to(dev)
        bf16 = layer.x_dtype == "bf16"
        self.X = torch.empty((N, d_in), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
        row = 0
        self.x_host = [] if keep_host_x else None
        for x in synth.activation_chunks_threaded(layer, workers=min(16, os.cpu_count() or 1), as_bf16_bits=bf16):
            t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(x)
            self.X[row:row + x.shape[0]].copy_(t)
            row += x.shape[0]
            if keep_host_x:
                self.x_host.append(x)
        assert row == N
        self.S = torch.empty((d_in, d_in), dtype=torch.float32, device=dev)
        self.U = torch.empty((d_in, d_in), dtype=torch.float32, device=dev)
        self.perm = torch.empty(d_in, dtype=torch.int32, device=dev)
        self.info = torch.empty(1, dtype=torch.int32, device=dev)
        u8 = torch.uint8
        self.ws_h = torch.empty(max(256, G.gptq_hessian_workspace_size(d_in, N, self.X.dtype)), dtype=u8, device=dev)
        self.ws_p = torch.empty(max(256, G.gptq_prepare_workspace_size(d_in)), dtype=u8, device=dev)
        self.ws_q = torch.empty(max(256, G.gptq_workspace_size(d_out, d_in, cfg)), dtype=u8, device=dev)
        ng = cfg.n_groups(d_in)
        self.out = {"codes": torch.empty((d_out, d_in), dtype=torch.uint8, device=dev),
                    "scales": torch.empty((ng, d_out), dtype=torch.float32, device=dev),
                    "zeros": torch.empty((ng, d_out), dtype=torch.int32, device=dev),
                    "g_idx": torch.empty(d_in, dtype=torch.int32, device=dev),
                    "row_loss": torch.empty(d_out, dtype=torch.float32, device=dev)}
        self.qweight = torch.empty((d_in * cfg.bits // 32, d_out), dtype=torch.int32, device=dev)
        if copy_calib_mib > 0:
            a = torch.ones((copy_calib_mib << 20) // 4, dtype=torch.float32, device=dev)
            b = torch.empty_like(a)
            b.copy_(a)
            torch.cuda.synchronize()
            del a, b
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    def step(self, record=False):
        G, ev, cfg = self.G, self.ev, self.cfg
        self.S.zero_()
        if record:
            ev[0].record()
        G.gptq_hessian_accumulate(self.S, self.X, ws=self.ws_h)
        if record:
            ev[1].record()
        G.gptq_prepare_hinv(self.S, self.layer.n_tokens, cfg, U=self.U, perm=self.perm, info=self.info, ws=self.ws_p,
                            check=False)
        if record:
            ev[2].record()
        G.gptq_quantize_layer(self.W, self.U, self.perm, cfg, want_q=False, want_loss=True, out=self.out,
                              ws=self.ws_q)
        if record:
            ev[3].record()
        G.gptq_pack(self.out["codes"], cfg.bits, qweight=self.qweight)
        if record:
            ev[4].record()

    def measure(self, steps, warmup):
        """Wall ms per step over exactly `steps` steps (synchronised on both
        sides), then the mean per-stage durations from HIP events."""
        import numpy as np
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        if int(self.info.item()) != 0:
            raise RuntimeError(f"prepare reported a failed pivot: info={int(self.info.item())}")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
        stage_ms = {"hessian": [], "prepare": [], "quantize": [], "pack": []}
        ev = self.ev
        for _ in range(steps):
            self.step(True)
            torch.cuda.synchronize()
            stage_ms["hessian"].append(ev[0].elapsed_time(ev[1]))
            stage_ms["prepare"].append(ev[1].elapsed_time(ev[2]))
            stage_ms["quantize"].append(ev[2].elapsed_time(ev[3]))
            stage_ms["pack"].append(ev[3].elapsed_time(ev[4]))
        codes_max = int(self.out["codes"].max().item())
        assert 0 <= codes_max <= (1 << self.cfg.bits) - 1
        return ms_per_step, {k: float(np.mean(v)) for k, v in stage_ms.items()}

    def phases(self, reps=3):
        """Per-phase launch times of `reps` more steps from the library's own
        HIP events (recorded around each launch on its stream); mean per step."""
        from post_weight_quantization_07_amd import _lib
        torch = self.torch
        torch.cuda.synchronize()
        _lib.phase_timing(True)
        try:
            for _ in range(reps):
                self.step()
            torch.cuda.synchronize()
            ph = _lib.phase_read()
        finally:
            _lib.phase_timing(False)
        return {k: (ms / reps, n // reps) for k, (ms, n) in ph.items()}


def update_gemm_flops(d_out, d_in, group_size, static_groups, group_launch=False):
    """Algorithmic flops of the trailing-update products the quantize stage
    launches as separate products, as (fp32 products, three-part products).
    Blocks are swept in pairs, pairs in groups of four (1024 columns) where
    the groups allow; the columns past each group take one product with all
    of the group's errors, on the bf16 matrix cores for groups of 1024
    columns (fp32 otherwise).  One sweep launch per group (group_launch;
    layers whose rows fit one workgroup per CU) runs the products inside a
    group in the sweep kernel; otherwise a later pair of a group is first
    brought up to date with the group's earlier pairs (an fp32 product), the
    second block of a pair inside its sweep kernel."""
    B = 128
    g = group_size if group_size > 0 else 0
    preset = static_groups or g == 0
    pair = preset or g <= B or g % (2 * B) == 0
    SB = 2 * B if pair else B
    grouped = pair and (preset or g <= 2 * B or g % (2 * B * 4) == 0)
    NU = 4 if grouped else 1
    GW = NU * SB
    f32, x3 = 0.0, 0.0
    for g0 in range(0, d_in, GW):
        for u in range(1, NU):
            j0 = g0 + u * SB
            if j0 >= d_in or group_launch:
                break
            f32 += 2.0 * d_out * min(SB, d_in - j0) * (j0 - g0)
        rest = d_in - g0 - GW
        if rest > 0:
            if GW == 1024:
                x3 += 2.0 * d_out * rest * GW
            else:
                f32 += 2.0 * d_out * rest * GW
    return f32, x3


def cross_block_flops(d_out, d_in):
    """Flops of every cross-block update of the lazy-batch sweep: each block's
    columns take the errors of all earlier columns (2 d_out flops a pair)."""
    B = 128
    return sum(2.0 * d_out * min(B, d_in - j0) * j0 for j0 in range(0, d_in, B))


def kernel_metrics(layer, ph):
    """Rates of the sweep kernel and of the trailing-update products from their
    own launch times: algorithmic bytes (sweep) or flops (update) over the
    summed launch time, with the fraction of HBM / fp32 MFMA peak.  The sweep
    kernel also runs the cross-block products the separate launches do not
    (inside a group, or the pair bring-up); their flops over the sweep time are
    reported beside its bytes."""
    d_out, d_in = layer.d_out, layer.d_in
    G = layer.group_size if layer.group_size > 0 else d_in
    sw_ms, sw_n = ph["sweep"]
    up_ms, up_n = ph["trailing_update"]
    n_blocks = -(-d_in // 128)
    group_launch = 0 < sw_n < n_blocks
    b_sweep = float(d_out) * d_in * (9 + 8.0 / G)
    f_f32, f_x3 = update_gemm_flops(d_out, d_in, layer.group_size, layer.static_groups, group_launch)
    f_up = f_f32 + f_x3
    f_in = cross_block_flops(d_out, d_in) - f_up
    out = {"phases_ms": {k: round(v[0], 4) for k, v in ph.items()},
           "phases_launches": {k: v[1] for k, v in ph.items()}}
    if sw_ms > 0:
        gbs = b_sweep / (sw_ms * 1e-3) / 1e9
        out["sweep"] = {"launches": sw_n, "blocks": n_blocks, "us_per_block": 1e3 * sw_ms / n_blocks,
                        "bytes": b_sweep, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
                        "in_kernel_product_flops": f_in,
                        "in_kernel_TFLOP/s": f_in / (sw_ms * 1e-3) / 1e12}
    if up_ms > 0:
        tf = f_up / (up_ms * 1e-3) / 1e12
        # fp32 products on the bf16 matrix cores: each operand split into three
        # bf16 parts, six part products a flop, so their ceiling is the bf16
        # dense peak over six (fp32-equivalent flops); the rest on the fp32
        # matrix cores.  The ceiling of the mix: its flops over the least time.
        peak_x3 = PEAK_BF16_TFLOPS / 6.0
        t_min = f_f32 / (PEAK_FP32_TFLOPS * 1e12) + f_x3 / (peak_x3 * 1e12)
        peak = f_up / t_min / 1e12
        how = ("bf16 matrix cores, three-part split, six products" if f_f32 == 0 else
               "fp32 matrix cores" if f_x3 == 0 else
               f"fp32 matrix cores ({f_f32 / f_up:.0%} of flops), bf16 three-part split (the rest)")
        out["trailing_update"] = {"launches": up_n, "ms": up_ms, "flops": f_up, "flops_three_part": f_x3,
                                  "TFLOP/s": tf, "on": how, "peak_TFLOP/s": peak, "frac_peak": tf / peak}
    return out


def all_configs(args):
    """Every layer of the five configurations: ms per solve, weight columns/s
    and each stage's rate with its fraction of the bound; a markdown table."""
    import torch

    import synth
    lines = ["| cfg | layer | d_out x d_in | N | x | bits/G | ms per solve | weight cols/s | accumulate "
             "TFLOP/s (% peak) | prepare TFLOP/s (% of fp32 peak) | quantize: update TFLOP/s (% of fp32 peak), sweep "
             "GB/s (% HBM) | sweep kernel: us per block, GB/s (% HBM) | update products: TFLOP/s (% of their ceiling) "
             "| pack GB/s |",
             "|---|---|---|---:|---|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for c in (1, 2, 3, 4, 5):
        for layer in synth.config_layers(c):
            print(f"[all-configs] cfg{c} {layer.name} {layer.d_out}x{layer.d_in} N={layer.n_tokens}", flush=True)
            ls = LayerSolve(layer)
            ms, st = ls.measure(args.all_configs_steps, 1)
            m = stage_metrics(layer, st)
            km = kernel_metrics(layer, ls.phases(reps=1))
            sw, up = km.get("sweep", {}), km.get("trailing_update", {})
            g = layer.group_size
            lines.append(
                f"| {c} | {layer.name} | {layer.d_out}x{layer.d_in} | {layer.n_tokens} | {layer.x_dtype} | "
                f"b{layer.bits}/{g}{' act-order' if layer.desc_act else ''}{' static' if layer.static_groups else ''} | "
                f"{ms:.2f} | {layer.d_in / (ms * 1e-3):,.0f} | "
                f"{m['hessian']['TFLOP/s']:.0f} ({100 * m['hessian']['frac']:.1f}%) | "
                f"{m['prepare']['TFLOP/s']:.1f} ({100 * m['prepare']['frac']:.1f}%) | "
                f"{m['quantize']['update TFLOP/s']:.1f} ({100 * m['quantize']['frac']:.1f}%), "
                f"{m['quantize']['sweep GB/s']:.0f} ({100 * m['quantize']['sweep frac of HBM']:.1f}%) | "
                f"{sw.get('us_per_block', 0):.1f}, {sw.get('GB/s', 0):.0f} ({100 * sw.get('frac_hbm', 0):.1f}%) | " +
                (f"{up['TFLOP/s']:.1f} ({100 * up['frac_peak']:.1f}% of {up['peak_TFLOP/s']:.0f}) | " if up else
                 "— | ") +
                f"{m['pack']['GB/s']:.0f} |")
            del ls
            torch.cuda.empty_cache()
    text = "\n".join(lines) + "\n"
    with open(args.all_configs, "w") as f:
        f.write(text)
    print(text, flush=True)


def shared_groups_table(args):
    """Layers that read one input (q/k/v, gate/up) solved against one H and one
    U, against solving each on its own from the same input; a markdown table."""
    import torch

    import synth
    lines = ["| cfg | group | layers | N | separate: ms (sum of solves) | shared: ms | speed-up | "
             "shared weight cols/s |", "|---|---|---|---:|---:|---:|---:|---:|"]
    for c in (2, 3):
        for name, members in synth.shared_groups(c):
            L0 = members[0]
            desc = " + ".join(f"{L.name} {L.d_out}x{L.d_in}" for L in members)
            print(f"[shared] cfg{c} {name}: {desc} N={L0.n_tokens}", flush=True)
            sep = 0.0
            for L in members:
                ls = LayerSolve(L)
                ms, _ = ls.measure(args.all_configs_steps, 1)
                sep += ms
                del ls
                torch.cuda.empty_cache()
            ls = LayerSolve(L0, members=members)
            ms_sh, _ = ls.measure(args.all_configs_steps, 1)
            del ls
            torch.cuda.empty_cache()
            cols = len(members) * L0.d_in
            lines.append(f"| {c} | {name} | {desc} | {L0.n_tokens} | {sep:.2f} | {ms_sh:.2f} | {sep / ms_sh:.2f}x | "
                         f"{cols / (ms_sh * 1e-3):,.0f} |")
    text = "\n".join(lines) + "\n"
    with open(args.shared, "w") as f:
        f.write(text)
    print(text, flush=True)


def dequant_table(args):
    """gptq_dequant_matmul on the layer shapes of configurations 3 and 5:
    microseconds per call and algorithmic bytes (packed weights, scales, zeros,
    g_idx, x, y) per second against HBM; a markdown table."""
    import numpy as np
    import torch

    import post_weight_quantization_07_amd as G
    dev = torch.device("cuda:0")
    lines = ["| d_out x d_in | bits / G | g_idx | tokens m | us per call | GB/s | % of 8 TB/s |",
             "|---|---|---|---:|---:|---:|---:|"]
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008), (8192, 8192), (28672, 8192), (8192, 28672)]
    cases = [(4, 128, False), (3, 32, True), (4, 128, True)]
    act_shapes = {(3, 32): ((4096, 4096), (8192, 8192)), (4, 128): ((4096, 4096), (28672, 8192))}
    gen = torch.Generator(device="cpu").manual_seed(0)
    for d_out, d_in in shapes:
        for bits, group, act in cases:
            if act and (d_out, d_in) not in act_shapes[(bits, group)]:
                continue
            ng = -(-d_in // group)
            codes = torch.randint(0, 1 << bits, (d_out, d_in), dtype=torch.uint8, generator=gen).to(dev)
            qweight = G.gptq_pack(codes, bits)
            scales = (torch.rand((ng, d_out), generator=gen) * 0.01 + 0.001).to(dev)
            zeros = torch.randint(0, 1 << bits, (ng, d_out), dtype=torch.int32, generator=gen).to(dev)
            if act:  # act-order dynamic groups: group of column k = sweep position // G
                perm = torch.randperm(d_in, generator=gen)
                g_idx = torch.empty(d_in, dtype=torch.int32)
                g_idx[perm] = torch.arange(d_in, dtype=torch.int32) // group
                g_idx = g_idx.to(dev)
            else:
                g_idx = (torch.arange(d_in, dtype=torch.int32) // group).to(dev)
            # act-order layers: as stored, and put in group order once by
            # gptq_dequant_order (the timed call then gathers x and runs the
            # product on the reordered codes)
            modes = [False, True] if act else [False]
            if act:
                q_ord, g_ord, order = G.gptq_dequant_order(qweight, g_idx, bits)
            for ordered in modes:
                for m in (1, 8, 16):
                    x = torch.randn((m, d_in), generator=gen).to(torch.bfloat16).to(dev)
                    y = torch.empty((m, d_out), dtype=torch.float32, device=dev)
                    if ordered:
                        ws = torch.empty(G.gptq_dequant_ordered_workspace_size(m, d_in, d_out), dtype=torch.uint8,
                                         device=dev)
                        call = lambda: G.gptq_dequant_matmul_ordered(x, q_ord, scales, zeros, g_ord, order, bits,
                                                                     y=y, ws=ws)
                    else:
                        ws = torch.empty(max(256, G.gptq_dequant_workspace_size(m, d_in, d_out)),
                                         dtype=torch.uint8, device=dev)
                        call = lambda: G.gptq_dequant_matmul(x, qweight, scales, zeros, g_idx, bits, y=y, ws=ws)
                    for _ in range(5):
                        call()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    reps = 50
                    torch.cuda.synchronize()
                    e0.record()
                    for _ in range(reps):
                        call()
                    e1.record()
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) * 1e3 / reps
                    nbytes = d_out * d_in * bits / 8 + ng * d_out * 8 + d_in * 4 + m * d_in * 2 + m * d_out * 4
                    gbs = nbytes / (us * 1e-6) / 1e9
                    kind = ("act-order, group order" if ordered else "act-order") if act else "k // G"
                    lines.append(f"| {d_out}x{d_in} | {bits} / {group} | {kind} | {m} | "
                                 f"{us:.1f} | {gbs:.0f} | {100 * gbs / (PEAK_HBM_GBS):.1f}% |")
                    print(lines[-1], flush=True)
            if act:
                del q_ord, g_ord, order
            del codes, qweight, scales, zeros, g_idx
            torch.cuda.empty_cache()
    text = "\n".join(lines) + "\n"
    with open(args.dequant, "w") as f:
        f.write(text)
    print(text, flush=True)


def block_table(args):
    """Layer-sequential quantization of a Llama-7B-shaped block (k/v/q, o,
    up/gate, down): per-stage times of the driver's forward pieces and of the
    group solves; a markdown table."""
    import numpy as np
    import torch

    import post_weight_quantization_07_amd as G
    import synth
    from post_weight_quantization_07_amd.block import Block, quantize_block
    shape = synth.BLOCKS["llama7b"]
    dev = torch.device("cuda:0")
    print(f"[block] generating {shape.n_tokens} tokens x {shape.d_model}", flush=True)
    x0 = torch.from_numpy(synth.block_input(shape)).to(dev)
    Wh = {n: torch.from_numpy(synth.weight(synth.block_linear_layer(shape, n))) for n in synth.BLOCK_LINEARS}
    cfg = G.QuantizeConfig(**shape.quant_kwargs())
    runs = []
    for r in range(2):  # the first run warms up
        blk = Block(shape.d_model, shape.n_heads, shape.d_ff, {n: w.to(dev) for n, w in Wh.items()})
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = quantize_block(blk, x0, shape.n_seq, shape.seq_len, cfg, timed=True)
        torch.cuda.synchronize()
        runs.append(((time.perf_counter() - t0) * 1e3, res.ms))
        print(f"[block] run {r}: {runs[-1][0]:.1f} ms", flush=True)
        del blk, res
        torch.cuda.empty_cache()
    total, ms = runs[-1]
    cols = sum(synth.block_linear_layer(shape, n).d_in for n in synth.BLOCK_LINEARS)
    solve_ms = sum(v for k, v in ms.items() if k.startswith("solve"))
    lines = [f"| stage | ms |", "|---|---:|"]
    for k in sorted(ms, key=lambda t: (t.split(" ")[0] != "forward", t)):
        lines.append(f"| {k} | {ms[k]:.2f} |")
    lines.append(f"| all solves (accumulate, prepare, quantize, pack of the four groups) | {solve_ms:.2f} |")
    lines.append(f"| whole block, wall clock | {total:.2f} |")
    lines.append(f"| weight columns/s over the block's seven layers (solves only) | {cols / (solve_ms * 1e-3):,.0f} |")
    text = "\n".join(lines) + "\n"
    with open(args.block, "w") as f:
        f.write(text)
    print(text, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the layer solve is measured on a single "
              "MI355X; multi-GPU sharding is described, not run.", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.all_configs:
        all_configs(args)
        return
    if args.shared:
        shared_groups_table(args)
        return
    if args.dequant:
        dequant_table(args)
        return
    if args.block:
        block_table(args)
        return
    layer = synth.config_layers(3)[0]
    d_out, d_in, N = layer.d_out, layer.d_in, layer.n_tokens
    t_setup = time.perf_counter()
    ls = LayerSolve(layer, args.copy_calib_mib, keep_host_x=not args.no_cpu_baseline)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    ms_per_step, st = ls.measure(args.steps, args.warmup)
    cfg = ls.cfg
    m = stage_metrics(layer, st)
    kern = kernel_metrics(layer, ls.phases())
    achieved = m["hessian"]["TFLOP/s"]
    rec = recorded_traffic()
    roofline = {"kernel": "gptq_hessian_accumulate = " + HESSIAN_KERNEL + " (S += X^T X)", "bound": "mfma",
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": (rec["bytes_per_launch"] if rec else None),
                "algorithmic_flops_per_launch": m["hessian"]["flops"], "launch_ms": st["hessian"]}

    result = {
        "metric": METRIC,
        "value": d_in / (ms_per_step * 1e-3),
        "unit": "weight cols/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gptq_layer_solve", "layer": "q_proj (Llama-2-7B shape)", "d_out": d_out,
                   "d_in": d_in, "n_tokens": N, "x_dtype": "bf16", "w_dtype": "bf16", "bits": cfg.bits,
                   "group_size": cfg.group_size, "sym": cfg.sym, "desc_act": cfg.desc_act,
                   "static_groups": cfg.static_groups, "damp_percent": cfg.damp_percent, "block_size": 128},
        "stages_ms": st,
        "stages": m,
        "kernels": kern,
        "roofline": roofline,
        "setup_s": t_setup,
    }
    if not args.no_cpu_baseline:
        x_host, W_host = ls.x_host, ls.W_host
        del ls
        torch.cuda.empty_cache()
        cb = cpu_baseline(layer, W_host, args, x_host)
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        result["cpu_baseline"]["est_total_s"] = cb["est_total_s"]
        result["cpu_baseline"]["measured_s"] = cb["measured_s"]
        result["cpu_baseline"]["stages_s"] = cb["stages_s"]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
