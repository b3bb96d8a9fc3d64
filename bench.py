#!/usr/bin/env python3
"""Benchmark of the fused QK-RMSNorm + 3D M-RoPE joint text+image attention
on one MI355X.

One step = one full pass of the path over one batch: the prologue pass
(rotary table + K') and the attend stage (the attention kernel, plus the
small merge kernel of the query tiles split across key ranges), i.e. one
``mrope_attn_fwd`` call, on inputs already resident in HBM. Default workload: the 1024px shape
(B=1, H=32, head_dim=128, 512 text + 64x64 image tokens = 4608 tokens).

Prints one JSON line. ``value`` is algorithmic TFLOP/s of the whole step
(4*H*D*sum_b n_b^2 over real tokens), ``roofline`` the attend stage's own
rate (HIP events around it on its stream) against the bf16 dense MFMA peak, and ``cpu_baseline`` the fp64 oracle timed on the host on
the same workload (with the GPU output checked against it).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused QK-norm+M-RoPE attention TFLOP/s & % bf16 MFMA peak, 4608 tok"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "diffusion_transformer_image_head_amd", "csrc")


# sources the forward attention's kernels and launches are built from
FORWARD_SOURCES = ("attn_bf16.hpp", "mra_common.hpp", "mrope_attn.hip", "prologue.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(config: str):
    """HBM bytes per attend stage from the committed rocprofv3 counter
    summary (``key: value`` lines), when it was taken on the current kernel
    sources; else None."""
    path = os.path.join(PROFILES, f"attn_bf16_{config}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return int(float(rec["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def calibrate_copy(nbytes: int = 256 << 20, reps: int = 5):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of the attention kernel."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_per_copy": nbytes, "copies": reps}), flush=True)


def cpu_baseline(w, gpu_out):
    """fp64 oracle on the host over the whole workload; also the parity check."""
    import numpy as np
    from oracle.reference import oracle_fwd
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    t0 = time.perf_counter()
    ref, _ = oracle_fwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens,
                        text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps)
    dt = time.perf_counter() - t0
    d = gpu_out - ref
    rel = float(np.sqrt((d * d).sum() / (ref * ref).sum()))
    return {
        "value": round(w.flops() / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
        "kind": "oracle", "seconds": round(dt, 3),
        "sample": f"the whole workload ({w.shape[2]} heads, all {w.shape[1]} query rows), fp64 NumPy",
    }, {"max_abs": float(np.abs(d).max()), "rel_rms": rel}


def bench_cfg(args):
    """One guided sampling step at 1024px: the conditional pass (512 text slots
    + 64x64 image) and the unconditional pass (the 4096 image tokens alone)
    as one grouped call, against the same two problems as two plain calls."""
    import numpy as np
    import torch
    from diffusion_transformer_image_head_amd.binding import lib, mrope_attn, mrope_attn_group
    from diffusion_transformer_image_head_amd.workloads import config_workload, make_workload

    lib()
    cond = config_workload("1024px")
    unc = make_workload(1, 32, 128, (16, 24, 24), 0, 64, 64, dtype="bf16", seed=21)
    unc.pos = np.ascontiguousarray(cond.pos[:, cond.text_pad:])
    dev = torch.device("cuda:0")
    probs = []
    for w in (cond, unc):
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
        probs.append(dict(q=t(w.q).to(torch.bfloat16), k=t(w.k).to(torch.bfloat16),
                          v=t(w.v).to(torch.bfloat16), pos=t(w.pos), gamma_q=t(w.gamma_q),
                          gamma_k=t(w.gamma_k), text_pad=w.text_pad, section=w.section))
    for p in probs:
        p["out"] = torch.empty_like(p["q"])
    ws = torch.empty(1 << 27, dtype=torch.uint8, device=dev)
    ws2 = torch.empty(1 << 27, dtype=torch.uint8, device=dev)

    def grouped():
        mrope_attn_group(probs, workspace=ws)

    def separate():
        for p, w in zip(probs, (ws, ws2)):
            mrope_attn(p["q"], p["k"], p["v"], p["pos"], p["gamma_q"], p["gamma_k"],
                       text_pad=p["text_pad"], section=p["section"], out=p["out"], workspace=w)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_sep = timed(separate)
    ms = timed(grouped)
    flops = cond.flops() + unc.flops()
    value = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC + " (guided step: cond + uncond)", "value": round(value, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, U[0.5,1.5) gammas; no dataset or weights)",
        "config": {"workload": "cfg1024: 1024px cond (B=1 H=32 D=128, 512 text + 64x64 image) "
                               "+ image-only uncond (4096 tokens), one grouped call"},
        "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "whole grouped call (prologues + attention + merge)"},
        "separate_calls": {"ms_per_step": round(ms_sep, 5),
                           "value": round(flops / (ms_sep * 1e-3) / 1e12, 3)},
    }
    if not args.no_cpu_baseline:
        base, par = cpu_baseline(cond, probs[0]["out"].float().cpu().numpy().astype(np.float64))
        rec["cpu_baseline"] = dict(base, sample="the conditional pass only (" + base["sample"] + ")")
        rec["parity"] = par
    print(json.dumps(rec), flush=True)


def bench_qkv(args):
    """The layer's attention input path at a configuration's shape: x [B*S,
    hidden = H*D] bf16 through the fp8 e4m3 fused qkv weight with the
    norm/rotation epilogue (one call), then the attention on those operands.
    value = the projection's FLOP rate (2 * tokens * hidden * 3 H D)."""
    import numpy as np
    import torch
    from diffusion_transformer_image_head_amd.binding import lib, mrope_attn, mrope_qkv_proj
    from diffusion_transformer_image_head_amd.workloads import CONFIGS, make_qkv_workload

    lib()
    c = CONFIGS[args.config]
    h, d = c["heads"], c["head_dim"]
    w = make_qkv_workload(c["batch"], h, d, c["section"], c["text_pad"], c["grid_h"], c["grid_w"],
                          h * d, seed=c["seed"])
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    x = t(w.x).to(torch.bfloat16)
    w8, wsc, pos, gq, gk = t(w.w8), t(w.w_scale), t(w.pos), t(w.gamma_q), t(w.gamma_k)
    outs = tuple(torch.empty((w.x.shape[0], h, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=dev)
    b, s = w.batch, w.seq
    q, k, v = (o.view(b, s, h, d) for o in outs)
    att_out = torch.empty_like(q)
    att_ws = torch.empty(1 << 26, dtype=torch.uint8, device=dev)

    def proj():
        mrope_qkv_proj(x, w8, wsc, pos, gq, gk, heads=h, section=w.section, out=outs, workspace=ws)

    def attend():
        mrope_attn(q, k, v, None, None, None, text_pad=w.text_pad, kprologue="none", out=att_out,
                   workspace=att_ws)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_p = timed(proj)
    ms_a = timed(attend)
    value = w.flops() / (ms_p * 1e-3) / 1e12
    att_flops = 4 * h * d * s * s * b
    rec = {
        "metric": "fp8 QKV projection + norm/rotation epilogue TFLOP/s (bf16 matrix cores)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_p, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) x, N(0,1/hidden) weight quantized to e4m3 per row)",
        "config": {"workload": f"{args.config} qkv: tokens={b * s} hidden={h * d} out={3 * h * d}"},
        "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "rope_table_kernel + qkv_proj_kernel"},
        "attention_on_operands": {"ms": round(ms_a, 5),
                                  "TFLOP/s": round(att_flops / (ms_a * 1e-3) / 1e12, 3)},
    }
    print(json.dumps(rec), flush=True)


def bench_bwd(args):
    """Backward pass on a configuration: the forward runs once (untimed) for
    out and lse, then `steps` backward calls are timed. FLOPs: the usual 2.5x
    the forward's (dV, dP, dQ, dK and the recomputed S: five S^2 D products
    against the forward's two)."""
    import numpy as np
    import torch
    from diffusion_transformer_image_head_amd.binding import lib, mrope_attn, mrope_attn_bwd
    from diffusion_transformer_image_head_amd.workloads import config_workload, round_to_bf16

    lib()
    w = config_workload(args.config)
    dev = torch.device("cuda:0")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    q, k, v = (t(x).to(torch.bfloat16) for x in (w.q, w.k, w.v))
    pos, gq, gk = t(w.pos), t(w.gamma_q), t(w.gamma_k)
    sl = None if w.seq_lens is None else t(w.seq_lens)
    kw = dict(text_pad=w.text_pad, section=w.section)
    out, lse = mrope_attn(q, k, v, pos, gq, gk, sl, return_lse=True, **kw)
    do = t(round_to_bf16(np.random.default_rng(3).standard_normal(w.q.shape).astype(np.float32))).to(torch.bfloat16)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(1 << 28, dtype=torch.uint8, device=dev)

    def step():
        mrope_attn_bwd(q, k, v, pos, gq, gk, sl, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    flops = 2.5 * w.flops()
    value = flops / (ms * 1e-3) / 1e12
    bb, s, h, d = w.shape
    rec = {
        "metric": "fused QK-norm+M-RoPE attention backward TFLOP/s (2.5x forward FLOPs)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v/dO, U[0.5,1.5) gammas; no dataset or weights)",
        "config": {"workload": f"{args.config} backward: B={bb} H={h} head_dim={d} tokens={s}"},
        "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "whole backward call (prologues, delta, dk/dv, dq, dgamma)"},
    }
    print(json.dumps(rec), flush=True)


def bench_packed(args):
    """A configuration's prompts packed back to back (cu_seqlens; each
    prompt's true-length text tokens then its image) instead of padded:
    `steps` calls of the packed forward (prologue + attention), or with
    --backward of the packed backward after one untimed forward. FLOPs are the
    sequences' own: 4 H D sum(n_b^2), times 2.5 for the backward."""
    import numpy as np
    import torch
    from diffusion_transformer_image_head_amd.binding import lib, mrope_attn_bwd_varlen, mrope_attn_varlen
    from diffusion_transformer_image_head_amd.workloads import CONFIGS, make_varlen_workload, round_to_bf16

    lib()
    c = CONFIGS[args.config]
    lens = c["text_lens"] if c["text_lens"] is not None else (c["text_pad"],) * c["batch"]
    w = make_varlen_workload(c["heads"], c["head_dim"], c["section"], text_lens=lens,
                             grids=[(c["grid_h"], c["grid_w"])] * c["batch"], sigma=c["sigma"],
                             seed=c["seed"])
    dev = torch.device("cuda:0")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    q, k, v = (t(x).to(torch.bfloat16) for x in (w.q, w.k, w.v))
    pos, gq, gk = t(w.pos), t(w.gamma_q), t(w.gamma_k)
    cu = t(w.cu_seqlens.astype(np.int32))
    ms_len = w.max_seqlen
    out = torch.empty_like(q)
    ws = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
    _, lse = mrope_attn_varlen(q, k, v, pos, gq, gk, cu, ms_len, section=w.section, return_lse=True,
                               out=out, workspace=ws)
    if args.backward:
        do = t(round_to_bf16(np.random.default_rng(3).standard_normal(w.q.shape).astype(np.float32)))
        do = do.to(torch.bfloat16)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def step():
            mrope_attn_bwd_varlen(q, k, v, pos, gq, gk, cu, ms_len, out, lse, do, section=w.section,
                                  dq=dq, dk=dk, dv=dv, workspace=ws)
    else:
        def step():
            mrope_attn_varlen(q, k, v, pos, gq, gk, cu, ms_len, section=w.section, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    mult = 2.5 if args.backward else 1.0
    value = mult * w.flops() / (ms * 1e-3) / 1e12
    what = "backward" if args.backward else "forward"
    rec = {
        "metric": f"fused QK-norm+M-RoPE attention {what} TFLOP/s, packed sequences"
                  + (" (2.5x forward FLOPs)" if args.backward else ""),
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v/dO, U[0.5,1.5) gammas; no dataset or weights)",
        "config": {"workload": f"{args.config} packed {what}: {len(lens)} sequences, "
                               f"{w.q.shape[0]} tokens, H={c['heads']} head_dim={c['head_dim']}",
                   "cu_seqlens": [int(x) for x in w.cu_seqlens]},
        "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": f"whole packed {what} call"},
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="1024px",
                    choices=["512px", "1024px", "ragged", "long", "h36", "2048px", "cfg1024", "h4"],
                    help="cfg1024: one guided step, the 1024px conditional pass and its "
                         "image-only unconditional pass in one grouped call")
    ap.add_argument("--kprologue", default="auto", choices=["auto", "prepass", "fused"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--qkv", action="store_true",
                    help="time the fp8 QKV projection with the norm/rotation epilogue, then the "
                         "attention on its operands (kprologue none)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dq, dk, dv, dgammas) instead of the forward")
    ap.add_argument("--packed", action="store_true",
                    help="pack the configuration's prompts back to back (cu_seqlens) and time the "
                         "packed forward, or with --backward the packed backward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain copy of known size (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(heads/batch shard with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    if args.config == "cfg1024":
        bench_cfg(args)
        return
    if args.packed:
        bench_packed(args)
        return
    if args.backward:
        bench_bwd(args)
        return
    if args.qkv:
        bench_qkv(args)
        return

    import numpy as np
    import torch
    from diffusion_transformer_image_head_amd.binding import lib, prepared_call
    from diffusion_transformer_image_head_amd.workloads import config_workload

    lib()  # fail loudly without the HIP library
    dev = torch.device("cuda:0")
    w = config_workload(args.config)
    b, s, h, d = w.shape
    q = torch.from_numpy(w.q).to(dev).to(torch.bfloat16)
    k = torch.from_numpy(w.k).to(dev).to(torch.bfloat16)
    v = torch.from_numpy(w.v).to(dev).to(torch.bfloat16)
    pos = torch.from_numpy(w.pos).to(dev)
    gq = torch.from_numpy(w.gamma_q).to(dev)
    gk = torch.from_numpy(w.gamma_k).to(dev)
    sl = None if w.seq_lens is None else torch.from_numpy(w.seq_lens).to(dev)
    prepare, attend, out = prepared_call(q, k, v, pos, gq, gk, sl, text_pad=w.text_pad,
                                         section=w.section, kprologue=args.kprologue)

    for _ in range(args.warmup):
        prepare()
        attend()
    torch.cuda.synchronize()

    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        prepare()
        mids[i].record()
        attend()
        ends[i].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    attn_ms = float(np.mean([m.elapsed_time(e) for m, e in zip(mids, ends)]))

    flops = w.flops()
    ms_step = total_ms / args.steps
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, U[0.5,1.5) gammas; no dataset or weights)",
        "config": {"workload": f"{args.config}: B={b} H={h} head_dim={d} tokens={s} "
                               f"(text_pad={w.text_pad} + {w.grid[0]}x{w.grid[1]} image)",
                   "batch": b, "heads": h, "head_dim": d, "seq_len": s,
                   "section": list(w.section), "kprologue": args.kprologue,
                   "text_lens": None if w.seq_lens is None else [int(x) for x in w.seq_lens]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(args.config),
                     "kernel_ms": round(attn_ms, 5), "kernel": "attn_bf16_kernel + split_merge_kernel"},
        "frac_of_peak_whole_step": round(value / PEAK_BF16_TFLOPS, 4),
        "wall_s": round(wall, 4),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        got = out.float().cpu().numpy().astype(np.float64)
        base, parity = cpu_baseline(w, got)
        rec["cpu_baseline"] = base
        rec["parity"] = dict(parity, bars={"max_abs": 2e-2, "rel_rms": 5e-3},
                             ok=bool(parity["max_abs"] <= 2e-2 and parity["rel_rms"] <= 5e-3))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
