#!/usr/bin/env python3
"""Benchmark of the fused QK-RMSNorm + 3D M-RoPE joint text+image attention
on one MI355X.

One step = one full pass of the path over one batch: the prologue pass
(rotary table + K') and the attend stage (the attention kernel, plus the
small merge kernel of the query tiles split across key ranges), i.e. one
``mrope_attn_fwd`` call, on inputs already resident in HBM. Default workload:
the 1024px shape (B=1, H=32, head_dim=128, 512 text + 64x64 image tokens =
4608 tokens).

Timing protocol. Before the counted warm-up, a declared time-based pre-warm
runs back-to-back steps for ``--prewarm-s`` seconds (the engine clock of a
GPU that was idle ramps up over the first few hundred milliseconds of load;
the pre-warm and its length are reported as ``prewarm``). Then ``--warmup``
untimed steps, then exactly ``--steps`` timed steps launched back to back on
the stream the kernels run on, bracketed by synchronisation and by one HIP
event at each end of the region: an event recorded between two kernels holds
the next launch for a few microseconds, so none is recorded inside it.

Prints one JSON line. ``value`` is algorithmic TFLOP/s of the whole timed
region (4*H*D*sum_b n_b^2 over real tokens, times the steps, over the events
around all of them). ``roofline`` is the attend stage's rate at its mean time
over ``--steps`` attend-stage calls launched back to back after the timed
region, against the bf16 dense MFMA peak. Then ``--steps`` more steps with an
event after every stage give the per-step distributions (``attend_ms``,
``step_ms``: median, min / p90 / max, first- and last-quarter medians; these
include the events' own gaps). ``cpu_baseline`` is the fp64 oracle timed on
the host on the same workload (with the GPU output checked against it).
``extras`` carries the grouped guided step, the backward and the fp8
projection at the same shape, each timed after the headline region with its
own warm-up, the same way (rates from back-to-back calls, per-call event
medians beside them).

Runtime setting. Unless the environment already sets it, the process asks the
HIP runtime to keep kernel arguments in device memory
(``HIP_FORCE_DEV_KERNARG=1``, read when the runtime initialises, so it is set
before torch is imported). Back-to-back launches then start about 3 us
sooner; the kernels and their results are the same either way. The setting
in force is reported as ``runtime_env``.
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
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

METRIC = "fused QK-norm+M-RoPE attention TFLOP/s & % bf16 MFMA peak, 4608 tok"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "diffusion_transformer_image_head_amd", "csrc")
DATA = "synthetic (seeded N(0,1) q/k/v, U[0.5,1.5) gammas; no dataset or weights)"


# sources the forward attention's kernels and launches are built from
# Kernel sources each profiled path is built from (host files included: they
# choose the launch configuration).
SOURCES = {
    "forward": ("attn_bf16.hpp", "mra_common.hpp", "mrope_attn.hip", "prologue.hpp"),
    "backward": ("attn_bwd.hpp", "bwd_host.hpp", "attn_bf16.hpp", "mra_common.hpp", "mrope_attn.hip",
                 "prologue.hpp"),
    "qkv": ("qkv_proj.hpp", "qkv_host.hpp", "attn_bf16.hpp", "mra_common.hpp", "mrope_attn.hip",
            "prologue.hpp"),
}
FORWARD_SOURCES = SOURCES["forward"]


def kernel_source_hash(path: str = "forward") -> str:
    h = hashlib.sha256()
    for name in SOURCES[path]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def profile_record(name: str) -> dict:
    """``key: value`` lines of a committed rocprofv3 summary, or {}."""
    path = os.path.join(PROFILES, name)
    rec = {}
    if not os.path.exists(path):
        return rec
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    return rec


def traffic_from_profile(config: str):
    """HBM bytes per attend stage from the committed rocprofv3 counter
    summary, when it was taken on the current kernel sources; else None."""
    rec = profile_record(f"attn_bf16_{config}_hbm_traffic.txt")
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return int(float(rec["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def profiles_status(config: str) -> dict:
    """For each committed forward profile of this config: whether it was
    taken on the current kernel sources (its kernel_source_hash), and the
    matrix-core occupancy when the counter profile is current."""
    cur = kernel_source_hash()
    out = {}
    for kind in ("kernel_trace", "hbm_traffic", "mfma_counters"):
        rec = profile_record(f"attn_bf16_{config}_{kind}.txt")
        if rec:
            out[kind] = "current" if rec.get("kernel_source_hash") == cur else "stale"
    rec = profile_record(f"attn_bf16_{config}_mfma_counters.txt")
    if rec.get("kernel_source_hash") == cur and "mfma_busy_frac" in rec:
        out["mfma_busy_frac"] = float(rec["mfma_busy_frac"])
    return out


def path_profile_status(name: str, path: str) -> str:
    """'current' when the committed summary `name` was taken on the current
    sources of `path` (backward or qkv), 'stale' otherwise, 'absent'."""
    rec = profile_record(name)
    if not rec:
        return "absent"
    return "current" if rec.get("kernel_source_hash") == kernel_source_hash(path) else "stale"


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


# ---- timing -----------------------------------------------------------------

def summarize(ms) -> dict:
    """Median, mean, min, p90, max and first/last-quarter medians (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    q = max(1, len(a) // 4)
    r = lambda x: round(float(x), 5)  # noqa: E731
    return {"median": r(np.median(a)), "mean": r(a.mean()), "min": r(a.min()),
            "p90": r(np.percentile(a, 90)), "max": r(a.max()),
            "first_quarter_median": r(np.median(a[:q])), "last_quarter_median": r(np.median(a[-q:]))}


def prewarm(stages, seconds: float) -> dict:
    """Back-to-back calls for at least `seconds` of wall time (synchronising
    every 10 calls), so the timed region does not start on an idle clock."""
    import torch
    if seconds <= 0:
        return {"seconds": 0.0, "calls": 0}
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(10):
            for fn in stages:
                fn()
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    return {"seconds": round(time.perf_counter() - t0, 3), "calls": n}


def back_to_back(stages, steps: int) -> tuple:
    """`steps` calls launched back to back on the current stream, bracketed by
    synchronisation and one HIP event at each end; no event inside (an event
    recorded between two kernels holds the next launch for a few
    microseconds). Returns (event ms of the region, wall seconds)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        for fn in stages:
            fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), time.perf_counter() - wall0


def timed_calls(stages, warmup: int, steps: int) -> dict:
    """`warmup` untimed calls; the timed region: `steps` calls back to back
    (back_to_back), whose event time gives the throughput; then `steps` more
    calls, each bracketed by HIP events with one more event after every stage,
    for per-call and per-stage distributions (these include the events' own
    gaps). Returns the region's time, per-call totals and per-stage times
    (ms)."""
    import torch
    for _ in range(warmup):
        for fn in stages:
            fn()
    region, wall = back_to_back(stages, steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        for j, fn in enumerate(stages):
            fn()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    total = [e[0].elapsed_time(e[-1]) for e in ev]
    per_stage = [[e[j].elapsed_time(e[j + 1]) for e in ev] for j in range(len(stages))]
    return {"total": total, "stages": per_stage, "region_ms": region, "wall_s": wall}


def tflops(flops: float, ms: float) -> float:
    return flops / (ms * 1e-3) / 1e12


# ---- the workloads ----------------------------------------------------------

def to_dev(x, dtype=None):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.device("cuda:0"))
    return t if dtype is None else t.to(dtype)


def setup_forward(config: str, kprologue: str = "auto"):
    """(workload, [prepare, attend], out) of one plain call on a configuration."""
    import torch
    from diffusion_transformer_image_head_amd.binding import prepared_call
    from diffusion_transformer_image_head_amd.workloads import config_workload

    w = config_workload(config)
    q, k, v = (to_dev(x, torch.bfloat16) for x in (w.q, w.k, w.v))
    sl = None if w.seq_lens is None else to_dev(w.seq_lens)
    prepare, attend, out = prepared_call(q, k, v, to_dev(w.pos), to_dev(w.gamma_q), to_dev(w.gamma_k), sl,
                                         text_pad=w.text_pad, section=w.section, kprologue=kprologue)
    return w, [prepare, attend], out


def setup_cfg():
    """One guided sampling step at 1024px: the conditional pass (512 text
    slots + 64x64 image) and the unconditional pass (the 4096 image tokens
    alone) as one grouped call; also the same two problems as two plain calls.
    Returns (cond workload, flops, grouped fn, separate fn, cond out)."""
    import numpy as np
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn, mrope_attn_group
    from diffusion_transformer_image_head_amd.workloads import config_workload, make_workload

    cond = config_workload("1024px")
    unc = make_workload(1, 32, 128, (16, 24, 24), 0, 64, 64, dtype="bf16", seed=21)
    unc.pos = np.ascontiguousarray(cond.pos[:, cond.text_pad:])
    probs = []
    for w in (cond, unc):
        probs.append(dict(q=to_dev(w.q, torch.bfloat16), k=to_dev(w.k, torch.bfloat16),
                          v=to_dev(w.v, torch.bfloat16), pos=to_dev(w.pos), gamma_q=to_dev(w.gamma_q),
                          gamma_k=to_dev(w.gamma_k), text_pad=w.text_pad, section=w.section))
    for p in probs:
        p["out"] = torch.empty_like(p["q"])
    dev = torch.device("cuda:0")
    ws = torch.empty(1 << 27, dtype=torch.uint8, device=dev)
    ws2 = torch.empty(1 << 27, dtype=torch.uint8, device=dev)

    def grouped():
        mrope_attn_group(probs, workspace=ws)

    def separate():
        for p, wsp in zip(probs, (ws, ws2)):
            mrope_attn(p["q"], p["k"], p["v"], p["pos"], p["gamma_q"], p["gamma_k"],
                       text_pad=p["text_pad"], section=p["section"], out=p["out"], workspace=wsp)

    return cond, cond.flops() + unc.flops(), grouped, separate, probs[0]["out"]


def setup_bwd(config: str):
    """The backward pass on a configuration: one untimed forward for out and
    lse, then a callable running one backward. FLOPs: the usual 2.5x the
    forward's (dV, dP, dQ, dK and the recomputed S: five S^2 D products
    against the forward's two)."""
    import numpy as np
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn, mrope_attn_bwd
    from diffusion_transformer_image_head_amd.workloads import config_workload, round_to_bf16

    w = config_workload(config)
    q, k, v = (to_dev(x, torch.bfloat16) for x in (w.q, w.k, w.v))
    pos, gq, gk = to_dev(w.pos), to_dev(w.gamma_q), to_dev(w.gamma_k)
    sl = None if w.seq_lens is None else to_dev(w.seq_lens)
    kw = dict(text_pad=w.text_pad, section=w.section)
    out, lse = mrope_attn(q, k, v, pos, gq, gk, sl, return_lse=True, **kw)
    do = to_dev(round_to_bf16(np.random.default_rng(3).standard_normal(w.q.shape).astype(np.float32)),
                torch.bfloat16)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(1 << 28, dtype=torch.uint8, device=torch.device("cuda:0"))

    def step():
        mrope_attn_bwd(q, k, v, pos, gq, gk, sl, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    return w, 2.5 * w.flops(), step


def setup_qkv(config: str):
    """The layer's attention input path at a configuration's shape: x [B*S,
    hidden = H*D] bf16 through the fp8 e4m3 fused qkv weight with the
    norm/rotation epilogue (one call), and the attention on those operands.
    Returns (workload, projection flops, proj fn, attend fn, attention flops)."""
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn, mrope_qkv_proj
    from diffusion_transformer_image_head_amd.workloads import CONFIGS, make_qkv_workload

    c = CONFIGS[config]
    h, d = c["heads"], c["head_dim"]
    w = make_qkv_workload(c["batch"], h, d, c["section"], c["text_pad"], c["grid_h"], c["grid_w"],
                          h * d, seed=c["seed"])
    dev = torch.device("cuda:0")
    x = to_dev(w.x, torch.bfloat16)
    w8, wsc, pos, gq, gk = to_dev(w.w8), to_dev(w.w_scale), to_dev(w.pos), to_dev(w.gamma_q), to_dev(w.gamma_k)
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

    return w, w.flops(), proj, attend, 4 * h * d * s * s * b


# ---- oracle baseline --------------------------------------------------------

def host_threads() -> dict:
    """os.cpu_count(), the affinity count and the BLAS thread count."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = None
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = None
    return {"cpu_count": os.cpu_count(), "affinity": aff, "blas_threads": blas}


def cpu_baseline(w, gpu_out, runs: int):
    """The fp64 oracle on the host over the whole workload, `runs` times
    (median reported); also the parity check of the GPU output."""
    import numpy as np
    from oracle.reference import oracle_fwd
    secs = []
    ref = None
    for _ in range(runs):
        t0 = time.perf_counter()
        ref, _ = oracle_fwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens,
                            text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps)
        secs.append(time.perf_counter() - t0)
    dt = float(np.median(secs))
    d = gpu_out - ref
    rel = float(np.sqrt((d * d).sum() / (ref * ref).sum()))
    th = host_threads()
    return {
        "value": round(w.flops() / dt / 1e12, 6), "unit": "TFLOP/s",
        # matmuls run on the BLAS pool, the elementwise steps on one thread
        "cores": int(th["blas_threads"] or th["affinity"] or th["cpu_count"]),
        "kind": "oracle", "seconds": round(dt, 3), "runs": [round(s, 3) for s in secs], **th,
        "sample": f"the whole workload ({w.shape[2]} heads, all {w.shape[1]} query rows), fp64 NumPy, "
                  f"median of {runs} runs",
    }, {"max_abs": float(np.abs(d).max()), "rel_rms": rel}


# ---- sub-benchmarks ---------------------------------------------------------

def base_record(args, metric, value, ms, workload, dtype="bf16"):
    return {"metric": metric, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": DATA, "config": {"workload": workload},
            "runtime_env": {"HIP_FORCE_DEV_KERNARG": os.environ.get("HIP_FORCE_DEV_KERNARG")}}


def roofline(achieved, kernel, **kw):
    return dict({"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": kernel}, **kw)


def bench_cfg(args):
    """cfg1024: one guided step (cond + uncond) as one grouped call, against
    the same two problems as two plain calls."""
    import numpy as np
    cond, flops, grouped, separate, out = setup_cfg()
    pw = prewarm([grouped], args.prewarm_s)
    sep = timed_calls([separate], args.warmup, args.steps)
    grp = timed_calls([grouped], args.warmup, args.steps)
    ms = grp["region_ms"] / args.steps
    rec = base_record(args, METRIC + " (guided step: cond + uncond)", tflops(flops, ms), ms,
                      "cfg1024: 1024px cond (B=1 H=32 D=128, 512 text + 64x64 image) "
                      "+ image-only uncond (4096 tokens), one grouped call")
    rec["roofline"] = roofline(tflops(flops, ms), "whole grouped call (prologues + attention + merge)",
                               kernel_ms=round(ms, 5), statistic="mean over the back-to-back timed calls (HIP events at the region's ends)")
    rec["prewarm"] = pw
    rec["call_ms"] = summarize(grp["total"])
    sms = sep["region_ms"] / args.steps
    rec["separate_calls"] = {"ms_mean": round(sms, 5), "value": round(tflops(flops, sms), 3)}
    if not args.no_cpu_baseline:
        base, par = cpu_baseline(cond, out.float().cpu().numpy().astype(np.float64), 1)
        rec["cpu_baseline"] = dict(base, sample="the conditional pass only (" + base["sample"] + ")")
        rec["parity"] = par
    print(json.dumps(rec), flush=True)


def bench_qkv(args):
    """fp8 QKV projection with the norm/rotation epilogue, then the attention
    on its operands. value = the projection's FLOP rate (2 * tokens * hidden
    * 3 H D)."""
    import numpy as np
    w, flops, proj, attend, att_flops = setup_qkv(args.config)
    pw = prewarm([proj], args.prewarm_s)
    tp = timed_calls([proj], args.warmup, args.steps)
    ta = timed_calls([attend], args.warmup, args.steps)
    ms = tp["region_ms"] / args.steps
    rec = base_record(args, "fp8 QKV projection + norm/rotation epilogue TFLOP/s (bf16 matrix cores)",
                      tflops(flops, ms), ms,
                      f"{args.config} qkv: tokens={w.batch * w.seq} hidden={w.heads * w.head_dim} "
                      f"out={3 * w.heads * w.head_dim}")
    rec["data"] = "synthetic (seeded N(0,1) x, N(0,1/hidden) weight quantized to e4m3 per row)"
    rec["roofline"] = roofline(tflops(flops, ms), "rope_table_kernel + qkv_proj_kernel", kernel_ms=round(ms, 5),
                               statistic="mean over the back-to-back timed calls (HIP events at the region's ends)")
    rec["prewarm"] = pw
    rec["call_ms"] = summarize(tp["total"])
    am = ta["region_ms"] / args.steps
    rec["attention_on_operands"] = {"ms_mean": round(am, 5), "TFLOP/s": round(tflops(att_flops, am), 3)}
    rec["kernel_source_hash"] = kernel_source_hash("qkv")
    if args.config == "1024px":
        rec["profile"] = path_profile_status("qkv_proj_1024px_kernel_trace.txt", "qkv")
    print(json.dumps(rec), flush=True)


def bench_bwd(args):
    """Backward pass on a configuration (2.5x the forward's FLOPs)."""
    import numpy as np
    w, flops, step = setup_bwd(args.config)
    pw = prewarm([step], args.prewarm_s)
    tb = timed_calls([step], args.warmup, args.steps)
    ms = tb["region_ms"] / args.steps
    bb, s, h, d = w.shape
    rec = base_record(args, "fused QK-norm+M-RoPE attention backward TFLOP/s (2.5x forward FLOPs)",
                      tflops(flops, ms), ms, f"{args.config} backward: B={bb} H={h} head_dim={d} tokens={s}")
    rec["data"] = DATA.replace("q/k/v", "q/k/v/dO")
    rec["roofline"] = roofline(tflops(flops, ms), "whole backward call (prologues, delta, dk/dv/dq, dgamma)",
                               kernel_ms=round(ms, 5), statistic="mean over the back-to-back timed calls (HIP events at the region's ends)")
    rec["prewarm"] = pw
    rec["call_ms"] = summarize(tb["total"])
    rec["kernel_source_hash"] = kernel_source_hash("backward")
    if args.config == "1024px":
        rec["profile"] = path_profile_status("attn_bwd_1024px_kernel_trace.txt", "backward")
    print(json.dumps(rec), flush=True)


def bench_packed(args):
    """A configuration's prompts packed back to back (cu_seqlens; each
    prompt's true-length text tokens then its image) instead of padded:
    the packed forward (prologue + attention), or with --backward the packed
    backward after one untimed forward. FLOPs are the sequences' own: 4 H D
    sum(n_b^2), times 2.5 for the backward."""
    import numpy as np
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn_bwd_varlen, mrope_attn_varlen
    from diffusion_transformer_image_head_amd.workloads import CONFIGS, make_varlen_workload, round_to_bf16

    c = CONFIGS[args.config]
    lens = c["text_lens"] if c["text_lens"] is not None else (c["text_pad"],) * c["batch"]
    w = make_varlen_workload(c["heads"], c["head_dim"], c["section"], text_lens=lens,
                             grids=[(c["grid_h"], c["grid_w"])] * c["batch"], sigma=c["sigma"],
                             seed=c["seed"])
    q, k, v = (to_dev(x, torch.bfloat16) for x in (w.q, w.k, w.v))
    pos, gq, gk = to_dev(w.pos), to_dev(w.gamma_q), to_dev(w.gamma_k)
    cu = to_dev(w.cu_seqlens.astype(np.int32))
    ms_len = w.max_seqlen
    out = torch.empty_like(q)
    ws = torch.empty(1 << 29, dtype=torch.uint8, device=torch.device("cuda:0"))
    _, lse = mrope_attn_varlen(q, k, v, pos, gq, gk, cu, ms_len, section=w.section, return_lse=True,
                               out=out, workspace=ws)
    if args.backward:
        do = to_dev(round_to_bf16(np.random.default_rng(3).standard_normal(w.q.shape).astype(np.float32)),
                    torch.bfloat16)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def step():
            mrope_attn_bwd_varlen(q, k, v, pos, gq, gk, cu, ms_len, out, lse, do, section=w.section,
                                  dq=dq, dk=dk, dv=dv, workspace=ws)
    else:
        def step():
            mrope_attn_varlen(q, k, v, pos, gq, gk, cu, ms_len, section=w.section, out=out, workspace=ws)

    pw = prewarm([step], args.prewarm_s)
    tm = timed_calls([step], args.warmup, args.steps)
    ms = tm["region_ms"] / args.steps
    mult = 2.5 if args.backward else 1.0
    what = "backward" if args.backward else "forward"
    rec = base_record(args, f"fused QK-norm+M-RoPE attention {what} TFLOP/s, packed sequences"
                      + (" (2.5x forward FLOPs)" if args.backward else ""), tflops(mult * w.flops(), ms), ms,
                      f"{args.config} packed {what}: {len(lens)} sequences, {w.q.shape[0]} tokens, "
                      f"H={c['heads']} head_dim={c['head_dim']}")
    rec["config"]["cu_seqlens"] = [int(x) for x in w.cu_seqlens]
    rec["roofline"] = roofline(tflops(mult * w.flops(), ms), f"whole packed {what} call", kernel_ms=round(ms, 5),
                               statistic="mean over the back-to-back timed calls (HIP events at the region's ends)")
    rec["prewarm"] = pw
    rec["call_ms"] = summarize(tm["total"])
    print(json.dumps(rec), flush=True)


def extras(args) -> dict:
    """The grouped guided step, the backward and the fp8 projection at the
    1024px shape, each after its own warm-up; rates from the mean of
    back-to-back calls, with the median of per-call events beside them."""
    import numpy as np
    import torch
    res = {}
    warm, steps = max(args.warmup, 10), max(args.steps, 20)
    _, flops, grouped, _, _ = setup_cfg()
    g = timed_calls([grouped], warm, steps)
    gm = g["region_ms"] / steps
    res["cfg1024_grouped"] = {"ms_mean": round(gm, 5), "TFLOP/s": round(tflops(flops, gm), 3),
                              "ms_median_events": round(float(np.median(g["total"])), 5),
                              "what": "cond 4608 + image-only uncond 4096 tokens, H=32, one grouped call"}
    torch.cuda.empty_cache()
    _, flops, step = setup_bwd("1024px")
    b = timed_calls([step], warm, steps)
    bm = b["region_ms"] / steps
    res["backward_1024px"] = {"ms_mean": round(bm, 5), "TFLOP/s": round(tflops(flops, bm), 3),
                              "ms_median_events": round(float(np.median(b["total"])), 5),
                              "what": "dq, dk, dv, dgammas; FLOPs 2.5x the forward's",
                              "kernel_source_hash": kernel_source_hash("backward"),
                              "profile": path_profile_status("attn_bwd_1024px_kernel_trace.txt", "backward")}
    torch.cuda.empty_cache()
    _, flops, proj, _, _ = setup_qkv("1024px")
    p = timed_calls([proj], warm, steps)
    pm = p["region_ms"] / steps
    res["qkv_proj_1024px"] = {"ms_mean": round(pm, 5), "TFLOP/s": round(tflops(flops, pm), 3),
                              "ms_median_events": round(float(np.median(p["total"])), 5),
                              "what": "x [4608, 4096] bf16 x fp8 e4m3 W [12288, 4096] with row scales, "
                                      "norm/rotation epilogue",
                              "kernel_source_hash": kernel_source_hash("qkv"),
                              "profile": path_profile_status("qkv_proj_1024px_kernel_trace.txt", "qkv")}
    for r in res.values():
        r["frac"] = round(r["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
    res["protocol"] = (f"{warm} warm-up + {steps} back-to-back timed calls each (TFLOP/s from their mean), "
                       f"then {steps} calls with per-call events (ms_median_events), after the headline region")
    return res


def bench_forward(args):
    import numpy as np
    from diffusion_transformer_image_head_amd.binding import lib

    lib()  # fail loudly without the HIP library
    w, stages, out = setup_forward(args.config, args.kprologue)
    b, s, h, d = w.shape
    pw = prewarm(stages, args.prewarm_s)
    tm = timed_calls(stages, args.warmup, args.steps)
    flops = w.flops()
    ms_step = tm["region_ms"] / args.steps
    # the attend stage alone, back to back: its mean launch time
    att_region, _ = back_to_back([stages[1]], args.steps)
    att_mean = att_region / args.steps
    att = tm["stages"][1]
    value = tflops(flops, ms_step)
    achieved = tflops(flops, att_mean)
    rec = base_record(args, METRIC, value, ms_step,
                      f"{args.config}: B={b} H={h} head_dim={d} tokens={s} "
                      f"(text_pad={w.text_pad} + {w.grid[0]}x{w.grid[1]} image)")
    rec["config"].update({"batch": b, "heads": h, "head_dim": d, "seq_len": s, "section": list(w.section),
                          "kprologue": args.kprologue,
                          "text_lens": None if w.seq_lens is None else [int(x) for x in w.seq_lens]})
    rec["roofline"] = roofline(achieved, "attn_bf16_kernel + split_merge_kernel (attend stage)",
                               traffic=traffic_from_profile(args.config), kernel_ms=round(att_mean, 5),
                               statistic=f"mean over {args.steps} back-to-back attend-stage calls (HIP events "
                                         "at the region's ends), after the timed steps")
    rec["timing"] = (f"value: {args.steps} steps back to back, HIP events at the region's ends only; roofline: "
                     f"{args.steps} attend-stage calls back to back; attend_ms / step_ms: {args.steps} more steps "
                     "with an event after every stage (they include the events' own gaps)")
    rec["attend_ms"] = summarize(att)
    rec["step_ms"] = summarize(tm["total"])
    rec["prologue_ms_median"] = round(float(np.median(tm["stages"][0])), 5)
    rec["frac_of_peak_whole_step"] = round(value / PEAK_BF16_TFLOPS, 4)
    rec["prewarm"] = pw
    rec["wall_s"] = round(tm["wall_s"], 4)
    rec["kernel_source_hash"] = kernel_source_hash()
    rec["profiles"] = profiles_status(args.config)
    if not args.no_extras and args.config == "1024px":
        rec["extras"] = extras(args)
    if not args.no_cpu_baseline:
        got = out.float().cpu().numpy().astype(np.float64)
        runs = 3 if s <= 4608 and b == 1 else 1
        base, parity = cpu_baseline(w, got, runs)
        rec["cpu_baseline"] = base
        rec["parity"] = dict(parity, bars={"max_abs": 2e-2, "rel_rms": 5e-3},
                             ok=bool(parity["max_abs"] <= 2e-2 and parity["rel_rms"] <= 5e-3))
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of back-to-back untimed steps before the counted warm-up (declared "
                         "in the output; the clock of an idle GPU ramps up under load)")
    ap.add_argument("--config", default="1024px",
                    choices=["512px", "1024px", "ragged", "long", "h36", "2048px", "cfg1024", "h4"],
                    help="cfg1024: one guided step, the 1024px conditional pass and its "
                         "image-only unconditional pass in one grouped call")
    ap.add_argument("--kprologue", default="auto", choices=["auto", "prepass", "fused"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the grouped-step / backward / projection timings of the default line")
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
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    from diffusion_transformer_image_head_amd.binding import lib
    lib()  # fail loudly without the HIP library
    if args.config == "cfg1024":
        bench_cfg(args)
    elif args.packed:
        bench_packed(args)
    elif args.backward:
        bench_bwd(args)
    elif args.qkv:
        bench_qkv(args)
    else:
        bench_forward(args)


if __name__ == "__main__":
    main()
