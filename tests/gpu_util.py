"""Helpers shared by the GPU tests: move a workload to the device, run the
HIP path through the binding, run the oracle, and measure the difference."""

from __future__ import annotations

import sys

import numpy as np

from oracle.reference import oracle_fwd

# Parity bars: bf16 max-abs <= 2e-2 and relative RMS <= 5e-3; fp32 both <= 1e-5.
TOL = {"bf16": (2e-2, 5e-3), "fp32": (1e-5, 1e-5)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(w, device="cuda"):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(device)  # noqa: E731
    return dict(
        q=t(w.q).to(dt), k=t(w.k).to(dt), v=t(w.v).to(dt), pos=t(w.pos),
        gamma_q=t(w.gamma_q), gamma_k=t(w.gamma_k),
        seq_lens=None if w.seq_lens is None else t(w.seq_lens.astype(np.int32)))


def run_gpu(w, dev=None, **kw):
    """HIP path on workload w; returns (out, lse) as float64 numpy arrays."""
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn
    dev = dev or to_dev(w)
    kw.setdefault("rope_pairs", w.rope_pairs)
    out, lse = mrope_attn(dev["q"], dev["k"], dev["v"], dev["pos"], dev["gamma_q"],
                          dev["gamma_k"], dev["seq_lens"], text_pad=w.text_pad,
                          section=w.section, theta=w.theta, eps=w.eps, return_lse=True, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_oracle(w, rows=None, heads=None):
    return oracle_fwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens,
                      text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps,
                      rows=rows, heads=heads, rope_pairs=w.rope_pairs)


def errors(got, ref):
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.sqrt(np.sum(ref * ref)))
    rel = float(np.sqrt(np.sum(d * d)) / den) if den > 0 else float(np.sqrt(np.sum(d * d)))
    return max_abs, rel


def check_parity(got, ref, dtype, what=""):
    ma, rr = errors(got, ref)
    tol_abs, tol_rel = TOL[dtype]
    say(f"  parity {what}: max_abs={ma:.3e} rel_rms={rr:.3e} (bars {tol_abs:g}/{tol_rel:g})")
    assert np.isfinite(got).all(), "non-finite output"
    assert ma <= tol_abs, f"max-abs {ma} > {tol_abs}"
    assert rr <= tol_rel, f"rel-RMS {rr} > {tol_rel}"
    return ma, rr


def check_lse(got, ref, tol=2e-2):
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), "lse finiteness differs"
    if fin.any():
        err = float(np.max(np.abs(got[fin] - ref[fin])))
        say(f"  lse max_abs={err:.3e}")
        assert err <= tol


def sample_rows(w, n=160, seed=0):
    """Query rows for full-size checks: both ends, every text/image boundary,
    tile edges, and a seeded random draw."""
    s = w.q.shape[1]
    rng = np.random.default_rng(seed)
    fixed = {0, 1, s - 1, s - 2, w.text_pad - 1, w.text_pad, 127, 128, 255, 256}
    if w.seq_lens is not None:
        for l in w.seq_lens:
            fixed.update({int(l) - 1, int(l)})
    fixed = {r for r in fixed if 0 <= r < s}
    extra = rng.choice(s, size=min(n, s), replace=False)
    return np.array(sorted(fixed | set(int(x) for x in extra)))
