"""Where the bf16 parity bars come from (CPU only).

The bf16 path rounds Q' and K' once to bf16 (after norm and rotation) and the
probabilities once before P.V. The error that the Q'/K' rounding alone
causes is computed here by evaluating the oracle's attention step on
bf16-rounded Q', K' (rounding is the workload module's round-to-nearest-even);
it is a floor no bf16 implementation of the same numerics can go below.

* For the shapes of the named workloads (logit spread ~ 1) the floor is
  max-abs ~1.5e-3 / rel-RMS ~2.7e-3, inside the bars max-abs 2e-2 /
  rel-RMS 5e-3 that the GPU parity tests use (rel-RMS is the binding one).
* For the peaked stress case (gammas x3, logit spread ~ 10) the floor alone
  is ~0.095 max-abs, so that case gets bars scaled from its own floor.
"""

import numpy as np

import oracle.reference as ref
from diffusion_transformer_image_head_amd.workloads import make_workload, round_to_bf16

CONFIG_BARS = (2e-2, 5e-3)
PEAKED_BARS = (0.15, 1.2e-2)   # ~1.5x the rounding floor derived below


def peaked_workload():
    w = make_workload(1, 2, 128, (16, 24, 24), 64, 16, 16, dtype="bf16", seed=320)
    w.gamma_q = w.gamma_q * 3
    w.gamma_k = w.gamma_k * 3
    return w


def _rounding_floor(w):
    exact, _ = ref.oracle_fwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens,
                              text_pad=w.text_pad, section=w.section)
    qr = ref.mrope(ref.rms_norm(w.q, w.gamma_q, w.eps), w.pos, w.section, w.theta)
    kr = ref.mrope(ref.rms_norm(w.k, w.gamma_k, w.eps), w.pos, w.section, w.theta)
    qb = round_to_bf16(qr.astype(np.float32)).astype(np.float64)
    kb = round_to_bf16(kr.astype(np.float32)).astype(np.float64)
    valid = ref.valid_tokens(w.q.shape[0], w.q.shape[1], w.text_pad, w.seq_lens)
    rounded, _ = ref.attention(qb, kb, w.v, valid, 1.0 / np.sqrt(w.q.shape[-1]))
    d = rounded - exact
    return float(np.abs(d).max()), float(np.sqrt((d * d).sum() / (exact * exact).sum()))


def test_config_like_floor_is_well_inside_the_bars():
    w = make_workload(1, 4, 128, (16, 24, 24), 128, 24, 24, dtype="bf16", seed=401)
    ma, rr = _rounding_floor(w)
    # rel-RMS is the binding bar: the Q'/K' rounding alone uses ~55% of it
    # (P and output rounding add the rest on the GPU), max-abs is loose
    assert ma < CONFIG_BARS[0] / 4 and rr < CONFIG_BARS[1] * 0.7, (ma, rr)


def test_peaked_floor_sets_its_bars():
    ma, rr = _rounding_floor(peaked_workload())
    # the floor alone breaks the config bars, and the peaked bars leave ~1.5x room
    assert ma > CONFIG_BARS[0] and rr > CONFIG_BARS[1]
    assert ma * 1.3 < PEAKED_BARS[0] and rr * 1.3 < PEAKED_BARS[1], (ma, rr)


# ---------------------------------------------------------------- backward
# Backward bars: rel-RMS of each gradient and max-abs relative to the
# gradient's largest magnitude. The emulated bf16 rounding floor of the
# kernels (tests/bwd_emul.py) is ~4.5e-3 rel-RMS and ~0.7% relative max-abs.
BWD_BARS = (2e-2, 1e-2)


def bwd_errors(got, ref):
    d = got - ref
    scale = float(np.abs(ref).max()) or 1.0
    rel = float(np.sqrt(np.sum(d * d) / max(float(np.sum(ref * ref)), 1e-300)))
    return float(np.abs(d).max()) / scale, rel


def test_bwd_bars_sit_above_the_rounding_floor():
    from oracle.backward import oracle_bwd
    from tests.bwd_emul import emulate
    w = make_workload(2, 3, 128, (16, 24, 24), 40, 9, 13, text_lens=(17, 40), seed=600)
    do = round_to_bf16(np.random.default_rng(3).standard_normal(w.q.shape).astype(np.float32))
    ref = oracle_bwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens, do,
                     text_pad=w.text_pad, section=w.section)
    for got, r in zip(emulate(w, do.astype(np.float64)), ref):
        ma, rr = bwd_errors(got, r)
        assert ma * 1.5 <= BWD_BARS[0] and rr * 1.5 <= BWD_BARS[1], (ma, rr)
        assert rr > 1e-3          # the floor is real: the bars are not loose by orders
