"""Pins for the fp64 oracle: checks against facts fixed outside the oracle.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the source pages or the mathematics fix. They are collected by
``test_oracle.py`` and also replayed there against deliberately broken copies
of the oracle (planted on the CPU), to show every plausible slip trips one.

The oracle functions are looked up through the module object at call time
so a planted mistake is seen by every pin.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.reference as ref
from oracle.brute import brute_fwd
from diffusion_transformer_image_head_amd.workloads import make_workload, config_workload, CONFIGS

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _run(w, **kw):
    return ref.oracle_fwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens,
                          text_pad=w.text_pad, section=w.section, theta=w.theta,
                          eps=w.eps, **kw)


def _prologue(x, gamma, pos, section, theta=1e4, eps=1e-6):
    return ref.mrope(ref.rms_norm(x, gamma, eps), pos, section, theta)


# --------------------------------------------------------------------- P1
def _brute_case(w):
    out, lse = _run(w)
    bo, bl = brute_fwd(w.q.tolist(), w.k.tolist(), w.v.tolist(), w.pos.tolist(),
                       w.gamma_q.tolist(), w.gamma_k.tolist(),
                       None if w.seq_lens is None else w.seq_lens.tolist(),
                       text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps)
    bo = np.array(bo)
    bl = np.array(bl)
    assert np.max(np.abs(out - bo)) < 1e-12, np.max(np.abs(out - bo))
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - bl[fin])) < 1e-12


def pin_brute_tiny():
    """P1: scalar loops == vectorised oracle on the tiny config (8/12/12)."""
    _brute_case(config_workload("tiny"))


def pin_brute_sections():
    """P1/P12: both section splits of the pages and configs, small grids."""
    _brute_case(make_workload(1, 2, 16, (2, 3, 3), 5, 3, 4, seed=11, dtype="fp32"))
    # the deep-dive split (24,20,20) at head_dim 128
    _brute_case(make_workload(1, 1, 128, (24, 20, 20), 6, 3, 3, seed=12, dtype="fp32"))
    _brute_case(make_workload(1, 1, 128, (16, 24, 24), 6, 3, 3, seed=13, dtype="bf16"))


def pin_brute_ragged():
    """P1: ragged batch with padded text slots (including an empty text)."""
    _brute_case(make_workload(3, 2, 16, (2, 3, 3), 6, 2, 3, text_lens=(0, 3, 6),
                              seed=14, dtype="fp32"))


def pin_brute_peaked():
    """P1: peaked attention (large gammas -> logit spread ~ 10)."""
    w = make_workload(1, 1, 32, (4, 6, 6), 4, 4, 4, seed=15, dtype="fp32")
    w.gamma_q = w.gamma_q * 3.0
    w.gamma_k = w.gamma_k * 3.0
    _brute_case(w)


# --------------------------------------------------------------------- P2
def pin_rope_norm_preserving():
    """P2: M-RoPE keeps the norm of every row and of every rotary pair."""
    rng = np.random.default_rng(21)
    for d, sec in ((64, (8, 12, 12)), (128, (16, 24, 24)), (128, (24, 20, 20))):
        x = rng.standard_normal((2, 7, 3, d))
        pos = rng.integers(-50, 700, size=(2, 7, 3))
        y = ref.mrope(x, pos, sec, 1e4)
        h = d // 2
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
        px = x[..., :h] ** 2 + x[..., h:] ** 2
        py = y[..., :h] ** 2 + y[..., h:] ** 2
        assert np.allclose(px, py, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------- P3
def pin_relative_positions():
    """P3: after M-RoPE, q.k depends only on the per-axis position differences."""
    rng = np.random.default_rng(31)
    d, sec = 128, (16, 24, 24)
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, 1, d))
    for _ in range(20):
        pq = rng.integers(0, 600, size=3)
        pk = rng.integers(0, 600, size=3)
        shift = rng.integers(-300, 300, size=3)
        a = (ref.mrope(q, pq[None, None], sec, 1e4) * ref.mrope(k, pk[None, None], sec, 1e4)).sum()
        b = (ref.mrope(q, (pq + shift)[None, None], sec, 1e4)
             * ref.mrope(k, (pk + shift)[None, None], sec, 1e4)).sum()
        assert abs(a - b) < 1e-10 * (1 + abs(a)), (a, b)
    # and changing one axis's difference does change it (the axis is used)
    for ax in range(3):
        pk2 = pk.copy()
        pk2[ax] += 7
        c = (ref.mrope(q, pq[None, None], sec, 1e4) * ref.mrope(k, pk2[None, None], sec, 1e4)).sum()
        assert abs(c - a) > 1e-6


def pin_shift_whole_output():
    """P3 on the whole op: shifting all positions per axis leaves the output."""
    w = make_workload(2, 2, 32, (4, 6, 6), 8, 3, 5, text_lens=(3, 8), seed=32, dtype="fp32")
    o1, l1 = _run(w)
    w.pos = w.pos + np.array([37, 11, 5], dtype=np.int32)
    o2, l2 = _run(w)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    fin = np.isfinite(l1)
    assert np.max(np.abs(l1[fin] - l2[fin])) < 1e-12


# --------------------------------------------------------------------- P4
def _rope_1d_roformer(x, m, theta):
    """Textbook 1D RoPE (RoFormer): block-diagonal rotation over consecutive
    pairs (2i, 2i+1) with angle m * theta^(-2i/d), built as a matrix."""
    d = x.shape[-1]
    rmat = np.zeros((d, d))
    for i in range(d // 2):
        ang = m * theta ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        rmat[2 * i, 2 * i] = c
        rmat[2 * i, 2 * i + 1] = -s
        rmat[2 * i + 1, 2 * i] = s
        rmat[2 * i + 1, 2 * i + 1] = c
    return rmat @ x


def pin_text_tokens_are_1d_rope():
    """P4: text tokens (t = h = w = i) get exactly textbook 1D RoPE.

    Half-split pair (j, j + D/2) is RoFormer's consecutive pair (2j, 2j+1)
    after the interleaving permutation.
    """
    rng = np.random.default_rng(41)
    for d, sec in ((64, (8, 12, 12)), (128, (16, 24, 24)), (128, (24, 20, 20))):
        h = d // 2
        perm = np.empty(d, dtype=np.int64)   # interleaved index -> half-split index
        perm[0::2] = np.arange(h)
        perm[1::2] = np.arange(h) + h
        for m in (0, 1, 5, 77, 511):
            x = rng.standard_normal(d)
            y = ref.mrope(x[None, None, None, :], np.array([[[m, m, m]]]), sec, 1e4)[0, 0, 0]
            want = _rope_1d_roformer(x[perm], float(m), 1e4)
            assert np.max(np.abs(y[perm] - want)) < 1e-12, (d, sec, m)


def pin_axis_blocks_and_angles():
    """Each section block turns by exactly pos[axis] * theta^(-2j/D), and only
    the block of the axis whose position is nonzero turns."""
    rng = np.random.default_rng(42)
    d, sec = 128, (16, 24, 24)
    h = d // 2
    bounds = [0, sec[0], sec[0] + sec[1], h]
    x = rng.standard_normal(d)
    for ax in range(3):
        p = np.zeros(3, dtype=np.int64)
        p[ax] = 3
        y = ref.mrope(x[None, None, None, :], p[None, None], sec, 1e4)[0, 0, 0]
        ang_in = np.arctan2(x[h:], x[:h])
        ang_out = np.arctan2(y[h:], y[:h])
        turned = np.angle(np.exp(1j * (ang_out - ang_in)))
        for j in range(h):
            want = 3.0 * 1e4 ** (-2.0 * j / d) if bounds[ax] <= j < bounds[ax + 1] else 0.0
            want = math.atan2(math.sin(want), math.cos(want))
            assert abs(turned[j] - want) < 1e-12, (ax, j, turned[j], want)


# --------------------------------------------------------------------- P5
def pin_rows_sum_to_one():
    """P5: with one-hot V rows (S <= D) the output is the probability matrix:
    non-negative rows summing to one, zero at padded keys."""
    for lens in (None, (2, 5)):
        w = make_workload(2, 2, 32, (4, 6, 6), 5, 3, 4, text_lens=lens, seed=51, dtype="fp32")
        s = w.q.shape[1]
        eye = np.zeros((2, s, 2, 32))
        for j in range(s):
            eye[:, j, :, j] = 1.0
        w.v = eye
        out, _ = _run(w)
        valid = ref.valid_tokens(2, s, w.text_pad, w.seq_lens)
        p = out[..., :s]
        assert np.all(p >= 0)
        for b in range(2):
            rs = p[b].sum(axis=-1)
            assert np.allclose(rs[valid[b]], 1.0, atol=1e-13)
            assert np.all(rs[~valid[b]] == 0)
            assert np.all(p[b][:, :, ~valid[b]] == 0)


# --------------------------------------------------------------------- P6 / P7
def pin_uniform_v():
    """P6: a uniform V comes back unchanged (weights are a convex combination)."""
    w = make_workload(2, 3, 64, (8, 12, 12), 8, 3, 3, text_lens=(2, 8), seed=61, dtype="fp32")
    w.v = np.full_like(w.v, 0.375)
    out, _ = _run(w)
    valid = ref.valid_tokens(2, w.q.shape[1], w.text_pad, w.seq_lens)
    assert np.max(np.abs(out[valid] - 0.375)) < 1e-15
    assert np.all(out[~valid] == 0)


def pin_single_key():
    """P7: one real token attends only to itself: out = v, lse = its logit."""
    w = make_workload(1, 2, 16, (2, 3, 3), 3, 0, 0, text_lens=(1,), seed=71, dtype="fp32")
    out, lse = _run(w)
    assert np.array_equal(out[0, 0], w.v[0, 0].astype(np.float64))
    assert np.all(out[0, 1:] == 0)
    qp = _prologue(w.q, w.gamma_q, w.pos, w.section)
    kp = _prologue(w.k, w.gamma_k, w.pos, w.section)
    z = (qp[0, 0] * kp[0, 0]).sum(-1) / 4.0
    assert np.allclose(lse[0, :, 0], z, atol=1e-14)
    assert np.all(np.isneginf(lse[0, :, 1:]))


# --------------------------------------------------------------------- P8
def pin_torch_special_case():
    """P8: zero positions (RoPE = identity) and unit gammas reduce the path to
    torch's rms_norm + scaled_dot_product_attention, in float64 on the CPU."""
    import torch
    import torch.nn.functional as F
    w = make_workload(2, 3, 64, (8, 12, 12), 6, 4, 4, seed=81, dtype="fp32")
    w.pos = np.zeros_like(w.pos)
    w.gamma_q = np.ones_like(w.gamma_q)
    w.gamma_k = np.ones_like(w.gamma_k)
    out, lse = _run(w)
    q = torch.from_numpy(w.q.astype(np.float64)).permute(0, 2, 1, 3)
    k = torch.from_numpy(w.k.astype(np.float64)).permute(0, 2, 1, 3)
    v = torch.from_numpy(w.v.astype(np.float64)).permute(0, 2, 1, 3)
    qn = F.rms_norm(q, (64,), eps=1e-6)
    kn = F.rms_norm(k, (64,), eps=1e-6)
    o = F.scaled_dot_product_attention(qn, kn, v).permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(out - o)) < 1e-12
    zl = torch.logsumexp(qn @ kn.transpose(-1, -2) / 8.0, dim=-1).numpy()
    assert np.max(np.abs(lse - zl)) < 1e-12


# --------------------------------------------------------------------- P9
def pin_masking_equals_unpadded():
    """P9: a padded item equals the same item run alone without its padded
    text slots; poison in padded K/V (NaN, 1e30) changes nothing."""
    lens = (0, 2, 5, 7)
    w = make_workload(4, 2, 32, (4, 6, 6), 7, 3, 2, text_lens=lens, seed=91, dtype="fp32")
    out, lse = _run(w)
    valid = ref.valid_tokens(4, w.q.shape[1], w.text_pad, w.seq_lens)
    for b, lb in enumerate(lens):
        keep = valid[b]
        o1, l1 = ref.oracle_fwd(w.q[b:b + 1, keep], w.k[b:b + 1, keep], w.v[b:b + 1, keep],
                                w.pos[b:b + 1, keep], w.gamma_q, w.gamma_k, None,
                                text_pad=lb, section=w.section)
        assert np.max(np.abs(out[b, keep] - o1[0])) < 1e-12
        assert np.max(np.abs(lse[b][:, keep] - l1[0])) < 1e-12
        assert np.all(out[b, ~keep] == 0)
    for poison in (np.nan, 1e30, -np.inf):
        w2 = make_workload(4, 2, 32, (4, 6, 6), 7, 3, 2, text_lens=lens, seed=91, dtype="fp32")
        pad = ~valid
        w2.k[pad] = poison
        w2.v[pad] = poison
        w2.q[pad] = poison
        o2, l2 = _run(w2)
        assert not np.isnan(o2).any()
        assert np.array_equal(o2, out)


# --------------------------------------------------------------------- P10
def pin_scale_invariance():
    """P10: RMSNorm removes the scale of q and k (exactly when eps = 0)."""
    w = make_workload(1, 2, 64, (8, 12, 12), 4, 3, 3, seed=101, dtype="fp32")
    w.eps = 0.0
    o1, _ = _run(w)
    for c in (1.5, 0.01, 37.0):
        w2 = make_workload(1, 2, 64, (8, 12, 12), 4, 3, 3, seed=101, dtype="fp32")
        w2.eps = 0.0
        w2.q = w2.q.astype(np.float64) * c
        w2.k = w2.k.astype(np.float64) * c
        o2, _ = _run(w2)
        assert np.max(np.abs(o1 - o2)) < 1e-12
    # with eps > 0 the change is of order eps / mean(x^2)
    w.eps = 1e-6
    o3, _ = _run(w)
    assert 0 < np.max(np.abs(o1 - o3)) < 1e-5


# --------------------------------------------------------------------- P11
def pin_permutation_equivariance():
    """P11: permuting image tokens with their positions permutes output rows."""
    w = make_workload(1, 2, 32, (4, 6, 6), 4, 3, 4, seed=111, dtype="fp32")
    out, lse = _run(w)
    rng = np.random.default_rng(112)
    s = w.q.shape[1]
    perm = np.concatenate([np.arange(4), 4 + rng.permutation(s - 4)])
    for name in ("q", "k", "v", "pos"):
        setattr(w, name, getattr(w, name)[:, perm])
    o2, l2 = _run(w)
    assert np.max(np.abs(o2 - out[:, perm])) < 1e-12
    assert np.max(np.abs(l2 - lse[:, :, perm])) < 1e-12


# --------------------------------------------------------------------- closed form
def pin_two_token_closed_form():
    """Two tokens, head_dim 2 (one rotary pair on the t axis), by hand.

    RMSNorm of (a, b) is (a, b) / sqrt((a^2 + b^2)/2 + eps) * gamma; the pair is
    turned by t * 1 (theta^0); z = (q'.k')/sqrt(2); two-key softmax is a
    logistic in the logit difference.
    """
    eps = 1e-6
    q = np.array([[[[3.0, 4.0]], [[-1.0, 2.0]]]])
    k = np.array([[[[1.0, -2.0]], [[0.5, 0.5]]]])
    v = np.array([[[[10.0, -1.0]], [[2.0, 6.0]]]])
    gq = np.array([1.25, 0.75])
    gk = np.array([0.5, 2.0])
    pos = np.array([[[0, 0, 0], [3, 9, 9]]])

    def pro(x, g, t):
        r = 1.0 / math.sqrt((x[0] ** 2 + x[1] ** 2) / 2 + eps)
        u, w_ = x[0] * r * g[0], x[1] * r * g[1]
        return (u * math.cos(t) - w_ * math.sin(t), w_ * math.cos(t) + u * math.sin(t))

    qs = [pro(q[0, i, 0], gq, pos[0, i, 0]) for i in range(2)]
    ks = [pro(k[0, i, 0], gk, pos[0, i, 0]) for i in range(2)]
    out, lse = ref.oracle_fwd(q, k, v, pos, gq, gk, None, text_pad=0, section=(1, 0, 0))
    for i in range(2):
        z = [(qs[i][0] * ks[j][0] + qs[i][1] * ks[j][1]) / math.sqrt(2) for j in range(2)]
        p0 = 1.0 / (1.0 + math.exp(z[1] - z[0]))
        want = p0 * v[0, 0, 0] + (1 - p0) * v[0, 1, 0]
        assert np.max(np.abs(out[0, i, 0] - want)) < 1e-13
        want_lse = max(z) + math.log(math.exp(z[0] - max(z)) + math.exp(z[1] - max(z)))
        assert abs(lse[0, 0, i] - want_lse) < 1e-13


# --------------------------------------------------------------------- page facts
def pin_page_geometry():
    """Workload geometry against the numbers the pages print (golden file)."""
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    comp = facts["spatial_compression"]
    assert [1024 // comp, 1024 // comp] == facts["tokens_1024px"]
    for name, px in (("512px", 512), ("1024px", 1024)):
        c = CONFIGS[name]
        assert c["grid_h"] == px // comp and c["grid_w"] == px // comp
        assert c["text_pad"] + c["grid_h"] * c["grid_w"] == {512: 1280, 1024: 4608}[px]
    # the largest-side config is exactly the largest side the pages allow
    c = CONFIGS["2048px"]
    assert c["grid_h"] * comp == facts["max_side_px"] and c["grid_w"] * comp == facts["max_side_px"]
    # the longest measured config's grid fits the largest side the pages allow
    c = CONFIGS["long"]
    assert max(c["grid_h"], c["grid_w"]) * comp <= facts["max_side_px"]
    assert min(c["grid_h"], c["grid_w"]) * comp >= facts["min_side_px"]
    # the printed section split names 64 rotary pairs: head_dim 128
    sec = tuple(facts["mrope_section"])
    half = sum(sec)
    assert 2 * half == CONFIGS["1024px"]["head_dim"]
    ax = ref.axis_of_pair(sec, half)
    assert [int((ax == a).sum()) for a in range(3)] == list(sec)


# --------------------------------------------------------------------- packed varlen
def _varlen_case():
    from diffusion_transformer_image_head_amd.workloads import make_varlen_workload
    return make_varlen_workload(2, 16, (2, 3, 3), text_lens=(3, 0, 5), grids=((2, 3), (3, 3), (1, 2)),
                                dtype="fp32", seed=60)


def pin_varlen_brute():
    """Packed sequences: each sequence by the scalar loops, on its own."""
    w = _varlen_case()
    out, lse = ref.oracle_fwd_varlen(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.cu_seqlens,
                                     section=w.section)
    cu = w.cu_seqlens
    for b in range(len(cu) - 1):
        a0, a1 = int(cu[b]), int(cu[b + 1])
        bo, bl = brute_fwd(w.q[None, a0:a1].tolist(), w.k[None, a0:a1].tolist(),
                           w.v[None, a0:a1].tolist(), w.pos[None, a0:a1].tolist(),
                           w.gamma_q.tolist(), w.gamma_k.tolist(), None, text_pad=0,
                           section=w.section, theta=w.theta, eps=w.eps)
        assert np.max(np.abs(out[a0:a1] - np.array(bo)[0])) < 1e-12
        assert np.max(np.abs(lse[:, a0:a1] - np.array(bl)[0])) < 1e-12


def pin_varlen_equals_padded_batch():
    """Packing and in-memory padding carry the same per-prompt text length:
    the packed result equals the padded batch's on the real tokens."""
    lens, gh, gw, pad = (3, 0, 6), 2, 3, 6
    from diffusion_transformer_image_head_amd.workloads import make_varlen_workload
    w = make_varlen_workload(2, 16, (2, 3, 3), text_lens=lens, grids=[(gh, gw)] * 3, dtype="fp32",
                             seed=61)
    out, lse = ref.oracle_fwd_varlen(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.cu_seqlens,
                                     section=w.section)
    s = pad + gh * gw
    shp = (3, s, 2, 16)
    qp, kp, vp = np.zeros(shp), np.zeros(shp), np.zeros(shp)
    pp = np.zeros((3, s, 3), dtype=np.int32)
    for b, l in enumerate(lens):
        a0 = int(w.cu_seqlens[b])
        idx = list(range(l)) + list(range(pad, s))        # real slots in the padded item
        for j, t in enumerate(idx):
            qp[b, t], kp[b, t], vp[b, t], pp[b, t] = w.q[a0 + j], w.k[a0 + j], w.v[a0 + j], w.pos[a0 + j]
    po, pl = ref.oracle_fwd(qp, kp, vp, pp, w.gamma_q, w.gamma_k, np.array(lens), text_pad=pad,
                            section=w.section)
    for b, l in enumerate(lens):
        a0 = int(w.cu_seqlens[b])
        idx = list(range(l)) + list(range(pad, s))
        assert np.max(np.abs(po[b, idx] - out[a0:a0 + len(idx)])) < 1e-12
        assert np.max(np.abs(pl[b][:, idx] - lse[:, a0:a0 + len(idx)])) < 1e-12


def pin_varlen_sequences_are_isolated():
    """Changing one sequence leaves every other sequence's output as it was."""
    w = _varlen_case()
    out, _ = ref.oracle_fwd_varlen(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.cu_seqlens,
                                   section=w.section)
    a0, a1 = int(w.cu_seqlens[1]), int(w.cu_seqlens[2])
    k2, v2 = w.k.copy(), w.v.copy()
    k2[a0:a1] += 3.0
    v2[a0:a1] -= 7.0
    out2, _ = ref.oracle_fwd_varlen(w.q, k2, v2, w.pos, w.gamma_q, w.gamma_k, w.cu_seqlens,
                                    section=w.section)
    keep = np.ones(len(w.q), bool)
    keep[a0:a1] = False
    assert np.array_equal(out[keep], out2[keep])
    assert np.max(np.abs(out[~keep] - out2[~keep])) > 1e-3


# --------------------------------------------------------------------- conventions
def pin_interleaved_text_tokens_are_complex_rope():
    """Interleaved pairs (2j, 2j + 1) on a text token (t = h = w = m): each
    pair, read as the complex number x_2j + i x_2j+1, is multiplied by
    exp(i m theta^(-2j/D)) -- the complex form of 1D RoPE, evaluated with
    numpy's complex type -- and equals RoFormer's rotation matrix directly."""
    rng = np.random.default_rng(42)
    for d, sec in ((64, (8, 12, 12)), (128, (16, 24, 24)), (128, (24, 20, 20))):
        for m in (0, 1, 5, 77, 511):
            x = rng.standard_normal(d)
            y = ref.mrope(x[None, None, None, :], np.array([[[m, m, m]]]), sec, 1e4,
                          "interleaved")[0, 0, 0]
            z = x.view(np.complex128) * np.exp(1j * m * 1e4 ** (-np.arange(d // 2) * 2.0 / d))
            assert np.max(np.abs(y - z.view(np.float64))) < 1e-12, (d, sec, m)
            assert np.max(np.abs(y - _rope_1d_roformer(x, float(m), 1e4))) < 1e-12


def pin_interleaved_brute():
    """Scalar loops (complex form, per-row Python) == vectorised oracle with
    interleaved pairs, on a ragged batch with distinct t, h, w positions."""
    w = make_workload(2, 2, 16, (2, 3, 3), 5, 3, 4, text_lens=(2, 5), seed=43, dtype="fp32",
                      rope_pairs="interleaved")
    out, lse = _run(w, rope_pairs="interleaved")
    bo, bl = brute_fwd(w.q.tolist(), w.k.tolist(), w.v.tolist(), w.pos.tolist(),
                       w.gamma_q.tolist(), w.gamma_k.tolist(), w.seq_lens.tolist(),
                       text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps,
                       rope_pairs="interleaved")
    assert np.max(np.abs(out - np.array(bo))) < 1e-12
    fin = np.isfinite(lse)
    assert np.max(np.abs(lse[fin] - np.array(bl)[fin])) < 1e-12
    # and the layout matters: the half-split result differs
    o2, _ = _run(w)
    assert np.max(np.abs(o2 - out)) > 1e-3


def pin_interleaved_is_half_split_of_permuted_dims():
    """Dot products ignore the order of head_dim, and RMSNorm only scales it,
    so interleaved pairs on (q, k, gamma) equal half-split pairs on the same
    tensors with their dims reordered (even dims, then odd dims); v and the
    output are untouched."""
    w = make_workload(2, 3, 32, (4, 6, 6), 6, 3, 4, text_lens=(1, 6), seed=44, dtype="fp32")
    out, lse = _run(w, rope_pairs="interleaved")
    p = np.concatenate([np.arange(0, 32, 2), np.arange(1, 32, 2)])
    o2, l2 = ref.oracle_fwd(w.q[..., p], w.k[..., p], w.v, w.pos, w.gamma_q[p], w.gamma_k[p],
                            w.seq_lens, text_pad=w.text_pad, section=w.section, theta=w.theta,
                            eps=w.eps)
    assert np.max(np.abs(out - o2)) < 1e-12
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(l2)) and np.max(np.abs(lse[fin] - l2[fin])) < 1e-12


def pin_interleaved_relative_positions():
    """Relative encoding holds for interleaved pairs too: shifting both
    tokens' positions per axis leaves q.k, and a change of one axis's
    difference changes it."""
    rng = np.random.default_rng(45)
    d, sec = 128, (16, 24, 24)
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, 1, d))
    dot = lambda pq, pk: float((ref.mrope(q, pq[None, None], sec, 1e4, "interleaved")  # noqa: E731
                                * ref.mrope(k, pk[None, None], sec, 1e4, "interleaved")).sum())
    for _ in range(10):
        pq = rng.integers(0, 600, size=3)
        pk = rng.integers(0, 600, size=3)
        sh = rng.integers(-300, 300, size=3)
        a = dot(pq, pk)
        assert abs(a - dot(pq + sh, pk + sh)) < 1e-10 * (1 + abs(a))
        for ax in range(3):
            pk2 = pk.copy()
            pk2[ax] += 7
            assert abs(dot(pq, pk2) - a) > 1e-6


def pin_per_head_gamma():
    """An [H, D] gamma: head h of the output equals a one-head run on head h
    alone with gamma[h] as its [D] weight; equal rows reproduce the shared
    [D] gamma; the scalar loops agree."""
    w = make_workload(2, 3, 16, (2, 3, 3), 4, 2, 3, text_lens=(1, 4), seed=46, dtype="fp32",
                      gamma_per_head=True)
    assert w.gamma_q.shape == (3, 16)
    for pairs in ("half", "interleaved"):
        out, lse = _run(w, rope_pairs=pairs)
        for h in range(3):
            oh, lh = ref.oracle_fwd(w.q[:, :, h:h + 1], w.k[:, :, h:h + 1], w.v[:, :, h:h + 1],
                                    w.pos, w.gamma_q[h], w.gamma_k[h], w.seq_lens,
                                    text_pad=w.text_pad, section=w.section, rope_pairs=pairs)
            assert np.max(np.abs(out[:, :, h:h + 1] - oh)) < 1e-13
            fin = np.isfinite(lh)
            assert np.max(np.abs(lse[:, h:h + 1][fin] - lh[fin])) < 1e-13
        bo, _ = brute_fwd(w.q.tolist(), w.k.tolist(), w.v.tolist(), w.pos.tolist(),
                          w.gamma_q.tolist(), w.gamma_k.tolist(), w.seq_lens.tolist(),
                          text_pad=w.text_pad, section=w.section, rope_pairs=pairs)
        assert np.max(np.abs(out - np.array(bo))) < 1e-12
    shared = make_workload(2, 3, 16, (2, 3, 3), 4, 2, 3, text_lens=(1, 4), seed=46, dtype="fp32")
    o1, _ = _run(shared)
    shared.gamma_q = np.tile(shared.gamma_q, (3, 1))
    shared.gamma_k = np.tile(shared.gamma_k, (3, 1))
    o2, _ = _run(shared)
    assert np.array_equal(o1, o2)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
