"""Pins of the fp8 QKV projection oracle: the e4m3 decoder against the
library's float8_e4m3fn, the projection against scalar loops, and the
composition with the attention oracle."""

import numpy as np
import pytest

import oracle.qkv as qkv
from oracle.reference import mrope, oracle_fwd, rms_norm


def test_e4m3_decoder_matches_the_library_type():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = qkv.e4m3_decode(codes)
    fin = np.isfinite(want)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[fin], want[fin])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9      # largest normal, smallest subnormal


def _case(seed=0, m=7, hidden=16, heads=2, d=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, hidden))
    w8 = rng.integers(0, 256, size=(3 * heads * d, hidden), dtype=np.uint8)
    w8[(w8 & 0x7F) == 0x7F] = 0x38                            # no NaN codes
    sc = rng.uniform(0.01, 0.1, 3 * heads * d)
    pos = rng.integers(0, 20, size=(m, 3)).astype(np.int32)
    gq, gk = rng.uniform(0.5, 1.5, d), rng.uniform(0.5, 1.5, d)
    return x, w8, sc, pos, gq, gk


def test_projection_against_scalar_loops():
    x, w8, sc, pos, gq, gk = _case()
    m, hidden = x.shape
    heads, d = 2, 8
    q, k, v = qkv.oracle_qkv_proj(x, w8, sc, pos, gq, gk, heads=heads, head_dim=d, section=(2, 1, 1),
                                  qscale=0.7)
    table = qkv.e4m3_decode(np.arange(256, dtype=np.uint8))
    y = np.zeros((m, 3 * heads * d))
    for t in range(m):
        for o in range(3 * heads * d):
            acc = 0.0
            for i in range(hidden):
                acc += x[t, i] * table[w8[o, i]]
            y[t, o] = acc * sc[o]
    hd = heads * d
    assert np.max(np.abs(v - y[:, 2 * hd:].reshape(m, heads, d))) < 1e-12
    qr = y[:, :hd].reshape(1, m, heads, d)
    kr = y[:, hd:2 * hd].reshape(1, m, heads, d)
    assert np.max(np.abs(q - 0.7 * mrope(rms_norm(qr, gq, 1e-6), pos[None], (2, 1, 1), 1e4)[0])) < 1e-12
    assert np.max(np.abs(k - mrope(rms_norm(kr, gk, 1e-6), pos[None], (2, 1, 1), 1e4)[0])) < 1e-12


@pytest.mark.parametrize("per_head,pairs", [(False, "half"), (True, "interleaved")])
def test_rows_subset_and_composition_with_attention(per_head, pairs):
    x, w8, sc, pos, gq, gk = _case(seed=1, m=9, hidden=32, heads=2, d=16)
    if per_head:
        rng = np.random.default_rng(3)
        gq = rng.uniform(0.5, 1.5, (2, 16))
        gk = rng.uniform(0.5, 1.5, (2, 16))
    full = qkv.oracle_qkv_proj(x, w8, sc, pos, gq, gk, heads=2, head_dim=16, section=(2, 3, 3),
                               rope_pairs=pairs)
    sub = qkv.oracle_qkv_proj(x, w8, sc, pos, gq, gk, heads=2, head_dim=16, section=(2, 3, 3),
                              rows=[2, 5], rope_pairs=pairs)
    for a, b in zip(full, sub):
        assert np.max(np.abs(a[[2, 5]] - b)) < 1e-12
    # q_op / k_op are exactly the attention oracle's rotated operands: attention
    # on the raw projections equals softmax over q_op . k_op
    w = qkv.e4m3_decode(w8) * sc[:, None]
    y = x @ w.T
    q, k, v = (y[:, i * 32:(i + 1) * 32].reshape(1, 9, 2, 16) for i in range(3))
    out, _ = oracle_fwd(q, k, v, pos[None], gq, gk, None, text_pad=0, section=(2, 3, 3),
                        rope_pairs=pairs)
    qo, ko, vo = full
    z = np.einsum("qhd,khd->hqk", qo, ko) / 4.0
    p = np.exp(z - z.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    o2 = np.einsum("hqk,khd->qhd", p, vo)
    assert np.max(np.abs(out[0] - o2)) < 1e-12
