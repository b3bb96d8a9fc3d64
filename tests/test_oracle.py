"""The fp64 oracle against its pins, and the pins against planted mistakes.

CPU only. A planted mistake is a broken copy of one oracle function swapped
in for the duration of one check; every such mutant must trip at least one
pin, which shows the pins would catch that slip in the oracle itself.
"""

import numpy as np
import pytest

import oracle.reference as ref
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


_orig = {n: getattr(ref, n) for n in ("rms_norm", "mrope", "axis_of_pair", "inv_freq",
                                       "attention", "valid_tokens")}


def _m_no_gamma(x, gamma, eps):
    return _orig["rms_norm"](x, np.ones_like(np.asarray(gamma, dtype=np.float64)), eps)


def _m_sum_not_mean(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * gamma


def _m_eps_outside(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + 1e-2) * gamma





def _flip(x, pos, section, theta, pairs="half"):
    # rotation with the sine terms' signs swapped (x'_j = x_j c + x_{j+h} s, ...)
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[:, :, ref.axis_of_pair(section, h)] * ref.inv_freq(d, theta)
    c = np.cos(ang)[:, :, None, :]
    s = np.sin(ang)[:, :, None, :]
    y = np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., h:] * c + x[..., :h] * s], -1)
    return y if pairs == "half" else _orig["mrope"](x, pos, section, theta, pairs)


def _m_interleaved(x, pos, section, theta, pairs="half"):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    perm = np.empty(d, dtype=np.int64)
    perm[0::2] = np.arange(h)
    perm[1::2] = np.arange(h) + h
    inv = np.argsort(perm)
    return _orig["mrope"](x[..., inv], pos, section, theta)[..., perm]


def _m_pairs_ignored(x, pos, section, theta, pairs="half"):
    # the layout argument dropped: interleaved requests get half-split pairs
    return _orig["mrope"](x, pos, section, theta)


def _m_interleaved_swapped(x, pos, section, theta, pairs="half"):
    # interleaved pairs read as (2j + 1, 2j): the rotation runs backwards
    if pairs != "interleaved":
        return _orig["mrope"](x, pos, section, theta, pairs)
    x = np.asarray(x, dtype=np.float64)
    sw = np.arange(x.shape[-1]) ^ 1
    return _orig["mrope"](x[..., sw], pos, section, theta, pairs)[..., sw]


def _m_gamma_head0(x, gamma, eps):
    # a per-head gamma collapsed to its first row
    g = np.asarray(gamma, dtype=np.float64)
    return _orig["rms_norm"](x, g[0] if g.ndim == 2 else g, eps)


def _m_axis_order(section, half):
    return 2 - _orig["axis_of_pair"](tuple(reversed(tuple(section))), half)


def _m_axis_all_t(section, half):
    return np.zeros(half, dtype=np.int64)


def _m_freq(head_dim, theta):
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -j / head_dim)


def _m_no_scale(qr, kr, v, valid, scale, rows=None, heads=None):
    return _orig["attention"](qr, kr, v, valid, 1.0, rows, heads)


def _m_transposed(qr, kr, v, valid, scale, rows=None, heads=None):
    return _orig["attention"](kr, qr, v, valid, scale, rows, heads)


def _m_no_zero_rows(qr, kr, v, valid, scale, rows=None, heads=None):
    ones = np.ones_like(valid)
    out, lse = _orig["attention"](qr, kr, v, valid, scale, rows, heads)
    o2, l2 = _orig["attention"](qr, kr, v, ones, scale, rows, heads)
    rr = slice(None) if rows is None else rows
    inval = ~valid[:, rr]
    out[inval] = o2[inval]
    return out, lse


def _m_mask_off_by_one(batch, seq, text_pad, seq_lens=None):
    v = _orig["valid_tokens"](batch, seq, text_pad, seq_lens)
    if seq_lens is None:
        return v
    s = np.arange(seq)[None, :]
    lens = np.clip(np.asarray(seq_lens), 0, text_pad)[:, None]
    return (s >= text_pad) | (s <= lens)


def _m_no_mask(batch, seq, text_pad, seq_lens=None):
    return np.ones((batch, seq), dtype=bool)


MUTANTS = [
    ("rms_norm", _m_no_gamma), ("rms_norm", _m_sum_not_mean), ("rms_norm", _m_eps_outside),
    ("mrope", _flip), ("mrope", _m_interleaved), ("mrope", _m_pairs_ignored),
    ("mrope", _m_interleaved_swapped), ("rms_norm", _m_gamma_head0),
    ("axis_of_pair", _m_axis_order), ("axis_of_pair", _m_axis_all_t),
    ("inv_freq", _m_freq),
    ("attention", _m_no_scale), ("attention", _m_transposed), ("attention", _m_no_zero_rows),
    ("valid_tokens", _m_mask_off_by_one), ("valid_tokens", _m_no_mask),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=lambda x: getattr(x, "__name__", x))
def test_pins_catch_planted_mistake(monkeypatch, name, mutant):
    monkeypatch.setattr(ref, name, mutant)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake in {name}"
