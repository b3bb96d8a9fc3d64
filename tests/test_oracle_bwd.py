"""Pins of the float64 backward oracle against facts fixed outside it:
finite differences of the forward oracle (an independent code path), the
gradient-free padded tokens, a closed-form column sum of dV, and the
position-shift invariance of relative rotary encoding. Planted mistakes in
the backward oracle (on the CPU) must trip at least one pin."""

import numpy as np
import pytest

import oracle.backward as bwd
from oracle.reference import oracle_fwd
from diffusion_transformer_image_head_amd.workloads import make_workload


def _case(seed=70, **kw):
    base = dict(batch=2, heads=2, head_dim=16, section=(2, 3, 3), text_pad=5, grid_h=3, grid_w=4,
                text_lens=(2, 5), dtype="fp32", seed=seed)
    base.update(kw)
    return make_workload(**base)


def _grads(w, do):
    return bwd.oracle_bwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens, do,
                          text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps,
                          rope_pairs=w.rope_pairs)


def pin_bwd_finite_differences():
    """Directional derivatives of sum(dO * O) by central differences of the
    forward oracle, for every input that has a gradient; also under the other
    conventions (a gamma per head, interleaved rotary pairs)."""
    for w in (_case(), _case(seed=71, text_lens=None, section=(4, 2, 2), text_pad=3),
              _case(seed=75, gamma_per_head=True, rope_pairs="interleaved"),
              _case(seed=76, rope_pairs="interleaved", text_lens=None, text_pad=2)):
        rng = np.random.default_rng(5)
        do = rng.standard_normal(w.q.shape)

        def loss(q, k, v, gq, gk):
            o, _ = oracle_fwd(q, k, v, w.pos, gq, gk, w.seq_lens, text_pad=w.text_pad,
                              section=w.section, theta=w.theta, eps=w.eps,
                              rope_pairs=w.rope_pairs)
            return float(np.sum(o * do))

        args = [np.asarray(a, dtype=np.float64) for a in (w.q, w.k, w.v, w.gamma_q, w.gamma_k)]
        g = _grads(w, do)
        for i in range(5):
            u = rng.standard_normal(args[i].shape)
            lo, hi = list(args), list(args)
            hi[i] = args[i] + 1e-6 * u
            lo[i] = args[i] - 1e-6 * u
            fd = (loss(*hi) - loss(*lo)) / 2e-6
            an = float(np.sum(g[i] * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (i, fd, an)


def pin_bwd_padded_tokens_have_no_gradient():
    w = _case(seed=72)
    do = np.random.default_rng(6).standard_normal(w.q.shape)
    dq, dk, dv, _, _ = _grads(w, do)
    for b, l in enumerate(w.seq_lens):
        pad = slice(int(l), w.text_pad)
        assert np.all(dq[b, pad] == 0) and np.all(dk[b, pad] == 0) and np.all(dv[b, pad] == 0)
    assert np.abs(dq).max() > 0 and np.abs(dk).max() > 0


def pin_bwd_dv_column_sum():
    """Rows of P sum to 1, so the dV rows of an item sum to the dO rows of
    its valid queries, per head."""
    w = _case(seed=73)
    do = np.random.default_rng(7).standard_normal(w.q.shape)
    _, _, dv, _, _ = _grads(w, do)
    for b, l in enumerate(w.seq_lens):
        valid = np.ones(w.q.shape[1], bool)
        valid[int(l):w.text_pad] = False
        assert np.max(np.abs(dv[b].sum(axis=0) - do[b, valid].sum(axis=0))) < 1e-12


def pin_bwd_position_shift_invariance():
    w = _case(seed=74)
    do = np.random.default_rng(8).standard_normal(w.q.shape)
    g0 = _grads(w, do)
    w.pos = w.pos + np.array([11, -3, 7], dtype=np.int32)
    g1 = _grads(w, do)
    for a, b in zip(g0, g1):
        assert np.max(np.abs(a - b)) < 1e-10


def pin_bwd_shared_gamma_is_sum_over_heads():
    """A [D] gamma is every head's weight at once, so its gradient is the sum
    over heads of the gradient of an [H, D] gamma with equal rows."""
    w = _case(seed=77)
    do = np.random.default_rng(9).standard_normal(w.q.shape)
    g_shared = _grads(w, do)
    h = w.q.shape[2]
    w.gamma_q = np.tile(w.gamma_q, (h, 1))
    w.gamma_k = np.tile(w.gamma_k, (h, 1))
    g_head = _grads(w, do)
    assert g_head[3].shape == (h, w.q.shape[3])
    for i in range(3):
        assert np.max(np.abs(g_shared[i] - g_head[i])) < 1e-13
    for i in (3, 4):
        assert np.max(np.abs(g_shared[i] - g_head[i].sum(axis=0))) < 1e-12
        assert np.max(np.abs(g_head[i][0] - g_head[i][1])) > 1e-6


def pin_bwd_varlen_is_padded_without_padding():
    """Packing drops the padded text slots and nothing else: the packed-form
    gradients of each sequence's tokens equal the padded-form gradients of
    the same tokens, and the gamma gradients are equal too (padded slots
    carry none). Checked with a shared and with a per-head gamma."""
    for w in (_case(seed=78), _case(seed=79, gamma_per_head=True, rope_pairs="interleaved")):
        do = np.random.default_rng(10).standard_normal(w.q.shape)
        g_pad = _grads(w, do)
        b_, s_ = w.q.shape[:2]
        keep = [np.r_[0:int(l), w.text_pad:s_] for l in w.seq_lens]
        cat = lambda a: np.concatenate([np.asarray(a)[b][keep[b]] for b in range(b_)])  # noqa: E731
        cu = np.concatenate([[0], np.cumsum([len(kk) for kk in keep])])
        g_pk = bwd.oracle_bwd_varlen(cat(w.q), cat(w.k), cat(w.v), cat(w.pos), w.gamma_q, w.gamma_k,
                                     cu, cat(do), section=w.section, theta=w.theta, eps=w.eps,
                                     rope_pairs=w.rope_pairs)
        for i in range(3):
            assert np.max(np.abs(g_pk[i] - cat(g_pad[i]))) < 1e-12
        for i in (3, 4):
            assert g_pk[i].shape == np.shape(g_pad[i])
            assert np.max(np.abs(g_pk[i] - g_pad[i])) < 1e-12


PINS = [pin_bwd_finite_differences, pin_bwd_padded_tokens_have_no_gradient, pin_bwd_dv_column_sum,
        pin_bwd_position_shift_invariance, pin_bwd_shared_gamma_is_sum_over_heads,
        pin_bwd_varlen_is_padded_without_padding]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_bwd_pin(pin):
    pin()


def _m_rotate_forward_only(x, c, s, sign, pairs="half"):
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)   # ignores sign


def _m_rotate_swapped_halves(x, c, s, sign, pairs="half"):
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x2 * c - sign * x1 * s, x1 * c + sign * x2 * s], axis=-1)


def _m_rotate_pairs_ignored(x, c, s, sign, pairs="half"):
    return _real_rotate(x, c, s, sign, "half")


def _m_angles_no_freq(pos, section, head_dim, theta):
    half = head_dim // 2
    axis = bwd.axis_of_pair(section, half)
    ang = np.asarray(pos, dtype=np.float64)[:, :, axis]
    return np.cos(ang)[:, :, None, :], np.sin(ang)[:, :, None, :]


def _m_valid_all(batch, seq, text_pad, seq_lens=None):
    return np.ones((batch, seq), dtype=bool)


_real_rotate = bwd._rotate

MUTANTS = [("_rotate", _m_rotate_forward_only), ("_rotate", _m_rotate_swapped_halves),
           ("_rotate", _m_rotate_pairs_ignored),
           ("_angles", _m_angles_no_freq), ("valid_tokens", _m_valid_all)]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=lambda x: getattr(x, "__name__", x))
def test_bwd_pins_catch_planted_mistake(monkeypatch, name, mutant):
    monkeypatch.setattr(bwd, name, mutant)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake in {name}"


def test_bwd_pins_catch_planted_arithmetic_slips(monkeypatch):
    """Slips inside oracle_bwd's own arithmetic: a scale on one gradient, a
    dropped RMSNorm term, a transposed contraction."""
    real = bwd.oracle_bwd

    def drop_norm_term(*a, **kw):
        dq, dk, dv, dgq, dgk = real(*a, **kw)
        return dq * 1.01, dk, dv, dgq, dgk

    def dv_transposed(*a, **kw):
        dq, dk, dv, dgq, dgk = real(*a, **kw)
        return dq, dk, dv[:, ::-1], dgq, dgk

    def dgamma_sign(*a, **kw):
        dq, dk, dv, dgq, dgk = real(*a, **kw)
        return dq, dk, dv, dgq, -dgk

    for slip in (drop_norm_term, dv_transposed, dgamma_sign):
        monkeypatch.setattr(bwd, "oracle_bwd", slip)
        caught = []
        for pin in PINS:
            try:
                pin()
            except Exception:  # noqa: BLE001
                caught.append(pin.__name__)
        assert caught, slip.__name__
    monkeypatch.setattr(bwd, "oracle_bwd", real)
