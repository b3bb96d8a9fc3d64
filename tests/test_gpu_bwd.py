"""GPU parity of the backward pass (dq, dk, dv, dgamma_q, dgamma_k) against
the fp64 backward oracle, with the bars of tests/test_tolerance.py (derived
from an emulation of where the kernels round)."""

import numpy as np
import pytest

from diffusion_transformer_image_head_amd.workloads import config_workload, make_workload, round_to_bf16
from oracle.backward import oracle_bwd
from tests.gpu_util import say, to_dev
from tests.test_tolerance import BWD_BARS, bwd_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_image_head_amd import binding
    binding.lib()


def dout_for(w, seed=3):
    return round_to_bf16(np.random.default_rng(seed).standard_normal(w.q.shape).astype(np.float32))


def run_bwd(w, do, dev=None):
    """GPU forward (for out and lse) then GPU backward; float64 numpy results."""
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn, mrope_attn_bwd
    dev = dev or to_dev(w)
    kw = dict(text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps,
              rope_pairs=w.rope_pairs)
    out, lse = mrope_attn(dev["q"], dev["k"], dev["v"], dev["pos"], dev["gamma_q"], dev["gamma_k"],
                          dev["seq_lens"], return_lse=True, **kw)
    dot = torch.from_numpy(do).cuda().to(torch.bfloat16)
    g = mrope_attn_bwd(dev["q"], dev["k"], dev["v"], dev["pos"], dev["gamma_q"], dev["gamma_k"],
                       dev["seq_lens"], out, lse, dot, **kw)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in g]


def check_bwd(got, ref, what):
    for name, a, r in zip(("dq", "dk", "dv", "dgamma_q", "dgamma_k"), got, ref):
        ma, rr = bwd_errors(a, r)
        say(f"  {what} {name}: max_abs/max={ma:.3e} rel_rms={rr:.3e} (bars {BWD_BARS})")
        assert np.isfinite(a).all(), name
        assert ma <= BWD_BARS[0] and rr <= BWD_BARS[1], (name, ma, rr)


SMALL = {
    "s88": dict(batch=1, heads=2, head_dim=128, section=(16, 24, 24), text_pad=16, grid_h=8, grid_w=9),
    "ragged157": dict(batch=2, heads=3, head_dim=128, section=(16, 24, 24), text_pad=40, grid_h=9,
                      grid_w=13, text_lens=(17, 40)),
    "multi_tile": dict(batch=1, heads=2, head_dim=128, section=(16, 24, 24), text_pad=64, grid_h=20,
                       grid_w=23, text_lens=(33,)),
    "all_pad_text": dict(batch=3, heads=2, head_dim=128, section=(16, 24, 24), text_pad=200, grid_h=6,
                         grid_w=6, text_lens=(0, 1, 199)),
    "sec242020": dict(batch=1, heads=2, head_dim=128, section=(24, 20, 20), text_pad=30, grid_h=10,
                      grid_w=10),
    "s1": dict(batch=1, heads=1, head_dim=128, section=(16, 24, 24), text_pad=1, grid_h=0, grid_w=0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_bwd_small(name):
    say(f"case: bwd small {name}")
    w = make_workload(**SMALL[name], dtype="bf16", seed=700 + list(SMALL).index(name))
    do = dout_for(w)
    got = run_bwd(w, do)
    ref = oracle_bwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens, do,
                     text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps)
    if name == "s1":   # one token: P = 1, dS = 0, so dq, dk and the gammas are exactly 0
        assert all(np.all(got[i] == 0) for i in (0, 1, 3, 4))
        assert np.max(np.abs(got[2] - ref[2])) <= 1e-2 * np.abs(ref[2]).max()
        return
    check_bwd(got, ref, name)
    if w.seq_lens is not None:
        for b, l in enumerate(w.seq_lens):
            for t in got[:3]:
                assert np.all(t[b, int(l):w.text_pad] == 0)


@pytest.mark.parametrize("per_head,pairs", [(True, "half"), (False, "interleaved"),
                                            (True, "interleaved")])
@pytest.mark.parametrize("name", ["ragged157", "multi_tile"])
def test_bwd_conventions(name, per_head, pairs):
    """A gamma per head (its gradient per head, [H, D]) and interleaved
    rotary pairs, every output compared with the oracle."""
    say(f"case: bwd {name} gamma_per_head={per_head} rope_pairs={pairs}")
    w = make_workload(**SMALL[name], dtype="bf16", seed=730 + list(SMALL).index(name),
                      gamma_per_head=per_head, rope_pairs=pairs)
    do = dout_for(w)
    got = run_bwd(w, do)
    ref = oracle_bwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens, do,
                     text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps,
                     rope_pairs=pairs)
    assert got[3].shape == ref[3].shape and got[4].shape == ref[4].shape
    check_bwd(got, ref, f"{name} {per_head} {pairs}")


def test_bwd_poisoned_padding_is_invisible():
    say("case: bwd poisoned padding")
    w = make_workload(3, 2, 128, (16, 24, 24), 70, 9, 9, text_lens=(0, 31, 70), dtype="bf16", seed=720)
    do = dout_for(w)
    clean = run_bwd(w, do)
    for b, l in enumerate(w.seq_lens):
        for f in ("q", "k", "v"):
            getattr(w, f)[b, l:w.text_pad] = np.nan
        do[b, l:w.text_pad] = np.nan
    dirty = run_bwd(w, do)
    for a, b in zip(clean, dirty):
        assert np.array_equal(a, b)


def test_bwd_is_deterministic():
    say("case: bwd determinism")
    w = make_workload(**SMALL["multi_tile"], dtype="bf16", seed=721)
    do = dout_for(w)
    a, b = run_bwd(w, do), run_bwd(w, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_1024px_two_heads():
    """The 1024px shape (512 text slots + 64x64 image) on two of its heads:
    heads are independent, so this is the full-size problem for them."""
    say("case: bwd 1024px two heads")
    w = config_workload("1024px")
    for f in ("q", "k", "v"):
        setattr(w, f, np.ascontiguousarray(getattr(w, f)[:, :, [0, 17]]))
    do = dout_for(w)
    got = run_bwd(w, do)
    ref = oracle_bwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens, do,
                     text_pad=w.text_pad, section=w.section)
    check_bwd(got, ref, "1024px heads 0,17")


def test_bwd_ragged_items():
    """Ragged true text lengths at a mid-size shape, every output compared."""
    say("case: bwd ragged mid-size")
    w = make_workload(4, 4, 128, (16, 24, 24), 128, 16, 20, text_lens=(1, 37, 100, 128), dtype="bf16",
                      seed=722)
    do = dout_for(w)
    got = run_bwd(w, do)
    ref = oracle_bwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens, do,
                     text_pad=w.text_pad, section=w.section)
    check_bwd(got, ref, "ragged 4x448")


def test_bwd_fused_qkv_views():
    """q, k, v as strided views of one [B, S, 3, H, D] projection output, and
    dq, dk, dv written into the matching views of one gradient buffer (the
    layout a fused qkv projection's backward consumes): equal to the
    contiguous call, bit for bit."""
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn, mrope_attn_bwd
    say("case: bwd on fused qkv views")
    w = make_workload(**SMALL["ragged157"], dtype="bf16", seed=740)
    dev = to_dev(w)
    do = torch.from_numpy(dout_for(w)).cuda().to(torch.bfloat16)
    kw = dict(text_pad=w.text_pad, section=w.section)
    qkv = torch.stack([dev["q"], dev["k"], dev["v"]], dim=2)            # [B, S, 3, H, D]
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    out, lse = mrope_attn(q, k, v, dev["pos"], dev["gamma_q"], dev["gamma_k"], dev["seq_lens"],
                          return_lse=True, **kw)
    grad = torch.full_like(qkv, float("nan"))
    g1 = mrope_attn_bwd(q, k, v, dev["pos"], dev["gamma_q"], dev["gamma_k"], dev["seq_lens"], out,
                        lse, do, dq=grad[:, :, 0], dk=grad[:, :, 1], dv=grad[:, :, 2], **kw)
    out2, lse2 = mrope_attn(dev["q"], dev["k"], dev["v"], dev["pos"], dev["gamma_q"], dev["gamma_k"],
                            dev["seq_lens"], return_lse=True, **kw)
    g2 = mrope_attn_bwd(dev["q"], dev["k"], dev["v"], dev["pos"], dev["gamma_q"], dev["gamma_k"],
                        dev["seq_lens"], out2, lse2, do, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    for a, b in zip((grad[:, :, 0], grad[:, :, 1], grad[:, :, 2], g1[3], g1[4]), (g2[0], g2[1], g2[2], g2[3], g2[4])):
        assert torch.equal(a, b)
