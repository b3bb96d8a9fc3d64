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


def test_bwd_1024px_all_heads():
    """The benchmark's backward as it is timed: the 1024px shape with all 32
    heads, 1152 workgroups per gradient role in one launch (every XCD's share
    of every role) and the shared gammas' 1152 partials; every output
    compared (the oracle loops over the heads, about half a minute)."""
    say("case: bwd 1024px all 32 heads")
    w = config_workload("1024px")
    do = dout_for(w)
    got = run_bwd(w, do)
    say("  gpu done; oracle running")
    ref = oracle_bwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens, do,
                     text_pad=w.text_pad, section=w.section)
    check_bwd(got, ref, "1024px all heads")


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


# ---------------------------------------------------------------- packed sequences
def run_bwd_varlen(w, do, max_seqlen=None, fill=None):
    """GPU packed forward (out, lse) then GPU packed backward; float64
    numpy results. fill: the value dq, dk, dv hold before the call."""
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn_bwd_varlen, mrope_attn_varlen
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    q, k, v = (t(x).to(torch.bfloat16) for x in (w.q, w.k, w.v))
    pos, gq, gk = t(w.pos), t(w.gamma_q), t(w.gamma_k)
    cu = t(np.asarray(w.cu_seqlens, dtype=np.int32))
    ms = w.max_seqlen if max_seqlen is None else max_seqlen
    kw = dict(section=w.section, theta=w.theta, eps=w.eps, rope_pairs=w.rope_pairs)
    out, lse = mrope_attn_varlen(q, k, v, pos, gq, gk, cu, ms, return_lse=True, **kw)
    bufs = {} if fill is None else {n: torch.full_like(q, fill) for n in ("dq", "dk", "dv")}
    g = mrope_attn_bwd_varlen(q, k, v, pos, gq, gk, cu, ms, out, lse, t(do).to(torch.bfloat16), **kw,
                              **bufs)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy().astype(np.float64) for x in g]


def oracle_varlen(w, do):
    from oracle.backward import oracle_bwd_varlen
    return oracle_bwd_varlen(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.cu_seqlens, do,
                             section=w.section, theta=w.theta, eps=w.eps, rope_pairs=w.rope_pairs)


def inside(w):
    cu = np.asarray(w.cu_seqlens)
    m = np.zeros(w.q.shape[0], bool)
    for a0, a1 in zip(cu[:-1], cu[1:]):
        m[a0:a1] = True
    return m


def check_bwd_varlen(got, ref, w, what):
    m = inside(w)
    check_bwd([g[m] for g in got[:3]] + got[3:], [r[m] for r in ref[:3]] + list(ref[3:]), what)


VARLEN = {
    # lengths 134, 49, 160, 8: two 128-row tiles for the longest, so the
    # shorter sequences' second tiles are past their ends
    "mixed": dict(heads=3, text_lens=(17, 0, 40, 5), grids=((9, 13), (7, 7), (10, 12), (1, 3))),
    # 493 and 84 tokens: four tiles for the first
    "multi_tile": dict(heads=2, text_lens=(33, 64), grids=((20, 23), (4, 5))),
}


@pytest.mark.parametrize("name", list(VARLEN))
def test_bwd_varlen(name):
    from diffusion_transformer_image_head_amd.workloads import make_varlen_workload
    c = VARLEN[name]
    w = make_varlen_workload(c["heads"], 128, (16, 24, 24), c["text_lens"], c["grids"],
                             seed=760 + list(VARLEN).index(name))
    say(f"case: bwd varlen {name} cu={w.cu_seqlens.tolist()}")
    do = dout_for(w)
    check_bwd_varlen(run_bwd_varlen(w, do), oracle_varlen(w, do), w, f"varlen {name}")


def test_bwd_varlen_gaps_empty_and_long_max():
    """Tokens before, between (none) and after the sequences belong to no
    sequence, one sequence is empty, and max_seqlen is the whole slice (many
    tiles past every sequence's end): the sequences' gradients match the
    oracle and the outside rows keep what dq, dk, dv held."""
    from diffusion_transformer_image_head_amd.workloads import make_varlen_workload
    w = make_varlen_workload(2, 128, (16, 24, 24), (9, 30), ((5, 7), (8, 8)), seed=770)
    rng = np.random.default_rng(771)
    t0, t1 = 5, 7                                       # tokens outside, before and after
    grow = lambda a: np.concatenate([round_to_bf16(rng.standard_normal((t0,) + a.shape[1:]).astype(np.float32)),  # noqa: E731
                                     a, round_to_bf16(rng.standard_normal((t1,) + a.shape[1:]).astype(np.float32))])
    w.q, w.k, w.v = grow(w.q), grow(w.k), grow(w.v)
    w.pos = np.concatenate([np.zeros((t0, 3), np.int32), w.pos, np.zeros((t1, 3), np.int32)])
    cu = np.asarray(w.cu_seqlens) + t0
    w.cu_seqlens = np.insert(cu, 1, cu[1]).astype(np.int32)    # an empty second sequence
    say(f"case: bwd varlen gaps cu={w.cu_seqlens.tolist()} T={w.q.shape[0]}")
    do = dout_for(w)
    got = run_bwd_varlen(w, do, max_seqlen=w.q.shape[0], fill=7.0)
    check_bwd_varlen(got, oracle_varlen(w, do), w, "varlen gaps")
    out_rows = ~inside(w)
    assert out_rows.sum() == t0 + t1
    for g in got[:3]:
        assert np.all(g[out_rows] == 7.0)


@pytest.mark.parametrize("per_head,pairs", [(True, "interleaved"), (False, "interleaved"), (True, "half")])
def test_bwd_varlen_conventions(per_head, pairs):
    from diffusion_transformer_image_head_amd.workloads import make_varlen_workload
    w = make_varlen_workload(3, 128, (16, 24, 24), (17, 40), ((9, 13), (6, 7)), seed=780,
                             gamma_per_head=per_head, rope_pairs=pairs)
    say(f"case: bwd varlen gamma_per_head={per_head} rope_pairs={pairs}")
    do = dout_for(w)
    got = run_bwd_varlen(w, do)
    ref = oracle_varlen(w, do)
    assert got[3].shape == ref[3].shape
    check_bwd_varlen(got, ref, w, f"varlen {per_head} {pairs}")
