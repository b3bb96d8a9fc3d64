"""GPU parity of the fp8 e4m3 QKV projection with its norm/rotation
epilogue, and of the attention on the operands it writes (kprologue="none"),
against the fp64 oracles."""

import numpy as np
import pytest

from diffusion_transformer_image_head_amd.workloads import make_qkv_workload
from oracle.qkv import e4m3_decode, oracle_qkv_proj
from oracle.reference import oracle_fwd
from tests.gpu_util import check_parity, say

pytestmark = pytest.mark.gpu

# projection outputs are rounded once to bf16 (relative error <= 2^-9 each):
# max-abs relative to the largest magnitude, and rel-RMS
QKV_BARS = (1e-2, 4e-3)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_image_head_amd import binding
    binding.lib()


def to_dev(w):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    return dict(x=t(w.x).to(torch.bfloat16), w8=t(w.w8), w_scale=t(w.w_scale), pos=t(w.pos),
                gamma_q=t(w.gamma_q), gamma_k=t(w.gamma_k))


def run_proj(w):
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_qkv_proj
    d = to_dev(w)
    outs = mrope_qkv_proj(d["x"], d["w8"], d["w_scale"], d["pos"], d["gamma_q"], d["gamma_k"],
                          heads=w.heads, section=w.section, rope_pairs=w.rope_pairs)
    torch.cuda.synchronize()
    return outs, [o.float().cpu().numpy().astype(np.float64) for o in outs]


def qscale(d=128):
    return float(np.float32(np.float32(1.0 / np.sqrt(d)) * 1.4426950408889634))


def check_proj(got, ref, what):
    for name, a, r in zip(("q_op", "k_op", "v"), got, ref):
        d = a - r
        ma = float(np.abs(d).max()) / float(np.abs(r).max())
        rr = float(np.sqrt((d * d).sum() / (r * r).sum()))
        say(f"  {what} {name}: max_abs/max={ma:.3e} rel_rms={rr:.3e} (bars {QKV_BARS})")
        assert np.isfinite(a).all()
        assert ma <= QKV_BARS[0] and rr <= QKV_BARS[1], (name, ma, rr)


@pytest.mark.parametrize("shape", [(1, 2, 30, 9, 13, 256), (2, 3, 40, 5, 7, 128), (1, 1, 1, 0, 0, 64)])
def test_qkv_small(shape):
    b, h, tp, gh, gw, hidden = shape
    say(f"case: qkv small {shape}")
    w = make_qkv_workload(b, h, 128, (16, 24, 24), tp, gh, gw, hidden, seed=800 + hidden)
    _, got = run_proj(w)
    ref = oracle_qkv_proj(w.x, w.w8, w.w_scale, w.pos, w.gamma_q, w.gamma_k, heads=h, head_dim=128,
                          section=w.section, qscale=qscale())
    check_proj(got, ref, f"{shape}")


@pytest.mark.parametrize("per_head,pairs", [(True, "half"), (False, "interleaved"),
                                            (True, "interleaved")])
def test_qkv_conventions(per_head, pairs):
    say(f"case: qkv gamma_per_head={per_head} rope_pairs={pairs}")
    w = make_qkv_workload(2, 3, 128, (16, 24, 24), 40, 5, 7, 128, seed=830, gamma_per_head=per_head,
                          rope_pairs=pairs)
    _, got = run_proj(w)
    ref = oracle_qkv_proj(w.x, w.w8, w.w_scale, w.pos, w.gamma_q, w.gamma_k, heads=3, head_dim=128,
                          section=w.section, qscale=qscale(), rope_pairs=pairs)
    check_proj(got, ref, f"{per_head} {pairs}")


def test_qkv_1024px_sampled_rows():
    """The 1024px layout (4608 tokens), hidden 4096 = 32 heads x 128."""
    say("case: qkv 1024px sampled rows")
    w = make_qkv_workload(1, 32, 128, (16, 24, 24), 512, 64, 64, 4096, seed=810)
    _, got = run_proj(w)
    rows = np.array(sorted({0, 1, 255, 256, 511, 512, 4095, 4096, 4159, 4160, 4606, 4607} |
                           set(np.random.default_rng(0).choice(4608, 40, replace=False).tolist())))
    ref = oracle_qkv_proj(w.x, w.w8, w.w_scale, w.pos, w.gamma_q, w.gamma_k, heads=32, head_dim=128,
                          section=w.section, qscale=qscale(), rows=rows)
    check_proj([g[rows] for g in got], ref, "1024px rows")


def test_qkv_more_than_one_round():
    """32 heads (48 head pairs), 1380 tokens: 11 token tiles of 128 (the last
    ragged, 100 tokens) make 528 workgroups, past one round of the 512
    resident slots. Every element is checked."""
    say("case: qkv more than one round of workgroups (1380 tokens, 32 heads)")
    w = make_qkv_workload(1, 32, 128, (16, 24, 24), 8, 28, 49, 256, seed=840)
    assert w.x.shape[0] == 1380
    _, got = run_proj(w)
    ref = oracle_qkv_proj(w.x, w.w8, w.w_scale, w.pos, w.gamma_q, w.gamma_k, heads=32, head_dim=128,
                          section=w.section, qscale=qscale())
    check_proj(got, ref, "1380 tokens")


def test_projection_then_attention_end_to_end():
    """x -> fp8 projection + epilogue -> attention on the given operands,
    against the oracle attention on the exact projections."""
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn
    say("case: qkv -> attention end to end")
    b, h, tp, gh, gw, hidden = 2, 2, 40, 9, 11, 256
    lens = np.array([17, 40], dtype=np.int32)
    w = make_qkv_workload(b, h, 128, (16, 24, 24), tp, gh, gw, hidden, seed=820)
    outs, _ = run_proj(w)
    s = w.seq
    q, k, v = (o.view(b, s, h, 128) for o in outs)
    sl = torch.from_numpy(lens).cuda()
    out, lse = mrope_attn(q, k, v, None, None, None, sl, text_pad=tp, kprologue="none", return_lse=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    wt = e4m3_decode(w.w8) * w.w_scale.astype(np.float64)[:, None]
    y = w.x.astype(np.float64) @ wt.T
    hd = h * 128
    qr, kr, vr = (y[:, i * hd:(i + 1) * hd].reshape(b, s, h, 128) for i in range(3))
    ref, rlse = oracle_fwd(qr, kr, vr, w.pos.reshape(b, s, 3), w.gamma_q, w.gamma_k, lens,
                           text_pad=tp, section=w.section)
    check_parity(got, ref, "bf16", "end to end")
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(lse.cpu().numpy()))
    for bi, l in enumerate(lens):
        assert np.all(got[bi, l:tp] == 0)
