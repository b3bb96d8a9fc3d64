"""GPU parity of the packed variable-length form (cu_seqlens): every
sequence attends within itself, checked against the fp64 oracle, against the
padded form of the same batch, and for rows outside every sequence being left
untouched."""

import numpy as np
import pytest

from diffusion_transformer_image_head_amd.workloads import make_varlen_workload
from oracle.reference import oracle_fwd_varlen
from tests.gpu_util import check_lse, check_parity, errors, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_image_head_amd import binding
    binding.lib()


def to_dev(w):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    return dict(q=t(w.q).to(dt), k=t(w.k).to(dt), v=t(w.v).to(dt), pos=t(w.pos),
                gamma_q=t(w.gamma_q), gamma_k=t(w.gamma_k), cu=t(w.cu_seqlens.astype(np.int32)))


def run_varlen(w, max_seqlen=None, out=None, **kw):
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn_varlen
    d = to_dev(w)
    o, l = mrope_attn_varlen(d["q"], d["k"], d["v"], d["pos"], d["gamma_q"], d["gamma_k"], d["cu"],
                             w.max_seqlen if max_seqlen is None else max_seqlen,
                             section=w.section, return_lse=True, out=out,
                             rope_pairs=w.rope_pairs, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)


def oracle(w):
    return oracle_fwd_varlen(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.cu_seqlens,
                             section=w.section, theta=w.theta, eps=w.eps, rope_pairs=w.rope_pairs)


@pytest.mark.parametrize("kpro", ["prepass", "fused"])
def test_varlen_small_bf16(kpro):
    say(f"case: varlen small bf16 kprologue={kpro}")
    w = make_varlen_workload(3, 128, (16, 24, 24), text_lens=(17, 0, 40, 5),
                             grids=((9, 13), (7, 7), (10, 12), (1, 3)), seed=500)
    out, lse = run_varlen(w, kprologue=kpro)
    ref, rlse = oracle(w)
    check_parity(out, ref, "bf16", f"varlen {w.q.shape} cu={w.cu_seqlens.tolist()}")
    check_lse(lse, rlse)


@pytest.mark.parametrize("kpro", ["prepass", "fused"])
def test_varlen_conventions(kpro):
    say(f"case: varlen gamma per head + interleaved pairs kprologue={kpro}")
    w = make_varlen_workload(3, 128, (16, 24, 24), text_lens=(17, 0, 40), grids=((9, 13), (7, 7), (10, 12)),
                             seed=510, gamma_per_head=True, rope_pairs="interleaved")
    out, lse = run_varlen(w, kprologue=kpro)
    ref, rlse = oracle(w)
    check_parity(out, ref, "bf16", f"varlen conventions cu={w.cu_seqlens.tolist()}")
    check_lse(lse, rlse)


def test_varlen_fp32_and_d64():
    say("case: varlen fp32 d64")
    w = make_varlen_workload(2, 64, (8, 12, 12), text_lens=(3, 12), grids=((4, 5), (6, 3)),
                             dtype="fp32", seed=501)
    out, lse = run_varlen(w)
    ref, rlse = oracle(w)
    check_parity(out, ref, "fp32", "varlen fp32")
    check_lse(lse, rlse, 1e-5)
    wb = make_varlen_workload(2, 64, (8, 12, 12), text_lens=(3, 12), grids=((4, 5), (6, 3)),
                              dtype="bf16", seed=502)
    out, _ = run_varlen(wb)
    check_parity(out, oracle(wb)[0], "bf16", "varlen bf16 d64")


def test_varlen_matches_padded_batch():
    """The packed form and the padded form of the same batch agree."""
    from diffusion_transformer_image_head_amd.workloads import make_workload
    say("case: varlen vs padded batch")
    lens, pad, gh, gw = (37, 128, 0, 90), 128, 12, 11
    w = make_varlen_workload(4, 128, (16, 24, 24), text_lens=lens, grids=[(gh, gw)] * 4, seed=503)
    out, _ = run_varlen(w)
    s = pad + gh * gw
    pw = make_workload(4, 4, 128, (16, 24, 24), pad, gh, gw, text_lens=lens, dtype="bf16", seed=1)
    for b, l in enumerate(lens):
        a0 = int(w.cu_seqlens[b])
        idx = list(range(l)) + list(range(pad, s))
        for f in ("q", "k", "v", "pos"):
            getattr(pw, f)[b, idx] = getattr(w, f)[a0:a0 + len(idx)]
    pw.gamma_q, pw.gamma_k = w.gamma_q, w.gamma_k
    pout, _ = run_gpu(pw)
    for b, l in enumerate(lens):
        a0 = int(w.cu_seqlens[b])
        idx = list(range(l)) + list(range(pad, s))
        ma, rr = errors(out[a0:a0 + len(idx)], pout[b, idx])
        say(f"  item {b}: packed vs padded max_abs={ma:.3e} rel_rms={rr:.3e}")
        assert ma < 2e-2 and rr < 5e-3


def test_varlen_leaves_uncovered_rows_alone():
    import torch
    say("case: varlen uncovered rows")
    w = make_varlen_workload(2, 128, (16, 24, 24), text_lens=(10, 20), grids=((5, 6), (8, 8)),
                             seed=504)
    total = len(w.q)
    w.cu_seqlens = np.array([0, 40, 60], dtype=np.int32)        # rows 60.. belong to no sequence
    sentinel = torch.full((total, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    out, lse = run_varlen(w, max_seqlen=40, out=sentinel)
    ref, rlse = oracle(w)
    check_parity(out[:60], ref[:60], "bf16", "covered rows")
    assert np.all(out[60:] == 3.0)


def test_varlen_ragged_1024px_full():
    """The ragged configuration's four prompts (true text 37/128/300/512 +
    64x64 image each) packed instead of padded: 17,361 tokens. Every output
    and LSE against the per-sequence oracle."""
    say("case: varlen ragged 1024px, all outputs")
    w = make_varlen_workload(32, 128, (16, 24, 24), text_lens=(37, 128, 300, 512),
                             grids=[(64, 64)] * 4, seed=505)
    out, lse = run_varlen(w)
    ref, rlse = oracle(w)
    check_parity(out, ref, "bf16", f"varlen ragged {w.q.shape} cu={w.cu_seqlens.tolist()}")
    check_lse(lse, rlse)


def make_sub(w, b):
    a0, a1 = int(w.cu_seqlens[b]), int(w.cu_seqlens[b + 1])
    return {f: getattr(w, f)[None, a0:a1] for f in ("q", "k", "v", "pos")}
