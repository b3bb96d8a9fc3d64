"""GPU parity of the grouped launch (several problems in one attention
launch): every member against the fp64 oracle, and against its own plain
call. The canonical group is one guided sampling step: the conditional pass
over [text + image] tokens and the unconditional pass over the image tokens
alone (text_pad = 0)."""

import numpy as np
import pytest

from diffusion_transformer_image_head_amd.workloads import config_workload, make_workload
from tests.gpu_util import check_lse, check_parity, run_gpu, run_oracle, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_image_head_amd import binding
    binding.lib()


def run_group(ws, **kw):
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn_group
    probs = []
    for w in ws:
        d = to_dev(w)
        probs.append(dict(d, text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps,
                          rope_pairs=w.rope_pairs))
    res = mrope_attn_group(probs, return_lse=True, **kw)
    torch.cuda.synchronize()
    return [(o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64))
            for o, l in res]


def cfg_pair(batch, heads, head_dim, section, text_pad, gh, gw, text_lens, seed):
    """Conditional [text + image] and unconditional [image only] workloads of
    one step: the unconditional pass sees the same image tokens (same
    positions) and no text."""
    cond = make_workload(batch, heads, head_dim, section, text_pad, gh, gw, text_lens=text_lens,
                         dtype="bf16", seed=seed)
    unc = make_workload(batch, heads, head_dim, section, 0, gh, gw, dtype="bf16", seed=seed + 1)
    unc.pos = np.ascontiguousarray(cond.pos[:, text_pad:])
    return cond, unc


@pytest.mark.parametrize("kpro", ["prepass", "fused"])
def test_cfg_pair_small(kpro):
    say(f"case: group cfg pair small kprologue={kpro}")
    cond, unc = cfg_pair(2, 3, 128, (16, 24, 24), 40, 9, 13, (17, 40), seed=400)
    got = run_group([cond, unc], kprologue=kpro)
    for w, (out, lse), name in zip((cond, unc), got, ("cond", "uncond")):
        ref, rlse = run_oracle(w)
        check_parity(out, ref, "bf16", f"{name} {w.shape}")
        check_lse(lse, rlse)
        alone, _ = run_gpu(w, kprologue=kpro)
        assert np.max(np.abs(out - alone)) < 2e-2


def test_group_of_four_mixed_shapes():
    say("case: group of four mixed shapes")
    ws = [
        make_workload(1, 2, 128, (16, 24, 24), 30, 10, 10, text_lens=(11,), dtype="bf16", seed=410),
        make_workload(2, 4, 128, (24, 20, 20), 0, 7, 9, dtype="bf16", seed=411),
        make_workload(1, 1, 128, (16, 24, 24), 200, 6, 6, text_lens=(0,), dtype="bf16", seed=412),
        make_workload(3, 2, 128, (16, 24, 24), 64, 20, 23, text_lens=(1, 33, 64), dtype="bf16",
                      seed=413),
    ]
    got = run_group(ws)
    for i, (w, (out, lse)) in enumerate(zip(ws, got)):
        ref, rlse = run_oracle(w)
        check_parity(out, ref, "bf16", f"member {i} {w.shape}")
        check_lse(lse, rlse)
        if w.seq_lens is not None:
            for b, l in enumerate(w.seq_lens):
                assert np.all(out[b, int(l):w.text_pad] == 0)


@pytest.mark.parametrize("kpro", ["prepass", "fused"])
def test_group_mixed_conventions(kpro):
    """Members with different conventions in one launch: each keeps its own
    gamma shape and rotary pair layout."""
    say(f"case: group mixed conventions kprologue={kpro}")
    ws = [
        make_workload(2, 3, 128, (16, 24, 24), 40, 9, 13, text_lens=(17, 40), dtype="bf16", seed=440,
                      gamma_per_head=True, rope_pairs="interleaved"),
        make_workload(1, 2, 128, (16, 24, 24), 0, 10, 11, dtype="bf16", seed=441),
        make_workload(1, 4, 128, (24, 20, 20), 30, 8, 8, text_lens=(9,), dtype="bf16", seed=442,
                      rope_pairs="interleaved"),
    ]
    got = run_group(ws, kprologue=kpro)
    for i, (w, (out, lse)) in enumerate(zip(ws, got)):
        ref, rlse = run_oracle(w)
        check_parity(out, ref, "bf16", f"member {i} {w.shape} {w.rope_pairs}")
        check_lse(lse, rlse)


def test_group_d64_and_empty_member():
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn_group
    say("case: group d64 with an empty member")
    w = make_workload(1, 2, 64, (8, 12, 12), 10, 12, 12, dtype="bf16", seed=420)
    d = to_dev(w)
    z = torch.zeros(0, 16, 2, 64, dtype=torch.bfloat16, device="cuda")
    empty = dict(q=z, k=z, v=z, pos=torch.zeros(0, 16, 3, dtype=torch.int32, device="cuda"),
                 gamma_q=d["gamma_q"], gamma_k=d["gamma_k"], text_pad=4, section=(8, 12, 12))
    outs = mrope_attn_group([empty, dict(d, text_pad=w.text_pad, section=w.section)])
    torch.cuda.synchronize()
    assert outs[0].shape == z.shape
    ref, _ = run_oracle(w)
    check_parity(outs[1].float().cpu().numpy().astype(np.float64), ref, "bf16", "d64 member")


def test_fp32_group():
    say("case: fp32 group")
    ws = [config_workload("tiny"),
          make_workload(1, 2, 64, (8, 12, 12), 0, 5, 6, dtype="fp32", seed=430)]
    for w, (out, lse) in zip(ws, run_group(ws)):
        ref, rlse = run_oracle(w)
        check_parity(out, ref, "fp32", f"fp32 member {w.shape}")
        check_lse(lse, rlse, 1e-5)


def test_cfg_pair_1024px_full():
    """The full-size step: 1024px conditional (512 text slots + 64x64 image)
    and its image-only unconditional pass in one launch. Every output and
    LSE of both members against the oracle."""
    say("case: group cfg pair 1024px, all outputs")
    cond = config_workload("1024px")
    unc = make_workload(1, 32, 128, (16, 24, 24), 0, 64, 64, dtype="bf16", seed=21)
    unc.pos = np.ascontiguousarray(cond.pos[:, cond.text_pad:])
    got = run_group([cond, unc])
    for w, (out, lse), name in zip((cond, unc), got, ("cond", "uncond")):
        ref, rlse = run_oracle(w)
        check_parity(out, ref, "bf16", f"{name} all outputs")
        check_lse(lse, rlse)
