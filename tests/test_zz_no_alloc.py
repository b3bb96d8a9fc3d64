"""The forward without allocation (mrope_attn_fwd_noalloc, for callers that
cannot allocate: graph capture, serving loops) against the plain forward with
a caller workspace (mrope_attn_fwd), through the C ABI.

Both run the same kernels, so outputs and LSE must be bitwise equal. The
calls come in a row with the second one smaller, so the library's scratch
array still holds the first call's (larger) intermediates when the second
runs; outputs are pre-filled with NaN so an unwritten element shows. Each
case is also held to the oracle's parity bar.
"""

import numpy as np
import pytest

from diffusion_transformer_image_head_amd.workloads import config_workload, make_workload
from tests.gpu_util import check_lse, check_parity, run_oracle, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_image_head_amd import binding
    binding.lib()  # fail loudly if the HIP library is missing


def _run_both(w):
    """(noalloc out, noalloc lse, plain out, plain lse) as torch tensors."""
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn, mrope_attn_noalloc
    dev = to_dev(w)
    kw = dict(text_pad=w.text_pad, section=w.section, theta=w.theta, eps=w.eps, rope_pairs=w.rope_pairs)
    b, s, h, _ = w.q.shape
    out = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((b, h, s), float("nan"), dtype=torch.float32, device=dev["q"].device)
    mrope_attn_noalloc(dev["q"], dev["k"], dev["v"], dev["pos"], dev["gamma_q"], dev["gamma_k"],
                       dev["seq_lens"], out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    ref_out, ref_lse = mrope_attn(dev["q"], dev["k"], dev["v"], dev["pos"], dev["gamma_q"], dev["gamma_k"],
                                  dev["seq_lens"], return_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def _bitwise_equal(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_calls_in_a_row_second_smaller():
    # first: the 1024px layer (the timed shape; about 57 MB of scratch, with
    # split tiles); second: a small ragged batch reusing the array
    first = config_workload("1024px")
    second = make_workload(2, 4, 128, (16, 24, 24), 48, 12, 14, text_lens=(19, 48), seed=7)
    for name, w in (("1024px", first), ("small ragged", second)):
        say(f"case: noalloc {name} {w.q.shape}")
        out, lse, ref_out, ref_lse = _run_both(w)
        assert _bitwise_equal(out, ref_out), f"{name}: output differs from mrope_attn_fwd"
        assert _bitwise_equal(lse, ref_lse), f"{name}: lse differs from mrope_attn_fwd"
        got, glse = _np(out), _np(lse)
        if name == "1024px":
            rows = sample_rows(w, n=48)
            ref, rlse = run_oracle(w, rows=rows)
            check_parity(got[:, rows], ref, w.dtype, f"noalloc {name} sampled rows")
            check_lse(glse[:, :, rows], rlse)
        else:
            ref, rlse = run_oracle(w)
            check_parity(got, ref, w.dtype, f"noalloc {name}")
            check_lse(glse, rlse)


def test_fp32_needs_no_scratch():
    w = config_workload("tiny")
    say(f"case: noalloc fp32 tiny {w.q.shape}")
    out, lse, ref_out, ref_lse = _run_both(w)
    assert _bitwise_equal(out, ref_out) and _bitwise_equal(lse, ref_lse)
    ref, rlse = run_oracle(w)
    check_parity(_np(out), ref, "fp32", "noalloc fp32 tiny")
    check_lse(_np(lse), rlse, 1e-5)


def test_too_large_is_refused_and_writes_nothing():
    import torch
    from diffusion_transformer_image_head_amd.binding import MraError, mrope_attn_noalloc
    say("case: noalloc 12800-token problem refused")
    dev = torch.device("cuda")
    b, s, h, d = 1, 12800, 32, 128
    q = torch.zeros((b, s, h, d), dtype=torch.bfloat16, device=dev)
    pos = torch.zeros((b, s, 3), dtype=torch.int32, device=dev)
    g = torch.ones(d, dtype=torch.float32, device=dev)
    out = torch.full_like(q, 7.0)
    with pytest.raises(MraError) as e:
        mrope_attn_noalloc(q, q, q, pos, g, g, None, text_pad=512, out=out)
    assert e.value.status == -10
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
