"""GPU tests of the attention on plain given operands (kprologue "given"):
q and k hold Q' and K', already normalised and rotated but not scaled; the
kernel multiplies q by softmax_scale * log2(e) as it loads it. The operands
are made by the oracle's own RMSNorm and M-RoPE and rounded to bf16; the
output is checked against the oracle attention on those operands, and
bitwise against the scaled-operand mode ("none") fed bf16(Q' * c2) made on
the host with the same fp32 multiply."""

import numpy as np
import pytest

from diffusion_transformer_image_head_amd.workloads import make_workload, round_to_bf16
from oracle.reference import attention, mrope, rms_norm, valid_tokens
from tests.gpu_util import check_parity, say

pytestmark = pytest.mark.gpu

CASES = [
    # ragged text, two items, tiles with a ragged tail (139 tokens)
    dict(id="b2_h3_ragged", batch=2, heads=3, text_pad=40, grid=(9, 11), lens=(17, 40), seed=9100),
    # one GPU's 4 heads of the 1024px layer: every tile cut into key ranges
    dict(id="h4_split", batch=1, heads=4, text_pad=512, grid=(64, 64), lens=None, seed=9101),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_image_head_amd import binding
    binding.lib()  # fail loudly if the HIP library is missing


def _c2(head_dim):
    """softmax_scale * log2(e) as the library rounds it to fp32."""
    scale = np.float32(1.0 / np.sqrt(np.float64(head_dim)))
    return np.float32(np.float64(scale) * 1.4426950408889634)


@pytest.mark.parametrize("c", CASES, ids=[c["id"] for c in CASES])
def test_given_plain_operands(c):
    import torch
    from diffusion_transformer_image_head_amd.binding import mrope_attn
    w = make_workload(c["batch"], c["heads"], 128, (16, 24, 24), c["text_pad"], *c["grid"],
                      text_lens=c["lens"], dtype="bf16", seed=c["seed"])
    say(f"case: given operands {c['id']} shape={w.shape}")
    qp = round_to_bf16(mrope(rms_norm(w.q.astype(np.float64), w.gamma_q, w.eps), w.pos, w.section,
                             w.theta).astype(np.float32))
    kp = round_to_bf16(mrope(rms_norm(w.k.astype(np.float64), w.gamma_k, w.eps), w.pos, w.section,
                             w.theta).astype(np.float32))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)  # noqa: E731
    sl = None if w.seq_lens is None else torch.from_numpy(w.seq_lens).cuda()
    out, lse = mrope_attn(t(qp), t(kp), t(w.v), None, None, None, sl, text_pad=w.text_pad,
                          kprologue="given", return_lse=True)
    # the same call on Q'' = bf16(Q' * c2) made here, in the scaled-operand mode
    qpp = round_to_bf16(qp * _c2(128))
    out2, lse2 = mrope_attn(t(qpp), t(kp), t(w.v), None, None, None, sl, text_pad=w.text_pad,
                            kprologue="none", return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)
    got = out.float().cpu().numpy().astype(np.float64)
    b, s, h, d = w.shape
    valid = valid_tokens(b, s, w.text_pad, w.seq_lens)
    ref, rlse = attention(qp.astype(np.float64), kp.astype(np.float64), w.v, valid, 1.0 / np.sqrt(d))
    check_parity(got, ref, "bf16", c["id"])
    fin = np.isfinite(rlse)
    gl = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(fin, np.isfinite(gl))
    assert np.abs(gl[fin] - rlse[fin]).max() <= 2e-2
    assert np.all(got[~valid] == 0)
