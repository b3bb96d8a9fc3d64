"""GPU parity sweep: seeded small problems whose sequence lengths sit on and
around the key-tile (64) and query-tile (128 / 256 row) edges, with random
text padding and true text lengths, head counts, head_dim 64 / 128, both K'
prologues, both gamma layouts and both rotary pair conventions. Every output
and LSE is compared with the fp64 oracle, and padded text rows must be exact
zeros. The case list is drawn once from a fixed seed, so it is the same on
every run."""

import numpy as np
import pytest

from diffusion_transformer_image_head_amd.workloads import make_workload
from tests.gpu_util import check_lse, check_parity, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

# sequence lengths around the edges of 64-key tiles and 128 / 256-row tiles
LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 300]


def _cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for i, s in enumerate(LENGTHS * 2):
        d = 64 if i % 5 == 4 else 128
        section = (8, 12, 12) if d == 64 else (16, 24, 24)
        text_pad = int(rng.integers(0, min(s, 96) + 1))
        img = s - text_pad
        # an image of 1 x img tokens (or none) keeps the length exact
        grid = (1, img) if img > 0 else (0, 0)
        batch = int(rng.integers(1, 3))
        heads = int(rng.integers(1, 4))
        lens = None
        if text_pad > 0 and rng.random() < 0.6:
            lens = tuple(int(x) for x in rng.integers(0, text_pad + 1, size=batch))
        cases.append(dict(
            id=f"s{s}_d{d}_t{text_pad}_b{batch}_h{heads}" + ("_lens" if lens else ""),
            batch=batch, heads=heads, head_dim=d, section=section, text_pad=text_pad, grid=grid,
            text_lens=lens, kpro="fused" if i % 3 == 2 else "prepass",
            per_head=bool(i % 4 == 1), pairs="interleaved" if i % 4 == 3 else "half", seed=7000 + i))
    return cases


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_image_head_amd import binding
    binding.lib()  # fail loudly if the HIP library is missing


def test_case_list_covers_the_edges():
    lengths = {c["text_pad"] + c["grid"][0] * c["grid"][1] for c in CASES}
    assert set(LENGTHS) <= lengths
    assert {c["head_dim"] for c in CASES} == {64, 128}
    assert {c["kpro"] for c in CASES} == {"prepass", "fused"}
    assert any(c["text_lens"] for c in CASES) and any(c["per_head"] for c in CASES)
    assert any(c["pairs"] == "interleaved" for c in CASES)


@pytest.mark.parametrize("c", CASES, ids=[c["id"] for c in CASES])
def test_sweep_case(c):
    w = make_workload(c["batch"], c["heads"], c["head_dim"], c["section"], c["text_pad"], c["grid"][0],
                      c["grid"][1], text_lens=c["text_lens"], dtype="bf16", seed=c["seed"],
                      gamma_per_head=c["per_head"], rope_pairs=c["pairs"])
    say(f"case: sweep {c['id']} kprologue={c['kpro']} per_head={c['per_head']} pairs={c['pairs']}")
    out, lse = run_gpu(w, kprologue=c["kpro"])
    ref, rlse = run_oracle(w)
    check_parity(out, ref, "bf16", c["id"])
    check_lse(lse, rlse)
    if w.seq_lens is not None:
        for b, l in enumerate(w.seq_lens):
            assert np.all(out[b, int(l):w.text_pad] == 0), "padded text rows must be zero"
