"""Register budgets of the HIP kernels, checked on the CPU from the device
assembly the compiler writes for gfx950 (no GPU needed).

A kernel that spills, or a 4-wave attention kernel that needs more than 256
VGPRs (so only one workgroup fits per CU instead of two), still computes the
right result, so no parity test notices it; only its speed collapses. These
ceilings catch that at build time.
"""

import os
import re
import subprocess

import pytest

from diffusion_transformer_image_head_amd import build as B

# no default kernel may spill (the fused-K attention, not the default, may:
# see _scratch_allowed)
SPILL_CEILING = {}
# two workgroups per CU need each wave within 256 registers
VGPR_CEILING = {"attn_bf16_kernel": 256, "bwd_fused_kernel": 256, "qkv_proj_kernel": 256}


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "mrope_attn.s"
    flags = [f for f in B.flags() if f not in ("-shared", "-fPIC")]
    cmd = [B.hipcc()] + flags + ["--cuda-device-only", "-S",
                                 os.path.join(B.CSRC, "mrope_attn.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = out.read_text()
    meta = text[text.index("amdhsa.kernels:"):]
    res = {}
    for ent in meta.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", ent)
        if not name:
            continue
        res[name.group(1)] = (int(re.search(r"\.vgpr_count:\s+(\d+)", ent).group(1)),
                              int(re.search(r"\.vgpr_spill_count:\s+(\d+)", ent).group(1)),
                              int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", ent).group(1)))
    return res


def _kind(mangled):
    """Unqualified name of a kernel in namespace mra (templates or not)."""
    m = re.match(r"_ZN3mra(\d+)", mangled)
    if not m:
        return mangled
    n = int(m.group(1))
    return mangled[m.end():m.end() + n]


def test_every_kernel_is_reported(kernels):
    kinds = {_kind(k) for k in kernels}
    for k in ("attn_bf16_kernel", "split_merge_kernel", "k_prologue_kernel", "rope_table_kernel",
              "attn_fp32_kernel", "bwd_delta_kernel", "bwd_dgamma_kernel", "bwd_fused_kernel",
              "qkv_proj_kernel"):
        assert k in kinds, k


def test_only_launched_kernels_are_built(kernels):
    # every kernel in the library is one an entry point launches
    kinds = {_kind(k) for k in kernels}
    assert kinds <= {"attn_bf16_kernel", "split_merge_kernel", "clear_counters_kernel", "k_prologue_kernel",
                     "rope_table_kernel", "attn_fp32_kernel", "bwd_delta_kernel", "bwd_dgamma_kernel",
                     "bwd_fused_kernel", "qkv_proj_kernel"}, kinds


def test_spills_within_ceiling(kernels):
    for name, (vgpr, spill, _) in kernels.items():
        if _scratch_allowed(name):
            continue
        assert spill <= SPILL_CEILING.get(_kind(name), 0), (name, vgpr, spill)


def _scratch_allowed(name):
    """Kernels allowed per-lane scratch: the attention with the K prologue
    fused into the tile loads (kprologue "fused", not the default), whose
    staging helper the compiler keeps out of line, so its captures live in
    scratch; inlined, it needs more than 256 VGPRs."""
    if _kind(name) == "attn_bf16_kernel":
        args = re.findall(r"Li(\d+)E", name)
        return len(args) >= 6 and args[4] == "1"
    return False


def test_no_scratch_in_default_kernels(kernels):
    for name, (_, _, scratch) in kernels.items():
        if not _scratch_allowed(name):
            assert scratch == 0, (name, scratch)


def test_occupancy_register_budgets(kernels):
    for name, (vgpr, _, _) in kernels.items():
        ceiling = VGPR_CEILING.get(_kind(name))
        if ceiling is not None:
            assert vgpr <= ceiling, (name, vgpr)
