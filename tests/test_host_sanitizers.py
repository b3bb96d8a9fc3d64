"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/host_sanitize/abi_walk.cpp drives every entry point's host path
(validation, the attention plan and workspace layout, group, packed, backward
and projection sizing, the no-allocation refusals, status strings) over the
benchmark's shapes and 20,000 seeded random descriptors, with the launch hook
set so no call reaches the device. The library source is compiled with both
sanitizers on its host half only (the device half is built normally and never
runs); any report aborts the run, and the walk also checks each status
against the calling contract.
"""

import os
import subprocess

import pytest

from diffusion_transformer_image_head_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def test_host_paths_clean_under_asan_ubsan(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    exe = tmp_path / "abi_walk"
    host_san = []
    for s in ("address", "undefined"):
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [hipcc, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
           "-I", os.path.join(B.ROOT, "include"), os.path.join(B.CSRC, "mrope_attn.hip"),
           os.path.join(HERE, "host_sanitize", "abi_walk.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert run.returncode == 0 and "abi walk ok" in run.stdout, out[-4000:]
