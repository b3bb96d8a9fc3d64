"""The committed rocprofv3 summaries: each one states the command that made it
and the hash of the kernel sources it was taken on, and bench.py can tell
whether that hash still matches the sources (CPU only)."""

import os
import re

import pytest

import bench

PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")

# profile file prefix -> the source set bench.py hashes for that path
PATHS = {"attn_bf16_": "forward", "attn_bwd_": "backward", "qkv_proj_": "qkv"}


def summaries():
    return sorted(f for f in os.listdir(PROFILES) if f.endswith((".txt", ".md")))


def path_of(name):
    for prefix, path in PATHS.items():
        if name.startswith(prefix):
            return path
    return None


def test_profiles_exist():
    assert summaries(), "no rocprofv3 summaries under profiles/"


@pytest.mark.parametrize("name", summaries())
def test_summary_names_its_kernel_path_command_and_hash(name):
    path = path_of(name)
    assert path is not None, f"{name}: not named for a known kernel path {sorted(PATHS)}"
    text = open(os.path.join(PROFILES, name)).read()
    assert "rocprofv3" in text and "--" in text, f"{name}: no rocprofv3 command"
    rec = bench.profile_record(name)
    assert re.fullmatch(r"[0-9a-f]{16}", rec.get("kernel_source_hash", "")), f"{name}: no kernel_source_hash"
    # never a reference to the working area or to raw profiler output files
    assert "_work/" not in text
    assert len(text.encode()) < 16384, f"{name}: summaries stay short"


def test_source_sets_exist_and_differ():
    csrc = os.path.join(os.path.dirname(bench.__file__), "diffusion_transformer_image_head_amd", "csrc")
    hashes = set()
    for path, files in bench.SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(csrc, f)), f"{path}: {f} missing"
        hashes.add(bench.kernel_source_hash(path))
    assert len(hashes) == len(bench.SOURCES)


def test_profile_status_reports_match():
    for name in summaries():
        path = path_of(name)
        rec = bench.profile_record(name)
        want = "current" if rec["kernel_source_hash"] == bench.kernel_source_hash(path) else "stale"
        if path == "forward":
            config = name[len("attn_bf16_"):].split("_")[0]
            kind = name[len(f"attn_bf16_{config}_"):].rsplit(".", 1)[0]
            assert bench.profiles_status(config).get(kind) == want
        else:
            assert bench.path_profile_status(name, path) == want
