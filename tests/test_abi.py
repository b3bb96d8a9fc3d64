"""C ABI contract on the CPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any device work.

No compute call runs here (there is no GPU); the calls below either fail
validation, take the empty-input early return, or stop at the fault-injection
hook that sits just before the first launch.
"""

import ctypes
import os
import re
import subprocess
import sys

import pytest

from diffusion_transformer_image_head_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mrope_attn.h")

FAKE = 0x10000  # aligned, non-null; never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from diffusion_transformer_image_head_amd.build import build
        build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(mrope_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "mrope_attn_abi_version", "mrope_attn_attend", "mrope_attn_bwd",
        "mrope_attn_bwd_varlen", "mrope_attn_bwd_varlen_workspace_size",
        "mrope_attn_bwd_workspace_size", "mrope_attn_fwd", "mrope_attn_fwd_group",
        "mrope_attn_fwd_noalloc", "mrope_attn_fwd_varlen", "mrope_attn_group_workspace_size",
        "mrope_attn_last_hip_error", "mrope_attn_launch_plan", "mrope_attn_prepare",
        "mrope_attn_status_string", "mrope_attn_validate", "mrope_attn_varlen_workspace_size",
        "mrope_attn_workspace_size", "mrope_qkv_proj", "mrope_qkv_proj_workspace_size"])


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True)
    exported = set(l.split()[-1] for l in out.stdout.splitlines() if l.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def _c_layout(tmp_path, struct, fields):
    """sizeof and offsetof of a header struct, from a C program built with gcc."""
    src = tmp_path / f"{struct}.c"
    lines = [f'#include "{HEADER}"', "#include <stdio.h>", "#include <stddef.h>", "int main(void) {",
             f'  printf("%zu\\n", sizeof({struct}));']
    lines += [f'  printf("%zu\\n", offsetof({struct}, {f}));' for f in fields]
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / struct
    subprocess.run(["gcc", "-std=c11", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    return [int(x) for x in out]


def test_one_hip_runtime_in_the_process():
    # torch bundles a HIP runtime with the soname of the system one; loading
    # the library before torch would map both, and the second finds no
    # device. The binding imports torch first, so a fresh process that only
    # loads the library maps exactly one of each runtime library.
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from diffusion_transformer_image_head_amd import binding\n"
            "binding.lib()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "for key in ('libamdhip64', 'libhsa-runtime64'):\n"
            "    print(key, len(set(l.split()[-1] for l in maps if key in l)))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True).stdout
    assert "libamdhip64 1" in out and "libhsa-runtime64 1" in out, out


@pytest.mark.parametrize("cls,struct", [(B.Desc, "mra_desc"), (B.QkvDesc, "mra_qkv_desc"),
                                        (B.Problem, "mra_problem"), (B.LaunchPlan, "mra_launch_plan")])
def test_struct_layouts_match_header(tmp_path, cls, struct):
    names = [f[0] for f in cls._fields_]
    got = _c_layout(tmp_path, struct, names)
    assert ctypes.sizeof(cls) == got[0]
    for name, off in zip(names, got[1:]):
        assert getattr(cls, name).offset == off, name


def test_version_and_status_strings(lib):
    assert lib.mrope_attn_abi_version() == 109
    for st in range(0, -11, -1):
        s = B.status_string(st)
        assert s and s != "unknown status"
    assert B.status_string(-77) == "unknown status"


def desc(**kw):
    base = dict(batch=2, seq=100, heads=4, head_dim=128, text_pad=20)
    base.update(kw)
    args = {k: base.pop(k) for k in ("batch", "seq", "heads", "head_dim")}
    return B.make_desc(args["batch"], args["seq"], args["heads"], args["head_dim"], **base)


def val(d, **ptr):
    p = dict(q=FAKE, k=FAKE, v=FAKE, pos=FAKE, gq=FAKE, gk=FAKE, seq=None, out=FAKE)
    p.update(ptr)
    return B.validate(d, p["q"], p["k"], p["v"], p["pos"], p["gq"], p["gk"], p["seq"], p["out"])


def test_validate_accepts_good_calls(lib):
    assert val(desc()) == 0
    assert val(desc(section=(24, 20, 20))) == 0
    assert val(desc(head_dim=64, section=(8, 12, 12))) == 0
    assert val(desc(dtype=B.MRA_FP32, head_dim=64, section=(8, 12, 12))) == 0
    assert val(desc(text_pad=0)) == 0
    assert val(desc(text_pad=100)) == 0
    assert val(desc(rope_pairs="interleaved", gamma_per_head=True)) == 0
    assert val(desc(), seq=FAKE) == 0
    # strided views of one fused [B, S, 3, H, D] qkv buffer
    st = (100 * 3 * 4 * 128, 3 * 4 * 128, 128)
    assert val(desc(q_stride=st, k_stride=st, v_stride=st)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96, section=(16, 16, 16)), -2),
    (dict(head_dim=32, section=(4, 6, 6)), -2),
    (dict(heads=0), -2),
    (dict(batch=-1), -2),
    (dict(text_pad=101), -2),
    (dict(text_pad=-1), -2),
    (dict(dtype=7), -3),
    (dict(section=(16, 24, 23)), -4),
    (dict(section=(-1, 33, 32)), -4),
    (dict(theta=0.0), -9),
    (dict(theta=float("nan")), -9),
    (dict(eps=-1e-6), -9),
    (dict(scale=float("inf")), -9),
    (dict(kprologue=5), -9),
    (dict(rope_pairs=2), -9),
    (dict(gamma_per_head=2), -9),
    (dict(q_stride=(100 * 4 * 128, 4 * 128, 100)), -5),     # bf16 needs multiples of 8
    (dict(o_stride=(-1, 4 * 128, 128)), -5),
    (dict(seq=1 << 20, text_pad=0, k_stride=(0, 1 << 11, 128)), -6),   # > 2 GiB per slice
])
def test_validate_rejects(lib, kw, code):
    assert val(desc(**kw)) == code


def test_validate_pointers(lib):
    d = desc()
    for name in ("q", "k", "v", "pos", "gq", "gk", "out"):
        assert val(d, **{name: None}) == -1, name
    assert val(d, q=FAKE + 8) == -5          # bf16 pointers need 16-byte alignment
    assert val(d, out=FAKE + 2) == -5
    assert val(d, seq=FAKE + 2) == -5
    assert B.lib().mrope_attn_validate(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE) == -1


def test_empty_inputs_are_noops(lib):
    for d in (desc(batch=0), desc(seq=0, text_pad=0)):
        assert val(d, q=None, k=None, v=None, out=None) == 0
        rc = lib.mrope_attn_fwd(ctypes.byref(d), None, None, None, None, None, None, None,
                                None, None, None, 0, None)
        assert rc == 0
        assert B.workspace_size(d) == 0


def test_workspace_sizes(lib):
    d = desc(batch=1, seq=4608, heads=32, text_pad=512)
    table = 4608 * 64 * 8
    kprime = 4608 * 32 * 128 * 2
    # 1152 query tiles of 128 rows over 512 resident workgroups leave 128 for
    # the last wave, each cut into 2 key ranges (one workgroup per CU): a
    # (O[64], m, l) fp32 record per lane of 256 lanes per part
    split = 128 * 2 * 256 * (128 // 2 + 2) * 4
    assert B.workspace_size(d) == table + kprime + split           # auto = prepass
    assert B.workspace_size(desc(batch=1, seq=4608, heads=32, text_pad=512,
                                 kprologue="fused")) == table + split
    # 1024 tiles fill two waves exactly: nothing is split
    assert B.workspace_size(desc(batch=1, seq=4096, heads=32, text_pad=512,
                                 kprologue="fused")) == 4096 * 64 * 8
    assert B.workspace_size(desc(dtype=B.MRA_FP32, head_dim=64, section=(8, 12, 12))) == 0
    assert B.workspace_size(desc(section=(1, 2, 3))) == 0          # invalid -> 0
    rec4 = 4 * 64 * (128 // 2 + 2) * 4                             # one part's records, 4 waves
    rec8 = 8 * 64 * (128 // 2 + 2) * 4                             # 8 waves
    # 8-wave workgroups (256 rows, one per CU) from 2.5 rounds of them: 36
    # heads at 4608 tokens make 648, whose 136-tile last wave is not cut
    h36 = desc(batch=1, seq=4608, heads=36, text_pad=512)
    assert B.workspace_size(h36) == table + 4608 * 36 * 128 * 2
    # 12800 tokens: 1600 tiles of 256 rows leave 64, cut into 4 key ranges
    lng = desc(batch=1, seq=12800, heads=32, text_pad=512)
    assert B.workspace_size(lng) == 12800 * 64 * 8 + 12800 * 32 * 128 * 2 + 64 * 4 * rec8
    # 4-wave problems (under 2.5 rounds of 256-row tiles): 2 x 196 heads x
    # 200 tokens make 784 tiles of 128 rows, a 272-tile last wave, a few more
    # than the 256 compute units: cut into 2 key ranges
    d3 = desc(batch=2, seq=200, heads=196, text_pad=32)
    assert B.workspace_size(d3) == 2 * 200 * 64 * 8 + 2 * 200 * 196 * 128 * 2 + 272 * 2 * rec4
    # one partial round of 4 x 18 = 72 tiles of 256 rows (4 heads at 4608
    # tokens, 72 key tiles each): 8 waves, every tile in 3 key ranges (the
    # same bytes as 144 tiles of 128 rows); 512px (240 tiles of 128 rows, 20
    # key tiles): 4 waves, no cut
    h4 = desc(batch=1, seq=4608, heads=4, text_pad=512)
    assert B.workspace_size(h4) == table + 4608 * 4 * 128 * 2 + 72 * 3 * rec8
    p512 = desc(batch=1, seq=1280, heads=24, text_pad=256)
    assert B.workspace_size(p512) == 1280 * 64 * 8 + 1280 * 24 * 128 * 2
    # 928 tiles leave 416: not cut; 704 tiles leave 192: not cut
    for seq, heads in ((3712, 32), (2816, 32)):
        d2 = desc(batch=1, seq=seq, heads=heads, text_pad=512)
        assert B.workspace_size(d2) == seq * 64 * 8 + seq * heads * 128 * 2
    assert lib.mrope_attn_workspace_size(None) == 0


def test_launch_plans(lib):
    d = desc(batch=1, seq=4608, heads=32, text_pad=512)
    p = B.launch_plan(d)                       # no device here: the MI355X's shape
    # 1152 tiles of 128 rows over 512 slots: the 128-tile last round is cut
    # into 2 key ranges, one workgroup per CU
    assert (p.waves, p.grid, p.xcds, p.tiles, p.split_tiles, p.parts) == (4, 1280, 8, 1152, 128, 2)
    assert p.workspace_bytes == B.workspace_size(d)
    q = B.launch_plan(d, 256, 8)
    assert (q.grid, q.split_tiles, q.workspace_bytes) == (p.grid, p.split_tiles, p.workspace_bytes)
    # a 304-CU device: 608 slots leave a 544-tile round, too full to cut
    q = B.launch_plan(d, 304, 8)
    assert (q.waves, q.grid, q.split_tiles, q.parts) == (4, 1152, 0, 1)
    # one XCD of 32 CUs: 576 tiles of 256 rows are 18 rounds of one per CU
    q = B.launch_plan(d, 32, 1)
    assert (q.waves, q.grid, q.xcds, q.split_tiles) == (8, 576, 1, 0)
    # 80 CUs: 8 waves, 576 = 7 x 80 + 16; the 16 tiles are cut into 80 / 16
    # = 5 key ranges
    q = B.launch_plan(d, 80, 0)
    assert (q.waves, q.xcds, q.split_tiles, q.parts, q.grid) == (8, 1, 16, 5, 560 + 80)
    # 4 heads on 64 CUs: 4 waves, 144 tiles over 128 slots leave 16, cut
    # into 64 / 16 = 4 ranges
    h4 = desc(batch=1, seq=4608, heads=4, text_pad=512)
    q = B.launch_plan(h4, 64, 8)
    assert (q.waves, q.tiles, q.split_tiles, q.parts, q.grid) == (4, 144, 16, 4, 128 + 64)
    # the split records always fit the workspace
    for seq in (1, 64, 500, 1280, 4608, 12800):
        for heads in (1, 4, 24, 36):
            for cus, x in ((256, 8), (304, 8), (80, 1), (38, 2)):
                e = desc(batch=2, seq=seq, heads=heads, text_pad=min(seq, 16))
                r = B.launch_plan(e, cus, x)
                assert r.grid == r.tiles - r.split_tiles + r.split_tiles * r.parts
                assert 1 <= r.parts <= 8 and r.split_tiles <= r.tiles
                assert r.workspace_bytes >= r.split_tiles * r.parts * r.waves * 64 * 66 * 4
    assert B.launch_plan(desc(batch=0)).grid == 0
    with pytest.raises(B.MraError):
        B.launch_plan(desc(dtype=B.MRA_FP32, head_dim=64, section=(8, 12, 12)))
    with pytest.raises(B.MraError):
        B.launch_plan(desc(section=(1, 2, 3)))


def _fwd(d, ws, nbytes, lse=None):
    return B.lib().mrope_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                  FAKE, lse, ws, nbytes, None)


def test_fwd_rejects_before_launch(lib, monkeypatch):
    d = desc()
    need = B.workspace_size(d)
    assert _fwd(d, None, 0) == -7
    assert _fwd(d, FAKE, need - 1) == -7
    assert _fwd(d, FAKE + 4, need) == -7
    assert _fwd(d, FAKE, need, lse=FAKE + 1) == -5
    assert _fwd(desc(section=(1, 1, 1)), FAKE, need) == -4
    # fault injection: everything valid, the call stops right before launching
    monkeypatch.setenv("MRA_FAULT_INJECT", "launch")
    assert _fwd(d, FAKE, need) == -8
    assert _fwd(desc(dtype=B.MRA_FP32, head_dim=64, section=(8, 12, 12)), None, 0) == -8
    L = B.lib()
    assert L.mrope_attn_prepare(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, need, None) == -8
    assert L.mrope_attn_attend(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                               None, FAKE, need, None) == -8


def _noalloc(d, lse=None):
    return B.lib().mrope_attn_fwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          FAKE, lse, None)


def test_noalloc_rejects_before_any_device_call(lib):
    # the arguments are checked like mrope_attn_fwd's; then a problem whose
    # scratch exceeds the library's array is refused before the array is
    # looked up (no HIP call is made on these paths)
    assert B.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert _noalloc(desc(section=(1, 1, 1))) == -4
    assert _noalloc(desc(head_dim=96)) == -2
    assert _noalloc(desc(theta=0.0)) == -9
    assert B.lib().mrope_attn_fwd_noalloc(ctypes.byref(desc()), None, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          FAKE, None, None) == -1
    long_ = desc(batch=1, seq=12800, heads=32, text_pad=512)
    assert B.workspace_size(long_) > B.NOALLOC_SCRATCH_BYTES
    assert _noalloc(long_) == -10
    ragged = desc(batch=4, seq=4608, heads=32, text_pad=512)
    assert _noalloc(ragged) == -10
    # the 1024px layer (32 heads; also 36) fits
    assert B.workspace_size(desc(batch=1, seq=4608, heads=32, text_pad=512)) <= B.NOALLOC_SCRATCH_BYTES
    assert B.workspace_size(desc(batch=1, seq=4608, heads=36, text_pad=512)) <= B.NOALLOC_SCRATCH_BYTES
    assert "no-allocation" in B.status_string(-10)


def test_last_hip_error_starts_clear(lib):
    # no HIP error has happened on this thread (nothing here reaches the device)
    assert B.last_hip_error() == (0, "none")


def test_stages_validate_like_fwd(lib):
    d = desc()
    need = B.workspace_size(d)
    L = B.lib()
    assert L.mrope_attn_prepare(ctypes.byref(d), None, FAKE, FAKE, FAKE, need, None) == -1
    assert L.mrope_attn_prepare(ctypes.byref(d), FAKE, FAKE, FAKE, None, 0, None) == -7
    assert L.mrope_attn_attend(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                               None, FAKE, need - 1, None) == -7
    e = desc(batch=0)
    assert L.mrope_attn_prepare(ctypes.byref(e), None, None, None, None, 0, None) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 4, 1, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        B.mrope_attn(x, x, x, torch.zeros(1, 4, 3, dtype=torch.int32), torch.ones(64),
                     torch.ones(64), text_pad=0, section=(8, 12, 12))


# ---------------------------------------------------------------- grouped call
def _group(descs, probs=None, ws=FAKE, nbytes=1 << 40):
    n = len(descs)
    darr = (B.Desc * max(n, 1))(*descs)
    if probs is None:
        probs = [B.Problem(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) for _ in descs]
    parr = (B.Problem * max(n, 1))(*probs)
    return B.lib().mrope_attn_fwd_group(darr, parr, n, ws, nbytes, None)


def test_group_workspace_is_the_sum_of_its_parts(lib):
    cond = desc(batch=1, seq=4608, heads=32, text_pad=512)
    uncond = desc(batch=1, seq=4096, heads=32, text_pad=0)
    # per problem: rotary table + K'; then the split records of the combined
    # grid: 576 + 512 = 1088 tiles of 256 rows (8-wave workgroups, over 2.5
    # rounds) leave 64 for the last wave -> 4 parts
    per = [s * 64 * 8 + s * 32 * 128 * 2 for s in (4608, 4096)]
    split = 64 * 4 * 512 * (128 // 2 + 2) * 4
    assert B.group_workspace_size([cond, uncond]) == sum(per) + split
    # a group of one is the plain call
    assert B.group_workspace_size([cond]) == B.workspace_size(cond)
    # empty members take nothing; fp32 groups need none
    assert B.group_workspace_size([cond, desc(batch=0)]) == B.workspace_size(cond)
    f32 = dict(dtype=B.MRA_FP32, head_dim=64, section=(8, 12, 12))
    assert B.group_workspace_size([desc(**f32), desc(**f32)]) == 0
    # invalid or mixed groups -> 0
    assert B.group_workspace_size([cond, desc(head_dim=64, section=(8, 12, 12))]) == 0
    assert B.group_workspace_size([cond, desc(section=(1, 2, 3))]) == 0


def test_group_rejects_before_launch(lib, monkeypatch):
    d = desc()
    assert _group([]) == -9                                     # n = 0
    assert _group([d] * 5) == -9                                # n > MRA_MAX_GROUP
    L = B.lib()
    assert L.mrope_attn_fwd_group(None, None, 1, FAKE, 1 << 40, None) == -1
    assert _group([d, desc(head_dim=64, section=(8, 12, 12))]) == -6
    assert _group([d, desc(kprologue="fused")]) == -6
    assert _group([d, desc(section=(1, 2, 3))]) == -4          # per-problem validation
    bad = B.Problem(FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None)
    good = B.Problem(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None)
    assert _group([d, d], [good, bad]) == -1
    assert _group([d, d], [good, B.Problem(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE + 2)]) == -5
    need = B.group_workspace_size([d, d])
    assert _group([d, d], ws=FAKE, nbytes=need - 1) == -7
    assert _group([d, d], ws=None, nbytes=need) == -7
    assert _group([desc(batch=0), desc(seq=0, text_pad=0)], ws=None, nbytes=0) == 0   # nothing to do
    monkeypatch.setenv("MRA_FAULT_INJECT", "launch")
    assert _group([d, d], nbytes=need) == -8
    assert _group([d, desc(batch=3, seq=40, text_pad=0)], nbytes=need) == -8


# ---------------------------------------------------------------- packed varlen
def _varlen(d, max_seqlen, cu=FAKE, ws=FAKE, nbytes=1 << 40, lse=None):
    return B.lib().mrope_attn_fwd_varlen(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cu,
                                         max_seqlen, FAKE, lse, ws, nbytes, None)


def test_varlen_workspace(lib):
    # 3 sequences packed into 9000 tokens, the longest 4608: the table and K'
    # cover the packed tokens, the tiles 3 x 32 heads x 36 query tiles
    d = desc(batch=3, seq=9000, heads=32, text_pad=0)
    tiles = 3 * 32 * 36                       # 3456 = 6 x 512 + 384: no split
    assert tiles % 512 == 384
    assert B.lib().mrope_attn_varlen_workspace_size(ctypes.byref(d), 4608) == \
        9000 * 64 * 8 + 9000 * 32 * 128 * 2
    # 1 sequence of 4608: 1152 tiles -> 128 split in 2
    d1 = desc(batch=1, seq=4608, heads=32, text_pad=0)
    assert B.lib().mrope_attn_varlen_workspace_size(ctypes.byref(d1), 4608) == \
        B.workspace_size(d1)
    assert B.lib().mrope_attn_varlen_workspace_size(ctypes.byref(d), 9001) == 0    # > seq
    assert B.lib().mrope_attn_varlen_workspace_size(ctypes.byref(desc(text_pad=5)), 10) == 0
    assert B.lib().mrope_attn_varlen_workspace_size(ctypes.byref(d), 0) == 0


def test_varlen_rejects_before_launch(lib, monkeypatch):
    d = desc(batch=3, seq=100, text_pad=0)
    need = B.lib().mrope_attn_varlen_workspace_size(ctypes.byref(d), 60)
    assert _varlen(desc(batch=3, seq=100, text_pad=4), 60) == -2
    assert _varlen(d, 101) == -2
    assert _varlen(d, -1) == -2
    assert _varlen(d, 60, cu=None) == -1
    assert _varlen(d, 60, cu=FAKE + 2) == -5
    assert _varlen(d, 60, lse=FAKE + 1) == -5
    assert _varlen(d, 60, nbytes=need - 1) == -7
    assert _varlen(d, 60, ws=None) == -7
    assert _varlen(desc(batch=0, seq=100, text_pad=0), 60, cu=None, ws=None, nbytes=0) == 0
    assert _varlen(d, 0, cu=None, ws=None, nbytes=0) == 0           # nothing to compute
    monkeypatch.setenv("MRA_FAULT_INJECT", "launch")
    assert _varlen(d, 60, nbytes=need) == -8
    f32 = desc(batch=3, seq=100, text_pad=0, dtype=B.MRA_FP32, head_dim=64, section=(8, 12, 12))
    assert _varlen(f32, 60, ws=None, nbytes=0) == -8


# ---------------------------------------------------------------- backward
def _bwd(d, lse=FAKE, dout=FAKE, dq=FAKE, ws=FAKE, nbytes=1 << 40, dg=FAKE):
    return B.lib().mrope_attn_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                  lse, dout, dq, FAKE, FAKE, dg, dg, ws, nbytes, None)


def test_bwd_workspace(lib):
    d = desc(batch=1, seq=4608, heads=32, text_pad=512)
    rows = 4608 * 32
    n_wg = 32 * 36
    want = 4608 * 64 * 8 + 2 * rows * 128 * 2 + 2 * rows * 4 + 2 * n_wg * 128 * 4
    assert B.lib().mrope_attn_bwd_workspace_size(ctypes.byref(d)) == want
    assert B.lib().mrope_attn_bwd_workspace_size(ctypes.byref(desc(head_dim=64, section=(8, 12, 12)))) == 0
    assert B.lib().mrope_attn_bwd_workspace_size(ctypes.byref(desc(dtype=B.MRA_FP32))) == 0


def test_bwd_rejects_before_launch(lib, monkeypatch):
    d = desc()
    need = B.lib().mrope_attn_bwd_workspace_size(ctypes.byref(d))
    assert _bwd(desc(head_dim=64, section=(8, 12, 12))) == -6
    assert _bwd(desc(dtype=B.MRA_FP32)) == -6
    assert _bwd(desc(section=(1, 2, 3))) == -4
    assert _bwd(d, lse=None) == -1
    assert _bwd(d, dout=None) == -1
    assert _bwd(d, dq=None) == -1
    assert _bwd(d, dq=FAKE + 8) == -5
    assert _bwd(d, lse=FAKE + 2) == -5
    assert _bwd(d, nbytes=need - 1) == -7
    assert _bwd(d, ws=None) == -7
    assert _bwd(desc(batch=0), lse=None, dout=None, dq=None, ws=None, nbytes=0) == 0
    monkeypatch.setenv("MRA_FAULT_INJECT", "launch")
    assert _bwd(d, nbytes=need) == -8
    assert _bwd(d, nbytes=need, dg=None) == -8


def _bwd_varlen(d, maxlen, cu=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, ws=FAKE, nbytes=1 << 40, dg=FAKE):
    return B.lib().mrope_attn_bwd_varlen(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cu, maxlen,
                                         FAKE, lse, dout, dq, FAKE, FAKE, dg, dg, ws, nbytes, None)


def test_bwd_varlen_workspace(lib):
    # 3 packed sequences, 6000 tokens in all, the longest 2500: the row-wise
    # pieces cover every token of the slice, the per-tile gamma partials
    # 3 sequences x 32 heads x ceil(2500 / 128) tiles
    d = desc(batch=3, seq=6000, heads=32, text_pad=0)
    rows = 6000 * 32
    n_wg = 3 * 32 * 20
    want = 6000 * 64 * 8 + 2 * rows * 128 * 2 + 2 * rows * 4 + 2 * n_wg * 128 * 4
    assert B.lib().mrope_attn_bwd_varlen_workspace_size(ctypes.byref(d), 2500) == want
    assert B.lib().mrope_attn_bwd_varlen_workspace_size(ctypes.byref(d), 0) == 0
    assert B.lib().mrope_attn_bwd_varlen_workspace_size(ctypes.byref(d), 6001) == 0
    assert B.lib().mrope_attn_bwd_varlen_workspace_size(ctypes.byref(desc(text_pad=5)), 50) == 0
    assert B.lib().mrope_attn_bwd_varlen_workspace_size(ctypes.byref(desc(text_pad=0, dtype=B.MRA_FP32)),
                                                        50) == 0


def test_bwd_varlen_rejects_before_launch(lib, monkeypatch):
    d = desc(text_pad=0)
    need = B.lib().mrope_attn_bwd_varlen_workspace_size(ctypes.byref(d), 60)
    assert need > 0
    assert _bwd_varlen(desc(text_pad=5), 60) == -2                # text_pad must be 0
    assert _bwd_varlen(d, 101) == -2                              # max_seqlen > seq
    assert _bwd_varlen(d, -1) == -2
    assert _bwd_varlen(desc(text_pad=0, head_dim=64, section=(8, 12, 12)), 60) == -6
    assert _bwd_varlen(desc(text_pad=0, dtype=B.MRA_FP32), 60) == -6
    assert _bwd_varlen(desc(text_pad=0, kprologue="none"), 60) == -6
    assert _bwd_varlen(d, 60, cu=None) == -1
    assert _bwd_varlen(d, 60, cu=FAKE + 2) == -5
    assert _bwd_varlen(d, 60, lse=None) == -1
    assert _bwd_varlen(d, 60, dout=None) == -1
    assert _bwd_varlen(d, 60, dq=FAKE + 8) == -5
    assert _bwd_varlen(d, 60, nbytes=need - 1) == -7
    assert _bwd_varlen(d, 60, ws=None) == -7
    # nothing to do: no sequences, no tokens, or every sequence empty
    assert _bwd_varlen(desc(batch=0, text_pad=0), 0, cu=None, lse=None, dout=None, dq=None, ws=None,
                       nbytes=0) == 0
    assert _bwd_varlen(d, 0, cu=None, lse=None, dout=None, dq=None, ws=None, nbytes=0) == 0
    monkeypatch.setenv("MRA_FAULT_INJECT", "launch")
    assert _bwd_varlen(d, 60, nbytes=need) == -8
    assert _bwd_varlen(d, 60, nbytes=need, dg=None) == -8


# ---------------------------------------------------------------- operands given / fp8 QKV
def test_kprologue_none_needs_no_positions_or_table(lib):
    d = desc(kprologue="none")
    assert val(d, pos=None, gq=None, gk=None) == 0
    assert val(desc(), pos=None) == -1                         # other modes still need them
    dd = desc(batch=1, seq=4608, heads=32, text_pad=512, kprologue="none")
    split = 128 * 2 * 256 * (128 // 2 + 2) * 4                 # the split records only
    assert B.workspace_size(dd) == split
    assert val(desc(kprologue=3, dtype=B.MRA_FP32, head_dim=64, section=(8, 12, 12))) == 0
    # no backward on given operands
    assert _bwd(desc(kprologue="none")) == -6


def test_kprologue_given_plain_operands(lib):
    # plain Q', K' (q scaled as it is loaded): the same contract as Q'', K'
    d = desc(kprologue="given")
    assert d.kprologue == 4
    assert val(d, pos=None, gq=None, gk=None) == 0
    for kw in (dict(), dict(batch=1, seq=4608, heads=32, text_pad=512)):
        assert B.workspace_size(desc(kprologue="given", **kw)) == B.workspace_size(desc(kprologue="none", **kw))
    assert _bwd(desc(kprologue="given")) == -6
    assert val(desc(kprologue=5)) == -9                         # unknown mode
    assert "rope_pairs" in B.status_string(-9)


def _qkv(d, **ptr):
    p = dict(x=FAKE, w=FAKE, s=FAKE, pos=FAKE, gq=FAKE, gk=FAKE, q=FAKE, k=FAKE, v=FAKE, ws=FAKE,
             n=1 << 40)
    p.update(ptr)
    return B.lib().mrope_qkv_proj(ctypes.byref(d), p["x"], p["w"], p["s"], p["pos"], p["gq"], p["gk"],
                                  p["q"], p["k"], p["v"], p["ws"], p["n"], None)


def test_qkv_proj_contract(lib, monkeypatch):
    d = B.make_qkv_desc(4608, 4096, 32)
    assert B.lib().mrope_qkv_proj_workspace_size(ctypes.byref(d)) == 4608 * 64 * 8
    assert _qkv(B.make_qkv_desc(10, 100, 2)) == -2                       # hidden % 64
    assert _qkv(B.make_qkv_desc(10, 128, 0)) == -2
    assert _qkv(B.make_qkv_desc(10, 128, 2, head_dim=64, section=(8, 12, 12))) == -6
    assert _qkv(B.make_qkv_desc(10, 128, 2, section=(16, 24, 23))) == -4
    assert _qkv(B.make_qkv_desc(10, 128, 2, theta=0.0)) == -9
    assert _qkv(B.make_qkv_desc(10, 128, 2, x_stride=100)) == -5
    assert _qkv(B.make_qkv_desc(10, 128, 2, q_stride=(260, 128))) == -5
    assert _qkv(B.make_qkv_desc(1 << 20, 1024, 2)) == -6               # 32-bit offsets into x
    d = B.make_qkv_desc(10, 128, 2)
    assert _qkv(d, w=None) == -1
    assert _qkv(d, x=FAKE + 8) == -5
    assert _qkv(d, n=10) == -7
    assert _qkv(B.make_qkv_desc(0, 128, 2), x=None, ws=None, n=0) == 0
    monkeypatch.setenv("MRA_FAULT_INJECT", "launch")
    assert _qkv(d) == -8
