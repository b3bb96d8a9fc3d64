"""ctypes binding of libmrope_attn.so (argument marshalling only).

Every step of the attention path runs in the HIP library. This module turns
torch tensors into the C ABI's pointers, strides and stream, allocates the
output / workspace through torch's caching allocator, and raises on a
non-zero status. There is no fallback: without the built library, or for
tensors not on a GPU, the call fails.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmrope_attn.so")

MRA_BF16, MRA_FP32 = 0, 1
KPRO_AUTO, KPRO_FUSED, KPRO_PREPASS = 0, 1, 2
_KPRO = {"auto": KPRO_AUTO, "fused": KPRO_FUSED, "prepass": KPRO_PREPASS}
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
_PAIRS = {"half": ROPE_HALF, "interleaved": ROPE_INTERLEAVED}


def _pairs(rope_pairs) -> int:
    if isinstance(rope_pairs, str):
        if rope_pairs not in _PAIRS:
            raise ValueError(f"rope_pairs must be one of {sorted(_PAIRS)}")
        return _PAIRS[rope_pairs]
    return int(rope_pairs)


class Desc(ctypes.Structure):
    """Mirror of ``mra_desc`` (include/mrope_attn.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("text_pad", ctypes.c_int32),
        ("section", ctypes.c_int32 * 3),
        ("theta", ctypes.c_float), ("eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("kprologue", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("rope_pairs", ctypes.c_int32), ("gamma_per_head", ctypes.c_int32),
    ]


class Problem(ctypes.Structure):
    """Mirror of ``mra_problem`` (include/mrope_attn.h)."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q", "k", "v", "pos_thw", "gamma_q", "gamma_k", "seq_lens", "out", "lse")]


MAX_GROUP = 4


class QkvDesc(ctypes.Structure):
    """Mirror of ``mra_qkv_desc`` (include/mrope_attn.h)."""
    _fields_ = [
        ("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("section", ctypes.c_int32 * 3),
        ("theta", ctypes.c_float), ("eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("x_stride", ctypes.c_int64), ("q_stride", ctypes.c_int64 * 2),
        ("k_stride", ctypes.c_int64 * 2), ("v_stride", ctypes.c_int64 * 2),
        ("rope_pairs", ctypes.c_int32), ("gamma_per_head", ctypes.c_int32),
    ]


KPRO_NONE = 3
_KPRO["none"] = KPRO_NONE
KPRO_GIVEN = 4
_KPRO["given"] = KPRO_GIVEN


class LaunchPlan(ctypes.Structure):
    """Mirror of ``mra_launch_plan`` (include/mrope_attn.h)."""
    _fields_ = [("waves", ctypes.c_int32), ("grid", ctypes.c_int32), ("xcds", ctypes.c_int32),
                ("tiles", ctypes.c_int32), ("split_tiles", ctypes.c_int32), ("parts", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


class MraError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mrope_attn status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m diffusion_transformer_image_head_amd.build`")
        # torch ships its own HIP runtime under the same soname
        # (libamdhip64.so.7). Importing torch first makes the library bind to
        # that one instance: a second runtime loaded beside it sees no device,
        # and torch's stream handles belong to torch's runtime.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        L.mrope_attn_validate.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, i32p, f32p, f32p, i32p, vp]
        L.mrope_attn_validate.restype = ctypes.c_int
        L.mrope_attn_workspace_size.argtypes = [ctypes.POINTER(Desc)]
        L.mrope_attn_workspace_size.restype = ctypes.c_size_t
        L.mrope_attn_fwd.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, i32p, f32p, f32p, i32p, vp,
                                     f32p, vp, ctypes.c_size_t, vp]
        L.mrope_attn_fwd.restype = ctypes.c_int
        L.mrope_attn_prepare.argtypes = [ctypes.POINTER(Desc), vp, i32p, f32p, vp, ctypes.c_size_t, vp]
        L.mrope_attn_prepare.restype = ctypes.c_int
        L.mrope_attn_attend.argtypes = L.mrope_attn_fwd.argtypes
        L.mrope_attn_attend.restype = ctypes.c_int
        L.mrope_attn_status_string.argtypes = [ctypes.c_int]
        L.mrope_attn_status_string.restype = ctypes.c_char_p
        L.mrope_attn_launch_plan.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(LaunchPlan)]
        L.mrope_attn_launch_plan.restype = ctypes.c_int
        L.mrope_attn_last_hip_error.argtypes = [ctypes.POINTER(ctypes.c_char_p)]
        L.mrope_attn_last_hip_error.restype = ctypes.c_int
        L.mrope_attn_fwd_noalloc.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, i32p, f32p, f32p, i32p, vp,
                                             f32p, vp]
        L.mrope_attn_fwd_noalloc.restype = ctypes.c_int
        L.mrope_attn_group_workspace_size.argtypes = [ctypes.POINTER(Desc), ctypes.c_int]
        L.mrope_attn_group_workspace_size.restype = ctypes.c_size_t
        L.mrope_attn_fwd_group.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Problem), ctypes.c_int,
                                           vp, ctypes.c_size_t, vp]
        L.mrope_attn_fwd_group.restype = ctypes.c_int
        L.mrope_attn_varlen_workspace_size.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32]
        L.mrope_attn_varlen_workspace_size.restype = ctypes.c_size_t
        L.mrope_attn_fwd_varlen.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, i32p, f32p, f32p, i32p,
                                            ctypes.c_int32, vp, f32p, vp, ctypes.c_size_t, vp]
        L.mrope_attn_fwd_varlen.restype = ctypes.c_int
        L.mrope_attn_bwd_workspace_size.argtypes = [ctypes.POINTER(Desc)]
        L.mrope_attn_bwd_workspace_size.restype = ctypes.c_size_t
        L.mrope_attn_bwd.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, i32p, f32p, f32p, i32p, vp, f32p,
                                     vp, vp, vp, vp, f32p, f32p, vp, ctypes.c_size_t, vp]
        L.mrope_attn_bwd.restype = ctypes.c_int
        L.mrope_attn_bwd_varlen_workspace_size.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32]
        L.mrope_attn_bwd_varlen_workspace_size.restype = ctypes.c_size_t
        L.mrope_attn_bwd_varlen.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, i32p, f32p, f32p, i32p,
                                            ctypes.c_int32, vp, f32p, vp, vp, vp, vp, f32p, f32p, vp,
                                            ctypes.c_size_t, vp]
        L.mrope_attn_bwd_varlen.restype = ctypes.c_int
        L.mrope_qkv_proj_workspace_size.argtypes = [ctypes.POINTER(QkvDesc)]
        L.mrope_qkv_proj_workspace_size.restype = ctypes.c_size_t
        L.mrope_qkv_proj.argtypes = [ctypes.POINTER(QkvDesc), vp, vp, f32p, i32p, f32p, f32p, vp, vp, vp,
                                     vp, ctypes.c_size_t, vp]
        L.mrope_qkv_proj.restype = ctypes.c_int
        L.mrope_attn_abi_version.argtypes = []
        L.mrope_attn_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mrope_attn_status_string(status).decode()


def last_hip_error():
    """(hipError_t, name) behind this thread's most recent MRA_ERR_HIP."""
    name = ctypes.c_char_p()
    code = lib().mrope_attn_last_hip_error(ctypes.byref(name))
    return int(code), (name.value or b"").decode()


def _error(rc: int) -> MraError:
    msg = status_string(rc)
    if rc == -8:
        code, name = last_hip_error()
        msg += f" (hipError_t {code}: {name})"
    return MraError(rc, msg)


def make_desc(batch, seq, heads, head_dim, *, text_pad, section=(16, 24, 24), theta=10000.0,
              eps=1e-6, scale=None, dtype=MRA_BF16, kprologue="auto",
              q_stride=None, k_stride=None, v_stride=None, o_stride=None,
              rope_pairs="half", gamma_per_head=False) -> Desc:
    """Build a descriptor; strides default to contiguous [B, S, H, D]."""
    d = Desc()
    d.rope_pairs = _pairs(rope_pairs)
    d.gamma_per_head = int(gamma_per_head)
    d.batch, d.seq, d.heads, d.head_dim, d.text_pad = batch, seq, heads, head_dim, text_pad
    d.section[:] = [int(x) for x in section]
    d.theta, d.eps = float(theta), float(eps)
    d.softmax_scale = 0.0 if scale is None else float(scale)
    d.dtype = dtype
    d.kprologue = _KPRO[kprologue] if isinstance(kprologue, str) else int(kprologue)
    cont = (seq * heads * head_dim, heads * head_dim, head_dim)
    for name, st in (("q_stride", q_stride), ("k_stride", k_stride), ("v_stride", v_stride),
                     ("o_stride", o_stride)):
        getattr(d, name)[:] = list(cont if st is None else st)
    return d


def launch_plan(desc: Desc, compute_units: int = 0, xcds: int = 0) -> LaunchPlan:
    """The bf16 attention launch for desc on a device of that shape (0: the
    current device's); host only."""
    p = LaunchPlan()
    rc = lib().mrope_attn_launch_plan(ctypes.byref(desc), compute_units, xcds, ctypes.byref(p))
    if rc != 0:
        raise _error(rc)
    return p


def workspace_size(desc: Desc) -> int:
    return int(lib().mrope_attn_workspace_size(ctypes.byref(desc)))


def validate(desc: Desc, q, k, v, pos, gq, gk, seq_lens, out) -> int:
    """Host-only contract check on raw integer addresses (0 = NULL)."""
    return int(lib().mrope_attn_validate(ctypes.byref(desc), q, k, v, pos, gq, gk, seq_lens, out))


def _bsd_strides(t):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("q/k/v/out must be [B, S, H, D] views with head_dim contiguous")
    return (t.stride(0), t.stride(1), t.stride(2))


def _checked(q, k, v, pos, gamma_q, gamma_k, seq_lens, out, return_lse, *, text_pad, section,
             theta, eps, scale, kprologue, rope_pairs="half"):
    """Shape/dtype/device checks; returns (desc, out, lse, seq_lens)."""
    import torch

    given = kprologue in ("none", KPRO_NONE, "given", KPRO_GIVEN)
    for name, t in (("q", q), ("k", k), ("v", v), ("pos", pos), ("gamma_q", gamma_q),
                    ("gamma_k", gamma_k)):
        if t is None and given and name in ("pos", "gamma_q", "gamma_k"):
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if q.dtype == torch.bfloat16:
        dt = MRA_BF16
    elif q.dtype == torch.float32:
        dt = MRA_FP32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    b, s, h, d = q.shape
    if tuple(k.shape) != (b, s, h, d) or tuple(v.shape) != (b, s, h, d):
        raise ValueError("q, k, v shapes differ")
    if pos is not None and (pos.dtype != torch.int32 or tuple(pos.shape) != (b, s, 3)
                            or not pos.is_contiguous()):
        raise ValueError("pos must be contiguous int32 [B, S, 3]")
    # gammas: both [D] (shared by the heads) or both [H, D] (one per head)
    gshape = None if gamma_q is None else tuple(gamma_q.shape)
    for name, g in (("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        if g is not None and (g.dtype != torch.float32 or tuple(g.shape) not in ((d,), (h, d))
                              or tuple(g.shape) != gshape or not g.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 [D] or [H, D], like the other gamma")
    if seq_lens is not None:
        if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (b,) or not seq_lens.is_cuda:
            raise ValueError("seq_lens must be a GPU int32 [B] tensor")
        seq_lens = seq_lens.contiguous()
    if out is None:
        out = torch.empty((b, s, h, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((b, h, s), dtype=torch.float32, device=q.device) if return_lse else None
    desc = make_desc(b, s, h, d, text_pad=text_pad, section=section, theta=theta, eps=eps,
                     scale=scale, dtype=dt, kprologue=kprologue, q_stride=_bsd_strides(q),
                     k_stride=_bsd_strides(k), v_stride=_bsd_strides(v), o_stride=_bsd_strides(out),
                     rope_pairs=rope_pairs, gamma_per_head=gshape is not None and len(gshape) == 2)
    return desc, out, lse, seq_lens


def mrope_attn(q, k, v, pos, gamma_q, gamma_k, seq_lens=None, *, text_pad: int,
               section=(16, 24, 24), theta: float = 10000.0, eps: float = 1e-6, scale=None,
               return_lse: bool = False, kprologue="auto", out=None, workspace=None,
               stage: str = "fwd", rope_pairs="half"):
    """Fused QK-RMSNorm + 3D M-RoPE joint attention on the current HIP stream.

    q, k, v: [B, S, H, D] bf16 or fp32 GPU tensors (head_dim contiguous; any
    batch/token/head strides, e.g. views of one fused qkv buffer).
    pos: [B, S, 3] int32 (t, h, w). gamma_q, gamma_k: [D] fp32 (shared by
    the heads) or [H, D] (one per head).
    seq_lens: [B] int32 true text lengths (<= text_pad) or None.
    rope_pairs: "half" (pairs (j, j + D/2)) or "interleaved" ((2j, 2j + 1)).
    Returns out [B, S, H, D] (q's dtype), and lse [B, H, S] fp32 if asked.
    """
    import torch

    desc, out, lse, seq_lens = _checked(q, k, v, pos, gamma_q, gamma_k, seq_lens, out, return_lse,
                                        text_pad=text_pad, section=section, theta=theta, eps=eps,
                                        scale=scale, kprologue=kprologue, rope_pairs=rope_pairs)
    need = workspace_size(desc)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    ws = None if not need else workspace.data_ptr()
    if stage in ("fwd", "attend"):
        fn = lib().mrope_attn_fwd if stage == "fwd" else lib().mrope_attn_attend
        ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        rc = fn(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), ptr(pos),
                ptr(gamma_q), ptr(gamma_k),
                None if seq_lens is None else seq_lens.data_ptr(), out.data_ptr(),
                None if lse is None else lse.data_ptr(), ws, need, stream)
    elif stage == "prepare":
        rc = lib().mrope_attn_prepare(ctypes.byref(desc), k.data_ptr(),
                                      None if pos is None else pos.data_ptr(),
                                      None if gamma_k is None else gamma_k.data_ptr(), ws, need, stream)
    else:
        raise ValueError(f"unknown stage {stage}")
    if rc != 0:
        raise _error(rc)
    return (out, lse) if return_lse else out


NOALLOC_SCRATCH_BYTES = 64 << 20


def mrope_attn_noalloc(q, k, v, pos, gamma_q, gamma_k, seq_lens=None, *, text_pad: int, out,
                       lse=None, section=(16, 24, 24), theta: float = 10000.0, eps: float = 1e-6,
                       scale=None, kprologue="auto", rope_pairs="half"):
    """The forward through ``mrope_attn_fwd_noalloc``: arguments as for
    :func:`mrope_attn`, but the caller passes ``out`` (and ``lse`` [B, H, S]
    fp32, or None) and no workspace: the library's own per-GPU scratch array
    (``NOALLOC_SCRATCH_BYTES``) holds the intermediates. Calls that overlap
    in time on one GPU race on that array. Returns ``out``."""
    import torch

    desc, out, _, seq_lens = _checked(q, k, v, pos, gamma_q, gamma_k, seq_lens, out, False,
                                      text_pad=text_pad, section=section, theta=theta, eps=eps,
                                      scale=scale, kprologue=kprologue, rope_pairs=rope_pairs)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[0], q.shape[2], q.shape[1])
                            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse must be a contiguous float32 [B, H, S] GPU tensor")
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().mrope_attn_fwd_noalloc(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), ptr(pos),
                                      ptr(gamma_q), ptr(gamma_k), ptr(seq_lens), out.data_ptr(), ptr(lse),
                                      stream)
    if rc != 0:
        raise _error(rc)
    return out


def prepared_call(q, k, v, pos, gamma_q, gamma_k, seq_lens=None, **kw):
    """(prepare, attend): two closures running the two stages of one call on
    the current stream with shared output / workspace buffers, so a caller
    can place events between them (used by the benchmark)."""
    import torch
    b, s, h, d = q.shape
    desc = make_desc(b, s, h, d, text_pad=kw["text_pad"], section=kw.get("section", (16, 24, 24)),
                     kprologue=kw.get("kprologue", "auto"),
                     dtype=MRA_BF16 if q.dtype == torch.bfloat16 else MRA_FP32)
    need = workspace_size(desc)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    common = dict(kw, out=out, workspace=ws)

    def prepare():
        return mrope_attn(q, k, v, pos, gamma_q, gamma_k, seq_lens, stage="prepare", **common)

    def attend():
        return mrope_attn(q, k, v, pos, gamma_q, gamma_k, seq_lens, stage="attend", **common)

    return prepare, attend, out


def group_workspace_size(descs) -> int:
    arr = (Desc * len(descs))(*descs)
    return int(lib().mrope_attn_group_workspace_size(arr, len(descs)))


def mrope_attn_group(problems, *, return_lse: bool = False, kprologue="auto", workspace=None):
    """Several attention problems in one attention launch (e.g. the
    conditional [text + image] and unconditional [image only] passes of one
    guided sampling step). ``problems`` is a list of dicts with the arguments
    of :func:`mrope_attn`: q, k, v, pos, gamma_q, gamma_k, and optionally
    seq_lens, text_pad (default 0), section, theta, eps, scale, rope_pairs, out.
    Returns the list of outputs (of (out, lse) pairs if ``return_lse``)."""
    import torch

    if not 1 <= len(problems) <= MAX_GROUP:
        raise ValueError(f"1..{MAX_GROUP} problems per group")
    descs, probs, results = [], [], []
    for p in problems:
        desc, out, lse, sl = _checked(
            p["q"], p["k"], p["v"], p["pos"], p["gamma_q"], p["gamma_k"], p.get("seq_lens"),
            p.get("out"), return_lse, text_pad=p.get("text_pad", 0),
            section=p.get("section", (16, 24, 24)), theta=p.get("theta", 10000.0),
            eps=p.get("eps", 1e-6), scale=p.get("scale"), kprologue=kprologue,
            rope_pairs=p.get("rope_pairs", "half"))
        descs.append(desc)
        probs.append(Problem(p["q"].data_ptr(), p["k"].data_ptr(), p["v"].data_ptr(),
                             p["pos"].data_ptr(), p["gamma_q"].data_ptr(), p["gamma_k"].data_ptr(),
                             None if sl is None else sl.data_ptr(), out.data_ptr(),
                             None if lse is None else lse.data_ptr()))
        results.append((out, lse) if return_lse else out)
    n = len(descs)
    darr = (Desc * n)(*descs)
    parr = (Problem * n)(*probs)
    need = int(lib().mrope_attn_group_workspace_size(darr, n))
    dev = problems[0]["q"].device
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().mrope_attn_fwd_group(darr, parr, n, None if not need else workspace.data_ptr(),
                                    need, stream)
    if rc != 0:
        raise _error(rc)
    return results


def mrope_attn_varlen(q, k, v, pos, gamma_q, gamma_k, cu_seqlens, max_seqlen: int, *,
                      section=(16, 24, 24), theta: float = 10000.0, eps: float = 1e-6,
                      scale=None, return_lse: bool = False, kprologue="auto", out=None,
                      workspace=None, rope_pairs="half"):
    """Packed variable-length form: q, k, v [T, H, D], pos [T, 3] int32,
    cu_seqlens [B + 1] int32 on the GPU (sequence b = tokens cu[b]:cu[b+1]),
    max_seqlen >= every sequence length. Returns out [T, H, D] (and lse
    [H, T] if asked)."""
    import torch

    if q.dim() != 3:
        raise ValueError("q, k, v must be [T, H, D] for the packed form")
    t, h, d = q.shape
    if pos.dim() != 2:
        raise ValueError("pos must be [T, 3] for the packed form")
    if not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a GPU int32 [B + 1] tensor")
    cu_seqlens = cu_seqlens.contiguous()
    nseq = cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty((t, h, d), dtype=q.dtype, device=q.device)
    desc, out4, lse, _ = _checked(q[None], k[None], v[None], pos[None], gamma_q, gamma_k, None,
                                  out[None], False, text_pad=0, section=section, theta=theta,
                                  eps=eps, scale=scale, kprologue=kprologue, rope_pairs=rope_pairs)
    lse = torch.empty((h, t), dtype=torch.float32, device=q.device) if return_lse else None
    desc.batch = nseq
    need = int(lib().mrope_attn_varlen_workspace_size(ctypes.byref(desc), int(max_seqlen)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().mrope_attn_fwd_varlen(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     pos.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(),
                                     cu_seqlens.data_ptr(), int(max_seqlen), out.data_ptr(),
                                     None if lse is None else lse.data_ptr(),
                                     None if not need else workspace.data_ptr(), need, stream)
    if rc != 0:
        raise _error(rc)
    return (out, lse) if return_lse else out


def mrope_attn_bwd(q, k, v, pos, gamma_q, gamma_k, seq_lens, out, lse, dout, *, text_pad: int,
                   section=(16, 24, 24), theta: float = 10000.0, eps: float = 1e-6, scale=None,
                   dq=None, dk=None, dv=None, workspace=None, rope_pairs="half"):
    """Backward of :func:`mrope_attn` (bf16, head_dim 128): gradients of
    sum(dout * out) given the forward's out and lse. Returns (dq, dk, dv,
    dgamma_q, dgamma_k); dq/dk/dv take q/k/v's strides, dout out's, and each
    dgamma its gamma's shape."""
    import torch

    desc, out_, _, seq_lens = _checked(q, k, v, pos, gamma_q, gamma_k, seq_lens, out, False,
                                       text_pad=text_pad, section=section, theta=theta, eps=eps,
                                       scale=scale, kprologue="auto", rope_pairs=rope_pairs)
    if tuple(dout.shape) != tuple(q.shape) or _bsd_strides(dout) != _bsd_strides(out):
        raise ValueError("dout must have out's shape and strides")
    b, s, h, d = q.shape
    if lse is None or lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, s) or not lse.is_contiguous():
        raise ValueError("lse must be the forward's contiguous float32 [B, H, S] log-sum-exp")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or _bsd_strides(t) != _bsd_strides(ref):
            raise ValueError(f"{name} must have the strides of its input")
    dgq = torch.empty(gamma_q.shape, dtype=torch.float32, device=q.device)
    dgk = torch.empty(gamma_k.shape, dtype=torch.float32, device=q.device)
    need = int(lib().mrope_attn_bwd_workspace_size(ctypes.byref(desc)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().mrope_attn_bwd(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              pos.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(),
                              None if seq_lens is None else seq_lens.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), dgq.data_ptr(), dgk.data_ptr(),
                              None if not need else workspace.data_ptr(), need, stream)
    if rc != 0:
        raise _error(rc)
    return dq, dk, dv, dgq, dgk


def mrope_attn_bwd_varlen(q, k, v, pos, gamma_q, gamma_k, cu_seqlens, max_seqlen: int, out, lse,
                          dout, *, section=(16, 24, 24), theta: float = 10000.0, eps: float = 1e-6,
                          scale=None, dq=None, dk=None, dv=None, workspace=None,
                          rope_pairs="half"):
    """Backward of :func:`mrope_attn_varlen` (bf16, head_dim 128): q, k, v,
    out, dout [T, H, D], pos [T, 3], cu_seqlens [B + 1] int32 on the GPU, lse
    the forward's [H, T]. Returns (dq, dk, dv, dgamma_q, dgamma_k); rows of
    tokens outside every sequence are left as they were in dq, dk, dv."""
    import torch

    if q.dim() != 3 or pos.dim() != 2:
        raise ValueError("q, k, v must be [T, H, D] and pos [T, 3] for the packed form")
    if not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a GPU int32 [B + 1] tensor")
    cu_seqlens = cu_seqlens.contiguous()
    t, h, d = q.shape
    desc, _, _, _ = _checked(q[None], k[None], v[None], pos[None], gamma_q, gamma_k, None, out[None],
                             False, text_pad=0, section=section, theta=theta, eps=eps, scale=scale,
                             kprologue="auto", rope_pairs=rope_pairs)
    desc.batch = cu_seqlens.numel() - 1
    if tuple(dout.shape) != tuple(q.shape) or _bsd_strides(dout[None]) != _bsd_strides(out[None]):
        raise ValueError("dout must have out's shape and strides")
    if lse is None or lse.dtype != torch.float32 or tuple(lse.shape) != (h, t) or not lse.is_contiguous():
        raise ValueError("lse must be the forward's contiguous float32 [H, T] log-sum-exp")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, tt, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if tt.shape != ref.shape or _bsd_strides(tt[None]) != _bsd_strides(ref[None]):
            raise ValueError(f"{name} must have the strides of its input")
    dgq = torch.empty(gamma_q.shape, dtype=torch.float32, device=q.device)
    dgk = torch.empty(gamma_k.shape, dtype=torch.float32, device=q.device)
    need = int(lib().mrope_attn_bwd_varlen_workspace_size(ctypes.byref(desc), int(max_seqlen)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().mrope_attn_bwd_varlen(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     pos.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(),
                                     cu_seqlens.data_ptr(), int(max_seqlen), out.data_ptr(),
                                     lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                     dv.data_ptr(), dgq.data_ptr(), dgk.data_ptr(),
                                     None if not need else workspace.data_ptr(), need, stream)
    if rc != 0:
        raise _error(rc)
    return dq, dk, dv, dgq, dgk


def make_qkv_desc(tokens, hidden, heads, head_dim=128, *, section=(16, 24, 24), theta=10000.0,
                  eps=1e-6, scale=None, x_stride=None, q_stride=None, k_stride=None,
                  v_stride=None, rope_pairs="half", gamma_per_head=False) -> QkvDesc:
    d = QkvDesc()
    d.rope_pairs = _pairs(rope_pairs)
    d.gamma_per_head = int(gamma_per_head)
    d.tokens, d.hidden, d.heads, d.head_dim = tokens, hidden, heads, head_dim
    d.section[:] = [int(x) for x in section]
    d.theta, d.eps = float(theta), float(eps)
    d.softmax_scale = 0.0 if scale is None else float(scale)
    d.x_stride = hidden if x_stride is None else int(x_stride)
    cont = (heads * head_dim, head_dim)
    for name, st in (("q_stride", q_stride), ("k_stride", k_stride), ("v_stride", v_stride)):
        getattr(d, name)[:] = list(cont if st is None else st)
    return d


def mrope_qkv_proj(x, w8, w_scale, pos, gamma_q, gamma_k, *, heads: int, section=(16, 24, 24),
                   theta: float = 10000.0, eps: float = 1e-6, scale=None, out=None, workspace=None,
                   rope_pairs="half"):
    """fp8 e4m3 QKV projection with the norm/rotation epilogue.

    x [M, hidden] bf16, w8 [3 H D, hidden] uint8 (e4m3 codes), w_scale [3 H D]
    fp32, pos [M, 3] int32, gammas [D] or [H, D] fp32. Returns (q_op, k_op,
    v), each [M, H, D] bf16: the operands mrope_attn takes with
    kprologue="none"."""
    import torch

    for name, t in (("x", x), ("w8", w8), ("w_scale", w_scale), ("pos", pos), ("gamma_q", gamma_q),
                    ("gamma_k", gamma_k)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be bf16 [M, hidden] with contiguous rows")
    m, hidden = x.shape
    d = gamma_q.shape[-1]
    for name, g in (("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        if (g.dtype != torch.float32 or tuple(g.shape) not in ((d,), (heads, d))
                or g.shape != gamma_q.shape or not g.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 [D] or [H, D], like the other gamma")
    if w8.dtype != torch.uint8 or tuple(w8.shape) != (3 * heads * d, hidden) or not w8.is_contiguous():
        raise ValueError("w8 must be contiguous uint8 [3 H D, hidden]")
    if w_scale.dtype != torch.float32 or w_scale.numel() != 3 * heads * d or not w_scale.is_contiguous():
        raise ValueError("w_scale must be contiguous float32 [3 H D]")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (m, 3) or not pos.is_contiguous():
        raise ValueError("pos must be contiguous int32 [M, 3]")
    if out is None:
        out = tuple(torch.empty((m, heads, d), dtype=torch.bfloat16, device=x.device) for _ in range(3))
    st = [(t.stride(0), t.stride(1)) for t in out]
    desc = make_qkv_desc(m, hidden, heads, d, section=section, theta=theta, eps=eps, scale=scale,
                         x_stride=x.stride(0), q_stride=st[0], k_stride=st[1], v_stride=st[2],
                         rope_pairs=rope_pairs, gamma_per_head=gamma_q.dim() == 2)
    need = int(lib().mrope_qkv_proj_workspace_size(ctypes.byref(desc)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = lib().mrope_qkv_proj(ctypes.byref(desc), x.data_ptr(), w8.data_ptr(), w_scale.data_ptr(),
                              pos.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(), out[0].data_ptr(),
                              out[1].data_ptr(), out[2].data_ptr(),
                              None if not need else workspace.data_ptr(), need, stream)
    if rc != 0:
        raise _error(rc)
    return out
