"""Seeded synthetic workloads for the joint text+image attention path.

This module only draws random numbers and lays out token positions; it holds
none of the attention arithmetic. Both the GPU library's tests/bench and the
CPU oracle consume what it returns.

Token layout (Ideogram 4 deep dive, section 4 part 2: text and image tokens
form one sequence; part 6, the generation sketch: the latent is a
``grid_h * grid_w`` raster of tokens; part 5: 16x spatial compression, so a
1024x1024 image is a 64x64 token grid): ``text_pad`` text slots first, then
the image grid in row-major order. Positions put everything in one (t, h, w)
frame (Ideogram 4.0 announcement thread): text slot i gets (i, i, i); image
token (r, c) gets (L, L + r, L + c) with L the item's true text length; a
padded text slot keeps (i, i, i) (it is masked anyway).

Values: q, k, v ~ N(0, sigma^2) drawn in float32, gamma_q, gamma_k ~
U[0.5, 1.5) ([D] each, or [H, D] each with ``gamma_per_head``), in that
order from ``numpy.random.default_rng(seed)``. For bf16
workloads q, k, v are rounded to bf16 (round-to-nearest-even) and returned as
float32 arrays holding bf16-exact values, so the device cast is exact.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# The five named shapes. Image grids: tiny 4x4, 512px 32x32, 1024px 64x64,
# long 128x96 (non-square; gh=128 rows, gw=96 columns).
CONFIGS = {
    "tiny": dict(batch=1, heads=1, head_dim=64, section=(8, 12, 12), text_pad=16,
                 text_lens=None, grid_h=4, grid_w=4, sigma=1.0, dtype="fp32", seed=0),
    "512px": dict(batch=1, heads=24, head_dim=128, section=(16, 24, 24), text_pad=256,
                  text_lens=None, grid_h=32, grid_w=32, sigma=1.0, dtype="bf16", seed=1),
    "1024px": dict(batch=1, heads=32, head_dim=128, section=(16, 24, 24), text_pad=512,
                   text_lens=None, grid_h=64, grid_w=64, sigma=1.0, dtype="bf16", seed=2),
    "ragged": dict(batch=4, heads=32, head_dim=128, section=(16, 24, 24), text_pad=512,
                   text_lens=(37, 128, 300, 512), grid_h=64, grid_w=64, sigma=1.0,
                   dtype="bf16", seed=3),
    "long": dict(batch=1, heads=32, head_dim=128, section=(16, 24, 24), text_pad=512,
                 text_lens=None, grid_h=128, grid_w=96, sigma=1.5, dtype="bf16", seed=4),
    # variants beyond the measured set: 36 heads of 128 (hidden 4608) at
    # 1024px, and the largest side the pages allow (2048 px -> 128x128 tokens)
    "h36": dict(batch=1, heads=36, head_dim=128, section=(16, 24, 24), text_pad=512,
                text_lens=None, grid_h=64, grid_w=64, sigma=1.0, dtype="bf16", seed=5),
    "2048px": dict(batch=1, heads=32, head_dim=128, section=(16, 24, 24), text_pad=512,
                   text_lens=None, grid_h=128, grid_w=128, sigma=1.0, dtype="bf16", seed=6),
    # the 1024px ragged batch under the other conventions: a gamma per head
    # and interleaved rotary pairs (2j, 2j + 1)
    "conv": dict(batch=2, heads=32, head_dim=128, section=(16, 24, 24), text_pad=512,
                 text_lens=(77, 512), grid_h=64, grid_w=64, sigma=1.0, dtype="bf16", seed=7,
                 gamma_per_head=True, rope_pairs="interleaved"),
    # one GPU's share of the 1024px layer when its 32 heads are split over 8
    # GPUs (heads need no exchange): 4 heads x 4608 tokens
    "h4": dict(batch=1, heads=4, head_dim=128, section=(16, 24, 24), text_pad=512,
               text_lens=None, grid_h=64, grid_w=64, sigma=1.0, dtype="bf16", seed=8),
}


@dataclass
class Workload:
    q: np.ndarray          # [B, S, H, D] float32 (bf16-exact when dtype == "bf16")
    k: np.ndarray
    v: np.ndarray
    pos: np.ndarray        # [B, S, 3] int32, (t, h, w)
    gamma_q: np.ndarray    # [D] or [H, D] float32
    gamma_k: np.ndarray
    seq_lens: np.ndarray | None   # [B] int32 or None (no padding)
    text_pad: int
    section: tuple
    dtype: str
    theta: float = 10000.0
    eps: float = 1e-6
    grid: tuple = field(default=(0, 0))
    rope_pairs: str = "half"   # rotary pair layout: "half" or "interleaved"

    @property
    def shape(self):
        return self.q.shape

    def valid_counts(self):
        """Real tokens per item: true text length + image tokens."""
        b, s = self.q.shape[:2]
        if self.seq_lens is None:
            return [s] * b
        img = s - self.text_pad
        return [int(min(max(l, 0), self.text_pad)) + img for l in self.seq_lens]

    def flops(self):
        """Algorithmic FLOPs of the two contractions over real tokens only."""
        _, _, h, d = self.q.shape
        return 4 * h * d * sum(n * n for n in self.valid_counts())


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), kept as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def positions(batch: int, text_pad: int, grid_h: int, grid_w: int, text_lens=None) -> np.ndarray:
    """(t, h, w) positions [B, S, 3] int32 for text slots then the image raster."""
    s = text_pad + grid_h * grid_w
    pos = np.zeros((batch, s, 3), dtype=np.int32)
    ti = np.arange(text_pad, dtype=np.int32)
    rr, cc = np.meshgrid(np.arange(grid_h, dtype=np.int32),
                         np.arange(grid_w, dtype=np.int32), indexing="ij")
    rr = rr.reshape(-1)
    cc = cc.reshape(-1)
    for b in range(batch):
        lb = text_pad if text_lens is None else int(min(max(text_lens[b], 0), text_pad))
        pos[b, :text_pad, :] = ti[:, None]
        pos[b, text_pad:, 0] = lb
        pos[b, text_pad:, 1] = lb + rr
        pos[b, text_pad:, 2] = lb + cc
    return pos


def make_workload(batch, heads, head_dim, section, text_pad, grid_h, grid_w,
                  text_lens=None, sigma=1.0, dtype="bf16", seed=0,
                  theta=10000.0, eps=1e-6, gamma_per_head=False,
                  rope_pairs="half") -> Workload:
    """Draw one seeded workload (see the module docstring for the recipe)."""
    s = text_pad + grid_h * grid_w
    rng = np.random.default_rng(seed)
    shp = (batch, s, heads, head_dim)
    q = rng.standard_normal(shp, dtype=np.float32)
    k = rng.standard_normal(shp, dtype=np.float32)
    v = rng.standard_normal(shp, dtype=np.float32)
    if sigma != 1.0:
        q *= np.float32(sigma)
        k *= np.float32(sigma)
        v *= np.float32(sigma)
    gshape = (heads, head_dim) if gamma_per_head else head_dim
    gq = rng.uniform(0.5, 1.5, gshape).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, gshape).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype}")
    lens = None if text_lens is None else np.asarray(text_lens, dtype=np.int32)
    return Workload(q=q, k=k, v=v, pos=positions(batch, text_pad, grid_h, grid_w, text_lens),
                    gamma_q=gq, gamma_k=gk, seq_lens=lens, text_pad=text_pad,
                    section=tuple(section), dtype=dtype, theta=theta, eps=eps,
                    grid=(grid_h, grid_w), rope_pairs=rope_pairs)


def config_workload(name: str) -> Workload:
    """The named configuration with its own seed."""
    return make_workload(**CONFIGS[name])


@dataclass
class VarlenWorkload:
    """Sequences packed back to back (no padding): q, k, v [T, H, D],
    pos [T, 3], cu_seqlens [B + 1]."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    pos: np.ndarray
    gamma_q: np.ndarray
    gamma_k: np.ndarray
    cu_seqlens: np.ndarray
    section: tuple
    dtype: str
    theta: float = 10000.0
    eps: float = 1e-6
    rope_pairs: str = "half"

    @property
    def max_seqlen(self):
        return int(np.max(np.diff(self.cu_seqlens))) if len(self.cu_seqlens) > 1 else 0

    def flops(self):
        _, h, d = self.q.shape
        return 4 * h * d * int(sum(int(n) ** 2 for n in np.diff(self.cu_seqlens)))


def make_varlen_workload(heads, head_dim, section, text_lens, grids, sigma=1.0, dtype="bf16",
                         seed=0, gamma_per_head=False, rope_pairs="half") -> VarlenWorkload:
    """Sequence b = text_lens[b] real text tokens then a grids[b] = (gh, gw)
    image raster, each drawn as its own unpadded one-item workload (seed +
    b), with the first item's gammas shared by all."""
    parts = [make_workload(1, heads, head_dim, section, int(l), gh, gw, sigma=sigma, dtype=dtype,
                           seed=seed + b, gamma_per_head=gamma_per_head)
             for b, (l, (gh, gw)) in enumerate(zip(text_lens, grids))]
    lens = [p.q.shape[1] for p in parts]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cat = lambda f: np.ascontiguousarray(np.concatenate([getattr(p, f)[0] for p in parts]))  # noqa: E731
    return VarlenWorkload(q=cat("q"), k=cat("k"), v=cat("v"), pos=cat("pos"),
                          gamma_q=parts[0].gamma_q, gamma_k=parts[0].gamma_k, cu_seqlens=cu,
                          section=tuple(section), dtype=dtype, rope_pairs=rope_pairs)


@dataclass
class QkvWorkload:
    """Inputs of the fp8 QKV projection for a [batch, text_pad + image]
    layout: x [B*S, hidden] (bf16-exact), w8 [3 H D, hidden] e4m3 codes,
    w_scale [3 H D], pos [B*S, 3]."""
    x: np.ndarray
    w8: np.ndarray
    w_scale: np.ndarray
    pos: np.ndarray
    gamma_q: np.ndarray
    gamma_k: np.ndarray
    batch: int
    seq: int
    heads: int
    head_dim: int
    text_pad: int
    section: tuple
    rope_pairs: str = "half"

    def flops(self):
        return 2 * self.x.shape[0] * self.x.shape[1] * self.w8.shape[0]


def make_qkv_workload(batch, heads, head_dim, section, text_pad, grid_h, grid_w, hidden,
                      seed=0, gamma_per_head=False, rope_pairs="half") -> QkvWorkload:
    """x ~ N(0, 1) rounded to bf16; a dense weight ~ N(0, 1/hidden) quantized
    per output row to float8 e4m3 (scale = row max / 448, round to nearest via
    the library's float8_e4m3fn cast), as the checkpoint stores it."""
    import torch
    rng = np.random.default_rng(seed)
    s = text_pad + grid_h * grid_w
    m = batch * s
    x = round_to_bf16(rng.standard_normal((m, hidden), dtype=np.float32))
    n = 3 * heads * head_dim
    w = rng.standard_normal((n, hidden), dtype=np.float32) / np.float32(np.sqrt(hidden))
    scale = (np.abs(w).max(axis=1) / 448.0).astype(np.float32)
    codes = torch.from_numpy(w / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    gshape = (heads, head_dim) if gamma_per_head else head_dim
    gq = rng.uniform(0.5, 1.5, gshape).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, gshape).astype(np.float32)
    pos = positions(batch, text_pad, grid_h, grid_w).reshape(m, 3)
    return QkvWorkload(x=x, w8=np.ascontiguousarray(codes), w_scale=scale, pos=np.ascontiguousarray(pos),
                       gamma_q=gq, gamma_k=gk, batch=batch, seq=s, heads=heads, head_dim=head_dim,
                       text_pad=text_pad, section=tuple(section), rope_pairs=rope_pairs)
