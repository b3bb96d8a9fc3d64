"""Float64 oracle of the fp8 QKV projection feeding the attention hot path.

TEST INFRASTRUCTURE ONLY -- imported by tests and the bench's CPU-baseline
leg, never by the product path.

The Ideogram 4 checkpoint stores the DiT attention's Q, K and V projections as
one fused weight with the Q, K and V rows stacked ([3 * hidden, hidden]), and
every quantized weight as float8 e4m3 with a per-output-channel scale: the
real weight is the fp8 value times the scale of its output row (unsloth commit
log for the Ideogram 4 backend, the fp8 loader commit). The projection feeds
the QK-RMSNorm and 3D M-RoPE of the attention (Ideogram 4.0 announcement
thread), so the fused form returns the attention's operands directly:

  y = x W^T with W[o, i] = e4m3(w8[o, i]) * w_scale[o];
  q, k, v = the three row blocks of y, each [M, H, D];
  q_op = qscale * rope(rmsnorm(q) * gamma_q),  k_op = rope(rmsnorm(k) * gamma_k),
  v_op = v,
with qscale the query factor the attention folds in (softmax scale * log2 e).
"""

from __future__ import annotations

import numpy as np

from oracle.reference import mrope, rms_norm


def e4m3_decode(codes) -> np.ndarray:
    """OCP 8-bit float E4M3 (the float8_e4m3fn of the checkpoint): sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
    (m / 8 * 2^-6); exponent 15 with mantissa 7 is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return s * val


def oracle_qkv_proj(x, w8, w_scale, pos, gamma_q, gamma_k, *, heads: int, head_dim: int,
                    section=(16, 24, 24), theta: float = 10000.0, eps: float = 1e-6,
                    qscale: float = 1.0, rows=None, rope_pairs: str = "half"):
    """x [M, hidden], w8 [3 H D, hidden] e4m3 codes, w_scale [3 H D], pos [M, 3],
    gamma_q and gamma_k [D] or [H, D].
    Returns (q_op, k_op, v_op), each [R, H, D] float64 for the rows `rows`
    (all by default)."""
    x = np.asarray(x, dtype=np.float64)
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    w = e4m3_decode(w8) * np.asarray(w_scale, dtype=np.float64)[:, None]
    y = x[rows] @ w.T                                          # [R, 3 H D]
    hd = heads * head_dim
    q = y[:, :hd].reshape(len(rows), heads, head_dim)
    k = y[:, hd:2 * hd].reshape(len(rows), heads, head_dim)
    v = y[:, 2 * hd:].reshape(len(rows), heads, head_dim)
    p = np.asarray(pos)[rows][None]                            # [1, R, 3]
    q_op = qscale * mrope(rms_norm(q[None], gamma_q, eps), p, section, theta, rope_pairs)[0]
    k_op = mrope(rms_norm(k[None], gamma_k, eps), p, section, theta, rope_pairs)[0]
    return q_op, k_op, v
