"""Float64 oracle of the backward pass of the attention hot path.

TEST INFRASTRUCTURE ONLY -- imported by tests and the bench's CPU-baseline
leg, never by the product path.

The forward pass is the one in ``oracle.reference`` (Ideogram 4.0
announcement thread: QK-RMSNorm and 3D M-RoPE inside the single-stream DiT's
self-attention; "Ideogram 4 deep dive", section 4 part 2: one joint
sequence). Its gradients are what LoRA training on the attention projections
needs (SimpleTuner quickstart: LoRA training of the Ideogram 4 DiT with
gradient checkpointing, which recomputes the forward). They are written out
by the chain rule, step by step in reverse order of the forward:

4. attention  O = softmax(scale * Q' K'^T) V over valid keys:
     dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id,
     dS = P * (dP - D),  dQ' = scale dS K',  dK' = scale dS^T Q';
3. M-RoPE  x' = R(phi) x_hat: the transpose rotation, by -phi, of each pair;
2. RMSNorm x_hat = x r gamma with r = (mean(x^2) + eps)^-1/2:
     dgamma_d = sum_rows dx_hat_d x_d r,
     dx_d = r gamma_d dx_hat_d - (r^3 / D) x_d sum_e dx_hat_e gamma_e x_e.
Padded query rows have a constant zero output, padded keys are excluded:
neither carries gradient. A [D] gamma is shared by every head and token, so
its gradient sums over all valid rows; an [H, D] gamma gets one gradient row
per head, summed over that head's rows.
"""

from __future__ import annotations

import numpy as np

from oracle.reference import axis_of_pair, inv_freq, pair_slots, valid_tokens


def _angles(pos, section, head_dim, theta):
    half = head_dim // 2
    axis = axis_of_pair(section, half)
    ang = np.asarray(pos, dtype=np.float64)[:, :, axis] * inv_freq(head_dim, theta)
    return np.cos(ang)[:, :, None, :], np.sin(ang)[:, :, None, :]


def _rotate(x, c, s, sign, pairs):
    """Turn every rotary pair (x_a, x_b) of the given layout by sign * phi."""
    ia, ib = pair_slots(x.shape[-1], pairs)
    x1, x2 = x[..., ia], x[..., ib]
    out = np.empty_like(x)
    out[..., ia] = x1 * c - sign * x2 * s
    out[..., ib] = x2 * c + sign * x1 * s
    return out


def oracle_bwd(q, k, v, pos, gamma_q, gamma_k, seq_lens, dout, *, text_pad: int,
               section=(16, 24, 24), theta: float = 10000.0, eps: float = 1e-6, scale=None,
               rope_pairs: str = "half"):
    """Gradients of sum(dout * out) for out = oracle_fwd(...).

    Returns (dq, dk, dv [B, S, H, D], dgamma_q, dgamma_k) in float64; each
    dgamma has its gamma's shape ([D] or [H, D]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    gq = np.asarray(gamma_q, dtype=np.float64)
    gk = np.asarray(gamma_k, dtype=np.float64)
    b_, s_, h_, d_ = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(np.float64(d_))
    c, s = _angles(pos, section, d_, theta)

    def norm(x, g):
        r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + np.float64(eps))
        return x * r * g, r

    xq, rq = norm(q, gq)
    xk, rk = norm(k, gk)
    qr = _rotate(xq, c, s, +1.0, rope_pairs)
    kr = _rotate(xk, c, s, +1.0, rope_pairs)
    valid = valid_tokens(b_, s_, text_pad, seq_lens)

    dqr = np.zeros_like(q)
    dkr = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(b_):
        kv = valid[b]
        if not kv.any():
            continue
        for h in range(h_):
            z = scale * (qr[b, :, h, :] @ kr[b, kv, h, :].T)      # all queries, valid keys
            z -= z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p /= p.sum(axis=1, keepdims=True)
            g = do[b, :, h, :] * kv[:, None]                      # padded query rows: no gradient
            o = p @ v[b, kv, h, :]
            dv[b, kv, h, :] = p.T @ g
            dp = g @ v[b, kv, h, :].T
            dlt = np.sum(g * o, axis=1, keepdims=True)
            ds = p * (dp - dlt)
            dqr[b, :, h, :] = scale * ds @ kr[b, kv, h, :]
            dkr[b, kv, h, :] = scale * ds.T @ qr[b, :, h, :]

    dxq = _rotate(dqr, c, s, -1.0, rope_pairs)
    dxk = _rotate(dkr, c, s, -1.0, rope_pairs)

    def norm_bwd(x, r, g, dxh):
        dg = np.sum(dxh * x * r, axis=(0, 1) if g.ndim == 2 else (0, 1, 2))
        inner = np.sum(dxh * g * x, axis=-1, keepdims=True)
        dx = r * g * dxh - (r ** 3 / x.shape[-1]) * x * inner
        return dx, dg

    dq, dgq = norm_bwd(q, rq, gq, dxq)
    dk, dgk = norm_bwd(k, rk, gk, dxk)
    return dq, dk, dv, dgq, dgk


def oracle_bwd_varlen(q, k, v, pos, gamma_q, gamma_k, cu_seqlens, dout, *, section=(16, 24, 24),
                      theta: float = 10000.0, eps: float = 1e-6, scale=None,
                      rope_pairs: str = "half"):
    """Gradients of sum(dout * out) for the packed form
    (``oracle.reference.oracle_fwd_varlen``): sequence b is tokens
    [cu_seqlens[b], cu_seqlens[b+1]) of q, k, v, dout [T, H, D] and pos
    [T, 3]. Each sequence is an independent padding-free problem, so its
    gradients are :func:`oracle_bwd` of that sequence alone; a gamma is
    shared by every sequence, so its gradient is the sum over them.

    Returns (dq, dk, dv [T, H, D], dgamma_q, dgamma_k) in float64; rows of
    tokens outside every sequence are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    t_, h_, d_ = q.shape
    dq = np.full((t_, h_, d_), np.nan)
    dk = np.full((t_, h_, d_), np.nan)
    dv = np.full((t_, h_, d_), np.nan)
    dgq = np.zeros(np.shape(gamma_q))
    dgk = np.zeros(np.shape(gamma_k))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(len(cu) - 1):
        a0, a1 = int(cu[b]), int(cu[b + 1])
        if a1 <= a0:
            continue
        r = oracle_bwd(q[None, a0:a1], np.asarray(k)[None, a0:a1], np.asarray(v)[None, a0:a1],
                       np.asarray(pos)[None, a0:a1], gamma_q, gamma_k, None,
                       np.asarray(dout)[None, a0:a1], text_pad=0, section=section, theta=theta,
                       eps=eps, scale=scale, rope_pairs=rope_pairs)
        dq[a0:a1], dk[a0:a1], dv[a0:a1] = r[0][0], r[1][0], r[2][0]
        dgq += r[3]
        dgk += r[4]
    return dq, dk, dv, dgq, dgk
