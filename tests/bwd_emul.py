"""CPU emulation of where the bf16 backward kernels round, used to derive
the GPU parity bars of the backward pass (test infrastructure).

The kernels round Q'' = c2 * rope(rmsnorm(q)) and K' to bf16 (as the forward
does), recompute P from them and the forward's LSE, round P to bf16 (the dV
operand and the dS factor), round dS to bf16 (the dQ/dK operand), take D from
the forward's bf16 output, and round dq, dk, dv to bf16. Everything else is
float64 here.
"""

import numpy as np

from diffusion_transformer_image_head_amd.workloads import round_to_bf16 as bf
from oracle.backward import _angles, _rotate
from oracle.reference import mrope, oracle_fwd, rms_norm, valid_tokens


def emulate(w, do):
    q, k, v = (np.asarray(x, np.float64) for x in (w.q, w.k, w.v))
    b_, s_, h_, d_ = q.shape
    scale = d_ ** -0.5
    c2 = np.float32(scale * 1.4426950408889634)
    out, lse = oracle_fwd(w.q, w.k, w.v, w.pos, w.gamma_q, w.gamma_k, w.seq_lens, text_pad=w.text_pad, section=w.section)
    outb = bf(out.astype(np.float32)).astype(np.float64)
    qr = mrope(rms_norm(q, w.gamma_q, w.eps), w.pos, w.section, w.theta)
    kr = mrope(rms_norm(k, w.gamma_k, w.eps), w.pos, w.section, w.theta)
    q2 = bf((qr * c2).astype(np.float32)).astype(np.float64)
    k2 = bf(kr.astype(np.float32)).astype(np.float64)
    valid = valid_tokens(b_, s_, w.text_pad, w.seq_lens)
    dqr = np.zeros_like(q); dkr = np.zeros_like(q); dv = np.zeros_like(q)
    for b in range(b_):
        kv = valid[b]
        for h in range(h_):
            l2 = np.where(valid[b], lse[b, h] * np.log2(np.e), np.inf)
            s2 = q2[b, :, h] @ k2[b, kv, h].T
            p = np.exp2(s2 - l2[:, None])
            pb = bf(p.astype(np.float32)).astype(np.float64)
            g = do[b, :, h] * valid[b][:, None]
            dv[b, kv, h] = pb.T @ g
            dp = g @ v[b, kv, h].T
            D = np.sum(g * outb[b, :, h], axis=1, keepdims=True)
            ds = bf((pb * (dp - D)).astype(np.float32)).astype(np.float64)
            dqr[b, :, h] = scale * ds @ k2[b, kv, h]
            dkr[b, kv, h] = np.log(2) * ds.T @ q2[b, :, h]
    c, s = _angles(w.pos, w.section, d_, w.theta)
    dxq = _rotate(dqr, c, s, -1.0, "half"); dxk = _rotate(dkr, c, s, -1.0, "half")
    def nb(x, g, dxh):
        r = 1 / np.sqrt(np.mean(x * x, -1, keepdims=True) + w.eps)
        dg = np.sum(dxh * x * r, axis=(0, 1, 2))
        inner = np.sum(dxh * g * x, -1, keepdims=True)
        return r * g * dxh - r ** 3 / d_ * x * inner, dg
    dq, dgq = nb(q, w.gamma_q, dxq); dk, dgk = nb(k, w.gamma_k, dxk)
    r16 = lambda a: bf(a.astype(np.float32)).astype(np.float64)
    return r16(dq), r16(dk), r16(dv), dgq, dgk
