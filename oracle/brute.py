"""Naive scalar-loop oracle for tiny inputs (pure Python, float64).

TEST INFRASTRUCTURE ONLY. Written independently of ``reference``: it walks
every scalar with Python loops, uses the complex-number form of the rotary
step and the ``math`` module, and shares no helper with the vectorised
oracle. The two must agree to rounding (1e-12) on tiny cases.

Same definition as ``reference`` (Ideogram 4.0 announcement thread: QK-RMSNorm
and 3D multimodal RoPE inside single-stream self-attention; "Ideogram 4 deep
dive", section 4 part 2 and section 6 part 3).
"""

from __future__ import annotations

import cmath
import math


def _axis(j: int, section) -> int:
    # pair j belongs to t, then h, then w, in contiguous blocks
    if j < section[0]:
        return 0
    if j < section[0] + section[1]:
        return 1
    return 2


def _prologue_row(x, gamma, p3, section, theta, eps, pairs="half"):
    """RMSNorm then M-RoPE of one head row x (a list of D floats). Rotary
    pair j is the complex number (x_j, x_{j+D/2}) for pairs="half", or
    (x_2j, x_2j+1) for pairs="interleaved"."""
    d = len(x)
    half = d // 2
    acc = 0.0
    for xi in x:
        acc += float(xi) * float(xi)
    r = 1.0 / math.sqrt(acc / d + eps)
    xn = [float(x[i]) * r * float(gamma[i]) for i in range(d)]
    out = [0.0] * d
    for j in range(half):
        phi = float(p3[_axis(j, section)]) * (float(theta) ** (-(2.0 * j) / d))
        a, b = (j, j + half) if pairs == "half" else (2 * j, 2 * j + 1)
        z = complex(xn[a], xn[b]) * cmath.exp(1j * phi)
        out[a] = z.real
        out[b] = z.imag
    return out


def brute_fwd(q, k, v, pos, gamma_q, gamma_k, seq_lens=None, *, text_pad,
              section, theta=10000.0, eps=1e-6, scale=None, rope_pairs="half"):
    """Returns (out, lse) as nested lists: out[b][s][h][d], lse[b][h][s].
    gamma_q and gamma_k are one list of D weights, or one such list per head."""
    bn = len(q)
    sn = len(q[0])
    hn = len(q[0][0])
    dn = len(q[0][0][0])
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(dn)
    out = [[[[0.0] * dn for _ in range(hn)] for _ in range(sn)] for _ in range(bn)]
    lse = [[[-math.inf] * sn for _ in range(hn)] for _ in range(bn)]
    for b in range(bn):
        if seq_lens is None:
            real = [True] * sn
        else:
            lb = min(max(int(seq_lens[b]), 0), text_pad)
            real = [(s >= text_pad) or (s < lb) for s in range(sn)]
        for h in range(hn):
            gq = gamma_q[h] if hasattr(gamma_q[0], "__len__") else gamma_q
            gk = gamma_k[h] if hasattr(gamma_k[0], "__len__") else gamma_k
            qp = [_prologue_row(q[b][s][h], gq, pos[b][s], section, theta, eps, rope_pairs)
                  for s in range(sn)]
            kp = [_prologue_row(k[b][s][h], gk, pos[b][s], section, theta, eps, rope_pairs)
                  for s in range(sn)]
            for i in range(sn):
                if not real[i]:
                    continue
                zs = []
                for j in range(sn):
                    if real[j]:
                        dot = 0.0
                        for c in range(dn):
                            dot += qp[i][c] * kp[j][c]
                        zs.append((j, scale * dot))
                zmax = max(z for _, z in zs)
                den = 0.0
                for _, z in zs:
                    den += math.exp(z - zmax)
                for c in range(dn):
                    num = 0.0
                    for j, z in zs:
                        num += math.exp(z - zmax) * float(v[b][j][h][c])
                    out[b][i][h][c] = num / den
                lse[b][h][i] = zmax + math.log(den)
    return out, lse
