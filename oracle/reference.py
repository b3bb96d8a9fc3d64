"""Vectorised float64 oracle: the plain definition of the attention hot path.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
bench's CPU-baseline leg, never by the product path.

What is computed (Ideogram 4.0 announcement thread, the post that lists the
DiT's parts: a single-stream DiT whose self-attention applies QK-RMSNorm and
a 3D multimodal RoPE putting text and image tokens into one positional
frame; "Ideogram 4 deep dive", section 4 part 2 "DiT backbone": text and
image tokens are concatenated into one sequence and share every
self-attention layer):

1. RMSNorm over head_dim of every (batch, token, head) row of Q and of K,
   each with its own per-channel weight.
2. 3D M-RoPE: rotary pair j takes its angle from the t, h or w position of
   the token, chosen by the section split ("Ideogram 4 deep dive",
   section 6 part 3 "3D MRoPE", which names ``mrope_section=(24,20,20)``).
3. Bidirectional softmax attention over the joint sequence, with padded
   text slots (the per-prompt true text length; SimpleTuner quickstart,
   "Text Embed Cache": caches hold each prompt at its real length and batch
   padding happens in memory) excluded as keys and zeroed as queries.

The flash/online form on the GPU is only a reordering of this definition,
so the oracle is the definition itself: no tiling, no online softmax, the
full score matrix per (batch, head). Everything runs in float64; inputs are
taken exactly as stored (bf16 and fp32 widen to fp64 exactly).

Readings of points the pages leave open (each is a descriptor field or an
input, so both sides use the same value): epsilon inside the root, weight
applied as x_hat * gamma (gamma shared by the heads by default, or one per
head), norm before rotation, half-split rotary pairs (j, j + D/2) by default
(interleaved pairs (2j, 2j + 1) on request), one global frequency ladder
theta^(-2j/D) across the three axes, contiguous sections in t, h, w order, softmax scale D^-1/2, no causal
mask, equal head counts for Q, K and V.
"""

from __future__ import annotations

import numpy as np


def axis_of_pair(section, half: int) -> np.ndarray:
    """Axis (0 = t, 1 = h, 2 = w) that drives rotary pair j, for j < half.

    Contiguous blocks in pair order: the first section[0] pairs follow t,
    the next section[1] follow h, the last section[2] follow w ("Ideogram 4
    deep dive", section 6 part 3, the three-axis RoPE split).
    """
    st, sh, sw = (int(s) for s in section)
    if st + sh + sw != half or min(st, sh, sw) < 0:
        raise ValueError(f"section {section} does not split {half} rotary pairs")
    axis = np.empty(half, dtype=np.int64)
    axis[:st] = 0
    axis[st:st + sh] = 1
    axis[st + sh:] = 2
    return axis


def inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Rotary frequency of pair j: theta ** (-2 j / head_dim), in float64.

    One ladder for all three axes (the reading under which a text token, whose
    t, h and w positions are equal, gets ordinary 1D RoPE -- the "one positional
    frame" of the Ideogram 4.0 announcement thread). The unsloth commit log
    states the model builds ``inv_freq`` in explicit fp32; the GPU rounds it to
    fp32, the oracle keeps it exact.
    """
    half = head_dim // 2
    j = np.arange(half, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / head_dim)


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Per-row RMSNorm over the last axis: x * (mean(x^2) + eps)^-1/2 * gamma.

    The QK-RMSNorm of the Ideogram 4.0 announcement thread, applied per head
    (the last axis is head_dim). gamma is [D] (one weight shared by every
    head) or, for x [..., H, D], [H, D] (a weight per head); either
    broadcasts against x.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + np.float64(eps)) * np.asarray(gamma, dtype=np.float64)


def pair_slots(head_dim: int, pairs: str = "half"):
    """Element indices (first, second) of every rotary pair j < D/2.

    "half": pair j is (j, j + D/2), the rotate-half layout; "interleaved":
    pair j is (2j, 2j + 1). The pages name neither; both are conventions in
    use for rotary encodings, and a descriptor field picks one.
    """
    half = head_dim // 2
    j = np.arange(half)
    if pairs == "half":
        return j, j + half
    if pairs == "interleaved":
        return 2 * j, 2 * j + 1
    raise ValueError(f"unknown rotary pair layout {pairs!r}")


def mrope(x: np.ndarray, pos: np.ndarray, section, theta: float, pairs: str = "half") -> np.ndarray:
    """3D multimodal RoPE on x [B, S, H, D] with positions pos [B, S, 3].

    Pair j = (x_a, x_b) (slots from :func:`pair_slots`) is turned by the
    angle pos[axis(j)] * inv_freq(j):
    x'_a = x_a cos - x_b sin,  x'_b = x_b cos + x_a sin.
    (Ideogram 4.0 announcement thread: 3D multimodal RoPE; "Ideogram 4 deep
    dive", section 6 part 3: rotary encoding extended to three axes.)
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    axis = axis_of_pair(section, half)
    p = np.asarray(pos, dtype=np.float64)              # [B, S, 3]
    ang = p[:, :, axis] * inv_freq(d, theta)           # [B, S, half]
    c = np.cos(ang)[:, :, None, :]                     # broadcast over heads
    s = np.sin(ang)[:, :, None, :]
    ia, ib = pair_slots(d, pairs)
    x1 = x[..., ia]
    x2 = x[..., ib]
    out = np.empty_like(x)
    out[..., ia] = x1 * c - x2 * s
    out[..., ib] = x2 * c + x1 * s
    return out


def valid_tokens(batch: int, seq: int, text_pad: int, seq_lens=None) -> np.ndarray:
    """valid[b, s]: token s of item b is real (not a padded text slot).

    The first text_pad slots hold text, of which only the first L_b are real
    (SimpleTuner quickstart, "Text Embed Cache": per-prompt true length,
    padding in memory); image tokens after the text slots are always real.
    """
    s = np.arange(seq)[None, :]
    if seq_lens is None:
        return np.ones((batch, seq), dtype=bool)
    lens = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, text_pad)[:, None]
    return (s >= text_pad) | (s < lens)


def attention(qr: np.ndarray, kr: np.ndarray, v: np.ndarray, valid: np.ndarray,
              scale: float, rows=None, heads=None):
    """Softmax self-attention per (batch, head), no causal mask.

    z_ij = scale * q_i . k_j over valid keys j; p_ij = exp(z_ij - m_i) / sum;
    o_i = sum_j p_ij v_j for valid queries, 0 for padded ones;
    lse_i = m_i + log(sum_j exp(z_ij - m_i)), -inf for padded queries.
    (Ideogram 4 deep dive, section 4 part 2: one joint sequence through the
    same self-attention.)

    rows: optional query indices to evaluate (all keys are always used).
    heads: optional head indices to evaluate.
    Returns out [B, R, Hs, D] and lse [B, Hs, R].
    """
    b_, s_, h_, d_ = qr.shape
    rows = np.arange(s_) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(h_) if heads is None else np.asarray(heads, dtype=np.int64)
    out = np.zeros((b_, len(rows), len(heads), d_), dtype=np.float64)
    lse = np.full((b_, len(heads), len(rows)), -np.inf, dtype=np.float64)
    for b in range(b_):
        kv = valid[b]
        qv = valid[b, rows]
        if not kv.any():
            continue
        for hi, h in enumerate(heads):
            z = np.float64(scale) * (qr[b, rows, h, :] @ kr[b, :, h, :].T)
            z = z[:, kv]
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            l = e.sum(axis=1, keepdims=True)
            o = (e @ np.asarray(v[b, kv, h, :], dtype=np.float64)) / l
            out[b, qv, hi, :] = o[qv]
            lse[b, hi, qv] = (m[:, 0] + np.log(l[:, 0]))[qv]
    return out, lse


def oracle_fwd(q, k, v, pos, gamma_q, gamma_k, seq_lens=None, *, text_pad: int,
               section=(16, 24, 24), theta: float = 10000.0, eps: float = 1e-6,
               scale=None, rows=None, heads=None, rope_pairs: str = "half"):
    """The whole hot path: RMSNorm -> M-RoPE on Q and K, then attention.

    q, k, v: [B, S, H, D] (any real dtype; widened to float64).
    pos: [B, S, 3] integer (t, h, w) positions.  gamma_q, gamma_k: [D] or
    [H, D].  rope_pairs: "half" or "interleaved" (:func:`pair_slots`).
    seq_lens: [B] true text lengths (<= text_pad) or None for no padding.
    scale: softmax scale; None or <= 0 means head_dim ** -0.5.
    Returns (out [B, R, Hs, D], lse [B, Hs, R]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    b_, s_, h_, d_ = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(np.float64(d_))
    qr = mrope(rms_norm(q, gamma_q, eps), pos, section, theta, rope_pairs)
    kr = mrope(rms_norm(k, gamma_k, eps), pos, section, theta, rope_pairs)
    valid = valid_tokens(b_, s_, text_pad, seq_lens)
    return attention(qr, kr, v, valid, scale, rows=rows, heads=heads)


def oracle_fwd_varlen(q, k, v, pos, gamma_q, gamma_k, cu_seqlens, *, section=(16, 24, 24),
                      theta: float = 10000.0, eps: float = 1e-6, scale=None,
                      rope_pairs: str = "half"):
    """Packed variable-length form of the same path: sequence b is tokens
    [cu_seqlens[b], cu_seqlens[b+1]) of q, k, v [T, H, D] and pos [T, 3] (its
    true-length text tokens, then its image tokens), and attends to its own
    tokens only (the per-prompt true text length of the SimpleTuner
    quickstart's "Text Embed Cache", carried by packing instead of padding).
    Each sequence is the padding-free case of :func:`oracle_fwd`.

    Returns (out [T, H, D], lse [H, T]) in float64; tokens outside every
    sequence are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    t_, h_, d_ = q.shape
    out = np.full((t_, h_, d_), np.nan)
    lse = np.full((h_, t_), np.nan)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(len(cu) - 1):
        a0, a1 = int(cu[b]), int(cu[b + 1])
        if a1 <= a0:
            continue
        o, l = oracle_fwd(q[None, a0:a1], np.asarray(k)[None, a0:a1], np.asarray(v)[None, a0:a1],
                          np.asarray(pos)[None, a0:a1], gamma_q, gamma_k, None, text_pad=0,
                          section=section, theta=theta, eps=eps, scale=scale,
                          rope_pairs=rope_pairs)
        out[a0:a1] = o[0]
        lse[:, a0:a1] = l[0]
    return out, lse
