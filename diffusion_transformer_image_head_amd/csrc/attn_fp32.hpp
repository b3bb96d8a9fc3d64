// fp32 path: fused QK-RMSNorm + 3D M-RoPE + softmax attention with no
// rounding below fp32. It serves the small fp32 workloads (correctness
// shapes), so it is written for clarity: one thread per query row, keys
// streamed through LDS 16 at a time, online softmax in natural-exp form.
//
// Operation: Ideogram 4.0 announcement thread (QK-RMSNorm, 3D multimodal
// RoPE, self-attention over text and image tokens in one frame); "Ideogram 4
// deep dive", section 4 part 2 (joint sequence) and section 6 part 3 (the
// three-axis rotary split); SimpleTuner quickstart, "Text Embed Cache"
// (padded text slots are not real tokens).
#pragma once

#include "mra_common.hpp"

namespace mra {

// RMSNorm then M-RoPE of one fp32 row x[D] in place, for a token at (pt, ph, pw).
// Rotary pair j is elements (j, j + D/2), or (2j, 2j + 1) when inter is set.
template <int D>
__device__ __forceinline__ void prologue_row_f32(float* x, const float* g, const Rope& rope,
                                                 int pt, int ph, int pw, float eps, bool inter) {
  constexpr int HALF = D / 2;
  float ss = 0.f;
  for (int d = 0; d < D; ++d) ss += x[d] * x[d];
  const float r = 1.0f / sqrtf(ss / D + eps);
  for (int j = 0; j < HALF; ++j) {
    const int i1 = inter ? 2 * j : j, i2 = inter ? 2 * j + 1 : j + HALF;
    const float u = x[i1] * r * g[i1];
    const float w = x[i2] * r * g[i2];
    float sn, cs;
    sincosf((float)axis_pos(rope, j, pt, ph, pw) * rope.inv_freq[j], &sn, &cs);
    x[i1] = u * cs - w * sn;
    x[i2] = w * cs + u * sn;
  }
}

template <int D>
__global__ __launch_bounds__(64) void attn_fp32_kernel(Args a) {
  constexpr int BM = 64, BN = 16;
  __shared__ float Qs[BM][D + 1];
  __shared__ float Ks[BN][D + 1];
  __shared__ float Vs[BN][D];

  const int t = threadIdx.x;
  const int bid = blockIdx.x;
  const int qt = bid % a.n_qt, bh = bid / a.n_qt;
  const int head = bh % a.H, b = bh / a.H;
  const SeqView sv = seq_view(a, b);
  const int S = sv.S, T = a.T, Sx = a.S, bl = sv.bl;
  const int64_t tok0 = sv.tok0;
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), T) : T;
  if (qt * BM >= S) return;  // packed layout: tile past this item's end
  const int row = qt * BM + t;
  const bool in_seq = row < S;
  const bool valid_row = in_seq && !(row >= L && row < T);
  const float* q = (const float*)a.q;
  const float* k = (const float*)a.k;
  const float* v = (const float*)a.v;

  if (in_seq) {
    const float* src = q + bl * a.qs0 + (tok0 + row) * a.qs1 + head * a.qs2;
    for (int d = 0; d < D; ++d) Qs[t][d] = src[d];
    const int32_t* p3 = a.pos + ((int64_t)bl * Sx + tok0 + row) * 3;
    prologue_row_f32<D>(Qs[t], a.gq + head * a.gqs, a.rope, p3[0], p3[1], p3[2], a.eps, a.inter);
  }

  float o[D];
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  for (int n0 = 0; n0 < S; n0 += BN) {
    __syncthreads();
    if (t < BN) {
      const int n = n0 + t;
      if (n < S) {
        const float* src = k + bl * a.ks0 + (tok0 + n) * a.ks1 + head * a.ks2;
        for (int d = 0; d < D; ++d) Ks[t][d] = src[d];
        const int32_t* p3 = a.pos + ((int64_t)bl * Sx + tok0 + n) * 3;
        prologue_row_f32<D>(Ks[t], a.gk + head * a.gqs, a.rope, p3[0], p3[1], p3[2], a.eps, a.inter);
      }
    }
    for (int i = t; i < BN * D; i += 64) {
      const int kk = i / D, d = i - kk * D;
      const int n = n0 + kk;
      Vs[kk][d] = n < S ? v[bl * a.vs0 + (tok0 + n) * a.vs1 + head * a.vs2 + d] : 0.f;
    }
    __syncthreads();
    if (!valid_row) continue;
    for (int kk = 0; kk < BN; ++kk) {
      const int n = n0 + kk;
      if (n >= S || (n >= L && n < T)) continue;
      float z = 0.f;
      for (int d = 0; d < D; ++d) z += Qs[t][d] * Ks[kk][d];
      z *= a.scale;
      if (z > mrun) {
        const float f = expf(mrun - z);
        lrun *= f;
        for (int d = 0; d < D; ++d) o[d] *= f;
        mrun = z;
      }
      const float p = expf(z - mrun);
      lrun += p;
      for (int d = 0; d < D; ++d) o[d] += p * Vs[kk][d];
    }
  }
  if (!in_seq) return;
  float* dst = (float*)a.out + bl * a.os0 + (tok0 + row) * a.os1 + head * a.os2;
  const float inv = valid_row ? 1.0f / lrun : 0.f;
  for (int d = 0; d < D; ++d) dst[d] = valid_row ? o[d] * inv : 0.f;
  if (a.lse) a.lse[((int64_t)bl * a.H + head) * Sx + tok0 + row] = valid_row ? mrun + logf(lrun) : -INFINITY;
}

}  // namespace mra
