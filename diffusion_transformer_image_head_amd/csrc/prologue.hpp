// Prologue passes run before the attention kernel: the per-token rotary
// (cos, sin) table (shared by the Q and K sides, so both turn by bitwise the
// same values), and optionally K' = RMSNorm + 3D M-RoPE of K in bf16.
//
// Operation: Ideogram 4.0 announcement thread (QK-RMSNorm and 3D multimodal
// RoPE in the DiT's self-attention); "Ideogram 4 deep dive", section 6 part 3
// (three-axis rotary split). Rotary pairs are (j, j + D/2); pair j's angle is
// pos[axis(j)] * inv_freq[j] with inv_freq in fp32 (unsloth Ideogram 4
// backend commit log: inv_freq computed in explicit fp32).
#pragma once

#include "mra_common.hpp"

namespace mra {

// K' = bf16(pscale * rope(rmsnorm(K))) into [B, H, S, D], plus (when a.cs is
// set) the (cos, sin) table [B, S, D/2]. One wave per token; 16 lanes
// per head row, so a wave covers 4 heads per step. The token's rotary angles
// are shared by all heads and computed once per lane with the accurate sincosf.
template <int D>
__global__ __launch_bounds__(256) void k_prologue_kernel(Args a) {
  constexpr int HALF = D / 2;
  constexpr int PPL = HALF / 16;  // rotary pairs per lane
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= a.B * a.S) return;
  const int b = tok / a.S, s = tok - b * a.S;
  const int sub = lane & 15, hq = lane >> 4;
  const int32_t* p3 = a.pos + (int64_t)tok * 3;
  const int pt = p3[0], ph = p3[1], pw = p3[2];

  float cs[PPL], sn[PPL], g1[PPL], g2[PPL];
#pragma unroll
  for (int p = 0; p < PPL; ++p) {
    const int j = sub * PPL + p;
    const float ang = (float)axis_pos(a.rope, j, pt, ph, pw) * a.rope.inv_freq[j];
    sincosf(ang, &sn[p], &cs[p]);
    g1[p] = a.gk[j];
    g2[p] = a.gk[j + HALF];
    // the same rotation feeds the Q side inside the attention kernel
    if (hq == 0 && a.cs) a.cs[(int64_t)tok * HALF + j] = make_float2(cs[p], sn[p]);
  }
  const uint16_t* kb = (const uint16_t*)a.k + b * a.ks0 + s * a.ks1;
  for (int h = hq; h < a.H; h += 4) {
    const uint16_t* src = kb + h * a.ks2 + sub * PPL;
    float x1[PPL], x2[PPL];
    if constexpr (PPL == 4) {
      const u32x2 w1 = *(const u32x2*)src;
      const u32x2 w2 = *(const u32x2*)(src + HALF);
      x1[0] = bf16_lo(w1[0]); x1[1] = bf16_hi(w1[0]); x1[2] = bf16_lo(w1[1]); x1[3] = bf16_hi(w1[1]);
      x2[0] = bf16_lo(w2[0]); x2[1] = bf16_hi(w2[0]); x2[2] = bf16_lo(w2[1]); x2[3] = bf16_hi(w2[1]);
    } else {
      const uint32_t w1 = *(const uint32_t*)src;
      const uint32_t w2 = *(const uint32_t*)(src + HALF);
      x1[0] = bf16_lo(w1); x1[1] = bf16_hi(w1);
      x2[0] = bf16_lo(w2); x2[1] = bf16_hi(w2);
    }
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < PPL; ++p) ss += x1[p] * x1[p] + x2[p] * x2[p];
    ss += __shfl_xor(ss, 1, 16);
    ss += __shfl_xor(ss, 2, 16);
    ss += __shfl_xor(ss, 4, 16);
    ss += __shfl_xor(ss, 8, 16);
    const float r = rsqrtf(ss * (1.0f / D) + a.eps) * a.pscale;
    uint32_t o1[PPL / 2], o2[PPL / 2];
#pragma unroll
    for (int p = 0; p < PPL; p += 2) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float u = x1[p + e] * r * g1[p + e];
        const float w = x2[p + e] * r * g2[p + e];
        y[e] = u * cs[p + e] - w * sn[p + e];
        y[2 + e] = w * cs[p + e] + u * sn[p + e];
      }
      o1[p / 2] = pack_bf16(y[0], y[1]);
      o2[p / 2] = pack_bf16(y[2], y[3]);
    }
    uint16_t* dst = a.kp + (((int64_t)b * a.H + h) * a.S + s) * D + sub * PPL;
    if constexpr (PPL == 4) {
      *(u32x2*)dst = u32x2{o1[0], o1[1]};
      *(u32x2*)(dst + HALF) = u32x2{o2[0], o2[1]};
    } else {
      *(uint32_t*)dst = o1[0];
      *(uint32_t*)(dst + HALF) = o2[0];
    }
  }
}

// (cos, sin) of every token's rotary angles: [B, S, D/2] float2.
template <int D>
__global__ __launch_bounds__(256) void rope_table_kernel(Args a) {
  constexpr int HALF = D / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * a.S * HALF) return;
  const int64_t tok = i / HALF;
  const int j = (int)(i - tok * HALF);
  const int32_t* p3 = a.pos + tok * 3;
  const float ang = (float)axis_pos(a.rope, j, p3[0], p3[1], p3[2]) * a.rope.inv_freq[j];
  float sn, cs;
  sincosf(ang, &sn, &cs);
  a.cs[i] = make_float2(cs, sn);
}

}  // namespace mra
