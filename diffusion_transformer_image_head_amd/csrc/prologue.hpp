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
// are shared by all heads: each is computed once, by one lane, with the
// accurate sincosf.
// Lane `sub` owns rotary pairs sub*PPL .. +PPL-1: with half-split pairs their
// elements are the runs [sub*PPL, +PPL) and [D/2 + sub*PPL, +PPL); with
// interleaved pairs, the one run [2*sub*PPL, +2*PPL). K' keeps the element
// order of K.
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
  const bool inter = a.inter;
  // element offsets of this lane's first and second pair members
  const int o1 = inter ? 2 * sub * PPL : sub * PPL;
  const int o2 = inter ? o1 + 1 : o1 + HALF;

  const uint16_t* kb = (const uint16_t*)a.k + b * a.ks0 + s * a.ks1;
  // Raw K words of head h for this lane's pairs (first members then second
  // members for half-split pairs; the pairs in order for interleaved ones),
  // and the gammas of those elements. Head group h + 4's loads are issued
  // before head group h is computed, the first before the angles, so two
  // groups' loads are in flight per wave.
  auto load_k = [&](int h) {
    const uint16_t* src = kb + h * a.ks2;
    u32x4 w = {0u, 0u, 0u, 0u};
    if constexpr (PPL == 4) {
      if (inter) {
        w = *(const u32x4*)(src + o1);
      } else {
        const u32x2 w1 = *(const u32x2*)(src + o1), w2 = *(const u32x2*)(src + o2);
        w = u32x4{w1[0], w1[1], w2[0], w2[1]};
      }
    } else {
      if (inter) {
        const u32x2 v = *(const u32x2*)(src + o1);
        w = u32x4{v[0], v[1], 0u, 0u};
      } else {
        w = u32x4{*(const uint32_t*)(src + o1), *(const uint32_t*)(src + o2), 0u, 0u};
      }
    }
    return w;
  };
  auto load_g = [&](int h, float (&g1)[PPL], float (&g2)[PPL]) {
    const float* gk = a.gk + h * a.gqs;
    if (inter) {
      float gv[2 * PPL];
#pragma unroll
      for (int i = 0; i < 2 * PPL; i += 4) *(f32x4*)(gv + i) = *(const f32x4*)(gk + o1 + i);
#pragma unroll
      for (int p = 0; p < PPL; ++p) { g1[p] = gv[2 * p]; g2[p] = gv[2 * p + 1]; }
    } else {
#pragma unroll
      for (int p = 0; p < PPL; ++p) { g1[p] = gk[o1 + p]; g2[p] = gk[o2 + p]; }
    }
  };
  u32x4 wc = {0u, 0u, 0u, 0u};
  float g1[PPL], g2[PPL];
  if (hq < a.H) {
    wc = load_k(hq);
    load_g(hq, g1, g2);
  }

  // One rotary pair per lane (lane mod HALF), then each lane gathers the
  // (cos, sin) of its own pairs from the lanes that computed them.
  float cs[PPL], sn[PPL];
  {
    const int j = lane % HALF;
    const float ang = (float)axis_pos(a.rope, j, pt, ph, pw) * a.rope.inv_freq[j];
    float s1, c1;
    sincosf(ang, &s1, &c1);
    // the same rotation feeds the Q side inside the attention kernel
    if (lane < HALF && a.cs) a.cs[(int64_t)tok * HALF + j] = make_float2(c1, s1);
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      cs[p] = __shfl(c1, sub * PPL + p, 64);
      sn[p] = __shfl(s1, sub * PPL + p, 64);
    }
  }
  for (int h = hq; h < a.H; h += 4) {
    u32x4 wn = {0u, 0u, 0u, 0u};
    float n1[PPL] = {}, n2[PPL] = {};
    if (h + 4 < a.H) {
      wn = load_k(h + 4);
      load_g(h + 4, n1, n2);
    }
    float x1[PPL], x2[PPL];
    if (inter) {
#pragma unroll
      for (int p = 0; p < PPL; ++p) { x1[p] = bf16_lo(wc[p]); x2[p] = bf16_hi(wc[p]); }
    } else {
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        const uint32_t u1 = wc[p / 2], u2 = wc[PPL / 2 + p / 2];
        x1[p] = (p & 1) ? bf16_hi(u1) : bf16_lo(u1);
        x2[p] = (p & 1) ? bf16_hi(u2) : bf16_lo(u2);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < PPL; ++p) ss += x1[p] * x1[p] + x2[p] * x2[p];
    ss += __shfl_xor(ss, 1, 16);
    ss += __shfl_xor(ss, 2, 16);
    ss += __shfl_xor(ss, 4, 16);
    ss += __shfl_xor(ss, 8, 16);
    const float r = rsqrtf(ss * (1.0f / D) + a.eps) * a.pscale;
    float y1[PPL], y2[PPL];
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      const float u = x1[p] * r * g1[p];
      const float w = x2[p] * r * g2[p];
      y1[p] = u * cs[p] - w * sn[p];
      y2[p] = w * cs[p] + u * sn[p];
    }
    uint16_t* dst = a.kp + (((int64_t)b * a.H + h) * a.S + s) * D;
    if (inter) {
      if constexpr (PPL == 4)
        *(u32x4*)(dst + o1) = u32x4{pack_bf16(y1[0], y2[0]), pack_bf16(y1[1], y2[1]),
                                    pack_bf16(y1[2], y2[2]), pack_bf16(y1[3], y2[3])};
      else
        *(u32x2*)(dst + o1) = u32x2{pack_bf16(y1[0], y2[0]), pack_bf16(y1[1], y2[1])};
    } else if constexpr (PPL == 4) {
      *(u32x2*)(dst + o1) = u32x2{pack_bf16(y1[0], y1[1]), pack_bf16(y1[2], y1[3])};
      *(u32x2*)(dst + o2) = u32x2{pack_bf16(y2[0], y2[1]), pack_bf16(y2[2], y2[3])};
    } else {
      *(uint32_t*)(dst + o1) = pack_bf16(y1[0], y1[1]);
      *(uint32_t*)(dst + o2) = pack_bf16(y2[0], y2[1]);
    }
    wc = wn;
#pragma unroll
    for (int p = 0; p < PPL; ++p) { g1[p] = n1[p]; g2[p] = n2[p]; }
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
