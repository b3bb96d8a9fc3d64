// bf16 path: fused QK-RMSNorm + 3D M-RoPE + flash-style softmax attention on
// gfx950 matrix cores.
//
// Operation: Ideogram 4.0 announcement thread (QK-RMSNorm and 3D multimodal
// RoPE inside the single-stream DiT's self-attention, text and image tokens in
// one positional frame); "Ideogram 4 deep dive", section 4 part 2 (one joint
// sequence through the same self-attention) and section 6 part 3 (three-axis
// rotary split); SimpleTuner quickstart, "Text Embed Cache" (per-prompt true
// text length, padding in memory -> padded text slots are masked keys and
// zero output rows).
//
// Work decomposition: one workgroup per (batch, head, BM-row query tile),
// WAVES waves of 32 query rows each. Per wave, everything is held "transposed"
// so a query row lives in one lane pair (lanes m and m + 32):
//   S^T (keys x queries) = K' Q'^T   v_mfma_f32_32x32x16_bf16, A = K' from LDS,
//                                    B = Q' from registers;
//   O^T (dims x queries) += V^T P^T  same MFMA, A = V^T from LDS, B = P from
//                                    the S^T accumulators (no LDS round trip).
// Row max / row sum are lane-local plus one permlane32 swap. K' rows are
// stored in LDS in the order that makes each lane's 16 S^T values 16
// consecutive keys, so the P fragment feeds P.V directly. V is transposed
// into LDS ([dim][key]) by an in-register transpose during staging.
//
// K/V tiles are double-buffered in LDS: tile t+1 is fetched with buffer loads
// (out-of-range rows read as zero) while tile t is computed, then stored to
// the other buffer, so each tile costs one workgroup barrier.
//
// Softmax runs in the log2 domain with a lazily updated running max: the
// output accumulators are rescaled only when some row's tile max exceeds its
// running max by more than kRescaleLog2 (so probabilities stay <= 2^8 before
// normalisation). The result is the same softmax; only the moment of
// rescaling changes.
#pragma once

#include "mra_common.hpp"

namespace mra {

constexpr float kRescaleLog2 = 8.0f;
constexpr int kBufFlags = 0x00020000;  // raw buffer resource, 32-bit data format

// LDS row of key n (within a 32-key block) so that MFMA output element i of
// lane half h corresponds to key h * 16 + i.
__device__ __forceinline__ int key_lds_row(int n) {
  const int blk = n & ~31, w = n & 31;
  return blk | (((w >> 2) & 3) << 3) | ((w >> 4) << 2) | (w & 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufFlags);
}

template <int D, int WAVES, int BN, bool KFUSED>
__global__ __launch_bounds__(WAVES * 64, 2) void attn_bf16_kernel(Args a) {
  constexpr int BM = WAVES * 32;
  constexpr int NT = WAVES * 64;
  constexpr int KC = D / 16;          // 16-wide head_dim chunks (QK^T k-steps)
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int NB = BN / 32;         // 32-key blocks per tile
  constexpr int KP = D + 8;           // LDS pitch of K' rows (elements)
  constexpr int VP = BN + 8;          // LDS pitch of V^T rows (elements)
  constexpr int DCH = D / 8;          // 8-element chunks per row
  constexpr int KCH = BN * DCH / NT;  // K chunks staged per thread
  constexpr int VKR = BN * DCH / NT;  // V keys per thread's transposed block
  constexpr int VKG = BN / VKR;       // key groups across the workgroup
  constexpr int KBUF = BN * KP, VBUF = D * VP;
  static_assert(KCH >= 1 && VKR >= 2 && (VKR & 1) == 0, "tile too small for the workgroup");
  static_assert(VKG * DCH == NT, "V staging must cover the tile exactly");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2 * VBUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, hf = lane >> 5;
  const int bid = xcd_remap(blockIdx.x, a.grid);
  const int qt = bid % a.n_qt, bh = bid / a.n_qt;
  const int head = bh % a.H, b = bh / a.H;
  const int S = a.S, T = a.T;
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), T) : T;
  const int q0 = qt * BM;
  const int row = q0 + wave * 32 + m;
  const bool in_seq = row < S;
  const bool valid_row = in_seq && !(row >= L && row < T);

  uint16_t* outp = (uint16_t*)a.out + b * a.os0 + (int64_t)row * a.os1 + head * a.os2;
  float* lsep = a.lse ? a.lse + ((int64_t)b * a.H + head) * S + row : nullptr;

  // Query tile made only of padded text slots: zeros, no attention.
  const int q_end = min(q0 + BM, S);
  if (q0 >= L && q_end <= T) {
    if (in_seq) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2*)(outp + db * 32 + g * 8 + hf * 4) = u32x2{0u, 0u};
      if (lsep && hf == 0) *lsep = -INFINITY;
    }
    return;
  }

  // ---- Q prologue: RMSNorm + M-RoPE in fp32, one bf16 rounding, kept as the
  // B operand of S^T: lane (m, hf) holds Q'[row][c*16 + hf*8 + e].
  bf16x8 qf[KC];
  {
    float x[KC][8];
    if (in_seq) {
      const uint16_t* src = (const uint16_t*)a.q + b * a.qs0 + (int64_t)row * a.qs1 + head * a.qs2;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 w = *(const u32x4*)(src + c * 16 + hf * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[c][2 * e] = bf16_lo(w[e]);
          x[c][2 * e + 1] = bf16_hi(w[e]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[c][e] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[c][e] * x[c][e];
    ss = half_swap_sum(ss);
    const float r = rsqrtf(ss * (1.0f / D) + a.eps);
    // (cos, sin) of this token's pairs from the table the prologue pass wrote
    const float2* csrow = a.cs + ((int64_t)b * S + min(row, S - 1)) * (D / 2);
#pragma unroll
    for (int c = 0; c < KC / 2; ++c) {
      const f32x4 g1a = *(const f32x4*)(a.gq + c * 16 + hf * 8);
      const f32x4 g1b = *(const f32x4*)(a.gq + c * 16 + hf * 8 + 4);
      const f32x4 g2a = *(const f32x4*)(a.gq + D / 2 + c * 16 + hf * 8);
      const f32x4 g2b = *(const f32x4*)(a.gq + D / 2 + c * 16 + hf * 8 + 4);
      f32x4 t4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) t4[e] = *(const f32x4*)(csrow + c * 16 + hf * 8 + 2 * e);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g1 = e < 4 ? g1a[e & 3] : g1b[e & 3];
        const float g2 = e < 4 ? g2a[e & 3] : g2b[e & 3];
        const float cs = t4[e >> 1][(e & 1) * 2], sn = t4[e >> 1][(e & 1) * 2 + 1];
        const float u = x[c][e] * r * g1;
        const float w = x[c + KC / 2][e] * r * g2;
        qf[c][e] = (__bf16)(u * cs - w * sn);
        qf[c + KC / 2][e] = (__bf16)(w * cs + u * sn);
      }
    }
  }

  // ---- K/V tile staging: buffer loads -> registers -> LDS (double buffered)
  const int ntiles = (S + BN - 1) / BN;
  // a tile with no valid key (all of its in-sequence keys are padded text) is skipped
  auto skipped = [&](int t) { const int n0 = t * BN; return n0 >= L && min(n0 + BN, S) <= T; };
  auto next_tile = [&](int t) {
    ++t;
    while (t < ntiles && skipped(t)) ++t;
    return t;
  };

  // K rows: K' (dense [S, D] per (b, head)) or raw K (token stride ks1).
  const int64_t krow = KFUSED ? a.ks1 : D;
  const uint16_t* kbase = KFUSED ? (const uint16_t*)a.k + b * a.ks0 + head * a.ks2
                                 : a.kp + ((int64_t)b * a.H + head) * S * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (uint32_t)(((int64_t)(S - 1) * krow + D) * 2));
  const uint16_t* vbase = (const uint16_t*)a.v + b * a.vs0 + head * a.vs2;
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (uint32_t)(((int64_t)(S - 1) * a.vs1 + D) * 2));

  // per-thread staging coordinates (fixed for the whole loop)
  int k_key[KCH], k_dch[KCH], k_off[KCH], k_lds[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int ci = tid + i * NT;
    k_key[i] = ci / DCH;
    int dch = ci % DCH;
    if constexpr (KFUSED) dch = (dch >> 1) + (dch & 1) * (DCH / 2);  // pair partner = lane ^ 1
    k_dch[i] = dch;
    k_off[i] = (int)((k_key[i] * krow + dch * 8) * 2);
    k_lds[i] = key_lds_row(k_key[i]) * KP + dch * 8;
  }
  const int vkg = tid % VKG, vdc = tid / VKG;
  const int v_off = (int)(((int64_t)vkg * VKR * a.vs1 + vdc * 8) * 2);
  const int v_rowb = (int)(a.vs1 * 2);
  const int v_lds = (vdc * 8) * VP + vkg * VKR;

  u32x4 kr[KCH], vr[VKR];
  float2 csr[KFUSED ? KCH : 1][4];

  auto load_tile = [&](int t) {
    const int n0 = t * BN;
    const int ks = (int)(n0 * krow * 2);
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, k_off[i], ks, 0);
      if constexpr (KFUSED) {
        const int n = min(n0 + k_key[i], S - 1);
        const int j0 = (k_dch[i] % (DCH / 2)) * 8 + (k_dch[i] >= DCH / 2 ? 4 : 0);
        const float2* cp = a.cs + ((int64_t)b * S + n) * (D / 2) + j0;
        // lanes dch and dch^1 share one group of 8 pair angles: each fetches
        // 4 and the halves are swapped at store time
#pragma unroll
        for (int e = 0; e < 4; ++e) csr[i][e] = cp[e];
      }
    }
    const int vs = n0 * v_rowb;
#pragma unroll
    for (int i = 0; i < VKR; ++i)
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vrs, v_off + i * v_rowb, vs, 0);
  };

  auto store_tile = [&](int t, int buf) {
    const int n0 = t * BN;
    uint16_t* kd = Ks + buf * KBUF;
    uint16_t* vd = Vt + buf * VBUF;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      u32x4 w = kr[i];
      if constexpr (KFUSED) {
        // RMSNorm over the lanes holding this key row, then rotate pairs
        // (the lane holding chunk c < DCH/2 has x1, its neighbour lane^1 x2).
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[2 * e] = bf16_lo(w[e]); x[2 * e + 1] = bf16_hi(w[e]); }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
        for (int s = 1; s < DCH; s <<= 1) ss += __shfl_xor(ss, s, DCH);
        const float r = rsqrtf(ss * (1.0f / D) + a.eps);
        const int dch = k_dch[i];
        const bool first = dch < DCH / 2;
        float y[8], px[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[e] * r * a.gk[dch * 8 + e];
#pragma unroll
        for (int e = 0; e < 8; ++e) px[e] = __shfl_xor(y[e], 1, 64);
        float2 cs8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 mine = csr[i][e];
          const float2 other = make_float2(__shfl_xor(mine.x, 1, 64), __shfl_xor(mine.y, 1, 64));
          cs8[e] = first ? mine : other;
          cs8[4 + e] = first ? other : mine;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = cs8[e].x, s = cs8[e].y;
          y[e] = first ? (y[e] * c - px[e] * s) : (y[e] * c + px[e] * s);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16(y[2 * e], y[2 * e + 1]);
      }
      *(u32x4*)&kd[k_lds[i]] = w;
    }
    // V rows of padded text keys (and rows past the end) become zeros so a
    // non-finite value there cannot reach P.V (their P is exactly 0).
    if (n0 + BN > S || (n0 + BN > L && n0 < T)) {
#pragma unroll
      for (int i = 0; i < VKR; ++i) {
        const int n = n0 + vkg * VKR + i;
        if (n >= S || (n >= L && n < T)) vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    // VKR keys x 8 dims -> 8 rows of V^T, VKR keys each
#pragma unroll
    for (int d2 = 0; d2 < 4; ++d2) {
      uint32_t lo[VKR / 2], hi[VKR / 2];
#pragma unroll
      for (int i = 0; i < VKR; i += 2) {
        lo[i / 2] = __builtin_amdgcn_perm(vr[i + 1][d2], vr[i][d2], 0x05040100u);
        hi[i / 2] = __builtin_amdgcn_perm(vr[i + 1][d2], vr[i][d2], 0x07060302u);
      }
      uint16_t* r0 = vd + v_lds + 2 * d2 * VP;
      uint16_t* r1 = r0 + VP;
      if constexpr (VKR == 4) {
        *(u32x2*)r0 = u32x2{lo[0], lo[1]};
        *(u32x2*)r1 = u32x2{hi[0], hi[1]};
      } else {
        *(uint32_t*)r0 = lo[0];
        *(uint32_t*)r1 = hi[0];
      }
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const float c2 = a.c2;

  int t = 0;
  while (t < ntiles && skipped(t)) ++t;
  int buf = 0;
  if (t < ntiles) {
    load_tile(t);
    store_tile(t, 0);
  }
  __syncthreads();

  while (t < ntiles) {
    const int tn = next_tile(t);
    if (tn < ntiles) load_tile(tn);

    const int n0 = t * BN;
    const uint16_t* kc = Ks + buf * KBUF;
    const uint16_t* vc = Vt + buf * VBUF;
    // S^T = K' Q'^T for each 32-key block
    f32x16 st[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kb][i] = 0.f;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const bf16x8 av = *(const bf16x8*)&kc[(kb * 32 + m) * KP + c * 16 + hf * 8];
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[c], st[kb], 0, 0, 0);
      }
    }
    // key-padding / sequence-end mask (select, so NaN in masked keys cannot leak)
    if (n0 + BN > S || (n0 + BN > L && n0 < T)) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int n = n0 + kb * 32 + hf * 16 + i;
          const bool ok = n < S && !(n >= L && n < T);
          st[kb][i] = ok ? st[kb][i] : -INFINITY;
        }
    }
    // online softmax in the log2 domain, lazily rescaled
    float mx = st[0][0];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kb][i]);
    mx = half_swap_max(mx) * c2;
    if (__builtin_amdgcn_ballot_w64(mx > mrun + kRescaleLog2) != 0) {
      const float mnew = fmaxf(mrun, mx);
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      lrun *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    bf16x8 pf[NB][2];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[kb][u][e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][u * 8 + e], c2, -mrun));
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pp = {pf[kb][u][e], pf[kb][u][e + 1]};
          lrun = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, lrun, false);
        }
      }
    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 av = *(const bf16x8*)&vc[(db * 32 + m) * VP + kb * 32 + hf * 16 + u * 8];
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[kb][u], oacc[db], 0, 0, 0);
        }
    if (tn < ntiles) store_tile(tn, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    t = tn;
  }

  // ---- epilogue: O / l, padded rows are exact zeros (selected, not scaled,
  // so whatever a padded query row computed cannot leak)
  const float ltot = half_swap_sum(lrun);
  if (!in_seq) return;
  const float inv = 1.0f / ltot;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w0 = pack_bf16(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      uint32_t w1 = pack_bf16(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
      w0 = valid_row ? w0 : 0u;
      w1 = valid_row ? w1 : 0u;
      *(u32x2*)(outp + db * 32 + g * 8 + hf * 4) = u32x2{w0, w1};
    }
  if (lsep && hf == 0) *lsep = valid_row ? mrun * kLn2 + logf(ltot) : -INFINITY;
}

}  // namespace mra
