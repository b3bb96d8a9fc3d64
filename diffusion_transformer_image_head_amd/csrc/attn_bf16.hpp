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
// WAVES waves of RB x 32 query rows each. Per wave, everything is held
// "transposed" so a query row lives in one lane pair (lanes m and m + 32):
//   S^T (keys x queries) = K' Q'^T   v_mfma_f32_32x32x16_bf16, A = K' from LDS,
//                                    B = Q' from registers;
//   O^T (dims x queries) += V^T P^T  same MFMA, A = V^T read from LDS with the
//                                    gfx950 transposing LDS read, B = P taken
//                                    straight from the S^T accumulators.
// Row max / row sum are lane-local plus one permlane32 swap. With RB = 2 a
// wave owns two 32-row blocks, so every K'/V fragment read from LDS feeds two
// MFMAs (half the LDS traffic per FLOP of RB = 1); it then needs ~380
// registers and runs one wave per SIMD.
//
// LDS: K' and V tiles arrive by buffer loads that write LDS directly (lane L of
// a load lands at 16*L of a 1 KiB run), with 16-byte chunks XOR-swizzled per
// row so the matrix-operand reads are free of bank conflicts. K' rows sit in
// the order that makes each lane's 16 S^T values 16 consecutive keys, so the P
// fragment feeds P.V directly. K' and V are double-buffered: after each
// tile's barrier the loads of tile t+1 are issued, then Q.K'(t), the softmax
// and P.V(t) run; the two waves sharing a SIMD (two 4-wave workgroups per
// CU, or one 8-wave workgroup) overlap one's matrix work with the other's
// exponentials, and a wave raises its issue priority for its P.V run.
//
// Numerics: Q' is rounded to bf16 already multiplied by softmax_scale*log2(e),
// so S^T is in log2 units; the S^T accumulators start at -m (the running row
// max), which makes P = exp2(S^T) with no further arithmetic. The running max
// is updated lazily: only when some row's tile max exceeds it by more than
// kRescaleLog2 are the output accumulators rescaled (probabilities stay below
// 2^8 before normalisation). The row sum adds the bf16-rounded P, the same
// values P.V uses.
#pragma once

#include "mra_common.hpp"

namespace mra {

constexpr float kRescaleLog2 = 8.0f;
// operand read pacing: K' fragment reads kept in flight ahead of the Q.K'
// MFMAs, and transposing V reads ahead of the P.V MFMAs
constexpr int kKAhead = 4, kPvPace = 8;

constexpr int kBufFlags = 0x00020000;  // raw buffer resource, 32-bit data format

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Key held by LDS row r of a 32-row block: rows are ordered so that MFMA
// output element i of lane half h is key h * 16 + i.
__device__ __forceinline__ int key_of_row(int r) {
  return (r & ~31) | (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
}

template <int N>
struct Parity {
  static constexpr int value = N;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufFlags);
}

// LDS swizzles. The gfx950 LDS has 64 four-byte banks (256 bytes per bank
// row) and serves a 128-bit read for 16 lanes, a 64-bit read for 32 lanes, per
// clock. Logical 16-byte chunk c of tile row r sits at physical chunk
// c ^ swz(r) (XOR: the map is its own inverse, so the direct loads use it to
// pick the source chunk of each LDS slot). With RPB tile rows per bank row:
// - K' (128-bit reads, 16 lanes = 16 consecutive rows, same chunk): the rows
//   that share banks get distinct chunks, swz = (r / RPB) mod chunks-per-row;
// - V (transposing 64-bit reads, 32 lanes = 4 consecutive keys x 4 chunks):
//   the 4 keys get disjoint 4-chunk groups, swz = 4 * ((r / RPB) mod (4 / RPB)).
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  constexpr int RPB = 256 / (D * 2), CPR = D / 8;
  return (r / RPB) & (CPR - 1);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  constexpr int RPB = 256 / (D * 2);
  return ((r / RPB) & (4 / RPB - 1)) << 2;
}
// Byte offset inside a swizzled LDS tile of logical 16-byte chunk c of row r.
template <int D>
__device__ __forceinline__ int k_lds_off(int r, int c) { return r * (D * 2) + ((c ^ k_swz<D>(r)) << 4); }
template <int D>
__device__ __forceinline__ int v_lds_off(int r, int c) { return r * (D * 2) + ((c ^ v_swz<D>(r)) << 4); }

// Split query tiles: part p of split tile st stores, for each 32-row block rr
// of the tile, one record of 64 * (D/2 + 2) floats: the unnormalised O^T
// accumulators as [D/8 chunks][64 lanes][4] (chunk db*4 + g of lane (m, hf)
// holds dims db*32 + g*8 + hf*4 .. +3 of query row rr*32 + m), then the running
// max (log2 units) and the row sum, [64 lanes] each.
template <int D, int WAVES, int RB>
__device__ __forceinline__ float* part_record(float* part, int nsplit, int st, int p, int rr) {
  constexpr int REC = 64 * (D / 2 + 2);
  return part + (((int64_t)st * nsplit + p) * (WAVES * RB) + rr) * REC;
}

// KPM: where Q' and K' come from. 0: K' from the prepass in the workspace,
// Q' made here from q; 1: both made here (K while its tile is staged);
// 2: q and k already hold the operands Q'' (scaled by c2) and K'.
template <int D, int WAVES, int BN, int RB, int KPM, int G>
__global__ __launch_bounds__(WAVES * 64, WAVES * RB >= 8 ? 1 : 2) void attn_bf16_kernel(Group<G> gp) {
  constexpr bool KFUSED = KPM == 1, PRE = KPM == 2;
  constexpr int BM = WAVES * 32 * RB;
  constexpr int NT = WAVES * 64;
  constexpr int KC = D / 16;                 // 16-wide head_dim chunks (QK^T k-steps)
  constexpr int DB = D / 32;                 // 32-row blocks of O^T
  constexpr int NB = BN / 32;                // 32-key blocks per tile
  constexpr int ROWB = D * 2;                // bytes per LDS row
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILEB = BN * ROWB;           // bytes per K or V tile
  constexpr int RUNS = TILEB / 1024 / WAVES; // 1 KiB direct-load runs per wave per tile
  constexpr int RPR = 1024 / ROWB;           // rows per run
  constexpr int KCH = BN * CPR / NT;         // fused mode: K chunks per thread
  static_assert(RUNS >= 1 && RUNS * WAVES * 1024 == TILEB, "tile must split into whole runs");
  static_assert(KCH >= 1 && KCH * NT == BN * CPR, "fused staging must cover the tile");

  // Four separate LDS objects (not one indexed array): the buffer parity is a
  // compile-time constant in each unrolled step, so the compiler can see that
  // a step's direct loads and its LDS reads touch different objects and does
  // not make the reads wait for the loads just issued.
  __shared__ __attribute__((aligned(1024))) char K0[TILEB];
  __shared__ __attribute__((aligned(1024))) char K1[TILEB];
  __shared__ __attribute__((aligned(1024))) char V0[TILEB];
  __shared__ __attribute__((aligned(1024))) char V1[TILEB];
  auto kbuf = [&](int i) -> char* { return i ? K1 : K0; };
  auto vbuf = [&](int i) -> char* { return i ? V1 : V0; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, hf = lane >> 5;
  // workgroup -> (global tile, key-range part): whole tiles first (XCD-aware
  // order), then nsplit parts of each of the last n_split tiles
  int gt, part = 0, nparts = 1;
  if ((int)blockIdx.x < gp.n_whole) {
    gt = xcd_remap(blockIdx.x, gp.n_whole, gp.nxcd);
  } else {
    const int s_ = blockIdx.x - gp.n_whole;
    gt = gp.n_whole + s_ / gp.nsplit;
    part = s_ % gp.nsplit;
    nparts = gp.nsplit;
  }
  int tile;
  const Args& a = gp.p[group_problem(gp, gt, tile)];
  const int qt = tile % a.n_qt, bh = tile / a.n_qt;
  const int head = bh % a.H, b = bh / a.H;
  const SeqView sv = seq_view(a, b);
  const int S = sv.S, T = a.T, Sx = a.S, bl = sv.bl;
  const int64_t tok0 = sv.tok0;
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), T) : T;
  const int q0 = qt * BM;
  if (q0 >= S) return;  // packed layout: tile past this item's end
  int row[RB];
  bool in_seq[RB], valid_row[RB];
  uint16_t* outp[RB];
  float* lsep[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    row[rb] = q0 + (wave * RB + rb) * 32 + m;
    in_seq[rb] = row[rb] < S;
    valid_row[rb] = in_seq[rb] && !(row[rb] >= L && row[rb] < T);
    outp[rb] = (uint16_t*)a.out + bl * a.os0 + (tok0 + row[rb]) * a.os1 + head * a.os2;
    lsep[rb] = a.lse ? a.lse + ((int64_t)bl * a.H + head) * Sx + tok0 + row[rb] : nullptr;
  }

  // Query tile made only of padded text slots: zeros, no attention.
  const int q_end = min(q0 + BM, S);
  if (q0 >= L && q_end <= T) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (in_seq[rb]) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(u32x2*)(outp[rb] + db * 32 + g * 8 + hf * 4) = u32x2{0u, 0u};
        if (lsep[rb] && hf == 0) *lsep[rb] = -INFINITY;
      }
    }
    return;
  }

  // gamma_k for the logit bound, loaded with the Q prologue's loads
  float gk0 = 0.f, gk1 = 0.f;
  if constexpr (!PRE) {
    const float* gkp = a.gk + head * a.gqs;
    gk0 = gkp[lane];
    if constexpr (D > 64) gk1 = gkp[lane + 64];
  }
  // ---- Q prologue: RMSNorm + M-RoPE in fp32, scaled by softmax_scale*log2(e),
  // one bf16 rounding, kept as the B operand of S^T: lane (m, hf) holds
  // Q'[row][c*16 + hf*8 + e].
  bf16x8 qf[RB][KC];
  if constexpr (PRE) {
    // the operand as given (Q''), or a plain Q' times qmul =
    // softmax_scale*log2(e) rounded again to bf16; rows past the end read as
    // zeros
    const float qmul = a.qmul;
    const bool scale_q = qmul != 1.0f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint16_t* src = (const uint16_t*)a.q + bl * a.qs0 + (tok0 + min(row[rb], S - 1)) * a.qs1 + head * a.qs2;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 w = *(const u32x4*)(src + c * 16 + hf * 8);
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 x = in_seq[rb] ? w : z;
        qf[rb][c] = __builtin_bit_cast(bf16x8, x);
        if (scale_q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qf[rb][c][2 * e] = (__bf16)(bf16_lo(x[e]) * qmul);
            qf[rb][c][2 * e + 1] = (__bf16)(bf16_hi(x[e]) * qmul);
          }
        }
      }
    }
  } else
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // Every load of the row block (the q row, its row of the rotary table and
    // the gammas) is issued before any of them is used, so their latencies
    // overlap; a row past the end reads the last row and is zeroed.
    const int rowc = min(row[rb], S - 1);
    const uint16_t* src = (const uint16_t*)a.q + bl * a.qs0 + (tok0 + rowc) * a.qs1 + head * a.qs2;
    // (cos, sin) of this token's pairs from the table the prologue pass wrote
    const float2* csrow = a.cs + ((int64_t)bl * Sx + tok0 + rowc) * (D / 2);
    const float* gq = a.gq + head * a.gqs;
    const float c2 = a.c2;
    u32x4 qw[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) qw[c] = *(const u32x4*)(src + c * 16 + hf * 8);
    // the row as fp32 (zeros past the end) and its RMSNorm factor
    auto unpack_rms = [&](float (&x)[KC][8]) {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 w = in_seq[rb] ? qw[c] : z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[c][2 * e] = bf16_lo(w[e]);
          x[c][2 * e + 1] = bf16_hi(w[e]);
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[c][e] * x[c][e];
      ss = half_swap_sum(ss);
      return rsqrtf(ss * (1.0f / D) + a.eps);
    };
    if (a.inter) {
      // pairs (2j, 2j + 1): elements e, e + 1 of one chunk, pair index
      // (c*16 + hf*8 + e) / 2; Q' keeps the element order of q
      f32x4 ga[KC], gb[KC], t01[KC], t23[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        ga[c] = *(const f32x4*)(gq + c * 16 + hf * 8);
        gb[c] = *(const f32x4*)(gq + c * 16 + hf * 8 + 4);
        t01[c] = *(const f32x4*)(csrow + c * 8 + hf * 4);
        t23[c] = *(const f32x4*)(csrow + c * 8 + hf * 4 + 2);
      }
      float x[KC][8];
      const float r = unpack_rms(x);
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float g1 = e < 4 ? ga[c][e] : gb[c][e - 4];
          const float g2 = e < 4 ? ga[c][e + 1] : gb[c][e - 3];
          const f32x4 t = e < 4 ? t01[c] : t23[c];
          const float cs = t[(e & 2)], sn = t[(e & 2) + 1];
          const float u = x[c][e] * r * g1;
          const float w = x[c][e + 1] * r * g2;
          qf[rb][c][e] = (__bf16)((u * cs - w * sn) * c2);
          qf[rb][c][e + 1] = (__bf16)((w * cs + u * sn) * c2);
        }
    } else {
      f32x4 g1a[KC / 2], g1b[KC / 2], g2a[KC / 2], g2b[KC / 2], t4[KC / 2][4];
#pragma unroll
      for (int c = 0; c < KC / 2; ++c) {
        g1a[c] = *(const f32x4*)(gq + c * 16 + hf * 8);
        g1b[c] = *(const f32x4*)(gq + c * 16 + hf * 8 + 4);
        g2a[c] = *(const f32x4*)(gq + D / 2 + c * 16 + hf * 8);
        g2b[c] = *(const f32x4*)(gq + D / 2 + c * 16 + hf * 8 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) t4[c][e] = *(const f32x4*)(csrow + c * 16 + hf * 8 + 2 * e);
      }
      float x[KC][8];
      const float r = unpack_rms(x);
#pragma unroll
      for (int c = 0; c < KC / 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g1 = e < 4 ? g1a[c][e & 3] : g1b[c][e & 3];
          const float g2 = e < 4 ? g2a[c][e & 3] : g2b[c][e & 3];
          const float cs = t4[c][e >> 1][(e & 1) * 2], sn = t4[c][e >> 1][(e & 1) * 2 + 1];
          const float u = x[c][e] * r * g1;
          const float w = x[c + KC / 2][e] * r * g2;
          qf[rb][c][e] = (__bf16)((u * cs - w * sn) * c2);
          qf[rb][c + KC / 2][e] = (__bf16)((w * cs + u * sn) * c2);
        }
    }
  }

  // ---- tile bookkeeping: this workgroup covers key tiles [t_lo, ntiles);
  // tiles with no valid key are skipped
  const int ktiles = (S + BN - 1) / BN;
  const int t_lo = (int)((int64_t)part * ktiles / nparts);
  const int ntiles = (int)((int64_t)(part + 1) * ktiles / nparts);
  auto skipped = [&](int t) { const int n0 = t * BN; return n0 >= L && min(n0 + BN, S) <= T; };
  auto next_tile = [&](int t) {
    ++t;
    while (t < ntiles && skipped(t)) ++t;
    return t;
  };
  auto tile_masked = [&](int n0) { return n0 + BN > S || (L < T && n0 + BN > L && n0 < T); };
  auto key_ok = [&](int n) { return n < S && !(n >= L && n < T); };

  // ---- operand sources. All bounds live in the per-lane offset: a row that
  // must not be read gets an offset at the resource size, which reads zeros.
  const int64_t krow = (KFUSED || PRE) ? a.ks1 : D;  // elements between K rows
  const uint16_t* kbase = (KFUSED || PRE) ? (const uint16_t*)a.k + bl * a.ks0 + tok0 * a.ks1 + head * a.ks2
                                 : a.kp + (((int64_t)bl * a.H + head) * Sx + tok0) * D;
  const uint32_t knrec = (uint32_t)(((int64_t)(S - 1) * krow + D) * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, knrec);
  const uint16_t* vbase = (const uint16_t*)a.v + bl * a.vs0 + tok0 * a.vs1 + head * a.vs2;
  const uint32_t vnrec = (uint32_t)(((int64_t)(S - 1) * a.vs1 + D) * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, vnrec);

  // direct-load lane roles: run j of this wave covers LDS bytes
  // [(wave*RUNS + j) * 1024, +1024); lane L fills 16 bytes at 16*L of it
  int k_row[RUNS], k_src[RUNS], v_row[RUNS], v_src[RUNS];
#pragma unroll
  for (int j = 0; j < RUNS; ++j) {
    const int run = wave * RUNS + j;
    const int rr = run * RPR + lane / CPR;  // LDS row
    const int pos = lane % CPR;             // physical chunk in the row
    k_row[j] = key_of_row(rr);
    k_src[j] = (int)((k_row[j] * krow + (pos ^ k_swz<D>(rr)) * 8) * 2);
    v_row[j] = rr;
    v_src[j] = (int)(((int64_t)rr * a.vs1 + (pos ^ v_swz<D>(rr)) * 8) * 2);
  }

  // fused mode stages raw K through registers: chunk roles per thread
  int fk_key[KFUSED ? KCH : 1], fk_c[KFUSED ? KCH : 1];
  u32x4 fkr[KFUSED ? KCH : 1];
  float2 fcs[KFUSED ? KCH : 1][4];
  if constexpr (KFUSED) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + i * NT;
      fk_key[i] = ci / CPR;
      const int raw = ci % CPR;
      fk_c[i] = (raw >> 1) + (raw & 1) * (CPR / 2);  // rotary partner chunk sits in lane ^ 1
    }
  }

  auto issue_k = [&](int t, int buf) {
    const int n0 = t * BN;
    if constexpr (!KFUSED) {
      const bool msk = tile_masked(n0);
      const int nb = n0 * (int)(krow * 2);
      char* dst = kbuf(buf);
#pragma unroll
      for (int j = 0; j < RUNS; ++j) {
        uint32_t off = (uint32_t)(k_src[j] + nb);
        if (msk) off = key_ok(n0 + k_row[j]) ? off : knrec;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(dst + (wave * RUNS + j) * 1024), 16,
                                                 off, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int n = n0 + fk_key[i];
        const uint32_t off = key_ok(n) ? (uint32_t)((n * krow + fk_c[i] * 8) * 2) : knrec;
        fkr[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
        // half-split pairs: lanes c and c^1 share one group of 8 pair
        // angles and each fetches 4; interleaved: chunk c holds pairs 4c..4c+3
        const int j0 = a.inter ? 4 * fk_c[i] : (fk_c[i] % (CPR / 2)) * 8 + (fk_c[i] >= CPR / 2 ? 4 : 0);
        const float2* cp = a.cs + ((int64_t)bl * Sx + tok0 + min(n, S - 1)) * (D / 2) + j0;
#pragma unroll
        for (int e = 0; e < 4; ++e) fcs[i][e] = cp[e];
      }
    }
  };

  // fused mode: RMSNorm + M-RoPE of the staged raw K rows, written as K'
  auto finish_k = [&](int buf) {
    if constexpr (KFUSED) {
      char* dst = kbuf(buf);
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const u32x4 w = fkr[i];
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[2 * e] = bf16_lo(w[e]); x[2 * e + 1] = bf16_hi(w[e]); }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
        for (int s = 1; s < CPR; s <<= 1) ss += __shfl_xor(ss, s, CPR);
        const float r = rsqrtf(ss * (1.0f / D) + a.eps);
        const int c = fk_c[i];
        const bool first = c < CPR / 2;
        const float* gk = a.gk + head * a.gqs;
        float y[8], px[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[e] * r * gk[c * 8 + e];
        u32x4 o;
        if (a.inter) {
          // pairs (2j, 2j + 1) lie inside the chunk: elements e, e + 1
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float2 t = fcs[i][e >> 1];
            o[e >> 1] = pack_bf16(y[e] * t.x - y[e + 1] * t.y, y[e + 1] * t.x + y[e] * t.y);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) px[e] = __shfl_xor(y[e], 1, 64);
          float2 cs8[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 mine = fcs[i][e];
            const float2 other = make_float2(__shfl_xor(mine.x, 1, 64), __shfl_xor(mine.y, 1, 64));
            cs8[e] = first ? mine : other;
            cs8[4 + e] = first ? other : mine;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float z[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int q = 2 * e + h;
              z[h] = first ? (y[q] * cs8[q].x - px[q] * cs8[q].y) : (y[q] * cs8[q].x + px[q] * cs8[q].y);
            }
            o[e] = pack_bf16(z[0], z[1]);
          }
        }
        // LDS row holding key fk_key: inverse of key_of_row within its 32-block
        const int kk = fk_key[i], w5 = kk & 31;
        const int rr = (kk & ~31) | (((w5 >> 2) & 3) << 3) | ((w5 >> 4) << 2) | (w5 & 3);
        *(u32x4*)(dst + k_lds_off<D>(rr, c)) = o;
      }
    }
  };

  auto issue_v = [&](int t, int buf) {
    const int n0 = t * BN;
    const bool msk = tile_masked(n0);
    const int nb = n0 * (int)(a.vs1 * 2);
    char* dst = vbuf(buf);
#pragma unroll
    for (int j = 0; j < RUNS; ++j) {
      // V rows of padded keys read as zeros, so non-finite values there
      // cannot reach P.V (their probability is exactly 0)
      uint32_t off = (uint32_t)(v_src[j] + nb);
      if (msk) off = key_ok(n0 + v_row[j]) ? off : vnrec;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(dst + (wave * RUNS + j) * 1024), 16, off, 0, 0, 0);
    }
  };

  f32x16 oacc[RB][DB];
  float mrun[RB], lrun[RB], lrun2[RB], neg_m[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[rb][db][i] = 0.f;
    mrun[rb] = 0.f;
    lrun[rb] = 0.f;
    lrun2[rb] = 0.f;  // second partial row sum (two chains for latency)
  }
  // -m broadcast over a lane's 16 accumulators: the C input of each tile's
  // first Q.K' MFMA (read-only, so the tile loop copies nothing into S)
  f32x16 negm_vec[RB];
  auto refresh_neg_m = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      neg_m[rb] = -mrun[rb];
#pragma unroll
      for (int i = 0; i < 16; ++i) negm_vec[rb][i] = neg_m[rb];
    }
  };

  // v-operand read roles (transposing LDS read): lane 16g + j of a 16-lane
  // group addresses key (g/2)*16 + j/4 (+ u*8 + half*4 + kb*32) and head_dim
  // 16*(g%2) + 4*(j%4) (+ db*32); lane l then holds 4 consecutive keys of
  // dim db*32 + l%32.
  const int vg = lane >> 4, vj = lane & 15;
  const int v_key0 = (vg >> 1) * 16 + (vj >> 2);
  const int v_dim0 = 16 * (vg & 1) + 4 * (vj & 3);

  int t = t_lo;
  while (t < ntiles && skipped(t)) ++t;
  refresh_neg_m();
  bool first = true;
  // QK-RMSNorm bounds every logit: |Q''.K'| <= |Q''| |K'| and |K'| <=
  // max|gamma_k| sqrt(D) (a normalised row has mean square <= 1; the margin
  // covers K''s bf16 rounding). When that bound m is at most 40, m serves as
  // the row's "running max" from the start: no row max, no rescaling. Then
  // every P = exp2(S - m) >= 2^-80, so P and the P.V products stay normal
  // floats for any |V| >= 2^-46 (a larger m could push them into the
  // subnormal range, which the matrix cores flush).
  bool fixed_max = false;
  if constexpr (!PRE) {
    float gmax = fabsf(gk0);
    if constexpr (D > 64) gmax = fmaxf(gmax, fabsf(gk1));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) gmax = fmaxf(gmax, __shfl_xor(gmax, o, 64));
    const float kb = gmax * sqrtf((float)D) * (1.0f + 1.0f / 128);
    bool big = false;
    float mf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float n2 = 0.f;
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) n2 += (float)qf[rb][c][e] * (float)qf[rb][c][e];
      // padded query rows (whose output is zero whatever they hold) neither
      // decide nor need the bound
      mf[rb] = valid_row[rb] ? sqrtf(half_swap_sum(n2)) * kb : 0.f;
      big = big || !(mf[rb] <= 40.f);
    }
    if (__builtin_amdgcn_ballot_w64(big) == 0) {
      fixed_max = true;
      first = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) mrun[rb] = mf[rb];
      refresh_neg_m();
    }
  }

  // S^T = K'(t) Q'^T - m from K' buffer `kpar`: all K' fragments of the tile
  // are read first so the reads overlap each other and the MFMAs using them
  auto qk = [&](auto kpar, f32x16 (&st)[RB][NB]) {
    constexpr int cur = decltype(kpar)::value;
    const char* src = kbuf(cur);
    bf16x8 kf[KC][NB];
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
        kf[c][kb] = *(const bf16x8*)(src + k_lds_off<D>(kb * 32 + m, 2 * c + hf));
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          st[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c][kb], qf[rb][c],
                                                               c == 0 ? negm_vec[rb] : st[rb][kb], 0, 0, 0);
    // keep kAhead fragment reads in flight ahead of the MFMAs
    constexpr int kFrags = KC * NB, kAhead = kKAhead;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < kFrags; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
      if (i + kAhead < kFrags) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // masking, running max (lazy rescale of O and the row sums), exponentials
  // rounded to bf16 as the P operand, and the row sum of the rounded P
  auto softmax = [&](f32x16 (&st)[RB][NB], int n0, bf16x8 (&pf)[RB][NB][2]) {
    if (tile_masked(n0)) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool ok = key_ok(n0 + kb * 32 + hf * 16 + i);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) st[rb][kb][i] = ok ? st[rb][kb][i] : -INFINITY;
        }
    }
    if (!fixed_max) {
    // row max of this tile relative to the running max
    float mx[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float v = st[rb][0][0];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) v = fmaxf(v, st[rb][kb][i]);
      mx[rb] = half_swap_max(v);
      grow = grow || mx[rb] > kRescaleLog2;
    }
    if (first || __builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float delta = first ? mx[rb] : fmaxf(mx[rb], 0.f);
        const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-delta);
        mrun[rb] += delta;
        lrun[rb] *= alpha;
        lrun2[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[rb][db][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) st[rb][kb][i] -= delta;
      }
      first = false;
      refresh_neg_m();
    }
    }
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[rb][kb][u][e] = (__bf16)__builtin_amdgcn_exp2f(st[rb][kb][u * 8 + e]);
#pragma unroll
          for (int e = 0; e < 8; e += 4) {
            const bf16x2 p0 = {pf[rb][kb][u][e], pf[rb][kb][u][e + 1]};
            const bf16x2 p1 = {pf[rb][kb][u][e + 2], pf[rb][kb][u][e + 3]};
            lrun[rb] = __builtin_amdgcn_fdot2_f32_bf16(p0, one, lrun[rb], false);
            lrun2[rb] = __builtin_amdgcn_fdot2_f32_bf16(p1, one, lrun2[rb], false);
          }
        }
  };

  // O^T += V^T P^T from V buffer `vpar`
  auto pv = [&](auto vpar, const bf16x8 (&pf)[RB][NB][2]) {
    constexpr int cur = decltype(vpar)::value;
    const char* vsrc = vbuf(cur);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int key = kb * 32 + u * 8 + v_key0;
          const int dim = db * 32 + v_dim0;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vsrc + v_lds_off<D>(key, dim >> 3) + (dim & 7) * 2));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vsrc + v_lds_off<D>(key + 4, dim >> 3) + (dim & 7) * 2));
          // assemble the operand from whole dwords: building it from 16-bit
          // elements is miscompiled by this toolchain (halves get duplicated)
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[rb][kb][u], oacc[rb][db], 0, 0, 0);
        }
    {
      // two transposing reads per MFMA; keep kPvPace of them in flight
      constexpr int vM = NB * 2 * DB, vA = kPvPace;
      __builtin_amdgcn_sched_group_barrier(0x100, vA, 0);
#pragma unroll
      for (int i = 0; i < vM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
        if (2 * i + 2 + vA <= 2 * vM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (2 * i + 1 + vA <= 2 * vM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };

  if (t < ntiles) {
    issue_v(t, 0);
    issue_k(t, 0);
    if constexpr (KFUSED) finish_k(0);
  }
  // one tile t whose K' and V were loaded into buffer `parity`; the loads
  // of the next tile go to the other buffer while this one is computed
  auto step = [&](auto parity) {
    constexpr int cur = decltype(parity)::value;
    const int tn = next_tile(t);
    // K'(t) and V(t) are in LDS and every wave is done with buffer cur ^ 1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tn < ntiles) {
      issue_v(tn, cur ^ 1);
      issue_k(tn, cur ^ 1);
      if constexpr (KFUSED) finish_k(cur ^ 1);
    }
    f32x16 st[RB][NB];
    qk(parity, st);
    bf16x8 pf[RB][NB][2];
    softmax(st, t * BN, pf);
    // The wave raises its issue priority for this matrix-core run so the
    // SIMD's other wave (in its exponential phase) fills around it.
    __builtin_amdgcn_s_setprio(1);
    pv(parity, pf);
    __builtin_amdgcn_s_setprio(0);
    t = tn;
  };
  while (t < ntiles) {
    step(Parity<0>{});
    if (t >= ntiles) break;
    step(Parity<1>{});
  }

  // ---- row sums (both lane halves hold a share of each row)
  float ltot[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) ltot[rb] = half_swap_sum(lrun[rb] + lrun2[rb]);

  // ---- split tile: this part's unnormalised (O, m, l) go to the workspace;
  // split_merge_kernel combines the parts after this launch
  if (nparts > 1) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float* rec = part_record<D, WAVES, RB>(gp.part, nparts, gt - gp.n_whole, part, wave * RB + rb);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(rec + ((db * 4 + g) * 64 + lane) * 4) =
              f32x4{oacc[rb][db][g * 4], oacc[rb][db][g * 4 + 1], oacc[rb][db][g * 4 + 2], oacc[rb][db][g * 4 + 3]};
      // a part that processed no key tile contributes nothing
      rec[DB * 16 * 64 + lane] = first ? -INFINITY : mrun[rb];
      rec[DB * 16 * 64 + 64 + lane] = ltot[rb];
    }
    return;
  }

  // ---- epilogue: O / l, padded rows are exact zeros (selected, not scaled,
  // so whatever a padded query row computed cannot leak)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!in_seq[rb]) continue;
    const float inv = 1.0f / ltot[rb];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t w0 = pack_bf16(oacc[rb][db][g * 4 + 0] * inv, oacc[rb][db][g * 4 + 1] * inv);
        uint32_t w1 = pack_bf16(oacc[rb][db][g * 4 + 2] * inv, oacc[rb][db][g * 4 + 3] * inv);
        w0 = valid_row[rb] ? w0 : 0u;
        w1 = valid_row[rb] ? w1 : 0u;
        *(u32x2*)(outp[rb] + db * 32 + g * 8 + hf * 4) = u32x2{w0, w1};
      }
    if (lsep[rb] && hf == 0) *lsep[rb] = valid_row[rb] ? mrun[rb] * kLn2 + logf(ltot[rb]) : -INFINITY;
  }
}

// Combines the nsplit parts of each split query tile by the log-sum-exp rule
// and writes the output rows and LSE exactly as the attention epilogue does.
// One thread per (split tile, 32-row block, 4-dim chunk, lane).
template <int D, int WAVES, int RB, int G>
__global__ __launch_bounds__(256) void split_merge_kernel(Group<G> gp) {
  constexpr int BM = WAVES * 32 * RB;
  constexpr int CH = D / 8;  // 4-float chunks per lane record
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int lane = gid & 63, m = lane & 31, hf = lane >> 5;
  const int c = (gid >> 6) % CH;
  const int rr = (gid >> 6) / CH % (WAVES * RB);
  const int st = (gid >> 6) / CH / (WAVES * RB);
  if (st >= gp.n_split) return;
  int tile;
  const Args& a = gp.p[group_problem(gp, gp.n_whole + st, tile)];
  const int qt = tile % a.n_qt, bh = tile / a.n_qt;
  const int head = bh % a.H, b = bh / a.H;
  const SeqView sv = seq_view(a, b);
  const int S = sv.S, T = a.T, bl = sv.bl;
  const int64_t tok0 = sv.tok0;
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), T) : T;
  const int q0 = qt * BM;
  // a tile made only of padded text slots was written by the attention kernel
  if (q0 >= L && min(q0 + BM, S) <= T) return;
  const int row = q0 + rr * 32 + m;
  if (row >= S) return;
  const bool valid_row = !(row >= L && row < T);
  const int nparts = gp.nsplit;

  // every part's loads are issued before any is used
  float mp[kMaxSplit], lp[kMaxSplit];
  f32x4 op[kMaxSplit];
#pragma unroll
  for (int p = 0; p < kMaxSplit; ++p) {
    if (p < nparts) {
      const float* rec = part_record<D, WAVES, RB>(gp.part, nparts, st, p, rr);
      mp[p] = rec[CH * 4 * 64 + lane];
      lp[p] = rec[CH * 4 * 64 + 64 + lane];
      op[p] = *(const f32x4*)(rec + (c * 64 + lane) * 4);
    }
  }
  float m_all = -INFINITY;
#pragma unroll
  for (int p = 0; p < kMaxSplit; ++p)
    if (p < nparts) m_all = fmaxf(m_all, mp[p]);
  float l_all = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < kMaxSplit; ++p) {
    if (p < nparts) {
      const float f = mp[p] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp[p] - m_all);
      l_all += f * lp[p];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += f * op[p][e];
    }
  }
  const float inv = 1.0f / l_all;
  uint32_t w0 = pack_bf16(o[0] * inv, o[1] * inv);
  uint32_t w1 = pack_bf16(o[2] * inv, o[3] * inv);
  w0 = valid_row ? w0 : 0u;
  w1 = valid_row ? w1 : 0u;
  const int db = c >> 2, g = c & 3;
  uint16_t* outp = (uint16_t*)a.out + bl * a.os0 + (tok0 + row) * a.os1 + head * a.os2;
  *(u32x2*)(outp + db * 32 + g * 8 + hf * 4) = u32x2{w0, w1};
  if (a.lse && c == 0 && hf == 0)
    a.lse[((int64_t)bl * a.H + head) * a.S + tok0 + row] = valid_row ? m_all * kLn2 + logf(l_all) : -INFINITY;
}

}  // namespace mra
