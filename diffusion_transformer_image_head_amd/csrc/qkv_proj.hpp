// fp8 e4m3 QKV projection with the QK-RMSNorm + 3D M-RoPE epilogue (gfx950).
//
// The checkpoint stores the fused qkv weight [3 * H * D, hidden] (Q, K, V rows
// stacked) as float8 e4m3 with one scale per output row; the real weight is
// the fp8 value times its row's scale (unsloth commit log for the Ideogram 4
// backend). The projection feeds the attention's QK-RMSNorm and 3D M-RoPE
// (Ideogram 4.0 announcement thread), so its epilogue produces the attention's
// operands directly:
//   q_op = bf16(qscale * rope(rmsnorm(x Wq^T) * gamma_q)),
//   k_op = bf16(rope(rmsnorm(x Wk^T) * gamma_k)),  v = bf16(x Wv^T).
//
// One workgroup per (128 tokens, a pair of heads of the stacked Q|K|V rows =
// 256 output rows), 4 waves, each 64 tokens x one head; two workgroups per
// CU. Output transposed on the matrix cores: C^T (rows x tokens) = W x^T with
// v_mfma_f32_32x32x16_bf16, A = W rows and B = x rows, both read from LDS.
// Each 64-wide hidden chunk of x (bf16) and of W (fp8, as stored) arrives by
// buffer loads that write LDS directly, one chunk ahead into the other of two
// stages, so there is one barrier per chunk. W stays fp8 in LDS (half the
// bytes of bf16) and is widened in registers right before its MFMA with
// v_cvt_scalef32_pk_bf16_fp8 (exact for e4m3); the row scale factors out of
// the sum and is applied in the epilogue. A lane pair then holds all 128 rows
// of one token, so the RMSNorm is lane-local plus one swap and each rotary
// pair sits in one lane.
#pragma once

#include "attn_bf16.hpp"

namespace mra {

struct QkvArgs {
  const uint16_t* x;      // [M, hidden] bf16, row stride xs
  int64_t xs;
  const uint8_t* w8;      // [3 H D, hidden] e4m3
  const float* wsc;       // [3 H D]
  const float2* cs;       // (cos, sin) [M, D/2]
  const float* gq;
  const float* gk;
  uint16_t* out[3];       // q_op, k_op, v: [M, H, D] with (token, head) strides
  int64_t os[3][2];
  int32_t M, hidden, H, n_mt;
  int32_t nxcd;           // XCDs of the device
  int32_t gqs;            // elements between two heads' gamma rows (0: shared [D])
  int32_t inter;          // rotary pairs (2j, 2j + 1) instead of (j, j + D/2)
  float eps, qscale;
};

// The launch configuration: 4 waves of 64 tokens (two waves per head of a
// head pair, so 128 tokens x 2 heads per workgroup), 64-wide hidden chunks,
// 2 LDS stages.
constexpr int kQkvWaves = 4, kQkvChunk = 64, kQkvStages = 2, kQkvTokPerWave = 64;

// WAVES waves per workgroup, half of them on each head of the pair, each
// wave TPW tokens: a workgroup computes (TPW * WAVES / 2 tokens) x (2 heads).
// KB hidden elements per pipeline stage, NST stages in LDS. The defaults
// (4 waves, 64 tokens per wave, 64-wide chunks, 2 stages: 64 KB of LDS, two
// workgroups per CU) measured fastest; 8-wave workgroups (one per CU, three
// stages), 32-wide chunks with 3 to 6 stages, and 128 tokens per wave (one
// wave per SIMD, accumulators in AGPRs) were slower.
template <int D, int WAVES, int KB, int NST, int TPW>
__global__ __launch_bounds__(WAVES * 64, (WAVES == 4 && TPW <= 64) ? 2 : 1) void qkv_proj_kernel(QkvArgs g) {
  constexpr int TOK = TPW * (WAVES / 2);   // token rows per workgroup
  constexpr int TB = TPW / 32;             // 32-token blocks per wave
  constexpr int XRB = KB * 2, WRB = KB;    // bytes per x row (bf16) and per W row (fp8)
  constexpr int XB = TOK * XRB, WB = 2 * D * WRB;
  constexpr int XRUNS = XB / 1024 / WAVES, WRUNS = WB / 1024 / WAVES;
  constexpr int XCPR = XRB / 16, WCPR = WRB / 16;        // 16-byte chunks per row
  constexpr int XRPB = 256 / XRB, WRPB = 256 / WRB;      // rows per 256-byte bank row
  constexpr int NL = XRUNS + WRUNS;                      // direct loads per thread per stage
  constexpr int DB = D / 32, NP = KB / 32;
  static_assert(D == 128, "written for head_dim 128");
  static_assert(XRUNS >= 1 && XRUNS * WAVES * 1024 == XB && WRUNS >= 1 && WRUNS * WAVES * 1024 == WB,
                "stages must split into whole 1 KiB runs per wave");
  static_assert(NST >= 2 && NST <= 6 && (NST - 2) * NL < 64, "stage count and vmcnt range");
  // Each stage is its own LDS object (the stage index is a compile-time
  // constant in every unrolled step, so reads of one stage never wait for the
  // loads in flight into another). 16-byte chunk c of row r sits at
  // c ^ ((r / RPB) mod CPR): the 16 consecutive rows that one 128-bit read
  // serves per clock land in 16 distinct chunk slots of the 64 banks.
  __shared__ __attribute__((aligned(1024))) char X0[XB];
  __shared__ __attribute__((aligned(1024))) char X1[XB];
  __shared__ __attribute__((aligned(1024))) char X2[NST > 2 ? XB : 16];
  __shared__ __attribute__((aligned(1024))) char X3[NST > 3 ? XB : 16];
  __shared__ __attribute__((aligned(1024))) char X4[NST > 4 ? XB : 16];
  __shared__ __attribute__((aligned(1024))) char X5[NST > 5 ? XB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t W0[WB];
  __shared__ __attribute__((aligned(1024))) uint8_t W1[WB];
  __shared__ __attribute__((aligned(1024))) uint8_t W2[NST > 2 ? WB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t W3[NST > 3 ? WB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t W4[NST > 4 ? WB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t W5[NST > 5 ? WB : 16];
  auto xst = [&](auto st) -> char* {
    constexpr int i = decltype(st)::value;
    if constexpr (i == 0) return X0; else if constexpr (i == 1) return X1; else if constexpr (i == 2) return X2;
    else if constexpr (i == 3) return X3; else if constexpr (i == 4) return X4; else return X5;
  };
  auto wst = [&](auto st) -> uint8_t* {
    constexpr int i = decltype(st)::value;
    if constexpr (i == 0) return W0; else if constexpr (i == 1) return W1; else if constexpr (i == 2) return W2;
    else if constexpr (i == 3) return W3; else if constexpr (i == 4) return W4; else return W5;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m = lane & 31, hf = lane >> 5;
  const int tg = wave % (WAVES / 2), hh = wave / (WAVES / 2);  // tokens tg*64.., head hh of the pair
  // Logical tile order (each XCD runs a contiguous range): groups of GT
  // token tiles; within a group, head pair after head pair, GT token tiles
  // each. The workgroups resident together then share a few token tiles of x
  // and a few head pairs of W per hidden chunk, so both are fetched into L2 a
  // few times instead of x once per head pair.
  constexpr int GT = 8;
  const int nhp = (3 * g.H + 1) / 2;
  const int tile = xcd_remap(blockIdx.x, gridDim.x, g.nxcd);
  const int full = g.n_mt / GT;
  int mt, hp;
  if (tile < full * GT * nhp) {
    const int tq = tile / (GT * nhp), w = tile % (GT * nhp);
    hp = w / GT;
    mt = tq * GT + w % GT;
  } else {
    const int r = tile - full * GT * nhp, gsz = g.n_mt - full * GT;
    hp = r / gsz;
    mt = full * GT + r % gsz;
  }
  const int hb0 = 2 * hp, nvalid = min(2, 3 * g.H - hb0);
  const int hb = hb0 + hh;
  const int t0 = mt * TOK + tg * TPW;
  auto xswz = [](int r) { return (r / XRPB) & (XCPR - 1); };
  auto wswz = [](int r) { return (r / WRPB) & (WCPR - 1); };

  // Direct loads: lane L of 1 KiB run q fills row q * (1024 / RB) + L / CPR,
  // physical chunk L % CPR. x rows past M and W rows of a second head past
  // the last one read zeros.
  const uint32_t xnrec = (uint32_t)((int64_t)g.M * g.xs * 2);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(g.x, xnrec);
  // (fixed-size arrays: a lambda capturing an array sized by a constexpr
  // local makes the host compiler drop the kernel's launch stub)
  static_assert(XRUNS <= 8 && WRUNS <= 8, "offset arrays hold 8 runs");
  uint32_t xoff[8];
#pragma unroll
  for (int j = 0; j < XRUNS; ++j) {
    const int r = (wave * XRUNS + j) * (1024 / XRB) + lane / XCPR;
    const int tok = mt * TOK + r;
    const int c = (lane % XCPR) ^ xswz(r);
    xoff[j] = tok < g.M ? (uint32_t)(((int64_t)tok * g.xs + c * 8) * 2) : xnrec;
  }
  const uint32_t wnrec = (uint32_t)nvalid * D * (uint32_t)g.hidden;
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(g.w8 + (int64_t)hb0 * D * g.hidden, wnrec);
  uint32_t woff[8];
#pragma unroll
  for (int j = 0; j < WRUNS; ++j) {
    const int r = (wave * WRUNS + j) * (1024 / WRB) + lane / WCPR;
    woff[j] = (uint32_t)r * (uint32_t)g.hidden + (uint32_t)(((lane % WCPR) ^ wswz(r)) * 16);
  }
  auto issue = [&](int kc, char* xd, uint8_t* wd) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < XRUNS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr_t)(xd + (wave * XRUNS + j) * 1024), 16,
                                               xoff[j] == xnrec ? xnrec : xoff[j] + kc * KB * 2, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < WRUNS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr_t)(wd + (wave * WRUNS + j) * 1024), 16,
                                               woff[j] + kc * KB, 0, 0, 0);
  };

  f32x16 acc[TB][DB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tb][db][i] = 0.f;

  // A stage of KB hidden elements = KB / 16 MFMA k-steps, taken in pairs. In
  // pair j, lane half hf holds the 16 consecutive hidden elements
  // 16*(2j + hf) .. +15 of its W row (one 128-bit read of fp8) and the same
  // elements of its x row (two 128-bit reads); the first k-step of the pair
  // uses the lower 8 of them, the second the upper 8. Every k-step thus sums
  // the same 16 hidden elements in W and in x (the MFMA's k order inside a
  // step does not matter), and the steps cover the stage once. The fp8 codes
  // are widened in registers (v_cvt_scalef32_pk_bf16_fp8, exact for e4m3);
  // the row scale factors out of the sum and is applied at the end.
  auto compute = [&](const char* Xs, const uint8_t* Ws) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      u32x4 wr[DB];
      bf16x8 xb[TB][2];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int r = hh * D + db * 32 + m;
        wr[db] = *(const u32x4*)(Ws + r * WRB + (((2 * j + hf) ^ wswz(r)) << 4));
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int r = tg * TPW + tb * 32 + m;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          xb[tb][s] = *(const bf16x8*)(Xs + r * XRB + (((2 * (2 * j + hf) + s) ^ xswz(r)) << 4));
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          u32x4 o;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t w = wr[db][2 * s + e];
            o[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
            o[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
          }
          const bf16x8 a = __builtin_bit_cast(bf16x8, o);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
            acc[tb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xb[tb][s], acc[tb][db], 0, 0, 0);
        }
    }
  };

  // Stage i holds the chunks kc with kc % NST == i. Before chunk kc is
  // computed, each wave waits for its own loads of kc (those of the next
  // NST - 2 chunks may stay in flight) and the barrier makes every wave's
  // loads visible; after the barrier every wave is done with chunk kc - 1,
  // whose stage then receives chunk kc + NST - 1. The bare s_barrier (not
  // __syncthreads, whose fence waits for every load) keeps the later chunks
  // in flight across it.
  const int nk = g.hidden / KB;
  auto wait_ahead = [&](int n) __attribute__((always_inline)) {
    // vmcnt(n * NL): vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt not waited
    constexpr int c1 = NL, c2 = 2 * NL, c3 = 3 * NL, c4 = 4 * NL;
    if (n >= 4) __builtin_amdgcn_s_waitcnt(0x0F70 | (c4 & 15) | ((c4 >> 4) << 14));
    else if (n == 3) __builtin_amdgcn_s_waitcnt(0x0F70 | (c3 & 15) | ((c3 >> 4) << 14));
    else if (n == 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (c2 & 15) | ((c2 >> 4) << 14));
    else if (n == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (c1 & 15) | ((c1 >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  };
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) {
    if (i < nk) {
      if (i == 0) issue(0, X0, W0);
      else if (i == 1) issue(1, X1, W1);
      else if (i == 2) issue(2, xst(Parity<(NST > 2 ? 2 : 0)>{}), wst(Parity<(NST > 2 ? 2 : 0)>{}));
      else if (i == 3) issue(3, xst(Parity<(NST > 3 ? 3 : 0)>{}), wst(Parity<(NST > 3 ? 3 : 0)>{}));
      else issue(4, xst(Parity<(NST > 4 ? 4 : 0)>{}), wst(Parity<(NST > 4 ? 4 : 0)>{}));
    }
  }
  auto step = [&](int kc, auto stage) __attribute__((always_inline)) {
    constexpr int cur = decltype(stage)::value;
    constexpr int nxt = (cur + NST - 1) % NST;
    wait_ahead(min(NST - 2, nk - 1 - kc));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kc + NST - 1 < nk) {
      issue(kc + NST - 1, xst(Parity<nxt>{}), wst(Parity<nxt>{}));
    }
    compute(xst(stage), wst(stage));
  };
  for (int kc = 0; kc < nk; kc += NST) {
    step(kc, Parity<0>{});
    if (kc + 1 < nk) step(kc + 1, Parity<1>{});
    if constexpr (NST > 2) if (kc + 2 < nk) step(kc + 2, Parity<(NST > 2 ? 2 : 0)>{});
    if constexpr (NST > 3) if (kc + 3 < nk) step(kc + 3, Parity<(NST > 3 ? 3 : 0)>{});
    if constexpr (NST > 4) if (kc + 4 < nk) step(kc + 4, Parity<(NST > 4 ? 4 : 0)>{});
    if constexpr (NST > 5) if (kc + 5 < nk) step(kc + 5, Parity<(NST > 5 ? 5 : 0)>{});
  }
  if (hh >= nvalid) return;
  const int part = hb / g.H, head = hb % g.H;

  // ---- epilogue: row scale; Q/K heads: RMSNorm, gamma, rotation (Q: qscale)
  const float* wsc = g.wsc + hb * D;
  const float* gamma = (part == 0 ? g.gq : g.gk) + head * g.gqs;
  const float qs = part == 0 ? g.qscale : 1.0f;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int tok = t0 + tb * 32 + m;
    float y[DB][16];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const f32x4 sc = *(const f32x4*)(wsc + db * 32 + gg * 8 + hf * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[db][gg * 4 + e] = acc[tb][db][gg * 4 + e] * sc[e];
      }
    if (part < 2) {
      float ss = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += y[db][i] * y[db][i];
      ss = half_swap_sum(ss);
      const float r = rsqrtf(ss * (1.0f / D) + g.eps);
      const float2* csrow = g.cs + (int64_t)min(tok, g.M - 1) * (D / 2);
      if (g.inter) {
        // pair j = (2j, 2j + 1): registers e and e + 1 of one lane; the four
        // dims d0..d0+3 of a register group are pairs d0/2 and d0/2 + 1
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const int d0 = db * 32 + gg * 8 + hf * 4;
            const f32x4 c01 = *(const f32x4*)(csrow + d0 / 2);
            const f32x4 gv = *(const f32x4*)(gamma + d0);
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const float cs = c01[e], sn = c01[e + 1];
              const float u = y[db][gg * 4 + e] * r * gv[e];
              const float w = y[db][gg * 4 + e + 1] * r * gv[e + 1];
              y[db][gg * 4 + e] = (u * cs - w * sn) * qs;
              y[db][gg * 4 + e + 1] = (w * cs + u * sn) * qs;
            }
          }
      } else
#pragma unroll
      for (int db = 0; db < DB / 2; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int j0 = db * 32 + gg * 8 + hf * 4;
          const f32x4 c01 = *(const f32x4*)(csrow + j0);
          const f32x4 c23 = *(const f32x4*)(csrow + j0 + 2);
          const f32x4 g1 = *(const f32x4*)(gamma + j0);
          const f32x4 g2 = *(const f32x4*)(gamma + j0 + D / 2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float cs = e < 2 ? c01[2 * e] : c23[2 * (e - 2)];
            const float sn = e < 2 ? c01[2 * e + 1] : c23[2 * (e - 2) + 1];
            const float u = y[db][gg * 4 + e] * r * g1[e];
            const float w = y[db + DB / 2][gg * 4 + e] * r * g2[e];
            y[db][gg * 4 + e] = (u * cs - w * sn) * qs;
            y[db + DB / 2][gg * 4 + e] = (w * cs + u * sn) * qs;
          }
        }
    }
    if (tok < g.M) {
      uint16_t* dst = g.out[part] + (int64_t)tok * g.os[part][0] + (int64_t)head * g.os[part][1];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
          *(u32x2*)(dst + db * 32 + gg * 8 + hf * 4) =
              u32x2{pack_bf16(y[db][gg * 4], y[db][gg * 4 + 1]), pack_bf16(y[db][gg * 4 + 2], y[db][gg * 4 + 3])};
    }
  }
}

}  // namespace mra
