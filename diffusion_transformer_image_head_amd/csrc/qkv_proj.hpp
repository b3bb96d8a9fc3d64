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
// One workgroup per (256 tokens, one head of Q, K or V = 128 output rows),
// 4 waves of 64 tokens. Output transposed on the matrix cores:
// C^T (rows x tokens) = W x^T with v_mfma_f32_32x32x16_bf16, A = W rows and
// B = x rows, both read from LDS. Each 32-wide hidden chunk of x (256 rows)
// arrives by direct loads one chunk ahead (16 rows per load instruction,
// instead of one row per lane); the W chunk arrives as fp8 two chunks ahead,
// is widened once to bf16 in LDS by the whole workgroup one chunk ahead
// (v_cvt_scalef32_pk_bf16_fp8: exact for e4m3; double-buffered, so one
// barrier per chunk) and is read by the four waves; the row scale factors out
// of the sum and is applied in the epilogue. A lane pair then holds all 128 rows of one token, so the RMSNorm
// is lane-local plus one swap and each rotary pair (j, j + 64) sits in one
// lane.
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
  int32_t gqs;            // elements between two heads' gamma rows (0: shared [D])
  int32_t inter;          // rotary pairs (2j, 2j + 1) instead of (j, j + D/2)
  float eps, qscale;
};

template <int D>
__global__ __launch_bounds__(256, 2) void qkv_proj_kernel(QkvArgs g) {
  constexpr int KB = 32;              // hidden chunk
  constexpr int W8B = D * KB;         // fp8 chunk bytes (4 KB)
  constexpr int XB = 256 * KB * 2;    // bf16 x chunk bytes (16 KB)
  constexpr int DB = D / 32, KS = KB / 16;
  static_assert(D == 128, "written for head_dim 128");
  // x chunk: 256 token rows of 64 bytes; W chunk: 128 rows of 32 fp8 bytes,
  // widened to 128 rows of 64 bytes. 16-byte chunk c of a 64-byte row r sits
  // at c ^ ((r >> 2) & 3): 16 consecutive rows read at one chunk are
  // conflict-free on 64 banks.
  __shared__ __attribute__((aligned(1024))) char X0[XB];
  __shared__ __attribute__((aligned(1024))) char X1[XB];
  __shared__ __attribute__((aligned(1024))) uint8_t W0[W8B];
  __shared__ __attribute__((aligned(1024))) uint8_t W1[W8B];
  __shared__ __attribute__((aligned(1024))) char Wb0[D * KB * 2];
  __shared__ __attribute__((aligned(1024))) char Wb1[D * KB * 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m = lane & 31, hf = lane >> 5;
  // Logical tile order (each XCD runs a contiguous range): groups of GT
  // token tiles; within a group, head after head, GT token tiles each. The
  // workgroups resident together then share a few token tiles of x and a few
  // heads of W per hidden chunk, so both are fetched into L2 a few times
  // instead of x once per head.
  constexpr int GT = 8;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int nh = 3 * g.H, full = g.n_mt / GT;
  int mt, hb;
  if (tile < full * GT * nh) {
    const int tg = tile / (GT * nh), w = tile % (GT * nh);
    hb = w / GT;
    mt = tg * GT + w % GT;
  } else {
    const int r = tile - full * GT * nh, gsz = g.n_mt - full * GT;
    hb = r / gsz;
    mt = full * GT + r % gsz;
  }
  const int part = hb / g.H, head = hb % g.H;
  const int t0 = mt * 256 + wave * 64;
  auto swz = [](int r) { return (r >> 2) & 3; };

  // x chunk: run j of this wave = bytes [(wave*4+j)*1024, +1024) = rows
  // (wave*4+j)*16 + L/4, physical chunk L%4; rows past M read zeros
  const uint32_t xnrec = (uint32_t)((int64_t)g.M * g.xs * 2);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(g.x, xnrec);
  uint32_t xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (wave * 4 + j) * 16 + (lane >> 2);
    const int tok = mt * 256 + r;
    const int c = (lane & 3) ^ swz(r);
    xoff[j] = tok < g.M ? (uint32_t)(((int64_t)tok * g.xs + c * 8) * 2) : xnrec;
  }
  auto issue_x = [&](int kc, char* dst) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr_t)(dst + (wave * 4 + j) * 1024), 16,
                                               xoff[j] == xnrec ? xnrec : xoff[j] + kc * KB * 2, 0, 0, 0);
  };
  // W chunk: wave's run = bytes [wave*1024, +1024) = rows wave*32 + L/2, bytes (L%2)*16
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(g.w8 + (int64_t)hb * D * g.hidden, (uint32_t)(D * g.hidden));
  const uint32_t woff = (uint32_t)((wave * 32 + (lane >> 1)) * g.hidden + (lane & 1) * 16);
  auto issue_w = [&](int kc, uint8_t* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr_t)(dst + wave * 1024), 16, woff + kc * KB, 0, 0, 0);
  };
  // widen: thread t converts row t/2, fp8 bytes (t%2)*16..+15 into logical
  // chunks (t%2)*2, +1 of the bf16 row
  auto widen = [&](const uint8_t* src, char* Wb) {
    const int row = tid >> 1, h = tid & 1;
    const u32x4 a = *(const u32x4*)(src + row * KB + h * 16);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t w = a[2 * c + e];
        o[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
        o[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
      }
      *(u32x4*)(Wb + row * (KB * 2) + (((h * 2 + c) ^ swz(row)) << 4)) = o;
    }
  };

  f32x16 acc[2][DB];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tb][db][i] = 0.f;

  // Chunk i: W8(i) lands two steps ahead and is widened one step ahead, x(i)
  // lands one step ahead; one barrier per step: after it x(i) and W8(i+1)
  // have landed, Wb(i) is complete, and every wave is done with x(i-1),
  // Wb(i-1) and W8(i).
  const int nk = g.hidden / KB;
  issue_x(0, X0);
  issue_w(0, W0);
  if (nk > 1) issue_w(1, W1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  widen(W0, Wb0);
  auto step = [&](int kc, auto parity) {
    constexpr int cur = decltype(parity)::value;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kc + 1 < nk) issue_x(kc + 1, cur ? X0 : X1);
    if (kc + 2 < nk) issue_w(kc + 2, cur ? W1 : W0);
    if (kc + 1 < nk) widen(cur ? W0 : W1, cur ? Wb0 : Wb1);
    const char* Wb = cur ? Wb1 : Wb0;
    const char* Xs = cur ? X1 : X0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 xb[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int r = wave * 64 + tb * 32 + m;
        xb[tb] = *(const bf16x8*)(Xs + r * (KB * 2) + (((2 * ks + hf) ^ swz(r)) << 4));
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = db * 32 + m;
        const bf16x8 a = *(const bf16x8*)(Wb + row * (KB * 2) + (((2 * ks + hf) ^ swz(row)) << 4));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[tb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xb[tb], acc[tb][db], 0, 0, 0);
      }
    }
  };
  for (int kc = 0; kc < nk; kc += 2) {
    step(kc, Parity<0>{});
    if (kc + 1 < nk) step(kc + 1, Parity<1>{});
  }

  // ---- epilogue: row scale; Q/K heads: RMSNorm, gamma, rotation (Q: qscale)
  const float* wsc = g.wsc + hb * D;
  const float* gamma = (part == 0 ? g.gq : g.gk) + head * g.gqs;
  const float qs = part == 0 ? g.qscale : 1.0f;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
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
