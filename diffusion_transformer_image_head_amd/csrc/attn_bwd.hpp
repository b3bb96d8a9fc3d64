// Backward pass of the fused QK-RMSNorm + 3D M-RoPE attention (bf16, D=128),
// for training (LoRA on the attention projections with gradient
// checkpointing: SimpleTuner quickstart for the Ideogram 4 DiT; the forward
// is the operation of the Ideogram 4.0 announcement thread and of "Ideogram 4
// deep dive", section 4 part 2).
//
// With Q'' = bf16(c2 * rope(rmsnorm(q))) (c2 = scale * log2 e, the forward's
// query operand), K' = bf16(rope(rmsnorm(k))), S2 = Q'' K'^T (log2 units) and
// the forward's LSE in log2 units l2:
//   P = exp2(S2 - l2),  D_i = sum_d dO_id O_id,
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),
//   dQ' = scale dS K',  dK' = scale dS^T Q' = ln2 * dS^T Q'',
// then the transpose rotation and the RMSNorm backward turn dQ', dK' into dq,
// dk and the gamma gradients.
//
// Kernels: bwd_delta_kernel (D and l2 per row); bwd_fused_kernel, one launch
// of three independent roles: dK, and dV, each recomputing S (bwd_dkdv_body:
// one workgroup per 128 keys, 32 per wave, streaming 32-query tiles of Q''
// and dO through LDS), and dQ (bwd_dq_body: one workgroup per 128 queries,
// streaming 32-key tiles of K' and V); bwd_dgamma_kernel (fixed-order sum of
// the per-workgroup gamma partials).
// The dk/dv and dq roles work per item
// (seq_view): a padded batch item, or one sequence of a packed layout whose
// streams start at the sequence's first token and end with its last, so a
// sequence only sees its own tokens. All matrix products use
// v_mfma_f32_32x32x16_bf16 in the transposed-output form of the forward: the
// lane's resident row (a key in dk/dv, a query in dq) is the B-operand
// column, and the streamed tile's rows are A-operand rows read from LDS either
// directly (128-bit reads) or transposed (ds_read_b64_tr_b16).
//
// Streamed tiles hold row r = item key_of_row(r) of the tile (the order that
// makes a lane's 16 accumulator values 16 consecutive items), with the 16-byte
// chunks of row r XOR-swizzled by ((r & 3) << 2) | ((r >> 2) & 3): with 64
// banks this keeps both the direct reads (16 consecutive rows, one chunk) and
// the transposing reads (4 consecutive rows, 4 consecutive chunks) free of
// bank conflicts.
#pragma once

#include "attn_bf16.hpp"

namespace mra {

struct BwdArgs {
  Args a;                  // forward arguments; a.kp = K', a.cs = (cos, sin) table
  const void* dout;        // dO, strides ds0..2 (batch, token, head)
  int64_t ds0, ds1, ds2;
  void* dq;                // strides of q
  void* dk;                // strides of k
  void* dv;                // strides of v
  const uint16_t* qp;      // Q'' [B, H, S, D]
  float* ld;               // per row (l2, D) [B, H, S, 2]: l2 = lse * log2 e for valid
                           // rows, +inf otherwise; D = sum_d dO O (0 for invalid rows)
  float* dgq_part;         // [n_wg_q, D] per-workgroup gamma_q partials
  float* dgk_part;         // [n_wg_k, D]
  float* dgq;              // [D] or null
  float* dgk;              // [D] or null
  int32_t n_t;             // 128-row tiles per (batch, head)
  int32_t nxcd;            // XCDs of the device
};

__device__ __forceinline__ int bwd_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// byte offset of logical chunk c of row r in a 32 x 128 bf16 streamed tile
__device__ __forceinline__ int bwd_off(int r, int c) { return r * 256 + ((c ^ bwd_swz(r)) << 4); }
// tile row holding item k (inverse of key_of_row)
__device__ __forceinline__ int row_of_item(int k) {
  return (k & ~31) | (((k >> 4) & 1) << 2) | (((k >> 2) & 3) << 3) | (k & 3);
}

// D_i = sum_d dO_id O_id and l2_i for every (batch, token, head) row: 16 lanes
// per row, 8 dims each.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs g) {
  const Args& a = g.a;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;  // (b * S + s) * H + h
  const int sub = threadIdx.x & 15;
  if (row >= (int64_t)a.B * a.S * a.H) return;
  const int h = (int)(row % a.H);
  const int64_t bs = row / a.H;
  const int s = (int)(bs % a.S), b = (int)(bs / a.S);
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), a.T) : a.T;
  const bool valid = !(s >= L && s < a.T);
  const u32x4 wo = *(const u32x4*)((const uint16_t*)a.out + b * a.os0 + (int64_t)s * a.os1 + h * a.os2 + sub * 8);
  const u32x4 wd = *(const u32x4*)((const uint16_t*)g.dout + b * g.ds0 + (int64_t)s * g.ds1 + h * g.ds2 + sub * 8);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc += bf16_lo(wo[e]) * bf16_lo(wd[e]) + bf16_hi(wo[e]) * bf16_hi(wd[e]);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o, 16);
  if (sub == 0) {
    const int64_t i = ((int64_t)b * a.H + h) * a.S + s;
    g.ld[2 * i] = valid ? a.lse[i] * kLog2e : INFINITY;
    g.ld[2 * i + 1] = valid ? acc : 0.f;
  }
}

// Transpose rotation and RMSNorm backward of one row whose gradient w.r.t.
// the rotated, normalised row is held transposed across a lane pair: lane
// (m, hf) holds dims db*32 + (r/4)*8 + hf*4 + r%4 (r < 16, db < D/32) in
// acc[db][r], scaled by `mult`. Rotary partners sit in the same lane: j and
// j + D/2 in db and db + D/64, or (inter) 2j and 2j + 1 in r and r + 1.
// Writes the bf16 input gradient of the row to dst (if in_seq; zeros for an
// invalid row) and returns this lane's gamma gradient contributions in dg
// (zero for an invalid row). INTER is a template parameter: a runtime choice
// keeps both rotations' values live and the dK/dV kernel spills.
template <int D, bool INTER>
__device__ __forceinline__ void rope_rms_bwd(const f32x16 (&acc)[D / 32], float mult,
                                             const uint16_t* xrow, const float* gamma,
                                             const float2* csrow, float eps, bool valid,
                                             bool in_seq, uint16_t* dst, int hf,
                                             float (&dg)[D / 32][16]) {
  constexpr int DB = D / 32, HB = DB / 2;
  float dx[DB][16], x[DB][16];
  if constexpr (INTER) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        // dims d0 .. d0 + 3 are pairs d0/2 and d0/2 + 1
        const f32x4 c01 = *(const f32x4*)(csrow + (db * 32 + gq * 8 + hf * 4) / 2);
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const float cs = c01[e], sn = c01[e + 1];
          const float d1 = acc[db][gq * 4 + e] * mult, d2 = acc[db][gq * 4 + e + 1] * mult;
          dx[db][gq * 4 + e] = d1 * cs + d2 * sn;
          dx[db][gq * 4 + e + 1] = d2 * cs - d1 * sn;
        }
      }
  } else
#pragma unroll
  for (int db = 0; db < HB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int j0 = db * 32 + gq * 8 + hf * 4;
      const f32x4 c01 = *(const f32x4*)(csrow + j0);
      const f32x4 c23 = *(const f32x4*)(csrow + j0 + 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float cs = e < 2 ? c01[2 * e] : c23[2 * (e - 2)];
        const float sn = e < 2 ? c01[2 * e + 1] : c23[2 * (e - 2) + 1];
        const float d1 = acc[db][gq * 4 + e] * mult, d2 = acc[db + HB][gq * 4 + e] * mult;
        dx[db][gq * 4 + e] = d1 * cs + d2 * sn;
        dx[db + HB][gq * 4 + e] = d2 * cs - d1 * sn;
      }
    }
  // gamma is re-read where it is used (cached) rather than held in registers
  float ss = 0.f, inner = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = db * 32 + gq * 8 + hf * 4;
      const u32x2 w = *(const u32x2*)(xrow + d0);
      const f32x4 gv = *(const f32x4*)(gamma + d0);
      x[db][gq * 4 + 0] = bf16_lo(w[0]);
      x[db][gq * 4 + 1] = bf16_hi(w[0]);
      x[db][gq * 4 + 2] = bf16_lo(w[1]);
      x[db][gq * 4 + 3] = bf16_hi(w[1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xe = x[db][gq * 4 + e];
        ss += xe * xe;
        inner += dx[db][gq * 4 + e] * gv[e] * xe;
      }
    }
  ss = half_swap_sum(ss);
  inner = half_swap_sum(inner);
  const float r = rsqrtf(ss * (1.0f / D) + eps);
  const float c3 = r * r * r * (1.0f / D) * inner;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 gv = *(const f32x4*)(gamma + db * 32 + gq * 8 + hf * 4);
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = gq * 4 + e;
        y[e] = r * gv[e] * dx[db][i] - c3 * x[db][i];
        dg[db][i] = valid ? dx[db][i] * x[db][i] * r : 0.f;
      }
      if (in_seq) {
        const uint32_t w0 = valid ? pack_bf16(y[0], y[1]) : 0u;
        const uint32_t w1 = valid ? pack_bf16(y[2], y[3]) : 0u;
        *(u32x2*)(dst + db * 32 + gq * 8 + hf * 4) = u32x2{w0, w1};
      }
    }
}

// Fixed-order workgroup sum of the lanes' gamma contributions (lanes of a
// half-wave hold the same dims), written as this workgroup's partial [D].
template <int D>
__device__ __forceinline__ void dgamma_partial(float (&dg)[D / 32][16], float* red, float* part,
                                               int wave, int lane) {
  constexpr int DB = D / 32;
  const int hf = lane >> 5;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = dg[db][i];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o, 32);
      dg[db][i] = v;
    }
  if ((lane & 31) == 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[wave * D + db * 32 + (i >> 2) * 8 + hf * 4 + (i & 3)] = dg[db][i];
  }
  __syncthreads();
  if ((int)threadIdx.x < D) {
    const int d = threadIdx.x;
    part[d] = ((red[d] + red[D + d]) + red[2 * D + d]) + red[3 * D + d];
  }
}

// LDS of a dK or dV workgroup: stage p holds Q'' (q[p]), dO (o[p]) and the
// (l2, D) pairs (l[p]) of one query tile, each its own object so that a
// stage's reads never wait on another stage's loads; vk holds the V rows of
// the workgroup's 128 keys (row = key, chunk c at c ^ (row & 15)), read back
// as B operands each tile instead of held in registers (dK only); red is the
// gamma reduction's buffer.
struct DkdvLds {
  char* q[2];
  char* o[2];
  float* l[2];
  char* vk;
  float* red;
};

// dV (MODE 1) or dK (MODE 2) of workgroup `tile`: (batch, head, 128 keys),
// 32 keys per wave; query tiles of 32 stream through two LDS stages (one
// tile in flight ahead). Each role recomputes S, which keeps it within two
// waves per SIMD. INTER: interleaved rotary pairs (2j, 2j + 1) in the
// epilogue's inverse rotation.
template <int D, bool INTER, int MODE>
__device__ __forceinline__ void bwd_dkdv_body(const BwdArgs& g, const int tile, const DkdvLds& sm) {
  constexpr int KC = D / 16, DB = D / 32, BQ = 32, TILEB = BQ * D * 2;
  constexpr int RUNS = TILEB / 1024 / 4;
  constexpr bool DO_DV = MODE == 1, DO_DK = MODE == 2;
  constexpr int NST = 2;  // pipeline stages: one query tile in flight
  constexpr int LOADS = 2 * RUNS + 1;  // direct loads per wave per tile
  static_assert(MODE == 1 || MODE == 2, "dV or dK");
  static_assert(D == 128, "the backward kernels are written for head_dim 128");
  char* const Vk = sm.vk;
  float* const red = sm.red;
  auto qb = [&](auto par) -> char* { return sm.q[decltype(par)::value]; };
  auto ob = [&](auto par) -> char* { return sm.o[decltype(par)::value]; };
  auto lb = [&](auto par) -> float* { return sm.l[decltype(par)::value]; };

  const Args& a = g.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m = lane & 31, hf = lane >> 5;
  const int kt = tile % g.n_t, bh = tile / g.n_t;
  const int head = bh % a.H, b = bh / a.H;
  // item b: S tokens from token tok0 of slice bl (packed sequences: one
  // slice of Ss tokens); token indices below are the item's own
  const SeqView sv = seq_view(a, b);
  const int S = sv.S, T = a.T, Ss = a.S, bl = sv.bl;
  const int64_t tok0 = sv.tok0;
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), T) : T;
  auto tok_ok = [&](int n) { return n < S && !(n >= L && n < T); };
  const int key = kt * 128 + wave * 32 + m;
  const bool kvalid = tok_ok(key), kin = key < S;
  // slice row of this lane's key, clamped into the slice (keys past the
  // item's end read some row of it and are then zeroed or not written)
  const int64_t kg = min(tok0 + max(min(key, S - 1), 0), (int64_t)Ss - 1);

  // this lane's key row of K' as B operands (dims c*16 + hf*8 + e); its V
  // row goes to LDS in the same chunk order
  bf16x8 kf[KC];
  char* vrow = Vk + (wave * 32 + m) * (D * 2);
  {
    const uint16_t* kr = a.kp + (((int64_t)bl * a.H + head) * Ss + kg) * D;
    const uint16_t* vr = (const uint16_t*)a.v + bl * a.vs0 + kg * a.vs1 + head * a.vs2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 wk = *(const u32x4*)(kr + c * 16 + hf * 8);
      const u32x4 wv = *(const u32x4*)(vr + c * 16 + hf * 8);
      const u32x4 z = {0u, 0u, 0u, 0u};
      kf[c] = __builtin_bit_cast(bf16x8, kvalid ? wk : z);
      if constexpr (DO_DK) *(u32x4*)(vrow + (((2 * c + hf) ^ (m & 15)) << 4)) = kvalid ? wv : z;
    }
  }

  // streamed tiles: run j of this wave fills LDS bytes [(wave*RUNS+j)*1024,
  // +1024) = rows 4*(wave*RUNS+j) + L/16, physical chunk L%16; every wave also
  // loads the tile's 32 (l2, D) pairs (lane L: float L), the same 256 bytes
  // every stream covers the item's S rows only: rows past them read zeros
  const uint16_t* qbase = g.qp + (((int64_t)bl * a.H + head) * Ss + tok0) * D;
  const uint32_t qnrec = (uint32_t)((int64_t)S * D * 2);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, qnrec);
  const uint16_t* obase = (const uint16_t*)g.dout + bl * g.ds0 + tok0 * g.ds1 + head * g.ds2;
  const uint32_t onrec = S > 0 ? (uint32_t)(((int64_t)(S - 1) * g.ds1 + D) * 2) : 0u;
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(obase, onrec);
  const float* ldbase = g.ld + (((int64_t)bl * a.H + head) * Ss + tok0) * 2;
  const uint32_t lnrec = (uint32_t)((int64_t)S * 2 * 4);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(ldbase, lnrec);
  int t_item[RUNS], q_src[RUNS], o_src[RUNS];
#pragma unroll
  for (int j = 0; j < RUNS; ++j) {
    const int rr = (wave * RUNS + j) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ bwd_swz(rr);
    t_item[j] = key_of_row(rr);
    q_src[j] = (t_item[j] * D + c * 8) * 2;
    o_src[j] = (int)(((int64_t)t_item[j] * g.ds1 + c * 8) * 2);
  }
  auto issue = [&](int qt, auto par) {
    const int n0 = qt * BQ;
    char* qd = qb(par);
    char* od = ob(par);
#pragma unroll
    for (int j = 0; j < RUNS; ++j) {
      const bool ok = tok_ok(n0 + t_item[j]);
      const uint32_t oq = ok ? (uint32_t)(q_src[j] + n0 * D * 2) : qnrec;
      const uint32_t oo = ok ? (uint32_t)(o_src[j] + (int64_t)n0 * g.ds1 * 2) : onrec;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_ptr_t)(qd + (wave * RUNS + j) * 1024), 16, oq, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, (lds_ptr_t)(od + (wave * RUNS + j) * 1024), 16, oo, 0, 0, 0);
    }
    // rows past the end read as (0, 0): their Q'' and dO rows are zero too,
    // so they add nothing
    __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (lds_ptr_t)lb(par), 4, (uint32_t)((n0 * 2 + lane) * 4), 0, 0, 0);
  };
  // wait until at most n tiles' loads of this wave are in flight
  auto wait_tiles = [&](int n) {
    if (n >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * LOADS));
    else if (n == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  static_assert(2 * LOADS < 16, "vmcnt immediates");

  const int nq = (S + BQ - 1) / BQ;
  auto skipped = [&](int qt) { const int n0 = qt * BQ; return n0 >= L && min(n0 + BQ, S) <= T; };
  auto next_q = [&](int qt) { ++qt; while (qt < nq && skipped(qt)) ++qt; return qt; };

  f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dvacc[db][i] = 0.f; dkacc[db][i] = 0.f; }

  // transposing-read roles, as in the forward's P.V
  const int vg = lane >> 4, vj = lane & 15;
  const int t_key0 = (vg >> 1) * 16 + (vj >> 2);
  const int t_dim0 = 16 * (vg & 1) + 4 * (vj & 3);

  // a workgroup whose 128 keys are all padding or past the item's end has
  // zero dk and dv
  const int k0 = kt * 128;
  const bool all_pad = (k0 >= L && min(k0 + 128, S) <= T) || k0 >= S;
  int qt = 0;
  while (qt < nq && skipped(qt)) ++qt;
  if (all_pad) qt = nq;
  // prologue: the first tile into stage 0
  int last = qt, ahead = 0;  // last tile issued; tiles issued after qt
  if (qt < nq) issue(qt, Parity<0>{});

  // tile qt sits in stage `parity`; the tile issued here goes to the stage
  // the previous tile used
  auto step = [&](auto parity) {
    constexpr int cur = decltype(parity)::value;
    wait_tiles(ahead);
    __syncthreads();
    const int tn = last < nq ? next_q(last) : nq;
    if (tn < nq) { issue(tn, Parity<(cur + NST - 1) % NST>{}); last = tn; ++ahead; }
    const char* qs = qb(parity);
    const char* os = ob(parity);
    const float* ls = lb(parity);
    // S2 (queries x keys) = Q'' K'^T; element i of this lane <-> query hf*16 + i
    f32x16 sacc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qs + bwd_off(m, 2 * c + hf)), kf[c],
                                                      sacc, 0, 0, 0);
    // (l2, D) of the lane's 16 queries
    f32x4 ldv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ldv[e] = *(const f32x4*)(ls + hf * 32 + e * 4);
    __builtin_amdgcn_sched_barrier(0);  // phases in order: bounds the live fragments
    // P rounded once to bf16: the operand of dV and the factor of dS
    bf16x8 pf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      pf[i >> 3][i & 7] = (__bf16)__builtin_amdgcn_exp2f(sacc[i] - ldv[i >> 1][(i & 1) * 2]);
    __builtin_amdgcn_sched_barrier(0);
    // dV^T += dO^T P
    if constexpr (DO_DV) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int it = u * 8 + t_key0, dim = db * 32 + t_dim0;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(os + bwd_off(row_of_item(it), dim >> 3) + (dim & 7) * 2));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(os + bwd_off(row_of_item(it + 4), dim >> 3) + (dim & 7) * 2));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
        dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[u], dvacc[db], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DO_DK) {
    // dP (queries x keys) = dO V^T
    f32x16 dpacc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c)
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *(const bf16x8*)(os + bwd_off(m, 2 * c + hf)),
          *(const bf16x8*)(vrow + (((2 * c + hf) ^ (m & 15)) << 4)), dpacc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 dsf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dsf[i >> 3][i & 7] = (__bf16)((float)pf[i >> 3][i & 7] * (dpacc[i] - ldv[i >> 1][(i & 1) * 2 + 1]));
    __builtin_amdgcn_sched_barrier(0);
    // dK'^T += Q''^T dS
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int it = u * 8 + t_key0, dim = db * 32 + t_dim0;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(qs + bwd_off(row_of_item(it), dim >> 3) + (dim & 7) * 2));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(qs + bwd_off(row_of_item(it + 4), dim >> 3) + (dim & 7) * 2));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
        dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dsf[u], dkacc[db], 0, 0, 0);
      }
    }
    qt = next_q(qt);
    --ahead;
  };
  while (qt < nq) {
    step(Parity<0>{});
    if (qt >= nq) break;
    step(Parity<1>{});
  }

  // dV rows: dims db*32 + (i/4)*8 + hf*4 + i%4 of key `key`
  if (DO_DV && kin) {
    uint16_t* dvp = (uint16_t*)g.dv + bl * a.vs0 + (tok0 + key) * a.vs1 + head * a.vs2;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const uint32_t w0 = kvalid ? pack_bf16(dvacc[db][gq * 4], dvacc[db][gq * 4 + 1]) : 0u;
        const uint32_t w1 = kvalid ? pack_bf16(dvacc[db][gq * 4 + 2], dvacc[db][gq * 4 + 3]) : 0u;
        *(u32x2*)(dvp + db * 32 + gq * 8 + hf * 4) = u32x2{w0, w1};
      }
  }
  if constexpr (!DO_DK) return;
  // dK' = ln2 * Q''-accumulator, then the transpose rotation and RMSNorm backward
  float dg[DB][16];
  {
    const uint16_t* xrow = (const uint16_t*)a.k + bl * a.ks0 + kg * a.ks1 + head * a.ks2;
    const float2* csrow = a.cs + ((int64_t)bl * Ss + kg) * (D / 2);
    uint16_t* dst = (uint16_t*)g.dk + bl * a.ks0 + kg * a.ks1 + head * a.ks2;
    rope_rms_bwd<D, INTER>(dkacc, kLn2, xrow, a.gk + head * a.gqs, csrow, a.eps, kvalid, kin, dst,
                           hf, dg);
  }
  dgamma_partial<D>(dg, red, g.dgk_part + (int64_t)tile * D, wave, lane);
}

// LDS of a dQ workgroup: K' (k[p]) and V (v[p]) of key tile stage p, the
// gamma reduction's buffer.
struct DqLds {
  char* k[2];
  char* v[2];
  float* red;
};

// dQ of workgroup `tile`: (batch, head, 128 queries), 32 per wave; key tiles
// of 32 (K' and V) stream through double-buffered LDS. INTER as for dK/dV.
template <int D, bool INTER>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& g, const int tile, const DqLds& sm) {
  constexpr int KC = D / 16, DB = D / 32, BK = 32, TILEB = BK * D * 2;
  constexpr int RUNS = TILEB / 1024 / 4;
  static_assert(D == 128, "the backward kernels are written for head_dim 128");
  char* const K0 = sm.k[0];
  char* const K1 = sm.k[1];
  char* const V0 = sm.v[0];
  char* const V1 = sm.v[1];
  float* const red = sm.red;

  const Args& a = g.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m = lane & 31, hf = lane >> 5;
  const int qtile = tile % g.n_t, bh = tile / g.n_t;
  const int head = bh % a.H, b = bh / a.H;
  // item b: S tokens from token tok0 of slice bl, as in the dK/dV kernel
  const SeqView sv = seq_view(a, b);
  const int S = sv.S, T = a.T, Ss = a.S, bl = sv.bl;
  const int64_t tok0 = sv.tok0;
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), T) : T;
  auto tok_ok = [&](int n) { return n < S && !(n >= L && n < T); };
  const int qrow = qtile * 128 + wave * 32 + m;
  const bool qvalid = tok_ok(qrow), qin = qrow < S;
  const int64_t qg = min(tok0 + max(min(qrow, S - 1), 0), (int64_t)Ss - 1);

  // this lane's query row of Q'' and dO as B operands
  bf16x8 qf[KC], dof[KC];
  {
    const uint16_t* qr = g.qp + (((int64_t)bl * a.H + head) * Ss + qg) * D;
    const uint16_t* dr = (const uint16_t*)g.dout + bl * g.ds0 + qg * g.ds1 + head * g.ds2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 wq = *(const u32x4*)(qr + c * 16 + hf * 8);
      const u32x4 wd = *(const u32x4*)(dr + c * 16 + hf * 8);
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[c] = __builtin_bit_cast(bf16x8, qvalid ? wq : z);
      dof[c] = __builtin_bit_cast(bf16x8, qvalid ? wd : z);
    }
  }
  const int64_t rowi = ((int64_t)bl * a.H + head) * Ss + qg;
  const float l2v = qvalid ? g.ld[2 * rowi] : INFINITY;
  const float dl = qvalid ? g.ld[2 * rowi + 1] : 0.f;

  const uint16_t* kbase = a.kp + (((int64_t)bl * a.H + head) * Ss + tok0) * D;
  const uint32_t knrec = (uint32_t)((int64_t)S * D * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, knrec);
  const uint16_t* vbase = (const uint16_t*)a.v + bl * a.vs0 + tok0 * a.vs1 + head * a.vs2;
  const uint32_t vnrec = S > 0 ? (uint32_t)(((int64_t)(S - 1) * a.vs1 + D) * 2) : 0u;
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, vnrec);
  int t_item[RUNS], k_src[RUNS], v_src[RUNS];
#pragma unroll
  for (int j = 0; j < RUNS; ++j) {
    const int rr = (wave * RUNS + j) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ bwd_swz(rr);
    t_item[j] = key_of_row(rr);
    k_src[j] = (t_item[j] * D + c * 8) * 2;
    v_src[j] = (int)(((int64_t)t_item[j] * a.vs1 + c * 8) * 2);
  }
  auto issue = [&](int kt, int buf) {
    const int n0 = kt * BK;
    char* kd = buf ? K1 : K0;
    char* vd = buf ? V1 : V0;
#pragma unroll
    for (int j = 0; j < RUNS; ++j) {
      const bool ok = tok_ok(n0 + t_item[j]);
      const uint32_t ok_ = ok ? (uint32_t)(k_src[j] + n0 * D * 2) : knrec;
      const uint32_t ov = ok ? (uint32_t)(v_src[j] + (int64_t)n0 * a.vs1 * 2) : vnrec;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(kd + (wave * RUNS + j) * 1024), 16, ok_, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(vd + (wave * RUNS + j) * 1024), 16, ov, 0, 0, 0);
    }
  };

  const int nk = (S + BK - 1) / BK;
  auto skipped = [&](int kt) { const int n0 = kt * BK; return n0 >= L && min(n0 + BK, S) <= T; };
  auto next_k = [&](int kt) { ++kt; while (kt < nk && skipped(kt)) ++kt; return kt; };
  auto masked = [&](int n0) { return n0 + BK > S || (L < T && n0 + BK > L && n0 < T); };

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  const int vg = lane >> 4, vj = lane & 15;
  const int t_key0 = (vg >> 1) * 16 + (vj >> 2);
  const int t_dim0 = 16 * (vg & 1) + 4 * (vj & 3);

  // a workgroup whose 128 queries are all padding or past the item's end
  // computes nothing
  const int q0 = qtile * 128;
  const bool all_pad = (q0 >= L && min(q0 + 128, S) <= T) || q0 >= S;
  int kt = 0;
  while (kt < nk && skipped(kt)) ++kt;
  if (all_pad) kt = nk;
  if (kt < nk) issue(kt, 0);

  auto step = [&](auto parity) {
    constexpr int cur = decltype(parity)::value;
    const int kn = next_k(kt);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kn < nk) issue(kn, cur ^ 1);
    const char* ks = cur ? K1 : K0;
    const char* vs = cur ? V1 : V0;
    const int n0 = kt * BK;
    // S2^T (keys x queries) = K' Q''^T; element i of this lane <-> key hf*16 + i
    f32x16 sacc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(ks + bwd_off(m, 2 * c + hf)), qf[c],
                                                      sacc, 0, 0, 0);
    // dP^T (keys x queries) = V dO^T
    f32x16 dpacc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c)
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vs + bwd_off(m, 2 * c + hf)), dof[c],
                                                       dpacc, 0, 0, 0);
    const bool msk = masked(n0);
    bf16x8 dsf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = !msk || tok_ok(n0 + hf * 16 + i);
      const float p = ok ? __builtin_amdgcn_exp2f(sacc[i] - l2v) : 0.f;
      dsf[i >> 3][i & 7] = (__bf16)(p * (dpacc[i] - dl));
    }
    // dQ'^T += K'^T dS^T
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int it = u * 8 + t_key0, dim = db * 32 + t_dim0;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(ks + bwd_off(row_of_item(it), dim >> 3) + (dim & 7) * 2));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(ks + bwd_off(row_of_item(it + 4), dim >> 3) + (dim & 7) * 2));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dsf[u], dqacc[db], 0, 0, 0);
      }
    kt = kn;
  };
  while (kt < nk) {
    step(Parity<0>{});
    if (kt >= nk) break;
    step(Parity<1>{});
  }

  float dg[DB][16];
  {
    const uint16_t* xrow = (const uint16_t*)a.q + bl * a.qs0 + qg * a.qs1 + head * a.qs2;
    const float2* csrow = a.cs + ((int64_t)bl * Ss + qg) * (D / 2);
    uint16_t* dst = (uint16_t*)g.dq + bl * a.qs0 + qg * a.qs1 + head * a.qs2;
    rope_rms_bwd<D, INTER>(dqacc, a.scale, xrow, a.gq + head * a.gqs, csrow, a.eps, qvalid, qin, dst,
                           hf, dg);
  }
  dgamma_partial<D>(dg, red, g.dgq_part + (int64_t)tile * D, wave, lane);
}

// dK, dQ and dV in one launch: the three are independent, and one grid of
// 3 x n_wg workgroups leaves one partial round of workgroups at its end where
// three launches of n_wg leave one each. Workgroup i runs on XCD i % nxcd
// (the dispatcher's round robin); XCD x takes, in order, its contiguous share
// of the dK tiles, then of the dQ tiles, then of the dV tiles (the lightest
// role last), each share ceil(n_wg / nxcd) tiles (the grid is 3 x nxcd x
// that; workgroups past the last tile exit). The roles share one set of LDS objects, so the
// kernel needs the largest role's LDS, not their sum.
template <int D, bool INTER>
__global__ __launch_bounds__(256, 2) void bwd_fused_kernel(BwdArgs g) {
  constexpr int TILEB = 32 * D * 2;
  __shared__ __attribute__((aligned(1024))) char B0[TILEB];
  __shared__ __attribute__((aligned(1024))) char B1[TILEB];
  __shared__ __attribute__((aligned(1024))) char B2[TILEB];
  __shared__ __attribute__((aligned(1024))) char B3[TILEB];
  __shared__ __attribute__((aligned(256))) float L0[64];
  __shared__ __attribute__((aligned(256))) float L1[64];
  __shared__ __attribute__((aligned(1024))) char Vk[128 * D * 2];
  __shared__ float red[4 * D];
  const int n_wg = g.a.B * g.a.H * g.n_t, nx = g.nxcd;
  const int per = (n_wg + nx - 1) / nx;
  const int x = blockIdx.x % nx, j = blockIdx.x / nx;
  const int role = j / per, tile = x * per + j % per;
  if (tile >= n_wg) return;
  if (role == 1) {
    const DqLds sm{{B0, B1}, {B2, B3}, red};
    bwd_dq_body<D, INTER>(g, tile, sm);
  } else {
    const DkdvLds sm{{B0, B1}, {B2, B3}, {L0, L1}, Vk, red};
    if (role == 0) bwd_dkdv_body<D, INTER, 2>(g, tile, sm);
    else bwd_dkdv_body<D, INTER, 1>(g, tile, sm);
  }
}

// gamma gradient = sum of the workgroup partials in a fixed order. The
// partials of tile (b, h, t) sit at row (b * H + h) * n_t + t. Workgroup
// (which, h, chunk) -- which 0: gamma_q, 1: gamma_k -- sums dims
// [chunk * DC, chunk * DC + DC) of the n partials of its gradient row h:
// partial i < n is row (i / run) * stride + h * run + i % run (a shared [D]
// gamma: one row, run = n = every tile, stride 0; an [H, D] gamma: row h,
// run = n_t, stride = H * n_t, n = B * n_t). Thread (grp, d) of G x DC sums
// partials grp, grp + G, ... with four interleaved accumulators, then the
// G x 4 sums are added in a fixed order.
template <int D>
__global__ __launch_bounds__(1024) void bwd_dgamma_kernel(const float* part_q, const float* part_k, int n,
                                                          int run, int64_t stride, float* out_q,
                                                          float* out_k) {
  constexpr int DC = 32, G = 1024 / DC, NC = D / DC;
  static_assert(D % DC == 0, "head_dim is a multiple of the dim chunk");
  __shared__ float red[G][DC];
  const int chunk = blockIdx.x % NC, rest = blockIdx.x / NC;
  const int which = rest & 1, h = rest >> 1;
  const float* part = (which ? part_k : part_q) + (int64_t)h * run * D;
  float* out = which ? out_k : out_q;
  if (!out) return;
  out += (int64_t)h * D;
  const int d = chunk * DC + threadIdx.x % DC, grp = threadIdx.x / DC;
  // a shared gamma sums every partial in order (run == n: no division)
  auto at = [&](int i) {
    const int64_t r = run == n ? i : (int64_t)(i / run) * stride + i % run;
    return part[r * D + d];
  };
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int i = grp;
  for (; i + 3 * G < n; i += 4 * G) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += at(i + G * u);
  }
  for (int u = 0; i < n; i += G, ++u) acc[u & 3] += at(i);
  red[grp][threadIdx.x % DC] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (grp == 0) {
    float t = 0.f;
#pragma unroll 8
    for (int g = 0; g < G; ++g) t += red[g][threadIdx.x];
    out[d] = t;
  }
}

}  // namespace mra
