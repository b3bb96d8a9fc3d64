// Host side of the backward entry points (mrope_attn_bwd, its packed
// variable-length form mrope_attn_bwd_varlen, and their workspace queries).
// Included once, at the end of mrope_attn.hip, whose helpers it uses; kept in
// its own file so the forward path's sources stand alone.
#pragma once

extern "C" {

// ---- backward pass ---------------------------------------------------------
// Workspace: (cos, sin) table [B, S, D/2] float2, K' and Q'' [B, H, S, D] bf16,
// (l2, D) pairs [B, H, S, 2] fp32, then the gamma partials of the dq and dk/dv
// workgroups [n_wg, D] fp32 each; every piece 256-byte aligned. B and S are
// the tensor layout's (one slice of every token for packed sequences); the
// workgroups cover nseq items of at most maxlen tokens, 128 per tile.
struct BwdPlan {
  int n_t, n_wg;
  size_t off_cs, off_kp, off_qp, off_ld, off_gq, off_gk, bytes;
};

static BwdPlan bwd_plan(const mra_desc* d, int nseq, int maxlen) {
  BwdPlan p;
  const size_t rows = (size_t)d->batch * d->seq * d->heads;
  p.n_t = (maxlen + 127) / 128;
  p.n_wg = nseq * d->heads * p.n_t;
  size_t off = 0;
  p.off_cs = off; off += table_bytes(d);
  p.off_kp = off; off += round_up(rows * d->head_dim * 2, kWsAlign);
  p.off_qp = off; off += round_up(rows * d->head_dim * 2, kWsAlign);
  p.off_ld = off; off += round_up(rows * 8, kWsAlign);
  p.off_gq = off; off += round_up((size_t)p.n_wg * d->head_dim * 4, kWsAlign);
  p.off_gk = off; off += round_up((size_t)p.n_wg * d->head_dim * 4, kWsAlign);
  p.bytes = off;
  return p;
}

static int bwd_check(const mra_desc* d) {
  int rc = check_desc(d);
  if (rc != MRA_OK) return rc;
  if (d->dtype != MRA_BF16 || d->head_dim != 128) return MRA_ERR_UNSUPPORTED;
  if (d->kprologue == MRA_KPRO_NONE || d->kprologue == MRA_KPRO_GIVEN) return MRA_ERR_UNSUPPORTED;
  return MRA_OK;
}

static int bwd_pointers(const void* out, const float* lse, const void* dout, void* dq, void* dk,
                        void* dv, const float* dgq, const float* dgk) {
  if (!out || !lse || !dout || !dq || !dk || !dv) return MRA_ERR_NULL;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16)) return MRA_ERR_STRIDE;
  if (!aligned(lse, 4) || !aligned(dgq, 4) || !aligned(dgk, 4)) return MRA_ERR_STRIDE;
  return MRA_OK;
}

// Launches the backward over layout d (validated) for nseq items of at most
// maxlen tokens: per-item views come from seq_lens (padded layout) or
// cu_seqlens (packed layout, d->batch == 1).
static int bwd_run(const mra_desc* d, int nseq, int maxlen, const int32_t* seq_lens,
                   const int32_t* cu_seqlens, const void* q, const void* k, const void* v,
                   const int32_t* pos, const float* gq, const float* gk, const void* out,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dgamma_q,
                   float* dgamma_k, void* workspace, hipStream_t s) {
  const BwdPlan p = bwd_plan(d, nseq, maxlen);
  char* w = (char*)workspace;
  mra::BwdArgs g;
  std::memset(&g, 0, sizeof(g));
  fill_args(g.a, d, q, k, v, pos, gq, gk, seq_lens, (void*)out, (float*)lse);
  g.a.cs = (float2*)(w + p.off_cs);
  g.a.kp = (uint16_t*)(w + p.off_kp);
  g.dout = dout;
  g.ds0 = d->o_stride[0]; g.ds1 = d->o_stride[1]; g.ds2 = d->o_stride[2];
  g.dq = dq; g.dk = dk; g.dv = dv;
  g.qp = (const uint16_t*)(w + p.off_qp);
  g.ld = (float*)(w + p.off_ld);
  g.dgq_part = (float*)(w + p.off_gq);
  g.dgk_part = (float*)(w + p.off_gk);
  g.dgq = dgamma_q; g.dgk = dgamma_k;
  g.n_t = p.n_t;
  g.nxcd = current_device_shape().xcds;

  // the row-wise passes run over the whole layout (every token of a packed
  // slice): K' and the rotary table, then Q'' = c2 * rope(rmsnorm(q)) (same
  // kernel), then the (l2, D) pairs
  const int64_t tokens = (int64_t)d->batch * d->seq;
  hipLaunchKernelGGL(mra::k_prologue_kernel<128>, dim3((unsigned)((tokens + 3) / 4)), dim3(256), 0, s, g.a);
  Args aq = g.a;
  aq.k = q; aq.ks0 = aq.qs0; aq.ks1 = aq.qs1; aq.ks2 = aq.qs2;
  aq.gk = gq; aq.kp = (uint16_t*)g.qp; aq.cs = nullptr; aq.pscale = aq.c2;
  hipLaunchKernelGGL(mra::k_prologue_kernel<128>, dim3((unsigned)((tokens + 3) / 4)), dim3(256), 0, s, aq);
  const int64_t rows = tokens * d->heads;
  hipLaunchKernelGGL(mra::bwd_delta_kernel<128>, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, s, g);
  // the matrix-core kernels work per item
  g.a.B = nseq;
  g.a.cu_seqlens = cu_seqlens;
  // dK, dQ and dV: one launch of the three roles (3 x nxcd x
  // ceil(n_wg / nxcd) workgroups; see bwd_fused_kernel)
  const unsigned nwg = (unsigned)p.n_wg, nx = (unsigned)g.nxcd;
  const unsigned grid = 3u * nx * ((nwg + nx - 1u) / nx);
  if (g.a.inter) hipLaunchKernelGGL((mra::bwd_fused_kernel<128, true>), dim3(grid), dim3(256), 0, s, g);
  else hipLaunchKernelGGL((mra::bwd_fused_kernel<128, false>), dim3(grid), dim3(256), 0, s, g);
  if (dgamma_q || dgamma_k) {
    // per-tile partials are laid out [nseq, H, n_t, D]: a shared gamma sums
    // all of them, a per-head gamma sums head h's nseq * n_t rows
    const bool ph = d->gamma_per_head;
    const int n = ph ? nseq * p.n_t : p.n_wg;
    const int run = ph ? p.n_t : p.n_wg;
    const int64_t stride = ph ? (int64_t)d->heads * p.n_t : 0;
    hipLaunchKernelGGL(mra::bwd_dgamma_kernel<128>, dim3(2u * (ph ? d->heads : 1) * (128 / 32)), dim3(1024), 0, s,
                       (const float*)g.dgq_part, (const float*)g.dgk_part, n, run, stride, dgamma_q,
                       dgamma_k);
  }
  return hip_status(hipGetLastError());
}

size_t mrope_attn_bwd_workspace_size(const mra_desc* d) {
  if (bwd_check(d) != MRA_OK || d->batch == 0 || d->seq == 0) return 0;
  return bwd_plan(d, d->batch, d->seq).bytes;
}

int mrope_attn_bwd(const mra_desc* d, const void* q, const void* k, const void* v,
                   const int32_t* pos, const float* gq, const float* gk, const int32_t* seq_lens,
                   const void* out, const float* lse, const void* dout, void* dq, void* dk,
                   void* dv, float* dgamma_q, float* dgamma_k, void* workspace, size_t ws_bytes,
                   void* stream) {
  int rc = bwd_check(d);
  if (rc != MRA_OK) return rc;
  rc = mrope_attn_validate(d, q, k, v, pos, gq, gk, seq_lens, out);
  if (rc != MRA_OK) return rc;
  if (d->batch == 0 || d->seq == 0) return MRA_OK;
  rc = bwd_pointers(out, lse, dout, dq, dk, dv, dgamma_q, dgamma_k);
  if (rc != MRA_OK) return rc;
  const BwdPlan p = bwd_plan(d, d->batch, d->seq);
  if (!workspace || ws_bytes < p.bytes || !aligned(workspace, 16)) return MRA_ERR_WORKSPACE;
  const char* fi = std::getenv("MRA_FAULT_INJECT");
  if (fi && std::strcmp(fi, "launch") == 0) return MRA_ERR_HIP;
  clear_stale_hip_error();
  return bwd_run(d, d->batch, d->seq, seq_lens, nullptr, q, k, v, pos, gq, gk, out, lse, dout, dq, dk, dv,
                 dgamma_q, dgamma_k, workspace, (hipStream_t)stream);
}

size_t mrope_attn_bwd_varlen_workspace_size(const mra_desc* d, int32_t max_seqlen) {
  mra_desc lay;
  if (varlen_layout(d, max_seqlen, lay) != MRA_OK || bwd_check(d) != MRA_OK) return 0;
  if (d->batch == 0 || d->seq == 0 || max_seqlen == 0) return 0;
  return bwd_plan(&lay, d->batch, max_seqlen).bytes;
}

int mrope_attn_bwd_varlen(const mra_desc* d, const void* q, const void* k, const void* v,
                          const int32_t* pos, const float* gq, const float* gk,
                          const int32_t* cu_seqlens, int32_t max_seqlen, const void* out,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          float* dgamma_q, float* dgamma_k, void* workspace, size_t ws_bytes,
                          void* stream) {
  mra_desc lay;
  int rc = varlen_layout(d, max_seqlen, lay);
  if (rc != MRA_OK) return rc;
  rc = bwd_check(d);
  if (rc != MRA_OK) return rc;
  if (d->batch == 0 || d->seq == 0 || max_seqlen == 0) return MRA_OK;
  rc = mrope_attn_validate(&lay, q, k, v, pos, gq, gk, nullptr, out);
  if (rc != MRA_OK) return rc;
  if (!cu_seqlens) return MRA_ERR_NULL;
  if (!aligned(cu_seqlens, 4)) return MRA_ERR_STRIDE;
  rc = bwd_pointers(out, lse, dout, dq, dk, dv, dgamma_q, dgamma_k);
  if (rc != MRA_OK) return rc;
  const BwdPlan p = bwd_plan(&lay, d->batch, max_seqlen);
  if (!workspace || ws_bytes < p.bytes || !aligned(workspace, 16)) return MRA_ERR_WORKSPACE;
  const char* fi = std::getenv("MRA_FAULT_INJECT");
  if (fi && std::strcmp(fi, "launch") == 0) return MRA_ERR_HIP;
  clear_stale_hip_error();
  return bwd_run(&lay, d->batch, max_seqlen, nullptr, cu_seqlens, q, k, v, pos, gq, gk, out, lse, dout, dq,
                 dk, dv, dgamma_q, dgamma_k, workspace, (hipStream_t)stream);
}

}  // extern "C"
