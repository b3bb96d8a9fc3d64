// Host side of the fp8 QKV projection entry points (mrope_qkv_proj and its
// workspace query). Included once, at the end of mrope_attn.hip, whose
// helpers it uses; kept in its own file so the forward path's sources stand
// alone.
#pragma once

extern "C" {

// ---- fp8 QKV projection --------------------------------------------------
static int qkv_check(const mra_qkv_desc* d) {
  if (!d) return MRA_ERR_NULL;
  if (d->tokens < 0 || d->heads < 1 || d->hidden <= 0 || d->hidden % 64 != 0) return MRA_ERR_SHAPE;
  if (d->head_dim != 128) return MRA_ERR_UNSUPPORTED;
  if (d->section[0] < 0 || d->section[1] < 0 || d->section[2] < 0 ||
      (int64_t)d->section[0] + d->section[1] + d->section[2] != d->head_dim / 2)
    return MRA_ERR_SECTION;
  if (!(d->theta > 0.f) || !std::isfinite(d->theta)) return MRA_ERR_PARAM;
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps)) return MRA_ERR_PARAM;
  if (!std::isfinite(d->softmax_scale)) return MRA_ERR_PARAM;
  if (d->rope_pairs != MRA_ROPE_HALF && d->rope_pairs != MRA_ROPE_INTERLEAVED) return MRA_ERR_PARAM;
  if (d->gamma_per_head != 0 && d->gamma_per_head != 1) return MRA_ERR_PARAM;
  if (d->x_stride < d->hidden || d->x_stride % 8 != 0) return MRA_ERR_STRIDE;
  const int64_t* st[3] = {d->q_stride, d->k_stride, d->v_stride};
  for (int i = 0; i < 3; ++i)
    if (st[i][0] < 0 || st[i][1] < 0 || st[i][0] % 8 != 0 || st[i][1] % 8 != 0) return MRA_ERR_STRIDE;
  // 32-bit byte offsets inside x and each weight block
  if ((int64_t)d->tokens * d->x_stride * 2 >= ((int64_t)1 << 31)) return MRA_ERR_UNSUPPORTED;
  if ((int64_t)d->head_dim * d->hidden >= ((int64_t)1 << 31)) return MRA_ERR_UNSUPPORTED;
  return MRA_OK;
}

size_t mrope_qkv_proj_workspace_size(const mra_qkv_desc* d) {
  if (qkv_check(d) != MRA_OK || d->tokens == 0) return 0;
  return round_up((size_t)d->tokens * (d->head_dim / 2) * sizeof(float2), kWsAlign);
}

int mrope_qkv_proj(const mra_qkv_desc* d, const void* x, const uint8_t* w8, const float* w_scale,
                   const int32_t* pos, const float* gq, const float* gk, void* q_out, void* k_out,
                   void* v_out, void* workspace, size_t ws_bytes, void* stream) {
  int rc = qkv_check(d);
  if (rc != MRA_OK) return rc;
  if (d->tokens == 0) return MRA_OK;
  if (!x || !w8 || !w_scale || !pos || !gq || !gk || !q_out || !k_out || !v_out) return MRA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w8, 16) || !aligned(w_scale, 16) || !aligned(gq, 16) ||
      !aligned(gk, 16) || !aligned(pos, 4) || !aligned(q_out, 16) || !aligned(k_out, 16) ||
      !aligned(v_out, 16))
    return MRA_ERR_STRIDE;
  const size_t need = mrope_qkv_proj_workspace_size(d);
  if (!workspace || ws_bytes < need || !aligned(workspace, 16)) return MRA_ERR_WORKSPACE;
  const char* fi = std::getenv("MRA_FAULT_INJECT");
  if (fi && std::strcmp(fi, "launch") == 0) return MRA_ERR_HIP;
  clear_stale_hip_error();

  // the rotary table of the tokens, from the same kernel the attention uses
  Args a;
  std::memset(&a, 0, sizeof(a));
  a.pos = pos;
  a.B = 1;
  a.S = d->tokens;
  a.cs = (float2*)workspace;
  const int half = d->head_dim / 2;
  for (int j = 0; j < half; ++j)
    a.rope.inv_freq[j] = (float)std::pow((double)d->theta, -2.0 * j / d->head_dim);
  a.rope.sec_t = d->section[0];
  a.rope.sec_th = d->section[0] + d->section[1];
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = (int64_t)d->tokens * half;
  hipLaunchKernelGGL(mra::rope_table_kernel<128>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);

  mra::QkvArgs g;
  std::memset(&g, 0, sizeof(g));
  g.x = (const uint16_t*)x;
  g.xs = d->x_stride;
  g.w8 = w8;
  g.wsc = w_scale;
  g.cs = (const float2*)workspace;
  g.gq = gq;
  g.gk = gk;
  g.gqs = d->gamma_per_head ? d->head_dim : 0;
  g.inter = d->rope_pairs == MRA_ROPE_INTERLEAVED;
  g.out[0] = (uint16_t*)q_out; g.out[1] = (uint16_t*)k_out; g.out[2] = (uint16_t*)v_out;
  const int64_t* st[3] = {d->q_stride, d->k_stride, d->v_stride};
  for (int i = 0; i < 3; ++i) { g.os[i][0] = st[i][0]; g.os[i][1] = st[i][1]; }
  g.nxcd = current_device_shape().xcds;
  g.M = d->tokens;
  g.hidden = d->hidden;
  g.H = d->heads;
  g.eps = d->eps;
  const float scale = d->softmax_scale > 0.f ? d->softmax_scale : (float)(1.0 / std::sqrt((double)d->head_dim));
  g.qscale = (float)((double)scale * 1.4426950408889634);
  // one workgroup per (token tile, head pair); two workgroups share a CU
  constexpr int kWaves = mra::kQkvWaves, kTok = mra::kQkvTokPerWave * (mra::kQkvWaves / 2);
  const int head_pairs = (3 * d->heads + 1) / 2;
  g.n_mt = (d->tokens + kTok - 1) / kTok;
  hipLaunchKernelGGL((mra::qkv_proj_kernel<128, kWaves, mra::kQkvChunk, mra::kQkvStages, mra::kQkvTokPerWave>),
                     dim3((unsigned)(g.n_mt * head_pairs)), dim3(64 * kWaves), 0, s, g);
  return hip_status(hipGetLastError());
}

}  // extern "C"
