// Host-side walk of every entry point of libmrope_attn, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
// device code is compiled but never launched). With MRA_FAULT_INJECT=launch
// every call stops at the hook right before its first HIP call, so the whole
// host path runs: descriptor and pointer validation, the attention plan and
// workspace layout, group/varlen/backward/projection sizing, status strings.
// Besides the sanitizers' own checks, each call's status is checked against
// the contract: a call fails with the validator's status, or reaches the
// launch hook (MRA_ERR_HIP) when valid, or returns MRA_OK for empty input.
// Exits non-zero on the first violation.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "mrope_attn.h"

namespace {

const uintptr_t kFake = 0x10000;  // aligned, non-null, never dereferenced here
void* P(uintptr_t off = 0) { return (void*)(kFake + off); }

int failures = 0;
void expect(bool ok, const char* what, int line, long long a = 0, long long b = 0) {
  if (!ok) {
    std::fprintf(stderr, "contract violation at line %d: %s (%lld, %lld)\n", line, what, a, b);
    ++failures;
  }
}
#define EXPECT(c, ...) expect((c), #c, __LINE__, ##__VA_ARGS__)

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint32_t rnd() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
int pick(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }

mra_desc make(int b, int s, int h, int d, int text_pad, int dtype = MRA_BF16) {
  mra_desc x;
  std::memset(&x, 0, sizeof(x));
  x.batch = b; x.seq = s; x.heads = h; x.head_dim = d; x.text_pad = text_pad;
  const int half = d / 2, st = half / 4;
  x.section[0] = st; x.section[1] = (half - st) / 2; x.section[2] = half - st - (half - st) / 2;
  x.theta = 10000.f; x.eps = 1e-6f; x.softmax_scale = 0.f; x.dtype = dtype;
  x.kprologue = MRA_KPRO_AUTO;
  const int64_t c[3] = {(int64_t)s * h * d, (int64_t)h * d, d};
  for (int i = 0; i < 3; ++i) x.q_stride[i] = x.k_stride[i] = x.v_stride[i] = x.o_stride[i] = c[i];
  return x;
}

int fwd(const mra_desc& d, size_t ws_bytes, float* lse = nullptr) {
  return mrope_attn_fwd(&d, P(), P(), P(), (const int32_t*)P(), (const float*)P(), (const float*)P(),
                        nullptr, P(), lse, ws_bytes ? P() : nullptr, ws_bytes, nullptr);
}
int validate(const mra_desc& d) {
  return mrope_attn_validate(&d, P(), P(), P(), (const int32_t*)P(), (const float*)P(), (const float*)P(),
                             nullptr, P());
}

// One descriptor through fwd / prepare / attend / noalloc / bwd.
void walk(const mra_desc& d) {
  const int v = validate(d);
  const size_t need = mrope_attn_workspace_size(&d);
  const bool empty = d.batch == 0 || d.seq == 0;
  const int rc = fwd(d, need);
  if (v != MRA_OK) EXPECT(rc == v, rc, v);
  else if (empty) EXPECT(rc == MRA_OK, rc);
  else EXPECT(rc == MRA_ERR_HIP, rc);
  if (v == MRA_OK && !empty && need > 0) {
    EXPECT(fwd(d, need - 1) == MRA_ERR_WORKSPACE);
    EXPECT(need % 256 == 0, (long long)need);
  }
  const int rp = mrope_attn_prepare(&d, P(), (const int32_t*)P(), (const float*)P(), need ? P() : nullptr,
                                    need, nullptr);
  const int ra = mrope_attn_attend(&d, P(), P(), P(), (const int32_t*)P(), (const float*)P(),
                                   (const float*)P(), nullptr, P(), nullptr, need ? P() : nullptr, need, nullptr);
  EXPECT(ra == rc, ra, rc);
  if (v == MRA_OK) EXPECT(rp == (empty ? MRA_OK : MRA_ERR_HIP) || (d.dtype == MRA_FP32 && rp == MRA_ERR_HIP), rp);
  // the no-allocation forward: invalid input and oversize problems are
  // refused before any device call
  if (v != MRA_OK || need > MRA_NOALLOC_SCRATCH_BYTES) {
    const int rn = mrope_attn_fwd_noalloc(&d, P(), P(), P(), (const int32_t*)P(), (const float*)P(),
                                          (const float*)P(), nullptr, P(), nullptr, nullptr);
    EXPECT(rn == (v != MRA_OK ? v : MRA_ERR_SCRATCH), rn, v);
  }
  // backward sizing and host checks
  const size_t bneed = mrope_attn_bwd_workspace_size(&d);
  const int rb = mrope_attn_bwd(&d, P(), P(), P(), (const int32_t*)P(), (const float*)P(), (const float*)P(),
                                nullptr, P(), (const float*)P(), P(), P(), P(), P(), (float*)P(), (float*)P(),
                                bneed ? P() : nullptr, bneed, nullptr);
  if (v == MRA_OK && !empty && d.dtype == MRA_BF16 && d.head_dim == 128 && d.kprologue != MRA_KPRO_NONE &&
      d.kprologue != MRA_KPRO_GIVEN)
    EXPECT(rb == MRA_ERR_HIP && bneed > 0, rb);
  else
    EXPECT(rb != MRA_ERR_HIP || v != MRA_OK, rb);
}

void varlen(const mra_desc& d, int max_seqlen) {
  const size_t need = mrope_attn_varlen_workspace_size(&d, max_seqlen);
  const int rc = mrope_attn_fwd_varlen(&d, P(), P(), P(), (const int32_t*)P(), (const float*)P(),
                                       (const float*)P(), (const int32_t*)P(), max_seqlen, P(), nullptr,
                                       need ? P() : nullptr, need, nullptr);
  EXPECT(rc <= 0, rc);
  const size_t bneed = mrope_attn_bwd_varlen_workspace_size(&d, max_seqlen);
  const int rb = mrope_attn_bwd_varlen(&d, P(), P(), P(), (const int32_t*)P(), (const float*)P(),
                                       (const float*)P(), (const int32_t*)P(), max_seqlen, P(),
                                       (const float*)P(), P(), P(), P(), P(), nullptr, nullptr,
                                       bneed ? P() : nullptr, bneed, nullptr);
  EXPECT(rb <= 0, rb);
  if (d.text_pad != 0 || max_seqlen < 0 || max_seqlen > d.seq) EXPECT(rc == MRA_ERR_SHAPE || rc < 0, rc);
}

void group(const mra_desc* ds, int n) {
  mra_problem probs[MRA_MAX_GROUP + 1];
  for (int i = 0; i < MRA_MAX_GROUP + 1; ++i)
    probs[i] = mra_problem{P(), P(), P(), (const int32_t*)P(), (const float*)P(), (const float*)P(), nullptr,
                           P(1 << 20), nullptr};
  const size_t need = mrope_attn_group_workspace_size(ds, n);
  const int rc = mrope_attn_fwd_group(ds, probs, n, need ? P() : nullptr, need, nullptr);
  EXPECT(rc <= 0, rc);
}

void qkv(int tokens, int hidden, int heads) {
  mra_qkv_desc d;
  std::memset(&d, 0, sizeof(d));
  d.tokens = tokens; d.hidden = hidden; d.heads = heads; d.head_dim = 128;
  d.section[0] = 16; d.section[1] = 24; d.section[2] = 24;
  d.theta = 10000.f; d.eps = 1e-6f; d.x_stride = hidden;
  const int64_t hs = 128, ts = (int64_t)heads * 128;
  d.q_stride[0] = d.k_stride[0] = d.v_stride[0] = ts;
  d.q_stride[1] = d.k_stride[1] = d.v_stride[1] = hs;
  const size_t need = mrope_qkv_proj_workspace_size(&d);
  const int rc = mrope_qkv_proj(&d, P(), (const uint8_t*)P(), (const float*)P(), (const int32_t*)P(),
                                (const float*)P(), (const float*)P(), P(), P(), P(), need ? P() : nullptr, need,
                                nullptr);
  EXPECT(rc <= 0, rc);
}

}  // namespace

int main() {
  setenv("MRA_FAULT_INJECT", "launch", 1);
  EXPECT(mrope_attn_abi_version() >= 100);
  for (int st = 1; st >= -12; --st) EXPECT(mrope_attn_status_string(st) != nullptr);
  const char* name = nullptr;
  EXPECT(mrope_attn_last_hip_error(&name) == 0 && name != nullptr);
  EXPECT(mrope_attn_last_hip_error(nullptr) == 0);
  EXPECT(mrope_attn_workspace_size(nullptr) == 0);
  EXPECT(validate(make(1, 8, 1, 96, 0)) == MRA_ERR_SHAPE);

  // the configurations of the benchmark and tests
  const int shapes[][5] = {{1, 32, 1, 64, 16},      {1, 1280, 24, 128, 256},  {1, 4608, 32, 128, 512},
                           {4, 4608, 32, 128, 512}, {1, 12800, 32, 128, 512}, {1, 4608, 36, 128, 512},
                           {1, 16896, 32, 128, 512}, {1, 4608, 4, 128, 512},  {2, 4608, 32, 128, 512},
                           {0, 100, 2, 128, 0},     {2, 0, 2, 128, 0},        {1, 261632, 32, 128, 512}};
  for (const auto& s : shapes) {
    for (int dt = 0; dt < 2; ++dt)
      for (int kp = 0; kp < 6; ++kp) {  // every mode, then one unknown
        mra_desc d = make(s[0], s[1], s[2], s[3], s[4], dt);
        d.kprologue = kp;
        walk(d);
      }
  }

  // randomized descriptors: shapes, tails, conventions, strides, bad fields
  for (int it = 0; it < 20000; ++it) {
    const int hd = (rnd() % 8 == 0) ? 96 : ((rnd() & 1) ? 64 : 128);
    const int s = pick(0, (rnd() % 4 == 0) ? 40000 : 3000);
    mra_desc d = make(pick(0, 6), s, pick(1, 80), hd, s ? pick(0, s) : 0, (rnd() % 10 == 0) ? 2 : (int)(rnd() & 1));
    d.kprologue = pick(0, 5);
    d.rope_pairs = (rnd() % 20 == 0) ? 2 : (int)(rnd() & 1);
    d.gamma_per_head = (rnd() % 20 == 0) ? 3 : (int)(rnd() & 1);
    if (rnd() % 10 == 0) d.section[0] += 1;
    if (rnd() % 10 == 0) d.theta = (rnd() & 1) ? -1.f : 0.f;
    if (rnd() % 15 == 0) d.eps = -1e-3f;
    if (rnd() % 5 == 0) {  // strided views, e.g. of one fused qkv buffer
      const int64_t tok = (int64_t)d.heads * d.head_dim * 3;
      d.q_stride[1] = d.k_stride[1] = d.v_stride[1] = tok + 8 * pick(-1, 2);
      d.q_stride[0] = d.k_stride[0] = d.v_stride[0] = (int64_t)s * tok;
    }
    if (rnd() % 25 == 0) d.o_stride[2] = -8;
    walk(d);
    mra_desc v = d;
    v.text_pad = (rnd() % 8 == 0) ? 1 : 0;
    varlen(v, pick(-1, d.seq + 1));
    if (it % 4 == 0) {
      mra_desc ds[MRA_MAX_GROUP + 1];
      const int n = pick(0, MRA_MAX_GROUP + 1);
      for (int i = 0; i < MRA_MAX_GROUP + 1; ++i) {
        ds[i] = d;
        ds[i].seq = pick(0, 5000);
        ds[i].text_pad = ds[i].seq ? pick(0, ds[i].seq) : 0;
        for (int k = 0; k < 3; ++k) ds[i].q_stride[k] = ds[i].k_stride[k] = ds[i].v_stride[k] = ds[i].o_stride[k] = 0;
        ds[i].q_stride[0] = ds[i].k_stride[0] = ds[i].v_stride[0] = ds[i].o_stride[0] =
            (int64_t)ds[i].seq * d.heads * d.head_dim;
        ds[i].q_stride[1] = ds[i].k_stride[1] = ds[i].v_stride[1] = ds[i].o_stride[1] = (int64_t)d.heads * d.head_dim;
        ds[i].q_stride[2] = ds[i].k_stride[2] = ds[i].v_stride[2] = ds[i].o_stride[2] = d.head_dim;
      }
      group(ds, n);
    }
    if (it % 8 == 0) qkv(pick(-1, 20000), 64 * pick(0, 80) + ((rnd() % 10 == 0) ? 32 : 0), pick(0, 48));
  }
  if (failures) {
    std::fprintf(stderr, "%d contract violations\n", failures);
    return 1;
  }
  std::printf("abi walk ok\n");
  return 0;
}
