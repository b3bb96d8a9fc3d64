// C ABI of libmrope_attn.so: argument validation, workspace sizing, kernel
// selection and launch on the caller's stream. The operation and the
// conventions are documented in include/mrope_attn.h.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mrope_attn.h"
#include "attn_bf16.hpp"
#include "attn_bwd.hpp"
#include "qkv_proj.hpp"
#include "attn_fp32.hpp"
#include "prologue.hpp"

namespace {

using mra::Args;

constexpr int kBlockN = 64;     // keys per K/V tile
constexpr int kRowBlocks = 1;   // 32-row blocks per wave
constexpr int kFp32BlockM = 64;
constexpr size_t kWsAlign = 256;
// A split part keeps at least this many key tiles (shorter parts lose more to
// their own prologue and the merge than the idle slots they fill).
constexpr int kMinPartKeyTiles = 24;
constexpr int kMaxXcds = 16;

// Compute units and XCDs of a device, for the attention launch plan.
struct DeviceShape {
  int cus, xcds;
};
constexpr DeviceShape kDefaultShape{256, 8};  // MI355X
constexpr int kMaxDevices = 64;

// The current device's shape, queried once per device and cached; the
// MI355X's when no device can be queried (host-only use, e.g. sizing a
// workspace on a machine without a GPU).
DeviceShape current_device_shape() {
  static std::mutex mu;
  static DeviceShape cache[kMaxDevices];
  static bool have[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultShape;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!have[dev]) {
    DeviceShape d = kDefaultShape;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) d.cus = v;
    v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0) d.xcds = v;
    else d.xcds = 1;
    (void)hipGetLastError();
    cache[dev] = d;
    have[dev] = true;
  }
  return cache[dev];
}

// hipError_t behind the calling thread's most recent MRA_ERR_HIP
// (mrope_attn_last_hip_error), 0 if none yet.
thread_local int t_last_hip_error = 0;

// Takes the calling thread's pending HIP error (left by whatever ran before
// this call) off, so that the check after this call's launches sees only
// their own errors.
void clear_stale_hip_error() { (void)hipGetLastError(); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MRA_OK;
  t_last_hip_error = (int)e;
  return MRA_ERR_HIP;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int resolve_kprologue(const mra_desc* d) {
  const int k = d->kprologue == MRA_KPRO_AUTO ? MRA_KPRO_PREPASS : d->kprologue;
  // plain given operands take the same kernels as scaled ones (q scaled on load)
  return k == MRA_KPRO_GIVEN ? MRA_KPRO_NONE : k;
}

// Descriptor-only checks (no pointers).
int check_desc(const mra_desc* d) {
  if (!d) return MRA_ERR_NULL;
  if (d->batch < 0 || d->seq < 0 || d->heads < 1) return MRA_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return MRA_ERR_SHAPE;
  if (d->text_pad < 0 || d->text_pad > d->seq) return MRA_ERR_SHAPE;
  if ((int64_t)d->batch * d->seq > (int64_t)1 << 30) return MRA_ERR_SHAPE;
  if (d->dtype != MRA_BF16 && d->dtype != MRA_FP32) return MRA_ERR_DTYPE;
  const int half = d->head_dim / 2;
  if (d->section[0] < 0 || d->section[1] < 0 || d->section[2] < 0 ||
      (int64_t)d->section[0] + d->section[1] + d->section[2] != half)
    return MRA_ERR_SECTION;
  if (!(d->theta > 0.f) || !std::isfinite(d->theta)) return MRA_ERR_PARAM;
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps)) return MRA_ERR_PARAM;
  if (!std::isfinite(d->softmax_scale)) return MRA_ERR_PARAM;
  if (d->dtype == MRA_BF16 && d->kprologue != MRA_KPRO_AUTO && d->kprologue != MRA_KPRO_FUSED &&
      d->kprologue != MRA_KPRO_PREPASS && d->kprologue != MRA_KPRO_NONE && d->kprologue != MRA_KPRO_GIVEN)
    return MRA_ERR_PARAM;
  if (d->rope_pairs != MRA_ROPE_HALF && d->rope_pairs != MRA_ROPE_INTERLEAVED) return MRA_ERR_PARAM;
  if (d->gamma_per_head != 0 && d->gamma_per_head != 1) return MRA_ERR_PARAM;
  return MRA_OK;
}

int check_strides(const int64_t* st, int dtype) {
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0) return MRA_ERR_STRIDE;
  if (dtype == MRA_BF16)
    for (int i = 0; i < 3; ++i)
      if (st[i] % 8 != 0) return MRA_ERR_STRIDE;
  return MRA_OK;
}

// How the bf16 attention grid of a group of problems is laid out (a plain
// call is a group of one). Query tiles are numbered problem after problem.
// When the last round of whole tiles would leave most resident slots idle, the
// last n_split tiles are cut into nsplit key ranges each, computed by separate
// workgroups and merged by a second kernel. The workspace holds, problem after
// problem, the (cos, sin) table [B, S, D/2] float2 and (prepass K prologue
// only) K' [B, H, S, D] bf16, then the fp32 split-tile records; every piece
// starts 256-byte aligned. The resident slots and the XCD count come from the
// device's shape.
struct Plan {
  int n, waves, grid, tiles, nxcd;
  int n_qt[MRA_MAX_GROUP];
  int tile_end[MRA_MAX_GROUP];
  int n_whole, n_split, nsplit;
  size_t off_table[MRA_MAX_GROUP], off_kp[MRA_MAX_GROUP], off_part, bytes;
};

size_t table_bytes(const mra_desc* d) {
  if (d->dtype == MRA_BF16 && resolve_kprologue(d) == MRA_KPRO_NONE) return 0;
  return round_up((size_t)d->batch * d->seq * (d->head_dim / 2) * sizeof(float2), kWsAlign);
}
size_t kprime_bytes(const mra_desc* d) {
  if (resolve_kprologue(d) != MRA_KPRO_PREPASS) return 0;
  return round_up((size_t)d->batch * d->seq * d->heads * d->head_dim * sizeof(uint16_t), kWsAlign);
}

// bf16 problems with at least one token; ds[i] valid (checked by the caller).
// Problem i's query tiles cover qbatch[i] items of qlen[i] rows (defaults:
// the descriptor's batch and seq; a packed layout passes its item count and
// longest item), its table and K' the descriptor's [batch, seq] layout.
Plan make_plan(const mra_desc* const* ds, int n, DeviceShape dev, const int* qbatch = nullptr,
               const int* qlen = nullptr) {
  Plan p;
  std::memset(&p, 0, sizeof(p));
  p.n = n;
  const int cus = std::max(dev.cus, 1);
  p.nxcd = std::min(std::max(dev.xcds, 1), kMaxXcds);
  // attention workgroups of w waves resident at once: two per CU below 8
  // waves, one from 8
  auto resident_slots = [&](int w) { return cus * (w * kRowBlocks >= 8 ? 1 : 2); };
  // 8-wave workgroups (256 query rows, one per CU) when the problems hold at
  // least 2.5 rounds of them, or one partial round that the third split rule
  // below cuts into 3 key ranges; 4-wave ones (128 rows, two per CU)
  // otherwise. 8 waves measured 1.4-4% faster on h36, ragged, long and
  // 2048px, 6% on 4 heads and 1.5% on 8 heads at 4608 tokens (a cut single
  // round either way), 0.7% slower at 1024px (2.25 rounds) and 27% slower at
  // 512px (0.5 round, too few key tiles to cut)
  int64_t tiles8 = 0;
  int kt_min = 1 << 30;
  for (int i = 0; i < n; ++i) {
    const int qb = qbatch ? qbatch[i] : ds[i]->batch, ql = qlen ? qlen[i] : ds[i]->seq;
    tiles8 += (int64_t)qb * ds[i]->heads * ((ql + 8 * 32 * kRowBlocks - 1) / (8 * 32 * kRowBlocks));
    kt_min = std::min(kt_min, (ql + kBlockN - 1) / kBlockN);
  }
  const int64_t s8 = resident_slots(8);
  const bool cut_round8 = 4 * tiles8 > s8 && 5 * tiles8 <= 3 * s8 && kt_min >= 3 * kMinPartKeyTiles;
  const int waves = (2 * tiles8 >= 5 * s8 || cut_round8) ? 8 : 4;
  const int bm = waves * 32 * kRowBlocks, slots = resident_slots(waves);
  p.waves = waves;
  int tiles = 0, ktiles = 1 << 30;
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const mra_desc* d = ds[i];
    const int qb = qbatch ? qbatch[i] : d->batch, ql = qlen ? qlen[i] : d->seq;
    p.n_qt[i] = (ql + bm - 1) / bm;
    tiles += qb * d->heads * p.n_qt[i];
    p.tile_end[i] = tiles;
    ktiles = std::min(ktiles, (ql + kBlockN - 1) / kBlockN);
    p.off_table[i] = off;
    off += table_bytes(d);
    p.off_kp[i] = off;
    off += kprime_bytes(d);
  }
  int r = tiles >= slots ? tiles % slots : tiles;
  int k = 1;
  // split when the last wave would leave at least half of the compute units
  // idle (a unit running one workgroup instead of two is not idle), spreading
  // the parts over one workgroup per CU (measured faster than filling both
  // slots of every CU, which doubles the partial results the merge reads), or,
  // after whole waves, when it holds a few more tiles than there are units (a
  // few units would run two tiles while the rest run one: halves even them
  // out; measured on last waves of 192 to 416 tiles, it pays only in that
  // band)
  if (r > 0 && 4 * r <= slots) k = std::min(std::min(cus / r, mra::kMaxSplit), ktiles);
  else if (tiles >= slots && r > cus && 4 * r <= 5 * cus) k = std::min(2, ktiles);
  // a single wave too full for the first rule but at most 3/5 of the slots
  // (say one GPU's 4 or 8 heads of a head-sharded layer): every tile in 3 key
  // ranges, when each range keeps at least 24 key tiles (measured at 4608
  // tokens: 144 tiles 90.6 -> 66.3 us, 288 tiles 129.6 -> 119.0 us; 2 or 4
  // ranges less; 512px, 20 key tiles, loses with any cut)
  else if (tiles < slots && 5 * r <= 3 * slots && ktiles >= 3 * kMinPartKeyTiles) k = std::min(3, mra::kMaxSplit);
  if (k < 2) { r = 0; k = 1; }
  p.n_split = r;
  p.nsplit = k;
  p.n_whole = tiles - r;
  p.tiles = tiles;
  p.grid = p.n_whole + p.n_split * p.nsplit;
  p.off_part = off;
  const size_t rec_floats = (size_t)kRowBlocks * waves * 64 * (ds[0]->head_dim / 2 + 2);
  p.bytes = off + round_up((size_t)r * k * rec_floats * sizeof(float), kWsAlign);
  return p;
}

size_t workspace_bytes(const mra_desc* d, DeviceShape dev) {
  if (d->dtype != MRA_BF16 || d->batch == 0 || d->seq == 0) return 0;
  return make_plan(&d, 1, dev).bytes;
}

void fill_args(Args& a, const mra_desc* d, const void* q, const void* k, const void* v,
               const int32_t* pos, const float* gq, const float* gk, const int32_t* seq_lens,
               void* out, float* lse) {
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.pos = pos; a.gq = gq; a.gk = gk; a.seq_lens = seq_lens;
  a.out = out; a.lse = lse;
  a.qs0 = d->q_stride[0]; a.qs1 = d->q_stride[1]; a.qs2 = d->q_stride[2];
  a.ks0 = d->k_stride[0]; a.ks1 = d->k_stride[1]; a.ks2 = d->k_stride[2];
  a.vs0 = d->v_stride[0]; a.vs1 = d->v_stride[1]; a.vs2 = d->v_stride[2];
  a.os0 = d->o_stride[0]; a.os1 = d->o_stride[1]; a.os2 = d->o_stride[2];
  a.B = d->batch; a.S = d->seq; a.H = d->heads; a.T = d->text_pad;
  a.eps = d->eps;
  a.scale = d->softmax_scale > 0.f ? d->softmax_scale : (float)(1.0 / std::sqrt((double)d->head_dim));
  a.c2 = (float)((double)a.scale * 1.4426950408889634);
  a.pscale = 1.0f;
  a.qmul = d->kprologue == MRA_KPRO_GIVEN ? a.c2 : 1.0f;
  a.gqs = d->gamma_per_head ? d->head_dim : 0;
  a.inter = d->rope_pairs == MRA_ROPE_INTERLEAVED;
  const int half = d->head_dim / 2;
  for (int j = 0; j < half; ++j)
    a.rope.inv_freq[j] = (float)std::pow((double)d->theta, -2.0 * j / d->head_dim);
  a.rope.sec_t = d->section[0];
  a.rope.sec_th = d->section[0] + d->section[1];
}

// Points problem j's Args at its pieces of the workspace.
void bind_workspace(Args& a, const mra_desc* d, const Plan& p, int j, void* workspace) {
  char* w = (char*)workspace;
  a.cs = resolve_kprologue(d) == MRA_KPRO_NONE ? nullptr : (float2*)(w + p.off_table[j]);
  a.kp = resolve_kprologue(d) == MRA_KPRO_PREPASS ? (uint16_t*)(w + p.off_kp[j]) : nullptr;
  a.n_qt = p.n_qt[j];
}

template <int D>
hipError_t launch_prologue_bf16(Args& a, int kpro, hipStream_t s) {
  const int64_t tokens = (int64_t)a.B * a.S;
  if (kpro == MRA_KPRO_NONE) return hipSuccess;  // the operands are given
  if (kpro == MRA_KPRO_PREPASS) {
    hipLaunchKernelGGL(mra::k_prologue_kernel<D>, dim3((unsigned)((tokens + 3) / 4)), dim3(256), 0, s, a);
  } else {
    const int64_t n = tokens * (D / 2);
    hipLaunchKernelGGL(mra::rope_table_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int W, int G>
hipError_t launch_attend_waves(const mra::Group<G>& g, int grid, int kpro, hipStream_t s) {
  if (kpro == MRA_KPRO_PREPASS)
    hipLaunchKernelGGL((mra::attn_bf16_kernel<D, W, kBlockN, kRowBlocks, 0, G>), dim3(grid), dim3(W * 64), 0, s, g);
  else if (kpro == MRA_KPRO_FUSED)
    hipLaunchKernelGGL((mra::attn_bf16_kernel<D, W, kBlockN, kRowBlocks, 1, G>), dim3(grid), dim3(W * 64), 0, s, g);
  else
    hipLaunchKernelGGL((mra::attn_bf16_kernel<D, W, kBlockN, kRowBlocks, 2, G>), dim3(grid), dim3(W * 64), 0, s, g);
  if (g.n_split) {
    const int64_t threads = (int64_t)g.n_split * W * kRowBlocks * (D / 8) * 64;
    hipLaunchKernelGGL((mra::split_merge_kernel<D, W, kRowBlocks, G>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}
template <int D, int G>
hipError_t launch_attend_group(const mra::Group<G>& g, int grid, int kpro, int waves, hipStream_t s) {
  return waves == 8 ? launch_attend_waves<D, 8>(g, grid, kpro, s) : launch_attend_waves<D, 4>(g, grid, kpro, s);
}
static_assert(sizeof(mra::Group<MRA_MAX_GROUP>) <= 4096, "kernel argument size");

// Group descriptor for the attention launch of the problems in `as`, which
// fill_args and bind_workspace have prepared.
template <int G>
void make_group(mra::Group<G>& g, const Args* as, const Plan& p, void* workspace) {
  std::memset(&g, 0, sizeof(g));
  for (int i = 0; i < p.n; ++i) {
    g.p[i] = as[i];
    g.tile_end[i] = p.tile_end[i];
  }
  for (int i = p.n; i < G; ++i) g.tile_end[i] = p.tile_end[p.n - 1];
  g.n_whole = p.n_whole;
  g.n_split = p.n_split;
  g.nsplit = p.nsplit;
  g.nxcd = p.nxcd;
  g.part = p.n_split ? (float*)((char*)workspace + p.off_part) : nullptr;
}

hipError_t launch_attend(const Args* as, const Plan& p, void* workspace, int D, int kpro, hipStream_t s) {
  if (p.n == 1) {
    mra::Group<1> g;
    make_group(g, as, p, workspace);
    return D == 128 ? launch_attend_group<128>(g, p.grid, kpro, p.waves, s)
                    : launch_attend_group<64>(g, p.grid, kpro, p.waves, s);
  }
  mra::Group<MRA_MAX_GROUP> g;
  make_group(g, as, p, workspace);
  return D == 128 ? launch_attend_group<128>(g, p.grid, kpro, p.waves, s)
                  : launch_attend_group<64>(g, p.grid, kpro, p.waves, s);
}

// qlen: rows per item (a.S for the padded layout, the longest item for a
// packed one)
template <int D>
hipError_t launch_fp32(Args& a, hipStream_t s, int qlen) {
  a.n_qt = (qlen + kFp32BlockM - 1) / kFp32BlockM;
  a.grid = a.B * a.H * a.n_qt;
  hipLaunchKernelGGL(mra::attn_fp32_kernel<D>, dim3(a.grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int mrope_attn_abi_version(void) { return 109; }

int mrope_attn_last_hip_error(const char** name) {
  if (name) *name = t_last_hip_error ? hipGetErrorName((hipError_t)t_last_hip_error) : "none";
  return t_last_hip_error;
}

const char* mrope_attn_status_string(int status) {
  switch (status) {
    case MRA_OK: return "ok";
    case MRA_ERR_NULL: return "a required pointer is NULL";
    case MRA_ERR_SHAPE: return "shape out of range (batch/seq/heads/head_dim/text_pad)";
    case MRA_ERR_DTYPE: return "unknown dtype";
    case MRA_ERR_SECTION: return "rotary section entries must be >= 0 and sum to head_dim/2";
    case MRA_ERR_STRIDE: return "unusable strides or alignment";
    case MRA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MRA_ERR_WORKSPACE: return "workspace missing or too small";
    case MRA_ERR_HIP: return "HIP launch or runtime error";
    case MRA_ERR_PARAM: return "invalid theta/eps/softmax_scale/kprologue/rope_pairs/gamma_per_head, or group size";
    case MRA_ERR_SCRATCH: return "problem needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int mrope_attn_validate(const mra_desc* d, const void* q, const void* k, const void* v,
                        const int32_t* pos, const float* gq, const float* gk,
                        const int32_t* seq_lens, const void* out) {
  (void)seq_lens;
  int rc = check_desc(d);
  if (rc != MRA_OK) return rc;
  if (d->batch == 0 || d->seq == 0) return MRA_OK;
  // operands given (MRA_KPRO_NONE, MRA_KPRO_GIVEN): positions and gammas are not read
  const bool given = d->dtype == MRA_BF16 && resolve_kprologue(d) == MRA_KPRO_NONE;
  if (!q || !k || !v || !out || (!given && (!pos || !gq || !gk))) return MRA_ERR_NULL;
  if ((rc = check_strides(d->q_stride, d->dtype)) != MRA_OK) return rc;
  if ((rc = check_strides(d->k_stride, d->dtype)) != MRA_OK) return rc;
  if ((rc = check_strides(d->v_stride, d->dtype)) != MRA_OK) return rc;
  if ((rc = check_strides(d->o_stride, d->dtype)) != MRA_OK) return rc;
  // the bf16 kernels address each (batch, head) slice with 32-bit byte offsets
  if (d->dtype == MRA_BF16) {
    const int64_t lim = (int64_t)1 << 31;
    const int64_t* st[4] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
    for (int i = 0; i < 4; ++i)
      if (((int64_t)d->seq * st[i][1] + d->head_dim) * 2 >= lim) return MRA_ERR_UNSUPPORTED;
    if ((int64_t)d->seq * d->head_dim * 2 >= lim) return MRA_ERR_UNSUPPORTED;
  }
  const size_t al = d->dtype == MRA_BF16 ? 16 : 4;
  if (!aligned(q, al) || !aligned(k, al) || !aligned(v, al) || !aligned(out, al)) return MRA_ERR_STRIDE;
  if (!aligned(pos, 4) || !aligned(seq_lens, 4)) return MRA_ERR_STRIDE;
  if (!aligned(gq, al) || !aligned(gk, al)) return MRA_ERR_STRIDE;
  return MRA_OK;
}

int mrope_attn_launch_plan(const mra_desc* d, int32_t cus, int32_t xcds, mra_launch_plan* out) {
  if (!out) return MRA_ERR_NULL;
  std::memset(out, 0, sizeof(*out));
  const int rc = check_desc(d);
  if (rc != MRA_OK) return rc;
  if (d->dtype != MRA_BF16) return MRA_ERR_UNSUPPORTED;
  if (d->batch == 0 || d->seq == 0) return MRA_OK;
  const DeviceShape dev = cus > 0 ? DeviceShape{cus, xcds > 0 ? xcds : 1} : current_device_shape();
  const Plan p = make_plan(&d, 1, dev);
  out->waves = p.waves;
  out->grid = p.grid;
  out->xcds = p.nxcd;
  out->tiles = p.tiles;
  out->split_tiles = p.n_split;
  out->parts = p.nsplit;
  out->workspace_bytes = p.bytes;
  return MRA_OK;
}

size_t mrope_attn_workspace_size(const mra_desc* d) {
  if (check_desc(d) != MRA_OK) return 0;
  return workspace_bytes(d, current_device_shape());
}

// Shared front half of the three launching entry points: validation,
// workspace check, fault-injection hook and argument packing.
static int prepare_call(const mra_desc* d, const void* q, const void* k, const void* v,
                        const int32_t* pos, const float* gq, const float* gk,
                        const int32_t* seq_lens, void* out, float* lse, void* workspace,
                        size_t ws_bytes, Args& a, Plan& plan, bool& empty) {
  int rc = mrope_attn_validate(d, q, k, v, pos, gq, gk, seq_lens, out);
  if (rc != MRA_OK) return rc;
  empty = d->batch == 0 || d->seq == 0;
  if (empty) return MRA_OK;
  if (lse && !aligned(lse, 4)) return MRA_ERR_STRIDE;
  const DeviceShape dev = current_device_shape();
  const size_t need = workspace_bytes(d, dev);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 16))) return MRA_ERR_WORKSPACE;
  const char* fi = std::getenv("MRA_FAULT_INJECT");
  if (fi && std::strcmp(fi, "launch") == 0) return MRA_ERR_HIP;
  clear_stale_hip_error();
  fill_args(a, d, q, k, v, pos, gq, gk, seq_lens, out, lse);
  if (d->dtype == MRA_BF16) {
    plan = make_plan(&d, 1, dev);
    bind_workspace(a, d, plan, 0, workspace);
  }
  return MRA_OK;
}

int mrope_attn_prepare(const mra_desc* d, const void* k, const int32_t* pos, const float* gk,
                       void* workspace, size_t ws_bytes, void* stream) {
  // q/v/out/gamma_q are not touched by this stage; validate with k standing in
  Args a;
  Plan plan;
  bool empty = false;
  int rc = prepare_call(d, k, k, k, pos, gk, gk, nullptr, (void*)k, nullptr, workspace, ws_bytes, a, plan, empty);
  if (rc != MRA_OK || empty || d->dtype != MRA_BF16) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int kpro = resolve_kprologue(d);
  hipError_t e = d->head_dim == 128 ? launch_prologue_bf16<128>(a, kpro, s) : launch_prologue_bf16<64>(a, kpro, s);
  return hip_status(e);
}

int mrope_attn_attend(const mra_desc* d, const void* q, const void* k, const void* v,
                      const int32_t* pos, const float* gq, const float* gk, const int32_t* seq_lens,
                      void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  Args a;
  Plan plan;
  bool empty = false;
  int rc = prepare_call(d, q, k, v, pos, gq, gk, seq_lens, out, lse, workspace, ws_bytes, a, plan, empty);
  if (rc != MRA_OK || empty) return rc;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d->dtype == MRA_FP32)
    e = d->head_dim == 128 ? launch_fp32<128>(a, s, a.S) : launch_fp32<64>(a, s, a.S);
  else
    e = launch_attend(&a, plan, workspace, d->head_dim, resolve_kprologue(d), s);
  return hip_status(e);
}

int mrope_attn_fwd(const mra_desc* d, const void* q, const void* k, const void* v,
                   const int32_t* pos, const float* gq, const float* gk, const int32_t* seq_lens,
                   void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  Args a;
  Plan plan;
  bool empty = false;
  int rc = prepare_call(d, q, k, v, pos, gq, gk, seq_lens, out, lse, workspace, ws_bytes, a, plan, empty);
  if (rc != MRA_OK || empty) return rc;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d->dtype == MRA_FP32) {
    e = d->head_dim == 128 ? launch_fp32<128>(a, s, a.S) : launch_fp32<64>(a, s, a.S);
  } else {
    const int kpro = resolve_kprologue(d);
    e = d->head_dim == 128 ? launch_prologue_bf16<128>(a, kpro, s) : launch_prologue_bf16<64>(a, kpro, s);
    if (e == hipSuccess) e = launch_attend(&a, plan, workspace, d->head_dim, kpro, s);
  }
  return hip_status(e);
}

}  // extern "C"

// ---- forward without allocation ---------------------------------------------
// The scratch of mrope_attn_fwd_noalloc: one array per GPU, allocated with the
// library's code object on that GPU and held until the process ends. Host
// code never uses the name itself (on the host it is only a stand-in for the
// symbol): it takes each device's address of the array once, below.
static __device__ __align__(256) unsigned char scratch[MRA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// This process's current device's copy of `scratch`, looked up on the first
// call on that device (with it current), or nullptr if the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    hip_status(e != hipSuccess ? e : hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int mrope_attn_fwd_noalloc(const mra_desc* d, const void* q, const void* k, const void* v,
                           const int32_t* pos, const float* gq, const float* gk,
                           const int32_t* seq_lens, void* out, float* lse, void* stream) {
  int rc = mrope_attn_validate(d, q, k, v, pos, gq, gk, seq_lens, out);
  if (rc != MRA_OK) return rc;
  const size_t need = mrope_attn_workspace_size(d);
  if (need > MRA_NOALLOC_SCRATCH_BYTES) return MRA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && !(ws = scratch_on_current_device())) return MRA_ERR_HIP;
  return mrope_attn_fwd(d, q, k, v, pos, gq, gk, seq_lens, out, lse, ws, need, stream);
}

// Problems of a group call that hold at least one token, in call order;
// checks the group-wide conditions. Returns MRA_OK and their count in *m.
static int group_members(const mra_desc* descs, const mra_problem* probs, int n, int* idx, int* m) {
  if (!descs || !probs) return MRA_ERR_NULL;
  if (n < 1 || n > MRA_MAX_GROUP) return MRA_ERR_PARAM;
  *m = 0;
  for (int i = 0; i < n; ++i) {
    const mra_desc* d = &descs[i];
    const mra_problem& p = probs[i];
    int rc = mrope_attn_validate(d, p.q, p.k, p.v, p.pos_thw, p.gamma_q, p.gamma_k, p.seq_lens, p.out);
    if (rc != MRA_OK) return rc;
    if (p.lse && !aligned(p.lse, 4)) return MRA_ERR_STRIDE;
    if (d->dtype != descs[0].dtype || d->head_dim != descs[0].head_dim) return MRA_ERR_UNSUPPORTED;
    if (d->dtype == MRA_BF16 && resolve_kprologue(d) != resolve_kprologue(&descs[0])) return MRA_ERR_UNSUPPORTED;
    if (d->batch > 0 && d->seq > 0) idx[(*m)++] = i;
  }
  return MRA_OK;
}

size_t mrope_attn_group_workspace_size(const mra_desc* descs, int n) {
  if (!descs || n < 1 || n > MRA_MAX_GROUP) return 0;
  const mra_desc* ds[MRA_MAX_GROUP];
  int m = 0;
  for (int i = 0; i < n; ++i) {
    if (check_desc(&descs[i]) != MRA_OK) return 0;
    if (descs[i].dtype != descs[0].dtype || descs[i].head_dim != descs[0].head_dim) return 0;
    if (descs[i].batch > 0 && descs[i].seq > 0) ds[m++] = &descs[i];
  }
  if (m == 0 || descs[0].dtype != MRA_BF16) return 0;
  return make_plan(ds, m, current_device_shape()).bytes;
}

int mrope_attn_fwd_group(const mra_desc* descs, const mra_problem* probs, int n, void* workspace,
                         size_t ws_bytes, void* stream) {
  int idx[MRA_MAX_GROUP], m = 0;
  int rc = group_members(descs, probs, n, idx, &m);
  if (rc != MRA_OK) return rc;
  if (m == 0) return MRA_OK;
  const size_t need = mrope_attn_group_workspace_size(descs, n);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 16))) return MRA_ERR_WORKSPACE;
  const char* fi = std::getenv("MRA_FAULT_INJECT");
  if (fi && std::strcmp(fi, "launch") == 0) return MRA_ERR_HIP;
  clear_stale_hip_error();
  hipStream_t s = (hipStream_t)stream;
  Args as[MRA_MAX_GROUP];
  const mra_desc* ds[MRA_MAX_GROUP];
  for (int j = 0; j < m; ++j) {
    const mra_problem& p = probs[idx[j]];
    ds[j] = &descs[idx[j]];
    fill_args(as[j], ds[j], p.q, p.k, p.v, p.pos_thw, p.gamma_q, p.gamma_k, p.seq_lens, p.out, p.lse);
  }
  const int D = descs[0].head_dim;
  hipError_t e = hipSuccess;
  if (descs[0].dtype == MRA_FP32) {
    for (int j = 0; j < m && e == hipSuccess; ++j)
      e = D == 128 ? launch_fp32<128>(as[j], s, as[j].S) : launch_fp32<64>(as[j], s, as[j].S);
    return hip_status(e);
  }
  const Plan plan = make_plan(ds, m, current_device_shape());
  const int kpro = resolve_kprologue(ds[0]);
  for (int j = 0; j < m && e == hipSuccess; ++j) {
    bind_workspace(as[j], ds[j], plan, j, workspace);
    e = D == 128 ? launch_prologue_bf16<128>(as[j], kpro, s) : launch_prologue_bf16<64>(as[j], kpro, s);
  }
  if (e == hipSuccess) e = launch_attend(as, plan, workspace, D, kpro, s);
  return hip_status(e);
}

// ---- packed variable-length sequences (cu_seqlens) ------------------------
// The descriptor describes the packed layout: seq = total tokens, batch =
// number of sequences; tensors are one [seq, H, D] slice (the batch stride is
// not used), pos_thw [seq, 3], lse [H, seq].
static int varlen_layout(const mra_desc* d, int32_t max_seqlen, mra_desc& lay) {
  int rc = check_desc(d);
  if (rc != MRA_OK) return rc;
  if (d->text_pad != 0) return MRA_ERR_SHAPE;
  if (max_seqlen < 0 || max_seqlen > d->seq) return MRA_ERR_SHAPE;
  lay = *d;
  lay.batch = 1;
  return MRA_OK;
}

size_t mrope_attn_varlen_workspace_size(const mra_desc* d, int32_t max_seqlen) {
  mra_desc lay;
  if (varlen_layout(d, max_seqlen, lay) != MRA_OK) return 0;
  if (d->dtype != MRA_BF16 || d->batch == 0 || d->seq == 0 || max_seqlen == 0) return 0;
  const mra_desc* ds[1] = {&lay};
  const int qb = d->batch, ql = max_seqlen;
  return make_plan(ds, 1, current_device_shape(), &qb, &ql).bytes;
}

int mrope_attn_fwd_varlen(const mra_desc* d, const void* q, const void* k, const void* v,
                          const int32_t* pos, const float* gq, const float* gk,
                          const int32_t* cu_seqlens, int32_t max_seqlen, void* out, float* lse,
                          void* workspace, size_t ws_bytes, void* stream) {
  mra_desc lay;
  int rc = varlen_layout(d, max_seqlen, lay);
  if (rc != MRA_OK) return rc;
  if (d->batch == 0 || d->seq == 0 || max_seqlen == 0) return MRA_OK;
  rc = mrope_attn_validate(&lay, q, k, v, pos, gq, gk, nullptr, out);
  if (rc != MRA_OK) return rc;
  if (!cu_seqlens) return MRA_ERR_NULL;
  if (!aligned(cu_seqlens, 4) || (lse && !aligned(lse, 4))) return MRA_ERR_STRIDE;
  const size_t need = mrope_attn_varlen_workspace_size(d, max_seqlen);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 16))) return MRA_ERR_WORKSPACE;
  const char* fi = std::getenv("MRA_FAULT_INJECT");
  if (fi && std::strcmp(fi, "launch") == 0) return MRA_ERR_HIP;
  clear_stale_hip_error();
  Args a;
  fill_args(a, &lay, q, k, v, pos, gq, gk, nullptr, out, lse);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d->dtype == MRA_FP32) {
    a.B = d->batch;
    a.cu_seqlens = cu_seqlens;
    e = d->head_dim == 128 ? launch_fp32<128>(a, s, max_seqlen) : launch_fp32<64>(a, s, max_seqlen);
  } else {
    const mra_desc* ds[1] = {&lay};
    const int qb = d->batch, ql = max_seqlen;
    const Plan plan = make_plan(ds, 1, current_device_shape(), &qb, &ql);
    bind_workspace(a, &lay, plan, 0, workspace);
    const int kpro = resolve_kprologue(d);
    // the prologue pass runs over the packed layout (one item of seq tokens)
    e = d->head_dim == 128 ? launch_prologue_bf16<128>(a, kpro, s) : launch_prologue_bf16<64>(a, kpro, s);
    if (e == hipSuccess) {
      a.B = d->batch;
      a.cu_seqlens = cu_seqlens;
      e = launch_attend(&a, plan, workspace, d->head_dim, kpro, s);
    }
  }
  return hip_status(e);
}

}  // extern "C"

// the backward and projection entry points share the helpers above
#include "bwd_host.hpp"
#include "qkv_host.hpp"
