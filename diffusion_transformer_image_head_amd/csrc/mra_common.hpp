// Shared device-side types and helpers for the fused QK-RMSNorm + 3D M-RoPE
// attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace mra {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxHalf = 64;  // head_dim <= 128
constexpr int kMaxSplit = 8;  // key-range parts per split query tile

// Rotary frequencies theta^(-2j/D), rounded once to fp32 on the host, and the
// section boundaries: pair j follows t if j < sec_t, h if j < sec_th, else w.
struct Rope {
  float inv_freq[kMaxHalf];
  int32_t sec_t;
  int32_t sec_th;
};

struct Args {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pos;       // [B, S, 3]
  const float* gq;          // [D], or [H, D] when gqs == D
  const float* gk;          // same shape as gq
  const int32_t* seq_lens;  // [B] or null
  const int32_t* cu_seqlens;  // [B + 1] or null: packed sequences (see seq_view)
  void* out;
  float* lse;               // [B, H, S] or null
  uint16_t* kp;             // K' (bf16) [B, H, S, D] in the workspace, or null
  float2* cs;               // (cos, sin) [B, S, D/2] in the workspace, or null
  int64_t qs0, qs1, qs2;
  int64_t ks0, ks1, ks2;
  int64_t vs0, vs1, vs2;
  int64_t os0, os1, os2;
  int32_t B, S, H, T;
  int32_t n_qt;             // query tiles per (batch, head)
  int32_t grid;             // workgroups launched (single-problem kernels)
  float eps;
  float c2;                 // softmax scale * log2(e)
  float scale;
  float pscale;             // factor applied by k_prologue_kernel before rounding
  float qmul;               // given operands: factor q is multiplied by as it is loaded
  int32_t gqs;              // elements between the gamma rows of two heads (0: shared)
  int32_t inter;            // rotary pairs (2j, 2j + 1) instead of (j, j + D/2)
  Rope rope;
};

// Where batch item b's tokens sit in the tensors. Padded layout (no
// cu_seqlens): item b holds tokens [0, S) of its own [S, ...] slice. Packed
// layout: one [S_total, ...] slice (a.S = S_total) holds item b's tokens at
// [cu_seqlens[b], cu_seqlens[b+1]), clamped into [0, S_total].
struct SeqView {
  int bl;        // batch index into the tensors
  int64_t tok0;  // first token of the item within that slice
  int S;         // tokens of the item
};
__device__ __forceinline__ SeqView seq_view(const Args& a, int b) {
  if (!a.cu_seqlens) return SeqView{b, 0, a.S};
  const int t0 = min(max(a.cu_seqlens[b], 0), a.S);
  const int t1 = min(max(a.cu_seqlens[b + 1], t0), a.S);
  return SeqView{0, t0, t1 - t0};
}

// Up to G problems in one attention launch (G = 1 for a plain call). Their
// query tiles are numbered one after another: problem i owns global tiles
// [tile_end[i-1], tile_end[i]). Global tiles [0, n_whole) are computed by one
// workgroup each; the remaining n_split tiles by nsplit workgroups each over
// disjoint key ranges, whose partial (O, max, sum) records go to `part` and
// are merged by a second launch.
template <int G>
struct Group {
  Args p[G];
  int32_t tile_end[G];
  int32_t n_whole;
  int32_t n_split;
  int32_t nsplit;
  int32_t nxcd;   // XCDs of the device (workgroups are dealt to them in turn)
  float* part;
};

// Problem owning global tile gt, and the tile's index within that problem.
template <int G>
__device__ __forceinline__ int group_problem(const Group<G>& g, int gt, int& tile) {
  int k = 0;
#pragma unroll
  for (int i = 0; i + 1 < G; ++i) k += gt >= g.tile_end[i];
  tile = k ? gt - g.tile_end[k - 1] : gt;
  return k;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two fp32 values to bf16 (nearest, ties to even) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Value of lane (l ^ 32) for a 32-bit quantity, via the gfx950 permlane32 swap
// (swaps the upper half-wave of the first operand with the lower half of the
// second; with both operands x the two results are {x, partner} in some order).
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Rotary axis position of pair j for a token with positions (pt, ph, pw).
__device__ __forceinline__ int axis_pos(const Rope& r, int j, int pt, int ph, int pw) {
  return j < r.sec_t ? pt : (j < r.sec_th ? ph : pw);
}

// Bijective remap of a linear workgroup id i < n so consecutive logical tiles
// land on the same XCD: the hardware deals workgroups round-robin over the
// device's nx XCDs, so ids i, i+nx, i+2nx, ... share an XCD; give each XCD a
// contiguous logical range.
__device__ __forceinline__ int xcd_remap(int i, int n, int nx) {
  const int q = n / nx, r = n % nx;
  const int x = i % nx, local = i / nx;
  return x * q + (x < r ? x : r) + local;
}

}  // namespace mra
