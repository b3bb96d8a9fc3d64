/*
 * mrope_attn.h -- C ABI of the fused QK-RMSNorm + 3D M-RoPE joint text+image
 * attention library for AMD Instinct MI355X (gfx950), libmrope_attn.so.
 *
 * The operation (Ideogram 4.0 announcement thread, the post listing the DiT's
 * parts: single-stream self-attention with QK-RMSNorm and a 3D multimodal RoPE
 * that puts text and image tokens in one positional frame; "Ideogram 4 deep
 * dive", section 4 part 2: text and image tokens concatenated into one
 * sequence through the same self-attention), for every batch item b, head h
 * and token s of a sequence of S = text_pad + image tokens:
 *
 *   1. RMSNorm over head_dim:  x_hat = x * (mean_d x_d^2 + eps)^-1/2 * gamma
 *      (gamma_q for Q, gamma_k for K; one [head_dim] weight shared by heads,
 *      or one per head with mra_desc.gamma_per_head);
 *   2. 3D M-RoPE: rotary pair j = (x_hat_j, x_hat_{j+D/2}), j < D/2 (or
 *      (x_hat_2j, x_hat_2j+1) with mra_desc.rope_pairs = MRA_ROPE_INTERLEAVED),
 *      is turned by pos[b,s,axis(j)] * theta^(-2j/D), where axis(j) is t for the first
 *      section[0] pairs, h for the next section[1], w for the last section[2]
 *      ("Ideogram 4 deep dive", section 6 part 3 names the split (24,20,20));
 *      the frequency is computed in fp32 (the unsloth commit log for the
 *      Ideogram 4 backend: rotary inv_freq is built in explicit fp32);
 *   3. non-causal softmax attention with scale softmax_scale over the valid
 *      keys of the item; text slot s < text_pad is valid iff s < seq_lens[b]
 *      (per-prompt true text length, padded in memory: SimpleTuner
 *      quickstart, "Text Embed Cache"); image tokens are always valid.
 *      Output rows of invalid tokens are written as exact zeros.
 *
 * Numerics of the bf16 path: fp32 norm/rotation math, Q' and K' rounded once
 * to bf16 (round-to-nearest-even), bf16 x bf16 -> fp32 matrix-core products,
 * fp32 online softmax, probabilities rounded once to bf16 before P.V (the row
 * sum uses the same rounded values), output rounded once. The fp32 path
 * rounds nowhere beyond fp32 arithmetic.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE memory owned by the caller; the library
 *    keeps no pointer after a call returns and never frees caller memory.
 *  - q, k, v, out are [B, S, H, D] views with head_dim contiguous and element
 *    strides given for the batch, token and head axes (so Q, K, V may be
 *    strided views of one fused [B, S, 3, H, D] projection output -- the
 *    Ideogram 4 checkpoint stores Q/K/V rows stacked in one fused weight, per
 *    the unsloth commit log; Q, K and V have the same head count there).
 *  - pos_thw is [B, S, 3] int32 contiguous, (t, h, w) per token.
 *  - gamma_q, gamma_k are [D] fp32 contiguous ([H, D] with gamma_per_head).
 *    seq_lens is [B] int32 or NULL (no padding); values are read on the
 *    device and clamped to [0, text_pad].
 *  - lse, when not NULL, is [B, H, S] fp32 contiguous: natural-log
 *    log-sum-exp of the scaled logits of each valid row, -inf for invalid rows.
 *  - stream is a hipStream_t (NULL = the legacy default stream). Calls are
 *    asynchronous; results are valid after the stream synchronises.
 *  - Errors are negative mra_status values. Every contract check runs on the
 *    host before any device work; on error nothing is launched or written.
 *  - Calls are thread-safe. The library's only global state is the per-thread
 *    record behind mrope_attn_last_hip_error and a per-device cache of the
 *    no-allocation scratch array's address (see mrope_attn_fwd_noalloc).
 */
#ifndef MROPE_ATTN_H
#define MROPE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MRA_OK = 0,
  MRA_ERR_NULL = -1,        /* a required pointer is NULL */
  MRA_ERR_SHAPE = -2,       /* batch/seq/heads/head_dim/text_pad out of range */
  MRA_ERR_DTYPE = -3,       /* unknown dtype */
  MRA_ERR_SECTION = -4,     /* section entries negative or not summing to D/2 */
  MRA_ERR_STRIDE = -5,      /* strides/alignment unusable (see mra_desc) */
  MRA_ERR_UNSUPPORTED = -6, /* valid request this build does not implement */
  MRA_ERR_WORKSPACE = -7,   /* workspace missing or smaller than required */
  MRA_ERR_HIP = -8,         /* a HIP launch or runtime call failed */
  MRA_ERR_PARAM = -9,       /* theta/eps/scale/kprologue/rope_pairs/gamma_per_head invalid,
                               or a group size outside 1..MRA_MAX_GROUP */
  MRA_ERR_SCRATCH = -10     /* mrope_attn_fwd_noalloc: the problem needs more scratch than
                               MRA_NOALLOC_SCRATCH_BYTES */
} mra_status;

typedef enum { MRA_BF16 = 0, MRA_FP32 = 1 } mra_dtype;

/* Where the K prologue (RMSNorm + M-RoPE of K) runs in the bf16 path. */
typedef enum {
  MRA_KPRO_AUTO = 0,    /* library's choice (currently MRA_KPRO_PREPASS) */
  MRA_KPRO_FUSED = 1,   /* applied while each K tile is staged into LDS */
  MRA_KPRO_PREPASS = 2, /* one pass writes K' (bf16) to the workspace first */
  MRA_KPRO_NONE = 3,    /* q and k already hold the operands Q'' and K' (as written
                           by mrope_qkv_proj with the same softmax_scale): q is
                           Q' already multiplied by softmax_scale * log2(e); no
                           norm or rotation is applied; pos_thw, gamma_q, gamma_k
                           are not read and may be NULL */
  MRA_KPRO_GIVEN = 4    /* q and k hold Q' and K', normalised and rotated but not
                           scaled: q is multiplied by softmax_scale * log2(e) as
                           it is loaded (one more bf16 rounding than
                           MRA_KPRO_NONE); no norm or rotation is applied;
                           pos_thw, gamma_q, gamma_k are not read and may be NULL */
} mra_kprologue;

/* Which elements of a head row form rotary pair j. The pages do not say;
 * both layouts are in use for rotary encodings. */
typedef enum {
  MRA_ROPE_HALF = 0,        /* (j, j + D/2): the rotate-half layout (default) */
  MRA_ROPE_INTERLEAVED = 1  /* (2j, 2j + 1) */
} mra_rope_pairs;

typedef struct {
  int32_t batch;          /* B >= 0 (0 = nothing to do) */
  int32_t seq;            /* S >= 0: text_pad text slots, then image tokens */
  int32_t heads;          /* H >= 1, same for Q, K, V */
  int32_t head_dim;       /* D: 64 or 128 */
  int32_t text_pad;       /* text slots at the start of each sequence, 0..S */
  int32_t section[3];     /* rotary pairs driven by t, h, w; sum == D/2 */
  float theta;            /* rotary base, > 0 (10000) */
  float eps;              /* RMSNorm epsilon, >= 0 (1e-6) */
  float softmax_scale;    /* > 0, or <= 0 for 1/sqrt(D) */
  int32_t dtype;          /* mra_dtype of q, k, v and out */
  int32_t kprologue;      /* mra_kprologue (bf16 only; ignored for fp32) */
  int64_t q_stride[3];    /* element strides of the batch, token, head axes */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int32_t rope_pairs;     /* mra_rope_pairs */
  int32_t gamma_per_head; /* 0: gamma_q, gamma_k are [D]; 1: [H, D] (row h for head h) */
} mra_desc;

/* Host-only check of a call's arguments; touches no device and reads no
 * device memory. Returns MRA_OK or the error mrope_attn_fwd would return.
 * bf16 requires 16-byte aligned q, k, v, out, gamma_q, gamma_k and
 * token/head/batch strides that are multiples of 8 elements; fp32 requires
 * 4-byte alignment. */
int mrope_attn_validate(const mra_desc* desc, const void* q, const void* k, const void* v,
                        const int32_t* pos_thw, const float* gamma_q, const float* gamma_k,
                        const int32_t* seq_lens, const void* out);

/* Bytes of device workspace mrope_attn_fwd needs for this descriptor
 * (0 when none). Returns 0 for an invalid descriptor. */
size_t mrope_attn_workspace_size(const mra_desc* desc);

/* The fused forward pass (see the top of this file). workspace must hold at
 * least mrope_attn_workspace_size(desc) bytes (16-byte aligned) when that
 * size is nonzero; it is scratch, overwritten by the call (for bf16 it holds
 * the rotary table, K' with MRA_KPRO_PREPASS, and the fp32 partial results of
 * the query tiles that would otherwise run in a last, mostly idle wave of
 * workgroups: those are cut into key ranges and merged by a second kernel). out must not
 * overlap q, k, v or the workspace. Launches on `stream` and returns without
 * synchronising. */
int mrope_attn_fwd(const mra_desc* desc, const void* q, const void* k, const void* v,
                   const int32_t* pos_thw, const float* gamma_q, const float* gamma_k,
                   const int32_t* seq_lens, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ---- Forward without any allocation ------------------------------------
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. mrope_attn_fwd_noalloc computes exactly what
 * mrope_attn_fwd computes (the same kernels, bitwise equal results), but its
 * scratch (the rotary table, K' and the split-tile partial results) lives in
 * one file-scope device array of MRA_NOALLOC_SCRATCH_BYTES bytes inside the
 * library instead of a caller workspace. Each GPU the library runs on holds
 * its own copy of that array from the library's first use on it until the
 * process ends. The call allocates nothing and frees nothing.
 *
 * It runs on the current HIP device; stream must belong to that device. The
 * arguments, validation and errors are those of mrope_attn_fwd, plus
 * MRA_ERR_SCRATCH (nothing launched) when mrope_attn_workspace_size(desc)
 * exceeds MRA_NOALLOC_SCRATCH_BYTES (64 MiB: enough for one 1024px layer of
 * 32 or 36 heads, B=1, 4608 tokens; not for the 4-item ragged batch or 12800
 * tokens), and MRA_ERR_HIP when the array's device address cannot be
 * obtained. Every call on one GPU uses that GPU's one array: calls that
 * overlap in time on one GPU (on different streams, or from several host
 * threads without ordering their streams) race and give wrong results;
 * calls ordered on one stream are safe. The array keeps the last call's
 * contents; no result depends on them (every byte a call reads from it was
 * written earlier in the same call). */
#define MRA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int mrope_attn_fwd_noalloc(const mra_desc* desc, const void* q, const void* k, const void* v,
                           const int32_t* pos_thw, const float* gamma_q, const float* gamma_k,
                           const int32_t* seq_lens, void* out, float* lse, void* stream);

/* ---- The launch plan (host only) -----------------------------------------
 *
 * The bf16 attention launches one workgroup per query tile, dealt so that the
 * tiles each XCD runs are neighbours (shared K'/V in its L2); when the last
 * round of workgroups would leave most of the device idle, its tiles are cut
 * into key-range parts merged by a second kernel. The plan depends on the
 * device's compute units and XCDs, which the library queries once per
 * device; mrope_attn_workspace_size and every launching call use the current
 * device's. mrope_attn_launch_plan reports the plan for a given device shape
 * without touching a device: compute_units <= 0 asks for the current
 * device's (the MI355X's 256 CUs in 8 XCDs when no device can be queried);
 * xcds <= 0 means 1. Returns the descriptor checks' error, MRA_ERR_NULL for
 * a NULL plan, MRA_ERR_UNSUPPORTED for fp32 (which has no such plan), else
 * MRA_OK; an empty problem gives a zero plan. */
typedef struct {
  int32_t waves;            /* waves per attention workgroup: 4 (128 query rows) or 8 (256) */
  int32_t grid;             /* attention workgroups launched */
  int32_t xcds;             /* XCDs the workgroups are dealt to */
  int32_t tiles;            /* query tiles */
  int32_t split_tiles;      /* tiles computed as key-range parts and merged */
  int32_t parts;            /* key-range parts per split tile (1: no split) */
  uint64_t workspace_bytes; /* mrope_attn_workspace_size on such a device */
} mra_launch_plan;

int mrope_attn_launch_plan(const mra_desc* desc, int32_t compute_units, int32_t xcds,
                           mra_launch_plan* plan);

/* The two stages of mrope_attn_fwd, for callers that schedule or time them
 * separately. mrope_attn_prepare runs the prologue pass (the per-token
 * rotary (cos, sin) table, plus K' for MRA_KPRO_PREPASS) into the workspace;
 * it reads only k, pos_thw and gamma_k (a no-op for fp32). mrope_attn_attend
 * then runs the attention kernel and requires that mrope_attn_prepare has run
 * on the same stream (or been ordered before it) with the same descriptor,
 * inputs and workspace. fwd == prepare followed by attend. Arguments,
 * validation and errors are as for mrope_attn_fwd. */
int mrope_attn_prepare(const mra_desc* desc, const void* k, const int32_t* pos_thw,
                       const float* gamma_k, void* workspace, size_t workspace_bytes,
                       void* stream);
int mrope_attn_attend(const mra_desc* desc, const void* q, const void* k, const void* v,
                      const int32_t* pos_thw, const float* gamma_q, const float* gamma_k,
                      const int32_t* seq_lens, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- Grouped launch: several problems in one attention launch ----------
 *
 * One sampling step of the model runs the DiT twice: the conditional pass on
 * [text + image] tokens and the unconditional pass on the image tokens alone
 * (text_pad = 0), which is the cheaper of the two ("Ideogram 4 deep dive",
 * section 4 part 4, asymmetric classifier-free guidance). mrope_attn_fwd_group
 * computes up to MRA_MAX_GROUP such problems, each with its own descriptor
 * and tensors, as if by one mrope_attn_fwd call each, but with the query
 * tiles of all of them in one attention launch (one tail of partly filled
 * workgroup waves instead of one per problem). Problems may differ in batch,
 * seq, heads, text_pad, section, theta, eps, softmax_scale and strides; they
 * must share dtype, head_dim and (bf16) the resolved kprologue, else
 * MRA_ERR_UNSUPPORTED. Problems with batch == 0 or seq == 0 are skipped.
 * Outputs must not overlap each other or any input. Errors are those of
 * mrope_attn_fwd for the first failing problem, MRA_ERR_PARAM for n outside
 * [1, MRA_MAX_GROUP], MRA_ERR_NULL for NULL descs/probs; as for every call,
 * nothing is launched on error. */
#define MRA_MAX_GROUP 4

typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pos_thw;
  const float* gamma_q;
  const float* gamma_k;
  const int32_t* seq_lens; /* or NULL */
  void* out;
  float* lse;              /* or NULL */
} mra_problem;

/* Bytes of device workspace mrope_attn_fwd_group needs (0 when none or when
 * the descriptors are invalid). */
size_t mrope_attn_group_workspace_size(const mra_desc* descs, int n);

int mrope_attn_fwd_group(const mra_desc* descs, const mra_problem* probs, int n,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- Packed variable-length sequences -----------------------------------
 *
 * The per-prompt text length can also be carried by packing instead of
 * padding (the padding convention is the SimpleTuner quickstart's "Text Embed
 * Cache"; packing drops the padded slots): desc->batch sequences of varying
 * length are stored back to back, sequence b holding tokens
 * [cu_seqlens[b], cu_seqlens[b+1]) of one [desc->seq, H, D] slice (its own
 * true-length text tokens followed by its image tokens, each with its (t, h, w)
 * in pos_thw), and every token attends to the tokens of its own sequence
 * only. desc->seq is the total token count, desc->text_pad must be 0
 * (MRA_ERR_SHAPE), the batch strides are not used, pos_thw is [seq, 3] and
 * lse [H, seq]. cu_seqlens is a device [batch + 1] int32 array, read on the
 * device and clamped into [0, seq]; it must be non-decreasing (an entry below
 * its predecessor makes that sequence empty, and sequences that overlap
 * write the same rows in an unspecified order); max_seqlen (0..seq, else MRA_ERR_SHAPE)
 * must be at least every sequence's length: rows past max_seqlen of a longer
 * sequence are not computed. Tokens outside every sequence are not written. */
size_t mrope_attn_varlen_workspace_size(const mra_desc* desc, int32_t max_seqlen);

int mrope_attn_fwd_varlen(const mra_desc* desc, const void* q, const void* k, const void* v,
                          const int32_t* pos_thw, const float* gamma_q, const float* gamma_k,
                          const int32_t* cu_seqlens, int32_t max_seqlen, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- Backward pass ---------------------------------------------------------
 *
 * Gradients for training (LoRA on the attention projections with gradient
 * checkpointing, as the SimpleTuner quickstart trains the Ideogram 4 DiT): given
 * the forward's out and lse (mrope_attn_fwd with a non-NULL lse) and the
 * upstream gradient dout, writes dq, dk, dv (the gradients of sum(dout * out)
 * w.r.t. q, k, v; zero rows for padded text slots) and, when not NULL,
 * dgamma_q and dgamma_k (fp32 with gamma's shape: [D] summed over every
 * valid row and head, or with gamma_per_head [H, D] with row h summed over
 * head h's valid rows; the sums run in a fixed order, so results are
 * reproducible). bf16 with
 * head_dim 128 only (else MRA_ERR_UNSUPPORTED). dout has out's strides
 * (o_stride); dq, dk, dv have q's, k's and v's strides; all four must be
 * 16-byte aligned and must not overlap the inputs or each other. The packed
 * (cu_seqlens) layout's backward is mrope_attn_bwd_varlen below. */
size_t mrope_attn_bwd_workspace_size(const mra_desc* desc);

int mrope_attn_bwd(const mra_desc* desc, const void* q, const void* k, const void* v,
                   const int32_t* pos_thw, const float* gamma_q, const float* gamma_k,
                   const int32_t* seq_lens, const void* out, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, float* dgamma_q, float* dgamma_k,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Backward of mrope_attn_fwd_varlen (packed variable-length sequences; the
 * layout, cu_seqlens, max_seqlen and lse [H, seq] as described there): the
 * same gradients as mrope_attn_bwd, each sequence attending to its own
 * tokens only; dgamma sums every sequence's rows. desc->text_pad must be 0
 * and max_seqlen 0..seq (MRA_ERR_SHAPE); bf16 with head_dim 128 only
 * (MRA_ERR_UNSUPPORTED). Tokens outside every sequence are not written in
 * dq, dk, dv. batch, seq or max_seqlen 0: nothing is done. */
size_t mrope_attn_bwd_varlen_workspace_size(const mra_desc* desc, int32_t max_seqlen);

int mrope_attn_bwd_varlen(const mra_desc* desc, const void* q, const void* k, const void* v,
                          const int32_t* pos_thw, const float* gamma_q, const float* gamma_k,
                          const int32_t* cu_seqlens, int32_t max_seqlen, const void* out,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          float* dgamma_q, float* dgamma_k, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ---- fp8 QKV projection with the norm/rotation epilogue ------------------
 *
 * The checkpoint's attention projection is one fused weight [3 * H * D, hidden]
 * with the Q, K and V rows stacked, stored as float8 e4m3 (OCP E4M3, the
 * float8_e4m3fn type) with one fp32 scale per output row: the real weight is
 * fp8 value * scale (unsloth commit log for the Ideogram 4 backend, the fp8
 * loader commit). mrope_qkv_proj computes y = x W^T for bf16 activations x
 * [tokens, hidden] (fp32 accumulation, the row scale applied to the sums) and
 * writes the attention's operands:
 *   q_out = bf16(softmax_scale * log2(e) * rope(rmsnorm(y_q) * gamma_q))  (Q'')
 *   k_out = bf16(rope(rmsnorm(y_k) * gamma_k))                            (K')
 *   v_out = bf16(y_v)
 * per head, with the rotation and norm of mrope_attn_fwd (pos_thw [tokens, 3]).
 * Feed them to mrope_attn_fwd with kprologue = MRA_KPRO_NONE and the same
 * softmax_scale. head_dim 128 only; hidden a positive multiple of 64.
 * Outputs are [tokens, H, D] views with the given token and head strides
 * (multiples of 8 elements, 16-byte aligned bases, no overlap). */
typedef struct {
  int32_t tokens;         /* rows of x (B * S for a padded batch), >= 0 */
  int32_t hidden;         /* columns of x, multiple of 64 */
  int32_t heads;          /* H >= 1 */
  int32_t head_dim;       /* 128 */
  int32_t section[3];     /* rotary pairs driven by t, h, w; sum == D/2 */
  float theta;            /* rotary base, > 0 */
  float eps;              /* RMSNorm epsilon, >= 0 */
  float softmax_scale;    /* > 0, or <= 0 for 1/sqrt(D) */
  int64_t x_stride;       /* elements between rows of x (multiple of 8) */
  int64_t q_stride[2];    /* token, head strides of q_out (elements) */
  int64_t k_stride[2];
  int64_t v_stride[2];
  int32_t rope_pairs;     /* mra_rope_pairs */
  int32_t gamma_per_head; /* 0: gamma_q, gamma_k are [D]; 1: [H, D] */
} mra_qkv_desc;

size_t mrope_qkv_proj_workspace_size(const mra_qkv_desc* desc);

int mrope_qkv_proj(const mra_qkv_desc* desc, const void* x, const uint8_t* w8, const float* w_scale,
                   const int32_t* pos_thw, const float* gamma_q, const float* gamma_k,
                   void* q_out, void* k_out, void* v_out, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Static, human-readable text for a status code. */
const char* mrope_attn_status_string(int status);

/* The hipError_t behind the calling thread's most recent MRA_ERR_HIP (0 when
 * this thread has had none), and in *name (when name is not NULL) HIP's
 * static name for it. Each call clears a HIP error still pending on its
 * thread from earlier, unrelated work before its own launches, so the value
 * is the call's own. */
int mrope_attn_last_hip_error(const char** name);

/* ABI version of this header (major * 100 + minor). */
int mrope_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MROPE_ATTN_H */
