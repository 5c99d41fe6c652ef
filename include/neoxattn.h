/*
 * neoxattn.h -- C ABI of libneoxattn: exact causal multi-head attention with
 * GPT-NeoX rotary position embedding (rotate-half, optionally partial), in a
 * tiled IO-aware form, forward and backward, on AMD MI355X (gfx950).
 *
 * What is computed.  For every batch row b and head h, with positions
 * t = 0..S-1 and R_t the rotary matrix below:
 *     q~_i = R_i q_i,   k~_j = R_j k_j                        (v is not rotated)
 *     s_ij = softmax_scale * (q~_i . k~_j) + bias_ij
 *     lse_i = log sum_{j allowed} exp(s_ij)        (natural log, fp32)
 *     o_i   = sum_{j allowed} exp(s_ij - lse_i) v_j
 * allowed(i, j) = (causal == 0 or j <= i) and doc(i) == doc(j).
 * The attention is exact: the GPT-NeoX pages state that FlashAttention-2 keeps
 * the mathematical result and changes only tiling and memory traffic, with
 * O(n) instead of O(n^2) memory ("GPT-NeoX 开源训练框架深度解读", section
 * "问题二：注意力计算太慢").  No S x S matrix is ever stored.
 *
 * Rotary (NeoX style, on both Q and K: "FasterTransformer GPT-NeoX 推理指南",
 * GptNeoX.h facts neox_rotary_style_ and section "模型配置", rotary_embedding
 * 24 of size_per_head 96): with half = rotary_dim / 2 and, for p < half,
 * theta_{t,p} = t * rope_base^(-2p / rotary_dim):
 *     y_p        = x_p cos(theta) - x_{p+half} sin(theta)
 *     y_{p+half} = x_{p+half} cos(theta) + x_p sin(theta)
 *     y_d        = x_d                                  for d >= rotary_dim.
 * ALiBi (the alternative position scheme, "GPT-NeoX 开源训练框架深度解读",
 * section "架构创新"): bias_ij = -slope_h * (i - j), added after the scaling,
 * default slope_h = 2^(-8 (h+1) / H).  With RoPE the bias is 0.
 *
 * Conventions for every entry point:
 *  - Tensors q, k, v, o, dout, dq, dk, dv are [B, H, S, D] with the head dim
 *    contiguous; by default fully contiguous, otherwise strided (see
 *    neox_attn_args.strides).  lse is [B, H, S] contiguous fp32.
 *  - Every pointer argument that names tensor data is a DEVICE pointer owned
 *    by the caller; the library keeps no pointer past the call.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work is enqueued on it and the call returns without waiting.
 *  - Arguments are validated before any device work; a failed validation
 *    returns a negative status and enqueues nothing.  Launch failures return
 *    NEOX_E_LAUNCH.  Faults inside kernels surface at the caller's next
 *    synchronisation.  Outputs are undefined after an error.
 *  - Supported: D in {64, 96, 128}; 0 <= rotary_dim <= D, rotary_dim even;
 *    rope_base > 0 and finite; softmax_scale > 0 and finite; B, H, S >= 1;
 *    B*H*S < 2^31; tensor base pointers 16-byte aligned; row strides multiples
 *    of 8 elements (bf16, fp16) or 4 elements (fp32), and at most 2^22
 *    elements between consecutive rows (NEOX_E_UNSUPPORTED beyond).
 *  - The compute calls (forward, backward, decode, FP8 forward) allocate
 *    nothing and never wait: every buffer is the caller's, and the rotary
 *    cos/sin table of a (rotary_dim, rope_base) pair -- the per-layer
 *    inv_freq buffer of the checkpoint ("FasterTransformer GPT-NeoX 推理指南",
 *    the attention.rotary_emb.inv_freq tensor of the converted model) turned
 *    into cos/sin of t * inv_freq -- must have been built beforehand by
 *    neox_rope_table_prepare() on the calling device for at least the
 *    sequence length (the decode cache capacity) of the call.  A call that
 *    needs a table that has not been prepared returns NEOX_E_NOT_PREPARED
 *    and enqueues nothing.  Calls with rotary_dim = 0, ALiBi or no position
 *    scheme need no table.
 */
#ifndef NEOXATTN_H
#define NEOXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NEOX_OK 0
#define NEOX_E_ARG (-1)         /* null pointer, bad size, bad scalar, bad enum */
#define NEOX_E_UNSUPPORTED (-2) /* valid but not implemented (e.g. D = 80) */
#define NEOX_E_ALIGN (-3)       /* base pointer or row stride misaligned */
#define NEOX_E_WORKSPACE (-4)   /* workspace NULL or smaller than required */
#define NEOX_E_LAUNCH (-5)      /* a kernel launch failed */
#define NEOX_E_DEVICE (-6)      /* no usable gfx950 device / HIP runtime error */
#define NEOX_E_ALLOC (-7)       /* rotary table allocation failed (neox_rope_table_prepare) */
#define NEOX_E_NOT_PREPARED (-8) /* rotary table not prepared: call neox_rope_table_prepare */
#define NEOX_E_TOO_LARGE (-9)   /* beyond NEOX_DECODE_SCRATCH_BYTES (no-allocation decode) */

/* Size of the fixed device array behind neox_rope_attn_decode_noalloc. */
#define NEOX_DECODE_SCRATCH_BYTES ((size_t)8 << 20)

/* Storage type of q, k, v, o, dout (and of dq, dk, dv unless out_dtype says fp32). */
#define NEOX_F32 0
#define NEOX_BF16 1
#define NEOX_F16 2 /* IEEE half ("FasterTransformer GPT-NeoX 推理指南": FP16 inference) */

/* Position scheme. */
#define NEOX_POS_NONE 0
#define NEOX_POS_ROPE 1
#define NEOX_POS_ALIBI 2

/* Output type selector of the _ex calls. */
#define NEOX_OUT_SAME 0 /* outputs in the input storage type */
#define NEOX_OUT_F32 1  /* outputs in fp32 */

/* Element strides of one [B, H, S, D] tensor whose head dim is contiguous. */
typedef struct neox_strides {
  int64_t batch;
  int64_t head;
  int64_t seq;
} neox_strides;

/*
 * Arguments of the _ex calls.
 *  pos           NEOX_POS_NONE / NEOX_POS_ROPE / NEOX_POS_ALIBI.
 *  rotary_dim,   used when pos == NEOX_POS_ROPE (rotary_dim may then be 0,
 *  rope_base     which is plain attention); must be 0 otherwise.
 *  alibi_slopes  device fp32 [H] or NULL for 2^(-8 (h+1) / H); pos == ALIBI only.
 *  doc_offsets   device int32 [B][n_docs + 1] or NULL (one document per row).
 *                Row b lists document starts: offsets[b][0] = 0, non-decreasing,
 *                offsets[b][n_docs] = S; equal neighbours are empty documents.
 *                Tokens of different documents never attend to each other.
 *                Values are not read by the host; neox_check_doc_offsets()
 *                validates a host copy.  Kernels clamp what they read, so
 *                malformed offsets give undefined values but no stray access.
 *  out_dtype     NEOX_OUT_SAME or NEOX_OUT_F32, for o (fwd) and dq, dk, dv (bwd).
 *  strides       NULL for contiguous tensors, else 8 entries in the order
 *                q, k, v, o, dout, dq, dk, dv (the fwd reads the first 4).
 *  phase_events  NULL, or hipEvent_t handles (as void*) that the call records
 *                on `stream` around its kernels, for timing by the caller: the
 *                forward records [0] before its first kernel, [1] after the q/k
 *                rotation pass (right after [0] when none runs) and [2] after
 *                the attention kernel; the backward records [0] before its
 *                first kernel, [1] after the preprocess kernel (right after
 *                [0] when none runs), [2] after the 16-bit paths' dQ kernel
 *                (which also forms the row terms) or after the fp32 path's
 *                two main kernels, and [3] at its end (after the dK/dV kernel,
 *                or the fp32 path's dq finalize).  The events are owned by
 *                the caller.
 *  reuse_rotated_qk  0 or 1, backward only (16-bit storage with rotary_dim > 0;
 *                ignored otherwise).  1 promises that the backward workspace
 *                already holds the rotated rows q~ and k~ because it was passed
 *                as the workspace of the forward call with the same q, k and
 *                rotary arguments and nothing wrote to it since; the backward
 *                then skips recomputing them (saving a read of q, k and a
 *                write of q~, k~).  The results are bit-identical to 0.
 */
typedef struct neox_attn_args {
  int B, H, S, D;
  int dtype;
  int pos;
  int rotary_dim;
  float rope_base;
  const float* alibi_slopes;
  int causal;
  float softmax_scale;
  const int32_t* doc_offsets;
  int n_docs;
  int out_dtype;
  const neox_strides* strides;
  void* const* phase_events;
  int reuse_rotated_qk;
} neox_attn_args;

/* Text of a status code (static storage, never NULL).  The codes name the
 * argument rules stated above. */
const char* neox_status_str(int status);

/*
 * Bytes of the optional forward workspace: two 16-bit [B, H, S, D] buffers that
 * receive the rotated rows q~ = R q and k~ = R k (NeoX rotate-half with each
 * row's own position; "FasterTransformer GPT-NeoX 推理指南", section
 * "模型配置": both Q and K are rotated), written by one row pass so that the
 * attention kernel itself does no rotation.  2 * (B*H*S*D*2 rounded up to
 * 256) bytes.  Returns 0 for sizes that are invalid (<= 0) or overflow.
 */
size_t neox_rope_attn_fwd_workspace_size(int B, int H, int S, int D);

/*
 * Forward of causal self-attention with NeoX rotary embedding, in the tiled
 * exact form with an online softmax ("GPT-NeoX 开源训练框架深度解读",
 * section on attention speed: FlashAttention).  q, k, v: [B, H, S, D] of
 * `dtype` (read only).  o: [B, H, S, D] of `dtype` (written).  lse: [B, H, S]
 * fp32 natural-log logsumexp of each row's allowed scores (written; the
 * backward needs it).  rotary_dim = 0 turns the rotation off.  Causal masking
 * when causal != 0.  workspace: NULL, or caller-owned device memory of at
 * least neox_rope_attn_fwd_workspace_size() bytes, 256-byte aligned,
 * overwritten by the call; it is used by the bf16 and fp16 paths with
 * rotary_dim > 0 (the faster path) and ignored otherwise.  Results do not
 * depend on whether a workspace is given beyond fp32 rounding order of the
 * rotation.
 */
int neox_rope_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int S, int D, int rotary_dim, float rope_base,
                       int causal, float softmax_scale, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Bytes of device workspace the backward needs.  The backward recomputes the
 * probabilities from lse instead of storing the S x S matrix -- the O(n)
 * memory of the tiled form ("GPT-NeoX 开源训练框架深度解读", section
 * "问题二：注意力计算太慢") -- so the workspace is linear in S: the rotated q
 * and k in the 16-bit storage type, [B, H, S, D] each (bf16 and fp16 paths;
 * placed first, exactly where the forward workspace holds them, so a
 * backward workspace also serves as the forward's -- see reuse_rotated_qk),
 * or over the same bytes an fp32 [B, H, S, D] dq accumulator (fp32 path),
 * then two fp32 [B, H, S] row terms (the softmax-gradient row sum and the
 * negated base-2 log-sum-exp); 256-byte aligned parts, B*H*S*(4D + 8) bytes
 * up to rounding for every dtype.  Returns 0 for sizes that are invalid
 * (<= 0) or overflow. */
size_t neox_rope_attn_bwd_workspace_size(int B, int H, int S, int D);

/*
 * Backward of the same attention (the pages' subject is training GPT-NeoX with
 * this attention: "GPT-NeoX 开源训练框架深度解读", section "问题二：注意力计算
 * 太慢").  With P_ij = exp(s_ij - lse_i), dP_ij = dout_i . v_j,
 * Delta_i = dout_i . o_i and dS_ij = P_ij (dP_ij - Delta_i):
 *     dv_j = sum_i P_ij dout_i
 *     dq_i = R_i^T softmax_scale sum_j dS_ij k~_j
 *     dk_j = R_j^T softmax_scale sum_i dS_ij q~_i
 * Inputs q, k, v, o, dout ([B, H, S, D], `dtype`) and lse (from the forward
 * with the same arguments) are read only.  dq, dk, dv ([B, H, S, D], `dtype`)
 * are written and must not alias the inputs.  workspace: device memory of at
 * least neox_rope_attn_bwd_workspace_size() bytes, 256-byte aligned, owned by
 * the caller, overwritten by the call (its contents afterwards are
 * unspecified).  Deterministic for every dtype: dq, dk and dv are each reduced
 * by one workgroup in a fixed order (no atomics).
 */
int neox_rope_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       int B, int H, int S, int D, int rotary_dim, float rope_base,
                       int causal, float softmax_scale, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Forward with ALiBi (the pages' alternative position scheme, "GPT-NeoX 开源训练
 * 框架深度解读", section "架构创新"), packed documents, strides (NeoX's fused
 * per-head [heads, 3, head_dim] QKV read in place, "FasterTransformer GPT-NeoX
 * 推理指南", the QKV weight conversion step) and output type (see
 * neox_attn_args); workspace as for neox_rope_attn_fwd. */
int neox_attn_fwd_ex(const neox_attn_args* args, const void* q, const void* k, const void* v,
                     void* o, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Backward counterpart of neox_attn_fwd_ex (same passages as neox_attn_fwd_ex
 * and neox_rope_attn_bwd); workspace as for neox_rope_attn_bwd. */
int neox_attn_bwd_ex(const neox_attn_args* args, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decoding (one new token per sequence against a key/value cache): the
 * token-by-token generation mode of the GPT-NeoX decoder ("FasterTransformer
 * GPT-NeoX 推理指南", section "背景").  The new token sits at position
 * t = cache_lens[b]; the cache already holds the rotated keys k~_0 .. k~_{t-1}
 * and the values of the earlier tokens of that sequence.
 *
 * Bytes of the decode workspace: fp32 partial results (running max, sum and
 * weighted value sum) of [B, H, ceil(cap / 256), D + 4], rounded up to 256
 * bytes.  Returns 0 for invalid sizes (<= 0, D > 4096) or overflow.
 */
size_t neox_rope_attn_decode_workspace_size(int B, int H, int D, int cap);

/*
 * One decoding step for every (batch row, head).  With t = cache_lens[b]:
 *     q~ = R_t q,  k~ = R_t k         (rotation as above, position t)
 *     k_cache[b, h, t] = k~,  v_cache[b, h, t] = v       (written)
 *     s_j = softmax_scale * (q~ . k_cache[b, h, j])      for j = 0 .. t
 *     lse = log sum_j exp(s_j),  o = sum_j exp(s_j - lse) v_cache[b, h, j]
 * which is row t of the causal forward over positions 0 .. t.
 *  q, k, v      device [B, H, D] of `dtype`, contiguous, the new token's raw
 *               projections (read only).
 *  k_cache,     device [B, H, cap, D] of `dtype`, contiguous; rows 0 .. t-1
 *  v_cache      are read, row t is written (keys stored rotated).
 *  cache_lens   device int32 [B]: tokens already cached per batch row, each in
 *               [0, cap - 1]; not read by the host.  Values outside are
 *               clamped into that range by the kernels (undefined results, no
 *               stray access).  The call does not update them: the caller
 *               increments them after the step.
 *  o            device [B, H, D] of `dtype` (written).
 *  lse          device fp32 [B, H], natural log (written).
 *  workspace    device memory of at least
 *               neox_rope_attn_decode_workspace_size(B, H, D, cap) bytes,
 *               256-byte aligned, owned by the caller, overwritten.
 * Supported: D in {64, 96, 128}; cap >= 1; B*H*cap < 2^31; 0 <= rotary_dim
 * <= D, even; pointers 16-byte aligned.  The rotary table must cover
 * positions 0 .. cap - 1 (neox_rope_table_prepare(cap, ...)).  Same status
 * codes as the other entry points; o and lse must not alias the inputs or
 * the cache.
 */
int neox_rope_attn_decode(const void* q, const void* k, const void* v, void* k_cache,
                          void* v_cache, const int32_t* cache_lens, void* o, float* lse,
                          int B, int H, int D, int cap, int rotary_dim, float rope_base,
                          float softmax_scale, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * neox_rope_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same step, the same kernels and the same results bit for
 * bit, with no workspace argument.  The chunk partials go to a fixed
 * NEOX_DECODE_SCRATCH_BYTES array that every device holds from the library's
 * first use of it until the process ends.  The caller still passes every
 * input and output (and prepares the rotary table, as for the other calls).
 * Accepts the problems whose neox_rope_attn_decode_workspace_size() is at
 * most NEOX_DECODE_SCRATCH_BYTES (for example B*H = 512 heads of D = 96 with
 * an 8192-row cache); larger ones return NEOX_E_TOO_LARGE before any work.
 * All calls on one device share its array: calls that may overlap on one
 * device (different streams without ordering between them) race and must be
 * serialised by the caller.  Nothing in the array needs to start at zero:
 * every partial a call reads is written earlier in the same call.  Other
 * status codes as for neox_rope_attn_decode (never NEOX_E_WORKSPACE).
 */
int neox_rope_attn_decode_noalloc(const void* q, const void* k, const void* v, void* k_cache,
                                  void* v_cache, const int32_t* cache_lens, void* o, float* lse,
                                  int B, int H, int D, int cap, int rotary_dim, float rope_base,
                                  float softmax_scale, int dtype, void* stream);

/*
 * FP8 forward: causal (or full) attention with q~, k~ and v stored as FP8 E4M3
 * codes (OCP format: bias 7, 3 mantissa bits, largest finite 448), one scale
 * per tensor: value = code x scale.  The GPT-NeoX stack computes in FP8
 * through Transformer Engine ("GPT-NeoX 开源训练框架深度解读", the TE image); in
 * that arrangement the rotation comes before quantisation, so q8 and k8 hold
 * the ROTATED projections (q~ = R q, k~ = R k, quantised by the caller).
 *  q8, k8, v8  device [B, H, S, D] E4M3 codes, contiguous (read only).
 *  o           device [B, H, S, D] bf16, or fp32 with out_dtype NEOX_OUT_F32.
 *  lse         device [B, H, S] fp32, natural log (written).
 * Both products run on the FP8 matrix cores with fp32 accumulation; the
 * probabilities are rounded to E4M3 (scaled by 2^4) for the P V product, so o
 * differs from exact attention over the dequantised inputs by at most about
 * 2^-4 of sum_j p_j |v_j| per element (plus the output rounding).
 * Supported: D in {64, 96, 128}; scales finite and > 0; pointers 16-byte
 * aligned; B*H*S < 2^31.  Same status codes as the other entry points.
 */
int neox_attn_fwd_fp8(const void* q8, const void* k8, const void* v8, float q_scale,
                      float k_scale, float v_scale, void* o, float* lse, int B, int H, int S,
                      int D, int causal, float softmax_scale, int out_dtype, void* stream);

/*
 * Host-side check of a HOST copy of doc_offsets ([B][n_docs + 1] int32), the
 * packed-document layout of neox_attn_args (documents packed into one
 * sequence, no attention across them; the pages leave packing open, the
 * document boundaries come with the workload):
 * returns NEOX_OK when every row starts at 0, never decreases and ends at S,
 * NEOX_E_ARG otherwise (or for a NULL pointer / bad sizes).  No device work.
 */
int neox_check_doc_offsets(const int32_t* host_offsets, int B, int n_docs, int S);

/* Kernel forms a call with given arguments runs (see neox_attn_plan). */
typedef struct neox_plan {
  int fp32_path;          /* fp32 storage: the vector-ALU kernels (no other field applies) */
  int fwd_rotation_pass;  /* forward: a row pass writes q~ = R q, k~ = R k to the workspace,
                             then the rotation-free attention kernel runs */
  int fwd_k_staging;      /* forward attention kernel's K tiles: 0 plain or pre-rotated,
                             1 rotary pairs 8 wide (rotary_dim % 16 == 0), 2 pairs 4 wide
                             (rotary_dim % 8 == 0), 3 every chunk through registers */
  int fwd_rotate_q;       /* forward attention kernel rotates Q~ as it loads it */
  int alibi;              /* the ALiBi forms of the kernels */
  int bwd_rotation_pass;  /* backward: rotates q and k into its workspace itself (no
                             rotated rows reused from the forward) */
} neox_plan;

/*
 * Which kernel forms the forward (with fwd_workspace = 1: a workspace given)
 * and the backward (its reuse_rotated_qk taken from *a) would launch for these
 * arguments -- the same host-side choice the launchers make -- without
 * touching any device.  The forms follow the rotation's place in the pages'
 * method (q and k rotated before attention, "FasterTransformer GPT-NeoX
 * 推理指南", the rotary_embedding field of the 20B configuration) and the
 * ALiBi alternative ("GPT-NeoX 开源训练框架深度解读", section "架构创新").
 * Returns NEOX_OK, NEOX_E_ARG (as for neox_attn_fwd_ex's arguments, NULL out)
 * or NEOX_E_UNSUPPORTED.
 */
int neox_attn_plan(const neox_attn_args* a, int fwd_workspace, neox_plan* out);

/*
 * Set-up call: builds the rotary cos/sin table of the current device for
 * positions 0..max_S-1, rotary_dim and rope_base (the checkpoint's
 * attention.rotary_emb.inv_freq, "FasterTransformer GPT-NeoX 推理指南", as
 * cos/sin of t * base^(-2p / rotary_dim), computed in double and stored as
 * fp32), allocating about max_S * rotary_dim * 4 bytes of device memory, and waits for
 * it (max_S is rounded up to a multiple of 256 positions).  Tables live until
 * the process ends; compute calls with S <= max_S and the same pair then find
 * it.  Not to be called under stream capture.
 * Returns NEOX_OK (also when a covering table exists), NEOX_E_ARG,
 * NEOX_E_ALLOC, NEOX_E_LAUNCH or NEOX_E_DEVICE.
 */
int neox_rope_table_prepare(int max_S, int rotary_dim, float rope_base);

#ifdef __cplusplus
}
#endif

#endif /* NEOXATTN_H */
