/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention forward library
 * (libattn_mi355x.so).
 *
 * The operation is the FlashAttention-2 style forward pass that the four
 * source pages share: for each query row i of a (batch, head),
 *
 *     S_ij   = sm_scale * <q_i, k_j>
 *     O_i    = sum_j softmax_j(S_i.) v_j
 *     LSE_i  = log sum_j exp(S_ij)                      (natural log, fp32)
 *
 * computed in one streaming pass over key/value tiles with an online softmax
 * (Triton fused-attention tutorial with JVP, "_06_fused_attention_blockptr_jvp.py":
 * _attn_fwd and _attn_fwd_inner; "Flash Attention v2 with JVP", flm/utils/jvp.py:
 * _attn_fwd and its epilogue).  The LSE follows the JVP page, which stores the
 * natural-log value in fp32.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *   every buffer; the library never allocates or frees device memory.
 * - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *   default stream).  Calls are asynchronous: nothing synchronises the host.
 * - Strides are in ELEMENTS.  The innermost (head-dim) stride must be 1.
 *   Base pointers must be 16-byte aligned and every other stride a multiple of
 *   16 bytes (8 bf16 or fp16 elements, 4 fp32 elements), and the row (n)
 *   stride of K and V at most 2^22 elements; contiguous torch tensors
 *   satisfy this.  Anything else is ATTN_ERR_UNSUPPORTED.
 * - Tangent tensors (JVP) share the strides of their primals, and tO shares
 *   the strides of O (as the JVP page's wrapper requires).
 * - Supported head dims: 16, 32, 64, 128 and 256 everywhere (the forward,
 *   plain, biased or jagged, either side of attn_fwd_dv, the JVP and the
 *   backward).  dtype ATTN_BF16 (ATTN_FP16) computes
 *   the products on bf16 (fp16) MFMA with fp32 accumulation and rounds O/tO to
 *   the input format (RNE); ATTN_FP32 computes everything in fp32.  LSE is
 *   always fp32.
 * - sm_scale must be finite and >= 0 (every page uses a positive scale,
 *   by default D^-0.5).
 * - Sizes: Nq, Nkv, total_len and num_seqs + 1 at most 2^31 - 1, and
 *   B * H at most 2^31 - 1 (the device indexes rows, tiles and (batch, head)
 *   pairs with 32-bit integers); every launch grid within 2^31 - 1 blocks (for
 *   the backward: B * H * Nq, or H * total_len, at most 8 (2^31 - 1) rows);
 *   larger extents are ATTN_ERR_INVALID, and the workspace-size functions
 *   return 0 for extents they cannot serve.
 * - A query row with no key to attend (Nkv == 0, or a jagged row beyond
 *   max_seq_len inside its sequence) gets O = 0, tO = 0 and LSE = -inf.
 * - All argument checks happen on the host before anything is enqueued; a
 *   failed check enqueues nothing and returns a negative status.
 * - The library keeps no mutable global state beyond a per-process cache of
 *   kernel attributes and device addresses, so concurrent calls on different
 *   streams are safe -- except jagged_attn_fwd_noalloc, whose calls share one
 *   static device array per GPU (see there).
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points (the library is built with hidden visibility). */
#define ATTN_API __attribute__((visibility("default")))

/* Status codes (every entry point returns one). */
enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = -1,      /* null pointer with work to do, negative or oversized size, bad stride, bad scale */
  ATTN_ERR_UNSUPPORTED = -2,  /* head dim not supported by the call, unknown dtype, misaligned pointer/stride */
  ATTN_ERR_CAUSAL_SHAPE = -3, /* causal with Nq != Nkv (the mask is top-left aligned) */
  ATTN_ERR_WORKSPACE = -4,    /* workspace missing or too small; for jagged_attn_fwd_noalloc, a plan beyond its static scratch */
  ATTN_ERR_HIP = -5           /* the HIP runtime reported an error while enqueuing */
};

/*
 * Element type of q, k, v (and tangents), o, to.  ATTN_BF16 and ATTN_FP16
 * run on the 16-bit MFMA kernels (P and H rounded to the input format for
 * their products, fp32 accumulation); ATTN_FP32 runs an fp32 vector-ALU
 * kernel with no rounding below fp32.  LSE is fp32 in every case.
 */
typedef enum attn_dtype { ATTN_BF16 = 0, ATTN_FP32 = 1, ATTN_FP16 = 2 } attn_dtype;

/* Element strides of a dense [B, H, N, D] view. */
typedef struct attn_strides4 { int64_t b, h, n, d; } attn_strides4;

/* Element strides of a jagged [H, total_len, D] view. */
typedef struct attn_strides3 { int64_t h, t, d; } attn_strides3;

/*
 * Dense attention forward (tutorial page: _attn_fwd with ENABLE_JVP off;
 * JVP page: _attn_fwd).
 *   q  [B, H, Nq,  D]   k, v [B, H, Nkv, D]   (dtype)
 *   o  [B, H, Nq,  D]   written (dtype)
 *   lse [B, H, Nq] contiguous fp32, written (natural log)
 *   causal != 0: query i attends key j only when j <= i (top-left mask,
 *   the pages' on-band stage); requires Nq == Nkv.
 * B*H*Nq == 0 is a no-op returning ATTN_OK.
 */
ATTN_API int attn_fwd(attn_dtype dtype,
             const void* q, attn_strides4 q_strides,
             const void* k, attn_strides4 k_strides,
             const void* v, attn_strides4 v_strides,
             void* o, attn_strides4 o_strides,
             float* lse,
             int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
             float sm_scale, int causal, void* stream);

/* Kind of the score operand of attn_fwd_bias. */
typedef enum attn_bias_kind {
  ATTN_BIAS_ADD = 1,  /* additive float bias, element type = dtype */
  ATTN_BIAS_MASK = 2  /* uint8 boolean mask: 0 removes the key, nonzero keeps it */
} attn_bias_kind;

/*
 * Dense attention forward with an additive bias or a boolean mask on the
 * scores (flash attention with bias page: _attn_fwd_inner, _attn_fwd and
 * the wrapper _flash_attn_fwd):
 *     S_ij = sm_scale <q_i, k_j> + bias_ij        (ATTN_BIAS_ADD)
 *     S_ij = -inf where mask_ij == 0              (ATTN_BIAS_MASK)
 * combined with the causal mask when causal != 0; O and LSE as attn_fwd.
 *   bias          [B, H, Nq, Nkv] read through bias_strides = {b, h, n, d}
 *                 (n: query row, d: key).  d must be 1; b, h and n may be 0
 *                 to broadcast, e.g. {0, 0, 0, 1} for one key-padding row
 *                 shared by every query, or {Nq*Nkv, 0, Nkv, 1} for a
 *                 per-batch bias shared by the heads.
 *   ATTN_BIAS_ADD: element type `dtype`, in the units of the scores (natural
 *                 log: the page's wrapper divides by ln 2 for its base-2
 *                 kernel; the result is the same).  Values must be finite or
 *                 -inf (which removes the key); +inf and NaN give NaN rows.
 *                 Base 16-byte aligned, b/h/n strides multiples of 16 bytes.
 *   ATTN_BIAS_MASK: uint8; base 8-byte aligned, b/h/n strides multiples of 8.
 *   A row left with no key gets O = 0, LSE = -inf (the page's additive -1e6
 *   mask would instead attend every key of such a row).
 *   bias may be NULL only when Nkv == 0.  Other arguments as attn_fwd.
 */
ATTN_API int attn_fwd_bias(attn_dtype dtype,
                  const void* q, attn_strides4 q_strides,
                  const void* k, attn_strides4 k_strides,
                  const void* v, attn_strides4 v_strides,
                  void* o, attn_strides4 o_strides,
                  float* lse,
                  const void* bias, attn_bias_kind bias_kind, attn_strides4 bias_strides,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                  float sm_scale, int causal, void* stream);

/*
 * Dense attention forward fused with its forward-mode JVP (tutorial page:
 * _attn_fwd_inner / _attn_fwd with ENABLE_JVP; JVP page: _attn_fwd_inner and
 * the epilogue).  With tangents (tq, tk, tv) of the inputs, it writes the
 * output tangent
 *     tS = sm_scale (tq k^T + q tk^T),  tP = P * (tS - rowsum(P * tS)),
 *     to = tP v + P tv
 * alongside o and lse in the same pass.  Tangents use the primal strides;
 * `to` uses o_strides.
 *   tlse  optional [B, H, Nq] contiguous fp32 (NULL: not written): the
 *         tangent of lse, rowsum(P * tS) (0 for a row without keys) -- the
 *         term that merging JVPs of key-sharded attention needs.
 * Other arguments as attn_fwd.
 */
ATTN_API int attn_fwd_jvp(attn_dtype dtype,
                 const void* q, const void* k, const void* v,
                 const void* tq, const void* tk, const void* tv,
                 attn_strides4 q_strides, attn_strides4 k_strides, attn_strides4 v_strides,
                 void* o, void* to, attn_strides4 o_strides,
                 float* lse, float* tlse,
                 int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                 float sm_scale, int causal, void* stream);

/*
 * Dense forward (and, with tangents, its JVP) whose values have their own
 * head dim (JVP page: _attention.forward takes d_v != d_qk, and _test_jvp_ca
 * checks it):
 *   q, tq [B, H, Nq, Dqk]   k, tk [B, H, Nkv, Dqk]   v, tv [B, H, Nkv, Dv]
 *   o, to [B, H, Nq, Dv]    lse, tlse [B, H, Nq]
 * tq == NULL: the plain forward of attn_fwd (tk, tv, to and tlse must be
 * NULL too); otherwise the fused JVP of attn_fwd_jvp (tlse optional).
 * Dqk and Dv each in {16, 32, 64, 128, 256}; with Dqk == Dv this is
 * exactly attn_fwd / attn_fwd_jvp.  Some wide combinations run as several
 * launches over slices of the value columns, each recomputing the scores
 * (the same bits as one launch).  sm_scale is the caller's (the page's default is
 * Dqk^-0.5).  Other arguments, checks and errors as attn_fwd_jvp.
 */
ATTN_API int attn_fwd_dv(attn_dtype dtype,
                const void* q, const void* k, const void* v,
                const void* tq, const void* tk, const void* tv,
                attn_strides4 q_strides, attn_strides4 k_strides, attn_strides4 v_strides,
                void* o, void* to, attn_strides4 o_strides,
                float* lse, float* tlse,
                int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t Dqk, int64_t Dv,
                float sm_scale, int causal, void* stream);

/*
 * Bytes of device workspace jagged_attn_fwd needs (host function, no GPU
 * access).  Returns 0 for invalid sizes.
 */
ATTN_API size_t jagged_attn_workspace_bytes(int64_t num_seqs, int64_t total_len);

/*
 * Jagged multi-head attention forward (FBGEMM SLL page,
 * triton_multi_head_jagged_flash_attention.py:
 * _multi_head_jagged_flash_attention_fwd_kernel and the public wrapper).
 *   q, k, v, o  [H, total_len, D]  (dtype)
 *   lse         [H, total_len] contiguous fp32, written
 *   offsets     DEVICE int64 [num_seqs + 1]: offsets[0] = 0, non-decreasing,
 *               offsets[num_seqs] = total_len.  Sequence s owns rows
 *               [offsets[s], offsets[s+1]).  Not checked (reading them would
 *               need a host sync); out-of-range values are clamped so that no
 *               access leaves the buffers, with unspecified results.
 *   Only the first min(len_s, max_seq_len) rows of a sequence take part, as
 *   queries and as keys; its later rows get O = 0, LSE = -inf.  There is no
 *   attention across sequences.  causal != 0 masks key j > query i within a
 *   sequence.  Unlike the SLL page, O is not divided by max_seq_len, and the
 *   caller passes sm_scale (1.0 reproduces that page's unscaled logits).
 *   workspace   DEVICE scratch of at least jagged_attn_workspace_bytes(...)
 *               bytes, used for the on-device tile plan; its contents on entry
 *               are ignored.  Calls that share a workspace must not overlap.
 */
ATTN_API int jagged_attn_fwd(attn_dtype dtype,
                    const void* q, attn_strides3 q_strides,
                    const void* k, attn_strides3 k_strides,
                    const void* v, attn_strides3 v_strides,
                    void* o, attn_strides3 o_strides,
                    float* lse,
                    const int64_t* offsets,
                    int64_t num_seqs, int64_t H, int64_t total_len, int64_t D,
                    int64_t max_seq_len, float sm_scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the static device scratch behind jagged_attn_fwd_noalloc (one
 * copy per GPU the library runs on, held until the process ends).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (1u << 20)

/*
 * jagged_attn_fwd for callers that cannot allocate device memory (code under
 * stream or graph capture, serving loops and harnesses that forbid
 * allocation): the same arguments and results without a workspace.  The tile
 * plan goes to a static device array of the library instead, so the call
 * allocates nothing and calls no allocating routine.
 *   Limit: the plan must fit ATTN_NOALLOC_SCRATCH_BYTES, i.e.
 *   16 + 8 * floor((total_len + (BM - 1) * num_seqs) / BM) <= 2^20 bytes with
 *   BM = 128 query rows per tile for bf16 and fp16, 64 for fp32: at most
 *   131070 query tiles (total_len up to 16.7M rows in bf16 with few
 *   sequences, or up to 131070 short sequences); larger inputs return
 *   ATTN_ERR_WORKSPACE before anything is enqueued.
 *   Every call on a GPU shares that GPU's array and leaves its plan there:
 *   calls that overlap on one GPU (on different streams, or from different
 *   threads) race and must be serialised by the caller; calls on different
 *   GPUs do not interact.  Nothing in the array needs clearing between calls.
 */
ATTN_API int jagged_attn_fwd_noalloc(attn_dtype dtype,
                    const void* q, attn_strides3 q_strides,
                    const void* k, attn_strides3 k_strides,
                    const void* v, attn_strides3 v_strides,
                    void* o, attn_strides3 o_strides,
                    float* lse,
                    const int64_t* offsets,
                    int64_t num_seqs, int64_t H, int64_t total_len, int64_t D,
                    int64_t max_seq_len, float sm_scale, int causal,
                    void* stream);

/*
 * Bytes of device workspace attn_bwd needs (host function, no GPU access):
 * two fp32 values per query row.  Returns 0 for invalid sizes.
 */
ATTN_API size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq);

/*
 * Dense attention backward: the gradients of attn_fwd's output o for a given
 * d_o = dL/do (tutorial page: _attn_bwd_preprocess, _attn_bwd_dkdv,
 * _attn_bwd_dq and _attn_bwd):
 *     delta_i = sum_d o_id d_o_id,   P = exp(sm_scale q k^T - lse)  (0 where masked),
 *     dv = P^T d_o,   dP = d_o v^T,   dS = P * (dP - delta),
 *     dq = sm_scale dS k,   dk = sm_scale dS^T q.
 *   q, o, d_o, dq  [B, H, Nq, D]   k, v, dk, dv  [B, H, Nkv, D]  (bf16 or fp16)
 *   lse            [B, H, Nq] contiguous fp32: the natural-log LSE that
 *                  attn_fwd wrote for these q, k, v (a row with LSE = -inf
 *                  gets dq = 0 and adds nothing to dk, dv)
 *   o              the forward's output (delta is formed from it, as the page does)
 *   dq, dk, dv     written (every element; rows with no attended key get 0)
 *   workspace      DEVICE scratch of at least attn_bwd_workspace_bytes(B, H, Nq)
 *                  bytes, 16-byte aligned; contents on entry are ignored.
 *                  Calls that share a workspace must not overlap.
 * Strides, alignment, sm_scale, causal (Nq == Nkv) and D in {16, 32, 64, 128, 256} as for
 * attn_fwd.  P and dS are rounded to the input format for their products,
 * with fp32 accumulation.  Each output element is written by exactly one
 * thread: the result is deterministic.  ATTN_FP32 returns ATTN_ERR_UNSUPPORTED.  Three
 * kernels are enqueued on `stream`; B*H*(Nq+Nkv) == 0 is a no-op.
 */
ATTN_API int attn_bwd(attn_dtype dtype,
             const void* q, attn_strides4 q_strides,
             const void* k, attn_strides4 k_strides,
             const void* v, attn_strides4 v_strides,
             const void* o, attn_strides4 o_strides,
             const void* d_o, attn_strides4 do_strides,
             const float* lse,
             void* dq, attn_strides4 dq_strides,
             void* dk, attn_strides4 dk_strides,
             void* dv, attn_strides4 dv_strides,
             int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
             float sm_scale, int causal,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense attention backward with the score operand of attn_fwd_bias (flash
 * attention with bias page: _attn_bwd_dkdv, _attn_bwd_dq and
 * _flash_attn_bwd): P is recomputed as exp(sm_scale q k^T + bias - lse)
 * (ATTN_BIAS_ADD) or with the masked keys removed (ATTN_BIAS_MASK), and the
 * gradients are those of attn_bwd.  bias, bias_kind and bias_strides as for
 * attn_fwd_bias, and lse must be what attn_fwd_bias wrote with that operand.
 *   dbias   optional (NULL: not written) gradient of the bias, dS =
 *           P * (dP - delta), [B, H, Nq, Nkv] in the input element type
 *           through dbias_strides = {b, h, n, d}: d must be 1, no stride may be
 *           0 where its extent exceeds 1 and distinct elements must not
 *           overlap; base 16-byte aligned, b/h/n strides multiples of 16
 *           bytes.  Every element is written, 0 for masked pairs.  With a
 *           broadcast bias the caller sums dbias over the broadcast dims.
 *           Only with ATTN_BIAS_ADD (a mask has no gradient).
 * bf16 or fp16; other arguments, checks and errors as attn_bwd.
 */
ATTN_API int attn_bwd_bias(attn_dtype dtype,
                  const void* q, attn_strides4 q_strides,
                  const void* k, attn_strides4 k_strides,
                  const void* v, attn_strides4 v_strides,
                  const void* o, attn_strides4 o_strides,
                  const void* d_o, attn_strides4 do_strides,
                  const float* lse,
                  const void* bias, attn_bias_kind bias_kind, attn_strides4 bias_strides,
                  void* dbias, attn_strides4 dbias_strides,
                  void* dq, attn_strides4 dq_strides,
                  void* dk, attn_strides4 dk_strides,
                  void* dv, attn_strides4 dv_strides,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                  float sm_scale, int causal,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace jagged_attn_bwd needs (host function, no GPU
 * access): the tile plan plus two fp32 values per row of every head.
 * Returns 0 for invalid sizes.
 */
ATTN_API size_t jagged_attn_bwd_workspace_bytes(int64_t num_seqs, int64_t H, int64_t total_len);

/*
 * Jagged multi-head attention backward: the gradients of jagged_attn_fwd's
 * output for a given d_o (FBGEMM SLL page,
 * triton_multi_head_jagged_flash_attention.py:
 * _multi_head_jagged_flash_attention_bwd_preprocess_kernel,
 * _multi_head_jagged_flash_attention_bwd_kernel and
 * multi_head_jagged_flash_attention_bwd), with the steps of attn_bwd applied
 * to each sequence (delta from this library's O, which is not divided by
 * max_seq_len).
 *   q, k, v, o, d_o, dq, dk, dv  [H, total_len, D]  (bf16 or fp16)
 *   lse        [H, total_len] contiguous fp32: what jagged_attn_fwd wrote
 *   offsets    as jagged_attn_fwd (DEVICE int64 [num_seqs + 1], not checked,
 *              clamped so that no access leaves the buffers)
 *   Within sequence s only the first min(len_s, max_seq_len) rows take part,
 *   as queries and as keys; dq, dk and dv of its later rows are written as 0.
 *   workspace  DEVICE scratch of at least jagged_attn_bwd_workspace_bytes(...)
 *              bytes, 16-byte aligned; contents on entry are ignored.  Calls
 *              that share a workspace must not overlap.
 * Strides, alignment, sm_scale and D as jagged_attn_fwd; causal masks key
 * j > query i within a sequence.  Every element of dq, dk, dv inside a
 * sequence is written once by one thread (deterministic); rows outside every
 * sequence are not touched.  ATTN_FP32 returns ATTN_ERR_UNSUPPORTED.  Four
 * kernels are enqueued on `stream` (plan, prep, dQ, dK/dV).
 */
ATTN_API int jagged_attn_bwd(attn_dtype dtype,
                    const void* q, attn_strides3 q_strides,
                    const void* k, attn_strides3 k_strides,
                    const void* v, attn_strides3 v_strides,
                    const void* o, attn_strides3 o_strides,
                    const void* d_o, attn_strides3 do_strides,
                    const float* lse,
                    void* dq, attn_strides3 dq_strides,
                    void* dk, attn_strides3 dk_strides,
                    void* dv, attn_strides3 dv_strides,
                    const int64_t* offsets,
                    int64_t num_seqs, int64_t H, int64_t total_len, int64_t D,
                    int64_t max_seq_len, float sm_scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text for a status code (host, static storage). */
ATTN_API const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */
