/*
 * attn_bwd.h -- C ABI of the MI355X (gfx950) fused attention backward library
 * (libattnbwd.so).
 *
 * Sources, cited by page title and section:
 *  [GQA-BWD] CK FMHA dispatcher example 34, "Backward Pass with GQA": the CPU
 *            backward reference (module docstring, cpu_bwd_gqa) and the
 *            FmhaProblem fields batch, nhead_q, nhead_k, seqlen_q, seqlen_k,
 *            hdim_q, hdim_v, scale.
 *  [DBIAS]   CK FMHA dispatcher example 28, "Backward Bias Gradient (dbias)
 *            FMHA": elementwise bias [H, Sq, Sk] broadcast over batch, dbias
 *            summed over batch (cpu_attention_bwd_dbias); bias/dbias feature
 *            flags of the backward kernel family.
 *  [SFMG]    CANN ops-transformer sparse_flash_mla_grad: "Formula" Phase 2/3
 *            (P, dP, dS, dQ, dKV, dSinks), "Prototype" (q, dout, attn_out,
 *            softmax_lse, sinks, softmax_scale, window left/right with -1 as
 *            unbounded), "Constraints" (consistent dtypes), "Deterministic
 *            Computation" (determinism is opt-in), bottom-right rule in
 *            "Example".
 *  [SINK]    CK FMHA dispatcher example 22, "Sink Token Attention FMHA":
 *            causal, causal + sink-token and sliding-window + sink-token masks.
 *  [RING]    "Ring attention for PyTorch" gist: the forward returns (out, lse);
 *            partial (o, lse) pairs are merged with logaddexp (_ring_fwd);
 *            per-chunk backward against the global o and lse (_ring_bwd);
 *            caller-allocated dq/dk/dv.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    keeps no state between calls and never allocates device memory.
 *  - Layout: Q, dO, O, dQ are [B, Hq, S_q, D]; K, V, dK, dV are
 *    [B, Hk, S_k, D]; the last dimension is contiguous and the other three
 *    are given as element strides {b, h, s}.  LSE and delta are contiguous
 *    fp32 [B, Hq, S_q].  bias and dbias are fp32 [Hq, S_q, S_k] shared over
 *    the batch, strides {h, i} with j contiguous.  sinks / dsinks are fp32
 *    [Hq].  Gradients are written in fp32.
 *  - Query head h reads KV head h / (Hq / Hk) ([GQA-BWD]: K/V repeated along
 *    the head axis, dK/dV summed back over each group).
 *  - LSE is in natural-log units and is -inf for a row with no allowed key
 *    and no sink; such a row has O = 0 and zero gradients.
 *  - Every call validates its arguments on the host first and returns
 *    ATTN_EINVAL / ATTN_EUNSUPPORTED without touching the GPU; HIP launch
 *    errors return ATTN_EHIP.  Nothing is printed, no exception crosses the
 *    ABI.  Calls are ordered on the given stream (NULL = the default stream)
 *    and never synchronise the device.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = -1,        /* inconsistent or out-of-range argument          */
  ATTN_EUNSUPPORTED = -2,  /* valid problem outside what the kernels cover   */
  ATTN_EHIP = -3,          /* a HIP launch or runtime call failed            */
  ATTN_ENOSCRATCH = -4     /* attn_bwd_static: needs more than its scratch   */
} attn_status_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Mask kinds ([SINK] make_causal_mask; [SFMG] "Example" bottom-right rule).
 * With global indices i' = q_offset + i, j' = k_offset + j and
 * delta = 0 (TOP_LEFT) or sk_total - sq_total (BOTTOM_RIGHT), a pair is
 * allowed when
 *     i' + delta - window_left <= j' <= i' + delta + window_right
 *     (no lower bound when window_left < 0)
 *  or j' < num_sink_tokens  (sink tokens are visible to every row).
 * Plain causal is window_left = -1, window_right = 0; a sliding window of
 * width W ([SINK] make_sliding_window_sink_mask) is window_left = W - 1,
 * window_right = 0.  ATTN_MASK_NONE allows every pair; it requires
 * window_left = -1, window_right = 0 and num_sink_tokens = 0. */
typedef enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_TOP_LEFT = 1,
  ATTN_MASK_BOTTOM_RIGHT = 2
} attn_mask_t;

/* attn_bwd flags.
 * ATTN_DETERMINISTIC: two calls give bitwise identical results.  dQ always
 *   comes from a query-block-parallel pass that accumulates in registers,
 *   and dbias is summed over the batch in a fixed order.  Without the flag
 *   the dK / dV of a key block may be split into more than two parts whose
 *   fp32 adds into the output can come in any order, so the low bits may
 *   vary -- except for bf16 problems with head dim 64 / 128, no bias and no
 *   packed batch given a workspace of attn_bwd_workspace_size bytes, whose
 *   parts are summed in a fixed order either way.
 * ATTN_ACCUMULATE_DQ: add into dQ instead of overwriting it (chunked /
 *   ring use, [RING] _ring_bwd accumulates dq over the K/V chunks).
 * ATTN_ACCUMULATE_DKDV: add into dK and dV instead of overwriting them
 *   ([RING] _ring_bwd adds each chunk's dk/dv into travelling
 *   accumulators).
 * ATTN_SHARED_KV: one tensor serves as keys and values ([SFMG] "Formula",
 *   sliding-window case: the selected KV is the original KV, used in
 *   Q KV^T, dO KV^T and dS KV).  k and v must be the same pointer with the
 *   same strides and Dqk == Dv; dk receives the gradient of the shared
 *   tensor, dKV = scale * dS^T Q + P^T dO ([SFMG] Phase 3), and dv must be
 *   null.  Covered for head dim 512 (the page's D) with bf16 inputs and no
 *   bias; head dim 512 requires the flag (else ATTN_EUNSUPPORTED). */
enum {
  ATTN_DETERMINISTIC = 1u,
  ATTN_ACCUMULATE_DQ = 2u,
  ATTN_ACCUMULATE_DKDV = 4u,
  ATTN_SHARED_KV = 8u
};

/* Problem description ([GQA-BWD] FmhaProblem; [SFMG] "Prototype"). */
typedef struct attn_problem {
  int32_t B, Hq, Hk;        /* batch, query heads, KV heads; Hq % Hk == 0        */
  int32_t Sq, Sk;           /* local sequence lengths (this call's rows / keys)  */
  int32_t Dqk, Dv;          /* head dims of Q/K and of V/O (at most 512)         */
  float scale;              /* softmax scale, applied to Q K^T before bias       */
  int32_t in_dtype;         /* attn_dtype_t of Q, K, V and dO                    */
  int32_t o_dtype;          /* attn_dtype_t of O                                 */
  int32_t mask;             /* attn_mask_t                                       */
  int32_t window_left;      /* -1 = unbounded                                    */
  int32_t window_right;     /* >= 0                                              */
  int32_t num_sink_tokens;  /* keys with global index below this always visible  */
  int64_t q_offset;         /* global index of local query row 0                 */
  int64_t k_offset;         /* global index of local key 0                       */
  int64_t sq_total;         /* global query length for bottom-right (0 => Sq)    */
  int64_t sk_total;         /* global key length for bottom-right (0 => Sk)      */
  int64_t q_str[3], k_str[3], v_str[3], o_str[3], do_str[3];  /* {b, h, s}      */
  int64_t dq_str[3], dk_str[3], dv_str[3];                    /* {b, h, s}      */
  int64_t bias_str[2];      /* {h, i} of bias and dbias                          */
  /* Variable-length packed batch ([SFMG] "Prototype": TND layout with
   * cumulative sequence lengths).  Both null: dense batch.  Otherwise device
   * arrays of B + 1 non-decreasing int32 prefix sums: sequence b owns the
   * packed query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and keys
   * [cu_seqlens_k[b], cu_seqlens_k[b+1]) along the s index of every q-side
   * (Q, O, dO, dQ) and k-side (K, V, dK, dV) tensor, whose b strides are
   * then unused (e.g. TND: strides {0, D, H * D}).  Sq and Sk are the
   * longest lengths; total_q and total_k the packed row counts of the
   * tensors.  Offsets and lengths read from the arrays are clamped to those
   * counts and maxima, so no access leaves the tensors.  The bottom-right
   * mask is aligned per sequence.  LSE and delta stay [B, Hq, Sq]: rows past
   * a sequence's length are not written by the forward, delta is 0 there.
   * Requires bf16 inputs with Dqk == Dv in {64, 128}, no bias, and zero
   * q_offset / k_offset / sq_total / sk_total (else ATTN_EUNSUPPORTED or
   * ATTN_EINVAL).  Zero-filled by attn_problem_init. */
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int64_t total_q, total_k;
  /* Optional device scratch of attn_bwd, owned by the caller (nullable;
   * zero-filled by attn_problem_init).  When the dK / dV of key blocks are
   * split over workgroups into more than two parts, a call with at least
   * attn_bwd_workspace_size bytes here (16-byte aligned) keeps the parts'
   * partial sums in it and adds them into dK / dV in a fixed order; with
   * less, or none, the parts add atomically into the output.  A call uses
   * the buffer in the order of its stream until it completes there, so calls
   * that may overlap need buffers of their own.  Its contents on entry do
   * not matter. */
  void* workspace;
  int64_t workspace_bytes;
} attn_problem_t;

/* Fill *p with contiguous [B, H, S, D] strides and defaults: scale =
 * 1/sqrt(Dqk), dtypes bf16 (inputs) / fp32 (O), no mask, no window, no
 * sinks, zero offsets, bias strides {Sq*Sk, Sk}. */
void attn_problem_init(attn_problem_t* p, int32_t B, int32_t Hq, int32_t Hk, int32_t Sq,
                       int32_t Sk, int32_t Dqk, int32_t Dv);

/* Forward with log-sum-exp ([RING] _flash_fwd returns (out, lse); [GQA-BWD]
 * cpu_fwd_with_intermediates; [DBIAS] cpu_attention_fwd_bias; [SINK]
 * cpu_attention_fwd_masked).  S = scale * Q K^T + bias (masked pairs
 * excluded); the optional sink logit of each query head joins the softmax
 * normaliser without a value row.  Writes O (o_dtype, strides o_str) and
 * LSE (fp32 [B, Hq, Sq]).
 *   bias:  nullable fp32 [Hq, Sq, Sk];  sinks: nullable fp32 [Hq].
 * Head dim 512 ([SFMG] shared KV): k and v must be the same tensor (same
 * pointer and strides), bf16, no bias (else ATTN_EUNSUPPORTED). */
attn_status_t attn_fwd_lse(const attn_problem_t* p, const void* q, const void* k,
                           const void* v, const float* bias, const float* sinks, void* o,
                           float* lse, void* stream);

/* Backward preprocess ([GQA-BWD] cpu_bwd_gqa: D = rowsum(dO * O); [SFMG]
 * Phase 2 SoftmaxGrad(dO, O) and Phase 3 dSinks).
 *   delta[b,h,i] = sum_d dO[b,h,i,d] * O[b,h,i,d]               (fp32 [B,Hq,Sq])
 *   if sinks: dsinks[h] = -sum_{b,i} exp(sinks[h] - lse[b,h,i]) * delta[b,h,i]
 * dsinks is required iff sinks is given; it is overwritten.
 * dq_zero, dk_zero, dv_zero are nullable: each given fp32 gradient buffer
 * (strides dq_str / dk_str / dv_str) is zeroed here -- dQ in the same pass
 * as delta -- so that a following attn_bwd with ATTN_ACCUMULATE_DQ /
 * ATTN_ACCUMULATE_DKDV accumulates into zeroed buffers without further
 * fills. */
attn_status_t attn_bwd_preprocess(const attn_problem_t* p, const void* o, const void* dout,
                                  const float* lse, const float* sinks, float* delta,
                                  float* dsinks, float* dq_zero, float* dk_zero, float* dv_zero,
                                  void* stream);

/* Backward main pass ([GQA-BWD] module docstring and cpu_bwd_gqa; [DBIAS]
 * cpu_attention_bwd_dbias; [SFMG] Phase 2 and 3):
 *   P = exp(S - LSE) on allowed pairs, dP = dO V^T, dS = P * (dP - delta),
 *   dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO  (dK, dV summed over
 *   each KV head's query group), dbias = sum over batch of dS.
 * dq is overwritten (or added into with ATTN_ACCUMULATE_DQ); dk, dv and
 * dbias are overwritten.  bias is nullable; dbias is nullable and requires
 * bias.  dbias is written through bias_str, so with dbias the strides must
 * keep rows and heads apart (bias_str[1] >= Sk when Sq > 1, and
 * bias_str[0] >= (Sq - 1) * bias_str[1] + Sk when Hq > 1; a broadcast bias
 * with zero strides is readable but has no room for its gradient):
 * ATTN_EINVAL otherwise.  delta must come from attn_bwd_preprocess on the
 * same O / dO.
 * The library allocates nothing: scratch for the partial sums of split key
 * blocks comes from p->workspace when the caller provides one (see
 * attn_problem_t).  The call records no memset, so it can be captured
 * into a graph.
 * For a K/V chunk pass the chunk's K/V views with k_offset / sk_total and
 * the GLOBAL O, LSE and delta ([RING] _ring_bwd). */
attn_status_t attn_bwd(const attn_problem_t* p, const void* q, const void* k, const void* v,
                       const void* dout, const float* lse, const float* delta,
                       const float* bias, float* dq, float* dk, float* dv, float* dbias,
                       uint32_t flags, void* stream);

/* Size of the device scratch array of attn_bwd_static, per GPU. */
#define ATTN_STATIC_SCRATCH_BYTES (64u * 1024u * 1024u)

/* attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, results and validation as attn_bwd, but the partial
 * sums that attn_bwd keeps in p->workspace live in a static device array
 * of ATTN_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on each GPU
 * it runs on until the process ends; p->workspace and p->workspace_bytes
 * are ignored.  The call allocates nothing.  A problem whose
 * attn_bwd_workspace_size exceeds ATTN_STATIC_SCRATCH_BYTES returns
 * ATTN_ENOSCRATCH before any HIP call (it fits attn_bwd with a caller
 * workspace, or without one).  Every call on a GPU shares that GPU's array
 * and leaves its contents behind; a call stores every element of it that it
 * reads first, so nothing needs to be cleared, but calls that overlap on one
 * GPU (on different streams, or concurrent host threads) race on it and
 * must be serialised by the caller.  The first call on a GPU looks up the
 * array's device address there (hipGetSymbolAddress). */
attn_status_t attn_bwd_static(const attn_problem_t* p, const void* q, const void* k, const void* v,
                              const void* dout, const float* lse, const float* delta,
                              const float* bias, float* dq, float* dk, float* dv, float* dbias,
                              uint32_t flags, void* stream);

/* Bytes of p->workspace with which attn_bwd(p, ..., flags) keeps the
 * partial sums of split key blocks (with ATTN_SHARED_KV: of the query-head
 * parts of a KV head) instead of adding them atomically (a bias problem
 * does not use it; 0: the call splits nothing into more than two parts, or
 * takes a path without partial sums).  Host-only: makes no HIP call.
 * ATTN_EINVAL for an invalid problem or a null `bytes`. */
attn_status_t attn_bwd_workspace_size(const attn_problem_t* p, uint32_t flags, int64_t* bytes);

/* In-place log-sum-exp merge of a partial result into an accumulator
 * ([RING] _ring_fwd):  lse = logaddexp(lse_acc, lse_part),
 *   o_acc = o_acc * exp(lse_acc - lse) + o_part * exp(lse_part - lse).
 * Both o buffers are contiguous fp32 [B, H, Sq, Dv], both lse buffers
 * contiguous fp32 [B, H, Sq].  Where both lse are -inf the result is o = 0,
 * lse = -inf. */
attn_status_t attn_lse_merge(int32_t B, int32_t H, int32_t Sq, int32_t Dv, float* o_acc,
                             float* lse_acc, const float* o_part, const float* lse_part,
                             void* stream);

/* Static description of a status code. */
const char* attn_status_string(attn_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
