/*
 * kda.h -- C ABI of the MI355X (gfx950) chunked Kimi Delta Attention forward.
 *
 * The call contract follows the "FlashKDA Delta Attention" skill page
 * (atskills.one/aradotso): section "Core Kernel API", the "Tensor shapes and
 * dtypes" table and "Constraints":
 *   q, k, g  [B, T, H, K] bf16     (K must be 128; g are gate logits)
 *   v        [B, T, H, V] bf16     (V must be 128)
 *   beta     [B, T, H]    bf16     logits, sigmoid applied inside
 *   A_log    [H] fp32, dt_bias [H, K] fp32, scale, lower_bound
 *   out      [B, T, H, V] bf16, allocated by the caller
 *   initial_state / final_state [N, H, V, K] bf16 or fp32 or absent
 *     (note the V-before-K orientation); dtypes must match when both given
 *   cu_seqlens [N+1] int64 for packed variable-length batches (then B == 1
 *     and T is the total token count)
 * Grouped value heads (several v/gate/beta heads sharing one q/k head) are
 * the "grouped value heads" axis of the fla-kda SKILL.md "Validation"
 * section: H_v = G * H_qk, and v-head h reads q/k head h / G.
 *
 * Gate activations ("fla-kda" skill listing and fla-kda SKILL.md, "Gate
 * contracts"):
 *   KDA_GATE_SOFTPLUS     a = -exp(A_log[h]) * softplus(g + dt_bias[h])
 *                         (A_log required)
 *   KDA_GATE_SAFE_SIGMOID a = lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h])),
 *                         with -5 <= lower_bound < 0; A_log may be NULL, which
 *                         means a multiplier of one
 *   KDA_GATE_PREGATED     a = g: the caller passes the log-space decay itself
 *                         (natural log, per token and key channel); it must be
 *                         <= 0 (device data, not validated).  A_log is unused
 *                         and dt_bias must be NULL.
 * dt_bias may be NULL for the two activated gates (zero bias).
 * The recurrence (per sequence and v-head, state S in R^{V x K}):
 *   S <- S Diag(e^{a_t});  S <- S + b_t (v_t - S k_t) k_t^T;  o_t = scale * S q_t
 * with b_t = sigmoid(beta_t) (beta_t itself with KDA_FLAG_BETA_IS_PROB) and q,
 * k L2-normalised in the kernel with KDA_FLAG_QK_L2NORM.
 *
 * Magnitudes: v and the states may hold any finite bf16 / fp32 values; both
 * entries scale their out and final_state exactly (bit for bit) when v and
 * initial_state are scaled together by a power of two, as long as the results
 * stay normal in their own dtype.  With KDA_FLAG_QK_L2NORM, q and k may hold
 * any values whose squares still sum within fp32 (elements below about 2^60
 * in size).  One limit is particular to the chunked entries: within a
 * 64-token chunk they carry the decay factors of the chunk in 16-bit operands,
 * so a state decayed within one chunk below about 2^-24 of its size (fp16
 * subnormals lose precision from 2^-14) drops out of that chunk's outputs.
 * That is far below the output tolerance while the state and the values
 * written next are of similar size, which the delta rule keeps, unless v
 * changes by a large factor from one chunk to the next while strong decays
 * act: with a per-token decay down to e^-1 (safe gate, lower bound -1) a
 * change by 2^14 costs the following outputs about 1 % relative, 2^16 about
 * 3 %; with mild decays a change by 2^18 stays at 0.2 %.  Tested down to
 * steps of 2^12 per chunk over a total range of 2^88.  kda_fused_recurrent_fwd,
 * fp32 throughout, has no such limit.  Without the L2 norm q and k are used as
 * given, and the chunked
 * entry rounds them (times decay factors <= 1) to fp16, so their elements
 * must stay well below 2^15 in size -- far beyond where the recurrence with
 * beta near 1 stays bounded.
 *
 * Ownership: every buffer is allocated and owned by the caller.  The library
 * allocates no device memory of its own (the one exception is the fixed
 * device array of kda_fwd_noalloc, part of the loaded code object), keeps no
 * mutable global state except a thread-local error string and that array's
 * address per device, and never synchronises: kda_fwd returns once its
 * kernels are enqueued on `stream`.  Calls that use distinct workspaces are
 * independent; two calls in flight must not share a workspace.
 *
 * Errors: all argument predicates are checked on the host before anything is
 * enqueued; on error nothing is launched and nothing is written.  The values
 * inside device tensors (e.g. that cu_seqlens is non-decreasing and ends at
 * T) are not validated.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer is NULL */
  KDA_ERR_SHAPE = -2,       /* a size is out of the supported set; besides the rules
                               below: fewer than 2^24 64-token chunks per head (B *
                               ceil(T/64), or that plus num_seqs when packed), at most
                               2^30 chunk-heads, at most 2^21 (sequence, v-head) pairs,
                               H_v <= 65535 -- what one launch dimension holds */
  KDA_ERR_DTYPE = -3,       /* unknown or mismatched state dtype code */
  KDA_ERR_RANGE = -4,       /* scalar outside its allowed range */
  KDA_ERR_ALIGN = -5,       /* a tensor base is not 16-byte aligned */
  KDA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than kda_fwd_workspace_size */
  KDA_ERR_LAUNCH = -7,      /* the HIP runtime rejected a launch */
  KDA_ERR_UNSUPPORTED = -8  /* unknown gate mode or flag */
} kda_status;

typedef enum { KDA_GATE_SOFTPLUS = 0, KDA_GATE_SAFE_SIGMOID = 1, KDA_GATE_PREGATED = 2 } kda_gate_mode;
typedef enum { KDA_STATE_NONE = 0, KDA_STATE_F32 = 1, KDA_STATE_BF16 = 2 } kda_state_dtype;

/* flags (any combination; other bits are rejected).  Raw and post-sigmoid
 * beta, and the in-kernel q/k norm on and off, are among the variants the
 * "fla-kda" skill listing names as test axes:
 *   KDA_FLAG_QK_L2NORM     normalise q and k (eps 1e-6 inside the root) in the kernel
 *   KDA_FLAG_BETA_IS_PROB  beta holds probabilities: no sigmoid is applied */
enum { KDA_FLAG_QK_L2NORM = 1, KDA_FLAG_BETA_IS_PROB = 2 };

typedef struct {
  int32_t B, T;               /* batch rows and tokens per row (total tokens when packed) */
  int32_t H_qk, H_v;          /* q/k heads and v/gate/beta heads; H_v % H_qk == 0 */
  int32_t K, V;               /* head dims; both must be 128 */
  int32_t num_seqs;           /* N: equals B without cu_seqlens; else the packed count */
  float scale;                /* output scale (typically 1/sqrt(K)) */
  float lower_bound;          /* safe gate only: -5 <= lower_bound < 0 */
  int32_t gate_mode;          /* kda_gate_mode */
  int32_t init_state_dtype;   /* kda_state_dtype of initial_state (NONE: zero state) */
  int32_t final_state_dtype;  /* kda_state_dtype of final_state (NONE: not written) */
  int32_t flags;              /* KDA_FLAG_* bits */
  int32_t segments;           /* time segments per state chain; dense input only (ignored
                                 with cu_seqlens).  The chunk chain of each (sequence, v-head)
                                 is cut into runs that proceed in parallel: each run's state
                                 carried from zero and its linear map give its entry state,
                                 then every run emits its outputs -- the one-GPU form of the
                                 context parallelism the fla-kda SKILL.md "Validation" section
                                 lists.  0 = automatic (split only when there are few
                                 (sequence, v-head) pairs), 1 = never, n in [2, 256] = up to n
                                 (at most one per 64-token chunk).  Other values are rejected
                                 with KDA_ERR_RANGE.  Results agree with the unsplit chain
                                 within rounding, not bit for bit. */
} kda_fwd_params;

/* Bytes of device workspace kda_fwd needs for these parameters; host only,
 * no HIP calls.  Returns 0 if the parameters are invalid. */
size_t kda_fwd_workspace_size(const kda_fwd_params* p);

/* Time segments per state chain that kda_fwd uses for these parameters (1:
 * the chain is not split), for dense input (packed == 0) or input with
 * cu_seqlens (packed != 0, always 1); host only.  Returns 0 if the
 * parameters are invalid. */
int kda_fwd_segments(const kda_fwd_params* p, int packed);

/* Validates parameters and pointers exactly as kda_fwd does, without
 * launching anything; host only, no HIP calls.  Pointers are device
 * pointers (never dereferenced here).  initial_state / final_state /
 * cu_seqlens may be NULL as the parameters allow.  Returns KDA_OK or the
 * first failing predicate's code (detail in kda_last_error()). */
kda_status kda_fwd_check(const kda_fwd_params* p,
                         const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* A_log, const float* dt_bias,
                         const int64_t* cu_seqlens, const void* initial_state,
                         const void* final_state, const void* out,
                         const void* workspace, size_t workspace_bytes);

/* Chunked KDA forward.  All pointers are device pointers:
 *   q, k      bf16 [B, T, H_qk, 128]       v, g  bf16 [B, T, H_v, 128]
 *   beta      bf16 [B, T, H_v] (logits, or probabilities with KDA_FLAG_BETA_IS_PROB)
 *   A_log     fp32 [H_v] or NULL (see the gate modes)
 *   dt_bias   fp32 [H_v, 128] or NULL (see the gate modes)
 *   cu_seqlens int64 [num_seqs + 1] or NULL (dense: sequence n is batch row n)
 *   initial_state [num_seqs, H_v, 128, 128] of init_state_dtype, or NULL
 *   final_state   [num_seqs, H_v, 128, 128] of final_state_dtype, or NULL
 *   out       bf16 [B, T, H_v, 128] -- every element is written
 *   workspace at least kda_fwd_workspace_size(p) bytes, 256-byte aligned
 *   stream    a hipStream_t (NULL: the default stream)
 * Tensors are dense row-major.  initial_state and final_state may be the
 * same buffer (an in-place state update): every element of the initial state
 * is read before the launch that writes the final state, or by the workgroup
 * that later writes it.  Returns after enqueueing; KDA_ERR_LAUNCH if the
 * runtime reports a launch error. */
kda_status kda_fwd(const kda_fwd_params* p,
                   const void* q, const void* k, const void* v, const void* g,
                   const void* beta, const float* A_log, const float* dt_bias,
                   const int64_t* cu_seqlens, const void* initial_state, void* final_state,
                   void* out, void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of kda_fwd, for timing each kernel on its own: kda_fwd is
 * exactly kda_fwd_intra followed by kda_fwd_state on the same stream, with
 * the same parameters, tensors and workspace.  kda_fwd_intra runs the
 * per-chunk work (gate, cumulative decay, Akk/Aqk, triangular solve, WY
 * factors) over all chunks in parallel and leaves its results in the
 * workspace; kda_fwd_state then runs the inter-chunk state recurrence and
 * writes out and final_state.  Arguments, validation and errors are those of
 * kda_fwd (every pointer is checked, even ones the stage does not read). */
kda_status kda_fwd_intra(const kda_fwd_params* p,
                         const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* A_log, const float* dt_bias,
                         const int64_t* cu_seqlens, const void* initial_state, void* final_state,
                         void* out, void* workspace, size_t workspace_bytes, void* stream);
kda_status kda_fwd_state(const kda_fwd_params* p,
                         const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* A_log, const float* dt_bias,
                         const int64_t* cu_seqlens, const void* initial_state, void* final_state,
                         void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free form of kda_fwd, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same parameters, tensors,
 * validation and results as kda_fwd (the same kernels, bit for bit), minus the
 * workspace: its calls use a device array of KDA_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on from the first such call until the
 * process ends.  It calls no allocating routine.  Calls whose workspace
 * (kda_fwd_workspace_size) exceeds that size are rejected with
 * KDA_ERR_WORKSPACE before anything is enqueued.  All calls on one GPU share
 * its array: two calls whose work overlaps in time on the same GPU (different
 * streams, or host threads) race and corrupt each other's results; serialise
 * them (one stream, or one call in flight per GPU).  Nothing in the array
 * needs to start at zero.  Returns after enqueueing. */
#define KDA_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
kda_status kda_fwd_noalloc(const kda_fwd_params* p,
                           const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const float* A_log, const float* dt_bias,
                           const int64_t* cu_seqlens, const void* initial_state, void* final_state,
                           void* out, void* stream);

/* Token-recurrent forward, for decode steps and short sequences: the second
 * public entry point (fused recurrent, beside the chunked one) that the
 * fla-kda SKILL.md names in its opening paragraph.
 * Same parameters, tensors and validation as kda_fwd, minus the workspace: it
 * evaluates the recurrence token by token with the fp32 state in registers,
 * one workgroup per (sequence, v-head, 32-row slice of V), so its cost grows
 * with the longest sequence; for long sequences kda_fwd is the faster path
 * (measured at B=16, H=32: this entry is faster up to about 32 tokens per
 * sequence, kda_fwd from 64 on).
 * initial_state and final_state may be the same buffer (an in-place state
 * update), since every element is read before any is written by the same
 * workgroup.  Returns after enqueueing. */
kda_status kda_fused_recurrent_fwd(const kda_fwd_params* p,
                                   const void* q, const void* k, const void* v, const void* g,
                                   const void* beta, const float* A_log, const float* dt_bias,
                                   const int64_t* cu_seqlens, const void* initial_state, void* final_state,
                                   void* out, void* stream);

/* Bytes of device workspace kda_bwd needs for these parameters; host only,
 * no HIP calls.  Returns 0 if the parameters are invalid. */
size_t kda_bwd_workspace_size(const kda_fwd_params* p);

/* Gradients of kda_fwd: the backward pass that the fla-kda SKILL.md lists in
 * its "Code map" (backward passes) and "Validation" (supported gradients)
 * sections.  Inputs are those of kda_fwd (the forward is recomputed, so no
 * forward output is needed) plus
 *   d_out          bf16 [B, T, H_v, 128]  gradient of out
 *   d_final_state  fp32 [num_seqs, H_v, 128, 128] gradient of the final state,
 *                  or NULL (zero)
 * and writes fp32 gradients, every element of each:
 *   dq, dk  [B, T, H_qk, 128] (summed over the v-heads of each q/k head)
 *   dv      [B, T, H_v, 128]     dg [B, T, H_v, 128]     dbeta [B, T, H_v]
 *           (with respect to the logits, or the probabilities with
 *           KDA_FLAG_BETA_IS_PROB)
 *   dA_log  [H_v] or NULL (must be NULL when A_log is NULL or the decay is
 *           pre-gated)
 *   ddt_bias [H_v, 128] or NULL (the bias gradient, also when dt_bias is
 *           NULL; must be NULL with pre-gated decay)
 *   d_initial_state fp32 [num_seqs, H_v, 128, 128] or NULL
 * params->final_state_dtype is not used; params->segments splits both
 * state passes (over the chunks forward, then backward) as in kda_fwd, the
 * segment count kda_fwd_segments reports.  The workspace
 * (kda_bwd_workspace_size bytes, 256-byte aligned) holds fp32 per-chunk
 * intermediates and the segment scratch; the library allocates nothing.  Every predicate
 * is checked before anything is enqueued; returns after enqueueing. */
kda_status kda_bwd(const kda_fwd_params* p,
                   const void* q, const void* k, const void* v, const void* g,
                   const void* beta, const float* A_log, const float* dt_bias,
                   const int64_t* cu_seqlens, const void* initial_state,
                   const void* d_out, const float* d_final_state,
                   float* dq, float* dk, float* dv, float* dg, float* dbeta,
                   float* dA_log, float* ddt_bias, float* d_initial_state,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Static name of a status code. */
const char* kda_status_string(kda_status s);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* kda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
