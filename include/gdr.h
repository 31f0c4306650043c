/*
 * gdr.h -- C ABI of libgdr, a gated delta-rule (Gated DeltaNet) engine for
 * AMD MI355X (gfx950).
 *
 * The operation (the "com.microsoft.GatedDeltaNet" README, section
 * Description): per value head, a V-major fp32 state S (dv rows of dk) is
 * updated token by token,
 *     S_t = exp(g_t) S_{t-1} + k_t (beta_t (v_t - exp(g_t) S_{t-1}^T k_t))^T
 *     o_t = scale * S_t^T q_t
 * where update_rule (README, Attributes) selects which terms survive:
 *     GDR_RULE_LINEAR        no decay, no retrieval: S += k v^T
 *     GDR_RULE_GATED         decay only
 *     GDR_RULE_DELTA         retrieval (delta correction) only
 *     GDR_RULE_GATED_DELTA   both (the default)
 *     GDR_RULE_GATED_DELTA_V2  the Gated DeltaNet-2 recurrence with a key-axis
 *         erase gate b_t and no update rate (ONNX issue "Spec gap:
 *         LinearAttention (opset 27) cannot represent Gated DeltaNet-2's
 *         channel-wise erase gate", sections "The GDN-2 recurrence" and
 *         "Proposed extension"):
 *             S_t = D_t S_{t-1} - k_t (b_t o k_t)^T D_t S_{t-1} + k_t v_t^T
 *         with D_t = Diag(exp(decay_t)) acting on the key axis.
 * A per-key-dimension decay (gate shaped (..., HV, dk)) is accepted for the
 * decayed rules: it multiplies key channel j of every state row by
 * exp(decay[j]) (Ascend "aclnnRecurrentGatedDeltaRule" page, Formula;
 * CLIKA "gatedDeltaUpdate": a [B,T,HV,K] gate is per key dim).
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   q, k            (T, H, dk)   act dtype   -- or (B, L, H, dk), same bytes
 *   v, o            (T, HV, dv)  act dtype
 *   gate            (T, HV) or (T, HV, dk) per key; fp32, or the act dtype
 *                   when gate_activation = QWEN and gate_dtype = act dtype
 *   beta            (T, HV) fp32, or (T, 1) with beta_per_token: one rate per
 *                   token for every value head (the ONNX issue's LinearAttention
 *                   schema allows beta's last axis in {kv_num_heads, 1})
 *   erase           (T, HV, dk)  fp32 (GATED_DELTA_V2 only)
 *   a_log           (HV)         fp32 (gate_activation = QWEN, unless gate_scale)
 *   gate_scale      (HV)         fp32: the once-folded -exp(a_log), instead of a_log
 *   dt_bias         (HV), or (HV, dk) beside a per-key gate; fp32 (QWEN only)
 *   cu_seqlens      (B + 1)      int32, rank-3 spelling only
 *   seq_lens        (B)          int32, uniform packing only
 *   slot_ids        (B)          int32
 *   initial_state   (B, HV, dv, dk) fp32, or NULL for a zero state
 *   final_state     (B, HV, dv, dk) fp32; with num_slots > 0 it is instead
 *                   the slab (num_slots, HV, dv, dk), read and updated in
 *                   place at rows slot_ids[b] (CLIKA "gatedDeltaUpdate")
 * with T total tokens, H query/key heads, HV value heads (a positive multiple
 * of H; value head h reads q/k head floor(h * H / HV), README Description),
 * act dtype fp32 or fp16 (README, Type constraints), or bf16.
 *
 * Requests: with cu_seqlens, request b covers tokens
 * [clamp(cu[b], 0, T), clamp(cu[b+1], 0, T)) and is empty when the end is not
 * past the start (README, Inputs cu_seqlens); the clamp happens on the
 * device, the host never reads cu_seqlens or slot_ids.  Without cu_seqlens
 * the packing is uniform: request b covers [b*L, (b+1)*L), T = B * L, or only
 * its first clamp(seq_lens[b], 0, L) tokens when seq_lens is given (CLIKA
 * "gatedDeltaUpdate": seq_lens bounds ragged prefill rows; the padding rows'
 * outputs are left unwritten, like tokens outside every request).  An
 * empty request copies its incoming state to final_state (README, Outputs);
 * o rows of tokens that no request covers are left unwritten.  A slot id
 * outside [0, num_slots) skips its request entirely (nothing read or
 * written).  Slot ids must be distinct within one call (the caller's
 * contract, CLIKA "gatedDeltaUpdate"); duplicates give undefined results.
 *
 * Ownership: the caller owns every buffer; the library allocates and frees
 * nothing and keeps no state between calls (gdr_forward_noalloc's workspace is
 * a fixed array in the library's device code, see there).  All device work is enqueued on
 * the caller's stream; no call synchronises the stream or reads device
 * memory from the host.  final_state may be the same pointer as
 * initial_state (in-place update); any other overlap between an output and
 * an input is rejected with GDR_E_ALIAS.
 *
 * Errors: every function returns a gdr_status.  Argument errors are found on
 * the host before anything is enqueued (two-phase use as on the Ascend page:
 * query, then execute).  Bad device-side addressing data is clamped or
 * skipped as described above, never reported.  gdr_last_error() returns a
 * thread-local message for the last failing call.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 3

typedef enum {
    GDR_OK = 0,
    GDR_E_INVALID = 1,      /* bad shape, missing or unexpected tensor, bad enum */
    GDR_E_UNSUPPORTED = 2,  /* valid request the library does not implement */
    GDR_E_ALIAS = 3,        /* overlapping input/output buffers */
    GDR_E_WORKSPACE = 4,    /* workspace missing or smaller than gdr_workspace_size */
    GDR_E_HIP = 5           /* a HIP runtime call failed (message in gdr_last_error) */
} gdr_status;

/* Activation dtypes.  bf16 goes beyond the pages' type list (fp32, fp16;
 * README, Type constraints): the loads widen it exactly to fp32 and the
 * output is rounded to nearest even on store.  The chunked kernels read it
 * as fp16 when the decay is per head (a (request, head) pair holding a
 * value fp16 cannot represent exactly, outside magnitudes 2^-17 to 65504,
 * is computed by the recurrent kernel instead) and widen it to fp32 in the
 * per-key form. */
typedef enum { GDR_F32 = 0, GDR_F16 = 1, GDR_BF16 = 2 } gdr_dtype;

typedef enum {
    GDR_RULE_LINEAR = 0,
    GDR_RULE_GATED = 1,
    GDR_RULE_DELTA = 2,
    GDR_RULE_GATED_DELTA = 3,
    GDR_RULE_GATED_DELTA_V2 = 4
} gdr_update_rule;

/* README, Attributes gate_activation: NONE takes gate as the log decay g;
 * QWEN forms g = -exp(a_log[h]) * softplus(gate + dt_bias[h]) in fp32, or
 * g = gate_scale[h] * softplus(gate + dt_bias[h]) with the folded scale, and
 * with a per-key gate dt_bias[h][j] per key channel (CLIKA "gatedDeltaUpdate",
 * the gate_bias / gate_scale arm). */
typedef enum { GDR_GATE_NONE = 0, GDR_GATE_QWEN = 1 } gdr_gate_activation;

/* README, Attributes beta_activation: NONE takes beta as the rate; SIGMOID
 * applies 1 / (1 + exp(-beta)) in fp32. */
typedef enum { GDR_BETA_NONE = 0, GDR_BETA_SIGMOID = 1 } gdr_beta_activation;

/* Which kernel family runs; AUTO picks from the shapes.  The result does not
 * depend on the choice beyond rounding (README, Attributes chunk_size). */
typedef enum {
    GDR_ALGO_AUTO = 0,
    GDR_ALGO_RECURRENT = 1,  /* state tile in registers across the token loop */
    GDR_ALGO_DECODE = 2,     /* one workgroup streams one (request, head) state */
    GDR_ALGO_CHUNKED = 3     /* chunk-parallel form (fp16 or bf16, dk = dv = 128).  Its products
                              * run on fp16 matrix cores with every fp32 operand split
                              * into an fp16 (hi, lo) pair.  Each state tile runs scaled
                              * by a power of two that brings the larger of max |v| over
                              * its chunks and max |S0| of the tile to [4, 8), so inputs
                              * of any overall size keep ~22 bits.  A (request, head)
                              * pair whose split operands reach 60000 (a state grown
                              * about 8000 times past that size, or inputs such as
                              * unnormalised keys that push the chunk's own operands
                              * there) is recomputed on the recurrent kernel in fp32, as
                              * are requests whose cu_seqlens ranges overlap an earlier
                              * request's beyond the chunk budget.  In-place final states
                              * (a slab, or final == initial) are staged in the workspace
                              * and copied back for the pairs not recomputed. */
} gdr_algo;

typedef struct {
    int64_t total_tokens;       /* T >= 0 */
    int32_t batch;              /* B >= 0: requests (cu_seqlens has B + 1 entries) */
    int32_t seq_len;            /* L: uniform request length; 0 when cu_seqlens is used */
    int32_t num_heads_qk;       /* H >= 1 */
    int32_t num_heads_v;        /* HV, a positive multiple of H */
    int32_t head_dim_k;         /* dk in [1, 256] */
    int32_t head_dim_v;         /* dv in [1, 256] */
    int32_t num_slots;          /* > 0: final_state is a slab addressed by slot_ids */
    int32_t act_dtype;          /* gdr_dtype of q, k, v, o */
    int32_t gate_dtype;         /* gdr_dtype of gate; must be F32 unless QWEN */
    int32_t update_rule;        /* gdr_update_rule */
    int32_t gate_activation;    /* gdr_gate_activation */
    int32_t beta_activation;    /* gdr_beta_activation */
    int32_t qk_l2_norm;         /* 1: q, k <- x / sqrt(sum x^2 + 1e-12) (README, Attributes) */
    int32_t decay_per_key;      /* 1: gate is (T, HV, dk) */
    int32_t rank4;              /* 1: q is spelled (B, L, H, dk); forbids cu_seqlens */
    int32_t chunk_size;         /* scheduling hint for GDR_ALGO_CHUNKED (0 -> 64) */
    int32_t algo;               /* gdr_algo */
    int32_t state_update_capacity; /* must be 0 (README, Attributes) */
    int32_t beta_per_token;     /* 1: beta is (T, 1), shared by every value head */
    float scale;                /* 0 -> 1 / sqrt(dk) (README, Attributes) */
    int32_t scan_segments;      /* chunked form only, a scheduling choice like chunk_size:
                                 * 0 -> chosen from the shapes; 1 -> each request's chunks
                                 * in one serial pass; 2..16 -> each request's chain of
                                 * chunk steps cut into that many segments whose affine
                                 * transitions are composed (more workgroups, two passes).
                                 * The result is the same up to rounding. */
} gdr_problem;

typedef struct {
    const void *q, *k, *v;
    void *o;
    const void *gate;           /* NULL unless the rule decays */
    const float *beta;          /* NULL unless the rule is DELTA or GATED_DELTA */
    const float *erase;         /* NULL unless GATED_DELTA_V2 */
    const float *a_log, *dt_bias; /* QWEN: dt_bias and exactly one of a_log, gate_scale */
    const int32_t *cu_seqlens;  /* NULL: uniform packing */
    const int32_t *slot_ids;    /* non-NULL iff num_slots > 0 */
    const float *initial_state; /* NULL: zero state; must be NULL with slots */
    float *final_state;         /* required: final state, or the slab */
    const float *gate_scale;    /* (HV) folded -exp(a_log), or NULL */
    const int32_t *seq_lens;    /* (B) valid tokens per request with uniform packing, or NULL */
} gdr_tensors;

/* ABI version of the loaded library (GDR_ABI_VERSION at build time). */
int gdr_abi_version(void);

/* Static, human-readable name of a status code. */
const char *gdr_status_str(gdr_status status);

/* Thread-local description of the last failure in this thread ("" if none). */
const char *gdr_last_error(void);

/* Host-only argument check: presence rules (README, Inputs: gate present
 * exactly for decayed rules, beta exactly for DELTA/GATED_DELTA; with QWEN
 * dt_bias plus one of a_log / gate_scale, without it none of them -- CLIKA
 * "gatedDeltaUpdate": one without the other rejects), shapes, enum ranges,
 * cu_seqlens only with the rank-3 spelling, seq_lens only without cu_seqlens,
 * state_update_capacity == 0, aliasing.  Reads no tensor memory and makes no
 * HIP call.  `tensors` may be NULL to check the problem alone. */
gdr_status gdr_validate(const gdr_problem *problem, const gdr_tensors *tensors);

/* Bytes of device workspace gdr_forward needs for `problem` (first phase of
 * the two-phase use); 0 for the decode and recurrent kernels. */
gdr_status gdr_workspace_size(const gdr_problem *problem, size_t *bytes);

/* Kernel family AUTO would run for `problem` (a gdr_algo value), host only. */
gdr_status gdr_select_algo(const gdr_problem *problem, int32_t *algo);

/* Enqueue the whole operation on `stream` (a hipStream_t; NULL = the null
 * stream).  `workspace` is caller-owned device memory of at least
 * gdr_workspace_size bytes (may be NULL when that size is 0). */
gdr_status gdr_forward(const gdr_problem *problem, const gdr_tensors *tensors,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Largest workspace gdr_forward_noalloc can serve (256 MiB). */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* gdr_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * workspace comes from a fixed array of GDR_NOALLOC_SCRATCH_BYTES in the
 * library's device code: each GPU the library runs on holds its own copy
 * from the first use of the library's code there until the process ends.
 * The first call on a device looks up that device's copy (the current
 * device; `stream` must belong to it, as for any launch).  The call then
 * allocates nothing and launches exactly what gdr_forward launches.
 *
 * Problems whose gdr_workspace_size exceeds GDR_NOALLOC_SCRATCH_BYTES are
 * rejected with GDR_E_WORKSPACE before anything is enqueued (gdr_forward
 * with a caller workspace serves them).  Calls on one GPU share its array:
 * calls ordered on one stream are fine, calls that overlap in time on one GPU
 * (different streams, or other threads) race on it.  Nothing in the array
 * needs to start at zero: every byte a call reads is written earlier in the
 * same call. */
gdr_status gdr_forward_noalloc(const gdr_problem *problem, const gdr_tensors *tensors, void *stream);

/* Standalone gate fusion ("com.microsoft.LinearAttentionGate", Description):
 *   decay[n] = decay_scale[h] * softplus(a[n] + dt_bias[h])
 *   beta[n]  = sigmoid(b[n])          (only when beta != NULL; needs b)
 * for n over `count` elements whose last axis is the head axis (h = n % heads).
 * a, b, decay, beta share `dtype` (F32, F16 or BF16); dt_bias and decay_scale are
 * fp32 (heads).  Arithmetic in fp32, narrowed only on store.  b may be given
 * without beta (it is then unused). */
gdr_status gdr_gate(int64_t count, int32_t heads, int32_t dtype, const void *a,
                    const float *dt_bias, const float *decay_scale, const void *b,
                    void *decay, void *beta, void *stream);

/* Memory-traffic floor of a decode step over a state slab: a measurement
 * aid beside the operation, which computes nothing of it.  Multiplies in place
 * by `factor` each fp32 matrix slab[slot_ids[b], h] (b < batch, h < heads,
 * `matrix` floats each, a positive multiple of 4; slab laid out (num_slots,
 * heads, matrix) as gdr_forward's slab) and touches nothing else, so it moves
 * exactly the state bytes a decode step over the same slot ids reads and
 * writes, in the same order of requests.  factor = 1 leaves the values
 * unchanged.  A slot id outside [0, num_slots) skips its request, as in
 * gdr_forward.  slab (16-byte aligned) and slot_ids are device memory owned
 * by the caller; enqueued on `stream`.  GDR_E_INVALID for bad sizes, NULL or
 * misaligned pointers, or a grid past one launch's limit. */
gdr_status gdr_slab_stream(float *slab, const int32_t *slot_ids, int32_t batch, int32_t heads, int64_t matrix,
                           int32_t num_slots, float factor, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
