/*
 * gdr_oracle.c -- fp64 CPU oracle for the gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no header, helper, table or constant with
 * the HIP library.
 *
 * What it computes (all arithmetic in double precision, inputs upcast
 * exactly from fp16/fp32 by the Python caller):
 *
 *   Per value head, with a V-major state S (dv rows, each a dk-vector),
 *   "com.microsoft.GatedDeltaNet" README, section Description:
 *     S_t = exp(g_t) * S_{t-1} + k_t (beta_t (v_t - exp(g_t) S_{t-1}^T k_t))^T
 *     o_t = scale * S_t^T q_t
 *   and update_rule (same README, section Attributes) keeps:
 *     linear      -> no decay, no retrieval, unscaled write k v^T
 *     gated       -> decay only
 *     delta       -> retrieval only
 *     gated_delta -> both
 *   The per-key-dimension decay (one log-decay per key channel) follows the
 *   Ascend "aclnnRecurrentGatedDeltaRule" page, section Formula (Diag(alpha_k)
 *   acting on the key axis of the dv x dk state), and the CLIKA
 *   "gatedDeltaUpdate" page ([B,T,HV,K] gate = per key dim).
 *   gated_delta_v2 is the Gated DeltaNet-2 recurrence of the ONNX issue
 *   "Spec gap: LinearAttention (opset 27) cannot represent Gated DeltaNet-2's
 *   channel-wise erase gate", sections "The GDN-2 recurrence" and "Proposed
 *   extension" (A):  S_t = D_t S_{t-1} - k_t (b_t o k_t)^T D_t S_{t-1} + k_t v_t^T
 *   with the erase gate b_t on the key axis (K-major reading); in the V-major
 *   rows used here that is  r_i = sum_j b_j k_j (D S)_ij,
 *   S_ij <- (D S)_ij - r_i k_j + v_i k_j.
 *
 * Step order is the textbook one, token by token, row by row:
 *   decay the row, retrieve from the decayed row, form the delta value,
 *   rank-1 write, read out from the updated row.
 *
 * Gates ("com.microsoft.GatedDeltaNet" README, Attributes gate_activation and
 * beta_activation; "com.microsoft.LinearAttentionGate", Description):
 *   qwen:    g = -exp(a_log[h]) * softplus(raw[t,h] + dt_bias[h])
 *            (CLIKA "gatedDeltaUpdate": gate_scale[h], the once-folded
 *            -exp(a_log[h]), may be bound instead of a_log; beside a per-key
 *            gate [T, HV, K] the bias is per key channel, dt_bias[h][j])
 *   sigmoid: beta = 1 / (1 + exp(-b))
 * qk_l2_norm (README, Attributes): x <- x / sqrt(sum x^2 + 1e-12).
 *
 * Requests (README, Inputs cu_seqlens): request b covers tokens
 * [clamp(cu[b],0,T), clamp(cu[b+1],0,T)); empty when the end is not past the
 * start, in which case its incoming state is copied to final_state (README,
 * Outputs final_state).  Without cu_seqlens the packing is uniform, L tokens
 * per request, or only the first seq_lens[b] of them (clamped to [0, L];
 * CLIKA "gatedDeltaUpdate": seq_lens bounds ragged prefill rows; the rest
 * of the request's rows produce no output).  slot_ids (same page): request b reads and
 * updates slab row slot_ids[b] in place; an id outside [0, num_slots) skips
 * the request (no state or output is touched).
 *
 * Parallelism: OpenMP over (request, value head, block of state rows).  Rows
 * of a V-major state evolve independently, so the split changes no result.
 *
 * gdro_gate (at the end of the file) is the standalone gate of the
 * "com.microsoft.LinearAttentionGate" README: decay and update rate only.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { RULE_LINEAR = 0, RULE_GATED = 1, RULE_DELTA = 2, RULE_GATED_DELTA = 3, RULE_GATED_DELTA_V2 = 4 };

typedef struct {
    int64_t T;          /* total tokens */
    int32_t B;          /* requests */
    int32_t L;          /* uniform request length (used when cu_seqlens is NULL) */
    int32_t H, HV, DK, DV;
    int32_t rule;       /* RULE_* */
    int32_t gate_qwen;  /* 1: gate is the raw projection, decay formed from a_log/dt_bias */
    int32_t beta_sigmoid;
    int32_t qk_l2_norm;
    int32_t per_key;    /* gate shaped (T, HV, DK) instead of (T, HV) */
    int32_t erase_value_axis; /* 0: erase gate on the key axis (adopted); 1: value-axis parse */
    int32_t num_slots;  /* > 0: state is a slab addressed by slot_ids */
    int32_t row_block;  /* rows per parallel work item (0 -> 16) */
    double scale;       /* 0 -> 1/sqrt(DK) */
    const double *q, *k, *v;          /* (T,H,DK) (T,H,DK) (T,HV,DV) */
    const double *gate;               /* (T,HV) or (T,HV,DK), or NULL */
    const double *beta;               /* (T,HV) or NULL */
    const double *erase;              /* (T,HV,DK) or NULL */
    const double *a_log, *dt_bias;    /* (HV) each, or NULL */
    const int32_t *cu_seqlens;        /* (B+1) or NULL */
    const int32_t *slot_ids;          /* (B) or NULL */
    const double *initial_state;      /* (B,HV,DV,DK) or NULL (zeros); unused with slots */
    double *o;                        /* (T,HV,DV) */
    double *state;                    /* (B,HV,DV,DK) final state, or the slab in place */
    const double *gate_scale;         /* (HV) folded -exp(a_log), or NULL (then a_log) */
    const int32_t *seq_lens;          /* (B) valid tokens per uniform request, or NULL */
} gdro_problem;

static double softplus(double x)
{
    /* log(1 + e^x), written so neither branch overflows */
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static int has_decay(int rule)
{
    return rule == RULE_GATED || rule == RULE_GATED_DELTA || rule == RULE_GATED_DELTA_V2;
}

static int has_beta(int rule) { return rule == RULE_DELTA || rule == RULE_GATED_DELTA; }

static int has_retrieval(int rule)
{
    return rule == RULE_DELTA || rule == RULE_GATED_DELTA || rule == RULE_GATED_DELTA_V2;
}

static void request_range(const gdro_problem *p, int b, int64_t *s, int64_t *e)
{
    if (p->cu_seqlens) {
        int64_t a = p->cu_seqlens[b], z = p->cu_seqlens[b + 1];
        if (a < 0) a = 0;
        if (a > p->T) a = p->T;
        if (z < 0) z = 0;
        if (z > p->T) z = p->T;
        *s = a;
        *e = z > a ? z : a;
    } else {
        int64_t len = p->L;
        if (p->seq_lens) {
            len = p->seq_lens[b];
            if (len < 0) len = 0;
            if (len > p->L) len = p->L;
        }
        *s = (int64_t)b * p->L;
        *e = *s + len;
    }
}

/* One (request, head, row block): rows [r0, r1) of that head's state. */
static void run_block(const gdro_problem *p, int b, int h, int r0, int r1,
                      double *qn, double *kn, double *alpha)
{
    const int DK = p->DK, DV = p->DV, H = p->H, HV = p->HV;
    const int qh = (int)(((int64_t)h * H) / HV);  /* grouped heads: floor(h*H/HV) */
    const double scale = p->scale != 0.0 ? p->scale : 1.0 / sqrt((double)DK);
    const size_t head_elems = (size_t)DV * DK;

    double *S;
    const double *S0 = NULL;
    if (p->num_slots > 0) {
        int32_t slot = p->slot_ids[b];
        if (slot < 0 || slot >= p->num_slots) return;     /* skipped request */
        S = p->state + ((size_t)slot * HV + h) * head_elems;
        /* in place: S is both the incoming and the outgoing state */
    } else {
        S = p->state + ((size_t)b * HV + h) * head_elems;
        if (p->initial_state) S0 = p->initial_state + ((size_t)b * HV + h) * head_elems;
        for (int i = r0; i < r1; ++i)
            for (int j = 0; j < DK; ++j)
                S[(size_t)i * DK + j] = S0 ? S0[(size_t)i * DK + j] : 0.0;
    }

    int64_t s, e;
    request_range(p, b, &s, &e);
    for (int64_t t = s; t < e; ++t) {
        /* 1. query / key vectors, optionally L2-normalised */
        const double *qt = p->q + ((size_t)t * H + qh) * DK;
        const double *kt = p->k + ((size_t)t * H + qh) * DK;
        double qss = 0.0, kss = 0.0;
        for (int j = 0; j < DK; ++j) { qss += qt[j] * qt[j]; kss += kt[j] * kt[j]; }
        double qs = p->qk_l2_norm ? 1.0 / sqrt(qss + 1e-12) : 1.0;
        double ks = p->qk_l2_norm ? 1.0 / sqrt(kss + 1e-12) : 1.0;
        for (int j = 0; j < DK; ++j) { qn[j] = qt[j] * qs; kn[j] = kt[j] * ks; }

        /* 2. decay factor per key channel (constant over j for a per-head gate) */
        for (int j = 0; j < DK; ++j) alpha[j] = 1.0;
        if (has_decay(p->rule)) {
            for (int j = 0; j < DK; ++j) {
                double raw = p->per_key ? p->gate[((size_t)t * HV + h) * DK + j]
                                        : p->gate[(size_t)t * HV + h];
                double g = raw;
                if (p->gate_qwen) {
                    double gs = p->gate_scale ? p->gate_scale[h] : -exp(p->a_log[h]);
                    double bias = p->per_key ? p->dt_bias[(size_t)h * DK + j] : p->dt_bias[h];
                    g = gs * softplus(raw + bias);
                }
                alpha[j] = exp(g);
            }
        }

        /* 3. update rate */
        double beta = 1.0;
        if (has_beta(p->rule)) {
            beta = p->beta[(size_t)t * HV + h];
            if (p->beta_sigmoid) beta = sigmoid(beta);
        }
        const double *bt = p->rule == RULE_GATED_DELTA_V2 ? p->erase + ((size_t)t * HV + h) * DK : NULL;
        const double *vt = p->v + ((size_t)t * HV + h) * DV;
        double *ot = p->o + ((size_t)t * HV + h) * DV;

        /* 4. every state row, textbook order */
        for (int i = r0; i < r1; ++i) {
            double *Si = S + (size_t)i * DK;
            for (int j = 0; j < DK; ++j) Si[j] *= alpha[j];                  /* decay */
            double vprime = vt[i];
            if (has_retrieval(p->rule)) {
                double r = 0.0;
                if (bt && !p->erase_value_axis) {
                    for (int j = 0; j < DK; ++j) r += Si[j] * bt[j] * kn[j]; /* erase on key axis */
                } else {
                    for (int j = 0; j < DK; ++j) r += Si[j] * kn[j];          /* S^T k, row i */
                    if (bt) r *= bt[i];                                       /* value-axis parse */
                }
                if (p->rule == RULE_GATED_DELTA_V2)
                    vprime = vt[i] - r;          /* erase r_i k^T, write v_i k^T */
                else
                    vprime = beta * (vt[i] - r);
            }
            for (int j = 0; j < DK; ++j) Si[j] += vprime * kn[j];            /* rank-1 write */
            double acc = 0.0;
            for (int j = 0; j < DK; ++j) acc += Si[j] * qn[j];               /* read out S_t^T q */
            ot[i] = scale * acc;
        }
    }
}

/* Returns 0 on success, a negative code on inconsistent arguments. */
int gdro_forward(const gdro_problem *p)
{
    if (!p || !p->q || !p->k || !p->v || !p->o || !p->state) return -1;
    if (p->H <= 0 || p->HV <= 0 || p->HV % p->H != 0 || p->DK <= 0 || p->DV <= 0 || p->B < 0) return -2;
    if (has_decay(p->rule) && !p->gate) return -3;
    if (has_beta(p->rule) && !p->beta) return -4;
    if (p->rule == RULE_GATED_DELTA_V2 && !p->erase) return -5;
    if (p->gate_qwen && ((!p->a_log && !p->gate_scale) || !p->dt_bias)) return -6;
    if (p->num_slots > 0 && !p->slot_ids) return -7;
    if (p->rule < RULE_LINEAR || p->rule > RULE_GATED_DELTA_V2) return -8;
    if (!p->cu_seqlens && (int64_t)p->B * p->L != p->T) return -9;
    const int rb = p->row_block > 0 ? p->row_block : 16;
    const int nblk = (p->DV + rb - 1) / rb;
    const long items = (long)p->B * p->HV * nblk;

#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * 3 * (size_t)p->DK);
        double *qn = scratch, *kn = scratch + p->DK, *alpha = scratch + 2 * p->DK;
#pragma omp for schedule(dynamic, 1)
        for (long it = 0; it < items; ++it) {
            int blk = (int)(it % nblk);
            int h = (int)((it / nblk) % p->HV);
            int b = (int)(it / ((long)nblk * p->HV));
            int r0 = blk * rb, r1 = r0 + rb < p->DV ? r0 + rb : p->DV;
            run_block(p, b, h, r0, r1, qn, kn, alpha);
        }
        free(scratch);
    }
    return 0;
}

/* Standalone gate fusion, "com.microsoft.LinearAttentionGate" README,
 * Description and Outputs: for each of `count` elements n of a tensor whose
 * last axis holds the `heads` heads (element n belongs to head h = n mod heads),
 *     decay = decay_scale[h] * softplus(a + dt_bias[h])
 *     beta  = sigmoid(b)                       (only when beta is requested)
 * in double precision; the page narrows only on store, which the caller's
 * comparison accounts for.  Returns 0, or a negative code on bad arguments. */
int gdro_gate(int64_t count, int32_t heads, const double *a, const double *dt_bias,
              const double *decay_scale, const double *b, double *decay, double *beta)
{
    if (count < 0 || heads < 1 || count % heads != 0) return -1;
    if (count > 0 && (!a || !dt_bias || !decay_scale || !decay)) return -2;
    if (beta && !b) return -3;
    for (int64_t n = 0; n < count; ++n) {
        const int64_t head = n % heads;
        decay[n] = decay_scale[head] * softplus(a[n] + dt_bias[head]);
        if (beta) beta[n] = sigmoid(b[n]);
    }
    return 0;
}

/* Number of OpenMP threads the oracle will use (reported as the CPU core count). */
int gdro_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
