// gdr_api.cpp -- the C ABI of libgdr (declared in include/gdr.h): host-side
// argument validation, kernel selection and launch.  Nothing here touches
// tensor memory; cu_seqlens and slot_ids stay on the device.
#include "gdr.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "gdr_launch.hpp"

// Workspace of gdr_forward_noalloc, one copy per GPU (see include/gdr.h).  In
// host code `scratch` is only a handle: its device address comes from
// hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

gdr_status fail(gdr_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dsize(int32_t dt) { return dt == GDR_F32 ? 4 : 2; }

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Number of state rows (batch or slab) the final_state buffer holds.
int64_t state_rows(const gdr_problem *p) { return p->num_slots > 0 ? p->num_slots : p->batch; }

// Shapes the chunk-parallel kernels implement (every rule; a per-key decay
// and the erase gate take the per-key form).
bool chunked_per_key(const gdr_problem *p)
{
    return p->decay_per_key != 0 || p->update_rule == GDR_RULE_GATED_DELTA_V2;
}

bool chunked_ok(const gdr_problem *p)
{
    return p->head_dim_k == 128 && p->head_dim_v == 128 && (p->act_dtype == GDR_F16 || p->act_dtype == GDR_BF16);
}

gdr_status check_problem(const gdr_problem *p)
{
    if (!p) return fail(GDR_E_INVALID, "problem is NULL");
    if (p->state_update_capacity != 0)
        return fail(GDR_E_UNSUPPORTED, "state_update_capacity must be 0 (compact capture is not implemented)");
    if (p->beta_per_token != 0 && p->beta_per_token != 1) return fail(GDR_E_INVALID, "beta_per_token must be 0 or 1");
    if (p->beta_per_token && !gdr::rule_has_beta(p->update_rule))
        return fail(GDR_E_INVALID, "beta_per_token given to an update_rule without beta");
    if (p->act_dtype != GDR_F32 && p->act_dtype != GDR_F16 && p->act_dtype != GDR_BF16)
        return fail(GDR_E_INVALID, "act_dtype must be GDR_F32, GDR_F16 or GDR_BF16");
    if (p->gate_dtype != GDR_F32 && p->gate_dtype != p->act_dtype)
        return fail(GDR_E_INVALID, "gate_dtype must be GDR_F32 or the activation dtype");
    if (p->update_rule < GDR_RULE_LINEAR || p->update_rule > GDR_RULE_GATED_DELTA_V2)
        return fail(GDR_E_INVALID, "update_rule %d out of range", p->update_rule);
    if (p->gate_activation != GDR_GATE_NONE && p->gate_activation != GDR_GATE_QWEN)
        return fail(GDR_E_INVALID, "gate_activation %d out of range", p->gate_activation);
    if (p->beta_activation != GDR_BETA_NONE && p->beta_activation != GDR_BETA_SIGMOID)
        return fail(GDR_E_INVALID, "beta_activation %d out of range", p->beta_activation);
    if (p->algo < GDR_ALGO_AUTO || p->algo > GDR_ALGO_CHUNKED)
        return fail(GDR_E_INVALID, "algo %d out of range", p->algo);
    if (p->num_heads_qk < 1 || p->num_heads_v < 1 || p->num_heads_v % p->num_heads_qk != 0)
        return fail(GDR_E_INVALID, "num_heads_v (%d) must be a positive multiple of num_heads_qk (%d)",
                    p->num_heads_v, p->num_heads_qk);
    if (p->head_dim_k < 1 || p->head_dim_k > 256 || p->head_dim_v < 1 || p->head_dim_v > 256)
        return fail(GDR_E_INVALID, "head dims must lie in [1, 256] (dk=%d, dv=%d)", p->head_dim_k, p->head_dim_v);
    if (p->total_tokens < 0 || p->batch < 0 || p->seq_len < 0 || p->num_slots < 0 || p->chunk_size < 0)
        return fail(GDR_E_INVALID, "negative size");
    if (p->total_tokens > INT32_MAX) return fail(GDR_E_INVALID, "total_tokens above 2^31-1");
    if (p->scan_segments < 0 || p->scan_segments > 16) return fail(GDR_E_INVALID, "scan_segments must lie in [0, 16]");
    const bool decays = gdr::rule_decays(p->update_rule);
    if (p->gate_activation == GDR_GATE_QWEN && !decays)
        return fail(GDR_E_INVALID, "gate_activation qwen needs a decayed update_rule");
    if (p->decay_per_key && !decays) return fail(GDR_E_INVALID, "decay_per_key needs a decayed update_rule");
    if (!std::isfinite(p->scale)) return fail(GDR_E_INVALID, "scale is not finite");
    const int64_t blocks = (int64_t)p->batch * p->num_heads_v * 16;
    if (blocks > INT32_MAX) return fail(GDR_E_INVALID, "batch * num_heads_v too large");
    if (p->algo == GDR_ALGO_DECODE && (p->head_dim_k != 128 || p->head_dim_v != 128))
        return fail(GDR_E_UNSUPPORTED, "the decode kernel needs dk = dv = 128");
    if (p->algo == GDR_ALGO_CHUNKED && !chunked_ok(p))
        return fail(GDR_E_UNSUPPORTED, "the chunked kernels need dk = dv = 128 and fp16 or bf16 activations");
    return GDR_OK;
}

gdr_status check_tensors(const gdr_problem *p, const gdr_tensors *t)
{
    const int rule = p->update_rule;
    const bool decays = gdr::rule_decays(rule);
    const bool has_beta = gdr::rule_has_beta(rule);
    const bool v2 = rule == GDR_RULE_GATED_DELTA_V2;
    const bool qwen = p->gate_activation == GDR_GATE_QWEN;
    const int64_t T = p->total_tokens;

    if (p->rank4 && t->cu_seqlens) return fail(GDR_E_INVALID, "cu_seqlens requires the rank-3 spelling");
    if (!t->cu_seqlens) {
        if ((int64_t)p->batch * p->seq_len != T)
            return fail(GDR_E_INVALID, "uniform packing needs total_tokens == batch * seq_len (%lld != %d * %d)",
                        (long long)T, p->batch, p->seq_len);
    }
    // Token-indexed inputs may be NULL when there are no tokens (a zero-size
    // tensor has no storage); otherwise presence follows the update rule.
    if (t->gate && !decays) return fail(GDR_E_INVALID, "gate given to an update_rule without decay");
    if (t->beta && !has_beta) return fail(GDR_E_INVALID, "beta given to an update_rule without it");
    if (t->erase && !v2) return fail(GDR_E_INVALID, "erase given to an update_rule without it");
    if (T > 0 && decays && !t->gate) return fail(GDR_E_INVALID, "gate is required by this update_rule");
    if (T > 0 && has_beta && !t->beta) return fail(GDR_E_INVALID, "beta is required by this update_rule");
    if (T > 0 && v2 && !t->erase) return fail(GDR_E_INVALID, "erase is required by gated_delta_v2");
    if (qwen) {
        if (!t->dt_bias || (t->a_log != nullptr) == (t->gate_scale != nullptr))
            return fail(GDR_E_INVALID, "gate_activation qwen requires dt_bias and exactly one of a_log, gate_scale");
    } else if (t->a_log || t->dt_bias || t->gate_scale) {
        return fail(GDR_E_INVALID, "a_log/gate_scale/dt_bias given without gate_activation qwen");
    }
    if (t->seq_lens && t->cu_seqlens) return fail(GDR_E_INVALID, "seq_lens bounds uniform packing; not with cu_seqlens");
    if ((p->num_slots > 0) != (t->slot_ids != nullptr))
        return fail(GDR_E_INVALID, "slot_ids must be given exactly when num_slots > 0");
    if (p->num_slots > 0 && t->initial_state)
        return fail(GDR_E_INVALID, "with a slot slab the state is read in place; initial_state must be NULL");
    if (!t->final_state && state_rows(p) > 0) return fail(GDR_E_INVALID, "final_state (or the slab) is required");
    if (T > 0 && (!t->q || !t->k || !t->v || !t->o)) return fail(GDR_E_INVALID, "q, k, v and o are required");
    if (p->batch > 0 && !t->cu_seqlens && p->seq_len == 0 && T != 0)
        return fail(GDR_E_INVALID, "seq_len must be set without cu_seqlens");

    const void *ptrs[] = {t->q, t->k, t->v, t->o, t->gate, t->beta, t->erase, t->a_log, t->dt_bias,
                          t->cu_seqlens, t->slot_ids, t->initial_state, t->final_state, t->gate_scale,
                          t->seq_lens};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return fail(GDR_E_INVALID, "every tensor pointer must be 16-byte aligned");

    // aliasing: outputs must not overlap inputs or each other; final == initial is the in-place case
    const int64_t H = p->num_heads_qk, HV = p->num_heads_v, dk = p->head_dim_k, dv = p->head_dim_v;
    const size_t a = dsize(p->act_dtype);
    const size_t state_bytes = (size_t)state_rows(p) * HV * dv * dk * 4;
    auto rng = [](const char *n, const void *ptr, size_t bytes) {
        uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
        return Range{n, lo, ptr ? lo + bytes : lo};
    };
    const Range out_o = rng("o", t->o, (size_t)T * HV * dv * a);
    const Range out_s = rng("final_state", t->final_state, state_bytes);
    const Range ins[] = {
        rng("q", t->q, (size_t)T * H * dk * a),
        rng("k", t->k, (size_t)T * H * dk * a),
        rng("v", t->v, (size_t)T * HV * dv * a),
        rng("gate", t->gate, (size_t)T * HV * (p->decay_per_key ? dk : 1) * dsize(p->gate_dtype)),
        rng("beta", t->beta, (size_t)T * (p->beta_per_token ? 1 : HV) * 4),
        rng("erase", t->erase, (size_t)T * HV * dk * 4),
        rng("a_log", t->a_log, (size_t)HV * 4),
        rng("gate_scale", t->gate_scale, (size_t)HV * 4),
        rng("dt_bias", t->dt_bias, (size_t)HV * (p->decay_per_key ? dk : 1) * 4),
        rng("seq_lens", t->seq_lens, (size_t)p->batch * 4),
        rng("cu_seqlens", t->cu_seqlens, (size_t)(p->batch + 1) * 4),
        rng("slot_ids", t->slot_ids, (size_t)p->batch * 4),
        rng("initial_state", t->initial_state, (size_t)p->batch * HV * dv * dk * 4),
    };
    if (overlaps(out_o, out_s)) return fail(GDR_E_ALIAS, "o overlaps final_state");
    for (const Range &r : ins) {
        if (overlaps(out_o, r)) return fail(GDR_E_ALIAS, "o overlaps %s", r.name);
        const bool same_state = r.name[0] == 'i' && r.lo == out_s.lo && r.hi == out_s.hi;
        if (!same_state && overlaps(out_s, r)) return fail(GDR_E_ALIAS, "final_state overlaps %s", r.name);
    }
    return GDR_OK;
}

int32_t pick_algo(const gdr_problem *p)
{
    if (p->algo != GDR_ALGO_AUTO) return p->algo;
    const bool d128 = p->head_dim_k == 128 && p->head_dim_v == 128;
    // tokens per request on average; decode when requests are a handful of tokens
    const int64_t per_req = p->batch > 0 ? (p->total_tokens + p->batch - 1) / p->batch : 0;
    if (d128 && per_req <= 8) return GDR_ALGO_DECODE;
    // long requests: the chunk-parallel form when its shapes are supported
    if (chunked_ok(p) && per_req >= 128) return GDR_ALGO_CHUNKED;
    return GDR_ALGO_RECURRENT;
}

// Segments of the chunked scan's chain: the caller's count, or a split of
// long requests when few (request, head) pairs leave most CUs idle.  The
// count gives pass 2 about 64 (request, head, segment) groups -- 256
// workgroups, one per CU, in 32-row tiles (or 16-row tiles when there are
// at most 32 groups) -- and pass 1 twice that; with a power-of-two number of
// pairs every CU gets the same number of workgroups (uneven counts leave
// some CUs one more than the rest).  At most 16 segments of at least 16
// chunks each.  Measured on
// MI355X (prologue + scan, one request): 65,536 tokens x 16 heads 2.0 ms in
// one pass, 1.68 / 1.81 / 1.55 / 1.94 ms in 3 / 4 / 5 / 6 segments; x 8 heads
// 1.71 ms, 1.01 / 0.94 ms in 5 / 9; 32,768 tokens x 4 heads 0.70 ms,
// 0.36 / 0.41 ms in 9 / 16; 16,384 tokens x 16 heads 0.55 -> 0.47 ms in 5;
// shorter requests gain nothing and 32 pairs or more lose (32,768 tokens x
// 32 heads 1.35 -> 1.36 ms in 3).
int scan_segments(const gdr_problem *p)
{
    if (p->scan_segments > 0) return p->scan_segments;
    const int64_t pairs = (int64_t)p->batch * p->num_heads_v;
    const int64_t chunks_per_req = p->batch > 0 ? p->total_tokens / p->batch / 64 : 0;
    if (pairs < 1 || pairs > 16 || chunks_per_req < 256) return 1;
    int64_t groups = 64 / pairs;  // (request, head, segment) groups per pair in pass 2
    while (groups > 15) groups /= 2;
    if (groups > chunks_per_req / 16 - 1) groups = chunks_per_req / 16 - 1;
    return groups >= 2 ? (int)groups + 1 : 1;
}

int dk_tile(int dk) { return dk <= 32 ? 32 : dk <= 64 ? 64 : dk <= 128 ? 128 : 256; }

// rows per workgroup = 16 * g.  Measured on MI355X (dv = 128): g = 2 beats
// g = 4 (more workgroups per CU to hide the token loop's latency) and g = 1
// (per-token staging amortised over too few rows) on both the varlen and the
// per-key workloads.
int rows_group(const gdr_problem *p)
{
    return p->head_dim_v <= 16 ? 1 : 2;
}

gdr_status fail(gdr_status st, const char *fmt, ...);

// Device address of the current device's scratch copy, looked up once per device.
gdr_status scratch_address(void **out)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(GDR_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(GDR_E_UNSUPPORTED, "device ordinal %d beyond %d", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !ptr)
            return fail(GDR_E_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(err));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GDR_OK;
}

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char *gdr_status_str(gdr_status s)
{
    switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_E_INVALID: return "GDR_E_INVALID";
    case GDR_E_UNSUPPORTED: return "GDR_E_UNSUPPORTED";
    case GDR_E_ALIAS: return "GDR_E_ALIAS";
    case GDR_E_WORKSPACE: return "GDR_E_WORKSPACE";
    case GDR_E_HIP: return "GDR_E_HIP";
    }
    return "GDR_E_UNKNOWN";
}

const char *gdr_last_error(void) { return g_last_error.c_str(); }

gdr_status gdr_validate(const gdr_problem *problem, const gdr_tensors *tensors)
{
    g_last_error.clear();
    gdr_status st = check_problem(problem);
    if (st != GDR_OK || !tensors) return st;
    return check_tensors(problem, tensors);
}

gdr_status gdr_workspace_size(const gdr_problem *problem, size_t *bytes)
{
    g_last_error.clear();
    if (!bytes) return fail(GDR_E_INVALID, "bytes is NULL");
    gdr_status st = check_problem(problem);
    if (st != GDR_OK) return st;
    *bytes = pick_algo(problem) == GDR_ALGO_CHUNKED
                 ? gdr::chunked_workspace_bytes(problem->total_tokens, problem->batch, problem->num_heads_qk,
                                                problem->num_heads_v, chunked_per_key(problem), scan_segments(problem))
                 : 0;
    return GDR_OK;
}

gdr_status gdr_select_algo(const gdr_problem *problem, int32_t *algo)
{
    g_last_error.clear();
    if (!algo) return fail(GDR_E_INVALID, "algo is NULL");
    gdr_status st = check_problem(problem);
    if (st != GDR_OK) return st;
    *algo = pick_algo(problem);
    return GDR_OK;
}

}  // extern "C"

namespace {

// Enqueue every kernel of a validated call on `stream`; `workspace` holds at
// least gdr_workspace_size bytes.
gdr_status launch_all(const gdr_problem *problem, const gdr_tensors *tensors, void *workspace, void *stream)
{
    const gdr_problem &p = *problem;
    const gdr_tensors &t = *tensors;
    gdr::Params k{};
    k.q = t.q;
    k.k = t.k;
    k.v = t.v;
    k.o = t.o;
    k.gate = t.gate;
    k.beta = t.beta;
    k.erase = t.erase;
    k.a_log = t.a_log;
    k.dt_bias = t.dt_bias;
    k.gate_scale = t.gate_scale;
    k.seq_lens = t.seq_lens;
    k.cu_seqlens = t.cu_seqlens;
    k.slot_ids = t.slot_ids;
    k.init = t.initial_state;
    k.state = t.final_state;
    k.T = p.total_tokens;
    k.B = p.batch;
    k.L = t.cu_seqlens ? 0 : p.seq_len;
    k.H = p.num_heads_qk;
    k.HV = p.num_heads_v;
    k.dk = p.head_dim_k;
    k.dv = p.head_dim_v;
    k.num_slots = p.num_slots;
    k.gate_qwen = p.gate_activation == GDR_GATE_QWEN;
    k.gate_dt = p.gate_dtype == GDR_F16 ? 1 : p.gate_dtype == GDR_BF16 ? 2 : 0;
    k.beta_sigmoid = p.beta_activation == GDR_BETA_SIGMOID;
    k.qk_l2_norm = p.qk_l2_norm != 0;
    k.beta_bcast = p.beta_per_token != 0;
    k.scale = p.scale != 0.f ? p.scale : 1.f / std::sqrt((float)p.head_dim_k);
    if (p.batch == 0) return GDR_OK;

    const int act = p.act_dtype == GDR_F16 ? 1 : p.act_dtype == GDR_BF16 ? 2 : 0;
    const bool pk = p.decay_per_key != 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (pick_algo(problem)) {
    case GDR_ALGO_DECODE: err = gdr::launch_decode128(k, p.update_rule, pk, act, s); break;
    case GDR_ALGO_CHUNKED:
        err = gdr::launch_chunked(k, p.update_rule, pk, scan_segments(problem), act, workspace, s);
        break;
    default: err = gdr::launch_recurrent(k, p.update_rule, pk, act, dk_tile(p.head_dim_k), rows_group(problem), s); break;
    }
    if (err != hipSuccess) return fail(GDR_E_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_forward(const gdr_problem *problem, const gdr_tensors *tensors, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    g_last_error.clear();
    if (!tensors) return fail(GDR_E_INVALID, "tensors is NULL");
    gdr_status st = gdr_validate(problem, tensors);
    if (st != GDR_OK) return st;
    size_t need = 0;
    gdr_workspace_size(problem, &need);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GDR_E_WORKSPACE, "workspace of %zu bytes required", need);
    return launch_all(problem, tensors, workspace, stream);
}

gdr_status gdr_forward_noalloc(const gdr_problem *problem, const gdr_tensors *tensors, void *stream)
{
    g_last_error.clear();
    if (!tensors) return fail(GDR_E_INVALID, "tensors is NULL");
    gdr_status st = gdr_validate(problem, tensors);
    if (st != GDR_OK) return st;
    size_t need = 0;
    gdr_workspace_size(problem, &need);
    if (need > GDR_NOALLOC_SCRATCH_BYTES)
        return fail(GDR_E_WORKSPACE,
                    "this problem needs %zu bytes of workspace, above the %zu bytes gdr_forward_noalloc holds; "
                    "call gdr_forward with a workspace instead",
                    need, (size_t)GDR_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0) {
        st = scratch_address(&ws);
        if (st != GDR_OK) return st;
    }
    return launch_all(problem, tensors, ws, stream);
}

gdr_status gdr_gate(int64_t count, int32_t heads, int32_t dtype, const void *a, const float *dt_bias,
                    const float *decay_scale, const void *b, void *decay, void *beta, void *stream)
{
    g_last_error.clear();
    if (count < 0 || heads < 1) return fail(GDR_E_INVALID, "count must be >= 0 and heads >= 1");
    if (count % heads != 0) return fail(GDR_E_INVALID, "count must be a multiple of heads (last axis)");
    if (dtype != GDR_F32 && dtype != GDR_F16 && dtype != GDR_BF16)
        return fail(GDR_E_INVALID, "dtype must be GDR_F32, GDR_F16 or GDR_BF16");
    if (count > 0 && (!a || !dt_bias || !decay_scale || !decay)) return fail(GDR_E_INVALID, "a, dt_bias, decay_scale and decay are required");
    if (beta && !b) return fail(GDR_E_INVALID, "beta requested without b");
    hipError_t err = gdr::launch_gate(count, heads, dtype == GDR_F16 ? 1 : dtype == GDR_BF16 ? 2 : 0, a, dt_bias, decay_scale, beta ? b : nullptr,
                                      decay, beta, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(GDR_E_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

gdr_status gdr_slab_stream(float *slab, const int32_t *slot_ids, int32_t batch, int32_t heads, int64_t matrix,
                           int32_t num_slots, float factor, void *stream)
{
    g_last_error.clear();
    if (batch < 0 || heads < 1 || num_slots < 1) return fail(GDR_E_INVALID, "batch must be >= 0, heads and num_slots >= 1");
    if (matrix < 4 || matrix % 4 != 0) return fail(GDR_E_INVALID, "matrix must be a positive multiple of 4 floats");
    if (batch == 0) return GDR_OK;
    if (!slab || !slot_ids) return fail(GDR_E_INVALID, "slab and slot_ids are required");
    if (!aligned16(slab)) return fail(GDR_E_INVALID, "slab must be 16-byte aligned");
    if (gdr::slab_stream_blocks(batch, heads, matrix) > INT32_MAX)
        return fail(GDR_E_INVALID, "batch * heads * matrix is too large for one launch");
    hipError_t err = gdr::launch_slab_stream(slab, slot_ids, batch, heads, matrix, num_slots, factor,
                                             static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(GDR_E_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GDR_OK;
}

}  // extern "C"
