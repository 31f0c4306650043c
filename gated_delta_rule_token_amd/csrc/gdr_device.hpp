// gdr_device.hpp -- device-side building blocks shared by the gated delta-rule
// kernels (gfx950 / CDNA4, wave64).
//
// The recurrence (the "com.microsoft.GatedDeltaNet" README, Description) is
// evaluated per V-major state row i (a dk-vector S_i).  Because
//   S_i' = alpha (.) S_i + c_i k,    c_i = beta (v_i - (alpha (.) S_i) . k)
// the new row and the read-out o_i = scale S_i' . q both follow from two dot
// products of the OLD row with per-token vectors:
//   r_i = S_i . (alpha (.) k),  u_i = S_i . (alpha (.) q),
//   o_i = scale (u_i + (q . k) c_i)
// so every kernel reads a row once, reduces two partial sums across the 16
// lanes that hold the row, and writes it once.  (For a per-head scalar decay
// alpha is factored out of the dot products.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_chunk_plan.hpp"

namespace gdr {

enum Rule : int { LINEAR = 0, GATED = 1, DELTA = 2, GATED_DELTA = 3, GATED_DELTA_V2 = 4 };

__host__ __device__ constexpr bool rule_decays(int r) { return r == GATED || r == GATED_DELTA || r == GATED_DELTA_V2; }
__host__ __device__ constexpr bool rule_has_beta(int r) { return r == DELTA || r == GATED_DELTA; }
__host__ __device__ constexpr bool rule_retrieves(int r) { return r == DELTA || r == GATED_DELTA || r == GATED_DELTA_V2; }

// Kernel argument block, passed by value.
struct Params {
    const void *q, *k, *v;
    void *o;
    const void *gate;
    const float *beta, *erase, *a_log, *dt_bias;
    const float *gate_scale;   // folded -exp(a_log) per head, or nullptr (then a_log)
    const int32_t *cu_seqlens, *slot_ids;
    const int32_t *seq_lens;   // valid tokens per uniform-packed request, or nullptr
    const float *init;      // incoming states (B,HV,dv,dk) or nullptr (zeros); unused with slots
    float *state;           // outgoing states, or the slab updated in place
    int64_t T;
    int32_t B, L, H, HV, dk, dv, num_slots;
    int32_t gate_qwen, gate_dt, beta_sigmoid, qk_l2_norm;  // gate_dt: 0 fp32, 1 fp16, 2 bf16
    int32_t beta_bcast;        // 1: beta is (T, 1), one update rate per token for every head
    float scale;
    // (B * HV) flags, or nullptr: the recurrent kernel then runs only the
    // (request, value head) pairs whose flag is set (the chunked form's
    // hand-over of the pairs it did not take)
    const int32_t *run_only;
};

typedef _Float16 half_t;
typedef __bf16 bf16_t;

template <typename TA> __device__ __forceinline__ float to_f32(TA x) { return static_cast<float>(x); }
template <typename TA> __device__ __forceinline__ TA from_f32(float x) { return static_cast<TA>(x); }

// ---------------------------------------------------------------- lane reductions
// DPP moves within a 16-lane row.  Every step adds a bitwise-identical pair in
// both partner lanes (fp addition commutes), so after the four steps all 16
// lanes hold the same sum, which keeps redundant per-row work consistent.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float sum16(float x)
{
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
    x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <-> 7 - i within 8
    x += dpp_mov<0x140>(x);  // row_mirror: lane i <-> 15 - i within 16
    return x;
}

// ---------------------------------------------------------------- barriers
// Workgroup barrier that orders LDS only.  __syncthreads() also releases
// global memory, which makes every wave wait for its outstanding global loads
// (vmcnt 0) -- including loads issued early on purpose to prefetch the next
// block.  Kernels whose waves exchange data through LDS only use this one.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- gate math (fp32)
// softplus(x) = log(1 + e^x), evaluated without overflow on either side.
__device__ __forceinline__ float softplus_f32(float x)
{
    return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.f / (1.f + expf(-x)); }

// Scale of the raw-gate arm for head h: -exp(a_log[h]) (README Attributes
// gate_activation), or the caller's once-folded gate_scale[h] (CLIKA
// "gatedDeltaUpdate": gate_bias and gate_scale bound together).
__device__ __forceinline__ float gate_scale(const Params &p, int h)
{
    return p.gate_scale ? p.gate_scale[h] : -expf(p.a_log[h]);
}

// One gate element: fp32, or the activations' 16-bit dtype (raw-gate arm).
__device__ __forceinline__ float load_gate(const Params &p, size_t idx)
{
    if (p.gate_dt == 1) return to_f32(static_cast<const half_t *>(p.gate)[idx]);
    if (p.gate_dt == 2) return to_f32(static_cast<const bf16_t *>(p.gate)[idx]);
    return static_cast<const float *>(p.gate)[idx];
}

// Log decay g for token t, head h (scalar gate): README Attributes
// gate_activation; the raw-gate arm reads the projection in its dtype.
__device__ __forceinline__ float log_decay(const Params &p, size_t idx, int h)
{
    float x = load_gate(p, idx);
    if (p.gate_qwen) x = gate_scale(p, h) * softplus_f32(x + p.dt_bias[h]);
    return x;
}

// Raw-gate arm of a per-key gate: x is key channel j of head h's projection;
// the bias is per (head, key channel), [HV, K] beside a [B, T, HV, K] gate
// (CLIKA "gatedDeltaUpdate").
__device__ __forceinline__ float key_decay_from_raw(const Params &p, float x, int h, int j)
{
    return gate_scale(p, h) * softplus_f32(x + p.dt_bias[(size_t)h * p.dk + j]);
}

// Log decay of key channel j for token-head th (= t * HV + h) of a per-key gate.
__device__ __forceinline__ float log_decay_key(const Params &p, size_t th, int h, int j)
{
    const float x = load_gate(p, th * p.dk + j);
    return p.gate_qwen ? key_decay_from_raw(p, x, h, j) : x;
}

// Element of beta for token-head th (= t * HV + h); a (T, 1) beta is one rate
// per token for every value head (the ONNX issue's LinearAttention schema
// restricts beta's last axis to {kv_num_heads, 1}).
__device__ __forceinline__ size_t beta_index(const Params &p, size_t th)
{
    return p.beta_bcast ? th / (size_t)p.HV : th;
}

__device__ __forceinline__ float update_rate(const Params &p, size_t th)
{
    float b = p.beta[beta_index(p, th)];
    return p.beta_sigmoid ? sigmoid_f32(b) : b;
}

// ---------------------------------------------------------------- addressing
// Request b's token range: README Inputs cu_seqlens (clamped to [0,T]; a
// decreasing entry gives an empty request) or uniform packing, optionally
// bounded by seq_lens[b] clamped to [0, L] (CLIKA "gatedDeltaUpdate": seq_lens
// bounds ragged prefill rows).
__device__ __forceinline__ void request_range(const Params &p, int b, int64_t &s, int64_t &e)
{
    if (p.cu_seqlens) {
        clamp_request(p.cu_seqlens[b], p.cu_seqlens[b + 1], p.T, s, e);
    } else {
        s = (int64_t)b * p.L;
        int64_t len = p.L;
        if (p.seq_lens) {
            len = p.seq_lens[b];
            len = len < 0 ? 0 : (len > p.L ? p.L : len);
        }
        e = s + len;
    }
}

// Base element offsets of request b / head h's incoming and outgoing state.
// Returns false when the request is skipped (slot id out of range).
__device__ __forceinline__ bool state_ptrs(const Params &p, int b, int h, const float *&src, float *&dst)
{
    const size_t head = (size_t)p.dv * p.dk;
    if (p.num_slots > 0) {
        const int32_t slot = p.slot_ids[b];
        if (slot < 0 || slot >= p.num_slots) return false;
        dst = p.state + ((size_t)slot * p.HV + h) * head;
        src = dst;
    } else {
        dst = p.state + ((size_t)b * p.HV + h) * head;
        src = p.init ? p.init + ((size_t)b * p.HV + h) * head : nullptr;
    }
    return true;
}

// ---------------------------------------------------------------- vector loads
template <typename TA, int N>
__device__ __forceinline__ void load_act(const TA *__restrict__ ptr, float (&out)[N])
{
    if constexpr (sizeof(TA) == 2 && N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const uint2 w = *reinterpret_cast<const uint2 *>(ptr + i);
            const TA *h = reinterpret_cast<const TA *>(&w);
            out[i] = to_f32(h[0]); out[i + 1] = to_f32(h[1]);
            out[i + 2] = to_f32(h[2]); out[i + 3] = to_f32(h[3]);
        }
    } else if constexpr (sizeof(TA) == 4 && N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 w = *reinterpret_cast<const float4 *>(ptr + i);
            out[i] = w.x; out[i + 1] = w.y; out[i + 2] = w.z; out[i + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = to_f32(ptr[i]);
    }
}

template <typename TA, int N>
__device__ __forceinline__ void load_act_masked(const TA *__restrict__ ptr, int valid, float (&out)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = i < valid ? to_f32(ptr[i]) : 0.f;
}

}  // namespace gdr
