// gdr_recurrent.hip -- recurrent prefill kernel: a tile of state rows lives in
// VGPRs for the whole token loop of one (request, value head).
//
// Recurrence: "com.microsoft.GatedDeltaNet" README, Description, with the
// update_rule terms of its Attributes table; per-key decay from the Ascend
// "aclnnRecurrentGatedDeltaRule" Formula; the Gated DeltaNet-2 erase gate from
// the ONNX issue on LinearAttention (opset 27), "Proposed extension" (A).
//
// Layout of work:
//   workgroup = 256 threads = 4 waves, owns ROWS = 16*G consecutive state
//   rows of one (request b, value head h); grid = B * HV * ceil(dv / ROWS).
//   Inside a wave, 16 lanes hold one row (C = DKT/16 key columns each, as
//   VEC-wide interleaved chunks so global and LDS accesses are 16-byte
//   vectors), 4 rows per wave-instruction, G such row groups per wave.
//   Tokens are processed in staged blocks of NB: all 256 threads load the
//   block's q/k (fp16 or fp32), L2-normalise them (16-lane DPP reductions),
//   form the gate / update rate / per-key vectors in fp32 (the fused
//   prologue), and park everything in LDS; then each wave runs the serial
//   token loop on its rows from LDS, writing o into an LDS tile that is
//   stored coalesced after the block.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <typename TA, int RULE, bool PK, int DKT, int G>
__global__ __launch_bounds__(256) void k_recurrent(const Params p)
{
    constexpr int NT = 256;
    constexpr int C = DKT / 16;
    constexpr int VEC = C < 4 ? C : 4;
    constexpr int NCH = C / VEC;
    constexpr int RW = 4 * G;
    constexpr int ROWS = 4 * RW;
    constexpr bool VD = PK || RULE == GATED_DELTA_V2;  // decay applied per key column
    constexpr bool DEC = rule_decays(RULE);
    constexpr bool RET = rule_retrieves(RULE);
    constexpr bool BETA = rule_has_beta(RULE);
    constexpr int NB = (VD || DKT > 128) ? 16 : 32;

    __shared__ __align__(16) float s_k[NB][DKT];   // normalised k
    __shared__ __align__(16) float s_q[NB][DKT];   // normalised q (times alpha on the VD path)
    __shared__ __align__(16) float s_kb[VD ? NB : 1][DKT];  // erase * alpha * k
    __shared__ __align__(16) float s_a[VD ? NB : 1][DKT];   // alpha per key column
    __shared__ float s_sc[NB][4];                  // alpha (scalar), beta, q.k
    __shared__ float s_v[NB][ROWS];
    __shared__ float s_o[NB][ROWS];

    const int ntile = (p.dv + ROWS - 1) / ROWS;
    const int tile = blockIdx.x % ntile;
    const int h = (blockIdx.x / ntile) % p.HV;
    const int b = blockIdx.x / (ntile * p.HV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, r4 = lane >> 4;
    const int row0 = tile * ROWS;
    const int H = p.H, HV = p.HV, dk = p.dk, dv = p.dv;
    const int qh = (int)(((int64_t)h * H) / HV);
    const bool fullk = dk == DKT;

    const float *src;
    float *dst;
    if (!state_ptrs(p, b, h, src, dst)) return;
    int64_t s, e;
    request_range(p, b, s, e);

    const TA *__restrict__ q = static_cast<const TA *>(p.q);
    const TA *__restrict__ k = static_cast<const TA *>(p.k);
    const TA *__restrict__ v = static_cast<const TA *>(p.v);
    TA *__restrict__ o = static_cast<TA *>(p.o);

    // ---- state tile -> registers
    float S[G][C];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int row = row0 + wave * RW + g * 4 + r4;
#pragma unroll
        for (int m = 0; m < NCH; ++m)
#pragma unroll
            for (int x = 0; x < VEC; ++x) {
                const int col = m * 16 * VEC + l16 * VEC + x;
                S[g][m * VEC + x] = (src && row < dv && col < dk) ? src[(size_t)row * dk + col] : 0.f;
            }
    }

    for (int64_t t0 = s; t0 < e; t0 += NB) {
        const int nb = (int)((e - t0) < NB ? (e - t0) : NB);
        __syncthreads();

        // ---- A: q/k of the block, L2 norms, q.k, per-key decay vectors
        for (int task = tid; task < NB * 16; task += NT) {
            const int tau = task >> 4, c16 = task & 15;
            const int col0 = c16 * C;
            const int64_t t = t0 + tau;
            float qv[C], kv[C];
            if (tau < nb) {
                const TA *qp = q + ((size_t)t * H + qh) * dk + col0;
                const TA *kp = k + ((size_t)t * H + qh) * dk + col0;
                if (fullk) {
                    load_act<TA, C>(qp, qv);
                    load_act<TA, C>(kp, kv);
                } else {
                    load_act_masked<TA, C>(qp, dk - col0, qv);
                    load_act_masked<TA, C>(kp, dk - col0, kv);
                }
            } else {
#pragma unroll
                for (int c = 0; c < C; ++c) qv[c] = kv[c] = 0.f;
            }
            float qss = 0.f, kss = 0.f, qk = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                qss = fmaf(qv[c], qv[c], qss);
                kss = fmaf(kv[c], kv[c], kss);
                qk = fmaf(qv[c], kv[c], qk);
            }
            qss = sum16(qss);
            kss = sum16(kss);
            qk = sum16(qk);
            const float inq = p.qk_l2_norm ? 1.f / sqrtf(qss + 1e-12f) : 1.f;
            const float ink = p.qk_l2_norm ? 1.f / sqrtf(kss + 1e-12f) : 1.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                qv[c] *= inq;
                kv[c] *= ink;
            }
            if constexpr (VD) {
                float av[C], kb[C];
                const size_t th = (size_t)t * HV + h;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int col = col0 + c;
                    float a = 1.f, er = 1.f;
                    if (tau < nb && col < dk) {
                        a = expf(PK ? static_cast<const float *>(p.gate)[th * dk + col] : log_decay(p, th, h));
                        if constexpr (RULE == GATED_DELTA_V2) er = p.erase[th * dk + col];
                    }
                    av[c] = a;
                    kb[c] = er * a * kv[c];
                    qv[c] *= a;
                }
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    s_a[tau][col0 + c] = av[c];
                    s_kb[tau][col0 + c] = kb[c];
                }
            }
#pragma unroll
            for (int c = 0; c < C; ++c) {
                s_k[tau][col0 + c] = kv[c];
                s_q[tau][col0 + c] = qv[c];
            }
            if (c16 == 0) s_sc[tau][2] = qk * inq * ink;
        }

        // ---- B: per-token scalar gate and update rate (fp32)
        if (tid < NB) {
            float a = 1.f, bb = 1.f;
            if (tid < nb) {
                const size_t th = (size_t)(t0 + tid) * HV + h;
                if constexpr (DEC && !VD) a = expf(log_decay(p, th, h));
                if constexpr (BETA) bb = update_rate(p, th);
            }
            s_sc[tid][0] = a;
            s_sc[tid][1] = bb;
        }

        // ---- C: value channels of this tile
        for (int task = tid; task < NB * ROWS; task += NT) {
            const int tau = task / ROWS, rr = task % ROWS, row = row0 + rr;
            float val = 0.f;
            if (tau < nb && row < dv) val = to_f32(v[((size_t)(t0 + tau) * HV + h) * dv + row]);
            s_v[tau][rr] = val;
        }
        __syncthreads();

        // ---- serial token loop on the register-resident rows
        for (int tau = 0; tau < nb; ++tau) {
            float kv[C], qv[C], kb[C], av[C];
#pragma unroll
            for (int m = 0; m < NCH; ++m)
#pragma unroll
                for (int x = 0; x < VEC; ++x) {
                    const int col = m * 16 * VEC + l16 * VEC + x;
                    kv[m * VEC + x] = s_k[tau][col];
                    qv[m * VEC + x] = s_q[tau][col];
                    if constexpr (VD) {
                        kb[m * VEC + x] = s_kb[tau][col];
                        av[m * VEC + x] = s_a[tau][col];
                    }
                }
            const float a = s_sc[tau][0], bb = s_sc[tau][1], qk = s_sc[tau][2];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int rl = wave * RW + g * 4 + r4;
                const float vi = s_v[tau][rl];
                float r = 0.f, u = 0.f;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    if constexpr (RET) r = fmaf(S[g][c], VD ? kb[c] : kv[c], r);
                    u = fmaf(S[g][c], qv[c], u);
                }
                if constexpr (RET) r = sum16(r);
                u = sum16(u);
                if constexpr (DEC && !VD) {
                    r *= a;
                    u *= a;
                }
                float cc;
                if constexpr (RULE == GATED_DELTA_V2) cc = vi - r;
                else if constexpr (BETA) cc = bb * (vi - r);
                else cc = vi;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    if constexpr (VD) S[g][c] = fmaf(av[c], S[g][c], cc * kv[c]);
                    else if constexpr (DEC) S[g][c] = fmaf(a, S[g][c], cc * kv[c]);
                    else S[g][c] = fmaf(cc, kv[c], S[g][c]);
                }
                if (l16 == 0) s_o[tau][rl] = p.scale * (u + qk * cc);
            }
        }
        __syncthreads();

        // ---- o tile of the block -> global (act dtype, round to nearest even)
        for (int task = tid; task < NB * ROWS; task += NT) {
            const int tau = task / ROWS, rr = task % ROWS, row = row0 + rr;
            if (tau < nb && row < dv) o[((size_t)(t0 + tau) * HV + h) * dv + row] = from_f32<TA>(s_o[tau][rr]);
        }
    }

    // ---- registers -> outgoing state
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int row = row0 + wave * RW + g * 4 + r4;
        if (row >= dv) continue;
#pragma unroll
        for (int m = 0; m < NCH; ++m)
#pragma unroll
            for (int x = 0; x < VEC; ++x) {
                const int col = m * 16 * VEC + l16 * VEC + x;
                if (col < dk) dst[(size_t)row * dk + col] = S[g][m * VEC + x];
            }
    }
}

template <typename TA, int RULE, bool PK, int DKT, int G>
static hipError_t launch_one(const Params &p, hipStream_t stream)
{
    constexpr int ROWS = 16 * G;
    const int64_t ntile = (p.dv + ROWS - 1) / ROWS;
    const int64_t blocks = (int64_t)p.B * p.HV * ntile;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_recurrent<TA, RULE, PK, DKT, G>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename TA, int RULE, bool PK, int DKT>
static hipError_t by_rows(const Params &p, int g, hipStream_t s)
{
    switch (g) {
    case 1: return launch_one<TA, RULE, PK, DKT, 1>(p, s);
    case 2: return launch_one<TA, RULE, PK, DKT, 2>(p, s);
    default: return launch_one<TA, RULE, PK, DKT, 4>(p, s);
    }
}

template <typename TA, int RULE, bool PK>
static hipError_t by_dk(const Params &p, int dkt, int g, hipStream_t s)
{
    switch (dkt) {
    case 32: return by_rows<TA, RULE, PK, 32>(p, g, s);
    case 64: return by_rows<TA, RULE, PK, 64>(p, g, s);
    case 128: return by_rows<TA, RULE, PK, 128>(p, g, s);
    default: return by_rows<TA, RULE, PK, 256>(p, g, s);
    }
}

template <typename TA>
static hipError_t by_rule(const Params &p, int rule, bool pk, int dkt, int g, hipStream_t s)
{
    switch (rule) {
    case LINEAR: return by_dk<TA, LINEAR, false>(p, dkt, g, s);
    case DELTA: return by_dk<TA, DELTA, false>(p, dkt, g, s);
    case GATED: return pk ? by_dk<TA, GATED, true>(p, dkt, g, s) : by_dk<TA, GATED, false>(p, dkt, g, s);
    case GATED_DELTA:
        return pk ? by_dk<TA, GATED_DELTA, true>(p, dkt, g, s) : by_dk<TA, GATED_DELTA, false>(p, dkt, g, s);
    default:
        return pk ? by_dk<TA, GATED_DELTA_V2, true>(p, dkt, g, s) : by_dk<TA, GATED_DELTA_V2, false>(p, dkt, g, s);
    }
}

hipError_t launch_recurrent(const Params &p, int rule, bool per_key, bool f16, int dkt, int g, hipStream_t s)
{
    return f16 ? by_rule<half_t>(p, rule, per_key, dkt, g, s) : by_rule<float>(p, rule, per_key, dkt, g, s);
}

}  // namespace gdr
