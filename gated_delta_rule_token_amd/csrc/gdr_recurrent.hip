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
//   stored coalesced at the start of the next block.  A block's raw inputs
//   are loaded into registers while the previous block runs its loop.
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
    __shared__ float s_sc[NB][4];                  // alpha (scalar), beta, q.k, raw gate
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

    if (p.run_only && !p.run_only[(size_t)b * HV + h]) return;
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

    // The inputs of a token block are loaded into registers one block ahead
    // (while the previous block runs its token loop) and turned into the LDS
    // operands afterwards, so global-memory latency overlaps the serial loop.
    // Every load is unconditional: token and column indices are clamped into
    // the request / row, and the staging step zeroes what lies outside.
    constexpr int NTA = NB * 16 / NT;                 // (token, 16-lane column chunk) tasks per thread
    constexpr int NTC = (NB * ROWS + NT - 1) / NT;    // value-channel tasks per thread
    // raw chunks as vector types, so each is one (or two) 16-byte loads into
    // consecutive registers
    typedef TA AV __attribute__((ext_vector_type(C), aligned(sizeof(TA) * C < 16 ? sizeof(TA) * C : 16)));
    typedef float FV __attribute__((ext_vector_type(C), aligned(4 * C < 16 ? 4 * C : 16)));
    struct Raw {
        AV q[NTA], k[NTA];
        FV dec[VD && PK ? NTA : 1];            // per-key log decay
        FV er[RULE == GATED_DELTA_V2 ? NTA : 1];  // erase gate
        TA v[NTC];
        float g, bt;  // raw per-token gate and update rate (tid < NB)
    };
    const int64_t tlast = e - 1;
    auto tok = [&](int64_t t) { return t < tlast ? t : tlast; };
    auto load_raw = [&](int64_t tb0, Raw &r) {
#pragma unroll
        for (int i = 0; i < NTA; ++i) {
            const int task = tid + NT * i, tau = task >> 4, col0 = (task & 15) * C;
            const int64_t t = tok(tb0 + tau);
            const TA *qp = q + ((size_t)t * H + qh) * dk;
            const TA *kp = k + ((size_t)t * H + qh) * dk;
            const size_t th = (size_t)t * HV + h;
            if (fullk) {
                // whole chunks: vector loads (rows and chunks are 16-byte aligned)
                r.q[i] = *reinterpret_cast<const AV *>(qp + col0);
                r.k[i] = *reinterpret_cast<const AV *>(kp + col0);
                if constexpr (VD && PK) {
                    // a per-key raw gate comes in fp32 or the activations' dtype
                    bool act_gate = false;
                    if constexpr (sizeof(TA) == 2) act_gate = p.gate_dt != 0;
                    if (act_gate) {
                        const AV gh = *reinterpret_cast<const AV *>(static_cast<const TA *>(p.gate) + th * dk + col0);
#pragma unroll
                        for (int c = 0; c < C; ++c) r.dec[i][c] = to_f32((TA)gh[c]);
                    } else {
                        r.dec[i] = *reinterpret_cast<const FV *>(static_cast<const float *>(p.gate) + th * dk + col0);
                    }
                }
                if constexpr (RULE == GATED_DELTA_V2) r.er[i] = *reinterpret_cast<const FV *>(p.erase + th * dk + col0);
            } else {
                // partial key rows: element loads with the column clamped into the row
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int col = col0 + c < dk ? col0 + c : dk - 1;
                    r.q[i][c] = qp[col];
                    r.k[i][c] = kp[col];
                    if constexpr (VD && PK)
                        r.dec[i][c] = load_gate(p, th * dk + col);
                    if constexpr (RULE == GATED_DELTA_V2) r.er[i][c] = p.erase[th * dk + col];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NTC; ++i) {
            const int task = tid + NT * i, tau = task / ROWS, rr = task % ROWS;
            const int row = row0 + rr < dv ? row0 + rr : dv - 1;
            r.v[i] = v[((size_t)tok(tb0 + (tau < NB ? tau : NB - 1)) * HV + h) * dv + row];
        }
        // every thread reads a token's scalars (threads past NB re-read the
        // block's last one), so no load sits behind a divergent branch
        r.g = 0.f;
        r.bt = 1.f;
        {
            const size_t th = (size_t)tok(tb0 + (tid < NB ? tid : NB - 1)) * HV + h;
            if constexpr (DEC && (!VD || !PK)) r.g = load_gate(p, th);
            if constexpr (BETA) r.bt = p.beta[beta_index(p, th)];
        }
    };
    // LDS operands of the block starting at tb0 (nb valid tokens) from its raw inputs
    auto stage = [&](int nb, const Raw &r) {
#pragma unroll
        for (int i = 0; i < NTA; ++i) {
            const int task = tid + NT * i, tau = task >> 4, col0 = (task & 15) * C;
            const bool live = tau < nb;
            float qv[C], kv[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const bool in = live && col0 + c < dk;
                qv[c] = in ? to_f32((TA)r.q[i][c]) : 0.f;
                kv[c] = in ? to_f32((TA)r.k[i][c]) : 0.f;
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
                // per-key decay: the per-key log decay, or the token's scalar one
                // broadcast over the keys
                float gs = 0.f;
                if constexpr (!PK) gs = p.gate_qwen ? gate_scale(p, h) * softplus_f32(s_sc[tau][3] + p.dt_bias[h])
                                                    : s_sc[tau][3];
                float av[C], kb[C];
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const bool in = live && col0 + c < dk;
                    float a = 1.f, er = 1.f;
                    if (in) {
                        float g = gs;
                        if constexpr (PK) g = p.gate_qwen ? key_decay_from_raw(p, r.dec[i][c], h, col0 + c) : r.dec[i][c];
                        a = expf(g);
                        if constexpr (RULE == GATED_DELTA_V2) er = r.er[i][c];
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
            if ((task & 15) == 0) s_sc[tau][2] = qk * inq * ink;
        }
#pragma unroll
        for (int i = 0; i < NTC; ++i) {
            const int task = tid + NT * i, tau = task / ROWS, rr = task % ROWS;
            if (task < NB * ROWS) s_v[tau][rr] = (tau < nb && row0 + rr < dv) ? to_f32(r.v[i]) : 0.f;
        }
    };

    const int nblk = (int)((e - s + NB - 1) / NB);
    Raw ra, rb;
    if (nblk > 0) load_raw(s, ra);
    // one block: its scalars and operands, then the token loop; the o tile of
    // the previous block is stored at the start (after the barrier that
    // follows its loop)
    auto block = [&](int n, const Raw &cur, Raw &nxt) {
        const int64_t t0 = s + (int64_t)n * NB;
        const int nb = (int)((e - t0) < NB ? (e - t0) : NB);
        __syncthreads();  // the previous block's loop is done with LDS
        if (n > 0) {
            const int64_t tp = t0 - NB;
            for (int task = tid; task < NB * ROWS; task += NT) {
                const int tau = task / ROWS, rr = task % ROWS, row = row0 + rr;
                if (row < dv) o[((size_t)(tp + tau) * HV + h) * dv + row] = from_f32<TA>(s_o[tau][rr]);
            }
        }
        // per-token scalar gate (the raw value parked in column 3 for the
        // per-key staging of a scalar decay) and update rate
        if (tid < NB) {
            float a = 1.f, bb = 1.f, graw = cur.g;
            if (tid < nb) {
                if constexpr (DEC && !VD) a = expf(p.gate_qwen ? gate_scale(p, h) * softplus_f32(graw + p.dt_bias[h]) : graw);
                if constexpr (BETA) bb = p.beta_sigmoid ? sigmoid_f32(cur.bt) : cur.bt;
            }
            s_sc[tid][0] = a;
            s_sc[tid][1] = bb;
            s_sc[tid][3] = graw;
        }
        if constexpr (VD && !PK) __syncthreads();  // the raw scalar gate feeds the staging below
        stage(nb, cur);
        if (n + 1 < nblk) load_raw(t0 + NB, nxt);
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
    };
    for (int n = 0; n < nblk; n += 2) {
        block(n, ra, rb);
        if (n + 1 < nblk) block(n + 1, rb, ra);
    }
    // ---- o tile of the last block
    if (nblk > 0) {
        __syncthreads();
        const int64_t tp = s + (int64_t)(nblk - 1) * NB;
        const int nb = (int)(e - tp);
        for (int task = tid; task < NB * ROWS; task += NT) {
            const int tau = task / ROWS, rr = task % ROWS, row = row0 + rr;
            if (tau < nb && row < dv) o[((size_t)(tp + tau) * HV + h) * dv + row] = from_f32<TA>(s_o[tau][rr]);
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

hipError_t launch_recurrent(const Params &p, int rule, bool per_key, int act, int dkt, int g, hipStream_t s)
{
    if (act == 1) return by_rule<half_t>(p, rule, per_key, dkt, g, s);
    if (act == 2) return by_rule<bf16_t>(p, rule, per_key, dkt, g, s);
    return by_rule<float>(p, rule, per_key, dkt, g, s);
}

}  // namespace gdr
