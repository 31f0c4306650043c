// gdr_decode.hip -- decode kernel for dk = dv = 128: one workgroup streams the
// whole 64 KiB state of one (request, value head) through registers.
//
// Decode is HBM-bound: each addressed state byte is read once and written
// once per call (in place for a slot slab, CLIKA "gatedDeltaUpdate"), and all
// other traffic is a few hundred bytes per (request, head).  So the kernel
// is built around the state stream:
//   * 16 lanes hold a row (key columns l16*4 .. +3 and 64 + l16*4 .. +3),
//     4 rows per wave-instruction, G row groups per wave, WAVES waves per
//     workgroup (the library build: G = 8, 4 waves, the whole head).
//     Every state access is a 16-byte vector; one wave-instruction covers
//     4 rows x 256 contiguous bytes.
//   * All 16 row-group loads of a lane (64 fp32 values, 16 KiB per wave) are
//     issued before the first one is used, so each wave keeps 16 KiB of reads
//     in flight; state loads and stores carry the non-temporal hint, since
//     no state byte is touched twice in a call.
//   * The per-token prologue (q/k L2 norms, q.k, raw-gate decay, sigmoid
//     update rate, per-key decay vectors) is computed in fp32 registers by
//     every wave for its own use; nothing goes through memory.
// Tokens of the request (normally one) are applied in order with the state
// resident in registers; the recurrence and rule terms are those of the
// "com.microsoft.GatedDeltaNet" README (Description, Attributes).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

typedef float f4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ f4 ld4(const f4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void st4(f4 *p, f4 x)
{
    if constexpr (NT) __builtin_nontemporal_store(x, p);
    else *p = x;
}

// G row groups (4 rows each) per wave, WAVES waves per workgroup; a head's
// 128 rows are split over 128 / (4 * G * WAVES) workgroups.  NT marks the
// state stream non-temporal (read once, written once).  STG stages the token
// inputs of up to 8 tokens at a time through LDS: the workgroup loads them
// together (alongside the state, for the first block) instead of one global
// round trip per token inside the loop; used when requests carry several
// tokens (speculative / multi-token verify).
template <typename TA, int RULE, bool PK, int G, int WAVES, bool NT, bool STG>
__global__ __launch_bounds__(64 * WAVES) void k_decode128(const Params p)
{
    constexpr int DK = 128, C = 8;
    constexpr int RW = 4 * G, PARTS = DK / (RW * WAVES);
    static_assert(PARTS * RW * WAVES == DK, "row split must cover the head");
    constexpr bool VD = PK || RULE == GATED_DELTA_V2;
    constexpr bool DEC = rule_decays(RULE);
    constexpr bool RET = rule_retrieves(RULE);
    constexpr bool BETA = rule_has_beta(RULE);

    const int HV = p.HV, H = p.H;
    const int part = blockIdx.x % PARTS;
    const int h = (blockIdx.x / PARTS) % HV, b = blockIdx.x / (PARTS * HV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, r4 = lane >> 4;
    const int qh = (int)(((int64_t)h * H) / HV);
    const int wrow0 = (part * WAVES + wave) * RW;  // first row of this wave

    const float *src;
    float *dst;
    if (!state_ptrs(p, b, h, src, dst)) return;
    int64_t s, e;
    request_range(p, b, s, e);

    const TA *__restrict__ q = static_cast<const TA *>(p.q);
    const TA *__restrict__ k = static_cast<const TA *>(p.k);
    const TA *__restrict__ v = static_cast<const TA *>(p.v);
    TA *__restrict__ o = static_cast<TA *>(p.o);

    // Staged token inputs (STG): the raw inputs of up to TB tokens, NI
    // elements per thread, loaded into registers and parked in LDS.  The first
    // block is requested before the state stream, so waiting for it never
    // waits for the state.
    constexpr int TB = 8, NTH = 64 * WAVES, NI = TB * DK / NTH;
    constexpr bool ER = RULE == GATED_DELTA_V2;
    struct Raw {
        float q[NI], k[NI], v[NI], g[VD ? NI : 1], e[ER ? NI : 1];
        float ga, bt;  // scalar log decay and update rate (thread tid < nt: token tid)
    };
    auto load_block = [&](int64_t t0, int nt, Raw &r) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int i = tid + NTH * j, tt = i / DK, c = i % DK;
            const int ts = tt < nt ? tt : nt - 1;  // rows past the block repeat its last token
            const size_t t = (size_t)(t0 + ts), th = t * HV + h;
            r.q[j] = to_f32(q[(t * H + qh) * DK + c]);
            r.k[j] = to_f32(k[(t * H + qh) * DK + c]);
            r.v[j] = to_f32(v[th * DK + c]);
            if constexpr (VD) r.g[j] = PK ? log_decay_key(p, th, h, c) : log_decay(p, th, h);
            if constexpr (ER) r.e[j] = p.erase[th * DK + c];
        }
        r.ga = 0.f;
        r.bt = 1.f;
        if (tid < nt) {
            const size_t th = (size_t)(t0 + tid) * HV + h;
            if constexpr (DEC && !VD) r.ga = log_decay(p, th, h);
            if constexpr (BETA) r.bt = update_rate(p, th);
        }
    };
    Raw raw;
    if constexpr (STG) {
        if (e > s) load_block(s, (int)((e - s) < TB ? (e - s) : TB), raw);
    }

    // lane's first element within row group g: row (wrow0 + 4*g + r4), column l16*4
    const size_t lane_off = (size_t)(wrow0 + r4) * DK + l16 * 4;
    f4 S[G][2];
    if (src) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const f4 *rp = reinterpret_cast<const f4 *>(src + lane_off + (size_t)g * 4 * DK);
            S[g][0] = ld4<NT>(rp);
            S[g][1] = ld4<NT>(rp + 16);
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) S[g][0] = S[g][1] = f4{0.f, 0.f, 0.f, 0.f};
    }

    // One token: q and k columns (l16*4 .. +3, 64 + l16*4 .. +3) of this lane,
    // v of its rows, and for a per-key decay / the erase gate their values at
    // the lane's columns (gk: log decay, er: erase).  ga, bt: scalar log decay
    // and update rate.
    auto token = [&](int64_t t, float (&qv)[C], float (&kv)[C], const float (&vi)[G], float ga, float bt,
                     const float (&gk)[C], const float (&er)[C]) {
        const size_t th = (size_t)t * HV + h;
        float qss = 0.f, kss = 0.f, qk = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            qss = fmaf(qv[c], qv[c], qss);
            kss = fmaf(kv[c], kv[c], kss);
            qk = fmaf(qv[c], kv[c], qk);
        }
        qk = sum16(qk);
        float inq = 1.f, ink = 1.f;
        if (p.qk_l2_norm) {
            inq = 1.f / sqrtf(sum16(qss) + 1e-12f);
            ink = 1.f / sqrtf(sum16(kss) + 1e-12f);
        }
        qk *= inq * ink;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            qv[c] *= inq;
            kv[c] *= ink;
        }

        float a = 1.f, bb = 1.f;
        if constexpr (DEC && !VD) a = expf(ga);
        if constexpr (BETA) bb = bt;
        float av[C], kb[C];
        if constexpr (VD) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                av[c] = expf(gk[c]);
                kb[c] = (RULE == GATED_DELTA_V2 ? er[c] : 1.f) * av[c] * kv[c];
                qv[c] *= av[c];
            }
        }

#pragma unroll
        for (int g = 0; g < G; ++g) {
            float sv[C];
#pragma unroll
            for (int x = 0; x < 4; ++x) { sv[x] = S[g][0][x]; sv[4 + x] = S[g][1][x]; }
            float r = 0.f, u = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if constexpr (RET) r = fmaf(sv[c], VD ? kb[c] : kv[c], r);
                u = fmaf(sv[c], qv[c], u);
            }
            if constexpr (RET) r = sum16(r);
            u = sum16(u);
            if constexpr (DEC && !VD) {
                r *= a;
                u *= a;
            }
            float cc;
            if constexpr (RULE == GATED_DELTA_V2) cc = vi[g] - r;
            else if constexpr (BETA) cc = bb * (vi[g] - r);
            else cc = vi[g];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if constexpr (VD) sv[c] = fmaf(av[c], sv[c], cc * kv[c]);
                else if constexpr (DEC) sv[c] = fmaf(a, sv[c], cc * kv[c]);
                else sv[c] = fmaf(cc, kv[c], sv[c]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) { S[g][0][x] = sv[x]; S[g][1][x] = sv[4 + x]; }
            if (l16 == 0) o[th * DK + wrow0 + g * 4 + r4] = from_f32<TA>(p.scale * (u + qk * cc));
        }
    };
    auto col_of = [&](int c) { return (c < 4 ? 0 : 64) + l16 * 4 + (c & 3); };

    if constexpr (!STG) {
        for (int64_t t = s; t < e; ++t) {
            const size_t th = (size_t)t * HV + h;
            float qv[C], kv[C];
            {
                const TA *qp = q + ((size_t)t * H + qh) * DK + l16 * 4;
                const TA *kp = k + ((size_t)t * H + qh) * DK + l16 * 4;
                float lo[4], hi[4];
                load_act<TA, 4>(qp, lo);
                load_act<TA, 4>(qp + 64, hi);
#pragma unroll
                for (int x = 0; x < 4; ++x) { qv[x] = lo[x]; qv[4 + x] = hi[x]; }
                load_act<TA, 4>(kp, lo);
                load_act<TA, 4>(kp + 64, hi);
#pragma unroll
                for (int x = 0; x < 4; ++x) { kv[x] = lo[x]; kv[4 + x] = hi[x]; }
            }
            float vi[G];
#pragma unroll
            for (int g = 0; g < G; ++g) vi[g] = to_f32(v[th * DK + wrow0 + g * 4 + r4]);
            float ga = 0.f, bt = 1.f, gk[C] = {}, er[C] = {};
            if constexpr (DEC && !VD) ga = log_decay(p, th, h);
            if constexpr (BETA) bt = update_rate(p, th);
            if constexpr (VD) {
                float sa = 0.f;
                if constexpr (!PK) sa = log_decay(p, th, h);
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    gk[c] = PK ? log_decay_key(p, th, h, col_of(c)) : sa;
                    if constexpr (RULE == GATED_DELTA_V2) er[c] = p.erase[th * DK + col_of(c)];
                }
            }
            token(t, qv, kv, vi, ga, bt, gk, er);
        }
    } else {
        // Staged tokens.  Per block: park the raw inputs in LDS, normalise
        // each token once for the workgroup (q and k by their L2 norms, q.k,
        // the decay factor, and on the per-key path q o alpha and
        // erase o alpha o k), then apply the block's tokens to the row groups
        // in two halves.
        __shared__ float stq[TB][DK], stk[TB][DK], stv[TB][DK];
        __shared__ float sta[VD ? TB : 1][DK], stb[VD ? TB : 1][DK];
        __shared__ float sts[TB][4];  // q.k (normalised), decay factor, update rate
        auto park = [&](const Raw &r, int nt) {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int i = tid + NTH * j, tt = i / DK, c = i % DK;
                stq[tt][c] = r.q[j];
                stk[tt][c] = r.k[j];
                stv[tt][c] = r.v[j];
                if constexpr (VD) sta[tt][c] = r.g[j];
                if constexpr (ER) stb[tt][c] = r.e[j];
            }
            if (tid < TB) {
                sts[tid][1] = r.ga;
                sts[tid][2] = r.bt;
            }
        };
        // one wave per token, two columns per lane (c = lane, lane + 64)
        auto prep = [&](int nt) {
            for (int tt = wave; tt < nt; tt += WAVES) {
                float qx[2], kx[2], qss = 0.f, kss = 0.f, qk = 0.f;
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    qx[x] = stq[tt][lane + 64 * x];
                    kx[x] = stk[tt][lane + 64 * x];
                    qss = fmaf(qx[x], qx[x], qss);
                    kss = fmaf(kx[x], kx[x], kss);
                    qk = fmaf(qx[x], kx[x], qk);
                }
#pragma unroll
                for (int o2 = 32; o2 > 0; o2 >>= 1) {
                    qss += __shfl_xor(qss, o2);
                    kss += __shfl_xor(kss, o2);
                    qk += __shfl_xor(qk, o2);
                }
                float inq = 1.f, ink = 1.f;
                if (p.qk_l2_norm) {
                    inq = 1.f / sqrtf(qss + 1e-12f);
                    ink = 1.f / sqrtf(kss + 1e-12f);
                }
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int c = lane + 64 * x;
                    const float kn = kx[x] * ink;
                    float qn = qx[x] * inq;
                    if constexpr (VD) {
                        const float av = expf(sta[tt][c]);
                        qn *= av;
                        stb[tt][c] = (ER ? stb[tt][c] : 1.f) * av * kn;
                        sta[tt][c] = av;
                    }
                    stq[tt][c] = qn;
                    stk[tt][c] = kn;
                }
                if (lane == 0) {
                    sts[tt][0] = qk * inq * ink;
                    if constexpr (DEC && !VD) sts[tt][1] = expf(sts[tt][1]);
                }
            }
        };
        for (int64_t t0 = s; t0 < e; t0 += TB) {
            const int nt = (int)((e - t0) < TB ? (e - t0) : TB);
            if (t0 != s) load_block(t0, nt, raw);
            park(raw, nt);
            lds_barrier();
            prep(nt);
            lds_barrier();
            // two halves of the row groups: every token goes to the first half
            // while the second half of the state is still arriving; inside a
            // half, the row groups are independent chains
            constexpr int GH = G / 2;
#pragma unroll
            for (int gh = 0; gh < 2; ++gh) {
                for (int tt = 0; tt < nt; ++tt) {
                    const size_t th = (size_t)(t0 + tt) * HV + h;
                    float qv[C], kv[C], av[C], kb[C];
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        qv[c] = stq[tt][col_of(c)];
                        kv[c] = stk[tt][col_of(c)];
                        if constexpr (VD) {
                            av[c] = sta[tt][col_of(c)];
                            kb[c] = stb[tt][col_of(c)];
                        }
                    }
                    const float qk = sts[tt][0], a = sts[tt][1], bb = sts[tt][2];
#pragma unroll
                    for (int gi = 0; gi < GH; ++gi) {
                        const int g = gh * GH + gi;
                        const float vi = stv[tt][wrow0 + g * 4 + r4];
                        float sv[C];
#pragma unroll
                        for (int x = 0; x < 4; ++x) { sv[x] = S[g][0][x]; sv[4 + x] = S[g][1][x]; }
                        float r = 0.f, u = 0.f;
#pragma unroll
                        for (int c = 0; c < C; ++c) {
                            if constexpr (RET) r = fmaf(sv[c], VD ? kb[c] : kv[c], r);
                            u = fmaf(sv[c], qv[c], u);
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
                            if constexpr (VD) sv[c] = fmaf(av[c], sv[c], cc * kv[c]);
                            else if constexpr (DEC) sv[c] = fmaf(a, sv[c], cc * kv[c]);
                            else sv[c] = fmaf(cc, kv[c], sv[c]);
                        }
#pragma unroll
                        for (int x = 0; x < 4; ++x) { S[g][0][x] = sv[x]; S[g][1][x] = sv[4 + x]; }
                        if (l16 == 0) o[th * DK + wrow0 + g * 4 + r4] = from_f32<TA>(p.scale * (u + qk * cc));
                    }
                }
            }
            lds_barrier();  // every wave is done with this block before the next one lands
        }
    }

#pragma unroll
    for (int g = 0; g < G; ++g) {
        f4 *rp = reinterpret_cast<f4 *>(dst + lane_off + (size_t)g * 4 * DK);
        st4<NT>(rp, S[g][0]);
        st4<NT>(rp + 16, S[g][1]);
    }
}

// Tiling of the library build: 8 row groups per wave, 4 waves, one
// workgroup per (request, head), state stream marked non-temporal.  Measured
// on MI355X at B=256, HV=32 (1.08 GB per step): 189.8 us with non-temporal
// loads and stores against 213 us without; splitting a head over 2-4
// workgroups, 128- or 512-thread workgroups, and a persistent grid that
// prefetches the next head while updating the current one were all slower.
constexpr int DEC_G = 8, DEC_WAVES = 4;
constexpr bool DEC_NT = true;

// Requests of several tokens (more tokens than requests) take the staged
// variant; one token per request keeps the direct loads.
template <typename TA, int RULE, bool PK>
static hipError_t launch_one(const Params &p, hipStream_t stream)
{
    constexpr int PARTS = 128 / (4 * DEC_G * DEC_WAVES);
    const int64_t blocks = (int64_t)p.B * p.HV * PARTS;
    if (blocks == 0) return hipSuccess;
    if (p.T > p.B)
        hipLaunchKernelGGL((k_decode128<TA, RULE, PK, DEC_G, DEC_WAVES, DEC_NT, true>), dim3((unsigned)blocks),
                           dim3(64 * DEC_WAVES), 0, stream, p);
    else
        hipLaunchKernelGGL((k_decode128<TA, RULE, PK, DEC_G, DEC_WAVES, DEC_NT, false>), dim3((unsigned)blocks),
                           dim3(64 * DEC_WAVES), 0, stream, p);
    return hipGetLastError();
}

template <typename TA>
static hipError_t by_rule(const Params &p, int rule, bool pk, hipStream_t s)
{
    switch (rule) {
    case LINEAR: return launch_one<TA, LINEAR, false>(p, s);
    case DELTA: return launch_one<TA, DELTA, false>(p, s);
    case GATED: return pk ? launch_one<TA, GATED, true>(p, s) : launch_one<TA, GATED, false>(p, s);
    case GATED_DELTA: return pk ? launch_one<TA, GATED_DELTA, true>(p, s) : launch_one<TA, GATED_DELTA, false>(p, s);
    default: return pk ? launch_one<TA, GATED_DELTA_V2, true>(p, s) : launch_one<TA, GATED_DELTA_V2, false>(p, s);
    }
}

hipError_t launch_decode128(const Params &p, int rule, bool per_key, int act, hipStream_t s)
{
    if (act == 1) return by_rule<half_t>(p, rule, per_key, s);
    if (act == 2) return by_rule<bf16_t>(p, rule, per_key, s);
    return by_rule<float>(p, rule, per_key, s);
}

}  // namespace gdr
