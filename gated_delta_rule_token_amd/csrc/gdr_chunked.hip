// gdr_chunked.hip -- chunk-parallel prefill (chunk = 64 tokens) on MFMA.
//
// The "com.microsoft.GatedDeltaNet" README (Attributes, chunk_size) names a
// chunk-parallel prefill whose chunk size does not change the result.  The
// form used here is the recurrence of the README's Description unrolled over
// one chunk (scalar per-head decay; V-major state S, rows = value index):
//   gamma_t = exp(G_t), G_t = sum of the log decays up to t inside the chunk,
//   A_ts = beta_t (gamma_t / gamma_s) kn_t.kn_s (s < t),  kn = k / |k|,
//   W = (I+A)^-1 diag(beta gamma |k|^-1) K,   U = (I+A)^-1 diag(beta) V,
//   D = U - W S0^T                     (the chunk's effective value updates)
//   S_C = gamma_C S0 + D^T diag(kd) K,  kd_t = (gamma_C / gamma_t) / |k_t|,
//   O = gq (Q S0^T) + P D,  P_ts = scale (gamma_t/gamma_s) q_t.k_s/(|q_t||k_s|) (s <= t),
//   gq_t = scale gamma_t / |q_t|.
// Rules without retrieval (linear, gated) have D = V.
//
// Three launches:
//   k_chunk_table  one workgroup: per-request chunk offsets (exclusive scan of
//                  ceil(len/64)); the host never reads cu_seqlens.
//   k_chunk_prep   one workgroup per (chunk, head), all chunks in parallel:
//                  K Q^T and K K^T on 16x16x32 f16 MFMA (q/k are fp16, so the
//                  products are exact up to fp32 accumulation), the unit
//                  lower-triangular solve for [W | U] by fp32 forward
//                  substitution (one column per thread), the per-token
//                  scalars, and every operand of the scan written in the
//                  order the scan's lanes load it.
//   k_chunk_scan   one workgroup per (request, head, 32 state rows), chunks
//                  in order; the transposed state tile lives in MFMA
//                  accumulators.  Each chunk: D = U - W S^T, then
//                  S^T <- gamma_C S^T + K^T (kd D) on four "chain" waves, and
//                  O^T = gq S Q^T + D^T P^T on four "output" waves.
// Every fp32 operand is split into fp16 hi + lo and multiplied as
// hi*hi + hi*lo + lo*hi (fp16 operands need no split), which keeps the
// products at about fp32 accuracy on the f16 matrix cores.  The four row
// tiles of a head are dispatched to the same XCD so their identical
// per-chunk reads are shared through its L2.

#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u4v ld_b128_lds(const void *p) { return *reinterpret_cast<const u4v *>(p); }

constexpr int CH = 64;          // chunk length
constexpr int D128 = 128;       // dk = dv

// Workspace record of one (chunk, head).  Every operand of the scan is stored
// in MFMA fragment order: 1 KB blocks holding the 16 bytes lane l (= 16 lq + lr)
// of a wave loads at l * 16, so each wave-wide load reads 1 KB of consecutive
// bytes (eight whole cache lines).
//   R_W   W (hi, lo) fp16, block (tb * 4 + kk) * 2 + plane: token 16 tb + lr, keys 32 kk + 8 lq .. +7
//   R_KT  K^T fp16,        block mt * 2 + ks:              key 16 mt + lr, tokens 32 ks + 8 lq .. +7
//   R_U   U fp32,          block tb * 8 + rt:              tokens 16 tb + 4 lq .. +3, row 16 rt + lr
//   R_Q   q fp16,          block tb * 4 + kk:              token 16 tb + lr, keys 32 kk + 8 lq .. +7
//   R_P   P (hi, lo) fp16, block (tb * 2 + ks) * 2 + plane: token 16 tb + lr, tokens 32 ks + 8 lq .. +7
//   R_SC  fp32 scalars: kd[64], gq[64], gamma_C
constexpr uint32_t R_W = 0;
constexpr uint32_t R_KT = R_W + 32 * 1024;
constexpr uint32_t R_U = R_KT + 16 * 1024;
constexpr uint32_t R_Q = R_U + 32 * 1024;
constexpr uint32_t R_P = R_Q + 16 * 1024;
constexpr uint32_t R_SC = R_P + 16 * 1024;
constexpr uint32_t WS_REC = R_SC + 1024;

__device__ __forceinline__ f4v mfma16(h8 a, h8 b, f4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp32 -> (hi, lo) fp16 pair with hi + lo ~ x to about 22 bits
__device__ __forceinline__ void split8(const float (&x)[8], h8 &hi, h8 &lo)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const half_t h = (half_t)x[i];
        hi[i] = h;
        lo[i] = (half_t)(x[i] - (float)h);
    }
}

__device__ __forceinline__ h8 ld_h8(const half_t *p) { return *reinterpret_cast<const h8 *>(p); }

// Raw buffer resource over one workspace record (the record's bytes only:
// an offset past it reads zero instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *rec)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(rec), 0, (int)WS_REC, 0x00020000);
}

template <typename T>
__device__ __forceinline__ T ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// four fp32 -> (hi, lo) fp16 quads
__device__ __forceinline__ void split4(f4v x, h4 &hi, h4 &lo)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = (half_t)x[i];
        lo[i] = (half_t)(x[i] - (float)hi[i]);
    }
}

// Locate request b and the chunk's first token for global chunk index ci.
__device__ __forceinline__ int chunk_request(const int32_t *off, int B, int64_t ci)
{
    int lo = 0, hi = B;  // largest b in [0, B) with off[b] <= ci
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= ci) lo = mid;
        else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------------------ table
__global__ __launch_bounds__(256) void k_chunk_table(const Params p, int32_t *off)
{
    __shared__ int32_t s[256];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < p.B; base += 256) {
        const int b = base + tid;
        int n = 0;
        if (b < p.B) {
            int64_t st, en;
            request_range(p, b, st, en);
            n = (int)((en - st + CH - 1) / CH);
        }
        s[tid] = n;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int v = tid >= o ? s[tid - o] : 0;
            __syncthreads();
            s[tid] += v;
            __syncthreads();
        }
        if (b < p.B) off[b] = carry + s[tid] - n;
        __syncthreads();
        if (tid == 255) carry += s[255];
        __syncthreads();
    }
    if (tid == 0) off[p.B] = carry;
}


// ------------------------------------------------------------------ phase 1
// 256 threads.  LDS: K, V and Q rows of the chunk; A (fp32) replaces Q once
// K Q^T and K K^T are formed; after the solve W (hi, lo) rows replace K and V.
template <int RULE>
__global__ __launch_bounds__(256, 3) void k_chunk_prep(const Params p, const int32_t *__restrict__ off,
                                                   char *__restrict__ ws)
{
    constexpr bool DEC = rule_decays(RULE);
    constexpr bool RET = rule_retrieves(RULE);
    constexpr bool BETA = rule_has_beta(RULE);
    constexpr int LD = D128 + 8;  // padded fp16 row (bank spread)
    constexpr int LA = CH + 4;    // 16-byte rows: the solve reads A rows as float4 broadcasts
    constexpr int SLOT = CH * LD * 2;
    static_assert(CH * LA * 4 == SLOT, "Q rows and A rows share one LDS footprint");

    __shared__ __align__(16) char sm[3 * SLOT];
    half_t(*sK)[LD] = reinterpret_cast<half_t(*)[LD]>(sm);
    half_t(*sV)[LD] = reinterpret_cast<half_t(*)[LD]>(sm + SLOT);
    half_t(*sQ)[LD] = reinterpret_cast<half_t(*)[LD]>(sm + 2 * SLOT);
    float(*sA)[LA] = reinterpret_cast<float(*)[LA]>(sm + 2 * SLOT);
    half_t(*sW)[CH][LD] = reinterpret_cast<half_t(*)[CH][LD]>(sm);  // [hi, lo][token][key], after the solve
    __shared__ float sG[CH], sBeta[CH], sIk[CH], sIq[CH], sRw[CH];

    const int HV = p.HV, H = p.H;
    const int64_t ci = blockIdx.x / HV;
    const int h = blockIdx.x % HV;
    if (ci >= off[p.B]) return;
    const int b = chunk_request(off, p.B, ci);
    int64_t rs, re;
    request_range(p, b, rs, re);
    const int64_t t0 = rs + (ci - off[b]) * CH;
    const int n = (int)((re - t0) < CH ? (re - t0) : CH);
    const int qh = (int)(((int64_t)h * H) / HV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4, lk = lq * 8;
    char *rec = ws + ((size_t)ci * HV + h) * WS_REC;

    const half_t *__restrict__ q = static_cast<const half_t *>(p.q);
    const half_t *__restrict__ k = static_cast<const half_t *>(p.k);
    const half_t *__restrict__ v = static_cast<const half_t *>(p.v);

    // ---- chunk rows of K, Q (head qh) and V (head h): issue the loads first,
    // compute the gates while they are in flight, then park them in LDS
    h8 ldk[4], ldq[4], ldv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
        ldk[i] = ldq[i] = ldv[i] = h8{};
        if (r < n) {
            const size_t tq = ((size_t)(t0 + r) * H + qh) * D128 + c8;
            ldk[i] = ld_h8(k + tq);
            ldq[i] = ld_h8(q + tq);
            ldv[i] = ld_h8(v + ((size_t)(t0 + r) * HV + h) * D128 + c8);
        }
    }
    // ---- per-token log decay (cumulated over the chunk by a 64-lane scan) and update rate
    if (tid < CH) {
        const int t = tid;
        float g = 0.f, bt = 0.f;
        if (t < n) {
            const size_t th = (size_t)(t0 + t) * HV + h;
            if constexpr (DEC) g = log_decay(p, th, h);
            bt = BETA ? update_rate(p, th) : 1.f;
        }
#pragma unroll
        for (int o = 1; o < CH; o <<= 1) {
            const float y = __shfl_up(g, o, CH);
            if (t >= o) g += y;
        }
        sG[t] = g;  // inclusive cumulative log decay inside the chunk
        sBeta[t] = bt;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
        *reinterpret_cast<h8 *>(&sK[r][c8]) = ldk[i];
        *reinterpret_cast<h8 *>(&sQ[r][c8]) = ldq[i];
        *reinterpret_cast<h8 *>(&sV[r][c8]) = ldv[i];
        // q in fragment order for the scan's output waves (rows past the end are zero)
        *reinterpret_cast<h8 *>(rec + R_Q + ((((r >> 4) * 4 + (c8 >> 5)) * 64) + ((c8 & 31) >> 3) * 16 + (r & 15)) * 16) = ldq[i];
    }
    lds_barrier();

    // ---- K^T fragments (key 16 mt + lr, tokens 32 ks + 8 lq .. +7); fragment f = block * 64 + lane
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int f = tid + 256 * g, blk = f >> 6, fl = f & 63;
        const int key = 16 * (blk >> 1) + (fl & 15), tk = 32 * (blk & 1) + 8 * (fl >> 4);
        h8 col;
#pragma unroll
        for (int x = 0; x < 8; ++x) col[x] = sK[tk + x][key];
        *reinterpret_cast<h8 *>(rec + R_KT + (size_t)f * 16) = col;
    }
    // ---- inverse L2 norms of the chunk's q and k rows: 4 threads per row
    {
        const int t = tid >> 2, part = tid & 3;
        float ss = 0.f, sq = 0.f;
        if (p.qk_l2_norm) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const h8 kk = ld_h8(&sK[t][32 * part + 8 * g]);
                const h8 qq = ld_h8(&sQ[t][32 * part + 8 * g]);
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    ss = fmaf((float)kk[x], (float)kk[x], ss);
                    sq = fmaf((float)qq[x], (float)qq[x], sq);
                }
            }
            ss += dpp_mov<0xB1>(ss);  // sum over the 4 lanes of the row
            ss += dpp_mov<0x4E>(ss);
            sq += dpp_mov<0xB1>(sq);
            sq += dpp_mov<0x4E>(sq);
        }
        if (part == 0) {
            const bool on = p.qk_l2_norm && t < n;
            sIk[t] = on ? 1.f / sqrtf(ss + 1e-12f) : 1.f;
            sIq[t] = on ? 1.f / sqrtf(sq + 1e-12f) : 1.f;
        }
    }
    lds_barrier();
    const float scale = p.scale;
    if (tid < CH) {
        const int t = tid;
        const float gl = sG[n - 1];
        sRw[t] = sBeta[t] * expf(sG[t]) * sIk[t];  // row scale of K in W's right-hand side
        float *sc = reinterpret_cast<float *>(rec + R_SC);
        sc[t] = t < n ? expf(gl - sG[t]) * sIk[t] : 0.f;  // kd: key weight of token t in the state update
        sc[CH + t] = scale * sIq[t] * expf(sG[t]);        // gq: read-out weight of the incoming state
        if (t == 0) sc[2 * CH] = DEC ? expf(gl) : 1.f;    // gamma_C
    }

    // ---- K Q^T and K K^T, 16 x 16 tiles (wave = token block tb, tiles sb <= tb);
    // the accumulators hold [s = 16 sb + 4 lq + i][t = 16 tb + lr]
    {
        const int tb = wave;
        f4v accq[4], acck[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            accq[sb] = acck[sb] = f4v{0.f, 0.f, 0.f, 0.f};
            if (sb <= tb) {
#pragma unroll
                for (int kk = 0; kk < D128; kk += 32) {
                    const h8 ak = ld_h8(&sK[16 * sb + lr][kk + lk]);
                    accq[sb] = mfma16(ak, ld_h8(&sQ[16 * tb + lr][kk + lk]), accq[sb]);
                    if constexpr (RET) acck[sb] = mfma16(ak, ld_h8(&sK[16 * tb + lr][kk + lk]), acck[sb]);
                }
            }
        }
        lds_barrier();  // Q is dead: A takes its rows
        const int t = 16 * tb + lr;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const int s0 = 16 * sb + 4 * lq;
            f4v pv, av;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = s0 + i;
                const float dg = (s <= t) ? expf(sG[t] - sG[s]) : 0.f;
                pv[i] = scale * sIq[t] * sIk[s] * dg * accq[sb][i];
                av[i] = (s < t) ? sBeta[t] * sIk[t] * sIk[s] * dg * acck[sb][i] : 0.f;
            }
            h4 hi, lo;
            split4(pv, hi, lo);
            // P rows in fragment order: block (tb * 2 + s0 / 32) * 2 + plane
            const uint32_t po = R_P + ((uint32_t)((tb * 2 + (s0 >> 5)) * 2) * 64 + ((s0 & 31) >> 3) * 16 + lr) * 16 + ((s0 & 7) >> 2) * 8;
            *reinterpret_cast<h4 *>(rec + po) = hi;
            *reinterpret_cast<h4 *>(rec + po + 1024) = lo;
            if constexpr (RET) *reinterpret_cast<f4v *>(&sA[t][s0]) = av;
        }
    }
    lds_barrier();

    // ---- [W | U] = (I + A)^-1 [diag(beta gamma / |k|) K | diag(beta) V]; column per thread
    const int col = tid & (D128 - 1);
    const bool wcol = tid < D128;
    float x[CH];
    if constexpr (RET) {
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            // four independent partial sums keep the FMA pipeline busy
            float r[4] = {wcol ? sRw[t] * (float)sK[t][col] : sBeta[t] * (float)sV[t][col], 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < t; ++s) r[s & 3] = fmaf(-sA[t][s], x[s], r[s & 3]);
            x[t] = (r[0] + r[1]) + (r[2] + r[3]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < CH; ++t) x[t] = wcol ? 0.f : (float)sV[t][col];
    }
    // U in fragment order: tokens 4 qd .. 4 qd + 3 of row col (block (qd / 4) * 8 + col / 16)
    if (!wcol) {
#pragma unroll
        for (int qd = 0; qd < CH / 4; ++qd)
            *reinterpret_cast<f4v *>(rec + R_U + ((uint32_t)(((qd >> 2) * 8 + (col >> 4)) * 64 + (qd & 3) * 16 + (col & 15))) * 16) =
                f4v{x[4 * qd], x[4 * qd + 1], x[4 * qd + 2], x[4 * qd + 3]};
    }
    if constexpr (RET) {
        lds_barrier();  // K and V are dead: W (hi, lo) rows take their place
        if (wcol) {
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const half_t hi = (half_t)x[t];
                sW[0][t][col] = hi;
                sW[1][t][col] = (half_t)(x[t] - (float)hi);
            }
        }
        lds_barrier();
        // W fragments: f = block * 64 + lane, block = (tb * 4 + kk) * 2 + plane
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int f = tid + 256 * g, blk = f >> 6, fl = f & 63;
            const int tb = blk >> 3, kk = (blk >> 1) & 3, pl = blk & 1;
            *reinterpret_cast<h8 *>(rec + R_W + (size_t)f * 16) = ld_h8(&sW[pl][16 * tb + (fl & 15)][32 * kk + 8 * (fl >> 4)]);
        }
    }
}

// ------------------------------------------------------------------ phase 2
// 512 threads.  Waves 0-3 carry the state chain of a 32-row tile, kept
// transposed (key rows, state-row columns) in MFMA accumulators; waves 4-7
// compute the outputs from the chain's LDS copies of S and D.  Per chunk j
// (LDS buffer j & 1):
//   chain:  A  S (hi, lo) -> sS[b]                         | output: -
//           == barrier 1 ==
//           B  D = U - W S^T -> sDt[b], (kd D) -> sDs      | O1 O^T = S Q^T
//           == barrier 2 ==
//           E  S^T <- gamma_C S^T + K^T (kd D)             | O2 O^T = gq O^T + D^T P^T, store
// S and D are double-buffered, so a buffer is rewritten only after every
// output wave has passed the barrier that follows its last read.  Operands
// are read with buffer loads: the chunk record's base goes into a scalar
// resource descriptor and each lane's offset is a loop-invariant register, so
// the loop does no vector address arithmetic.  The operands of chunk j + 1
// are loaded during chunk j into the second of two register sets; every load
// is unconditional, since a branch around a load makes the compiler wait for
// it on the spot.
template <int RULE, int NVB>
__global__ __launch_bounds__(512) void k_chunk_scan(const Params p, const int32_t *off, const char *ws)
{
    constexpr bool RET = rule_retrieves(RULE);
    constexpr int TR = 16 * NVB;          // state rows of this workgroup
    constexpr int NTILE = D128 / TR;      // workgroups per head
    constexpr int LS = D128 + 8;  // fp16 state row (272 B)
    constexpr int LDT = CH + 8;   // fp16 row of the transposed delta (144 B)

    // Row strides of 68 and 36 dwords put the 16 lanes of a 16-byte access
    // phase on 16 distinct 4-bank groups.
    __shared__ __align__(16) half_t sS[2][2][TR][LS];    // [buffer][hi, lo][row][key]
    __shared__ __align__(16) half_t sDt[2][2][TR][LDT];  // [buffer][hi, lo][row][token] D^T
    __shared__ __align__(16) half_t sDs[2][TR][LDT];     // [hi, lo][row][token] (kd D)^T, chain only
    __shared__ __align__(16) half_t sO[4][16][TR + 8];   // per output wave: [token][row] staging for the store

    const int HV = p.HV;
    // XCD-aware order: blocks i, i + 8, ... (one XCD) are the row tiles of one head
    const int xl = blockIdx.x & 7, tile = (blockIdx.x >> 3) % NTILE, grp = blockIdx.x / (8 * NTILE);
    const int bh = grp * 8 + xl;
    if (bh >= p.B * HV) return;
    const int b = bh / HV, h = bh % HV;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4, lk = lq * 8;
    const int row0 = tile * TR;
    const uint32_t l16 = (uint32_t)lane * 16;

    const float *src;
    float *dst;
    if (!state_ptrs(p, b, h, src, dst)) return;
    int64_t rs, re;
    request_range(p, b, rs, re);
    const int c0 = off[b], nch = off[b + 1] - off[b];
    const int tb = wave & 3;  // token block of this wave (D rows for the chain, O columns for the output)

    if (wave < 4) {
        // ================================================================ chain
        // Sc[a][rt][i] = S[row0 + 16 rt + lr][16 (2 wave + a) + 4 lq + i]
        f4v Sc[2][NVB];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int rt = 0; rt < NVB; ++rt)
                Sc[a][rt] = src ? *reinterpret_cast<const f4v *>(src + (size_t)(row0 + 16 * rt + lr) * D128 + 16 * (2 * wave + a) + 4 * lq)
                                : f4v{0.f, 0.f, 0.f, 0.f};
        struct Ops {
            h8 wh[4], wl[4];  // W (hi, lo) of token block tb, four k-steps of 32
            h8 kt[2][2];      // K^T fragments: key tiles 2 wave + a, token steps ks
            f4v u[NVB];       // U at this lane's D positions, one per row block
            f4v kd;           // kd of this lane's four D tokens
            float gc;         // gamma_C
        };
        const uint32_t offW = R_W + (uint32_t)tb * 8 * 1024 + l16;
        const uint32_t offK = R_KT + (uint32_t)(2 * wave) * 2 * 1024 + l16;
        const uint32_t offU = R_U + (uint32_t)(tb * 8 + NVB * tile) * 1024 + l16;
        const uint32_t offKd = R_SC + (uint32_t)(16 * tb + 4 * lq) * 4;
        auto fetch = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(ws + ((size_t)(c0 + jj) * HV + h) * WS_REC);
            if constexpr (RET) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    f.wh[kk] = ld_b128<h8>(r, offW + 2048 * kk);
                    f.wl[kk] = ld_b128<h8>(r, offW + 2048 * kk + 1024);
                }
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) f.kt[a][ks] = ld_b128<h8>(r, offK + (2 * a + ks) * 1024);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) f.u[vb] = ld_b128<f4v>(r, offU + vb * 1024);
            f.kd = ld_b128<f4v>(r, offKd);
            f.gc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, R_SC + 2 * CH * 4, 0, 0));
        };
        auto step = [&](int j, const Ops &cur, Ops &nxt) {
            const int bf = j & 1;
            // ---- A: state tile -> LDS (hi, lo), four consecutive keys per write
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt) {
                    h4 hi, lo;
                    split4(Sc[a][rt], hi, lo);
                    *reinterpret_cast<h4 *>(&sS[bf][0][16 * rt + lr][16 * (2 * wave + a) + 4 * lq]) = hi;
                    *reinterpret_cast<h4 *>(&sS[bf][1][16 * rt + lr][16 * (2 * wave + a) + 4 * lq]) = lo;
                }
            fetch(j + 1 < nch ? j + 1 : j, nxt);  // the last chunk re-reads itself
            // keep the prefetch where it is: neither the optimiser nor the
            // scheduler may move the loads past this point in either direction
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();  // 1
            // ---- B: D = U - W S^T for token block tb and every row block (D rows = tokens)
            f4v accD[NVB];
            {
                // hi*hi and lo*hi share a chain; with two row blocks hi*lo gets its
                // own (enough independent chains to keep the matrix core busy)
                constexpr int NA = NVB >= 4 ? 1 : 2;
                f4v a2[NVB][2] = {};
                if constexpr (RET) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                        for (int vb = 0; vb < NVB; ++vb) {
                            const h8 shi = ld_h8(&sS[bf][0][16 * vb + lr][32 * kk + lk]);
                            const h8 slo = ld_h8(&sS[bf][1][16 * vb + lr][32 * kk + lk]);
                            a2[vb][0] = mfma16(cur.wh[kk], shi, a2[vb][0]);
                            a2[vb][NA - 1] = mfma16(cur.wh[kk], slo, a2[vb][NA - 1]);
                            a2[vb][0] = mfma16(cur.wl[kk], shi, a2[vb][0]);
                        }
                }
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) accD[vb] = NA == 2 ? a2[vb][0] + a2[vb][1] : a2[vb][0];
            }
            // D at (tokens 16 tb + 4 lq + i, state row 16 vb + lr): four consecutive
            // tokens per lane -> one 8-byte write per plane
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                f4v d, ds;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    d[i] = cur.u[vb][i] - accD[vb][i];
                    ds[i] = cur.kd[i] * d[i];
                }
                h4 dh, dl, sh, sl;
                split4(d, dh, dl);
                split4(ds, sh, sl);
                const int r = 16 * vb + lr, c = 16 * tb + 4 * lq;
                *reinterpret_cast<h4 *>(&sDt[bf][0][r][c]) = dh;
                *reinterpret_cast<h4 *>(&sDt[bf][1][r][c]) = dl;
                *reinterpret_cast<h4 *>(&sDs[0][r][c]) = sh;
                *reinterpret_cast<h4 *>(&sDs[1][r][c]) = sl;
            }
            lds_barrier();  // 2
            // ---- E: S^T <- gamma_C S^T + K^T (kd D) for key tiles 2 wave + a, row blocks rt
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt) Sc[a][rt] *= cur.gc;
            {
                // with two row blocks the lo products get their own chains
                constexpr bool SEPL = NVB < 4;
                f4v lo4[2][NVB] = {};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int rt = 0; rt < NVB; ++rt) {
                        const h8 dhi = ld_h8(&sDs[0][16 * rt + lr][32 * ks + lk]);
                        const h8 dlo = ld_h8(&sDs[1][16 * rt + lr][32 * ks + lk]);
#pragma unroll
                        for (int a = 0; a < 2; ++a) {
                            Sc[a][rt] = mfma16(cur.kt[a][ks], dhi, Sc[a][rt]);
                            if constexpr (SEPL) lo4[a][rt] = mfma16(cur.kt[a][ks], dlo, lo4[a][rt]);
                            else Sc[a][rt] = mfma16(cur.kt[a][ks], dlo, Sc[a][rt]);
                        }
                    }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int rt = 0; rt < NVB; ++rt)
                        if constexpr (SEPL) Sc[a][rt] += lo4[a][rt];
            }
        };
        // two operand sets used in turn, so no register copy waits on a prefetch
        Ops opa, opb;
        if (nch > 0) fetch(0, opa);
        for (int j = 0; j < nch; j += 2) {
            step(j, opa, opb);
            if (j + 1 < nch) step(j + 1, opb, opa);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int rt = 0; rt < NVB; ++rt)
                *reinterpret_cast<f4v *>(dst + (size_t)(row0 + 16 * rt + lr) * D128 + 16 * (2 * wave + a) + 4 * lq) = Sc[a][rt];
    } else {
        // ================================================================ outputs
        half_t *o = static_cast<half_t *>(p.o);
        struct Ops {
            h8 q[4];          // q rows of token block tb, four k-steps of 32
            h8 ph[2], pl[2];  // P (hi, lo) rows of token block tb, two token steps of 32
            float gq;         // gq of this lane's token
        };
        const uint32_t offQ = R_Q + (uint32_t)tb * 4 * 1024 + l16;
        // o byte offset of this lane's token (16 tb + lr) and rows 4 lq .. +3 inside a chunk
        const int tok_bytes = HV * D128 * 2;
        // after the LDS transpose each lane stores 16 bytes: token 16 tb + (lane >> 2),
        // rows 8 (lane & 3) .. +7 of the tile (TR = 32: four lanes per token)
        static_assert(TR == 32, "the output transpose assumes 32-row tiles");
        const int st_tok = lane >> 2, st_q = lane & 3;
        const uint32_t offO = (uint32_t)((16 * tb + st_tok) * tok_bytes + 16 * st_q);
        const uint32_t offP = R_P + (uint32_t)tb * 4 * 1024 + l16;
        const uint32_t offG = R_SC + (uint32_t)(CH + 16 * tb + lr) * 4;
        auto fetch = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(ws + ((size_t)(c0 + jj) * HV + h) * WS_REC);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.q[kk] = ld_b128<h8>(r, offQ + kk * 1024);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                f.ph[ks] = ld_b128<h8>(r, offP + ks * 2048);
                f.pl[ks] = ld_b128<h8>(r, offP + ks * 2048 + 1024);
            }
            f.gq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, offG, 0, 0));
        };
        // Store the output tile of chunk jo, staged in sO, as one 16-byte write per
        // lane.  The store is unconditional: the resource spans the chunk's
        // valid tokens only (none for jo < 0), so lanes past the request's end
        // write nothing (a branch here would make every later wait drain it).
        auto store_out = [&](int jo) {
            const int64_t t0 = rs + (int64_t)jo * CH;
            const int n = jo >= 0 ? (int)((re - t0) < CH ? (re - t0) : CH) : 0;
            half_t *base = jo >= 0 ? o + ((size_t)t0 * HV + h) * D128 + row0 : o;
            const __amdgpu_buffer_rsrc_t ro =
                __builtin_amdgcn_make_buffer_rsrc(base, 0, n > 0 ? (int)((n - 1) * tok_bytes + TR * 2) : 0, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b128(ld_b128_lds(&sO[tb][st_tok][8 * st_q]), ro, offO, 0, 0);
        };
        auto step = [&](int j, const Ops &cur, Ops &nxt) {
            const int bf = j & 1;
            fetch(j + 1 < nch ? j + 1 : j, nxt);
            asm volatile("" ::: "memory");  // pin the prefetch (see the chain role)
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();  // 1 (also completes this wave's staging of chunk j - 1)
            store_out(j - 1);
            // ---- O1: O^T = S Q^T for row blocks 0, 1 and token block tb:
            // rows 16 vb + 4 lq + i, token 16 tb + lr
            f4v acc[NVB], acl[NVB];
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) acc[vb] = acl[vb] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    const h8 shi = ld_h8(&sS[bf][0][16 * vb + lr][32 * kk + lk]);
                    const h8 slo = ld_h8(&sS[bf][1][16 * vb + lr][32 * kk + lk]);
                    acc[vb] = mfma16(shi, cur.q[kk], acc[vb]);
                    acl[vb] = mfma16(slo, cur.q[kk], acl[vb]);
                }
            lds_barrier();  // 2
            // ---- O2: O^T = gq O^T + D^T P^T; P is lower triangular (zeros above the
            // diagonal are multiplied anyway so every prefetched fragment is used)
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) acc[vb] = cur.gq * (acc[vb] + acl[vb]);
            {
                f4v p3[NVB] = {};  // the two lo products in their own chain
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) {
                        const h8 dhi = ld_h8(&sDt[bf][0][16 * vb + lr][32 * ks + lk]);
                        const h8 dlo = ld_h8(&sDt[bf][1][16 * vb + lr][32 * ks + lk]);
                        acc[vb] = mfma16(dhi, cur.ph[ks], acc[vb]);
                        p3[vb] = mfma16(dlo, cur.ph[ks], p3[vb]);
                        p3[vb] = mfma16(dhi, cur.pl[ks], p3[vb]);
                    }
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) acc[vb] += p3[vb];
            }
            // stage the tile as [token][row]; the next chunk (or the loop's end) stores it
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                h4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = (half_t)acc[vb][i];
                *reinterpret_cast<h4 *>(&sO[tb][lr][16 * vb + 4 * lq]) = ov;
            }
        };
        Ops opa, opb;
        if (nch > 0) fetch(0, opa);
        {
            // a store that writes nothing (empty resource): on entry the loop
            // then sees the same outstanding pattern as in steady state (the
            // previous chunk's output store behind the prefetch), so the
            // compiler's waits for the prefetch need not cover a real store
            const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(o, 0, 0, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b128(u4v{0u, 0u, 0u, 0u}, none, 0, 0, 0);
        }
        for (int j = 0; j < nch; j += 2) {
            step(j, opa, opb);
            if (j + 1 < nch) step(j + 1, opb, opa);
        }
        if (nch > 0) {
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging has landed
            store_out(nch - 1);
        }
    }
}

// ------------------------------------------------------------------ host side

size_t chunked_workspace_bytes(int64_t T, int B, int HV)
{
    const int64_t maxch = (T + CH - 1) / CH + B;
    const size_t table = ((size_t)(B + 1) * 4 + 255) / 256 * 256;
    return table + (size_t)maxch * HV * WS_REC;
}

// Row tile of the scan: 32 rows (measured on MI355X: 64-row tiles halve the
// per-row operand reads but lengthen each chunk step by 1.7x, which loses on
// both the single long sequence and the batched prefill).
template <int RULE, int NVB>
static void launch_scan(const Params &p, const int32_t *off, const char *rec, hipStream_t s)
{
    constexpr int NTILE = D128 / (16 * NVB);
    const int64_t nbh = (int64_t)p.B * p.HV;
    const int64_t blocks = (nbh + 7) / 8 * 8 * NTILE;
    if (blocks > 0) hipLaunchKernelGGL((k_chunk_scan<RULE, NVB>), dim3((unsigned)blocks), dim3(512), 0, s, p, off, rec);
}

template <int RULE>
static hipError_t launch_rule(const Params &p, void *ws, hipStream_t s)
{
    const int64_t maxch = (p.T + CH - 1) / CH + p.B;
    const size_t table = ((size_t)(p.B + 1) * 4 + 255) / 256 * 256;
    char *base = static_cast<char *>(ws);
    int32_t *off = reinterpret_cast<int32_t *>(base);
    char *rec = base + table;
    hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(256), 0, s, p, off);
    if (maxch * p.HV > 0)
        hipLaunchKernelGGL((k_chunk_prep<RULE>), dim3((unsigned)(maxch * p.HV)), dim3(256), 0, s, p, off, rec);
    launch_scan<RULE, 2>(p, off, rec, s);
    return hipGetLastError();
}

hipError_t launch_chunked(const Params &p, int rule, void *ws, hipStream_t s)
{
    switch (rule) {
    case LINEAR: return launch_rule<LINEAR>(p, ws, s);
    case GATED: return launch_rule<GATED>(p, ws, s);
    case DELTA: return launch_rule<DELTA>(p, ws, s);
    default: return launch_rule<GATED_DELTA>(p, ws, s);
    }
}

}  // namespace gdr
