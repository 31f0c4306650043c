// gdr_chunked.hip -- chunk-parallel prefill (chunk = 64 tokens) on MFMA.
//
// The "com.microsoft.GatedDeltaNet" README (Attributes, chunk_size) names a
// chunk-parallel prefill whose chunk size does not change the result.  The
// form used here is the recurrence of the README's Description unrolled over
// one chunk (scalar per-head decay; K-major notation M = S^T for the
// derivation, V-major S in memory):
//   gamma_t = exp(G_t), G_t = sum of the log decays up to t inside the chunk,
//   (I + A) D = diag(beta) V - diag(beta gamma) K_n S0^T,
//   A_ts = beta_t (gamma_t / gamma_s) k_t.k_s  (s < t),  k_n = k / |k|
// so D = U - W S0^T with
//   W = (I+A)^-1 diag(beta gamma |k|^-1) K,   U = (I+A)^-1 diag(beta) V,
//   O = gq (Q S0^T) + P D,  P_ts = scale (gamma_t/gamma_s) (q_t.k_s)/(|q_t||k_s|)  (s <= t),
//       gq_t = scale gamma_t / |q_t|,
//   S_C = gamma_C S0 + (diag(kd) D)^T K,  kd_t = (gamma_C / gamma_t) / |k_t|.
// Rules without retrieval (linear, gated) have D = V.
//
// Three launches:
//   k_chunk_table  one workgroup: per-request chunk offsets (exclusive scan of
//                  ceil(len/64)); the host never reads cu_seqlens.
//   k_chunk_prep   one workgroup per (chunk, head), all chunks in parallel:
//                  Q K^T and K K^T on 16x16x32 f16 MFMA (q/k are fp16, so the
//                  products are exact up to fp32 accumulation), the unit
//                  lower-triangular solve for [W | U] by fp32 forward
//                  substitution (one column per thread), and the per-token
//                  scalars.  W and P are stored as fp16 (hi, lo) pairs, and
//                  the chunk's K transposed (dk x 64) for the scan.
//   k_chunk_scan   one workgroup per (request, head, 32 state rows), chunks
//                  in order; the state tile lives in MFMA accumulators.  Each
//                  chunk: D = U - W S^T, S <- gamma_C S + (kd D)^T K on four
//                  "chain" waves, O = gq (Q S^T) + P D on four "output" waves.  Every fp32 operand is split
//                  into fp16 hi + lo and multiplied as hi*hi + hi*lo + lo*hi
//                  (fp16 operands need no split), which keeps the products at
//                  about fp32 accuracy on the f16 matrix cores.  The four
//                  row tiles of a head are dispatched to the same XCD so the
//                  per-chunk W, P, Q, K reads are shared through its L2.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int CH = 64;          // chunk length
constexpr int D128 = 128;       // dk = dv
constexpr int TR = 32;          // state rows per scan workgroup
constexpr int NTILE = D128 / TR;
constexpr int SC_STRIDE = 256;  // floats of per-chunk scalars

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
template <int RULE>
__global__ __launch_bounds__(256) void k_chunk_prep(const Params p, const int32_t *__restrict__ off,
                                                   half_t *__restrict__ ws_w, half_t *__restrict__ ws_p,
                                                   float *__restrict__ ws_u, float *__restrict__ ws_s,
                                                   half_t *__restrict__ ws_kt)
{
    constexpr bool DEC = rule_decays(RULE);
    constexpr bool RET = rule_retrieves(RULE);
    constexpr bool BETA = rule_has_beta(RULE);
    constexpr int LD = D128 + 8;  // padded fp16 row (bank spread)
    constexpr int LA = CH + 4;    // 16-byte rows: the solve reads A rows as float4 broadcasts

    static_assert(LD * sizeof(half_t) == LA * sizeof(float), "Q rows and A rows share one LDS footprint");
    __shared__ __align__(16) half_t sK[CH][LD];
    __shared__ __align__(16) half_t sV[CH][LD];
    // Q is dead once Q K^T is formed; the fp32 matrix A reuses its rows
    // (same 272-byte row stride), which keeps three workgroups per CU.
    __shared__ __align__(16) char sQA[CH * LD * sizeof(half_t)];
    half_t(*sQ)[LD] = reinterpret_cast<half_t(*)[LD]>(sQA);
    float(*sA)[LA] = reinterpret_cast<float(*)[LA]>(sQA);
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
    const size_t ch = (size_t)ci * HV + h;

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
    }
    lds_barrier();

    // ---- K^T of the chunk (dk rows, 64 tokens each) for the scan's state update;
    // thread = (key column, half of the tokens), lanes read one LDS row each step
    {
        const int c = tid & (D128 - 1), th = tid >> 7;
        h8 col[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int x = 0; x < 8; ++x) col[g][x] = sK[32 * th + 8 * g + x][c];
        h8 *dstk = reinterpret_cast<h8 *>(ws_kt + ch * D128 * CH + (size_t)c * CH + 32 * th);
#pragma unroll
        for (int g = 0; g < 4; ++g) dstk[g] = col[g];
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
    if (tid < CH) sRw[tid] = sBeta[tid] * expf(sG[tid]) * sIk[tid];  // row scale of K in the W right-hand side

    // ---- Q K^T -> P (hi, lo) and K K^T -> A, tiles of 16 x 16 (wave = token block).
    // Wave tb reads only Q rows of its block and writes only A rows of its
    // block, so once all its products are formed it may overwrite them.
    const float scale = p.scale;
    {
        const int tb = wave;
        const int lr = lane & 15, lk = (lane >> 4) * 8;
        f4v accq[4], acck[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            accq[sb] = acck[sb] = f4v{0.f, 0.f, 0.f, 0.f};
            if (sb <= tb) {
#pragma unroll
                for (int kk = 0; kk < D128; kk += 32) {
                    const h8 bk = ld_h8(&sK[16 * sb + lr][kk + lk]);
                    accq[sb] = mfma16(ld_h8(&sQ[16 * tb + lr][kk + lk]), bk, accq[sb]);
                    if constexpr (RET) acck[sb] = mfma16(ld_h8(&sK[16 * tb + lr][kk + lk]), bk, acck[sb]);
                }
            }
        }
        // all of this wave's LDS reads of Q must land before its A rows overwrite them
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const int s = 16 * sb + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + (lane >> 4) * 4 + i;
                const float dg = (s <= t) ? expf(sG[t] - sG[s]) : 0.f;
                const float pv = scale * sIq[t] * sIk[s] * dg * accq[sb][i];
                const half_t hi = (half_t)pv;
                ws_p[(ch * 2 + 0) * CH * CH + t * CH + s] = hi;
                ws_p[(ch * 2 + 1) * CH * CH + t * CH + s] = (half_t)(pv - (float)hi);
                if constexpr (RET) sA[t][s] = (s < t) ? sBeta[t] * sIk[t] * sIk[s] * dg * acck[sb][i] : 0.f;
            }
        }
    }
    lds_barrier();

    // ---- [W | U] = (I + A)^-1 [diag(beta gamma / |k|) K | diag(beta) V]; column per thread
    if constexpr (RET) {
        const int c = tid;
        const bool wcol = c < D128;
        const int cc = wcol ? c : c - D128;
        float x[CH];
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            // four independent partial sums keep the FMA pipeline busy
            float r[4] = {wcol ? sRw[t] * (float)sK[t][cc] : sBeta[t] * (float)sV[t][cc], 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < t; ++s) r[s & 3] = fmaf(-sA[t][s], x[s], r[s & 3]);
            x[t] = (r[0] + r[1]) + (r[2] + r[3]);
        }
        if (wcol) {
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const half_t hi = (half_t)x[t];
                ws_w[(ch * 2 + 0) * CH * D128 + t * D128 + cc] = hi;
                ws_w[(ch * 2 + 1) * CH * D128 + t * D128 + cc] = (half_t)(x[t] - (float)hi);
            }
        } else {
            // U^T: state row cc, 64 tokens, written as 16-byte vectors
            f4v *ut = reinterpret_cast<f4v *>(ws_u + ch * CH * D128 + (size_t)cc * CH);
#pragma unroll
            for (int t = 0; t < CH; t += 4) ut[t / 4] = f4v{x[t], x[t + 1], x[t + 2], x[t + 3]};
        }
    } else {
        // no retrieval: D = V, stored transposed like U
        const int c = tid & (D128 - 1), half = tid >> 7;
        f4v *ut = reinterpret_cast<f4v *>(ws_u + ch * CH * D128 + (size_t)c * CH + 32 * half);
#pragma unroll
        for (int t = 0; t < 32; t += 4)
            ut[t / 4] = f4v{(float)sV[32 * half + t][c], (float)sV[32 * half + t + 1][c], (float)sV[32 * half + t + 2][c],
                            (float)sV[32 * half + t + 3][c]};
    }

    // ---- per-token scalars for the scan
    if (tid < CH) {
        const int t = tid;
        const float gl = sG[n - 1];
        float *sc = ws_s + ch * SC_STRIDE;
        sc[t] = scale * sIq[t] * expf(sG[t]);
        sc[CH + t] = t < n ? expf(gl - sG[t]) * sIk[t] : 0.f;
        if (t == 0) sc[2 * CH] = expf(gl);
    }
}

// ------------------------------------------------------------------ phase 2
// 512 threads.  Waves 0-3 carry the state chain of a 32-row tile; waves 4-7
// compute the outputs from the chain's LDS copies of S and D, so the output
// work stays off the serial path.  Per chunk j (LDS buffer j & 1):
//   chain:  A  S (hi, lo) -> sS[b]          | output: -
//           == barrier 1 ==
//           B  D = U - W S^T -> sDt[b], and (kd D) -> sDs   | O1 Opre = Q S^T
//           == barrier 2 ==
//           E  S <- gamma_C S + (kd D)^T K  | O2 O = gq Opre + P D, store
// S and D are double-buffered, so a buffer is rewritten only after every
// output wave has passed the barrier that follows its last read.
// (no __restrict__ on the operands: loads through restrict pointers may be
// moved across the prefetch fences below, which would put two prefetches in
// flight and exhaust the registers)
template <int RULE>
__global__ __launch_bounds__(512) void k_chunk_scan(const Params p, const int32_t *off, const half_t *ws_w,
                                                   const half_t *ws_p, const float *ws_u, const float *ws_s,
                                                   const half_t *ws_kt)
{
    constexpr bool RET = rule_retrieves(RULE);
    constexpr int LS = D128 + 8;   // fp16 state row (272 B)
    constexpr int LDT = CH + 8;    // fp16 row of the transposed delta (144 B)

    // Operands are split into fp16 (hi, lo) once, by the lane that owns the
    // value, and stored as planes; every MFMA fragment is then one 16-byte
    // LDS read.  Row strides of 68 and 36 dwords put the 16 lanes of a
    // 16-byte access phase on 16 distinct 4-bank groups.
    __shared__ __align__(16) half_t sS[2][2][TR][LS];    // [buffer][hi, lo] state tile
    __shared__ __align__(16) half_t sDt[2][2][TR][LDT];  // [buffer][hi, lo] D^T
    __shared__ __align__(16) half_t sDs[2][TR][LDT];     // [hi, lo] (kd D)^T, chain only

    const int HV = p.HV, H = p.H;
    // XCD-aware order: blocks i, i+8, i+16, i+24 (one XCD) are the 4 tiles of one head
    const int xl = blockIdx.x & 7, tile = (blockIdx.x >> 3) & (NTILE - 1), grp = blockIdx.x >> 5;
    const int bh = grp * 8 + xl;
    if (bh >= p.B * HV) return;
    const int b = bh / HV, h = bh % HV;
    const int qh = (int)(((int64_t)h * H) / HV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4, lk = lq * 8;
    const int row0 = tile * TR;

    const float *src;
    float *dst;
    if (!state_ptrs(p, b, h, src, dst)) return;
    int64_t rs, re;
    request_range(p, b, rs, re);
    const int c0 = off[b], nch = off[b + 1] - off[b];
    const int tb = wave & 3;      // token block of this wave in steps B, O1, O2
    const int tr = 16 * tb + lr;  // A-operand row (token) of this lane

    if (wave < 4) {
        // ================================================================ chain
        // the wave owns key-column tiles 2 wave and 2 wave + 1 of both 16-row
        // blocks: Sacc[2 vb + jj] holds rows 16 vb + 4 lq + i, columns
        // 16 (2 wave + jj) + lr (accumulator layout); distinct waves need
        // distinct K^T fragments
        const int dkb0 = 2 * wave;
        f4v Sacc[4];
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = row0 + 16 * vb + 4 * lq + i, c = 16 * (dkb0 + jj) + lr;
                    Sacc[2 * vb + jj][i] = src ? src[(size_t)r * D128 + c] : 0.f;
                }
        struct Ops {
            h8 wh[4], wl[4];  // W (hi, lo) rows of token block tb, four k-steps of 32
            h8 kt[2][2];      // K^T fragments: token steps x this wave's two dk tiles
            f4v u[2];         // U at this lane's D-layout positions (four tokens each)
            f4v kd;           // kd of this lane's four D-layout tokens
            float gc;         // gamma_C
        };
        // every load unconditional: a branch around a load makes the compiler
        // wait for it on the spot, which would defeat the prefetch
        auto fetch = [&](int jj, Ops &f) {
            const size_t ch = (size_t)(c0 + jj) * HV + h;
            if constexpr (RET) {
                const half_t *wh = ws_w + (ch * 2 + 0) * CH * D128 + (size_t)tr * D128;
                const half_t *wl = ws_w + (ch * 2 + 1) * CH * D128 + (size_t)tr * D128;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    f.wh[kk] = ld_h8(wh + 32 * kk + lk);
                    f.wl[kk] = ld_h8(wl + 32 * kk + lk);
                }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int jj2 = 0; jj2 < 2; ++jj2)
                    f.kt[ks][jj2] = ld_h8(ws_kt + ch * D128 * CH + (size_t)(16 * (dkb0 + jj2) + lr) * CH + 32 * ks + lk);
#pragma unroll
            for (int vb = 0; vb < 2; ++vb)
                f.u[vb] = *reinterpret_cast<const f4v *>(ws_u + ch * CH * D128 + (size_t)(row0 + 16 * vb + lr) * CH +
                                                          16 * tb + 4 * lq);
            f.kd = *reinterpret_cast<const f4v *>(ws_s + ch * SC_STRIDE + CH + 16 * tb + 4 * lq);
            f.gc = ws_s[ch * SC_STRIDE + 2 * CH];
        };
        auto step = [&](int j, const Ops &cur, Ops &nxt) {
            const int bf = j & 1;
            // ---- A: state tile -> LDS (hi, lo)
#pragma unroll
            for (int vb = 0; vb < 2; ++vb)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = Sacc[2 * vb + jj][i];
                        const half_t hi = (half_t)x;
                        sS[bf][0][16 * vb + 4 * lq + i][16 * (dkb0 + jj) + lr] = hi;
                        sS[bf][1][16 * vb + 4 * lq + i][16 * (dkb0 + jj) + lr] = (half_t)(x - (float)hi);
                    }
            fetch(j + 1 < nch ? j + 1 : j, nxt);  // the last chunk re-reads itself
            // keep the prefetch where it is: neither the optimiser nor the
            // scheduler may move the loads past this point in either direction
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();  // 1
            // ---- B: D = U - W S^T for token block tb, state-row blocks 0, 1.
            // The three split products accumulate separately: six independent
            // MFMA chains of four instead of two chains of twelve.
            f4v accD[2];
            {
                f4v a3[2][3] = {};
                if constexpr (RET) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                        for (int vb = 0; vb < 2; ++vb) {
                            const h8 shi = ld_h8(&sS[bf][0][16 * vb + lr][32 * kk + lk]);
                            const h8 slo = ld_h8(&sS[bf][1][16 * vb + lr][32 * kk + lk]);
                            a3[vb][0] = mfma16(cur.wh[kk], shi, a3[vb][0]);
                            a3[vb][1] = mfma16(cur.wh[kk], slo, a3[vb][1]);
                            a3[vb][2] = mfma16(cur.wl[kk], shi, a3[vb][2]);
                        }
                }
#pragma unroll
                for (int vb = 0; vb < 2; ++vb) accD[vb] = a3[vb][0] + (a3[vb][1] + a3[vb][2]);
            }
            // D at (tokens 16 tb + 4 lq + i, state row 16 vb + lr): four consecutive
            // tokens per lane -> one 8-byte write per plane
#pragma unroll
            for (int vb = 0; vb < 2; ++vb) {
                h4 dh, dl, sh, sl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d = cur.u[vb][i] - accD[vb][i];
                    const float ds = cur.kd[i] * d;
                    dh[i] = (half_t)d;
                    dl[i] = (half_t)(d - (float)dh[i]);
                    sh[i] = (half_t)ds;
                    sl[i] = (half_t)(ds - (float)sh[i]);
                }
                const int r = 16 * vb + lr, c = 16 * tb + 4 * lq;
                *reinterpret_cast<h4 *>(&sDt[bf][0][r][c]) = dh;
                *reinterpret_cast<h4 *>(&sDt[bf][1][r][c]) = dl;
                *reinterpret_cast<h4 *>(&sDs[0][r][c]) = sh;
                *reinterpret_cast<h4 *>(&sDs[1][r][c]) = sl;
            }
            lds_barrier();  // 2
            // ---- E: S <- gamma_C S + (kd D)^T K for the wave's 4 state tiles
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) Sacc[jj][i] *= cur.gc;
            {
                f4v lo4[4] = {};  // lo products in their own chains
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int vb = 0; vb < 2; ++vb) {
                        const h8 dhi = ld_h8(&sDs[0][16 * vb + lr][32 * ks + lk]);
                        const h8 dlo = ld_h8(&sDs[1][16 * vb + lr][32 * ks + lk]);
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) {
                            Sacc[2 * vb + jj] = mfma16(dhi, cur.kt[ks][jj], Sacc[2 * vb + jj]);
                            lo4[2 * vb + jj] = mfma16(dlo, cur.kt[ks][jj], lo4[2 * vb + jj]);
                        }
                    }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) Sacc[jj] += lo4[jj];
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
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = row0 + 16 * vb + 4 * lq + i, c = 16 * (dkb0 + jj) + lr;
                    dst[(size_t)r * D128 + c] = Sacc[2 * vb + jj][i];
                }
    } else {
        // ================================================================ outputs
        const half_t *q = static_cast<const half_t *>(p.q);
        half_t *o = static_cast<half_t *>(p.o);
        struct Ops {
            h8 aq[4];          // Q rows of token block tb, four k-steps of 32
            h8 ph[2], pl[2];   // P (hi, lo) rows, two k-steps of 32
            f4v gq;            // gq of this lane's four D-layout tokens
            int n;             // valid tokens in the chunk
            int64_t t0;
        };
        auto fetch = [&](int jj, Ops &f) {
            const size_t ch = (size_t)(c0 + jj) * HV + h;
            f.t0 = rs + (int64_t)jj * CH;
            f.n = (int)((re - f.t0) < CH ? (re - f.t0) : CH);
            // rows past the request end read its last row; their outputs are not stored
            const int tq = tr < f.n ? tr : f.n - 1;
            const half_t *qp = q + ((size_t)(f.t0 + tq) * H + qh) * D128;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.aq[kk] = ld_h8(qp + 32 * kk + lk);
            const half_t *ph = ws_p + (ch * 2 + 0) * CH * CH + (size_t)tr * CH;
            const half_t *pl = ws_p + (ch * 2 + 1) * CH * CH + (size_t)tr * CH;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                f.ph[ks] = ld_h8(ph + 32 * ks + lk);
                f.pl[ks] = ld_h8(pl + 32 * ks + lk);
            }
            f.gq = *reinterpret_cast<const f4v *>(ws_s + ch * SC_STRIDE + 16 * tb + 4 * lq);
        };
        auto step = [&](int j, const Ops &cur, Ops &nxt) {
            const int bf = j & 1;
            fetch(j + 1 < nch ? j + 1 : j, nxt);
            asm volatile("" ::: "memory");  // pin the prefetch (see the chain role)
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();  // 1
            // ---- O1: Opre = Q S^T for token block tb, state-row blocks 0, 1
            f4v acc[2], acl[2] = {};
            acc[0] = acc[1] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int vb = 0; vb < 2; ++vb) {
                    const h8 shi = ld_h8(&sS[bf][0][16 * vb + lr][32 * kk + lk]);
                    const h8 slo = ld_h8(&sS[bf][1][16 * vb + lr][32 * kk + lk]);
                    acc[vb] = mfma16(cur.aq[kk], shi, acc[vb]);
                    acl[vb] = mfma16(cur.aq[kk], slo, acl[vb]);
                }
            lds_barrier();  // 2
            // ---- O2: O = gq Opre + P D; P is lower triangular (zeros above the
            // diagonal are multiplied anyway so every prefetched fragment is used)
#pragma unroll
            for (int vb = 0; vb < 2; ++vb)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[vb][i] = cur.gq[i] * (acc[vb][i] + acl[vb][i]);
            {
                f4v p3[2][2] = {};  // the two lo products in their own chains
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int vb = 0; vb < 2; ++vb) {
                        const h8 dhi = ld_h8(&sDt[bf][0][16 * vb + lr][32 * ks + lk]);
                        const h8 dlo = ld_h8(&sDt[bf][1][16 * vb + lr][32 * ks + lk]);
                        acc[vb] = mfma16(cur.ph[ks], dhi, acc[vb]);
                        p3[vb][0] = mfma16(cur.ph[ks], dlo, p3[vb][0]);
                        p3[vb][1] = mfma16(cur.pl[ks], dhi, p3[vb][1]);
                    }
#pragma unroll
                for (int vb = 0; vb < 2; ++vb) acc[vb] += p3[vb][0] + p3[vb][1];
            }
#pragma unroll
            for (int vb = 0; vb < 2; ++vb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tb + 4 * lq + i;
                    if (t < cur.n)
                        o[((size_t)(cur.t0 + t) * HV + h) * D128 + row0 + 16 * vb + lr] = (half_t)acc[vb][i];
                }
        };
        Ops opa, opb;
        if (nch > 0) fetch(0, opa);
        for (int j = 0; j < nch; j += 2) {
            step(j, opa, opb);
            if (j + 1 < nch) step(j + 1, opb, opa);
        }
    }
}

// ------------------------------------------------------------------ host side
size_t chunked_workspace_bytes(int64_t T, int B, int HV)
{
    const int64_t maxch = (T + CH - 1) / CH + B;
    const size_t per = (size_t)2 * CH * D128 * 2 + (size_t)2 * CH * CH * 2 + (size_t)CH * D128 * 4 + SC_STRIDE * 4 +
                       (size_t)D128 * CH * 2;
    const size_t table = ((size_t)(B + 1) * 4 + 255) / 256 * 256;
    return table + (size_t)maxch * HV * per;
}

template <int RULE>
static hipError_t launch_rule(const Params &p, void *ws, hipStream_t s)
{
    const int64_t maxch = (p.T + CH - 1) / CH + p.B;
    const size_t table = ((size_t)(p.B + 1) * 4 + 255) / 256 * 256;
    char *base = static_cast<char *>(ws);
    int32_t *off = reinterpret_cast<int32_t *>(base);
    const size_t nch = (size_t)maxch * p.HV;
    half_t *ws_w = reinterpret_cast<half_t *>(base + table);
    half_t *ws_p = ws_w + nch * 2 * CH * D128;
    float *ws_u = reinterpret_cast<float *>(ws_p + nch * 2 * CH * CH);
    float *ws_s = ws_u + nch * CH * D128;
    half_t *ws_kt = reinterpret_cast<half_t *>(ws_s + nch * SC_STRIDE);
    hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(256), 0, s, p, off);
    if (maxch * p.HV > 0)
        hipLaunchKernelGGL((k_chunk_prep<RULE>), dim3((unsigned)(maxch * p.HV)), dim3(256), 0, s, p, off, ws_w, ws_p,
                           ws_u, ws_s, ws_kt);
    const int64_t nbh = (int64_t)p.B * p.HV;
    const int64_t blocks = (nbh + 7) / 8 * 8 * NTILE;
    if (blocks > 0)
        hipLaunchKernelGGL((k_chunk_scan<RULE>), dim3((unsigned)blocks), dim3(512), 0, s, p, off, ws_w, ws_p, ws_u,
                           ws_s, ws_kt);
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
