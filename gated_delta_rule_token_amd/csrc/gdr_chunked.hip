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
//                  chunk: D = U - W S^T, O = gq (Q S^T) + P D,
//                  S <- gamma_C S + (kd D)^T K.  Every fp32 operand is split
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

    __shared__ __align__(16) half_t sK[CH][LD];
    __shared__ __align__(16) half_t sQ[CH][LD];
    __shared__ __align__(16) half_t sV[CH][LD];
    __shared__ float sA[CH][LA];
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

    // ---- chunk rows of K, Q (head qh) and V (head h) -> LDS, zero past the end
    for (int idx = tid; idx < CH * 16; idx += 256) {
        const int r = idx >> 4, c8 = (idx & 15) * 8;
        h8 kk = {}, qq = {}, vv = {};
        if (r < n) {
            const size_t tq = ((size_t)(t0 + r) * H + qh) * D128 + c8;
            kk = ld_h8(k + tq);
            qq = ld_h8(q + tq);
            vv = ld_h8(v + ((size_t)(t0 + r) * HV + h) * D128 + c8);
        }
        *reinterpret_cast<h8 *>(&sK[r][c8]) = kk;
        *reinterpret_cast<h8 *>(&sQ[r][c8]) = qq;
        *reinterpret_cast<h8 *>(&sV[r][c8]) = vv;
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

    // ---- per-token scalars: log decay, update rate, inverse norms
    if (tid < CH) {
        const int t = tid;
        float g = 0.f, bt = 0.f, ik = 1.f, iq = 1.f;
        if (t < n) {
            const size_t th = (size_t)(t0 + t) * HV + h;
            if constexpr (DEC) g = log_decay(p, th, h);
            bt = BETA ? update_rate(p, th) : 1.f;
            if (p.qk_l2_norm) {
                float ss = 0.f, sq = 0.f;
                for (int c = 0; c < D128; ++c) {
                    const float a = (float)sK[t][c], qv = (float)sQ[t][c];
                    ss = fmaf(a, a, ss);
                    sq = fmaf(qv, qv, sq);
                }
                ik = 1.f / sqrtf(ss + 1e-12f);
                iq = 1.f / sqrtf(sq + 1e-12f);
            }
        }
        sG[t] = g;
        sBeta[t] = bt;
        sIk[t] = ik;
        sIq[t] = iq;
    }
    lds_barrier();
    if (tid == 0) {
        float acc = 0.f;
        for (int t = 0; t < CH; ++t) {
            acc += sG[t];
            sG[t] = acc;  // inclusive cumulative log decay inside the chunk
        }
    }
    lds_barrier();
    if (tid < CH) sRw[tid] = sBeta[tid] * expf(sG[tid]) * sIk[tid];  // row scale of K in the W right-hand side

    // ---- Q K^T -> P (hi, lo) and K K^T -> A, tiles of 16 x 16 (wave = token block)
    const float scale = p.scale;
    {
        const int tb = wave;
        const int lr = lane & 15, lk = (lane >> 4) * 8;
        for (int sb = 0; sb < 4; ++sb) {
            f4v accq = {0.f, 0.f, 0.f, 0.f}, acck = {0.f, 0.f, 0.f, 0.f};
            if (sb <= tb) {
#pragma unroll
                for (int kk = 0; kk < D128; kk += 32) {
                    const h8 bk = ld_h8(&sK[16 * sb + lr][kk + lk]);
                    accq = mfma16(ld_h8(&sQ[16 * tb + lr][kk + lk]), bk, accq);
                    if constexpr (RET) acck = mfma16(ld_h8(&sK[16 * tb + lr][kk + lk]), bk, acck);
                }
            }
            const int s = 16 * sb + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + (lane >> 4) * 4 + i;
                const float dg = (s <= t) ? expf(sG[t] - sG[s]) : 0.f;
                const float pv = scale * sIq[t] * sIk[s] * dg * accq[i];
                const half_t hi = (half_t)pv;
                ws_p[(ch * 2 + 0) * CH * CH + t * CH + s] = hi;
                ws_p[(ch * 2 + 1) * CH * CH + t * CH + s] = (half_t)(pv - (float)hi);
                if constexpr (RET) sA[t][s] = (s < t) ? sBeta[t] * sIk[t] * sIk[s] * dg * acck[i] : 0.f;
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
            float r = wcol ? sRw[t] * (float)sK[t][cc] : sBeta[t] * (float)sV[t][cc];
#pragma unroll
            for (int s = 0; s < t; ++s) r = fmaf(-sA[t][s], x[s], r);
            x[t] = r;
        }
        if (wcol) {
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const half_t hi = (half_t)x[t];
                ws_w[(ch * 2 + 0) * CH * D128 + t * D128 + cc] = hi;
                ws_w[(ch * 2 + 1) * CH * D128 + t * D128 + cc] = (half_t)(x[t] - (float)hi);
            }
        } else {
#pragma unroll
            for (int t = 0; t < CH; ++t) ws_u[ch * CH * D128 + t * D128 + cc] = x[t];
        }
    } else {
        // no retrieval: D = V
        for (int idx = tid; idx < CH * D128; idx += 256) {
            const int t = idx / D128, c = idx % D128;
            ws_u[ch * CH * D128 + idx] = (float)sV[t][c];
        }
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
template <int RULE>
__global__ __launch_bounds__(256) void k_chunk_scan(const Params p, const int32_t *__restrict__ off,
                                                   const half_t *__restrict__ ws_w,
                                                   const half_t *__restrict__ ws_p,
                                                   const float *__restrict__ ws_u,
                                                   const float *__restrict__ ws_s,
                                                   const half_t *__restrict__ ws_kt)
{
    constexpr bool RET = rule_retrieves(RULE);
    constexpr int LS = D128 + 8;   // fp16 state row (272 B)
    constexpr int LDT = CH + 8;    // fp16 row of the transposed delta (144 B)

    // Operands are split into fp16 (hi, lo) once, by the lane that owns the
    // value, and stored as planes; every MFMA fragment is then one 16-byte
    // LDS read.  Row strides of 68 and 36 dwords put the 16 lanes of a
    // 16-byte access phase on 16 distinct 4-bank groups.
    __shared__ __align__(16) half_t sS[2][TR][LS];    // state tile, hi / lo
    __shared__ __align__(16) half_t sDt[4][TR][LDT];  // D^T hi / lo, (kd D)^T hi / lo
    __shared__ float sSc[256];

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

    const half_t *__restrict__ q = static_cast<const half_t *>(p.q);
    const half_t *__restrict__ k = static_cast<const half_t *>(p.k);
    half_t *__restrict__ o = static_cast<half_t *>(p.o);

    // state tile in accumulator layout: wave owns dv block (wave >> 1), dk blocks 4*(wave & 1) + j
    const int dvb = wave >> 1, dkb0 = 4 * (wave & 1);
    f4v Sacc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = row0 + 16 * dvb + 4 * lq + i, c = 16 * (dkb0 + j) + lr;
            Sacc[j][i] = src ? src[(size_t)r * D128 + c] : 0.f;
        }

    // Operands of one chunk, loaded one chunk ahead so their global-memory
    // latency hides behind the previous chunk's matrix work.  Rows past the
    // end of the request read as zero.
    const int tb = wave;          // token block of this wave in steps B and D
    const int tr = 16 * tb + lr;  // A-operand row (token) of this lane
    struct Ops {
        h8 kt[2][4];              // K^T fragments of the state update: token steps x dk tiles
        h8 wh[4], wl[4], aq[4];   // W (hi, lo) and Q rows, four k-steps of 32
        h8 ph[2], pl[2];          // P (hi, lo) rows, two k-steps of 32
        float u[2][4];            // U at this lane's D-layout positions
        float kd[4];              // kd of this lane's four D-layout tokens
        float sc;                 // one per-chunk scalar (threads < 129)
        int n;                    // valid tokens in the chunk
        int64_t t0;
    };
    // Every load below is unconditional (a branch around a load makes the
    // compiler wait for it on the spot, which would defeat the prefetch).
    auto fetch = [&](int jj, Ops &f) {
        const size_t ch = (size_t)(c0 + jj) * HV + h;
        f.t0 = rs + (int64_t)jj * CH;
        f.n = (int)((re - f.t0) < CH ? (re - f.t0) : CH);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                f.kt[ks][jj] = ld_h8(ws_kt + ch * D128 * CH + (size_t)(16 * (dkb0 + jj) + lr) * CH + 32 * ks + lk);
        f.sc = ws_s[ch * SC_STRIDE + (tid < 2 * CH ? tid : 2 * CH)];
        const half_t *wh = ws_w + (ch * 2 + 0) * CH * D128 + (size_t)tr * D128;
        const half_t *wl = ws_w + (ch * 2 + 1) * CH * D128 + (size_t)tr * D128;
        // rows past the request end read its last row; their outputs are never stored
        const int tq = tr < f.n ? tr : f.n - 1;
        const half_t *qp = q + ((size_t)(f.t0 + tq) * H + qh) * D128;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            f.aq[kk] = ld_h8(qp + 32 * kk + lk);
            if constexpr (RET) {
                f.wh[kk] = ld_h8(wh + 32 * kk + lk);
                f.wl[kk] = ld_h8(wl + 32 * kk + lk);
            }
        }
        const half_t *ph = ws_p + (ch * 2 + 0) * CH * CH + (size_t)tr * CH;
        const half_t *pl = ws_p + (ch * 2 + 1) * CH * CH + (size_t)tr * CH;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            f.ph[ks] = ld_h8(ph + 32 * ks + lk);
            f.pl[ks] = ld_h8(pl + 32 * ks + lk);
        }
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                f.u[vb][i] = ws_u[ch * CH * D128 + (size_t)(16 * tb + 4 * lq + i) * D128 + row0 + 16 * vb + lr];
#pragma unroll
        for (int i = 0; i < 4; ++i) f.kd[i] = ws_s[ch * SC_STRIDE + CH + 16 * tb + 4 * lq + i];
    };

    // one chunk: consumes `cur`, prefetches chunk j + 1 into `nxt`
    auto step = [&](int j, const Ops &cur, Ops &nxt) {
        const int64_t t0 = cur.t0;
        const int n = cur.n;
        lds_barrier();
        // ---- A: state tile -> LDS (hi, lo); scalars
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = Sacc[jj][i];
                const half_t hi = (half_t)x;
                sS[0][16 * dvb + 4 * lq + i][16 * (dkb0 + jj) + lr] = hi;
                sS[1][16 * dvb + 4 * lq + i][16 * (dkb0 + jj) + lr] = (half_t)(x - (float)hi);
            }
        sSc[tid] = cur.sc;  // entries past 2 * CH repeat gamma_C and are not read
        // next chunk's operands (the last chunk re-reads itself: every lane
        // issues the same loads on every iteration)
        fetch(j + 1 < nch ? j + 1 : j, nxt);
        lds_barrier();

        // ---- B: D = U - W S^T and Opre = Q S^T for token block tb, dv blocks 0, 1
        f4v accD[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f4v accO[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int vb = 0; vb < 2; ++vb) {
                const h8 shi = ld_h8(&sS[0][16 * vb + lr][32 * kk + lk]);
                const h8 slo = ld_h8(&sS[1][16 * vb + lr][32 * kk + lk]);
                if constexpr (RET) {
                    accD[vb] = mfma16(cur.wh[kk], shi, accD[vb]);
                    accD[vb] = mfma16(cur.wh[kk], slo, accD[vb]);
                    accD[vb] = mfma16(cur.wl[kk], shi, accD[vb]);
                }
                accO[vb] = mfma16(cur.aq[kk], shi, accO[vb]);
                accO[vb] = mfma16(cur.aq[kk], slo, accO[vb]);
            }
        }
        // D at (tokens 16 tb + 4 lq + i, state row 16 vb + lr): four consecutive
        // tokens per lane -> one 8-byte write per plane of D^T
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
            *reinterpret_cast<h4 *>(&sDt[0][r][c]) = dh;
            *reinterpret_cast<h4 *>(&sDt[1][r][c]) = dl;
            *reinterpret_cast<h4 *>(&sDt[2][r][c]) = sh;
            *reinterpret_cast<h4 *>(&sDt[3][r][c]) = sl;
        }
        lds_barrier();

        // ---- D: O = gq (Q S^T) + P D for token block tb, dv blocks 0, 1
        {
            f4v accP[2];
#pragma unroll
            for (int vb = 0; vb < 2; ++vb)
#pragma unroll
                for (int i = 0; i < 4; ++i) accP[vb][i] = sSc[16 * tb + 4 * lq + i] * accO[vb][i];
            // P is lower triangular; the block above the diagonal holds zeros
            // and is multiplied anyway so that every prefetched fragment is used
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int vb = 0; vb < 2; ++vb) {
                    const h8 dhi = ld_h8(&sDt[0][16 * vb + lr][32 * ks + lk]);
                    const h8 dlo = ld_h8(&sDt[1][16 * vb + lr][32 * ks + lk]);
                    accP[vb] = mfma16(cur.ph[ks], dhi, accP[vb]);
                    accP[vb] = mfma16(cur.ph[ks], dlo, accP[vb]);
                    accP[vb] = mfma16(cur.pl[ks], dhi, accP[vb]);
                }
            }
#pragma unroll
            for (int vb = 0; vb < 2; ++vb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tb + 4 * lq + i;
                    if (t < n) o[((size_t)(t0 + t) * HV + h) * D128 + row0 + 16 * vb + lr] = (half_t)accP[vb][i];
                }
        }

        // ---- E: S <- gamma_C S + (kd D)^T K for the wave's 4 state tiles
        {
            const float gC = sSc[2 * CH];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) Sacc[jj][i] *= gC;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const h8 dhi = ld_h8(&sDt[2][16 * dvb + lr][32 * ks + lk]);
                const h8 dlo = ld_h8(&sDt[3][16 * dvb + lr][32 * ks + lk]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    Sacc[jj] = mfma16(dhi, cur.kt[ks][jj], Sacc[jj]);
                    Sacc[jj] = mfma16(dlo, cur.kt[ks][jj], Sacc[jj]);
                }
            }
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
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = row0 + 16 * dvb + 4 * lq + i, c = 16 * (dkb0 + j) + lr;
            dst[(size_t)r * D128 + c] = Sacc[j][i];
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
        hipLaunchKernelGGL((k_chunk_scan<RULE>), dim3((unsigned)blocks), dim3(256), 0, s, p, off, ws_w, ws_p, ws_u,
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
