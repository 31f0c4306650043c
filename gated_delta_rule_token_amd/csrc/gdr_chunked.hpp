// gdr_chunked.hpp -- chunk-parallel prefill (chunk = 64 tokens) on MFMA.
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
//                  substitution (four lanes per column), the per-token
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

#include <type_traits>

#include "gdr_device.hpp"
#include "gdr_launch.hpp"

// Each translation unit that includes this file names its own namespace for
// the kernels (one unit per activation dtype, compiled in parallel), so the
// kernels of different units never share a symbol.
#ifndef GDR_CHUNK_NS
#error "define GDR_CHUNK_NS before including gdr_chunked.hpp"
#endif

namespace gdr {
namespace GDR_CHUNK_NS {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

// 8- and 4-element vectors of an activation dtype (16- and 8-byte loads)
template <typename TA> struct ActVec;
template <> struct ActVec<half_t> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    typedef _Float16 v4 __attribute__((ext_vector_type(4)));
};
template <> struct ActVec<bf16_t> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    typedef __bf16 v4 __attribute__((ext_vector_type(4)));
};
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u4v ld_b128_lds(const void *p) { return *reinterpret_cast<const u4v *>(p); }

constexpr int CH = 64;          // chunk length
constexpr int D128 = 128;       // dk = dv

// Workspace record of one (chunk, head).  Every operand of the scan is stored
// in MFMA fragment order: 1 KB blocks holding the 16 bytes lane l (= 16 lq + lr)
// of a wave loads at l * 16, so each wave-wide load reads 1 KB of consecutive
// bytes (eight whole cache lines).  Per-head decay (PK = false):
//   W   W (hi, lo) fp16, block (tb * 4 + kk) * 2 + plane: token 16 tb + lr, keys 32 kk + 8 lq .. +7
//   U   U fp32,          block tb * 8 + rt:              tokens 16 tb + 4 lq .. +3, row 16 rt + lr
//   P   P fp16,          block tb * 2 + ks:              token 16 tb + lr, tokens 32 ks + 8 lq .. +7
//       (P enters only the 16-bit outputs: one plane, rounded to nearest)
//   SC  fp32 scalars: kd[64], gq[64], gamma_C
// and, once per (chunk, q/k head) -- the same for every value head of the
// group, written by its first value head (struct KQ):
//   KT  K^T fp16,        block mt * 2 + ks:              key 16 mt + lr, tokens 32 ks + 8 lq .. +7
// (the scan's output waves read the q rows from the activations themselves:
// a row of 8 keys per lane is already their fragment layout)
// Decay per key channel (PK = true): the per-token weights kd and gq become
// per-element factors, so two operands carry fp32 values:
//   KT  Kd^T (hi, lo),   block (mt * 2 + ks) * 2 + plane,  Kd = kn o exp(G_C - G)
//   Q   Qg fp16,         block tb * 4 + kk,                Qg = scale qn o exp(G)
//   SC  fp32 gamma_C of each of the 128 key channels
// Kd^T enters the state update and keeps (hi, lo) planes; Qg enters only the
// outputs, which are stored in 16 bits, so one fp16 plane (round to nearest,
// 2^-11 relative) adds an error of the order of that store's own rounding.
template <bool PK>
struct Rec {
    static constexpr uint32_t W = 0;
    static constexpr uint32_t KT = W + 32 * 1024;
    static constexpr uint32_t U = KT + (PK ? 32 : 0) * 1024;
    static constexpr uint32_t Q = U + 32 * 1024;
    static constexpr uint32_t P = Q + (PK ? 16 : 0) * 1024;
    static constexpr uint32_t SC = P + 8 * 1024;
    static constexpr uint32_t SIZE = SC + 1024;
};
constexpr uint32_t R_W = Rec<false>::W, R_U = Rec<false>::U, R_P = Rec<false>::P, R_SC = Rec<false>::SC,
                   WS_REC = Rec<false>::SIZE;

// Record of one (chunk, value head) in the T form (per-head decay, fp16
// activations): the scan forms W S^T and U itself as T (beta V - w K S^T)
// from the raw k and v rows, and P from the raw q and k rows, so the record
// holds only what needs the whole chunk at once:
//   T   T = (I + A)^-1 (hi, lo) fp16, block (tb * 2 + ks) * 2 + plane: token 16 tb + lr,
//       tokens 32 ks + 8 lq .. +7 (blocks tb < 2, ks = 1 lie above the diagonal: not stored)
//   SC  fp32: kd[64], gq[64], gamma_C, max |v| at SC_VMAX, beta[64] at SCT_BETA,
//       w[64] at SCT_RW (w = beta gamma / |k|, the row weight of K in W), and
//       P's per-token factors: G[64] at SCT_G (cumulative log decay in log2
//       units) with its rounding error at SCT_GL, 1 / |k| [64] at SCT_IK,
//       scale / |q| [64] at SCT_QS
// (the state update's left operand K^T the scan gathers from the k rows it
// parks in LDS).
struct RecT {
    static constexpr uint32_t T = 0;
    static constexpr uint32_t SC = 16 * 1024;
    static constexpr uint32_t SIZE = SC + 2560;
};
constexpr int SCT_BETA = 256, SCT_RW = 320, SCT_G = 384, SCT_IK = 448, SCT_QS = 512, SCT_GL = 576;
struct KQ {
    static constexpr uint32_t KT = 0, SIZE = 16 * 1024;
};

__device__ __forceinline__ f4v mfma16(h8 a, h8 b, f4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr double LOG2E_D = 1.4426950408889634;

// 2^x on the transcendental unit (one instruction; results below the normal
// range flush toward zero, which only ever drops terms smaller than 1e-38)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> (hi, lo) fp16 pairs with hi + lo ~ x to about 22 bits: hi = fp16(x)
// (nearest), lo = fp16(x - hi), where x - hi is exact in fp32.  Two values at
// a time, in three instructions: one packed conversion gives both hi, then
// v_fma_mix{lo,hi}_f16 forms each lo from its hi half and x.  The three are
// one asm block that takes x as fp32 registers: left to itself, contraction
// fuses the product or sum that feeds a split into the conversion of one part
// and not of the other, and within half an fp32 unit of an fp16 rounding
// midpoint the two parts then disagree by a unit in the last fp16 place
// (measured: one state entry in error by 5e-4 of itself).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    asm("v_cvt_pk_f16_f32 %0, %2, %3\n\t"
        "v_fma_mixlo_f16 %1, %0, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %1, %0, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(hi), "=&v"(lo)
        : "v"(x0), "v"(x1));
}
__device__ __forceinline__ void split8(const float (&x)[8], h8 &hi, h8 &lo)
{
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(x[2 * i], x[2 * i + 1], h[i], l[i]);
    hi = __builtin_bit_cast(h8, u4v{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(h8, u4v{l[0], l[1], l[2], l[3]});
}

__device__ __forceinline__ h8 ld_h8(const half_t *p) { return *reinterpret_cast<const h8 *>(p); }

// Eight 16-bit activations as fp16.  bf16 values convert exactly when they
// lie in fp16's range with no more than its precision (every bf16 value of
// magnitude 2^-17 to 65504); `exact` is cleared for any other (and for NaN).
__device__ __forceinline__ h8 to_h8(h8 x, bool &) { return x; }
__device__ __forceinline__ h8 to_h8(ActVec<bf16_t>::v8 x, bool &exact)
{
    h8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float f = (float)x[e];
        r[e] = (half_t)f;
        exact = exact && (float)r[e] == f;
    }
    return r;
}
template <typename TI>
__device__ __forceinline__ h8 ld_as_h8(const TI *p, bool &exact)
{
    return to_h8(*reinterpret_cast<const typename ActVec<TI>::v8 *>(p), exact);
}

// 16x16x32 matrix product of 16-bit activations with fp32 accumulation (the
// products of two fp16 or two bf16 values are exact in fp32)
__device__ __forceinline__ f4v mfma16x32(ActVec<half_t>::v8 a, ActVec<half_t>::v8 b, f4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4v mfma16x32(ActVec<bf16_t>::v8 a, ActVec<bf16_t>::v8 b, f4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer resource over one workspace record of `bytes` bytes (an offset
// past it reads zero instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *rec, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(rec), 0, (int)bytes, 0x00020000);
}

template <typename T>
__device__ __forceinline__ T ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// four fp32 -> (hi, lo) fp16 quads
__device__ __forceinline__ void split4(f4v x, h4 &hi, h4 &lo)
{
    uint32_t h0, h1, l0, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    hi = __builtin_bit_cast(h4, u2v{h0, h1});
    lo = __builtin_bit_cast(h4, u2v{l0, l1});
}

// One fp16 plane: each value rounded to nearest (the hi part of a split),
// for operands that enter only the 16-bit outputs.
__device__ __forceinline__ h4 round_h4(f4v x) { return __builtin_convertvector(x, h4); }
__device__ __forceinline__ h8 round_h8(const float (&x)[8])
{
    return h8{(half_t)x[0], (half_t)x[1], (half_t)x[2], (half_t)x[3], (half_t)x[4], (half_t)x[5], (half_t)x[6], (half_t)x[7]};
}

// Column index of a swizzled LDS row of fp16: the 16-byte chunk (8 values)
// holding column x moves to chunk (x / 8) XOR f(row), with f(row) = row mod 16
// for 128-column rows and (row / 2) mod 8 for 64-column rows.  With it, the
// matrix-core operand reads (16 bytes per lane, 16 rows x 4 chunks per wave)
// are free of bank conflicts on gfx950, whose ds_read_b128 serves lanes 0-7
// together with 24-31 (and 8-15 with 16-23), as a counter probe showed;
// padded row strides leave a 2-way conflict there.  Only the row's low four
// bits enter, so rows 16 apart share one pattern.
__device__ __forceinline__ int sw_key(int row, int key) { return (((key >> 3) ^ (row & 15)) << 3) | (key & 7); }
__device__ __forceinline__ int sw_tok(int row, int tok) { return (((tok >> 3) ^ ((row >> 1) & 7)) << 3) | (tok & 7); }

// Magnitude of the split operands.  The recurrence is linear in (initial
// state, v) for fixed keys, gates and update rates, so the scan may run a
// state tile multiplied by 2^e and divide o and the final state by 2^e: a
// power of two changes no digit.  e brings the larger of max |v| of the
// (request, head) and max |S0| of the tile into [4, 8), where the fp16
// (hi, lo) pairs of the state and the value updates keep ~22 bits: about
// 2^13 of headroom above it for state growth, and entries far below it keep
// an absolute error near 2^-25 of that maximum instead of turning into fp16
// subnormals (inputs of size 1e-5 lost most of their digits unscaled).  Each
// scan unit takes max |v| over its own chunks (post_vmax) and max |S0| over
// its own tile, so units need not agree.
// Magnitude past which an fp32 operand is not split into fp16 (hi, lo): the
// hi part would round to infinity at 65520; the margin keeps the sums of the
// products that follow finite as well.
constexpr float SPLIT_LIMIT = 60000.f;

// Largest magnitude, as the bits of |x| (so that inf and NaN rank above every
// finite value), of the fp32 values one thread splits into fp16 (hi, lo).
struct SplitWatch {
    uint32_t big = 0u;
    __device__ __forceinline__ void note(float x) { big = max(big, __float_as_uint(x) & 0x7FFFFFFFu); }
    __device__ __forceinline__ void note(f4v x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) note(x[i]);
    }
    __device__ __forceinline__ void note(const float (&x)[8])
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) note(x[i]);
    }
    __device__ __forceinline__ bool over() const { return big >= __float_as_uint(SPLIT_LIMIT); }
};

// The scans' watch: a float maximum of |x| (v_max3_f32 with absolute-value
// operands, half an instruction per value against one and a half for the
// bits).  It does not see a NaN, and needs not: the prologues hand every
// pair whose inputs hold one to the recurrent kernel (post_vmax and their
// own watches), and a NaN that arises in the scan needs an infinite or
// out-of-range operand first, which it sees.
struct ScanWatch {
    float big = 0.f;
    __device__ __forceinline__ void note(f4v x)
    {
        big = fmaxf(fmaxf(big, fabsf(x[0])), fabsf(x[1]));
        big = fmaxf(fmaxf(big, fabsf(x[2])), fabsf(x[3]));
    }
    __device__ __forceinline__ bool over() const { return !(big < SPLIT_LIMIT); }
};

// The caller of solve_blocked stores A with each row permuted, entry s at
// a_pos(s) = 16 (s mod 4) + s / 4, so that the diagonal blocks' forward
// substitution reads its terms as 16-byte vectors; it must store the
// diagonal 16 x 16 blocks in full (zeros on and above the diagonal).
__device__ __forceinline__ int a_pos(int s) { return 16 * (s & 3) + (s >> 2); }

// T = (I + A)^-1 of a chunk's strictly lower triangular 64 x 64 matrix A
// (rows of LA floats), by blocks of 16 (row block i, column block j), on the
// four waves of a 256-thread workgroup.  Wave i inverts its unit lower
// diagonal block I + A_ii by forward substitution down its 16 rows,
//   T_tc = [t == c] - sum_{s<t} A_ts T_sc,
// four lanes per column (lane q of column c the terms s = q (mod 4), a quad
// reduction completing the row), then the blocks below the diagonal follow
// by their distance d = i - j from it, one level per barrier,
//   T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj,
// on the fp32 matrix cores (16x16x4: fp32 products and sums; lane (g, r) of
// an operand holds row r, k-index g of the left one and k-index g, column r
// of the right one, and result rows 4 g .. 4 g + 3 of column r).  A is read
// as the caller stores it (row t, column s at a_pos(s); only s < t is read);
// wave i keeps its row block's A blocks in registers before it writes T over
// them, and reads other row blocks only as T.  T ends up over A in natural
// order with zeros above the diagonal, without a trailing barrier.  wgt[c] is
// column c's weight: each lane watches its T entries and the entries times
// their column's weight, the products the caller forms from them.
template <int LA>
__device__ __forceinline__ void solve_blocked(float (*sA)[LA], int tid, const float *wgt, SplitWatch &wt)
{
    const int i = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // (a scalar: branches on i stay scalar)
    const int r16 = lane & 15, g4 = lane >> 4;  // operand lane (row / column r16, k-index g4)
    const int c = lane >> 2, q = lane & 3;      // forward substitution: column c, terms s = q (mod 4)
    // this row block's A_ik (k < i) in the left-operand layout
    float ab[3][4];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ab[k][ks] = k < i ? sA[16 * i + r16][a_pos(16 * k + 4 * ks + g4)] : 0.f;
    // T_ii: x[m] = T_ii[4 m + q][c]; row t's terms A_ii[t][4 m + q] lie at a_pos = 16 q + 4 i + m
    float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const f4v a = *reinterpret_cast<const f4v *>(&sA[16 * i + t][16 * q + 4 * i]);
        float r = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) r = fmaf(a[m], x[m], r);  // zero past the diagonal (A) or not yet formed (x)
        r += dpp_mov<0xB1>(r);  // the quad's four partial sums
        r += dpp_mov<0x4E>(r);
        const float xt = (t == c ? 1.f : 0.f) - r;
        if ((t & 3) == q) x[t >> 2] = xt;
    }
    const float wd = wgt[16 * i + c];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        wt.note(x[m]);
        wt.note(x[m] * wd);
        sA[16 * i + 4 * m + q][16 * i + c] = x[m];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j > i) sA[16 * i + 4 * m + q][16 * j + c] = 0.f;
    }
    lds_barrier();  // every T_ii is in place
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (i >= d) {
            const int j = i - d;
            f4v acc = {0.f, 0.f, 0.f, 0.f};
            // X = sum_k A_ik T_kj
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (k >= j && k < i) {  // (static k: the register array is not indexed at run time)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ab[k][ks], sA[16 * k + 4 * ks + g4][16 * j + r16], acc, 0, 0, 0);
                }
            }
            // X through block (i, j), then T_ij = -T_ii X there
#pragma unroll
            for (int r = 0; r < 4; ++r) sA[16 * i + 4 * g4 + r][16 * j + r16] = acc[r];
            f4v tij = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                tij = __builtin_amdgcn_mfma_f32_16x16x4f32(-sA[16 * i + r16][16 * i + 4 * ks + g4],
                                                           sA[16 * i + 4 * ks + g4][16 * j + r16], tij, 0, 0, 0);
            const float wj = wgt[16 * j + r16];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                wt.note(tij[r]);
                wt.note(tij[r] * wj);
                sA[16 * i + 4 * g4 + r][16 * j + r16] = tij[r];
            }
        }
        if (d < 3) lds_barrier();  // level d is in place
    }
}

__device__ __forceinline__ int tile_exponent(float m)
{
    if (!(m > 0.f) || !(m <= 3.0e38f)) return 0;  // zero, or not finite
    int e;
    frexpf(m, &e);  // m in [2^(e-1), 2^e)
    const int x = 3 - e;
    return x < -100 ? -100 : (x > 100 ? 100 : x);
}

// Largest |v| of a prologue wave's chunk rows (4 vectors of 8 per thread),
// stored as one float per wave at SC[252 + wave] of the chunk record, where
// the scan reads it back.  Returns false when the wave's rows hold an
// infinite value or a NaN: the caller then hands the pair to the recurrent
// kernel (in the chunk products a NaN would reach earlier tokens through the
// zero entries of T above the diagonal).
constexpr int SC_VMAX = 252;
template <typename V8>
__device__ __forceinline__ bool post_vmax(const V8 (&x)[4], char *rec_sc)
{
    uint32_t m = 0u;  // bits of |v|: NaN ranks above every finite value
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = max(m, __float_as_uint(to_f32(x[i][e])) & 0x7FFFFFFFu);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0) reinterpret_cast<float *>(rec_sc)[SC_VMAX + (threadIdx.x >> 6)] = __uint_as_float(m);
    return m < 0x7F800000u;
}

// Segments of the scan's chain (see k_chunk_scan).  pass 0: one pass over
// every chunk; pass 1 / 2: the two passes of an nseg-segment scan.  xs holds,
// per (request, head), seg_slots(nseg) states of 128 x 128 fp32: the start of
// segment p (1 <= p < nseg), and the carry and transition of middle segment p
// (1 <= p < nseg - 1).
struct ScanSeg {
    int nseg;
    int pass;
    float *xs;
    float *stage;  // in-place state (slab, or final == initial): final states go here first, else nullptr
};
enum SegMode : int { SEG_REAL = 0, SEG_CARRY = 1, SEG_TRANS = 2 };

// Value heads of one q/k head that a single-pass scan places on one XCD
// (consecutive groups), so that the k, q and K^T rows they share are fetched
// into its L2 once: the largest power of two up to 8 dividing HV / H (1
// without grouped heads, and for the passes of a segmented scan).
__host__ __device__ inline int xcd_heads(int H, int HV, int pass)
{
    if (pass != 0 || H <= 0 || HV % H != 0) return 1;
    const int r = HV / H;
    int g = 1;
    while (g < 8 && r % (2 * g) == 0) g *= 2;
    return g;
}
__host__ __device__ constexpr int seg_slots(int nseg) { return 3 * nseg; }
__host__ __device__ constexpr int seg_start(int p) { return p; }
// First chunk of segment p (0 <= p <= ns) of a request's nch chunks.  Segment
// 0 runs for real in pass 1 beside carry and transition tiles, which form no
// outputs and take ~7/8 of its time per chunk step (measured on MI355X), so
// it gets 7/8 of the others' share: every tile of pass 1 then ends about
// together.
__host__ __device__ inline int seg_lo(int p, int nch, int ns)
{
    if (p <= 0) return 0;
    if (p >= ns) return nch;
    return (int)(((int64_t)nch * (8 * p - 1)) / (8 * ns - 1));
}
__host__ __device__ constexpr int seg_carry(int nseg, int p) { return nseg + p; }
__host__ __device__ constexpr int seg_trans(int nseg, int p) { return 2 * nseg + p; }

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

// Chunk and value head of a prologue workgroup.  Blocks x and x + 8 run on
// the same XCD (workgroups go round-robin over the 8 XCDs), so they take
// heads h and h + 1 of one chunk: value heads that share a q/k head read its
// rows once into that XCD's L2 instead of once per head from HBM (measured on
// the varlen workload: 0.75 -> 0.47 GB read by the prologue).
__device__ __forceinline__ void prep_block(int HV, int64_t &ci, int &h)
{
    const int64_t x = blockIdx.x, rest = x >> 3;
    h = (int)(rest % HV);
    ci = (rest / HV) * 8 + (x & 7);
}

// ------------------------------------------------------------------ table
// Chunk plan of gdr_chunk_plan.hpp: off[b] = first chunk of request b (B + 1
// entries, off[B] <= budget), and redo[b * HV + h] = 1 for the pairs of the
// requests that get no chunks although they have tokens (ranges that overlap
// after a decreasing cu_seqlens entry); the recurrent kernel takes those.
// Prefix sums are 64-bit: overlapping ranges can sum to B * ceil(T / 64).
constexpr int ORDER_MAX = 1024;
__global__ __launch_bounds__(256) void k_chunk_table(const Params p, int32_t *off, int32_t *redo)
{
    __shared__ int64_t s[256];
    __shared__ int32_t s_cnt[ORDER_MAX];
    __shared__ int64_t carry;
    __shared__ unsigned long long best;  // largest granted inclusive prefix
    const int tid = threadIdx.x;
    const int64_t budget = chunk_budget(p.T, p.B);
    if (tid == 0) {
        carry = 0;
        best = 0;
    }
    __syncthreads();
    for (int base = 0; base < p.B; base += 256) {
        const int b = base + tid;
        int64_t n = 0;
        if (b < p.B) {
            int64_t st, en;
            request_range(p, b, st, en);
            n = request_chunks(st, en);
        }
        s[tid] = n;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int64_t v = tid >= o ? s[tid - o] : 0;
            __syncthreads();
            s[tid] += v;
            __syncthreads();
        }
        if (b < p.B) {
            const int64_t excl = carry + s[tid] - n;
            // provisional entry (capped so it fits 32 bits); the second pass caps it at best
            off[b] = (int32_t)(excl < budget + 1 ? excl : budget + 1);
            const int32_t denied = chunk_denied(excl, n, budget) ? 1 : 0;
            for (int h = 0; h < p.HV; ++h) redo[(size_t)b * p.HV + h] = denied;
            if (chunk_granted(excl, n, budget)) atomicMax(&best, (unsigned long long)(excl + n));
        }
        __syncthreads();
        if (tid == 255) carry += s[255];
        __syncthreads();
    }
    const int64_t top = (int64_t)best;
    for (int b = tid; b < p.B; b += 256) off[b] = chunk_offset(off[b], top);
    if (tid == 0) off[p.B] = chunk_offset(carry, top);
    __syncthreads();
    // The scans take the requests longest first (order[i] = the request of
    // rank i by granted chunks, ties by index): with one workgroup per CU a
    // long request placed late in the batch would start only when an early
    // one ends and finish last.  Rank by counting, up to ORDER_MAX requests;
    // past that, batch order.
    int32_t *order = redo + (size_t)p.B * p.HV;
    if (p.B <= ORDER_MAX) {
        for (int b = tid; b < p.B; b += 256) s_cnt[b] = off[b + 1] - off[b];
        __syncthreads();
        for (int b = tid; b < p.B; b += 256) {
            const int c = s_cnt[b];
            int rank = 0;
            for (int x = 0; x < p.B; ++x) {
                const int cx = s_cnt[x];
                rank += (cx > c || (cx == c && x < b)) ? 1 : 0;
            }
            order[rank] = b;
        }
    } else {
        for (int b = tid; b < p.B; b += 256) order[b] = b;
    }
}

// ------------------------------------------------------------------ phase 1
// 256 threads.  LDS: K, V and Q rows of the chunk; A (fp32) replaces Q once
// K Q^T and K K^T are formed; after the solve W (hi, lo) rows replace K and V.
// TF: the T form (RecT: T and the scalars; no W, U, P or q), else Rec<false>
// plus the K^T area.
// TI: the activations' dtype (bf16 rows are converted to fp16 as they load;
// a pair with a value fp16 cannot hold exactly goes to the recurrent kernel).
template <typename TI, int RULE, bool TF>
__global__ __launch_bounds__(256, TF ? 4 : 3) void k_chunk_prep(const Params p, int32_t *__restrict__ off,
                                                              char *__restrict__ ws, char *__restrict__ kqs)
{
    constexpr bool DEC = rule_decays(RULE);
    constexpr bool RET = rule_retrieves(RULE);
    constexpr bool BETA = rule_has_beta(RULE);
    constexpr int LD = D128 + 8;  // padded fp16 row (bank spread)
    constexpr int LA = CH + 4;    // 16-byte rows: the solve reads A rows as float4 broadcasts
    constexpr int SLOT = CH * LD * 2;
    static_assert(CH * LA * 4 == SLOT, "Q rows and A rows share one LDS footprint");

    // the T form keeps no V rows: K and Q (then A) only, so four workgroups fit a CU
    __shared__ __align__(16) char sm[(TF ? 2 : 3) * SLOT];
    half_t(*sK)[LD] = reinterpret_cast<half_t(*)[LD]>(sm);
    half_t(*sV)[LD] = reinterpret_cast<half_t(*)[LD]>(sm + SLOT);
    half_t(*sQ)[LD] = reinterpret_cast<half_t(*)[LD]>(sm + (TF ? 1 : 2) * SLOT);
    float(*sA)[LA] = reinterpret_cast<float(*)[LA]>(sm + (TF ? 1 : 2) * SLOT);
    half_t(*sW)[CH][D128] = reinterpret_cast<half_t(*)[CH][D128]>(sm);  // [hi, lo][token][key, swizzled], after the solve
    // G_t = sG + sGl (the cumulative log decay and its fp32 rounding error).
    // LDS per workgroup: 53,760 bytes at most for three workgroups per CU
    // (measured on MI355X: 512 bytes more cost the W/U form's prologue 18 %).
    __shared__ float sG[CH], sGl[CH], sBeta[CH], sIk[CH], sIq[CH], sRw[CH];

    const int HV = p.HV, H = p.H;
    int64_t ci;
    int h;
    prep_block(HV, ci, h);
    if (ci >= off[p.B]) return;
    const int b = chunk_request(off, p.B, ci);
    int64_t rs, re;
    request_range(p, b, rs, re);
    const int64_t t0 = rs + (ci - off[b]) * CH;
    const int n = (int)((re - t0) < CH ? (re - t0) : CH);
    const int qh = (int)(((int64_t)h * H) / HV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4, lk = lq * 8;
    constexpr uint32_t OSC = TF ? RecT::SC : R_SC;
    char *rec = ws + ((size_t)ci * HV + h) * (TF ? RecT::SIZE : WS_REC);
    // K^T once per (chunk, q/k head): the group's first value head writes it
    // (W/U form only; the T form's scan gathers it from the k rows itself)
    char *kq = TF ? nullptr : kqs + ((size_t)ci * H + qh) * KQ::SIZE;
    const bool kq_writer = !TF && h % (HV / H) == 0;
    // A split operand past the fp16 range hands the pair to the recurrent
    // kernel.  Each phase watches its own operands and posts at its end, so no
    // register stays live across the phases.
    int32_t *const flag = off + p.B + 1 + (size_t)b * HV + h;
    auto post = [&](const SplitWatch &w) {
        if (w.over()) *flag = 2;
    };

    const TI *__restrict__ q = static_cast<const TI *>(p.q);
    const TI *__restrict__ k = static_cast<const TI *>(p.k);
    const TI *__restrict__ v = static_cast<const TI *>(p.v);

    // ---- chunk rows of K, Q (head qh) and V (head h): issue the loads first,
    // compute the gates while they are in flight, then park them in LDS
    h8 ldk[4], ldq[4], ldv[4];
    bool exact = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
        ldk[i] = ldq[i] = ldv[i] = h8{};
        if (r < n) {
            const size_t tq = ((size_t)(t0 + r) * H + qh) * D128 + c8;
            ldk[i] = ld_as_h8(k + tq, exact);
            ldq[i] = ld_as_h8(q + tq, exact);
            ldv[i] = ld_as_h8(v + ((size_t)(t0 + r) * HV + h) * D128 + c8, exact);
        }
    }
    // ---- per-token log decay (cumulated over the chunk by a 64-lane scan) and
    // update rate.  The sums run in fp64: in a strongly decaying chunk two
    // prefix sums of hundreds of nats differ by a few late in the chunk, and
    // their fp32 roundings alone would put relative errors of 1e-5 .. 1e-4
    // into the decay factors between them (kd, A, P).  G_t is kept in log2
    // units (scaled in fp64) as fp32 (hi, lo), so that (hi_t - hi_s) +
    // (lo_t - lo_s) -- the first difference exact whenever it is small against
    // the sums -- recovers G_t - G_s, and every factor is one v_exp_f32.
    float gend = 0.f;  // G_end - G_t (log2 units) of this thread's token t = tid < CH (kd below)
    if (tid < CH) {
        const int t = tid;
        float gt = 0.f, bt = 0.f;
        if (t < n) {
            const size_t th = (size_t)(t0 + t) * HV + h;
            if constexpr (DEC) gt = log_decay(p, th, h);
            bt = BETA ? update_rate(p, th) : 1.f;
        }
        double g = gt;
#pragma unroll
        for (int o = 1; o < CH; o <<= 1) {
            const double y = __shfl_up(g, o, CH);
            if (t >= o) g += y;
        }
        g *= LOG2E_D;
        const double ge = __shfl(g, n - 1, CH);
        const float gh = (float)g;
        sG[t] = gh;  // inclusive cumulative log2 decay inside the chunk
        sGl[t] = (float)(g - (double)gh);
        gend = (float)(ge - g);
        sBeta[t] = bt;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
        *reinterpret_cast<h8 *>(&sK[r][c8]) = ldk[i];
        *reinterpret_cast<h8 *>(&sQ[r][c8]) = ldq[i];
        if constexpr (!TF) *reinterpret_cast<h8 *>(&sV[r][c8]) = ldv[i];
    }
    if (!post_vmax(ldv, rec + OSC)) *flag = 2;
    if (!exact) *flag = 2;  // a bf16 value fp16 cannot hold: the recurrent kernel takes the pair
    lds_barrier();

    // ---- K^T fragments (key 16 mt + lr, tokens 32 ks + 8 lq .. +7); fragment f = block * 64 + lane
#pragma unroll
    for (int g = 0; g < (kq_writer ? 4 : 0); ++g) {
        const int f = tid + 256 * g, blk = f >> 6, fl = f & 63;
        const int key = 16 * (blk >> 1) + (fl & 15), tk = 32 * (blk & 1) + 8 * (fl >> 4);
        h8 col;
#pragma unroll
        for (int x = 0; x < 8; ++x) col[x] = sK[tk + x][key];
        *reinterpret_cast<h8 *>(kq + KQ::KT + (size_t)f * 16) = col;
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
        sRw[t] = sBeta[t] * ex2(sG[t]) * sIk[t];  // row scale of K in W's right-hand side
        float *sc = reinterpret_cast<float *>(rec + OSC);
        sc[t] = t < n ? ex2(gend) * sIk[t] : 0.f;  // kd: key weight of token t in the state update
        sc[CH + t] = scale * sIq[t] * ex2(sG[t]);        // gq: read-out weight of the incoming state
        if (t == 0) sc[2 * CH] = DEC ? ex2(gl) : 1.f;    // gamma_C
        if constexpr (TF) {
            sc[SCT_BETA + t] = sBeta[t];  // zero past the request's end, like w
            sc[SCT_RW + t] = sRw[t];
            const double g2 = (double)sG[t] + (double)sGl[t];
            sc[SCT_G + t] = (float)g2;
            sc[SCT_GL + t] = (float)(g2 - (double)(float)g2);
            sc[SCT_IK + t] = sIk[t];
            sc[SCT_QS + t] = scale * sIq[t];
        }
    }

    // ---- K Q^T (not in the T form: its scan forms P) and K K^T, 16 x 16 tiles
    // (wave = token block tb, tiles sb <= tb); the accumulators hold
    // [s = 16 sb + 4 lq + i][t = 16 tb + lr]
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
                    if constexpr (!TF) accq[sb] = mfma16(ak, ld_h8(&sQ[16 * tb + lr][kk + lk]), accq[sb]);
                    if constexpr (RET) acck[sb] = mfma16(ak, ld_h8(&sK[16 * tb + lr][kk + lk]), acck[sb]);
                }
            }
        }
        lds_barrier();  // Q is dead: A takes its rows
        const int t = 16 * tb + lr;
        SplitWatch wp;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const int s0 = 16 * sb + 4 * lq;
            f4v pv, av;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = s0 + i;
                const float e2 = ex2((sG[t] - sG[s]) + (sGl[t] - sGl[s]));  // (select, not branch, past the diagonal)
                const float dg = s <= t ? e2 : 0.f;
                pv[i] = scale * sIq[t] * sIk[s] * dg * accq[sb][i];
                av[i] = (s < t) ? sBeta[t] * sIk[t] * sIk[s] * dg * acck[sb][i] : 0.f;
            }
            // P rows in fragment order: block (tb * 2 + s0 / 32) * 2 + plane; the
            // fragments of token blocks 0, 1 against tokens 32 .. 63 are all zero
            // and are not stored (the scan reads zero past the record instead)
            if (!TF && (tb >= 2 || sb < 2)) {
                wp.note(pv);
                const uint32_t po = R_P + ((uint32_t)(tb * 2 + (s0 >> 5)) * 64 + ((s0 & 31) >> 3) * 16 + lr) * 16 + ((s0 & 7) >> 2) * 8;
                *reinterpret_cast<h4 *>(rec + po) = round_h4(pv);  // P enters only the outputs
            }
            if constexpr (RET) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sA[t][a_pos(s0 + i)] = av[i];
            }
        }
        post(wp);
    }
    lds_barrier();

    if constexpr (!RET) {
        // no retrieval: U = V, stored in fragment order by the row-column threads
        // (the T form reads v itself)
        const int col = tid & (D128 - 1);
        if (!TF && tid >= D128) {
#pragma unroll
            for (int qd = 0; qd < CH / 4; ++qd) {
                f4v u;
#pragma unroll
                for (int i = 0; i < 4; ++i) u[i] = (float)sV[4 * qd + i][col];
                *reinterpret_cast<f4v *>(rec + R_U + ((uint32_t)(((qd >> 2) * 8 + (col >> 4)) * 64 + (qd & 3) * 16 + (col & 15))) * 16) = u;
            }
        }
        return;
    } else {
        // ---- [W | U] = T [diag(beta gamma / |k|) K | diag(beta) V],  T = (I + A)^-1,
        // on all four waves.  The column times its weight (split beside T below)
        // peaks where |T| does: rounding is monotone (the T form watches T as it
        // exports it).
        {
            SplitWatch wt;
            solve_blocked(sA, tid, sBeta, wt);
            if constexpr (!TF) post(wt);
        }
        lds_barrier();  // T is complete
        if constexpr (TF) {
            // T fragments (hi, lo) in the order the scan's chain waves load them:
            // blocks (tb, ks) on or below the diagonal, 64 fragments of 8 tokens each
            SplitWatch wtf;
            for (int it = tid; it < 6 * 64; it += 256) {
                const int blk = it >> 6, fl = it & 63;
                // (tb, ks) = (0, 0) (1, 0) (2, 0) (2, 1) (3, 0) (3, 1)
                const int tb = blk < 2 ? blk : 2 + ((blk - 2) >> 1), ks = blk < 2 ? 0 : (blk - 2) & 1;
                const int t = 16 * tb + (fl & 15), s0 = 32 * ks + 8 * (fl >> 4);
                const f4v a0 = *reinterpret_cast<const f4v *>(&sA[t][s0]);
                const f4v a1 = *reinterpret_cast<const f4v *>(&sA[t][s0 + 4]);
                float x8[8];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    x8[x] = a0[x];
                    x8[4 + x] = a1[x];
                }
                wtf.note(x8);
                h8 hi, lo;
                split8(x8, hi, lo);
                char *dst = rec + RecT::T + (uint32_t)((tb * 2 + ks) * 2) * 1024 + (uint32_t)fl * 16;
                *reinterpret_cast<h8 *>(dst) = hi;
                *reinterpret_cast<h8 *>(dst + 1024) = lo;
            }
            post(wtf);
            return;
        }
        // Wave w forms key columns and value rows 32 w .. 32 w + 31 on the matrix
        // cores.  Right-hand-side fragments hold 8 consecutive tokens of one key
        // or value column; W's right-hand side is fp32 and gets (hi, lo) fp16
        // planes, V is exact in fp16.
        h8 bwh[2][2], bwl[2][2], bv[2][2];  // [column block c][token step ks]
        SplitWatch wx, wa;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int cc = 16 * (2 * wave + c) + lr, s0 = 32 * ks + lk;
                float xw[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    xw[x] = sRw[s0 + x] * (float)sK[s0 + x][cc];
                    bv[c][ks][x] = sV[s0 + x][cc];
                }
                wx.note(xw);
                split8(xw, bwh[c][ks], bwl[c][ks]);
            }
        post(wx);
        f4v accW[4][2], accU[4][2];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
            for (int c = 0; c < 2; ++c) accW[mb][c] = accU[mb][c] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < (mb < 2 ? 1 : 2); ++ks) {
                // T rows 16 mb + lr, columns 32 ks + 8 lq .. +7 (zero above the diagonal)
                const int t = 16 * mb + lr, s0 = 32 * ks + lk;
                const f4v t0v = *reinterpret_cast<const f4v *>(&sA[t][s0]);
                const f4v t1v = *reinterpret_cast<const f4v *>(&sA[t][s0 + 4]);
                float tv[8], tb8[8];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    tv[x] = t0v[x];
                    tv[4 + x] = t1v[x];
                }
#pragma unroll
                for (int x = 0; x < 8; ++x) tb8[x] = tv[x] * sBeta[s0 + x];
                h8 th, tl, uh, ul;
                split8(tv, th, tl);
                split8(tb8, uh, ul);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    // W^T = RHS^T T^T: each lane ends with four consecutive keys of one token
                    accW[mb][c] = mfma16(bwh[c][ks], th, accW[mb][c]);
                    accW[mb][c] = mfma16(bwl[c][ks], th, accW[mb][c]);
                    accW[mb][c] = mfma16(bwh[c][ks], tl, accW[mb][c]);
                    accU[mb][c] = mfma16(uh, bv[c][ks], accU[mb][c]);
                    accU[mb][c] = mfma16(ul, bv[c][ks], accU[mb][c]);
                }
            }
        }
        // U in fragment order: block tb * 8 + rt holds tokens 16 tb + 4 lq .. +3 of value row 16 rt + lr,
        // which is the accumulator layout of (mb = tb, value row block 2 wave + c)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                *reinterpret_cast<f4v *>(rec + R_U + ((uint32_t)((mb * 8 + 2 * wave + c) * 64 + lane)) * 16) = accU[mb][c];
        lds_barrier();  // every wave holds its K and V fragments: W rows may overwrite them
        // W (hi, lo) rows into LDS over K and V: accumulator (mb, c) holds
        // keys 16 (2 wave + c) + 4 lq + i of token 16 mb + lr
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                h4 hi, lo;
                wa.note(accW[mb][c]);
                split4(accW[mb][c], hi, lo);
                const int key = sw_key(lr, 16 * (2 * wave + c) + 4 * lq);
                *reinterpret_cast<h4 *>(&sW[0][16 * mb + lr][key]) = hi;
                *reinterpret_cast<h4 *>(&sW[1][16 * mb + lr][key]) = lo;
            }
        post(wa);
        lds_barrier();
        // W fragments: f = block * 64 + lane, block = (tb * 4 + kk) * 2 + plane
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int f = tid + 256 * g, blk = f >> 6, fl = f & 63;
            const int tb = blk >> 3, kk = (blk >> 1) & 3, pl = blk & 1;
            *reinterpret_cast<h8 *>(rec + R_W + (size_t)f * 16) = ld_h8(&sW[pl][16 * tb + (fl & 15)][sw_key(fl, 32 * kk + 8 * (fl >> 4))]);
        }
    }
}

// ------------------------------------------------------------------ phase 1, per-key decay
// Decay per key channel (Ascend "aclnnRecurrentGatedDeltaRule", Formula) and
// the key-axis erase gate of Gated DeltaNet-2 (ONNX issue "Spec gap ...
// Gated DeltaNet-2", "The GDN-2 recurrence").  With G[t][j] the cumulative
// log decay of key channel j up to token t inside the chunk, kn = k / |k|,
// qn = q / |q| (or the raw vectors without qk_l2_norm), and the retrieval key
// l_t = beta_t kn_t (delta rules) or b_t o kn_t (erase gate), unrolling the
// recurrence over the chunk gives
//   A_ts = sum_j l_tj kn_sj exp(G_tj - G_sj)  (s < t),   P_ts = scale sum_j qn_tj kn_sj exp(G_tj - G_sj)  (s <= t)
//   W = (I + A)^-1 (l o e^G),   U = (I + A)^-1 diag(w) V   (w = beta, or 1 for the erase gate)
//   Qg = scale qn o e^G,   Kd = kn o e^(G_C - G),   gamma_C = e^(G_C)
// and the scan's chunk step D = U - W S^T, O = Qg S^T + P D,
// S^T <- Diag(gamma_C) S^T + Kd^T D.
//
// A and P are 16 x 16 blocks (s block sb <= t block tb) of fp32 matrix-core
// products over the key channels.  A per-head decay broadcast over the
// channels (the erase gate with a scalar decay, every bf16 problem) leaves
// exp(G_t - G_s) outside the key sum and takes it per element afterwards.  Each block splits its decay at the last
// token e = 16 sb + 15 of block sb: exp(G_t - G_s) = exp(G_t - G_e) exp(G_e - G_s).
// For decaying channels the second factor is <= 1, and so is the first off
// the diagonal; on the diagonal the first is >= 1 and bounded by the decay
// inside the block.  A diagonal block whose decay can exceed DIAG_NATS in
// some channel (and, with growing channels, every block of the chunk) is
// summed term by term instead, so no factor leaves the fp32 range.
//
// 256 threads, two workgroups per CU.  LDS: K and Q rows (fp16) and G (fp32);
// after the Gram products A takes Q's rows and V takes K's, and after the
// solve the W (hi, lo) rows take Q's and G's.
constexpr float DIAG_NATS = 80.f;

template <typename TA, int RULE, bool PKG>
__global__ __launch_bounds__(256, 2) void k_chunk_prep_pk(const Params p, int32_t *__restrict__ off,
                                                          char *__restrict__ ws)
{
    using RC = Rec<true>;
    typedef typename ActVec<TA>::v8 a8;
    typedef typename ActVec<TA>::v4 a4;
    constexpr bool DEC = rule_decays(RULE);
    constexpr bool RET = rule_retrieves(RULE);
    constexpr bool BETA = rule_has_beta(RULE);
    constexpr bool V2 = RULE == GATED_DELTA_V2;
    constexpr int LD = D128 + 8;   // padded fp16 row
    constexpr int LF = D128 + 4;   // padded fp32 row
    constexpr int LA = CH + 4;
    constexpr int SLOT = CH * LD * 2;
    static_assert(CH * LA * 4 == SLOT, "A rows fill Q's slot");
    static_assert(2 * SLOT <= SLOT + CH * LF * 4, "W planes fit over Q and G");

    __shared__ __align__(16) char sm[2 * SLOT + CH * LF * 4];
    TA(*sK)[LD] = reinterpret_cast<TA(*)[LD]>(sm);            // K rows; V rows after the Gram
    TA(*sQ)[LD] = reinterpret_cast<TA(*)[LD]>(sm + SLOT);     // Q rows
    float(*sA)[LA] = reinterpret_cast<float(*)[LA]>(sm + SLOT);       // A after the Gram
    float(*sG)[LF] = reinterpret_cast<float(*)[LF]>(sm + 2 * SLOT);   // G log2(e): cumulative log2 decay
    half_t(*sW)[CH][D128] = reinterpret_cast<half_t(*)[CH][D128]>(sm + SLOT);  // W (hi, lo) after the solve, swizzled rows
    __shared__ float sIk[CH], sIq[CH], sWt[CH];
    __shared__ float sTot[2][D128], sPos[2][D128];
    __shared__ int sFlag;
    // one decay for every key channel: per-token cumulative log2 decay G_t and
    // the factors 2^(G_C - G_t), 2^(G_t)
    __shared__ float sGt[PKG ? 1 : CH], sFk[PKG ? 1 : CH], sFq[PKG ? 1 : CH];

    const int HV = p.HV, H = p.H;
    int64_t ci;
    int h;
    prep_block(HV, ci, h);
    if (ci >= off[p.B]) return;
    const int b = chunk_request(off, p.B, ci);
    int64_t rs, re;
    request_range(p, b, rs, re);
    const int64_t t0 = rs + (ci - off[b]) * CH;
    const int n = (int)((re - t0) < CH ? (re - t0) : CH);
    const int qh = (int)(((int64_t)h * H) / HV);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    const int col = tid & (D128 - 1);
    char *rec = ws + ((size_t)ci * HV + h) * RC::SIZE;
    // A split operand past the fp16 range hands the pair to the recurrent
    // kernel.  Each phase watches its own operands and posts at its end, so no
    // register stays live across the phases.
    int32_t *const flag = off + p.B + 1 + (size_t)b * HV + h;
    auto post = [&](const SplitWatch &w) {
        if (w.over()) *flag = 2;
    };
    const TA *__restrict__ q = static_cast<const TA *>(p.q);
    const TA *__restrict__ k = static_cast<const TA *>(p.k);
    const TA *__restrict__ v = static_cast<const TA *>(p.v);
    const float scale = p.scale;
    // erase gate row of chunk token t (rows past the end read the last token's)
    auto erase_row = [&](int t) { return p.erase + ((size_t)(t0 + (t < n ? t : n - 1)) * HV + h) * D128; };

    // ---- load phase: K, Q, V rows (fp16), log decay rows (fp32); the W-column
    // threads also fetch their erase-gate column for the solve's right-hand side
    a8 ldk[4], ldq[4], ldv[4];
    f4v ldg[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
        ldk[i] = ldq[i] = ldv[i] = a8{};
        if (r < n) {
            const size_t tq = ((size_t)(t0 + r) * H + qh) * D128 + c8;
            ldk[i] = *reinterpret_cast<const a8 *>(k + tq);
            ldq[i] = *reinterpret_cast<const a8 *>(q + tq);
            ldv[i] = *reinterpret_cast<const a8 *>(v + ((size_t)(t0 + r) * HV + h) * D128 + c8);
        }
    }
    if constexpr (PKG) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + 256 * i, r = idx >> 5, c4 = (idx & 31) * 4;
            ldg[i] = f4v{0.f, 0.f, 0.f, 0.f};
            if (r < n) {
                const size_t th = (size_t)(t0 + r) * HV + h;
                if (p.gate_dt == 0 && !p.gate_qwen) {
                    ldg[i] = *reinterpret_cast<const f4v *>(static_cast<const float *>(p.gate) + th * D128 + c4);
                } else {
#pragma unroll
                    for (int x = 0; x < 4; ++x) ldg[i][x] = log_decay_key(p, th, h, c4 + x);
                }
            }
        }
    } else if (tid < CH) {
        // one value per token: a 64-lane inclusive scan, then log2 units
        float g = 0.f;
        if (DEC && tid < n) g = log_decay(p, (size_t)(t0 + tid) * HV + h, h);
#pragma unroll
        for (int o = 1; o < CH; o <<= 1) {
            const float y = __shfl_up(g, o, CH);
            if (tid >= o) g += y;
        }
        g *= LOG2E;
        const float gc = __shfl(g, CH - 1, CH);
        sGt[tid] = g;
        sFk[tid] = tid < n ? ex2(gc - g) : 0.f;
        sFq[tid] = ex2(g);
    }
    if (tid < CH) {
        const int t = tid;
        float w = 0.f;
        if (t < n) w = BETA ? update_rate(p, (size_t)(t0 + t) * HV + h) : 1.f;
        sWt[t] = w;
    }
    if (tid == 0) sFlag = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
        *reinterpret_cast<a8 *>(&sK[r][c8]) = ldk[i];
        *reinterpret_cast<a8 *>(&sQ[r][c8]) = ldq[i];
    }
    if constexpr (PKG) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + 256 * i, r = idx >> 5, c4 = (idx & 31) * 4;
            *reinterpret_cast<f4v *>(&sG[r][c4]) = ldg[i];
        }
    }
    lds_barrier();

    // ---- cumulative log decay: thread (key col, half hf) scans tokens
    // 32 hf .. 32 hf + 31 (bands 2 hf, 2 hf + 1), then adds the first half's total.
    // Guard sums: the decay inside each band (past its first token) bounds the
    // diagonal split factor; the total growth of the chunk bounds every other.
    if constexpr (!PKG) {
        // the per-token values across the row (log2 units already)
        const int hf = tid >> 7;
#pragma unroll
        for (int r = 0; r < 32; ++r) sG[32 * hf + r][col] = sGt[32 * hf + r];
    } else {
        const int hf = tid >> 7;
        float run = 0.f, pos = 0.f, neg[2] = {0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const int t = 32 * hf + r;
            const float g = sG[t][col];
            run += g;
            sG[t][col] = run;
            pos += fmaxf(g, 0.f);
            if (r & 15) neg[r >> 4] += fmaxf(-g, 0.f);
        }
        sTot[hf][col] = run;
        sPos[hf][col] = pos;
        int big = 0;
        if (neg[0] > DIAG_NATS) big |= 1 << (2 * hf);
        if (neg[1] > DIAG_NATS) big |= 1 << (2 * hf + 1);
        if (big) atomicOr(&sFlag, big);
    }
    // ---- inverse L2 norms of the chunk's q and k rows: 4 threads per row
    {
        const int t = tid >> 2, part = tid & 3;
        float ss = 0.f, sq = 0.f;
        if (p.qk_l2_norm) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const a8 kk = *reinterpret_cast<const a8 *>(&sK[t][32 * part + 8 * g]);
                const a8 qq = *reinterpret_cast<const a8 *>(&sQ[t][32 * part + 8 * g]);
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
    // per key: the second half adds the first half's total; both convert to
    // log2 units (a per-token decay is final already)
    if constexpr (PKG) {
        if (tid >= D128) {
            const float add = sTot[0][col];
#pragma unroll
            for (int r = 32; r < CH; ++r) sG[r][col] = (sG[r][col] + add) * LOG2E;
        } else {
#pragma unroll
            for (int r = 0; r < 32; ++r) sG[r][col] *= LOG2E;
            if (sPos[0][col] + sPos[1][col] > DIAG_NATS) atomicOr(&sFlag, 16);
        }
    }
    lds_barrier();

    // A and P come in 16 x 16 blocks (sb <= tb); wave w takes pairs w, w + 4,
    // w + 8 (slots 0, 1, 2).  The erase gate rows of a slot's left operands
    // (token 16 tb + lr, key channels 32 lq .. 32 lq + 31) are loaded one slot
    // ahead, slot 0's while the operands below are built.
    constexpr int8_t PTB[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int8_t PSB[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    f4v ebuf[2][8];
    auto load_eb = [&](int slot, f4v(&e)[8]) {
        const int pi = wave + 4 * slot;
        if (pi < 10) {
            const float *er = erase_row(16 * PTB[pi] + lr);
#pragma unroll
            for (int kq = 0; kq < 8; ++kq) e[kq] = *reinterpret_cast<const f4v *>(er + 32 * lq + 4 * kq);
        }
    };
    if constexpr (V2) load_eb(0, ebuf[0]);

    // ---- operands built from G: Kd^T and Qg fragments (4 + 4 per thread), gamma_C
    SplitWatch wg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // Kd^T: key j, tokens 32 ks + 8 l4 .. +7
        const int f = tid + 256 * i, j = f & (D128 - 1), grp = f >> 7, ks = grp >> 2, l4 = grp & 3;
        const float gc = sG[CH - 1][j];
        float x8[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            const int u = 32 * ks + 8 * l4 + x;
            x8[x] = (float)sK[u][j] * sIk[u] * (PKG ? ex2(gc - sG[u][j]) : sFk[u]);
        }
        h8 hi, lo;
        wg.note(x8);
        split8(x8, hi, lo);
        char *dst = rec + RC::KT + ((uint32_t)(((j >> 4) * 2 + ks) * 2) * 64 + l4 * 16 + (j & 15)) * 16;
        *reinterpret_cast<h8 *>(dst) = hi;
        *reinterpret_cast<h8 *>(dst + 1024) = lo;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // Qg: token 16 tb + lr, keys 32 kk + 8 lq .. +7
        const int f = tid + 256 * i, blk = f >> 6, fl = f & 63;
        const int t = 16 * (blk >> 2) + (fl & 15), key = 32 * (blk & 3) + 8 * (fl >> 4);
        const a8 qq = *reinterpret_cast<const a8 *>(&sQ[t][key]);
        float x8[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) x8[x] = scale * sIq[t] * (float)qq[x] * (PKG ? ex2(sG[t][key + x]) : sFq[t]);
        wg.note(x8);
        *reinterpret_cast<h8 *>(rec + RC::Q + ((uint32_t)blk * 64 + fl) * 16) = round_h8(x8);
    }
    post(wg);
    if (tid < D128) reinterpret_cast<float *>(rec + RC::SC)[tid] = ex2(sG[CH - 1][tid]);

    // erase gate at this lane's right-hand-side fragment positions of W
    // (tokens 32 ks + 8 lq + x, key 16 (2 wave + c) + lr), in flight during the Gram blocks
    float ev[2][2][8];
    if constexpr (V2) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int x = 0; x < 8; ++x) ev[c][ks][x] = erase_row(32 * ks + 8 * lq + x)[16 * (2 * wave + c) + lr];
    }

    // ---- A and P blocks on the fp32 matrix cores.  Lane (lr, lq) sums key
    // channels 32 lq .. 32 lq + 31, and the accumulators hold
    // [s = 16 sb + 4 lq + i][t = 16 tb + lr] without the per-token factors
    // (applied below).
    const int flags = sFlag;
    f4v resA[3], resP[3];
#pragma unroll
    for (int slot = 0; slot < 3; ++slot) {
        if constexpr (V2) {
            if (slot + 1 < 3) load_eb(slot + 1, ebuf[(slot + 1) & 1]);
        }
        const f4v(&eb)[8] = ebuf[slot & 1];
        const int pi = wave + 4 * slot;
        resA[slot] = resP[slot] = f4v{0.f, 0.f, 0.f, 0.f};
        if (pi < 10) {
            const int tb = PTB[pi], sb = PSB[pi], e = 16 * sb + 15;
            const int t = 16 * tb + lr, sr = 16 * sb + lr;
            const float *er = V2 ? erase_row(t) : nullptr;
            if constexpr (!PKG) {
                // one decay for every key channel: exp(G_t - G_s) leaves the key sum
                // as a scalar, so the products carry no exponentials and the factor
                // (<= 1 for s <= t when the head decays) is applied per element after
                f4v accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
                if constexpr (!V2) {
                    // plain products of the stored 16-bit values, exact in fp32: the
                    // 16x16x32 matrix op takes 8 keys per lane and step (lane (lr, lq):
                    // keys 32 kk + 8 lq .. +7), same accumulator layout
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const int key = 32 * kk + 8 * lq;
                        const a8 ks8 = *reinterpret_cast<const a8 *>(&sK[sr][key]);
                        if constexpr (RET) accA = mfma16x32(ks8, *reinterpret_cast<const a8 *>(&sK[t][key]), accA);
                        accP = mfma16x32(ks8, *reinterpret_cast<const a8 *>(&sQ[t][key]), accP);
                    }
                } else {
                    // b o k is not a 16-bit value: fp32 products, 4 keys per step
#pragma unroll
                    for (int kq = 0; kq < 8; ++kq) {
                        const int key = 32 * lq + 4 * kq;
                        const a4 kt = *reinterpret_cast<const a4 *>(&sK[t][key]);
                        const a4 ks = *reinterpret_cast<const a4 *>(&sK[sr][key]);
                        const a4 qt = *reinterpret_cast<const a4 *>(&sQ[t][key]);
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const float right = to_f32(ks[x]);
                            accA = __builtin_amdgcn_mfma_f32_16x16x4f32(right, eb[kq][x] * to_f32(kt[x]), accA, 0, 0, 0);
                            accP = __builtin_amdgcn_mfma_f32_16x16x4f32(right, to_f32(qt[x]), accP, 0, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 16 * sb + 4 * lq + i;
                    const float f = s <= t ? ex2(sG[t][0] - sG[s][0]) : 0.f;
                    resA[slot][i] = accA[i] * f;
                    resP[slot][i] = accP[i] * f;
                }
            } else if ((flags & 16) || (tb == sb && ((flags >> tb) & 1))) {
                // strong decay inside the block (or growth): every term with its own exponential
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 16 * sb + 4 * lq + i;
                    float a = 0.f, pq = 0.f;
                    if (s <= t) {
                        for (int j = 0; j < D128; ++j) {
                            const float kx = (float)sK[s][j] * ex2(sG[t][j] - sG[s][j]);
                            if constexpr (RET) a = fmaf((V2 ? er[j] : 1.f) * (float)sK[t][j], kx, a);
                            pq = fmaf((float)sQ[t][j], kx, pq);
                        }
                    }
                    resA[slot][i] = a;
                    resP[slot][i] = pq;
                }
            } else {
                f4v accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kq = 0; kq < 8; ++kq) {
                    const int key = 32 * lq + 4 * kq;
                    const f4v gt = *reinterpret_cast<const f4v *>(&sG[t][key]);
                    const f4v ge = *reinterpret_cast<const f4v *>(&sG[e][key]);
                    const f4v gs = *reinterpret_cast<const f4v *>(&sG[sr][key]);
                    const a4 kt = *reinterpret_cast<const a4 *>(&sK[t][key]);
                    const a4 ks = *reinterpret_cast<const a4 *>(&sK[sr][key]);
                    const a4 qt = *reinterpret_cast<const a4 *>(&sQ[t][key]);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const float exa = ex2(gt[x] - ge[x]);
                        const float right = (float)ks[x] * ex2(ge[x] - gs[x]);
                        if constexpr (RET)
                            accA = __builtin_amdgcn_mfma_f32_16x16x4f32(right, (V2 ? eb[kq][x] : 1.f) * (float)kt[x] * exa, accA, 0, 0, 0);
                        accP = __builtin_amdgcn_mfma_f32_16x16x4f32(right, (float)qt[x] * exa, accP, 0, 0, 0);
                    }
                }
                resA[slot] = accA;
                resP[slot] = accP;
            }
        }
    }
    // ---- right-hand side of W, l o e^G, in matrix-core fragments: wave w takes
    // key columns 32 w .. 32 w + 31 (blocks c), tokens 32 ks + 8 lq .. +7;
    // fp32 values, so (hi, lo) fp16 planes
    h8 bwh[2][2], bwl[2][2];
    if constexpr (RET) {
        SplitWatch wx;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int j = 16 * (2 * wave + c) + lr, s0 = 32 * ks + 8 * lq;
                float xw[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const int u = s0 + x;
                    xw[x] = (V2 ? ev[c][ks][x] : sWt[u]) * sIk[u] * to_f32(sK[u][j]) * (PKG ? ex2(sG[u][j]) : sFq[u]);
                }
                wx.note(xw);
                split8(xw, bwh[c][ks], bwl[c][ks]);
            }
        post(wx);
    }
    lds_barrier();  // K, Q and G are dead: V takes K's rows, A takes Q's, W's right-hand side G's

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, r = idx >> 4, c8 = (idx & 15) * 8;
        *reinterpret_cast<a8 *>(&sK[r][c8]) = ldv[i];
    }
    if (!post_vmax(ldv, rec + RC::SC)) *flag = 2;
    // W's right-hand-side fragments wait in LDS (in fragment order: one
    // 16-byte read each later), so no register holds them across the solve
    h8 *sBw = reinterpret_cast<h8 *>(sm + 2 * SLOT);  // [plane][wave][c][ks][lane]
    static_assert(2 * 4 * 4 * 64 * sizeof(h8) <= CH * LF * 4, "W's right-hand-side fragments fit in G's slot");
    if constexpr (RET) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                sBw[((0 * 4 + wave) * 4 + c * 2 + ks) * 64 + lane] = bwh[c][ks];
                sBw[((1 * 4 + wave) * 4 + c * 2 + ks) * 64 + lane] = bwl[c][ks];
            }
    }
    SplitWatch wp;
#pragma unroll
    for (int slot = 0; slot < 3; ++slot) {
        const int pi = wave + 4 * slot;
        if (pi < 10) {
            const int tb = PTB[pi], sb = PSB[pi];
            const int t = 16 * tb + lr, s0 = 16 * sb + 4 * lq;
            const float at = (V2 ? 1.f : sWt[t]) * sIk[t], pt = scale * sIq[t];
            f4v pv, av;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = s0 + i;
                pv[i] = s <= t ? pt * sIk[s] * resP[slot][i] : 0.f;
                av[i] = s < t ? at * sIk[s] * resA[slot][i] : 0.f;
            }
            wp.note(pv);
            const uint32_t po = RC::P + ((uint32_t)(tb * 2 + (s0 >> 5)) * 64 + ((s0 & 31) >> 3) * 16 + lr) * 16 + ((s0 & 7) >> 2) * 8;
            *reinterpret_cast<h4 *>(rec + po) = round_h4(pv);  // P enters only the outputs
            if constexpr (RET) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sA[t][a_pos(s0 + i)] = av[i];
            }
        }
    }
    post(wp);
    if (wave < 2) {
        // the P blocks above the diagonal are zero (the scan multiplies them
        // anyway); only the two that share a fragment with nonzero blocks are
        // stored -- (tb, sb) = (0, 1) on wave 0, (2, 3) on wave 1 -- while the
        // all-zero fragments of token blocks 0, 1 against tokens 32 .. 63 are
        // read as zero past the record's end
        const int tb = 2 * wave, sb = 2 * wave + 1, s0 = 16 * sb + 4 * lq;
        const uint32_t po = RC::P + ((uint32_t)(tb * 2 + (s0 >> 5)) * 64 + ((s0 & 31) >> 3) * 16 + lr) * 16 + ((s0 & 7) >> 2) * 8;
        *reinterpret_cast<h4 *>(rec + po) = h4{};
    }
    lds_barrier();

    if constexpr (!RET) {
        // no retrieval: U = V, stored in fragment order by the row-column threads
        if (tid >= D128) {
#pragma unroll
            for (int qd = 0; qd < CH / 4; ++qd) {
                f4v u;
#pragma unroll
                for (int i = 0; i < 4; ++i) u[i] = to_f32(sK[4 * qd + i][col]);
                *reinterpret_cast<f4v *>(rec + RC::U + ((uint32_t)(((qd >> 2) * 8 + (col >> 4)) * 64 + (qd & 3) * 16 + (col & 15))) * 16) = u;
            }
        }
        return;
    } else {
        // ---- [W | U] = T [l o e^G | diag(w) V],  T = (I + A)^-1, as in the
        // per-head prologue: the four waves form T by forward substitution,
        // then wave w takes key columns and value rows 32 w .. 32 w + 31
        // on the matrix cores (W: three split products, U: V is exact in the
        // activation dtype only when that is fp16, so both operands of U get
        // (hi, lo) planes for bf16).
        {
            // the column times its weight (split beside T below) peaks where
            // |T| does: rounding is monotone
            SplitWatch wt;
            solve_blocked(sA, tid, sWt, wt);
            post(wt);
        }
        lds_barrier();  // T is complete
        constexpr bool VX = sizeof(TA) == 2 && !__is_same(TA, bf16_t);  // V exact in fp16
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bwh[c][ks] = sBw[((0 * 4 + wave) * 4 + c * 2 + ks) * 64 + lane];
                bwl[c][ks] = sBw[((1 * 4 + wave) * 4 + c * 2 + ks) * 64 + lane];
            }
        h8 bvh[2][2], bvl[2][2];
        SplitWatch wv, wa;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int cc = 16 * (2 * wave + c) + lr, s0 = 32 * ks + 8 * lq;
                float xv[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) xv[x] = to_f32(sK[s0 + x][cc]);
                wv.note(xv);
                split8(xv, bvh[c][ks], bvl[c][ks]);
            }
        post(wv);
        f4v accW[4][2], accU[4][2];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
            for (int c = 0; c < 2; ++c) accW[mb][c] = accU[mb][c] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < (mb < 2 ? 1 : 2); ++ks) {
                const int t = 16 * mb + lr, s0 = 32 * ks + 8 * lq;
                const f4v t0v = *reinterpret_cast<const f4v *>(&sA[t][s0]);
                const f4v t1v = *reinterpret_cast<const f4v *>(&sA[t][s0 + 4]);
                float tv[8], tw[8];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    tv[x] = t0v[x];
                    tv[4 + x] = t1v[x];
                }
#pragma unroll
                for (int x = 0; x < 8; ++x) tw[x] = tv[x] * sWt[s0 + x];
                h8 th, tl, uh, ul;
                split8(tv, th, tl);
                split8(tw, uh, ul);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    // W^T = RHS^T T^T: each lane ends with four consecutive keys of one token
                    accW[mb][c] = mfma16(bwh[c][ks], th, accW[mb][c]);
                    accW[mb][c] = mfma16(bwl[c][ks], th, accW[mb][c]);
                    accW[mb][c] = mfma16(bwh[c][ks], tl, accW[mb][c]);
                    accU[mb][c] = mfma16(uh, bvh[c][ks], accU[mb][c]);
                    accU[mb][c] = mfma16(ul, bvh[c][ks], accU[mb][c]);
                    if constexpr (!VX) accU[mb][c] = mfma16(uh, bvl[c][ks], accU[mb][c]);
                }
            }
        }
        // U: accumulator (mb, c) is block mb * 8 + 2 wave + c of the record
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                *reinterpret_cast<f4v *>(rec + RC::U + ((uint32_t)((mb * 8 + 2 * wave + c) * 64 + lane)) * 16) = accU[mb][c];
        lds_barrier();  // T and V are read: W (hi, lo) rows take the place of A and G
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                h4 hi, lo;
                wa.note(accW[mb][c]);
                split4(accW[mb][c], hi, lo);
                const int key = sw_key(lr, 16 * (2 * wave + c) + 4 * lq);
                *reinterpret_cast<h4 *>(&sW[0][16 * mb + lr][key]) = hi;
                *reinterpret_cast<h4 *>(&sW[1][16 * mb + lr][key]) = lo;
            }
        post(wa);
        lds_barrier();
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int f = tid + 256 * g, blk = f >> 6, fl = f & 63;
            const int tb = blk >> 3, kk = (blk >> 1) & 3, pl = blk & 1;
            *reinterpret_cast<h8 *>(rec + RC::W + (size_t)f * 16) = ld_h8(&sW[pl][16 * tb + (fl & 15)][sw_key(fl, 32 * kk + 8 * (fl >> 4))]);
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
// With a decay per key channel (PK) the state decays by a vector gamma_C, and
// Kd^T and Qg carry fp32 values split into (hi, lo) planes, so stage E and O1
// take three products each; stage E then reads D^T directly (no kd D copy).
//
// Segmented chain.  A chunk step maps every state row affinely,
// s <- s M_j + c_j (M_j = gamma_C I - W^T diag(kd) K, c_j the row's share of
// kd U K), so a request's chunks can be cut into nseg segments that run side
// by side.  Pass 1 runs segment 0 for real (writing its end state as the start
// of segment 1) and, for each middle segment p, a carry tile (zero start:
// c_p = the segment's end state from zero) and a transition tile (the 128 rows
// of the identity as start, U left out: M_p = the product of the segment's
// M_j).  k_seg_combine then forms start_{p+1} = start_p M_p + c_p, and pass 2
// runs segments 1 .. nseg-1 for real from those starts.  The longest serial
// chain shrinks from n chunk steps to about 2 n / nseg.
template <typename TA, int RULE, int NVB, bool PK>
__global__ __launch_bounds__(512) void k_chunk_scan(const Params p, int32_t *off, const char *ws, const char *kqs,
                                                   const ScanSeg sg)
{
    using RC = Rec<PK>;
    constexpr int NPL = PK ? 2 : 1;       // fp16 planes of the K^T and q operands
    constexpr bool RET = rule_retrieves(RULE);
    constexpr int TR = 16 * NVB;          // state rows of this workgroup
    constexpr int NTILE = D128 / TR;      // workgroups per head
    // unpadded rows, 16-byte chunks swizzled per row (sw_key, sw_tok)
    __shared__ __align__(16) half_t sS[2][2][TR][D128];  // [buffer][hi, lo][row][key]
    __shared__ __align__(16) half_t sDt[2][2][TR][CH];   // [buffer][hi, lo][row][token] D^T
    __shared__ __align__(16) half_t sDs[2][PK ? 1 : TR][CH];  // [hi, lo][row][token] (kd D)^T, chain only
    __shared__ __align__(16) TA sO[4][16][TR + 8];       // per output wave: [token][row] staging for the store
    __shared__ float sTM[4][2];                           // per chain wave: max |S0| of its part, max |v|

    const int HV = p.HV;
    // A group is one (request, head) -- with segments one (request, head,
    // segment) -- and its units are its row tiles (pass 1: carry tiles, then
    // transition tiles).  XCD-aware order: blocks i, i + 8, ... (one XCD) are
    // the units of one group, which read the same chunk records, and with
    // grouped heads the next groups there are the other value heads of the
    // same q/k head (xcd_heads).
    const int NU = (sg.pass == 1 ? 2 : 1) * NTILE;
    const int nsg = sg.pass == 0 ? 1 : sg.nseg - 1;  // groups per (request, head)
    const int gs = xcd_heads(p.H, HV, sg.pass);      // groups in a row on one XCD
    const int xl = blockIdx.x & 7, q8 = blockIdx.x >> 3, unit = q8 % NU, rest = q8 / NU;
    const int64_t gi = ((int64_t)(rest / gs) * 8 + xl) * gs + rest % gs;
    if (gi >= (int64_t)p.B * HV * nsg) return;
    // group -> (request, head): requests longest first (k_chunk_table's order)
    const int pr = (int)(gi / nsg), seg = (int)(gi % nsg) + (sg.pass == 2 ? 1 : 0);
    const int bh = off[p.B + 1 + (size_t)p.B * HV + pr / HV] * HV + pr % HV;
    const int tile = unit % NTILE;
    const int mode = sg.pass != 1 ? SEG_REAL : unit < NTILE ? (seg == 0 ? SEG_REAL : SEG_CARRY) : SEG_TRANS;
    if (mode == SEG_TRANS && seg == 0) return;  // segment 0 has no transition tiles
    const int b = bh / HV, h = bh % HV;
    if (off[p.B + 1 + bh]) return;  // the recurrent kernel takes this pair
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
    // this unit's chunks [cb, ce) of the request, its start state and where its end state goes
    const int ns = sg.pass == 0 ? 1 : sg.nseg;
    const int cb = seg_lo(seg, nch, ns), ce = seg_lo(seg + 1, nch, ns);
    const float *from = src;
    // an in-place final state is staged (the commit kernel copies it back unless
    // the pair is handed to the recurrent kernel, which then reads the intact state)
    float *const fin = sg.stage ? sg.stage + (size_t)bh * (D128 * D128) : dst;
    float *to = fin;
    if (sg.pass != 0) {
        float *xs = sg.xs + (size_t)bh * seg_slots(ns) * (D128 * D128);
        if (mode == SEG_REAL) {
            from = seg == 0 ? src : xs + (size_t)seg_start(seg) * (D128 * D128);
            to = seg == ns - 1 ? fin : seg == 0 ? xs + (size_t)seg_start(1) * (D128 * D128) : nullptr;
        } else {
            from = nullptr;
            to = xs + (size_t)(mode == SEG_CARRY ? seg_carry(ns, seg) : seg_trans(ns, seg)) * (D128 * D128);
        }
    }
    const int tb = wave & 3;  // token block of this wave (D rows for the chain, O columns for the output)
    const int qh = (int)(((int64_t)h * p.H) / HV);
    // The tile runs scaled by 2^e (tile_exponent): from max |v| over the
    // unit's chunks (a transition tile leaves v out) and the tile's max |S0|,
    // which the chain waves post before the first barrier.  A unit with no
    // chunks copies its state unscaled.
    auto scale_exp = [&]() {
        const float ms = fmaxf(fmaxf(sTM[0][0], sTM[1][0]), fmaxf(sTM[2][0], sTM[3][0]));
        const float mv = fmaxf(fmaxf(sTM[0][1], sTM[1][1]), fmaxf(sTM[2][1], sTM[3][1]));
        return ce > cb ? tile_exponent(fmaxf(mode == SEG_TRANS ? 0.f : mv, ms)) : 0;
    };
    // per head: K^T of chunk jj comes from the (chunk, q/k head) area, else from the record
    auto kq_rsrc = [&](int jj) {
        if constexpr (PK) return make_rsrc(ws + ((size_t)(c0 + jj) * HV + h) * RC::SIZE, RC::SIZE);
        else return make_rsrc(kqs + ((size_t)(c0 + jj) * p.H + qh) * KQ::SIZE, KQ::SIZE);
    };

    if (wave < 4) {
        // ================================================================ chain
        // max |v| over the unit's chunks, as the prologue waves posted it
        float mv = 0.f;
        for (int j = cb + tid; j < ce; j += 256) {
            const f4v m4 = *reinterpret_cast<const f4v *>(ws + ((size_t)(c0 + j) * HV + h) * RC::SIZE + RC::SC +
                                                          SC_VMAX * 4);
            mv = fmaxf(mv, fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
        }
        // Sc[a][rt][i] = S[row0 + 16 rt + lr][16 (2 wave + a) + 4 lq + i]
        f4v Sc[2][NVB];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int rt = 0; rt < NVB; ++rt)
            {
                const int row = row0 + 16 * rt + lr, col = 16 * (2 * wave + a) + 4 * lq;
                if (from) {
                    Sc[a][rt] = *reinterpret_cast<const f4v *>(from + (size_t)row * D128 + col);
                } else {
                    // zero, or row `row` of the identity for a transition tile
                    const float one = mode == SEG_TRANS ? 1.f : 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) Sc[a][rt][i] = row == col + i ? one : 0.f;
                }
            }
        {
            float mx = 0.f;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(Sc[a][rt][i]));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                mx = fmaxf(mx, __shfl_xor(mx, o));
                mv = fmaxf(mv, __shfl_xor(mv, o));
            }
            if (lane == 0) {
                sTM[wave][0] = mx;
                sTM[wave][1] = mv;
            }
        }
        lds_barrier();  // 0: the tile's max |S0| is posted
        const int sx = scale_exp();
        const float up = ldexpf(1.f, sx), down = ldexpf(1.f, -sx);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int rt = 0; rt < NVB; ++rt) Sc[a][rt] *= up;
        const float um = mode == SEG_TRANS ? 0.f : up;  // a transition tile leaves U out
        ScanWatch sw;
        struct Ops {
            h8 wh[4], wl[4];    // W (hi, lo) of token block tb, four k-steps of 32
            h8 kt[2][2][NPL];   // K^T (per key: Kd^T hi, lo) fragments: key tiles 2 wave + a, token steps ks
            f4v u[NVB];         // U at this lane's D positions, one per row block
            f4v kd;             // per head: kd of this lane's four D tokens
            float gc;           // per head: gamma_C
            f4v gk[2];          // per key: gamma_C of keys 16 (2 wave + a) + 4 lq .. +3
        };
        const uint32_t offW = RC::W + (uint32_t)tb * 8 * 1024 + l16;
        const uint32_t offK = (PK ? RC::KT : KQ::KT) + (uint32_t)(2 * wave) * 2 * NPL * 1024 + l16;
        const uint32_t offU = RC::U + (uint32_t)(tb * 8 + NVB * tile) * 1024 + l16;
        const uint32_t offKd = RC::SC + (uint32_t)(16 * tb + 4 * lq) * 4;
        const uint32_t offGk = RC::SC + (uint32_t)(32 * wave + 4 * lq) * 4;
        // One operand set, reloaded for chunk jj right after its last use in the
        // current chunk (stage B's operands after D is formed, stage E's after the
        // state update), so the loads overlap the rest of the step.
        auto fetchB = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(ws + ((size_t)(c0 + jj) * HV + h) * RC::SIZE, RC::SIZE);
            if constexpr (RET) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    f.wh[kk] = ld_b128<h8>(r, offW + 2048 * kk);
                    f.wl[kk] = ld_b128<h8>(r, offW + 2048 * kk + 1024);
                }
            }
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) f.u[vb] = ld_b128<f4v>(r, offU + vb * 1024);
            if constexpr (!PK) f.kd = ld_b128<f4v>(r, offKd);
        };
        auto fetchE = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(ws + ((size_t)(c0 + jj) * HV + h) * RC::SIZE, RC::SIZE);
            const __amdgpu_buffer_rsrc_t rk = kq_rsrc(jj);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int pl = 0; pl < NPL; ++pl) f.kt[a][ks][pl] = ld_b128<h8>(rk, offK + ((2 * a + ks) * NPL + pl) * 1024);
            if constexpr (PK) {
                f.gk[0] = ld_b128<f4v>(r, offGk);
                f.gk[1] = ld_b128<f4v>(r, offGk + 64);
            } else {
                f.gc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, RC::SC + 2 * CH * 4, 0, 0));
            }
        };
        auto step = [&](int j, Ops &cur) {
            const int bf = j & 1;
            const int jn = j + 1 < ce ? j + 1 : j;  // the last chunk re-reads itself
            // ---- A: state tile -> LDS (hi, lo), four consecutive keys per write
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt) {
                    h4 hi, lo;
                    sw.note(Sc[a][rt]);
                    split4(Sc[a][rt], hi, lo);
                    *reinterpret_cast<h4 *>(&sS[bf][0][16 * rt + lr][sw_key(lr, 16 * (2 * wave + a) + 4 * lq)]) = hi;
                    *reinterpret_cast<h4 *>(&sS[bf][1][16 * rt + lr][sw_key(lr, 16 * (2 * wave + a) + 4 * lq)]) = lo;
                }
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
                            const h8 shi = ld_h8(&sS[bf][0][16 * vb + lr][sw_key(lr, 32 * kk + lk)]);
                            const h8 slo = ld_h8(&sS[bf][1][16 * vb + lr][sw_key(lr, 32 * kk + lk)]);
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
            f4v dv[NVB], dsv[NVB];
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) dv[vb][i] = um * cur.u[vb][i] - accD[vb][i];
                if constexpr (!PK) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) dsv[vb][i] = cur.kd[i] * dv[vb][i];
                }
            }
            // stage B's operands are used up: load chunk jn's, and keep the loads
            // here (neither the optimiser nor the scheduler may move them)
            fetchB(jn, cur);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                h4 dh, dl;
                sw.note(dv[vb]);
                split4(dv[vb], dh, dl);
                const int r = 16 * vb + lr, c = 16 * tb + 4 * lq;
                *reinterpret_cast<h4 *>(&sDt[bf][0][r][sw_tok(lr, c)]) = dh;
                *reinterpret_cast<h4 *>(&sDt[bf][1][r][sw_tok(lr, c)]) = dl;
                if constexpr (!PK) {
                    h4 sh, sl;
                    sw.note(dsv[vb]);
                    split4(dsv[vb], sh, sl);
                    *reinterpret_cast<h4 *>(&sDs[0][r][sw_tok(lr, c)]) = sh;
                    *reinterpret_cast<h4 *>(&sDs[1][r][sw_tok(lr, c)]) = sl;
                }
            }
            lds_barrier();  // 2
            // ---- E: S^T <- gamma_C S^T + K^T (kd D) for key tiles 2 wave + a, row blocks rt
            // (per key: S^T <- Diag(gamma_C) S^T + Kd^T D)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt) {
                    if constexpr (PK) Sc[a][rt] *= cur.gk[a];
                    else Sc[a][rt] *= cur.gc;
                }
            {
                // with two row blocks the lo products get their own chains
                constexpr bool SEPL = NVB < 4 || PK;
                f4v lo4[2][NVB] = {};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int rt = 0; rt < NVB; ++rt) {
                        const h8 dhi = PK ? ld_h8(&sDt[bf][0][16 * rt + lr][sw_tok(lr, 32 * ks + lk)]) : ld_h8(&sDs[0][16 * rt + lr][sw_tok(lr, 32 * ks + lk)]);
                        const h8 dlo = PK ? ld_h8(&sDt[bf][1][16 * rt + lr][sw_tok(lr, 32 * ks + lk)]) : ld_h8(&sDs[1][16 * rt + lr][sw_tok(lr, 32 * ks + lk)]);
#pragma unroll
                        for (int a = 0; a < 2; ++a) {
                            Sc[a][rt] = mfma16(cur.kt[a][ks][0], dhi, Sc[a][rt]);
                            if constexpr (SEPL) lo4[a][rt] = mfma16(cur.kt[a][ks][0], dlo, lo4[a][rt]);
                            else Sc[a][rt] = mfma16(cur.kt[a][ks][0], dlo, Sc[a][rt]);
                            if constexpr (PK) lo4[a][rt] = mfma16(cur.kt[a][ks][NPL - 1], dhi, lo4[a][rt]);
                        }
                    }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int rt = 0; rt < NVB; ++rt)
                        if constexpr (SEPL) Sc[a][rt] += lo4[a][rt];
            }
            fetchE(jn, cur);  // stage E's operands are used up
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        };
        Ops op;
        if (ce > cb) {
            fetchB(cb, op);
            fetchE(cb, op);
        }
        for (int j = cb; j < ce; ++j) step(j, op);
        if (to) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt)
                    *reinterpret_cast<f4v *>(to + (size_t)(row0 + 16 * rt + lr) * D128 + 16 * (2 * wave + a) + 4 * lq) = Sc[a][rt] * down;
        }
        // A split operand at or past SPLIT_LIMIT (or not finite) leaves the fp16
        // range of its hi part: the pair goes to the recurrent kernel, which
        // recomputes it in fp32 (its o rows and its final state).
        if (sw.over()) off[p.B + 1 + bh] = 2;
    } else if (mode != SEG_REAL) {
        // carry and transition tiles write no output: these waves only keep
        // the chain's barriers (one at the start, two per chunk step)
        lds_barrier();  // 0
        for (int j = cb; j < ce; ++j) {
            lds_barrier();
            lds_barrier();
        }
    } else {
        // ================================================================ outputs
        TA *o = static_cast<TA *>(p.o);
        lds_barrier();  // 0: the chain waves have posted the tile's max |S0|
        const float down = ldexpf(1.f, -scale_exp());  // o = (scaled o) / 2^e
        struct Ops {
            h8 q[4][1];       // q rows (per key: Qg, one fp16 plane) of token block tb, four k-steps of 32
            h8 ph[2];         // P rows (one fp16 plane) of token block tb, two token steps of 32
            float gq;         // per head: gq of this lane's token
        };
        // per key: Qg from the record; per head: q rows from the
        // activations (row 16 tb + lr, keys 32 kk + 8 lq .. +7), converted to fp16
        // as they load (the prologue has handed pairs with values fp16 cannot
        // hold to the recurrent kernel); rows past the request's end read zero
        const uint32_t offQ = PK ? RC::Q + (uint32_t)tb * 4 * 1024 + l16
                                 : (uint32_t)((16 * tb + lr) * p.H * D128 * 2 + 2 * lk);
        // o byte offset of this lane's token (16 tb + lr) and rows 4 lq .. +3 inside a chunk
        const int tok_bytes = HV * D128 * 2;
        // after the LDS transpose each lane stores 16 bytes (8 rows of a token):
        // TR / 8 lanes per token, so a 32-row tile uses every lane for its 16
        // tokens, a 64-row tile every lane twice (tokens 0-7, then 8-15) and a
        // 16-row tile the first 32 lanes; the others get an offset past the
        // store's range, which the buffer store drops
        static_assert(TR == 64 || TR == 32 || TR == 16, "the output transpose takes 16-, 32- or 64-row tiles");
        constexpr int LPT = TR / 8;                       // lanes per token
        constexpr int NST = TR == 64 ? 2 : 1;             // stores per lane
        constexpr int TPS = 16 / NST;                     // tokens per store pass
        const bool st_live = lane / LPT < TPS;
        const int st_tok = st_live ? lane / LPT : TPS - 1, st_q = lane % LPT;
        const uint32_t offO = st_live ? (uint32_t)((16 * tb + st_tok) * tok_bytes + 16 * st_q) : 0x7FFFFFF0u;
        const uint32_t offP = RC::P + (uint32_t)tb * 2 * 1024 + l16;
        // token blocks 0, 1 against tokens 32 .. 63: all zero, not stored; an offset
        // past the record makes the buffer load return zero
        const uint32_t offP1 = tb < 2 ? 0x7FFFF000u : offP + 1024;
        const uint32_t offG = RC::SC + (uint32_t)(CH + 16 * tb + lr) * 4;
        // one operand set, each part reloaded for chunk jj right after its last use
        auto fetchQ = [&](int jj, Ops &f) {
            if constexpr (PK) {
                const __amdgpu_buffer_rsrc_t r = kq_rsrc(jj);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) f.q[kk][0] = ld_b128<h8>(r, offQ + kk * 1024);
            } else {
                const int64_t t0 = rs + (int64_t)jj * CH;
                const int n = (int)((re - t0) < CH ? (re - t0) : CH);
                const TA *base = static_cast<const TA *>(p.q) + ((size_t)t0 * p.H + qh) * D128;
                const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<TA *>(base), 0, (n - 1) * p.H * D128 * 2 + D128 * 2, 0x00020000);
                bool ok = true;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) f.q[kk][0] = to_h8(ld_b128<typename ActVec<TA>::v8>(r, offQ + 64 * kk), ok);
            }
        };
        auto fetchG = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(ws + ((size_t)(c0 + jj) * HV + h) * RC::SIZE, RC::SIZE);
            if constexpr (!PK) f.gq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, offG, 0, 0));
        };
        auto fetchP = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(ws + ((size_t)(c0 + jj) * HV + h) * RC::SIZE, RC::SIZE);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                f.ph[ks] = ld_b128<h8>(r, ks ? offP1 : offP);
            }
        };
        // Store the output tile of chunk jo, staged in sO, as one 16-byte write per
        // lane.  The store is unconditional: the resource spans the chunk's
        // valid tokens only (none for jo < 0), so lanes past the request's end
        // write nothing (a branch here would make every later wait drain it).
        auto store_out = [&](int jo) {
            const int64_t t0 = rs + (int64_t)jo * CH;
            const int n = jo >= cb ? (int)((re - t0) < CH ? (re - t0) : CH) : 0;
            TA *base = jo >= cb ? o + ((size_t)t0 * HV + h) * D128 + row0 : o;
            const __amdgpu_buffer_rsrc_t ro =
                __builtin_amdgcn_make_buffer_rsrc(base, 0, n > 0 ? (int)((n - 1) * tok_bytes + TR * 2) : 0, 0x00020000);
#pragma unroll
            for (int ps = 0; ps < NST; ++ps)
                __builtin_amdgcn_raw_buffer_store_b128(ld_b128_lds(&sO[tb][st_tok + TPS * ps][8 * st_q]), ro,
                                                       offO + (uint32_t)(TPS * ps * tok_bytes), 0, 0);
        };
        auto step = [&](int j, Ops &cur) {
            const int bf = j & 1;
            const int jn = j + 1 < ce ? j + 1 : j;
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
                    const h8 shi = ld_h8(&sS[bf][0][16 * vb + lr][sw_key(lr, 32 * kk + lk)]);
                    const h8 slo = ld_h8(&sS[bf][1][16 * vb + lr][sw_key(lr, 32 * kk + lk)]);
                    acc[vb] = mfma16(shi, cur.q[kk][0], acc[vb]);
                    acl[vb] = mfma16(slo, cur.q[kk][0], acl[vb]);
                }
            fetchQ(jn, cur);  // pinned like the chain's loads
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();  // 2
            // ---- O2: O^T = gq O^T + D^T P^T; P is lower triangular (zeros above the
            // diagonal are multiplied anyway so every prefetched fragment is used)
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                if constexpr (PK) acc[vb] = acc[vb] + acl[vb];
                else acc[vb] = cur.gq * (acc[vb] + acl[vb]);
            }
            fetchG(jn, cur);
            {
                f4v p3[NVB] = {};  // the lo product in its own chain
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) {
                        const h8 dhi = ld_h8(&sDt[bf][0][16 * vb + lr][sw_tok(lr, 32 * ks + lk)]);
                        const h8 dlo = ld_h8(&sDt[bf][1][16 * vb + lr][sw_tok(lr, 32 * ks + lk)]);
                        acc[vb] = mfma16(dhi, cur.ph[ks], acc[vb]);
                        p3[vb] = mfma16(dlo, cur.ph[ks], p3[vb]);
                    }
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) acc[vb] += p3[vb];
            }
            fetchP(jn, cur);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            // stage the tile as [token][row]; the next chunk (or the loop's end) stores it
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                typename ActVec<TA>::v4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = from_f32<TA>(acc[vb][i] * down);
                *reinterpret_cast<typename ActVec<TA>::v4 *>(&sO[tb][lr][16 * vb + 4 * lq]) = ov;
            }
        };
        Ops op;
        if (ce > cb) {
            fetchQ(cb, op);
            fetchG(cb, op);
            fetchP(cb, op);
        }
        {
            // a store that writes nothing (empty resource): on entry the loop
            // then sees the same outstanding pattern as in steady state (the
            // previous chunk's output store behind the prefetch), so the
            // compiler's waits for the prefetch need not cover a real store
            const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(o, 0, 0, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b128(u4v{0u, 0u, 0u, 0u}, none, 0, 0, 0);
        }
        for (int j = cb; j < ce; ++j) step(j, op);
        if (ce > cb) {
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging has landed
            store_out(ce - 1);
        }
    }
}

// ------------------------------------------------------------------ phase 2, T form
// Per-head decay; fp16 activations, or bf16 converted to fp16 as they load
// (the prologue has handed pairs with values fp16 cannot hold to the
// recurrent kernel).  The chain forms the chunk's value
// updates from the raw rows instead of loading W and U: with the key rows
// against the incoming state, Y = K S^T, and Z = diag(beta) V - diag(w) Y,
//   D = U - W S^T = T Z,
// since U = T diag(beta) V and W = T diag(w) K (w = beta gamma / |k|).  The
// output waves form P from the q rows and the k rows that the chain waves
// park in LDS with the state tile (fp16 products, exact in fp32, scaled per
// element as the prologue of the W/U form scales them), and the chain waves
// gather the state update's K^T fragments from the same k rows (eight 16-bit
// LDS reads per fragment, issued after barrier 1 and consumed at stage E).
// The record holds T and the per-token scalars; k, v and q are read from the
// activations.  A chunk step has three barriers: the state tile and the k
// rows are in LDS (1), Z is (1.5, retrieving rules only), D is (2).  Workgroup layout, segments, tile scaling and the output path follow
// k_chunk_scan.
template <typename TA, int RULE, int NVB>
__global__ __launch_bounds__(512) void k_chunk_scan_t(const Params p, int32_t *off, const char *ws,
                                                     const ScanSeg sg)
{
    constexpr bool RET = rule_retrieves(RULE);
    constexpr int TR = 16 * NVB;          // state rows of this workgroup
    constexpr int NTILE = D128 / TR;      // workgroups per head
    // [hi, lo][row][key]: one buffer suffices, since every read of chunk j's
    // planes (B1, O1) precedes barrier 1.5 (or 2), which precedes their rewrite
    __shared__ __align__(16) half_t sS[2][TR][D128];
    __shared__ __align__(16) half_t sDt[2][2][TR][CH];   // [buffer][hi, lo][row][token]: D^T of chunk j in j & 1, Z^T in the other
    __shared__ __align__(16) half_t sDs[2][TR][CH];      // [hi, lo][row][token] (kd D)^T
    __shared__ __align__(16) half_t sKr[CH][D128];       // chunk j's k rows [token][key]: P's and (gathered) K^T's source
    __shared__ __align__(16) TA sO[4][16][TR + 8];       // per output wave: [token][row] staging for the store
    __shared__ float sTM[4][2];                           // per chain wave: max |S0| of its part, max |v|

    const int HV = p.HV;
    const int NU = (sg.pass == 1 ? 2 : 1) * NTILE;
    const int nsg = sg.pass == 0 ? 1 : sg.nseg - 1;
    const int gs = xcd_heads(p.H, HV, sg.pass);
    const int xl = blockIdx.x & 7, q8 = blockIdx.x >> 3, unit = q8 % NU, rest = q8 / NU;
    const int64_t gi = ((int64_t)(rest / gs) * 8 + xl) * gs + rest % gs;
    if (gi >= (int64_t)p.B * HV * nsg) return;
    // group -> (request, head): requests longest first (k_chunk_table's order)
    const int pr = (int)(gi / nsg), seg = (int)(gi % nsg) + (sg.pass == 2 ? 1 : 0);
    const int bh = off[p.B + 1 + (size_t)p.B * HV + pr / HV] * HV + pr % HV;
    const int tile = unit % NTILE;
    const int mode = sg.pass != 1 ? SEG_REAL : unit < NTILE ? (seg == 0 ? SEG_REAL : SEG_CARRY) : SEG_TRANS;
    if (mode == SEG_TRANS && seg == 0) return;
    const int b = bh / HV, h = bh % HV;
    if (off[p.B + 1 + bh]) return;  // the recurrent kernel takes this pair
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
    const int ns = sg.pass == 0 ? 1 : sg.nseg;
    const int cb = seg_lo(seg, nch, ns), ce = seg_lo(seg + 1, nch, ns);
    const float *from = src;
    float *const fin = sg.stage ? sg.stage + (size_t)bh * (D128 * D128) : dst;
    float *to = fin;
    if (sg.pass != 0) {
        float *xs = sg.xs + (size_t)bh * seg_slots(ns) * (D128 * D128);
        if (mode == SEG_REAL) {
            from = seg == 0 ? src : xs + (size_t)seg_start(seg) * (D128 * D128);
            to = seg == ns - 1 ? fin : seg == 0 ? xs + (size_t)seg_start(1) * (D128 * D128) : nullptr;
        } else {
            from = nullptr;
            to = xs + (size_t)(mode == SEG_CARRY ? seg_carry(ns, seg) : seg_trans(ns, seg)) * (D128 * D128);
        }
    }
    const int tb = wave & 3;
    const int qh = (int)(((int64_t)h * p.H) / HV);
    auto scale_exp = [&]() {
        const float ms = fmaxf(fmaxf(sTM[0][0], sTM[1][0]), fmaxf(sTM[2][0], sTM[3][0]));
        const float mv = fmaxf(fmaxf(sTM[0][1], sTM[1][1]), fmaxf(sTM[2][1], sTM[3][1]));
        return ce > cb ? tile_exponent(fmaxf(mode == SEG_TRANS ? 0.f : mv, ms)) : 0;
    };
    auto rec_of = [&](int jj) { return ws + ((size_t)(c0 + jj) * HV + h) * RecT::SIZE; };
    // chunk jj's rows of an activation with `heads` heads (head hh, columns c0 ..):
    // a resource over its valid tokens only, so rows past the request's end read zero
    const int tok_k = p.H * D128 * 2, tok_v = HV * D128 * 2;  // bytes from one token to the next
    auto act_rsrc = [&](const void *x, int heads, int hh, int col, int tok_bytes, int row_bytes, int jj) {
        const int64_t t0 = rs + (int64_t)jj * CH;
        const int n = (int)((re - t0) < CH ? (re - t0) : CH);
        const half_t *base = static_cast<const half_t *>(x) + ((size_t)t0 * heads + hh) * D128 + col;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t *>(base), 0, (n - 1) * tok_bytes + row_bytes,
                                                 0x00020000);
    };

    if (wave < 4) {
        // ================================================================ chain
        float mv = 0.f;
        for (int j = cb + tid; j < ce; j += 256) {
            const f4v m4 = *reinterpret_cast<const f4v *>(rec_of(j) + RecT::SC + SC_VMAX * 4);
            mv = fmaxf(mv, fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
        }
        // Sc[a][rt][i] = S[row0 + 16 rt + lr][16 (2 wave + a) + 4 lq + i]
        f4v Sc[2][NVB];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int rt = 0; rt < NVB; ++rt) {
                const int row = row0 + 16 * rt + lr, col = 16 * (2 * wave + a) + 4 * lq;
                if (from) {
                    Sc[a][rt] = *reinterpret_cast<const f4v *>(from + (size_t)row * D128 + col);
                } else {
                    const float one = mode == SEG_TRANS ? 1.f : 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) Sc[a][rt][i] = row == col + i ? one : 0.f;
                }
            }
        {
            float mx = 0.f;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(Sc[a][rt][i]));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                mx = fmaxf(mx, __shfl_xor(mx, o));
                mv = fmaxf(mv, __shfl_xor(mv, o));
            }
            if (lane == 0) {
                sTM[wave][0] = mx;
                sTM[wave][1] = mv;
            }
        }
        lds_barrier();  // 0: the tile's max |S0| is posted
        const int sx = scale_exp();
        const float up = ldexpf(1.f, sx), down = ldexpf(1.f, -sx);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int rt = 0; rt < NVB; ++rt) Sc[a][rt] *= up;
        const float um = mode == SEG_TRANS ? 0.f : up;  // a transition tile leaves V out
        ScanWatch sw;
        struct Ops {
            h8 k[4];        // k row 16 tb + lr, keys 32 kk + 8 lq .. +7
            h4 v[NVB];      // v at (tokens 16 tb + 4 lq + i, row 16 vb + lr)
            h8 kt[2][2];    // K^T fragments: key tiles 2 wave + a, token steps ks (from sKr)
            h8 th[2], tl[2];  // T (hi, lo): token 16 tb + lr, tokens 32 ks + 8 lq .. +7
            f4v kd, bt, rw;   // kd, beta and w of this lane's four D tokens 16 tb + 4 lq + i
            float gc;         // gamma_C
        };
        const uint32_t offK = (uint32_t)((16 * tb + lr) * tok_k + 2 * lk);
        const uint32_t offSc = RecT::SC + (uint32_t)(16 * tb + 4 * lq) * 4;
        auto fetchK = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = act_rsrc(p.k, p.H, qh, 0, tok_k, D128 * 2, jj);
            bool ok = true;  // exactness was checked by the prologue
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.k[kk] = to_h8(ld_b128<typename ActVec<TA>::v8>(r, offK + 64 * kk), ok);
        };
        // v in the layout of D's accumulators: four tokens of one row per lane
        auto fetchV = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = act_rsrc(p.v, HV, h, row0, tok_v, TR * 2, jj);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f.v[vb][i] = (half_t)to_f32(__builtin_bit_cast(TA, __builtin_amdgcn_raw_buffer_load_b16(
                                     r, (uint32_t)((16 * tb + 4 * lq + i) * tok_v + 2 * (16 * vb + lr)), 0, 0)));
        };
        auto fetchT = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(rec_of(jj), RecT::SIZE);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                // blocks above the diagonal are not stored: an offset past the record reads zero
                const uint32_t o = (tb < 2 && ks == 1) ? 0x7FFFF000u : RecT::T + (uint32_t)((tb * 2 + ks) * 2) * 1024 + l16;
                f.th[ks] = ld_b128<h8>(r, o);
                f.tl[ks] = ld_b128<h8>(r, o + 1024);
            }
        };
        auto fetchS = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(rec_of(jj), RecT::SIZE);
            f.kd = ld_b128<f4v>(r, offSc);
            if constexpr (RET) {
                f.bt = ld_b128<f4v>(r, offSc + SCT_BETA * 4);
                f.rw = ld_b128<f4v>(r, offSc + SCT_RW * 4);
            }
            f.gc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, RecT::SC + 2 * CH * 4, 0, 0));
        };
        // D at (tokens 16 bt + 4 lq + i, state row 16 vb + lr) -> D^T and (kd D)^T.
        // D^T takes the output waves' token order: within each 32-token step,
        // position 8 lq + 4 h + i holds token 16 h + 4 lq + i (the order in
        // which their P fragments come out of the matrix cores).
        auto put_d = [&](int bf, f4v dv, f4v kd, int bt, int vb) {
            f4v dsv;
#pragma unroll
            for (int i = 0; i < 4; ++i) dsv[i] = kd[i] * dv[i];
            const int r = 16 * vb + lr, c = 16 * bt + 4 * lq, cp = 32 * (bt >> 1) + 8 * lq + 4 * (bt & 1);
            h4 dh, dl, sh, sl;
            sw.note(dv);
            split4(dv, dh, dl);
            *reinterpret_cast<h4 *>(&sDt[bf][0][r][sw_tok(lr, cp)]) = dh;
            *reinterpret_cast<h4 *>(&sDt[bf][1][r][sw_tok(lr, cp)]) = dl;
            sw.note(dsv);
            split4(dsv, sh, sl);
            *reinterpret_cast<h4 *>(&sDs[0][r][sw_tok(lr, c)]) = sh;
            *reinterpret_cast<h4 *>(&sDs[1][r][sw_tok(lr, c)]) = sl;
        };
        auto step = [&](int j, Ops &cur) {
            const int bf = j & 1;
            const int jn = j + 1 < ce ? j + 1 : j;  // the last chunk re-reads itself
            // ---- A: state tile -> LDS (hi, lo)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt) {
                    h4 hi, lo;
                    sw.note(Sc[a][rt]);
                    split4(Sc[a][rt], hi, lo);
                    *reinterpret_cast<h4 *>(&sS[0][16 * rt + lr][sw_key(lr, 16 * (2 * wave + a) + 4 * lq)]) = hi;
                    *reinterpret_cast<h4 *>(&sS[1][16 * rt + lr][sw_key(lr, 16 * (2 * wave + a) + 4 * lq)]) = lo;
                }
            // the chunk's k rows: the output waves' P, and K^T for stage E
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) *reinterpret_cast<h8 *>(&sKr[16 * tb + lr][sw_key(lr, 32 * kk + lk)]) = cur.k[kk];
            lds_barrier();  // 1
            // K^T fragments (key 16 (2 wave + a) + lr, tokens 32 ks + 8 lq .. +7),
            // gathered from the k rows now, consumed at stage E
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const int t = 32 * ks + 8 * lq + x;
                        cur.kt[a][ks][x] = sKr[t][sw_key(t, 16 * (2 * wave + a) + lr)];
                    }
            if constexpr (RET) {
                // ---- B1: Y = K S^T at (tokens 16 tb + 4 lq + i, rows 16 vb + lr), then
                // Z = um beta V - w Y as Z^T into the free D buffer
                f4v y[NVB], yl[NVB];
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) y[vb] = yl[vb] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) {
                        const h8 shi = ld_h8(&sS[0][16 * vb + lr][sw_key(lr, 32 * kk + lk)]);
                        const h8 slo = ld_h8(&sS[1][16 * vb + lr][sw_key(lr, 32 * kk + lk)]);
                        y[vb] = mfma16(cur.k[kk], shi, y[vb]);
                        yl[vb] = mfma16(cur.k[kk], slo, yl[vb]);
                    }
                fetchK(jn, cur);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    f4v z;
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[i] = um * cur.bt[i] * (float)cur.v[vb][i] - cur.rw[i] * (y[vb][i] + yl[vb][i]);
                    h4 zh, zl;
                    sw.note(z);
                    split4(z, zh, zl);
                    const int r = 16 * vb + lr, c = 16 * tb + 4 * lq;
                    *reinterpret_cast<h4 *>(&sDt[bf ^ 1][0][r][sw_tok(lr, c)]) = zh;
                    *reinterpret_cast<h4 *>(&sDt[bf ^ 1][1][r][sw_tok(lr, c)]) = zl;
                }
                fetchV(jn, cur);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();  // 1.5
                // ---- B2: D = T Z; T is lower triangular, so token block tb reads
                // Z tokens 0 .. 16 tb + 15 (one token step for tb < 2)
                f4v d[NVB], dl[NVB];
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) d[vb] = dl[vb] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks == 1 && tb < 2) break;
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) {
                        const h8 zhi = ld_h8(&sDt[bf ^ 1][0][16 * vb + lr][sw_tok(lr, 32 * ks + lk)]);
                        const h8 zlo = ld_h8(&sDt[bf ^ 1][1][16 * vb + lr][sw_tok(lr, 32 * ks + lk)]);
                        d[vb] = mfma16(cur.th[ks], zhi, d[vb]);
                        dl[vb] = mfma16(cur.th[ks], zlo, dl[vb]);
                        dl[vb] = mfma16(cur.tl[ks], zhi, dl[vb]);
                    }
                }
                fetchT(jn, cur);
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) put_d(bf, d[vb] + dl[vb], cur.kd, tb, vb);
            } else {
                // no retrieval: D = V
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    f4v dv;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dv[i] = um * (float)cur.v[vb][i];
                    put_d(bf, dv, cur.kd, tb, vb);
                }
                fetchK(jn, cur);
                fetchV(jn, cur);
            }
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();  // 2
            // ---- E: S^T <- gamma_C S^T + K^T (kd D) for key tiles 2 wave + a, row blocks rt
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt) Sc[a][rt] *= cur.gc;
            {
                constexpr bool SEPL = NVB < 4;
                f4v lo4[2][NVB] = {};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int rt = 0; rt < NVB; ++rt) {
                        const h8 dhi = ld_h8(&sDs[0][16 * rt + lr][sw_tok(lr, 32 * ks + lk)]);
                        const h8 dlo = ld_h8(&sDs[1][16 * rt + lr][sw_tok(lr, 32 * ks + lk)]);
#pragma unroll
                        for (int a = 0; a < 2; ++a) {
                            Sc[a][rt] = mfma16(cur.kt[a][ks], dhi, Sc[a][rt]);
                            if constexpr (SEPL) lo4[a][rt] = mfma16(cur.kt[a][ks], dlo, lo4[a][rt]);
                            else Sc[a][rt] = mfma16(cur.kt[a][ks], dlo, Sc[a][rt]);
                        }
                    }
                }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int rt = 0; rt < NVB; ++rt)
                        if constexpr (SEPL) Sc[a][rt] += lo4[a][rt];
            }
            fetchS(jn, cur);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        };
        Ops op;
        if (ce > cb) {
            fetchK(cb, op);
            if constexpr (RET) fetchT(cb, op);
            fetchV(cb, op);
            fetchS(cb, op);
        }
        for (int j = cb; j < ce; ++j) step(j, op);
        if (to) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int rt = 0; rt < NVB; ++rt)
                    *reinterpret_cast<f4v *>(to + (size_t)(row0 + 16 * rt + lr) * D128 + 16 * (2 * wave + a) + 4 * lq) = Sc[a][rt] * down;
        }
        // a split operand at or past SPLIT_LIMIT hands the pair to the recurrent kernel
        if (sw.over()) off[p.B + 1 + bh] = 2;
    } else if (mode != SEG_REAL) {
        // carry and transition tiles write no output: these waves only keep
        // the chain's barriers (one at the start, two or three per chunk step)
        lds_barrier();  // 0
        for (int j = cb; j < ce; ++j) {
            lds_barrier();
            if constexpr (RET) lds_barrier();
            lds_barrier();
        }
    } else {
        // ================================================================ outputs
        TA *o = static_cast<TA *>(p.o);
        lds_barrier();  // 0
        const float down = ldexpf(1.f, -scale_exp());
        struct Ops {
            h8 q[4];          // q row 16 tb + lr, keys 32 kk + 8 lq .. +7
            float gq;         // gq of this lane's token t = 16 tb + lr
            float pg, pgl, pq;        // G_t (hi, lo) and scale / |q_t|
            f4v sg[4], sgl[4], sk[4];  // G_s (hi, lo) and 1 / |k_s| of tokens s = 16 sb + 4 lq + i
        };
        const uint32_t offQ = (uint32_t)((16 * tb + lr) * tok_k + 2 * lk);
        const int tok_bytes = HV * D128 * 2;
        static_assert(TR == 64 || TR == 32 || TR == 16, "the output transpose takes 16-, 32- or 64-row tiles");
        constexpr int LPT = TR / 8;
        constexpr int NST = TR == 64 ? 2 : 1;
        constexpr int TPS = 16 / NST;
        const bool st_live = lane / LPT < TPS;
        const int st_tok = st_live ? lane / LPT : TPS - 1, st_q = lane % LPT;
        const uint32_t offO = st_live ? (uint32_t)((16 * tb + st_tok) * tok_bytes + 16 * st_q) : 0x7FFFFFF0u;
        const uint32_t offG = RecT::SC + (uint32_t)(CH + 16 * tb + lr) * 4;
        const uint32_t offPt = RecT::SC + (uint32_t)(16 * tb + lr) * 4, offPs = RecT::SC + (uint32_t)(4 * lq) * 4;
        auto fetchQ = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = act_rsrc(p.q, p.H, qh, 0, tok_k, D128 * 2, jj);
            bool ok = true;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.q[kk] = to_h8(ld_b128<typename ActVec<TA>::v8>(r, offQ + 64 * kk), ok);
        };
        auto fetchG = [&](int jj, Ops &f) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(rec_of(jj), RecT::SIZE);
            f.gq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, offG, 0, 0));
            f.pg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, offPt + SCT_G * 4, 0, 0));
            f.pgl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, offPt + SCT_GL * 4, 0, 0));
            f.pq = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, offPt + SCT_QS * 4, 0, 0));
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                f.sg[sb] = ld_b128<f4v>(r, offPs + (SCT_G + 16 * sb) * 4);
                f.sgl[sb] = ld_b128<f4v>(r, offPs + (SCT_GL + 16 * sb) * 4);
                f.sk[sb] = ld_b128<f4v>(r, offPs + (SCT_IK + 16 * sb) * 4);
            }
        };
        auto store_out = [&](int jo) {
            const int64_t t0 = rs + (int64_t)jo * CH;
            const int n = jo >= cb ? (int)((re - t0) < CH ? (re - t0) : CH) : 0;
            TA *base = jo >= cb ? o + ((size_t)t0 * HV + h) * D128 + row0 : o;
            const __amdgpu_buffer_rsrc_t ro =
                __builtin_amdgcn_make_buffer_rsrc(base, 0, n > 0 ? (int)((n - 1) * tok_bytes + TR * 2) : 0, 0x00020000);
#pragma unroll
            for (int ps = 0; ps < NST; ++ps)
                __builtin_amdgcn_raw_buffer_store_b128(ld_b128_lds(&sO[tb][st_tok + TPS * ps][8 * st_q]), ro,
                                                       offO + (uint32_t)(TPS * ps * tok_bytes), 0, 0);
        };
        ScanWatch pw;
        auto step = [&](int j, Ops &cur) {
            const int bf = j & 1;
            const int jn = j + 1 < ce ? j + 1 : j;
            lds_barrier();  // 1
            store_out(j - 1);
            // ---- O1: O^T = S Q^T at (rows 16 vb + 4 lq + i, token 16 tb + lr)
            // (the state's hi plane only: O1 enters only the 16-bit outputs; the
            // W/U scan keeps both planes, where dropping the lo product measured
            // slower)
            f4v acc[NVB];
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) acc[vb] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    const h8 shi = ld_h8(&sS[0][16 * vb + lr][sw_key(lr, 32 * kk + lk)]);
                    acc[vb] = mfma16(shi, cur.q[kk], acc[vb]);
                }
            // ---- P_ts = scale / |q_t| / |k_s| exp(G_t - G_s) q_t . k_s (s <= t) from
            // the k rows the chain parked with the state tile and this wave's q
            // rows.  K Q^T at [s = 16 sb + 4 lq + i][t = 16 tb + lr] (fp16
            // products, exact in fp32) right after O1, where these waves would
            // wait for the chain at barrier 1.5; then, while the chain forms D,
            // the per-element factors and the (hi, lo) fragments whose element
            // 4 h + i of token step ks is token 32 ks + 16 h + 4 lq + i (the
            // order of D^T in LDS).  The k rows stay in LDS until the chain's
            // next stage A, after barrier 2.
            f4v c4[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                c4[sb] = f4v{0.f, 0.f, 0.f, 0.f};
                if (sb <= tb) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        c4[sb] = mfma16(ld_h8(&sKr[16 * sb + lr][sw_key(lr, 32 * kk + lk)]), cur.q[kk], c4[sb]);
                }
            }
            if constexpr (RET) lds_barrier();  // 1.5
            // the factors' exponentials stay below the barrier: their inputs pass
            // through an asm the compiler keeps after it (hoisted above it, they
            // made these waves late for it)
            asm volatile("" : "+v"(cur.pg), "+v"(cur.pgl));
            h8 ph[2];  // P enters only the 16-bit outputs: one fp16 plane
            {
                const int t = 16 * tb + lr;
                h4 hh[4];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    f4v pv;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int sx = 16 * sb + 4 * lq + i;
                        const float d2 = (cur.pg - cur.sg[sb][i]) + (cur.pgl - cur.sgl[sb][i]);
                        pv[i] = sx <= t ? cur.pq * cur.sk[sb][i] * ex2(d2) * c4[sb][i] : 0.f;
                    }
                    pw.note(pv);
                    hh[sb] = round_h4(pv);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) ph[ks] = __builtin_shufflevector(hh[2 * ks], hh[2 * ks + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            }
            fetchQ(jn, cur);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();  // 2
            // ---- O2: O^T = gq O^T + D^T P^T
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) acc[vb] = cur.gq * acc[vb];
            fetchG(jn, cur);
            // (the delta's hi plane only: this product enters only the 16-bit
            // outputs; the chain's state update keeps both planes)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks == 1 && tb < 2) break;  // P is zero there (tokens 32 .. 63 follow t)
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    const h8 dhi = ld_h8(&sDt[bf][0][16 * vb + lr][sw_tok(lr, 32 * ks + lk)]);
                    acc[vb] = mfma16(dhi, ph[ks], acc[vb]);
                }
            }
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                typename ActVec<TA>::v4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = from_f32<TA>(acc[vb][i] * down);
                *reinterpret_cast<typename ActVec<TA>::v4 *>(&sO[tb][lr][16 * vb + 4 * lq]) = ov;
            }
        };
        Ops op;
        if (ce > cb) {
            fetchQ(cb, op);
            fetchG(cb, op);
        }
        {
            const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(o, 0, 0, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b128(u4v{0u, 0u, 0u, 0u}, none, 0, 0, 0);
        }
        for (int j = cb; j < ce; ++j) step(j, op);
        if (ce > cb) {
            __builtin_amdgcn_s_waitcnt(0xc07f);
            store_out(ce - 1);
        }
        if (pw.over()) off[p.B + 1 + bh] = 2;  // P past the split range: the recurrent kernel takes the pair
    }
}

// ------------------------------------------------------------------ segment starts
// start_{p+1} = start_p M_p + c_p for the middle segments p = 1 .. nseg - 2,
// in order; rows are independent, so one workgroup takes 16 rows of one
// (request, head) and keeps them in LDS from one segment to the next.  The
// products run on the fp32 matrix cores (16x16x4: fp32 products and sums),
// wave w forming the output column blocks 2 w and 2 w + 1: lane (g, r) gives
// row r, k-index 4 ks + g of the rows and k-index 4 ks + g, column r of M at
// step ks, and holds result rows 4 g .. 4 g + 3 of column r.
__global__ __launch_bounds__(256) void k_seg_combine(const Params p, const int32_t *off, const ScanSeg sg)
{
    const int64_t bh = blockIdx.x >> 3;
    const int rb = blockIdx.x & 7;
    if (bh >= (int64_t)p.B * p.HV) return;
    if (off[p.B + 1 + bh]) return;  // the recurrent kernel takes this pair
    const float *src;
    float *dst;
    if (!state_ptrs(p, (int)(bh / p.HV), (int)(bh % p.HV), src, dst)) return;
    __shared__ float sR[16][D128 + 4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g4 = lane >> 4;
    constexpr size_t HEAD = (size_t)D128 * D128;
    float *xs = sg.xs + (size_t)bh * seg_slots(sg.nseg) * HEAD;
    const size_t rows = (size_t)(16 * rb) * D128;
    for (int i = tid; i < 16 * D128; i += 256) sR[i >> 7][i & 127] = xs[seg_start(1) * HEAD + rows + i];
    __syncthreads();
    for (int sp = 1; sp + 1 < sg.nseg; ++sp) {
        const float *M = xs + (size_t)seg_trans(sg.nseg, sp) * HEAD;
        const float *C = xs + (size_t)seg_carry(sg.nseg, sp) * HEAD + rows;
        f4v acc[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[cb][r] = C[(size_t)(4 * g4 + r) * D128 + 16 * (2 * wave + cb) + r16];
#pragma unroll 8
        for (int ks = 0; ks < D128 / 4; ++ks) {
            const float a = sR[r16][4 * ks + g4];
            const float *mrow = M + (size_t)(4 * ks + g4) * D128 + 32 * wave + r16;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, mrow[16 * cb], acc[cb], 0, 0, 0);
        }
        __syncthreads();  // every wave has read the old rows
        float *S = xs + (size_t)seg_start(sp + 1) * HEAD + rows;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g4 + r, col = 16 * (2 * wave + cb) + r16;
                sR[row][col] = acc[cb][r];
                S[(size_t)row * D128 + col] = acc[cb][r];
            }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ commit
// In-place states (a slab, or final == initial): copy each pair's staged final
// state to its place unless the pair went to the recurrent kernel (which
// wrote it from the intact incoming state).  One workgroup per pair.
__global__ __launch_bounds__(256) void k_chunk_commit(const Params p, const int32_t *off, const float *stage)
{
    const int64_t bh = blockIdx.x;
    if (bh >= (int64_t)p.B * p.HV || off[p.B + 1 + bh]) return;
    const float *src;
    float *dst;
    if (!state_ptrs(p, (int)(bh / p.HV), (int)(bh % p.HV), src, dst)) return;
    const f4v *from = reinterpret_cast<const f4v *>(stage + (size_t)bh * (D128 * D128));
    f4v *to = reinterpret_cast<f4v *>(dst);
#pragma unroll 4
    for (int i = threadIdx.x; i < D128 * D128 / 4; i += 256) to[i] = from[i];
}

// ------------------------------------------------------------------ host side

// The per-head form has two variants.  With a single-pass scan over 128 or
// more (request, head) pairs it takes the T form (k_chunk_prep<RULE, true>,
// k_chunk_scan_t): records of 18 KB per (chunk, value head) and no K^T area,
// instead of 81 KB plus 16 KB of K^T per (chunk, q/k head), at
// the price of one more product on the scan's serial chain per chunk and P
// formed by the output waves.  Measured on MI355X in one
// session: the varlen workload (8 requests, 32 heads) 0.974 -> 0.924 ms; the
// 65,536-token sequence (16 heads, 5 scan segments) 1.53 -> 1.65 ms (and
// 1.42 -> 1.56 ms once the T form formed P in its scan), so segmented and
// few-pair scans keep W and U in the records.
static bool t_form(bool per_key, int B, int HV, int nseg) { return !per_key && nseg <= 1 && (int64_t)B * HV >= 128; }

// Workspace: chunk table (off[B + 1], the (B * HV) hand-over flags, the scan
// order of the B requests) |
// records of every (chunk, value head) (Rec<true>, Rec<false> or RecT) |
// per-head W/U form: K^T of every (chunk, q/k head) |
// segment states | staging for in-place final states (one 128 x 128 fp32
// state per pair).  The chunk budget of gdr_chunk_plan.hpp sizes the
// records; the table never assigns a chunk index at or past it.
struct Layout {
    size_t kq, seg, stage, total;
};
static size_t table_bytes(int B, int HV) { return ((size_t)(B + 1) * 4 + (size_t)B * HV * 4 + (size_t)B * 4 + 255) / 256 * 256; }
static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

static Layout layout(int64_t T, int B, int H, int HV, bool per_key, int nseg)
{
    const int64_t maxch = chunk_budget(T, B);
    const bool tf = t_form(per_key, B, HV, nseg);
    const size_t rec = per_key ? Rec<true>::SIZE : tf ? RecT::SIZE : Rec<false>::SIZE;
    const size_t kq = per_key || tf ? 0 : KQ::SIZE;
    Layout l;
    l.kq = table_bytes(B, HV) + round256((size_t)maxch * HV * rec);
    l.seg = l.kq + round256((size_t)maxch * H * kq);
    l.stage = l.seg + (nseg > 1 ? (size_t)B * HV * seg_slots(nseg) * D128 * D128 * 4 : 0);
    l.total = l.stage + (size_t)B * HV * D128 * D128 * 4;
    return l;
}

static size_t workspace_bytes(int64_t T, int B, int H, int HV, bool per_key, int nseg)
{
    return layout(T, B, H, HV, per_key, nseg).total;
}

// Row tile of the scan: 16 * NVB rows, NVB = 1, 2 or 4 (launch_scans picks).
// TF: the per-head T form (fp16 activations).
template <typename TA, int RULE, int NVB, bool PK, bool TF>
static void launch_scan(const Params &p, int32_t *off, const char *rec, const char *kq, const ScanSeg &sg,
                        hipStream_t s)
{
    constexpr int NTILE = D128 / (16 * NVB);
    const int64_t groups = (int64_t)p.B * p.HV * (sg.pass == 0 ? 1 : sg.nseg - 1);
    const int64_t per = 8 * xcd_heads(p.H, p.HV, sg.pass);  // groups per round of the eight XCDs
    const int64_t blocks = (groups + per - 1) / per * per * NTILE * (sg.pass == 1 ? 2 : 1);
    if (blocks <= 0) return;
    if constexpr (TF)
        hipLaunchKernelGGL((k_chunk_scan_t<TA, RULE, NVB>), dim3((unsigned)blocks), dim3(512), 0, s, p, off, rec, sg);
    else
        hipLaunchKernelGGL((k_chunk_scan<TA, RULE, NVB, PK>), dim3((unsigned)blocks), dim3(512), 0, s, p, off, rec, kq,
                           sg);
}

// Scan launches.  Few (request, head) pairs leave most CUs idle with 32-row
// tiles; 16-row tiles double the workgroups and shorten each chunk step
// (measured on MI355X: one 65,536-token sequence x 16 heads 2.65 -> 2.18 ms),
// while with many pairs the GPU is full and the larger tiles amortise the
// operand reads (8 x 32 heads: 1.27 ms with 32-row tiles, 1.47 ms with 16-row
// tiles).  A chunk step is bound by the bytes of its operand reads (W, U,
// K^T, q and P: ~84 KB per 32-row tile; skipping the reloads of W alone took
// the varlen scan 479 -> 400 us), and W, K^T, q and P are the same for every
// row tile of a head, so from 128 pairs on (at least two 64-row workgroups
// per CU) the single pass takes 64-row tiles: varlen 8 x 32 heads 0.98 ->
// 0.94 ms, 4 x 32 heads per-key 0.99 -> 0.94 ms; with fewer pairs they leave
// CUs idle (16 heads in 4 segments: pass 2 398 -> 542 us).  A segmented scan
// runs pass 1 (carry and transition tiles: twice the workgroups of pass 2) in
// 32-row tiles and pass 2 by the same rule as a single pass over its
// (request, head, segment) groups: two workgroups of this kernel on one CU
// share its vector-memory pipeline and each chunk step then takes about twice
// as long (measured on MI355X, 65,536 tokens x 16 heads in 3 segments: 1.82 ms
// with 32-row pass-1 tiles, 1.89 ms with 16-row).  Pass 1 takes 64-row tiles
// when that gives 192 to 256 workgroups (one per CU on 3/4 of the chip or
// more), which then read each chunk's operands half as often: 65,536 tokens
// x 16 heads in 4 segments 1.75 -> 1.69 ms, in 5 segments 1.51 -> 1.50 ms;
// fewer (3 segments, 128 workgroups: 1.64 -> 1.97 ms) or more (6 segments,
// 320: 1.91 -> 2.07 ms) lose.
template <typename TA, int RULE, bool PK>
static void launch_scans(const Params &p, int32_t *off, const char *rec, const char *kq, float *xs, float *stage,
                         int nseg, hipStream_t s)
{
    const int64_t pairs = (int64_t)p.B * p.HV;
    if (nseg <= 1) {
        const ScanSeg one{1, 0, nullptr, stage};
        if (pairs <= 32) launch_scan<TA, RULE, 1, PK, false>(p, off, rec, kq, one, s);
        else if (pairs < 128) launch_scan<TA, RULE, 2, PK, false>(p, off, rec, kq, one, s);
        else if constexpr (PK) launch_scan<TA, RULE, 4, PK, false>(p, off, rec, kq, one, s);
        else launch_scan<TA, RULE, 4, PK, true>(p, off, rec, kq, one, s);  // the T form (t_form)
        return;
    }
    const int64_t pass1_64 = pairs * (nseg - 1) * 4;  // pass-1 workgroups in 64-row tiles
    if (pass1_64 >= 192 && pass1_64 <= 256)
        launch_scan<TA, RULE, 4, PK, false>(p, off, rec, kq, ScanSeg{nseg, 1, xs, stage}, s);
    else
        launch_scan<TA, RULE, 2, PK, false>(p, off, rec, kq, ScanSeg{nseg, 1, xs, stage}, s);
    if (nseg > 2) {
        const int64_t blocks = pairs * 8;
        hipLaunchKernelGGL(k_seg_combine, dim3((unsigned)blocks), dim3(256), 0, s, p, off, ScanSeg{nseg, 0, xs, stage});
    }
    if (pairs * (nseg - 1) <= 32) launch_scan<TA, RULE, 1, PK, false>(p, off, rec, kq, ScanSeg{nseg, 2, xs, stage}, s);
    else launch_scan<TA, RULE, 2, PK, false>(p, off, rec, kq, ScanSeg{nseg, 2, xs, stage}, s);
}

// PK: the per-key record and kernels; PKG: the gate itself is per key (else
// a per-head gate broadcast over the key channels).  The per-head form
// (PK = false) reads bf16 activations as fp16 (exact for values of magnitude
// 2^-17 to 65504; its prologue hands pairs with any other value to the
// recurrent kernel) and stores o in the activations' dtype.
template <typename TA, int RULE, bool PK, bool PKG>
static hipError_t launch_rule(const Params &p, int nseg, void *ws, hipStream_t s)
{
    const int64_t maxch = chunk_budget(p.T, p.B);
    char *base = static_cast<char *>(ws);
    int32_t *off = reinterpret_cast<int32_t *>(base);
    int32_t *redo = off + p.B + 1;
    const Layout l = layout(p.T, p.B, p.H, p.HV, PK, nseg);
    char *rec = base + table_bytes(p.B, p.HV);
    char *kq = base + l.kq;
    float *xs = reinterpret_cast<float *>(base + l.seg);
    // the incoming state is overwritten in place: stage the final states
    const bool in_place = p.num_slots > 0 || (p.init != nullptr && p.init == p.state);
    float *stage = in_place ? reinterpret_cast<float *>(base + l.stage) : nullptr;
    hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(256), 0, s, p, off, redo);
    if (maxch * p.HV > 0) {
        const dim3 grid((unsigned)((maxch + 7) / 8 * 8 * p.HV));
        if constexpr (PK)
            hipLaunchKernelGGL((k_chunk_prep_pk<TA, RULE, PKG>), grid, dim3(256), 0, s, p, off, rec);
        else if (t_form(PK, p.B, p.HV, nseg))
            hipLaunchKernelGGL((k_chunk_prep<TA, RULE, true>), grid, dim3(256), 0, s, p, off, rec, kq);
        else
            hipLaunchKernelGGL((k_chunk_prep<TA, RULE, false>), grid, dim3(256), 0, s, p, off, rec, kq);
    }
    launch_scans<TA, RULE, PK>(p, off, rec, kq, xs, stage, nseg, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // The recurrent kernel runs exactly the flagged pairs: requests the chunk
    // plan left out (ranges that overlap after a decreasing cu_seqlens entry)
    // and pairs whose split operands left the fp16 range.  With no flag set
    // its workgroups return at once.
    Params r = p;
    r.run_only = redo;
    err = launch_recurrent(r, RULE, PKG, std::is_same<TA, bf16_t>::value ? 2 : 1, D128, 2, s);
    if (err != hipSuccess) return err;
    if (stage && p.B * p.HV > 0)
        hipLaunchKernelGGL(k_chunk_commit, dim3((unsigned)(p.B * p.HV)), dim3(256), 0, s, p, off, stage);
    return hipGetLastError();
}

}  // namespace GDR_CHUNK_NS
}  // namespace gdr
