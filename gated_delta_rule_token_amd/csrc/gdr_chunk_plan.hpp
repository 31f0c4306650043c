// gdr_chunk_plan.hpp -- which requests of a call the chunked prefill takes.
//
// Request b covers tokens [clamp(cu[b], 0, T), max(that, clamp(cu[b+1], 0, T)))
// ("com.microsoft.GatedDeltaNet" README, Inputs cu_seqlens: a decreasing or
// out-of-range entry gives an empty request, never an out-of-bounds read).
// Clamped ranges of a monotone cu_seqlens tile [0, T), so their chunk counts
// ceil(len / 64) sum to at most ceil(T / 64) + B: the budget that sizes the
// chunk records and the prologue grid.  A non-monotone cu_seqlens can make a
// later request start again from an earlier token, so the ranges overlap and
// the sum can reach B * ceil(T / 64).  The plan therefore grants chunks to
// requests in order while the running total stays within the budget; the
// first request that would pass it, and every request after it, get none and
// are marked for the recurrent kernel, which needs no workspace.  For a
// monotone cu_seqlens (and for uniform packing) every request is granted.
//
// With excl = chunks of the requests before b (uncapped) and n = b's chunks:
//   granted(b)  <=>  excl + n <= budget
//   best        =    the largest excl + n of a granted request (0 if none)
//   off[b]      =    min(excl, best)            (off[B] = min(total, best))
// so off[] is non-decreasing, off[B] <= budget, a granted request owns
// chunks [off[b], off[b] + n) and a denied one owns none.
//
// These functions are compiled for the device (the chunk-table kernel) and,
// with GDR_HD defined empty before inclusion, for a host check.
#pragma once

#include <stdint.h>

#ifndef GDR_HD
#define GDR_HD __host__ __device__
#endif

namespace gdr {

constexpr int CHUNK_LEN = 64;

GDR_HD inline void clamp_request(int64_t a, int64_t z, int64_t T, int64_t &s, int64_t &e)
{
    a = a < 0 ? 0 : (a > T ? T : a);
    z = z < 0 ? 0 : (z > T ? T : z);
    s = a;
    e = z > a ? z : a;
}

GDR_HD inline int64_t chunk_budget(int64_t T, int64_t B) { return (T + CHUNK_LEN - 1) / CHUNK_LEN + B; }

GDR_HD inline int64_t request_chunks(int64_t s, int64_t e) { return (e - s + CHUNK_LEN - 1) / CHUNK_LEN; }

GDR_HD inline bool chunk_granted(int64_t excl, int64_t n, int64_t budget) { return excl + n <= budget; }

GDR_HD inline int32_t chunk_offset(int64_t excl, int64_t best) { return (int32_t)(excl < best ? excl : best); }

// A request the chunked kernels leave to the recurrent kernel: it has tokens
// but was not granted its chunks.
GDR_HD inline bool chunk_denied(int64_t excl, int64_t n, int64_t budget) { return n > 0 && !chunk_granted(excl, n, budget); }

}  // namespace gdr
