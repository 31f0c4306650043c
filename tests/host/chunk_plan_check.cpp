// Host build of the chunked prefill's chunk plan (gdr_chunk_plan.hpp), in the
// order the chunk-table kernel computes it: blocks of 256 requests, an
// inclusive prefix sum inside each block plus the running carry, the largest
// granted prefix, then off[] capped at it.  Reads cases from stdin
//   T B  cu[0] .. cu[B]
// and prints, per case, "off[0..B] | denied[0..B-1] | owner of every chunk".
// Compiled with g++ by tests/test_chunk_plan.py (no GPU involved).
#define GDR_HD
#include "gdr_chunk_plan.hpp"

#include <cstdio>
#include <vector>

int main()
{
    long long T;
    int B;
    while (std::scanf("%lld %d", &T, &B) == 2) {
        std::vector<long long> cu(B + 1);
        for (int i = 0; i <= B; ++i) std::scanf("%lld", &cu[i]);
        const long long budget = gdr::chunk_budget(T, B);
        std::vector<long long> off(B + 1, 0);
        std::vector<int> denied(B, 0);
        long long carry = 0, best = 0;
        for (int base = 0; base < B; base += 256) {
            long long s[256];
            for (int tid = 0; tid < 256; ++tid) {
                const int b = base + tid;
                long long n = 0;
                if (b < B) {
                    int64_t st, en;
                    gdr::clamp_request(cu[b], cu[b + 1], T, st, en);
                    n = gdr::request_chunks(st, en);
                }
                s[tid] = n;
            }
            long long incl[256], run = 0;
            for (int tid = 0; tid < 256; ++tid) incl[tid] = (run += s[tid]);
            for (int tid = 0; tid < 256; ++tid) {
                const int b = base + tid;
                if (b >= B) continue;
                const long long n = s[tid], excl = carry + incl[tid] - n;
                off[b] = excl < budget + 1 ? excl : budget + 1;
                denied[b] = gdr::chunk_denied(excl, n, budget) ? 1 : 0;
                if (gdr::chunk_granted(excl, n, budget) && excl + n > best) best = excl + n;
            }
            carry += incl[255];
        }
        for (int b = 0; b < B; ++b) off[b] = gdr::chunk_offset(off[b], best);
        off[B] = gdr::chunk_offset(carry, best);
        std::printf("%lld", budget);
        for (int b = 0; b <= B; ++b) std::printf(" %lld", off[b]);
        std::printf(" |");
        for (int b = 0; b < B; ++b) std::printf(" %d", denied[b]);
        std::printf("\n");
    }
    return 0;
}
