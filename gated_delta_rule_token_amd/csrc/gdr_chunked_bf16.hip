// gdr_chunked_bf16.hip -- chunk-parallel prefill for bf16 activations
// (kernels in gdr_chunked.hpp).  bf16 values are not all exact in fp16, so
// every rule takes the per-key form: its prologue widens q, k and v to fp32,
// forms the Gram blocks on the fp32 matrix cores, and hands the scan (hi, lo)
// fp16 planes of every fp32 operand; a per-head decay is broadcast over the
// key channels.  The scan stores o in bf16, rounded to nearest even.
#define GDR_CHUNK_NS bf16
#include "gdr_chunked.hpp"

namespace gdr {

hipError_t launch_chunked_bf16(const Params &p, int rule, bool per_key, int nseg, void *ws, hipStream_t s)
{
    using namespace bf16;
    switch (rule) {
    case LINEAR: return launch_rule<bf16_t, LINEAR, true, false>(p, nseg, ws, s);
    case DELTA: return launch_rule<bf16_t, DELTA, true, false>(p, nseg, ws, s);
    case GATED:
        return per_key ? launch_rule<bf16_t, GATED, true, true>(p, nseg, ws, s)
                       : launch_rule<bf16_t, GATED, true, false>(p, nseg, ws, s);
    case GATED_DELTA:
        return per_key ? launch_rule<bf16_t, GATED_DELTA, true, true>(p, nseg, ws, s)
                       : launch_rule<bf16_t, GATED_DELTA, true, false>(p, nseg, ws, s);
    default:
        return per_key ? launch_rule<bf16_t, GATED_DELTA_V2, true, true>(p, nseg, ws, s)
                       : launch_rule<bf16_t, GATED_DELTA_V2, true, false>(p, nseg, ws, s);
    }
}

}  // namespace gdr
