// gdr_chunked_bf16.hip -- chunk-parallel prefill for bf16 activations
// (kernels in gdr_chunked.hpp).  A per-head decay takes the per-head form,
// whose kernels convert q, k and v to fp16 as they load them (exact for
// values of magnitude 2^-17 to 65504; the prologue hands a (request, head)
// pair with any other value to the recurrent kernel).  A decay per key
// channel and the erase gate take the per-key form, whose prologue widens q,
// k and v to fp32 and hands the scan (hi, lo) fp16 planes of every fp32
// operand.  Both store o in bf16, rounded to nearest even.
#define GDR_CHUNK_NS bf16
#include "gdr_chunked.hpp"

namespace gdr {

hipError_t launch_chunked_bf16(const Params &p, int rule, bool per_key, int nseg, void *ws, hipStream_t s)
{
    using namespace bf16;
    switch (rule) {
    case LINEAR: return launch_rule<bf16_t, LINEAR, false, false>(p, nseg, ws, s);
    case DELTA: return launch_rule<bf16_t, DELTA, false, false>(p, nseg, ws, s);
    case GATED:
        return per_key ? launch_rule<bf16_t, GATED, true, true>(p, nseg, ws, s)
                       : launch_rule<bf16_t, GATED, false, false>(p, nseg, ws, s);
    case GATED_DELTA:
        return per_key ? launch_rule<bf16_t, GATED_DELTA, true, true>(p, nseg, ws, s)
                       : launch_rule<bf16_t, GATED_DELTA, false, false>(p, nseg, ws, s);
    default:
        return per_key ? launch_rule<bf16_t, GATED_DELTA_V2, true, true>(p, nseg, ws, s)
                       : launch_rule<bf16_t, GATED_DELTA_V2, true, false>(p, nseg, ws, s);
    }
}

}  // namespace gdr
