// gdr_chunked.hip -- chunk-parallel prefill for fp16 activations, and the
// entry points of the chunked form (the kernels are in gdr_chunked.hpp; bf16
// activations are instantiated in gdr_chunked_bf16.hip).
#define GDR_CHUNK_NS f16
#include "gdr_chunked.hpp"

namespace gdr {

size_t chunked_workspace_bytes(int64_t T, int B, int H, int HV, bool per_key, int nseg)
{
    return f16::workspace_bytes(T, B, H, HV, per_key, nseg);
}

// A decay per key channel and the erase gate take the per-key form; other
// scalar-decay rules the per-head form.
hipError_t launch_chunked(const Params &p, int rule, bool per_key, int nseg, int act, void *ws, hipStream_t s)
{
    using namespace f16;
    if (act == 2) return launch_chunked_bf16(p, rule, per_key, nseg, ws, s);
    if (rule == GATED_DELTA_V2)
        return per_key ? launch_rule<half_t, GATED_DELTA_V2, true, true>(p, nseg, ws, s)
                       : launch_rule<half_t, GATED_DELTA_V2, true, false>(p, nseg, ws, s);
    if (per_key)
        return rule == GATED ? launch_rule<half_t, GATED, true, true>(p, nseg, ws, s)
                             : launch_rule<half_t, GATED_DELTA, true, true>(p, nseg, ws, s);
    switch (rule) {
    case LINEAR: return launch_rule<half_t, LINEAR, false, false>(p, nseg, ws, s);
    case GATED: return launch_rule<half_t, GATED, false, false>(p, nseg, ws, s);
    case DELTA: return launch_rule<half_t, DELTA, false, false>(p, nseg, ws, s);
    default: return launch_rule<half_t, GATED_DELTA, false, false>(p, nseg, ws, s);
    }
}

}  // namespace gdr
