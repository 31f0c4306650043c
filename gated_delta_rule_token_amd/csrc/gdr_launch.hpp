// gdr_launch.hpp -- host-side launchers of the gated delta-rule kernels
// (internal to libgdr; the public surface is include/gdr.h).
#pragma once

#include <hip/hip_runtime.h>

#include "gdr_device.hpp"

namespace gdr {

// Recurrent kernel: dkt in {32, 64, 128, 256} (>= dk), g in {1, 2, 4}
// (rows per workgroup = 16 * g).
hipError_t launch_recurrent(const Params &p, int rule, bool per_key, int act, int dkt, int g, hipStream_t s);

// Decode kernel, dk = dv = 128 only.
hipError_t launch_decode128(const Params &p, int rule, bool per_key, int act, hipStream_t s);

// Chunk-parallel prefill (chunk 64, dk = dv = 128, fp16 or bf16 activations,
// act = 1 or 2); the per-key form serves a decay per key channel and the
// erase gate (per_key here: the gate itself is per key).
// nseg > 1 cuts each request's chain of chunk steps into that many segments
// (two scan passes and a combine step).  `ws` holds
// chunked_workspace_bytes(T, B, H, HV, per-key form, nseg) bytes.
size_t chunked_workspace_bytes(int64_t T, int B, int H, int HV, bool per_key_form, int nseg);
hipError_t launch_chunked(const Params &p, int rule, bool per_key, int nseg, int act, void *ws, hipStream_t s);
hipError_t launch_chunked_bf16(const Params &p, int rule, bool per_key, int nseg, void *ws, hipStream_t s);

// Standalone gate fusion.
hipError_t launch_gate(int64_t count, int heads, int dtype, const void *a, const float *dt_bias,
                       const float *decay_scale, const void *b, void *decay, void *beta, hipStream_t s);
// gdr_stream.hip: read and rewrite, scaled, the state matrices slab[slot_ids[b], h]
int64_t slab_stream_blocks(int batch, int heads, int64_t matrix);
hipError_t launch_slab_stream(float *slab, const int32_t *slot_ids, int batch, int heads, int64_t matrix,
                              int num_slots, float factor, hipStream_t s);

}  // namespace gdr
