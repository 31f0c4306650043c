// gdr_stream.hip -- the state-traffic floor of a decode step over a slab of
// states: each addressed fp32 state matrix is read and written back in place,
// scaled by a factor, with no other work.  A measurement aid that sits beside
// the decode kernel; it computes nothing of the method.  A request's states
// (every head of its slot) are one contiguous row of the slab; requests in
// order, block -> (request, piece of the row); each wave streams one
// contiguous 32 KB span (64 lanes x 32 16-byte vectors, lane l taking
// vectors l + 64 i), four waves per workgroup, non-temporal loads and stores.  Of the plain in-place
// copies measured on MI355X over randomly placed 2 MiB slots, longer
// contiguous spans per wave ran faster: 16 KB per workgroup with the vectors
// of its four waves interleaved 192 us per 1 GiB, 16 KB per wave 182 us,
// 32 KB per wave 176 us.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

typedef float f4s __attribute__((ext_vector_type(4)));
constexpr int STREAM_WAVES = 4, STREAM_VECS = 32;
constexpr int64_t STREAM_SPAN = 64 * STREAM_VECS;                 // 16-byte vectors per wave
constexpr int64_t STREAM_PIECE = STREAM_WAVES * STREAM_SPAN;      // per workgroup

// row4: 16-byte vectors per slot row (heads x matrix floats / 4)
__global__ __launch_bounds__(64 * STREAM_WAVES) void k_slab_stream(f4s *slab, const int32_t *__restrict__ slot_ids,
                                                                   int64_t row4, int64_t pieces, int num_slots,
                                                                   float factor)
{
    const int b = (int)((int64_t)blockIdx.x / pieces);
    const int64_t piece = (int64_t)blockIdx.x % pieces;
    const int slot = slot_ids[b];
    if (slot < 0 || slot >= num_slots) return;  // as in the decode kernel: the request is skipped
    f4s *base = slab + (int64_t)slot * row4;
    const int64_t i0 = piece * STREAM_PIECE + (int64_t)(threadIdx.x >> 6) * STREAM_SPAN + (threadIdx.x & 63);
    f4s r[STREAM_VECS];
#pragma unroll
    for (int i = 0; i < STREAM_VECS; ++i) {
        const int64_t at = i0 + 64 * i;
        r[i] = at < row4 ? __builtin_nontemporal_load(base + at) : f4s{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < STREAM_VECS; ++i) {
        const int64_t at = i0 + 64 * i;
        if (at < row4) __builtin_nontemporal_store(r[i] * factor, base + at);
    }
}

int64_t slab_stream_blocks(int batch, int heads, int64_t matrix)
{
    return (int64_t)batch * (((int64_t)heads * matrix / 4 + STREAM_PIECE - 1) / STREAM_PIECE);
}

// matrix: floats per state matrix (a multiple of 4); the caller checks the
// arguments and that slab_stream_blocks fits one launch.
hipError_t launch_slab_stream(float *slab, const int32_t *slot_ids, int batch, int heads, int64_t matrix,
                              int num_slots, float factor, hipStream_t s)
{
    if (batch == 0) return hipSuccess;
    const int64_t row4 = (int64_t)heads * matrix / 4, pieces = (row4 + STREAM_PIECE - 1) / STREAM_PIECE;
    hipLaunchKernelGGL(k_slab_stream, dim3((unsigned)slab_stream_blocks(batch, heads, matrix)),
                       dim3(64 * STREAM_WAVES), 0, s, reinterpret_cast<f4s *>(slab), slot_ids, row4, pieces,
                       num_slots, factor);
    return hipGetLastError();
}

}  // namespace gdr
