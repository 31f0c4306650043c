// gdr_gate.hip -- standalone gate fusion ("com.microsoft.LinearAttentionGate",
// Description): decay = decay_scale[h] * softplus(a + dt_bias[h]) and,
// when requested, beta = sigmoid(b); fp32 arithmetic, narrowed on store.
// The head axis is the last one, so h = n % heads.  Memory-bound and
// elementwise: a grid-stride loop over the flattened elements.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <typename T>
__global__ __launch_bounds__(256) void k_gate(int64_t count, int heads, const T *__restrict__ a,
                                              const float *__restrict__ dt_bias,
                                              const float *__restrict__ decay_scale,
                                              const T *__restrict__ b, T *__restrict__ decay,
                                              T *__restrict__ beta)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < count; n += stride) {
        const int h = (int)(n % heads);
        decay[n] = from_f32<T>(decay_scale[h] * softplus_f32(to_f32(a[n]) + dt_bias[h]));
        if (beta) beta[n] = from_f32<T>(sigmoid_f32(to_f32(b[n])));
    }
}

hipError_t launch_gate(int64_t count, int heads, bool f16, const void *a, const float *dt_bias,
                       const float *decay_scale, const void *b, void *decay, void *beta, hipStream_t s)
{
    if (count == 0) return hipSuccess;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (f16)
        hipLaunchKernelGGL(k_gate<half_t>, dim3((unsigned)blocks), dim3(256), 0, s, count, heads,
                           static_cast<const half_t *>(a), dt_bias, decay_scale,
                           static_cast<const half_t *>(b), static_cast<half_t *>(decay),
                           static_cast<half_t *>(beta));
    else
        hipLaunchKernelGGL(k_gate<float>, dim3((unsigned)blocks), dim3(256), 0, s, count, heads,
                           static_cast<const float *>(a), dt_bias, decay_scale,
                           static_cast<const float *>(b), static_cast<float *>(decay),
                           static_cast<float *>(beta));
    return hipGetLastError();
}

}  // namespace gdr
