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

template <typename T>
static void launch_typed(int64_t count, int heads, const void *a, const float *dt_bias, const float *decay_scale,
                         const void *b, void *decay, void *beta, hipStream_t s)
{
    int64_t blocks = (count + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_gate<T>, dim3((unsigned)blocks), dim3(256), 0, s, count, heads,
                       static_cast<const T *>(a), dt_bias, decay_scale, static_cast<const T *>(b),
                       static_cast<T *>(decay), static_cast<T *>(beta));
}

hipError_t launch_gate(int64_t count, int heads, int dtype, const void *a, const float *dt_bias,
                       const float *decay_scale, const void *b, void *decay, void *beta, hipStream_t s)
{
    if (count == 0) return hipSuccess;
    if (dtype == 1) launch_typed<half_t>(count, heads, a, dt_bias, decay_scale, b, decay, beta, s);
    else if (dtype == 2) launch_typed<bf16_t>(count, heads, a, dt_bias, decay_scale, b, decay, beta, s);
    else launch_typed<float>(count, heads, a, dt_bias, decay_scale, b, decay, beta, s);
    return hipGetLastError();
}

}  // namespace gdr
