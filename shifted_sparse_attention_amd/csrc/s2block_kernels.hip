// Elementwise helpers of the attention block.
#include "s2_device.h"

namespace s2 {

// 8 floats -> 8 bf16 (round to nearest even) per thread, grid-stride.
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ in,
                                                          bf16* __restrict__ out, size_t n8) {
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
        const f32x4 a = reinterpret_cast<const f32x4*>(in)[2 * i];
        const f32x4 b = reinterpret_cast<const f32x4*>(in)[2 * i + 1];
        bf16x8 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = (bf16)a[e];
            r[4 + e] = (bf16)b[e];
        }
        reinterpret_cast<bf16x8*>(out)[i] = r;
    }
}

__global__ void f32_to_bf16_tail_kernel(const float* __restrict__ in, bf16* __restrict__ out,
                                        size_t start, size_t n) {
    const size_t i = start + threadIdx.x;
    if (i < n) out[i] = (bf16)in[i];
}

hipError_t launch_f32_to_bf16(const float* in, void* out, size_t n, hipStream_t s) {
    const size_t n8 = n / 8;
    bf16* o = static_cast<bf16*>(out);
    if (n8 > 0) {
        size_t blocks = (n8 + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, in, o, n8);
    }
    if (n % 8) hipLaunchKernelGGL(f32_to_bf16_tail_kernel, dim3(1), dim3(8), 0, s, in, o, n8 * 8, n);
    return hipGetLastError();
}

}  // namespace s2
