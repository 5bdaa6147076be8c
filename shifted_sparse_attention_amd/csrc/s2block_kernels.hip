// Elementwise helpers of the attention block.
#include "s2_device.h"
#include "s2block_kernels.h"

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

namespace s2 {

// dst[r, dcol0 + c] = src[r, c] (bf16), for r < rows, c < cols, 16 bytes per
// thread; when src is null the block is filled with zeros.  Strides and
// column offsets are in elements and multiples of 8 (16-byte aligned rows).
__global__ __launch_bounds__(256) void copy_cols_kernel(const bf16* __restrict__ src, long src_ld,
                                                        bf16* __restrict__ dst, long dst_ld,
                                                        long rows, int chunks_per_row) {
    const long n = rows * chunks_per_row;
    for (long i = blockIdx.x * (long)256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        const long r = i / chunks_per_row;
        const int c = (int)(i % chunks_per_row) * 8;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (src) v = *reinterpret_cast<const u32x4*>(src + r * src_ld + c);
        *reinterpret_cast<u32x4*>(dst + r * dst_ld + c) = v;
    }
}

hipError_t launch_copy_cols(const void* src, long src_ld, void* dst, long dst_ld, long rows,
                            long cols, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const long chunks = cols / 8;
    long blocks = (rows * chunks + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(copy_cols_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const bf16*>(src), src_ld, static_cast<bf16*>(dst), dst_ld,
                       rows, (int)chunks);
    return hipGetLastError();
}

}  // namespace s2
