// Elementwise helpers of the attention block.
#include "s2_device.h"
#include "s2block_kernels.h"

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
