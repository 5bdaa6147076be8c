// Elementwise helpers of the attention block (s2block_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace s2 {

// Copy a rows x cols bf16 block between row-major matrices (zeros when src is
// null); cols, strides and the pointers' element offsets are multiples of 8.
hipError_t launch_copy_cols(const void* src, long src_ld, void* dst, long dst_ld, long rows,
                            long cols, hipStream_t s);

}  // namespace s2
