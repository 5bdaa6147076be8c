// The plain backward with its row term in library-owned device memory, for
// callers that cannot allocate: code under HIP graph capture, tight serving
// loops, harnesses that forbid device allocation.  Same kernels as
// s2attn_bwd; the only difference is where the row term -rowsum(dout * o)
// lives between the row-term kernel and the gradient kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "s2_params.h"
#include "s2attn.h"

namespace {

// Row-term floats the array holds: B * Hq * L at most (32 MiB of fp32 per GPU,
// kept until the process ends).
constexpr size_t kNoallocRows = S2ATTN_NOALLOC_MAX_ROWS;
static_assert(kNoallocRows == ((size_t)1 << 23), "header and library agree on the bound");

static __device__ __align__(256) float scratch[kNoallocRows];

// Device address of `scratch` on each GPU, taken once per device with that
// device current.  In host code the array's name stands for a host-side
// symbol, not a device address, so only these addresses are ever passed on.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_scratch[kMaxDevices] = {};

int scratch_on_current_device(float** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return S2ATTN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return S2ATTN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return S2ATTN_ERR_HIP;
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return S2ATTN_OK;
}

}  // namespace

extern "C" int s2attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk,
                                  void* dv, int B, int L, int Hq, int Hkv, int d, int G,
                                  int shifted_heads, hipStream_t stream) {
    // Host checks first (no HIP call before them), then the size bound.
    int st = s2::bwd_plain(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, L, Hq, Hkv, d, G,
                           shifted_heads, stream, 0);
    if (st != S2ATTN_OK) return st;
    if ((size_t)B * (size_t)Hq * (size_t)L > kNoallocRows) return S2ATTN_ERR_WORKSPACE;
    float* rows = nullptr;
    st = scratch_on_current_device(&rows);
    if (st != S2ATTN_OK) return st;
    // Every element the gradient kernels read is written first by the
    // row-term kernel of this call, so nothing needs clearing.
    return s2::bwd_plain(q, k, v, o, lse, dout, dq, dk, dv, rows, B, L, Hq, Hkv, d, G,
                         shifted_heads, stream, 1);
}
