// Launch parameters passed by value to every S2-Attn kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "s2attn.h"

namespace s2 {

struct Params {
    // Tensors.  Element types follow the dtype fields of the launcher.
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;   // [B, Hq, L] -rowsum(dout * o)
    // dS tiles of the backward (null: dQ recomputes S and dP).  For unit
    // (b, h, g), tile (q32, k32) with k32 <= q32 < T = ceil(G/32) holds dS of
    // queries 32 q32 .. +31 against keys 32 k32 .. +31, 2 KB.  Query rows go
    // in blocks of 8 (t = q32 / 8), each block stored k32-major over its
    // 8 (t + 1) key tiles: tile (q32, k32) is number 32 t (t + 1) + 8 k32 +
    // q32 % 8 of the unit, whose UT = 32 NB (NB + 1) tiles (NB = ceil(T / 8))
    // start at tile ((b Hq + h) n_g + g) UT.  So the 8 rows one dQ
    // workgroup reads advance through consecutive memory.  Within a tile,
    // the four bf16 of key r (0..31) and query quad c (queries 4c .. 4c+3)
    // sit at byte 1024 (c >> 2) + 16 (r + 32 (c & 1)) + 8 ((c >> 1) & 1): the
    // order the dK/dV kernel holds them in registers.
    void* ds;
    // Sizes.
    int B, L, Hq, Hkv, d, G, shifted_heads;
    int r;          // Hq / Hkv
    int n_g;        // L / G
    float scale;    // softmax scale
    float scale_log2;  // scale * log2(e)
    // RoPE with position interpolation: angle = t * pos_scale * rope_base^(-2c/d), with
    // pos_scale = L0 / L.  rope_rev[c] is that angle per unit of t, in revolutions
    // (divided by 2 pi), formed in double precision on the host.  With rope set,
    // the bf16 forward rotates its query fragments (k comes pre-rotated) and the
    // backward epilogues rotate dq, dk back (q and k come pre-rotated).
    int rope;
    double rope_rev[64];
    // Units per dispatch band of the tiled kernels (see decode_work; >= 1).
    int band;
};

// Dispatch band for a kernel whose workgroups of one unit re-read
// `reuse_bytes` (K and V, K alone, or Q and dO): as many units as keep the
// bands of the 8 XCDs within the 256 MB last-level cache (32 MiB per XCD),
// at least 1 and at most the units of one XCD.  Measured at 8k-100k tokens,
// wider bands than that lose (more misses), narrower ones leave the tail of
// few-tile units and a less even memory stream.
inline int dispatch_band(int n_units, size_t reuse_bytes) {
    const size_t budget = (size_t)32 << 20;
    const size_t upx = (size_t)(n_units / 8);
    size_t band = reuse_bytes > 0 ? budget / reuse_bytes : 1;
    if (band > upx) band = upx;
    return band < 1 ? 1 : (int)band;
}

// Head shift: half a group for the last `shifted_heads` query heads.
__host__ __device__ inline int head_shift(const Params& p, int h) {
    return h >= p.Hq - p.shifted_heads ? p.G / 2 : 0;
}

// Row strides (in elements) of the [B, L, H, d] layouts.
__host__ __device__ inline size_t q_row(const Params& p, int b, int t, int h) {
    return ((size_t)(b * (size_t)p.L + t) * p.Hq + h) * p.d;
}
__host__ __device__ inline size_t kv_row(const Params& p, int b, int t, int h) {
    return ((size_t)(b * (size_t)p.L + t) * p.Hkv + h) * p.d;
}
__host__ __device__ inline size_t lse_idx(const Params& p, int b, int h, int t) {
    return ((size_t)b * p.Hq + h) * p.L + t;
}

// Launchers (one per kernel family).  Return hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const Params& p, hipStream_t s);
hipError_t launch_fwd_f32(const Params& p, hipStream_t s);
hipError_t launch_bwd_pre(const Params& p, int f32_io, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const Params& p, int grad_f32, int split, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const Params& p, int grad_f32, hipStream_t s);
hipError_t launch_bwd_dq_ds_bf16(const Params& p, int grad_f32, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const Params& p, hipStream_t s);
hipError_t launch_bwd_dq_f32(const Params& p, hipStream_t s);
// Rotated q into q_out (skipped when q_out is null) and rotated k into k_out.
hipError_t launch_rope_prepass(const Params& p, void* q_out, void* k_out, hipStream_t s);

// The plain backward (s2attn_bwd) with the row term in `delta`; with launch = 0
// only its host checks run (delta may then be null) and nothing is enqueued.
int bwd_plain(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int L, int Hq,
              int Hkv, int d, int G, int shifted_heads, hipStream_t stream, int launch);

// The checks s2attn_fwd_ex (is_bwd = 0) or s2attn_bwd_ex (is_bwd = 1) run on
// their sizes and options, without pointers: for callers that must validate
// a whole sequence of work before enqueueing any of it.
int attention_config_status(int is_bwd, int B, int L, int Hq, int Hkv, int d, int G,
                            int shifted_heads, const s2attn_opts* opts);

}  // namespace s2
