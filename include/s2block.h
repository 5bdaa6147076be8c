/*
 * s2block: one Llama-style attention block around S2-Attn, as LongLoRA
 * fine-tunes it on MI355X (gfx950).
 *
 *   y = A(x) Wo^T + s (A(x) Ao^T) Bo^T,   A = S2-Attn with RoPE-PI on
 *   q = x Wq^T + s (x Aq^T) Bq^T,  k, v likewise,
 *
 * with frozen projection weights W and trainable LoRA factors A (down, r
 * rows) and B (up, r columns) on the Q, K, V and O projections (LongLoRA
 * blog, section 3.2: LoRA on the Q, K, V, O projections; section 3.4:
 * position interpolation; section 3.3: shift short attention).  The
 * backward returns dx and the LoRA gradients (W is frozen: no dW).
 *
 * The projection GEMMs are plain library GEMMs (hipBLASLt, bf16 inputs,
 * fp32 accumulation); attention runs in libs2attn's kernels.
 *
 * Conventions (as for s2attn.h):
 *   - all pointers are device memory owned by the caller, 16-byte aligned,
 *     row-major and contiguous; outputs must not alias inputs;
 *   - x, y, dx: [B, L, Dm] bf16 with Dm = Hq * d; q, attn: [B, L, Hq, d];
 *     k, v: [B, L, Hkv, d]; lse: [B, Hq, L] fp32;
 *   - Wq: [Hq d, Dm], Wk, Wv: [Hkv d, Dm], Wo: [Dm, Hq d];
 *     Aq, Ak, Av: [r, Dm], Ao: [r, Hq d]; Bq: [Hq d, r], Bk, Bv: [Hkv d, r],
 *     Bo: [Dm, r]; all bf16;
 *   - LoRA gradients are fp32 with the shapes of their factors;
 *   - calls only enqueue work on `stream`; the status covers validation and
 *     launch.  All argument checks run on the host before any HIP call.
 *   - the library keeps one hipBLASLt handle per device and a cache of
 *     chosen GEMM algorithms for the life of the process (guarded by a
 *     mutex); it allocates no device memory: scratch comes from `ws`.
 */
#ifndef S2BLOCK_H
#define S2BLOCK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct s2block_config {
    uint32_t struct_size;  /* sizeof(s2block_config) */
    int32_t B, L, Hq, Hkv, d;
    int32_t G, shifted_heads;
    int32_t lora_rank;     /* r: 8, 16, 24, .. 64 (a multiple of 8; INVALID_ARG otherwise) */
    float lora_scale;      /* s, multiplies every B A product */
    int32_t rope;          /* 1: RoPE with position interpolation inside attention */
    float rope_base;
    int32_t rope_orig_len;
} s2block_config;

typedef struct s2block_params {
    const void *wq, *wk, *wv, *wo;
    const void *aq, *ak, *av, *ao;
    const void *bq, *bk, *bv, *bo;
} s2block_params;

/* Activations the forward writes and the backward reads. */
typedef struct s2block_saved {
    void *q, *k, *v;  /* pre-RoPE projections */
    void *attn;       /* attention output [B, L, Hq, d] */
    float *lse;       /* [B, Hq, L] */
    void *u;          /* [B L, 4 r] bf16, s times: x Aq^T | x Ak^T | x Av^T | attn Ao^T */
} s2block_saved;

typedef struct s2block_grads {
    void *dx;                         /* [B, L, Dm] bf16 */
    float *daq, *dak, *dav, *dao;     /* fp32, shapes of Aq .. Ao */
    float *dbq, *dbk, *dbv, *dbo;     /* fp32, shapes of Bq .. Bo */
} s2block_grads;

/* s2block_config with the defaults: rank 8, scale 2 (alpha 16 over rank 8),
 * RoPE base 10000, original length 4096; sizes zero. */
s2block_config s2block_config_init(void);

/* Workspace bytes for the forward (is_bwd = 0) or backward; 0 for an
 * invalid config. */
size_t s2block_workspace_size(int is_bwd, const s2block_config* cfg);

/* Forward: y and the saved activations from x. */
int s2block_fwd(const s2block_config* cfg, const void* x, const s2block_params* w, void* y,
                const s2block_saved* saved, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward: dx and the LoRA gradients from dy and the forward's saved
 * activations.  Gradients are written, not accumulated. */
int s2block_bwd(const s2block_config* cfg, const void* x, const s2block_params* w,
                const s2block_saved* saved, const void* dy, const s2block_grads* g, void* ws,
                size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* S2BLOCK_H */
