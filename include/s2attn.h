/*
 * libs2attn -- S2-Attn (shift short attention, from LongLoRA) on MI355X (gfx950).
 *
 * The operation (LongLoRA blog summary, smallflyingpig.github.io, section 3.3;
 * nearauto.com LongLoRA article, shift-short-attention section; python88.com
 * LongLoRA article, section on reducing computation):
 *   A sequence of L tokens is cut into L/G groups of G tokens and causal
 *   softmax attention runs only inside each group.  The last `shifted_heads`
 *   query heads see the sequence rolled left by G/2 (token t sits at rolled
 *   position (t - G/2) mod L) before grouping, and their outputs are rolled
 *   back, so groups of shifted and unshifted heads overlap.  Causality is by
 *   in-group index in the rolled order; the roll is cyclic, so the last
 *   shifted group holds the last G/2 tokens followed by the first G/2.
 *   The roll, grouping and un-roll are address arithmetic in the kernels: no
 *   copy of any tensor is made.
 *
 * Layout (all tensors contiguous, row-major):
 *   q, o, dout, dq : [B, L, Hq, d]
 *   k, v, dk, dv   : [B, L, Hkv, d]      query head h uses KV head h / (Hq/Hkv)
 *   lse, delta     : [B, Hq, L] float32, indexed by original token position
 *   lse[b,h,t] = ln sum_j exp(scale * q_t . k_j) over the keys t may attend to.
 *
 * Conventions for every entry point:
 *   - Pointers are device memory owned by the caller; the library allocates
 *     nothing and keeps nothing after it returns.  Pointers must be 16-byte
 *     aligned.  Outputs must not alias inputs.  Outputs are overwritten, not
 *     accumulated into (dk, dv already hold the sum over the query heads that
 *     share a KV head).
 *   - Calls only enqueue kernel launches on `stream` (0 = the default
 *     stream): no allocation, copy, memset or synchronisation, so they can be
 *     captured in a HIP graph.  The returned status covers argument checks
 *     and kernel launch; faults during execution surface at the caller's next
 *     synchronisation.
 *   - Every argument check runs on the host before any HIP call, so invalid
 *     arguments are reported without touching the GPU.  Nothing is printed.
 *   - Stateless and thread-safe.
 */
#ifndef S2ATTN_H
#define S2ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    S2ATTN_OK = 0,
    S2ATTN_ERR_INVALID_ARG = 1,  /* null pointer, size <= 0, L % G != 0, odd G with shifted
                                    heads, Hq % Hkv != 0, shifted_heads outside [0, Hq],
                                    bad opts (struct_size, dtype, rope fields,
                                    ds_max_mib < -1, residual_split outside [-1, 1]) */
    S2ATTN_ERR_UNSUPPORTED = 2,  /* d not in {64, 128}; backward with shifted_heads % (Hq/Hkv)
                                    != 0 (a KV head shared by shifted and unshifted query
                                    heads); RoPE with float32 inputs; bf16 gradients of
                                    float32 inputs; sizes past the kernels' index ranges:
                                    a (batch, head) plane of L*H*d*2 >= 2^31 bytes,
                                    a token row of H*d*2 >= 2^24 bytes (H = max(Hq, Hkv)),
                                    L >= 2^24, L*Hq >= 2^31, or a grid of 2^31 or more
                                    workgroups */
    S2ATTN_ERR_WORKSPACE = 3,    /* workspace missing or smaller than s2attn_workspace_size() */
    S2ATTN_ERR_HIP = 4           /* a HIP runtime error (no device, launch failure, ...) */
} s2attn_status;

typedef enum {
    S2ATTN_BF16 = 0,
    S2ATTN_F32 = 1
} s2attn_dtype;

/* Stages of the backward, for s2attn_bwd_stage_ex. */
enum {
    S2ATTN_BWD_STAGE_PRE = 0,
    S2ATTN_BWD_STAGE_DKDV = 1,
    S2ATTN_BWD_STAGE_DQ = 2
};

/*
 * Options for the _ex entry points.  Fill with s2attn_opts_init() first.
 *   dtype        element type of q, k, v, o, dout.  BF16: bf16 MFMA with fp32
 *                accumulation; F32: fp32 arithmetic throughout.
 *   grad_dtype   element type of dq, dk, dv (BF16 only with bf16 inputs, or F32).
 *   softmax_scale  <= 0 selects 1/sqrt(d).
 *   rope         nonzero: rotate q and k at their original positions t by
 *                angle t * (rope_orig_len / L) * rope_base^(-2c/d) on channel
 *                pairs (c, c + d/2), c < d/2, before attention (RoPE with
 *                position interpolation, LongLoRA blog section 3.4).
 *                Gradients are then w.r.t. the un-rotated q and k.
 *   ds_max_mib   largest region of dS tiles, in MiB, the backward may keep in
 *                its workspace (see s2attn_workspace_size); above it dQ
 *                recomputes the scores instead.  Keeping dS trades about
 *                B*Hq*L*G bytes of workspace for a dQ pass that reads dS back
 *                instead of recomputing the scores (one product in place of
 *                three).  -1 selects the default, 16384 (16 GiB); 0 never
 *                keeps dS.  Values below -1: S2ATTN_ERR_INVALID_ARG.
 *   residual_split  bf16 backward only.  P and dS enter the dV and dK
 *                products as bf16 (8 significant bits).  With the split, a
 *                32 x 32 (query, key) tile whose largest P is at least 1/16
 *                also adds the products of the residuals x - bf16(x), rounded
 *                to bf16, so those terms carry about 16 bits; dQ is not
 *                affected.  1 always, 0 never, -1 (default) when a KV head
 *                serves several query heads (Hq != Hkv) or G < 4096.  Other
 *                values: S2ATTN_ERR_INVALID_ARG.
 */
typedef struct {
    uint32_t struct_size;  /* must equal sizeof(s2attn_opts) */
    int32_t dtype;
    int32_t grad_dtype;
    float softmax_scale;
    int32_t rope;
    float rope_base;
    int32_t rope_orig_len;
    int32_t ds_max_mib;
    int32_t residual_split;
} s2attn_opts;

/* Defaults: bf16 inputs and gradients, scale 1/sqrt(d), no RoPE, dS kept up
   to 16 GiB, residual split chosen by shape. */
void s2attn_opts_init(s2attn_opts* opts);

/*
 * Forward, bf16, scale 1/sqrt(d), no RoPE.
 * Reads q, k, v; writes o (bf16) and lse (fp32).
 */
int s2attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int L, int Hq, int Hkv, int d, int G, int shifted_heads,
               hipStream_t stream);

/*
 * Backward, bf16 inputs and gradients, scale 1/sqrt(d), no RoPE.
 * Reads q, k, v, o, lse (as written by s2attn_fwd on the same inputs) and
 * dout; writes dq, dk, dv.  delta_ws is caller scratch of B*Hq*L floats,
 * [B, Hq, L]: it receives the row term -rowsum(dout * o) (its contents on
 * return are that term; nothing else is written to it).
 * Gradient formulas: with P the attention probabilities,
 * dS = P * (dout . v_j - delta), dq = scale dS k, dk = scale dS^T q,
 * dv = P^T dout (summed over query heads per KV head).
 */
int s2attn_bwd(const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv,
               float* delta_ws,
               int B, int L, int Hq, int Hkv, int d, int G, int shifted_heads,
               hipStream_t stream);

/* Row-term floats (B * Hq * L) s2attn_bwd_noalloc's device array holds. */
#define S2ATTN_NOALLOC_MAX_ROWS (1u << 23)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the plain
 * backward (bf16, scale 1/sqrt(d), no RoPE, the same kernels and results as
 * s2attn_bwd) without delta_ws.  The row term lives in a device array inside
 * the library, S2ATTN_NOALLOC_MAX_ROWS floats (32 MiB) on each GPU it runs on,
 * held until the process ends; the call itself allocates nothing.
 * B * Hq * L above S2ATTN_NOALLOC_MAX_ROWS: S2ATTN_ERR_WORKSPACE (after the
 * argument checks of s2attn_bwd, which come first and run on the host).
 * Every call on one GPU uses that GPU's one array: calls whose execution
 * overlaps on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Nothing needs clearing between calls: each
 * call's row-term kernel writes every element its gradient kernels read.
 * The array's address is looked up once per device, on the first call with
 * that device current (a HIP runtime query; not inside the stream's work).
 */
int s2attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       int B, int L, int Hq, int Hkv, int d, int G, int shifted_heads,
                       hipStream_t stream);

/*
 * Bytes of workspace the _ex entry points need for these sizes and options
 * (0 when none).  is_bwd selects the backward.  Returns 0 for invalid
 * arguments as well; the _ex call then reports the error.
 *
 * Forward workspace: with RoPE the rotated k (bf16, the size of k); the
 * kernel rotates its own query tile in registers.  None without RoPE.
 *
 * Backward workspace, each part 256-byte aligned: the row term -delta
 * (B Hq L floats); with RoPE the rotated q and k (bf16, the sizes of q and
 * k); for bf16 inputs, the dS tiles: per (batch, head, group) the 32 x 32
 * tiles on or below the causal diagonal, padded to whole blocks of 8 query
 * rows: 32 NB (NB + 1) tiles of 2 KB with NB = ceil(ceil(G / 32) / 8), i.e.
 * B Hq (L / G) 32 NB (NB + 1) * 2048 bytes (about B Hq L G bytes), kept only
 * while that is at most opts->ds_max_mib MiB (16 GiB by default).  The dK/dV
 * kernel writes dS there and the dQ kernel reads it, so dQ is one product
 * instead of recomputing the scores; above the bound dQ recomputes them.  The
 * plain s2attn_bwd has no workspace and always recomputes.
 */
size_t s2attn_workspace_size(int is_bwd, int B, int L, int Hq, int Hkv, int d, int G,
                             const s2attn_opts* opts);

/* Forward with options; `ws` may be NULL when the workspace size is 0. */
int s2attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int L, int Hq, int Hkv, int d, int G, int shifted_heads,
                  const s2attn_opts* opts, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward with options; the row term delta lives in the workspace. */
int s2attn_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  int B, int L, int Hq, int Hkv, int d, int G, int shifted_heads,
                  const s2attn_opts* opts, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The backward as its three kernels, for callers that time or overlap them.
 * Arguments are those of s2attn_bwd_ex, with the same workspace.
 *   S2ATTN_BWD_STAGE_PRE   -delta = -rowsum(dout * o) into the workspace (and,
 *                          with RoPE, the rotated q and k).
 *   S2ATTN_BWD_STAGE_DKDV  dk, dv (and, bf16, the dS tiles into the
 *                          workspace when it holds them).  Needs PRE complete.
 *   S2ATTN_BWD_STAGE_DQ    dq.  Needs PRE complete, and DKDV complete when the
 *                          workspace holds dS tiles (see s2attn_workspace_size).
 * PRE, DKDV, DQ in that order on one stream equal s2attn_bwd_ex.  Without dS
 * tiles (fp32 inputs, or a dS region above opts->ds_max_mib) DKDV and DQ read
 * only PRE's results and the inputs and may run concurrently on two streams
 * once PRE has finished.
 * Any other stage value: S2ATTN_ERR_INVALID_ARG.
 */
int s2attn_bwd_stage_ex(int stage, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        int B, int L, int Hq, int Hkv, int d, int G, int shifted_heads,
                        const s2attn_opts* opts, void* ws, size_t ws_bytes, hipStream_t stream);

/* Static string naming a status code. */
const char* s2attn_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int s2attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* S2ATTN_H */
