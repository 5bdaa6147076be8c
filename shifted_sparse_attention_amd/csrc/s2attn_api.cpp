// libs2attn C ABI: argument checks, workspace sizing and kernel dispatch.
//
// Every check below is pure host arithmetic and runs before the first HIP
// call, so invalid arguments are reported without touching a device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "s2_params.h"
#include "s2attn.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The backward keeps dS (bf16, 32 x 32 tiles of each group's causal
// triangle) for the dQ kernel while the tiles fit the caller's bound; above
// it, dQ recomputes S and dP instead.  Default bound: 16 GiB (about a
// seventeenth of the MI355X's 288 GB of HBM), enough for 32k tokens of 32
// heads in groups of 8192 (8.3 GiB); larger regions are the caller's choice.
constexpr double kDefaultDsMaxMib = 16.0 * 1024.0;

struct Resolved {
    int dtype;       // S2ATTN_BF16 / S2ATTN_F32
    int grad_dtype;
    float scale;
    int rope;
    float rope_base;
    int rope_orig_len;
    double ds_max_bytes;  // dS tiles are kept in the workspace up to this size
    int residual_split;   // -1 auto, 0 off, 1 on (see s2attn_opts)
};

// The automatic choice of opts.residual_split: on where several query heads
// share a KV head (dK, dV sum the rounding of r heads' P and dS) or where
// groups are shorter than 4096 tokens (a larger share of rows sits near the
// start of a group, where a query sees few keys and P is large).
bool residual_split_auto(int Hq, int Hkv, int G) { return Hq != Hkv || G < 4096; }

// Sizes shared by forward and backward.
int check_sizes(int B, int L, int Hq, int Hkv, int d, int G, int shifted_heads) {
    if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || G <= 0) return S2ATTN_ERR_INVALID_ARG;
    if (L % G != 0) return S2ATTN_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return S2ATTN_ERR_INVALID_ARG;
    if (shifted_heads < 0 || shifted_heads > Hq) return S2ATTN_ERR_INVALID_ARG;
    if (shifted_heads > 0 && (G % 2) != 0) return S2ATTN_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return S2ATTN_ERR_UNSUPPORTED;
    // Element counts must fit the 64-bit offsets; workgroup counts fit a 32-bit grid.
    const double elems = (double)B * L * Hq * d;
    if (elems > 9.0e18) return S2ATTN_ERR_UNSUPPORTED;
    const double wgs = (double)B * Hq * (L / G) * ((G + 63) / 64);
    if (wgs > 2147483647.0) return S2ATTN_ERR_UNSUPPORTED;
    if ((double)L * Hq > 2147483647.0) return S2ATTN_ERR_UNSUPPORTED;
    // Tiles are fetched as a 64-bit (batch, head) base plus 32-bit byte offsets,
    // a row's offset as a 24-bit by 24-bit product (row index times row bytes).
    const int Hmax = Hq > Hkv ? Hq : Hkv;
    if ((double)L * Hmax * d * 4 > 4294967295.0 || L >= (1 << 24)) return S2ATTN_ERR_UNSUPPORTED;
    if ((double)Hmax * d * 2 >= (double)(1 << 24)) return S2ATTN_ERR_UNSUPPORTED;
    return S2ATTN_OK;
}

int resolve_opts(const s2attn_opts* o, int d, Resolved* r) {
    s2attn_opts def;
    s2attn_opts_init(&def);
    if (o == nullptr) o = &def;
    if (o->struct_size != sizeof(s2attn_opts)) return S2ATTN_ERR_INVALID_ARG;
    if (o->dtype != S2ATTN_BF16 && o->dtype != S2ATTN_F32) return S2ATTN_ERR_INVALID_ARG;
    if (o->grad_dtype != S2ATTN_BF16 && o->grad_dtype != S2ATTN_F32) return S2ATTN_ERR_INVALID_ARG;
    if (isnan(o->softmax_scale) || isinf(o->softmax_scale)) return S2ATTN_ERR_INVALID_ARG;
    if (o->rope) {
        if (!(o->rope_base > 1.0f) || isinf(o->rope_base)) return S2ATTN_ERR_INVALID_ARG;
        if (o->rope_orig_len <= 0) return S2ATTN_ERR_INVALID_ARG;
        if (o->dtype == S2ATTN_F32) return S2ATTN_ERR_UNSUPPORTED;
    }
    if (o->dtype == S2ATTN_F32 && o->grad_dtype == S2ATTN_BF16) return S2ATTN_ERR_UNSUPPORTED;
    if (o->ds_max_mib < -1) return S2ATTN_ERR_INVALID_ARG;
    if (o->residual_split < -1 || o->residual_split > 1) return S2ATTN_ERR_INVALID_ARG;
    r->dtype = o->dtype;
    r->grad_dtype = o->grad_dtype;
    r->scale = o->softmax_scale > 0.f ? o->softmax_scale : 1.0f / sqrtf((float)d);
    r->rope = o->rope ? 1 : 0;
    r->rope_base = o->rope_base;
    r->rope_orig_len = o->rope_orig_len;
    r->ds_max_bytes = (o->ds_max_mib < 0 ? kDefaultDsMaxMib : (double)o->ds_max_mib) * 1048576.0;
    r->residual_split = o->residual_split;
    return S2ATTN_OK;
}

// Bytes of the dS tiles (blocks of 8 query rows, see Params::ds), in double so
// the bound check cannot wrap for any accepted size.
double ds_bytes_f(int B, int Hq, int L, int G) {
    const double NB = (double)((((size_t)G + 31) / 32 + 7) / 8);
    return (double)B * Hq * (L / G) * (32.0 * NB * (NB + 1)) * 2048.0;
}

bool use_ds(int B, int Hq, int L, int G, const Resolved& r) {
    return r.dtype == S2ATTN_BF16 && ds_bytes_f(B, Hq, L, G) <= r.ds_max_bytes;
}

// Exact byte count; called only when use_ds holds (within the bound, so the
// size_t product cannot wrap).
size_t ds_bytes(int B, int Hq, int L, int G) {
    const size_t NB = (((size_t)G + 31) / 32 + 7) / 8;
    return (size_t)B * Hq * (L / G) * (32 * NB * (NB + 1)) * 2048;
}

// Workspace layout: [row term (bwd): -delta | rotated q | rotated k | dS tiles (bwd,
// when kept)], each 256-byte aligned.
struct WsLayout {
    size_t delta_off, delta_bytes;
    size_t rq_off, rq_bytes;
    size_t rk_off, rk_bytes;
    size_t ds_off, ds_bytes;
    size_t total;
};

// is_bwd: 0 forward, 1 backward with the row term in the workspace, 2 backward
// with the row term supplied separately (the plain entry point: no dS tiles).
WsLayout ws_layout(int is_bwd, int B, int L, int Hq, int Hkv, int d, int G, const Resolved& r) {
    WsLayout w{};
    size_t off = 0;
    if (is_bwd == 1) {
        w.delta_off = off;
        w.delta_bytes = (size_t)B * Hq * L * sizeof(float);
        off += align_up(w.delta_bytes);
    }
    if (r.rope) {
        // The forward rotates its stationary query tile in registers; only the
        // backward (which streams q) keeps a rotated copy of q.
        if (is_bwd) {
            w.rq_off = off;
            w.rq_bytes = (size_t)B * L * Hq * d * 2;
            off += align_up(w.rq_bytes);
        }
        w.rk_off = off;
        w.rk_bytes = (size_t)B * L * Hkv * d * 2;
        off += align_up(w.rk_bytes);
    }
    if (is_bwd == 1 && use_ds(B, Hq, L, G, r)) {
        w.ds_off = off;
        w.ds_bytes = ds_bytes(B, Hq, L, G);
        off += align_up(w.ds_bytes);
    }
    w.total = off;
    return w;
}

s2::Params make_params(int B, int L, int Hq, int Hkv, int d, int G, int shifted_heads,
                       const Resolved& r) {
    s2::Params p;
    memset(&p, 0, sizeof(p));
    p.B = B;
    p.L = L;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.d = d;
    p.G = G;
    p.shifted_heads = shifted_heads;
    p.r = Hq / Hkv;
    p.n_g = L / G;
    p.scale = r.scale;
    p.scale_log2 = r.scale * 1.4426950408889634f;
    p.band = 1;
    p.rope = r.rope;
    if (r.rope) {
        // LongLoRA blog, section 3.4: positions [0, L) are squeezed onto [0, L0).
        const double pos_scale = (double)r.rope_orig_len / (double)L;
        const double two_pi = 6.283185307179586476925286766559;
        for (int c = 0; c < d / 2; ++c)
            p.rope_rev[c] = pos_scale * pow((double)r.rope_base, -2.0 * c / (double)d) / two_pi;
    }
    return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? S2ATTN_OK : S2ATTN_ERR_HIP; }

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int L,
             int Hq, int Hkv, int d, int G, int shifted_heads, const s2attn_opts* opts, void* ws,
             size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return S2ATTN_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return S2ATTN_ERR_INVALID_ARG;
    int st = check_sizes(B, L, Hq, Hkv, d, G, shifted_heads);
    if (st) return st;
    Resolved r;
    st = resolve_opts(opts, d, &r);
    if (st) return st;
    const WsLayout wl = ws_layout(0, B, L, Hq, Hkv, d, G, r);
    if (wl.total > 0 && (ws == nullptr || ws_bytes < wl.total || !aligned16(ws)))
        return S2ATTN_ERR_WORKSPACE;

    s2::Params p = make_params(B, L, Hq, Hkv, d, G, shifted_heads, r);
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    if (r.dtype == S2ATTN_F32) return hip_status(s2::launch_fwd_f32(p, stream));
    if (r.rope) {
        // k is streamed by every query tile, so it is rotated once by the
        // pre-pass; the kernel rotates its query fragments itself (p.rope).
        void* rk = static_cast<char*>(ws) + wl.rk_off;
        hipError_t e = s2::launch_rope_prepass(p, nullptr, rk, stream);
        if (e != hipSuccess) return S2ATTN_ERR_HIP;
        p.k = rk;
    }
    return hip_status(s2::launch_fwd_bf16(p, stream));
}

constexpr int kStagePre = 1, kStageDkdv = 2, kStageDq = 4, kStageAll = 7;

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int L, int Hq,
             int Hkv, int d, int G, int shifted_heads, const s2attn_opts* opts, void* ws,
             size_t ws_bytes, hipStream_t stream, int stages) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return S2ATTN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return S2ATTN_ERR_INVALID_ARG;
    int st = check_sizes(B, L, Hq, Hkv, d, G, shifted_heads);
    if (st) return st;
    Resolved r;
    st = resolve_opts(opts, d, &r);
    if (st) return st;
    if (shifted_heads % (Hq / Hkv) != 0) return S2ATTN_ERR_UNSUPPORTED;

    WsLayout wl = ws_layout(1, B, L, Hq, Hkv, d, G, r);
    char* base = static_cast<char*>(ws);
    if (delta != nullptr) {
        // Plain entry point: delta supplied separately, workspace holds the rest.
        if (!aligned16(delta)) return S2ATTN_ERR_INVALID_ARG;
        wl = ws_layout(2, B, L, Hq, Hkv, d, G, r);
    }
    if (wl.total > 0 && (ws == nullptr || ws_bytes < wl.total || !aligned16(ws)))
        return S2ATTN_ERR_WORKSPACE;
    if (delta == nullptr) delta = reinterpret_cast<float*>(base + wl.delta_off);

    s2::Params p = make_params(B, L, Hq, Hkv, d, G, shifted_heads, r);
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = const_cast<void*>(o);
    p.lse = const_cast<float*>(lse);
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.delta = delta;
    p.ds = wl.ds_bytes ? base + wl.ds_off : nullptr;

    char* rq = base + wl.rq_off;
    char* rk = base + wl.rk_off;
    if (stages & kStagePre) {
        if (s2::launch_bwd_pre(p, r.dtype == S2ATTN_F32, stream) != hipSuccess)
            return S2ATTN_ERR_HIP;
        if (r.rope && s2::launch_rope_prepass(p, rq, rk, stream) != hipSuccess)
            return S2ATTN_ERR_HIP;
    }
    if (r.rope) {
        p.q = rq;
        p.k = rk;  // p.rope stays set: the epilogues rotate dq, dk back
    }
    const int gf = r.grad_dtype == S2ATTN_F32;
    if (stages & kStageDkdv) {
        const int split = r.residual_split >= 0 ? r.residual_split : residual_split_auto(Hq, Hkv, G);
        hipError_t e = r.dtype == S2ATTN_F32 ? s2::launch_bwd_dkdv_f32(p, stream)
                                              : s2::launch_bwd_dkdv_bf16(p, gf, split, stream);
        if (e != hipSuccess) return S2ATTN_ERR_HIP;
    }
    if (stages & kStageDq) {
        hipError_t e = r.dtype == S2ATTN_F32 ? s2::launch_bwd_dq_f32(p, stream)
                       : p.ds               ? s2::launch_bwd_dq_ds_bf16(p, gf, stream)
                                            : s2::launch_bwd_dq_bf16(p, gf, stream);
        if (e != hipSuccess) return S2ATTN_ERR_HIP;
    }
    return S2ATTN_OK;
}

}  // namespace

namespace s2 {

int bwd_plain(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int L, int Hq,
              int Hkv, int d, int G, int shifted_heads, hipStream_t stream, int launch) {
    // Without a launch only the host checks run; any aligned non-null address
    // stands in for the row term's buffer then.
    float* dl = launch ? delta : reinterpret_cast<float*>(kAlign);
    if (!dl) return S2ATTN_ERR_INVALID_ARG;
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, dl, B, L, Hq, Hkv, d, G, shifted_heads,
                    nullptr, nullptr, 0, stream, launch ? kStageAll : 0);
}

int attention_config_status(int is_bwd, int B, int L, int Hq, int Hkv, int d, int G,
                            int shifted_heads, const s2attn_opts* opts) {
    int st = check_sizes(B, L, Hq, Hkv, d, G, shifted_heads);
    if (st) return st;
    Resolved r;
    st = resolve_opts(opts, d, &r);
    if (st) return st;
    if (is_bwd && shifted_heads % (Hq / Hkv) != 0) return S2ATTN_ERR_UNSUPPORTED;
    return S2ATTN_OK;
}

}  // namespace s2

extern "C" {

void s2attn_opts_init(s2attn_opts* opts) {
    if (!opts) return;
    memset(opts, 0, sizeof(*opts));
    opts->struct_size = sizeof(s2attn_opts);
    opts->dtype = S2ATTN_BF16;
    opts->grad_dtype = S2ATTN_BF16;
    opts->softmax_scale = 0.f;
    opts->rope = 0;
    opts->rope_base = 10000.f;
    opts->rope_orig_len = 4096;
    opts->ds_max_mib = -1;
    opts->residual_split = -1;
}

int s2attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int L,
               int Hq, int Hkv, int d, int G, int shifted_heads, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, L, Hq, Hkv, d, G, shifted_heads, nullptr, nullptr, 0,
                    stream);
}

int s2attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, float* delta_ws, int B, int L,
               int Hq, int Hkv, int d, int G, int shifted_heads, hipStream_t stream) {
    if (!delta_ws) return S2ATTN_ERR_INVALID_ARG;
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, L, Hq, Hkv, d, G,
                    shifted_heads, nullptr, nullptr, 0, stream, kStageAll);
}

size_t s2attn_workspace_size(int is_bwd, int B, int L, int Hq, int Hkv, int d, int G,
                             const s2attn_opts* opts) {
    if (check_sizes(B, L, Hq, Hkv, d, G, 0) != S2ATTN_OK) return 0;
    Resolved r;
    if (resolve_opts(opts, d, &r) != S2ATTN_OK) return 0;
    return ws_layout(is_bwd ? 1 : 0, B, L, Hq, Hkv, d, G, r).total;
}

int s2attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int L,
                  int Hq, int Hkv, int d, int G, int shifted_heads, const s2attn_opts* opts,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, L, Hq, Hkv, d, G, shifted_heads, opts, ws, ws_bytes,
                    stream);
}

int s2attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, int B, int L, int Hq, int Hkv,
                  int d, int G, int shifted_heads, const s2attn_opts* opts, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, L, Hq, Hkv, d, G,
                    shifted_heads, opts, ws, ws_bytes, stream, kStageAll);
}

int s2attn_bwd_stage_ex(int stage, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                        int L, int Hq, int Hkv, int d, int G, int shifted_heads,
                        const s2attn_opts* opts, void* ws, size_t ws_bytes, hipStream_t stream) {
    int mask;
    switch (stage) {
        case S2ATTN_BWD_STAGE_PRE: mask = kStagePre; break;
        case S2ATTN_BWD_STAGE_DKDV: mask = kStageDkdv; break;
        case S2ATTN_BWD_STAGE_DQ: mask = kStageDq; break;
        default: return S2ATTN_ERR_INVALID_ARG;
    }
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, L, Hq, Hkv, d, G,
                    shifted_heads, opts, ws, ws_bytes, stream, mask);
}

const char* s2attn_status_string(int status) {
    switch (status) {
        case S2ATTN_OK: return "S2ATTN_OK";
        case S2ATTN_ERR_INVALID_ARG: return "S2ATTN_ERR_INVALID_ARG";
        case S2ATTN_ERR_UNSUPPORTED: return "S2ATTN_ERR_UNSUPPORTED";
        case S2ATTN_ERR_WORKSPACE: return "S2ATTN_ERR_WORKSPACE";
        case S2ATTN_ERR_HIP: return "S2ATTN_ERR_HIP";
        default: return "S2ATTN_UNKNOWN_STATUS";
    }
}

int s2attn_version(void) { return 100; }

}  // extern "C"
