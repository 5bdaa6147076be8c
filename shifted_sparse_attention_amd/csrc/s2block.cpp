// The attention block around S2-Attn: LoRA-adapted Q, K, V, O projections
// (hipBLASLt GEMMs), RoPE-PI and S2-Attn (libs2attn's kernels).
//
// LongLoRA blog (smallflyingpig.github.io), section 3.2: the trainable parts
// of attention are LoRA adapters on the Q, K, V and O projections; the base
// weights stay frozen.  Each adapted projection is x W^T + s (x A^T) B^T.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>
#include <tuple>

#include "s2_params.h"
#include "s2attn.h"
#include "s2block.h"
#include "s2block_kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kLtWorkspace = 32u << 20;  // hipBLASLt scratch slice of the caller's workspace

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
// GEMM depths are padded to whole 64-wide K steps (zero columns against zero rows).
int64_t kpad(int64_t k) { return (k + 63) / 64 * 64; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Row-major GEMM on hipBLASLt: C[M x N] = alpha op(A) op(B) + beta C, with A,
// B bf16 and C bf16 or fp32, fp32 accumulation.  hipBLASLt is column-major:
// a row-major X viewed column-major is X^T, so C^T = op(B)^T op(A)^T is the
// column-major product with the operands swapped.
// ---------------------------------------------------------------------------
struct Plan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
};

using PlanKey = std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                           int, size_t>;

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<PlanKey, Plan> g_plans;

int lt_handle(int dev, hipblasLtHandle_t* h) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_handles.find(dev);
    if (it != g_handles.end()) {
        *h = it->second;
        return S2ATTN_OK;
    }
    hipblasLtHandle_t nh;
    if (hipblasLtCreate(&nh) != HIPBLAS_STATUS_SUCCESS) return S2ATTN_ERR_HIP;
    g_handles[dev] = nh;
    *h = nh;
    return S2ATTN_OK;
}

struct Gemm {
    hipStream_t stream;
    int dev;
    hipblasLtHandle_t h;
    void* lt_ws;
    size_t lt_ws_bytes;

    // transA: op(A) = A^T with A stored [K x M]; otherwise A stored [M x K].
    // transB: op(B) = B^T with B stored [N x K]; otherwise B stored [K x N].
    int run(bool transA, bool transB, int64_t M, int64_t N, int64_t K, float alpha,
            const void* A, int64_t lda, const void* B, int64_t ldb, float beta, void* C,
            int64_t ldc, bool c_f32) {
        const int c32 = c_f32 ? 1 : 0;
        PlanKey key{dev, transA, transB, M, N, K, lda, ldb, ldc, c32, lt_ws_bytes};
        Plan plan;
        {
            std::lock_guard<std::mutex> lk(g_mu);
            auto it = g_plans.find(key);
            if (it != g_plans.end()) plan = it->second;
        }
        if (plan.desc == nullptr) {
            int st = make_plan(transA, transB, M, N, K, lda, ldb, ldc, c_f32, &plan);
            if (st) return st;
            std::lock_guard<std::mutex> lk(g_mu);
            auto ins = g_plans.emplace(key, plan);
            if (!ins.second) {  // another thread made one first: keep theirs
                destroy(&plan);
                plan = ins.first->second;
            }
        }
        // column-major: D (N x M) = opB'(B) opA'(A)
        hipblasStatus_t s = hipblasLtMatmul(h, plan.desc, &alpha, B, plan.la, A, plan.lb, &beta, C,
                                            plan.lc, C, plan.lc, &plan.algo, lt_ws, plan.ws, stream);
        return s == HIPBLAS_STATUS_SUCCESS ? S2ATTN_OK : S2ATTN_ERR_HIP;
    }

    static void destroy(Plan* p) {
        if (p->la) hipblasLtMatrixLayoutDestroy(p->la);
        if (p->lb) hipblasLtMatrixLayoutDestroy(p->lb);
        if (p->lc) hipblasLtMatrixLayoutDestroy(p->lc);
        if (p->desc) hipblasLtMatmulDescDestroy(p->desc);
        *p = Plan{};
    }

    int make_plan(bool transA, bool transB, int64_t M, int64_t N, int64_t K, int64_t lda,
                  int64_t ldb, int64_t ldc, bool c_f32, Plan* plan) {
        bool ok = hipblasLtMatmulDescCreate(&plan->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) ==
                  HIPBLAS_STATUS_SUCCESS;
        // Column-major operand 1 is B: stored [K x N] row-major = [N x K] column-major (op N),
        // or [N x K] row-major = [K x N] column-major (op T).
        hipblasOperation_t op1 = transB ? HIPBLAS_OP_T : HIPBLAS_OP_N;
        hipblasOperation_t op2 = transA ? HIPBLAS_OP_T : HIPBLAS_OP_N;
        if (ok)
            ok = hipblasLtMatmulDescSetAttribute(plan->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op1,
                                                 sizeof(op1)) == HIPBLAS_STATUS_SUCCESS &&
                 hipblasLtMatmulDescSetAttribute(plan->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op2,
                                                 sizeof(op2)) == HIPBLAS_STATUS_SUCCESS;
        if (ok)
            ok = hipblasLtMatrixLayoutCreate(&plan->la, HIP_R_16BF, transB ? K : N,
                                             transB ? N : K, ldb) == HIPBLAS_STATUS_SUCCESS &&
                 hipblasLtMatrixLayoutCreate(&plan->lb, HIP_R_16BF, transA ? M : K,
                                             transA ? K : M, lda) == HIPBLAS_STATUS_SUCCESS &&
                 hipblasLtMatrixLayoutCreate(&plan->lc, c_f32 ? HIP_R_32F : HIP_R_16BF, N, M,
                                             ldc) == HIPBLAS_STATUS_SUCCESS;
        hipblasLtMatmulPreference_t pref = nullptr;
        if (ok) ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
        uint64_t wsb = lt_ws_bytes;
        if (ok)
            ok = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                       &wsb, sizeof(wsb)) == HIPBLAS_STATUS_SUCCESS;
        hipblasLtMatmulHeuristicResult_t res[1];
        int n_res = 0;
        if (ok)
            ok = hipblasLtMatmulAlgoGetHeuristic(h, plan->desc, plan->la, plan->lb, plan->lc,
                                                 plan->lc, pref, 1, res, &n_res) ==
                     HIPBLAS_STATUS_SUCCESS &&
                 n_res > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS &&
                 res[0].workspaceSize <= lt_ws_bytes;
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        if (!ok) {
            destroy(plan);
            return S2ATTN_ERR_HIP;
        }
        plan->algo = res[0].algo;
        plan->ws = res[0].workspaceSize;
        return S2ATTN_OK;
    }
};

// ---------------------------------------------------------------------------
// Sizes and checks.
// ---------------------------------------------------------------------------
struct Dims {
    int64_t M, Dm, Nq, Nkv, r;
};

int check_config(const s2block_config* c, int is_bwd, s2attn_opts* att, Dims* dm) {
    if (c == nullptr || c->struct_size != sizeof(s2block_config)) return S2ATTN_ERR_INVALID_ARG;
    // r a multiple of 8: the column slices of the [B L, 4 r] LoRA buffers then
    // start 16-byte aligned, as the GEMMs' vector loads assume.
    if (c->lora_rank < 8 || c->lora_rank > 64 || c->lora_rank % 8 != 0) return S2ATTN_ERR_INVALID_ARG;
    if (isnan(c->lora_scale) || isinf(c->lora_scale)) return S2ATTN_ERR_INVALID_ARG;
    s2attn_opts_init(att);
    att->rope = c->rope ? 1 : 0;
    att->rope_base = c->rope_base;
    att->rope_orig_len = c->rope_orig_len;
    int st = s2::attention_config_status(is_bwd, c->B, c->L, c->Hq, c->Hkv, c->d, c->G,
                                         c->shifted_heads, att);
    if (st) return st;
    dm->M = (int64_t)c->B * c->L;
    dm->Nq = (int64_t)c->Hq * c->d;
    dm->Dm = dm->Nq;
    dm->Nkv = (int64_t)c->Hkv * c->d;
    dm->r = c->lora_rank;
    // One GEMM operand or result must stay below 2^31 elements (hipBLASLt int64
    // sizes are fine; this bounds the fp32 dx scratch at 8 GB).
    if ((double)dm->M * dm->Dm > 2147483647.0) return S2ATTN_ERR_UNSUPPORTED;
    return S2ATTN_OK;
}

// Workspace: [attention | hipBLASLt | A_cat (3r x Dm bf16) | forward or backward scratch].
// Forward: X_ext = [x | s x A_cat^T | 0] (M x Kx, Kx = Dm + 3r padded to 64)
// and W_ext for q, k, v (N_i x Kx: W_i, then B_i in its own r columns, zeros
// in the others), so each projection with its LoRA term is one GEMM.
// Backward: dq, dk, dv; dattn; D_ext = [dq | dk | dv | s t | 0] (M x Kd, Kd =
// Nq + 2 Nkv + 3r padded to 64) and W_dx = [Wq; Wk; Wv; A_cat; 0] (Kd x Dm),
// so dx is one GEMM; dA_cat (fp32).
struct BlockWs {
    size_t att_off, att_bytes, lt_off, acat_off;
    size_t xext_off, wext_off[3];                         // forward
    size_t t_off, dattn_off, dq_off, dk_off, dv_off;      // backward
    size_t dext_off, wdx_off, dacat_off;
    size_t total;
};

BlockWs block_ws(int is_bwd, const s2block_config* c, const s2attn_opts* att, const Dims& d) {
    BlockWs w{};
    size_t off = 0;
    const int64_t Nt = d.Nq + 2 * d.Nkv;
    const int64_t Kx = kpad(d.Dm + 3 * d.r), Kd = kpad(Nt + 3 * d.r);
    w.att_off = off;
    w.att_bytes = s2attn_workspace_size(is_bwd, c->B, c->L, c->Hq, c->Hkv, c->d, c->G, att);
    off += align_up(w.att_bytes);
    w.lt_off = off;
    off += align_up(kLtWorkspace);
    w.acat_off = off;
    off += align_up((size_t)3 * d.r * d.Dm * 2);
    if (!is_bwd) {
        w.xext_off = off;
        off += align_up((size_t)d.M * Kx * 2);
        const int64_t ns[3] = {d.Nq, d.Nkv, d.Nkv};
        for (int i = 0; i < 3; ++i) {
            w.wext_off[i] = off;
            off += align_up((size_t)ns[i] * Kx * 2);
        }
    } else {
        w.t_off = off;
        off += align_up((size_t)d.M * d.r * 2);
        w.dattn_off = off;
        off += align_up((size_t)d.M * d.Nq * 2);
        w.dq_off = off;
        off += align_up((size_t)d.M * d.Nq * 2);
        w.dk_off = off;
        off += align_up((size_t)d.M * d.Nkv * 2);
        w.dv_off = off;
        off += align_up((size_t)d.M * d.Nkv * 2);
        w.dext_off = off;
        off += align_up((size_t)d.M * Kd * 2);
        w.wdx_off = off;
        off += align_up((size_t)Kd * d.Dm * 2);
        w.dacat_off = off;
        off += align_up((size_t)3 * d.r * d.Dm * 4);
    }
    w.total = off;
    return w;
}

bool params_ok(const s2block_params* w) {
    if (w == nullptr) return false;
    const void* ps[] = {w->wq, w->wk, w->wv, w->wo, w->aq, w->ak, w->av, w->ao,
                        w->bq, w->bk, w->bv, w->bo};
    for (const void* p : ps)
        if (p == nullptr || !aligned16(p)) return false;
    return true;
}

bool saved_ok(const s2block_saved* s) {
    if (s == nullptr) return false;
    const void* ps[] = {s->q, s->k, s->v, s->attn, s->lse, s->u};
    for (const void* p : ps)
        if (p == nullptr || !aligned16(p)) return false;
    return true;
}

int setup(void* ws, size_t ws_bytes, const BlockWs& bw, hipStream_t stream, Gemm* g) {
    if (ws == nullptr || ws_bytes < bw.total || !aligned16(ws)) return S2ATTN_ERR_WORKSPACE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return S2ATTN_ERR_HIP;
    g->stream = stream;
    g->dev = dev;
    g->lt_ws = static_cast<char*>(ws) + bw.lt_off;
    g->lt_ws_bytes = kLtWorkspace;
    return lt_handle(dev, &g->h);
}

// Concatenate Aq, Ak, Av ([r x Dm] each) into A_cat [3r x Dm].
int concat_a(const s2block_params* w, char* acat, const Dims& d, hipStream_t st) {
    const size_t bytes = (size_t)d.r * d.Dm * 2;
    const void* src[3] = {w->aq, w->ak, w->av};
    for (int i = 0; i < 3; ++i)
        if (hipMemcpyAsync(acat + i * bytes, src[i], bytes, hipMemcpyDeviceToDevice, st) !=
            hipSuccess)
            return S2ATTN_ERR_HIP;
    return S2ATTN_OK;
}

#define TRY(x)                 \
    do {                       \
        int st_ = (x);         \
        if (st_) return st_;   \
    } while (0)

}  // namespace

extern "C" {

s2block_config s2block_config_init(void) {
    s2block_config c;
    memset(&c, 0, sizeof(c));
    c.struct_size = sizeof(s2block_config);
    c.lora_rank = 8;
    c.lora_scale = 2.0f;
    c.rope = 0;
    c.rope_base = 10000.0f;
    c.rope_orig_len = 4096;
    return c;
}

size_t s2block_workspace_size(int is_bwd, const s2block_config* cfg) {
    s2attn_opts att;
    Dims d;
    if (check_config(cfg, is_bwd ? 1 : 0, &att, &d) != S2ATTN_OK) return 0;
    return block_ws(is_bwd ? 1 : 0, cfg, &att, d).total;
}

int s2block_fwd(const s2block_config* cfg, const void* x, const s2block_params* w, void* y,
                const s2block_saved* saved, void* ws, size_t ws_bytes, hipStream_t stream) {
    s2attn_opts att;
    Dims d;
    TRY(check_config(cfg, 0, &att, &d));
    if (!x || !y || !aligned16(x) || !aligned16(y) || !params_ok(w) || !saved_ok(saved))
        return S2ATTN_ERR_INVALID_ARG;
    const BlockWs bw = block_ws(0, cfg, &att, d);
    Gemm g;
    TRY(setup(ws, ws_bytes, bw, stream, &g));
    char* base = static_cast<char*>(ws);
    char* acat = base + bw.acat_off;
    char* xext = base + bw.xext_off;
    const int64_t M = d.M, Dm = d.Dm, Nq = d.Nq, Nkv = d.Nkv, r = d.r, ldu = 4 * r;
    const int64_t Kx = kpad(Dm + 3 * r);
    const float s = cfg->lora_scale;
    char* u = static_cast<char*>(saved->u);

    // u[:, 0:3r] = s x A_cat^T (the LoRA down-projections for q, k, v, in one
    // pass over x), then X_ext = [x | u[:, 0:3r]].
    TRY(concat_a(w, acat, d, stream));
    TRY(g.run(false, true, M, 3 * r, Dm, s, x, Dm, acat, Dm, 0.f, u, ldu, false));
    if (s2::launch_copy_cols(x, Dm, xext, Kx, M, Dm, stream) != hipSuccess ||
        s2::launch_copy_cols(u, ldu, xext + Dm * 2, Kx, M, 3 * r, stream) != hipSuccess ||
        s2::launch_copy_cols(nullptr, 0, xext + (Dm + 3 * r) * 2, Kx, M, Kx - Dm - 3 * r,
                             stream) != hipSuccess)
        return S2ATTN_ERR_HIP;
    // q, k, v = X_ext W_ext^T: W x^T + B (s A x^T) in one GEMM each
    void* outs[3] = {saved->q, saved->k, saved->v};
    const void* ws3[3] = {w->wq, w->wk, w->wv};
    const void* bs3[3] = {w->bq, w->bk, w->bv};
    const int64_t ns[3] = {Nq, Nkv, Nkv};
    for (int i = 0; i < 3; ++i) {
        char* wext = base + bw.wext_off[i];
        if (s2::launch_copy_cols(ws3[i], Dm, wext, Kx, ns[i], Dm, stream) != hipSuccess ||
            s2::launch_copy_cols(nullptr, 0, wext + Dm * 2, Kx, ns[i], Kx - Dm, stream) != hipSuccess ||
            s2::launch_copy_cols(bs3[i], r, wext + (Dm + i * r) * 2, Kx, ns[i], r, stream) !=
                hipSuccess)
            return S2ATTN_ERR_HIP;
        TRY(g.run(false, true, M, ns[i], Kx, 1.f, xext, Kx, wext, Kx, 0.f, outs[i], ns[i], false));
    }
    // attention (RoPE-PI inside)
    TRY(s2attn_fwd_ex(saved->q, saved->k, saved->v, saved->attn, saved->lse, cfg->B, cfg->L,
                      cfg->Hq, cfg->Hkv, cfg->d, cfg->G, cfg->shifted_heads, &att,
                      bw.att_bytes ? base + bw.att_off : nullptr, bw.att_bytes, stream));
    // u[:, 3r:4r] = s attn Ao^T; y = attn Wo^T + u_o Bo^T
    TRY(g.run(false, true, M, r, Nq, s, saved->attn, Nq, w->ao, Nq, 0.f, u + 3 * r * 2, ldu,
              false));
    TRY(g.run(false, true, M, Dm, Nq, 1.f, saved->attn, Nq, w->wo, Nq, 0.f, y, Dm, false));
    TRY(g.run(false, true, M, Dm, r, 1.f, u + 3 * r * 2, ldu, w->bo, r, 1.f, y, Dm, false));
    return S2ATTN_OK;
}

int s2block_bwd(const s2block_config* cfg, const void* x, const s2block_params* w,
                const s2block_saved* saved, const void* dy, const s2block_grads* gr, void* ws,
                size_t ws_bytes, hipStream_t stream) {
    s2attn_opts att;
    Dims d;
    TRY(check_config(cfg, 1, &att, &d));
    if (!x || !dy || !aligned16(x) || !aligned16(dy) || !params_ok(w) || !saved_ok(saved) || !gr)
        return S2ATTN_ERR_INVALID_ARG;
    {
        const void* ps[] = {gr->dx, gr->daq, gr->dak, gr->dav, gr->dao,
                            gr->dbq, gr->dbk, gr->dbv, gr->dbo};
        for (const void* p : ps)
            if (p == nullptr || !aligned16(p)) return S2ATTN_ERR_INVALID_ARG;
    }
    const BlockWs bw = block_ws(1, cfg, &att, d);
    Gemm g;
    TRY(setup(ws, ws_bytes, bw, stream, &g));
    char* base = static_cast<char*>(ws);
    char* t_o = base + bw.t_off;  // dy Bo
    char* dattn = base + bw.dattn_off;
    char* dqkv[3] = {base + bw.dq_off, base + bw.dk_off, base + bw.dv_off};
    char* dext = base + bw.dext_off;
    char* wdx = base + bw.wdx_off;
    float* dacat = reinterpret_cast<float*>(base + bw.dacat_off);
    const int64_t M = d.M, Dm = d.Dm, Nq = d.Nq, Nkv = d.Nkv, r = d.r, ldu = 4 * r;
    const int64_t Nt = Nq + 2 * Nkv, Kd = kpad(Nt + 3 * r);
    const float s = cfg->lora_scale;
    const char* u = static_cast<const char*>(saved->u);  // s x A^T | s attn Ao^T

    // O projection: t_o = dy Bo; dBo = dy^T u_o; dAo = s t_o^T attn; dattn = dy Wo + s t_o Ao
    TRY(g.run(false, false, M, r, Dm, 1.f, dy, Dm, w->bo, r, 0.f, t_o, r, false));
    TRY(g.run(true, false, Dm, r, M, 1.f, dy, Dm, u + 3 * r * 2, ldu, 0.f, gr->dbo, r, true));
    TRY(g.run(true, false, r, Nq, M, s, t_o, r, saved->attn, Nq, 0.f, gr->dao, Nq, true));
    TRY(g.run(false, false, M, Nq, Dm, 1.f, dy, Dm, w->wo, Nq, 0.f, dattn, Nq, false));
    TRY(g.run(false, false, M, Nq, r, s, t_o, r, w->ao, Nq, 1.f, dattn, Nq, false));
    // attention backward: gradients w.r.t. the pre-RoPE q, k and v
    TRY(s2attn_bwd_ex(saved->q, saved->k, saved->v, saved->attn, saved->lse, dattn, dqkv[0],
                      dqkv[1], dqkv[2], cfg->B, cfg->L, cfg->Hq, cfg->Hkv, cfg->d, cfg->G,
                      cfg->shifted_heads, &att, base + bw.att_off, bw.att_bytes, stream));
    // D_ext = [dq | dk | dv | s t_qkv] with t_i = dz_i B_i; dB_i = dz_i^T u_i
    const void* bs3[3] = {w->bq, w->bk, w->bv};
    const void* ws3[3] = {w->wq, w->wk, w->wv};
    float* dbs[3] = {gr->dbq, gr->dbk, gr->dbv};
    const int64_t ns[3] = {Nq, Nkv, Nkv};
    int64_t col = 0;
    for (int i = 0; i < 3; ++i) {
        if (s2::launch_copy_cols(dqkv[i], ns[i], dext + col * 2, Kd, M, ns[i], stream) !=
            hipSuccess)
            return S2ATTN_ERR_HIP;
        col += ns[i];
        TRY(g.run(false, false, M, r, ns[i], s, dqkv[i], ns[i], bs3[i], r, 0.f,
                  dext + (Nt + i * r) * 2, Kd, false));
        TRY(g.run(true, false, ns[i], r, M, 1.f, dqkv[i], ns[i], u + i * r * 2, ldu, 0.f, dbs[i],
                  r, true));
    }
    // dA_cat = (s t_qkv)^T x, split into dAq, dAk, dAv
    TRY(g.run(true, false, 3 * r, Dm, M, 1.f, dext + Nt * 2, Kd, x, Dm, 0.f, dacat, Dm, true));
    float* das[3] = {gr->daq, gr->dak, gr->dav};
    for (int i = 0; i < 3; ++i)
        if (hipMemcpyAsync(das[i], dacat + (size_t)i * r * Dm, (size_t)r * Dm * 4,
                           hipMemcpyDeviceToDevice, stream) != hipSuccess)
            return S2ATTN_ERR_HIP;
    // W_dx = [Wq; Wk; Wv; A_cat]; dx = D_ext W_dx (one GEMM, K = Nq + 2 Nkv + 3r)
    size_t off = 0;
    for (int i = 0; i < 3; ++i) {
        const size_t bytes = (size_t)ns[i] * Dm * 2;
        if (hipMemcpyAsync(wdx + off, ws3[i], bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
            return S2ATTN_ERR_HIP;
        off += bytes;
    }
    TRY(concat_a(w, wdx + off, d, stream));
    // zero padding: D_ext's last columns against W_dx's last rows
    if (s2::launch_copy_cols(nullptr, 0, dext + (Nt + 3 * r) * 2, Kd, M, Kd - Nt - 3 * r,
                             stream) != hipSuccess ||
        s2::launch_copy_cols(nullptr, 0, wdx + (Nt + 3 * r) * Dm * 2, Dm, Kd - Nt - 3 * r, Dm,
                             stream) != hipSuccess)
        return S2ATTN_ERR_HIP;
    TRY(g.run(false, false, M, Dm, Kd, 1.f, dext, Kd, wdx, Dm, 0.f, gr->dx, Dm, false));
    return S2ATTN_OK;
}

}  // extern "C"
