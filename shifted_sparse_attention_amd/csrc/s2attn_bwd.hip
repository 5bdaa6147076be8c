// S2-Attn backward kernels.
//
// With P the probabilities of a group (recomputed from the scores and the
// forward's LSE), delta_i = dO_i . O_i, dP = dO V^T and dS = P * (dP - delta):
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO,
// with dK and dV summed over the query heads that share a KV head.  Groups
// are independent, so every unit is handled by its own workgroups with no
// atomics: one kernel owns a key tile and loops over the queries after it
// (dK, dV), another owns a query tile and loops over the keys before it (dQ).
#include <math.h>

#include "s2_device.h"

namespace s2 {

// ---------------------------------------------------------------------------
// delta[b, h, t] = sum_c dO[b, t, h, c] * O[b, t, h, c]   (fp32)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(Params p, long n_rows) {
    constexpr int TPR = D / 8;          // threads per row, 8 elements each
    constexpr int RPB = 256 / TPR;      // rows per block
    const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int part = threadIdx.x % TPR;
    float acc = 0.f;
    if (row < n_rows) {
        const T* o = static_cast<const T*>(p.o) + row * D + part * 8;
        const T* g = static_cast<const T*>(p.dout) + row * D + part * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf((float)o[i], (float)g[i], acc);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
    if (row < n_rows && part == 0) {
        // row = (b * L + t) * Hq + h
        const int h = (int)(row % p.Hq);
        const long bt = row / p.Hq;
        const int t = (int)(bt % p.L);
        const int b = (int)(bt / p.L);
        p.delta[lse_idx(p, b, h, t)] = acc;
    }
}

// ---------------------------------------------------------------------------
// RoPE with position interpolation.  Angle for original position t and
// channel pair c: t * pos_scale * base^(-2c/d) (LongLoRA blog, section 3.4),
// formed and reduced modulo 2*pi in double precision so that the float
// sine/cosine see an argument below pi whatever the position.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_cs(const Params& p, int t, int c, float* cs, float* sn) {
    const double omega = pow((double)p.rope_base, -2.0 * (double)c / (double)p.d);
    const double th = (double)t * p.rope_pos_scale * omega;
    const double two_pi = 6.283185307179586476925286766559;
    const double red = th - two_pi * rint(th / two_pi);
    sincosf((float)red, sn, cs);
}

// Rotated copies of q and k (bf16 in, bf16 out), one thread per channel pair.
template <int D>
__global__ __launch_bounds__(256) void rope_prepass_kernel(Params p, bf16* qo, bf16* ko,
                                                           long q_rows, long k_rows) {
    constexpr int HALF = D / 2;
    constexpr int RPB = 256 / HALF;
    const long row = (long)blockIdx.x * RPB + threadIdx.x / HALF;
    const int c = threadIdx.x % HALF;
    if (row >= q_rows + k_rows) return;
    const bool is_q = row < q_rows;
    const long r = is_q ? row : row - q_rows;
    const int H = is_q ? p.Hq : p.Hkv;
    const int t = (int)((r / H) % p.L);
    const bf16* src = static_cast<const bf16*>(is_q ? p.q : p.k) + r * D;
    bf16* dst = (is_q ? qo : ko) + r * D;
    float cs, sn;
    rope_cs(p, t, c, &cs, &sn);
    const float x1 = (float)src[c], x2 = (float)src[c + HALF];
    dst[c] = (bf16)(x1 * cs - x2 * sn);
    dst[c + HALF] = (bf16)(x1 * sn + x2 * cs);
}

// ---------------------------------------------------------------------------
// bf16 dK / dV.  A workgroup owns 128 keys (4 waves x 32) of one KV head and
// group; K and V of a wave's keys stay in registers as MFMA B operands.  It
// loops over the query heads sharing the KV head and over 64-query tiles at
// or after its keys, staging Q and dO tiles (and their LSE and delta) in LDS.
//   S  = Q K^T, dP = dO V^T           (M = query, N = key; A from LDS rows)
//   dV^T += dO^T P,  dK^T += Q^T dS   (M = channel, K = query; A from
//                                      transposed LDS reads, B = P / dS
//                                      straight from the score registers)
// ---------------------------------------------------------------------------
constexpr int DKV_BK = 128;
constexpr int DKV_BQ = 64;

template <int D, bool GRAD_F32>
__global__ __launch_bounds__(256) void bwd_dkdv_bf16_kernel(Params p, int n_kt) {
    constexpr int KS = D / 16;
    constexpr int CB = D / 32;
    __shared__ __attribute__((aligned(16))) char smem[2 * DKV_BQ * D * 2];
    __shared__ __attribute__((aligned(16))) float s_lse[DKV_BQ];
    __shared__ __attribute__((aligned(16))) float s_dl[DKV_BQ];
    char* sQ = smem;
    char* sO = smem + DKV_BQ * D * 2;  // dO tile

    const int n_units = p.B * p.Hkv * p.n_g;
    Work w = decode_work(blockIdx.x, n_units, n_kt, p.Hkv, p.n_g);
    w.tile = n_kt - 1 - w.tile;  // key tile 0 has the most queries: issue it first
    const int hk = w.h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, l32 = lane & 31;
    const int g16 = lane >> 4, jj = lane & 15;
    const int s = head_shift(p, hk * p.r);  // all query heads of this KV head share it
    const bf16* __restrict__ q = static_cast<const bf16*>(p.q);
    const bf16* __restrict__ k = static_cast<const bf16*>(p.k);
    const bf16* __restrict__ v = static_cast<const bf16*>(p.v);
    const bf16* __restrict__ dout = static_cast<const bf16*>(p.dout);

    const int k0 = w.tile * DKV_BK;
    const int kw = k0 + wave * 32;     // first key of this wave
    const int kj = kw + l32;           // this lane's key
    const bool k_valid = kj < p.G;
    const int k_t = orig_row(w.g, p.G, k_valid ? kj : 0, s, p.L);

    bf16x8 kf[KS], vf[KS];
    {
        const size_t off = kv_row(p, w.b, k_t, hk) + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 kr = k_valid ? ld_global16(k + off + 16 * ks) : u32x4{0, 0, 0, 0};
            u32x4 vr = k_valid ? ld_global16(v + off + 16 * ks) : u32x4{0, 0, 0, 0};
            kf[ks] = __builtin_bit_cast(bf16x8, kr);
            vf[ks] = __builtin_bit_cast(bf16x8, vr);
        }
    }
    f32x16 dk[CB], dv[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        dk[cb] = f32x16{};
        dv[cb] = f32x16{};
    }

    const int qt_first = k0 / DKV_BQ;
    const int n_qt = (p.G + DKV_BQ - 1) / DKV_BQ;
    for (int hr = 0; hr < p.r; ++hr) {
        const int h = hk * p.r + hr;
        for (int qt = qt_first; qt < n_qt; ++qt) {
            const int q0 = qt * DKV_BQ;
            __syncthreads();
            {
                constexpr int CPR = D / 8;
#pragma unroll
                for (int c = tid; c < DKV_BQ * CPR; c += 256) {
                    const int row = c / CPR, col = (c % CPR) * 8;
                    const int i = q0 + row;
                    u32x4 qr = {0, 0, 0, 0}, gr = {0, 0, 0, 0};
                    if (i < p.G) {
                        const size_t off = q_row(p, w.b, orig_row(w.g, p.G, i, s, p.L), h) + col;
                        qr = ld_global16(q + off);
                        gr = ld_global16(dout + off);
                    }
                    st_lds16(sQ, tile_off<D>(row, col), qr);
                    st_lds16(sO, tile_off<D>(row, col), gr);
                }
                if (tid < DKV_BQ) {
                    const int i = q0 + tid;
                    float l2 = INFINITY, dl = 0.f;  // rows past the group: P = 0
                    if (i < p.G) {
                        const size_t li = lse_idx(p, w.b, h, orig_row(w.g, p.G, i, s, p.L));
                        l2 = p.lse[li] * kLog2e;
                        dl = p.delta[li];
                    }
                    s_lse[tid] = l2;
                    s_dl[tid] = dl;
                }
            }
            __syncthreads();
            if (q0 + DKV_BQ - 1 < kw) continue;  // every query of the tile is before every key
            const bool diag = q0 < kw + 31;

            f32x16 sacc[2], pacc[2];
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) {
                sacc[mq] = f32x16{};
                pacc[mq] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int off = tile_off<D>(32 * mq + l32, 16 * ks + 8 * hh);
                    sacc[mq] = mfma32(ld_lds16(sQ, off), kf[ks], sacc[mq]);
                    pacc[mq] = mfma32(ld_lds16(sO, off), vf[ks], pacc[mq]);
                }
            }
            // P and dS.  Row (query) index of element i: 32mq + 8(i/4) + 4hh + i%4.
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int qr0 = 32 * mq + 8 * j + 4 * hh;
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(&s_lse[qr0]);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(&s_dl[qr0]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * j + e;
                        float pv = __builtin_amdgcn_exp2f(sacc[mq][i] * p.scale_log2 - l4[e]);
                        if (diag && kj > q0 + qr0 + e) pv = 0.f;
                        sacc[mq][i] = pv;
                        pacc[mq][i] = pv * (pacc[mq][i] - d4[e]);
                    }
                }
            }
            bf16x8 pb[4], db[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float t1[8], t2[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    t1[i] = sacc[kk >> 1][8 * (kk & 1) + i];
                    t2[i] = pacc[kk >> 1][8 * (kk & 1) + i];
                }
                pb[kk] = to_bf16x8(t1);
                db[kk] = to_bf16x8(t2);
            }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int col = 32 * cb + 16 * (g16 & 1) + 4 * (jj & 3);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int row = 16 * kk + 4 * hh + (jj >> 2);
                    const bf16x8 go = cat(ld_lds_tr(sO, tile_off<D>(row, col)),
                                          ld_lds_tr(sO, tile_off<D>(row + 8, col)));
                    dv[cb] = mfma32(go, pb[kk], dv[cb]);
                    const bf16x8 qq = cat(ld_lds_tr(sQ, tile_off<D>(row, col)),
                                          ld_lds_tr(sQ, tile_off<D>(row + 8, col)));
                    dk[cb] = mfma32(qq, db[kk], dk[cb]);
                }
            }
        }
    }

    if (!k_valid) return;
    // Lane holds key kj, channels 32cb + 8j + 4hh + 0..3.
    float dkr[CB][16];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dkr[cb][i] = dk[cb][i] * p.scale;
    if (p.rope) {
        // dk = R^T dk~ on pairs (c, c + D/2): blocks cb and cb + CB/2 of the same lane.
#pragma unroll
        for (int cb = 0; cb < CB / 2; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = 32 * cb + 8 * (i >> 2) + 4 * hh + (i & 3);
                float cs, sn;
                rope_cs(p, k_t, c, &cs, &sn);
                const float g1 = dkr[cb][i], g2 = dkr[cb + CB / 2][i];
                dkr[cb][i] = g1 * cs + g2 * sn;
                dkr[cb + CB / 2][i] = -g1 * sn + g2 * cs;
            }
    }
    const size_t off = kv_row(p, w.b, k_t, hk);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 32 * cb + 8 * j + 4 * hh;
            if (GRAD_F32) {
                f32x4 a, b;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = dkr[cb][4 * j + e];
                    b[e] = dv[cb][4 * j + e];
                }
                *reinterpret_cast<f32x4*>(static_cast<float*>(p.dk) + off + c) = a;
                *reinterpret_cast<f32x4*>(static_cast<float*>(p.dv) + off + c) = b;
            } else {
                bf16x4 a, b;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = (bf16)dkr[cb][4 * j + e];
                    b[e] = (bf16)dv[cb][4 * j + e];
                }
                *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.dk) + off + c) = a;
                *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.dv) + off + c) = b;
            }
        }
}

// ---------------------------------------------------------------------------
// bf16 dQ.  A workgroup owns 128 queries (4 waves x 32) of one head and
// group; Q and dO of a wave's queries stay in registers.  It loops over the
// 64-key tiles up to its last query.
//   S^T = K Q^T, dP^T = V dO^T   (M = key; A from LDS rows, B from registers)
//   dQ^T += K^T dS^T             (A by transposed LDS reads of the K tile)
// ---------------------------------------------------------------------------
constexpr int DQ_BQ = 128;
constexpr int DQ_BK = 64;

template <int D, bool GRAD_F32>
__global__ __launch_bounds__(256) void bwd_dq_bf16_kernel(Params p, int n_qt) {
    constexpr int KS = D / 16;
    constexpr int CB = D / 32;
    __shared__ __attribute__((aligned(16))) char smem[2 * DQ_BK * D * 2];
    char* sK = smem;
    char* sV = smem + DQ_BK * D * 2;

    const int n_units = p.B * p.Hq * p.n_g;
    const Work w = decode_work(blockIdx.x, n_units, n_qt, p.Hq, p.n_g);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, l32 = lane & 31;
    const int g16 = lane >> 4, jj = lane & 15;
    const int s = head_shift(p, w.h);
    const int hk = w.h / p.r;
    const bf16* __restrict__ q = static_cast<const bf16*>(p.q);
    const bf16* __restrict__ k = static_cast<const bf16*>(p.k);
    const bf16* __restrict__ v = static_cast<const bf16*>(p.v);
    const bf16* __restrict__ dout = static_cast<const bf16*>(p.dout);

    const int q0 = w.tile * DQ_BQ;
    const int qw = q0 + wave * 32;
    const int qi = qw + l32;
    const bool q_valid = qi < p.G;
    const int q_t = orig_row(w.g, p.G, q_valid ? qi : 0, s, p.L);

    bf16x8 qf[KS], gf[KS];
    {
        const size_t off = q_row(p, w.b, q_t, w.h) + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 a = q_valid ? ld_global16(q + off + 16 * ks) : u32x4{0, 0, 0, 0};
            u32x4 b = q_valid ? ld_global16(dout + off + 16 * ks) : u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, a);
            gf[ks] = __builtin_bit_cast(bf16x8, b);
        }
    }
    float lse2 = 0.f, dl = 0.f;
    if (q_valid) {
        const size_t li = lse_idx(p, w.b, w.h, q_t);
        lse2 = p.lse[li] * kLog2e;
        dl = p.delta[li];
    }
    f32x16 dq[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dq[cb] = f32x16{};

    const int q_end = min(q0 + DQ_BQ, p.G);
    const int n_kt = (q_end + DQ_BK - 1) / DQ_BK;
    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * DQ_BK;
        __syncthreads();
        {
            constexpr int CPR = D / 8;
#pragma unroll
            for (int c = tid; c < DQ_BK * CPR; c += 256) {
                const int row = c / CPR, col = (c % CPR) * 8;
                const int j = k0 + row;
                u32x4 kr = {0, 0, 0, 0}, vr = {0, 0, 0, 0};
                if (j < p.G) {
                    const size_t off = kv_row(p, w.b, orig_row(w.g, p.G, j, s, p.L), hk) + col;
                    kr = ld_global16(k + off);
                    vr = ld_global16(v + off);
                }
                st_lds16(sK, tile_off<D>(row, col), kr);
                st_lds16(sV, tile_off<D>(row, col), vr);
            }
        }
        __syncthreads();
        if (k0 > qw + 31) continue;
        const bool diag = (k0 + DQ_BK - 1 > qw);

        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            sacc[mb] = f32x16{};
            pacc[mb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = tile_off<D>(32 * mb + l32, 16 * ks + 8 * hh);
                sacc[mb] = mfma32(ld_lds16(sK, off), qf[ks], sacc[mb]);
                pacc[mb] = mfma32(ld_lds16(sV, off), gf[ks], pacc[mb]);
            }
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
                float pv = __builtin_amdgcn_exp2f(sacc[mb][i] * p.scale_log2 - lse2);
                if (diag && key > qi) pv = 0.f;
                pacc[mb][i] = pv * (pacc[mb][i] - dl);
            }
        bf16x8 db[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float t2[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t2[i] = pacc[kk >> 1][8 * (kk & 1) + i];
            db[kk] = to_bf16x8(t2);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int col = 32 * cb + 16 * (g16 & 1) + 4 * (jj & 3);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int row = 16 * kk + 4 * hh + (jj >> 2);
                const bf16x8 kt_ = cat(ld_lds_tr(sK, tile_off<D>(row, col)),
                                       ld_lds_tr(sK, tile_off<D>(row + 8, col)));
                dq[cb] = mfma32(kt_, db[kk], dq[cb]);
            }
        }
    }

    if (!q_valid) return;
    // Lane holds query qi, channels 32cb + 8j + 4hh + 0..3 (O^T accumulator layout).
    float r_[CB][16];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) r_[cb][i] = dq[cb][i] * p.scale;
    if (p.rope) {
#pragma unroll
        for (int cb = 0; cb < CB / 2; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = 32 * cb + 8 * (i >> 2) + 4 * hh + (i & 3);
                float cs, sn;
                rope_cs(p, q_t, c, &cs, &sn);
                const float g1 = r_[cb][i], g2 = r_[cb + CB / 2][i];
                r_[cb][i] = g1 * cs + g2 * sn;
                r_[cb + CB / 2][i] = -g1 * sn + g2 * cs;
            }
    }
    const size_t off = q_row(p, w.b, q_t, w.h);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 32 * cb + 8 * j + 4 * hh;
            if (GRAD_F32) {
                f32x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = r_[cb][4 * j + e];
                *reinterpret_cast<f32x4*>(static_cast<float*>(p.dq) + off + c) = a;
            } else {
                bf16x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = (bf16)r_[cb][4 * j + e];
                *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.dq) + off + c) = a;
            }
        }
}

// ---------------------------------------------------------------------------
// fp32 backward: one thread per row, plain FMA arithmetic.
// dQ: thread per query, loop over its keys.  dK/dV: thread per key, loop
// over the query heads sharing the KV head and the queries at or after it.
// ---------------------------------------------------------------------------
constexpr int F32_ROWS = 64;

template <int D>
__global__ __launch_bounds__(F32_ROWS) void bwd_dq_f32_kernel(Params p, int n_qt) {
    __shared__ float sK[F32_ROWS][D];
    __shared__ float sV[F32_ROWS][D];
    const int n_units = p.B * p.Hq * p.n_g;
    const Work w = decode_work(blockIdx.x, n_units, n_qt, p.Hq, p.n_g);
    const int tid = threadIdx.x;
    const int s = head_shift(p, w.h);
    const int hk = w.h / p.r;
    const float* __restrict__ k = static_cast<const float*>(p.k);
    const float* __restrict__ v = static_cast<const float*>(p.v);
    const int q0 = w.tile * F32_ROWS;
    const int qi = q0 + tid;
    const bool q_valid = qi < p.G;
    const int q_t = orig_row(w.g, p.G, q_valid ? qi : 0, s, p.L);
    const size_t qo = q_row(p, w.b, q_t, w.h);
    float qr[D], gr[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = q_valid ? static_cast<const float*>(p.q)[qo + c] : 0.f;
        gr[c] = q_valid ? static_cast<const float*>(p.dout)[qo + c] : 0.f;
        acc[c] = 0.f;
    }
    const size_t li = lse_idx(p, w.b, w.h, q_t);
    const float lse = q_valid ? p.lse[li] : 0.f;
    const float dl = q_valid ? p.delta[li] : 0.f;
    const int q_end = min(q0 + F32_ROWS, p.G);
    for (int k0 = 0; k0 < q_end; k0 += F32_ROWS) {
        __syncthreads();
        for (int e = tid; e < F32_ROWS * D; e += F32_ROWS) {
            const int row = e / D, col = e % D, j = k0 + row;
            float kv = 0.f, vv = 0.f;
            if (j < p.G) {
                const size_t off = kv_row(p, w.b, orig_row(w.g, p.G, j, s, p.L), hk) + col;
                kv = k[off];
                vv = v[off];
            }
            sK[row][col] = kv;
            sV[row][col] = vv;
        }
        __syncthreads();
        const int jmax = min(F32_ROWS, qi - k0 + 1);
        for (int j = 0; j < jmax; ++j) {
            float sd = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                sd = fmaf(qr[c], sK[j][c], sd);
                dp = fmaf(gr[c], sV[j][c], dp);
            }
            const float pv = expf(sd * p.scale - lse);
            const float ds = pv * (dp - dl) * p.scale;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, sK[j][c], acc[c]);
        }
    }
    if (q_valid) {
        float* dst = static_cast<float*>(p.dq) + qo;
#pragma unroll
        for (int c = 0; c < D; ++c) dst[c] = acc[c];
    }
}

template <int D>
__global__ __launch_bounds__(F32_ROWS) void bwd_dkdv_f32_kernel(Params p, int n_kt) {
    __shared__ float sQ[F32_ROWS][D];
    __shared__ float sG[F32_ROWS][D];
    __shared__ float sL[F32_ROWS], sD[F32_ROWS];
    const int n_units = p.B * p.Hkv * p.n_g;
    Work w = decode_work(blockIdx.x, n_units, n_kt, p.Hkv, p.n_g);
    w.tile = n_kt - 1 - w.tile;
    const int hk = w.h;
    const int tid = threadIdx.x;
    const int s = head_shift(p, hk * p.r);
    const int k0 = w.tile * F32_ROWS;
    const int kj = k0 + tid;
    const bool k_valid = kj < p.G;
    const int k_t = orig_row(w.g, p.G, k_valid ? kj : 0, s, p.L);
    const size_t ko = kv_row(p, w.b, k_t, hk);
    float kr[D], vr[D], dk[D], dv[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        kr[c] = k_valid ? static_cast<const float*>(p.k)[ko + c] : 0.f;
        vr[c] = k_valid ? static_cast<const float*>(p.v)[ko + c] : 0.f;
        dk[c] = 0.f;
        dv[c] = 0.f;
    }
    for (int hr = 0; hr < p.r; ++hr) {
        const int h = hk * p.r + hr;
        for (int q0 = k0; q0 < p.G; q0 += F32_ROWS) {
            __syncthreads();
            for (int e = tid; e < F32_ROWS * D; e += F32_ROWS) {
                const int row = e / D, col = e % D, i = q0 + row;
                float a = 0.f, b = 0.f;
                if (i < p.G) {
                    const size_t off = q_row(p, w.b, orig_row(w.g, p.G, i, s, p.L), h) + col;
                    a = static_cast<const float*>(p.q)[off];
                    b = static_cast<const float*>(p.dout)[off];
                }
                sQ[row][col] = a;
                sG[row][col] = b;
            }
            {
                const int i = q0 + tid;
                float l = INFINITY, dl = 0.f;
                if (i < p.G) {
                    const size_t li = lse_idx(p, w.b, h, orig_row(w.g, p.G, i, s, p.L));
                    l = p.lse[li];
                    dl = p.delta[li];
                }
                sL[tid] = l;
                sD[tid] = dl;
            }
            __syncthreads();
            for (int i = 0; i < F32_ROWS; ++i) {
                if (q0 + i < kj) continue;  // causal: queries at or after the key
                float sd = 0.f, dp = 0.f;
#pragma unroll
                for (int c = 0; c < D; ++c) {
                    sd = fmaf(sQ[i][c], kr[c], sd);
                    dp = fmaf(sG[i][c], vr[c], dp);
                }
                const float pv = expf(sd * p.scale - sL[i]);
                const float ds = pv * (dp - sD[i]) * p.scale;
#pragma unroll
                for (int c = 0; c < D; ++c) {
                    dv[c] = fmaf(pv, sG[i][c], dv[c]);
                    dk[c] = fmaf(ds, sQ[i][c], dk[c]);
                }
            }
        }
    }
    if (k_valid) {
        float* a = static_cast<float*>(p.dk) + ko;
        float* b = static_cast<float*>(p.dv) + ko;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            a[c] = dk[c];
            b[c] = dv[c];
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_bwd_pre(const Params& p, int f32_io, hipStream_t st) {
    const long rows = (long)p.B * p.L * p.Hq;
    const int rpb = 256 / (p.d / 8);
    const long blocks = (rows + rpb - 1) / rpb;
    if (f32_io) {
        if (p.d == 128)
            hipLaunchKernelGGL((bwd_pre_kernel<float, 128>), dim3(blocks), dim3(256), 0, st, p, rows);
        else
            hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), dim3(blocks), dim3(256), 0, st, p, rows);
    } else {
        if (p.d == 128)
            hipLaunchKernelGGL((bwd_pre_kernel<bf16, 128>), dim3(blocks), dim3(256), 0, st, p, rows);
        else
            hipLaunchKernelGGL((bwd_pre_kernel<bf16, 64>), dim3(blocks), dim3(256), 0, st, p, rows);
    }
    return hipGetLastError();
}

hipError_t launch_rope_prepass(const Params& p, void* q_out, void* k_out, hipStream_t st) {
    const long q_rows = (long)p.B * p.L * p.Hq, k_rows = (long)p.B * p.L * p.Hkv;
    const int rpb = 256 / (p.d / 2);
    const long blocks = (q_rows + k_rows + rpb - 1) / rpb;
    if (p.d == 128)
        hipLaunchKernelGGL(rope_prepass_kernel<128>, dim3(blocks), dim3(256), 0, st, p,
                           static_cast<bf16*>(q_out), static_cast<bf16*>(k_out), q_rows, k_rows);
    else
        hipLaunchKernelGGL(rope_prepass_kernel<64>, dim3(blocks), dim3(256), 0, st, p,
                           static_cast<bf16*>(q_out), static_cast<bf16*>(k_out), q_rows, k_rows);
    return hipGetLastError();
}

template <int D, bool GF>
static void launch_dkdv_t(const Params& p, hipStream_t st) {
    const int n_kt = (p.G + DKV_BK - 1) / DKV_BK;
    const long blocks = (long)p.B * p.Hkv * p.n_g * n_kt;
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, GF>), dim3(blocks), dim3(256), 0, st, p, n_kt);
}

template <int D, bool GF>
static void launch_dq_t(const Params& p, hipStream_t st) {
    const int n_qt = (p.G + DQ_BQ - 1) / DQ_BQ;
    const long blocks = (long)p.B * p.Hq * p.n_g * n_qt;
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, GF>), dim3(blocks), dim3(256), 0, st, p, n_qt);
}

hipError_t launch_bwd_dkdv_bf16(const Params& p, int grad_f32, hipStream_t st) {
    if (p.d == 128)
        grad_f32 ? launch_dkdv_t<128, true>(p, st) : launch_dkdv_t<128, false>(p, st);
    else
        grad_f32 ? launch_dkdv_t<64, true>(p, st) : launch_dkdv_t<64, false>(p, st);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const Params& p, int grad_f32, hipStream_t st) {
    if (p.d == 128)
        grad_f32 ? launch_dq_t<128, true>(p, st) : launch_dq_t<128, false>(p, st);
    else
        grad_f32 ? launch_dq_t<64, true>(p, st) : launch_dq_t<64, false>(p, st);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const Params& p, hipStream_t st) {
    const int n_kt = (p.G + F32_ROWS - 1) / F32_ROWS;
    const long blocks = (long)p.B * p.Hkv * p.n_g * n_kt;
    if (p.d == 128)
        hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, dim3(blocks), dim3(F32_ROWS), 0, st, p, n_kt);
    else
        hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, dim3(blocks), dim3(F32_ROWS), 0, st, p, n_kt);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const Params& p, hipStream_t st) {
    const int n_qt = (p.G + F32_ROWS - 1) / F32_ROWS;
    const long blocks = (long)p.B * p.Hq * p.n_g * n_qt;
    if (p.d == 128)
        hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, dim3(blocks), dim3(F32_ROWS), 0, st, p, n_qt);
    else
        hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, dim3(blocks), dim3(F32_ROWS), 0, st, p, n_qt);
    return hipGetLastError();
}

}  // namespace s2
