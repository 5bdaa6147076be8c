// S2-Attn forward kernels.
//
// One workgroup computes a tile of queries of one group of one head (a unit
// (b, h, g)).  Rows are read and written at their original positions through
// the roll map (orig_row), so the roll / regroup / un-roll of the method
// (nearauto.com LongLoRA article, shift-short-attention section: shift half
// the heads, then fold groups into the batch) never materialises a copy.
// Causal masking uses in-group indices in rolled order.
#include <math.h>

#include "s2_device.h"

namespace s2 {

// ---------------------------------------------------------------------------
// bf16 forward.  8 waves x 32 queries per workgroup; K and V tiles of 128
// keys are staged in LDS by direct global->LDS loads into two buffers, so the
// next tile streams in while the current one is consumed (one barrier per
// tile).
// Scores are formed transposed, S^T = K Q^T, so a lane owns one query column
// and 16 of the 32 keys of each 32-key block (the other 16 sit in lane ^ 32):
// the row max needs one permlane32 swap, the row sum none until the end.
// P^T feeds O^T += V^T P^T directly from the score registers; V is read from
// its row-major tile with transposed LDS reads.  The epilogue stages O through
// LDS so that every global store writes whole rows.
// ---------------------------------------------------------------------------
constexpr int FWD_WAVES = 8;
constexpr int FWD_BM = 32 * FWD_WAVES;
constexpr int FWD_BN = 128;
constexpr int FWD_THREADS = 64 * FWD_WAVES;

// ROPE: rotate the query fragments after loading them (k arrives rotated).
template <int D, bool ROPE>
__global__ __launch_bounds__(FWD_THREADS) void fwd_bf16_kernel(Params p, int n_qt) {
    constexpr int KS = D / 16;  // MFMA k-steps over the head dimension
    constexpr int CB = D / 32;  // 32-channel blocks of the output
    constexpr int TILE = FWD_BN * D * 2;
    constexpr int NCH = TILE / 1024;  // 1 KB DMA chunks per tile
    constexpr int MB = FWD_BN / 32;   // 32-key blocks of a tile
    constexpr int KK = FWD_BN / 16;   // 16-key MFMA k-steps of P V
    __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILE];

    const int n_units = p.B * p.Hq * p.n_g;
    const Work w = decode_work(blockIdx.x, n_units, n_qt, p.Hq, p.n_g, p.band);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, l32 = lane & 31;
    const int g16 = lane >> 4, jj = lane & 15;
    const int s = head_shift(p, w.h);
    const int hk = w.h / p.r;
    const bf16* __restrict__ q = static_cast<const bf16*>(p.q);
    const bf16* __restrict__ k = static_cast<const bf16*>(p.k);
    const bf16* __restrict__ v = static_cast<const bf16*>(p.v);

    const int q0 = w.tile * FWD_BM;
    const int qw = q0 + wave * 32;   // first query (in-group index) of this wave
    const int qi = qw + l32;         // this lane's query
    const bool q_valid = qi < p.G;
    const int q_end = min(q0 + FWD_BM, p.G);
    const int n_kt = (q_end + FWD_BN - 1) / FWD_BN;

    // K, V tile kt -> buffer `buf`.  Rows past the group are clamped to its last
    // row: those keys come after every query, so the causal mask removes them.
    constexpr int NSLOT = 2 * NCH / FWD_WAVES;  // 1 KB chunks per wave per tile; K first, then V
    const uint32_t rowb = (uint32_t)p.Hkv * D * 2;
    const size_t plane = ((size_t)w.b * p.L * p.Hkv + hk) * D;
    // K and V use the same chunks (j and j + NSLOT/2), so a wave holds
    // NSLOT/2 slots.  A tile that neither wraps past the end of the sequence
    // nor runs past the group is one run of rows starting at original row
    // t0: its loads take a wave-uniform base and a fixed per-lane offset,
    // with no per-load address arithmetic.
    constexpr int NS2 = NSLOT / 2;
    static_assert(NSLOT % 2 == 0 && (FWD_WAVES * NS2) % NCH == 0, "K and V share chunk slots");
    ChunkSlot slot[NS2];
    uint32_t lane_off[NS2];
#pragma unroll
    for (int j = 0; j < NS2; ++j) {
        slot[j] = chunk_slot<D>((wave + FWD_WAVES * j) % NCH, lane);
        lane_off[j] = (uint32_t)slot[j].row * rowb + slot[j].colb;
    }
    auto stage = [&](int kt, int buf) {
        char* base = smem + buf * 2 * TILE;
        int t0 = w.g * p.G + s + kt * FWD_BN;  // original row of in-group index kt * FWD_BN
        if (t0 >= p.L) t0 -= p.L;
        const bool run = kt * FWD_BN + FWD_BN <= p.G && t0 + FWD_BN <= p.L;
        if (run) {
            const char* kb = reinterpret_cast<const char*>(k + plane) + (size_t)t0 * rowb;
            const char* vb = reinterpret_cast<const char*>(v + plane) + (size_t)t0 * rowb;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const bool isv = j >= NS2;
                const int cc = (wave + FWD_WAVES * j) % NCH;
                dma16(isv ? vb : kb, lane_off[j % NS2], base + (isv ? TILE : 0) + cc * 1024);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const bool isv = j >= NS2;
                const int cc = (wave + FWD_WAVES * j) % NCH;
                const ChunkSlot& sl = slot[j % NS2];
                const uint32_t off = row_off(w.g, p.G, kt * FWD_BN + sl.row, s, p.L, rowb) + sl.colb;
                dma16((isv ? v : k) + plane, off, base + (isv ? TILE : 0) + cc * 1024);
            }
        }
    };
    stage(0, 0);

    bf16x8 qf[KS];
    {
        const int q_t = orig_row(w.g, p.G, q_valid ? qi : 0, s, p.L);
        const bf16* qr = q + q_row(p, w.b, q_t, w.h) + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 raw = q_valid ? ld_global16(qr + 16 * ks) : u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, raw);
        }
        // RoPE on the stationary query: fragment ks holds channels
        // 16 ks + 8 hh + i, and its pair partner (+ D/2) sits in fragment
        // ks + KS/2 of the same lane, so the rotation stays in registers.
        if constexpr (ROPE) {
#pragma unroll
            for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const BfPair r2 = rope_turn(p, q_t, 16 * ks + 8 * hh + i, qf[ks][i], qf[ks + KS / 2][i]);
                    qf[ks][i] = r2.a;
                    qf[ks + KS / 2][i] = r2.b;
                }
        }
    }

    f32x16 oacc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
    float m = -INFINITY, lsum = 0.f;
    constexpr float kLazy = 8.0f;
    const float lazy_raw = kLazy / p.scale_log2;

    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * FWD_BN;
        wait_vmem();
        __syncthreads();
        if (kt + 1 < n_kt) stage(kt + 1, (kt + 1) & 1);
        if (k0 > qw + 31) continue;  // every key of the tile is after every query of the wave
        const char* sK = smem + (kt & 1) * 2 * TILE;
        const char* sV = sK + TILE;

        f32x16 sacc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            sacc[mb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 a = ld_lds16(sK, tile_off<D>(32 * mb + l32, 16 * ks + 8 * hh));
                sacc[mb] = mfma32(a, qf[ks], sacc[mb]);
            }
        }
        // Keep several K reads in flight ahead of the MFMAs that consume them.
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < MB * KS - 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);

        // Raw scores; keys after the query are -inf (only on diagonal tiles).
        if (k0 + FWD_BN - 1 > qw) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
                    if (key > qi) sacc[mb][i] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mb][i]);
        mx = xhalf_max(mx);
        // The reference maximum m (raw score units) moves only when a score
        // exceeds it by more than kLazy / scale_log2 (a factor 2^kLazy in the
        // exponentials): O and l are then rescaled together, so every row
        // keeps one consistent reference and the result is exact.
        if (__builtin_amdgcn_ballot_w64(mx > m + lazy_raw) != 0) {
            const float m_new = fmaxf(m, mx);
            const float alpha = __builtin_amdgcn_exp2f((m - m_new) * p.scale_log2);
            m = m_new;
            lsum *= alpha;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;
        }
        const float mc = m * p.scale_log2;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = __builtin_amdgcn_exp2f(fmaf(sacc[mb][i], p.scale_log2, -mc));
                sacc[mb][i] = e;
                lsum += e;
            }

        bf16x8 pb[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            float tmp[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) tmp[i] = sacc[kk >> 1][8 * (kk & 1) + i];
            pb[kk] = to_bf16x8(tmp);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int col = 32 * cb + 16 * (g16 & 1) + 4 * (jj & 3);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int row = 16 * kk + 4 * hh + (jj >> 2);
                bf16x4 a0 = ld_lds_tr(sV, tile_off<D>(row, col));
                bf16x4 a1 = ld_lds_tr(sV, tile_off<D>(row + 8, col));
                oacc[cb] = mfma32(cat(a0, a1), pb[kk], oacc[cb]);
            }
        }
        // Same for the transposed V reads (two per MFMA).
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < KK * CB - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }

    // Epilogue: O / l through LDS (each wave its own 32 rows), then whole-row stores.
    const float l_tot = xhalf_sum(lsum);
    const float inv = 1.0f / l_tot;
    __syncthreads();  // every wave is done with the K/V buffers
    char* so = smem + wave * 32 * D * 2;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 val;
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = (bf16)(oacc[cb][4 * j + e] * inv);
            *reinterpret_cast<bf16x4*>(so + tile_off<D>(l32, 32 * cb + 8 * j + 4 * hh)) = val;
        }
    }
    if (q_valid && hh == 0)
        p.lse[lse_idx(p, w.b, w.h, orig_row(w.g, p.G, qi, s, p.L))] = fmaf(m, p.scale, log2f(l_tot) * kLn2);
    __syncthreads();
    constexpr int LPR = D / 8;
    bf16* o = static_cast<bf16*>(p.o);
#pragma unroll
    for (int it = 0; it < 32 * LPR / 64; ++it) {
        const int id = it * 64 + lane;
        const int row = id / LPR, col = (id % LPR) * 8;
        const int i = qw + row;
        if (i < p.G) {
            const u32x4 val = *reinterpret_cast<const u32x4*>(so + tile_off<D>(row, col));
            *reinterpret_cast<u32x4*>(o + q_row(p, w.b, orig_row(w.g, p.G, i, s, p.L), w.h) + col) = val;
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 forward: one thread per query row, 64 rows per workgroup, K/V tiles of
// 64 keys in LDS, exact online softmax in natural exponentials.  Plain fp32
// FMA arithmetic throughout.
// ---------------------------------------------------------------------------
constexpr int F32_ROWS = 64;

template <int D>
__global__ __launch_bounds__(F32_ROWS) void fwd_f32_kernel(Params p, int n_qt) {
    __shared__ float sK[F32_ROWS][D];
    __shared__ float sV[F32_ROWS][D];
    const int n_units = p.B * p.Hq * p.n_g;
    const Work w = decode_work(blockIdx.x, n_units, n_qt, p.Hq, p.n_g, p.band);
    const int tid = threadIdx.x;
    const int s = head_shift(p, w.h);
    const int hk = w.h / p.r;
    const float* __restrict__ q = static_cast<const float*>(p.q);
    const float* __restrict__ k = static_cast<const float*>(p.k);
    const float* __restrict__ v = static_cast<const float*>(p.v);

    const int q0 = w.tile * F32_ROWS;
    const int qi = q0 + tid;
    const bool q_valid = qi < p.G;
    const int q_t = orig_row(w.g, p.G, q_valid ? qi : 0, s, p.L);
    float qr[D], acc[D];
    const float* qp = q + q_row(p, w.b, q_t, w.h);
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = q_valid ? qp[c] : 0.f;
        acc[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
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
        const int jmax = min(F32_ROWS, qi - k0 + 1);  // keys k0 .. qi
        for (int j = 0; j < jmax; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) dot = fmaf(qr[c], sK[j][c], dot);
            const float x = dot * p.scale;
            if (x > m) {
                const float a = expf(m - x);
                l *= a;
#pragma unroll
                for (int c = 0; c < D; ++c) acc[c] *= a;
                m = x;
            }
            const float e = expf(x - m);
            l += e;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = fmaf(e, sV[j][c], acc[c]);
        }
    }
    if (q_valid) {
        float* op = static_cast<float*>(p.o) + q_row(p, w.b, q_t, w.h);
        const float inv = 1.0f / l;
#pragma unroll
        for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
        p.lse[lse_idx(p, w.b, w.h, q_t)] = m + logf(l);
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_fwd_bf16(const Params& p0, hipStream_t st) {
    const int n_qt = (p0.G + FWD_BM - 1) / FWD_BM;
    const long blocks = (long)p0.B * p0.Hq * p0.n_g * n_qt;
    Params p = p0;
    p.band = dispatch_band(p.B * p.Hq * p.n_g, (size_t)p.G * p.d * 4);  // K and V of the unit
    auto kernel = p.d == 128 ? (p.rope ? fwd_bf16_kernel<128, true> : fwd_bf16_kernel<128, false>)
                             : (p.rope ? fwd_bf16_kernel<64, true> : fwd_bf16_kernel<64, false>);
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(FWD_THREADS), 0, st, p, n_qt);
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const Params& p, hipStream_t st) {
    const int n_qt = (p.G + F32_ROWS - 1) / F32_ROWS;
    const long blocks = (long)p.B * p.Hq * p.n_g * n_qt;
    if (p.d == 128)
        hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(blocks), dim3(F32_ROWS), 0, st, p, n_qt);
    else
        hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(blocks), dim3(F32_ROWS), 0, st, p, n_qt);
    return hipGetLastError();
}

}  // namespace s2
