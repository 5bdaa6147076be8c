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

#include <type_traits>

#include "s2_device.h"

namespace s2 {

// dS tile layout (see Params::ds): tiles per (batch, head, group) unit, and
// the number of tile (q32, k32), k32 <= q32, within its unit.
__device__ __forceinline__ size_t ds_unit_tiles(int G) {
    const size_t nb = ((size_t)(G + 31) / 32 + 7) / 8;
    return 32 * nb * (nb + 1);
}
__device__ __forceinline__ size_t ds_tile(int q32, int k32) {
    const size_t t = (size_t)(q32 >> 3);
    return 32 * t * (t + 1) + 8 * (size_t)k32 + (q32 & 7);
}

// ---------------------------------------------------------------------------
// The row term, stored negated: p.delta[b, h, t] = -sum_c dO[b, t, h, c] *
// O[b, t, h, c] (fp32; the dK/dV kernel starts its dP accumulation from it,
// so the MFMA yields dP - delta directly).
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
        p.delta[lse_idx(p, b, h, t)] = -acc;
    }
}

// Rotated copies of q (when qo is set) and k (bf16 in, bf16 out).  A thread turns 8 channel
// pairs: 16 bytes from each half of the row in, 16 bytes to each half out.
template <int D>
__global__ __launch_bounds__(256) void rope_prepass_kernel(Params p, bf16* qo, bf16* ko,
                                                           long q_rows, long k_rows) {
    constexpr int HALF = D / 2;
    constexpr int TPR = HALF / 8;  // threads per row
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const long row = gid / TPR;
    const int c0 = (int)(gid % TPR) * 8;
    if (row >= q_rows + k_rows) return;
    const bool is_q = row < q_rows;
    const long r = is_q ? row : row - q_rows;
    const int H = is_q ? p.Hq : p.Hkv;
    const int t = (int)((r / H) % p.L);
    const bf16* src = static_cast<const bf16*>(is_q ? p.q : p.k) + r * D + c0;
    bf16* dst = (is_q ? qo : ko) + r * D + c0;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(src);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(src + HALF);
    bf16x8 oa, ob;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const BfPair r2 = rope_turn(p, t, c0 + i, a[i], b[i]);
        oa[i] = r2.a;
        ob[i] = r2.b;
    }
    *reinterpret_cast<bf16x8*>(dst) = oa;
    *reinterpret_cast<bf16x8*>(dst + HALF) = ob;
}

// ---------------------------------------------------------------------------
// Gradient rows out of the accumulators.  A wave's accumulator holds row
// row0 + l32 and channels 32cb + 8j + 4hh + e (the O^T layout of the MFMA).
// `grad_rows` scales them (and rotates dq~ / dk~ back when RoPE was applied);
// bf16 rows are then staged in LDS and written as whole rows by
// `flush_rows`, fp32 rows go straight from registers.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void grad_rows(const Params& p, f32x16* acc, float mul, int g, int s,
                                          int row0, int lane, bool rope_rows) {
    constexpr int CB = D / 32;
    const int hh = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] *= mul;
    if (rope_rows) {
        const int i = row0 + l32;
        const int t = orig_row(g, p.G, i < p.G ? i : 0, s, p.L);
        // pairs (c, c + D/2) sit in blocks cb and cb + CB/2 of the same lane
#pragma unroll
        for (int cb = 0; cb < CB / 2; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int c = 32 * cb + 8 * (e >> 2) + 4 * hh + (e & 3);
                float cs, sn;
                rope_cs(p, t, c, &cs, &sn);
                const float g1 = acc[cb][e], g2 = acc[cb + CB / 2][e];
                acc[cb][e] = g1 * cs + g2 * sn;
                acc[cb + CB / 2][e] = -g1 * sn + g2 * cs;
            }
    }
}

template <int D>
__device__ __forceinline__ void stage_rows_bf16(const f32x16* r_, char* stage_lds, int lane) {
    constexpr int CB = D / 32;
    const int hh = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 a;
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = (bf16)r_[cb][4 * j + e];
            *reinterpret_cast<bf16x4*>(stage_lds + tile_off<D>(l32, 32 * cb + 8 * j + 4 * hh)) = a;
        }
}

template <int D>
__device__ __forceinline__ void store_rows_f32(const Params& p, const f32x16* r_, void* dst, int b,
                                               int H, int h, int g, int s, int row0, int lane) {
    constexpr int CB = D / 32;
    const int hh = lane >> 5, l32 = lane & 31;
    const int i = row0 + l32;
    if (i >= p.G) return;
    const int t = orig_row(g, p.G, i, s, p.L);
    float* out = static_cast<float*>(dst) + ((size_t)(b * (size_t)p.L + t) * H + h) * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 a;
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = r_[cb][4 * j + e];
            *reinterpret_cast<f32x4*>(out + 32 * cb + 8 * j + 4 * hh) = a;
        }
}

// Write 32 staged bf16 rows as whole rows (LPR lanes per row, 16 bytes each).
template <int D>
__device__ __forceinline__ void flush_rows(const Params& p, const char* stage_lds, void* dst, int b,
                                           int H, int h, int g, int s, int row0, int lane) {
    constexpr int LPR = D / 8;
    bf16* out = static_cast<bf16*>(dst);
#pragma unroll
    for (int it = 0; it < 32 * LPR / 64; ++it) {
        const int id = it * 64 + lane;
        const int row = id / LPR, col = (id % LPR) * 8;
        const int i = row0 + row;
        if (i < p.G) {
            const u32x4 val = *reinterpret_cast<const u32x4*>(stage_lds + tile_off<D>(row, col));
            const int t = orig_row(g, p.G, i, s, p.L);
            *reinterpret_cast<u32x4*>(out + ((size_t)(b * (size_t)p.L + t) * H + h) * D + col) = val;
        }
    }
}

// Sum a key group's two partial accumulators (the wave with qh = 1 hands
// its partial to the wave with qh = 0 through LDS) and store the rows.
// Every wave of the workgroup calls it (it holds workgroup barriers).
template <int D, bool GRAD_F32>
__device__ __forceinline__ void reduce_store(const Params& p, f32x16 (&acc)[D / 32], f32x4* red,
                                             char* stg, float mul, bool rope_rows, void* dst,
                                             int b, int hk, int g, int s, int kw, int lane,
                                             int qh) {
    constexpr int CB = D / 32;
    __syncthreads();  // previous readers of the LDS areas are done
    if (qh == 1) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[(cb * 4 + j) * 64 + lane] = f32x4{acc[cb][4 * j], acc[cb][4 * j + 1],
                                                      acc[cb][4 * j + 2], acc[cb][4 * j + 3]};
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 o = red[(cb * 4 + j) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[cb][4 * j + e] += o[e];
            }
        grad_rows<D>(p, acc, mul, g, s, kw, lane, rope_rows);
    }
    if (GRAD_F32) {
        if (qh == 0) store_rows_f32<D>(p, acc, dst, b, p.Hkv, hk, g, s, kw, lane);
        return;
    }
    if (qh == 0) stage_rows_bf16<D>(acc, stg, lane);
    __syncthreads();
    if (qh == 0) flush_rows<D>(p, stg, dst, b, p.Hkv, hk, g, s, kw, lane);
}

// ---------------------------------------------------------------------------
// bf16 dK / dV.  A workgroup owns 128 keys of one KV head and group, held by
// 8 waves: waves w and w+4 share keys 32(w%4) .. +31 and split every 64-query
// tile into its first and second 32 queries; each keeps partial dK, dV for
// its keys, and the two halves are summed through LDS at the end.  The K and
// V rows of the workgroup's keys sit in LDS for the whole kernel (MFMA B
// operands; half of each wave's K fragments are also kept in registers).  The workgroup walks the query heads sharing the KV head and,
// for each, the 64-query tiles at or after its keys; Q, dO, LSE and delta of
// the next tile stream into the other of two LDS buffers while the current
// one is consumed.
//   S  = Q K^T, dP = dO V^T           (M = query, N = key; A and B from LDS rows)
//   dV^T += dO^T P,  dK^T += Q^T dS   (M = channel, K = query; A from
//                                      transposed LDS reads, B = P / dS
//                                      straight from the score registers)
// ---------------------------------------------------------------------------
constexpr int DKV_WAVES = 8;
constexpr int DKV_BK = 128;
constexpr int DKV_BQ = 64;
// P and dS enter the dV and dK products as bf16, each rounded by up to 2^-9
// of itself.  The terms of a query row with the largest P dominate those
// sums (the first rows of a group, where a query sees few keys, or rows with
// concentrated attention), so a 32 x 32 tile whose largest P reaches 1/16
// adds the products of the residuals x - bf16(x), rounded to bf16 in turn:
// about 16 bits of P and dS there.  Tiles below it hold terms at least 16
// times smaller than the largest of their row.  With standard-normal inputs
// at the 32k-token shapes (groups of 8192) about 0.13% of tiles qualify.
constexpr float kSplitP = 0.0625f;

template <int D, bool GRAD_F32, bool SPLIT>
__global__ __launch_bounds__(64 * DKV_WAVES) void bwd_dkdv_bf16_kernel(Params p, int n_kt) {
    constexpr int KS = D / 16;
    constexpr int CB = D / 32;
    constexpr int TILE = DKV_BQ * D * 2;             // one Q or dO tile
    constexpr int KTILE = DKV_BK * D * 2;            // the workgroup's K (or V) rows
    constexpr int NCH = TILE / 1024;
    constexpr int KNCH = KTILE / 1024;
    constexpr int BUF = 2 * TILE + 2 * DKV_BQ * 4;   // Q, dO, lse, delta
    constexpr int RED = CB * 4 * 64 * 16;            // one wave's fp32 partial (dK or dV)
    static_assert(4 * RED <= 2 * BUF + 2 * KTILE, "reduction area");
    // With SPLIT, the residual stash of split steps (kSplitP): per wave 4 KB,
    // the P and dS residuals of its 32 x 32 tile.  Where that does not fit
    // beside the buffers (D = 128), the first 1 KB of the dS residual goes to
    // the K rows' channels held in registers (kreg), whose LDS copy is not
    // read.
    constexpr int NOSTASH = 2 * KTILE + 2 * BUF;
    constexpr bool DS0_IN_K = SPLIT && NOSTASH + DKV_WAVES * 4096 > 160 * 1024;
    constexpr int STASH_W = !SPLIT ? 0 : DS0_IN_K ? 3072 : 4096;   // per wave, beside the buffers
    __shared__ __attribute__((aligned(1024))) char smem[NOSTASH + DKV_WAVES * STASH_W];
    char* sKt = smem;
    char* sVt = smem + KTILE;
    char* bufs = smem + 2 * KTILE;

    const int n_units = p.B * p.Hkv * p.n_g;
    Work w = decode_work(blockIdx.x, n_units, n_kt, p.Hkv, p.n_g, p.band);
    w.tile = n_kt - 1 - w.tile;  // key tile 0 has the most queries: issue it first
    const int hk = w.h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3, qh = wave >> 2;  // key group, query half
    const int hh = lane >> 5, l32 = lane & 31;
    const int g16 = lane >> 4, jj = lane & 15;
    const int s = head_shift(p, hk * p.r);  // all query heads of this KV head share it
    const bf16* __restrict__ q = static_cast<const bf16*>(p.q);
    const bf16* __restrict__ k = static_cast<const bf16*>(p.k);
    const bf16* __restrict__ v = static_cast<const bf16*>(p.v);
    const bf16* __restrict__ dout = static_cast<const bf16*>(p.dout);

    const int k0 = w.tile * DKV_BK;
    const int kw = k0 + kg * 32;       // first key of this wave
    const int kj = kw + l32;           // this lane's key
    const int qt_first = k0 / DKV_BQ;
    const int nq = (p.G + DKV_BQ - 1) / DKV_BQ - qt_first;
    const int n_it = p.r * nq;

    // The workgroup's K and V rows (rows past the group clamped; their
    // gradients are never stored).
    {
        const uint32_t rowb = (uint32_t)p.Hkv * D * 2;
        const size_t plane = ((size_t)w.b * p.L * p.Hkv + hk) * D;
        for (int c = wave; c < 2 * KNCH; c += DKV_WAVES) {
            const bool isv = c >= KNCH;
            const int cc = isv ? c - KNCH : c;
            const ChunkSlot sl = chunk_slot<D>(cc, lane);
            const uint32_t off = row_off(w.g, p.G, k0 + sl.row, s, p.L, rowb) + sl.colb;
            dma16((isv ? v : k) + plane, off, (isv ? sVt : sKt) + cc * 1024);
        }
    }
    // Q, dO, lse, delta of a step: query head h, tile qt_first + t.  Steps
    // walk t = 0 .. nq - 1 for each query head of the KV head in turn.  Rows
    // past the group are clamped to its last row and masked in the loop.
    constexpr int NSLOT = 2 * NCH / DKV_WAVES;  // 1 KB chunks per wave per tile; Q first, then dO
    const uint32_t qrowb = (uint32_t)p.Hq * D * 2;
    auto stage = [&](int h, int t, int buf) {
        char* base = bufs + buf * BUF;
        const int q0 = (qt_first + t) * DKV_BQ;
        const size_t plane = ((size_t)w.b * p.L * p.Hq + h) * D;
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            const bool isg = j >= NSLOT / 2;
            const int cc = (wave + DKV_WAVES * j) % NCH;
            const ChunkSlot sl = chunk_slot<D>(cc, lane);  // recomputed: frees registers for kreg
            const uint32_t off = row_off(w.g, p.G, q0 + sl.row, s, p.L, qrowb) + sl.colb;
            dma16((isg ? dout : q) + plane, off, base + (isg ? TILE : 0) + cc * 1024);
        }
        if (wave < 2) {  // LSE and delta of the tile's 64 queries
            const float* rb = (wave == 0 ? p.lse : p.delta) + ((size_t)w.b * p.Hq + h) * p.L;
            const uint32_t off = 4u * (uint32_t)orig_row(w.g, p.G, min(q0 + lane, p.G - 1), s, p.L);
            dma4(rb, off, base + 2 * TILE + wave * DKV_BQ * 4);
        }
    };
    stage(hk * p.r, 0, 0);

    // The first KREG channel blocks of this wave's K rows stay in registers
    // (the B operands of S for k-steps ks < KREG): fewer LDS reads per step,
    // within the register budget of two waves per SIMD.
    // (Two 16-channel blocks: with four the register budget spills.)
    constexpr int KREG = 2;
    static_assert(!DS0_IN_K || (D == 128 && KREG == 2), "the K rows' unread block is 64 bytes of a row");
    bf16x8 kreg[KREG];
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KREG; ++ks) kreg[ks] = ld_lds16(sKt, tile_off<D>(32 * kg + l32, 16 * ks + 8 * hh));

    f32x16 dk[CB], dv[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        dk[cb] = f32x16{};
        dv[cb] = f32x16{};
    }

    // dS tiles of the current query head (see Params::ds): the head's base,
    // and the tile of this wave's keys in query row q32 at
    // + ds_tile(q32, kw / 32) * 2048.
    const size_t TT = ds_unit_tiles(p.G);
    auto ds_head = [&](int h) {
        return p.ds == nullptr ? nullptr
                               : static_cast<char*>(p.ds) +
                                     (((size_t)w.b * p.Hq + h) * p.n_g + w.g) * TT * 2048;
    };
    // This lane's 16-byte slot for part kk (0, 1) of the P (which = 0) or dS
    // (which = 1) residual: chunk 64 kk + lane of that tile.  At D = 128 the
    // dS residual's part 0 sits in K row r = 16 wave + lane / 4, in the 64
    // bytes holding channels 0..31 (logical slots 0..3, physically slots
    // 4 (r & 3) .. + 3 under the row's XOR swizzle).  Formed where it is used
    // (the empty asm keeps the addresses out of the loop's live set).
    auto res_slot = [&](int which, int kk) -> char* {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        char* free_w = smem + NOSTASH + wave * STASH_W;
        if constexpr (DS0_IN_K) {
            if (which == 0) return free_w + 1024 * kk + 16 * ln;
            if (kk == 1) return free_w + 2048 + 16 * ln;
            const int r = 16 * wave + ln / 4;
            return sKt + r * (D * 2) + 64 * (r & 3) + 16 * (ln % 4);
        } else {
            return free_w + 2048 * which + 1024 * kk + 16 * ln;
        }
    };
    int h = hk * p.r, t = 0;   // current step
    char* ds_base = ds_head(h);
    // dS stores of the previous step still in flight (0 or 2; wave-uniform):
    // they were issued after that step's loads, so waiting down to them awaits
    // the loads and leaves the stores a whole step to drain.
    int ds_inflight = 0;
    for (int it = 0; it < n_it; ++it) {
        if (ds_inflight)
            wait_vmem_n<2>();
        else
            wait_vmem();
        // Wave 0 loaded this step's LSE (natural log) into LDS: turn it into
        // base 2 in place before the barrier publishes the buffer.
        if (wave == 0) {
            float* l = reinterpret_cast<float*>(bufs + (it & 1) * BUF + 2 * TILE) + lane;
            *l *= kLog2e;
        }
        __syncthreads();
        if (it + 1 < n_it) {
            if (t + 1 < nq)
                stage(h, t + 1, (it + 1) & 1);
            else
                stage(h + 1, 0, (it + 1) & 1);
        }
        ds_inflight = 0;
        const int qb = (qt_first + t) * DKV_BQ + 32 * qh;  // first query of this wave
        char* const it_ds = ds_base;
        if (++t == nq) {
            t = 0;
            ++h;
            ds_base = ds_head(h);
        }
        if (qb + 31 < kw) continue;  // every query of the half-tile is before every key
        const bool masked = (qb < kw + 31) || (qb + 32 > p.G);
        const char* sQ = bufs + (it & 1) * BUF + 32 * qh * D * 2;
        const char* sO = sQ + TILE;
        const float* s_lse = reinterpret_cast<const float*>(bufs + (it & 1) * BUF + 2 * TILE) + 32 * qh;  // base 2
        const float* s_dl = s_lse + DKV_BQ;

        // dP accumulates onto -delta of its query row (element i is row
        // 8(i/4) + 4hh + i%4), so pacc ends as dP - delta.
        f32x16 sacc = f32x16{}, pacc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(&s_dl[8 * j + 4 * hh]);
#pragma unroll
            for (int e = 0; e < 4; ++e) pacc[4 * j + e] = d4[e];
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = tile_off<D>(l32, 16 * ks + 8 * hh);
            const int koff = tile_off<D>(32 * kg + l32, 16 * ks + 8 * hh);
            const bf16x8 kf = ks < KREG ? kreg[ks < KREG ? ks : 0] : ld_lds16(sKt, koff);
            sacc = mfma32(ld_lds16(sQ, off), kf, sacc);
            pacc = mfma32(ld_lds16(sO, off), ld_lds16(sVt, koff), pacc);
        }
        // LDS operand reads run 8 ahead of the MFMAs that use them, then two
        // per MFMA: the default schedule kept them one or two ahead, so each
        // MFMA waited on its own operands (5% of the kernel).
        {
            constexpr int NR = 4 * KS - KREG, NM = 2 * KS, AHEAD = 8, PAIRS = (NR - AHEAD) / 2;
            __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
            for (int i = 0; i < PAIRS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NM - PAIRS, 0);
        }
        // P and dS; element i is query qb + 8(i/4) + 4hh + i%4 and key kj.
        auto softmax_grad = [&](bool mask) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r0 = 8 * j + 4 * hh;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(&s_lse[r0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * j + e;
                    float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i], p.scale_log2, -l4[e]));
                    if (mask) {
                        const int qq = qb + r0 + e;
                        if (kj > qq || qq >= p.G) pv = 0.f;
                    }
                    sacc[i] = pv;
                    pacc[i] = pv * pacc[i];
                }
            }
        };
        if (masked)
            softmax_grad(true);
        else
            softmax_grad(false);
        bf16x8 pb[2], db[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            float t1[8], t2[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                t1[i] = sacc[8 * kk + i];
                t2[i] = pacc[8 * kk + i];
            }
            pb[kk] = to_bf16x8(t1);
            db[kk] = to_bf16x8(t2);
        }
        // A tile holding a probability of at least 1/16 also feeds the
        // rounding residuals of P and dS (their next 8 bits, bf16(x -
        // bf16(x))) to dV and dK; see kSplitP.
        // (P >= 0, so the largest P has the largest bit pattern.)
        uint32_t pmax = __float_as_uint(sacc[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) pmax = max(pmax, __float_as_uint(sacc[i]));
        const bool split = SPLIT && __builtin_amdgcn_ballot_w64(pmax >= __float_as_uint(kSplitP)) != 0;
        if (it_ds != nullptr && qb < p.G) {
            // dS tile out for the dQ kernel, in register order: db[kk] of
            // every lane at byte 1024 kk + 16 lane, so each store writes 1 KB
            // of whole cache lines.  Streaming (non-temporal): it is read once.
            u32x4* out = reinterpret_cast<u32x4*>(it_ds + ds_tile(qb >> 5, kw >> 5) * 2048) + lane;
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, db[0]), out);
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, db[1]), out + 64);
            ds_inflight = 2;
        }
        // The residual tiles of a split step wait in LDS (see res_slot), so
        // that no register stays live across the main products for them.
        if (split) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float t1[8], t2[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    t1[i] = sacc[8 * kk + i] - (float)pb[kk][i];
                    t2[i] = pacc[8 * kk + i] - (float)db[kk][i];
                }
                *reinterpret_cast<bf16x8*>(res_slot(0, kk)) = to_bf16x8(t1);
                *reinterpret_cast<bf16x8*>(res_slot(1, kk)) = to_bf16x8(t2);
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS (bf16 P and dS as B operands;
        // with `lo`, their residuals from the stash).
        auto grad_products = [&](bool lo) {
            bf16x8 bp[2], bd[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (lo) {
                    bp[kk] = *reinterpret_cast<const bf16x8*>(res_slot(0, kk));
                    bd[kk] = *reinterpret_cast<const bf16x8*>(res_slot(1, kk));
                } else {
                    bp[kk] = pb[kk];
                    bd[kk] = db[kk];
                }
            }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int col = 32 * cb + 16 * (g16 & 1) + 4 * (jj & 3);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int row = 16 * kk + 4 * hh + (jj >> 2);
                    const bf16x8 go = cat(ld_lds_tr(sO, tile_off<D>(row, col)),
                                          ld_lds_tr(sO, tile_off<D>(row + 8, col)));
                    dv[cb] = mfma32(go, bp[kk], dv[cb]);
                    const bf16x8 qq = cat(ld_lds_tr(sQ, tile_off<D>(row, col)),
                                          ld_lds_tr(sQ, tile_off<D>(row + 8, col)));
                    dk[cb] = mfma32(qq, bd[kk], dk[cb]);
                }
            }
            // Transposed reads 12 ahead, then two per MFMA.
            constexpr int NR = 8 * CB, NM = 4 * CB, AHEAD = 12, PAIRS = (NR - AHEAD) / 2;
            __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
            for (int i = 0; i < PAIRS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NM - PAIRS, 0);
        };
        grad_products(false);
        if (split) grad_products(true);
    }

    // Sum the two query halves (waves 4..7 hand their partials to waves 0..3),
    // dK first, then dV, and write each out.
    f32x4* red = reinterpret_cast<f32x4*>(smem + kg * RED);
    char* stg = smem + 4 * RED + kg * 32 * D * 2;  // bf16 staging of one tensor's rows
    reduce_store<D, GRAD_F32>(p, dk, red, stg, p.scale, p.rope != 0, p.dk, w.b, hk, w.g, s, kw,
                              lane, qh);
    reduce_store<D, GRAD_F32>(p, dv, red, stg, 1.0f, false, p.dv, w.b, hk, w.g, s, kw, lane, qh);
}

// Wait until at most n (wave-uniform) vector memory operations are in flight;
// n above 15 waits down to 15, which is only stricter.
__device__ __forceinline__ void wait_vmem_upto(int n) {
    switch (n) {
#define S2_WAIT_CASE(N) \
    case N: wait_vmem_n<N>(); break;
        S2_WAIT_CASE(0) S2_WAIT_CASE(1) S2_WAIT_CASE(2) S2_WAIT_CASE(3) S2_WAIT_CASE(4)
        S2_WAIT_CASE(5) S2_WAIT_CASE(6) S2_WAIT_CASE(7) S2_WAIT_CASE(8) S2_WAIT_CASE(9)
        S2_WAIT_CASE(10) S2_WAIT_CASE(11) S2_WAIT_CASE(12) S2_WAIT_CASE(13) S2_WAIT_CASE(14)
#undef S2_WAIT_CASE
        default: wait_vmem_n<15>(); break;
    }
}

// ---------------------------------------------------------------------------
// bf16 dQ.  8 waves x 32 queries per workgroup; Q and dO of a wave's queries
// stay in registers.  K and V tiles of 64 keys up to the last query stream
// through two LDS buffers by direct global->LDS loads.
//   S^T = K Q^T, dP^T = V dO^T   (M = key; A from LDS rows, B from registers)
//   dQ^T += K^T dS^T             (A by transposed LDS reads of the K tile)
// ---------------------------------------------------------------------------
constexpr int DQ_WAVES = 8;
constexpr int DQ_BQ = 32 * DQ_WAVES;
constexpr int DQ_BK = 64;

template <int D, bool GRAD_F32>
__global__ __launch_bounds__(64 * DQ_WAVES) void bwd_dq_bf16_kernel(Params p, int n_qt) {
    constexpr int KS = D / 16;
    constexpr int CB = D / 32;
    constexpr int TILE = DQ_BK * D * 2;
    constexpr int NCH = TILE / 1024;
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
    const bf16* __restrict__ dout = static_cast<const bf16*>(p.dout);

    const int q0 = w.tile * DQ_BQ;
    const int qw = q0 + wave * 32;
    const int qi = qw + l32;
    const bool q_valid = qi < p.G;
    const int q_t = orig_row(w.g, p.G, q_valid ? qi : 0, s, p.L);
    const int q_end = min(q0 + DQ_BQ, p.G);
    const int n_kt = (q_end + DQ_BK - 1) / DQ_BK;

    constexpr int NSLOT = 2 * NCH / DQ_WAVES;  // 1 KB chunks per wave per tile; K first, then V
    const uint32_t rowb = (uint32_t)p.Hkv * D * 2;
    const size_t plane = ((size_t)w.b * p.L * p.Hkv + hk) * D;
    ChunkSlot slot[NSLOT];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) slot[j] = chunk_slot<D>((wave + DQ_WAVES * j) % NCH, lane);
    auto stage = [&](int kt, int buf) {
        char* base = smem + buf * 2 * TILE;
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            const bool isv = j >= NSLOT / 2;
            const int cc = (wave + DQ_WAVES * j) % NCH;
            const uint32_t off = row_off(w.g, p.G, kt * DQ_BK + slot[j].row, s, p.L, rowb) + slot[j].colb;
            dma16((isv ? v : k) + plane, off, base + (isv ? TILE : 0) + cc * 1024);
        }
    };
    stage(0, 0);

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
    float lse2 = 0.f, dl = 0.f;  // LSE in base 2, -delta
    if (q_valid) {
        const size_t li = lse_idx(p, w.b, w.h, q_t);
        lse2 = p.lse[li] * kLog2e;
        dl = p.delta[li];
    }
    f32x16 dq[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dq[cb] = f32x16{};

    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * DQ_BK;
        wait_vmem();
        __syncthreads();
        if (kt + 1 < n_kt) stage(kt + 1, (kt + 1) & 1);
        if (k0 > qw + 31) continue;
        const bool diag = (k0 + DQ_BK - 1 > qw);
        const char* sK = smem + (kt & 1) * 2 * TILE;
        const char* sV = sK + TILE;

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
        // K and V operand reads run 6 ahead of their MFMAs (then one per MFMA).
        {
            constexpr int NR = 4 * KS, NM = 4 * KS, AHEAD = 6;
            __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
            for (int i = 0; i < NR - AHEAD; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NM - (NR - AHEAD), 0);
        }
        auto softmax_grad = [&](bool mask) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float pv = __builtin_amdgcn_exp2f(fmaf(sacc[mb][i], p.scale_log2, -lse2));
                    if (mask) {
                        const int key = k0 + 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
                        if (key > qi) pv = 0.f;
                    }
                    pacc[mb][i] = pv * (pacc[mb][i] + dl);  // dl = -delta
                }
        };
        if (diag)
            softmax_grad(true);
        else
            softmax_grad(false);
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
        // Transposed K reads 8 ahead (then two per MFMA).
        {
            constexpr int NR = 8 * CB, NM = 4 * CB, AHEAD = 8, PAIRS = (NR - AHEAD) / 2;
            __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
            for (int i = 0; i < PAIRS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NM - PAIRS, 0);
        }
    }

    grad_rows<D>(p, dq, p.scale, w.g, s, qw, lane, p.rope != 0);
    if (GRAD_F32) {
        store_rows_f32<D>(p, dq, p.dq, w.b, p.Hq, w.h, w.g, s, qw, lane);
        return;
    }
    __syncthreads();  // every wave is done with the K/V buffers
    char* st = smem + wave * 32 * D * 2;
    stage_rows_bf16<D>(dq, st, lane);
    __syncthreads();
    flush_rows<D>(p, st, p.dq, w.b, p.Hq, w.h, w.g, s, qw, lane);
}

// ---------------------------------------------------------------------------
// bf16 dQ from stored dS.  When the dK/dV kernel has written its dS tiles
// (dS^T per 32 keys x 32 queries, see Params::ds), dQ = scale dS K needs no
// recomputation of S and dP: one product instead of three.  8 waves x 32
// queries per workgroup; K tiles of 64 keys and each wave's two dS tiles
// stream through three LDS buffers by direct global->LDS loads, two stages in
// flight while one is consumed.  The kernel is bound by the HBM reads of the
// stored dS (about B Hq L G bytes), not by its MFMA work.
//   dQ^T += K^T dS^T   (A: transposed reads of the K tile; B: transposed
//                        reads of the dS^T tiles, in the same key order)
// ---------------------------------------------------------------------------
constexpr int DQS_WAVES = 8;
constexpr int DQS_BQ = 32 * DQS_WAVES;
// Keys per stage and stages in LDS; DQS_NBUF - 1 stages are in flight while
// one is consumed.
constexpr int DQS_BK = 64;
constexpr int DQS_NBUF = 3;

template <int D, bool GRAD_F32>
__global__ __launch_bounds__(64 * DQS_WAVES) void bwd_dq_ds_kernel(Params p, int n_qt) {
    constexpr int CB = D / 32;
    constexpr int BK = DQS_BK;
    constexpr int NBUF = DQS_NBUF;
    constexpr int KT32 = BK / 32;              // dS tiles per wave per stage
    constexpr int KTILE = BK * D * 2;          // one K tile
    constexpr int KNCH = KTILE / 1024;
    constexpr int DSW = KT32 * 2048;           // a wave's dS tiles of one stage
    constexpr int STAGE = KTILE + DQS_WAVES * DSW;
    static_assert(BK % 32 == 0 && KNCH % DQS_WAVES == 0 && NBUF >= 2, "stage shape");
    static_assert(NBUF * STAGE >= DQS_WAVES * 32 * D * 2, "epilogue staging fits");
    __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];

    const int n_units = p.B * p.Hq * p.n_g;
    const Work w = decode_work(blockIdx.x, n_units, n_qt, p.Hq, p.n_g, p.band);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5;
    const int g16 = lane >> 4, jj = lane & 15;
    const int s = head_shift(p, w.h);
    const int hk = w.h / p.r;
    const bf16* __restrict__ k = static_cast<const bf16*>(p.k);

    const int q0 = w.tile * DQS_BQ;
    const int qw = q0 + wave * 32;
    const int q32 = qw >> 5;
    const bool wave_valid = qw < p.G;   // the wave owns queries of the group
    const int q_end = min(q0 + DQS_BQ, p.G);
    const int n_kt = (q_end + BK - 1) / BK;
    const char* ds_unit = static_cast<const char*>(p.ds) +
                          (((size_t)w.b * p.Hq + w.h) * p.n_g + w.g) * ds_unit_tiles(p.G) * 2048;

    const uint32_t rowb = (uint32_t)p.Hkv * D * 2;
    const size_t plane = ((size_t)w.b * p.L * p.Hkv + hk) * D;
    // Loads this wave issues for stage kt (uniform across the wave).
    auto n_loads = [&](int kt) {
        int n = KNCH / DQS_WAVES;
        if (wave_valid)
#pragma unroll
            for (int sb = 0; sb < KT32; ++sb) n += KT32 * kt + sb <= q32 ? 2 : 0;
        return n;
    };
    // K tile kt and this wave's dS tiles (key tiles KT32 kt + sb when they
    // are at or before its queries) -> buffer `b`.
    auto stage = [&](int kt, int b) {
        char* base = smem + b * STAGE;
#pragma unroll
        for (int j = 0; j < KNCH / DQS_WAVES; ++j) {
            const int cc = wave + DQS_WAVES * j;
            const ChunkSlot sl = chunk_slot<D>(cc, lane);
            const uint32_t off = row_off(w.g, p.G, kt * BK + sl.row, s, p.L, rowb) + sl.colb;
            dma16(k + plane, off, base + cc * 1024);
        }
        if (wave_valid) {
#pragma unroll
            for (int sb = 0; sb < KT32; ++sb) {
                const int k32 = KT32 * kt + sb;
                if (k32 <= q32) {
                    const char* tile = ds_unit + ds_tile(q32, k32) * 2048;
                    char* dst = base + KTILE + wave * DSW + sb * 2048;
                    dma16_nt(tile, 16u * lane, dst);  // read once: streaming
                    dma16_nt(tile + 1024, 16u * lane, dst + 1024);
                }
            }
        }
    };
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j)
        if (j < n_kt) stage(j, j);

    f32x16 dq[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dq[cb] = f32x16{};

    int buf = 0;  // kt % NBUF
    for (int kt = 0; kt < n_kt; ++kt) {
        // Stage kt landed (stages kt + 1 .. kt + NBUF - 2, issued after it,
        // may still be in flight); after the barrier every wave has also
        // finished reading the buffer that stage kt + NBUF - 1 overwrites
        // (consumed at step kt - 1).
        int pending = 0;
#pragma unroll
        for (int j = 1; j < NBUF - 1; ++j) pending += kt + j < n_kt ? n_loads(kt + j) : 0;
        wait_vmem_upto(pending);
        __syncthreads();
        if (kt + NBUF - 1 < n_kt) stage(kt + NBUF - 1, buf == 0 ? NBUF - 1 : buf - 1);
        const char* sK = smem + buf * STAGE;
        buf = buf == NBUF - 1 ? 0 : buf + 1;
        if (!wave_valid || KT32 * kt > q32) continue;
        const int n_kk = 2 * min(KT32, q32 - KT32 * kt + 1);  // 16-key steps with stored dS
        const char* sD = sK + KTILE + wave * DSW;
#pragma unroll
        for (int kk = 0; kk < 2 * KT32; ++kk) {
            if (kk >= n_kk) break;
            // B: dS^T rows (keys) 16kk + 4hh + {0..3, 8..11}, column = this
            // lane's query (see Params::ds for where key r, quad c sits).
            const int drow = 16 * (kk & 1) + 4 * hh + (jj >> 2);
            const int quad = 4 * (g16 & 1) + (jj & 3);
            const int dbyte = (quad >> 2) * 1024 + 512 * (quad & 1) + 8 * ((quad >> 1) & 1);
            const char* dsb = sD + (kk >> 1) * 2048;
            const bf16x8 dsv = cat(ld_lds_tr(dsb, drow * 16 + dbyte),
                                   ld_lds_tr(dsb, (drow + 8) * 16 + dbyte));
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int col = 32 * cb + 16 * (g16 & 1) + 4 * (jj & 3);
                const int row = 16 * kk + 4 * hh + (jj >> 2);
                const bf16x8 kt_ = cat(ld_lds_tr(sK, tile_off<D>(row, col)),
                                       ld_lds_tr(sK, tile_off<D>(row + 8, col)));
                dq[cb] = mfma32(kt_, dsv, dq[cb]);
            }
        }
    }

    grad_rows<D>(p, dq, p.scale, w.g, s, qw, lane, p.rope != 0);
    if (GRAD_F32) {
        store_rows_f32<D>(p, dq, p.dq, w.b, p.Hq, w.h, w.g, s, qw, lane);
        return;
    }
    __syncthreads();  // every wave is done with the buffers
    char* st = smem + wave * 32 * D * 2;
    stage_rows_bf16<D>(dq, st, lane);
    __syncthreads();
    flush_rows<D>(p, st, p.dq, w.b, p.Hq, w.h, w.g, s, qw, lane);
}

// ---------------------------------------------------------------------------
// fp32 backward: plain FMA arithmetic, F32_TPR = D / 32 threads per row, each
// holding 32 of its channels (a whole row per thread would need more
// registers than a wave has at D = 128).  Dot products over the row add the
// threads' partial sums with lane shuffles.
// dQ: threads per query, loop over its keys.  dK/dV: threads per key, loop
// over the query heads sharing the KV head and the queries at or after it.
// ---------------------------------------------------------------------------
constexpr int F32_ROWS = 64;
constexpr int F32_CH = 32;   // channels per thread

template <int TPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, TPR);
    return x;
}

template <int D>
__global__ __launch_bounds__(F32_ROWS * (D / F32_CH)) void bwd_dq_f32_kernel(Params p, int n_qt) {
    constexpr int TPR = D / F32_CH;
    __shared__ float sK[F32_ROWS][D];
    __shared__ float sV[F32_ROWS][D];
    const int n_units = p.B * p.Hq * p.n_g;
    const Work w = decode_work(blockIdx.x, n_units, n_qt, p.Hq, p.n_g, p.band);
    const int tid = threadIdx.x, nthr = F32_ROWS * TPR;
    const int rloc = tid / TPR, c0 = (tid % TPR) * F32_CH;
    const int s = head_shift(p, w.h);
    const int hk = w.h / p.r;
    const float* __restrict__ k = static_cast<const float*>(p.k);
    const float* __restrict__ v = static_cast<const float*>(p.v);
    const int q0 = w.tile * F32_ROWS;
    const int qi = q0 + rloc;
    const bool q_valid = qi < p.G;
    const int q_t = orig_row(w.g, p.G, q_valid ? qi : 0, s, p.L);
    const size_t qo = q_row(p, w.b, q_t, w.h) + c0;
    float qr[F32_CH], gr[F32_CH], acc[F32_CH];
#pragma unroll
    for (int c = 0; c < F32_CH; ++c) {
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
        for (int e = tid; e < F32_ROWS * D; e += nthr) {
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
        // keys k0 .. qi; the TPR threads of a row share the bound
        const int jmax = min(F32_ROWS, qi - k0 + 1);
        for (int j = 0; j < jmax; ++j) {
            float sd = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < F32_CH; ++c) {
                sd = fmaf(qr[c], sK[j][c0 + c], sd);
                dp = fmaf(gr[c], sV[j][c0 + c], dp);
            }
            sd = row_sum<TPR>(sd);
            dp = row_sum<TPR>(dp);
            const float pv = expf(sd * p.scale - lse);
            const float ds = pv * (dp + dl) * p.scale;  // dl = -delta
#pragma unroll
            for (int c = 0; c < F32_CH; ++c) acc[c] = fmaf(ds, sK[j][c0 + c], acc[c]);
        }
    }
    if (q_valid) {
        float* dst = static_cast<float*>(p.dq) + qo;
#pragma unroll
        for (int c = 0; c < F32_CH; ++c) dst[c] = acc[c];
    }
}

template <int D>
__global__ __launch_bounds__(F32_ROWS * (D / F32_CH)) void bwd_dkdv_f32_kernel(Params p, int n_kt) {
    constexpr int TPR = D / F32_CH;
    __shared__ float sQ[F32_ROWS][D];
    __shared__ float sG[F32_ROWS][D];
    __shared__ float sL[F32_ROWS], sD[F32_ROWS];
    const int n_units = p.B * p.Hkv * p.n_g;
    Work w = decode_work(blockIdx.x, n_units, n_kt, p.Hkv, p.n_g, p.band);
    w.tile = n_kt - 1 - w.tile;
    const int hk = w.h;
    const int tid = threadIdx.x, nthr = F32_ROWS * TPR;
    const int rloc = tid / TPR, c0 = (tid % TPR) * F32_CH;
    const int s = head_shift(p, hk * p.r);
    const int k0 = w.tile * F32_ROWS;
    const int kj = k0 + rloc;
    const bool k_valid = kj < p.G;
    const int k_t = orig_row(w.g, p.G, k_valid ? kj : 0, s, p.L);
    const size_t ko = kv_row(p, w.b, k_t, hk) + c0;
    float kr[F32_CH], vr[F32_CH], dk[F32_CH], dv[F32_CH];
#pragma unroll
    for (int c = 0; c < F32_CH; ++c) {
        kr[c] = k_valid ? static_cast<const float*>(p.k)[ko + c] : 0.f;
        vr[c] = k_valid ? static_cast<const float*>(p.v)[ko + c] : 0.f;
        dk[c] = 0.f;
        dv[c] = 0.f;
    }
    for (int hr = 0; hr < p.r; ++hr) {
        const int h = hk * p.r + hr;
        for (int q0 = k0; q0 < p.G; q0 += F32_ROWS) {
            __syncthreads();
            for (int e = tid; e < F32_ROWS * D; e += nthr) {
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
            if (tid < F32_ROWS) {
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
            // causal: queries at or after the key (shared by a row's threads)
            const int i0 = max(0, kj - q0);
            for (int i = i0; i < F32_ROWS; ++i) {
                float sd = 0.f, dp = 0.f;
#pragma unroll
                for (int c = 0; c < F32_CH; ++c) {
                    sd = fmaf(sQ[i][c0 + c], kr[c], sd);
                    dp = fmaf(sG[i][c0 + c], vr[c], dp);
                }
                sd = row_sum<TPR>(sd);
                dp = row_sum<TPR>(dp);
                const float pv = expf(sd * p.scale - sL[i]);
                const float ds = pv * (dp + sD[i]) * p.scale;  // sD = -delta
#pragma unroll
                for (int c = 0; c < F32_CH; ++c) {
                    dv[c] = fmaf(pv, sG[i][c0 + c], dv[c]);
                    dk[c] = fmaf(ds, sQ[i][c0 + c], dk[c]);
                }
            }
        }
    }
    if (k_valid) {
        float* a = static_cast<float*>(p.dk) + ko;
        float* b = static_cast<float*>(p.dv) + ko;
#pragma unroll
        for (int c = 0; c < F32_CH; ++c) {
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
    const long q_rows = q_out ? (long)p.B * p.L * p.Hq : 0, k_rows = (long)p.B * p.L * p.Hkv;
    const long threads = (q_rows + k_rows) * (p.d / 16);  // 8 channel pairs per thread
    const long blocks = (threads + 255) / 256;
    if (p.d == 128)
        hipLaunchKernelGGL(rope_prepass_kernel<128>, dim3(blocks), dim3(256), 0, st, p,
                           static_cast<bf16*>(q_out), static_cast<bf16*>(k_out), q_rows, k_rows);
    else
        hipLaunchKernelGGL(rope_prepass_kernel<64>, dim3(blocks), dim3(256), 0, st, p,
                           static_cast<bf16*>(q_out), static_cast<bf16*>(k_out), q_rows, k_rows);
    return hipGetLastError();
}

template <int D, bool GF, bool SPLIT>
static void launch_dkdv_t(const Params& p0, hipStream_t st) {
    const int n_kt = (p0.G + DKV_BK - 1) / DKV_BK;
    const long blocks = (long)p0.B * p0.Hkv * p0.n_g * n_kt;
    Params p = p0;  // band: Q and dO of the r query heads of the unit
    p.band = dispatch_band(p.B * p.Hkv * p.n_g, (size_t)p.r * p.G * p.d * 4);
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, GF, SPLIT>), dim3(blocks), dim3(64 * DKV_WAVES), 0,
                       st, p, n_kt);
}

template <int D, bool GF>
static void launch_dkdv_split(const Params& p, bool split, hipStream_t st) {
    split ? launch_dkdv_t<D, GF, true>(p, st) : launch_dkdv_t<D, GF, false>(p, st);
}

template <int D, bool GF>
static void launch_dq_t(const Params& p0, hipStream_t st) {
    const int n_qt = (p0.G + DQ_BQ - 1) / DQ_BQ;
    const long blocks = (long)p0.B * p0.Hq * p0.n_g * n_qt;
    Params p = p0;  // band: K and V of the unit
    p.band = dispatch_band(p.B * p.Hq * p.n_g, (size_t)p.G * p.d * 4);
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, GF>), dim3(blocks), dim3(64 * DQ_WAVES), 0, st, p,
                       n_qt);
}

hipError_t launch_bwd_dkdv_bf16(const Params& p, int grad_f32, int split, hipStream_t st) {
    if (p.d == 128)
        grad_f32 ? launch_dkdv_split<128, true>(p, split, st) : launch_dkdv_split<128, false>(p, split, st);
    else
        grad_f32 ? launch_dkdv_split<64, true>(p, split, st) : launch_dkdv_split<64, false>(p, split, st);
    return hipGetLastError();
}

template <int D, bool GF>
static void launch_dq_ds_t(const Params& p0, hipStream_t st) {
    const int n_qt = (p0.G + DQS_BQ - 1) / DQS_BQ;
    const long blocks = (long)p0.B * p0.Hq * p0.n_g * n_qt;
    Params p = p0;  // band: K of the unit (the dS tiles stream through once)
    p.band = dispatch_band(p.B * p.Hq * p.n_g, (size_t)p.G * p.d * 2);
    hipLaunchKernelGGL((bwd_dq_ds_kernel<D, GF>), dim3(blocks), dim3(64 * DQS_WAVES), 0, st, p,
                       n_qt);
}

hipError_t launch_bwd_dq_ds_bf16(const Params& p, int grad_f32, hipStream_t st) {
    if (p.d == 128)
        grad_f32 ? launch_dq_ds_t<128, true>(p, st) : launch_dq_ds_t<128, false>(p, st);
    else
        grad_f32 ? launch_dq_ds_t<64, true>(p, st) : launch_dq_ds_t<64, false>(p, st);
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
        hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, dim3(blocks), dim3(F32_ROWS * 128 / F32_CH), 0,
                           st, p, n_kt);
    else
        hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, dim3(blocks), dim3(F32_ROWS * 64 / F32_CH), 0,
                           st, p, n_kt);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const Params& p, hipStream_t st) {
    const int n_qt = (p.G + F32_ROWS - 1) / F32_ROWS;
    const long blocks = (long)p.B * p.Hq * p.n_g * n_qt;
    if (p.d == 128)
        hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, dim3(blocks), dim3(F32_ROWS * 128 / F32_CH), 0,
                           st, p, n_qt);
    else
        hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, dim3(blocks), dim3(F32_ROWS * 64 / F32_CH), 0,
                           st, p, n_qt);
    return hipGetLastError();
}

}  // namespace s2
