// Device helpers shared by the S2-Attn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "s2_params.h"

namespace s2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Index map.  Head h with shift s reads the sequence rolled left by s: the
// token at rolled position p is original token (p + s) mod L.  In-group index
// i of group g is rolled position g*G + i.  (LongLoRA blog, section 3.3,
// worked shift example: shifted groups start half a group later, wrapping.)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int orig_row(int g, int G, int i, int s, int L) {
    int t = g * G + i + s;
    return t >= L ? t - L : t;
}

// ---------------------------------------------------------------------------
// Row-major bf16 tiles of D = 128 (or 64) columns in LDS, with the 16-byte
// column slots of each row permuted by an XOR of the row.  The LDS serves 64
// four-byte banks per cycle, i.e. 16 slots; the permutation makes both access
// patterns of the kernels hit 16 distinct slots: 16 consecutive rows read at
// one logical slot (MFMA operands from a row-major tile), and 4 consecutive
// rows x 4 slots (transposed reads).  With 8 slots per row (D = 64) it covers
// 8 rows / 4 rows x 2 slots.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) ^ ((row >> 2) & 3);
    return ((row & 3) << 1) | ((row >> 2) & 1);
}

// Byte offset of element (row, col) in a row-major tile with `D` bf16 columns.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
    int slot = (col >> 3) ^ swz<D>(row);
    return row * (D * 2) + slot * 16 + (col & 7) * 2;
}

// 16-byte global load / LDS load.
__device__ __forceinline__ u32x4 ld_global16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ bf16x8 ld_lds16(const char* lds, int off) {
    return *reinterpret_cast<const bf16x8*>(lds + off);
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane
// group, lane j supplies the address of 4 consecutive bf16 (8 bytes);
// result lane i receives, in slot s, element (i % 4) of source lane 4s + i/4.
// With source lane j pointing at row r0 + j/4, columns c0 + 4(j%4) .. +3,
// result lane i gets column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ bf16x4 ld_lds_tr(const char* lds, int off) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<char*>(lds) + off));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 32x32x16 bf16 MFMA.  Lane l holds A[l%32][8(l/32) + 0..7] and
// B[8(l/32) + 0..7][l%32]; C[8j + 4(l/32) + k][l%32] is acc[4j + k].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum with the lane 32 apart (v_permlane32_swap gives both halves' values).
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)x[i];
    return r;
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4 / _dword): lane i
// of the wave deposits its 16 (or 4) bytes at lds_base + 16 i (4 i), so one
// instruction fills 1 KB of LDS with no registers in between.  The LDS base is
// wave-uniform and travels in M0.
//
// They are issued from inline assembly on purpose: the compiler cannot tell
// which of the two tile buffers a DMA targets, and when it sees one in flight
// it waits for it before every transposed LDS read, serialising the prefetch
// of the next tile with the work on the current one.  Here no waits are
// inserted for them; completion is awaited explicitly (wait_vmem) before the
// barrier that hands the buffer to the readers.  Nothing else in these
// kernels uses M0.
// ---------------------------------------------------------------------------
// The LDS address of a generic pointer into LDS is its low 32 bits (the
// shared aperture is 4 GB aligned); truncating directly skips the null check
// an address-space cast carries, which costs two scalar instructions per load.
__device__ __forceinline__ uint32_t lds_addr(const char* lds) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
}
// gsrc = sbase + voff (voff a 32-bit byte offset, sbase wave-uniform).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, char* lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_addr(lds_base)), "v"(voff), "s"(sbase) : "memory");
}
// The same with the non-temporal hint, for data read exactly once.
__device__ __forceinline__ void dma16_nt(const void* sbase, uint32_t voff, char* lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :: "s"(lds_addr(lds_base)), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, char* lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(lds_addr(lds_base)), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt untouched
}

// Wait until at most N vector memory operations of this wave are in flight.
// They complete in issue order, so this awaits all but the last N issued.
// (vmcnt is 6 bits: 3:0 and 15:14 of the immediate.)
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// One 1 KB chunk `cc` of a row-major swizzled tile with D bf16 columns: the
// tile row and the byte offset of the logical 16-byte column slot that lane
// `lane` must fetch so that the DMA lands it at its swizzled place (the XOR
// swizzle is its own inverse).
struct ChunkSlot {
    int row;
    uint32_t colb;
};
template <int D>
__device__ __forceinline__ ChunkSlot chunk_slot(int cc, int lane) {
    constexpr int LPR = D / 8;  // lanes (16-byte slots) per row
    const int r = cc * (64 / LPR) + lane / LPR;
    const int phys = lane % LPR;
    return ChunkSlot{r, (uint32_t)(16 * (phys ^ swz<D>(r)))};
}

// Byte offset, within one (batch, head) plane of a [B, L, H, D] tensor, of
// the row holding in-group index jg (clamped to the group's last row) of
// group g under shift s.  rowbytes = H * D * 2 < 2^24.
__device__ __forceinline__ uint32_t row_off(int g, int G, int jg, int s, int L, uint32_t rowbytes) {
    const int t = orig_row(g, G, min(jg, G - 1), s, L);
    return __umul24((uint32_t)t, rowbytes);
}

// Work decode shared by the tiled kernels: unit (b, h, g) and tile index
// from the flat block id.  Workgroups are dispatched round-robin over the 8
// XCDs; when the unit count is a multiple of 8, every tile of a unit lands
// on the same XCD (so the data its workgroups re-read stays in that XCD's
// L2 or the last-level cache).  Each XCD takes its units in bands of `band`
// units (dispatch_band; the last band may be smaller).  Inside a band the
// tiles go longest first across the band's units, tile-major.  Bands of
// several units keep the longest tiles of an XCD's last units from starting
// last when units have few tiles (small groups) and spread the memory
// stream over more units.  Band 1 is unit by unit, each unit's tiles
// longest first.
struct Work {
    int b, h, g, tile;
};

__device__ __forceinline__ Work decode_work(int bid, int n_units, int n_tiles, int Hh, int n_g,
                                            int band) {
    int u, t;
    if ((n_units & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        const int upx = n_units >> 3;                          // units per XCD
        const int first = slot / (band * n_tiles) * band;      // the band's first unit on the XCD
        const int nb = min(band, upx - first);                 // units in the band
        const int r = slot - first * n_tiles;                  // position inside the band
        t = r / nb;
        u = (first + r % nb) * 8 + xcd;
    } else {
        u = bid / n_tiles;
        t = bid % n_tiles;
    }
    Work w;
    w.g = u % n_g;
    int bh = u / n_g;
    w.h = bh % Hh;
    w.b = bh / Hh;
    w.tile = n_tiles - 1 - t;  // longest first
    return w;
}

// ---------------------------------------------------------------------------
// RoPE with position interpolation (LongLoRA blog, section 3.4): channel pair
// (c, c + d/2) of original position t turns by t * (L0/L) * base^(-2c/d).
// The angle is formed in revolutions in double precision and reduced to
// [-1/2, 1/2] there, so the hardware sine / cosine (which take revolutions)
// see a small argument whatever the position.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_cs(const Params& p, int t, int c, float* cs, float* sn) {
    // t * w less its nearest integer, with the product unrounded (one FMA), so
    // every kernel that calls this forms the same angle.
    const double tt = (double)t, w = p.rope_rev[c];
    const double r = fma(tt, w, -rint(tt * w));
    const float x = (float)r;
    *sn = __builtin_amdgcn_sinf(x);
    *cs = __builtin_amdgcn_cosf(x);
}

// One channel pair of a bf16 row turned by the angle of (t, c), rounded to
// bf16.  The pre-pass and the forward's query fragments both call this, so a
// rotated operand is the same value whichever of them formed it.
struct BfPair {
    bf16 a, b;
};
__device__ __forceinline__ BfPair rope_turn(const Params& p, int t, int c, bf16 a, bf16 b) {
    float cs, sn;
    rope_cs(p, t, c, &cs, &sn);
    const float x1 = (float)a, x2 = (float)b;
    return {(bf16)fmaf(x1, cs, -(x2 * sn)), (bf16)fmaf(x1, sn, x2 * cs)};
}

}  // namespace s2
