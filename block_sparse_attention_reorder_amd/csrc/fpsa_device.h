// Device-side helpers shared by the gfx950 kernels: geometry of the tiled token
// layout, vector types for MFMA operands, and wave-wide reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fpsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kBlock = 64;                       // tokens per tile (block)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Tile geometry of a token grid. Blocks are numbered in raster order over the
// tile grid; slots inside a block follow the raster order of the tile.
struct Geom {
    int T, Hg, Wg;          // token grid
    int tt, th, tw;         // tile shape (product 64)
    int nt, nh, nw;         // tiles per axis
    int nb;                 // blocks

    // Raster token index of (block, slot), or -1 for a padding slot.
    __host__ __device__ inline long token(int blk, int e) const {
        int bt = blk / (nh * nw), r = blk - bt * (nh * nw);
        int bh = r / nw, bw = r - bh * nw;
        int et = e / (th * tw), r2 = e - et * (th * tw);
        int eh = r2 / tw, ew = r2 - eh * tw;
        int t = bt * tt + et, h = bh * th + eh, w = bw * tw + ew;
        if (t >= T || h >= Hg || w >= Wg) return -1;
        return ((long)t * Hg + h) * Wg + w;
    }
    __host__ __device__ inline bool valid(int blk, int e) const { return token(blk, e) >= 0; }
    // Number of real tokens in a block.
    __host__ __device__ inline int count(int blk) const {
        int bt = blk / (nh * nw), r = blk - bt * (nh * nw);
        int bh = r / nw, bw = r - bh * nw;
        int ct = min(tt, T - bt * tt), ch = min(th, Hg - bh * th), cw = min(tw, Wg - bw * tw);
        return ct * ch * cw;
    }
    __host__ __device__ inline bool full(int blk) const { return count(blk) == kBlock; }
};

// 64-bit mask of the real slots of a block (bit e set when slot e holds a token).
// Every lane of the wave must call it; lane e tests slot e.
__device__ inline uint64_t block_valid_mask(const Geom& g, int blk) {
    int lane = threadIdx.x & 63;
    return __ballot(g.valid(blk, lane));
}

// Fast per-block validity for kernels that visit many blocks: the in-tile position
// of this lane's slot is decomposed once, and only blocks on a ragged edge of the
// grid (last tile of an axis the tile does not divide) need a ballot.
struct SlotMask {
    int et, eh, ew;                 // in-tile coordinates of slot (lane)
    bool rt, rh, rw;                // axis is ragged (grid not a multiple of the tile)
    __device__ inline void init(const Geom& g, int lane) {
        int plane = g.th * g.tw;
        et = lane / plane;
        eh = (lane - et * plane) / g.tw;
        ew = lane - et * plane - eh * g.tw;
        rt = g.T % g.tt != 0;
        rh = g.Hg % g.th != 0;
        rw = g.Wg % g.tw != 0;
    }
    // All-ones for an interior block; otherwise the ballot of the real slots.
    __device__ inline uint64_t mask(const Geom& g, int blk) const {
        int plane = g.nh * g.nw;
        int bt = blk / plane, r = blk - bt * plane;
        int bh = r / g.nw, bw = r - bh * g.nw;
        bool edge = (rt && bt == g.nt - 1) || (rh && bh == g.nh - 1) || (rw && bw == g.nw - 1);
        if (!edge) return ~0ull;
        return __ballot(bt * g.tt + et < g.T && bh * g.th + eh < g.Hg && bw * g.tw + ew < g.Wg);
    }
};

// 0.0f when bit `pos` of m is set, -inf otherwise (an additive score mask that
// needs no compare/select).
__device__ inline float mask_bias(uint32_t m, int pos) {
    const uint32_t off = ((m >> pos) & 1u) ^ 1u;        // 1 for a padding key
    return __uint_as_float((0u - off) & 0xFF800000u);
}

// x when bit `pos` of m is set, -inf otherwise: one bitfield extract (0 or all
// ones) and one bitfield insert.
__device__ inline float keep_or_neg_inf(float x, uint32_t m, int pos) {
    const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)m, pos, 1);
    return __uint_as_float((__float_as_uint(x) & sel) | (0xFF800000u & ~sel));
}

// Block validity for kernels that read each kept block's index once per 64 blocks:
// the block's edge code (bit a set when the block is the last, partial tile along
// a ragged axis a = t, h, w) travels with its index, and the real slots of an edge
// block follow from this lane's precomputed in-tile bounds without any division.
struct EdgeSlots {
    int ok;   // bit a: this lane's slot lies inside the partial last tile along axis a
    __device__ inline void init(const Geom& g, int lane) {
        const int plane = g.th * g.tw;
        const int et = lane / plane, eh = (lane - et * plane) / g.tw, ew = lane - et * plane - eh * g.tw;
        ok = (et < g.T - (g.nt - 1) * g.tt ? 1 : 0) | (eh < g.Hg - (g.nh - 1) * g.th ? 2 : 0) |
             (ew < g.Wg - (g.nw - 1) * g.tw ? 4 : 0);
    }
    // Ballot of the real slots of a block with edge code `code` (uniform).
    __device__ inline uint64_t mask(int code) const { return __ballot(((ok | ~code) & 7) == 7); }
};

// Index word of a kept block: the block index in bits 0..23 and its edge code in
// bits 24..26; -1 for an entry outside [0, nb).
constexpr int kEdgeShift = 24;
constexpr int kBlockIdMask = (1 << kEdgeShift) - 1;
__device__ inline int block_info(const Geom& g, int kb) {
    if (kb < 0 || kb >= g.nb) return -1;
    const int plane = g.nh * g.nw;
    const int bt = kb / plane, rr = kb - bt * plane;
    const int bh = rr / g.nw, bw = rr - bh * g.nw;
    const int code = ((bt + 1) * g.tt > g.T ? 1 : 0) | ((bh + 1) * g.th > g.Hg ? 2 : 0) |
                     ((bw + 1) * g.tw > g.Wg ? 4 : 0);
    return kb | (code << kEdgeShift);
}

// Combine lane l with lane l ^ 32 (the two 32-lane halves of the wave) with one
// v_permlane32_swap: with both operands holding x, the two results hold x of this
// lane and of its partner half.
__device__ inline float wave_max32(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float wave_add32(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ inline uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor((unsigned long long)x, o);
    return x;
}

__device__ inline float bf16_to_f32(__bf16 x) { return (float)x; }

// Pack 8 floats into 8 bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ inline bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                     float a6, float a7) {
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

// Which slot of a 16-slot run feeds operand position j of the P*V product: the
// score accumulator of a 32x32 MFMA hands lane half h the rows 4h..4h+3 and
// 8+4h..8+4h+3 of each 16-row run, and operand position 8h + j must hold them.
__host__ __device__ inline int vt_slot_of_position(int pos) {
    int run = pos & ~15, p = pos & 15;
    int h = p >> 3, j = p & 7;
    return run + 4 * h + (j & 3) + 8 * (j >> 2);
}

}  // namespace fpsa
