// Pieces shared by the block-sparse forward kernels (one query block per workgroup,
// and two query blocks sharing each K/V tile): operand layouts, the per-block
// online-softmax step and the hand-ordered main section of one kept block, and the
// final merge of the two key halves.
//
// Conventions (gfx950, v_mfma_f32_32x32x16_bf16 / v_mfma_scale_f32_32x32x64_f8f6f4):
// a wave owns 32 queries (qh) x 32 keys (kh) of each 64 x 64 block pair. Scores are
// formed transposed, S^T = K * Q^T, so lane (col, half) holds query col and keys
// 8*(i/4) + 4*half + i%4 of the wave's key half in accumulator element i; the output
// O^T = V^T * P^T keeps one query per lane as well. The S accumulator is already the
// B operand of the P*V product (with V stored in the VT layout), so P stays in
// registers. Online softmax in base 2: p = 2^(s*c - m) with c the softmax scale
// times log2(e); the reference m only moves when a block maximum exceeds it by more
// than 8, and the denominator is the sum of the bf16-rounded probabilities that
// multiply V.
#pragma once

#include "fpsa_device.h"

namespace fpsa {

// blockIdx.x -> work item: workgroups are dispatched round-robin over the 8 XCDs, so
// give each XCD a contiguous slice of items (neighbouring query blocks of one head,
// which share K/V tiles in that XCD's L2).
__device__ inline long xcd_row(long nwg) {
    long i = blockIdx.x;
    long full = nwg - nwg % 8;
    if (i >= full) return i;
    return (i % 8) * (full / 8) + i / 8;
}

// blockIdx.x -> work item for grids whose concurrent workgroups should all serve one
// (batch, head): each XCD still takes 64 consecutive items (what its 32 CUs run at
// once at two workgroups per CU), but the eight XCDs take the eight consecutive
// chunks of 64 in turn, so the whole chip works through the items in order and one
// head's K and V, rather than eight heads', compete for the 256 MB infinity cache.
// A bijection on [0, nwg); the last nwg % 512 items keep their own index.
__device__ inline long xcd_chunk_row(long nwg) {
    const long i = blockIdx.x;
    const long full = nwg - nwg % 512;
    if (i >= full) return i;
    const long x = i % 8, s = i / 8;
    return (s / 64) * 512 + x * 64 + (s % 64);
}

// Order of the query blocks of a 2D (image) grid: vertical strips of kStripW block
// columns, row-major inside a strip, so the ~64 workgroups an XCD runs at a time cover
// an 8 x 8 patch of blocks. Under a criss-cross mask (a group keeps its whole block row
// and column) a patch shares each row block among 8 workgroups and each column block
// among 8, where a row-major order shares row blocks among 64 and column blocks among
// none. A bijection on each (batch, head)'s rows; identity for 3D grids and for grids
// at most kStripW blocks wide.
constexpr int kStripW = 8;
__device__ inline bool strip_grid(const Geom& g) { return g.nt == 1 && g.nw > kStripW; }
__device__ inline long strip_row(long r, const Geom& g) {
    if (!strip_grid(g)) return r;
    const long bh = r / g.nb;
    const int i = (int)(r - bh * g.nb);
    const int ns = (g.nw + kStripW - 1) / kStripW, full = (ns - 1) * g.nh * kStripW;
    int rb, cb;
    if (i < full) {
        const int st = i / (g.nh * kStripW), rem = i - st * g.nh * kStripW;
        rb = rem / kStripW;
        cb = kStripW * st + rem % kStripW;
    } else {
        const int wl = g.nw - kStripW * (ns - 1), rem = i - full;
        rb = rem / wl;
        cb = kStripW * (ns - 1) + rem % wl;
    }
    return bh * g.nb + (long)rb * g.nw + cb;
}

// Direct global-to-LDS copies are counted by vmcnt, and __syncthreads() alone only
// waits for LDS instructions (lgkmcnt), so a barrier that hands copied tiles to the
// other waves must first wait for this wave's copies. s_waitcnt immediate on
// gfx9-family targets: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt
// [11:8]; the other counters are left at their maximum (no wait).
template <int N>
__device__ __attribute__((always_inline)) inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((short)((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14)));
}
__device__ inline void copies_landed_barrier() {
    wait_vmcnt<0>();
    __syncthreads();
}

constexpr float kRescaleSlack = 8.0f;   // log2 units

// Keep a value's computation at this point of the program: an empty volatile asm
// that reads and rewrites the register, so IR passes cannot sink the arithmetic that
// produces it past this point (sched_barrier only constrains the machine scheduler).
__device__ __attribute__((always_inline)) inline void pin(float& x) { asm volatile("" : "+v"(x)); }

// Direct global-to-LDS copies go through a buffer resource (base and size in SGPRs,
// the raw buffer format of gfx9-family targets in dword 3) rather than global_load_lds:
// the compiler counts the global form against lgkmcnt as well, so every LDS read issued
// before such a copy would wait for all of them at its first use, while the buffer form
// leaves one wait per read. Offsets are 32-bit: a resource spans one (batch, head)'s
// tiles, which callers keep below 2^31 bytes.
__device__ __attribute__((always_inline)) inline __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)bytes, 0x00020000);
}
// Copy one kilobyte at byte `off` (wave-uniform) of buffer `rs` to LDS `dst`, lane l
// carrying bytes 16*l .. 16*l+15 (buffer_load_dwordx4 ... lds: the LDS address comes
// from M0, set from the uniform `dst`). Completion is counted by vmcnt.
__device__ __attribute__((always_inline)) inline void copy_kb_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                                                      uint8_t* dst, int lane16) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, lane16,
                                             (int)__builtin_amdgcn_readfirstlane(off), 0, 0);
}
template <int KB>
__device__ __attribute__((always_inline)) inline void copy_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                                                   uint8_t* dst, int lane16) {
#pragma unroll
    for (int j = 0; j < KB; ++j) copy_kb_to_lds(rs, off + j * 1024, dst + j * 1024, lane16);
}

// Direct global-to-LDS copy of one kilobyte (buffer_load_dwordx4 ... lds: lane l carries
// the 16 bytes at its own source offset `lane16` past `off` to M0 + 16*l) issued from
// inline asm, for loops that keep a copy in flight while they read other LDS slots: the
// compiler does not see it and so adds no waits of its own before LDS reads; the caller
// orders every read of a slot after the copy into it has landed (vmcnt, then a barrier),
// every copy into a slot after the last read of it (a barrier), and drains the copies
// before the kernel ends. The asm has no register outputs besides the M0 save, and
// restores M0.
typedef int i32x4r __attribute__((ext_vector_type(4)));
__device__ __attribute__((always_inline)) inline i32x4r tile_rsrc_raw(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4r r;
    r[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}
__device__ __attribute__((always_inline)) inline void copy_kb_asm(i32x4r rs, uint32_t off, uint8_t* dst,
                                                                   int lane16) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)dst);
    const uint32_t so = __builtin_amdgcn_readfirstlane(off);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(la), "v"(lane16), "s"(rs), "s"(so)
                 : "memory");
}

// K operand of one 32-key half: bf16 (D/16 steps of 8 values) or e4m3 (D/64 steps
// of 32 bytes) per lane.
template <int D, bool FP8>
struct KHalf {
    bf16x8 b[FP8 ? 1 : D / 16];
    i32x8 f[FP8 ? D / 64 : 1];
};

// Operand loads from the QK tiled layout in global memory: each (tile, step) is one
// contiguous kilobyte (bf16) or two (e4m3) across the wave, lane l at 16*l or 32*l.
template <int D, bool FP8>
__device__ inline void load_khalf(KHalf<D, FP8>& k, const void* base, long row0, int kt, int lane) {
    if constexpr (FP8) {
        const uint8_t* p = static_cast<const uint8_t*>(base) + row0 * D + 32 * lane;
#pragma unroll
        for (int st = 0; st < D / 64; ++st)
            k.f[st] = *reinterpret_cast<const i32x8*>(p + (kt * (D / 64) + st) * 2048);
    } else {
        const __bf16* p = static_cast<const __bf16*>(base) + row0 * D + 8 * lane;
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            k.b[st] = *reinterpret_cast<const bf16x8*>(p + (kt * (D / 16) + st) * 512);
    }
}

// LDS operand reads: bf16, the same lane-order kilobytes the global layout holds; e4m3,
// each 2 KB step split by halves (the first 16 bytes of every lane's 32, in lane order,
// then the second 16), so that both reads run over a contiguous kilobyte instead of
// striding 32 bytes (which used half of the banks).
template <int D, bool FP8>
__device__ inline void lds_khalf(KHalf<D, FP8>& k, const uint8_t* st, int kh, int lane) {
    if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
            const uint8_t* p = st + (kh * (D / 64) + j) * 2048 + 16 * lane;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 1024);
            k.f[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    } else {
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
            k.b[j] = *reinterpret_cast<const bf16x8*>(st + (kh * (D / 16) + j) * 1024 + 16 * lane);
    }
}

// V^T operand of key half kh: v[t][c] covers channels 32t..32t+31 and operand
// positions 16*(2*kh + c) .. +15 of the block.
template <int D>
__device__ inline void lds_vhalf(bf16x8 (&v)[D / 32][2], const uint8_t* st, int kh, int lane) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            v[t][c] = *reinterpret_cast<const bf16x8*>(st + (t * 4 + 2 * kh + c) * 1024 + 16 * lane);
}

// S^T tile of this wave's 32 keys x 32 queries.
template <int D, bool FP8>
__device__ __attribute__((always_inline)) inline void qk_scores(f32x16& out, const KHalf<D, FP8>& k,
                                                                const KHalf<D, FP8>& q) {
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = 0.0f;
    if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
            out = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k.f[j], q.f[j], out, 0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < D / 16; ++j) out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.b[j], q.b[j], out, 0, 0, 0);
    }
}

// Maximum over the wave's 32 keys of each query (unmasked).
__device__ inline float max16(const f32x16& x) {
    const float a = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    const float b = fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]));
    const float d = fmaxf(fmaxf(x[8], x[9]), fmaxf(x[10], x[11]));
    const float e = fmaxf(fmaxf(x[12], x[13]), fmaxf(x[14], x[15]));
    return wave_max32(fmaxf(fmaxf(a, b), fmaxf(d, e)));
}

// First part of a kept block's step: mask the padding keys (or every key, for a
// block this wave's query block does not keep), take the block maximum and rescale
// the running state when the maximum moved by more than the slack. `vm` is the
// 64-bit mask of the block's keys to keep (uniform), `all_keys` tells that every key
// is kept and `smax` already holds the unmasked maximum. Returns -m (0 before any
// key), the offset of the exponent.
template <int kDT>
__device__ __attribute__((always_inline)) inline float softmax_enter(
    f32x16& s, bool all_keys, uint64_t vm, float smax, float c, int kh, int half,
    f32x16 (&acc)[kDT], float& m, float& l) {
    float mx = smax;
    if (!all_keys) {
        // bit 8*(i/4) + i%4 of m32 tells whether element i's key is kept
        const uint32_t m32 = (uint32_t)(vm >> (32 * kh + 4 * half));
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = keep_or_neg_inf(s[i], m32, 8 * (i >> 2) + (i & 3));
        mx = max16(s);
    }
    const float mloc = mx * c;                    // c > 0
    const bool grow = mloc > m + kRescaleSlack;
    if (__ballot(grow)) {
        const float mnew = grow ? mloc : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // 0 when m = -inf
#pragma unroll
        for (int t = 0; t < kDT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][i] *= alpha;
        l *= alpha;
        m = mnew;
    }
    return m == -INFINITY ? 0.0f : -m;
}

// The same for scores that arrive in base-2 units already shifted by the reference r
// (r = m, or 0 before any key; the tile mt holds -r and starts the score products):
// smax and s are relative to r, and moving the reference shifts s and mt with it.
template <int kDT>
__device__ __attribute__((always_inline)) inline void softmax_enter_shifted(
    f32x16& s, bool all_keys, uint64_t vm, float smax, int kh, int half, f32x16 (&acc)[kDT], f32x16& mt,
    float& m, float& l) {
    float mx = smax;
    if (!all_keys) {
        const uint32_t m32 = (uint32_t)(vm >> (32 * kh + 4 * half));
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = keep_or_neg_inf(s[i], m32, 8 * (i >> 2) + (i & 3));
        mx = max16(s);
    }
    const bool grow = mx > (m == -INFINITY ? -INFINITY : kRescaleSlack);
    if (__ballot(grow)) {
        const float r = m == -INFINITY ? 0.0f : m;
        const float mnew = r + mx;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;   // 0 when m = -inf
        const float d = grow ? mx : 0.0f;
#pragma unroll
        for (int t = 0; t < kDT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][i] *= alpha;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] -= d;
        if (grow) m = mnew;
        const float nr = m == -INFINITY ? 0.0f : -m;
#pragma unroll
        for (int i = 0; i < 16; ++i) mt[i] = nr;
    }
}

// Main section of a kept block in its plain form (any D, bf16 or e4m3 scores):
// read K of the next block and V of this one from LDS, then start the copies (after
// the reads, for the reason given below), issue the next block's QK^T, then this
// block's exponentials and P*V.
template <int D, bool FP8, int NC, class Copy>
__device__ __attribute__((always_inline)) inline void block_main_generic(
    const uint8_t* kst, const uint8_t* vst, int kh, int lane, const KHalf<D, FP8>& q, KHalf<D, FP8>& k,
    bf16x8 (&v)[D / 32][2], f32x16 (&acc)[D / 32], const f32x16& s, f32x16& sn, float c, float nref,
    float& l, float& smax, Copy&& copy_one) {
    constexpr int kDT = D / 32;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    lds_khalf<D, FP8>(k, kst, kh, lane);
    lds_vhalf<D>(v, vst, kh, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NC; ++i) copy_one(i);
    __builtin_amdgcn_sched_barrier(0);
    qk_scores<D, FP8>(sn, k, q);
    bf16x8 pb[2];
    float rs0 = 0.0f, rs1 = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
            bf16x2 pr;
            pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * cc + jj], c, nref));
            pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * cc + jj + 1], c, nref));
            pb[cc][jj] = pr[0];
            pb[cc][jj + 1] = pr[1];
            if (cc == 0) rs0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs0, false);
            else rs1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs1, false);
        }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int t = 0; t < kDT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[t][cc], pb[cc], acc[t], 0, 0, 0);
    l += rs0 + rs1;
    smax = max16(sn);
}

// Main section of a kept block for bf16, D = 128, in hand-chosen issue order
// (sched_barrier fences keep the scheduler from regrouping it): each of the 16
// matrix products is followed by one exponential and a few other vector
// instructions. All LDS operand reads are issued before the copies into LDS (a read
// issued after a copy that might write the same LDS bytes would have to wait for the
// copy to land), and the copies (NC single-kilobyte instructions, `copy_one(i)`) go
// one after each QK^T product, so that their issue overlaps the matrix core instead
// of stalling the wave. The QK^T chain of the next block comes first, then P*V of
// this block,
// whose first half needs the first eight probabilities and whose second half the
// rest; the next block's score maximum is taken under the last products. SHIFT: the
// queries carry the base-2 scale and the score chain starts from mt (-r), so the scores
// need no scale-and-shift step before their exponentials.
template <int NC, bool SHIFT, class Copy>
__device__ __attribute__((always_inline)) inline void block_main_bf16_d128(
    const uint8_t* kst, const uint8_t* vst, int kh, int lane, const KHalf<128, false>& q,
    KHalf<128, false>& k, bf16x8 (&v)[4][2], f32x16 (&acc)[4], const f32x16& s, f32x16& sn, const f32x16& mt,
    float c, float nref, float& l, float& smax, Copy&& copy_one) {
    static_assert(NC <= 8, "one copy per QK^T product");
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float pf[16];
    uint32_t pw[8];
    float rs0 = 0.0f, rs1 = 0.0f;
    float ma, mb, md, me;
    auto FM = [&](int i) { pf[i] = SHIFT ? s[i] : __builtin_fmaf(s[i], c, nref); };
    auto EX = [&](int i) { pf[i] = __builtin_amdgcn_exp2f(pf[i]); };
    auto CV = [&](int i) {
        bf16x2 pr;
        pr[0] = (__bf16)pf[i];
        pr[1] = (__bf16)pf[i + 1];
        pw[i >> 1] = __builtin_bit_cast(uint32_t, pr);
    };
    auto DT = [&](int wi) {
        const bf16x2 pr = __builtin_bit_cast(bf16x2, pw[wi]);
        if (wi < 4) rs0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs0, false);
        else rs1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs1, false);
    };
    auto QK = [&](int i) {
        if (i == 0 && !SHIFT) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sn[e] = 0.0f;
        }
        sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.b[i], q.b[i], (SHIFT && i == 0) ? mt : sn, 0, 0, 0);
    };
    auto PV = [&](int t, int cc) {
        const i32x4 wv = {(int)pw[4 * cc], (int)pw[4 * cc + 1], (int)pw[4 * cc + 2], (int)pw[4 * cc + 3]};
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[t][cc], __builtin_bit_cast(bf16x8, wv), acc[t], 0, 0, 0);
    };
    auto VREAD = [&](int t) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
            v[t][cc] = *reinterpret_cast<const bf16x8*>(vst + (t * 4 + 2 * kh + cc) * 1024 + 16 * lane);
    };
#define FPSA_SB __builtin_amdgcn_sched_barrier(0)
    auto CP = [&](int i) {
        if (i < NC) copy_one(i);
    };
    lds_khalf<128, false>(k, kst, kh, lane);
    VREAD(0); VREAD(1); VREAD(2); VREAD(3);
    FM(0); FM(1); FM(2); FM(3); EX(0); EX(1);
    FPSA_SB;
    QK(0); CP(0); EX(2); FM(4);
    FPSA_SB;
    QK(1); CP(1); EX(3); FM(5);
    FPSA_SB;
    QK(2); CP(2); EX(4); FM(6); CV(0);
    FPSA_SB;
    QK(3); CP(3); EX(5); FM(7); CV(2);
    FPSA_SB;
    QK(4); CP(4); EX(6); FM(8); DT(0); CV(4);
    FPSA_SB;
    QK(5); CP(5); EX(7); FM(9); DT(1);
    FPSA_SB;
    QK(6); CP(6); EX(8); FM(10); CV(6); DT(2);
    FPSA_SB;
    QK(7); CP(7); EX(9); FM(11); DT(3);
    FPSA_SB;
    PV(0, 0); EX(10); FM(12); CV(8);
    FPSA_SB;
    PV(1, 0); EX(11); FM(13); DT(4);
    FPSA_SB;
    PV(2, 0); EX(12); FM(14); CV(10);
    FPSA_SB;
    PV(3, 0); EX(13); FM(15); DT(5);
    FPSA_SB;
    EX(14); EX(15); CV(12); CV(14);
    FPSA_SB;
    PV(0, 1); DT(6); DT(7);
    ma = fmaxf(fmaxf(sn[0], sn[1]), fmaxf(sn[2], sn[3]));
    FPSA_SB;
    PV(1, 1); mb = fmaxf(fmaxf(sn[4], sn[5]), fmaxf(sn[6], sn[7]));
    md = fmaxf(fmaxf(sn[8], sn[9]), fmaxf(sn[10], sn[11]));
    FPSA_SB;
    PV(2, 1); me = fmaxf(fmaxf(sn[12], sn[13]), fmaxf(sn[14], sn[15]));
    l += rs0 + rs1;
    FPSA_SB;
    PV(3, 1); smax = wave_max32(fmaxf(fmaxf(ma, mb), fmaxf(md, me)));
    FPSA_SB;
#undef FPSA_SB
}


// Main section of a kept block for e4m3 Q/K, D = 128, in hand-chosen issue order:
// the two fp8 QK^T products of the next block (64-key steps) and the eight bf16 P*V
// products of this one, each followed by exponentials and other vector work, with
// the copies (NC kilobytes) after the QK^T and first P*V products.
template <int NC, class Copy>
__device__ __attribute__((always_inline)) inline void block_main_fp8_d128(
    const uint8_t* kst, const uint8_t* vst, int kh, int lane, const KHalf<128, true>& q,
    KHalf<128, true>& k, bf16x8 (&v)[4][2], f32x16 (&acc)[4], const f32x16& s, f32x16& sn, float c,
    float nref, float& l, float& smax, Copy&& copy_one) {
    static_assert(NC <= 8, "copies fit the issue slots");
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float pf[16];
    uint32_t pw[8];
    float rs0 = 0.0f, rs1 = 0.0f;
    float ma, mb, md, me;
    auto FM = [&](int i) { pf[i] = __builtin_fmaf(s[i], c, nref); };
    auto EX = [&](int i) { pf[i] = __builtin_amdgcn_exp2f(pf[i]); };
    auto CV = [&](int i) {
        bf16x2 pr;
        pr[0] = (__bf16)pf[i];
        pr[1] = (__bf16)pf[i + 1];
        pw[i >> 1] = __builtin_bit_cast(uint32_t, pr);
    };
    auto DT = [&](int wi) {
        const bf16x2 pr = __builtin_bit_cast(bf16x2, pw[wi]);
        if (wi < 4) rs0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs0, false);
        else rs1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs1, false);
    };
    auto QK = [&](int i) {
        if (i == 0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sn[e] = 0.0f;
        }
        sn = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k.f[i], q.f[i], sn, 0, 0, 0, 0, 0, 0);
    };
    auto PV = [&](int t, int cc) {
        const i32x4 wv = {(int)pw[4 * cc], (int)pw[4 * cc + 1], (int)pw[4 * cc + 2], (int)pw[4 * cc + 3]};
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[t][cc], __builtin_bit_cast(bf16x8, wv), acc[t], 0, 0, 0);
    };
    auto CP = [&](int i) {
        if (i < NC) copy_one(i);
    };
#define FPSA_SB __builtin_amdgcn_sched_barrier(0)
    auto VR = [&](int t, int cc) {     // V operand, read a few products before its use
        v[t][cc] = *reinterpret_cast<const bf16x8*>(vst + (t * 4 + 2 * kh + cc) * 1024 + 16 * lane);
    };
    lds_khalf<128, true>(k, kst, kh, lane);
    VR(0, 0); VR(1, 0); VR(2, 0); VR(3, 0);
    FM(0); FM(1); FM(2); FM(3); EX(0); EX(1);
    FPSA_SB;
    QK(0); CP(0); CP(1); EX(2); FM(4); EX(3); FM(5); CV(0); FM(6);
    FPSA_SB;
    QK(1); CP(2); CP(3); EX(4); FM(7); EX(5); FM(8); CV(2); FM(9); EX(6); EX(7); CV(4); CV(6);
    FPSA_SB;
    PV(0, 0); VR(0, 1); CP(4); EX(8); FM(10); DT(0); DT(1);
    FPSA_SB;
    PV(1, 0); VR(1, 1); CP(5); EX(9); FM(11); DT(2); CV(8);
    FPSA_SB;
    PV(2, 0); VR(2, 1); CP(6); EX(10); FM(12); EX(11); FM(13); DT(3);
    FPSA_SB;
    PV(3, 0); VR(3, 1); CP(7); EX(12); FM(14); EX(13); FM(15); CV(10); DT(4);
    FPSA_SB;
    EX(14); EX(15); CV(12); CV(14); DT(5);
    FPSA_SB;
    PV(0, 1); DT(6); DT(7);
    ma = fmaxf(fmaxf(sn[0], sn[1]), fmaxf(sn[2], sn[3]));
    FPSA_SB;
    PV(1, 1); mb = fmaxf(fmaxf(sn[4], sn[5]), fmaxf(sn[6], sn[7]));
    md = fmaxf(fmaxf(sn[8], sn[9]), fmaxf(sn[10], sn[11]));
    FPSA_SB;
    PV(2, 1); me = fmaxf(fmaxf(sn[12], sn[13]), fmaxf(sn[14], sn[15]));
    l += rs0 + rs1;
    FPSA_SB;
    PV(3, 1); smax = wave_max32(fmaxf(fmaxf(ma, mb), fmaxf(md, me)));
    FPSA_SB;
#undef FPSA_SB
}

// Merge the two key halves of each query row and store: wave (qh, 1) hands its
// state to wave (qh, 0) through `xch` (LDS the caller no longer uses, 2 x (kDT*16+2)
// x 64 floats); wave (qh, 0) rescales both to the larger reference, normalises and
// writes its 32 query rows of O (bf16) and lse. The caller has synchronised the
// workgroup before; this function synchronises once more (all waves must call it).
template <int D>
__device__ __attribute__((always_inline)) inline void merge_and_store(
    float* xch_base, int qh, int kh, int lane, f32x16 (&acc)[D / 32], float m, float l, bool store,
    const Geom& g, int qb, long qblk0, __bf16* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ o32) {
    constexpr int kDT = D / 32;
    float* xch = xch_base + qh * (kDT * 16 + 2) * 64;
    if (kh == 1) {
#pragma unroll
        for (int t = 0; t < kDT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) xch[(t * 16 + i) * 64 + lane] = acc[t][i];
        xch[(kDT * 16) * 64 + lane] = m;
        xch[(kDT * 16 + 1) * 64 + lane] = l;
    }
    __syncthreads();
    if (kh == 1 || !store) return;
    const float m1 = xch[(kDT * 16) * 64 + lane], l1 = xch[(kDT * 16 + 1) * 64 + lane];
    const float mm = fmaxf(m, m1);
    const float mref = mm == -INFINITY ? 0.0f : mm;
    const float a0 = __builtin_amdgcn_exp2f(m - mref), a1 = __builtin_amdgcn_exp2f(m1 - mref);
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = acc[t][i] * a0 + xch[(t * 16 + i) * 64 + lane] * a1;
    l = l * a0 + l1 * a1;
    m = mm;

    const int col = lane & 31, half = lane >> 5;
    const int qslot = 32 * qh + col;
    const bool qvalid = g.valid(qb, qslot);
    const float inv = (qvalid && l > 0.0f) ? 1.0f / l : 0.0f;
    __bf16* orow = o + (qblk0 + qslot) * D;
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 v4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(acc[t][4 * g4 + j] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g4 + 4 * half) = v4;
        }
    if (o32 != nullptr) {
        float* frow = o32 + (qblk0 + qslot) * D;
#pragma unroll
        for (int t = 0; t < kDT; ++t)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 v4;
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] = acc[t][4 * g4 + j] * inv;
                *reinterpret_cast<f32x4*>(frow + 32 * t + 8 * g4 + 4 * half) = v4;
            }
    }
    if (lse != nullptr && half == 0) {
        float val = 0.0f;
        if (qvalid) val = l > 0.0f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
        lse[qblk0 + qslot] = val;
    }
}

}  // namespace fpsa
