// Block-sparse attention forward over the kept key blocks of each query block,
// with an online softmax (FlashAttention style) [FPSAttention: Training-Aware FP8
// and Sparsity Co-Design for Fast Video Diffusion, Abstract] and the frozen block
// indices of the retained-mass selection [LoSA: Near-Lossless Sparse Attention for
// Training-Free Video Diffusion Acceleration, Abstract].
//
// gfx950 mapping. A workgroup of four waves owns one query block (64 rows) of one
// (batch, head) and walks the block's CSR list. The K and V tiles of each kept
// block (32 KB in bf16) are copied once per workgroup into LDS with direct
// global-to-LDS loads (global_load_lds_dwordx4, each wave moving a quarter of each
// tile in contiguous kilobytes) into two-slot K and V rings, K two blocks and V one
// block ahead of use, so the copies overlap the computation; one barrier per block. Wave w takes query rows 32*(w & 1) .. +31 and
// key rows 32*(w >> 1) .. +31 of every block, so each wave holds a 32-query x 32-key
// score tile, a 32 x D output accumulator and the matching K and V halves read from
// LDS: small enough for two waves per SIMD, which lets one wave's softmax overlap
// the other's matrix products. The two key halves of a query row carry separate
// online-softmax states that are merged once at the end through LDS.
//
// Scores are formed transposed, S^T = K * Q^T, with v_mfma_f32_32x32x16_bf16 (or
// v_mfma_f32_32x32x64_f8f6f4 on e4m3 Q/K): in the 32x32 accumulator a lane holds
// one query column, so the softmax row reductions are in-lane plus one swap of the
// two 32-lane halves, and the output O^T = V^T * P^T keeps one query per lane too,
// making the rescale a per-lane scalar. The S accumulator already sits in the
// B-operand order of the P*V product, so P never leaves registers. Q and K come in
// the QK tiled layout and V in the VT layout, both stored in lane order, so every
// copy is a contiguous kilobyte and every LDS operand read is a conflict-free
// 16-byte-per-lane ds_read_b128. Workgroups are remapped so that each XCD gets a
// contiguous range of rows (same heads), which keeps the shared K/V tiles in that
// XCD's L2.
//
// Softmax details: scores stay raw until the exponent, exp2(s * c - m) with c the
// scale times log2(e) (times the two FP8 tile scales), so one FMA per element;
// the running reference m only moves when a block's maximum exceeds it by more than
// 8 (a factor 2^8), which keeps every probability <= 256 and makes the rescale of
// the output accumulator rare. The denominator is the sum of the bf16-rounded
// probabilities (v_dot2c_f32_bf16 against ones), the same values fed to P*V.
#include "fpsa_device.h"
#include "fpsa_internal.h"

namespace fpsa {

// blockIdx.x -> row: workgroups are dispatched round-robin over the 8 XCDs, so give
// each XCD a contiguous slice of rows.
__device__ inline long xcd_row(long nwg) {
    long i = blockIdx.x;
    long full = nwg - nwg % 8;
    if (i >= full) return i;
    return (i % 8) * (full / 8) + i / 8;
}

// Direct global-to-LDS copies are counted by vmcnt, and __syncthreads() alone only
// waits for LDS instructions (lgkmcnt), so a barrier that hands copied tiles to the
// other waves must first drain this wave's copies. s_waitcnt immediate on gfx9-family
// targets: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]; this asks
// for vmcnt = 0 and leaves the other counters at their maximum (no wait).
constexpr short kWaitVmcnt0 = 0x0F70;
__device__ inline void copies_landed_barrier() {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
}

constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr int kAttnThreads = 256;

// K operand of one 32-key half: bf16 (D/16 steps of 8 values) or e4m3 (D/64 steps
// of 32 bytes) per lane.
template <int D, bool FP8>
struct KHalf {
    bf16x8 b[FP8 ? 1 : D / 16];
    i32x8 f[FP8 ? D / 64 : 1];
};

// Operand loads from the QK / VT tiled layouts: each (tile, step) is one contiguous
// kilobyte (bf16) or two (e4m3) across the wave, lane l at 16*l or 32*l bytes.
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

// V^T operand for the two 16-key chunks of key half kh: v[t][c] covers channels
// 32t..32t+31 and operand positions 16*(2*kh + c) .. +15 of the block.
template <int D>
__device__ inline void load_vhalf(bf16x8 (&v)[D / 32][2], const __bf16* vb, int kh, int lane) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            v[t][c] = *reinterpret_cast<const bf16x8*>(vb + (t * 4 + 2 * kh + c) * 512 + 8 * lane);
}

// LDS operand reads: the same lane-order kilobytes the global layouts hold.
template <int D, bool FP8>
__device__ inline void lds_khalf(KHalf<D, FP8>& k, const uint8_t* st, int kh, int lane) {
    if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
            k.f[j] = *reinterpret_cast<const i32x8*>(st + (kh * (D / 64) + j) * 2048 + 32 * lane);
    } else {
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
            k.b[j] = *reinterpret_cast<const bf16x8*>(st + (kh * (D / 16) + j) * 1024 + 16 * lane);
    }
}

template <int D>
__device__ inline void lds_vhalf(bf16x8 (&v)[D / 32][2], const uint8_t* st, int kh, int lane) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            v[t][c] = *reinterpret_cast<const bf16x8*>(st + (t * 4 + 2 * kh + c) * 1024 + 16 * lane);
}

template <int D, bool FP8>
__global__ __launch_bounds__(kAttnThreads, 2) void k_sparse_attn(
    const void* __restrict__ qv, const void* __restrict__ kv, const __bf16* __restrict__ vt,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, Geom g, long R,
    float scale_log2, __bf16* __restrict__ o, float* __restrict__ lse) {
    constexpr int kDT = D / 32;
    constexpr int kKBytes = kBlock * D * (FP8 ? 1 : 2);   // K tile of one block
    constexpr int kVBytes = kBlock * D * 2;               // V tile of one block
    constexpr int kKChunks = kKBytes / 1024 / 4;          // kilobytes per wave per copy
    constexpr int kVChunks = kVBytes / 1024 / 4;
    static_assert(kKBytes % 4096 == 0 && kVBytes % 4096 == 0, "copies split into whole kilobytes");
    static_assert(2 * (kDT * 16 + 2) * 64 * 4 <= 2 * (kKBytes + kVBytes), "merge buffer fits");
    // LDS: K ring [K0 | K1] then V ring [V0 | V1]
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (kKBytes + kVBytes)];
    uint8_t* const kring = lds;
    uint8_t* const vring = lds + 2 * kKBytes;

    const long r = xcd_row(R);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int qh = w & 1, kh = w >> 1;
    const int col = lane & 31, half = lane >> 5;
    const long bh = r / g.nb;
    const int qb = (int)(r - bh * g.nb);
    const long npad = (long)g.nb * kBlock;
    const long qblk0 = bh * npad + (long)qb * kBlock;
    SlotMask sm;
    sm.init(g, lane);

    // Q operand (B of S^T = K * Q^T) for query rows 32*qh .. +31.
    KHalf<D, FP8> q;
    load_khalf<D, FP8>(q, qv, qblk0, qh, lane);
    const float cq = FP8 ? scale_log2 * q_scale[r] : scale_log2;

    f32x16 acc[kDT];
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
    float m = -INFINITY, l = 0.0f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    const int e0 = row_ptr[r], e1 = row_ptr[r + 1];
    const uint8_t* kbytes = static_cast<const uint8_t*>(kv) + bh * npad * D * (FP8 ? 1 : 2);
    const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(vt) + bh * (long)g.nb * kVBytes;
    // The CSR list is read 64 entries at a time into one VGPR (lane j holds entry
    // base + j) and single entries are picked with v_readlane, so no iteration
    // waits on a scalar load.
    int batch_base = e0;
    int batch = e0 + lane < e1 ? col_idx[e0 + lane] : -1;
    auto block_at = [&](int e) {
        if (e >= e1) return -1;
        if (e - batch_base >= 64) {
            batch_base += 64;
            batch = batch_base + lane < e1 ? col_idx[batch_base + lane] : -1;
        }
        int kb = __builtin_amdgcn_readlane(batch, e - batch_base);
        return (kb < 0 || kb >= g.nb) ? -1 : kb;
    };
    // Copy the K (or V) tile of block kb into ring slot `slot`: this wave moves
    // its share of contiguous kilobytes, lane l carrying 16 bytes each.
    auto copy_k = [&](int kb, int slot) {
        const uint8_t* src = kbytes + (long)(kb < 0 ? 0 : kb) * kKBytes;
#pragma unroll
        for (int j = 0; j < kKChunks; ++j) {
            const int c = kKChunks * w + j;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(src + c * 1024 + 16 * lane),
                (__attribute__((address_space(3))) void*)(kring + slot * kKBytes + c * 1024), 16, 0, 0);
        }
    };
    auto copy_v = [&](int kb, int slot) {
        const uint8_t* src = vbytes + (long)(kb < 0 ? 0 : kb) * kVBytes;
#pragma unroll
        for (int j = 0; j < kVChunks; ++j) {
            const int c = kVChunks * w + j;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(src + c * 1024 + 16 * lane),
                (__attribute__((address_space(3))) void*)(vring + slot * kVBytes + c * 1024), 16, 0, 0);
        }
    };

    // Software pipeline across kept blocks. Iteration j holds the scores of block j
    // (issued one iteration earlier); after the barrier it reads K of block j+1 and
    // V of block j from LDS, starts the copies of K(j+2) (over K(j)) and V(j+1)
    // (over V(j-1)), both read by every wave before this barrier, issues the QK^T
    // products of block j+1, and only then runs the softmax and P*V of block j, so
    // the matrix pipe works on block j+1 while the vector ALUs work on block j.
    const int n = e1 - e0;
    KHalf<D, FP8> k;
    bf16x8 v[kDT][2];
    f32x16 s, sn;
    int kb = -1, kbn = -1;
    auto scores = [&](f32x16& out) {
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
    };
    if (n > 0) {
        kb = block_at(e0);
        copy_k(kb, 0);
        copy_v(kb, 0);
        if (n > 1) {
            kbn = block_at(e0 + 1);
            copy_k(kbn, 1);
        }
        copies_landed_barrier();                      // K(0), V(0), K(1) landed
        lds_khalf<D, FP8>(k, kring, kh, lane);
        scores(s);
    }
    for (int j = 0; j < n; ++j) {
        const int kb2 = block_at(e0 + j + 2);
        // K(j+1) and V(j) landed; every wave is done with iteration j-1's reads
        copies_landed_barrier();
        lds_vhalf<D>(v, vring + (j & 1) * kVBytes, kh, lane);
        if (j + 1 < n) {
            lds_khalf<D, FP8>(k, kring + ((j + 1) & 1) * kKBytes, kh, lane);
            copy_v(kbn, (j + 1) & 1);
            if (j + 2 < n) copy_k(kb2, j & 1);
            scores(sn);
        }
        {
            // An entry outside [0, nb) is processed as a block with no real key: all
            // its scores are masked, so it adds nothing. Every iteration takes the
            // same path, and the scores are always read an iteration after their
            // products were issued.
            const float c = FP8 ? cq * k_scale[bh * g.nb + (kb < 0 ? 0 : kb)] : cq;
            const uint64_t vmask = kb >= 0 ? sm.mask(g, kb) : 0ull;
            if (vmask != ~0ull) {
                // bit 8*(i/4) + i%4 of m32 tells whether element i's key is real
                const uint32_t m32 = (uint32_t)(vmask >> (32 * kh + 4 * half));
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] += mask_bias(m32, 8 * (i >> 2) + (i & 3));
            }
            float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            float mx2 = fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]));
            float mx3 = fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11]));
            float mx4 = fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]));
            mx = fmaxf(fmaxf(mx, mx2), fmaxf(mx3, mx4));
            const float mloc = wave_max32(mx) * c;          // c > 0
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
            const float mref = m == -INFINITY ? 0.0f : m;
            bf16x8 pb[2];
            float rs0 = 0.0f, rs1 = 0.0f;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    bf16x2 pr;
                    pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * cc + jj], c, -mref));
                    pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * cc + jj + 1], c, -mref));
                    pb[cc][jj] = pr[0];
                    pb[cc][jj + 1] = pr[1];
                    if (cc == 0) rs0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs0, false);
                    else rs1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs1, false);
                }
            l += wave_add32(rs0 + rs1);
#pragma unroll
            for (int t = 0; t < kDT; ++t)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[t][cc], pb[cc], acc[t], 0, 0, 0);
        }
        s = sn;
        kb = kbn;
        kbn = kb2;
    }

    // Merge the two key halves of each query row: wave (qh, 1) hands its state to
    // wave (qh, 0) through the (now idle) stage memory; wave (qh, 0) rescales both
    // to the larger reference and finishes.
    __syncthreads();
    float* xch = reinterpret_cast<float*>(lds) + qh * (kDT * 16 + 2) * 64;
    if (kh == 1) {
#pragma unroll
        for (int t = 0; t < kDT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) xch[(t * 16 + i) * 64 + lane] = acc[t][i];
        xch[(kDT * 16) * 64 + lane] = m;
        xch[(kDT * 16 + 1) * 64 + lane] = l;
    }
    __syncthreads();
    if (kh == 1) return;
    {
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
    }

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
    if (lse != nullptr && half == 0) {
        float val = 0.0f;
        if (qvalid) val = l > 0.0f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
        lse[qblk0 + qslot] = val;
    }
}

void launch_sparse_attn(const void* q, const void* k, const void* v, int fp8, const float* q_scale,
                        const float* k_scale, const int32_t* row_ptr, const int32_t* col_idx,
                        int B, int H, int D, const Geom& g, float scale, void* o, float* lse,
                        hipStream_t st) {
    const long R = (long)B * H * g.nb;
    const float sl2 = scale * kLog2e;
    const __bf16* vt = static_cast<const __bf16*>(v);
    __bf16* out = static_cast<__bf16*>(o);
    dim3 grid((unsigned)R), block(kAttnThreads);
    if (D == 128) {
        if (fp8) k_sparse_attn<128, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse);
        else k_sparse_attn<128, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse);
    } else {
        if (fp8) k_sparse_attn<64, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse);
        else k_sparse_attn<64, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse);
    }
}

}  // namespace fpsa
