// Block-sparse attention forward over the kept key blocks of each query block,
// with an online softmax (FlashAttention style) [FPSAttention: Training-Aware FP8
// and Sparsity Co-Design for Fast Video Diffusion, Abstract] and the frozen block
// indices of the retained-mass selection [LoSA: Near-Lossless Sparse Attention for
// Training-Free Video Diffusion Acceleration, Abstract].
//
// gfx950 mapping. A workgroup owns one query block (64 rows) of one (batch, head);
// each of its two waves owns 32 query rows and walks the block's CSR list. Scores
// are formed transposed, S^T = K * Q^T, with v_mfma_f32_32x32x16_bf16 (or
// v_mfma_f32_32x32x64_f8f6f4 on e4m3 Q/K): in the 32x32 accumulator a lane holds
// one query column, so the softmax row reductions are in-lane plus one swap of the
// two 32-lane halves, and the output O^T = V^T * P^T keeps one query per lane too,
// making the rescale a per-lane scalar. The accumulator of S already sits in the
// B-operand order of the P*V product once V is stored in the VT layout, so P never
// leaves registers. Q and K come in the QK tiled layout and V in the VT layout,
// both stored in lane order, so every operand load is one contiguous kilobyte per
// wave straight from HBM/L2 into registers; no LDS is used. K of the next kept block is
// loaded while the current block is computed (two register buffers).
// Workgroups are remapped so that each XCD gets a contiguous range of rows (same
// heads), which keeps the shared K/V tiles in that XCD's L2.
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

constexpr float kRescaleSlack = 8.0f;   // log2 units

template <int D, bool FP8>
struct KOperand {
    // per key-tile (2) and d-step: bf16x8 (bf16) or i32x8 (e4m3)
    bf16x8 b[FP8 ? 1 : 2][D / 16];
    i32x8 f[FP8 ? 2 : 1][FP8 ? D / 64 : 1];
};

// Operand loads from the QK / VT tiled layouts: for every (tile, step) the 64 lanes
// read one contiguous kilobyte (bf16) or two (e4m3), lane l at offset 16*l or 32*l.
template <int D, bool FP8>
__device__ inline void load_k(KOperand<D, FP8>& k, const void* kv, long krow0, int lane) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        if constexpr (FP8) {
            const uint8_t* p = static_cast<const uint8_t*>(kv) + krow0 * D + 32 * lane;
#pragma unroll
            for (int st = 0; st < D / 64; ++st)
                k.f[kt][st] = *reinterpret_cast<const i32x8*>(p + (kt * (D / 64) + st) * 2048);
        } else {
            const __bf16* p = static_cast<const __bf16*>(kv) + krow0 * D + 8 * lane;
#pragma unroll
            for (int st = 0; st < D / 16; ++st)
                k.b[kt][st] = *reinterpret_cast<const bf16x8*>(p + (kt * (D / 16) + st) * 512);
        }
    }
}

template <int D>
__device__ inline void load_v(bf16x8 (&v)[D / 32][4], const __bf16* vb, int lane) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
            v[t][cc] = *reinterpret_cast<const bf16x8*>(vb + (t * 4 + cc) * 512 + 8 * lane);
}

template <int D, bool FP8>
struct AttnState {
    f32x16 acc[D / 32];
    float m, l;
};

template <int D, bool FP8>
__device__ inline void attend_block(AttnState<D, FP8>& st, const KOperand<D, FP8>& k,
                                    const bf16x8 (&v)[D / 32][4], const bf16x8* qop,
                                    const i32x8* qop8, float c, uint64_t vmask, int half) {
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kt][i] = 0.0f;
        if constexpr (FP8) {
#pragma unroll
            for (int j = 0; j < D / 64; ++j)
                s[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k.f[kt][j], qop8[j], s[kt], 0, 0, 0, 0, 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < D / 16; ++j)
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.b[kt][j], qop[j], s[kt], 0, 0, 0);
        }
    }
    if (vmask != ~0ull) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int key = 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3);
                if (!((vmask >> key) & 1ull)) s[kt][i] = -INFINITY;
            }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
    const float mloc = wave_max32(mx) * c;          // c > 0
    const bool grow = mloc > st.m + kRescaleSlack;
    if (__ballot(grow)) {
        const float mnew = grow ? mloc : st.m;
        const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);   // 0 when m = -inf
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.acc[t][i] *= alpha;
        st.l *= alpha;
        st.m = mnew;
    }
    const float mref = st.m == -INFINITY ? 0.0f : st.m;
    bf16x8 pb[4];
    float rs = 0.0f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        const int kt = cc >> 1, b0 = 8 * (cc & 1);
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            bf16x2 pr;
            pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][b0 + j], c, -mref));
            pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][b0 + j + 1], c, -mref));
            pb[cc][j] = pr[0];
            pb[cc][j + 1] = pr[1];
            rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
        }
    }
    st.l += wave_add32(rs);
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
            st.acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[t][cc], pb[cc], st.acc[t], 0, 0, 0);
}

template <int D, bool FP8>
__global__ __launch_bounds__(128) void k_sparse_attn(const void* __restrict__ qv,
                                                     const void* __restrict__ kv,
                                                     const __bf16* __restrict__ vt,
                                                     const float* __restrict__ q_scale,
                                                     const float* __restrict__ k_scale,
                                                     const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ col_idx, Geom g,
                                                     long R, float scale_log2, __bf16* __restrict__ o,
                                                     float* __restrict__ lse) {
    const long r = xcd_row(R);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const long bh = r / g.nb;
    const int qb = (int)(r - bh * g.nb);
    const long npad = (long)g.nb * kBlock;
    const long qrow = bh * npad + (long)qb * kBlock + 32 * w + col;   // this lane's query row
    SlotMask sm;
    sm.init(g, lane);

    // Q operand (B of S^T = K * Q^T): lane holds 8 (bf16) or 32 (e4m3) d-values.
    bf16x8 qop[FP8 ? 1 : D / 16];
    i32x8 qop8[FP8 ? D / 64 : 1];
    const long qblk0 = bh * npad + (long)qb * kBlock;                  // first row of the block
    if constexpr (FP8) {
        const uint8_t* q8 = static_cast<const uint8_t*>(qv) + qblk0 * D + 32 * lane;
#pragma unroll
        for (int s = 0; s < D / 64; ++s) qop8[s] = *reinterpret_cast<const i32x8*>(q8 + (w * (D / 64) + s) * 2048);
    } else {
        const __bf16* q = static_cast<const __bf16*>(qv) + qblk0 * D + 8 * lane;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qop[s] = *reinterpret_cast<const bf16x8*>(q + (w * (D / 16) + s) * 512);
    }
    const float cq = FP8 ? scale_log2 * q_scale[r] : scale_log2;

    AttnState<D, FP8> st;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.acc[t][i] = 0.0f;
    st.m = -INFINITY;
    st.l = 0.0f;

    const int e0 = row_ptr[r], e1 = row_ptr[r + 1];
    const __bf16* vbase = vt + bh * (long)g.nb * (kBlock * D);
    const long kbase = bh * npad;
    auto clamp_kb = [&](int e) {
        int kb = col_idx[e];
        return (kb < 0 || kb >= g.nb) ? -1 : kb;
    };

    // K of the next kept block is prefetched one block ahead (two register buffers);
    // V of the current block is issued before its scores are formed, so its latency
    // hides behind the QK^T product and the softmax.
    KOperand<D, FP8> ka, kb2;
    bf16x8 vv[D / 32][4];
    int kbA = e0 < e1 ? clamp_kb(e0) : -1;
    load_k<D, FP8>(ka, kv, kbase + (long)(kbA < 0 ? 0 : kbA) * kBlock, lane);
    for (int e = e0; e < e1; e += 2) {
        int kbB = e + 1 < e1 ? clamp_kb(e + 1) : -1;
        load_v<D>(vv, vbase + (long)(kbA < 0 ? 0 : kbA) * (kBlock * D), lane);
        load_k<D, FP8>(kb2, kv, kbase + (long)(kbB < 0 ? 0 : kbB) * kBlock, lane);
        if (kbA >= 0) {
            const float c = FP8 ? cq * k_scale[bh * g.nb + kbA] : cq;
            attend_block<D, FP8>(st, ka, vv, qop, qop8, c, sm.mask(g, kbA), half);
        }
        if (e + 1 >= e1) break;
        kbA = e + 2 < e1 ? clamp_kb(e + 2) : -1;
        load_v<D>(vv, vbase + (long)(kbB < 0 ? 0 : kbB) * (kBlock * D), lane);
        load_k<D, FP8>(ka, kv, kbase + (long)(kbA < 0 ? 0 : kbA) * kBlock, lane);
        if (kbB >= 0) {
            const float c = FP8 ? cq * k_scale[bh * g.nb + kbB] : cq;
            attend_block<D, FP8>(st, kb2, vv, qop, qop8, c, sm.mask(g, kbB), half);
        }
    }

    const bool qvalid = g.valid(qb, 32 * w + col);
    const float inv = (qvalid && st.l > 0.0f) ? 1.0f / st.l : 0.0f;
    __bf16* orow = o + qrow * D;
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 v4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(st.acc[t][4 * g4 + j] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g4 + 4 * half) = v4;
        }
    if (lse != nullptr && half == 0) {
        float val = 0.0f;
        if (qvalid) val = st.l > 0.0f ? (st.m + __builtin_amdgcn_logf(st.l)) * kLn2 : -INFINITY;
        lse[qrow] = val;
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
    dim3 grid((unsigned)R), block(128);
    if (D == 128) {
        if (fp8) k_sparse_attn<128, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse);
        else k_sparse_attn<128, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse);
    } else {
        if (fp8) k_sparse_attn<64, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse);
        else k_sparse_attn<64, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse);
    }
}

}  // namespace fpsa
