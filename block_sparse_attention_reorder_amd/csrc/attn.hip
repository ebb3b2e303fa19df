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
// leaves registers, and every operand (Q, K, V^T) is a 16-byte-per-lane load
// straight from HBM/L2 into registers; no LDS is used. Workgroups are remapped so
// that each XCD gets a contiguous range of rows (same heads), which keeps the
// shared K/V tiles in that XCD's L2.
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
    constexpr int kDT = D / 32;                       // 32-wide d tiles of O
    const long r = xcd_row(R);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const long bh = r / g.nb;
    const int qb = (int)(r - bh * g.nb);
    const long npad = (long)g.nb * kBlock;
    const long qrow = bh * npad + (long)qb * kBlock + 32 * w + col;   // this lane's query row

    // Q operand (B of S^T = K * Q^T): lane holds 8 (bf16) or 32 (e4m3) d-values.
    bf16x8 qop[FP8 ? 1 : D / 16];
    i32x8 qop8[FP8 ? D / 64 : 1];
    if constexpr (FP8) {
        const uint8_t* q8 = static_cast<const uint8_t*>(qv) + qrow * D;
#pragma unroll
        for (int s = 0; s < D / 64; ++s) qop8[s] = *reinterpret_cast<const i32x8*>(q8 + 64 * s + 32 * half);
    } else {
        const __bf16* q = static_cast<const __bf16*>(qv) + qrow * D;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qop[s] = *reinterpret_cast<const bf16x8*>(q + 16 * s + 8 * half);
    }
    const float qs = FP8 ? q_scale[r] : 1.0f;

    f32x16 acc[kDT];
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
    float m = -INFINITY, l = 0.0f;

    const int e0 = row_ptr[r], e1 = row_ptr[r + 1];
    for (int e = e0; e < e1; ++e) {
        const int kb = col_idx[e];
        if (kb < 0 || kb >= g.nb) continue;
        const long krow0 = bh * npad + (long)kb * kBlock;

        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.0f;
            if constexpr (FP8) {
                const uint8_t* k8 = static_cast<const uint8_t*>(kv) + (krow0 + 32 * kt + col) * D;
#pragma unroll
                for (int st = 0; st < D / 64; ++st) {
                    i32x8 a = *reinterpret_cast<const i32x8*>(k8 + 64 * st + 32 * half);
                    s[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qop8[st], s[kt], 0, 0,
                                                                           0, 0, 0, 0);
                }
            } else {
                const __bf16* k = static_cast<const __bf16*>(kv) + (krow0 + 32 * kt + col) * D;
#pragma unroll
                for (int st = 0; st < D / 16; ++st) {
                    bf16x8 a = *reinterpret_cast<const bf16x8*>(k + 16 * st + 8 * half);
                    s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[st], s[kt], 0, 0, 0);
                }
            }
        }

        const float c = FP8 ? scale_log2 * qs * k_scale[bh * g.nb + kb] : scale_log2;
        const uint64_t vmask = block_valid_mask(g, kb);
        const bool full = vmask == ~0ull;
        float mloc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float t = s[kt][i] * c;
                if (!full) {
                    int key = 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3);
                    if (!((vmask >> key) & 1ull)) t = -INFINITY;
                }
                s[kt][i] = t;
                mloc = fmaxf(mloc, t);
            }
        mloc = wave_max32(mloc);
        const float mnew = fmaxf(m, mloc);
        const float mref = mnew == -INFINITY ? 0.0f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - mref);
        // Probabilities are rounded to bf16 for the P*V product; the row sum is taken
        // over the same rounded values so that the weights applied to V sum to one.
        bf16x8 pb[4];
        float rs = 0.0f;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int kt = cc >> 1, b0 = 8 * (cc & 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __bf16 pr = (__bf16)__builtin_amdgcn_exp2f(s[kt][b0 + j] - mref);
                pb[cc][j] = pr;
                rs += (float)pr;
            }
        }
        rs = wave_add32(rs);
        l = l * alpha + rs;
        m = mnew;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int t = 0; t < kDT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[t][i] *= alpha;
        }

        const __bf16* vb = vt + (bh * g.nb + kb) * (long)(kBlock * D);
#pragma unroll
        for (int t = 0; t < kDT; ++t)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                bf16x8 a = *reinterpret_cast<const bf16x8*>(vb + (32 * t + col) * kBlock + 16 * cc + 8 * half);
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc], acc[t], 0, 0, 0);
            }
    }

    const bool qvalid = g.valid(qb, 32 * w + col);
    const float inv = (qvalid && l > 0.0f) ? 1.0f / l : 0.0f;
    __bf16* orow = o + qrow * D;
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x2 lo, hi;
            lo[0] = (__bf16)(acc[t][4 * g4 + 0] * inv);
            lo[1] = (__bf16)(acc[t][4 * g4 + 1] * inv);
            hi[0] = (__bf16)(acc[t][4 * g4 + 2] * inv);
            hi[1] = (__bf16)(acc[t][4 * g4 + 3] * inv);
            typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
            bf16x4 v4;
            v4[0] = lo[0]; v4[1] = lo[1]; v4[2] = hi[0]; v4[3] = hi[1];
            *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g4 + 4 * half) = v4;
        }
    if (lse != nullptr && half == 0) {
        float val = 0.0f;
        if (qvalid) val = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
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
