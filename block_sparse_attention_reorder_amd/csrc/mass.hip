// Exact dense block attention mass: the one dense measurement step whose
// per-(head, query block, key block) softmax masses drive the retained-mass
// selection [LoSA: Near-Lossless Sparse Attention for Training-Free Video Diffusion
// Acceleration, Abstract].
//
// mass[qb, kb] = (1 / c(qb)) * sum_{i in qb} sum_{j in kb} exp(s_ij - lse_i), with
// s = scale * q . k over real tokens and lse_i the log-sum-exp of query i over all
// real keys. One sweep over the key blocks computes, for every query i and key
// block kb, the block's own log-sum-exp L_ib = log2 sum_{j in kb} 2^(t_ij) (t the
// score in base 2), kept in a workspace, while an online log-sum-exp per query
// accumulates lse_i. The tile mass is then sum_i 2^(L_ib - lse_i) / c(qb): the same
// quantity as summing every probability, with one exponential per score instead
// of two passes over QK^T.
//
// A workgroup of four waves owns one query block; wave w visits the key blocks
// kb = w (mod 4), each against all 64 queries, so every K byte is loaded by exactly
// one wave. Scores use the transposed MFMA form of the sparse forward (S^T = K * Q^T
// with v_mfma_f32_32x32x16_bf16): a lane holds 32 of a query's 64 block scores, so
// the block max and sum are in-lane plus one swap of the wave halves. After the
// sweep the four online states merge through LDS and each thread turns the
// workspace column of one key block into its mass (a fixed-order sum over the 64
// queries, so results are reproducible).
#include "fpsa_device.h"
#include "fpsa_internal.h"

namespace fpsa {

__device__ inline long xcd_row_mass(long nwg) {
    long i = blockIdx.x;
    long full = nwg - nwg % 8;
    if (i >= full) return i;
    return (i % 8) * (full / 8) + i / 8;
}

constexpr int kMassThreads = 256;

template <int D>
__global__ __launch_bounds__(kMassThreads, 2) void k_block_mass(const __bf16* __restrict__ q,
                                                                const __bf16* __restrict__ k,
                                                                Geom g, long r_begin, long r_count,
                                                                float scale_log2,
                                                                float* __restrict__ mass,
                                                                float* __restrict__ lse,
                                                                float* __restrict__ ws) {
    __shared__ float ml[4][2][64];                 // [wave][m | l][query]
    __shared__ float lse_q[64];
    const long r = r_begin + xcd_row_mass(r_count);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const long bh = r / g.nb;
    const int qb = (int)(r - bh * g.nb);
    const long npad = (long)g.nb * kBlock;
    const long qblk0 = bh * npad + (long)qb * kBlock;
    float* wrow = ws + (r - r_begin) * (long)g.nb * kBlock;   // [nb][64] block lse of each query
    SlotMask sm;
    sm.init(g, lane);

    bf16x8 qop[2][D / 16];
    const __bf16* qp = q + qblk0 * D + 8 * lane;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            qop[qt][st] = *reinterpret_cast<const bf16x8*>(qp + (qt * (D / 16) + st) * 512);

    // K of a block is loaded one visit ahead (register double buffer), so the
    // product of this block never waits on memory.
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
    const __bf16* kbase = k + bh * npad * D + 8 * lane;
    bf16x8 kcur[2][D / 16], knext[2][D / 16];
    auto load_block = [&](bf16x8 (&dst)[2][D / 16], int kb) {
        const __bf16* kp = kbase + (long)(kb < g.nb ? kb : 0) * kBlock * D;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int st = 0; st < D / 16; ++st)
                dst[kt][st] = *reinterpret_cast<const bf16x8*>(kp + (kt * (D / 16) + st) * 512);
    };
    load_block(kcur, w);
    for (int kb = w; kb < g.nb; kb += 4) {
        load_block(knext, kb + 4);
        f32x16 s[2][2];                            // [key tile][query tile]
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kt][qt][i] = 0.0f;
#pragma unroll
                for (int st = 0; st < D / 16; ++st)
                    s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[kt][st], qop[qt][st], s[kt][qt], 0, 0, 0);
            }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int st = 0; st < D / 16; ++st) kcur[kt][st] = knext[kt][st];
        const uint64_t vmask = sm.mask(g, kb);
        if (vmask != ~0ull) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const uint32_t m32 = (uint32_t)(vmask >> (32 * kt + 4 * half));
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float bias = mask_bias(m32, 8 * (i >> 2) + (i & 3));
                    s[kt][0][i] += bias;
                    s[kt][1][i] += bias;
                }
            }
        }
        float lb[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            float mx = s[0][qt][0];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][qt][i]);
            const float mb = wave_max32(mx) * scale_log2;     // block max (base 2); a block always has a real key
            float sum = 0.0f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][qt][i], scale_log2, -mb));
            sum = wave_add32(sum);                            // >= 1: the max term is 2^0
            lb[qt] = mb + __builtin_amdgcn_logf(sum);         // v_log_f32 is log2
            const float mnew = fmaxf(m[qt], mb);
            l[qt] = l[qt] * __builtin_amdgcn_exp2f(m[qt] - mnew) + sum * __builtin_amdgcn_exp2f(mb - mnew);
            m[qt] = mnew;
        }
        // query 32*half + col of this block: lanes of half h store query tile h
        wrow[(long)kb * kBlock + lane] = half ? lb[1] : lb[0];
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
        if (half == qt) {
            ml[w][0][32 * qt + col] = m[qt];
            ml[w][1][32 * qt + col] = l[qt];
        }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int qi = threadIdx.x;
        float mm = ml[0][0][qi];
#pragma unroll
        for (int j = 1; j < 4; ++j) mm = fmaxf(mm, ml[j][0][qi]);
        float ll = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ll += ml[j][1][qi] == 0.0f ? 0.0f : ml[j][1][qi] * __builtin_amdgcn_exp2f(ml[j][0][qi] - mm);
        const bool valid = g.valid(qb, qi);
        const float l2 = mm + __builtin_amdgcn_logf(ll);
        if (lse != nullptr) lse[qblk0 + qi] = valid ? l2 * kLn2 : 0.0f;
        lse_q[qi] = valid ? l2 : INFINITY;          // padding queries contribute 2^-inf = 0
    }
    __syncthreads();
    const float inv = 1.0f / (float)g.count(qb);
    float* out = mass + r * g.nb;
    for (int kb = threadIdx.x; kb < g.nb; kb += kMassThreads) {
        const f32x4* src = reinterpret_cast<const f32x4*>(wrow + (long)kb * kBlock);
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const f32x4 v4 = src[j];
#pragma unroll
            for (int t = 0; t < 4; ++t) acc += __builtin_amdgcn_exp2f(v4[t] - lse_q[4 * j + t]);
        }
        out[kb] = acc * inv;
    }
}

size_t mass_workspace_bytes_per_row(int nb) { return (size_t)nb * kBlock * sizeof(float); }

void launch_block_mass(const void* q, const void* k, int B, int H, int D, const Geom& g,
                       float scale, float* mass, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t st) {
    const long R = (long)B * H * g.nb;
    const float sl2 = scale * kLog2e;
    const __bf16* qb = static_cast<const __bf16*>(q);
    const __bf16* kb = static_cast<const __bf16*>(k);
    const long chunk = (long)(ws_bytes / mass_workspace_bytes_per_row(g.nb));   // >= 1, checked by the caller
    for (long r0 = 0; r0 < R; r0 += chunk) {
        const long n = R - r0 < chunk ? R - r0 : chunk;
        if (D == 128)
            k_block_mass<128><<<(unsigned)n, kMassThreads, 0, st>>>(qb, kb, g, r0, n, sl2, mass, lse, (float*)ws);
        else
            k_block_mass<64><<<(unsigned)n, kMassThreads, 0, st>>>(qb, kb, g, r0, n, sl2, mass, lse, (float*)ws);
    }
}

}  // namespace fpsa
