// Exact dense block attention mass: the one dense measurement step whose
// per-(head, query block, key block) softmax masses drive the retained-mass
// selection [LoSA: Near-Lossless Sparse Attention for Training-Free Video Diffusion
// Acceleration, Abstract].
//
// mass[qb, kb] = (1 / c(qb)) * sum_{i in qb} sum_{j in kb} exp(s_ij - lse_i), with
// s = scale * q . k over real tokens and lse_i the log-sum-exp of query i over all
// real keys. A workgroup owns one query block and sweeps every key block twice:
// pass 1 builds each query's running max and sum (online softmax, base 2), pass 2
// recomputes the scores, exponentiates against the final log-sum-exp and reduces
// each 64x64 tile to one number. Scores use the same transposed MFMA form as the
// sparse forward (S^T = K * Q^T with v_mfma_f32_32x32x16_bf16, one query per lane),
// so the per-query reductions stay in-lane; the per-tile sum is a wave reduction
// whose result is parked in LDS until the row of nb masses is written out.
#include "fpsa_device.h"
#include "fpsa_internal.h"

namespace fpsa {

__device__ inline long xcd_row_mass(long nwg) {
    long i = blockIdx.x;
    long full = nwg - nwg % 8;
    if (i >= full) return i;
    return (i % 8) * (full / 8) + i / 8;
}

// Scores of one key block against this wave's 32 queries; K in the QK tiled layout
// (each wave-wide operand load is one contiguous kilobyte).
template <int D>
__device__ inline void tile_scores(const __bf16* __restrict__ k, long krow0, int lane,
                                   const bf16x8* qop, f32x16* s) {
    const __bf16* kp = k + krow0 * D + 8 * lane;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kt][i] = 0.0f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + (kt * (D / 16) + st) * 512);
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[st], s[kt], 0, 0, 0);
        }
    }
}

// Dynamic LDS: 2 * nb floats (one partial per wave and key block).
template <int D>
__global__ __launch_bounds__(128) void k_block_mass(const __bf16* __restrict__ q,
                                                    const __bf16* __restrict__ k, Geom g, long R,
                                                    float scale_log2, float* __restrict__ mass,
                                                    float* __restrict__ lse) {
    extern __shared__ float part[];
    const long r = xcd_row_mass(R);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const long bh = r / g.nb;
    const int qb = (int)(r - bh * g.nb);
    const long npad = (long)g.nb * kBlock;
    const long qrow = bh * npad + (long)qb * kBlock + 32 * w + col;
    const bool qvalid = g.valid(qb, 32 * w + col);
    SlotMask sm;
    sm.init(g, lane);

    bf16x8 qop[D / 16];
    const __bf16* qp = q + (bh * npad + (long)qb * kBlock) * D + 8 * lane;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qop[s] = *reinterpret_cast<const bf16x8*>(qp + (w * (D / 16) + s) * 512);

    // Pass 1: running max and sum of exp2 over all real keys.
    float m = -INFINITY, l = 0.0f;
    for (int kb = 0; kb < g.nb; ++kb) {
        f32x16 s[2];
        tile_scores<D>(k, bh * npad + (long)kb * kBlock, lane, qop, s);
        const uint64_t vmask = sm.mask(g, kb);
        const bool full = vmask == ~0ull;
        float mloc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float t = s[kt][i] * scale_log2;
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
        float rs = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) rs += __builtin_amdgcn_exp2f(s[kt][i] - mref);
        rs = wave_add32(rs);
        l = l * __builtin_amdgcn_exp2f(m - mref) + rs;
        m = mnew;
    }
    const float lse2 = m + __builtin_amdgcn_logf(l);   // v_log_f32 is log2
    if (lse != nullptr && half == 0) lse[qrow] = qvalid ? lse2 * kLn2 : 0.0f;

    // Pass 2: probabilities against the final lse, summed per 64x64 tile.
    for (int kb = 0; kb < g.nb; ++kb) {
        f32x16 s[2];
        tile_scores<D>(k, bh * npad + (long)kb * kBlock, lane, qop, s);
        const uint64_t vmask = sm.mask(g, kb);
        const bool full = vmask == ~0ull;
        float ps = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = __builtin_amdgcn_exp2f(s[kt][i] * scale_log2 - lse2);
                if (!full) {
                    int key = 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3);
                    if (!((vmask >> key) & 1ull)) p = 0.0f;
                }
                ps += p;
            }
        if (!qvalid) ps = 0.0f;
        ps = wave_sum(ps);
        if (lane == 0) part[w * g.nb + kb] = ps;
    }
    __syncthreads();
    const float inv = 1.0f / (float)g.count(qb);
    float* out = mass + r * g.nb;
    for (int kb = threadIdx.x; kb < g.nb; kb += 128) out[kb] = (part[kb] + part[g.nb + kb]) * inv;
}

void launch_block_mass(const void* q, const void* k, int B, int H, int D, const Geom& g,
                       float scale, float* mass, float* lse, hipStream_t st) {
    const long R = (long)B * H * g.nb;
    const float sl2 = scale * kLog2e;
    const size_t lds = (size_t)2 * g.nb * sizeof(float);
    const __bf16* qb = static_cast<const __bf16*>(q);
    const __bf16* kb = static_cast<const __bf16*>(k);
    if (D == 128) k_block_mass<128><<<(unsigned)R, 128, lds, st>>>(qb, kb, g, R, sl2, mass, lse);
    else k_block_mass<64><<<(unsigned)R, 128, lds, st>>>(qb, kb, g, R, sl2, mass, lse);
}

}  // namespace fpsa
