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
// gfx950 mapping. The pass is dense, so two query blocks (2i, 2i+1 of one head)
// share every key tile: a workgroup of four waves owns both, wave w taking query
// rows 32*(w & 1) .. +31 of block 2i + (w >> 1) against all 64 keys of each key
// block. The K tile of each block is copied once per workgroup into a two-slot LDS
// ring with direct global-to-LDS loads issued from inline asm (so that the compiler
// adds no wait for them before reads of the other slot), and each wave streams the
// operands one step ahead of their products: 126 registers, four workgroups per
// CU. Padding keys of edge blocks get -2^100 from the bias tile that starts each score
// product. Every wave reads the tile in the lane order of the MFMA operand (QK tiled
// layout). Scores use the transposed MFMA form of the sparse
// forward (S^T = K * Q^T, v_mfma_f32_32x32x16_bf16), so a lane holds 32 of its
// query's 64 block scores and the block sums are in-lane plus one swap of the wave
// halves. The products of block j+1 are issued between the exponentials of block j
// (software pipeline, hand-ordered issue).
//
// Exponent reference. Instead of a per-block maximum, each query keeps a lazy
// reference m: the block's terms 2^(t - m) are summed directly, and only when a sum
// exceeds 2^64 (or m is still -inf) is the block redone with m raised to the block
// maximum. Terms far below m underflow to 0; such a block's mass is below 2^-120 of
// the row's. After the sweep the workgroup's threads turn each workspace column
// into a mass with a fixed-order sum over the 64 queries (reproducible results).
#include "attn_common.h"
#include "fpsa_internal.h"

namespace fpsa {

constexpr int kMassThreads = 256;
constexpr float kMassSumLimit = 18446744073709551616.0f;   // 2^64

template <int D>
__global__ __launch_bounds__(kMassThreads, 4) void k_block_mass(const __bf16* __restrict__ q,
                                                                const __bf16* __restrict__ k,
                                                                Geom g, long p_begin, long p_count,
                                                                float scale_log2,
                                                                float* __restrict__ mass,
                                                                float* __restrict__ lse,
                                                                float* __restrict__ ws) {
    constexpr int kKBytes = kBlock * D * 2;                  // K tile of one block
    constexpr int kKChunks = kKBytes / 1024 / 4;             // kilobytes per wave per copy
    static_assert(kKBytes % 4096 == 0, "copies split into whole kilobytes");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kKBytes];
    __shared__ float lse_q[2][64];
    __shared__ __attribute__((aligned(16))) float kbias[8 * 2 * 2 * 16];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qh = w & 1, sel = w >> 1;
    const int col = lane & 31, half = lane >> 5;
    const long p = p_begin + xcd_row(p_count);
    const int ph = (g.nb + 1) >> 1;                          // pairs per (batch, head)
    const long bh = p / ph;
    const int qbA = 2 * (int)(p - bh * ph);
    const int qb = qbA + sel;                                // this wave's query block
    const bool hasrow = qb < g.nb;                           // uniform per wave
    const long npad = (long)g.nb * kBlock;
    const long qblk0 = bh * npad + (long)qb * kBlock;
    // workspace [pair slot][sel][nb][64]: block log-sum-exp of each query
    float* wrow = ws + ((p - p_begin) * 2 + sel) * (long)g.nb * kBlock;
    for (int x = threadIdx.x; x < 8 * 64; x += kMassThreads) {
        const int code = x >> 6, hf = (x >> 5) & 1, kt = (x >> 4) & 1, i = x & 15;
        const int key = 32 * kt + 8 * (i >> 2) + 4 * hf + (i & 3);
        const int plane = g.th * g.tw;
        const int et = key / plane, eh = (key - et * plane) / g.tw, ew = key - et * plane - eh * g.tw;
        const int ok = (et < g.T - (g.nt - 1) * g.tt ? 1 : 0) | (eh < g.Hg - (g.nh - 1) * g.th ? 2 : 0) |
                       (ew < g.Wg - (g.nw - 1) * g.tw ? 4 : 0);
        kbias[x] = ((ok | ~code) & 7) == 7 ? 0.0f : -0x1p100f;
    }
    // (read only after the prologue's barrier)

    KHalf<D, false> qop;
    if (hasrow) {
        load_khalf<D, false>(qop, q, qblk0, qh, lane);
    } else {
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) qop.b[j][e] = (__bf16)0.0f;
    }

    const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(k) + bh * npad * D * 2;
    const int lane16 = 16 * lane;
    // copies from inline asm: the compiler adds no wait for them before the K reads of
    // the other slot that follow them (every read of a slot comes after the vmcnt(0) and
    // barrier that follow the copy into it)
    const i32x4r krs = tile_rsrc_raw(kbytes, (uint32_t)(npad * D * 2));
    auto copy_k = [&](int kb, int slot) {
#pragma unroll
        for (int i = 0; i < kKChunks; ++i)
            copy_kb_asm(krs, (uint32_t)((kb < g.nb ? kb : 0) * kKBytes + (kKChunks * w + i) * 1024),
                        lds + slot * kKBytes + (kKChunks * w + i) * 1024, lane16);
    };

    // Edge code of block kb (bit a: last, partial tile along a ragged axis), kept
    // incrementally as kb walks the blocks in raster order.
    const int rag = (g.T % g.tt ? 1 : 0) | (g.Hg % g.th ? 2 : 0) | (g.Wg % g.tw ? 4 : 0);
    int bt = 0, bhh = 0, bw = 0;
    auto edge_code = [&]() {
        return ((bt == g.nt - 1 ? 1 : 0) | (bhh == g.nh - 1 ? 2 : 0) | (bw == g.nw - 1 ? 4 : 0)) & rag;
    };
    auto next_coords = [&]() {
        if (++bw == g.nw) {
            bw = 0;
            if (++bhh == g.nh) {
                bhh = 0;
                ++bt;
            }
        }
    };

    float m = -INFINITY, l = 0.0f;                           // this lane's query: lazy reference, sum
    KHalf<D, false> k0, k1;                                  // key tiles 0 and 1 of the next block
    f32x16 sa[2], sb[2];                                     // scores [key tile] of two blocks

    // Sum of 2^(t - m) over this wave's 64 keys of a block (both lanes of a query
    // hold it after the half swap).
    auto block_sum = [&](const f32x16 (&s)[2], float nref) {
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            a += __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][i], scale_log2, nref));
            b += __builtin_amdgcn_exp2f(__builtin_fmaf(s[1][i], scale_log2, nref));
        }
        return wave_add32(a + b);
    };
    // Finish block kb: redo the sum with a raised reference when needed, record
    // L = m + log2(sum) and accumulate the row sum. `sum` is the sum formed in the
    // main section; the padding keys of s already hold -2^100.
    auto finish = [&](const f32x16 (&s)[2], int kb, float sum) {
        if (__ballot(!(sum <= kMassSumLimit) || m == -INFINITY)) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
            const float mb = wave_max32(mx) * scale_log2;   // a block always has a real key
            const float mnew = fmaxf(m, mb);
            l *= __builtin_amdgcn_exp2f(m - mnew);          // 0 while m = -inf
            m = mnew;
            sum = block_sum(s, -m);
        }
        l += sum;
        if (hasrow && half == 0) wrow[(long)kb * kBlock + 32 * qh + col] = m + __builtin_amdgcn_logf(sum);
    };

    // Padding keys of an edge block are excluded by the C operand that starts the score
    // products: a tile of 0 (real key) or -2^100 (padding key) from a table per edge code,
    // so a real key's score is bit-identical to the unbiased product and a padding key's
    // term 2^(t - m) underflows to 0. Entry ((code * 2 + half) * 2 + kt) * 16 + i is for
    // key 32 kt + 8 (i / 4) + 4 half + i % 4.
    auto load_block_bias = [&](int code, f32x16 (&sn)[2]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(kbias + ((code * 2 + half) * 2 + kt) * 16 + 4 * j4);
#pragma unroll
                for (int e = 0; e < 4; ++e) sn[kt][4 * j4 + e] = v4[e];
            }
    };

    // Main section of block j (scores s) with the products of block j+1 (into sn, with
    // that block's key bias), in hand-chosen issue order: K(j+1) is read from LDS, K(j+2)
    // copied into the slot K(j) used (after the reads: a read issued after a copy that
    // might write the same bytes has to wait for it), then each product of block j+1 is
    // followed by exponentials of block j. Returns the sum of block j's terms against
    // the current reference.
    auto main_ordered = [&](int j, const f32x16 (&s)[2], f32x16 (&sn)[2], int code_next) {
        const float nref = m == -INFINITY ? 0.0f : -m;
        const uint8_t* kst = lds + ((j + 1) & 1) * kKBytes;
        // the K(j+1) operands stream in one step ahead of their products, which keeps
        // the kernel within 128 registers (four workgroups per CU)
        constexpr int kAheadSt = 1;
        auto kread = [&](int st) {
            k0.b[st] = *reinterpret_cast<const bf16x8*>(kst + st * 1024 + 16 * lane);
            k1.b[st] = *reinterpret_cast<const bf16x8*>(kst + (D / 16 + st) * 1024 + 16 * lane);
        };
#pragma unroll
        for (int st = 0; st < kAheadSt && st < D / 16; ++st) kread(st);
        __builtin_amdgcn_sched_barrier(0);
        copy_k(j + 2, j & 1);
        __builtin_amdgcn_sched_barrier(0);
        load_block_bias(code_next, sn);
        // 2 * D/16 products of block j+1; the 32 exponentials of block j spread over them
        constexpr int kProducts = 2 * (D / 16);
        constexpr int kPerProduct = (32 + kProducts - 1) / kProducts;
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int pi = 0; pi < kProducts; ++pi) {
            const int kt = pi & 1, st = pi >> 1;
            if (kt == 0) sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0.b[st], qop.b[st], sn[0], 0, 0, 0);
            else sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1.b[st], qop.b[st], sn[1], 0, 0, 0);
#pragma unroll
            for (int e = 0; e < kPerProduct; ++e) {
                const int i = pi * kPerProduct + e;
                if (i < 32) {
                    const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i >> 4][i & 15], scale_log2, nref));
                    if (i & 1) acc1 += t;
                    else acc0 += t;
                }
            }
            pin(acc0);
            pin(acc1);
            if (kt == 1 && st + kAheadSt < D / 16) kread(st + kAheadSt);
            __builtin_amdgcn_sched_barrier(0);
        }
        return wave_add32(acc0 + acc1);
    };

    const int nb = g.nb;
    // prologue: K(0), K(1) in flight, K(0) read, products of block 0
    copy_k(0, 0);
    copy_k(1, 1);
    copies_landed_barrier();
    {
        lds_khalf<D, false>(k0, lds, 0, lane);
        lds_khalf<D, false>(k1, lds, 1, lane);
        load_block_bias(edge_code(), sa);
        next_coords();                                       // the coordinates run one block ahead
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            sa[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0.b[st], qop.b[st], sa[0], 0, 0, 0);
            sa[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1.b[st], qop.b[st], sa[1], 0, 0, 0);
        }
    }
    auto step = [&](int j, f32x16 (&s)[2], f32x16 (&sn)[2]) {
        const int code_next = edge_code();                   // of block j+1
        // K(j+1) landed; every wave is done reading K(j) (its slot is refilled below)
        copies_landed_barrier();
        const float sum = main_ordered(j, s, sn, code_next);
        finish(s, j, sum);
        next_coords();
    };
    for (int j = 0; j < nb; j += 2) {
        step(j, sa, sb);
        if (j + 1 < nb) step(j + 1, sb, sa);
    }

    wait_vmcnt<0>();                                         // drain the last (unused) copies

    // Row log-sum-exp (base 2) of each query; padding queries take +inf so that
    // they add 2^-inf = 0 to every mass.
    const int qslot = 32 * qh + col;
    const bool qvalid = hasrow && g.valid(qb, qslot);
    const float l2 = m + __builtin_amdgcn_logf(l);
    if (half == 0) {
        lse_q[sel][qslot] = qvalid ? l2 : INFINITY;
        if (hasrow && lse != nullptr) lse[qblk0 + qslot] = qvalid ? l2 * kLn2 : 0.0f;
    }
    // the workspace rows written above are read back by other threads below
    __syncthreads();
    {
        const int s2 = threadIdx.x >> 7, t = threadIdx.x & 127;   // threads 0-127: block 2i, 128-255: 2i+1
        if (qbA + s2 < nb) {
            const float* wr = ws + ((p - p_begin) * 2 + s2) * (long)nb * kBlock;
            const float inv = 1.0f / (float)g.count(qbA + s2);
            float* out = mass + (bh * nb + qbA + s2) * (long)nb;
            for (int kb = t; kb < nb; kb += 128) {
                const f32x4* src = reinterpret_cast<const f32x4*>(wr + (long)kb * kBlock);
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const f32x4 v4 = src[j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc += __builtin_amdgcn_exp2f(v4[e] - lse_q[s2][4 * j + e]);
                }
                out[kb] = acc * inv;
            }
        }
    }
}

size_t mass_workspace_bytes_per_row(int nb) { return (size_t)nb * kBlock * sizeof(float); }

size_t mass_workspace_bytes_min(int nb) { return 2 * mass_workspace_bytes_per_row(nb); }

size_t mass_workspace_bytes_all(int B, int H, int nb) {
    return mass_workspace_bytes_min(nb) * (size_t)B * H * ((nb + 1) / 2);
}

void launch_block_mass(const void* q, const void* k, int B, int H, int D, const Geom& g,
                       float scale, float* mass, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t st) {
    const long P = (long)B * H * ((g.nb + 1) / 2);              // query-block pairs
    const float sl2 = scale * kLog2e;
    const __bf16* qb = static_cast<const __bf16*>(q);
    const __bf16* kb = static_cast<const __bf16*>(k);
    long chunk = (long)(ws_bytes / mass_workspace_bytes_min(g.nb));   // >= 1, checked by the caller
    if (chunk < P) {
        // a workspace smaller than the whole grid: launch whole waves of workgroups
        // (four per compute unit), so that no launch but the last ends on a partial wave
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
            const long wave = 4L * cus;
            if (chunk >= wave) chunk -= chunk % wave;
        }
    }
    for (long p0 = 0; p0 < P; p0 += chunk) {
        const long n = P - p0 < chunk ? P - p0 : chunk;
        if (D == 128)
            k_block_mass<128><<<(unsigned)n, kMassThreads, 0, st>>>(qb, kb, g, p0, n, sl2, mass, lse, (float*)ws);
        else
            k_block_mass<64><<<(unsigned)n, kMassThreads, 0, st>>>(qb, kb, g, p0, n, sl2, mass, lse, (float*)ws);
    }
}

}  // namespace fpsa
