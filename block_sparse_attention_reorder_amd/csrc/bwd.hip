// Block-sparse attention backward over a frozen block CSR (bf16 operands, float32
// accumulation): the gradients of the FlashAttention-style forward, which is what
// training through the same 64-token tiles needs [FPSAttention: Training-Aware FP8
// and Sparsity Co-Design for Fast Video Diffusion, Abstract].
//
// With s = scale q.k, p = exp(s - lse) (lse from the forward), dp = dO.v and
// delta = dO.O per query:
//   dV_j = sum_i p_ij dO_i,  dS_ij = p_ij (dp_ij - delta_i),
//   dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j.
// Three kernels, no atomics (deterministic):
//   k_bwd_prep  per query slot: delta = dO.O (O in bf16 or, more accurately, the
//               forward's float32 copy) and lse in base 2 (+inf for padding or
//               a query without keys, so its probabilities are exactly 0);
//   k_bwd_dkdv  one workgroup per key block, walking the query blocks that keep it
//               (the transposed CSR); dK and dV stay in registers, each wave holding
//               half the channels of its 32 keys (P and dS are exchanged through LDS);
//   k_bwd_dq    one workgroup per query block, walking its kept key blocks; for
//               D = 128 on video grids (k_bwd_dq_pair) one workgroup per two
//               neighbouring query blocks, walking the union of their rows.
// Both copy each block's tiles (Q and dO, or K and V) straight into one of two LDS
// slots an iteration ahead, with copies issued from inline asm that the compiler does
// not wait for; without register staging both fit 256 registers, so two workgroups
// share a CU.
// Every operand comes from the QK tiled layout. Products whose reduction runs over
// tokens (P^T dO, dS^T Q, dS K) need the tile transposed - channel per lane, tokens
// along the operand - which the gfx950 transposing LDS read (ds_read_b64_tr_b16)
// delivers from the same LDS copy: within each 16-lane group, output lane i element
// j is element i%4 of input lane 4j + i/4. Each wave owns a 32 x 32 (query, key)
// sub-tile of every block pair; the two partial sums of each output half are added
// through LDS at the end (dQ) or exchanged before the products (dK, dV).
#include <type_traits>

#include "attn_common.h"
#include "fpsa_internal.h"

namespace fpsa {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Byte offset of element (token e, channel d) inside a bf16 QK tile (include/fpsa.h).
template <int D>
__device__ inline int qk_off(int e, int d) {
    return 2 * (((((e >> 5) * (D / 16) + (d >> 4)) * 2 + ((d >> 3) & 1)) * 32 + (e & 31)) * 8 + (d & 7));
}

// LDS copies of the QK tiles are swizzled: within each kilobyte (two 512-byte groups of
// 32 tokens x 8 channels), the odd group has its 8-token runs of 128 bytes swapped in
// pairs (16-byte unit e of an odd group sits at unit e ^ 8). A copy lane l therefore
// fetches source unit l ^ 8*(l >> 5) of its kilobyte, and a plain operand read by lane l
// of unit l of a kilobyte reads position l ^ 8*(l >> 5) (swz_unit). The transposing reads
// below touch four groups at once; without the swap the even and odd groups share their
// banks (two-way conflicts), with it they fall on different halves of the banks.
__device__ inline int swz_unit(int l) { return l ^ ((l >> 5) << 3); }

// Offset of this lane's 8-byte source for a transposing read of the swizzled QK tile
// that gives each lane of a 16-lane group g one channel (16*(g%2) + lane%16 of a
// 32-channel tile) and four consecutive tokens, starting at token t0 + 4*(g/2): input
// lane a supplies token t0 + 4*(g/2) + a/4, channels 4*(a%4) .. +3 (t0 a multiple of
// 32). Tokens t0 + 8 .. follow at offset ^ 128 bytes, the next 16 tokens at +256, the
// next 32-channel tile at +2048. Channels 8 .. 15 of a 16 (a%4 >= 2) sit in the odd
// group, whose 8-token halves are swapped: +128 for those lanes.
template <int D>
__device__ inline int tr_base(int t0, int lane) {
    const int g = lane >> 4, a = lane & 15;
    return qk_off<D>(t0 + 4 * (g >> 1) + (a >> 2), 16 * (g & 1) + 4 * (a & 3)) + 128 * ((a >> 1) & 1);
}

// Operand of 8 tokens in position order (t0..t0+3, then t0+8..t0+11 of the lane's
// half) for one channel per lane.
__device__ inline bf16x8 tr_operand(const uint8_t* tile, int off) {
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off));
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + (off ^ 128)));
    const s16x8 z = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, z);
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = B .. E-1.
template <int B, int E, class F>
__device__ __attribute__((always_inline)) inline void bwd_static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        bwd_static_for<B + 1, E>(f);
    }
}

// The value lane I of this lane's 16-lane row holds (DPP row broadcast).
template <int I>
__device__ inline float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + I, 0xF, 0xF, true));
}

// Fragments loaded once and reused for every block: an empty asm that rewrites each
// register keeps the compiler from re-issuing the global loads inside the loop.
template <int D>
__device__ __attribute__((always_inline)) inline void keep_resident(KHalf<D, false>& x) {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        i32x4 r = __builtin_bit_cast(i32x4, x.b[st]);
        asm volatile("" : "+v"(r));
        x.b[st] = __builtin_bit_cast(bf16x8, r);
    }
}

// ---------------------------------------------------------------- preprocessing

template <int D, class OT>
__global__ __launch_bounds__(256) void k_bwd_prep(const OT* __restrict__ o,
                                                  const __bf16* __restrict__ dout,
                                                  const float* __restrict__ lse, Geom g,
                                                  float* __restrict__ lse2, float* __restrict__ delta) {
    const long blk = blockIdx.x;                   // (b*H + h)*nb + qb
    const int qb = (int)(blk % g.nb);
    const int e = threadIdx.x >> 2, part = threadIdx.x & 3;
    const OT* ot = o + blk * 64 * D;
    const uint8_t* gt = reinterpret_cast<const uint8_t*>(dout + blk * 64 * D);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        const int d0 = 8 * (part + 4 * j);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(gt + qk_off<D>(e, d0));
#pragma unroll
        for (int t = 0; t < 8; ++t) acc += (float)ot[e * D + d0 + t] * (float)b[t];
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (part == 0) {
        const long i = blk * 64 + e;
        const float L = lse[i];
        const bool live = g.valid(qb, e) && L > -INFINITY;
        lse2[i] = live ? L * kLog2e : INFINITY;
        delta[i] = live ? acc : 0.0f;
    }
}

// ---------------------------------------------------------------- dK, dV

// Two phases per query block. Phase 1, wave (kh, r): the S and dP products of its 32
// keys against query half r, then P and dS for those 32 x 32 pairs, packed as the A
// operands of the token-reduction products and written to an exchange buffer in LDS.
// Phase 2, wave (kh, r): dV and dK of its 32 keys for channel half r, over all 64
// queries, from the four P and dS operands of its key half. Each wave's accumulators
// thus cover half the channels (64 registers instead of 128), which with the direct
// copies into two slots keeps the kernel at two workgroups per CU.
// SCALED: e4m3 Q/K (tile scales multiply the scores and dS); without it the scales
// are 1 and their multiplications are left out.
template <int D, bool SCALED>
__global__ __launch_bounds__(256, 2) void k_bwd_dkdv(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale, Geom g, float c,
    float scale, __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
    constexpr int kTile = 64 * D * 2;
    constexpr int kSlot = 2 * kTile;              // Q tile, dO tile
    constexpr int kDT = D / 32;
    constexpr int kHT = kDT / 2;                  // 32-channel tiles per channel half
    static_assert(kHT >= 1, "two channel halves");
    // two slots, then the exchange buffer [kh][r][ks][P, dS] of 1 KB operands
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kSlot + 16 * 1024];
    uint8_t* const xbuf = lds + 2 * kSlot;

    const int tid = threadIdx.x, lane = tid & 63, hb = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = w & 1, r = w >> 1;             // phase 1: query half r; phase 2: channel half r
    const long col = xcd_row(gridDim.x);
    const long bh = col / g.nb;
    const int kb = (int)(col - bh * g.nb);
    const long npad = 64L * g.nb;

    KHalf<D, false> kf, vf;                        // B operands: key (lane % 32) of half kh
    load_khalf<D, false>(kf, k, col * 64, kh, lane);
    load_khalf<D, false>(vf, v, col * 64, kh, lane);
    keep_resident<D>(kf);
    keep_resident<D>(vf);
    const bool kvalid = g.valid(kb, 32 * kh + (lane & 31));
    // e4m3 Q/K: q and k hold code values, the tile scales multiply the scores and, for
    // dK = dS^T Q-hat, each query block's dS
    const float sk = k_scale != nullptr ? k_scale[col] : 1.0f;

    f32x16 accv[kHT], acck[kHT];
#pragma unroll
    for (int t = 0; t < kHT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) accv[t][i] = acck[t][i] = 0.0f;

    const int e0 = col_ptr[col], n = col_ptr[col + 1] - e0;
    // query block of entry jj (-1: none or out of range)
    auto qb_at = [&](int jj) {
        if (jj >= n) return -1;
        const int x = __builtin_amdgcn_readfirstlane(row_idx[e0 + jj]);
        return (x >= 0 && x < g.nb) ? x : -1;
    };
    // Q and dO tiles of a query block copied straight into a slot, this wave moving a
    // quarter of each in whole kilobytes (a missing block copies block 0)
    constexpr int kCh = kTile / 1024 / 4;
    const int lane16 = 16 * swz_unit(lane);       // swizzled source unit of this lane
    const i32x4r qrs = tile_rsrc_raw(q + bh * npad * D, (uint32_t)(npad * D * 2));
    const i32x4r grs = tile_rsrc_raw(dout + bh * npad * D, (uint32_t)(npad * D * 2));
    auto copy_block = [&](int qbk, uint8_t* dst) {
        const uint32_t base = (uint32_t)((qbk < 0 ? 0 : qbk) * kTile);
#pragma unroll
        for (int ch = 0; ch < kCh; ++ch) {
            copy_kb_asm(qrs, base + (kCh * w + ch) * 1024, dst + (kCh * w + ch) * 1024, lane16);
            copy_kb_asm(grs, base + (kCh * w + ch) * 1024, dst + kTile + (kCh * w + ch) * 1024, lane16);
        }
    };
    // exchange operand (key half kh, query half qq, step ks, kind 0 = P / 1 = dS)
    auto xop = [&](int qq, int ks, int kind) -> uint8_t* {
        return xbuf + (((kh * 2 + qq) * 2 + ks) * 2 + kind) * 1024 + 16 * lane;
    };

    // lse2 and delta of the 32 queries of this wave's phase-1 half, one per lane: lane
    // 16 g + n (g the 16-lane row) holds query 32*r + 8*(n/4) + 4*(g/2) + n%4, which is
    // exactly the query of phase-1 element i = n for the lanes of row g, so element i
    // takes it from lane i of its own row (a DPP row broadcast). Loaded one block ahead:
    // issued right after the barrier, before the copies, and first used an iteration
    // later, after the next vmcnt(0), so no wait of the compiler's ever covers a copy in
    // flight. (e4m3: also the query tile's scale, as a vector load: its index is moved
    // into a vector register, since a scalar load shares the LDS reads' wait counter and
    // returns out of order, which would turn every operand wait into a full drain.)
    float LG[2][2];                                // [set][L or G]
    float TQ[2];                                   // [set]
    auto load_lg = [&](int qbk, float (&X)[2], float& T) {
        const long qrow = (bh * g.nb + (qbk < 0 ? 0 : qbk)) * 64 + 32 * r + 8 * ((lane & 15) >> 2) + 4 * hb + (lane & 3);
        X[0] = lse2[qrow];
        X[1] = delta[qrow];
        T = 1.0f;
        if (q_scale != nullptr) {
            long idx = bh * g.nb + (qbk < 0 ? 0 : qbk);
            asm volatile("" : "+v"(idx));
            T = q_scale[idx];
        }
    };

    auto phase1 = [&](const uint8_t* sq, const float (&X)[2], float tq) {
        const uint8_t* sg = sq + kTile;
        const float cs = c * tq * sk;
        bf16x8 qa[D / 16], ga[D / 16];
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const int off = (r * (D / 16) + st) * 1024 + 16 * swz_unit(lane);
            qa[st] = *reinterpret_cast<const bf16x8*>(sq + off);
            ga[st] = *reinterpret_cast<const bf16x8*>(sg + off);
        }
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.0f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[st], kf.b[st], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[st], vf.b[st], dp, 0, 0, 0);
        }
        // element i: query 32*r + 8*(i/4) + 4*hb + i%4, key 32*kh + lane%32
        float pv[16], ds[16];
        bwd_static_for<0, 16>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const float lq = row_bcast<i>(X[0]);
            const float gq = row_bcast<i>(X[1]);
            const float pp = kvalid ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cs, -lq)) : 0.0f;
            pv[i] = pp;
            ds[i] = SCALED ? pp * (dp[i] - gq) * tq : pp * (dp[i] - gq);
        });
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int b = 8 * ks;
            *reinterpret_cast<bf16x8*>(xop(r, ks, 0)) =
                pack_bf16x8(pv[b], pv[b + 1], pv[b + 2], pv[b + 3], pv[b + 4], pv[b + 5], pv[b + 6], pv[b + 7]);
            *reinterpret_cast<bf16x8*>(xop(r, ks, 1)) =
                pack_bf16x8(ds[b], ds[b + 1], ds[b + 2], ds[b + 3], ds[b + 4], ds[b + 5], ds[b + 6], ds[b + 7]);
        }
    };
    auto phase2 = [&](const uint8_t* sq) {
        const uint8_t* sg = sq + kTile;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int trb = tr_base<D>(32 * qq, lane);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 pa = *reinterpret_cast<const bf16x8*>(xop(qq, ks, 0));
                const bf16x8 da = *reinterpret_cast<const bf16x8*>(xop(qq, ks, 1));
#pragma unroll
                for (int t = 0; t < kHT; ++t) {
                    const int off = trb + (kHT * r + t) * 2048 + ks * 256;
                    accv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, tr_operand(sg, off), accv[t], 0, 0, 0);
                    acck[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, tr_operand(sq, off), acck[t], 0, 0, 0);
                }
            }
        }
    };

    // Two slots: block j sits in slot j % 2; iteration j waits for its copy (issued an
    // iteration earlier) and for every wave to leave iteration j - 1, starts the copy of
    // block j + 1 into the other slot, then runs both phases with a barrier between them
    // (the exchange buffer is rewritten only after the next iteration's barrier).
    // iteration jj uses register set P = jj % 2 and slot jj % 2 (the loop is unrolled by
    // two so both stay compile-time: a register copy would make the compiler wait for
    // the loads, and with them for the copies in flight)
    auto iter = [&](auto set, int jj, int qcur, int qnext) {
        constexpr int P = decltype(set)::value;
        wait_vmcnt<0>();
        __syncthreads();
        load_lg(qnext, LG[1 - P], TQ[1 - P]);         // unconditional (block 0 past the end)
        if (jj + 1 < n) copy_block(qnext, lds + (1 - P) * kSlot);
        if (qcur >= 0) {                               // uniform
            phase1(lds + P * kSlot, LG[P], TQ[P]);
            __syncthreads();
            phase2(lds + P * kSlot);
        }
    };
    if (n > 0) {
        int qcur = qb_at(0);
        load_lg(qcur, LG[0], TQ[0]);
        copy_block(qcur, lds);
        for (int jj = 0; jj < n; jj += 2) {
            const int q1 = qb_at(jj + 1);
            iter(std::integral_constant<int, 0>(), jj, qcur, q1);
            if (jj + 1 < n) {
                const int q2 = qb_at(jj + 2);
                iter(std::integral_constant<int, 1>(), jj + 1, q1, q2);
                qcur = q2;
            }
        }
    }
    wait_vmcnt<0>();

    // element i of tile t: key 32*kh + 8*(i/4) + 4*hb + i%4, channel 32*(kHT*r + t) + lane%32
    const long row0 = bh * npad + 64L * kb + 32 * kh;
#pragma unroll
    for (int t = 0; t < kHT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const long rr = row0 + 8 * (i >> 2) + 4 * hb + (i & 3);
            const int ch = 32 * (kHT * r + t) + (lane & 31);
            dv[rr * D + ch] = (__bf16)accv[t][i];
            dk[rr * D + ch] = (__bf16)(scale * acck[t][i]);
        }
}

// ---------------------------------------------------------------- dQ

template <int D, bool SCALED>
__global__ __launch_bounds__(256, 2) void k_bwd_dq(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale, Geom g, float c,
    float scale, __bf16* __restrict__ dq) {
    constexpr int kTile = 64 * D * 2;
    constexpr int kSlot = 2 * kTile;              // K tile, V tile
    constexpr int kDT = D / 32;
    static_assert(kDT * 16 * 64 * 4 <= kSlot, "reduction buffer fits a slot");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kSlot];   // two slots
    // bias tiles: entry ((code * 2 + kh) * 2 + hb) * 16 + i is 0 when key 32 kh + 8 (i / 4)
    // + 4 hb + i % 4 of a block with edge code `code` is real, else -inf; used as the
    // C operand that starts the score products, so padding keys get p = 0 without any
    // per-score masking
    __shared__ __attribute__((aligned(16))) float sbias[8 * 2 * 2 * 16];

    const int tid = threadIdx.x, lane = tid & 63, hb = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qh = w & 1, kh = w >> 1;
    const long row = xcd_row(gridDim.x);
    const long bh = row / g.nb;
    const long npad = 64L * g.nb;

    KHalf<D, false> qf, gf;                        // B operands: query (lane % 32) of half qh
    load_khalf<D, false>(qf, q, row * 64, qh, lane);
    load_khalf<D, false>(gf, dout, row * 64, qh, lane);
    keep_resident<D>(qf);
    keep_resident<D>(gf);
    const float lq = lse2[row * 64 + 32 * qh + (lane & 31)];
    const float gq = delta[row * 64 + 32 * qh + (lane & 31)];
    // e4m3 Q/K: code values in q and k; the tile scales multiply the scores and, for
    // dQ = dS K-hat, each key block's dS
    const float tq = q_scale != nullptr ? q_scale[row] : 1.0f;
    const int trb = tr_base<D>(32 * kh, lane);
    for (int x = tid; x < 8 * 64; x += 256) {
        const int code = x >> 6, kx = (x >> 5) & 1, hx = (x >> 4) & 1, i = x & 15;
        const int key = 32 * kx + 8 * (i >> 2) + 4 * hx + (i & 3);
        const int plane = g.th * g.tw;
        const int et = key / plane, eh = (key - et * plane) / g.tw, ew = key - et * plane - eh * g.tw;
        const int ok = (et < g.T - (g.nt - 1) * g.tt ? 1 : 0) | (eh < g.Hg - (g.nh - 1) * g.th ? 2 : 0) |
                       (ew < g.Wg - (g.nw - 1) * g.tw ? 4 : 0);
        sbias[x] = ((ok | ~code) & 7) == 7 ? 0.0f : -INFINITY;
    }
    // (the first iteration's barrier precedes every read of the table)

    f32x16 acc[kDT];
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;

    const int e0 = row_ptr[row], n = row_ptr[row + 1] - e0;
    // index word (block and edge code) of entry jj, -1 when none; jj = 0, 1, 2, ... in
    // order. The words of 64 entries are formed at once, a lane each (the edge code's
    // divisions run once per 64 blocks), and the next 64 indices load a window ahead.
    // e4m3: `cursc` holds the key tile scales of the same 64 entries, gathered at each
    // window switch (a scale read per block in the loop would be a scalar load, which
    // shares the LDS reads' wait counter and returns out of order, turning every
    // operand wait into a full drain)
    int cur = lane < n ? block_info(g, col_idx[e0 + lane]) : -1;
    int raw = 64 + lane < n ? col_idx[e0 + 64 + lane] : -1;
    int wbase = 0;
    auto gather_scales = [&]() {
        return k_scale != nullptr ? k_scale[bh * g.nb + (cur < 0 ? 0 : (cur & kBlockIdMask))] : 1.0f;
    };
    float cursc = gather_scales();
    auto info_at = [&](int jj) {
        if (jj >= n) return -1;
        if (jj - wbase == 64) {
            wbase += 64;
            cur = block_info(g, raw);
            cursc = gather_scales();
            raw = wbase + 64 + lane < n ? col_idx[e0 + wbase + 64 + lane] : -1;
        }
        return __builtin_amdgcn_readlane(cur, jj - wbase);
    };
    // scale of entry jj, right after info_at(jj) (1 past the end)
    auto scale_at = [&](int jj) {
        return jj >= n ? 1.0f
                       : __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cursc), jj - wbase));
    };
    // K and V tiles of a block copied straight into an LDS slot, this wave moving its
    // quarter of each in whole kilobytes (a missing block copies block 0)
    constexpr int kCh = kTile / 1024 / 4;
    const int lane16 = 16 * swz_unit(lane);       // swizzled source unit of this lane
    const i32x4r krs = tile_rsrc_raw(k + bh * npad * D, (uint32_t)(npad * D * 2));
    const i32x4r vrs = tile_rsrc_raw(v + bh * npad * D, (uint32_t)(npad * D * 2));
    auto copy_block = [&](int info, uint8_t* dst) {
        const uint32_t base = (uint32_t)((info < 0 ? 0 : (info & kBlockIdMask)) * kTile);
#pragma unroll
        for (int ch = 0; ch < kCh; ++ch) {
            copy_kb_asm(krs, base + (kCh * w + ch) * 1024, dst + (kCh * w + ch) * 1024, lane16);
            copy_kb_asm(vrs, base + (kCh * w + ch) * 1024, dst + kTile + (kCh * w + ch) * 1024, lane16);
        }
    };

    auto compute = [&](const uint8_t* sk, int icur, float tk) {
        const uint8_t* sv = sk + kTile;
        const int code = icur >> kEdgeShift;
        const float cs = c * tq * tk;
        bf16x8 ka[D / 16], va[D / 16];
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const int off = (kh * (D / 16) + st) * 1024 + 16 * swz_unit(lane);
            ka[st] = *reinterpret_cast<const bf16x8*>(sk + off);
            va[st] = *reinterpret_cast<const bf16x8*>(sv + off);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s, dp;
        {
            const float* bt = sbias + ((code * 2 + kh) * 2 + hb) * 16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(bt + 4 * j);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * j + e] = v[e];
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] = 0.0f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], qf.b[st], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[st], gf.b[st], dp, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 ktr[2][kDT];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int t = 0; t < kDT; ++t) ktr[ks][t] = tr_operand(sk, trb + t * 2048 + ks * 256);
        __builtin_amdgcn_sched_barrier(0);
        // element i: key 32*kh + 8*(i/4) + 4*hb + i%4, query 32*qh + lane%32
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float ds[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int i = 8 * ks + t;
                const float pp = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cs, -lq));
                ds[t] = SCALED ? pp * (dp[i] - gq) * tk : pp * (dp[i] - gq);
            }
            const bf16x8 da = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
#pragma unroll
            for (int t = 0; t < kDT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, ktr[ks][t], acc[t], 0, 0, 0);
        }
    };

    // Two slots: block j sits in slot j % 2. Iteration j first waits for its own copy
    // (issued an iteration earlier) and for every wave to leave iteration j - 1, then
    // starts the copy of block j + 1 into the other slot and computes block j.
    if (n > 0) {
        int icur = info_at(0);
        float tcur = scale_at(0);
        copy_block(icur, lds);
        for (int jj = 0; jj < n; ++jj) {
            const int inext = info_at(jj + 1);
            const float tnext = scale_at(jj + 1);
            wait_vmcnt<0>();
            __syncthreads();
            if (jj + 1 < n) copy_block(inext, lds + ((jj + 1) & 1) * kSlot);
            if (icur >= 0) compute(lds + (jj & 1) * kSlot, icur, tcur);
            icur = inext;
            tcur = tnext;
        }
    }
    wait_vmcnt<0>();
    __syncthreads();

    // add the two key halves; element i of tile t: query 32*qh + 8*(i/4) + 4*hb +
    // i%4, channel 32*t + lane%32
    float* xch = reinterpret_cast<float*>(lds + qh * kSlot);
    if (kh == 1) {
#pragma unroll
        for (int t = 0; t < kDT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) xch[(t * 16 + i) * 64 + lane] = acc[t][i];
    }
    __syncthreads();
    if (kh == 0) {
        const long row0 = row * 64 + 32 * qh;
#pragma unroll
        for (int t = 0; t < kDT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const long r = row0 + 8 * (i >> 2) + 4 * hb + (i & 3);
                dq[r * D + 32 * t + (lane & 31)] = (__bf16)(scale * (acc[t][i] + xch[(t * 16 + i) * 64 + lane]));
            }
    }
}

// ---------------------------------------------------------------- dQ, paired form

// D = 128, video grids (t > 1) of at most 4096 blocks: a workgroup owns two
// neighbouring query blocks of one (batch, head) and walks the union of their kept
// lists in ascending block order, as the paired forward does, so each K/V tile copied
// into LDS serves 128 queries instead of 64 (half the copy bytes and barriers per
// product). Wave w takes the 32 queries 32*(w & 1) .. of query block w >> 1 against
// both 32-key halves of every union block its own block keeps, one half after the
// other (scores, dP, dS and the dQ products of a half before the next), and skips the
// blocks its block does not keep; each wave then holds its queries' whole sum, so no
// partial sums are added at the end. The lists become membership bitmaps in LDS
// (entries outside [0, nb) dropped, repeats collapsing, as in the transpose the dK/dV
// pass walks). SCALED (e4m3 Q/K): the key tile scales of each 64-block window of the
// bitmaps arrive with one vector load, a lane each, and are picked per block.
constexpr int kDqMaxWords = 4096 / 32;                    // 32-bit words of one row's bitmap

template <int D, bool SCALED>
__global__ __launch_bounds__(256, 2) void k_bwd_dq_pair(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ delta,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale, Geom g, long P, float c,
    float scale, __bf16* __restrict__ dq) {
    static_assert(D == 128, "paired dQ: D = 128");
    constexpr int kTile = 64 * D * 2;
    constexpr int kSlot = 2 * kTile;              // K tile, V tile
    constexpr int kDT = D / 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kSlot];   // two slots
    // bias tiles as in k_bwd_dq: entry ((code * 2 + kh) * 2 + hb) * 16 + i is 0 when key
    // 32 kh + 8 (i / 4) + 4 hb + i % 4 of a block with edge code `code` is real, else -inf
    __shared__ __attribute__((aligned(16))) float sbias[8 * 2 * 2 * 16];
    __shared__ uint32_t bits[2][kDqMaxWords];

    const int tid = threadIdx.x, lane = tid & 63, hb = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qsel = w >> 1, qh = w & 1;
    const long p = xcd_row(P);
    const int ph = (g.nb + 1) >> 1;
    const long bh = p / ph;
    const int v0 = 2 * (int)(p - bh * ph);
    const bool hasrow = v0 + qsel < g.nb;         // uniform per wave
    const long row = bh * g.nb + (hasrow ? v0 + qsel : v0);
    const long npad = 64L * g.nb;

    KHalf<D, false> qf, gf;                        // B operands: query (lane % 32) of half qh
    load_khalf<D, false>(qf, q, row * 64, qh, lane);
    load_khalf<D, false>(gf, dout, row * 64, qh, lane);
    keep_resident<D>(qf);
    keep_resident<D>(gf);
    const float lq = lse2[row * 64 + 32 * qh + (lane & 31)];
    const float gq = delta[row * 64 + 32 * qh + (lane & 31)];
    const float tq = SCALED ? q_scale[row] : 1.0f;       // e4m3: this query block's tile scale
    const float* ksc_row = SCALED ? k_scale + bh * g.nb : nullptr;
    for (int x = tid; x < 8 * 64; x += 256) {
        const int code = x >> 6, kx = (x >> 5) & 1, hx = (x >> 4) & 1, i = x & 15;
        const int key = 32 * kx + 8 * (i >> 2) + 4 * hx + (i & 3);
        const int plane = g.th * g.tw;
        const int et = key / plane, eh = (key - et * plane) / g.tw, ew = key - et * plane - eh * g.tw;
        const int ok = (et < g.T - (g.nt - 1) * g.tt ? 1 : 0) | (eh < g.Hg - (g.nh - 1) * g.th ? 2 : 0) |
                       (ew < g.Wg - (g.nw - 1) * g.tw ? 4 : 0);
        sbias[x] = ((ok | ~code) & 7) == 7 ? 0.0f : -INFINITY;
    }
    for (int i = tid; i < 2 * kDqMaxWords; i += 256) (&bits[0][0])[i] = 0u;
    __syncthreads();
    if (hasrow) {
        const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
        for (int e = e0 + 64 * qh + lane; e < e1; e += 128) {
            const int x = col_idx[e];
            if ((unsigned)x < (unsigned)g.nb) atomicOr(&bits[qsel][x >> 5], 1u << (x & 31));
        }
    }
    __syncthreads();
    // number of union entries: lane l counts 32-bit words l and l + 64 of both bitmaps
    const int nwords = (g.nb + 63) >> 6;
    int n_union;
    {
        int cnt = 0;
        if (lane < 2 * nwords) cnt = __builtin_popcount(bits[0][lane] | bits[1][lane]);
        if (lane + 64 < 2 * nwords) cnt += __builtin_popcount(bits[0][lane + 64] | bits[1][lane + 64]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
        n_union = __builtin_amdgcn_readfirstlane(cnt);
    }
    // union entries in ascending order: the index word (block | edge code << kEdgeShift)
    // and whether this wave's query block keeps it; -1 past the end
    int gw = -1, winfo = -1;
    float wsc = 1.0f;
    uint64_t rem = 0, own = 0;
    auto word = [&](int sel, int i) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane(bits[sel][2 * i]);
        const uint32_t hi = __builtin_amdgcn_readfirstlane(bits[sel][2 * i + 1]);
        return ((uint64_t)hi << 32) | lo;
    };
    auto gen = [&](int& info, bool& mine, float& tk) {
        while (rem == 0) {
            if (gw + 1 >= nwords) {
                info = -1;
                mine = false;
                tk = 1.0f;
                return;
            }
            ++gw;
            const uint64_t a = word(0, gw), b = word(1, gw);
            rem = a | b;
            own = qsel ? b : a;
            winfo = block_info(g, 64 * gw + lane);
            if constexpr (SCALED) wsc = 64 * gw + lane < g.nb ? ksc_row[64 * gw + lane] : 1.0f;
        }
        const int bit = __builtin_ctzll(rem);
        rem &= rem - 1;
        info = __builtin_amdgcn_readlane(winfo, bit);
        mine = (own >> bit) & 1ull;
        tk = SCALED ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wsc), bit)) : 1.0f;
    };

    f32x16 acc[kDT];
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;

    constexpr int kCh = kTile / 1024 / 4;
    const int lane16 = 16 * swz_unit(lane);       // swizzled source unit of this lane
    const i32x4r krs = tile_rsrc_raw(k + bh * npad * D, (uint32_t)(npad * D * 2));
    const i32x4r vrs = tile_rsrc_raw(v + bh * npad * D, (uint32_t)(npad * D * 2));
    auto copy_block = [&](int info, uint8_t* dst) {
        const uint32_t base = (uint32_t)((info < 0 ? 0 : (info & kBlockIdMask)) * kTile);
#pragma unroll
        for (int ch = 0; ch < kCh; ++ch) {
            copy_kb_asm(krs, base + (kCh * w + ch) * 1024, dst + (kCh * w + ch) * 1024, lane16);
            copy_kb_asm(vrs, base + (kCh * w + ch) * 1024, dst + kTile + (kCh * w + ch) * 1024, lane16);
        }
    };

    // key half kh of a kept block: scores and dP (starting from the block's bias tile),
    // then dS, then the dQ products over the half's 32 keys
    auto compute_half = [&](const uint8_t* sk, int code, float tk, auto khc) {
        constexpr int kh = decltype(khc)::value;
        const float cs = SCALED ? c * tq * tk : c;
        const uint8_t* sv = sk + kTile;
        bf16x8 ka[D / 16], va[D / 16];
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const int off = (kh * (D / 16) + st) * 1024 + 16 * swz_unit(lane);
            ka[st] = *reinterpret_cast<const bf16x8*>(sk + off);
            va[st] = *reinterpret_cast<const bf16x8*>(sv + off);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s, dp;
        {
            const float* bt = sbias + ((code * 2 + kh) * 2 + hb) * 16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(bt + 4 * j);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * j + e] = b4[e];
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] = 0.0f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], qf.b[st], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[st], gf.b[st], dp, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int trb = tr_base<D>(32 * kh, lane);
        bf16x8 ktr[2][kDT];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int t = 0; t < kDT; ++t) ktr[ks][t] = tr_operand(sk, trb + t * 2048 + ks * 256);
        __builtin_amdgcn_sched_barrier(0);
        // element i: key 32*kh + 8*(i/4) + 4*hb + i%4, query 32*qh + lane%32
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float ds[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int i = 8 * ks + t;
                const float pp = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cs, -lq));
                ds[t] = SCALED ? pp * (dp[i] - gq) * tk : pp * (dp[i] - gq);
            }
            const bf16x8 da = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
#pragma unroll
            for (int t = 0; t < kDT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, ktr[ks][t], acc[t], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Two slots: union block j sits in slot j % 2. Iteration j waits for its own copy
    // (issued an iteration earlier) and for every wave to leave iteration j - 1, then
    // starts the copy of block j + 1 into the other slot and computes block j if this
    // wave's query block keeps it.
    if (n_union > 0) {
        int icur;
        bool mcur;
        float tcur;
        gen(icur, mcur, tcur);
        copy_block(icur, lds);
        for (int jj = 0; jj < n_union; ++jj) {
            int inext;
            bool mnext;
            float tnext;
            gen(inext, mnext, tnext);
            wait_vmcnt<0>();
            __syncthreads();
            if (jj + 1 < n_union) copy_block(inext, lds + ((jj + 1) & 1) * kSlot);
            if (mcur && hasrow) {                      // uniform per wave
                const uint8_t* sk = lds + (jj & 1) * kSlot;
                const int code = icur >> kEdgeShift;
                compute_half(sk, code, tcur, std::integral_constant<int, 0>());
                compute_half(sk, code, tcur, std::integral_constant<int, 1>());
            }
            icur = inext;
            mcur = mnext;
            tcur = tnext;
        }
    }
    wait_vmcnt<0>();
    if (!hasrow) return;
    // element i of tile t: query 32*qh + 8*(i/4) + 4*hb + i%4, channel 32*t + lane%32
    const long row0 = row * 64 + 32 * qh;
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const long r = row0 + 8 * (i >> 2) + 4 * hb + (i & 3);
            dq[r * D + 32 * t + (lane & 31)] = (__bf16)(scale * acc[t][i]);
        }
}

// ---------------------------------------------------------------- host

size_t bwd_workspace_bytes(int B, int H, int nb) { return 2 * (size_t)B * H * nb * 64 * sizeof(float); }

template <int D>
static void launch_bwd_d(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                         const int32_t* col_ptr, const int32_t* row_idx, const float* q_scale,
                         const float* k_scale, int B, int H, const Geom& g, float scale, int o_f32,
                         void* dq, void* dk, void* dv, void* ws, hipStream_t st) {
    const long rows = (long)B * H * g.nb;
    float* lse2 = static_cast<float*>(ws);
    float* delta = lse2 + rows * 64;
    const float c = scale * kLog2e;
    auto bq = static_cast<const __bf16*>(q);
    auto bk = static_cast<const __bf16*>(k);
    auto bv = static_cast<const __bf16*>(v);
    auto bg = static_cast<const __bf16*>(dout);
    if (o_f32)
        k_bwd_prep<D, float><<<(unsigned)rows, 256, 0, st>>>(static_cast<const float*>(o), bg, lse, g, lse2, delta);
    else
        k_bwd_prep<D, __bf16><<<(unsigned)rows, 256, 0, st>>>(static_cast<const __bf16*>(o), bg, lse, g, lse2, delta);
    // the host checks that q_scale and k_scale are both given or both NULL
    if (q_scale != nullptr) {
        k_bwd_dkdv<D, true><<<(unsigned)rows, 256, 0, st>>>(bq, bk, bv, bg, lse2, delta, col_ptr, row_idx, q_scale,
                                                            k_scale, g, c, scale, static_cast<__bf16*>(dk),
                                                            static_cast<__bf16*>(dv));
        if constexpr (D == 128) {
            if (g.T > 1 && g.nb <= kDqMaxWords * 32) {
                const long P = (long)B * H * ((g.nb + 1) / 2);
                k_bwd_dq_pair<D, true><<<(unsigned)P, 256, 0, st>>>(bq, bk, bv, bg, lse2, delta, row_ptr, col_idx,
                                                                     q_scale, k_scale, g, P, c, scale,
                                                                     static_cast<__bf16*>(dq));
                return;
            }
        }
        k_bwd_dq<D, true><<<(unsigned)rows, 256, 0, st>>>(bq, bk, bv, bg, lse2, delta, row_ptr, col_idx, q_scale,
                                                          k_scale, g, c, scale, static_cast<__bf16*>(dq));
    } else {
        k_bwd_dkdv<D, false><<<(unsigned)rows, 256, 0, st>>>(bq, bk, bv, bg, lse2, delta, col_ptr, row_idx, nullptr,
                                                             nullptr, g, c, scale, static_cast<__bf16*>(dk),
                                                             static_cast<__bf16*>(dv));
        if constexpr (D == 128) {
            if (g.T > 1 && g.nb <= kDqMaxWords * 32) {
                const long P = (long)B * H * ((g.nb + 1) / 2);
                k_bwd_dq_pair<D, false><<<(unsigned)P, 256, 0, st>>>(bq, bk, bv, bg, lse2, delta, row_ptr, col_idx,
                                                                      nullptr, nullptr, g, P, c, scale,
                                                                      static_cast<__bf16*>(dq));
                return;
            }
        }
        k_bwd_dq<D, false><<<(unsigned)rows, 256, 0, st>>>(bq, bk, bv, bg, lse2, delta, row_ptr, col_idx, nullptr,
                                                           nullptr, g, c, scale, static_cast<__bf16*>(dq));
    }
}

void launch_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, const int32_t* row_ptr,
                            const int32_t* col_idx, const int32_t* col_ptr, const int32_t* row_idx,
                            const float* q_scale, const float* k_scale, int B, int H, int D, const Geom& g,
                            float scale, int o_f32, void* dq, void* dk, void* dv, void* ws, hipStream_t st) {
    if (D == 128)
        launch_bwd_d<128>(q, k, v, o, dout, lse, row_ptr, col_idx, col_ptr, row_idx, q_scale, k_scale, B, H, g,
                          scale, o_f32, dq, dk, dv, ws, st);
    else
        launch_bwd_d<64>(q, k, v, o, dout, lse, row_ptr, col_idx, col_ptr, row_idx, q_scale, k_scale, B, H, g,
                         scale, o_f32, dq, dk, dv, ws, st);
}

}  // namespace fpsa
