// Block-sparse attention forward over the kept key blocks of each query block,
// with an online softmax (FlashAttention style) [FPSAttention: Training-Aware FP8
// and Sparsity Co-Design for Fast Video Diffusion, Abstract] and the frozen block
// indices of the retained-mass selection [LoSA: Near-Lossless Sparse Attention for
// Training-Free Video Diffusion Acceleration, Abstract].
//
// gfx950 mapping. A workgroup of four waves owns one query block (64 rows) of one
// (batch, head) and walks the block's CSR list in order. The K and V tiles of each
// kept block are copied once per workgroup into LDS with direct global-to-LDS loads
// (buffer_load_dwordx4 ... lds, each wave moving a quarter of each tile in contiguous
// kilobytes) into two-slot K and V rings, K two blocks and V one block ahead of
// use; one barrier per block. The e4m3 variant issues its copies from inline asm and
// reads the second half of its V operands later in the block, which fits it in 168
// registers and three workgroups per CU (its K ring is half the size). Wave w takes query rows 32*(w & 1) .. +31 and key
// rows 32*(w >> 1) .. +31 of every block (the layout conventions are described in
// attn_common.h); the two key halves of a query row carry separate online-softmax
// states that are merged once at the end through LDS. Workgroups are remapped so
// that each XCD gets a contiguous range of rows (same heads), which keeps the
// shared K/V tiles in that XCD's L2; on 2D grids the rows run in strips of 8 block
// columns (strip_row), which keeps a structured mask's row and column blocks shared.
#include "attn_common.h"
#include "fpsa_internal.h"

namespace fpsa {

constexpr int kAttnThreads = 256;

// CNT: the real keys of each key block are its first kcount[(b*H + h)*nb + kb] slots
// (blocks of a cluster-contiguous layout) instead of following from the token grid.
template <int D, bool FP8, bool CNT>
__global__ __launch_bounds__(kAttnThreads, FP8 ? 3 : 2) void k_sparse_attn(
    const void* __restrict__ qv, const void* __restrict__ kv, const __bf16* __restrict__ vt,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, Geom g, long R,
    float scale_log2, __bf16* __restrict__ o, float* __restrict__ lse, float* __restrict__ o32,
    const int32_t* __restrict__ kcount) {
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

    const long r = strip_row(xcd_row(R), g);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qh = w & 1, kh = w >> 1;
    const int half = lane >> 5;
    const long bh = r / g.nb;
    const int qb = (int)(r - bh * g.nb);
    const long npad = (long)g.nb * kBlock;
    const long qblk0 = bh * npad + (long)qb * kBlock;
    EdgeSlots edge;
    edge.init(g, lane);

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

    const int e0 = __builtin_amdgcn_readfirstlane(row_ptr[r]);
    const int n = __builtin_amdgcn_readfirstlane(row_ptr[r + 1]) - e0;
    const uint8_t* kbytes = static_cast<const uint8_t*>(kv) + bh * npad * D * (FP8 ? 1 : 2);
    const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(vt) + bh * (long)g.nb * kVBytes;
    const float* ksc_row = FP8 ? k_scale + bh * g.nb : nullptr;

    // Kept-block indices, 64 per VGPR: `cur` holds the index words (block index and
    // edge code) of entries base .. base+63, `raw` the plain indices of the next 64,
    // loaded 64 blocks before they are needed; single entries are picked with
    // v_readlane, so the loop never waits on an index load.
    auto info_of = [&](int x) {
        if constexpr (CNT) {
            if (x < 0 || x >= g.nb) return -1;
            const int c = kcount[bh * g.nb + x];
            return c >= kBlock ? x : (x | ((kBlock - max(c, 0)) << kEdgeShift));
        } else {
            return block_info(g, x);
        }
    };
    int cur = info_of(lane < n ? col_idx[e0 + lane] : -1);
    int raw = 64 + lane < n ? col_idx[e0 + 64 + lane] : -1;
    int base = 0;
    auto info_at = [&](int jj) {          // jj = 0, 1, 2, ... in order
        if (jj - base == 64) {
            base += 64;
            cur = info_of(raw);
            raw = base + 64 + lane < n ? col_idx[e0 + base + 64 + lane] : -1;
        }
        return __builtin_amdgcn_readlane(cur, jj - base);
    };
    auto block_of = [](int info) { return info < 0 ? 0 : (info & kBlockIdMask); };

    // Copy the K (or V) tile of a block into ring slot `slot`: this wave moves its
    // share of the tile's LDS kilobytes, lane l carrying 16 bytes each. LDS kilobyte c
    // of a K tile holds, for bf16, the same kilobyte of the tile (lane l: bytes 16 l);
    // for e4m3, half c % 2 of the 2 KB operand step c / 2 (lane l: bytes 32 l + 16 (c % 2)),
    // the split layout the e4m3 operand reads expect. An entry with no block copies
    // block 0 (never read as data).
    const int lane16 = 16 * lane;
    const int klane = FP8 ? 32 * lane : 16 * lane;
    auto ksrc = [](int c) -> uint32_t { return FP8 ? (c >> 1) * 2048 + 16 * (c & 1) : c * 1024; };
    const __amdgpu_buffer_rsrc_t krs = tile_rsrc(kbytes, (uint32_t)(g.nb * kKBytes));
    const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(vbytes, (uint32_t)(g.nb * kVBytes));
    const i32x4r krs_a = tile_rsrc_raw(kbytes, (uint32_t)(g.nb * kKBytes));
    const i32x4r vrs_a = tile_rsrc_raw(vbytes, (uint32_t)(g.nb * kVBytes));
    auto kcopy = [&](uint32_t off, uint8_t* dst) {
        if constexpr (FP8) copy_kb_asm(krs_a, off, dst, klane);
        else copy_kb_to_lds(krs, off, dst, klane);
    };
    auto vcopy = [&](uint32_t off, uint8_t* dst) {
        if constexpr (FP8) copy_kb_asm(vrs_a, off, dst, lane16);
        else copy_kb_to_lds(vrs, off, dst, lane16);
    };
    auto copy_k = [&](int info, int slot) {
#pragma unroll
        for (int i = 0; i < kKChunks; ++i)
            kcopy((uint32_t)(block_of(info) * kKBytes) + ksrc(kKChunks * w + i),
                  kring + slot * kKBytes + (kKChunks * w + i) * 1024);
    };
    auto copy_v = [&](int info, int slot) {
#pragma unroll
        for (int i = 0; i < kVChunks; ++i)
            vcopy((uint32_t)(block_of(info) * kVBytes + (kVChunks * w + i) * 1024),
                  vring + slot * kVBytes + (kVChunks * w + i) * 1024);
    };

    // Software pipeline across kept blocks. Iteration j holds the scores of block j
    // (issued one iteration earlier). Its first part masks the padding keys of an
    // edge block, takes the block maximum and rescales the running state when the
    // maximum moved (rare). After the barrier, one straight-line section reads K of
    // block j+1 and V of block j from LDS, starts the copies of V(j+1) (over V(j-1))
    // and K(j+2) (over K(j)), both read by every wave before the barrier, issues the
    // QK^T products of block j+1 and, interleaved with them, the exponentials and
    // P*V products of block j. The last iteration's reads and copies touch unused
    // slots and block 0 only; its extra products are discarded.
    KHalf<D, FP8> k;
    bf16x8 v[kDT][2];
    int inf = -1, infn = -1;
    float ksc = 1.0f, kscn = 1.0f;
    float smax = -INFINITY;       // unmasked maximum of the current block's scores
    auto step = [&](int j, f32x16& s, f32x16& sn) {
        const int inf2 = info_at(j + 2);
        const float ksc2 = FP8 ? ksc_row[block_of(inf2)] : 1.0f;
        const float c = FP8 ? cq * ksc : cq;
        const int code = inf >> kEdgeShift;           // 0: interior block; < 0: no block
        uint64_t vm;
        if constexpr (CNT)   // code = 64 - real keys, which are the block's first slots
            vm = code == 0 ? ~0ull : ((inf < 0 || code >= kBlock) ? 0ull : (~0ull >> code));
        else
            vm = code == 0 ? ~0ull : (inf < 0 ? 0ull : edge.mask(code));
        const float nref = softmax_enter<kDT>(s, code == 0, vm, smax, c, kh, half, acc, m, l);

        // K(j+1) and V(j) landed; every wave is done with iteration j-1's reads
        copies_landed_barrier();
        const uint8_t* kst = kring + ((j + 1) & 1) * kKBytes;
        const uint8_t* vst = vring + (j & 1) * kVBytes;
        // copy i < kKChunks: kilobyte i of this wave's share of K(j+2); then V(j+1)
        auto copy_one = [&](int i) {
            if (i < kKChunks)
                kcopy((uint32_t)(block_of(inf2) * kKBytes) + ksrc(kKChunks * w + i),
                      kring + (j & 1) * kKBytes + (kKChunks * w + i) * 1024);
            else
                vcopy((uint32_t)(block_of(infn) * kVBytes + (kVChunks * w + i - kKChunks) * 1024),
                      vring + ((j + 1) & 1) * kVBytes + (kVChunks * w + i - kKChunks) * 1024);
        };
        constexpr int kCopies = kKChunks + kVChunks;
        if constexpr (D == 128 && !FP8)
            block_main_bf16_d128<kCopies>(kst, vst, kh, lane, q, k, v, acc, s, sn, c, nref, l, smax, copy_one);
        else if constexpr (D == 128 && FP8)
            block_main_fp8_d128<kCopies>(kst, vst, kh, lane, q, k, v, acc, s, sn, c, nref, l, smax, copy_one);
        else
            block_main_generic<D, FP8, kCopies>(kst, vst, kh, lane, q, k, v, acc, s, sn, c, nref, l, smax, copy_one);

        inf = infn;
        infn = inf2;
        ksc = kscn;
        kscn = ksc2;
    };

    f32x16 s0, s1;
    if (n > 0) {
        inf = info_at(0);
        infn = info_at(1);
        if constexpr (FP8) {
            ksc = ksc_row[block_of(inf)];
            kscn = ksc_row[block_of(infn)];
        }
        copy_k(inf, 0);
        copy_v(inf, 0);
        copy_k(infn, 1);
        copies_landed_barrier();                      // K(0), V(0), K(1) landed
        lds_khalf<D, FP8>(k, kring, kh, lane);
        qk_scores<D, FP8>(s0, k, q);
        smax = max16(s0);
        for (int j = 0; j < n; j += 2) {
            step(j, s0, s1);
            if (j + 1 < n) step(j + 1, s1, s0);
        }
    }

    // The last iteration's copies target the memory the merge uses: drain them.
    copies_landed_barrier();
    merge_and_store<D>(reinterpret_cast<float*>(lds), qh, kh, lane, acc, m, l, true, g, qb, qblk0, o, lse, o32);
}

void launch_sparse_attn(const void* q, const void* k, const void* v, int fp8, const float* q_scale,
                        const float* k_scale, const int32_t* row_ptr, const int32_t* col_idx,
                        int B, int H, int D, const Geom& g, float scale, void* o, float* lse, float* o32,
                        const int32_t* kcount, hipStream_t st) {
    const long R = (long)B * H * g.nb;
    const float sl2 = scale * kLog2e;
    const __bf16* vt = static_cast<const __bf16*>(v);
    __bf16* out = static_cast<__bf16*>(o);
    dim3 grid((unsigned)R), block(kAttnThreads);
    if (D == 128) {
        if (fp8) k_sparse_attn<128, true, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse, o32, nullptr);
        else if (kcount) k_sparse_attn<128, false, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse, o32, kcount);
        else k_sparse_attn<128, false, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse, o32, nullptr);
    } else {
        if (fp8) k_sparse_attn<64, true, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse, o32, nullptr);
        else if (kcount) k_sparse_attn<64, false, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse, o32, kcount);
        else k_sparse_attn<64, false, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R, sl2, out, lse, o32, nullptr);
    }
}

}  // namespace fpsa
