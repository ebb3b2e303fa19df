// Block-sparse attention forward over the kept key blocks of each query block,
// with an online softmax (FlashAttention style) [FPSAttention: Training-Aware FP8
// and Sparsity Co-Design for Fast Video Diffusion, Abstract] and the frozen block
// indices of the retained-mass selection [LoSA: Near-Lossless Sparse Attention for
// Training-Free Video Diffusion Acceleration, Abstract].
//
// Two gfx950 kernels.
//
// k_sparse_attn_pair (bf16 or e4m3 Q/K, D = 128, blocks of a video grid (T > 1) or bf16
// blocks with counted keys, at most 4096 blocks; the main path): a workgroup of four waves owns two neighbouring query
// blocks and walks the union of their kept lists in ascending block order, so every
// K/V tile copied into LDS serves 128 queries (half the copy bytes and barriers per
// product of a one-block workgroup). Each wave takes 32 query rows of one of the two
// blocks against all 64 keys of every union block; blocks its own query block does
// not keep, and padding keys, are excluded by a -inf bias tile that starts the QK^T
// chain. The bf16 call without lse takes queries pre-scaled to base-2 units (rounded to
// bf16 once) and shifted scores, with no scale-and-shift step per score. See the
// comment above the kernel.
//
// k_sparse_attn (D = 64, 2D grids, grids over 4096 blocks):
// a workgroup of four waves owns one query block (64 rows) of one (batch, head) and walks the
// block's CSR list in order (bf16, D = 128, no lse: pre-scaled queries, as in the paired
// kernel). The K and V tiles of each kept block are copied once per
// workgroup into LDS with direct global-to-LDS loads (buffer_load_dwordx4 ... lds,
// each wave moving a quarter of each tile in contiguous kilobytes) into two-slot K
// and V rings, K two blocks and V one block ahead of use; one barrier per block. The
// e4m3 variant issues its copies from inline asm and reads the second half of its V
// operands later in the block, which fits it in 168 registers and three workgroups
// per CU (its K ring is half the size). Wave w takes query rows 32*(w & 1) .. +31 and
// key rows 32*(w >> 1) .. +31 of every block (the layout conventions are described in
// attn_common.h); the two key halves of a query row carry separate online-softmax
// states that are merged once at the end through LDS.
//
// On video grids both remap workgroups so that each XCD gets a contiguous range of
// rows (same heads), which keeps the shared K/V tiles in that XCD's L2. On 2D grids the
// rows run in strips of 8 block columns (strip_row), which keeps a structured mask's
// row and column blocks shared, and the eight XCDs take consecutive 64-row patches of
// one head at a time (xcd_chunk_row), so that head's K and V stay in the infinity
// cache.
#include <type_traits>

#include "attn_common.h"
#include "fpsa_internal.h"

namespace fpsa {

constexpr int kAttnThreads = 256;

// CNT: the real keys of each key block are its first kcount[(b*H + h)*nb + kb] slots
// (blocks of a cluster-contiguous layout) instead of following from the token grid.
// SHIFT (bf16, D = 128, the call without lse): queries pre-scaled to base-2 units and
// score chains that start from -r, as in the paired kernel.
template <int D, bool FP8, bool CNT, bool SHIFT = false>
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

    // 2D grids: the strip order's 8 x 8 patches, one per XCD, all eight from one head at
    // a time (its K and V fit the infinity cache: 8.6 % faster at 8192 x 8192 than one
    // range of heads per XCD); video grids keep one contiguous range per XCD
    const long r = strip_row(strip_grid(g) ? xcd_chunk_row(R) : xcd_row(R), g);
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
    static_assert(!SHIFT || (D == 128 && !FP8), "pre-scaled queries: bf16, D = 128");
    if constexpr (SHIFT) {
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) q.b[j][e] = (__bf16)((float)q.b[j][e] * scale_log2);
    }
    f32x16 mt;                                        // SHIFT: -r in every element
#pragma unroll
    for (int i = 0; i < 16; ++i) mt[i] = 0.0f;

    f32x16 acc[kDT];
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
    // m: the query's running reference (the same in both lane halves); l: this lane's share
    // of the row sum (its keys of each block), the two halves added once at the end
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
    // e4m3: `cursc` holds the key tile scales of the same 64 entries, gathered at each
    // window switch (a scale read per block inside the loop would be a scalar load,
    // which shares the LDS reads' wait counter and returns out of order, turning every
    // operand wait into a full drain)
    int cur = info_of(lane < n ? col_idx[e0 + lane] : -1);
    int raw = 64 + lane < n ? col_idx[e0 + 64 + lane] : -1;
    int base = 0;
    auto gather_scales = [&]() { return FP8 ? ksc_row[cur < 0 ? 0 : (cur & kBlockIdMask)] : 1.0f; };
    float cursc = gather_scales();
    auto info_at = [&](int jj) {          // jj = 0, 1, 2, ... in order
        if (jj - base == 64) {
            base += 64;
            cur = info_of(raw);
            cursc = gather_scales();
            raw = base + 64 + lane < n ? col_idx[e0 + base + 64 + lane] : -1;
        }
        return __builtin_amdgcn_readlane(cur, jj - base);
    };
    // scale of entry jj, right after info_at(jj)
    auto scale_at = [&](int jj) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cursc), jj - base));
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
        const float ksc2 = FP8 ? scale_at(j + 2) : 1.0f;
        const float c = FP8 ? cq * ksc : cq;
        const int code = inf >> kEdgeShift;           // 0: interior block; < 0: no block
        uint64_t vm;
        if constexpr (CNT)   // code = 64 - real keys, which are the block's first slots
            vm = code == 0 ? ~0ull : ((inf < 0 || code >= kBlock) ? 0ull : (~0ull >> code));
        else
            vm = code == 0 ? ~0ull : (inf < 0 ? 0ull : edge.mask(code));
        float nref = 0.0f;
        if constexpr (SHIFT) softmax_enter_shifted<kDT>(s, code == 0, vm, smax, kh, half, acc, mt, m, l);
        else nref = softmax_enter<kDT>(s, code == 0, vm, smax, c, kh, half, acc, m, l);

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
            block_main_bf16_d128<kCopies, SHIFT>(kst, vst, kh, lane, q, k, v, acc, s, sn, mt, c, nref, l, smax,
                                                 copy_one);
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
        if constexpr (FP8) ksc = scale_at(0);
        infn = info_at(1);
        if constexpr (FP8) kscn = scale_at(1);
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
    l = wave_add32(l);                                // the two lane halves of each query
    merge_and_store<D>(reinterpret_cast<float*>(lds), qh, kh, lane, acc, m, l, true, g, qb, qblk0, o, lse, o32);
}

// ---------------------------------------------------------------------------------
// Paired form (D = 128, token-grid or counted blocks, nb <= 4096). One workgroup owns two
// neighbouring query blocks of one (batch, head) and walks the union of their kept
// lists, so each K/V tile copied into LDS serves 128 queries instead of 64: half the
// copy bytes and barriers per product. Wave w takes the 32 query rows 32*(w & 1) ..
// of query block w >> 1 against all 64 keys of every union block. The union is
// walked in ascending block order from two 4096-bit membership bitmaps built in LDS
// (a repeated entry counts once; entries outside [0, nb) are ignored). A union block
// the wave's own query block does not keep contributes nothing: its scores are -inf.
//
// Key masking costs no vector instruction: every QK^T chain starts from a bias tile
// instead of from zero, 0 for a real key and -inf for a padding key of an edge block
// (or for every key of a block the wave does not keep). A small LDS table holds, per
// edge code (and the "nothing" code), the 2 x 16 accumulator values of each lane half;
// for counted blocks (the real keys of key block kb are its first kcount[kb] slots) the
// code is the number of padding keys and the table holds the 17 prefix patterns of a
// 16-element tile.
//
// Two forms for bf16. The inference form (SHIFT; the call without lse) multiplies the
// queries by scale * log2(e) once and rounds them to bf16, so the products give base-2
// scores; its C tiles also carry -r, the running reference of the online softmax, so
// the scores come out shifted and go straight into the exponentials (no scale-and-shift
// instruction per score). Those tiles stay in registers and are re-read from the table
// only when the edge code changes between union blocks (a run of block columns shares
// it) and moved with r when the reference grows. The form that also returns lse (for a
// backward pass, which recomputes exact scores against it) and the e4m3 form keep the
// float32 scale-and-shift per score and read each block's tile at the end of block
// u-1's section into the registers that hold its scores one section later.
// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1, so that every
// index into a section's register arrays is a constant whatever the unroller decides.
template <int B, int E, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

constexpr int kPairThreads = 256;
constexpr int kMaxBitmapWords = 4096 / 32;               // 32-bit words of one row's bitmap
constexpr int kBiasCodes = 9;                            // edge codes 0..7, then "nothing kept"

__device__ inline float max16_lane(const f32x16& x) {
    const float a = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    const float b = fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]));
    const float d = fmaxf(fmaxf(x[8], x[9]), fmaxf(x[10], x[11]));
    const float e = fmaxf(fmaxf(x[12], x[13]), fmaxf(x[14], x[15]));
    return fmaxf(fmaxf(a, b), fmaxf(d, e));
}

// Bias tiles of code `bc` for this lane: element i of tile kt is key 32 kt + 8 (i / 4)
// + 4 half + i % 4 of the block. Grid blocks (CNT false): the table holds both tiles per
// edge code. Counted blocks (CNT): `bc` is the number of padding keys at the block's end
// (64 - real keys; 64 for a block the wave does not keep). A tile's keys increase with i,
// so its real keys are a prefix of v elements, and row v of a table of the 17 prefix
// patterns (v zeros, then -inf) is the tile.
template <bool CNT>
__device__ __attribute__((always_inline)) inline void load_bias(f32x16 (&t)[2], const float* table, int bc,
                                                                 int half) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        const float* row;
        if constexpr (CNT) {
            // real keys of this tile: those below c' = (64 - bc) - 32 kt - 4 half among
            // 0..3, 8..11, 16..19, 24..27 (arithmetic shift and mask also hold for c' < 0)
            const int cp = kBlock - bc - 32 * kt - 4 * half;
            const int v = min(max(4 * (cp >> 3) + min(cp & 7, 4), 0), 16);
            row = table + 16 * v;
        } else {
            row = table + ((bc * 2 + half) * 2 + kt) * 16;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(row + 4 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) t[kt][4 * j + e] = v4[e];
        }
    }
}

// Main section of union block u for this wave: the QK^T of block u+1 (two 32-key
// halves) and the exponentials and P*V of block u (16 products), in a fixed issue
// order. Each QK^T chain starts from a tile of the block's bias: with SHIFT the tile
// ct[kt], which also carries -r and so shifts the scores to the reference r; otherwise
// the tile already in sn (read at the end of the previous section). K(u+1) and V(u)
// operands are read from LDS four products ahead of use; the NC copies into LDS
// (inline asm, so that no read waits for them) go one after each of the first NC
// products. The vector steps of the softmax (per pair of scores: two exponentials,
// one bf16 pack, one dot into the row sum, and without SHIFT first two scale-and-shift
// FMAs; with SHIFT the scores already sit in base-2 units relative to r) run as a
// stream after a few up front. Without SHIFT, s receives the bias tile of block u+2 at
// the end.
template <bool FP8, bool SHIFT, bool CNT, int NC, class Copy>
__device__ __attribute__((always_inline)) inline void pair_main(
    const uint8_t* kst, const uint8_t* vst, int lane, int half, const KHalf<128, FP8>& q, f32x16 (&acc)[4],
    f32x16 (&s)[2], f32x16 (&sn)[2], const f32x16 (&ct)[2], float c, float nref, float& l, float& smax,
    const float* bias_table, int bias_next, Copy&& copy_one) {
    // products of the next block's QK^T: 16 bf16 32x32x16, or 4 e4m3 32x32x64
    constexpr int kQK = FP8 ? 4 : 16;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8 kk[8];
    i32x8 kf[4];
    bf16x8 vv[8];
    float pf[2][16];
    uint32_t pw[2][8];
    float rs[2] = {0.0f, 0.0f};
    float mx0 = -INFINITY, mx1 = -INFINITY;
    // K operand of product n: bf16, half n / 8 and step n % 8, one kilobyte; e4m3, half
    // n / 2 and step n % 2, the two halves of a 2 KB step split in LDS
    auto KR = [&](int n) {
        if constexpr (FP8) {
            const uint8_t* p = kst + n * 2048 + 16 * lane;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 1024);
            kf[n & 3] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            kk[n & 7] = *reinterpret_cast<const bf16x8*>(kst + n * 1024 + 16 * lane);
        }
    };
    // V operand of P*V product n (0..15: half kt = n / 8, cc = (n / 4) % 2, t = n % 4)
    auto VR = [&](int n) {
        const int kt = n >> 3, cc = (n >> 2) & 1, t = n & 3;
        vv[n & 7] = *reinterpret_cast<const bf16x8*>(vst + (t * 4 + 2 * kt + cc) * 1024 + 16 * lane);
    };
    auto QK = [&](int n) {
        if constexpr (FP8) {
            const int kt = n >> 1, st = n & 1;
            sn[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[n & 3], q.f[st], sn[kt], 0, 0, 0, 0, 0, 0);
        } else {
            const int kt = n >> 3, st = n & 7;
            sn[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[n & 7], q.b[st], (SHIFT && st == 0) ? ct[kt] : sn[kt],
                                                             0, 0, 0);
        }
    };
    auto PV = [&](int n) {
        const int kt = n >> 3, cc = (n >> 2) & 1, t = n & 3;
        const i32x4 wv = {(int)pw[kt][4 * cc], (int)pw[kt][4 * cc + 1], (int)pw[kt][4 * cc + 2],
                          (int)pw[kt][4 * cc + 3]};
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[n & 7], __builtin_bit_cast(bf16x8, wv), acc[t], 0, 0, 0);
    };
    // vector step k of the softmax stream (k = 0..95)
    auto VS = [&](int k) {
        const int pr = k / 6, op = k % 6, kt = pr >> 3, i = 2 * (pr & 7);
        if (op == 0) pf[kt][i] = SHIFT ? s[kt][i] : __builtin_fmaf(s[kt][i], c, nref);
        else if (op == 1) pf[kt][i + 1] = SHIFT ? s[kt][i + 1] : __builtin_fmaf(s[kt][i + 1], c, nref);
        else if (op == 2) pf[kt][i] = __builtin_amdgcn_exp2f(pf[kt][i]);
        else if (op == 3) pf[kt][i + 1] = __builtin_amdgcn_exp2f(pf[kt][i + 1]);
        else if (op == 4) {
            bf16x2 b;
            b[0] = (__bf16)pf[kt][i];
            b[1] = (__bf16)pf[kt][i + 1];
            pw[kt][i >> 1] = __builtin_bit_cast(uint32_t, b);
        } else {
            rs[kt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[kt][i >> 1]), ones, rs[kt], false);
        }
    };
    // running maximum over the next block's scores 4 gi .. 4 gi + 3 of half kt (a chain of
    // three-input maxima)
    auto MX = [&](int kt, int gi) {
        float& mx = kt == 0 ? mx0 : mx1;
        mx = fmaxf(fmaxf(mx, sn[kt][4 * gi]), sn[kt][4 * gi + 1]);
        mx = fmaxf(fmaxf(mx, sn[kt][4 * gi + 2]), sn[kt][4 * gi + 3]);
    };
#define FPSA_SB __builtin_amdgcn_sched_barrier(0)
    if constexpr (FP8) {
        // 20 products: the 4 QK^T first (their K operands read up front), then the 16
        // P*V, V read four products ahead; 32 vector steps up front and 4 per product
        // finish the softmax stream before the last P*V product that needs it
        static_for<0, 4>([&](auto kc) { KR(decltype(kc)::value); });
        static_for<0, 32>([&](auto kc) { VS(decltype(kc)::value); });
        FPSA_SB;
        static_for<0, 20>([&](auto nc) {
            constexpr int n = decltype(nc)::value;
            if constexpr (n < kQK) QK(n);
            else PV(n - kQK);
            if constexpr (n < NC) copy_one(n);
            if constexpr (n < 16) VR(n);
            static_for<32 + 4 * n, (36 + 4 * n < 96 ? 36 + 4 * n : 96)>([&](auto kc) { VS(decltype(kc)::value); });
            if constexpr (n >= 8 && n < 12) MX(0, n - 8);
            if constexpr (n >= 12 && n < 16) MX(1, n - 12);
            if constexpr (n == 16) load_bias<CNT>(s, bias_table, bias_next, half);   // every score of block u is consumed
            if constexpr (n == 17) l += rs[0] + rs[1];
            if constexpr (n == 19) smax = wave_max32(fmaxf(mx0, mx1));
            FPSA_SB;
        });
    } else {
        KR(0); KR(1); KR(2); KR(3);
        static_for<0, 12>([&](auto kc) { VS(decltype(kc)::value); });
        FPSA_SB;
        static_for<0, 32>([&](auto nc) {
            constexpr int n = decltype(nc)::value;
            if constexpr (n < kQK) QK(n);
            else PV(n - kQK);
            if constexpr (n < NC) copy_one(n);
            // operand reads four products ahead: K of products 4..15, then V of 0..15
            if constexpr (n + 4 < 16) KR(n + 4);
            else if constexpr (n + 4 - 16 < 16) VR(n + 4 - 16);
            static_for<12 + 3 * n, (15 + 3 * n < 96 ? 15 + 3 * n : 96)>([&](auto kc) { VS(decltype(kc)::value); });
            if constexpr (n >= 20 && n < 24) MX(0, n - 20);
            if constexpr (n >= 24 && n < 28) MX(1, n - 24);
            // every score of block u is consumed: s takes block u+2's bias tile
            if constexpr (!SHIFT && n == 28) load_bias<CNT>(s, bias_table, bias_next, half);
            if constexpr (n == 30) l += rs[0] + rs[1];
            if constexpr (n == 31) smax = wave_max32(fmaxf(mx0, mx1));
            FPSA_SB;
        });
    }
#undef FPSA_SB
}

// Lazy rescale at the entry of a union block: when the block's maximum (bias included,
// so padding keys and blocks the wave does not keep are excluded) exceeds the running
// reference by more than the slack, move the reference and rescale the state. Returns
// -m (0 before any key).
__device__ __attribute__((always_inline)) inline float pair_enter(float smax, float c, f32x16 (&acc)[4], float& m,
                                                                  float& l) {
    const float mloc = smax * c;
    const bool grow = mloc > m + kRescaleSlack;
    if (__ballot(grow)) {
        const float mnew = grow ? mloc : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][i] *= alpha;
        l *= alpha;
        m = mnew;
    }
    return m == -INFINITY ? 0.0f : -m;
}

// The same for scores that arrive in base-2 units already shifted by the reference r
// (r = m, or 0 before any key): smax and the scores s of the block are relative to r.
// Moving the reference shifts s and the C tiles ct (which carry -r) with it.
__device__ __attribute__((always_inline)) inline void pair_enter_shifted(float smax, f32x16 (&acc)[4],
                                                                         f32x16 (&s)[2], f32x16 (&ct)[2], float& m,
                                                                         float& l) {
    const bool grow = smax > (m == -INFINITY ? -INFINITY : kRescaleSlack);
    if (__ballot(grow)) {
        const float r = m == -INFINITY ? 0.0f : m;
        const float mnew = r + smax;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;   // 0 when m = -inf
        const float d = grow ? smax : 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][i] *= alpha;
        l *= alpha;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[kt][i] -= d;
                ct[kt][i] -= d;
            }
        if (grow) m = mnew;
    }
}

template <bool FP8, bool SHIFT, bool CNT>
__global__ __launch_bounds__(kPairThreads, 2) void k_sparse_attn_pair(
    const void* __restrict__ qv, const void* __restrict__ kv, const __bf16* __restrict__ vt,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, Geom g, long P, float scale_log2,
    __bf16* __restrict__ o, float* __restrict__ lse, float* __restrict__ o32, const int32_t* __restrict__ kcount) {
    constexpr int D = 128;
    constexpr int kKBytes = kBlock * D * (FP8 ? 1 : 2), kVBytes = kBlock * D * 2;
    constexpr int kKChunks = kKBytes / 1024 / 4;          // kilobytes per wave per tile
    constexpr int kVChunks = kVBytes / 1024 / 4;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (kKBytes + kVBytes)];
    __shared__ uint32_t bits[2][kMaxBitmapWords];
    __shared__ __attribute__((aligned(16))) float bias_table[kBiasCodes * 2 * 2 * 16];
    // e4m3: the key tile scales of this (batch, head), staged once; a scale read from
    // memory inside the loop would be a scalar load, which shares the LDS reads' wait
    // counter and returns out of order, so every operand wait would become a full drain
    __shared__ float ksc_lds[FP8 ? kMaxBitmapWords * 32 : 1];
    // counted blocks: each key block's code (64 - real keys), staged once for the same reason
    __shared__ uint8_t kcode_lds[CNT ? kMaxBitmapWords * 32 : 1];
    static_assert(!(FP8 && CNT), "counted blocks are bf16");
    uint8_t* const kring = lds;
    uint8_t* const vring = lds + 2 * kKBytes;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qsel = w >> 1, qh = w & 1;
    const int half = lane >> 5;
    const long p = xcd_row(P);
    const int ph = (g.nb + 1) >> 1;
    const long bh = p / ph;
    const int v0 = 2 * (int)(p - bh * ph);
    const bool hasrow = v0 + qsel < g.nb;                 // uniform per wave
    const long r = strip_row(bh * g.nb + (hasrow ? v0 + qsel : v0), g);
    const int qb = (int)(r - bh * g.nb);
    const long npad = (long)g.nb * kBlock;
    const long qblk0 = bh * npad + (long)qb * kBlock;

    KHalf<D, FP8> q;
    if (hasrow) {
        load_khalf<D, FP8>(q, qv, qblk0, qh, lane);
    } else if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) q.f[j][e] = 0;
    } else {
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) q.b[j][e] = (__bf16)0.0f;
    }
    // base-2 softmax scale, times this query block's e4m3 tile scale; a block's own
    // key tile scale multiplies it per block
    const float cq = FP8 ? scale_log2 * (hasrow ? q_scale[r] : 1.0f) : scale_log2;
    const float* ksc_row = FP8 ? k_scale + bh * g.nb : nullptr;
    // SHIFT (bf16 only): the base-2 softmax scale goes into the query operand (one more
    // rounding to bf16, at most 2^-8 relative per element), so that the products give
    // base-2 scores and the exponentials need no scale-and-shift step
    static_assert(!(FP8 && SHIFT), "e4m3 scores are scaled per key block");
    if constexpr (SHIFT) {
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) q.b[j][e] = (__bf16)((float)q.b[j][e] * scale_log2);
    }

    // bias table: entry ((code * 2 + half) * 2 + kt) * 16 + i is 0 when key 32 kt + 8 (i / 4)
    // + 4 half + i % 4 of a block with edge code `code` is real, else -inf (code 8: none);
    // counted blocks: entry 16 v + i is 0 for i < v, else -inf
    if constexpr (CNT) {
        for (int x = threadIdx.x; x < 17 * 16; x += kPairThreads)
            bias_table[x] = (x & 15) < (x >> 4) ? 0.0f : -INFINITY;
        for (int i = threadIdx.x; i < g.nb; i += kPairThreads)
            kcode_lds[i] = (uint8_t)(kBlock - min(max(kcount[bh * g.nb + i], 0), kBlock));
    }
    for (int x = threadIdx.x; !CNT && x < kBiasCodes * 64; x += kPairThreads) {
        const int code = x >> 6, i = x & 15, kt = (x >> 4) & 1, hf = (x >> 5) & 1;
        const int key = 32 * kt + 8 * (i >> 2) + 4 * hf + (i & 3);
        const int plane = g.th * g.tw;
        const int et = key / plane, eh = (key - et * plane) / g.tw, ew = key - et * plane - eh * g.tw;
        const int ok = (et < g.T - (g.nt - 1) * g.tt ? 1 : 0) | (eh < g.Hg - (g.nh - 1) * g.th ? 2 : 0) |
                       (ew < g.Wg - (g.nw - 1) * g.tw ? 4 : 0);
        const bool real = code < 8 && ((ok | ~code) & 7) == 7;
        bias_table[((code * 2 + hf) * 2 + kt) * 16 + i] = real ? 0.0f : -INFINITY;
    }
    // membership bitmaps of the two kept lists
    const int nwords = (g.nb + 63) >> 6;
    for (int i = threadIdx.x; i < 2 * kMaxBitmapWords; i += kPairThreads) (&bits[0][0])[i] = 0u;
    if constexpr (FP8)
        for (int i = threadIdx.x; i < g.nb; i += kPairThreads) ksc_lds[i] = ksc_row[i];
    __syncthreads();
    if (hasrow) {
        const int e0 = row_ptr[r], e1 = row_ptr[r + 1];
        for (int e = e0 + 64 * qh + lane; e < e1; e += 128) {
            const int x = col_idx[e];
            if ((unsigned)x < (unsigned)g.nb) atomicOr(&bits[qsel][x >> 5], 1u << (x & 31));
        }
    }
    __syncthreads();
    // number of union entries: lane l counts word l of the two bitmaps
    int n_union;
    {
        int cnt = 0;
        if (lane < 2 * nwords) cnt = __builtin_popcount(bits[0][lane] | bits[1][lane]);
        if (lane + 64 < 2 * nwords) cnt += __builtin_popcount(bits[0][lane + 64] | bits[1][lane + 64]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
        n_union = __builtin_amdgcn_readfirstlane(cnt);
    }

    // Union entries in ascending order: the index word (block | edge code << kEdgeShift)
    // and whether this wave's query block keeps it; -1 past the end. The bitmap words
    // are read once per 64 blocks.
    int gw = -1, winfo = -1;
    uint64_t rem = 0, own = 0;
    auto word = [&](int sel, int i) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane(bits[sel][2 * i]);
        const uint32_t hi = __builtin_amdgcn_readfirstlane(bits[sel][2 * i + 1]);
        return ((uint64_t)hi << 32) | lo;
    };
    auto gen = [&](int& info, bool& mine) {
        while (rem == 0) {
            if (gw + 1 >= nwords) {
                info = -1;
                mine = false;
                return;
            }
            ++gw;
            const uint64_t a = word(0, gw), b = word(1, gw);
            rem = a | b;
            own = qsel ? b : a;
            const int kb = 64 * gw + lane;
            if constexpr (CNT) winfo = kb < g.nb ? kb | ((int)kcode_lds[kb] << kEdgeShift) : -1;
            else winfo = block_info(g, kb);
        }
        const int bit = __builtin_ctzll(rem);
        rem &= rem - 1;
        info = __builtin_amdgcn_readlane(winfo, bit);
        mine = (own >> bit) & 1ull;
    };
    auto block_of = [](int info) { return info < 0 ? 0 : (info & kBlockIdMask); };
    // the code of a block the wave does not keep: every key masked
    constexpr int kNone = CNT ? kBlock : kBiasCodes - 1;
    auto bias_code = [](int info, bool mine) { return (info < 0 || !mine) ? kNone : (info >> kEdgeShift); };

    const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(kv) + bh * npad * D * (FP8 ? 1 : 2);
    const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(vt) + bh * npad * D * 2;
    const i32x4r krs = tile_rsrc_raw(kbytes, (uint32_t)(g.nb * kKBytes));
    const i32x4r vrs = tile_rsrc_raw(vbytes, (uint32_t)(g.nb * kVBytes));
    const int lane16 = 16 * lane;
    // kilobyte c of a tile in LDS: for V and bf16 K the same kilobyte of the tile (lane
    // l: bytes 16 l); for e4m3 K, half c % 2 of the 2 KB operand step c / 2 (lane l: bytes
    // 32 l + 16 (c % 2)), the split layout the e4m3 operand reads expect
    auto copy_k = [&](int info, uint8_t* ring, int i) {
        const int c = kKChunks * w + i;
        const uint32_t src = FP8 ? (c >> 1) * 2048 + 16 * (c & 1) : c * 1024;
        copy_kb_asm(krs, (uint32_t)(block_of(info) * kKBytes) + src, ring + c * 1024, FP8 ? 32 * lane : lane16);
    };
    auto copy_v = [&](int info, uint8_t* ring, int i) {
        const int c = kVChunks * w + i;
        copy_kb_asm(vrs, (uint32_t)(block_of(info) * kVBytes + c * 1024), ring + c * 1024, lane16);
    };
    auto kscale = [&](int info) { return FP8 ? ksc_lds[block_of(info)] : 1.0f; };

    f32x16 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
    // m: the query's running reference (the same in both lane halves); l: this lane's share
    // of the row sum (its keys of each block), the two halves added once at the end
    float m = -INFINITY, l = 0.0f;
    // SHIFT: C tiles of the QK^T chains, the bias tile of edge code `ccode` plus -r, r
    // the reference the scores are shifted by (m once a key has been seen, 0 before).
    // Neighbouring union blocks mostly share their code (a run of block columns), so
    // the tiles are re-read from the table only when the code changes.
    f32x16 ct[2];
    int ccode = -1;

    int inf, infn;
    bool mine, minen;
    gen(inf, mine);
    gen(infn, minen);
    float ksc = kscale(inf), kscn = kscale(infn);
    float smax = -INFINITY;
    // iteration parity selects the ring slots: K(u+1) is read from slot (u+1)&1 while
    // K(u+2) is copied into slot u&1; V(u) from slot u&1 while V(u+1) goes to (u+1)&1
    auto step = [&](int par, f32x16 (&s)[2], f32x16 (&sn)[2]) {
        int inf2;
        bool mine2;
        gen(inf2, mine2);
        const float ksc2 = kscale(inf2);
        const float c = cq * ksc;
        float nref = 0.0f;
        if constexpr (SHIFT) pair_enter_shifted(smax, acc, s, ct, m, l);
        else nref = pair_enter(smax, c, acc, m, l);
        const int code1 = bias_code(infn, minen);
        if (SHIFT && code1 != ccode) {
            ccode = code1;
            load_bias<CNT>(ct, bias_table, code1, half);
            const float nr = m == -INFINITY ? 0.0f : -m;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) ct[kt][i] += nr;
        }
        copies_landed_barrier();                          // K(u+1), V(u) landed; slots of u-1 free
        const uint8_t* kst = kring + (par ^ 1) * kKBytes;
        const uint8_t* vst = vring + par * kVBytes;
        auto copy_one = [&](int i) {
            if (i < kKChunks) copy_k(inf2, kring + par * kKBytes, i);
            else copy_v(infn, vring + (par ^ 1) * kVBytes, i - kKChunks);
        };
        pair_main<FP8, SHIFT, CNT, kKChunks + kVChunks>(kst, vst, lane, half, q, acc, s, sn, ct, c, nref, l, smax, bias_table,
                                             bias_code(inf2, mine2), copy_one);
        inf = infn;
        mine = minen;
        infn = inf2;
        minen = mine2;
        ksc = kscn;
        kscn = ksc2;
    };

    f32x16 s0[2], s1[2];
    if (n_union > 0) {
#pragma unroll
        for (int i = 0; i < kKChunks; ++i) {
            copy_k(inf, kring, i);
            copy_k(infn, kring + kKBytes, i);
        }
#pragma unroll
        for (int i = 0; i < kVChunks; ++i) copy_v(inf, vring, i);
        copies_landed_barrier();                          // K(0), V(0), K(1) landed
        if constexpr (!SHIFT) {
            load_bias<CNT>(s0, bias_table, bias_code(inf, mine), half);
            load_bias<CNT>(s1, bias_table, bias_code(infn, minen), half);
        } else {
            ccode = bias_code(inf, mine);
            load_bias<CNT>(ct, bias_table, ccode, half);   // r = 0 so far
            s0[0] = ct[0];
            s0[1] = ct[1];
        }
        {
            KHalf<D, FP8> k0, k1;
            lds_khalf<D, FP8>(k0, kring, 0, lane);
            lds_khalf<D, FP8>(k1, kring, 1, lane);
            if constexpr (FP8) {
#pragma unroll
                for (int st = 0; st < D / 64; ++st) {
                    s0[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k0.f[st], q.f[st], s0[0], 0, 0, 0, 0, 0, 0);
                    s0[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k1.f[st], q.f[st], s0[1], 0, 0, 0, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int st = 0; st < D / 16; ++st) {
                    s0[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0.b[st], q.b[st], s0[0], 0, 0, 0);
                    s0[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1.b[st], q.b[st], s0[1], 0, 0, 0);
                }
            }
        }
        smax = wave_max32(fmaxf(max16_lane(s0[0]), max16_lane(s0[1])));
        for (int j = 0; j < n_union; j += 2) {
            step(0, s0, s1);
            if (j + 1 < n_union) step(1, s1, s0);
        }
    }
    wait_vmcnt<0>();                                      // drain the last copies
    l = wave_add32(l);                                    // the two lane halves of each query

    if (!hasrow) return;
    const int col = lane & 31;
    const int qslot = 32 * qh + col;
    const bool qvalid = g.valid(qb, qslot);
    const float inv = (qvalid && l > 0.0f) ? 1.0f / l : 0.0f;
    __bf16* orow = o + (qblk0 + qslot) * D;
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
#pragma unroll
    for (int t = 0; t < 4; ++t)
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
        for (int t = 0; t < 4; ++t)
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

void launch_sparse_attn(const void* q, const void* k, const void* v, int fp8, const float* q_scale,
                        const float* k_scale, const int32_t* row_ptr, const int32_t* col_idx,
                        int B, int H, int D, const Geom& g, float scale, void* o, float* lse, float* o32,
                        const int32_t* kcount, hipStream_t st) {
    const long R = (long)B * H * g.nb;
    const float sl2 = scale * kLog2e;
    const __bf16* vt = static_cast<const __bf16*>(v);
    __bf16* out = static_cast<__bf16*>(o);
    dim3 grid((unsigned)R), block(kAttnThreads);
    // Paired query blocks pay off when neighbouring query blocks keep nearly the same key
    // blocks, as measured selections on video grids do (the union adds 1.4 % at 480p), and
    // as the blocks of one query cluster do in a cluster-contiguous layout (counted keys:
    // they keep the same key clusters; 1.5 % at 480p with 128 clusters). On 2D grids the
    // workloads are group-structured masks, whose neighbouring groups share only their
    // row (or column) of groups, so a pair's union is about 1.5 times either list: those
    // take the one-block kernel.
    if (D == 128 && g.nb <= kMaxBitmapWords * 32 && (kcount != nullptr ? !fp8 : g.T > 1)) {
        const long P = (long)B * H * ((g.nb + 1) / 2);
        const unsigned n = (unsigned)P;
        // bf16 without lse (inference) pre-scales the queries; with lse, whose consumer
        // (the backward) recomputes exact scores against it, the scores are scaled in
        // float32
        if (fp8)
            k_sparse_attn_pair<true, false, false><<<n, kPairThreads, 0, st>>>(
                q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, P, sl2, out, lse, o32, nullptr);
        else if (kcount != nullptr && lse == nullptr)
            k_sparse_attn_pair<false, true, true><<<n, kPairThreads, 0, st>>>(
                q, k, vt, nullptr, nullptr, row_ptr, col_idx, g, P, sl2, out, lse, o32, kcount);
        else if (kcount != nullptr)
            k_sparse_attn_pair<false, false, true><<<n, kPairThreads, 0, st>>>(
                q, k, vt, nullptr, nullptr, row_ptr, col_idx, g, P, sl2, out, lse, o32, kcount);
        else if (lse == nullptr)
            k_sparse_attn_pair<false, true, false><<<n, kPairThreads, 0, st>>>(
                q, k, vt, nullptr, nullptr, row_ptr, col_idx, g, P, sl2, out, lse, o32, nullptr);
        else
            k_sparse_attn_pair<false, false, false><<<n, kPairThreads, 0, st>>>(
                q, k, vt, nullptr, nullptr, row_ptr, col_idx, g, P, sl2, out, lse, o32, nullptr);
        return;
    }
    if (D == 128) {
        // bf16 without lse (inference) takes pre-scaled queries, as in the paired kernel
        const bool shift = !fp8 && lse == nullptr;
        if (fp8)
            k_sparse_attn<128, true, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R,
                                                                    sl2, out, lse, o32, nullptr);
        else if (kcount && shift)
            k_sparse_attn<128, false, true, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx,
                                                                          g, R, sl2, out, lse, o32, kcount);
        else if (kcount)
            k_sparse_attn<128, false, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R,
                                                                    sl2, out, lse, o32, kcount);
        else if (shift)
            k_sparse_attn<128, false, false, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx,
                                                                           g, R, sl2, out, lse, o32, nullptr);
        else
            k_sparse_attn<128, false, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R,
                                                                     sl2, out, lse, o32, nullptr);
    } else {
        if (fp8)
            k_sparse_attn<64, true, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R,
                                                                   sl2, out, lse, o32, nullptr);
        else if (kcount)
            k_sparse_attn<64, false, true><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R,
                                                                   sl2, out, lse, o32, kcount);
        else
            k_sparse_attn<64, false, false><<<grid, block, 0, st>>>(q, k, vt, q_scale, k_scale, row_ptr, col_idx, g, R,
                                                                    sl2, out, lse, o32, nullptr);
    }
}

}  // namespace fpsa
