// Token permutation between raster order and 64-token tiles, with the FP8 e4m3
// per-tile quantization folded into the same pass (one tile = one sparsity block =
// one quantization group, [FPSAttention: Training-Aware FP8 and Sparsity Co-Design
// for Fast Video Diffusion, Abstract]).
//
// One workgroup per (block, head, batch) moves 64 x D values. Both sides are
// contiguous: a source token row is H*D elements with this head's D in the middle,
// a destination block is 64*D contiguous elements, so every access is a 16-byte
// vector load or store. HBM-bound by construction.
#include "fpsa_device.h"
#include "fpsa_internal.h"

namespace fpsa {

// Nearest-even OCP e4m3fn encoding of a finite float, saturating to +-448.
__device__ inline uint32_t encode_e4m3(float y) {
    uint32_t bits = __float_as_uint(y);
    uint32_t sign = (bits >> 24) & 0x80u;
    float a = fabsf(y);
    if (!(a == a)) return 0x7Fu;                        // NaN
    if (a > 448.0f) return sign | 0x7Eu;                // beyond the largest finite: saturate
    if (a < 0.015625f) {                                // below 2^-6: subnormal step 2^-9
        float q = rintf(a * 512.0f);                    // exact scaling; rint rounds to even
        return sign | (uint32_t)q;                      // q == 8 is code 0x08 = 2^-6
    }
    uint32_t ab = __float_as_uint(a);
    int e = (int)((ab >> 23) & 0xFF) - 127;             // -6 .. 8
    uint32_t man = ab & 0x7FFFFFu;
    uint32_t keep = man >> 20, rest = man & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep++;
    if (keep == 8u) { keep = 0; e++; }
    return sign | ((uint32_t)(e + 7) << 3) | keep;      // a <= 448 keeps this <= 0x7E
}

template <typename SrcT>
__device__ inline void load8(const SrcT* p, float* v);

template <>
__device__ inline void load8<__bf16>(const __bf16* p, float* v) {
    bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
}

template <>
__device__ inline void load8<float>(const float* p, float* v) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

// Output layouts (see include/fpsa.h): rows, QK operand order, VT operand order.
enum { kRows = 0, kVT = 1, kQK = 2 };

// Where output chunk `oc` (16 bytes) of a block comes from: slot and first channel,
// for a layout whose 16-byte chunks each hold consecutive channels of one slot.
template <int D, int ESIZE, int LAYOUT>
__device__ inline void chunk_source(int oc, int& e, int& d0) {
    constexpr int kPer = 16 / ESIZE;                     // elements per chunk
    if constexpr (LAYOUT == kRows) {
        e = oc / (D / kPer);
        d0 = (oc % (D / kPer)) * kPer;
    } else if constexpr (ESIZE == 2) {                   // QK, bf16: units of 8 channels
        int col = oc & 31, half = (oc >> 5) & 1, rest = oc >> 6;
        int st = rest % (D / 16), kt = rest / (D / 16);
        e = 32 * kt + col;
        d0 = 16 * st + 8 * half;
    } else {                                             // QK, e4m3: units of 32 channels, two chunks each
        int part = oc & 1, u = oc >> 1;
        int col = u & 31, half = (u >> 5) & 1, rest = u >> 6;
        int st = rest % (D / 64), kt = rest / (D / 64);
        e = 32 * kt + col;
        d0 = 64 * st + 32 * half + 16 * part;
    }
}

// Where the tokens of a block come from: the token grid (raster order, tiles in
// raster order), or an explicit per-(b, h) slot map (-1 for padding), as for the
// cluster-contiguous layout of the k-means permutation.
struct GridMap {
    Geom g;
    __device__ inline long token(long, int blk, int e) const { return g.token(blk, e); }
    __host__ __device__ inline int nb() const { return g.nb; }
};
struct SlotMap {
    const int32_t* slot_token;   // [B*H, nblocks*64]
    int nblocks;
    __device__ inline long token(long bh, int blk, int e) const {
        return slot_token[(bh * nblocks + blk) * kBlock + e];
    }
    __host__ __device__ inline int nb() const { return nblocks; }
};

// One workgroup per (block, head, batch). Phase 1 reads the block's 64 token rows
// in raster order (coalesced), converts (and for e4m3 computes the tile scale and
// encodes) into an LDS tile; phase 2 writes the block in the requested layout as
// contiguous 16-byte chunks.
template <typename SrcT, int D, bool FP8, int LAYOUT, class Map>
__global__ __launch_bounds__(256) void k_tile_forward(const SrcT* __restrict__ src,
                                                      void* __restrict__ dst,
                                                      float* __restrict__ scale_out, Map map,
                                                      long N, int H) {
    constexpr int kIn = kBlock * D / 8;                 // 8-element input chunks
    constexpr int kInPerThread = kIn / 256;
    constexpr int ESIZE = FP8 ? 1 : 2;
    constexpr int kRowBytes = D * ESIZE + 16;           // padded LDS row
    __shared__ __attribute__((aligned(16))) uint8_t tile[kBlock * kRowBytes];
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const long bh = (long)b * H + h;

    float v[kInPerThread][8];
#pragma unroll
    for (int i = 0; i < kInPerThread; ++i) {
        int c = tid + 256 * i;
        int e = c / (D / 8), d0 = (c % (D / 8)) * 8;
        long n = map.token(bh, blk, e);
        if (n >= 0) {
            load8<SrcT>(src + (((long)b * N + n) * H + h) * D + d0, v[i]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
        }
    }

    if constexpr (FP8) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kInPerThread; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        __shared__ float wmax[4];
        if ((tid & 63) == 0) wmax[tid >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        const float s = amax > 0.0f ? amax / 448.0f : 1.0f;   // IEEE division
        if (tid == 0) scale_out[bh * map.nb() + blk] = s;
#pragma unroll
        for (int i = 0; i < kInPerThread; ++i) {
            int c = tid + 256 * i;
            int e = c / (D / 8), d0 = (c % (D / 8)) * 8;
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo |= encode_e4m3(v[i][j] / s) << (8 * j);
                hi |= encode_e4m3(v[i][4 + j] / s) << (8 * j);
            }
            i32x2 w2;
            w2[0] = (int)lo;
            w2[1] = (int)hi;
            *reinterpret_cast<i32x2*>(tile + e * kRowBytes + d0) = w2;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kInPerThread; ++i) {
            int c = tid + 256 * i;
            int e = c / (D / 8), d0 = (c % (D / 8)) * 8;
            *reinterpret_cast<bf16x8*>(tile + e * kRowBytes + 2 * d0) =
                pack_bf16x8(v[i][0], v[i][1], v[i][2], v[i][3], v[i][4], v[i][5], v[i][6], v[i][7]);
        }
    }
    __syncthreads();

    constexpr int kOut = kBlock * D * ESIZE / 16;       // 16-byte output chunks
    uint8_t* out = reinterpret_cast<uint8_t*>(dst) + (bh * map.nb() + blk) * (long)(kBlock * D * ESIZE);
#pragma unroll
    for (int i = 0; i < kOut / 256; ++i) {
        int oc = tid + 256 * i;
        i32x4 val;
        if constexpr (LAYOUT == kVT) {
            // chunk = 8 positions of one channel: ((t*4 + cc)*2 + half)*32 + col
            int col = oc & 31, half = (oc >> 5) & 1, cc = (oc >> 6) & 3, t = oc >> 8;
            int d = 32 * t + col, p0 = 16 * cc + 8 * half;
            bf16x8 r;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                r[j] = *reinterpret_cast<const __bf16*>(tile + vt_slot_of_position(p0 + j) * kRowBytes + 2 * d);
            val = *reinterpret_cast<i32x4*>(&r);
        } else {
            int e, d0;
            chunk_source<D, ESIZE, LAYOUT>(oc, e, d0);
            val = *reinterpret_cast<const i32x4*>(tile + e * kRowBytes + d0 * ESIZE);
        }
        *reinterpret_cast<i32x4*>(out + (long)oc * 16) = val;
    }
}

template <typename DstT, int D, class Map>
__global__ __launch_bounds__(256) void k_tile_inverse(const __bf16* __restrict__ src,
                                                      DstT* __restrict__ dst, Map map, long N,
                                                      int H) {
    constexpr int kChunks = kBlock * D / 8;
    constexpr int kPerThread = kChunks / 256;
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const long bh = (long)b * H + h;
    const __bf16* in = src + (bh * map.nb() + blk) * (long)(kBlock * D);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        int c = threadIdx.x + 256 * i;
        int e = c / (D / 8), d0 = (c % (D / 8)) * 8;
        long n = map.token(bh, blk, e);
        if (n < 0) continue;
        bf16x8 x = *reinterpret_cast<const bf16x8*>(in + (long)c * 8);
        DstT* o = dst + (((long)b * N + n) * H + h) * D + d0;
        if constexpr (sizeof(DstT) == 2) {
            *reinterpret_cast<bf16x8*>(o) = x;
        } else {
            f32x4 a, bq;
#pragma unroll
            for (int j = 0; j < 4; ++j) { a[j] = (float)x[j]; bq[j] = (float)x[4 + j]; }
            *reinterpret_cast<f32x4*>(o) = a;
            *reinterpret_cast<f32x4*>(o + 4) = bq;
        }
    }
}

template <typename SrcT, int D, class Map>
static void launch_forward_t(const SrcT* s, void* dst, bool fp8, int layout, float* scale,
                             const Map& map, long N, int B, int H, hipStream_t st) {
    dim3 grid(map.nb(), H, B);
    if (fp8) {
        if (layout == kQK) k_tile_forward<SrcT, D, true, kQK, Map><<<grid, 256, 0, st>>>(s, dst, scale, map, N, H);
        else k_tile_forward<SrcT, D, true, kRows, Map><<<grid, 256, 0, st>>>(s, dst, scale, map, N, H);
    } else {
        if (layout == kQK) k_tile_forward<SrcT, D, false, kQK, Map><<<grid, 256, 0, st>>>(s, dst, scale, map, N, H);
        else if (layout == kVT) k_tile_forward<SrcT, D, false, kVT, Map><<<grid, 256, 0, st>>>(s, dst, scale, map, N, H);
        else k_tile_forward<SrcT, D, false, kRows, Map><<<grid, 256, 0, st>>>(s, dst, scale, map, N, H);
    }
}

template <class Map>
static void launch_forward_map(const void* src, int src_dt, void* dst, int fp8, int layout, float* scale,
                               const Map& map, long N, int B, int H, int D, hipStream_t st) {
    if (src_dt == 0) {
        const float* s = static_cast<const float*>(src);
        if (D == 128) launch_forward_t<float, 128>(s, dst, fp8, layout, scale, map, N, B, H, st);
        else launch_forward_t<float, 64>(s, dst, fp8, layout, scale, map, N, B, H, st);
    } else {
        const __bf16* s = static_cast<const __bf16*>(src);
        if (D == 128) launch_forward_t<__bf16, 128>(s, dst, fp8, layout, scale, map, N, B, H, st);
        else launch_forward_t<__bf16, 64>(s, dst, fp8, layout, scale, map, N, B, H, st);
    }
}

template <class Map>
static void launch_inverse_map(const void* src, void* dst, int dst_dt, const Map& map, long N, int B,
                               int H, int D, hipStream_t st) {
    dim3 grid(map.nb(), H, B);
    const __bf16* s = static_cast<const __bf16*>(src);
    if (D == 128) {
        if (dst_dt == 0) k_tile_inverse<float, 128, Map><<<grid, 256, 0, st>>>(s, (float*)dst, map, N, H);
        else k_tile_inverse<__bf16, 128, Map><<<grid, 256, 0, st>>>(s, (__bf16*)dst, map, N, H);
    } else {
        if (dst_dt == 0) k_tile_inverse<float, 64, Map><<<grid, 256, 0, st>>>(s, (float*)dst, map, N, H);
        else k_tile_inverse<__bf16, 64, Map><<<grid, 256, 0, st>>>(s, (__bf16*)dst, map, N, H);
    }
}

// Value of an OCP e4m3fn code (finite codes only; the encoder above never writes the
// NaN codes): sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormal step 2^-9.
__device__ inline float decode_e4m3(uint32_t c) {
    const uint32_t ex = (c >> 3) & 0xFu, man = c & 7u;
    const float mag = ex == 0 ? ldexpf((float)man, -9) : ldexpf((float)(8u + man), (int)ex - 10);
    return (c & 0x80u) ? -mag : mag;
}

// Dequantized Q or K tiles: the e4m3 QK tile of a block times its scale, rounded to
// bf16 (the float32 product, then nearest-even), or without a scale the code values
// themselves (exact in bf16), written in the bf16 QK layout. Each
// thread converts 16-byte chunks of 16 consecutive channels of one slot (two bf16
// chunks out).
template <int D>
__global__ __launch_bounds__(256) void k_dequant_tiles(const uint8_t* __restrict__ src,
                                                       const float* __restrict__ scale,
                                                       __bf16* __restrict__ dst) {
    const long blk = blockIdx.x;                         // (b*H + h)*nb + block
    const float s = scale != nullptr ? scale[blk] : 1.0f;
    const uint8_t* in = src + blk * 64 * D;
    uint8_t* out = reinterpret_cast<uint8_t*>(dst + blk * 64 * D);
    for (int oc = threadIdx.x; oc < 64 * D / 16; oc += 256) {
        int e, d0;
        chunk_source<D, 1, kQK>(oc, e, d0);
        const i32x4 codes = *reinterpret_cast<const i32x4*>(in + 16 * oc);
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            bf16x8 o;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t c = ((uint32_t)codes[(8 * h8 + j) >> 2] >> (8 * ((8 * h8 + j) & 3))) & 0xFFu;
                o[j] = (__bf16)(decode_e4m3(c) * s);
            }
            const int d = d0 + 8 * h8;
            const int off = ((((e >> 5) * (D / 16) + (d >> 4)) * 2 + ((d >> 3) & 1)) * 32 + (e & 31)) * 8 + (d & 7);
            *reinterpret_cast<bf16x8*>(out + 2 * off) = o;
        }
    }
}

void launch_dequant_tiles(const void* src, const float* scale, void* dst, long blocks, int D, hipStream_t st) {
    const uint8_t* s = static_cast<const uint8_t*>(src);
    __bf16* d = static_cast<__bf16*>(dst);
    if (D == 128) k_dequant_tiles<128><<<(unsigned)blocks, 256, 0, st>>>(s, scale, d);
    else k_dequant_tiles<64><<<(unsigned)blocks, 256, 0, st>>>(s, scale, d);
}

void launch_tile_forward(const void* src, int src_dt, void* dst, int fp8, int layout, float* scale,
                         const Geom& g, long N, int B, int H, int D, hipStream_t st) {
    launch_forward_map(src, src_dt, dst, fp8, layout, scale, GridMap{g}, N, B, H, D, st);
}

void launch_tile_inverse(const void* src, void* dst, int dst_dt, const Geom& g, long N, int B,
                         int H, int D, hipStream_t st) {
    launch_inverse_map(src, dst, dst_dt, GridMap{g}, N, B, H, D, st);
}

void launch_gather_tiles(const void* src, int src_dt, const int32_t* slot_token, int nblocks, void* dst,
                         int layout, long N, int B, int H, int D, hipStream_t st) {
    launch_forward_map(src, src_dt, dst, 0, layout, nullptr, SlotMap{slot_token, nblocks}, N, B, H, D, st);
}

void launch_scatter_tiles(const void* src, const int32_t* slot_token, int nblocks, void* dst, int dst_dt,
                          long N, int B, int H, int D, hipStream_t st) {
    launch_inverse_map(src, dst, dst_dt, SlotMap{slot_token, nblocks}, N, B, H, D, st);
}

}  // namespace fpsa
