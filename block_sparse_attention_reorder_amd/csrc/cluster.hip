// Semantic-aware permutation: tokens of each (batch, head) are clustered by k-means
// over their own query (or key) vectors and laid out cluster by cluster, so that the
// tokens a query cluster needs sit in a few dense 64-token blocks; clusters are
// represented by their centroids and sizes to estimate which key clusters matter
// [Sparse VideoGen2: Accelerate Video Generation with Sparse Attention via
// Semantic-Aware Permutation, Abstract].
//
// k-means is Lloyd's algorithm in float64 with a fixed order of every operation: a
// token goes to the centroid of least e = |c|^2 - 2 x.c (the squared distance less
// |x|^2, common to every candidate), each of |c|^2 and x.c a chain of fused
// multiply-adds over the channels in order; ties to the lower cluster; member sums in
// eight interleaved partials combined pairwise. This file is compiled with
// contraction off, so every fused operation is an explicit one. The assignment is
// therefore the same on every device and run.
//
// Kernels: k_km_init (strided starting centroids), k_km_assign (nearest centroid as
// float64 matrix products; cluster sizes per 256-token chunk), k_km_chunk_scan +
// k_km_scatter (member lists in token order from the chunk counts), k_km_update
// (centroid = member mean), k_cluster_layout (slot map of the cluster-contiguous blocks), k_cluster_mass
// (centroid-based cluster masses), k_cblk_count / k_cblk_fill (block CSR of a cluster
// selection).
#include "fpsa_device.h"
#include "fpsa_internal.h"

namespace fpsa {

template <typename T>
__device__ inline float as_float(T x) { return (float)x; }

// ---------------------------------------------------------------- k-means

template <typename T>
__global__ __launch_bounds__(128) void k_km_init(const T* __restrict__ x, int N, int H, int D, int C,
                                                 double* __restrict__ cent) {
    const long bh = blockIdx.y;
    const int c = blockIdx.x, d = threadIdx.x;
    if (d >= D) return;
    const long b = bh / H, h = bh % H;
    const long t = (long)c * N / C;
    cent[(bh * C + c) * D + d] = (double)as_float(x[((b * N + t) * H + h) * D + d]);
}

// Assignment as float64 matrix products. v_mfma_f64_16x16x4 forms each output as a
// chain of four fused multiply-adds in k order on top of the accumulator, so a run of
// them over channel groups 0..3, 4..7, ... is exactly the channel-order fused chain of
// x.c. Tokens are the A rows (a wave holds two 16-token tiles as loaded and converts
// each operand when it is used), centroids the B columns (16-centroid tiles staged
// through LDS in operand order, double-buffered). Each lane keeps the first minimum of
// e over its centroid column across the tiles, and the 16 columns then merge on
// (e, cluster): the least e, ties to the lower cluster.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kKmWaves = 8;                     // waves x 32 tokens per workgroup
constexpr int kKmTokens = kKmWaves * 32;

// operand A of a 16-token tile, kept as loaded: lane l holds channels 4s + l/16 of its
// token, s = 0 .. D/4-1, two bf16 channels (steps 2q and 2q+1) per word, or one float
template <typename T, int D> struct TileA;
template <int D> struct TileA<__bf16, D> {
    uint32_t w[D / 8];
    __device__ void load(const __bf16* row, int k) {
#pragma unroll
        for (int q = 0; q < D / 8; ++q) {       // channels 8q .. 8q+7
            const uint4 u = reinterpret_cast<const uint4*>(row)[q];
            const uint32_t w0 = (k >> 1) ? u.y : u.x, w1 = (k >> 1) ? u.w : u.z;
            const uint32_t lo = (k & 1) ? (w0 >> 16) : (w0 & 0xffffu);   // channel 8q + k
            const uint32_t hi = (k & 1) ? (w1 & 0xffff0000u) : (w1 << 16); // channel 8q + 4 + k
            w[q] = lo | hi;
        }
    }
    __device__ double get(int s) const {
        return (double)__uint_as_float((s & 1) ? (w[s >> 1] & 0xffff0000u) : (w[s >> 1] << 16));
    }
    __device__ void keep() {                    // converted per use: no float64 copy held across tiles
#pragma unroll
        for (int q = 0; q < D / 8; ++q) asm volatile("" : "+v"(w[q]));
    }
};
template <int D> struct TileA<float, D> {
    float w[D / 4];
    __device__ void load(const float* row, int k) {
#pragma unroll
        for (int q = 0; q < D / 4; ++q) {       // channels 4q .. 4q+3
            const float4 u = reinterpret_cast<const float4*>(row)[q];
            const float lo = (k & 1) ? u.y : u.x, hi = (k & 1) ? u.w : u.z;
            w[q] = (k >> 1) ? hi : lo;
        }
    }
    __device__ double get(int s) const { return (double)w[s]; }
    __device__ void keep() {
#pragma unroll
        for (int q = 0; q < D / 4; ++q) asm volatile("" : "+v"(w[q]));
    }
};

template <typename T, int D>
__global__ __launch_bounds__(kKmWaves * 64) void k_km_assign(const T* __restrict__ x, int N, int H, int C,
                                                           const double* __restrict__ cent,
                                                           int32_t* __restrict__ assign,
                                                           int32_t* __restrict__ chunk_count) {
    constexpr int kSteps = D / 4;               // products per tile pair
    constexpr int kTile = kSteps * 64;          // doubles per staged centroid tile
    constexpr int kPer = 16 * D / (kKmWaves * 64);   // staged doubles per thread
    extern __shared__ double km_lds[];          // two staged tiles, then C squared norms
    double* tiles = km_lds;
    double* cnorm = km_lds + 2 * kTile;
    const long bh = blockIdx.y;
    const long b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const double* cb = cent + bh * (long)C * D;
    const int ntile = (C + 15) / 16;

    // staging: element e = tid + 512 r of tile t is centroid 16t + e / D, channel e % D,
    // stored at operand position (channel / 4) * 64 + (e / D) + 16 (channel % 4)
    double stage[kPer];
    auto fetch = [&](int t) {
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int e = tid + kKmWaves * 64 * r;
            const int c = 16 * t + e / D;
            stage[r] = c < C ? cb[(long)c * D + (e % D)] : 0.0;
        }
    };
    auto put = [&](int t) {
        double* dst = tiles + (t & 1) * kTile;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int e = tid + kKmWaves * 64 * r;
            const int jj = e / D, d = e % D;
            dst[(d >> 2) * 64 + jj + 16 * (d & 3)] = stage[r];
        }
    };
    fetch(0);
    for (int c = tid; c < C; c += kKmWaves * 64) {  // |c|^2: one sequential fused chain per centroid
        const double* p = cb + (long)c * D;
        double s = 0.0;
        for (int d = 0; d < D; ++d) s = __builtin_fma(p[d], p[d], s);
        cnorm[c] = s;
    }
    // the wave's two token tiles
    const long tok0 = (long)blockIdx.x * kKmTokens + wave * 32;
    TileA<T, D> a0, a1;
    {
        const long t0 = min(tok0 + (lane & 15), (long)N - 1), t1 = min(tok0 + 16 + (lane & 15), (long)N - 1);
        a0.load(x + ((b * N + t0) * H + h) * D, lane >> 4);   // past N: a real row, result unused
        a1.load(x + ((b * N + t1) * H + h) * D, lane >> 4);
    }
    put(0);
    __syncthreads();

    double bd0[4], bd1[4];
    int bi0[4], bi1[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) bi0[v] = bi1[v] = -1, bd0[v] = bd1[v] = 0.0;
    for (int t = 0; t < ntile; ++t) {
        if (t + 1 < ntile) fetch(t + 1);
        const double* bt = tiles + (t & 1) * kTile;
        a0.keep();
        a1.keep();
        f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const double bv = bt[s * 64 + lane];
            acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0.get(s), bv, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1.get(s), bv, acc1, 0, 0, 0);
        }
        const int j = 16 * t + (lane & 15);     // this lane's centroid; rows l/16 + 4v
        if (j < C) {
            const double cn = cnorm[j];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const double e0 = cn - 2.0 * acc0[v], e1 = cn - 2.0 * acc1[v];
                if (bi0[v] < 0 || e0 < bd0[v]) bd0[v] = e0, bi0[v] = j;
                if (bi1[v] < 0 || e1 < bd1[v]) bd1[v] = e1, bi1[v] = j;
            }
        }
        if (t + 1 < ntile) put(t + 1);
        __syncthreads();
    }
    // merge the 16 centroid columns of each row on (e, cluster)
    auto merge = [&](double& bd, int& bi) {
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
            const double od = __shfl_xor(bd, m);
            const int oi = __shfl_xor(bi, m);
            if (oi >= 0 && (bi < 0 || od < bd || (od == bd && oi < bi))) bd = od, bi = oi;
        }
    };
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        merge(bd0[v], bi0[v]);
        merge(bd1[v], bi1[v]);
    }
    // lane (g, u): u < 4 writes row g + 4u of tile 0, 4 <= u < 8 row g + 4(u-4) of tile 1;
    // the workgroup's cluster sizes (its 256 tokens are one chunk of the member
    // scatter) are counted in LDS, where the staged tiles were
    int* hist = reinterpret_cast<int*>(tiles);
    for (int c = tid; c < C; c += kKmWaves * 64) hist[c] = 0;
    __syncthreads();
    const int u = lane & 15, g = lane >> 4;
    if (u < 8) {
        const int v = u & 3;
        int bi = bi0[0];
#pragma unroll
        for (int w = 0; w < 4; ++w)
            if (v == w) bi = u < 4 ? bi0[w] : bi1[w];
        const long n = tok0 + (u < 4 ? 0 : 16) + g + 4 * v;
        if (n < N) {
            assign[bh * N + n] = bi;
            atomicAdd(&hist[bi], 1);
        }
    }
    __syncthreads();
    int32_t* row = chunk_count + (bh * C) * (long)gridDim.x + blockIdx.x;   // [bh][c][chunk]
    for (int c = tid; c < C; c += kKmWaves * 64) row[(long)c * gridDim.x] = hist[c];
}

// Per (slice, cluster): the chunk counts [bh][c][chunk] become exclusive prefix sums over
// the chunks (a wave per row), and the total is the cluster's size.
__global__ __launch_bounds__(256) void k_km_chunk_scan(int32_t* __restrict__ chunk_count, int nchunk, long rows,
                                                       int32_t* __restrict__ count) {
    const int lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    int32_t* p = chunk_count + r * nchunk;
    int base = 0;
    for (int k0 = 0; k0 < nchunk; k0 += 64) {
        const int k = k0 + lane;
        const int v = k < nchunk ? p[k] : 0;
        int s = v;                              // inclusive prefix over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(s, o);
            if (lane >= o) s += t;
        }
        if (k < nchunk) p[k] = base + s - v;
        base += __shfl(s, 63);
    }
    if (lane == 0) count[r] = base;
}

// Members in token order: token n of chunk k (the assignment's workgroups) goes to
// member_off[bh*C + c] + (members of c in chunks before k) + (members of c before n in
// chunk k).
__global__ __launch_bounds__(kKmTokens) void k_km_scatter(const int32_t* __restrict__ assign, int N, int C,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ off,
                                                          int32_t* __restrict__ members) {
    __shared__ int cl[kKmTokens];
    const long bh = blockIdx.y;
    const int t = threadIdx.x;
    const long n = (long)blockIdx.x * kKmTokens + t;
    const int c = n < N ? assign[bh * N + n] : -1;
    cl[t] = c;
    __syncthreads();
    if (c < 0) return;
    int rank = 0;
    for (int s = 0; s < t; ++s) rank += cl[s] == c;
    members[off[bh * C + c] + chunk_base[(bh * C + c) * (long)gridDim.x + blockIdx.x] + rank] = (int32_t)n;
}

// Centroid = member mean. The r-th member of a cluster (token order) goes to partial
// sum r % 8; thread (p, j) adds its partial's members in order for channels 2j and
// 2j + 1 of a 64-channel slice, and the eight partials combine as ((p0 + p1) + (p2 +
// p3)) + ((p4 + p5) + (p6 + p7)). Eight independent chains per channel instead of one.
// Members are taken in stages of 256: the stage's member indices sit in LDS (loaded
// one stage ahead, one per thread), and each thread has its 32 values of the stage in
// flight at once, so a large cluster costs one memory round trip per 256 members.
constexpr int kKmParts = 8;
constexpr int kKmSlice = 64;                    // channels per workgroup
constexpr int kKmThreads = kKmParts * kKmSlice / 2;
constexpr int kKmStage = kKmThreads;            // members per stage
constexpr int kKmPer = kKmStage / kKmParts;     // values per thread per stage

__device__ inline uint32_t two_raw(const __bf16* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ inline float2 two_raw(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ inline void two_channels(uint32_t w, float& a, float& b) {
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xffff0000u);
}
__device__ inline void two_channels(float2 w, float& a, float& b) {
    a = w.x;
    b = w.y;
}

template <typename T, int D>
__global__ __launch_bounds__(kKmThreads) void k_km_update(const T* __restrict__ x, int N, int H, int C,
                                                         const int32_t* __restrict__ off,
                                                         const int32_t* __restrict__ members,
                                                         double* __restrict__ cent) {
    __shared__ double part[kKmParts][kKmSlice];
    __shared__ int32_t sidx[2][kKmStage];
    const long bh = blockIdx.z;
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    const int p = tid / (kKmSlice / 2), j = tid % (kKmSlice / 2);
    const int d = blockIdx.y * kKmSlice + 2 * j;  // this thread's first channel
    const long b = bh / H, h = bh % H;
    const int r0 = off[bh * C + c], r1 = off[bh * C + c + 1];
    if (r1 == r0) return;                        // an empty cluster keeps its centroid (uniform)
    const T* xb = x + (b * N * H + h) * (long)D + d;   // token t at xb + t * H * D
    double s0 = 0.0, s1 = 0.0;
    int nxt = r0 + tid < r1 ? members[r0 + tid] : 0;
    for (int base = r0, st = 0; base < r1; base += kKmStage, st ^= 1) {
        sidx[st][tid] = nxt;
        __syncthreads();                         // indices of this stage visible; the other buffer free
        const int cnt = min(kKmStage, r1 - base);
        decltype(two_raw(xb)) raw[kKmPer];
#pragma unroll
        for (int i = 0; i < kKmPer; ++i) {
            const int q = p + kKmParts * i;      // member base + q of partial p
            raw[i] = two_raw(xb + (long)sidx[st][q < cnt ? q : 0] * H * D);
        }
        nxt = base + kKmStage + tid < r1 ? members[base + kKmStage + tid] : 0;
#pragma unroll
        for (int i = 0; i < kKmPer; ++i)
            if (p + kKmParts * i < cnt) {
                float va, vb;
                two_channels(raw[i], va, vb);
                s0 = s0 + (double)va;
                s1 = s1 + (double)vb;
            }
    }
    part[p][2 * j] = s0;
    part[p][2 * j + 1] = s1;
    __syncthreads();
    if (tid < kKmSlice) {
        const int dd = tid;
        const double s01 = part[0][dd] + part[1][dd], s23 = part[2][dd] + part[3][dd];
        const double s45 = part[4][dd] + part[5][dd], s67 = part[6][dd] + part[7][dd];
        cent[(bh * C + c) * D + blockIdx.y * kKmSlice + dd] = ((s01 + s23) + (s45 + s67)) / (double)(r1 - r0);
    }
}

size_t kmeans_workspace_bytes(int B, int H, int N, int C) {
    return (size_t)B * H * C * ((N + kKmTokens - 1) / kKmTokens) * sizeof(int32_t);
}

template <typename T>
static void kmeans_t(const T* x, int B, int N, int H, int D, int C, int iters, int32_t* assign, double* cent,
                     int32_t* count, int32_t* off, int32_t* members, int32_t* chunk, hipStream_t st) {
    const long rows = (long)B * H * C;
    dim3 gc(C, B * H);
    k_km_init<T><<<gc, 128, 0, st>>>(x, N, H, D, C, cent);
    const int nchunk = (N + kKmTokens - 1) / kKmTokens;
    dim3 ga(nchunk, B * H);
    const unsigned wb = (unsigned)((rows + 3) / 4);
    dim3 gu(C, D / kKmSlice, B * H);
    for (int it = 0; it < iters; ++it) {
        if (D == 128)
            k_km_assign<T, 128><<<ga, kKmWaves * 64, (size_t)(2 * 32 * 64 + C) * 8, st>>>(x, N, H, C, cent, assign,
                                                                                          chunk);
        else
            k_km_assign<T, 64><<<ga, kKmWaves * 64, (size_t)(2 * 16 * 64 + C) * 8, st>>>(x, N, H, C, cent, assign,
                                                                                         chunk);
        k_km_chunk_scan<<<wb, 256, 0, st>>>(chunk, nchunk, rows, count);
        launch_scan(count, rows, off, st);
        k_km_scatter<<<ga, kKmTokens, 0, st>>>(assign, N, C, chunk, off, members);
        if (D == 128) k_km_update<T, 128><<<gu, kKmThreads, 0, st>>>(x, N, H, C, off, members, cent);
        else k_km_update<T, 64><<<gu, kKmThreads, 0, st>>>(x, N, H, C, off, members, cent);
    }
}

void launch_kmeans(const void* x, int x_f32, int B, int N, int H, int D, int C, int iters, int32_t* assign,
                   double* cent, int32_t* count, int32_t* off, int32_t* members, void* ws, hipStream_t st) {
    int32_t* chunk = static_cast<int32_t*>(ws);
    if (x_f32)
        kmeans_t(static_cast<const float*>(x), B, N, H, D, C, iters, assign, cent, count, off, members, chunk, st);
    else
        kmeans_t(static_cast<const __bf16*>(x), B, N, H, D, C, iters, assign, cent, count, off, members, chunk, st);
}

// ---------------------------------------------------------------- layout

// One workgroup per slice: block offsets of the clusters (ceil(count / 64) blocks
// each), then every slot of the slice's nblocks blocks.
__global__ __launch_bounds__(1024) void k_cluster_layout(const int32_t* __restrict__ off,
                                                         const int32_t* __restrict__ members, int C,
                                                         int nblocks, int32_t* __restrict__ slot_token,
                                                         int32_t* __restrict__ blk_off,
                                                         int32_t* __restrict__ blk_count) {
    extern __shared__ int32_t bo[];             // C + 1 block offsets
    const long bh = blockIdx.x;
    const int32_t* o = off + bh * C;
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int c = 0; c < C; ++c) {
            bo[c] = acc;
            acc += (o[c + 1] - o[c] + 63) / 64;
        }
        bo[C] = acc;
    }
    __syncthreads();
    for (int c = threadIdx.x; c <= C; c += blockDim.x) blk_off[bh * (C + 1) + c] = bo[c];
    auto cluster_of = [&](int blk) {            // largest c with bo[c] <= blk (blk < bo[C])
        int lo = 0, hi = C - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (bo[mid] <= blk) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    for (int blk = threadIdx.x; blk < nblocks; blk += blockDim.x) {
        int cnt = 0;
        if (blk < bo[C]) {
            const int c = cluster_of(blk);
            cnt = min(64, (o[c + 1] - o[c]) - 64 * (blk - bo[c]));
        }
        blk_count[bh * nblocks + blk] = cnt;
    }
    const long slots = (long)nblocks * 64;
    for (long sl = threadIdx.x; sl < slots; sl += blockDim.x) {
        const int blk = (int)(sl >> 6);
        int tok = -1;
        if (blk < bo[C]) {
            const int c = cluster_of(blk);
            const long rr = sl - 64L * bo[c];
            if (rr < o[c + 1] - o[c]) tok = members[o[c] + rr];
        }
        slot_token[bh * slots + sl] = tok;
    }
}

void launch_cluster_layout(const int32_t* off, const int32_t* members, int B, int H, int C, int nblocks,
                           int32_t* slot_token, int32_t* blk_off, int32_t* blk_count, hipStream_t st) {
    k_cluster_layout<<<B * H, 1024, (size_t)(C + 1) * 4, st>>>(off, members, C, nblocks, slot_token, blk_off,
                                                               blk_count);
}

// ---------------------------------------------------------------- cluster masses

// One workgroup per (slice, query cluster); a thread per key cluster forms the
// centroid dot product in channel order; the row is normalised with a block max and
// sum.
__global__ __launch_bounds__(256) void k_cluster_mass(const double* __restrict__ cq, const int32_t* __restrict__ nq,
                                                      const double* __restrict__ ck, const int32_t* __restrict__ nk,
                                                      int Cq, int Ck, int D, double scale,
                                                      float* __restrict__ est) {
    extern __shared__ double sh[];              // D query-centroid values, then Ck weights
    double* qc = sh;
    double* wj = sh + D;
    __shared__ double red[4];
    const long row = blockIdx.x;                // bh*Cq + i
    const long bh = row / Cq;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    float* out = est + row * Ck;
    if (nq[row] == 0) {
        for (int j = tid; j < Ck; j += 256) out[j] = 0.0f;
        return;
    }
    for (int d = tid; d < D; d += 256) qc[d] = cq[row * D + d];
    __syncthreads();
    double mloc = -INFINITY;
    for (int j = tid; j < Ck; j += 256) {
        double s = -INFINITY;
        if (nk[bh * Ck + j] > 0) {
            const double* kc = ck + (bh * Ck + j) * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc = acc + qc[d] * kc[d];
            s = scale * acc;
        }
        wj[j] = s;
        mloc = fmax(mloc, s);
    }
    for (int o = 32; o >= 1; o >>= 1) mloc = fmax(mloc, __shfl_xor(mloc, o));
    if (lane == 0) red[wv] = mloc;
    __syncthreads();
    const double m = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    __syncthreads();
    double zloc = 0.0;
    for (int j = tid; j < Ck; j += 256) {
        const int cnt = nk[bh * Ck + j];
        const double w = cnt > 0 ? (double)cnt * exp(wj[j] - m) : 0.0;
        wj[j] = w;
        zloc += w;
    }
    for (int o = 32; o >= 1; o >>= 1) zloc += __shfl_xor(zloc, o);
    if (lane == 0) red[wv] = zloc;
    __syncthreads();
    const double z = (red[0] + red[1]) + (red[2] + red[3]);
    for (int j = tid; j < Ck; j += 256) out[j] = (float)(wj[j] / z);
}

void launch_cluster_mass(const double* cq, const int32_t* nq, const double* ck, const int32_t* nk, int B, int H,
                         int Cq, int Ck, int D, double scale, float* est, hipStream_t st) {
    const size_t lds = (size_t)(D + Ck) * sizeof(double);
    k_cluster_mass<<<(unsigned)((long)B * H * Cq), 256, lds, st>>>(cq, nq, ck, nk, Cq, Ck, D, scale, est);
}

// ---------------------------------------------------------------- cluster CSR -> block CSR

// Query cluster holding block qb of slice bh, or -1 (qoff ascending, Cq + 1 entries).
__device__ inline int cluster_of_block(const int32_t* qoff, int Cq, int qb) {
    if (qb >= qoff[Cq]) return -1;
    int lo = 0, hi = Cq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qoff[mid] <= qb) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_cblk_count(const int32_t* __restrict__ crow_ptr,
                                                    const int32_t* __restrict__ ccol_idx,
                                                    const int32_t* __restrict__ qoff,
                                                    const int32_t* __restrict__ koff, int Cq, int Ck, int NB,
                                                    long rows, int32_t* __restrict__ count) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * 4 + w;
    if (r >= rows) return;
    const long bh = r / NB;
    const int qb = (int)(r - bh * NB);
    const int ci = cluster_of_block(qoff + bh * (Cq + 1), Cq, qb);
    int n = 0;
    if (ci >= 0) {
        const int32_t* ko = koff + bh * (Ck + 1);
        const long cr = bh * Cq + ci;
        for (int e = crow_ptr[cr] + lane; e < crow_ptr[cr + 1]; e += 64) {
            const int j = ccol_idx[e];
            if (j >= 0 && j < Ck) n += ko[j + 1] - ko[j];
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o);
    }
    if (lane == 0) count[r] = n;
}

__global__ __launch_bounds__(256) void k_cblk_fill(const int32_t* __restrict__ crow_ptr,
                                                   const int32_t* __restrict__ ccol_idx,
                                                   const int32_t* __restrict__ qoff,
                                                   const int32_t* __restrict__ koff, int Cq, int Ck, int NB,
                                                   long rows, const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * 4 + w;
    if (r >= rows) return;
    const long bh = r / NB;
    const int qb = (int)(r - bh * NB);
    const int ci = cluster_of_block(qoff + bh * (Cq + 1), Cq, qb);
    if (ci < 0) return;
    const int32_t* ko = koff + bh * (Ck + 1);
    const long cr = bh * Cq + ci;
    int32_t* out = col_idx + row_ptr[r];
    int pos = 0;
    for (int e = crow_ptr[cr]; e < crow_ptr[cr + 1]; ++e) {
        const int j = ccol_idx[e];
        if (j < 0 || j >= Ck) continue;
        const int k0 = ko[j], nk = ko[j + 1] - k0;
        for (int t = lane; t < nk; t += 64) out[pos + t] = k0 + t;
        pos += nk;
    }
}

void launch_cluster_blocks(const int32_t* crow_ptr, const int32_t* ccol_idx, const int32_t* qoff,
                           const int32_t* koff, int B, int H, int Cq, int Ck, int NB, int32_t* row_ptr,
                           int32_t* col_idx, int32_t* count, hipStream_t st) {
    const long rows = (long)B * H * NB;
    const unsigned wb = (unsigned)((rows + 3) / 4);
    k_cblk_count<<<wb, 256, 0, st>>>(crow_ptr, ccol_idx, qoff, koff, Cq, Ck, NB, rows, count);
    launch_scan(count, rows, row_ptr, st);
    k_cblk_fill<<<wb, 256, 0, st>>>(crow_ptr, ccol_idx, qoff, koff, Cq, Ck, NB, rows, row_ptr, col_idx);
}

}  // namespace fpsa
