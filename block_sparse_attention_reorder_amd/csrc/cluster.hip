// Semantic-aware permutation: tokens of each (batch, head) are clustered by k-means
// over their own query (or key) vectors and laid out cluster by cluster, so that the
// tokens a query cluster needs sit in a few dense 64-token blocks; clusters are
// represented by their centroids and sizes to estimate which key clusters matter
// [Sparse VideoGen2: Accelerate Video Generation with Sparse Attention via
// Semantic-Aware Permutation, Abstract].
//
// k-means is Lloyd's algorithm in float64 with a fixed order of every operation:
// distances summed over channels in order (no fused multiply-add: this file is
// compiled with contraction off), ties to the lower cluster, member sums in eight
// interleaved partials combined pairwise. The assignment is therefore the same on
// every device and run.
//
// Kernels: k_km_init (strided starting centroids), k_km_assign (nearest centroid; a
// lane per token, token vectors and centroids staged through LDS; cluster sizes by
// atomic counts), k_km_fill (member lists in token order, a wave per cluster with
// ballots),
// k_km_update (centroid = member mean), k_cluster_layout (slot map of the
// cluster-contiguous blocks), k_cluster_mass (centroid-based cluster masses),
// k_cblk_count / k_cblk_fill (block CSR of a cluster selection).
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

// A lane per token of a 64-token tile; the tile's vectors sit in LDS (rows padded by
// one float so that the 64 lanes read 64 different banks) and centroids pass through
// LDS in chunks of kKmChunk clusters (every lane reads the same centroid value: a
// broadcast). Within a chunk wave w takes a quarter of the clusters, four at a time so that
// each converted token value serves four distances. Each wave keeps the first strict
// minimum of its clusters (visited in increasing order), and the four candidates are
// merged on (distance, cluster), which is the sequential scan's answer.
constexpr int kKmChunk = 16;

template <typename T, int D>
__global__ __launch_bounds__(256) void k_km_assign(const T* __restrict__ x, int N, int H, int C,
                                                   const double* __restrict__ cent,
                                                   int32_t* __restrict__ assign, int32_t* __restrict__ count) {
    constexpr int kRow = D + 1;
    __shared__ float xs[64 * kRow];
    __shared__ double cs[kKmChunk * D];
    __shared__ double bestd[4][64];
    __shared__ int bestc[4][64];
    const long bh = blockIdx.y;
    const long b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = blockIdx.x * 64 + lane;
    for (int i = tid; i < 64 * D; i += 256) {
        const int t = i / D, d = i - t * D;
        const long nn = (long)blockIdx.x * 64 + t;
        xs[t * kRow + d] = nn < N ? as_float(x[((b * N + nn) * H + h) * D + d]) : 0.0f;
    }
    const float* xrow = xs + lane * kRow;
    const double* cb = cent + bh * C * D;
    double bd = INFINITY;
    int bc = C;
    for (int c0 = 0; c0 < C; c0 += kKmChunk) {
        __syncthreads();
        const long lim = (long)(C - c0) * D;
        for (int i = tid; i < kKmChunk * D; i += 256) cs[i] = i < lim ? cb[(long)c0 * D + i] : 0.0;
        __syncthreads();
#pragma unroll
        for (int g = 0; g < kKmChunk / 16; ++g) {
            const int cc = (kKmChunk / 4) * w + 4 * g;  // chunk-local cluster of this group
            if (c0 + cc >= C) break;
            const double* p = cs + cc * D;
            double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll 8
            for (int d = 0; d < D; ++d) {
                const double xd = (double)xrow[d];
                const double t0 = xd - p[d], t1 = xd - p[D + d], t2 = xd - p[2 * D + d], t3 = xd - p[3 * D + d];
                s0 = s0 + t0 * t0;
                s1 = s1 + t1 * t1;
                s2 = s2 + t2 * t2;
                s3 = s3 + t3 * t3;
            }
            const double sv[4] = {s0, s1, s2, s3};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + cc + u;
                if (c < C && sv[u] < bd) {
                    bd = sv[u];
                    bc = c;
                }
            }
        }
    }
    bestd[w][lane] = bd;
    bestc[w][lane] = bc;
    __syncthreads();
    if (w == 0 && n < N) {
#pragma unroll
        for (int u = 1; u < 4; ++u) {
            const double d2 = bestd[u][lane];
            const int c2 = bestc[u][lane];
            if (d2 < bd || (d2 == bd && c2 < bc)) {
                bd = d2;
                bc = c2;
            }
        }
        const int a = bc < C ? bc : 0;
        assign[bh * N + n] = a;
        atomicAdd(&count[bh * C + a], 1);            // sizes only: the order is irrelevant
    }
}

__global__ __launch_bounds__(256) void k_zero_i32(int32_t* __restrict__ p, long n) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0;
}

// Members of cluster c of slice bh (row bh*C + c), written in token order with
// ballots over the slice's assignment.
__global__ __launch_bounds__(256) void k_km_fill(const int32_t* __restrict__ assign, int N, int C, long rows,
                                                 const int32_t* __restrict__ off, int32_t* __restrict__ members) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * 4 + w;
    if (r >= rows) return;
    const long bh = r / C;
    const int c = (int)(r - bh * C);
    const int32_t* a = assign + bh * N;
    int32_t* out = members + off[r];
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
    for (int n0 = 0; n0 < N; n0 += 64) {
        const int n = n0 + lane;
        const bool mine = n < N && a[n] == c;
        const uint64_t m = __ballot(mine);
        if (mine) out[base + __popcll(m & lt)] = n;
        base += __popcll(m);
    }
}

// Centroid = member mean. The r-th member of a cluster (token order) goes to partial
// sum r % 8; thread (p, d) adds its partial's members in order (loads fetched 16 at a
// time), and the eight partials combine as ((p0 + p1) + (p2 + p3)) + ((p4 + p5) +
// (p6 + p7)). Eight independent chains per channel instead of one.
constexpr int kKmParts = 8;

template <typename T, int D>
__global__ __launch_bounds__(kKmParts * D) void k_km_update(const T* __restrict__ x, int N, int H, int C,
                                                            const int32_t* __restrict__ off,
                                                            const int32_t* __restrict__ members,
                                                            double* __restrict__ cent) {
    __shared__ double part[kKmParts][D];
    const long bh = blockIdx.y;
    const int c = blockIdx.x;
    const int p = threadIdx.x / D, d = threadIdx.x - (threadIdx.x / D) * D;
    const long b = bh / H, h = bh % H;
    const int r0 = off[bh * C + c], r1 = off[bh * C + c + 1];
    if (r1 == r0) return;                        // an empty cluster keeps its centroid
    double s = 0.0;
    constexpr int kBatch = 16;
    for (int r = r0 + p; r < r1; r += kKmParts * kBatch) {
        float v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int rr = r + kKmParts * i;
            v[i] = rr < r1 ? as_float(x[((b * N + members[rr]) * H + h) * D + d]) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (r + kKmParts * i < r1) s = s + (double)v[i];
    }
    part[p][d] = s;
    __syncthreads();
    if (p == 0) {
        const double s01 = part[0][d] + part[1][d], s23 = part[2][d] + part[3][d];
        const double s45 = part[4][d] + part[5][d], s67 = part[6][d] + part[7][d];
        cent[(bh * C + c) * D + d] = ((s01 + s23) + (s45 + s67)) / (double)(r1 - r0);
    }
}

template <typename T>
static void kmeans_t(const T* x, int B, int N, int H, int D, int C, int iters, int32_t* assign, double* cent,
                     int32_t* count, int32_t* off, int32_t* members, hipStream_t st) {
    const long rows = (long)B * H * C;
    dim3 gc(C, B * H);
    k_km_init<T><<<gc, 128, 0, st>>>(x, N, H, D, C, cent);
    dim3 ga((N + 63) / 64, B * H);
    const unsigned wb = (unsigned)((rows + 3) / 4);
    const unsigned zb = (unsigned)min((rows + 255) / 256, 4096L);
    for (int it = 0; it < iters; ++it) {
        k_zero_i32<<<zb, 256, 0, st>>>(count, rows);
        if (D == 128) k_km_assign<T, 128><<<ga, 256, 0, st>>>(x, N, H, C, cent, assign, count);
        else k_km_assign<T, 64><<<ga, 256, 0, st>>>(x, N, H, C, cent, assign, count);
        launch_scan(count, rows, off, st);
        k_km_fill<<<wb, 256, 0, st>>>(assign, N, C, rows, off, members);
        if (D == 128) k_km_update<T, 128><<<gc, kKmParts * 128, 0, st>>>(x, N, H, C, off, members, cent);
        else k_km_update<T, 64><<<gc, kKmParts * 64, 0, st>>>(x, N, H, C, off, members, cent);
    }
}

void launch_kmeans(const void* x, int x_f32, int B, int N, int H, int D, int C, int iters, int32_t* assign,
                   double* cent, int32_t* count, int32_t* off, int32_t* members, hipStream_t st) {
    if (x_f32)
        kmeans_t(static_cast<const float*>(x), B, N, H, D, C, iters, assign, cent, count, off, members, st);
    else
        kmeans_t(static_cast<const __bf16*>(x), B, N, H, D, C, iters, assign, cent, count, off, members, st);
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
