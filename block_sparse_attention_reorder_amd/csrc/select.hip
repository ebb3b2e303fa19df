// Retained-mass block selection: for each (head, query block) row of block masses,
// keep the smallest set of key blocks whose mass reaches the threshold (99 %),
// ranking by mass and breaking ties toward the lower block index [LoSA:
// Near-Lossless Sparse Attention for Training-Free Video Diffusion Acceleration,
// Abstract]. Also builds fixed masks into the same CSR form (the group-shared
// structured mask and per-head diagonal / multi-diagonal / stripe patterns) and
// measures how much of a later step's mass a frozen CSR retains.
//
// Arithmetic is on integer keys floor(m * 2^40), so the cut is exact and
// reproducible. The kept set is the top of the ranking up to the cut key v*:
// every key above v*, plus the lowest-indexed keys equal to v* that are still
// needed. v* is the largest key value v for which the keys >= v already reach the
// threshold; it is found one 8-bit digit at a time, most significant first (six
// passes over the row, each summing the keys per digit value in LDS), instead of
// by sorting, which gives the same set as sort + prefix sum + cut. One wavefront
// per row; the ascending output order falls out of ballot prefix counts over
// index order.
#include <mutex>

#include "fpsa_device.h"
#include "fpsa_internal.h"

namespace fpsa {

constexpr int kSelWaves = 4;               // rows per workgroup (one wave each)
constexpr size_t kSelLdsBytes = 64 * 1024; // keys of all rows of a workgroup live in LDS
constexpr int kDigitBits = 8;              // the cut key is found 8 bits at a time
constexpr int kDigits = 1 << kDigitBits;   // digit values, 4 per lane

// LDS bytes of one row of the counting kernel: its keys and its per-digit sums.
static size_t select_row_lds(int nb) { return (size_t)nb * 8 + kDigits * 8; }

// Rows (waves) per workgroup of the counting kernel so that their keys fit in LDS
// (nb <= 4096: one row takes at most 34 KB).
static int select_waves(int nb) {
    int w = (int)(kSelLdsBytes / select_row_lds(nb));
    return w < 1 ? 1 : (w > kSelWaves ? kSelWaves : w);
}

__device__ inline uint64_t mass_key(float m) {
    if (!(m > 0.0f)) return 0;             // zero, negative, NaN
    if (m >= 1.0f) return 1ull << 40;
    // m < 1: m * 2^40 is an exact exponent shift of a 24-bit significand < 2^40.
    return (uint64_t)(double)(m * 1099511627776.0f);
}

// Makes each lane's LDS writes visible to the other lanes of its wave before the
// accesses that follow (without it the compiler may, for example, hand a lane its
// own earlier store instead of reading what other lanes added since).
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ inline uint64_t lanemask_lt() {
    int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Per row: kept count, cut key and how many keys equal to the cut key are kept.
// Dynamic LDS: (blockDim.x / 64) rows of nb keys, then as many rows of 256 digit sums.
//
// The cut v* is the largest v with den * (sum of keys >= v) >= num * S. Keys are
// below 2^41, so v* has six 8-bit digits (bits 47..40, the top one 0 or 1, down to
// 7..0). With the digits above `shift + 8` fixed at `prefix`, `above` is the sum of
// the keys whose top digits exceed the prefix; the next digit is the largest d for
// which den * (above + sum of the keys that carry the prefix and a digit >= d)
// reaches the target. The condition holds at d = 0 (it held for the prefix) and
// weakens as d grows, so d is the number of digits where it holds, minus one. After
// the last digit, prefix = v* and above = the sum of the keys above v*. Every step
// is exact integer arithmetic, so v* is the same value a bit-by-bit search finds.
__global__ __launch_bounds__(64 * kSelWaves) void k_select_count(const float* __restrict__ mass,
                                                                 long R, int nb, uint32_t num,
                                                                 uint32_t den,
                                                                 int32_t* __restrict__ count,
                                                                 uint64_t* __restrict__ cut,
                                                                 int32_t* __restrict__ ties) {
    extern __shared__ uint64_t keys[];
    const int waves = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * waves + w;
    if (r >= R) return;
    const float* row = mass + r * nb;
    uint64_t* kk = keys + (size_t)w * nb;
    // this wave's digit sums; lane l owns digits 4l .. 4l+3
    unsigned long long* dsum = reinterpret_cast<unsigned long long*>(keys + (size_t)waves * nb + (size_t)w * kDigits);
    uint64_t part = 0;
    for (int i = lane; i < nb; i += 64) {
        uint64_t key = mass_key(row[i]);
        kk[i] = key;
        part += key;
    }
    const uint64_t S = wave_sum_u64(part);
    int kept = 0;
    uint64_t vstar = 0;
    int nties = 0;
    if (S > 0 && num > 0) {
        const uint64_t target = (uint64_t)num * S;     // <= 1000 * 2^52
        uint64_t prefix = 0, above = 0;
        for (int shift = 40; shift >= 0; shift -= kDigitBits) {
#pragma unroll
            for (int j = 0; j < 4; ++j) dsum[4 * lane + j] = 0;
            wave_lds_sync();
            for (int i = lane; i < nb; i += 64) {
                const uint64_t key = kk[i];
                if ((key >> (shift + kDigitBits)) == prefix) atomicAdd(&dsum[(key >> shift) & (kDigits - 1)], (unsigned long long)key);
            }
            wave_lds_sync();
            uint64_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = dsum[4 * lane + j];
            // suffix sum over lanes: this lane's four digits and every higher lane's
            uint64_t suf = h[0] + h[1] + h[2] + h[3];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint64_t t = __shfl_down((unsigned long long)suf, o);
                if (lane + o < 64) suf += t;
            }
            // sv[j]: sum of the prefix's keys whose digit is >= 4 lane + j
            uint64_t sv[4];
            sv[0] = suf;
#pragma unroll
            for (int j = 1; j < 4; ++j) sv[j] = sv[j - 1] - h[j - 1];
            int holds = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) holds += __popcll(__ballot((uint64_t)den * (above + sv[j]) >= target));
            const int d = holds - 1;                     // >= 0, uniform
            // keys of the prefix with a digit above d join `above`
            if (d + 1 < kDigits) {
                const int j1 = (d + 1) & 3;
                const uint64_t pick = j1 == 0 ? sv[0] : j1 == 1 ? sv[1] : j1 == 2 ? sv[2] : sv[3];
                above += __shfl((unsigned long long)pick, (d + 1) >> 2);
            }
            prefix = (prefix << kDigitBits) | (uint64_t)d;
        }
        const uint64_t v = prefix;                       // >= 1: all positive keys sum to S, den >= num
        int ngt = 0;
        for (int i = lane; i < nb; i += 64) ngt += kk[i] > v ? 1 : 0;
        for (int o = 32; o >= 1; o >>= 1) ngt += __shfl_xor(ngt, o);
        // den * above < target by maximality of v; the tied keys needed, each worth v:
        const uint64_t need = target - (uint64_t)den * above;
        const uint64_t per = (uint64_t)den * v;
        nties = (int)((need + per - 1) / per);
        kept = ngt + nties;
        vstar = v;
    }
    if (lane == 0) {
        count[r] = kept;
        cut[r] = vstar;
        ties[r] = nties;
    }
}

// Exclusive scan of per-row counts into row_ptr[R + 1] with a single workgroup.
__global__ __launch_bounds__(1024) void k_scan_counts(const int32_t* __restrict__ count, long R,
                                                      int32_t* __restrict__ row_ptr) {
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x;
    const long per = (R + 1023) / 1024;
    const long lo = min((long)tid * per, R), hi = min(lo + per, R);
    int32_t local = 0;
    for (long i = lo; i < hi; ++i) local += count[i];
    // inclusive scan of `local` across the workgroup
    int lane = tid & 63, w = tid >> 6;
    int32_t x = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int32_t before = 0;
    for (int i = 0; i < w; ++i) before += wsum[i];
    int32_t run = before + x - local;            // exclusive prefix of this thread's chunk
    for (long i = lo; i < hi; ++i) {
        row_ptr[i] = run;
        run += count[i];
    }
    if (tid == 1023) {
        int32_t total = 0;
        for (int i = 0; i < 16; ++i) total += wsum[i];
        row_ptr[R] = total;
    }
}

// Write kept indices of each row in ascending order.
__global__ __launch_bounds__(64 * kSelWaves) void k_select_fill(const float* __restrict__ mass,
                                                                long R, int nb,
                                                                const uint64_t* __restrict__ cut,
                                                                const int32_t* __restrict__ ties,
                                                                const int32_t* __restrict__ row_ptr,
                                                                int32_t* __restrict__ col_idx) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * kSelWaves + w;
    if (r >= R) return;
    const float* row = mass + r * nb;
    const uint64_t v = cut[r];
    const int need_ties = ties[r];
    int32_t* out = col_idx + row_ptr[r];
    if (row_ptr[r + 1] == row_ptr[r]) return;
    const uint64_t lt = lanemask_lt();
    int tie_base = 0, out_base = 0;
    for (int i0 = 0; i0 < nb; i0 += 64) {
        int i = i0 + lane;
        uint64_t key = i < nb ? mass_key(row[i]) : 0;
        bool tie = i < nb && key == v;
        uint64_t tmask = __ballot(tie);
        int tie_rank = tie_base + __popcll(tmask & lt);
        bool keep = i < nb && (key > v || (tie && tie_rank < need_ties));
        uint64_t kmask = __ballot(keep);
        if (keep) out[out_base + __popcll(kmask & lt)] = i;
        tie_base += __popcll(tmask);
        out_base += __popcll(kmask);
    }
}

size_t select_workspace_bytes(long R) {
    // count int32 [R] | ties int32 [R] | cut uint64 [R], each 256-byte aligned
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return up((size_t)R * 4) * 2 + up((size_t)R * 8);
}

// Scratch of the no-allocation entry point (fpsa_select_blocks_noalloc): per row a
// kept count, a tie count and a cut key, 16 bytes, for up to kSelectNoAllocMaxRows
// rows (16 MiB). One copy lives on every GPU the library runs on, until the process
// ends. In host code `scratch` only names the symbol: kernels receive the device
// address that hipGetSymbolAddress returns for the current device, kept per device.
constexpr size_t kSelectScratchBytes = (size_t)kSelectNoAllocMaxRows * 16;
static __device__ __align__(256) uint8_t scratch[kSelectScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t select_scratch(void** out) {
    static_assert(kSelectScratchBytes >= 16 * (size_t)kSelectNoAllocMaxRows, "16 bytes per row");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

static void carve(void* ws, long R, int32_t** count, int32_t** ties, uint64_t** cut) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char* p = static_cast<char*>(ws);
    *count = reinterpret_cast<int32_t*>(p);
    *ties = reinterpret_cast<int32_t*>(p + up((size_t)R * 4));
    *cut = reinterpret_cast<uint64_t*>(p + 2 * up((size_t)R * 4));
}

void launch_select(const float* mass, long R, int nb, uint32_t num, uint32_t den, int32_t* row_ptr,
                   int32_t* col_idx, void* ws, hipStream_t st) {
    int32_t *count, *ties;
    uint64_t* cut;
    carve(ws, R, &count, &ties, &cut);
    const int cw = select_waves(nb);
    unsigned cblocks = (unsigned)((R + cw - 1) / cw);
    k_select_count<<<cblocks, 64 * cw, (size_t)cw * select_row_lds(nb), st>>>(mass, R, nb, num, den, count, cut,
                                                                  ties);
    unsigned blocks = (unsigned)((R + kSelWaves - 1) / kSelWaves);
    k_scan_counts<<<1, 1024, 0, st>>>(count, R, row_ptr);
    k_select_fill<<<blocks, 64 * kSelWaves, 0, st>>>(mass, R, nb, cut, ties, row_ptr, col_idx);
}

// ---------------------------------------------------------------- rule-built masks
//
// A fixed mask is a per-row predicate keep(kb); one count kernel, the scan, and one
// fill kernel turn it into the CSR. Rows are (b*H + h)*nb + qb, one wave each;
// ballots over 64 consecutive kb give the ascending order directly.

// Group-shared structured mask [Grouping First, Attending Smartly: Training-Free
// Acceleration for Diffusion Transformers, Abstract]: blocks form an nh x nw grid of
// groups; a query group keeps its 3x3 neighbourhood, its whole row and its whole
// column of groups.
struct StructuredRule {
    int nb, nw;
    struct Row {
        int r, c, nw;
        __device__ bool keep(int kb) const {
            int r2 = kb / nw, c2 = kb - r2 * nw;
            return (abs(r - r2) <= 1 && abs(c - c2) <= 1) || r2 == r || c2 == c;
        }
    };
    __device__ Row row(long r) const {
        int qb = (int)(r % nb);
        return Row{qb / nw, qb % nw, nw};
    }
};

// Per-head fixed patterns [Sparse-vDiT: Unleashing the Power of Sparse Attention to
// Accelerate Video Diffusion Transformers, Abstract] on the raster sequence of
// blocks: a diagonal band |kb - qb| <= band; the band repeated every `period` blocks
// (multi-diagonal); the first `stripe` blocks for every query (vertical stripe); or
// everything (dense). A head keeps the union of what it enables.
struct PatternRule {
    int nb, H;
    const int32_t* pat;                    // [H][4]: band, period, stripe, dense
    struct Row {
        int qb, band, period, stripe, dense;
        __device__ bool keep(int kb) const {
            if (dense || kb < stripe) return true;
            if (band < 0) return false;
            const int d = kb - qb;
            if (abs(d) <= band) return true;
            if (period <= 0) return false;
            int m = d % period;
            if (m < 0) m += period;
            return min(m, period - m) <= band;
        }
    };
    __device__ Row row(long r) const {
        const int qb = (int)(r % nb);
        const int32_t* p = pat + 4 * (int)((r / nb) % H);
        return Row{qb, p[0], p[1], p[2], p[3] != 0};
    }
};

template <class Rule>
__global__ __launch_bounds__(64 * kSelWaves) void k_rule_count(Rule rule, int nb, long R,
                                                               int32_t* __restrict__ count) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * kSelWaves + w;
    if (r >= R) return;
    const auto row = rule.row(r);
    int n = 0;
    for (int i0 = 0; i0 < nb; i0 += 64) {
        int kb = i0 + lane;
        n += __popcll(__ballot(kb < nb && row.keep(kb)));
    }
    if (lane == 0) count[r] = n;
}

template <class Rule>
__global__ __launch_bounds__(64 * kSelWaves) void k_rule_fill(Rule rule, int nb, long R,
                                                              const int32_t* __restrict__ row_ptr,
                                                              int32_t* __restrict__ col_idx) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * kSelWaves + w;
    if (r >= R) return;
    const auto row = rule.row(r);
    int32_t* out = col_idx + row_ptr[r];
    const uint64_t lt = lanemask_lt();
    int base = 0;
    for (int i0 = 0; i0 < nb; i0 += 64) {
        int kb = i0 + lane;
        bool keep = kb < nb && row.keep(kb);
        uint64_t m = __ballot(keep);
        if (keep) out[base + __popcll(m & lt)] = kb;
        base += __popcll(m);
    }
}

template <class Rule>
static void launch_rule(const Rule& rule, int nb, long R, int32_t* row_ptr, int32_t* col_idx,
                        void* ws, hipStream_t st) {
    int32_t *count, *ties;
    uint64_t* cut;
    carve(ws, R, &count, &ties, &cut);
    unsigned blocks = (unsigned)((R + kSelWaves - 1) / kSelWaves);
    k_rule_count<<<blocks, 64 * kSelWaves, 0, st>>>(rule, nb, R, count);
    k_scan_counts<<<1, 1024, 0, st>>>(count, R, row_ptr);
    k_rule_fill<<<blocks, 64 * kSelWaves, 0, st>>>(rule, nb, R, row_ptr, col_idx);
}

void launch_structured(const Geom& g, int copies, int32_t* row_ptr, int32_t* col_idx, void* ws,
                       hipStream_t st) {
    launch_rule(StructuredRule{g.nb, g.nw}, g.nb, (long)copies * g.nb, row_ptr, col_idx, ws, st);
}

void launch_pattern(int nb, int B, int H, const int32_t* patterns, int32_t* row_ptr,
                    int32_t* col_idx, void* ws, hipStream_t st) {
    launch_rule(PatternRule{nb, H, patterns}, nb, (long)B * H * nb, row_ptr, col_idx, ws, st);
}

// ---------------------------------------------------------------- retained-mass monitor
//
// The share of each row's block mass that a frozen block set still holds at a later
// step: sum of mass[r, kb] over the distinct in-range kb that CSR row r lists. The
// frozen indices rest on the support staying put across steps [LoSA: Near-Lossless
// Sparse Attention for Training-Free Video Diffusion Acceleration, Abstract]; this
// measures how much of the new mass they cover. One wave per row: the row's indices
// are marked in an LDS bitmap (duplicates collapse), then the dense mass row is read
// once, coalesced, and the marked entries are summed in float64 (lane-strided
// partial sums, then a fixed butterfly: deterministic).

__global__ __launch_bounds__(64 * kSelWaves) void k_retained_mass(const float* __restrict__ mass,
                                                                  long R, int nb,
                                                                  const int32_t* __restrict__ row_ptr,
                                                                  const int32_t* __restrict__ col_idx,
                                                                  float* __restrict__ out) {
    extern __shared__ uint32_t marks[];    // kSelWaves bitmaps of ceil(nb / 32) words
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int words = (nb + 31) >> 5;
    uint32_t* my = marks + w * words;
    const long r = (long)blockIdx.x * kSelWaves + w;
    const bool live = r < R;
    for (int i = lane; i < words; i += 64) my[i] = 0;
    __syncthreads();
    if (live) {
        const int32_t e1 = row_ptr[r + 1];
        for (int32_t e = row_ptr[r] + lane; e < e1; e += 64) {
            const int kb = col_idx[e];
            if ((unsigned)kb < (unsigned)nb) atomicOr(&my[kb >> 5], 1u << (kb & 31));
        }
    }
    __syncthreads();
    if (!live) return;
    const float* row = mass + r * nb;
    double s = 0.0;
    for (int kb = lane; kb < nb; kb += 64)
        if ((my[kb >> 5] >> (kb & 31)) & 1u) s += (double)row[kb];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) out[r] = (float)s;
}

void launch_retained_mass(const float* mass, long R, int nb, const int32_t* row_ptr,
                          const int32_t* col_idx, float* out, hipStream_t st) {
    unsigned blocks = (unsigned)((R + kSelWaves - 1) / kSelWaves);
    size_t lds = (size_t)kSelWaves * ((nb + 31) / 32) * 4;
    k_retained_mass<<<blocks, 64 * kSelWaves, lds, st>>>(mass, R, nb, row_ptr, col_idx, out);
}

// ---------------------------------------------------------------- CSR transpose
//
// For each (b, h) and key block kb, the query blocks whose row keeps kb, ascending:
// the column view the key-gradient pass walks. The rows are first marked in a bitmap
// (one bit per (row, kb); repeats collapse, out-of-range indices are dropped), then a
// wave per column counts and writes its query blocks in index order from ballots, so
// the result is deterministic.

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* __restrict__ p, long n) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(64 * kSelWaves) void k_csr_bitmap(const int32_t* __restrict__ row_ptr,
                                                               const int32_t* __restrict__ col_idx,
                                                               long R, int nb, int words,
                                                               uint32_t* __restrict__ bits) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * kSelWaves + w;
    if (r >= R) return;
    uint32_t* row = bits + r * words;
    const int32_t e1 = row_ptr[r + 1];
    for (int32_t e = row_ptr[r] + lane; e < e1; e += 64) {
        const int kb = col_idx[e];
        if ((unsigned)kb < (unsigned)nb) atomicOr(&row[kb >> 5], 1u << (kb & 31));
    }
}

// bit (qb, kb) of head slice bh
__device__ inline bool csr_bit(const uint32_t* bits, long bh, int nb, int words, int qb, int kb) {
    return (bits[(bh * nb + qb) * words + (kb >> 5)] >> (kb & 31)) & 1u;
}

__global__ __launch_bounds__(64 * kSelWaves) void k_col_count(const uint32_t* __restrict__ bits, int nb,
                                                              int words, long C,
                                                              int32_t* __restrict__ count) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long c = (long)blockIdx.x * kSelWaves + w;
    if (c >= C) return;
    const long bh = c / nb;
    const int kb = (int)(c - bh * nb);
    int n = 0;
    for (int q0 = 0; q0 < nb; q0 += 64) {
        const int qb = q0 + lane;
        n += __popcll(__ballot(qb < nb && csr_bit(bits, bh, nb, words, qb, kb)));
    }
    if (lane == 0) count[c] = n;
}

__global__ __launch_bounds__(64 * kSelWaves) void k_col_fill(const uint32_t* __restrict__ bits, int nb,
                                                             int words, long C,
                                                             const int32_t* __restrict__ col_ptr,
                                                             int32_t* __restrict__ row_idx) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long c = (long)blockIdx.x * kSelWaves + w;
    if (c >= C) return;
    const long bh = c / nb;
    const int kb = (int)(c - bh * nb);
    int32_t* out = row_idx + col_ptr[c];
    const uint64_t lt = lanemask_lt();
    int base = 0;
    for (int q0 = 0; q0 < nb; q0 += 64) {
        const int qb = q0 + lane;
        const bool keep = qb < nb && csr_bit(bits, bh, nb, words, qb, kb);
        const uint64_t m = __ballot(keep);
        if (keep) out[base + __popcll(m & lt)] = qb;
        base += __popcll(m);
    }
}

void launch_scan(const int32_t* count, long R, int32_t* out, hipStream_t st) {
    k_scan_counts<<<1, 1024, 0, st>>>(count, R, out);
}

size_t transpose_workspace_bytes(long R, int nb) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return up((size_t)R * ((nb + 31) / 32) * 4) + up((size_t)R * 4);
}

void launch_csr_transpose(const int32_t* row_ptr, const int32_t* col_idx, long R, int nb,
                          int32_t* col_ptr, int32_t* row_idx, void* ws, hipStream_t st) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int words = (nb + 31) / 32;
    uint32_t* bits = static_cast<uint32_t*>(ws);
    int32_t* count = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + up((size_t)R * words * 4));
    const long nbits = R * words;
    const unsigned fill_blocks = (unsigned)min((nbits + 255) / 256, 65536L);
    k_fill_zero<<<fill_blocks, 256, 0, st>>>(bits, nbits);
    const unsigned blocks = (unsigned)((R + kSelWaves - 1) / kSelWaves);
    k_csr_bitmap<<<blocks, 64 * kSelWaves, 0, st>>>(row_ptr, col_idx, R, nb, words, bits);
    k_col_count<<<blocks, 64 * kSelWaves, 0, st>>>(bits, nb, words, R, count);
    k_scan_counts<<<1, 1024, 0, st>>>(count, R, col_ptr);
    k_col_fill<<<blocks, 64 * kSelWaves, 0, st>>>(bits, nb, words, R, col_ptr, row_idx);
}

}  // namespace fpsa
