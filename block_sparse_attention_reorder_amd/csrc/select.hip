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
// threshold; it is found one digit of up to 8 bits at a time, from the row's
// largest key down (at most six passes over the row's keys, held in registers, each
// summing the keys per digit value in LDS), instead of by sorting, which gives the
// same set as sort + prefix sum + cut. One wavefront
// per row; the ascending output order falls out of ballot prefix counts over
// index order.
#include <algorithm>
#include <mutex>

#include "fpsa_device.h"
#include "fpsa_internal.h"

namespace fpsa {

constexpr int kSelWaves = 4;               // rows per workgroup (one wave each)
constexpr int kDigitBits = 8;              // the cut key is found 8 bits at a time
constexpr int kDigits = 1 << kDigitBits;   // digit values, 4 per lane

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

// Lane shift of a float64 by DPP (both halves moved; lanes with no source, or in rows
// the row mask leaves out, get +0.0).
template <int CTRL, int ROWS>
__device__ inline double dpp_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Inclusive sum over lanes 0..l of x (every partial sum an integer below 2^53, so
// exact): shifts by 1, 2, 4, 8 within each row of 16 lanes, then row 0's total into
// rows 1 and 3 and the first two rows' total into rows 2 and 3.
__device__ inline double wave_prefix_sum_exact(double x) {
    x += dpp_f64<0x111, 0xF>(x);     // row_shr:1
    x += dpp_f64<0x112, 0xF>(x);     // row_shr:2
    x += dpp_f64<0x114, 0xF>(x);     // row_shr:4
    x += dpp_f64<0x118, 0xF>(x);     // row_shr:8
    x += dpp_f64<0x142, 0xA>(x);     // row_bcast:15
    x += dpp_f64<0x143, 0xC>(x);     // row_bcast:31
    return x;
}

// Maximum over lanes 0..l of x >= 0 (the same lane pattern as the prefix sum).
__device__ inline double wave_prefix_max(double x) {
    x = fmax(x, dpp_f64<0x111, 0xF>(x));
    x = fmax(x, dpp_f64<0x112, 0xF>(x));
    x = fmax(x, dpp_f64<0x114, 0xF>(x));
    x = fmax(x, dpp_f64<0x118, 0xF>(x));
    x = fmax(x, dpp_f64<0x142, 0xA>(x));
    x = fmax(x, dpp_f64<0x143, 0xC>(x));
    return x;
}

__device__ inline double lane_f64(double x, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ inline uint64_t lanemask_lt() {
    int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Per row: kept count, cut key and how many keys equal to the cut key are kept.
//
// The cut v* is the largest v with den * (sum of keys >= v) >= num * S. No key has a
// bit above the row's highest set bit `top`, so v* is found in digits of up to 8 bits
// from bit `top` down to bit 0 (bits hi .. lo per pass; a window aligned to the
// largest key spreads the first pass's keys over many digit values). With the bits
// above hi fixed at `prefix`, `above` is the sum of the keys whose bits above hi
// exceed the prefix; the next digit is the largest d for which den * (above + sum of
// the keys that carry the prefix and a digit >= d) reaches the target. The condition
// holds at d = 0 (it held for the prefix; above is 0 in the first pass, and den >=
// num) and weakens as d grows, so d is the number of digit values where it holds,
// minus one (values the window cannot hold count as empty and fail, den * above
// being below the target). After the last digit, prefix = v* and above = the sum of
// the keys above v*. Every step is exact integer arithmetic (sums of keys stay below
// 2^53 and are carried exactly in float64 through the lane scans), so v* is the
// value a bit-by-bit search finds.
//
// One wave per row; lane l holds keys l, l + 64, ... in registers (KPL per lane,
// nb <= 64 KPL). Per digit pass the matching keys are added into 256 digit sums in
// LDS (this wave's own 2 KB); lane l reads the four sums of digits 4 (63 - l) ..
// 4 (63 - l) + 3, so a prefix sum over lanes is a suffix sum over digits.
template <int KPL>
__global__ __launch_bounds__(64 * kSelWaves) void k_select_count(const float* __restrict__ mass,
                                                                 long R, int nb, uint32_t num,
                                                                 uint32_t den,
                                                                 int32_t* __restrict__ count,
                                                                 uint64_t* __restrict__ cut,
                                                                 int32_t* __restrict__ ties) {
    __shared__ unsigned long long dsum_all[kSelWaves][kDigits];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * kSelWaves + w;
    if (r >= R) return;
    const float* row = mass + r * nb;
    unsigned long long* dsum = dsum_all[w];
    float mv[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) mv[j] = lane + 64 * j < nb ? row[lane + 64 * j] : 0.0f;
    uint64_t key[KPL];
    double part = 0.0, kmax = 0.0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        key[j] = mass_key(mv[j]);
        part += (double)key[j];                          // < 2^47: exact
        kmax = fmax(kmax, (double)key[j]);
    }
    const double S = lane_f64(wave_prefix_sum_exact(part), 63);
    int kept = 0;
    uint64_t vstar = 0;
    int nties = 0;
    if (S > 0.0 && num > 0) {
        const uint64_t target = (uint64_t)num * (uint64_t)S;     // <= 1000 * 2^52
        const int g = 63 - lane;                                  // this lane's digit group
        const uint64_t kmx = (uint64_t)lane_f64(wave_prefix_max(kmax), 63);   // >= 1
        uint64_t prefix = 0, above = 0;
        for (int hi = 63 - __builtin_clzll(kmx); hi >= 0;) {
            const int lo = hi >= kDigitBits - 1 ? hi - (kDigitBits - 1) : 0;
            const int width = hi - lo + 1;
            const uint64_t dmask = (1ull << width) - 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) dsum[4 * g + j] = 0;
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < KPL; ++j)
                if ((key[j] >> (hi + 1)) == prefix && key[j] != 0)
                    atomicAdd(&dsum[(key[j] >> lo) & dmask], (unsigned long long)key[j]);
            wave_lds_sync();
            double h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = (double)dsum[4 * g + j];
            // sum of the prefix's keys with a digit >= 4 g, then >= 4 g + j
            double sv[4];
            sv[0] = wave_prefix_sum_exact(h[0] + h[1] + h[2] + h[3]);
#pragma unroll
            for (int j = 1; j < 4; ++j) sv[j] = sv[j - 1] - h[j - 1];
            int holds = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) holds += __popcll(__ballot((uint64_t)den * (above + (uint64_t)sv[j]) >= target));
            const int d = holds - 1;                     // >= 0, uniform
            // keys of the prefix with a digit above d join `above`
            if (d + 1 < kDigits) {
                const int j1 = (d + 1) & 3;
                const double pick = j1 == 0 ? sv[0] : j1 == 1 ? sv[1] : j1 == 2 ? sv[2] : sv[3];
                above += (uint64_t)lane_f64(pick, 63 - ((d + 1) >> 2));
            }
            prefix = (prefix << width) | (uint64_t)d;
            hi = lo - 1;
        }
        const uint64_t v = prefix;                       // >= 1: all positive keys sum to S, den >= num
        int ngt = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) ngt += __popcll(__ballot(key[j] > v));
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

// Exclusive scan of per-row counts into row_ptr[R + 1] with a single workgroup, in
// tiles of 4096 counts: each thread loads its four at once, the workgroup scans the
// tile's thread sums, and the running total carries to the next tile.
__global__ __launch_bounds__(1024) void k_scan_counts(const int32_t* __restrict__ count, long R,
                                                      int32_t* __restrict__ row_ptr) {
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int32_t carry = 0;
    for (long base = 0; base < R; base += 4096) {
        const long i0 = base + 4 * (long)tid;
        int32_t c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = i0 + j < R ? count[i0 + j] : 0;
        const int32_t local = c[0] + c[1] + c[2] + c[3];
        // inclusive scan of `local` across the wave, then across the 16 waves
        int32_t x = local;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) wsum[w] = x;
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int32_t t = wsum[i];
            before += i < w ? t : 0;
            total += t;
        }
        int32_t run = carry + before + x - local;        // exclusive prefix of this thread's four
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (i0 + j < R) row_ptr[i0 + j] = run;
            run += c[j];
        }
        carry += total;
        __syncthreads();                                 // wsum is rewritten by the next tile
    }
    if (tid == 0) row_ptr[R] = carry;
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
    unsigned blocks = (unsigned)((R + kSelWaves - 1) / kSelWaves);
    // keys of a row in registers: 16 per lane up to 1024 blocks, else 64 (nb <= 4096)
    if (nb <= 64 * 16)
        k_select_count<16><<<blocks, 64 * kSelWaves, 0, st>>>(mass, R, nb, num, den, count, cut, ties);
    else
        k_select_count<64><<<blocks, 64 * kSelWaves, 0, st>>>(mass, R, nb, num, den, count, cut, ties);
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
// are marked in an LDS byte map (duplicates collapse; plain byte stores of 1, so
// neighbouring indices in one word do not serialise as atomic ORs would), then the
// dense mass row is read once, coalesced, and the marked entries are summed in float64
// (lane-strided partial sums, then a fixed butterfly: deterministic). Each lane issues
// its first KPL index loads and its KPL mass loads (nb <= 64 KPL) before it waits.

template <int KPL>
__global__ __launch_bounds__(64 * kSelWaves) void k_retained_mass(const float* __restrict__ mass,
                                                                  long R, int nb,
                                                                  const int32_t* __restrict__ row_ptr,
                                                                  const int32_t* __restrict__ col_idx,
                                                                  float* __restrict__ out) {
    extern __shared__ uint32_t marks[];    // kSelWaves byte maps of ceil(nb / 4) words
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int words = (nb + 3) >> 2;
    uint32_t* myw = marks + w * words;
    uint8_t* my = reinterpret_cast<uint8_t*>(myw);
    const long r = (long)blockIdx.x * kSelWaves + w;
    const bool live = r < R;
    for (int i = lane; i < words; i += 64) myw[i] = 0;
    float mv[KPL];
    if (live) {
        const float* row = mass + r * nb;
#pragma unroll
        for (int j = 0; j < KPL; ++j) mv[j] = lane + 64 * j < nb ? row[lane + 64 * j] : 0.0f;
    }
    __syncthreads();
    if (live) {
        const int32_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
        int32_t kbs[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) kbs[j] = e0 + lane + 64 * j < e1 ? col_idx[e0 + lane + 64 * j] : -1;
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if ((unsigned)kbs[j] < (unsigned)nb) my[kbs[j]] = 1;
        // rows listing more than 64 KPL entries (repeats)
        for (int32_t e = e0 + lane + 64 * KPL; e < e1; e += 64) {
            const int kb = col_idx[e];
            if ((unsigned)kb < (unsigned)nb) my[kb] = 1;
        }
    }
    __syncthreads();
    if (!live) return;
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int kb = lane + 64 * j;
        if (kb < nb && my[kb]) s += (double)mv[j];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) out[r] = (float)s;
}

void launch_retained_mass(const float* mass, long R, int nb, const int32_t* row_ptr,
                          const int32_t* col_idx, float* out, hipStream_t st) {
    unsigned blocks = (unsigned)((R + kSelWaves - 1) / kSelWaves);
    size_t lds = (size_t)kSelWaves * ((nb + 3) / 4) * 4;
    if (nb <= 64 * 16)
        k_retained_mass<16><<<blocks, 64 * kSelWaves, lds, st>>>(mass, R, nb, row_ptr, col_idx, out);
    else
        k_retained_mass<64><<<blocks, 64 * kSelWaves, lds, st>>>(mass, R, nb, row_ptr, col_idx, out);
}

// ---------------------------------------------------------------- CSR transpose
//
// For each (b, h) and key block kb, the query blocks whose row keeps kb, ascending:
// the column view the key-gradient pass walks. The rows are first marked in a bitmap
// (one bit per (row, kb); repeats collapse, out-of-range indices are dropped), then a
// wave per column counts and writes its query blocks in index order from ballots, so
// the result is deterministic. A row's bitmap is formed in LDS as a byte map (plain
// byte stores: neighbouring indices would serialise as atomic ORs into one word) and
// written out as whole words from ballots.

// Dynamic LDS: (blockDim.x / 64) byte maps of nb rounded up to 4 bytes.
__global__ __launch_bounds__(64 * kSelWaves) void k_csr_bitmap(const int32_t* __restrict__ row_ptr,
                                                               const int32_t* __restrict__ col_idx,
                                                               long R, int nb, int words,
                                                               uint32_t* __restrict__ bits) {
    extern __shared__ uint32_t maps[];
    const int waves = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * waves + w;
    if (r >= R) return;
    const int mwords = (nb + 3) >> 2;
    uint32_t* mw = maps + (size_t)w * mwords;
    uint8_t* mb = reinterpret_cast<uint8_t*>(mw);
    for (int i = lane; i < mwords; i += 64) mw[i] = 0;
    wave_lds_sync();
    const int32_t e1 = row_ptr[r + 1];
    for (int32_t e = row_ptr[r] + lane; e < e1; e += 64) {
        const int kb = col_idx[e];
        if ((unsigned)kb < (unsigned)nb) mb[kb] = 1;
    }
    wave_lds_sync();
    uint32_t* row = bits + r * words;
    for (int c = 0; c < nb; c += 64) {
        const uint64_t m = __ballot(c + lane < nb && mb[c + lane] != 0);
        if (lane < 2 && (c >> 5) + lane < words) row[(c >> 5) + lane] = (uint32_t)(m >> (32 * lane));
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
    // every word of every row's bitmap is written by k_csr_bitmap (no clearing pass)
    const size_t map_bytes = (size_t)((nb + 3) / 4) * 4;           // <= 46,344 (R >= nb, R nb < 2^31)
    const int mw = (int)std::max<size_t>(1, std::min<size_t>(kSelWaves, 65536 / map_bytes));
    k_csr_bitmap<<<(unsigned)((R + mw - 1) / mw), 64 * mw, mw * map_bytes, st>>>(row_ptr, col_idx, R, nb, words,
                                                                                bits);
    const unsigned blocks = (unsigned)((R + kSelWaves - 1) / kSelWaves);
    k_col_count<<<blocks, 64 * kSelWaves, 0, st>>>(bits, nb, words, R, count);
    k_scan_counts<<<1, 1024, 0, st>>>(count, R, col_ptr);
    k_col_fill<<<blocks, 64 * kSelWaves, 0, st>>>(bits, nb, words, R, col_ptr, row_idx);
}

}  // namespace fpsa
