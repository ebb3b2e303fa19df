/*
 * CPU oracle for block-sparse attention with retained-mass block selection.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. The product path never calls it.
 *
 * Plain, slow, obviously correct: every score, exponential and sum is taken in
 * double precision, loops follow the definitions one token at a time, and tokens
 * stay in raster order: block membership comes from the tile formula, never from
 * a permuted layout. Parallelism: OpenMP over independent (batch, head, q-block)
 * rows only, which does not change any arithmetic.
 *
 * Sources: the retained-mass rule, per-head / per-query-block selection and frozen
 * reuse follow [LoSA: Near-Lossless Sparse Attention for Training-Free Video
 * Diffusion Acceleration, Abstract]; the 3D tile as the unit of both sparsity and
 * quantization follows [FPSAttention: Training-Aware FP8 and Sparsity Co-Design for
 * Fast Video Diffusion, Abstract]; the group-shared structured key set follows
 * [Grouping First, Attending Smartly: Training-Free Acceleration for Diffusion
 * Transformers, Abstract]; the diagonal, multi-diagonal and vertical-stripe patterns
 * follow [Sparse-vDiT: Unleashing the Power of Sparse Attention to Accelerate Video
 * Diffusion Transformers, Abstract].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Geometry                                                                   */
/* ------------------------------------------------------------------------- */

/* Number of tiles along one axis: the grid is padded up to a tile multiple. */
static int64_t tiles_along(int64_t g, int64_t tile) { return (g + tile - 1) / tile; }

int64_t orc_num_blocks(int T, int Hg, int Wg, int tt, int th, int tw) {
    if (T <= 0 || Hg <= 0 || Wg <= 0 || tt <= 0 || th <= 0 || tw <= 0) return -1;
    return tiles_along(T, tt) * tiles_along(Hg, th) * tiles_along(Wg, tw);
}

/*
 * For every raster token n = (t*Hg + h)*Wg + w: its block id (tiles numbered in
 * raster order over the tile grid) and its slot in the tiled sequence, i.e.
 * 64*block + the token's raster position inside its tile.
 */
void orc_token_blocks(int T, int Hg, int Wg, int tt, int th, int tw,
                      int32_t* block_of, int64_t* slot_of) {
    int64_t nh = tiles_along(Hg, th), nw = tiles_along(Wg, tw);
    int64_t tile_tokens = (int64_t)tt * th * tw;
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < Hg; ++h)
            for (int w = 0; w < Wg; ++w) {
                int64_t n = ((int64_t)t * Hg + h) * Wg + w;
                int64_t blk = ((int64_t)(t / tt) * nh + (h / th)) * nw + (w / tw);
                int64_t within = ((int64_t)(t % tt) * th + (h % th)) * tw + (w % tw);
                block_of[n] = (int32_t)blk;
                if (slot_of) slot_of[n] = blk * tile_tokens + within;
            }
}

/* Raster index of element (b, n, h, d) in a [B, N, H, D] array. */
#define RIX(b, n, h, d) ((((int64_t)(b) * N + (n)) * H + (h)) * D + (d))

static double dot_scaled(const float* q, const float* k, int D, double scale) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += (double)q[d] * (double)k[d];
    return s * scale;
}

/* ------------------------------------------------------------------------- */
/* Dense softmax attention (the reference every sparse result reduces to)    */
/* ------------------------------------------------------------------------- */

/*
 * out[b,n,h,:] = sum_j softmax_j(scale * q_n . k_j) v_j over all N keys, for the
 * queries listed in `queries` (all N when queries == NULL). out is [B, N, H, D].
 */
void orc_dense_attention(const float* q, const float* k, const float* v,
                         int B, int N, int H, int D, double scale,
                         const int32_t* queries, int nq, double* out) {
    int count = queries ? nq : N;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int qi = 0; qi < count; ++qi) {
                int i = queries ? queries[qi] : qi;
                double* s = (double*)malloc(sizeof(double) * (size_t)N);
                double m = -INFINITY;
                for (int j = 0; j < N; ++j) {
                    s[j] = dot_scaled(q + RIX(b, i, h, 0), k + RIX(b, j, h, 0), D, scale);
                    if (s[j] > m) m = s[j];
                }
                double z = 0.0;
                for (int j = 0; j < N; ++j) z += exp(s[j] - m);
                double* o = out + RIX(b, i, h, 0);
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                for (int j = 0; j < N; ++j) {
                    double p = exp(s[j] - m) / z;
                    const float* vj = v + RIX(b, j, h, 0);
                    for (int d = 0; d < D; ++d) o[d] += p * (double)vj[d];
                }
                free(s);
            }
}

/* ------------------------------------------------------------------------- */
/* Block attention masses (the exact dense measurement step)                  */
/* ------------------------------------------------------------------------- */

/*
 * mass[b,h,r,kb] for each requested query block qb = qblocks[r] (all nb blocks
 * when qblocks == NULL): the softmax probability that the real queries of qb put
 * on the real keys of kb, summed over those keys and averaged over those queries.
 * Each row therefore sums to one. Padding tokens do not exist in raster order, so
 * they carry no mass. mass is [B, H, nsel, nb] float64.
 */
void orc_block_mass(const float* q, const float* k, int B, int N, int H, int D,
                    const int32_t* block_of, int nb, double scale,
                    const int32_t* qblocks, int nsel, double* mass) {
    int count = qblocks ? nsel : nb;
    int64_t* cnt = (int64_t*)calloc((size_t)nb, sizeof(int64_t));
    for (int n = 0; n < N; ++n) cnt[block_of[n]]++;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int r = 0; r < count; ++r) {
                int qb = qblocks ? qblocks[r] : r;
                double* row = mass + (((int64_t)b * H + h) * count + r) * nb;
                for (int kb = 0; kb < nb; ++kb) row[kb] = 0.0;
                double* s = (double*)malloc(sizeof(double) * (size_t)N);
                for (int i = 0; i < N; ++i) {
                    if (block_of[i] != qb) continue;
                    double m = -INFINITY;
                    for (int j = 0; j < N; ++j) {
                        s[j] = dot_scaled(q + RIX(b, i, h, 0), k + RIX(b, j, h, 0), D, scale);
                        if (s[j] > m) m = s[j];
                    }
                    double z = 0.0;
                    for (int j = 0; j < N; ++j) z += exp(s[j] - m);
                    for (int j = 0; j < N; ++j) row[block_of[j]] += exp(s[j] - m) / z;
                }
                if (cnt[qb] > 0)
                    for (int kb = 0; kb < nb; ++kb) row[kb] /= (double)cnt[qb];
                free(s);
            }
    free(cnt);
}

/* ------------------------------------------------------------------------- */
/* Retained-mass selection                                                    */
/* ------------------------------------------------------------------------- */

/*
 * Fixed-point key of a mass: floor(m * 2^40) after clamping m to [0, 1] (NaN -> 0).
 * For a float32 m in [0, 1] the product is an exact power-of-two shift, so the key
 * is exact and identical wherever it is computed.
 */
uint64_t orc_mass_key(float m) {
    if (!(m > 0.0f)) return 0;          /* zero, negative, NaN */
    if (m >= 1.0f) return (uint64_t)1 << 40;
    return (uint64_t)floor((double)m * 1099511627776.0);
}

typedef struct { uint64_t key; int32_t idx; } ranked;

/* Larger key first; equal keys: lower block index first. */
static int rank_order(const void* a, const void* b) {
    const ranked* x = (const ranked*)a;
    const ranked* y = (const ranked*)b;
    if (x->key != y->key) return x->key > y->key ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0);
}

static int ascending_int(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

/*
 * For each of the R rows of mass [R, nb]: rank blocks by mass (ties to the lower
 * index), and keep the shortest leading run of that ranking whose summed mass
 * reaches thr_num/thr_den of the row total; the comparison is den*kept >= num*total
 * on the fixed-point keys. A row with zero total keeps nothing. Kept indices are
 * written in ascending order: row r occupies col_idx[row_ptr[r] .. row_ptr[r+1]).
 * col_idx must hold R*nb entries. Returns the number of kept pairs.
 */
int64_t orc_select_blocks(const float* mass, int64_t R, int nb, uint32_t thr_num, uint32_t thr_den,
                          int32_t* row_ptr, int32_t* col_idx) {
    ranked* order = (ranked*)malloc(sizeof(ranked) * (size_t)nb);
    int64_t nnz = 0;
    row_ptr[0] = 0;
    for (int64_t r = 0; r < R; ++r) {
        const float* row = mass + r * nb;
        uint64_t total = 0;
        for (int k = 0; k < nb; ++k) {
            order[k].key = orc_mass_key(row[k]);
            order[k].idx = k;
            total += order[k].key;
        }
        qsort(order, (size_t)nb, sizeof(ranked), rank_order);
        int keep = 0;
        uint64_t kept = 0;
        while (keep < nb && (uint64_t)thr_den * kept < (uint64_t)thr_num * total) {
            kept += order[keep].key;
            keep++;
        }
        /* total == 0 (or thr_num == 0): the loop never runs and nothing is kept. */
        int32_t* out = col_idx + nnz;
        for (int i = 0; i < keep; ++i) out[i] = order[i].idx;
        qsort(out, (size_t)keep, sizeof(int32_t), ascending_int);
        nnz += keep;
        row_ptr[r + 1] = (int32_t)nnz;
    }
    free(order);
    return nnz;
}

/*
 * How close each row's cut is to flipping, in real (float64) arithmetic on float64
 * masses: the smallest of (kept - p*total), (p*total - kept_without_last) and the
 * mass gap between the last kept block and the first dropped one, in the ranking of
 * the float64 masses. A row whose margin is below the error of a computed mass may
 * legitimately select differently.
 */
typedef struct { double val; int32_t idx; } ranked64;

/* Larger mass first; equal masses: lower block index first. */
static int rank_order64(const void* a, const void* b) {
    const ranked64* x = (const ranked64*)a;
    const ranked64* y = (const ranked64*)b;
    if (x->val != y->val) return x->val > y->val ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0);
}

void orc_cut_margin(const double* mass, int64_t R, int nb, double p, double* margin) {
    ranked64* order = (ranked64*)malloc(sizeof(ranked64) * (size_t)nb);
    for (int64_t r = 0; r < R; ++r) {
        const double* row = mass + r * nb;
        double total = 0.0;
        for (int k = 0; k < nb; ++k) {
            order[k].val = row[k];
            order[k].idx = k;
            total += row[k];
        }
        qsort(order, (size_t)nb, sizeof(ranked64), rank_order64);
        double target = p * total, c = 0.0, prev = 0.0;
        int keep = 0;
        while (keep < nb && c < target) { prev = c; c += order[keep].val; keep++; }
        double m = INFINITY;
        if (keep > 0) {
            if (c - target < m) m = c - target;
            if (target - prev < m) m = target - prev;
            if (keep < nb && order[keep - 1].val - order[keep].val < m)
                m = order[keep - 1].val - order[keep].val;
        }
        margin[r] = m;
    }
    free(order);
}

/* ------------------------------------------------------------------------- */
/* Masked (block-sparse) attention                                            */
/* ------------------------------------------------------------------------- */

/*
 * For each requested query block qb = qblocks[r] of each (b, h): every real query
 * i of qb attends to the real keys of the blocks kept for row (b*H + h)*nb + qb of
 * the CSR, with the softmax renormalised over exactly those keys. A query whose
 * allowed set is empty gets a zero output. Output rows are written to
 * out[b, h, r, e, :] for the e-th real token of qb in raster order (e < 64), and
 * token_of[b, h, r, e] holds that token's raster index (-1 past the last token).
 * out is [B, H, nsel, 64, D] float64.
 */
void orc_masked_attention(const float* q, const float* k, const float* v,
                          int B, int N, int H, int D, const int32_t* block_of, int nb, double scale,
                          const int32_t* row_ptr, const int32_t* col_idx,
                          const int32_t* qblocks, int nsel, double* out, int32_t* token_of) {
    int count = qblocks ? nsel : nb;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int r = 0; r < count; ++r) {
                int qb = qblocks ? qblocks[r] : r;
                int64_t row = ((int64_t)b * H + h) * nb + qb;
                char* allowed = (char*)calloc((size_t)nb, 1);
                for (int32_t e = row_ptr[row]; e < row_ptr[row + 1]; ++e)
                    if ((uint32_t)col_idx[e] < (uint32_t)nb) allowed[col_idx[e]] = 1;   /* others: nothing */
                double* s = (double*)malloc(sizeof(double) * (size_t)N);
                int64_t base = (((int64_t)b * H + h) * count + r) * 64;
                for (int e = 0; e < 64; ++e) {
                    token_of[base + e] = -1;
                    for (int d = 0; d < D; ++d) out[(base + e) * D + d] = 0.0;
                }
                int e = 0;
                for (int i = 0; i < N && e < 64; ++i) {
                    if (block_of[i] != qb) continue;
                    token_of[base + e] = i;
                    double* o = out + (base + e) * D;
                    double m = -INFINITY;
                    for (int j = 0; j < N; ++j) {
                        if (!allowed[block_of[j]]) continue;
                        s[j] = dot_scaled(q + RIX(b, i, h, 0), k + RIX(b, j, h, 0), D, scale);
                        if (s[j] > m) m = s[j];
                    }
                    if (m != -INFINITY) {
                        double z = 0.0;
                        for (int j = 0; j < N; ++j)
                            if (allowed[block_of[j]]) z += exp(s[j] - m);
                        for (int j = 0; j < N; ++j) {
                            if (!allowed[block_of[j]]) continue;
                            double p = exp(s[j] - m) / z;
                            const float* vj = v + RIX(b, j, h, 0);
                            for (int d = 0; d < D; ++d) o[d] += p * (double)vj[d];
                        }
                    }
                    e++;
                }
                free(s);
                free(allowed);
            }
}

/* ------------------------------------------------------------------------- */
/* FP8 e4m3 (OCP "e4m3fn") per-tile quantization, simulated                   */
/* ------------------------------------------------------------------------- */

/*
 * Value of an 8-bit e4m3fn code: 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); the all-ones pattern
 * S.1111.111 is NaN and there is no infinity, so the largest finite value is 448.
 */
double orc_e4m3_decode(uint8_t code) {
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/*
 * Nearest finite e4m3fn code to x (ties to the even code, i.e. the one whose
 * mantissa LSB is zero), found by comparing against every finite magnitude; values
 * beyond 448 therefore saturate to 448. NaN maps to the NaN code.
 */
static double e4m3_magnitude[0x7F];             /* decode of codes 0x00 .. 0x7E */
static int e4m3_table_ready = 0;

uint8_t orc_e4m3_encode(double x) {
    if (!e4m3_table_ready) {
        for (int c = 0; c < 0x7F; ++c) e4m3_magnitude[c] = orc_e4m3_decode((uint8_t)c);
        e4m3_table_ready = 1;
    }
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c < 0x7F; ++c) {            /* 0x00 .. 0x7E: all finite magnitudes */
        double err = fabs(e4m3_magnitude[c] - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

/*
 * Per (b, h, block): a = max |x| over the block's real tokens and all D channels,
 * scale = float32(a / 448) (1 when a == 0), and every element becomes
 * decode(encode(float32(x / scale))) * scale, stored as float32 (a relative
 * rounding of at most 2^-24 on top of the quantization). x and xhat are
 * [B, N, H, D]; scales is [B, H, nb] float32.
 */
void orc_fp8_tile_quantize(const float* x, int B, int N, int H, int D,
                           const int32_t* block_of, int nb, float* xhat, float* scales) {
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            float* sc = scales + ((int64_t)b * H + h) * nb;
            for (int blk = 0; blk < nb; ++blk) sc[blk] = 0.0f;
            for (int n = 0; n < N; ++n)
                for (int d = 0; d < D; ++d) {
                    float a = fabsf(x[RIX(b, n, h, d)]);
                    if (a > sc[block_of[n]]) sc[block_of[n]] = a;
                }
            for (int blk = 0; blk < nb; ++blk) sc[blk] = sc[blk] > 0.0f ? sc[blk] / 448.0f : 1.0f;
            for (int n = 0; n < N; ++n)
                for (int d = 0; d < D; ++d) {
                    float s = sc[block_of[n]];
                    float y = x[RIX(b, n, h, d)] / s;
                    xhat[RIX(b, n, h, d)] = (float)(orc_e4m3_decode(orc_e4m3_encode((double)y)) * (double)s);
                }
        }
}

/* ------------------------------------------------------------------------- */
/* Structured (group-shared) mask                                             */
/* ------------------------------------------------------------------------- */

/*
 * On a 2D grid of gh x gw token groups (block id = row*gw + col): query group
 * (r, c) may attend key group (r2, c2) when it is in the 3x3 neighbourhood
 * (|r-r2| <= 1 and |c-c2| <= 1, clipped at the border, itself included), or in the
 * same group-row (r2 == r), or in the same group-column (c2 == c). Rows are
 * replicated for `copies` (batch*head) copies; indices ascending. A row has at
 * most gh + gw + 9 entries, so col_idx must hold copies * gh*gw * (gh + gw + 9).
 * Returns the number of pairs.
 */
int64_t orc_structured_mask(int gh, int gw, int copies, int32_t* row_ptr, int32_t* col_idx) {
    int64_t nb = (int64_t)gh * gw, nnz = 0;
    row_ptr[0] = 0;
    for (int cp = 0; cp < copies; ++cp)
        for (int64_t qb = 0; qb < nb; ++qb) {
            int r = (int)(qb / gw), c = (int)(qb % gw);
            for (int64_t kb = 0; kb < nb; ++kb) {
                int r2 = (int)(kb / gw), c2 = (int)(kb % gw);
                int near = abs(r - r2) <= 1 && abs(c - c2) <= 1;
                if (near || r2 == r || c2 == c) col_idx[nnz++] = (int32_t)kb;
            }
            row_ptr[(int64_t)cp * nb + qb + 1] = (int32_t)nnz;
        }
    return nnz;
}

/*
 * The same per-tile quantization as orc_fp8_tile_quantize, returning the e4m3fn
 * codes themselves: codes [B, N, H, D] (raster) and scales [B, H, nb].
 */
void orc_fp8_tile_codes(const float* x, int B, int N, int H, int D,
                        const int32_t* block_of, int nb, uint8_t* codes, float* scales) {
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            float* sc = scales + ((int64_t)b * H + h) * nb;
            for (int blk = 0; blk < nb; ++blk) sc[blk] = 0.0f;
            for (int n = 0; n < N; ++n)
                for (int d = 0; d < D; ++d) {
                    float a = fabsf(x[RIX(b, n, h, d)]);
                    if (a > sc[block_of[n]]) sc[block_of[n]] = a;
                }
            for (int blk = 0; blk < nb; ++blk) sc[blk] = sc[blk] > 0.0f ? sc[blk] / 448.0f : 1.0f;
            for (int n = 0; n < N; ++n)
                for (int d = 0; d < D; ++d) {
                    float y = x[RIX(b, n, h, d)] / sc[block_of[n]];
                    codes[RIX(b, n, h, d)] = orc_e4m3_encode((double)y);
                }
        }
}

/*
 * bf16 value of a float32 under round-to-nearest-even: keep the upper 16 bits of the
 * IEEE single encoding, rounding on the 16 dropped bits (above half up, below half
 * down, exactly half to the even kept pattern). Infinities pass; NaN stays NaN. Used
 * for the dequantized e4m3 tiles the FP8 backward reads (code value times tile scale,
 * a float32 product, carried in bf16).
 */
void orc_round_bf16(const float* x, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b;
        memcpy(&b, &x[i], 4);
        if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu) != 0) {
            out[i] = x[i];                              /* NaN */
            continue;
        }
        const uint32_t dropped = b & 0xFFFFu, kept = b >> 16;
        uint32_t r = kept;
        if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) r = kept + 1u;
        const uint32_t o = r << 16;
        memcpy(&out[i], &o, 4);
    }
}

/* ------------------------------------------------------------------------- */
/* Retained mass of a frozen block set                                        */
/* ------------------------------------------------------------------------- */

/*
 * The fraction of a row's attention mass that a block set keeps: for row r,
 * out[r] = sum of mass[r, kb] over the distinct indices kb in [0, nb) that the row
 * lists (the block masses of a later step measured on the support frozen at the
 * dense step; the support's stability across steps is the observation the frozen
 * indices rest on [LoSA: Near-Lossless Sparse Attention for Training-Free Video
 * Diffusion Acceleration, Abstract]). Float64 sum in ascending kb order.
 */
void orc_retained_mass(const float* mass, int64_t R, int nb, const int32_t* row_ptr,
                       const int32_t* col_idx, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        char* seen = (char*)calloc((size_t)nb, 1);
        for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e)
            if (col_idx[e] >= 0 && col_idx[e] < nb) seen[col_idx[e]] = 1;
        double s = 0.0;
        for (int kb = 0; kb < nb; ++kb)
            if (seen[kb]) s += (double)mass[r * (int64_t)nb + kb];
        out[r] = s;
        free(seen);
    }
}

/* ------------------------------------------------------------------------- */
/* Fixed sparsity patterns (diagonal, multi-diagonal, vertical stripes)       */
/* ------------------------------------------------------------------------- */

/*
 * The three recurring patterns named for video DiT attention maps [Sparse-vDiT:
 * Unleashing the Power of Sparse Attention to Accelerate Video Diffusion
 * Transformers, Abstract], read on the sequence of 64-token blocks (raster tile order):
 *   diagonal:        key block kb with |kb - qb| <= band;
 *   multi-diagonal:  the same band repeated every `period` blocks, i.e. the distance
 *                    from kb - qb to the nearest multiple of period is <= band;
 *   vertical stripe: every query block keeps the key blocks kb < stripe;
 *   dense:           every key block.
 * A head's pattern is the union of the parts it enables (band < 0: no band;
 * period <= 0: no repeat; stripe <= 0: no stripe). pattern[h] = {band, period,
 * stripe, dense}; rows (b*H + h)*nb + qb; indices ascending. Returns the number of
 * pairs; col_idx must hold them.
 */
static int pattern_keep(const int32_t* p, int qb, int kb) {
    int band = p[0], period = p[1], stripe = p[2], dense = p[3];
    if (dense) return 1;
    if (kb < stripe) return 1;
    if (band >= 0) {
        int d = kb - qb;
        if (abs(d) <= band) return 1;
        if (period > 0) {
            int m = ((d % period) + period) % period;
            int dist = m < period - m ? m : period - m;
            if (dist <= band) return 1;
        }
    }
    return 0;
}

int64_t orc_pattern_mask(int nb, int B, int H, const int32_t* pattern, int32_t* row_ptr,
                         int32_t* col_idx) {
    int64_t nnz = 0;
    row_ptr[0] = 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int qb = 0; qb < nb; ++qb) {
                for (int kb = 0; kb < nb; ++kb)
                    if (pattern_keep(pattern + 4 * h, qb, kb)) col_idx[nnz++] = kb;
                row_ptr[((int64_t)b * H + h) * nb + qb + 1] = (int32_t)nnz;
            }
    return nnz;
}

/* ------------------------------------------------------------------------- */
/* Gradients of masked attention                                              */
/* ------------------------------------------------------------------------- */

/*
 * Backward of the masked attention above for a loss whose gradient with respect
 * to o_i is dout_i, written from the chain rule (the kernel is FlashAttention
 * style, and training through the same tiles is what the FP8 and sparsity
 * co-design is for [FPSAttention: Training-Aware FP8 and Sparsity Co-Design for
 * Fast Video Diffusion, Abstract]). With s_ij = scale q_i . k_j and p_ij the
 * softmax of s_i over the allowed keys A_i of query i:
 *   dv_j  = sum_i p_ij dout_i                    (o_i = sum_j p_ij v_j)
 *   dp_ij = dout_i . v_j
 *   ds_ij = p_ij (dp_ij - sum_j' p_ij' dp_ij')   (softmax Jacobian)
 *   dq_i  = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i.
 * Queries with an empty A_i contribute nothing. One query at a time; per (b, h) the
 * key gradients accumulate over queries in raster order.
 *
 * The per-query step writes dq_i into dq_row and, when dk / dv are given, adds the
 * query's contributions to the key gradients of the (b, h) slice.
 */
static void bwd_one_query(const float* q, const float* k, const float* v, const float* dout,
                          int N, int H, int D, int b, int h, int i, const int32_t* block_of,
                          const char* allowed, double scale, double* s, double* dp,
                          double* dq_row, double* dk, double* dv, double* mq_row, double* mk,
                          double* mv) {
    const float* qi = q + RIX(b, i, h, 0);
    const float* gi = dout + RIX(b, i, h, 0);
    for (int d = 0; d < D; ++d) dq_row[d] = 0.0;
    if (mq_row)
        for (int d = 0; d < D; ++d) mq_row[d] = 0.0;
    double m = -INFINITY;
    for (int j = 0; j < N; ++j) {
        if (!allowed[block_of[j]]) continue;
        s[j] = dot_scaled(qi, k + RIX(b, j, h, 0), D, scale);
        if (s[j] > m) m = s[j];
    }
    if (m == -INFINITY) return;
    double z = 0.0;
    for (int j = 0; j < N; ++j)
        if (allowed[block_of[j]]) z += exp(s[j] - m);
    double delta = 0.0;
    for (int j = 0; j < N; ++j) {
        if (!allowed[block_of[j]]) continue;
        s[j] = exp(s[j] - m) / z;                       /* s now holds p_ij */
        const float* vj = v + RIX(b, j, h, 0);
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += (double)gi[d] * (double)vj[d];
        dp[j] = acc;
        delta += s[j] * acc;
    }
    /* a_i = sum_d |dout_id| sum_j p_ij |v_jd|: how far rounding the output o_i (or
       the probabilities forming it) can move delta_i, per unit of relative error */
    double a_i = 0.0;
    if (mq_row) {
        for (int d = 0; d < D; ++d) {
            double w = 0.0;
            for (int j = 0; j < N; ++j)
                if (allowed[block_of[j]]) w += s[j] * fabs((double)v[RIX(b, j, h, d)]);
            a_i += fabs((double)gi[d]) * w;
        }
    }
    for (int j = 0; j < N; ++j) {
        if (!allowed[block_of[j]]) continue;
        const double p = s[j], ds = p * (dp[j] - delta);
        const double mag = fabs(ds) + 0.25 * p * a_i;
        const float* kj = k + RIX(b, j, h, 0);
        for (int d = 0; d < D; ++d) dq_row[d] += scale * ds * (double)kj[d];
        if (dk) {
            double* dkj = dk + RIX(b, j, h, 0);
            double* dvj = dv + RIX(b, j, h, 0);
            for (int d = 0; d < D; ++d) {
                dkj[d] += scale * ds * (double)qi[d];
                dvj[d] += p * (double)gi[d];
            }
        }
        if (mq_row) {
            for (int d = 0; d < D; ++d) mq_row[d] += scale * mag * fabs((double)kj[d]);
            if (mk) {
                double* mkj = mk + RIX(b, j, h, 0);
                double* mvj = mv + RIX(b, j, h, 0);
                for (int d = 0; d < D; ++d) {
                    mkj[d] += scale * mag * fabs((double)qi[d]);
                    mvj[d] += p * fabs((double)gi[d]);
                }
            }
        }
    }
}

/*
 * Full gradients, raster [B, N, H, D] float64 each. When mq is given, mq / mk / mv
 * receive magnitude sums that bound each gradient element and scale how far
 * rounding can move it: with delta_i = sum_j p_ij dp_ij, a_i = sum_d |dout_id|
 * sum_j p_ij |v_jd| (rounding the probabilities that form o_i, or o_i itself, by a
 * relative eps moves delta_i by at most about eps a_i) and m_ij = |ds_ij| +
 * p_ij a_i / 4, mq = scale sum_j m_ij |k_jd|, mk = scale sum_i m_ij |q_id| and
 * mv = sum_i p_ij |dout_id|.
 */
void orc_masked_attention_bwd(const float* q, const float* k, const float* v, const float* dout,
                              int B, int N, int H, int D, const int32_t* block_of, int nb,
                              double scale, const int32_t* row_ptr, const int32_t* col_idx,
                              double* dq, double* dk, double* dv, double* mq, double* mk,
                              double* mv) {
    memset(dq, 0, sizeof(double) * (size_t)B * N * H * D);
    memset(dk, 0, sizeof(double) * (size_t)B * N * H * D);
    memset(dv, 0, sizeof(double) * (size_t)B * N * H * D);
    if (mq) {
        memset(mk, 0, sizeof(double) * (size_t)B * N * H * D);
        memset(mv, 0, sizeof(double) * (size_t)B * N * H * D);
    }
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            char* allowed = (char*)malloc((size_t)nb);
            double* s = (double*)malloc(sizeof(double) * (size_t)N);
            double* dp = (double*)malloc(sizeof(double) * (size_t)N);
            for (int i = 0; i < N; ++i) {
                const int64_t row = ((int64_t)b * H + h) * nb + block_of[i];
                memset(allowed, 0, (size_t)nb);
                for (int32_t e = row_ptr[row]; e < row_ptr[row + 1]; ++e)
                    if (col_idx[e] >= 0 && col_idx[e] < nb) allowed[col_idx[e]] = 1;
                bwd_one_query(q, k, v, dout, N, H, D, b, h, i, block_of, allowed, scale, s, dp,
                              dq + RIX(b, i, h, 0), dk, dv, mq ? mq + RIX(b, i, h, 0) : NULL, mk,
                              mv);
            }
            free(dp);
            free(s);
            free(allowed);
        }
}

/*
 * Query gradients only, for the requested query blocks (the key gradients of a
 * block need every query that keeps it, so sampled checks take dq). Layout as in
 * orc_masked_attention: dq_out [B, H, nsel, 64, D], token_of [B, H, nsel, 64];
 * mq_out (optional, same layout) receives the term magnitudes as above.
 */
void orc_masked_attention_bwd_dq(const float* q, const float* k, const float* v, const float* dout,
                                 int B, int N, int H, int D, const int32_t* block_of, int nb,
                                 double scale, const int32_t* row_ptr, const int32_t* col_idx,
                                 const int32_t* qblocks, int nsel, double* dq_out,
                                 double* mq_out, int32_t* token_of) {
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int r = 0; r < nsel; ++r) {
                const int qb = qblocks[r];
                const int64_t row = ((int64_t)b * H + h) * nb + qb;
                char* allowed = (char*)calloc((size_t)nb, 1);
                for (int32_t e = row_ptr[row]; e < row_ptr[row + 1]; ++e)
                    if (col_idx[e] >= 0 && col_idx[e] < nb) allowed[col_idx[e]] = 1;
                double* s = (double*)malloc(sizeof(double) * (size_t)N);
                double* dp = (double*)malloc(sizeof(double) * (size_t)N);
                const int64_t base = (((int64_t)b * H + h) * nsel + r) * 64;
                for (int e = 0; e < 64; ++e) {
                    token_of[base + e] = -1;
                    for (int d = 0; d < D; ++d) dq_out[(base + e) * D + d] = 0.0;
                    if (mq_out)
                        for (int d = 0; d < D; ++d) mq_out[(base + e) * D + d] = 0.0;
                }
                int e = 0;
                for (int i = 0; i < N && e < 64; ++i) {
                    if (block_of[i] != qb) continue;
                    token_of[base + e] = i;
                    bwd_one_query(q, k, v, dout, N, H, D, b, h, i, block_of, allowed, scale, s, dp,
                                  dq_out + (base + e) * D, NULL, NULL,
                                  mq_out ? mq_out + (base + e) * D : NULL, NULL, NULL);
                    e++;
                }
                free(dp);
                free(s);
                free(allowed);
            }
}

/*
 * Transpose of a block CSR per (b, h): for each key block kb, the query blocks whose
 * row keeps it, ascending (the column view the key-gradient pass walks). Out-of-range
 * indices are dropped and repeats collapse. col_ptr [B*H*nb + 1], row_idx [nnz].
 * Returns nnz.
 */
int64_t orc_csr_transpose(const int32_t* row_ptr, const int32_t* col_idx, int B, int H, int nb,
                          int32_t* col_ptr, int32_t* row_idx) {
    int64_t nnz = 0;
    char* keep = (char*)malloc((size_t)nb * (size_t)nb);
    col_ptr[0] = 0;
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        memset(keep, 0, (size_t)nb * (size_t)nb);
        for (int qb = 0; qb < nb; ++qb) {
            const int64_t row = bh * nb + qb;
            for (int32_t e = row_ptr[row]; e < row_ptr[row + 1]; ++e)
                if (col_idx[e] >= 0 && col_idx[e] < nb) keep[(size_t)col_idx[e] * nb + qb] = 1;
        }
        for (int kb = 0; kb < nb; ++kb) {
            for (int qb = 0; qb < nb; ++qb)
                if (keep[(size_t)kb * nb + qb]) row_idx[nnz++] = qb;
            col_ptr[bh * nb + kb + 1] = (int32_t)nnz;
        }
    }
    free(keep);
    return nnz;
}

/* ------------------------------------------------------------------------- */
/* Semantic (k-means) permutation                                             */
/* ------------------------------------------------------------------------- */

/*
 * Tokens clustered by the similarity of their own vectors and reordered so that each
 * cluster is contiguous, which both sharpens the cluster representation used to find
 * the critical tokens and packs those tokens densely for the kernel [Sparse
 * VideoGen2: Accelerate Video Generation with Sparse Attention via Semantic-Aware
 * Permutation, Abstract]. Plain Lloyd k-means per (b, h) over the N vectors
 * x[b, :, h, :], in float64:
 *   start: centroid c = x of token floor(c N / C);
 *   iters times: assign every token to the centroid at the least squared Euclidean
 *   distance sum_d (x_d - c_d)^2 (channels summed in order; ties to the lower
 *   cluster), then move every non-empty cluster's centroid to the mean of its
 *   members (summed in token order, divided by the count); an empty cluster keeps
 *   its centroid.
 * Inputs are finite.
 */

/* Squared Euclidean distance, summed over the channels in order. */
static double sqdist(const float* x, const double* c, int D) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) {
        const double t = (double)x[d] - c[d];
        s += t * t;
    }
    return s;
}

/* Unit roundoff of float64 and the bound gamma_n = n u / (1 - n u) on the relative
   error of an n-term float64 sum or dot product (Higham, Accuracy and Stability of
   Numerical Algorithms, section 3.1). */
static double gamma_n(double n) {
    const double u = 0x1p-53;
    return n * u / (1.0 - n * u);
}

/*
 * One assignment step against given centroids cent [B, H, C, D]: assign [B, H, N]
 * the nearest centroid (least sqdist, ties to the lower cluster).
 * If `other` is given (another evaluation's assignment [B, H, N]), excess[n] =
 * dist(other) - dist(best) as computed here, and tol[n] bounds how far an
 * evaluation of the two distances may be from the exact ones: the sum, over both
 * candidates, of this function's own error bound gamma_{D+2} * dist and that of the
 * form |c|^2 - 2 x.c (each product chain within gamma_D of its absolute sum, plus
 * one rounding of the difference). An assignment `other` is a valid nearest
 * centroid choice when excess[n] <= tol[n] for every token.
 */
void orc_kmeans_assign(const float* x, int B, int N, int H, int D, int C, const double* cent,
                       int32_t* assign, const int32_t* other, double* excess, double* tol) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int64_t bh = (int64_t)b * H + h;
            const double* cc = cent + bh * C * D;
            for (int n = 0; n < N; ++n) {
                const float* xn = x + RIX(b, n, h, 0);
                int best = 0;
                double bd = sqdist(xn, cc, D);
                for (int c = 1; c < C; ++c) {
                    const double dd = sqdist(xn, cc + (int64_t)c * D, D);
                    if (dd < bd) {
                        bd = dd;
                        best = c;
                    }
                }
                assign[bh * N + n] = best;
                if (other) {
                    const int o = other[bh * N + n];
                    const int pick[2] = {best, o};
                    double t = 0.0;
                    for (int i = 0; i < 2; ++i) {
                        const double* ci = cc + (int64_t)pick[i] * D;
                        double c2 = 0.0, xc = 0.0;
                        for (int d = 0; d < D; ++d) {
                            c2 += ci[d] * ci[d];
                            xc += fabs((double)xn[d] * ci[d]);
                        }
                        const double di = sqdist(xn, ci, D);
                        t += gamma_n(D + 2) * di + gamma_n(D + 1) * (c2 + 2.0 * xc) + 0x1p-52 * (c2 + 2.0 * xc);
                    }
                    excess[bh * N + n] = sqdist(xn, cc + (int64_t)o * D, D) - bd;
                    tol[bh * N + n] = t;
                }
            }
        }
}

/*
 * One update step: for every cluster of every (b, h), count[c] = its members under
 * assign [B, H, N], and cent_out[c] = the mean of their vectors (summed in token
 * order, then divided by the count), or cent_in[c] when the cluster is empty.
 * abs_sum [B, H, C, D] (optional) receives sum |x_d| over the members, from which a
 * caller bounds the rounding of any order of the member sum (gamma_{count-1} of it).
 */
void orc_kmeans_means(const float* x, int B, int N, int H, int D, int C, const int32_t* assign,
                      const double* cent_in, double* cent_out, int32_t* count, double* abs_sum) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int64_t bh = (int64_t)b * H + h;
            const int32_t* as = assign + bh * N;
            double* co = cent_out + bh * C * D;
            double* sum = (double*)calloc((size_t)C * D, sizeof(double));
            double* sabs = (double*)calloc((size_t)C * D, sizeof(double));
            int32_t* cn = count + bh * C;
            for (int c = 0; c < C; ++c) cn[c] = 0;
            for (int n = 0; n < N; ++n) {
                const int c = as[n];
                cn[c]++;
                for (int d = 0; d < D; ++d) {
                    sum[(int64_t)c * D + d] += (double)x[RIX(b, n, h, d)];
                    sabs[(int64_t)c * D + d] += fabs((double)x[RIX(b, n, h, d)]);
                }
            }
            for (int c = 0; c < C; ++c)
                for (int d = 0; d < D; ++d) {
                    const int64_t i = (int64_t)c * D + d;
                    co[i] = cn[c] ? sum[i] / (double)cn[c] : cent_in[bh * C * D + i];
                    if (abs_sum) abs_sum[bh * C * D + i] = sabs[i];
                }
            free(sum);
            free(sabs);
        }
}

/*
 * The whole clustering: assign [B, H, N], cent [B, H, C, D] float64 and count
 * [B, H, C] after `iters` Lloyd steps from the strided start (the last assignment
 * and the centroids and sizes that follow from it).
 */
void orc_kmeans(const float* x, int B, int N, int H, int D, int C, int iters, int32_t* assign,
                double* cent, int32_t* count) {
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < C; ++c) {
                const int64_t t = (int64_t)c * N / C;
                for (int d = 0; d < D; ++d)
                    cent[(((int64_t)b * H + h) * C + c) * D + d] = (double)x[RIX(b, t, h, d)];
            }
    const size_t ncent = (size_t)B * H * C * D;
    double* prev = (double*)malloc(ncent * sizeof(double));
    for (int it = 0; it < iters; ++it) {
        memcpy(prev, cent, ncent * sizeof(double));
        orc_kmeans_assign(x, B, N, H, D, C, prev, assign, NULL, NULL, NULL);
        orc_kmeans_means(x, B, N, H, D, C, assign, prev, cent, count, NULL);
    }
    free(prev);
}

/*
 * Cluster-contiguous block layout of one (b, h): cluster c's members, in token order,
 * fill blocks off[c] .. off[c+1]-1 (off[c+1] = off[c] + ceil(count_c / 64)), the last
 * block of a cluster padded. slot_token [B, H, NB*64] holds each slot's token (-1 for
 * padding), off [B, H, C+1], blk_count [B, H, NB] the real slots of each block (0 for
 * blocks past off[C]). Returns 0, or -1 if some head needs more than NB blocks.
 */
int orc_cluster_layout(const int32_t* assign, int B, int H, int N, int C, int NB,
                       int32_t* slot_token, int32_t* off, int32_t* blk_count) {
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const int32_t* as = assign + bh * N;
        int32_t* o = off + bh * (C + 1);
        int32_t* st = slot_token + bh * (int64_t)NB * 64;
        int32_t* bc = blk_count + bh * NB;
        for (int64_t e = 0; e < (int64_t)NB * 64; ++e) st[e] = -1;
        for (int i = 0; i < NB; ++i) bc[i] = 0;
        o[0] = 0;
        for (int c = 0; c < C; ++c) {
            int cnt = 0;
            for (int n = 0; n < N; ++n)
                if (as[n] == c) {
                    if (o[c] * 64 + cnt >= NB * 64) return -1;
                    st[(int64_t)o[c] * 64 + cnt] = n;
                    cnt++;
                }
            o[c + 1] = o[c] + (cnt + 63) / 64;
            if (o[c + 1] > NB) return -1;
            for (int i = o[c]; i < o[c + 1]; ++i) bc[i] = (cnt - 64 * (i - o[c])) < 64 ? cnt - 64 * (i - o[c]) : 64;
        }
    }
    return 0;
}

/*
 * Estimated attention mass between query cluster i and key cluster j, from the
 * cluster representation: each key cluster stands for count_j keys at its centroid,
 * so est[i, j] = n_j exp(scale cq_i . ck_j) / sum_j' n_j' exp(scale cq_i . ck_j') over
 * non-empty key clusters (the dot product summed over channels in order, the
 * exponent taken relative to the row maximum). Rows of empty query clusters are 0.
 * est [B, H, Cq, Ck] float64.
 */
void orc_cluster_mass(const double* cq, const int32_t* nq, const double* ck, const int32_t* nk,
                      int B, int H, int Cq, int Ck, int D, double scale, double* est) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh)
        for (int i = 0; i < Cq; ++i) {
            double* row = est + (bh * Cq + i) * Ck;
            for (int j = 0; j < Ck; ++j) row[j] = 0.0;
            if (nq[bh * Cq + i] == 0) continue;
            const double* qi = cq + (bh * Cq + i) * D;
            double m = -INFINITY;
            for (int j = 0; j < Ck; ++j) {
                if (nk[bh * Ck + j] == 0) continue;
                const double* kj = ck + (bh * Ck + j) * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d) s = s + qi[d] * kj[d];
                row[j] = scale * s;
                if (row[j] > m) m = row[j];
            }
            double z = 0.0;
            for (int j = 0; j < Ck; ++j) {
                if (nk[bh * Ck + j] == 0) continue;
                row[j] = (double)nk[bh * Ck + j] * exp(row[j] - m);
                z += row[j];
            }
            for (int j = 0; j < Ck; ++j) row[j] = nk[bh * Ck + j] ? row[j] / z : 0.0;
        }
}

/*
 * Block CSR of the cluster selection: query block qb of (b, h) lies in query cluster
 * i when qoff[i] <= qb < qoff[i+1]; it keeps every block of every key cluster j that
 * cluster row (b*H + h)*Cq + i keeps, i.e. blocks koff[j] .. koff[j+1]-1, in the
 * row's order. Blocks past qoff[Cq] keep nothing. Rows (b*H + h)*NB + qb. Returns nnz.
 */
int64_t orc_cluster_blocks(const int32_t* crow_ptr, const int32_t* ccol_idx, const int32_t* qoff,
                           const int32_t* koff, int B, int H, int Cq, int Ck, int NB,
                           int32_t* row_ptr, int32_t* col_idx) {
    int64_t nnz = 0;
    row_ptr[0] = 0;
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const int32_t* qo = qoff + bh * (Cq + 1);
        const int32_t* ko = koff + bh * (Ck + 1);
        for (int qb = 0; qb < NB; ++qb) {
            int ci = -1;
            for (int i = 0; i < Cq; ++i)
                if (qo[i] <= qb && qb < qo[i + 1]) ci = i;
            if (ci >= 0) {
                const int64_t r = bh * Cq + ci;
                for (int32_t e = crow_ptr[r]; e < crow_ptr[r + 1]; ++e) {
                    const int j = ccol_idx[e];
                    for (int kb = ko[j]; kb < ko[j + 1]; ++kb) col_idx[nnz++] = kb;
                }
            }
            row_ptr[bh * NB + qb + 1] = (int32_t)nnz;
        }
    }
    return nnz;
}

/*
 * Attention under a cluster selection: query token n of (b, h), in query cluster
 * qassign[n], attends to the keys whose key cluster the cluster row (b*H + h)*Cq +
 * qassign[n] keeps, with the softmax over exactly those keys (zero output when
 * none). With tokens == NULL, out is raster [B, N, H, D] float64; otherwise only the
 * ntok listed query tokens are computed, into out [B, H, ntok, D].
 */
void orc_cluster_attention(const float* q, const float* k, const float* v, int B, int N, int H,
                           int D, const int32_t* qassign, const int32_t* kassign, int Cq, int Ck,
                           double scale, const int32_t* crow_ptr, const int32_t* ccol_idx,
                           const int32_t* tokens, int ntok, double* out) {
    const int count = tokens ? ntok : N;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int u = 0; u < count; ++u) {
                const int n = tokens ? tokens[u] : u;
                const int64_t bh = (int64_t)b * H + h;
                const int64_t r = bh * Cq + qassign[bh * N + n];
                char* allowed = (char*)calloc((size_t)Ck, 1);
                for (int32_t e = crow_ptr[r]; e < crow_ptr[r + 1]; ++e)
                    if (ccol_idx[e] >= 0 && ccol_idx[e] < Ck) allowed[ccol_idx[e]] = 1;
                double* o = tokens ? out + (bh * ntok + u) * D : out + RIX(b, n, h, 0);
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                double* s = (double*)malloc(sizeof(double) * (size_t)N);
                double m = -INFINITY;
                for (int j = 0; j < N; ++j) {
                    if (!allowed[kassign[bh * N + j]]) continue;
                    s[j] = dot_scaled(q + RIX(b, n, h, 0), k + RIX(b, j, h, 0), D, scale);
                    if (s[j] > m) m = s[j];
                }
                if (m != -INFINITY) {
                    double z = 0.0;
                    for (int j = 0; j < N; ++j)
                        if (allowed[kassign[bh * N + j]]) z += exp(s[j] - m);
                    for (int j = 0; j < N; ++j) {
                        if (!allowed[kassign[bh * N + j]]) continue;
                        const double p = exp(s[j] - m) / z;
                        for (int d = 0; d < D; ++d) o[d] += p * (double)v[RIX(b, j, h, d)];
                    }
                }
                free(s);
                free(allowed);
            }
}
