// C ABI of the block-sparse attention library (declared in include/fpsa.h).
// Every argument is checked on the host before anything is enqueued; kernels are
// launched asynchronously on the caller's stream and launch errors come back as
// FPSA_ERR_HIP. No device memory is allocated and no state is kept between calls.
#include <hip/hip_runtime.h>

#include "fpsa.h"
#include "fpsa_internal.h"

using fpsa::Geom;

namespace {

bool make_geom(const fpsa_grid* g, Geom* out) {
    if (g == nullptr) return false;
    if (g->t <= 0 || g->h <= 0 || g->w <= 0) return false;
    if (g->tile_t <= 0 || g->tile_h <= 0 || g->tile_w <= 0) return false;
    if ((long)g->tile_t * g->tile_h * g->tile_w != fpsa::kBlock) return false;
    Geom r;
    r.T = g->t; r.Hg = g->h; r.Wg = g->w;
    r.tt = g->tile_t; r.th = g->tile_h; r.tw = g->tile_w;
    r.nt = (g->t + g->tile_t - 1) / g->tile_t;
    r.nh = (g->h + g->tile_h - 1) / g->tile_h;
    r.nw = (g->w + g->tile_w - 1) / g->tile_w;
    long nb = (long)r.nt * r.nh * r.nw;
    if (nb > (1L << 24)) return false;                  // keeps 64*nb and grid sizes in range
    r.nb = (int)nb;
    *out = r;
    return true;
}

int32_t hip_status() {
    return hipGetLastError() == hipSuccess ? FPSA_OK : FPSA_ERR_HIP;
}

bool dims_ok(int32_t B, int32_t H) { return B >= 1 && H >= 1 && B <= 65535 && H <= 65535; }

}  // namespace

extern "C" {

int32_t fpsa_version(void) { return 100; }

int32_t fpsa_num_blocks(const fpsa_grid* g) {
    Geom geo;
    if (!make_geom(g, &geo)) return -1;
    return geo.nb;
}

const char* fpsa_status_string(int32_t s) {
    switch (s) {
        case FPSA_OK: return "ok";
        case FPSA_ERR_INVALID_ARG: return "invalid argument";
        case FPSA_ERR_UNSUPPORTED: return "unsupported configuration";
        case FPSA_ERR_CAPACITY: return "output capacity too small";
        case FPSA_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

size_t fpsa_select_workspace_bytes(int64_t R, int32_t nb) {
    if (R <= 0 || nb <= 0) return 0;
    return fpsa::select_workspace_bytes((long)R);
}

int32_t fpsa_tile_reorder(const void* src, int32_t src_dtype, void* dst, int32_t dst_dtype,
                          int32_t dst_layout, float* dst_scale, int32_t B, int32_t H, int32_t D,
                          const fpsa_grid* g, int32_t inverse, void* stream) {
    Geom geo;
    if (!make_geom(g, &geo) || !dims_ok(B, H)) return FPSA_ERR_INVALID_ARG;
    if (src == nullptr || dst == nullptr) return FPSA_ERR_INVALID_ARG;
    if (inverse != 0 && inverse != 1) return FPSA_ERR_INVALID_ARG;
    if (dst_layout != FPSA_LAYOUT_ROWS && dst_layout != FPSA_LAYOUT_VT && dst_layout != FPSA_LAYOUT_QK)
        return FPSA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    const long N = (long)g->t * g->h * g->w;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (inverse) {
        if (src_dtype != FPSA_BF16 || dst_layout != FPSA_LAYOUT_ROWS) return FPSA_ERR_UNSUPPORTED;
        if (dst_dtype != FPSA_F32 && dst_dtype != FPSA_BF16) return FPSA_ERR_UNSUPPORTED;
        if (dst_scale != nullptr) return FPSA_ERR_INVALID_ARG;
        fpsa::launch_tile_inverse(src, dst, dst_dtype == FPSA_F32 ? 0 : 1, geo, N, B, H, D, st);
        return hip_status();
    }
    if (src_dtype != FPSA_F32 && src_dtype != FPSA_BF16) return FPSA_ERR_UNSUPPORTED;
    int fp8;
    if (dst_dtype == FPSA_BF16) {
        if (dst_scale != nullptr) return FPSA_ERR_INVALID_ARG;
        fp8 = 0;
    } else if (dst_dtype == FPSA_FP8_E4M3) {
        if (dst_scale == nullptr) return FPSA_ERR_INVALID_ARG;
        if (dst_layout == FPSA_LAYOUT_VT) return FPSA_ERR_UNSUPPORTED;
        fp8 = 1;
    } else {
        return FPSA_ERR_UNSUPPORTED;
    }
    fpsa::launch_tile_forward(src, src_dtype == FPSA_F32 ? 0 : 1, dst, fp8, dst_layout, dst_scale, geo,
                              N, B, H, D, st);
    return hip_status();
}

int32_t fpsa_dequantize_tiles(const void* src, const float* scale, int32_t B, int32_t H, int32_t D,
                              const fpsa_grid* g, void* dst, void* stream) {
    Geom geo;
    if (!make_geom(g, &geo) || !dims_ok(B, H)) return FPSA_ERR_INVALID_ARG;
    if (src == nullptr || dst == nullptr) return FPSA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    const long blocks = (long)B * H * geo.nb;
    if (blocks > 0x7FFFFFFFL) return FPSA_ERR_UNSUPPORTED;
    fpsa::launch_dequant_tiles(src, scale, dst, blocks, D, static_cast<hipStream_t>(stream));
    return hip_status();
}

size_t fpsa_transpose_workspace_bytes(int64_t R, int32_t nb) {
    if (R <= 0 || nb <= 0 || R > (1L << 24)) return 0;
    return fpsa::transpose_workspace_bytes((long)R, nb);
}

size_t fpsa_bwd_workspace_bytes(int32_t B, int32_t H, const fpsa_grid* g) {
    Geom geo;
    if (!make_geom(g, &geo) || !dims_ok(B, H)) return 0;
    return fpsa::bwd_workspace_bytes(B, H, geo.nb);
}

size_t fpsa_mass_workspace_bytes(int32_t B, int32_t H, const fpsa_grid* g) {
    Geom geo;
    if (!make_geom(g, &geo) || !dims_ok(B, H)) return 0;
    return fpsa::mass_workspace_bytes_all(B, H, geo.nb);
}

int32_t fpsa_block_mass(const void* q_tiled, const void* k_tiled, int32_t B, int32_t H, int32_t D,
                        const fpsa_grid* g, float softmax_scale, float* mass, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
    Geom geo;
    if (!make_geom(g, &geo) || !dims_ok(B, H)) return FPSA_ERR_INVALID_ARG;
    if (q_tiled == nullptr || k_tiled == nullptr || mass == nullptr || workspace == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return FPSA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    if (geo.nb > FPSA_MAX_SELECT_BLOCKS) return FPSA_ERR_UNSUPPORTED;
    if ((long)B * H * geo.nb > 0x7FFFFFFFL) return FPSA_ERR_UNSUPPORTED;
    if (workspace_bytes < fpsa::mass_workspace_bytes_min(geo.nb)) return FPSA_ERR_CAPACITY;
    fpsa::launch_block_mass(q_tiled, k_tiled, B, H, D, geo, softmax_scale, mass, lse, workspace,
                            workspace_bytes, static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_select_blocks(const float* mass, int64_t R, int32_t nb, uint32_t thr_num,
                           uint32_t thr_den, int32_t* row_ptr, int32_t* col_idx,
                           int64_t col_capacity, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (mass == nullptr || row_ptr == nullptr || col_idx == nullptr || workspace == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (R <= 0 || R > (1L << 24) || nb <= 0) return FPSA_ERR_INVALID_ARG;
    if (nb > FPSA_MAX_SELECT_BLOCKS) return FPSA_ERR_UNSUPPORTED;
    if (thr_den < 1 || thr_den > 1000 || thr_num > thr_den) return FPSA_ERR_INVALID_ARG;
    if ((int64_t)R * nb > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;   // nnz must fit int32
    if (col_capacity < (int64_t)R * nb) return FPSA_ERR_CAPACITY;
    if (workspace_bytes < fpsa::select_workspace_bytes((long)R)) return FPSA_ERR_CAPACITY;
    fpsa::launch_select(mass, (long)R, nb, thr_num, thr_den, row_ptr, col_idx, workspace,
                        static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_select_blocks_noalloc(const float* mass, int64_t R, int32_t nb, uint32_t thr_num,
                                   uint32_t thr_den, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, void* stream) {
    if (mass == nullptr || row_ptr == nullptr || col_idx == nullptr) return FPSA_ERR_INVALID_ARG;
    if (R <= 0 || R > (1L << 24) || nb <= 0) return FPSA_ERR_INVALID_ARG;
    if (nb > FPSA_MAX_SELECT_BLOCKS) return FPSA_ERR_UNSUPPORTED;
    if (thr_den < 1 || thr_den > 1000 || thr_num > thr_den) return FPSA_ERR_INVALID_ARG;
    if ((int64_t)R * nb > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    if (col_capacity < (int64_t)R * nb) return FPSA_ERR_CAPACITY;
    if (R > FPSA_SELECT_NOALLOC_MAX_ROWS) return FPSA_ERR_CAPACITY;   // beyond the static scratch
    static_assert(FPSA_SELECT_NOALLOC_MAX_ROWS == fpsa::kSelectNoAllocMaxRows, "one limit");
    void* ws = nullptr;
    if (fpsa::select_scratch(&ws) != hipSuccess) return FPSA_ERR_HIP;
    fpsa::launch_select(mass, (long)R, nb, thr_num, thr_den, row_ptr, col_idx, ws,
                        static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_structured_mask(const fpsa_grid* g, int32_t copies, int32_t* row_ptr,
                             int32_t* col_idx, int64_t col_capacity, void* workspace,
                             size_t workspace_bytes, void* stream) {
    Geom geo;
    if (!make_geom(g, &geo)) return FPSA_ERR_INVALID_ARG;
    if (copies < 1 || row_ptr == nullptr || col_idx == nullptr || workspace == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (geo.nt != 1) return FPSA_ERR_UNSUPPORTED;          // a 2D grid of groups only
    const int64_t R = (int64_t)copies * geo.nb;
    if (R > (1L << 24)) return FPSA_ERR_UNSUPPORTED;
    const int64_t need = R * (int64_t)(geo.nh + geo.nw + 9);
    if (need > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    if (col_capacity < need) return FPSA_ERR_CAPACITY;
    if (workspace_bytes < fpsa::select_workspace_bytes((long)R)) return FPSA_ERR_CAPACITY;
    fpsa::launch_structured(geo, copies, row_ptr, col_idx, workspace,
                            static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_pattern_mask(const fpsa_grid* g, int32_t B, int32_t H, const int32_t* patterns,
                          int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                          void* workspace, size_t workspace_bytes, void* stream) {
    Geom geo;
    if (!make_geom(g, &geo) || !dims_ok(B, H)) return FPSA_ERR_INVALID_ARG;
    if (patterns == nullptr || row_ptr == nullptr || col_idx == nullptr || workspace == nullptr)
        return FPSA_ERR_INVALID_ARG;
    const int64_t R = (int64_t)B * H * geo.nb;
    if (R > (1L << 24)) return FPSA_ERR_UNSUPPORTED;
    const int64_t need = R * (int64_t)geo.nb;
    if (need > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    if (col_capacity < need) return FPSA_ERR_CAPACITY;
    if (workspace_bytes < fpsa::select_workspace_bytes((long)R)) return FPSA_ERR_CAPACITY;
    fpsa::launch_pattern(geo.nb, B, H, patterns, row_ptr, col_idx, workspace,
                         static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_retained_mass(const float* mass, int64_t R, int32_t nb, const int32_t* row_ptr,
                           const int32_t* col_idx, float* retained, void* stream) {
    if (mass == nullptr || row_ptr == nullptr || col_idx == nullptr || retained == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (R <= 0 || R > (1L << 24) || nb <= 0) return FPSA_ERR_INVALID_ARG;
    if (nb > FPSA_MAX_SELECT_BLOCKS) return FPSA_ERR_UNSUPPORTED;
    fpsa::launch_retained_mass(mass, (long)R, nb, row_ptr, col_idx, retained,
                               static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_sparse_attn_fwd(const void* q, const void* k, const void* v, int32_t qk_dtype,
                             const float* q_scale, const float* k_scale, const int32_t* row_ptr,
                             const int32_t* col_idx, int32_t B, int32_t H, int32_t D,
                             const fpsa_grid* g, float softmax_scale, void* o, float* lse,
                             float* o_f32, void* stream) {
    Geom geo;
    if (!make_geom(g, &geo) || !dims_ok(B, H)) return FPSA_ERR_INVALID_ARG;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FPSA_ERR_INVALID_ARG;
    if (row_ptr == nullptr || col_idx == nullptr) return FPSA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return FPSA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    if ((long)B * H * geo.nb > 0x7FFFFFFFL) return FPSA_ERR_UNSUPPORTED;
    if ((long)geo.nb * fpsa::kBlock * D * 2 > 0x7FFFFFFFL) return FPSA_ERR_UNSUPPORTED;   // 32-bit tile offsets
    int fp8;
    if (qk_dtype == FPSA_BF16) {
        if (q_scale != nullptr || k_scale != nullptr) return FPSA_ERR_INVALID_ARG;
        fp8 = 0;
    } else if (qk_dtype == FPSA_FP8_E4M3) {
        if (q_scale == nullptr || k_scale == nullptr) return FPSA_ERR_INVALID_ARG;
        fp8 = 1;
    } else {
        return FPSA_ERR_UNSUPPORTED;
    }
    fpsa::launch_sparse_attn(q, k, v, fp8, q_scale, k_scale, row_ptr, col_idx, B, H, D, geo,
                             softmax_scale, o, lse, o_f32, nullptr, static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_csr_transpose(const int32_t* row_ptr, const int32_t* col_idx, int32_t B, int32_t H,
                           int32_t nb, int32_t* col_ptr, int32_t* row_idx, int64_t capacity,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (row_ptr == nullptr || col_idx == nullptr || col_ptr == nullptr || row_idx == nullptr ||
        workspace == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (!dims_ok(B, H) || nb <= 0) return FPSA_ERR_INVALID_ARG;
    const int64_t R = (int64_t)B * H * nb;
    if (R > (1L << 24)) return FPSA_ERR_UNSUPPORTED;
    if (R * nb > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    if (capacity < R * nb) return FPSA_ERR_CAPACITY;
    if (workspace_bytes < fpsa::transpose_workspace_bytes((long)R, nb)) return FPSA_ERR_CAPACITY;
    fpsa::launch_csr_transpose(row_ptr, col_idx, (long)R, nb, col_ptr, row_idx, workspace,
                               static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                             int32_t o_dtype, const void* dout, const float* lse, const int32_t* row_ptr,
                             const int32_t* col_idx, const int32_t* col_ptr,
                             const int32_t* row_idx, const float* q_scale, const float* k_scale,
                             int32_t B, int32_t H, int32_t D,
                             const fpsa_grid* g, float softmax_scale, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, void* stream) {
    Geom geo;
    if (!make_geom(g, &geo) || !dims_ok(B, H)) return FPSA_ERR_INVALID_ARG;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr ||
        lse == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (row_ptr == nullptr || col_idx == nullptr || col_ptr == nullptr || row_idx == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (dq == nullptr || dk == nullptr || dv == nullptr || workspace == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return FPSA_ERR_INVALID_ARG;
    if (o_dtype != FPSA_BF16 && o_dtype != FPSA_F32) return FPSA_ERR_UNSUPPORTED;
    if ((q_scale == nullptr) != (k_scale == nullptr)) return FPSA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    if ((long)B * H * geo.nb > 0x7FFFFFFFL) return FPSA_ERR_UNSUPPORTED;
    if (workspace_bytes < fpsa::bwd_workspace_bytes(B, H, geo.nb)) return FPSA_ERR_CAPACITY;
    fpsa::launch_sparse_attn_bwd(q, k, v, o, dout, lse, row_ptr, col_idx, col_ptr, row_idx, q_scale, k_scale,
                                 B, H, D,
                                 geo, softmax_scale, o_dtype == FPSA_F32, dq, dk, dv, workspace,
                                 static_cast<hipStream_t>(stream));
    return hip_status();
}

size_t fpsa_kmeans_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t C) {
    if (B < 1 || H < 1 || N < 1 || C < 1) return 0;
    return fpsa::kmeans_workspace_bytes(B, H, N, C);
}

int32_t fpsa_kmeans(const void* x, int32_t x_dtype, int32_t B, int32_t N, int32_t H, int32_t D,
                    int32_t C, int32_t iters, int32_t* assign, double* centroids, int32_t* counts,
                    int32_t* member_off, int32_t* members, void* workspace, size_t workspace_bytes,
                    void* stream) {
    if (x == nullptr || assign == nullptr || centroids == nullptr || counts == nullptr ||
        member_off == nullptr || members == nullptr || workspace == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (!dims_ok(B, H) || N < 1 || C < 1 || C > N || iters < 1 || iters > 1000)
        return FPSA_ERR_INVALID_ARG;
    if (x_dtype != FPSA_F32 && x_dtype != FPSA_BF16) return FPSA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    if (C > FPSA_MAX_SELECT_BLOCKS) return FPSA_ERR_UNSUPPORTED;
    if ((int64_t)B * H * N > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    if (workspace_bytes < fpsa::kmeans_workspace_bytes(B, H, N, C)) return FPSA_ERR_CAPACITY;
    fpsa::launch_kmeans(x, x_dtype == FPSA_F32, B, N, H, D, C, iters, assign, centroids, counts, member_off,
                        members, workspace, static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_cluster_layout(const int32_t* member_off, const int32_t* members, int32_t B, int32_t H,
                            int32_t N, int32_t C, int32_t NB, int32_t* slot_token, int32_t* blk_off,
                            int32_t* blk_count, void* stream) {
    if (member_off == nullptr || members == nullptr || slot_token == nullptr || blk_off == nullptr ||
        blk_count == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (!dims_ok(B, H) || N < 1 || C < 1 || C > N || NB < 1) return FPSA_ERR_INVALID_ARG;
    if (C > FPSA_MAX_SELECT_BLOCKS) return FPSA_ERR_UNSUPPORTED;
    if ((int64_t)NB < ((int64_t)N + 63) / 64 + C) return FPSA_ERR_CAPACITY;
    if ((int64_t)B * H * NB * 64 > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    fpsa::launch_cluster_layout(member_off, members, B, H, C, NB, slot_token, blk_off, blk_count,
                                static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_gather_tiles(const void* src, int32_t src_dtype, const int32_t* slot_token, int32_t B,
                          int32_t N, int32_t H, int32_t D, int32_t NB, int32_t layout, void* dst,
                          void* stream) {
    if (src == nullptr || slot_token == nullptr || dst == nullptr) return FPSA_ERR_INVALID_ARG;
    if (!dims_ok(B, H) || N < 1 || NB < 1) return FPSA_ERR_INVALID_ARG;
    if (layout != FPSA_LAYOUT_ROWS && layout != FPSA_LAYOUT_VT && layout != FPSA_LAYOUT_QK)
        return FPSA_ERR_INVALID_ARG;
    if (src_dtype != FPSA_F32 && src_dtype != FPSA_BF16) return FPSA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    if (NB > 65535 || (int64_t)B * H * NB * 64 > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    fpsa::launch_gather_tiles(src, src_dtype == FPSA_F32 ? 0 : 1, slot_token, NB, dst, layout, N, B, H, D,
                              static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_scatter_tiles(const void* src, const int32_t* slot_token, int32_t B, int32_t N, int32_t H,
                           int32_t D, int32_t NB, void* dst, int32_t dst_dtype, void* stream) {
    if (src == nullptr || slot_token == nullptr || dst == nullptr) return FPSA_ERR_INVALID_ARG;
    if (!dims_ok(B, H) || N < 1 || NB < 1) return FPSA_ERR_INVALID_ARG;
    if (dst_dtype != FPSA_F32 && dst_dtype != FPSA_BF16) return FPSA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    if (NB > 65535 || (int64_t)B * H * NB * 64 > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    fpsa::launch_scatter_tiles(src, slot_token, NB, dst, dst_dtype == FPSA_F32 ? 0 : 1, N, B, H, D,
                               static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_cluster_mass(const double* cq, const int32_t* nq, const double* ck, const int32_t* nk,
                          int32_t B, int32_t H, int32_t Cq, int32_t Ck, int32_t D, float softmax_scale,
                          float* est, void* stream) {
    if (cq == nullptr || nq == nullptr || ck == nullptr || nk == nullptr || est == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (!dims_ok(B, H) || Cq < 1 || Ck < 1) return FPSA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return FPSA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    if (Ck > FPSA_MAX_SELECT_BLOCKS || (int64_t)B * H * Cq > (1L << 24)) return FPSA_ERR_UNSUPPORTED;
    fpsa::launch_cluster_mass(cq, nq, ck, nk, B, H, Cq, Ck, D, (double)softmax_scale, est,
                              static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_cluster_blocks(const int32_t* crow_ptr, const int32_t* ccol_idx, const int32_t* qoff,
                            const int32_t* koff, int32_t B, int32_t H, int32_t Cq, int32_t Ck,
                            int32_t NB, int32_t* row_ptr, int32_t* col_idx, int64_t capacity,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (crow_ptr == nullptr || ccol_idx == nullptr || qoff == nullptr || koff == nullptr ||
        row_ptr == nullptr || col_idx == nullptr || workspace == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (!dims_ok(B, H) || Cq < 1 || Ck < 1 || NB < 1) return FPSA_ERR_INVALID_ARG;
    const int64_t R = (int64_t)B * H * NB;
    if (R > (1L << 24) || R * NB > 0x7FFFFFFFLL) return FPSA_ERR_UNSUPPORTED;
    if (capacity < R * NB) return FPSA_ERR_CAPACITY;
    if (workspace_bytes < (size_t)R * 4) return FPSA_ERR_CAPACITY;
    fpsa::launch_cluster_blocks(crow_ptr, ccol_idx, qoff, koff, B, H, Cq, Ck, NB, row_ptr, col_idx,
                                static_cast<int32_t*>(workspace), static_cast<hipStream_t>(stream));
    return hip_status();
}

int32_t fpsa_sparse_attn_fwd_varlen(const void* q, const void* k, const void* v,
                                    const int32_t* key_counts, const int32_t* row_ptr,
                                    const int32_t* col_idx, int32_t B, int32_t H, int32_t D,
                                    int32_t NB, float softmax_scale, void* o, float* lse,
                                    float* o_f32, void* stream) {
    if (q == nullptr || k == nullptr || v == nullptr || key_counts == nullptr || row_ptr == nullptr ||
        col_idx == nullptr || o == nullptr)
        return FPSA_ERR_INVALID_ARG;
    if (!dims_ok(B, H) || NB < 1 || NB > (1 << 24)) return FPSA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY) return FPSA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FPSA_ERR_UNSUPPORTED;
    if ((long)B * H * NB > 0x7FFFFFFFL) return FPSA_ERR_UNSUPPORTED;
    if ((long)NB * fpsa::kBlock * D * 2 > 0x7FFFFFFFL) return FPSA_ERR_UNSUPPORTED;       // 32-bit tile offsets
    // the blocks as one flat row of 64-token tiles: every slot is a query slot
    fpsa_grid flat = {1, 1, 64 * NB, 1, 1, 64};
    Geom geo;
    if (!make_geom(&flat, &geo)) return FPSA_ERR_INVALID_ARG;
    fpsa::launch_sparse_attn(q, k, v, 0, nullptr, nullptr, row_ptr, col_idx, B, H, D, geo, softmax_scale, o,
                             lse, o_f32, key_counts, static_cast<hipStream_t>(stream));
    return hip_status();
}

}  // extern "C"
