// Kernel launchers behind the C ABI (host side). Arguments are validated by the
// caller in api.hip before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fpsa_device.h"

namespace fpsa {

// layout: 0 rows, 1 VT, 2 QK (fpsa_layout values)
void launch_dequant_tiles(const void* src, const float* scale, void* dst, long blocks, int D, hipStream_t st);
void launch_tile_forward(const void* src, int src_dt, void* dst, int fp8, int layout, float* scale,
                         const Geom& g, long N, int B, int H, int D, hipStream_t st);
void launch_tile_inverse(const void* src, void* dst, int dst_dt, const Geom& g, long N, int B,
                         int H, int D, hipStream_t st);
// The same moves driven by an explicit slot map [B*H, nblocks*64] (token or -1).
void launch_gather_tiles(const void* src, int src_dt, const int32_t* slot_token, int nblocks, void* dst,
                         int layout, long N, int B, int H, int D, hipStream_t st);
void launch_scatter_tiles(const void* src, const int32_t* slot_token, int nblocks, void* dst, int dst_dt,
                          long N, int B, int H, int D, hipStream_t st);

// Workspace of the mass pass: nb * 64 floats per query-block row in flight; rows
// are processed in launches of as many rows as the workspace holds.
size_t mass_workspace_bytes_per_row(int nb);
// The mass pass takes query blocks in pairs: the smallest workspace holds one pair,
// the full one every pair of every (batch, head).
size_t mass_workspace_bytes_min(int nb);
size_t mass_workspace_bytes_all(int B, int H, int nb);
void launch_block_mass(const void* q, const void* k, int B, int H, int D, const Geom& g,
                       float scale, float* mass, float* lse, void* ws, size_t ws_bytes,
                       hipStream_t st);

// Workspace layout for selection: per row a kept count (int32) and the cut key
// (uint64) with the number of tied keys kept (int32).
size_t select_workspace_bytes(long R);
// Rows the no-allocation selection entry point accepts; its file-scope device scratch
// holds select_workspace_bytes(kSelectNoAllocMaxRows) bytes on every GPU it runs on.
constexpr long kSelectNoAllocMaxRows = 1L << 20;
// The address of that scratch on the current device (looked up once per device).
hipError_t select_scratch(void** out);
void launch_select(const float* mass, long R, int nb, uint32_t num, uint32_t den, int32_t* row_ptr,
                   int32_t* col_idx, void* ws, hipStream_t st);
void launch_structured(const Geom& g, int copies, int32_t* row_ptr, int32_t* col_idx, void* ws,
                       hipStream_t st);
void launch_pattern(int nb, int B, int H, const int32_t* patterns, int32_t* row_ptr,
                    int32_t* col_idx, void* ws, hipStream_t st);
void launch_retained_mass(const float* mass, long R, int nb, const int32_t* row_ptr,
                          const int32_t* col_idx, float* out, hipStream_t st);

// Exclusive scan of R counts into out[R + 1] (one workgroup).
void launch_scan(const int32_t* count, long R, int32_t* out, hipStream_t st);

// k-means semantic permutation (cluster.hip).
size_t kmeans_workspace_bytes(int B, int H, int N, int C);
void launch_kmeans(const void* x, int x_f32, int B, int N, int H, int D, int C, int iters, int32_t* assign,
                   double* cent, int32_t* count, int32_t* off, int32_t* members, void* ws, hipStream_t st);
void launch_cluster_layout(const int32_t* off, const int32_t* members, int B, int H, int C, int nblocks,
                           int32_t* slot_token, int32_t* blk_off, int32_t* blk_count, hipStream_t st);
void launch_cluster_mass(const double* cq, const int32_t* nq, const double* ck, const int32_t* nk, int B, int H,
                         int Cq, int Ck, int D, double scale, float* est, hipStream_t st);
void launch_cluster_blocks(const int32_t* crow_ptr, const int32_t* ccol_idx, const int32_t* qoff,
                           const int32_t* koff, int B, int H, int Cq, int Ck, int NB, int32_t* row_ptr,
                           int32_t* col_idx, int32_t* count, hipStream_t st);

// CSR transpose: a bitmap of R * ceil(nb/32) words and R column counts.
size_t transpose_workspace_bytes(long R, int nb);
void launch_csr_transpose(const int32_t* row_ptr, const int32_t* col_idx, long R, int nb,
                          int32_t* col_ptr, int32_t* row_idx, void* ws, hipStream_t st);

// Backward: lse in base 2 and delta = dO.O per query slot (2 floats per slot).
size_t bwd_workspace_bytes(int B, int H, int nb);
void launch_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, const int32_t* row_ptr,
                            const int32_t* col_idx, const int32_t* col_ptr, const int32_t* row_idx,
                            const float* q_scale, const float* k_scale, int B, int H, int D, const Geom& g,
                            float scale, int o_f32, void* dq, void* dk, void* dv, void* ws, hipStream_t st);

void launch_sparse_attn(const void* q, const void* k, const void* v, int fp8, const float* q_scale,
                        const float* k_scale, const int32_t* row_ptr, const int32_t* col_idx,
                        int B, int H, int D, const Geom& g, float scale, void* o, float* lse,
                        float* o32, const int32_t* kcount, hipStream_t st);

}  // namespace fpsa
