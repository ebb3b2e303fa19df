/*
 * fpsa.h - block-sparse attention over 3D-tiled token sequences, for AMD MI355X (gfx950).
 *
 * The method: tokens of a video latent (or image) are grouped into 64-token tiles,
 * which serve both as the unit of sparsity and the unit of FP8 quantization
 * [FPSAttention: Training-Aware FP8 and Sparsity Co-Design for Fast Video Diffusion,
 * Abstract]. One dense step measures the exact softmax attention mass between every
 * query tile and key tile; for each head and query tile the smallest set of key
 * tiles holding 99 % of that mass is kept, and those frozen indices drive every
 * later step [LoSA: Near-Lossless Sparse Attention for Training-Free Video
 * Diffusion Acceleration, Abstract]. Attention then visits only kept tiles with an
 * online softmax (FlashAttention style). A fixed structured key set shared by each
 * query group (neighbouring groups plus the group's row and column) can replace the
 * measured selection [Grouping First, Attending Smartly: Training-Free Acceleration
 * for Diffusion Transformers, Abstract], as can fixed per-head diagonal,
 * multi-diagonal and vertical-stripe patterns [Sparse-vDiT: Unleashing the Power of
 * Sparse Attention to Accelerate Video Diffusion Transformers, Abstract]. A monitor
 * reports how much of a later step's mass the frozen indices still retain, and a
 * backward pass gives the gradients over the same blocks. A k-means semantic
 * permutation with centroid-based top-p cluster selection is the adaptive
 * alternative [Sparse VideoGen2: Accelerate Video Generation with Sparse Attention
 * via Semantic-Aware Permutation, Abstract].
 *
 * Conventions for every call:
 *   - Data pointers are DEVICE pointers owned by the caller, except `g`, which is a
 *     host pointer. `stream` is a hipStream_t passed as void* (NULL = default stream).
 *   - No call allocates device memory, synchronises the device or keeps state
 *     between calls; work is enqueued on `stream` and the status reports only
 *     argument validation (done on the host before any launch) and launch errors.
 *   - Buffers are contiguous, 16-byte aligned and must not overlap unless stated.
 *   - Status codes: FPSA_OK, FPSA_ERR_INVALID_ARG (bad shape, pointer or value),
 *     FPSA_ERR_UNSUPPORTED (valid but not implemented: head size, dtype combination,
 *     grid kind), FPSA_ERR_CAPACITY (an output buffer is declared too small),
 *     FPSA_ERR_HIP (the HIP runtime rejected a launch). Nothing is enqueued when a
 *     call returns anything but FPSA_OK, except for FPSA_ERR_HIP, where earlier
 *     kernels of the same call may have been enqueued.
 *
 * Geometry. A grid of T x Hg x Wg tokens (T = 1 for an image) in raster order
 * n = (t*Hg + h)*Wg + w is cut into tiles of tile_t x tile_h x tile_w = 64 tokens;
 * each axis is padded up to a multiple of its tile size. Tiles (blocks) are
 * numbered in raster order over the tile grid, nb = ceil(T/tile_t) *
 * ceil(Hg/tile_h) * ceil(Wg/tile_w), and inside a tile the 64 slots follow the
 * raster order of the tile's positions. Slots outside the grid are padding: their
 * tiled rows are zero, padding keys receive no attention and padding queries
 * produce zero output. Npad = 64 * nb.
 *
 * Tensor layouts (B = batch, H = heads, D = head size in {64, 128}). Every tiled
 * layout holds one contiguous 64*D-element block per (b, h, blk), blocks in order;
 * they differ only in how the 64 slots x D channels of a block are arranged:
 *   raster      [B, N, H, D]            N = T*Hg*Wg
 *   tiled rows  [B, H, Npad, D]         element (slot e, channel d) at e*D + d
 *   tiled QK    (bf16) element (e, d) at
 *                 ((((e/32)*(D/16) + d/16)*2 + (d/8)%2)*32 + e%32)*8 + d%8
 *               (e4m3) element (e, d) at
 *                 ((((e/32)*(D/64) + d/64)*2 + (d/32)%2)*32 + e%32)*32 + d%32
 *               i.e. the order in which the 64 lanes of a wavefront hold a 32-row
 *               operand of one 32x32 matrix-core step, so that each wave-wide load
 *               reads one contiguous kilobyte; used for Q and K.
 *   tiled VT    (bf16) with p the position of slot e inside its run of 16 slots
 *               (slots 0-3, 8-11, 4-7, 12-15 of each run take positions 0-15) and
 *               P = 16*(e/16) + p, element (e, d) at
 *                 ((((d/32)*4 + P/16)*2 + (P/8)%2)*32 + d%32)*8 + P%8
 *               i.e. the value operand of the P*V product in lane order; used for V.
 *   CSR         row_ptr[R + 1], col_idx[nnz] int32; R = B*H*nb rows, row
 *               (b*H + h)*nb + qb; each row's key blocks ascending.
 */
#ifndef FPSA_H
#define FPSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FPSA_OK = 0,
    FPSA_ERR_INVALID_ARG = 1,
    FPSA_ERR_UNSUPPORTED = 2,
    FPSA_ERR_CAPACITY = 3,
    FPSA_ERR_HIP = 4
} fpsa_status;

typedef enum { FPSA_F32 = 0, FPSA_BF16 = 1, FPSA_FP8_E4M3 = 2 } fpsa_dtype;

typedef enum { FPSA_LAYOUT_ROWS = 0, FPSA_LAYOUT_VT = 1, FPSA_LAYOUT_QK = 2 } fpsa_layout;

typedef struct {
    int32_t t, h, w;                 /* token grid (t = 1 for an image) */
    int32_t tile_t, tile_h, tile_w;  /* tile shape, product must be 64 */
} fpsa_grid;

/* Largest block count accepted by fpsa_block_mass and fpsa_select_blocks. */
#define FPSA_MAX_SELECT_BLOCKS 4096

/* Number of 64-token blocks of the grid; negative if the grid or tile is invalid.
   Host-only. */
int32_t fpsa_num_blocks(const fpsa_grid* g);

/* Static, NUL-terminated description of a status code. Host-only. */
const char* fpsa_status_string(int32_t status);

/* Library version as major*10000 + minor*100 + patch. Host-only. */
int32_t fpsa_version(void);

/* Device scratch bytes fpsa_select_blocks needs for R rows of nb blocks. Host-only. */
size_t fpsa_select_workspace_bytes(int64_t R, int32_t nb);

/*
 * Permute tokens between raster order and the tiled layout (the unified tile
 * granularity of [FPSAttention ..., Abstract]).
 *
 * Forward (inverse = 0): src raster [B, N, H, D] of src_dtype (F32 or BF16) ->
 *   dst tiled of dst_dtype in dst_layout:
 *     BF16 in ROWS, QK or VT: values rounded to nearest even;
 *     FP8_E4M3 in ROWS or QK: OCP e4m3fn bytes plus dst_scale [B, H, nb] float32:
 *       per (b, h, block) the scale is float32(amax / 448) over the block's 64 x D
 *       values (1 when amax = 0) and each byte is the nearest-even e4m3fn encoding
 *       of float32(x / scale), saturated to +-448.
 *   Padding slots are written as zero.
 * Inverse (inverse = 1): src tiled rows BF16 -> dst raster of dst_dtype (F32 or
 *   BF16); only real tokens are written; layout must be ROWS, dst_scale NULL.
 * dst_scale must be non-NULL exactly when dst_dtype is FP8_E4M3.
 */
int32_t fpsa_tile_reorder(const void* src, int32_t src_dtype, void* dst, int32_t dst_dtype,
                          int32_t dst_layout, float* dst_scale, int32_t B, int32_t H, int32_t D,
                          const fpsa_grid* g, int32_t inverse, void* stream);

/*
 * Dequantized e4m3 tiles, for the backward of the FP8 forward ([FPSAttention ...,
 * Abstract]: training through the FP8 tiles; the quantizer passes gradients straight
 * through, so the gradients are those of attention at the dequantized Q and K).
 *
 * src: tiled QK layout, e4m3 codes (as written by fpsa_tile_reorder with dst_dtype
 * FPSA_FP8_E4M3); scale: its [B, H, nb] float32 tile scales, or NULL. dst: tiled QK
 * layout, BF16, element = the float32 product code value * scale rounded to BF16
 * (nearest even), or with a NULL scale the code value itself (exact in BF16; the
 * form fpsa_sparse_attn_bwd takes for the FP8 backward). Deterministic; every element
 * of every block is written.
 */
int32_t fpsa_dequantize_tiles(const void* src, const float* scale, int32_t B, int32_t H, int32_t D,
                              const fpsa_grid* g, void* dst, void* stream);

/*
 * Exact dense block attention mass (the one dense measurement step of [LoSA ...,
 * Abstract]).
 *
 * q_tiled, k_tiled: tiled QK layout, BF16. For each (b, h) and query block qb,
 *   mass[b, h, qb, kb] = (1 / c(qb)) * sum over real queries i of qb and real keys j
 *   of kb of softmax_j(softmax_scale * q_i . k_j), the softmax running over all real
 *   keys and c(qb) the number of real queries in qb. Each row sums to 1.
 * mass: [B, H, nb, nb] float32. lse: [B, H, Npad] float32 natural-log log-sum-exp of
 *   each real query's scaled scores (padding rows get 0), or NULL.
 * workspace: device scratch of workspace_bytes, at least 2*nb*64*4 bytes (the
 *   pass takes query blocks in pairs, 2i and 2i+1 of a head, and keeps nb*64 floats
 *   per query block); fpsa_mass_workspace_bytes gives the size that lets one launch
 *   cover every pair. With less, the call issues several launches, each covering as
 *   many pairs as fit. Contents on return are unspecified.
 * nb must not exceed FPSA_MAX_SELECT_BLOCKS; FPSA_ERR_CAPACITY if the workspace
 *   holds less than one pair.
 */
int32_t fpsa_block_mass(const void* q_tiled, const void* k_tiled, int32_t B, int32_t H, int32_t D,
                        const fpsa_grid* g, float softmax_scale, float* mass, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for fpsa_block_mass to run in one launch
   (B*H*ceil(nb/2) pairs * 2*nb*64*4); 0 for an invalid grid. Host-only. */
size_t fpsa_mass_workspace_bytes(int32_t B, int32_t H, const fpsa_grid* g);

/*
 * Retained-mass block selection ([LoSA ..., Abstract]: per head and query block,
 * the smallest key-block set meeting the threshold).
 *
 * For each of the R rows of mass [R, nb] float32: key_k = floor(clamp(m_k, 0, 1) *
 * 2^40) (NaN -> 0) as an integer; blocks are ranked by key, larger first, equal keys
 * by lower index; the row keeps the shortest leading run of the ranking whose key
 * sum C satisfies thr_den * C >= thr_num * S, S the row's key sum (nothing when
 * S = 0). Kept indices are written ascending; row_ptr gets the exclusive prefix
 * sum of the kept counts (row_ptr[R] = nnz). The result is exact and deterministic.
 * Requires 0 <= thr_num <= thr_den, 1 <= thr_den <= 1000, 1 <= nb <=
 * FPSA_MAX_SELECT_BLOCKS, R <= 2^24, col_capacity >= R * nb (FPSA_ERR_CAPACITY
 * otherwise), workspace_bytes >= fpsa_select_workspace_bytes(R, nb).
 */
int32_t fpsa_select_blocks(const float* mass, int64_t R, int32_t nb, uint32_t thr_num,
                           uint32_t thr_den, int32_t* row_ptr, int32_t* col_idx,
                           int64_t col_capacity, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * fpsa_select_blocks without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Same arguments, rule, output and errors as fpsa_select_blocks;
 * the scratch is a static device array of the library (16 bytes per row, 16 MiB,
 * one copy per GPU, held until the process ends; nothing is allocated). R above
 * FPSA_SELECT_NOALLOC_MAX_ROWS returns FPSA_ERR_CAPACITY. The scratch of the current
 * device is used, so `stream` must belong to the current device. Every word of the
 * scratch that a call reads is first written by that call, so nothing needs
 * clearing between calls; but all calls on one GPU share the one scratch, so calls
 * that overlap in time on one GPU (concurrent streams, or threads) race and must be
 * serialised by the caller.
 */
#define FPSA_SELECT_NOALLOC_MAX_ROWS (1L << 20)
int32_t fpsa_select_blocks_noalloc(const float* mass, int64_t R, int32_t nb, uint32_t thr_num,
                                   uint32_t thr_den, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, void* stream);

/*
 * Structured group-shared mask ([Grouping First, Attending Smartly ..., Abstract]).
 *
 * Only for 2D grids (t = 1, tile_t = 1): the blocks form an nh x nw grid of token
 * groups. Query group (r, c) keeps key group (r2, c2) when |r - r2| <= 1 and
 * |c - c2| <= 1 (clipped at the border, itself included), or r2 = r, or c2 = c.
 * The same rows are written for each of `copies` (= B*H) copies, so the CSR has
 * R = copies * nb rows. col_capacity must be >= copies * nb * (nh + nw + 9);
 * workspace_bytes >= fpsa_select_workspace_bytes(copies * nb, nb).
 */
int32_t fpsa_structured_mask(const fpsa_grid* g, int32_t copies, int32_t* row_ptr,
                             int32_t* col_idx, int64_t col_capacity, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Fixed per-head patterns ([Sparse-vDiT: Unleashing the Power of Sparse Attention to
 * Accelerate Video Diffusion Transformers, Abstract]: diagonal, multi-diagonal and
 * vertical-stripe structures, chosen per head).
 *
 * patterns: DEVICE int32 [H][4], head h = {band, period, stripe, dense}. On the
 * raster sequence of blocks, query block qb of head h keeps key block kb when
 *   dense != 0, or kb < stripe (vertical stripe), or band >= 0 and either
 *   |kb - qb| <= band (diagonal) or period > 0 and the distance from kb - qb to the
 *   nearest multiple of period is <= band (multi-diagonal).
 * Any int32 values are accepted (band < 0, period <= 0, stripe <= 0 disable their
 * part); a head with nothing enabled gets empty rows, which the forward answers
 * with zero output (a skipped head). Rows (b*H + h)*nb + qb, indices ascending;
 * R = B*H*nb. All heads share one CSR, so one forward launch serves every pattern.
 * Requires R <= 2^24, R * nb < 2^31, col_capacity >= R * nb (FPSA_ERR_CAPACITY
 * otherwise), workspace_bytes >= fpsa_select_workspace_bytes(R, nb).
 */
int32_t fpsa_pattern_mask(const fpsa_grid* g, int32_t B, int32_t H, const int32_t* patterns,
                          int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Retained-mass monitor for frozen indices ([LoSA ..., Abstract]: the kept support
 * is taken as stable across denoising steps; this measures how much of a later
 * step's mass it still covers).
 *
 * mass: [R, nb] float32 block masses (e.g. fpsa_block_mass of a later step, R =
 * B*H*nb). row_ptr / col_idx: a CSR with R rows (e.g. the frozen selection).
 * retained[r] = sum of mass[r, kb] over the DISTINCT indices kb in [0, nb) listed by
 * row r (repeats count once, out-of-range indices are ignored, an empty row gives
 * 0), summed in float64 and rounded once to float32. The CSR must be well formed:
 * 0 <= row_ptr[r] <= row_ptr[r + 1] and col_idx holding row_ptr[R] entries.
 * Requires 1 <= R <= 2^24, 1 <= nb <= FPSA_MAX_SELECT_BLOCKS. Deterministic.
 */
int32_t fpsa_retained_mass(const float* mass, int64_t R, int32_t nb, const int32_t* row_ptr,
                           const int32_t* col_idx, float* retained, void* stream);

/*
 * Block-sparse attention forward with an online softmax over the kept blocks: the
 * FlashAttention-style kernel that visits only the frozen key/value blocks of each
 * query block ([LoSA ..., Abstract]: the kept block set of each head and query
 * block is reused for the remaining steps; [FPSAttention ..., Abstract]: the kernel
 * builds on FlashAttention, and one 3D tile is both the sparsity block and the FP8
 * quantization group, so a tile's scale factors out of its scores).
 *
 * q, k: tiled QK layout, BF16 when qk_dtype = FPSA_BF16, or FP8_E4M3 bytes with
 *   q_scale / k_scale [B, H, nb] float32, positive (as produced by
 *   fpsa_tile_reorder) when qk_dtype = FPSA_FP8_E4M3; scales must be NULL for BF16.
 * v: tiled VT, BF16.
 * row_ptr / col_idx: CSR with R = B*H*nb rows; key-block indices outside [0, nb)
 *   contribute nothing (they are treated as blocks without real keys). A row should
 *   list each block once (the selection and mask calls never repeat one): with
 *   D = 128 on video grids (t > 1) of at most FPSA_MAX_SELECT_BLOCKS blocks a
 *   repeated block counts once, on the other paths once per listing.
 * For each real query i of block qb of row r: o_i = sum_j p_ij v_j over the real
 *   keys j of the kept blocks, p the softmax of softmax_scale * q_i . k_j over
 *   exactly those keys (FP8: the scores use the decoded values, q8 * k8 * q_scale *
 *   k_scale). Queries with no kept key, and padding rows, get o = 0. The kept blocks
 *   are visited in ascending block order (D = 128 on video grids (t > 1) of at most
 *   FPSA_MAX_SELECT_BLOCKS blocks: two neighbouring query blocks share one pass over
 *   the union of their rows) or in CSR order (other paths); the order changes only
 *   rounding. Probabilities are rounded to BF16 for the P*V product, which
 *   accumulates in float32, and the softmax denominator is the sum of those rounded
 *   probabilities. Scores: BF16 Q/K with D = 128 and lse == NULL (the inference call)
 *   take q times softmax_scale * log2(e) rounded to BF16 once (at most 2^-8 relative per
 *   element, as a library attention that pre-scales q in the input precision); every
 *   other call (D = 64, FP8, or lse requested) scales the float32 score product.
 * o: tiled rows BF16 [B, H, Npad, D]. lse: [B, H, Npad] float32 natural-log
 *   log-sum-exp over the visited keys, taken from the same rounded probabilities
 *   that normalise o (-inf for a query with none; 0 for padding), or NULL.
 * o_f32: NULL, or tiled rows float32 [B, H, Npad, D] receiving o before its BF16
 *   rounding (the backward's delta = dO.o is then free of that rounding).
 * Requires B*H*nb < 2^31 and Npad*D*2 < 2^31 (one (batch, head)'s V tiles are
 * addressed with 32-bit offsets; FPSA_ERR_UNSUPPORTED otherwise).
 */
int32_t fpsa_sparse_attn_fwd(const void* q, const void* k, const void* v, int32_t qk_dtype,
                             const float* q_scale, const float* k_scale, const int32_t* row_ptr,
                             const int32_t* col_idx, int32_t B, int32_t H, int32_t D,
                             const fpsa_grid* g, float softmax_scale, void* o, float* lse,
                             float* o_f32, void* stream);

/*
 * Transpose of a block CSR, per (b, h): for key block kb of head slice (b, h), the
 * query blocks qb whose row (b*H + h)*nb + qb keeps kb, ascending - the column view
 * the key-gradient pass of fpsa_sparse_attn_bwd walks.
 *
 * row_ptr / col_idx: CSR with R = B*H*nb rows (out-of-range indices are dropped,
 * repeats collapse). col_ptr [R + 1] (column (b*H + h)*nb + kb), row_idx [nnz].
 * Requires R <= 2^24, R * nb < 2^31, capacity >= R * nb (FPSA_ERR_CAPACITY
 * otherwise), workspace_bytes >= fpsa_transpose_workspace_bytes(R, nb).
 * Deterministic.
 */
int32_t fpsa_csr_transpose(const int32_t* row_ptr, const int32_t* col_idx, int32_t B, int32_t H,
                           int32_t nb, int32_t* col_ptr, int32_t* row_idx, int64_t capacity,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for fpsa_csr_transpose (a bitmap of R x nb bits and R counts);
   0 for R <= 0 or nb <= 0. Host-only. */
size_t fpsa_transpose_workspace_bytes(int64_t R, int32_t nb);

/*
 * Block-sparse attention backward over the same CSR as the forward (the gradients
 * that training through the sparse, tiled kernel needs [FPSAttention ...,
 * Abstract]).
 *
 * q, k, v, dout: tiled QK layout, BF16 (V and the upstream gradient dO in the QK
 *   layout too, not VT). o: the forward's output in tiled rows, BF16 (o_dtype =
 *   FPSA_BF16) or its float32 copy o_f32 (o_dtype = FPSA_F32, more accurate delta).
 *   lse: the forward's lse [B, H, Npad] (natural log). row_ptr / col_idx: the forward's CSR;
 *   col_ptr / row_idx: its transpose (fpsa_csr_transpose). Entries outside [0, nb)
 *   contribute nothing. A row should list each block once; a repeated block counts once
 *   in dk and dv (the transpose collapses repeats) and, for BF16 with D = 128 on video
 *   grids (t > 1) of at most FPSA_MAX_SELECT_BLOCKS blocks, in dq (whose pass walks the
 *   union of two rows' membership bitmaps, as the forward does there); in dq on the
 *   other paths once per listing.
 * With p_ij = exp(softmax_scale q_i.k_j - lse_i) over the kept keys j of query i
 * and delta_i = dO_i.o_i:
 *   dv_j = sum_i p_ij dO_i,  ds_ij = p_ij (dO_i.v_j - delta_i),
 *   dk_j = softmax_scale sum_i ds_ij q_i,  dq_i = softmax_scale sum_j ds_ij k_j,
 * products in BF16 with float32 accumulation (p and ds are rounded to BF16 for the
 * matrix products). Padding rows and queries whose lse is -inf contribute nothing
 * and get zero gradients; so do key blocks no row keeps.
 * q_scale, k_scale: both NULL (q and k are the attention inputs), or, for the
 *   backward of the FP8 forward, the [B, H, nb] e4m3 tile scales, with q and k
 *   holding the e4m3 code values as BF16 (fpsa_dequantize_tiles with a NULL scale;
 *   e4m3 values are exact in BF16). The gradients are then those of attention at the
 *   dequantized inputs q-hat = q * q_scale, k-hat = k * k_scale (the quantizer passes
 *   gradients straight through): scores sq*sk*(q.k) exactly as the FP8 forward formed
 *   them, and ds pre-multiplied by the tile scale before the dq and dk products.
 *   Exactly one of the two NULL: FPSA_ERR_INVALID_ARG.
 * dq, dk, dv: tiled rows BF16 [B, H, Npad, D], fully written.
 * workspace_bytes >= fpsa_bwd_workspace_bytes(B, H, g) (two floats per query slot).
 * Deterministic: no atomics, fixed summation order.
 */
int32_t fpsa_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                             int32_t o_dtype, const void* dout, const float* lse, const int32_t* row_ptr,
                             const int32_t* col_idx, const int32_t* col_ptr,
                             const int32_t* row_idx, const float* q_scale, const float* k_scale,
                             int32_t B, int32_t H, int32_t D,
                             const fpsa_grid* g, float softmax_scale, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for fpsa_sparse_attn_bwd (B*H*Npad*8); 0 for an invalid grid.
   Host-only. */
size_t fpsa_bwd_workspace_bytes(int32_t B, int32_t H, const fpsa_grid* g);

/*
 * Semantic-aware permutation ([Sparse VideoGen2: Accelerate Video Generation with
 * Sparse Attention via Semantic-Aware Permutation, Abstract]): tokens are clustered
 * by k-means over their own query (or key) vectors, laid out cluster by cluster, and
 * attention keeps, per query cluster, the key clusters that the centroid-based mass
 * estimate ranks into the top-p. The calls below give the pieces; the block-sparse
 * forward over the cluster layout is fpsa_sparse_attn_fwd_varlen.
 *
 * fpsa_kmeans: Lloyd's k-means per (b, h) over x[b, :, h, :] (raster [B, N, H, D],
 * FPSA_BF16 or FPSA_F32), in float64 with a fixed operation order (results are the
 * same on every run and device):
 *   start: centroid c = x of token floor(c N / C);
 *   iters times: assign each token to the centroid of least e = |c|^2 - 2 x.c (the
 *   squared distance less |x|^2, common to every candidate; |c|^2 and x.c each a
 *   chain of fused multiply-adds over the channels in order from zero; ties to the
 *   lower cluster), then set each non-empty cluster's centroid to the mean of its
 *   members (member r, in token order, goes to partial sum r % 8, each partial
 *   summed in order, the partials combined as ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)));
 *   an empty cluster keeps its centroid.
 * Outputs (device): assign [B, H, N]; centroids [B, H, C, D] float64; counts
 * [B, H, C]; member_off [B*H*C + 1] and members [B*H*N]: the tokens of cluster c of
 * slice bh, ascending, are members[member_off[bh*C + c] .. member_off[bh*C + c + 1]).
 * workspace: device scratch of at least fpsa_kmeans_workspace_bytes(B, H, N, C) bytes
 * (per-chunk cluster counts; FPSA_ERR_CAPACITY if smaller), contents on return
 * unspecified. Requires D in {64, 128}, 1 <= C <= min(N, FPSA_MAX_SELECT_BLOCKS),
 * 1 <= iters <= 1000, B*H*N < 2^31, and finite inputs.
 */
int32_t fpsa_kmeans(const void* x, int32_t x_dtype, int32_t B, int32_t N, int32_t H, int32_t D,
                    int32_t C, int32_t iters, int32_t* assign, double* centroids, int32_t* counts,
                    int32_t* member_off, int32_t* members, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Device scratch bytes fpsa_kmeans needs (0 for invalid sizes). Host-only. */
size_t fpsa_kmeans_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t C);

/*
 * Cluster-contiguous block layout: cluster c of slice bh fills blocks
 * blk_off[bh][c] .. blk_off[bh][c+1]-1 (ceil(count_c / 64) blocks, its members in
 * token order, the last block padded). slot_token [B, H, NB*64]: the token of each
 * slot, -1 for padding; blk_off [B, H, C+1]; blk_count [B, H, NB]: the real slots of
 * each block (a block's real slots are its first ones; 0 past blk_off[bh][C]).
 * member_off / members as produced by fpsa_kmeans. NB >= ceil(N/64) + C is
 * required (FPSA_ERR_CAPACITY otherwise): any clustering fits in that many blocks.
 */
int32_t fpsa_cluster_layout(const int32_t* member_off, const int32_t* members, int32_t B, int32_t H,
                            int32_t N, int32_t C, int32_t NB, int32_t* slot_token, int32_t* blk_off,
                            int32_t* blk_count, void* stream);

/*
 * Tile moves driven by a slot map instead of the grid: gather raster [B, N, H, D]
 * (FPSA_BF16 or FPSA_F32) into B*H*NB blocks of layout FPSA_LAYOUT_ROWS, _QK or _VT
 * (BF16; padding slots zero), and scatter tiled rows (BF16) back to raster
 * (FPSA_BF16 or FPSA_F32; only slots holding a token are written). slot_token as
 * from fpsa_cluster_layout; every token must appear at most once per slice.
 */
int32_t fpsa_gather_tiles(const void* src, int32_t src_dtype, const int32_t* slot_token, int32_t B,
                          int32_t N, int32_t H, int32_t D, int32_t NB, int32_t layout, void* dst,
                          void* stream);
int32_t fpsa_scatter_tiles(const void* src, const int32_t* slot_token, int32_t B, int32_t N, int32_t H,
                           int32_t D, int32_t NB, void* dst, int32_t dst_dtype, void* stream);

/*
 * Cluster-level attention mass from the cluster representation: each key cluster
 * stands for n_j keys at its centroid, so for query cluster i of slice bh
 *   est[i, j] = n_j exp(s cq_i . ck_j) / sum_j' n_j' exp(s cq_i . ck_j')
 * over non-empty key clusters (s = softmax_scale; the dot product in float64 summed
 * over channels in order), rounded to float32; rows of empty query clusters are 0.
 * cq [B, H, Cq, D], ck [B, H, Ck, D] float64; nq [B, H, Cq], nk [B, H, Ck];
 * est [B, H, Cq, Ck] - rows ready for fpsa_select_blocks (R = B*H*Cq, nb = Ck).
 * Requires D in {64, 128}, 1 <= Cq, 1 <= Ck <= FPSA_MAX_SELECT_BLOCKS.
 */
int32_t fpsa_cluster_mass(const double* cq, const int32_t* nq, const double* ck, const int32_t* nk,
                          int32_t B, int32_t H, int32_t Cq, int32_t Ck, int32_t D, float softmax_scale,
                          float* est, void* stream);

/*
 * Block CSR of a cluster selection: query block qb of slice bh lies in query cluster
 * i when qoff[bh][i] <= qb < qoff[bh][i+1] and keeps every block of every key
 * cluster j listed in cluster row bh*Cq + i (blocks koff[bh][j] .. koff[bh][j+1]-1),
 * in the row's order; blocks past qoff[bh][Cq] keep nothing. Rows bh*NB + qb
 * (R = B*H*NB). qoff [B, H, Cq+1], koff [B, H, Ck+1] as blk_off of
 * fpsa_cluster_layout. capacity >= R * NB, workspace_bytes >= 4 * R.
 */
int32_t fpsa_cluster_blocks(const int32_t* crow_ptr, const int32_t* ccol_idx, const int32_t* qoff,
                            const int32_t* koff, int32_t B, int32_t H, int32_t Cq, int32_t Ck,
                            int32_t NB, int32_t* row_ptr, int32_t* col_idx, int64_t capacity,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse forward over blocks whose real keys are counted instead of following
 * from a token grid: block kb of slice bh holds key_counts[bh*NB + kb] real keys in
 * its first slots (values outside 0..64 are clamped to it). Otherwise as
 * fpsa_sparse_attn_fwd (size limits with nb = NB included) with BF16 q, k (QK layout)
 * and v (VT layout) of B*H*NB blocks; every query slot gets an output (the caller
 * scatters the real ones back); lse and o_f32 optional. With D = 128 and NB <=
 * FPSA_MAX_SELECT_BLOCKS, two neighbouring query blocks share one pass over the union
 * of their rows in ascending block order (the blocks of one query cluster keep the
 * same key clusters), and a repeated block counts once; with D = 64 or a larger NB the
 * rows are walked in CSR order, once per listing.
 */
int32_t fpsa_sparse_attn_fwd_varlen(const void* q, const void* k, const void* v,
                                    const int32_t* key_counts, const int32_t* row_ptr,
                                    const int32_t* col_idx, int32_t B, int32_t H, int32_t D,
                                    int32_t NB, float softmax_scale, void* o, float* lse,
                                    float* o_f32, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FPSA_H */
