/*
 * veda.h -- C ABI of the Veda block-sparse attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * The method (Miowtion project page, intro bullet "Sparse acceleration (Veda)"
 * and Key Features > "Veda sparse attention"): the video tokens of each head
 * are permuted into 3D (t, h, w) tiles of 128 tokens; a small per-head
 * predictor pools every tile (mean, max, min), projects it and scores every
 * (query tile, key tile) pair; a block mask keeps the top-scoring pairs under
 * equal-kernel-cost budgets with Bresenham rounding and a forced diagonal; and
 * flash attention computes only the kept 128x128 blocks.  "Deploying this
 * checkpoint", section 2 (SM90): the block mask reaches the kernel packed into
 * index lists, and query tiles are 128 rows.
 *
 * Conventions shared by every call:
 *  - Every pointer named "device" is caller-owned GPU memory (e.g. from torch),
 *    contiguous and 16-byte aligned.  The library never allocates GPU memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every compute call only enqueues work on it and returns; it never
 *    synchronises the host.
 *  - Every argument, shape and plan check happens on the host before any
 *    launch.  A failed check returns a non-zero veda_status, launches nothing,
 *    and leaves a message for veda_last_error() on the calling thread.
 *  - Nothing is ever silently computed another way: an unsupported device,
 *    dtype, head dim or plan returns VEDA_ERR_UNSUPPORTED (the pages' rule of
 *    an explicit error instead of a silent dense fallback, "Deploying this
 *    checkpoint", sections 2 and 5).
 *  - Tensors are bf16 (stored as uint16 bit patterns) unless stated otherwise.
 *
 * Layouts (N = tokens of the packed sequence, H = heads, D = head dim):
 *  - natural:   bf16 [N, H, D], token-major, as a fused QKV projection emits.
 *  - permuted:  bf16 [R, D] with R = sum_h L_h, head-major; head h owns rows
 *               [row_offset(h), row_offset(h) + L_h), L_h = 128 * n_h, and
 *               row row_offset(h) + 128*i + s is slot s of tile i.  The valid
 *               tokens of a tile occupy its first valid(i) slots; padding
 *               slots hold +0.
 *  - tile-transposed (V only): bf16 [T, D, 128] with T = sum_h n_h; block t
 *               holds tile t (head-major, like the rows above) with element
 *               [t][d][s] = V_perm[128 t + s][d].  This is the layout the
 *               attention kernel streams V in.
 *  - scores:    fp32, head h's n_h x n_h matrix (row = query tile, column =
 *               key tile) at offset pair_offset(h).
 *  - CSR mask:  row_ptr int32 [T + 1] over the global rows t = tile_offset(h)
 *               + i; col_idx int32 [nnz] holds head-local key tile indices,
 *               ascending within a row.
 */
#ifndef VEDA_H
#define VEDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VEDA_ABI_VERSION 9

typedef int32_t veda_status;
enum {
  VEDA_OK = 0,
  VEDA_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad enum value     */
  VEDA_ERR_SHAPE = 2,       /* sizes inconsistent with the plan              */
  VEDA_ERR_UNSUPPORTED = 3, /* device, head dim, plan form not supported     */
  VEDA_ERR_WORKSPACE = 4,   /* workspace missing or too small                */
  VEDA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a copy or a launch   */
  VEDA_ERR_STATE = 6        /* plan used before veda_plan_upload             */
};

/* Segment kinds of the packed sequence (Miowtion project page, Key Features >
 * "H3 DiT for training": packed t2va / fl2va / ref2va layouts). */
enum { VEDA_SEG_VIDEO3D = 0, VEDA_SEG_DENSE1D = 1 };

/* Budget modes.  KEEP_RATIO: equal-kernel-cost budgets, keep_num/keep_den of
 * the blocks a dense kernel over the valid tokens of each (query segment, key
 * segment) video pair would compute, spread over query tiles by midpoint
 * Bresenham rounding (Key Features > "Veda sparse attention").  FIXED_K:
 * fixed_k key tiles per query tile and key segment.  ALL: every block (dense
 * attention through the same kernel; used for the dense LSE). */
enum { VEDA_BUDGET_KEEP_RATIO = 0, VEDA_BUDGET_FIXED_K = 1, VEDA_BUDGET_ALL = 2 };

/* Layouts of the attention output O. */
enum { VEDA_LAYOUT_PERMUTED = 0, VEDA_LAYOUT_NATURAL = 1 };

/* Directions of veda_permute_tiles. */
enum {
  VEDA_PERMUTE_FORWARD = 0,            /* natural  -> permuted              */
  VEDA_PERMUTE_INVERSE = 1,            /* permuted -> natural (valid slots) */
  VEDA_PERMUTE_FORWARD_TRANSPOSED = 2  /* natural  -> tile-transposed (V)   */
};

typedef struct veda_segment {
  int32_t kind;         /* VEDA_SEG_VIDEO3D or VEDA_SEG_DENSE1D              */
  int32_t t, h, w;      /* grid; a DENSE1D segment of length n is (1, 1, n)  */
  int64_t token_offset; /* first token of the segment in the packed sequence */
} veda_segment;

typedef struct veda_plan_desc {
  int32_t num_segments;          /* 1 .. 8, in packed order, contiguous from 0 */
  const veda_segment* segments;  /* host array [num_segments]                 */
  int32_t num_heads;             /* 1 .. 1024                                 */
  int32_t head_dim;              /* 64 or 128                                 */
  const int32_t* tile_shape;     /* host array [num_heads][3]: (a, b, c) per
                                    head, a*b*c == 128, at most 2 distinct     */
  int32_t budget_mode;           /* VEDA_BUDGET_*                             */
  int32_t keep_num, keep_den;    /* KEEP_RATIO: 0 <= keep_num <= keep_den     */
  int32_t fixed_k;               /* FIXED_K: >= 0 (the diagonal is always kept)*/
} veda_plan_desc;

typedef struct veda_plan veda_plan; /* opaque, host memory */

typedef struct veda_plan_info {
  int64_t num_tokens;         /* N                                            */
  int32_t num_heads, head_dim, num_segments, num_shapes;
  int64_t total_rows;         /* R = sum_h 128 n_h                            */
  int64_t total_tiles;        /* T = sum_h n_h                                */
  int64_t total_pairs;        /* sum_h n_h^2 (length of the score array)      */
  int64_t nnz;                /* kept blocks over all heads (exact, from the
                                 budgets; known before any launch)            */
  int64_t max_row_blocks;     /* longest CSR row                              */
  int64_t device_table_bytes; /* bytes veda_plan_upload needs                 */
  int64_t score_workspace_bytes; /* bytes veda_score_tiles needs              */
  int64_t transpose_workspace_bytes; /* bytes veda_mask_transpose needs       */
  int64_t bwd_workspace_bytes; /* bytes veda_block_sparse_attn_bwd needs       */
  int32_t max_tiles_per_head;
  int32_t uploaded;           /* 1 after a successful veda_plan_upload        */
  int64_t heat_workspace_bytes; /* bytes veda_dense_lse_heat and (as the dense
                                   plan) veda_attn_fwd_lse_heat need: about
                                   nnz*516 + 4*T + 12*R                       */
  int64_t reduce_workspace_bytes; /* bytes veda_mask_mass / veda_output_error
                                     need (per-head partial sums)             */
} veda_plan_info;

/* ABI version of the loaded library (VEDA_ABI_VERSION it was built with). */
int veda_abi_version(void);

/* VEDA_OK iff `device` is a gfx950 GPU the library was built for; otherwise
 * VEDA_ERR_UNSUPPORTED and a reason in `reason` (may be NULL, truncated to n).
 * Every compute call re-checks the current device the same way. */
veda_status veda_available(int device, char* reason, size_t n);

/* Message of the last non-OK status on the calling thread ("" if none). */
const char* veda_last_error(void);

/* Build a plan on the host (no GPU call).  Validates the description and
 * computes the tiles of every head (readings of the Veda tiling: tiles
 * row-major over the padded tile grid, tokens row-major inside each tile's
 * valid box, valid prefix then padding), the slot->token tables, the per-row
 * budgets per key segment and the CSR row pointers.  *out receives a plan the
 * caller frees with veda_plan_destroy. */
veda_status veda_plan_create(const veda_plan_desc* desc, veda_plan** out);
void veda_plan_destroy(veda_plan* plan);

veda_status veda_plan_query(const veda_plan* plan, veda_plan_info* info);

/* Per-head geometry: tiles n_h, first row, first global tile, first score. */
veda_status veda_plan_head(const veda_plan* plan, int32_t head, int32_t* num_tiles,
                           int64_t* row_offset, int64_t* tile_offset,
                           int64_t* pair_offset);

/* Host copies of plan tables (for tests and tools).  Each takes the element
 * count of `out` and fails with VEDA_ERR_SHAPE if it differs from:
 *   perm:    L_h     int32 slot -> token, -1 for padding
 *   valid:   n_h     int32 valid tokens per tile
 *   budgets: n_h * S int32 blocks row i keeps from key segment s
 *   row_ptr: T + 1   int32 global CSR row pointers */
veda_status veda_plan_copy_perm(const veda_plan* plan, int32_t head, int32_t* out, int64_t n);
veda_status veda_plan_copy_valid(const veda_plan* plan, int32_t head, int32_t* out, int64_t n);
veda_status veda_plan_copy_budgets(const veda_plan* plan, int32_t head, int32_t* out, int64_t n);
veda_status veda_plan_copy_row_ptr(const veda_plan* plan, int32_t* out, int64_t n);

/* Copy the plan's tables into caller-owned device memory `dev_tables`
 * (device_table_bytes bytes, 256-byte aligned) with an async copy on `stream`.
 * The host plan keeps the device address; `dev_tables` must stay alive and
 * unmodified while the plan is used.  Upload once, before any compute call;
 * the plan is then immutable and may be used from several threads. */
veda_status veda_plan_upload(veda_plan* plan, void* dev_tables, size_t bytes, void* stream);

/* Tile permutation (Miowtion project page, "Sparse acceleration (Veda)" and
 * Key Features > "Veda sparse attention": per-head 3D tiles of 128 tokens,
 * padded grids with valid-prefix tiles).
 *   FORWARD:            src natural [N,H,D] -> dst permuted [R,D]
 *   FORWARD_TRANSPOSED: src natural [N,H,D] -> dst tile-transposed [T,D,128]
 *   INVERSE:            src permuted [R,D]  -> dst natural [N,H,D]; only
 *                       valid slots are written (padding rows are dropped).
 * Padding slots of the forward outputs are written as +0.  Bit copies. */
veda_status veda_permute_tiles(const veda_plan* plan, const void* src, void* dst,
                               int32_t direction, void* stream);

/* The three forward permutations of one attention layer in one pass, with
 * the predictor's pooling fused in: q -> q_perm and k -> k_perm (permuted
 * rows), v -> v_t (tile-transposed), each read once from HBM; while a tile of
 * Q or K is in flight its mean (fp64 sum), max and min over the valid slots
 * are written to `workspace` (fp32 [T, 3D] for Q, then for K), where
 * veda_score_pooled picks them up.  Outputs are bit-identical to three
 * veda_permute_tiles calls.  workspace may be NULL (no pooling); otherwise it
 * must hold score_workspace_bytes.  v and v_t may both be NULL: then only Q
 * and K are permuted (and pooled), e.g. so that V's permutation
 * (veda_permute_tiles, FORWARD_TRANSPOSED) can run on another stream while
 * the predictor scores; one NULL without the other is VEDA_ERR_INVALID_ARG.
 * q_perm may be NULL when workspace is given: Q is then read and pooled but
 * not written, for a layer whose attention reads Q in its natural layout
 * (q_layout VEDA_LAYOUT_NATURAL below). */
veda_status veda_permute_qkv(const veda_plan* plan, const void* q, const void* k, const void* v,
                             void* q_perm, void* k_perm, void* v_t, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Projection and pair scores from the pooled features that veda_permute_qkv
 * left in `workspace`; same results as veda_score_tiles on the permuted Q/K. */
veda_status veda_score_pooled(const veda_plan* plan, const float* w_q, const float* w_k, float* scores,
                              void* workspace, size_t workspace_bytes, void* stream);

/* The predictor (Key Features > "Veda sparse attention": mean/max/min pooling
 * plus a per-head residual projection; "Sparse acceleration (Veda)": scores
 * of (query tile, key tile) pairs).  For every tile, over its valid slots only:
 * f = [mean | max | min] (fp32; the mean from an fp64 sum), then
 * x_hat[d] = fp32(mean[d] + sum_e W[h][d][e] * f[e]) summed in fp64 over
 * e = 0..3D-1 ascending, and s[i][j] = fp32(sum_d q_hat_i[d] * k_hat_j[d]) in
 * fp64 over d ascending, with -0 written as +0.
 *   q_perm, k_perm: device permuted bf16 [R, D]
 *   w_q, w_k:       device fp32 [H, D, 3D]
 *   scores:         device fp32 [sum_h n_h^2]
 *   workspace:      device scratch of score_workspace_bytes (16-byte aligned).
 *                   After the call it holds, fp32 and in this order: the
 *                   pooled features of Q [T, 3D] and of K [T, 3D] (rows in
 *                   global tile order, columns [mean | max | min]), then the
 *                   projections q_hat [T, D] and k_hat [T, D]; so does it
 *                   after veda_permute_qkv (features) and veda_score_pooled
 *                   (projections). */
veda_status veda_score_tiles(const veda_plan* plan, const void* q_perm, const void* k_perm,
                             const float* w_q, const float* w_k, float* scores,
                             void* workspace, size_t workspace_bytes, void* stream);

/* veda_score_tiles without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same kernels and bitwise the same
 * scores as veda_score_tiles; the pooled features and projections go to a
 * static scratch array of the library, 128 MiB per GPU, reserved when the
 * library is loaded on that GPU and held until the process ends.  This call
 * allocates nothing and calls no allocating routine.
 *   Limit: the plan's score_workspace_bytes (T * head_dim * 32 bytes) must not
 *   exceed 128 MiB, i.e. at most 32,768 tiles over all heads at head dim 128
 *   (65,536 at 64); a larger plan returns VEDA_ERR_WORKSPACE before any launch.
 *   Every call on one GPU shares that GPU's scratch, and the kernels overwrite
 *   all of it that they read (nothing needs to start at zero): two calls whose
 *   work overlaps in time on one GPU (other streams, other threads) race and
 *   give wrong scores; calls ordered on one stream do not. */
veda_status veda_score_tiles_noalloc(const veda_plan* plan, const void* q_perm, const void* k_perm,
                                     const float* w_q, const float* w_k, float* scores, void* stream);

/* Budgeted top-k block mask (Key Features > "Veda sparse attention":
 * equal-kernel-cost budgets, Bresenham rounding, forced diagonal, segmented
 * reference/target budgets).  Row i of head h keeps, per key segment B, the
 * plan's budget k[i][B]: the diagonal tile first when i lies in B, then B's
 * highest-scoring tiles, ties to the lowest key tile index; pairs with a
 * DENSE1D segment keep every tile.  Outputs (device): row_ptr int32 [T+1],
 * col_idx int32 [nnz] ascending per row, and, if dense_mask is not NULL,
 * uint8 [sum_h n_h^2] with 1 for kept blocks.  Scores must be finite. */
veda_status veda_select_blocks(const veda_plan* plan, const float* scores, int32_t* row_ptr,
                               int32_t* col_idx, uint8_t* dense_mask, void* stream);

/* Block-sparse flash attention forward (Miowtion project page, "Sparse
 * acceleration (Veda)": only the kept blocks are computed; Key Features >
 * "Veda sparse attention": singleton mask_mod with full/partial block lists;
 * "Deploying this checkpoint", section 2 (SM90): 128x128 tiles).
 * For every query tile (head h, tile i) the kernel walks col_idx[row_ptr[t] ..
 * row_ptr[t+1]) and computes, for each query slot r,
 *   O[r] = softmax_c(scale * q_r . k_c) v_c,  LSE[r] = log sum_c exp(scale q_r.k_c)
 * over the valid slots c of the listed key tiles (slots >= valid(j) are
 * masked: the only mask rule).  bf16 MFMA products, fp32 softmax.
 *   q:      device bf16, q_layout VEDA_LAYOUT_PERMUTED: [R, D];
 *           VEDA_LAYOUT_NATURAL: [N, H, D], each query tile's rows gathered
 *           through the plan's slot -> token table when the tile is loaded
 *           (padding slots read as zeros), so no permuted copy of Q is
 *           needed; both layouts give bitwise the same O and LSE
 *   k:      device permuted bf16 [R, D]
 *   v_t:    device tile-transposed bf16 [T, D, 128]
 * The padding slots of k (rows) and v_t (columns) must hold zeros, as
 * veda_permute_qkv and veda_permute_tiles write them: the kernel removes the
 * padding keys' share of the softmax sum by count instead of masking each
 * logit (a padding key's logit is then exactly 0 and its PV term is 0).
 *   row_ptr, col_idx: device CSR as written by veda_select_blocks (or any CSR
 *           of this plan's shape with ascending, in-range, non-empty rows)
 *   o:      device bf16; o_layout VEDA_LAYOUT_PERMUTED: [R, D], rows of
 *           padding slots unspecified (finite); VEDA_LAYOUT_NATURAL:
 *           [N, H, D], every token of head h written at its natural place
 *           (the inverse permutation fused into the epilogue), padding
 *           slots dropped.  Or NULL: then only the LSE is computed (no PV
 *           products; v_t is not read), bitwise equal to the LSE of a call
 *           with o, e.g. the dense LSE that veda_block_heat takes.
 *   lse:    device fp32 [R] natural log, permuted row order, or NULL (not
 *           both o and lse NULL: VEDA_ERR_INVALID_ARG); rows of padding
 *           slots unspecified (finite)
 *   blocks_visited: device uint32 counter the kernel adds the number of
 *           blocks it computed to (caller zeroes it), or NULL.
 * softmax_scale must be finite and > 0 (1/sqrt(D) for the usual scale). */
veda_status veda_block_sparse_attn_fwd(const veda_plan* plan, const void* q, int32_t q_layout, const void* k,
                                       const void* v_t, const int32_t* row_ptr,
                                       const int32_t* col_idx, float softmax_scale, void* o,
                                       int32_t o_layout, float* lse, uint32_t* blocks_visited,
                                       void* stream);

/* Teacher block heat from the dense LSE (Key Features > "Veda sparse
 * attention": teacher block heat from the dense LSE, fused kernel).
 * heat[i][j] = (1/valid(i)) * sum over valid query slots r of tile i and valid
 * key slots c of tile j of exp(scale * q_r . k_c - lse[r]), for every pair of
 * tiles of every head; with the dense LSE each row sums to 1.  The padding
 * rows of k must hold zeros (as the permute entry points write them).
 *   q, k:  device permuted bf16 [R, D];  lse: device fp32 [R]
 *   heat:  device fp32 [sum_h n_h^2], layout of the scores.
 * A head may have at most 4096 tiles. */
veda_status veda_block_heat(const veda_plan* plan, const void* q, const void* k,
                            const float* lse, float softmax_scale, float* heat, void* stream);

/* The dense LSE and the teacher block heat in one pass (Key Features > "Veda
 * sparse attention": teacher block heat from the dense LSE, fused kernel).
 * The plan must have budget mode VEDA_BUDGET_ALL (else
 * VEDA_ERR_UNSUPPORTED) and row_ptr/col_idx its all-blocks CSR (from
 * veda_select_blocks).  Computes the same LSE as veda_block_sparse_attn_fwd
 * with o = NULL (bitwise equal) and the heat of veda_block_heat from that
 * LSE: heat[i][j] = (1/valid(i)) * sum over valid query slots r of tile i
 * and valid key slots c of tile j of exp(scale * q_r . k_c - lse[r]).  The
 * heat is formed from each block's sum of exp(scale * q_r . k_c - m_r)
 * against a fixed per-row reference m_r, divided by the row's final sum at
 * the end of the row, so the key tiles are walked once instead of twice
 * (rows that need the exact fallback pass are walked again with the final
 * LSE).  The padding rows of k must hold zeros.
 *   q:         device bf16 in q_layout, as for veda_block_sparse_attn_fwd
 *              (VEDA_LAYOUT_PERMUTED [R, D] or VEDA_LAYOUT_NATURAL [N, H, D])
 *   k:         device permuted bf16 [R, D]
 *   lse:       device fp32 [R] natural log, or NULL (not stored)
 *   heat:      device fp32 [sum_h n_h^2], layout of the scores; every pair
 *              is written
 *   workspace: device scratch of at least heat_workspace_bytes (its first
 *              nnz x 128 x 4 bytes are used: one fp32 per block and query),
 *              16-byte aligned; its contents on entry do not matter.
 * Errors: VEDA_ERR_WORKSPACE if workspace_bytes is too small;
 * VEDA_ERR_INVALID_ARG if lse, heat and workspace are not three different
 * buffers or one of them is q or k. */
veda_status veda_dense_lse_heat(const veda_plan* plan, const void* q, int32_t q_layout, const void* k,
                                const int32_t* row_ptr, const int32_t* col_idx, float softmax_scale,
                                float* lse, float* heat, void* workspace, size_t workspace_bytes,
                                void* stream);

/* The block-sparse attention of a selected mask and the dense LSE and
 * teacher block heat, without computing any block's scores twice (Key
 * Features > "Veda sparse attention": the block-sparse forward over the kept
 * blocks, and the teacher block heat from the dense LSE, fused kernel).
 * Computes what
 *   veda_block_sparse_attn_fwd(plan, q, q_layout, k, v_t, row_ptr, col_idx,
 *                              softmax_scale, o, o_layout, lse, NULL, stream)
 *   veda_dense_lse_heat(dense_plan, q, q_layout, k, dense_row_ptr,
 *                       dense_col_idx, softmax_scale, dense_lse, heat, ...)
 * compute: the attention over the selected blocks also keeps each selected
 * block's share of every query's probability; an LSE-only pass over the
 * rest of each dense row (its blocks that are not selected) joins its sum
 * with the selected row's LSE into the dense LSE,
 *   dense_lse[r] = log(exp(lse[r]) + sum over the rest of exp(s)),
 * and forms the heat of every block of the dense row.  o and lse are bitwise
 * those of veda_block_sparse_attn_fwd; dense_lse and heat agree with
 * veda_dense_lse_heat to fp32 rounding (other summation order; dense_lse
 * rows of padding slots are unspecified but finite, as in both calls).
 *   plan:       the plan of the selected mask; dense_plan: budget mode
 *               VEDA_BUDGET_ALL (else VEDA_ERR_UNSUPPORTED), same segments,
 *               heads, head dimension and tile shapes as plan (else
 *               VEDA_ERR_SHAPE)
 *   q, k, v_t:  as for veda_block_sparse_attn_fwd (q in q_layout, k permuted
 *               [R, D], v_t tile-transposed [T, D, 128]); padding rows of k
 *               and columns of v_t hold zeros
 *   row_ptr, col_idx: the selected CSR as veda_select_blocks writes it for
 *               plan: rows ascending, free of repeats, non-empty, each a
 *               subset of the same row of the dense CSR; a query tile whose
 *               selected row is not gets NaN in its dense_lse rows and its
 *               heat row (o and lse as veda_block_sparse_attn_fwd gives them)
 *   dense_row_ptr, dense_col_idx: dense_plan's all-blocks CSR, ascending
 *   o:          device bf16 in o_layout (required); lse, dense_lse: device
 *               fp32 [R] natural log, or NULL (not stored)
 *   heat:       device fp32 [sum_h n_h^2], every pair written
 *   workspace:  at least dense_plan's heat_workspace_bytes, 16-byte
 *               aligned; contents on entry do not matter
 * Three launches on `stream`.  Errors: VEDA_ERR_WORKSPACE if
 * workspace_bytes is too small; VEDA_ERR_INVALID_ARG if an output aliases an
 * input or another output, or the workspace is misaligned. */
veda_status veda_attn_fwd_lse_heat(const veda_plan* plan, const veda_plan* dense_plan, const void* q,
                                   int32_t q_layout, const void* k, const void* v_t, const int32_t* row_ptr,
                                   const int32_t* col_idx, const int32_t* dense_row_ptr,
                                   const int32_t* dense_col_idx, float softmax_scale, void* o, int32_t o_layout,
                                   float* lse, float* dense_lse, float* heat, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Attention mass a block mask keeps ("Deploying this checkpoint", section 4:
 * recall of a predicted mask against the oracle mask; section 6: the share
 * of the attention mass an oracle mask at 10% keep recovers).  Per head h:
 *   mass[h] = sum_i valid(i) * sum_{j in row i} heat[i][j] / sum_i valid(i),
 * i.e. with the dense-LSE heat of veda_block_heat, the fraction of the
 * attention probability of the head's valid queries that falls on the kept
 * blocks.  The oracle mask is veda_select_blocks applied to the heat in
 * place of the predicted scores (same budgets, forced diagonal, ties to the
 * lowest key tile); recall = mass(predicted mask) / mass(oracle mask).
 *   heat:    device fp32 [sum_h n_h^2], veda_block_heat's layout
 *   row_ptr, col_idx: device CSR of this plan's shape (as veda_select_blocks
 *            writes it); out-of-range columns are skipped
 *   mass:    device fp64 [num_heads]
 *   workspace: device scratch of at least reduce_workspace_bytes (per-head
 *            partial sums; contents on entry do not matter); too small is
 *            VEDA_ERR_WORKSPACE
 * fp64 accumulation in a fixed order (partial sums over 16-row chunks, then
 * the chunks in ascending order): bitwise reproducible. */
veda_status veda_mask_mass(const veda_plan* plan, const float* heat, const int32_t* row_ptr,
                           const int32_t* col_idx, double* mass, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Relative output error of a sparse attention output against a reference
 * (Miowtion project page, Key Features: oracle tile-plan search by relative
 * output MSE under the best mask).  Per head h, over every token and channel:
 *   err[h] = sum (o - o_ref)^2 / sum o_ref^2
 *   o, o_ref: device bf16 [N, H, D] (natural token order, as
 *             veda_block_sparse_attn_fwd writes with VEDA_LAYOUT_NATURAL)
 *   err:      device fp64 [num_heads]
 *   workspace: device scratch of at least reduce_workspace_bytes (per-head
 *             partial sums over 32 token chunks); too small is
 *             VEDA_ERR_WORKSPACE
 * fp64 accumulation in a fixed order: bitwise reproducible. */
veda_status veda_output_error(const veda_plan* plan, const void* o, const void* o_ref, double* err,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* Transposed block lists for the backward (Miowtion project page: the
 * block-sparse backward that predictor and LoRA training need; dK and dV are
 * gathered per key tile): for every head h and key tile j, the query tiles
 * whose rows hold j, ascending.
 *   row_ptr, col_idx: device CSR of this plan's shape (veda_select_blocks)
 *   col_ptr:  device int32 [T + 1], key tiles in the same head-major order as
 *             the rows; col_ptr[T] = nnz
 *   row_idx:  device int32 [nnz], head-local query tile indices
 *   workspace: device, transpose_workspace_bytes (contents overwritten)
 * Deterministic (no atomics). */
veda_status veda_mask_transpose(const veda_plan* plan, const int32_t* row_ptr, const int32_t* col_idx,
                                int32_t* col_ptr, int32_t* row_idx, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Block-sparse attention backward over the same mask as the forward
 * (same source).  With P = softmax over the valid keys of the kept blocks:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 * dK and dV are gathered per key tile over the transposed lists, dQ per query
 * tile over the row lists, so no output is accumulated by atomics.  The dK/dV
 * pass leaves dS of every kept block (bf16, 32 KB per block) in the workspace
 * for the dQ pass, which therefore computes neither S nor dP again; the
 * transposed lists must be veda_mask_transpose's output for exactly this
 * CSR, whose rows are ascending and free of repeats (veda_select_blocks'
 * output): a kept block missing from them leaves its share of dQ undefined.
 *   q, k, v, o, d_o: device permuted bf16 [R, D] (o and lse as the forward
 *             wrote them with VEDA_LAYOUT_PERMUTED; d_o's padding rows zero,
 *             as veda_permute_tiles writes them; k's and v's padding rows
 *             zero)
 *   lse:      device fp32 [R] (the forward's natural-log LSE, every row)
 *   row_ptr, col_idx: the forward's CSR; col_ptr, row_idx: its transpose
 *             (veda_mask_transpose)
 *   dq, dk, dv: device permuted bf16 [R, D]; rows of padding slots are zero
 *   workspace: device, bwd_workspace_bytes (contents overwritten): per row
 *             two fp32, per key tile and per kept block one int32, and
 *             nnz x 32 KB of dS
 * Errors: VEDA_ERR_INVALID_ARG if dq, dk, dv are not three different buffers
 * or one of them is an input or the workspace; VEDA_ERR_WORKSPACE if
 * workspace_bytes is too small. */
veda_status veda_block_sparse_attn_bwd(const veda_plan* plan, const void* q, const void* k, const void* v,
                                       const void* o, const void* d_o, const float* lse, const int32_t* row_ptr,
                                       const int32_t* col_idx, const int32_t* col_ptr, const int32_t* row_idx,
                                       float softmax_scale, void* dq, void* dk, void* dv, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Tile-shape vote of the tile-plan search (same source): a host-only step
 * on the error table of `samples` x `candidates` x `heads` (err[s][c][h],
 * host fp64, row-major), e.g. veda_output_error of the output under each
 * candidate tile shape's oracle mask for each sample.
 *   1. every sample votes, per head, for its lowest-error candidate;
 *   2. a head's preferred candidate is the one with the most votes;
 *   3. the layer keeps the max_shapes candidates preferred by the most heads;
 *   4. a head whose preferred candidate is kept uses it, any other head the
 *      kept candidate with the lowest mean error over the samples.
 * Every tie goes to the lower candidate index.  choice: host int32 [heads].
 * VEDA_ERR_INVALID_ARG for non-positive counts or a non-finite error. */
veda_status veda_tile_plan_vote(int32_t samples, int32_t candidates, int32_t heads, const double* err,
                                int32_t max_shapes, int32_t* choice);

#ifdef __cplusplus
}
#endif

#endif /* VEDA_H */
