// Internal declarations shared by the host side of libveda (plan, checks,
// C ABI) and its HIP kernels.  Not installed, not part of the ABI.
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "veda.h"

namespace veda {

constexpr int kTile = 128;          // tokens per tile, rows per query tile
constexpr int kMaxSegments = 8;
constexpr int kMaxShapes = 2;       // at most two tile shapes per layer
constexpr int kMaxTilesPerHead = 16384;
constexpr int kMaxHeatTiles = 4096;

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
// Byte matrix of the kept blocks (sum n_h^2) and per-key-tile counts.
inline int64_t transpose_workspace_bytes(int64_t total_pairs, int64_t total_tiles) {
  return align256(total_pairs) + align256(total_tiles * 4);
}
// Per permuted row: (lse * log2(e), rowsum(dO * O)), fp32 pairs [R, 2]; the
// dispatch order of the key tiles, int32 [T]; per transposed-list entry its
// position in the CSR, int32 [nnz]; then dS of every kept block as bf16
// (kBwdBlockBytes each, in the order of the CSR), written by the dK/dV pass
// and read by the dQ pass.
constexpr int64_t kBwdBlockBytes = 128 * 128 * 2;
inline int64_t bwd_workspace_bytes(int64_t total_rows, int64_t total_tiles, int64_t nnz) {
  return align256(total_rows * 8) + align256(total_tiles * 4) + align256(nnz * 4) + nnz * kBwdBlockBytes;
}
// One fp32 per (block, query slot): each block's sum of p per query.
// veda_dense_lse_heat: nnz x 128 block sums.  veda_attn_fwd_lse_heat (with
// this plan as the dense plan): the same floats split between the selected
// and the rest blocks (one more alignment gap), the rest's columns, one flag
// per tile, two factors per row and an LSE of the selected rows when the
// caller passes none.
inline int64_t heat_workspace_bytes(int64_t nnz, int64_t tiles, int64_t rows) {
  return align256(nnz * 128 * 4) + 256 + align256(nnz * 4) + align256(tiles * 4) + align256(rows * 8) +
         align256(rows * 4);
}
// Per-head partial sums of the two-launch reductions (mask mass: one per 16
// rows; output error: 32 token chunks), two fp64 each.
inline int mass_chunks(int32_t max_tiles) { return (max_tiles + 15) / 16; }
inline int64_t reduce_workspace_bytes(int32_t num_heads, int32_t max_tiles) {
  const int64_t c = mass_chunks(max_tiles) > 32 ? mass_chunks(max_tiles) : 32;
  return align256((int64_t)num_heads * c * 16);
}

// Device view of the tables of one distinct tile shape.  Heads that share a
// shape share these tables (tiling, valid counts, budgets, local CSR offsets).
struct DevShape {
  const int32_t* perm;           // [n * 128] slot -> token, -1 = padding
  const int32_t* valid;          // [n] valid tokens per tile
  const int32_t* tile_seg;       // [n] segment of each tile
  const int32_t* budget;         // [n * S] blocks kept per key segment
  const int32_t* local_row_ptr;  // [n + 1] CSR offsets inside one head
  int32_t num_tiles;
  int32_t seg_first[kMaxSegments];
  int32_t seg_count[kMaxSegments];
};

// Device view of a whole plan, passed to kernels by value.
struct DevPlan {
  int32_t num_heads, head_dim, num_segments, num_shapes;
  int64_t num_tokens, total_rows, total_tiles, total_pairs, nnz;
  int32_t seg_dense[kMaxSegments];   // 1 if every pair with this segment is dense
  int32_t all_dense;                 // budget mode ALL
  DevShape shape[kMaxShapes];
  const int32_t* head_shape;     // [H]
  const int64_t* head_row_off;   // [H] first permuted row
  const int32_t* head_tile_off;  // [H] first global tile / CSR row
  const int64_t* head_pair_off;  // [H] first score
  const int64_t* head_nnz_off;   // [H] first col_idx entry
  const int32_t* row_head;       // [T] head of every global tile
  const int32_t* row_ptr;        // [T + 1] global CSR row pointers
  const int32_t* attn_order;     // [attn_grid] global tile per workgroup, -1 idle
  int32_t attn_grid;
};

// Kernel launchers (veda_kernels.hip).  Shapes are validated by the caller;
// each returns the launch status.
hipError_t launch_permute(const DevPlan& p, const void* src, void* dst, int direction,
                          hipStream_t s);
hipError_t launch_score(const DevPlan& p, const void* q, const void* k, const float* wq,
                        const float* wk, float* scores, void* ws, hipStream_t s);
hipError_t launch_permute_qkv(const DevPlan& p, const void* q, const void* k, const void* v, void* qp,
                              void* kp, void* vt, void* ws, hipStream_t s);
hipError_t launch_score_pooled(const DevPlan& p, const float* wq, const float* wk, float* scores,
                               void* ws, hipStream_t s);
hipError_t launch_select(const DevPlan& p, const float* scores, int32_t* row_ptr,
                         int32_t* col_idx, uint8_t* dense_mask, hipStream_t s);
hipError_t launch_attn_fwd(const DevPlan& p, const void* q, int q_natural, const void* k, const void* vt,
                           const int32_t* row_ptr, const int32_t* col_idx, float scale,
                           void* o, int o_natural, float* lse, uint32_t* visited, hipStream_t s);
hipError_t launch_lse_heat(const DevPlan& p, const void* q, int q_natural, const void* k, const int32_t* row_ptr,
                           const int32_t* col_idx, float scale, float* lse, float* bsum, float* heat,
                           hipStream_t s);
// veda_attn_fwd_lse_heat's scratch: the selected blocks' sums of p (mass,
// sel nnz x 128 floats) and per query the factors that make them shares
// (fac), the rest's block sums (rest_nnz x 128 floats), the rest CSR's
// columns and the per-tile mismatch flags
struct SplitWorkspace {
  float* mass;
  float2* fac;
  float* rest_bsum;
  int32_t* rest_col;
  int32_t* cflag;
  int64_t rest_nnz;
};
hipError_t launch_attn_lse_heat(const DevPlan& sel, const DevPlan& dense, const void* q, int q_natural,
                                const void* k, const void* vt, const int32_t* row_ptr, const int32_t* col_idx,
                                const int32_t* dense_row_ptr, const int32_t* dense_col_idx, float scale, void* o,
                                int o_natural, float* lse_sel, float* dense_lse, float* heat,
                                const SplitWorkspace& ws, hipStream_t s);
hipError_t launch_heat(const DevPlan& p, const void* q, const void* k, const float* lse,
                       float scale, float* heat, hipStream_t s);
hipError_t launch_mask_mass(const DevPlan& p, int32_t max_tiles, const float* heat, const int32_t* row_ptr,
                            const int32_t* col_idx, double* mass, void* ws, hipStream_t s);
hipError_t launch_output_error(const DevPlan& p, int64_t num_tokens, const void* o, const void* o_ref, double* err,
                               void* ws, hipStream_t s);
hipError_t launch_mask_transpose(const DevPlan& p, const int32_t* row_ptr, const int32_t* col_idx, int32_t* col_ptr,
                                 int32_t* row_idx, void* workspace, int64_t total_pairs, hipStream_t s);
hipError_t launch_attn_bwd(const DevPlan& p, const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                           const int32_t* col_ptr, const int32_t* row_idx, float scale, void* dq, void* dk,
                           void* dv, void* workspace, hipStream_t s);

// The static scratch of veda_score_tiles_noalloc: one array per GPU, fixed
// size.  static_scratch() returns its device address on the current device
// (looked up once per device with hipGetSymbolAddress).
constexpr int64_t kStaticScratchBytes = int64_t(128) << 20;
hipError_t static_scratch(void** ptr);

// Scratch the score call needs: pooled features of Q and K (fp32 [T, 3D]
// each) and their projections (fp32 [T, D] each).
inline int64_t score_workspace_bytes(int64_t total_tiles, int32_t head_dim) {
  return total_tiles * (int64_t)head_dim * 4 * (3 + 3 + 1 + 1);
}

}  // namespace veda
