// HIP kernels of libveda for CDNA4 (gfx950, MI355X).
//
//   permute   gather natural [N,H,D] rows into per-head tile order (and back);
//             V can be written per tile transposed, [D][128], the layout the
//             attention kernel streams it in.                    HBM-bound
//   pool      mean (fp64 sum) / max / min of every tile's valid slots
//   project   per-head residual projection, fp64 sequential sums
//   score     pair scores q_hat . k_hat, fp64 sequential sums
//   select    per-row radix top-k on order-preserving 32-bit keys, ties to the
//             lowest key tile, ascending CSR by wavefront ballot compaction
//   attn_fwd  block-sparse flash attention over the CSR, bf16 MFMA
//             (32x32x16), fp32 softmax in the log2 domain against a fixed
//             per-row reference point (exact online-softmax fallback)
//   heat      block heat from the dense LSE, same QK^T machinery, no PV
//   mass      attention mass a block mask keeps (fp64, fixed order)
//   error     relative output error of two outputs per head (fp64)
//   backward  transposed (per key tile) block lists; dV and dK per key tile
//             (dV and dK waves, P' handed over in LDS), dQ per query tile,
//             both with LDS transpose reads and no atomics
//
// The method is the Veda sparse attention of the Miowtion project page
// ("Sparse acceleration (Veda)"; Key Features > "Veda sparse attention") and
// the 128x128 block tiling of "Deploying this checkpoint", section 2.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>

#include "veda_internal.h"

namespace veda {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Values every lane of a workgroup agrees on, moved to scalar registers so
// address arithmetic and buffer resources built from them stay scalar.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// ---------------------------------------------------------------------------
// permute
// ---------------------------------------------------------------------------

// Row-wise gather/scatter: one thread moves 16 bytes (8 channels) of one row.
template <int D>
__global__ void __launch_bounds__(kThreads) permute_rows_kernel(DevPlan p, const uint16_t* __restrict__ src,
                                                               uint16_t* __restrict__ dst, int inverse) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  const int64_t g = (int64_t)blockIdx.x * (kThreads / CH) + threadIdx.x / CH;
  const int c = threadIdx.x % CH;
  if (g >= p.total_rows) return;
  const int64_t tile = g / kTile;
  const int h = p.row_head[tile];
  const DevShape& sh = p.shape[p.head_shape[h]];
  const int64_t s = g - p.head_row_off[h];
  const int32_t tok = sh.perm[s];
  const int64_t nat = ((int64_t)tok * p.num_heads + h) * D + 8 * c;
  if (!inverse) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tok >= 0) v = ld16(src + nat);
    st16(dst + g * D + 8 * c, v);
  } else if (tok >= 0) {
    st16(dst + nat, ld16(src + g * D + 8 * c));
  }
}

// Forward permutation of Q, K and V in one launch, with the pooling of Q and
// K fused in.  Workgroup (tile t, tensor y); thread (cb, sb) owns channels
// 8cb..8cb+7 of slots 8sb..8sb+7: it gathers those eight 16-byte pieces of
// natural rows (for Q and K the D/8 threads sharing sb are consecutive and
// read whole rows; for V the 16 sharing cb are, so that each store writes
// whole 256-byte V^T rows), then
//  - Q, K: writes them as permuted rows and keeps fp64 sums / max / min of
//    the valid ones, combined over sb through LDS in a fixed order;
//  - V:    transposes the 8x8 block in registers and writes 8 rows of the
//    tile-transposed layout.
template <int D>
__global__ void __launch_bounds__(D * 2) permute_qkv_kernel(DevPlan p, const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, uint16_t* __restrict__ qp,
                                                           uint16_t* __restrict__ kp, uint16_t* __restrict__ vt,
                                                           float* __restrict__ feat_q, float* __restrict__ feat_k,
                                                           int y0) {
  constexpr int CB = D / 8;     // channel chunks
  constexpr int SB = 16;        // slot chunks of 8
  __shared__ double s_sum[SB][D];
  __shared__ float s_max[SB][D];
  __shared__ float s_min[SB][D];
  const int64_t t = blockIdx.x;
  const int y = y0 + (int)blockIdx.y;   // tensor: 0 Q, 1 K, 2 V
  // Q, K: the D/8 threads of a slot chunk are consecutive (whole rows per
  // load and store); V: the 16 threads of a channel chunk are (whole
  // 256-byte V^T rows per store)
  const int cb = y == 2 ? (int)threadIdx.x / SB : (int)threadIdx.x % CB;
  const int sb = y == 2 ? (int)threadIdx.x % SB : (int)threadIdx.x / CB;
  const int h = uni(p.row_head[t]);
  const DevShape& sh = p.shape[uni(p.head_shape[h])];
  const int i = (int)(t - uni(p.head_tile_off[h]));
  const int nv = sh.valid[i];
  const int H = p.num_heads;
  const uint16_t* src = y == 0 ? q : (y == 1 ? k : v);
  // the eight slot -> token entries of this thread (two 16-byte reads), then
  // eight independent gathers; padding slots read token 0 and are zeroed
  const u32x4 pa = ld16(sh.perm + (int64_t)kTile * i + 8 * sb);
  const u32x4 pb = ld16(sh.perm + (int64_t)kTile * i + 8 * sb + 4);
  const int32_t toks[8] = {(int32_t)pa[0], (int32_t)pa[1], (int32_t)pa[2], (int32_t)pa[3],
                           (int32_t)pb[0], (int32_t)pb[1], (int32_t)pb[2], (int32_t)pb[3]};
  u32x4 blk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int32_t tk = toks[e] >= 0 ? toks[e] : 0;
    blk[e] = ld16(src + ((int64_t)tk * H + h) * D + 8 * cb);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (toks[e] < 0) blk[e] = u32x4{0u, 0u, 0u, 0u};
  if (y == 2) {
    uint16_t* out = vt + t * (int64_t)D * kTile;
#pragma unroll
    for (int c = 0; c < 8; ++c) {           // channel 8cb + c
      uint32_t wv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a = blk[2 * m][c >> 1], b = blk[2 * m + 1][c >> 1];
        wv[m] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      st16(out + (int64_t)(8 * cb + c) * kTile + 8 * sb, u32x4{wv[0], wv[1], wv[2], wv[3]});
    }
    return;
  }
  uint16_t* dst = y == 0 ? qp : kp;   // qp NULL: Q pooled only
  if (dst) {
#pragma unroll
    for (int e = 0; e < 8; ++e) st16(dst + (t * kTile + 8 * sb + e) * D + 8 * cb, blk[e]);
  }
  float* feat = y == 0 ? feat_q : feat_k;
  if (!feat) return;
  double sum[8];
  float mx[8], mn[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    sum[c] = 0.0;
    mx[c] = -INFINITY;
    mn[c] = INFINITY;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (8 * sb + e >= nv) continue;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t wd = blk[e][c >> 1];
      const float x = __uint_as_float((c & 1) ? (wd & 0xffff0000u) : (wd << 16));
      sum[c] += (double)x;
      mx[c] = fmaxf(mx[c], x);
      mn[c] = fminf(mn[c], x);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    s_sum[sb][8 * cb + c] = sum[c];
    s_max[sb][8 * cb + c] = mx[c];
    s_min[sb][8 * cb + c] = mn[c];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    double tot = 0.0;
    float a = -INFINITY, b = INFINITY;
    for (int r = 0; r < SB; ++r) {
      tot += s_sum[r][d];
      a = fmaxf(a, s_max[r][d]);
      b = fminf(b, s_min[r][d]);
    }
    float* out = feat + t * (int64_t)(3 * D);
    out[d] = (float)(tot / (double)nv);
    out[D + d] = a;
    out[2 * D + d] = b;
  }
}

// ---------------------------------------------------------------------------
// predictor: pool, project, score
// ---------------------------------------------------------------------------

// One workgroup per (tile, tensor).  Thread (row group g, chunk c) sums 8
// channels over rows g, g+RG, ... < valid; partials meet in LDS and are
// combined in a fixed order.  The fp64 sum of bf16 inputs is exact for the
// inputs the method sees, so any order gives the same mean.
template <int D>
__global__ void __launch_bounds__(kThreads) pool_kernel(DevPlan p, const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k, float* __restrict__ feat_q,
                                                       float* __restrict__ feat_k) {
  constexpr int CH = D / 8;
  constexpr int RG = kThreads / CH;
  __shared__ double s_sum[RG][D];
  __shared__ float s_max[RG][D];
  __shared__ float s_min[RG][D];
  const int64_t t = blockIdx.x;
  const uint16_t* x = blockIdx.y ? k : q;
  float* feat = blockIdx.y ? feat_k : feat_q;
  const int h = p.row_head[t];
  const DevShape& sh = p.shape[p.head_shape[h]];
  const int i = (int)(t - p.head_tile_off[h]);
  const int nv = sh.valid[i];
  const int g = threadIdx.x / CH, c = threadIdx.x % CH;
  double sum[8];
  float mx[8], mn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sum[e] = 0.0;
    mx[e] = -INFINITY;
    mn[e] = INFINITY;
  }
  const uint16_t* base = x + t * (int64_t)kTile * D + 8 * c;
  for (int r = g; r < nv; r += RG) {
    u32x4 v = ld16(base + (int64_t)r * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(v[e] << 16);
      const float hi = __uint_as_float(v[e] & 0xffff0000u);
      sum[2 * e] += (double)lo;
      sum[2 * e + 1] += (double)hi;
      mx[2 * e] = fmaxf(mx[2 * e], lo);
      mx[2 * e + 1] = fmaxf(mx[2 * e + 1], hi);
      mn[2 * e] = fminf(mn[2 * e], lo);
      mn[2 * e + 1] = fminf(mn[2 * e + 1], hi);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s_sum[g][8 * c + e] = sum[e];
    s_max[g][8 * c + e] = mx[e];
    s_min[g][8 * c + e] = mn[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    double tot = 0.0;
    float a = -INFINITY, b = INFINITY;
    for (int r = 0; r < RG; ++r) {
      tot += s_sum[r][d];
      a = fmaxf(a, s_max[r][d]);
      b = fminf(b, s_min[r][d]);
    }
    float* out = feat + t * (int64_t)(3 * D);
    out[d] = (float)(tot / (double)nv);
    out[D + d] = a;
    out[2 * D + d] = b;
  }
}

// x_hat[t][d] = fp32(mean[d] + sum_e W[h][d][e] f[t][e]), e ascending, fp64
// (a product of two fp32 values is exact in fp64, so fma = multiply + add).
//
// On the fp64 matrix cores: v_mfma_f64_16x16x4_f64 adds its four products
// to the accumulator one after another in k order, each rounded as an fma
// (checked on gfx950 against sequential fmas over 128-step chains, all
// 65,536 outputs bit-equal), so a chain of them over e = 0, 1, ..., 3D-1 with
// the accumulator starting at the mean is exactly the sequential sum.
// Operand layout of that instruction: A (16 x 4) lane l holds A[l % 16][l / 16],
// B (4 x 16) lane l holds B[l / 16][l % 16], the accumulator's element r of
// lane l is D[l / 16 + 4r][l % 16].  Here rows are tiles, k runs over feature
// channels e and columns are output channels d.
// Workgroup = (16 tiles of one head, head, tensor), 4 waves; wave w owns the
// D/4 output channels from w D/4 on (D/64 16x16 blocks).  W (transposed to
// [e][d]) and the features ([e][tile]) pass through LDS as fp64 in chunks of
// kPrjE channels; the next chunk is loaded into registers while the current
// one is used.  Row strides are odd numbers of doubles, so the transposing
// LDS writes spread over the banks.
typedef __attribute__((ext_vector_type(4))) double f64x4;
constexpr int kPrjE = 32;    // feature channels per LDS chunk
constexpr int kPrjTB = 16;   // tiles per workgroup

template <int D>
__global__ void __launch_bounds__(kThreads) project_kernel(DevPlan p, const float* __restrict__ wq,
                                                          const float* __restrict__ wk,
                                                          const float* __restrict__ feat_q,
                                                          const float* __restrict__ feat_k, float* __restrict__ hat_q,
                                                          float* __restrict__ hat_k) {
  constexpr int E = 3 * D;
  constexpr int NB = D / 64;               // 16-channel blocks per wave
  constexpr int WS = D + 1;                // doubles per LDS row of W^T
  constexpr int FS = kPrjTB + 1;           // doubles per LDS row of the features
  constexpr int P4 = kPrjE / 4;            // 16-byte pieces per chunk row
  constexpr int WP = D * P4 / kThreads;    // W pieces per thread per chunk
  constexpr int FP = kPrjTB * P4;          // feature pieces per chunk (one per thread at most)
  static_assert(E % kPrjE == 0 && WP >= 1 && FP <= kThreads && NB >= 1, "chunking");
  __shared__ double ws[kPrjE * WS];
  __shared__ double fs[kPrjE * FS];
  const int h = blockIdx.y, y = blockIdx.z;
  const int n = p.shape[p.head_shape[h]].num_tiles;
  const int i0 = (int)blockIdx.x * kPrjTB;
  if (i0 >= n) return;
  const int cnt = min(kPrjTB, n - i0);
  const int64_t t0 = p.head_tile_off[h] + i0;
  const float* W = (y ? wk : wq) + (int64_t)h * D * E;
  const float* feat = y ? feat_k : feat_q;
  float* hat = y ? hat_k : hat_q;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  const int dw = wave * (D / 4);
  // the accumulators start at the tiles' means (features 0 .. D-1)
  f64x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[b][r] = (double)feat[(t0 + min(lk + 4 * r, cnt - 1)) * E + dw + 16 * b + lr];
  // piece q of W: row d = q / P4, channels 4 (q % P4) .. + 3 of the chunk
  // (P4 lanes read one row's chunk, 128 contiguous bytes)
  float4 wb[WP], fb = float4{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int c0) {
#pragma unroll
    for (int r = 0; r < WP; ++r) {
      const int q = r * kThreads + tid;
      wb[r] = *reinterpret_cast<const float4*>(W + (int64_t)(q / P4) * E + c0 + 4 * (q % P4));
    }
    if (tid < FP) {
      const int tl = tid / P4;
      fb = tl < cnt ? *reinterpret_cast<const float4*>(feat + (t0 + tl) * E + c0 + 4 * (tid % P4))
                    : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load(0);
#pragma unroll 1
  for (int c0 = 0; c0 < E; c0 += kPrjE) {
    __syncthreads();   // every wave is done with the previous chunk
#pragma unroll
    for (int r = 0; r < WP; ++r) {
      const int q = r * kThreads + tid;
      const int d = q / P4, e = 4 * (q % P4);
      ws[(e + 0) * WS + d] = (double)wb[r].x;
      ws[(e + 1) * WS + d] = (double)wb[r].y;
      ws[(e + 2) * WS + d] = (double)wb[r].z;
      ws[(e + 3) * WS + d] = (double)wb[r].w;
    }
    if (tid < FP) {
      const int tl = tid / P4, e = 4 * (tid % P4);
      fs[(e + 0) * FS + tl] = (double)fb.x;
      fs[(e + 1) * FS + tl] = (double)fb.y;
      fs[(e + 2) * FS + tl] = (double)fb.z;
      fs[(e + 3) * FS + tl] = (double)fb.w;
    }
    __syncthreads();
    if (c0 + kPrjE < E) load(c0 + kPrjE);
#pragma unroll
    for (int s4 = 0; s4 < kPrjE / 4; ++s4) {
      const int e = 4 * s4 + lk;
      const double a = fs[e * FS + lr];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, ws[e * WS + dw + 16 * b + lr], acc[b], 0, 0, 0);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lk + 4 * r < cnt) hat[(t0 + lk + 4 * r) * D + dw + 16 * b + lr] = (float)acc[b][r];
}

// s[i][j] = fp32(sum_d q_hat_i[d] k_hat_j[d]), d ascending in fp64, -0
// written as +0.  On the fp64 matrix cores like the projection: a chain of
// v_mfma_f64_16x16x4_f64 from a zero accumulator over d = 0, 1, ..., D-1 is
// the sequential sum.  Workgroup = 64 x 64 scores of one head; wave w owns
// query rows 16w .. 16w + 15 against all 64 key columns (four 16x16 blocks
// sharing the A operand of each step).  q_hat and k_hat pass through LDS
// kScoreChunk channels at a time, widened to fp64 and transposed to
// [channel][row] with an odd row stride.
constexpr int kScoreChunk = 32;

template <int D>
__global__ void __launch_bounds__(kThreads) score_kernel(DevPlan p, const float* __restrict__ hat_q,
                                                        const float* __restrict__ hat_k, float* __restrict__ scores) {
  static_assert(D % kScoreChunk == 0, "whole channel chunks");
  constexpr int RS = 64 + 1;   // doubles per LDS row
  __shared__ double qs[kScoreChunk * RS];
  __shared__ double ks[kScoreChunk * RS];
  const int h = blockIdx.z;
  const DevShape& sh = p.shape[p.head_shape[h]];
  const int n = sh.num_tiles;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  if (i0 >= n || j0 >= n) return;
  const int64_t t0 = p.head_tile_off[h];
  const int lane = lane_id(), wave = threadIdx.x >> 6, lr = lane & 15, lk = lane >> 4;
  // staging: thread -> (row r, 8 consecutive channels) of the chunk; rows
  // past the head's last tile read the last tile (in bounds) and are zeroed
  constexpr int PER_ROW = kScoreChunk / 8;                 // threads per row
  static_assert(64 * PER_ROW == kThreads, "one 8-channel piece per thread and matrix");
  const int sr = threadIdx.x / PER_ROW, sc = 8 * (threadIdx.x % PER_ROW);
  const bool qin = i0 + sr < n, kin = j0 + sr < n;
  const float* qrow = hat_q + (t0 + min(i0 + sr, n - 1)) * D + sc;
  const float* krow = hat_k + (t0 + min(j0 + sr, n - 1)) * D + sc;
  f64x4 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
  for (int c0 = 0; c0 < D; c0 += kScoreChunk) {
    const float4 q0 = *reinterpret_cast<const float4*>(qrow + c0);
    const float4 q1 = *reinterpret_cast<const float4*>(qrow + c0 + 4);
    const float4 k0 = *reinterpret_cast<const float4*>(krow + c0);
    const float4 k1 = *reinterpret_cast<const float4*>(krow + c0 + 4);
    if (c0 > 0) __syncthreads();       // every wave is done with the previous chunk
    const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      qs[(sc + u) * RS + sr] = qin ? (double)qv[u] : 0.0;
      ks[(sc + u) * RS + sr] = kin ? (double)kv[u] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int s4 = 0; s4 < kScoreChunk / 4; ++s4) {
      const int d = 4 * s4 + lk;
      const double a = qs[d * RS + 16 * wave + lr];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, ks[d * RS + 16 * b + lr], acc[b], 0, 0, 0);
    }
  }
  float* out = scores + p.head_pair_off[h];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int j = j0 + 16 * b + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 16 * wave + lk + 4 * r;
      if (i >= n || j >= n) continue;
      uint32_t u = __float_as_uint((float)acc[b][r]);
      if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0 -> +0
      out[(int64_t)i * n + j] = __uint_as_float(u);
    }
  }
}

// ---------------------------------------------------------------------------
// select: budgeted top-k per row
// ---------------------------------------------------------------------------

// Order-preserving key: larger score <=> larger unsigned key; -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// One 64-lane workgroup per CSR row.  Per budgeted key segment a 4-pass,
// 8-bit radix select finds the k-th largest key T and how many keys equal to
// T to take; the final pass walks the row's columns in ascending 64-wide
// chunks, decides each column and compacts with ballots, so col_idx comes out
// ascending.
__global__ void __launch_bounds__(64) select_kernel(DevPlan p, const float* __restrict__ scores,
                                                   int32_t* __restrict__ row_ptr_out, int32_t* __restrict__ col_idx,
                                                   uint8_t* __restrict__ dense_mask) {
  __shared__ uint32_t hist[256];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  const int h = p.row_head[t];
  const DevShape& sh = p.shape[p.head_shape[h]];
  const int n = sh.num_tiles;
  const int i = (int)(t - p.head_tile_off[h]);
  const int S = p.num_segments;
  const int A = sh.tile_seg[i];
  const float* srow = scores + p.head_pair_off[h] + (int64_t)i * n;
  const int32_t rp0 = p.row_ptr[t];
  const int32_t row_len = p.row_ptr[t + 1] - rp0;
  if (lane == 0) {
    row_ptr_out[t] = rp0;
    if (t == p.total_tiles - 1) row_ptr_out[t + 1] = p.row_ptr[t + 1];
  }
  // per segment: mode 0 = all, 1 = diagonal only / nothing, 2 = radix threshold
  uint32_t thr[kMaxSegments];
  int32_t rem[kMaxSegments], mode[kMaxSegments];
#pragma unroll
  for (int B = 0; B < kMaxSegments; ++B) {
    thr[B] = 0u;
    rem[B] = 0;
    mode[B] = 1;
    if (B >= S) continue;
    const int first = sh.seg_first[B], count = sh.seg_count[B];
    const int kb = sh.budget[(int64_t)i * S + B];
    if (kb >= count) {
      mode[B] = 0;
      continue;
    }
    const int diag = (A == B) ? i : -1;
    int need = kb - (diag >= 0 ? 1 : 0);
    if (need <= 0) continue;
    mode[B] = 2;
    uint32_t prefix = 0u, pmask = 0u;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int b = lane; b < 256; b += 64) hist[b] = 0u;
      __syncthreads();
      for (int j = first + lane; j < first + count; j += 64) {
        if (j == diag) continue;
        const uint32_t key = order_key(srow[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      // inclusive suffix sum over lanes: sum of bins of this lane and above
      uint32_t suf = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += y;
      }
      uint32_t above = suf - mine;
      int found = 0, digit = 0, need_left = 0;
      if (above < (uint32_t)need && (uint32_t)need <= suf) {
        const uint32_t cs[4] = {c0, c1, c2, c3};
        for (int b = 3; b >= 0; --b) {
          if (above + cs[b] >= (uint32_t)need) {
            digit = 4 * lane + b;
            need_left = need - (int)above;
            found = 1;
            break;
          }
          above += cs[b];
        }
      }
      const uint64_t fm = __ballot(found);
      const int src = fm ? __ffsll((unsigned long long)fm) - 1 : 0;
      digit = __shfl(digit, src, 64);
      need = __shfl(need_left, src, 64);
      prefix |= (uint32_t)digit << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    thr[B] = prefix;
    rem[B] = need;
  }
  // final pass over the columns in ascending order
  int32_t eq_seen[kMaxSegments];
#pragma unroll
  for (int B = 0; B < kMaxSegments; ++B) eq_seen[B] = 0;
  int32_t pos = 0;
  const uint64_t below = lanes_below();
  uint8_t* mrow = dense_mask ? dense_mask + p.head_pair_off[h] + (int64_t)i * n : nullptr;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int j = c0 + lane;
    const bool in = j < n;
    const int Bj = in ? sh.tile_seg[j] : -1;
    const uint32_t key = in ? order_key(srow[j]) : 0u;
    bool sel = false;
#pragma unroll
    for (int B = 0; B < kMaxSegments; ++B) {
      if (B >= S) continue;
      const bool mine = (Bj == B);
      if (mode[B] == 0) {
        sel = sel || mine;
        continue;
      }
      const bool isdiag = mine && (A == B) && (j == i);
      if (mode[B] == 1) {
        sel = sel || isdiag;
        continue;
      }
      const bool eq = mine && !isdiag && key == thr[B];
      const uint64_t em = __ballot(eq);
      const int rank = eq_seen[B] + __popcll(em & below);
      if (mine) sel = isdiag || (key > thr[B] && !isdiag) || (eq && rank < rem[B]);
      eq_seen[B] += __popcll(em);
    }
    const uint64_t sm = __ballot(sel);
    const int32_t at = pos + __popcll(sm & below);
    if (sel && at < row_len) col_idx[rp0 + at] = j;  // a row never exceeds its budget
    pos += __popcll(sm);
    if (mrow && in) mrow[j] = sel ? 1 : 0;
  }
}

// The same selection for long rows (more than 512 key tiles), with the row
// staged in LDS: the order keys and key segments are read from memory once,
// and the four radix passes and the final pass read LDS, where select_kernel
// reads a 4.5 KB row from the cache five times.  Short rows stay with
// select_kernel: their keys stay in the L1 cache between passes anyway.  The
// LDS (keys, 8-bit segments, one 256-bin histogram; about 7 KB for 1,152
// columns) is kept small so that many rows share a CU.
template <int CH>
__global__ void __launch_bounds__(64) select_staged_kernel(DevPlan p, const float* __restrict__ scores,
                                                          int32_t* __restrict__ row_ptr_out,
                                                          int32_t* __restrict__ col_idx,
                                                          uint8_t* __restrict__ dense_mask) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_key[64 * CH];
  __shared__ int8_t s_seg[64 * CH];   // key segment of the column, -1 past the row
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  const int h = p.row_head[t];
  const DevShape& sh = p.shape[p.head_shape[h]];
  const int n = sh.num_tiles;
  const int i = (int)(t - p.head_tile_off[h]);
  const int S = p.num_segments;
  const int A = sh.tile_seg[i];
  const float* srow = scores + p.head_pair_off[h] + (int64_t)i * n;
  const int32_t rp0 = p.row_ptr[t];
  const int32_t row_len = p.row_ptr[t + 1] - rp0;
  const int nch = (n + 63) / 64;
  if (lane == 0) {
    row_ptr_out[t] = rp0;
    if (t == p.total_tiles - 1) row_ptr_out[t + 1] = p.row_ptr[t + 1];
  }
  for (int r = 0; r < nch; ++r) {
    const int j = 64 * r + lane;
    const bool in = j < n;
    s_key[j] = in ? order_key(srow[j]) : 0u;
    s_seg[j] = (int8_t)(in ? sh.tile_seg[j] : -1);
  }
  // per segment: mode 0 = all, 1 = diagonal only / nothing, 2 = radix threshold
  uint32_t thr[kMaxSegments];
  int32_t rem[kMaxSegments], mode[kMaxSegments];
#pragma unroll
  for (int B = 0; B < kMaxSegments; ++B) {
    thr[B] = 0u;
    rem[B] = 0;
    mode[B] = 1;
    if (B >= S) continue;
    const int first = sh.seg_first[B], count = sh.seg_count[B];
    const int kb = sh.budget[(int64_t)i * S + B];
    if (kb >= count) {
      mode[B] = 0;
      continue;
    }
    const int diag = (A == B) ? i : -1;
    int need = kb - (diag >= 0 ? 1 : 0);
    if (need <= 0) continue;
    mode[B] = 2;
    uint32_t prefix = 0u, pmask = 0u;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int b = lane; b < 256; b += 64) hist[b] = 0u;
      __syncthreads();   // also makes the staged row visible on the first pass
      for (int j = first + lane; j < first + count; j += 64) {
        if (j == diag) continue;
        const uint32_t key = s_key[j];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      // inclusive suffix sum over lanes: sum of bins of this lane and above
      uint32_t suf = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += y;
      }
      uint32_t above = suf - mine;
      int found = 0, digit = 0, need_left = 0;
      if (above < (uint32_t)need && (uint32_t)need <= suf) {
        const uint32_t cs[4] = {c0, c1, c2, c3};
        for (int b = 3; b >= 0; --b) {
          if (above + cs[b] >= (uint32_t)need) {
            digit = 4 * lane + b;
            need_left = need - (int)above;
            found = 1;
            break;
          }
          above += cs[b];
        }
      }
      const uint64_t fm = __ballot(found);
      const int src = fm ? __ffsll((unsigned long long)fm) - 1 : 0;
      digit = __shfl(digit, src, 64);
      need = __shfl(need_left, src, 64);
      prefix |= (uint32_t)digit << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    thr[B] = prefix;
    rem[B] = need;
  }
  __syncthreads();   // the staged row is visible even when no segment needed a radix pass
  // final pass over the columns in ascending order
  int32_t eq_seen[kMaxSegments];
#pragma unroll
  for (int B = 0; B < kMaxSegments; ++B) eq_seen[B] = 0;
  int32_t pos = 0;
  const uint64_t below = lanes_below();
  uint8_t* mrow = dense_mask ? dense_mask + p.head_pair_off[h] + (int64_t)i * n : nullptr;
  for (int r = 0; r < nch; ++r) {
    const int j = 64 * r + lane;
    const bool in = j < n;
    const int Bj = s_seg[j];
    const uint32_t key = s_key[j];
    bool sel = false;
#pragma unroll
    for (int B = 0; B < kMaxSegments; ++B) {
      if (B >= S) continue;
      const bool mine = (Bj == B);
      if (mode[B] == 0) {
        sel = sel || mine;
        continue;
      }
      const bool isdiag = mine && (A == B) && (j == i);
      if (mode[B] == 1) {
        sel = sel || isdiag;
        continue;
      }
      const bool eq = mine && !isdiag && key == thr[B];
      const uint64_t em = __ballot(eq);
      const int rank = eq_seen[B] + __popcll(em & below);
      if (mine) sel = isdiag || (key > thr[B] && !isdiag) || (eq && rank < rem[B]);
      eq_seen[B] += __popcll(em);
    }
    const uint64_t sm = __ballot(sel);
    const int32_t at = pos + __popcll(sm & below);
    if (sel && at < row_len) col_idx[rp0 + at] = j;  // a row never exceeds its budget
    pos += __popcll(sm);
    if (mrow && in) mrow[j] = sel ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// block-sparse attention forward
// ---------------------------------------------------------------------------
//
// One workgroup (4 waves) per (head, 128-row query tile); wave w owns query
// rows 32w .. 32w+31.  Per key block the wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T from registers), so
// each lane holds one query column and the softmax reductions over keys stay
// inside the lane plus one exchange with the lane 32 away.  Then
// O^T += V^T P^T with A = V^T from LDS and B = P^T straight from the S^T
// registers: the K rows of each 32-key group are stored in LDS in the order
// pi(m) (bits 2 and 3 of m swapped) so that the eight S^T values a lane holds
// for one 16-key MFMA step are eight consecutive keys, i.e. one 16-byte
// V^T read.  LDS rows are XOR-swizzled by 16-byte chunk (chunk ^ (row & 15))
// so the 16-byte operand reads of consecutive lanes hit distinct banks.

__device__ __forceinline__ int pi_row(int m) {  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Key index (0..127 inside the block) held by S^T register r of key group kt.
__device__ __forceinline__ int sacc_key(int kt, int r, int hl) {
  return 32 * kt + 16 * (r >> 3) + 8 * hl + (r & 7);
}

// LDS synchronisation without the compiler's implicit full memory fences: a
// wave first waits for its own LDS reads (lgkmcnt) and, where asked, for all
// but its `pending` newest vector-memory operations (the asynchronous tile
// copies into LDS), then meets the other waves at s_barrier.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
template <int PENDING>
__device__ __forceinline__ void dma_sync() {
  static_assert(PENDING >= 0 && PENDING < 16, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | PENDING);  // vmcnt(PENDING) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Asynchronous copy of one K tile (rows in pi order, 16-byte chunks
// XOR-swizzled) straight into LDS through a buffer resource: every lane moves
// 16 bytes per instruction and the wave's 64 chunks land contiguously at a
// wave-uniform LDS base (M0), so the swizzle is applied on the global side.
// Chunk q = it*256 + tid sits in LDS row m = q / CH; with 256 threads that row
// is it*(256/CH) + tid/CH and its swizzled column does not depend on `it`, so
// all of a thread's instructions use one byte offset (VGPR) plus a uniform
// step (SGPR).  The resource covers one head's rows, so the hardware range
// check keeps every copy inside that head.
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, dword data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int64_t bytes) {
  const int records = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;   // integer compare, stays scalar
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, records, kBufferWord3);
}

template <int D>
__device__ __forceinline__ int k_lane_offset(int tid) {   // bytes; tid = thread index inside 256
  constexpr int CH = D / 8;
  const int r = tid / CH, pc = tid % CH;      // row inside a 256/CH-row step
  const int c = pc ^ (r & (CH - 1));
  const int key = (r & ~31) | pi_row(r & 31);
  return 2 * (key * D + 8 * c);
}
// Copy half hh (rows 64hh .. 64hh+63, i.e. key groups 2hh and 2hh+1) of a
// K tile into its own LDS array `dst`; D/32 instructions per thread.
template <int D>
__device__ __forceinline__ void dma_k_half(uint16_t* __restrict__ dst, __amdgpu_buffer_rsrc_t rk, int tile_byte,
                                           int lane_off, int wave, int hh) {
  constexpr int CH = D / 8;
  constexpr int STEP = kThreads / CH;           // rows per instruction
  static_assert(STEP % 32 == 0 || 32 % STEP == 0, "pi order stays inside one step");
#pragma unroll
  for (int it = 0; it < 64 / STEP; ++it) {
    const int r0 = it * STEP;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst + r0 * D + 512 * wave, 16, lane_off,
                                             tile_byte + (64 * hh + r0) * D * 2, 0, 0);
  }
}

// V^T in LDS: two halves [D][64 keys] (keys 64hh .. 64hh+63) in separate
// arrays, so the half a wave has finished with can be refilled while the
// other is in use.  In a half-row of eight 16-byte chunks, chunk c sits at
// position c ^ ((d >> 1) & 7): the 16 rows read by 16 consecutive lanes then
// start in 16 distinct 4-bank groups.
__device__ __forceinline__ int vt_lane_offset(int tid) {   // bytes; tid = thread index inside 256
  const int r = tid / 8, pos = tid % 8;                    // row inside a 32-row step
  const int c = pos ^ ((r >> 1) & 7);
  return 2 * (r * kTile + 8 * c);
}
template <int D>
__device__ __forceinline__ void dma_vt_half(uint16_t* __restrict__ dst, __amdgpu_buffer_rsrc_t rv, int tile_byte,
                                            int lane_off, int wave, int hh) {
#pragma unroll
  for (int it = 0; it < D / 32; ++it)            // 32 rows of 64 keys per instruction
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + it * 32 * 64 + 512 * wave, 16, lane_off,
                                             tile_byte + it * 32 * kTile * 2 + hh * 128, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Synchronous copy (plain loads and LDS stores) of one K tile and (with V)
// one V^T tile into the four half arrays in the layouts the asynchronous
// copies produce.
template <int D, bool V>
__device__ __forceinline__ void copy_kv_halves(uint16_t* __restrict__ kh0, uint16_t* __restrict__ kh1,
                                               uint16_t* __restrict__ vh0, uint16_t* __restrict__ vh1,
                                               const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg) {
  constexpr int CH = D / 8;
#pragma unroll 1
  for (int q = threadIdx.x; q < kTile * CH; q += kThreads) {
    const int m = q / CH, pos = q % CH;               // LDS row (pi order) and chunk position
    const int key = (m & ~31) | pi_row(m & 31);
    const int cc = pos ^ (m & (CH - 1));
    uint16_t* dst = (m < 64 ? kh0 : kh1) + (m & 63) * D + 8 * pos;
    st16(dst, ld16(kg + (int64_t)key * D + 8 * cc));
  }
  if (!V) return;
#pragma unroll 1
  for (int q = threadIdx.x; q < D * 16; q += kThreads) {
    const int d = q / 16, pc = q % 16;                // V^T row and 16-byte chunk position in LDS
    const int hh = pc / 8, pos = pc % 8;
    const int cc = pos ^ ((d >> 1) & 7);
    uint16_t* dst = (hh == 0 ? vh0 : vh1) + d * 64 + 8 * pos;
    st16(dst, ld16(vg + (int64_t)d * kTile + 64 * hh + 8 * cc));
  }
}

// S^T of key group kt (keys 32kt .. 32kt+31) against the wave's 32 queries,
// accumulated onto `init`; khalf is the LDS array of K rows 64(kt/2) ...
template <int D>
__device__ __forceinline__ f32x16 qk_group(const uint16_t* __restrict__ khalf, const bf16x8 (&qf)[D / 16], int kt,
                                           const f32x16& init) {
  constexpr int CH = D / 8;
  const int lane = lane_id();
  const int ln = lane & 31, hl = lane >> 5;
  const int m = 32 * (kt & 1) + ln;
  f32x16 acc = init;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(khalf + m * D + 8 * ((2 * s + hl) ^ (m & (CH - 1)))));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], acc, 0, 0, 0);
  }
  return acc;
}

// O^T += V^T P^T over key group kt; vhalf is the LDS array of V^T keys
// 64(kt/2) ..; pg[s2] holds the lane's P values for keys 32kt + 16s2 + 8hl
// .. +7.
template <int D>
__device__ __forceinline__ void pv_group(const uint16_t* __restrict__ vhalf, const bf16x8 (&pg)[2], int kt,
                                         f32x16 (&oacc)[D / 32]) {
  const int lane = lane_id();
  const int ln = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int c = 4 * (kt & 1) + 2 * s2 + hl;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = 32 * db + ln;
      const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(vhalf + d * 64 + 8 * (c ^ ((ln >> 1) & 7))));
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pg[s2], oacc[db], 0, 0, 0);
    }
  }
}

// One step of the continuous pipeline: S^T of key group kt (from khalf)
// and O^T += V^T P^T over key group ktv (from vhalf, P in pg), issued
// alternately so that neither MFMA chain waits on its own accumulator.
template <int D>
__device__ __forceinline__ f32x16 qk_pv_step(const uint16_t* __restrict__ khalf, const bf16x8 (&qf)[D / 16], int kt,
                                             const uint16_t* __restrict__ vhalf, const bf16x8 (&pg)[2], int ktv,
                                             f32x16 (&oacc)[D / 32]) {
  constexpr int CH = D / 8;
  constexpr int NQ = D / 16, NV = 2 * (D / 32);
  static_assert(NQ == NV, "as many PV as QK products per step");
  const int lane = lane_id();
  const int ln = lane & 31, hl = lane >> 5;
  const int m = 32 * (kt & 1) + ln;
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(khalf + m * D + 8 * ((2 * s + hl) ^ (m & (CH - 1)))));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], acc, 0, 0, 0);
    const int s2 = s / (D / 32), db = s % (D / 32);
    const int c = 4 * (ktv & 1) + 2 * s2 + hl;
    const int d = 32 * db + ln;
    const bf16x8 v = __builtin_bit_cast(bf16x8, ld16(vhalf + d * 64 + 8 * (c ^ ((ln >> 1) & 7))));
    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, pg[s2], oacc[db], 0, 0, 0);
  }
  return acc;
}

// Key slots >= nj of group kt become -inf (the singleton mask rule: slots at
// or past a tile's valid count are padding).
__device__ __forceinline__ void mask_group(f32x16& sg, int kt, int nj, int hl) {
  if (32 * kt + 32 <= nj) return;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (sacc_key(kt, r, hl) >= nj) sg[r] = -INFINITY;
}

// p = exp2(s*c - m) for the lane's 16 keys of a group, packed to bf16 in key
// order; with SUM, also returns the lane's fp32 sum of p.
// (Partial sums start from the first pair rather than from 0: p >= 0, so
// 0 + x == x and the order of the sum is unchanged, one add fewer per pair.)
template <bool SUM>
__device__ __forceinline__ float exp_group(const f32x16& sg, float c, float m, bf16x8 (&pg)[2]) {
  float acc[4];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sg[8 * s2 + 2 * e], c, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sg[8 * s2 + 2 * e + 1], c, -m));
      pk[e] = pack_bf16x2(p0, p1);
      if (SUM) acc[e] = s2 == 0 ? p0 + p1 : acc[e] + (p0 + p1);
    }
    pg[s2] = __builtin_bit_cast(bf16x8, pk);
  }
  return SUM ? (acc[0] + acc[1]) + (acc[2] + acc[3]) : 0.0f;
}

// The lane's fp32 sum of p = exp2(s*c - m) over a group's 16 keys, in the
// same order as exp_group<true> (so both give bitwise the same sum), without
// packing p.
__device__ __forceinline__ float exp_sum(const f32x16& sg, float c, float m) {
  float acc[4];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sg[8 * s2 + 2 * e], c, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sg[8 * s2 + 2 * e + 1], c, -m));
      acc[e] = s2 == 0 ? p0 + p1 : acc[e] + (p0 + p1);
    }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Scheduling pattern for one pipeline step: kLdsAhead LDS operand reads
// ahead, then per MFMA one more read and up to `valu` vector instructions, so
// the softmax work is spread between the MFMAs and an MFMA's operand has
// usually arrived when it issues (a wave issues in order: an operand wait
// also holds back the VALU work behind it).
constexpr int kLdsAhead = 2;
template <int NMFMA, int VALU>
__device__ __forceinline__ void interleave_step() {
  __builtin_amdgcn_sched_group_barrier(0x100, kLdsAhead, 0);  // DS read
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // DS read
    if (VALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);   // VALU
  }
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// Largest row sum of p that the fast pass accepts (p <= 2^64 keeps O and l
// finite), and the largest ratio of the removed padding mass to the
// remaining sum (bounds the cancellation in l).
constexpr float kMaxRowSum = 18446744073709551616.0f;   // 2^64
constexpr float kMaxPadRatio = 8.0f;

// Number of padding keys (slots >= nv) among the 64 keys of a block that a
// lane of half hh holds: the 16-byte chunks c = 2v + hh, v = 0..7, i.e. keys
// 8c .. 8c+7.
__device__ __forceinline__ int half_pads(int nv, int hh) {
  int n = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) n += min(max(8 * (2 * v + hh) + 8 - nv, 0), 8);
  return n;
}

// One workgroup of 4 waves per (head, 128-row query tile).  A key block is
// worked in four 32-key groups, software-pipelined inside each wave: the QK^T
// MFMAs of group t are issued together with the PV MFMAs of group t-2 and the
// softmax VALU work of group t-1, none of which depend on each other, so one
// wave keeps the matrix core and the vector ALU busy at the same time.  With
// PV the pipeline runs over the whole row, across block boundaries, so every
// step has the same mix (run_fast_pv); the LSE-only pass pipelines each block
// on its own.  VALU work competes with the matrix core for issue slots and
// for power (under random bf16 operands the chip runs these kernels at about
// two thirds of its nominal clock), so the fast pass spends none on maxima,
// rescaling or masking:
//
// Reference point.  p = exp2(s*c - m), c = softmax_scale * log2(e), with one
// m per query for the whole row: the exact maximum of the row's first key
// group.  Softmax does not depend on m; what matters is that no p overflows,
// and the first group already holds p = 1 for its largest key.
//
// Padding keys.  Key slots at or past a tile's valid count hold zero rows of
// K and zero columns of V^T (the permutation writes them so), so their logit
// is exactly 0, their p is exp2(-m) and their PV product is zero.  Instead of
// masking, the row's count of padding keys times exp2(-m) is subtracted from
// l at the end.
//
// Guard.  A valid query row whose l exceeds kMaxRowSum (a logit more than
// 64 log2 units above the first group's maximum; this also keeps O finite) or
// whose removed padding mass exceeds kMaxPadRatio times its final l is
// recomputed, together with the rest of its workgroup, by the classic online
// softmax (explicit masking, exact running maximum, O and l rescaled whenever
// it grows), block by block with plain synchronous tile copies.
//
// K and V^T are single buffers per workgroup, each in two 64-key halves
// (four LDS arrays) that are refilled separately as soon as every wave is
// done with them (run_fast_pv and the block lambda below say when).  Two
// workgroups share a CU (72 KB of LDS each).
//
// The attention and the dense heat of one layer split the dense row of a
// query tile in two (veda_attn_fwd_lse_heat): its selected blocks and the
// rest.
//  PV and HB (attn_mass_kernel): the attention over the selected row that
//    also keeps, per selected block and query, the block's sum of p (bsum)
//    and, per query, the two factors that turn those sums into the block's
//    share of the query's probability over the selected blocks (fac).
//  HB and REST (rest_heat_kernel): the LSE-only pass over the rest of the
//    dense row (the complement list); at the end of the row it joins its sum
//    with the selected row's LSE into the dense LSE and writes the heat of
//    every block of the dense row, the selected ones from the attention's
//    block sums and factors.
// So no block's QK^T product is computed twice.
struct HeatSplit {
  const int32_t* srow;    // the selected CSR (REST)
  const int32_t* scol;
  const int32_t* cflag;   // per query tile: the two lists do not match (REST)
  const float* lse_sel;   // the selected row's LSE, natural log (REST)
  const float* mass;      // per selected block and query, the sum of p (REST)
  float2* fac;            // per query: share = bsum * x - pads * y (MASS writes, REST reads)
};

template <int D, bool PV, bool HB, bool REST = false>
__device__ __forceinline__ void attn_fwd_body(const DevPlan& p, const uint16_t* __restrict__ q, int q_natural,
                                              const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
                                              const int32_t* __restrict__ row_ptr,
                                              const int32_t* __restrict__ col_idx, float scale_log2,
                                              uint16_t* __restrict__ o, int o_natural, float* __restrict__ lse,
                                              uint32_t* __restrict__ visited, float* __restrict__ bsum,
                                              float* __restrict__ heat, const HeatSplit hs) {
  static_assert(!REST || (HB && !PV), "the rest of the dense row is an LSE-only heat pass");
  constexpr bool MASS = PV && HB;
  constexpr int H = D / 32;   // copy instructions per thread and half tile (K or V^T)
  constexpr int kRowList = 2048;
  // K and V^T halves as four separate arrays: the compiler then knows that
  // reads of one half do not depend on copies into another, and does not
  // make those reads wait for the copies.
  __shared__ __attribute__((aligned(16))) uint16_t kh0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t kh1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vh0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vh1[64 * D];
  __shared__ int32_t rowlist[kRowList];
  __shared__ int32_t redo;
  __shared__ float s_inv[HB ? kTile : 1];   // heat: per query, the factor of its block sums
  __shared__ float s_pe[HB ? kTile : 1];    // heat: per query, one padding key's share of its row
  __shared__ float s_sel[REST ? kTile : 1]; // rest: per query, the factors of its selected blocks' sums
  __shared__ float s_spe[REST ? kTile : 1];
  const int t = uni(p.attn_order[blockIdx.x]);
  if (t < 0) return;
  const int h = uni(p.row_head[t]);
  const DevShape& sh = p.shape[uni(p.head_shape[h])];
  const int nt = sh.num_tiles;
  const int i = t - uni(p.head_tile_off[h]);
  const int64_t hrow = uni64(p.head_row_off[h]);
  const int64_t row0 = hrow + (int64_t)kTile * i;
  const int64_t htile = uni(p.head_tile_off[h]);
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + hrow * D, (int64_t)nt * kTile * D * 2);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(vt + htile * D * kTile, (int64_t)nt * kTile * D * 2);
  const int wave = uni(threadIdx.x >> 6);
  // REST: the row of the complement list sits at the dense row's start minus
  // the selected entries before it
  const int beg = uni(REST ? row_ptr[t] - hs.srow[t] : row_ptr[t]);
  const int end = uni(REST ? row_ptr[t + 1] - hs.srow[t + 1] : row_ptr[t + 1]);
  const int w = threadIdx.x >> 6, lane = lane_id(), ln = lane & 31, hl = lane >> 5;
  const int koff = k_lane_offset<D>(threadIdx.x), voff = vt_lane_offset(threadIdx.x);
  const float c = scale_log2;
  const bool qvalid = 32 * w + ln < sh.valid[i];
  if (threadIdx.x == 0) redo = 0;

  // Q^T operand: query row 32w + ln, channels 16s + 8hl .. +7; from the
  // permuted rows, or gathered from the natural [N, H, D] rows through the
  // slot -> token table (a padding slot reads zeros, as its permuted row holds)
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = q + (row0 + 32 * w + ln) * D + 8 * hl;
    bool qzero = false;
    if (q_natural) {
      const int tok = sh.perm[(int64_t)kTile * i + 32 * w + ln];
      qzero = tok < 0;
      qrow = q + ((int64_t)(qzero ? 0 : tok) * p.num_heads + h) * D + 8 * hl;
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, qzero ? u32x4{0u, 0u, 0u, 0u} : ld16(qrow + 16 * s));
  }

  f32x16 oacc[D / 32];
  float m_run, l_run;   // reference point (log2 units) and the lane's sum of p
  int npad;             // fast pass: padding keys over the row's blocks
  float bs = 0.0f;      // heat: the lane's sum of p over the current block
  float pend_b = 0.0f;  // heat: a finished block's sum per query, stored one block later
  int pend_pos = -1;    // heat: its position in the CSR (-1: none pending)

  // The row's key tiles, staged in LDS as (tile << 14 | pads1 << 7 | pads0)
  // (padsX = half_pads of the tile's valid count) so the loop issues no
  // vector loads besides the tile copies; rows longer than kRowList refill it
  // at that boundary.
  auto fill_entries = [&](const int32_t* __restrict__ cols, int base, int lim) {
    for (int e = threadIdx.x; e < kRowList && base + e < lim; e += kThreads) {
      const int jj = min(max(cols[base + e], 0), nt - 1);   // stay inside the head
      const int nv = sh.valid[jj];
      rowlist[e] = (jj << 14) | (half_pads(nv, 1) << 7) | half_pads(nv, 0);
    }
  };
  auto fill_list = [&](int base) { fill_entries(col_idx, base, end); };

  // exact maximum of a group over both lane halves
  auto group_max = [&](const f32x16& sg) {
    float gm = sg[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) gm = fmaxf(gm, sg[r]);
    return fmaxf(gm, __shfl_xor(gm, 32, 64));
  };

  // Keeps a group's softmax inside its own pipeline step: without it the
  // compiler sinks the (pure) VALU work past the step's barrier and copy
  // branch to its use in the next step, which leaves this step's MFMAs
  // without VALU work and doubles the next step's.
  auto pin = [](bf16x8 (&pg)[2]) { asm volatile("" : "+v"(pg[0]), "+v"(pg[1])); };

  // Without PV a group's softmax step is only the sum of p (pinned, so that
  // it stays in its pipeline step like the packed p with PV).
  auto pin_sum = [](float& l) { asm volatile("" : "+v"(l)); };

  // One key block of the LSE-only fast pass (without PV: the dense LSE and
  // the heat; the attention itself runs run_fast_pv below).  Steps are
  // separated by scheduling barriers so that the compiler keeps each step's
  // operand reads and MFMAs together with that step's softmax work (and
  // register lifetimes short).  It also issues the asynchronous copies of
  // the next block's K; `compute` = false runs only those (the pass's first
  // iteration).
  // With HB each finished block's sum of p per query (both lane halves) goes
  // to bsum[position][query]; the store waits until the next block's first
  // copy wait, where no copy is in flight, so the copy waits (which count
  // stores too) keep their meaning.
  auto flush_block_sum = [&]() {
    if constexpr (HB) {
      if (pend_pos >= 0) {
        if (hl == 0) bsum[(int64_t)pend_pos * kTile + 32 * w + ln] = pend_b;
        pend_pos = -1;
      }
    }
  };
  // the sum of p of one group, into l and (HB) the block's sum
  auto sum_group = [&](const f32x16& sg, bool first_of_block) {
    const float g = exp_sum(sg, c, m_run);
    if constexpr (!REST) {   // REST: l gathers whole blocks' sums in store_block_sum
      l_run += g;
      pin_sum(l_run);
    }
    if constexpr (HB) {
      bs = first_of_block ? g : bs + g;
      pin_sum(bs);
    }
  };
  auto block = [&](bool compute, bool first, int ent, bool more, int jn, int bpos) {
    const f32x16 zero16 = {};
    f32x16 s0, s1, s2, s3;
    if (compute) {
      s0 = qk_group<D>(kh0, qf, 0, zero16);
      interleave_step<8, 0>();
      if (first) m_run = group_max(s0) * c;   // finite: key 0 always exists
      __builtin_amdgcn_sched_barrier(0);
      s1 = qk_group<D>(kh0, qf, 1, zero16);
      sum_group(s0, true);
      interleave_step<8, 6>();
    }
    // every wave is done with K rows 0-63
    dma_sync<0>();
    flush_block_sum();
    if (more) dma_k_half<D>(kh0, rk, jn * kTile * D * 2, koff, wave, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (compute) {
      s2 = qk_group<D>(kh1, qf, 2, zero16);
      sum_group(s1, false);
      interleave_step<8, 3>();
      __builtin_amdgcn_sched_barrier(0);
      s3 = qk_group<D>(kh1, qf, 3, zero16);
      sum_group(s2, false);
      interleave_step<8, 3>();
    }
    // every wave is done with K rows 64-127 (with HB the block-sum store
    // issued before the K copies is allowed to stay in flight)
    if (more) dma_sync<HB ? H + 1 : H>(); else dma_sync<0>();
    if (more) dma_k_half<D>(kh1, rk, jn * kTile * D * 2, koff, wave, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (compute) {
      sum_group(s3, false);
      interleave_step<0, 6>();
      __builtin_amdgcn_sched_barrier(0);
      npad += ((ent >> 7) & 127) + (ent & 127);
      if constexpr (HB) {
        pend_b = bs + __shfl_xor(bs, 32, 64);
        pend_pos = bpos;
      }
    }
  };

  auto reset_row = [&]() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.0f;
    npad = 0;
  };

  // LSE-only fast pass.  Iteration b computes block b and copies block b+1;
  // the first iteration (b = beg-1) only copies block beg.  Its K copies come
  // from two call sites: the compiler tracks only a few distinct copy sites
  // precisely and makes every LDS read wait for all copies once there are
  // more.
  auto run_fast = [&]() {
    reset_row();
    fill_list(beg);
    dma_sync<0>();
    int ent = 0;
    int en = uni(beg < end ? rowlist[0] : 0);
    for (int b = beg - 1; b < end; ++b) {
      const bool more = b + 1 < end;
      const int jn = en >> 14;
      block(b >= beg, b == beg, ent, more, jn, b);
      if (more) dma_sync<H>();        // K(b+1) rows 0-63 have landed
      ent = en;
      if (b + 2 < end) {
        const int slot = (b + 2 - beg) % kRowList;
        if (slot == 0) {   // only rows longer than kRowList blocks get here
          lds_sync();
          fill_list(b + 2);
          dma_sync<0>();
        }
        en = uni(rowlist[slot]);
      }
    }
    flush_block_sum();
  };

  // LSE-only fast pass as one pipeline over the whole row: step t issues the
  // QK^T MFMAs of group t and the sum of p of group t-1, across block edges
  // too, so every step has the same mix (8 MFMAs and one group's sum).  K
  // halves are refilled at two barriers per block as in the pass with PV:
  // after step 4b+1 K rows 0-63 of b+1, after step 4b+3 K rows 64-127 of
  // b+1, each barrier first waiting for the copy issued at the previous one.
  // The LDS stays that of the block pass (K halves and the row list), so
  // three workgroups still share a CU.  With HB, block b's sum of p per query
  // is complete at step 4b+4 and stored there; the next barrier's copy wait
  // also covers the store.
  auto run_fast_lse = [&]() {
    reset_row();
    fill_list(beg);
    dma_sync<0>();
    const int nb = end - beg;
    int ent = uni(rowlist[0]);
    int jc = ent >> 14;
    dma_k_half<D>(kh0, rk, jc * kTile * D * 2, koff, wave, 0);
    dma_k_half<D>(kh1, rk, jc * kTile * D * 2, koff, wave, 1);
    dma_sync<0>();
    const f32x16 zero16 = {};
    f32x16 s0, s1;
    auto store_block_sum = [&](int bpos) {
      if constexpr (REST) l_run += bs;
      if constexpr (HB) {
        const float tot = bs + __shfl_xor(bs, 32, 64);
        if (hl == 0) bsum[(int64_t)bpos * kTile + 32 * w + ln] = tot;
      }
    };
    // block 0, step 0: S of group 0
    s0 = qk_group<D>(kh0, qf, 0, zero16);
    interleave_step<8, 0>();
    __builtin_amdgcn_sched_barrier(0);
    // step 1: S of group 1; the row's reference point (group 0's maximum) and group 0's sum
    s1 = qk_group<D>(kh0, qf, 1, zero16);
    m_run = group_max(s0) * c;   // finite: key 0 always exists
    sum_group(s0, true);
    interleave_step<8, 8>();
    __builtin_amdgcn_sched_barrier(0);
    for (int b = 0; b < nb; ++b) {
      const bool more = b + 1 < nb;
      // barrier A: K rows 64-127 of b have landed; every wave is done with rows 0-63
      dma_sync<0>();
      int en = 0, jn = 0;
      if (more) {
        const int slot = (b + 1) % kRowList;
        if (slot == 0) {   // only rows longer than kRowList blocks get here
          fill_list(beg + b + 1);
          dma_sync<0>();
        }
        en = uni(rowlist[slot]);
        jn = en >> 14;
        dma_k_half<D>(kh0, rk, jn * kTile * D * 2, koff, wave, 0);
      }
      npad += ((ent >> 7) & 127) + (ent & 127);
      __builtin_amdgcn_sched_barrier(0);
      // steps 4b+2, 4b+3: S of groups 2 and 3, sums of groups 1 and 2
      s0 = qk_group<D>(kh1, qf, 2, zero16);
      sum_group(s1, false);
      interleave_step<8, 6>();
      __builtin_amdgcn_sched_barrier(0);
      s1 = qk_group<D>(kh1, qf, 3, zero16);
      sum_group(s0, false);
      interleave_step<8, 6>();
      __builtin_amdgcn_sched_barrier(0);
      // barrier B: K rows 0-63 of b+1 have landed; every wave is done with rows 64-127
      dma_sync<0>();
      if (more) {
        dma_k_half<D>(kh1, rk, jn * kTile * D * 2, koff, wave, 1);
        __builtin_amdgcn_sched_barrier(0);
        // step 4(b+1): S of group 0 of b+1, the sum of group 3 of b (block b complete)
        s0 = qk_group<D>(kh0, qf, 0, zero16);
        sum_group(s1, false);
        store_block_sum(beg + b);
        interleave_step<8, 6>();
        __builtin_amdgcn_sched_barrier(0);
        // step 4(b+1)+1: S of group 1, the sum of group 0 of b+1
        s1 = qk_group<D>(kh0, qf, 1, zero16);
        sum_group(s0, true);
        interleave_step<8, 6>();
        __builtin_amdgcn_sched_barrier(0);
        ent = en;
      }
    }
    // drain: the sum of the last group 3, the last block's sum
    sum_group(s1, false);
    store_block_sum(end - 1);
  };

  // Fast pass with PV: one software pipeline over the whole row.  Step t
  // (t = 4b + g for group g of block b) issues the QK^T MFMAs of group t, the
  // PV MFMAs of group t-2 and the softmax of group t-1, which do not depend
  // on each other, so every step has the same mix (16 MFMAs and one group's
  // softmax), across block boundaries too.  S^T of a group waits for its
  // softmax in s0/s1 and its packed P for its PV in p0/p1 (by the parity of
  // t).  K and V^T halves are refilled at two workgroup barriers per block:
  //   A, after step 4b+1 (every wave is done with K rows 0-63 of b and V^T
  //      keys 64-127 of b-1): K rows 0-63 of b+1, V^T keys 64-127 of b;
  //   B, after step 4b+3 (done with K rows 64-127 and V^T keys 0-63 of b):
  //      K rows 64-127 and V^T keys 0-63 of b+1.
  // Each barrier first waits for the copies issued at the one before it, two
  // steps earlier.
  // The softmax of one group with PV: p packed into pg, its sum into l and
  // (MASS) into the block's sum, which store_bsum writes to bsum[position]
  // once the block is complete (both lane halves).
  auto soft_pv = [&](const f32x16& sg, bf16x8 (&pg)[2], bool first_of_block) {
    const float g = exp_group<true>(sg, c, m_run, pg);
    pin(pg);
    l_run += g;
    if constexpr (MASS) {
      bs = first_of_block ? g : bs + g;
      pin_sum(bs);
    }
  };
  auto store_bsum = [&](int bpos) {
    const float tot = bs + __shfl_xor(bs, 32, 64);
    if (hl == 0) bsum[(int64_t)bpos * kTile + 32 * w + ln] = tot;
  };

  auto run_fast_pv = [&]() {
    reset_row();
    fill_list(beg);
    dma_sync<0>();
    const int nb = end - beg;
    int ent = uni(rowlist[0]);      // current block's list entry
    int jc = ent >> 14;             // its key tile
    dma_k_half<D>(kh0, rk, jc * kTile * D * 2, koff, wave, 0);
    dma_k_half<D>(kh1, rk, jc * kTile * D * 2, koff, wave, 1);
    dma_vt_half<D>(vh0, rv, jc * kTile * D * 2, voff, wave, 0);
    dma_sync<0>();
    const f32x16 zero16 = {};
    f32x16 s0, s1;
    bf16x8 p0[2], p1[2];
    // block 0, step 0: S of group 0
    s0 = qk_group<D>(kh0, qf, 0, zero16);
    interleave_step<8, 0>();
    __builtin_amdgcn_sched_barrier(0);
    // step 1: S of group 1; the row's reference point (group 0's maximum) and group 0's softmax
    s1 = qk_group<D>(kh0, qf, 1, zero16);
    m_run = group_max(s0) * c;   // finite: key 0 always exists
    soft_pv(s0, p0, true);
    interleave_step<8, 8>();
    __builtin_amdgcn_sched_barrier(0);
    for (int b = 0; b < nb; ++b) {
      const bool more = b + 1 < nb;
      // barrier A: K rows 64-127 and V^T keys 0-63 of b have landed
      dma_sync<0>();
      int en = 0, jn = 0;
      if (more) {
        const int slot = (b + 1) % kRowList;
        if (slot == 0) {   // only rows longer than kRowList blocks get here
          fill_list(beg + b + 1);
          dma_sync<0>();
        }
        en = uni(rowlist[slot]);
        jn = en >> 14;
        dma_k_half<D>(kh0, rk, jn * kTile * D * 2, koff, wave, 0);
      }
      dma_vt_half<D>(vh1, rv, jc * kTile * D * 2, voff, wave, 1);
      npad += ((ent >> 7) & 127) + (ent & 127);
      __builtin_amdgcn_sched_barrier(0);
      // step 4b+2: S of group 2, softmax of group 1, PV of group 0
      s0 = qk_pv_step<D>(kh1, qf, 2, vh0, p0, 0, oacc);
      soft_pv(s1, p1, false);
      interleave_step<16, 4>();
      __builtin_amdgcn_sched_barrier(0);
      // step 4b+3: S of group 3, softmax of group 2, PV of group 1
      s1 = qk_pv_step<D>(kh1, qf, 3, vh0, p1, 1, oacc);
      soft_pv(s0, p0, false);
      interleave_step<16, 4>();
      __builtin_amdgcn_sched_barrier(0);
      // barrier B: K rows 0-63 of b+1 and V^T keys 64-127 of b have landed
      dma_sync<0>();
      if (more) {
        dma_k_half<D>(kh1, rk, jn * kTile * D * 2, koff, wave, 1);
        dma_vt_half<D>(vh0, rv, jn * kTile * D * 2, voff, wave, 0);
        __builtin_amdgcn_sched_barrier(0);
        // step 4(b+1): S of group 0 of b+1, softmax of group 3 of b, PV of group 2 of b
        s0 = qk_pv_step<D>(kh0, qf, 0, vh1, p0, 2, oacc);
        soft_pv(s1, p1, false);
        if constexpr (MASS) store_bsum(beg + b);   // block b is complete
        interleave_step<16, 4>();
        __builtin_amdgcn_sched_barrier(0);
        // step 4(b+1)+1: S of group 1 of b+1, softmax of group 0 of b+1, PV of group 3 of b
        s1 = qk_pv_step<D>(kh0, qf, 1, vh1, p1, 3, oacc);
        soft_pv(s0, p0, true);
        interleave_step<16, 4>();
        __builtin_amdgcn_sched_barrier(0);
        ent = en;
        jc = jn;
      }
    }
    // drain: softmax of the last group 3 and PV of groups 2 and 3
    soft_pv(s1, p1, false);
    if constexpr (MASS) store_bsum(end - 1);
    pv_group<D>(vh1, p0, 2, oacc);
    interleave_step<8, 7>();
    __builtin_amdgcn_sched_barrier(0);
    pv_group<D>(vh1, p1, 3, oacc);
    interleave_step<8, 0>();
  };

  // A wave whose 32 query slots all lie past the tile's valid count holds
  // only padding queries.  It computes nothing: it issues its share of the
  // tile copies and meets the barriers of run_fast_pv (with PV) or
  // run_fast_lse, in the same order, and (HB) stores zero block sums for its
  // queries where those passes store theirs.  About a tenth of the waves of
  // the video workloads (edge tiles of the grid).
  auto run_copies = [&]() {
    reset_row();
    fill_list(beg);
    dma_sync<0>();
    const int nb = end - beg;
    int jc = uni(rowlist[0]) >> 14;
    dma_k_half<D>(kh0, rk, jc * kTile * D * 2, koff, wave, 0);
    dma_k_half<D>(kh1, rk, jc * kTile * D * 2, koff, wave, 1);
    if constexpr (PV) dma_vt_half<D>(vh0, rv, jc * kTile * D * 2, voff, wave, 0);
    dma_sync<0>();
    auto zero_sum = [&](int bpos) {
      if constexpr (HB) {
        if (hl == 0) bsum[(int64_t)bpos * kTile + 32 * w + ln] = 0.0f;
      }
    };
    for (int b = 0; b < nb; ++b) {
      const bool more = b + 1 < nb;
      dma_sync<0>();                  // barrier A
      int jn = 0;
      if (more) {
        const int slot = (b + 1) % kRowList;
        if (slot == 0) {
          fill_list(beg + b + 1);
          dma_sync<0>();
        }
        jn = uni(rowlist[slot]) >> 14;
        dma_k_half<D>(kh0, rk, jn * kTile * D * 2, koff, wave, 0);
      }
      if constexpr (PV) dma_vt_half<D>(vh1, rv, jc * kTile * D * 2, voff, wave, 1);
      dma_sync<0>();                  // barrier B
      if (more) {
        dma_k_half<D>(kh1, rk, jn * kTile * D * 2, koff, wave, 1);
        if constexpr (PV) dma_vt_half<D>(vh0, rv, jn * kTile * D * 2, voff, wave, 0);
        zero_sum(beg + b);
        jc = jn;
      }
    }
    zero_sum(end - 1);
  };

  // Safe pass over the blocks b0 .. b1-1 of the list cols: per block a plain
  // synchronous tile copy, then the four groups one after another with
  // explicit masking and exact re-basing; with SPV also the PV products.
  auto run_safe = [&](auto pvc, const int32_t* __restrict__ cols, int b0, int b1) {
    constexpr bool SPV = decltype(pvc)::value;
    reset_row();
    for (int b = b0; b < b1; ++b) {
      const int slot = (b - b0) % kRowList;
      if (slot == 0) {
        lds_sync();
        fill_entries(cols, b, b1);
        dma_sync<0>();
      }
      const int ent = uni(rowlist[slot]);
      const int j = ent >> 14;
      const int nj = kTile - ((ent >> 7) & 127) - (ent & 127);
      lds_sync();                     // every wave is done with the previous tiles
      copy_kv_halves<D, SPV>(kh0, kh1, vh0, vh1, k + (hrow + (int64_t)kTile * j) * D,
                             vt + (htile + j) * D * kTile);
      lds_sync();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16 zero16 = {};
        f32x16 sg = qk_group<D>(kt < 2 ? kh0 : kh1, qf, kt, zero16);
        mask_group(sg, kt, nj, hl);
        const float m_new = fmaxf(m_run, group_max(sg) * c);
        if (m_new > m_run) {
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // m_run = -inf gives 0
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
          l_run *= alpha;
          m_run = m_new;
        }
        bf16x8 pg[2];
        l_run += exp_group<true>(sg, c, m_run, pg);
        if constexpr (SPV) pv_group<D>(kt < 2 ? vh0 : vh1, pg, kt, oacc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // REST: a query tile whose two lists do not match gets NaN; an empty rest
  // (every block selected) contributes nothing
  bool rbad = false;
  if constexpr (REST) rbad = uni(hs.cflag[t]) != 0;
  const bool empty = REST && (rbad || end <= beg);
  const bool wdead = 32 * wave >= sh.valid[i];   // only padding queries
  if (empty) reset_row();
  else if (wdead) run_copies();
  else if constexpr (PV) run_fast_pv();
  else run_fast_lse();
  float l_all = l_run + __shfl_xor(l_run, 32, 64);
  const float pad_mass = (empty || wdead) ? 0.0f : (float)npad * __builtin_amdgcn_exp2f(-m_run);
  l_all -= pad_mass;
  const bool bad = !empty && qvalid && !(l_all <= kMaxRowSum && pad_mass <= kMaxPadRatio * l_all);
  if (__any(bad) && lane == 0) redo = 1;
  lds_sync();
  if (uni(redo)) {
    run_safe(BoolC<PV>{}, col_idx, beg, end);
    l_all = l_run + __shfl_xor(l_run, 32, 64);
  } else if (wdead) {
    // a padding query's outputs: O = 0 and LSE = 0 (finite, so that a
    // backward over these rows, whose Q and dO are zero, stays finite)
    l_all = 1.0f;
    m_run = 0.0f;
  }
  const float m_all = m_run;

  // REST: the dense row's LSE (log2 units) from the rest's sum and the
  // selected row's LSE: L2 = log2(2^ls2 + l * 2^m)
  float L2 = 0.0f, ls2 = 0.0f;
  if constexpr (REST) {
    ls2 = hs.lse_sel[row0 + 32 * w + ln] * 1.4426950408889634f;
    const float lr2 = m_all + __log2f(l_all);         // -inf for an empty rest
    const float mx = fmaxf(ls2, lr2);
    L2 = rbad ? __builtin_nanf("") : mx + __log2f(__builtin_amdgcn_exp2f(ls2 - mx) + __builtin_amdgcn_exp2f(lr2 - mx));
    if (wdead && !uni(redo) && !rbad) L2 = 0.0f;   // padding queries: LSE 0, as the passes above give them
  }

  // Block heat of this query tile (HB): heat(i, j) is the mean over the
  // tile's valid queries of the probability mass on key tile j's valid keys.
  // After the fast pass, bsum holds per (block, query) the sum of
  // exp2(s*c - m) over the block's 128 key slots, so the mass is
  // (bsum - pads(j) * exp2(-m)) / l with the row's final l (REST: times
  // 2^(m + log2 l - L2), the rest's share of the dense row).  After the safe
  // pass those sums are not on one reference point, so every block is walked
  // again with the final LSE and its exact masked mass stored instead.
  // MASS keeps the sums per query and stores each query's two factors
  // instead of reducing them; REST adds the selected blocks from those.
  if constexpr (HB) {
    const bool exact = uni(redo) != 0;
    if (exact) {
      const float lse2 = REST ? L2 : m_all + __log2f(l_all);
      for (int b = beg; b < end; ++b) {
        const int j = min(max(col_idx[b], 0), nt - 1);
        const int nj = sh.valid[j];
        lds_sync();                     // every wave is done with the previous tile
        copy_kv_halves<D, false>(kh0, kh1, vh0, vh1, k + (hrow + (int64_t)kTile * j) * D, vt);
        lds_sync();
        float acc = 0.0f;
#pragma unroll 1
        for (int kt = 0; kt < 4; ++kt) {
          const f32x16 zero16 = {};
          const f32x16 sg = qk_group<D>(kt < 2 ? kh0 : kh1, qf, kt, zero16);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sg[r], c, -lse2));
            acc += sacc_key(kt, r, hl) < nj ? e : 0.0f;
          }
        }
        const float bq = acc + __shfl_xor(acc, 32, 64);
        if (hl == 0) bsum[(int64_t)b * kTile + 32 * w + ln] = bq;
      }
    }
    if constexpr (MASS) {
      // share of query r's probability on a block: bsum * x - pads * y
      if (hl == 0)
        hs.fac[row0 + 32 * w + ln] =
            make_float2(qvalid ? (exact ? 1.0f : 1.0f / l_all) : 0.0f,
                        (qvalid && !exact) ? __builtin_amdgcn_exp2f(-m_all) / l_all : 0.0f);
    } else {
      if (hl == 0) {
        if constexpr (REST) {
          s_inv[32 * w + ln] = qvalid ? (exact ? 1.0f : __builtin_amdgcn_exp2f(m_all - L2)) : 0.0f;
          s_pe[32 * w + ln] = (qvalid && !exact && !empty) ? __builtin_amdgcn_exp2f(-L2) : 0.0f;
          const float2 f = hs.fac[row0 + 32 * w + ln];
          const float g = __builtin_amdgcn_exp2f(ls2 - L2);
          s_sel[32 * w + ln] = qvalid ? f.x * g : 0.0f;
          s_spe[32 * w + ln] = qvalid ? f.y * g : 0.0f;
        } else {
          s_inv[32 * w + ln] = qvalid ? (exact ? 1.0f : 1.0f / l_all) : 0.0f;
          s_pe[32 * w + ln] = (qvalid && !exact) ? __builtin_amdgcn_exp2f(-m_all) / l_all : 0.0f;
        }
      }
      __syncthreads();                  // every wave's block sums and factors are visible
      float pe = 0.0f;                  // one padding key's mass, summed over the queries
#pragma unroll 4
      for (int qq = 0; qq < kTile; ++qq) pe += s_pe[qq];
      const float inv_nq = 1.0f / (float)sh.valid[i];
      float* hrow_out = heat + p.head_pair_off[h] + (int64_t)i * nt;
      if (rbad) {
        for (int j = threadIdx.x; j < nt; j += kThreads) hrow_out[j] = __builtin_nanf("");
      } else {
        for (int e = threadIdx.x; e < end - beg; e += kThreads) {
          const int j = min(max(col_idx[beg + e], 0), nt - 1);
          const float* bp = bsum + (int64_t)(beg + e) * kTile;
          float acc = 0.0f;
#pragma unroll 2
          for (int q4 = 0; q4 < kTile; q4 += 4) {
            const u32x4 bv = ld16(bp + q4);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc = fmaf(__uint_as_float(bv[u]), s_inv[q4 + u], acc);
          }
          hrow_out[j] = fmaf(-(float)(kTile - sh.valid[j]), pe, acc) * inv_nq;
        }
        if constexpr (REST) {
          // the selected blocks: their shares of the selected row times 2^(ls2 - L2)
          float pes = 0.0f;
#pragma unroll 4
          for (int qq = 0; qq < kTile; ++qq) pes += s_spe[qq];
          const int sb = uni(hs.srow[t]), se = uni(hs.srow[t + 1]);
          for (int e = threadIdx.x; e < se - sb; e += kThreads) {
            const int j = min(max(hs.scol[sb + e], 0), nt - 1);
            const float* mp = hs.mass + (int64_t)(sb + e) * kTile;
            float acc = 0.0f;
#pragma unroll 2
            for (int q4 = 0; q4 < kTile; q4 += 4) {
              const u32x4 mv = ld16(mp + q4);
#pragma unroll
              for (int u = 0; u < 4; ++u) acc = fmaf(__uint_as_float(mv[u]), s_sel[q4 + u], acc);
            }
            hrow_out[j] = fmaf(-(float)(kTile - sh.valid[j]), pes, acc) * inv_nq;
          }
        }
      }
    }
  }

  // epilogue: normalise, store (without PV only the LSE)
  if constexpr (PV) {
    const float inv = 1.0f / l_all;
    // permuted: row row0 + slot; natural: the slot's token, padding dropped
    uint16_t* orow = o + (row0 + 32 * w + ln) * D;
    bool store = true;
    if (o_natural) {
      const int slot = 32 * w + ln;
      const int32_t tok = sh.perm[(int64_t)kTile * i + slot];
      store = tok >= 0;
      orow = o + ((int64_t)(store ? tok : 0) * p.num_heads + h) * D;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x2 lo, hi;
        lo[0] = (__bf16)(oacc[db][4 * jj + 0] * inv);
        lo[1] = (__bf16)(oacc[db][4 * jj + 1] * inv);
        hi[0] = (__bf16)(oacc[db][4 * jj + 2] * inv);
        hi[1] = (__bf16)(oacc[db][4 * jj + 3] * inv);
        uint2 v;
        v.x = __builtin_bit_cast(uint32_t, lo);
        v.y = __builtin_bit_cast(uint32_t, hi);
        if (store) *reinterpret_cast<uint2*>(orow + 32 * db + 8 * jj + 4 * hl) = v;
      }
  }
  if (lse && hl == 0)
    lse[row0 + 32 * w + ln] = REST ? L2 * 0.69314718055994531f : m_run * 0.69314718055994531f + logf(l_all);
  if (visited && threadIdx.x == 0) atomicAdd(visited, (uint32_t)(end - beg));
}

template <int D, bool PV>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(DevPlan p, const uint16_t* __restrict__ q,
                                                              int q_natural, const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ vt,
                                                              const int32_t* __restrict__ row_ptr,
                                                              const int32_t* __restrict__ col_idx, float scale_log2,
                                                              uint16_t* __restrict__ o, int o_natural,
                                                              float* __restrict__ lse, uint32_t* __restrict__ visited) {
  attn_fwd_body<D, PV, false>(p, q, q_natural, k, vt, row_ptr, col_idx, scale_log2, o, o_natural, lse, visited,
                              nullptr, nullptr, HeatSplit{});
}

// The dense LSE and the block heat in one pass over an all-blocks mask: the
// LSE-only attention (no PV, no V^T) that also keeps every block's sum of p
// per query in bsum and reduces them into the heat at the end of each row.
template <int D>
__global__ void __launch_bounds__(kThreads, 2) lse_heat_kernel(DevPlan p, const uint16_t* __restrict__ q,
                                                              int q_natural, const uint16_t* __restrict__ k,
                                                              const int32_t* __restrict__ row_ptr,
                                                              const int32_t* __restrict__ col_idx, float scale_log2,
                                                              float* __restrict__ lse, float* __restrict__ bsum,
                                                              float* __restrict__ heat) {
  attn_fwd_body<D, false, true>(p, q, q_natural, k, k, row_ptr, col_idx, scale_log2, nullptr, 0, lse, nullptr, bsum,
                                heat, HeatSplit{});
}

// The attention and the dense heat of one layer without computing any
// block's QK^T twice (veda_attn_fwd_lse_heat), in three launches:
//  attn_mass_kernel: the attention over the selected CSR; it also leaves in
//    mass[position][query] each selected block's sum of p and in fac[query]
//    the factors that make it the block's share of the query's attention
//    probability (over the selected blocks);
//  complement_kernel: the rest of every dense row (its blocks that are not
//    selected) as a CSR of its own;
//  rest_heat_kernel: the LSE-only heat pass over that rest, which joins the
//    two rows into the dense LSE and writes the heat of every block.
template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_mass_kernel(
    DevPlan p, const uint16_t* __restrict__ q, int q_natural, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    float scale_log2, uint16_t* __restrict__ o, int o_natural, float* __restrict__ lse, float* __restrict__ mass,
    float2* __restrict__ fac) {
  attn_fwd_body<D, true, true>(p, q, q_natural, k, vt, row_ptr, col_idx, scale_log2, o, o_natural, lse, nullptr, mass,
                               nullptr, HeatSplit{nullptr, nullptr, nullptr, nullptr, nullptr, fac});
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) rest_heat_kernel(
    DevPlan p, const uint16_t* __restrict__ q, int q_natural, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ dense_row_ptr, const int32_t* __restrict__ rest_col, float scale_log2,
    float* __restrict__ lse, float* __restrict__ bsum, float* __restrict__ heat, HeatSplit hs) {
  attn_fwd_body<D, false, true, true>(p, q, q_natural, k, k, dense_row_ptr, rest_col, scale_log2, nullptr, 0, lse,
                                      nullptr, bsum, heat, hs);
}

// One workgroup per query tile t: the entries of the dense row that are not
// in the selected row, in order, at rest_col[dbeg - sbeg ..] (the selected
// row is a subset of the dense row, so the rest of row t starts after the
// rest of the rows before it).  Each dense entry finds its rank in the
// selected row by binary search (both rows ascending).  cflag[t] = 1 when the
// two rows do not fit that description (a selected column missing from the
// dense row, repeats, a longer selected row); nothing is then written
// outside the row's own range.
__global__ void __launch_bounds__(kThreads) complement_kernel(const int32_t* __restrict__ drow,
                                                              const int32_t* __restrict__ dcol,
                                                              const int32_t* __restrict__ srow,
                                                              const int32_t* __restrict__ scol, int64_t rest_nnz,
                                                              int32_t* __restrict__ rest_col,
                                                              int32_t* __restrict__ cflag) {
  __shared__ int32_t found, outside;
  const int64_t t = blockIdx.x;
  const int dbeg = drow[t], dend = drow[t + 1], sbeg = srow[t], send = srow[t + 1];
  const int cbeg = dbeg - sbeg, cend = dend - send;
  const bool bad = sbeg < 0 || send < sbeg || cbeg < 0 || cend < cbeg || cend > rest_nnz;
  if (threadIdx.x == 0) {
    found = 0;
    outside = 0;
  }
  __syncthreads();
  if (!bad) {
    for (int e = dbeg + (int)threadIdx.x; e < dend; e += kThreads) {
      const int col = dcol[e];
      int lo = sbeg, hi = send;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (scol[mid] < col) lo = mid + 1; else hi = mid;
      }
      if (lo < send && scol[lo] == col) {
        atomicAdd(&found, 1);
      } else {
        const int pos = cbeg + (e - dbeg) - (lo - sbeg);
        if (pos >= cbeg && pos < cend) rest_col[pos] = col;
        else outside = 1;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) cflag[t] = (bad || outside || found != send - sbeg) ? 1 : 0;
}

// ---------------------------------------------------------------------------
// block heat from the dense LSE
// ---------------------------------------------------------------------------
//
// One workgroup (4 waves, 32 queries each) per (head, query tile); it walks
// every key tile of the head with S^T = K Q^T on the matrix core as the
// attention kernel does, and sums exp2(s*c - lse*log2(e)) over valid
// (query, key) pairs.  Key tiles stream through two LDS buffers (A for even
// j, B for odd j) with asynchronous copies one tile ahead; inside a tile the
// four 32-key groups are software-pipelined (QK^T MFMAs of group g with the
// exp/sum VALU work of group g-1).
//
// Padding keys hold zero rows of K, so their logit is exactly 0 and their
// term is exp(-lse[r]); the fast variant sums all 128 keys and subtracts the
// lane's padding count times that term.  A workgroup with a valid query whose
// exp(-lse) exceeds 1/16 (where that subtraction could cancel) masks the
// padding keys explicitly instead.  Each wave reduces its partial over lanes;
// thread 0 adds the four wave partials in a fixed order one tile later.
template <int D>
__global__ void __launch_bounds__(kThreads, 2) heat_kernel(DevPlan p, const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const float* __restrict__ lse, float scale_log2,
                                                          float* __restrict__ heat) {
  __shared__ __attribute__((aligned(16))) uint16_t ka0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t ka1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t kb0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t kb1[64 * D];
  __shared__ float red[2][4];
  __shared__ int32_t masked_s;
  __shared__ uint8_t vcnt[kMaxHeatTiles];   // valid counts of the head's tiles (no vector loads in the loop)
  const int t = blockIdx.x;
  const int h = uni(p.row_head[t]);
  const DevShape& sh = p.shape[uni(p.head_shape[h])];
  const int n = sh.num_tiles;
  const int i = t - uni(p.head_tile_off[h]);
  const int ni = uni(sh.valid[i]);
  const int64_t hrow = uni64(p.head_row_off[h]);
  const int64_t row0 = hrow + (int64_t)kTile * i;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + hrow * D, (int64_t)n * kTile * D * 2);
  const int wave = uni(threadIdx.x >> 6);
  const int w = threadIdx.x >> 6, lane = lane_id(), ln = lane & 31, hl = lane >> 5;
  const int koff = k_lane_offset<D>(threadIdx.x);
  const int qr = 32 * w + ln;
  const bool qvalid = qr < ni;
  const float c = scale_log2;
  bf16x8 qf[D / 16];
  const uint16_t* qrow = q + (row0 + qr) * D + 8 * hl;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld16(qrow + 16 * s));
  const float l2 = qvalid ? lse[row0 + qr] * 1.4426950408889634f : 0.0f;
  const float e_pad = __builtin_amdgcn_exp2f(-l2);   // a padding key's term
  if (threadIdx.x == 0) masked_s = 0;
  for (int e = threadIdx.x; e < n; e += kThreads) vcnt[e] = (uint8_t)sh.valid[e];
  __syncthreads();
  if (__any(qvalid && !(e_pad <= 0.0625f)) && lane == 0) masked_s = 1;
  __syncthreads();
  const bool masked = uni(masked_s) != 0;
  float* hrow_out = heat + p.head_pair_off[h] + (int64_t)i * n;
  const float inv_ni = 1.0f / (float)ni;

  // sum of the lane's 64 terms of key tile j (nj valid keys) from one buffer
  auto tile_sum = [&](const uint16_t* __restrict__ k0, const uint16_t* __restrict__ k1, int nj, auto msk)
      __attribute__((always_inline)) {
    constexpr bool M = decltype(msk)::value;
    const f32x16 zero16 = {};
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    auto esum = [&](const f32x16& sg, int kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(fmaf(sg[r], c, -l2));
        if (M) e = (sacc_key(kt, r, hl) < nj) ? e : 0.0f;
        acc[r & 3] += e;
      }
    };
    f32x16 s0 = qk_group<D>(k0, qf, 0, zero16);
    interleave_step<8, 0>();
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s1 = qk_group<D>(k0, qf, 1, zero16);
    esum(s0, 0);
    interleave_step<8, 6>();
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s2 = qk_group<D>(k1, qf, 2, zero16);
    esum(s1, 1);
    interleave_step<8, 6>();
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s3 = qk_group<D>(k1, qf, 3, zero16);
    esum(s2, 2);
    interleave_step<8, 6>();
    __builtin_amdgcn_sched_barrier(0);
    esum(s3, 3);
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };

  // Tile j's partial: the fast variant subtracts the lane's padding terms.
  // The lane holds 64 keys, half of every 16-key run, so for nj valid keys
  // its padding count is half_pads(nj, hl).
  auto do_tile = [&](int j, auto bufb) {
    constexpr bool BB = decltype(bufb)::value;   // buffer B (odd j) or A, fixed at compile time
    const uint16_t* __restrict__ k0 = BB ? kb0 : ka0;
    const uint16_t* __restrict__ k1 = BB ? kb1 : ka1;
    const int nj = uni(vcnt[j]);
    float part;
    if (masked) {
      part = tile_sum(k0, k1, nj, BoolC<true>{});
    } else {
      part = tile_sum(k0, k1, nj, BoolC<false>{});
      part = fmaf(-(float)half_pads(nj, hl), e_pad, part);
    }
    if (!qvalid) part = 0.0f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) red[j & 1][w] = part;
  };

  // Iteration j: wait for K(j), copy K(j+1) into the other buffer, work on
  // tile j; thread 0 writes tile j-1's value.  The loop body handles an odd
  // j (buffer B) and the following even j (buffer A), so the kernel has four
  // copy call sites; the first iteration (j = -1) only copies K(0).
  for (int j = -1; j < n; j += 2) {
    // odd j (K(j) in B), copies K(j+1) into A
    dma_sync<0>();
    if (j >= 1 && threadIdx.x == 0) {
      const float* rr = red[(j - 1) & 1];
      hrow_out[j - 1] = (((rr[0] + rr[1]) + rr[2]) + rr[3]) * inv_ni;
    }
    if (j + 1 < n) {
      dma_k_half<D>(ka0, rk, (j + 1) * kTile * D * 2, koff, wave, 0);
      dma_k_half<D>(ka1, rk, (j + 1) * kTile * D * 2, koff, wave, 1);
    }
    if (j >= 0) do_tile(j, BoolC<true>{});
    // even j + 1 (K(j+1) in A), copies K(j+2) into B
    if (j + 1 >= n) break;
    dma_sync<0>();
    if (j >= 0 && threadIdx.x == 0) {
      const float* rr = red[j & 1];
      hrow_out[j] = (((rr[0] + rr[1]) + rr[2]) + rr[3]) * inv_ni;
    }
    if (j + 2 < n) {
      dma_k_half<D>(kb0, rk, (j + 2) * kTile * D * 2, koff, wave, 0);
      dma_k_half<D>(kb1, rk, (j + 2) * kTile * D * 2, koff, wave, 1);
    }
    do_tile(j + 1, BoolC<false>{});
  }
  dma_sync<0>();
  if (threadIdx.x == 0) {
    const float* rr = red[(n - 1) & 1];
    hrow_out[n - 1] = (((rr[0] + rr[1]) + rr[2]) + rr[3]) * inv_ni;
  }
}

// ---------------------------------------------------------------------------
// attention mass of a block mask
// ---------------------------------------------------------------------------
//
// Two launches, both in a fixed order (the result does not depend on
// timing).  Part: workgroup (chunk c, head h) takes rows 16c .. 16c+15 of the
// head, 16 threads per row; each thread sums its share of the row's listed
// heat in list order, the row's 16 partials are combined by a fixed shuffle
// tree, weighted by the row tile's valid query count, and the 16 rows by a
// fixed tree in LDS; (kept, count) go to part[h][c].  Final: thread h sums
// its chunks in ascending order.
constexpr int kMassRows = 16;

__global__ void __launch_bounds__(kThreads) mask_mass_part_kernel(DevPlan p, const float* __restrict__ heat,
                                                                 const int32_t* __restrict__ row_ptr,
                                                                 const int32_t* __restrict__ col_idx,
                                                                 double2* __restrict__ part, int chunks) {
  __shared__ double kept_s[kMassRows];
  __shared__ double cnt_s[kMassRows];
  const int c = blockIdx.x, h = blockIdx.y;
  const DevShape& sh = p.shape[p.head_shape[h]];
  const int n = sh.num_tiles;
  const int64_t t0 = p.head_tile_off[h];
  const float* hm = heat + p.head_pair_off[h];
  const int rr = threadIdx.x / 16, sub = threadIdx.x % 16;
  const int i = c * kMassRows + rr;
  double row = 0.0;
  if (i < n) {
    const int e1 = row_ptr[t0 + i + 1];
    for (int e = row_ptr[t0 + i] + sub; e < e1; e += 16) {
      const int j = col_idx[e];
      if (j >= 0 && j < n) row += (double)hm[(int64_t)i * n + j];
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) row += __shfl_xor(row, off, 16);
  if (sub == 0) {
    const double v = i < n ? (double)sh.valid[i] : 0.0;
    kept_s[rr] = v * row;
    cnt_s[rr] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double kept = 0.0, cnt = 0.0;
    for (int r = 0; r < kMassRows; ++r) {
      kept += kept_s[r];
      cnt += cnt_s[r];
    }
    part[(int64_t)h * chunks + c] = make_double2(kept, cnt);
  }
}

__global__ void __launch_bounds__(kThreads) mask_mass_final_kernel(int num_heads, const double2* __restrict__ part,
                                                                  int chunks, double* __restrict__ mass) {
  const int h = blockIdx.x * kThreads + threadIdx.x;
  if (h >= num_heads) return;
  double kept = 0.0, cnt = 0.0;
  for (int c = 0; c < chunks; ++c) {
    const double2 v = part[(int64_t)h * chunks + c];
    kept += v.x;
    cnt += v.y;
  }
  mass[h] = kept / cnt;
}

// ---------------------------------------------------------------------------
// relative output error of two natural-order outputs
// ---------------------------------------------------------------------------
//
// Two launches in a fixed order.  Part: workgroup (chunk c, head h) takes
// tokens [c N / C, (c+1) N / C) of the head; thread x takes the 16-byte
// pieces x, x + 256, ... of that range (strided by H*D between tokens),
// accumulates (o - o_ref)^2 and o_ref^2 in fp64, and the partials meet in a
// fixed-order tree in LDS.  Final: thread h sums its C chunks in ascending
// order and divides.
constexpr int kErrChunks = 32;

template <int D>
__global__ void __launch_bounds__(kThreads) output_error_part_kernel(int64_t num_tokens, int num_heads,
                                                                    const uint16_t* __restrict__ o,
                                                                    const uint16_t* __restrict__ o_ref,
                                                                    double2* __restrict__ part) {
  constexpr int CH = D / 8;
  __shared__ double num_s[kThreads];
  __shared__ double den_s[kThreads];
  const int c = blockIdx.x, h = blockIdx.y;
  const int64_t q0 = num_tokens * c / kErrChunks * CH, q1 = num_tokens * (c + 1) / kErrChunks * CH;
  double num = 0.0, den = 0.0;
  for (int64_t q = q0 + threadIdx.x; q < q1; q += kThreads) {
    const int64_t n = q / CH, off = (n * num_heads + h) * D + 8 * (q % CH);
    const u32x4 a = ld16(o + off), b = ld16(o_ref + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double a0 = bf16_to_f32((uint16_t)(a[e] & 0xffff)), a1 = bf16_to_f32((uint16_t)(a[e] >> 16));
      const double b0 = bf16_to_f32((uint16_t)(b[e] & 0xffff)), b1 = bf16_to_f32((uint16_t)(b[e] >> 16));
      num += (a0 - b0) * (a0 - b0) + (a1 - b1) * (a1 - b1);
      den += b0 * b0 + b1 * b1;
    }
  }
  num_s[threadIdx.x] = num;
  den_s[threadIdx.x] = den;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      num_s[threadIdx.x] += num_s[threadIdx.x + w];
      den_s[threadIdx.x] += den_s[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) part[(int64_t)h * kErrChunks + c] = make_double2(num_s[0], den_s[0]);
}

__global__ void __launch_bounds__(kThreads) output_error_final_kernel(int num_heads, const double2* __restrict__ part,
                                                                     double* __restrict__ err) {
  const int h = blockIdx.x * kThreads + threadIdx.x;
  if (h >= num_heads) return;
  double num = 0.0, den = 0.0;
  for (int c = 0; c < kErrChunks; ++c) {
    const double2 v = part[(int64_t)h * kErrChunks + c];
    num += v.x;
    den += v.y;
  }
  err[h] = num / den;
}

// ---------------------------------------------------------------------------
// backward: transposed lists
// ---------------------------------------------------------------------------
//
// The per-key-tile lists come from a byte matrix per head, stored key tile
// major (m[j][i] = 1 iff key tile j is in query tile i's row, so a column of
// the mask is contiguous): scatter the CSR into it, then one wave per key
// tile walks its column twice, 64 query tiles per ballot, counting and then
// listing the query tiles in ascending order (ballot ranks give each its
// position).  No atomics, so the order is fixed.
__global__ void __launch_bounds__(kThreads) fill_u32_kernel(uint32_t* __restrict__ x, int64_t n, uint32_t v) {
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += (int64_t)gridDim.x * kThreads) x[e] = v;
}

__global__ void __launch_bounds__(64) csc_scatter_kernel(DevPlan p, const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ col_idx,
                                                        uint8_t* __restrict__ bitmap) {
  const int t = blockIdx.x;
  const int h = p.row_head[t];
  const int n = p.shape[p.head_shape[h]].num_tiles;
  const int i = t - p.head_tile_off[h];
  uint8_t* m = bitmap + p.head_pair_off[h] + i;
  for (int e = row_ptr[t] + (int)threadIdx.x; e < row_ptr[t + 1]; e += 64) {
    const int j = col_idx[e];
    if (j >= 0 && j < n) m[(int64_t)j * n] = 1;
  }
}

template <bool FILL>
__global__ void __launch_bounds__(64) csc_column_kernel(DevPlan p, const uint8_t* __restrict__ bitmap,
                                                       int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ col_ptr,
                                                       int32_t* __restrict__ row_idx) {
  const int64_t tc = blockIdx.x;           // one wave per key tile
  const int h = uni(p.row_head[tc]);
  const int n = uni(p.shape[uni(p.head_shape[h])].num_tiles);
  const int j = (int)(tc - uni(p.head_tile_off[h]));
  const uint8_t* m = bitmap + uni64(p.head_pair_off[h]) + (int64_t)j * n;
  const int lane = lane_id();
  const uint64_t below = lanes_below();
  int32_t pos = FILL ? col_ptr[tc] : 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const bool set = i < n && m[i] != 0;
    const uint64_t bal = __ballot(set);
    if (FILL && set) row_idx[pos + __popcll(bal & below)] = i;
    pos += __popcll(bal);
  }
  if (!FILL && lane == 0) counts[tc] = pos;
}

// Exclusive scan of counts[0..n) into col_ptr[0..n]; one workgroup, chunks
// of 1024 with a running carry.
__global__ void __launch_bounds__(1024) csc_scan_kernel(const int32_t* __restrict__ counts, int64_t n,
                                                       int32_t* __restrict__ col_ptr) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < n; base += 1024) {
    const int64_t e = base + threadIdx.x;
    const int32_t v = e < n ? counts[e] : 0;
    buf[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {       // inclusive Hillis-Steele scan
      const int32_t add = (int)threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += add;
      __syncthreads();
    }
    if (e < n) col_ptr[e] = carry + buf[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry += buf[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) col_ptr[n] = carry;
}

// ---------------------------------------------------------------------------
// backward: helpers
// ---------------------------------------------------------------------------

// Dispatch order of the dK/dV workgroups.  Workgroup b runs on XCD b mod 8,
// so the key tiles are cut into 8 contiguous index ranges of equal count
// (one per XCD: whole heads or runs of neighbouring tiles, whose lists share
// query tiles in that XCD's L2), and inside each range ordered by descending
// list length (a counting sort over 8 x 1,024 length bins in one
// workgroup), so that each XCD starts its long lists first and ends evenly.
// Range x's k-th tile gets slot 8k + x.  The order inside one length bin is
// that of the LDS atomics; it only changes the schedule, never a result.
constexpr int kXcds = 8;
constexpr int kOrderBins = 1024;   // list lengths 0 .. 1,023; longer lists share the top bin
__global__ void __launch_bounds__(1024) bwd_order_kernel(const int32_t* __restrict__ col_ptr, int64_t n,
                                                        int32_t* __restrict__ order) {
  constexpr int NB = kXcds * kOrderBins;
  __shared__ int32_t start[NB];
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = n / kXcds, extra = n % kXcds;
  auto range = [&](int64_t t) -> int {   // ranges 0 .. extra-1 hold per + 1 tiles
    return t < (per + 1) * extra ? (int)(t / (per + 1)) : (int)(extra + (t - (per + 1) * extra) / per);
  };
  for (int b = tid; b < NB; b += 1024) start[b] = 0;
  __syncthreads();
  auto bin = [&](int64_t t) {   // inside a range, bin 0 holds the longest lists
    return range(t) * kOrderBins + kOrderBins - 1 - min(col_ptr[t + 1] - col_ptr[t], kOrderBins - 1);
  };
  for (int64_t t = tid; t < n; t += 1024) atomicAdd(&start[bin(t)], 1);
  __syncthreads();
  int32_t loc[NB / 1024], sum = 0;
#pragma unroll
  for (int u = 0; u < NB / 1024; ++u) {
    loc[u] = start[(NB / 1024) * tid + u];
    sum += loc[u];
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {          // inclusive Hillis-Steele scan
    const int32_t add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;
#pragma unroll
  for (int u = 0; u < NB / 1024; ++u) {
    start[(NB / 1024) * tid + u] = run;
    run += loc[u];
  }
  __syncthreads();
  for (int64_t t = tid; t < n; t += 1024) {
    const int x = range(t);
    const int64_t k = atomicAdd(&start[bin(t)], 1) - (x * per + min((int64_t)x, extra));   // rank inside the range
    order[k < per ? kXcds * k + x : kXcds * per + x] = (int32_t)t;
  }
}

// aux[r] = (lse[r] * log2(e), sum_d dO[r][d] * O[r][d]) in fp32 for every
// permuted row; D/8 lanes per row, one 16-byte chunk of O and dO each.
template <int D>
__global__ void __launch_bounds__(kThreads) bwd_prep_kernel(int64_t rows, const uint16_t* __restrict__ o,
                                                           const uint16_t* __restrict__ d_o,
                                                           const float* __restrict__ lse,
                                                           float2* __restrict__ aux) {
  constexpr int CH = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t r = idx / CH;
  const int c = (int)(idx % CH);
  float acc = 0.0f;
  if (r < rows) {
    const u32x4 a = ld16(o + r * D + 8 * c), b = ld16(d_o + r * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_to_f32((uint16_t)(a[e] & 0xffff)), bf16_to_f32((uint16_t)(b[e] & 0xffff)), acc);
      acc = fmaf(bf16_to_f32((uint16_t)(a[e] >> 16)), bf16_to_f32((uint16_t)(b[e] >> 16)), acc);
    }
  }
#pragma unroll
  for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (r < rows && c == 0) aux[r] = make_float2(lse[r] * 1.4426950408889634f, acc);
}

// Row tiles of the backward in LDS: 128 rows of D bf16, rows in pi order
// inside every 32 (as the attention kernels hold K), 16-byte chunk c of row m
// at position c ^ bsw(m).  Both ways the tile is read stay free of bank
// conflicts: row reads (16 consecutive rows, one chunk each) and transpose
// reads (4 consecutive rows, 32 bytes of each per 16 lanes).
template <int D>
__device__ __forceinline__ int bsw(int m) {
  if constexpr (D == 128)
    return ((m & 3) << 2) | ((m >> 2) & 3);
  else
    return (((m >> 1) & 1) << 2) | ((m >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int brow_off(int m, int c) {
  return m * D + 8 * (c ^ bsw<D>(m));
}

// Asynchronous copy of a [128, D] row tile into that layout through a buffer
// resource: each lane moves 16 bytes per instruction and a wave's 64 chunks
// land contiguously, so the swizzle is applied on the global side.  A
// workgroup instruction of 512 threads fills STEP = 512 / (D / 8) rows (32 or
// 64); the swizzle and the pi order only use the low five bits of the row, so
// every instruction of a thread uses one byte offset plus a uniform step.
constexpr int kBwdThreads = 512;   // dQ workgroups: 8 waves, 2 per SIMD

template <int D>
__device__ __forceinline__ int brow_lane_offset(int tid) {   // bytes
  constexpr int CH = D / 8;
  const int m = tid / CH, pos = tid % CH;
  return 2 * (((m & ~31) | pi_row(m & 31)) * D + 8 * (pos ^ bsw<D>(m)));
}
template <int D>
__device__ __forceinline__ void dma_row_tile(uint16_t* __restrict__ dst, __amdgpu_buffer_rsrc_t rs, int tile_byte,
                                             int lane_off, int wave) {
  constexpr int STEP = kBwdThreads / (D / 8);   // rows per workgroup instruction (32 or 64)
#pragma unroll
  for (int it = 0; it < kTile / STEP; ++it)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + it * STEP * D + 512 * wave, 16, lane_off,
                                             tile_byte + it * STEP * D * 2, 0, 0);
}

// Per-lane byte offsets of a wave's operand reads inside a backward row
// tile.  Row group g adds 32 g D 2 bytes and the 16-row step s2 of a
// transpose read 16 s2 D 2 bytes: neither changes the swizzle (it only uses
// the row's low bits), so both become immediate offsets of the reads.
template <int D>
struct BwdOffsets {
  int row[D / 16];     // row reads, 16-channel step s: row ln, chunk 2s + hl
  int tr[D / 32][2];   // transpose reads, channel block db, 4-row half r
};

template <int D>
__device__ __forceinline__ BwdOffsets<D> bwd_offsets(int lane) {
  const int ln = lane & 31, hl = lane >> 5, gq = (lane >> 4) & 1, j = lane & 15;
  BwdOffsets<D> o;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) o.row[s] = 2 * brow_off<D>(ln, 2 * s + hl);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      // query 8hl + 4r + (j >> 2) of the first 16-row step, in pi order
      const int m = pi_row(8 * hl + 4 * r + (j >> 2));
      const int d = 32 * db + 16 * gq + 4 * (j & 3);
      o.tr[db][r] = 2 * (brow_off<D>(m, d >> 3) + (d & 7));
    }
  return o;
}

// The offsets formed where a tile's products start, from a lane index the
// compiler cannot see through: the addresses are then computed per tile and
// not kept live across the tile loop.
template <int D>
__device__ __forceinline__ BwdOffsets<D> bwd_offsets_here() {
  int lane = lane_id();
  asm volatile("" : "+v"(lane));
  return bwd_offsets<D>(lane);
}

template <int D>
__device__ __forceinline__ const uint16_t* at_byte(const uint16_t* tile, int bytes) {
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(tile) + bytes);
}

// Rows 32g .. 32g+31 of a row tile (A operand) against the wave's B operand
// (32 columns of D channels).
template <int D>
__device__ __forceinline__ f32x16 brows_group(const uint16_t* __restrict__ tile, const BwdOffsets<D>& o,
                                              const bf16x8 (&bop)[D / 16], int g) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(at_byte<D>(tile, o.row[s] + 64 * g * D)));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[s], acc, 0, 0, 0);
  }
  return acc;
}

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS transpose read (CDNA4): in every group of 16 lanes, lane 4x + a names
// 4 consecutive 16-bit values; lane 4a + b receives value b of lanes a, 4 + a,
// 8 + a, 12 + a, in that order.
__device__ __forceinline__ s16x4 tr_read(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// acc^T (D x 32) += T^T * pg, T the 32 rows of group g of a row tile and pg
// the 32 columns' packed bf16 values (8 consecutive rows per lane and 16-row
// step, rows in natural order).  The A operand (lane (ln, hl) of channel
// block db: channel 32db + ln, rows 16 s2 + 8hl .. +7) comes from two
// transpose reads of 4 rows each: in each 16-lane group, lane j names row
// 4r + (j >> 2) of the 8 and channels 4 (j & 3) .. +3 of the group's 16.
template <int D>
__device__ __forceinline__ void tr_group(const uint16_t* __restrict__ tile, const BwdOffsets<D>& o,
                                         const bf16x8 (&pg)[2], int g, f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int imm = (64 * g + 32 * s2) * D;   // bytes: 32g + 16 s2 rows
      const s16x4 lo = tr_read(at_byte<D>(tile, o.tr[db][0] + imm));
      const s16x4 hi = tr_read(at_byte<D>(tile, o.tr[db][1] + imm));
      const s16x8 a8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pg[s2], acc[db], 0, 0, 0);
    }
  }
}

// dS of one 32-key x 32-query block as a dK wave holds it (pg: lane (ln, hl)
// has key ln, queries 16 s2 + 8 hl .. +7), stored in the order the dQ pass
// takes it as its B operand (lane (ln, hl) of 16-key step s2: query ln, keys
// 16 s2 + 8 hl .. +7; 1 KB per step).  The transpose goes through 2 KB of LDS
// that only this wave touches meanwhile (`sb`): 32 rows of 32 queries, one
// per key, then two transpose reads per step.  Two halves, so that the wave
// can issue its products between writing the block into the slot
// (stage_ds_block) and reading it back transposed for the global stores
// (flush_ds_block).
__device__ __forceinline__ void stage_ds_block(char* sb, const bf16x8 (&pg)[2]) {
  const int lane = lane_id(), ln = lane & 31, hl = lane >> 5;
  asm volatile("" ::: "memory");
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
    *reinterpret_cast<u32x4*>(sb + ln * 64 + 32 * s2 + 16 * hl) = __builtin_bit_cast(u32x4, pg[s2]);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void flush_ds_block(const char* sb, u32x4* __restrict__ dst) {
  const int lane = lane_id();
  // in each 16-lane group G, lane 4x + a names key 8(G >> 1) + 4r + x (+16 s2)
  // and queries 16(G & 1) + 4a .. +3
  const int G = lane >> 4, x = (lane >> 2) & 3, a = lane & 3;
  const int rd = (8 * (G >> 1) + x) * 64 + (16 * (G & 1) + 4 * a) * 2;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const s16x4 lo = tr_read(reinterpret_cast<const uint16_t*>(sb + rd + 16 * s2 * 64));
    const s16x4 hi = tr_read(reinterpret_cast<const uint16_t*>(sb + rd + (16 * s2 + 4) * 64));
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), dst + 64 * s2 + lane);
  }
}
// The wave's B operand for 32 rows of a permuted tile: lane (ln, hl) holds
// row r0 + ln, channels 16s + 8hl .. +7.
template <int D>
__device__ __forceinline__ void load_bop(bf16x8 (&bop)[D / 16], const uint16_t* __restrict__ rows, int64_t r0) {
  const int lane = lane_id();
  const int ln = lane & 31, hl = lane >> 5;
  const uint16_t* r = rows + (r0 + ln) * D + 8 * hl;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) bop[s] = __builtin_bit_cast(bf16x8, ld16(r + 16 * s));
}

// Store acc^T (D x 32 columns; lane (ln, hl) holds rows 32db + 8j + 4hl + i)
// times `mul` as bf16 into row r0 + ln of a [R, D] array, or zeros.
template <int D>
__device__ __forceinline__ void store_t_rows(uint16_t* __restrict__ out, int64_t r0, const f32x16 (&acc)[D / 32],
                                             float mul, bool zero) {
  const int lane = lane_id();
  const int ln = lane & 31, hl = lane >> 5;
  uint16_t* row = out + (r0 + ln) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint2 v;
      v.x = zero ? 0u : pack_bf16x2(acc[db][4 * jj + 0] * mul, acc[db][4 * jj + 1] * mul);
      v.y = zero ? 0u : pack_bf16x2(acc[db][4 * jj + 2] * mul, acc[db][4 * jj + 3] * mul);
      *reinterpret_cast<uint2*>(row + 32 * db + 8 * jj + 4 * hl) = v;
    }
}

// ---------------------------------------------------------------------------
// backward: dK, dV over the transposed lists
// ---------------------------------------------------------------------------
//
// Two workgroups of 4 waves per (head, key tile j), one per 64-key half, so
// that two of them share a CU and one computes while the other waits at its
// barrier.  Waves 0-1 are dV waves, waves 2-3 dK waves; wave w & 1 of either
// kind owns keys 64 half + 32(w & 1) .. +31, whose K (dV wave) or V (dK
// wave) rows it holds as B operands.  The query tiles i that selected j
// are walked as a stream of 32-query chunks c = 4 e + g (entry e of the
// column, group g of tile i); for every chunk:
//   dV wave:  S' = Q K_w^T, P' = exp2(S' c - lse2) (packed bf16, also handed
//             to the dK wave of the same keys through LDS), dV_w^T += dO^T P'
//   dK wave:  dP' = dO V_w^T, dS' = P' (dP' - Dsum), dK_w^T += Q^T dS', and
//             dS' stored for the dQ pass
// (A = Q and dO rows from LDS, read as rows or transposed; B = P' / dS'
// straight from registers: with the pi row order a lane's eight values of a
// 16-query step are eight consecutive queries); one workgroup barrier per
// chunk publishes P'.  The chunks (Q and dO rows, 8 KB each at D = 128, and
// their 32 (lse2, Dsum) pairs) go through a ring of 4 LDS slots, copied by
// the dV waves only: at chunk c's barrier the copy of chunk c + 1 has landed
// and chunk c + 3 is issued into the slot chunk c - 1 has left (every wave
// is past it).  Workgroup b runs on XCD b mod 8; the two halves of a key
// tile take slots 16k + x and 16k + 8 + x, so they run on one XCD one after
// the other and share the column's query tiles in its L2.  Padding keys'
// rows are written as zeros; padding queries have zero Q and dO rows and
// contribute nothing.
// s_waitcnt immediate for vmcnt(n), n = 0 .. 63 (bits 3:0 and 15:14), with
// lgkmcnt(0); expcnt not waited for.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

constexpr int kBwdHalfThreads = 256;   // dK/dV workgroups: 4 waves, 64 keys

template <int D>
__global__ void __launch_bounds__(kBwdHalfThreads, 2) attn_bwd_dkdv_kernel(
    DevPlan p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ d_o, const float2* __restrict__ aux, const int32_t* __restrict__ col_ptr,
    const int32_t* __restrict__ row_idx, const int32_t* __restrict__ order, const int32_t* __restrict__ pos,
    float scale_log2, float scale, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, u32x4* __restrict__ xds) {
  constexpr int CS = 32 * D;                // bf16 elements of a 32-row chunk
  constexpr int SLOT = 2 * CS + 128;        // Q chunk, dO chunk, 32 (lse2, Dsum) pairs
  constexpr int AHEAD = 3;                  // chunks issued ahead of the one computing
  constexpr int CH = D / 8;                 // 16-byte pieces of a row
  constexpr int NIT = 32 * CH / 128;        // copy instructions per chunk, tensor and dV wave
  constexpr int NCOPY = 2 * NIT;            // per chunk and dV wave (wave 0: one more, the pairs)
  static_assert(NIT * 128 == 32 * CH, "a chunk is a whole number of copy instructions");
  // four separate slot arrays: a read of one slot never waits for the copies
  // still in flight into the others
  __shared__ __attribute__((aligned(16))) uint16_t r0[SLOT], r1[SLOT], r2[SLOT], r3[SLOT];
  // P' of chunk c handed from the dV wave to the dK wave of the same keys:
  // [chunk parity][key slice][16-query step][lane], packed bf16
  __shared__ __attribute__((aligned(16))) u32x4 xp[2][2][2][64];
  const int64_t T = p.total_tiles;
  const int bx = blockIdx.x, x8 = bx & 7, k2 = bx >> 3, half = k2 & 1;
  const int64_t slot_idx = (int64_t)8 * (k2 >> 1) + x8;
  if (slot_idx >= T) return;                // past the last key tile (uniform)
  const int t = uni(order[slot_idx]);
  const int h = uni(p.row_head[t]);
  const DevShape& sh = p.shape[uni(p.head_shape[h])];
  const int nt = sh.num_tiles;
  const int j = t - uni(p.head_tile_off[h]);
  const int nvk = uni(sh.valid[j]);
  const int64_t hrow = uni64(p.head_row_off[h]);
  const int wave = uni(threadIdx.x >> 6), w = wave & 1, lane = lane_id(), ln = lane & 31, hl = lane >> 5;
  const bool dk_wave = wave >= 2;
  const int kslice = 2 * half + w;          // the wave's 32-key group inside the tile
  const float c = scale_log2;
  const int64_t krow0 = hrow + (int64_t)kTile * j + 32 * kslice;
  const int64_t tile_bytes = (int64_t)kTile * D * 2;
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(q + hrow * D, nt * tile_bytes);
  const __amdgpu_buffer_rsrc_t rd = head_rsrc(d_o + hrow * D, nt * tile_bytes);
  const __amdgpu_buffer_rsrc_t rx = head_rsrc(aux + hrow, (int64_t)nt * kTile * 8);
  const int e0 = uni(col_ptr[t]), e1 = uni(col_ptr[t + 1]);
  const int nchunk = 4 * (e1 - e0);
  auto slot_of = [&](int cc) -> uint16_t* {
    const int sl = cc & 3;
    return sl < 2 ? (sl == 0 ? r0 : r1) : (sl == 2 ? r2 : r3);
  };
  // chunk cc into its ring slot (dV waves, 128 threads: instruction it moves
  // LDS positions 128 it + tid of the chunk, whose source rows follow the
  // row-tile layout)
  auto copy = [&](int cc) {
    const int i = min(max(uni(row_idx[e0 + (cc >> 2)]), 0), nt - 1);   // stay inside the head
    const int g = cc & 3;
    uint16_t* sl = slot_of(cc);
    const int cb = (i * kTile + 32 * g) * D * 2;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int loff = brow_lane_offset<D>((int)threadIdx.x + 128 * it);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, sl + it * 8 * 128 + 512 * wave, 16, loff, cb, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, sl + CS + it * 8 * 128 + 512 * wave, 16, loff, cb, 0, 0);
    }
    if (wave == 0 && lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, sl + 2 * CS, 16, 16 * lane, (i * kTile + 32 * g) * 8, 0, 0);
  };
  // The dV waves wait until a chunk's copy has landed, `younger` later
  // chunks (0 .. AHEAD - 1) being allowed in flight (per dV wave NCOPY copy
  // instructions a chunk, wave 0 one more for the pairs; the dV waves issue
  // no other vector memory instruction), then every wave meets at the barrier.
  auto chunk_sync = [&](int younger) {
    asm volatile("" ::: "memory");
    if (!dk_wave) {
      if (wave == 0) {
        if (younger >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (NCOPY + 1)));
        else if (younger == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NCOPY + 1));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      } else {
        if (younger >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NCOPY));
        else if (younger == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NCOPY));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  static_assert(2 * (NCOPY + 1) < 64, "vmcnt counts fit the 6-bit field");
  auto run = [&](auto dkc) {
    constexpr bool DK = decltype(dkc)::value;
    bf16x8 bop[D / 16];   // K rows (dV wave) or V rows (dK wave) of the wave's 32 keys
    load_bop<D>(bop, DK ? v : k, krow0);
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    // prologue: chunks 0 .. AHEAD-1 issued, chunk 0 waited for
    if constexpr (!DK) {
      for (int cc = 0; cc < min(nchunk, AHEAD); ++cc) copy(cc);
    }
    if (nchunk > 0) chunk_sync(min(nchunk, AHEAD) - 1);
    u32x4* xb = nullptr;   // the current block's dS in the workspace (nullptr: not stored)
    const BwdOffsets<D> o = bwd_offsets<D>(lane);   // the operand offsets, kept for the whole column
#pragma unroll 1
    for (int cc = 0; cc < nchunk; ++cc) {
      const int g = cc & 3;
      if constexpr (DK) {
        if (g == 0) {
          const int pe = uni(pos[e0 + (cc >> 2)]);
          xb = pe >= 0 ? xds + (int64_t)pe * (kBwdBlockBytes / 16) : nullptr;
        }
      }
      const uint16_t* qc = slot_of(cc);
      const uint16_t* dc = qc + CS;
      const float2* xc = reinterpret_cast<const float2*>(qc + 2 * CS);
      // register r holds query 16(r >> 3) + 8hl + (r & 7) of the chunk
      u32x4* slot = &xp[cc & 1][w][0][lane];
      bf16x8 pg[2];
      if constexpr (!DK) {
        const f32x16 sg = brows_group<D>(qc, o, bop, 0);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const float2* src = &xc[16 * s2 + 8 * hl];
          u32x4 pk;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float4 f = __builtin_bit_cast(float4, ld16(src + 2 * e2));   // (lse2, Dsum) of two queries
            const int r0i = 8 * s2 + 2 * e2, r1i = r0i + 1;
            pk[e2] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sg[r0i], c, -f.x)),
                                 __builtin_amdgcn_exp2f(fmaf(sg[r1i], c, -f.z)));
          }
          slot[64 * s2] = pk;      // P' for the dK wave of the same keys
          pg[s2] = __builtin_bit_cast(bf16x8, pk);
        }
        // P'(cc) published and chunk cc+1 landed; chunks up to cc+AHEAD-1 were
        // issued, so min(AHEAD-2, nchunk-2-cc) of them are younger than cc+1
        chunk_sync(min(AHEAD - 2, nchunk - 2 - cc));
        if (cc + AHEAD < nchunk) copy(cc + AHEAD);    // into the slot chunk cc-1 has left
        tr_group<D>(dc, o, pg, 0, acc);
      } else {
        const f32x16 dpg = brows_group<D>(dc, o, bop, 0);
        chunk_sync(0);   // the dK waves issue no copies: their count is not used
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const float2* src = &xc[16 * s2 + 8 * hl];
          const u32x4 pk = slot[64 * s2];
          u32x4 dk4;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float4 f = __builtin_bit_cast(float4, ld16(src + 2 * e2));
            const int r0i = 8 * s2 + 2 * e2, r1i = r0i + 1;
            const float p0 = __uint_as_float(pk[e2] << 16), p1 = __uint_as_float(pk[e2] & 0xffff0000u);
            dk4[e2] = pack_bf16x2(p0 * (dpg[r0i] - f.y), p1 * (dpg[r1i] - f.w));
          }
          pg[s2] = __builtin_bit_cast(bf16x8, dk4);
        }
        char* sb = reinterpret_cast<char*>(&xp[cc & 1][w][0][0]);
        if (xb) stage_ds_block(sb, pg);
        tr_group<D>(qc, o, pg, 0, acc);
        if (xb) flush_ds_block(sb, xb + (g * 4 + kslice) * 128);   // the transpose reads under the products
      }
    }
    const bool pad = 32 * kslice + ln >= nvk;
    if constexpr (DK)
      store_t_rows<D>(dk, krow0, acc, scale, pad);
    else
      store_t_rows<D>(dv, krow0, acc, 1.0f, pad);
  };
  if (dk_wave)
    run(BoolC<true>{});
  else
    run(BoolC<false>{});
}

// ---------------------------------------------------------------------------
// backward: dQ over the row lists
// ---------------------------------------------------------------------------
//
// dQ = scale dS K per query tile, with dS read back from the workspace where
// the dK/dV pass left it (one 32 KB block per kept block, in CSR order, in
// this kernel's operand order), so S and dP are not computed a second time.
// One workgroup of 8 waves per (head, query tile i): wave w & 3 owns queries
// 32(w & 3) .. +31 and wave w >> 2 of the pair key groups 2(w >> 2) and
// 2(w >> 2) + 1 of every key tile; dQ^T += K^T dS^T (A = the K tile read
// transposed, B = the dS operands, one 16-byte LDS read per lane each).  K
// tiles are double-buffered in LDS and the dS blocks, a stream from HBM,
// go through a ring of three LDS buffers: while block e computes, K tile
// e + 1 and dS block e + 2 are in flight.  The two partial dQ of a pair are
// summed through LDS at the end.
template <int D>
__global__ void __launch_bounds__(kBwdThreads, 1) attn_bwd_dq_kernel(
    DevPlan p, const uint16_t* __restrict__ k, const u32x4* __restrict__ xds, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, float scale, uint16_t* __restrict__ dq) {
  constexpr int TS = kTile * D;
  constexpr int XS = (int)(kBwdBlockBytes / 2);   // bf16 elements of a dS block
  __shared__ __attribute__((aligned(16))) uint16_t k0[TS];
  __shared__ __attribute__((aligned(16))) uint16_t k1[TS];
  __shared__ __attribute__((aligned(16))) uint16_t xr0[XS];
  __shared__ __attribute__((aligned(16))) uint16_t xr1[XS];
  __shared__ __attribute__((aligned(16))) uint16_t xr2[XS];
  const int t = blockIdx.x;
  const int h = uni(p.row_head[t]);
  const DevShape& sh = p.shape[uni(p.head_shape[h])];
  const int nt = sh.num_tiles;
  const int i = t - uni(p.head_tile_off[h]);
  const int64_t hrow = uni64(p.head_row_off[h]);
  const int wave = uni(threadIdx.x >> 6), w = wave & 3, kh = wave >> 2, lane = lane_id();
  const int64_t qrow0 = hrow + (int64_t)kTile * i + 32 * w;
  const int64_t tile_bytes = (int64_t)kTile * D * 2;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + hrow * D, nt * tile_bytes);
  const int loff = brow_lane_offset<D>(threadIdx.x);
  f32x16 dqacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};
  auto copy_k = [&](uint16_t* kd, int e) {
    const int jj = min(max(uni(col_idx[e]), 0), nt - 1);   // stay inside the head
    dma_row_tile<D>(kd, rk, jj * (int)tile_bytes, loff, wave);
  };
  // dS block e, a plain 32 KB copy (four 16-byte pieces per thread), with
  // the non-temporal cache policy: each block is read once, the K tiles
  // should keep the L2
  constexpr int kStreamLoad = 2;
  auto copy_x = [&](uint16_t* xd, int e) {
    const __amdgpu_buffer_rsrc_t rx = head_rsrc(xds + (int64_t)e * (kBwdBlockBytes / 16), kBwdBlockBytes);
#pragma unroll
    for (int it = 0; it < (int)(kBwdBlockBytes / (16 * kBwdThreads)); ++it)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, xd + it * 8 * kBwdThreads + 512 * wave, 16, 16 * (int)threadIdx.x,
                                               it * 16 * kBwdThreads, 0, kStreamLoad);
  };
  constexpr int XCOPY = (int)(kBwdBlockBytes / (16 * kBwdThreads));   // copy instructions per dS block
  const BwdOffsets<D> o = bwd_offsets<D>(lane);
  auto tile = [&](const uint16_t* kc, const uint16_t* xc) {
    // the wave's operands: key groups 2kh, 2kh+1, two 16-key steps each
    const u32x4* xw = reinterpret_cast<const u32x4*>(xc) + (w * 4 + 2 * kh) * 128 + lane;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 xv[2] = {__builtin_bit_cast(bf16x8, xw[u * 128]), __builtin_bit_cast(bf16x8, xw[u * 128 + 64])};
      tr_group<D>(kc, o, xv, 2 * kh + u, dqacc);
    }
  };
  const int e0 = uni(row_ptr[t]), e1 = uni(row_ptr[t + 1]);
  // step e: K tile e+1 and dS block e+2 are issued, block e computes; the
  // wait at its end leaves the copy of e+2 (issued last) in flight
  auto step = [&](int e, const uint16_t* kc, uint16_t* kn, const uint16_t* xc, uint16_t* xn) {
    if (e + 1 < e1) copy_k(kn, e + 1);
    const bool x2 = e + 2 < e1;
    if (x2) copy_x(xn, e + 2);
    __builtin_amdgcn_sched_barrier(0);
    tile(kc, xc);
    __builtin_amdgcn_sched_barrier(0);   // this block's products stay before the wait
    if (x2) dma_sync<XCOPY>(); else dma_sync<0>();
  };
  if (e0 < e1) {
    copy_k(k0, e0);
    copy_x(xr0, e0);
    if (e0 + 1 < e1) copy_x(xr1, e0 + 1);
  }
  dma_sync<0>();
  int xi = 0;   // ring slot of block e
#pragma unroll 1
  for (int e = e0; e < e1; ++e) {
    const bool odd = ((e - e0) & 1) != 0;
    uint16_t* xc = xi == 0 ? xr0 : (xi == 1 ? xr1 : xr2);
    uint16_t* xn = xi == 0 ? xr2 : (xi == 1 ? xr0 : xr1);   // the slot of block e + 2
    step(e, odd ? k1 : k0, odd ? k0 : k1, xc, xn);
    xi = xi == 2 ? 0 : xi + 1;
  }
  // pair reduction: the second wave of each pair parks its partial dQ in the
  // (now free) tile buffers, lane-major, the first adds it and stores
  float* park = reinterpret_cast<float*>(w < 2 ? k0 : k1) + (w & 1) * (D / 2) * 64;
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) park[(16 * db + r) * 64 + lane] = dqacc[db][r];
  }
  lds_sync();
  if (kh == 0) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqacc[db][r] += park[(16 * db + r) * 64 + lane];
    store_t_rows<D>(dq, qrow0, dqacc, scale, false);
  }
}

// Position in the CSR of every transposed-list entry: for key tile t and
// entry e (query tile i = row_idx[e] of the same head), the index of t's
// head-local key tile in row i's ascending col_idx (binary search), or -1 if
// the row does not hold it.  One wave per key tile.
__global__ void __launch_bounds__(64) bwd_pos_kernel(DevPlan p, const int32_t* __restrict__ row_ptr,
                                                    const int32_t* __restrict__ col_idx,
                                                    const int32_t* __restrict__ col_ptr,
                                                    const int32_t* __restrict__ row_idx, int32_t* __restrict__ pos) {
  const int64_t t = blockIdx.x;
  const int h = p.row_head[t];
  const int64_t toff = p.head_tile_off[h];
  const int n = p.shape[p.head_shape[h]].num_tiles;
  const int j = (int)(t - toff);
  const int e1 = col_ptr[t + 1];
  for (int e = col_ptr[t] + threadIdx.x; e < e1; e += 64) {
    const int64_t ti = toff + min(max(row_idx[e], 0), n - 1);
    const int end = row_ptr[ti + 1];
    int lo = row_ptr[ti], hi = end;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (col_idx[mid] < j)
        lo = mid + 1;
      else
        hi = mid;
    }
    pos[e] = (lo < end && col_idx[lo] == j) ? lo : -1;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_permute(const DevPlan& p, const void* src, void* dst, int direction, hipStream_t s) {
  const uint16_t* in = static_cast<const uint16_t*>(src);
  uint16_t* out = static_cast<uint16_t*>(dst);
  if (direction == VEDA_PERMUTE_FORWARD_TRANSPOSED) {   // the V path of the fused permutation alone
    const dim3 grid((unsigned)p.total_tiles, 1);
    if (p.head_dim == 128)
      hipLaunchKernelGGL(permute_qkv_kernel<128>, grid, dim3(256), 0, s, p, in, in, in, nullptr, nullptr, out, nullptr,
                         nullptr, 2);
    else
      hipLaunchKernelGGL(permute_qkv_kernel<64>, grid, dim3(128), 0, s, p, in, in, in, nullptr, nullptr, out, nullptr,
                         nullptr, 2);
    return hipGetLastError();
  }
  const int inverse = direction == VEDA_PERMUTE_INVERSE;
  const int rows_per_block = kThreads / (p.head_dim / 8);
  const dim3 grid((unsigned)((p.total_rows + rows_per_block - 1) / rows_per_block));
  if (p.head_dim == 128)
    hipLaunchKernelGGL(permute_rows_kernel<128>, grid, dim3(kThreads), 0, s, p, in, out, inverse);
  else
    hipLaunchKernelGGL(permute_rows_kernel<64>, grid, dim3(kThreads), 0, s, p, in, out, inverse);
  return hipGetLastError();
}

hipError_t launch_permute_qkv(const DevPlan& p, const void* q, const void* k, const void* v, void* qp, void* kp,
                              void* vt, void* ws, hipStream_t s) {
  const int D = p.head_dim;
  const int64_t T = p.total_tiles;
  float* feat_q = ws ? static_cast<float*>(ws) : nullptr;
  float* feat_k = ws ? feat_q + T * 3 * D : nullptr;
  const dim3 grid((unsigned)T, v ? 3 : 2);   // blockIdx.y: Q, K, V
  auto cq = static_cast<const uint16_t*>(q);
  auto ck = static_cast<const uint16_t*>(k);
  auto cv = static_cast<const uint16_t*>(v);
  auto oq = static_cast<uint16_t*>(qp);
  auto ok = static_cast<uint16_t*>(kp);
  auto ov = static_cast<uint16_t*>(vt);
  if (D == 128)
    hipLaunchKernelGGL(permute_qkv_kernel<128>, grid, dim3(256), 0, s, p, cq, ck, cv, oq, ok, ov, feat_q, feat_k, 0);
  else
    hipLaunchKernelGGL(permute_qkv_kernel<64>, grid, dim3(128), 0, s, p, cq, ck, cv, oq, ok, ov, feat_q, feat_k, 0);
  return hipGetLastError();
}

hipError_t launch_score_pooled(const DevPlan& p, const float* wq, const float* wk, float* scores, void* ws,
                               hipStream_t s) {
  const int D = p.head_dim;
  const int64_t T = p.total_tiles;
  float* feat_q = static_cast<float*>(ws);
  float* feat_k = feat_q + T * 3 * D;
  float* hat_q = feat_k + T * 3 * D;
  float* hat_k = hat_q + T * D;
  int maxn = 0;
  for (int g = 0; g < p.num_shapes; ++g) maxn = maxn > p.shape[g].num_tiles ? maxn : p.shape[g].num_tiles;
  const dim3 gproj((unsigned)((maxn + kPrjTB - 1) / kPrjTB), (unsigned)p.num_heads, 2);
  const dim3 gscore((unsigned)((maxn + 63) / 64), (unsigned)((maxn + 63) / 64), (unsigned)p.num_heads);
  if (D == 128) {
    hipLaunchKernelGGL(project_kernel<128>, gproj, dim3(kThreads), 0, s, p, wq, wk, feat_q, feat_k, hat_q, hat_k);
    hipLaunchKernelGGL(score_kernel<128>, gscore, dim3(kThreads), 0, s, p, hat_q, hat_k, scores);
  } else {
    hipLaunchKernelGGL(project_kernel<64>, gproj, dim3(kThreads), 0, s, p, wq, wk, feat_q, feat_k, hat_q, hat_k);
    hipLaunchKernelGGL(score_kernel<64>, gscore, dim3(kThreads), 0, s, p, hat_q, hat_k, scores);
  }
  return hipGetLastError();
}

hipError_t launch_score(const DevPlan& p, const void* q, const void* k, const float* wq, const float* wk,
                        float* scores, void* ws, hipStream_t s) {
  const int D = p.head_dim;
  const int64_t T = p.total_tiles;
  float* feat_q = static_cast<float*>(ws);
  float* feat_k = feat_q + T * 3 * D;
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const dim3 gpool((unsigned)T, 2);
  if (D == 128)
    hipLaunchKernelGGL(pool_kernel<128>, gpool, dim3(kThreads), 0, s, p, qq, kk, feat_q, feat_k);
  else
    hipLaunchKernelGGL(pool_kernel<64>, gpool, dim3(kThreads), 0, s, p, qq, kk, feat_q, feat_k);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_score_pooled(p, wq, wk, scores, ws, s);
}

hipError_t launch_select(const DevPlan& p, const float* scores, int32_t* row_ptr, int32_t* col_idx,
                         uint8_t* dense_mask, hipStream_t s) {
  int maxn = 0;
  for (int g = 0; g < p.num_shapes; ++g) maxn = maxn > p.shape[g].num_tiles ? maxn : p.shape[g].num_tiles;
  const dim3 grid((unsigned)p.total_tiles), block(64);
  // rows of 513 .. 2048 key tiles are staged in LDS (sized to 1,152 or 2,048
  // columns); shorter and longer rows read the scores in every pass
  if (maxn > 512 && maxn <= 1152)
    hipLaunchKernelGGL(select_staged_kernel<18>, grid, block, 0, s, p, scores, row_ptr, col_idx, dense_mask);
  else if (maxn > 1152 && maxn <= 2048)
    hipLaunchKernelGGL(select_staged_kernel<32>, grid, block, 0, s, p, scores, row_ptr, col_idx, dense_mask);
  else
    hipLaunchKernelGGL(select_kernel, grid, block, 0, s, p, scores, row_ptr, col_idx, dense_mask);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const DevPlan& p, const void* q, int q_natural, const void* k, const void* vt,
                           const int32_t* row_ptr,
                           const int32_t* col_idx, float scale, void* o, int o_natural, float* lse,
                           uint32_t* visited, hipStream_t s) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)p.attn_grid);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(vt);
  uint16_t* oo = static_cast<uint16_t*>(o);
  // o == nullptr: only the LSE (no PV products, no V^T copies)
  if (p.head_dim == 128) {
    if (oo)
      hipLaunchKernelGGL((attn_fwd_kernel<128, true>), grid, dim3(kThreads), 0, s, p, qq, q_natural, kk, vv, row_ptr, col_idx,
                         scale_log2, oo, o_natural, lse, visited);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<128, false>), grid, dim3(kThreads), 0, s, p, qq, q_natural, kk, vv, row_ptr, col_idx,
                         scale_log2, oo, o_natural, lse, visited);
  } else {
    if (oo)
      hipLaunchKernelGGL((attn_fwd_kernel<64, true>), grid, dim3(kThreads), 0, s, p, qq, q_natural, kk, vv, row_ptr, col_idx,
                         scale_log2, oo, o_natural, lse, visited);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<64, false>), grid, dim3(kThreads), 0, s, p, qq, q_natural, kk, vv, row_ptr, col_idx,
                         scale_log2, oo, o_natural, lse, visited);
  }
  return hipGetLastError();
}

hipError_t launch_lse_heat(const DevPlan& p, const void* q, int q_natural, const void* k, const int32_t* row_ptr,
                           const int32_t* col_idx, float scale, float* lse, float* bsum, float* heat, hipStream_t s) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)p.attn_grid);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  if (p.head_dim == 128)
    hipLaunchKernelGGL(lse_heat_kernel<128>, grid, dim3(kThreads), 0, s, p, qq, q_natural, kk, row_ptr, col_idx, scale_log2, lse,
                       bsum, heat);
  else
    hipLaunchKernelGGL(lse_heat_kernel<64>, grid, dim3(kThreads), 0, s, p, qq, q_natural, kk, row_ptr, col_idx, scale_log2, lse,
                       bsum, heat);
  return hipGetLastError();
}

hipError_t launch_attn_lse_heat(const DevPlan& sel, const DevPlan& dense, const void* q, int q_natural,
                                const void* k, const void* vt, const int32_t* row_ptr, const int32_t* col_idx,
                                const int32_t* dense_row_ptr, const int32_t* dense_col_idx, float scale, void* o,
                                int o_natural, float* lse_sel, float* dense_lse, float* heat,
                                const SplitWorkspace& ws, hipStream_t s) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(vt);
  uint16_t* oo = static_cast<uint16_t*>(o);
  if (sel.head_dim == 128)
    hipLaunchKernelGGL(attn_mass_kernel<128>, dim3((unsigned)sel.attn_grid), dim3(kThreads), 0, s, sel, qq, q_natural,
                       kk, vv, row_ptr, col_idx, scale_log2, oo, o_natural, lse_sel, ws.mass, ws.fac);
  else
    hipLaunchKernelGGL(attn_mass_kernel<64>, dim3((unsigned)sel.attn_grid), dim3(kThreads), 0, s, sel, qq, q_natural,
                       kk, vv, row_ptr, col_idx, scale_log2, oo, o_natural, lse_sel, ws.mass, ws.fac);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(complement_kernel, dim3((unsigned)dense.total_tiles), dim3(kThreads), 0, s, dense_row_ptr,
                     dense_col_idx, row_ptr, col_idx, ws.rest_nnz, ws.rest_col, ws.cflag);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const HeatSplit hs{row_ptr, col_idx, ws.cflag, lse_sel, ws.mass, ws.fac};
  if (dense.head_dim == 128)
    hipLaunchKernelGGL(rest_heat_kernel<128>, dim3((unsigned)dense.attn_grid), dim3(kThreads), 0, s, dense, qq,
                       q_natural, kk, dense_row_ptr, ws.rest_col, scale_log2, dense_lse, ws.rest_bsum, heat, hs);
  else
    hipLaunchKernelGGL(rest_heat_kernel<64>, dim3((unsigned)dense.attn_grid), dim3(kThreads), 0, s, dense, qq,
                       q_natural, kk, dense_row_ptr, ws.rest_col, scale_log2, dense_lse, ws.rest_bsum, heat, hs);
  return hipGetLastError();
}

hipError_t launch_heat(const DevPlan& p, const void* q, const void* k, const float* lse, float scale, float* heat,
                       hipStream_t s) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)p.total_tiles);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  if (p.head_dim == 128)
    hipLaunchKernelGGL(heat_kernel<128>, grid, dim3(kThreads), 0, s, p, qq, kk, lse, scale_log2, heat);
  else
    hipLaunchKernelGGL(heat_kernel<64>, grid, dim3(kThreads), 0, s, p, qq, kk, lse, scale_log2, heat);
  return hipGetLastError();
}

hipError_t launch_mask_mass(const DevPlan& p, int32_t max_tiles, const float* heat, const int32_t* row_ptr,
                            const int32_t* col_idx, double* mass, void* ws, hipStream_t s) {
  const int chunks = mass_chunks(max_tiles);
  double2* part = static_cast<double2*>(ws);
  hipLaunchKernelGGL(mask_mass_part_kernel, dim3((unsigned)chunks, (unsigned)p.num_heads), dim3(kThreads), 0, s, p,
                     heat, row_ptr, col_idx, part, chunks);
  hipLaunchKernelGGL(mask_mass_final_kernel, dim3((unsigned)((p.num_heads + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, s, p.num_heads, part, chunks, mass);
  return hipGetLastError();
}

hipError_t launch_output_error(const DevPlan& p, int64_t num_tokens, const void* o, const void* o_ref, double* err,
                               void* ws, hipStream_t s) {
  const uint16_t* a = static_cast<const uint16_t*>(o);
  const uint16_t* b = static_cast<const uint16_t*>(o_ref);
  double2* part = static_cast<double2*>(ws);
  const dim3 grid(kErrChunks, (unsigned)p.num_heads);
  if (p.head_dim == 128)
    hipLaunchKernelGGL(output_error_part_kernel<128>, grid, dim3(kThreads), 0, s, num_tokens, p.num_heads, a, b, part);
  else
    hipLaunchKernelGGL(output_error_part_kernel<64>, grid, dim3(kThreads), 0, s, num_tokens, p.num_heads, a, b, part);
  hipLaunchKernelGGL(output_error_final_kernel, dim3((unsigned)((p.num_heads + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, p.num_heads, part, err);
  return hipGetLastError();
}

hipError_t launch_mask_transpose(const DevPlan& p, const int32_t* row_ptr, const int32_t* col_idx, int32_t* col_ptr,
                                 int32_t* row_idx, void* workspace, int64_t total_pairs, hipStream_t s) {
  uint8_t* bitmap = static_cast<uint8_t*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(bitmap + align256(total_pairs));
  const int64_t words = (total_pairs + 3) / 4;
  const unsigned fill_blocks = (unsigned)std::min<int64_t>((words + kThreads - 1) / kThreads, 65536);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(std::max(fill_blocks, 1u)), dim3(kThreads), 0, s,
                     reinterpret_cast<uint32_t*>(bitmap), words, 0u);
  hipLaunchKernelGGL(csc_scatter_kernel, dim3((unsigned)p.total_tiles), dim3(64), 0, s, p, row_ptr, col_idx, bitmap);
  const dim3 gcol((unsigned)p.total_tiles);
  hipLaunchKernelGGL(csc_column_kernel<false>, gcol, dim3(64), 0, s, p, bitmap, counts, nullptr, nullptr);
  hipLaunchKernelGGL(csc_scan_kernel, dim3(1), dim3(1024), 0, s, counts, (int64_t)p.total_tiles, col_ptr);
  hipLaunchKernelGGL(csc_column_kernel<true>, gcol, dim3(64), 0, s, p, bitmap, counts, col_ptr, row_idx);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const DevPlan& p, const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                           const int32_t* col_ptr, const int32_t* row_idx, float scale, void* dq, void* dk,
                           void* dv, void* workspace, hipStream_t s) {
  const int D = p.head_dim;
  const int64_t R = p.total_rows, T = p.total_tiles;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float2* aux = reinterpret_cast<float2*>(ws);
  int32_t* order = reinterpret_cast<int32_t*>(ws + align256(R * 8));
  int32_t* pos = reinterpret_cast<int32_t*>(ws + align256(R * 8) + align256(T * 4));
  u32x4* xds = reinterpret_cast<u32x4*>(ws + align256(R * 8) + align256(T * 4) + align256(p.nnz * 4));
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  const uint16_t* oo = static_cast<const uint16_t*>(o);
  const uint16_t* dd = static_cast<const uint16_t*>(d_o);
  uint16_t* dqq = static_cast<uint16_t*>(dq);
  uint16_t* dkk = static_cast<uint16_t*>(dk);
  uint16_t* dvv = static_cast<uint16_t*>(dv);
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 gt((unsigned)T), gprep((unsigned)((R * (D / 8) + kThreads - 1) / kThreads));
  const dim3 gkv((unsigned)(16 * ((T + 7) / 8)));   // two halves per key tile, slots as bwd_order_kernel deals them
  hipLaunchKernelGGL(bwd_order_kernel, dim3(1), dim3(1024), 0, s, col_ptr, T, order);
  hipLaunchKernelGGL(bwd_pos_kernel, gt, dim3(64), 0, s, p, row_ptr, col_idx, col_ptr, row_idx, pos);
  if (D == 128) {
    hipLaunchKernelGGL(bwd_prep_kernel<128>, gprep, dim3(kThreads), 0, s, R, oo, dd, lse, aux);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, gkv, dim3(kBwdHalfThreads), 0, s, p, qq, kk, vv, dd, aux, col_ptr,
                       row_idx,
                       order, pos, scale_log2, scale, dkk, dvv, xds);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, gt, dim3(kBwdThreads), 0, s, p, kk, xds, row_ptr, col_idx, scale, dqq);
  } else {
    hipLaunchKernelGGL(bwd_prep_kernel<64>, gprep, dim3(kThreads), 0, s, R, oo, dd, lse, aux);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, gkv, dim3(kBwdHalfThreads), 0, s, p, qq, kk, vv, dd, aux, col_ptr,
                       row_idx,
                       order, pos, scale_log2, scale, dkk, dvv, xds);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, gt, dim3(kBwdThreads), 0, s, p, kk, xds, row_ptr, col_idx, scale, dqq);
  }
  return hipGetLastError();
}

}  // namespace veda

// ---------------------------------------------------------------------------
// static scratch for callers that cannot allocate
// ---------------------------------------------------------------------------
//
// One fixed array per GPU, reserved when the library's code object is loaded
// on that GPU and held until the process ends.  On the host the array's name
// only stands in for the device symbol: it is never passed to a kernel or a
// copy.  The first use on a device asks HIP for the array's device address on
// that device (with it current) and keeps it; every later use takes the kept
// address.
static __device__ __align__(256) uint8_t scratch[veda::kStaticScratchBytes];

namespace veda {

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;   // device -> device address of `scratch`
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

}  // namespace veda
