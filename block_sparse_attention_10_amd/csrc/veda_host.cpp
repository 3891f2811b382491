// Host side of libveda: plan construction (GPU-free), argument checks and the
// C ABI declared in include/veda.h.
//
// The plan fixes everything the Veda method decides before it looks at data
// (Miowtion project page, Key Features > "Veda sparse attention"): the 3D
// tiles of every head with their valid-prefix padding, the slot->token tables,
// the equal-kernel-cost budgets with Bresenham rounding and the forced
// diagonal, and with them the CSR row pointers and the exact block count.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "veda.h"
#include "veda_internal.h"

using namespace veda;

namespace {

thread_local std::string g_last_error;

veda_status fail(veda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

veda_status ok() { return VEDA_OK; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// floor(x + 1/2) for the non-negative rational x = num / den.
int64_t round_half_up(__int128 num, __int128 den) {
  return (int64_t)((2 * num + den) / (2 * den));
}

struct HostShape {
  int32_t a = 0, b = 0, c = 0;
  int32_t num_tiles = 0;
  std::vector<int32_t> perm, valid, tile_seg, budget, local_row_ptr;
  std::vector<int32_t> seg_first, seg_count;
  int64_t nnz = 0;  // kept blocks of one head with this shape
  int32_t max_row = 0, min_row = 0;
};

}  // namespace

struct veda_plan {
  veda_plan_info info{};
  std::vector<veda_segment> segs;
  int32_t budget_mode = 0, keep_num = 0, keep_den = 1, fixed_k = 0;
  std::vector<HostShape> shapes;
  std::vector<int32_t> head_shape, head_tile_off, row_head, row_ptr, attn_order;
  std::vector<int64_t> head_row_off, head_pair_off, head_nnz_off;
  // device tables
  std::vector<uint8_t> staging;     // host image of the device tables
  std::vector<size_t> table_offset; // byte offsets of each table in the image
  DevPlan dev{};
  int32_t device = -1;
};

namespace {

// Tiles of one segment in order (row-major over the padded tile grid; inside a
// tile, the valid box row-major; valid prefix, then padding).
void tile_segment(const veda_segment& sg, int32_t si, int a, int b, int c, HostShape& hs) {
  if (sg.kind == VEDA_SEG_DENSE1D) {
    const int64_t n = sg.w;
    for (int64_t tau = 0; tau < ceil_div(n, kTile); ++tau) {
      const int32_t v = (int32_t)std::min<int64_t>(kTile, n - kTile * tau);
      for (int s = 0; s < kTile; ++s)
        hs.perm.push_back(s < v ? (int32_t)(sg.token_offset + kTile * tau + s) : -1);
      hs.valid.push_back(v);
      hs.tile_seg.push_back(si);
    }
    return;
  }
  const int64_t T = sg.t, H = sg.h, W = sg.w;
  const int64_t nt = ceil_div(T, a), nh = ceil_div(H, b), nw = ceil_div(W, c);
  for (int64_t ta = 0; ta < nt; ++ta)
    for (int64_t tb = 0; tb < nh; ++tb)
      for (int64_t tc = 0; tc < nw; ++tc) {
        const int64_t vt = std::min<int64_t>(a, T - ta * a);
        const int64_t vh = std::min<int64_t>(b, H - tb * b);
        const int64_t vw = std::min<int64_t>(c, W - tc * c);
        const int64_t v = vt * vh * vw;
        for (int64_t s = 0; s < kTile; ++s) {
          if (s >= v) {
            hs.perm.push_back(-1);
            continue;
          }
          const int64_t u = s / (vh * vw), y = (s / vw) % vh, x = s % vw;
          const int64_t tok = sg.token_offset + ((ta * a + u) * H + (tb * b + y)) * W + (tc * c + x);
          hs.perm.push_back((int32_t)tok);
        }
        hs.valid.push_back((int32_t)v);
        hs.tile_seg.push_back(si);
      }
}

// Budgets k[i][B] of every row of one shape, then local CSR offsets.
void build_budgets(veda_plan& p, HostShape& hs) {
  const int S = (int)p.segs.size();
  const int n = hs.num_tiles;
  hs.budget.assign((size_t)n * S, 0);
  for (int A = 0; A < S; ++A) {
    const int64_t nA = hs.seg_count[A];
    const int64_t NA = (int64_t)p.segs[A].t * p.segs[A].h * p.segs[A].w;
    for (int B = 0; B < S; ++B) {
      const int64_t nB = hs.seg_count[B];
      const int64_t NB = (int64_t)p.segs[B].t * p.segs[B].h * p.segs[B].w;
      const bool dense = p.budget_mode == VEDA_BUDGET_ALL || p.segs[A].kind != VEDA_SEG_VIDEO3D ||
                         p.segs[B].kind != VEDA_SEG_VIDEO3D;
      for (int64_t li = 0; li < nA; ++li) {
        int64_t k;
        if (dense) {
          k = nB;
        } else {
          if (p.budget_mode == VEDA_BUDGET_FIXED_K) {
            k = p.fixed_k;
          } else {
            // per-row budget b = keep * N_A * N_B / (128^2 * n_A); midpoint Bresenham
            const __int128 num = (__int128)p.keep_num * NA * NB;
            const __int128 den = (__int128)p.keep_den * kTile * kTile * nA;
            k = round_half_up((li + 1) * num, den) - round_half_up(li * num, den);
          }
          if (A == B) k = std::max<int64_t>(k, 1);
          k = std::min<int64_t>(k, nB);
        }
        hs.budget[(size_t)(hs.seg_first[A] + li) * S + B] = (int32_t)k;
      }
    }
  }
  hs.local_row_ptr.assign(n + 1, 0);
  hs.max_row = 0;
  hs.min_row = INT32_MAX;
  for (int i = 0; i < n; ++i) {
    int32_t len = 0;
    for (int B = 0; B < S; ++B) len += hs.budget[(size_t)i * S + B];
    hs.local_row_ptr[i + 1] = hs.local_row_ptr[i] + len;
    hs.max_row = std::max(hs.max_row, len);
    hs.min_row = std::min(hs.min_row, len);
  }
  hs.nnz = hs.local_row_ptr[n];
}

template <typename T>
size_t append_table(std::vector<uint8_t>& img, const std::vector<T>& v) {
  size_t off = (img.size() + 255) & ~size_t(255);
  img.resize(off + v.size() * sizeof(T));
  if (!v.empty()) std::memcpy(img.data() + off, v.data(), v.size() * sizeof(T));
  return off;
}

// Order in which attention workgroups take query tiles.  Rows of equal cost
// keep head-major order so neighbouring query tiles of one head (which keep
// overlapping key tiles) run close in time; when some rows cost far more
// than the typical row (the dense audio rows of a packed sequence) those go
// first, longest first, and the rest keep the head-major order.
void build_attn_order(veda_plan& p) {
  const int64_t T = p.info.total_tiles;
  std::vector<int32_t> len(T);
  for (int64_t t = 0; t < T; ++t) len[t] = p.row_ptr[t + 1] - p.row_ptr[t];
  std::vector<int32_t> sorted(len);
  std::nth_element(sorted.begin(), sorted.begin() + T / 2, sorted.end());
  const int32_t median = T > 0 ? sorted[T / 2] : 0;
  std::vector<int32_t> longs, rest;
  for (int64_t t = 0; t < T; ++t) (len[t] > 2 * median + 2 ? longs : rest).push_back((int32_t)t);
  std::stable_sort(longs.begin(), longs.end(), [&](int32_t x, int32_t y) { return len[x] > len[y]; });
  // Workgroup b runs on XCD b % 8 (8 XCDs, each with its own L2).  The long
  // rows take the first workgroups (spread over the XCDs); after them each
  // XCD gets one contiguous run of the head-major order, so the query tiles
  // that are resident together on an XCD are spatial neighbours of one head
  // and share most of their key tiles in that XCD's L2.
  constexpr int64_t kXcds = 8;
  const int64_t L = (int64_t)longs.size();
  const int64_t L8 = (L + kXcds - 1) / kXcds * kXcds;   // the rest starts on XCD 0
  const int64_t R = (int64_t)rest.size();
  const int64_t per = (R + kXcds - 1) / kXcds;
  p.attn_order.assign(L8 + per * kXcds, -1);
  for (int64_t b = 0; b < L; ++b) p.attn_order[b] = longs[b];
  for (int64_t b = 0; b < per * kXcds; ++b) {
    const int64_t logical = (b % kXcds) * per + b / kXcds;
    if (logical < R) p.attn_order[L8 + b] = rest[logical];
  }
}

void build_staging(veda_plan& p) {
  std::vector<uint8_t>& img = p.staging;
  img.clear();
  p.table_offset.clear();
  for (auto& s : p.shapes) {
    p.table_offset.push_back(append_table(img, s.perm));
    p.table_offset.push_back(append_table(img, s.valid));
    p.table_offset.push_back(append_table(img, s.tile_seg));
    p.table_offset.push_back(append_table(img, s.budget));
    p.table_offset.push_back(append_table(img, s.local_row_ptr));
  }
  p.table_offset.push_back(append_table(img, p.head_shape));
  p.table_offset.push_back(append_table(img, p.head_row_off));
  p.table_offset.push_back(append_table(img, p.head_tile_off));
  p.table_offset.push_back(append_table(img, p.head_pair_off));
  p.table_offset.push_back(append_table(img, p.head_nnz_off));
  p.table_offset.push_back(append_table(img, p.row_head));
  p.table_offset.push_back(append_table(img, p.row_ptr));
  p.table_offset.push_back(append_table(img, p.attn_order));
  img.resize((img.size() + 255) & ~size_t(255));
}

void bind_device(veda_plan& p, uint8_t* base) {
  DevPlan& d = p.dev;
  d = DevPlan{};
  d.num_heads = p.info.num_heads;
  d.head_dim = p.info.head_dim;
  d.num_segments = p.info.num_segments;
  d.num_shapes = p.info.num_shapes;
  d.num_tokens = p.info.num_tokens;
  d.total_rows = p.info.total_rows;
  d.total_tiles = p.info.total_tiles;
  d.total_pairs = p.info.total_pairs;
  d.nnz = p.info.nnz;
  d.all_dense = p.budget_mode == VEDA_BUDGET_ALL;
  for (int s = 0; s < (int)p.segs.size(); ++s) d.seg_dense[s] = p.segs[s].kind != VEDA_SEG_VIDEO3D;
  size_t k = 0;
  for (int s = 0; s < (int)p.shapes.size(); ++s) {
    DevShape& ds = d.shape[s];
    const HostShape& hs = p.shapes[s];
    ds.perm = (const int32_t*)(base + p.table_offset[k++]);
    ds.valid = (const int32_t*)(base + p.table_offset[k++]);
    ds.tile_seg = (const int32_t*)(base + p.table_offset[k++]);
    ds.budget = (const int32_t*)(base + p.table_offset[k++]);
    ds.local_row_ptr = (const int32_t*)(base + p.table_offset[k++]);
    ds.num_tiles = hs.num_tiles;
    for (int g = 0; g < (int)p.segs.size(); ++g) {
      ds.seg_first[g] = hs.seg_first[g];
      ds.seg_count[g] = hs.seg_count[g];
    }
  }
  d.head_shape = (const int32_t*)(base + p.table_offset[k++]);
  d.head_row_off = (const int64_t*)(base + p.table_offset[k++]);
  d.head_tile_off = (const int32_t*)(base + p.table_offset[k++]);
  d.head_pair_off = (const int64_t*)(base + p.table_offset[k++]);
  d.head_nnz_off = (const int64_t*)(base + p.table_offset[k++]);
  d.row_head = (const int32_t*)(base + p.table_offset[k++]);
  d.row_ptr = (const int32_t*)(base + p.table_offset[k++]);
  d.attn_order = (const int32_t*)(base + p.table_offset[k++]);
  d.attn_grid = (int32_t)p.attn_order.size();
}

// ---------------------------------------------------------------------------
// device support
// ---------------------------------------------------------------------------

std::mutex g_dev_mu;
std::map<int, std::pair<bool, std::string>> g_dev_cache;

bool device_supported(int dev, std::string* why) {
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    auto it = g_dev_cache.find(dev);
    if (it != g_dev_cache.end()) {
      if (why) *why = it->second.second;
      return it->second.first;
    }
  }
  bool okay = false;
  std::string reason;
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) {
    reason = "no HIP device visible";
  } else if (dev < 0 || dev >= count) {
    reason = "device index " + std::to_string(dev) + " out of range";
  } else {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      reason = std::string("hipGetDeviceProperties failed: ") + hipGetErrorString(e);
    } else if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      reason = std::string("libveda is built for gfx950 (MI355X) only; device is ") + prop.gcnArchName;
    } else {
      okay = true;
    }
  }
  (void)hipGetLastError();  // do not leave a sticky error from the probe
  std::lock_guard<std::mutex> lk(g_dev_mu);
  g_dev_cache[dev] = {okay, reason};
  if (why) *why = reason;
  return okay;
}

veda_status check_device(const veda_plan* p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(VEDA_ERR_UNSUPPORTED, "no current HIP device");
  std::string why;
  if (!device_supported(dev, &why)) return fail(VEDA_ERR_UNSUPPORTED, "%s", why.c_str());
  if (p && p->device != dev)
    return fail(VEDA_ERR_STATE, "plan tables were uploaded to device %d, current device is %d",
                p->device, dev);
  return ok();
}

veda_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(VEDA_ERR_INVALID_ARG, "%s is NULL", name);
  if ((reinterpret_cast<uintptr_t>(ptr) & 15) != 0)
    return fail(VEDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return ok();
}

veda_status check_plan_ready(const veda_plan* p) {
  if (!p) return fail(VEDA_ERR_INVALID_ARG, "plan is NULL");
  if (!p->info.uploaded) return fail(VEDA_ERR_STATE, "plan tables not uploaded (veda_plan_upload)");
  return check_device(p);
}

veda_status launched(hipError_t e, const char* what) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(VEDA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int veda_abi_version(void) { return VEDA_ABI_VERSION; }

const char* veda_last_error(void) { return g_last_error.c_str(); }

veda_status veda_available(int device, char* reason, size_t n) {
  std::string why;
  const bool okay = device_supported(device, &why);
  if (reason && n > 0) {
    std::snprintf(reason, n, "%s", okay ? "" : why.c_str());
  }
  if (!okay) return fail(VEDA_ERR_UNSUPPORTED, "%s", why.c_str());
  return ok();
}

veda_status veda_plan_create(const veda_plan_desc* d, veda_plan** out) {
  if (!out) return fail(VEDA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!d) return fail(VEDA_ERR_INVALID_ARG, "desc is NULL");
  if (!d->segments || !d->tile_shape) return fail(VEDA_ERR_INVALID_ARG, "segments / tile_shape is NULL");
  if (d->num_segments < 1 || d->num_segments > kMaxSegments)
    return fail(VEDA_ERR_UNSUPPORTED, "num_segments %d not in 1..%d", d->num_segments, kMaxSegments);
  if (d->num_heads < 1 || d->num_heads > 1024)
    return fail(VEDA_ERR_UNSUPPORTED, "num_heads %d not in 1..1024", d->num_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(VEDA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->budget_mode < VEDA_BUDGET_KEEP_RATIO || d->budget_mode > VEDA_BUDGET_ALL)
    return fail(VEDA_ERR_INVALID_ARG, "unknown budget_mode %d", d->budget_mode);
  if (d->budget_mode == VEDA_BUDGET_KEEP_RATIO &&
      (d->keep_den <= 0 || d->keep_num < 0 || d->keep_num > d->keep_den))
    return fail(VEDA_ERR_INVALID_ARG, "keep ratio %d/%d not in [0, 1]", d->keep_num, d->keep_den);
  if (d->budget_mode == VEDA_BUDGET_FIXED_K && d->fixed_k < 0)
    return fail(VEDA_ERR_INVALID_ARG, "fixed_k %d < 0", d->fixed_k);

  veda_plan* p = new (std::nothrow) veda_plan();
  if (!p) return fail(VEDA_ERR_INVALID_ARG, "out of host memory");
  p->budget_mode = d->budget_mode;
  p->keep_num = d->keep_num;
  p->keep_den = d->keep_den;
  p->fixed_k = d->fixed_k;

  int64_t next = 0;
  for (int s = 0; s < d->num_segments; ++s) {
    const veda_segment& sg = d->segments[s];
    if (sg.kind != VEDA_SEG_VIDEO3D && sg.kind != VEDA_SEG_DENSE1D) {
      delete p;
      return fail(VEDA_ERR_INVALID_ARG, "segment %d: unknown kind %d", s, sg.kind);
    }
    if (sg.t < 1 || sg.h < 1 || sg.w < 1 || (sg.kind == VEDA_SEG_DENSE1D && (sg.t != 1 || sg.h != 1))) {
      delete p;
      return fail(VEDA_ERR_SHAPE, "segment %d: bad grid (%d,%d,%d)", s, sg.t, sg.h, sg.w);
    }
    if (sg.token_offset != next) {
      delete p;
      return fail(VEDA_ERR_SHAPE, "segment %d: token_offset %lld, expected %lld (segments are contiguous from 0)",
                  s, (long long)sg.token_offset, (long long)next);
    }
    next += (int64_t)sg.t * sg.h * sg.w;
    p->segs.push_back(sg);
  }
  if (next >= (int64_t(1) << 31)) {
    delete p;
    return fail(VEDA_ERR_UNSUPPORTED, "%lld tokens: more than 2^31 - 1", (long long)next);
  }

  // distinct shapes
  std::vector<std::array<int32_t, 3>> shape_list;
  p->head_shape.resize(d->num_heads);
  for (int h = 0; h < d->num_heads; ++h) {
    std::array<int32_t, 3> sh = {d->tile_shape[3 * h], d->tile_shape[3 * h + 1], d->tile_shape[3 * h + 2]};
    if (sh[0] < 1 || sh[1] < 1 || sh[2] < 1 || (int64_t)sh[0] * sh[1] * sh[2] != kTile) {
      delete p;
      return fail(VEDA_ERR_UNSUPPORTED, "head %d: tile shape (%d,%d,%d) does not hold 128 tokens", h,
                  sh[0], sh[1], sh[2]);
    }
    int idx = -1;
    for (int k = 0; k < (int)shape_list.size(); ++k)
      if (shape_list[k] == sh) idx = k;
    if (idx < 0) {
      if ((int)shape_list.size() == kMaxShapes) {
        delete p;
        return fail(VEDA_ERR_UNSUPPORTED, "more than %d distinct tile shapes in one layer", kMaxShapes);
      }
      shape_list.push_back(sh);
      idx = (int)shape_list.size() - 1;
    }
    p->head_shape[h] = idx;
  }

  for (auto& sh : shape_list) {
    HostShape hs;
    hs.a = sh[0];
    hs.b = sh[1];
    hs.c = sh[2];
    for (int s = 0; s < (int)p->segs.size(); ++s) {
      hs.seg_first.push_back((int32_t)hs.valid.size());
      tile_segment(p->segs[s], s, hs.a, hs.b, hs.c, hs);
      hs.seg_count.push_back((int32_t)hs.valid.size() - hs.seg_first.back());
      if ((int64_t)hs.valid.size() > kMaxTilesPerHead) {
        delete p;
        return fail(VEDA_ERR_UNSUPPORTED, "more than %d tiles per head", kMaxTilesPerHead);
      }
    }
    hs.num_tiles = (int32_t)hs.valid.size();
    build_budgets(*p, hs);
    p->shapes.push_back(std::move(hs));
  }

  // per-head offsets
  const int H = d->num_heads;
  p->head_row_off.resize(H);
  p->head_tile_off.resize(H);
  p->head_pair_off.resize(H);
  p->head_nnz_off.resize(H);
  int64_t rows = 0, tiles = 0, pairs = 0, nnz = 0, maxrow = 0;
  int32_t maxtiles = 0;
  for (int h = 0; h < H; ++h) {
    const HostShape& hs = p->shapes[p->head_shape[h]];
    p->head_row_off[h] = rows;
    p->head_tile_off[h] = (int32_t)tiles;
    p->head_pair_off[h] = pairs;
    p->head_nnz_off[h] = nnz;
    rows += (int64_t)kTile * hs.num_tiles;
    tiles += hs.num_tiles;
    pairs += (int64_t)hs.num_tiles * hs.num_tiles;
    nnz += hs.nnz;
    maxrow = std::max<int64_t>(maxrow, hs.max_row);
    maxtiles = std::max(maxtiles, hs.num_tiles);
  }
  if (nnz >= (int64_t(1) << 31) || tiles >= (int64_t(1) << 31)) {
    delete p;
    return fail(VEDA_ERR_UNSUPPORTED, "block count %lld does not fit int32 CSR", (long long)nnz);
  }
  p->row_head.resize(tiles);
  p->row_ptr.resize(tiles + 1);
  for (int h = 0; h < H; ++h) {
    const HostShape& hs = p->shapes[p->head_shape[h]];
    for (int i = 0; i < hs.num_tiles; ++i) {
      const int64_t t = p->head_tile_off[h] + i;
      p->row_head[t] = h;
      p->row_ptr[t] = (int32_t)(p->head_nnz_off[h] + hs.local_row_ptr[i]);
    }
  }
  p->row_ptr[tiles] = (int32_t)nnz;

  veda_plan_info& in = p->info;
  in.num_tokens = next;
  in.num_heads = H;
  in.head_dim = d->head_dim;
  in.num_segments = d->num_segments;
  in.num_shapes = (int32_t)p->shapes.size();
  in.total_rows = rows;
  in.total_tiles = tiles;
  in.total_pairs = pairs;
  in.nnz = nnz;
  in.max_row_blocks = maxrow;
  in.max_tiles_per_head = maxtiles;
  in.score_workspace_bytes = score_workspace_bytes(tiles, d->head_dim);
  in.transpose_workspace_bytes = transpose_workspace_bytes(in.total_pairs, in.total_tiles);
  in.bwd_workspace_bytes = bwd_workspace_bytes(in.total_rows, in.total_tiles, in.nnz);
  in.heat_workspace_bytes = heat_workspace_bytes(in.nnz, in.total_tiles, in.total_rows);
  in.reduce_workspace_bytes = reduce_workspace_bytes(H, maxtiles);
  build_attn_order(*p);
  build_staging(*p);
  in.device_table_bytes = (int64_t)p->staging.size();
  in.uploaded = 0;
  *out = p;
  return ok();
}

void veda_plan_destroy(veda_plan* plan) { delete plan; }

veda_status veda_plan_query(const veda_plan* p, veda_plan_info* info) {
  if (!p || !info) return fail(VEDA_ERR_INVALID_ARG, "plan or info is NULL");
  *info = p->info;
  return ok();
}

veda_status veda_plan_head(const veda_plan* p, int32_t head, int32_t* num_tiles, int64_t* row_offset,
                           int64_t* tile_offset, int64_t* pair_offset) {
  if (!p) return fail(VEDA_ERR_INVALID_ARG, "plan is NULL");
  if (head < 0 || head >= p->info.num_heads) return fail(VEDA_ERR_SHAPE, "head %d out of range", head);
  if (num_tiles) *num_tiles = p->shapes[p->head_shape[head]].num_tiles;
  if (row_offset) *row_offset = p->head_row_off[head];
  if (tile_offset) *tile_offset = p->head_tile_off[head];
  if (pair_offset) *pair_offset = p->head_pair_off[head];
  return ok();
}

static veda_status copy_out(const std::vector<int32_t>& v, int32_t* out, int64_t n, const char* what) {
  if (!out) return fail(VEDA_ERR_INVALID_ARG, "out is NULL");
  if (n != (int64_t)v.size())
    return fail(VEDA_ERR_SHAPE, "%s has %lld entries, caller gave %lld", what, (long long)v.size(), (long long)n);
  std::memcpy(out, v.data(), v.size() * sizeof(int32_t));
  return ok();
}

veda_status veda_plan_copy_perm(const veda_plan* p, int32_t head, int32_t* out, int64_t n) {
  if (!p) return fail(VEDA_ERR_INVALID_ARG, "plan is NULL");
  if (head < 0 || head >= p->info.num_heads) return fail(VEDA_ERR_SHAPE, "head %d out of range", head);
  return copy_out(p->shapes[p->head_shape[head]].perm, out, n, "perm");
}

veda_status veda_plan_copy_valid(const veda_plan* p, int32_t head, int32_t* out, int64_t n) {
  if (!p) return fail(VEDA_ERR_INVALID_ARG, "plan is NULL");
  if (head < 0 || head >= p->info.num_heads) return fail(VEDA_ERR_SHAPE, "head %d out of range", head);
  return copy_out(p->shapes[p->head_shape[head]].valid, out, n, "valid");
}

veda_status veda_plan_copy_budgets(const veda_plan* p, int32_t head, int32_t* out, int64_t n) {
  if (!p) return fail(VEDA_ERR_INVALID_ARG, "plan is NULL");
  if (head < 0 || head >= p->info.num_heads) return fail(VEDA_ERR_SHAPE, "head %d out of range", head);
  return copy_out(p->shapes[p->head_shape[head]].budget, out, n, "budgets");
}

veda_status veda_plan_copy_row_ptr(const veda_plan* p, int32_t* out, int64_t n) {
  if (!p) return fail(VEDA_ERR_INVALID_ARG, "plan is NULL");
  return copy_out(p->row_ptr, out, n, "row_ptr");
}

veda_status veda_plan_upload(veda_plan* p, void* dev_tables, size_t bytes, void* stream) {
  if (!p) return fail(VEDA_ERR_INVALID_ARG, "plan is NULL");
  if (!dev_tables) return fail(VEDA_ERR_INVALID_ARG, "dev_tables is NULL");
  if ((reinterpret_cast<uintptr_t>(dev_tables) & 255) != 0)
    return fail(VEDA_ERR_INVALID_ARG, "dev_tables is not 256-byte aligned");
  if ((int64_t)bytes < p->info.device_table_bytes)
    return fail(VEDA_ERR_WORKSPACE, "dev_tables holds %zu bytes, plan needs %lld", bytes,
                (long long)p->info.device_table_bytes);
  if (p->info.uploaded) return fail(VEDA_ERR_STATE, "plan already uploaded");
  veda_status st = check_device(nullptr);
  if (st != VEDA_OK) return st;
  int dev = -1;
  (void)hipGetDevice(&dev);
  hipError_t e = hipMemcpyAsync(dev_tables, p->staging.data(), p->staging.size(), hipMemcpyHostToDevice,
                                (hipStream_t)stream);
  if (e != hipSuccess) return fail(VEDA_ERR_LAUNCH, "plan upload: %s", hipGetErrorString(e));
  // The staging image is pageable host memory owned by the plan; wait for the
  // copy so the caller may use the tables from any stream right away.
  e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(VEDA_ERR_LAUNCH, "plan upload: %s", hipGetErrorString(e));
  bind_device(*p, (uint8_t*)dev_tables);
  p->device = dev;
  p->info.uploaded = 1;
  return ok();
}

veda_status veda_permute_tiles(const veda_plan* p, const void* src, void* dst, int32_t direction,
                               void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(src, "src")) || (st = check_ptr(dst, "dst"))) return st;
  if (direction != VEDA_PERMUTE_FORWARD && direction != VEDA_PERMUTE_INVERSE &&
      direction != VEDA_PERMUTE_FORWARD_TRANSPOSED)
    return fail(VEDA_ERR_INVALID_ARG, "unknown direction %d", direction);
  if (src == dst) return fail(VEDA_ERR_INVALID_ARG, "src and dst alias");
  return launched(launch_permute(p->dev, src, dst, direction, (hipStream_t)stream), "permute");
}

veda_status veda_score_tiles(const veda_plan* p, const void* q_perm, const void* k_perm, const float* w_q,
                             const float* w_k, float* scores, void* workspace, size_t workspace_bytes,
                             void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(q_perm, "q_perm")) || (st = check_ptr(k_perm, "k_perm")) ||
      (st = check_ptr(w_q, "w_q")) || (st = check_ptr(w_k, "w_k")) || (st = check_ptr(scores, "scores")))
    return st;
  if (!workspace) return fail(VEDA_ERR_WORKSPACE, "workspace is NULL");
  if ((st = check_ptr(workspace, "workspace"))) return st;
  if ((int64_t)workspace_bytes < p->info.score_workspace_bytes)
    return fail(VEDA_ERR_WORKSPACE, "workspace holds %zu bytes, %lld needed", workspace_bytes,
                (long long)p->info.score_workspace_bytes);
  return launched(launch_score(p->dev, q_perm, k_perm, w_q, w_k, scores, workspace, (hipStream_t)stream),
                  "score");
}

veda_status veda_score_tiles_noalloc(const veda_plan* p, const void* q_perm, const void* k_perm,
                                     const float* w_q, const float* w_k, float* scores, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(q_perm, "q_perm")) || (st = check_ptr(k_perm, "k_perm")) ||
      (st = check_ptr(w_q, "w_q")) || (st = check_ptr(w_k, "w_k")) || (st = check_ptr(scores, "scores")))
    return st;
  if (p->info.score_workspace_bytes > kStaticScratchBytes)
    return fail(VEDA_ERR_WORKSPACE,
                "the plan's predictor needs %lld bytes of scratch; the static scratch holds %lld "
                "(T * head_dim * 32 bytes: at most %lld tiles at head dim %d); use veda_score_tiles "
                "with a workspace",
                (long long)p->info.score_workspace_bytes, (long long)kStaticScratchBytes,
                (long long)(kStaticScratchBytes / (32LL * p->info.head_dim)), p->info.head_dim);
  void* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess)
    return fail(VEDA_ERR_LAUNCH, "static scratch address on the current device: %s", hipGetErrorString(e));
  return launched(launch_score(p->dev, q_perm, k_perm, w_q, w_k, scores, ws, (hipStream_t)stream),
                  "score (static scratch)");
}

veda_status veda_permute_qkv(const veda_plan* p, const void* q, const void* k, const void* v, void* q_perm,
                             void* k_perm, void* v_t, void* workspace, size_t workspace_bytes, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(k_perm, "k_perm")))
    return st;
  if (q_perm && (st = check_ptr(q_perm, "q_perm"))) return st;
  if (!q_perm && !workspace)
    return fail(VEDA_ERR_INVALID_ARG, "q_perm may be NULL only with a workspace (Q pooled, not written)");
  if ((v == nullptr) != (v_t == nullptr)) return fail(VEDA_ERR_INVALID_ARG, "v and v_t must both be given or both NULL");
  if (v && ((st = check_ptr(v, "v")) || (st = check_ptr(v_t, "v_t")))) return st;
  const int nt = v ? 3 : 2;   // without V: Q and K only
  const void* ins[3] = {q, k, v};
  void* outs[3] = {q_perm, k_perm, v_t};
  for (int a = 0; a < nt; ++a)
    for (int b = 0; b < nt; ++b)
      if (outs[b] && ins[a] == outs[b]) return fail(VEDA_ERR_INVALID_ARG, "an input aliases an output");
  if (workspace) {
    if ((st = check_ptr(workspace, "workspace"))) return st;
    if ((int64_t)workspace_bytes < p->info.score_workspace_bytes)
      return fail(VEDA_ERR_WORKSPACE, "workspace holds %zu bytes, %lld needed", workspace_bytes,
                  (long long)p->info.score_workspace_bytes);
  }
  return launched(launch_permute_qkv(p->dev, q, k, v, q_perm, k_perm, v_t, workspace, (hipStream_t)stream),
                  "permute qkv");
}

veda_status veda_score_pooled(const veda_plan* p, const float* w_q, const float* w_k, float* scores,
                              void* workspace, size_t workspace_bytes, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(w_q, "w_q")) || (st = check_ptr(w_k, "w_k")) || (st = check_ptr(scores, "scores")))
    return st;
  if (!workspace) return fail(VEDA_ERR_WORKSPACE, "workspace is NULL");
  if ((st = check_ptr(workspace, "workspace"))) return st;
  if ((int64_t)workspace_bytes < p->info.score_workspace_bytes)
    return fail(VEDA_ERR_WORKSPACE, "workspace holds %zu bytes, %lld needed", workspace_bytes,
                (long long)p->info.score_workspace_bytes);
  return launched(launch_score_pooled(p->dev, w_q, w_k, scores, workspace, (hipStream_t)stream), "score pooled");
}

veda_status veda_select_blocks(const veda_plan* p, const float* scores, int32_t* row_ptr, int32_t* col_idx,
                               uint8_t* dense_mask, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(scores, "scores")) || (st = check_ptr(row_ptr, "row_ptr")) ||
      (st = check_ptr(col_idx, "col_idx")))
    return st;
  if (dense_mask && (st = check_ptr(dense_mask, "dense_mask"))) return st;
  return launched(launch_select(p->dev, scores, row_ptr, col_idx, dense_mask, (hipStream_t)stream), "select");
}

veda_status veda_block_sparse_attn_fwd(const veda_plan* p, const void* q, int32_t q_layout, const void* k,
                                       const void* v_t,
                                       const int32_t* row_ptr, const int32_t* col_idx, float softmax_scale,
                                       void* o, int32_t o_layout, float* lse, uint32_t* blocks_visited,
                                       void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v_t, "v_t")) ||
      (st = check_ptr(row_ptr, "row_ptr")) || (st = check_ptr(col_idx, "col_idx")))
    return st;
  if (o && (st = check_ptr(o, "o"))) return st;
  if (lse && (st = check_ptr(lse, "lse"))) return st;
  if (!o && !lse) return fail(VEDA_ERR_INVALID_ARG, "o and lse are both NULL: nothing to compute");
  if (blocks_visited && (reinterpret_cast<uintptr_t>(blocks_visited) & 3))
    return fail(VEDA_ERR_INVALID_ARG, "blocks_visited is not 4-byte aligned");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(VEDA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (o_layout != VEDA_LAYOUT_PERMUTED && o_layout != VEDA_LAYOUT_NATURAL)
    return fail(VEDA_ERR_INVALID_ARG, "unknown o_layout %d", o_layout);
  if (q_layout != VEDA_LAYOUT_PERMUTED && q_layout != VEDA_LAYOUT_NATURAL)
    return fail(VEDA_ERR_INVALID_ARG, "unknown q_layout %d", q_layout);
  if (o && (o == q || o == k || o == v_t)) return fail(VEDA_ERR_INVALID_ARG, "o aliases an input");
  return launched(launch_attn_fwd(p->dev, q, q_layout == VEDA_LAYOUT_NATURAL, k, v_t, row_ptr, col_idx,
                                  softmax_scale, o, o_layout == VEDA_LAYOUT_NATURAL, lse, blocks_visited,
                                  (hipStream_t)stream),
                  "block-sparse attention");
}

veda_status veda_block_heat(const veda_plan* p, const void* q, const void* k, const float* lse,
                            float softmax_scale, float* heat, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(lse, "lse")) ||
      (st = check_ptr(heat, "heat")))
    return st;
  if (p->info.max_tiles_per_head > kMaxHeatTiles)
    return fail(VEDA_ERR_UNSUPPORTED, "block heat supports at most %d tiles per head", kMaxHeatTiles);
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(VEDA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  return launched(launch_heat(p->dev, q, k, lse, softmax_scale, heat, (hipStream_t)stream), "block heat");
}

veda_status veda_dense_lse_heat(const veda_plan* p, const void* q, int32_t q_layout, const void* k,
                                const int32_t* row_ptr, const int32_t* col_idx, float softmax_scale, float* lse,
                                float* heat, void* workspace, size_t workspace_bytes, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(row_ptr, "row_ptr")) ||
      (st = check_ptr(col_idx, "col_idx")) || (st = check_ptr(heat, "heat")) ||
      (st = check_ptr(workspace, "workspace")))
    return st;
  if (lse && (st = check_ptr(lse, "lse"))) return st;
  if (p->budget_mode != VEDA_BUDGET_ALL)
    return fail(VEDA_ERR_UNSUPPORTED, "the fused dense LSE and heat needs a plan with budget mode ALL");
  if (heat == workspace || (lse && ((const void*)lse == workspace || lse == heat)) || heat == q || heat == k ||
      (lse && ((const void*)lse == q || (const void*)lse == k)))
    return fail(VEDA_ERR_INVALID_ARG, "lse, heat and workspace must be distinct from each other and the inputs");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(VEDA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (q_layout != VEDA_LAYOUT_PERMUTED && q_layout != VEDA_LAYOUT_NATURAL)
    return fail(VEDA_ERR_INVALID_ARG, "unknown q_layout %d", q_layout);
  if ((int64_t)workspace_bytes < p->info.heat_workspace_bytes)
    return fail(VEDA_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", workspace_bytes,
                (long long)p->info.heat_workspace_bytes);
  return launched(launch_lse_heat(p->dev, q, q_layout == VEDA_LAYOUT_NATURAL, k, row_ptr, col_idx, softmax_scale, lse,
                                  static_cast<float*>(workspace), heat, (hipStream_t)stream),
                  "dense LSE and heat");
}

namespace {
// Two plans tile the same sequence the same way: same segments, heads, head
// dimension and per-head tile shape (the tiling is a function of these).
bool same_geometry(const veda_plan* a, const veda_plan* b) {
  if (a->info.num_heads != b->info.num_heads || a->info.head_dim != b->info.head_dim ||
      a->info.num_tokens != b->info.num_tokens || a->segs.size() != b->segs.size())
    return false;
  for (size_t i = 0; i < a->segs.size(); ++i) {
    const veda_segment &x = a->segs[i], &y = b->segs[i];
    if (x.kind != y.kind || x.t != y.t || x.h != y.h || x.w != y.w || x.token_offset != y.token_offset) return false;
  }
  for (int32_t h = 0; h < a->info.num_heads; ++h) {
    const HostShape &x = a->shapes[a->head_shape[h]], &y = b->shapes[b->head_shape[h]];
    if (x.a != y.a || x.b != y.b || x.c != y.c) return false;
  }
  return true;
}
}  // namespace

veda_status veda_attn_fwd_lse_heat(const veda_plan* plan, const veda_plan* dense_plan, const void* q,
                                   int32_t q_layout, const void* k, const void* v_t, const int32_t* row_ptr,
                                   const int32_t* col_idx, const int32_t* dense_row_ptr,
                                   const int32_t* dense_col_idx, float softmax_scale, void* o, int32_t o_layout,
                                   float* lse, float* dense_lse, float* heat, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  veda_status st = check_plan_ready(plan);
  if (st) return st;
  if ((st = check_plan_ready(dense_plan))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v_t, "v_t")) ||
      (st = check_ptr(row_ptr, "row_ptr")) || (st = check_ptr(col_idx, "col_idx")) ||
      (st = check_ptr(dense_row_ptr, "dense_row_ptr")) || (st = check_ptr(dense_col_idx, "dense_col_idx")) ||
      (st = check_ptr(o, "o")) || (st = check_ptr(heat, "heat")) || (st = check_ptr(workspace, "workspace")))
    return st;
  if (lse && (st = check_ptr(lse, "lse"))) return st;
  if (dense_lse && (st = check_ptr(dense_lse, "dense_lse"))) return st;
  if (dense_plan->budget_mode != VEDA_BUDGET_ALL)
    return fail(VEDA_ERR_UNSUPPORTED, "dense_plan must have budget mode ALL");
  if (!same_geometry(plan, dense_plan))
    return fail(VEDA_ERR_SHAPE, "plan and dense_plan do not tile the same sequence the same way");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(VEDA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (o_layout != VEDA_LAYOUT_PERMUTED && o_layout != VEDA_LAYOUT_NATURAL)
    return fail(VEDA_ERR_INVALID_ARG, "unknown o_layout %d", o_layout);
  if (q_layout != VEDA_LAYOUT_PERMUTED && q_layout != VEDA_LAYOUT_NATURAL)
    return fail(VEDA_ERR_INVALID_ARG, "unknown q_layout %d", q_layout);
  const void* outs[5] = {o, heat, workspace, lse, dense_lse};
  const void* ins[3] = {q, k, v_t};
  for (int i = 0; i < 5; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 3; ++j)
      if (outs[i] == ins[j]) return fail(VEDA_ERR_INVALID_ARG, "an output aliases an input");
    for (int j = i + 1; j < 5; ++j)
      if (outs[i] == outs[j]) return fail(VEDA_ERR_INVALID_ARG, "o, heat, workspace, lse and dense_lse must be distinct");
  }
  if ((int64_t)workspace_bytes < dense_plan->info.heat_workspace_bytes)
    return fail(VEDA_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", workspace_bytes,
                (long long)dense_plan->info.heat_workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return fail(VEDA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  const int64_t sel_nnz = plan->info.nnz, dense_nnz = dense_plan->info.nnz;
  if (sel_nnz > dense_nnz)
    return fail(VEDA_ERR_SHAPE, "plan keeps %lld blocks, more than the dense plan's %lld", (long long)sel_nnz,
                (long long)dense_nnz);
  // layout: sums of the selected blocks | block sums of the rest | rest
  // columns | per-tile flags | per-row factors | the selected rows' LSE (if
  // lse is NULL)
  uint8_t* base = static_cast<uint8_t*>(workspace);
  SplitWorkspace ws{};
  ws.rest_nnz = dense_nnz - sel_nnz;
  int64_t off = 0;
  ws.mass = reinterpret_cast<float*>(base + off);
  off += align256(sel_nnz * 128 * 4);
  ws.rest_bsum = reinterpret_cast<float*>(base + off);
  off += align256(ws.rest_nnz * 128 * 4);
  ws.rest_col = reinterpret_cast<int32_t*>(base + off);
  off += align256(dense_nnz * 4);
  ws.cflag = reinterpret_cast<int32_t*>(base + off);
  off += align256(dense_plan->info.total_tiles * 4);
  ws.fac = reinterpret_cast<float2*>(base + off);
  off += align256(dense_plan->info.total_rows * 8);
  float* lse_sel = lse ? lse : reinterpret_cast<float*>(base + off);
  off += align256(dense_plan->info.total_rows * 4);
  if (off > dense_plan->info.heat_workspace_bytes)
    return fail(VEDA_ERR_WORKSPACE, "internal: workspace layout of %lld bytes exceeds %lld", (long long)off,
                (long long)dense_plan->info.heat_workspace_bytes);
  return launched(launch_attn_lse_heat(plan->dev, dense_plan->dev, q, q_layout == VEDA_LAYOUT_NATURAL, k, v_t,
                                       row_ptr, col_idx, dense_row_ptr, dense_col_idx, softmax_scale, o,
                                       o_layout == VEDA_LAYOUT_NATURAL, lse_sel, dense_lse, heat, ws,
                                       (hipStream_t)stream),
                  "attention with the dense LSE and heat");
}

namespace {
veda_status check_reduce_ws(const veda_plan* p, void* workspace, size_t workspace_bytes) {
  veda_status st = check_ptr(workspace, "workspace");
  if (st) return st;
  if ((int64_t)workspace_bytes < p->info.reduce_workspace_bytes)
    return fail(VEDA_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", workspace_bytes,
                (long long)p->info.reduce_workspace_bytes);
  return ok();
}
}  // namespace

veda_status veda_mask_mass(const veda_plan* p, const float* heat, const int32_t* row_ptr, const int32_t* col_idx,
                           double* mass, void* workspace, size_t workspace_bytes, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(heat, "heat")) || (st = check_ptr(row_ptr, "row_ptr")) ||
      (st = check_ptr(col_idx, "col_idx")) || (st = check_ptr(mass, "mass")) ||
      (st = check_reduce_ws(p, workspace, workspace_bytes)))
    return st;
  return launched(launch_mask_mass(p->dev, p->info.max_tiles_per_head, heat, row_ptr, col_idx, mass, workspace,
                                   (hipStream_t)stream),
                  "mask mass");
}

veda_status veda_output_error(const veda_plan* p, const void* o, const void* o_ref, double* err, void* workspace,
                              size_t workspace_bytes, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(o, "o")) || (st = check_ptr(o_ref, "o_ref")) || (st = check_ptr(err, "err")) ||
      (st = check_reduce_ws(p, workspace, workspace_bytes)))
    return st;
  return launched(launch_output_error(p->dev, p->info.num_tokens, o, o_ref, err, workspace, (hipStream_t)stream),
                  "output error");
}

veda_status veda_mask_transpose(const veda_plan* p, const int32_t* row_ptr, const int32_t* col_idx, int32_t* col_ptr,
                                int32_t* row_idx, void* workspace, size_t workspace_bytes, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(row_ptr, "row_ptr")) || (st = check_ptr(col_idx, "col_idx")) ||
      (st = check_ptr(col_ptr, "col_ptr")) || (st = check_ptr(row_idx, "row_idx")) ||
      (st = check_ptr(workspace, "workspace")))
    return st;
  if ((int64_t)workspace_bytes < p->info.transpose_workspace_bytes)
    return fail(VEDA_ERR_WORKSPACE, "mask transpose needs %lld workspace bytes",
                (long long)p->info.transpose_workspace_bytes);
  return launched(launch_mask_transpose(p->dev, row_ptr, col_idx, col_ptr, row_idx, workspace,
                                        p->info.total_pairs, (hipStream_t)stream),
                  "mask transpose");
}

veda_status veda_block_sparse_attn_bwd(const veda_plan* p, const void* q, const void* k, const void* v,
                                       const void* o, const void* d_o, const float* lse, const int32_t* row_ptr,
                                       const int32_t* col_idx, const int32_t* col_ptr, const int32_t* row_idx,
                                       float softmax_scale, void* dq, void* dk, void* dv, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  veda_status st = check_plan_ready(p);
  if (st) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(o, "o")) ||
      (st = check_ptr(d_o, "d_o")) || (st = check_ptr(lse, "lse")) || (st = check_ptr(row_ptr, "row_ptr")) ||
      (st = check_ptr(col_idx, "col_idx")) || (st = check_ptr(col_ptr, "col_ptr")) ||
      (st = check_ptr(row_idx, "row_idx")) || (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) ||
      (st = check_ptr(dv, "dv")) || (st = check_ptr(workspace, "workspace")))
    return st;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(VEDA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  {
    const void* ins[7] = {q, k, v, o, d_o, lse, workspace};
    const void* outs[3] = {dq, dk, dv};
    for (int a = 0; a < 3; ++a) {
      for (int b = 0; b < 7; ++b)
        if (outs[a] == ins[b]) return fail(VEDA_ERR_INVALID_ARG, "dq, dk or dv aliases an input or the workspace");
      for (int b = a + 1; b < 3; ++b)
        if (outs[a] == outs[b]) return fail(VEDA_ERR_INVALID_ARG, "dq, dk and dv must be distinct buffers");
    }
  }
  if ((int64_t)workspace_bytes < p->info.bwd_workspace_bytes)
    return fail(VEDA_ERR_WORKSPACE, "backward needs %lld workspace bytes", (long long)p->info.bwd_workspace_bytes);
  return launched(launch_attn_bwd(p->dev, q, k, v, o, d_o, lse, row_ptr, col_idx, col_ptr, row_idx, softmax_scale, dq,
                                  dk, dv, workspace, (hipStream_t)stream),
                  "attention backward");
}

veda_status veda_tile_plan_vote(int32_t samples, int32_t candidates, int32_t heads, const double* err,
                                int32_t max_shapes, int32_t* choice) {
  if (samples <= 0 || candidates <= 0 || heads <= 0 || max_shapes <= 0)
    return fail(VEDA_ERR_INVALID_ARG, "tile plan vote: counts must be positive");
  if (!err || !choice) return fail(VEDA_ERR_INVALID_ARG, "tile plan vote: null pointer");
  const int64_t S = samples, C = candidates, H = heads;
  for (int64_t e = 0; e < S * C * H; ++e)
    if (!std::isfinite(err[e])) return fail(VEDA_ERR_INVALID_ARG, "tile plan vote: non-finite error");
  auto at = [&](int64_t s, int64_t c, int64_t h) { return err[(s * C + c) * H + h]; };
  // 1-2: per sample and head the lowest-error candidate; per head the most voted
  std::vector<int32_t> pref(H);
  for (int64_t h = 0; h < H; ++h) {
    std::vector<int64_t> votes(C, 0);
    for (int64_t s = 0; s < S; ++s) {
      int64_t best = 0;
      for (int64_t c = 1; c < C; ++c)
        if (at(s, c, h) < at(s, best, h)) best = c;
      ++votes[best];
    }
    int64_t top = 0;
    for (int64_t c = 1; c < C; ++c)
      if (votes[c] > votes[top]) top = c;
    pref[h] = (int32_t)top;
  }
  // 3: the max_shapes candidates preferred by the most heads
  std::vector<int64_t> heads_for(C, 0);
  for (int64_t h = 0; h < H; ++h) ++heads_for[pref[h]];
  std::vector<int32_t> order(C);
  for (int64_t c = 0; c < C; ++c) order[c] = (int32_t)c;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return heads_for[a] > heads_for[b]; });
  std::vector<int32_t> kept;
  for (int64_t r = 0; r < C && (int64_t)kept.size() < max_shapes; ++r)
    if (heads_for[order[r]] > 0) kept.push_back(order[r]);
  // 4: preferred if kept, else the kept candidate with the lowest mean error
  for (int64_t h = 0; h < H; ++h) {
    if (std::find(kept.begin(), kept.end(), pref[h]) != kept.end()) {
      choice[h] = pref[h];
      continue;
    }
    int32_t best = -1;
    double best_mean = 0.0;
    for (int32_t c : kept) {
      double m = 0.0;
      for (int64_t s = 0; s < S; ++s) m += at(s, c, h);
      m /= (double)S;
      if (best < 0 || m < best_mean || (m == best_mean && c < best)) {
        best = c;
        best_mean = m;
      }
    }
    choice[h] = best;
  }
  return VEDA_OK;
}

}  // extern "C"
