// Host side of the C ABI declared in include/vdsa.h: argument checks (all of
// them before anything is enqueued), kernel parameter setup and dispatch,
// effective-work counters and error strings.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>

#include "internal.h"
#include "vdsa.h"

namespace vdsa {
int box_attn_bf16_block_m();
int box_attn_bf16_pp_block_m();
int box_attn_f32_block_m();
}  // namespace vdsa

namespace {

thread_local std::string g_last_error;

vdsa_status fail(vdsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

vdsa_status ok() {
  g_last_error.clear();
  return VDSA_OK;
}

size_t elem_size(vdsa_dtype t) { return t == VDSA_BF16 ? 2 : 4; }

vdsa_status check_problem(const vdsa_problem* p) {
  if (!p) return fail(VDSA_ERR_NULL, "problem descriptor is NULL");
  if (p->batch <= 0 || p->heads <= 0 || p->grid_t <= 0 || p->grid_h <= 0 || p->grid_w <= 0)
    return fail(VDSA_ERR_SHAPE, "batch, heads and grid dims must be > 0 (got batch=%d heads=%d grid=%dx%dx%d)",
                p->batch, p->heads, p->grid_t, p->grid_h, p->grid_w);
  if (p->dtype != VDSA_F32 && p->dtype != VDSA_BF16)
    return fail(VDSA_ERR_UNSUPPORTED, "dtype %d is not VDSA_F32 or VDSA_BF16", (int)p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(VDSA_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", p->head_dim);
  if (!std::isfinite(p->scale) || p->scale < 0.f)
    return fail(VDSA_ERR_UNSUPPORTED, "scale must be finite and >= 0 (got %g)", (double)p->scale);
  const int64_t n = (int64_t)p->grid_t * p->grid_h * p->grid_w;
  if (n >= (int64_t(1) << 31)) return fail(VDSA_ERR_SHAPE, "N = %lld tokens is too large", (long long)n);
  return VDSA_OK;
}

int64_t n_tokens(const vdsa_problem* p) { return (int64_t)p->grid_t * p->grid_h * p->grid_w; }

// A [batch, heads, rows, head_dim] view: checks and its byte range.
struct View {
  const char* name;
  const void* ptr;
  const vdsa_strides* st;
  int64_t rows;
  uintptr_t lo = 0, hi = 0;  // byte range [lo, hi)
};

vdsa_status check_view(const vdsa_problem* p, View& v, bool is_output) {
  if (!v.ptr) return fail(VDSA_ERR_NULL, "%s pointer is NULL", v.name);
  if (!v.st) return fail(VDSA_ERR_NULL, "%s strides pointer is NULL", v.name);
  const size_t es = elem_size(p->dtype);
  const int64_t ext[3] = {p->batch, p->heads, v.rows};
  const int64_t str[3] = {v.st->b, v.st->h, v.st->n};
  const char* nm[3] = {"batch", "head", "token"};
  if ((uintptr_t)v.ptr % 16 != 0) return fail(VDSA_ERR_ALIGN, "%s pointer is not 16-byte aligned", v.name);
  int64_t max_off = p->head_dim;
  for (int d = 0; d < 3; ++d) {
    if (ext[d] == 1) continue;  // the stride of an extent-1 dim is never used
    if (str[d] <= 0) return fail(VDSA_ERR_SHAPE, "%s %s stride must be > 0 (got %lld)", v.name, nm[d], (long long)str[d]);
    if ((str[d] * (int64_t)es) % 16 != 0)
      return fail(VDSA_ERR_ALIGN, "%s %s stride %lld x %zu bytes is not a multiple of 16", v.name, nm[d],
                  (long long)str[d], es);
    max_off += (ext[d] - 1) * str[d];
  }
  // kernels address one (batch, head) slice with 32-bit byte offsets
  const int64_t row_span = ((v.rows - 1) * (v.rows > 1 ? str[2] : 0) + p->head_dim) * (int64_t)es;
  if (row_span >= (int64_t(1) << 32))
    return fail(VDSA_ERR_SHAPE, "%s: token offsets within one head reach %lld bytes (limit 2^32)", v.name,
                (long long)row_span);
  if (is_output) {
    // rows of the output must not overlap each other: sort the used dims by
    // stride; each stride must cover the span of all smaller ones.
    std::pair<int64_t, int64_t> dims[3];  // (stride, extent)
    int nd = 0;
    for (int d = 0; d < 3; ++d)
      if (ext[d] > 1) dims[nd++] = {str[d], ext[d]};
    std::sort(dims, dims + nd);
    int64_t span = p->head_dim;
    for (int i = 0; i < nd; ++i) {
      if (dims[i].first < span) return fail(VDSA_ERR_ALIAS, "%s: strides make output rows overlap each other", v.name);
      span = dims[i].first * (dims[i].second - 1) + span;
    }
  }
  v.lo = (uintptr_t)v.ptr;
  v.hi = v.lo + (uintptr_t)(max_off * (int64_t)es);
  return VDSA_OK;
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

vdsa_status check_sta_cfg(const vdsa_sta_cfg* c) {
  if (!c) return fail(VDSA_ERR_NULL, "sta config is NULL");
  const char* nm[3] = {"t", "h", "w"};
  for (int d = 0; d < 3; ++d) {
    if (c->tile[d] < 1) return fail(VDSA_ERR_WINDOW, "tile[%s] = %d must be >= 1", nm[d], c->tile[d]);
    if (c->window[d] < 1 || c->window[d] % 2 == 0)
      return fail(VDSA_ERR_WINDOW, "window[%s] = %d must be odd and >= 1", nm[d], c->window[d]);
    if (c->shift[d] < 0 || c->shift[d] >= c->tile[d])
      return fail(VDSA_ERR_WINDOW, "shift[%s] = %d must be in [0, tile = %d)", nm[d], c->shift[d], c->tile[d]);
  }
  if (c->window_mode != VDSA_WINDOW_CLIP && c->window_mode != VDSA_WINDOW_INWARD &&
      c->window_mode != VDSA_WINDOW_CYCLIC)
    return fail(VDSA_ERR_WINDOW, "window_mode = %d is not a vdsa_window_mode", c->window_mode);
  return VDSA_OK;
}

int tiles_along(int L, int b, int s) { return (L + s + b - 1) / b; }

// Lattice offset the kernels tile with: the cyclic mode tiles the rolled
// grid from 0 and carries the shift as the roll instead.
int lattice_shift(const vdsa_sta_cfg* c, int d) { return c->window_mode == VDSA_WINDOW_CYCLIC ? 0 : c->shift[d]; }

// Sliding-tile geometry of cfg on the token grid: query tiles, window radii,
// the window mode and, for the cyclic mode, the roll; keys on the same grid.
void set_sta_geometry(vdsa::BoxAttnParams& g, const vdsa_problem* prob, const vdsa_sta_cfg* cfg) {
  g.qT = prob->grid_t; g.qH = prob->grid_h; g.qW = prob->grid_w;
  g.bT = cfg->tile[0]; g.bH = cfg->tile[1]; g.bW = cfg->tile[2];
  g.sT = lattice_shift(cfg, 0); g.sH = lattice_shift(cfg, 1); g.sW = lattice_shift(cfg, 2);
  g.nT = tiles_along(g.qT, g.bT, g.sT);
  g.nH = tiles_along(g.qH, g.bH, g.sH);
  g.nW = tiles_along(g.qW, g.bW, g.sW);
  g.rT = (cfg->window[0] - 1) / 2; g.rH = (cfg->window[1] - 1) / 2; g.rW = (cfg->window[2] - 1) / 2;
  g.kT = g.qT; g.kH = g.qH; g.kW = g.qW;
  g.dense_keys = 0;
  g.wmode = cfg->window_mode == VDSA_WINDOW_INWARD ? vdsa::WIN_INWARD : vdsa::WIN_CLIP;
  const bool cyc = cfg->window_mode == VDSA_WINDOW_CYCLIC;
  // a roll by s is a roll by s mod L (s may exceed L when the tile does)
  g.rlT = cyc ? cfg->shift[0] % g.qT : 0;
  g.rlH = cyc ? cfg->shift[1] % g.qH : 0;
  g.rlW = cyc ? cfg->shift[2] % g.qW : 0;
}

// Largest number of real tokens in one tile along a dim.
int max_tile_extent(int L, int b, int s) {
  const int n = tiles_along(L, b, s);
  int best = 0;
  // interior tiles have b tokens; only the first and last can be partial
  for (int i : {0, 1, n - 2, n - 1}) {
    if (i < 0 || i >= n) continue;
    const int lo = std::max(0, i * b - s), hi = std::min(L, (i + 1) * b - s);
    best = std::max(best, hi - lo);
  }
  return best;
}

// bf16 kernel shapes: queries per workgroup and the kernel that runs them.
enum Bf16Kernel { K_M32 = 0, K_M16_4W = 1, K_PP_8W = 2 };
struct Bf16Shape {
  int block_m;
  Bf16Kernel kernel;
};

// Largest block whose padding wastes at most 1/8 of the launched query slots,
// else the least padding.  The 384- and 192-query kernels (head_dim 128 only)
// map keys to tokens with 24-bit multiplies; the offset check makes that exact,
// since ((N-1)*stride_n + 128) * 2 < 2^32 with stride_n >= 128 gives N < 2^24.
Bf16Shape choose_bf16_shape(int64_t max_tile_vol, int head_dim) {
  const Bf16Shape m32{vdsa::box_attn_bf16_block_m(), K_M32};
  if (head_dim != 128) return m32;
  const Bf16Shape shapes[] = {{vdsa::box_attn_bf16_pp_block_m(), K_PP_8W}, {192, K_M16_4W}, m32};
  Bf16Shape best = m32;
  double best_waste = 2.0;
  for (const Bf16Shape& sh : shapes) {
    const int64_t blocks = (max_tile_vol + sh.block_m - 1) / sh.block_m;
    const double waste = (double)(blocks * sh.block_m - max_tile_vol) / (double)(blocks * sh.block_m);
    if (waste <= 0.125) return sh;
    if (waste < best_waste) {
      best_waste = waste;
      best = sh;
    }
  }
  return best;
}

// Largest number of real tokens in one query tile of bp's lattice.
int64_t max_tile_volume(const vdsa::BoxAttnParams& bp) {
  return (int64_t)max_tile_extent(bp.qT, bp.bT, bp.sT) * max_tile_extent(bp.qH, bp.bH, bp.sH) *
         max_tile_extent(bp.qW, bp.bW, bp.sW);
}

// Key walk of the 384- and 192-query kernels: dense keys in token order (the
// 384-query kernel only); tile by tile when every tile of the lattice is full
// (no lattice shift, grid dims multiples of the tile) and a tile frame holds
// exactly one 64-key block (tile h x w = 64), on the rolled grid for the
// cyclic mode; else the raster walk over the key box.
int tile_walk_mode(const vdsa::BoxAttnParams& bp) {
  if (bp.dense_keys) return (bp.rlT | bp.rlH | bp.rlW) ? 0 : 3;
  if (bp.kpT > 1 || bp.kpH > 1 || bp.kpW > 1) return 0;
  if (bp.sT || bp.sH || bp.sW || bp.bH * bp.bW != 64) return 0;
  if (bp.qT % bp.bT || bp.qH % bp.bH || bp.qW % bp.bW) return 0;
  if (bp.kT != bp.qT || bp.kH != bp.qH || bp.kW != bp.qW) return 0;
  return (bp.rlT | bp.rlH | bp.rlW) ? 2 : 1;
}

// Name of the kernel launch_attn runs for bp (the same choice, no launch).
const char* attn_kernel_name(const vdsa_problem* prob, const vdsa::BoxAttnParams& bp) {
  const bool d128 = prob->head_dim == 128;
  if (prob->dtype == VDSA_F32) return d128 ? "box_attn_f32_kernel<128>" : "box_attn_f32_kernel<64>";
  static const char* const pp_names[4] = {"box_attn_bf16_pp_kernel<0>", "box_attn_bf16_pp_kernel<1>",
                                          "box_attn_bf16_pp_kernel<2>", "box_attn_bf16_pp_kernel<3>"};
  switch (choose_bf16_shape(max_tile_volume(bp), prob->head_dim).kernel) {
    case K_PP_8W: return pp_names[tile_walk_mode(bp)];
    case K_M16_4W: {
      if (tile_walk_mode(bp) != 1) return "box_attn_bf16_m16_kernel<4, 0>";
      // one query block per tile and two or more tiles along w: tile pairs
      const int64_t qblocks = (max_tile_volume(bp) + 191) / 192;
      return qblocks == 1 && bp.nW >= 2 ? "box_attn_bf16_m16_kernel<8, 1, true>" : "box_attn_bf16_m16_kernel<4, 1>";
    }
    default: return d128 ? "box_attn_bf16_kernel<128>" : "box_attn_bf16_kernel<64>";
  }
}

vdsa_status launch_attn(const vdsa_problem* prob, vdsa::BoxAttnParams& bp, hipStream_t stream) {
  const int64_t mv = max_tile_volume(bp);
  Bf16Shape shape{vdsa::box_attn_f32_block_m(), K_M32};
  if (prob->dtype == VDSA_BF16) shape = choose_bf16_shape(mv, prob->head_dim);
  bp.qblocks = (int32_t)((mv + shape.block_m - 1) / shape.block_m);
  bp.variant = (int32_t)shape.kernel;
  // (the 192-query kernel has no rolled tile walk: the cyclic mode stays raster)
  bp.tile_walk = prob->dtype != VDSA_BF16                                   ? 0
                 : shape.kernel == K_PP_8W                                  ? tile_walk_mode(bp)
                 : shape.kernel == K_M16_4W && tile_walk_mode(bp) == 1      ? 1
                                                                            : 0;
  const int64_t total = (int64_t)bp.batch * bp.heads * bp.nT * bp.nH * bp.nW * bp.qblocks;
  if (total >= (int64_t(1) << 31) / 512)
    return fail(VDSA_ERR_SHAPE, "problem needs %lld workgroups, beyond the launch limit", (long long)total);
  bp.total_wg = (int32_t)total;
  bp.scale_log2e = prob->scale * 1.4426950408889634f;
  bp.fd_qblocks = vdsa::make_fastdiv((uint32_t)bp.qblocks);
  bp.fd_tiles = vdsa::make_fastdiv((uint32_t)(bp.nT * bp.nH * bp.nW));
  bp.fd_heads = vdsa::make_fastdiv((uint32_t)bp.heads);
  bp.fd_nw = vdsa::make_fastdiv((uint32_t)bp.nW);
  bp.fd_nh = vdsa::make_fastdiv((uint32_t)bp.nH);
  hipError_t e;
  if (prob->dtype == VDSA_F32)
    e = vdsa::launch_box_attn_f32(bp, prob->head_dim, stream);
  else if (shape.kernel == K_PP_8W)
    e = vdsa::launch_box_attn_bf16_pp(bp, stream);
  else if (shape.kernel == K_M16_4W)
    e = vdsa::launch_box_attn_bf16_m16(bp, stream);
  else
    e = vdsa::launch_box_attn_bf16(bp, prob->head_dim, stream);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

void set_qkvo(vdsa::BoxAttnParams& bp, const View& q, const View& k, const View& v, const View& o) {
  bp.q = q.ptr;
  bp.k = k.ptr;
  bp.v = v.ptr;
  bp.o = const_cast<void*>(o.ptr);
  bp.q_sb = q.st->b; bp.q_sh = q.st->h; bp.q_sn = q.st->n;
  bp.k_sb = k.st->b; bp.k_sh = k.st->h; bp.k_sn = k.st->n;
  bp.v_sb = v.st->b; bp.v_sh = v.st->h; bp.v_sn = v.st->n;
  bp.o_sb = o.st->b; bp.o_sh = o.st->h; bp.o_sn = o.st->n;
}

vdsa_status check_pool(const vdsa_problem* p, const int32_t* pool) {
  if (!pool) return fail(VDSA_ERR_NULL, "pool_hw is NULL");
  if (pool[0] < 1 || pool[1] < 1) return fail(VDSA_ERR_WINDOW, "pool sizes must be >= 1 (got %d x %d)", pool[0], pool[1]);
  (void)p;
  return VDSA_OK;
}

int64_t pooled_tokens(const vdsa_problem* p, const int32_t* pool) {
  return (int64_t)p->grid_t * ((p->grid_h + pool[0] - 1) / pool[0]) * ((p->grid_w + pool[1] - 1) / pool[1]);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t pooled_bytes(const vdsa_problem* p, const int32_t* pool) {
  return align_up((size_t)p->batch * p->heads * pooled_tokens(p, pool) * p->head_dim * elem_size(p->dtype), 256);
}

vdsa_status check_lse(const vdsa_problem* p, float* lse, uintptr_t& lo, uintptr_t& hi) {
  lo = hi = 0;
  if (!lse) return VDSA_OK;
  if ((uintptr_t)lse % 4 != 0) return fail(VDSA_ERR_ALIGN, "lse pointer is not 4-byte aligned");
  lo = (uintptr_t)lse;
  hi = lo + (uintptr_t)((int64_t)p->batch * p->heads * n_tokens(p) * 4);
  return VDSA_OK;
}

vdsa::PoolParams pool_params(const vdsa_problem* p, const int32_t* pool, const void* x, const vdsa_strides* xs,
                             void* y, const vdsa_strides* ys) {
  vdsa::PoolParams pp{};
  pp.x = x;
  pp.y = y;
  pp.x_sb = xs->b; pp.x_sh = xs->h; pp.x_sn = xs->n;
  pp.y_sb = ys->b; pp.y_sh = ys->h; pp.y_sn = ys->n;
  pp.batch = p->batch;
  pp.heads = p->heads;
  pp.head_dim = p->head_dim;
  pp.T = p->grid_t; pp.H = p->grid_h; pp.W = p->grid_w;
  pp.kh = pool[0]; pp.kw = pool[1];
  pp.Hp = (p->grid_h + pool[0] - 1) / pool[0];
  pp.Wp = (p->grid_w + pool[1] - 1) / pool[1];
  pp.fd_wp = vdsa::make_fastdiv((uint32_t)pp.Wp);
  pp.fd_hp = vdsa::make_fastdiv((uint32_t)pp.Hp);
  return pp;
}

// [batch, heads, N] fp32 contiguous LSE array: required (or nullable) pointer
// checks and its byte range.
vdsa_status check_lse_in(const vdsa_problem* p, const float* lse, const char* name, uintptr_t& lo, uintptr_t& hi) {
  if (!lse) return fail(VDSA_ERR_NULL, "%s is NULL", name);
  return check_lse(p, const_cast<float*>(lse), lo, hi) == VDSA_OK ? VDSA_OK
                                                                   : fail(VDSA_ERR_ALIGN, "%s is not 4-byte aligned", name);
}

bool same_view(const void* a, const vdsa_strides* sa, const void* b, const vdsa_strides* sb) {
  return a == b && sa->b == sb->b && sa->h == sb->h && sa->n == sb->n;
}

// The other branch's output and how it merges into the global branch (the
// fused form); mode < 0 means no merge.
struct FusedMerge {
  int mode = -1;
  const void* o_local = nullptr;
  const vdsa_strides* local_strides = nullptr;
  const float* lse_local = nullptr;
  const float* w_local = nullptr;
  const float* w_global = nullptr;
};

vdsa_status global_attn_impl(const vdsa_problem* prob, const int32_t pool_hw[2], const void* q,
                             const vdsa_strides* q_strides, const void* k, const vdsa_strides* k_strides,
                             const void* v, const vdsa_strides* v_strides, void* o, const vdsa_strides* o_strides,
                             float* lse, void* workspace, size_t workspace_bytes, const FusedMerge& fm,
                             void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  const int64_t N = n_tokens(prob);
  const int64_t M = pooled_tokens(prob, pool_hw);
  View vq{"q", q, q_strides, N}, vk{"k", k, k_strides, N}, vv{"v", v, v_strides, N},
      vo{fm.mode < 0 ? "o" : "out", o, o_strides, N};
  if ((s = check_view(prob, vq, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vk, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vv, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vo, true)) != VDSA_OK) return s;
  uintptr_t l0, l1;
  if ((s = check_lse(prob, lse, l0, l1)) != VDSA_OK) return s;
  const size_t need = 2 * pooled_bytes(prob, pool_hw);
  if (!workspace) return fail(VDSA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need)
    return fail(VDSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if ((uintptr_t)workspace % 16 != 0) return fail(VDSA_ERR_ALIGN, "workspace is not 16-byte aligned");
  const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + need;
  for (const View* in : {&vq, &vk, &vv})
    if (overlaps(vo.lo, vo.hi, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "%s overlaps %s", vo.name, in->name);
  for (const View* in : {&vq, &vk, &vv, &vo})
    if (overlaps(w0, w1, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "workspace overlaps %s", in->name);
  if (lse) {
    for (const View* in : {&vq, &vk, &vv, &vo})
      if (overlaps(l0, l1, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "lse overlaps %s", in->name);
    if (overlaps(l0, l1, w0, w1)) return fail(VDSA_ERR_ALIAS, "lse overlaps workspace");
  }

  vdsa::BoxAttnParams bp{};
  if (fm.mode >= 0) {
    if (fm.mode != VDSA_MERGE_GATED && fm.mode != VDSA_MERGE_LSE)
      return fail(VDSA_ERR_UNSUPPORTED, "unknown merge mode %d", fm.mode);
    View vl{"o_local", fm.o_local, fm.local_strides, N};
    if ((s = check_view(prob, vl, false)) != VDSA_OK) return s;
    if (!same_view(o, o_strides, fm.o_local, fm.local_strides) && overlaps(vo.lo, vo.hi, vl.lo, vl.hi))
      return fail(VDSA_ERR_ALIAS, "out overlaps o_local");
    if (overlaps(w0, w1, vl.lo, vl.hi)) return fail(VDSA_ERR_ALIAS, "workspace overlaps o_local");
    if (lse && overlaps(l0, l1, vl.lo, vl.hi)) return fail(VDSA_ERR_ALIAS, "lse_out overlaps o_local");
    if (fm.mode == VDSA_MERGE_LSE) {
      uintptr_t a0, a1;
      if ((s = check_lse_in(prob, fm.lse_local, "lse_local", a0, a1)) != VDSA_OK) return s;
      if (overlaps(vo.lo, vo.hi, a0, a1)) return fail(VDSA_ERR_ALIAS, "out overlaps lse_local");
      if (overlaps(w0, w1, a0, a1)) return fail(VDSA_ERR_ALIAS, "workspace overlaps lse_local");
      if (lse && lse != fm.lse_local && overlaps(l0, l1, a0, a1))
        return fail(VDSA_ERR_ALIAS, "lse_out overlaps lse_local");
      bp.merge = vdsa::MERGE_LSE;
      bp.lse_l = fm.lse_local;
    } else {
      if (!fm.w_global) return fail(VDSA_ERR_NULL, "w_global is NULL");
      if ((uintptr_t)fm.w_global % 4 != 0 || (fm.w_local && (uintptr_t)fm.w_local % 4 != 0))
        return fail(VDSA_ERR_ALIGN, "gate pointers must be 4-byte aligned");
      for (const float* w : {fm.w_global, fm.w_local}) {
        if (!w) continue;
        const uintptr_t a0 = (uintptr_t)w, a1 = a0 + 4 * (uintptr_t)prob->heads;
        if (overlaps(vo.lo, vo.hi, a0, a1) || overlaps(w0, w1, a0, a1) || (lse && overlaps(l0, l1, a0, a1)))
          return fail(VDSA_ERR_ALIAS, "a gate array overlaps an output or the workspace");
      }
      bp.merge = vdsa::MERGE_GATED;
      bp.w_l = fm.w_local;
      bp.w_g = fm.w_global;
    }
    bp.ol = fm.o_local;
    bp.ol_sb = fm.local_strides->b;
    bp.ol_sh = fm.local_strides->h;
    bp.ol_sn = fm.local_strides->n;
  }

  // pooled K then pooled V, each [batch, heads, M, head_dim] contiguous
  const size_t half = pooled_bytes(prob, pool_hw);
  void* kp = workspace;
  void* vp = (char*)workspace + half;
  vdsa_strides ps{(int64_t)prob->heads * M * prob->head_dim, M * prob->head_dim, prob->head_dim};
  hipError_t e = vdsa::launch_avgpool(pool_params(prob, pool_hw, k, k_strides, kp, &ps), prob->dtype == VDSA_BF16,
                                      (hipStream_t)stream);
  if (e == hipSuccess)
    e = vdsa::launch_avgpool(pool_params(prob, pool_hw, v, v_strides, vp, &ps), prob->dtype == VDSA_BF16,
                             (hipStream_t)stream);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "pooling launch failed: %s", hipGetErrorString(e));

  View vkp{"k_pooled", kp, &ps, M}, vvp{"v_pooled", vp, &ps, M};
  set_qkvo(bp, vq, vkp, vvp, vo);
  bp.lse = lse;
  bp.batch = prob->batch;
  bp.heads = prob->heads;
  bp.qT = prob->grid_t; bp.qH = prob->grid_h; bp.qW = prob->grid_w;
  // one query tile covering the whole grid; every query sees every pooled key
  bp.bT = bp.qT; bp.bH = bp.qH; bp.bW = bp.qW;
  bp.sT = bp.sH = bp.sW = 0;
  bp.nT = bp.nH = bp.nW = 1;
  bp.rT = bp.rH = bp.rW = 0;
  bp.kT = prob->grid_t;
  bp.kH = (prob->grid_h + pool_hw[0] - 1) / pool_hw[0];
  bp.kW = (prob->grid_w + pool_hw[1] - 1) / pool_hw[1];
  bp.dense_keys = 1;
  return launch_attn(prob, bp, (hipStream_t)stream);
}


// ---- backward
struct BwdViews {
  View q, k, v, o, dout, dq, dk, dv;
};

vdsa_status check_bwd(const vdsa_problem* prob, BwdViews& bv, const float* lse, uintptr_t& l0, uintptr_t& l1) {
  vdsa_status s;
  if (prob->dtype == VDSA_BF16 && prob->head_dim != 128)
    return fail(VDSA_ERR_UNSUPPORTED, "the bf16 backward supports head_dim 128 (got %d)", prob->head_dim);
  for (View* in : {&bv.q, &bv.k, &bv.v, &bv.o, &bv.dout})
    if ((s = check_view(prob, *in, false)) != VDSA_OK) return s;
  for (View* out : {&bv.dq, &bv.dk, &bv.dv})
    if ((s = check_view(prob, *out, true)) != VDSA_OK) return s;
  if ((s = check_lse_in(prob, lse, "lse", l0, l1)) != VDSA_OK) return s;
  const View* outs[3] = {&bv.dq, &bv.dk, &bv.dv};
  for (int i = 0; i < 3; ++i) {
    for (const View* in : {&bv.q, &bv.k, &bv.v, &bv.o, &bv.dout})
      if (overlaps(outs[i]->lo, outs[i]->hi, in->lo, in->hi))
        return fail(VDSA_ERR_ALIAS, "%s overlaps %s", outs[i]->name, in->name);
    if (overlaps(outs[i]->lo, outs[i]->hi, l0, l1)) return fail(VDSA_ERR_ALIAS, "%s overlaps lse", outs[i]->name);
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i]->lo, outs[i]->hi, outs[j]->lo, outs[j]->hi))
        return fail(VDSA_ERR_ALIAS, "%s overlaps %s", outs[i]->name, outs[j]->name);
  }
  return VDSA_OK;
}

vdsa_status check_workspace(const BwdViews& bv, uintptr_t l0, uintptr_t l1, void* workspace, size_t bytes,
                            size_t need) {
  if (!workspace) return fail(VDSA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (bytes < need) return fail(VDSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", bytes, need);
  if ((uintptr_t)workspace % 16 != 0) return fail(VDSA_ERR_ALIGN, "workspace is not 16-byte aligned");
  const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + need;
  for (const View* v : {&bv.q, &bv.k, &bv.v, &bv.o, &bv.dout, &bv.dq, &bv.dk, &bv.dv})
    if (overlaps(w0, w1, v->lo, v->hi)) return fail(VDSA_ERR_ALIAS, "workspace overlaps %s", v->name);
  if (overlaps(w0, w1, l0, l1)) return fail(VDSA_ERR_ALIAS, "workspace overlaps lse");
  return VDSA_OK;
}

size_t delta_bytes(const vdsa_problem* p) { return align_up((size_t)p->batch * p->heads * n_tokens(p) * 4, 256); }

vdsa::BoxBwdParams bwd_params(const vdsa_problem* prob, const BwdViews& bv, const float* lse, const float* delta) {
  vdsa::BoxBwdParams P{};
  P.q = bv.q.ptr; P.k = bv.k.ptr; P.v = bv.v.ptr; P.dout = bv.dout.ptr;
  P.lse = lse;
  P.delta = delta;
  P.dq = const_cast<void*>(bv.dq.ptr); P.dk = const_cast<void*>(bv.dk.ptr); P.dv = const_cast<void*>(bv.dv.ptr);
  P.q_sb = bv.q.st->b; P.q_sh = bv.q.st->h; P.q_sn = bv.q.st->n;
  P.k_sb = bv.k.st->b; P.k_sh = bv.k.st->h; P.k_sn = bv.k.st->n;
  P.v_sb = bv.v.st->b; P.v_sh = bv.v.st->h; P.v_sn = bv.v.st->n;
  P.do_sb = bv.dout.st->b; P.do_sh = bv.dout.st->h; P.do_sn = bv.dout.st->n;
  P.dq_sb = bv.dq.st->b; P.dq_sh = bv.dq.st->h; P.dq_sn = bv.dq.st->n;
  P.dk_sb = bv.dk.st->b; P.dk_sh = bv.dk.st->h; P.dk_sn = bv.dk.st->n;
  P.dv_sb = bv.dv.st->b; P.dv_sh = bv.dv.st->h; P.dv_sn = bv.dv.st->n;
  P.n_q = n_tokens(prob);
  P.n_k = n_tokens(prob);
  P.head_dim = prob->head_dim;
  P.scale = prob->scale;
  P.g.batch = prob->batch;
  P.g.heads = prob->heads;
  P.g.scale_log2e = prob->scale * 1.4426950408889634f;
  return P;
}

// Launch one backward pass over the geometry in P.g (own tiles from qT.. /
// bT.. / sT.., iterated boxes from rT.. or dense_keys over kT..).
vdsa_status launch_bwd_pass(const vdsa_problem* prob, vdsa::BoxBwdParams& P, bool kv, hipStream_t stream) {
  const int bf16 = prob->dtype == VDSA_BF16;
  const int bm = vdsa::attn_bwd_block_m(bf16, kv);
  vdsa::BoxAttnParams& g = P.g;
  const int64_t mv = (int64_t)max_tile_extent(g.qT, g.bT, g.sT) * max_tile_extent(g.qH, g.bH, g.sH) *
                     max_tile_extent(g.qW, g.bW, g.sW);
  g.qblocks = (int32_t)((mv + bm - 1) / bm);
  const int64_t total = (int64_t)g.batch * g.heads * g.nT * g.nH * g.nW * g.qblocks;
  if (total >= (int64_t(1) << 31) / 512)
    return fail(VDSA_ERR_SHAPE, "problem needs %lld workgroups, beyond the launch limit", (long long)total);
  g.total_wg = (int32_t)total;
  const hipError_t e = kv ? vdsa::launch_attn_bwd_dkdv(P, bf16, stream) : vdsa::launch_attn_bwd_dq(P, bf16, stream);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return VDSA_OK;
}

vdsa_status launch_delta(const vdsa_problem* prob, const BwdViews& bv, float* delta, hipStream_t stream) {
  vdsa::RowDotParams rp{};
  rp.a = bv.dout.ptr;
  rp.b = bv.o.ptr;
  rp.out = delta;
  rp.a_sb = bv.dout.st->b; rp.a_sh = bv.dout.st->h; rp.a_sn = bv.dout.st->n;
  rp.b_sb = bv.o.st->b; rp.b_sh = bv.o.st->h; rp.b_sn = bv.o.st->n;
  rp.batch = prob->batch;
  rp.heads = prob->heads;
  rp.head_dim = prob->head_dim;
  rp.n = n_tokens(prob);
  const hipError_t e = vdsa::launch_rowdot(rp, prob->dtype == VDSA_BF16, stream);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "delta launch failed: %s", hipGetErrorString(e));
  return VDSA_OK;
}

size_t pooled_f32_bytes(const vdsa_problem* p, const int32_t* pool) {
  return align_up((size_t)p->batch * p->heads * pooled_tokens(p, pool) * p->head_dim * 4, 256);
}


// Pooled K then pooled V (and, for the compressed global branch, pooled Q and
// the pooled output) at the start of the workspace.
vdsa_status check_pooled_call(const vdsa_problem* prob, const int32_t* pool_hw, View& vq, View& vk, View& vv,
                              View& vo, float* lse, void* workspace, size_t workspace_bytes, size_t need) {
  vdsa_status s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  if ((s = check_view(prob, vq, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vk, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vv, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vo, true)) != VDSA_OK) return s;
  uintptr_t l0, l1;
  if ((s = check_lse(prob, lse, l0, l1)) != VDSA_OK) return s;
  if (!workspace) return fail(VDSA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need) return fail(VDSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if ((uintptr_t)workspace % 16 != 0) return fail(VDSA_ERR_ALIGN, "workspace is not 16-byte aligned");
  const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + need;
  for (const View* in : {&vq, &vk, &vv})
    if (overlaps(vo.lo, vo.hi, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "o overlaps %s", in->name);
  for (const View* in : {&vq, &vk, &vv, &vo})
    if (overlaps(w0, w1, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "workspace overlaps %s", in->name);
  if (lse) {
    for (const View* in : {&vq, &vk, &vv, &vo})
      if (overlaps(l0, l1, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "lse overlaps %s", in->name);
    if (overlaps(l0, l1, w0, w1)) return fail(VDSA_ERR_ALIAS, "lse overlaps workspace");
  }
  return VDSA_OK;
}

}  // namespace

extern "C" {

int vdsa_abi_version(void) { return VDSA_ABI_VERSION; }

const char* vdsa_sta_kernel(const vdsa_problem* prob, const vdsa_sta_cfg* cfg) {
  if (check_problem(prob) != VDSA_OK || check_sta_cfg(cfg) != VDSA_OK) return nullptr;
  vdsa::BoxAttnParams bp{};
  bp.batch = prob->batch;
  bp.heads = prob->heads;
  set_sta_geometry(bp, prob, cfg);
  ok();
  return attn_kernel_name(prob, bp);
}

const char* vdsa_status_string(vdsa_status s) {
  switch (s) {
    case VDSA_OK: return "ok";
    case VDSA_ERR_NULL: return "null pointer";
    case VDSA_ERR_SHAPE: return "invalid shape";
    case VDSA_ERR_WINDOW: return "invalid tile, window, shift or pool";
    case VDSA_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or scale";
    case VDSA_ERR_ALIGN: return "misaligned pointer or stride";
    case VDSA_ERR_ALIAS: return "output overlaps an input";
    case VDSA_ERR_WORKSPACE: return "workspace missing or too small";
    case VDSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* vdsa_last_error(void) { return g_last_error.c_str(); }

vdsa_status sta_attn_fwd(const vdsa_problem* prob, const vdsa_sta_cfg* cfg, const void* q,
                         const vdsa_strides* q_strides, const void* k, const vdsa_strides* k_strides,
                         const void* v, const vdsa_strides* v_strides, void* o,
                         const vdsa_strides* o_strides, float* lse, void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_sta_cfg(cfg)) != VDSA_OK) return s;
  const int64_t N = n_tokens(prob);
  View vq{"q", q, q_strides, N}, vk{"k", k, k_strides, N}, vv{"v", v, v_strides, N}, vo{"o", o, o_strides, N};
  if ((s = check_view(prob, vq, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vk, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vv, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vo, true)) != VDSA_OK) return s;
  uintptr_t l0, l1;
  if ((s = check_lse(prob, lse, l0, l1)) != VDSA_OK) return s;
  for (const View* in : {&vq, &vk, &vv})
    if (overlaps(vo.lo, vo.hi, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "o overlaps %s", in->name);
  if (lse) {
    for (const View* in : {&vq, &vk, &vv, &vo})
      if (overlaps(l0, l1, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "lse overlaps %s", in->name);
  }

  vdsa::BoxAttnParams bp{};
  set_qkvo(bp, vq, vk, vv, vo);
  bp.lse = lse;
  bp.batch = prob->batch;
  bp.heads = prob->heads;
  set_sta_geometry(bp, prob, cfg);
  return launch_attn(prob, bp, (hipStream_t)stream);
}

vdsa_status global_pooled_attn_workspace_size(const vdsa_problem* prob, const int32_t pool_hw[2], size_t* bytes) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  if (!bytes) return fail(VDSA_ERR_NULL, "bytes is NULL");
  *bytes = 2 * pooled_bytes(prob, pool_hw);
  return ok();
}

vdsa_status kv_avgpool_fwd(const vdsa_problem* prob, const int32_t pool_hw[2], const void* x,
                           const vdsa_strides* x_strides, void* x_pooled, const vdsa_strides* pooled_strides,
                           void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  const int64_t M = pooled_tokens(prob, pool_hw);
  View vx{"x", x, x_strides, n_tokens(prob)}, vy{"x_pooled", x_pooled, pooled_strides, M};
  if ((s = check_view(prob, vx, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vy, true)) != VDSA_OK) return s;
  if (overlaps(vx.lo, vx.hi, vy.lo, vy.hi)) return fail(VDSA_ERR_ALIAS, "x_pooled overlaps x");
  const vdsa::PoolParams pp = pool_params(prob, pool_hw, x, x_strides, x_pooled, pooled_strides);
  hipError_t e = vdsa::launch_avgpool(pp, prob->dtype == VDSA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "pooling launch failed: %s", hipGetErrorString(e));
  return ok();
}

vdsa_status global_pooled_attn_fwd(const vdsa_problem* prob, const int32_t pool_hw[2], const void* q,
                                   const vdsa_strides* q_strides, const void* k, const vdsa_strides* k_strides,
                                   const void* v, const vdsa_strides* v_strides, void* o,
                                   const vdsa_strides* o_strides, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return global_attn_impl(prob, pool_hw, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, workspace,
                          workspace_bytes, FusedMerge{}, stream);
}

vdsa_status global_pooled_attn_fwd_noalloc(const vdsa_problem* prob, const int32_t pool_hw[2], const void* q,
                                           const vdsa_strides* q_strides, const void* k,
                                           const vdsa_strides* k_strides, const void* v,
                                           const vdsa_strides* v_strides, void* o, const vdsa_strides* o_strides,
                                           float* lse, void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  const size_t need = 2 * pooled_bytes(prob, pool_hw);
  if (need > vdsa::STATIC_SCRATCH_BYTES)
    return fail(VDSA_ERR_WORKSPACE, "pooled K and V need %zu bytes, beyond the %zu-byte static scratch", need,
                vdsa::STATIC_SCRATCH_BYTES);
  // every argument check before the scratch lookup (the first HIP call);
  // global_attn_impl repeats them and adds the aliasing checks
  const int64_t N = n_tokens(prob);
  View vq{"q", q, q_strides, N}, vk{"k", k, k_strides, N}, vv{"v", v, v_strides, N}, vo{"o", o, o_strides, N};
  for (View* vw : {&vq, &vk, &vv})
    if ((s = check_view(prob, *vw, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vo, true)) != VDSA_OK) return s;
  uintptr_t l0, l1;
  if ((s = check_lse(prob, lse, l0, l1)) != VDSA_OK) return s;
  for (const View* in : {&vq, &vk, &vv})
    if (overlaps(vo.lo, vo.hi, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "o overlaps %s", in->name);
  void* scratch = nullptr;
  const hipError_t e = vdsa::static_scratch(&scratch);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  return global_attn_impl(prob, pool_hw, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, scratch,
                          vdsa::STATIC_SCRATCH_BYTES, FusedMerge{}, stream);
}

vdsa_status global_pooled_attn_merge_fwd(const vdsa_problem* prob, const int32_t pool_hw[2], const void* q,
                                         const vdsa_strides* q_strides, const void* k, const vdsa_strides* k_strides,
                                         const void* v, const vdsa_strides* v_strides, vdsa_merge_mode mode,
                                         const void* o_local, const vdsa_strides* local_strides,
                                         const float* lse_local, const float* w_local, const float* w_global,
                                         void* out, const vdsa_strides* out_strides, float* lse_out,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  FusedMerge fm;
  fm.mode = (int)mode;
  fm.o_local = o_local;
  fm.local_strides = local_strides;
  fm.lse_local = lse_local;
  fm.w_local = w_local;
  fm.w_global = w_global;
  if (fm.mode < 0) return fail(VDSA_ERR_UNSUPPORTED, "unknown merge mode %d", fm.mode);
  return global_attn_impl(prob, pool_hw, q, q_strides, k, k_strides, v, v_strides, out, out_strides, lse_out,
                          workspace, workspace_bytes, fm, stream);
}

vdsa_status dual_branch_merge(const vdsa_problem* prob, const void* o_local, const vdsa_strides* local_strides,
                              const void* o_global, const vdsa_strides* global_strides, const float* w_local,
                              const float* w_global, void* out, const vdsa_strides* out_strides, void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  const int64_t N = n_tokens(prob);
  View va{"o_local", o_local, local_strides, N}, vg{"o_global", o_global, global_strides, N},
      vo{"out", out, out_strides, N};
  if ((s = check_view(prob, va, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vg, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vo, true)) != VDSA_OK) return s;
  if (!w_global) return fail(VDSA_ERR_NULL, "w_global is NULL");
  if ((uintptr_t)w_global % 4 != 0 || (w_local && (uintptr_t)w_local % 4 != 0))
    return fail(VDSA_ERR_ALIGN, "gate pointers must be 4-byte aligned");
  const bool in_place = out == o_local && out_strides->b == local_strides->b && out_strides->h == local_strides->h &&
                        out_strides->n == local_strides->n;
  if (!in_place && overlaps(vo.lo, vo.hi, va.lo, va.hi)) return fail(VDSA_ERR_ALIAS, "out overlaps o_local");
  if (overlaps(vo.lo, vo.hi, vg.lo, vg.hi)) return fail(VDSA_ERR_ALIAS, "out overlaps o_global");
  const uintptr_t g0 = (uintptr_t)w_global, g1 = g0 + 4 * (uintptr_t)prob->heads;
  if (overlaps(vo.lo, vo.hi, g0, g1)) return fail(VDSA_ERR_ALIAS, "out overlaps w_global");
  if (w_local) {
    const uintptr_t a0 = (uintptr_t)w_local, a1 = a0 + 4 * (uintptr_t)prob->heads;
    if (overlaps(vo.lo, vo.hi, a0, a1)) return fail(VDSA_ERR_ALIAS, "out overlaps w_local");
  }
  vdsa::MergeParams mp{};
  mp.a = o_local;
  mp.g = o_global;
  mp.w_a = w_local;
  mp.w_g = w_global;
  mp.out = out;
  mp.a_sb = local_strides->b; mp.a_sh = local_strides->h; mp.a_sn = local_strides->n;
  mp.g_sb = global_strides->b; mp.g_sh = global_strides->h; mp.g_sn = global_strides->n;
  mp.o_sb = out_strides->b; mp.o_sh = out_strides->h; mp.o_sn = out_strides->n;
  mp.batch = prob->batch;
  mp.heads = prob->heads;
  mp.head_dim = prob->head_dim;
  mp.n_tokens = N;
  hipError_t e = vdsa::launch_merge(mp, prob->dtype == VDSA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

vdsa_status dual_branch_merge_lse(const vdsa_problem* prob, const void* o_local, const vdsa_strides* local_strides,
                                  const float* lse_local, const void* o_global, const vdsa_strides* global_strides,
                                  const float* lse_global, void* out, const vdsa_strides* out_strides, float* lse_out,
                                  void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  const int64_t N = n_tokens(prob);
  View va{"o_local", o_local, local_strides, N}, vg{"o_global", o_global, global_strides, N},
      vo{"out", out, out_strides, N};
  if ((s = check_view(prob, va, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vg, false)) != VDSA_OK) return s;
  if ((s = check_view(prob, vo, true)) != VDSA_OK) return s;
  uintptr_t la0, la1, lg0, lg1, lo0, lo1;
  if ((s = check_lse_in(prob, lse_local, "lse_local", la0, la1)) != VDSA_OK) return s;
  if ((s = check_lse_in(prob, lse_global, "lse_global", lg0, lg1)) != VDSA_OK) return s;
  if ((s = check_lse(prob, lse_out, lo0, lo1)) != VDSA_OK) return s;
  if (!same_view(out, out_strides, o_local, local_strides) && overlaps(vo.lo, vo.hi, va.lo, va.hi))
    return fail(VDSA_ERR_ALIAS, "out overlaps o_local");
  if (!same_view(out, out_strides, o_global, global_strides) && overlaps(vo.lo, vo.hi, vg.lo, vg.hi))
    return fail(VDSA_ERR_ALIAS, "out overlaps o_global");
  if (overlaps(vo.lo, vo.hi, la0, la1)) return fail(VDSA_ERR_ALIAS, "out overlaps lse_local");
  if (overlaps(vo.lo, vo.hi, lg0, lg1)) return fail(VDSA_ERR_ALIAS, "out overlaps lse_global");
  if (lse_out) {
    if (lse_out != lse_local && overlaps(lo0, lo1, la0, la1)) return fail(VDSA_ERR_ALIAS, "lse_out overlaps lse_local");
    if (lse_out != lse_global && overlaps(lo0, lo1, lg0, lg1))
      return fail(VDSA_ERR_ALIAS, "lse_out overlaps lse_global");
    for (const View* in : {&va, &vg, &vo})
      if (overlaps(lo0, lo1, in->lo, in->hi)) return fail(VDSA_ERR_ALIAS, "lse_out overlaps %s", in->name);
  }
  vdsa::MergeParams mp{};
  mp.a = o_local;
  mp.g = o_global;
  mp.lse_a = lse_local;
  mp.lse_g = lse_global;
  mp.lse_out = lse_out;
  mp.out = out;
  mp.a_sb = local_strides->b; mp.a_sh = local_strides->h; mp.a_sn = local_strides->n;
  mp.g_sb = global_strides->b; mp.g_sh = global_strides->h; mp.g_sn = global_strides->n;
  mp.o_sb = out_strides->b; mp.o_sh = out_strides->h; mp.o_sn = out_strides->n;
  mp.batch = prob->batch;
  mp.heads = prob->heads;
  mp.head_dim = prob->head_dim;
  mp.n_tokens = N;
  hipError_t e = vdsa::launch_merge(mp, prob->dtype == VDSA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

vdsa_status hier_pooled_attn_workspace_size(const vdsa_problem* prob, const int32_t pool_hw[2], size_t* bytes) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  if (!bytes) return fail(VDSA_ERR_NULL, "bytes is NULL");
  *bytes = 2 * pooled_bytes(prob, pool_hw);
  return ok();
}

vdsa_status hier_pooled_attn_fwd(const vdsa_problem* prob, const vdsa_sta_cfg* cfg, const int32_t pool_hw[2],
                                 const void* q, const vdsa_strides* q_strides, const void* k,
                                 const vdsa_strides* k_strides, const void* v, const vdsa_strides* v_strides,
                                 void* o, const vdsa_strides* o_strides, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_sta_cfg(cfg)) != VDSA_OK) return s;
  if (cfg->window_mode != VDSA_WINDOW_CLIP)
    return fail(VDSA_ERR_WINDOW, "hier_pooled_attn_fwd supports window_mode VDSA_WINDOW_CLIP only");
  const int64_t N = n_tokens(prob);
  View vq{"q", q, q_strides, N}, vk{"k", k, k_strides, N}, vv{"v", v, v_strides, N}, vo{"o", o, o_strides, N};
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  const size_t half = pooled_bytes(prob, pool_hw);
  if ((s = check_pooled_call(prob, pool_hw, vq, vk, vv, vo, lse, workspace, workspace_bytes, 2 * half)) != VDSA_OK)
    return s;
  const int64_t M = pooled_tokens(prob, pool_hw);
  void* kp = workspace;
  void* vp = (char*)workspace + half;
  vdsa_strides ps{(int64_t)prob->heads * M * prob->head_dim, M * prob->head_dim, prob->head_dim};
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e = vdsa::launch_avgpool(pool_params(prob, pool_hw, k, k_strides, kp, &ps), prob->dtype == VDSA_BF16, st);
  if (e == hipSuccess)
    e = vdsa::launch_avgpool(pool_params(prob, pool_hw, v, v_strides, vp, &ps), prob->dtype == VDSA_BF16, st);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "pooling launch failed: %s", hipGetErrorString(e));

  vdsa::BoxAttnParams bp{};
  View vkp{"k_pooled", kp, &ps, M}, vvp{"v_pooled", vp, &ps, M};
  set_qkvo(bp, vq, vkp, vvp, vo);
  bp.lse = lse;
  bp.batch = prob->batch;
  bp.heads = prob->heads;
  bp.qT = prob->grid_t; bp.qH = prob->grid_h; bp.qW = prob->grid_w;
  bp.bT = cfg->tile[0]; bp.bH = cfg->tile[1]; bp.bW = cfg->tile[2];
  bp.sT = cfg->shift[0]; bp.sH = cfg->shift[1]; bp.sW = cfg->shift[2];
  bp.nT = tiles_along(bp.qT, bp.bT, bp.sT);
  bp.nH = tiles_along(bp.qH, bp.bH, bp.sH);
  bp.nW = tiles_along(bp.qW, bp.bW, bp.sW);
  bp.rT = (cfg->window[0] - 1) / 2; bp.rH = (cfg->window[1] - 1) / 2; bp.rW = (cfg->window[2] - 1) / 2;
  bp.kT = prob->grid_t;
  bp.kH = (prob->grid_h + pool_hw[0] - 1) / pool_hw[0];
  bp.kW = (prob->grid_w + pool_hw[1] - 1) / pool_hw[1];
  bp.kpT = 1; bp.kpH = pool_hw[0]; bp.kpW = pool_hw[1];
  bp.dense_keys = 0;
  return launch_attn(prob, bp, st);
}

vdsa_status compressed_global_attn_workspace_size(const vdsa_problem* prob, const int32_t pool_hw[2],
                                                  size_t* bytes) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  if (!bytes) return fail(VDSA_ERR_NULL, "bytes is NULL");
  *bytes = 4 * pooled_bytes(prob, pool_hw);
  return ok();
}

vdsa_status compressed_global_attn_fwd(const vdsa_problem* prob, const int32_t pool_hw[2], const void* q,
                                       const vdsa_strides* q_strides, const void* k, const vdsa_strides* k_strides,
                                       const void* v, const vdsa_strides* v_strides, void* o,
                                       const vdsa_strides* o_strides, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  const int64_t N = n_tokens(prob);
  View vq{"q", q, q_strides, N}, vk{"k", k, k_strides, N}, vv{"v", v, v_strides, N}, vo{"o", o, o_strides, N};
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  const size_t part = pooled_bytes(prob, pool_hw);
  if ((s = check_pooled_call(prob, pool_hw, vq, vk, vv, vo, nullptr, workspace, workspace_bytes, 4 * part)) !=
      VDSA_OK)
    return s;
  const int64_t M = pooled_tokens(prob, pool_hw);
  const int Hp = (prob->grid_h + pool_hw[0] - 1) / pool_hw[0], Wp = (prob->grid_w + pool_hw[1] - 1) / pool_hw[1];
  void* qp = workspace;
  void* kp = (char*)workspace + part;
  void* vp = (char*)workspace + 2 * part;
  void* op = (char*)workspace + 3 * part;
  vdsa_strides ps{(int64_t)prob->heads * M * prob->head_dim, M * prob->head_dim, prob->head_dim};
  const hipStream_t st = (hipStream_t)stream;
  const int bf16 = prob->dtype == VDSA_BF16;
  hipError_t e = vdsa::launch_avgpool(pool_params(prob, pool_hw, q, q_strides, qp, &ps), bf16, st);
  if (e == hipSuccess) e = vdsa::launch_avgpool(pool_params(prob, pool_hw, k, k_strides, kp, &ps), bf16, st);
  if (e == hipSuccess) e = vdsa::launch_avgpool(pool_params(prob, pool_hw, v, v_strides, vp, &ps), bf16, st);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "pooling launch failed: %s", hipGetErrorString(e));

  // full attention among the pooled tokens: one query tile over the pooled grid
  vdsa::BoxAttnParams bp{};
  View vqp{"q_pooled", qp, &ps, M}, vkp{"k_pooled", kp, &ps, M}, vvp{"v_pooled", vp, &ps, M},
      vop{"o_pooled", op, &ps, M};
  set_qkvo(bp, vqp, vkp, vvp, vop);
  bp.batch = prob->batch;
  bp.heads = prob->heads;
  bp.qT = prob->grid_t; bp.qH = Hp; bp.qW = Wp;
  bp.bT = bp.qT; bp.bH = bp.qH; bp.bW = bp.qW;
  bp.nT = bp.nH = bp.nW = 1;
  bp.kT = prob->grid_t; bp.kH = Hp; bp.kW = Wp;
  bp.dense_keys = 1;
  if ((s = launch_attn(prob, bp, st)) != VDSA_OK) return s;

  vdsa::UpsampleParams up{};
  up.xp = op;
  up.out = o;
  up.o_sb = o_strides->b; up.o_sh = o_strides->h; up.o_sn = o_strides->n;
  up.batch = prob->batch; up.heads = prob->heads; up.head_dim = prob->head_dim;
  up.T = prob->grid_t; up.H = prob->grid_h; up.W = prob->grid_w; up.Hp = Hp; up.Wp = Wp;
  up.fd_hw = vdsa::make_fastdiv((uint32_t)(up.H * up.W));
  up.fd_w = vdsa::make_fastdiv((uint32_t)up.W);
  e = vdsa::launch_upsample(up, bf16, st);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "upsampling launch failed: %s", hipGetErrorString(e));
  return ok();
}

vdsa_status sta_attn_bwd_workspace_size(const vdsa_problem* prob, size_t* bytes) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if (!bytes) return fail(VDSA_ERR_NULL, "bytes is NULL");
  *bytes = delta_bytes(prob);
  return ok();
}

vdsa_status sta_attn_bwd(const vdsa_problem* prob, const vdsa_sta_cfg* cfg, const void* q,
                         const vdsa_strides* q_strides, const void* k, const vdsa_strides* k_strides,
                         const void* v, const vdsa_strides* v_strides, const void* o,
                         const vdsa_strides* o_strides, const void* d_o, const vdsa_strides* do_strides,
                         const float* lse, void* dq, const vdsa_strides* dq_strides, void* dk,
                         const vdsa_strides* dk_strides, void* dv, const vdsa_strides* dv_strides,
                         void* workspace, size_t workspace_bytes, void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_sta_cfg(cfg)) != VDSA_OK) return s;
  const int64_t N = n_tokens(prob);
  BwdViews bv{{"q", q, q_strides, N},   {"k", k, k_strides, N},    {"v", v, v_strides, N},
              {"o", o, o_strides, N},   {"d_o", d_o, do_strides, N}, {"dq", dq, dq_strides, N},
              {"dk", dk, dk_strides, N}, {"dv", dv, dv_strides, N}};
  uintptr_t l0, l1;
  if ((s = check_bwd(prob, bv, lse, l0, l1)) != VDSA_OK) return s;
  if ((s = check_workspace(bv, l0, l1, workspace, workspace_bytes, delta_bytes(prob))) != VDSA_OK) return s;

  float* delta = (float*)workspace;
  if ((s = launch_delta(prob, bv, delta, (hipStream_t)stream)) != VDSA_OK) return s;
  vdsa::BoxBwdParams P = bwd_params(prob, bv, lse, delta);
  vdsa::BoxAttnParams& g = P.g;
  set_sta_geometry(g, prob, cfg);
  if ((s = launch_bwd_pass(prob, P, false, (hipStream_t)stream)) != VDSA_OK) return s;
  // The clipped relation is symmetric (also in the rolled grid), so the dK/dV
  // pass walks the same boxes; inward windows walk their transpose.
  if (g.wmode == vdsa::WIN_INWARD) g.wmode = vdsa::WIN_INWARD_T;
  if ((s = launch_bwd_pass(prob, P, true, (hipStream_t)stream)) != VDSA_OK) return s;
  return ok();
}

vdsa_status global_pooled_attn_bwd_workspace_size(const vdsa_problem* prob, const int32_t pool_hw[2],
                                                  size_t* bytes) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  if (!bytes) return fail(VDSA_ERR_NULL, "bytes is NULL");
  *bytes = delta_bytes(prob) + 2 * pooled_bytes(prob, pool_hw) + 2 * pooled_f32_bytes(prob, pool_hw);
  return ok();
}

vdsa_status global_pooled_attn_bwd(const vdsa_problem* prob, const int32_t pool_hw[2], const void* q,
                                   const vdsa_strides* q_strides, const void* k, const vdsa_strides* k_strides,
                                   const void* v, const vdsa_strides* v_strides, const void* o,
                                   const vdsa_strides* o_strides, const void* d_o, const vdsa_strides* do_strides,
                                   const float* lse, void* dq, const vdsa_strides* dq_strides, void* dk,
                                   const vdsa_strides* dk_strides, void* dv, const vdsa_strides* dv_strides,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  const int64_t N = n_tokens(prob);
  const int64_t M = pooled_tokens(prob, pool_hw);
  BwdViews bv{{"q", q, q_strides, N},   {"k", k, k_strides, N},    {"v", v, v_strides, N},
              {"o", o, o_strides, N},   {"d_o", d_o, do_strides, N}, {"dq", dq, dq_strides, N},
              {"dk", dk, dk_strides, N}, {"dv", dv, dv_strides, N}};
  uintptr_t l0, l1;
  if ((s = check_bwd(prob, bv, lse, l0, l1)) != VDSA_OK) return s;
  const size_t need = delta_bytes(prob) + 2 * pooled_bytes(prob, pool_hw) + 2 * pooled_f32_bytes(prob, pool_hw);
  if ((s = check_workspace(bv, l0, l1, workspace, workspace_bytes, need)) != VDSA_OK) return s;

  char* ws = (char*)workspace;
  float* delta = (float*)ws;
  void* kp = ws + delta_bytes(prob);
  void* vp = (char*)kp + pooled_bytes(prob, pool_hw);
  float* dkp = (float*)((char*)vp + pooled_bytes(prob, pool_hw));
  float* dvp = (float*)((char*)dkp + pooled_f32_bytes(prob, pool_hw));
  const hipStream_t st = (hipStream_t)stream;
  if ((s = launch_delta(prob, bv, delta, st)) != VDSA_OK) return s;
  vdsa_strides ps{(int64_t)prob->heads * M * prob->head_dim, M * prob->head_dim, prob->head_dim};
  hipError_t e = vdsa::launch_avgpool(pool_params(prob, pool_hw, k, k_strides, kp, &ps), prob->dtype == VDSA_BF16, st);
  if (e == hipSuccess)
    e = vdsa::launch_avgpool(pool_params(prob, pool_hw, v, v_strides, vp, &ps), prob->dtype == VDSA_BF16, st);
  if (e != hipSuccess) return fail(VDSA_ERR_HIP, "pooling launch failed: %s", hipGetErrorString(e));
  const int Hp = (prob->grid_h + pool_hw[0] - 1) / pool_hw[0], Wp = (prob->grid_w + pool_hw[1] - 1) / pool_hw[1];

  // dQ pass: the forward's geometry (one query tile over the grid, every
  // pooled key)
  vdsa::BoxBwdParams P = bwd_params(prob, bv, lse, delta);
  P.k = kp; P.v = vp;
  P.k_sb = ps.b; P.k_sh = ps.h; P.k_sn = ps.n;
  P.v_sb = ps.b; P.v_sh = ps.h; P.v_sn = ps.n;
  P.n_k = M;
  vdsa::BoxAttnParams& g = P.g;
  g.qT = prob->grid_t; g.qH = prob->grid_h; g.qW = prob->grid_w;
  g.bT = g.qT; g.bH = g.qH; g.bW = g.qW;
  g.nT = g.nH = g.nW = 1;
  g.kT = prob->grid_t; g.kH = Hp; g.kW = Wp;
  g.dense_keys = 1;
  if ((s = launch_bwd_pass(prob, P, false, st)) != VDSA_OK) return s;

  // dK/dV pass: own rows = pooled keys (one tile over the pooled grid), every
  // query iterated; fp32 gradients of the pooled keys into the workspace
  vdsa::BoxBwdParams Pk = P;
  Pk.dk = dkp; Pk.dv = dvp;
  Pk.dk_sb = ps.b; Pk.dk_sh = ps.h; Pk.dk_sn = ps.n;
  Pk.dv_sb = ps.b; Pk.dv_sh = ps.h; Pk.dv_sn = ps.n;
  Pk.grad_f32 = 1;
  vdsa::BoxAttnParams& gk = Pk.g;
  gk.qT = prob->grid_t; gk.qH = Hp; gk.qW = Wp;
  gk.bT = gk.qT; gk.bH = gk.qH; gk.bW = gk.qW;
  gk.nT = gk.nH = gk.nW = 1;
  gk.kT = prob->grid_t; gk.kH = prob->grid_h; gk.kW = prob->grid_w;
  gk.dense_keys = 1;
  if ((s = launch_bwd_pass(prob, Pk, true, st)) != VDSA_OK) return s;

  // through the pooling: every token of a cell gets the cell's gradient / count
  for (int which = 0; which < 2; ++which) {
    vdsa::UnpoolParams up{};
    up.gp = which == 0 ? dkp : dvp;
    up.g = which == 0 ? dk : dv;
    const vdsa_strides* gs = which == 0 ? dk_strides : dv_strides;
    up.g_sb = gs->b; up.g_sh = gs->h; up.g_sn = gs->n;
    up.batch = prob->batch; up.heads = prob->heads; up.head_dim = prob->head_dim;
    up.T = prob->grid_t; up.H = prob->grid_h; up.W = prob->grid_w;
    up.kh = pool_hw[0]; up.kw = pool_hw[1];
    up.Hp = Hp; up.Wp = Wp;
    up.fd_hw = vdsa::make_fastdiv((uint32_t)(up.H * up.W));
    up.fd_w = vdsa::make_fastdiv((uint32_t)up.W);
    up.fd_kh = vdsa::make_fastdiv((uint32_t)up.kh);
    up.fd_kw = vdsa::make_fastdiv((uint32_t)up.kw);
    e = vdsa::launch_unpool_grad(up, prob->dtype == VDSA_BF16, st);
    if (e != hipSuccess) return fail(VDSA_ERR_HIP, "pooling-gradient launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

vdsa_status vdsa_sta_flops(const vdsa_problem* prob, const vdsa_sta_cfg* cfg, double* flops) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_sta_cfg(cfg)) != VDSA_OK) return s;
  if (!flops) return fail(VDSA_ERR_NULL, "flops is NULL");
  // The window mask is a product over dims and tile sizes factorise, so the
  // attended-pair count is the product of per-dim counts
  //   sum_a size(a) * sum_{|c-a| <= r} size(c).
  // (the cyclic mode counts on the rolled grid, tiled from 0)
  const int L[3] = {prob->grid_t, prob->grid_h, prob->grid_w};
  const int mode = cfg->window_mode == VDSA_WINDOW_INWARD ? vdsa::WIN_INWARD : vdsa::WIN_CLIP;
  double pairs = 1.0;
  for (int d = 0; d < 3; ++d) {
    const int b = cfg->tile[d], sh = lattice_shift(cfg, d), r = (cfg->window[d] - 1) / 2;
    const int n = tiles_along(L[d], b, sh);
    auto size = [&](int i) { return std::min(L[d], (i + 1) * b - sh) - std::max(0, i * b - sh); };
    double acc = 0.0;
    for (int a = 0; a < n; ++a) {
      int c0, c1;
      vdsa::window_range(a, r, n, mode, c0, c1);
      double keys = 0.0;
      for (int c = c0; c <= c1; ++c) keys += size(c);
      acc += size(a) * keys;
    }
    pairs *= acc;
  }
  *flops = 4.0 * prob->head_dim * prob->batch * prob->heads * pairs;
  return ok();
}

vdsa_status vdsa_hier_flops(const vdsa_problem* prob, const vdsa_sta_cfg* cfg, const int32_t pool_hw[2],
                            double* flops) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_sta_cfg(cfg)) != VDSA_OK) return s;
  if (cfg->window_mode != VDSA_WINDOW_CLIP)
    return fail(VDSA_ERR_WINDOW, "vdsa_hier_flops supports window_mode VDSA_WINDOW_CLIP only");
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  if (!flops) return fail(VDSA_ERR_NULL, "flops is NULL");
  // per dim: sum over query tiles of size(a) * cells intersecting the window
  // box of a (the key set is a product of per-dim intervals)
  const int L[3] = {prob->grid_t, prob->grid_h, prob->grid_w};
  const int pk[3] = {1, pool_hw[0], pool_hw[1]};
  double pairs = 1.0;
  for (int d = 0; d < 3; ++d) {
    const int b = cfg->tile[d], sh = cfg->shift[d], r = (cfg->window[d] - 1) / 2;
    const int n = tiles_along(L[d], b, sh);
    double acc = 0.0;
    for (int a = 0; a < n; ++a) {
      const int size = std::min(L[d], (a + 1) * b - sh) - std::max(0, a * b - sh);
      const int c0 = std::max(0, a - r), c1 = std::min(n - 1, a + r);
      const int lo = std::max(0, c0 * b - sh), hi = std::min(L[d], (c1 + 1) * b - sh);
      const int cells = (hi + pk[d] - 1) / pk[d] - lo / pk[d];
      acc += (double)size * cells;
    }
    pairs *= acc;
  }
  *flops = 4.0 * prob->head_dim * prob->batch * prob->heads * pairs;
  return ok();
}

vdsa_status vdsa_compressed_global_flops(const vdsa_problem* prob, const int32_t pool_hw[2], double* flops) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  if (!flops) return fail(VDSA_ERR_NULL, "flops is NULL");
  const double M = (double)pooled_tokens(prob, pool_hw);
  *flops = 4.0 * prob->head_dim * prob->batch * prob->heads * M * M;
  return ok();
}

vdsa_status vdsa_global_flops(const vdsa_problem* prob, const int32_t pool_hw[2], double* flops) {
  vdsa_status s;
  if ((s = check_problem(prob)) != VDSA_OK) return s;
  if ((s = check_pool(prob, pool_hw)) != VDSA_OK) return s;
  if (!flops) return fail(VDSA_ERR_NULL, "flops is NULL");
  *flops = 4.0 * prob->head_dim * prob->batch * prob->heads * (double)n_tokens(prob) *
           (double)pooled_tokens(prob, pool_hw);
  return ok();
}

}  // extern "C"
