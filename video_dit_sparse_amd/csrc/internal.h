// Internal interface between the host-side validation (api.cpp) and the
// kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdsa {

// Division by a runtime constant d >= 1, valid for 0 <= n < 2^31
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994): q = (umulhi(n, m) + n) >> s.
struct FastDiv {
  uint32_t d, m, s;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{d, uint32_t(m), s};
}

// The same constants for 1 <= d <= 2^31 without a 64-bit integer division
// (which kernels would expand into a long instruction sequence).  With
// r = 2^s - d < d, m - 1 = floor(r 2^32 / d) < 2^32.  r 2^32 (at most 32
// significant bits) and d are exact in double precision and the quotient is
// correctly rounded (error below 2^-21), so the truncated quotient is the
// floor or one off it; the integer check q d <= r 2^32 < (q + 1) d, whose
// products stay below 2^64, corrects it.
__host__ __device__ inline FastDiv make_fastdiv_fp64(uint32_t d) {
  uint32_t s = 0;
  while ((uint32_t(1) << s) < d) ++s;
  const uint64_t num = (uint64_t)((uint32_t(1) << s) - d) << 32;
  uint64_t q = (uint64_t)((double)num / (double)d);
  if (q * d > num) --q;
  else if ((q + 1) * d <= num) ++q;
  return FastDiv{d, uint32_t(q + 1), s};
}

// Per-dim description of the query tiling and of where the keys come from.
//
// Query side: the query grid (qT, qH, qW) is cut into tiles of (bT, bH, bW)
// tokens, lattice offset by (sT, sH, sW); there are (nT, nH, nW) tiles.
// Key side: either the tiles within radius (rT, rH, rW) of the query tile on
// the same grid (sliding-tile attention), or, with dense_keys, the whole key
// grid (kT, kH, kW) (global attention over pooled tokens).  Either way the
// keys of one query tile form a box of tokens.
struct BoxAttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;                 // nullable, [batch, heads, N] contiguous
  int64_t q_sb, q_sh, q_sn;   // element strides
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int32_t batch, heads;
  int32_t qT, qH, qW;
  int32_t bT, bH, bW;
  int32_t sT, sH, sW;
  int32_t nT, nH, nW;
  int32_t rT, rH, rW;
  int32_t kT, kH, kW;
  int32_t dense_keys;
  int32_t kpT, kpH, kpW;      // pooled keys (> 1): the key box is every k-grid cell holding
                              // a token of the window box; the k grid is the pooled grid
  int32_t wmode;              // WIN_CLIP / WIN_INWARD / WIN_INWARD_T (window_range)
  int32_t rlT, rlH, rlW;      // cyclic roll of the query and key grids (0: none): box
                              // coordinate x' is the token at (x' - rl) mod L
  int32_t qblocks;            // query blocks per tile
  int32_t variant;            // which kernel shape the launcher runs (set by the host)
  int32_t tile_walk;          // 384-query kernel's key walk: 0 raster, 1 whole tiles, 2 whole
                              // tiles of the rolled grid, 3 the whole key grid in token order
                              // (set by the host; see box_common.h)
  int32_t total_wg;           // batch * heads * tiles * qblocks
  float scale_log2e;          // scale * log2(e)
  // Optional merge with another branch's output in the epilogue (merge !=
  // MERGE_NONE): out row = wa * ol row + wb * this kernel's normalised row.
  int32_t merge;              // MERGE_NONE / MERGE_GATED / MERGE_LSE
  const void* ol;             // other branch output, same dtype, [batch, heads, N, D]
  int64_t ol_sb, ol_sh, ol_sn;
  const float* lse_l;         // MERGE_LSE: other branch LSE, [batch, heads, N] contiguous
  const float* w_l;           // MERGE_GATED: weight of ol per head (nullable => 1)
  const float* w_g;           // MERGE_GATED: weight of this kernel's output per head
  // Division by invariants for decoding a work-item index (set by the host):
  // by qblocks, by the tile count nT*nH*nW, by heads, by nW and by nH.
  FastDiv fd_qblocks, fd_tiles, fd_heads, fd_nw, fd_nh;
};
enum { MERGE_NONE = 0, MERGE_GATED = 1, MERGE_LSE = 2 };

// How a window meets the lattice edge, per dim.  For query tile a of n tiles
// and radius r, [c0, c1] are the key tiles of its window:
//   WIN_CLIP:    [max(0, a - r), min(n - 1, a + r)];
//   WIN_INWARD:  the 2r+1 tiles (all n if fewer) starting at
//                clamp(a - r, 0, max(0, n - 2r - 1));
//   WIN_INWARD_T the transpose of WIN_INWARD: the query tiles whose inward
//                windows hold tile a.  The inward start is non-decreasing in
//                the query tile, so these form an interval: the start values
//                v in [max(0, a - 2r), min(m, a)], m = max(0, n - 2r - 1),
//                and the queries taking them (v = 0 for every query up to r,
//                v = m for every query from m + r on, else query v + r).
enum { WIN_CLIP = 0, WIN_INWARD = 1, WIN_INWARD_T = 2 };
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline void window_range(int a, int r, int n, int mode, int& c0, int& c1) {
  if (mode == WIN_INWARD) {
    c0 = imax(0, imin(a - r, n - (2 * r + 1)));
    c1 = imin(n - 1, c0 + 2 * r);
  } else if (mode == WIN_INWARD_T) {
    const int m = imax(0, n - (2 * r + 1));
    const int vlo = imax(0, a - 2 * r), vhi = imin(m, a);
    c0 = vlo == 0 ? 0 : vlo + r;
    c1 = vhi == m ? n - 1 : vhi + r;
  } else {
    c0 = imax(0, a - r);
    c1 = imin(n - 1, a + r);
  }
}

struct PoolParams {
  const void* x;
  void* y;
  int64_t x_sb, x_sh, x_sn;
  int64_t y_sb, y_sh, y_sn;
  int32_t batch, heads, head_dim;
  int32_t T, H, W;
  int32_t kh, kw;
  int32_t Hp, Wp;
  FastDiv fd_wp, fd_hp;   // division by Wp and Hp (pooled cell coordinates)
};

struct MergeParams {
  const void* a;
  const void* g;
  const float* w_a;   // nullable => 1
  const float* w_g;
  const float* lse_a; // lse_a and lse_g set: LSE merge (weights from them, w_* unused)
  const float* lse_g;
  float* lse_out;     // LSE merge only, nullable
  void* out;
  int64_t a_sb, a_sh, a_sn;
  int64_t g_sb, g_sh, g_sn;
  int64_t o_sb, o_sh, o_sn;
  int32_t batch, heads, head_dim;
  int64_t n_tokens;
};

// Backward pass of box attention.  `g` carries the geometry: the pass's own
// rows are cut into the tiles of g (qT.. / bT.. / sT.. / nT..), and each own
// tile iterates the box of tokens given by g's key side (rT.. or dense_keys
// over kT, kH, kW); g's pointers are unused.
//   dQ pass:    own rows = queries (Q, dO in registers), iterated = their key
//               boxes (K, V), exactly the forward's geometry.
//   dK/dV pass: own rows = keys (K, V in registers), iterated = the queries
//               whose windows contain the key tile.  The clipped window
//               relation |a - c| <= r is symmetric, so for sliding tiles this
//               is the box around the key tile on the same lattice (also in
//               the rolled grid of the cyclic mode); inward windows take the
//               transposed range (WIN_INWARD_T); for pooled keys (one tile
//               over the pooled grid) it is every query (dense_keys over the
//               query grid).
struct BoxBwdParams {
  BoxAttnParams g;
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;     // forward LSE (natural log), [batch, heads, n_q] contiguous
  const float* delta;   // rowsum(dO * O), [batch, heads, n_q] contiguous
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_sh, q_sn;   // element strides
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t do_sb, do_sh, do_sn;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  int64_t n_q;                // query tokens per head
  int64_t n_k;                // key tokens per head
  int32_t grad_f32;           // dK/dV pass: store fp32 gradients (else the I/O dtype)
  int32_t head_dim;
  float scale;                // softmax scale
};

// rowsum(dO * O) per row of [batch, heads, n, head_dim] tensors into
// delta [batch, heads, n] fp32 contiguous.
struct RowDotParams {
  const void* a;
  const void* b;
  float* out;
  int64_t a_sb, a_sh, a_sn;
  int64_t b_sb, b_sh, b_sn;
  int32_t batch, heads, head_dim;
  int64_t n;
};

// Gradient of k_h x k_w frame-wise average pooling: every token of a cell
// receives the cell's fp32 gradient divided by the cell's token count.
struct UnpoolParams {
  const float* gp;   // [batch, heads, M, head_dim] fp32 contiguous
  void* g;           // [batch, heads, N, head_dim] in the I/O dtype, strided
  int64_t g_sb, g_sh, g_sn;
  int32_t batch, heads, head_dim;
  int32_t T, H, W;
  int32_t kh, kw;
  int32_t Hp, Wp;
  FastDiv fd_hw, fd_w;    // division by H*W and W (a token's frame and row)
  FastDiv fd_kh, fd_kw;   // division by kh and kw (a token's cell)
};

// Frame-wise bilinear upsampling of a pooled tensor back to the grid
// (half-pixel sample positions, edge rows / columns repeated).
struct UpsampleParams {
  const void* xp;    // [batch, heads, T*Hp*Wp, head_dim] contiguous, I/O dtype
  void* out;         // [batch, heads, T*H*W, head_dim], strided
  int64_t o_sb, o_sh, o_sn;
  int32_t batch, heads, head_dim;
  int32_t T, H, W, Hp, Wp;
  FastDiv fd_hw, fd_w;    // division by H*W and W (a token's frame and row)
};

// The static device scratch of the entry point that allocates nothing
// (scratch.hip): STATIC_SCRATCH_BYTES on every device, 256-byte aligned.
// static_scratch() returns the current device's copy, resolving its address
// with hipGetSymbolAddress on the first call for that device.
constexpr size_t STATIC_SCRATCH_BYTES = size_t(128) << 20;
hipError_t static_scratch(void** ptr);

// Grid for per-slice work: the y index over the (batch, head) slices, at most
// max_wg workgroups of 256 threads in all (the kernels' loops stride over the
// rest).  pool_merge.hip.
dim3 slice_grid(int64_t slices, int64_t per_slice_work, int64_t max_wg);

// Launchers: return hipSuccess or the launch error.  They assume the
// parameters were validated.
hipError_t launch_box_attn_bf16(const BoxAttnParams& p, int head_dim, hipStream_t stream);
// head_dim 128 only, 48 queries per wave: 4 waves (192 queries per workgroup).
hipError_t launch_box_attn_bf16_m16(const BoxAttnParams& p, hipStream_t stream);
// head_dim 128 only, 48 queries per wave: 8 waves (384 queries per workgroup)
// in two groups whose matrix-core and softmax phases alternate.
hipError_t launch_box_attn_bf16_pp(const BoxAttnParams& p, hipStream_t stream);
hipError_t launch_box_attn_f32(const BoxAttnParams& p, int head_dim, hipStream_t stream);
hipError_t launch_avgpool(const PoolParams& p, int bf16, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, int bf16, hipStream_t stream);
hipError_t launch_upsample(const UpsampleParams& p, int bf16, hipStream_t stream);
// backward: bf16 head_dim 128 on the matrix cores, fp32 (head_dim 64, 128)
// on the vector ALU; grad_f32 applies to the fp32 kernel trivially
hipError_t launch_attn_bwd_dq(const BoxBwdParams& p, int bf16, hipStream_t stream);
hipError_t launch_attn_bwd_dkdv(const BoxBwdParams& p, int bf16, hipStream_t stream);
int attn_bwd_block_m(int bf16, bool kv);   // own rows per workgroup of the dQ or the dK/dV pass
hipError_t launch_rowdot(const RowDotParams& p, int bf16, hipStream_t stream);
hipError_t launch_unpool_grad(const UnpoolParams& p, int bf16, hipStream_t stream);

}  // namespace vdsa
