/*
 * vdsa.h - tile-window sparse attention for video latents on MI355X (gfx950).
 *
 * C ABI of libvdsa.so.  Plain pointers, sizes and small descriptor structs; no
 * C++ or framework types cross it.
 *
 * The problem these calls solve:
 *   A video latent of T x H x W positions is a sequence of N = T*H*W tokens in
 *   raster order n = (t*H + h)*W + w (UltraGen, arXiv 2510.18775, summary
 *   section 3 "Preliminaries").  Each of Q, K, V, O is logically
 *   [batch, heads, N, head_dim] with head_dim contiguous; the batch, head and
 *   token strides are free (BHND and BNHD storage both work).
 *
 * Conventions shared by every call:
 *   - Memory is caller-owned device memory.  No call allocates, frees or
 *     keeps a pointer after it returns.
 *   - Every argument check runs on the host before anything is enqueued.  On
 *     error nothing is launched, outputs are untouched, a status is returned
 *     and vdsa_last_error() describes it.  Nothing aborts; no exception
 *     crosses the ABI.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  A fault during a kernel surfaces at the caller's next
 *     synchronisation, as with any HIP launch.
 *   - Calls are thread-safe (no global mutable state except a thread-local
 *     error string).
 *   - dtype VDSA_BF16: bf16 inputs and outputs (upper 16 bits of IEEE fp32),
 *     fp32 accumulation and fp32 softmax.  VDSA_F32: fp32 throughout.
 *   - Alignment: every tensor pointer 16-byte aligned; every batch, head and
 *     token stride times the element size a multiple of 16 bytes.
 *   - Size limit: within one (batch, head), the largest byte offset
 *     ((N-1)*stride_n + head_dim) * element size must be below 2^32.
 *   - Inputs must be finite.  The kernels are built without NaN handling in
 *     their maximum operations, so a NaN or infinity in Q, K, V or the gate
 *     gives unspecified (possibly non-NaN) outputs for the rows it reaches;
 *     it is never an error and never faults.
 */
#ifndef VDSA_H
#define VDSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VDSA_ABI_VERSION 5

typedef enum {
  VDSA_OK = 0,
  VDSA_ERR_NULL = 1,        /* a required pointer is NULL */
  VDSA_ERR_SHAPE = 2,       /* a dimension <= 0, or an offset beyond the size limit */
  VDSA_ERR_WINDOW = 3,      /* tile < 1, window even or < 1, shift outside [0, tile), pool < 1,
                               unknown window_mode */
  VDSA_ERR_UNSUPPORTED = 4, /* head_dim not in {64, 128}, unknown dtype, scale not finite or < 0 */
  VDSA_ERR_ALIGN = 5,       /* pointer or stride breaks the 16-byte rule */
  VDSA_ERR_ALIAS = 6,       /* an output overlaps an input it must not overlap */
  VDSA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than the reported size */
  VDSA_ERR_HIP = 8          /* the HIP runtime rejected a launch */
} vdsa_status;

typedef enum { VDSA_F32 = 0, VDSA_BF16 = 1 } vdsa_dtype;

/* Element strides of a [batch, heads, N, head_dim] view; head_dim stride is 1. */
typedef struct {
  int64_t b, h, n;
} vdsa_strides;

typedef struct {
  int32_t batch, heads, head_dim;   /* head_dim in {64, 128} */
  int32_t grid_t, grid_h, grid_w;   /* N = grid_t * grid_h * grid_w */
  vdsa_dtype dtype;
  float scale;                      /* logits = scale * (q . k); finite, >= 0 */
} vdsa_problem;

/*
 * Sliding-tile configuration, all in tokens except `window` (in tiles).
 *   tile[d]   >= 1: tile extent per dim (t, h, w).
 *   window[d] odd >= 1: a query tile attends the key tiles whose tile index
 *             differs from its own by at most (window[d]-1)/2 in every dim,
 *             clipped at the grid edge (Sliding Tile Attention, arXiv
 *             2502.04507, abstract: tile-by-tile attention over a local 3D
 *             window of tiles).  window[d] >= 2*tiles[d]-1 in every dim is
 *             full attention.
 *   shift[d]  in [0, tile[d]): tile index of coordinate x is
 *             floor((x + shift) / tile), a non-cyclic offset of the tile
 *             lattice that makes edge tiles partial (the shifted partition of
 *             UltraGen section 4.3, "Cross-window Hierarchical Local
 *             Attention").  Partial tiles hold only real tokens.  Under
 *             VDSA_WINDOW_CYCLIC the shift is a cyclic roll instead (below).
 *   window_mode (vdsa_window_mode) how windows meet the grid edge; 0 (the
 *             value of a zero-initialised struct) is VDSA_WINDOW_CLIP.
 */
typedef enum {
  /* windows clipped at the lattice edge (the definition above) */
  VDSA_WINDOW_CLIP = 0,
  /* every window spans min(window[d], tiles[d]) tiles: a window that would
   * cross the lattice edge is moved inward, so its first tile along d is
   * max(0, min(a - r, tiles[d] - window[d])) for query tile a, r =
   * (window[d]-1)/2 (the other reading of the edge rule, which the Sliding
   * Tile Attention abstract leaves open) */
  VDSA_WINDOW_INWARD = 1,
  /* the token grid is rolled cyclically before tiling: the token at x lands
   * at (x + shift[d]) mod L_d, the rolled grid is tiled from 0 and windows
   * are clipped there (the cyclic shift of Swin windows, the local module
   * UltraGen's ablation swaps in, section 5.3 and appendix F; no seam mask,
   * so tiles at the seam mix tokens of both grid edges) */
  VDSA_WINDOW_CYCLIC = 2
} vdsa_window_mode;

typedef struct {
  int32_t tile[3];
  int32_t window[3];
  int32_t shift[3];
  int32_t window_mode;
} vdsa_sta_cfg;

/*
 * sta_attn_fwd - sliding-tile 3D attention (local branch).
 *
 * For every (b, h, query token n):
 *   O[n] = sum_m softmax_m(scale * Q[n].K[m]) V[m]
 * over the keys m whose tile is inside the window of n's tile, under
 * cfg->window_mode (tiles and windows of the rolled grid for
 * VDSA_WINDOW_CYCLIC; O and LSE stay in the caller's token order).  The
 * window map is computed in-kernel; no mask is materialised.
 *
 *   q, k, v : device, [batch, heads, N, head_dim] with the given strides.
 *   o       : device output, same shape; must not overlap q, k, v or lse.
 *   lse     : optional device output (NULL to skip), fp32 [batch, heads, N]
 *             contiguous: natural-log sum of exp(scale * q.k) over the window.
 * Errors: VDSA_ERR_NULL, _SHAPE, _WINDOW, _UNSUPPORTED, _ALIGN, _ALIAS, _HIP.
 */
vdsa_status sta_attn_fwd(const vdsa_problem* prob, const vdsa_sta_cfg* cfg,
                         const void* q, const vdsa_strides* q_strides,
                         const void* k, const vdsa_strides* k_strides,
                         const void* v, const vdsa_strides* v_strides,
                         void* o, const vdsa_strides* o_strides,
                         float* lse, void* stream);

/*
 * global_pooled_attn_workspace_size - bytes of device workspace that
 * global_pooled_attn_fwd needs for `prob` and `pool_hw` (pooled K and V).
 */
vdsa_status global_pooled_attn_workspace_size(const vdsa_problem* prob, const int32_t pool_hw[2],
                                              size_t* bytes);

/*
 * global_pooled_attn_fwd - compressed global branch.
 *
 * K and V are average-pooled pool_hw[0] x pool_hw[1] within each frame
 * (frames are not pooled; a cell past the frame edge averages its real
 * tokens only), giving M = T * ceil(H/ph) * ceil(W/pw) pooled tokens in raster
 * order; then every full-resolution query attends all M pooled keys, unmasked:
 *   O[n] = sum_m softmax_m(scale * Q[n].Kp[m]) Vp[m].
 * (UltraGen section 4.2 "Spatially-Compressed Global Attention": frame-wise
 * stride-k compression before attention, here with uniform 1/(ph*pw)
 * weights; AtlasVid, arXiv 2605.16649, abstract: asymmetric global-local
 * attention, i.e. queries stay at full resolution.)  Pooled K/V are stored in
 * the I/O dtype in `workspace`.
 *
 *   workspace : device, at least global_pooled_attn_workspace_size() bytes,
 *               16-byte aligned, not overlapping any tensor argument.  Its
 *               contents after the call are the pooled K then pooled V,
 *               each [batch, heads, M, head_dim] contiguous.
 * Errors: as sta_attn_fwd, plus VDSA_ERR_WORKSPACE.
 */
vdsa_status global_pooled_attn_fwd(const vdsa_problem* prob, const int32_t pool_hw[2],
                                   const void* q, const vdsa_strides* q_strides,
                                   const void* k, const vdsa_strides* k_strides,
                                   const void* v, const vdsa_strides* v_strides,
                                   void* o, const vdsa_strides* o_strides,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Size of the static device scratch of global_pooled_attn_fwd_noalloc. */
#define VDSA_STATIC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * global_pooled_attn_fwd_noalloc - global_pooled_attn_fwd without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Computes exactly what global_pooled_attn_fwd computes (the same kernels) but
 * keeps the pooled K and V in a static device array of
 * VDSA_STATIC_SCRATCH_BYTES (128 MiB) that the library owns: one copy per
 * GPU, held from the first use of the library's device code on that GPU
 * until the process ends.  It calls no hipMalloc, hipFree or other
 * allocating routine.  The scratch of the calling thread's current device is
 * used, so `stream` must belong to that device; its address is resolved on
 * the first call on each device (make that first call outside graph
 * capture).  Every call on one GPU shares that GPU's scratch and leaves its
 * pooled K/V there; calls that overlap in time on one GPU (other streams,
 * other threads) race on it and must be serialised by the caller.  Nothing in
 * it needs to start at zero: the pooling writes every byte the attention
 * then reads.
 *
 * Errors: as global_pooled_attn_fwd; VDSA_ERR_WORKSPACE (before anything is
 * launched) when the pooled K and V, 2 * round_up(batch * heads * M *
 * head_dim * esize, 256) bytes, exceed VDSA_STATIC_SCRATCH_BYTES.
 */
vdsa_status global_pooled_attn_fwd_noalloc(const vdsa_problem* prob, const int32_t pool_hw[2],
                                           const void* q, const vdsa_strides* q_strides,
                                           const void* k, const vdsa_strides* k_strides,
                                           const void* v, const vdsa_strides* v_strides,
                                           void* o, const vdsa_strides* o_strides,
                                           float* lse, void* stream);

/*
 * dual_branch_merge - gated sum of the two branch outputs (UltraGen section
 * 4.1 "Time-Aware Global-Local Attention": a fusion factor combines the local
 * and the global latent; here one factor per head):
 *   out[b,h,n,:] = w_local[h] * o_local[b,h,n,:] + w_global[h] * o_global[b,h,n,:]
 *
 *   w_local  : device fp32 [heads], or NULL for all ones.
 *   w_global : device fp32 [heads].
 *   out      : may be exactly o_local (same pointer and strides, in place);
 *              must not otherwise overlap o_local or o_global.
 * Errors: VDSA_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIGN, _ALIAS, _HIP.
 */
vdsa_status dual_branch_merge(const vdsa_problem* prob,
                              const void* o_local, const vdsa_strides* local_strides,
                              const void* o_global, const vdsa_strides* global_strides,
                              const float* w_local, const float* w_global,
                              void* out, const vdsa_strides* out_strides, void* stream);

/*
 * How two branch outputs are combined (UltraGen section 4.1 "Time-Aware
 * Global-Local Attention" fuses the local and the global latent):
 *   VDSA_MERGE_GATED: out = w_local[h] * o_local + w_global[h] * o_global, the
 *                     per-head gate of dual_branch_merge;
 *   VDSA_MERGE_LSE:   one softmax over the union of both branches' key sets,
 *                     from their log-sum-exps (natural log):
 *                       a = 1 / (1 + exp(lse_global - lse_local)),
 *                       out = a * o_local + (1 - a) * o_global,
 *                       lse = log(exp(lse_local) + exp(lse_global)).
 *                     Exact when the key sets are disjoint (window tokens vs
 *                     pooled tokens).
 */
typedef enum {
  VDSA_MERGE_GATED = 0,
  VDSA_MERGE_LSE = 1
} vdsa_merge_mode;

/*
 * dual_branch_merge_lse - the VDSA_MERGE_LSE combination of two attention
 * outputs given their log-sum-exps.
 *
 *   lse_local, lse_global : device fp32 [batch, heads, N] contiguous (as
 *                           written by sta_attn_fwd / global_pooled_attn_fwd).
 *   out                   : may be exactly o_local or exactly o_global (same
 *                           pointer and strides); must not otherwise overlap them.
 *   lse_out               : nullable, [batch, heads, N] fp32 contiguous; may be
 *                           exactly lse_local or lse_global; must not otherwise
 *                           overlap any argument.
 * Errors: VDSA_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIGN, _ALIAS, _HIP.
 */
vdsa_status dual_branch_merge_lse(const vdsa_problem* prob,
                                  const void* o_local, const vdsa_strides* local_strides,
                                  const float* lse_local,
                                  const void* o_global, const vdsa_strides* global_strides,
                                  const float* lse_global,
                                  void* out, const vdsa_strides* out_strides, float* lse_out,
                                  void* stream);

/*
 * global_pooled_attn_merge_fwd - global_pooled_attn_fwd with the merge of
 * `mode` fused into the attention epilogue: the global branch's output never
 * reaches memory; each query row reads o_local (and lse_local) and writes the
 * merged row, saving the separate merge pass (one read and one write of a
 * [batch, heads, N, head_dim] tensor).
 *
 *   mode       : VDSA_MERGE_GATED (w_global required, w_local nullable =>
 *                ones; lse_local ignored) or VDSA_MERGE_LSE (lse_local
 *                required, w_* ignored).
 *   o_local    : the local branch output, [batch, heads, N, head_dim] in the
 *                problem dtype.
 *   lse_local  : device fp32 [batch, heads, N] contiguous.
 *   out        : may be exactly o_local (same pointer and strides); must not
 *                otherwise overlap o_local, and must not overlap q, k, v or
 *                the workspace.
 *   lse_out    : nullable, [batch, heads, N] fp32 contiguous: the merged LSE
 *                in LSE mode, the global branch's LSE in GATED mode.  May be
 *                exactly lse_local.
 *   workspace  : as global_pooled_attn_fwd (global_pooled_attn_workspace_size).
 * Errors: as global_pooled_attn_fwd.
 */
vdsa_status global_pooled_attn_merge_fwd(const vdsa_problem* prob, const int32_t pool_hw[2],
                                         const void* q, const vdsa_strides* q_strides,
                                         const void* k, const vdsa_strides* k_strides,
                                         const void* v, const vdsa_strides* v_strides,
                                         vdsa_merge_mode mode,
                                         const void* o_local, const vdsa_strides* local_strides,
                                         const float* lse_local,
                                         const float* w_local, const float* w_global,
                                         void* out, const vdsa_strides* out_strides, float* lse_out,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * hier_pooled_attn_fwd - intermediate-scale windowed attention (UltraGen
 * section 4.3 "Cross-window Hierarchical Local Attention": attention over
 * coarse windows; its cost term in App. B "Efficiency Analysis" is that of
 * full-resolution queries against 2x2-pooled keys within each window).  Each
 * query attends the pooled K/V (pool_hw = [ph, pw] cell means within each
 * frame, as global_pooled_attn_fwd) of every pooling cell that holds a token
 * of its sliding-tile window (cfg as in sta_attn_fwd, on the full grid):
 *   O[n] = sum_c softmax_c(scale * Q[n].Kp[c]) Vp[c],  c over those cells.
 * With tiles and shifts that are multiples of the pooling these are exactly
 * the pooled tokens of the window.  cfg->window_mode must be
 * VDSA_WINDOW_CLIP (VDSA_ERR_WINDOW otherwise).
 *
 *   workspace : at least hier_pooled_attn_workspace_size() bytes (pooled K
 *               then pooled V, as in global_pooled_attn_fwd).
 * Errors: as sta_attn_fwd and global_pooled_attn_fwd.
 */
vdsa_status hier_pooled_attn_workspace_size(const vdsa_problem* prob, const int32_t pool_hw[2], size_t* bytes);
vdsa_status hier_pooled_attn_fwd(const vdsa_problem* prob, const vdsa_sta_cfg* cfg, const int32_t pool_hw[2],
                                 const void* q, const vdsa_strides* q_strides,
                                 const void* k, const vdsa_strides* k_strides,
                                 const void* v, const vdsa_strides* v_strides,
                                 void* o, const vdsa_strides* o_strides, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * compressed_global_attn_fwd - UltraGen's own compressed global attention
 * (section 4.2 "Spatially-Compressed Global Attention"; App. B's
 * (THW)^2 D / K^4 term): Q, K and V pooled pool_hw within each frame, full
 * attention among the pooled tokens, then frame-wise bilinear upsampling of
 * the pooled output back to the grid (half-pixel sample positions, edge rows
 * and columns repeated; the pages' learned 3D convolution after it is not
 * part of this call).
 *
 *   workspace : at least compressed_global_attn_workspace_size() bytes
 *               (pooled Q, K, V and the pooled output).
 * Errors: as global_pooled_attn_fwd.
 */
vdsa_status compressed_global_attn_workspace_size(const vdsa_problem* prob, const int32_t pool_hw[2],
                                                  size_t* bytes);
vdsa_status compressed_global_attn_fwd(const vdsa_problem* prob, const int32_t pool_hw[2],
                                       const void* q, const vdsa_strides* q_strides,
                                       const void* k, const vdsa_strides* k_strides,
                                       const void* v, const vdsa_strides* v_strides,
                                       void* o, const vdsa_strides* o_strides,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward passes.  Gradients of a forward call's output O given dO, from the
 * forward's inputs, its output O and its LSE (natural log, as written by the
 * forward's `lse` argument).  With P the attention weights of a query row:
 *   delta = rowsum(dO * O),  dS = P * (dO.V^T - delta),
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
 * summed over every query whose keys include the key (the softmax Jacobian
 * of the definitions above).  Gradients are written (not accumulated) in the
 * problem dtype with fp32 accumulation.  bf16 supports head_dim 128; fp32
 * supports 64 and 128 (VDSA_ERR_UNSUPPORTED otherwise).
 *
 *   workspace : device, at least *_bwd_workspace_size() bytes, 16-byte
 *               aligned, not overlapping any argument.
 *   dq, dk, dv: must not overlap each other, any input, lse or the workspace.
 * Errors: as the forward call, plus VDSA_ERR_WORKSPACE.
 */
vdsa_status sta_attn_bwd_workspace_size(const vdsa_problem* prob, size_t* bytes);
vdsa_status sta_attn_bwd(const vdsa_problem* prob, const vdsa_sta_cfg* cfg,
                         const void* q, const vdsa_strides* q_strides,
                         const void* k, const vdsa_strides* k_strides,
                         const void* v, const vdsa_strides* v_strides,
                         const void* o, const vdsa_strides* o_strides,
                         const void* d_o, const vdsa_strides* do_strides,
                         const float* lse,
                         void* dq, const vdsa_strides* dq_strides,
                         void* dk, const vdsa_strides* dk_strides,
                         void* dv, const vdsa_strides* dv_strides,
                         void* workspace, size_t workspace_bytes, void* stream);

/* The global branch's backward, through the pooling: the pooled K and V get
 * their gradients as above (every query attends every pooled token), then
 * every token of a pooling cell receives its cell's gradient divided by the
 * cell's token count (the derivative of the cell mean).  o and lse are the
 * outputs of global_pooled_attn_fwd (not of a fused merge call). */
vdsa_status global_pooled_attn_bwd_workspace_size(const vdsa_problem* prob, const int32_t pool_hw[2],
                                                  size_t* bytes);
vdsa_status global_pooled_attn_bwd(const vdsa_problem* prob, const int32_t pool_hw[2],
                                   const void* q, const vdsa_strides* q_strides,
                                   const void* k, const vdsa_strides* k_strides,
                                   const void* v, const vdsa_strides* v_strides,
                                   const void* o, const vdsa_strides* o_strides,
                                   const void* d_o, const vdsa_strides* do_strides,
                                   const float* lse,
                                   void* dq, const vdsa_strides* dq_strides,
                                   void* dk, const vdsa_strides* dk_strides,
                                   void* dv, const vdsa_strides* dv_strides,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_avgpool_fwd - the pooling step of global_pooled_attn_fwd on one tensor,
 * exported so it can be checked and timed alone.  x_pooled is
 * [batch, heads, M, head_dim] with its own strides; must not overlap x.
 */
vdsa_status kv_avgpool_fwd(const vdsa_problem* prob, const int32_t pool_hw[2],
                           const void* x, const vdsa_strides* x_strides,
                           void* x_pooled, const vdsa_strides* pooled_strides, void* stream);

/* Effective work: 4 * head_dim FLOP per attended (query, key) token pair
 * (2*head_dim for q.k, 2*head_dim for p*v), summed over batch and heads;
 * partial tiles count their real tokens only; vdsa_sta_flops follows
 * cfg->window_mode.  Host only. */
vdsa_status vdsa_sta_flops(const vdsa_problem* prob, const vdsa_sta_cfg* cfg, double* flops);
vdsa_status vdsa_global_flops(const vdsa_problem* prob, const int32_t pool_hw[2], double* flops);
/* hier_pooled_attn_fwd: 4 * head_dim per (query, pooled cell of its window);
 * compressed_global_attn_fwd: 4 * head_dim per (pooled query, pooled key). */
vdsa_status vdsa_hier_flops(const vdsa_problem* prob, const vdsa_sta_cfg* cfg, const int32_t pool_hw[2],
                            double* flops);
vdsa_status vdsa_compressed_global_flops(const vdsa_problem* prob, const int32_t pool_hw[2], double* flops);

/* Name of the kernel sta_attn_fwd launches for this problem and
 * configuration: the host picks among the attention kernels by head_dim and
 * by the largest query tile's token count (384-, 192- or 128-query
 * workgroups, whichever pads the tiles least; fp32 inputs take the fp32
 * kernel).  A static string; NULL, with vdsa_last_error set, when prob or
 * cfg is invalid.  Host only. */
const char* vdsa_sta_kernel(const vdsa_problem* prob, const vdsa_sta_cfg* cfg);

const char* vdsa_status_string(vdsa_status s);
const char* vdsa_last_error(void);   /* thread-local detail of the last failed call */
int vdsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VDSA_H */
