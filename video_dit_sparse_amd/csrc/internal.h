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
  int32_t qblocks;            // query blocks per tile
  int32_t variant;            // which kernel shape the launcher runs (set by the host)
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
};
enum { MERGE_NONE = 0, MERGE_GATED = 1, MERGE_LSE = 2 };

struct PoolParams {
  const void* x;
  void* y;
  int64_t x_sb, x_sh, x_sn;
  int64_t y_sb, y_sh, y_sn;
  int32_t batch, heads, head_dim;
  int32_t T, H, W;
  int32_t kh, kw;
  int32_t Hp, Wp;
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

}  // namespace vdsa
