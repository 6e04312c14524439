// Device helpers shared by the attention kernels: key-box geometry of a query
// tile, XCD-aware workgroup numbering, division by invariants.
#pragma once

#include "internal.h"

namespace vdsa {

// Vector types of MFMA operands and accumulators and of 8- and 16-byte
// memory chunks; LDS pointer types for direct global->LDS loads and 4-byte
// LDS stores.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
// raw buffer resource word 3 for gfx9-class parts (32-bit data format)
constexpr int BUF_FLAGS = 0x00020000;

// One 16-byte MFMA operand fragment read from LDS.
__device__ __forceinline__ bf16x8 lds_frag(const char* p) { return __builtin_bit_cast(bf16x8, *(const u32x4*)p); }

// Empty asm statements that claim to rewrite their operands: the values are
// computed before this point, so the work of a phase cannot sink into the
// next one across the kernels' phase barriers.
__device__ __forceinline__ void pin(f32x4& a) { asm volatile("" : "+v"(a)); }
__device__ __forceinline__ void pin(f32x4& a, f32x4& b, f32x4& c) { asm volatile("" : "+v"(a), "+v"(b), "+v"(c)); }
__device__ __forceinline__ void pin(float& a, float& b, float& c) { asm volatile("" : "+v"(a), "+v"(b), "+v"(c)); }
__device__ __forceinline__ void pin(bf16x8& x) {
  u32x4 u = __builtin_bit_cast(u32x4, x);
  asm volatile("" : "+v"(u));
  x = __builtin_bit_cast(bf16x8, u);
}

// Max over the two 32-lane halves of a wave (lanes l and l ^ 32), on the
// vector ALU: v_permlane32_swap with both operands x hands every lane both
// halves' values.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Max over the four 16-lane rows of a wave (lanes l % 16 + 16 G):
// v_permlane16_swap pairs rows (0,1) and (2,3), then the 32-lane swap pairs
// the halves.
__device__ __forceinline__ float xrow4_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Weights of the epilogue merge for one query row: out = wa * o_other +
// wb * o_this, where o_this is the kernel's normalised output row and
// lse_this its log-sum-exp (natural log).  lse is the row's merged LSE (LSE
// mode) or lse_this (gated mode).
struct RowMerge {
  float wa, wb, lse;
};
__device__ __forceinline__ RowMerge row_merge(const BoxAttnParams& p, int b, int h, uint32_t tok, float lse_this) {
  RowMerge r{0.f, 1.f, lse_this};
  if (p.merge == MERGE_GATED) {
    r.wa = p.w_l != nullptr ? p.w_l[h] : 1.f;
    r.wb = p.w_g[h];
  } else if (p.merge == MERGE_LSE) {
    constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.69314718055994531f;
    const int64_t N = (int64_t)p.qT * p.qH * p.qW;
    const float la = p.lse_l[((int64_t)b * p.heads + h) * N + tok];
    const float m = fmaxf(la, lse_this);
    const float ea = __builtin_amdgcn_exp2f((la - m) * LOG2E);
    const float eb = __builtin_amdgcn_exp2f((lse_this - m) * LOG2E);
    const float z = ea + eb;
    r.wa = ea / z;
    r.wb = eb / z;
    r.lse = m + __builtin_amdgcn_logf(z) * LN2;
  }
  return r;
}

// Four bf16 (packed in two dwords) to fp32.
__device__ __forceinline__ void bf16x4_to_f32(uint32_t lo, uint32_t hi, float (&f)[4]) {
  f[0] = __uint_as_float(lo << 16);
  f[1] = __uint_as_float(lo & 0xFFFF0000u);
  f[2] = __uint_as_float(hi << 16);
  f[3] = __uint_as_float(hi & 0xFFFF0000u);
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// s_waitcnt immediate: vmcnt(vm), lgkmcnt(lgkm), expcnt untouched
__device__ __forceinline__ constexpr int wait_enc(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// Phase boundary of the kernels whose two wave groups alternate matrix-core
// and vector phases: this wave's LDS accesses are complete, then a workgroup
// barrier.  Outstanding global loads stay in flight.  Neither the compiler's
// scheduler nor its memory optimisations move work across it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(wait_enc(63, 0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The hardware hands workgroup i to XCD i % 8.  Renumber so that consecutive
// logical ids (the query blocks of one tile, then neighbouring tiles, whose
// key boxes overlap) run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int hw, int total) {
  constexpr int NX = 8;
  const int per = total / NX, extra = total % NX;
  const int xcd = hw % NX, slot = hw / NX;
  const int base = xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per;
  return base + slot;
}

struct Box {
  int t0, h0, w0, et, eh, ew;
};

// Token index of box coordinate (t, h, w) on the query grid / the key grid.
// Boxes live in the rolled grid when the window mode is cyclic (rl != 0):
// rolled coordinate x holds the token at (x - rl) mod L.
__device__ __forceinline__ int unroll(int x, int rl, int L) { return x - rl + (x < rl ? L : 0); }
__device__ __forceinline__ uint32_t q_token(const BoxAttnParams& p, int t, int h, int w) {
  return (uint32_t)((unroll(t, p.rlT, p.qT) * p.qH + unroll(h, p.rlH, p.qH)) * p.qW + unroll(w, p.rlW, p.qW));
}
__device__ __forceinline__ uint32_t k_token(const BoxAttnParams& p, int t, int h, int w) {
  return (uint32_t)((unroll(t, p.rlT, p.kT) * p.kH + unroll(h, p.rlH, p.kH)) * p.kW + unroll(w, p.rlW, p.kW));
}

// Key j of a key box (extent ew along w, plane = eh * ew tokens) -> token, in
// full-rate 24-bit multiplies.  Valid when the key grid has fewer than 2^24
// tokens, which the 32-bit byte-offset bound guarantees for head_dim 128 in
// bf16 (a key row is at least 256 bytes).
__device__ __forceinline__ uint32_t box_key_token24(const BoxAttnParams& p, const Box& kb, uint32_t j,
                                                    const FastDiv& fd_plane, const FastDiv& fd_row) {
  const uint32_t jt = fast_div(j, fd_plane);
  const uint32_t r = j - __umul24(jt, fd_plane.d);
  const uint32_t jh = fast_div(r, fd_row);
  const uint32_t jw = r - __umul24(jh, fd_row.d);
  const uint32_t t = (uint32_t)unroll(kb.t0 + (int)jt, p.rlT, p.kT);
  const uint32_t h = (uint32_t)unroll(kb.h0 + (int)jh, p.rlH, p.kH);
  const uint32_t w = (uint32_t)unroll(kb.w0 + (int)jw, p.rlW, p.kW);
  return __umul24(__umul24(t, (uint32_t)p.kH) + h, (uint32_t)p.kW) + w;
}

// Query box of tile (at, ah, aw) of the lattice and the box of its keys.
// (PT: BoxAttnParams, in whichever address space the caller reads it from.)
template <class PT>
__device__ __forceinline__ void tile_boxes_at(const PT& p, int at, int ah, int aw, Box& qb, Box& kb) {
  auto span = [](int a, int b, int s, int L, int& lo, int& ext) {
    lo = max(0, a * b - s);
    ext = min(L, (a + 1) * b - s) - lo;
  };
  span(at, p.bT, p.sT, p.qT, qb.t0, qb.et);
  span(ah, p.bH, p.sH, p.qH, qb.h0, qb.eh);
  span(aw, p.bW, p.sW, p.qW, qb.w0, qb.ew);
  if (p.dense_keys) {
    kb = Box{0, 0, 0, p.kT, p.kH, p.kW};
  } else {
    auto wspan = [&](int a, int r, int n, int b, int s, int L, int& lo, int& ext) {
      int c0, c1;
      window_range(a, r, n, p.wmode, c0, c1);
      lo = max(0, c0 * b - s);
      ext = min(L, (c1 + 1) * b - s) - lo;
    };
    wspan(at, p.rT, p.nT, p.bT, p.sT, p.qT, kb.t0, kb.et);
    wspan(ah, p.rH, p.nH, p.bH, p.sH, p.qH, kb.h0, kb.eh);
    wspan(aw, p.rW, p.nW, p.bW, p.sW, p.qW, kb.w0, kb.ew);
    if (p.kpT > 1 || p.kpH > 1 || p.kpW > 1) {
      // keys pooled k x k: the cells holding a token of the window box
      auto cells = [](int k, int& lo, int& ext) {
        if (k <= 1) return;
        const int hi = lo + ext;
        lo /= k;
        ext = (hi + k - 1) / k - lo;
      };
      cells(p.kpT, kb.t0, kb.et);
      cells(p.kpH, kb.h0, kb.eh);
      cells(p.kpW, kb.w0, kb.ew);
    }
  }
}

__device__ __forceinline__ void tile_boxes(const BoxAttnParams& p, int tile, Box& qb, Box& kb) {
  tile_boxes_at(p, tile / (p.nW * p.nH), (tile / p.nW) % p.nH, tile % p.nW, qb, kb);
}

// Key walks of the 384- and 192-query kernels (BoxAttnParams::tile_walk):
//   WALK_RASTER        the key box in raster order, 64 consecutive keys per
//                      block (each lane's key token from two divisions by
//                      invariants, handed to the loading lanes by shuffles);
//   WALK_TILES         every tile of the lattice full, no lattice shift, 64
//                      tokens per tile frame: the box tile by tile (raster
//                      order of tiles), one frame of one tile per block, so a
//                      lane's rows sit at fixed token offsets from the block's
//                      first token;
//   WALK_TILES_ROLLED  the same on the rolled grid of the cyclic mode (uniform
//                      frame, per-lane unroll of h and w), visiting keys in
//                      the order the clipped walk visits rolled tensors;
//   WALK_LINEAR        dense keys (the box is the whole key grid, unrolled):
//                      key j is token j, so block b is tokens 64b .. 64b+63
//                      and a lane's rows again sit at fixed offsets.
enum { WALK_RASTER = 0, WALK_TILES = 1, WALK_TILES_ROLLED = 2, WALK_LINEAR = 3 };

// Cursor of a tile walk: the next block is frame f of key-box tile
// (tt, th, tw); the box is whole tiles, so its extents are multiples of the
// tile and its origin on tile boundaries.  Uniform over the workgroup.
struct TileCursor {
  int tt = 0, th = 0, tw = 0, f = 0;
  int n_th = 1, n_tw = 1;
  __device__ void init(const BoxAttnParams& p, const Box& kb) {
    n_th = kb.eh / p.bH;
    n_tw = kb.ew / p.bW;
  }
  // Rolled-grid coordinates of the next block's first token; then advance.
  __device__ void next(const BoxAttnParams& p, const Box& kb, int& t, int& h, int& w) {
    t = kb.t0 + tt * p.bT + f;
    h = kb.h0 + th * p.bH;
    w = kb.w0 + tw * p.bW;
    if (++f == p.bT) {
      f = 0;
      if (++tw == n_tw) {
        tw = 0;
        if (++th == n_th) {
          th = 0;
          ++tt;
        }
      }
    }
  }
};

// Token offset, within the key grid, of row r of a tile-frame block from the
// block's first token (tile width 2^w_log).
__device__ __forceinline__ int tile_row_offset(const BoxAttnParams& p, int r, int w_log) {
  return (r >> w_log) * p.kW + (r & (p.bW - 1));
}
// Token of row r of the tile-frame block at rolled (t, h, w), cyclic mode.
__device__ __forceinline__ uint32_t tile_row_token_rolled(const BoxAttnParams& p, int t, int h, int w, int r,
                                                          int w_log) {
  const int tu = unroll(t, p.rlT, p.kT);
  const int hu = unroll(h + (r >> w_log), p.rlH, p.kH);
  const int wu = unroll(w + (r & (p.bW - 1)), p.rlW, p.kW);
  return (uint32_t)((tu * p.kH + hu) * p.kW + wu);
}


}  // namespace vdsa
