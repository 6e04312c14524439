// Device helpers shared by the attention kernels: key-box geometry of a query
// tile, XCD-aware workgroup numbering, division by invariants.
#pragma once

#include "internal.h"

namespace vdsa {

// Max over the two 32-lane halves of a wave (lanes l and l ^ 32), on the
// vector ALU: v_permlane32_swap with both operands x hands every lane both
// halves' values.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Max / sum over the four 16-lane rows of a wave (lanes l % 16 + 16 G):
// v_permlane16_swap pairs rows (0,1) and (2,3), then the 32-lane swap pairs
// the halves.
__device__ __forceinline__ float xrow4_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float xrow4_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
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

__device__ __forceinline__ void tile_boxes(const BoxAttnParams& p, int tile, Box& qb, Box& kb) {
  const int aw = tile % p.nW;
  const int ah = (tile / p.nW) % p.nH;
  const int at = tile / (p.nW * p.nH);
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
    auto wspan = [](int a, int r, int n, int b, int s, int L, int& lo, int& ext) {
      const int c0 = max(0, a - r), c1 = min(n - 1, a + r);
      lo = max(0, c0 * b - s);
      ext = min(L, (c1 + 1) * b - s) - lo;
    };
    wspan(at, p.rT, p.nT, p.bT, p.sT, p.qT, kb.t0, kb.et);
    wspan(ah, p.rH, p.nH, p.bH, p.sH, p.qH, kb.h0, kb.eh);
    wspan(aw, p.rW, p.nW, p.bW, p.sW, p.qW, kb.w0, kb.ew);
  }
}


}  // namespace vdsa
