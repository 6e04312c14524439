// Memory-bound helpers of the global-local path:
//  * frame-wise k_h x k_w average pooling of K or V (UltraGen, arXiv
//    2510.18775, summary section 4.2: compression with stride k inside each
//    frame before global attention; here the stride-k depthwise convolution
//    with uniform weights, i.e. the cell mean);
//  * the per-head gated merge of the local and global outputs (UltraGen
//    summary section 4.1: a fusion factor combines the two branches).
//
// Both kernels move 16-byte chunks: one thread per (row, chunk), so 16
// (bf16, head_dim 128) consecutive threads cover one 256-byte row and a wave
// reads whole rows; accumulation is in fp32.  Each thread keeps several
// independent loads in flight (the taps of a pooling cell, or several merge
// chunks) so that HBM latency is covered without relying on occupancy alone.
// The streamed rows are read and written with nontemporal loads and stores:
// nothing re-reads them soon, and keeping them out of the caches' normal
// replacement raised the sustained rate by 5-14% (pooling about 6.1 TB/s).
#include "box_common.h"

namespace vdsa {
namespace {

constexpr int NTHREADS = 256;

template <bool BF16>
struct Chunk;

template <>
struct Chunk<true> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void unpack(const u32x4& u, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float* f) {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (__bf16)f[i];
    return __builtin_bit_cast(u32x4, b);
  }
};

template <>
struct Chunk<false> {
  static constexpr int E = 4;
  static __device__ __forceinline__ void unpack(const u32x4& u, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(u[i]);
  }
  static __device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = __float_as_uint(f[i]);
    return u;
  }
};

// The grid's y index walks the (batch, head) slices; within a slice, chunk i
// is pooled cell i / cpr, chunk i % cpr (cpr a power of two), and the cell's
// (t, i, j) come from divisions by invariants.
template <bool BF16>
__global__ __launch_bounds__(NTHREADS) void avgpool_kernel(const PoolParams p) {
  using C = Chunk<BF16>;
  constexpr int NF = 8;               // taps of a cell whose loads are in flight together
  const int cpr = p.head_dim / C::E;  // chunks per row
  const int cpr_log = __builtin_ctz((unsigned)cpr);
  const int M = p.T * p.Hp * p.Wp;
  const int64_t per_slice = (int64_t)M * cpr;
  const size_t esz = BF16 ? 2 : 4;
  const int64_t col_step = p.x_sn * (int64_t)esz, row_step = (int64_t)p.W * col_step;
  for (int bh = blockIdx.y; bh < p.batch * p.heads; bh += gridDim.y) {
    const int h = bh % p.heads, b = bh / p.heads;
    const char* xb = (const char*)p.x + (b * p.x_sb + h * p.x_sh) * (int64_t)esz;
    char* yb = (char*)p.y + (b * p.y_sb + h * p.y_sh) * (int64_t)esz;
    for (int64_t idx = (int64_t)blockIdx.x * NTHREADS + threadIdx.x; idx < per_slice;
         idx += (int64_t)gridDim.x * NTHREADS) {
      const int ch = (int)(idx & (cpr - 1));
      const uint32_t m = (uint32_t)(idx >> cpr_log);
      const uint32_t q = fast_div(m, p.fd_wp);   // t * Hp + i
      const int j = (int)(m - q * (uint32_t)p.Wp);
      const uint32_t t = fast_div(q, p.fd_hp);
      const int i = (int)(q - t * (uint32_t)p.Hp);
      const int h0 = i * p.kh, h1 = min(p.H, h0 + p.kh);
      const int w0 = j * p.kw, w1 = min(p.W, w0 + p.kw);
      const int nw = w1 - w0, ntap = (h1 - h0) * nw;
      // the cell's first token; taps in row-major order, NF loads issued before their adds
      const char* cell = xb + ch * 16 + (((int64_t)t * p.H + h0) * p.W + w0) * col_step;
      float acc[C::E];
#pragma unroll
      for (int e = 0; e < C::E; ++e) acc[e] = 0.f;
      int dh = 0, dw = 0;
      for (int c0 = 0; c0 < ntap; c0 += NF) {
        u32x4 u[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (c0 + f < ntap) u[f] = __builtin_nontemporal_load((const u32x4*)(cell + dh * row_step + dw * col_step));
          if (++dw == nw) {
            dw = 0;
            ++dh;
          }
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (c0 + f < ntap) {
            float x[C::E];
            C::unpack(u[f], x);
#pragma unroll
            for (int e = 0; e < C::E; ++e) acc[e] += x[e];
          }
        }
      }
      const float inv = 1.f / (float)ntap;
#pragma unroll
      for (int e = 0; e < C::E; ++e) acc[e] *= inv;
      __builtin_nontemporal_store(C::pack(acc), (u32x4*)(yb + (int64_t)m * p.y_sn * (int64_t)esz + ch * 16));
    }
  }
}

// The grid's y index walks the (batch, head) slices, so batch, head and the
// gates are uniform per workgroup; within a slice, chunk i of the slice is
// token i / cpr, chunk i % cpr (cpr a power of two: a shift and a mask).  Each
// thread takes MU chunks, one grid stride apart, and issues all their loads
// before the arithmetic.  One chunk per thread over a grid that covers the
// slice keeps the most requests in flight: 8% faster on the 720P tensors than
// four chunks per thread over a quarter of the grid, and faster than two or
// eight.
constexpr int MU = 1;

template <bool BF16>
__global__ __launch_bounds__(NTHREADS) void merge_kernel(const MergeParams p) {
  using C = Chunk<BF16>;
  const int cpr = p.head_dim / C::E;
  const int cpr_log = __builtin_ctz((unsigned)cpr);
  const int64_t per_slice = p.n_tokens * cpr;
  const size_t esz = BF16 ? 2 : 4;
  const int64_t a_row = p.a_sn * (int64_t)esz, g_row = p.g_sn * (int64_t)esz, o_row = p.o_sn * (int64_t)esz;
  const bool lse_mode = p.lse_a != nullptr;
  const int64_t stride = (int64_t)gridDim.x * NTHREADS;
  for (int bh = blockIdx.y; bh < p.batch * p.heads; bh += gridDim.y) {
    const int h = bh % p.heads, b = bh / p.heads;
    const char* ab = (const char*)p.a + (b * p.a_sb + h * p.a_sh) * (int64_t)esz;
    const char* gb = (const char*)p.g + (b * p.g_sb + h * p.g_sh) * (int64_t)esz;
    char* ob = (char*)p.out + (b * p.o_sb + h * p.o_sh) * (int64_t)esz;
    const int64_t row0 = (int64_t)bh * p.n_tokens;   // the slice's first row of the LSE arrays
    const float wa_gate = lse_mode ? 0.f : (p.w_a ? p.w_a[h] : 1.f);
    const float wg_gate = lse_mode ? 0.f : p.w_g[h];
    for (int64_t i0 = (int64_t)blockIdx.x * NTHREADS + threadIdx.x; i0 < per_slice; i0 += MU * stride) {
      u32x4 ua[MU], ug[MU];
      float la[MU], lg[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int64_t idx = i0 + u * stride;
        if (idx < per_slice) {
          const int64_t n = idx >> cpr_log;
          const int ch = (int)(idx & (cpr - 1));
          ua[u] = __builtin_nontemporal_load((const u32x4*)(ab + n * a_row + ch * 16));
          ug[u] = __builtin_nontemporal_load((const u32x4*)(gb + n * g_row + ch * 16));
          if (lse_mode) {
            la[u] = p.lse_a[row0 + n];
            lg[u] = p.lse_g[row0 + n];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int64_t idx = i0 + u * stride;
        if (idx >= per_slice) continue;
        const int64_t n = idx >> cpr_log;
        const int ch = (int)(idx & (cpr - 1));
        float wa = wa_gate, wg = wg_gate;
        if (lse_mode) {
          // one softmax over the union of both key sets: weights from the two
          // log-sum-exps (natural log) of the row
          constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.69314718055994531f;
          const float m = fmaxf(la[u], lg[u]);
          const float ea = __builtin_amdgcn_exp2f((la[u] - m) * LOG2E), eg = __builtin_amdgcn_exp2f((lg[u] - m) * LOG2E);
          const float z = ea + eg;
          wa = ea / z;
          wg = eg / z;
          if (p.lse_out != nullptr && ch == 0) p.lse_out[row0 + n] = m + __builtin_amdgcn_logf(z) * LN2;
        }
        float fa[C::E], fg[C::E];
        C::unpack(ua[u], fa);
        C::unpack(ug[u], fg);
#pragma unroll
        for (int e = 0; e < C::E; ++e) fa[e] = fmaf(wg, fg[e], wa * fa[e]);
        __builtin_nontemporal_store(C::pack(fa), (u32x4*)(ob + n * o_row + ch * 16));
      }
    }
  }
}

// One thread per 16-byte chunk of an output row: the four pooled taps of the
// row's position, fp32 weights.  The grid's y index walks the (batch, head)
// slices; within a slice, chunk i is token i / cpr, piece i % cpr (a shift and
// a mask), and a token's frame and row come from division by invariants.
template <bool BF16>
__global__ __launch_bounds__(NTHREADS) void upsample_kernel(const UpsampleParams p) {
  using C = Chunk<BF16>;
  const int cpr = p.head_dim / C::E;
  const int cpr_log = __builtin_ctz((unsigned)cpr);
  const int64_t N = (int64_t)p.T * p.H * p.W;
  const int64_t M = (int64_t)p.T * p.Hp * p.Wp;
  const int64_t per_slice = N * cpr;
  const size_t esz = BF16 ? 2 : 4;
  const int64_t o_row = p.o_sn * (int64_t)esz;
  const int64_t tap_row = (int64_t)p.head_dim * esz;
  const float sy = (float)p.Hp / (float)p.H, sx = (float)p.Wp / (float)p.W;
  for (int bh = blockIdx.y; bh < p.batch * p.heads; bh += gridDim.y) {
    const int h = bh % p.heads, b = bh / p.heads;
    const char* xb = (const char*)p.xp + (int64_t)bh * M * tap_row;
    char* ob = (char*)p.out + (b * p.o_sb + h * p.o_sh) * (int64_t)esz;
    for (int64_t i = (int64_t)blockIdx.x * NTHREADS + threadIdx.x; i < per_slice; i += (int64_t)gridDim.x * NTHREADS) {
      const uint32_t n = (uint32_t)(i >> cpr_log);
      const int ch = (int)(i & (cpr - 1));
      const uint32_t t = fast_div(n, p.fd_hw);
      const uint32_t rem = n - t * p.fd_hw.d;
      const uint32_t y = fast_div(rem, p.fd_w);
      const uint32_t x = rem - y * p.fd_w.d;
      const float fy = fmaxf(((float)y + 0.5f) * sy - 0.5f, 0.f), fx = fmaxf(((float)x + 0.5f) * sx - 0.5f, 0.f);
      const int y0 = min((int)fy, p.Hp - 1), x0 = min((int)fx, p.Wp - 1);
      const int y1 = min(y0 + 1, p.Hp - 1), x1 = min(x0 + 1, p.Wp - 1);
      const float ly = fy - (float)y0, lx = fx - (float)x0;
      const char* base = xb + (int64_t)t * p.Hp * p.Wp * tap_row + ch * 16;
      auto tap = [&](int yy, int xx, float (&f)[C::E]) {
        C::unpack(*(const u32x4*)(base + (int64_t)(yy * p.Wp + xx) * tap_row), f);
      };
      float a[C::E], c[C::E], acc[C::E];
      tap(y0, x0, a);
      tap(y0, x1, c);
#pragma unroll
      for (int e = 0; e < C::E; ++e) acc[e] = (1.f - ly) * ((1.f - lx) * a[e] + lx * c[e]);
      tap(y1, x0, a);
      tap(y1, x1, c);
#pragma unroll
      for (int e = 0; e < C::E; ++e) acc[e] += ly * ((1.f - lx) * a[e] + lx * c[e]);
      __builtin_nontemporal_store(C::pack(acc), (u32x4*)(ob + (int64_t)n * o_row + ch * 16));
    }
  }
}

int grid_for(int64_t work) {
  int64_t blocks = (work + NTHREADS - 1) / NTHREADS;
  const int64_t cap = 256 * 8 * 16;  // enough waves to saturate HBM; the loop strides the rest
  return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace

dim3 slice_grid(int64_t slices, int64_t per_slice_work, int64_t max_wg) {
  const int gy = (int)(slices < 65535 ? slices : 65535);
  const int64_t gx = (per_slice_work + NTHREADS - 1) / NTHREADS;
  const int64_t cap = (max_wg + gy - 1) / gy;
  return dim3((unsigned)(gx < cap ? (gx > 0 ? gx : 1) : cap), (unsigned)gy);
}

hipError_t launch_avgpool(const PoolParams& p, int bf16, hipStream_t stream) {
  const int cpr = p.head_dim / (bf16 ? 8 : 4);
  const dim3 grid = slice_grid((int64_t)p.batch * p.heads, (int64_t)p.T * p.Hp * p.Wp * cpr, 256 * 8 * 16);
  if (bf16)
    hipLaunchKernelGGL(avgpool_kernel<true>, grid, dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(avgpool_kernel<false>, grid, dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, int bf16, hipStream_t stream) {
  const int cpr = p.head_dim / (bf16 ? 8 : 4);
  // every chunk its own thread: no cap on the grid (12% faster at 4K than
  // a grid capped at a quarter of the chunks)
  const dim3 grid = slice_grid((int64_t)p.batch * p.heads, (p.n_tokens * cpr + MU - 1) / MU, (int64_t)1 << 40);
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_upsample(const UpsampleParams& p, int bf16, hipStream_t stream) {
  const int cpr = p.head_dim / (bf16 ? 8 : 4);
  // every chunk its own thread: no cap on the grid
  const dim3 grid = slice_grid((int64_t)p.batch * p.heads, (int64_t)p.T * p.H * p.W * cpr, (int64_t)1 << 40);
  if (bf16)
    hipLaunchKernelGGL(upsample_kernel<true>, grid, dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(upsample_kernel<false>, grid, dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vdsa
