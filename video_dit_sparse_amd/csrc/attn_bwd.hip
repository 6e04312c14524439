// Backward pass: the fp32 path of the attention gradients on the vector ALU,
// the delta = rowsum(dO * O) preprocessing, the gradient of the average
// pooling, and the launchers that pick the bf16 matrix-core kernel or the
// fp32 one.
//
// fp32 attention gradients (BoxBwdParams, the same two passes as the bf16
// kernel): 64 owned tokens per workgroup, four lanes per owned token each
// holding a quarter of head_dim, iterated rows staged through LDS 16 at a
// time.  Per owned token and iterated row:
//   dQ pass (own = query q, rows = keys j):
//     p = exp(scale q.k_j - LSE_q), dS = p (dO_q.v_j - delta_q), dQ += dS k_j
//   dK/dV pass (own = key k, rows = queries i):
//     p = exp(scale q_i.k - LSE_i), dS = p (dO_i.v - delta_i),
//     dK += dS q_i, dV += p dO_i
// then dQ and dK are multiplied by the softmax scale.  This path exists for
// fp32 inputs; it is not tuned.
#include "box_common.h"

namespace vdsa {

hipError_t launch_attn_bwd_dkdv_pp(const BoxBwdParams& p, hipStream_t stream);
int attn_bwd_dkdv_pp_block_m();
hipError_t launch_attn_bwd_dq_pp(const BoxBwdParams& p, hipStream_t stream);
int attn_bwd_dq_pp_block_m();

namespace {

constexpr int OPB = 64;        // owned tokens per workgroup
constexpr int RPB = 16;        // iterated rows per LDS stage
constexpr int NTHREADS = 256;  // 4 lanes per owned token

template <int HD, bool KV>
__global__ __launch_bounds__(NTHREADS) void box_attn_bwd_f32_kernel(const BoxBwdParams P) {
  constexpr int DPL = HD / 4;
  const BoxAttnParams& g = P.g;
  __shared__ float xs[RPB][HD];   // K rows (dQ pass) or Q rows
  __shared__ float ys[RPB][HD];   // V rows (dQ pass) or dO rows
  __shared__ float ls[RPB], dls[RPB];

  const int tid = threadIdx.x;
  const int part = tid & 3;
  const int oi = tid >> 2;
  const int wg = xcd_remap(blockIdx.x, g.total_wg);
  const int oblk = wg % g.qblocks;
  const int rest = wg / g.qblocks;
  const int ntiles = g.nT * g.nH * g.nW;
  const int tile = rest % ntiles;
  const int bh = rest / ntiles;
  const int h = bh % g.heads;
  const int b = bh / g.heads;
  Box ob, ib;
  tile_boxes(g, tile, ob, ib);
  const int ovol = ob.et * ob.eh * ob.ew;
  const int o0 = oblk * OPB;
  if (o0 >= ovol) return;
  const int ivol = ib.et * ib.eh * ib.ew;

  const float* qp = (const float*)P.q + b * P.q_sb + h * P.q_sh;
  const float* kp = (const float*)P.k + b * P.k_sb + h * P.k_sh;
  const float* vp = (const float*)P.v + b * P.v_sb + h * P.v_sh;
  const float* dop = (const float*)P.dout + b * P.do_sb + h * P.do_sh;
  const float* lse_bh = P.lse + ((int64_t)b * g.heads + h) * P.n_q;
  const float* del_bh = P.delta + ((int64_t)b * g.heads + h) * P.n_q;

  const int jo = o0 + oi;
  const bool own_valid = jo < ovol;
  int own_tok;
  {
    const int j = min(jo, ovol - 1);
    const int jt = j / (ob.eh * ob.ew), r = j % (ob.eh * ob.ew);
    own_tok = (int)q_token(g, ob.t0 + jt, ob.h0 + r / ob.ew, ob.w0 + r % ob.ew);
  }
  // own operands: (q, dO) in the dQ pass, (k, v) in the dK/dV pass
  float a[DPL], c[DPL], acc1[DPL], acc2[DPL];
  const float* ap = KV ? kp + (int64_t)own_tok * P.k_sn : qp + (int64_t)own_tok * P.q_sn;
  const float* cp = KV ? vp + (int64_t)own_tok * P.v_sn : dop + (int64_t)own_tok * P.do_sn;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    a[i] = ap[part * DPL + i];
    c[i] = cp[part * DPL + i];
    acc1[i] = 0.f;
    acc2[i] = 0.f;
  }
  float own_lse = 0.f, own_del = 0.f;
  if (!KV) {
    own_lse = lse_bh[own_tok];
    own_del = del_bh[own_tok];
  }
  const float scale = P.scale;

  for (int r0 = 0; r0 < ivol; r0 += RPB) {
    __syncthreads();
    for (int e = tid; e < RPB * HD; e += NTHREADS) {
      const int r = e / HD, d = e % HD;
      const int j = min(r0 + r, ivol - 1);
      const int jt = j / (ib.eh * ib.ew), rr = j % (ib.eh * ib.ew);
      const int tok = (int)k_token(g, ib.t0 + jt, ib.h0 + rr / ib.ew, ib.w0 + rr % ib.ew);
      xs[r][d] = KV ? qp[(int64_t)tok * P.q_sn + d] : kp[(int64_t)tok * P.k_sn + d];
      ys[r][d] = KV ? dop[(int64_t)tok * P.do_sn + d] : vp[(int64_t)tok * P.v_sn + d];
      if (KV && d == 0) {
        ls[r] = lse_bh[tok];
        dls[r] = del_bh[tok];
      }
    }
    __syncthreads();
    const int nr = min(RPB, ivol - r0);
    for (int r = 0; r < nr; ++r) {
      float sd = 0.f, pd = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        sd = fmaf(a[i], xs[r][part * DPL + i], sd);
        pd = fmaf(c[i], ys[r][part * DPL + i], pd);
      }
      sd += __shfl_xor(sd, 1, 4);
      sd += __shfl_xor(sd, 2, 4);
      pd += __shfl_xor(pd, 1, 4);
      pd += __shfl_xor(pd, 2, 4);
      const float l = KV ? ls[r] : own_lse;
      const float dl = KV ? dls[r] : own_del;
      const float pr = expf(scale * sd - l);
      const float ds = pr * (pd - dl);
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        acc1[i] = fmaf(ds, xs[r][part * DPL + i], acc1[i]);
        if (KV) acc2[i] = fmaf(pr, ys[r][part * DPL + i], acc2[i]);
      }
    }
  }
  if (!own_valid) return;
  if (!KV) {
    float* dq = (float*)P.dq + b * P.dq_sb + h * P.dq_sh + (int64_t)own_tok * P.dq_sn + part * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) dq[i] = acc1[i] * scale;
  } else {
    float* dk = (float*)P.dk + b * P.dk_sb + h * P.dk_sh + (int64_t)own_tok * P.dk_sn + part * DPL;
    float* dv = (float*)P.dv + b * P.dv_sb + h * P.dv_sh + (int64_t)own_tok * P.dv_sn + part * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      dk[i] = acc1[i] * scale;
      dv[i] = acc2[i];
    }
  }
}

// delta[row] = sum_d a[row, d] * b[row, d]: HD / E lanes per row (E elements
// of 16 bytes each), reduced across the row's lanes.
template <bool BF16, int HD>
__global__ __launch_bounds__(256) void rowdot_kernel(const RowDotParams p) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int LPR = HD / E;   // lanes per row (power of two, <= 64)
  const int64_t rows = (int64_t)p.batch * p.heads * p.n;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / LPR;
  const int ch = (int)(gid % LPR);
  float acc = 0.f;
  if (row < rows) {
    const int64_t n = row % p.n;
    const int bh = (int)(row / p.n);
    const int h = bh % p.heads, b = bh / p.heads;
    const size_t es = BF16 ? 2 : 4;
    const uint32_t* ar = (const uint32_t*)((const char*)p.a + (b * p.a_sb + h * p.a_sh + n * p.a_sn) * es + ch * 16);
    const uint32_t* br = (const uint32_t*)((const char*)p.b + (b * p.b_sb + h * p.b_sh + n * p.b_sn) * es + ch * 16);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = ar[w], y = br[w];
      if (BF16) {
        acc = fmaf(__uint_as_float(x << 16), __uint_as_float(y << 16), acc);
        acc = fmaf(__uint_as_float(x & 0xFFFF0000u), __uint_as_float(y & 0xFFFF0000u), acc);
      } else {
        acc = fmaf(__uint_as_float(x), __uint_as_float(y), acc);
      }
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && ch == 0) p.out[row] = acc;
}

// g[token] = gp[cell(token)] / count(cell): one thread per 16 bytes of output.
// The grid's y index walks the (batch, head) slices; within a slice, chunk i
// is token i / cpr, piece i % cpr (a shift and a mask), and a token's frame,
// row and cell come from division by invariants.
template <bool BF16>
__global__ __launch_bounds__(256) void unpool_grad_kernel(const UnpoolParams p) {
  constexpr int E = BF16 ? 8 : 4;
  const int cpr = p.head_dim / E;
  const int cpr_log = __builtin_ctz((unsigned)cpr);
  const int64_t N = (int64_t)p.T * p.H * p.W;
  const int64_t per_slice = N * cpr;
  const int64_t g_row = p.g_sn * (BF16 ? 2 : 4);
  for (int bh = blockIdx.y; bh < p.batch * p.heads; bh += gridDim.y) {
    const int h = bh % p.heads, b = bh / p.heads;
    const float* gpb = p.gp + (int64_t)bh * p.Hp * p.Wp * p.T * p.head_dim;
    char* gb = (char*)p.g + (b * p.g_sb + h * p.g_sh) * (BF16 ? 2 : 4);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < per_slice; i += (int64_t)gridDim.x * 256) {
      const uint32_t n = (uint32_t)(i >> cpr_log);
      const int ch = (int)(i & (cpr - 1));
      const uint32_t t = fast_div(n, p.fd_hw);
      const uint32_t rem = n - t * p.fd_hw.d;
      const uint32_t hh = fast_div(rem, p.fd_w);
      const uint32_t ww = rem - hh * p.fd_w.d;
      const int ci = (int)fast_div(hh, p.fd_kh), cj = (int)fast_div(ww, p.fd_kw);
      const int cnt = (min(p.H, (ci + 1) * p.kh) - ci * p.kh) * (min(p.W, (cj + 1) * p.kw) - cj * p.kw);
      const float inv = 1.f / (float)cnt;
      const int64_t m = ((int64_t)t * p.Hp + ci) * p.Wp + cj;
      const float* src = gpb + m * p.head_dim + ch * E;
      char* dst = gb + (int64_t)n * g_row + ch * 16;
      if (BF16) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const __bf16 lo = (__bf16)(src[2 * k] * inv), hi = (__bf16)(src[2 * k + 1] * inv);
          w[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        *(float4*)dst = make_float4(src[0] * inv, src[1] * inv, src[2] * inv, src[3] * inv);
      }
    }
  }
}


}  // namespace

int attn_bwd_block_m(int bf16, bool kv) {
  if (!bf16) return OPB;
  return kv ? attn_bwd_dkdv_pp_block_m() : attn_bwd_dq_pp_block_m();
}

hipError_t launch_attn_bwd_dq(const BoxBwdParams& p, int bf16, hipStream_t stream) {
  if (bf16) return launch_attn_bwd_dq_pp(p, stream);
  const dim3 grid(p.g.total_wg), block(NTHREADS);
  if (p.head_dim == 128)
    hipLaunchKernelGGL((box_attn_bwd_f32_kernel<128, false>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((box_attn_bwd_f32_kernel<64, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(const BoxBwdParams& p, int bf16, hipStream_t stream) {
  if (bf16) return launch_attn_bwd_dkdv_pp(p, stream);
  const dim3 grid(p.g.total_wg), block(NTHREADS);
  if (p.head_dim == 128)
    hipLaunchKernelGGL((box_attn_bwd_f32_kernel<128, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((box_attn_bwd_f32_kernel<64, true>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_rowdot(const RowDotParams& p, int bf16, hipStream_t stream) {
  const int lpr = p.head_dim / (bf16 ? 8 : 4);
  const int64_t threads = (int64_t)p.batch * p.heads * p.n * lpr;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (bf16) {
    if (p.head_dim == 128) hipLaunchKernelGGL((rowdot_kernel<true, 128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((rowdot_kernel<true, 64>), grid, block, 0, stream, p);
  } else {
    if (p.head_dim == 128) hipLaunchKernelGGL((rowdot_kernel<false, 128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((rowdot_kernel<false, 64>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_unpool_grad(const UnpoolParams& p, int bf16, hipStream_t stream) {
  // every chunk its own thread: no cap on the grid
  const int64_t per_slice = (int64_t)p.T * p.H * p.W * (p.head_dim / (bf16 ? 8 : 4));
  const dim3 grid = slice_grid((int64_t)p.batch * p.heads, per_slice, (int64_t)1 << 40);
  if (bf16)
    hipLaunchKernelGGL(unpool_grad_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(unpool_grad_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vdsa
