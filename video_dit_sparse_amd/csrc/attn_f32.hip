// Tile-window ("box") attention forward in fp32 on the vector ALUs.
//
// Same key-box walk as the bf16 MFMA kernel (the keys of a query tile are the
// union of the key tiles in its window, which is one box of tokens), with a
// simpler inner loop: 64 queries per workgroup, four lanes per query each
// owning a quarter of head_dim, keys staged through LDS 32 at a time, and an
// fp32 online softmax.  This path exists for fp32 inputs; it is not tuned.
#include "box_common.h"

namespace vdsa {
namespace {

constexpr int QPB = 64;        // queries per workgroup
constexpr int KPB = 32;        // keys per LDS stage
constexpr int NTHREADS = 256;  // 4 lanes per query

template <int HD>
__global__ __launch_bounds__(NTHREADS) void box_attn_f32_kernel(const BoxAttnParams p) {
  constexpr int DPL = HD / 4;  // head_dim elements per lane
  __shared__ float ks[KPB][HD];
  __shared__ float vs[KPB][HD];

  const int tid = threadIdx.x;
  const int part = tid & 3;
  const int qi = tid >> 2;

  const int wg = xcd_remap(blockIdx.x, p.total_wg);
  const int qblk = wg % p.qblocks;
  const int rest = wg / p.qblocks;
  const int ntiles = p.nT * p.nH * p.nW;
  const int tile = rest % ntiles;
  const int bh = rest / ntiles;
  const int h = bh % p.heads;
  const int b = bh / p.heads;
  Box qbx, kbx;
  tile_boxes(p, tile, qbx, kbx);
  const int qt0 = qbx.t0, qet = qbx.et, qh0 = qbx.h0, qeh = qbx.eh, qw0 = qbx.w0, qew = qbx.ew;
  const int kt0 = kbx.t0, ket = kbx.et, kh0 = kbx.h0, keh = kbx.eh, kw0 = kbx.w0, kew = kbx.ew;
  const int qvol = qet * qeh * qew;
  const int q0 = qblk * QPB;
  if (q0 >= qvol) return;
  const int kvol = ket * keh * kew;

  const float* qp = (const float*)p.q + b * p.q_sb + h * p.q_sh;
  const float* kp = (const float*)p.k + b * p.k_sb + h * p.k_sh;
  const float* vp = (const float*)p.v + b * p.v_sb + h * p.v_sh;
  float* op = (float*)p.o + b * p.o_sb + h * p.o_sh;

  const int jq = q0 + qi;
  const bool q_valid = jq < qvol;
  int qtok;
  {
    const int j = min(jq, qvol - 1);
    const int jt = j / (qeh * qew), r = j % (qeh * qew);
    qtok = (int)q_token(p, qt0 + jt, qh0 + r / qew, qw0 + r % qew);
  }
  float q[DPL], o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    q[i] = qp[(int64_t)qtok * p.q_sn + part * DPL + i];
    o[i] = 0.f;
  }
  const float c = p.scale_log2e;
  float m_run = -INFINITY, l_run = 0.f;

  for (int k0 = 0; k0 < kvol; k0 += KPB) {
    __syncthreads();
    for (int e = tid; e < KPB * HD; e += NTHREADS) {
      const int r = e / HD, d = e % HD;
      const int j = min(k0 + r, kvol - 1);
      const int jt = j / (keh * kew), rr = j % (keh * kew);
      const int tok = (int)k_token(p, kt0 + jt, kh0 + rr / kew, kw0 + rr % kew);
      ks[r][d] = kp[(int64_t)tok * p.k_sn + d];
      vs[r][d] = vp[(int64_t)tok * p.v_sn + d];
    }
    __syncthreads();
    const int nk = min(KPB, kvol - k0);
    float s[KPB];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < KPB; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc = fmaf(q[i], ks[j][part * DPL + i], acc);
      acc += __shfl_xor(acc, 1, 4);
      acc += __shfl_xor(acc, 2, 4);
      s[j] = acc;
      if (j < nk) mx = fmaxf(mx, acc);
    }
    const float m_new = fmaxf(m_run, mx * c);
    const float corr = exp2f(m_run - m_new);
    l_run *= corr;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] *= corr;
#pragma unroll
    for (int j = 0; j < KPB; ++j) {
      const float pj = j < nk ? exp2f(fmaf(s[j], c, -m_new)) : 0.f;
      l_run += pj;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] = fmaf(pj, vs[j][part * DPL + i], o[i]);
    }
    m_run = m_new;
  }

  if (q_valid) {
    const float inv = 1.f / l_run;
    float lse_row = (m_run + log2f(l_run)) * 0.69314718055994531f;
    if (p.merge != MERGE_NONE) {
      // combine with the other branch's row, read at the positions written
      const RowMerge rm = row_merge(p, b, h, (uint32_t)qtok, lse_row);
      const float* olp = (const float*)p.ol + b * p.ol_sb + h * p.ol_sh + (int64_t)qtok * p.ol_sn + part * DPL;
#pragma unroll
      for (int i = 0; i < DPL; ++i)
        op[(int64_t)qtok * p.o_sn + part * DPL + i] = fmaf(rm.wa, olp[i], rm.wb * (o[i] * inv));
      lse_row = rm.lse;
    } else {
#pragma unroll
      for (int i = 0; i < DPL; ++i) op[(int64_t)qtok * p.o_sn + part * DPL + i] = o[i] * inv;
    }
    if (p.lse != nullptr && part == 0) {
      const int64_t N = (int64_t)p.qT * p.qH * p.qW;
      p.lse[((int64_t)b * p.heads + h) * N + qtok] = lse_row;
    }
  }
}

}  // namespace

hipError_t launch_box_attn_f32(const BoxAttnParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.total_wg), block(NTHREADS);
  if (head_dim == 128)
    hipLaunchKernelGGL(box_attn_f32_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(box_attn_f32_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

int box_attn_f32_block_m() { return QPB; }

}  // namespace vdsa
