// Tile-window ("box") attention forward, bf16 in/out, fp32 accumulation, on
// the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// One workgroup = 4 waves = 128 queries of one query tile (tile-local raster
// order), all attending the same key set.  The key set of a query tile is the
// union of the key tiles in its window (Sliding Tile Attention, arXiv
// 2502.04507, abstract: attention proceeds tile by tile over a local 3D
// window); since tiles are boxes of tokens and the window is a box of tiles,
// that union is itself one box of tokens, clipped to the grid.  The kernel
// walks this box in 64-key blocks, computing each key's address from its box
// coordinates; no mask or index list is ever stored.  The global branch uses
// the same kernel with the key box set to the whole pooled grid.
//
// Per 64-key block and wave (32 queries):
//   S^T = K Q^T      (keys x queries; K from LDS, Q^T resident in registers)
//   online softmax   (fp32, exp2 with scale*log2(e) folded into one FMA;
//                     row statistics live in one lane pair, so the only
//                     cross-lane step is one exchange with lane ^ 32)
//   O^T += V^T P^T   (P^T taken straight from the S^T accumulators)
// Both products keep the query index on the MFMA column (= lane % 32), which
// is what lets the softmax statistics and the output rescale stay per lane.
//
// Key order inside a 32-key MFMA block is permuted (bits 2 and 3 of the row
// index swapped) so that the eight P values a lane holds per 16-key chunk are
// eight consecutive keys; the V^T operand is then one 16-byte LDS read.
#include "internal.h"

namespace vdsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BLOCK_M = 128;   // queries per workgroup
constexpr int BLOCK_N = 64;    // keys per iteration
constexpr int NTHREADS = 256;  // 4 waves of 64

__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
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

template <int HD>
__global__ __launch_bounds__(NTHREADS, 2) void box_attn_bf16_kernel(const BoxAttnParams p) {
  constexpr int NCH = HD / 8;          // 16-byte chunks per row
  constexpr int KSTEPS = HD / 16;      // MFMA steps over head_dim
  constexpr int NB = HD / 32;          // 32-row blocks of O^T
  constexpr int RPT = HD / 32;         // key rows loaded per thread (NCH * 64 / 256)
  static_assert(NCH * BLOCK_N == NTHREADS * RPT, "load mapping");

  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][BLOCK_N * HD];
  __shared__ __attribute__((aligned(16))) uint16_t lds_vt[2][HD * BLOCK_N];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- which (batch, head, query tile, query block) this workgroup owns
  const int wg = xcd_remap(blockIdx.x, p.total_wg);
  const int qblk = wg % p.qblocks;
  const int rest = wg / p.qblocks;
  const int ntiles = p.nT * p.nH * p.nW;
  const int tile = rest % ntiles;
  const int bh = rest / ntiles;
  const int h = bh % p.heads;
  const int b = bh / p.heads;

  Box qb, kb;
  tile_boxes(p, tile, qb, kb);
  const int qvol = qb.et * qb.eh * qb.ew;
  const int q0 = qblk * BLOCK_M;
  if (q0 >= qvol) return;  // uniform over the workgroup
  const int kvol = kb.et * kb.eh * kb.ew;
  const int nkb = (kvol + BLOCK_N - 1) / BLOCK_N;

  const uint16_t* __restrict__ qp = (const uint16_t*)p.q + b * p.q_sb + h * p.q_sh;
  const uint16_t* __restrict__ kp = (const uint16_t*)p.k + b * p.k_sb + h * p.k_sh;
  const uint16_t* __restrict__ vp = (const uint16_t*)p.v + b * p.v_sb + h * p.v_sh;
  uint16_t* __restrict__ op = (uint16_t*)p.o + b * p.o_sb + h * p.o_sh;

  // ---- this lane's query (MFMA column l32 of wave `wave`)
  const int jq = q0 + wave * 32 + l32;
  const bool q_valid = jq < qvol;
  int qtok;
  {
    const int j = min(jq, qvol - 1);
    const int plane = qb.eh * qb.ew;
    const int jt = j / plane;
    const int r = j - jt * plane;
    const int jh = r / qb.ew;
    const int jw = r - jh * qb.ew;
    qtok = ((qb.t0 + jt) * p.qH + qb.h0 + jh) * p.qW + qb.w0 + jw;
  }
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* src = qp + (uint32_t)qtok * (uint32_t)p.q_sn + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 16 * ks));
  }

  // ---- key box addressing: key j -> token, via two divisions by invariants
  const FastDiv fd_plane = make_fastdiv((uint32_t)(kb.eh * kb.ew));
  const FastDiv fd_row = make_fastdiv((uint32_t)kb.ew);
  auto key_token = [&](int j) -> uint32_t {
    j = min(j, kvol - 1);
    const uint32_t jt = fast_div((uint32_t)j, fd_plane);
    const uint32_t r = (uint32_t)j - jt * fd_plane.d;
    const uint32_t jh = fast_div(r, fd_row);
    const uint32_t jw = r - jh * fd_row.d;
    return ((kb.t0 + jt) * p.kH + kb.h0 + jh) * p.kW + kb.w0 + jw;
  };

  // Load mapping: thread owns chunk `lc` (8 head_dim elements) of key rows
  // RPT*lr .. RPT*lr+RPT-1 of the block.
  const int lc = tid % NCH;
  const int lr = tid / NCH;
  u32x4 kreg[RPT], vreg[RPT];
  auto load_block = [&](int blk) {
    const uint32_t my_tok = key_token(blk * BLOCK_N + lane);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const uint32_t tok = (uint32_t)__shfl((int)my_tok, RPT * lr + i, 64);
      kreg[i] = *(const u32x4*)(kp + tok * (uint32_t)p.k_sn + 8 * lc);
      vreg[i] = *(const u32x4*)(vp + tok * (uint32_t)p.v_sn + 8 * lc);
    }
  };
  auto store_block = [&](int stage) {
    uint16_t* kd = lds_k[stage];
    uint16_t* vd = lds_vt[stage];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = RPT * lr + i;
      *(u32x4*)(kd + row * HD + ((lc ^ (row & (NCH - 1))) * 8)) = kreg[i];
    }
    // V^T: element (d, key) with d = 8*lc + e; this thread's RPT keys are
    // consecutive, so each d gets one RPT*2-byte store.
    const int key0 = RPT * lr;
    const int kchunk = key0 >> 3, kin = key0 & 7;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lc + e;
      const int w = e >> 1, hi = e & 1;
      uint16_t vals[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) vals[i] = (uint16_t)(hi ? (vreg[i][w] >> 16) : (vreg[i][w] & 0xffffu));
      uint16_t* dst = vd + d * BLOCK_N + ((kchunk ^ (d & 7)) * 8) + kin;
      if constexpr (RPT == 4) {
        u32x2 pk;
        pk[0] = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
        pk[1] = (uint32_t)vals[2] | ((uint32_t)vals[3] << 16);
        *(u32x2*)dst = pk;
      } else {
        *(uint32_t*)dst = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
      }
    }
  };

  f32x16 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2(e)*logit
  float l_run = 0.f;         // this lane's share of the running denominator
  const float c = p.scale_log2e;

  load_block(0);
  store_block(0);
  __syncthreads();

  const int krow_a = swap_bits23(l32);   // key row this lane feeds to the S^T MFMA

  for (int blk = 0; blk < nkb; ++blk) {
    const int stage = blk & 1;
    const bool more = blk + 1 < nkb;
    if (more) load_block(blk + 1);

    // S^T = K Q^T for two 32-key halves
    const uint16_t* kd = lds_k[stage];
    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x16{};
      const int row = sb * 32 + krow_a;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int ch = 2 * ks + g;
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(kd + row * HD + ((ch ^ (row & (NCH - 1))) * 8)));
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[sb], 0, 0, 0);
      }
    }

    // online softmax over this block's keys (register v of half sb holds key
    // 32*sb + 16*(v/8) + 8*g + v%8)
    const bool partial = (blk + 1) * BLOCK_N > kvol;
    if (partial) {
      const int kbase = blk * BLOCK_N + 8 * g;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kbase + 32 * sb + 16 * (v >> 3) + (v & 7) >= kvol) s[sb][v] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[0][v]);
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[1][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * c);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {   // rescale only when some max grew
      const float corr = exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < NB; ++i) oacc[i] *= corr;
    }
    m_run = m_new;
    bf16x8 pf[4];
    float lsum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        bf16x8 pk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float pv = exp2f(fmaf(s[sb][8 * hlf + e], c, -m_new));
          if (partial && s[sb][8 * hlf + e] == -INFINITY) pv = 0.f;
          lsum += pv;
          pk[e] = (__bf16)pv;
        }
        pf[2 * sb + hlf] = pk;
      }
    }
    l_run += lsum;

    // O^T += V^T P^T
    const uint16_t* vd = lds_vt[stage];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int ch = 2 * kc + g;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int d = 32 * nb + l32;
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(vd + d * BLOCK_N + ((ch ^ (d & 7)) * 8)));
        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], oacc[nb], 0, 0, 0);
      }
    }

    if (more) store_block(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and store (lane owns query l32; register v of
  // block nb holds head_dim index 32*nb + 8*(v/4) + 4*g + v%4)
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  if (q_valid) {
    uint16_t* dst = op + (uint32_t)qtok * (uint32_t)p.o_sn + 4 * g;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(oacc[nb][4 * r4 + e] * inv);
        *(u32x2*)(dst + 32 * nb + 8 * r4) = __builtin_bit_cast(u32x2, ov);
      }
    if (p.lse != nullptr && g == 0) {
      const int64_t N = (int64_t)p.qT * p.qH * p.qW;
      p.lse[((int64_t)b * p.heads + h) * N + qtok] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

hipError_t launch_box_attn_bf16(const BoxAttnParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.total_wg), block(NTHREADS);
  if (head_dim == 128)
    hipLaunchKernelGGL(box_attn_bf16_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(box_attn_bf16_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

int box_attn_bf16_block_m() { return BLOCK_M; }

}  // namespace vdsa
