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
//   online softmax   (fp32, v_exp_f32 with scale*log2(e) folded into one FMA;
//                     row maxima live in one lane pair, so the only
//                     cross-lane step is one exchange with lane ^ 32)
//   O^T += V^T P^T   (P^T taken straight from the S^T accumulators) and the
//                     denominators: an all-ones A operand times P^T sums the
//                     probabilities exactly as rounded to bf16 for the
//                     product, so a weight's rounding cancels in O
// Both products keep the query index on the MFMA column (= lane % 32), which
// is what lets the softmax statistics and the output rescale stay per lane.
//
// Key order inside a 32-key MFMA block is permuted (bits 2 and 3 of the row
// index swapped) so that the eight P values a lane holds per 16-key chunk are
// eight consecutive keys; the V^T operand is then one 16-byte LDS read.
//
// Data movement per block (double-buffered LDS, one barrier per block):
//   K  : global -> LDS directly (buffer_load_dwordx4 ... lds, no registers),
//        into "k-planes": plane ks holds head_dim elements [16ks, 16ks+16) of
//        all 64 keys as [32-key half][8-element half][32 keys][16 bytes].
//        Each S^T operand read is one contiguous 1 KB per wave, and any 16
//        consecutive lanes read 256 contiguous bytes.
//   V  : global -> registers -> LDS transposed ("v-planes": plane kc holds
//        keys [16kc, 16kc+16) of every head_dim row as
//        [32-row block][8-key half][32 rows][16 bytes], rows XOR-swizzled by
//        (kc, half)).  The lane mapping and the swizzle make the transposing
//        stores free of bank conflicts; each V^T operand read is again one
//        contiguous 1 KB per wave.
// Global reads use buffer resources (scalar base + 32-bit lane offsets).
#include <type_traits>

#include "box_common.h"

namespace vdsa {
namespace {

constexpr int BLOCK_M = 128;   // queries per workgroup
constexpr int BLOCK_N = 64;    // keys per iteration
constexpr int NTHREADS = 256;  // 4 waves of 64
// s_waitcnt with vmcnt = 0 and expcnt / lgkmcnt left at their maxima
constexpr int WAIT_VMCNT0 = 0x0F70;
constexpr float RESCALE_MARGIN = 8.f;

__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

template <int HD>
__global__ __launch_bounds__(NTHREADS, 2) void box_attn_bf16_kernel(const BoxAttnParams p) {
  constexpr int KSTEPS = HD / 16;          // MFMA steps over head_dim = k-planes
  constexpr int NB = HD / 32;              // 32-row blocks of O^T
  constexpr int RPT = HD / 32;             // V key rows loaded per thread
  constexpr int NLR = BLOCK_N / RPT;       // threads sharing one V chunk column
  constexpr int KPLANE = BLOCK_N * 32;     // bytes
  constexpr int VPLANE = HD * 32;          // bytes
  constexpr int K_STAGE = KSTEPS * KPLANE;
  constexpr int STAGE = K_STAGE + 4 * VPLANE;
  constexpr int DMA_PER_WAVE = KSTEPS * 2 / 4;  // 1 KB K-plane segments per wave
  static_assert(NLR * (HD / 8) == NTHREADS, "V load mapping");

  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- which (batch, head, query tile, query block) this workgroup owns
  // (divisions by invariants the host prepared)
  const uint32_t wg = (uint32_t)xcd_remap(blockIdx.x, p.total_wg);
  const uint32_t rest = fast_div(wg, p.fd_qblocks);
  const int qblk = (int)(wg - rest * p.fd_qblocks.d);
  const uint32_t bh = fast_div(rest, p.fd_tiles);
  const uint32_t tile = rest - bh * p.fd_tiles.d;
  const int b = (int)fast_div(bh, p.fd_heads);
  const int h = (int)(bh - (uint32_t)b * p.fd_heads.d);

  Box qb, kb;
  {
    const uint32_t tw = fast_div(tile, p.fd_nw);
    const uint32_t at = fast_div(tw, p.fd_nh);
    tile_boxes_at(p, (int)at, (int)(tw - at * p.fd_nh.d), (int)(tile - tw * p.fd_nw.d), qb, kb);
  }
  const int qvol = qb.et * qb.eh * qb.ew;
  const int q0 = qblk * BLOCK_M;
  if (q0 >= qvol) return;  // uniform over the workgroup
  const int kvol = kb.et * kb.eh * kb.ew;
  const int nkb = (kvol + BLOCK_N - 1) / BLOCK_N;

  const char* __restrict__ qp = (const char*)p.q + 2 * (b * p.q_sb + h * p.q_sh);
  const char* kp = (const char*)p.k + 2 * (b * p.k_sb + h * p.k_sh);
  const char* vp = (const char*)p.v + 2 * (b * p.v_sb + h * p.v_sh);
  // the byte range one head's keys can reach: (kT*kH*kW - 1) rows + one row of head_dim
  const uint32_t krange = ((uint32_t)(p.kT * p.kH * p.kW) - 1u) * 2u * (uint32_t)p.k_sn + 2u * HD;
  const uint32_t vrange = ((uint32_t)(p.kT * p.kH * p.kW) - 1u) * 2u * (uint32_t)p.v_sn + 2u * HD;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, (int)krange, BUF_FLAGS);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, (int)vrange, BUF_FLAGS);
  char* op = (char*)p.o + 2 * (b * p.o_sb + h * p.o_sh);
  const uint32_t q_row = 2u * (uint32_t)p.q_sn, k_row = 2u * (uint32_t)p.k_sn;
  const uint32_t v_row = 2u * (uint32_t)p.v_sn, o_row = 2u * (uint32_t)p.o_sn;

  // ---- this lane's query (MFMA column l32 of wave `wave`)
  const int jq = q0 + wave * 32 + l32;
  const bool q_valid = jq < qvol;
  uint32_t qtok;
  {
    const FastDiv fq_plane = make_fastdiv_fp64((uint32_t)(qb.eh * qb.ew));
    const FastDiv fq_row = make_fastdiv_fp64((uint32_t)qb.ew);
    const uint32_t j = (uint32_t)min(jq, qvol - 1);
    const uint32_t jt = fast_div(j, fq_plane);
    const uint32_t r = j - jt * fq_plane.d;
    const uint32_t jh = fast_div(r, fq_row);
    const uint32_t jw = r - jh * fq_row.d;
    qtok = q_token(p, qb.t0 + (int)jt, qb.h0 + (int)jh, qb.w0 + (int)jw);
  }
  bf16x8 qf[KSTEPS];
  {
    const char* src = qp + qtok * q_row + 16 * g;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 32 * ks));
  }

  // ---- key box addressing: key j -> token, via two divisions by invariants
  const FastDiv fd_plane = make_fastdiv_fp64((uint32_t)(kb.eh * kb.ew));
  const FastDiv fd_row = make_fastdiv_fp64((uint32_t)kb.ew);
  auto key_token = [&](int j) -> uint32_t {
    j = min(j, kvol - 1);   // keys past the box repeat the last key; masked later
    const uint32_t jt = fast_div((uint32_t)j, fd_plane);
    const uint32_t r = (uint32_t)j - jt * fd_plane.d;
    const uint32_t jh = fast_div(r, fd_row);
    const uint32_t jw = r - jh * fd_row.d;
    return k_token(p, kb.t0 + (int)jt, kb.h0 + (int)jh, kb.w0 + (int)jw);
  };

  // V mapping: thread owns 16-byte chunk vc (head_dim [8vc, 8vc+8)) of keys
  // RPT*vr .. RPT*vr+RPT-1.
  const int vr = tid % NLR;
  const int vc = tid / NLR;
  u32x4 vreg[RPT];

  // Issue the global reads of block `blk` into LDS stage `stage` (K) and
  // registers (V).
  auto load_block = [&](int blk, int stage) {
    const uint32_t my_tok = key_token(blk * BLOCK_N + lane);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int sb = i & 1;                           // key rows [32sb, 32sb+32)
      const int plane = wave * (DMA_PER_WAVE / 2) + (i >> 1);
      // lane L fills key row 32sb + L%32, head_dim half L/32 of the plane
      const uint32_t tok = (uint32_t)__shfl((int)my_tok, 32 * sb + l32, 64);
      const uint32_t off = tok * k_row + (uint32_t)(2 * plane + g) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)(lds + stage * STAGE + plane * KPLANE + sb * 1024),
                                               16, (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const uint32_t tok = (uint32_t)__shfl((int)my_tok, RPT * vr + i, 64);
      vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrsrc, (int)(tok * v_row + vc * 16), 0, 0));
    }
  };
  // Transpose the V registers into the v-planes of `stage`: element (key k,
  // head_dim row d = 32nb + r) sits at byte
  //   (k>>4)*VPLANE + nb*1024 + ((k>>3)&1)*512 + (r ^ swz)*16 + (k&7)*2,
  //   swz = (k>>4) | (((k>>3)&1) << 2).
  auto store_v = [&](int stage) {
    char* vst = lds + stage * STAGE + K_STAGE;
    const int k0 = RPT * vr;
    const int kc = k0 >> 4, half = (k0 >> 3) & 1;
    const int swz = kc | (half << 2);
    char* base = vst + kc * VPLANE + half * 512 + (k0 & 7) * 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * vc + e;
      const int w = e >> 1;
      // v_perm_b32 byte selectors: low halves (0x05040100) or high halves
      // (0x07060302) of two words packed into one
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      char* dst = base + (d >> 5) * 1024 + (((d & 31) ^ swz) * 16);
      if constexpr (RPT == 4) {
        u32x2 pk;
        pk[0] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
        pk[1] = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
        *(u32x2*)dst = pk;
      } else {
        *(uint32_t*)dst = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
      }
    }
  };

  f32x16 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2(e)*logit
  f32x16 lacc = f32x16{};    // row sums of P: every register holds the lane's query's sum
  bf16x8 ones8;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones8[e] = (__bf16)1.f;
  const float c = p.scale_log2e;

  load_block(0, 0);
  store_v(0);
  __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);
  __syncthreads();

  const int k_rd = g * 512 + swap_bits23(l32) * 16;   // this lane's S^T operand (key row, half)
  int v_rd[4];                                         // this lane's V^T operand per kc
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) v_rd[kc] = kc * VPLANE + g * 512 + ((l32 ^ (kc | (g << 2))) * 16);

  // One 64-key block.  Only the last block of the box can hold keys past its
  // end; it is the only one that runs the masking code.
  auto process = [&](int blk, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int stage = blk & 1;
    const bool more = blk + 1 < nkb;
    if (more) load_block(blk + 1, stage ^ 1);

    // S^T = K Q^T for two 32-key halves
    const char* kst = lds + stage * STAGE;
    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(kst + ks * KPLANE + sb * 1024 + k_rd));
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[sb], 0, 0, 0);
      }
    }

    // online softmax over this block's keys (register v of half sb holds key
    // 32*sb + 16*(v/8) + 8*g + v%8 of the block).  Keys past the box end are
    // copies of the box's last key, so they may take part in the max; their
    // probabilities are zeroed.
    float mx = s[0][0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[0][v]);
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[1][v]);
    mx = xhalf_max(mx) * c;
    // Lazy rescale: keep the reference max m_run until some query's block
    // max exceeds it by more than RESCALE_MARGIN (log2 units).  Until then
    // probabilities stay below 2^RESCALE_MARGIN, well inside bf16/fp32 range,
    // and the final normalisation by the same reference is exact.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + RESCALE_MARGIN)) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      lacc *= corr;
#pragma unroll
      for (int i = 0; i < NB; ++i) oacc[i] *= corr;
      m_run = m_new;
    }
    const float m_new = m_run;
    const int nvalid = PARTIAL ? kvol - blk * BLOCK_N : BLOCK_N;
    bf16x8 pf[4];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        bf16x8 pk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // v_exp_f32 directly: arguments are <= 0, results in [0, 1]
          float pv = __builtin_amdgcn_exp2f(fmaf(s[sb][8 * hlf + e], c, -m_new));
          if constexpr (PARTIAL) {
            if (32 * sb + 16 * hlf + 8 * g + e >= nvalid) pv = 0.f;
          }
          pk[e] = (__bf16)pv;
        }
        pf[2 * sb + hlf] = pk;
      }
    }

    // O^T += V^T P^T
    const char* vst = lds + stage * STAGE + K_STAGE;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(vst + v_rd[kc] + nb * 1024));
        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], oacc[nb], 0, 0, 0);
      }
      // the softmax denominator over the weights exactly as rounded for the
      // product: an all-ones A operand sums each query's column of P^T
      lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones8, pf[kc], lacc, 0, 0, 0);
    }

    if (more) store_v(stage ^ 1);
    __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);   // K of the next block has landed in LDS
    __syncthreads();
  };

  const bool last_partial = kvol % BLOCK_N != 0;
  const int nfull = last_partial ? nkb - 1 : nkb;
  for (int blk = 0; blk < nfull; ++blk) process(blk, std::false_type{});
  if (last_partial) process(nkb - 1, std::true_type{});

  // ---- epilogue: normalise and store (lane owns query l32; register v of
  // block nb holds head_dim index 32*nb + 8*(v/4) + 4*g + v%4)
  const float l_tot = lacc[0];
  const float inv = 1.f / l_tot;
  if (p.merge == MERGE_NONE) {
    // The wave's 32 rows go through LDS (row-major, 8-byte pieces XOR-
    // swizzled by row, free of bank conflicts) so that every store writes
    // whole rows, 16 bytes per lane: a lane's own pieces of O are 8 bytes
    // of each of 16 head_dim quarters, which as direct stores leave every
    // cache line to be assembled from 8 partial writes.  The loop's last
    // barrier has retired every read of the K/V stages.
    constexpr int ROWB = 2 * HD;             // bytes per row
    constexpr int NC8 = HD / 4;              // 8-byte pieces per row
    constexpr int LPR = ROWB / 16;           // lanes per row in the stores
    constexpr int RPI = 64 / LPR;            // rows per store instruction
    char* stg = lds + wave * (32 * ROWB + 128);
    uint32_t* toks = (uint32_t*)(stg + 32 * ROWB);   // row -> token, ~0u past the tile
    const int xw = l32 & (NC8 - 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(oacc[nb][4 * r4 + e] * inv);
        const int c8 = 8 * nb + 2 * r4 + g;
        *(u32x2*)(stg + l32 * ROWB + (c8 ^ xw) * 8) = __builtin_bit_cast(u32x2, ov);
      }
    if (g == 0) {
      toks[l32] = q_valid ? qtok : ~0u;
      if (q_valid && p.lse != nullptr) {
        const int64_t N = (int64_t)p.qT * p.qH * p.qW;
        p.lse[((int64_t)b * p.heads + h) * N + qtok] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
      }
    }
    __syncthreads();
    const int j = lane % LPR;   // 16-byte piece of the row: 8-byte pieces 2j, 2j+1
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / LPR;
      const uint32_t tok = toks[r];
      const int xr = r & (NC8 - 1);
      u32x4 v = *(const u32x4*)(stg + r * ROWB + (((2 * j) ^ xr) & ~1) * 8);
      if (xr & 1) v = u32x4{v[2], v[3], v[0], v[1]};
      if (tok != ~0u) *(u32x4*)(op + tok * o_row + 16 * j) = v;
    }
    return;
  }
  // with a merge, the row combines with the other branch's row read at the
  // same positions
  if (q_valid) {
    float lse_row = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    const RowMerge rm = row_merge(p, b, h, qtok, lse_row);
    const float wa = rm.wa;
    const float sc = rm.wb * inv;
    lse_row = rm.lse;
    char* dst = op + qtok * o_row + 8 * g;
    const char* src = (const char*)p.ol + 2 * (b * p.ol_sb + h * p.ol_sh) + qtok * (2u * (uint32_t)p.ol_sn) + 8 * g;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = oacc[nb][4 * r4 + e] * sc;
        const u32x2 raw = *(const u32x2*)(src + 64 * nb + 16 * r4);
        float a[4];
        bf16x4_to_f32(raw[0], raw[1], a);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = fmaf(wa, a[e], f[e]);
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)f[e];
        *(u32x2*)(dst + 64 * nb + 16 * r4) = __builtin_bit_cast(u32x2, ov);
      }
    if (p.lse != nullptr && g == 0) {
      const int64_t N = (int64_t)p.qT * p.qH * p.qW;
      p.lse[((int64_t)b * p.heads + h) * N + qtok] = lse_row;
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
