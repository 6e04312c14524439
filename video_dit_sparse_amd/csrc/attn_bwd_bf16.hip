// Backward pass of tile-window ("box") attention, bf16 in/out, head_dim 128,
// fp32 accumulation, on v_mfma_f32_16x16x32_bf16.
//
// Gradients of O = softmax(scale Q K^T) V over each query's key box, from the
// forward's LSE and delta = rowsum(dO * O) (the softmax Jacobian applied row
// by row):
//   P = exp(scale q.k - LSE),  dP = dO.v,  dS = P * (dP - delta),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// Two passes share one kernel template (BoxBwdParams):
//   dQ pass (KV = false): a wave owns OT tiles of 16 queries (Q and dO
//     resident as MFMA B operands) and walks the key box: S^T = K Q^T,
//     dP^T = V dO^T, dQ^T += K^T dS^T.
//   dK/dV pass (KV = true): a wave owns OT tiles of 16 keys (K and V
//     resident) and walks the queries whose windows contain its key tile:
//     S = Q K^T, dP = dO V^T, dK^T += Q^T dS, dV^T += dO^T P.
// Every operand fragment read from LDS feeds OT products, one per own tile.
// The dQ pass runs OT = 2 with 4 waves and 32-token blocks (two workgroups
// per CU); the dK/dV pass, whose two accumulator sets leave no registers for
// a second tile, runs OT = 1 with 8 waves and 64-token blocks.
// In both, the iterated tokens sit on the MFMA rows and the owned tokens on
// the column, so every probability of an owned token is computed by one lane
// group and the products reuse the forward's operand layouts: iterated rows
// are permuted inside each 32-row chunk (row r of 16-row tile t is token
// 8*(r/4) + 4t + r%4) so that the lane group G holds tokens 8G .. 8G+7 after
// the two tiles, which is exactly the k-slice of the following product.
//
// Per block of the iterated box (one or two 32-token chunks), LDS holds
// (double-buffered):
//   X fragments (K or Q; DMA'd, as the forward's K fragments),
//   Y fragments (V or dO; DMA'd the same way),
//   X^T fragments (K^T or Q^T; transposed through registers with the
//     forward's XOR-swizzled V^T layout),
//   and in the dK/dV pass Y^T fragments (dO^T) and the block's LSE (log2
//   units) and delta.
#include <type_traits>

#include "box_common.h"

namespace vdsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
constexpr int BUF_FLAGS = 0x00020000;   // raw buffer resource word 3 (gfx9-class)

constexpr int HD = 128;
constexpr int KS = HD / 32;            // 32-wide head_dim steps
constexpr int ND = HD / 16;            // 16-row head_dim tiles
constexpr int WAIT_VMCNT0 = 0x0F70;    // s_waitcnt vmcnt(0), other counters untouched
constexpr int RA = 3;                  // operand fragments read ahead of their products

// Shape of one pass: OT own 16-token tiles per wave, NW waves, NCH 32-token
// chunks per block of the iterated box.
template <bool KV, int OT_, int NW_, int NCH_>
struct Cfg {
  static constexpr int OT = OT_, NW = NW_, NCH = NCH_;
  static constexpr int BLOCK_N = 32 * NCH;                 // iterated tokens per block
  static constexpr int BLOCK_M = NW * 16 * OT;             // owned tokens per workgroup
  static constexpr int NFRAG = NCH * 2 * KS;               // (chunk, t, ks) fragments of X and of Y
  static constexpr int FRAG_BYTES = NFRAG * 1024;
  static constexpr int T_BYTES = NCH * ND * 1024;          // (chunk, dt) fragments of X^T, Y^T
  static constexpr int DMA_W = NFRAG / NW;                 // fragments per wave per tensor
  static constexpr int VPT = BLOCK_N * HD / 8 / (NW * 64); // 16-byte chunks per thread for a transposed copy
  static constexpr int NKG = BLOCK_N / VPT;
  // LDS layout of one stage
  static constexpr int XF = 0;
  static constexpr int YF = FRAG_BYTES;
  static constexpr int XT = 2 * FRAG_BYTES;
  static constexpr int YT = XT + T_BYTES;                  // dK/dV pass only
  static constexpr int LSE = KV ? YT + T_BYTES : XT + T_BYTES;
  static constexpr int DEL = LSE + BLOCK_N * 4;
  static constexpr int STAGE = KV ? DEL + BLOCK_N * 4 : XT + T_BYTES;
  static_assert(DMA_W * NW == NFRAG && VPT == 2 && VPT * NKG == BLOCK_N && BLOCK_N <= 64, "work split");
};
using CfgDQ = Cfg<false, 2, 4, 1>;
using CfgKV = Cfg<true, 1, 8, 2>;

template <bool KV, class C>
__global__ __launch_bounds__(C::NW * 64) void box_attn_bwd_bf16_kernel(const BoxBwdParams P) {
  using Lay = C;
  constexpr int OT = C::OT, NW = C::NW, NCH = C::NCH, BLOCK_N = C::BLOCK_N, BLOCK_M = C::BLOCK_M;
  constexpr int DMA_W = C::DMA_W, VPT = C::VPT, NKG = C::NKG;
  const BoxAttnParams& g = P.g;
  __shared__ __attribute__((aligned(16))) char lds[2 * Lay::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int G = lane >> 4;

  // ---- which (batch, head, own tile, own block) this workgroup owns
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
  const int o0 = oblk * BLOCK_M;
  if (o0 >= ovol) return;  // uniform over the workgroup
  const int ivol = ib.et * ib.eh * ib.ew;
  const int nib = (ivol + BLOCK_N - 1) / BLOCK_N;

  // own side A (S operand) and B (dP operand); iterated side X (S) and Y (dP)
  const char* ap = KV ? (const char*)P.k + 2 * (b * P.k_sb + h * P.k_sh) : (const char*)P.q + 2 * (b * P.q_sb + h * P.q_sh);
  const char* bp = KV ? (const char*)P.v + 2 * (b * P.v_sb + h * P.v_sh) : (const char*)P.dout + 2 * (b * P.do_sb + h * P.do_sh);
  const char* xp = KV ? (const char*)P.q + 2 * (b * P.q_sb + h * P.q_sh) : (const char*)P.k + 2 * (b * P.k_sb + h * P.k_sh);
  const char* yp = KV ? (const char*)P.dout + 2 * (b * P.do_sb + h * P.do_sh) : (const char*)P.v + 2 * (b * P.v_sb + h * P.v_sh);
  const uint32_t a_row = 2u * (uint32_t)(KV ? P.k_sn : P.q_sn), b_row = 2u * (uint32_t)(KV ? P.v_sn : P.do_sn);
  const uint32_t x_row = 2u * (uint32_t)(KV ? P.q_sn : P.k_sn), y_row = 2u * (uint32_t)(KV ? P.do_sn : P.v_sn);
  const uint32_t n_iter = (uint32_t)(g.kT * g.kH * g.kW);
  const uint32_t xrange = (n_iter - 1u) * x_row + 2u * HD;
  const uint32_t yrange = (n_iter - 1u) * y_row + 2u * HD;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)xp, 0, (int)xrange, BUF_FLAGS);
  const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)yp, 0, (int)yrange, BUF_FLAGS);
  const float* lse_bh = P.lse + ((int64_t)b * g.heads + h) * P.n_q;
  const float* del_bh = P.delta + ((int64_t)b * g.heads + h) * P.n_q;
  constexpr float LOG2E = 1.4426950408889634f;
  const float cl2 = g.scale_log2e;

  // ---- this lane's own tokens: column l16 of each of the wave's OT tiles
  bool own_valid[OT];
  uint32_t own_tok[OT];
  bf16x8 af[OT][KS], bf[OT][KS];
  float own_lse2[OT], own_del[OT];
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    const int jo = o0 + (wave * OT + ot) * 16 + l16;
    own_valid[ot] = jo < ovol;
    const int j = min(jo, ovol - 1);
    const int plane = ob.eh * ob.ew;
    const int jt = j / plane;
    const int r = j - jt * plane;
    const int jh = r / ob.ew;
    const int jw = r - jh * ob.ew;
    own_tok[ot] = q_token(g, ob.t0 + jt, ob.h0 + jh, ob.w0 + jw);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      af[ot][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(ap + own_tok[ot] * a_row + 64 * ks + 16 * G));
      bf[ot][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(bp + own_tok[ot] * b_row + 64 * ks + 16 * G));
    }
    own_lse2[ot] = 0.f;
    own_del[ot] = 0.f;
    if constexpr (!KV) {
      own_lse2[ot] = lse_bh[own_tok[ot]] * LOG2E;
      own_del[ot] = del_bh[own_tok[ot]];
    }
  }

  // ---- iterated box addressing: token j of the box -> token index
  const FastDiv fd_plane = make_fastdiv((uint32_t)(ib.eh * ib.ew));
  const FastDiv fd_row = make_fastdiv((uint32_t)ib.ew);
  auto iter_token = [&](int j) -> uint32_t {
    j = min(j, ivol - 1);   // past the box: repeat the last token; masked later
    const uint32_t jt = fast_div((uint32_t)j, fd_plane);
    const uint32_t r = (uint32_t)j - jt * fd_plane.d;
    const uint32_t jh = fast_div(r, fd_row);
    const uint32_t jw = r - jh * fd_row.d;
    return k_token(g, ib.t0 + (int)jt, ib.h0 + (int)jh, ib.w0 + (int)jw);
  };

  const int row_in_chunk = 8 * (l16 >> 2) + (l16 & 3);
  const int vk = tid % NKG;
  const int vc = tid / NKG;
  u32x4 xreg[VPT], yreg[VPT];
  float lse_reg = 0.f, del_reg = 0.f;
  auto load_block = [&](int blk, int stage) {
    const uint32_t my_tok = iter_token(blk * BLOCK_N + lane);
    char* st = lds + stage * Lay::STAGE;
#pragma unroll
    for (int i = 0; i < DMA_W; ++i) {
      const int f = wave * DMA_W + i;   // fragment = (c*2 + t)*KS + ks
      const int ks = f % KS, t = (f / KS) & 1, c = f / (2 * KS);
      const uint32_t tok = (uint32_t)__shfl((int)my_tok, 32 * c + 4 * t + row_in_chunk, 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (lds_void*)(st + Lay::XF + f * 1024), 16,
                                               (int)(tok * x_row + (uint32_t)(4 * ks + G) * 16u), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(yrsrc, (lds_void*)(st + Lay::YF + f * 1024), 16,
                                               (int)(tok * y_row + (uint32_t)(4 * ks + G) * 16u), 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const uint32_t tok = (uint32_t)__shfl((int)my_tok, VPT * vk + i, 64);
      xreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, (int)(tok * x_row + vc * 16), 0, 0));
      if constexpr (KV)
        yreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(yrsrc, (int)(tok * y_row + vc * 16), 0, 0));
    }
    if constexpr (KV) {
      if (wave == 0) {   // the block's 64 query rows: LSE and delta
        lse_reg = lse_bh[my_tok] * LOG2E;
        del_reg = del_bh[my_tok];
      }
    }
  };
  // transposed copies: element e of the thread's two rows (head_dim 8vc + e)
  // goes to piece (8(vc&1) + (e ^ sig)) of head_dim tile vc/2 of chunk c
  const int vk0 = VPT * vk;
  const int vsig = (((vk0 & 31) >> 3) << 1) | (vk0 >> 5);
  const uint32_t vw_base = (uint32_t)((vk0 >> 5) * ND * 1024 + ((vk0 & 31) >> 3) * 256 + (vk0 & 7) * 2 +
                                      (vc >> 1) * 1024 + (vc & 1) * 128);
  auto store_t = [&](int stage) {
    const uint32_t sbase = (uint32_t)(uintptr_t)(lds + stage * Lay::STAGE);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low bf16 halves
      const uint32_t off = vw_base + (uint32_t)((e ^ vsig) * 16);
      *(lds_u32*)(uintptr_t)(sbase + Lay::XT + off) = __builtin_amdgcn_perm(xreg[1][e >> 1], xreg[0][e >> 1], sel);
      if constexpr (KV)
        *(lds_u32*)(uintptr_t)(sbase + Lay::YT + off) = __builtin_amdgcn_perm(yreg[1][e >> 1], yreg[0][e >> 1], sel);
    }
    if constexpr (KV) {
      if (wave == 0 && lane < BLOCK_N) {
        *(float*)(lds + stage * Lay::STAGE + Lay::LSE + 4 * lane) = lse_reg;
        *(float*)(lds + stage * Lay::STAGE + Lay::DEL + 4 * lane) = del_reg;
      }
    }
  };

  // A-operand read offset of a transposed fragment in chunk c: piece
  // 16G + (l16 ^ ((G << 1) | c))
  int t_rd[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) t_rd[c] = c * ND * 1024 + (16 * G + (l16 ^ ((G << 1) | c))) * 16;

  f32x4 acc1[ND][OT], acc2[ND][OT];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int ot = 0; ot < OT; ++ot) {
      acc1[dt][ot] = f32x4{};
      acc2[dt][ot] = f32x4{};
    }

  load_block(0, 0);
  store_t(0);
  __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);
  __syncthreads();

  auto process = [&](int blk, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int stage = blk & 1;
    const bool more = blk + 1 < nib;
    if (more) load_block(blk + 1, stage ^ 1);
    const char* st = lds + stage * Lay::STAGE;
    const int nvalid = PARTIAL ? ivol - blk * BLOCK_N : BLOCK_N;

#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      // S and dP, register v of tile (t, ot) = iterated row 32c + 8G + 4t + v.
      // Operand fragments of the chunk in the order of their products: steps
      // 0..7 the (X, Y) pairs of S and dP in (ks, t) order, steps 8..15 the
      // X^T (and Y^T) tiles dt; each read RA steps ahead of its products.
      bf16x8 fx[16], fy[16];
      auto rd = [&](int i) __attribute__((always_inline)) {
        if (i < 8) {
          const int f = (c * 2 + (i & 1)) * KS + (i >> 1);
          fx[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + Lay::XF + f * 1024 + lane * 16));
          fy[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + Lay::YF + f * 1024 + lane * 16));
        } else {
          const int dt = i - 8;
          fx[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + Lay::XT + t_rd[c] + dt * 1024));
          if constexpr (KV) fy[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + Lay::YT + t_rd[c] + dt * 1024));
        }
      };
      f32x4 s[2][OT], dp[2][OT];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) {
          s[t][ot] = f32x4{};
          dp[t][ot] = f32x4{};
        }
#pragma unroll
      for (int i = 0; i < RA; ++i) rd(i);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rd(i + RA);
        __builtin_amdgcn_sched_barrier(0);
        const int ks = i >> 1, t = i & 1;
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) {
          s[t][ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx[i], af[ot][ks], s[t][ot], 0, 0, 0);
          dp[t][ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fy[i], bf[ot][ks], dp[t][ot], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      float l2[OT][8], dl[OT][8];
      if constexpr (KV) {
        const f32x4 la = *(const f32x4*)(st + Lay::LSE + 4 * (32 * c + 8 * G));
        const f32x4 lb = *(const f32x4*)(st + Lay::LSE + 4 * (32 * c + 8 * G + 4));
        const f32x4 da = *(const f32x4*)(st + Lay::DEL + 4 * (32 * c + 8 * G));
        const f32x4 db = *(const f32x4*)(st + Lay::DEL + 4 * (32 * c + 8 * G + 4));
#pragma unroll
        for (int ot = 0; ot < OT; ++ot)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            l2[ot][v] = la[v];
            l2[ot][v + 4] = lb[v];
            dl[ot][v] = da[v];
            dl[ot][v + 4] = db[v];
          }
      } else {
#pragma unroll
        for (int ot = 0; ot < OT; ++ot)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            l2[ot][e] = own_lse2[ot];
            dl[ot][e] = own_del[ot];
          }
      }
      bf16x8 pb[OT], dsb[OT];
#pragma unroll
      for (int ot = 0; ot < OT; ++ot)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = e >> 2, v = e & 3;
          float pv = __builtin_amdgcn_exp2f(fmaf(s[t][ot][v], cl2, -l2[ot][e]));
          if constexpr (PARTIAL) {
            if (32 * c + 8 * G + e >= nvalid) pv = 0.f;
          }
          pb[ot][e] = (__bf16)pv;
          dsb[ot][e] = (__bf16)(pv * (dp[t][ot][v] - dl[ot][e]));
        }
      // acc1 += X^T dS (dQ^T or dK^T); dK/dV pass: acc2 += Y^T P (dV^T)
#pragma unroll
      for (int i = 8; i < 16; ++i) {
        if (i + RA < 16) rd(i + RA);
        __builtin_amdgcn_sched_barrier(0);
        const int dt = i - 8;
#pragma unroll
        for (int ot = 0; ot < OT; ++ot)
          acc1[dt][ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx[i], dsb[ot], acc1[dt][ot], 0, 0, 0);
        if constexpr (KV) {
#pragma unroll
          for (int ot = 0; ot < OT; ++ot)
            acc2[dt][ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fy[i], pb[ot], acc2[dt][ot], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    if (more) store_t(stage ^ 1);
    __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);   // DMA of the next block has landed in LDS
    __syncthreads();
  };

  const bool last_partial = ivol % BLOCK_N != 0;
  const int nfull = last_partial ? nib - 1 : nib;
  for (int blk = 0; blk < nfull; ++blk) process(blk, std::false_type{});
  if (last_partial) process(nib - 1, std::true_type{});

  // ---- epilogue: register v of acc tile (dt, ot) is head_dim 16dt + 4G + v
  // of the lane's own token of tile ot
  const float s1 = P.scale;
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    if (!own_valid[ot]) continue;
    if constexpr (!KV) {
      char* dst = (char*)P.dq + 2 * (b * P.dq_sb + h * P.dq_sh) + own_tok[ot] * (2u * (uint32_t)P.dq_sn) + 8 * G;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        bf16x4 ov;
#pragma unroll
        for (int v = 0; v < 4; ++v) ov[v] = (__bf16)(acc1[dt][ot][v] * s1);
        *(u32x2*)(dst + 32 * dt) = __builtin_bit_cast(u32x2, ov);
      }
    } else if (P.grad_f32) {
      float* dk = (float*)P.dk + b * P.dk_sb + h * P.dk_sh + (int64_t)own_tok[ot] * P.dk_sn + 4 * G;
      float* dv = (float*)P.dv + b * P.dv_sb + h * P.dv_sh + (int64_t)own_tok[ot] * P.dv_sn + 4 * G;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        *(f32x4*)(dk + 16 * dt) = acc1[dt][ot] * s1;
        *(f32x4*)(dv + 16 * dt) = acc2[dt][ot];
      }
    } else {
      char* dk = (char*)P.dk + 2 * (b * P.dk_sb + h * P.dk_sh) + own_tok[ot] * (2u * (uint32_t)P.dk_sn) + 8 * G;
      char* dv = (char*)P.dv + 2 * (b * P.dv_sb + h * P.dv_sh) + own_tok[ot] * (2u * (uint32_t)P.dv_sn) + 8 * G;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        bf16x4 kv, vv;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          kv[v] = (__bf16)(acc1[dt][ot][v] * s1);
          vv[v] = (__bf16)acc2[dt][ot][v];
        }
        *(u32x2*)(dk + 32 * dt) = __builtin_bit_cast(u32x2, kv);
        *(u32x2*)(dv + 32 * dt) = __builtin_bit_cast(u32x2, vv);
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BoxBwdParams& p, bool kv, hipStream_t stream) {
  if (kv)
    hipLaunchKernelGGL((box_attn_bwd_bf16_kernel<true, CfgKV>), dim3(p.g.total_wg), dim3(CfgKV::NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((box_attn_bwd_bf16_kernel<false, CfgDQ>), dim3(p.g.total_wg), dim3(CfgDQ::NW * 64), 0, stream, p);
  return hipGetLastError();
}

int attn_bwd_bf16_block_m(bool kv) { return kv ? CfgKV::BLOCK_M : CfgDQ::BLOCK_M; }

}  // namespace vdsa
