// dK/dV pass of the tile-window ("box") attention backward, bf16 in, head_dim
// 128, fp32 accumulation, with the matrix-core work of one half of the
// workgroup overlapping the softmax terms of the other half.
//
// What it computes: for the keys a workgroup owns, over every query whose key
// box holds them (the queries of the key tile's transposed window),
//   P = exp(scale q.k - LSE),  dP = dO.v,  dS = P * (dP - delta),
//   dK = scale dS^T Q,  dV = P^T dO.
// Each wave owns one 16-key tile (K and V resident as MFMA B operands) and
// walks the queries of its tile's transposed window in 32-query chunks:
// S = Q K^T and dP = dO V^T (rows: queries, columns: the wave's keys), then
// dK^T += Q^T dS and dV^T += dO^T P.  The queries sit on the MFMA rows, so
// every probability of a key is computed by one lane group and the S and dP
// accumulators are already the B operands of the gradient products: query
// rows are permuted inside each chunk (row r of 16-row tile t is query
// 8*(r/4) + 4t + r%4), so that lane group G holds queries 8G .. 8G+7 after
// the two tiles, the k-slice of the following product.  The Q^T and dO^T
// operands use the forward kernels' XOR-swizzled transposed layout.
//
// Schedule.  Eight waves, two per SIMD: group A (waves 0-3) and group B
// (waves 4-7) hold one wave on every SIMD each.  Every wave alternates
//   M(j)  matrix-core phase: dK/dV products of chunk j-1, S and dP of
//         chunk j (32 MFMAs);
//   V(j)  the probabilities and dS of chunk j (VALU and exp),
// group B one phase behind group A, a workgroup barrier between phases, so
// on each SIMD one wave issues MFMAs while the other computes its softmax
// terms.  Every wave passes the same number of barriers: B takes one extra
// before its first phase, A one after its last.
//
// LDS: a ring of four stages, one chunk each: the Q and dO fragments (direct
// global->LDS loads, as the forward's K fragments), the Q^T and dO^T
// fragments (rows loaded into registers, group A's waves Q and group B's dO,
// stored transposed), and the chunk's LSE (log2 units) and delta.  Stage use
// of chunk c: A reads it in M(c), V(c) and M(c+1), B one phase later each;
// so the stage is free from A's M(c+2) on.  In M(j) each wave requests chunk
// j+2 (into the stage of chunk j-2) and at the end of M(j) waits for its
// requests of chunk j+1, which group A then reads in M(j+1) after the
// barrier; in V(j) it stores chunk j+1's transposed fragments and, in wave
// 0, its LSE and delta.
#include <type_traits>

#include "box_common.h"

namespace vdsa {
namespace {

constexpr int HD = 128;
constexpr int KS = HD / 32;             // 32-wide head_dim steps of S and dP
constexpr int ND = HD / 16;             // 16-row head_dim tiles of dK^T and dV^T
constexpr int NW = 8;                   // waves per workgroup
constexpr int BLOCK_M = NW * 16;        // owned keys per workgroup
constexpr int CHUNK = 32;               // queries per chunk
constexpr int NFRAG = 2 * KS;           // (t, ks) fragments of Q and of dO per chunk
// LDS layout of one stage
constexpr int XF = 0;                   // Q fragments
constexpr int YF = NFRAG * 1024;        // dO fragments
constexpr int XT = 2 * NFRAG * 1024;    // Q^T fragments (dt)
constexpr int YT = XT + ND * 1024;      // dO^T fragments (dt)
constexpr int LD = YT + ND * 1024;      // 32 LSE (log2 units), then 32 delta
constexpr int STAGE = LD + 2 * CHUNK * 4;
constexpr int NSTAGE = 4;
constexpr int NLOAD = 5;                // vector-memory requests per wave per chunk
constexpr int PF = 3;                   // fragment pairs read ahead in an M phase
static_assert(NFRAG == NW, "one Q and one dO fragment per wave and chunk");
static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS");

// Lane n of each 16-lane row broadcast to the whole row (DPP row_newbcast:n).
template <int N>
__device__ __forceinline__ float row_bcast(int x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x150 + N, 0xF, 0xF, false));
}
// a[e] = x of lane e of the row, b[e] = x of lane 8 + e.
__device__ __forceinline__ void row_bcast8(int x, float (&a)[8], float (&b)[8]) {
  a[0] = row_bcast<0>(x); a[1] = row_bcast<1>(x); a[2] = row_bcast<2>(x); a[3] = row_bcast<3>(x);
  a[4] = row_bcast<4>(x); a[5] = row_bcast<5>(x); a[6] = row_bcast<6>(x); a[7] = row_bcast<7>(x);
  b[0] = row_bcast<8>(x); b[1] = row_bcast<9>(x); b[2] = row_bcast<10>(x); b[3] = row_bcast<11>(x);
  b[4] = row_bcast<12>(x); b[5] = row_bcast<13>(x); b[6] = row_bcast<14>(x); b[7] = row_bcast<15>(x);
}

// LIN: the iterated box is the whole grid in token order (dense keys: every
// query of the global branch), so query j is token j and a lane's rows sit at
// fixed offsets from the chunk's first token; else raster order over the box.
template <bool LIN>
__global__ __launch_bounds__(NW * 64) void box_attn_bwd_dkdv_pp_kernel(const BoxBwdParams P) {
  __shared__ __attribute__((aligned(16))) char lds[NSTAGE * STAGE];
  const BoxAttnParams& g = P.g;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int G = lane >> 4;
  const bool grp_b = wave >= NW / 2;   // waves w and w + 4 share a SIMD

  // ---- which (batch, head, key tile, key block) this workgroup owns
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
  if (o0 >= ovol) return;  // uniform over the workgroup, before any barrier
  const int ivol = ib.et * ib.eh * ib.ew;
  const int nch = (ivol + CHUNK - 1) / CHUNK;

  const char* kp = (const char*)P.k + 2 * (b * P.k_sb + h * P.k_sh);
  const char* vp = (const char*)P.v + 2 * (b * P.v_sb + h * P.v_sh);
  const char* qp = (const char*)P.q + 2 * (b * P.q_sb + h * P.q_sh);
  const char* dop = (const char*)P.dout + 2 * (b * P.do_sb + h * P.do_sh);
  const uint32_t q_row = 2u * (uint32_t)P.q_sn, do_row = 2u * (uint32_t)P.do_sn;
  const uint32_t n_q = (uint32_t)(g.kT * g.kH * g.kW);   // the iterated tokens: queries on the key grid
  const __amdgpu_buffer_rsrc_t qrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)qp, 0, (int)((n_q - 1u) * q_row + 2u * HD), BUF_FLAGS);
  const __amdgpu_buffer_rsrc_t dorsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)dop, 0, (int)((n_q - 1u) * do_row + 2u * HD), BUF_FLAGS);
  const float* lse_bh = P.lse + ((int64_t)b * g.heads + h) * P.n_q;
  const float* del_bh = P.delta + ((int64_t)b * g.heads + h) * P.n_q;
  constexpr float LOG2E = 1.4426950408889634f;
  const float cl2 = g.scale_log2e;

  // ---- this lane's key: column l16 of the wave's tile
  const int jo = o0 + wave * 16 + l16;
  const bool own_valid = jo < ovol;
  // A wave whose keys all lie past the tile (the last workgroup of a tile
  // whose size is not a multiple of BLOCK_M) keeps its requests, stores and
  // barriers but skips its products and softmax terms.
  const bool active = o0 + wave * 16 < ovol;   // uniform over the wave
  uint32_t own_tok;
  bf16x8 kf[KS], vf[KS];
  {
    const int j = min(jo, ovol - 1);
    const int plane = ob.eh * ob.ew;
    const int jt = j / plane;
    const int r = j - jt * plane;
    const int jh = r / ob.ew;
    const int jw = r - jh * ob.ew;
    own_tok = q_token(g, ob.t0 + jt, ob.h0 + jh, ob.w0 + jw);
    const char* ks_src = kp + own_tok * (2u * (uint32_t)P.k_sn) + 16 * G;
    const char* vs_src = vp + own_tok * (2u * (uint32_t)P.v_sn) + 16 * G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(ks_src + 64 * ks));
      vf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(vs_src + 64 * ks));
    }
  }

  // ---- iterated box addressing: query j of the box -> token
  const FastDiv fd_plane = make_fastdiv((uint32_t)(ib.eh * ib.ew));
  const FastDiv fd_row = make_fastdiv((uint32_t)ib.ew);
  auto iter_token = [&](int j) -> uint32_t {
    j = min(j, ivol - 1);   // past the box: repeat the last query; masked later
    const uint32_t jt = fast_div((uint32_t)j, fd_plane);
    const uint32_t r = (uint32_t)j - jt * fd_plane.d;
    const uint32_t jh = fast_div(r, fd_row);
    const uint32_t jw = r - jh * fd_row.d;
    return k_token(g, ib.t0 + (int)jt, ib.h0 + (int)jh, ib.w0 + (int)jw);
  };
  auto stage_of = [&](int c) -> char* { return lds + (c % NSTAGE) * STAGE; };

  // Requests of one chunk, NLOAD per wave: the wave's Q and dO fragment
  // (fragment f = t*KS + ks = wave: lane L = 16G + p fetches query row
  // 8*(p/4) + 4t + p%4, head_dim chunk 4ks + G), two rows of Q (group A) or
  // dO (group B) for the transposed copies (rows 2vk, 2vk+1, head_dim chunk
  // vc), and the chunk's LSE (lanes 0-31) and delta (lanes 32-63).
  const int frag_t = wave / KS, frag_ks = wave % KS;
  const int frag_row = 8 * (l16 >> 2) + (l16 & 3) + 4 * frag_t;
  const uint32_t frag_col = (uint32_t)(4 * frag_ks + G) * 16u;
  const int u = tid & 255;
  const int vk = u % 16, vc = u / 16;
  const __amdgpu_buffer_rsrc_t trsrc = grp_b ? dorsrc : qrsrc;
  const uint32_t t_row = grp_b ? do_row : q_row;
  const float* ld_src = lane < 32 ? lse_bh : del_bh;
  // Two register sets, by chunk parity (a compile-time index: the set of
  // chunk c+1 waits for its store while chunk c+2's requests are in flight).
  u32x4 treg[2][2];   // [chunk parity][row]
  float ldreg[2];
  auto load_chunk = [&](int c, auto par) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    char* st = stage_of(c);
    // rows past the box repeat its last token (their terms are masked)
    auto lin_tok = [&](int r) { return (uint32_t)min(c * CHUNK + r, ivol - 1); };
    const uint32_t my_tok = LIN ? lin_tok(lane & 31) : iter_token(c * CHUNK + (lane & 31));
    const uint32_t ftok = LIN ? lin_tok(frag_row) : (uint32_t)__shfl((int)my_tok, frag_row, 64);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, (lds_void*)(st + XF + wave * 1024), 16,
                                             (int)(ftok * q_row + frag_col), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(dorsrc, (lds_void*)(st + YF + wave * 1024), 16,
                                             (int)(ftok * do_row + frag_col), 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t tok = LIN ? lin_tok(2 * vk + i) : (uint32_t)__shfl((int)my_tok, 2 * vk + i, 64);
      treg[PAR][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(trsrc, (int)(tok * t_row + vc * 16), 0, 0));
    }
    ldreg[PAR] = ld_src[my_tok];
  };
  // Every chunk's M phase requests chunk c+2, also past the last chunk
  // (clamped rows into a stage no later phase reads), so that every wave
  // always has exactly one chunk's requests in flight after its wait and the
  // compiler's own wait counts see the same request stream on every path.
  auto vm_wait_keep_one = [&] { __builtin_amdgcn_s_waitcnt(wait_enc(NLOAD, 15)); };

  // Transposed copies: element e of the thread's two rows (head_dim 8vc + e)
  // goes to piece 8(vc&1) + (e ^ sig) of head_dim tile vc/2, row group
  // 2vk/8 (the forward's XOR-swizzled V^T layout).
  const int vk0 = 2 * vk;
  const int vsig = ((vk0 >> 3) << 1);
  const uint32_t vw_base =
      (uint32_t)((grp_b ? YT : XT) + (vk0 >> 3) * 256 + (vk0 & 7) * 2 + (vc >> 1) * 1024 + (vc & 1) * 128);
  auto store_chunk = [&](int c, auto par) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    const uint32_t sbase = (uint32_t)(uintptr_t)stage_of(c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low bf16 halves
      *(lds_u32*)(uintptr_t)(sbase + vw_base + (uint32_t)((e ^ vsig) * 16)) =
          __builtin_amdgcn_perm(treg[PAR][1][e >> 1], treg[PAR][0][e >> 1], sel);
    }
    if (wave == 0) {
      const float x = ldreg[PAR];
      *(float*)(stage_of(c) + LD + 4 * lane) = lane < 32 ? x * LOG2E : x;
    }
  };
  // A-operand read offset of a transposed fragment: piece 16G + (l16 ^ (G << 1))
  const int t_rd = (16 * G + (l16 ^ (G << 1))) * 16;

  f32x4 dk_acc[ND], dv_acc[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    dk_acc[dt] = f32x4{};
    dv_acc[dt] = f32x4{};
  }
  f32x4 s[2], dp[2];   // register v of tile t: query row 8G + 4t + v, key l16
  bf16x8 pb, dsb;      // P and dS of the previous chunk as B operands (queries 8G .. 8G+7)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pb[e] = (__bf16)0.f;
    dsb[e] = (__bf16)0.f;
  }

  // ---- M phase: the dK/dV products of the chunk in st_g (steps 0..7: Q^T
  // and dO^T tile dt; P and dS zero in the first phase) and, WITH_S, the S
  // and dP products of the chunk in st_s (steps 8..15: Q and dO fragment
  // (t, ks) in (ks, t) order, dependent products four MFMAs apart).
  // Fragment pairs are read PF steps ahead.
  bf16x8 fx[16], fy[16];
  auto mphase = [&](const char* st_g, const char* st_s, auto with_s_tag) __attribute__((always_inline)) {
    constexpr bool WITH_S = decltype(with_s_tag)::value;
    constexpr int i1 = WITH_S ? 16 : 8;
    auto rd = [&](int i) __attribute__((always_inline)) {
      if (i < 8) {
        fx[i] = lds_frag(st_g + XT + t_rd + i * 1024);
        fy[i] = lds_frag(st_g + YT + t_rd + i * 1024);
      } else {
        const int j = i - 8, f = (j & 1) * KS + (j >> 1);
        fx[i] = lds_frag(st_s + XF + f * 1024 + lane * 16);
        fy[i] = lds_frag(st_s + YF + f * 1024 + lane * 16);
      }
    };
    if constexpr (WITH_S) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = f32x4{};
        dp[t] = f32x4{};
      }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) rd(i);
#pragma unroll
    for (int i = 0; i < i1; ++i) {
      if (i + PF < i1) rd(i + PF);
      __builtin_amdgcn_sched_barrier(0);
      if (i < 8) {
        dk_acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx[i], dsb, dk_acc[i], 0, 0, 0);
        dv_acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fy[i], pb, dv_acc[i], 0, 0, 0);
      } else {
        const int j = i - 8, ks = j >> 1, t = j & 1;
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx[i], kf[ks], s[t], 0, 0, 0);
        dp[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fy[i], vf[ks], dp[t], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      pin(dk_acc[dt]);
      pin(dv_acc[dt]);
    }
    if constexpr (WITH_S) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        pin(s[t]);
        pin(dp[t]);
      }
    }
  };

  // ---- V phase: P and dS of chunk c from its S and dP; nvalid = queries of
  // the box from this chunk on (masking only in the last, partial chunk).
  // Each lane of 16-lane row G reads one value, LSE (lanes 0-7) or delta
  // (lanes 8-15) of query row 8G + (lane & 7); row broadcasts (DPP
  // row_newbcast) hand every lane of the row all sixteen.
  const int ld_rd = LD + 4 * (8 * G + (l16 & 7)) + (l16 >> 3) * (4 * CHUNK);
  auto vphase = [&](const char* st, int nvalid, auto partial_tag) __attribute__((always_inline)) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int x = *(const int*)(st + ld_rd);
    float l2s[8], dls[8];
    row_bcast8(x, l2s, dls);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = e >> 2, v = e & 3;
      const float l2 = l2s[e];
      const float dl = dls[e];
      float pv = __builtin_amdgcn_exp2f(fmaf(s[t][v], cl2, -l2));
      if constexpr (PARTIAL) {
        if (8 * G + e >= nvalid) pv = 0.f;
      }
      pb[e] = (__bf16)pv;
      dsb[e] = (__bf16)(pv * (dp[t][v] - dl));
    }
    pin(pb);
    pin(dsb);
  };

  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  // ---- prologue: chunk 0 complete in LDS, chunk 1 in flight
  load_chunk(0, Even{});
  load_chunk(1, Odd{});
  vm_wait_keep_one();
  store_chunk(0, Even{});
  phase_barrier();
  if (grp_b) phase_barrier();

  // chunk c, of parity PAR (c % 2); ACTIVE: the wave computes (a compile-time
  // flag: the whole walk is instantiated with and without the compute)
  auto do_chunk = [&](int c, auto par, auto partial_tag, auto active_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool ACTIVE = decltype(active_tag)::value;
    using Next = std::integral_constant<int, PAR ^ 1>;
    // M(c)
    load_chunk(c + 2, par);
    // (chunk 0's M phase multiplies zero P and dS into chunk 0's finite
    // transposed fragments: it adds exactly zero)
    if constexpr (ACTIVE) mphase(stage_of(c > 0 ? c - 1 : 0), stage_of(c), std::true_type{});
    vm_wait_keep_one();   // this wave's requests of chunk c+1 have landed
    phase_barrier();
    // V(c)
    if (c + 1 < nch) store_chunk(c + 1, Next{});
    if constexpr (ACTIVE) vphase(stage_of(c), ivol - c * CHUNK, partial_tag);
    phase_barrier();
  };
  const bool last_partial = ivol % CHUNK != 0;
  const int nfull = last_partial ? nch - 1 : nch;
  auto walk = [&](auto active_tag) __attribute__((always_inline)) {
    constexpr bool ACTIVE = decltype(active_tag)::value;
    int c = 0;
    for (; c + 1 < nfull; c += 2) {
      do_chunk(c, Even{}, std::false_type{}, active_tag);
      do_chunk(c + 1, Odd{}, std::false_type{}, active_tag);
    }
    if (c < nfull) do_chunk(c++, Even{}, std::false_type{}, active_tag);
    if (last_partial) {
      if (c & 1)
        do_chunk(c, Odd{}, std::true_type{}, active_tag);
      else
        do_chunk(c, Even{}, std::true_type{}, active_tag);
    }
    if constexpr (ACTIVE) mphase(stage_of(nch - 1), stage_of(nch - 1), std::false_type{});
  };
  if (active)
    walk(std::true_type{});
  else
    walk(std::false_type{});
  __builtin_amdgcn_s_waitcnt(wait_enc(0, 15));   // the requests past the end have landed
  if (!grp_b) phase_barrier();

  // ---- epilogue: register v of tile dt is head_dim 16dt + 4G + v of the
  // lane's key
  if (!own_valid) return;
  const float s1 = P.scale;
  if (P.grad_f32) {
    float* dk = (float*)P.dk + b * P.dk_sb + h * P.dk_sh + (int64_t)own_tok * P.dk_sn + 4 * G;
    float* dv = (float*)P.dv + b * P.dv_sb + h * P.dv_sh + (int64_t)own_tok * P.dv_sn + 4 * G;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      *(f32x4*)(dk + 16 * dt) = dk_acc[dt] * s1;
      *(f32x4*)(dv + 16 * dt) = dv_acc[dt];
    }
  } else {
    char* dk = (char*)P.dk + 2 * (b * P.dk_sb + h * P.dk_sh) + own_tok * (2u * (uint32_t)P.dk_sn) + 8 * G;
    char* dv = (char*)P.dv + 2 * (b * P.dv_sb + h * P.dv_sh) + own_tok * (2u * (uint32_t)P.dv_sn) + 8 * G;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      bf16x4 kv, vv;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        kv[v] = (__bf16)(dk_acc[dt][v] * s1);
        vv[v] = (__bf16)dv_acc[dt][v];
      }
      *(u32x2*)(dk + 32 * dt) = __builtin_bit_cast(u32x2, kv);
      *(u32x2*)(dv + 32 * dt) = __builtin_bit_cast(u32x2, vv);
    }
  }
}

}  // namespace

hipError_t launch_attn_bwd_dkdv_pp(const BoxBwdParams& p, hipStream_t stream) {
  if (p.g.dense_keys && !(p.g.rlT | p.g.rlH | p.g.rlW))
    hipLaunchKernelGGL(box_attn_bwd_dkdv_pp_kernel<true>, dim3(p.g.total_wg), dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(box_attn_bwd_dkdv_pp_kernel<false>, dim3(p.g.total_wg), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

int attn_bwd_dkdv_pp_block_m() { return BLOCK_M; }

}  // namespace vdsa
