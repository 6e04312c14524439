// dQ pass of the tile-window ("box") attention backward, bf16 in/out, head_dim
// 128, fp32 accumulation, with the matrix-core work of one half of the
// workgroup overlapping the softmax terms of the other half.
//
// What it computes: for the queries a workgroup owns, over the keys of their
// key box,
//   P = exp(scale q.k - LSE),  dP = dO.v,  dS = P * (dP - delta),
//   dQ = scale dS K.
// Every wave owns two 16-query tiles (Q and dO resident as MFMA B operands,
// the queries' LSE and delta in registers) and works on 32-key chunks of the
// key box: S^T = K Q^T and dP^T = V dO^T (rows: keys, columns: the wave's
// queries), then dQ^T += K^T dS^T.  Fragment layouts are those of the dK/dV
// pass (attn_bwd_dkdv_pp.hip) with keys and queries exchanged.
//
// Schedule.  Eight waves, two per SIMD: group A (waves 0-3) and group B
// (waves 4-7) own the same 128 queries (waves w and w + 4 the same two
// tiles); A takes the even chunks, B the odd ones.  Time runs in slots
// separated by workgroup barriers; in slot j the group of chunk j runs
//   M(j)  matrix-core phase: dQ products of its previous chunk j-2, S and dP
//         of chunk j (48 MFMAs)
// while the other group runs
//   V(j-1)  P and dS of chunk j-1 (VALU and exp),
// so on each SIMD one wave issues MFMAs while the other computes its softmax
// terms.  There are nch + 2 slots for nch chunks (the last two carry the
// groups' final dQ products); each group idles in the slots it has no
// phase in.  After the last slot group B hands its partial dQ^T to group A
// through LDS, and A writes the sum.
//
// LDS: a ring of six stages, one chunk each: K and V fragments (direct
// global->LDS loads) and K^T fragments (rows loaded into registers, stored
// transposed).  Chunk x's K and V fragments are read in slot x, its K^T
// fragments in slot x+2, so its stage is free from slot x+3 on.  In M(j) the
// waves of the group request chunk j+3 (into the stage of chunk j-3); at the
// end of M(j+2) they wait for those requests (the other group reads the K
// and V fragments in slot j+3) and in V(j+2), slot j+3, they store the
// chunk's K^T fragments (first read in slot j+5).  Chunks 0-2 are loaded
// before the first slot.
#include <type_traits>

#include "box_common.h"

namespace vdsa {
namespace {

constexpr int HD = 128;
constexpr int KS = HD / 32;             // 32-wide head_dim steps of S and dP
constexpr int ND = HD / 16;             // 16-row head_dim tiles of dQ^T
constexpr int NW = 8;                   // waves per workgroup
constexpr int OT = 2;                   // 16-query tiles per wave
constexpr int BLOCK_M = (NW / 2) * 16 * OT;   // owned queries per workgroup (both groups the same)
constexpr int CHUNK = 32;               // keys per chunk
constexpr int NFRAG = 2 * KS;           // (t, ks) fragments of K and of V per chunk
// LDS layout of one stage
constexpr int XF = 0;                   // K fragments
constexpr int YF = NFRAG * 1024;        // V fragments
constexpr int XT = 2 * NFRAG * 1024;    // K^T fragments (dt)
constexpr int STAGE = XT + ND * 1024;
constexpr int NSTAGE = 6;
constexpr int AHEAD = 3;                // a group's M(j) requests chunk j + AHEAD
constexpr int FPW = NFRAG / (NW / 2);   // K and V fragments each loaded per wave of a group
constexpr int NLOAD = 2 * FPW + 2;      // vector-memory requests per wave per chunk
constexpr int PF = 2;                   // fragment pairs read ahead in an M phase
static_assert(FPW * (NW / 2) == NFRAG, "fragments per wave");
static_assert(NSTAGE * STAGE <= 160 * 1024, "LDS");
static_assert((NW / 2) * 64 * OT * ND * 16 <= NSTAGE * STAGE, "partial dQ hand-over fits the ring");

// LIN: the iterated box is the whole key grid in token order (dense keys:
// the global branch's pooled keys), so key j is token j and a lane's rows sit
// at fixed offsets from the chunk's first token; else raster order over the box.
template <bool LIN>
__global__ __launch_bounds__(NW * 64) void box_attn_bwd_dq_pp_kernel(const BoxBwdParams P) {
  __shared__ __attribute__((aligned(16))) char lds[NSTAGE * STAGE];
  const BoxAttnParams& g = P.g;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w4 = wave & 3;                // wave within its group
  const int l16 = lane & 15;
  const int G = lane >> 4;
  const int grp = wave >= NW / 2 ? 1 : 0;   // waves w and w + 4 share a SIMD

  // ---- which (batch, head, query tile, query block) this workgroup owns
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

  const char* qp = (const char*)P.q + 2 * (b * P.q_sb + h * P.q_sh);
  const char* dop = (const char*)P.dout + 2 * (b * P.do_sb + h * P.do_sh);
  const char* kp = (const char*)P.k + 2 * (b * P.k_sb + h * P.k_sh);
  const char* vp = (const char*)P.v + 2 * (b * P.v_sb + h * P.v_sh);
  const uint32_t k_row = 2u * (uint32_t)P.k_sn, v_row = 2u * (uint32_t)P.v_sn;
  const uint32_t n_k = (uint32_t)(g.kT * g.kH * g.kW);
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, (int)((n_k - 1u) * k_row + 2u * HD), BUF_FLAGS);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, (int)((n_k - 1u) * v_row + 2u * HD), BUF_FLAGS);
  const float* lse_bh = P.lse + ((int64_t)b * g.heads + h) * P.n_q;
  const float* del_bh = P.delta + ((int64_t)b * g.heads + h) * P.n_q;
  constexpr float LOG2E = 1.4426950408889634f;
  const float cl2 = g.scale_log2e;

  // ---- this lane's queries: column l16 of each of the wave's two tiles
  bool own_valid[OT];
  uint32_t own_tok[OT];
  bf16x8 qf[OT][KS], dof[OT][KS];
  float own_lse2[OT], own_del[OT];
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    const int jo = o0 + (w4 * OT + ot) * 16 + l16;
    own_valid[ot] = jo < ovol;
    const int j = min(jo, ovol - 1);
    const int plane = ob.eh * ob.ew;
    const int jt = j / plane;
    const int r = j - jt * plane;
    const int jh = r / ob.ew;
    const int jw = r - jh * ob.ew;
    own_tok[ot] = q_token(g, ob.t0 + jt, ob.h0 + jh, ob.w0 + jw);
    const char* qs = qp + own_tok[ot] * (2u * (uint32_t)P.q_sn) + 16 * G;
    const char* ds = dop + own_tok[ot] * (2u * (uint32_t)P.do_sn) + 16 * G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ot][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qs + 64 * ks));
      dof[ot][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(ds + 64 * ks));
    }
    own_lse2[ot] = lse_bh[own_tok[ot]] * LOG2E;
    own_del[ot] = del_bh[own_tok[ot]];
  }

  // A wave whose queries all lie past the tile (the last workgroup of a tile
  // whose size is not a multiple of BLOCK_M) keeps its requests, stores and
  // barriers but skips its products and softmax terms (its partner in the
  // other group owns the same queries and skips them too).
  const bool active = o0 + w4 * OT * 16 < ovol;   // uniform over the wave

  // ---- key box addressing: key j of the box -> token
  const FastDiv fd_plane = make_fastdiv((uint32_t)(ib.eh * ib.ew));
  const FastDiv fd_row = make_fastdiv((uint32_t)ib.ew);
  auto iter_token = [&](int j) -> uint32_t {
    j = min(j, ivol - 1);   // past the box: repeat the last key; masked later
    const uint32_t jt = fast_div((uint32_t)j, fd_plane);
    const uint32_t r = (uint32_t)j - jt * fd_plane.d;
    const uint32_t jh = fast_div(r, fd_row);
    const uint32_t jw = r - jh * fd_row.d;
    return k_token(g, ib.t0 + (int)jt, ib.h0 + (int)jh, ib.w0 + (int)jw);
  };
  auto stage_of = [&](int c) -> char* { return lds + (c % NSTAGE) * STAGE; };

  // Requests of one chunk by the four waves of a group, NLOAD per wave: the
  // wave's FPW K and V fragments (fragment f = t*KS + ks: lane L = 16G + p
  // fetches key row 8*(p/4) + 4t + p%4, head_dim chunk 4ks + G) and two K
  // rows for the transposed copy (rows 2vk, 2vk+1, head_dim chunk vc).
  const int frow_base = 8 * (l16 >> 2) + (l16 & 3);
  const int u = tid & 255;
  const int vk = u % 16, vc = u / 16;
  // Two register sets of the K rows by the parity of the group's chunk
  // index (a compile-time index): a set waits two slots for its store while
  // the next chunk's requests are in flight.
  u32x4 treg[2][2];
  auto load_chunk = [&](int c, auto par) {
    constexpr int PAR = decltype(par)::value;
    char* st = stage_of(c);
    // rows past the box repeat its last token (their terms are masked)
    auto lin_tok = [&](int r) { return (uint32_t)min(c * CHUNK + r, ivol - 1); };
    const uint32_t my_tok = LIN ? 0u : iter_token(c * CHUNK + (lane & 31));
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
      const int f = w4 * FPW + i;
      const int t = f / KS, ks = f % KS;
      const uint32_t ftok = LIN ? lin_tok(frow_base + 4 * t) : (uint32_t)__shfl((int)my_tok, frow_base + 4 * t, 64);
      const uint32_t col = (uint32_t)(4 * ks + G) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)(st + XF + f * 1024), 16, (int)(ftok * k_row + col),
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lds_void*)(st + YF + f * 1024), 16, (int)(ftok * v_row + col),
                                               0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t tok = LIN ? lin_tok(2 * vk + i) : (uint32_t)__shfl((int)my_tok, 2 * vk + i, 64);
      treg[PAR][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krsrc, (int)(tok * k_row + vc * 16), 0, 0));
    }
  };
  // Transposed copy: element e of the thread's two rows (head_dim 8vc + e)
  // goes to piece 8(vc&1) + (e ^ sig) of head_dim tile vc/2, row group 2vk/8.
  const int vk0 = 2 * vk;
  const int vsig = ((vk0 >> 3) << 1);
  const uint32_t vw_base = (uint32_t)(XT + (vk0 >> 3) * 256 + (vk0 & 7) * 2 + (vc >> 1) * 1024 + (vc & 1) * 128);
  auto store_chunk = [&](int c, auto par) {
    constexpr int PAR = decltype(par)::value;
    const uint32_t sbase = (uint32_t)(uintptr_t)stage_of(c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low bf16 halves
      *(lds_u32*)(uintptr_t)(sbase + vw_base + (uint32_t)((e ^ vsig) * 16)) =
          __builtin_amdgcn_perm(treg[PAR][1][e >> 1], treg[PAR][0][e >> 1], sel);
    }
  };
  // A-operand read offset of a transposed fragment: piece 16G + (l16 ^ (G << 1))
  const int t_rd = (16 * G + (l16 ^ (G << 1))) * 16;
  auto vm_wait_keep_one = [&] { __builtin_amdgcn_s_waitcnt(wait_enc(NLOAD, 15)); };

  f32x4 acc[ND][OT];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int ot = 0; ot < OT; ++ot) acc[dt][ot] = f32x4{};
  f32x4 s[2][OT], dp[2][OT];   // register v of tile (t, ot): key row 8G + 4t + v, query l16 of tile ot
  bf16x8 dsb[OT];              // dS^T of the group's previous chunk as B operands (keys 8G .. 8G+7)
#pragma unroll
  for (int ot = 0; ot < OT; ++ot)
#pragma unroll
    for (int e = 0; e < 8; ++e) dsb[ot][e] = (__bf16)0.f;

  // ---- M phase: the dQ products of the chunk in st_g (steps 0..7: K^T
  // tile dt; dS zero in a group's first phase) and, WITH_S, the S and dP
  // products of the chunk in st_s (steps 8..15: K and V fragment (t, ks) in
  // (ks, t) order).  Fragments are read PF steps ahead.
  bf16x8 fx[16], fy[16];
  auto mphase = [&](const char* st_g, const char* st_s, auto with_s_tag) {
    constexpr bool WITH_S = decltype(with_s_tag)::value;
    constexpr int i1 = WITH_S ? 16 : 8;
    auto rd = [&](int i) __attribute__((always_inline)) {
      if (i < 8) {
        fx[i] = lds_frag(st_g + XT + t_rd + i * 1024);
      } else {
        const int j = i - 8, f = (j & 1) * KS + (j >> 1);
        fx[i] = lds_frag(st_s + XF + f * 1024 + lane * 16);
        fy[i] = lds_frag(st_s + YF + f * 1024 + lane * 16);
      }
    };
    if constexpr (WITH_S) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) {
          s[t][ot] = f32x4{};
          dp[t][ot] = f32x4{};
        }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) rd(i);
#pragma unroll
    for (int i = 0; i < i1; ++i) {
      if (i + PF < i1) rd(i + PF);
      __builtin_amdgcn_sched_barrier(0);
      if (i < 8) {
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) acc[i][ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx[i], dsb[ot], acc[i][ot], 0, 0, 0);
      } else {
        const int j = i - 8, ks = j >> 1, t = j & 1;
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) {
          s[t][ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx[i], qf[ot][ks], s[t][ot], 0, 0, 0);
          dp[t][ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fy[i], dof[ot][ks], dp[t][ot], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) pin(acc[dt][ot]);
    if constexpr (WITH_S) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) {
          pin(s[t][ot]);
          pin(dp[t][ot]);
        }
    }
  };

  // ---- V phase: dS^T of chunk c from its S^T and dP^T; keys of the box
  // from this chunk on: nvalid (masking only in the last, partial chunk).
  auto vphase_impl = [&](int nvalid, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int lim = nvalid - 8 * G;   // rows e >= lim of this lane are past the box
#pragma unroll
    for (int ot = 0; ot < OT; ++ot) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = e >> 2, v = e & 3;
        float pv = __builtin_amdgcn_exp2f(fmaf(s[t][ot][v], cl2, -own_lse2[ot]));
        if constexpr (PARTIAL) {
          if (e >= lim) pv = 0.f;
        }
        dsb[ot][e] = (__bf16)(pv * (dp[t][ot][v] - own_del[ot]));
      }
      pin(dsb[ot]);
    }
  };
  auto vphase = [&](int nvalid) {
    if (nvalid >= CHUNK)   // uniform: every chunk but a partial last one
      vphase_impl(nvalid, std::false_type{});
    else
      vphase_impl(nvalid, std::true_type{});
  };

  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  // ---- prologue: chunks 0-2 complete in LDS (group A loads 0 and 2, B 1)
  if (grp == 0) {
    load_chunk(0, Even{});
    load_chunk(2, Odd{});
  } else {
    load_chunk(1, Even{});
  }
  __builtin_amdgcn_s_waitcnt(wait_enc(0, 15));
  if (grp == 0) {
    store_chunk(0, Even{});
    store_chunk(2, Odd{});
  } else {
    store_chunk(1, Even{});
  }
  phase_barrier();

  // ---- the group's chunks c = grp + 2k.  M(c) in slot c requests chunk c+3
  // into set k%2; V(c) in slot c+1 stores chunk c+1 (requested in M(c-2),
  // set (k-1)%2; chunks up to 2 came with the prologue).
  if (grp == 1) phase_barrier();   // slot 0: group A's M(0)
  auto do_chunk = [&](int c, auto par) {
    constexpr int PAR = decltype(par)::value;
    using Prev = std::integral_constant<int, PAR ^ 1>;
    // M(c), slot c
    load_chunk(c + AHEAD, par);
    // (a group's first M phase multiplies zero dS into the finite K^T
    // fragments of its own chunk: it adds exactly zero)
    if (active) mphase(stage_of(c >= 2 ? c - 2 : c), stage_of(c), std::true_type{});
    vm_wait_keep_one();   // this wave's requests of chunk c+1 have landed
    phase_barrier();
    // V(c), slot c+1
    if (c >= 2) store_chunk(c + 1, Prev{});
    if (active) vphase(ivol - c * CHUNK);
    phase_barrier();
  };
  int c = grp;
  for (; c + 2 < nch; c += 4) {
    do_chunk(c, Even{});
    do_chunk(c + 2, Odd{});
  }
  if (c < nch) do_chunk(c, Even{});
  // the group's final dQ products (its last chunk), slot c_last + 2
  const int n_own = (nch - grp + 1) / 2;   // chunks of this group
  if (n_own > 0) {
    const int c_last = grp + 2 * (n_own - 1);
    if (active) mphase(stage_of(c_last), stage_of(c_last), std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(wait_enc(0, 15));   // every request (also past the end) has landed
  phase_barrier();
  // every group passes nch + 2 slot barriers: grp + 2 n_own + 1 so far
  if (grp + 2 * n_own + 1 < nch + 2) phase_barrier();

  // ---- group B hands its partial dQ^T to group A through the free ring:
  // tile (dt, ot) of wave w4 at ((dt*OT + ot)*4 + w4) KB + 16 lane
  auto hand = [&](int dt, int ot) { return lds + (((dt * OT + ot) * 4 + w4) * 64 + lane) * 16; };
  if (grp == 1) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) *(f32x4*)hand(dt, ot) = acc[dt][ot];
  }
  __syncthreads();
  if (grp == 1) return;

  // ---- epilogue (group A): register v of tile (dt, ot) is head_dim
  // 16dt + 4G + v of the lane's query of tile ot
  const float s1 = P.scale;
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    if (!own_valid[ot]) continue;
    char* dst = (char*)P.dq + 2 * (b * P.dq_sb + h * P.dq_sh) + own_tok[ot] * (2u * (uint32_t)P.dq_sn) + 8 * G;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const f32x4 sum = acc[dt][ot] + *(const f32x4*)hand(dt, ot);
      bf16x4 ov;
#pragma unroll
      for (int v = 0; v < 4; ++v) ov[v] = (__bf16)(sum[v] * s1);
      *(u32x2*)(dst + 32 * dt) = __builtin_bit_cast(u32x2, ov);
    }
  }
}

}  // namespace

hipError_t launch_attn_bwd_dq_pp(const BoxBwdParams& p, hipStream_t stream) {
  if (p.g.dense_keys && !(p.g.rlT | p.g.rlH | p.g.rlW))
    hipLaunchKernelGGL(box_attn_bwd_dq_pp_kernel<true>, dim3(p.g.total_wg), dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(box_attn_bwd_dq_pp_kernel<false>, dim3(p.g.total_wg), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

int attn_bwd_dq_pp_block_m() { return BLOCK_M; }

}  // namespace vdsa
