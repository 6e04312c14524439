// Tile-window ("box") attention forward for head_dim 128, bf16 in/out, fp32
// accumulation, 384 queries per workgroup (one 6x8x8 query tile), with the
// matrix-core work of one half of the workgroup overlapping the softmax of
// the other half.
//
// Same method as the other box kernels: the keys of a query tile (the union of
// the key tiles in its window, Sliding Tile Attention, arXiv 2502.04507,
// abstract) form one box of tokens, walked in 64-key blocks (two 32-key
// chunks) with every key's address computed from its box coordinates; each
// wave owns three 16-query tiles of v_mfma_f32_16x16x32_bf16 (48 queries).
//
// Schedule.  Eight waves, two per SIMD: group A (waves 0-3) and group B
// (waves 4-7) hold one wave on every SIMD each.  Every wave alternates two
// kinds of phase:
//   M  matrix-core phase: P*V of the previous chunk (plus the row sums of P,
//      below) and S^T = K Q^T of the current chunk, 51 MFMAs;
//   V  softmax phase of the current chunk (VALU and exp only).
// Group B runs one phase behind group A and a workgroup barrier separates
// consecutive phases, so on each SIMD one wave issues MFMAs while the other
// runs its softmax.  Every wave passes the same number of barriers: B takes
// one extra before its first phase, A one after its last.
//
// Per wave and 64-key block b the phases are
//   M(b,0): P*V(b-1, chunk 1), S(b, chunk 0)   V(b,0): softmax(b, chunk 0)
//   M(b,1): P*V(b, chunk 0),   S(b, chunk 1)   V(b,1): softmax(b, chunk 1)
// with one trailing P*V after the last block.
//
// LDS: a ring of three stages of (16 KB K fragments + 16 KB V^T fragments),
// each fragment the 1 KB operand of one MFMA, read as one contiguous 1 KB per
// wave.  Block b+2 is requested at the start of V(b,1), the softmax phase
// with the most slack: K by direct global->LDS loads, V into registers,
// stored transposed into its V^T fragments in V(b+1,0).  K of block b+1 must
// have landed before group A's M(b+1,0): A waits for it at the end of V(b,1)
// keeping the loads of block b+2 in flight, B at the end of M(b,1) (the same
// barrier), before it requests block b+2.  The stage a block overwrites was
// last read at least three phases before its first write.
//
// Fragment layouts (lane L = 16G + p of a wave):
//   K fragment (c, t, ks): lane L holds head_dim [32ks + 8G, +8) of key row
//     8*(p/4) + 4t + p%4 of chunk c, so that after the two 16-row tiles t the
//     lane group G holds keys 8G .. 8G+7 of its query;
//   V^T fragment (c, dt): lane L holds keys 8G .. 8G+7 of chunk c at head_dim
//     16dt + p, stored at piece 16G + (p ^ ((G << 1) | c)) so that the
//     transposing stores are free of bank conflicts.
//
// Softmax: probabilities are exp2(s*scale*log2(e) - m) for a per-query
// reference m that is raised only when some score of the wave exceeds it by
// more than RESCALE_MARGIN (log2 units), so probabilities stay below
// 2^RESCALE_MARGIN and the final normalisation by the same reference is
// exact.  Each lane tests its own eight scores of a query (a chunk maximum
// exceeds the threshold exactly when one of its lanes' maxima does); the
// cross-lane maximum is formed only when some lane fires.  The row sums of P
// (the softmax denominators) come from the matrix core: an all-ones A operand
// times the P^T operand puts each query's chunk sum in every row of a 16x16
// product, accumulated in fp32 like O^T.
#include <type_traits>

#include "box_common.h"

namespace vdsa {
namespace {

constexpr int HD = 128;
constexpr int BLOCK_N = 64;             // keys per block
constexpr int QT = 3;                   // 16-query tiles per wave
constexpr int NW = 8;                   // waves per workgroup
constexpr int BLOCK_M = NW * 16 * QT;   // 384 queries per workgroup
constexpr int KS = HD / 32;             // 32-wide head_dim steps of S^T
constexpr int ND = HD / 16;             // 16-row head_dim tiles of O^T
constexpr int NFRAG_K = 2 * 2 * KS;     // (chunk, t, ks)
constexpr int K_STAGE = NFRAG_K * 1024;
constexpr int V_STAGE = 2 * ND * 1024;  // (chunk, dt)
constexpr int STAGE = K_STAGE + V_STAGE;
constexpr int NSTAGE = 3;
constexpr int KDMA_W = NFRAG_K / NW;                 // K fragments loaded per wave per block
constexpr int VPT = BLOCK_N * HD / 8 / (NW * 64);    // V 16-byte chunks per thread
constexpr int NKG = BLOCK_N / VPT;                   // threads per V head_dim chunk
constexpr int NLOAD = KDMA_W + VPT;                  // vector-memory loads per wave per block
constexpr int PF = 4;                                // operand fragments read ahead in an M phase
constexpr float RESCALE_MARGIN = 8.f;
static_assert(KDMA_W * NW == NFRAG_K && VPT == 2 && VPT * NKG == BLOCK_N, "work split");

// Wait until at most `keep` of this wave's vector-memory loads are in flight.
__device__ __forceinline__ void vm_wait(bool keep_one_block) {
  if (keep_one_block)
    __builtin_amdgcn_s_waitcnt(wait_enc(NLOAD, 15));
  else
    __builtin_amdgcn_s_waitcnt(wait_enc(0, 15));
}

// WALK: the key walk (box_common.h), chosen by the host.
template <int WALK>
__global__ __launch_bounds__(NW * 64) void box_attn_bf16_pp_kernel(const BoxAttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds[NSTAGE * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int G = lane >> 4;
  const bool grp_b = wave >= NW / 2;   // waves w and w + 4 share a SIMD

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
  if (q0 >= qvol) return;  // uniform over the workgroup, before any barrier
  const int kvol = kb.et * kb.eh * kb.ew;
  const int nkb = (kvol + BLOCK_N - 1) / BLOCK_N;

  const char* __restrict__ qp = (const char*)p.q + 2 * (b * p.q_sb + h * p.q_sh);
  const char* kp = (const char*)p.k + 2 * (b * p.k_sb + h * p.k_sh);
  const char* vp = (const char*)p.v + 2 * (b * p.v_sb + h * p.v_sh);
  const uint32_t nkeys = (uint32_t)(p.kT * p.kH * p.kW);
  const uint32_t krange = (nkeys - 1u) * 2u * (uint32_t)p.k_sn + 2u * HD;
  const uint32_t vrange = (nkeys - 1u) * 2u * (uint32_t)p.v_sn + 2u * HD;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, (int)krange, BUF_FLAGS);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, (int)vrange, BUF_FLAGS);
  char* op = (char*)p.o + 2 * (b * p.o_sb + h * p.o_sh);
  const uint32_t q_row = 2u * (uint32_t)p.q_sn, k_row = 2u * (uint32_t)p.k_sn;
  const uint32_t v_row = 2u * (uint32_t)p.v_sn, o_row = 2u * (uint32_t)p.o_sn;

  // ---- this lane's queries: column l16 of each of the wave's three tiles
  uint32_t qtok[QT];
  bool q_valid[QT];
  bf16x8 qf[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int jq = q0 + wave * 16 * QT + 16 * qt + l16;
    q_valid[qt] = jq < qvol;
    const int j = min(jq, qvol - 1);
    const int plane = qb.eh * qb.ew;
    const int jt = j / plane;
    const int r = j - jt * plane;
    const int jh = r / qb.ew;
    const int jw = r - jh * qb.ew;
    qtok[qt] = q_token(p, qb.t0 + jt, qb.h0 + jh, qb.w0 + jw);
    const char* src = qp + qtok[qt] * q_row + 16 * G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qt][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 64 * ks));
  }

  // ---- key box addressing: key j -> token, via two divisions by invariants
  const FastDiv fd_plane = make_fastdiv((uint32_t)(kb.eh * kb.ew));
  const FastDiv fd_row = make_fastdiv((uint32_t)kb.ew);
  auto key_token = [&](int j) -> uint32_t {
    j = min(j, kvol - 1);   // keys past the box repeat the last key; masked later
    return box_key_token24(p, kb, (uint32_t)j, fd_plane, fd_row);
  };
  auto stage_of = [&](int blk) -> char* { return lds + (blk % NSTAGE) * STAGE; };

  // K: lane L of fragment (c, t, ks) fetches key row 32c + 8*((L%16)/4) +
  // 4t + L%4, head_dim chunk 4ks + L/16.  V: thread owns head_dim chunk vc
  // (8 elements) of keys VPT*vk .. VPT*vk + VPT-1.
  const int k_row_in_chunk = 8 * (l16 >> 2) + (l16 & 3);
  const int vk = tid % NKG;
  const int vc = tid / NKG;
  u32x4 vreg[VPT];
  // the block rows this lane loads: K row of each of its KDMA_W fragments,
  // V rows VPT*vk + i
  auto k_row_of = [&](int i) {
    const int f = wave * KDMA_W + i;   // fragment = (c*2 + t)*KS + ks
    return 32 * (f / (2 * KS)) + 4 * ((f / KS) & 1) + k_row_in_chunk;
  };
  auto k_chunk_of = [&](int i) { return (uint32_t)(4 * ((wave * KDMA_W + i) % KS) + G) * 16u; };

  // ---- tile walk (WALK_TILES*): the request cursor, and in WALK_TILES the
  // rows' byte offsets from the block's first token
  const int w_log = __builtin_ctz((unsigned)max(p.bW, 1));   // bW divides 64: a power of two
  TileCursor cur;
  if constexpr (WALK == WALK_TILES || WALK == WALK_TILES_ROLLED) cur.init(p, kb);
  uint32_t k_off[KDMA_W], v_off[VPT];
  if constexpr (WALK == WALK_LINEAR) {
#pragma unroll
    for (int i = 0; i < KDMA_W; ++i) k_off[i] = (uint32_t)k_row_of(i) * k_row + k_chunk_of(i);
#pragma unroll
    for (int i = 0; i < VPT; ++i) v_off[i] = (uint32_t)(VPT * vk + i) * v_row + (uint32_t)vc * 16u;
  }
  if constexpr (WALK == WALK_TILES) {
#pragma unroll
    for (int i = 0; i < KDMA_W; ++i)
      k_off[i] = (uint32_t)tile_row_offset(p, k_row_of(i), w_log) * k_row + k_chunk_of(i);
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      v_off[i] = (uint32_t)tile_row_offset(p, VPT * vk + i, w_log) * v_row + (uint32_t)vc * 16u;
  }

  auto load_block = [&](int blk) {
    char* st = stage_of(blk);
    if constexpr (WALK == WALK_RASTER) {
      const uint32_t my_tok = key_token(blk * BLOCK_N + lane);
#pragma unroll
      for (int i = 0; i < KDMA_W; ++i) {
        const int f = wave * KDMA_W + i;
        const uint32_t tok = (uint32_t)__shfl((int)my_tok, k_row_of(i), 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)(st + f * 1024), 16,
                                                 (int)(tok * k_row + k_chunk_of(i)), 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t tok = (uint32_t)__shfl((int)my_tok, VPT * vk + i, 64);
        vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrsrc, (int)(tok * v_row + vc * 16), 0, 0));
      }
    } else if constexpr (WALK == WALK_LINEAR) {
      // rows past the box (only in the last block) are clamped to its last
      // key at the same 16-byte piece, as the raster walk repeats that key
      const uint32_t base = (uint32_t)blk * BLOCK_N;
      const uint32_t kb_off = base * k_row, vb_off = base * v_row;
      const uint32_t k_last = (uint32_t)(kvol - 1) * k_row, v_last = (uint32_t)(kvol - 1) * v_row;
#pragma unroll
      for (int i = 0; i < KDMA_W; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)(st + (wave * KDMA_W + i) * 1024), 16,
                                                 (int)min(kb_off + k_off[i], k_last + k_chunk_of(i)), 0, 0, 0);
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                vrsrc, (int)min(vb_off + v_off[i], v_last + (uint32_t)vc * 16u), 0, 0));
    } else {
      int t, h, w;
      cur.next(p, kb, t, h, w);
      if constexpr (WALK == WALK_TILES) {
        const uint32_t base = (uint32_t)((t * p.kH + h) * p.kW + w);
        const uint32_t kb_off = base * k_row, vb_off = base * v_row;
#pragma unroll
        for (int i = 0; i < KDMA_W; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)(st + (wave * KDMA_W + i) * 1024), 16,
                                                   (int)(kb_off + k_off[i]), 0, 0, 0);
#pragma unroll
        for (int i = 0; i < VPT; ++i)
          vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrsrc, (int)(vb_off + v_off[i]), 0, 0));
      } else {
        auto tok_of = [&](int r) { return tile_row_token_rolled(p, t, h, w, r, w_log); };
#pragma unroll
        for (int i = 0; i < KDMA_W; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)(st + (wave * KDMA_W + i) * 1024), 16,
                                                   (int)(tok_of(k_row_of(i)) * k_row + k_chunk_of(i)), 0, 0, 0);
#pragma unroll
        for (int i = 0; i < VPT; ++i)
          vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  vrsrc, (int)(tok_of(VPT * vk + i) * v_row + vc * 16), 0, 0));
      }
    }
  };
  // Transposing store of the V registers: element e of the thread's two keys
  // (head_dim 8vc + e) goes to a fixed offset in the stage's V^T area.
  uint32_t vw_off[8];
  {
    const int k0 = VPT * vk;
    const int c = k0 >> 5, kg = (k0 & 31) >> 3;
    const int sig = (kg << 1) | c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * vc + e;
      vw_off[e] = (uint32_t)(c * ND * 1024 + kg * 256 + (k0 & 7) * 2 + (d >> 4) * 1024 + (((d & 15) ^ sig) * 16));
    }
  }
  auto store_v = [&](int blk) {
    const uint32_t vbase = (uint32_t)(uintptr_t)(stage_of(blk) + K_STAGE);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low bf16 halves
      *(lds_u32*)(uintptr_t)(vbase + vw_off[e]) = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
    }
  };

  // V^T operand read offset per chunk c: piece 16G + (l16 ^ ((G << 1) | c))
  int v_rd[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) v_rd[c] = K_STAGE + c * ND * 1024 + (16 * G + (l16 ^ ((G << 1) | c))) * 16;

  f32x4 oacc[ND][QT];
  f32x4 lacc[QT];    // row sums of P, the same value in all four registers
  float m_run[QT];   // per-query reference maximum (log2 units)
  float m_thr[QT];   // (m_run + RESCALE_MARGIN) / (scale*log2(e)): the test runs on raw scores
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) oacc[dt][qt] = f32x4{};
    lacc[qt] = f32x4{};
    m_run[qt] = -INFINITY;
    m_thr[qt] = -INFINITY;
  }
  bf16x8 ones8;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones8[e] = (__bf16)1.f;
  const float cl2 = p.scale_log2e;
  const float inv_cl2 = 1.f / cl2;   // +inf for scale 0: no growth test fires after the first chunk

  // ---- M phase: the 8 V^T fragments of chunk cv of st_v (P*V, fragments
  // 0..7, the first PF read by prefetch_pv in the preceding V phase), then the
  // 8 K fragments of chunk ck of st_k (S, fragments 8..15 in (ks, t) order so
  // that dependent products are six MFMAs apart).  Reads run PF ahead.
  bf16x8 fb[16];
  auto frag_ptr = [&](const char* st_v, int cv, const char* st_k, int ck, int i) -> const char* {
    if (i < 8) return st_v + v_rd[cv] + i * 1024;
    const int j = i - 8, ks = j >> 1, t = j & 1;
    return st_k + ((ck * 2 + t) * KS + ks) * 1024 + lane * 16;
  };
  auto prefetch_pv = [&](const char* st_v, int cv) {
#pragma unroll
    for (int i = 0; i < PF; ++i) fb[i] = lds_frag(st_v + v_rd[cv] + i * 1024);
  };
  f32x4 s[2][QT];
  bf16x8 pf[QT];
  auto mphase = [&](bool with_pv, const char* st_v, int cv, bool with_s, const char* st_k, int ck) {
    const int i0 = with_pv ? 0 : 8;
    const int i1 = with_s ? 16 : 8;
    if (!with_pv) {
#pragma unroll
      for (int i = 8; i < 8 + PF; ++i) fb[i] = lds_frag(frag_ptr(st_v, cv, st_k, ck, i));
    }
    if (with_s) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[t][qt] = f32x4{};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < i0 || i >= i1) continue;
      if (i + PF < i1) fb[i + PF] = lds_frag(frag_ptr(st_v, cv, st_k, ck, i + PF));
      __builtin_amdgcn_sched_barrier(0);
      if (i < 8) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[i][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[i], pf[qt], oacc[i][qt], 0, 0, 0);
        if (i == 3) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pf[qt], lacc[qt], 0, 0, 0);
        }
      } else {
        const int j = i - 8, ks = j >> 1, t = j & 1;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          s[t][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[i], qf[qt][ks], s[t][qt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (with_pv) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) pin(oacc[dt][0], oacc[dt][1], oacc[dt][2]);
      pin(lacc[0], lacc[1], lacc[2]);
    }
    if (with_s) {
#pragma unroll
      for (int t = 0; t < 2; ++t) pin(s[t][0], s[t][1], s[t][2]);
    }
  };

  // ---- V phase: online softmax of one chunk; nvalid = keys of the block
  // from this chunk on (masking only in the last, partial block).
  auto softmax = [&](int nvalid, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    float lmax[QT];
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      // a running chain, so that the compiler fuses it into three v_max3 and one v_max
      float m = fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), s[0][qt][2]);
      m = fmaxf(fmaxf(m, s[0][qt][3]), s[1][qt][0]);
      m = fmaxf(fmaxf(m, s[1][qt][1]), s[1][qt][2]);
      m = fmaxf(m, s[1][qt][3]);
      lmax[qt] = m;
      grow = grow || (m > m_thr[qt]);
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float m_new = fmaxf(m_run[qt], xrow4_max(lmax[qt]) * cl2);
        const float corr = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
        lacc[qt] *= corr;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) oacc[dt][qt] *= corr;
        m_run[qt] = m_new;
        m_thr[qt] = (m_new + RESCALE_MARGIN) * inv_cl2;
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pv = __builtin_amdgcn_exp2f(fmaf(s[e >> 2][qt][e & 3], cl2, -m_run[qt]));
        if constexpr (PARTIAL) {
          if (8 * G + e >= nvalid) pv = 0.f;
        }
        pf[qt][e] = (__bf16)pv;
      }
      pin(pf[qt]);
    }
    pin(m_run[0], m_run[1], m_run[2]);
  };

  // ---- prologue: block 0 complete in LDS, block 1 in flight
  load_block(0);
  store_v(0);
  if (nkb > 1) load_block(1);
  vm_wait(nkb > 1);
  phase_barrier();
  if (grp_b) phase_barrier();

  auto do_block = [&](int blk, auto partial_tag) {
    const char* st = stage_of(blk);
    const int nvalid = kvol - blk * BLOCK_N;
    const bool more2 = blk + 2 < nkb;
    // M(blk, 0)
    if (blk > 0)
      mphase(true, stage_of(blk - 1), 1, true, st, 0);
    else
      mphase(false, st, 0, true, st, 0);
    phase_barrier();
    // V(blk, 0)
    prefetch_pv(st, 0);
    softmax(nvalid, partial_tag);
    if (blk + 1 < nkb) store_v(blk + 1);
    phase_barrier();
    // M(blk, 1)
    mphase(true, st, 0, true, st, 1);
    if (grp_b) vm_wait(false);   // K of block blk+1 has landed
    phase_barrier();
    // V(blk, 1)
    if (more2) load_block(blk + 2);
    prefetch_pv(st, 1);
    softmax(nvalid - 32, partial_tag);
    if (!grp_b) vm_wait(more2);
    phase_barrier();
  };
  const bool last_partial = kvol % BLOCK_N != 0;
  const int nfull = last_partial ? nkb - 1 : nkb;
  for (int blk = 0; blk < nfull; ++blk) do_block(blk, std::false_type{});
  if (last_partial) do_block(nkb - 1, std::true_type{});
  mphase(true, stage_of(nkb - 1), 1, false, stage_of(nkb - 1), 0);
  if (!grp_b) phase_barrier();

  // ---- epilogue of the dense-key instance (the global branch, which carries
  // the fused merges) with a merge: each row combines with the other branch's
  // row at the positions it is written to (so out may be that tensor itself).
  // The wave's scaled rows go through LDS in fp32, one query tile at a time
  // (row-major, 16-byte pieces XOR-swizzled by row), so that the other
  // branch's rows are read and the merged rows written whole, 16 bytes per
  // lane and 16 lanes per row, with the same single rounding as below.  The
  // areas lie in the two stages the other group's last products do not read,
  // four waves to a stage; LDS requests of a wave complete in order, so a
  // wave reuses its area for its three tiles without waiting.  (In the other
  // instances the longer epilogue makes the main loop spill.)
  if constexpr (WALK == WALK_LINEAR) {
    if (p.merge != MERGE_NONE) {
      char* stg = stage_of(nkb + (wave & 1)) + (wave >> 1) * (16 * 512);
      const char* olp = (const char*)p.ol + 2 * (b * p.ol_sb + h * p.ol_sh);
      const uint32_t ol_row = 2u * (uint32_t)p.ol_sn;
      const int j = lane & 15;   // this lane's 16-byte piece of a bf16 row: head_dim 8j .. 8j+7
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float l_tot = lacc[qt][0];
        const float inv = 1.f / l_tot;
        float wa = 0.f, sc = 0.f;
        if (q_valid[qt]) {
          const float lse_row = (m_run[qt] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
          const RowMerge rm = row_merge(p, b, h, qtok[qt], lse_row);
          wa = rm.wa;
          sc = rm.wb * inv;
          if (p.lse != nullptr && G == 0) {
            const int64_t N = (int64_t)p.qT * p.qH * p.qW;
            p.lse[((int64_t)b * p.heads + h) * N + qtok[qt]] = rm.lse;
          }
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          f32x4 f;
#pragma unroll
          for (int v = 0; v < 4; ++v) f[v] = oacc[dt][qt][v] * sc;
          *(f32x4*)(stg + l16 * 512 + ((4 * dt + G) ^ l16) * 16) = f;
        }
        const uint32_t tok_own = q_valid[qt] ? qtok[qt] : ~0u;
        asm volatile("" ::: "memory");
#pragma unroll 1
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * i + (lane >> 4);   // row of the tile: its owner is lane r
          const uint32_t tok = (uint32_t)__shfl((int)tok_own, r, 64);
          const float war = __shfl(wa, r, 64);
          const f32x4 f0 = *(const f32x4*)(stg + r * 512 + ((2 * j) ^ r) * 16);
          const f32x4 f1 = *(const f32x4*)(stg + r * 512 + ((2 * j + 1) ^ r) * 16);
          if (tok != ~0u) {
            const u32x4 raw = *(const u32x4*)(olp + tok * ol_row + 16 * j);
            float a0[4], a1[4];
            bf16x4_to_f32(raw[0], raw[1], a0);
            bf16x4_to_f32(raw[2], raw[3], a1);
            bf16x8 ov;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              ov[v] = (__bf16)fmaf(war, a0[v], f0[v]);
              ov[4 + v] = (__bf16)fmaf(war, a1[v], f1[v]);
            }
            *(bf16x8*)(op + tok * o_row + 16 * j) = ov;
          }
        }
        asm volatile("" ::: "memory");
      }
      return;
    }
  }

  // ---- epilogue: O^T register v of tile (dt, qt) is head_dim 16dt + 4G + v;
  // with a merge, each row combines with the other branch's row (read at the
  // positions this lane writes, so out may be that tensor itself).
  const char* olp = p.merge != MERGE_NONE ? (const char*)p.ol + 2 * (b * p.ol_sb + h * p.ol_sh) : nullptr;
  const uint32_t ol_row = 2u * (uint32_t)p.ol_sn;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l_tot = lacc[qt][0];
    const float inv = 1.f / l_tot;
    if (q_valid[qt]) {
      float lse_row = (m_run[qt] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
      float wa = 0.f, sc = inv;
      if (p.merge != MERGE_NONE) {
        const RowMerge rm = row_merge(p, b, h, qtok[qt], lse_row);
        wa = rm.wa;
        sc = rm.wb * inv;
        lse_row = rm.lse;
      }
      char* dst = op + qtok[qt] * o_row + 8 * G;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        float f[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) f[v] = oacc[dt][qt][v] * sc;
        if (p.merge != MERGE_NONE) {
          const u32x2 raw = *(const u32x2*)(olp + qtok[qt] * ol_row + 8 * G + 32 * dt);
          float a[4];
          bf16x4_to_f32(raw[0], raw[1], a);
#pragma unroll
          for (int v = 0; v < 4; ++v) f[v] = fmaf(wa, a[v], f[v]);
        }
        bf16x4 ov;
#pragma unroll
        for (int v = 0; v < 4; ++v) ov[v] = (__bf16)f[v];
        *(u32x2*)(dst + 32 * dt) = __builtin_bit_cast(u32x2, ov);
      }
      if (p.lse != nullptr && G == 0) {
        const int64_t N = (int64_t)p.qT * p.qH * p.qW;
        p.lse[((int64_t)b * p.heads + h) * N + qtok[qt]] = lse_row;
      }
    }
  }
}

}  // namespace

hipError_t launch_box_attn_bf16_pp(const BoxAttnParams& p, hipStream_t stream) {
  if (p.tile_walk == WALK_TILES)
    hipLaunchKernelGGL(box_attn_bf16_pp_kernel<WALK_TILES>, dim3(p.total_wg), dim3(NW * 64), 0, stream, p);
  else if (p.tile_walk == WALK_LINEAR)
    hipLaunchKernelGGL(box_attn_bf16_pp_kernel<WALK_LINEAR>, dim3(p.total_wg), dim3(NW * 64), 0, stream, p);
  else if (p.tile_walk == WALK_TILES_ROLLED)
    hipLaunchKernelGGL(box_attn_bf16_pp_kernel<WALK_TILES_ROLLED>, dim3(p.total_wg), dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(box_attn_bf16_pp_kernel<WALK_RASTER>, dim3(p.total_wg), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

int box_attn_bf16_pp_block_m() { return BLOCK_M; }

}  // namespace vdsa
