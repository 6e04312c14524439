// Tile-window ("box") attention forward for head_dim 128, bf16 in/out, fp32
// accumulation, on 16x16x32 matrix-core products (v_mfma_f32_16x16x32_bf16),
// with 48 queries per wave.
//
// Same method as attn_bf16.hip: the keys of a query tile (the union of the
// key tiles in its window, Sliding Tile Attention, arXiv 2502.04507,
// abstract) form one box of tokens, walked in 64-key blocks with every key's
// address computed from its box coordinates.  What differs is the work split:
// each wave owns three 16-query MFMA columns (48 queries) that share every K
// and V operand it reads, and a workgroup of NW = 4 waves owns 192 queries
// (one 3x8x8 tile; 384-query tiles run on the 8-wave kernel of
// attn_bf16_pp.hip).  Every 64-key block loaded into LDS thus feeds 1.5x the
// queries of a 128-query workgroup, and every LDS operand read feeds 1.5x the
// products.
//
// Per 32-key chunk c of a block, per wave:
//   S^T = K Q^T   for two 16-key MFMA row tiles t x three 16-query tiles;
//                 K rows are permuted so that row r of tile t is key
//                 8*(r/4) + 4t + r%4 of the chunk: lane group G = lane/16 then
//                 holds keys 8G .. 8G+7 of its query after the two tiles.
//   softmax       fp32, v_exp_f32 with scale*log2(e) folded into one FMA,
//                 against a lazy per-query reference raised only when some
//                 score of the wave exceeds it by more than RESCALE_MARGIN;
//                 each lane tests its own eight raw scores against that
//                 threshold in raw-score units, and the cross-lane maximum
//                 (two exchanges) is formed only when one fires.
//   O^T += V^T P^T with P^T straight from the S^T accumulators (those eight
//                 consecutive keys are one MFMA k-slice) and V^T from LDS;
//                 an all-ones A operand times the same P^T gives the row sums
//                 of P (the softmax denominators) on the matrix core.
// Operand fragments are read RA ahead of the MFMAs that use them.
//
// LDS (double-buffered, one barrier per block), all in 1 KB MFMA operand
// fragments, each read as one contiguous 1 KB per wave:
//   K fragment (c, t, ks): lane L holds head_dim [32ks + 8(L/16), +8) of key
//     row 8*((L%16)/4) + 4t + L%4 of chunk c; filled by direct global->LDS
//     loads (buffer_load_dwordx4 ... lds).
//   V fragment (c, dt): lane L = 16G + p holds keys 8G .. 8G+7 of chunk c at
//     head_dim 16dt + p, stored at piece 16G + (p ^ ((G << 1) | c)); filled by
//     transposing register copies of V, the XOR making those stores free of
//     bank conflicts.
#include <type_traits>

#include "box_common.h"

namespace vdsa {
namespace {

constexpr int HD = 128;
constexpr int BLOCK_N = 64;   // keys per block
constexpr int QT = 3;         // 16-query tiles per wave
constexpr int KS = HD / 32;   // 32-wide head_dim steps of the S^T product
constexpr int ND = HD / 16;   // 16-row head_dim tiles of O^T
constexpr int NFRAG_K = 2 * 2 * KS;   // (chunk, t, ks)
constexpr int NFRAG_V = 2 * ND;       // (chunk, dt)
constexpr int K_STAGE = NFRAG_K * 1024;
constexpr int V_STAGE = NFRAG_V * 1024;
constexpr int STAGE = K_STAGE + V_STAGE;
constexpr int WAIT_VMCNT0 = 0x0F70;   // s_waitcnt vmcnt(0), other counters untouched
constexpr float RESCALE_MARGIN = 8.f;
constexpr int RA = 3;   // operand fragments read ahead of their MFMAs

// WALK: the key walk (box_common.h), chosen by the host.  PAIR (NW = 8, the
// tile walk): the workgroup owns two tiles adjacent along w, waves 0-3 the
// first and 4-7 the second.  Both walk the union of their key boxes (their t
// and h ranges are the same), so each block is loaded once for both tiles,
// and a wave skips the products and softmax of blocks outside its own box;
// its own blocks come in the order of its own box's walk.
template <int NW, int WALK, bool PAIR = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void box_attn_bf16_m16_kernel(const BoxAttnParams p) {
  constexpr int BLOCK_M = NW * 16 * QT;
  constexpr int KDMA_W = NFRAG_K / NW;           // K fragments loaded per wave per block
  constexpr int VPT = BLOCK_N * HD / 8 / (NW * 64);   // V 16-byte chunks per thread (2 or 4)
  constexpr int NKG = BLOCK_N / VPT;             // threads per V head_dim chunk
  static_assert(KDMA_W * NW == NFRAG_K && VPT * NKG == BLOCK_N && (VPT == 2 || VPT == 4), "split");

  __shared__ __attribute__((aligned(16))) char lds[(PAIR ? 3 : 2) * STAGE];   // PAIR: a three-stage ring
  constexpr int RAW = RA;   // operand read-ahead (4 would spill registers in the pair form's loop)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int G = lane >> 4;   // lane group

  // ---- which (batch, head, query tile, query block) this workgroup owns
  const int wg = xcd_remap(blockIdx.x, p.total_wg);
  int qblk, tile, bh;
  Box qb, kb, kw;   // kw: the box the walk covers (kb, or the pair's union)
  bool own = true;  // PAIR: this wave's tile exists (uniform over the wave)
  int wq = wave;    // the wave's index among the waves sharing its tile
  if constexpr (PAIR) {
    const int npw = (p.nW + 1) >> 1;   // tile pairs per row of the lattice
    const int pairs = p.nT * p.nH * npw;
    const int pr = wg % pairs;
    bh = wg / pairs;
    const int pw = pr % npw, row = pr / npw;   // row = at * nH + ah
    const int grp = wave >> 2;
    own = 2 * pw + grp < p.nW;
    wq = wave & 3;
    qblk = 0;
    tile = row * p.nW + min(2 * pw + grp, p.nW - 1);
    tile_boxes(p, tile, qb, kb);
    Box qa, ka, qc, kc;
    tile_boxes(p, row * p.nW + 2 * pw, qa, ka);
    tile_boxes(p, row * p.nW + min(2 * pw + 1, p.nW - 1), qc, kc);
    kw = ka;
    kw.w0 = min(ka.w0, kc.w0);
    kw.ew = max(ka.w0 + ka.ew, kc.w0 + kc.ew) - kw.w0;
  } else {
    qblk = wg % p.qblocks;
    const int rest = wg / p.qblocks;
    const int ntiles = p.nT * p.nH * p.nW;
    tile = rest % ntiles;
    bh = rest / ntiles;
    tile_boxes(p, tile, qb, kb);
    kw = kb;
  }
  const int h = bh % p.heads;
  const int b = bh / p.heads;

  const int qvol = qb.et * qb.eh * qb.ew;
  const int q0 = qblk * BLOCK_M;
  if (q0 >= qvol) return;  // uniform over the workgroup
  const int kvol = kw.et * kw.eh * kw.ew;
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
    const int jq = q0 + wq * 16 * QT + 16 * qt + l16;
    q_valid[qt] = own && jq < qvol;
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

  // K DMA: lane L of fragment (c, t, ks) fetches key row 32c + 8*((L%16)/4) +
  // 4t + L%4, head_dim chunk 4ks + L/16.
  const int k_row_in_chunk = 8 * (l16 >> 2) + (l16 & 3);
  // V load mapping: thread owns head_dim chunk vc (8 elements) of keys
  // VPT*vk .. VPT*vk + VPT-1.
  const int vk = tid % NKG;
  const int vc = tid / NKG;
  u32x4 vregs[2][VPT];   // PAIR: one set per block parity (blocks requested two ahead)

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
  if constexpr (WALK != WALK_RASTER) cur.init(p, kw);
  uint32_t k_off[KDMA_W], v_off[VPT];
  if constexpr (WALK == WALK_TILES) {
#pragma unroll
    for (int i = 0; i < KDMA_W; ++i)
      k_off[i] = (uint32_t)tile_row_offset(p, k_row_of(i), w_log) * k_row + k_chunk_of(i);
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      v_off[i] = (uint32_t)tile_row_offset(p, VPT * vk + i, w_log) * v_row + (uint32_t)vc * 16u;
  }

  // Requests of consecutive blocks come in order (the tile cursor advances
  // once per call).
  auto load_block = [&](int blk, int stage, auto set_tag) {
    u32x4 (&vreg)[VPT] = vregs[decltype(set_tag)::value];
    char* st = lds + stage * STAGE;
    if constexpr (WALK == WALK_RASTER) {
      const uint32_t my_tok = key_token(blk * BLOCK_N + lane);
#pragma unroll
      for (int i = 0; i < KDMA_W; ++i) {
        const uint32_t tok = (uint32_t)__shfl((int)my_tok, k_row_of(i), 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)(st + (wave * KDMA_W + i) * 1024), 16,
                                                 (int)(tok * k_row + k_chunk_of(i)), 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t tok = (uint32_t)__shfl((int)my_tok, VPT * vk + i, 64);
        vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrsrc, (int)(tok * v_row + vc * 16), 0, 0));
      }
    } else {
      int t, h, w;
      cur.next(p, kw, t, h, w);
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
  // Transposing store of the V registers into the V fragments of `stage`.
  auto store_v = [&](int stage, auto set_tag) {
    const u32x4 (&vreg)[VPT] = vregs[decltype(set_tag)::value];
    char* vst = lds + stage * STAGE + K_STAGE;
    const int k0 = VPT * vk;
    const int c = k0 >> 5, kg = (k0 & 31) >> 3;
    const int sig = (kg << 1) | c;
    char* base = vst + c * ND * 1024 + kg * 256 + (k0 & 7) * 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * vc + e;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low bf16 halves
      char* dst = base + (d >> 4) * 1024 + (((d & 15) ^ sig) * 16);
      if constexpr (VPT == 4) {
        u32x2 pk;
        pk[0] = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
        pk[1] = __builtin_amdgcn_perm(vreg[3][e >> 1], vreg[2][e >> 1], sel);
        *(u32x2*)dst = pk;
      } else {
        *(uint32_t*)dst = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
      }
    }
  };

  // V operand read offset per chunk c: piece 16G + (l16 ^ ((G << 1) | c))
  int v_rd[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) v_rd[c] = K_STAGE + c * ND * 1024 + (16 * G + (l16 ^ ((G << 1) | c))) * 16;

  f32x4 oacc[ND][QT];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = f32x4{};
  float m_run[QT];
  float m_thr[QT];   // (m_run + RESCALE_MARGIN) / (scale*log2(e)), in raw-score units
  f32x4 lacc[QT];   // row sums of P (all-ones A operand times P^T)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    m_thr[qt] = -INFINITY;
    lacc[qt] = f32x4{};
  }
  bf16x8 ones8;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones8[e] = (__bf16)1.f;
  const float cl2 = p.scale_log2e;
  const float inv_cl2 = 1.f / cl2;

  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  if constexpr (!PAIR) {
    load_block(0, 0, Set0{});
    store_v(0, Set0{});
    __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);
    __syncthreads();
  }

  // PAIR: the processed block's key tile along w (blocks are the frames of
  // the union box's tiles, w fastest after the frame) and this wave's range
  int wf = 0, wtw = 0;
  const int ntw = kw.ew / max(p.bW, 1);
  const int my_tw0 = (kb.w0 - kw.w0) / max(p.bW, 1), my_tw1 = my_tw0 + kb.ew / max(p.bW, 1);

  // One 32-key chunk c of the block in stage st for this wave: S^T, the
  // online softmax (nvalid = keys of the block; masking only in a partial
  // last block) and O^T += V^T P^T.
  auto chunk = [&](const char* st, int c, int nvalid, auto partial_tag) __attribute__((always_inline)) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    // S^T for the chunk: s[t][qt] register v = key 32c + 8G + 4t + v, query 16qt + l16
    f32x4 s[2][QT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[t][qt] = f32x4{};
    {
      // K fragments in (ks, t) order, read RAW ahead of their products
      auto kfp = [&](int i) { return st + ((c * 2 + (i & 1)) * KS + (i >> 1)) * 1024 + lane * 16; };
      bf16x8 kb[8];
#pragma unroll
      for (int i = 0; i < RAW; ++i) kb[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)kfp(i));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i + RAW < 8) kb[i + RAW] = __builtin_bit_cast(bf16x8, *(const u32x4*)kfp(i + RAW));
        __builtin_amdgcn_sched_barrier(0);
        const int ks = i >> 1, t = i & 1;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          s[t][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[i], qf[qt][ks], s[t][qt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // online softmax over the chunk's 32 keys.  Lazy rescale: keep each
    // query's reference max until some score of the wave exceeds it by more
    // than RESCALE_MARGIN (log2 units); each lane tests its own eight scores
    // of a query, and the cross-lane maximum is formed only when one fires.
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
    bf16x8 pf[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pv = __builtin_amdgcn_exp2f(fmaf(s[e >> 2][qt][e & 3], cl2, -m_run[qt]));
        if constexpr (PARTIAL) {
          if (32 * c + 8 * G + e >= nvalid) pv = 0.f;
        }
        pf[qt][e] = (__bf16)pv;
      }
    }
    // O^T += V^T P^T for the chunk, V^T fragments read RAW ahead
    {
      bf16x8 vb[ND];
#pragma unroll
      for (int i = 0; i < RAW; ++i) vb[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + v_rd[c] + i * 1024));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        if (dt + RAW < ND) vb[dt + RAW] = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + v_rd[c] + (dt + RAW) * 1024));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[dt], pf[qt], oacc[dt][qt], 0, 0, 0);
        if (dt == 3) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pf[qt], lacc[qt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto process = [&](int blk, auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    const int stage = blk & 1;
    const bool more = blk + 1 < nkb;
    if (more) load_block(blk + 1, stage ^ 1, Set0{});
    bool active = true;
    if constexpr (PAIR) {
      active = own && wtw >= my_tw0 && wtw < my_tw1;
      if (++wf == p.bT) {
        wf = 0;
        if (++wtw == ntw) wtw = 0;
      }
    }
    if (active) {
    const char* st = lds + stage * STAGE;
    const int nvalid = PARTIAL ? kvol - blk * BLOCK_N : BLOCK_N;

#pragma unroll
    for (int c = 0; c < 2; ++c) chunk(st, c, nvalid, partial_tag);


    }
    if (more) store_v(stage ^ 1, Set0{});
    __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);   // K of the next block has landed in LDS
    __syncthreads();
  };

  if constexpr (PAIR) {
    // Three stages, blocks requested two ahead: in block b the requests of
    // block b+2 (stage (b+2) % 3, V register set b % 2) go out first, and the
    // wait at its end keeps them in flight while block b+1's have landed.
    // Every step requests and stores unconditionally (past the box, the last
    // block again, into stages no later step reads), so that every path
    // issues the same memory requests and the counted waits stay exact; the
    // box has whole 64-key blocks only (the tile walk).
    constexpr int NST = 3;
    constexpr int NLOAD = KDMA_W + VPT;   // vector-memory requests per wave per block
    auto req = [&](int blk, auto set_tag) __attribute__((always_inline)) {
      load_block(min(blk, nkb - 1), blk % NST, set_tag);
    };
    req(0, Set0{});
    req(1, Set1{});
    __builtin_amdgcn_s_waitcnt(wait_enc(NLOAD, 15));   // block 0's requests have landed
    store_v(0, Set0{});
    __syncthreads();
    auto step = [&](int blk, auto par_tag) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_tag)::value;
      using Own = std::integral_constant<int, PAR>;
      using Next = std::integral_constant<int, PAR ^ 1>;
      req(blk + 2, Own{});
      __builtin_amdgcn_sched_barrier(0);
      bool active = blk < nkb;
      if (active) {
        active = own && wtw >= my_tw0 && wtw < my_tw1;
        if (++wf == p.bT) {
          wf = 0;
          if (++wtw == ntw) wtw = 0;
        }
      }
      if (active) {
        const char* st = lds + (blk % NST) * STAGE;
#pragma unroll
        for (int c = 0; c < 2; ++c) chunk(st, c, BLOCK_N, std::false_type{});
      }
      store_v((blk + 1) % NST, Next{});
      __builtin_amdgcn_s_waitcnt(wait_enc(NLOAD, 15));   // block blk+1 has landed, blk+2 in flight
      // a barrier without the memory fence of __syncthreads(), which would
      // also wait for block blk+2's K transfers into LDS
      phase_barrier();
    };
    for (int blk = 0; blk < nkb; blk += 2) {
      step(blk, Set0{});
      step(blk + 1, Set1{});
    }
    __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);   // the requests past the box have landed
  } else {
    const bool last_partial = kvol % BLOCK_N != 0;
    const int nfull = last_partial ? nkb - 1 : nkb;
    for (int blk = 0; blk < nfull; ++blk) process(blk, std::false_type{});
    if (last_partial) process(nkb - 1, std::true_type{});
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

// The rolled tile walk is not instantiated here: unrolling the eight rows a
// thread loads spills registers, so the host keeps the cyclic mode on the
// raster walk for this kernel.
hipError_t launch_box_attn_bf16_m16(const BoxAttnParams& p, hipStream_t stream) {
  if (p.tile_walk == WALK_TILES && p.qblocks == 1 && p.nW >= 2) {
    BoxAttnParams pp = p;   // one workgroup per pair of tiles along w
    pp.total_wg = p.batch * p.heads * p.nT * p.nH * ((p.nW + 1) / 2);
    hipLaunchKernelGGL((box_attn_bf16_m16_kernel<8, WALK_TILES, true>), dim3(pp.total_wg), dim3(8 * 64), 0, stream, pp);
  } else if (p.tile_walk == WALK_TILES)
    hipLaunchKernelGGL((box_attn_bf16_m16_kernel<4, WALK_TILES>), dim3(p.total_wg), dim3(4 * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((box_attn_bf16_m16_kernel<4, WALK_RASTER>), dim3(p.total_wg), dim3(4 * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vdsa
