// Tree-masked GQA attention for the verify forward.
//
// Node i, query head h reads KV head g = h / (Hq / Hkv): every prefix token,
// then the tree nodes on i's root path (i included), scale 1/sqrt(d).  One
// forward over the whole tree is what makes the drafted tree cheap to verify
// ("Lucebox Hub", section "Speculative decoding 계층 (DFlash / DDTree /
// DSpark)"); with a long context the KV prefix is most of the bytes, so it is
// read exactly once per layer and every query row of a KV head shares it.
//
// Two kernels:
//   partial : grid (prefix chunk, KV head).  The n * Hq/Hkv query rows of the
//             KV head live in the block (16-row MFMA tiles, one or two per
//             wave; past 16 tiles, in row groups of at most 16, one block
//             each); K and V tiles of 64 tokens are staged through LDS.
//             S^T = K Q^T puts the softmax axis (keys) inside each lane, so
//             the running max needs only two cross-lane steps; P then feeds
//             O^T = V^T P^T directly from registers (the key order inside a
//             16-key S tile is permuted so each lane already holds the 8
//             consecutive keys the second MFMA wants).  Output per (chunk,
//             row): max and sum in log2 units and the chunk-normalised O.
//   combine: one block per (node, query head): merges the chunk partials and
//             the (at most 64) ancestor keys with a log-sum-exp merge.
#include <stdio.h>

#include <type_traits>

#include "attn_common.h"

namespace lucev {

constexpr int kMaxChunkPages = 1024;  // 16-token pages of one block's prefix chunk (paged cache)

// Waves of the partial kernel: ROWW row waves (one to three per SIMD), each
// holding up to QPW whole 16-row query tiles in registers and reading each K
// and V^T fragment of a tile from LDS once for all of them; with SPLIT the
// last four waves (one per SIMD) also hold one key quarter each of the last
// query tile.
constexpr int attn_waves(int roww, bool split) { return (void)split, roww; }

// One block per (prefix chunk, KV head).  K and V^T tiles of 64 tokens go
// straight from HBM into a ring of NBUF LDS buffers with 16-byte
// direct-to-LDS loads, NBUF - 1 tiles ahead: after the barrier that
// publishes tile t, every wave issues its share of tile t + NBUF - 1 into
// the buffer tile t - 1 used, then computes tile t.  Before that barrier each
// wave waits until only its loads of the tiles after t are in flight
// (vmcnt); no other vector-memory load is issued inside the loop.  A load
// instruction fills 1 KB of LDS, 16 bytes per lane in lane order, so the bank
// swizzles are applied on the global side: LDS chunk c of K row `key` holds
// the row's 16-byte chunk c ^ ((key & 3) | ((key >> 3) & 3) << 2), and chunk
// c of V^T row `dim` holds chunk c ^ ((dim >> 1) & 7).  The ragged last tile
// of the prefix goes through registers so tokens past it are zero.
//
// A row wave takes one 32-key half of a tile at a time: all of the half's K
// fragments and V^T fragments are read from LDS up front, the scores of all
// its query tiles go to the MFMA pipe, and the softmax of one query tile (VALU)
// then runs while the MFMAs of the next are still in flight.  Cross-lane
// reductions use the gfx950 permlane swaps (no LDS traffic).
//
// SPLIT (RT = 4k + 1 query tiles): the four SIMDs would carry k + 1, k, k, k
// tiles, so the last (ragged) tile is instead shared by the last four waves
// (one per SIMD), wave ROWW - 4 + q taking the fixed 16-key quarter q of every
// 64-key tile with its own (max, sum, O) beside any whole tiles it owns; the
// four states are merged through LDS at the end.  The quarter's PV product is a 16x16x16
// MFMA, whose B operand (4 keys per lane) is exactly the layout the 16-key
// score tile comes out in.
//
// PAGED: the prefix lives in 16-token pages, K as [page][Hkv][16][d] and V as
// [page][Hkv][d][16], and table[t / 16] names the page holding token t.  Only
// the global addresses of the tile loads change (a 1 KB K load covers 4 keys
// of one page; a 16-byte V chunk covers 8 tokens of one page), so the LDS
// tiles, and hence the results, are those of the contiguous cache.  The
// block's slice of the table is copied into LDS first, clamped to the pool.

// ROW GROUPS (more than 16 query tiles): the tiles are cut into groups of at
// most 16, one block per (chunk, group) holding two tiles per wave on 8 waves;
// the groups of a chunk sit on one XCD (block ids 8 apart), so the later
// groups' tile reads hit that XCD's L2.
//
// SPLITM: 0 no split tile; 1 the quarters go to the last four of the waves
// that own whole tiles; 2 to four extra waves that own no whole tile.
template <int D, int QPW, int ROWW, int NBUF, bool QLO, int SPLITM, bool PAGED>
__global__ __launch_bounds__(ROWW * 64) void attn_partial_kernel(AttnParams p) {
  constexpr bool SPLIT = SPLITM != 0;
  constexpr int WAVES = ROWW;
  constexpr int KCPR = D / 8;                    // 16-byte chunks per K row
  constexpr int KROWS = 64 / KCPR;               // K rows per 1 KB load
  constexpr int KBYTES = KT * D * 2;             // one K tile
  constexpr int VBYTES = D * KT * 2;             // one V^T tile (rows of 128 bytes)
  constexpr int NLD = (KBYTES + VBYTES) / 1024;  // 1 KB loads per tile
  constexpr int LPW = (NLD + WAVES - 1) / WAVES; // loads per wave per tile (some waves one fewer)
  constexpr int BUF = KBYTES + VBYTES;
  constexpr int MERGE = SPLIT ? 4 * 16 * D * 4 + 2 * 64 * 4 : 0;  // quarter states, after the loop
  constexpr int LDS_BYTES = NBUF * BUF > MERGE ? NBUF * BUF : MERGE;
  static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
  static_assert(!SPLIT || ROWW >= 4, "the split tile's four key quarters go to the last four waves");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  __shared__ __attribute__((aligned(16))) int s_tab[PAGED ? kMaxChunkPages : 1];

  const int tid = threadIdx.x;
  // the wave index as a scalar: every branch on it is then a scalar branch
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  // block x -> (chunk, row group): chunks c and c + 8 are 8 * groups ids apart,
  // the groups of chunk c ids 8 apart (one XCD); padding blocks past the
  // last chunk leave at once
  const int x = blockIdx.x;
  const int grp = (x >> 3) % p.row_groups;
  const int chunk = (x / (8 * p.row_groups)) * 8 + (x & 7);
  if (chunk >= p.n_chunks) return;
  const int g = blockIdx.y;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int RT = (p.rows + 15) / 16;
  const int FT = SPLIT ? RT - 1 : RT;  // tiles the row waves own whole
  // this block's whole tiles: T0 .. TE - 1 (one group; a split plan has one)
  const int T0 = grp * p.group_tiles;
  const int TE = min(FT, T0 + p.group_tiles);
  const bool has_q = SPLIT && wave >= ROWW - 4;  // holds a key quarter of tile FT
  const int qq = wave - (ROWW - 4);              // which quarter
  const bool full_lpw = wave + (LPW - 1) * WAVES < NLD;  // issues LPW loads per tile (else LPW - 1)
  // query tiles held; the quarter's slot is QS (after the whole tiles when the
  // wave owns both, else the wave's first)
  constexpr int NQ = QPW + (SPLITM == 1 ? 1 : 0);
  constexpr int QS = SPLITM == 1 ? QPW : 0;
  const int k_begin = chunk * p.chunk;
  const int k_end = min(p.prefix_len, k_begin + p.chunk);
  const int n_tiles = (k_end - k_begin + KT - 1) / KT;

  const uint16_t* kbase = p.kc + (int64_t)g * p.cap * D;
  const uint16_t* vbase = p.vc + (int64_t)g * D * p.cap;

  // issue this wave's loads of tile t (< n_tiles) into buffer b: load j =
  // wave + r * WAVES; K rows for j < KBYTES / 1024, else V^T rows
  // the pages of tile t (paged cache): its KT / 16 = 4 table entries, one
  // 16-byte LDS read, taken before the barrier that precedes the tile's
  // loads so the table lookup is off their path
  typedef int int4v __attribute__((ext_vector_type(4)));
  static_assert(KT / 16 == 4, "four pages per tile");
  auto pages_of = [&](int t) __attribute__((always_inline)) -> int4v {
    if constexpr (PAGED) return *reinterpret_cast<const int4v*>(&s_tab[t * (KT / 16)]);
    return int4v{0, 0, 0, 0};
  };
  auto issue = [&](int t, int b, int4v pg4) __attribute__((always_inline)) {
    (void)pg4;
    const int k0 = k_begin + t * KT;
    const bool ragged = k0 + KT > k_end;
#pragma unroll
    for (int r = 0; r < LPW; ++r) {
      const int j = wave + r * WAVES;
      if (j >= NLD) continue;  // (wave-uniform)
      uint8_t* dst = lds + b * BUF + j * 1024;
      int tok, row, goff, cofs;
      bool is_v;
      if (j < KBYTES / 1024) {
        const int key = j * KROWS + lane / KCPR, pc = lane % KCPR;
        const int sw = ((key & 3) | (((key >> 3) & 3) << 2)) & (KCPR - 1);
        goff = key * D + (pc ^ sw) * 8;
        tok = key;
        is_v = false;
        row = key;
        cofs = (pc ^ sw) * 8;
      } else {
        const int dim = (j - KBYTES / 1024) * 8 + lane / 8, pc = lane % 8;
        goff = dim * p.cap + (pc ^ ((dim >> 1) & 7)) * 8;
        tok = (pc ^ ((dim >> 1) & 7)) * 8;
        is_v = true;
        row = dim;
        cofs = 0;
      }
      const uint16_t* src;
      if constexpr (PAGED) {
        // token of the chunk this lane's 16 bytes start at, and its page
        // (page tok / 16 of the tile)
        const int tic = k0 - k_begin + tok;
        const int c = tok >> 4;
        const int64_t pg = c == 0 ? pg4[0] : c == 1 ? pg4[1] : c == 2 ? pg4[2] : pg4[3];
        src = !is_v ? p.kc + ((pg * p.n_kv_heads + g) * 16 + (tic & 15)) * D + cofs
                    : p.vc + ((pg * p.n_kv_heads + g) * D + row) * 16 + (tic & 15);
      } else {
        src = is_v ? vbase + goff + k0 : kbase + goff + (int64_t)k0 * D;
      }
      if (!ragged) {
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      } else {
        // tokens past the prefix are zero: through registers (the compiler
        // waits for these loads before the LDS store)
        const int gk = k0 + tok;
        u32x4 val = u32x4{0u, 0u, 0u, 0u};
        if (gk < k_end) val = ld16(src);
        const int valid = k_end - gk;
        if (is_v && valid < 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= valid) val[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        *reinterpret_cast<u32x4*>(dst + lane * 16) = val;
      }
    }
  };

  // this wave's query tiles (row wave w: tiles w, w + ROWW, ..., then with
  // SPLIT the shared tile FT); Q^T fragments stay in registers, as bf16 hi +
  // lo when QLO
  auto is_quarter = [&](int i) __attribute__((always_inline)) { return SPLIT && i == QS && (SPLITM == 1 || has_q); };
  auto my_tile = [&](int i) __attribute__((always_inline)) { return is_quarter(i) ? FT : T0 + wave + ROWW * i; };
  bf16x8 qf[NQ][D / 32];
  bf16x8 ql[QLO ? NQ : 1][D / 32];
  f32x4 O[NQ][D / 16];
  float m[NQ], l[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int qt = my_tile(i);
    const int row = qt * 16 + lr;
    const bool ok = (is_quarter(i) ? qt < RT : qt < TE) && row < p.rows;
    int node = 0, head = 0;
    if (ok) {
      node = row / G;
      head = g * G + (row - node * G);
    }
    // all of this lane's q loads are issued before any is used
    const int64_t qoff = ((int64_t)node * p.n_q_heads + head) * D + lq * 8;
    if constexpr (QLO) {
      u32x4 raw[D / 32][2];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        raw[kk][0] = ld16(p.q32 + qoff + kk * 32);
        raw[kk][1] = ld16(p.q32 + qoff + kk * 32 + 4);
      }
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        uint32_t hv[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // scores come out in log2 units: q carries log2(e) / sqrt(d)
          const float x0 = ok ? __uint_as_float(raw[kk][e >> 1][(e & 1) * 2]) * p.scale_log2 : 0.f;
          const float x1 = ok ? __uint_as_float(raw[kk][e >> 1][(e & 1) * 2 + 1]) * p.scale_log2 : 0.f;
          split_pair(x0, x1, hv[e], lv[e]);
        }
        qf[i][kk] = __builtin_bit_cast(bf16x8, u32x4{hv[0], hv[1], hv[2], hv[3]});
        ql[i][kk] = __builtin_bit_cast(bf16x8, u32x4{lv[0], lv[1], lv[2], lv[3]});
      }
    } else {
      u32x4 raw[D / 32];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) raw[kk] = ld16(p.q + qoff + kk * 32);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        qf[i][kk] = __builtin_bit_cast(bf16x8, ok ? raw[kk] : u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[i] = -INFINITY;
    l[i] = 0.f;
  }

  // Lazy online softmax of one query tile over one block of scores, then its
  // PV.  The reference max only moves when some row's scores exceed it by more
  // than 8 (log2 units): the exponentials stay below 2^8, the final division by
  // l is unchanged, and most blocks skip the O rescale.  `sc` holds the scores
  // taken against `bias`.
  auto rescale_if_needed = [&](int i, float mx_here, float bias, auto& sc) __attribute__((always_inline)) {
    constexpr int cnt = sizeof(sc) / sizeof(sc[0]);
    const float mx = rows_max(mx_here);
    if (__builtin_amdgcn_ballot_w64(bias + mx > m[i] + 8.f) != 0) {
      const float m_new = fmaxf(m[i], bias + mx);
      const float alpha = __builtin_amdgcn_exp2f(m[i] - m_new);
      const float moved = m_new - bias;
#pragma unroll
      for (int e = 0; e < cnt; ++e) sc[e] -= moved;
      l[i] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) O[i][dt] *= alpha;
      m[i] = m_new;
    }
  };

  // One 32-key half (keys ks*32 ..) of a tile for every whole query tile of a
  // row wave.  The score MFMA's row r is key ks*32 + (r >> 2)*8 + h*4 + (r & 3),
  // so this lane gets keys ks*32 + lq*8 + h*4 + ii of query lr: the 8
  // consecutive keys the PV MFMA's B operand wants.
  auto row_half = [&](const uint16_t* K, const uint16_t* V, int ks, int k0, auto masked) __attribute__((always_inline)) {
    bf16x8 kf[2][D / 32];
    bf16x8 vf[D / 16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = ks * 32 + (lr >> 2) * 8 + h * 4 + (lr & 3);  // its swizzle is lr
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        kf[h][kk] = *reinterpret_cast<const bf16x8*>(K + key * D + (((kk * 4 + lq) ^ lr) & (KCPR - 1)) * 8);
    }
    f32x4 sc[QPW][2];
    float bias[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      if (my_tile(i) >= TE) continue;
      bias[i] = m[i] == -INFINITY ? 0.f : m[i];
      const float init = QLO ? -bias[i] : 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 a4 = f32x4{init, init, init, init};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[h][kk], qf[i][kk], a4, 0, 0, 0);
          if constexpr (QLO) a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[h][kk], ql[i][kk], a4, 0, 0, 0);
        }
        if constexpr (!QLO) a4 = a4 * p.scale_log2 - bias[i];
        sc[i][h] = a4;
      }
    }
    // the half's V^T fragments, read while the score MFMAs run (the K
    // fragments are dead by now)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      // V^T row dt*16 + lr (swizzle (lr >> 1) & 7), keys ks*32 + lq*8 ..
      vf[dt] = *reinterpret_cast<const bf16x8*>(V + (dt * 16 + lr) * KT + (((ks * 4 + lq) ^ ((lr >> 1) & 7)) * 8));
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      if (my_tile(i) >= TE) continue;
      float s[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = sc[i][e >> 2][e & 3];
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + ks * 32 + lq * 8 + (e >> 2) * 4 + (e & 3) >= k_end) s[e] = -INFINITY;
      }
      const float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      rescale_if_needed(i, mx, bias[i], s);
      float pv[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(s[e]);
        psum += pv[e];
      }
      l[i] += psum;
      // P as bf16 hi + lo (about 16 significant bits)
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_pair(pv[2 * e], pv[2 * e + 1], ph[e], pl[e]);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
      const bf16x8 plo = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        O[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pb, O[i][dt], 0, 0, 0);
        O[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], plo, O[i][dt], 0, 0, 0);
      }
    }
  };

  // A split tile's quarter: keys ks*32 + lq*8 + h*4 + ii (ks = qq >> 1,
  // h = qq & 1) of every 64-key tile, with the same lazy online softmax as a
  // whole tile; PV as 16x16x16 MFMAs on 4 keys per lane.
  auto quarter_tile = [&](const uint16_t* K, const uint16_t* V, int k0, auto masked) __attribute__((always_inline)) {
    constexpr int Q = QS;  // the quarter's slot in the tile arrays
    const int ks = qq >> 1, h = qq & 1;
    const int key = ks * 32 + (lr >> 2) * 8 + h * 4 + (lr & 3);
    bf16x8 kf[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      kf[kk] = *reinterpret_cast<const bf16x8*>(K + key * D + (((kk * 4 + lq) ^ lr) & (KCPR - 1)) * 8);
    const float bias = m[Q] == -INFINITY ? 0.f : m[Q];
    const float init = QLO ? -bias : 0.f;
    f32x4 a4 = f32x4{init, init, init, init};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[Q][kk], a4, 0, 0, 0);
      if constexpr (QLO) a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], ql[Q][kk], a4, 0, 0, 0);
    }
    if constexpr (!QLO) a4 = a4 * p.scale_log2 - bias;
    s16x4 vq[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      // V^T row dt*16 + lr, keys ks*32 + lq*8 + h*4 .. + 3: 8 bytes of chunk
      // ks*4 + lq, which the row's swizzle moved to (ks*4 + lq) ^ ((lr >> 1) & 7)
      vq[dt] = *reinterpret_cast<const s16x4*>(V + (dt * 16 + lr) * KT + (((ks * 4 + lq) ^ ((lr >> 1) & 7)) * 8) +
                                               h * 4);
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = a4[e];
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k0 + ks * 32 + lq * 8 + h * 4 + e >= k_end) s[e] = -INFINITY;
    }
    rescale_if_needed(Q, fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), bias, s);
    float pv[4], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pv[e] = __builtin_amdgcn_exp2f(s[e]);
      psum += pv[e];
    }
    l[Q] += psum;
    uint32_t ph[2], pl[2];
    split_pair(pv[0], pv[1], ph[0], pl[0]);
    split_pair(pv[2], pv[3], ph[1], pl[1]);
    const s16x4 pbs = __builtin_bit_cast(s16x4, u32x2{ph[0], ph[1]});
    const s16x4 pls = __builtin_bit_cast(s16x4, u32x2{pl[0], pl[1]});
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      O[Q][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vq[dt], pbs, O[Q][dt], 0, 0, 0);
      O[Q][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vq[dt], pls, O[Q][dt], 0, 0, 0);
    }
  };

  auto compute = [&](int buf, int k0, auto masked) __attribute__((always_inline)) {
    const uint16_t* K = reinterpret_cast<const uint16_t*>(lds + buf * BUF);
    const uint16_t* V = reinterpret_cast<const uint16_t*>(lds + buf * BUF + KBYTES);
    // (scheduling fences: no half's LDS reads are hoisted into the one
    // before it, which would hold two halves' fragments in registers)
    if (T0 + wave < TE) {  // a row wave with no query tile only loads
      row_half(K, V, 0, k0, masked);
      __builtin_amdgcn_sched_barrier(0);
      row_half(K, V, 1, k0, masked);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SPLIT) {
      if (has_q) quarter_tile(K, V, k0, masked);
    }
  };
  if constexpr (PAGED) {
    // the pages of this chunk's tiles (entries past the prefix: page 0, never read)
    const int pg0 = k_begin >> 4, npg = (k_end - k_begin + 15) >> 4;
    for (int i = tid; i < n_tiles * (KT / 16); i += WAVES * 64)
      s_tab[i] = i < npg ? min(max(p.table[pg0 + i], 0), p.n_phys - 1) : 0;
    __syncthreads();
  }
  if (n_tiles > 0) {
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t)
      if (t < n_tiles) issue(t, t, pages_of(t));
    // whole tiles in the loop; a ragged last tile (masked keys) after it, so
    // the loop body has a single path
    const int n_whole = (k_end - k_begin) / KT;
    auto step = [&](int t) __attribute__((always_inline)) {
      // this wave's part of tile t has landed once at most its direct-to-LDS
      // loads of the whole tiles after t (issued later, at most NBUF - 2 of
      // them) are in flight; a ragged tile's register loads are complete
      // before issue() returns, so they never count
      const int4v pg_next = t + NBUF - 1 < n_tiles ? pages_of(t + NBUF - 1) : int4v{0, 0, 0, 0};
      const int ahead = min(n_whole - 1 - t, NBUF - 2);
      if (NBUF >= 4 && ahead >= 2) {
        if (full_lpw) wait_vmcnt<2 * LPW>();
        else wait_vmcnt<2 * (LPW - 1)>();
      } else if (NBUF >= 3 && ahead >= 1) {
        if (full_lpw) wait_vmcnt<LPW>();
        else wait_vmcnt<LPW - 1>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();  // every part has; every wave is done with tile t - 1
      if (t + NBUF - 1 < n_tiles) issue(t + NBUF - 1, (t + NBUF - 1) % NBUF, pg_next);  // into tile t - 1's buffer
    };
    for (int t = 0; t < n_whole; ++t) {
      step(t);
      compute(t % NBUF, k_begin + t * KT, std::integral_constant<bool, false>());
    }
    if (n_whole < n_tiles) {
      step(n_whole);
      compute(n_whole % NBUF, k_begin + n_whole * KT, std::integral_constant<bool, true>());
    }
  }

#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int qt = my_tile(i);
    if (qt >= TE) continue;
    const float lt = rows_sum(l[i]);
    const int row = qt * 16 + lr;
    if (row < p.rows) {
      const float inv = 1.0f / lt;
      const int64_t prow = ((int64_t)chunk * p.n_kv_heads + g) * p.rows + row;
      float* dst = p.o_part + prow * D + lq * 4;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        // O^T layout: this lane holds query lr, dims dt*16 + 4*lq + ii
        *reinterpret_cast<f32x4*>(dst + dt * 16) = O[i][dt] * inv;
      if (lq == 0) {
        p.ml_part[prow * 2] = m[i];
        p.ml_part[prow * 2 + 1] = lt;
      }
    }
  }

  if constexpr (SPLIT) {
    // merge the four quarter states of tile FT: O = sum_q 2^(m_q - M) O_q / L
    // (the merge area reuses the tile ring)
    float* sO = reinterpret_cast<float*>(lds);  // [4][16][D]
    float* sm = sO + 4 * 16 * D;                // [4][16]
    float* sl = sm + 64;
    __syncthreads();  // every wave is done with the tile ring
    if (has_q) {
      const float lt = rows_sum(l[QS]);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<f32x4*>(sO + (qq * 16 + lr) * D + dt * 16 + lq * 4) = O[QS][dt];
      if (lq == 0) {
        sm[qq * 16 + lr] = m[QS];
        sl[qq * 16 + lr] = lt;
      }
    }
    __syncthreads();
    const int row = FT * 16 + lr;
    if (wave == 0 && row < p.rows) {
      float mq[4], M = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mq[q] = sm[q * 16 + lr];
        M = fmaxf(M, mq[q]);
      }
      float w[4], L = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = __builtin_amdgcn_exp2f(mq[q] - M);
        L += w[q] * sl[q * 16 + lr];
      }
      const float inv = 1.0f / L;
      const int64_t prow = ((int64_t)chunk * p.n_kv_heads + g) * p.rows + row;
      float* dst = p.o_part + prow * D + lq * 4;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o += w[q] * *reinterpret_cast<const f32x4*>(sO + (q * 16 + lr) * D + dt * 16 + lq * 4);
        *reinterpret_cast<f32x4*>(dst + dt * 16) = o * inv;
      }
      if (lq == 0) {
        p.ml_part[prow * 2] = M;
        p.ml_part[prow * 2 + 1] = L;
      }
    }
  }
}

constexpr int kMaxChunks = 512;

// One block (256 threads) per (node, query head): log-sum-exp merge of the
// prefix-chunk partials with the node's ancestor keys.  The chunk maxima and
// sums and the first chunk outputs are loaded before the ancestor scores are
// formed, so their latency overlaps.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineParams c, TreeArgs t) {
  constexpr int PARTS = 256 / D;  // threads per output dim
  constexpr int DPL = D / 64;     // dims per lane in the ancestor dot products
  constexpr int PRE = 16;         // chunk outputs per thread loaded up front
  constexpr int kAncRound = 4;    // ancestors per wave per round of key loads
  __shared__ float s_w[kMaxChunks];
  __shared__ float s_anc[kMaxNodes];
  __shared__ float s_wa[kMaxNodes];
  __shared__ int s_alist[kMaxNodes];
  __shared__ float s_red[4], s_red2[4];
  __shared__ float s_acc[PARTS][D];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int node = blockIdx.x / c.n_q_heads;
  const int h = blockIdx.x - node * c.n_q_heads;
  const int G = c.n_q_heads / c.n_kv_heads;
  const int g = h / G;
  const int row = node * G + (h - g * G);
  const uint64_t anc = t.anc[node];
  const int j = tid % D, part = tid / D;
  auto prow = [&](int ch) { return ((int64_t)ch * c.n_kv_heads + g) * c.rows + row; };

  // chunk statistics (one chunk per thread, more in a loop) and the first
  // PRE chunk outputs of this thread's dim
  float cm = -INFINITY, cl = 0.f;
  if (tid < c.n_chunks) {
    cm = c.ml_part[prow(tid) * 2];
    cl = c.ml_part[prow(tid) * 2 + 1];
  }
  float ov[PRE];
#pragma unroll
  for (int r = 0; r < PRE; ++r) {
    const int ch = part + r * PARTS;
    ov[r] = ch < c.n_chunks ? c.o_part[prow(ch) * D + j] : 0.f;
  }

  // the node's ancestors (itself included), in increasing order: node j
  // (lane j of the first wave) is the k-th, k = its set bits below j
  const int na = __popcll(anc);
  if (tid < kMaxNodes && ((anc >> tid) & 1ull)) s_alist[__popcll(anc & ((1ull << tid) - 1ull))] = tid;
  __syncthreads();
  // ancestor scores: wave w takes ancestors w, w + 4, ..., kAncRound of them
  // per round with every key load of the round in flight at once
  {
    float qv[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int64_t o = ((int64_t)node * c.n_q_heads + h) * D + lane * DPL + i;
      qv[i] = c.q32 ? c.q32[o] : bf16_bits_to_f32(c.q[o]);
    }
    // (one loop per key precision, so no load sits behind a branch)
    auto rounds = [&](auto kload) {
      for (int k0 = wave; k0 < na; k0 += 4 * kAncRound) {
        float kv[kAncRound][DPL];
#pragma unroll
        for (int r = 0; r < kAncRound; ++r) {
          const int a = s_alist[min(k0 + 4 * r, na - 1)];
#pragma unroll
          for (int i = 0; i < DPL; ++i) kv[r][i] = kload(((int64_t)a * c.n_kv_heads + g) * D + lane * DPL + i);
        }
#pragma unroll
        for (int r = 0; r < kAncRound; ++r) {
          if (k0 + 4 * r >= na) break;
          float sdot = 0.f;
#pragma unroll
          for (int i = 0; i < DPL; ++i) sdot += qv[i] * kv[r][i];
          sdot = wave_sum(sdot) * c.scale_log2;
          if (lane == 0) s_anc[k0 + 4 * r] = sdot;
        }
      }
    };
    if (c.k32)
      rounds([&](int64_t o) { return c.k32[o]; });
    else
      rounds([&](int64_t o) { return bf16_bits_to_f32(c.k_tree[o]); });
  }
  // running max over chunk maxima and ancestor scores
  float mx = cm;
  for (int ch = tid + 256; ch < c.n_chunks; ch += 256) mx = fmaxf(mx, c.ml_part[prow(ch) * 2]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  // ancestor k's score on lane k (at most 64 ancestors), reduced in the wave
  const float sa = lane < na ? s_anc[lane] : -INFINITY;
  M = fmaxf(M, wave_max(sa));
  float lsum = 0.f;
  if (tid < c.n_chunks) {
    const float w = __builtin_amdgcn_exp2f(cm - M) * cl;
    s_w[tid] = w;
    lsum = w;
  }
  for (int ch = tid + 256; ch < c.n_chunks; ch += 256) {
    const float w = __builtin_amdgcn_exp2f(c.ml_part[prow(ch) * 2] - M) * c.ml_part[prow(ch) * 2 + 1];
    s_w[ch] = w;
    lsum += w;
  }
  lsum = wave_sum(lsum);
  if (lane == 0) s_red2[wave] = lsum;
  __syncthreads();
  float L = (s_red2[0] + s_red2[1]) + (s_red2[2] + s_red2[3]);
  // the ancestors' weights: lane k's, kept for the values' sum below
  const float wa = lane < na ? __builtin_amdgcn_exp2f(sa - M) : 0.f;
  if (tid < kMaxNodes) s_wa[tid] = wa;
  L += wave_sum(wa);

  // weighted sum of the chunk outputs: PARTS threads per dim, fixed order
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < PRE; ++r) {
    const int ch = part + r * PARTS;
    if (ch < c.n_chunks) acc += s_w[ch] * ov[r];
  }
  for (int ch = part + PRE * PARTS; ch < c.n_chunks; ch += PARTS) acc += s_w[ch] * c.o_part[prow(ch) * D + j];
  s_acc[part][j] = acc;
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) o += s_acc[q][j];
    // the ancestors' values, kAncRound * 4 loads in flight per round, added in
    // ancestor order
    auto rounds = [&](auto vload) {
      for (int k0 = 0; k0 < na; k0 += 4 * kAncRound) {
        float vv[4 * kAncRound];
#pragma unroll
        for (int r = 0; r < 4 * kAncRound; ++r)
          vv[r] = vload(((int64_t)s_alist[min(k0 + r, na - 1)] * c.n_kv_heads + g) * D + j);
        // a select, not a break: every load above is then used, and none is
        // moved down behind a branch
#pragma unroll
        for (int r = 0; r < 4 * kAncRound; ++r) {
          const float w = k0 + r < na ? s_wa[min(k0 + r, na - 1)] : 0.f;
          o += w * vv[r];
        }
      }
    };
    if (c.v32)
      rounds([&](int64_t vo) { return c.v32[vo]; });
    else
      rounds([&](int64_t vo) { return bf16_bits_to_f32(c.v_tree[vo]); });
    o /= L;
    if (c.out32) {
      c.out32[((int64_t)node * c.n_q_heads + h) * D + j] = o;
    } else if (c.out_hilo) {
      // the Wo projection's operand: fp16 rows 2 node (hi) and 2 node + 1 (lo)
      const int64_t width = (int64_t)c.n_q_heads * D;
      const int64_t oo = (int64_t)(2 * node) * width + h * D + j;
      const f16 hi = (f16)o;
      c.out[oo] = __builtin_bit_cast(uint16_t, hi);
      c.out[oo + width] = f32_to_f16_bits(o - (float)hi);
    } else {
      c.out[((int64_t)node * c.n_q_heads + h) * D + j] = f32_to_bf16_bits(o);
    }
  }
}


// Depth of the partial kernel's LDS tile ring.
#ifndef LUCEV_ATTN_NBUF
#define LUCEV_ATTN_NBUF 2
#endif
constexpr int kAttnBufs = LUCEV_ATTN_NBUF;

int attention_max_chunks(int n_kv_heads) { return (device_cu_count() + n_kv_heads - 1) / n_kv_heads; }

// Wave layout knobs (fixed at build time): where the quarters of a split
// tile go (0: four extra waves beside one-tile waves; 1: the last four of
// the one-tile waves; 2: four waves of two whole tiles each), and whether 13
// to 16 query tiles take four waves of four tiles (1) or eight of two (0).
#ifndef LUCEV_ATTN_SPLIT_LAYOUT
#define LUCEV_ATTN_SPLIT_LAYOUT 0
#endif
#ifndef LUCEV_ATTN_WIDE4
#define LUCEV_ATTN_WIDE4 0
#endif

// Query tiles per SIMD as even as possible.  RT <= 4: one tile per wave, four
// waves; RT = 5 or 9 (4k + 1): the last tile split by key quarter; other RT up
// to 12: one tile per wave, 8 or 12 waves; 13 to 16: eight waves of two tiles;
// above 16: row groups of at most 16 tiles, eight waves of two (partial_layout).
AttnPlan plan_attention(int n_nodes, int n_q_heads, int n_kv_heads, int head_dim, int prefix_len) {
  (void)head_dim;
  AttnPlan a;
  a.rows = n_nodes * (n_q_heads / n_kv_heads);
  const int rt = (a.rows + 15) / 16;
  a.split = false;
  if (rt <= 4) {
    a.roww = 4;
    a.qpw = 1;
  } else if (rt % 4 == 1 && rt <= 9) {
    a.split = true;
    if (LUCEV_ATTN_SPLIT_LAYOUT == 2) {
      a.roww = 4;
      a.qpw = (rt - 1) / 4;
    } else {
      a.qpw = 1;
      a.roww = LUCEV_ATTN_SPLIT_LAYOUT == 1 ? rt - 1 : rt + 3;
    }
  } else if (rt <= 12) {
    a.roww = 4 * ((rt + 3) / 4);
    a.qpw = 1;
  } else if (rt <= 16) {
    a.roww = LUCEV_ATTN_WIDE4 ? 4 : 8;
    a.qpw = LUCEV_ATTN_WIDE4 ? 4 : 2;
  } else {
    a.roww = 8;  // row groups of at most 16 tiles, two per wave (partial_layout)
    a.qpw = 2;
  }
  a.waves = a.roww;
  // one block per CU over (chunk, KV head): chunks a multiple of the LDS tile
  const int cus = device_cu_count();
  int chunk = (int)(((int64_t)prefix_len * n_kv_heads + cus - 1) / cus);
  chunk = ((chunk + KT - 1) / KT) * KT;
  if (chunk < KT) chunk = KT;
  a.chunk = chunk;
  a.n_chunks = prefix_len > 0 ? (prefix_len + chunk - 1) / chunk : 0;
  return a;
}

// Blocks of a launch: chunks rounded up to 8 (the block -> chunk map keeps a
// chunk's row groups on one XCD), times the row groups.
static int partial_blocks(const AttnPlan& plan, int groups) { return ((plan.n_chunks + 7) / 8) * 8 * groups; }

template <int D, int QPW, int ROWW, int SPLITM>
static void launch_partial(const AttnPlan& plan, const AttnParams& p, int groups, hipStream_t s) {
  const dim3 grid(partial_blocks(plan, groups), p.n_kv_heads), block(64 * ROWW);
  if (p.table)
    hipLaunchKernelGGL((attn_partial_kernel<D, QPW, ROWW, kAttnBufs, false, SPLITM, true>), grid, block, 0, s, p);
  else if (p.q32)
    hipLaunchKernelGGL((attn_partial_kernel<D, QPW, ROWW, kAttnBufs, true, SPLITM, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((attn_partial_kernel<D, QPW, ROWW, kAttnBufs, false, SPLITM, false>), grid, block, 0, s, p);
}

// The partial kernel's wave layout for a plan: (tiles per row wave, row
// waves, where a split tile goes, row groups, tiles per group), as
// launch_partial_d instantiates it.  Past 16 query tiles, row groups of at
// most 16 tiles at two per wave: three or four tiles per wave on 8 waves
// spill (94 and 186 registers with q as hi + lo), and a 64-node tree at the
// 27B shape took 202 us a layer that way.
struct PartialLayout {
  int qpw, roww, splitm, groups, tiles;
};
static PartialLayout partial_layout(const AttnPlan& plan) {
  const int rt = (plan.rows + 15) / 16;
  if (plan.split) {
#if LUCEV_ATTN_SPLIT_LAYOUT == 2
    return {plan.qpw == 1 ? 1 : 2, 4, 1, 1, rt};
#elif LUCEV_ATTN_SPLIT_LAYOUT == 1
    return {1, plan.roww == 4 ? 4 : 8, 1, 1, rt};
#else
    return {1, plan.roww == 8 ? 8 : 12, 2, 1, rt};
#endif
  }
  if (plan.qpw == 1) return {1, plan.roww == 4 ? 4 : (plan.roww == 8 ? 8 : 12), 0, 1, rt};
#if LUCEV_ATTN_WIDE4
  if (plan.roww == 4) return {4, 4, 0, 1, rt};
#endif
  const int groups = (rt + 15) / 16;
  return {2, 8, 0, groups, (rt + groups - 1) / groups};
}

template <int D>
static void launch_partial_d(const AttnPlan& plan, AttnParams p, hipStream_t s) {
  const PartialLayout v = partial_layout(plan);
  p.row_groups = v.groups;
  p.group_tiles = v.tiles;
#define LUCEV_PARTIAL(Q, R, S)                            \
  if (v.qpw == Q && v.roww == R && v.splitm == S) {       \
    launch_partial<D, Q, R, S>(plan, p, v.groups, s);     \
    return;                                               \
  }
#if LUCEV_ATTN_SPLIT_LAYOUT == 2
  LUCEV_PARTIAL(1, 4, 1)
  LUCEV_PARTIAL(2, 4, 1)
#elif LUCEV_ATTN_SPLIT_LAYOUT == 1
  LUCEV_PARTIAL(1, 4, 1)
  LUCEV_PARTIAL(1, 8, 1)
#else
  LUCEV_PARTIAL(1, 8, 2)
  LUCEV_PARTIAL(1, 12, 2)
#endif
#if LUCEV_ATTN_WIDE4
  LUCEV_PARTIAL(4, 4, 0)
#endif
  LUCEV_PARTIAL(1, 4, 0)
  LUCEV_PARTIAL(1, 8, 0)
  LUCEV_PARTIAL(1, 12, 0)
  LUCEV_PARTIAL(2, 8, 0)
#undef LUCEV_PARTIAL
}

int describe_attention(const AttnPlan& plan, int head_dim, int n_kv_heads, int combine_blocks, bool fp32_q,
                       bool paged, char* buf, size_t len) {
  const PartialLayout v = partial_layout(plan);
  return snprintf(buf, len,
                  "attn_partial_kernel<%d, %d, %d, %d, %s, %d, %s> grid (%d, %d) block %d, %d-token chunks, "
                  "%d row group(s) of %d tiles; attn_combine_kernel<%d> grid %d block 256",
                  head_dim, v.qpw, v.roww, kAttnBufs, (fp32_q && !paged) ? "true" : "false", v.splitm,
                  paged ? "true" : "false", partial_blocks(plan, v.groups), n_kv_heads, 64 * v.roww, plan.chunk,
                  v.groups, v.tiles, head_dim, combine_blocks);
}

hipError_t launch_attention(const AttnPlan& plan, int head_dim, const AttnParams& p,
                            const CombineParams& c, const TreeArgs& t, hipStream_t s) {
  if (plan.n_chunks > 0) {
    if (head_dim == 128)
      launch_partial_d<128>(plan, p, s);
    else
      launch_partial_d<64>(plan, p, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_combine(head_dim, c, t, s);
}

hipError_t launch_combine(int head_dim, const CombineParams& c, const TreeArgs& t, hipStream_t s) {
  const int blocks = c.n * c.n_q_heads;
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(blocks), dim3(256), 0, s, c, t);
  else
    hipLaunchKernelGGL((attn_combine_kernel<64>), dim3(blocks), dim3(256), 0, s, c, t);
  return hipGetLastError();
}

}  // namespace lucev
