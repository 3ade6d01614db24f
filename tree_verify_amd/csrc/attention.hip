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
//   partial : grid (prefix chunk, KV head).  All n * Hq/Hkv query rows of the
//             KV head live in the block (16-row MFMA tiles, one or more per
//             wave); K and V tiles of 64 tokens are staged through LDS.
//             S^T = K Q^T puts the softmax axis (keys) inside each lane, so
//             the running max needs only two cross-lane steps; P then feeds
//             O^T = V^T P^T directly from registers (the key order inside a
//             16-key S tile is permuted so each lane already holds the 8
//             consecutive keys the second MFMA wants).  Output per (chunk,
//             row): max and sum in log2 units and the chunk-normalised O.
//   combine: one block per (node, query head): merges the chunk partials and
//             the (at most 64) ancestor keys with a log-sum-exp merge.
#include <type_traits>

#include "internal.h"

namespace lucev {

constexpr int KT = 64;  // tokens per LDS tile
constexpr int kMaxChunkPages = 1024;  // 16-token pages of one block's prefix chunk (paged cache)

// Waves per block for a query-tile count and tiles per wave.
constexpr int attn_max_waves(int qpw) { return qpw == 1 ? 12 : 8; }

// One block per (prefix chunk, KV head), one wave per QPW query tiles (waves
// past the last query tile only load).  K and V^T tiles of 64 tokens go
// straight from HBM into two LDS buffers with 16-byte direct-to-LDS loads:
// the next tile's loads are issued right after the barrier that publishes
// the current one, so they fly while the current tile is in the MFMAs, and
// each wave waits for all of its loads (vmcnt 0) before the next barrier.
// A load
// instruction fills 1 KB of LDS, 16 bytes per lane in lane order, so the bank
// swizzles are applied on the global side: LDS chunk c of K row `key` holds
// the row's 16-byte chunk c ^ ((key & 3) | ((key >> 3) & 3) << 2), and chunk
// c of V^T row `dim` holds chunk c ^ ((dim >> 1) & 7); the 16 rows one
// 16-lane group reads at once then fall in 16 different bank groups.  The
// ragged last tile of the prefix goes through registers so tokens past it
// are zero.
//
// SPLIT (one query tile per wave, RT = 4k + 1 tiles, RT + 3 <= 12): the four
// SIMDs of a CU would carry k + 1, k, k, k tiles, so the last (ragged) tile
// is instead shared by four waves, one per SIMD, each taking a fixed 16-key
// quarter of every 64-key tile with its own (max, sum, O); the four states
// are merged through LDS at the end.  The quarter's PV product is a
// 16x16x16 MFMA, whose B operand (4 keys per lane) is exactly the layout the
// 16-key score tile comes out in.
//
// PAGED: the prefix lives in 16-token pages, K as [page][Hkv][16][d] and V as
// [page][Hkv][d][16], and table[t / 16] names the page holding token t.  Only
// the global addresses of the tile loads change (a 1 KB K load covers 4 keys
// of one page; a 16-byte V chunk covers 8 tokens of one page), so the LDS
// tiles, and hence the results, are those of the contiguous cache.  The
// block's slice of the table is copied into LDS first, clamped to the pool.
template <int D, int QPW, bool QLO, bool SPLIT, bool PAGED = false>
__global__ __launch_bounds__(attn_max_waves(QPW) * 64) void attn_partial_kernel(AttnParams p) {
  static_assert(!SPLIT || QPW == 1, "split tiles use one query tile per wave");
  constexpr int WAVES = attn_max_waves(QPW);
  constexpr int KCPR = D / 8;                   // 16-byte chunks per K row
  constexpr int KROWS = 64 / KCPR;              // K rows per 1 KB load
  constexpr int KBYTES = KT * D * 2;            // one K tile
  constexpr int VBYTES = D * KT * 2;            // one V^T tile (rows of 128 bytes)
  constexpr int NLD = (KBYTES + VBYTES) / 1024; // 1 KB loads per tile
  constexpr int LPW = (NLD + WAVES - 1) / WAVES;  // loads per wave per tile
  constexpr int BUF = KBYTES + VBYTES;
  constexpr int MERGE = SPLIT ? 4 * 16 * D * 4 + 2 * 64 * 4 : 0;  // quarter states
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * BUF + MERGE];
  __shared__ int s_tab[PAGED ? kMaxChunkPages : 1];

  const int tid = threadIdx.x;
  // the wave index as a scalar: every branch on it is then a scalar branch
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int chunk = blockIdx.x;
  const int g = blockIdx.y;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int RT = (p.rows + 15) / 16;
  const int FT = SPLIT ? RT - 1 : RT;           // tiles a wave owns whole
  const bool quarter = SPLIT && wave >= FT && wave < FT + 4;
  const int qq = wave - FT;                     // quarter: keys (qq >> 1) * 32 + (qq & 1) * 4 + ..
  const int k_begin = chunk * p.chunk;
  const int k_end = min(p.prefix_len, k_begin + p.chunk);
  const int n_tiles = (k_end - k_begin + KT - 1) / KT;

  const uint16_t* kbase = p.kc + (int64_t)g * p.cap * D;
  const uint16_t* vbase = p.vc + (int64_t)g * D * p.cap;

  // Load j of a tile (j < NLD): K rows for j < KBYTES / 1024, else V^T rows.
  // This lane's global element offset at token 0 and its LDS byte offset.
  // (offsets within a tile's K rows or V^T rows: below D * cap < 2^31)
  auto load_slot = [&](int j, int& goff, int& loff, int& tok, bool& is_v, int& row, int& cofs) {
    if (j < KBYTES / 1024) {
      const int key = j * KROWS + lane / KCPR, pc = lane % KCPR;
      const int sw = ((key & 3) | (((key >> 3) & 3) << 2)) & (KCPR - 1);
      goff = key * D + (pc ^ sw) * 8;
      loff = j * 1024;
      tok = key;
      is_v = false;
      row = key;
      cofs = (pc ^ sw) * 8;
    } else {
      const int dim = (j - KBYTES / 1024) * 8 + lane / 8, pc = lane % 8;
      goff = dim * p.cap + (pc ^ ((dim >> 1) & 7)) * 8;
      loff = j * 1024;
      tok = (pc ^ ((dim >> 1) & 7)) * 8;
      is_v = true;
      row = dim;
      cofs = 0;
    }
  };
  // issue this wave's loads of tile t (< n_tiles) into buffer b
  auto issue = [&](int t, int b) {
    const int k0 = k_begin + t * KT;
    const bool ragged = k0 + KT > k_end;
#pragma unroll
    for (int r = 0; r < LPW; ++r) {
      const int j = wave + r * WAVES;
      // no load past the tile's last (surplus direct-to-LDS loads from
      // several waves into one shared scratch area made GEMM replays differ)
      if (j >= NLD) continue;
      uint8_t* dst = lds + b * BUF + j * 1024;
      int goff = 0;
      int loff = 0, tok = 0, row = 0, cofs = 0;
      bool is_v = false;
      if (j < NLD) load_slot(j, goff, loff, tok, is_v, row, cofs);
      const uint16_t* src;
      if constexpr (PAGED) {
        // token of the chunk this lane's 16 bytes start at, and its page
        const int tic = k0 - k_begin + tok;
        const int64_t pg = s_tab[tic >> 4];
        src = j >= NLD ? p.kc
              : !is_v ? p.kc + ((pg * p.n_kv_heads + g) * 16 + (tic & 15)) * D + cofs
                      : p.vc + ((pg * p.n_kv_heads + g) * D + row) * 16 + (tic & 15);
      } else {
        src = j < NLD ? (is_v ? vbase + goff + k0 : kbase + goff + (int64_t)k0 * D) : kbase;
      }
      if (!ragged || j >= NLD) {
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      } else {
        // tokens past the prefix are zero: through registers
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

  // query tiles of this wave; Q^T fragments stay in registers as bf16 hi + lo
  // (about 16 significant bits of q; the keys are exact bf16)
  bf16x8 qf[QPW][D / 32];
  bf16x8 ql[QPW][D / 32];
  f32x4 O[QPW][D / 16];
  float m[QPW], l[QPW];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int qt = SPLIT ? min(wave, FT) : wave * QPW + i;
    const int row = qt * 16 + lr;
    const bool ok = qt < RT && row < p.rows;
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
        bf16x8 hv, lv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // scores come out in log2 units: q carries log2(e) / sqrt(d)
          const float x = ok ? __uint_as_float(raw[kk][e >> 2][e & 3]) * p.scale_log2 : 0.f;
          const __bf16 hb = (__bf16)x;
          hv[e] = hb;
          lv[e] = (__bf16)(x - (float)hb);
        }
        qf[i][kk] = hv;
        ql[i][kk] = lv;
      }
    } else {
      u32x4 raw[D / 32];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) raw[kk] = ld16(p.q + qoff + kk * 32);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        qf[i][kk] = __builtin_bit_cast(bf16x8, ok ? raw[kk] : u32x4{0u, 0u, 0u, 0u});
        ql[i][kk] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  // One 16-key score tile of query tile i: A row r is key
  // ks*32 + (r >> 2)*8 + h*4 + (r & 3), so this lane gets keys
  // ks*32 + lq*8 + h*4 + ii of query lr (the order the PV operand wants).
  auto score16 = [&](const uint16_t* K, int i, int ks, int h, float init) -> f32x4 {
    f32x4 a4 = f32x4{init, init, init, init};
    // this lane's key row; its swizzle is lr, so d chunk kk*4 + lq sits at
    // (kk*4 + lq) ^ lr
    const int key = ks * 32 + (lr >> 2) * 8 + h * 4 + (lr & 3);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const bf16x8 a =
          *reinterpret_cast<const bf16x8*>(K + key * D + (((kk * 4 + lq) ^ lr) & (KCPR - 1)) * 8);
      a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[i][kk], a4, 0, 0, 0);
      if constexpr (QLO) a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[i][kk], a4, 0, 0, 0);
    }
    return a4;
  };
  // Scores of one 32-key half (keys ks*32 ..) for query tile i, as two 16-key
  // MFMA tiles.  With the hi/lo q (already scaled to log2 units) the
  // accumulators start at -bias, so they come out relative to the running
  // max; bias is the reference the scores were taken against.
  auto scores = [&](const uint16_t* K, int i, int ks, f32x4 (&sc)[2], float& bias) {
    bias = m[i] == -INFINITY ? 0.f : m[i];
    const float init = QLO ? -bias : 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) sc[h] = score16(K, i, ks, h, init);
    if constexpr (!QLO) {
#pragma unroll
      for (int h = 0; h < 2; ++h) sc[h] = sc[h] * p.scale_log2 - bias;
    }
  };

  // A split tile's quarter: keys ks*32 + lq*8 + h*4 + ii (ks = qq >> 1,
  // h = qq & 1) of every 64-key tile, with the same lazy online softmax as a
  // whole tile; PV as 16x16x16 MFMAs on 4 keys per lane.
  auto quarter_tile = [&](const uint16_t* K, const uint16_t* V, int k0, auto masked) {
    const int ks = qq >> 1, h = qq & 1;
    const float bias = m[0] == -INFINITY ? 0.f : m[0];
    f32x4 sc = score16(K, 0, ks, h, QLO ? -bias : 0.f);
    if constexpr (!QLO) sc = sc * p.scale_log2 - bias;
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (k0 + ks * 32 + lq * 8 + h * 4 + ii >= k_end) sc[ii] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    if (__builtin_amdgcn_ballot_w64(bias + mx > m[0] + 8.f) != 0) {
      const float m_new = fmaxf(m[0], bias + mx);
      const float alpha = __builtin_amdgcn_exp2f(m[0] - m_new);
      sc -= m_new - bias;
      l[0] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) O[0][dt] *= alpha;
      m[0] = m_new;
    }
    float psum = 0.f;
    bf16x4 pb, pl;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const float pv = __builtin_amdgcn_exp2f(sc[ii]);
      psum += pv;
      const __bf16 hb = (__bf16)pv;
      pb[ii] = hb;
      pl[ii] = (__bf16)(pv - (float)hb);
    }
    l[0] += psum;
    const s16x4 pbs = __builtin_bit_cast(s16x4, pb), pls = __builtin_bit_cast(s16x4, pl);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      // V^T row dt*16 + lr, keys ks*32 + lq*8 + h*4 .. + 3: 8 bytes of chunk
      // ks*4 + lq, which the row's swizzle moved to (ks*4 + lq) ^ ((lr >> 1) & 7)
      const s16x4 a = *reinterpret_cast<const s16x4*>(
          V + (dt * 16 + lr) * KT + (((ks * 4 + lq) ^ ((lr >> 1) & 7)) * 8) + h * 4);
      O[0][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbs, O[0][dt], 0, 0, 0);
      O[0][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pls, O[0][dt], 0, 0, 0);
    }
  };

  // Online softmax of one half and its PV product.  The reference max only
  // moves when some row's scores exceed it by more than 8 (log2 units): the
  // exponentials stay below 2^8, the final division by l is unchanged, and
  // most halves skip the rescale.  Returns by how much the reference moved.
  auto softmax_pv = [&](const uint16_t* V, int i, int ks, f32x4 (&sc)[2], float bias, int k0,
                        auto masked) -> float {
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          if (k0 + ks * 32 + lq * 8 + h * 4 + ii >= k_end) sc[h][ii] = -INFINITY;
    }
    // this lane holds query lr, keys ks*32 + lq*8 + h*4 + ii
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    float moved = 0.f;
    if (__builtin_amdgcn_ballot_w64(bias + mx > m[i] + 8.f) != 0) {
      const float m_new = fmaxf(m[i], bias + mx);
      const float alpha = __builtin_amdgcn_exp2f(m[i] - m_new);
      moved = m_new - bias;
#pragma unroll
      for (int h = 0; h < 2; ++h) sc[h] -= moved;
      l[i] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) O[i][dt] *= alpha;
      m[i] = m_new;
    }
    float psum = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float pv = __builtin_amdgcn_exp2f(sc[h][ii]);
        sc[h][ii] = pv;
        psum += pv;
      }
    l[i] += psum;
    // P as bf16 hi + lo (about 16 significant bits)
    bf16x8 pb, pl;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const __bf16 h0 = (__bf16)sc[0][ii];
      const __bf16 h1 = (__bf16)sc[1][ii];
      pb[ii] = h0;
      pb[4 + ii] = h1;
      pl[ii] = (__bf16)(sc[0][ii] - (float)h0);
      pl[4 + ii] = (__bf16)(sc[1][ii] - (float)h1);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      // V^T row dt*16 + lr (swizzle (lr >> 1) & 7), keys ks*32 + lq*8 ..
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          V + (dt * 16 + lr) * KT + (((ks * 4 + lq) ^ ((lr >> 1) & 7)) * 8));
      O[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, O[i][dt], 0, 0, 0);
      O[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl, O[i][dt], 0, 0, 0);
    }
    // relative to m after this half, scores taken against bias sit lower by:
    return m[i] - bias;
  };

  // one 64-key tile, half after half (the second half's scores are taken
  // against the reference the first half left)
  auto compute = [&](int buf, int k0, auto masked) {
    const uint16_t* K = reinterpret_cast<const uint16_t*>(lds + buf * BUF);
    const uint16_t* V = reinterpret_cast<const uint16_t*>(lds + buf * BUF + KBYTES);
    if constexpr (SPLIT) {
      if (quarter) {
        quarter_tile(K, V, k0, masked);
        return;
      }
      if (wave >= FT) return;
    }
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int qt = wave * QPW + i;
      if (qt >= RT) continue;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f32x4 sc[2];
        float bias;
        scores(K, i, ks, sc, bias);
        softmax_pv(V, i, ks, sc, bias, k0, masked);
      }
    }
  };
  auto compute_tile = [&](int buf, int t) {
    const int k0 = k_begin + t * KT;
    if (k0 + KT <= k_end)
      compute(buf, k0, std::integral_constant<bool, false>());
    else
      compute(buf, k0, std::integral_constant<bool, true>());
  };

  if constexpr (PAGED) {
    // the pages of this chunk's tiles (entries past the prefix: page 0, never read)
    const int pg0 = k_begin >> 4, npg = (k_end - k_begin + 15) >> 4;
    for (int i = tid; i < n_tiles * (KT / 16); i += WAVES * 64)
      s_tab[i] = i < npg ? min(max(p.table[pg0 + i], 0), p.n_phys - 1) : 0;
    __syncthreads();
  }
  if (n_tiles > 0) {
    issue(0, 0);
    for (int t = 0; t < n_tiles; ++t) {
      wait_vmcnt<0>();  // this wave's part of tile t has landed
      lds_barrier();    // every part has; every wave is done with tile t - 1
      if (t + 1 < n_tiles) issue(t + 1, (t + 1) & 1);  // into tile t - 1's buffer
      compute_tile(t & 1, t);
    }
  }

#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int qt = wave * QPW + i;
    if (qt >= FT) continue;
    float lt = l[i] + shfl_xor(l[i], 16);
    lt += shfl_xor(lt, 32);
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
    float* sO = reinterpret_cast<float*>(lds + 2 * BUF);  // [4][16][D]
    float* sm = sO + 4 * 16 * D;                                 // [4][16]
    float* sl = sm + 64;
    __syncthreads();  // (also: every wave is done with the tile ring)
    if (quarter) {
      float lt = l[0] + shfl_xor(l[0], 16);
      lt += shfl_xor(lt, 32);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<f32x4*>(sO + (qq * 16 + lr) * D + dt * 16 + lq * 4) = O[0][dt];
      if (lq == 0) {
        sm[qq * 16 + lr] = m[0];
        sl[qq * 16 + lr] = lt;
      }
    }
    __syncthreads();
    const int row = FT * 16 + lr;
    if (wave == FT && row < p.rows) {
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
  __shared__ int s_alist[kMaxNodes];
  __shared__ float s_red[4];
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

  // the node's ancestors (itself included), in increasing order
  const int na = __popcll(anc);
  if (tid == 0) {
    uint64_t m = anc;
    for (int k = 0; k < na; ++k) {
      s_alist[k] = __builtin_ctzll(m);
      m &= m - 1;
    }
  }
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
  for (int k = 0; k < na; ++k) M = fmaxf(M, s_anc[k]);
  __syncthreads();
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
  if (lane == 0) s_red[wave] = lsum;
  __syncthreads();
  float L = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  for (int k = 0; k < na; ++k) L += __builtin_amdgcn_exp2f(s_anc[k] - M);

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
          const float w = k0 + r < na ? __builtin_amdgcn_exp2f(s_anc[min(k0 + r, na - 1)] - M) : 0.f;
          o += w * vv[r];
        }
      }
    };
    if (c.v32)
      rounds([&](int64_t vo) { return c.v32[vo]; });
    else
      rounds([&](int64_t vo) { return bf16_bits_to_f32(c.v_tree[vo]); });
    o /= L;
    if (c.out_hilo) {
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

static_assert(kMaxAttnRows == attn_max_waves(4) * 4 * 16, "the widest plan covers every allowed row");

int attention_max_chunks(int n_kv_heads) { return (256 + n_kv_heads - 1) / n_kv_heads; }

AttnPlan plan_attention(int n_nodes, int n_q_heads, int n_kv_heads, int head_dim, int prefix_len) {
  (void)head_dim;
  AttnPlan a;
  a.rows = n_nodes * (n_q_heads / n_kv_heads);
  const int rt = (a.rows + 15) / 16;
  a.qpw = rt <= attn_max_waves(1) ? 1 : (rt + attn_max_waves(2) - 1) / attn_max_waves(2);
  a.waves = attn_max_waves(a.qpw);
  // a ragged last tile that would leave one SIMD a tile more than the others
  // is shared by four waves, one per SIMD
  a.split = a.qpw == 1 && rt % 4 == 1 && rt + 3 <= a.waves;
  // one block per CU over (chunk, KV head): chunks a multiple of the LDS tile
  int chunk = (int)(((int64_t)prefix_len * n_kv_heads + 255) / 256);
  chunk = ((chunk + KT - 1) / KT) * KT;
  if (chunk < KT) chunk = KT;
  a.chunk = chunk;
  a.n_chunks = prefix_len > 0 ? (prefix_len + chunk - 1) / chunk : 0;
  return a;
}

template <int D, int QPW, bool SPLIT>
static void launch_partial3(const AttnPlan& plan, const AttnParams& p, hipStream_t s) {
  if (p.table)
    hipLaunchKernelGGL((attn_partial_kernel<D, QPW, false, SPLIT, true>), dim3(plan.n_chunks, p.n_kv_heads),
                       dim3(64 * attn_max_waves(QPW)), 0, s, p);
  else if (p.q32)
    hipLaunchKernelGGL((attn_partial_kernel<D, QPW, true, SPLIT>), dim3(plan.n_chunks, p.n_kv_heads),
                       dim3(64 * attn_max_waves(QPW)), 0, s, p);
  else
    hipLaunchKernelGGL((attn_partial_kernel<D, QPW, false, SPLIT>), dim3(plan.n_chunks, p.n_kv_heads),
                       dim3(64 * attn_max_waves(QPW)), 0, s, p);
}

template <int D, int QPW>
static void launch_partial(const AttnPlan& plan, const AttnParams& p, hipStream_t s) {
  if constexpr (QPW == 1) {
    if (plan.split) {
      launch_partial3<D, 1, true>(plan, p, s);
      return;
    }
  }
  launch_partial3<D, QPW, false>(plan, p, s);
}

hipError_t launch_attention(const AttnPlan& plan, int head_dim, const AttnParams& p,
                            const CombineParams& c, const TreeArgs& t, hipStream_t s) {
  if (plan.n_chunks > 0) {
    if (head_dim == 128) {
      switch (plan.qpw) {
        case 1: launch_partial<128, 1>(plan, p, s); break;
        case 2: launch_partial<128, 2>(plan, p, s); break;
        case 3: launch_partial<128, 3>(plan, p, s); break;
        default: launch_partial<128, 4>(plan, p, s); break;
      }
    } else {
      switch (plan.qpw) {
        case 1: launch_partial<64, 1>(plan, p, s); break;
        case 2: launch_partial<64, 2>(plan, p, s); break;
        case 3: launch_partial<64, 3>(plan, p, s); break;
        default: launch_partial<64, 4>(plan, p, s); break;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int blocks = c.n * c.n_q_heads;
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(blocks), dim3(256), 0, s, c, t);
  else
    hipLaunchKernelGGL((attn_combine_kernel<64>), dim3(blocks), dim3(256), 0, s, c, t);
  return hipGetLastError();
}

}  // namespace lucev
