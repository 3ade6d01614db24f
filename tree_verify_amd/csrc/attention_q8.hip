// Tree attention over an int8 KV prefix, and the quantiser that writes one.
//
// The KV cache is held as int8 codes with one fp16 scale per 32 values, the
// q8_0 cache type the pages run beside F16 and Q4_0 ("Lucebox Hub", sections
// "Paged attention + continuous batching" and "설치·사용법"; KV size is the
// VRAM limit of section "배경: 어떤 문제를 푸는가", item 3).  Keys are blocked
// along the head dim of each token, values along the tokens of each dim (the
// cache keeps V dim-major), so a 32-key half of a tile and a 32-dim slice of
// a key each carry one scale.
//
// The partial kernel follows the bf16 one (blocks over prefix chunk and KV
// head, 64-token tiles in a two-buffer LDS ring), with four differences:
//   * one query tile (16 rows) per wave, and the query tiles of a KV head
//     spread over up to 8-tile row groups, one block per (chunk, group):
//     a wave's scores, O and fp16 hi/lo queries leave no room for a second
//     tile in 256 registers.  The groups of a chunk sit on one XCD (block
//     ids 8 apart), so the second group's tile reads hit that XCD's L2;
//   * tiles go through registers: 16 codes per lane are loaded, turned into
//     16 exact fp16 values (1024 + u under the fp16 exponent, then minus
//     1152) and stored into LDS in the bf16 kernel's swizzled layout, with
//     the tile's scales beside them; the next tile's loads fly while the
//     current tile is computed;
//   * the MFMAs are f16 (codes exact; queries and P as nearest fp16, each
//     off by at most 2^-11 of itself), one 32-deep block at a time, and each
//     block's fp32 result is multiplied by its scale as it is accumulated, so
//     d * code enters exactly;
//   * no split query tile.
// The combine kernel is the bf16 path's.
#include <stdio.h>

#include "attn_common.h"

namespace lucev {

typedef f16 f16x4 __attribute__((ext_vector_type(4)));

// 4 int8 codes (one dword) -> 4 exact fp16 values, in order: byte b of
// w ^ 0x80808080 is u = code + 128; placed under the exponent of 1024 it reads
// 1024 + u, and 1024 + u - 1152 = code.
__device__ __forceinline__ u32x2 codes4_f16(uint32_t w) {
  const uint32_t x = w ^ 0x80808080u;
  // v_perm_b32 bytes: selectors 0-3 take bytes of the second operand (x),
  // 4-7 bytes of the first (0x64 everywhere)
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);  // [x0, 64, x1, 64]
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);  // [x2, 64, x3, 64]
  const f16x2 bias = {(f16)1152.0f, (f16)1152.0f};
  const f16x2 a = __builtin_bit_cast(f16x2, lo) - bias;
  const f16x2 b = __builtin_bit_cast(f16x2, hi) - bias;
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// Two fp32 values as fp16 (nearest), packed
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(f16)a, (f16)b});
}

// LDS tile of the int8 path: K [64 keys][D] fp16 and V^T [D][64] fp16 in the
// bf16 kernel's swizzled layouts, then the scales widened to fp32 once, as
// they are stored: K scales [D/32 blocks][64 keys] and V scales [2 token
// blocks][D], so the four a lane applies to one MFMA result are one 16-byte
// read.
template <int D>
struct Q8Tile {
  static constexpr int KBYTES = KT * D * 2;
  static constexpr int VBYTES = D * KT * 2;
  static constexpr int KSC = KBYTES + VBYTES;             // K scales
  static constexpr int VSC = KSC + KT * (D / 32) * 4;     // V scales
  static constexpr int BYTES = VSC + D * 2 * 4;
  // global loads per tile, 16 bytes a lane: K codes (one lane: 16 codes of a
  // key), V codes (16 tokens of a dim), K scales (8 bytes a lane), V scales
  // (4 bytes a lane per dim, two loads)
  static constexpr int NK = KT * D / 1024;  // 1 KB of codes per wave-load
  static constexpr int NV = D * KT / 1024;
  static constexpr int NS = 1 + (D * 4 + 255) / 256;  // K scales, then V scales (64 dims a load)
  static constexpr int SLOTS = NK + NV + NS;
};

template <int D, int ROWW>
__global__ __launch_bounds__(ROWW * 64) void attn_partial_q8_kernel(
    AttnParams p) {
  using T = Q8Tile<D>;
  constexpr int WAVES = ROWW;
  constexpr int KCPR = D / 8;  // 16-byte chunks per K row
  constexpr int LPW = (T::SLOTS + WAVES - 1) / WAVES;
  constexpr int NBLK = D / 32;  // key scale blocks per key
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * T::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  // block x -> (chunk, row group): chunks c and c + 8 are 8 * groups ids apart,
  // the groups of chunk c ids 8 apart (one XCD); padding blocks past the
  // last chunk leave at once
  const int x = blockIdx.x;
  const int grp = (x >> 3) % p.q8_groups;
  const int chunk = (x / (8 * p.q8_groups)) * 8 + (x & 7);
  if (chunk >= p.n_chunks) return;
  const int g = blockIdx.y;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int RT = (p.rows + 15) / 16;
  const int qt = grp * p.q8_tiles + wave;  // this wave's query tile
  const bool active = wave < p.q8_tiles && qt < RT;
  const int k_begin = chunk * p.chunk;
  const int k_end = min(p.prefix_len, k_begin + p.chunk);
  const int n_tiles = (k_end - k_begin + KT - 1) / KT;

  const int8_t* kcode = p.kc8 + (int64_t)g * p.cap * D;
  const int8_t* vcode = p.vc8 + (int64_t)g * D * p.cap;
  const uint16_t* kscale = p.ks16 + (int64_t)g * p.cap * NBLK;
  const uint16_t* vscale = p.vs16 + (int64_t)g * D * (p.cap / 32);

  // One wave-load slot j of tile t into registers (zeros past the prefix).
  // Slot kinds: [0, NK) K codes, [NK, NK + NV) V codes, then the scales.
  auto load_slot = [&](int t, int j) -> u32x4 {
    const int k0 = k_begin + t * KT;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (j < T::NK) {
      const int key = j * (1024 / D) + lane / (D / 16);  // 16 codes a lane: D / 16 lanes per key
      const int c16 = lane % (D / 16);
      if (k0 + key < k_end) v = ld16(kcode + (int64_t)(k0 + key) * D + c16 * 16);
    } else if (j < T::NK + T::NV) {
      const int jj = j - T::NK;
      const int dim = jj * 16 + lane / 4, part = lane % 4;  // 16 tokens a lane: 4 lanes per dim
      if (k0 + part * 16 < k_end) v = ld16(vcode + (int64_t)dim * p.cap + k0 + part * 16);
    } else if (j == T::NK + T::NV) {
      // K scales: key `lane`, its NBLK scales (NBLK * 2 bytes)
      if (k0 + lane < k_end) {
        const uint16_t* src = kscale + (int64_t)(k0 + lane) * NBLK;
        if constexpr (NBLK == 4) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(src);
          v = u32x4{w[0], w[1], 0u, 0u};
        } else {
          v = u32x4{*reinterpret_cast<const uint32_t*>(src), 0u, 0u, 0u};
        }
      }
    } else {
      // V scales: dim (j - NK - NV - 1) * 64 + lane, the tile's two 32-token blocks
      const int dim = (j - T::NK - T::NV - 1) * 64 + lane;
      if (dim < D) {
        const uint16_t* src = vscale + (int64_t)dim * (p.cap / 32) + k0 / 32;
        const uint32_t s0 = k0 < k_end ? src[0] : 0u;
        const uint32_t s1 = k0 + 32 < k_end ? src[1] : 0u;
        v = u32x4{s0 | (s1 << 16), 0u, 0u, 0u};
      }
    }
    return v;
  };
  // Slot j's registers into LDS buffer b: codes converted to fp16 in the
  // swizzled tile layouts (tokens past the prefix were loaded as zero codes).
  auto store_slot = [&](int t, int j, const u32x4& v, int b) {
    uint8_t* base = lds + b * T::BYTES;
    const int k0 = k_begin + t * KT;
    if (j < T::NK) {
      const int key = j * (1024 / D) + lane / (D / 16);
      const int c16 = lane % (D / 16);
      const int sw = ((key & 3) | (((key >> 3) & 3) << 2)) & (KCPR - 1);
      const u32x2 a = codes4_f16(v[0]), bb = codes4_f16(v[1]), c = codes4_f16(v[2]), d = codes4_f16(v[3]);
      uint8_t* row = base + key * D * 2;
      *reinterpret_cast<u32x4*>(row + (((2 * c16) ^ sw) * 16)) = u32x4{a[0], a[1], bb[0], bb[1]};
      *reinterpret_cast<u32x4*>(row + (((2 * c16 + 1) ^ sw) * 16)) = u32x4{c[0], c[1], d[0], d[1]};
    } else if (j < T::NK + T::NV) {
      const int jj = j - T::NK;
      const int dim = jj * 16 + lane / 4, part = lane % 4;
      const int swz = (dim >> 1) & 7;
      u32x4 w = v;
      // tokens past the prefix inside this 16-token run read as code 0
      const int valid = k_end - (k0 + part * 16);
      if (valid < 16) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (e >= valid) w[e >> 2] &= ~(0xFFu << (8 * (e & 3)));
      }
      const u32x2 a = codes4_f16(w[0]), bb = codes4_f16(w[1]), c = codes4_f16(w[2]), d = codes4_f16(w[3]);
      uint8_t* row = base + T::KBYTES + dim * KT * 2;
      *reinterpret_cast<u32x4*>(row + (((2 * part) ^ swz) * 16)) = u32x4{a[0], a[1], bb[0], bb[1]};
      *reinterpret_cast<u32x4*>(row + (((2 * part + 1) ^ swz) * 16)) = u32x4{c[0], c[1], d[0], d[1]};
    } else if (j == T::NK + T::NV) {
      float* ksc = reinterpret_cast<float*>(base + T::KSC);
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
        ksc[b * KT + lane] = (float)__builtin_bit_cast(f16, (uint16_t)(v[b >> 1] >> (16 * (b & 1))));
    } else {
      const int dim = (j - T::NK - T::NV - 1) * 64 + lane;
      float* vsc = reinterpret_cast<float*>(base + T::VSC);
      if (dim < D) {
        vsc[dim] = (float)__builtin_bit_cast(f16, (uint16_t)(v[0] & 0xFFFFu));
        vsc[D + dim] = (float)__builtin_bit_cast(f16, (uint16_t)(v[0] >> 16));
      }
    }
  };

  // this wave's query tile; Q^T as fp16, scaled to log2 units
  typedef f16 f16x8_t __attribute__((ext_vector_type(8)));
  f16x8_t qf[D / 32];
  f32x4 O[D / 16];
  float m = -INFINITY, l = 0.f;
  {
    const int row = qt * 16 + lr;
    const bool ok = active && row < p.rows;
    int node = 0, head = 0;
    if (ok) {
      node = row / G;
      head = g * G + (row - node * G);
    }
    const int64_t qoff = ((int64_t)node * p.n_q_heads + head) * D + lq * 8;
    u32x4 raw[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) raw[kk] = ld16(p.q + qoff + kk * 32);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint32_t hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = ok ? bf16_bits_to_f32(raw[kk][e] & 0xFFFFu) * p.scale_log2 : 0.f;
        const float x1 = ok ? bf16_bits_to_f32(raw[kk][e] >> 16) * p.scale_log2 : 0.f;
        hv[e] = pack_f16(x0, x1);
      }
      qf[kk] = __builtin_bit_cast(f16x8_t, u32x4{hv[0], hv[1], hv[2], hv[3]});
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One 32-key half of a tile: scores (the K fragments and scales of one
  // 16-key group at a time), their softmax, then PV one 16-dim tile at a time.
  auto row_half = [&](const uint8_t* buf, int ks, int k0, bool masked) {
    const uint16_t* K = reinterpret_cast<const uint16_t*>(buf);
    const uint16_t* V = reinterpret_cast<const uint16_t*>(buf + T::KBYTES);
    const float bias = m == -INFINITY ? 0.f : m;
    float s[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = ks * 32 + (lr >> 2) * 8 + h * 4 + (lr & 3);  // its swizzle is lr
      // scales of this lane's MFMA output rows: keys ks*32 + lq*8 + h*4 + ii
      const float* sp = reinterpret_cast<const float*>(buf + T::KSC) + ks * 32 + lq * 8 + h * 4;
      f32x4 a4 = f32x4{-bias, -bias, -bias, -bias};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        // one 32-dim block of the keys: its fp32 sum times the block scale
        const f16x8_t kf =
            *reinterpret_cast<const f16x8_t*>(K + key * D + (((kk * 4 + lq) ^ lr) & (KCPR - 1)) * 8);
        const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[kk], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const f32x4 sc = *reinterpret_cast<const f32x4*>(sp + kk * KT);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) a4[ii] = __builtin_fmaf(t[ii], sc[ii], a4[ii]);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) s[h * 4 + ii] = a4[ii];
    }
    if (masked) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k0 + ks * 32 + lq * 8 + e >= k_end) s[e] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = rows_max(mx);
    // lazy rescale: only when the running max moves up by more than 2^8
    if (__builtin_amdgcn_ballot_w64(bias + mx > m + 8.f) != 0) {
      const float m_new = fmaxf(m, bias + mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      const float moved = m_new - bias;
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] -= moved;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) O[dt] *= alpha;
      m = m_new;
    }
    float pv[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = __builtin_amdgcn_exp2f(s[e]);
      psum += pv[e];
    }
    l += psum;
    const f16x8_t pb = __builtin_bit_cast(
        f16x8_t, u32x4{pack_f16(pv[0], pv[1]), pack_f16(pv[2], pv[3]), pack_f16(pv[4], pv[5]), pack_f16(pv[6], pv[7])});
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      // V^T row dt*16 + lr; the scales of this lane's 4 output dims (the half
      // is one 32-token block of every dim)
      const f16x8_t vf =
          *reinterpret_cast<const f16x8_t*>(V + (dt * 16 + lr) * KT + (((ks * 4 + lq) ^ ((lr >> 1) & 7)) * 8));
      const f32x4 sc = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(buf + T::VSC) + ks * D + dt * 16 +
                                                      4 * lq);
      const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) O[dt][ii] = __builtin_fmaf(t[ii], sc[ii], O[dt][ii]);
    }
  };

  // Tiles go through registers two ahead: at step t the loads of tile t + 2
  // are issued into the register set tile t used, tile t is computed, and
  // tile t + 1 (loaded during step t - 1) is converted into the LDS buffer
  // tile t - 1 used, which every wave has finished (the barrier at the top of
  // step t).
  if (n_tiles > 0) {
    u32x4 regs[2][LPW];
    auto load_tile = [&](int t, u32x4 (&r)[LPW]) {
#pragma unroll
      for (int k = 0; k < LPW; ++k) {
        const int j = wave + k * WAVES;
        if (j < T::SLOTS) r[k] = load_slot(t, j);
      }
    };
    auto store_tile = [&](int t, const u32x4 (&r)[LPW], int b) {
#pragma unroll
      for (int k = 0; k < LPW; ++k) {
        const int j = wave + k * WAVES;
        if (j < T::SLOTS) store_slot(t, j, r[k], b);
      }
    };
    load_tile(0, regs[0]);
    if (n_tiles > 1) load_tile(1, regs[1]);
    store_tile(0, regs[0], 0);
    auto step = [&](int t, u32x4 (&mine)[LPW], u32x4 (&next)[LPW]) {
      lds_barrier();  // tile t is in buffer t & 1; every wave is done with tile t - 1
      if (t + 2 < n_tiles) load_tile(t + 2, mine);
      const int k0 = k_begin + t * KT;
      if (active) {
        const uint8_t* buf = lds + (t & 1) * T::BYTES;
        const bool masked = k0 + KT > k_end;
        row_half(buf, 0, k0, masked);
        row_half(buf, 1, k0, masked);
      }
      if (t + 1 < n_tiles) store_tile(t + 1, next, (t + 1) & 1);
    };
    // unrolled by two so each register set is a fixed array
    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
      step(t, regs[0], regs[1]);
      step(t + 1, regs[1], regs[0]);
    }
    if (t < n_tiles) step(t, regs[0], regs[1]);
  }

  if (active) {
    const float lt = rows_sum(l);
    const int row = qt * 16 + lr;
    if (row < p.rows) {
      const float inv = 1.0f / lt;
      const int64_t prow = ((int64_t)chunk * p.n_kv_heads + g) * p.rows + row;
      float* dst = p.o_part + prow * D + lq * 4;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(dst + dt * 16) = O[dt] * inv;
      if (lq == 0) {
        p.ml_part[prow * 2] = m;
        p.ml_part[prow * 2 + 1] = lt;
      }
    }
  }
}

// Row groups: up to 4 query tiles in one 4-wave block, else groups of at
// most 8 tiles (as even as they come) on 8-wave blocks.
static void q8_groups(const AttnPlan& plan, int& groups, int& tiles) {
  const int rt = (plan.rows + 15) / 16;
  groups = rt <= 4 ? 1 : (rt + 7) / 8;
  tiles = (rt + groups - 1) / groups;
}

template <int D>
static void launch_q8_d(const AttnPlan& plan, AttnParams p, hipStream_t s) {
  q8_groups(plan, p.q8_groups, p.q8_tiles);
  const dim3 grid(((plan.n_chunks + 7) / 8) * 8 * p.q8_groups, p.n_kv_heads);
  if (p.q8_tiles <= 4)
    hipLaunchKernelGGL((attn_partial_q8_kernel<D, 4>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_partial_q8_kernel<D, 8>), grid, dim3(512), 0, s, p);
}

int describe_attention_q8(const AttnPlan& plan, int head_dim, int n_kv_heads, int combine_blocks, char* buf,
                          size_t len) {
  int groups, tiles;
  q8_groups(plan, groups, tiles);
  const int roww = tiles <= 4 ? 4 : 8;
  return snprintf(buf, len,
                  "attn_partial_q8_kernel<%d, %d> grid (%d, %d) block %d, %d-token chunks, %d row group(s) of %d "
                  "tiles; attn_combine_kernel<%d> grid %d block 256",
                  head_dim, roww, ((plan.n_chunks + 7) / 8) * 8 * groups, n_kv_heads, 64 * roww, plan.chunk, groups,
                  tiles, head_dim, combine_blocks);
}

hipError_t launch_attention_q8(const AttnPlan& plan, int head_dim, const AttnParams& p,
                               const CombineParams& c, const TreeArgs& t, hipStream_t s) {
  if (plan.n_chunks > 0) {
    if (head_dim == 128)
      launch_q8_d<128>(plan, p, s);
    else
      launch_q8_d<64>(plan, p, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_combine(head_dim, c, t, s);
}

// ------------------------------------------------------------ quantiser
// One thread per block of 32 values: amax, d = fp16(amax / 127) (fp32
// division), codes rint(x / d) (fp32 division, ties to even) clamped to
// [-127, 127]; a block of zeros gets d = 0 and codes 0.  K blocks run along
// the head dim of a token, V blocks along the tokens of a dim.
__device__ __forceinline__ void quantize_block32(const uint16_t* src, int8_t* codes, uint16_t* scale) {
  float x[32];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 w = ld16(src + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = bf16_bits_to_f32(e & 1 ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
      x[c * 8 + e] = v;
      amax = fmaxf(amax, fabsf(v));
    }
  }
  const f16 d16 = (f16)(amax / 127.0f);
  const float dw = (float)d16;
  uint32_t packed[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float cf = dw > 0.f ? rintf(x[q * 4 + e] / dw) : 0.f;
      cf = fminf(fmaxf(cf, -127.f), 127.f);
      w |= ((uint32_t)(int)cf & 0xFFu) << (8 * e);
    }
    packed[q] = w;
  }
  st16(codes, u32x4{packed[0], packed[1], packed[2], packed[3]});
  st16(codes + 16, u32x4{packed[4], packed[5], packed[6], packed[7]});
  *scale = __builtin_bit_cast(uint16_t, d16);
}

__global__ __launch_bounds__(256) void quantize_q8_kernel(const uint16_t* kc, const uint16_t* vc, int hkv, int cap,
                                                          int d, int8_t* k_codes, uint16_t* k_scales,
                                                          int8_t* v_codes, uint16_t* v_scales) {
  const int64_t nk = (int64_t)hkv * cap * (d / 32);  // K blocks: (g, t, b)
  const int64_t nv = (int64_t)hkv * d * (cap / 32);  // V blocks: (g, j, tb)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nk) {
    quantize_block32(kc + i * 32, k_codes + i * 32, k_scales + i);
  } else if (i < nk + nv) {
    const int64_t v = i - nk;
    quantize_block32(vc + v * 32, v_codes + v * 32, v_scales + v);
  }
}

hipError_t launch_quantize_q8(const uint16_t* kc, const uint16_t* vc, int hkv, int cap, int d, int8_t* k_codes,
                              uint16_t* k_scales, int8_t* v_codes, uint16_t* v_scales, hipStream_t s) {
  const int64_t n = (int64_t)hkv * cap * (d / 32) + (int64_t)hkv * d * (cap / 32);
  hipLaunchKernelGGL(quantize_q8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kc, vc, hkv, cap, d,
                     k_codes, k_scales, v_codes, v_scales);
  return hipGetLastError();
}

}  // namespace lucev
