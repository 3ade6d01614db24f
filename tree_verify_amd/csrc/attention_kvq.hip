// Tree attention over a quantised KV prefix (int8 or 4-bit codes), and the
// quantisers that write one.
//
// The KV cache is held as int8 codes or 4-bit nibbles with one fp16 scale per
// 32 values, the q8_0 and Q4_0 cache types the pages run beside F16 ("Lucebox
// Hub", sections "Paged attention + continuous batching" and "설치·사용법";
// KV size is the VRAM limit of section "배경: 어떤 문제를 푸는가", item 3).
// Keys are blocked along the head dim of each token, values along the tokens
// of each dim (the cache keeps V dim-major), so 16 consecutive codes a lane
// loads share one scale.  A value is d * code (int8, code in [-127, 127]) or
// d * (q - 8) (4-bit, nibble q in [0, 15]).  Nibbles are packed 8 to a
// dword, value e of the 8 at bit 4 (e / 2) + 16 (e % 2), so that placing
// them under an fp16 exponent with one v_bfi_b32 per pair yields them in
// order.
//
// The partial kernel follows the bf16 one (blocks over prefix chunk and KV
// head, 64-token tiles in a two-buffer LDS ring, S^T = K Q^T with the softmax
// axis inside each lane, lazy rescale, P fed to O^T = V^T P^T from
// registers), with these differences:
//   * tiles go through registers, two tiles ahead: a lane loads 16 codes and
//     their scale, turns the codes into exact fp16 values (an int8 byte XOR
//     0x80 placed under the exponent of 1024 with v_perm_b32, minus 1152; a
//     nibble under the exponent of 1024 or 64 with v_bfi_b32, minus 1032 or
//     72), scales them with one packed fp16 multiply -- the value rounded
//     once to fp16, within 2^-11 of itself, finer than either format's step
//     -- and stores them into the bf16 kernel's swizzled LDS layouts;
//   * every MFMA is f16 and single: K' q (q -- bf16, or the verify step's
//     fp32 -- as nearest fp16) and V' P (P as nearest fp16), accumulated
//     directly; the quantised cache's own rounding dwarfs these, so no hi/lo
//     halves are carried;
//   * no split query tile: query tiles go one per wave up to 12, then two
//     per wave on 8 waves, and past 16 tiles to row groups, one block per
//     (chunk, group); the groups of a chunk sit on one XCD (block ids 8
//     apart) so the later groups' tile reads hit that XCD's L2.
// Values of magnitude above the fp16 range (65504) are outside what the
// fp16 tiles hold.  The combine kernel is the bf16 path's.
#include <stdio.h>

#include "attn_common.h"

namespace lucev {

typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8_t __attribute__((ext_vector_type(8)));

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

// 16 codes (four dwords) times their scale: 16 fp16 values d * code, each
// rounded once, as two 16-byte chunks in order
__device__ __forceinline__ void scaled16(const u32x4& w, uint32_t scale16, u32x4& out0, u32x4& out1) {
  const f16 d = __builtin_bit_cast(f16, (uint16_t)scale16);
  const f16x2 dd = {d, d};
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x2 c = codes4_f16(w[q]);
    // An empty asm makes the two converted pairs opaque before the multiply:
    // without it this compiler keeps only the first pair's v_perm_b32 and
    // stores its product for both pairs (a miscompile seen in the ISA and in
    // wrong attention outputs).  It emits no instruction.
    uint32_t c0 = c[0], c1 = c[1];
    asm("" : "+v"(c0), "+v"(c1));
    o[2 * q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, c0) * dd);
    o[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, c1) * dd);
  }
  out0 = u32x4{o[0], o[1], o[2], o[3]};
  out1 = u32x4{o[4], o[5], o[6], o[7]};
}

// v_bfi_b32: (a & mask) | (b & ~mask)
__device__ __forceinline__ uint32_t bfi_kv(uint32_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(b));
  return r;
}

// 8 nibbles of one dword (value e at bit 4 (e / 2) + 16 (e % 2)) times their
// scale: fp16 d * (q - 8) in order, as four dwords.  A nibble in the low
// mantissa bits of 1024 reads 1024 + q, one four bits higher under 64 reads
// 64 + q; subtracting 1032 or 72 leaves q - 8 exactly.
__device__ __forceinline__ void nibbles8_scaled(uint32_t w, f16x2 dd, uint32_t* o) {
  const uint32_t w8 = w >> 8;
  const f16x2 b1032 = {(f16)1032.0f, (f16)1032.0f};
  const f16x2 b72 = {(f16)72.0f, (f16)72.0f};
  o[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, bfi_kv(0x000F000Fu, w, 0x64006400u)) - b1032) * dd);
  o[1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, bfi_kv(0x00F000F0u, w, 0x54005400u)) - b72) * dd);
  o[2] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, bfi_kv(0x000F000Fu, w8, 0x64006400u)) - b1032) * dd);
  o[3] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, bfi_kv(0x00F000F0u, w8, 0x54005400u)) - b72) * dd);
}

// 16 codes of a lane (int8: four dwords; 4-bit: the first two) times their
// scale, as two 16-byte chunks in order
template <int BITS>
__device__ __forceinline__ void scaled16_kv(const u32x4& w, uint32_t scale16, u32x4& out0, u32x4& out1) {
  if constexpr (BITS == 8) {
    scaled16(w, scale16, out0, out1);
  } else {
    const f16 d = __builtin_bit_cast(f16, (uint16_t)scale16);
    const f16x2 dd = {d, d};
    uint32_t a[4], b[4];
    nibbles8_scaled(w[0], dd, a);
    nibbles8_scaled(w[1], dd, b);
    out0 = u32x4{a[0], a[1], a[2], a[3]};
    out1 = u32x4{b[0], b[1], b[2], b[3]};
  }
}

// Two fp32 values as fp16 (nearest), packed
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(f16)a, (f16)b});
}

// LDS tile of the int8 path: K' [64 keys][D] and V'^T [D][64], fp16, in the
// bf16 kernel's swizzled layouts.
template <int D>
struct Q8Tile {
  static constexpr int KBYTES = KT * D * 2;
  static constexpr int BYTES = 2 * KBYTES;
  // wave-loads per tile, 16 codes a lane: K (D / 16 lanes per key), V (4
  // lanes per dim, 16 tokens each)
  static constexpr int NK = KT * D / 1024;
  static constexpr int NV = D * KT / 1024;
  static constexpr int SLOTS = NK + NV;
};

struct Q8Slot {
  u32x4 codes;
  uint32_t scale;  // fp16 bits
};

template <int D, int QPW, int ROWW, int BITS>
__global__ __launch_bounds__(ROWW * 64) void attn_partial_q8_kernel(AttnParams p) {
  static_assert(BITS == 8 || BITS == 4, "int8 or 4-bit codes");
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
  const int grp = (x >> 3) % p.row_groups;
  const int chunk = (x / (8 * p.row_groups)) * 8 + (x & 7);
  if (chunk >= p.n_chunks) return;
  const int g = blockIdx.y;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int RT = (p.rows + 15) / 16;
  const int k_begin = chunk * p.chunk;
  const int k_end = min(p.prefix_len, k_begin + p.chunk);
  const int n_tiles = (k_end - k_begin + KT - 1) / KT;
  // this wave's query tiles: group tiles wave, wave + ROWW, ...
  auto tile_of = [&](int i) __attribute__((always_inline)) { return grp * p.group_tiles + wave + ROWW * i; };
  auto has_tile = [&](int i) __attribute__((always_inline)) { return wave + ROWW * i < p.group_tiles && tile_of(i) < RT; };

  // code bytes of this KV head (BITS / 8 bytes per code)
  const uint8_t* kcode = reinterpret_cast<const uint8_t*>(p.kc8) + (int64_t)g * p.cap * D * BITS / 8;
  const uint8_t* vcode = reinterpret_cast<const uint8_t*>(p.vc8) + (int64_t)g * D * p.cap * BITS / 8;
  const uint16_t* kscale = p.ks16 + (int64_t)g * p.cap * NBLK;
  const uint16_t* vscale = p.vs16 + (int64_t)g * D * (p.cap / 32);

  // One wave-load slot j of tile t: 16 codes of this lane and their scale
  // (zeros past the prefix).  Slots [0, NK) hold K, [NK, NK + NV) V.
  auto load_slot = [&](int t, int j) __attribute__((always_inline)) -> Q8Slot {
    const int k0 = k_begin + t * KT;
    Q8Slot r{u32x4{0u, 0u, 0u, 0u}, 0u};
    if (j < T::NK) {
      const int key = j * (1024 / D) + lane / (D / 16);
      const int c16 = lane % (D / 16);  // codes 16 c16 .. + 15 of the key: scale block c16 / 2
      if (k0 + key < k_end) {
        if constexpr (BITS == 8) {
          r.codes = ld16(kcode + (int64_t)(k0 + key) * D + c16 * 16);
        } else {
          const u32x2 w = *reinterpret_cast<const u32x2*>(kcode + (int64_t)(k0 + key) * (D / 2) + c16 * 8);
          r.codes = u32x4{w[0], w[1], 0u, 0u};
        }
        r.scale = kscale[(int64_t)(k0 + key) * NBLK + (c16 >> 1)];
      }
    } else {
      const int jj = j - T::NK;
      const int dim = jj * 16 + lane / 4, part = lane % 4;  // tokens k0 + 16 part .. + 15
      if (k0 + part * 16 < k_end) {
        if constexpr (BITS == 8) {
          r.codes = ld16(vcode + (int64_t)dim * p.cap + k0 + part * 16);
        } else {
          const u32x2 w = *reinterpret_cast<const u32x2*>(vcode + (int64_t)dim * (p.cap / 2) + (k0 + part * 16) / 2);
          r.codes = u32x4{w[0], w[1], 0u, 0u};
        }
        r.scale = vscale[(int64_t)dim * (p.cap / 32) + ((k0 + part * 16) >> 5)];
      }
    }
    return r;
  };
  // Slot j's registers into LDS buffer b, scaled to fp16 in the swizzled
  // layouts (tokens past the prefix read as zero).
  auto store_slot = [&](int t, int j, const Q8Slot& v, int b) __attribute__((always_inline)) {
    uint8_t* base = lds + b * T::BYTES;
    const int k0 = k_begin + t * KT;
    if (j < T::NK) {
      const int key = j * (1024 / D) + lane / (D / 16);
      const int c16 = lane % (D / 16);
      const int sw = ((key & 3) | (((key >> 3) & 3) << 2)) & (KCPR - 1);
      u32x4 c0, c1;
      scaled16_kv<BITS>(v.codes, v.scale, c0, c1);
      uint8_t* row = base + key * D * 2;
      *reinterpret_cast<u32x4*>(row + (((2 * c16) ^ sw) * 16)) = c0;
      *reinterpret_cast<u32x4*>(row + (((2 * c16 + 1) ^ sw) * 16)) = c1;
    } else {
      const int jj = j - T::NK;
      const int dim = jj * 16 + lane / 4, part = lane % 4;
      const int swz = (dim >> 1) & 7;
      u32x4 w = v.codes;
      // tokens past the prefix inside this 16-token run read as value 0
      // (int8 code 0; nibble 8)
      const int valid = k_end - (k0 + part * 16);
      if (valid < 16) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (e < valid) continue;
          if constexpr (BITS == 8) {
            w[e >> 2] &= ~(0xFFu << (8 * (e & 3)));
          } else {
            const int b = 4 * ((e & 7) >> 1) + 16 * (e & 1);
            w[e >> 3] = (w[e >> 3] & ~(0xFu << b)) | (8u << b);
          }
        }
      }
      u32x4 c0, c1;
      scaled16_kv<BITS>(w, v.scale, c0, c1);
      uint8_t* row = base + T::KBYTES + dim * KT * 2;
      *reinterpret_cast<u32x4*>(row + (((2 * part) ^ swz) * 16)) = c0;
      *reinterpret_cast<u32x4*>(row + (((2 * part + 1) ^ swz) * 16)) = c1;
    }
  };

  // this wave's query tiles; Q^T as fp16, scaled to log2 units
  f16x8_t qf[QPW][D / 32];
  f32x4 O[QPW][D / 16];
  float m[QPW], l[QPW];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int row = tile_of(i) * 16 + lr;
    const bool ok = has_tile(i) && row < p.rows;
    int node = 0, head = 0;
    if (ok) {
      node = row / G;
      head = g * G + (row - node * G);
    }
    const int64_t qoff = ((int64_t)node * p.n_q_heads + head) * D + lq * 8;
    // q as bf16 (p.q), or fp32 (p.q32: the verify step's), to the nearest fp16
    float qv[D / 32][8];
    if (p.q32) {
      u32x4 raw[D / 32][2];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        raw[kk][0] = ld16(p.q32 + qoff + kk * 32);
        raw[kk][1] = ld16(p.q32 + qoff + kk * 32 + 4);
      }
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[kk][e] = __uint_as_float(raw[kk][e >> 2][e & 3]);
    } else {
      u32x4 raw[D / 32];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) raw[kk] = ld16(p.q + qoff + kk * 32);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          qv[kk][e] = bf16_bits_to_f32(e & 1 ? (raw[kk][e >> 1] >> 16) : (raw[kk][e >> 1] & 0xFFFFu));
    }
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint32_t hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = ok ? qv[kk][2 * e] * p.scale_log2 : 0.f;
        const float x1 = ok ? qv[kk][2 * e + 1] * p.scale_log2 : 0.f;
        hv[e] = pack_f16(x0, x1);
      }
      qf[i][kk] = __builtin_bit_cast(f16x8_t, u32x4{hv[0], hv[1], hv[2], hv[3]});
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[i] = -INFINITY;
    l[i] = 0.f;
  }

  // One 32-key half of a tile for every query tile of this wave: the half's
  // K' fragments (one 16-key group at a time) against each tile's q, the
  // softmax of each tile, then V'^T P^T one 16-dim tile at a time.
  auto row_half = [&](const uint8_t* buf, int ks, int k0, bool masked) __attribute__((always_inline)) {
    const f16* K = reinterpret_cast<const f16*>(buf);
    const f16* V = reinterpret_cast<const f16*>(buf + T::KBYTES);
    f32x4 sc[QPW][2];
    float bias[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) bias[i] = m[i] == -INFINITY ? 0.f : m[i];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = ks * 32 + (lr >> 2) * 8 + h * 4 + (lr & 3);  // its swizzle is lr
      f16x8_t kf[D / 32];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        kf[kk] = *reinterpret_cast<const f16x8_t*>(K + key * D + (((kk * 4 + lq) ^ lr) & (KCPR - 1)) * 8);
#pragma unroll
      for (int i = 0; i < QPW; ++i) {
        if (!has_tile(i)) continue;
        f32x4 a4 = f32x4{-bias[i], -bias[i], -bias[i], -bias[i]};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kk], qf[i][kk], a4, 0, 0, 0);
        sc[i][h] = a4;
      }
    }
    f16x8_t pb[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      if (!has_tile(i)) continue;
      float s[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = sc[i][e >> 2][e & 3];
      if (masked) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + ks * 32 + lq * 8 + e >= k_end) s[e] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      mx = rows_max(mx);
      // lazy rescale: only when the running max moves up by more than 2^8
      if (__builtin_amdgcn_ballot_w64(bias[i] + mx > m[i] + 8.f) != 0) {
        const float m_new = fmaxf(m[i], bias[i] + mx);
        const float alpha = __builtin_amdgcn_exp2f(m[i] - m_new);
        const float moved = m_new - bias[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] -= moved;
        l[i] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) O[i][dt] *= alpha;
        m[i] = m_new;
      }
      float pv[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(s[e]);
        psum += pv[e];
      }
      l[i] += psum;
      pb[i] = __builtin_bit_cast(
          f16x8_t, u32x4{pack_f16(pv[0], pv[1]), pack_f16(pv[2], pv[3]), pack_f16(pv[4], pv[5]), pack_f16(pv[6], pv[7])});
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      // V'^T row dt*16 + lr, tokens ks*32 + lq*8 .. + 7
      const f16x8_t vf =
          *reinterpret_cast<const f16x8_t*>(V + (dt * 16 + lr) * KT + (((ks * 4 + lq) ^ ((lr >> 1) & 7)) * 8));
#pragma unroll
      for (int i = 0; i < QPW; ++i) {
        if (!has_tile(i)) continue;
        O[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[i], O[i][dt], 0, 0, 0);
      }
    }
  };

  // Tiles go through registers two ahead: at step t the loads of tile t + 2
  // are issued into the register set tile t used, tile t is computed, and
  // tile t + 1 (loaded during step t - 1) is scaled into the LDS buffer tile
  // t - 1 used, which every wave has finished (the barrier at the top of
  // step t).
  if (n_tiles > 0) {
    Q8Slot regs[2][LPW];
    auto load_tile = [&](int t, Q8Slot (&r)[LPW]) {
#pragma unroll
      for (int k = 0; k < LPW; ++k) {
        const int j = wave + k * WAVES;
        if (j < T::SLOTS) r[k] = load_slot(t, j);
      }
    };
    auto store_tile = [&](int t, const Q8Slot (&r)[LPW], int b) {
#pragma unroll
      for (int k = 0; k < LPW; ++k) {
        const int j = wave + k * WAVES;
        if (j < T::SLOTS) store_slot(t, j, r[k], b);
      }
    };
    const bool any = has_tile(0);
    load_tile(0, regs[0]);
    if (n_tiles > 1) load_tile(1, regs[1]);
    store_tile(0, regs[0], 0);
    auto step = [&](int t, Q8Slot (&mine)[LPW], Q8Slot (&next)[LPW]) {
      lds_barrier();  // tile t is in buffer t & 1; every wave is done with tile t - 1
      if (t + 2 < n_tiles) load_tile(t + 2, mine);
      const int k0 = k_begin + t * KT;
      if (any) {
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

#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    if (!has_tile(i)) continue;
    const float lt = rows_sum(l[i]);
    const int row = tile_of(i) * 16 + lr;
    if (row < p.rows) {
      const float inv = 1.0f / lt;
      const int64_t prow = ((int64_t)chunk * p.n_kv_heads + g) * p.rows + row;
      float* dst = p.o_part + prow * D + lq * 4;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(dst + dt * 16) = O[i][dt] * inv;
      if (lq == 0) {
        p.ml_part[prow * 2] = m[i];
        p.ml_part[prow * 2 + 1] = lt;
      }
    }
  }
}

// Layouts: one query tile per wave up to 12 tiles (4, 8 or 12 waves), then
// two tiles per wave on 8 waves, past 16 tiles in row groups of 16.  Measured
// per layer: 9 tiles (the 27B shape, 22 nodes) 57-59 us on 12 one-tile waves
// against 67 us on 8 two-tile waves; 15 tiles (40 nodes) 229-232 us on 8
// two-tile waves against 232-233 us on 16 one-tile waves.
struct Q8Layout {
  int qpw, roww, groups, tiles;
};
static Q8Layout q8_layout(const AttnPlan& plan) {
  const int rt = (plan.rows + 15) / 16;
  if (rt <= 4) return {1, 4, 1, rt};
  if (rt <= 8) return {1, 8, 1, rt};
  if (rt <= 12) return {1, 12, 1, rt};
  const int groups = (rt + 15) / 16;
  return {2, 8, groups, (rt + groups - 1) / groups};
}

template <int D, int BITS>
static void launch_q8_d(const AttnPlan& plan, AttnParams p, hipStream_t s) {
  const Q8Layout v = q8_layout(plan);
  p.row_groups = v.groups;
  p.group_tiles = v.tiles;
  const dim3 grid(((plan.n_chunks + 7) / 8) * 8 * v.groups, p.n_kv_heads);
  if (v.roww == 4)
    hipLaunchKernelGGL((attn_partial_q8_kernel<D, 1, 4, BITS>), grid, dim3(256), 0, s, p);
  else if (v.qpw == 2)
    hipLaunchKernelGGL((attn_partial_q8_kernel<D, 2, 8, BITS>), grid, dim3(512), 0, s, p);
  else if (v.roww == 8)
    hipLaunchKernelGGL((attn_partial_q8_kernel<D, 1, 8, BITS>), grid, dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((attn_partial_q8_kernel<D, 1, 12, BITS>), grid, dim3(768), 0, s, p);
}

int describe_attention_q8(const AttnPlan& plan, int head_dim, int n_kv_heads, int combine_blocks, int bits,
                          char* buf, size_t len) {
  const Q8Layout v = q8_layout(plan);
  return snprintf(buf, len,
                  "attn_partial_q8_kernel<%d, %d, %d, %d> grid (%d, %d) block %d, %d-token chunks, %d row group(s) of "
                  "%d tiles; attn_combine_kernel<%d> grid %d block 256",
                  head_dim, v.qpw, v.roww, bits, ((plan.n_chunks + 7) / 8) * 8 * v.groups, n_kv_heads, 64 * v.roww,
                  plan.chunk, v.groups, v.tiles, head_dim, combine_blocks);
}

hipError_t launch_attention_q8(const AttnPlan& plan, int head_dim, int bits, const AttnParams& p,
                               const CombineParams& c, const TreeArgs& t, hipStream_t s) {
  if (plan.n_chunks > 0) {
    if (head_dim == 128) {
      if (bits == 8)
        launch_q8_d<128, 8>(plan, p, s);
      else
        launch_q8_d<128, 4>(plan, p, s);
    } else {
      if (bits == 8)
        launch_q8_d<64, 8>(plan, p, s);
      else
        launch_q8_d<64, 4>(plan, p, s);
    }
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

// The 4-bit form: d = fp16(amax / 7) (fp32 division), codes rint(x / d)
// clamped to [-7, 7] (fp32, ties to even), stored as nibbles code + 8 in the
// order the attention decodes (value e of each 8 at bit 4 (e / 2) +
// 16 (e % 2)); a block of zeros gets d = 0 and nibbles 8.
__device__ __forceinline__ void quantize_block32_q4(const uint16_t* src, uint8_t* nib, uint16_t* scale) {
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
  const f16 d16 = (f16)(amax / 7.0f);
  const float dw = (float)d16;
  uint32_t packed[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float cf = dw > 0.f ? rintf(x[q * 8 + e] / dw) : 0.f;
      cf = fminf(fmaxf(cf, -7.f), 7.f);
      w |= ((uint32_t)((int)cf + 8) & 0xFu) << (4 * (e >> 1) + 16 * (e & 1));
    }
    packed[q] = w;
  }
  st16(nib, u32x4{packed[0], packed[1], packed[2], packed[3]});
  *scale = __builtin_bit_cast(uint16_t, d16);
}

__global__ __launch_bounds__(256) void quantize_q4_kernel(const uint16_t* kc, const uint16_t* vc, int hkv, int cap,
                                                          int d, uint8_t* k_nib, uint16_t* k_scales, uint8_t* v_nib,
                                                          uint16_t* v_scales) {
  const int64_t nk = (int64_t)hkv * cap * (d / 32);  // K blocks: (g, t, b)
  const int64_t nv = (int64_t)hkv * d * (cap / 32);  // V blocks: (g, j, tb)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nk) {
    quantize_block32_q4(kc + i * 32, k_nib + i * 16, k_scales + i);
  } else if (i < nk + nv) {
    const int64_t v = i - nk;
    quantize_block32_q4(vc + v * 32, v_nib + v * 16, v_scales + v);
  }
}

hipError_t launch_quantize_q4(const uint16_t* kc, const uint16_t* vc, int hkv, int cap, int d, uint8_t* k_nib,
                              uint16_t* k_scales, uint8_t* v_nib, uint16_t* v_scales, hipStream_t s) {
  const int64_t n = (int64_t)hkv * cap * (d / 32) + (int64_t)hkv * d * (cap / 32);
  hipLaunchKernelGGL(quantize_q4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kc, vc, hkv, cap, d,
                     k_nib, k_scales, v_nib, v_scales);
  return hipGetLastError();
}

hipError_t launch_quantize_q8(const uint16_t* kc, const uint16_t* vc, int hkv, int cap, int d, int8_t* k_codes,
                              uint16_t* k_scales, int8_t* v_codes, uint16_t* v_scales, hipStream_t s) {
  const int64_t n = (int64_t)hkv * cap * (d / 32) + (int64_t)hkv * d * (cap / 32);
  hipLaunchKernelGGL(quantize_q8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kc, vc, hkv, cap, d,
                     k_codes, k_scales, v_codes, v_scales);
  return hipGetLastError();
}

}  // namespace lucev
