// int4 block-32 skinny GEMM: Y[node, f] = sum_k X[node, k] * W[f, k] with
// W[f, k] = d[f, k/32] * (q[f, k] - 8), for up to 64 tree nodes.
//
// The target reads every weight once per forward and checks all drafted
// tokens in that one pass ("Lucebox Hub", section "배경: 어떤 문제를 푸는가",
// item 1; section "Speculative decoding 계층"), so this kernel streams the
// packed weights exactly once and reuses each dequantised weight for every
// tree node.  With 8..64 nodes that reuse is a dense contraction, so the MAC
// work goes to MFMA (v_mfma_f32_16x16x32_f16); the codes are expanded in
// registers (exponent-bias trick: exact q - 8 as fp16, then times the
// block's fp16 scale), and the weights never touch LDS.
//
// Packed layout (private to this library, written by lucev_q4_pack*):
//   nibble region, per 16-row tile t and 128-column group c, 1024 bytes:
//     lane l (0..63) owns 16 bytes at l*16: dword j (block j of the group)
//     holds the 8 codes of row 16t + l%16, columns 128c + 32j + 8(l/16) + e,
//     code e at bit 4*(e/2) + 16*(e%2) (so (w & 0x000F000F) etc. yields fp16
//     pairs in column order).
//   scale region (after n_out*k_in/2 bytes), per (t, c), 128 bytes:
//     fp16 scale of row 16t + r, block j at element r*4 + j.
// A wave streams a tile-group with one coalesced 16-byte load per lane.
#include "internal.h"

namespace lucev {

// ------------------------------------------------------------ packing

__host__ __device__ inline int64_t packed_row_to_logical(int64_t p, int kind, int head_dim,
                                                         int64_t n_out) {
  if (kind == W_QKV) {
    // per head, tile i holds dims [8i, 8i+8) and [d/2 + 8i, d/2 + 8i + 8):
    // each rotate-half RoPE pair (j, j + d/2) sits in one tile, 8 rows apart
    int64_t head = p / head_dim;
    int r = (int)(p % head_dim);
    int i = r / 16, loc = r % 16;
    int j = loc < 8 ? 8 * i + loc : head_dim / 2 + 8 * i + (loc - 8);
    return head * head_dim + j;
  }
  if (kind == W_GU) {
    // packed tile 2i = gate rows [16i, 16i+16), tile 2i+1 = up rows of the same i
    int64_t F = n_out / 2;
    int64_t t = p / 16;
    int r = (int)(p % 16);
    return (t & 1) ? F + (t / 2) * 16 + r : (t / 2) * 16 + r;
  }
  return p;
}

__host__ __device__ inline void pack_row_group(const uint8_t* q, const uint16_t* d, int64_t n_out,
                                               int64_t k_in, int kind, int head_dim, int64_t p,
                                               int c, uint8_t* dst) {
  const int64_t kgroups = k_in / 128;
  const int64_t L = packed_row_to_logical(p, kind, head_dim, n_out);
  const uint8_t* src = q + L * k_in + (int64_t)c * 128;
  const int64_t t = p / 16;
  const int lr = (int)(p % 16);
  uint8_t* nib = dst + (t * kgroups + c) * 1024;
  for (int q4 = 0; q4 < 4; ++q4) {
    uint32_t out[4];
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0;
      for (int e = 0; e < 8; ++e) {
        uint32_t code = src[j * 32 + q4 * 8 + e] & 15u;
        w |= code << ((e & 1) * 16 + (e >> 1) * 4);
      }
      out[j] = w;
    }
    uint32_t* o = reinterpret_cast<uint32_t*>(nib + (q4 * 16 + lr) * 16);
    o[0] = out[0];
    o[1] = out[1];
    o[2] = out[2];
    o[3] = out[3];
  }
  uint16_t* sc = reinterpret_cast<uint16_t*>(dst + n_out * k_in / 2) + (t * kgroups + c) * 64 + lr * 4;
  for (int j = 0; j < 4; ++j) sc[j] = d[L * (k_in / 32) + c * 4 + j];
}

void pack_q4_host(const uint8_t* q, const uint16_t* d, int64_t n_out, int64_t k_in, int kind,
                  int head_dim, void* dst) {
  const int64_t kgroups = k_in / 128;
  for (int64_t p = 0; p < n_out; ++p)
    for (int c = 0; c < kgroups; ++c)
      pack_row_group(q, d, n_out, k_in, kind, head_dim, p, c, static_cast<uint8_t*>(dst));
}

__global__ __launch_bounds__(256) void pack_q4_kernel(const uint8_t* q, const uint16_t* d,
                                                      int64_t n_out, int64_t k_in, int kind,
                                                      int head_dim, uint8_t* dst) {
  const int64_t kgroups = k_in / 128;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_out * kgroups) return;
  pack_row_group(q, d, n_out, k_in, kind, head_dim, idx / kgroups, (int)(idx % kgroups), dst);
}

hipError_t launch_pack_q4(const uint8_t* q, const uint16_t* d, int64_t n_out, int64_t k_in,
                          int kind, int head_dim, void* dst, hipStream_t s) {
  const int64_t work = n_out * (k_in / 128);
  const int64_t blocks = (work + 255) / 256;
  hipLaunchKernelGGL(pack_q4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, d, n_out, k_in,
                     kind, head_dim, static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

// ------------------------------------------------------------ dequant

// v_bfi_b32: (a & mask) | (b & ~mask), one VALU op for a masked merge
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(b));
  return r;
}

// 8 codes of one dword -> the 8 exact values (q - 8) as fp16, column order.
// A code placed in the low mantissa bits of 0x6400 (1024) reads 1024 + q; one
// placed four bits higher under 0x5400 (64) reads 64 + q.
__device__ __forceinline__ f16x8 codes8(uint32_t w) {
  const uint32_t w8 = w >> 8;
  const uint32_t v0 = bfi(0x000F000Fu, w, 0x64006400u);   // 1024 + q (cols 0, 1)
  const uint32_t v1 = bfi(0x00F000F0u, w, 0x54005400u);   //   64 + q (cols 2, 3)
  const uint32_t v2 = bfi(0x000F000Fu, w8, 0x64006400u);  // 1024 + q (cols 4, 5)
  const uint32_t v3 = bfi(0x00F000F0u, w8, 0x54005400u);  //   64 + q (cols 6, 7)
  const f16x2 b1032 = {(f16)1032.0f, (f16)1032.0f};
  const f16x2 b72 = {(f16)72.0f, (f16)72.0f};
  const f16x2 h0 = __builtin_bit_cast(f16x2, v0) - b1032;
  const f16x2 h1 = __builtin_bit_cast(f16x2, v1) - b72;
  const f16x2 h2 = __builtin_bit_cast(f16x2, v2) - b1032;
  const f16x2 h3 = __builtin_bit_cast(f16x2, v3) - b72;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// 8 codes of one dword times the block scale: fp16 d * (q - 8), column order
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 dd) {
  const f16x8 c = codes8(w);
  const f16x2 a = f16x2{c[0], c[1]} * dd;
  const f16x2 b = f16x2{c[2], c[3]} * dd;
  const f16x2 cc = f16x2{c[4], c[5]} * dd;
  const f16x2 d = f16x2{c[6], c[7]} * dd;
  return f16x8{a[0], a[1], b[0], b[1], cc[0], cc[1], d[0], d[1]};
}

// The same product split exactly: hi = fp16(d * (q - 8)) and lo = d * (q - 8)
// - hi.  d has 11 significant bits and q - 8 at most 3, so the residual has at
// most 3 bits, is a multiple of ulp(d) >= 2^-19 and fits fp16; the fused
// multiply-add forms it without rounding.
__device__ __forceinline__ void dequant8_split(uint32_t w, f16x2 dd, f16x8& hi, f16x8& lo) {
  const f16x8 c = codes8(w);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 ci = f16x2{c[2 * i], c[2 * i + 1]};
    const f16x2 h = ci * dd;
    const f16x2 l = __builtin_elementwise_fma(ci, dd, -h);
    hi[2 * i] = h[0];
    hi[2 * i + 1] = h[1];
    lo[2 * i] = l[0];
    lo[2 * i + 1] = l[1];
  }
}

// the block-j scale of this lane's row, splatted to both fp16 halves
__device__ __forceinline__ f16x2 scale_pair(u32x2 s, int j) {
  const uint32_t word = (j < 2) ? s[0] : s[1];
  const uint32_t h = (j & 1) ? (word >> 16) : (word & 0xFFFFu);
  return __builtin_bit_cast(f16x2, h | (h << 16));
}

__device__ __forceinline__ void rope_pair_angle(int pos, int jj, const double* inv_freq, float& cs,
                                                float& sn) {
  // angle in fp64, reduced to [-pi, pi] before the fp32 sin / cos
  const double th = (double)pos * inv_freq[jj];
  const double two_pi = 6.283185307179586476925286766559;
  const double r = th - two_pi * rint(th / two_pi);
  sincosf((float)r, &sn, &cs);
}

__device__ __forceinline__ void merge_top2(float& v1, int& i1, float& v2, float b1, int bi, float b2) {
  if (b1 > v1 || (b1 == v1 && bi < i1)) {
    v2 = fmaxf(v1, b2);
    v1 = b1;
    i1 = bi;
  } else {
    v2 = fmaxf(v2, b1);
  }
}

__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Block barrier that orders LDS only: outstanding global loads (the weight
// prefetch) stay in flight across it, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int UG, int FT>
struct WRegs {
  u32x4 w[UG][FT];  // per column group and tile: 4 blocks x 8 codes of this lane's row
  u32x2 s[UG][FT];  // the row's 4 block scales
};

template <int UG>
constexpr int gemm_xld() { return UG * 128 + 8; }  // staged activation row (fp16), padded

template <int WAVES, int FT, int NTX, int UG, int EPI, bool EXACT>
__global__ __launch_bounds__(WAVES * 64) void gemm_q4_kernel(GemmParams p, EpiArgs e) {
  constexpr int NTH = WAVES * 64;
  constexpr int PT = WAVES * FT;   // tiles per panel
  constexpr int TILE_F = PT * 16;
  constexpr int XR = NTX * 16;     // staged hi/lo rows
  constexpr int XLD = gemm_xld<UG>();
  constexpr int XCPR = UG * 16;    // 16-byte chunks per staged row
  constexpr int XCH = (XR * XCPR + NTH - 1) / NTH;  // staging chunks per thread
  constexpr int TILE_N = NTX * 8;  // nodes
  constexpr int TILE = TILE_F * TILE_N;
  __shared__ __attribute__((aligned(16))) uint16_t sx[2 * XR * XLD];
  __shared__ float tile[TILE_F][TILE_N + 1];
  __shared__ float best1[TILE_N], best2[TILE_N];
  __shared__ int besti[TILE_N];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int b = blockIdx.x;
  const int B = p.blocks;
  const int64_t U = p.units;
  const int G = p.kgroups;   // 128-column groups
  const int GU = G / UG;     // units per panel
  const int nn = p.n_nodes;
  const int64_t K = p.k_in;
  const int64_t u_begin = range_start(b, U, B);
  const int64_t u_end = range_start(b + 1, U, B);

  if constexpr (EPI == EPI_LOGITS) {
    if (tid < TILE_N) {
      best1[tid] = -INFINITY;
      best2[tid] = -INFINITY;
      besti[tid] = 0x7fffffff;
    }
  }

  // A unit as (panel, unit within the panel), advanced without divisions.
  struct Cur {
    int pnl, c;
  };
  auto cur_of = [&](int64_t u) { return Cur{(int)(u / GU), (int)(u % GU)}; };
  auto advance = [&](Cur& k) {
    if (++k.c == GU) {
      k.c = 0;
      ++k.pnl;
    }
  };
  // the weights are read once: non-temporal loads keep them from evicting
  // the activation rows, which every block re-reads, from L2
  auto wload = [&](Cur k, WRegs<UG, FT>& r) {
#pragma unroll
    for (int g = 0; g < UG; ++g)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        int t = k.pnl * PT + wave * FT + ft;
        t = t < p.n_tiles ? t : p.n_tiles - 1;  // ragged last panel: re-read a valid tile
        const int64_t tg = (int64_t)t * G + k.c * UG + g;
        r.w[g][ft] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.wq + tg * 1024 + lane * 16));
        r.s[g][ft] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p.wsc + tg * 64 + lr * 4));
      }
  };
  // activation slice of a unit: XR rows x UG * 128 columns, in 16-byte chunks
  // (every lane loads from a valid row and zeroes what lies past the 2n rows,
  // so the load count does not depend on the lane)
  auto xload = [&](Cur k, u32x4 (&xr)[XCH]) {
    const int col0 = k.c * UG * 128;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int id = tid + NTH * i;
      const int row = id / XCPR, part = id % XCPR;
      const bool ok = id < XR * XCPR && row < 2 * nn;
      const u32x4 v = ld16(p.X + (ok ? row : 0) * K + col0 + part * 8);
      xr[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto xstore = [&](int buf, const u32x4 (&xr)[XCH]) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int id = tid + NTH * i;
      const int row = id / XCPR, part = id % XCPR;
      if (id < XR * XCPR) *reinterpret_cast<u32x4*>(&sx[(buf * XR + row) * XLD + part * 8]) = xr[i];
    }
  };

  f32x4 acc[FT][NTX];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int nt = 0; nt < NTX; ++nt) acc[ft][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, const WRegs<UG, FT>& r) {
    const uint16_t* xs = sx + (buf * XR + lr) * XLD + lq * 8;
#pragma unroll
    for (int g = 0; g < UG; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f16x8 xa[NTX];
#pragma unroll
        for (int nt = 0; nt < NTX; ++nt)
          xa[nt] = *reinterpret_cast<const f16x8*>(xs + nt * 16 * XLD + g * 128 + j * 32);
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          if constexpr (EXACT) {
            // d * (q - 8) split exactly into fp16 hi + lo, both through the MFMA
            f16x8 wh, wl;
            dequant8_split(r.w[g][ft][j], scale_pair(r.s[g][ft], j), wh, wl);
#pragma unroll
            for (int nt = 0; nt < NTX; ++nt) {
              acc[ft][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[nt], wh, acc[ft][nt], 0, 0, 0);
              acc[ft][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[nt], wl, acc[ft][nt], 0, 0, 0);
            }
          } else {
            const f16x8 wb = dequant8(r.w[g][ft][j], scale_pair(r.s[g][ft], j));
#pragma unroll
            for (int nt = 0; nt < NTX; ++nt)
              acc[ft][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[nt], wb, acc[ft][nt], 0, 0, 0);
          }
        }
      }
  };

  // finish panel pnl: hi/lo rows merged into the LDS tile [feature][node],
  // split panels reduced across blocks, then the epilogue
  auto flush = [&](int64_t pnl) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int nt = 0; nt < NTX; ++nt) {
        // D layout: column (feature) = lane % 16, rows 4 * (lane / 16) + i =
        // hi/lo rows of nodes nt * 8 + 2 * (lane / 16) + {0, 1}
        const int fl = (wave * FT + ft) * 16 + lr;
        const int n0 = nt * 8 + 2 * lq;
        tile[fl][n0] = acc[ft][nt][0] + acc[ft][nt][1];
        tile[fl][n0 + 1] = acc[ft][nt][2] + acc[ft][nt][3];
        acc[ft][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    lds_barrier();

    const int64_t first = pnl * GU, last = pnl * GU + GU - 1;
    const int bf = block_of_unit(first, U, B);
    const int bl = block_of_unit(last, U, B);
    if constexpr (EPI == EPI_PARTIAL) {
      // this block's share of the panel, node-major; a later kernel sums
      // the contributors and applies the epilogue (plain stores: that kernel
      // starts after this one has finished)
      float* dst = p.partials + ((int64_t)pnl * p.c_max + (b - bf)) * TILE;
      for (int i = tid; i < TILE; i += NTH) {
        const int n = i / TILE_F, fl = i - n * TILE_F;
        dst[i] = tile[fl][n];
      }
      lds_barrier();  // the LDS tile is reused by the next panel
      return;
    }
    if (bf != bl) {
      constexpr int PER = (TILE + NTH - 1) / NTH;
      const int slot = (u_begin >= first) ? 0 : 1;
      float* part = p.partials + ((int64_t)b * 2 + slot) * TILE;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = tid + k * NTH;
        if (i < TILE) st_coherent(part + i, tile[i / TILE_N][i % TILE_N]);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every wave's stores done
      lds_barrier();
      if (tid == 0) {
        // the partials were written through (agent-scope stores) and every
        // wave waited for them before the barrier, so a relaxed count suffices
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[pnl], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned)(bl - bf);
      }
      lds_barrier();
      if (!s_last) return;
      // sum the contributors in block order, CB at a time with all their
      // loads in flight together
      constexpr int CB = PER <= 12 ? 6 : 3;
      float sum[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) sum[k] = 0.f;
      for (int b0 = bf; b0 <= bl; b0 += CB) {
        float v[CB][PER];
#pragma unroll
        for (int uu = 0; uu < CB; ++uu) {
          const int bb = min(b0 + uu, bl);  // past the last contributor: re-read it, unused
          const int sl = (range_start(bb, U, B) >= first) ? 0 : 1;
          const float* src = p.partials + ((int64_t)bb * 2 + sl) * TILE + tid;
#pragma unroll
          for (int k = 0; k < PER; ++k)
            v[uu][k] = (tid + k * NTH < TILE) ? ld_coherent(src + k * NTH) : 0.f;
        }
#pragma unroll
        for (int uu = 0; uu < CB; ++uu)
          if (b0 + uu <= bl)
#pragma unroll
            for (int k = 0; k < PER; ++k) sum[k] += v[uu][k];
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = tid + k * NTH;
        if (i < TILE) tile[i / TILE_N][i % TILE_N] = sum[k];
      }
      if (tid == 0)
        __hip_atomic_store(&p.counters[pnl], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_barrier();
    }

    const int64_t t0 = pnl * PT;
    // ---------------- epilogues on the finished tile [feature][node]
    if constexpr (EPI == EPI_RESID) {
      // x += y: all of this thread's residual loads are issued before any store
      constexpr int EPT = (TILE_F * TILE_N + NTH - 1) / NTH;
      float xv[EPT];
#pragma unroll
      for (int k = 0; k < EPT; ++k) {
        const int i = tid + k * NTH;
        const int n = i / TILE_F, fl = i - n * TILE_F;
        const int64_t f = t0 * 16 + fl;
        xv[k] = (n < nn && f < p.n_out) ? e.resid[(int64_t)n * e.ld_out + f] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < EPT; ++k) {
        const int i = tid + k * NTH;
        const int n = i / TILE_F, fl = i - n * TILE_F;
        const int64_t f = t0 * 16 + fl;
        if (n < nn && f < p.n_out) e.resid[(int64_t)n * e.ld_out + f] = xv[k] + tile[fl][n];
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      // packed tiles (2i, 2i+1) = (gate, up) rows [16i, 16i + 16); m as hi/lo rows
      for (int i = tid; i < (TILE_F / 2) * nn; i += NTH) {
        const int n = i / (TILE_F / 2), rl = i - n * (TILE_F / 2);
        const int a = rl / 16, r = rl % 16;
        const int64_t row = (t0 / 2 + a) * 16 + r;
        if (2 * row < p.n_out) {
          const float gt = tile[(2 * a) * 16 + r][n];
          const float up = tile[(2 * a + 1) * 16 + r][n];
          const float m = gt / (1.0f + expf(-gt)) * up;
          const f16 hi = (f16)m;
          e.out16[(int64_t)(2 * n) * e.ld_out + row] = __builtin_bit_cast(uint16_t, hi);
          e.out16[(int64_t)(2 * n + 1) * e.ld_out + row] = f32_to_f16_bits(m - (float)hi);
        }
      }
    } else if constexpr (EPI == EPI_QKV) {
      // rotate-half RoPE on q and k at pos = prefix_len + depth; v unrotated
      const int hd = e.head_dim;
      for (int i = tid; i < TILE_F * nn; i += NTH) {
        const int n = i / TILE_F, fl = i - n * TILE_F;
        const int64_t prow = t0 * 16 + fl;
        if (prow >= p.n_out) continue;
        const int head = (int)(prow / hd);
        const int r = (int)(prow % hd);
        const int ti = r / 16, loc = r % 16;
        const int j = loc < 8 ? 8 * ti + loc : hd / 2 + 8 * ti + (loc - 8);
        float val = tile[fl][n];
        if (head < e.n_q_heads + e.n_kv_heads) {
          const float partner = tile[fl ^ 8][n];
          float cs, sn;
          const int jj = j < hd / 2 ? j : j - hd / 2;
          rope_pair_angle(e.pos[n], jj, e.inv_freq, cs, sn);
          val = j < hd / 2 ? val * cs - partner * sn : partner * sn + val * cs;
        }
        if (head < e.n_q_heads) {
          const int64_t o = ((int64_t)n * e.n_q_heads + head) * hd + j;
          e.q32[o] = val;
          if (e.out16) e.out16[o] = f32_to_bf16_bits(val);
        } else if (head < e.n_q_heads + e.n_kv_heads) {
          const int64_t o = ((int64_t)n * e.n_kv_heads + (head - e.n_q_heads)) * hd + j;
          e.k32[o] = val;
          e.k_out[o] = f32_to_bf16_bits(val);
        } else {
          const int64_t o = ((int64_t)n * e.n_kv_heads + (head - e.n_q_heads - e.n_kv_heads)) * hd + j;
          e.v32[o] = val;
          e.v_out[o] = f32_to_bf16_bits(val);
        }
      }
    } else if constexpr (EPI == EPI_LOGITS) {
      if (e.out16) {
        for (int i = tid; i < TILE_F * nn; i += NTH) {
          const int n = i / TILE_F, fl = i - n * TILE_F;
          const int64_t f = t0 * 16 + fl;
          if (f < p.n_out) e.out16[(int64_t)n * e.ld_out + f] = f32_to_bf16_bits(tile[fl][n]);
        }
      }
      // this panel's best / runner-up per node, merged into the block's running pair
      if (tid < nn) {
        float v1 = best1[tid], v2 = best2[tid];
        int i1 = besti[tid];
        for (int fl = 0; fl < TILE_F; ++fl) {
          const int64_t f = t0 * 16 + fl;
          if (f >= p.n_out) break;
          merge_top2(v1, i1, v2, tile[fl][tid], (int)f, -INFINITY);
        }
        best1[tid] = v1;
        best2[tid] = v2;
        besti[tid] = i1;
      }
    }
    lds_barrier();  // the LDS tile is reused by the next panel
  };

  // One unit u: load the activation slice of unit u + 2, MFMA unit u from
  // LDS, refill this weight slot with unit u + 2, publish the slice of unit
  // u + 1 (loaded one unit earlier) to the other LDS buffer.  Prefetches past
  // the block's last unit re-read that unit, so every path issues the same
  // loads and the loop body is straight-line: the compiler then keeps the
  // prefetch in flight instead of draining it with a conservative wait.
  int xb = 0;
  const int64_t u_last = u_end - 1;
  Cur pf;            // the unit being prefetched
  int64_t pf_u = 0;
  auto step = [&](WRegs<UG, FT>& r, u32x4 (&xr_store)[XCH], u32x4 (&xr_load)[XCH]) {
    xload(pf, xr_load);
    compute(xb, r);
    wload(pf, r);
    xstore(xb ^ 1, xr_store);
    lds_barrier();
    xb ^= 1;
    if (pf_u < u_last) {
      ++pf_u;
      advance(pf);
    }
  };

  if (u_begin < u_end) {
    // weights: r0 / r1 hold units u / u + 1 at the top of the loop; slices:
    // x1 holds unit u + 1, x0 receives unit u + 2
    WRegs<UG, FT> r0, r1;
    u32x4 x0[XCH], x1[XCH];
    {
      Cur k = cur_of(u_begin);
      wload(k, r0);
      xload(k, x0);
      pf_u = u_begin;
      if (pf_u < u_last) {
        ++pf_u;
        advance(k);
      }
      wload(k, r1);
      xload(k, x1);
      if (pf_u < u_last) {
        ++pf_u;
        advance(k);
      }
      pf = k;
      xstore(0, x0);
    }
    lds_barrier();
    int64_t u = u_begin;
    while (u < u_end) {
      const int64_t pnl = u / GU;
      const int64_t s_end = min((pnl + 1) * GU, u_end);
      for (; u + 2 <= s_end; u += 2) {
        step(r0, x1, x0);
        step(r1, x0, x1);
      }
      if (u < s_end) {  // odd segment: one more unit, then the rings turn by one
        step(r0, x1, x0);
        const WRegs<UG, FT> t = r0;
        r0 = r1;
        r1 = t;
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
          const u32x4 tx = x0[i];
          x0[i] = x1[i];
          x1[i] = tx;
        }
        u += 1;
      }
      flush(pnl);
    }
  }

  if constexpr (EPI == EPI_LOGITS) {
    if (tid < nn) e.cand[(int64_t)b * nn + tid] = f32x4{best1[tid], __int_as_float(besti[tid]), best2[tid], 0.f};
  }
}

template <int FT, int NTX, int EPI, bool EXACT>
static hipError_t launch_t(const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  bool two = false;
  if constexpr (NTX <= 4) two = gemm_ug(p.kgroups, NTX) == 2;
  if constexpr (NTX <= 4) {
    if (two) {
      hipLaunchKernelGGL((gemm_q4_kernel<kGemmWaves, FT, NTX, 2, EPI, EXACT>), dim3(p.blocks),
                         dim3(kGemmWaves * 64), 0, s, p, e);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_q4_kernel<kGemmWaves, FT, NTX, 1, EPI, EXACT>), dim3(p.blocks),
                     dim3(kGemmWaves * 64), 0, s, p, e);
  return hipGetLastError();
}

template <int EPI, bool EXACT>
static hipError_t launch_ntx(const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  switch (gemm_ntx(p.n_nodes)) {
    case 1: return launch_t<gemm_ft_for(1), 1, EPI, EXACT>(p, e, s);
    case 2: return launch_t<gemm_ft_for(2), 2, EPI, EXACT>(p, e, s);
    case 3: return launch_t<gemm_ft_for(3), 3, EPI, EXACT>(p, e, s);
    case 4: return launch_t<gemm_ft_for(4), 4, EPI, EXACT>(p, e, s);
    case 5: return launch_t<gemm_ft_for(5), 5, EPI, EXACT>(p, e, s);
    case 6: return launch_t<gemm_ft_for(6), 6, EPI, EXACT>(p, e, s);
    case 7: return launch_t<gemm_ft_for(7), 7, EPI, EXACT>(p, e, s);
    default: return launch_t<gemm_ft_for(8), 8, EPI, EXACT>(p, e, s);
  }
}

int gemm_ntx(int n_nodes) { return (2 * n_nodes + 15) / 16; }

// column groups per unit: two (256 inputs) when k_in allows it and the LDS
// staging of two groups fits beside the tile
int gemm_ug(int kgroups, int ntx) { return (kgroups % 2 == 0 && ntx <= 4) ? 2 : 1; }

GemmPlan plan_gemm(int64_t n_out, int64_t k_in, int n_nodes) {
  GemmPlan g;
  g.ntx = gemm_ntx(n_nodes);
  g.ft = gemm_ft_for(g.ntx);
  g.n_tiles = (int)(n_out / 16);
  g.kgroups = (int)(k_in / 128);
  const int pt = kGemmWaves * g.ft;
  g.panels = (g.n_tiles + pt - 1) / pt;
  g.ug = gemm_ug(g.kgroups, g.ntx);
  g.units = (int64_t)g.panels * (g.kgroups / g.ug);
  // kGemmBlocksPerCU resident blocks on each of the 256 CUs; blocks take
  // whole pairs of units
  const int64_t pairs = (g.units + 1) / 2;
  const int64_t target = 256 * kGemmBlocksPerCU;
  g.blocks = (int)(pairs < target ? pairs : target);
  g.tile_floats = pt * 16 * g.ntx * 8;
  const int gu = g.kgroups / g.ug;
  g.c_max = 1;
  for (int pnl = 0; pnl < g.panels; ++pnl) {
    const int c = block_of_unit((int64_t)pnl * gu + gu - 1, g.units, g.blocks) -
                  block_of_unit((int64_t)pnl * gu, g.units, g.blocks) + 1;
    if (c > g.c_max) g.c_max = c;
  }
  return g;
}

SplitOut split_out(const GemmPlan& g, const float* part) {
  SplitOut so;
  so.part = part;
  so.units = g.units;
  so.blocks = g.blocks;
  so.gu = g.kgroups / g.ug;
  so.c_max = g.c_max;
  so.tile_f = kGemmWaves * g.ft * 16;
  so.tile_n = g.ntx * 8;
  so.panels = g.panels;
  return so;
}

hipError_t launch_gemm(int epi, bool exact, const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  switch (epi) {
    case EPI_PARTIAL:
      return exact ? launch_ntx<EPI_PARTIAL, true>(p, e, s) : launch_ntx<EPI_PARTIAL, false>(p, e, s);
    case EPI_QKV: return launch_ntx<EPI_QKV, true>(p, e, s);
    case EPI_SWIGLU: return launch_ntx<EPI_SWIGLU, false>(p, e, s);
    case EPI_LOGITS: return launch_ntx<EPI_LOGITS, true>(p, e, s);
    default:
      return exact ? launch_ntx<EPI_RESID, true>(p, e, s) : launch_ntx<EPI_RESID, false>(p, e, s);
  }
}

}  // namespace lucev
