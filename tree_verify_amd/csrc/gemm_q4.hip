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

// the block-j scale of this lane's row, splatted to both fp16 halves (a
// shuffle of the scale word, which the packed multiply takes as its operand
// select rather than as separate instructions)
__device__ __forceinline__ f16x2 scale_pair(u32x2 s, int j) {
  const f16x2 w = __builtin_bit_cast(f16x2, (j < 2) ? s[0] : s[1]);
  return (j & 1) ? __builtin_shufflevector(w, w, 1, 1) : __builtin_shufflevector(w, w, 0, 0);
}

template <int UG, int FT>
struct WRegs {
  u32x4 w[UG][FT];  // per column group and tile: 4 blocks x 8 codes of this lane's row
  u32x2 s[UG][FT];  // the row's 4 block scales
};

// 16-byte buffer load into registers.  (A function of its own: called from a
// lambda inside the kernel template, the builtin keeps the host pass from
// emitting the kernel's launch stub.)
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0));
}
// the same, non-temporal (the weights are read once)
__device__ __forceinline__ u32x4 buffer_load16_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 2));
}
__device__ __forceinline__ u32x2 buffer_load8_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, 2));
}

// the smallest multiple of 16 rows >= rows whose slice (rows x rb bytes) is a
// multiple of `waves` 1 KB pieces
constexpr int stage_rows(int rows, int rb, int waves) {
  int r = rows;
  while ((r * rb) % (1024 * waves) != 0) r += 16;
  return r;
}

// sum of a lane's 8 products with an fp16 operand row, on top of c
__device__ __forceinline__ float dot8(f16x8 a, f16x8 b, float c) {
  c = __builtin_amdgcn_fdot2(f16x2{a[0], a[1]}, f16x2{b[0], b[1]}, c, false);
  c = __builtin_amdgcn_fdot2(f16x2{a[2], a[3]}, f16x2{b[2], b[3]}, c, false);
  c = __builtin_amdgcn_fdot2(f16x2{a[4], a[5]}, f16x2{b[4], b[5]}, c, false);
  return __builtin_amdgcn_fdot2(f16x2{a[6], a[7]}, f16x2{b[6], b[7]}, c, false);
}

// VR = 0: the products go to MFMA (NTX 16-row operand tiles).  VR in
// {1, 2, 4, 8}: at most VR operand rows, too few for a dense contraction, so
// each lane takes fp16 dot products (v_dot2_f32_f16) of its row's dequantised
// weights with each operand row (read once per 16 lanes from the staged
// slice), and the four column lanes of a row are summed at the panel's end;
// the sums then take the MFMA accumulator layout, so the flush is shared.
template <int WAVES, int FT, int NTX, int UG, bool EXACT, int VR>
__global__ __launch_bounds__(WAVES * 64, 2) void gemm_q4_kernel(GemmParams p) {
  static_assert(VR == 0 || (NTX == 1 && VR <= 8), "the dot-product path covers one operand tile");
  constexpr int NTH = WAVES * 64;
  constexpr int PT = WAVES * FT;   // tiles per panel
  constexpr int TILE_F = PT * 16;
  // staged hi/lo rows: whole row tiles, rounded up (extra tiles re-read row
  // 0 and are never used) so a slice is the same whole number of 1 KB
  // pieces for every wave
  constexpr int XR = stage_rows(NTX * 16, UG * 256, WAVES);
  constexpr int RB = UG * 256;     // bytes of a staged row (UG * 128 fp16)
  constexpr int XBUF = XR * RB;    // bytes of one staged slice
  constexpr int XI = XBUF / 1024;  // 1 KB pieces per slice (16 bytes a lane)
  constexpr int XIW = XI / WAVES;  // of them per wave
  // operand rows per node: hi and lo (exact projections), or hi alone (gate/up
  // and down, whose weights are themselves rounded once to fp16)
  constexpr int RPN = EXACT ? 2 : 1;
  constexpr int TILE_N = NTX * 16 / RPN;  // nodes
  constexpr int TILE = TILE_F * TILE_N;
  static_assert(XI % WAVES == 0, "a staged slice is whole 1 KB pieces per wave");
  // three slice buffers as separate arrays: the compiler can then tell the
  // stores into one from the operand reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t sx0[XBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t sx1[XBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t sx2[XBUF];
  __shared__ float tile[TILE_F][TILE_N + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int b = blockIdx.x;
  const int B = p.blocks;
  const int U = (int)p.units;  // unit counts and offsets below stay far below 2^31
  const int G = p.kgroups;   // 128-column groups
  const int GU = G / UG;     // units per panel
  const int nn = p.n_nodes;
  const int K = (int)p.k_in;
  const int u_begin = b * U / B;  // range_start, in 32 bits (b * U < 2^31)
  const int u_end = (b + 1) * U / B;


  // A unit as (panel, unit within the panel) plus this wave's first tile in
  // the panel, advanced without divisions; all scalar and 32-bit.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  struct Cur {
    int pnl, c, t0;  // t0 = pnl * PT + wave * FT
  };
  auto cur_of = [&](int u) {
    const int pnl = u / GU;
    return Cur{pnl, u - pnl * GU, pnl * PT + wave_s * FT};
  };
  auto advance = [&](Cur& k) {
    if (++k.c == GU) {
      k.c = 0;
      ++k.pnl;
      k.t0 += PT;
    }
  };
  // Load addresses: a wave-uniform base (scalar registers, advanced per
  // unit with scalar arithmetic) plus a per-lane offset fixed for the whole
  // kernel, so the loads cost no vector address arithmetic.
  const uint32_t w_off = (uint32_t)lane * 16u;  // bytes into a 1 KB tile-group
  const uint32_t s_off = (uint32_t)lr * 8u;     // bytes into its 128-byte scale group
  // the weights are read once: non-temporal loads keep them from evicting
  // the activation rows, which every block re-reads, from L2
  // Buffer descriptors over the nibble and scale regions (each below 2 GB), so
  // a tile-group's address is a 32-bit scalar offset: tg * 1024 and tg * 128.
  const __amdgpu_buffer_rsrc_t wq_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.wq, (short)0, (int)(p.n_out * K / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.wsc, (short)0, (int)(p.n_out * K / 16), 0x00020000);
  auto wload_one = [&](Cur k, WRegs<UG, FT>& r, int g, int ft) {
    // ragged last panel: re-read a valid tile (a wave-uniform clamp)
    const int t = min(k.t0 + ft, p.n_tiles - 1);
    const uint32_t tg = (uint32_t)(t * G + k.c * UG + g);
    r.w[g][ft] = buffer_load16_nt(wq_rsrc, w_off, tg * 1024u);
    r.s[g][ft] = buffer_load8_nt(ws_rsrc, s_off, tg * 128u);
  };
  auto wload = [&](Cur k, WRegs<UG, FT>& r) {
#pragma unroll
    for (int g = 0; g < UG; ++g)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) wload_one(k, r, g, ft);
  };
  // Activation slice of a unit: XR rows x UG * 128 columns, loaded into
  // registers (16 bytes a lane, 1 KB a wave instruction) one step before it
  // is stored to LDS, the step before the unit's own.  A 1 KB piece fills
  // RB-byte rows in lane order; the lane at 16-byte position p of row r
  // fetches chunk p ^ (r % 16) of that row, so chunk c of row r sits at
  // position c ^ (r % 16) and the MFMA operand reads (16 rows, one chunk)
  // fall in 16 different bank groups.  Rows past the 2n operand rows re-read
  // row 0: they only feed accumulator rows of padding nodes, which no
  // epilogue or consumer reads.
  uint32_t x_off[XIW];  // bytes from the slice's first column, per piece of this wave
#pragma unroll
  for (int q = 0; q < XIW; ++q) {
    const int ins = wave + WAVES * q;
    const int row = ins * (1024 / RB) + lane / (RB / 16);
    const int pos = lane % (RB / 16);
    // (hi-only: staged row r is node r's hi row, 2r)
    const int src_row = EXACT ? (row < 2 * nn ? row : 0) : (row < nn ? 2 * row : 0);
    x_off[q] = (uint32_t)((src_row * K + (pos ^ (row & 15)) * 8) * 2);
  }
  // Buffer loads: the per-lane offset is a register fixed for the whole
  // kernel and the unit's column offset a scalar, so a load costs no vector
  // address arithmetic; the descriptor's range is the operand rows, so a
  // stray offset reads zeros.
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.X, (short)0, (int)(2 * nn * K * 2), 0x00020000);
  struct XRegs {
    u32x4 v[XIW];
  };
  auto xload = [&](Cur k, XRegs& xr) {
    const uint32_t col_bytes = (uint32_t)(k.c * UG * 256);
#pragma unroll
    for (int q = 0; q < XIW; ++q) xr.v[q] = buffer_load16(x_rsrc, x_off[q], col_bytes);
  };
  auto xstore = [&](const XRegs& xr, uint8_t* dst) {
#pragma unroll
    for (int q = 0; q < XIW; ++q)
      *reinterpret_cast<u32x4*>(dst + (wave_s + WAVES * q) * 1024 + lane * 16) = xr.v[q];
  };

  f32x4 acc[FT][NTX];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int nt = 0; nt < NTX; ++nt) acc[ft][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float accv[FT][VR > 0 ? VR : 1];  // dot-product path: this lane's share, per operand row
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int r = 0; r < (VR > 0 ? VR : 1); ++r) accv[ft][r] = 0.f;

  // this lane's A-operand chunk (row lr, chunk 4j + lq of a 128-column
  // group) in a staged slice, per j
  uint32_t a_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a_off[j] = (uint32_t)(lr * RB + (((j * 4 + lq) ^ lr) * 16));
  // The weight prefetch of unit pf (into slot rf) is spread over the MFMA
  // iterations, one tile-group per iteration, so the block's waves do not all
  // queue their loads at the memory pipeline at the same moment.  The
  // scheduling fence keeps each load at its site while the arithmetic moves
  // freely around it.
  constexpr int kLoads = UG * FT;
  auto prefetch = [&](int q, Cur pf, WRegs<UG, FT>& rf) {
    if (q < kLoads) wload_one(pf, rf, q / FT, q % FT);
  };
  auto compute = [&](const uint8_t* xs, const WRegs<UG, FT>& r, Cur pf, WRegs<UG, FT>& rf) {
#pragma unroll
    for (int g = 0; g < UG; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        prefetch(g * 4 + j, pf, rf);
        __builtin_amdgcn_sched_barrier(kGemmSchedMask);
        if constexpr (VR > 0) {
          // columns 32j + 8lq .. + 7 of operand rows 0 .. VR - 1 (chunk 4j + lq
          // of row r sits at position (4j + lq) ^ r)
          f16x8 xv[VR];
#pragma unroll
          for (int rr = 0; rr < VR; ++rr)
            xv[rr] = *reinterpret_cast<const f16x8*>(xs + rr * RB + g * 256 + (((j * 4 + lq) ^ rr) * 16));
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) {
            if constexpr (EXACT) {
              // exact codes q - 8 times fp16 operands, summed in fp32 over the
              // lane's 8 columns of block j, then times the block scale
              const f16x8 cq = codes8(r.w[g][ft][j]);
              const float dj = (float)scale_pair(r.s[g][ft], j)[0];
#pragma unroll
              for (int rr = 0; rr < VR; ++rr) accv[ft][rr] = __builtin_fmaf(dot8(cq, xv[rr], 0.f), dj, accv[ft][rr]);
            } else {
              const f16x8 wb = dequant8(r.w[g][ft][j], scale_pair(r.s[g][ft], j));
#pragma unroll
              for (int rr = 0; rr < VR; ++rr) accv[ft][rr] = dot8(wb, xv[rr], accv[ft][rr]);
            }
          }
          continue;
        }
        f16x8 xa[NTX];
#pragma unroll
        for (int nt = 0; nt < NTX; ++nt)
          xa[nt] = *reinterpret_cast<const f16x8*>(xs + a_off[j] + nt * 16 * RB + g * 256);
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          if constexpr (EXACT) {
            // The exact codes q - 8 go through the MFMA, whose 32-deep sum
            // covers exactly one scale block; the block scale then multiplies
            // the fp32 sum.  Output column = lane % 16 = the row whose scale
            // this lane holds, so one scale serves all four outputs.
            const f16x8 cq = codes8(r.w[g][ft][j]);
            const float dj = (float)scale_pair(r.s[g][ft], j)[0];
#pragma unroll
            for (int nt = 0; nt < NTX; ++nt) {
              const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[nt], cq, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[ft][nt][i] = __builtin_fmaf(t[i], dj, acc[ft][nt][i]);
            }
          } else {
            const f16x8 wb = dequant8(r.w[g][ft][j], scale_pair(r.s[g][ft], j));
#pragma unroll
            for (int nt = 0; nt < NTX; ++nt)
              acc[ft][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[nt], wb, acc[ft][nt], 0, 0, 0);
          }
        }
      }
#pragma unroll
    for (int q = UG * 4; q < kLoads; ++q) prefetch(q, pf, rf);
  };

  // finish panel pnl: hi/lo rows merged into the LDS tile [feature][node],
  // split panels reduced across blocks, then the epilogue
  auto flush = [&](int pnl) {
    if constexpr (VR > 0) {
      // the four column lanes of a weight row summed; operand row 4 lq + i
      // then goes where the MFMA would have left it
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        float tot[VR];
#pragma unroll
        for (int r = 0; r < VR; ++r) {
          tot[r] = rows_sum(accv[ft][r]);
          accv[ft][r] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = 0.f;
#pragma unroll
          for (int r = 0; r < VR; ++r) v = (r == 4 * lq + i) ? tot[r] : v;
          acc[ft][0][i] = v;
        }
      }
    }
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int nt = 0; nt < NTX; ++nt) {
        // D layout: column (feature) = lane % 16, rows 4 * (lane / 16) + i =
        // hi/lo rows of nodes nt * 8 + 2 * (lane / 16) + {0, 1}
        const int fl = (wave * FT + ft) * 16 + lr;
        if constexpr (EXACT) {
          const int n0 = nt * 8 + 2 * lq;
          tile[fl][n0] = acc[ft][nt][0] + acc[ft][nt][1];
          tile[fl][n0 + 1] = acc[ft][nt][2] + acc[ft][nt][3];
        } else {
          // rows 4 * (lane / 16) + i are nodes nt * 16 + 4 * (lane / 16) + i
#pragma unroll
          for (int i = 0; i < 4; ++i) tile[fl][nt * 16 + 4 * lq + i] = acc[ft][nt][i];
        }
        acc[ft][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    lds_barrier();

    // this block's share of the panel, node-major; a later kernel sums the
    // contributors and applies the epilogue (plain stores: that kernel starts
    // after this one has finished).  A fixed store count per thread, with no
    // branch (padding nodes past the last are masked off, not skipped), lets
    // the compiler count the loads still in flight across the flush exactly
    // rather than wait for all of them.
    const int bf = ((pnl * GU + 1) * B - 1) / U;  // block_of_unit, in 32 bits
    static_assert(TILE % NTH == 0, "partial tile must split evenly over the threads");
    float* dst = p.partials + ((int64_t)pnl * p.c_max + (b - bf)) * TILE;
#pragma unroll
    for (int k = 0; k < TILE / NTH; ++k) {
      const int i = tid + k * NTH;
      const int n = i / TILE_F, fl = i - n * TILE_F;
      if (n < nn) dst[i] = tile[fl][n];
    }
    lds_barrier();  // the LDS tile is reused by the next panel
  };

  // One unit u: load the activation slice of unit u + 2 into registers, MFMA
  // unit u (its slice in LDS) while loading the weights of unit u + 2 into
  // the register slot unit u - 1 used, store the slice of unit u + 1 (loaded
  // one step earlier) into the LDS buffer unit u - 2 used, which every wave
  // has finished, and finish the panel when u ends a segment.  Unit u uses
  // slice buffer, slice registers and weight slot u % 3 (counted from the
  // block's first unit).  The compiler waits for each register load where
  // its value is used.  Prefetches past the block's last unit re-read that
  // unit, so every path issues the same loads.
  const int u_last = u_end - 1;
  if (u_begin < u_end) {
    WRegs<UG, FT> r0, r1, r2;
    XRegs x0, x1, x2;
    Cur pf = cur_of(u_begin);  // next unit to prefetch
    int pf_u = u_begin;
    // (selects, not branches: with a branch the compiler may reuse an earlier
    // load's registers on the path that does not advance, which makes every
    // later wait drain the queue)
    auto next = [&](Cur& k, int& ku) {
      const int adv = ku < u_last ? 1 : 0;
      ku += adv;
      const int c = k.c + adv;
      const int wrap = c == GU ? 1 : 0;
      k.pnl += wrap;
      k.t0 += wrap * PT;
      k.c = wrap ? 0 : c;
    };
    // The prologue asks for the first unit's weights alone: every block's
    // requests reach memory at once, and the first unit's arrive sooner
    // without the second's queued beside them; the second unit's weights
    // are requested at the start of the first step.
    xload(pf, x0);
    __builtin_amdgcn_sched_barrier(0);
    wload(pf, r0);
    next(pf, pf_u);
    __builtin_amdgcn_sched_barrier(0);
    xload(pf, x1);
    __builtin_amdgcn_sched_barrier(0);
    xstore(x0, sx0);
    lds_barrier();
    int u = u_begin;
    Cur cu = cur_of(u_begin);
    auto step = [&](const uint8_t* xs, uint8_t* xw, const XRegs& xr_w, XRegs& xr_l, WRegs<UG, FT>& r,
                    WRegs<UG, FT>& rf) {
      xload(pf, xr_l);
      __builtin_amdgcn_sched_barrier(0);
      compute(xs, r, pf, rf);
      __builtin_amdgcn_sched_barrier(0);
      xstore(xr_w, xw);
      lds_barrier();
      next(pf, pf_u);
      if (cu.c == GU - 1 || u == u_last) flush(cu.pnl);
      advance(cu);
      ++u;
    };
    // first unit: the second unit's weights, then the regular step
    wload(pf, r1);
    next(pf, pf_u);
    __builtin_amdgcn_sched_barrier(0);
    step(sx0, sx1, x1, x2, r0, r2);
    // a counted loop with the remainder after it: no exit from the middle of
    // the loop body, whose paths would make the load waits conservative
    const int n_units = u_end - u_begin;
    int k = 1;
    for (; k + 3 <= n_units; k += 3) {
      step(sx1, sx2, x2, x0, r1, r0);
      step(sx2, sx0, x0, x1, r2, r1);
      step(sx0, sx1, x1, x2, r0, r2);
    }
    if (k < n_units) step(sx1, sx2, x2, x0, r1, r0);
    if (k + 1 < n_units) step(sx2, sx0, x0, x1, r2, r1);
  }
}

template <int FT, int NTX, bool EXACT, int VR = 0>
static hipError_t launch_t(const GemmParams& p, hipStream_t s) {
  bool two = false;
  if constexpr (NTX <= 3 && VR < 8) two = p.ug == 2;
  if constexpr (NTX <= 3 && VR < 8) {
    if (two) {
      hipLaunchKernelGGL((gemm_q4_kernel<kGemmWaves, FT, NTX, 2, EXACT, VR>), dim3(p.blocks), dim3(kGemmWaves * 64),
                         0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_q4_kernel<kGemmWaves, FT, NTX, 1, EXACT, VR>), dim3(p.blocks), dim3(kGemmWaves * 64), 0,
                     s, p);
  return hipGetLastError();
}

// the dot-product path: one operand tile, the plan's tiles per wave
template <bool EXACT, int VR>
static hipError_t launch_vr(const GemmParams& p, hipStream_t s) {
  if constexpr (gemm_ft_for(1) > 1) {
    if (p.ft == 1) return launch_t<1, 1, EXACT, VR>(p, s);
  }
  return launch_t<gemm_ft_for(1), 1, EXACT, VR>(p, s);
}

// the plan's tiles per wave: gemm_ft_for(ntx), or one (kGemmNarrowUnits,
// kGemmMidUnits)
template <int NTX, bool EXACT>
static hipError_t launch_ft(const GemmParams& p, hipStream_t s) {
  if constexpr (gemm_ft_for(NTX) > 1) {
    if (p.ft == 1) return launch_t<1, NTX, EXACT>(p, s);
  }
  return launch_t<gemm_ft_for(NTX), NTX, EXACT>(p, s);
}

template <bool EXACT>
static hipError_t launch_ntx(const GemmParams& p, hipStream_t s) {
  switch (p.vr) {
    case 1: return launch_vr<EXACT, 1>(p, s);
    case 2: return launch_vr<EXACT, 2>(p, s);
    case 4: return launch_vr<EXACT, 4>(p, s);
    case 8: return launch_vr<EXACT, 8>(p, s);
    default: break;
  }
  switch (gemm_ntx(p.n_nodes, EXACT)) {
    case 1: return launch_ft<1, EXACT>(p, s);
    case 2: return launch_ft<2, EXACT>(p, s);
    case 3: return launch_ft<3, EXACT>(p, s);
    case 4: return launch_ft<4, EXACT>(p, s);
    default: break;
  }
  // more than four operand tiles: the hi/lo rows of more than 32 nodes (the
  // hi-only kernel has at most four tiles for 64 nodes)
  if constexpr (EXACT) {
    switch (gemm_ntx(p.n_nodes, EXACT)) {
      case 5: return launch_t<gemm_ft_for(5), 5, EXACT>(p, s);
      case 6: return launch_t<gemm_ft_for(6), 6, EXACT>(p, s);
      case 7: return launch_t<gemm_ft_for(7), 7, EXACT>(p, s);
      default: return launch_t<gemm_ft_for(8), 8, EXACT>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

int gemm_ntx(int n_nodes, bool exact) { return exact ? (2 * n_nodes + 15) / 16 : (n_nodes + 15) / 16; }

int g_gemv_max_rows = 0;

// operand rows at or below g_gemv_max_rows take the dot-product path (rounded
// up to 1, 2, 4 or 8 rows), more go to MFMA
int gemm_vr(int n_nodes, bool exact) {
  const int rows = exact ? 2 * n_nodes : n_nodes;
  if (rows > g_gemv_max_rows) return 0;
  return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : 8;
}

// column groups per unit: two (256 inputs) when k_in allows it and the
// registers hold two groups' weights beside the accumulators of ntx tiles
// (one-group units measured slower inside the verify step, also for the
// projections whose weights spread thinly over the blocks)
// (the 8-row dot-product path takes one group: two would spill)
int gemm_ug(int kgroups, int ntx, int vr) { return (kgroups % 2 == 0 && ntx <= 3 && vr < 8) ? 2 : 1; }

GemmPlan plan_gemm(int64_t n_out, int64_t k_in, int n_nodes, bool exact) {
  GemmPlan g;
  g.ntx = gemm_ntx(n_nodes, exact);
  g.vr = gemm_vr(n_nodes, exact);
  g.tile_n = exact ? g.ntx * 8 : g.ntx * 16;
  g.n_tiles = (int)(n_out / 16);
  g.kgroups = (int)(k_in / 128);
  auto shape = [&](int ft, int ug) {
    g.ft = ft;
    g.ug = ug;
    const int pt = kGemmWaves * ft;
    g.panels = (g.n_tiles + pt - 1) / pt;
    g.units = (int64_t)g.panels * (g.kgroups / ug);
  };
  // kGemmBlocksPerCU resident blocks on each CU, at least one unit each
  const int64_t target = (int64_t)device_cu_count() * kGemmBlocksPerCU;
  shape(gemm_ft_for(g.ntx), gemm_ug(g.kgroups, g.ntx, g.vr));
  if (g.ft > 1 && g.units < kGemmNarrowUnits * target) shape(1, 1);
  else if (g.ft > 1 && g.units < kGemmMidUnits * target) shape(1, g.ug);
  g.blocks = (int)(g.units < target ? g.units : target);
  g.tile_floats = kGemmWaves * g.ft * 16 * g.tile_n;
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
  so.tile_n = g.tile_n;
  so.panels = g.panels;
  return so;
}

hipError_t launch_gemm(bool exact, const GemmParams& p, hipStream_t s) {
  return exact ? launch_ntx<true>(p, s) : launch_ntx<false>(p, s);
}

}  // namespace lucev
