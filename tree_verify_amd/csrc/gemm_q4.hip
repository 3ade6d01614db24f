// int4 block-32 skinny GEMM: Y[node, f] = sum_k X[node, k] * W[f, k] with
// W[f, k] = d[f, k/32] * (q[f, k] - 8), for up to 64 tree nodes.
//
// The target reads every weight once per forward and checks all drafted
// tokens in that one pass ("Lucebox Hub", section "배경: 어떤 문제를 푸는가",
// item 1; section "Speculative decoding 계층"), so this kernel streams the
// packed weights exactly once and reuses each dequantised weight for every
// tree node.  With 16..64 nodes that reuse is a dense contraction, so the
// MAC work goes to MFMA (v_mfma_f32_16x16x32_f16); the weights are
// dequantised in registers (exponent-bias trick, exact q - 8, one fp16
// rounding of d * (q - 8)) and never touch LDS.
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

// 8 codes of one dword -> 8 fp16 weights d * (q - 8) in column order.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 s2) {
  const uint32_t v0 = (w & 0x000F000Fu) | 0x64006400u;       // 1024 + q (cols 0, 1)
  const uint32_t v1 = (w & 0x00F000F0u) | 0x54005400u;       //   64 + q (cols 2, 3)
  const uint32_t w8 = w >> 8;
  const uint32_t v2 = (w8 & 0x000F000Fu) | 0x64006400u;      // 1024 + q (cols 4, 5)
  const uint32_t v3 = (w8 & 0x00F000F0u) | 0x54005400u;      //   64 + q (cols 6, 7)
  const f16x2 b1032 = {(f16)1032.0f, (f16)1032.0f};
  const f16x2 b72 = {(f16)72.0f, (f16)72.0f};
  f16x2 h0 = (__builtin_bit_cast(f16x2, v0) - b1032) * s2;
  f16x2 h1 = (__builtin_bit_cast(f16x2, v1) - b72) * s2;
  f16x2 h2 = (__builtin_bit_cast(f16x2, v2) - b1032) * s2;
  f16x2 h3 = (__builtin_bit_cast(f16x2, v3) - b72) * s2;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ f16x2 scale_pair(u32x2 s, int j) {
  const uint32_t word = (j < 2) ? s[0] : s[1];
  const uint16_t bits = (uint16_t)((j & 1) ? (word >> 16) : (word & 0xFFFFu));
  const f16 v = __builtin_bit_cast(f16, bits);
  return f16x2{v, v};
}

// ------------------------------------------------------------ the GEMM

template <int NT, int FT>
struct Frag {
  u32x4 w[FT];
  u32x2 s[FT];
  u32x4 x[NT][4];
};

template <int NT, int FT>
__device__ __forceinline__ void load_frag(const GemmParams& p, int c, int t0, int lane,
                                          Frag<NT, FT>& f) {
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    int t = t0 + ft;
    t = t < p.n_tiles ? t : p.n_tiles - 1;  // ragged last group: re-read a valid tile
    const int64_t tg = (int64_t)t * p.kgroups + c;
    f.w[ft] = ld16(p.wq + tg * 1024 + lane * 16);
    f.s[ft] = *reinterpret_cast<const u32x2*>(p.wsc + tg * 64 + lr * 4);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int node = nt * 16 + lr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (node < p.n_nodes)
        f.x[nt][j] = ld16(p.X + (int64_t)node * p.ldx + c * 128 + j * 32 + lq * 8);
      else
        f.x[nt][j] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int NT, int FT>
__device__ __forceinline__ void mma_frag(const Frag<NT, FT>& f, f32x4 (&acc)[FT][NT]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const f16x8 b = dequant8(f.w[ft][j], scale_pair(f.s[ft], j));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f16x8 a = __builtin_bit_cast(f16x8, f.x[nt][j]);
        acc[ft][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[ft][nt], 0, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ void rope_pair_angle(int pos, int jj, int head_dim, const double* inv_freq,
                                                float& cs, float& sn) {
  // angle in fp64, reduced to [-pi, pi] before the fp32 sin / cos
  const double th = (double)pos * inv_freq[jj];
  const double two_pi = 6.283185307179586476925286766559;
  const double r = th - two_pi * rint(th / two_pi);
  const float rf = (float)r;
  sincosf(rf, &sn, &cs);
}

template <int NT, int FT, int EPI>
__global__ __launch_bounds__(256) void gemm_q4_kernel(GemmParams p, EpiArgs e) {
  constexpr int TILE_F = FT * 16;
  constexpr int TILE_N = NT * 16;
  __shared__ float red[3][FT][NT][4][64];
  __shared__ float tile[TILE_F][TILE_N + 1];
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int fg = blockIdx.x / p.ksplit;
  const int ks = blockIdx.x - fg * p.ksplit;
  const int t0 = fg * FT;
  const int g_begin = ks * p.gps;
  const int g_end = min(p.kgroups, g_begin + p.gps);

  f32x4 acc[FT][NT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[ft][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the 4 waves interleave over the block's column groups; loads of the next
  // group are issued before the current one is consumed
  Frag<NT, FT> fa, fb;
  int c = g_begin + wave;
  if (c < g_end) load_frag(p, c, t0, lane, fa);
  while (c < g_end) {
    int cn = c + 4;
    if (cn < g_end) load_frag(p, cn, t0, lane, fb);
    mma_frag(fa, acc);
    c = cn;
    if (c >= g_end) break;
    cn = c + 4;
    if (cn < g_end) load_frag(p, cn, t0, lane, fa);
    mma_frag(fb, acc);
    c = cn;
  }

  // cross-wave reduction in a fixed order (deterministic)
  if (wave > 0) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][ft][nt][i][lane] = acc[ft][nt][i];
  }
  __syncthreads();
  if (wave == 0) {
    const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[ft][nt][i];
          v += red[0][ft][nt][i][lane];
          v += red[1][ft][nt][i][lane];
          v += red[2][ft][nt][i][lane];
          // D layout: column (feature) = lane % 16, row (node) = 4 * (lane / 16) + i
          tile[ft * 16 + lr][nt * 16 + lq * 4 + i] = v;
        }
  }
  __syncthreads();

  if (p.ksplit > 1) {
    // split-K: publish this block's partial tile; the last block of the
    // feature group sums all partials in split order and runs the epilogue
    float* part = p.partials + ((int64_t)fg * p.ksplit + ks) * (TILE_F * TILE_N);
    for (int i = tid; i < TILE_F * TILE_N; i += 256) part[i] = tile[i / TILE_N][i % TILE_N];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&p.counters[fg], 1u);
      is_last = (prev == (unsigned)(p.ksplit - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    const float* base = p.partials + (int64_t)fg * p.ksplit * (TILE_F * TILE_N);
    for (int i = tid; i < TILE_F * TILE_N; i += 256) {
      float s = 0.f;
      for (int k = 0; k < p.ksplit; ++k) s += __builtin_nontemporal_load(base + (int64_t)k * (TILE_F * TILE_N) + i);
      tile[i / TILE_N][i % TILE_N] = s;
    }
    if (tid == 0) atomicExch(&p.counters[fg], 0u);
    __syncthreads();
  }

  const int nn = p.n_nodes;
  if constexpr (EPI == EPI_RESID) {
    // x += y (fp32 residual stream, plain row order)
    for (int i = tid; i < TILE_F * nn; i += 256) {
      const int n = i / TILE_F, fl = i - n * TILE_F;
      const int64_t f = (int64_t)t0 * 16 + fl;
      if (f < p.n_out) e.resid[(int64_t)n * e.ld_out + f] += tile[fl][n];
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // packed tiles (2i, 2i+1) = (gate, up) rows [16i, 16i + 16)
    for (int i = tid; i < (TILE_F / 2) * nn; i += 256) {
      const int n = i / (TILE_F / 2), rl = i - n * (TILE_F / 2);
      const int a = rl / 16, r = rl % 16;
      const int64_t row = ((int64_t)t0 / 2 + a) * 16 + r;
      if (2 * row < p.n_out) {
        const float gt = tile[(2 * a) * 16 + r][n];
        const float up = tile[(2 * a + 1) * 16 + r][n];
        const float m = gt / (1.0f + expf(-gt)) * up;
        e.out16[(int64_t)n * e.ld_out + row] = f32_to_f16_bits(m);
      }
    }
  } else if constexpr (EPI == EPI_QKV) {
    // rotate-half RoPE on q and k at pos = prefix_len + depth; v unrotated
    const int hd = e.head_dim;
    for (int i = tid; i < TILE_F * nn; i += 256) {
      const int n = i / TILE_F, fl = i - n * TILE_F;
      const int64_t prow = (int64_t)t0 * 16 + fl;
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
        rope_pair_angle(e.pos[n], jj, hd, e.inv_freq, cs, sn);
        val = j < hd / 2 ? val * cs - partner * sn : partner * sn + val * cs;
      }
      uint16_t* dst;
      if (head < e.n_q_heads)
        dst = e.out16 + ((int64_t)n * e.n_q_heads + head) * hd + j;
      else if (head < e.n_q_heads + e.n_kv_heads)
        dst = e.k_out + ((int64_t)n * e.n_kv_heads + (head - e.n_q_heads)) * hd + j;
      else
        dst = e.v_out + ((int64_t)n * e.n_kv_heads + (head - e.n_q_heads - e.n_kv_heads)) * hd + j;
      *dst = f32_to_bf16_bits(val);
    }
  } else if constexpr (EPI == EPI_LOGITS) {
    if (e.out16) {
      for (int i = tid; i < TILE_F * nn; i += 256) {
        const int n = i / TILE_F, fl = i - n * TILE_F;
        const int64_t f = (int64_t)t0 * 16 + fl;
        if (f < p.n_out) e.out16[(int64_t)n * e.ld_out + f] = f32_to_bf16_bits(tile[fl][n]);
      }
    }
    // per node: best, its index (lowest on ties) and runner-up of this group
    if (tid < nn) {
      float v1 = -INFINITY, v2 = -INFINITY;
      int i1 = 0x7fffffff;
      for (int fl = 0; fl < TILE_F; ++fl) {
        const int64_t f = (int64_t)t0 * 16 + fl;
        if (f >= p.n_out) break;
        const float v = tile[fl][tid];
        if (v > v1) {
          v2 = v1;
          v1 = v;
          i1 = (int)f;
        } else if (v > v2) {
          v2 = v;
        }
      }
      e.cand[(int64_t)fg * e.cand_stride + tid] =
          f32x4{v1, __int_as_float(i1), v2, 0.f};
    }
  }
}

template <int NT, int FT, int EPI>
static hipError_t launch_t(const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  const int blocks = p.fgroups * p.ksplit;
  hipLaunchKernelGGL((gemm_q4_kernel<NT, FT, EPI>), dim3(blocks), dim3(256), 0, s, p, e);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_nt(const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  const int nt = (p.n_nodes + 15) / 16;
  switch (nt) {
    case 1: return launch_t<1, 4, EPI>(p, e, s);
    case 2: return launch_t<2, 4, EPI>(p, e, s);
    case 3: return launch_t<3, 2, EPI>(p, e, s);
    default: return launch_t<4, 2, EPI>(p, e, s);
  }
}

int gemm_ft(int n_nodes) { return ((n_nodes + 15) / 16) <= 2 ? 4 : 2; }

GemmPlan plan_gemm(int64_t n_out, int64_t k_in, int n_nodes, int max_ksplit) {
  GemmPlan g;
  g.ft = gemm_ft(n_nodes);
  g.nt = (n_nodes + 15) / 16;
  g.n_tiles = (int)(n_out / 16);
  g.kgroups = (int)(k_in / 128);
  g.fgroups = (g.n_tiles + g.ft - 1) / g.ft;
  // aim for ~2 blocks per CU; each wave should still own >= 2 column groups
  int ks = (512 + g.fgroups - 1) / g.fgroups;
  const int ks_cap = g.kgroups / 8 > 0 ? g.kgroups / 8 : 1;
  if (ks > ks_cap) ks = ks_cap;
  if (ks > max_ksplit) ks = max_ksplit;
  if (ks < 1) ks = 1;
  g.gps = (g.kgroups + ks - 1) / ks;
  g.ksplit = (g.kgroups + g.gps - 1) / g.gps;
  g.tile_floats = g.ft * 16 * g.nt * 16;
  return g;
}

hipError_t launch_gemm(int epi, const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  switch (epi) {
    case EPI_RESID: return launch_nt<EPI_RESID>(p, e, s);
    case EPI_SWIGLU: return launch_nt<EPI_SWIGLU>(p, e, s);
    case EPI_QKV: return launch_nt<EPI_QKV>(p, e, s);
    default: return launch_nt<EPI_LOGITS>(p, e, s);
  }
}

}  // namespace lucev
