// int4 block-32 skinny GEMM: Y[node, f] = sum_k X[node, k] * W[f, k] with
// W[f, k] = d[f, k/32] * (q[f, k] - 8), for up to 64 tree nodes.
//
// The target reads every weight once per forward and checks all drafted
// tokens in that one pass ("Lucebox Hub", section "배경: 어떤 문제를 푸는가",
// item 1; section "Speculative decoding 계층"), so this kernel streams the
// packed weights exactly once and reuses each dequantised weight for every
// tree node.  With 16..64 nodes that reuse is a dense contraction, so the
// MAC work goes to MFMA (v_mfma_f32_16x16x32_f16); the codes are expanded in
// registers (exponent-bias trick: exact q - 8 as fp16), each 32-column block
// is one MFMA K-step whose fp32 result takes the block's scale d, and the
// weights never touch LDS.
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

// 8 codes of one dword -> the 8 exact values (q - 8) as fp16, column order.
__device__ __forceinline__ f16x8 codes8(uint32_t w) {
  const uint32_t v0 = (w & 0x000F000Fu) | 0x64006400u;       // 1024 + q (cols 0, 1)
  const uint32_t v1 = (w & 0x00F000F0u) | 0x54005400u;       //   64 + q (cols 2, 3)
  const uint32_t w8 = w >> 8;
  const uint32_t v2 = (w8 & 0x000F000Fu) | 0x64006400u;      // 1024 + q (cols 4, 5)
  const uint32_t v3 = (w8 & 0x00F000F0u) | 0x54005400u;      //   64 + q (cols 6, 7)
  const f16x2 b1032 = {(f16)1032.0f, (f16)1032.0f};
  const f16x2 b72 = {(f16)72.0f, (f16)72.0f};
  const f16x2 h0 = __builtin_bit_cast(f16x2, v0) - b1032;
  const f16x2 h1 = __builtin_bit_cast(f16x2, v1) - b72;
  const f16x2 h2 = __builtin_bit_cast(f16x2, v2) - b1032;
  const f16x2 h3 = __builtin_bit_cast(f16x2, v3) - b72;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// fp16 scale of block j (of 4) from the lane's 4 packed scales, as fp32
__device__ __forceinline__ float scale_f32(u32x2 s, int j) {
  const uint32_t word = (j < 2) ? s[0] : s[1];
  const uint16_t bits = (uint16_t)((j & 1) ? (word >> 16) : (word & 0xFFFFu));
  return (float)__builtin_bit_cast(f16, bits);
}

// ------------------------------------------------------------ the GEMM
//
// Work: units (fg, c) = (FT-tile feature group, 128-column group), fg-major,
// split into equal contiguous ranges, one per block (block-level stream-K:
// every block gets the same number of weight bytes).  Inside a block the 4
// waves take a segment's column groups round-robin; partial sums meet in LDS.
// A feature group cut between blocks is finished by whichever contributor
// arrives last: partial tiles are written through with agent-scope stores
// that every wave waits for before the block counts in (no cache flush), read
// back with agent-scope loads and summed in block order, so results do not
// depend on timing.
//
// Precision: the activation operand is carried as two fp16 halves
// (x = hi + lo, about 22 significant bits) and both go through the MFMA, and
// the weights enter exactly, so rounding does not compound through a deep
// stack.  The
// normalised inputs of the QKV / gate-up / lm_head projections are formed
// here from the fp32 residual: u = x * rsqrt(mean(x^2) + eps) * g, with the
// row sums of x^2 produced by the previous kernel.

template <int NT, int FT, int AM>
struct Raw {
  u32x4 w[FT];
  u32x2 s[FT];
  u32x4 x[NT][4][2];                  // fp16 hi / lo planes, or fp32 x4 pairs
  u32x4 g[AM == A_F32N ? 4 : 1];      // bf16 gain x8 per block
};

template <int NT, int FT>
struct Ready {
  u32x4 w[FT];
  u32x2 s[FT];
  f16x8 hi[NT][4];
  f16x8 lo[NT][4];
};

template <int NT, int FT, int AM>
__device__ __forceinline__ void load_raw(const GemmParams& p, int c, int t0, int lane,
                                         Raw<NT, FT, AM>& r) {
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    int t = t0 + ft;
    t = t < p.n_tiles ? t : p.n_tiles - 1;  // ragged last group: re-read a valid tile
    const int64_t tg = (int64_t)t * p.kgroups + c;
    r.w[ft] = ld16(p.wq + tg * 1024 + lane * 16);
    r.s[ft] = *reinterpret_cast<const u32x2*>(p.wsc + tg * 64 + lr * 4);
  }
  if constexpr (AM == A_F32N) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r.g[j] = ld16(p.g + c * 128 + j * 32 + lq * 8);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int node = nt * 16 + lr;
    const bool ok = node < p.n_nodes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t off = (int64_t)node * p.ldx + c * 128 + j * 32 + lq * 8;
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      if constexpr (AM == A_F32N) {
        r.x[nt][j][0] = ok ? ld16(p.Xf + off) : z;
        r.x[nt][j][1] = ok ? ld16(p.Xf + off + 4) : z;
      } else {
        r.x[nt][j][0] = ok ? ld16(p.Xhi + off) : z;
        r.x[nt][j][1] = ok ? ld16(p.Xlo + off) : z;
      }
    }
  }
}

template <int NT, int FT, int AM>
__device__ __forceinline__ void make_ready(const Raw<NT, FT, AM>& r, Ready<NT, FT>& q,
                                           const float (&rinv)[NT]) {
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    q.w[ft] = r.w[ft];
    q.s[ft] = r.s[ft];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (AM == A_F32N) {
      float gf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gf[2 * e] = __uint_as_float(r.g[j][e] << 16);
        gf[2 * e + 1] = __uint_as_float(r.g[j][e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f16x8 h, l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float u = __uint_as_float(r.x[nt][j][e >> 2][e & 3]) * rinv[nt] * gf[e];
          const f16 hh = (f16)u;
          h[e] = hh;
          l[e] = (f16)(u - (float)hh);
        }
        q.hi[nt][j] = h;
        q.lo[nt][j] = l;
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        q.hi[nt][j] = __builtin_bit_cast(f16x8, r.x[nt][j][0]);
        q.lo[nt][j] = __builtin_bit_cast(f16x8, r.x[nt][j][1]);
      }
    }
  }
}

// Per 32-column block: MFMA of the exact codes against x_hi and x_lo, then
// the block's fp16 scale d (the MFMA column = lane % 16 = this lane's
// feature) is applied in fp32, so every weight enters as exactly d * (q - 8).
template <int NT, int FT>
__device__ __forceinline__ void mma_ready(const Ready<NT, FT>& q, f32x4 (&acc)[FT][NT]) {
  const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const f16x8 b = codes8(q.w[ft][j]);
      const float dsc = scale_f32(q.s[ft], j);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(q.hi[nt][j], b, zero, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_f16(q.lo[nt][j], b, t, 0, 0, 0);
        acc[ft][nt] += dsc * t;
      }
    }
  }
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

// the block whose unit range holds unit u (ranges are [b*U/B, (b+1)*U/B))
__device__ __forceinline__ int block_of(int64_t u, int64_t U, int B) {
  return (int)(((u + 1) * B - 1) / U);
}

template <int NT, int FT, int AM, int EPI>
__global__ __launch_bounds__(256) void gemm_q4_kernel(GemmParams p, EpiArgs e) {
  constexpr int TILE_F = FT * 16;
  constexpr int TILE_N = NT * 16;
  constexpr int TILE = TILE_F * TILE_N;
  __shared__ float red[3][FT][NT][4][64];
  __shared__ float tile[TILE_F][TILE_N + 1];
  __shared__ float s_rinv[TILE_N];
  __shared__ float best1[TILE_N], best2[TILE_N];
  __shared__ int besti[TILE_N];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int b = blockIdx.x;
  const int B = p.blocks;
  const int64_t U = p.units;
  const int G = p.kgroups;
  const int nn = p.n_nodes;
  const int64_t u_begin = (int64_t)b * U / B;
  const int64_t u_end = (int64_t)(b + 1) * U / B;

  if constexpr (EPI == EPI_LOGITS) {
    if (tid < TILE_N) {
      best1[tid] = -INFINITY;
      best2[tid] = -INFINITY;
      besti[tid] = 0x7fffffff;
    }
  }
  // 1/rms per row for the normalised input, from the producer's partial sums
  if constexpr (AM == A_F32N) {
    if (tid < TILE_N) {
      float r = 0.f;
      if (tid < nn) {
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
        int i = 0;
        for (; i + 4 <= p.ssq_groups; i += 4) {
          s0 += p.ssq[(int64_t)i * nn + tid];
          s1 += p.ssq[(int64_t)(i + 1) * nn + tid];
          s2 += p.ssq[(int64_t)(i + 2) * nn + tid];
          s3 += p.ssq[(int64_t)(i + 3) * nn + tid];
        }
        for (; i < p.ssq_groups; ++i) s0 += p.ssq[(int64_t)i * nn + tid];
        r = 1.0f / sqrtf(((s0 + s1) + (s2 + s3)) / (float)p.k_in + p.rms_eps);
      }
      s_rinv[tid] = r;
    }
  }
  __syncthreads();
  float rinv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) rinv[nt] = AM == A_F32N ? s_rinv[nt * 16 + lr] : 1.f;

  for (int64_t u = u_begin; u < u_end;) {
    const int fg = (int)(u / G);
    const int c0 = (int)(u - (int64_t)fg * G);
    const int c1 = (int)min((int64_t)G, (int64_t)c0 + (u_end - u));
    u += c1 - c0;
    const int t0 = fg * FT;

    f32x4 acc[FT][NT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[ft][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    {
      Raw<NT, FT, AM> raw;
      Ready<NT, FT> rdy;
      int c = c0 + wave;
      if (c < c1) load_raw(p, c, t0, lane, raw);
      while (c < c1) {
        make_ready(raw, rdy, rinv);
        const int cn = c + 4;
        if (cn < c1) load_raw(p, cn, t0, lane, raw);
        mma_ready(rdy, acc);
        c = cn;
      }
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

    // a feature group cut between blocks: last contributor to arrive sums
    const int bf = block_of((int64_t)fg * G, U, B);
    const int bl = block_of((int64_t)fg * G + G - 1, U, B);
    if (bf != bl) {
      const int slot = (u_begin >= (int64_t)fg * G) ? 0 : 1;
      float* part = p.partials + ((int64_t)b * 2 + slot) * TILE;
      for (int i = tid; i < TILE; i += 256) st_coherent(part + i, tile[i / TILE_N][i % TILE_N]);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every wave's stores done
      __syncthreads();
      if (tid == 0) {
        // the partials were written through (agent-scope stores) and every
        // wave waited for them before the barrier, so a relaxed count suffices
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[fg], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned)(bl - bf);
      }
      __syncthreads();
      if (!s_last) continue;
      // sum the contributors in block order; all loads of a batch of 8
      // contributors are issued before any add so their latencies overlap
      constexpr int PER = TILE / 256;
      float acc_s[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) acc_s[k] = 0.f;
      for (int b0 = bf; b0 <= bl; b0 += 8) {
        float v[8][PER];
#pragma unroll
        for (int uu = 0; uu < 8; ++uu) {
          const int bb = b0 + uu;
          if (bb <= bl) {
            const int sl = ((int64_t)bb * U / B >= (int64_t)fg * G) ? 0 : 1;
            const float* src = p.partials + ((int64_t)bb * 2 + sl) * TILE + tid;
#pragma unroll
            for (int k = 0; k < PER; ++k) v[uu][k] = ld_coherent(src + k * 256);
          }
        }
#pragma unroll
        for (int uu = 0; uu < 8; ++uu)
          if (b0 + uu <= bl)
#pragma unroll
            for (int k = 0; k < PER; ++k) acc_s[k] += v[uu][k];
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = tid + k * 256;
        tile[i / TILE_N][i % TILE_N] = acc_s[k];
      }
      if (tid == 0)
        __hip_atomic_store(&p.counters[fg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
    }

    // ---------------- epilogues on the finished tile [feature][node]
    if constexpr (EPI == EPI_RESID) {
      // x += y; the new rows' per-group sums of x^2 feed the next RMSNorm
      for (int i = tid; i < TILE_F * nn; i += 256) {
        const int n = i / TILE_F, fl = i - n * TILE_F;
        const int64_t f = (int64_t)t0 * 16 + fl;
        float xn = 0.f;
        if (f < p.n_out) {
          float* r = e.resid + (int64_t)n * e.ld_out + f;
          xn = *r + tile[fl][n];
          *r = xn;
        }
        tile[fl][n] = xn * xn;
      }
      if (e.ssq_out) {
        __syncthreads();
        if (tid < nn) {
          float s = 0.f;
          for (int fl = 0; fl < TILE_F; ++fl) s += tile[fl][tid];
          e.ssq_out[(int64_t)fg * nn + tid] = s;
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      // packed tiles (2i, 2i+1) = (gate, up) rows [16i, 16i + 16); m as fp16 hi + lo
      for (int i = tid; i < (TILE_F / 2) * nn; i += 256) {
        const int n = i / (TILE_F / 2), rl = i - n * (TILE_F / 2);
        const int a = rl / 16, r = rl % 16;
        const int64_t row = ((int64_t)t0 / 2 + a) * 16 + r;
        if (2 * row < p.n_out) {
          const float gt = tile[(2 * a) * 16 + r][n];
          const float up = tile[(2 * a + 1) * 16 + r][n];
          const float m = gt / (1.0f + expf(-gt)) * up;
          const f16 hi = (f16)m;
          e.out16[(int64_t)n * e.ld_out + row] = __builtin_bit_cast(uint16_t, hi);
          e.out16_lo[(int64_t)n * e.ld_out + row] = f32_to_f16_bits(m - (float)hi);
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
        for (int i = tid; i < TILE_F * nn; i += 256) {
          const int n = i / TILE_F, fl = i - n * TILE_F;
          const int64_t f = (int64_t)t0 * 16 + fl;
          if (f < p.n_out) e.out16[(int64_t)n * e.ld_out + f] = f32_to_bf16_bits(tile[fl][n]);
        }
      }
      // this group's best / runner-up per node, merged into the block's running pair
      if (tid < nn) {
        float v1 = best1[tid], v2 = best2[tid];
        int i1 = besti[tid];
        for (int fl = 0; fl < TILE_F; ++fl) {
          const int64_t f = (int64_t)t0 * 16 + fl;
          if (f >= p.n_out) break;
          merge_top2(v1, i1, v2, tile[fl][tid], (int)f, -INFINITY);
        }
        best1[tid] = v1;
        best2[tid] = v2;
        besti[tid] = i1;
      }
    }
    __syncthreads();  // LDS tiles are reused by the next segment
  }

  if constexpr (EPI == EPI_LOGITS) {
    if (tid < nn) e.cand[(int64_t)b * nn + tid] = f32x4{best1[tid], __int_as_float(besti[tid]), best2[tid], 0.f};
  }
}

template <int NT, int FT, int AM, int EPI>
static hipError_t launch_t(const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  hipLaunchKernelGGL((gemm_q4_kernel<NT, FT, AM, EPI>), dim3(p.blocks), dim3(256), 0, s, p, e);
  return hipGetLastError();
}

template <int AM, int EPI>
static hipError_t launch_nt(const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  const int nt = (p.n_nodes + 15) / 16;
  switch (nt) {
    case 1: return launch_t<1, 4, AM, EPI>(p, e, s);
    case 2: return launch_t<2, 4, AM, EPI>(p, e, s);
    case 3: return launch_t<3, 2, AM, EPI>(p, e, s);
    default: return launch_t<4, 2, AM, EPI>(p, e, s);
  }
}

int gemm_ft(int n_nodes) { return ((n_nodes + 15) / 16) <= 2 ? 4 : 2; }

GemmPlan plan_gemm(int64_t n_out, int64_t k_in, int n_nodes) {
  GemmPlan g;
  g.ft = gemm_ft(n_nodes);
  g.nt = (n_nodes + 15) / 16;
  g.n_tiles = (int)(n_out / 16);
  g.kgroups = (int)(k_in / 128);
  g.fgroups = (g.n_tiles + g.ft - 1) / g.ft;
  g.units = (int64_t)g.fgroups * g.kgroups;
  // two resident blocks per CU on 256 CUs, never more blocks than units
  g.blocks = (int)(g.units < 512 ? g.units : 512);
  g.tile_floats = g.ft * 16 * g.nt * 16;
  return g;
}

hipError_t launch_gemm(int epi, const GemmParams& p, const EpiArgs& e, hipStream_t s) {
  if (p.a_mode == A_F32N) {
    switch (epi) {
      case EPI_QKV: return launch_nt<A_F32N, EPI_QKV>(p, e, s);
      case EPI_SWIGLU: return launch_nt<A_F32N, EPI_SWIGLU>(p, e, s);
      default: return launch_nt<A_F32N, EPI_LOGITS>(p, e, s);
    }
  }
  return launch_nt<A_F16HL, EPI_RESID>(p, e, s);
}

}  // namespace lucev
