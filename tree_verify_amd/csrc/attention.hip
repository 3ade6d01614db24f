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
#include "internal.h"

namespace lucev {

constexpr int KT = 64;  // tokens per LDS tile

// Blocks have at least 512 threads (8 waves); with one query tile per wave
// up to 16 waves share the LDS tiles, with more tiles per wave 8 waves do.
template <int D, int QPW>
__global__ __launch_bounds__(QPW == 1 ? 1024 : 512) void attn_partial_kernel(AttnParams p) {
  constexpr int KLD = D + 8;   // padded K row (elements): spreads LDS banks
  constexpr int VLD = KT + 8;  // padded V^T row
  constexpr int KCH = KT * D / 8;  // 16-byte chunks of a K tile
  constexpr int VCH = D * KT / 8;
  constexpr int MAXC = (KCH + VCH) / 512;
  __shared__ __attribute__((aligned(16))) uint16_t sK[KT * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VLD];

  const int tid = threadIdx.x;
  const int nth = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int chunk = blockIdx.x;
  const int g = blockIdx.y;
  const int G = p.n_q_heads / p.n_kv_heads;
  const int RT = (p.rows + 15) / 16;
  const int k_begin = chunk * p.chunk;
  const int k_end = min(p.prefix_len, k_begin + p.chunk);

  const uint16_t* kbase = p.kc + (int64_t)g * p.cap * D;
  const uint16_t* vbase = p.vc + (int64_t)g * D * p.cap;

  u32x4 pre[MAXC];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < MAXC; ++r) {
      const int cid = tid + r * nth;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (cid < KCH) {
        const int key = cid / (D / 8), part = cid % (D / 8);
        const int gk = k0 + key;
        if (gk < k_end) val = ld16(kbase + (int64_t)gk * D + part * 8);
      } else if (cid < KCH + VCH) {
        const int v = cid - KCH;
        const int dim = v / (KT / 8), part = v % (KT / 8);
        const int gk = k0 + part * 8;
        if (gk < k_end) {
          val = ld16(vbase + (int64_t)dim * p.cap + gk);
          const int valid = k_end - gk;
          if (valid < 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e >= valid) val[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
          }
        }
      }
      pre[r] = val;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int r = 0; r < MAXC; ++r) {
      const int cid = tid + r * nth;
      if (cid < KCH) {
        const int key = cid / (D / 8), part = cid % (D / 8);
        *reinterpret_cast<u32x4*>(sK + key * KLD + part * 8) = pre[r];
      } else if (cid < KCH + VCH) {
        const int v = cid - KCH;
        const int dim = v / (KT / 8), part = v % (KT / 8);
        *reinterpret_cast<u32x4*>(sV + dim * VLD + part * 8) = pre[r];
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
    const int qt = wave * QPW + i;
    const int row = qt * 16 + lr;
    const bool ok = qt < RT && row < p.rows;
    int node = 0, head = 0;
    if (ok) {
      node = row / G;
      head = g * G + (row - node * G);
    }
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const int64_t off = ((int64_t)node * p.n_q_heads + head) * D + kk * 32 + lq * 8;
      if (p.q32) {
        bf16x8 hv, lv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = ok ? p.q32[off + e] : 0.f;
          const __bf16 hb = (__bf16)x;
          hv[e] = hb;
          lv[e] = (__bf16)(x - (float)hb);
        }
        qf[i][kk] = hv;
        ql[i][kk] = lv;
      } else {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (ok) v = ld16(p.q + off);
        qf[i][kk] = __builtin_bit_cast(bf16x8, v);
        ql[i][kk] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  const bool q_lo = p.q32 != nullptr;

  gload(k_begin);
  sstore();
  __syncthreads();

  for (int k0 = k_begin; k0 < k_end; k0 += KT) {
    const bool more = k0 + KT < k_end;
    if (more) gload(k0 + KT);

#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int qt = wave * QPW + i;
      if (qt >= RT) continue;
      // S^T tiles: subtile s = 2*ks + h covers keys ks*32 + 8*(r/4) + 4*h + r%4
      f32x4 sacc[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int ks = s >> 1, h = s & 1;
        const int key = ks * 32 + (lr >> 2) * 8 + h * 4 + (lr & 3);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + key * KLD + kk * 32 + lq * 8);
          sacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[i][kk], sacc[s], 0, 0, 0);
          if (q_lo) sacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[i][kk], sacc[s], 0, 0, 0);
        }
      }
      // this lane holds query lr, keys ks*32 + lq*8 + h*4 + ii
      float mx = -INFINITY;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ks = s >> 1, h = s & 1;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          float v = sacc[s][ii] * p.scale_log2;
          if (k0 + ks * 32 + lq * 8 + h * 4 + ii >= k_end) v = -INFINITY;
          sacc[s][ii] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m[i], mx);
      const float alpha = __builtin_amdgcn_exp2f(m[i] - m_new);
      float psum = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float pv = __builtin_amdgcn_exp2f(sacc[s][ii] - m_new);
          sacc[s][ii] = pv;
          psum += pv;
        }
      l[i] = l[i] * alpha + psum;
      m[i] = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) O[i][dt] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // P as bf16 hi + lo (about 16 significant bits)
        bf16x8 pb, pl;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const __bf16 h0 = (__bf16)sacc[2 * ks][ii];
          const __bf16 h1 = (__bf16)sacc[2 * ks + 1][ii];
          pb[ii] = h0;
          pb[4 + ii] = h1;
          pl[ii] = (__bf16)(sacc[2 * ks][ii] - (float)h0);
          pl[4 + ii] = (__bf16)(sacc[2 * ks + 1][ii] - (float)h1);
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(sV + (dt * 16 + lr) * VLD + ks * 32 + lq * 8);
          O[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, O[i][dt], 0, 0, 0);
          O[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl, O[i][dt], 0, 0, 0);
        }
      }
    }

    __syncthreads();
    if (more) {
      sstore();
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int qt = wave * QPW + i;
    if (qt >= RT) continue;
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
}

constexpr int kMaxChunks = 512;

// One block (256 threads) per (node, query head): log-sum-exp merge of the
// prefix-chunk partials with the node's ancestor keys.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineParams c, TreeArgs t) {
  constexpr int PARTS = 256 / D;  // threads per output dim
  constexpr int DPL = D / 64;     // dims per lane in the ancestor dot products
  __shared__ float s_w[kMaxChunks];
  __shared__ float s_anc[kMaxNodes];
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

  // ancestor scores: wave w takes every 4th ancestor
  {
    float qv[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int64_t o = ((int64_t)node * c.n_q_heads + h) * D + lane * DPL + i;
      qv[i] = c.q32 ? c.q32[o] : bf16_bits_to_f32(c.q[o]);
    }
    int k = 0;
    for (int a = 0; a < t.n; ++a) {
      if (!((anc >> a) & 1ull)) continue;
      if ((k & 3) == wave) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          const int64_t o = ((int64_t)a * c.n_kv_heads + g) * D + lane * DPL + i;
          s += qv[i] * (c.k32 ? c.k32[o] : bf16_bits_to_f32(c.k_tree[o]));
        }
        s = wave_sum(s) * c.scale_log2;
        if (lane == 0) s_anc[k] = s;
      }
      ++k;
    }
  }
  const int na = __popcll(anc);
  // running max over chunk maxima and ancestor scores
  float mx = -INFINITY;
  for (int ch = tid; ch < c.n_chunks; ch += 256)
    mx = fmaxf(mx, c.ml_part[(((int64_t)ch * c.n_kv_heads + g) * c.rows + row) * 2]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  for (int k = 0; k < na; ++k) M = fmaxf(M, s_anc[k]);
  __syncthreads();
  float lsum = 0.f;
  for (int ch = tid; ch < c.n_chunks; ch += 256) {
    const int64_t prow = ((int64_t)ch * c.n_kv_heads + g) * c.rows + row;
    const float w = __builtin_amdgcn_exp2f(c.ml_part[prow * 2] - M) * c.ml_part[prow * 2 + 1];
    s_w[ch] = w;
    lsum += w;
  }
  lsum = wave_sum(lsum);
  if (lane == 0) s_red[wave] = lsum;
  __syncthreads();
  float L = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  for (int k = 0; k < na; ++k) L += __builtin_amdgcn_exp2f(s_anc[k] - M);

  // weighted sum of the chunk outputs: PARTS threads per dim, fixed order
  const int j = tid % D, part = tid / D;
  float acc = 0.f;
#pragma unroll 8
  for (int ch = part; ch < c.n_chunks; ch += PARTS) {
    const int64_t prow = ((int64_t)ch * c.n_kv_heads + g) * c.rows + row;
    acc += s_w[ch] * c.o_part[prow * D + j];
  }
  s_acc[part][j] = acc;
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) o += s_acc[q][j];
    int k = 0;
    for (int a = 0; a < t.n; ++a) {
      if (!((anc >> a) & 1ull)) continue;
      const int64_t vo = ((int64_t)a * c.n_kv_heads + g) * D + j;
      o += __builtin_amdgcn_exp2f(s_anc[k++] - M) * (c.v32 ? c.v32[vo] : bf16_bits_to_f32(c.v_tree[vo]));
    }
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

int attention_max_chunks(int n_kv_heads) { return (512 + n_kv_heads - 1) / n_kv_heads; }

AttnPlan plan_attention(int n_nodes, int n_q_heads, int n_kv_heads, int head_dim, int prefix_len) {
  (void)head_dim;
  AttnPlan a;
  a.rows = n_nodes * (n_q_heads / n_kv_heads);
  const int rt = (a.rows + 15) / 16;
  if (rt <= 16) {
    a.qpw = 1;
    a.waves = rt < 8 ? 8 : rt;
  } else {
    a.qpw = (rt + 7) / 8;
    a.waves = 8;
  }
  // ~512 blocks over (chunk, KV head), chunks a multiple of the LDS tile
  int chunk = (int)(((int64_t)prefix_len * n_kv_heads + 511) / 512);
  chunk = ((chunk + KT - 1) / KT) * KT;
  if (chunk < KT) chunk = KT;
  a.chunk = chunk;
  a.n_chunks = prefix_len > 0 ? (prefix_len + chunk - 1) / chunk : 0;
  return a;
}

template <int D, int QPW>
static void launch_partial(const AttnPlan& plan, const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL((attn_partial_kernel<D, QPW>), dim3(plan.n_chunks, p.n_kv_heads),
                     dim3(64 * plan.waves), 0, s, p);
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
