// Split-K consumers: the int4 GEMM leaves each block's share of
// a panel as a partial tile; these kernels add the shares of every output in
// contributor order (deterministic) and apply the epilogue the projection
// needs.  Doing the reduction here, after the GEMM has finished, needs no
// synchronisation between the GEMM's blocks.
#include "internal.h"

namespace lucev {

// Sum of the contributors of output feature column fl (of panel pnl) for
// node n, added in contributor order.  The first CM contributors' loads are
// unconditional (past the last contributor they re-read it and the value is
// dropped by a select), so a caller's loads for several columns can all be
// in flight before the first sum; CM is the GEMM's most contributors per
// panel rounded up to 4, 8 or 16 (kernels are instantiated per CM).
template <int CM>
struct SplitLoads {
  float v[CM];
  const float* src;
  int nc;
  int64_t tile;
};
template <int CM>
__device__ __forceinline__ void split_issue(const SplitOut& so, int pnl, int fl, int n, SplitLoads<CM>& l) {
  const int bf = block_of_unit((int64_t)pnl * so.gu, so.units, so.blocks);
  const int bl = block_of_unit((int64_t)pnl * so.gu + so.gu - 1, so.units, so.blocks);
  l.tile = (int64_t)so.tile_n * so.tile_f;
  l.src = so.part + (int64_t)pnl * so.c_max * l.tile + (int64_t)n * so.tile_f + fl;
  l.nc = bl - bf + 1;
#pragma unroll
  for (int c = 0; c < CM; ++c) l.v[c] = l.src[min(c, l.nc - 1) * l.tile];
}
template <int CM>
__device__ __forceinline__ float split_finish(const SplitLoads<CM>& l) {
  float y = 0.f;
#pragma unroll
  for (int c = 0; c < CM; ++c) y += c < l.nc ? l.v[c] : 0.f;
  for (int c = CM; c < l.nc; ++c) y += l.src[c * l.tile];
  return y;
}

// launch a consumer kernel template instantiated for the GEMM's contributor count
#define LUCEV_SPLIT_LAUNCH(KERNEL, GRID, BLOCK, SO, ...)                                        \
  do {                                                                                         \
    if ((SO).c_max <= 4)                                                                       \
      hipLaunchKernelGGL(KERNEL<4>, GRID, BLOCK, 0, s, SO, __VA_ARGS__);                       \
    else if ((SO).c_max <= 8)                                                                  \
      hipLaunchKernelGGL(KERNEL<8>, GRID, BLOCK, 0, s, SO, __VA_ARGS__);                       \
    else                                                                                       \
      hipLaunchKernelGGL(KERNEL<16>, GRID, BLOCK, 0, s, SO, __VA_ARGS__);                      \
  } while (0)

// ------------------------------------------------------------ QKV + RoPE
// One block per (panel, node), one thread per panel row (at most 256).  Packed rows of a
// head tile 16i..16i+15 hold dims [8i, 8i+8) and [d/2 + 8i, d/2 + 8i + 8), so
// a rotate-half RoPE pair is rows fl and fl ^ 8 of the same tile.
template <int CM>
__global__ __launch_bounds__(256) void qkv_finish_kernel(SplitOut so, EpiArgs e) {
  __shared__ float s_y[256];
  const int pnl = blockIdx.x, n = blockIdx.y;
  const int fl = threadIdx.x;
  const int hd = e.head_dim;
  const int64_t n_out = (int64_t)(e.n_q_heads + 2 * e.n_kv_heads) * hd;
  const int64_t prow = (int64_t)pnl * so.tile_f + fl;
  const bool ok = prow < n_out;
  SplitLoads<CM> ld;
  split_issue(so, pnl, fl, n, ld);
  s_y[fl] = ok ? split_finish(ld) : 0.f;
  __syncthreads();
  if (!ok) return;
  const int head = (int)(prow / hd);
  const int r = (int)(prow % hd);
  const int ti = r / 16, loc = r % 16;
  const int j = loc < 8 ? 8 * ti + loc : hd / 2 + 8 * ti + (loc - 8);
  float val = s_y[fl];
  if (head < e.n_q_heads + e.n_kv_heads) {
    const float partner = s_y[fl ^ 8];
    const int jj = j < hd / 2 ? j : j - hd / 2;
    // angle in fp64, reduced to [-pi, pi] before the fp32 sin / cos
    const double th = (double)e.pos[n] * e.inv_freq[jj];
    const double two_pi = 6.283185307179586476925286766559;
    const double rr = th - two_pi * rint(th / two_pi);
    float cs, sn;
    sincosf((float)rr, &sn, &cs);
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

hipError_t launch_qkv_finish(const SplitOut& so, const EpiArgs& e, int n, hipStream_t s) {
  if (so.tile_f > 256 || so.tile_f % 32) return hipErrorInvalidValue;
  LUCEV_SPLIT_LAUNCH(qkv_finish_kernel, dim3(so.panels, n), dim3(so.tile_f), so, e);
  return hipGetLastError();
}

// ------------------------------------------------------------ SwiGLU
// One block per (panel, group of nodes).  Packed tiles (2i, 2i+1) of a panel
// are the gate and up rows [16i, 16i + 16) of the same FFN unit.
constexpr int kSwiNodes = 4;  // nodes per block

template <int CM>
__global__ __launch_bounds__(256) void swiglu_finish_kernel(SplitOut so, uint16_t* __restrict__ m, int ffn, int n) {
  __shared__ float s_y[kSwiNodes][256];
  const int pnl = blockIdx.x, n0 = blockIdx.y * kSwiNodes;
  const int fl = threadIdx.x;
  const int64_t n_out = 2 * (int64_t)ffn;
  const bool ok = (int64_t)pnl * so.tile_f + fl < n_out;
  SplitLoads<CM> ld[kSwiNodes];
#pragma unroll
  for (int k = 0; k < kSwiNodes; ++k) split_issue(so, pnl, fl, min(n0 + k, n - 1), ld[k]);
#pragma unroll
  for (int k = 0; k < kSwiNodes; ++k) s_y[k][fl] = (ok && n0 + k < n) ? split_finish(ld[k]) : 0.f;
  __syncthreads();
  // thread fl < tile_f / 2 forms row fl of the panel's FFN units for every node
  if (fl >= so.tile_f / 2) return;
  const int a = fl / 16, r = fl % 16;
  const int64_t row = ((int64_t)pnl * (so.tile_f / 32) + a) * 16 + r;
  if (2 * row >= n_out) return;
#pragma unroll
  for (int k = 0; k < kSwiNodes; ++k) {
    const int node = n0 + k;
    if (node >= n) break;
    const float gt = s_y[k][(2 * a) * 16 + r];
    const float up = s_y[k][(2 * a + 1) * 16 + r];
    const float mv = gt / (1.0f + expf(-gt)) * up;
    // the down projection reads the hi rows only (its weights are rounded
    // once to fp16): no lo row is written
    m[(int64_t)(2 * node) * ffn + row] = f32_to_f16_bits(mv);
  }
}

hipError_t launch_swiglu_finish(const SplitOut& so, uint16_t* m, int ffn, int n, hipStream_t s) {
  if (so.tile_f > 256 || so.tile_f % 32) return hipErrorInvalidValue;
  LUCEV_SPLIT_LAUNCH(swiglu_finish_kernel, dim3(so.panels, (n + kSwiNodes - 1) / kSwiNodes), dim3(so.tile_f), so, m,
                     ffn, n);
  return hipGetLastError();
}

// ------------------------------------------------------------ residual
// One block per (panel, node), x += y.
template <int CM>
__global__ __launch_bounds__(256) void resid_finish_kernel(SplitOut so, float* resid, int hidden) {
  const int pnl = blockIdx.x, n = blockIdx.y;
  const int fl = threadIdx.x;
  const int64_t f = (int64_t)pnl * so.tile_f + fl;
  if (f >= hidden) return;
  float* r = resid + (int64_t)n * hidden + f;
  SplitLoads<CM> ld;
  split_issue(so, pnl, fl, n, ld);
  const float x = *r;
  *r = x + split_finish(ld);
}

hipError_t launch_resid_finish(const SplitOut& so, float* resid, int hidden, int n, hipStream_t s) {
  if (so.tile_f > 256) return hipErrorInvalidValue;
  LUCEV_SPLIT_LAUNCH(resid_finish_kernel, dim3(so.panels, n), dim3(so.tile_f), so, resid, hidden);
  return hipGetLastError();
}

// ------------------------------------------------------------ lm_head
// One block per (panel, group of nodes), one thread per panel row: the
// logits (bf16, if asked for) and the panel's top-2 per node, reduced
// lane-pairwise in each wave and then over the waves in wave order.
constexpr int kLogNodes = 4;  // nodes per block

template <int CM>
__global__ __launch_bounds__(256) void logits_finish_kernel(SplitOut so, uint16_t* __restrict__ logits,
                                                            int64_t vocab, f32x4* __restrict__ cand, int n) {
  __shared__ float s_v1[kLogNodes][4], s_v2[kLogNodes][4];
  __shared__ int s_i1[kLogNodes][4];
  const int pnl = blockIdx.x, n0 = blockIdx.y * kLogNodes;
  const int fl = threadIdx.x, lane = fl & 63, wave = fl >> 6;
  const int64_t f = (int64_t)pnl * so.tile_f + fl;
  const bool ok = f < vocab;
  SplitLoads<CM> ld[kLogNodes];
#pragma unroll
  for (int k = 0; k < kLogNodes; ++k) split_issue(so, pnl, fl, min(n0 + k, n - 1), ld[k]);
#pragma unroll
  for (int k = 0; k < kLogNodes; ++k) {
    const int node = n0 + k;
    const float y = split_finish(ld[k]);
    if (logits && ok && node < n) logits[(int64_t)node * vocab + f] = f32_to_bf16_bits(y);
    float v1 = ok ? y : -INFINITY, v2 = -INFINITY;
    int i1 = ok ? (int)f : 0x7fffffff;
    wave_top2(v1, i1, v2);
    if (lane == 0) {
      s_v1[k][wave] = v1;
      s_v2[k][wave] = v2;
      s_i1[k][wave] = i1;
    }
  }
  __syncthreads();
  if (fl < kLogNodes && n0 + fl < n) {
    float v1 = s_v1[fl][0], v2 = s_v2[fl][0];
    int i1 = s_i1[fl][0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) merge_top2(v1, i1, v2, s_v1[fl][w], s_i1[fl][w], s_v2[fl][w]);
    cand[(int64_t)pnl * n + n0 + fl] = f32x4{v1, __int_as_float(i1), v2, 0.f};
  }
}

hipError_t launch_logits_finish(const SplitOut& so, uint16_t* logits, int64_t vocab, f32x4* cand, int n,
                                hipStream_t s) {
  if (so.tile_f > 256 || so.tile_f % 64) return hipErrorInvalidValue;
  LUCEV_SPLIT_LAUNCH(logits_finish_kernel, dim3(so.panels, (n + kLogNodes - 1) / kLogNodes), dim3(so.tile_f), so,
                     logits, vocab, cand, n);
  return hipGetLastError();
}

}  // namespace lucev
