// RMSNorm into the GEMM operand, greedy-acceptance finalisation and a fill kernel.
#include "internal.h"

namespace lucev {

// RMSNorm of one row per block into the GEMM operand: u = x * g / sqrt(mean(x^2)
// + eps), written as fp16 rows 2i (hi) and, when the GEMM reads it, 2i+1
// (lo = u - hi).  The row is
// read once into registers (all loads in flight together); the sum of
// squares is reduced in a fixed order.
constexpr int kNormThreads = 512;
constexpr int kNormMaxPer = 4;  // float4 per thread: rows up to 512 * 16 = 8192 wide

__global__ __launch_bounds__(kNormThreads) void norm_hilo_kernel(const float* __restrict__ x, int hidden,
                                                                 const uint16_t* __restrict__ g, float eps,
                                                                 uint16_t* __restrict__ out, int write_lo) {
  __shared__ float red[kNormThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* xr = x + (int64_t)row * hidden;
  float4 v[kNormMaxPer];
  uint2 gw[kNormMaxPer];
#pragma unroll
  for (int k = 0; k < kNormMaxPer; ++k) {
    const int i = (tid + k * kNormThreads) * 4;
    const bool ok = i < hidden;
    v[k] = ok ? *reinterpret_cast<const float4*>(xr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    gw[k] = ok ? *reinterpret_cast<const uint2*>(g + i) : make_uint2(0u, 0u);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kNormMaxPer; ++k) s += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
  s = wave_sum(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += red[w];
  const float rinv = 1.0f / sqrtf(tot / (float)hidden + eps);
  uint16_t* hi = out + (int64_t)(2 * row) * hidden;
  uint16_t* lo = hi + hidden;
#pragma unroll
  for (int k = 0; k < kNormMaxPer; ++k) {
    const int i = (tid + k * kNormThreads) * 4;
    if (i >= hidden) break;
    const float u[4] = {v[k].x * rinv * bf16_bits_to_f32(gw[k].x & 0xFFFFu),
                        v[k].y * rinv * bf16_bits_to_f32(gw[k].x >> 16),
                        v[k].z * rinv * bf16_bits_to_f32(gw[k].y & 0xFFFFu),
                        v[k].w * rinv * bf16_bits_to_f32(gw[k].y >> 16)};
    uint16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f16 hh = (f16)u[e];
      h[e] = __builtin_bit_cast(uint16_t, hh);
      l[e] = f32_to_f16_bits(u[e] - (float)hh);
    }
    *reinterpret_cast<uint2*>(hi + i) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
    if (write_lo)
      *reinterpret_cast<uint2*>(lo + i) = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
  }
}

hipError_t launch_norm_hilo(const float* x, int n, int hidden, const uint16_t* g, float eps,
                            uint16_t* out, bool write_lo, hipStream_t s) {
  hipLaunchKernelGGL(norm_hilo_kernel, dim3(n), dim3(kNormThreads), 0, s, x, hidden, g, eps, out,
                     write_lo ? 1 : 0);
  return hipGetLastError();
}

// One block: merge the lm_head panels' candidates into the greedy token and
// top1 - top2 gap of every node, then walk the tree in one wave (node i on
// lane i).  Acceptance is greedy ("Lucebox: 추측 디코딩과 전용 커널로 ...",
// section "Lucebox 설치 및 실행": temperature 0): a node is accepted when
// every node on its root path drafted the greedy token of its parent; the kept
// path ends at the deepest accepted node, lowest index on ties, and commits
// the accepted drafts plus the greedy token at the path's end.
__global__ __launch_bounds__(1024) void finalize_kernel(const f32x4* __restrict__ cand, int n_cand,
                                                        TreeArgs t, int32_t* argmax, float* gap,
                                                        int32_t* path, int32_t* path_len,
                                                        int32_t* committed) {
  // the candidate list of every node split over 1024 / n parts, so all
  // threads load (a few candidates each, all in flight), then the parts of a
  // node merged pairwise in log2(parts) rounds (the merge is associative and
  // commutative, so the tree does not change the result)
  __shared__ float s1[1024], s2[1024];
  __shared__ int si[1024];
  const int tid = threadIdx.x;
  const int n = t.n;
  const int parts = 1024 / n;
  const int node = tid % n, part = tid / n;
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = 0x7fffffff;
  if (part < parts) {
#pragma unroll 16
    for (int c = part; c < n_cand; c += parts) {
      const f32x4 v = cand[(int64_t)c * n + node];
      merge_top2(v1, i1, v2, v[0], __float_as_int(v[1]), v[2]);
    }
    s1[part * n + node] = v1;
    s2[part * n + node] = v2;
    si[part * n + node] = i1;
  }
  int half = 1;
  while (half < parts) half <<= 1;
  for (half >>= 1; half >= 1; half >>= 1) {
    __syncthreads();
    if (part < half && part + half < parts) {
      const int o = (part + half) * n + node;
      merge_top2(v1, i1, v2, s1[o], si[o], s2[o]);
      s1[part * n + node] = v1;
      s2[part * n + node] = v2;
      si[part * n + node] = i1;
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  int am = 0;
  if (lane < n) {
    v1 = s1[lane];
    v2 = s2[lane];
    i1 = si[lane];
    am = i1;
    argmax[lane] = am;
    if (gap) gap[lane] = v1 - v2;
  }
  if (!path) return;  // a plain projection: no tree to walk
  // acceptance walk
  const int par = lane < n ? t.parent[lane] : 0;
  const int tok = lane < n ? t.token[lane] : 0;
  const int am_par = __shfl(am, par < 0 ? 0 : par, 64);
  const bool match = lane == 0 || (lane < n && tok == am_par);
  const uint64_t mm = __ballot(match);
  const uint64_t anc = lane < n ? t.anc[lane] : 0ull;
  const bool acc = lane < n && ((anc & ~mm) == 0ull);
  const int depth = __popcll(anc) - 1;
  const int key = (int)wave_max((float)(acc ? (depth << 8) | (255 - lane) : -1));
  const int end = 255 - (key & 255);
  const uint64_t anc_end = __shfl(anc, end, 64);
  const int am_end = __shfl(am, end, 64);
  const int len = __popcll(anc_end);
  // path position p holds the p-th ancestor of `end` in index order (on a
  // root path, index order is depth order); every output written once
  uint64_t x = anc_end;
  for (int i = 0; i < lane && x; ++i) x &= x - 1ull;
  const int nd = (lane < len && x) ? (__ffsll((long long)x) - 1) : 0;
  const int nxt = __shfl(nd, lane < 63 ? lane + 1 : 63, 64);
  const int tok_nxt = __shfl(tok, nxt, 64);
  if (lane < n) {
    path[lane] = lane < len ? nd : -1;
    committed[lane] = lane + 1 < len ? tok_nxt : (lane + 1 == len ? am_end : -1);
  }
  if (lane == 0) *path_len = len;
}

hipError_t launch_finalize(const f32x4* cand, int n_cand, const TreeArgs& t, int32_t* argmax,
                           float* gap, int32_t* path, int32_t* path_len, int32_t* committed,
                           hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, s, cand, n_cand, t, argmax, gap,
                     path, path_len, committed);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(u32x4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

// ------------------------------------------------------------ streaming read
// One read of a buffer with non-temporal 16-byte loads, four per thread per
// step and every CU busy: the rate a kernel that streams that many bytes can
// reach.  The loads are folded into one word so they are not dropped; sink is
// written only if the fold hits one fixed value.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* sink) {
  uint32_t acc = 0;
  const int64_t step = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024; base < n16; base += step) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t want = (n16 + 1023) / 1024;
  const int blocks = (int)(want < 1 ? 1 : (want > 2048 ? 2048 : want));
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

// Commit of the accepted path: block (j, KV head, layer), one thread per dim.
// Path position j holds node path[j] at depth j (RoPE position prefix_len +
// j); its key row goes to K token prefix_len + j and its value to column
// prefix_len + j of the dim-major V.  Positions past *path_len do nothing.
__global__ __launch_bounds__(128) void commit_kernel(CommitArgs a) {
  const int j = blockIdx.x, g = blockIdx.y, l = blockIdx.z, t = threadIdx.x;
  if (j >= *a.path_len) return;
  const int node = a.path[j];
  if (node < 0 || node >= a.n) return;
  const int64_t src = ((int64_t)node * a.n_kv_heads + g) * a.head_dim + t;
  const int64_t tok = a.prefix_len + j;
  a.kc[l][((int64_t)g * a.cap + tok) * a.head_dim + t] = a.kt[l][src];
  a.vc[l][((int64_t)g * a.head_dim + t) * a.cap + tok] = a.vt[l][src];
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t s) {
  if (a.head_dim > 128 || a.n_layers < 1 || a.n_layers > kMaxCommitLayers) return hipErrorInvalidValue;
  hipLaunchKernelGGL(commit_kernel, dim3(a.n, a.n_kv_heads, a.n_layers), dim3(a.head_dim), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ device
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
    cached[dev] = cus;
  }
  return cached[dev];
}

}  // namespace lucev
