// RMSNorm, the greedy-acceptance finalisation and a fill kernel.
#include "internal.h"

namespace lucev {

// u = x / sqrt(mean(x^2) + eps) * g, one block per row, fp16 output for the
// next projection (pre-norm decoder layer).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int hidden,
                                                      const uint16_t* __restrict__ g, float eps,
                                                      uint16_t* __restrict__ out, int ld_out) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const float* xr = x + (int64_t)row * hidden;
  float ss = 0.f;
  for (int i = threadIdx.x * 4; i < hidden; i += 256 * 4) {
    const float4 v = *reinterpret_cast<const float4*>(xr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rinv = 1.0f / sqrtf(tot / (float)hidden + eps);
  for (int i = threadIdx.x; i < hidden; i += 256)
    out[(int64_t)row * ld_out + i] = f32_to_f16_bits(xr[i] * rinv * bf16_bits_to_f32(g[i]));
}

hipError_t launch_rmsnorm(const float* x, int n, int hidden, const uint16_t* g, float eps,
                          uint16_t* out_f16, int ld_out, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(n), dim3(256), 0, s, x, hidden, g, eps, out_f16, ld_out);
  return hipGetLastError();
}

// Top-2 merge: best value, its index (lowest on exact ties) and the runner-up
// (a tie at the top makes the runner-up equal to the best).
__device__ __forceinline__ void merge_top2(float& v1, int& i1, float& v2, float b1, int bi, float b2) {
  if (b1 > v1 || (b1 == v1 && bi < i1)) {
    v2 = fmaxf(v1, b2);
    v1 = b1;
    i1 = bi;
  } else {
    v2 = fmaxf(v2, b1);
  }
}

// One block per node reduces the lm_head candidates to the greedy token and
// the top1 - top2 gap; the last block to finish walks the tree.  Acceptance
// is greedy ("Lucebox: 추측 디코딩과 전용 커널로 ...", section "Lucebox 설치
// 및 실행": temperature 0): node i is accepted when its parent is and its
// drafted token equals the parent's greedy token; the kept path ends at the
// deepest accepted node, lowest index on ties, and commits the accepted
// drafts plus the greedy token at the path's end.
__global__ __launch_bounds__(256) void finalize_kernel(const f32x4* __restrict__ cand, int n_fg,
                                                       int stride, TreeArgs t, int32_t* argmax,
                                                       float* gap, int32_t* path, int32_t* path_len,
                                                       int32_t* committed, uint32_t* counter) {
  __shared__ float s1[256], s2[256];
  __shared__ int si[256];
  __shared__ int is_last;
  const int node = blockIdx.x;
  const int tid = threadIdx.x;
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = 0x7fffffff;
  for (int f = tid; f < n_fg; f += 256) {
    const f32x4 c = cand[(int64_t)f * stride + node];
    merge_top2(v1, i1, v2, c[0], __float_as_int(c[1]), c[2]);
  }
  s1[tid] = v1;
  s2[tid] = v2;
  si[tid] = i1;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) {
      float a1 = s1[tid], a2 = s2[tid];
      int ai = si[tid];
      merge_top2(a1, ai, a2, s1[tid + w], si[tid + w], s2[tid + w]);
      s1[tid] = a1;
      s2[tid] = a2;
      si[tid] = ai;
    }
    __syncthreads();
  }
  if (tid == 0) {
    argmax[node] = si[0];
    if (gap) gap[node] = s1[0] - s2[0];
    __threadfence();
    const unsigned prev = atomicAdd(counter, 1u);
    is_last = prev == (unsigned)(t.n - 1);
  }
  __syncthreads();
  if (!is_last || tid != 0) return;
  __threadfence();
  const int n = t.n;
  bool acc[kMaxNodes];
  int am[kMaxNodes];
  for (int i = 0; i < n; ++i) am[i] = __hip_atomic_load(argmax + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  acc[0] = true;
  int end = 0;
  for (int i = 1; i < n; ++i) {
    const int pr = t.parent[i];
    acc[i] = acc[pr] && t.token[i] == am[pr];
    if (acc[i] && t.pos[i] > t.pos[end]) end = i;  // pos = prefix_len + depth
  }
  int len = 0;
  int rev[kMaxNodes];
  for (int j = end; j >= 0; j = t.parent[j]) rev[len++] = j;
  for (int k = 0; k < len; ++k) path[k] = rev[len - 1 - k];
  for (int k = len; k < n; ++k) path[k] = -1;
  for (int k = 1; k < len; ++k) committed[k - 1] = t.token[rev[len - 1 - k]];
  committed[len - 1] = am[end];
  for (int k = len; k < n; ++k) committed[k] = -1;
  *path_len = len;
  atomicExch(counter, 0u);
}

hipError_t launch_finalize(const f32x4* cand, int n_fg, int cand_stride, const TreeArgs& t,
                           int32_t* argmax, float* gap, int32_t* path, int32_t* path_len,
                           int32_t* committed, uint32_t* counter, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(t.n), dim3(256), 0, s, cand, n_fg, cand_stride, t,
                     argmax, gap, path, path_len, committed, counter);
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

}  // namespace lucev
