// Device twin of the seeded input generator in synth/__init__.py: the same
// Philox4x64-10 streams and the same inverse-CDF tables, so large synthetic
// workloads are filled in device memory with values bit-identical to the
// CPU generator.  Input generation only; none of the method's arithmetic.
//
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of
//   (x0, x1, x2, x3) -> (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0))
// with the key bumped by the Weyl constants (W0, W1) before rounds 2..10.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
    const uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
    const uint64_t x1 = c[1], x3 = c[3];
    c[0] = hi1 ^ x1 ^ k0;
    c[1] = lo1;
    c[2] = hi0 ^ x3 ^ k1;
    c[3] = lo0;
  }
}

// the 8 32-bit words of Philox block b (low half of each 64-bit word first)
__device__ __forceinline__ void block_words(uint64_t k0, uint64_t k1, uint64_t b, uint32_t w[8]) {
  uint64_t c[4] = {b, 0, 0, 0};
  philox4x64_10(c, k0, k1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[2 * i] = (uint32_t)c[i];
    w[2 * i + 1] = (uint32_t)(c[i] >> 32);
  }
}

__global__ void raw_words_kernel(uint64_t k0, uint64_t k1, uint64_t start, uint64_t n, uint32_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t wi = start + i;
  uint32_t w[8];
  block_words(k0, k1, wi / 8, w);
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if ((int)(wi % 8) == j) v = w[j];
  out[i] = v;
}

// codes: element e of the tensor is nibble e % 8 of word e / 8; words
// [start_word, start_word + n_words) -> 8 bytes each
__global__ void nibbles_kernel(uint64_t k0, uint64_t k1, uint64_t start_word, uint64_t n_words,
                               uint8_t* out) {
  const uint64_t blk = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;  // Philox block offset
  const uint64_t first = start_word / 8 + blk;
  uint32_t w[8];
  block_words(k0, k1, first, w);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint64_t wi = first * 8 + j;
    if (wi < start_word || wi >= start_word + n_words) continue;
    const uint64_t o = (wi - start_word) * 8;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= ((w[j] >> (4 * e)) & 15u) << (8 * e);
      hi |= ((w[j] >> (4 * (e + 4))) & 15u) << (8 * e);
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(out + o);
    dst[0] = lo;
    dst[1] = hi;
  }
}

__device__ __forceinline__ uint16_t table_lookup(uint32_t u, const uint32_t* thr, int n_thr,
                                                 const uint16_t* vals) {
  int lo = 0, hi = n_thr;  // count of thresholds <= u
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (thr[mid] <= u)
      lo = mid + 1;
    else
      hi = mid;
  }
  return vals[lo];
}

// element i (i < n) reads word start + i; its logical index (i0, i1, i2) over
// dims (., D1, D2) is written at i0*s0 + i1*s1 + i2*s2
__global__ void table_kernel(uint64_t k0, uint64_t k1, uint64_t start, uint64_t n,
                             const uint32_t* thr, int n_thr, const uint16_t* vals, uint16_t* out,
                             int64_t D1, int64_t D2, int64_t s0, int64_t s1, int64_t s2) {
  const uint64_t blk = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t first = start / 8 + blk;
  uint32_t w[8];
  block_words(k0, k1, first, w);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint64_t wi = first * 8 + j;
    if (wi < start || wi >= start + n) continue;
    const uint64_t i = wi - start;
    const int64_t i2 = (int64_t)(i % (uint64_t)D2);
    const int64_t r = (int64_t)(i / (uint64_t)D2);
    const int64_t i1 = r % D1, i0 = r / D1;
    out[i0 * s0 + i1 * s1 + i2 * s2] = table_lookup(w[j], thr, n_thr, vals);
  }
}

inline unsigned blocks_for(uint64_t start, uint64_t n) {
  const uint64_t nb = (start + n + 7) / 8 - start / 8;
  return (unsigned)((nb + 255) / 256);
}

}  // namespace

extern "C" {

int synth_dev_raw_words(uint64_t k0, uint64_t k1, uint64_t start, uint64_t n, uint32_t* out,
                        void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(raw_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, k0, k1, start, n, out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int synth_dev_nibbles(uint64_t k0, uint64_t k1, uint64_t start_word, uint64_t n_words, uint8_t* out,
                      void* stream) {
  if (n_words == 0) return 0;
  hipLaunchKernelGGL(nibbles_kernel, dim3(blocks_for(start_word, n_words)), dim3(256), 0,
                     (hipStream_t)stream, k0, k1, start_word, n_words, out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int synth_dev_table(uint64_t k0, uint64_t k1, uint64_t start, uint64_t n, const uint32_t* thr,
                    int n_thr, const uint16_t* vals, uint16_t* out, int64_t D1, int64_t D2,
                    int64_t s0, int64_t s1, int64_t s2, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(table_kernel, dim3(blocks_for(start, n)), dim3(256), 0, (hipStream_t)stream,
                     k0, k1, start, n, thr, n_thr, vals, out, D1, D2, s0, s1, s2);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
