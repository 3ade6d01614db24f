// Shared device-side definitions of the lucev kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lucev {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxNodes = 64;
constexpr int kWave = 64;

// Tree facts derived on the host and passed by value as kernel arguments.
struct TreeArgs {
  int32_t n;
  int32_t pos[kMaxNodes];     // prefix_len + depth
  int32_t parent[kMaxNodes];  // parent[0] = -1
  int32_t token[kMaxNodes];
  uint64_t anc[kMaxNodes];    // bit j: node j is node i or one of its ancestors
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (f16)x);  // round to nearest even
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(f16, (uint16_t)b);
}

// Top-2 merge: best value, its index (lowest on exact ties) and the runner-up
// (a tie at the top makes the runner-up equal to the best).  Associative and
// commutative, so any fixed merge tree gives the same result.
__device__ __forceinline__ void merge_top2(float& v1, int& i1, float& v2, float b1, int bi, float b2) {
  if (b1 > v1 || (b1 == v1 && bi < i1)) {
    v2 = fmaxf(v1, b2);
    v1 = b1;
    i1 = bi;
  } else {
    v2 = fmaxf(v2, b1);
  }
}

// Block barrier that orders LDS only: global loads in flight (prefetches)
// stay in flight across it, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block barrier after direct-to-LDS loads, which the caller has waited for
// with wait_vmcnt: no release fence (one would make the compiler wait for
// every outstanding direct-to-LDS load, including later prefetches); the
// acquire fence keeps the LDS reads that follow below the barrier.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// wait until at most N of this wave's vector-memory operations are in
// flight (vmcnt only; LDS and export counters left alone).  Direct-to-LDS
// loads count here and are not waited for by the compiler.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// max and sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The value of a partner lane within each row of 16 (DPP: quad_perm, half-row
// and row mirrors), with no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each 16

// Sum / max over the 64 lanes, every lane getting the same bits (each step
// combines a lane with a partner that combines the same two values): pairs,
// quads, eights and rows of 16 by DPP, then the four rows by the permlane
// swaps.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_partner<kDppXor1>(v);
  v += dpp_partner<kDppXor2>(v);
  v += dpp_partner<kDppHalfMirror>(v);
  v += dpp_partner<kDppMirror>(v);
  return rows_sum(v);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_partner<kDppXor1>(v));
  v = fmaxf(v, dpp_partner<kDppXor2>(v));
  v = fmaxf(v, dpp_partner<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_partner<kDppMirror>(v));
  return rows_max(v);
}

// Top-2 over the 64 lanes (merge_top2 at every step, so the result is the
// same whatever the pairing): DPP partners within rows of 16, then the
// permlane swaps across rows, which hand each lane its own and its partner's
// triple (in either order; the merge does not care).
template <int CTRL>
__device__ __forceinline__ void top2_dpp_step(float& v1, int& i1, float& v2) {
  merge_top2(v1, i1, v2, dpp_partner<CTRL>(v1),
             __builtin_amdgcn_update_dpp(0, i1, CTRL, 0xF, 0xF, false), dpp_partner<CTRL>(v2));
}
template <bool ROW32>
__device__ __forceinline__ void top2_swap_step(float& v1, int& i1, float& v2) {
  auto sw = [](uint32_t x) {
    if constexpr (ROW32) return __builtin_amdgcn_permlane32_swap(x, x, false, false);
    else return __builtin_amdgcn_permlane16_swap(x, x, false, false);
  };
  const auto a = sw(__float_as_uint(v1)), b = sw((uint32_t)i1), c = sw(__float_as_uint(v2));
  float w1 = __uint_as_float(a[0]), w2 = __uint_as_float(c[0]);
  int j1 = (int)b[0];
  merge_top2(w1, j1, w2, __uint_as_float(a[1]), (int)b[1], __uint_as_float(c[1]));
  v1 = w1;
  i1 = j1;
  v2 = w2;
}
__device__ __forceinline__ void wave_top2(float& v1, int& i1, float& v2) {
  top2_dpp_step<kDppXor1>(v1, i1, v2);
  top2_dpp_step<kDppXor2>(v1, i1, v2);
  top2_dpp_step<kDppHalfMirror>(v1, i1, v2);
  top2_dpp_step<kDppMirror>(v1, i1, v2);
  top2_swap_step<false>(v1, i1, v2);
  top2_swap_step<true>(v1, i1, v2);
}

}  // namespace lucev
