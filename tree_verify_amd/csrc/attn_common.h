// Pieces shared by the tree-attention kernels (bf16 and int8 prefix).
#pragma once

#include "internal.h"

namespace lucev {

constexpr int KT = 64;  // prefix tokens per LDS tile

// Two fp32 values as bf16 hi (nearest) and lo (the nearest bf16 of the
// remainder): about 16 significant bits.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(a - ha), (__bf16)(b - hb)});
}

}  // namespace lucev
