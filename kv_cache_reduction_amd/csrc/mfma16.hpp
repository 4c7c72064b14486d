// Operands of the 32x32x16 bf16 MFMA (8 bf16 per lane) built from 4-element
// halves, for the GEMM and the many-query kernels.
#pragma once

#include "common.hpp"

namespace slim {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Elements 0-3 from a, 4-7 from b.
__device__ __forceinline__ bf16x8_t join_bf16x8(s16x4 a, s16x4 b) {
  return __builtin_bit_cast(bf16x8_t, (s16x8)__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace slim
