// Storage and vector types of the shard kernels, usable from host code.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace tp
