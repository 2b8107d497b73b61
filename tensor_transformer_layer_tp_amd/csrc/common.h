// Device helpers of the gfx950 shard kernels (included by the .hip sources;
// host code includes kernels.h alone).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tp {

// fp32 -> bf16, round to nearest even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, RNE under the default rounding mode, NaN kept NaN).
__device__ __forceinline__ bf16 f2bf(float f) { return (bf16)f; }
__device__ __forceinline__ uint16_t f2bf_bits(float f) { return __builtin_bit_cast(uint16_t, (bf16)f); }
__device__ __forceinline__ float bf2f(bf16 b) {
    return __uint_as_float(((uint32_t)__builtin_bit_cast(uint16_t, b)) << 16);
}
__device__ __forceinline__ float bfbits2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round a float to the nearest bf16 value, kept as float.
__device__ __forceinline__ float round_bf(float f) { return bfbits2f(f2bf_bits(f)); }

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float gelu_erf_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Sum over the 64 lanes without LDS round trips: DPP quad permutes and row
// mirrors leave each 16-lane row's sum in all its lanes, then the four row
// sums are read out to scalars.  The result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    v += dpp_mov<0x140>(v);   // row_mirror
    const int i = __float_as_int(v);
    return (__int_as_float(__builtin_amdgcn_readlane(i, 0)) + __int_as_float(__builtin_amdgcn_readlane(i, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(i, 32)) + __int_as_float(__builtin_amdgcn_readlane(i, 48)));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    const int i = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(i, 0)), __int_as_float(__builtin_amdgcn_readlane(i, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(i, 32)), __int_as_float(__builtin_amdgcn_readlane(i, 48))));
}

// Address of cache row (sequence b, kv head h, position p) in a contiguous
// cache [B, kvl, ld_seq, d] or, with a block table, in a paged pool.
// The paged form is split in two steps (table read, then the row address)
// so that callers can issue the table reads of several rows together.  The
// block size is a power of two (checked when a paged cache is created).
__device__ __forceinline__ int kv_block(int b, int p, const int* table, int bsz, int max_blocks) {
    const int blk = p >> (31 - __builtin_clz(bsz));
    return table[(long long)b * max_blocks + min(blk, max_blocks - 1)];   // clamped: in bounds
}
__device__ __forceinline__ long long kv_row_in_block(int blk, int h, int p, int kvl, int bsz, int d) {
    return (((long long)blk * kvl + h) * bsz + (p & (bsz - 1))) * d;
}
__device__ __forceinline__ long long kv_row(int b, int h, int p, int kvl, int ld_seq, int d, const int* table,
                                            int bsz, int max_blocks) {
    if (table == nullptr) return (((long long)b * kvl + h) * ld_seq + p) * d;
    return kv_row_in_block(kv_block(b, p, table, bsz, max_blocks), h, p, kvl, bsz, d);
}

__device__ __forceinline__ void apply_len_update(const LenUpdate& u) {
    if (u.ptr == nullptr) return;
    if (u.value >= 0) {
        *u.ptr = u.value;
        if (u.overflow != nullptr) *u.overflow = 0;
    } else {
        const int v = *u.ptr;
        if (v < u.cap) *u.ptr = v + 1;
        else if (u.overflow != nullptr) *u.overflow = 1;
    }
}

// Packed column layout shared by the projection kernels: for Q/K/V heads and
// for the gate/up pair, every 64-row group of the packed weight holds two
// 32-row halves that belong together: (dims i, i + d/2) of one head for the
// rotary embedding, or (gate j, up j) for SwiGLU.  Packed row p of a head's
// block maps to head dim:  g = p / 64, w = p % 64,
//   dim = 32 g + w            (w < 32)
//   dim = d/2 + 32 g + w - 32 (w >= 32).
__host__ __device__ inline int packed_to_dim(int p, int d) {
    int g = p >> 6, w = p & 63;
    return w < 32 ? 32 * g + w : (d >> 1) + 32 * g + (w - 32);
}

}  // namespace tp
