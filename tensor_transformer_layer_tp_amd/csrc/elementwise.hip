// Bandwidth-bound helpers: RMSNorm, the rank-partial reduce, the RoPE table.
#include "kernels.h"

namespace tp {

namespace {

__device__ __forceinline__ float block_sum_256(float v, float* red) {
    v = wave_sum_dpp(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// n = x / sqrt(mean(x^2) + eps) * g, one row per work-group, fp32 arithmetic,
// bf16 result rounded to nearest even.  Requires n % 8 == 0.  With MAXC > 0
// the row (at most 2048 * MAXC elements) is read once and kept in registers;
// MAXC = 0 reads it twice, for any width.
template <int MAXC>
__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const bf16* __restrict__ x,
                                                           const bf16* __restrict__ g,
                                                           bf16* __restrict__ out, int n, float eps) {
    __shared__ float red[4];
    const bf16* xr = x + (long long)blockIdx.x * n;
    bf16* orow = out + (long long)blockIdx.x * n;
    const int nc = n / 8;
    float ss = 0.f;
    if constexpr (MAXC > 0) {
        u16x8 v[MAXC], w[MAXC];
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            const int c = min((int)threadIdx.x + 256 * i, nc - 1);   // clamped: issued and in bounds
            v[i] = *(const u16x8*)(xr + c * 8);
            w[i] = *(const u16x8*)(g + c * 8);
        }
#pragma unroll
        for (int i = 0; i < MAXC; ++i)
            if ((int)threadIdx.x + 256 * i < nc)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = bfbits2f(v[i][e]);
                    ss += f * f;
                }
        const float rs = rsqrtf(block_sum_256(ss, red) / (float)n + eps);
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            const int c = threadIdx.x + 256 * i;
            if (c < nc) {
                u16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = f2bf_bits(bfbits2f(v[i][e]) * rs * bfbits2f(w[i][e]));
                *(u16x8*)(orow + c * 8) = o;
            }
        }
    } else {
        for (int c = threadIdx.x; c < nc; c += 256) {
            u16x8 v = *(const u16x8*)(xr + c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float f = bfbits2f(v[e]);
                ss += f * f;
            }
        }
        const float rs = rsqrtf(block_sum_256(ss, red) / (float)n + eps);
        for (int c = threadIdx.x; c < nc; c += 256) {
            u16x8 v = *(const u16x8*)(xr + c * 8);
            u16x8 w = *(const u16x8*)(g + c * 8);
            u16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = f2bf_bits(bfbits2f(v[e]) * rs * bfbits2f(w[e]));
            *(u16x8*)(orow + c * 8) = o;
        }
    }
}

__global__ __launch_bounds__(256) void rmsnorm_f32_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ g,
                                                          float* __restrict__ out, int n, float eps) {
    __shared__ float red[4];
    const float* xr = x + (long long)blockIdx.x * n;
    float* orow = out + (long long)blockIdx.x * n;
    float ss = 0.f;
    for (int c = threadIdx.x; c < n; c += 256) ss += xr[c] * xr[c];
    const float rs = rsqrtf(block_sum_256(ss, red) / (float)n + eps);
    for (int c = threadIdx.x; c < n; c += 256) orow[c] = xr[c] * rs * g[c];
}

struct Parts {
    const float* p[64];
};

// out = (sum_r parts[r]) + residual, fp32 in rank order, stored as bf16 or fp32.
// TT > 0: t == TT is known at compile time, so the t partial loads and the
// residual load of an element go out together before any add (a loop over
// a run-time t waits for each load in turn, which is the whole duration of
// a decode-sized reduce).  The sum is the same rank-order sum either way.
template <bool BF16_OUT, int TT>
__global__ __launch_bounds__(256) void reduce_kernel(Parts parts, int t, const void* __restrict__ residual,
                                                     void* __restrict__ out, long long n) {
    const long long n4 = n >> 2;
    const long long stride = (long long)gridDim.x * 256;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n4; i += stride) {
        f32x4 s;
        if constexpr (TT > 0) {
            // the residual is loaded with the partials (from a valid dummy address when
            // there is none) and the sum with it selected afterwards, so no load waits
            // behind a branch; selecting, not adding zero, keeps a -0 sum intact
            const bool hr = residual != nullptr;
            f32x4 rf;
            if constexpr (BF16_OUT) {
                const uint2 rv = *(const uint2*)((const uint16_t*)(hr ? residual : (const void*)parts.p[0]) + i * 4);
                rf = (f32x4){__uint_as_float(rv.x << 16), __uint_as_float(rv.x & 0xffff0000u),
                             __uint_as_float(rv.y << 16), __uint_as_float(rv.y & 0xffff0000u)};
            } else {
                rf = *(const f32x4*)((const float*)(hr ? residual : (const void*)parts.p[0]) + i * 4);
            }
            f32x4 v[TT];
#pragma unroll
            for (int r = 0; r < TT; ++r) v[r] = *(const f32x4*)(parts.p[r] + i * 4);
            s = v[0];
#pragma unroll
            for (int r = 1; r < TT; ++r) s += v[r];
            const f32x4 sr = s + rf;
            s = hr ? sr : s;
            if constexpr (BF16_OUT) {
                uint2 ov;
                ov.x = (uint32_t)f2bf_bits(s[0]) | ((uint32_t)f2bf_bits(s[1]) << 16);
                ov.y = (uint32_t)f2bf_bits(s[2]) | ((uint32_t)f2bf_bits(s[3]) << 16);
                *(uint2*)((uint16_t*)out + i * 4) = ov;
            } else {
                *(f32x4*)((float*)out + i * 4) = s;
            }
            continue;
        } else {
            // streamed once: non-temporal loads keep the partials from displacing
            // the residual and the output in the caches
            s = __builtin_nontemporal_load((const f32x4*)(parts.p[0] + i * 4));
            for (int r = 1; r < t; ++r) s += __builtin_nontemporal_load((const f32x4*)(parts.p[r] + i * 4));
        }
        if (BF16_OUT) {
            if (residual) {
                const uint16_t* rp = (const uint16_t*)residual + i * 4;
                uint2 rv = *(const uint2*)rp;
                s[0] += __uint_as_float(rv.x << 16);
                s[1] += __uint_as_float(rv.x & 0xffff0000u);
                s[2] += __uint_as_float(rv.y << 16);
                s[3] += __uint_as_float(rv.y & 0xffff0000u);
            }
            uint2 ov;
            ov.x = (uint32_t)f2bf_bits(s[0]) | ((uint32_t)f2bf_bits(s[1]) << 16);
            ov.y = (uint32_t)f2bf_bits(s[2]) | ((uint32_t)f2bf_bits(s[3]) << 16);
            *(uint2*)((uint16_t*)out + i * 4) = ov;
        } else {
            if (residual) s += *(const f32x4*)((const float*)residual + i * 4);
            *(f32x4*)((float*)out + i * 4) = s;
        }
    }
    // scalar tail (n % 4 elements), handled by the first threads of block 0
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const long long i = n4 * 4 + threadIdx.x;
        float s = parts.p[0][i];
        for (int r = 1; r < t; ++r) s += parts.p[r][i];
        if (BF16_OUT) {
            if (residual) s += bfbits2f(((const uint16_t*)residual)[i]);
            ((uint16_t*)out)[i] = f2bf_bits(s);
        } else {
            if (residual) s += ((const float*)residual)[i];
            ((float*)out)[i] = s;
        }
    }
}

// All-gather on one device: out = rank-order concatenation of t pieces of
// `units` 16-byte vectors each (pieces and out 16-byte aligned).
struct Pieces {
    const u32x4* p[64];
};

__global__ __launch_bounds__(256) void gather_kernel(Pieces pieces, int t, long long units, u32x4* __restrict__ out) {
    const long long total = units * t;
    const long long stride = (long long)gridDim.x * 256;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += stride) {
        const int r = (int)(i / units);
        out[i] = pieces.p[r][i - (long long)r * units];
    }
}

// cos/sin of p * theta^(-2i/d) for p < npos, i < d/2, evaluated in double.
__global__ void rope_table_kernel(float* cos_t, float* sin_t, double* rev, int npos, int d, double theta) {
    const int half = d / 2;
    const long long total = (long long)npos * half;
    for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
        const int p = (int)(idx / half), i = (int)(idx % half);
        const double inv = pow(theta, -2.0 * i / (double)d);
        if (p == 0) rev[i] = inv * 0.15915494309189535;   // theta_i / (2 pi): turns per position
        const double a = (double)p * inv;
        cos_t[idx] = (float)cos(a);
        sin_t[idx] = (float)sin(a);
    }
}

// theta^(-2i/d) / (2 pi) for i < d/2: the rotation per position in turns
__global__ void rope_turns_kernel(double* rev, int d, double theta) {
    const int i = threadIdx.x;
    if (i < d / 2) rev[i] = pow(theta, -2.0 * i / (double)d) * 0.15915494309189535;
}

}  // namespace

void rope_turns(double* rev, int d, float theta, hipStream_t st) {
    hipLaunchKernelGGL(rope_turns_kernel, dim3(1), dim3(64), 0, st, rev, d, (double)theta);
}

void rmsnorm_bf16(const bf16* x, const bf16* g, bf16* out, int rows, int n, float eps, hipStream_t st) {
    if (rows <= 0 || n <= 0) return;
    if (n <= 2048 * 2)
        hipLaunchKernelGGL(rmsnorm_bf16_kernel<2>, dim3(rows), dim3(256), 0, st, x, g, out, n, eps);
    else if (n <= 2048 * 4)
        hipLaunchKernelGGL(rmsnorm_bf16_kernel<4>, dim3(rows), dim3(256), 0, st, x, g, out, n, eps);
    else
        hipLaunchKernelGGL(rmsnorm_bf16_kernel<0>, dim3(rows), dim3(256), 0, st, x, g, out, n, eps);
}

void rmsnorm_f32(const float* x, const float* g, float* out, int rows, int n, float eps, hipStream_t st) {
    if (rows <= 0) return;
    hipLaunchKernelGGL(rmsnorm_f32_kernel, dim3(rows), dim3(256), 0, st, x, g, out, n, eps);
}

void all_gather(const void* const* pieces, int t, long long piece_bytes, void* out, hipStream_t st) {
    if (piece_bytes <= 0) return;
    Pieces P;
    for (int r = 0; r < 64; ++r) P.p[r] = r < t ? (const u32x4*)pieces[r] : nullptr;
    const long long units = piece_bytes / 16;
    const int blocks = (int)std::min<long long>(std::max<long long>((units * t + 255) / 256, 1), 256LL * 8);
    hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(256), 0, st, P, t, units, (u32x4*)out);
}

void partial_reduce(const float* const* parts, int t, const void* residual, void* out, long long n,
                    int bf16_out, hipStream_t st) {
    if (n <= 0) return;
    Parts P;
    for (int r = 0; r < 64; ++r) P.p[r] = r < t ? parts[r] : nullptr;
    long long n4 = n >> 2;
    int blocks = (int)std::min<long long>(std::max<long long>((n4 + 255) / 256, 1), 256LL * 8);
#define TP_RED(BO, TT) hipLaunchKernelGGL((reduce_kernel<BO, TT>), dim3(blocks), dim3(256), 0, st, P, t, residual, out, n)
    // the all-loads-first kernels are for reductions that one pass of the grid covers
    // (decode sizes); a long grid-stride loop streams better with one load at a time
    const int tt = n4 <= (long long)blocks * 256 ? t : 0;
    if (bf16_out) {
        switch (tt) {
            case 1: TP_RED(true, 1); break;
            case 2: TP_RED(true, 2); break;
            case 4: TP_RED(true, 4); break;
            case 8: TP_RED(true, 8); break;
            default: TP_RED(true, 0); break;
        }
    } else {
        switch (tt) {
            case 1: TP_RED(false, 1); break;
            case 2: TP_RED(false, 2); break;
            case 4: TP_RED(false, 4); break;
            case 8: TP_RED(false, 8); break;
            default: TP_RED(false, 0); break;
        }
    }
#undef TP_RED
}

void rope_table(float* cos_t, float* sin_t, double* rev, int npos, int d, float theta, hipStream_t st) {
    long long total = (long long)npos * (d / 2);
    int blocks = (int)std::min<long long>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, st, cos_t, sin_t, rev, npos, d, (double)theta);
}

}  // namespace tp
