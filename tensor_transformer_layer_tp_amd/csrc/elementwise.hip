// Bandwidth-bound helpers: RMSNorm, the rank-partial reduce, the RoPE table.
#include "common.h"

namespace tp {

namespace {

// The cache length and its overflow flag, written in stream order (a kernel,
// so that a captured graph records no memset node).
__global__ void set_len_kernel(int* dlen, int len) {
    if (threadIdx.x == 0) {
        dlen[0] = len;
        dlen[1] = 0;
    }
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
    v = wave_sum_dpp(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// bf16 pair <-> floats
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf(float a, float b) {
    return (uint32_t)f2bf_bits(a) | ((uint32_t)f2bf_bits(b) << 16);
}

// n = x / sqrt(mean(x^2) + eps) * g, one row per work-group, fp32 arithmetic,
// bf16 result rounded to nearest even.  Thread t owns the 4-value groups
// t + 256 j of the row (8-byte loads, a wave's load covering 512 contiguous
// bytes) and sums the squares of its groups in order; reduce_norm_bf16_kernel
// uses the same ownership and order, so the two agree bit for bit.  With
// MAXJ > 0 the row (at most 1024 * MAXJ values) is read once and kept in
// registers; MAXJ = 0 reads it twice, for any width.  Requires n % 4 == 0.
template <int MAXJ>
__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const bf16* __restrict__ x,
                                                           const bf16* __restrict__ g,
                                                           bf16* __restrict__ out, int n, float eps) {
    __shared__ float red[4];
    const bf16* xr = x + (long long)blockIdx.x * n;
    bf16* orow = out + (long long)blockIdx.x * n;
    const int nq = n / 4;
    float ss = 0.f;
    if constexpr (MAXJ > 0) {
        uint2 v[MAXJ], w[MAXJ];
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            const int q = min((int)threadIdx.x + 256 * j, nq - 1);   // clamped: issued and in bounds
            v[j] = *(const uint2*)(xr + 4 * q);
            w[j] = *(const uint2*)(g + 4 * q);
        }
#pragma unroll
        for (int j = 0; j < MAXJ; ++j)
            if ((int)threadIdx.x + 256 * j < nq) {
                const float f0 = lo_bf(v[j].x), f1 = hi_bf(v[j].x), f2 = lo_bf(v[j].y), f3 = hi_bf(v[j].y);
                ss += f0 * f0;
                ss += f1 * f1;
                ss += f2 * f2;
                ss += f3 * f3;
            }
        const float rs = rsqrtf(block_sum_256(ss, red) / (float)n + eps);
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            const int q = threadIdx.x + 256 * j;
            if (q < nq) {
                uint2 o;
                o.x = pack_bf(lo_bf(v[j].x) * rs * lo_bf(w[j].x), hi_bf(v[j].x) * rs * hi_bf(w[j].x));
                o.y = pack_bf(lo_bf(v[j].y) * rs * lo_bf(w[j].y), hi_bf(v[j].y) * rs * hi_bf(w[j].y));
                *(uint2*)(orow + 4 * q) = o;
            }
        }
    } else {
        for (int q = threadIdx.x; q < nq; q += 256) {
            const uint2 v = *(const uint2*)(xr + 4 * q);
            const float f0 = lo_bf(v.x), f1 = hi_bf(v.x), f2 = lo_bf(v.y), f3 = hi_bf(v.y);
            ss += f0 * f0;
            ss += f1 * f1;
            ss += f2 * f2;
            ss += f3 * f3;
        }
        const float rs = rsqrtf(block_sum_256(ss, red) / (float)n + eps);
        for (int q = threadIdx.x; q < nq; q += 256) {
            const uint2 v = *(const uint2*)(xr + 4 * q);
            const uint2 w = *(const uint2*)(g + 4 * q);
            uint2 o;
            o.x = pack_bf(lo_bf(v.x) * rs * lo_bf(w.x), hi_bf(v.x) * rs * hi_bf(w.x));
            o.y = pack_bf(lo_bf(v.y) * rs * lo_bf(w.y), hi_bf(v.y) * rs * hi_bf(w.y));
            *(uint2*)(orow + 4 * q) = o;
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

// The reduce and the next stage's RMSNorm in one pass, one row of n values
// per work-group: out = bf16(sum_r parts[r] + residual) exactly as
// reduce_kernel stores it (fp32 adds in rank order, then the residual, then
// RNE), and nout = bf16(out * rsqrt(mean(out^2) + eps) * g) exactly as
// rmsnorm_bf16_kernel<MAXJ> computes it from the stored out (same 4-value
// group ownership, same order of the sum of squares), so the fused pass
// equals the two separate launches bit for bit.  Each partial is read with
// one 16-byte load per lane, a wave covering 1 KB of contiguous fp32; the
// row's bf16 values stay in registers between the two halves.
// n % 4 == 0, n <= 1024 * MAXJ.
template <int TT, int MAXJ>
__global__ __launch_bounds__(256) void reduce_norm_bf16_kernel(Parts parts, int t, const bf16* __restrict__ residual,
                                                               bf16* __restrict__ out, const bf16* __restrict__ g,
                                                               bf16* __restrict__ nout, int n, float eps) {
    __shared__ float red[4];
    const long long row0 = (long long)blockIdx.x * n;
    const int nq = n / 4;
    uint2 hv[MAXJ];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
        const int q = threadIdx.x + 256 * j;
        if (q < nq) {
            const long long e = row0 + 4LL * q;
            f32x4 s;
            if constexpr (TT > 0) {
                f32x4 v[TT];
#pragma unroll
                for (int r = 0; r < TT; ++r) v[r] = __builtin_nontemporal_load((const f32x4*)(parts.p[r] + e));
                s = v[0];
#pragma unroll
                for (int r = 1; r < TT; ++r) s += v[r];
            } else {
                s = __builtin_nontemporal_load((const f32x4*)(parts.p[0] + e));
                for (int r = 1; r < t; ++r) s += __builtin_nontemporal_load((const f32x4*)(parts.p[r] + e));
            }
            if (residual != nullptr) {
                const uint2 rv = *(const uint2*)(residual + e);
                s[0] += lo_bf(rv.x);
                s[1] += hi_bf(rv.x);
                s[2] += lo_bf(rv.y);
                s[3] += hi_bf(rv.y);
            }
            uint2 h;
            h.x = pack_bf(s[0], s[1]);
            h.y = pack_bf(s[2], s[3]);
            *(uint2*)(out + e) = h;
            hv[j] = h;
            const float f0 = lo_bf(h.x), f1 = hi_bf(h.x), f2 = lo_bf(h.y), f3 = hi_bf(h.y);
            ss += f0 * f0;
            ss += f1 * f1;
            ss += f2 * f2;
            ss += f3 * f3;
        }
    }
    const float rs = rsqrtf(block_sum_256(ss, red) / (float)n + eps);
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
        const int q = threadIdx.x + 256 * j;
        if (q < nq) {
            const uint2 w = *(const uint2*)(g + 4LL * q);
            uint2 o;
            o.x = pack_bf(lo_bf(hv[j].x) * rs * lo_bf(w.x), hi_bf(hv[j].x) * rs * hi_bf(w.x));
            o.y = pack_bf(lo_bf(hv[j].y) * rs * lo_bf(w.y), hi_bf(hv[j].y) * rs * hi_bf(w.y));
            *(uint2*)(nout + row0 + 4LL * q) = o;
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

__global__ void zero_ints_kernel(int* p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

}  // namespace

void zero_ints(int* p, int n, hipStream_t st) {
    if (n <= 0) return;
    hipLaunchKernelGGL(zero_ints_kernel, dim3(std::min((n + 255) / 256, 1024)), dim3(256), 0, st, p, n);
}

void rope_turns(double* rev, int d, float theta, hipStream_t st) {
    hipLaunchKernelGGL(rope_turns_kernel, dim3(1), dim3(64), 0, st, rev, d, (double)theta);
}

void set_kv_len(int* dlen, int len, hipStream_t st) {
    hipLaunchKernelGGL(set_len_kernel, dim3(1), dim3(64), 0, st, dlen, len);
}

void rmsnorm_bf16(const bf16* x, const bf16* g, bf16* out, int rows, int n, float eps, hipStream_t st) {
    if (rows <= 0 || n <= 0) return;
    if (n <= 1024 * 4)
        hipLaunchKernelGGL(rmsnorm_bf16_kernel<4>, dim3(rows), dim3(256), 0, st, x, g, out, n, eps);
    else if (n <= 1024 * 8)
        hipLaunchKernelGGL(rmsnorm_bf16_kernel<8>, dim3(rows), dim3(256), 0, st, x, g, out, n, eps);
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

bool reduce_norm_bf16(const float* const* parts, int t, const bf16* residual, bf16* out, const bf16* g, bf16* nout,
                      int rows, int n, float eps, hipStream_t st) {
    if (n % 4 || n > 1024 * 8) return false;   // the caller takes the two separate launches
    if (rows <= 0) return true;
    Parts P;
    for (int r = 0; r < 64; ++r) P.p[r] = r < t ? parts[r] : nullptr;
    // the same group ownership as rmsnorm_bf16 (MAXJ 4 up to 4096 values, else 8)
#define TP_RN(TT, MC) hipLaunchKernelGGL((reduce_norm_bf16_kernel<TT, MC>), dim3(rows), dim3(256), 0, st, P, t, residual, \
                                         out, g, nout, n, eps)
#define TP_RN_T(MC)                         \
    switch (t) {                            \
        case 1: TP_RN(1, MC); break;        \
        case 2: TP_RN(2, MC); break;        \
        case 4: TP_RN(4, MC); break;        \
        case 8: TP_RN(8, MC); break;        \
        default: TP_RN(0, MC); break;       \
    }
    if (n <= 1024 * 4) {
        TP_RN_T(4)
    } else {
        TP_RN_T(8)
    }
#undef TP_RN_T
#undef TP_RN
    return true;
}

void rope_table(float* cos_t, float* sin_t, double* rev, int npos, int d, float theta, hipStream_t st) {
    long long total = (long long)npos * (d / 2);
    int blocks = (int)std::min<long long>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, st, cos_t, sin_t, rev, npos, d, (double)theta);
}

}  // namespace tp
