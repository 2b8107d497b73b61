// fp32 variant of the shard kernels (small layers computed in full precision).
//
// Same contracts as the bf16 path -- C = A * B^T with the same epilogues and
// the same packed weight layout, causal attention with grouped KV heads --
// on plain FMA arithmetic.  These kernels serve correctness at fp32; the
// bf16 MFMA kernels are the throughput path.
#include "common.h"

namespace tp {

namespace {

constexpr int T = 64, TK = 16;

// 64x64 output tile, 256 threads, thread (ty, tx) owns rows ty + 16 i and
// columns tx + 16 j (i, j < 4): columns j and j + 2 are the two 32-column
// halves of the tile's 64-column group (RoPE / SwiGLU partners).
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, long long lda,
                                                       const float* __restrict__ B, long long ldb, int M, int N,
                                                       int K, Epilogue epi) {
    __shared__ float As[TK][T + 1];
    __shared__ float Bs[TK][T + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) apply_len_update(epi.len);
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += TK) {
        for (int i = tid; i < T * TK; i += 256) {
            const int r = i / TK, kk = i % TK;
            const int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
            As[kk][r] = (gm < M && gk < K) ? A[(long long)gm * lda + gk] : 0.f;
            Bs[kk][r] = (gn < N && gk < K) ? B[(long long)gn * ldb + gk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + ty + 16 * i;
        if (row >= M) continue;
        if constexpr (MODE == EPI_F32 || MODE == EPI_STORE || MODE == EPI_GELU) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + tx + 16 * j;
                if (col >= N) continue;
                float v = acc[i][j];
                if (MODE == EPI_GELU) v = gelu_erf_f(v);
                ((float*)epi.out)[(long long)row * epi.ldo + col] = v;
            }
        } else if constexpr (MODE == EPI_SWIGLU) {
            if (n0 >= N) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float g = acc[i][j], u = acc[i][j + 2];
                ((float*)epi.out)[(long long)row * epi.ldo + (n0 >> 1) + tx + 16 * j] = silu_f(g) * u;
            }
        } else {  // EPI_QKV
            if (n0 >= N) continue;
            const QKVDest& q = epi.qkv;
            const int d = q.d, half = d >> 1;
            const int qcols = q.hl * d, kcols = q.kvl * d;
            const int region = n0 < qcols ? 0 : (n0 < qcols + kcols ? 1 : 2);
            const int base = region == 0 ? 0 : (region == 1 ? qcols : qcols + kcols);
            const int head = (n0 - base) / d;
            const int b = row / q.S, s = row % q.S;
            const int pos = q.pos0 + s;
            float* dst = region == 0 ? (float*)q.q + (((long long)b * q.hl + head) * q.S + s) * d
                                     : (float*)(region == 1 ? q.k : q.v) +
                                           (((long long)b * q.kvl + head) * q.ld_seq + pos) * d;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int i1 = 32 * (((n0 - base) % d) >> 6) + tx + 16 * j;
                float y1 = acc[i][j], y2 = acc[i][j + 2];
                if (region < 2 && q.rope_cos != nullptr) {
                    const float c = q.rope_cos[(long long)pos * half + i1];
                    const float sn = q.rope_sin[(long long)pos * half + i1];
                    const float a = y1;
                    y1 = a * c - y2 * sn;
                    y2 = y2 * c + a * sn;
                }
                dst[i1] = y1;
                dst[i1 + half] = y2;
            }
        }
    }
}

// One work-group per (query, head, batch): scores of every visible key in
// LDS, softmax with work-group reductions, then o = P V.
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, float* __restrict__ O, int hl,
                                                       int kvl, int Sq, int q_pos0, int ld_seq, int d, float scale) {
    extern __shared__ float sm[];
    float* sq = sm;          // [d]
    float* sp = sm + 128;    // [nk]
    __shared__ float red[4];
    const int qi = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
    const int kvh = head / (hl / kvl);
    const int nk = q_pos0 + qi + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* qp = Q + (((long long)b * hl + head) * Sq + qi) * d;
    for (int i = tid; i < d; i += 256) sq[i] = qp[i];
    __syncthreads();
    const float* Kb = K + ((long long)b * kvl + kvh) * ld_seq * d;
    const float* Vb = V + ((long long)b * kvl + kvh) * ld_seq * d;
    float mx = -INFINITY;
    for (int k = tid; k < nk; k += 256) {
        float s = 0.f;
        for (int e = 0; e < d; ++e) s += sq[e] * Kb[(long long)k * d + e];
        s *= scale;
        sp[k] = s;
        mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.f;
    for (int k = tid; k < nk; k += 256) {
        const float p = expf(sp[k] - mx);
        sp[k] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    sum = red[0] + red[1] + red[2] + red[3];
    for (int e = tid; e < d; e += 256) {
        float a = 0.f;
        for (int k = 0; k < nk; ++k) a += sp[k] * Vb[(long long)k * d + e];
        O[((long long)b * Sq + qi) * hl * d + (long long)head * d + e] = a / sum;
    }
}

}  // namespace

void gemm_f32(const float* A, long long lda, const float* B, long long ldb, int M, int N, int K,
              const Epilogue& epi, hipStream_t st) {
    dim3 g(cdiv(N, T), cdiv(M, T)), b(256);
    switch (epi.mode) {
        case EPI_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_F32>, g, b, 0, st, A, lda, B, ldb, M, N, K, epi); break;
        case EPI_QKV: hipLaunchKernelGGL(gemm_f32_kernel<EPI_QKV>, g, b, 0, st, A, lda, B, ldb, M, N, K, epi); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, g, b, 0, st, A, lda, B, ldb, M, N, K, epi); break;
        case EPI_GELU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_GELU>, g, b, 0, st, A, lda, B, ldb, M, N, K, epi); break;
        default: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, g, b, 0, st, A, lda, B, ldb, M, N, K, epi); break;
    }
}

void attn_f32(const float* Q, const float* K, const float* V, float* O, int B, int hl, int kvl, int Sq,
              int q_pos0, int ld_seq, int d, hipStream_t st) {
    if (B <= 0 || Sq <= 0) return;
    const size_t lds = (128 + (size_t)(q_pos0 + Sq)) * sizeof(float);
    hipLaunchKernelGGL(attn_f32_kernel, dim3(Sq, hl, B), dim3(256), lds, st, Q, K, V, O, hl, kvl, Sq, q_pos0,
                       ld_seq, d, (float)(1.0 / sqrt((double)d)));
}

}  // namespace tp
