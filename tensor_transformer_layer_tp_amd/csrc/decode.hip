// Decode (one new token per sequence): weight-streaming GEMV and split-KV
// attention over the rank's KV-cache heads.
//
// Decode is a sequence of small steps whose local products are too small to
// keep a GPU busy (clusterbid "When Tensor Parallelism Makes a Small Model
// Slower"): at batch 1..8 every projection reads its weight slice once and
// does ~1 FLOP per byte, so these kernels are organised around streaming
// the weights from HBM with 16-byte coalesced loads, not around MFMA.
#include "common.h"

#include <algorithm>

namespace tp {

namespace {

// The all-reduce's sum in a row-parallel projection's epilogue (EPI_SUM):
// the other ranks' partials and the residual at rows r1 and r1 + 32 of
// sequence b (slot `self` and ranks past t read nothing), ...
__device__ __forceinline__ void sum_load(const Epilogue& epi, int b, int r1, float (&v1)[kSumMaxRanks],
                                         float (&v2)[kSumMaxRanks], float& res1, float& res2, bool on = true) {
    const SumDest& s = epi.sum;
    const long long o = (long long)b * epi.ldo;
#pragma unroll
    for (int j = 0; j < kSumMaxRanks; ++j) {
        const bool ld = on && j < s.t && j != s.self;
        v1[j] = ld ? s.p[j][o + r1] : 0.f;
        v2[j] = ld ? s.p[j][o + r1 + 32] : 0.f;
    }
    const bool hr = on && s.residual != nullptr;
    res1 = hr ? bf2f(s.residual[o + r1]) : 0.f;
    res2 = hr ? bf2f(s.residual[o + r1 + 32]) : 0.f;
}

// ... and h = (sum over ranks, in rank order, of the partials) + residual,
// the order and rounding of the reduce kernel, with this projection's own
// results y1, y2 in slot `self`.
__device__ __forceinline__ void sum_store(const Epilogue& epi, int b, int r1, float y1, float y2,
                                          const float (&v1)[kSumMaxRanks], const float (&v2)[kSumMaxRanks],
                                          float res1, float res2) {
    const SumDest& s = epi.sum;
    float a1 = s.self == 0 ? y1 : v1[0], a2 = s.self == 0 ? y2 : v2[0];
#pragma unroll
    for (int j = 1; j < kSumMaxRanks; ++j)
        if (j < s.t) {
            a1 += j == s.self ? y1 : v1[j];
            a2 += j == s.self ? y2 : v2[j];
        }
    if (s.residual != nullptr) {   // added only when present, so that a -0 sum stays -0
        a1 += res1;
        a2 += res2;
    }
    bf16* out = (bf16*)epi.out + (long long)b * epi.ldo;
    out[r1] = f2bf(a1);
    out[r1 + 32] = f2bf(a2);
}

// Stores output rows r1 and r1 + 32 (partners in one packed 64-row group) of
// sequence b: fp32 partial, bf16 (GELU), SwiGLU of the (gate, up) pair, or
// the rotary embedding of the (i, i + d/2) pair scattered to q and to the
// KV cache at position pos0.
template <int MODE>
__device__ __forceinline__ void pair_store(const Epilogue& epi, int b, int r1, float y1, float y2) {
    const int r2 = r1 + 32;
    if constexpr (MODE == EPI_F32) {
        float* o = (float*)epi.out + (long long)b * epi.ldo;
        o[r1] = y1;
        o[r2] = y2;
    } else if constexpr (MODE == EPI_SUM) {
        float v1[kSumMaxRanks], v2[kSumMaxRanks], res1, res2;
        sum_load(epi, b, r1, v1, v2, res1, res2);
        sum_store(epi, b, r1, y1, y2, v1, v2, res1, res2);
    } else if constexpr (MODE == EPI_STORE || MODE == EPI_GELU) {
        bf16* o = (bf16*)epi.out + (long long)b * epi.ldo;
        o[r1] = f2bf(MODE == EPI_GELU ? gelu_erf_f(y1) : y1);
        o[r2] = f2bf(MODE == EPI_GELU ? gelu_erf_f(y2) : y2);
    } else if constexpr (MODE == EPI_SWIGLU) {
        bf16* o = (bf16*)epi.out + (long long)b * epi.ldo;
        o[(r1 >> 6) * 32 + (r1 & 31)] = f2bf(silu_f(y1) * y2);
    } else {  // EPI_QKV, one token per sequence at position pos0
        const QKVDest& q = epi.qkv;
        const int d = q.d, half = d >> 1;
        const int qcols = q.hl * d, kcols = q.kvl * d;
        const int region = r1 < qcols ? 0 : (r1 < qcols + kcols ? 1 : 2);
        const int base = region == 0 ? 0 : (region == 1 ? qcols : qcols + kcols);
        const int head = (r1 - base) / d;
        const int i1 = 32 * (((r1 - base) % d) >> 6) + (r1 & 31);
        const int pos = q.pos_dev ? *q.pos_dev : q.pos0;
        if (region > 0 && pos >= q.ld_seq) return;   // cache full: nothing to append
        float o1 = y1, o2 = y2;
        if (region < 2 && q.rope_rev != nullptr) {
            // pos * theta_i turns: the fraction, formed in double (exact for any
            // position), goes to the hardware sine and cosine, which take turns;
            // no table, so the decode path needs nothing sized by the cache
            const double a = (double)pos * q.rope_rev[i1];
            const float f = (float)(a - floor(a));
            const float c = __builtin_amdgcn_cosf(f), sn = __builtin_amdgcn_sinf(f);
            o1 = y1 * c - y2 * sn;
            o2 = y2 * c + y1 * sn;
        }
        bf16* dst = region == 0 ? (bf16*)q.q + ((long long)b * q.hl + head) * d
                                : (bf16*)(region == 1 ? q.k : q.v) +
                                      kv_row(b, head, pos, q.kvl, q.ld_seq, d, q.table, q.bsz, q.max_blocks);
        dst[i1] = f2bf(o1);
        dst[i1 + half] = f2bf(o2);
    }
}

// ---------------------------------------------------------------------------
// GEMV: y[b, n] = sum_k W[n, k] * in[b, k] for b < NB, optionally with the
// RMSNorm of x fused in front (in = bf16(x * rsqrt(mean x^2 + eps) * gamma)).
//
// A work-group of T threads owns P row pairs (rows r and r + 32 of one 64-row
// group of the packed weight; see packed_to_dim) so that the RoPE / SwiGLU
// partners meet in one work-group.  Thread t owns the 16-byte K-chunks
// t + T i (i < NI), so the threads sweep each row in contiguous bursts; T is
// the smallest of 64, 128, 256 that covers a row's chunks.  Every weight load
// of the thread is issued first; the norm's sum of squares comes from the
// same x chunks while those loads are in flight (the thread chunks together
// cover all of K, so one work-group reduction gives the whole row's sum).
//
// Weights are bf16 (8 per chunk) or, with W8, OCP E4M3 codes (16 per chunk,
// decoded exactly by the hardware conversion, two per instruction) with one
// fp32 scale per row applied to the finished dot product.
template <int NB, int P, int NI, int MODE, bool NORM, bool W8, int T>
__global__ __launch_bounds__(T) void gemv_kernel(const bf16* __restrict__ x, const bf16* __restrict__ gamma,
                                                 float eps, const void* __restrict__ Wv,
                                                 const float* __restrict__ wscale, int N, int K, Epilogue epi) {
    constexpr int R = 2 * P, NW = T / 64;
    constexpr int CW = W8 ? 16 : 8;      // weights per 16-byte chunk
    constexpr int XC = CW / 8;           // 16-byte activation chunks per weight chunk
    __shared__ float red[NW][R * NB];
    __shared__ float rs_s[NB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (blockIdx.x == 0 && tid == 0) apply_len_update(epi.len);
    const int per_group = 32 / P;
    const int grp = blockIdx.x / per_group, sub = blockIdx.x % per_group;
    const int rbase = 64 * grp + P * sub;   // rows rbase + e and rbase + 32 + e, e < P
    const int KC = K / CW;
    const char* W = (const char*)Wv;
    const long long row_bytes = (long long)K * (W8 ? 1 : 2);

    int cofs[NI];
    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = tid + T * i;
        valid[i] = c < KC;
        cofs[i] = min(c, KC - 1);   // clamped: every load is issued and in bounds
    }
    // Activation (and gain) loads first, then every weight load, and nothing
    // scheduled above the last weight load: the norm below then waits only
    // for the activations (the memory counter retires in issue order) while
    // the weights stream in.  Left to itself the scheduler hoists activation
    // arithmetic between the loads and waits for the activations before the
    // first weight load, which costs one whole memory latency per work-group.
    u16x8 xv[NB][NI][XC];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int h = 0; h < XC; ++h) xv[b][i][h] = *(const u16x8*)(x + (long long)b * K + cofs[i] * CW + 8 * h);
    u16x8 gv[NI][XC];
    if constexpr (NORM) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int h = 0; h < XC; ++h) gv[i][h] = *(const u16x8*)(gamma + cofs[i] * CW + 8 * h);
    }
    // EPI_SUM: the epilogue thread's other-rank partials and residual are
    // loaded before the weights, so that their latency is spent while the
    // weights stream instead of at the end of the work-group
    float sv1[kSumMaxRanks], sv2[kSumMaxRanks], sr1 = 0.f, sr2 = 0.f;
    if constexpr (MODE == EPI_SUM)
        sum_load(epi, tid % NB, rbase + min(tid / NB, P - 1), sv1, sv2, sr1, sr2, tid < P * NB);
    // Weight rows are read once per call: non-temporal loads stream them
    // without displacing the activations and partials from the caches.
    u32x4 wv[R][NI];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const char* wrow = W + (long long)(rbase + (r < P ? r : 32 + r - P)) * row_bytes;
#pragma unroll
        for (int i = 0; i < NI; ++i) wv[r][i] = __builtin_nontemporal_load((const u32x4*)(wrow + 16LL * cofs[i]));
    }
    __builtin_amdgcn_sched_barrier(0);

    float rs[NB];
    if constexpr (NORM) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int h = 0; h < XC; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float f = bfbits2f(xv[b][i][h][e]);
                        ss += valid[i] ? f * f : 0.f;
                    }
            ss = wave_sum_dpp(ss);
            if (lane == 0) red[wave][b] = ss;
        }
        __syncthreads();
        if (tid < NB) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) t += red[w][tid];
            rs_s[tid] = rsqrtf(t / (float)K + eps);
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < NB; ++b) rs[b] = rs_s[b];
    }

    float acc[R][NB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (!valid[i]) continue;
        if constexpr (!W8) {
            // bf16 weights: packed-pair dot products (v_dot2c_f32_bf16) on the
            // weight words as loaded and the activation words (normalised and
            // rounded to bf16 first, as the staged activation of a GEMM is)
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                bf16x2 xp[4];
                if constexpr (NORM) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float f0 = bfbits2f(xv[b][i][0][2 * j]) * rs[b] * bfbits2f(gv[i][0][2 * j]);
                        const float f1 = bfbits2f(xv[b][i][0][2 * j + 1]) * rs[b] * bfbits2f(gv[i][0][2 * j + 1]);
                        xp[j] = (bf16x2){f2bf(f0), f2bf(f1)};
                    }
                } else {
                    // (vector elements are copied to scalars before the bit
                    // casts: a cast of the element expression itself reads
                    // element 0)
                    const u32x4 w = __builtin_bit_cast(u32x4, xv[b][i][0]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t wj = w[j];
                        xp[j] = __builtin_bit_cast(bf16x2, wj);
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t wj = wv[r][i][j];
                        acc[r][b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wj), xp[j], acc[r][b],
                                                                    false);
                    }
            }
            continue;
        }
        float wf[R][CW];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (W8) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[r][i][j], false);
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[r][i][j], true);
                    wf[r][4 * j] = lo[0];
                    wf[r][4 * j + 1] = lo[1];
                    wf[r][4 * j + 2] = hi[0];
                    wf[r][4 * j + 3] = hi[1];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wf[r][2 * j] = __uint_as_float(wv[r][i][j] << 16);
                    wf[r][2 * j + 1] = __uint_as_float(wv[r][i][j] & 0xFFFF0000u);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float xin[CW];
#pragma unroll
            for (int h = 0; h < XC; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float f = bfbits2f(xv[b][i][h][e]);
                    if constexpr (NORM) f = round_bf(f * rs[b] * bfbits2f(gv[i][h][e]));
                    xin[8 * h + e] = f;
                }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int e = 0; e < CW; ++e) acc[r][b] += wf[r][e] * xin[e];
        }
    }

    // reduce: wave sums, then across the waves
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float s = wave_sum_dpp(acc[r][b]);
            if (lane == 0) red[wave][r * NB + b] = s;
        }
    __syncthreads();
    if (tid >= P * NB) return;
    const int e = tid / NB, b = tid % NB;
    const int j2 = (P + e) * NB + b;
    float y1 = 0.f, y2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        y1 += red[w][e * NB + b];
        y2 += red[w][j2];
    }
    if constexpr (W8) {
        y1 *= wscale[rbase + e];
        y2 *= wscale[rbase + 32 + e];
    }
    if constexpr (MODE == EPI_SUM) sum_store(epi, b, rbase + e, y1, y2, sv1, sv2, sr1, sr2);
    else pair_store<MODE>(epi, b, rbase + e, y1, y2);
}

// Per-row E4M3 quantisation of a bf16 matrix [N, K]: one work-group per
// row; scale = max|w| / 448 (1 for a zero row); code = nearest E4M3 value of
// the fp32 quotient w / scale clamped to +-448, ties to the even code.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fminf(fabsf(v), 448.f);
    uint32_t code;
    if (a < 0.015625f) {                       // below 2^-6: subnormal spacing 2^-9
        code = (uint32_t)__builtin_rintf(a * 512.f);   // 0..8; 8 is the smallest normal
    } else {
        const uint32_t ab = __float_as_uint(a);
        uint32_t e = (ab >> 23) - 120;         // biased E4M3 exponent 1..15
        uint32_t m = (ab >> 20) & 7u;
        const uint32_t rem = ab & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) {
            if (++m == 8u) {
                m = 0;
                ++e;
            }
        }
        code = (e << 3) | m;
    }
    return code | sign;
}

__global__ __launch_bounds__(256) void quant_rows_kernel(const bf16* __restrict__ W, int K, uint8_t* __restrict__ Q,
                                                         float* __restrict__ scale) {
    __shared__ float red[4];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bf16* w = W + (long long)row * K;
    float amax = 0.f;
    for (int k = tid; k < K; k += 256) amax = fmaxf(amax, fabsf(bf2f(w[k])));
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax > 0.f ? amax / 448.f : 1.f;
    if (tid == 0) scale[row] = s;
    uint8_t* q = Q + (long long)row * K;
    for (int k = tid; k < K; k += 256) q[k] = (uint8_t)e4m3_code(bf2f(w[k]) / s);
}

// ---------------------------------------------------------------------------
// Split-KV decode attention.  Work-group (chunk, kv head, sequence) takes a
// chunk of cached positions for every query head of the GQA group and
// writes, per head, the chunk's maximum, sum and unnormalised output; a
// second kernel merges the chunks.  Chunks at or past the device-resident
// cache length exit at once (the grid is sized for the capacity).
//
// One query head per KV head (G = 1): chunks of 64 positions; thread = (key,
// quarter of the head dim) for the scores, (8-dim chunk, key group) for P V.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_chunk_mha(const bf16* __restrict__ q, const bf16* __restrict__ K,
                                                         const bf16* __restrict__ V, float* __restrict__ scr,
                                                         int hl, int kvl, const int* __restrict__ len_dev,
                                                         int ld_seq, float scale_log2, const int* __restrict__ table,
                                                         int bsz, int max_blocks) {
    const int G = hl / kvl;
    const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int nchunks = gridDim.x;   // chunk stride of the scratch (sized for ld_seq positions)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    extern __shared__ float sm[];
    float* sq = sm;                 // [G][D]
    float* ss = sm + G * D;         // [G][64]
    const int k0 = chunk * 64;

    // Every load is issued before the cache length arrives: rows are clamped
    // to the capacity (always addressable) and positions at or past the
    // length are masked once it is known.
    constexpr int QD = D / 4;                   // score thread = (key, quarter of the head dim)
    constexpr int DC = D / 8;                   // P V thread = (8-dim chunk, key group)
    constexpr int KG = 256 / DC;
    constexpr int KPG = 64 / KG;
    const int key = tid >> 2, seg = tid & 3;
    const int dc = tid % DC, kg = tid / DC;
    u16x8 kraw[QD / 8], vraw[KPG];
    {
        const bf16* krow = K + kv_row(b, kvh, min(k0 + key, ld_seq - 1), kvl, ld_seq, D, table, bsz, max_blocks);
#pragma unroll
        for (int c = 0; c < QD / 8; ++c) kraw[c] = *(const u16x8*)(krow + seg * QD + c * 8);
    }
#pragma unroll
    for (int i = 0; i < KPG; ++i) {
        const int gk = min(k0 + kg * KPG + i, ld_seq - 1);
        vraw[i] = *(const u16x8*)(V + kv_row(b, kvh, gk, kvl, ld_seq, D, table, bsz, max_blocks) + dc * 8);
    }
    for (int i = tid; i < G * D; i += 256) {
        const int g = i / D, dd = i % D;
        sq[i] = bf2f(q[((long long)b * hl + kvh * G + g) * D + dd]);
    }
    const int len = min(*len_dev + 1, ld_seq);
    if (k0 >= len) return;   // past the cache length: no work (uniform per work-group)
    __syncthreads();

    // scores
    {
        float kf[QD];
#pragma unroll
        for (int c = 0; c < QD / 8; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[c * 8 + e] = bfbits2f(kraw[c][e]);
        for (int g = 0; g < G; ++g) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < QD; ++e) s += kf[e] * sq[g * D + seg * QD + e];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            if (seg == 0) ss[g * 64 + key] = (k0 + key < len) ? s * scale_log2 : -INFINITY;
        }
    }
    __syncthreads();
    // softmax pieces per head: wave w handles heads w, w+4, ...
    float* stat = scr + ((long long)b * hl + kvh * G) * nchunks * (D + 2);
    for (int g = wave; g < G; g += 4) {
        const float s = ss[g * 64 + lane];
        const float m = wave_max_dpp(s);
        const float p = exp2f(s - m);
        const float l = wave_sum_dpp(p);
        ss[g * 64 + lane] = p;
        if (lane == 0) {
            float* st = stat + ((long long)g * nchunks + chunk) * (D + 2);
            st[D] = m;
            st[D + 1] = l;
        }
    }
    __syncthreads();
    // o[g][dim] = sum_key p[g][key] V[key][dim]
    {
        float vf[KPG][8];   // rows past the length (stale cache contents) count as zero
#pragma unroll
        for (int i = 0; i < KPG; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[i][e] = k0 + kg * KPG + i < len ? bfbits2f(vraw[i][e]) : 0.f;
        float* pg = sm + G * D + G * 64;  // [KG][D] partial sums, after sq and ss
        for (int g = 0; g < G; ++g) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
            for (int i = 0; i < KPG; ++i) {
                const float p = ss[g * 64 + kg * KPG + i];   // zero past the length
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += p * vf[i][e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) pg[kg * D + dc * 8 + e] = o[e];
            __syncthreads();
            if (tid < D) {
                float a = 0.f;
                for (int k = 0; k < KG; ++k) a += pg[k * D + tid];
                stat[((long long)g * nchunks + chunk) * (D + 2) + tid] = a;
            }
            __syncthreads();
        }
    }
}

// Query groups (G >= 2): chunks of CH positions and every pass covers all G
// heads at once, so a work-group has three barriers whatever G is:
//  * scores: thread (key, segment) dots its D/SEG dims of the key with every
//    head's query (from LDS) and the SEG threads of a key sum by shuffles;
//  * softmax: wave w takes heads w, w+4, ... (one lane per key);
//  * P V: item (head, 8-dim chunk, key split) sums its keys from the V chunk
//    in LDS; the KS splits of one output are adjacent lanes, summed by
//    shuffles.
template <int D, int CH>
__global__ __launch_bounds__(256) void attn_decode_chunk(const bf16* __restrict__ q, const bf16* __restrict__ K,
                                                         const bf16* __restrict__ V, float* __restrict__ scr,
                                                         int hl, int kvl, const int* __restrict__ len_dev,
                                                         int ld_seq, float scale_log2, const int* __restrict__ table,
                                                         int bsz, int max_blocks) {
    constexpr int SEG = 256 / CH, SD = D / SEG, DC = D / 8;
    static_assert(SD % 8 == 0, "score segment");
    const int G = hl / kvl;
    const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int nchunks = gridDim.x;   // chunk stride of the scratch (sized for ld_seq positions)
    const int k0 = chunk * CH;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    extern __shared__ float sm[];
    float* sq = sm;                              // [G][D] queries
    float* sp = sm + G * D;                      // [G][CH] scores, then probabilities
    bf16* sv = (bf16*)(sp + G * CH);             // [CH][D] values

    // The loads are issued before the cache length arrives: rows are clamped
    // to the capacity (always addressable) and rows at or past the length are
    // masked once it is known.
    const int lenp = *len_dev;
    const bf16* qg = q + ((long long)b * hl + kvh * G) * D;   // the group's heads are adjacent
    const int key = tid / SEG, seg = tid % SEG;
    // every load first (fixed trip counts, clamped addresses), then the LDS writes
    constexpr int VCH = CH * DC / 256;           // 16-byte V chunks per thread
    static_assert(VCH >= 1 && CH * DC % 256 == 0, "V chunk split");
    u16x8 kraw[SD / 8], vraw[VCH], qraw[2];
    {
        const int gk = min(k0 + key, ld_seq - 1);
        const bf16* krow = K + kv_row(b, kvh, gk, kvl, ld_seq, D, table, bsz, max_blocks);
#pragma unroll
        for (int c = 0; c < SD / 8; ++c) kraw[c] = *(const u16x8*)(krow + seg * SD + c * 8);
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
        const int i = tid + 256 * j, kk = i / DC, c = i % DC;
        vraw[j] = *(const u16x8*)(V + kv_row(b, kvh, min(k0 + kk, ld_seq - 1), kvl, ld_seq, D, table, bsz, max_blocks) +
                                  c * 8);
    }
    const int nq8 = G * D / 8;                   // two chunks per thread cover G * D <= 4096
#pragma unroll
    for (int j = 0; j < 2; ++j) qraw[j] = *(const u16x8*)(qg + 8 * min(tid + 256 * j, nq8 - 1));
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
        const int i = tid + 256 * j, kk = i / DC, c = i % DC;
        *(u16x8*)(sv + kk * D + c * 8) = vraw[j];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = tid + 256 * j;
        if (i < nq8)
#pragma unroll
            for (int e = 0; e < 8; ++e) sq[8 * i + e] = bfbits2f(qraw[j][e]);
    }
    for (int i = tid + 512; i < nq8; i += 256) {   // larger query groups
        const u16x8 v = *(const u16x8*)(qg + 8 * i);
#pragma unroll
        for (int e = 0; e < 8; ++e) sq[8 * i + e] = bfbits2f(v[e]);
    }
    const int len = min(lenp + 1, ld_seq);
    if (k0 >= len) return;           // past the cache length: no work (uniform per work-group)
    float kf[SD];
#pragma unroll
    for (int c = 0; c < SD / 8; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[c * 8 + e] = bfbits2f(kraw[c][e]);
    __syncthreads();
    const bool kvalid = k0 + key < len;
    for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < SD; ++e) s += kf[e] * sq[g * D + seg * SD + e];
#pragma unroll
        for (int off = 1; off < SEG; off <<= 1) s += __shfl_xor(s, off, 64);
        if (seg == 0) sp[g * CH + key] = kvalid ? s * scale_log2 : -INFINITY;
    }
    __syncthreads();
    float* stat = scr + ((long long)b * hl + kvh * G) * nchunks * (D + 2);
    for (int g = wave; g < G; g += 4) {
        const float s = lane < CH ? sp[g * CH + lane] : -INFINITY;
        const float m = wave_max_dpp(s);
        const float p = lane < CH ? __builtin_amdgcn_exp2f(s - m) : 0.f;
        const float l = wave_sum_dpp(p);
        if (lane < CH) sp[g * CH + lane] = p;
        if (lane == 0) {
            float* st = stat + ((long long)g * nchunks + chunk) * (D + 2);
            st[D] = m;
            st[D + 1] = l;
        }
    }
    __syncthreads();
    int KS = 1;   // key splits: the largest power of two with G * DC * KS <= 256, at most CH
    while (KS < CH && G * DC * KS * 2 <= 256) KS <<= 1;
    const int kper = CH / KS, total = G * DC * KS;
    for (int base = 0; base < total; base += 256) {
        const int item = base + tid;
        const bool valid = item < total;
        const int ks = item % KS, dc = (item / KS) % DC, g = min(item / (KS * DC), G - 1);
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        if (valid) {
            const int kend = min(kper, len - k0 - ks * kper);   // keys past the length hold no value
            for (int i = 0; i < kend; ++i) {
                const int kk = ks * kper + i;
                const float p = sp[g * CH + kk];
                const u16x8 v = *(const u16x8*)(sv + kk * D + dc * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += p * bfbits2f(v[e]);
            }
        }
        for (int off = 1; off < KS; off <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off, 64);
        if (valid && ks == 0) {
            float* st = stat + ((long long)g * nchunks + chunk) * (D + 2) + dc * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) st[e] = o[e];
        }
    }
}

// Copies prefill K/V rows [B, kvl, S, d] into the pages of a paged pool.
__global__ __launch_bounds__(256) void pages_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v,
                                                    bf16* __restrict__ kpool, bf16* __restrict__ vpool, int B,
                                                    int kvl, int S, int d, const int* __restrict__ table, int bsz,
                                                    int max_blocks) {
    const int dc = d / 8;
    const long long total = (long long)B * kvl * S * dc;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const int c = (int)(i % dc);
        const long long row = i / dc;                 // (b, h, p) row of the contiguous layout
        const int p = (int)(row % S), h = (int)((row / S) % kvl), b = (int)(row / ((long long)S * kvl));
        const long long dst = kv_row(b, h, p, kvl, 0, d, table, bsz, max_blocks) + c * 8;
        *(u16x8*)(kpool + dst) = *(const u16x8*)(k + row * d + c * 8);
        *(u16x8*)(vpool + dst) = *(const u16x8*)(v + row * d + c * 8);
    }
}

// Merge the chunks of one (batch, query head) with NT threads.  The chunk
// maxima are reduced by all threads; the chunk weights exp2(m_c - M) go to
// LDS a tile of 1024 chunks at a time; thread (dim, part) sums the weighted
// outputs of a contiguous share (one of NT / D) of the chunks with eight
// loads in flight, and the parts meet in LDS.  st: the head's chunk records
// (D outputs, max, sum; stride D + 2); lds: MERGE_LDS floats.
constexpr int MERGE_TILE = 1024;
template <int D, int NT>
constexpr int merge_lds_floats() { return MERGE_TILE + NT / 64 + (NT / D) * D; }

template <int D, int NT>
__device__ void merge_head(const float* __restrict__ st, int nchunks, bf16* __restrict__ out, float* lds) {
    constexpr int NW = NT / 64, P = NT / D;
    float* sw = lds;                  // [MERGE_TILE] chunk weights
    float* sred = sw + MERGE_TILE;    // [NW]
    float* spart = sred + NW;         // [P][D]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dim = tid % D, part = tid / D;
    float m = -INFINITY;
    for (int c = tid; c < nchunks; c += NT) m = fmaxf(m, st[(long long)c * (D + 2) + D]);
    m = wave_max_dpp(m);
    if (lane == 0) sred[wave] = m;
    __syncthreads();
    float M = sred[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sred[w]);
    float l = 0.f, acc = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += MERGE_TILE) {
        const int n = min(MERGE_TILE, nchunks - c0);
        __syncthreads();
        for (int c = tid; c < n; c += NT) {
            const float* sc = st + (long long)(c0 + c) * (D + 2);
            const float w = __builtin_amdgcn_exp2f(sc[D] - M);
            sw[c] = w;
            l += w * sc[D + 1];
        }
        __syncthreads();
        const int lo = part * n / P, hi = (part + 1) * n / P;
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        int c = lo;
        for (; c + 8 <= hi; c += 8)
#pragma unroll
            for (int u = 0; u < 8; ++u) a[u] += sw[c + u] * st[(long long)(c0 + c + u) * (D + 2) + dim];
        for (; c < hi; ++c) a[0] += sw[c] * st[(long long)(c0 + c) * (D + 2) + dim];
        acc += ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    }
    spart[part * D + dim] = acc;
    l = wave_sum_dpp(l);
    __syncthreads();
    if (lane == 0) sred[wave] = l;
    __syncthreads();
    if (tid < D) {
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) L += sred[w];
#pragma unroll
        for (int p = 0; p < P; ++p) o += spart[p * D + tid];
        out[tid] = f2bf(o / L);
    }
    __syncthreads();   // the LDS may be reused by the caller
}

template <int D, int NT>
__global__ __launch_bounds__(NT) void attn_decode_combine(const float* __restrict__ scr, bf16* __restrict__ O,
                                                          int hl, int stride, const int* __restrict__ len_dev,
                                                          int ld_seq, int CH) {
    __shared__ float lds[merge_lds_floats<D, NT>()];
    const int head = blockIdx.x, b = blockIdx.y;
    const int nchunks = (min(*len_dev + 1, ld_seq) + CH - 1) / CH;   // chunks written by the chunk kernel
    merge_head<D, NT>(scr + ((long long)b * hl + head) * stride * (D + 2), nchunks,
                      O + ((long long)b * hl + head) * D, lds);
}

// Merge with every load in one round: thread (dim, part) of a (head,
// sequence) work-group of D * P threads owns the chunks c = part + P i
// (at most MAXI of them) and loads their maxima, sums and its dim's
// outputs at once; a block maximum gives the reference M, then each thread
// weights its chunks by exp2(m_c - M) and the parts meet in LDS.  The record
// loads do not wait for the device-resident cache length: they cover every
// record slot the grid has (`stride`, the capacity's chunk count), and the
// length, loaded with them, only decides which of the loaded records count.
template <int D, int P, int MAXI>
__global__ __launch_bounds__(D * P) void attn_decode_merge(const float* __restrict__ scr, bf16* __restrict__ O, int hl,
                                                          int stride, const int* __restrict__ len_dev, int ld_seq,
                                                          int CH) {
    constexpr int NT = D * P, NW = NT / 64;
    __shared__ float sred[NW];
    __shared__ float spart[P][D];
    __shared__ float sl[P];
    const int head = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dim = tid % D, part = tid / D;
    const float* st = scr + ((long long)b * hl + head) * stride * (D + 2);
    float mv[MAXI], lv[MAXI], ov[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int c = min(part + P * i, stride - 1);   // clamped to the record slots: every load in bounds
        const float* r = st + (long long)c * (D + 2);
        mv[i] = r[D];
        lv[i] = r[D + 1];
        ov[i] = r[dim];
    }
    // chunks written by the chunk kernel; the others' slots hold older records
    const int nchunks = (min(*len_dev + 1, ld_seq) + CH - 1) / CH;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < MAXI; ++i)
        if (part + P * i < nchunks) m = fmaxf(m, mv[i]);
    m = wave_max_dpp(m);
    if (lane == 0) sred[wave] = m;
    __syncthreads();
    float M = sred[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sred[w]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int i = 0; i < MAXI; ++i)
        if (part + P * i < nchunks) {
            const float wgt = __builtin_amdgcn_exp2f(mv[i] - M);
            acc += wgt * ov[i];
            lsum += wgt * lv[i];
        }
    spart[part][dim] = acc;
    if (dim == 0) sl[part] = lsum;
    __syncthreads();
    if (part == 0) {
        float o = 0.f, L = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            o += spart[p][dim];
            L += sl[p];
        }
        O[((long long)b * hl + head) * D + dim] = f2bf(o / L);
    }
}

// Split-KV decode attention with the merge in the same launch.  Work-group
// (chunk, query head, sequence) attends one query head (GQA: its KV head is
// head / G, so the G heads of a KV head read the same chunk; the grid's
// chunk count is a multiple of 8, which puts them on one XCD and its L2)
// over CH cached positions: thread (key, segment) dots SD = D / SEG dims of
// its key with the query, the SEG threads of a key sum by shuffles, wave 0
// takes the chunk's softmax pieces, thread (8-dim chunk, key group) sums
// P V over its keys and the groups meet in LDS.  The chunk's record (D
// unnormalised outputs, max, sum) is published with a device-scope release
// and counted on the (sequence, head)'s counter; the work-group that brings
// the count to the number of chunks holding positions merges the head's
// records (device-scope acquire first) and resets the counter for the next
// call.  Chunks at or past the device-resident cache length exit at once,
// uncounted.
template <int D, int CH, bool MERGE>
__global__ __launch_bounds__(256) void attn_decode_fused(const bf16* __restrict__ q, const bf16* __restrict__ K,
                                                         const bf16* __restrict__ V, float* __restrict__ scr,
                                                         int* __restrict__ cnt, bf16* __restrict__ O, int hl, int kvl,
                                                         const int* __restrict__ len_dev, int ld_seq,
                                                         float scale_log2, const int* __restrict__ table, int bsz,
                                                         int max_blocks) {
    constexpr int SEG = 256 / CH, SD = D / SEG;          // score threads per key, dims per score thread
    constexpr int DC = D / 8, KG = 256 / DC, KPG = CH / KG;  // P V thread = (8-dim chunk, key group)
    static_assert(SD % 8 == 0 && SEG <= 64 && KPG >= 1, "chunk shape");
    __shared__ float sq[D];
    __shared__ float sp[CH];
    __shared__ float pg[KG][D];
    __shared__ float mrg[merge_lds_floats<D, 256>()];
    __shared__ int last;
    const int G = hl / kvl;
    const int chunk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
    const int kvh = head / G;
    const int nch = gridDim.x;   // record stride
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int k0 = chunk * CH;
    const int key = tid / SEG, seg = tid % SEG;
    const int dc = tid % DC, kg = tid / DC;
    // every load before the cache length arrives: rows clamped to the capacity
    u16x8 kraw[SD / 8], vraw[KPG], qraw;
    {
        const bf16* krow = K + kv_row(b, kvh, min(k0 + key, ld_seq - 1), kvl, ld_seq, D, table, bsz, max_blocks);
#pragma unroll
        for (int c = 0; c < SD / 8; ++c) kraw[c] = *(const u16x8*)(krow + seg * SD + c * 8);
    }
#pragma unroll
    for (int i = 0; i < KPG; ++i) {
        const int gk = min(k0 + kg * KPG + i, ld_seq - 1);
        vraw[i] = *(const u16x8*)(V + kv_row(b, kvh, gk, kvl, ld_seq, D, table, bsz, max_blocks) + dc * 8);
    }
    qraw = *(const u16x8*)(q + ((long long)b * hl + head) * D + 8 * min(tid, DC - 1));
    const int len = min(*len_dev + 1, ld_seq);
    if (k0 >= len) return;   // no positions in this chunk (uniform per work-group)
    if (tid < DC)
#pragma unroll
        for (int e = 0; e < 8; ++e) sq[8 * tid + e] = bfbits2f(qraw[e]);
    __syncthreads();
    {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < SD / 8; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) s += bfbits2f(kraw[c][e]) * sq[seg * SD + c * 8 + e];
#pragma unroll
        for (int off = 1; off < SEG; off <<= 1) s += __shfl_xor(s, off, 64);
        if (seg == 0) sp[key] = k0 + key < len ? s * scale_log2 : -INFINITY;
    }
    __syncthreads();
    float m = 0.f, l = 0.f;   // the chunk's max and sum (wave 0)
    if (wave == 0) {
        const float sv = lane < CH ? sp[lane] : -INFINITY;
        m = wave_max_dpp(sv);
        const float p = lane < CH ? __builtin_amdgcn_exp2f(sv - m) : 0.f;
        l = wave_sum_dpp(p);
        if (lane < CH) sp[lane] = p;   // zero past the length (exp2 of -inf)
    }
    __syncthreads();
    {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
        for (int i = 0; i < KPG; ++i) {
            const int kk = kg * KPG + i;
            const float p = sp[kk];
            const bool ok = k0 + kk < len;   // rows past the length may hold stale values
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += p * (ok ? bfbits2f(vraw[i][e]) : 0.f);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) pg[kg][dc * 8 + e] = o[e];
    }
    __syncthreads();
    // wave 0 stores the record (D / 64 outputs per lane, then max and sum)
    float* rec = scr + (((long long)b * hl + head) * nch + chunk) * (D + 2);
    if (wave == 0) {
#pragma unroll
        for (int h = 0; h < D / 64; ++h) {
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < KG; ++k) a += pg[k][64 * h + lane];
            rec[64 * h + lane] = a;
        }
        if (lane == 0) {
            rec[D] = m;
            rec[D + 1] = l;
        }
        // release (an L2 write-back) by the one wave that stored the record, so
        // that it is visible device-wide before it is counted; no acquire here:
        // an invalidation would drop the other work-groups' cached K/V lines
        if constexpr (MERGE) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    }
    if constexpr (!MERGE) return;   // a merge launch follows
    __syncthreads();
    const int nact = (len + CH - 1) / CH;   // chunks holding positions
    int* c = cnt + (long long)b * hl + head;
    if (tid == 0) last = atomicAdd(c, 1) == nact - 1;
    __syncthreads();
    if (!last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // every other chunk's record
    merge_head<D, 256>(scr + ((long long)b * hl + head) * nch * (D + 2), nact, O + ((long long)b * hl + head) * D,
                       mrg);
    if (tid == 0) *c = 0;   // the count starts from zero on the next call
}

// ---------------------------------------------------------------------------
// Skinny GEMM for small decode batches (2..64 sequences; the shard uses it
// from 5), split over K.
//
// y[b, n] = sum_k W[n, k] x[b, k] with v_mfma_f32_32x32x16_bf16: the weight
// rows are the A operand (32 rows per tile), the batch the B operand (32
// sequences per column tile, rows past B clamped to B-1 and discarded).
// Work-group (g, z) owns the 64 rows of packed group g and the z-th share of
// K; its 4 waves split that share in groups of 64 k.  Within a group each lane
// reads 64 contiguous bytes of its row: the contraction order is free, so
// half h of the lanes feeds k = 32 h + 8 j + [0, 8) into MFMA step j, for the
// weights and the activations alike.  The waves' sums meet in LDS and go to
// an fp32 scratch [z][b][n]; a second kernel sums the z shares and applies
// the epilogue of the row pair (r, r + 32).
constexpr int SK_ROWS = 64, SK_KG = 64;

template <int NC>
__global__ __launch_bounds__(256) void skinny_kernel(const bf16* __restrict__ x, int B, const bf16* __restrict__ W,
                                                     int N, int K, int ks, float* __restrict__ part) {
    __shared__ float red[4][2][NC][16][65];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * SK_ROWS, kz = blockIdx.y;
    const int G = K / SK_KG, slot = kz * 4 + wave, nslots = ks * 4;
    const int g0 = (int)((long long)G * slot / nslots), g1 = (int)((long long)G * (slot + 1) / nslots);
    const int row = lane & 31, h = lane >> 5;
    const bf16* w0 = W + (long long)(n0 + row) * K + 32 * h;
    const bf16* w1 = w0 + 32LL * K;
    const bf16* xr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) xr[c] = x + (long long)min(32 * c + row, B - 1) * K + 32 * h;

    f32x16 acc[2][NC];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[t][c] = (f32x16){};
    // two k-groups per iteration, all loads issued before the MFMAs (plain
    // loads: a lane reads 64 bytes of a row in four 16-byte loads, and
    // non-temporal ones refetched the line for each, 20-30 % slower); past the
    // wave's last group the second group re-reads it (in bounds) with its
    // activations zeroed, so no branch splits the loads from their use
    for (int g = g0; g < g1; g += 2) {
        const bool two = g + 1 < g1;
        const int ka = g * SK_KG, kb = (two ? g + 1 : g) * SK_KG;
        bf16x8 wf[2][2][4], xf[2][NC][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                wf[0][t][j] = *(const bf16x8*)((t ? w1 : w0) + ka + 8 * j);
                wf[1][t][j] = *(const bf16x8*)((t ? w1 : w0) + kb + 8 * j);
            }
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xf[0][c][j] = *(const bf16x8*)(xr[c] + ka + 8 * j);
                xf[1][c][j] = *(const bf16x8*)(xr[c] + kb + 8 * j);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (!two) xf[1][c][j] = (bf16x8){};
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        acc[t][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[u][t][j], xf[u][c][j], acc[t][c], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[wave][t][c][r][lane] = acc[t][c][r];
    __syncthreads();
    // accumulator register r of lane l holds row 8(r/4) + 4(l/32) + r%4, column l%32
    for (int idx = tid; idx < SK_ROWS * B; idx += 256) {
        const int i = idx & 63, b = idx >> 6;
        const int t = i >> 5, rr = i & 31, c = b >> 5, col = b & 31;
        const int ln = col + 32 * ((rr >> 2) & 1), r = 4 * (rr >> 3) + (rr & 3);
        const float v = red[0][t][c][r][ln] + red[1][t][c][r][ln] + red[2][t][c][r][ln] + red[3][t][c][r][ln];
        part[((long long)kz * B + b) * N + n0 + i] = v;
    }
}

template <int MODE>
__global__ __launch_bounds__(256) void skinny_fixup(const float* __restrict__ part, int ks, int B, int N,
                                                    Epilogue epi) {
    const int npairs = N >> 1;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx == 0) apply_len_update(epi.len);
    if (idx >= B * npairs) return;
    const int b = idx / npairs, p = idx - b * npairs;
    const int r1 = (p >> 5) * 64 + (p & 31);
    float y1 = 0.f, y2 = 0.f;
    for (int z = 0; z < ks; ++z) {
        const float* pz = part + ((long long)z * B + b) * N;
        y1 += pz[r1];
        y2 += pz[r1 + 32];
    }
    pair_store<MODE>(epi, b, r1, y1, y2);
}

int skinny_splits(int N, int K) {
    const int groups = N / SK_ROWS, kgroups = K / SK_KG;
    const int want = (512 + groups - 1) / groups;   // at least ~512 work-groups
    return std::max(1, std::min(want, kgroups / 4));
}

template <int NB, int P, int NI, bool NORM, bool W8, int T>
void gemv_mode(const bf16* x, const bf16* gamma, float eps, const void* W, const float* ws, int N, int K,
               const Epilogue& epi, hipStream_t st) {
    dim3 g(N / (2 * P)), b(T);
    switch (epi.mode) {
        case EPI_F32: hipLaunchKernelGGL((gemv_kernel<NB, P, NI, EPI_F32, NORM, W8, T>), g, b, 0, st, x, gamma, eps, W, ws, N, K, epi); break;
        case EPI_SUM: hipLaunchKernelGGL((gemv_kernel<NB, P, NI, EPI_SUM, NORM, W8, T>), g, b, 0, st, x, gamma, eps, W, ws, N, K, epi); break;
        case EPI_QKV: hipLaunchKernelGGL((gemv_kernel<NB, P, NI, EPI_QKV, NORM, W8, T>), g, b, 0, st, x, gamma, eps, W, ws, N, K, epi); break;
        case EPI_SWIGLU: hipLaunchKernelGGL((gemv_kernel<NB, P, NI, EPI_SWIGLU, NORM, W8, T>), g, b, 0, st, x, gamma, eps, W, ws, N, K, epi); break;
        case EPI_GELU: hipLaunchKernelGGL((gemv_kernel<NB, P, NI, EPI_GELU, NORM, W8, T>), g, b, 0, st, x, gamma, eps, W, ws, N, K, epi); break;
        default: hipLaunchKernelGGL((gemv_kernel<NB, P, NI, EPI_STORE, NORM, W8, T>), g, b, 0, st, x, gamma, eps, W, ws, N, K, epi); break;
    }
}

template <int NB, int NI, bool W8, int T>
void gemv_ni(const bf16* x, const bf16* gamma, float eps, const void* W, const float* ws, int N, int K,
             const Epilogue& epi, hipStream_t st) {
    // 8 rows per work-group keep 8 x NI loads in flight per thread; 4 rows
    // (twice the work-groups) are faster up to N 5504 and for E4M3 rows, and
    // where 8 would leave the thread short of registers
    if constexpr (NI <= 2 && !W8) {
        if (N / 8 >= 1024) {
            if (gamma) gemv_mode<NB, 4, NI, true, W8, T>(x, gamma, eps, W, ws, N, K, epi, st);
            else gemv_mode<NB, 4, NI, false, W8, T>(x, gamma, eps, W, ws, N, K, epi, st);
            return;
        }
    }
    // few rows (the 70B-shaped Q/K/V at t=8: 1280): 2 rows per work-group, so
    // that the grid still spreads evenly over the CUs
    if constexpr (NB == 1) {
        if (N / 4 < 512) {
            if (gamma) gemv_mode<NB, 1, NI, true, W8, T>(x, gamma, eps, W, ws, N, K, epi, st);
            else gemv_mode<NB, 1, NI, false, W8, T>(x, gamma, eps, W, ws, N, K, epi, st);
            return;
        }
    }
    if (gamma) gemv_mode<NB, 2, NI, true, W8, T>(x, gamma, eps, W, ws, N, K, epi, st);
    else gemv_mode<NB, 2, NI, false, W8, T>(x, gamma, eps, W, ws, N, K, epi, st);
}

template <int NB, bool W8>
void gemv_nb(const bf16* x, const bf16* gamma, float eps, const void* W, const float* ws, int N, int K,
             const Epilogue& epi, hipStream_t st) {
    const int kc = K / (W8 ? 16 : 8);   // 16-byte chunks per row (K <= 16384)
    if (kc <= 64) return gemv_ni<NB, 1, W8, 64>(x, gamma, eps, W, ws, N, K, epi, st);
    if (kc <= 128) return gemv_ni<NB, 1, W8, 128>(x, gamma, eps, W, ws, N, K, epi, st);
    switch ((kc + 255) / 256) {
        case 1: gemv_ni<NB, 1, W8, 256>(x, gamma, eps, W, ws, N, K, epi, st); break;
        case 2: gemv_ni<NB, 2, W8, 256>(x, gamma, eps, W, ws, N, K, epi, st); break;
        case 3: gemv_ni<NB, 3, W8, 256>(x, gamma, eps, W, ws, N, K, epi, st); break;
        case 4: gemv_ni<NB, 4, W8, 256>(x, gamma, eps, W, ws, N, K, epi, st); break;
        default: gemv_ni<NB, 8, W8, 256>(x, gamma, eps, W, ws, N, K, epi, st); break;
    }
}

}  // namespace

void gemv_bf16(const bf16* x, int B, const bf16* gamma, float eps, const bf16* W, int N, int K,
               const Epilogue& epi, hipStream_t st) {
    switch (B) {
        case 1: gemv_nb<1, false>(x, gamma, eps, W, nullptr, N, K, epi, st); break;
        case 2: gemv_nb<2, false>(x, gamma, eps, W, nullptr, N, K, epi, st); break;
        case 3: gemv_nb<3, false>(x, gamma, eps, W, nullptr, N, K, epi, st); break;
        default: gemv_nb<4, false>(x, gamma, eps, W, nullptr, N, K, epi, st); break;
    }
}

void gemv_fp8(const bf16* x, const bf16* gamma, float eps, const uint8_t* W, const float* scale, int N, int K,
              const Epilogue& epi, hipStream_t st) {
    gemv_nb<1, true>(x, gamma, eps, W, scale, N, K, epi, st);
}

void quant_rows_e4m3(const bf16* W, int N, int K, uint8_t* Q, float* scale, hipStream_t st) {
    hipLaunchKernelGGL(quant_rows_kernel, dim3(N), dim3(256), 0, st, W, K, Q, scale);
}

size_t skinny_scratch_bytes(int B, int N, int K) {
    return (size_t)skinny_splits(N, K) * B * N * sizeof(float);
}

void skinny_bf16(const bf16* x, int B, const bf16* W, int N, int K, float* part, const Epilogue& epi,
                 hipStream_t st) {
    const int ks = skinny_splits(N, K);
    const dim3 grid(N / SK_ROWS, ks);
    if (B <= 32)
        hipLaunchKernelGGL(skinny_kernel<1>, grid, dim3(256), 0, st, x, B, W, N, K, ks, part);
    else
        hipLaunchKernelGGL(skinny_kernel<2>, grid, dim3(256), 0, st, x, B, W, N, K, ks, part);
    const dim3 fg(cdiv(B * (N >> 1), 256));
    switch (epi.mode) {
        case EPI_F32: hipLaunchKernelGGL(skinny_fixup<EPI_F32>, fg, dim3(256), 0, st, part, ks, B, N, epi); break;
        case EPI_SUM: hipLaunchKernelGGL(skinny_fixup<EPI_SUM>, fg, dim3(256), 0, st, part, ks, B, N, epi); break;
        case EPI_QKV: hipLaunchKernelGGL(skinny_fixup<EPI_QKV>, fg, dim3(256), 0, st, part, ks, B, N, epi); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(skinny_fixup<EPI_SWIGLU>, fg, dim3(256), 0, st, part, ks, B, N, epi); break;
        case EPI_GELU: hipLaunchKernelGGL(skinny_fixup<EPI_GELU>, fg, dim3(256), 0, st, part, ks, B, N, epi); break;
        default: hipLaunchKernelGGL(skinny_fixup<EPI_STORE>, fg, dim3(256), 0, st, part, ks, B, N, epi); break;
    }
}

// Split kernels (the merge a second launch): positions per chunk 64; query
// groups take fewer when 64 leaves fewer than 128 chunk work-groups (few KV
// heads and sequences), down to 16 (32 for d = 64).
int g_decode_chunk = 0;   // 0: automatic; 16, 32, 64: forced
int g_decode_mode = 0;    // 0: automatic; 1: split kernels + merge launch; 2: fused merge;
                          // 3: one-head chunk kernel + merge launch

int split_chunk(int B, int hl, int kvl, int cap, int d) {
    int ch = 64;
    if (hl == kvl) return ch;
    const int lo = d == 128 ? 16 : 32;
    if (g_decode_chunk) return std::max(g_decode_chunk, lo);
    while (ch > lo && (long long)((cap + ch - 1) / ch) * kvl * B < 128) ch >>= 1;
    return ch;
}

struct DecodeAttnPlan {
    bool fused;     // one query head per work-group (attn_decode_fused)
    bool merge_in;  // ... with the merge in the same launch
    int ch;         // positions per chunk
    int nch;        // chunk work-groups per (sequence, head) = record stride
};

// The fused kernel (one query head per work-group) takes 64 positions per
// chunk, halved while the grid would have fewer than 256 work-groups; it is
// used while a head has at most 256 chunks, whose records its last
// work-group merges, and while the workspace's counters cover batch x heads.
DecodeAttnPlan decode_attn_plan(int B, int hl, int kvl, int cap, int d) {
    const int lo = d == 128 ? 16 : 32;
    int ch = 64;
    if (g_decode_chunk)
        ch = std::max(g_decode_chunk, lo);
    else
        while (ch > lo && (long long)((cap + ch - 1) / ch) * hl * B < 256) ch >>= 1;
    const int n = (cap + ch - 1) / ch;
    // With several query heads per KV head, a multiple of 8 chunks puts the
    // heads' work-groups for one chunk on one XCD (its L2 serves the shared
    // K/V rows); one query head per KV head, or a short cache, gains nothing
    // from it and would only launch empty work-groups.
    const int nf = hl / kvl > 1 && n >= 8 ? (n + 7) / 8 * 8 : n;
    const bool fits = (long long)B * hl <= kDecodeCounters;
    if (g_decode_mode == 2 && fits) return {true, true, ch, nf};
    if (g_decode_mode == 0 || g_decode_mode == 3) return {true, false, ch, nf};
    const int chs = split_chunk(B, hl, kvl, cap, d);
    return {false, false, chs, (cap + chs - 1) / chs};
}

void set_decode_chunk(int ch) { g_decode_chunk = ch; }
void set_decode_attn_mode(int mode) { g_decode_mode = mode; }

size_t attn_decode_scratch_bytes(int B, int hl, int kvl, int cap, int d) {
    const DecodeAttnPlan p = decode_attn_plan(B, hl, kvl, cap, d);
    return (size_t)B * hl * p.nch * (d + 2) * sizeof(float);
}

template <int D, int CHT>
void launch_decode_attn(const bf16* q, const bf16* K, const bf16* V, bf16* O, float* scratch, int* counters, int B,
                        int hl, int kvl, const int* len_dev, int ld_seq, const int* table, int bsz, int mb,
                        const DecodeAttnPlan& p, hipStream_t st) {
    const int nchunks = p.nch;
    const int G = hl / kvl;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    if (p.fused && p.merge_in) {
        hipLaunchKernelGGL((attn_decode_fused<D, CHT, true>), dim3(nchunks, hl, B), dim3(256), 0, st, q, K, V,
                           scratch, counters, O, hl, kvl, len_dev, ld_seq, scale_log2, table, bsz, mb);
        return;
    }
    if (p.fused) {
        hipLaunchKernelGGL((attn_decode_fused<D, CHT, false>), dim3(nchunks, hl, B), dim3(256), 0, st, q, K, V,
                           scratch, counters, O, hl, kvl, len_dev, ld_seq, scale_log2, table, bsz, mb);
    } else if (G == 1) {
        // LDS: q [D], scores [64], per-head partial sums [256/(D/8)][D]
        const size_t lds = ((size_t)D + 64 + (size_t)(256 / (D / 8)) * D) * sizeof(float);
        hipLaunchKernelGGL(attn_decode_chunk_mha<D>, dim3(nchunks, kvl, B), dim3(256), lds, st, q, K, V, scratch, hl,
                           kvl, len_dev, ld_seq, scale_log2, table, bsz, mb);
    } else {
        // LDS: queries [G][D] and scores [G][CH] fp32, values [CH][D] bf16
        const size_t lds = ((size_t)G * D + (size_t)G * CHT) * sizeof(float) + (size_t)CHT * D * sizeof(bf16);
        hipLaunchKernelGGL((attn_decode_chunk<D, CHT>), dim3(nchunks, kvl, B), dim3(256), lds, st, q, K, V, scratch,
                           hl, kvl, len_dev, ld_seq, scale_log2, table, bsz, mb);
    }
    // up to 128 chunks: every load in one round (4 or 8 parts of up to 16
    // chunks per thread); longer chunk lists: the tiled merge
    if (nchunks <= 64)
        hipLaunchKernelGGL((attn_decode_merge<D, 4, 16>), dim3(hl, B), dim3(D * 4), 0, st, scratch, O, hl, nchunks,
                           len_dev, ld_seq, CHT);
    else if (nchunks <= 128)
        hipLaunchKernelGGL((attn_decode_merge<D, 8, 16>), dim3(hl, B), dim3(D * 8), 0, st, scratch, O, hl, nchunks,
                           len_dev, ld_seq, CHT);
    else
        hipLaunchKernelGGL((attn_decode_combine<D, 512>), dim3(hl, B), dim3(512), 0, st, scratch, O, hl, nchunks,
                           len_dev, ld_seq, CHT);
}

void attn_decode_bf16(const bf16* q, const bf16* K, const bf16* V, bf16* O, float* scratch, int* counters, int B,
                      int hl, int kvl, const int* len_dev, int ld_seq, int d, const int* table, int bsz, int mb,
                      hipStream_t st) {
    const DecodeAttnPlan p = decode_attn_plan(B, hl, kvl, ld_seq, d);
    // the G = 1 split kernel is built for 64-position chunks
    const int ch = !p.fused && hl == kvl ? 64 : p.ch;
#define TP_DA(DD, CC) \
    launch_decode_attn<DD, CC>(q, K, V, O, scratch, counters, B, hl, kvl, len_dev, ld_seq, table, bsz, mb, p, st)
    if (d == 128) {
        if (ch == 64) TP_DA(128, 64);
        else if (ch == 32) TP_DA(128, 32);
        else TP_DA(128, 16);
    } else {
        if (ch == 64) TP_DA(64, 64);
        else TP_DA(64, 32);
    }
#undef TP_DA
}

void kv_to_pages(const bf16* k, const bf16* v, bf16* kpool, bf16* vpool, int B, int kvl, int S, int d,
                 const int* table, int bsz, int max_blocks, hipStream_t st) {
    const long long rows = (long long)B * kvl * S;
    const int blocks = (int)std::min<long long>((rows * (d / 8) + 255) / 256, 256LL * 8);
    hipLaunchKernelGGL(pages_kernel, dim3(blocks), dim3(256), 0, st, k, v, kpool, vpool, B, kvl, S, d, table, bsz,
                       max_blocks);
}

}  // namespace tp
