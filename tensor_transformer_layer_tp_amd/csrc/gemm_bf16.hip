// bf16 projection GEMM for gfx950: C[M,N] = A[M,K] * B[N,K]^T, fp32 accumulate.
//
// Both operands are K-contiguous (activations [tokens, in], weights [out, in]),
// which is the layout the MFMA fragments want: every lane reads 8 consecutive
// k-values of one row with one 16-byte LDS read.
//
// Column-parallel projections (Q/K/V, gate/up) and row-parallel ones (out,
// down) all run through this kernel; they differ only in the epilogue
// (undercodenews post 110319 on tensor parallelism, section "the Original":
// column-parallel = full input times a column slice, row-parallel = matching
// blocks giving partial results).
//
// Structure: 256 threads = 4 waves in a WM x WN grid; each wave owns a
// (BM/WM) x (BN/WN) tile of 32x32 MFMA accumulators (v_mfma_f32_32x32x16_bf16).
// K advances in steps of 64 through a double-buffered LDS stage filled from
// registers; LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled
// by (row & 7) so that the fragment reads hit distinct banks.  Work-groups
// are remapped so that each XCD (hardware places work-group i on XCD i % 8)
// receives a contiguous, L2-friendly block of tiles.
#include "kernels.h"

#include <stdlib.h>

namespace tp {

namespace {

constexpr int BK = 64;

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const bf16* __restrict__ A, long long lda,
                                                        const bf16* __restrict__ B, long long ldb, int M,
                                                        int N, int K, Epilogue epi, int tiles_m,
                                                        int tiles_n) {
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int CA = BM * 8 / 256, CB = BN * 8 / 256;  // 16-byte chunks per thread
    static_assert(WM * WN == 4, "4 waves");
    static_assert(FN % 2 == 0, "wave N-tile must cover whole 64-column groups");

    __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // ---- tile index: XCD-contiguous blocks, then grouped row-major order
    int bid = blockIdx.x;
    const int ntiles = tiles_m * tiles_n;
    if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
    constexpr int GROUP = 4;
    const int gsize = GROUP * tiles_n;
    const int gidx = bid / gsize;
    const int first_m = gidx * GROUP;
    const int gm = min(tiles_m - first_m, GROUP);
    const int tm = first_m + (bid % gsize) % gm;
    const int tn = (bid % gsize) / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- global -> register staging assignment: thread t copies 16-byte chunk
    // (t & 7) of rows (t >> 3) + 32 i; the swizzle (row & 7) is the same for all i.
    const int srow = tid >> 3, skc = tid & 7;
    const bf16* pa0 = A + skc * 8;
    const bf16* pb0 = B + skc * 8;
    long long oa[CA], ob[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) oa[i] = (long long)min(m0 + srow + 32 * i, M - 1) * lda;
#pragma unroll
    for (int i = 0; i < CB; ++i) ob[i] = (long long)min(n0 + srow + 32 * i, N - 1) * ldb;
    const int l0 = srow * BK + ((skc ^ (srow & 7)) << 3);

    bf16x8 ra[CA], rb[CB];
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16){};

    const int KT = K / BK;

#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *(const bf16x8*)(pa0 + oa[i]);
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[i] = *(const bf16x8*)(pb0 + ob[i]);
#pragma unroll
    for (int i = 0; i < CA; ++i) *(bf16x8*)(&sA[0][l0 + i * 32 * BK]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *(bf16x8*)(&sB[0][l0 + i * 32 * BK]) = rb[i];
    __syncthreads();

    // fragment read offsets (row part); row & 7 == lane & 7 since tile rows are 32-aligned
    const int frow = lane & 31;
    const int khalf = lane >> 5;
    const int swz = lane & 7;

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) {
            const int koff = (kt + 1) * BK;
#pragma unroll
            for (int i = 0; i < CA; ++i) ra[i] = *(const bf16x8*)(pa0 + oa[i] + koff);
#pragma unroll
            for (int i = 0; i < CB; ++i) rb[i] = *(const bf16x8*)(pb0 + ob[i] + koff);
        }
        const bf16* a_s = sA[cur];
        const bf16* b_s = sB[cur];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int kc = ((kk * 2 + khalf) ^ swz) << 3;
            bf16x8 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = *(const bf16x8*)(a_s + (wm * TM + i * 32 + frow) * BK + kc);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = *(const bf16x8*)(b_s + (wn * TN + j * 32 + frow) * BK + kc);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < CA; ++i) *(bf16x8*)(&sA[cur ^ 1][l0 + i * 32 * BK]) = ra[i];
#pragma unroll
            for (int i = 0; i < CB; ++i) *(bf16x8*)(&sB[cur ^ 1][l0 + i * 32 * BK]) = rb[i];
        }
        __syncthreads();
    }

    // ---- epilogue.  acc[i][j][r] sits at row 8*(r/4) + 4*(lane/32) + r%4 and
    // column lane%32 of MFMA tile (i, j).
    const int col_in = lane & 31;
    const int row_in = 4 * (lane >> 5);
    const int wrow0 = m0 + wm * TM;
    const int wcol0 = n0 + wn * TN;

    // Stores are predicated per element (no early exits): divergent control
    // flow around the accumulator tile makes the compiler spill it.
    if constexpr (MODE == EPI_F32) {
        float* o = (float*)epi.out;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wrow0 + i * 32 + 8 * (r >> 2) + row_in + (r & 3);
                    const int col = wcol0 + j * 32 + col_in;
                    if (row < M && col < N) o[(long long)row * epi.ldo + col] = acc[i][j][r];
                }
    } else if constexpr (MODE == EPI_STORE || MODE == EPI_GELU) {
        bf16* o = (bf16*)epi.out;
        constexpr bool gelu = MODE == EPI_GELU;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wrow0 + i * 32 + 8 * (r >> 2) + row_in + (r & 3);
                    const int col = wcol0 + j * 32 + col_in;
                    float v = acc[i][j][r];
                    if constexpr (gelu) v = gelu_erf_f(v);
                    if (row < M && col < N) o[(long long)row * epi.ldo + col] = f2bf(v);
                }
    } else if constexpr (MODE == EPI_SWIGLU) {
        bf16* o = (bf16*)epi.out;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int p = 0; p < FN / 2; ++p)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wrow0 + i * 32 + 8 * (r >> 2) + row_in + (r & 3);
                    const int gcol = wcol0 + p * 64;  // 64-aligned group: [gate 32 | up 32]
                    const float g = acc[i][2 * p][r], u = acc[i][2 * p + 1][r];
                    if (row < M && gcol < N) o[(long long)row * epi.ldo + (gcol >> 1) + col_in] = f2bf(silu_f(g) * u);
                }
    } else {  // MODE == EPI_QKV
        // EPI_QKV: the 64-column group at gcol holds dims (i1, i1 + d/2) of one
        // head in its two 32-column halves; rotate the pair, then scatter.
        const QKVDest& q = epi.qkv;
        const int d = q.d;
        const int half = d >> 1;
        const int qcols = q.hl * d, kcols = q.kvl * d;
#pragma unroll
        for (int p = 0; p < FN / 2; ++p) {
            const int gcol = wcol0 + p * 64;
            const int region = gcol < qcols ? 0 : (gcol < qcols + kcols ? 1 : 2);
            const int base = region == 0 ? 0 : (region == 1 ? qcols : qcols + kcols);
            const int head = (gcol - base) / d;
            const int i1 = 32 * (((gcol - base) % d) >> 6) + col_in;
            const bool rot = region < 2 && q.rope_cos != nullptr;
            bf16* dbase = region == 0 ? (bf16*)q.q : (region == 1 ? (bf16*)q.k : (bf16*)q.v);
            const int nh = region == 0 ? q.hl : q.kvl;
            const int ld = region == 0 ? q.S : q.ld_seq;
            const int poff = region == 0 ? 0 : q.pos0;   // q is stored by token index, k/v by position
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wrow0 + i * 32 + 8 * (r >> 2) + row_in + (r & 3);
                    const int rr = min(row, M - 1);
                    const int b = rr / q.S, s = rr - b * q.S;
                    const int pos = q.pos0 + s;
                    float y1 = acc[i][2 * p][r], y2 = acc[i][2 * p + 1][r];
                    float c = 1.f, sn = 0.f;
                    if (rot) {
                        c = q.rope_cos[(long long)pos * half + i1];
                        sn = q.rope_sin[(long long)pos * half + i1];
                    }
                    const float o1 = y1 * c - y2 * sn;
                    const float o2 = y2 * c + y1 * sn;
                    bf16* dst = dbase + (((long long)b * nh + head) * ld + poff + s) * d;
                    if (row < M && gcol < N) {
                        dst[i1] = f2bf(o1);
                        dst[i1 + half] = f2bf(o2);
                    }
                }
        }
    }
}

struct Cfg {
    int bm, bn;
    float eff;   // guessed relative MFMA efficiency of one work-group
    int occ;     // work-groups per CU
};
const Cfg kCfgs[] = {
    {256, 256, 1.00f, 1},
    {256, 128, 0.90f, 1},
    {128, 128, 0.70f, 2},
    {128, 256, 0.90f, 1},
};
constexpr int kNumCfg = sizeof(kCfgs) / sizeof(kCfgs[0]);
int g_forced_cfg = -1;

template <int BM, int BN, int WM, int WN>
void launch(const bf16* A, long long lda, const bf16* B, long long ldb, int M, int N, int K,
            const Epilogue& epi, hipStream_t st) {
    int tm = cdiv(M, BM), tn = cdiv(N, BN);
    dim3 g(tm * tn), b(256);
    switch (epi.mode) {
        case EPI_F32:
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI_F32>), g, b, 0, st, A, lda, B, ldb, M, N, K, epi, tm, tn);
            break;
        case EPI_QKV:
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI_QKV>), g, b, 0, st, A, lda, B, ldb, M, N, K, epi, tm, tn);
            break;
        case EPI_SWIGLU:
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI_SWIGLU>), g, b, 0, st, A, lda, B, ldb, M, N, K, epi, tm, tn);
            break;
        case EPI_GELU:
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI_GELU>), g, b, 0, st, A, lda, B, ldb, M, N, K, epi, tm, tn);
            break;
        default:
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI_STORE>), g, b, 0, st, A, lda, B, ldb, M, N, K, epi, tm, tn);
            break;
    }
}

// The 256x256 tile keeps 256 accumulators per lane; with the rotary and the
// erf epilogues the compiler spills them, so those modes skip it.
bool usable(int c, int mode) { return !(c == 0 && (mode == EPI_QKV || mode == EPI_GELU)); }

int pick(int M, int N, int mode) {
    if (g_forced_cfg >= 0 && g_forced_cfg < kNumCfg && usable(g_forced_cfg, mode)) return g_forced_cfg;
    int best = 1;
    double best_t = 1e30;
    for (int c = 0; c < kNumCfg; ++c) {
        if (!usable(c, mode)) continue;
        const Cfg& f = kCfgs[c];
        long long tiles = (long long)cdiv(M, f.bm) * cdiv(N, f.bn);
        long long slots = 256LL * f.occ;
        long long waves = (tiles + slots - 1) / slots;
        double t = (double)waves * f.bm * f.bn * f.occ / f.eff;
        if (t < best_t * 0.999) { best_t = t; best = c; }
    }
    return best;
}

}  // namespace

void set_gemm_config(int cfg) { g_forced_cfg = cfg; }
int gemm_config_count() { return kNumCfg; }

void gemm_bf16(const bf16* A, long long lda, const bf16* B, long long ldb, int M, int N, int K,
               const Epilogue& epi, hipStream_t st) {
    switch (pick(M, N, epi.mode)) {
        case 0: launch<256, 256, 2, 2>(A, lda, B, ldb, M, N, K, epi, st); break;
        case 1: launch<256, 128, 2, 2>(A, lda, B, ldb, M, N, K, epi, st); break;
        case 2: launch<128, 128, 2, 2>(A, lda, B, ldb, M, N, K, epi, st); break;
        default: launch<128, 256, 2, 2>(A, lda, B, ldb, M, N, K, epi, st); break;
    }
}

}  // namespace tp
