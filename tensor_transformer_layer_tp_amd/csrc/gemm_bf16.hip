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
// Every family computes 32x32 MFMA accumulator tiles (v_mfma_f32_32x32x16_bf16)
// from fragments in LDS; they differ in who moves the tiles into LDS:
//  * producer/consumer (gemm_ws_kernel, the default for large projections):
//    eight waves only read fragments and issue MFMAs, four more only load
//    the next tile into registers and write it to the free LDS stage;
//  * register-pipelined (gemm_vgpr_kernel): eight waves do both, the loads
//    of tile kt+2 spread over the k-slices of tile kt;
//  * four-wave kernels in a 2 x 2 grid: "dma" (buffer_load ... lds into a ring
//    of ST stages, no staging registers) and "reg" (two register stages, then
//    a double-buffered LDS stage).
// A planner (plan(), from a per-CU cost model) picks the tile and family per
// shape, and may run a GEMM as two launches over column ranges.  LDS rows
// hold BK bf16 with the 16-byte chunk index XOR-swizzled by row so that the
// fragment reads of 16 consecutive rows hit distinct bank groups.  Work-groups
// are remapped so that each XCD (hardware places work-group i on XCD i % 8)
// receives a contiguous, L2-friendly block of tiles.
#include "common.h"

#include <stdint.h>

#include <type_traits>

namespace tp {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// tile (tm, tn) of block b: XCD-contiguous ranges, then groups of GROUP tile rows
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int ntiles = tiles_m * tiles_n;
    if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
    constexpr int GROUP = 4;
    const int gsize = GROUP * tiles_n;
    const int first_m = (bid / gsize) * GROUP;
    const int gm = min(tiles_m - first_m, GROUP);
    tm = first_m + (bid % gsize) % gm;
    tn = (bid % gsize) / gm;
}

// 16-byte chunk slot of logical chunk c in LDS row r (CPR chunks per row)
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
    return CPR == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt with only vmcnt constrained (expcnt 7, lgkmcnt 15: no wait)
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The all-reduce's sum in a row-parallel projection's epilogue (EPI_SUM):
// h = (sum over ranks, in rank order, of the partials) + residual at the W
// consecutive elements from element offset `off` of the [M, ldo] partials,
// with this projection's own values in slot `self` -- the order and rounding
// of the reduce kernel.  The other ranks' partials are read once
// (non-temporal); the residual is added only when present, so that a -0 sum
// stays -0.
template <int W>
__device__ __forceinline__ void sum_ranks(const SumDest& sd, long long off, float (&v)[W]) {
    float p[kSumMaxRanks][W];
#pragma unroll
    for (int j = 0; j < kSumMaxRanks; ++j) {
        if (j < sd.t && j != sd.self) {
            if constexpr (W == 4) {
                const f32x4 q = __builtin_nontemporal_load((const f32x4*)(sd.p[j] + off));
#pragma unroll
                for (int e = 0; e < 4; ++e) p[j][e] = q[e];
            } else {
#pragma unroll
                for (int e = 0; e < W; ++e) p[j][e] = __builtin_nontemporal_load(sd.p[j] + off + e);
            }
        } else {
#pragma unroll
            for (int e = 0; e < W; ++e) p[j][e] = v[e];
        }
    }
    float r[W];
    if (sd.residual != nullptr) {
#pragma unroll
        for (int e = 0; e < W; ++e) r[e] = bf2f(sd.residual[off + e]);
    }
#pragma unroll
    for (int e = 0; e < W; ++e) {
        float a = p[0][e];
#pragma unroll
        for (int j = 1; j < kSumMaxRanks; ++j)
            if (j < sd.t) a += p[j][e];
        if (sd.residual != nullptr) a += r[e];
        v[e] = a;
    }
}

// Write the accumulator tile of one wave.  acc[i][j][r] sits at row
// 8*(r/4) + 4*(lane/32) + r%4 and column lane%32 of MFMA tile (i, j).
template <int FM, int FN, int MODE, int QB = 16>
__device__ __forceinline__ void epilogue(f32x16 (&acc)[FM][FN], const Epilogue& epi, int lane, int wrow0,
                                         int wcol0, int M, int N) {
    static_assert(QB == 4 || QB == 8 || QB == 16, "rotary gather batch");
    const int col_in = lane & 31;
    const int row_in = 4 * (lane >> 5);
    const int cb = epi.col0;   // this launch's first output column (bounds stay launch-relative)
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
                    if (row < M && col < N) o[(long long)row * epi.ldo + cb + col] = acc[i][j][r];
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
                    if (row < M && col < N) o[(long long)row * epi.ldo + cb + col] = f2bf(v);
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
                    if (row < M && gcol < N)
                        o[(long long)row * epi.ldo + ((cb + gcol) >> 1) + col_in] = f2bf(silu_f(g) * u);
                }
    } else if constexpr (MODE == EPI_SUM) {
        bf16* o = (bf16*)epi.out;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wrow0 + i * 32 + 8 * (r >> 2) + row_in + (r & 3);
                    const int col = wcol0 + j * 32 + col_in;
                    if (row < M && col < N) {
                        const long long off = (long long)row * epi.ldo + cb + col;
                        float v[1] = {acc[i][j][r]};
                        sum_ranks<1>(epi.sum, off, v);
                        o[off] = f2bf(v[0]);
                    }
                }
    } else {  // MODE == EPI_QKV
        // EPI_QKV: the 64-column group at gcol holds dims (i1, i1 + d/2) of one
        // head in its two 32-column halves; rotate the pair, then scatter.
        const QKVDest& q = epi.qkv;
        const int d = q.d;
        const int half = d >> 1;
        const int qcols = q.hl * d, kcols = q.kvl * d;
        // Everything the stores depend on is read before the first store: the
        // compiler cannot prove the stores leave these locations alone, so a
        // load placed after a store waits for it.
        const int base_pos = q.pos_dev ? *q.pos_dev : q.pos0;
        // Token row -> (sequence b, offset s), without integer divisions (their
        // reciprocal constants stay live through the epilogue).  The first row
        // of each 32-row tile: a double quotient corrected by one step, exact
        // for any int row.  The other rows lie at most 27 rows further, so
        // their extra wrap count n / S is below 29 and a float quotient
        // corrected by one step is exact.  Rows past M take row M-1's pair
        // (their stores are dropped; their reads stay in range).
        const float inv_s = 1.f / (float)q.S;
        const double inv_sd = 1.0 / (double)q.S;
        auto seq_of = [&](int row) {
            int w = (int)((double)row * inv_sd);
            const int t = row - w * q.S;
            return t < 0 ? w - 1 : (t >= q.S ? w + 1 : w);
        };
        const int b_last = seq_of(M - 1), s_last = (M - 1) - b_last * q.S;
        // d is 64 or 128 (checked when a shard is created): shifts, no divisions
        const int dlog = 31 - __builtin_clz(d);
        auto dim_of = [&](int p) { return 32 * (((cb + wcol0 + p * 64) & (d - 1)) >> 6) + col_in; };
        // rotation turns per position of each pair's dim, read before any store
        double turns_p[FN / 2];
#pragma unroll
        for (int p = 0; p < FN / 2; ++p) turns_p[p] = q.rope_rev != nullptr ? q.rope_rev[dim_of(p)] : 0.0;
#pragma unroll
        for (int p = 0; p < FN / 2; ++p) {
            const int gcol = wcol0 + p * 64;          // launch-relative (bounds)
            const int acol = cb + gcol;               // absolute packed column
            const int region = acol < qcols ? 0 : (acol < qcols + kcols ? 1 : 2);
            const int base = region == 0 ? 0 : (region == 1 ? qcols : qcols + kcols);
            const int head = (acol - base) >> dlog;
            const int i1 = 32 * (((acol - base) & (d - 1)) >> 6) + col_in;
            const bool rot = region < 2 && q.rope_rev != nullptr;
            bf16* dbase = region == 0 ? (bf16*)q.q : (region == 1 ? (bf16*)q.k : (bf16*)q.v);
            const int nh = region == 0 ? q.hl : q.kvl;
            const int ld = region == 0 ? q.S : q.ld_seq;
            const int poff = region == 0 ? 0 : base_pos;   // q is stored by token index, k/v by position
            const bool paged = region != 0 && q.table != nullptr;
            // The rotation of row position pos is pos * theta_i turns: its
            // fraction, formed in double (exact for any position), goes to the
            // hardware sine and cosine, which take turns (|error| <= 1.3e-7 on
            // [0, 1)).  No table reads: without a block table the epilogue
            // issues no loads at all.
            const double turns = turns_p[p];
            auto rotation = [&](int pos, float& c, float& sn) {
                c = 1.f;
                sn = 0.f;
                if (rot) {
                    const double a = (double)pos * turns;
                    const float f = (float)(a - floor(a));
                    c = __builtin_amdgcn_cosf(f);
                    sn = __builtin_amdgcn_sinf(f);
                }
            };
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row0 = wrow0 + i * 32 + row_in;
                const int b0 = seq_of(row0), s0 = row0 - b0 * q.S;
#pragma unroll
                for (int r0 = 0; r0 < 16; r0 += QB) {
                    // QB of the lane's 16 rows of this MFMA tile.  With a block
                    // table, the table reads of the QB rows are issued together
                    // and waited for once (a wait per row would also wait for
                    // the stores before it).
                    int key[QB], ps[QB];   // key: sequence, or pool block of a paged cache
#pragma unroll
                    for (int rq = 0; rq < QB; ++rq) {
                        const int r = r0 + rq;
                        const int row = row0 + 8 * (r >> 2) + (r & 3);
                        const int n = s0 + 8 * (r >> 2) + (r & 3);
                        int w = (int)((float)n * inv_s);
                        const int t = n - w * q.S;
                        w = t < 0 ? w - 1 : (t >= q.S ? w + 1 : w);
                        const int b = row < M ? b0 + w : b_last;
                        ps[rq] = row < M ? n - w * q.S : s_last;
                        key[rq] = b;
                    }
                    if (paged) {
#pragma unroll
                        for (int rq = 0; rq < QB; ++rq)
                            key[rq] = kv_block(key[rq], base_pos + ps[rq], q.table, q.bsz, q.max_blocks);
                        wait_vm<0>();
                    }
#pragma unroll
                    for (int rq = 0; rq < QB; ++rq) {
                        const int r = r0 + rq;
                        const int row = row0 + 8 * (r >> 2) + (r & 3);
                        const int pos = base_pos + ps[rq];
                        float c, sn;
                        rotation(pos, c, sn);
                        const float y1 = acc[i][2 * p][r], y2 = acc[i][2 * p + 1][r];
                        const float o1 = y1 * c - y2 * sn;
                        const float o2 = y2 * c + y1 * sn;
                        const long long off =
                            paged ? kv_row_in_block(key[rq], head, pos, q.kvl, q.bsz, d)
                                  : (((long long)key[rq] * nh + head) * ld + poff + ps[rq]) * d;
                        if (row < M && gcol < N && (region == 0 || pos < q.ld_seq)) {
                            dbase[off + i1] = f2bf(o1);
                            dbase[off + i1 + half] = f2bf(o2);
                        }
                    }
                }
            }
        }
    }
}

// Epilogue through LDS (SwiGLU and fp32 partials): the wave writes its
// accumulator tile, finished, into a private LDS region in row order, then
// stores whole 16-byte row chunks.  The direct epilogue stores 2 or 4 bytes
// per lane and instruction (one instruction per accumulator register); this
// one a sixth to a quarter of the instructions.  The caller guarantees that no
// other wave touches the region any more (RB bf16 elements, 16-byte aligned).
template <int FM, int FN, int MODE, int RB>
__device__ __forceinline__ void epilogue_staged(f32x16 (&acc)[FM][FN], const Epilogue& epi, int lane, int wrow0,
                                                int wcol0, int M, int N, bf16* sreg) {
    static_assert(MODE == EPI_SWIGLU || MODE == EPI_F32 || MODE == EPI_SUM, "staged epilogue modes");
    const int col_in = lane & 31;
    const int row_in = 4 * (lane >> 5);
    const int cb = epi.col0;
    if constexpr (MODE == EPI_SWIGLU) {
        constexpr int OC = FN * 16;        // output columns of the wave's tile (one per gate/up pair)
        constexpr int OCP = OC + 8;        // padded LDS row (bf16)
        constexpr int CPR = OC / 8;        // 16-byte chunks per row
        static_assert(FM * 32 * OCP <= RB, "LDS region");
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int p = 0; p < FN / 2; ++p)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rl = i * 32 + 8 * (r >> 2) + row_in + (r & 3);
                    sreg[rl * OCP + p * 32 + col_in] = f2bf(silu_f(acc[i][2 * p][r]) * acc[i][2 * p + 1][r]);
                }
        bf16* o = (bf16*)epi.out;
#pragma unroll
        for (int k = 0; k < FM * 32 * CPR / 64; ++k) {
            const int c = lane + 64 * k;
            const int rl = c / CPR, ch = c % CPR;
            const int row = wrow0 + rl;
            const int gcol = wcol0 + (ch >> 2) * 64;   // the chunk's 64-column input group
            if (row < M && gcol < N)
                *(u32x4_t*)(o + (long long)row * epi.ldo + ((cb + wcol0) >> 1) + ch * 8) =
                    *(const u32x4_t*)(sreg + rl * OCP + ch * 8);
        }
    } else {
        constexpr int TN = FN * 32;
        constexpr int TNP = TN + 4;        // padded LDS row (fp32)
        constexpr int CPR = TN / 4;        // 16-byte chunks per row
        static_assert(32 * TNP * 2 <= RB, "LDS region");
        float* sf = (float*)sreg;
        float* o = (float*)epi.out;
#pragma unroll
        for (int i = 0; i < FM; ++i) {     // 32 rows at a time
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) sf[(8 * (r >> 2) + row_in + (r & 3)) * TNP + j * 32 + col_in] = acc[i][j][r];
#pragma unroll
            for (int k = 0; k < 32 * CPR / 64; ++k) {
                const int c = lane + 64 * k;
                const int rl = c / CPR, ch = c % CPR;
                const int row = wrow0 + i * 32 + rl;
                const int col = wcol0 + ch * 4;
                if constexpr (MODE == EPI_SUM) {
                    // the reduce of the ranks' partials, stored as 4 bf16
                    if (row < M && col < N) {
                        const long long off = (long long)row * epi.ldo + cb + col;
                        const f32x4 a = *(const f32x4*)(sf + rl * TNP + ch * 4);
                        float v[4] = {a[0], a[1], a[2], a[3]};
                        sum_ranks<4>(epi.sum, off, v);
                        uint32_t w[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e)
                            w[e] = (uint32_t)f2bf_bits(v[2 * e]) | ((uint32_t)f2bf_bits(v[2 * e + 1]) << 16);
                        *(uint2*)((bf16*)epi.out + off) = make_uint2(w[0], w[1]);
                    }
                } else {
                    // non-temporal: the partial is read once, by the reduce that follows,
                    // which then finds no dirty lines of it to write back from L2
                    if (row < M && col < N)
                        __builtin_nontemporal_store(*(const u32x4_t*)(sf + rl * TNP + ch * 4),
                                                    (u32x4_t*)(o + (long long)row * epi.ldo + cb + col));
                }
            }
        }
    }
}

// Direct-to-LDS load of one 16-byte chunk per lane (buffer_load_dwordx4 ...
// lds): lane i of the wave lands at LDS byte lds + 16 i.  The caller waits on
// vmcnt before the barrier that publishes a stage.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(uintptr_t)lds, 16, (int)voff, (int)soff, 0, 0);
}

// Buffer resource over `bytes` bytes from base (raw, no stride): reads past
// the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// The MFMAs of one LDS stage.  Fragments of k-slice kk+1 are read before the
// MFMAs of slice kk issue (the scheduling barriers keep that order), so the
// LDS latency of every slice but the first hides behind 16-wide MFMA work.
template <int FM, int FN>
__device__ __forceinline__ void interleave_reads_mfma() {
    // one fragment read, then its share of the MFMAs, repeated: keeps both the
    // LDS and the matrix pipe busy instead of queueing all reads up front
#pragma unroll
    for (int q = 0; q < FM + FN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);                      // DS read
        __builtin_amdgcn_sched_group_barrier(0x0008, FM * FN / (FM + FN), 0);    // MFMA
    }
}

template <int FM, int FN, int BK, int CPR>
__device__ __forceinline__ void mma_stage(f32x16 (&acc)[FM][FN], const bf16* a_s, const bf16* b_s, int frow,
                                          int khalf) {
    bf16x8 fa[2][FM], fb[2][FN];
    auto rd = [&](int kk, int buf) {
        const int c = swz<CPR>(frow, 2 * kk + khalf) << 3;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = *(const bf16x8*)(a_s + i * 32 * BK + c);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = *(const bf16x8*)(b_s + j * 32 * BK + c);
    };
    rd(0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < BK / 16) rd(kk + 1, cur ^ 1);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
        if (kk + 1 < BK / 16) interleave_reads_mfma<FM, FN>();
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// DMA main loop: ST-stage LDS ring, tile k+ST-1 requested while tile k is used.
template <int BM, int BN, int BK, int ST, int MODE>
__global__ __launch_bounds__(256) void gemm_dma_kernel(const bf16* __restrict__ A, long long lda,
                                                       const bf16* __restrict__ B, long long ldb, int M, int N,
                                                       int K, Epilogue epi, int tiles_m, int tiles_n) {
    constexpr int TM = BM / 2, TN = BN / 2, FM = TM / 32, FN = TN / 32;
    constexpr int CPR = BK / 8;              // 16-byte chunks per LDS row
    constexpr int RPI = 64 / CPR;            // rows per wave-wide DMA (64 lanes x 16 B)
    constexpr int IA = BM / RPI / 4, IB = BN / RPI / 4;  // DMAs per wave per stage
    constexpr int STAGE = (BM + BN) * BK;    // bf16 elements per stage
    static_assert(FN % 2 == 0 && IA >= 1 && IB >= 1, "tile shape");
    __shared__ __attribute__((aligned(1024))) bf16 smem[ST * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    if (blockIdx.x == 0 && threadIdx.x == 0) apply_len_update(epi.len);
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // rows past M / N fall outside the resources and read as zeros
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(A + (long long)m0 * lda, (uint32_t)(min(BM, M - m0) * lda * 2));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(B + (long long)n0 * ldb, (uint32_t)(min(BN, N - n0) * ldb * 2));
    const int lrow = lane / CPR, lslot = lane % CPR;
    uint32_t va[IA], vb[IB];
#pragma unroll
    for (int j = 0; j < IA; ++j) {
        const int r = (wave * IA + j) * RPI + lrow;
        va[j] = (uint32_t)((r * lda + 8 * swz<CPR>(r, lslot)) * 2);
    }
#pragma unroll
    for (int j = 0; j < IB; ++j) {
        const int r = (wave * IB + j) * RPI + lrow;
        vb[j] = (uint32_t)((r * ldb + 8 * swz<CPR>(r, lslot)) * 2);
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    auto issue = [&](int kt, int slot) {
        const uint32_t soff = (uint32_t)(kt * BK * 2);
        const uint32_t sa = lds0 + (uint32_t)(slot * STAGE * 2);
        const uint32_t sb = sa + (uint32_t)(BM * BK * 2);
#pragma unroll
        for (int j = 0; j < IA; ++j)
            dma16(rsa, va[j], soff, __builtin_amdgcn_readfirstlane(sa + (uint32_t)((wave * IA + j) * RPI * BK * 2)));
#pragma unroll
        for (int j = 0; j < IB; ++j)
            dma16(rsb, vb[j], soff, __builtin_amdgcn_readfirstlane(sb + (uint32_t)((wave * IB + j) * RPI * BK * 2)));
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16){};

    const int KT = K / BK;
    const int frow = lane & 31, khalf = lane >> 5;
#pragma unroll
    for (int s = 0; s < ST - 1; ++s) issue(min(s, KT - 1), s);

    for (int kt = 0; kt < KT; ++kt) {
        // tile kt has landed once at most the (ST-2) newer tiles are pending
        wait_vm<(ST - 2) * (IA + IB)>();
        __syncthreads();
        // every wave is past tile kt-1: its slot takes tile kt+ST-1
        issue(min(kt + ST - 1, KT - 1), (kt + ST - 1) % ST);
        const bf16* a_s = smem + (kt % ST) * STAGE + (wm * TM + frow) * BK;
        const bf16* b_s = smem + (kt % ST) * STAGE + BM * BK + (wn * TN + frow) * BK;
        mma_stage<FM, FN, BK, CPR>(acc, a_s, b_s, frow, khalf);
    }
    wait_vm<0>();  // no LDS write may still be in flight when the work-group ends
    epilogue<FM, FN, MODE>(acc, epi, lane, m0 + wm * TM, n0 + wn * TN, M, N);
}

// ---------------------------------------------------------------------------
// DMA main loop for rings of ST >= 3 stages, software-pipelined across the
// stage boundary: the barrier that publishes tile k+1, the DMA request for
// tile k+ST-1 and the first fragment reads of tile k+1 all happen before the
// MFMAs of tile k's last k-slice, and the DMA requests are interleaved with
// those MFMAs, so the matrix pipe keeps issuing across the boundary.  The
// DMA of a tile always targets the slot of the tile before the current one,
// whose fragment reads completed before that tile's MFMAs issued.
template <int BM, int BN, int BK, int ST, int MODE>
__global__ __launch_bounds__(256) void gemm_dma_pipe_kernel(const bf16* __restrict__ A, long long lda,
                                                            const bf16* __restrict__ B, long long ldb, int M,
                                                            int N, int K, Epilogue epi, int tiles_m, int tiles_n) {
    constexpr int TM = BM / 2, TN = BN / 2, FM = TM / 32, FN = TN / 32;
    constexpr int CPR = BK / 8;
    constexpr int RPI = 64 / CPR;
    constexpr int IA = BM / RPI / 4, IB = BN / RPI / 4;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int KK = BK / 16;
    static_assert(ST >= 3 && FN % 2 == 0 && IA >= 1 && IB >= 1, "tile shape");
    __shared__ __attribute__((aligned(1024))) bf16 smem[ST * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps DMA addressing scalar
    const int wm = wave >> 1, wn = wave & 1;
    if (blockIdx.x == 0 && threadIdx.x == 0) apply_len_update(epi.len);
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(A + (long long)m0 * lda, (uint32_t)(min(BM, M - m0) * lda * 2));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(B + (long long)n0 * ldb, (uint32_t)(min(BN, N - n0) * ldb * 2));
    const int lrow = lane / CPR, lslot = lane % CPR;
    uint32_t vab[IA + IB];
#pragma unroll
    for (int j = 0; j < IA; ++j) {
        const int r = (wave * IA + j) * RPI + lrow;
        vab[j] = (uint32_t)((r * lda + 8 * swz<CPR>(r, lslot)) * 2);
    }
#pragma unroll
    for (int j = 0; j < IB; ++j) {
        const int r = (wave * IB + j) * RPI + lrow;
        vab[IA + j] = (uint32_t)((r * ldb + 8 * swz<CPR>(r, lslot)) * 2);
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    // LDS byte address of DMA j of this wave in stage `slot`
    auto dma_lds = [&](int slot, int j) -> uint32_t {
        const uint32_t base = lds0 + (uint32_t)(slot * STAGE * 2);
        return j < IA ? base + (uint32_t)((wave * IA + j) * RPI * BK * 2)
                      : base + (uint32_t)(BM * BK * 2 + (wave * IB + (j - IA)) * RPI * BK * 2);
    };
    auto dma = [&](int j, int kt, int slot) {
        dma16(j < IA ? rsa : rsb, vab[j], (uint32_t)(kt * BK * 2), __builtin_amdgcn_readfirstlane(dma_lds(slot, j)));
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16){};

    const int KT = K / BK;
    const int frow = lane & 31, khalf = lane >> 5;
    bf16x8 fa[2][FM], fb[2][FN];
    auto read = [&](int slot, int kk, int buf) {
        const bf16* a_s = smem + slot * STAGE + (wm * TM + frow) * BK;
        const bf16* b_s = smem + slot * STAGE + BM * BK + (wn * TN + frow) * BK;
        const int c = swz<CPR>(frow, 2 * kk + khalf) << 3;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = *(const bf16x8*)(a_s + i * 32 * BK + c);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = *(const bf16x8*)(b_s + j * 32 * BK + c);
    };
    auto mma = [&](int buf, int i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
    };

#pragma unroll
    for (int t = 0; t < ST - 1; ++t)
#pragma unroll
        for (int j = 0; j < IA + IB; ++j) dma(j, min(t, KT - 1), t);
    wait_vm<(ST - 2) * (IA + IB)>();
    __syncthreads();
    read(0, 0, 0);

    // all tiles but the last: no branch inside the body (a branch here makes
    // the compiler shuffle the accumulators between register ranges)
    for (int kt = 0; kt < KT - 1; ++kt) {
        const int slot = kt % ST;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            if (kk + 1 < KK) {
                read(slot, kk + 1, nxt);
#pragma unroll
                for (int i = 0; i < FM; ++i) mma(cur, i);
                interleave_reads_mfma<FM, FN>();
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // tile kt+1 must have landed: only the ST-3 newer tiles may be pending
                wait_vm<(ST - 3) * (IA + IB)>();
                __syncthreads();
                const int dslot = (kt + ST - 1) % ST, dtile = min(kt + ST - 1, KT - 1);
                // interleave: one MFMA row group, then a share of the DMA requests
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    mma(cur, i);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = i * (IA + IB) / FM; j < (i + 1) * (IA + IB) / FM; ++j) dma(j, dtile, dslot);
                    __builtin_amdgcn_sched_barrier(0);
                    if (i == 0) {
                        read((kt + 1) % ST, 0, nxt);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
    }
    {
        const int slot = (KT - 1) % ST;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            if (kk + 1 < KK) read(slot, kk + 1, nxt);
#pragma unroll
            for (int i = 0; i < FM; ++i) mma(cur, i);
        }
    }
    wait_vm<0>();  // no LDS write may still be in flight when the work-group ends
    epilogue<FM, FN, MODE>(acc, epi, lane, m0 + wm * TM, n0 + wn * TN, M, N);
}

// ---------------------------------------------------------------------------
// Register-pipelined main loop for 64-k tiles: plain 16-byte buffer loads
// into two register sets (each tile is requested two tiles before its MFMAs),
// ds_write into a double-buffered LDS stage.  On gfx950 vector loads into
// registers stream this tile traffic about 1.5x faster than the LDS DMA path,
// and a 64-k tile reads whole 128-byte lines of every row.
//
// Tile kt (4 k-slices) uses LDS stage kt % 2 and register set kt % 2:
//  slice 0: loads of tile kt+2 into set kt % 2 (its tile was written to LDS
//           at the end of tile kt-1), interleaved with the MFMAs;
//  slice 3: set (kt+1) % 2 is written to stage (kt+1) % 2 between the first
//           MFMAs, then the barrier publishes it, the first fragments of tile
//           kt+1 are read, and the remaining MFMAs of the slice cover that read.
// Stage (kt+1) % 2 last held tile kt-1, whose reads all completed before the
// barrier at the end of tile kt-1.
template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(64 * WM * WN) void gemm_vgpr_kernel(const bf16* __restrict__ A, long long lda,
                                                                 const bf16* __restrict__ B, long long ldb, int M,
                                                                 int N, int K, Epilogue epi, int tiles_m,
                                                                 int tiles_n) {
    constexpr int NT = 64 * WM * WN;            // threads
    constexpr int BK = 64, KK = 4;
    constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
    constexpr int RS = NT / 8;                   // rows per load step (8 chunks per 64-k row)
    constexpr int CA = BM / RS, CB = BN / RS;    // 16-byte chunks per thread per tile
    constexpr int STAGE = (BM + BN) * BK;
    static_assert(FN % 2 == 0 && BM % RS == 0 && BN % RS == 0, "tile shape");
    __shared__ __attribute__((aligned(1024))) bf16 smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    if (blockIdx.x == 0 && threadIdx.x == 0) apply_len_update(epi.len);
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // thread t copies 16-byte chunk (t & 7) of tile rows (t >> 3) + RS i.  Each
    // row step i has a buffer resource of its own (scalar registers) covering
    // only its rows, so one vector offset serves every load and rows past M
    // (or N) read as zeros.
    const int srow = tid >> 3, skc = tid & 7;
    __amdgpu_buffer_rsrc_t rsa[CA], rsb[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i)
        rsa[i] = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long long)(m0 + i * RS) * lda), (short)0,
                                                   max(0, min(RS, M - m0 - i * RS)) * (int)lda * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < CB; ++i)
        rsb[i] = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (long long)(n0 + i * RS) * ldb), (short)0,
                                                   max(0, min(RS, N - n0 - i * RS)) * (int)ldb * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs0 = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0, 0x00020000);
    const int va0 = (srow * (int)lda + skc * 8) * 2;
    const int vb0 = (srow * (int)ldb + skc * 8) * 2;
    const int l0 = srow * BK + (swz<8>(srow, skc) << 3);   // rows srow + RS i share the swizzle

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16){};

    const int KT = K / BK;
    const int frow = lane & 31, khalf = lane >> 5;
    u32x4 ra[2][CA], rb[2][CB];
    bf16x8 fa[2][FM], fb[2][FN];

    // Quarter q (of four) of the loads of tile kt into register set `set`:
    // each k-slice of a tile issues one quarter, so the CU's 16-byte loads are
    // spread evenly over the MFMA time instead of queueing up in one slice.
    constexpr int NL = CA + CB, QL = (NL + 3) / 4;
    auto gload = [&](auto set, int kt, int q) {
        // a tile past the end reads zeros through an empty resource
        const bool in = kt < KT;
        const int koff = in ? kt * BK * 2 : 0;
#pragma unroll
        for (int j = q * QL; j < min(NL, (q + 1) * QL); ++j) {
            if (j < CA) ra[set][j] = __builtin_amdgcn_raw_buffer_load_b128(in ? rsa[j] : rs0, va0, koff, 0);
            else rb[set][j - CA] = __builtin_amdgcn_raw_buffer_load_b128(in ? rsb[j - CA] : rs0, vb0, koff, 0);
        }
    };
    auto lstore = [&](auto set, int stage) {
        bf16* sa = smem + stage * STAGE;
#pragma unroll
        for (int i = 0; i < CA; ++i) *(u32x4*)(sa + l0 + i * RS * BK) = ra[set][i];
#pragma unroll
        for (int i = 0; i < CB; ++i) *(u32x4*)(sa + BM * BK + l0 + i * RS * BK) = rb[set][i];
    };
    auto read = [&](int stage, int kk, int buf) {
        const bf16* a_s = smem + stage * STAGE + (wm * TM + frow) * BK;
        const bf16* b_s = smem + stage * STAGE + BM * BK + (wn * TN + frow) * BK;
        const int c = swz<8>(frow, 2 * kk + khalf) << 3;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = *(const bf16x8*)(a_s + i * 32 * BK + c);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = *(const bf16x8*)(b_s + j * 32 * BK + c);
    };
    // MFMAs q0 .. q1-1 of a k-slice, numbered i * FN + j
    auto mma = [&](int buf, int q0, int q1) {
#pragma unroll
        for (int q = q0; q < q1; ++q)
            acc[q / FN][q % FN] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][q / FN], fb[buf][q % FN], acc[q / FN][q % FN], 0, 0, 0);
    };
    constexpr int NQ = FM * FN, HQ = NQ / 2;

    // One tile.  SET = kt % 2.  Slices 0-2: a quarter of the loads of tile
    // kt+2, the fragments of the next slice, this slice's MFMAs.  Slice 3:
    // write tile kt+1 to the other stage, publish it, read its first
    // fragments and issue the last quarter of the loads under the remaining
    // MFMAs.
    auto tile = [&](auto set, int kt) {
        constexpr int S = decltype(set)::value;
        const int stage = S;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            if (kk + 1 < KK) {
                gload(set, kt + 2, kk);
                read(stage, kk + 1, nxt);
                mma(cur, 0, NQ);
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // DS read
                    __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);   // VMEM read
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
                lstore(std::integral_constant<int, 1 - S>{}, 1 - S);
                mma(cur, 0, HQ);
#pragma unroll
                for (int q = 0; q < NL; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x0200, 1, 0);   // DS write
                    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
                }
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
                read(1 - S, 0, nxt);
                gload(set, kt + 2, 3);
                mma(cur, HQ, NQ);
#pragma unroll
                for (int q = 0; q < NQ - HQ; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // DS read
                    __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);   // VMEM read
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    using T0 = std::integral_constant<int, 0>;
    using T1 = std::integral_constant<int, 1>;

    // An odd tile count runs one all-zero tile more: the loop body stays free
    // of branches (a tail with its own control flow makes the compiler spill
    // the accumulators).  The last pair also writes and publishes a tile that
    // no MFMA reads.
#pragma unroll
    for (int q = 0; q < 4; ++q) gload(T0{}, 0, q);
#pragma unroll
    for (int q = 0; q < 4; ++q) gload(T1{}, 1, q);
    lstore(T0{}, 0);
    __syncthreads();
    read(0, 0, 0);
    for (int kt = 0; kt < KT; kt += 2) {
        tile(T0{}, kt);
        tile(T1{}, kt + 1);
    }
    epilogue<FM, FN, MODE>(acc, epi, lane, m0 + wm * TM, n0 + wn * TN, M, N);
}

// ---------------------------------------------------------------------------
// Producer/consumer tile, BK 64, twelve waves: 256x256 as 2 x 4 MFMA waves
// of 128x64, 256x192 as 8 x 1 of 32x192, or 256x128 as 4 x 2 of 64x64.
// Waves 0-7 (two per SIMD) only read MFMA fragments from LDS and issue MFMAs;
// waves 8-11 (one per SIMD) only move tiles from global memory into LDS.
// The 256x256 tile's epilogue with the all-reduce's sum (EPI_SUM), shared
// by all twelve waves: the tile goes through LDS as fp32 in two 128-row
// halves, and every thread of the work-group -- producers included, whose
// registers are free once the main loop ends -- streams the other ranks'
// partials and the residual for several 16-byte chunks at a time.  A wave that
// reduces only its own rows keeps about one chunk's loads in flight, its
// accumulators filling the rest of its registers.
constexpr int kCoopRows = 128, kCoopLd = 256 + 4;   // fp32 row stride of the staged half (padded)
constexpr int kCoopChunks = 2;                       // 16-byte chunks in flight per thread (4: no faster)

__device__ __forceinline__ void coop_sum_half(const float* sf, const Epilogue& epi, int row0, int n0, int M, int N,
                                              int tid, int nthreads) {
    constexpr int CPR = 256 / 4;                          // 16-byte chunks per row
    constexpr int NCH = kCoopRows * CPR;
    const int cb = epi.col0;
    bf16* o = (bf16*)epi.out;
    auto one = [&](int c, float (&v)[4], long long& off, bool& ok) {
        const int rl = c / CPR, ch = c % CPR;
        const int row = row0 + rl, col = n0 + ch * 4;
        ok = c < NCH && row < M && col < N;
        off = (long long)row * epi.ldo + cb + col;
        const f32x4 a = *(const f32x4*)(sf + (c < NCH ? rl : 0) * kCoopLd + ch * 4);
        v[0] = a[0];
        v[1] = a[1];
        v[2] = a[2];
        v[3] = a[3];
    };
    auto put = [&](const float (&v)[4], long long off) {
        uint32_t w0 = (uint32_t)f2bf_bits(v[0]) | ((uint32_t)f2bf_bits(v[1]) << 16);
        uint32_t w1 = (uint32_t)f2bf_bits(v[2]) | ((uint32_t)f2bf_bits(v[3]) << 16);
        *(uint2*)(o + off) = make_uint2(w0, w1);
    };
    constexpr int U = kCoopChunks;
    for (int c = tid; c < NCH; c += U * nthreads) {
        float v[U][4];
        long long off[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) one(c + u * nthreads, v[u], off[u], ok[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) sum_ranks<4>(epi.sum, off[u], v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) put(v[u], off[u]);
    }
}

// With the loads and LDS writes on waves of their own, the MFMA waves never
// wait for global memory and never issue a memory-unit instruction.  Two LDS
// stages: while the MFMA waves read tile kt from one, the producers write
// tile kt+1 into the other; one barrier per tile hands both over.  Register
// budget with eight MFMA waves: three waves per SIMD, 168 each (up to 128
// accumulators + one set of fragments; two register sets of staged loads on
// the producers); the rotary epilogue gathers 4 rows at a time to stay inside
// it.  With four MFMA waves (WM x WN = 4) two waves share a SIMD, 256
// registers each: a 64x192 wave tile holds 192 accumulators and reads 0.67
// fragments per MFMA instead of the 32x192 tile's 1.17.
template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(64 * (WM * WN + 4)) void gemm_ws_kernel(const bf16* __restrict__ A, long long lda,
                                                                   const bf16* __restrict__ B, long long ldb,
                                                                   int M, int N, int K, Epilogue epi, int tiles_m,
                                                                   int tiles_n) {
    constexpr int BK = 64, KK = 4;
    constexpr int NW = WM * WN;                  // MFMA waves; the four producer waves follow them
    constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int RS = 32;                       // rows per producer load step (256 threads x 16 B)
    constexpr int NL = (BM + BN) / RS;           // 16-byte loads per producer thread per tile
    static_assert((NW == 8 || NW == 4) && FN % 2 == 0 && BM % RS == 0 && BN % RS == 0, "tile shape");
    // the 256x256 tile's sum epilogue runs on every wave (coop_sum_half)
    constexpr bool COOP = MODE == EPI_SUM && BM == 256 && BN == 256 && WM == 2 && WN == 4;
    constexpr int SMEM = COOP && kCoopRows * kCoopLd * 2 > 2 * STAGE ? kCoopRows * kCoopLd * 2 : 2 * STAGE;
    __shared__ __attribute__((aligned(1024))) bf16 smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (blockIdx.x == 0 && threadIdx.x == 0) apply_len_update(epi.len);
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int KT = K / BK;

    if (wave >= NW) {
        // Producer thread p copies 16-byte chunk (p & 7) of rows (p >> 3) + 32 i
        // of the A tile (i < 8) and the B tile (i >= 8).  Rows past M (N) lie
        // outside the tile's buffer resource and read as zeros; tiles past
        // the end read zeros through an empty resource.
        const int p = tid - 64 * NW, srow = p >> 3, skc = p & 7;
        const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(A + (long long)m0 * lda), (short)0, max(0, min(BM, M - m0)) * (int)lda * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(B + (long long)n0 * ldb), (short)0, max(0, min(BN, N - n0)) * (int)ldb * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t rs0 = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0, 0x00020000);
        int voff[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i)
            voff[i] = i < BM / RS ? ((srow + RS * i) * (int)lda + skc * 8) * 2
                                  : ((srow + RS * (i - BM / RS)) * (int)ldb + skc * 8) * 2;
        const int l0 = srow * BK + (swz<8>(srow, skc) << 3);   // rows srow + 32 i share the swizzle
        u32x4 r[2][NL];
        auto gload = [&](auto set, int kt) {
            constexpr int S = decltype(set)::value;
            const bool in = kt < KT;
            const int koff = in ? kt * BK * 2 : 0;
#pragma unroll
            for (int i = 0; i < NL; ++i)
                r[S][i] = __builtin_amdgcn_raw_buffer_load_b128(in ? (i < BM / RS ? rsa : rsb) : rs0, voff[i], koff, 0);
        };
        auto lstore = [&](auto set, int stage) {
            constexpr int S = decltype(set)::value;
            bf16* sa = smem + stage * STAGE;
#pragma unroll
            for (int i = 0; i < NL; ++i) *(u32x4*)(sa + l0 + i * RS * BK) = r[S][i];
        };
        using T0 = std::integral_constant<int, 0>;
        using T1 = std::integral_constant<int, 1>;
        gload(T0{}, 0);
        gload(T1{}, 1);
        wait_vm<NL>();
        lstore(T0{}, 0);
        __syncthreads();
        // iteration kt: set kt%2 is free (its tile is in LDS), set 1-kt%2 holds tile kt+1
        for (int kt = 0; kt < KT; kt += 2) {
            gload(T0{}, kt + 2);
            wait_vm<NL>();
            lstore(T1{}, 1);
            __syncthreads();
            gload(T1{}, kt + 3);
            wait_vm<NL>();
            lstore(T0{}, 0);
            __syncthreads();
        }
        wait_vm<0>();
        if constexpr (COOP) {
            // the same four barriers as the MFMA waves' epilogue; no rows of their own to stage.
            // Half 0 is reduced by the producers and the waves of row block 0 (512 threads),
            // half 1 by every thread.
            __syncthreads();
            __syncthreads();
            coop_sum_half((const float*)smem, epi, m0, n0, M, N, tid - 256, 512);
            __syncthreads();
            __syncthreads();
            coop_sum_half((const float*)smem, epi, m0 + kCoopRows, n0, M, N, tid, 64 * (NW + 4));
        }
        return;
    }

    // MFMA waves
    const int wm = wave / WN, wn = wave % WN;
    const int frow = lane & 31, khalf = lane >> 5;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16){};
    // Fragments of the next k-slice are read while the current one's MFMAs
    // run: into a second set where the register budget allows two (not with
    // 128 accumulators), else into the registers of the current set that its
    // MFMAs have finished with.
    constexpr bool DB = FM * FN * 16 + 8 * (FM + FN) <= (NW == 4 ? 232 : 152);
    bf16x8 fa[DB ? 2 : 1][FM], fb[DB ? 2 : 1][FN];
    auto rd = [&](int st, int kk, int buf) {
        const bf16* a_s = smem + st * STAGE + (wm * TM + frow) * BK;
        const bf16* b_s = smem + st * STAGE + BM * BK + (wn * TN + frow) * BK;
        const int c = swz<8>(frow, 2 * kk + khalf) << 3;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = *(const bf16x8*)(a_s + i * 32 * BK + c);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = *(const bf16x8*)(b_s + j * 32 * BK + c);
    };
    auto mm = [&](int buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
    };
    __syncthreads();
    // An odd tile count runs one more (all-zero) tile: the loop stays in pairs
    // so that the stage index is static, like the producers' loop.
    if constexpr (DB) {
        rd(0, 0, 0);
        for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const int cur = kk & 1;
                    if (kk + 1 < KK) rd(st, kk + 1, cur ^ 1);
                    mm(cur);
#pragma unroll
                    for (int q = 0; q < FM * FN; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // DS read
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                __syncthreads();
                rd(st ^ 1, 0, 0);   // the next tile's first slice, published by the barrier
            }
        }
    } else if constexpr (FN == 2) {
        // One fragment set, read ahead into the registers the current
        // slice's MFMAs are done with: in B-major order fb[0] is free after
        // the first FM MFMAs of a slice and fa[i] after MFMA (i, 1), so the
        // next slice's fragments are read while the slice's second half runs.
        // The tile's last slice starts with the barrier (its fragments are
        // already in registers), and its MFMAs cover the first reads of the
        // next tile.  Same MFMAs per accumulator, in the same k order.
        auto rd_a = [&](int st, int kk, int i) {
            const bf16* a_s = smem + st * STAGE + (wm * TM + frow) * BK;
            fa[0][i] = *(const bf16x8*)(a_s + i * 32 * BK + (swz<8>(frow, 2 * kk + khalf) << 3));
        };
        auto rd_b = [&](int st, int kk, int j) {
            const bf16* b_s = smem + st * STAGE + BM * BK + (wn * TN + frow) * BK;
            fb[0][j] = *(const bf16x8*)(b_s + j * 32 * BK + (swz<8>(frow, 2 * kk + khalf) << 3));
        };
        // the slice's MFMAs, reading slice (st_n, kk_n) into the freed registers
        auto slice = [&](int st_n, int kk_n) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][i], fb[0][0], acc[i][0], 0, 0, 0);
            rd_b(st_n, kk_n, 0);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][i], fb[0][1], acc[i][1], 0, 0, 0);
                rd_a(st_n, kk_n, i);
            }
            rd_b(st_n, kk_n, 1);
#pragma unroll
            for (int q = 0; q < FM; ++q) __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);                                // DS read
#pragma unroll
            for (int q = 0; q < FM; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);       // DS read
            __builtin_amdgcn_sched_barrier(0);
        };
        rd(0, 0, 0);
        for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int kk = 0; kk < KK - 1; ++kk) slice(st, kk + 1);
                __syncthreads();       // publishes tile kt + st + 1 in the other stage
                slice(st ^ 1, 0);      // (past the last tile: a read whose result is unused)
            }
        }
        // no fragment read of this wave is still in flight when its epilogue
        // writes its part of LDS
        __builtin_amdgcn_s_waitcnt(0xc07f);
    } else if constexpr (FN > 2) {
        // Wide wave tiles (64x192): A fragments in two register sets, B in one.
        // A slice's MFMAs run B-major; the next slice's A fragments are read
        // during the first column of MFMAs, its B fragment j as soon as column
        // j's MFMAs have issued, so every read has at least FM * (FN - 1)
        // MFMAs to land.  Same MFMAs per accumulator, in the same k order.
        bf16x8 xa[2][FM], xb[FN];
        auto rd_a = [&](int st, int kk, int i, int set) {
            const bf16* a_s = smem + st * STAGE + (wm * TM + frow) * BK;
            xa[set][i] = *(const bf16x8*)(a_s + i * 32 * BK + (swz<8>(frow, 2 * kk + khalf) << 3));
        };
        auto rd_b = [&](int st, int kk, int j) {
            const bf16* b_s = smem + st * STAGE + BM * BK + (wn * TN + frow) * BK;
            xb[j] = *(const bf16x8*)(b_s + j * 32 * BK + (swz<8>(frow, 2 * kk + khalf) << 3));
        };
        // the MFMAs of the slice held in set `cur`, reading slice (st_n, kk_n)
        auto slice = [&](auto cur_c, int st_n, int kk_n) {
            constexpr int cur = decltype(cur_c)::value;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[cur][i], xb[j], acc[i][j], 0, 0, 0);
                    if (j == 0) rd_a(st_n, kk_n, i, cur ^ 1);
                }
                rd_b(st_n, kk_n, j);
            }
#pragma unroll
            for (int q = 0; q < FM; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // DS read (A)
            }
            __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);       // DS read (B 0)
#pragma unroll
            for (int q = 1; q < FN; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x0008, FM, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // DS read (B q)
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        static_assert(KK == 4, "set parity per slice");
#pragma unroll
        for (int i = 0; i < FM; ++i) rd_a(0, 0, i, 0);
#pragma unroll
        for (int j = 0; j < FN; ++j) rd_b(0, 0, j);
        for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                slice(S0{}, st, 1);
                slice(S1{}, st, 2);
                slice(S0{}, st, 3);
                __syncthreads();        // publishes tile kt + st + 1 in the other stage
                slice(S1{}, st ^ 1, 0); // (past the last tile: a read whose result is unused)
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
    } else {
        for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    rd(st, kk, 0);
                    mm(0);
                }
                __syncthreads();
            }
        }
    }
    if constexpr (COOP) {
        // Half h holds the rows of MFMA row block h: its four waves stage their
        // 128 x 64 tiles as fp32 rows, then the half is reduced.  Row block 1
        // keeps its accumulators through half 0 and takes no part in reducing
        // it (its registers are full); the paths differ per wave, the barrier
        // count does not.
        float* sf = (float*)smem;
        const int col_in = lane & 31, row_in = 4 * (lane >> 5);
        auto stage = [&]() {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        sf[(i * 32 + 8 * (r >> 2) + row_in + (r & 3)) * kCoopLd + wn * TN + j * 32 + col_in] =
                            acc[i][j][r];
        };
        __syncthreads();   // every wave is past the main loop's LDS reads
        if (wm == 0) {
            stage();
            __syncthreads();
            coop_sum_half(sf, epi, m0, n0, M, N, tid, 512);
            __syncthreads();   // half 0 read out of LDS
            __syncthreads();
        } else {
            __syncthreads();
            __syncthreads();
            stage();
            __syncthreads();
        }
        coop_sum_half(sf, epi, m0 + kCoopRows, n0, M, N, tid, 64 * (NW + 4));
        return;
    }
    // Every wave, producers included, has passed the loop's last barrier:
    // no LDS read or write of the main loop is still pending, so each MFMA
    // wave may use a private part of the stages for its epilogue.
    constexpr int RB = 2 * STAGE / NW;
    constexpr bool staged = (MODE == EPI_SWIGLU && FM * 32 * (FN * 16 + 8) <= RB) ||
                            ((MODE == EPI_F32 || MODE == EPI_SUM) && 32 * (FN * 32 + 4) * 2 <= RB);
    if constexpr (staged)
        epilogue_staged<FM, FN, MODE, RB>(acc, epi, lane, m0 + wm * TM, n0 + wn * TN, M, N, smem + wave * RB);
    else
        epilogue<FM, FN, MODE, 4>(acc, epi, lane, m0 + wm * TM, n0 + wn * TN, M, N);
}

// ---------------------------------------------------------------------------
// Register-staged main loop (two register stages, double-buffered LDS, BK 64).
template <int BM, int BN, int MODE>
__global__ __launch_bounds__(256) void gemm_reg_kernel(const bf16* __restrict__ A, long long lda,
                                                       const bf16* __restrict__ B, long long ldb, int M, int N,
                                                       int K, Epilogue epi, int tiles_m, int tiles_n) {
    constexpr int BK = 64;
    constexpr int TM = BM / 2, TN = BN / 2, FM = TM / 32, FN = TN / 32;
    constexpr int CA = BM * 8 / 256, CB = BN * 8 / 256;  // 16-byte chunks per thread
    static_assert(FN % 2 == 0, "wave N-tile must cover whole 64-column groups");
    __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    if (blockIdx.x == 0 && threadIdx.x == 0) apply_len_update(epi.len);
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // thread t copies 16-byte chunk (t & 7) of tile rows (t >> 3) + 32 i; rows
    // past M (or N) fall outside the buffer resources and read as zeros
    const int srow = tid >> 3, skc = tid & 7;
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t rsa =
        __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long long)m0 * lda), (short)0, rows_a * (int)lda * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb =
        __builtin_amdgcn_make_buffer_rsrc((void*)(B + (long long)n0 * ldb), (short)0, rows_b * (int)ldb * 2, 0x00020000);
    const int va0 = (srow * (int)lda + skc * 8) * 2;
    const int vb0 = (srow * (int)ldb + skc * 8) * 2;
    const int l0 = srow * BK + (swz<8>(srow, skc) << 3);   // (srow + 32 i) has the same swizzle

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16){};

    const int KT = K / BK;
    const int frow = lane & 31, khalf = lane >> 5;
    // Two register stages: the global loads of tile k+2 are issued before the
    // MFMAs of tile k, so each load has two K-steps of compute to arrive.
    // The loop body covers two tiles so that every register set is named
    // statically.
    u32x4 ra0[CA], rb0[CB], ra1[CA], rb1[CB];
#define TP_GLOAD(RA, RB, KT)                                                                             \
    do {                                                                                                 \
        const int koff_ = (KT) * BK * 2;                                                                 \
        _Pragma("unroll") for (int i = 0; i < CA; ++i)                                                   \
            RA[i] = __builtin_amdgcn_raw_buffer_load_b128(rsa, va0 + i * 32 * (int)lda * 2, koff_, 0);   \
        _Pragma("unroll") for (int i = 0; i < CB; ++i)                                                   \
            RB[i] = __builtin_amdgcn_raw_buffer_load_b128(rsb, vb0 + i * 32 * (int)ldb * 2, koff_, 0);   \
    } while (0)
#define TP_LSTORE(RA, RB, BUF)                                                                           \
    do {                                                                                                 \
        _Pragma("unroll") for (int i = 0; i < CA; ++i) *(u32x4*)(&sA[BUF][l0 + i * 32 * BK]) = RA[i];    \
        _Pragma("unroll") for (int i = 0; i < CB; ++i) *(u32x4*)(&sB[BUF][l0 + i * 32 * BK]) = RB[i];    \
    } while (0)
#define TP_COMPUTE(BUF) \
    mma_stage<FM, FN, BK, 8>(acc, sA[BUF] + (wm * TM + frow) * BK, sB[BUF] + (wn * TN + frow) * BK, frow, khalf)

    TP_GLOAD(ra0, rb0, 0);
    TP_GLOAD(ra1, rb1, min(1, KT - 1));
    TP_LSTORE(ra0, rb0, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        // buffer 0 holds tile kt; ra1/rb1 carry tile kt+1
        TP_GLOAD(ra0, rb0, min(kt + 2, KT - 1));
        TP_COMPUTE(0);
        TP_LSTORE(ra1, rb1, 1);
        __syncthreads();
        // buffer 1 holds tile kt+1; ra0/rb0 carry tile kt+2
        TP_GLOAD(ra1, rb1, min(kt + 3, KT - 1));
        TP_COMPUTE(1);
        if (kt + 2 < KT) TP_LSTORE(ra0, rb0, 0);
        __syncthreads();
    }
    if (kt < KT) TP_COMPUTE(0);  // odd tile count: the last tile sits in buffer 0
#undef TP_GLOAD
#undef TP_LSTORE
#undef TP_COMPUTE
    epilogue<FM, FN, MODE>(acc, epi, lane, m0 + wm * TM, n0 + wn * TN, M, N);
}

struct Cfg {
    int bm, bn;
    float eff;   // relative MFMA efficiency of one work-group (measured on the 7B/70B shapes)
    int occ;     // work-groups per CU
};
// index: 0-2 register-staged, 3-10 DMA ring, 11-12 register-pipelined
const Cfg kCfgs[] = {
    {256, 128, 0.86f, 1},  // 0 reg 256x128
    {128, 128, 0.90f, 2},  // 1 reg 128x128
    {128, 256, 0.88f, 1},  // 2 reg 128x256
    {256, 256, 1.00f, 1},  // 3 dma 256x256 BK64 ST2
    {256, 256, 1.03f, 1},  // 4 dma 256x256 BK32 ST4
    {256, 128, 0.95f, 1},  // 5 dma 256x128 BK64 ST3
    {128, 128, 0.78f, 1},  // 6 dma 128x128 BK64 ST4
    {128, 128, 0.90f, 2},  // 7 dma 128x128 BK64 ST2
    {256, 128, 0.85f, 1},  // 8 dma 256x128 BK32 ST4
    {128, 384, 0.95f, 1},  // 9 dma 128x384 BK32 ST4
    {128, 384, 0.95f, 1},  // 10 dma 128x384 BK32 ST3
    {256, 256, 1.08f, 1},  // 11 register-pipelined 256x256 BK64, 8 waves
    {256, 128, 1.00f, 1},  // 12 register-pipelined 256x128 BK64, 8 waves
    {256, 192, 0.84f, 1},  // 13 register-pipelined 256x192 BK64, 8 waves of 32x192
    {256, 256, 1.12f, 1},  // 14 producer/consumer 256x256 BK64, 8 MFMA waves + 4 load waves
    {256, 192, 1.10f, 1},  // 15 producer/consumer 256x192 BK64, 8 MFMA waves of 32x192 + 4 load waves
    {256, 128, 1.02f, 1},  // 16 producer/consumer 256x128 BK64, 8 MFMA waves of 64x64 + 4 load waves
    {256, 192, 1.13f, 1},  // 17 producer/consumer 256x192 BK64, 4 MFMA waves of 64x192 + 4 load waves
    {256, 128, 1.05f, 1},  // 18 producer/consumer 256x128 BK64, 4 MFMA waves of 64x128 + 4 load waves
};
constexpr int kNumCfg = sizeof(kCfgs) / sizeof(kCfgs[0]);
int g_forced_cfg = -1;
// forced two-launch split (tests): the first g_split_cols columns with
// configuration g_split_cfg[0], the rest with g_split_cfg[1]; 0 = off
int g_split_cols = 0;
int g_split_cfg[2] = {0, 0};

struct Args {
    const bf16* A;
    long long lda;
    const bf16* B;
    long long ldb;
    int M, N, K;
    Epilogue epi;
    hipStream_t st;
};

template <int BM, int BN, int BK, int ST, int MODE>
void launch_dma(const Args& a) {
    const int tm = cdiv(a.M, BM), tn = cdiv(a.N, BN);
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, BK, ST, MODE>), dim3(tm * tn), dim3(256), 0, a.st, a.A, a.lda, a.B,
                       a.ldb, a.M, a.N, a.K, a.epi, tm, tn);
}
template <int BM, int BN, int BK, int ST, int MODE>
void launch_pipe(const Args& a) {
    const int tm = cdiv(a.M, BM), tn = cdiv(a.N, BN);
    hipLaunchKernelGGL((gemm_dma_pipe_kernel<BM, BN, BK, ST, MODE>), dim3(tm * tn), dim3(256), 0, a.st, a.A, a.lda,
                       a.B, a.ldb, a.M, a.N, a.K, a.epi, tm, tn);
}
template <int BM, int BN, int WM, int WN, int MODE>
void launch_ws(const Args& a) {
    const int tm = cdiv(a.M, BM), tn = cdiv(a.N, BN);
    hipLaunchKernelGGL((gemm_ws_kernel<BM, BN, WM, WN, MODE>), dim3(tm * tn), dim3(64 * (WM * WN + 4)), 0, a.st, a.A,
                       a.lda, a.B, a.ldb, a.M, a.N, a.K, a.epi, tm, tn);
}

template <int BM, int BN, int WM, int WN, int MODE>
void launch_vgpr(const Args& a) {
    const int tm = cdiv(a.M, BM), tn = cdiv(a.N, BN);
    hipLaunchKernelGGL((gemm_vgpr_kernel<BM, BN, WM, WN, MODE>), dim3(tm * tn), dim3(64 * WM * WN), 0, a.st, a.A,
                       a.lda, a.B, a.ldb, a.M, a.N, a.K, a.epi, tm, tn);
}
template <int BM, int BN, int MODE>
void launch_reg(const Args& a) {
    const int tm = cdiv(a.M, BM), tn = cdiv(a.N, BN);
    hipLaunchKernelGGL((gemm_reg_kernel<BM, BN, MODE>), dim3(tm * tn), dim3(256), 0, a.st, a.A, a.lda, a.B, a.ldb,
                       a.M, a.N, a.K, a.epi, tm, tn);
}

template <int MODE>
void launch_cfg(int c, const Args& a) {
    switch (c) {
        case 0: launch_reg<256, 128, MODE>(a); break;
        case 1: launch_reg<128, 128, MODE>(a); break;
        case 2: launch_reg<128, 256, MODE>(a); break;
        case 3: launch_dma<256, 256, 64, 2, MODE>(a); break;
        case 4: launch_pipe<256, 256, 32, 4, MODE>(a); break;
        case 5: launch_pipe<256, 128, 64, 3, MODE>(a); break;
        case 6: launch_pipe<128, 128, 64, 4, MODE>(a); break;
        case 7: launch_dma<128, 128, 64, 2, MODE>(a); break;
        case 8: launch_pipe<256, 128, 32, 4, MODE>(a); break;
        case 9: launch_pipe<128, 384, 32, 4, MODE>(a); break;
        case 10: launch_pipe<128, 384, 32, 3, MODE>(a); break;
        case 11: launch_vgpr<256, 256, 2, 4, MODE>(a); break;
        case 12: launch_vgpr<256, 128, 4, 2, MODE>(a); break;
        case 13: launch_vgpr<256, 192, 8, 1, MODE>(a); break;
        case 14: launch_ws<256, 256, 2, 4, MODE>(a); break;
        case 15: launch_ws<256, 192, 8, 1, MODE>(a); break;
        case 16: launch_ws<256, 128, 4, 2, MODE>(a); break;
        case 17:
            // the rotary epilogue does not fit beside 192 accumulators (usable() keeps it away)
            if constexpr (MODE != EPI_QKV) launch_ws<256, 192, 4, 1, MODE>(a);
            break;
        default: launch_ws<256, 128, 4, 1, MODE>(a); break;
    }
}

// The 256x256 DMA kernels hold 256 accumulators per lane: the two-stage one
// spills them with the rotary, erf and plain-store epilogues, the four-stage
// ring with the rotary one.  The four-wave 256x192 producer/consumer tile's
// 192 accumulators leave no room for the rotary epilogue either.
bool usable(int c, int mode) {
    if (c == 3 && (mode == EPI_QKV || mode == EPI_GELU || mode == EPI_STORE)) return false;
    return !((c == 4 || c == 17) && mode == EPI_QKV);
}

// Modelled time of one launch: rounds of 256 tiles (one per CU), each the
// tile's FLOPs at the configuration's per-CU rate, plus a launch.  The DMA
// rings lose 20% with the rotary epilogue (measured on the 7B Q/K/V shape);
// the register-pipelined kernels do not.
constexpr double kCuFlopPerUs = 4.7e6;   // per-CU bf16 rate of a configuration with eff = 1
constexpr double kLaunchUs = 3.0;

double model_us(int c, int mode, int M, int N, int K) {
    const Cfg& f = kCfgs[c];
    const long long tiles = (long long)cdiv(M, f.bm) * cdiv(N, f.bn);
    double eff = f.eff * ((c >= 3 && c <= 10 && mode == EPI_QKV) ? 0.8 : 1.0);
    // the four-wave 256x192 tile beat the eight-wave one only with the SwiGLU
    // epilogue (7B gate/up 167-168 against 174-186 us); with the fp32 partial
    // it ran 1-6 % behind the 256x128 and 256x256 tiles
    if (c == 17 && mode != EPI_SWIGLU) eff = 0.95f;
    // the four-wave 256x128 tile beat the eight-wave one with the fp32
    // partial (7B out and down 2-5 % faster), not with the other epilogues
    if (c == 18 && mode != EPI_F32 && mode != EPI_SUM) eff = 0.95f;
    // a configuration with `occ` work-groups per CU reaches its rate only with all of them resident: a
    // round is 256 * occ tiles and costs occ tiles' time, however few tiles the last round has
    const long long per_round = 256LL * f.occ;
    return kLaunchUs + (double)((tiles + per_round - 1) / per_round) * f.occ * 2.0 * f.bm * f.bn * K /
                           (eff * kCuFlopPerUs);
}

// A GEMM runs as one launch, or as two over column ranges: the first covers
// whole rounds of a large tile, the second the remaining columns with a
// smaller tile, so that the last round is not mostly idle (the tile count of
// a shape like 2048 x 11008 leaves 88 of 344 tiles for a second round).
struct Plan {
    int parts;
    int cfg[2];
    int c0[2], ncols[2];
};

Plan plan(int M, int N, int K, int mode) {
    Plan best{1, {1, 1}, {0, 0}, {N, 0}};
    if (g_split_cols > 0 && g_split_cols < N && usable(g_split_cfg[0], mode) && usable(g_split_cfg[1], mode))
        return Plan{2, {g_split_cfg[0], g_split_cfg[1]}, {0, g_split_cols}, {g_split_cols, N - g_split_cols}};
    if (g_forced_cfg >= 0 && g_forced_cfg < kNumCfg && usable(g_forced_cfg, mode)) {
        best.cfg[0] = g_forced_cfg;
        return best;
    }
    double best_t = 1e30;
    for (int c = 0; c < kNumCfg; ++c) {
        if (!usable(c, mode)) continue;
        const double t = model_us(c, mode, M, N, K);
        if (t < best_t * 0.999) {
            best_t = t;
            best = Plan{1, {c, c}, {0, 0}, {N, 0}};
        }
    }
    Plan split{};
    double split_t = 1e30;
    for (int b = 0; b < kNumCfg; ++b) {
        if (!usable(b, mode) || kCfgs[b].occ != 1) continue;
        const int tiles_m = cdiv(M, kCfgs[b].bm);
        if (tiles_m > 256) continue;
        const int round_cols = (256 / tiles_m) * kCfgs[b].bn;
        const int n_big = (N / round_cols) * round_cols;
        if (n_big == 0 || n_big == N) continue;
        const double t_big = model_us(b, mode, M, n_big, K);
        for (int c = 0; c < kNumCfg; ++c) {
            if (!usable(c, mode)) continue;
            const double t = t_big + model_us(c, mode, M, N - n_big, K);
            if (t < split_t * 0.999) {
                split_t = t;
                split = Plan{2, {b, c}, {0, n_big}, {n_big, N - n_big}};
            }
        }
    }
    return split_t < best_t * 0.97 ? split : best;   // a second launch must clearly pay for itself
}

}  // namespace

void set_gemm_config(int cfg) { g_forced_cfg = cfg; }
int gemm_config_count() { return kNumCfg; }

void set_gemm_split(int cfg0, int cfg1, int cols0) {
    g_split_cfg[0] = cfg0;
    g_split_cfg[1] = cfg1;
    g_split_cols = cols0;
}

void gemm_plan_info(int M, int N, int K, int mode, int* parts, int cfg[2], int ncols[2]) {
    const Plan p = plan(M, N, K, mode);
    *parts = p.parts;
    for (int i = 0; i < 2; ++i) {
        cfg[i] = i < p.parts ? p.cfg[i] : -1;
        ncols[i] = i < p.parts ? p.ncols[i] : 0;
    }
}

void gemm_bf16(const bf16* A, long long lda, const bf16* B, long long ldb, int M, int N, int K,
               const Epilogue& epi, hipStream_t st) {
    const Plan p = plan(M, N, K, epi.mode);
    for (int i = 0; i < p.parts; ++i) {
        Epilogue e = epi;
        e.col0 = epi.col0 + p.c0[i];
        if (i > 0) e.len = LenUpdate{nullptr, 0, 0, nullptr};   // one launch updates the cache length
        const Args a{A, lda, B + (long long)p.c0[i] * ldb, ldb, M, p.ncols[i], K, e, st};
        switch (epi.mode) {
            case EPI_F32: launch_cfg<EPI_F32>(p.cfg[i], a); break;
            case EPI_QKV: launch_cfg<EPI_QKV>(p.cfg[i], a); break;
            case EPI_SWIGLU: launch_cfg<EPI_SWIGLU>(p.cfg[i], a); break;
            case EPI_GELU: launch_cfg<EPI_GELU>(p.cfg[i], a); break;
            case EPI_SUM: launch_cfg<EPI_SUM>(p.cfg[i], a); break;
            default: launch_cfg<EPI_STORE>(p.cfg[i], a); break;
        }
    }
}

}  // namespace tp
