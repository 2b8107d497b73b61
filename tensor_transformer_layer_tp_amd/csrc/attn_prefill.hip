// Causal attention over one rank's own heads (prefill), bf16 MFMA, fp32 softmax.
//
// Each rank attends locally over the heads it owns; no other rank's data is
// needed (undercodenews post 110319 on tensor parallelism, sections "the
// Original" and "What Undercode Say": heads are independent, so the
// column-parallel split of Q/K/V needs no communication inside attention).
//
// Work-group = 4 waves (or 2 x 4, see below) = 128 queries of one (batch,
// head); each wave owns 32 queries.  Keys stream through LDS in blocks of
// 64.  The wave computes the transposed score tile S^T = K Q^T
// (v_mfma_f32_32x32x16_bf16, K block as the A operand from LDS, the wave's Q
// fragment held in registers as the B operand), so that every lane owns ONE
// query column: the online-softmax
// row max / row sum is a per-lane reduction over 16 registers plus one
// exchange between the two 32-lane halves.  The probabilities are then fed
// straight from the accumulator registers as the B operand of
// O^T += V^T P^T.  Grouped-query attention maps query head j to KV head
// j / (Hl / Hkvl).
//
// Two kernels share this structure.  attn_prefill_pipe (the default) loads K
// and V straight into two LDS stages each and reads the P·V operand from
// row-major V with the transposing LDS read; attn_prefill_kernel stages each
// block through registers into one LDS stage, with V stored transposed and
// its keys permuted to the accumulator's register order.
#include "common.h"

namespace tp {

namespace {

constexpr int BQ = 128, BKV = 64;

// LDS position of key k (0..63) inside a transposed V row: keys are ordered
// to match the PV MFMA operand, (16j + 4h + p%4 + 8(p/4)) -> 16j + 8h + p.
__device__ __forceinline__ int vt_pos(int k) {
    const int j = k >> 4, w = k & 15;
    return (j << 4) + (((w >> 2) & 1) << 3) + (w & 3) + ((w >> 3) << 2);
}

// 16-byte chunk slot of chunk c in LDS row r: 16 lanes reading 16 consecutive
// rows hit 16 distinct bank groups (256-byte rows: r & 15; 128-byte rows:
// consecutive even and odd rows alternate halves, so (r >> 1) & 7).
template <int CPR>
__device__ __forceinline__ int kslot(int r, int c) {
    return CPR == 16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

// The other 32-lane half's value of v, one VALU op (no LDS round trip): the
// half swap leaves each lane its own value in one result and its partner's
// in the other, so max and sum over the pair are the same in every lane.
__device__ __forceinline__ float half_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// KG key groups of 4 waves: group g takes the key blocks kb = g (mod KG) for
// the same 128 queries, with its own LDS buffers and online-softmax state;
// the states merge through LDS at the end.  KG = 2 halves the critical path
// of the longest (latest) query blocks and puts two waves on each SIMD when
// the grid alone would give one.
template <int D, int KG>
__global__ __launch_bounds__(256 * KG, 2 / KG) void attn_prefill_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, bf16* __restrict__ O,
    int hl, int kvl, int S, int ld_seq, float scale_log2, int B) {
    constexpr int KC = D / 8;        // 16-byte chunks per K row
    constexpr int NT = D / 32;       // O^T tiles (32 dims each)
    constexpr int KSTEPS = D / 16;   // k16 steps of the QK^T contraction
    constexpr int BUF = 2 * BKV * D;                      // bf16 per group: K block + transposed V block
    // staging row (bf16): padded against bank conflicts where the registers
    // allow it (the one-group kernel spills with the padded addressing)
    constexpr int OROW = KG > 1 ? D + 8 : D;
    constexpr int MERGE = (KG > 1 ? 4 * NT * 16 * 64 + 2 * 256 : 0) * 2;   // fp32 merge area, in bf16 units
    constexpr int STAGE_O = 4 * 32 * OROW;
    constexpr int SMEM = (KG * BUF > MERGE ? (KG * BUF > STAGE_O ? KG * BUF : STAGE_O)
                                           : (MERGE > STAGE_O ? MERGE : STAGE_O));
    __shared__ __attribute__((aligned(16))) bf16 smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: block starts stay scalar
    const int grp = KG > 1 ? wave >> 2 : 0, qw = KG > 1 ? wave & 3 : wave, gtid = KG > 1 ? tid & 255 : tid;
    bf16* sK = smem + grp * BUF;
    bf16* sVt = sK + BKV * D;
    const int h = lane >> 5, col = lane & 31;
    // Work-group -> (query block, head, sequence): the query block is the
    // slowest index, counted from the latest (longest) one, so the whole grid
    // goes out in order of decreasing work and the dispatcher can pack the
    // short blocks behind the long ones.
    const int nqb = (S + BQ - 1) / BQ;
    const int nhb = hl * B;
    const int rank = blockIdx.x / nhb, hb = blockIdx.x - rank * nhb;
    const int qb = nqb - 1 - rank;
    const int head = hb % hl, b = hb / hl;
    const int kvh = head / (hl / kvl);
    const int q0 = qb * BQ + qw * 32;
    const int qme = q0 + col;                  // this lane's query

    const bf16* Kb = K + ((long long)b * kvl + kvh) * ld_seq * D;
    const bf16* Vb = V + ((long long)b * kvl + kvh) * ld_seq * D;

    bf16x8 qf[KSTEPS];
    {
        const int qrow = min(qme, S - 1);
        const bf16* qp = Q + (((long long)b * hl + head) * S + qrow) * D + 8 * h;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = *(const bf16x8*)(qp + 16 * kk);
    }

    f32x16 oacc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) oacc[i] = (f32x16){};
    float m_run = -INFINITY, l_run = 0.f;

    const int kv_end = min(S, qb * BQ + BQ);
    const int nkb = (kv_end + BKV - 1) / BKV;
    const int nit = (nkb + KG - 1) / KG;

    // The group's next block is fetched into registers while its current one
    // is computed from LDS.  Each block is read through a buffer resource
    // that covers only its rows below S, so rows past the sequence (and whole
    // blocks past it) read as zeros: every load is issued unconditionally,
    // with per-lane offsets that stay the same for every block.
    constexpr int KLD = BKV * KC / 256;         // K chunks per thread
    constexpr int VLD = (BKV / 2) * KC / 256;   // V key pairs per thread
    u32x4 kreg[KLD];
    u32x4 vreg[VLD][2];
    int koff[KLD], voff[VLD][2];
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
        const int idx = gtid + 256 * i;
        koff[i] = ((idx / KC) * D + (idx % KC) * 8) * 2;
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
        const int idx = gtid + 256 * i;
        const int a = idx % (BKV / 2), dc = idx / (BKV / 2);
        voff[i][0] = ((2 * a) * D + dc * 8) * 2;
        voff[i][1] = ((2 * a + 1) * D + dc * 8) * 2;
    }
    auto fetch = [&](int k0) {
        const int bytes = __builtin_amdgcn_readfirstlane(max(0, min(BKV, S - k0)) * D * 2);   // uniform
        const long long base = (long long)min(k0, S) * D;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(Kb + base), (short)0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(Vb + base), (short)0, bytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < KLD; ++i) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[i], 0, 0);
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            vreg[i][0] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i][0], 0, 0);
            vreg[i][1] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i][1], 0, 0);
        }
    };
    // byte selectors of v_perm_b32 that pack the low (high) bf16 halves of two words
    constexpr uint32_t SEL_LO = 0x05040100u, SEL_HI = 0x07060302u;
    const uint32_t sel_even = h ? SEL_HI : SEL_LO, sel_odd = h ? SEL_LO : SEL_HI;
    fetch(grp * BKV);
    for (int it = 0; it < nit; ++it) {
        const int k0 = (it * KG + grp) * BKV;
        __syncthreads();
        // K block -> LDS [key][dim], chunk swizzled by key
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int idx = gtid + 256 * i;
            const int key = idx / KC, dc = idx % KC;
            *(u32x4*)(sK + key * D + (kslot<KC>(key, dc) << 3)) = kreg[i];
        }
        // V block -> LDS transposed [dim][permuted key], two keys per 32-bit store
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int idx = gtid + 256 * i;
            const int a = idx % (BKV / 2), dc = idx / (BKV / 2);
            const u32x4 v0 = vreg[i][0], v1 = vreg[i][1];
            const int p = vt_pos(2 * a);
#pragma unroll
            for (int e0 = 0; e0 < 8; ++e0) {
                // the two 32-lane halves write rows of opposite parity (distinct banks);
                // register indices stay static, the upper half takes the partner element
                // (the other bf16 half of the same word: one byte permute per store)
                const uint32_t w = __builtin_amdgcn_perm(v1[e0 >> 1], v0[e0 >> 1], (e0 & 1) ? sel_odd : sel_even);
                const int dim = dc * 8 + (e0 ^ h);
                const int off = dim * BKV + ((((p >> 3) ^ ((dim >> 1) & 7)) << 3) | (p & 7));
                *(uint32_t*)(sVt + off) = w;
            }
        }
        __syncthreads();
        fetch(k0 + KG * BKV);
        if (k0 > q0 + 31) continue;  // every key of this block is after every query of the wave
        // S^T tile: keys (32t + row) x this wave's 32 queries
        f32x16 st[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            st[t] = (f32x16){};
            const int krow = 32 * t + col;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const bf16x8 a = *(const bf16x8*)(sK + krow * D + (kslot<KC>(krow, 2 * kk + h) << 3));
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], st[t], 0, 0, 0);
            }
        }
        // causal mask only where the block reaches past the wave's first query
        const bool diag = k0 + BKV - 1 > q0;
        // the max is taken on the raw scores and scaled once (the scale is
        // positive); the exponent below is one fma per score
        // (a branch of its own on the uniform flag: folded into the loop
        // below, the compares and selects would run on every block)
        if (diag) {
            const int lim = qme - k0 - 4 * h;   // masked: 32t + 8(r/4) + r%4 > lim
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    st[t][r] = 32 * t + 8 * (r >> 2) + (r & 3) > lim ? -INFINITY : st[t][r];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[t][r]);
        mx = half_max(mx) * scale_log2;
        // The running max is raised (and the output rescaled) only when a score
        // exceeds it by more than 2^8: softmax does not depend on the reference
        // value, so a stale max only scales P and l by the same factor <= 2^8.
        if (__any(mx > m_run + 8.f)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NT; ++i) oacc[i] *= alpha;
        }
        float lsum = 0.f;
        const float neg_m = -m_run;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(st[t][r], scale_log2, neg_m));
                st[t][r] = p;
                lsum += p;
            }
        l_run += lsum;

        // O^T[dim][q] += V^T[dim][key] P^T[key][q], 16 keys per MFMA
#pragma unroll
        for (int j = 0; j < BKV / 16; ++j) {
            bf16x8 pb;
#pragma unroll
            for (int p = 0; p < 8; ++p) pb[p] = f2bf(st[j >> 1][8 * (j & 1) + p]);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const int dim = 32 * i + col;
                const bf16x8 a = *(const bf16x8*)(sVt + dim * BKV + (((2 * j + h) ^ ((dim >> 1) & 7)) << 3));
                oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[i], 0, 0, 0);
            }
        }
    }

    if constexpr (KG > 1) {
        // group 1 hands its state to group 0 through LDS: the same (wave,
        // lane) slot holds the same query and dims in both groups
        float* mo = (float*)smem;
        float* mm = mo + 4 * NT * 16 * 64;
        float* ml = mm + 256;
        __syncthreads();   // every group is done with its K/V buffers
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) mo[((qw * NT + i) * 16 + r) * 64 + lane] = oacc[i][r];
            mm[qw * 64 + lane] = m_run;
            ml[qw * 64 + lane] = l_run;
        }
        __syncthreads();
        if (grp == 0) {
            const float m1 = mm[qw * 64 + lane], l1 = ml[qw * 64 + lane];
            const float m = fmaxf(m_run, m1);   // group 0 always saw key 0: m_run is finite
            const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
            l_run = l_run * a0 + l1 * a1;
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    oacc[i][r] = oacc[i][r] * a0 + mo[((qw * NT + i) * 16 + r) * 64 + lane] * a1;
        }
        __syncthreads();   // the staging below reuses the merge area
    } else {
        __syncthreads();   // the staging below reuses the K/V buffers
    }

    // normalise and store through LDS so that the global writes are whole rows
    if (grp == 0) {
        const float l_tot = half_sum(l_run);
        const float inv = 1.f / l_tot;
        bf16* sO = smem + qw * 32 * OROW;   // 32 queries x D per wave
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dim = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                sO[col * OROW + dim] = f2bf(oacc[i][r] * inv);
            }
    }
    __syncthreads();
    if (grp == 0) {
        const bf16* sO = smem + qw * 32 * OROW;
        const long long ldo = (long long)hl * D;
#pragma unroll
        for (int i = 0; i < 32 * KC / 64; ++i) {
            const int idx = lane + 64 * i;
            const int qr = idx / KC, dc = idx % KC;
            const int q = q0 + qr;
            if (q < S)
                *(bf16x8*)(O + ((long long)b * S + q) * ldo + head * D + dc * 8) = *(const bf16x8*)(sO + qr * OROW + dc * 8);
        }
    }
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer straight into LDS: a wave fills 1 KB at
// the (wave-uniform) LDS byte address lds, lane L at lds + 16 L.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, int voff, uint32_t lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(uintptr_t)lds, 16, voff, 0, 0, 0);
}

// Software-pipelined form of the same computation.  K and V reach LDS by
// direct loads (no register staging), each key group holding two stages of
// each, so one barrier per key block suffices: after barrier i the waves
// compute the scores of block i+1 from one K stage while the exponentials of
// block i run, then P·V of block i from one V stage, while K of block i+2
// and V of block i+1 land in the stages that blocks i and i-1 freed.
//
// V stays row-major in LDS and the P·V operand is read with the gfx950
// transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// i receives element i % 4 of the 8-byte rows that lanes i/4, i/4 + 4, i/4 +
// 8 and i/4 + 12 of the group address.  Lane r of group g therefore points at
// key 16 j + 4 (g / 2) + r / 4, dims 32 T + 16 (g % 2) + 4 (r % 4) .. + 3; two
// such reads (keys + 8) give lane (col, h) the dims-32T+col column of the 8
// keys that its P^T operand holds.
//
// The running max starts at a finite floor instead of -inf, so a key block
// that is masked for every query of a wave contributes exp2(-inf) = 0 with no
// branch around it; the row sum adds the bf16 probabilities that P·V uses.
template <int D>
__device__ __forceinline__ int vswz(int key) {   // 16-byte chunk XOR of a V row
    return D == 128 ? (key & 3) << 2 : ((key >> 1) & 1) << 2;
}

template <int D, int KG>
__global__ __launch_bounds__(256 * KG, 2 / KG) void attn_prefill_pipe(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, bf16* __restrict__ O,
    int hl, int kvl, int S, int ld_seq, float scale_log2, int B) {
    constexpr int KC = D / 8;
    constexpr int NT = D / 32;
    constexpr int KSTEPS = D / 16;
    constexpr int BLK = BKV * D;    // bf16 of one K or V block
    constexpr int GBUF = 4 * BLK;   // per group: K stages 0, 1 and V stages 0, 1
    constexpr int OROW = KG > 1 ? D + 8 : D;
    constexpr int MERGE = (KG > 1 ? 4 * NT * 16 * 64 + 2 * 256 : 0) * 2;
    constexpr int STAGE_O = 4 * 32 * OROW;
    constexpr int SMEM = cmax(cmax(KG * GBUF, MERGE), STAGE_O);
    __shared__ __attribute__((aligned(16))) bf16 smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = KG > 1 ? wave >> 2 : 0, qw = KG > 1 ? wave & 3 : wave;
    bf16* const gbuf = smem + grp * GBUF;
    const uint32_t gbuf_lds = (uint32_t)(uintptr_t)gbuf;
    const int h = lane >> 5, col = lane & 31;
    const int nqb = (S + BQ - 1) / BQ;
    const int nhb = hl * B;
    const int rank = blockIdx.x / nhb, hb = blockIdx.x - rank * nhb;
    const int qb = nqb - 1 - rank;
    const int head = hb % hl, b = hb / hl;
    const int kvh = head / (hl / kvl);
    const int q0 = qb * BQ + qw * 32;
    const int qme = q0 + col;

    const bf16* Kb = K + ((long long)b * kvl + kvh) * ld_seq * D;
    const bf16* Vb = V + ((long long)b * kvl + kvh) * ld_seq * D;

    bf16x8 qf[KSTEPS];
    {
        const int qrow = min(qme, S - 1);
        const bf16* qp = Q + (((long long)b * hl + head) * S + qrow) * D + 8 * h;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = *(const bf16x8*)(qp + 16 * kk);
    }

    f32x16 oacc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) oacc[i] = (f32x16){};
    float m_run = -1e30f, l_run = 0.f;

    const int kv_end = min(S, qb * BQ + BQ);
    const int nkb = (kv_end + BKV - 1) / BKV;
    const int nit = (nkb + KG - 1) / KG;

    // Direct loads, 1 KB per wave instruction: lane L of instruction i of
    // wave w fills slot L % KC of row (w NLD + i) RPK + L / KC and reads the
    // chunk that the row's swizzle puts in that slot.
    constexpr int NLD = BKV * KC / 256;   // direct loads per wave per block (K or V)
    constexpr int RPK = 512 / D;          // rows per 1 KB
    int kdoff[NLD], vdoff[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int row = (qw * NLD + i) * RPK + lane / KC, slot = lane % KC;
        kdoff[i] = (row * D + kslot<KC>(row, slot) * 8) * 2;
        vdoff[i] = (row * D + (slot ^ vswz<D>(row)) * 8) * 2;
    }
    // block j of this group starts at key (j KG + grp) BKV; rows at or past S
    // (and whole blocks past it) read as zeros through the resource's extent
    auto dma = [&](const bf16* base_ptr, const int (&off)[NLD], int j, int buf) {
        const int k0 = (j * KG + grp) * BKV;
        const int bytes = __builtin_amdgcn_readfirstlane(max(0, min(BKV, S - k0)) * D * 2);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(base_ptr + (long long)min(k0, S) * D), (short)0, bytes, 0x00020000);
        const uint32_t lds = gbuf_lds + buf * BLK * 2 + qw * NLD * 1024;
#pragma unroll
        for (int i = 0; i < NLD; ++i) load_lds16(r, off[i], __builtin_amdgcn_readfirstlane(lds + i * 1024));
    };
    auto dma_k = [&](int j, int stage) { dma(Kb, kdoff, j, stage); };
    auto dma_v = [&](int j, int stage) { dma(Vb, vdoff, j, 2 + stage); };

    auto scores = [&](int stage, f32x16(&st)[2]) {
        const bf16* sK = gbuf + stage * BLK;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            st[t] = (f32x16){};
            const int krow = 32 * t + col;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const bf16x8 a = *(const bf16x8*)(sK + krow * D + (kslot<KC>(krow, 2 * kk + h) << 3));
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], st[t], 0, 0, 0);
            }
        }
    };
    // byte offset of this lane's transposed-read row for tile T of a V stage
    // (key 16 j + 4 h + r / 4 of the group, + 8 for the second read)
    const int r16 = lane & 15, gh = (lane >> 4) & 1;
    const int vkey = 4 * h + (r16 >> 2);
    int vtoff[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
        const int c = 4 * T + 2 * gh + ((r16 & 3) >> 1);
        vtoff[T] = vkey * D * 2 + ((c ^ vswz<D>(vkey)) << 4) + ((r16 & 1) << 3);
    }
    // (the compiler cannot tell these reads from the destinations of direct
    // loads in flight, so it waits for every outstanding one before the
    // first of them; plain 16-byte reads of the shared array are not held)
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    auto pv = [&](int stage, const bf16x8 (&pb)[BKV / 16]) {
        const bf16* base = gbuf + (2 + stage) * BLK;
#pragma unroll
        for (int j = 0; j < BKV / 16; ++j)
#pragma unroll
            for (int T = 0; T < NT; ++T) {
                const bf16* a0 = base + (vtoff[T] >> 1) + j * 16 * D;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a0);
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 8 * D));
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[j], oacc[T], 0, 0, 0);
            }
    };

    // prologue: K of blocks 0 and 1 and V of block 0 in LDS, scores of block
    // 0 in registers.  Block i loads K of block i+2 into the stage that K of
    // block i held, so every wave must have read the scores of block 0 first.
    dma_k(0, 0);
    dma_k(1, 1);
    dma_v(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the direct loads have landed
    __syncthreads();
    f32x16 sa[2], sb[2];   // scores of the current and the next block, alternating
    scores(0, sa);
    __syncthreads();

    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
    // one key block; LAST is a constant at both call sites, so its branches fold
    auto block = [&](int it, f32x16(&sc)[2], f32x16(&sn)[2], const bool LAST) __attribute__((always_inline)) {
        const int k0 = (it * KG + grp) * BKV;
        if (!LAST) {
            // the last barrier freed the stages of K of block it and V of block it-1
            if (it + 2 < nit) dma_k(it + 2, it & 1);
            dma_v(it + 1, (it + 1) & 1);
        }
        if (k0 + BKV - 1 > q0) {   // causal mask where the block reaches past the wave's first query
            const int lim = qme - k0 - 4 * h;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sc[t][r] = 32 * t + 8 * (r >> 2) + (r & 3) > lim ? -INFINITY : sc[t][r];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
        mx = half_max(mx) * scale_log2;
        if (__any(mx > m_run + 8.f)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NT; ++i) oacc[i] *= alpha;
        }
        const float neg_m = -m_run;
        // scores of the next block (MFMA) under the exponentials of this one (VALU)
        if (!LAST) scores((it + 1) & 1, sn);
        float lsum = 0.f;
        bf16x8 pb[BKV / 16];
#pragma unroll
        for (int j = 0; j < BKV / 16; ++j) {
#pragma unroll
            for (int p = 0; p < 8; ++p)
                pb[j][p] = f2bf(__builtin_amdgcn_exp2f(fmaf(sc[j >> 1][8 * (j & 1) + p], scale_log2, neg_m)));
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[j], pb[j], 0, 1), ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[j], pb[j], 2, 3), ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[j], pb[j], 4, 5), ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[j], pb[j], 6, 7), ones, lsum, false);
        }
        l_run += lsum;
        pv(it & 1, pb);
        if (!LAST) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): K of block it+2, V of block it+1 have landed
            __syncthreads();
        }
    };
    // two blocks per trip, so that the score registers alternate without copies
    int it = 0;
    for (; it + 2 < nit; it += 2) {
        block(it, sa, sb, false);
        block(it + 1, sb, sa, false);
    }
    if (it + 1 < nit) {
        block(it, sa, sb, false);
        block(it + 1, sb, sa, true);
    } else {
        block(it, sa, sb, true);
    }

    if constexpr (KG > 1) {
        float* mo = (float*)smem;
        float* mm = mo + 4 * NT * 16 * 64;
        float* ml = mm + 256;
        __syncthreads();
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) mo[((qw * NT + i) * 16 + r) * 64 + lane] = oacc[i][r];
            mm[qw * 64 + lane] = m_run;
            ml[qw * 64 + lane] = l_run;
        }
        __syncthreads();
        if (grp == 0) {
            const float m1 = mm[qw * 64 + lane], l1 = ml[qw * 64 + lane];
            const float m = fmaxf(m_run, m1);
            const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
            l_run = l_run * a0 + l1 * a1;
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    oacc[i][r] = oacc[i][r] * a0 + mo[((qw * NT + i) * 16 + r) * 64 + lane] * a1;
        }
        __syncthreads();
    } else {
        __syncthreads();
    }

    if (grp == 0) {
        const float l_tot = half_sum(l_run);
        const float inv = 1.f / l_tot;
        bf16* sO = smem + qw * 32 * OROW;
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dim = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                sO[col * OROW + dim] = f2bf(oacc[i][r] * inv);
            }
    }
    __syncthreads();
    if (grp == 0) {
        const bf16* sO = smem + qw * 32 * OROW;
        const long long ldo = (long long)hl * D;
#pragma unroll
        for (int i = 0; i < 32 * KC / 64; ++i) {
            const int idx = lane + 64 * i;
            const int qr = idx / KC, dc = idx % KC;
            const int q = q0 + qr;
            if (q < S)
                *(bf16x8*)(O + ((long long)b * S + q) * ldo + head * D + dc * 8) = *(const bf16x8*)(sO + qr * OROW + dc * 8);
        }
    }
}

int g_attn_groups = 0;   // 0: by grid size; 1 or 2: forced
int g_attn_kernel = 0;   // 0 or 2: pipelined; 1: one LDS stage per key group, two barriers per key block

template <int D, int KG>
void launch_attn(dim3 grid, hipStream_t st, const bf16* Q, const bf16* K, const bf16* V, bf16* O, int B, int hl,
                 int kvl, int S, int ld_seq, float scale_log2) {
    if (g_attn_kernel == 1)
        hipLaunchKernelGGL((attn_prefill_kernel<D, KG>), grid, dim3(256 * KG), 0, st, Q, K, V, O, hl, kvl, S, ld_seq,
                           scale_log2, B);
    else
        hipLaunchKernelGGL((attn_prefill_pipe<D, KG>), grid, dim3(256 * KG), 0, st, Q, K, V, O, hl, kvl, S, ld_seq,
                           scale_log2, B);
}

}  // namespace

void set_attn_groups(int kg) { g_attn_groups = kg; }
void set_attn_kernel(int k) { g_attn_kernel = k; }

void attn_prefill_bf16(const bf16* Q, const bf16* K, const bf16* V, bf16* O, int B, int hl, int kvl, int S,
                       int ld_seq, int d, hipStream_t st) {
    if (B <= 0 || S <= 0) return;
    dim3 grid((S + BQ - 1) / BQ * hl * B);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    // Two key groups while the grid alone leaves a SIMD with at most one wave
    // (two 4-wave work-groups fit a CU): up to 512 work-groups.
    const long long wgs = grid.x;
    const int kg = g_attn_groups ? g_attn_groups : (wgs <= 512 ? 2 : 1);
    if (d == 128) {
        if (kg == 2) launch_attn<128, 2>(grid, st, Q, K, V, O, B, hl, kvl, S, ld_seq, scale_log2);
        else launch_attn<128, 1>(grid, st, Q, K, V, O, B, hl, kvl, S, ld_seq, scale_log2);
    } else {
        if (kg == 2) launch_attn<64, 2>(grid, st, Q, K, V, O, B, hl, kvl, S, ld_seq, scale_log2);
        else launch_attn<64, 1>(grid, st, Q, K, V, O, B, hl, kvl, S, ld_seq, scale_log2);
    }
}

}  // namespace tp
