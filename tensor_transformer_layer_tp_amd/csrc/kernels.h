// Internal launch API of the shard kernels (not part of the C ABI): the
// epilogue and cache descriptors and the launchers.  Host-safe: the host
// runtime includes it alone; device helpers live in common.h.
#pragma once

#include "types.h"

namespace tp {

// What a projection does with its fp32 accumulator tile.
enum EpiMode {
    EPI_F32 = 0,     // out[m, n] = acc (fp32 partial sum of a row-parallel linear)
    EPI_QKV = 1,     // rotary embedding on q/k, scatter q to [B,Hl,S,d], k/v to the cache
    EPI_SWIGLU = 2,  // act[m, j] = SiLU(gate) * up, gate/up interleaved in 32-column blocks
    EPI_GELU = 3,    // act[m, n] = GELU_erf(acc)
    EPI_STORE = 4,   // out[m, n] = acc in the storage type
    EPI_SUM = 5,     // out[m, n] = bf16(sum of the t ranks' partials in rank order + residual), with acc as
                     // the partial of rank `self` (decode GEMV and split-K paths only)
};

// The all-reduce's sum folded into a row-parallel projection's epilogue: the
// other ranks' fp32 partials [rows, ldo] (p[self] is not read), an optional
// bf16 residual of the same layout.
constexpr int kSumMaxRanks = 8;
struct SumDest {
    const float* p[kSumMaxRanks];
    const bf16* residual;   // nullptr: none
    int t;                  // 1 <= t <= kSumMaxRanks
    int self;               // the rank whose partial is the accumulator
};

struct QKVDest {
    int S;              // tokens per sequence in this call (1 for decode)
    int pos0;           // position of token 0 (0 for prefill, L for decode)
    const int* pos_dev; // if set, token 0's position is read from device memory instead
                        // (the cache length); k/v stores at positions >= ld_seq are dropped
    int hl, kvl, d;     // local query heads, local kv heads, head dim
    void* q;            // [B, hl, S, d]
    void* k;            // [B, kvl, ld_seq, d], written at slots pos0 + s
    void* v;
    int ld_seq;         // cache capacity (positions)
    const float* rope_cos;  // [max_pos, d/2] or nullptr: the fp32 path's rotation tables
    const float* rope_sin;
    const double* rope_rev; // [d/2] turns per position (theta_i / 2 pi), or nullptr (no rotary
                            // embedding): the bf16 kernels form the rotation from it
    // paged cache: k/v are pools [blocks, kvl, bsz, d]; position p of sequence
    // b lives in block table[b * max_blocks + p / bsz] at row p % bsz
    const int* table;   // nullptr: contiguous [B, kvl, ld_seq, d]
    int bsz, max_blocks;
};

// Update of a device-resident cache length, done by one thread of the
// projection that follows the last reader of the length in a stage.
struct LenUpdate {
    int* ptr;           // nullptr: no update
    int value;          // >= 0: *ptr = value;  < 0: *ptr = min(*ptr + 1, cap)
    int cap;
    int* overflow;      // set to 1 when an advance finds the length at cap: that
                        // call's token was not appended (nullptr: not reported)
};

struct Epilogue {
    int mode;
    void* out;          // F32: float*, others: element-type pointer
    long long ldo;      // leading dimension of out, in elements
    QKVDest qkv;
    LenUpdate len;
    int col0;           // GEMM launches over a column range: its first column (multiple of 64)
    SumDest sum;        // EPI_SUM only
};

// ---- bf16 path (gfx950 MFMA) ----
void gemm_bf16(const bf16* A, long long lda, const bf16* B, long long ldb, int M, int N, int K,
               const Epilogue& epi, hipStream_t st);
void rmsnorm_bf16(const bf16* x, const bf16* g, bf16* out, int rows, int n, float eps, hipStream_t st);
void attn_prefill_bf16(const bf16* Q, const bf16* K, const bf16* V, bf16* O, int B, int hl, int kvl,
                       int S, int ld_seq, int d, hipStream_t st);
void set_attn_groups(int kg);   // prefill attention key groups: 0 automatic, 1 or 2 forced
void set_attn_kernel(int k);   // prefill attention kernel: 0 default, 1 two barriers per key block, 2 pipelined
// decode GEMV for B <= 4 sequences (K <= 16384, N a multiple of 64)
void gemv_bf16(const bf16* x, int B, const bf16* gamma, float eps, const bf16* W, int N, int K,
               const Epilogue& epi, hipStream_t st);
// one sequence, E4M3 weights [N, K] with one fp32 scale per row
void gemv_fp8(const bf16* x, const bf16* gamma, float eps, const uint8_t* W, const float* scale, int N, int K,
              const Epilogue& epi, hipStream_t st);
// per-row E4M3 quantisation: Q [N, K] codes, scale [N]
void quant_rows_e4m3(const bf16* W, int N, int K, uint8_t* Q, float* scale, hipStream_t st);
// decode attention over positions [0, *len_dev + 1) (capped at ld_seq); the
// grid and the scratch are sized for ld_seq positions so that one launch
// stays valid while the device length grows (graph replay)
// `counters` (kDecodeCounters ints) must be zero before the first call; each
// call leaves them zero again
constexpr int kDecodeCounters = 16384;
void attn_decode_bf16(const bf16* q, const bf16* K, const bf16* V, bf16* O, float* scratch, int* counters, int B,
                      int hl, int kvl, const int* len_dev, int ld_seq, int d, const int* table, int bsz,
                      int max_blocks, hipStream_t st);
// copy K and V [B, kvl, S, d] (contiguous) into a paged pool at positions 0..S-1
void kv_to_pages(const bf16* k, const bf16* v, bf16* kpool, bf16* vpool, int B, int kvl, int S, int d,
                 const int* table, int bsz, int max_blocks, hipStream_t st);
size_t attn_decode_scratch_bytes(int B, int hl, int kvl, int cap, int d);
void set_decode_chunk(int ch);   // decode attention positions per chunk: 0 automatic, 16/32/64 forced
void set_decode_attn_mode(int mode);   // 0 automatic, 1 split kernels + merge launch, 2 fused merge
// small decode batches (2..64; the shard runs 5..64 through it and up to 4
// through gemv_bf16): split-K MFMA projection + epilogue pass; part is fp32
// scratch of skinny_scratch_bytes(B, N, K); N and K multiples of 64
void skinny_bf16(const bf16* x, int B, const bf16* W, int N, int K, float* part, const Epilogue& epi,
                 hipStream_t st);
size_t skinny_scratch_bytes(int B, int N, int K);

// ---- fp32 path ----
void gemm_f32(const float* A, long long lda, const float* B, long long ldb, int M, int N, int K,
              const Epilogue& epi, hipStream_t st);
void rmsnorm_f32(const float* x, const float* g, float* out, int rows, int n, float eps, hipStream_t st);
void attn_f32(const float* Q, const float* K, const float* V, float* O, int B, int hl, int kvl, int Sq,
              int q_pos0, int ld_seq, int d, hipStream_t st);

// ---- shared ----
void partial_reduce(const float* const* parts, int t, const void* residual, void* out, long long n,
                    int bf16_out, hipStream_t st);
// partial_reduce of rows x n values (bf16 out) and rmsnorm_bf16 of the result
// in one pass, bit-equal to the two launches; false (nothing launched) when
// n is not a multiple of 4 or exceeds 8192
bool reduce_norm_bf16(const float* const* parts, int t, const bf16* residual, bf16* out, const bf16* g, bf16* nout,
                      int rows, int n, float eps, hipStream_t st);
// cos/sin of p * theta_i for p < npos, i < d/2 ([npos, d/2] fp32), and rev[i] =
// theta_i / (2 pi) in double (the rotation per position in turns)
void rope_table(float* cos_t, float* sin_t, double* rev, int npos, int d, float theta, hipStream_t st);
// p[0, n) = 0 (a fill kernel: callers may be under graph capture)
void zero_ints(int* p, int n, hipStream_t st);
// rev[i] = theta_i / (2 pi) alone (d <= 128): what the bf16 kernels rotate with
void rope_turns(double* rev, int d, float theta, hipStream_t st);
// out = rank-order concatenation of t pieces of piece_bytes each (multiple of 16, 16-byte aligned)
void all_gather(const void* const* pieces, int t, long long piece_bytes, void* out, hipStream_t st);

// tuning: -1 = heuristic, otherwise a fixed GEMM tile configuration index
void set_gemm_config(int cfg);
int gemm_config_count();
// tests: force every GEMM wider than cols0 columns to run as two launches
// (columns [0, cols0) with cfg0, the rest with cfg1); cols0 = 0 turns it off
void set_gemm_split(int cfg0, int cfg1, int cols0);
// the launch plan the planner picks for a shape (host only)
void gemm_plan_info(int M, int N, int K, int mode, int* parts, int cfg[2], int ncols[2]);

}  // namespace tp
