// Host test doubles for the host runtime (tp_shard.cpp) built without a GPU
// under AddressSanitizer: the HIP runtime calls it makes, on host memory,
// and the kernel launchers it calls, which launch nothing but check that
// every range the kernel would read or write lies inside one allocation.
// Test infrastructure only; the library never links this file.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iterator>
#include <map>

#include "../../include/tp_shard.h"
#include "../../tensor_transformer_layer_tp_amd/csrc/kernels.h"

namespace {

std::map<const char*, size_t>& allocs() {   // hipMalloc'ed blocks
    static std::map<const char*, size_t> m;
    return m;
}

std::map<const char*, size_t>& symbols() {  // static device arrays looked up by address
    static std::map<const char*, size_t> m;
    return m;
}

bool inside(const std::map<const char*, size_t>& m, const char* c, long long bytes) {
    auto it = m.upper_bound(c);
    if (it == m.begin()) return false;
    --it;
    return c >= it->first && c + bytes <= it->first + it->second;
}

[[noreturn]] void fail(const char* what, const void* p, size_t bytes) {
    std::fprintf(stderr, "range check failed: %s: %zu bytes at %p lie in no allocation\n", what, bytes, p);
    std::abort();
}

// [p, p + bytes) must lie inside one allocation
void in_alloc(const void* p, long long bytes, const char* what) {
    if (bytes <= 0) return;
    const char* c = (const char*)p;
    if (!inside(allocs(), c, bytes) && !inside(symbols(), c, bytes)) fail(what, p, (size_t)bytes);
}

}  // namespace

int g_fail_malloc_at = -1;   // the n-th hipMalloc from now fails (-1: none)
long long g_launches = 0;    // kernel launches the doubles saw

// live hipMalloc'ed blocks
size_t live_device_allocations() { return allocs().size(); }

void dump_device_allocations() {
    for (const auto& a : allocs()) std::fprintf(stderr, "  live block %p: %zu bytes\n", (const void*)a.first, a.second);
}

extern "C" {

hipError_t hipMalloc(void** p, size_t n) {
    if (g_fail_malloc_at == 0) {
        g_fail_malloc_at = -1;
        *p = nullptr;
        return hipErrorOutOfMemory;
    }
    if (g_fail_malloc_at > 0) --g_fail_malloc_at;
    *p = std::malloc(n ? n : 1);
    if (!*p) return hipErrorOutOfMemory;
    allocs()[(const char*)*p] = n;
    return hipSuccess;
}

hipError_t hipFree(void* p) {
    if (!p) return hipSuccess;
    auto& m = allocs();
    auto it = m.find((const char*)p);
    if (it == m.end()) fail("hipFree of an unknown pointer", p, 0);
    m.erase(it);
    std::free(p);
    return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind kind) {
    if (kind == hipMemcpyHostToDevice || kind == hipMemcpyDeviceToDevice) in_alloc(dst, (long long)n, "copy destination");
    if (kind == hipMemcpyDeviceToHost || kind == hipMemcpyDeviceToDevice) in_alloc(src, (long long)n, "copy source");
    if (n) std::memcpy(dst, src, n);   // host sides are plain memory that the sanitizer watches
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t) {
    return hipMemcpy(dst, src, n, kind);
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                            hipMemcpyKind, hipStream_t) {
    if (!height || !width) return hipSuccess;
    in_alloc(dst, (long long)((height - 1) * dpitch + width), "hipMemcpy2DAsync destination");
    in_alloc(src, (long long)((height - 1) * spitch + width), "hipMemcpy2DAsync source");
    for (size_t r = 0; r < height; ++r) std::memcpy((char*)dst + r * dpitch, (const char*)src + r * spitch, width);
    return hipSuccess;
}

hipError_t hipMemset(void* p, int v, size_t n) {
    in_alloc(p, (long long)n, "hipMemset");
    std::memset(p, v, n);
    return hipSuccess;
}

hipError_t hipDeviceSynchronize() { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipGetLastError() { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "host double"; }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s) {
    *s = hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
    *e = (hipEvent_t)std::malloc(8);
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
    std::free((void*)e);
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
    *ms = 0.f;
    return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void* symbol) {
    *p = (void*)symbol;
    symbols()[(const char*)symbol] = TP_NOALLOC_SCRATCH_BYTES;   // the static array is device memory too
    return hipSuccess;
}

}  // extern "C"

namespace tp {
namespace {

// what an epilogue writes for rows x n columns of output
void epilogue_ranges(const Epilogue& e, long long rows, int n, size_t esz) {
    const long long col_end = (long long)e.col0 + n;
    switch (e.mode) {
        case EPI_F32:
            in_alloc(e.out, ((rows - 1) * e.ldo + col_end) * 4, "fp32 partial");
            break;
        case EPI_SWIGLU:
            in_alloc(e.out, ((rows - 1) * e.ldo + col_end / 2) * (long long)esz, "SwiGLU output");
            break;
        case EPI_GELU:
        case EPI_STORE:
            in_alloc(e.out, ((rows - 1) * e.ldo + col_end) * (long long)esz, "projection output");
            break;
        case EPI_SUM: {
            const long long n = (rows - 1) * e.ldo + col_end;
            if (e.sum.t < 1 || e.sum.t > kSumMaxRanks || e.sum.self < 0 || e.sum.self >= e.sum.t)
                fail("fused sum: rank count or slot", e.out, 0);
            in_alloc(e.out, n * 2, "reduced output");
            for (int j = 0; j < e.sum.t; ++j)
                if (j != e.sum.self) in_alloc(e.sum.p[j], n * 4, "other rank's partial");
            if (e.sum.residual) in_alloc(e.sum.residual, n * 2, "residual");
            break;
        }
        default: {
            const QKVDest& q = e.qkv;
            const long long B = rows / q.S;
            in_alloc(q.q, B * q.hl * q.S * q.d * (long long)esz, "q");
            if (q.table == nullptr) {
                const long long kv = B * q.kvl * (long long)q.ld_seq * q.d * (long long)esz;
                in_alloc(q.k, kv, "K cache");
                in_alloc(q.v, kv, "V cache");
                if (q.pos_dev == nullptr && q.pos0 + q.S > q.ld_seq) fail("K/V rows past the cache", q.k, 0);
            }
            if (q.pos_dev) in_alloc(q.pos_dev, 4, "cache length");
            if (q.rope_rev) in_alloc(q.rope_rev, q.d / 2 * 8, "rotation turns");
            if (q.rope_cos) in_alloc(q.rope_cos, (long long)q.d / 2 * 4, "rotation table");
        }
    }
    if (e.len.ptr) in_alloc(e.len.ptr, 4, "cache length");
    if (e.len.overflow) in_alloc(e.len.overflow, 4, "overflow flag");
    ++g_launches;
}

int splits(int N, int K) {
    const int groups = N / 64, kg = K / 64;
    const int want = (512 + groups - 1) / groups;
    return want < kg / 4 ? (want > 1 ? want : 1) : (kg / 4 > 1 ? kg / 4 : 1);
}

int g_chunk = 0;

}  // namespace

void gemm_bf16(const bf16* A, long long lda, const bf16* B, long long ldb, int M, int N, int K, const Epilogue& epi,
               hipStream_t) {
    in_alloc(A, ((long long)(M - 1) * lda + K) * 2, "GEMM A");
    in_alloc(B, ((long long)(N - 1) * ldb + K) * 2, "GEMM B");
    epilogue_ranges(epi, M, N, 2);
}
void gemm_f32(const float* A, long long lda, const float* B, long long ldb, int M, int N, int K, const Epilogue& epi,
              hipStream_t) {
    in_alloc(A, ((long long)(M - 1) * lda + K) * 4, "GEMM A");
    in_alloc(B, ((long long)(N - 1) * ldb + K) * 4, "GEMM B");
    epilogue_ranges(epi, M, N, 4);
}
void set_kv_len(int* dlen, int len, hipStream_t) {
    in_alloc(dlen, 8, "cache length and overflow flag");
    dlen[0] = len;   // host memory here: the double performs the kernel's two stores
    dlen[1] = 0;
    ++g_launches;
}
void rmsnorm_bf16(const bf16* x, const bf16* g, bf16* out, int rows, int n, float, hipStream_t) {
    in_alloc(x, (long long)rows * n * 2, "norm input");
    in_alloc(g, (long long)n * 2, "norm gain");
    in_alloc(out, (long long)rows * n * 2, "norm output");
    ++g_launches;
}
void rmsnorm_f32(const float* x, const float* g, float* out, int rows, int n, float, hipStream_t) {
    in_alloc(x, (long long)rows * n * 4, "norm input");
    in_alloc(g, (long long)n * 4, "norm gain");
    in_alloc(out, (long long)rows * n * 4, "norm output");
    ++g_launches;
}
void attn_prefill_bf16(const bf16* Q, const bf16* K, const bf16* V, bf16* O, int B, int hl, int kvl, int S, int ld_seq,
                       int d, hipStream_t) {
    in_alloc(Q, (long long)B * hl * S * d * 2, "attention q");
    in_alloc(K, (long long)B * kvl * ld_seq * d * 2, "attention K");
    in_alloc(V, (long long)B * kvl * ld_seq * d * 2, "attention V");
    in_alloc(O, (long long)B * S * hl * d * 2, "attention o");
    ++g_launches;
}
void attn_f32(const float* Q, const float* K, const float* V, float* O, int B, int hl, int kvl, int Sq, int q_pos0,
              int ld_seq, int d, hipStream_t) {
    in_alloc(Q, (long long)B * hl * Sq * d * 4, "attention q");
    in_alloc(K, (long long)B * kvl * ld_seq * d * 4, "attention K");
    in_alloc(V, (long long)B * kvl * ld_seq * d * 4, "attention V");
    in_alloc(O, (long long)B * Sq * hl * d * 4, "attention o");
    if (q_pos0 + Sq > ld_seq) fail("attention past the cache", K, 0);
    ++g_launches;
}
void set_attn_groups(int) {}
void set_attn_kernel(int) {}
void gemv_bf16(const bf16* x, int B, const bf16* gamma, float, const bf16* W, int N, int K, const Epilogue& epi,
               hipStream_t) {
    in_alloc(x, (long long)B * K * 2, "GEMV input");
    if (gamma) in_alloc(gamma, (long long)K * 2, "GEMV gain");
    in_alloc(W, (long long)N * K * 2, "GEMV weights");
    epilogue_ranges(epi, B, N, 2);
}
void gemv_fp8(const bf16* x, const bf16* gamma, float, const uint8_t* W, const float* scale, int N, int K,
              const Epilogue& epi, hipStream_t) {
    in_alloc(x, (long long)K * 2, "GEMV input");
    if (gamma) in_alloc(gamma, (long long)K * 2, "GEMV gain");
    in_alloc(W, (long long)N * K, "E4M3 weights");
    in_alloc(scale, (long long)N * 4, "E4M3 scales");
    epilogue_ranges(epi, 1, N, 2);
}
void quant_rows_e4m3(const bf16* W, int N, int K, uint8_t* Q, float* scale, hipStream_t) {
    in_alloc(W, (long long)N * K * 2, "quantised weights");
    in_alloc(Q, (long long)N * K, "E4M3 codes");
    in_alloc(scale, (long long)N * 4, "E4M3 scales");
    ++g_launches;
}
size_t attn_decode_scratch_bytes(int B, int hl, int, int cap, int d) {
    return (size_t)B * hl * ((cap + 15) / 16 + 8) * (d + 2) * 4;
}
void attn_decode_bf16(const bf16* q, const bf16* K, const bf16* V, bf16* O, float* scratch, int* counters, int B,
                      int hl, int kvl, const int* len_dev, int ld_seq, int d, const int* table, int, int,
                      hipStream_t) {
    in_alloc(q, (long long)B * hl * d * 2, "decode q");
    if (!table) {
        in_alloc(K, (long long)B * kvl * ld_seq * d * 2, "decode K");
        in_alloc(V, (long long)B * kvl * ld_seq * d * 2, "decode V");
    }
    in_alloc(O, (long long)B * hl * d * 2, "decode o");
    in_alloc(scratch, (long long)attn_decode_scratch_bytes(B, hl, kvl, ld_seq, d), "decode attention records");
    in_alloc(counters, (long long)kDecodeCounters * 4, "merge counters");
    in_alloc(len_dev, 4, "cache length");
    ++g_launches;
}
void kv_to_pages(const bf16* k, const bf16* v, bf16* kpool, bf16* vpool, int B, int kvl, int S, int d, const int* table,
                 int, int max_blocks, hipStream_t) {
    in_alloc(k, (long long)B * kvl * S * d * 2, "contiguous K");
    in_alloc(v, (long long)B * kvl * S * d * 2, "contiguous V");
    in_alloc(table, (long long)B * max_blocks * 4, "block table");
    in_alloc(kpool, 2, "K pool");
    in_alloc(vpool, 2, "V pool");
    ++g_launches;
}
void set_decode_chunk(int ch) { g_chunk = ch; }
void set_decode_attn_mode(int) {}
size_t skinny_scratch_bytes(int B, int N, int K) { return (size_t)splits(N, K) * B * N * 4; }
void skinny_bf16(const bf16* x, int B, const bf16* W, int N, int K, float* part, const Epilogue& epi, hipStream_t) {
    in_alloc(x, (long long)B * K * 2, "split-K input");
    in_alloc(W, (long long)N * K * 2, "split-K weights");
    in_alloc(part, (long long)skinny_scratch_bytes(B, N, K), "split-K partials");
    epilogue_ranges(epi, B, N, 2);
}
void partial_reduce(const float* const* parts, int t, const void* residual, void* out, long long n, int bf16_out,
                    hipStream_t) {
    for (int r = 0; r < t; ++r) in_alloc(parts[r], n * 4, "partial");
    if (residual) in_alloc(residual, n * (bf16_out ? 2 : 4), "residual");
    in_alloc(out, n * (bf16_out ? 2 : 4), "reduce output");
    ++g_launches;
}
bool reduce_norm_bf16(const float* const* parts, int t, const bf16* residual, bf16* out, const bf16* g, bf16* nout,
                      int rows, int n, float, hipStream_t) {
    if (n % 4 || n > 8192) return false;
    const long long e = (long long)rows * n;
    for (int r = 0; r < t; ++r) in_alloc(parts[r], e * 4, "partial");
    if (residual) in_alloc(residual, e * 2, "residual");
    in_alloc(out, e * 2, "reduce output");
    in_alloc(g, (long long)n * 2, "norm gain");
    in_alloc(nout, e * 2, "norm output");
    ++g_launches;
    return true;
}
void rope_table(float* c, float* s, double* rev, int npos, int d, float, hipStream_t) {
    in_alloc(c, (long long)npos * d / 2 * 4, "cos table");
    in_alloc(s, (long long)npos * d / 2 * 4, "sin table");
    in_alloc(rev, (long long)d / 2 * 8, "rotation turns");
    ++g_launches;
}
void rope_turns(double* rev, int d, float, hipStream_t) {
    in_alloc(rev, (long long)d / 2 * 8, "rotation turns");
    ++g_launches;
}
void zero_ints(int* p, int n, hipStream_t) {
    in_alloc(p, (long long)n * 4, "zeroed ints");
    std::memset(p, 0, (size_t)n * 4);
    ++g_launches;
}
void all_gather(const void* const* pieces, int t, long long piece_bytes, void* out, hipStream_t) {
    for (int r = 0; r < t; ++r) in_alloc(pieces[r], piece_bytes, "gathered piece");
    in_alloc(out, piece_bytes * t, "gather output");
    ++g_launches;
}
int g_cfg = -1, g_split[3] = {0, 0, 0};
void set_gemm_config(int cfg) { g_cfg = cfg; }
int gemm_config_count() { return 17; }
void set_gemm_split(int c0, int c1, int cols) {
    g_split[0] = c0;
    g_split[1] = c1;
    g_split[2] = cols;
}
void gemm_plan_info(int, int N, int, int, int* parts, int cfg[2], int ncols[2]) {
    *parts = 1;
    cfg[0] = 15;
    cfg[1] = -1;
    ncols[0] = N;
    ncols[1] = 0;
}

}  // namespace tp
