// Drives the whole C ABI of the host runtime against the host test doubles
// (hip_doubles.cpp) under AddressSanitizer and UBSan: argument and state
// errors, every forward path's launches (each range-checked against the
// allocations it may touch), and an injected failure of every device
// allocation the weight loader, the workspace and the caches make, with a
// retry after each.  Exit status 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/tp_shard.h"

extern int g_fail_malloc_at;
extern long long g_launches;
size_t live_device_allocations();
void dump_device_allocations();

static int g_checks = 0, g_failed = 0;

#define EXPECT(cond)                                                            \
    do {                                                                        \
        ++g_checks;                                                             \
        if (!(cond)) {                                                          \
            ++g_failed;                                                         \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
        }                                                                       \
    } while (0)
#define EXPECT_RC(call, want)                                                   \
    do {                                                                        \
        const int rc_ = (call);                                                 \
        ++g_checks;                                                             \
        if (rc_ != (want)) {                                                    \
            ++g_failed;                                                         \
            std::fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, rc_, (want)); \
        }                                                                       \
    } while (0)

namespace {

struct Dev {   // a "device" allocation made through the doubles
    void* p = nullptr;
    explicit Dev(size_t n) {
        if (hipMalloc(&p, n) != hipSuccess) std::abort();
        std::memset(p, 0, n);
    }
    ~Dev() { (void)hipFree(p); }
    Dev(const Dev&) = delete;
    Dev& operator=(const Dev&) = delete;
    template <class T>
    T* as() const { return (T*)p; }
};

struct Shape {
    int hidden, heads, kv_heads, ffn, t, rank;
    int d() const { return hidden / heads; }
};

struct Weights {
    std::vector<Dev*> bufs;
    tp_weights w{};
    Weights(const Shape& s, int esz) {
        const size_t h = s.hidden, d = s.d();
        auto mk = [&](size_t n) {
            bufs.push_back(new Dev(n * esz));
            return bufs.back()->p;
        };
        w.wq = mk(s.heads * d * h);
        w.wk = mk(s.kv_heads * d * h);
        w.wv = mk(s.kv_heads * d * h);
        w.wo = mk(h * s.heads * d);
        w.w_gate = mk((size_t)s.ffn * h);
        w.w_up = mk((size_t)s.ffn * h);
        w.w_down = mk(h * s.ffn);
        w.g1 = mk(h);
        w.g2 = mk(h);
    }
    ~Weights() {
        for (Dev* b : bufs) delete b;
    }
};

tp_opts opts(int dtype, int act, int fp8) {
    tp_opts o{};
    o.dtype = dtype;
    o.act = act;
    o.rmsnorm = 1;
    o.eps = 1e-5f;
    o.rope = 1;
    o.rope_theta = 10000.f;
    o.decode_fp8 = fp8;
    return o;
}

void create_errors() {
    tp_shard* s = nullptr;
    tp_opts o = opts(TP_BF16, TP_ACT_SWIGLU, 0);
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 3, 0, &o, &s), TP_E_DIVIDE);    // heads % t
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 16, 0, &o, &s), TP_E_DIVIDE);   // t > heads
    EXPECT_RC(tp_shard_create(512, 8, 2, 1024, 4, 0, &o, &s), TP_E_DIVIDE);    // kv_heads % t
    EXPECT_RC(tp_shard_create(512, 8, 8, 1002, 4, 0, &o, &s), TP_E_DIVIDE);    // ffn % t
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 2, 2, &o, &s), TP_E_RANK);
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 2, -1, &o, &s), TP_E_RANK);
    EXPECT_RC(tp_shard_create(512, 16, 16, 1024, 2, 0, &o, &s), TP_E_ARG);     // head dim 32
    EXPECT_RC(tp_shard_create(512, 8, 3, 1024, 1, 0, &o, &s), TP_E_ARG);       // heads % kv_heads
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024 + 64, 2, 0, &o, &s), TP_E_ARG);  // (ffn / t) % 64
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 2, 0, &o, nullptr), TP_E_ARG);
    EXPECT_RC(tp_shard_create(0, 8, 8, 1024, 2, 0, &o, &s), TP_E_ARG);
    tp_opts bad = opts(TP_F32, TP_ACT_SWIGLU, 1);
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 2, 0, &bad, &s), TP_E_ARG);     // E4M3 on fp32
    bad = opts(7, TP_ACT_SWIGLU, 0);
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 2, 0, &bad, &s), TP_E_ARG);
    bad = opts(TP_BF16, 5, 0);
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 2, 0, &bad, &s), TP_E_ARG);
    bad = opts(TP_BF16, TP_ACT_SWIGLU, 0);
    bad.rope_theta = -1.f;
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 2, 0, &bad, &s), TP_E_ARG);
    EXPECT(s == nullptr);
    EXPECT_RC(tp_shard_create(512, 8, 8, 1024, 2, 1, nullptr, &s), TP_OK);     // default options
    tp_shard_destroy(s);
    EXPECT(std::strlen(tp_status_string(TP_E_SCRATCH)) > 0 && std::strlen(tp_status_string(12345)) > 0);
}

// The order checks that need no weights, then the whole flow of one shard.
void flow(const Shape& sh, int dtype, int act, int fp8) {
    const int esz = dtype == TP_BF16 ? 2 : 4;
    tp_opts o = opts(dtype, act, fp8);
    tp_shard* s = nullptr;
    EXPECT_RC(tp_shard_create(sh.hidden, sh.heads, sh.kv_heads, sh.ffn, sh.t, sh.rank, &o, &s), TP_OK);
    if (!s) return;
    const int B = 2, S = 40, cap = 96, h = sh.hidden;
    Dev x((size_t)B * S * h * esz), part((size_t)B * S * h * 4), part2((size_t)B * S * h * 4);
    Dev out((size_t)B * S * h * esz), nout((size_t)B * S * h * esz);
    const float* parts[2] = {part.as<float>(), part2.as<float>()};
    void* dbg = nullptr;
    // before the weights
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_ATTN, x.p, B, S, nullptr, part.as<float>(), nullptr), TP_E_STATE);
    EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_MLP, x.p, B, nullptr, part.as<float>(), nullptr), TP_E_STATE);
    EXPECT_RC(tp_shard_reduce_norm(s, 2, parts, 2, x.p, out.p, nout.p, B * S, nullptr), TP_E_STATE);
    EXPECT_RC(tp_shard_norm(s, 1, x.p, B * S, out.p, nullptr), TP_E_STATE);
    EXPECT_RC(tp_shard_fp8_view(s, 0, nullptr, nullptr, nullptr, nullptr), TP_E_STATE);
    EXPECT_RC(tp_shard_debug_view(s, 0, &dbg), TP_E_ARG);
    {
        Weights W(sh, esz);
        tp_weights missing = W.w;
        missing.wo = nullptr;
        EXPECT_RC(tp_shard_load_weights(s, &missing, nullptr), TP_E_ARG);
        EXPECT_RC(tp_shard_load_weights(s, &W.w, nullptr), TP_OK);
        EXPECT_RC(tp_shard_load_weights(s, &W.w, nullptr), TP_OK);   // replacing the weights
    }   // the caller's weights are gone: the shard keeps its own copies
    // a decode MLP stage before any ATTN stage
    EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_MLP, x.p, B, nullptr, part.as<float>(), nullptr), TP_E_STATE);
    tp_kv* kv = nullptr;
    EXPECT_RC(tp_kv_create(s, B, cap, &kv), TP_OK);
    // argument errors
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_ATTN, x.as<char>() + 2, B, S, kv, part.as<float>(), nullptr),
              TP_E_ARG);   // misaligned
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_ATTN, x.p, B + 1, S, kv, part.as<float>(), nullptr), TP_E_ARG);
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_ATTN, x.p, B, cap + 1, kv, part.as<float>(), nullptr),
              TP_E_KV_FULL);
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_MLP, x.p, B, S, kv, part.as<float>(), nullptr), TP_E_ARG);
    EXPECT_RC(tp_shard_forward_prefill(s, 7, x.p, B, S, nullptr, part.as<float>(), nullptr), TP_E_ARG);
    EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_ATTN, x.p, B, nullptr, part.as<float>(), nullptr), TP_E_ARG);
    // prefill: both stages, with and without a cache, pre-normalised input
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_ATTN, x.p, B, S, kv, part.as<float>(), nullptr), TP_OK);
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_ATTN | TP_STAGE_PRENORM, x.p, B, S, nullptr, part.as<float>(),
                                       nullptr), TP_OK);
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_MLP, x.p, B, S, nullptr, part.as<float>(), nullptr), TP_OK);
    // prefill with the reduce folded in: the GEMM's sum epilogue (bf16), or
    // the workspace partial and a reduce (fp32 shards)
    {
        const float* others[2] = {part.as<float>(), part2.as<float>()};
        EXPECT_RC(tp_shard_forward_prefill_reduce(s, TP_STAGE_ATTN, x.p, B, S, kv, others, x.p, out.p, nullptr),
                  TP_OK);
        EXPECT_RC(tp_shard_forward_prefill_reduce(s, TP_STAGE_MLP | TP_STAGE_PRENORM, out.p, B, S, nullptr, others,
                                                  out.p, nout.p, nullptr), TP_OK);
        EXPECT_RC(tp_shard_forward_prefill_reduce(s, TP_STAGE_MLP, out.p, B, S, nullptr, others, nullptr, nout.p,
                                                  nullptr), TP_OK);
        const float* lost_other[2] = {sh.rank == 0 ? part.as<float>() : nullptr,
                                      sh.rank == 1 ? part.as<float>() : nullptr};
        EXPECT_RC(tp_shard_forward_prefill_reduce(s, TP_STAGE_MLP, out.p, B, S, nullptr, lost_other, out.p, nout.p,
                                                  nullptr), TP_E_ARG);   // the other rank's partial is missing
        EXPECT_RC(tp_shard_forward_prefill_reduce(s, TP_STAGE_MLP, out.p, B, S, nullptr, others, out.p,
                                                  out.as<char>() + 64, nullptr), TP_E_ARG);   // out overlaps x
        EXPECT_RC(tp_shard_forward_prefill_reduce(s, TP_STAGE_MLP, out.p, B, S, nullptr, nullptr, out.p, nout.p,
                                                  nullptr), TP_E_ARG);
        EXPECT_RC(tp_shard_forward_prefill_reduce(s, TP_STAGE_MLP, out.p, B, S, kv, others, out.p, nout.p, nullptr),
                  TP_E_ARG);   // no cache for the MLP stage
    }
    for (int w = 0; w < 3; ++w) EXPECT_RC(tp_shard_debug_view(s, w, &dbg), TP_OK);
    EXPECT_RC(tp_shard_debug_view(s, 3, &dbg), TP_E_ARG);
    int len = -1;
    EXPECT_RC(tp_kv_get_len(kv, &len), TP_OK);
    // the reduce and its fused norm
    EXPECT_RC(tp_partial_reduce(parts, 2, x.p, out.p, (long long)B * S * h, dtype, nullptr), TP_OK);
    EXPECT_RC(tp_partial_reduce(parts, 2, nullptr, out.p, 0, dtype, nullptr), TP_OK);
    const float* lost[2] = {part.as<float>(), nullptr};
    EXPECT_RC(tp_partial_reduce(lost, 2, x.p, out.p, (long long)B * S * h, dtype, nullptr), TP_E_ARG);
    EXPECT_RC(tp_partial_reduce(parts, 65, x.p, out.p, 16, dtype, nullptr), TP_E_ARG);
    EXPECT_RC(tp_shard_reduce_norm(s, 1, parts, 2, x.p, out.p, nout.p, B * S, nullptr), TP_OK);
    EXPECT_RC(tp_shard_reduce_norm(s, 2, parts, 2, nullptr, out.p, nout.p, B * S, nullptr), TP_OK);
    EXPECT_RC(tp_shard_reduce_norm(s, 3, parts, 2, x.p, out.p, nout.p, B * S, nullptr), TP_E_ARG);
    EXPECT_RC(tp_shard_reduce_norm(s, 1, lost, 2, x.p, out.p, nout.p, B * S, nullptr), TP_E_ARG);
    EXPECT_RC(tp_shard_reduce_norm(s, 1, parts, 2, x.p, out.as<char>() + 4, nout.p, B * S, nullptr), TP_E_ARG);
    // the sequence-parallel calls
    EXPECT_RC(tp_partial_reduce_scatter(parts, 2, 1, x.p, out.p, B * S, h, dtype, nullptr), TP_OK);
    EXPECT_RC(tp_partial_reduce_scatter(parts, 2, 2, x.p, out.p, B * S, h, dtype, nullptr), TP_E_RANK);
    EXPECT_RC(tp_partial_reduce_scatter(parts, 2, 0, x.p, out.p, B * S - 1, h, dtype, nullptr), TP_E_DIVIDE);
    const void* pieces[2] = {x.p, (const char*)x.p + (size_t)S * h * esz};
    EXPECT_RC(tp_all_gather(pieces, 2, S, h, dtype, out.p, nullptr), TP_OK);
    EXPECT_RC(tp_shard_norm(s, 2, x.p, B * S, out.p, nullptr), TP_OK);
    // decode: one token per sequence, both stages, then through the allocation-free entry point
    EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_ATTN, x.p, B, kv, part.as<float>(), nullptr), TP_OK);
    EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_MLP, x.p, B, nullptr, part.as<float>(), nullptr), TP_OK);
    EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_MLP, x.p, B, kv, part.as<float>(), nullptr), TP_E_ARG);
    const int want_noalloc = dtype == TP_BF16 ? TP_OK : TP_E_STATE;
    EXPECT_RC(tp_shard_forward_decode_noalloc(s, TP_STAGE_ATTN, x.p, B, kv, part.as<float>(), nullptr), want_noalloc);
    EXPECT_RC(tp_shard_forward_decode_noalloc(s, TP_STAGE_MLP | TP_STAGE_PRENORM, x.p, B, nullptr, part.as<float>(),
                                              nullptr), want_noalloc);
    // decode with the reduce folded in: the GEMV / split-K epilogue, or the
    // workspace partial and a reduce (GEMM path, fp32 shards)
    {
        const float* others[2] = {part.as<float>(), part2.as<float>()};
        EXPECT_RC(tp_shard_forward_decode_reduce(s, TP_STAGE_ATTN, x.p, B, kv, others, x.p, out.p, nullptr), TP_OK);
        EXPECT_RC(tp_shard_forward_decode_reduce(s, TP_STAGE_MLP, out.p, B, nullptr, others, out.p, nout.p, nullptr),
                  TP_OK);
        EXPECT_RC(tp_shard_forward_decode_reduce(s, TP_STAGE_MLP, out.p, B, nullptr, others, nullptr, nout.p,
                                                 nullptr), TP_OK);
        const float* lost_other[2] = {sh.rank == 0 ? part.as<float>() : nullptr,
                                      sh.rank == 1 ? part.as<float>() : nullptr};
        EXPECT_RC(tp_shard_forward_decode_reduce(s, TP_STAGE_MLP, out.p, B, nullptr, lost_other, out.p, nout.p,
                                                 nullptr), TP_E_ARG);   // the other rank's partial is missing
        EXPECT_RC(tp_shard_forward_decode_reduce(s, TP_STAGE_MLP, out.p, B, nullptr, others, out.p,
                                                 out.as<char>() + 64, nullptr), TP_E_ARG);   // out overlaps x
        EXPECT_RC(tp_shard_forward_decode_reduce(s, TP_STAGE_MLP, out.p, B, nullptr, nullptr, out.p, nout.p,
                                                 nullptr), TP_E_ARG);
    }
    // the cache length in stream order
    EXPECT_RC(tp_kv_set_len_async(kv, cap + 1, nullptr), TP_E_ARG);
    EXPECT_RC(tp_kv_set_len_async(nullptr, 1, nullptr), TP_E_ARG);
    EXPECT_RC(tp_kv_set_len_async(kv, 3, nullptr), TP_OK);
    {
        int l3 = -1;
        EXPECT_RC(tp_kv_get_len_stream(kv, &l3, nullptr), TP_OK);
        EXPECT_RC(l3 == 3 ? TP_OK : TP_E_ARG, TP_OK);
        EXPECT_RC(tp_kv_get_len_stream(kv, nullptr, nullptr), TP_E_ARG);
    }
    // the cache fills up: an eager call on a full cache is refused up front
    EXPECT_RC(tp_kv_set_len(kv, cap + 1), TP_E_ARG);
    EXPECT_RC(tp_kv_set_len(kv, cap), TP_OK);
    EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_ATTN, x.p, B, kv, part.as<float>(), nullptr), TP_E_KV_FULL);
    EXPECT_RC(tp_kv_set_len(kv, cap - 1), TP_OK);
    EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_ATTN, x.p, B, kv, part.as<float>(), nullptr), TP_OK);
    // batch 1 (the GEMV kernels, or E4M3 ones) and a batch beyond the split-K path
    {
        tp_kv* kv1 = nullptr;
        EXPECT_RC(tp_kv_create(s, 1, cap, &kv1), TP_OK);
        EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_ATTN, x.p, 1, 5, kv1, part.as<float>(), nullptr), TP_OK);
        EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_ATTN, x.p, 1, kv1, part.as<float>(), nullptr), TP_OK);
        EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_MLP, x.p, 1, nullptr, part.as<float>(), nullptr), TP_OK);
        EXPECT_RC(tp_shard_forward_decode_noalloc(s, TP_STAGE_ATTN, x.p, 1, kv1, part.as<float>(), nullptr),
                  want_noalloc);
        tp_kv_destroy(kv1);
        const int BB = 70;
        Dev xb((size_t)BB * h * esz), pb((size_t)BB * h * 4);
        tp_kv* kvb = nullptr;
        EXPECT_RC(tp_kv_create(s, BB, 8, &kvb), TP_OK);
        EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_ATTN, xb.p, BB, kvb, pb.as<float>(), nullptr), TP_OK);
        EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_MLP, xb.p, BB, nullptr, pb.as<float>(), nullptr), TP_OK);
        Dev pb2((size_t)BB * h * 4), hb((size_t)BB * h * esz);
        const float* others[2] = {pb.as<float>(), pb2.as<float>()};
        EXPECT_RC(tp_shard_forward_decode_reduce(s, TP_STAGE_MLP, xb.p, BB, nullptr, others, xb.p, hb.p, nullptr),
                  TP_OK);
        {
            // batch 1 through the GEMV epilogue (the E4M3 one on an fp8 shard)
            Dev x1((size_t)h * esz), p1((size_t)h * 4), p2((size_t)h * 4), h1((size_t)h * esz);
            const float* o1[2] = {p1.as<float>(), p2.as<float>()};
            EXPECT_RC(tp_shard_forward_decode_reduce(s, TP_STAGE_MLP, x1.p, 1, nullptr, o1, x1.p, h1.p, nullptr),
                      TP_OK);
        }
        tp_kv_destroy(kvb);
    }
    if (fp8) {
        void* codes = nullptr;
        float* scales = nullptr;
        int r = 0, c = 0;
        for (int i = 0; i < 4; ++i) {
            EXPECT_RC(tp_shard_fp8_view(s, i, &codes, &scales, &r, &c), TP_OK);
            EXPECT(codes && scales && r > 0 && c > 0);
        }
        EXPECT_RC(tp_shard_fp8_view(s, 4, &codes, &scales, &r, &c), TP_E_ARG);
    }
    // paged cache (bf16)
    if (dtype == TP_BF16) {
        tp_kv* pk = nullptr;
        EXPECT_RC(tp_kv_create_paged(s, B, cap, 24, 16, &pk), TP_E_ARG);   // block size not a power of two
        EXPECT_RC(tp_kv_create_paged(s, B, cap, 16, 16, &pk), TP_OK);
        std::vector<int> table((size_t)B * (cap / 16));
        for (size_t i = 0; i < table.size(); ++i) table[i] = (int)((i * 5) % 16);
        table[3] = 16;
        EXPECT_RC(tp_kv_set_block_table(pk, table.data()), TP_E_ARG);   // id out of range
        table[3] = 15;
        EXPECT_RC(tp_kv_set_block_table(pk, table.data()), TP_OK);
        EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_ATTN, x.p, B, S, pk, part.as<float>(), nullptr), TP_OK);
        EXPECT_RC(tp_shard_forward_decode(s, TP_STAGE_ATTN, x.p, B, pk, part.as<float>(), nullptr), TP_OK);
        EXPECT_RC(tp_shard_forward_decode_noalloc(s, TP_STAGE_ATTN, x.p, B, pk, part.as<float>(), nullptr), TP_OK);
        EXPECT_RC(tp_kv_set_block_table(kv, table.data()), TP_E_STATE);   // a contiguous cache has no table
        tp_kv_destroy(pk);
    } else {
        tp_kv* pk = nullptr;
        EXPECT_RC(tp_kv_create_paged(s, B, cap, 16, 16, &pk), TP_E_ARG);
        EXPECT_RC(tp_kv_create(s, 1, 16001, &pk), TP_E_ARG);
    }
    // the kernel timer
    EXPECT_RC(tp_shard_timing(s, TP_K_MASK(TP_K_GEMM_UP) | TP_K_MASK(TP_K_GEMV_UP)), TP_OK);
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_MLP, x.p, B, S, nullptr, part.as<float>(), nullptr), TP_OK);
    double ms = -1;
    long long n = -1;
    EXPECT_RC(tp_shard_timing_read(s, TP_K_GEMM_UP, &ms, &n), TP_OK);
    EXPECT(n == 1);
    EXPECT_RC(tp_shard_timing_read(s, TP_K_COUNT, &ms, &n), TP_E_ARG);
    EXPECT_RC(tp_shard_timing(s, 0), TP_OK);
    // a reserved workspace, then the largest call it covers
    EXPECT_RC(tp_shard_reserve(s, 2 * B * S), TP_OK);
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_MLP, x.p, 2, B * S / 2, nullptr, part.as<float>(), nullptr),
              TP_OK);
    tp_kv_destroy(kv);
    tp_shard_destroy(s);
}

// A failed workspace allocation fails the call and a repeat succeeds; a cache
// whose k-th allocation fails is not created and frees what it had.
void workspace_failures(const Shape& sh, const tp_opts& o, const Weights& W, int esz) {
    tp_shard* s = nullptr;
    EXPECT_RC(tp_shard_create(sh.hidden, sh.heads, sh.kv_heads, sh.ffn, sh.t, sh.rank, &o, &s), TP_OK);
    EXPECT_RC(tp_shard_load_weights(s, &W.w, nullptr), TP_OK);
    const int B = 2, S = 16;
    Dev x((size_t)B * S * sh.hidden * esz), part((size_t)B * S * sh.hidden * 4);
    g_fail_malloc_at = 0;
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_MLP, x.p, B, S, nullptr, part.as<float>(), nullptr), TP_E_NOMEM);
    g_fail_malloc_at = -1;
    EXPECT_RC(tp_shard_forward_prefill(s, TP_STAGE_MLP, x.p, B, S, nullptr, part.as<float>(), nullptr), TP_OK);
    for (int k = 0; k < 3; ++k) {
        tp_kv* kv = nullptr;
        g_fail_malloc_at = k;
        EXPECT_RC(tp_kv_create(s, B, 32, &kv), TP_E_NOMEM);
        EXPECT(kv == nullptr);
        g_fail_malloc_at = -1;
    }
    if (o.dtype == TP_BF16)
        for (int k = 0; k < 4; ++k) {
            tp_kv* kv = nullptr;
            g_fail_malloc_at = k;
            EXPECT_RC(tp_kv_create_paged(s, B, 32, 16, 8, &kv), TP_E_NOMEM);
            EXPECT(kv == nullptr);
            g_fail_malloc_at = -1;
        }
    tp_shard_destroy(s);
}

// Fail the k-th device allocation of a call for every k it makes: the call
// reports TP_E_NOMEM, leaks nothing, and the same call then succeeds.
void injected_failures(const Shape& sh, int dtype, int act, int fp8) {
    const int esz = dtype == TP_BF16 ? 2 : 4;
    tp_opts o = opts(dtype, act, fp8);
    Weights W(sh, esz);
    const size_t base = live_device_allocations();
    int failures = 0;
    for (int k = 0; k < 64; ++k) {
        tp_shard* s = nullptr;
        if (tp_shard_create(sh.hidden, sh.heads, sh.kv_heads, sh.ffn, sh.t, sh.rank, &o, &s) != TP_OK) break;
        g_fail_malloc_at = k;
        const int rc = tp_shard_load_weights(s, &W.w, nullptr);
        const bool injected = g_fail_malloc_at == -1 && rc != TP_OK;
        g_fail_malloc_at = -1;
        if (rc == TP_OK) {
            tp_shard_destroy(s);
            break;
        }
        ++failures;
        EXPECT(injected);
        EXPECT(rc == TP_E_NOMEM);
        EXPECT_RC(tp_shard_load_weights(s, &W.w, nullptr), TP_OK);   // the retry starts clean
        if (fp8)
            for (int i = 0; i < 4; ++i) {
                void* codes = nullptr;
                float* scales = nullptr;
                EXPECT_RC(tp_shard_fp8_view(s, i, &codes, &scales, nullptr, nullptr), TP_OK);
                EXPECT(codes != nullptr && scales != nullptr);
            }
        tp_shard_destroy(s);
        EXPECT(live_device_allocations() == base);
    }
    EXPECT(failures == 6 + o.rope + 8 * fp8);   // six packed weights, the rotary turns, four E4M3 pairs
    // the workspace and the caches
    workspace_failures(sh, o, W, esz);
    EXPECT(live_device_allocations() == base);
    if (live_device_allocations() != base) dump_device_allocations();
}

}  // namespace

int main() {
    const size_t base = live_device_allocations();
    create_errors();
    const Shape gqa{256, 4, 2, 512, 2, 1};     // head dim 64, grouped KV heads
    const Shape mha{512, 4, 4, 1024, 2, 0};    // head dim 128
    flow(gqa, TP_BF16, TP_ACT_SWIGLU, 0);
    flow(mha, TP_BF16, TP_ACT_GELU, 0);
    flow(gqa, TP_BF16, TP_ACT_SWIGLU, 1);
    flow(gqa, TP_F32, TP_ACT_SWIGLU, 0);
    flow(mha, TP_F32, TP_ACT_GELU, 0);
    injected_failures(gqa, TP_BF16, TP_ACT_SWIGLU, 1);
    injected_failures(mha, TP_F32, TP_ACT_GELU, 0);
    EXPECT(live_device_allocations() == base);
    std::printf("host sanitizer driver: %d checks, %d failed, %lld range-checked launches\n", g_checks, g_failed,
                g_launches);
    return g_failed ? 1 : 0;
}
