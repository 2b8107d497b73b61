// Host runtime and C ABI of one rank's tensor-parallel layer shard.
//
// Validation happens here, before any device call, so that every argument or
// state error returns without side effects.  The partition rules are the
// pages' (undercodenews post 110319 on tensor parallelism, section "the
// Original": the degree may not exceed the head count; heads and FFN width
// must divide by it), plus kv_heads % degree == 0 so that the KV heads --
// and with them the KV cache (byteledger "Tensor Parallelism: Splitting One
// Layer Across GPUs", "Interaction with the rest of serving") -- split too.
#include "../../include/tp_shard.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"

using namespace tp;

// Workspace of the allocation-free decode entry point: a static device array
// that the code object brings along on every device the library runs on.
// In host code its name is a host-side stand-in, never a device address:
// host code uses only the per-device address looked up once at set-up.
static __device__ __attribute__((aligned(256))) char scratch[TP_NOALLOC_SCRATCH_BYTES];

struct tp_shard {
    int hidden, heads, kv_heads, ffn, t, rank;
    tp_opts o;
    int d, hl, kvl, fl, nqkv, nup;
    size_t esz;
    int device;
    bool loaded;
    void *w_qkv, *w_o, *w_up, *w_down, *g1, *g2;
    // E4M3 copies of the four packed projections (decode_fp8) and their row scales
    uint8_t* q8[4];
    float* s8[4];
    char* ws;
    size_t ws_bytes;
    float *rcos, *rsin;
    double* rrev;     // [d/2] rotary turns per position
    int rope_npos;
    // base and offsets of the last call's workspace tensors (debug view)
    char* dbg_base;
    size_t off_n, off_o, off_act;
    // kernel timer: event pairs in launch order and the kind of each pair
    bool timing;
    unsigned tmask;   // kernel kinds being bracketed (bit k = TP_K_k)
    std::vector<hipEvent_t> ev;
    std::vector<int> evkind;
    size_t evused;
    bool attn_seen;   // an ATTN stage has run on this shard (decode MLP needs one first)
};

struct tp_kv {
    int batch, max_seq;
    int len;      // host copy of the cache length, advanced by every enqueued call
    int* dlen;    // device copy [length, overflow flag]: the kernels read and advance
                  // the length and raise the flag when a decode call finds it at max_seq
    int kvl, d;
    size_t esz;
    int dtype;
    void *k, *v;
    // paged layout: k/v are pools [num_blocks, kvl, block_size, d]; table [batch, max_blocks]
    int* table;
    int block_size, num_blocks, max_blocks;
};

namespace {

thread_local char g_hip_msg[256] = "";

int hip_fail(hipError_t e, const char* what) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s: %s", what, hipGetErrorString(e));
    return TP_E_HIP;
}

#define HIP_TRY(call)                                         \
    do {                                                      \
        hipError_t e_ = (call);                               \
        if (e_ != hipSuccess) return hip_fail(e_, #call);     \
    } while (0)

#define LAUNCH_CHECK(what)                                    \
    do {                                                      \
        hipError_t e_ = hipGetLastError();                    \
        if (e_ != hipSuccess) return hip_fail(e_, what);      \
    } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Device address of `scratch` per device, looked up once with the device
// current (hipGetSymbolAddress), kept for every later call on that device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};

int scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return TP_E_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[device]) return TP_OK;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    // the array's workspace starts with the decode merge counters: zero them once
    zero_ints((int*)p, kDecodeCounters, nullptr);
    const hipError_t z = hipGetLastError();
    if (z != hipSuccess) return hip_fail(z, "zero counters");
    const hipError_t sy = hipDeviceSynchronize();
    if (sy != hipSuccess) return hip_fail(sy, "hipDeviceSynchronize");
    g_scratch_dev[device] = (char*)p;
    return TP_OK;
}

char* scratch_of(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_dev[device];
}

// The workspace starts with the decode attention's merge counters, which
// must be zero before a call (every call leaves them zero again).
constexpr size_t kCounterBytes = (size_t)kDecodeCounters * sizeof(int);

int ensure_ws(tp_shard* s, size_t bytes, hipStream_t st) {
    if (bytes <= s->ws_bytes) return TP_OK;
    if (s->ws) {
        hipError_t e = hipFree(s->ws);  // waits for work that may still use it
        s->ws = nullptr;
        s->ws_bytes = 0;
        if (e != hipSuccess) return hip_fail(e, "hipFree(workspace)");
    }
    size_t b = (bytes + 255) & ~(size_t)255;
    hipError_t e = hipMalloc((void**)&s->ws, b);
    if (e != hipSuccess) {
        s->ws = nullptr;
        hip_fail(e, "hipMalloc(workspace)");
        return TP_E_NOMEM;
    }
    s->ws_bytes = b;
    zero_ints((int*)s->ws, kDecodeCounters, st);
    LAUNCH_CHECK("zero counters");
    return TP_OK;
}

// cos/sin tables of the fp32 path (the bf16 kernels rotate with s->rrev alone)
int ensure_rope(tp_shard* s, int npos, hipStream_t st) {
    if (!s->o.rope || s->o.dtype != TP_F32 || npos <= s->rope_npos) return TP_OK;
    int want = std::max(npos, std::max(2 * s->rope_npos, 4096));
    if (s->rcos) {
        hipError_t e1 = hipFree(s->rcos), e2 = hipFree(s->rsin);
        s->rcos = s->rsin = nullptr;
        s->rope_npos = 0;
        if (e1 != hipSuccess) return hip_fail(e1, "hipFree(rope)");
        if (e2 != hipSuccess) return hip_fail(e2, "hipFree(rope)");
    }
    if (!s->rrev && hipMalloc((void**)&s->rrev, (size_t)(s->d / 2) * sizeof(double)) != hipSuccess) {
        s->rrev = nullptr;
        return TP_E_NOMEM;
    }
    size_t bytes = (size_t)want * (s->d / 2) * sizeof(float);
    if (hipMalloc((void**)&s->rcos, bytes) != hipSuccess || hipMalloc((void**)&s->rsin, bytes) != hipSuccess) {
        if (s->rcos) (void)hipFree(s->rcos);
        s->rcos = s->rsin = nullptr;
        return TP_E_NOMEM;
    }
    rope_table(s->rcos, s->rsin, s->rrev, want, s->d, s->o.rope_theta, st);
    LAUNCH_CHECK("rope_table");
    s->rope_npos = want;
    return TP_OK;
}

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout for T tokens: merge counters | n | q | o | k,v (when no
// cache) | act | decode scratch | decode partial (the fused-sum entry point's
// own partial where its epilogue cannot take the sum)
struct Layout {
    size_t n, q, o, kv, act, scr, part, total;
};
Layout layout(const tp_shard* s, long long T, int len_decode, int batch_decode) {
    Layout L;
    size_t e = s->esz;
    L.n = al(kCounterBytes);
    L.q = L.n + al((size_t)T * s->hidden * e);
    L.o = L.q + al((size_t)T * s->hl * s->d * e);
    L.kv = L.o + al((size_t)T * s->hl * s->d * e);
    L.act = L.kv + al((size_t)2 * T * s->kvl * s->d * e);
    L.scr = L.act + al((size_t)T * s->fl * e);
    size_t scr = len_decode > 0 ? attn_decode_scratch_bytes(batch_decode, s->hl, s->kvl, len_decode, s->d) : 0;
    if (batch_decode > 1) {
        // split-K scratch of the small-batch decode projections
        const int shapes[4][2] = {{s->nqkv, s->hidden}, {s->hidden, s->hl * s->d}, {s->nup, s->hidden},
                                  {s->hidden, s->fl}};
        for (const auto& nk : shapes) scr = std::max(scr, skinny_scratch_bytes(batch_decode, nk[0], nk[1]));
    }
    L.part = L.scr + al(scr);
    L.total = L.part + (batch_decode > 0 ? al((size_t)batch_decode * s->hidden * sizeof(float)) : 0);
    return L;
}

// rows x cols of packed projection i (0 Q/K/V, 1 W_o block, 2 gate/up, 3 W_down block)
void fp8_shape(const tp_shard* s, int i, int* rows, int* cols) {
    const int R[4] = {s->nqkv, s->hidden, s->nup, s->hidden};
    const int C[4] = {s->hidden, s->hl * s->d, s->hidden, s->fl};
    *rows = R[i];
    *cols = C[i];
}

int launch_qkv(tp_shard* s, const void* n_in, long long M, int S, int pos0, void* q, void* k, void* v,
               int ld_seq, hipStream_t st, const int* pos_dev = nullptr, const tp_kv* paged = nullptr) {
    Epilogue epi{};
    epi.mode = EPI_QKV;
    epi.qkv.S = S;
    epi.qkv.pos0 = pos0;
    epi.qkv.pos_dev = pos_dev;
    if (paged && paged->table) {
        epi.qkv.table = paged->table;
        epi.qkv.bsz = paged->block_size;
        epi.qkv.max_blocks = paged->max_blocks;
    }
    epi.qkv.hl = s->hl;
    epi.qkv.kvl = s->kvl;
    epi.qkv.d = s->d;
    epi.qkv.q = q;
    epi.qkv.k = k;
    epi.qkv.v = v;
    epi.qkv.ld_seq = ld_seq;
    epi.qkv.rope_cos = s->o.rope ? s->rcos : nullptr;
    epi.qkv.rope_sin = s->o.rope ? s->rsin : nullptr;
    epi.qkv.rope_rev = s->o.rope ? s->rrev : nullptr;
    if (s->o.dtype == TP_BF16)
        gemm_bf16((const bf16*)n_in, s->hidden, (const bf16*)s->w_qkv, s->hidden, (int)M, s->nqkv, s->hidden, epi, st);
    else
        gemm_f32((const float*)n_in, s->hidden, (const float*)s->w_qkv, s->hidden, (int)M, s->nqkv, s->hidden, epi, st);
    LAUNCH_CHECK("qkv projection");
    return TP_OK;
}

int launch_proj(tp_shard* s, const void* A, long long M, int K, const void* W, int N, int mode, void* out,
                long long ldo, hipStream_t st, LenUpdate len = LenUpdate{nullptr, 0, 0, nullptr}) {
    Epilogue epi{};
    epi.mode = mode;
    epi.out = out;
    epi.ldo = ldo;
    epi.len = len;
    if (s->o.dtype == TP_BF16)
        gemm_bf16((const bf16*)A, K, (const bf16*)W, K, (int)M, N, K, epi, st);
    else
        gemm_f32((const float*)A, K, (const float*)W, K, (int)M, N, K, epi, st);
    LAUNCH_CHECK("projection");
    return TP_OK;
}

int launch_norm(tp_shard* s, const void* x, const void* g, void* out, long long rows, hipStream_t st) {
    if (s->o.dtype == TP_BF16)
        rmsnorm_bf16((const bf16*)x, (const bf16*)g, (bf16*)out, (int)rows, s->hidden, s->o.eps, st);
    else
        rmsnorm_f32((const float*)x, (const float*)g, (float*)out, (int)rows, s->hidden, s->o.eps, st);
    LAUNCH_CHECK("rmsnorm");
    return TP_OK;
}

// Decode projections stream each weight once.  Up to four sequences: the
// GEMV kernel, whose threads hold a whole input row of every sequence in
// registers (K <= 16384), with the norm and the epilogue fused (one launch per
// projection).  5..64 sequences: RMSNorm (if any) into the workspace, then the
// split-K MFMA projection and its epilogue pass.  More sequences take the GEMM
// path.
constexpr int kGemvMaxBatch = 4;
constexpr int kSkinnyMaxBatch = 64;
constexpr int kGemvMaxK = 16384;

int launch_gemv(tp_shard* s, const void* x, int B, const void* gamma, const void* W, int N, int K,
                const Epilogue& epi, void* nbuf, void* scratch, hipStream_t st, int fp8_index) {
    if (B == 1 && s->o.decode_fp8) {
        gemv_fp8((const bf16*)x, (const bf16*)gamma, s->o.eps, s->q8[fp8_index], s->s8[fp8_index], N, K, epi, st);
        LAUNCH_CHECK("fp8 gemv");
        return TP_OK;
    }
    if (B <= kGemvMaxBatch) {
        gemv_bf16((const bf16*)x, B, (const bf16*)gamma, s->o.eps, (const bf16*)W, N, K, epi, st);
        LAUNCH_CHECK("gemv");
        return TP_OK;
    }
    const void* xin = x;
    if (gamma) {
        rmsnorm_bf16((const bf16*)x, (const bf16*)gamma, (bf16*)nbuf, B, K, s->o.eps, st);
        LAUNCH_CHECK("rmsnorm");
        xin = nbuf;
    }
    skinny_bf16((const bf16*)xin, B, (const bf16*)W, N, K, (float*)scratch, epi, st);
    LAUNCH_CHECK("skinny projection");
    return TP_OK;
}

// Brackets one kernel launch with two events when the shard's timer is on.
struct KTimer {
    tp_shard* s;
    hipStream_t st;
    size_t slot;
    bool on;
    KTimer(tp_shard* s_, int kind, hipStream_t st_) : s(s_), st(st_), slot(0), on(false) {
        if (s->timing && ((s->tmask >> kind) & 1u) && s->evused + 2 <= s->ev.size()) {
            on = true;
            slot = s->evused;
            s->evused += 2;
            s->evkind.push_back(kind);
            (void)hipEventRecord(s->ev[slot], st);
        }
    }
    ~KTimer() {
        if (on) (void)hipEventRecord(s->ev[slot + 1], st);
    }
};
constexpr size_t kTimerEvents = 8192;

#define TRY(x)                    \
    do {                          \
        int r_ = (x);             \
        if (r_ != TP_OK) return r_; \
    } while (0)

}  // namespace

extern "C" {

const char* tp_status_string(int status) {
    switch (status) {
        case TP_OK: return "ok";
        case TP_E_ARG: return "invalid argument";
        case TP_E_DIVIDE: return "heads, kv_heads or ffn not divisible by the tp degree, or degree above the head count";
        case TP_E_RANK: return "rank outside [0, tp_degree)";
        case TP_E_NOMEM: return "out of memory";
        case TP_E_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
        case TP_E_KV_FULL: return "KV cache full";
        case TP_E_STATE: return "call out of order (weights not loaded?)";
        case TP_E_SCRATCH: return "the call needs more workspace than the allocation-free entry point's static "
                                  "scratch array holds (TP_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int tp_shard_create(int hidden, int heads, int kv_heads, int ffn, int tp_degree, int rank, const tp_opts* opts,
                    tp_shard** out) {
    if (!out) return TP_E_ARG;
    *out = nullptr;
    if (hidden <= 0 || heads <= 0 || kv_heads <= 0 || ffn <= 0 || tp_degree <= 0) return TP_E_ARG;
    tp_opts o = {TP_BF16, TP_ACT_SWIGLU, 1, 1e-5f, 1, 10000.0f, 0};
    if (opts) o = *opts;
    if (o.decode_fp8 != 0 && o.decode_fp8 != 1) return TP_E_ARG;
    if (o.decode_fp8 && o.dtype != TP_BF16) return TP_E_ARG;
    if (o.dtype != TP_BF16 && o.dtype != TP_F32) return TP_E_ARG;
    if (o.act != TP_ACT_SWIGLU && o.act != TP_ACT_GELU) return TP_E_ARG;
    if (o.rmsnorm && !(o.eps >= 0.f)) return TP_E_ARG;
    if (o.rope && !(o.rope_theta > 0.f)) return TP_E_ARG;
    if (hidden % heads || heads % kv_heads) return TP_E_ARG;
    if (rank < 0 || rank >= tp_degree) return TP_E_RANK;
    if (tp_degree > heads || heads % tp_degree || kv_heads % tp_degree || ffn % tp_degree) return TP_E_DIVIDE;
    const int d = hidden / heads;
    if (d != 64 && d != 128) return TP_E_ARG;         // packed head layout and attention tiles
    if (hidden % 64) return TP_E_ARG;                 // GEMM K steps / GEMV rows
    if ((ffn / tp_degree) % 64) return TP_E_ARG;      // gate/up pairing and down-projection K steps
    tp_shard* s = new (std::nothrow) tp_shard();
    if (!s) return TP_E_NOMEM;
    s->hidden = hidden;
    s->heads = heads;
    s->kv_heads = kv_heads;
    s->ffn = ffn;
    s->t = tp_degree;
    s->rank = rank;
    s->o = o;
    s->d = d;
    s->hl = heads / tp_degree;
    s->kvl = kv_heads / tp_degree;
    s->fl = ffn / tp_degree;
    s->nqkv = (s->hl + 2 * s->kvl) * d;
    s->nup = o.act == TP_ACT_SWIGLU ? 2 * s->fl : s->fl;
    s->esz = o.dtype == TP_BF16 ? 2 : 4;
    s->device = -1;
    *out = s;
    return TP_OK;
}

int tp_shard_load_weights(tp_shard* s, const tp_weights* W, void* stream) {
    if (!s || !W) return TP_E_ARG;
    const bool swiglu = s->o.act == TP_ACT_SWIGLU;
    if (!W->wq || !W->wk || !W->wv || !W->wo || !W->w_up || !W->w_down) return TP_E_ARG;
    if (swiglu && !W->w_gate) return TP_E_ARG;
    if (s->o.rmsnorm && (!W->g1 || !W->g2)) return TP_E_ARG;
    hipStream_t st = (hipStream_t)stream;
    const size_t e = s->esz;
    const int h = s->hidden, d = s->d, r = s->rank;
    if (!s->w_qkv) {
        HIP_TRY(hipGetDevice(&s->device));
        TRY(scratch_setup(s->device));
        void** bufs[] = {&s->w_qkv, &s->w_o, &s->w_up, &s->w_down, &s->g1, &s->g2};
        size_t sizes[] = {(size_t)s->nqkv * h * e, (size_t)h * s->hl * d * e, (size_t)s->nup * h * e,
                          (size_t)h * s->fl * e, (size_t)h * e, (size_t)h * e};
        for (int i = 0; i < 6; ++i) {
            if (hipMalloc(bufs[i], sizes[i]) != hipSuccess) {
                for (int j = 0; j < 6; ++j)
                    if (*bufs[j]) { (void)hipFree(*bufs[j]); *bufs[j] = nullptr; }
                return TP_E_NOMEM;
            }
        }
    }
    // Q/K/V rows of the rank's heads, each head's rows packed in 64-row groups
    // whose halves are the rotate-half partners (dims 32g.. and d/2 + 32g..).
    struct Region { const void* src; int heads_total, first, count; size_t dst_row; };
    Region regs[3] = {{W->wq, s->heads, r * s->hl, s->hl, 0},
                      {W->wk, s->kv_heads, r * s->kvl, s->kvl, (size_t)s->hl * d},
                      {W->wv, s->kv_heads, r * s->kvl, s->kvl, (size_t)(s->hl + s->kvl) * d}};
    for (const Region& R : regs) {
        for (int g = 0; g < d / 64; ++g)
            for (int c = 0; c < 2; ++c) {
                char* dst = (char*)s->w_qkv + (R.dst_row + 64 * g + 32 * c) * h * e;
                const char* src = (const char*)R.src + ((size_t)R.first * d + c * (d / 2) + 32 * g) * h * e;
                HIP_TRY(hipMemcpy2DAsync(dst, (size_t)d * h * e, src, (size_t)d * h * e, (size_t)32 * h * e, R.count,
                                         hipMemcpyDeviceToDevice, st));
            }
    }
    // W_o columns of the rank's heads (row-parallel): [h, hl*d] from [h, heads*d]
    HIP_TRY(hipMemcpy2DAsync(s->w_o, (size_t)s->hl * d * e, (const char*)W->wo + (size_t)r * s->hl * d * e,
                             (size_t)s->heads * d * e, (size_t)s->hl * d * e, h, hipMemcpyDeviceToDevice, st));
    // FFN up (and gate): the rank's FFN rows; SwiGLU interleaves gate/up in 32-row blocks
    if (swiglu) {
        const size_t blk = (size_t)32 * h * e;
        const char* gsrc = (const char*)W->w_gate + (size_t)r * s->fl * h * e;
        const char* usrc = (const char*)W->w_up + (size_t)r * s->fl * h * e;
        HIP_TRY(hipMemcpy2DAsync(s->w_up, 2 * blk, gsrc, blk, blk, s->fl / 32, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpy2DAsync((char*)s->w_up + blk, 2 * blk, usrc, blk, blk, s->fl / 32, hipMemcpyDeviceToDevice, st));
    } else {
        HIP_TRY(hipMemcpyAsync(s->w_up, (const char*)W->w_up + (size_t)r * s->fl * h * e, (size_t)s->fl * h * e,
                               hipMemcpyDeviceToDevice, st));
    }
    // W_down columns of the rank's FFN block (row-parallel): [h, fl] from [h, ffn]
    HIP_TRY(hipMemcpy2DAsync(s->w_down, (size_t)s->fl * e, (const char*)W->w_down + (size_t)r * s->fl * e,
                             (size_t)s->ffn * e, (size_t)s->fl * e, h, hipMemcpyDeviceToDevice, st));
    if (s->o.rmsnorm) {
        HIP_TRY(hipMemcpyAsync(s->g1, W->g1, (size_t)h * e, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(s->g2, W->g2, (size_t)h * e, hipMemcpyDeviceToDevice, st));
    }
    if (s->o.rope) {
        // the rotation per position of every dim pair, in turns
        if (!s->rrev && hipMalloc((void**)&s->rrev, (size_t)(d / 2) * sizeof(double)) != hipSuccess) {
            s->rrev = nullptr;
            return TP_E_NOMEM;
        }
        rope_turns(s->rrev, d, s->o.rope_theta, st);
        LAUNCH_CHECK("rope_turns");
    }
    if (s->o.decode_fp8) {
        const void* src[4] = {s->w_qkv, s->w_o, s->w_up, s->w_down};
        for (int i = 0; i < 4; ++i) {
            int rows, cols;
            fp8_shape(s, i, &rows, &cols);
            if (!s->q8[i] || !s->s8[i]) {
                // both or neither: a half-made pair is freed, so a retry starts clean
                if (hipMalloc((void**)&s->q8[i], (size_t)rows * cols) != hipSuccess ||
                    hipMalloc((void**)&s->s8[i], (size_t)rows * sizeof(float)) != hipSuccess) {
                    if (s->q8[i]) (void)hipFree(s->q8[i]);
                    if (s->s8[i]) (void)hipFree(s->s8[i]);
                    s->q8[i] = nullptr;
                    s->s8[i] = nullptr;
                    return TP_E_NOMEM;
                }
            }
            quant_rows_e4m3((const bf16*)src[i], rows, cols, s->q8[i], s->s8[i], st);
            LAUNCH_CHECK("fp8 quantisation");
        }
    }
    s->loaded = true;
    return TP_OK;
}

int tp_shard_fp8_view(tp_shard* s, int which, void** codes, float** scales, int* rows, int* cols) {
    if (!s || which < 0 || which > 3) return TP_E_ARG;
    if (!s->o.decode_fp8 || !s->loaded || !s->q8[which]) return TP_E_STATE;
    int r, c;
    fp8_shape(s, which, &r, &c);
    if (codes) *codes = s->q8[which];
    if (scales) *scales = s->s8[which];
    if (rows) *rows = r;
    if (cols) *cols = c;
    return TP_OK;
}

int tp_shard_reserve(tp_shard* s, long long max_tokens) {
    if (!s || max_tokens <= 0) return TP_E_ARG;
    Layout L = layout(s, max_tokens, 0, 0);
    TRY(ensure_ws(s, L.total, nullptr));
    HIP_TRY(hipDeviceSynchronize());   // the counters are zero before any stream uses the workspace
    return TP_OK;
}

int tp_kv_create(const tp_shard* s, int batch, int max_seq, tp_kv** out) {
    if (!s || !out || batch <= 0 || max_seq <= 0) return TP_E_ARG;
    if (s->o.dtype == TP_F32 && max_seq > 16000) return TP_E_ARG;  // fp32 attention keeps scores in LDS
    *out = nullptr;
    tp_kv* kv = new (std::nothrow) tp_kv();
    if (!kv) return TP_E_NOMEM;
    kv->batch = batch;
    kv->max_seq = max_seq;
    kv->len = 0;
    kv->kvl = s->kvl;
    kv->d = s->d;
    kv->esz = s->esz;
    kv->dtype = s->o.dtype;
    size_t bytes = (size_t)batch * s->kvl * max_seq * s->d * s->esz;
    if (hipMalloc(&kv->k, bytes) != hipSuccess || hipMalloc(&kv->v, bytes) != hipSuccess ||
        hipMalloc((void**)&kv->dlen, 2 * sizeof(int)) != hipSuccess) {
        if (kv->k) (void)hipFree(kv->k);
        if (kv->v) (void)hipFree(kv->v);
        delete kv;
        return TP_E_NOMEM;
    }
    if (hipMemset(kv->k, 0, bytes) != hipSuccess || hipMemset(kv->v, 0, bytes) != hipSuccess ||
        hipMemset(kv->dlen, 0, 2 * sizeof(int)) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(kv->k);
        (void)hipFree(kv->v);
        (void)hipFree(kv->dlen);
        delete kv;
        return hip_fail(hipGetLastError(), "hipMemset(kv)");
    }
    *out = kv;
    return TP_OK;
}

int tp_kv_create_paged(const tp_shard* s, int batch, int max_seq, int block_size, int num_blocks, tp_kv** out) {
    if (!s || !out || batch <= 0 || max_seq <= 0 || num_blocks <= 0) return TP_E_ARG;
    if (s->o.dtype != TP_BF16) return TP_E_ARG;
    if (block_size < 16 || block_size > 1024 || (block_size & (block_size - 1))) return TP_E_ARG;
    *out = nullptr;
    tp_kv* kv = new (std::nothrow) tp_kv();
    if (!kv) return TP_E_NOMEM;
    kv->batch = batch;
    kv->max_seq = max_seq;
    kv->kvl = s->kvl;
    kv->d = s->d;
    kv->esz = s->esz;
    kv->dtype = s->o.dtype;
    kv->block_size = block_size;
    kv->num_blocks = num_blocks;
    kv->max_blocks = (max_seq + block_size - 1) / block_size;
    const size_t pool = (size_t)num_blocks * s->kvl * block_size * s->d * s->esz;
    const size_t tbytes = (size_t)batch * kv->max_blocks * sizeof(int);
    if (hipMalloc(&kv->k, pool) != hipSuccess || hipMalloc(&kv->v, pool) != hipSuccess ||
        hipMalloc((void**)&kv->dlen, 2 * sizeof(int)) != hipSuccess || hipMalloc((void**)&kv->table, tbytes) != hipSuccess) {
        tp_kv_destroy(kv);
        return TP_E_NOMEM;
    }
    // until a table is set, sequence b uses blocks b * max_blocks + i (block 0 past the pool)
    std::vector<int> t0((size_t)batch * kv->max_blocks);
    for (size_t i = 0; i < t0.size(); ++i) t0[i] = (int)(i < (size_t)num_blocks ? i : 0);
    if (hipMemset(kv->k, 0, pool) != hipSuccess || hipMemset(kv->v, 0, pool) != hipSuccess ||
        hipMemset(kv->dlen, 0, 2 * sizeof(int)) != hipSuccess ||
        hipMemcpy(kv->table, t0.data(), tbytes, hipMemcpyHostToDevice) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        const int rc = hip_fail(hipGetLastError(), "paged kv init");
        tp_kv_destroy(kv);
        return rc;
    }
    *out = kv;
    return TP_OK;
}

int tp_kv_set_block_table(tp_kv* kv, const int* host_table) {
    if (!kv || !host_table) return TP_E_ARG;
    if (!kv->table) return TP_E_STATE;
    const size_t n = (size_t)kv->batch * kv->max_blocks;
    for (size_t i = 0; i < n; ++i)
        if (host_table[i] < 0 || host_table[i] >= kv->num_blocks) return TP_E_ARG;
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipMemcpy(kv->table, host_table, n * sizeof(int), hipMemcpyHostToDevice));
    return TP_OK;
}

int tp_kv_view(tp_kv* kv, void** k, void** v) {
    if (!kv) return TP_E_ARG;
    if (k) *k = kv->k;
    if (v) *v = kv->v;
    return TP_OK;
}

int tp_kv_set_len(tp_kv* kv, int len) {
    if (!kv || len < 0 || len > kv->max_seq) return TP_E_ARG;
    const int v[2] = {len, 0};   // the length, and a cleared overflow flag
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipMemcpy(kv->dlen, v, sizeof(v), hipMemcpyHostToDevice));
    kv->len = len;
    return TP_OK;
}

int tp_kv_get_len(const tp_kv* kv, int* len) {
    if (!kv || !len) return TP_E_ARG;
    int v[2] = {0, 0};
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipMemcpy(v, kv->dlen, sizeof(v), hipMemcpyDeviceToHost));
    const_cast<tp_kv*>(kv)->len = v[0];   // replays of captured calls advance only the device copy
    *len = v[0];
    return v[1] ? TP_E_KV_FULL : TP_OK;
}

}  // extern "C"

namespace tp {
// elementwise.hip: dlen[0] = len, dlen[1] = 0 (the cache length and a
// cleared overflow flag), in stream order
void set_kv_len(int* dlen, int len, hipStream_t st);
}  // namespace tp

extern "C" {

int tp_kv_set_len_async(tp_kv* kv, int len, void* stream) {
    if (!kv || len < 0 || len > kv->max_seq) return TP_E_ARG;
    set_kv_len(kv->dlen, len, (hipStream_t)stream);
    LAUNCH_CHECK("set_kv_len");
    kv->len = len;
    return TP_OK;
}

int tp_kv_get_len_stream(const tp_kv* kv, int* len, void* stream) {
    if (!kv || !len) return TP_E_ARG;
    int v[2] = {0, 0};
    hipStream_t st = (hipStream_t)stream;
    HIP_TRY(hipMemcpyAsync(v, kv->dlen, sizeof(v), hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    const_cast<tp_kv*>(kv)->len = v[0];
    *len = v[0];
    return v[1] ? TP_E_KV_FULL : TP_OK;
}

}  // extern "C"

namespace {

// The all-reduce's sum of a fused-sum call: the t ranks' partials (slot
// `self` unused), the residual and the reduced output.
struct FuseSum {
    const float* const* parts;
    const void* residual;
    void* out;
};

// Epilogue of a row-parallel projection whose all-reduce sum is folded in.
Epilogue sum_epilogue(const tp_shard* s, const FuseSum& f) {
    Epilogue e{};
    e.mode = EPI_SUM;
    e.out = f.out;
    e.ldo = s->hidden;
    for (int r = 0; r < kSumMaxRanks; ++r) e.sum.p[r] = r < s->t && r != s->rank ? f.parts[r] : nullptr;
    e.sum.residual = (const bf16*)f.residual;
    e.sum.t = s->t;
    e.sum.self = s->rank;
    return e;
}

// One prefill stage.  With `fuse`, the stage's row-parallel projection ends
// in the all-reduce's sum: in its epilogue (bf16 shards, up to kSumMaxRanks
// ranks), else through this rank's partial in the workspace and a reduce.
int prefill_stage(tp_shard* s, int stage, const void* x, int batch, int seq, tp_kv* kv, float* partial,
                  hipStream_t st, const FuseSum* fuse) {
    const bool prenorm = (stage & TP_STAGE_PRENORM) != 0;
    stage &= ~TP_STAGE_PRENORM;
    if (stage != TP_STAGE_ATTN && stage != TP_STAGE_MLP) return TP_E_ARG;
    if (!s->loaded) return TP_E_STATE;
    const long long T = (long long)batch * seq;
    if (T > INT32_MAX / 2) return TP_E_ARG;
    if (stage == TP_STAGE_MLP && kv) return TP_E_ARG;
    if (stage == TP_STAGE_ATTN && kv) {
        if (kv->batch != batch || kv->dtype != s->o.dtype || kv->kvl != s->kvl) return TP_E_ARG;
        if (seq > kv->max_seq) return TP_E_KV_FULL;
    }
    if (s->o.dtype == TP_F32 && stage == TP_STAGE_ATTN && seq > 16000) return TP_E_ARG;
    const bool bf = s->o.dtype == TP_BF16;
    const bool sum_epi = fuse && bf && s->t <= kSumMaxRanks;
    Layout L = layout(s, T, 0, 0);
    if (fuse && !sum_epi) {   // this rank's partial goes to the workspace, then the reduce
        L.part = L.total;
        L.total += al((size_t)T * s->hidden * sizeof(float));
    }
    TRY(ensure_ws(s, L.total, st));
    char* ws = s->ws;
    if (fuse && !sum_epi) partial = (float*)(ws + L.part);
    // the stage's row-parallel projection: an fp32 partial, or the sum folded in
    auto row_parallel = [&](const void* A, int K, const void* W, LenUpdate len) -> int {
        if (!sum_epi) {
            TRY(launch_proj(s, A, T, K, W, s->hidden, EPI_F32, partial, s->hidden, st, len));
            if (!fuse) return TP_OK;
            const float* ptrs[64];
            for (int r = 0; r < s->t; ++r) ptrs[r] = r == s->rank ? partial : fuse->parts[r];
            partial_reduce(ptrs, s->t, fuse->residual, fuse->out, T * s->hidden, bf, st);
            LAUNCH_CHECK("partial_reduce");
            return TP_OK;
        }
        Epilogue e = sum_epilogue(s, *fuse);
        e.len = len;
        gemm_bf16((const bf16*)A, K, (const bf16*)W, K, (int)T, s->hidden, K, e, st);
        LAUNCH_CHECK("projection with the reduce");
        return TP_OK;
    };
    s->dbg_base = ws;
    s->off_n = L.n;
    s->off_o = L.o;
    s->off_act = L.act;
    const void* xin = x;
    if (stage == TP_STAGE_ATTN) {
        TRY(ensure_rope(s, seq, st));
        if (s->o.rmsnorm && !prenorm) {
            KTimer kt(s, TP_K_RMSNORM, st);
            TRY(launch_norm(s, x, s->g1, ws + L.n, T, st));
            xin = ws + L.n;
        }
        void *kd, *vd;
        int ld_seq;
        const bool paged = kv && kv->table;
        if (kv && !paged) {
            kd = kv->k;
            vd = kv->v;
            ld_seq = kv->max_seq;
        } else {   // no cache, or a paged one (filled from the contiguous rows below)
            kd = ws + L.kv;
            vd = ws + L.kv + (size_t)T * s->kvl * s->d * s->esz;
            ld_seq = seq;
        }
        {
            KTimer kt(s, TP_K_GEMM_QKV, st);
            TRY(launch_qkv(s, xin, T, seq, 0, ws + L.q, kd, vd, ld_seq, st));
        }
        if (paged) {
            kv_to_pages((const bf16*)kd, (const bf16*)vd, (bf16*)kv->k, (bf16*)kv->v, batch, s->kvl, seq, s->d,
                        kv->table, kv->block_size, kv->max_blocks, st);
            LAUNCH_CHECK("kv pages");
        }
        {
            KTimer kt(s, TP_K_ATTN_PREFILL, st);
            if (s->o.dtype == TP_BF16)
                attn_prefill_bf16((const bf16*)(ws + L.q), (const bf16*)kd, (const bf16*)vd, (bf16*)(ws + L.o),
                                  batch, s->hl, s->kvl, seq, ld_seq, s->d, st);
            else
                attn_f32((const float*)(ws + L.q), (const float*)kd, (const float*)vd, (float*)(ws + L.o), batch,
                         s->hl, s->kvl, seq, 0, ld_seq, s->d, st);
            LAUNCH_CHECK("attention");
        }
        {
            KTimer kt(s, TP_K_GEMM_OUT, st);
            TRY(row_parallel(ws + L.o, s->hl * s->d, s->w_o,
                             kv ? LenUpdate{kv->dlen, seq, 0, kv->dlen + 1} : LenUpdate{nullptr, 0, 0, nullptr}));
        }
        if (kv) kv->len = seq;
        s->attn_seen = true;
    } else {
        if (s->o.rmsnorm && !prenorm) {
            KTimer kt(s, TP_K_RMSNORM, st);
            TRY(launch_norm(s, x, s->g2, ws + L.n, T, st));
            xin = ws + L.n;
        }
        const int mode = s->o.act == TP_ACT_SWIGLU ? EPI_SWIGLU : EPI_GELU;
        {
            KTimer kt(s, TP_K_GEMM_UP, st);
            TRY(launch_proj(s, xin, T, s->hidden, s->w_up, s->nup, mode, ws + L.act, s->fl, st));
        }
        {
            KTimer kt(s, TP_K_GEMM_DOWN, st);
            TRY(row_parallel(ws + L.act, s->fl, s->w_down, LenUpdate{nullptr, 0, 0, nullptr}));
        }
    }
    return TP_OK;
}

}  // namespace

extern "C" {

int tp_shard_forward_prefill(tp_shard* s, int stage, const void* x, int batch, int seq, tp_kv* kv, float* partial,
                             void* stream) {
    if (!s || !x || !partial || batch <= 0 || seq <= 0) return TP_E_ARG;
    if (!aligned16(x) || !aligned16(partial)) return TP_E_ARG;
    return prefill_stage(s, stage, x, batch, seq, kv, partial, (hipStream_t)stream, nullptr);
}

int tp_shard_forward_prefill_reduce(tp_shard* s, int stage, const void* x, int batch, int seq, tp_kv* kv,
                                    const float* const* partials, const void* residual, void* out, void* stream) {
    if (!s || !x || !partials || !out || batch <= 0 || seq <= 0) return TP_E_ARG;
    for (int r = 0; r < s->t; ++r)
        if (r != s->rank && (!partials[r] || !aligned16(partials[r]))) return TP_E_ARG;
    if (!aligned16(x) || !aligned16(out) || (residual && !aligned16(residual))) return TP_E_ARG;
    // out must not overlap the stage's input or any other rank's partial
    const size_t n = (size_t)batch * seq * s->hidden;
    const uintptr_t xb = (uintptr_t)x, ob = (uintptr_t)out, oe = ob + n * s->esz;
    if (xb < oe && ob < xb + n * s->esz) return TP_E_ARG;
    for (int r = 0; r < s->t; ++r)
        if (r != s->rank) {
            const uintptr_t pb = (uintptr_t)partials[r];
            if (pb < oe && ob < pb + n * sizeof(float)) return TP_E_ARG;
        }
    const FuseSum f{partials, residual, out};
    return prefill_stage(s, stage, x, batch, seq, kv, nullptr, (hipStream_t)stream, &f);
}

}  // extern "C"

namespace {

// One decode stage over the workspace at `base`: the library's own workspace
// (grown on demand) or, for the allocation-free entry point, the device's
// static scratch array.  With `fuse`, the stage's row-parallel projection
// also takes the reduce over the ranks: in its epilogue on the GEMV and
// split-K paths, else as a reduce of its partial (kept in the workspace).
int decode_stage(tp_shard* s, int stage, const void* x, int batch, tp_kv* kv, float* partial, void* stream,
                 bool noalloc, const FuseSum* fuse = nullptr) {
    const bool prenorm = (stage & TP_STAGE_PRENORM) != 0;
    stage &= ~TP_STAGE_PRENORM;
    if (!s || !x || (!partial && !fuse) || batch <= 0) return TP_E_ARG;
    if (stage != TP_STAGE_ATTN && stage != TP_STAGE_MLP) return TP_E_ARG;
    if (!aligned16(x) || (partial && !aligned16(partial))) return TP_E_ARG;
    if (!s->loaded) return TP_E_STATE;
    hipStream_t st = (hipStream_t)stream;
    const bool bf = s->o.dtype == TP_BF16;
    const int kmax = batch == 1 && s->o.decode_fp8 ? 2 * kGemvMaxK : kGemvMaxK;   // E4M3 rows are half as long
    const bool use_gemv = bf && (batch <= kGemvMaxBatch ? s->hidden <= kmax && s->hl * s->d <= kmax && s->fl <= kmax
                                                         : batch <= kSkinnyMaxBatch);
    if (stage == TP_STAGE_ATTN) {
        if (!kv) return TP_E_ARG;
        if (kv->batch != batch || kv->dtype != s->o.dtype || kv->kvl != s->kvl) return TP_E_ARG;
        if (kv->len >= kv->max_seq) return TP_E_KV_FULL;
    } else if (kv) {
        return TP_E_ARG;
    } else if (!s->attn_seen) {
        return TP_E_STATE;   // a decode MLP stage follows the step's ATTN stage
    }
    // bf16 decode takes the cache length from the device copy, so a captured
    // call stays valid on replay; the fp32 path uses the host copy.  Capture
    // executes nothing, so it leaves the host copy alone.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(st, &cs));
    const bool capturing = cs != hipStreamCaptureStatusNone;
    if (!bf && capturing) return TP_E_STATE;
    if (noalloc && !bf) return TP_E_STATE;   // the fp32 path's rotation tables grow with the cache
    const int L = stage == TP_STAGE_ATTN ? kv->len : 0;
    Layout lay = layout(s, batch, stage == TP_STAGE_ATTN ? kv->max_seq : 0, batch);
    char* ws;
    if (noalloc) {
        if (lay.total > (size_t)TP_NOALLOC_SCRATCH_BYTES) return TP_E_SCRATCH;
        ws = scratch_of(s->device);
        if (ws == nullptr) return TP_E_STATE;
    } else {
        TRY(ensure_ws(s, lay.total, st));
        ws = s->ws;
    }
    s->dbg_base = ws;
    s->off_n = lay.n;
    s->off_o = lay.o;
    s->off_act = lay.act;
    // the sum goes into the GEMV or split-K epilogue (bf16, up to kSumMaxRanks
    // ranks); otherwise the stage writes its partial into the workspace and a
    // reduce follows
    const bool sum_epi = fuse && use_gemv && s->t <= kSumMaxRanks;
    float* own = fuse ? (float*)(ws + lay.part) : partial;
    auto set_sum = [&](Epilogue& e) {
        e.mode = EPI_SUM;
        e.out = fuse->out;
        e.ldo = s->hidden;
        for (int r = 0; r < kSumMaxRanks; ++r) e.sum.p[r] = r < s->t && r != s->rank ? fuse->parts[r] : nullptr;
        e.sum.residual = (const bf16*)fuse->residual;
        e.sum.t = s->t;
        e.sum.self = s->rank;
    };
    auto reduce_own = [&]() -> int {
        if (!fuse || sum_epi) return TP_OK;
        const float* ptrs[64];
        for (int r = 0; r < s->t; ++r) ptrs[r] = r == s->rank ? own : fuse->parts[r];
        partial_reduce(ptrs, s->t, fuse->residual, fuse->out, (long long)batch * s->hidden, bf, st);
        LAUNCH_CHECK("partial_reduce");
        return TP_OK;
    };
    if (stage == TP_STAGE_ATTN) {
        if (!noalloc) TRY(ensure_rope(s, kv->max_seq + 1, st));   // fp32: a query at position max_seq stays in range
        void* qbuf = ws + lay.q;
        if (use_gemv) {
            Epilogue epi{};
            epi.mode = EPI_QKV;
            epi.qkv = QKVDest{1, L, kv->dlen, s->hl, s->kvl, s->d, qbuf, kv->k, kv->v, kv->max_seq,
                              s->o.rope ? s->rcos : nullptr, s->o.rope ? s->rsin : nullptr,
                              s->o.rope ? s->rrev : nullptr, kv->table, kv->block_size, kv->max_blocks};
            KTimer kt(s, TP_K_GEMV_QKV, st);
            const void* g1 = s->o.rmsnorm && !prenorm ? s->g1 : nullptr;
            TRY(launch_gemv(s, x, batch, g1, s->w_qkv, s->nqkv, s->hidden, epi, ws + lay.n, ws + lay.scr, st, 0));
        } else {
            const void* xin = x;
            if (s->o.rmsnorm && !prenorm) {
                KTimer kt(s, TP_K_RMSNORM, st);
                TRY(launch_norm(s, x, s->g1, ws + lay.n, batch, st));
                xin = ws + lay.n;
            }
            KTimer kt(s, TP_K_GEMM_QKV, st);
            TRY(launch_qkv(s, xin, batch, 1, L, qbuf, kv->k, kv->v, kv->max_seq, st, bf ? kv->dlen : nullptr, kv));
        }
        {
            KTimer kt(s, TP_K_ATTN_DECODE, st);
            if (bf)
                attn_decode_bf16((const bf16*)qbuf, (const bf16*)kv->k, (const bf16*)kv->v, (bf16*)(ws + lay.o),
                                 (float*)(ws + lay.scr), (int*)ws, batch, s->hl, s->kvl, kv->dlen, kv->max_seq, s->d, kv->table,
                                 kv->block_size, kv->max_blocks, st);
            else
                attn_f32((const float*)qbuf, (const float*)kv->k, (const float*)kv->v, (float*)(ws + lay.o), batch,
                         s->hl, s->kvl, 1, L, kv->max_seq, s->d, st);
            LAUNCH_CHECK("decode attention");
        }
        if (use_gemv) {
            Epilogue epi{};
            epi.mode = EPI_F32;
            epi.out = own;
            epi.ldo = s->hidden;
            epi.len = LenUpdate{kv->dlen, -1, kv->max_seq, kv->dlen + 1};
            if (sum_epi) set_sum(epi);
            KTimer kt(s, TP_K_GEMV_OUT, st);
            TRY(launch_gemv(s, ws + lay.o, batch, nullptr, s->w_o, s->hidden, s->hl * s->d, epi, ws + lay.n,
                            ws + lay.scr, st, 1));
        } else {
            KTimer kt(s, TP_K_GEMM_OUT, st);
            TRY(launch_proj(s, ws + lay.o, batch, s->hl * s->d, s->w_o, s->hidden, EPI_F32, own, s->hidden, st,
                            LenUpdate{kv->dlen, -1, kv->max_seq, kv->dlen + 1}));
        }
        TRY(reduce_own());
        if (!capturing) kv->len = L + 1;
        s->attn_seen = true;
    } else {
        const int mode = s->o.act == TP_ACT_SWIGLU ? EPI_SWIGLU : EPI_GELU;
        if (use_gemv) {
            Epilogue epi{};
            epi.mode = mode;
            epi.out = ws + lay.act;
            epi.ldo = s->fl;
            {
                KTimer kt(s, TP_K_GEMV_UP, st);
                const void* g2 = s->o.rmsnorm && !prenorm ? s->g2 : nullptr;
                TRY(launch_gemv(s, x, batch, g2, s->w_up, s->nup, s->hidden, epi, ws + lay.n, ws + lay.scr, st, 2));
            }
            Epilogue e2{};
            e2.mode = EPI_F32;
            e2.out = own;
            e2.ldo = s->hidden;
            if (sum_epi) set_sum(e2);
            KTimer kt(s, TP_K_GEMV_DOWN, st);
            TRY(launch_gemv(s, ws + lay.act, batch, nullptr, s->w_down, s->hidden, s->fl, e2, ws + lay.n,
                            ws + lay.scr, st, 3));
        } else {
            const void* xin = x;
            if (s->o.rmsnorm && !prenorm) {
                KTimer kt(s, TP_K_RMSNORM, st);
                TRY(launch_norm(s, x, s->g2, ws + lay.n, batch, st));
                xin = ws + lay.n;
            }
            {
                KTimer kt(s, TP_K_GEMM_UP, st);
                TRY(launch_proj(s, xin, batch, s->hidden, s->w_up, s->nup, mode, ws + lay.act, s->fl, st));
            }
            KTimer kt(s, TP_K_GEMM_DOWN, st);
            TRY(launch_proj(s, ws + lay.act, batch, s->fl, s->w_down, s->hidden, EPI_F32, own, s->hidden, st));
        }
        TRY(reduce_own());
    }
    return TP_OK;
}

}  // namespace

extern "C" {

int tp_shard_forward_decode(tp_shard* s, int stage, const void* x, int batch, tp_kv* kv, float* partial,
                            void* stream) {
    return decode_stage(s, stage, x, batch, kv, partial, stream, false);
}

int tp_shard_forward_decode_noalloc(tp_shard* s, int stage, const void* x, int batch, tp_kv* kv, float* partial,
                                    void* stream) {
    return decode_stage(s, stage, x, batch, kv, partial, stream, true);
}

int tp_shard_forward_decode_reduce(tp_shard* s, int stage, const void* x, int batch, tp_kv* kv,
                                   const float* const* partials, const void* residual, void* out, void* stream) {
    if (!s || !x || !partials || !out || batch <= 0) return TP_E_ARG;
    for (int r = 0; r < s->t; ++r)
        if (r != s->rank && (!partials[r] || !aligned16(partials[r]))) return TP_E_ARG;
    if (!aligned16(out) || (residual && !aligned16(residual))) return TP_E_ARG;
    // the projections read all of x while the epilogue writes out
    const uintptr_t xb = (uintptr_t)x, ob = (uintptr_t)out;
    const uintptr_t xe = xb + (size_t)batch * s->hidden * s->esz, oe = ob + (size_t)batch * s->hidden * s->esz;
    if (xb < oe && ob < xe) return TP_E_ARG;
    const FuseSum f{partials, residual, out};
    return decode_stage(s, stage, x, batch, kv, nullptr, stream, false, &f);
}

int tp_partial_reduce(const float* const* partials, int t, const void* residual, void* out, long long n,
                      int out_dtype, void* stream) {
    if (!partials || t < 1 || t > 64 || n < 0) return TP_E_ARG;
    if (out_dtype != TP_BF16 && out_dtype != TP_F32) return TP_E_ARG;
    if (n == 0) return TP_OK;  // nothing to sum (empty tensors may have NULL addresses)
    if (!out) return TP_E_ARG;
    for (int r = 0; r < t; ++r)
        if (!partials[r] || !aligned16(partials[r])) return TP_E_ARG;
    if (!aligned16(out) || (residual && !aligned16(residual))) return TP_E_ARG;
    partial_reduce(partials, t, residual, out, n, out_dtype == TP_BF16, (hipStream_t)stream);
    LAUNCH_CHECK("partial_reduce");
    return TP_OK;
}

int tp_shard_reduce_norm(tp_shard* s, int which, const float* const* partials, int t, const void* residual, void* out,
                         void* norm_out, long long rows, void* stream) {
    if (!s || (which != 1 && which != 2) || !partials || t < 1 || t > 64 || rows < 0) return TP_E_ARG;
    if (rows == 0) return TP_OK;
    if (!out || !norm_out || !aligned16(out) || !aligned16(norm_out) || (residual && !aligned16(residual)) ||
        rows > INT32_MAX)
        return TP_E_ARG;
    for (int r = 0; r < t; ++r)
        if (!partials[r] || !aligned16(partials[r])) return TP_E_ARG;
    if (!s->loaded) return TP_E_STATE;
    hipStream_t st = (hipStream_t)stream;
    const bool bf = s->o.dtype == TP_BF16;
    const void* g = which == 1 ? s->g1 : s->g2;
    KTimer kt(s, TP_K_REDUCE_NORM, st);
    if (bf && s->o.rmsnorm &&
        reduce_norm_bf16(partials, t, (const bf16*)residual, (bf16*)out, (const bf16*)g, (bf16*)norm_out, (int)rows,
                         s->hidden, s->o.eps, st)) {
        LAUNCH_CHECK("reduce_norm");
        return TP_OK;
    }
    // other widths and the fp32 path: the reduce, then the norm (a copy without one)
    partial_reduce(partials, t, residual, out, rows * s->hidden, bf, st);
    LAUNCH_CHECK("partial_reduce");
    if (!s->o.rmsnorm) {
        HIP_TRY(hipMemcpyAsync(norm_out, out, (size_t)rows * s->hidden * s->esz, hipMemcpyDeviceToDevice, st));
        return TP_OK;
    }
    return launch_norm(s, out, g, norm_out, rows, st);
}

int tp_partial_reduce_scatter(const float* const* partials, int t, int rank, const void* residual_rows,
                              void* out_rows, long long rows, int cols, int out_dtype, void* stream) {
    if (!partials || t < 1 || t > 64 || rows < 0 || cols <= 0 || cols % 8) return TP_E_ARG;
    if (rank < 0 || rank >= t) return TP_E_RANK;
    if (rows % t) return TP_E_DIVIDE;
    if (out_dtype != TP_BF16 && out_dtype != TP_F32) return TP_E_ARG;
    const long long n = rows / t * (long long)cols;
    if (n == 0) return TP_OK;
    if (!out_rows || !aligned16(out_rows) || (residual_rows && !aligned16(residual_rows))) return TP_E_ARG;
    std::vector<const float*> mine(t);
    for (int r = 0; r < t; ++r) {
        if (!partials[r] || !aligned16(partials[r])) return TP_E_ARG;
        mine[r] = partials[r] + (long long)rank * n;   // this rank's rows of every partial
    }
    partial_reduce(mine.data(), t, residual_rows, out_rows, n, out_dtype == TP_BF16, (hipStream_t)stream);
    LAUNCH_CHECK("partial_reduce_scatter");
    return TP_OK;
}

int tp_all_gather(const void* const* pieces, int t, long long rows_per_rank, int cols, int dtype, void* out,
                  void* stream) {
    if (!pieces || t < 1 || t > 64 || rows_per_rank < 0 || cols <= 0) return TP_E_ARG;
    if (dtype != TP_BF16 && dtype != TP_F32) return TP_E_ARG;
    const long long row_bytes = (long long)cols * (dtype == TP_BF16 ? 2 : 4);
    if (row_bytes % 16) return TP_E_ARG;
    if (rows_per_rank == 0) return TP_OK;
    if (!out || !aligned16(out)) return TP_E_ARG;
    for (int r = 0; r < t; ++r)
        if (!pieces[r] || !aligned16(pieces[r])) return TP_E_ARG;
    all_gather(pieces, t, rows_per_rank * row_bytes, out, (hipStream_t)stream);
    LAUNCH_CHECK("all_gather");
    return TP_OK;
}

int tp_shard_norm(tp_shard* s, int which, const void* x, long long rows, void* out, void* stream) {
    if (!s || (which != 1 && which != 2) || rows < 0) return TP_E_ARG;
    if (rows == 0) return TP_OK;
    if (!x || !out || !aligned16(x) || !aligned16(out) || rows > INT32_MAX) return TP_E_ARG;
    if (!s->loaded) return TP_E_STATE;
    hipStream_t st = (hipStream_t)stream;
    if (!s->o.rmsnorm) {
        HIP_TRY(hipMemcpyAsync(out, x, (size_t)rows * s->hidden * s->esz, hipMemcpyDeviceToDevice, st));
        return TP_OK;
    }
    KTimer kt(s, TP_K_RMSNORM, st);
    return launch_norm(s, x, which == 1 ? s->g1 : s->g2, out, rows, st);
}

int tp_shard_debug_view(tp_shard* s, int which, void** ptr) {
    if (!s || !ptr || !s->dbg_base) return TP_E_ARG;
    switch (which) {
        case 0: *ptr = s->dbg_base + s->off_o; return TP_OK;
        case 1: *ptr = s->dbg_base + s->off_act; return TP_OK;
        case 2: *ptr = s->dbg_base + s->off_n; return TP_OK;
        default: return TP_E_ARG;
    }
}

int tp_shard_timing(tp_shard* s, int enable) {
    if (!s) return TP_E_ARG;
    if (enable) {
        if (s->ev.empty()) {
            s->ev.resize(kTimerEvents, nullptr);
            for (size_t i = 0; i < kTimerEvents; ++i) {
                hipError_t e = hipEventCreate(&s->ev[i]);
                if (e != hipSuccess) {
                    for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(s->ev[j]);
                    s->ev.clear();
                    return hip_fail(e, "hipEventCreate");
                }
            }
        }
        s->evused = 0;
        s->evkind.clear();
    }
    s->timing = enable != 0;
    s->tmask = enable == -1 ? 0xffffffffu : (unsigned)enable;
    return TP_OK;
}

int tp_shard_timing_read(tp_shard* s, int kernel, double* total_ms, long long* launches) {
    if (!s || !total_ms || !launches || kernel < 0 || kernel >= TP_K_COUNT) return TP_E_ARG;
    double tot = 0.0;
    long long n = 0;
    for (size_t i = 0; i < s->evkind.size(); ++i) {
        if (s->evkind[i] != kernel) continue;
        HIP_TRY(hipEventSynchronize(s->ev[2 * i + 1]));
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, s->ev[2 * i], s->ev[2 * i + 1]));
        tot += ms;
        ++n;
    }
    *total_ms = tot;
    *launches = n;
    return TP_OK;
}

int tp_tune_set_gemm_config(int cfg) {
    if (cfg < -1 || cfg >= gemm_config_count()) return TP_E_ARG;
    set_gemm_config(cfg);
    return TP_OK;
}

int tp_tune_gemm_plan(int M, int N, int K, int proj, int* parts, int cfg[2], int ncols[2]) {
    if (M <= 0 || N <= 0 || K <= 0 || !parts || !cfg || !ncols) return TP_E_ARG;
    if (proj != TP_PROJ_PARTIAL && proj != TP_PROJ_QKV && proj != TP_PROJ_SWIGLU && proj != TP_PROJ_GELU)
        return TP_E_ARG;
    gemm_plan_info(M, N, K, proj, parts, cfg, ncols);
    return TP_OK;
}

int tp_tune_set_gemm_split(int cfg0, int cfg1, int cols0) {
    if (cols0 < 0 || cols0 % 64) return TP_E_ARG;
    if (cols0 > 0 && (cfg0 < 0 || cfg0 >= gemm_config_count() || cfg1 < 0 || cfg1 >= gemm_config_count()))
        return TP_E_ARG;
    set_gemm_split(cfg0, cfg1, cols0);
    return TP_OK;
}

int tp_tune_set_decode_chunk(int ch) {
    if (ch != 0 && ch != 16 && ch != 32 && ch != 64) return TP_E_ARG;
    set_decode_chunk(ch);
    return TP_OK;
}

int tp_tune_set_decode_attn(int mode) {
    if (mode < 0 || mode > 3) return TP_E_ARG;
    set_decode_attn_mode(mode);
    return TP_OK;
}

int tp_tune_set_attn_groups(int kg) {
    if (kg < 0 || kg > 2) return TP_E_ARG;
    set_attn_groups(kg);
    return TP_OK;
}

int tp_tune_set_attn_kernel(int k) {
    if (k < 0 || k > 2) return TP_E_ARG;
    set_attn_kernel(k);
    return TP_OK;
}

void tp_shard_destroy(tp_shard* s) {
    if (!s) return;
    for (hipEvent_t e : s->ev)
        if (e) (void)hipEventDestroy(e);
    void* bufs[] = {s->w_qkv, s->w_o, s->w_up, s->w_down, s->g1, s->g2, s->ws, s->rcos, s->rsin, s->rrev,
                    s->q8[0], s->q8[1], s->q8[2], s->q8[3], s->s8[0], s->s8[1], s->s8[2], s->s8[3]};
    for (void* b : bufs)
        if (b) (void)hipFree(b);
    delete s;
}

void tp_kv_destroy(tp_kv* kv) {
    if (!kv) return;
    if (kv->k) (void)hipFree(kv->k);
    if (kv->v) (void)hipFree(kv->v);
    if (kv->dlen) (void)hipFree(kv->dlen);
    if (kv->table) (void)hipFree(kv->table);
    delete kv;
}

}  // extern "C"
