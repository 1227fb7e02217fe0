// C ABI of the attention half: the packed-weight descriptor, workspace
// layout, argument validation and kernel dispatch.  Every check runs before
// the first HIP call.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>

#include "../../include/tpmlp.h"
#include "launch.h"

using namespace tpmlp;

struct tpmlp_attn {
    int64_t h;
    int heads;
    int p;
    bool has_wo;
    void* packed;  // Wqkv^T (3h x h) bf16 | 3h fp32 column sums of [Wq|Wk|Wv] | Wo^T (h x h) bf16
};

namespace {

constexpr int64_t kMaxTokens = (int64_t)1 << 21;
constexpr int64_t kMaxHidden = (int64_t)1 << 16;
constexpr int64_t kMaxBatch = 65535;  // one grid dimension of the attention kernel per sequence
constexpr int kHeadDim = 64;
constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }
tpmlp_status from_hip(hipError_t e) { return e == hipSuccess ? TPMLP_OK : TPMLP_ERR_HIP; }

tpmlp_status check_pack_args(int64_t h, int heads, int p, int dtype) {
    if (dtype != TPMLP_BF16) return TPMLP_ERR_DTYPE;
    if (heads <= 0 || p <= 0 || h <= 0 || h > kMaxHidden) return TPMLP_ERR_SHAPE;
    if (h != (int64_t)heads * kHeadDim) return TPMLP_ERR_SHAPE;
    if (heads % p != 0) return TPMLP_ERR_INDIVISIBLE;
    return TPMLP_OK;
}

struct PackLayout {
    size_t qkv, csum, wo, total;
};

PackLayout pack_layout(int64_t h, bool with_wo) {
    PackLayout L;
    size_t off = 0;
    L.qkv = off; off += round_up((size_t)(3 * h) * (size_t)h * 2);
    L.csum = off; off += round_up((size_t)(3 * h) * 4);
    L.wo = off; if (with_wo) off += round_up((size_t)h * (size_t)h * 2);
    L.total = off;
    return L;
}

// A projection GEMM's shape (stand-in aligned pointers), for sizing the
// split-K scratch.
GemmArgs proj_shape(int64_t M, int64_t N, int64_t K) {
    GemmArgs g;
    char* const fake = reinterpret_cast<char*>((uintptr_t)256);
    g.A = fake; g.lda = K;
    g.B = fake; g.ldb = K;
    g.M = M; g.N = N; g.K = K;
    g.C = fake; g.ldc = N; g.c_dtype = kBF16;
    g.epi = kEpiStore;
    g.ab_dtype = kBF16;
    g.allow_split = true;
    return g;
}

// Workspace: [mean: M fp32][rstd: M fp32][QKV: M x 3h]
// [O: M x h, with W^O][split-K scratch], 256-byte aligned segments.
struct WsLayout {
    size_t mean, rstd, qkv, o, split, split_bytes, total;
};

WsLayout ws_layout(const tpmlp_attn* a, int64_t M) {
    const size_t h = (size_t)a->h, m = (size_t)M;
    WsLayout L;
    size_t off = 0;
    L.mean = off; off += round_up(m * 4);
    L.rstd = off; off += round_up(m * 4);
    L.qkv = off; off += round_up(m * 3 * h * 2);
    L.o = off; if (a->has_wo) off += round_up(m * h * 2);
    size_t sb = 0;
    if (M > 0) {
        sb = gemm_split_bytes(proj_shape(M, 3 * a->h, a->h));
        if (a->has_wo) {
            const size_t so = gemm_split_bytes(proj_shape(M, a->h, a->h));
            sb = so > sb ? so : sb;
        }
    }
    L.split = off;
    L.split_bytes = sb;
    off += round_up(sb);
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

size_t tpmlp_attn_pack_bytes(int64_t hidden, int heads, int p, int dtype, int with_out_proj) {
    if (check_pack_args(hidden, heads, p, dtype) != TPMLP_OK) return 0;
    return pack_layout(hidden, with_out_proj != 0).total;
}

tpmlp_status tpmlp_attn_pack(const void* Wq, const void* Wk, const void* Wv, const void* Wo, int64_t hidden,
                             int heads, int p, int dtype, void* packed, size_t packed_bytes, tpmlp_attn** out,
                             void* stream) {
    if (!out) return TPMLP_ERR_NULL;
    *out = nullptr;
    const tpmlp_status st = check_pack_args(hidden, heads, p, dtype);
    if (st != TPMLP_OK) return st;
    if (!Wq || !Wk || !Wv || !packed) return TPMLP_ERR_NULL;
    const PackLayout L = pack_layout(hidden, Wo != nullptr);
    if (packed_bytes < L.total) return TPMLP_ERR_WORKSPACE;
    if (!aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) || (Wo && !aligned16(Wo)) || !aligned16(packed))
        return TPMLP_ERR_ALIGN;
    tpmlp_attn* a = new (std::nothrow) tpmlp_attn;
    if (!a) return TPMLP_ERR_HIP;
    a->h = hidden;
    a->heads = heads;
    a->p = p;
    a->has_wo = Wo != nullptr;
    a->packed = packed;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int64_t h = hidden;
    char* base = static_cast<char*>(packed);
    char* wt = base + L.qkv;
    // [Wq | Wk | Wv]^T: row n of block b is column n of W_b (K-contiguous for the GEMM)
    const void* W[3] = {Wq, Wk, Wv};
    hipError_t e = hipSuccess;
    for (int b = 0; b < 3 && e == hipSuccess; ++b)
        e = launch_transpose(W[b], h, wt + (size_t)b * h * h * 2, h, h, h, 2, hs);
    // column sums of [Wq | Wk | Wv] (row sums of the transpose): the
    // LayerNorm correction of the projection's epilogue
    if (e == hipSuccess) e = launch_rowsum(wt, 3 * h, h, kBF16, reinterpret_cast<float*>(base + L.csum), hs);
    if (e == hipSuccess && Wo) e = launch_transpose(Wo, h, base + L.wo, h, h, h, 2, hs);
    if (e != hipSuccess) {
        delete a;
        return TPMLP_ERR_HIP;
    }
    *out = a;
    return TPMLP_OK;
}

void tpmlp_attn_destroy(tpmlp_attn* a) { delete a; }

size_t tpmlp_attn_workspace_bytes(const tpmlp_attn* a, int64_t batch, int64_t seq) {
    // the sizes tpmlp_attention accepts, and no others
    if (!a || batch < 0 || seq < 0 || (seq > 0 && batch > kMaxTokens / seq) || seq > kMaxTokens) return 0;
    if (batch > kMaxBatch || (seq > 0 && !attention_fits(seq, a->heads))) return 0;
    return ws_layout(a, batch * seq).total;
}

tpmlp_status tpmlp_attention(const void* x, int64_t batch, int64_t seq, const tpmlp_attn* a, void* out, int flags,
                             float ln_eps, void* workspace, size_t workspace_bytes, void* const* events,
                             void* stream) {
    if (!a) return TPMLP_ERR_NULL;
    if (batch < 0 || seq < 0 || seq > kMaxTokens || (seq > 0 && batch > kMaxTokens / seq)) return TPMLP_ERR_SHAPE;
    if (batch > kMaxBatch) return TPMLP_ERR_SHAPE;
    if (seq > 0 && !attention_fits(seq, a->heads)) return TPMLP_ERR_SHAPE;
    if (flags & ~(TPMLP_ATTN_LAYERNORM | TPMLP_ATTN_RESIDUAL)) return TPMLP_ERR_SHAPE;
    const float eps = ln_eps > 0.f ? ln_eps : 1e-5f;
    if (!(eps < 1e30f)) return TPMLP_ERR_SHAPE;
    const int64_t M = batch * seq;
    if (M == 0) return TPMLP_OK;
    if (!x || !out) return TPMLP_ERR_NULL;
    if (!aligned16(x) || !aligned16(out)) return TPMLP_ERR_ALIGN;
    const WsLayout L = ws_layout(a, M);
    if (!workspace || workspace_bytes < L.total) return TPMLP_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TPMLP_ERR_ALIGN;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int64_t h = a->h;
    const bool ln = (flags & TPMLP_ATTN_LAYERNORM) != 0;
    const bool resid = (flags & TPMLP_ATTN_RESIDUAL) != 0;
    const char* pk = static_cast<const char*>(a->packed);
    const PackLayout P = pack_layout(h, a->has_wo);
    char* w = static_cast<char*>(workspace);
    float* mean = reinterpret_cast<float*>(w + L.mean);
    float* rstd = reinterpret_cast<float*>(w + L.rstd);
    char* qkv = w + L.qkv;

    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (events)
        for (int k = 0; k < 4; ++k) ev[k] = static_cast<hipEvent_t>(events[k]);
    auto mark = [&](int k) -> hipError_t { return ev[k] ? hipEventRecord(ev[k], hs) : hipSuccess; };

    hipError_t e = mark(0);
    if (e == hipSuccess && ln) e = launch_ln_stats(x, M, h, kBF16, eps, mean, rstd, hs);
    if (e == hipSuccess) e = mark(1);
    // [Q | K | V] = LayerNorm?(x) [Wq | Wk | Wv]: one GEMM for every head of every rank
    if (e == hipSuccess) {
        GemmArgs g = proj_shape(M, 3 * h, h);
        g.A = x;
        g.B = pk + P.qkv;
        g.C = qkv;
        g.ln_mean = ln ? mean : nullptr;
        g.ln_rstd = ln ? rstd : nullptr;
        g.ln_csum = ln ? reinterpret_cast<const float*>(pk + P.csum) : nullptr;
        g.split_ws = w + L.split;
        g.split_ws_bytes = L.split_bytes;
        e = launch_gemm(g, hs);
    }
    if (e == hipSuccess) e = mark(2);
    if (e == hipSuccess) {
        if (!a->has_wo) {
            // the heads' outputs side by side (all_gather + cat), plus x
            e = launch_attention(qkv, 3 * h, resid ? x : nullptr, h, out, h, batch, seq, a->heads, hs);
        } else {
            char* o = w + L.o;
            e = launch_attention(qkv, 3 * h, nullptr, h, o, h, batch, seq, a->heads, hs);
            // row-parallel output projection: the K loop over h sums every rank's part
            if (e == hipSuccess) {
                GemmArgs g = proj_shape(M, h, h);
                g.A = o;
                g.B = pk + P.wo;
                g.C = out;
                g.R = resid ? x : nullptr;
                g.ldr = h;
                g.split_ws = w + L.split;
                g.split_ws_bytes = L.split_bytes;
                e = launch_gemm(g, hs);
            }
        }
    }
    if (e == hipSuccess) e = mark(3);
    return from_hip(e);
}

}  // extern "C"
