// C ABI of the tpmlp library: argument validation, the shard descriptor,
// workspace layout and kernel dispatch.  Every check runs before the first
// HIP call so argument errors never reach the GPU.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>

#include "../../include/tpmlp.h"
#include "launch.h"

using namespace tpmlp;

struct tpmlp_shards {
    int64_t D;
    int64_t F;
    int n;
    int dtype;
    void* packed;        // A^T (F x D), B^T (D x F), both `dtype`, then F fp32 column sums of A
    size_t packed_bytes;
    void* ws;            // bound workspace (caller-owned)
    size_t ws_bytes;
};

namespace {

// Largest size of a single dimension (rows or columns) accepted: keeps every
// grid dimension and every 32-bit in-tile offset of the kernels in range.
constexpr int64_t kMaxDim = (int64_t)1 << 21;
constexpr size_t kAlign = 256;

size_t elem_size(int dtype) { return dtype == TPMLP_F32 ? 4 : 2; }
bool valid_dtype(int dtype) { return dtype == TPMLP_F32 || dtype == TPMLP_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

tpmlp_status from_hip(hipError_t e) { return e == hipSuccess ? TPMLP_OK : TPMLP_ERR_HIP; }

tpmlp_status check_shard_args(int64_t D, int64_t F, int n, int dtype) {
    if (!valid_dtype(dtype)) return TPMLP_ERR_DTYPE;
    if (D <= 0 || F <= 0 || n <= 0 || D > kMaxDim || F > kMaxDim) return TPMLP_ERR_SHAPE;
    if (n > F) return TPMLP_ERR_SHAPE;
    if (F % n != 0) return TPMLP_ERR_INDIVISIBLE;
    return TPMLP_OK;
}

// Workspace layout for a forward over M rows with N_h intermediate columns:
//   [H: M x N_h, weights' dtype][mean: M fp32][rstd: M fp32]
//   [Z = residual + Y: M x D fp32, normalised last],
// each segment 256-byte aligned; the statistics exist only with the
// LayerNorm before, Z only with the LayerNorm after.  GEMM2 never splits
// its K loop (the shard sum stays in one accumulator), so it needs no
// scratch of its own.
struct WsLayout {
    size_t h_off, mean_off, rstd_off, z_off, total;
};

WsLayout ws_layout(const tpmlp_shards* s, int64_t M, int flags, int single_shard) {
    const int64_t nh = single_shard ? s->F / s->n : s->F;
    WsLayout L;
    L.h_off = 0;
    size_t off = round_up((size_t)M * (size_t)nh * elem_size(s->dtype));
    L.mean_off = L.rstd_off = off;
    if (flags & TPMLP_OPT_LAYERNORM) {
        L.mean_off = off;
        off += round_up((size_t)M * 4);
        L.rstd_off = off;
        off += round_up((size_t)M * 4);
    }
    L.z_off = off;
    if (flags & TPMLP_OPT_LAYERNORM_AFTER) off += round_up((size_t)M * (size_t)s->D * 4);
    L.total = off;
    return L;
}

// The GEMMs of the backward, C[m][n] = sum_k Aop[m][k] Bop[n][k], with every
// operand read where it lies (K-major where the contraction runs over its
// rows), so nothing is transposed:
//   S  = X A:     Aop = X (M x D),          Bop = A^T, packed (F x D)
//   dS = dY B^T:  Aop = dY (M x D),         Bop = B (F x D), the packed copy as given
//   dX = dS A^T:  Aop = dS (M x F),         Bop = A (D x F), the packed copy as given
//   dA = X^T dS:  Aop = X^T: X read K-major, Bop = dS^T: dS read K-major   (K = M)
//   dB = H^T dY:  Aop = H^T: H read K-major, Bop = dY^T: dY read K-major   (K = M)
enum { kBwdS, kBwdDS, kBwdDX, kBwdDA, kBwdDB };
struct BwdPtrs {
    const void *X, *dY, *at, *a, *b, *S;
    void *H, *dS, *dX, *dA, *dB;
};

GemmArgs bwd_args(const tpmlp_shards* s, int64_t M, int which, const BwdPtrs& q) {
    const int64_t D = s->D, F = s->F;
    GemmArgs g;
    g.allow_split = true;
    g.ab_dtype = s->dtype;
    g.c_dtype = s->dtype;
    g.epi = kEpiStore;
    switch (which) {
        case kBwdS:
            g.A = q.X; g.lda = D; g.B = q.at; g.ldb = D;
            g.M = M; g.N = F; g.K = D; g.C = const_cast<void*>(q.S); g.ldc = F;
            break;
        case kBwdDS:
            g.A = q.dY; g.lda = D; g.B = q.b; g.ldb = D;
            g.M = M; g.N = F; g.K = D; g.C = q.dS; g.ldc = F;
            g.epi = kEpiGeluGrad; g.aux = q.S; g.ldaux = F;
            g.gelu_out = q.H;
            break;
        case kBwdDX:
            g.A = q.dS; g.lda = F; g.B = q.a; g.ldb = F;
            g.M = M; g.N = D; g.K = F; g.C = q.dX; g.ldc = D;
            break;
        case kBwdDA:
            g.A = q.X; g.lda = D; g.a_kmajor = true; g.B = q.dS; g.ldb = F; g.b_kmajor = true;
            g.M = D; g.N = F; g.K = M; g.C = q.dA; g.ldc = F;
            break;
        default:  // kBwdDB
            g.A = q.H; g.lda = F; g.a_kmajor = true; g.B = q.dY; g.ldb = D; g.b_kmajor = true;
            g.M = F; g.N = D; g.K = M; g.C = q.dB; g.ldc = D;
            break;
    }
    return g;
}

// Backward workspace, each segment 256-byte aligned:
//   S = X A (M x F, unless the forward kept it);  H = GeLU(S) (M x F);
//   dS (M x F);  split-K scratch.
struct BwdLayout {
    size_t s, h, ds, split, split_bytes, total;
};

BwdLayout bwd_layout(const tpmlp_shards* s, int64_t M) {
    const size_t es = elem_size(s->dtype);
    const size_t F = (size_t)s->F, m = (size_t)M;
    BwdLayout L;
    size_t off = 0;
    L.s = off; off += round_up(m * F * es);
    L.h = off; off += round_up(m * F * es);
    L.ds = off; off += round_up(m * F * es);
    size_t sb = 0;
    if (M > 0) {
        // the split plan depends on shapes, leading dimensions and layouts, not
        // on addresses: aligned stand-ins
        char* const fake = reinterpret_cast<char*>((uintptr_t)256);
        const BwdPtrs q{fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake};
        for (int which = kBwdS; which <= kBwdDB; ++which) {
            const size_t c = gemm_split_bytes(bwd_args(s, M, which, q));
            sb = c > sb ? c : sb;
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

const char* tpmlp_status_string(int status) {
    switch (status) {
        case TPMLP_OK: return "TPMLP_OK";
        case TPMLP_ERR_NULL: return "TPMLP_ERR_NULL: a required pointer is NULL";
        case TPMLP_ERR_SHAPE: return "TPMLP_ERR_SHAPE: a size is out of range";
        case TPMLP_ERR_INDIVISIBLE: return "TPMLP_ERR_INDIVISIBLE: F is not divisible by n";
        case TPMLP_ERR_DTYPE: return "TPMLP_ERR_DTYPE: unsupported dtype";
        case TPMLP_ERR_WORKSPACE: return "TPMLP_ERR_WORKSPACE: buffer missing or too small";
        case TPMLP_ERR_ALIGN: return "TPMLP_ERR_ALIGN: device pointer not 16-byte aligned";
        case TPMLP_ERR_HIP: return "TPMLP_ERR_HIP: HIP runtime error";
        default: return "TPMLP_ERR_UNKNOWN";
    }
}

const char* tpmlp_version(void) { return "tpmlp 0.1 gfx950"; }

tpmlp_status tpmlp_gelu(const void* x, void* y, int64_t count, int dtype, void* stream) {
    if (!valid_dtype(dtype)) return TPMLP_ERR_DTYPE;
    if (count < 0) return TPMLP_ERR_SHAPE;
    if (count == 0) return TPMLP_OK;
    if (!x || !y) return TPMLP_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return TPMLP_ERR_ALIGN;
    return from_hip(launch_gelu(x, y, count, dtype, static_cast<hipStream_t>(stream)));
}

// Packed weight buffer, each segment 256-byte aligned:
//   A^T (F x D) and B^T (D x F): the forward's K-contiguous operands, pair i
//     in rows (columns) iF/n..(i+1)F/n-1;
//   F fp32 column sums of A (the LayerNorm epilogue);
//   A (D x F) and B (F x D) as given: K-contiguous operands of the backward's
//     dX = dS A^T and dS = dY B^T GEMMs.
struct PackLayout {
    size_t at, bt, csum, a, b, total;
};
PackLayout pack_layout(int64_t D, int64_t F, int dtype) {
    const size_t w = round_up((size_t)D * (size_t)F * elem_size(dtype));
    PackLayout L;
    L.at = 0;
    L.bt = w;
    L.csum = 2 * w;
    L.a = L.csum + round_up((size_t)F * 4);
    L.b = L.a + w;
    L.total = L.b + w;
    return L;
}

size_t tpmlp_shard_bytes(int64_t D, int64_t F, int n, int dtype) {
    if (check_shard_args(D, F, n, dtype) != TPMLP_OK) return 0;
    return pack_layout(D, F, dtype).total;
}

tpmlp_status tpmlp_shard(const void* A, const void* B, int64_t D, int64_t F, int n, int dtype,
                         void* packed, size_t packed_bytes, tpmlp_shards** out, void* stream) {
    if (out) *out = nullptr;
    if (!A || !B || !packed || !out) return TPMLP_ERR_NULL;
    tpmlp_status st = check_shard_args(D, F, n, dtype);
    if (st != TPMLP_OK) return st;
    if (packed_bytes < tpmlp_shard_bytes(D, F, n, dtype)) return TPMLP_ERR_WORKSPACE;
    if (!aligned16(A) || !aligned16(B) || !aligned16(packed)) return TPMLP_ERR_ALIGN;

    tpmlp_shards* s = new (std::nothrow) tpmlp_shards;
    if (!s) return TPMLP_ERR_HIP;
    s->D = D;
    s->F = F;
    s->n = n;
    s->dtype = dtype;
    s->packed = packed;
    s->packed_bytes = packed_bytes;
    s->ws = nullptr;
    s->ws_bytes = 0;

    // Pair i of "The split" is rows iF/n..(i+1)F/n-1 of A^T and columns
    // iF/n..(i+1)F/n-1 of B^T: one transpose of each matrix packs all pairs,
    // each K-contiguous for the matrix cores.  A and B are also kept as
    // given, the K-contiguous operands of the backward's dX and dS GEMMs.
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int eb = (int)elem_size(dtype);
    const PackLayout P = pack_layout(D, F, dtype);
    char* base = static_cast<char*>(packed);
    char* at = base + P.at;
    char* bt = base + P.bt;
    float* csum = reinterpret_cast<float*>(base + P.csum);
    const size_t bytes = (size_t)D * (size_t)F * eb;
    hipError_t e = launch_transpose(A, F, at, D, D, F, eb, hs);        // A (D x F) -> A^T (F x D)
    if (e == hipSuccess) e = launch_transpose(B, D, bt, F, F, D, eb, hs);  // B (F x D) -> B^T (D x F)
    if (e == hipSuccess) e = launch_rowsum(at, F, D, dtype, csum, hs);  // column sums of A
    if (e == hipSuccess) e = hipMemcpyAsync(base + P.a, A, bytes, hipMemcpyDeviceToDevice, hs);
    if (e == hipSuccess) e = hipMemcpyAsync(base + P.b, B, bytes, hipMemcpyDeviceToDevice, hs);
    if (e != hipSuccess) {
        delete s;
        return TPMLP_ERR_HIP;
    }
    *out = s;
    return TPMLP_OK;
}

int tpmlp_shard_count(const tpmlp_shards* s) { return s ? s->n : 0; }

tpmlp_status tpmlp_shard_info(const tpmlp_shards* s, int64_t* D, int64_t* F, int* n, int* dtype) {
    if (!s) return TPMLP_ERR_NULL;
    if (D) *D = s->D;
    if (F) *F = s->F;
    if (n) *n = s->n;
    if (dtype) *dtype = s->dtype;
    return TPMLP_OK;
}

tpmlp_status tpmlp_shard_unpack(const tpmlp_shards* s, int i, void* A_i, void* B_i, void* stream) {
    if (!s) return TPMLP_ERR_NULL;
    if (i < 0 || i >= s->n) return TPMLP_ERR_SHAPE;
    if ((A_i && !aligned16(A_i)) || (B_i && !aligned16(B_i))) return TPMLP_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int eb = (int)elem_size(s->dtype);
    const int64_t w = s->F / s->n;
    const char* at = static_cast<const char*>(s->packed);
    const char* bt = at + round_up((size_t)s->D * (size_t)s->F * eb);
    hipError_t e = hipSuccess;
    if (A_i)  // rows i*w.. of A^T (w x D) -> A_i (D x w)
        e = launch_transpose(at + (size_t)i * w * s->D * eb, s->D, A_i, w, w, s->D, eb, hs);
    if (e == hipSuccess && B_i)  // columns i*w.. of B^T (D x w, pitch F) -> B_i (w x D)
        e = launch_transpose(bt + (size_t)i * w * eb, s->F, B_i, s->D, s->D, w, eb, hs);
    return from_hip(e);
}

void tpmlp_shards_destroy(tpmlp_shards* s) { delete s; }

size_t tpmlp_forward_workspace_bytes(const tpmlp_shards* s, int64_t M, int flags, int single_shard) {
    if (!s || M < 0 || M > kMaxDim) return 0;
    return ws_layout(s, M, flags, single_shard).total;
}

tpmlp_status tpmlp_set_workspace(tpmlp_shards* s, void* ws, size_t bytes) {
    if (!s) return TPMLP_ERR_NULL;
    if (ws && !aligned16(ws)) return TPMLP_ERR_ALIGN;
    s->ws = ws;
    s->ws_bytes = ws ? bytes : 0;
    return TPMLP_OK;
}

void tpmlp_opts_init(tpmlp_opts* o) {
    if (!o) return;
    std::memset(o, 0, sizeof(*o));
    o->ln_eps = 1e-5f;
    o->y_dtype = -1;
    o->shard_index = -1;
}

tpmlp_status tpmlp_forward_ex(const void* X, int64_t M, const tpmlp_shards* s, void* Y,
                              const tpmlp_opts* opts, void* stream) {
    tpmlp_opts o;
    tpmlp_opts_init(&o);
    if (opts) o = *opts;
    if (!s) return TPMLP_ERR_NULL;
    if (M < 0 || M > kMaxDim) return TPMLP_ERR_SHAPE;
    if (o.flags & ~(TPMLP_OPT_LAYERNORM | TPMLP_OPT_LAYERNORM_AFTER)) return TPMLP_ERR_SHAPE;
    const bool ln_after = (o.flags & TPMLP_OPT_LAYERNORM_AFTER) != 0;
    if (ln_after && ((o.flags & TPMLP_OPT_LAYERNORM) || o.shard_index >= 0)) return TPMLP_ERR_SHAPE;
    const int y_dtype = o.y_dtype < 0 ? s->dtype : o.y_dtype;
    if (!valid_dtype(y_dtype)) return TPMLP_ERR_DTYPE;
    if (s->dtype == TPMLP_F32 && y_dtype != TPMLP_F32) return TPMLP_ERR_DTYPE;
    if (o.shard_index < -1 || o.shard_index >= s->n) return TPMLP_ERR_SHAPE;
    const bool ln = (o.flags & TPMLP_OPT_LAYERNORM) != 0;
    const float eps = o.ln_eps > 0.f ? o.ln_eps : 1e-5f;
    if (!(eps < 1e30f)) return TPMLP_ERR_SHAPE;
    if (M == 0) return TPMLP_OK;
    if (!X || !Y) return TPMLP_ERR_NULL;
    if (!aligned16(X) || !aligned16(Y) || (o.residual && !aligned16(o.residual)) ||
        (o.save_preact && !aligned16(o.save_preact)) || (o.save_act && !aligned16(o.save_act)))
        return TPMLP_ERR_ALIGN;

    const bool single = o.shard_index >= 0;
    void* ws = o.workspace ? o.workspace : s->ws;
    const size_t ws_bytes = o.workspace ? o.workspace_bytes : s->ws_bytes;
    const WsLayout L = ws_layout(s, M, o.flags, single);
    if (!ws || ws_bytes < L.total) return TPMLP_ERR_WORKSPACE;
    if (!aligned16(ws)) return TPMLP_ERR_ALIGN;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (o.events)
        for (int k = 0; k < 4; ++k) ev[k] = static_cast<hipEvent_t>(o.events[k]);
    auto mark = [&](int k) -> hipError_t { return ev[k] ? hipEventRecord(ev[k], hs) : hipSuccess; };

    const int64_t D = s->D, F = s->F, w = F / s->n;
    const int64_t n_lo = single ? o.shard_index * w : 0;
    const int64_t nh = single ? w : F;
    const int eb = (int)elem_size(s->dtype);
    const char* at = static_cast<const char*>(s->packed);
    const char* bt = at + round_up((size_t)D * (size_t)F * eb);
    const float* csum = reinterpret_cast<const float*>(bt + round_up((size_t)D * (size_t)F * eb));
    char* wsb = static_cast<char*>(ws);
    void* H = o.save_act ? o.save_act : wsb + L.h_off;  // the caller keeps H, or the workspace holds it
    float* mean = ln ? reinterpret_cast<float*>(wsb + L.mean_off) : nullptr;
    float* rstd = ln ? reinterpret_cast<float*>(wsb + L.rstd_off) : nullptr;

    hipError_t e = mark(0);
    if (e == hipSuccess && ln) e = launch_ln_stats(X, M, D, s->dtype, eps, mean, rstd, hs);
    if (e == hipSuccess) e = mark(1);

    // GEMM1, column-parallel: H[:, 0:nh] = GeLU(LN?(X) . A^T[n_lo:n_lo+nh, :]^T)
    if (e == hipSuccess) {
        GemmArgs g1;
        g1.A = X; g1.lda = D;
        g1.B = at + (size_t)n_lo * D * eb; g1.ldb = D;
        g1.M = M; g1.N = nh; g1.K = D;
        g1.C = H; g1.ldc = nh; g1.c_dtype = s->dtype;
        g1.ln_mean = mean; g1.ln_rstd = rstd;
        g1.ln_csum = ln ? csum + n_lo : nullptr;
        g1.epi = kEpiGelu;
        g1.ab_dtype = s->dtype;
        g1.preact_out = o.save_preact;
        e = launch_gemm(g1, hs);
    }
    if (e == hipSuccess) e = mark(2);

    // GEMM2, row-parallel with the shard sum in the accumulator:
    // Y = H[:, 0:nh] . B^T[:, n_lo:n_lo+nh]^T (+ residual), or, with the
    // LayerNorm after, Z = residual + Y kept in fp32 for the Norm.  Its K loop
    // is never split (allow_split stays false): every shard's partial goes
    // into the same fp32 accumulator and only the sum is stored.
    float* Z = ln_after ? reinterpret_cast<float*>(wsb + L.z_off) : nullptr;
    if (e == hipSuccess) {
        GemmArgs g2;
        g2.A = H; g2.lda = nh;
        g2.B = bt + (size_t)n_lo * eb; g2.ldb = F;
        g2.M = M; g2.N = D; g2.K = nh;
        if (ln_after) {
            g2.C = Z; g2.ldc = D; g2.c_dtype = TPMLP_F32;
        } else {
            g2.C = Y; g2.ldc = D; g2.c_dtype = y_dtype;
        }
        g2.R = o.residual; g2.ldr = D;
        g2.epi = kEpiStore;
        g2.ab_dtype = s->dtype;
        e = launch_gemm(g2, hs);
    }
    // out = LayerNorm(Z), one rounding to Y's dtype
    if (e == hipSuccess && ln_after) e = launch_ln_apply(Z, M, D, eps, Y, y_dtype, hs);
    if (e == hipSuccess) e = mark(3);
    return from_hip(e);
}

tpmlp_status tpmlp_forward(const void* X, int64_t M, const tpmlp_shards* s, void* Y, void* stream) {
    return tpmlp_forward_ex(X, M, s, Y, nullptr, stream);
}

size_t tpmlp_backward_workspace_bytes(const tpmlp_shards* s, int64_t M) {
    if (!s || M < 0 || M > kMaxDim) return 0;
    return bwd_layout(s, M).total;
}

tpmlp_status tpmlp_backward(const void* X, const void* dY, int64_t M, const tpmlp_shards* s, const void* preact,
                            const void* act, void* dX, void* dA, void* dB, void* workspace, size_t workspace_bytes,
                            void* stream) {
    if (!s) return TPMLP_ERR_NULL;
    if (M < 0 || M > kMaxDim) return TPMLP_ERR_SHAPE;
    if (!dA || !dB || (M > 0 && (!X || !dY || !dX))) return TPMLP_ERR_NULL;
    if (!aligned16(dA) || !aligned16(dB) || (M > 0 && (!aligned16(X) || !aligned16(dY) || !aligned16(dX))) ||
        (preact && !aligned16(preact)) || (act && !aligned16(act)))
        return TPMLP_ERR_ALIGN;
    const BwdLayout L = bwd_layout(s, M);  // 0 bytes for M = 0: the workspace may then be NULL
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return TPMLP_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return TPMLP_ERR_ALIGN;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int dt = s->dtype;
    const int64_t D = s->D, F = s->F;
    const PackLayout P = pack_layout(D, F, dt);
    const char* pk = static_cast<const char*>(s->packed);
    char* w = static_cast<char*>(workspace);

    if (M == 0) {
        // an empty batch contributes zero weight gradients: K = 0 GEMMs
        // read no operand and write zeros
        GemmArgs za;
        za.ab_dtype = dt; za.c_dtype = dt; za.epi = kEpiStore;
        za.M = D; za.N = F; za.K = 0;
        za.A = dA; za.B = dA; za.C = dA; za.ldc = F;
        GemmArgs zb = za;
        zb.M = F; zb.N = D;
        zb.A = dB; zb.B = dB; zb.C = dB; zb.ldc = D;
        hipError_t e = launch_gemm_generic(za, hs);
        if (e == hipSuccess) e = launch_gemm_generic(zb, hs);
        return from_hip(e);
    }

    BwdPtrs q;
    q.X = X; q.dY = dY;
    q.at = pk + P.at;   // A^T (F x D)
    q.a = pk + P.a;     // A (D x F)
    q.b = pk + P.b;     // B (F x D)
    q.S = preact ? preact : static_cast<const void*>(w + L.s);
    q.H = act ? const_cast<void*>(act) : static_cast<void*>(w + L.h);
    q.dS = w + L.ds;
    q.dX = dX; q.dA = dA; q.dB = dB;
    auto gemm = [&](int which) {
        GemmArgs g = bwd_args(s, M, which, q);
        if (which == kBwdDS && act) g.gelu_out = nullptr;  // H is the forward's
        g.split_ws = w + L.split;
        g.split_ws_bytes = L.split_bytes;
        return launch_gemm(g, hs);
    };

    hipError_t e = hipSuccess;
    // S = X A for all shards at once, unless the forward kept it
    if (!preact) e = gemm(kBwdS);
    // dS = (dY B^T) * GeLU'(S), the gradient at every shard's GeLU input; the
    // epilogue that reads S also writes H = GeLU(S) for dB, unless the
    // forward kept H
    if (e == hipSuccess) e = gemm(kBwdDS);
    // dX = sum_i dS_i A_i^T: the K loop over F sums the shards in registers
    if (e == hipSuccess) e = gemm(kBwdDX);
    // dA = X^T dS and dB = H^T dY contract over the batch axis M
    if (e == hipSuccess) e = gemm(kBwdDA);
    if (e == hipSuccess) e = gemm(kBwdDB);
    return from_hip(e);
}

}  // extern "C"
