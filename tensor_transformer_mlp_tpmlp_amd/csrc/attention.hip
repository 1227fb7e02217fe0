// Local attention of the head-sharded attention half of the block:
// O = softmax(Q K^T / sqrt(d)) V for every head of every sequence
// ("Tensor Parallelism in Megatron", section 4, the local-attention
// equation), d = 64, no mask, on v_mfma_f32_16x16x32_bf16.
//
// Layouts.  QKV is the projection output, one row per token (batch*seq rows,
// sequence b in rows b*seq ..), with Q in columns 0..h-1, K in h..2h-1, V in
// 2h..3h-1 and head j in columns j*64 .. j*64+63 of each (ld = 3h).  V^T is
// the V block transposed (h rows, one per head column; batch*seq columns),
// so the P V product reads 8 consecutive keys per lane.  O is written in the
// concatenated-heads layout (token row, column j*64 + dd), the all_gather-
// and-cat of "LLM Lab Notes 06", section 2, marker 3, optionally plus the
// residual x (marker 4).
//
// One block of 256 threads (4 waves) owns 64 query rows of one (sequence,
// head); wave w owns rows 16w .. 16w+15.  Keys and values stream through LDS
// in tiles of 64 keys, double-buffered: the next tile's global loads are
// issued before the current tile's products and written to the other buffer
// after them.  Per tile a wave forms S (16 x 64) in 8 MFMAs, updates the
// running row maximum and sum (online softmax in the log2 domain, fp32),
// rounds P to bf16 and accumulates O (16 x 64) in 8 MFMAs.
//
// MFMA operand order: the first operand's rows index the result's rows as
// seen by the lanes, so S = mfma(K frag, Q frag) leaves lane l with query
// row l & 15 and keys 4 (l >> 4) + r of a 16-key block, and
// O = mfma(V^T frag, P frag) leaves it with query row l & 15 and columns
// 4 (l >> 4) + r.  A lane's 8 k-slots of P are therefore keys {4g .. 4g+3}
// of the even 16-key block and {16 + 4g .. 16 + 4g + 3} of the odd one
// (g = l >> 4); the V^T fragment is read with the same key order, which is
// all the contraction needs.
#include "device_common.h"
#include "launch.h"

namespace tpmlp {

namespace {

typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kDH = 64;      // head width
constexpr int kQT = 64;      // query rows per block
constexpr int kKT = 64;      // keys per tile
constexpr int kRowB = 128;   // bytes per LDS row (64 bf16)

// 16-byte chunk swizzle of a 128-byte LDS row: the 16 lanes of a read pass
// hit 16 distinct chunk slots for the 16-row fragment pattern.
__device__ __forceinline__ int swz(int row) { return ((row & 8) >> 2) | ((row & 2) << 1); }

struct AttnParams {
    const bf16* qkv;   // batch*seq x 3h
    int64_t ldq;       // 3h
    const bf16* vt;    // h x batch*seq
    int64_t ldv;       // batch*seq
    const bf16* x;     // residual, batch*seq x h (nullptr: none)
    int64_t ldx;
    bf16* out;         // batch*seq x h
    int64_t ldo;
    int64_t h;
    int seq;
    float scale_log2;  // log2(e) / sqrt(d)
};

__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kKT * kRowB];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[2][kDH * kRowB];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int seq = p.seq;
    const int q0 = blockIdx.x * kQT;
    const int head = blockIdx.y;
    const int64_t tok0 = (int64_t)blockIdx.z * seq;  // first token row of this sequence
    const bool vt_vec = (seq & 7) == 0;              // 16-byte V^T chunks stay in one sequence

    // Q fragments of this lane's row (zeros past the sequence end)
    bf16x8 qf[2];
    {
        const int q = q0 + 16 * w + li;
        const bf16* qrow = p.qkv + (tok0 + q) * p.ldq + head * kDH;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (q < seq) raw = *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * g);
            __builtin_memcpy(&qf[c], &raw, 16);
        }
    }

    // tile loader: thread t moves K chunks (row t/8, t/8+32; chunk t%8) and
    // V^T chunks (head column t/8, t/8+32; keys 8 (t%8) ..), 16 bytes each
    const int lrow = t >> 3, lch = t & 7;
    u32x4 kreg[2], vreg[2];
    auto load_tile = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = lrow + 32 * i;
            u32x4 kv = {0u, 0u, 0u, 0u};
            if (kv0 + r < seq)
                kv = *reinterpret_cast<const u32x4*>(p.qkv + (tok0 + kv0 + r) * p.ldq + p.h + head * kDH + 8 * lch);
            kreg[i] = kv;
            const bf16* vsrc = p.vt + (int64_t)(head * kDH + r) * p.ldv + tok0 + kv0 + 8 * lch;
            const int valid = seq - (kv0 + 8 * lch);
            u32x4 vv = {0u, 0u, 0u, 0u};
            if (valid >= 8 && vt_vec) {
                vv = *reinterpret_cast<const u32x4*>(vsrc);
            } else if (valid > 0) {
                bf16 e[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) e[k] = k < valid ? vsrc[k] : static_cast<bf16>(0.0f);
                __builtin_memcpy(&vv, e, 16);
            }
            vreg[i] = vv;
        }
    };
    auto store_tile = [&](int b) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = lrow + 32 * i;
            *reinterpret_cast<u32x4*>(&kbuf[b][r * kRowB + ((lch ^ swz(r)) << 4)]) = kreg[i];
            *reinterpret_cast<u32x4*>(&vbuf[b][r * kRowB + ((lch ^ swz(r)) << 4)]) = vreg[i];
        }
    };

    f32x4 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff();
    float l_run = 0.f;

    const int ntiles = (seq + kKT - 1) / kKT;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int b = it & 1;
        const int kv0 = it * kKT;
        if (it + 1 < ntiles) load_tile(kv0 + kKT);

        // S = Q K^T for the 64 keys of the tile: lane holds query li, keys 16 jb + 4 g + r
        f32x4 s[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            s[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = 16 * jb + li;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                bf16x8 kf;
                const u32x4 raw = *reinterpret_cast<const u32x4*>(&kbuf[b][r * kRowB + (((4 * c + g) ^ swz(r)) << 4)]);
                __builtin_memcpy(&kf, &raw, 16);
                s[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], s[jb], 0, 0, 0);
            }
        }

        // online softmax in the log2 domain; keys past the sequence end are -inf
        float mt = -__builtin_inff();
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kv = kv0 + 16 * jb + 4 * g + r;
                const float v = kv < seq ? s[jb][r] * p.scale_log2 : -__builtin_inff();
                s[jb][r] = v;
                mt = fmaxf(mt, v);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float lsum = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bf16 pb = static_cast<bf16>(__builtin_amdgcn_exp2f(s[jb][r] - m_new));
                lsum += static_cast<float>(pb);
                pf[jb >> 1][4 * (jb & 1) + r] = pb;
            }
        l_run = __builtin_fmaf(l_run, alpha, lsum);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;

        // O += P V: V^T rows are head columns; keys in the P fragment's order
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int r = 16 * db + li;
            const uint8_t* vrow = &vbuf[b][r * kRowB];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // keys 32c + 4g .. +3 and 32c + 16 + 4g .. +3: 8-byte halves of 16-byte chunks
                const int ch0 = 4 * c + (g >> 1), ch1 = 4 * c + 2 + (g >> 1);
                const int half = (g & 1) << 3;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + ((ch0 ^ swz(r)) << 4) + half);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + ((ch1 ^ swz(r)) << 4) + half);
                const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
                bf16x8 vf;
                __builtin_memcpy(&vf, &raw, 16);
                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[c], o[db], 0, 0, 0);
            }
        }

        if (it + 1 < ntiles) store_tile(b ^ 1);
        __syncthreads();
    }

    // the row sum over the four lanes that share a query row, then O / l
    float l = l_run + __shfl_xor(l_run, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int q = q0 + 16 * w + li;
    if (q >= seq) return;
    const int64_t row = tok0 + q;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int64_t col = (int64_t)head * kDH + 16 * db + 4 * g;
        f32x4 v = o[db] * inv;
        if (p.x) {
            const bf16x4 xr = *reinterpret_cast<const bf16x4*>(p.x + row * p.ldx + col);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] += static_cast<float>(xr[r]);
        }
        bf16x4 ov;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = static_cast<bf16>(v[r]);
        *reinterpret_cast<bf16x4*>(p.out + row * p.ldo + col) = ov;
    }
}

}  // namespace

hipError_t launch_attention(const void* qkv, int64_t ldq, const void* vt, int64_t ldv, const void* x, int64_t ldx,
                            void* out, int64_t ldo, int64_t batch, int64_t seq, int64_t heads,
                            hipStream_t stream) {
    AttnParams p;
    p.qkv = static_cast<const bf16*>(qkv);
    p.ldq = ldq;
    p.vt = static_cast<const bf16*>(vt);
    p.ldv = ldv;
    p.x = static_cast<const bf16*>(x);
    p.ldx = ldx;
    p.out = static_cast<bf16*>(out);
    p.ldo = ldo;
    p.h = heads * kDH;
    p.seq = (int)seq;
    p.scale_log2 = (float)(kLog2e / 8.0);  // 1 / sqrt(64) = 1/8
    const dim3 grid((unsigned)((seq + kQT - 1) / kQT), (unsigned)heads, (unsigned)batch);
    attn_fwd_kernel<<<grid, dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace tpmlp
