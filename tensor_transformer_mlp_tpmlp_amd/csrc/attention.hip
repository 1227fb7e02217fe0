// Local attention of the head-sharded attention half of the block:
// O = softmax(Q K^T / sqrt(d)) V for every head of every sequence
// ("Tensor Parallelism in Megatron", section 4, the local-attention
// equation), d = 64, no mask, on v_mfma_f32_16x16x32_bf16.
//
// Layouts.  QKV is the projection output, one row per token (batch*seq rows,
// sequence b in rows b*seq ..), with Q in columns 0..h-1, K in h..2h-1, V in
// 2h..3h-1 and head j in columns j*64 .. j*64+63 of each (ld = 3h); all three
// are read where they lie.  O is written in the concatenated-heads layout
// (token row, column j*64 + dd), the all_gather-and-cat of "LLM Lab Notes
// 06", section 2, marker 3, optionally plus the residual x (marker 4).
//
// One block of 256 threads (4 waves) owns 64 QB query rows of one (sequence,
// head); wave w owns QB blocks of 16 rows, from row 16 QB w on.  Keys and
// values stream through LDS in tiles of 64 tokens (64 rows of 128 bytes
// each).  Per tile a wave forms S (16 QB x 64) in 8 QB MFMAs, updates the
// running row maximum and sum (online softmax in the log2 domain, fp32),
// rounds P to bf16 and accumulates O (16 QB x 64) in 8 QB MFMAs; each K and
// V fragment read from LDS feeds QB of them.
//
// MFMA operand order: the first operand's rows index the result's rows as
// seen by the lanes, so S = mfma(K frag, Q frag) leaves lane l with query
// row l & 15 and keys 4 (l >> 4) + r of a 16-key block, and
// O = mfma(V frag, P frag) leaves it with query row l & 15 and head columns
// 4 (l >> 4) + r.  A lane's 8 k-slots of P are therefore keys {4g .. 4g+3}
// of the even 16-key block and {16 + 4g .. 16 + 4g + 3} of the odd one
// (g = l >> 4).  The V fragment (head column l & 15, those 8 keys) comes from
// the V rows in LDS by two transposing reads (ds_read_b64_tr_b16), whose
// per-lane addresses pick exactly those keys.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace tpmlp {

namespace {

typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kDH = 64;      // head width
constexpr int kKT = 64;      // keys per tile
constexpr int kRowB = 128;   // bytes per LDS row (64 bf16)

// 16-byte chunk swizzles of the 128-byte LDS rows.  K tile (16-byte fragment
// reads of 16 rows): the 16 lanes of a read pass hit 16 distinct chunk
// slots.  V tile (transposing reads of 32 bytes from each of 16 consecutive
// rows): the 32-byte windows of those rows cover the 256-byte bank space
// twice.
__device__ __forceinline__ int swz(int row) { return ((row & 8) >> 2) | ((row & 2) << 1); }
__device__ __forceinline__ int vswz(int row) { return 2 * ((row >> 1) & 3); }

struct AttnParams {
    const bf16* qkv;   // batch*seq x 3h
    int64_t ldq;       // 3h
    int64_t tokens;    // batch*seq
    const bf16* x;     // residual, batch*seq x h (nullptr: none)
    int64_t ldx;
    bf16* out;         // batch*seq x h
    int64_t ldo;
    int64_t h;
    int seq;
    float scale_log2;  // log2(e) / sqrt(d)
};

// One tile of 64 keys for one wave's QB blocks of 16 query rows: S = Q K^T,
// the online softmax update, then O = alpha O + P V.  Every K and V^T
// fragment read from LDS feeds QB MFMAs.  kb: the K tile (64 keys x 128
// bytes), vb: the V^T tile (64 head columns x 128 bytes), both with the
// chunk swizzle.
//
// Softmax bookkeeping per row (log2 domain, c = log2(e)/sqrt(d)):
//   m_run: the reference maximum (in units of c s); P = 2^(c s - m_run);
//   ls: the row sums of P, formed by an MFMA of P with a block of ones (so
//       they sum exactly the bf16 P that multiplies V), scaled like O.
// The reference maximum is raised only when a score of the tile exceeds it
// by more than kLazy (then O and ls are rescaled by 2^(m_old - m_new));
// otherwise P stays below 2^kLazy and nothing is rescaled.  O / ls is the
// same for any reference at or below the true maximum, so this changes only
// where the bf16 rounding of P falls.  The decision is taken per wave, so a
// wave either rescales all its rows (each with its own factor) or none.
constexpr float kLazy = 8.0f;

// max(x[l], x[l ^ D]) in every lane l, D = 16 or 32, through the gfx950 lane
// swaps (each returns the pair {x[l], x[l ^ D]} in its two results; measured
// with an in-bounds probe): two VALU operations instead of an LDS permute.
template <int D>
__device__ __forceinline__ float pair_max(float x) {
    const uint32_t u = __float_as_uint(x);
    if constexpr (D == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    } else {
        static_assert(D == 16, "lane distance 16 or 32");
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
}

// vo[db]: this lane's byte offset in the V tile of its transposing read for
// head-column block db, keys 4 g .. 4 g + 3 (add 16 rows for keys 16 + 4 g ..,
// 32 rows per 32-key chunk).
__device__ __forceinline__ void v_offsets(int g, int li, uint32_t (&vo)[4]) {
    const int row = 4 * g + (li >> 2);
    const int vs = vswz(row);
#pragma unroll
    for (int db = 0; db < 4; ++db)
        vo[db] = (uint32_t)(row * kRowB + (((2 * db + ((li & 3) >> 1)) ^ vs) << 4) + ((li & 1) << 3));
}

template <int QB>
__device__ __forceinline__ void attn_tile(const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb,
                                          const bf16x8 (&qf)[QB][2], f32x4 (&o)[QB][4], f32x4 (&ls)[QB],
                                          float (&m_run)[QB], int kv0, int seq, float c_log2, int g, int li,
                                          const uint32_t (&vo)[4]) {
    // S = Q K^T for the 64 keys of the tile: lane holds query li of block i, keys 16 jb + 4 g + r
    f32x4 s[QB][4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        const int r = 16 * jb + li;
#pragma unroll
        for (int i = 0; i < QB; ++i) s[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bf16x8 kf;
            const u32x4 raw = *reinterpret_cast<const u32x4*>(&kb[r * kRowB + (((4 * c + g) ^ swz(r)) << 4)]);
            __builtin_memcpy(&kf, &raw, 16);
#pragma unroll
            for (int i = 0; i < QB; ++i)
                s[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[i][c], s[i][jb], 0, 0, 0);
        }
    }

    // keys past the sequence end (only in a partial last tile) score -inf
    if (kv0 + kKT > seq) {
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (kv0 + 16 * jb + 4 * g + r >= seq) s[i][jb][r] = -__builtin_inff();
    }

    float mc[QB];
    bool raise = false;
#pragma unroll
    for (int i = 0; i < QB; ++i) {
        float mt = fmaxf(fmaxf(s[i][0][0], s[i][0][1]), fmaxf(s[i][0][2], s[i][0][3]));
#pragma unroll
        for (int jb = 1; jb < 4; ++jb)
            mt = fmaxf(fmaxf(mt, fmaxf(s[i][jb][0], s[i][jb][1])), fmaxf(s[i][jb][2], s[i][jb][3]));
        mt = pair_max<16>(mt);
        mt = pair_max<32>(mt);
        mc[i] = mt * c_log2;
        raise |= mc[i] > m_run[i] + kLazy;
    }
    if (__any(raise)) {
#pragma unroll
        for (int i = 0; i < QB; ++i) {
            const float m_new = fmaxf(m_run[i], mc[i]);
            const float alpha = __builtin_amdgcn_exp2f(m_run[i] - m_new);
            m_run[i] = m_new;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[i][db] *= alpha;
            ls[i] *= alpha;
        }
    }

    // P = 2^(c s - m_run), rounded to bf16, in the k-slot order of the PV MFMA
    bf16x8 pf[QB][2];
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pf[i][jb >> 1][4 * (jb & 1) + r] =
                    static_cast<bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[i][jb][r], c_log2, -m_run[i])));

    // row sums: P times a 32 x 16 block of ones, per 32-key chunk
    bf16x8 ones;
#pragma unroll
    for (int k = 0; k < 8; ++k) ones[k] = static_cast<bf16>(1.0f);
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c) ls[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[i][c], ls[i], 0, 0, 0);

    // O += P V: the V fragment of head columns 16 db .. +15 holds, in lane l,
    // column 16 db + (l & 15) at the keys of P's k-slots
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint8_t* vp = vb + vo[db] + 32 * c * kRowB;
            const v4s lo = lds_read_tr16(vp);
            const v4s hi = lds_read_tr16(vp + 16 * kRowB);
            bf16x8 vf;
            __builtin_memcpy(&vf, &lo, 8);
            __builtin_memcpy(reinterpret_cast<uint8_t*>(&vf) + 8, &hi, 8);
#pragma unroll
            for (int i = 0; i < QB; ++i)
                o[i][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[i][c], o[i][db], 0, 0, 0);
        }
    }
}

// Q fragments of a wave's QB row blocks (zeros past the sequence end):
// lane l holds row 16 i + (l & 15) of the wave's rows, d = 32 c + 8 (l >> 4) ..
template <int QB>
__device__ __forceinline__ void load_q(const AttnParams& p, int64_t tok0, int qw, int g, int li,
                                       bf16x8 (&qf)[QB][2], int head) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
        const int q = qw + 16 * i + li;
        const bf16* qrow = p.qkv + (tok0 + q) * p.ldq + head * kDH;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (q < p.seq) raw = *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * g);
            __builtin_memcpy(&qf[i][c], &raw, 16);
        }
    }
}

// O / (row sum) for every row block, plus the residual, rounded to bf16; lane l
// writes row 16 i + (l & 15), columns 16 db + 4 (l >> 4) .. +3.
template <int QB>
__device__ __forceinline__ void store_o(const AttnParams& p, int64_t tok0, int qw, int g, int li, int head,
                                        f32x4 (&o)[QB][4], const f32x4 (&ls)[QB]) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
        // every column of the ones product holds the row sum of this lane's row
        const float inv = 1.0f / ls[i][0];
        const int q = qw + 16 * i + li;
        if (q >= p.seq) continue;
        const int64_t row = tok0 + q;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int64_t col = (int64_t)head * kDH + 16 * db + 4 * g;
            f32x4 v = o[i][db] * inv;
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
}

// s_waitcnt immediates (gfx9): vmcnt in bits [3:0] and [15:14], expcnt and
// lgkmcnt left at their maxima (no wait) unless asked for.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int waitcnt_lgkm0() { return 15 | (3 << 14) | (7 << 4); }

constexpr int kStages = 3;
constexpr int kTileB = kKT * kRowB;  // 8 KiB: one K tile or one V tile

// Key and value tiles move by direct global-to-LDS loads (16 bytes per
// lane) through a ring of three stages, so each tile's loads are issued two
// tiles ahead of its use and no registers stage them.  Wave w fills LDS rows
// 16 w .. 16 w + 15 of each tile in two loads of 8 rows; lane L lands at row
// 16 w + 8 q + L/8, physical chunk L % 8, so it reads the logical chunk
// (L % 8) ^ swizzle(row) of that row.  Buffer resources cover this
// sequence's rows (plus one tile) up to the end of QKV, and each load's
// whole byte offset, the tile's first row included, is a per-lane (VGPR)
// offset with a zero scalar offset: the hardware's range check covers only
// the per-lane offset, so this is what makes rows past the end of QKV read
// as zero.  Rows of the next sequence are masked (keys) or multiplied by
// P = 0 (values) like any row past the sequence end.  Requires (seq + 64)
// rows of QKV below 2 GiB (buffer offsets).
template <int QB>
__global__ __launch_bounds__(256) void attn_fwd_ring_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages][2][kTileB];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int g = lane >> 4;
    const int li = lane & 15;
    const int seq = p.seq;
    const int qw = blockIdx.x * 64 * QB + 16 * QB * w;
    const int head = blockIdx.y;
    const int64_t tok0 = (int64_t)blockIdx.z * seq;

    bf16x8 qf[QB][2];
    load_q<QB>(p, tok0, qw, g, li, qf, head);
    uint32_t vo[4];
    v_offsets(g, li, vo);

    const int64_t k_off = tok0 * p.ldq + p.h + (int64_t)head * kDH;
    const int64_t v_off = k_off + p.h;
    const int64_t total = p.tokens * p.ldq;
    const int64_t span = (int64_t)(seq + kKT) * p.ldq;
    const u32x4 rk = buffer_rsrc_sgpr(p.qkv + k_off, (uint32_t)(min(total - k_off, span) * 2));
    const u32x4 rv = buffer_rsrc_sgpr(p.qkv + v_off, (uint32_t)(min(total - v_off, span) * 2));
    const int r0 = 16 * w + (lane >> 3);
    const int r1 = r0 + 8;
    const int pc = lane & 7;
    const uint32_t kv_0 = (uint32_t)(r0 * p.ldq * 2 + ((pc ^ swz(r0)) << 4));
    const uint32_t kv_1 = (uint32_t)(r1 * p.ldq * 2 + ((pc ^ swz(r1)) << 4));
    const uint32_t vv_0 = (uint32_t)(r0 * p.ldq * 2 + ((pc ^ vswz(r0)) << 4));
    const uint32_t vv_1 = (uint32_t)(r1 * p.ldq * 2 + ((pc ^ vswz(r1)) << 4));
    const int dst0 = 16 * w * kRowB, dst1 = dst0 + 8 * kRowB;

    auto issue = [&](int kv0, int st) {
        const uint32_t so = (uint32_t)(kv0 * p.ldq * 2);
        dma16_asm(&ring[st][0][dst0], rk, kv_0 + so, 0u);
        dma16_asm(&ring[st][0][dst1], rk, kv_1 + so, 0u);
        dma16_asm(&ring[st][1][dst0], rv, vv_0 + so, 0u);
        dma16_asm(&ring[st][1][dst1], rv, vv_1 + so, 0u);
    };

    f32x4 o[QB][4], ls[QB];
    float m_run[QB];
#pragma unroll
    for (int i = 0; i < QB; ++i) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        ls[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[i] = -__builtin_inff();
    }

    const int ntiles = (seq + kKT - 1) / kKT;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the Q fragments
    issue(0, 0);
    if (ntiles > 1) issue(kKT, 1);
    int st = 0;
    for (int it = 0; it < ntiles; ++it) {
        // this tile's four loads have landed (the next tile's may be in flight),
        // and every wave is done reading the stage the next issue overwrites
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
        if (it + 1 < ntiles)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_s_barrier();
        if (it + 2 < ntiles) issue((it + 2) * kKT, st == 0 ? 2 : st - 1);
        attn_tile<QB>(ring[st][0], ring[st][1], qf, o, ls, m_run, it * kKT, seq, p.scale_log2, g, li, vo);
        st = st == 2 ? 0 : st + 1;
    }
    store_o<QB>(p, tok0, qw, g, li, head, o, ls);
}

}  // namespace

bool attention_fits(int64_t seq, int64_t heads) {
    return (seq + kKT) * 3 * heads * kDH * 2 < ((int64_t)1 << 31);
}

hipError_t launch_attention(const void* qkv, int64_t ldq, const void* x, int64_t ldx, void* out, int64_t ldo,
                            int64_t batch, int64_t seq, int64_t heads, hipStream_t stream) {
    AttnParams p;
    p.qkv = static_cast<const bf16*>(qkv);
    p.ldq = ldq;
    p.tokens = batch * seq;
    p.x = static_cast<const bf16*>(x);
    p.ldx = ldx;
    p.out = static_cast<bf16*>(out);
    p.ldo = ldo;
    p.h = heads * kDH;
    p.seq = (int)seq;
    p.scale_log2 = (float)(kLog2e / 8.0);  // 1 / sqrt(64) = 1/8
    if (!attention_fits(seq, heads)) return hipErrorInvalidValue;
    // 64 query rows per wave for long sequences (each K/V fragment feeds four
    // MFMAs); 32 when that still gives every CU a block; else 16, which
    // doubles the blocks of short sequences (s = 128, b = 8, 16 heads: 256
    // blocks instead of 128; measured 8.3 against 9.5 us, while at s = 256
    // and 512 the 32-row form is faster)
    auto launch = [&](auto qb) {
        constexpr int QB = decltype(qb)::value;
        const dim3 grid((unsigned)((seq + 64 * QB - 1) / (64 * QB)), (unsigned)heads, (unsigned)batch);
        attn_fwd_ring_kernel<QB><<<grid, dim3(256), 0, stream>>>(p);
    };
    const int64_t blocks_qb2 = (seq + 127) / 128 * heads * batch;
    if (seq >= 1024)
        launch(std::integral_constant<int, 4>{});
    else if (blocks_qb2 >= device_cu_count())
        launch(std::integral_constant<int, 2>{});
    else
        launch(std::integral_constant<int, 1>{});
    return hipGetLastError();
}

}  // namespace tpmlp
