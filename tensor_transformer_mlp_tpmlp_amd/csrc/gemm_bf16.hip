// Throughput GEMM for bf16 operands on gfx950 matrix cores.
//
// C[m][n] = epi( sum_k Aop[m][k] * Bop[n][k] ), Aop (M x K) and Bop (N x K)
// K-contiguous, fp32 accumulation in v_mfma_f32_16x16x32_bf16.
//
// Both GEMMs of the TP-MLP run here:
//   * column-parallel GEMM1 ("Tensor-Parallel MLP (Megatron)", section
//     "The split", bullet 1): Aop = X, Bop = packed A^T, all shards in one
//     launch (shard i is the N range iF/n..(i+1)F/n-1), GeLU fused in the
//     epilogue, H stored in bf16;
//   * row-parallel GEMM2 (bullet 2 and the sum of bullet 3): Aop = H,
//     Bop = packed B^T; each output tile's K loop runs over every shard's
//     rows, so all partials Y_i are summed in the same fp32 accumulator and
//     only the sum is written.  The forward never splits this K loop: when
//     its output has few tiles, narrower tiles fill the GPU instead.
//
// Tiling: one BM x BN output tile per workgroup of 4 waves (2x2, one wave
// per SIMD), each wave owning a (BM/2) x (BN/2) sub-tile of 16x16 MFMA
// blocks with its fp32 accumulators in AGPRs (256 per lane at 256x256).
// The tile shapes are 256x256, 128x128, 128x64 and 64x64; the host picks
// the one that fills the GPU best (see choose_cfg).  K advances 64 per step;
// each operand's 64-wide slice of a step is a "unit" (BM or BN rows of 128
// bytes), and a ring of NU unit slots holds the units in flight.
//
// The 16x16x32 MFMA is used rather than 32x32x16: with random operands it
// sustains a higher clock under the chip's power limit for the same FLOP.
// Each MFMA takes the Bop fragment as its first operand, so a lane's four
// accumulators are four consecutive output columns of one row: the epilogue
// writes 8 (bf16) or 16 (fp32) contiguous bytes per lane and block.
//
// Global -> LDS moves use the direct-to-LDS global load
// (global_load_lds_dwordx4, a scalar base and 32-bit lane offsets): no VGPR
// staging and no ds_write, and in the MFMA stream about half the issue cost
// of the buffer form.  Lane L of a wave's load lands at LDS base + 16 L, so
// the XOR swizzle of the LDS layout is applied on the global side by
// choosing which 16-byte chunk each lane fetches.
//
// Pipeline: unit u of the K loop is A_t for u = 2t and B_t for u = 2t + 1;
// it lives in ring slot u mod NU.  Step t computes two 32-deep sub-steps
// from A_t and B_t.  Sub-step 0 reads the fragments of sub-step 1 and issues
// unit 2t + NU - 1 into the slot of B_{t-1}; a barrier then publishes
// A_{t+1}, B_{t+1} and frees A_t, B_t; sub-step 1 reads the next step's
// first fragments and issues unit 2t + NU into the slot of A_t.  A unit is
// therefore issued (NU - 3) / 2 steps or more before the barrier that
// publishes it.  Each load covers whole 128-byte lines (8 rows x 128
// bytes), the unit the L1 fetches from L2 in, and loads and reads are
// spread evenly between the MFMAs.
//
// Ragged shapes: M and N need not be whole tiles.  Each lane's load rows
// are clamped to the last row of the operand, so an edge tile reads only
// rows that exist (its extra rows repeat the last one and their results
// are discarded), and the epilogue stores only rows below M and columns
// below N.  K must be a whole number of 64-wide steps.
//
// LayerNorm prologue (FFN half of the Post-LN block, "LLM Lab Notes 06",
// section 2, marker 5) is applied algebraically in GEMM1's epilogue:
//   sum_k (x_k - mu) r a_k = r * (sum_k x_k a_k - mu * sum_k a_k),
// with the per-row mean mu and r = 1/sqrt(var + eps) from the statistics
// kernel and the per-column sums of A from shard time.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace tpmlp {

namespace {

// K advances BK = 64 per step, two 16x16x32 MFMA sub-steps.
constexpr int BK = 64;
constexpr int kLdsBytes = 160 * 1024;
// MFMAs of a step's second sub-step issued before its barrier (256x256 tile,
// row-major operands; measured: the forward -0.2%, the backward -0.8%).
constexpr int kPreBarrier = 3;

// A tile shape: BM x BN output tile, NU ring slots.  Each wave owns NBM x NBN
// blocks of 16x16; a unit of Aop is BM rows of 128 bytes (UA), of Bop BN rows
// (UB); a slot holds either.  A wave issues LPA (LPB) direct loads of 1 KiB
// per unit of Aop (Bop).
template <int BM_, int BN_, int NU_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, NU = NU_;
    static constexpr int NBM = BM / 32, NBN = BN / 32;
    static constexpr int UA = BM * BK * 2, UB = BN * BK * 2;
    static constexpr int SLOT = UA > UB ? UA : UB;
    static constexpr int LPA = BM / 32, LPB = BN / 32;
    // loads in flight at a steady barrier: units 2t+4 .. 2t+NU-1, starting with an Aop unit
    static constexpr int VM_STEADY = ((NU - 3) / 2) * LPA + ((NU - 4) / 2) * LPB;
    // bf16 output staged through LDS after the K loop: each wave's
    // (BM/2) x (BN/2) block in rows of BN bytes plus 16 bytes of padding
    static constexpr int OUT_PITCH = BN + 16;
    static constexpr int OUT_WAVE = (BM / 2) * OUT_PITCH;
    static_assert(4 * OUT_WAVE <= NU * SLOT, "the staged output must fit in the ring");
    static_assert(NU >= 5, "the ring needs the four units of two steps plus one in flight");
    static_assert(NU * SLOT <= kLdsBytes, "the ring must fit in LDS");
    static_assert(BM % 64 == 0 && BN % 64 == 0, "tile edges of whole 64-row load groups");
};

using C256 = Cfg<256, 256, 5>;    // one workgroup per CU
using C128 = Cfg<128, 128, 5>;    // two per CU
using C128x64 = Cfg<128, 64, 10>; // one per CU, units issued 3 steps ahead
using C64 = Cfg<64, 64, 10>;      // two per CU, units issued 3 steps ahead

// The GeLU epilogue that also stores the pre-activation (GemmArgs::preact_out
// set), and the GeLU-derivative epilogue that also stores GeLU of its operand
// (GemmArgs::gelu_out set): their own instantiations, so the plain epilogues
// carry none of it.
constexpr int kEpiGeluSave = 3;
constexpr int kEpiGeluGradSave = 4;

struct FastParams {
    const bf16* A;
    int64_t lda;
    const bf16* B;
    int64_t ldb;
    int M, N, K;
    void* C;
    int64_t ldc;
    const bf16* R;
    int64_t ldr;
    const float* mean;   // LayerNorm: per-row mean and 1/sqrt(var+eps)
    const float* rstd;
    const float* csum;   // LayerNorm: per-column sums of Bop (= column sums of A)
    const bf16* aux;     // kEpiGeluGrad: pre-activation, M x N
    int64_t ldaux;
    bf16* preact;        // kEpiGelu: optional copy of the pre-activation (C's layout)
    bf16* gelu_out;      // kEpiGeluGrad: optional GeLU of the pre-activation (C's layout)
    int tiles_m, tiles_n;
    int group;           // tile rows walked together on one XCD
    int nt_store;        // write C with non-temporal stores
    int splits;          // K is split into `splits` equal ranges (grid = tiles x splits)
    int64_t c_split_stride;  // elements between the outputs of consecutive K ranges
};

// s_waitcnt encodings (gfx9): vmcnt in bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; a field at its maximum does not wait.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int waitcnt_lgkm0() { return 15 | (3 << 14) | (7 << 4); }

// LDS layout of a unit: tile row r at byte 128 r, its eight 16-byte
// k-chunks permuted: logical chunk c sits at physical chunk c ^ key(r),
// key(r) = ((r & 8) >> 2) | ((r & 2) << 1).  A 128-bit LDS read is served
// in four passes of 16 lanes; within each half-wave, the 4-lane groups whose
// index (0..7) has an even number of set bits form one pass and the others
// the second (measured with the bank-conflict counter).  A fragment read puts
// rows j, j+12 of one chunk and rows j+4, j+8 of the next into one pass; the
// key sends the sixteen lanes of every pass to distinct 16-byte bank groups,
// so the reads are conflict-free.  The direct loads write 1 KiB contiguously,
// which is conflict-free under any key.
__device__ __forceinline__ uint32_t lds_key(uint32_t r) { return ((r & 8) >> 2) | ((r & 2) << 1); }

// LDS layout of a K-major unit: row r (one k) of 2 BM bytes, its 16-byte
// chunk c at physical chunk c ^ kswz(r), kswz(r) = 2 ((r & 3) + 4 ((r >> 3) & 1)).
// Rows start on the same bank (their length is a multiple of 256 bytes); a
// transposing fragment read takes 32 bytes from each of 16 rows 8 g + 4 h + i
// (g = 0..3, i = 0..3), and the key gives the rows of each half-wave eight
// distinct 32-byte bank groups.  Needs rows of at least 16 chunks (BM >= 128).
__device__ __forceinline__ uint32_t kswz(uint32_t r) { return 2 * ((r & 3) + 4 * ((r >> 3) & 1)); }


// Blocks reach the 8 XCDs round-robin (block b runs on XCD b % 8).  Give each
// XCD a contiguous range of work ids, and walk the tiles of a K range in
// groups of `group` tile rows, column by column, so that the tiles running at
// once on an XCD share Aop rows and Bop columns in its L2.  Work id w is tile
// w % tiles of K range w / tiles.  Bijective for any tile count and group.
__device__ __forceinline__ void map_work(int bid, int tiles_m, int tiles_n, int splits, int group, int& tm,
                                         int& tn, int& kz) {
    const int tiles = tiles_m * tiles_n;
    const int total = tiles * splits;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    const int pid = xcd * per + min(xcd, rem) + idx;
    kz = pid / tiles;
    const int tid = pid - kz * tiles;
    const int group_tiles = group * tiles_n;
    const int g = tid / group_tiles;
    const int first_m = g * group;
    const int gm = min(tiles_m - first_m, group);
    const int local = tid - g * group_tiles;
    tm = first_m + local % gm;
    tn = local / gm;
}

typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int V> using ic = std::integral_constant<int, V>;

// gelu_tanh of N f32x4 values, one operation of the formula at a time over
// all of them (the same operations as gelu_tanh, so the same results).  The
// scheduling barriers keep the compiler from evaluating the values one
// after another, which would expose the latency of every step.
template <int N>
__device__ __forceinline__ void gelu_tanh_staged(f32x4 (&v)[N]) {
    f32x4 z[N];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) z[j][r] = v[j][r] * v[j][r];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) z[j][r] = v[j][r] * __builtin_fmaf(z[j][r], kGeluK1, kGeluK0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) z[j][r] = __builtin_amdgcn_exp2f(z[j][r]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) z[j][r] = __builtin_amdgcn_rcpf(1.0f + z[j][r]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[j][r] = v[j][r] * z[j][r];
}

// Per-load byte offsets of one lane into a row-major operand unit of R rows
// (R/4 rows per wave, LP = R/32 loads of 8 rows each).  In load q lane L
// fills unit row w R/4 + 8 q + L/8 at physical chunk L % 8, which must hold
// logical chunk (L % 8) ^ key(row).  The source row is clamped to the last
// of the operand's `rows` rows (r0 is the tile's first row, where the
// load's base points), so no load reads past the operand.
template <int R, int LP>
__device__ __forceinline__ void row_load_offsets(uint32_t (&v)[LP], int w, int lane, int64_t r0, int64_t rows,
                                                 int64_t ld) {
#pragma unroll
    for (int q = 0; q < LP; ++q) {
        const uint32_t row = (uint32_t)(w * (R / 4) + 8 * q + (lane >> 3));
        const int64_t src = min(r0 + (int64_t)row, rows - 1) - r0;
        v[q] = (uint32_t)(src * ld * 2) + ((((uint32_t)lane & 7u) ^ lds_key(row)) << 4);
    }
}

template <class C, int EPI, bool LN, typename TC, int KM>
__global__ __launch_bounds__(256) void gemm_bf16_mfma(FastParams p) {
    constexpr bool KA = (KM & 1) != 0, KB = (KM & 2) != 0;  // operand stored K-major
    constexpr int BM = C::BM, BN = C::BN, NU = C::NU;
    constexpr int NBM = C::NBM, NBN = C::NBN;
    constexpr int SLOT = C::SLOT;
    constexpr int LPA = C::LPA, LPB = C::LPB;
    static_assert(!KM || (BM >= 128 && BN >= 128), "K-major units need rows of at least 16 chunks");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NU * SLOT];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, kept in an SGPR
    const int wm = w >> 1, wn = w & 1;
    int tm, tn, kz;
    map_work(blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.group, tm, tn, kz);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const int kc = p.K / p.splits;      // this block's K range: [kz kc, (kz+1) kc)
    const int64_t k0 = (int64_t)kz * kc;

    // This tile's panel of each operand from its K range on: a row-major
    // operand's row m0 (n0) at column k0, a K-major operand's row k0 at
    // column m0 (n0).  A K-loop load of step ks reads panel + ks * step plus
    // a per-lane offset, with ks clamped to the range's last step and the
    // rows of a row-major operand clamped to the operand, so every load
    // reads inside the operand.  (K is a whole number of steps; K-major
    // operands come in whole tiles.)
    const uint8_t* const pan_a = reinterpret_cast<const uint8_t*>(KA ? p.A + k0 * p.lda + m0 : p.A + m0 * p.lda + k0);
    const uint8_t* const pan_b = reinterpret_cast<const uint8_t*>(KB ? p.B + k0 * p.ldb + n0 : p.B + n0 * p.ldb + k0);
    // bytes per K step (below 2^31: a K-major operand's K rows are, see fits_cfg)
    const uint32_t step_a = KA ? (uint32_t)(BK * p.lda * 2) : (uint32_t)(BK * 2);
    const uint32_t step_b = KB ? (uint32_t)(BK * p.ldb * 2) : (uint32_t)(BK * 2);
    const int nk = kc / BK;   // >= 1
    // row-major operands: per-load lane offsets (rows clamped to the operand)
    uint32_t va[KA ? 1 : LPA], vb[KB ? 1 : LPB];
    if constexpr (!KA) row_load_offsets<BM, LPA>(va, w, lane, m0, p.M, p.lda);
    if constexpr (!KB) row_load_offsets<BN, LPB>(vb, w, lane, n0, p.N, p.ldb);
    const uint32_t dst_a = (uint32_t)(w * (BM / 4) * 128), dst_b = (uint32_t)(w * (BN / 4) * 128);

    // slot s of the ring
    auto slot = [&](int s) { return ring + s * SLOT; };

    // K-major operand units: 64 rows (k) of 2 BM (2 BN) bytes (the tile's
    // columns), 16-byte chunk c of row r at physical chunk c ^ kswz(r).  Wave
    // w fills rows 16 w .. 16 w + 15 with LP loads of 1 KiB; in load q lane L
    // lands at row 16 w + q RPL + L / CPR, physical chunk L % CPR.
    constexpr int RBA = BM * 2, CPRA = RBA / 16, RPLA = 64 / CPRA;
    constexpr int RBB = BN * 2, CPRB = RBB / 16, RPLB = 64 / CPRB;
    uint32_t kv_a[KA ? LPA : 1], kv_b[KB ? LPB : 1];
    if constexpr (KA) {
#pragma unroll
        for (int q = 0; q < LPA; ++q) {
            const uint32_t r = (uint32_t)(16 * w + q * RPLA + lane / CPRA);
            kv_a[q] = r * (uint32_t)(p.lda * 2) + (((uint32_t)(lane % CPRA) ^ kswz(r)) << 4);
        }
    }
    if constexpr (KB) {
#pragma unroll
        for (int q = 0; q < LPB; ++q) {
            const uint32_t r = (uint32_t)(16 * w + q * RPLB + lane / CPRB);
            kv_b[q] = r * (uint32_t)(p.ldb * 2) + (((uint32_t)(lane % CPRB) ^ kswz(r)) << 4);
        }
    }

    // load q of the unit of operand `op` (0 = Aop, 1 = Bop) of K step kstep
    // into slot st; a step past the range's last reloads the last one (see
    // the main loop)
    const uint32_t ring_lds = lds_addr(ring);
    auto load_one = [&](uint8_t* st, int op, int kstep, int q) {
        const uint32_t ks = (uint32_t)(kstep < nk ? kstep : nk - 1);
        const uint32_t sl = ring_lds + (uint32_t)(st - ring);
        if (op) {
            uint32_t voff;
            if constexpr (KB) voff = kv_b[q];
            else voff = vb[q];
            gdma16_asm(sl + dst_b + q * 1024, pan_b + (uint64_t)ks * step_b, voff);
        } else {
            uint32_t voff;
            if constexpr (KA) voff = kv_a[q];
            else voff = va[q];
            gdma16_asm(sl + dst_a + q * 1024, pan_a + (uint64_t)ks * step_a, voff);
        }
    };

    // MFMA operand reads: a 16x16x32 fragment is 16 rows x 32 k; in sub-step
    // kk lane l reads row (l & 15) of the block at logical chunk
    // 4 kk + (l >> 4).  The same lane -> k assignment for both operands makes
    // each MFMA a plain 32-long dot product per output.
    const uint32_t kr = lds_key((uint32_t)lane & 15);
    const uint32_t rd_a = (uint32_t)((wm * 16 * NBM + (lane & 15)) * 128);
    const uint32_t rd_b = (uint32_t)((wn * 16 * NBN + (lane & 15)) * 128);
    const uint32_t ch0 = (((uint32_t)(lane >> 4)) ^ kr) << 4;
    const uint32_t ch1 = (((uint32_t)(4 + (lane >> 4))) ^ kr) << 4;

    // K-major fragment reads: two ds_read_b64_tr_b16 per 16 x 32 fragment.
    // In a 16-lane group, lane i addresses row (k) 8 g + 4 h + i / 4 (g the
    // group, h the half) at column 16 f + 4 (i % 4) of the fragment's 16
    // columns; the transposing read leaves lane i with column i and the four
    // rows 8 g + 4 h .. +3, so the two halves are k-slots 8 g .. 8 g + 7, the
    // same order as a row-major fragment.  kf_*[f] is fragment f's byte offset
    // in the unit at sub-step 0, h = 0; sub-step kk and half h add
    // (32 kk + 4 h) RB.
    uint32_t kf_a[KA ? NBM : 1], kf_b[KB ? NBN : 1];
    {
        const uint32_t li = (uint32_t)lane & 15, g = (uint32_t)lane >> 4;
        const uint32_t row = 8 * g + (li >> 2);
        const uint32_t sw = kswz(row);
        if constexpr (KA) {
#pragma unroll
            for (int f = 0; f < NBM; ++f) {
                const uint32_t col = (uint32_t)(wm * 16 * NBM + 16 * f) + 4 * (li & 3);
                kf_a[f] = row * RBA + ((((col >> 3) ^ sw)) << 4) + ((col & 7) << 1);
            }
        }
        if constexpr (KB) {
#pragma unroll
            for (int f = 0; f < NBN; ++f) {
                const uint32_t col = (uint32_t)(wn * 16 * NBN + 16 * f) + 4 * (li & 3);
                kf_b[f] = row * RBB + ((((col >> 3) ^ sw)) << 4) + ((col & 7) << 1);
            }
        }
    }
    auto read_frag = [&](const uint8_t* unit, uint32_t off, int kk, int rb) -> bf16x8 {
        const uint8_t* q = unit + off + kk * 32 * rb;
        const v4s lo = lds_read_tr16(q);
        const v4s hi = lds_read_tr16(q + 4 * rb);
        bf16x8 r;
        __builtin_memcpy(&r, &lo, 8);
        __builtin_memcpy(reinterpret_cast<uint8_t*>(&r) + 8, &hi, 8);
        return r;
    };

    // acc[i][j]: Aop block i (rows), Bop block j (columns).  With the Bop
    // fragment first, lane l holds row (l & 15) of block i and columns
    // 4 (l >> 4) + r, r = 0..3, of block j.  The MFMAs are issued as inline
    // assembly with the accumulator tied to AGPRs ("+a"): the compiler keeps
    // every accumulator in place for the whole K loop (its own MFMA builtin
    // lets the register allocator move some of 256 live accumulators between
    // AGPRs and VGPRs), and the order of MFMAs, LDS reads and direct loads
    // within a sub-step is the order written below.  The two hazards it no
    // longer sees are covered explicitly: the AGPR writes of the zero
    // initialisation before the first MFMA reads them, and the last MFMA's
    // results before the epilogue reads them.
    f32x4 acc[NBM][NBN];
#pragma unroll
    for (int i = 0; i < NBM; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j) {
            acc[i][j] = f32x4{};
            asm volatile("" : "+a"(acc[i][j]));
        }
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");

    bf16x8 fa0[NBM], fb0[NBN], fa1[NBM], fb1[NBN];

    // Per sub-step: NM MFMAs; the NR fragment reads of the next sub-step go
    // one after every RS-th MFMA from the first, the direct loads of one unit
    // one after every NM/LP-th.
    constexpr int NM = NBM * NBN, NR = NBM + NBN, RS = NM / NR / 2 > 0 ? NM / NR / 2 : 1;
    static_assert(NM % LPA == 0 && NM % LPB == 0, "sub-step layout");

    auto frag_a = [&](const uint8_t* ua, uint32_t ch, int kk, int f) -> bf16x8 {
        if constexpr (KA) return read_frag(ua, kf_a[f], kk, RBA);
        else return *reinterpret_cast<const bf16x8*>(ua + rd_a + ch + f * 2048);
    };
    auto frag_b = [&](const uint8_t* ub, uint32_t ch, int kk, int f) -> bf16x8 {
        if constexpr (KB) return read_frag(ub, kf_b[f], kk, RBB);
        else return *reinterpret_cast<const bf16x8*>(ub + rd_b + ch + f * 2048);
    };
    auto barrier_wait = [&](auto vm_left) {
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(decltype(vm_left)::value));
        __builtin_amdgcn_s_barrier();
    };
    // One sub-step: MFMAs on (fc, gc); read the next fragments at chunk
    // offset ch, sub-step kk, from units ua (Aop) and ub (Bop) into (fn, gn)
    // when do_read; with OP = 0 (1) issue the Aop (Bop) unit of K step ks
    // into slot dst, with OP = -1 nothing.  With PRE > 0 the step's barrier
    // comes after the first PRE MFMAs (which need only registers) and the
    // reads and loads, which need it, start after it: the matrix core works
    // through the MFMAs already issued while the waves meet.
    auto sub_step = [&](const bf16x8 (&fc)[NBM], const bf16x8 (&gc)[NBN], const uint8_t* ua, const uint8_t* ub,
                        uint32_t ch, int kk, bf16x8 (&fn)[NBM], bf16x8 (&gn)[NBN], bool do_read, auto op_c,
                        uint8_t* dst, int ks, auto pre_c) {
        constexpr int OP = decltype(op_c)::value;
        constexpr int PRE = decltype(pre_c)::value;
        static_assert(PRE >= 0 && PRE < NM / LPA && PRE < NM / LPB, "loads must fit after the barrier");
        constexpr int LP = OP == 1 ? LPB : LPA;
        constexpr int LS = NM / LP;
#pragma unroll
        for (int idx = 0; idx < NM; ++idx) {
            const int i = idx / NBN, j = idx % NBN;
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(gc[j]), "v"(fc[i]));
            if constexpr (PRE > 0)
                if (idx == PRE - 1) barrier_wait(ic<C::VM_STEADY>{});
            const int jdx = idx - PRE;
            if (jdx < 0) continue;
            if (do_read && jdx % RS == 0 && jdx / RS < NR) {
                // fragment reads in consumption order: Aop 0, Bop 0..NBN-1, Aop 1..NBM-1
                const int r = jdx / RS;
                if (r == 0) fn[0] = frag_a(ua, ch, kk, 0);
                else if (r <= NBN) gn[r - 1] = frag_b(ub, ch, kk, r - 1);
                else fn[r - NBN] = frag_a(ua, ch, kk, r - NBN);
            }
            if constexpr (OP >= 0)
                if (jdx % LS == 0) load_one(dst, OP, ks, jdx / LS);
        }
    };

    auto next = [](int s, int d) { s += d; return s >= NU ? s - NU : s; };

    // Units past the last one (u >= 2 nk) are issued like the others but
    // reload the last K step's unit into slots nobody reads again (they are
    // drained before the epilogue reuses the ring).  So every step but the
    // last issues the same instructions and has the same count of loads in
    // flight at its barrier (one loop, whose register assignment stays
    // fixed: two loops let the allocator move an accumulator through VGPRs
    // between the inline-assembly MFMAs, which the compiler cannot pad for).
    // prologue: units 0 .. NU-2; wait for A_0 and B_0
#pragma unroll
    for (int u = 0; u < NU - 1; ++u) {
        uint8_t* st = slot(u);
        if (u & 1) {
#pragma unroll
            for (int q = 0; q < LPB; ++q) load_one(st, 1, u >> 1, q);
        } else {
#pragma unroll
            for (int q = 0; q < LPA; ++q) load_one(st, 0, u >> 1, q);
        }
    }
    constexpr int VM_PRO = ((NU - 2) / 2) * LPA + ((NU - 3) / 2) * LPB;  // units 2 .. NU-2
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_PRO));
    __builtin_amdgcn_s_barrier();
    {
        fa0[0] = frag_a(slot(0), ch0, 0, 0);
#pragma unroll
        for (int j = 0; j < NBN; ++j) fb0[j] = frag_b(slot(1), ch0, 0, j);
#pragma unroll
        for (int i = 1; i < NBM; ++i) fa0[i] = frag_a(slot(0), ch0, 0, i);
    }

    // Sub-step 0 of step t issues unit 2t + NU - 1 (into the slot of B_{t-1},
    // which is slot(sa) - 1), sub-step 1 unit 2t + NU (into the slot of A_t);
    // their operands are fixed by the parity of NU.  Every barrier leaves the
    // units 2t+4 .. 2t+NU-1 in flight.
    constexpr int OP0 = (NU - 1) & 1, OP1 = NU & 1;
    // A_t sits in slot 2t mod NU.  For the 256x256 tile of row-major operands
    // the loop body is written out for the five phases of that slot (NU = 5)
    // with the slots as constants, each followed by the exit test: the slot
    // arithmetic otherwise opens a gap of about 25 scalar instructions in
    // the MFMA stream at every step.  (Written out for the other tiles, the
    // register allocator moves accumulators through VGPRs and spills.)
    auto step = [&](auto sa_c, int tt) {
        constexpr int SA = decltype(sa_c)::value;
        constexpr int SB = (SA + 1) % NU, SA1 = (SA + 2) % NU, SB1 = (SA + 3) % NU, SP = (SA + NU - 1) % NU;
        const int u0 = 2 * tt + NU - 1;
        sub_step(fa0, fb0, slot(SA), slot(SB), ch1, 1, fa1, fb1, true, ic<OP0>{}, slot(SP), u0 >> 1, ic<0>{});
        sub_step(fa1, fb1, slot(SA1), slot(SB1), ch0, 0, fa0, fb0, true, ic<OP1>{}, slot(SA), (u0 + 1) >> 1,
                 ic<(KM == 0 && BM == 256 && BN == 256) ? kPreBarrier : 0>{});
    };
    int tt = 0;
    if constexpr (KM == 0 && BM == 256 && BN == 256) {
        static_assert(NU == 5, "five slot phases");
        if (nk > 1) {
            for (;;) {
                step(ic<0>{}, tt);
                if (++tt == nk - 1) break;
                step(ic<2>{}, tt);
                if (++tt == nk - 1) break;
                step(ic<4>{}, tt);
                if (++tt == nk - 1) break;
                step(ic<1>{}, tt);
                if (++tt == nk - 1) break;
                step(ic<3>{}, tt);
                if (++tt == nk - 1) break;
            }
        }
    } else if constexpr (NU == 5) {
        // The other five-slot tiles carry the slots' LDS offsets instead: the
        // five slots of step t + 1 are those of step t rotated, (A_t, B_t,
        // A_t+1, B_t+1, P) -> (A_t+1, B_t+1, P, A_t, B_t), a few moves in
        // place of the slot arithmetic.
        uint32_t oa = 0, ob = SLOT, oa1 = 2 * SLOT, ob1 = 3 * SLOT, op = 4 * SLOT;
        for (; tt < nk - 1; ++tt) {
            const int u0 = 2 * tt + NU - 1;
            sub_step(fa0, fb0, ring + oa, ring + ob, ch1, 1, fa1, fb1, true, ic<OP0>{}, ring + op, u0 >> 1, ic<0>{});
            barrier_wait(ic<C::VM_STEADY>{});
            sub_step(fa1, fb1, ring + oa1, ring + ob1, ch0, 0, fa0, fb0, true, ic<OP1>{}, ring + oa, (u0 + 1) >> 1, ic<0>{});
            const uint32_t t0 = oa, t1 = ob;
            oa = oa1;
            ob = ob1;
            oa1 = op;
            ob1 = t0;
            op = t1;
        }
    } else {
        int sa = 0;  // slot of A_t
        for (; tt < nk - 1; ++tt) {
            const int sb = next(sa, 1), sa1 = next(sa, 2), sb1 = next(sa, 3), sp = next(sa, NU - 1);
            const int u0 = 2 * tt + NU - 1;
            sub_step(fa0, fb0, slot(sa), slot(sb), ch1, 1, fa1, fb1, true, ic<OP0>{}, slot(sp), u0 >> 1, ic<0>{});
            barrier_wait(ic<C::VM_STEADY>{});
            sub_step(fa1, fb1, slot(sa1), slot(sb1), ch0, 0, fa0, fb0, true, ic<OP1>{}, slot(sa), (u0 + 1) >> 1, ic<0>{});
            sa = sa1;
        }
    }
    const int sa = (2 * tt) % NU;  // slot of A of the last step
    // the last step: nothing left to load or to read ahead; the reloads
    // still in flight (the last units of the ring) finish before the epilogue
    sub_step(fa0, fb0, slot(sa), slot(next(sa, 1)), ch1, 1, fa1, fb1, true, ic<-1>{}, nullptr, 0, ic<0>{});
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
    sub_step(fa1, fb1, slot(sa), slot(sa), ch0, 0, fa0, fb0, false, ic<-1>{}, nullptr, 0, ic<0>{});
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    // a bf16 output is staged in the ring's LDS: every wave must be done
    // reading its last units first
    constexpr bool kStage = std::is_same<TC, bf16>::value;
    if constexpr (kStage) __builtin_amdgcn_s_barrier();
    // results of the last MFMAs are read by the epilogue
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // Epilogue: lane l writes row m = ... + (l & 15) of block i, columns
    // n .. n+3 with n = ... + 4 (l >> 4) of block j.  A whole row block is
    // transformed before it is stored, which gives the scheduler NBN * 4
    // independent GeLU chains to interleave.
    //
    // Every epilogue access goes through a buffer resource that starts at
    // this tile's first row and column and ends after its last row below M,
    // and a column at or past N gets the offset kOut, past every resource:
    // the hardware's range check then drops the stores of rows and columns
    // outside the matrix and returns zero for such loads, with no branch and
    // no clamping (edge tiles of ragged shapes; interior tiles pay one add
    // per access).
    constexpr uint32_t kOut = 0x80000000u;
    const int64_t rows_t = min((int64_t)BM, (int64_t)p.M - m0);
    const int64_t cols_t = (int64_t)p.N - n0;
    const uint32_t lr = (uint32_t)(wm * 16 * NBM + (lane & 15));       // lane's row in the tile, block 0
    const uint32_t lc = (uint32_t)(wn * 16 * NBN + 4 * (lane >> 4));   // lane's column in the tile, block 0
    uint32_t cb2[NBN], cbc[NBN];  // column byte offsets for 2-byte elements and for C's, or kOut
#pragma unroll
    for (int j = 0; j < NBN; ++j) {
        const bool in = (int64_t)(lc + 16 * j) < cols_t;
        cb2[j] = in ? (lc + 16 * j) * 2u : kOut;
        cbc[j] = in ? (lc + 16 * j) * (uint32_t)sizeof(TC) : kOut;
    }
    auto rsrc = [&](const void* base, int64_t ld, int es) {
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>(base), (short)0, (int)(rows_t * ld * es), 0x00020000);
    };
    TC* __restrict__ Cp = static_cast<TC*>(p.C) + kz * p.c_split_stride;
    const auto rc = rsrc(Cp + m0 * p.ldc + n0, p.ldc, (int)sizeof(TC));
    constexpr bool kGrad = EPI == kEpiGeluGrad || EPI == kEpiGeluGradSave;
    constexpr bool kHasAux = kGrad || EPI == kEpiStore;
    // The epilogue's operand (the pre-activation, or the residual) is read
    // EXA row blocks ahead: the first EXA before the first row block is
    // transformed, then block i + EXA as block i starts, so its memory
    // latency is paid about once while only EXA + 1 row blocks of it occupy
    // registers.
    constexpr int EXA = NBM > 1 ? NBM / 2 : 1;
    bf16x4 ex[kHasAux ? NBM : 1][kHasAux ? NBN : 1];
    const bool has_aux = kHasAux && (kGrad || p.R);
    const bf16* ex_src = kGrad ? p.aux : p.R;
    const int64_t ex_ld = kGrad ? p.ldaux : p.ldr;
    const auto rx = rsrc(ex_src + m0 * ex_ld + n0, ex_ld, 2);
    auto load_ex = [&](int i) {
        if constexpr (kHasAux) {
#pragma unroll
            for (int j = 0; j < NBN; ++j)
                ex[i][j] = __builtin_bit_cast(
                    bf16x4, __builtin_amdgcn_raw_buffer_load_b64(rx, (lr + 16 * i) * (uint32_t)(ex_ld * 2) + cb2[j], 0, 0));
        }
    };
    if (has_aux) {
#pragma unroll
        for (int i = 0; i < EXA; ++i) load_ex(i);
    }
    // one row block of bf16 stores (or C's dtype) at offsets row + cb[j], non-temporal when asked
    auto store_row = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t row_off, const uint32_t (&cb)[NBN],
                         const f32x4 (&v)[NBN], bool as_f32) {
        if (p.nt_store) {
#pragma unroll
            for (int j = 0; j < NBN; ++j) {
                if (as_f32) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[j]), r, row_off + cb[j], 0, 2);
                else {
                    bf16x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) o[q] = static_cast<bf16>(v[j][q]);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), r, row_off + cb[j], 0, 2);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NBN; ++j) {
                if (as_f32) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[j]), r, row_off + cb[j], 0, 0);
                else {
                    bf16x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) o[q] = static_cast<bf16>(v[j][q]);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), r, row_off + cb[j], 0, 0);
                }
            }
        }
    };
    __amdgpu_buffer_rsrc_t r_mean = rc, r_rstd = rc, r_csum = rc;
    if constexpr (LN) {
        r_mean = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.mean + m0), (short)0, (int)(rows_t * 4), 0x00020000);
        r_rstd = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.rstd + m0), (short)0, (int)(rows_t * 4), 0x00020000);
        r_csum = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.csum + n0), (short)0, (int)(cols_t * 4), 0x00020000);
    }
#pragma unroll
    for (int i = 0; i < NBM; ++i) {
        if (has_aux && i + EXA < NBM) load_ex(i + EXA);
        const uint32_t row = lr + 16 * i;
        f32x4 v[NBN];
#pragma unroll
        for (int j = 0; j < NBN; ++j) {
            // the empty asm orders this read after the s_nop padding that
            // follows the last MFMAs (volatile asm keeps its order; a plain
            // register copy could be hoisted above the padding)
            asm volatile("" : "+a"(acc[i][j]));
            v[j] = acc[i][j];
        }
        if constexpr (LN) {
            const float rs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_rstd, row * 4u, 0, 0));
            const float rm = rs * __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_mean, row * 4u, 0, 0));
#pragma unroll
            for (int j = 0; j < NBN; ++j) {
                const f32x4 cs = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(r_csum, (lc + 16 * j) * 4u, 0, 0));
#pragma unroll
                for (int r = 0; r < 4; ++r) v[j][r] = __builtin_fmaf(rs, v[j][r], -rm * cs[r]);
            }
        }
        if constexpr (EPI == kEpiGelu || EPI == kEpiGeluSave) {
            if constexpr (EPI == kEpiGeluSave)  // the pre-activation, kept for a backward pass
                store_row(rsrc(p.preact + m0 * p.ldc + n0, p.ldc, 2), row * (uint32_t)(p.ldc * 2), cb2, v, false);
            gelu_tanh_staged(v);
        } else if constexpr (kGrad) {
            if constexpr (EPI == kEpiGeluGradSave) {
                // GeLU of the pre-activation (the forward's H), for the
                // gradient of the second weight, from the same sigmoid as
                // the derivative
                f32x4 h[NBN];
#pragma unroll
                for (int j = 0; j < NBN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = static_cast<float>(ex[i][j][r]);
                        const float sg = gelu_sigmoid(x, x * x);
                        h[j][r] = x * sg;
                        v[j][r] *= gelu_grad_from(x, x * x, sg);
                    }
                store_row(rsrc(p.gelu_out + m0 * p.ldc + n0, p.ldc, 2), row * (uint32_t)(p.ldc * 2), cb2, h, false);
            } else {
#pragma unroll
                for (int j = 0; j < NBN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[j][r] *= gelu_tanh_grad(static_cast<float>(ex[i][j][r]));
            }
        } else {
            if (p.R) {
#pragma unroll
                for (int j = 0; j < NBN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[j][r] += static_cast<float>(ex[i][j][r]);
            }
        }
        // A large output (H of the big workloads) is written non-temporally:
        // it would not fit the caches anyway, and keeping it out of them
        // keeps the operands resident in the Infinity Cache.  A small one
        // stays cached for its reader.
        if constexpr (kStage) {
            // lane l: row 16 i + (l & 15), columns 16 j + 4 (l >> 4) .. +3 of the wave's block
            uint8_t* st = ring + w * C::OUT_WAVE + (16 * i + (lane & 15)) * C::OUT_PITCH + 8 * (lane >> 4);
#pragma unroll
            for (int j = 0; j < NBN; ++j) {
                bf16x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = static_cast<bf16>(v[j][q]);
                *reinterpret_cast<bf16x4*>(st + 32 * j) = o;
            }
        } else {
            store_row(rc, row * (uint32_t)(p.ldc * sizeof(TC)), cbc, v, true);
        }
    }
    if constexpr (kStage) {
        // The wave's block back from LDS in whole rows: lane l reads 16 bytes
        // (8 columns) of row 4 q + l / CPR at chunk l % CPR, so one store
        // instruction writes whole 128-byte lines of RPI rows.  Rows at or
        // past M fall outside the resource; N is a multiple of 8, so a chunk
        // lies wholly below N or wholly at or past it (kOut).
        constexpr int CPR = BN / 16, RPI = 64 / CPR, NQ = (BM / 2) / RPI;
        const uint32_t c = (uint32_t)(lane % CPR), rq = (uint32_t)(lane / CPR);
        const uint32_t colo = (uint32_t)(wn * (BN / 2)) + 8 * c;
        const uint32_t cb = (int64_t)colo < cols_t ? colo * 2u : kOut;
        const uint8_t* src = ring + w * C::OUT_WAVE + rq * C::OUT_PITCH + 16 * c;
        const uint32_t r0 = (uint32_t)(wm * (BM / 2)) + rq;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const u32x4 d = *reinterpret_cast<const u32x4*>(src + q * RPI * C::OUT_PITCH);
            const uint32_t off = (r0 + q * RPI) * (uint32_t)(p.ldc * 2) + cb;
            if (p.nt_store) __builtin_amdgcn_raw_buffer_store_b128(d, rc, off, 0, 2);
            else __builtin_amdgcn_raw_buffer_store_b128(d, rc, off, 0, 0);
        }
    }
}

template <class C, int EPI, typename TC, int KM = 0>
hipError_t launch_typed(const GemmArgs& g, int splits, hipStream_t stream) {
    FastParams p;
    p.A = static_cast<const bf16*>(g.A); p.lda = g.lda;
    p.B = static_cast<const bf16*>(g.B); p.ldb = g.ldb;
    p.M = (int)g.M; p.N = (int)g.N; p.K = (int)g.K;
    p.C = g.C; p.ldc = g.ldc;
    p.R = static_cast<const bf16*>(g.R); p.ldr = g.ldr;
    p.mean = g.ln_mean; p.rstd = g.ln_rstd; p.csum = g.ln_csum;
    p.aux = static_cast<const bf16*>(g.aux); p.ldaux = g.ldaux;
    p.preact = static_cast<bf16*>(g.preact_out);
    p.gelu_out = static_cast<bf16*>(g.gelu_out);
    p.tiles_m = (int)((g.M + C::BM - 1) / C::BM);
    p.tiles_n = (int)((g.N + C::BN - 1) / C::BN);
    p.group = 4;
    p.nt_store = g.M * g.N * (int64_t)sizeof(TC) > ((int64_t)128 << 20);
    p.splits = splits;
    p.c_split_stride = splits > 1 ? g.M * g.N : 0;
    const unsigned blocks = (unsigned)(p.tiles_m * p.tiles_n * splits);
    // the LayerNorm epilogue exists for the forward's epilogues only (the
    // GeLU-derivative ones never see a LayerNorm)
    constexpr bool kLnVariant = KM == 0 && EPI != kEpiGeluGrad && EPI != kEpiGeluGradSave;
    if constexpr (kLnVariant) {
        if (g.ln_mean) {
            gemm_bf16_mfma<C, EPI, true, TC, 0><<<dim3(blocks), dim3(256), 0, stream>>>(p);
            return hipGetLastError();
        }
    } else {
        if (g.ln_mean) return hipErrorInvalidValue;
    }
    gemm_bf16_mfma<C, EPI, false, TC, KM><<<dim3(blocks), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// CUs of the current device (queried once; 256 on MI355X).
int device_cu_count() {
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 256;
        return n;
    }();
    return cus;
}
static int device_cus() { return device_cu_count(); }

// Tile configurations (0: not for the MFMA kernel).
enum TileCfg { kCfgNone = 0, kCfg256 = 1, kCfg128 = 2, kCfg128x64 = 3, kCfg64 = 4 };
struct CfgInfo {
    int bm, bn;
    int per_cu;     // workgroups a CU holds at once (LDS)
    double step1;   // time of one 64-deep K step of a tile alone on its CU, relative to 256x256
    double step2;   // time of one K step of a round with per_cu tiles on each CU (= step1 if per_cu = 1)
};
// Measured on MI355X (K steps of the h1024 and Post-LN GEMMs, store and GeLU
// epilogues): a 128x128 tile alone on a CU takes 0.44 of a 256x256 step, two
// together 0.515; 128x64 (one per CU, deeper ring) 0.26; 64x64 alone 0.215,
// two together 0.31.
static CfgInfo cfg_info(int c) {
    switch (c) {
        case kCfg256: return {256, 256, 1, 1.0, 1.0};
        case kCfg128: return {128, 128, 2, 0.44, 0.515};
        case kCfg128x64: return {128, 64, 1, 0.26, 0.26};
        case kCfg64: return {64, 64, 2, 0.215, 0.31};
        default: return {0, 0, 0, 0.0, 0.0};
    }
}

// Whether the MFMA kernel can take a shape with a given tile: bf16 operands,
// K a whole number of 64-wide steps, 16-byte aligned rows, one operand tile's
// byte offsets below 2^31 (32-bit lane offsets), and, with the LayerNorm
// epilogue, the column sums of Bop.  M and N may be ragged (row-major
// operands only); N must be a multiple of 4 (the epilogue's quads).
// K-major operands: both at once (the backward's weight gradients), with
// the store epilogue, without LayerNorm or the pre-activation stash, on whole
// tiles of at least 128.  The GeLU output of the GeLU-derivative epilogue
// goes with that epilogue only.
static bool fits_cfg(const GemmArgs& g, int cfg) {
    const CfgInfo ci = cfg_info(cfg);
    if (!ci.bm) return false;
    if (g.ab_dtype != kBF16) return false;
    if (g.M <= 0 || g.N <= 0 || g.K <= 0) return false;
    if (g.K % BK || g.N % 4 || (g.c_dtype == kBF16 && g.N % 8)) return false;
    const bool km = g.a_kmajor || g.b_kmajor;
    if (km && (ci.bm < 128 || ci.bn < 128 || g.M % ci.bm || g.N % ci.bn)) return false;
    if (g.lda % 8 || g.ldb % 8 || !aligned16(g.A) || !aligned16(g.B)) return false;
    // 32-bit lane offsets: a tile's rows of a row-major operand, or all K rows of a K-major one
    if ((g.a_kmajor ? g.K : ci.bm) * g.lda * 2 >= ((int64_t)1 << 31)) return false;
    if ((g.b_kmajor ? g.K : ci.bn) * g.ldb * 2 >= ((int64_t)1 << 31)) return false;
    if (g.a_kmajor != g.b_kmajor) return false;
    if (g.a_kmajor && (g.epi != kEpiStore || g.ln_mean || g.preact_out)) return false;
    const int64_t tiles = ((g.M + ci.bm - 1) / ci.bm) * ((g.N + ci.bn - 1) / ci.bn);
    if (tiles * 8 >= ((int64_t)1 << 31) || g.M >= ((int64_t)1 << 31) || g.N >= ((int64_t)1 << 31) ||
        g.K >= ((int64_t)1 << 31))
        return false;
    if (g.ln_mean && !g.ln_csum) return false;
    // the epilogue moves four consecutive columns per lane: 16-byte (fp32)
    // or 8-byte (bf16) stores and residual loads, 16-byte column-sum loads,
    // all through buffer resources of one tile's rows (offsets below 2^31)
    const int64_t c_es = g.c_dtype == kF32 ? 4 : 2;
    if (ci.bm * g.ldc * c_es >= ((int64_t)1 << 31) || (g.R && ci.bm * g.ldr * 2 >= ((int64_t)1 << 31)) ||
        (g.aux && ci.bm * g.ldaux * 2 >= ((int64_t)1 << 31)) || g.N * 4 >= ((int64_t)1 << 31))
        return false;
    if (g.ldc % 4 || (reinterpret_cast<uintptr_t>(g.C) & (4 * c_es - 1))) return false;
    if (g.R && (g.ldr % 4 || (reinterpret_cast<uintptr_t>(g.R) & 7))) return false;
    if (g.ln_mean && !aligned16(g.ln_csum)) return false;
    if (g.epi == kEpiGeluGrad && (!g.aux || g.ldaux % 4 || (reinterpret_cast<uintptr_t>(g.aux) & 7) ||
                                  g.c_dtype != kBF16))
        return false;
    if (g.preact_out && (reinterpret_cast<uintptr_t>(g.preact_out) & 7)) return false;
    if (g.gelu_out && (g.epi != kEpiGeluGrad || (reinterpret_cast<uintptr_t>(g.gelu_out) & 7))) return false;
    return true;
}

// Modelled time of a GEMM on tile configuration cfg: with no more tiles than
// CUs, one round of tiles alone on their CUs; otherwise rounds of
// (CUs x workgroups per CU) tiles, the last, partial round costing its share
// (a round of fine tiles is balanced by the hardware's dispatch, a partial
// round of 256x256 tiles costs as much as a full one).
static double cfg_cost(const GemmArgs& g, int cfg) {
    const CfgInfo ci = cfg_info(cfg);
    const double cus = (double)device_cus();
    const double tiles = (double)((g.M + ci.bm - 1) / ci.bm) * (double)((g.N + ci.bn - 1) / ci.bn);
    double per_step;
    if (tiles <= cus) {
        per_step = ci.step1;
    } else {
        const double slots = cus * ci.per_cu;
        const double rounds = cfg == kCfg256 ? std::ceil(tiles / slots) : std::max(1.0, tiles / slots);
        per_step = rounds * ci.step2;
    }
    return per_step * (double)(g.K / BK);
}

static int choose_cfg(const GemmArgs& g) {
    int best = kCfgNone;
    double best_cost = 0.0;
    for (int c : {kCfg256, kCfg128, kCfg128x64, kCfg64}) {
        if (!fits_cfg(g, c)) continue;
        const double cost = cfg_cost(g, c);
        if (best == kCfgNone || cost < best_cost) {  // ties keep the larger tile (better L2 reuse)
            best = c;
            best_cost = cost;
        }
    }
    return best;
}

GemmPath choose_gemm_path(const GemmArgs& g) { return choose_cfg(g) ? kPathFastBf16 : kPathGeneric; }

// Split-K plan: only a GEMM that allows it (GemmArgs::allow_split: the
// backward's weight gradients and the attention projections, never the
// forward's shard sum), with a plain store epilogue and no LayerNorm, whose
// output tiles fill at most a quarter of the workgroup slots, runs its K loop
// as S equal ranges, S the largest power of two (at most 8) that keeps
// tiles x S within the slots and each range a whole number (at least three)
// of 64-wide steps.  Each range writes fp32 partial sums; split_reduce_kernel
// adds them in range order.
static int split_count(const GemmArgs& g, int cfg) {
    if (!g.allow_split || g.epi != kEpiStore || g.ln_mean) return 1;
    const CfgInfo ci = cfg_info(cfg);
    const int64_t tiles = ((g.M + ci.bm - 1) / ci.bm) * ((g.N + ci.bn - 1) / ci.bn);
    const int64_t slots = (int64_t)device_cus() * ci.per_cu;
    if (tiles * 4 > slots) return 1;  // at least a quarter of the slots busy: no split
    int s = 1;
    while (s < 8 && tiles * s * 2 <= slots && g.K % (2 * s * BK) == 0 && g.K / (2 * s) >= 3 * BK) s *= 2;
    return s;
}

size_t gemm_split_bytes(const GemmArgs& g) {
    const int cfg = choose_cfg(g);
    if (!cfg) return 0;
    const int s = split_count(g, cfg);
    return s > 1 ? (size_t)s * (size_t)g.M * (size_t)g.N * sizeof(float) : 0;
}

namespace {

// C[m][n] = sum over r = 0..S-1, in that order, of part[r][m][n] (+ R[m][n]),
// rounded to C's dtype: the epilogue of a split GEMM.  Four columns per
// thread (N is a multiple of 4).
template <typename TC>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int S, int64_t M,
                                                          int64_t N, const bf16* __restrict__ R, int64_t ldr,
                                                          TC* __restrict__ C, int64_t ldc) {
    const int64_t quads = M * N / 4;
    const int64_t slice = M * N;
    for (int64_t qi = (int64_t)blockIdx.x * 256 + threadIdx.x; qi < quads; qi += (int64_t)gridDim.x * 256) {
        const int64_t e = qi * 4;
        const int64_t m = e / N, n = e - m * N;
        f32x4 v = *reinterpret_cast<const f32x4*>(part + e);
        for (int r = 1; r < S; ++r) v += *reinterpret_cast<const f32x4*>(part + r * slice + e);
        if (R) {
            const bf16x4 rv = *reinterpret_cast<const bf16x4*>(R + m * ldr + n);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] += static_cast<float>(rv[k]);
        }
        if constexpr (std::is_same<TC, float>::value) {
            *reinterpret_cast<f32x4*>(C + m * ldc + n) = v;
        } else {
            bf16x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = static_cast<bf16>(v[k]);
            *reinterpret_cast<bf16x4*>(C + m * ldc + n) = o;
        }
    }
}

}  // namespace

// Store epilogue, with the split-K plan when it applies.
template <class C, int KM>
static hipError_t launch_store(const GemmArgs& g, int cfg, hipStream_t stream) {
    const int s = split_count(g, cfg);
    if (s > 1) {
        // K ranges write fp32 partials, then one pass sums them
        GemmArgs gp = g;
        gp.C = g.split_ws;
        gp.ldc = g.N;
        gp.c_dtype = kF32;
        gp.R = nullptr;
        hipError_t e = launch_typed<C, kEpiStore, float, KM>(gp, s, stream);
        if (e != hipSuccess) return e;
        const int64_t quads = g.M * g.N / 4;
        const unsigned blocks = (unsigned)std::min<int64_t>((quads + 255) / 256, 8 * (int64_t)device_cus());
        const float* part = static_cast<const float*>(g.split_ws);
        const bf16* R = static_cast<const bf16*>(g.R);
        if (g.c_dtype == kF32)
            split_reduce_kernel<float><<<dim3(blocks), dim3(256), 0, stream>>>(part, s, g.M, g.N, R, g.ldr,
                                                                            static_cast<float*>(g.C), g.ldc);
        else
            split_reduce_kernel<bf16><<<dim3(blocks), dim3(256), 0, stream>>>(part, s, g.M, g.N, R, g.ldr,
                                                                           static_cast<bf16*>(g.C), g.ldc);
        return hipGetLastError();
    }
    return g.c_dtype == kF32 ? launch_typed<C, kEpiStore, float, KM>(g, 1, stream)
                             : launch_typed<C, kEpiStore, bf16, KM>(g, 1, stream);
}

// Both operands K-major (fits_cfg admits them with the store epilogue and
// no LayerNorm), on the two square tiles.
template <class C>
static hipError_t launch_kmajor(const GemmArgs& g, int cfg, hipStream_t stream) {
    return launch_store<C, 3>(g, cfg, stream);
}

template <class C>
static hipError_t launch_rowmajor(const GemmArgs& g, int cfg, hipStream_t stream) {
    if (g.epi == kEpiGelu)
        return g.preact_out ? launch_typed<C, kEpiGeluSave, bf16>(g, 1, stream)
                            : launch_typed<C, kEpiGelu, bf16>(g, 1, stream);
    if (g.epi == kEpiGeluGrad)
        return g.gelu_out ? launch_typed<C, kEpiGeluGradSave, bf16>(g, 1, stream)
                          : launch_typed<C, kEpiGeluGrad, bf16>(g, 1, stream);
    return launch_store<C, 0>(g, cfg, stream);
}

hipError_t launch_gemm_bf16_fast(const GemmArgs& g, hipStream_t stream) {
    const int cfg = choose_cfg(g);
    if (!cfg) return hipErrorInvalidValue;
    if (gemm_split_bytes(g) > 0 && (!g.split_ws || g.split_ws_bytes < gemm_split_bytes(g) ||
                                    (reinterpret_cast<uintptr_t>(g.split_ws) & 15)))
        return hipErrorInvalidValue;
    if (g.a_kmajor || g.b_kmajor)
        return cfg == kCfg256 ? launch_kmajor<C256>(g, cfg, stream) : launch_kmajor<C128>(g, cfg, stream);
    switch (cfg) {
        case kCfg256: return launch_rowmajor<C256>(g, cfg, stream);
        case kCfg128: return launch_rowmajor<C128>(g, cfg, stream);
        case kCfg128x64: return launch_rowmajor<C128x64>(g, cfg, stream);
        default: return launch_rowmajor<C64>(g, cfg, stream);
    }
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    if (choose_gemm_path(g) == kPathFastBf16) return launch_gemm_bf16_fast(g, stream);
    return launch_gemm_generic(g, stream);
}

}  // namespace tpmlp
