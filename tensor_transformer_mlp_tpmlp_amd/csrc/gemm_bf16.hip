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
//     Bop = packed B^T; the K loop runs over every shard's rows, so all
//     partials Y_i are summed in the same fp32 accumulator and never leave
//     the chip.
//
// Tiling: one 256x256 output tile per workgroup of 4 waves (2x2, one wave per
// SIMD), each wave owning a 128x128 sub-tile: 8x8 MFMA blocks of 16x16, 256
// fp32 accumulators per lane held in AGPRs.  Shapes too small to fill the GPU
// with 256x256 tiles use 128x128 tiles (4x4 blocks per wave, 80 KiB of LDS,
// two workgroups per CU) with the same pipeline.  K advances 64 per step;
// each operand's 64-wide slice of a step is a "unit" (32 KiB at 256x256),
// and a ring of five unit slots fills the 160 KiB of LDS.
//
// The 16x16x32 MFMA is used rather than 32x32x16: with random operands it
// sustains a higher clock under the chip's power limit for the same FLOP.
// Each MFMA takes the Bop fragment as its first operand, so a lane's four
// accumulators are four consecutive output columns of one row: the epilogue
// writes 8 (bf16) or 16 (fp32) contiguous bytes per lane and block.
//
// Global -> LDS moves use the direct-to-LDS buffer load (buffer_load_dwordx4
// ... lds): no VGPR staging and no ds_write.  Lane L of a wave's load lands at
// LDS base + 16 L, so the XOR swizzle of the LDS layout is applied on the
// global side by choosing which 16-byte chunk each lane fetches.
//
// Pipeline: step t computes two 32-deep sub-steps from units A_t and B_t.
// Sub-step 0 reads the fragments of sub-step 1 and issues the loads of
// A_{t+2}; a barrier then publishes A_{t+1}, B_{t+1} and frees A_t, B_t;
// sub-step 1 reads the next step's first fragments and issues B_{t+2} into
// A_t's slot.  Each load covers whole 128-byte lines (8 rows x 128 bytes),
// the unit the L1 fetches from L2 in, so a step costs the CU's load path the
// fewest requests; loads and reads are spread evenly between the MFMAs.  A
// load of B has more than one sub-step, a load of A more than two, to land.
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

// WB: the tile is 64*WB square; 4 gives 256x256 (128x128 per wave), 2 gives
// 128x128 (64x64 per wave), used when 256x256 tiles would leave CUs idle.
// K advances BK = 64 per step, two 16x16x32 MFMA sub-steps.  The operands
// of a step live in LDS as two "units", one per operand (M rows of 128
// bytes), in a ring of NUNIT unit slots.
constexpr int BK = 64;
constexpr int NUNIT = 5;
template <int WB> struct Tile {
    static constexpr int M = 64 * WB;             // tile rows (= tile columns)
    static constexpr int UNIT_BYTES = M * BK * 2;  // one operand of one step
    static constexpr int NB = 2 * WB;             // 16x16 MFMA blocks per wave per side
    static constexpr int LPU = M / 32;            // direct loads per wave per unit
};

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
// distinct 32-byte bank groups.
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

template <int WB, int EPI, bool LN, typename TC, int KM>
__global__ __launch_bounds__(256) void gemm_bf16_mfma(FastParams p) {
    constexpr bool KA = (KM & 1) != 0, KB = (KM & 2) != 0;  // operand stored K-major
    constexpr int BM = Tile<WB>::M, BN = Tile<WB>::M;
    constexpr int NB = Tile<WB>::NB;
    constexpr int UB = Tile<WB>::UNIT_BYTES;
    constexpr int LPU = Tile<WB>::LPU;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NUNIT * UB];

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

    // Buffer resources over this tile's rows of each operand, from its K range
    // on; a K-major operand's resource starts at row k0, column m0 (n0) and
    // runs to the end of the operand.
    const uint32_t a_bytes = KA ? (uint32_t)((p.K - k0) * p.lda * 2 - m0 * 2) : (uint32_t)(BM * p.lda * 2 - k0 * 2);
    const uint32_t b_bytes = KB ? (uint32_t)((p.K - k0) * p.ldb * 2 - n0 * 2) : (uint32_t)(BN * p.ldb * 2 - k0 * 2);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(KA ? p.A + k0 * p.lda + m0 : p.A + m0 * p.lda + k0), (short)0, (int)a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(KB ? p.B + k0 * p.ldb + n0 : p.B + n0 * p.ldb + k0), (short)0, (int)b_bytes, 0x00020000);

    // Wave w fills rows [w BM/4, (w+1) BM/4) of a unit with LPU loads of 8
    // rows (1 KiB); in load q, lane L fills row w BM/4 + 8 q + L/8 at physical
    // chunk L % 8, which must hold logical chunk (L % 8) ^ key(row), and
    // row % 16 = 8 (q & 1) + L/8 since BM/4 is a multiple of 16.
    const uint32_t lrow = (uint32_t)(w * (BM / 4) + (lane >> 3));
    const uint32_t cx0 = ((uint32_t)(lane & 7) ^ lds_key((uint32_t)lane >> 3)) << 4;
    const uint32_t cx1 = ((uint32_t)(lane & 7) ^ lds_key(8u + ((uint32_t)lane >> 3))) << 4;
    const uint32_t a_v0 = lrow * (uint32_t)(p.lda * 2) + cx0, a_v1 = a_v0 - cx0 + cx1;
    const uint32_t b_v0 = lrow * (uint32_t)(p.ldb * 2) + cx0, b_v1 = b_v0 - cx0 + cx1;
    const uint32_t a_qstep = (uint32_t)(8 * p.lda * 2);
    const uint32_t b_qstep = (uint32_t)(8 * p.ldb * 2);
    const uint32_t dst_w = (uint32_t)(w * (BM / 4) * 128);

    // slot s of the ring
    auto slot = [&](int s) { return ring + s * UB; };

    // the same resources as SGPR dwords for the inline-assembly loads
    u32x4 ra4 = {}, rb4 = {};
    if constexpr (KM != 0) {
        ra4 = buffer_rsrc_sgpr(KA ? p.A + k0 * p.lda + m0 : p.A + m0 * p.lda + k0, a_bytes);
        rb4 = buffer_rsrc_sgpr(KB ? p.B + k0 * p.ldb + n0 : p.B + n0 * p.ldb + k0, b_bytes);
    }

    // K-major operand units: 64 rows (k) of RB = 2 BM bytes (the tile's columns),
    // 16-byte chunk c of row r at physical chunk c ^ kswz(r).  Wave w fills
    // rows 16 w .. 16 w + 15 with LPU loads of 1 KiB; in load q lane L lands at
    // row 16 w + q RPL + L / CPR, physical chunk L % CPR.
    constexpr int RB = BM * 2, CPR = RB / 16, RPL = 64 / CPR;
    uint32_t kv_a[KA ? LPU : 1], kv_b[KB ? LPU : 1];
#pragma unroll
    for (int q = 0; q < LPU; ++q) {
        const uint32_t r = (uint32_t)(16 * w + q * RPL + lane / CPR);
        const uint32_t c = ((uint32_t)(lane % CPR) ^ kswz(r)) << 4;
        if constexpr (KA) kv_a[q] = r * (uint32_t)(p.lda * 2) + c;
        if constexpr (KB) kv_b[q] = r * (uint32_t)(p.ldb * 2) + c;
    }

    // load q of the unit of operand `op` (0 = Aop, 1 = Bop) at k0 into slot st
    // (with a K-major operand every load goes through dma16_asm, since the
    // transposing reads would wait for any direct load the compiler sees)
    auto load_one = [&](uint8_t* st, int op, int k0, int q) {
        const uint32_t kb = (uint32_t)k0 * 2u;
        uint8_t* dst = st + dst_w + q * 1024;
        const __amdgpu_buffer_rsrc_t r = op ? rb : ra;
        uint32_t voff, soff;
        if (op) {
            if constexpr (KB) { voff = kv_b[q]; soff = (uint32_t)k0 * (uint32_t)(p.ldb * 2); }
            else { voff = (q & 1) ? b_v1 : b_v0; soff = kb + q * b_qstep; }
        } else {
            if constexpr (KA) { voff = kv_a[q]; soff = (uint32_t)k0 * (uint32_t)(p.lda * 2); }
            else { voff = (q & 1) ? a_v1 : a_v0; soff = kb + q * a_qstep; }
        }
        if constexpr (KM != 0) dma16_asm(dst, op ? rb4 : ra4, voff, soff);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
    };
    auto load_unit = [&](uint8_t* st, int op, int k0) {
#pragma unroll
        for (int q = 0; q < LPU; ++q) load_one(st, op, k0, q);
    };

    // MFMA operand reads: a 16x16x32 fragment is 16 rows x 32 k; in sub-step
    // kk lane l reads row (l & 15) of the block at logical chunk
    // 4 kk + (l >> 4).  The same lane -> k assignment for both operands makes
    // each MFMA a plain 32-long dot product per output.
    const uint32_t kr = lds_key((uint32_t)lane & 15);
    const uint32_t rd_a = (uint32_t)((wm * 16 * NB + (lane & 15)) * 128);
    const uint32_t rd_b = (uint32_t)((wn * 16 * NB + (lane & 15)) * 128);
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
    uint32_t kf_a[KA ? NB : 1], kf_b[KB ? NB : 1];
    {
        const uint32_t li = (uint32_t)lane & 15, g = (uint32_t)lane >> 4;
        const uint32_t row = 8 * g + (li >> 2);
        const uint32_t sw = kswz(row);
#pragma unroll
        for (int f = 0; f < NB; ++f) {
            const uint32_t col_a = (uint32_t)(wm * 16 * NB + 16 * f) + 4 * (li & 3);
            const uint32_t col_b = (uint32_t)(wn * 16 * NB + 16 * f) + 4 * (li & 3);
            if constexpr (KA) kf_a[f] = row * RB + ((((col_a >> 3) ^ sw)) << 4) + ((col_a & 7) << 1);
            if constexpr (KB) kf_b[f] = row * RB + ((((col_b >> 3) ^ sw)) << 4) + ((col_b & 7) << 1);
        }
    }
    auto read_frag = [&](const uint8_t* unit, uint32_t off, int kk) -> bf16x8 {
        const uint8_t* q = unit + off + kk * 32 * RB;
        const v4s lo = lds_read_tr16(q);
        const v4s hi = lds_read_tr16(q + 4 * RB);
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
    f32x4 acc[NB][NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            acc[i][j] = f32x4{};
            asm volatile("" : "+a"(acc[i][j]));
        }
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");

    bf16x8 fa0[NB], fb0[NB], fa1[NB], fb1[NB];
    const int nk = kc / BK;
    __builtin_assume(nk >= 3);

    // Per sub-step: NM MFMAs; the NR fragment reads of the next sub-step go
    // one after every RS-th MFMA from the first, the LPU direct loads of one
    // unit one after every LS-th.
    constexpr int NM = NB * NB, NR = 2 * NB, RS = NM / NR / 2 > 0 ? NM / NR / 2 : 1;
    constexpr int LS = NM / LPU;
    static_assert(NM % LPU == 0 && (NR - 1) * RS < NM, "sub-step layout");

    // One sub-step: MFMAs on (fc, gc); read the next fragments at chunk
    // offset ch from units ua (Aop) and ub (Bop) into (fn, gn); when
    // `load_op` >= 0, issue the unit of operand load_op at k_load into slot
    // `dst`.
    auto frag_a = [&](const uint8_t* ua, uint32_t ch, int kk, int f) -> bf16x8 {
        if constexpr (KA) return read_frag(ua, kf_a[f], kk);
        else return *reinterpret_cast<const bf16x8*>(ua + rd_a + ch + f * 2048);
    };
    auto frag_b = [&](const uint8_t* ub, uint32_t ch, int kk, int f) -> bf16x8 {
        if constexpr (KB) return read_frag(ub, kf_b[f], kk);
        else return *reinterpret_cast<const bf16x8*>(ub + rd_b + ch + f * 2048);
    };
    auto sub_step = [&](const bf16x8 (&fc)[NB], const bf16x8 (&gc)[NB], const uint8_t* ua, const uint8_t* ub,
                        uint32_t ch, int kk, bf16x8 (&fn)[NB], bf16x8 (&gn)[NB], bool do_read, uint8_t* dst,
                        int load_op, int k_load) {
#pragma unroll
        for (int idx = 0; idx < NM; ++idx) {
            const int i = idx / NB, j = idx % NB;
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(gc[j]), "v"(fc[i]));
            if (do_read && idx % RS == 0 && idx / RS < NR) {
                // fragment reads in consumption order: Aop 0, Bop 0..NB-1, Aop 1..NB-1
                const int r = idx / RS;
                if (r == 0) fn[0] = frag_a(ua, ch, kk, 0);
                else if (r <= NB) gn[r - 1] = frag_b(ub, ch, kk, r - 1);
                else fn[r - NB] = frag_a(ua, ch, kk, r - NB);
            }
            if (load_op >= 0 && idx % LS == 0) load_one(dst, load_op, k_load, idx / LS);
        }
    };

    // Step t reads units A_t, B_t (ring slots 2t, 2t+1 mod NUNIT).  Sub-step
    // 0 issues A_{t+2} into the slot of B_{t-1}; the barrier between the
    // sub-steps publishes A_{t+1}, B_{t+1} and frees A_t, B_t; sub-step 1
    // issues B_{t+2} into the slot of A_t.  A load of B has more than one
    // sub-step, a load of A more than two, to land before the barrier that
    // publishes it.
    auto next = [](int s, int d) { s += d; return s >= NUNIT ? s - NUNIT : s; };
    auto barrier_wait = [&](auto vm_left) {
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(decltype(vm_left)::value));
        __builtin_amdgcn_s_barrier();
    };

    // prologue: units A_0, B_0, A_1, B_1, A_2 into slots 0..4; wait for step 0
    load_unit(slot(0), 0, 0);
    load_unit(slot(1), 1, 0);
    load_unit(slot(2), 0, BK);
    load_unit(slot(3), 1, BK);
    load_unit(slot(4), 0, 2 * BK);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * LPU));
    __builtin_amdgcn_s_barrier();
    {
        fa0[0] = frag_a(slot(0), ch0, 0, 0);
#pragma unroll
        for (int j = 0; j < NB; ++j) fb0[j] = frag_b(slot(1), ch0, 0, j);
#pragma unroll
        for (int i = 1; i < NB; ++i) fa0[i] = frag_a(slot(0), ch0, 0, i);
    }

    // step 0: A_2 is already in flight
    sub_step(fa0, fb0, slot(0), slot(1), ch1, 1, fa1, fb1, true, nullptr, -1, 0);
    barrier_wait(ic<LPU>{});
    sub_step(fa1, fb1, slot(2), slot(3), ch0, 0, fa0, fb0, true, slot(0), 1, 2 * BK);

    // steps 1 .. nk-3
    int sa = 2;  // slot of A_t
    for (int kt = 1; kt + 2 < nk; ++kt) {
        const int sb = next(sa, 1), sa1 = next(sa, 2), sb1 = next(sa, 3), sa2 = next(sa, 4);
        sub_step(fa0, fb0, slot(sa), slot(sb), ch1, 1, fa1, fb1, true, slot(sa2), 0, (kt + 2) * BK);
        barrier_wait(ic<LPU>{});
        sub_step(fa1, fb1, slot(sa1), slot(sb1), ch0, 0, fa0, fb0, true, slot(sa), 1, (kt + 2) * BK);
        sa = sa1;
    }
    // step nk-2: nothing left to load
    {
        const int sb = next(sa, 1), sa1 = next(sa, 2), sb1 = next(sa, 3);
        sub_step(fa0, fb0, slot(sa), slot(sb), ch1, 1, fa1, fb1, true, nullptr, -1, 0);
        barrier_wait(ic<0>{});
        sub_step(fa1, fb1, slot(sa1), slot(sb1), ch0, 0, fa0, fb0, true, nullptr, -1, 0);
        sa = sa1;
    }
    // step nk-1
    sub_step(fa0, fb0, slot(sa), slot(next(sa, 1)), ch1, 1, fa1, fb1, true, nullptr, -1, 0);
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
    sub_step(fa1, fb1, slot(sa), slot(sa), ch0, 0, fa0, fb0, false, nullptr, -1, 0);
    // results of the last MFMAs are read by the epilogue
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // Epilogue: lane l writes row m = ... + (l & 15) of block i, columns
    // n .. n+3 with n = ... + 4 (l >> 4) of block j.  A whole row block is
    // transformed before it is stored, which gives the scheduler NB * 4
    // independent GeLU chains to interleave.
    TC* __restrict__ C = static_cast<TC*>(p.C) + kz * p.c_split_stride;
    const int64_t n_base = n0 + wn * 16 * NB + 4 * (lane >> 4);
    const int64_t m_base = m0 + wm * 16 * NB + (lane & 15);
    // The epilogue's operand (the pre-activation, or the residual) is read
    // for the whole wave tile before the first row block is transformed, so
    // its memory latency is paid once rather than once per row block.
    constexpr bool kGrad = EPI == kEpiGeluGrad || EPI == kEpiGeluGradSave;
    constexpr bool kHasAux = kGrad || EPI == kEpiStore;
    bf16x4 ex[kHasAux ? NB : 1][kHasAux ? NB : 1];
    if constexpr (kGrad) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                ex[i][j] = *reinterpret_cast<const bf16x4*>(p.aux + (m_base + i * 16) * p.ldaux + n_base + j * 16);
    } else if constexpr (EPI == kEpiStore) {
        if (p.R) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    ex[i][j] = *reinterpret_cast<const bf16x4*>(p.R + (m_base + i * 16) * p.ldr + n_base + j * 16);
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int64_t m = m_base + i * 16;
        f32x4 v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) v[j] = acc[i][j];
        if constexpr (LN) {
            const float rs = p.rstd[m];
            const float rm = rs * p.mean[m];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const f32x4 cs = *reinterpret_cast<const f32x4*>(p.csum + n_base + j * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) v[j][r] = __builtin_fmaf(rs, v[j][r], -rm * cs[r]);
            }
        }
        if constexpr (EPI == kEpiGelu || EPI == kEpiGeluSave) {
            if constexpr (EPI == kEpiGeluSave) {
                // the pre-activation, kept for a backward pass
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(v[j][r]);
                    bf16x4* dst = reinterpret_cast<bf16x4*>(p.preact + m * p.ldc + n_base + j * 16);
                    if (p.nt_store) __builtin_nontemporal_store(o, dst);
                    else *dst = o;
                }
            }
            gelu_tanh_staged(v);
        } else if constexpr (kGrad) {
            if constexpr (EPI == kEpiGeluGradSave) {
                // GeLU of the pre-activation (the forward's H), for the
                // gradient of the second weight
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(gelu_tanh(static_cast<float>(ex[i][j][r])));
                    bf16x4* dst = reinterpret_cast<bf16x4*>(p.gelu_out + m * p.ldc + n_base + j * 16);
                    if (p.nt_store) __builtin_nontemporal_store(o, dst);
                    else *dst = o;
                }
            }
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[j][r] *= gelu_tanh_grad(static_cast<float>(ex[i][j][r]));
        } else {
            if (p.R) {
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[j][r] += static_cast<float>(ex[i][j][r]);
            }
        }
        // A large output (H of the big workloads) is written non-temporally:
        // it would not fit the caches anyway, and keeping it out of them
        // keeps the operands resident in the Infinity Cache.  A small one
        // stays cached for its reader.
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            TC* row = C + m * p.ldc + n_base + j * 16;
            if constexpr (std::is_same<TC, float>::value) {
                f32x4* dst = reinterpret_cast<f32x4*>(row);
                if (p.nt_store) __builtin_nontemporal_store(v[j], dst);
                else *dst = v[j];
            } else {
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(v[j][r]);
                bf16x4* dst = reinterpret_cast<bf16x4*>(row);
                if (p.nt_store) __builtin_nontemporal_store(o, dst);
                else *dst = o;
            }
        }
    }
}

template <int WB, int EPI, typename TC, int KM = 0>
hipError_t launch_typed(const GemmArgs& g, int splits, hipStream_t stream) {
    constexpr int BM = Tile<WB>::M, BN = Tile<WB>::M;
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
    p.tiles_m = (int)(g.M / BM);
    p.tiles_n = (int)(g.N / BN);
    p.group = 4;
    p.nt_store = g.M * g.N * (int64_t)sizeof(TC) > ((int64_t)128 << 20);
    p.splits = splits;
    p.c_split_stride = splits > 1 ? g.M * g.N : 0;
    const unsigned blocks = (unsigned)(p.tiles_m * p.tiles_n * splits);
    if constexpr (KM != 0)
        gemm_bf16_mfma<WB, EPI, false, TC, KM><<<dim3(blocks), dim3(256), 0, stream>>>(p);
    else if (g.ln_mean)
        gemm_bf16_mfma<WB, EPI, true, TC, 0><<<dim3(blocks), dim3(256), 0, stream>>>(p);
    else
        gemm_bf16_mfma<WB, EPI, false, TC, 0><<<dim3(blocks), dim3(256), 0, stream>>>(p);
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

// Whether the MFMA kernel can take a shape with tiles of 64*wb rows: bf16
// operands, M and N whole tiles, K a whole number (at least three) of
// 64-wide steps, 16-byte aligned rows, one operand tile's byte offsets below 2^31
// (buffer offsets), and, with the LayerNorm epilogue, the column sums of Bop.
// K-major operands: Bop alone (store or GeLU-derivative epilogue) or both
// (store epilogue), without LayerNorm or the pre-activation stash.  The
// GeLU output of the GeLU-derivative epilogue goes with that epilogue only.
static bool fits_tile(const GemmArgs& g, int wb) {
    const int64_t tm = 64 * wb;
    if (g.ab_dtype != kBF16) return false;
    if (g.M <= 0 || g.N <= 0 || g.K <= 0) return false;
    if (g.M % tm || g.N % tm || g.K % BK || g.K < 3 * BK) return false;
    if (g.lda % 8 || g.ldb % 8 || !aligned16(g.A) || !aligned16(g.B)) return false;
    // buffer offsets: a tile's rows of a row-major operand, or all K rows of a K-major one
    if ((g.a_kmajor ? g.K : tm) * g.lda * 2 >= ((int64_t)1 << 31)) return false;
    if ((g.b_kmajor ? g.K : tm) * g.ldb * 2 >= ((int64_t)1 << 31)) return false;
    if (g.a_kmajor && (!g.b_kmajor || g.epi != kEpiStore)) return false;
    if (g.b_kmajor && ((g.epi != kEpiStore && g.epi != kEpiGeluGrad) || g.ln_mean || g.preact_out)) return false;
    if ((g.M / tm) * (g.N / tm) >= ((int64_t)1 << 31) || g.M >= ((int64_t)1 << 31) ||
        g.N >= ((int64_t)1 << 31) || g.K >= ((int64_t)1 << 31))
        return false;
    if (g.ln_mean && !g.ln_csum) return false;
    // the epilogue moves four consecutive columns per lane: 16-byte (fp32)
    // or 8-byte (bf16) stores and residual loads, 16-byte column-sum loads
    const int64_t c_es = g.c_dtype == kF32 ? 4 : 2;
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

// Tile size: 256x256 (wb = 4, one workgroup per CU) or 128x128 (wb = 2, two
// per CU); 0 = not for the MFMA kernel.  With t 256x256 tiles on C CUs, the
// 256x256 plan takes ceil(t / C) rounds, a partial round lasting as long as
// a full one.  A round of 128x128 tiles does half the work of a 256x256
// round in 0.515 of its time (measured at K = 1024 on MI355X) and, its tiles
// being finer, a partial round costs about its share: 0.515 * 4 t / (2 C).
// The cheaper plan wins; 256x256 on a tie (its L2 reuse is better).
static int choose_wb(const GemmArgs& g) {
    const bool f4 = fits_tile(g, 4), f2 = fits_tile(g, 2);
    if (f4 && f2) {
        const double cus = (double)device_cus();
        const double t4 = (double)(g.M / 256) * (double)(g.N / 256);
        const double rounds4 = std::ceil(t4 / cus);
        const double rounds2 = 0.515 * 4.0 * t4 / (2.0 * cus);
        return rounds2 < rounds4 ? 2 : 4;
    }
    if (f2) return 2;
    if (f4) return 4;
    return 0;
}

GemmPath choose_gemm_path(const GemmArgs& g) { return choose_wb(g) ? kPathFastBf16 : kPathGeneric; }

// Split-K plan: a GEMM with a plain store epilogue and no LayerNorm whose
// output tiles fill at most a quarter of the workgroup slots (two per CU at
// 128x128, one at 256x256) runs its K loop as S equal ranges, S the largest
// power of two (at most 8) that keeps tiles x S within the slots and each
// range a whole number (at least three) of 64-wide steps.  Each range
// writes fp32 partial sums; split_reduce_kernel adds them in range order.
static int split_count(const GemmArgs& g, int wb) {
    if (g.epi != kEpiStore || g.ln_mean) return 1;
    const int64_t tm = 64 * wb;
    const int64_t tiles = (g.M / tm) * (g.N / tm);
    const int64_t slots = (int64_t)device_cus() * (wb == 2 ? 2 : 1);
    if (tiles * 4 > slots) return 1;
    int s = 1;
    while (s < 8 && tiles * s * 2 <= slots && g.K % (2 * s * BK) == 0 && g.K / (2 * s) >= 3 * BK) s *= 2;
    return s;
}

size_t gemm_split_bytes(const GemmArgs& g) {
    const int wb = choose_wb(g);
    if (!wb) return 0;
    const int s = split_count(g, wb);
    return s > 1 ? (size_t)s * (size_t)g.M * (size_t)g.N * sizeof(float) : 0;
}

namespace {

// C[m][n] = sum over r = 0..S-1, in that order, of part[r][m][n] (+ R[m][n]),
// rounded to C's dtype: the epilogue of a split GEMM.  Four columns per
// thread (N is a multiple of 128).
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
template <int WB, int KM>
static hipError_t launch_store(const GemmArgs& g, hipStream_t stream) {
    const int s = split_count(g, WB);
    if (s > 1) {
        // K ranges write fp32 partials, then one pass sums them
        GemmArgs gp = g;
        gp.C = g.split_ws;
        gp.ldc = g.N;
        gp.c_dtype = kF32;
        gp.R = nullptr;
        hipError_t e = launch_typed<WB, kEpiStore, float, KM>(gp, s, stream);
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
    return g.c_dtype == kF32 ? launch_typed<WB, kEpiStore, float, KM>(g, 1, stream)
                             : launch_typed<WB, kEpiStore, bf16, KM>(g, 1, stream);
}

template <int WB>
static hipError_t launch_wb(const GemmArgs& g, hipStream_t stream) {
    // K-major operands (fits_tile admits Bop alone or both, with the store or
    // GeLU-derivative epilogue and no LayerNorm)
    if (g.a_kmajor && g.b_kmajor) return launch_store<WB, 3>(g, stream);
    if (g.b_kmajor) {
        if (g.epi == kEpiGeluGrad)
            return g.gelu_out ? launch_typed<WB, kEpiGeluGradSave, bf16, 2>(g, 1, stream)
                              : launch_typed<WB, kEpiGeluGrad, bf16, 2>(g, 1, stream);
        return launch_store<WB, 2>(g, stream);
    }
    if (g.epi == kEpiGelu)
        return g.preact_out ? launch_typed<WB, kEpiGeluSave, bf16>(g, 1, stream)
                            : launch_typed<WB, kEpiGelu, bf16>(g, 1, stream);
    if (g.epi == kEpiGeluGrad)
        return g.gelu_out ? launch_typed<WB, kEpiGeluGradSave, bf16>(g, 1, stream)
                          : launch_typed<WB, kEpiGeluGrad, bf16>(g, 1, stream);
    return launch_store<WB, 0>(g, stream);
}

hipError_t launch_gemm_bf16_fast(const GemmArgs& g, hipStream_t stream) {
    if (gemm_split_bytes(g) > 0 && (!g.split_ws || g.split_ws_bytes < gemm_split_bytes(g) ||
                                    (reinterpret_cast<uintptr_t>(g.split_ws) & 15)))
        return hipErrorInvalidValue;
    return choose_wb(g) == 2 ? launch_wb<2>(g, stream) : launch_wb<4>(g, stream);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    if (choose_gemm_path(g) == kPathFastBf16) return launch_gemm_bf16_fast(g, stream);
    return launch_gemm_generic(g, stream);
}

}  // namespace tpmlp
