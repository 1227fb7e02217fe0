// Throughput GEMM for bf16 operands on gfx950 matrix cores.
//
// C[m][n] = epi( sum_k Aop[m][k] * Bop[n][k] ), Aop (M x K) and Bop (N x K)
// K-contiguous, fp32 accumulation in v_mfma_f32_32x32x16_bf16.
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
// SIMD), each wave owning a 128x128 sub-tile: 4x4 MFMA 32x32 blocks, 256 fp32
// accumulators per lane held in AGPRs.  Shapes too small to fill the GPU with
// 256x256 tiles use 128x128 tiles (2x2 blocks per wave, 64 KiB of LDS, two
// workgroups per CU) with the same pipeline.  K advances in steps of 64 through two
// LDS stages of 64 KiB (A tile 32 KiB + B tile 32 KiB).
//
// Global -> LDS moves use the direct-to-LDS buffer load (buffer_load_dwordx4
// ... lds): no VGPR staging and no ds_write.  Lane L of a wave's load lands at
// LDS base + 16 L, so the XOR swizzle of the LDS layout is applied on the
// global side by choosing which 16-byte chunk each lane fetches.
//
// Pipeline per K step of tile t (k-sub-steps kk = 0..3, 16 MFMAs each):
//   kk = 0..2: read the MFMA fragments of kk+1 from LDS while the matrix
//              cores run kk; in kk = 0 also issue the second half of tile
//              t+1's loads;
//   kk = 3   : wait until this wave's LDS reads and tile t+1's loads have
//              landed, barrier (tile t+1 visible to all waves, tile t's stage
//              free), issue the first half of tile t+2's loads into the freed
//              stage, read tile t+1's first fragments, then run kk = 3.
// Splitting each tile's loads over two sub-steps, one load every few MFMAs,
// keeps a burst of loads from stalling MFMA issue; the loads still have most
// of a K step to arrive, LDS reads are always one sub-step ahead, and there is
// one barrier per K step.
//
// LayerNorm prologue (FFN half of the Post-LN block, "LLM Lab Notes 06",
// section 2, marker 5) is applied algebraically in GEMM1's epilogue:
//   sum_k (x_k - mu) r a_k = r * (sum_k x_k a_k - mu * sum_k a_k),
// with the per-row mean mu and r = 1/sqrt(var + eps) from the statistics
// kernel and the per-column sums of A from shard time.
#include "device_common.h"
#include "launch.h"

namespace tpmlp {

namespace {

// WB = MFMA blocks of 32x32 per wave per side: 4 gives the 256x256 tile
// (128x128 per wave), 2 the 128x128 tile (64x64 per wave) used when 256x256
// tiles would leave CUs idle.
constexpr int BK = 64;
template <int WB> struct Tile {
    static constexpr int M = 64 * WB;         // tile rows (= tile columns)
    static constexpr int BYTES = M * BK * 2;  // one operand tile of one stage
    static constexpr int QLOADS = M / 32;     // direct loads per wave per operand per K step
    static constexpr int LOADS = 2 * QLOADS;  // per wave per K step
};

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
    int tiles_m, tiles_n;
    int nt_store;        // write C with non-temporal stores
};

// s_waitcnt encodings (gfx9): vmcnt in bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; a field at its maximum does not wait.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int waitcnt_lgkm0() { return 15 | (3 << 14) | (7 << 4); }

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row` in LDS.  The
// XOR key (row & 7) ^ ((row >> 3) & 1) puts any 8 consecutive rows, and the
// even and the odd rows of any 16 consecutive rows, on distinct chunks, which
// keeps 128-bit accesses conflict-free whether the LDS serves 8 or 16 lanes
// per cycle.
__device__ __forceinline__ uint32_t lds_key(int row) { return (uint32_t)((row & 7) ^ ((row >> 3) & 1)); }

// Blocks reach the 8 XCDs round-robin (block b runs on XCD b % 8).  Give each
// XCD a contiguous range of tile ids, and walk that range in groups of 8 tile
// rows so that concurrently running tiles share A rows and B columns in the
// XCD's L2.  Bijective for any tile count.
__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    const int pid = xcd * per + min(xcd, rem) + idx;
    constexpr int GROUP = 8;
    const int group_tiles = GROUP * tiles_n;
    const int g = pid / group_tiles;
    const int first_m = g * GROUP;
    const int gm = min(tiles_m - first_m, GROUP);
    const int local = pid - g * group_tiles;
    tm = first_m + local % gm;
    tn = local / gm;
}

typedef __attribute__((address_space(3))) void lds_void;

template <int WB, int EPI, bool LN, bool ODD, typename TC>
__global__ __launch_bounds__(256) void gemm_bf16_mfma(FastParams p) {
    constexpr int BM = Tile<WB>::M, BN = Tile<WB>::M;
    constexpr int TILE_BYTES = Tile<WB>::BYTES;
    constexpr int LOADS_PER_TILE = Tile<WB>::LOADS;
    // two pipeline stages as distinct objects so the compiler can tell the
    // stage being filled from the stage being read
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[2 * TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[2 * TILE_BYTES];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, kept in an SGPR
    const int wm = w >> 1, wn = w & 1;
    int tm, tn;
    map_tile(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;

    // Buffer resources over this tile's 256 rows of each operand.
    const uint32_t a_bytes = (uint32_t)(BM * p.lda * 2);
    const uint32_t b_bytes = (uint32_t)(BN * p.ldb * 2);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(p.A + m0 * p.lda), (short)0, (int)a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(p.B + n0 * p.ldb), (short)0, (int)b_bytes, 0x00020000);

    // Wave w fills tile rows [w BM/4, (w+1) BM/4) of each operand with BM/32
    // loads of 8 rows; in load q, lane L fills row w BM/4 + 8 q + L/8 at
    // physical chunk L % 8, which must hold logical chunk (L % 8) ^ key(row),
    // and key(row) = (L / 8) ^ (q & 1).
    const uint32_t lrow = (uint32_t)(w * (BM / 4) + (lane >> 3));
    const uint32_t cx0 = (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
    const uint32_t cx1 = cx0 ^ 16u;
    const uint32_t a_v0 = lrow * (uint32_t)(p.lda * 2) + cx0, a_v1 = a_v0 - cx0 + cx1;
    const uint32_t b_v0 = lrow * (uint32_t)(p.ldb * 2) + cx0, b_v1 = b_v0 - cx0 + cx1;
    const uint32_t a_qstep = (uint32_t)(8 * p.lda * 2);
    const uint32_t b_qstep = (uint32_t)(8 * p.ldb * 2);
    const uint32_t dst_w = (uint32_t)(w * (BM / 4) * 128);

    auto load_tile = [&](uint8_t* st, int k0) {
        const uint32_t kb = (uint32_t)k0 * 2u;
#pragma unroll
        for (int q = 0; q < Tile<WB>::QLOADS; ++q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + dst_w + q * 1024),
                                                     16, (q & 1) ? a_v1 : a_v0, kb + q * a_qstep, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + TILE_BYTES + dst_w + q * 1024),
                                                     16, (q & 1) ? b_v1 : b_v0, kb + q * b_qstep, 0, 0);
        }
    };

    auto load_half = [&](uint8_t* st, int k0, int h) {
        const uint32_t kb = (uint32_t)k0 * 2u;
#pragma unroll
        for (int qq = 0; qq < Tile<WB>::QLOADS / 2; ++qq) {
            const int q = h * (Tile<WB>::QLOADS / 2) + qq;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + dst_w + q * 1024),
                                                     16, (q & 1) ? a_v1 : a_v0, kb + q * a_qstep, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + TILE_BYTES + dst_w + q * 1024),
                                                     16, (q & 1) ? b_v1 : b_v0, kb + q * b_qstep, 0, 0);
        }
    };

    // MFMA operand reads: lane l reads row (l & 31) of each 32-row block at
    // logical chunk 2 kk + (l >> 5); the swizzle key of those rows depends on
    // the lane only.
    const uint32_t key = lds_key(lane & 31);
    const int hi = lane >> 5;
    const uint32_t a_rd = (uint32_t)((wm * 32 * WB + (lane & 31)) * 128);
    const uint32_t b_rd = (uint32_t)((wn * 32 * WB + (lane & 31)) * 128) + TILE_BYTES;

    auto read_frags = [&](const uint8_t* st, int kk, bf16x8 (&fa)[WB], bf16x8 (&fb)[WB]) {
        const uint32_t ch = (((uint32_t)(2 * kk + hi)) ^ key) << 4;
#pragma unroll
        for (int i = 0; i < WB; ++i) {
            fa[i] = *reinterpret_cast<const bf16x8*>(st + a_rd + i * 32 * 128 + ch);
            fb[i] = *reinterpret_cast<const bf16x8*>(st + b_rd + i * 32 * 128 + ch);
        }
    };

    f32x16 acc[WB][WB];
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j) acc[i][j] = f32x16{};

    auto mfma16 = [&](const bf16x8 (&fa)[WB], const bf16x8 (&fb)[WB]) {
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
            for (int j = 0; j < WB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };

    bf16x8 fa0[WB], fb0[WB], fa1[WB], fb1[WB];
    const int nk = p.K / BK;
    __builtin_assume(nk >= 2);

    // Instruction order inside a K step is pinned with scheduling groups
    // (mask 0x008 = MFMA, 0x100 = LDS read, 0x020 = VMEM read): the LDS reads
    // of the next sub-step, and the next tile's global loads, are interleaved
    // one by one with the current sub-step's MFMAs.
    auto interleave_reads = [&]() {
#pragma unroll
        for (int i = 0; i < 2 * WB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (WB * WB > 2 * WB) __builtin_amdgcn_sched_group_barrier(0x008, WB * WB - 2 * WB, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // One K step on the tile held in `cur`.  has_next: a next tile exists (in
    // `nxt`); do_load: also refill `cur` with the tile two steps ahead.
    // 256x256 tiles split each tile's loads over two sub-steps; 128x128 tiles
    // have four times shorter K steps and issue a tile's loads at once, a full
    // K step ahead.
    constexpr bool kSplit = WB >= 4;
    constexpr int kLoadsPerGroup = Tile<WB>::LOADS / ((kSplit ? 2 : 1) * 2 * WB);

    auto k_step = [&](uint8_t* cur, uint8_t* nxt, int k_load, bool has_next, bool do_load, int k_pend, bool pend) {
        pend = pend && kSplit;
        read_frags(cur, 1, fa1, fb1);
        if (pend) load_half(nxt, k_pend, 1);
        mfma16(fa0, fb0);
        if (pend) {
#pragma unroll
            for (int i = 0; i < 2 * WB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerGroup, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if (WB * WB > 2 * WB) __builtin_amdgcn_sched_group_barrier(0x008, WB * WB - 2 * WB, 0);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            interleave_reads();
        }
        read_frags(cur, 2, fa0, fb0);
        mfma16(fa1, fb1);
        interleave_reads();
        read_frags(cur, 3, fa1, fb1);
        mfma16(fa0, fb0);
        interleave_reads();
        if (has_next) {
            __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (do_load) {
                if constexpr (kSplit) load_half(cur, k_load, 0);
                else load_tile(cur, k_load);
            }
            read_frags(nxt, 0, fa0, fb0);
            mfma16(fa1, fb1);
            if (do_load) {
#pragma unroll
                for (int i = 0; i < 2 * WB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerGroup, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                if (WB * WB > 2 * WB) __builtin_amdgcn_sched_group_barrier(0x008, WB * WB - 2 * WB, 0);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                interleave_reads();
            }
        } else {
            mfma16(fa1, fb1);
        }
    };

    // prologue: step 0 whole and the first half of step 1 (all of step 1
    // without the split); wait for step 0
    load_tile(stage0, 0);
    if constexpr (kSplit) {
        load_half(stage1, BK, 0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS_PER_TILE / 2));
    } else {
        load_tile(stage1, BK);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS_PER_TILE));
    }
    __builtin_amdgcn_s_barrier();
    read_frags(stage0, 0, fa0, fb0);

    // step t issues the second half of step t+1 (kk0) and the first half of
    // t+2 (kk3); without the split, all of t+2 at kk3
    int kt = 0;
    for (; kt + 3 < nk; kt += 2) {
        k_step(stage0, stage1, (kt + 2) * BK, true, true, (kt + 1) * BK, true);
        k_step(stage1, stage0, (kt + 3) * BK, true, true, (kt + 2) * BK, true);
    }
    if constexpr (ODD) {
        k_step(stage0, stage1, (kt + 2) * BK, true, true, (kt + 1) * BK, true);
        k_step(stage1, stage0, 0, true, false, (kt + 2) * BK, true);
        k_step(stage0, stage1, 0, false, false, 0, false);
    } else {
        k_step(stage0, stage1, 0, true, false, (kt + 1) * BK, true);
        k_step(stage1, stage0, 0, false, false, 0, false);
    }

    // Epilogue.  Accumulator layout of a 32x32 MFMA: lane l holds column
    // l % 32 and, in register r, row 8*(r/4) + 4*(l/32) + r%4.
    TC* __restrict__ C = static_cast<TC*>(p.C);
#pragma unroll
    for (int i = 0; i < WB; ++i) {
        const int64_t mb = m0 + wm * 32 * WB + i * 32 + hi * 4;
        float rs[16], rm[16];
        if constexpr (LN) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = mb + (r >> 2) * 8 + (r & 3);
                rs[r] = p.rstd[m];
                rm[r] = rs[r] * p.mean[m];
            }
        }
#pragma unroll
        for (int j = 0; j < WB; ++j) {
            const int64_t n = n0 + wn * 32 * WB + j * 32 + (lane & 31);
            float cs = 0.f;
            if constexpr (LN) cs = p.csum[n];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = mb + (r >> 2) * 8 + (r & 3);
                float v = acc[i][j][r];
                if constexpr (LN) v = __builtin_fmaf(rs[r], v, -rm[r] * cs);
                if constexpr (EPI == kEpiGelu) {
                    v = gelu_tanh(v);
                } else {
                    if (p.R) v += static_cast<float>(p.R[m * p.ldr + n]);
                }
                // A large output (H of the big workloads) is written
                // non-temporally: it would not fit the caches anyway, and
                // keeping it out of them keeps the operands resident in the
                // Infinity Cache.  A small one stays cached for its reader.
                if (p.nt_store)
                    __builtin_nontemporal_store(from_f32<TC>(v), &C[m * p.ldc + n]);
                else
                    C[m * p.ldc + n] = from_f32<TC>(v);
            }
        }
    }
}

template <int WB, int EPI, typename TC>
hipError_t launch_typed(const GemmArgs& g, hipStream_t stream) {
    constexpr int BM = Tile<WB>::M, BN = Tile<WB>::M;
    FastParams p;
    p.A = static_cast<const bf16*>(g.A); p.lda = g.lda;
    p.B = static_cast<const bf16*>(g.B); p.ldb = g.ldb;
    p.M = (int)g.M; p.N = (int)g.N; p.K = (int)g.K;
    p.C = g.C; p.ldc = g.ldc;
    p.R = static_cast<const bf16*>(g.R); p.ldr = g.ldr;
    p.mean = g.ln_mean; p.rstd = g.ln_rstd; p.csum = g.ln_csum;
    p.tiles_m = (int)(g.M / BM);
    p.tiles_n = (int)(g.N / BN);
    p.nt_store = g.M * g.N * (int64_t)sizeof(TC) > ((int64_t)128 << 20);
    const unsigned blocks = (unsigned)(p.tiles_m * p.tiles_n);
    const bool odd = (g.K / BK) & 1;
    if (g.ln_mean) {
        if (odd) gemm_bf16_mfma<WB, EPI, true, true, TC><<<dim3(blocks), dim3(256), 0, stream>>>(p);
        else gemm_bf16_mfma<WB, EPI, true, false, TC><<<dim3(blocks), dim3(256), 0, stream>>>(p);
    } else {
        if (odd) gemm_bf16_mfma<WB, EPI, false, true, TC><<<dim3(blocks), dim3(256), 0, stream>>>(p);
        else gemm_bf16_mfma<WB, EPI, false, false, TC><<<dim3(blocks), dim3(256), 0, stream>>>(p);
    }
    return hipGetLastError();
}

}  // namespace

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// CUs of the current device (queried once; 256 on MI355X).
static int device_cus() {
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 256;
        return n;
    }();
    return cus;
}

// Whether the MFMA kernel can take a shape with tiles of 64*wb rows: bf16
// operands, M and N whole tiles, K a whole number (at least two) of 64-wide
// steps, 16-byte aligned rows, one operand tile's byte offsets below 2^31
// (buffer offsets), and, with the LayerNorm epilogue, the column sums of Bop.
static bool fits_tile(const GemmArgs& g, int wb) {
    const int64_t tm = 64 * wb;
    if (g.ab_dtype != kBF16) return false;
    if (g.M <= 0 || g.N <= 0 || g.K <= 0) return false;
    if (g.M % tm || g.N % tm || g.K % BK || g.K < 2 * BK) return false;
    if (g.lda % 8 || g.ldb % 8 || !aligned16(g.A) || !aligned16(g.B)) return false;
    if (tm * g.lda * 2 >= ((int64_t)1 << 31) || tm * g.ldb * 2 >= ((int64_t)1 << 31)) return false;
    if ((g.M / tm) * (g.N / tm) >= ((int64_t)1 << 31) || g.M >= ((int64_t)1 << 31) ||
        g.N >= ((int64_t)1 << 31) || g.K >= ((int64_t)1 << 31))
        return false;
    if (g.ln_mean && !g.ln_csum) return false;
    return true;
}

// 256x256 tiles (wb = 4) when they keep at least 3/4 of the CUs busy, else
// 128x128 tiles (wb = 2, two workgroups per CU); 0 = not for the MFMA kernel.
static int choose_wb(const GemmArgs& g) {
    if (fits_tile(g, 4) && (g.M / 256) * (g.N / 256) * 4 >= 3 * (int64_t)device_cus()) return 4;
    if (fits_tile(g, 2)) return 2;
    if (fits_tile(g, 4)) return 4;
    return 0;
}

GemmPath choose_gemm_path(const GemmArgs& g) { return choose_wb(g) ? kPathFastBf16 : kPathGeneric; }

template <int WB>
static hipError_t launch_wb(const GemmArgs& g, hipStream_t stream) {
    if (g.epi == kEpiGelu) return launch_typed<WB, kEpiGelu, bf16>(g, stream);
    return g.c_dtype == kF32 ? launch_typed<WB, kEpiStore, float>(g, stream)
                             : launch_typed<WB, kEpiStore, bf16>(g, stream);
}

hipError_t launch_gemm_bf16_fast(const GemmArgs& g, hipStream_t stream) {
    return choose_wb(g) == 2 ? launch_wb<2>(g, stream) : launch_wb<4>(g, stream);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    if (choose_gemm_path(g) == kPathFastBf16) return launch_gemm_bf16_fast(g, stream);
    return launch_gemm_generic(g, stream);
}

}  // namespace tpmlp
