// Throughput GEMM for bf16 operands on gfx950 matrix cores.
//
// C[m][n] = epi( sum_k a(m,k) * Bop[n][k] ), Aop (M x K) and Bop (N x K)
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
// Tiling: one 256x256 output tile per workgroup of 4 waves (2x2), each wave
// owning a 128x128 sub-tile (4x4 MFMA 32x32 blocks, 256 fp32 accumulators per
// lane).  K advances in steps of 64 through a double-buffered LDS ring
// (2 stages x (32 KiB A + 32 KiB B) = 128 KiB of the 160 KiB LDS), with the
// next step's global loads in flight while the matrix cores work on the
// current one.  LDS rows are 128 bytes (64 bf16) with the 16-byte chunks
// XOR-swizzled so both the row-wise stores and the 32-row MFMA operand reads
// are bank-conflict free.  Workgroups are mapped so that each XCD works on a
// contiguous band of output tiles, grouped 8 tile-rows at a time for L2 reuse.
#include "device_common.h"
#include "launch.h"

namespace tpmlp {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int TILE_BYTES = BM * BK * 2;  // one operand, one stage

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
    const float* mean;
    const float* rstd;
    int tiles_m, tiles_n;
};

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row` in LDS.  The
// XOR key (row & 7) ^ ((row >> 3) & 1) makes any 8 consecutive rows, and the
// even and the odd rows of any 16 consecutive rows, land on distinct chunks,
// which keeps 128-bit accesses conflict-free whether the LDS serves 8 or 16
// lanes per cycle.
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
    return (uint32_t)(row * 128 + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 4));
}

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

template <int EPI, bool LN, typename TC>
__global__ __launch_bounds__(256, 1) void gemm_bf16_256x256(FastParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * TILE_BYTES];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int wm = w >> 1, wn = w & 1;
    int tm, tn;
    map_tile(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;

    // Global -> LDS staging: thread t moves 16-byte chunk (t & 7) of rows
    // (t >> 3) + 32 j, j < 8, of both operand tiles.
    const int lrow = t >> 3, lch = t & 7;
    const char* a_base = reinterpret_cast<const char*>(p.A + m0 * p.lda);
    const char* b_base = reinterpret_cast<const char*>(p.B + n0 * p.ldb);
    const uint32_t a_off = (uint32_t)(lrow * p.lda * 2 + lch * 16);
    const uint32_t b_off = (uint32_t)(lrow * p.ldb * 2 + lch * 16);
    const uint32_t a_step = (uint32_t)(32 * p.lda * 2);
    const uint32_t b_step = (uint32_t)(32 * p.ldb * 2);
    const uint32_t st_off = swz(lrow, lch);  // + j * 32 rows * 128 bytes

    float ln_mu[8], ln_rs[8];
    if constexpr (LN) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ln_mu[j] = p.mean[m0 + lrow + 32 * j];
            ln_rs[j] = p.rstd[m0 + lrow + 32 * j];
        }
    }

    u32x4 ra[8], rb[8];
    auto gload = [&](int k0) {
        const char* ab = a_base + (int64_t)k0 * 2;
        const char* bb = b_base + (int64_t)k0 * 2;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ra[j] = *reinterpret_cast<const u32x4*>(ab + a_off + j * a_step);
            rb[j] = *reinterpret_cast<const u32x4*>(bb + b_off + j * b_step);
        }
    };
    auto lstore = [&](int stage) {
        uint8_t* as = smem + stage * 2 * TILE_BYTES;
        uint8_t* bs = as + TILE_BYTES;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            u32x4 v = ra[j];
            if constexpr (LN) {
                bf16 e[8];
                __builtin_memcpy(e, &v, 16);
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    e[q] = static_cast<bf16>((static_cast<float>(e[q]) - ln_mu[j]) * ln_rs[j]);
                __builtin_memcpy(&v, e, 16);
            }
            *reinterpret_cast<u32x4*>(as + st_off + j * 4096) = v;
            *reinterpret_cast<u32x4*>(bs + st_off + j * 4096) = rb[j];
        }
    };

    // MFMA operand reads: lane l reads row (l & 31) of each 32-row block at
    // chunk 2*kk + (l >> 5); the swizzle key of those rows depends on the
    // lane only.
    const int key = (lane & 7) ^ ((lane >> 3) & 1);
    const int hi = lane >> 5;
    const uint32_t a_rd = (uint32_t)((wm * 128 + (lane & 31)) * 128);
    const uint32_t b_rd = (uint32_t)((wn * 128 + (lane & 31)) * 128) + TILE_BYTES;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    const int nk = p.K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const uint8_t* st = smem + cur * 2 * TILE_BYTES;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint32_t ch = (uint32_t)(((2 * kk + hi) ^ key) << 4);
            bf16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = *reinterpret_cast<const bf16x8*>(st + a_rd + i * 32 * 128 + ch);
                b[i] = *reinterpret_cast<const bf16x8*>(st + b_rd + i * 32 * 128 + ch);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator layout of a 32x32 MFMA: lane l holds column
    // l % 32 and, in register r, row 8*(r/4) + 4*(l/32) + r%4.
    TC* __restrict__ C = static_cast<TC*>(p.C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
                float v = acc[i][j][r];
                if constexpr (EPI == kEpiGelu) {
                    v = gelu_tanh(v);
                } else {
                    if (p.R) v += static_cast<float>(p.R[m * p.ldr + n]);
                }
                C[m * p.ldc + n] = from_f32<TC>(v);
            }
        }
    }
}

template <int EPI, typename TC>
hipError_t launch_typed(const GemmArgs& g, hipStream_t stream) {
    FastParams p;
    p.A = static_cast<const bf16*>(g.A); p.lda = g.lda;
    p.B = static_cast<const bf16*>(g.B); p.ldb = g.ldb;
    p.M = (int)g.M; p.N = (int)g.N; p.K = (int)g.K;
    p.C = g.C; p.ldc = g.ldc;
    p.R = static_cast<const bf16*>(g.R); p.ldr = g.ldr;
    p.mean = g.ln_mean; p.rstd = g.ln_rstd;
    p.tiles_m = (int)(g.M / BM);
    p.tiles_n = (int)(g.N / BN);
    const unsigned blocks = (unsigned)(p.tiles_m * p.tiles_n);
    if (g.ln_mean)
        gemm_bf16_256x256<EPI, true, TC><<<dim3(blocks), dim3(256), 0, stream>>>(p);
    else
        gemm_bf16_256x256<EPI, false, TC><<<dim3(blocks), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The 256x256 kernel takes bf16 operands whose M and N are whole tiles, K a
// whole number of 64-wide steps, 16-byte aligned rows, and byte offsets of
// one 256-row operand tile that fit in 32 bits.
GemmPath choose_gemm_path(const GemmArgs& g) {
    if (g.ab_dtype != kBF16) return kPathGeneric;
    if (g.M <= 0 || g.N <= 0 || g.K <= 0) return kPathGeneric;
    if (g.M % BM || g.N % BN || g.K % BK) return kPathGeneric;
    if (g.lda % 8 || g.ldb % 8 || !aligned16(g.A) || !aligned16(g.B)) return kPathGeneric;
    if ((int64_t)BM * g.lda * 2 >= (int64_t)1 << 32 || (int64_t)BN * g.ldb * 2 >= (int64_t)1 << 32)
        return kPathGeneric;
    if ((g.M / BM) * (g.N / BN) >= ((int64_t)1 << 31) || g.M >= ((int64_t)1 << 31) ||
        g.N >= ((int64_t)1 << 31) || g.K >= ((int64_t)1 << 31))
        return kPathGeneric;
    return kPathFastBf16;
}

hipError_t launch_gemm_bf16_fast(const GemmArgs& g, hipStream_t stream) {
    if (g.epi == kEpiGelu) return launch_typed<kEpiGelu, bf16>(g, stream);
    return g.c_dtype == kF32 ? launch_typed<kEpiStore, float>(g, stream)
                             : launch_typed<kEpiStore, bf16>(g, stream);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    if (choose_gemm_path(g) == kPathFastBf16) return launch_gemm_bf16_fast(g, stream);
    return launch_gemm_generic(g, stream);
}

}  // namespace tpmlp
