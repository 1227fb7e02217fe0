// Bandwidth-bound kernels of the tpmlp library: standalone GeLU, LayerNorm
// row statistics, and the strided transpose used to pack and unpack shards.
#include "device_common.h"
#include "launch.h"

namespace tpmlp {

// ---------------------------------------------------------------------------
// GeLU, elementwise ("Tensor-Parallel MLP (Megatron)", section "GeLU").
// 16-byte vector loads/stores (8 bf16 or 4 fp32 per lane), grid-stride; the
// count % vector-width tail is done by the first threads, element by element.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void gelu_kernel(const T* x, T* y,
                                                   int64_t count) {
    constexpr int V = 16 / sizeof(T);
    const int64_t nvec = count / V;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    u32x4* yv = reinterpret_cast<u32x4*>(y);
    for (int64_t v = tid; v < nvec; v += stride) {
        u32x4 raw = __builtin_nontemporal_load(xv + v);
        T vals[V];
        __builtin_memcpy(vals, &raw, 16);
#pragma unroll
        for (int e = 0; e < V; ++e) vals[e] = from_f32<T>(gelu_tanh(to_f32(vals[e])));
        __builtin_memcpy(&raw, vals, 16);
        __builtin_nontemporal_store(raw, yv + v);
    }
    const int64_t tail = nvec * V + tid;
    if (tail < count) y[tail] = from_f32<T>(gelu_tanh(to_f32(x[tail])));
}

hipError_t launch_gelu(const void* x, void* y, int64_t count, int dtype, hipStream_t stream) {
    const int64_t V = dtype == kF32 ? 4 : 8;
    int64_t work = count / V;
    if (work < V) work = V;  // the tail needs up to V-1 threads
    int64_t blocks = (work + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (dtype == kF32)
        gelu_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const float*>(x), static_cast<float*>(y), count);
    else
        gelu_kernel<bf16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const bf16*>(x), static_cast<bf16*>(y), count);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LayerNorm statistics: per-row mean and 1/sqrt(biased variance + eps), fp32
// ("LLM Lab Notes 06", section 2, markers 2 and 5: layer_norm over the hidden
// axis, no affine).  One wave per row, two passes over the row (mean, then
// sum of squared deviations) so a large mean does not cancel the variance.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <typename T>
__global__ __launch_bounds__(256) void ln_stats_kernel(const T* __restrict__ x, int64_t M, int64_t D,
                                                       float eps, float* __restrict__ mean,
                                                       float* __restrict__ rstd) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const T* xr = x + row * D;
    float s = 0.f;
    for (int64_t c = lane; c < D; c += 64) s += to_f32(xr[c]);
    const float mu = wave_sum(s) / (float)D;
    float q = 0.f;
    for (int64_t c = lane; c < D; c += 64) {
        const float d = to_f32(xr[c]) - mu;
        q = __builtin_fmaf(d, d, q);
    }
    const float var = wave_sum(q) / (float)D;
    if (lane == 0) {
        mean[row] = mu;
        rstd[row] = 1.0f / __builtin_sqrtf(var + eps);
    }
}

// Register-resident form for rows of at most 64 * CH 16-byte chunks whose
// length is a multiple of the chunk: the row is read once, with 16-byte
// loads (a wave reads 1 KiB contiguous per load), and both passes (mean,
// then squared deviations) run over registers.  With APPLY the wave also
// writes the normalised row, (x - mean) * rstd rounded once to TO; without
// it, it writes the two statistics.
template <typename T, typename TO, int CH, bool APPLY>
__global__ __launch_bounds__(256) void ln_rows_vec_kernel(const T* __restrict__ x, int64_t M, int64_t D,
                                                          float eps, float* __restrict__ mean,
                                                          float* __restrict__ rstd, TO* __restrict__ out) {
    constexpr int V = 16 / sizeof(T);
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const T* xr = x + row * D;
    float v[CH][V];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int64_t c = (int64_t)(lane + 64 * k) * V;
        if (c < D) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(xr + c);
            T e[V];
            __builtin_memcpy(e, &raw, 16);
#pragma unroll
            for (int r = 0; r < V; ++r) {
                v[k][r] = to_f32(e[r]);
                s += v[k][r];
            }
        }
    }
    const float mu = wave_sum(s) / (float)D;
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        if ((int64_t)(lane + 64 * k) * V < D) {
#pragma unroll
            for (int r = 0; r < V; ++r) {
                const float d = v[k][r] - mu;
                q = __builtin_fmaf(d, d, q);
            }
        }
    }
    const float var = wave_sum(q) / (float)D;
    const float rs = 1.0f / __builtin_sqrtf(var + eps);
    if constexpr (!APPLY) {
        if (lane == 0) {
            mean[row] = mu;
            rstd[row] = rs;
        }
    } else {
        TO* orow = out + row * D;
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int64_t c = (int64_t)(lane + 64 * k) * V;
            if (c < D) {
                TO o[V];
#pragma unroll
                for (int r = 0; r < V; ++r) o[r] = from_f32<TO>((v[k][r] - mu) * rs);
                if constexpr (sizeof(TO) * V == 16) {
                    u32x4 w;
                    __builtin_memcpy(&w, o, 16);
                    *reinterpret_cast<u32x4*>(orow + c) = w;
                } else {
                    static_assert(sizeof(TO) * V == 8, "8- or 16-byte output chunks");
                    uint2 w;
                    __builtin_memcpy(&w, o, 8);
                    *reinterpret_cast<uint2*>(orow + c) = w;
                }
            }
        }
    }
}

// Element-wise normalisation of an fp32 row for any length and alignment:
// one wave per row, the same two statistics passes, then a writing pass.
template <typename TO>
__global__ __launch_bounds__(256) void ln_apply_kernel(const float* __restrict__ x, int64_t M, int64_t D,
                                                       float eps, TO* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const float* xr = x + row * D;
    float s = 0.f;
    for (int64_t c = lane; c < D; c += 64) s += xr[c];
    const float mu = wave_sum(s) / (float)D;
    float q = 0.f;
    for (int64_t c = lane; c < D; c += 64) {
        const float d = xr[c] - mu;
        q = __builtin_fmaf(d, d, q);
    }
    const float rs = 1.0f / __builtin_sqrtf(wave_sum(q) / (float)D + eps);
    TO* orow = out + row * D;
    for (int64_t c = lane; c < D; c += 64) orow[c] = from_f32<TO>((xr[c] - mu) * rs);
}

// Chunks per lane for the register-resident form (1, 2, 4 or 8), or 0 when
// the row does not fit it.
static int ln_chunks(int64_t D, int V, const void* x, const void* out) {
    if (D % V != 0 || reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return 0;
    for (int ch = 1; ch <= 8; ch *= 2)
        if (D <= (int64_t)64 * V * ch) return ch;
    return 0;
}

template <typename T, typename TO, bool APPLY>
static void launch_ln_vec(int ch, dim3 grid, const T* x, int64_t M, int64_t D, float eps, float* mean,
                          float* rstd, TO* out, hipStream_t stream) {
    switch (ch) {
        case 1: ln_rows_vec_kernel<T, TO, 1, APPLY><<<grid, dim3(256), 0, stream>>>(x, M, D, eps, mean, rstd, out); break;
        case 2: ln_rows_vec_kernel<T, TO, 2, APPLY><<<grid, dim3(256), 0, stream>>>(x, M, D, eps, mean, rstd, out); break;
        case 4: ln_rows_vec_kernel<T, TO, 4, APPLY><<<grid, dim3(256), 0, stream>>>(x, M, D, eps, mean, rstd, out); break;
        default: ln_rows_vec_kernel<T, TO, 8, APPLY><<<grid, dim3(256), 0, stream>>>(x, M, D, eps, mean, rstd, out); break;
    }
}

hipError_t launch_ln_stats(const void* x, int64_t M, int64_t D, int dtype, float eps, float* mean,
                           float* rstd, hipStream_t stream) {
    const dim3 grid((unsigned)((M + 3) / 4));
    const int ch = ln_chunks(D, dtype == kF32 ? 4 : 8, x, x);
    if (dtype == kF32) {
        if (ch)
            launch_ln_vec<float, float, false>(ch, grid, static_cast<const float*>(x), M, D, eps, mean, rstd,
                                               nullptr, stream);
        else
            ln_stats_kernel<float><<<grid, dim3(256), 0, stream>>>(static_cast<const float*>(x), M, D, eps,
                                                                   mean, rstd);
    } else {
        if (ch)
            launch_ln_vec<bf16, float, false>(ch, grid, static_cast<const bf16*>(x), M, D, eps, mean, rstd,
                                              nullptr, stream);
        else
            ln_stats_kernel<bf16><<<grid, dim3(256), 0, stream>>>(static_cast<const bf16*>(x), M, D, eps,
                                                                  mean, rstd);
    }
    return hipGetLastError();
}

hipError_t launch_ln_apply(const float* x, int64_t M, int64_t D, float eps, void* out, int out_dtype,
                           hipStream_t stream) {
    const dim3 grid((unsigned)((M + 3) / 4));
    const int ch = ln_chunks(D, 4, x, out);
    if (out_dtype == kF32) {
        if (ch)
            launch_ln_vec<float, float, true>(ch, grid, x, M, D, eps, nullptr, nullptr, static_cast<float*>(out),
                                              stream);
        else
            ln_apply_kernel<float><<<grid, dim3(256), 0, stream>>>(x, M, D, eps, static_cast<float*>(out));
    } else {
        if (ch)
            launch_ln_vec<float, bf16, true>(ch, grid, x, M, D, eps, nullptr, nullptr, static_cast<bf16*>(out),
                                             stream);
        else
            ln_apply_kernel<bf16><<<grid, dim3(256), 0, stream>>>(x, M, D, eps, static_cast<bf16*>(out));
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row sums in fp32, one wave per row: the column sums of A (row sums of the
// packed A^T) that the LayerNorm epilogue of the first GEMM needs.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rowsum_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                     float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const T* xr = x + row * cols;
    float s = 0.f;
    for (int64_t c = lane; c < cols; c += 64) s += to_f32(xr[c]);
    s = wave_sum(s);
    if (lane == 0) out[row] = s;
}

hipError_t launch_rowsum(const void* x, int64_t rows, int64_t cols, int dtype, float* out, hipStream_t stream) {
    const int64_t blocks = (rows + 3) / 4;
    if (dtype == kF32)
        rowsum_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const float*>(x), rows, cols, out);
    else
        rowsum_kernel<bf16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const bf16*>(x), rows, cols, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Strided bit-exact transpose out[c][r] = in[r][c] (r < R, c < C).  Used to
// pack A (D x F) into K-contiguous A^T (F x D) and B (F x D) into B^T (D x F),
// to unpack a shard, and to pack the attention projections.
//
// Vector form: V = 16 / sizeof(T) elements per 16-byte chunk, a tile of 16V x
// 16V elements per block of 256 threads.  Every global access is a 16-byte
// chunk (a wave reads 4 rows x 256 contiguous bytes per load and writes 4 rows
// x 256 contiguous bytes per store).  Phase 1 stores the chunks in LDS,
// chunk slot = chunk ^ (row / V % 16); phase 2 gives thread (a, b) the V x V
// block at rows aV.., columns bV..: it reads V chunks of one slot column
// (16 lanes of a pass hit 16 distinct 16-byte slots, so no bank conflict),
// transposes the block in registers and writes V output chunks.  Requires R,
// C, ldi, ldo to be multiples of V and 16-byte aligned pointers; other shapes
// take the element-wise form below.
// ---------------------------------------------------------------------------
// x[i] holds row i of a V x V block as V elements packed in 4 dwords; y[c]
// receives column c.  For 4-byte elements this is a renaming of dwords; for
// 2-byte elements each output dword pairs the same half of two input dwords.
template <int V>
__device__ __forceinline__ void transpose_block(const u32x4 (&x)[V], u32x4 (&y)[V]);

template <>
__device__ __forceinline__ void transpose_block<4>(const u32x4 (&x)[4], u32x4 (&y)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) y[c][k] = x[k][c];
}

template <>
__device__ __forceinline__ void transpose_block<8>(const u32x4 (&x)[8], u32x4 (&y)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = x[2 * k][j], hi = x[2 * k + 1][j];
            y[2 * j][k] = (lo & 0xffffu) | (hi << 16);
            y[2 * j + 1][k] = (lo >> 16) | (hi & 0xffff0000u);
        }
}

template <typename T>
__global__ __launch_bounds__(256) void transpose_vec_kernel(const T* __restrict__ in, int64_t ldi,
                                                            T* __restrict__ out, int64_t ldo, int64_t R,
                                                            int64_t C) {
    constexpr int V = 16 / sizeof(T);
    constexpr int TR = 16 * V;  // tile rows = tile columns
    __shared__ u32x4 tile[TR * 16];
    const int64_t r0 = (int64_t)blockIdx.y * TR;
    const int64_t c0 = (int64_t)blockIdx.x * TR;
    const int t = threadIdx.x;
    const int ch = t & 15;
    const bool col_ok = c0 + (int64_t)ch * V < C;
#pragma unroll
    for (int p = 0; p < V; ++p) {
        const int row = (t >> 4) + 16 * p;
        if (col_ok && r0 + row < R) {
            const u32x4 v = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(in + (r0 + row) * ldi + c0 + (int64_t)ch * V));
            tile[row * 16 + (ch ^ ((row / V) & 15))] = v;
        }
    }
    __syncthreads();
    const int a = t & 15;  // block row: input rows aV .. aV+V-1
    const int b = t >> 4;  // block column: input columns bV .. bV+V-1
    if (r0 + (int64_t)a * V >= R || c0 + (int64_t)b * V >= C) return;
    u32x4 x[V], y[V];
#pragma unroll
    for (int i = 0; i < V; ++i) x[i] = tile[(a * V + i) * 16 + (b ^ a)];
    transpose_block<V>(x, y);
#pragma unroll
    for (int i = 0; i < V; ++i)
        __builtin_nontemporal_store(
            y[i], reinterpret_cast<u32x4*>(out + (c0 + (int64_t)b * V + i) * ldo + r0 + (int64_t)a * V));
}

// Element-wise form for any shape and alignment: a 64 x 64 tile, one element
// per thread and access, LDS padded by one element per row.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int64_t ldi,
                                                        T* __restrict__ out, int64_t ldo, int64_t R,
                                                        int64_t C) {
    __shared__ T tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64;
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63;
    const int ty = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int rr = ty + 4 * i;
        if (r0 + rr < R && c0 + tx < C) {
            tile[rr][tx] = in[(r0 + rr) * ldi + c0 + tx];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int cc = ty + 4 * i;
        if (c0 + cc < C && r0 + tx < R) out[(c0 + cc) * ldo + r0 + tx] = tile[tx][cc];
    }
}

template <typename T>
static hipError_t transpose_typed(const void* in, int64_t ldi, void* out, int64_t ldo, int64_t R, int64_t C,
                                  hipStream_t stream) {
    constexpr int64_t V = 16 / sizeof(T);
    const bool vec = R % V == 0 && C % V == 0 && ldi % V == 0 && ldo % V == 0 &&
                     reinterpret_cast<uintptr_t>(in) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0;
    const T* src = static_cast<const T*>(in);
    T* dst = static_cast<T*>(out);
    if (vec) {
        const dim3 grid((unsigned)((C + 16 * V - 1) / (16 * V)), (unsigned)((R + 16 * V - 1) / (16 * V)));
        transpose_vec_kernel<T><<<grid, dim3(256), 0, stream>>>(src, ldi, dst, ldo, R, C);
    } else {
        const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
        transpose_kernel<T><<<grid, dim3(256), 0, stream>>>(src, ldi, dst, ldo, R, C);
    }
    return hipGetLastError();
}

hipError_t launch_transpose(const void* in, int64_t ldi, void* out, int64_t ldo, int64_t R, int64_t C,
                            int elem_bytes, hipStream_t stream) {
    // bit-exact copies: the element's type only sets its width
    return elem_bytes == 4 ? transpose_typed<float>(in, ldi, out, ldo, R, C, stream)
                           : transpose_typed<bf16>(in, ldi, out, ldo, R, C, stream);
}

}  // namespace tpmlp
