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

hipError_t launch_ln_stats(const void* x, int64_t M, int64_t D, int dtype, float eps, float* mean,
                           float* rstd, hipStream_t stream) {
    const int64_t blocks = (M + 3) / 4;
    if (dtype == kF32)
        ln_stats_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const float*>(x), M, D, eps, mean, rstd);
    else
        ln_stats_kernel<bf16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const bf16*>(x), M, D, eps, mean, rstd);
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
// Strided transpose out[c][r] = in[r][c] (r < R, c < C), bit-exact, through a
// 64x64 LDS tile padded by one element against bank conflicts.  Used to pack
// A (D x F) into K-contiguous A^T (F x D) and B (F x D) into B^T (D x F), and
// to unpack a shard back into the page's layout.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E* __restrict__ in, int64_t ldi,
                                                        E* __restrict__ out, int64_t ldo, int64_t R,
                                                        int64_t C) {
    __shared__ E tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64;
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63;
    const int ty = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int rr = ty + 4 * i;
        if (r0 + rr < R && c0 + tx < C) tile[rr][tx] = in[(r0 + rr) * ldi + c0 + tx];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int cc = ty + 4 * i;
        if (c0 + cc < C && r0 + tx < R) out[(c0 + cc) * ldo + r0 + tx] = tile[tx][cc];
    }
}

hipError_t launch_transpose(const void* in, int64_t ldi, void* out, int64_t ldo, int64_t R, int64_t C,
                            int elem_bytes, hipStream_t stream) {
    const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
    if (elem_bytes == 4)
        transpose_kernel<uint32_t><<<grid, dim3(256), 0, stream>>>(
            static_cast<const uint32_t*>(in), ldi, static_cast<uint32_t*>(out), ldo, R, C);
    else
        transpose_kernel<uint16_t><<<grid, dim3(256), 0, stream>>>(
            static_cast<const uint16_t*>(in), ldi, static_cast<uint16_t*>(out), ldo, R, C);
    return hipGetLastError();
}

}  // namespace tpmlp
