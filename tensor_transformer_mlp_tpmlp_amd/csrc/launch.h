// Host-side launchers of the tpmlp kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

constexpr int kEpiGelu = 0;   // C = GeLU_tanh(acc), rounded to C's dtype
constexpr int kEpiStore = 1;  // C = acc (+ R), rounded to C's dtype
constexpr int kEpiGeluGrad = 2;  // C = acc * GeLU_tanh'(aux), aux M x N in ab_dtype (backward)

// C[m][n] = epi( sum_k a(m,k) * Bop[n][k] ), m < M, n < N, k < K, where
// a(m,k) = Aop[m][k], or (Aop[m][k] - ln_mean[m]) * ln_rstd[m] when ln_mean
// is given.  Aop is M x K row-major (lda), Bop is N x K row-major (ldb): both
// operands are K-contiguous, unless a_kmajor / b_kmajor say an operand is
// stored K-major (its transpose row-major).  Aop, Bop and R have dtype ab_dtype; C has
// c_dtype.  Products accumulate in fp32.
struct GemmArgs {
    const void* A = nullptr;
    int64_t lda = 0;
    const void* B = nullptr;
    int64_t ldb = 0;
    int64_t M = 0, N = 0, K = 0;
    void* C = nullptr;
    int64_t ldc = 0;
    int c_dtype = kBF16;
    const void* R = nullptr;  // optional residual, M x N, ab_dtype
    int64_t ldr = 0;
    const float* ln_mean = nullptr;
    const float* ln_rstd = nullptr;
    const float* ln_csum = nullptr;  // column sums of Bop over K (LayerNorm epilogue form)
    int epi = kEpiStore;
    int ab_dtype = kBF16;
    const void* aux = nullptr;  // kEpiGeluGrad: the pre-activation, M x N (ldaux)
    int64_t ldaux = 0;
    void* preact_out = nullptr;  // kEpiGelu: also store the pre-activation here (M x N, ldc, C's dtype)
    void* gelu_out = nullptr;    // kEpiGeluGrad: also store GeLU_tanh(aux) here (M x N, ldc, C's dtype)
    // Split-K: a GEMM that allows it and would leave most of the GPU idle
    // (few output tiles, long K, a plain store epilogue) runs its K loop as
    // several ranges whose fp32 partial sums go to split_ws
    // (gemm_split_bytes(g) bytes) and are then added.  The forward's second
    // GEMM (the shard sum) never allows it: its sum stays in one accumulator.
    bool allow_split = false;
    void* split_ws = nullptr;
    size_t split_ws_bytes = 0;
    // K-major operands: with a_kmajor, Aop[m][k] = A[k * lda + m] (A stored
    // K x M, M contiguous); with b_kmajor, Bop[n][k] = B[k * ldb + n].
    bool a_kmajor = false;
    bool b_kmajor = false;
};

// Bytes of split-K scratch launch_gemm will use for g (0: not split).
size_t gemm_split_bytes(const GemmArgs& g);

// Which kernel family a GEMM goes to.
enum GemmPath { kPathFastBf16 = 0, kPathGeneric = 1 };
GemmPath choose_gemm_path(const GemmArgs& g);

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);

// Compute units of the current device (queried once).
int device_cu_count();
hipError_t launch_gemm_generic(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gemm_bf16_fast(const GemmArgs& g, hipStream_t stream);

hipError_t launch_gelu(const void* x, void* y, int64_t count, int dtype, hipStream_t stream);
hipError_t launch_ln_stats(const void* x, int64_t M, int64_t D, int dtype, float eps, float* mean,
                           float* rstd, hipStream_t stream);
hipError_t launch_ln_apply(const float* x, int64_t M, int64_t D, float eps, void* out, int out_dtype,
                           hipStream_t stream);
// Whether one sequence's rows of Q|K|V (plus one key tile) stay below the
// 2 GiB that the attention kernel's buffer offsets address.
bool attention_fits(int64_t seq, int64_t heads);
hipError_t launch_attention(const void* qkv, int64_t ldq, const void* x, int64_t ldx, void* out, int64_t ldo,
                            int64_t batch, int64_t seq, int64_t heads, hipStream_t stream);
hipError_t launch_rowsum(const void* x, int64_t rows, int64_t cols, int dtype, float* out, hipStream_t stream);
hipError_t launch_transpose(const void* in, int64_t ldi, void* out, int64_t ldo, int64_t R, int64_t C,
                            int elem_bytes, hipStream_t stream);

}  // namespace tpmlp
