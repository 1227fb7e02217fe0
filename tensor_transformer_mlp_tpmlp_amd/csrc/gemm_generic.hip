// Bounds-checked MFMA GEMM for any shape and for fp32 operands.
//
// C[m][n] = epi( sum_k a(m,k) * Bop[n][k] ) with each operand K-contiguous or
// stored K-major (see GemmArgs).  64x64 output tile per 256-thread workgroup, four waves in
// a 2x2 grid, one 32x32 MFMA accumulator per wave, K staged through LDS in
// steps of 32 with zero fill outside the matrices.  fp32 operands use
// v_mfma_f32_32x32x2_f32, bf16 operands v_mfma_f32_32x32x16_bf16.
//
// This path serves the small fp32 workloads (the worked example of
// "Tensor-Parallel MLP (Megatron)", section "The split", and its random
// extension) and every shape the 256x256 bf16 kernel does not take; it is
// not the throughput path.
#include "device_common.h"
#include "launch.h"

namespace tpmlp {

namespace {

constexpr int GT = 64;   // output tile edge
constexpr int GK = 32;   // K step

struct GenericParams {
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    int64_t M, N, K;
    void* C;
    int64_t ldc;
    const void* R;
    int64_t ldr;
    const float* mean;
    const float* rstd;
    const void* aux;     // kEpiGeluGrad: pre-activation, operand dtype
    int64_t ldaux;
    void* preact;        // kEpiGelu: optional copy of the pre-activation (C's layout and dtype)
    void* gelu_out;      // kEpiGeluGrad: optional GeLU of the pre-activation (C's layout and dtype)
    int64_t tiles_n;
    int a_km, b_km;      // operand stored K-major (see GemmArgs)
};

// Row pitch of the LDS tiles in elements: fp32 pads by one word against bank
// conflicts; bf16 pads by 8 elements so each lane's 8-element K slice stays
// 16-byte aligned.
template <typename T> struct Pitch;
template <> struct Pitch<float> { static constexpr int v = GK + 1; };
template <> struct Pitch<bf16> { static constexpr int v = GK + 8; };

template <typename T, typename TC, int EPI, bool LN>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GenericParams p) {
    constexpr int P = Pitch<T>::v;
    __shared__ __attribute__((aligned(16))) T As[GT * P];
    __shared__ __attribute__((aligned(16))) T Bs[GT * P];

    const T* __restrict__ A = static_cast<const T*>(p.A);
    const T* __restrict__ B = static_cast<const T*>(p.B);
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int64_t tile = blockIdx.x;
    const int64_t m0 = (tile / p.tiles_n) * GT;
    const int64_t n0 = (tile % p.tiles_n) * GT;

    f32x16 acc = {};
    for (int64_t k0 = 0; k0 < p.K; k0 += GK) {
#pragma unroll
        for (int e = 0; e < (GT * GK) / 256; ++e) {
            const int idx = t + 256 * e;
            // consecutive threads walk the operand's contiguous axis
            const int ra = p.a_km ? idx % GT : idx / GK, ca = p.a_km ? idx / GT : idx % GK;
            const int rb = p.b_km ? idx % GT : idx / GK, cb = p.b_km ? idx / GT : idx % GK;
            const int64_t m = m0 + ra, ka = k0 + ca;
            const int64_t n = n0 + rb, kb = k0 + cb;
            float av = 0.f, bv = 0.f;
            if (m < p.M && ka < p.K) {
                av = to_f32(p.a_km ? A[ka * p.lda + m] : A[m * p.lda + ka]);
                if constexpr (LN) av = (av - p.mean[m]) * p.rstd[m];
            }
            if (n < p.N && kb < p.K) bv = to_f32(p.b_km ? B[kb * p.ldb + n] : B[n * p.ldb + kb]);
            As[ra * P + ca] = from_f32<T>(av);
            Bs[rb * P + cb] = from_f32<T>(bv);
        }
        __syncthreads();
        const int ra = (wm * 32 + (lane & 31)) * P;
        const int rb = (wn * 32 + (lane & 31)) * P;
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int kk = 0; kk < GK / 2; ++kk) {
                const int c = kk * 2 + (lane >> 5);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[ra + c], Bs[rb + c], acc, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < GK / 16; ++kk) {
                const int c = kk * 16 + (lane >> 5) * 8;
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&As[ra + c]);
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(&Bs[rb + c]);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // Accumulator layout of a 32x32 MFMA: lane l holds column l % 32 and, in
    // register r, row 8*(r/4) + 4*(l/32) + r%4.
    TC* __restrict__ C = static_cast<TC*>(p.C);
    const T* __restrict__ R = static_cast<const T*>(p.R);
    const int64_t n = n0 + wn * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < p.M && n < p.N) {
            float v = acc[r];
            if constexpr (EPI == kEpiGelu) {
                if (p.preact) static_cast<TC*>(p.preact)[m * p.ldc + n] = from_f32<TC>(v);
                v = gelu_tanh(v);
            } else if constexpr (EPI == kEpiGeluGrad) {
                const float s = to_f32(static_cast<const T*>(p.aux)[m * p.ldaux + n]);
                if (p.gelu_out) static_cast<TC*>(p.gelu_out)[m * p.ldc + n] = from_f32<TC>(gelu_tanh(s));
                v *= gelu_tanh_grad(s);
            } else {
                if (R) v += to_f32(R[m * p.ldr + n]);
            }
            C[m * p.ldc + n] = from_f32<TC>(v);
        }
    }
}

template <typename T, typename TC, int EPI>
hipError_t launch_typed(const GemmArgs& g, hipStream_t stream) {
    GenericParams p;
    p.A = g.A; p.lda = g.lda; p.B = g.B; p.ldb = g.ldb;
    p.M = g.M; p.N = g.N; p.K = g.K;
    p.C = g.C; p.ldc = g.ldc; p.R = g.R; p.ldr = g.ldr;
    p.mean = g.ln_mean; p.rstd = g.ln_rstd;
    p.aux = g.aux; p.ldaux = g.ldaux;
    p.preact = g.preact_out;
    p.gelu_out = g.gelu_out;
    p.tiles_n = (g.N + GT - 1) / GT;
    p.a_km = g.a_kmajor ? 1 : 0;
    p.b_km = g.b_kmajor ? 1 : 0;
    const int64_t tiles = ((g.M + GT - 1) / GT) * p.tiles_n;
    if (g.ln_mean)
        gemm_generic_kernel<T, TC, EPI, true><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(p);
    else
        gemm_generic_kernel<T, TC, EPI, false><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

template <typename T, typename TC>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t stream) {
    if (g.epi == kEpiGelu) return launch_typed<T, TC, kEpiGelu>(g, stream);
    if (g.epi == kEpiGeluGrad) return launch_typed<T, TC, kEpiGeluGrad>(g, stream);
    return launch_typed<T, TC, kEpiStore>(g, stream);
}

hipError_t launch_gemm_generic(const GemmArgs& g, hipStream_t stream) {
    if (g.ab_dtype == kF32) return launch_epi<float, float>(g, stream);  // fp32 weights: fp32 results
    if (g.c_dtype == kF32) return launch_epi<bf16, float>(g, stream);
    return launch_epi<bf16, bf16>(g, stream);
}

}  // namespace tpmlp
