// Device-side types and helpers shared by the tpmlp HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// sqrt(2/pi) and the cubic coefficient of the GPT-2 tanh approximation of
// GeLU ("Tensor-Parallel MLP (Megatron)", section "GeLU").
constexpr float kGeluC = 0.7978845608028654f;
constexpr float kGeluA = 0.044715f;

// GeLU_tanh(x) = x/2 (1 + tanh u), u = sqrt(2/pi) (x + 0.044715 x^3).
// Evaluated as x * sigmoid(2u) = x / (1 + exp(-2u)), which is the same
// function since (1 + tanh u)/2 = 1/(1 + exp(-2u)).  With exp(-2u) =
// 2^(x (k0 + k1 x^2)), k0 = -2 sqrt(2/pi) log2(e) and k1 = 0.044715 k0, that
// is two multiplies, one fma, one v_exp_f32, one add, one v_rcp_f32 and one
// multiply.  2^(...) overflows to +inf for very negative x, giving -0; it
// underflows to 0 for large x, giving x.  NaN propagates.
constexpr double kLog2e = 1.4426950408889634;
constexpr float kGeluK0 = (float)(-2.0 * (double)kGeluC * kLog2e);
constexpr float kGeluK1 = (float)(-2.0 * (double)kGeluC * (double)kGeluA * kLog2e);
// s = 1/(1 + exp(-2u)) of x, given x2 = x * x
__device__ __forceinline__ float gelu_sigmoid(float x, float x2) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * __builtin_fmaf(x2, kGeluK1, kGeluK0)));
}
__device__ __forceinline__ float gelu_tanh(float x) { return x * gelu_sigmoid(x, x * x); }

// d/dx GeLU_tanh(x), for the backward pass.  With s = (1 + tanh u)/2 =
// 1/(1 + exp(-2u)) and 1 - tanh^2 u = 4 s (1 - s), the product and chain
// rules give s + q s (1 - s), q = 2 sqrt(2/pi) x (1 + 3 * 0.044715 x^2).
// It is formed as fma(q, t, s) with t = s (1 - s) = fma(-s, s, s) and q =
// x fma(x^2, q1, q0), sharing x^2 (and the exponential and reciprocal, when
// GeLU of the same x is also wanted) with gelu_tanh.  At both ends s is
// exactly 0 or 1, so t = 0 and the result is s (q may overflow there, and
// q * 0 would be NaN); a NaN x gives a NaN t and result.
constexpr float kGeluQ0 = (float)(2.0 * (double)kGeluC);
constexpr float kGeluQ1 = (float)(6.0 * (double)kGeluC * (double)kGeluA);
// the derivative from x, x2 = x * x and s = gelu_sigmoid(x, x2)
__device__ __forceinline__ float gelu_grad_from(float x, float x2, float s) {
    const float q = x * __builtin_fmaf(x2, kGeluQ1, kGeluQ0);
    const float t = __builtin_fmaf(-s, s, s);
    const float r = __builtin_fmaf(q, t, s);
    return t == 0.0f ? s : r;
}
__device__ __forceinline__ float gelu_tanh_grad(float x) {
    return gelu_grad_from(x, x * x, gelu_sigmoid(x, x * x));
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

typedef __attribute__((address_space(3))) void lds_void;

// A raw buffer resource (base address, no stride, num_records bytes, the
// default data format) as four wave-uniform dwords, for the inline
// assembly below.  Each dword goes through readfirstlane so that it is an
// SGPR value whatever the compiler inferred about its uniformity.
__device__ __forceinline__ u32x4 buffer_rsrc_sgpr(const void* base, uint32_t num_records) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(num_records);
    r[3] = 0x00020000u;
    return r;
}

// One 16-byte-per-lane direct load from buffer resource r into LDS at the
// wave-uniform address dst (lane L's 16 bytes land at dst + 16 L), written
// out so that the compiler does not see an LDS write in flight: it would
// otherwise wait for every such load before each transposing LDS read
// (ds_read_b64_tr_b16), since it cannot tell LDS buffers apart.  Callers order
// these loads against their readers themselves (vmcnt waits and barriers).
// M0 holds the LDS address; the s_nop is the wait state an M0 write needs
// before an LDS direct load.
__device__ __forceinline__ void dma16_asm(uint8_t* dst, u32x4 r, uint32_t voff, uint32_t soff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_void*)dst));
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"{m0}"(m0), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory");
}

// One 16-byte-per-lane direct load from global memory into LDS: lane L's 16
// bytes at base + voff land at LDS byte address lds + 16 L (lds wave-uniform,
// an LDS address rather than a pointer, which the compiler would convert
// with a null check on every load).  base is wave-uniform (a scalar
// register pair), voff a per-lane 32-bit offset; there is no range check, so
// every address must lie inside the operand.  On gfx950 this form disturbs
// the matrix pipe much less than the buffer form: in a stream of 16x16x32
// MFMAs, one every eight MFMAs costs about 12 cycles against about 23-28.
// Like dma16_asm it is written out (the compiler sees no LDS write in
// flight) and needs one wait state after the M0 write.
__device__ __forceinline__ void gdma16_asm(uint32_t lds, const void* base, uint32_t voff) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"{m0}"(lds), "v"(voff), "s"(base) : "memory");
}

// The LDS byte address of a __shared__ object, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// Transposing LDS read of four 16-bit values (ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane i supplies the address of 4 consecutive
// elements (row i / 4 of a 4 x 16 block when the addresses are set up as
// row (i / 4), column 4 (i % 4)); lane j receives, for k = 0..3, element
// j % 4 of the four elements addressed by lane 4 k + j / 4.  With lane 4 k + q
// addressing row r_k at column c0 + 4 q, lane j receives column c0 + j of
// rows r_0 .. r_3.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4s lds_read_tr16(const uint8_t* p) {
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

}  // namespace tpmlp
