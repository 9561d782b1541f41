// gq_device.h -- device-side helpers shared by the gfx950 kernels of the
// library (HIP, wave64).  Nothing here is used by the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqd {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Block geometry (weights per block, bytes per block) of the three formats.
enum { T_Q4_0 = 1, T_Q4_K = 2, T_Q6_K = 3, T_Q5_K = 4 };
enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// fp16 pair (1024, 1024): OR-ing a small integer n into the low mantissa bits
// of each half gives the fp16 value 1024 + n exactly (the exponent field of
// 1024 leaves the ten mantissa bits free and their weight is one).
constexpr uint32_t MAGIC = 0x64006400u;

// The fp16-pair magic 0x64006400 as a register value.  gfx9 VOP3 instructions
// take no literal operands, so with a literal the compiler splits
// (w & mask) | MAGIC into v_and_b32 + v_or_b32; with the magic in a VGPR (and
// the mask in an SGPR) it is one v_and_or_b32.  The asm is not volatile, so it
// is hoisted out of loops.
__device__ __forceinline__ uint32_t magic_vgpr() {
    uint32_t r;
    __asm__("v_mov_b32 %0, 0x64006400" : "=v"(r));
    return r;
}

// Loads that may be only 2-byte aligned (Q4_0 and Q6_K blocks are 18 and 210
// bytes long).  gfx9 global memory instructions accept unaligned addresses.
__device__ __forceinline__ u32x4 ld16u(const uint8_t* p) {
    u32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}
__device__ __forceinline__ u32x2 ld8u(const uint8_t* p) {
    u32x2 v;
    __builtin_memcpy(&v, p, 8);
    return v;
}
__device__ __forceinline__ uint32_t ld4u(const uint8_t* p) {
    uint32_t v;
    __builtin_memcpy(&v, p, 4);
    return v;
}
__device__ __forceinline__ uint16_t ld2(const uint8_t* p) {
    uint16_t v;
    __builtin_memcpy(&v, p, 2);
    return v;
}
__device__ __forceinline__ u32x4 ld16a(const uint8_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// D = a.lo*b.lo + a.hi*b.hi + c (fp16 pairs, fp32 accumulate).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}

// (a.lo - b.lo, a.hi - b.hi) of two fp16 pairs: one packed fp16 add with the
// second operand negated.  Exact where both are integers of at most 11
// significant bits whose difference is too (the weight-minus-zero-point step).
__device__ __forceinline__ uint32_t sub_h2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a) - __builtin_bit_cast(half2v, b));
}

// Two fp32 -> fp16 (round to nearest even), packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    half2v h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// fp32 -> fp16, round to nearest even.  The empty asm keeps f an fp32 value in
// a register: otherwise the compiler may fold a preceding multiply and this
// rounding into one v_fma_mixlo_f16 with a +0 addend, which turns a -0 product
// into +0.
__device__ __forceinline__ uint16_t f2h(float f) {
    __asm__ volatile("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float bf2f(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Barrier for LDS traffic only.  __syncthreads() is a full workgroup fence,
// which on gfx950 also waits for every outstanding global load (vmcnt(0)) --
// a kernel that keeps global loads in flight across a barrier would stall on
// them.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; }

// Activation of a gated feed-forward unit, in fp32:
// act 0: silu(g) = g / (1 + e^-g);
// act 1: gelu_tanh(g) = g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))).
__device__ __forceinline__ float act_fn(int act, float g) {
    if (act == 0) return g / (1.0f + expf(-g));
    const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * g, g * g, g);
    return 0.5f * g * (1.0f + tanhf(u));
}

}  // namespace gqd
