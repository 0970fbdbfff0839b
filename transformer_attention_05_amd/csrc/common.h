// Device helpers shared by the gfx950 attention kernels: vector types for the
// MFMA builtins, bf16 packing, base-2 exponent, cross-lane reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// bf16 bit patterns → fp32 (exact): low / high half of a packed dword.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 → packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// acc + lo + hi of a packed bf16 pair, in fp32 (v_dot2c_f32_bf16 with (1, 1)).
// Two floats as two fp16 (round to nearest even), lo in the low half.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const f16x2 h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

// Lane-exchange through ds_bpermute (any permutation within the wave).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
    int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

// Reductions across the two 32-lane halves of a wave (lane l with l ^ 32):
// v_permlane32_swap(x, x) returns {x[l], x[l ^ 32]} in its two results.
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Order LDS traffic of one wave: every lane's earlier LDS writes are visible
// to every lane's later LDS reads (and no read is hoisted above a write).
// (A workgroup-scope fence waits for the wave's LDS operations to complete;
// the wave barrier keeps the compiler from moving memory operations across.)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T as(u32x4 v) { return __builtin_bit_cast(T, v); }

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// HBM → LDS without registers: each lane copies 16 (or 4) bytes from src to
// LDS byte lds_block + 16·lane (+ 4·lane); lds_block is wave-uniform (M0).
// Written as asm on purpose: the compiler then does not track the copy. When
// it does (the builtin), it cannot tell which LDS buffer a later read
// touches, and puts a wait for every copy in flight in front of the first
// LDS read after a copy and in front of each barrier, which leaves no copy in
// flight across compute. The caller orders each copy with wait_vmcnt and a
// barrier before any lane reads the block; there is no output register.
__device__ __forceinline__ void copy16_to_lds(const void *src, const void *lds_block) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const lds_char *)lds_block;
    asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void copy4_to_lds(const void *src, const void *lds_block) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const lds_char *)lds_block;
    asm volatile("global_load_lds_dword %0, off" :: "v"(src), "{m0}"(m0) : "memory");
}

// Uses register fragments here, so that the compiler waits for the loads
// that produce them at this point. Its own waits do not see the asm copies
// above; a wait it placed inside a loop for a fragment loaded before the
// loop would also wait for every copy in flight, each iteration.
template <int N>
__device__ __forceinline__ void regs_ready(const bf16x8 (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const u32x4 w = __builtin_bit_cast(u32x4, x[i]);
        asm volatile("" :: "v"(w));
    }
}
__device__ __forceinline__ void regs_ready(float x) { asm volatile("" :: "v"(x)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

}  // namespace attn
