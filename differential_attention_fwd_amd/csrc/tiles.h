// Tile layouts and small wave-level helpers shared by the bf16 kernels for gfx950 (forward and backward).
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layouts (lane l, h = l / 32, r = l % 32):
//   A (32 x 16): lane holds A[m = r][k = 8 h + j], j = 0..7      B (16 x 32): lane holds B[k = 8 h + j][n = r]
//   D (32 x 32): lane holds D[m = 8 (i / 4) + 4 h + i % 4][n = r], i = 0..15
// When a product consumes an accumulator of another product as its B operand, the k order is the accumulator's row
// order: position 8 h + j of a 16-slot k step holds row 8 (j / 4) + 4 h + j % 4.  The kernels read the matching A
// operands with transposing LDS reads (ds_read_b64_tr_b16) that pick rows in that order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float LOG2E = 1.4426950408889634f;

// Combine a per-lane value with the value of lane (l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ unsigned pack2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8): wait until at most `vm` vector
// memory operations of this wave are outstanding and all LDS operations are done.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | (0 << 8) | ((vm >> 4) << 14); }

// Workgroup barrier without the memory-model fence of __syncthreads (which would drain every outstanding load,
// including prefetches meant to stay in flight).  Callers first wait for their own LDS traffic with s_waitcnt;
// LDS is coherent inside the workgroup.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Check builds (compiled with -DDIFFATTN_CHECK, see build.py): before a wave issues a direct load of `size` bytes
// per lane into an LDS piece, each lane fills the bytes its load will write with NaN (bf16 and fp32 alike).  Call
// check_fence() after the fills of a tile and before its loads: the fills then complete before the loads can land,
// and a read of the piece before its load has landed returns NaN, which reaches the output.  Ordinary builds
// compile both to nothing.
__device__ __forceinline__ void check_fill(unsigned char* piece, int size) {
#ifdef DIFFATTN_CHECK
    unsigned char* p = piece + size * (int)(threadIdx.x & 63);
    if (size == 16) *(u32x4*)p = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
    else *(unsigned*)p = 0x7fc07fc0u;
#else
    (void)piece;
    (void)size;
#endif
}
__device__ __forceinline__ void check_fence() {
#ifdef DIFFATTN_CHECK
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
#endif
}

}  // namespace diffattn
