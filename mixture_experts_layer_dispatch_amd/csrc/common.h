// Device helpers shared by the MoE kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- address spaces
// Choosing between two global pointers with a per-lane select hides their
// address space from the compiler, which then emits FLAT loads (counted
// against the LDS wait counter too); the explicit global cast keeps them
// global loads.
template <class T>
__device__ __forceinline__ const T* global_select(bool second, const T* a, const T* b) {
    typedef const __attribute__((address_space(1))) T gT;
    gT* p = second ? (gT*)b : (gT*)a;
    return (const T*)p;
}

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// round-to-nearest-even float -> bf16 bits (NaN stays NaN)
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return f2bf(lo) | (f2bf(hi) << 16);
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- SwiGLU
// The forward computes h from the bf16-rounded g and u; the backward
// recomputes it from the saved bf16 g and u with this same function, so both
// see identical bits.
__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + __expf(-g)); }

__device__ __forceinline__ float swiglu_h(float g, float u) {
    float s = sigmoidf_(g);
    return (g * s) * u;
}

// ---------------------------------------------------------------- MFMA
// D(16x16, fp32) += A(16x32) * B(32x16), bf16 operands.  Lane l supplies
// row (l & 15) of A and column (l & 15) of B, each as 8 consecutive K values
// starting at K = 8 * (l >> 4); D row 4 * (l >> 4) + r, column (l & 15) lands
// in element r of lane l.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// the wave's index in its block, as a wave-uniform (scalar) value: LDS
// addresses built from it alone stay in scalar registers
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Maps a linear block id onto a logical tile id so that consecutive logical
// tiles run on the same XCD (blocks are dealt round-robin over the 8 XCDs).
// `count` is the number of live blocks; ids >= count are not remapped.
__device__ __forceinline__ int xcd_remap(int b, int count) {
    if (b >= count) return b;
    const int q = count >> 3, r = count & 7;
    const int x = b & 7;
    return x * q + (x < r ? x : r) + (b >> 3);
}

// sticky error bits kept in the first word of the workspace
enum : int32_t {
    ERR_BAD_EXPERT = 1,
    ERR_BAD_SLOT = 2,
    ERR_BAD_ROW = 4,
    ERR_BAD_OFFSETS = 8,
    ERR_ACC_CAPACITY = 16,    // more experts span macrobatches than the workspace keeps sums for
};

__device__ __forceinline__ void raise_err(int32_t* err, int32_t bit) {
    if (err) atomicOr(err, bit);
}

}  // namespace moe
