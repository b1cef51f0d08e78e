// Internal helpers shared by the HIP sources of the SFA library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hd_sfa.h"

namespace hdsfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// log2(e): the softmax is evaluated as exp2(s * scale * log2(e) - m).
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// Round-to-nearest-even float -> bf16 pair packed in one 32-bit word
// (lo in bits 0..15): one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 r = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Eight floats -> eight bf16 (RNE) as one MFMA operand.
__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) {
    return __builtin_convertvector(x, bf16x8);
}

__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);
}

// max / sum of x over lanes l and l^32, in registers (v_permlane32_swap):
// swapping the upper half of one copy with the lower half of another leaves
// lane l holding both x[l % 32] and x[l % 32 + 32].
__device__ __forceinline__ float halves_max(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// XOR swizzle of the 16-byte chunks of a row of D bf16 (D/8 chunks) staged in
// LDS, used for K/V tiles (and Q/dO tiles in the backward kernels).  Two read
// patterns must hit distinct banks:
//   direct:    16 consecutive rows, one logical chunk each (16-byte reads);
//   transpose: per 32 lanes, 4 consecutive rows x 4 consecutive logical
//              chunks (8-byte ds_read_b64_tr_b16 reads).
// D=128 (256-byte rows span all 64 banks): swz = (r%4)*4 + (r/4)%4.
// D=64 (128-byte rows, even/odd rows on opposite bank halves): the same idea
// over rows of one parity: swz = ((r/2)%2)*4 + (r/4)%4.
template <int D>
__device__ __forceinline__ uint32_t swz(uint32_t row) {
    if constexpr (D == 128) return ((row & 3u) << 2) | ((row >> 2) & 3u);
    else return (((row >> 1) & 1u) << 2) | ((row >> 2) & 3u);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The kernels mask scores with -inf and track the running max of the raw
// scores times the scale: both need a finite, positive softmax scale.
inline bool scale_ok(float scale) {
    return scale > 0.f && scale <= 3.4e38f;
}

inline bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline hd_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? HD_OK : HD_ERR_LAUNCH;
}

}  // namespace hdsfa
