// sv_device.h -- device-side helpers shared by the gfx950 kernels of
// libspecverify.so (mask predicate, RoPE angles, bf16 packing, reductions).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kTwoPi = 6.283185307179586476925286766559;

// Temporal-causal visibility of a response key for a response row
// ("SimSD ...", 关键设计 2, equation A_ij).  Labels are the step labels tau
// (1..B) of the row's and key's slots.  The four cases collapse into one
// compare and one flip:
//   data row  -> data key  iff t_key <= t_row, mask key iff t_key >  t_row
//   mask row  -> data key  iff t_key <  t_row, mask key iff t_key >= t_row
// Prompt keys are always visible and never reach this predicate.
__device__ __forceinline__ bool visible(int t_row, bool row_is_data, int t_key, bool key_is_data) {
    return (t_key < t_row + (row_is_data ? 1 : 0)) != !key_is_data;
}

// cos/sin of the RoPE angle pos * inv_freq, where inv_freq = theta^(-2i/d)
// is given in float64.  The angle is formed in revolutions and reduced to
// [-1/2, 1/2] in float64 (pos * inv_freq reaches ~1.6e4 rad for long
// prefixes, too coarse for float32); the hardware sine and cosine take their
// argument in revolutions, so the reduced value goes straight to them
// (measured on the device: max abs error 1.3e-7 over [-1/2, 1/2]).
__device__ __forceinline__ float2 rope_cs(double pos, double inv_freq) {
    double rev = pos * (inv_freq * (1.0 / kTwoPi));
    rev -= rint(rev);
    const float r = (float)rev;
    return make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
}

// theta^(-2i/d) in float64 from log2(theta).
__device__ __forceinline__ double rope_inv_freq(int i, int d, double log2_theta) {
    return exp2(-(2.0 * (double)i / (double)d) * log2_theta);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// round-to-nearest-even float -> bf16 bits (the gfx950 conversion is RNE).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace sv
