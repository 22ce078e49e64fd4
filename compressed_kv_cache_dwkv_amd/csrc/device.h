// Small device helpers shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dwkv {

constexpr int kWave = 64;

__device__ __forceinline__ float h2f(uint16_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> fp16, round to nearest even (the hardware conversion honours the
// default round-to-nearest-even mode).
__device__ __forceinline__ uint16_t f2h(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Orders LDS accesses of the lanes of one wave (a wave's LDS operations
// execute in issue order, so this costs no instruction).
__device__ __forceinline__ void wave_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

__device__ __forceinline__ uint64_t lanemask_lt() { return (uint64_t(1) << lane_id()) - 1; }

// Signed code u of a token's packed residual values (bits = 4 or 8).
__device__ __forceinline__ int unpack_code(const uint8_t *vals, int u, int bits)
{
    if (bits == 8) return static_cast<int8_t>(vals[u]);
    int byte = vals[u >> 1];
    int nib = (u & 1) ? (byte >> 4) : (byte & 0xF);
    return (nib ^ 8) - 8;  // sign-extend 4-bit two's complement
}

}  // namespace dwkv
