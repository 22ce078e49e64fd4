// Small device helpers shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dwkv {

constexpr int kWave = 64;

// Buffer resource over `bytes` bytes at p (a wave-uniform address, bytes
// below 2^32): buffer loads past its end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void *p, int64_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *u = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

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

// Value of another lane of the same row of 16 by a DPP move: quad_perm
// [1,0,3,2] (0xB1) and [2,3,0,1] (0x4E), row_half_mirror (0x141), row_mirror
// (0x140).  Each pairs every lane with one of the other half of its group.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Reductions over the 64 lanes of a (fully active) wave: within each row of
// 16 by DPP moves, then across the four rows by reading one lane of each.
// The result is the same in every lane.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48))));
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
