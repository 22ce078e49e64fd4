// Append step: encodes the new token's K and V of every (sequence, KV head)
// into the compressed form and stores it in its tier (DepthWeave-KV paper,
// arXiv 2607.06523, §3 Method, second paragraph: coefficients by projection
// onto the current basis, residual kept on the router-chosen number of
// channels with low-bit group quantisation).
//
// The encoder makes integer decisions (kept channels, codes) from floating
// point values, so it follows one fixed IEEE fp32 operation order --
// sequential fused multiply-adds in ascending index order, correctly rounded
// division, round-to-nearest-even conversions -- and must be built with
// -ffp-contract=off so no other multiply-add is fused.
#include <hip/hip_runtime.h>

#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

constexpr int kBStride = kMaxHeadDim + 2;   // fp16 per basis row in LDS: an odd number of
                                            // dwords, so lanes reading one column hit
                                            // distinct banks

__device__ __forceinline__ float half_at(const uint4 (&row)[kMaxHeadDim / 8], int j)
{
    const uint4 v = row[j / 8];
    const uint32_t w = (j & 7) < 2 ? v.x : (j & 7) < 4 ? v.y : (j & 7) < 6 ? v.z : v.w;
    return h2f((uint16_t)(w >> (16 * (j & 1))));
}

// Keeps a value as an fp32 in a register.  The fp16 conversion that follows
// then rounds that fp32 value, as the encoding requires; without it the
// compiler may fold the last multiply-add and the conversion into one
// mixed-precision instruction that rounds the exact sum to fp16 directly.
__device__ __forceinline__ float as_fp32(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// One workgroup of two waves per (sequence, KV head): wave 0 encodes K,
// wave 1 encodes V; both write the same slot of the token's tier.  Every
// input is requested up front (the tier, the token counts -- one lane per
// tier --, the new vector and the basis rows), so the kernel waits for
// memory once.  Lane i holds basis row i in registers for the projection
// and lane j reads column j from LDS for the residual; the other operand
// of each sum is an LDS read at one address for all lanes, so the
// fixed-order sums never wait on memory one term at a time.
template <int D>
__global__ __launch_bounds__(2 * kWave) void append_kernel(Layout ly, uint8_t *arena, int layer,
                                                           const uint16_t *kin, const uint16_t *vin,
                                                           const uint8_t *tier_in,
                                                           const uint16_t *gateK,
                                                           const uint16_t *gateV)
{
    constexpr int NJ = D / kWave;             // channels per lane
    constexpr int RW = D / 8;                 // 16-byte pieces of a basis row
    const int bh = blockIdx.x;
    const int b = bh / ly.Hkv, h = bh % ly.Hkv;
    const int tid = threadIdx.x, z = tid / kWave, lane = lane_id();
    const int R = ly.R, T = ly.T;

    __shared__ uint16_t s_B[2][kMaxRank * kBStride];
    __shared__ __attribute__((aligned(16))) float s_x[2][kMaxHeadDim];
    __shared__ __attribute__((aligned(16))) float s_c[2][kMaxRank];
    __shared__ int8_t s_code[2][kMaxResid];
    __shared__ uint8_t s_idx[2][kMaxResid];

    int32_t *cnt = counts_ptr(ly, arena, layer, b, h);
    const int k = __builtin_amdgcn_readfirstlane(tier_in[bh]);
    const int cnt_l = lane < T ? cnt[lane] : 0;
    const uint16_t *x = (z ? vin : kin) + (int64_t)bh * D;
    float xv[NJ];
#pragma unroll
    for (int q = 0; q < NJ; ++q) xv[q] = h2f(x[lane + q * kWave]);
    const uint16_t *Bg = basis_ptr(ly, arena, layer / ly.G, z, h);
    uint4 brow[2][kMaxHeadDim / 8];           // basis rows lane and lane + 64
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int row = lane + rr * kWave < R ? lane + rr * kWave : 0;
#pragma unroll
        for (int c = 0; c < RW; ++c) brow[rr][c] = reinterpret_cast<const uint4 *>(Bg + (int64_t)row * D)[c];
    }

    // admission: the tier must exist, its region and the position map must
    // have room (decided identically by both waves)
    int n = 0;
#pragma unroll
    for (int kk = 0; kk < kMaxTiers; ++kk) n += kk < T ? __builtin_amdgcn_readlane(cnt_l, kk) : 0;
    int ok = 1, slot = 0;
    if (k >= T) {
        ok = 0;
        if (tid == 0) atomicOr(err_ptr(ly, arena), DWKV_DEVERR_BAD_TIER);
    } else {
        slot = __builtin_amdgcn_readlane(cnt_l, k);
        if (slot >= ly.cap[k]) {
            ok = 0;
            if (tid == 0) atomicOr(err_ptr(ly, arena), DWKV_DEVERR_TIER_FULL);
        }
        if (n >= ly.max_tokens) {
            ok = 0;
            if (tid == 0) atomicOr(err_ptr(ly, arena), DWKV_DEVERR_POS_FULL);
        }
    }
    if (!ok) return;  // uniform across the workgroup
    const int r = ly.rank[k], s = ly.resid[k];
    uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);

    // the rows into LDS for column reads (each wave reads only its own copy)
    uint16_t *sB = s_B[z];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        if (lane + rr * kWave < R) {
            uint32_t *dst = reinterpret_cast<uint32_t *>(sB + (lane + rr * kWave) * kBStride);
#pragma unroll
            for (int c = 0; c < RW; ++c) {
                dst[4 * c + 0] = brow[rr][c].x;
                dst[4 * c + 1] = brow[rr][c].y;
                dst[4 * c + 2] = brow[rr][c].z;
                dst[4 * c + 3] = brow[rr][c].w;
            }
        }
    }

#pragma unroll
    for (int q = 0; q < NJ; ++q) s_x[z][lane + q * kWave] = xv[q];
    wave_fence();

    // 1. coefficients c_i = fp16(sum_j B[i][j] x_j), sequential in j (x read
    //    from LDS, the same address in every lane)
    uint16_t *cdst = reinterpret_cast<uint16_t *>(blk + (z ? ly.f_coefV[k] : ly.f_coefK[k]));
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        if (rr * kWave < r) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < D; ++j) acc = __builtin_fmaf(half_at(brow[rr], j), s_x[z][j], acc);
            const int i = lane + rr * kWave;
            const uint16_t c16 = f2h(as_fp32(acc));
            if (i < r) {
                cdst[z ? coefV_index(r, slot, i) : (int64_t)slot * r + i] = c16;
                s_c[z][i] = h2f(c16);
            }
        }
    }
    wave_fence();

    // 2. residual against the rounded coefficients, sequential in i
    float e[NJ];
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
        const int j = lane + q * kWave;
        float acc = 0.0f;
#pragma unroll 8
        for (int i = 0; i < r; ++i) acc = __builtin_fmaf(h2f(sB[i * kBStride + j]), s_c[z][i], acc);
        e[q] = xv[q] - acc;
    }

    if (s > 0) {
        // 3. the s kept channels: the largest in the order (larger |e| first,
        //    then smaller index).  Keys |e| bits << 8 | (255 - j) order the
        //    channels that way and are distinct; the s-th largest key is
        //    found bit by bit from wave-wide counts (ballots), and the
        //    channels at or above it are kept.  The largest |e| is the top
        //    key's.
        uint64_t key[2] = {0, 0};
#pragma unroll
        for (int q = 0; q < NJ; ++q)
            key[q] = ((uint64_t)__float_as_uint(fabsf(e[q])) << 8) | (uint64_t)(255 - (lane + q * kWave));
        uint64_t thr = 0, top = 0;
#pragma unroll
        for (int bit = 39; bit >= 0; --bit) {
            const uint64_t cand = thr | (1ull << bit);
            const int cnt = __popcll(__ballot(key[0] >= cand)) + (NJ > 1 ? __popcll(__ballot(key[1] >= cand)) : 0);
            if (cnt >= s) thr = cand;
            const uint64_t ctop = top | (1ull << bit);
            const int ctn = __popcll(__ballot(key[0] >= ctop)) + (NJ > 1 ? __popcll(__ballot(key[1] >= ctop)) : 0);
            if (ctn >= 1) top = ctop;
        }
        const float amax = __uint_as_float((uint32_t)(top >> 8));
        bool keep[2] = {false, false};
#pragma unroll
        for (int q = 0; q < NJ; ++q) keep[q] = key[q] >= thr;
        const uint64_t m0 = __ballot(keep[0]);
        const uint64_t m1 = __ballot(keep[1]);
        // 4. one fp16 scale per token: max kept |e| / qmax, correctly rounded
        const uint16_t s16 = f2h(__fdiv_rn(amax, (float)ly.qmax));
        const float sf = h2f(s16);
        // 5. codes, placed in ascending channel order
#pragma unroll
        for (int q = 0; q < NJ; ++q) {
            if (!keep[q]) continue;
            const int j = lane + q * kWave;
            const int pos = q == 0 ? __popcll(m0 & lanemask_lt())
                                   : __popcll(m0) + __popcll(m1 & lanemask_lt());
            float v = 0.0f;
            if (sf != 0.0f) {
                v = rintf(__fdiv_rn(e[q], sf));
                v = fminf(fmaxf(v, -(float)ly.qmax), (float)ly.qmax);
            }
            s_code[z][pos] = static_cast<int8_t>(v);
            s_idx[z][pos] = static_cast<uint8_t>(j);
        }
        wave_fence();
        const int vb = ly.vbytes[k];
        uint8_t *idst = blk + (z ? ly.f_idxV[k] : ly.f_idxK[k]) + (int64_t)slot * ly.istride[k];
        uint8_t *vdst = blk + (z ? ly.f_valV[k] : ly.f_valK[k]) + (int64_t)slot * ly.vstride[k];
        if (lane < s) idst[lane] = s_idx[z][lane];
        if (ly.bits == 8) {
            if (lane < s) vdst[lane] = static_cast<uint8_t>(s_code[z][lane]);
        } else if (lane < vb) {
            const int lo = s_code[z][2 * lane] & 0xF;
            const int hi = (2 * lane + 1 < s) ? (s_code[z][2 * lane + 1] & 0xF) : 0;
            vdst[lane] = static_cast<uint8_t>(lo | (hi << 4));
        }
        // 6. the gate folds into the stored scale
        if (lane == 0) {
            const uint16_t *gp = z ? gateV : gateK;
            const uint16_t g = gp ? gp[bh] : uint16_t(0x3C00);
            const uint16_t stored = (g == 0x3C00) ? s16 : f2h(h2f(g) * sf);
            reinterpret_cast<uint16_t *>(blk + (z ? ly.f_scaleV[k] : ly.f_scaleK[k]))[slot] = stored;
        }
    }
    __syncthreads();
    if (tid == 0) {
        cnt[k] = slot + 1;
        posmap_ptr(ly, arena, layer, b, h)[n] = (k << 28) | slot;
    }
}

}  // namespace

hipError_t launch_append(const Layout &ly, uint8_t *arena, int layer, const void *k,
                         const void *v, const void *tier, const void *gateK, const void *gateV,
                         int batch, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    const auto kern = ly.d == 64 ? append_kernel<64> : append_kernel<128>;
    hipLaunchKernelGGL(kern, dim3(batch * ly.Hkv), dim3(2 * kWave), 0, stream, ly, arena, layer,
                       static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                       static_cast<const uint8_t *>(tier), static_cast<const uint16_t *>(gateK),
                       static_cast<const uint16_t *>(gateV));
    return hipGetLastError();
}

}  // namespace dwkv
