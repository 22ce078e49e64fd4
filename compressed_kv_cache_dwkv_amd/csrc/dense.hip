// Uncompressed comparators of the decode path (DepthWeave-KV paper, arXiv
// 2607.06523, §5 Ablation Study: the decode throughput without the fused
// kernel; zhichai.net topic page, Ch. 3.3: base lookup, residual
// dequantisation and attention as launches of their own):
//
//   materialize_kernel -- writes the Eq. (1) reconstruction of every cached
//     token of one layer to a dense fp16 K^/V^ in position order (the "base
//     lookup + residual dequantisation" launch of an unfused decode);
//   dense_decode_kernel -- split-K flash-decode attention over a dense fp16
//     K/V cache (the attention launch of an unfused decode, and the dense
//     baseline the compressed cache is compared against).
//
// Dense cache layout (the caller's buffers): K token rows [B][H_kv][n_cap][d];
// V in 16-token blocks, channel-major inside a block, [B][H_kv][n_cap/16][d][16],
// so that both load straight into matrix-core operands (scores contract over
// channels, value sums over tokens).  n_cap is a multiple of 64.
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kDBlock = 256;               // 4 waves
constexpr int kDWaves = kDBlock / kWave;
constexpr int kDTile = 32;                 // tokens per tile: two 16-token blocks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLag = 8.0f;               // log2 units the running max may trail

__device__ __forceinline__ float4_t mma32(half8_t a, half8_t b, float4_t c)
{
    // D[m][n] += sum_k A[m][k] B[k][n]; lane l supplies A[l%16][8(l/16)+i],
    // B[8(l/16)+i][l%16] (i < 8) and holds D[4(l/16)+j][l%16], j < 4.
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8_t cat(half4_t a, half4_t b)
{
    return half8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ float shfl_xor(float v, int m)
{
    return __shfl_xor(v, m, kWave);
}

// Cross-workgroup partials: agent-scope relaxed atomics, two floats per
// access (the same handoff as the compressed decode's).
__device__ __forceinline__ void st_agent(float *p, float x)
{
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_agent(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ dense decode
template <int GQ, int D>
__global__ __launch_bounds__(kDBlock) void dense_decode_kernel(DenseArgs a)
{
    constexpr int NC = D / 32;                 // 32-channel chunks of the scores
    constexpr int NB = D / 16;                 // 16-channel blocks of the output
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int S = gridDim.x;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int c16 = lane & 15, g = lane >> 4;
    const int n = a.n[b * a.Hkv + h];
    const int nt = (n + kDTile - 1) / kDTile;
    const int t0 = (int)((int64_t)nt * split / S), t1 = (int)((int64_t)nt * (split + 1) / S);
    const uint16_t *Kb = a.k + ((int64_t)b * a.Hkv + h) * a.n_cap * D;
    const uint16_t *Vb = a.v + ((int64_t)b * a.Hkv + h) * a.n_cap * D;

    // scores' B operand: q of head c16 (zero past the group), channels
    // 32 c + 8 g ..
    half8_t qop[NC];
    {
        const uint16_t *qr = a.q + ((int64_t)b * a.Hq + h * GQ + (c16 < GQ ? c16 : 0)) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const half8_t v = *reinterpret_cast<const half8_t *>(qr + 32 * c + 8 * g);
            qop[c] = c16 < GQ ? v : half8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    const float zs = a.scale * kLog2e;
    float4_t O[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) O[cb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY;                      // running max of head c16 (base-2 logits)
    float l = 0.0f;                           // this lane's share of head c16's normaliser

    for (int t = t0 + wave; t < t1; t += kDWaves) {
        const int tok0 = t * kDTile;
        // K operand of 16-token block mb: token tok0 + 16 mb + c16, channels
        // 32 c + 8 g ..; V operand of output block cb: channel 16 cb + c16,
        // tokens 4 g .. 4 g + 3 of both blocks (the same token order as the
        // probabilities' operand below)
        half8_t kop[2][NC];
        half8_t vop[NB];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int tok = tok0 + 16 * mb + c16;
#pragma unroll
            for (int c = 0; c < NC; ++c) kop[mb][c] = *reinterpret_cast<const half8_t *>(Kb + (int64_t)tok * D + 32 * c + 8 * g);
        }
        const uint16_t *vb = Vb + ((int64_t)(tok0 / 16) * D) * 16 + 4 * g;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            const half4_t lo = *reinterpret_cast<const half4_t *>(vb + (16 * cb + c16) * 16);
            const half4_t hi = *reinterpret_cast<const half4_t *>(vb + (D + 16 * cb + c16) * 16);
            vop[cb] = cat(lo, hi);
        }
        // tokens of the tile that exist; operands of the others are zeroed
        // (whatever the buffer holds there must not meet a zero probability)
        const int left = n - tok0;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
            if (16 * mb + c16 >= left) {
#pragma unroll
                for (int c = 0; c < NC; ++c) kop[mb][c] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
            }
        if (left < kDTile) {
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (16 * (i >> 2) + 4 * g + (i & 3) >= left) vop[cb][i] = (_Float16)0.0f;
        }
        // scores: lane holds tokens 16 mb + 4 g + j of the tile for head c16
        float4_t s0 = float4_t{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            s0 = mma32(kop[0][c], qop[c], s0);
            s1 = mma32(kop[1][c], qop[c], s1);
        }
        float z[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            z[j] = 4 * g + j < left ? s0[j] * zs : -INFINITY;
            z[4 + j] = 16 + 4 * g + j < left ? s1[j] * zs : -INFINITY;
        }
        float tm = z[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tm = fmaxf(tm, z[i]);
        tm = fmaxf(tm, shfl_xor(tm, 16));
        tm = fmaxf(tm, shfl_xor(tm, 32));
        // lazy running max: moved (and the sums rescaled) only when a logit
        // passes it by more than the lag
        if (__builtin_amdgcn_ballot_w64(tm > m + kLag)) {
            const float nm = tm > m + kLag ? tm : m;
            const float f = m == -INFINITY ? 0.0f : exp2f(m - nm);
            m = nm;
            l *= f;
            // accumulator row 4 g + j is head 4 g + j: its factor from that head's lane
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fr = __shfl(f, 4 * g + j, kWave);
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) O[cb][j] *= fr;
            }
        }
        half8_t P;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 p = (_Float16)exp2f(z[i] - m);
            P[i] = p;
            l += (float)p;
        }
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) O[cb] = mma32(P, vop[cb], O[cb]);
    }

    // ---- this workgroup's waves merged through LDS
    __shared__ float s_m[kDWaves][GQ], s_l[kDWaves][GQ];
    __shared__ float s_o[kDWaves][GQ][D];
    __shared__ int s_last;
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (g == 0 && c16 < GQ) {
        s_m[wave][c16] = m;
        s_l[wave][c16] = l;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int hd = 4 * g + j;
        if (hd < GQ) {
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) s_o[wave][hd][16 * cb + c16] = O[cb][j];
        }
    }
    __syncthreads();
    // partial of this split: (max, normaliser, unnormalised output) per head
    float *po = a.ws.po, *pm = a.ws.pm;
    for (int e = tid; e < GQ * D; e += kDBlock) {
        const int hd = e / D, ch = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDWaves; ++w) M = fmaxf(M, s_m[w][hd]);
        float o = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < kDWaves; ++w) {
            const float f = M == -INFINITY ? 0.0f : exp2f(s_m[w][hd] - M);
            o += f * s_o[w][hd][ch];
            L += f * s_l[w][hd];
        }
        st_agent(po + (((int64_t)b * a.Hq + h * GQ + hd) * S + split) * D + ch, o);
        if (ch == 0) {
            const int64_t ml = (((int64_t)b * a.Hkv + h) * S + split) * kMlStride + hd;
            st_agent(pm + ml, M);
            st_agent(pm + ml + kMlNorm, L);
        }
    }
    // the last workgroup of this (sequence, KV head) merges the splits
    // (every store acknowledged before the arrival is counted)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&a.ws.arrive[(b * a.Hkv + h) * kArriveStride], 1u,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    for (int e = tid; e < GQ * D; e += kDBlock) {
        const int hd = e / D, ch = e % D;
        const int64_t ml0 = (((int64_t)b * a.Hkv + h) * S) * kMlStride + hd;
        float M = -INFINITY;
        for (int sp = 0; sp < S; ++sp) M = fmaxf(M, ld_agent(pm + ml0 + (int64_t)sp * kMlStride));
        float o = 0.0f, L = 0.0f;
        const float *pb = po + ((int64_t)b * a.Hq + h * GQ + hd) * S * D + ch;
        for (int sp = 0; sp < S; ++sp) {
            const float ms = ld_agent(pm + ml0 + (int64_t)sp * kMlStride);
            const float f = M == -INFINITY ? 0.0f : exp2f(ms - M);
            o += f * ld_agent(pb + (int64_t)sp * D);
            L += f * ld_agent(pm + ml0 + (int64_t)sp * kMlStride + kMlNorm);
        }
        a.out[((int64_t)b * a.Hq + h * GQ + hd) * D + ch] = L > 0.0f ? o / L : 0.0f;
    }
    if (tid == 0)
        __hip_atomic_store(&a.ws.arrive[(b * a.Hkv + h) * kArriveStride], 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------- materialisation
// One workgroup per 64 positions of one (sequence, KV head): each position's
// (tier, slot) from the position map, its coefficients gathered into LDS,
// the basis products on the matrix cores (coefficients times the transposed
// basis, 16 tokens x 16 channels per product, fp32 sums of exact fp16
// products), the residual channels added in fp32, one rounding to fp16.
constexpr int kMTok = 64;
constexpr int kMBlock = 256;

template <int D, int RM>
__global__ __launch_bounds__(kMBlock) void materialize_kernel(Layout ly, uint8_t *arena, int layer,
                                                              uint16_t *kout, uint16_t *vout, int64_t n_cap,
                                                              int32_t *n_out)
{
    constexpr int BS = RM + 8;                 // fp16 per transposed-basis row (padded)
    constexpr int CS = RM + 8;                 // fp16 per coefficient row
    constexpr int OS = D + 4;                  // fp32 per output row
    __shared__ __attribute__((aligned(16))) uint16_t s_bt[D * BS];      // basis^T [channel][rank]
    __shared__ __attribute__((aligned(16))) uint16_t s_c[kMTok * CS];    // coefficients [token][rank]
    __shared__ __attribute__((aligned(16))) float s_out[kMTok * OS];     // reconstruction [token][channel]
    __shared__ int s_tier[kMTok], s_slot[kMTok];
    const int p0 = blockIdx.x * kMTok, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int c16 = lane & 15, g = lane >> 4;
    const int32_t *cnt = counts_ptr(ly, arena, layer, b, h);
    int n = 0;
    for (int k = 0; k < ly.T; ++k) n += cnt[k];
    if (p0 == 0 && tid == 0 && n_out) n_out[b * ly.Hkv + h] = n;
    if (p0 >= n) return;
    const int32_t *pm = posmap_ptr(ly, arena, layer, b, h);
    if (tid < kMTok) {
        const int p = p0 + tid;
        const int e = p < n ? pm[p] : -1;
        s_tier[tid] = e < 0 ? -1 : (e >> 28);
        s_slot[tid] = e < 0 ? 0 : (e & 0x0FFFFFFF);
    }
    const uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);
    const int R = ly.R;
    for (int z = 0; z < 2; ++z) {
        __syncthreads();
        // transposed basis of this Z (zero past R)
        const uint16_t *Bz = basis_ptr(ly, arena, layer / ly.G, z, h);
        for (int e = tid; e < RM * D; e += kMBlock) {
            const int i = e / D, j = e % D;
            s_bt[j * BS + i] = i < R ? Bz[(int64_t)i * D + j] : (uint16_t)0;
        }
        // coefficients of the 64 positions (zero past each token's rank)
        for (int e = tid; e < kMTok * RM; e += kMBlock) {
            const int t = e / RM, i = e % RM;
            const int k = s_tier[t];
            uint16_t c = 0;
            if (k >= 0 && k < ly.T) {
                const int r = ly.rank[k];
                const int64_t slot = s_slot[t];
                if (i < r) {
                    const uint16_t *src = reinterpret_cast<const uint16_t *>(blk + (z ? ly.f_coefV[k] : ly.f_coefK[k]));
                    c = z ? src[coefV_index(r, slot, i)] : src[slot * r + i];
                }
            }
            s_c[t * CS + i] = c;
        }
        __syncthreads();
        // wave w: tokens 16 w .. 16 w + 15, every 16-channel block
        {
            const int tok = 16 * wave + c16;
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb) {
                float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int k0 = 0; k0 < RM; k0 += 32) {
                    const half8_t av = *reinterpret_cast<const half8_t *>(&s_c[tok * CS + k0 + 8 * g]);
                    const half8_t bv = *reinterpret_cast<const half8_t *>(&s_bt[(16 * cb + c16) * BS + k0 + 8 * g]);
                    acc = mma32(av, bv, acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) s_out[(16 * wave + 4 * g + j) * OS + 16 * cb + c16] = acc[j];
            }
        }
        __syncthreads();
        // residual channels: one thread per token
        if (tid < kMTok) {
            const int k = s_tier[tid];
            if (k >= 0 && k < ly.T) {
                const int s = ly.resid[k];
                const int64_t slot = s_slot[tid];
                if (s > 0) {
                    const uint8_t *idx = blk + (z ? ly.f_idxV[k] : ly.f_idxK[k]) + slot * ly.istride[k];
                    const uint8_t *val = blk + (z ? ly.f_valV[k] : ly.f_valK[k]) + slot * ly.vstride[k];
                    const float sc = h2f(reinterpret_cast<const uint16_t *>(blk + (z ? ly.f_scaleV[k] : ly.f_scaleK[k]))[slot]);
                    for (int u = 0; u < s; ++u) {
                        const int j = idx[u] < D ? idx[u] : D - 1;
                        s_out[tid * OS + j] += sc * (float)unpack_code(val, u, ly.bits);
                    }
                }
            }
        }
        __syncthreads();
        // fp16 out: K rows, V 16-token blocks (channel-major); positions past
        // the context are written as zeros
        uint16_t *dst = (z ? vout : kout) + ((int64_t)b * ly.Hkv + h) * n_cap * D;
        for (int e = tid; e < kMTok * D; e += kMBlock) {
            int t, j;
            if (z == 0) {
                t = e / D;
                j = e % D;
            } else {
                // element order of the blocked layout: [block][channel][token]
                const int blk16 = e / (16 * D), rem = e % (16 * D);
                j = rem / 16;
                t = 16 * blk16 + rem % 16;
            }
            const uint16_t v = p0 + t < n ? f2h(s_out[t * OS + j]) : (uint16_t)0;
            if (z == 0)
                dst[(int64_t)(p0 + t) * D + j] = v;
            else
                dst[((int64_t)(p0 + t) / 16 * D + j) * 16 + (p0 + t) % 16] = v;
        }
    }
}

template <int GQ, int D>
hipError_t launch_dense_gq(const DenseArgs &a, int splits, hipStream_t stream)
{
    hipLaunchKernelGGL((dense_decode_kernel<GQ, D>), dim3(splits, a.Hkv, a.B), dim3(kDBlock), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dense_d(const DenseArgs &a, int splits, hipStream_t stream)
{
    switch (a.Hq / a.Hkv) {
    case 1: return launch_dense_gq<1, D>(a, splits, stream);
    case 2: return launch_dense_gq<2, D>(a, splits, stream);
    case 4: return launch_dense_gq<4, D>(a, splits, stream);
    case 8: return launch_dense_gq<8, D>(a, splits, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_dense_decode(const DenseArgs &a, int splits, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    if (a.d == 64) return launch_dense_d<64>(a, splits, stream);
    if (a.d == 128) return launch_dense_d<128>(a, splits, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_materialize(const Layout &ly, uint8_t *arena, int layer, int batch, uint16_t *kout,
                              uint16_t *vout, int64_t n_cap, int32_t *n_out, hipStream_t stream)
{
    (void)hipGetLastError();
    const dim3 grid((unsigned)(n_cap / kMTok), ly.Hkv, batch);
    if (ly.d == 128 && ly.R <= 64)
        hipLaunchKernelGGL((materialize_kernel<128, 64>), grid, dim3(kMBlock), 0, stream, ly, arena, layer, kout, vout,
                           n_cap, n_out);
    else if (ly.d == 128)
        hipLaunchKernelGGL((materialize_kernel<128, 128>), grid, dim3(kMBlock), 0, stream, ly, arena, layer, kout,
                           vout, n_cap, n_out);
    else if (ly.R <= 64)
        hipLaunchKernelGGL((materialize_kernel<64, 64>), grid, dim3(kMBlock), 0, stream, ly, arena, layer, kout, vout,
                           n_cap, n_out);
    else
        hipLaunchKernelGGL((materialize_kernel<64, 128>), grid, dim3(kMBlock), 0, stream, ly, arena, layer, kout, vout,
                           n_cap, n_out);
    return hipGetLastError();
}

}  // namespace dwkv
