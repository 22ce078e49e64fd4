// Decode attention over the compressed cache (DepthWeave-KV paper, arXiv
// 2607.06523, §3 Method, Eq. (1) and the decoding data path of the last
// paragraph before Fig. 2): basis lookup, residual dequantisation,
// coefficient multiply and attention in one pass, with no reconstructed K or
// V ever written to memory.
//
// Algebra used (exact rewrites of Eq. (1)):
//   q . K^_t = (B_K q)[0:r_t] . c^K_t + scale^K_t * sum_u q[idx^K_{t,u}] code^K_{t,u}
//   sum_t p_t V^_t = B_V^T (sum_t p_t c^V_t) + sum_t p_t scale^V_t sum_u code^V_{t,u} e_{idx^V_{t,u}}
// so a query is projected once into the basis' coordinates (q' = B_K q), the
// values are accumulated in basis coordinates plus a dense residual-mass
// vector, and B_V is applied once per workgroup at the end.
//
// Work split (split-K "flash decode"): grid = (splits, KV heads, sequences).
// A workgroup takes a byte-balanced slice of the concatenated tier regions
// of its (sequence, KV head), runs an online softmax in base-2 units, and
// writes (running max, normaliser, unnormalised output) partials; the last
// workgroup of each (sequence, KV head) to arrive merges them.
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr float kLog2e = 1.4426950408889634f;

// First token of a tier whose byte offset (t * w) is >= x.
__device__ __forceinline__ int64_t first_token_at(int64_t x, int w)
{
    return x <= 0 ? 0 : (x + w - 1) / w;
}

template <int GQ>
__global__ __launch_bounds__(kBlock) void decode_kernel(Layout ly, uint8_t *arena, int layer,
                                                        const uint16_t *q, float *out,
                                                        DecodeWorkspace ws, int S, float qscale)
{
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int d = ly.d, R = ly.R;
    const int g0 = h * GQ;

    __shared__ float s_qt[GQ][kMaxHeadDim];          // q in base-2 logit units
    __shared__ float s_qp[GQ][kMaxRank];             // B_K q, later the merged basis accumulator
    __shared__ float s_rho[kWaves][GQ][kMaxHeadDim]; // residual-value mass per wave
    __shared__ float s_accw[kWaves][GQ][kMaxRank];   // basis accumulator per wave
    __shared__ float s_m[kWaves][GQ], s_l[kWaves][GQ], s_f[kWaves][GQ];
    __shared__ float s_M[GQ], s_L[GQ];
    __shared__ int s_last;

    for (int i = tid; i < GQ * kMaxHeadDim; i += kBlock) {
        const int g = i / kMaxHeadDim, j = i % kMaxHeadDim;
        s_qt[g][j] = j < d ? qscale * h2f(q[((int64_t)b * ly.Hq + g0 + g) * d + j]) : 0.0f;
    }
    for (int i = tid; i < kWaves * GQ * kMaxHeadDim; i += kBlock) (&s_rho[0][0][0])[i] = 0.0f;
    __syncthreads();
    // a1: q' = B_K q for every query head of the group
    const uint16_t *BK = basis_ptr(ly, arena, layer / ly.G, 0, h);
    for (int i = tid; i < GQ * kMaxRank; i += kBlock) {
        const int g = i / kMaxRank, ii = i % kMaxRank;
        float acc = 0.0f;
        if (ii < R)
            for (int j = 0; j < d; ++j) acc += h2f(BK[(int64_t)ii * d + j]) * s_qt[g][j];
        s_qp[g][ii] = acc;
    }
    __syncthreads();

    // this workgroup's byte-balanced slice of the tier regions
    const int32_t *cnt = counts_ptr(ly, arena, layer, b, h);
    int64_t W = 0;
    for (int k = 0; k < ly.T; ++k) W += (int64_t)cnt[k] * ly.weight[k];
    const int64_t lo = W * split / S, hi = W * (split + 1) / S;

    float m[GQ], l[GQ], a0[GQ], a1[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
        a0[g] = 0.0f;
        a1[g] = 0.0f;
    }
    const uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);
    int64_t wk = 0;
    for (int k = 0; k < ly.T; ++k) {
        const int w = ly.weight[k];
        const int64_t ck = cnt[k];
        int64_t t0 = first_token_at(lo - wk, w), t1 = first_token_at(hi - wk, w);
        wk += ck * w;
        t0 = t0 < ck ? t0 : ck;
        t1 = t1 < ck ? t1 : ck;
        if (t1 <= t0) continue;
        const int64_t len = t1 - t0;
        const int64_t wt0 = t0 + len * wave / kWaves, wt1 = t0 + len * (wave + 1) / kWaves;
        const int r = ly.rank[k], s = ly.resid[k], vb = ly.vbytes[k];
        const uint16_t *cK = reinterpret_cast<const uint16_t *>(blk + ly.f_coefK[k]);
        const uint16_t *cV = reinterpret_cast<const uint16_t *>(blk + ly.f_coefV[k]);
        const uint8_t *iK = blk + ly.f_idxK[k], *iV = blk + ly.f_idxV[k];
        const uint8_t *vK = blk + ly.f_valK[k], *vV = blk + ly.f_valV[k];
        const uint16_t *sK = reinterpret_cast<const uint16_t *>(blk + ly.f_scaleK[k]);
        const uint16_t *sV = reinterpret_cast<const uint16_t *>(blk + ly.f_scaleV[k]);
        for (int64_t t = wt0; t < wt1; ++t) {
            // score in basis coordinates plus the sparse residual term
            const float c0 = lane < r ? h2f(cK[t * r + lane]) : 0.0f;
            const float c1 = lane + kWave < r ? h2f(cK[t * r + lane + kWave]) : 0.0f;
            float part[GQ];
#pragma unroll
            for (int g = 0; g < GQ; ++g) part[g] = c0 * s_qp[g][lane] + c1 * s_qp[g][lane + kWave];
            if (lane < s) {
                const int j = iK[t * s + lane];
                const float wv = h2f(sK[t]) * (float)unpack_code(vK + t * vb, lane, ly.bits);
#pragma unroll
                for (int g = 0; g < GQ; ++g) part[g] += wv * s_qt[g][j];
            }
            float p[GQ];
#pragma unroll
            for (int g = 0; g < GQ; ++g) {
                const float zz = wave_sum(part[g]);
                const float mn = fmaxf(m[g], zz);
                const float corr = exp2f(m[g] - mn);
                p[g] = exp2f(zz - mn);
                l[g] = l[g] * corr + p[g];
                a0[g] *= corr;
                a1[g] *= corr;
                if (corr != 1.0f) {
                    s_rho[wave][g][lane] *= corr;
                    s_rho[wave][g][lane + kWave] *= corr;
                }
                m[g] = mn;
            }
            // values in basis coordinates plus the residual mass
            const float v0 = lane < r ? h2f(cV[t * r + lane]) : 0.0f;
            const float v1 = lane + kWave < r ? h2f(cV[t * r + lane + kWave]) : 0.0f;
#pragma unroll
            for (int g = 0; g < GQ; ++g) {
                a0[g] += p[g] * v0;
                a1[g] += p[g] * v1;
            }
            if (lane < s) {
                const int j = iV[t * s + lane];
                const float wv = h2f(sV[t]) * (float)unpack_code(vV + t * vb, lane, ly.bits);
#pragma unroll
                for (int g = 0; g < GQ; ++g) s_rho[wave][g][j] += p[g] * wv;
            }
        }
    }

    // merge the four waves
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
            s_m[wave][g] = m[g];
            s_l[wave][g] = l[g];
        }
    }
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
        s_accw[wave][g][lane] = a0[g];
        s_accw[wave][g][lane + kWave] = a1[g];
    }
    __syncthreads();
    if (tid < GQ) {
        const int g = tid;
        float M = -INFINITY;
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
        float L = 0.0f;
        for (int w = 0; w < kWaves; ++w) {
            const float f = M == -INFINITY ? 0.0f : exp2f(s_m[w][g] - M);
            s_f[w][g] = f;
            L += f * s_l[w][g];
        }
        s_M[g] = M;
        s_L[g] = L;
    }
    __syncthreads();
    for (int i = tid; i < GQ * kMaxRank; i += kBlock) {
        const int g = i / kMaxRank, ii = i % kMaxRank;
        float acc = 0.0f;
        for (int w = 0; w < kWaves; ++w) acc += s_f[w][g] * s_accw[w][g][ii];
        s_qp[g][ii] = acc;
    }
    __syncthreads();
    // a single back-projection through B_V, plus the residual mass
    const uint16_t *BV = basis_ptr(ly, arena, layer / ly.G, 1, h);
    for (int i = tid; i < GQ * d; i += kBlock) {
        const int g = i / d, j = i % d;
        float o = 0.0f;
        for (int ii = 0; ii < R; ++ii) o += h2f(BV[(int64_t)ii * d + j]) * s_qp[g][ii];
        for (int w = 0; w < kWaves; ++w) o += s_f[w][g] * s_rho[w][g][j];
        ws.po[(((int64_t)b * ly.Hq + g0 + g) * S + split) * d + j] = o;
    }
    if (tid < GQ) {
        ws.pm[((int64_t)b * ly.Hq + g0 + tid) * S + split] = s_M[tid];
        ws.pl[((int64_t)b * ly.Hq + g0 + tid) * S + split] = s_L[tid];
    }

    // a3: the last workgroup of this (sequence, KV head) merges the splits
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&ws.arrive[b * ly.Hkv + h], 1u);
        s_last = prev == (uint32_t)(S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (tid < GQ) {
        const float *pm = ws.pm + ((int64_t)b * ly.Hq + g0 + tid) * S;
        const float *pl = ws.pl + ((int64_t)b * ly.Hq + g0 + tid) * S;
        float M = -INFINITY;
        for (int i = 0; i < S; ++i) M = fmaxf(M, pm[i]);
        float L = 0.0f;
        if (M != -INFINITY)
            for (int i = 0; i < S; ++i) L += exp2f(pm[i] - M) * pl[i];
        s_M[tid] = M;
        s_L[tid] = L;
    }
    __syncthreads();
    for (int i = tid; i < GQ * d; i += kBlock) {
        const int g = i / d, j = i % d;
        const float M = s_M[g];
        float o = 0.0f;
        if (M != -INFINITY) {
            const float *pm = ws.pm + ((int64_t)b * ly.Hq + g0 + g) * S;
            const float *po = ws.po + ((int64_t)b * ly.Hq + g0 + g) * S * d + j;
            for (int sp = 0; sp < S; ++sp) o += exp2f(pm[sp] - M) * po[(int64_t)sp * d];
            o /= s_L[g];
        }
        out[((int64_t)b * ly.Hq + g0 + g) * d + j] = o;
    }
    if (tid == 0) ws.arrive[b * ly.Hkv + h] = 0u;
}

}  // namespace

hipError_t launch_decode(const Layout &ly, uint8_t *arena, int layer, const void *q, int batch,
                         float softmax_scale, float *out, const DecodeWorkspace &ws, int splits,
                         hipStream_t stream)
{
    const dim3 grid(splits, ly.Hkv, batch);
    const float qs = softmax_scale * kLog2e;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    switch (ly.gq) {
    case 1: hipLaunchKernelGGL(decode_kernel<1>, grid, dim3(kBlock), 0, stream, ly, arena, layer, qq, out, ws, splits, qs); break;
    case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, dim3(kBlock), 0, stream, ly, arena, layer, qq, out, ws, splits, qs); break;
    case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, dim3(kBlock), 0, stream, ly, arena, layer, qq, out, ws, splits, qs); break;
    case 8: hipLaunchKernelGGL(decode_kernel<8>, grid, dim3(kBlock), 0, stream, ly, arena, layer, qq, out, ws, splits, qs); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dwkv
