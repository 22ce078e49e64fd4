// Prefill compression of a DepthWeave-KV cache (DepthWeave-KV paper, arXiv
// 2607.06523, §3 Method: after prefill each depth window's shared bases are
// initialised from a randomized low-rank sketch of the cached keys and
// values, per KV head and separately for K and V; then every prefill token
// is projected onto its window's basis and its residual quantised at the
// router's channel count, the data path of Fig. 2).
//
// Three launch families:
//   gram   -- one layer's contribution to its window's Gram matrices
//             C^Z_h = sum over sequences b and positions t < n_b of x x^T:
//             64-token tiles staged through LDS in a transposed, swizzled
//             layout and contracted over tokens on the matrix cores (fp16
//             operands, exact products, fp32 sums per workgroup); the last
//             workgroup of a (Z, h) adds the fp32 partials in fp64, in split
//             order, into the window's fp64 accumulator in the workspace.
//   bases  -- one workgroup per (window, Z, h), in fp64: the randomized
//             range finder with power iterations and a Rayleigh-Ritz step
//             (Halko, Martinsson and Tropp, SIAM Review 2011, §4.5 and §5.3)
//             on C, with Gram-Schmidt twice per column over [Y | I] and a
//             parallel cyclic Jacobi eigensolver (round-robin pairs); the
//             Ritz vectors in decreasing Ritz value, sign-normalised, become
//             the basis rows in fp16 (rounded once from fp64).
//   encode -- a slot pass gives every prefill token its tier slot and
//             position-map entry (an append's admission, for all tokens of a
//             (sequence, KV head) at once); the encoder runs the append's
//             own body (append_body.h) over the tokens, several per wave with
//             the basis rows kept in registers; a publish pass sets the tier
//             counts.
#include <hip/hip_runtime.h>

#include "append_body.h"
#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ Gram

constexpr int kGramTile = 64;       // tokens per LDS tile
constexpr int kGramThreads = 256;

// An 8-token group's place in channel ch's row of a transposed tile.  The
// permutation spreads the fragment reads (16 consecutive channels, one
// group) and the tile writes (channels 8 apart) over the LDS banks.
__device__ __forceinline__ int gram_swz(int ch) { return ((ch >> 1) ^ (ch >> 3)) & 7; }

// fp16 index of (channel ch, tile token t) in a transposed tile.
__device__ __forceinline__ int gram_at(int ch, int t)
{
    return ch * kGramTile + 8 * ((t >> 3) ^ gram_swz(ch)) + (t & 7);
}

// Blocks (I, J), I <= J, of the 16x16 block grid of C, in row order.
__host__ __device__ constexpr int pair_i(int p, int nb)
{
    int i = 0;
    while (p >= nb - i) {
        p -= nb - i;
        ++i;
    }
    return i;
}
__host__ __device__ constexpr int pair_j(int p, int nb)
{
    int i = 0;
    while (p >= nb - i) {
        p -= nb - i;
        ++i;
    }
    return i + p;
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int m)
{
    return m == 0 ? v.x : m == 1 ? v.y : m == 2 ? v.z : v.w;
}

__device__ __forceinline__ float4_t mfma32(half8_t a, half8_t b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The products of wave W's blocks (pairs W, W + 4, ...) for one 32-token
// step: f[c] is the fragment of channel block c.
template <int D, int W>
__device__ __forceinline__ void gram_mma(const half8_t (&f)[D / 16], float4_t (&acc)[(D / 16 * (D / 16 + 1) / 2 + 3) / 4])
{
    constexpr int NB = D / 16, NP = NB * (NB + 1) / 2, PW = (NP + 3) / 4;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int p = W + 4 * i;
        if (p < NP) acc[i] = mfma32(f[pair_i(p, NB)], f[pair_j(p, NB)], acc[i]);
    }
}

template <int D>
__global__ __launch_bounds__(kGramThreads) void gram_kernel(Layout ly, uint8_t *arena, GramArgs a)
{
    constexpr int NB = D / 16, NP = NB * (NB + 1) / 2, PW = (NP + 3) / 4;
    constexpr int CPR = D / 8;                  // 16-byte pieces of a token row
    __shared__ __attribute__((aligned(16))) uint16_t sT[2][D * kGramTile];
    __shared__ int s_tile0[kGramMaxBatch + 1];  // first flat tile of each sequence
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int s = blockIdx.x, zh = blockIdx.y;
    const int z = zh / a.Hkv, h = zh % a.Hkv;
    const uint16_t *X = z ? a.v : a.k;

    if (tid == 0) {
        int f = 0;
        uint32_t bad = 0;
        for (int b = 0; b < a.B; ++b) {
            s_tile0[b] = f;
            int n = a.n_tokens[b];
            if (n < 0 || n > a.n_cap) {
                bad = DWKV_DEVERR_BAD_LENGTH;
                n = n < 0 ? 0 : (int)a.n_cap;
            }
            f += (n + kGramTile - 1) / kGramTile;
        }
        s_tile0[a.B] = f;
        if (bad && s == 0 && zh == 0) atomicOr(err_ptr(ly, arena), bad);
    }
    __syncthreads();
    const int F = s_tile0[a.B];
    const int f0 = (int)((int64_t)F * s / a.S), f1 = (int)((int64_t)F * (s + 1) / a.S);

    // this thread's share of a tile: 4 consecutive tokens x 8 channels
    const bool loader = tid < 2 * D;
    const int col8 = tid % CPR, rowq = tid / CPR;
    uint4 x[4];
    int b = 0;
    auto load = [&](int f) {
        while (f >= s_tile0[b + 1]) ++b;
        int n = a.n_tokens[b];
        n = n < 0 ? 0 : (n > a.n_cap ? (int)a.n_cap : n);
        const int t0 = (f - s_tile0[b]) * kGramTile + 4 * rowq;
        const uint16_t *src = X + ((int64_t)(b * a.Hkv + h) * a.n_cap) * D + 8 * col8;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            x[u] = (loader && t0 + u < n) ? *reinterpret_cast<const uint4 *>(src + (int64_t)(t0 + u) * D)
                                          : make_uint4(0, 0, 0, 0);
    };

    float4_t acc[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    if (f0 < f1) load(f0);
    for (int f = f0, buf = 0; f < f1; ++f, buf ^= 1) {
        // the loaded pieces into the tile, 4 tokens of one channel per store
        if (loader) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t w0 = word(x[0], m), w1 = word(x[1], m), w2 = word(x[2], m), w3 = word(x[3], m);
                const uint2 even = make_uint2((w0 & 0xFFFFu) | (w1 << 16), (w2 & 0xFFFFu) | (w3 << 16));
                const uint2 odd = make_uint2((w0 >> 16) | (w1 & 0xFFFF0000u), (w2 >> 16) | (w3 & 0xFFFF0000u));
                *reinterpret_cast<uint2 *>(&sT[buf][gram_at(8 * col8 + 2 * m, 4 * rowq)]) = even;
                *reinterpret_cast<uint2 *>(&sT[buf][gram_at(8 * col8 + 2 * m + 1, 4 * rowq)]) = odd;
            }
        }
        __syncthreads();
        if (f + 1 < f1) load(f + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            half8_t fr[NB];
            const int g = 4 * ks + (lane >> 4);
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                const int ch = 16 * c + (lane & 15);
                fr[c] = *reinterpret_cast<const half8_t *>(&sT[buf][ch * kGramTile + 8 * (g ^ gram_swz(ch))]);
            }
            switch (wave) {
            case 0: gram_mma<D, 0>(fr, acc); break;
            case 1: gram_mma<D, 1>(fr, acc); break;
            case 2: gram_mma<D, 2>(fr, acc); break;
            default: gram_mma<D, 3>(fr, acc); break;
            }
        }
    }

    // the partial sums, lane-major: element (p, j, lane) of block p is
    // C[16 I + 4 (lane / 16) + j][16 J + lane % 16]
    float *part = a.part + ((int64_t)zh * a.S + s) * NP * 256;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int p = wave + 4 * i;
        if (p < NP) {
#pragma unroll
            for (int j = 0; j < 4; ++j) part[(p * 4 + j) * kWave + lane] = acc[i][j];
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(a.arrive + zh * kArriveStride, 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (uint32_t)(a.S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // the last workgroup: sum the partials in split order, in fp64
    double *C = a.acc + (int64_t)zh * D * D;
    const float *P = a.part + (int64_t)zh * a.S * NP * 256;
    for (int e = tid; e < NP * 256; e += kGramThreads) {
        const int p = e >> 8, j = (e >> 6) & 3, l = e & 63;
        const int row = 16 * pair_i(p, NB) + 4 * (l >> 4) + j, col = 16 * pair_j(p, NB) + (l & 15);
        if (row > col) continue;                   // a diagonal block's lower half mirrors its upper half
        double sum = 0.0;
        for (int q = 0; q < a.S; ++q) sum += (double)__builtin_nontemporal_load(P + (int64_t)q * NP * 256 + e);
        const double v = a.first ? sum : C[row * D + col] + sum;
        C[row * D + col] = v;
        C[col * D + row] = v;
    }
    if (tid == 0)
        __hip_atomic_store(a.arrive + zh * kArriveStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ bases

constexpr int kBasesThreads = 512;
constexpr int kBasesWaves = kBasesThreads / kWave;
constexpr int kColsPerWave = (kMaxSketch + kBasesWaves - 1) / kBasesWaves;

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Sum over the workgroup, the same value in every thread.
__device__ __forceinline__ double block_sum(double v, double *sred)
{
    v = wave_sum_f64(v);
    __syncthreads();
    if (lane_id() == 0) sred[threadIdx.x / kWave] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kBasesWaves; ++w) s += sred[w];
    return s;
}

// fp64 -> fp16, rounded to nearest even once (frexp, ldexp and the division
// by a power of two are exact; rint rounds half to even).
__device__ __forceinline__ uint16_t d2h_rne(double x)
{
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double ax = fabs(x);
    if (!(ax < 65520.0)) return sign | (ax != ax ? 0x7E00 : 0x7C00);
    int e;
    (void)frexp(ax, &e);
    int E = e - 1;
    if (E < -14) E = -14;
    double m = rint(ax / ldexp(1.0, E - 10));
    if (m >= 2048.0) {
        m *= 0.5;
        E += 1;
    }
    if (m < 1024.0) return sign | (uint16_t)m;                  // subnormal (or 0x0400 after rounding up)
    if (E + 15 >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)m - 1024));
}

// W = C Q for the window's Gram matrix C (fp64 [D][D], symmetric, global)
// and Q (LDS [D][k]): lane l computes rows l, l + 64 for its wave's columns.
// Reads row j of C (equal to column j) so that the lanes' loads are
// contiguous.  Writes W into dst after every thread's reads of src.
template <int D>
__device__ void gemm_cq(const double *C, const double *src, double *dst, int k)
{
    constexpr int RI = D / kWave;
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int c0 = w * kColsPerWave;
    double acc[RI][kColsPerWave];
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int cc = 0; cc < kColsPerWave; ++cc) acc[ri][cc] = 0.0;
    for (int j = 0; j < D; ++j) {
        double cj[RI];
#pragma unroll
        for (int ri = 0; ri < RI; ++ri) cj[ri] = C[(int64_t)j * D + lane + kWave * ri];
#pragma unroll
        for (int cc = 0; cc < kColsPerWave; ++cc) {
            if (c0 + cc < k) {
                const double qv = src[j * k + c0 + cc];
#pragma unroll
                for (int ri = 0; ri < RI; ++ri) acc[ri][cc] = fma(cj[ri], qv, acc[ri][cc]);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int cc = 0; cc < kColsPerWave; ++cc)
            if (c0 + cc < k) dst[(lane + kWave * ri) * k + c0 + cc] = acc[ri][cc];
    __syncthreads();
}

// Q (LDS [D][k]) = k orthonormal columns spanning W's: classical
// Gram-Schmidt twice per column over the columns of [W | I], a column kept
// unless its norm after the two passes is at most 2^-40 of its norm before.
template <int D>
__device__ void orth(const double *W, double *Q, int k, double *sv, double *sr, double *sred)
{
    const int tid = threadIdx.x;
    int kept = 0;
    for (int cand = 0; kept < k && cand < k + D; ++cand) {
        if (tid < D) sv[tid] = cand < k ? W[tid * k + cand] : (tid == cand - k ? 1.0 : 0.0);
        double mine = tid < D ? sv[tid] : 0.0;
        const double n0 = sqrt(block_sum(mine * mine, sred));
        for (int pass = 0; pass < 2 && kept > 0; ++pass) {
            if (tid < kept) {
                double p0 = 0.0, p1 = 0.0, p2 = 0.0, p3 = 0.0;
                for (int i = 0; i < D; i += 4) {
                    p0 = fma(Q[i * k + tid], sv[i], p0);
                    p1 = fma(Q[(i + 1) * k + tid], sv[i + 1], p1);
                    p2 = fma(Q[(i + 2) * k + tid], sv[i + 2], p2);
                    p3 = fma(Q[(i + 3) * k + tid], sv[i + 3], p3);
                }
                sr[tid] = (p0 + p1) + (p2 + p3);
            }
            __syncthreads();
            if (tid < D) {
                double p0 = 0.0, p1 = 0.0;
                int cc = 0;
                for (; cc + 1 < kept; cc += 2) {
                    p0 = fma(Q[tid * k + cc], sr[cc], p0);
                    p1 = fma(Q[tid * k + cc + 1], sr[cc + 1], p1);
                }
                if (cc < kept) p0 = fma(Q[tid * k + cc], sr[cc], p0);
                sv[tid] -= p0 + p1;
            }
            __syncthreads();
        }
        mine = tid < D ? sv[tid] : 0.0;
        const double n1 = sqrt(block_sum(mine * mine, sred));
        if (n0 != 0.0 && n1 > 0x1p-40 * n0) {
            if (tid < D) Q[tid * k + kept] = sv[tid] / n1;
            ++kept;
        }
        __syncthreads();
    }
}

__device__ __forceinline__ int rr_index(int pos, int step, int kp)
{
    return pos == 0 ? 0 : 1 + (pos - 1 + step) % (kp - 1);
}

template <int D>
__global__ __launch_bounds__(kBasesThreads) void bases_kernel(Layout ly, uint8_t *arena, BasesArgs a)
{
    __shared__ double sQ[kMaxHeadDim * kMaxSketch];
    __shared__ double sW[kMaxHeadDim * kMaxSketch];
    __shared__ double sv[kMaxHeadDim];
    __shared__ double sr[kMaxSketch + 1];
    __shared__ double sred[kBasesWaves];
    __shared__ double s_c[kMaxSketch / 2 + 1], s_s[kMaxSketch / 2 + 1];
    __shared__ int s_a[kMaxSketch / 2 + 1], s_b[kMaxSketch / 2 + 1];
    __shared__ int s_perm[kMaxSketch];
    __shared__ double s_sgn[kMaxSketch];

    const int tid = threadIdx.x, k = a.k;
    const int zh = blockIdx.x, gi = blockIdx.y;
    const int z = zh / ly.Hkv, h = zh % ly.Hkv;
    const int m = a.group0 + gi;
    const double *C = a.acc + ((int64_t)gi * 2 * ly.Hkv + zh) * D * D;
    const float *om = a.omega + ((int64_t)gi * 2 * ly.Hkv + zh) * D * k;

    // 1. Y = C Omega;  2. Q = orth(Y)
    for (int e = tid; e < D * k; e += kBasesThreads) sQ[e] = (double)om[e];
    __syncthreads();
    gemm_cq<D>(C, sQ, sW, k);
    orth<D>(sW, sQ, k, sv, sr, sred);
    // 3. power iterations
    for (int it = 0; it < a.power_iters; ++it) {
        gemm_cq<D>(C, sQ, sW, k);
        orth<D>(sW, sQ, k, sv, sr, sred);
    }
    // 4. T = Q^T C Q, symmetrised, into sW
    gemm_cq<D>(C, sQ, sW, k);
    {
        constexpr int kPer = (kMaxSketch * kMaxSketch + kBasesThreads - 1) / kBasesThreads;
        double t[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = tid + u * kBasesThreads;
            t[u] = 0.0;
            if (e < k * k) {
                const int ra = e / k, cb = e % k;
                double p0 = 0.0, p1 = 0.0;
                for (int i = 0; i < D; i += 2) {
                    p0 = fma(sQ[i * k + ra], sW[i * k + cb], p0);
                    p1 = fma(sQ[(i + 1) * k + ra], sW[(i + 1) * k + cb], p1);
                }
                t[u] = p0 + p1;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = tid + u * kBasesThreads;
            if (e < k * k) sW[e] = t[u];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = tid + u * kBasesThreads;
            if (e < k * k) t[u] = 0.5 * (sW[e] + sW[(e % k) * k + e / k]);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = tid + u * kBasesThreads;
            if (e < k * k) sW[e] = t[u];
        }
        __syncthreads();
    }
    double *T = sW;

    // 4'. T = U diag(theta) U^T by cyclic Jacobi sweeps over round-robin
    //     pairs (k/2 disjoint rotations at a time), U accumulated into Q
    const int kp = k + (k & 1), P = kp / 2;
    for (int sweep = 0; sweep < kJacobiMaxSweeps; ++sweep) {
        double off = 0.0, all = 0.0;
        for (int e = tid; e < k * k; e += kBasesThreads) {
            const double v = T[e] * T[e];
            all += v;
            if (e / k != e % k) off += v;
        }
        off = block_sum(off, sred);
        all = block_sum(all, sred);
        if (off <= 1e-30 * all) break;
        for (int step = 0; step < kp - 1; ++step) {
            if (tid < P) {
                int pa = rr_index(tid, step, kp), pb = rr_index(kp - 1 - tid, step, kp);
                double c = 1.0, s = 0.0;
                if (pa < k && pb < k) {
                    const double apq = T[pa * k + pb];
                    if (apq != 0.0) {
                        const double tau = (T[pb * k + pb] - T[pa * k + pa]) / (2.0 * apq);
                        const double t = fabs(tau) > 1e150 ? 0.5 / tau
                                                           : (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                        c = 1.0 / sqrt(1.0 + t * t);
                        s = t * c;
                    }
                } else {
                    pa = pb = -1;
                }
                s_a[tid] = pa;
                s_b[tid] = pb;
                s_c[tid] = c;
                s_s[tid] = s;
            }
            __syncthreads();
            // rows: T <- J^T T
            for (int e = tid; e < P * k; e += kBasesThreads) {
                const int p = e / k, j = e % k, pa = s_a[p], pb = s_b[p];
                if (pa < 0 || s_s[p] == 0.0) continue;
                const double c = s_c[p], s = s_s[p];
                const double ta = T[pa * k + j], tb = T[pb * k + j];
                T[pa * k + j] = c * ta - s * tb;
                T[pb * k + j] = s * ta + c * tb;
            }
            __syncthreads();
            // columns: T <- T J, Q <- Q J
            for (int e = tid; e < P * (k + D); e += kBasesThreads) {
                const int p = e / (k + D), i = e % (k + D), pa = s_a[p], pb = s_b[p];
                if (pa < 0 || s_s[p] == 0.0) continue;
                const double c = s_c[p], s = s_s[p];
                double *M = i < k ? T : sQ;
                const int r = i < k ? i : i - k;
                const double ta = M[r * k + pa], tb = M[r * k + pb];
                double na = c * ta - s * tb, nb = s * ta + c * tb;
                if (i < k && r == pa) nb = 0.0;        // the rotated pair's off-diagonal entries
                if (i < k && r == pb) na = 0.0;
                M[r * k + pa] = na;
                M[r * k + pb] = nb;
            }
            __syncthreads();
        }
    }

    // 5. order by decreasing Ritz value (ties: smaller index first), sign
    if (tid < k) {
        const double th = T[tid * k + tid];
        int rank = 0;
        for (int j = 0; j < k; ++j) {
            const double tj = T[j * k + j];
            rank += (tj > th) || (tj == th && j < tid);
        }
        s_perm[rank] = tid;
        int best = 0;
        double bv = fabs(sQ[tid]);
        for (int i = 1; i < D; ++i) {
            const double v = fabs(sQ[i * k + tid]);
            if (v > bv) {
                bv = v;
                best = i;
            }
        }
        s_sgn[tid] = sQ[best * k + tid] < 0.0 ? -1.0 : 1.0;
    }
    __syncthreads();
    // 6. the first r_max Ritz vectors as the basis rows, in fp16
    uint16_t *Bz = basis_ptr(ly, arena, m, z, h);
    for (int e = tid; e < ly.R * D; e += kBasesThreads) {
        const int rho = e / D, i = e % D, col = s_perm[rho];
        Bz[e] = d2h_rne(s_sgn[col] * sQ[i * k + col]);
    }
    if (a.ritz && tid < k) a.ritz[((int64_t)gi * 2 * ly.Hkv + zh) * k + tid] = T[s_perm[tid] * k + s_perm[tid]];
}

// ------------------------------------------------------------------ encode

constexpr int kEncodeThreads = 256;
constexpr int kEncodeTokens = 256;   // tokens per workgroup (each wave: half of them, one Z)

// Tier slots of one (sequence, KV head)'s prefill tokens: admission of all
// of them at once (tiers valid, every tier region and the position map with
// room), then position n0 + t gets (tier << 28 | slot) with slots in
// position order after the tier's counted tokens.  status[b][h] = n0, or -1
// when refused (nothing is written then); newcnt gets the tier counts to
// publish.
__global__ __launch_bounds__(kEncodeThreads) void slots_kernel(Layout ly, uint8_t *arena, EncodeArgs a)
{
    __shared__ int s_tot[kMaxTiers], s_run[kMaxTiers], s_wc[kEncodeThreads / kWave][kMaxTiers];
    __shared__ int s_bad;
    const int bh = blockIdx.x, b = bh / ly.Hkv, h = bh % ly.Hkv;
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int32_t *cnt = counts_ptr(ly, arena, a.layer, b, h);
    if (tid < kMaxTiers) {
        s_tot[tid] = 0;
        s_run[tid] = 0;
    }
    if (tid == 0) s_bad = 0;
    __syncthreads();
    int n = a.n_tokens[b];
    const bool bad_len = n < 0 || n > a.n_cap;
    if (bad_len) n = 0;
    const uint8_t *tier = a.tier + (int64_t)bh * a.n_cap;
    int loc[kMaxTiers] = {0, 0, 0, 0, 0, 0, 0, 0};
    int bad = 0;
    for (int t = tid; t < n; t += kEncodeThreads) {
        const int k = tier[t];
        if (k >= ly.T) bad = 1;
#pragma unroll
        for (int kk = 0; kk < kMaxTiers; ++kk) loc[kk] += k == kk;
    }
#pragma unroll
    for (int kk = 0; kk < kMaxTiers; ++kk)
        if (kk < ly.T && loc[kk]) atomicAdd(&s_tot[kk], loc[kk]);
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    int n0 = 0;
    for (int kk = 0; kk < ly.T; ++kk) n0 += cnt[kk];
    uint32_t err = bad_len ? DWKV_DEVERR_BAD_LENGTH : 0u;
    if (s_bad) err |= DWKV_DEVERR_BAD_TIER;
    for (int kk = 0; kk < ly.T; ++kk)
        if (cnt[kk] + s_tot[kk] > ly.cap[kk]) err |= DWKV_DEVERR_TIER_FULL;
    if ((int64_t)n0 + n > ly.max_tokens) err |= DWKV_DEVERR_POS_FULL;
    if (err) {
        if (tid == 0) {
            atomicOr(err_ptr(ly, arena), err);
            a.status[bh] = -1;
        }
        return;
    }
    int32_t *pm = posmap_ptr(ly, arena, a.layer, b, h) + n0;
    for (int base = 0; base < n; base += kEncodeThreads) {
        const int t = base + tid;
        const int k = t < n ? tier[t] : -1;
        int rank = 0;
#pragma unroll
        for (int kk = 0; kk < kMaxTiers; ++kk) {
            if (kk >= ly.T) break;
            const uint64_t mk = __ballot(k == kk);
            if (k == kk) rank = __popcll(mk & lanemask_lt());
            if (lane == 0) s_wc[w][kk] = __popcll(mk);
        }
        __syncthreads();
        if (k >= 0) {
            int off = s_run[k];
            for (int ww = 0; ww < w; ++ww) off += s_wc[ww][k];
            pm[t] = (k << 28) | (cnt[k] + off + rank);
        }
        __syncthreads();
        if (tid < ly.T)
            for (int ww = 0; ww < kEncodeThreads / kWave; ++ww) s_run[tid] += s_wc[ww][tid];
        __syncthreads();
    }
    if (tid == 0) a.status[bh] = n0;
    if (tid < ly.T) a.newcnt[bh * kMaxTiers + tid] = cnt[tid] + s_tot[tid];
}

// Encodes the tokens [blockIdx.x * kEncodeTokens, +kEncodeTokens) of one
// (sequence, KV head): wave w encodes Z = w % 2 for every other token of
// the range, starting at w / 2, each token exactly as an append would.
template <int D>
__global__ __launch_bounds__(kEncodeThreads) void encode_kernel(Layout ly, uint8_t *arena, EncodeArgs a)
{
    constexpr int NJ = D / kWave;
    constexpr int NW = kEncodeThreads / kWave;
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][kMaxRank * kAppendBStride];
    __shared__ float sx[NW][kMaxHeadDim], sc[NW][kMaxRank];
    __shared__ int8_t scode[NW][kMaxResid];
    __shared__ uint8_t sidx[NW][kMaxResid];

    const int h = blockIdx.y, b = blockIdx.z, bh = b * ly.Hkv + h;
    const int n0 = a.status[bh];
    if (n0 < 0) return;
    const int n = a.n_tokens[b];
    const int t_begin = blockIdx.x * kEncodeTokens;
    if (t_begin >= n) return;
    const int t_end = min(n, t_begin + kEncodeTokens);
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave, z = w & 1;

    uint4 brow[2][D / 8];
    const uint16_t *Bg = basis_ptr(ly, arena, a.layer / ly.G, z, h);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int row = lane + rr * kWave < ly.R ? lane + rr * kWave : 0;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) brow[rr][c] = reinterpret_cast<const uint4 *>(Bg + (int64_t)row * D)[c];
    }
    if (w < 2) encode_stage_basis<D>(brow, sB[z], ly.R, lane);
    __syncthreads();

    const uint16_t *X = (z ? a.v : a.k) + (int64_t)bh * a.n_cap * D;
    const uint16_t *G = z ? a.gateV : a.gateK;
    const int32_t *pm = posmap_ptr(ly, arena, a.layer, b, h) + n0;
    uint8_t *blk = head_block_ptr(ly, arena, a.layer, b, h);
    for (int t = t_begin + (w >> 1); t < t_end; t += 2) {
        float xv[NJ];
#pragma unroll
        for (int q = 0; q < NJ; ++q) xv[q] = h2f(X[(int64_t)t * D + lane + q * kWave]);
        const int e = __builtin_amdgcn_readfirstlane(pm[t]);
        const uint16_t g = G ? G[(int64_t)bh * a.n_cap + t] : uint16_t(0x3C00);
        encode_store<D>(brow, xv, sB[z], sx[w], sc[w], scode[w], sidx[w], ly, blk, e >> 28, e & 0x0FFFFFFF, z,
                        lane, g);
    }
}

// Publishes the encoded tokens: the tier counts of every admitted
// (sequence, KV head).
__global__ void publish_kernel(Layout ly, uint8_t *arena, EncodeArgs a, int n_bh)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n_bh * ly.T) return;
    const int bh = e / ly.T, k = e % ly.T;
    if (a.status[bh] < 0) return;
    counts_ptr(ly, arena, a.layer, bh / ly.Hkv, bh % ly.Hkv)[k] = a.newcnt[bh * kMaxTiers + k];
}

}  // namespace

hipError_t launch_gram(const Layout &ly, uint8_t *arena, const GramArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    const auto kern = ly.d == 64 ? gram_kernel<64> : gram_kernel<128>;
    hipLaunchKernelGGL(kern, dim3(a.S, 2 * a.Hkv), dim3(kGramThreads), 0, stream, ly, arena, a);
    return hipGetLastError();
}

hipError_t launch_bases(const Layout &ly, uint8_t *arena, const BasesArgs &a, int n_groups, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    const auto kern = ly.d == 64 ? bases_kernel<64> : bases_kernel<128>;
    hipLaunchKernelGGL(kern, dim3(2 * ly.Hkv, n_groups), dim3(kBasesThreads), 0, stream, ly, arena, a);
    hipError_t e = hipGetLastError();
    for (int g = 0; g < n_groups && e == hipSuccess; ++g) e = launch_transpose_basis(ly, arena, a.group0 + g, stream);
    return e;
}

hipError_t launch_prefill_encode(const Layout &ly, uint8_t *arena, const EncodeArgs &a, int batch,
                                 hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    hipLaunchKernelGGL(slots_kernel, dim3(batch * ly.Hkv), dim3(kEncodeThreads), 0, stream, ly, arena, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const auto kern = ly.d == 64 ? encode_kernel<64> : encode_kernel<128>;
    const unsigned chunks = (unsigned)((a.n_cap + kEncodeTokens - 1) / kEncodeTokens);
    if (chunks > 0) {
        hipLaunchKernelGGL(kern, dim3(chunks, ly.Hkv, batch), dim3(kEncodeThreads), 0, stream, ly, arena, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int n = batch * ly.Hkv * ly.T;
    hipLaunchKernelGGL(publish_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, ly, arena, a, batch * ly.Hkv);
    return hipGetLastError();
}

}  // namespace dwkv
