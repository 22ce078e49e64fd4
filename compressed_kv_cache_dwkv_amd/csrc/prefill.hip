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
//             64-token tiles, two in flight per workgroup, staged through
//             LDS in a transposed, swizzled layout and contracted over
//             tokens on the matrix cores (fp16
//             operands, exact products, fp32 sums per workgroup); a second
//             kernel adds each element's fp32 partials in fp64, in split
//             order, into the window's fp64 accumulator in the workspace.
//   bases  -- one workgroup per (window, Z, h), in fp64: the randomized
//             range finder with power iterations and a Rayleigh-Ritz step
//             (Halko, Martinsson and Tropp, SIAM Review 2011, §4.5 and §5.3)
//             on C, with Gram-Schmidt twice per column over [Y | I] (or
//             two CholeskyQR passes where they keep exactly Y's columns) and
//             a parallel cyclic Jacobi eigensolver (round-robin pairs); the
//             Ritz vectors in decreasing Ritz value, sign-normalised, become
//             the basis rows in fp16 (rounded once from fp64).
//   encode -- count and place passes give every prefill token its tier slot and
//             position-map entry (an append's admission, for all tokens of a
//             (sequence, KV head) at once) and lists the tokens by tier; the
//             encoder takes 64 tokens of one tier per wave, one per lane, and
//             follows the append's order of operations exactly (so it gives
//             the append's bits), the fp16 basis values reaching every
//             lane through scalar loads as operands of mixed-precision
//             FMAs; a publish pass sets the tier counts.
#include <hip/hip_runtime.h>

#include <type_traits>

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
// step: f[c] is the fragment of channel block c.  The block indices are
// template arguments, so every operand is a fixed register.
template <int D, int W, int IDX>
__device__ __forceinline__ void gram_mma(const half8_t (&f)[D / 16], float4_t (&acc)[(D / 16 * (D / 16 + 1) / 2 + 3) / 4])
{
    constexpr int NB = D / 16, NP = NB * (NB + 1) / 2, P = W + 4 * IDX;
    if constexpr (P < NP) {
        constexpr int I = pair_i(P, NB), J = pair_j(P, NB);
        acc[IDX] = mfma32(f[I], f[J], acc[IDX]);
        gram_mma<D, W, IDX + 1>(f, acc);
    }
}

template <int D>
__global__ __launch_bounds__(kGramThreads) void gram_kernel(Layout ly, uint8_t *arena, GramArgs a)
{
    constexpr int NB = D / 16, NP = NB * (NB + 1) / 2, PW = (NP + 3) / 4;
    constexpr int CPR = D / 8;                  // 16-byte pieces of a token row
    __shared__ __attribute__((aligned(16))) uint16_t sT[2][D * kGramTile];
    __shared__ int s_tile0[kGramMaxBatch + 1];  // first flat tile of each sequence
    __shared__ int s_len[kGramMaxBatch];        // its length, clamped to [0, n_cap]

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
            s_len[b] = n;
            f += (n + kGramTile - 1) / kGramTile;
        }
        s_tile0[a.B] = f;
        if (bad && s == 0 && zh == 0) atomicOr(err_ptr(ly, arena), bad);
    }
    __syncthreads();
    const int F = s_tile0[a.B];
    const int f0 = (int)((int64_t)F * s / a.S), f1 = (int)((int64_t)F * (s + 1) / a.S);

    // this thread's share of a tile: 4 consecutive tokens x 8 channels; two
    // tiles are in flight (the loads of tiles f + 1 and f + 2 while tile f
    // is contracted)
    const bool loader = tid < 2 * D;
    const int col8 = tid % CPR, rowq = tid / CPR;
    uint4 xa[4], xb[4];
    int b = 0;
    auto load = [&](int f, uint4 (&x)[4]) {
        // (the length from LDS: a global load here would make the tile
        // loads wait for every load in flight)
        while (b < a.B - 1 && f >= s_tile0[b + 1]) ++b;
        const int n = f < f1 ? s_len[b] : 0;    // past this workgroup's share: zeros
        const int t0 = (f - s_tile0[b]) * kGramTile + 4 * rowq;
        // buffer loads over the sequence's first n rows: rows past them read
        // as zeros, and every load is issued, so the waits count the loads
        // in flight exactly
        const __amdgpu_buffer_rsrc_t rs = block_rsrc(X + (int64_t)(b * a.Hkv + h) * a.n_cap * D, (int64_t)n * D * 2);
        const uint32_t off = (uint32_t)t0 * (D * 2) + 16u * col8;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + (uint32_t)(u * D * 2), 0, 0);
            x[u] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };

    float4_t acc[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // tile f (registers x) into LDS buffer buf, then wave W's products; the
    // loads of tile f + 2 go into x once it is stored
    auto step = [&](auto wtag, int f, int buf, uint4 (&x)[4]) {
        constexpr int W = decltype(wtag)::value;
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
        load(f + 2 < f1 ? f + 2 : f1, x);       // past the share: zeros
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            half8_t fr[NB];
            const int g = 4 * ks + (lane >> 4);
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                const int ch = 16 * c + (lane & 15);
                fr[c] = *reinterpret_cast<const half8_t *>(&sT[buf][ch * kGramTile + 8 * (g ^ gram_swz(ch))]);
            }
            gram_mma<D, W, 0>(fr, acc);
        }
    };
    // whole pairs of tiles (an odd count ends with a tile of zeros: index
    // f1, whose loads all read past the rows), so that every pass through
    // the loop issues its loads in the same order; one copy of the loop per
    // wave, so that each wave's block list is fixed in its code
    auto run = [&](auto wtag) {
        if (f0 < f1) {
            load(f0, xa);
            load(f0 + 1, xb);
            for (int f = f0; f < f1; f += 2) {
                step(wtag, f, 0, xa);
                step(wtag, f + 1, 1, xb);
            }
        }
    };
    switch (wave) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    default: run(std::integral_constant<int, 3>{}); break;
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
}

// Sums the S partials of each Gram element in split order, in fp64, into
// the window's accumulator (or over it with a.first), and mirrors it: one
// thread per element of the blocks on and above the diagonal.
template <int D>
__global__ __launch_bounds__(256) void gram_reduce_kernel(GramArgs a)
{
    constexpr int NB = D / 16, NP = NB * (NB + 1) / 2;
    const int zh = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
    if (e >= NP * 256) return;
    const int p = e >> 8, j = (e >> 6) & 3, l = e & 63;
    const int row = 16 * pair_i(p, NB) + 4 * (l >> 4) + j, col = 16 * pair_j(p, NB) + (l & 15);
    if (row > col) return;                        // a diagonal block's lower half mirrors its upper half
    const float *P = a.part + (int64_t)zh * a.S * NP * 256 + e;
    double sum = 0.0;
    int q = 0;
    for (; q + 8 <= a.S; q += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = P[(int64_t)(q + u) * NP * 256];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += (double)v[u];
    }
    for (; q < a.S; ++q) sum += (double)P[(int64_t)q * NP * 256];
    double *C = a.acc + (int64_t)zh * D * D;
    const double v = a.first ? sum : C[row * D + col] + sum;
    C[row * D + col] = v;
    C[col * D + row] = v;
}

// ------------------------------------------------------------------ bases

constexpr int kBasesThreads = 1024;
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
__device__ void gemm_cq(const double *C, const double *src, double *dst, int k, int ks)
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
                const double qv = src[j * ks + c0 + cc];
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
            if (c0 + cc < k) dst[(lane + kWave * ri) * ks + c0 + cc] = acc[ri][cc];
    __syncthreads();
}

// Q (LDS [D][k]) = k orthonormal columns spanning W's: classical
// Gram-Schmidt twice per column over the columns of [W | I], a column kept
// unless its norm after the two passes is at most 2^-40 of its norm before.
// The projections' sums are split over the workgroup's four quarters
// (partials in sp, [4][max(D, k)]) and added in quarter order.
template <int D>
__device__ void orth(const double *W, double *Q, int k, int ks, double *sv, double *sr, double *sp, double *sred)
{
    constexpr int QT = kBasesThreads / 4;          // threads per quarter
    const int tid = threadIdx.x, qi = tid / QT, qt = tid % QT;
    int kept = 0;
    for (int cand = 0; kept < k && cand < k + D; ++cand) {
        if (tid < D) sv[tid] = cand < k ? W[tid * ks + cand] : (tid == cand - k ? 1.0 : 0.0);
        double mine = tid < D ? sv[tid] : 0.0;
        const double n0 = sqrt(block_sum(mine * mine, sred));
        for (int pass = 0; pass < 2 && kept > 0; ++pass) {
            // r = Q[:, :kept]^T v: quarter qi sums rows [qi D/4, (qi+1) D/4)
            if (qt < kept) {
                double p0 = 0.0, p1 = 0.0;
                const int i0 = qi * (D / 4);
#pragma unroll 4
                for (int i = i0; i < i0 + D / 4; i += 2) {
                    p0 = fma(Q[i * ks + qt], sv[i], p0);
                    p1 = fma(Q[(i + 1) * ks + qt], sv[i + 1], p1);
                }
                sp[qi * kMaxSketch + qt] = p0 + p1;
            }
            __syncthreads();
            if (tid < kept)
                sr[tid] = ((sp[tid] + sp[kMaxSketch + tid]) + sp[2 * kMaxSketch + tid]) + sp[3 * kMaxSketch + tid];
            __syncthreads();
            // v -= Q[:, :kept] r: quarter qi sums columns [c0, c1)
            if (qt < D) {
                const int per = (kept + 3) / 4, c0 = qi * per, c1 = min(kept, c0 + per);
                double p0 = 0.0, p1 = 0.0;
                int cc = c0;
                for (; cc + 1 < c1; cc += 2) {
                    p0 = fma(Q[qt * ks + cc], sr[cc], p0);
                    p1 = fma(Q[qt * ks + cc + 1], sr[cc + 1], p1);
                }
                if (cc < c1) p0 = fma(Q[qt * ks + cc], sr[cc], p0);
                sp[qi * kMaxHeadDim + qt] = p0 + p1;
            }
            __syncthreads();
            if (tid < D)
                sv[tid] -= ((sp[tid] + sp[kMaxHeadDim + tid]) + sp[2 * kMaxHeadDim + tid]) + sp[3 * kMaxHeadDim + tid];
            __syncthreads();
        }
        mine = tid < D ? sv[tid] : 0.0;
        const double n1 = sqrt(block_sum(mine * mine, sred));
        if (n0 != 0.0 && n1 > 0x1p-40 * n0) {
            if (tid < D) Q[tid * ks + kept] = sv[tid] / n1;
            ++kept;
        }
        __syncthreads();
    }
}

// One CholeskyQR pass over the k columns of X (LDS [D][ks], in place):
// G = X^T X (upper triangle, in g [k][k | 1]; a thread per 4x4 tile), G =
// R^T R (right-looking, the trailing update spread over the workgroup),
// X = X R^{-1} (a thread per row, forward substitution).
// Returns false, with X unchanged, when a pivot's remainder falls to 1e-5
// of its column's norm or below (the columns are then too close to
// dependent for this path).  scratch: 2 kMaxSketch doubles.
template <int D>
__device__ __forceinline__ bool cholqr_pass(double *X, double *g, int k, int ks, double *scratch)
{
    const int tid = threadIdx.x, kg = k | 1, nb = (k + 3) / 4;
    double *norm2 = scratch, *rdiag = scratch + kMaxSketch;
    if (tid < nb * (nb + 1) / 2) {
        // tile (A, B), A <= B, in row order
        int A = 0, t = tid;
        while (t >= nb - A) {
            t -= nb - A;
            ++A;
        }
        const int B = A + t;
        double acc[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
        for (int i = 0; i < D; ++i) {
            // (columns past k read other LDS values; their products are dropped)
            double xa[4], xb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                xa[u] = X[i * ks + 4 * A + u];
                xb[u] = X[i * ks + 4 * B + u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] = fma(xa[u], xb[v], acc[u][v]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int a = 4 * A + u, b = 4 * B + v;
                if (a <= b && b < k) g[a * kg + b] = acc[u][v];
            }
    }
    __syncthreads();
    if (tid < k) norm2[tid] = g[tid * kg + tid];
    for (int j = 0; j < k; ++j) {
        __syncthreads();
        // every thread reads the same pivot: the branch is uniform
        const double d = g[j * kg + j];
        if (!(d > 1e-10 * norm2[j])) return false;
        const double r = sqrt(d);
        if (tid == j) rdiag[j] = r;
        if (tid > j && tid < k) g[j * kg + tid] /= r;
        __syncthreads();
        const int w = k - j - 1;
        for (int e = tid; e < w * w; e += kBasesThreads) {
            const int a = j + 1 + e / w, b = j + 1 + e % w;
            if (a <= b) g[a * kg + b] = fma(-g[j * kg + a], g[j * kg + b], g[a * kg + b]);
        }
    }
    __syncthreads();
    if (tid < D) {
        double *x = X + tid * ks;
        for (int b = 0; b < k; ++b) {
            double p0 = x[b], p1 = 0.0;
            int a = 0;
            for (; a + 1 < b; a += 2) {
                p0 = fma(-x[a], g[a * kg + b], p0);
                p1 = fma(-x[a + 1], g[(a + 1) * kg + b], p1);
            }
            if (a < b) p0 = fma(-x[a], g[a * kg + b], p0);
            x[b] = (p0 + p1) / rdiag[b];
        }
    }
    __syncthreads();
    return true;
}

// Q (LDS [D][k]) = k orthonormal columns spanning W's.  Where two CholeskyQR
// passes hold (no column's remainder below 1e-5 of its norm, so that
// Gram-Schmidt over [W | I] would keep exactly W's columns), their result,
// which spans the same space (W is left holding it); else Gram-Schmidt as
// defined above (orth), on W or on the first pass's columns.
template <int D>
__device__ __forceinline__ void orth_fast(double *W, double *Q, int k, int ks, double *sv, double *sr, double *sp, double *sred)
{
    if (cholqr_pass<D>(W, Q, k, ks, sp) && cholqr_pass<D>(W, Q, k, ks, sp)) {
        for (int e = threadIdx.x; e < D * ks; e += kBasesThreads) Q[e] = W[e];
        __syncthreads();
        return;
    }
    orth<D>(W, Q, k, ks, sv, sr, sp, sred);
}

__device__ __forceinline__ int rr_index(int pos, int step, int kp)
{
    return pos == 0 ? 0 : 1 + (pos - 1 + step) % (kp - 1);
}

template <int D>
__global__ __launch_bounds__(kBasesThreads) void bases_kernel(Layout ly, uint8_t *arena, BasesArgs a)
{
    // Q and W rows padded to an odd number of doubles (ks = k | 1), so that
    // lanes walking consecutive rows of one column hit different banks
    __shared__ double sQ[kMaxHeadDim * (kMaxSketch + 1)];
    __shared__ double sW[kMaxHeadDim * (kMaxSketch + 1)];
    __shared__ double sv[kMaxHeadDim];
    __shared__ double sr[kMaxSketch + 1];
    __shared__ double sp[4 * kMaxHeadDim];
    __shared__ double sred[kBasesWaves];
    __shared__ double s_c[kMaxSketch / 2 + 1], s_s[kMaxSketch / 2 + 1];
    __shared__ int s_a[kMaxSketch / 2 + 1], s_b[kMaxSketch / 2 + 1];
    __shared__ int s_perm[kMaxSketch];
    __shared__ double s_sgn[kMaxSketch];

    const int tid = threadIdx.x, k = a.k, ks = k | 1;
    const int zh = blockIdx.x, gi = blockIdx.y;
    const int z = zh / ly.Hkv, h = zh % ly.Hkv;
    const int m = a.group0 + gi;
    const double *C = a.acc + ((int64_t)gi * 2 * ly.Hkv + zh) * D * D;
    const float *om = a.omega + ((int64_t)gi * 2 * ly.Hkv + zh) * D * k;

    // 1. Y = C Omega;  2. Q = orth(Y)
    for (int e = tid; e < D * k; e += kBasesThreads) sQ[(e / k) * ks + e % k] = (double)om[e];
    __syncthreads();
    gemm_cq<D>(C, sQ, sW, k, ks);
    orth_fast<D>(sW, sQ, k, ks, sv, sr, sp, sred);
    // 3. power iterations
    for (int it = 0; it < a.power_iters; ++it) {
        gemm_cq<D>(C, sQ, sW, k, ks);
        orth_fast<D>(sW, sQ, k, ks, sv, sr, sp, sred);
    }
    // 4. T = Q^T C Q, symmetrised, into sW
    gemm_cq<D>(C, sQ, sW, k, ks);
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
                    p0 = fma(sQ[i * ks + ra], sW[i * ks + cb], p0);
                    p1 = fma(sQ[(i + 1) * ks + ra], sW[(i + 1) * ks + cb], p1);
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
                    // the index paired with the absent one (k odd) sits out
                    // this step: a pair of one, never rotated
                    pa = pa < k ? pa : pb;
                    pb = -1;
                }
                s_a[tid] = pa;
                s_b[tid] = pb;
                s_c[tid] = c;
                s_s[tid] = s;
            }
            __syncthreads();
            // T <- J^T T J one 2x2 block (pairs p <= p2) per item, from the
            // block's old values, written with its mirror (T stays exactly
            // symmetric); Q <- Q J one (row, pair) per item
            for (int e = tid; e < P * P; e += kBasesThreads) {
                const int p = e / P, p2 = e - p * P;
                if (p > p2) continue;
                const int a0 = s_a[p], b0 = s_b[p], a1 = s_a[p2], b1 = s_b[p2];
                const double c0 = s_c[p], s0 = s_s[p], c1 = s_c[p2], s1 = s_s[p2];
                if (s0 == 0.0 && s1 == 0.0) continue;
                const bool hb0 = b0 >= 0, hb1 = b1 >= 0;   // false: a pair of one (s = 0)
                const double taa = T[a0 * k + a1], tab = hb1 ? T[a0 * k + b1] : 0.0;
                const double tba = hb0 ? T[b0 * k + a1] : 0.0, tbb = hb0 && hb1 ? T[b0 * k + b1] : 0.0;
                // rows: J_p^T
                const double raa = c0 * taa - s0 * tba, rab = c0 * tab - s0 * tbb;
                const double rba = s0 * taa + c0 * tba, rbb = s0 * tab + c0 * tbb;
                // columns: J_p2
                double naa = c1 * raa - s1 * rab, nab = s1 * raa + c1 * rab;
                double nba = c1 * rba - s1 * rbb, nbb = s1 * rba + c1 * rbb;
                if (p == p2) {                      // the rotated pair's off-diagonal entries
                    nab = 0.0;
                    nba = 0.0;
                }
                T[a0 * k + a1] = naa;
                if (hb1) T[a0 * k + b1] = nab;
                if (hb0) T[b0 * k + a1] = nba;
                if (hb0 && hb1) T[b0 * k + b1] = nbb;
                if (p != p2) {
                    T[a1 * k + a0] = naa;
                    if (hb1) T[b1 * k + a0] = nab;
                    if (hb0) T[a1 * k + b0] = nba;
                    if (hb0 && hb1) T[b1 * k + b0] = nbb;
                }
            }
            for (int e = tid; e < P * D; e += kBasesThreads) {
                const int p = e / D, i = e % D;
                const int a0 = s_a[p], b0 = s_b[p];
                if (s_s[p] == 0.0) continue;
                const double c0 = s_c[p], s0 = s_s[p];
                const double qa = sQ[i * ks + a0], qb = sQ[i * ks + b0];
                sQ[i * ks + a0] = c0 * qa - s0 * qb;
                sQ[i * ks + b0] = s0 * qa + c0 * qb;
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
            const double v = fabs(sQ[i * ks + tid]);
            if (v > bv) {
                bv = v;
                best = i;
            }
        }
        s_sgn[tid] = sQ[best * ks + tid] < 0.0 ? -1.0 : 1.0;
    }
    __syncthreads();
    // 6. the first r_max Ritz vectors as the basis rows, in fp16
    uint16_t *Bz = basis_ptr(ly, arena, m, z, h);
    for (int e = tid; e < ly.R * D; e += kBasesThreads) {
        const int rho = e / D, i = e % D, col = s_perm[rho];
        Bz[e] = d2h_rne(s_sgn[col] * sQ[i * ks + col]);
    }
    if (a.ritz && tid < k) a.ritz[((int64_t)gi * 2 * ly.Hkv + zh) * k + tid] = T[s_perm[tid] * k + s_perm[tid]];
}

// ------------------------------------------------------------------ encode

constexpr int kSlotThreads = 256;

// Tier counts of one chunk (kSlotChunk positions) of one (sequence, KV
// head)'s prefill tokens, and whether any tier is out of range:
// cntc[bh][c][0..T) and cntc[bh][c][kMaxTiers].
__global__ __launch_bounds__(kSlotThreads) void count_kernel(Layout ly, EncodeArgs a)
{
    __shared__ int s_cnt[kMaxTiers + 1];
    const int c = blockIdx.x, bh = blockIdx.y, b = bh / ly.Hkv;
    const int tid = threadIdx.x;
    if (tid <= kMaxTiers) s_cnt[tid] = 0;
    __syncthreads();
    int n = a.n_tokens[b];
    n = (n < 0 || n > a.n_cap) ? 0 : n;
    const uint8_t *tier = a.tier + (int64_t)bh * a.n_cap;
    int loc[kMaxTiers] = {0, 0, 0, 0, 0, 0, 0, 0};
    int bad = 0;
    const int t1 = min(n, (c + 1) * kSlotChunk);
    // the chunk's tiers, every load issued before any is used
    int kt[kSlotChunk / kSlotThreads];
#pragma unroll
    for (int u = 0; u < kSlotChunk / kSlotThreads; ++u) {
        const int t = c * kSlotChunk + u * kSlotThreads + tid;
        kt[u] = t < t1 ? tier[t] : -1;
    }
#pragma unroll
    for (int u = 0; u < kSlotChunk / kSlotThreads; ++u) {
        const int k = kt[u];
        bad |= k >= ly.T;
#pragma unroll
        for (int kk = 0; kk < kMaxTiers; ++kk) loc[kk] += k == kk;
    }
#pragma unroll
    for (int kk = 0; kk < kMaxTiers; ++kk)
        if (loc[kk]) atomicAdd(&s_cnt[kk], loc[kk]);
    if (bad) atomicOr(&s_cnt[kMaxTiers], 1);
    __syncthreads();
    if (tid <= kMaxTiers) a.cntc[((int64_t)bh * a.n_chunks + c) * kChunkStride + tid] = s_cnt[tid];
}

// Places one chunk of one (sequence, KV head)'s prefill tokens: admission
// of the whole call for that (sequence, KV head) from every chunk's counts
// (tiers valid, every tier region and the position map with room), then
// position n0 + t gets (tier << 28 | slot) with slots in position order
// after the tier's counted tokens, and the tokens are listed by tier (in
// position order within a tier) for the encoder: inv[base_k + u] is the
// u-th token of tier k.  status = n0, or -1 when refused (nothing is
// written then).
__global__ __launch_bounds__(kSlotThreads) void place_kernel(Layout ly, uint8_t *arena, EncodeArgs a)
{
    __shared__ int s_tot[kMaxTiers], s_off[kMaxTiers], s_run[kMaxTiers], s_wc[kSlotThreads / kWave][kMaxTiers];
    __shared__ int s_bad;
    const int c = blockIdx.x, bh = blockIdx.y, b = bh / ly.Hkv, h = bh % ly.Hkv;
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int32_t *cnt = counts_ptr(ly, arena, a.layer, b, h);
    if (tid < kMaxTiers) {
        s_tot[tid] = 0;
        s_off[tid] = 0;
        s_run[tid] = 0;
    }
    if (tid == 0) s_bad = 0;
    __syncthreads();
    // every chunk's counts and bad-tier flag, one load per (chunk, field),
    // all in flight at once (integer sums: the order does not matter)
    for (int e = tid; e < a.n_chunks * (kMaxTiers + 1); e += kSlotThreads) {
        const int cc = e / (kMaxTiers + 1), f = e - cc * (kMaxTiers + 1);
        const int v = a.cntc[((int64_t)bh * a.n_chunks + cc) * kChunkStride + f];
        if (v != 0) {
            if (f == kMaxTiers) {
                atomicOr(&s_bad, 1);
            } else {
                atomicAdd(&s_tot[f], v);
                if (cc < c) atomicAdd(&s_off[f], v);
            }
        }
    }
    __syncthreads();
    int n = a.n_tokens[b];
    const bool bad_len = n < 0 || n > a.n_cap;
    if (bad_len) n = 0;
    int n0 = 0;
    for (int kk = 0; kk < ly.T; ++kk) n0 += cnt[kk];
    uint32_t err = bad_len ? DWKV_DEVERR_BAD_LENGTH : 0u;
    if (s_bad) err |= DWKV_DEVERR_BAD_TIER;
    for (int kk = 0; kk < ly.T; ++kk)
        if (cnt[kk] + s_tot[kk] > ly.cap[kk]) err |= DWKV_DEVERR_TIER_FULL;
    if ((int64_t)n0 + n > ly.max_tokens || n > (int64_t)a.n_chunks * kSlotChunk) err |= DWKV_DEVERR_POS_FULL;
    if (err) {
        if (tid == 0 && c == 0) {
            atomicOr(err_ptr(ly, arena), err);
            a.status[bh] = -1;
        }
        return;
    }
    int base[kMaxTiers];
    {
        int acc = 0;
#pragma unroll
        for (int kk = 0; kk < kMaxTiers; ++kk) {
            base[kk] = acc;
            acc += kk < ly.T ? s_tot[kk] : 0;
        }
    }
    const uint8_t *tier = a.tier + (int64_t)bh * a.n_cap;
    int32_t *pm = posmap_ptr(ly, arena, a.layer, b, h) + n0;
    int32_t *inv = a.inv + (int64_t)bh * ly.max_tokens;
    const int t1 = min(n, (c + 1) * kSlotChunk);
    for (int t0 = c * kSlotChunk; t0 < t1; t0 += kSlotThreads) {
        const int t = t0 + tid;
        const int k = t < t1 ? tier[t] : -1;
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
            int off = s_off[k] + s_run[k];
            for (int ww = 0; ww < w; ++ww) off += s_wc[ww][k];
            off += rank;
            pm[t] = (k << 28) | (cnt[k] + off);
            int bk = 0;
#pragma unroll
            for (int kk = 0; kk < kMaxTiers; ++kk) bk = kk == k ? base[kk] : bk;
            inv[bk + off] = t;
        }
        __syncthreads();
        if (tid < ly.T)
            for (int ww = 0; ww < kSlotThreads / kWave; ++ww) s_run[tid] += s_wc[ww][tid];
        __syncthreads();
    }
    if (c == 0) {
        if (tid == 0) a.status[bh] = n0;
        if (tid < kMaxTiers) {
            a.cnt0[bh * kMaxTiers + tid] = tid < ly.T ? cnt[tid] : 0;
            a.tot[bh * kMaxTiers + tid] = tid < ly.T ? s_tot[tid] : 0;
        }
    }
}

// The window's bases for the encoder's scalar loads, fp16 as in the cache,
// in blocks of 8 rows [z][h][i / 8][j][i % 8] (a (z, h) spans d * kMaxRank
// values): the loads of one block sit at fixed offsets from one address and
// fill whole cache lines, and both encoder steps read them.
__global__ void basis_copy_kernel(Layout ly, uint8_t *arena, int m, uint16_t *blocks)
{
    const int64_t n = 2 * ly.basis_elems;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const int z = (int)(e / ly.basis_elems);
        const int64_t rem = e - (int64_t)z * ly.basis_elems;
        const int h = (int)(rem / ((int64_t)ly.R * ly.d));
        const int64_t r2 = rem - (int64_t)h * ly.R * ly.d;
        const int i = (int)(r2 / ly.d), j = (int)(r2 % ly.d);
        blocks[((int64_t)z * ly.Hkv + h) * ly.d * kMaxRank + ((int64_t)(i >> 3) * ly.d + j) * 8 + (i & 7)] =
            basis_ptr(ly, arena, m, z, h)[(int64_t)i * ly.d + j];
    }
}

// An fp32 value kept as such (the later fp16 conversion rounds this fp32
// value, not the exact sum), without the memory side effects of a volatile
// statement, so the basis loads around it stay scalar.
__device__ __forceinline__ float keep_fp32(float v)
{
    asm("" : "+v"(v));
    return v;
}

template <int N>
__device__ __forceinline__ void sload(const uint32_t *__restrict__ p, uint32_t (&v)[N])
{
#pragma unroll
    for (int u = 0; u < N; ++u) v[u] = p[u];
}

// fp16 halves of a 32-bit word, exactly in fp32 (the multiply-adds take them
// as fp16 operands of a mixed-precision FMA)
__device__ __forceinline__ float lo_h(uint32_t w) { return h2f((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi_h(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

// Encodes up to 64 tokens of one tier of one (sequence, KV head) and one Z,
// one token per lane, in exactly the append's order of operations: step 1
// sums sum_j B[i][j] x_j for every coefficient i sequentially in j (eight
// coefficients' sums interleaved), step 2 sums sum_i B[i][j] c_i for every
// channel j sequentially in i, the kept channels are the s largest |e|
// (ties to the lower channel, as in the append), and the scale, codes and
// gate follow as in the append.  The basis values are wave-uniform: they
// come through scalar loads of the window's fp16 block copy, as the fp16
// operand of mixed-precision FMAs (an exact conversion, so each is the
// append's fp32 FMA).
template <int D, int CB>  // CB: bytes per stored coefficient (2: fp16, 1: 8-bit codes)
__global__ __launch_bounds__(kWave) void encode_kernel(Layout ly, uint8_t *__restrict__ arena, EncodeArgs a,
                                                       const uint16_t *__restrict__ bblocks)
{
#pragma clang fp contract(off)
    // [r][64]: this wave's coefficients, lane-minor (fp16 when they are
    // stored as fp16, else fp32 sums and then the values step 2 uses); then
    // the kept channels
    extern __shared__ float s_c[];
    uint16_t *s_h = reinterpret_cast<uint16_t *>(s_c);
    const int zh = blockIdx.y, z = zh / ly.Hkv, h = zh % ly.Hkv, b = blockIdx.z;
    const int bh = b * ly.Hkv + h;
    const int lane = threadIdx.x;
    // the (sequence, KV head)'s status, tier totals and first slots in one
    // round trip (every load issued before any is used)
    const int n0 = a.status[bh];
    int totv[kMaxTiers], c0v[kMaxTiers];
#pragma unroll
    for (int kk = 0; kk < kMaxTiers; ++kk) {
        const int tv = a.tot[bh * kMaxTiers + kk], cv = a.cnt0[bh * kMaxTiers + kk];
        totv[kk] = kk < ly.T ? tv : 0;
        c0v[kk] = cv;
    }
    // the chunk's tier: chunks of 64 list entries, tier by tier from the
    // highest rank (the longest chunks are dispatched first); none for a
    // refused (sequence, KV head)
    const int chunk = n0 < 0 ? 0x7FFFFFFF : (int)blockIdx.x;
    int k = -1, first = 0, c0 = 0;
#pragma unroll
    for (int kk = kMaxTiers - 1; kk >= 0; --kk) {
        const int nc = (totv[kk] + kWave - 1) / kWave;
        if (k < 0 && chunk < c0 + nc) {
            k = kk;
            first = (chunk - c0) * kWave;
        }
        c0 += nc;
    }
    if (k < 0) return;
    int base = 0, tot = 0, cnt0 = 0;
#pragma unroll
    for (int kk = 0; kk < kMaxTiers; ++kk) {
        base += kk < k ? totv[kk] : 0;
        tot = kk == k ? totv[kk] : tot;
        cnt0 = kk == k ? c0v[kk] : cnt0;
    }
    const int u = first + lane;
    const bool live = u < tot;
    const int t = live ? a.inv[(int64_t)bh * ly.max_tokens + base + u] : a.inv[(int64_t)bh * ly.max_tokens + base + first];
    const int slot = cnt0 + (live ? u : first);
    const int r = ly.rank[k], s = ly.resid[k];
    uint8_t *blk = head_block_ptr(ly, arena, a.layer, b, h);
    // fp16 basis words in blocks of 8 rows: [i / 8][j][(i % 8) / 2]
    const uint32_t *__restrict__ Bblk = reinterpret_cast<const uint32_t *>(bblocks + (int64_t)zh * D * kMaxRank);
    const uint16_t *X = (z ? a.v : a.k) + ((int64_t)bh * a.n_cap + t) * D;

    // 1. the coefficient sums, eight at a time (x as fp16 pairs)
    {
        uint32_t xw[D / 2];
#pragma unroll
        for (int q = 0; q < D / 8; ++q) {
            const uint4 v = reinterpret_cast<const uint4 *>(X)[q];
            xw[4 * q] = v.x;
            xw[4 * q + 1] = v.y;
            xw[4 * q + 2] = v.z;
            xw[4 * q + 3] = v.w;
        }
        for (int i0 = 0; i0 < r; i0 += 8) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const uint32_t *__restrict__ bb = Bblk + (int64_t)i0 * D / 2;
            if (i0 + 8 <= r) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    uint32_t bw[4];
                    sload<4>(bb + j * 4, bw);
                    const float xj = (j & 1) ? hi_h(xw[j / 2]) : lo_h(xw[j / 2]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] = __builtin_fmaf(lo_h(bw[q]), xj, acc[2 * q]);
                        acc[2 * q + 1] = __builtin_fmaf(hi_h(bw[q]), xj, acc[2 * q + 1]);
                    }
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (CB == 2)
                        s_h[(i0 + q) * kWave + lane] = f2h(keep_fp32(acc[q]));
                    else
                        s_c[(i0 + q) * kWave + lane] = keep_fp32(acc[q]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    uint32_t bw[2];
                    sload<2>(bb + j * 4, bw);
                    const float xj = (j & 1) ? hi_h(xw[j / 2]) : lo_h(xw[j / 2]);
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        acc[2 * q] = __builtin_fmaf(lo_h(bw[q]), xj, acc[2 * q]);
                        acc[2 * q + 1] = __builtin_fmaf(hi_h(bw[q]), xj, acc[2 * q + 1]);
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (CB == 2)
                        s_h[(i0 + q) * kWave + lane] = f2h(keep_fp32(acc[q]));
                    else
                        s_c[(i0 + q) * kWave + lane] = keep_fp32(acc[q]);
                }
            }
        }
    }
    // the 8-bit form's rounding: codes with a block scale, and s_c then
    // holds code x scale, the values step 2 uses (the fp16 form was rounded
    // as it was written)
    float cs_f = 0.0f;
    uint16_t cs16 = 0;
    if (CB != 2) {
        float amax = 0.0f;
        for (int i = 0; i < r; ++i) amax = fmaxf(amax, fabsf(s_c[i * kWave + lane]));
        cs16 = f2h(__fdiv_rn(amax, 127.0f));
        cs_f = h2f(cs16);
        for (int i = 0; i < r; ++i) {
            const float sum = s_c[i * kWave + lane];
            float qv = 0.0f;
            if (cs_f != 0.0f) {
                qv = rintf(__fdiv_rn(sum, cs_f));
                qv = fminf(fmaxf(qv, -127.0f), 127.0f);
            }
            s_c[i * kWave + lane] = qv * cs_f;
        }
    }

    // 2. the residual sums, sequential in i for every channel
    float e[D];
    if (s > 0) {
#pragma unroll
        for (int j = 0; j < D; ++j) e[j] = 0.0f;
        // eight coefficients at a time from the same basis blocks as step 1
        // (then a last block of four): each channel's chain still runs over
        // i in ascending order
        int i0 = 0;
        for (; i0 + 8 <= r; i0 += 8) {
            const uint32_t *__restrict__ bb = Bblk + (int64_t)i0 * D / 2;
            float c[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) c[q] = CB == 2 ? h2f(s_h[(i0 + q) * kWave + lane]) : s_c[(i0 + q) * kWave + lane];
            // four channels per 64-byte load, their chains interleaved
#pragma unroll
            for (int j0 = 0; j0 < D; j0 += 4) {
                uint32_t bw[16];
                sload<16>(bb + j0 * 4, bw);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t w = bw[4 * u + q / 2];
                        e[j0 + u] = __builtin_fmaf((q & 1) ? hi_h(w) : lo_h(w), c[q], e[j0 + u]);
                    }
                }
            }
        }
        if (i0 < r) {
            const uint32_t *__restrict__ bb = Bblk + (int64_t)i0 * D / 2;
            float c[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) c[q] = CB == 2 ? h2f(s_h[(i0 + q) * kWave + lane]) : s_c[(i0 + q) * kWave + lane];
#pragma unroll
            for (int j = 0; j < D; ++j) {
                uint32_t bw[2];
                sload<2>(bb + j * 4, bw);
                float v = e[j];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    v = __builtin_fmaf(lo_h(bw[q]), c[2 * q], v);
                    v = __builtin_fmaf(hi_h(bw[q]), c[2 * q + 1], v);
                }
                e[j] = v;
            }
        }
#pragma unroll
        for (int q = 0; q < D / 8; ++q) {
            const uint4 v = reinterpret_cast<const uint4 *>(X)[q];
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                e[8 * q + 2 * m] = h2f((uint16_t)(wv[m] & 0xFFFF)) - e[8 * q + 2 * m];
                e[8 * q + 2 * m + 1] = h2f((uint16_t)(wv[m] >> 16)) - e[8 * q + 2 * m + 1];
            }
        }
    }

    // the coefficients into the tier region
    const int64_t coff = z ? ly.f_coefV[k] : ly.f_coefK[k];
    if (live) {
        if (CB == 2) {
            uint16_t *cdst = reinterpret_cast<uint16_t *>(blk + coff);
            for (int i = 0; i < r; ++i)
                cdst[z ? coefV_index(r, slot, i) : (int64_t)slot * r + i] = s_h[i * kWave + lane];
        } else {
            int8_t *cdst = reinterpret_cast<int8_t *>(blk + coff);
            for (int i = 0; i < r; ++i) {
                const float c = s_c[i * kWave + lane];
                cdst[z ? coefV_index(r, slot, i) : (int64_t)slot * r + i] =
                    static_cast<int8_t>(cs_f != 0.0f ? (int)__fdiv_rn(c, cs_f) : 0);
            }
            reinterpret_cast<uint16_t *>(blk + (z ? ly.f_cscV[k] : ly.f_cscK[k]))[slot] = cs16;
        }
    }
    if (s == 0) return;

    // 3. the s kept channels: the s largest |e| with ties to the lower
    //    channel.  First the largest kMaxResid + 1 |e|, in decreasing order,
    //    by an insertion in which entry q becomes the median of its old
    //    value, the old entry q - 1 and the new value (thr: the s-th of
    //    them); then, in ascending channel order, every channel above thr
    //    and the first (s - #above) channels at thr go to the next of this
    //    lane's s LDS slots (the others to a spare slot), value and channel
    //    together.  Where the (s + 1)-th largest is below thr in every lane
    //    (no tie at the threshold to break), the kept channels are those at
    //    or above thr.
    constexpr int kTop = kMaxResid + 1;
    float top[kTop];
#pragma unroll
    for (int q = 0; q < kTop; ++q) top[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const float v = fabsf(e[j]);
#pragma unroll
        for (int q = kTop - 1; q > 0; --q) top[q] = __builtin_amdgcn_fmed3f(top[q - 1], top[q], v);
        top[0] = fmaxf(top[0], v);
    }
    float thr = top[0], nxt = top[1];
    int above = 0;
#pragma unroll
    for (int q = 0; q < kMaxResid; ++q) {
        thr = q == s - 1 ? top[q] : thr;
        nxt = q == s - 1 ? top[q + 1] : nxt;
    }
#pragma unroll
    for (int q = 0; q < kMaxResid; ++q) above += (q < s && top[q] > thr) ? 1 : 0;
    const int need = s - above;
    float *s_ev = s_c;                                                     // [kMaxResid + 1][64]
    int *s_ej = reinterpret_cast<int *>(s_c) + (kMaxResid + 1) * kWave;    // the same, channels
    int cnt = 0;
    if (__all(nxt < thr)) {
        float *const spare = s_ev + kMaxResid * kWave + lane;
        float *next = s_ev + lane;
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const bool keep = fabsf(e[j]) >= thr;
            float *const p = keep ? next : spare;
            p[0] = e[j];
            reinterpret_cast<int *>(p)[(kMaxResid + 1) * kWave] = j;
            next += keep ? kWave : 0;
        }
    } else {
        int ties = 0;
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const float v = fabsf(e[j]);
            const int at = (v == thr) & (ties < need);
            const int keep = (v > thr) | at;
            ties += at;
            const int slot = (keep ? cnt : kMaxResid) * kWave + lane;
            s_ev[slot] = e[j];
            s_ej[slot] = j;
            cnt += keep;
        }
    }
    // 4. the scale from the largest kept |e|
    const float amax = top[0];
    const uint16_t s16 = f2h(__fdiv_rn(amax, (float)ly.qmax));
    const float sf = h2f(s16);
    // 5. codes and channel bytes, in ascending channel order (slot u is the
    //    u-th kept channel)
    uint64_t valw = 0, idxw = 0;
#pragma unroll
    for (int u = 0; u < kMaxResid; ++u) {
        if (u >= s) break;
        const float ev = s_ev[u * kWave + lane];
        float v = 0.0f;
        if (sf != 0.0f) {
            v = rintf(__fdiv_rn(ev, sf));
            v = fminf(fmaxf(v, -(float)ly.qmax), (float)ly.qmax);
        }
        const int code = (int)v;
        idxw |= (uint64_t)(uint32_t)s_ej[u * kWave + lane] << (8 * u);
        valw |= ly.bits == 8 ? (uint64_t)(code & 0xFF) << (8 * u) : (uint64_t)(code & 0xF) << (4 * u);
    }
    if (!live) return;
    uint32_t *idst = reinterpret_cast<uint32_t *>(blk + (z ? ly.f_idxV[k] : ly.f_idxK[k]) + (int64_t)slot * ly.istride[k]);
    uint32_t *vdst = reinterpret_cast<uint32_t *>(blk + (z ? ly.f_valV[k] : ly.f_valK[k]) + (int64_t)slot * ly.vstride[k]);
    idst[0] = (uint32_t)idxw;
    if (ly.istride[k] > 4) idst[1] = (uint32_t)(idxw >> 32);
    vdst[0] = (uint32_t)valw;
    if (ly.vstride[k] > 4) vdst[1] = (uint32_t)(valw >> 32);
    // 6. the gate folds into the stored scale
    const uint16_t *G = z ? a.gateV : a.gateK;
    const uint16_t g = G ? G[(int64_t)bh * a.n_cap + t] : uint16_t(0x3C00);
    reinterpret_cast<uint16_t *>(blk + (z ? ly.f_scaleV[k] : ly.f_scaleK[k]))[slot] =
        (g == 0x3C00) ? s16 : f2h(h2f(g) * sf);
}

// Publishes the encoded tokens: the tier counts of every admitted
// (sequence, KV head).
__global__ void publish_kernel(Layout ly, uint8_t *arena, EncodeArgs a, int n_bh)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n_bh * ly.T) return;
    const int bh = e / ly.T, k = e % ly.T;
    if (a.status[bh] < 0) return;
    counts_ptr(ly, arena, a.layer, bh / ly.Hkv, bh % ly.Hkv)[k] =
        a.cnt0[bh * kMaxTiers + k] + a.tot[bh * kMaxTiers + k];
}

}  // namespace

hipError_t launch_gram(const Layout &ly, uint8_t *arena, const GramArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    const auto kern = ly.d == 64 ? gram_kernel<64> : gram_kernel<128>;
    hipLaunchKernelGGL(kern, dim3(a.S, 2 * a.Hkv), dim3(kGramThreads), 0, stream, ly, arena, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const auto red = ly.d == 64 ? gram_reduce_kernel<64> : gram_reduce_kernel<128>;
    hipLaunchKernelGGL(red, dim3(gram_pairs(ly.d), 2 * a.Hkv), dim3(256), 0, stream, a);
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
    hipError_t e = hipSuccess;
    if (a.copy_basis) {
        const int64_t be = 2 * ly.basis_elems;
        hipLaunchKernelGGL(basis_copy_kernel, dim3((unsigned)((be + 255) / 256 < 1024 ? (be + 255) / 256 : 1024)),
                           dim3(256), 0, stream, ly, arena, a.layer / ly.G, a.basis_blocks);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(count_kernel, dim3(a.n_chunks, batch * ly.Hkv), dim3(kSlotThreads), 0, stream, ly, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(place_kernel, dim3(a.n_chunks, batch * ly.Hkv), dim3(kSlotThreads), 0, stream, ly, arena, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const auto kern = ly.cb == 2 ? (ly.d == 64 ? encode_kernel<64, 2> : encode_kernel<128, 2>)
                                 : (ly.d == 64 ? encode_kernel<64, 1> : encode_kernel<128, 1>);
    const unsigned chunks = (unsigned)((a.n_cap + kWave - 1) / kWave + ly.T);
    const size_t coef_lds = (size_t)ly.R * kWave * (ly.cb == 2 ? 2 : 4);
    const size_t sel_lds = (size_t)2 * (kMaxResid + 1) * kWave * 4;
    const size_t lds = coef_lds > sel_lds ? coef_lds : sel_lds;
    hipLaunchKernelGGL(kern, dim3(chunks, 2 * ly.Hkv, batch), dim3(kWave), lds, stream, ly, arena, a, a.basis_blocks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n = batch * ly.Hkv * ly.T;
    hipLaunchKernelGGL(publish_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, ly, arena, a, batch * ly.Hkv);
    return hipGetLastError();
}

}  // namespace dwkv
