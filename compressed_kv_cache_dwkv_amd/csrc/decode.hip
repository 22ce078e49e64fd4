// Decode attention over the compressed cache (DepthWeave-KV paper, arXiv
// 2607.06523, §3 Method, Eq. (1) and the decoding data path described in the
// paragraph before Fig. 2): basis lookup, residual dequantisation,
// coefficient multiply and attention in one pass, with no reconstructed K or
// V ever written to memory.
//
// Algebra used (exact rewrites of Eq. (1)):
//   q . K^_t = (B_K q)[0:r_t] . c^K_t + scale^K_t * sum_u q[idx^K_{t,u}] code^K_{t,u}
//   sum_t p_t V^_t = B_V^T (sum_t p_t c^V_t) + sum_t p_t scale^V_t sum_u code^V_{t,u} e_{idx^V_{t,u}}
// A query is projected once into basis coordinates (q' = B_K q); values are
// accumulated in basis coordinates plus a dense residual-mass vector, and
// B_V is applied once per workgroup at the end.
//
// Work split (split-K "flash decode"): grid = (splits, KV heads, sequences).
// A workgroup takes a byte-balanced run of 16-token blocks of the tier
// regions of its (sequence, KV head); its four waves take 64-token tiles in
// turn and each keeps its own online softmax (base-2 logits).  Per tile:
//   * scores of 16 tokens x 16 columns come from 16x16x16 fp16 matrix-core
//     products of the K coefficient rows with q' -- q' enters as two fp16
//     columns per query head (q'_hi = fp16(q'), q'_lo = fp16(q' - q'_hi)) so
//     the products keep fp32-level accuracy;
//   * the sparse K residual adds scale * sum_u q[idx] code per token (one
//     token per lane, q gathered from LDS);
//   * probabilities (fp16) times the V coefficient columns accumulate the
//     basis-space value sum, again on the matrix cores; the score
//     accumulator's register layout is exactly the probability operand's;
//   * the sparse V residual is added into an LDS residual-mass vector with
//     LDS float atomics (one token per lane).
// The running max may trail the true max by up to 8 (a factor 256) before
// the accumulators are rescaled, so rescaling is rare.  The last workgroup
// of a (sequence, KV head) to finish merges all partials.
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

constexpr int kBlock = 512;               // 8 waves: one workgroup fills a compute unit
constexpr int kWaves = kBlock / kWave;
constexpr int kTile = 64;                  // tokens per wave iteration (4 blocks of 16)
constexpr int kMaxKBlocks = kMaxRank / 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxLag = 8.0f;            // log2 units the running max may trail

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4_t mma16(half4_t a, half4_t b, float4_t c)
{
    // D[m][n] += sum_k A[m][k] B[k][n]; lane l supplies A[l%16][4(l/16)+j],
    // B[4(l/16)+j][l%16] and holds D[4(l/16)+j][l%16], j = 0..3.
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Value from the lane 8 positions away inside each row of 16 lanes.
__device__ __forceinline__ float row_swap8(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

// Marks a value the whole wave holds as wave-uniform (scalar register), so
// that branches and addresses derived from it stay scalar.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// 2^x on the transcendental unit (no denormal fix-up: results below 2^-126
// are irrelevant next to the >= 1 weight of the running max).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wave_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// n (<= 16) bytes of one token, read with the widest aligned loads the
// per-token stride allows, packed little-endian into w[0..3].
__device__ __forceinline__ void load_token_bytes(const uint8_t *p, int n, uint32_t w[4])
{
    w[0] = w[1] = w[2] = w[3] = 0u;
    if ((n & 3) == 0) {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < (n >> 2)) w[i] = q[i];
    } else if ((n & 1) == 0) {
        const uint16_t *q = reinterpret_cast<const uint16_t *>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < (n >> 1)) w[i >> 1] |= uint32_t(q[i]) << (16 * (i & 1));
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i < n) w[i >> 2] |= uint32_t(p[i]) << (8 * (i & 3));
    }
}

// Rotates a token's s <= 8 residual entries by `rot` positions (indices in
// wi, codes of `bits` bits in wc).  The entries of a token are stored in
// ascending channel order, so without rotation the lanes of a wave would all
// visit the u-th smallest channel of their tokens at the same step -- a
// narrow band of channels, i.e. LDS bank and same-address collisions.
template <int BITS>
__device__ __forceinline__ void rotate_entries(uint32_t wi[4], uint32_t wc[4], int s, int rot)
{
    if (s > 8 || rot == 0) return;
    const uint64_t iw = 8u * s, cw = (uint64_t)BITS * s;
    const uint64_t imask = iw == 64 ? ~0ull : ((1ull << iw) - 1);
    const uint64_t cmask = cw == 64 ? ~0ull : ((1ull << cw) - 1);
    const uint64_t i64 = ((uint64_t)wi[1] << 32) | wi[0];
    const uint64_t c64 = ((uint64_t)wc[1] << 32) | wc[0];
    const uint32_t ri = 8u * rot, rc = (uint32_t)BITS * rot;
    const uint64_t ni = ((i64 >> ri) | (i64 << (iw - ri))) & imask;
    const uint64_t nc = ((c64 >> rc) | (c64 << (cw - rc))) & cmask;
    wi[0] = (uint32_t)ni;
    wi[1] = (uint32_t)(ni >> 32);
    wc[0] = (uint32_t)nc;
    wc[1] = (uint32_t)(nc >> 32);
}

__device__ __forceinline__ int byte_at(const uint32_t w[4], int u)
{
    return (w[u >> 2] >> (8 * (u & 3))) & 0xFF;
}

template <int BITS>
__device__ __forceinline__ float code_at(const uint32_t w[4], int u)
{
    if (BITS == 8) return (float)(int)(int8_t)(w[u >> 2] >> (8 * (u & 3)));
    return (float)(((int)(w[u >> 3] << (28 - 4 * (u & 7)))) >> 28);
}

// Copies n fp16 values (n a multiple of 8, source 16-byte aligned) into LDS.
__device__ __forceinline__ void stage_basis(uint16_t *dst, const uint16_t *src, int n, int tid)
{
    const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
    uint4 *d4 = reinterpret_cast<uint4 *>(dst);
    for (int i = tid; i < n / 8; i += kBlock) d4[i] = s4[i];
}

__device__ __forceinline__ int64_t first_at(int64_t x, int64_t w)
{
    return x <= 0 ? 0 : (x + w - 1) / w;
}

// Shifts a token's packed residual entries so that entry (u + rot) lands at
// position u (rot < 4), for the lanes that each take every fourth entry.
template <int BITS>
__device__ __forceinline__ void shift_entries(uint32_t wi[4], uint32_t wc[4], int rot)
{
    const uint32_t si = 8u * rot, sc = (uint32_t)BITS * rot;
    wi[0] = __builtin_amdgcn_alignbit(wi[1], wi[0], si);
    wi[1] = __builtin_amdgcn_alignbit(wi[2], wi[1], si);
    wi[2] = __builtin_amdgcn_alignbit(wi[3], wi[2], si);
    wi[3] = si ? (wi[3] >> si) : wi[3];
    wc[0] = __builtin_amdgcn_alignbit(wc[1], wc[0], sc);
    wc[1] = __builtin_amdgcn_alignbit(wc[2], wc[1], sc);
    wc[2] = __builtin_amdgcn_alignbit(wc[3], wc[2], sc);
    wc[3] = sc ? (wc[3] >> sc) : wc[3];
}

template <int GQ, int BITS, int KB>
__global__ __launch_bounds__(kBlock, 1) void decode_kernel(Layout ly, uint8_t *arena, int layer,
                                                           const uint16_t *q, float *out,
                                                           DecodeWorkspace ws, int S, float qscale)
{
    constexpr int GP = GQ < 4 ? 4 : GQ;          // query heads padded for 16-byte gathers
    constexpr int ND = kMaxHeadDim / 16;          // channel blocks of the residual mass
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int c16 = lane & 15, grp = lane >> 4;
    const int d = ly.d, R = ly.R;
    const int g0 = h * GQ;

    __shared__ __attribute__((aligned(16))) float s_qt[kMaxHeadDim][GP];        // q, base-2 units
    __shared__ float s_qp[GQ][kMaxRank];                                        // q' = B_K q, then sums
    __shared__ float s_res[GQ][kMaxHeadDim];                                    // merged residual mass
    __shared__ __attribute__((aligned(16))) float s_rk[kWaves][8][kTile];       // K-residual logits
    __shared__ __attribute__((aligned(16))) _Float16 s_ev[kWaves][kMaxHeadDim][16];   // V residual block
    __shared__ float s_m[kWaves][GQ], s_l[kWaves][GQ], s_f[kWaves][GQ];
    __shared__ float s_M[GQ], s_L[GQ];
    __shared__ __attribute__((aligned(16))) uint16_t s_bas[kMaxRank * kMaxHeadDim];   // B_K, then B_V
    __shared__ int64_t s_b0[kMaxTiers], s_b1[kMaxTiers];
    __shared__ int s_nt[kMaxTiers], s_cnt[kMaxTiers];
    __shared__ int s_last;

    // ---- a1: the query in base-2 logit units, and q' = B_K q
    for (int i = tid; i < kMaxHeadDim * GP; i += kBlock) {
        const int j = i / GP, g = i % GP;
        s_qt[j][g] = (g < GQ && j < d) ? qscale * h2f(q[((int64_t)b * ly.Hq + g0 + g) * d + j]) : 0.0f;
    }
    for (int i = tid; i < kWaves * 8 * kTile; i += kBlock) (&s_rk[0][0][0])[i] = 0.0f;
    for (int i = tid; i < kWaves * kMaxHeadDim * 16; i += kBlock) (&s_ev[0][0][0])[i] = (_Float16)0.0f;
    if (tid == 0) {
        // this split's byte-balanced run of 16-token blocks, per tier
        const int32_t *cnt = counts_ptr(ly, arena, layer, b, h);
        int64_t W = 0;
        for (int k = 0; k < ly.T; ++k) {
            s_cnt[k] = cnt[k];
            W += (int64_t)((cnt[k] + 15) >> 4) * 16 * ly.weight[k];
        }
        const int64_t lo = W * split / S, hi = W * (split + 1) / S;
        int64_t wk = 0;
        for (int k = 0; k < ly.T; ++k) {
            const int64_t nb = (s_cnt[k] + 15) >> 4, wb = 16 * (int64_t)ly.weight[k];
            int64_t b0 = first_at(lo - wk, wb), b1 = first_at(hi - wk, wb);
            b0 = b0 < nb ? b0 : nb;
            b1 = b1 < nb ? b1 : nb;
            wk += nb * wb;
            s_b0[k] = b0;
            s_b1[k] = b1;
            s_nt[k] = (int)((b1 - b0 + 3) >> 2);
        }
    }
    __syncthreads();

    // score operand qb: q' = B_K q on the matrix cores, straight into operand
    // layout.  Column c16 carries query head c16 % 8 -- as fp16(q') for
    // c16 < 8 and as the remainder fp16(q' - fp16(q')) above -- so that the
    // fp16 products reproduce q' to ~2^-22.  Products of fp16 inputs are
    // exact and sums are fp32, so q' itself is fp32-accurate.
    half4_t qb[KB];
    {
        const uint16_t *BK = basis_ptr(ly, arena, layer / ly.G, 0, h);
        const int gq = c16 & 7;
        const uint16_t *qrow = q + ((int64_t)b * ly.Hq + g0 + (gq < GQ ? gq : 0)) * d;
#pragma unroll
        for (int mb = 0; mb < KB; ++mb) {
            float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (16 * mb < R) {
                const uint16_t *brow = BK + (int64_t)(16 * mb + c16) * d;
                for (int kb = 0; kb < d / 16; ++kb) {
                    half4_t a = half4_t{0, 0, 0, 0}, bq = half4_t{0, 0, 0, 0};
                    if (16 * mb + c16 < R) a = *reinterpret_cast<const half4_t *>(brow + 16 * kb + 4 * grp);
                    if (gq < GQ) bq = *reinterpret_cast<const half4_t *>(qrow + 16 * kb + 4 * grp);
                    acc = mma16(a, bq, acc);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = qscale * acc[j];
                const _Float16 hi = (_Float16)v;
                const _Float16 lo = (_Float16)(v - (float)hi);
                qb[mb][j] = (c16 < 8) ? hi : lo;
            }
        }
    }

    int ntiles = 0;
    for (int k = 0; k < ly.T; ++k) ntiles += s_nt[k];

    // value sums, rows = query heads (4 grp + j), cols = channel (16 nb + c16):
    // in basis coordinates (O) and as residual mass in head channels (Ores)
    float4_t O[KB], Ores[ND];
#pragma unroll
    for (int nb = 0; nb < KB; ++nb) O[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) Ores[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY;   // running max of query head c16 % 8
    float l_part = 0.0f;       // this lane's share of that head's normaliser
    float *sR = &s_rk[wave][0][0];
    _Float16 *ev = &s_ev[wave][0][0];
    const uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);

    for (int it = wave; it < ntiles; it += kWaves) {
        int k = 0, ti = it;
        while (ti >= s_nt[k]) {
            ti -= s_nt[k];
            ++k;
        }
        k = uni(k);
        ti = uni(ti);
        const int r = ly.rank[k], s = ly.resid[k], vb = ly.vbytes[k];
        const int64_t blk0 = uni64(s_b0[k] + 4 * (int64_t)ti);
        const int64_t tok0 = blk0 * 16;
        int nv = (int)(uni64(s_b1[k]) - blk0) * 16;
        if (nv > kTile) nv = kTile;
        const int left = (int)(uni(s_cnt[k]) - tok0);
        if (nv > left) nv = left;

        // ---- scores: K coefficient rows x (q'_hi, q'_lo)
        const uint16_t *cK = reinterpret_cast<const uint16_t *>(blk + ly.f_coefK[k]);
        float4_t Sc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            Sc[mb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (16 * mb < nv) {
                const int tr = 16 * mb + c16;
                const bool tv = tr < nv;
                const uint16_t *row = cK + (tok0 + tr) * r;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    if (16 * kb < r) {
                        const int ch = 16 * kb + 4 * grp;
                        half4_t a = half4_t{0, 0, 0, 0};
                        if (tv && ch < r) a = *reinterpret_cast<const half4_t *>(row + ch);
                        Sc[mb] = mma16(a, qb[kb], Sc[mb]);
                    }
                }
            }
        }

        // ---- K residual: one token per lane
        if (s > 0) {
            const int64_t t = tok0 + lane;
            uint32_t wi[4], wc[4];
            float sc = 0.0f;
            if (lane < nv) {
                load_token_bytes(blk + ly.f_idxK[k] + t * s, s, wi);
                load_token_bytes(blk + ly.f_valK[k] + t * vb, vb, wc);
                rotate_entries<BITS>(wi, wc, s, lane % s);
                sc = h2f(reinterpret_cast<const uint16_t *>(blk + ly.f_scaleK[k])[t]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) wi[i] = wc[i] = 0u;
            }
            float rk[GP];
#pragma unroll
            for (int g = 0; g < GP; ++g) rk[g] = 0.0f;
#pragma unroll
            for (int u = 0; u < kMaxResid; ++u) {
                if (u < s) {
                    const int j = byte_at(wi, u);
                    const float cv = code_at<BITS>(wc, u);
                    const float4_t q0 = *reinterpret_cast<const float4_t *>(&s_qt[j][0]);
#pragma unroll
                    for (int g = 0; g < 4; ++g) rk[g] += cv * q0[g];
                    if constexpr (GP == 8) {
                        const float4_t q1 = *reinterpret_cast<const float4_t *>(&s_qt[j][4]);
#pragma unroll
                        for (int g = 0; g < 4; ++g) rk[4 + g] += cv * q1[g];
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < GQ; ++g) sR[g * kTile + lane] = rk[g] * sc;
            wave_fence();
        }

        // ---- logits, tile max, lazy rescale, probabilities
        float z[4][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            float4_t rr = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (s > 0) rr = *reinterpret_cast<const float4_t *>(&sR[(c16 & 7) * kTile + 16 * mb + 4 * grp]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float zz = Sc[mb][j] + row_swap8(Sc[mb][j]) + rr[j];
                z[mb][j] = (16 * mb + 4 * grp + j < nv) ? zz : -INFINITY;
                tmax = fmaxf(tmax, z[mb][j]);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        const bool need = tmax > m_run + kMaxLag;
        if (__any(need)) {
            const float new_m = need ? tmax : m_run;
            const float f = fast_exp2(m_run - new_m);
            l_part *= f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fh = __shfl(f, 4 * grp + j, kWave);
#pragma unroll
                for (int nb = 0; nb < KB; ++nb) O[nb][j] *= fh;
#pragma unroll
                for (int nb = 0; nb < ND; ++nb) Ores[nb][j] *= fh;
            }
            m_run = new_m;
        }
        half4_t P[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const _Float16 ph = (_Float16)fast_exp2(z[mb][j] - m_run);
                P[mb][j] = ph;
                l_part += (float)ph;
            }
        }

        // ---- values: probabilities x V coefficient columns (16-token blocks)
        const uint16_t *cV = reinterpret_cast<const uint16_t *>(blk + ly.f_coefV[k]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if (16 * mb < nv) {
                const uint16_t *vblk = cV + (blk0 + mb) * (int64_t)r * 16;
                const bool partial = 16 * mb + 16 > nv;
#pragma unroll
                for (int nb = 0; nb < KB; ++nb) {
                    if (16 * nb < r) {
                        const int ch = 16 * nb + c16;
                        half4_t bv = half4_t{0, 0, 0, 0};
                        if (ch < r) bv = *reinterpret_cast<const half4_t *>(vblk + ch * 16 + 4 * grp);
                        if (partial) {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                if (16 * mb + 4 * grp + j >= nv) bv[j] = 0;
                        }
                        O[nb] = mma16(P[mb], bv, O[nb]);
                    }
                }
            }
        }

        // ---- V residual mass: each 16-token block's residuals written densely
        //      (code x scale, fp16) into an LDS tile [channel][token], then
        //      probabilities x tile on the matrix cores; written cells are
        //      cleared again afterwards.  Four lanes per token, each taking
        //      every fourth of its entries.
        if (s > 0) {
            const uint8_t *iV = blk + ly.f_idxV[k];
            const uint8_t *vV = blk + ly.f_valV[k];
            const uint16_t *sV = reinterpret_cast<const uint16_t *>(blk + ly.f_scaleV[k]);
            const int rot = lane & 3, tcol = lane >> 2;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (16 * mb < nv) {
                    const bool tv = 16 * mb + tcol < nv;
                    const int64_t t = tok0 + 16 * mb + tcol;
                    uint32_t wi[4] = {0u, 0u, 0u, 0u}, wc[4] = {0u, 0u, 0u, 0u};
                    float sc = 0.0f;
                    if (tv) {
                        load_token_bytes(iV + t * s, s, wi);
                        load_token_bytes(vV + t * vb, vb, wc);
                        sc = h2f(sV[t]);
                    }
                    shift_entries<BITS>(wi, wc, rot);
                    int js[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        js[e] = -1;
                        if (tv && 4 * e + rot < s) {
                            js[e] = byte_at(wi, 4 * e);
                            ev[js[e] * 16 + tcol] = (_Float16)(code_at<BITS>(wc, 4 * e) * sc);
                        }
                    }
                    wave_fence();
#pragma unroll
                    for (int nb = 0; nb < ND; ++nb) {
                        if (16 * nb < d) {
                            const half4_t bv = *reinterpret_cast<const half4_t *>(&ev[(16 * nb + c16) * 16 + 4 * grp]);
                            Ores[nb] = mma16(P[mb], bv, Ores[nb]);
                        }
                    }
                    wave_fence();
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (js[e] >= 0) ev[js[e] * 16 + tcol] = (_Float16)0.0f;
                    wave_fence();
                }
            }
        }
    }

    // ---- merge the waves of this workgroup
    l_part += __shfl_xor(l_part, 16, kWave);
    l_part += __shfl_xor(l_part, 32, kWave);
    if (lane < GQ) {
        s_m[wave][lane] = m_run;
        s_l[wave][lane] = l_part;
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
    for (int i = tid; i < GQ * kMaxRank; i += kBlock) (&s_qp[0][0])[i] = 0.0f;
    for (int i = tid; i < GQ * kMaxHeadDim; i += kBlock) (&s_res[0][0])[i] = 0.0f;
    stage_basis(s_bas, basis_ptr(ly, arena, layer / ly.G, 1, h), R * d, tid);
    __syncthreads();
    // waves add their rescaled sums in a fixed order (bitwise reproducible)
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 4 * grp + j;
                if (row < GQ) {
                    const float f = s_f[wave][row];
#pragma unroll
                    for (int nb = 0; nb < KB; ++nb)
                        if (16 * nb < R) s_qp[row][16 * nb + c16] += f * O[nb][j];
#pragma unroll
                    for (int nb = 0; nb < ND; ++nb)
                        if (16 * nb < d) s_res[row][16 * nb + c16] += f * Ores[nb][j];
                }
            }
        }
        __syncthreads();
    }
    // one back-projection through B_V plus the residual mass, on the matrix
    // cores in fp32: wave w forms output channels 16w..16w+15 as
    // out^T[j][g] = res[g][j] + sum_i B_V[i][j] a[g][i]
    if (16 * wave < d) {
        float4_t acc;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = c16 < GQ ? s_res[c16][16 * wave + 4 * grp + j] : 0.0f;
        for (int kb = 0; kb < R / 4; ++kb) {
            const int i = 4 * kb + grp;
            const float a = h2f(s_bas[i * d + 16 * wave + c16]);
            const float bb = c16 < GQ ? s_qp[c16][i] : 0.0f;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc, 0, 0, 0);
        }
        if (c16 < GQ) {
            float *po = ws.po + (((int64_t)b * ly.Hq + g0 + c16) * S + split) * d + 16 * wave + 4 * grp;
#pragma unroll
            for (int j = 0; j < 4; ++j) __hip_atomic_store(po + j, acc[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (tid < GQ) {
        __hip_atomic_store(ws.pm + ((int64_t)b * ly.Hq + g0 + tid) * S + split, s_M[tid], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ws.pl + ((int64_t)b * ly.Hq + g0 + tid) * S + split, s_L[tid], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- a3: the last workgroup of this (sequence, KV head) merges the splits.
    // Partials travel as agent-scope (cross-XCD coherent) relaxed stores and
    // loads; every store has completed (vmcnt 0) before the workgroup's
    // arrival is counted, so no cache-wide write-back or invalidate is needed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&ws.arrive[b * ly.Hkv + h], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    // weights 2^(m_s - M) of every split, through LDS (reusing the basis
    // buffer: [GQ][S] weights, [GQ][S] normalisers, then the reduction area)
    static_assert(kMaxSplits * 2 * 8 * 4 + kBlock * 16 <= kMaxRank * kMaxHeadDim * 2, "merge scratch");
    float *s_w = reinterpret_cast<float *>(s_bas);
    float *s_pl = s_w + GQ * S;
    for (int i = tid; i < GQ * S; i += kBlock) {
        const int g = i / S, sp = i % S;
        s_w[i] = __hip_atomic_load(ws.pm + ((int64_t)b * ly.Hq + g0 + g) * S + sp, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        s_pl[i] = __hip_atomic_load(ws.pl + ((int64_t)b * ly.Hq + g0 + g) * S + sp, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (tid < GQ) {
        float M = -INFINITY;
        for (int i = 0; i < S; ++i) M = fmaxf(M, s_w[tid * S + i]);
        s_M[tid] = M;
    }
    __syncthreads();
    for (int i = tid; i < GQ * S; i += kBlock) {
        const float M = s_M[i / S];
        s_w[i] = M == -INFINITY ? 0.0f : exp2f(s_w[i] - M);
    }
    __syncthreads();
    if (tid < GQ) {
        float L = 0.0f;
        for (int i = 0; i < S; ++i) L += s_w[tid * S + i] * s_pl[tid * S + i];
        s_L[tid] = L;
    }
    // each thread: 4 adjacent outputs of one head over an interleaved subset
    // of the splits, many independent 16-byte loads in flight
    const int quads = GQ * d / 4;
    const int parts = kBlock / quads;                        // 2 or 4 for d = 128
    float4_t accm = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int qd = tid % quads, part = tid / quads;
    const int gq = (4 * qd) / d, j4 = (4 * qd) % d;
    if (part < parts) {
        const float *po = ws.po + ((int64_t)b * ly.Hq + g0 + gq) * S * d + j4;
#pragma unroll 8
        for (int sp = part; sp < S; sp += parts) {
            float4_t v;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = __hip_atomic_load(po + (int64_t)sp * d + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            accm += s_w[gq * S + sp] * v;
        }
    }
    __syncthreads();
    float4_t *s_red = reinterpret_cast<float4_t *>(s_bas) + kMaxSplits * 2 * 8 / 4;   // [parts][quads]
    if (part < parts) s_red[part * quads + qd] = accm;
    __syncthreads();
    if (tid < quads) {
        float4_t o = s_red[tid];
        for (int p2 = 1; p2 < parts; ++p2) o += s_red[p2 * quads + tid];
        const float L = s_L[gq];
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        *reinterpret_cast<float4_t *>(out + ((int64_t)b * ly.Hq + g0 + gq) * d + j4) = o * inv;
    }
    if (tid == 0) __hip_atomic_store(&ws.arrive[b * ly.Hkv + h], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int GQ>
hipError_t launch_gq(const Layout &ly, uint8_t *arena, int layer, const uint16_t *q, int batch,
                     float qs, float *out, const DecodeWorkspace &ws, int splits, hipStream_t stream)
{
    const dim3 grid(splits, ly.Hkv, batch);
#define DWKV_LAUNCH(BITS, KB)                                                                      \
    hipLaunchKernelGGL((decode_kernel<GQ, BITS, KB>), grid, dim3(kBlock), 0, stream, ly, arena,   \
                       layer, q, out, ws, splits, qs)
    if (ly.R <= 64) {
        if (ly.bits == 4) DWKV_LAUNCH(4, 4); else DWKV_LAUNCH(8, 4);
    } else {
        if (ly.bits == 4) DWKV_LAUNCH(4, 8); else DWKV_LAUNCH(8, 8);
    }
#undef DWKV_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Layout &ly, uint8_t *arena, int layer, const void *q, int batch,
                         float softmax_scale, float *out, const DecodeWorkspace &ws, int splits,
                         hipStream_t stream)
{
    const float qs = softmax_scale * kLog2e;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    switch (ly.gq) {
    case 1: return launch_gq<1>(ly, arena, layer, qq, batch, qs, out, ws, splits, stream);
    case 2: return launch_gq<2>(ly, arena, layer, qq, batch, qs, out, ws, splits, stream);
    case 4: return launch_gq<4>(ly, arena, layer, qq, batch, qs, out, ws, splits, stream);
    case 8: return launch_gq<8>(ly, arena, layer, qq, batch, qs, out, ws, splits, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dwkv
