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
// Work split (split-K "flash decode"): grid = (splits, KV heads, sequences),
// one 8-wave workgroup per compute unit.  A workgroup takes a byte-balanced
// run of 16-token blocks of the tier regions of its (sequence, KV head) and
// cuts it into tiles of about 2 KiB of coefficients per K and V (64 tokens
// at rank <= 16, 32 at rank 32, 16 at rank 64 or more); wave w takes tiles
// w, w + 8, ...  Each wave keeps its own online softmax (base-2 logits) and
// runs a two-deep software pipeline: the loads of its next tile are in
// flight while the current one is computed.  Per tile:
//   * scores of 16 tokens x 16 columns on the matrix cores (16x16x16 fp16):
//     K coefficient rows times q', which enters as two fp16 columns per query
//     head (q'_hi = fp16(q'), q'_lo = fp16(q' - q'_hi)) so the products keep
//     fp32-level accuracy;
//   * the sparse K residual adds scale * sum_u q[idx] code per token (one
//     token per lane, q gathered from LDS);
//   * probabilities (fp16) times V coefficient columns accumulate the
//     basis-space value sum on the matrix cores -- the score accumulator's
//     register layout is exactly the probability operand's;
//   * the V residual of each 16-token block is written densely (code x
//     scale) into an LDS tile [channel][token] and multiplied by the same
//     probabilities on the matrix cores; the written cells are then cleared.
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
constexpr int kTile = 64;                 // most tokens in a tile
constexpr int kSlots = 4;                 // 16x16 operand blocks per tile and Z (rank <= 64)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxLag = 8.0f;           // log2 units the running max may trail

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

// 2^x on the transcendental unit (no denormal fix-up: results below 2^-126
// are irrelevant next to the >= 1 weight of the running max).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wave_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

__device__ __forceinline__ uint32_t ld32(const uint8_t *p)
{
    return *reinterpret_cast<const uint32_t *>(p);
}

// Index byte u (0..7) and code u of a token's residual record.
__device__ __forceinline__ int idx_at(uint32_t i0, uint32_t i1, int u)
{
    return ((u < 4 ? i0 : i1) >> (8 * (u & 3))) & 0xFF;
}

template <int BITS>
__device__ __forceinline__ float code_at(uint32_t c0, uint32_t c1, int u)
{
    if (BITS == 8) return (float)(int)(int8_t)((u < 4 ? c0 : c1) >> (8 * (u & 3)));
    return (float)(((int)(c0 << (28 - 4 * u))) >> 28);
}

// Rotates a token's s <= 8 entries by `rot` positions.  Entries are stored
// in ascending channel order; rotating by the lane number keeps the lanes of
// a wave from visiting the same narrow band of channels at the same step.
template <int BITS>
__device__ __forceinline__ void rotate_entries(uint32_t &i0, uint32_t &i1, uint32_t &c0, uint32_t &c1,
                                               int s, int rot)
{
    if (rot == 0) return;
    const uint32_t iw = 8u * s, cw = (uint32_t)BITS * s;
    const uint64_t imask = iw == 64 ? ~0ull : ((1ull << iw) - 1);
    const uint64_t cmask = cw == 64 ? ~0ull : ((1ull << cw) - 1);
    const uint64_t i64 = (((uint64_t)i1 << 32) | i0) & imask;
    const uint64_t c64 = (((uint64_t)c1 << 32) | c0) & cmask;
    const uint32_t ri = 8u * rot, rc = (uint32_t)BITS * rot;
    const uint64_t ni = ((i64 >> ri) | (i64 << (iw - ri))) & imask;
    const uint64_t nc = ((c64 >> rc) | (c64 << (cw - rc))) & cmask;
    i0 = (uint32_t)ni;
    i1 = (uint32_t)(ni >> 32);
    c0 = (uint32_t)nc;
    c1 = (uint32_t)(nc >> 32);
}

// Copies n fp16 values (n a multiple of 8, source 16-byte aligned) into LDS.
__device__ __forceinline__ void stage_basis(uint16_t *dst, const uint16_t *src, int n, int tid)
{
    const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
    uint4 *d4 = reinterpret_cast<uint4 *>(dst);
    for (int i = tid; i < n / 8; i += kBlock) d4[i] = s4[i];
}

// ceil(x / w) for 0 <= x < 2^53, w > 0 (exact: the quotient's distance to an
// integer is a multiple of 1/w, far above double rounding)
__device__ __forceinline__ int64_t ceil_div(int64_t x, int64_t w)
{
    return x <= 0 ? 0 : (int64_t)ceil((double)x / (double)w);
}

// Where a tile lies, uniform over the wave.
struct Tile {
    int valid;        // 0 once the wave has no more tiles
    int k;            // tier
    int r, s;         // rank and residual channels of the tier
    int kbr;          // 16-channel blocks of the rank (1, 2, 4, 8)
    int nv;           // valid tokens (<= 16 * slots / kbr)
    int64_t blk0;     // first 16-token block
};

// Loads of one tile in flight: coefficient operand slots (slot i is m-block
// i / kbr, channel block i % kbr) and token `lane`'s residual records.
template <int NS>
struct TileData {
    half4_t ka[NS], va[NS];
    uint32_t ki0, ki1, kc0, kc1, vi0, vi1, vc0, vc1;
    uint16_t ksc, vsc;
};

// Per-tier block ranges of this workgroup (uniform values).
struct Ranges {
    int T;
    int64_t b0[kMaxTiers], b1[kMaxTiers];
    int cnt[kMaxTiers], nt[kMaxTiers], kbr[kMaxTiers];
};

template <int NS>
__device__ __forceinline__ Tile locate(const Ranges &rg, const Layout &ly, int it)
{
    Tile t;
    t.valid = 0;
    t.k = 0;
    t.r = t.s = t.nv = 0;
    t.kbr = 1;
    t.blk0 = 0;
    int rem = it;
#pragma unroll
    for (int kk = 0; kk < kMaxTiers; ++kk) {
        if (kk < rg.T && !t.valid) {
            if (rem < rg.nt[kk]) {
                const int kbr = rg.kbr[kk], mbs = NS / kbr;
                t.valid = 1;
                t.k = kk;
                t.r = ly.rank[kk];
                t.s = ly.resid[kk];
                t.kbr = kbr;
                t.blk0 = rg.b0[kk] + (int64_t)rem * mbs;
                int nv = (int)(rg.b1[kk] - t.blk0) * 16;
                if (nv > 16 * mbs) nv = 16 * mbs;
                const int left = (int)(rg.cnt[kk] - t.blk0 * 16);
                t.nv = nv < left ? nv : left;
            } else {
                rem -= rg.nt[kk];
            }
        }
    }
    return t;
}

// Issues every load of a tile: always the same number of load instructions
// (slots the tile does not use read a harmless in-block address), so the
// compiler's wait counts stay exact and the next tile's loads are never
// waited for while the current tile is computed.
template <int NS>
__device__ __forceinline__ void issue_tile(const Tile &t, TileData<NS> &D, const uint8_t *blk,
                                           const Layout &ly, int lane)
{
    const int c16 = lane & 15, grp = lane >> 4;
    const int k = t.k, r = t.r, kbr = t.kbr;
    const uint16_t *cK = reinterpret_cast<const uint16_t *>(blk + ly.f_coefK[k]);
    const uint16_t *cV = reinterpret_cast<const uint16_t *>(blk + ly.f_coefV[k]);
    const int64_t tok0 = t.blk0 * 16;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int mb = i / kbr, kb = i - mb * kbr;
        const bool use = t.valid && 16 * mb < t.nv;
        const int tr = 16 * mb + c16;
        const int64_t ko = use && tr < t.nv && 16 * kb + 4 * grp < r
                               ? (tok0 + tr) * r + 16 * kb + 4 * grp : 0;
        const int64_t vo = use && 16 * kb + c16 < r
                               ? ((t.blk0 + mb) * r + 16 * kb + c16) * 16 + 4 * grp : 0;
        D.ka[i] = *reinterpret_cast<const half4_t *>(cK + ko);
        D.va[i] = *reinterpret_cast<const half4_t *>(cV + vo);
    }
    const bool tv = t.valid && t.s > 0 && lane < t.nv;
    const int64_t tt = tv ? tok0 + lane : 0;
    const uint8_t *iK = blk + ly.f_idxK[k] + tt * ly.istride[k];
    const uint8_t *vK = blk + ly.f_valK[k] + tt * ly.vstride[k];
    const uint8_t *iV = blk + ly.f_idxV[k] + tt * ly.istride[k];
    const uint8_t *vV = blk + ly.f_valV[k] + tt * ly.vstride[k];
    D.ki0 = ld32(iK);
    D.ki1 = ld32(iK + 4);
    D.kc0 = ld32(vK);
    D.kc1 = ld32(vK + 4);
    D.ksc = reinterpret_cast<const uint16_t *>(blk + ly.f_scaleK[k])[tt];
    D.vi0 = ld32(iV);
    D.vi1 = ld32(iV + 4);
    D.vc0 = ld32(vV);
    D.vc1 = ld32(vV + 4);
    D.vsc = reinterpret_cast<const uint16_t *>(blk + ly.f_scaleV[k])[tt];
}

// Per-wave state of the online softmax and the value sums.
template <int KB>
struct WaveAcc {
    float4_t O[KB];                      // basis-space value sums [head row][channel]
    float4_t Ores[kMaxHeadDim / 16];     // residual value mass [head row][channel]
    float m_run;                         // running max of head (lane % 16) % 8
    float l_part;                        // this lane's share of that head's normaliser
};

template <int GQ, int BITS, int KB, int KBR>
__device__ __forceinline__ void process_tile(const Tile &t, const TileData<kSlots * (KB / 4)> &D,
                                             const half4_t (&qb)[KB], WaveAcc<KB> &A,
                                             const float (*s_qt)[GQ < 4 ? 4 : GQ], float *sR,
                                             _Float16 *ev, uint32_t *srec, int d, int lane)
{
    constexpr int NS = kSlots * (KB / 4);
    constexpr int MBS = NS / KBR;                   // 16-token blocks in the tile
    constexpr int GP = GQ < 4 ? 4 : GQ;
    constexpr int ND = kMaxHeadDim / 16;
    const int c16 = lane & 15, grp = lane >> 4;
    const int r = t.r, s = t.s, nv = t.nv;

    // ---- scores: K coefficient rows x (q'_hi, q'_lo)
    float4_t Sc[MBS];
#pragma unroll
    for (int mb = 0; mb < MBS; ++mb) {
        Sc[mb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (16 * mb < nv) {
            const bool tv = 16 * mb + c16 < nv;
#pragma unroll
            for (int kb = 0; kb < KBR; ++kb) {
                half4_t a = D.ka[mb * KBR + kb];
                if (!(tv && 16 * kb + 4 * grp < r)) a = half4_t{0, 0, 0, 0};
                Sc[mb] = mma16(a, qb[kb], Sc[mb]);
            }
        }
    }

    // ---- K residual: one token per lane, q gathered from LDS
    if (s > 0) {
        uint32_t i0 = D.ki0, i1 = D.ki1, c0 = D.kc0, c1 = D.kc1;
        rotate_entries<BITS>(i0, i1, c0, c1, s, lane % s);
        float rk[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) rk[g] = 0.0f;
#pragma unroll
        for (int u = 0; u < kMaxResid; ++u) {
            if (u < s) {
                const int j = idx_at(i0, i1, u);
                const float cv = code_at<BITS>(c0, c1, u);
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
        const float sc = lane < nv ? h2f(D.ksc) : 0.0f;
#pragma unroll
        for (int g = 0; g < GQ; ++g) sR[g * kTile + lane] = rk[g] * sc;
        wave_fence();
    }

    // ---- logits, tile max, lazy rescale, probabilities
    float z[MBS][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < MBS; ++mb) {
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
    const bool need = tmax > A.m_run + kMaxLag;
    if (__any(need)) {
        const float new_m = need ? tmax : A.m_run;
        const float f = fast_exp2(A.m_run - new_m);
        A.l_part *= f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float fh = __shfl(f, 4 * grp + j, kWave);
#pragma unroll
            for (int nb = 0; nb < KB; ++nb) A.O[nb][j] *= fh;
#pragma unroll
            for (int nb = 0; nb < ND; ++nb) A.Ores[nb][j] *= fh;
        }
        A.m_run = new_m;
    }
    half4_t P[MBS];
#pragma unroll
    for (int mb = 0; mb < MBS; ++mb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const _Float16 ph = (_Float16)fast_exp2(z[mb][j] - A.m_run);
            P[mb][j] = ph;
            A.l_part += (float)ph;
        }
    }

    // ---- values: probabilities x V coefficient columns (16-token blocks)
#pragma unroll
    for (int mb = 0; mb < MBS; ++mb) {
        if (16 * mb < nv) {
            const bool partial = 16 * mb + 16 > nv;
#pragma unroll
            for (int nb = 0; nb < KBR; ++nb) {
                half4_t bv = D.va[mb * KBR + nb];
                if (16 * nb + c16 >= r) bv = half4_t{0, 0, 0, 0};
                if (partial) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (16 * mb + 4 * grp + j >= nv) bv[j] = 0;
                }
                A.O[nb] = mma16(P[mb], bv, A.O[nb]);
            }
        }
    }

    // ---- V residual mass: per 16-token block, a dense LDS tile of
    //      code x scale [channel][token] times the probabilities; four lanes
    //      per token (records handed over through LDS), lane taking entries
    //      rot and rot + 4 of its token; the written cells are cleared after.
    if (s > 0) {
        uint32_t *rec = srec + lane * 5;
        rec[0] = D.vi0;
        rec[1] = D.vi1;
        rec[2] = D.vc0;
        rec[3] = D.vc1;
        rec[4] = lane < nv ? D.vsc : 0u;
        wave_fence();
        const int rot = lane & 3, tcol = lane >> 2;
#pragma unroll
        for (int mb = 0; mb < MBS; ++mb) {
            if (16 * mb < nv) {
                const uint32_t *rr = srec + (16 * mb + tcol) * 5;
                const uint32_t i0 = rr[0], i1 = rr[1], c0 = rr[2], c1 = rr[3];
                const float sc = h2f((uint16_t)rr[4]);
                const bool tv = 16 * mb + tcol < nv;
                // entry rot lands in the low byte (nibble) of the first word,
                // entry rot + 4 in that of the second
                const uint32_t i0s = __builtin_amdgcn_alignbit(i1, i0, 8u * rot);
                const uint32_t i1s = rot ? (i1 >> (8u * rot)) : i1;
                uint32_t c0s, c1s;
                if (BITS == 8) {
                    c0s = __builtin_amdgcn_alignbit(c1, c0, 8u * rot);
                    c1s = rot ? (c1 >> (8u * rot)) : c1;
                } else {
                    c0s = c0 >> (4u * rot);
                    c1s = c0s >> 16;
                }
                int js[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    js[e] = -1;
                    if (tv && 4 * e + rot < s) {
                        const uint32_t iw = e == 0 ? i0s : i1s;
                        const uint32_t cw = e == 0 ? c0s : c1s;
                        js[e] = (int)(iw & 0xFF);
                        const float code = BITS == 8 ? (float)(int)(int8_t)(cw & 0xFF)
                                                     : (float)(((int)(cw << 28)) >> 28);
                        ev[js[e] * 16 + tcol] = (_Float16)(code * sc);
                    }
                }
                wave_fence();
#pragma unroll
                for (int nb = 0; nb < ND; ++nb) {
                    if (16 * nb < d) {
                        const half4_t bv = *reinterpret_cast<const half4_t *>(&ev[(16 * nb + c16) * 16 + 4 * grp]);
                        A.Ores[nb] = mma16(P[mb], bv, A.Ores[nb]);
                    }
                }
                wave_fence();
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    if (js[e] >= 0) ev[js[e] * 16 + tcol] = (_Float16)0.0f;
                wave_fence();
            }
        }
    }
}

template <int GQ, int BITS, int KB>
__device__ __forceinline__ void process_any(const Tile &t, const TileData<kSlots * (KB / 4)> &D,
                                            const half4_t (&qb)[KB], WaveAcc<KB> &A,
                                            const float (*s_qt)[GQ < 4 ? 4 : GQ], float *sR,
                                            _Float16 *ev, uint32_t *srec, int d, int lane)
{
    switch (t.kbr) {
    case 1: process_tile<GQ, BITS, KB, 1>(t, D, qb, A, s_qt, sR, ev, srec, d, lane); break;
    case 2: process_tile<GQ, BITS, KB, 2>(t, D, qb, A, s_qt, sR, ev, srec, d, lane); break;
    case 4: process_tile<GQ, BITS, KB, 4>(t, D, qb, A, s_qt, sR, ev, srec, d, lane); break;
    default:
        if constexpr (KB == 8) process_tile<GQ, BITS, KB, 8>(t, D, qb, A, s_qt, sR, ev, srec, d, lane);
        break;
    }
}

template <int GQ, int BITS, int KB>
__global__ __launch_bounds__(kBlock, 1) void decode_kernel(Layout ly, uint8_t *arena, int layer,
                                                           const uint16_t *q, float *out,
                                                           DecodeWorkspace ws, int S, float qscale)
{
    constexpr int GP = GQ < 4 ? 4 : GQ;           // query heads padded for 16-byte gathers
    constexpr int NS = kSlots * (KB / 4);          // operand slots per tile and Z
    constexpr int ND = kMaxHeadDim / 16;           // channel blocks of the residual mass
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int c16 = lane & 15, grp = lane >> 4;
    const int d = ly.d, R = ly.R;
    const int g0 = h * GQ;

    __shared__ __attribute__((aligned(16))) float s_qt[kMaxHeadDim][GP];        // q, base-2 units
    __shared__ float s_qp[GQ][kMaxRank];                                        // merged basis sums
    __shared__ float s_res[GQ][kMaxHeadDim];                                    // merged residual mass
    __shared__ __attribute__((aligned(16))) float s_rk[kWaves][8][kTile];       // K-residual logits
    __shared__ __attribute__((aligned(16))) _Float16 s_ev[kWaves][kMaxHeadDim][16];   // V residual block
    __shared__ uint32_t s_rec[kWaves][kTile * 5];                               // V residual records
    __shared__ float s_m[kWaves][GQ], s_l[kWaves][GQ], s_f[kWaves][GQ];
    __shared__ float s_M[GQ], s_L[GQ];
    __shared__ __attribute__((aligned(16))) uint16_t s_bas[kMaxRank * kMaxHeadDim];   // B_V
    __shared__ int s_last;

    // ---- this workgroup's byte-balanced run of 16-token blocks, per tier
    //      (computed by every wave from scalar loads: no barrier needed)
    const uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);
    Ranges rg;
    {
        const int32_t *cnt = counts_ptr(ly, arena, layer, b, h);
        rg.T = ly.T;
        int64_t W = 0;
#pragma unroll
        for (int k = 0; k < kMaxTiers; ++k) {
            rg.cnt[k] = k < ly.T ? uni(cnt[k]) : 0;
            W += (int64_t)((rg.cnt[k] + 15) >> 4) * 16 * (k < ly.T ? ly.weight[k] : 0);
        }
        const int64_t lo = (int64_t)floor((double)W * split / S);
        const int64_t hi = (int64_t)floor((double)W * (split + 1) / S);
        int64_t wk = 0;
#pragma unroll
        for (int k = 0; k < kMaxTiers; ++k) {
            rg.b0[k] = rg.b1[k] = 0;
            rg.nt[k] = 0;
            rg.kbr[k] = 1;
            if (k < ly.T) {
                const int64_t nb = (rg.cnt[k] + 15) >> 4, wb = 16 * (int64_t)ly.weight[k];
                int64_t b0 = ceil_div(lo - wk, wb), b1 = ceil_div(hi - wk, wb);
                b0 = b0 < nb ? b0 : nb;
                b1 = b1 < nb ? b1 : nb;
                wk += nb * wb;
                const int r = ly.rank[k];
                const int kbr = r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8;
                const int mbs = NS / kbr;
                rg.b0[k] = b0;
                rg.b1[k] = b1;
                rg.kbr[k] = kbr;
                rg.nt[k] = (int)((b1 - b0 + mbs - 1) / mbs);
            }
        }
    }

    // ---- first tile's loads go out before anything else
    TileData<NS> DA, DB;
    int it = wave;
    Tile ta = locate<NS>(rg, ly, it);
    issue_tile<NS>(ta, DA, blk, ly, lane);

    // ---- query in base-2 logit units (LDS, for residual gathers), B_V staged
    for (int i = tid; i < kMaxHeadDim * GP; i += kBlock) {
        const int j = i / GP, g = i % GP;
        s_qt[j][g] = (g < GQ && j < d) ? qscale * h2f(q[((int64_t)b * ly.Hq + g0 + g) * d + j]) : 0.0f;
    }
    for (int i = tid; i < kWaves * 8 * kTile; i += kBlock) (&s_rk[0][0][0])[i] = 0.0f;
    for (int i = tid; i < kWaves * kMaxHeadDim * 16; i += kBlock) (&s_ev[0][0][0])[i] = (_Float16)0.0f;
    stage_basis(s_bas, basis_ptr(ly, arena, layer / ly.G, 1, h), R * d, tid);

    // ---- score operand qb: q' = B_K q on the matrix cores, straight into
    //      operand layout.  Column c16 carries query head c16 % 8 -- as
    //      fp16(q') for c16 < 8 and as the remainder fp16(q' - fp16(q'))
    //      above -- so that the fp16 products reproduce q' to ~2^-22.
    //      Products of fp16 inputs are exact and sums fp32: q' is fp32-accurate.
    half4_t qb[KB];
    {
        const uint16_t *BK = basis_ptr(ly, arena, layer / ly.G, 0, h);
        const int gq = c16 & 7;
        const uint16_t *qrow = q + ((int64_t)b * ly.Hq + g0 + (gq < GQ ? gq : 0)) * d;
        half4_t bq[kMaxHeadDim / 16];
#pragma unroll
        for (int kb = 0; kb < kMaxHeadDim / 16; ++kb)
            bq[kb] = (gq < GQ && 16 * kb < d) ? *reinterpret_cast<const half4_t *>(qrow + 16 * kb + 4 * grp)
                                              : half4_t{0, 0, 0, 0};
#pragma unroll
        for (int mb = 0; mb < KB; ++mb) {
            float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (16 * mb < R) {
                const uint16_t *brow = BK + (int64_t)(16 * mb + c16 < R ? 16 * mb + c16 : 0) * d;
                half4_t a[kMaxHeadDim / 16];
#pragma unroll
                for (int kb = 0; kb < kMaxHeadDim / 16; ++kb)
                    a[kb] = 16 * kb < d ? *reinterpret_cast<const half4_t *>(brow + 16 * kb + 4 * grp)
                                        : half4_t{0, 0, 0, 0};
#pragma unroll
                for (int kb = 0; kb < kMaxHeadDim / 16; ++kb) {
                    half4_t aa = a[kb];
                    if (16 * mb + c16 >= R) aa = half4_t{0, 0, 0, 0};
                    acc = mma16(aa, bq[kb], acc);
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
    __syncthreads();

    // ---- main loop: two-deep pipeline over this wave's tiles
    WaveAcc<KB> A;
#pragma unroll
    for (int nb = 0; nb < KB; ++nb) A.O[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) A.Ores[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    A.m_run = -INFINITY;
    A.l_part = 0.0f;
    float *sR = &s_rk[wave][0][0];
    _Float16 *ev = &s_ev[wave][0][0];
    uint32_t *srec = &s_rec[wave][0];
    while (ta.valid) {
        it += kWaves;
        Tile tb = locate<NS>(rg, ly, it);
        issue_tile<NS>(tb, DB, blk, ly, lane);
        process_any<GQ, BITS, KB>(ta, DA, qb, A, s_qt, sR, ev, srec, d, lane);
        if (!tb.valid) break;
        it += kWaves;
        ta = locate<NS>(rg, ly, it);
        issue_tile<NS>(ta, DA, blk, ly, lane);
        process_any<GQ, BITS, KB>(tb, DB, qb, A, s_qt, sR, ev, srec, d, lane);
    }

    // ---- merge the waves of this workgroup
    float l_part = A.l_part;
    l_part += __shfl_xor(l_part, 16, kWave);
    l_part += __shfl_xor(l_part, 32, kWave);
    if (lane < GQ) {
        s_m[wave][lane] = A.m_run;
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
                        if (16 * nb < R) s_qp[row][16 * nb + c16] += f * A.O[nb][j];
#pragma unroll
                    for (int nb = 0; nb < ND; ++nb)
                        if (16 * nb < d) s_res[row][16 * nb + c16] += f * A.Ores[nb][j];
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
    // of the splits, many independent loads in flight
    const int quads = GQ * d / 4;
    const int parts = kBlock / quads;
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
