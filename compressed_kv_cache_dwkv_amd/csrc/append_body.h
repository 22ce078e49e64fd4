// The append of one (sequence, KV head): encodes the new token's K and V
// into the compressed form and stores it in its tier (DepthWeave-KV paper,
// arXiv 2607.06523, §3 Method, second paragraph: coefficients by projection
// onto the current basis, residual kept on the router-chosen number of
// channels with low-bit group quantisation).  Two waves do the work, wave z
// encoding Z = K (z = 0) or V (z = 1); the standalone append kernel and the
// fused decode step both run it.
//
// The encoder makes integer decisions (kept channels, codes) from floating
// point values, so it follows one fixed IEEE fp32 operation order --
// sequential fused multiply-adds in ascending index order, correctly rounded
// division, round-to-nearest-even conversions -- with contraction of any
// other multiply-add switched off in its body.
#pragma once

#include <hip/hip_runtime.h>

#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

constexpr int kAppendBStride = kMaxHeadDim + 2;   // fp16 per basis row in LDS: an odd
                                                  // number of dwords, so lanes reading
                                                  // one column hit distinct banks

// LDS the two waves use (each wave touches only its own half).
struct AppendLds {
    uint16_t *B;     // [2][kMaxRank * kAppendBStride]
    float *x;        // [2][kMaxHeadDim]
    float *c;        // [2][kMaxRank]
    int8_t *code;    // [2][kMaxResid]
    uint8_t *idx;    // [2][kMaxResid]
};
constexpr size_t kAppendLdsBytes =
    2 * (kMaxRank * kAppendBStride * 2 + kMaxHeadDim * 4 + kMaxRank * 4 + 2 * kMaxResid);

__device__ __forceinline__ AppendLds carve_append_lds(void *base)
{
    uint8_t *p = static_cast<uint8_t *>(base);
    AppendLds s;
    s.x = reinterpret_cast<float *>(p);
    p += 2 * kMaxHeadDim * 4;
    s.c = reinterpret_cast<float *>(p);
    p += 2 * kMaxRank * 4;
    s.B = reinterpret_cast<uint16_t *>(p);
    p += 2 * kMaxRank * kAppendBStride * 2;
    s.code = reinterpret_cast<int8_t *>(p);
    p += 2 * kMaxResid;
    s.idx = p;
    return s;
}

// What one wave loads before encoding: the tier, the token counts (lane k
// holding tier k's), its vector (lane j holding channels j, j + 64) and
// basis rows lane and lane + 64 in registers.
template <int D>
struct AppendRegs {
    int k;
    int cnt_l;
    float xv[D / kWave];
    uint4 brow[2][D / 8];
};

// Channel j of a basis row held as 16-byte pieces.
template <int D>
__device__ __forceinline__ float half_at(const uint4 (&row)[D / 8], int j)
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

// Requests every input of wave z's encoding at once, so it waits for
// memory once.
template <int D>
__device__ __forceinline__ void append_fetch(AppendRegs<D> &st, const Layout &ly, uint8_t *arena,
                                             int layer, int b, int h, int z, int lane,
                                             const AppendArgs &ap)
{
    constexpr int NJ = D / kWave;
    const int bh = b * ly.Hkv + h;
    const int32_t *cnt = counts_ptr(ly, arena, layer, b, h);
    st.k = __builtin_amdgcn_readfirstlane(ap.tier[bh]);
    st.cnt_l = lane < ly.T ? cnt[lane] : 0;
    const uint16_t *x = (z ? ap.v : ap.k) + (int64_t)bh * D;
#pragma unroll
    for (int q = 0; q < NJ; ++q) st.xv[q] = h2f(x[lane + q * kWave]);
    const uint16_t *Bg = basis_ptr(ly, arena, layer / ly.G, z, h);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int row = lane + rr * kWave < ly.R ? lane + rr * kWave : 0;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) st.brow[rr][c] = reinterpret_cast<const uint4 *>(Bg + (int64_t)row * D)[c];
    }
}

// Admission of the new token from its tier k and the token counts (lane kk
// holding tier kk's): the tier must exist and its region and the position
// map must have room.  Sets the token's tier slot and position; returns
// the device error bits that refuse it (0: admitted).  Wave-uniform.
__device__ __forceinline__ uint32_t append_admit(const Layout &ly, int k, int cnt_l, int &slot, int &n)
{
    n = 0;
#pragma unroll
    for (int kk = 0; kk < kMaxTiers; ++kk) n += kk < ly.T ? __builtin_amdgcn_readlane(cnt_l, kk) : 0;
    slot = 0;
    if (k >= ly.T) return DWKV_DEVERR_BAD_TIER;
    slot = __builtin_amdgcn_readlane(cnt_l, k);
    uint32_t err = 0;
    if (slot >= ly.cap[k]) err |= DWKV_DEVERR_TIER_FULL;
    if (n >= ly.max_tokens) err |= DWKV_DEVERR_POS_FULL;
    return err;
}

// Copies wave z's basis rows (held in registers by append_fetch or its
// bulk counterpart) into the LDS rows sB, for the column reads of step 2.
template <int D>
__device__ __forceinline__ void encode_stage_basis(const uint4 (&brow)[2][D / 8], uint16_t *sB, int R, int lane)
{
    constexpr int RW = D / 8;                 // 16-byte pieces of a basis row
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        if (lane + rr * kWave < R) {
            uint32_t *dst = reinterpret_cast<uint32_t *>(sB + (lane + rr * kWave) * kAppendBStride);
#pragma unroll
            for (int c = 0; c < RW; ++c) {
                dst[4 * c + 0] = brow[rr][c].x;
                dst[4 * c + 1] = brow[rr][c].y;
                dst[4 * c + 2] = brow[rr][c].z;
                dst[4 * c + 3] = brow[rr][c].w;
            }
        }
    }
}

// Encodes one vector (lane j holding channels j, j + 64 in xv) at tier k and
// stores its coefficients, residual record and scale at `slot` of the tier
// region in blk (the (layer, sequence, KV head) block).  brow: basis rows
// lane and lane + 64; sB: the same rows in LDS; sx, sc, scode, sidx: this
// wave's LDS scratch.  gate16: the fp16 gate (0x3C00 for a gate of 1).
// Every append and every bulk prefill encoding runs this one body, so both
// give the same bits for the same vector.
template <int D>
__device__ __forceinline__ void encode_store(const uint4 (&brow)[2][D / 8], const float (&xv)[D / kWave],
                                             const uint16_t *sB, float *sx, float *sc, int8_t *scode,
                                             uint8_t *sidx, const Layout &ly, uint8_t *blk, int k, int slot,
                                             int z, int lane, uint16_t gate16)
{
#pragma clang fp contract(off)
    constexpr int NJ = D / kWave;             // channels per lane
    const int r = ly.rank[k], s = ly.resid[k];

    wave_fence();                             // the previous vector's reads of sx, sc are issued
#pragma unroll
    for (int q = 0; q < NJ; ++q) sx[lane + q * kWave] = xv[q];
    wave_fence();

    // 1. coefficient sums sum_j B[i][j] x_j, sequential in j (x read from
    //    LDS, the same address in every lane), then stored as fp16, or in the
    //    8-bit blockwise form: block scale fp16(max |sum| / 127), codes
    //    rint(sum / scale) in [-127, 127] (0 for a zero scale); step 2 then
    //    uses the stored values (code * scale is exact in fp32)
    float acc1[2] = {0.0f, 0.0f};
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        if (rr * kWave < r) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < D; ++j) acc = __builtin_fmaf(half_at<D>(brow[rr], j), sx[j], acc);
            acc1[rr] = as_fp32(acc);
        }
    }
    const int64_t coff = z ? ly.f_coefV[k] : ly.f_coefK[k];
    if (ly.cb == 2) {
        uint16_t *cdst = reinterpret_cast<uint16_t *>(blk + coff);
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int i = lane + rr * kWave;
            if (i < r) {
                const uint16_t c16 = f2h(acc1[rr]);
                cdst[z ? coefV_index(r, slot, i) : (int64_t)slot * r + i] = c16;
                sc[i] = h2f(c16);
            }
        }
    } else {
        int8_t *cdst = reinterpret_cast<int8_t *>(blk + coff);
        float a = 0.0f;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
            if (lane + rr * kWave < r) a = fmaxf(a, fabsf(acc1[rr]));
        a = wave_max(a);
        const uint16_t cs16 = f2h(__fdiv_rn(a, 127.0f));
        const float sf = h2f(cs16);
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int i = lane + rr * kWave;
            if (i < r) {
                float qv = 0.0f;
                if (sf != 0.0f) {
                    qv = rintf(__fdiv_rn(acc1[rr], sf));
                    qv = fminf(fmaxf(qv, -127.0f), 127.0f);
                }
                cdst[z ? coefV_index(r, slot, i) : (int64_t)slot * r + i] = static_cast<int8_t>(qv);
                sc[i] = qv * sf;
            }
        }
        if (lane == 0) reinterpret_cast<uint16_t *>(blk + (z ? ly.f_cscV[k] : ly.f_cscK[k]))[slot] = cs16;
    }
    wave_fence();

    // 2. residual against the rounded coefficients, sequential in i
    float e[NJ];
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
        const int j = lane + q * kWave;
        float acc = 0.0f;
#pragma unroll 8
        for (int i = 0; i < r; ++i) acc = __builtin_fmaf(h2f(sB[i * kAppendBStride + j]), sc[i], acc);
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
            scode[pos] = static_cast<int8_t>(v);
            sidx[pos] = static_cast<uint8_t>(j);
        }
        wave_fence();
        const int vb = ly.vbytes[k];
        uint8_t *idst = blk + (z ? ly.f_idxV[k] : ly.f_idxK[k]) + (int64_t)slot * ly.istride[k];
        uint8_t *vdst = blk + (z ? ly.f_valV[k] : ly.f_valK[k]) + (int64_t)slot * ly.vstride[k];
        if (lane < s) idst[lane] = sidx[lane];
        if (ly.bits == 8) {
            if (lane < s) vdst[lane] = static_cast<uint8_t>(scode[lane]);
        } else if (lane < vb) {
            const int lo = scode[2 * lane] & 0xF;
            const int hi = (2 * lane + 1 < s) ? (scode[2 * lane + 1] & 0xF) : 0;
            vdst[lane] = static_cast<uint8_t>(lo | (hi << 4));
        }
        // 6. the gate folds into the stored scale
        if (lane == 0) {
            const uint16_t stored = (gate16 == 0x3C00) ? s16 : f2h(h2f(gate16) * sf);
            reinterpret_cast<uint16_t *>(blk + (z ? ly.f_scaleV[k] : ly.f_scaleK[k]))[slot] = stored;
        }
    }
}

// Encodes Z = z and stores the token's coefficients, residual record and
// scale at its slot, past the tier's counted tokens (so readers of the
// cache never use it before it is published).  Returns 1 if the token is
// admitted (the same answer in both waves), with its tier slot and
// position; the token is published by append_commit once both waves are
// done.
template <int D>
__device__ __forceinline__ int append_encode(const AppendRegs<D> &st, const Layout &ly, uint8_t *arena,
                                             int layer, int b, int h, int z, int lane,
                                             const AppendArgs &ap, const AppendLds &L, int &slot_out,
                                             int &n_out)
{
    const int bh = b * ly.Hkv + h;
    // admission (decided identically by both waves; wave 0 reports)
    int slot, n;
    const uint32_t err = append_admit(ly, st.k, st.cnt_l, slot, n);
    slot_out = slot;
    n_out = n;
    if (err) {
        if (z == 0 && lane == 0) atomicOr(err_ptr(ly, arena), err);
        return 0;
    }
    uint16_t *sB = L.B + z * (kMaxRank * kAppendBStride);
    encode_stage_basis<D>(st.brow, sB, ly.R, lane);
    const uint16_t *gp = z ? ap.gateV : ap.gateK;
    const uint16_t g = gp ? gp[bh] : uint16_t(0x3C00);
    encode_store<D>(st.brow, st.xv, sB, L.x + z * kMaxHeadDim, L.c + z * kMaxRank, L.code + z * kMaxResid,
                    L.idx + z * kMaxResid, ly, head_block_ptr(ly, arena, layer, b, h), st.k, slot, z, lane, g);
    return 1;
}

// Publishes an admitted token: its tier count and its position-map entry.
// Called by one thread after both waves' stores (a workgroup barrier).
__device__ __forceinline__ void append_commit(const Layout &ly, uint8_t *arena, int layer, int b, int h,
                                              int k, int slot, int n)
{
    counts_ptr(ly, arena, layer, b, h)[k] = slot + 1;
    posmap_ptr(ly, arena, layer, b, h)[n] = (k << 28) | slot;
}

}  // namespace dwkv
