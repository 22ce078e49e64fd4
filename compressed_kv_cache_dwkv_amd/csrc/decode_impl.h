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
// one 8-wave workgroup per compute unit.  A workgroup takes a work-balanced
// (tile shares plus a little of the bytes) run of 16-token blocks of the tier regions of its (sequence, KV head) and
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
//   * the V residual of the tile is written densely (code x scale) into a
//     per-wave LDS tile [channel][token] by the lane that owns the token and
//     multiplied by the same probabilities on the matrix cores; the written
//     cells are cleared afterwards.
// Inner loops have compile-time trip counts and no branches, so that a
// wave's LDS reads and matrix-core products stream back to back; only the
// tile's shape (its rank class) and its residual presence are branched on.
// The running max may trail the true max by up to 8 (a factor 256) before
// it moves, so probabilities stay well inside fp16.  The last workgroup
// of a (sequence, KV head) to finish merges all partials.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "append_body.h"
#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

constexpr int kBlock = 512;               // 8 waves: one workgroup fills a compute unit
constexpr int kWaves = kBlock / kWave;
constexpr int kTile = 64;                 // most tokens in a tile
constexpr int kSlots = 4;                 // 16x16 operand blocks per tile and Z (rank <= 64)
// The per-wave V-residual tile: channel rows (plus one row that absorbs
// unused entries) of fp16 cells, one column per token in 32-deep operand
// order.  Rows are padded so that the 16 rows of an operand read hit
// distinct banks: to 72 fp16 (16-byte reads) where the LDS holds it, else
// (8 query heads per KV head) to 68 (8-byte reads).
constexpr int kEvRows = kMaxHeadDim + 1;
constexpr int ev_stride(int gq) { return gq > 4 ? kTile + 4 : kTile + 8; }
constexpr int ev_wave(int gq) { return (kEvRows * ev_stride(gq) + 7) / 8 * 8; }   // fp16, 16-byte multiple
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxLag = 8.0f;           // log2 units the running max may trail

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// A loaded operand kept in registers: without it the compiler turns the
// per-block select of a shared operand into a masked reload for every block.
__device__ __forceinline__ half4_t in_reg(half4_t v)
{
    u32x2_t b = __builtin_bit_cast(u32x2_t, v);
    asm volatile("" : "+v"(b));
    return __builtin_bit_cast(half4_t, b);
}

// Ends a batch of LDS reads: the reads before it are all issued before
// anything after it, so a batch costs one LDS round trip (left alone, the
// compiler waits for each read before issuing the next).
__device__ __forceinline__ void lds_batch_end() { asm volatile("" ::: "memory"); }

// Eight loaded operands held in registers at once: the empty asm takes
// them all, so their reads are issued together and waited for once.
__device__ __forceinline__ void hold8(half8_t (&e)[4][2])
{
    asm volatile("" : "+v"(e[0][0]), "+v"(e[0][1]), "+v"(e[1][0]), "+v"(e[1][1]), "+v"(e[2][0]), "+v"(e[2][1]),
                 "+v"(e[3][0]), "+v"(e[3][1]));
}

__device__ __forceinline__ void hold8(float4_t (&e)[8])
{
    asm volatile("" : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), "+v"(e[6]),
                 "+v"(e[7]));
}

__device__ __forceinline__ void hold4(float4_t (&e)[4])
{
    asm volatile("" : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]));
}

// The fp16 values of v whose 16-bit lanes of (m0, m1) are ones; the others 0.
__device__ __forceinline__ half4_t keep_h4(half4_t v, uint32_t m0, uint32_t m1)
{
    const u32x2_t b = __builtin_bit_cast(u32x2_t, v);
    return __builtin_bit_cast(half4_t, u32x2_t{b[0] & m0, b[1] & m1});
}

__device__ __forceinline__ float4_t mma16(half4_t a, half4_t b, float4_t c)
{
    // D[m][n] += sum_k A[m][k] B[k][n]; lane l supplies A[l%16][4(l/16)+j],
    // B[4(l/16)+j][l%16] and holds D[4(l/16)+j][l%16], j = 0..3.
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// The same with 32-deep operands (two 4-deep pieces per lane).  Whatever
// order the hardware gives the 8 values of a lane in the contraction, A
// and B use the same one, so pairing two 16-deep operand pieces of A with
// the matching pieces of B sums exactly the products of the two 16-deep
// steps.
__device__ __forceinline__ float4_t mma32(half8_t a, half8_t b, float4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8_t cat(half4_t a, half4_t b)
{
    return half8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
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

// Index byte u (0..7) of a token's residual record.
__device__ __forceinline__ int idx_at(uint32_t i0, uint32_t i1, int u)
{
    return ((u < 4 ? i0 : i1) >> (8 * (u & 3))) & 0xFF;
}

// Signed code u of a token's record: `bits`-bit fields packed from bit 0 of
// the 64-bit word (c1:c0).
__device__ __forceinline__ float code_at(uint32_t c0, uint32_t c1, int u, int bits)
{
    const int pos = u * bits;
    // the builtin's result is typed unsigned: it must be read back as signed
    return (float)(int)__builtin_amdgcn_sbfe((int)(pos < 32 ? c0 : c1), pos & 31, bits);
}

// Partial results cross workgroups (and XCDs, whose L2s are not coherent
// with each other) as agent-scope relaxed atomics, two floats per access.
__device__ __forceinline__ void st_agent2(float *p, float x, float y)
{
    const uint64_t v = ((uint64_t)__float_as_uint(y) << 32) | __float_as_uint(x);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float4_t ld_agent4(const float *p)
{
    uint64_t *q = reinterpret_cast<uint64_t *>(const_cast<float *>(p));
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return float4_t{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                    __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}

// Where a tile lies, uniform over the wave.
struct Tile {
    int valid;        // 0 once the wave has no more tiles
    int k;            // tier
    int r, s;         // rank and residual channels of the tier
    int kbr;          // 16-channel blocks of the rank (1, 2, 4, 8)
    int lkbr;         // log2(kbr)
    int nv;           // valid tokens (<= 16 * slots / kbr)
    int blk0;         // first 16-token block
};

// Loads of one tile in flight: coefficient operand slots (slot i is m-block
// i / kbr, channel block i % kbr) and token `lane`'s residual records.
template <int NS>
struct TileData {
    half4_t ka[NS], va[NS];     // fp16 coefficients; with 8-bit ones, ka holds the back-projection operand
    uint32_t ka8[NS], va8[NS];  // 8-bit coefficient codes (4 per slot)
    uint32_t ki0, ki1, kc0, kc1, vi0, vi1, vc0, vc1;
    uint32_t ksc, vsc;          // fp16 scale in the low half
    uint32_t kcs;               // 8-bit form: the lane's token's K block scale (low half)
    u32x2_t vcs[4];             // 8-bit form: V block scales of tokens 4 grp .. 4 grp + 3 of 16-token block mb
};

// Four int8 codes (bytes of x) as exact fp16 values: each byte, sign bit
// flipped, becomes the low byte of an fp16 with exponent bits 0x64 (1024 +
// byte), and 1152 is subtracted (two packed fp16 subtractions).
__device__ __forceinline__ half4_t codes_h4(uint32_t x)
{
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    const uint32_t u = x ^ 0x80808080u;
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const half2_t off = half2_t{(_Float16)1152.0f, (_Float16)1152.0f};
    const half2_t a = __builtin_bit_cast(half2_t, lo) - off;
    const half2_t b = __builtin_bit_cast(half2_t, hi) - off;
    return half4_t{a[0], a[1], b[0], b[1]};
}

// This workgroup's block ranges, lane k holding tier k's values.
struct Ranges {
    int b0, b1;       // first and end 16-token block of the workgroup's run
    int cnt;          // tokens in the tier
    int nt;           // tiles of the run (low 28 bits) | log2(16-channel blocks) << 28
};

// A wave's position: its tiles are numbers wave, wave + 8, ... counted
// through the tiers in order, so the position only moves forward.
struct Cursor {
    int k;            // tier
    int rem;          // tile number within the tier's run
};

template <int NS>
__device__ __forceinline__ Tile locate(const Ranges &rg, Cursor &cur, const Layout &ly)
{
    int k = cur.k, rem = cur.rem;
    while (k < ly.T) {
        const int nt = __builtin_amdgcn_readlane(rg.nt, k) & 0x0FFFFFFF;
        if (rem < nt) break;
        rem -= nt;
        ++k;
    }
    cur.k = k;
    cur.rem = rem;
    Tile t;
    t.valid = k < ly.T;
    t.k = t.valid ? k : 0;
    const int lkbr = (int)((uint32_t)__builtin_amdgcn_readlane(rg.nt, t.k) >> 28);
    const int mbs = lkbr == 0 && NS == 8 ? 4 : NS >> lkbr;     // 16-token blocks: at most 4
    t.kbr = 1 << lkbr;
    t.lkbr = lkbr;
    t.r = ly.tier[t.k].rank;
    t.s = ly.tier[t.k].resid;
    const int blk0 = __builtin_amdgcn_readlane(rg.b0, t.k) + rem * mbs;
    int nv = (__builtin_amdgcn_readlane(rg.b1, t.k) - blk0) * 16;
    nv = nv < 16 * mbs ? nv : 16 * mbs;
    const int left = __builtin_amdgcn_readlane(rg.cnt, t.k) - blk0 * 16;
    t.nv = t.valid ? (nv < left ? nv : left) : 0;
    t.blk0 = t.valid ? blk0 : 0;
    return t;
}

// Issues every load of a tile: always the same number of load instructions,
// so the compiler's wait counts stay exact and the next tile's loads are
// never waited for while the current tile is computed.  The loads are
// buffer loads on the (layer, sequence, KV head) block: a 32-bit lane offset
// plus a wave-uniform offset per operand slot, so a tile costs almost no
// vector address arithmetic.  Slots and lanes past the tile's valid tokens
// or its rank read other bytes of the block, or zeros past its end; their
// values are zeroed where they are used.  A tile past the wave's last one
// loads, in its K slots, the wave's operand of the back-projection instead
// (slot i: channels 16 i + 4 grp.. of row `kbv` of the transposed V basis),
// so that operand arrives while the last tile is computed.
template <int NS, int CB>
__device__ __forceinline__ void issue_tile(const Tile &t, TileData<NS> &D, __amdgpu_buffer_rsrc_t rb,
                                           __amdgpu_buffer_rsrc_t rbv, uint32_t kbv, const Layout &ly,
                                           int lane)
{
    const int c16 = lane & 15, grp = lane >> 4;
    const TierDesc &td = ly.tier[t.k];
    const int r = t.r;
    const uint32_t tok0 = (uint32_t)t.blk0 * 16u;
    if constexpr (CB == 1) {
        // 8-bit codes: one byte per coefficient, the same arrangement; the
        // back-projection operand is loaded by every tile into ka (the loop
        // keeps the one of the tile past the last)
        const uint32_t sK = (uint32_t)td.coefK + tok0 * (uint32_t)r;
        const uint32_t sV = (uint32_t)td.coefV + tok0 * (uint32_t)r;
        const uint32_t kl = (uint32_t)(c16 * r + 4 * grp), vl = (uint32_t)(c16 * 16 + 4 * grp);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            D.ka8[i] = __builtin_amdgcn_raw_buffer_load_b32(rb, kl, sK + (uint32_t)td.koff[i], 0);
            D.va8[i] = __builtin_amdgcn_raw_buffer_load_b32(rb, vl, sV + (uint32_t)td.voff[i], 0);
            D.ka[i] = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(rbv, kbv, (uint32_t)i * 32u, 0));
        }
        // block scales: the lane's token's (K), tokens 4 grp .. of each 16-token block (V)
        const uint32_t tl = lane < t.nv ? (uint32_t)lane : 0u;
        D.kcs = __builtin_amdgcn_raw_buffer_load_b32(rb, (tl & ~1u) * 2u, (uint32_t)td.cscK + tok0 * 2u, 0) >>
                (16u * (tl & 1u));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            D.vcs[mb] = __builtin_amdgcn_raw_buffer_load_b64(rb, (uint32_t)(16 * mb + 4 * grp) * 2u,
                                                             (uint32_t)td.cscV + tok0 * 2u, 0);
    } else {
    // K: token rows of r fp16; V: 16-token blocks of r rows x 16 tokens --
    // both start r fp16 per token into their arrays
    const uint32_t sK = (uint32_t)td.coefK + tok0 * (uint32_t)r * 2u;
    const uint32_t sV = (uint32_t)td.coefV + tok0 * (uint32_t)r * 2u;
    const uint32_t vl = (uint32_t)(c16 * 16 + 4 * grp) * 2u;    // channel c16, tokens 4grp..
    const bool v = t.valid;
    const __amdgpu_buffer_rsrc_t rk = v ? rb : rbv;
    const uint32_t kl = v ? (uint32_t)(c16 * r + 4 * grp) * 2u : kbv;   // token c16, channels 4grp..
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const uint32_t ko = v ? sK + (uint32_t)td.koff[i] : (uint32_t)i * 32u;
        D.ka[i] = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(rk, kl, ko, 0));
        D.va[i] = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(rb, vl, sV + (uint32_t)td.voff[i], 0));
    }
    }
    // residual records of token `lane` (token 0's for lanes past the tile:
    // their indices must stay valid); a record's two words in one load
    const uint32_t tl = lane < t.nv ? (uint32_t)lane : 0u;
    const uint32_t io = tl * (uint32_t)td.istride, vo = tl * (uint32_t)td.vstride;
    const u32x2_t ki = __builtin_amdgcn_raw_buffer_load_b64(rb, io, (uint32_t)td.idxK + tok0 * (uint32_t)td.istride, 0);
    const u32x2_t kc = __builtin_amdgcn_raw_buffer_load_b64(rb, vo, (uint32_t)td.valK + tok0 * (uint32_t)td.vstride, 0);
    const u32x2_t vi = __builtin_amdgcn_raw_buffer_load_b64(rb, io, (uint32_t)td.idxV + tok0 * (uint32_t)td.istride, 0);
    const u32x2_t vc = __builtin_amdgcn_raw_buffer_load_b64(rb, vo, (uint32_t)td.valV + tok0 * (uint32_t)td.vstride, 0);
    // scales: the aligned 4-byte word holding this token's fp16 (tok0 is even)
    const uint32_t so = (tl & ~1u) * 2u, sh = 16u * (tl & 1u);
    D.ksc = __builtin_amdgcn_raw_buffer_load_b32(rb, so, (uint32_t)td.scaleK + tok0 * 2u, 0) >> sh;
    D.vsc = __builtin_amdgcn_raw_buffer_load_b32(rb, so, (uint32_t)td.scaleV + tok0 * 2u, 0) >> sh;
    D.ki0 = ki[0];
    D.ki1 = ki[1];
    D.kc0 = kc[0];
    D.kc1 = kc[1];
    D.vi0 = vi[0];
    D.vi1 = vi[1];
    D.vc0 = vc[0];
    D.vc1 = vc[1];
}

// Per-wave state of the online softmax and the value sums.
template <int GQ, int KB, int D>
struct WaveAcc {
    // basis-space value sums, 16 / GP channel blocks per accumulator: row
    // GP q + g, column c of accumulator a is head g, channel 16 (a 16 / GP + q) + c
    float4_t O[KB * (GQ < 4 ? 4 : GQ) / 16];
    float4_t Ores[D / 16];               // residual value mass [head row][channel]
    float l[GQ];                         // this lane's share of the normalisers
    float m[GQ];                         // running max per head (the same in every lane)
};

// fp16 probabilities of a wave's tile in LDS, [head][token] with the tokens
// of each 32-token chunk ordered as the lanes of a 32-deep operand hold
// them: token 16 h + 4 g + i of the chunk (h < 2, g < 4, i < 4) sits at
// 8 g + 4 h + i, so one 16-byte read gives a lane its operand.  Row GQ stays
// zero (the operand rows of padding heads).
constexpr int kPStride = kTile + 8;        // fp16 per head row (16-byte multiple)
__device__ __forceinline__ int p_slot(int t)
{
    return (t & ~31) | ((t & 12) << 1) | ((t & 16) >> 2) | (t & 3);
}

// Row h of the value products' A operand: 0 for the rows past the heads.
template <int GQ>
__device__ __forceinline__ const _Float16 *p_row(const _Float16 *sP, int c16)
{
    return sP + (c16 < GQ ? c16 : GQ) * kPStride;
}

// One tile of a wave: every rank class runs the same instructions, the
// slot -> (16-token block, 16-channel block) map coming from the tile at run
// time, so the accumulators never pass through per-class code paths.
template <int GQ, int KB, int D, int BITS, int CB>
__device__ __forceinline__ void process_tile(const Tile &t, const TileData<kSlots * (KB / 4)> &Dt,
                                             const half4_t *s_qb, WaveAcc<GQ, KB, D> &A,
                                             const float (*s_qt)[GQ < 4 ? 4 : GQ], _Float16 *sP,
                                             _Float16 *ev, const TierDesc *tiers, int lane)
{
    constexpr int bits = BITS;                      // code width: fields at fixed positions
    constexpr int NS = kSlots * (KB / 4);
    constexpr int GP = GQ < 4 ? 4 : GQ;
    constexpr int NU = GP / 4;                      // score accumulators (4 heads each)
    constexpr int ND = D / 16;
    constexpr int G4 = 16 / GP;                     // channel blocks per packed value accumulator
    constexpr int NA = KB / G4;
    const int c16 = lane & 15, grp = lane >> 4;
    const int r = t.r, s = t.s, nv = t.nv, kbr = t.kbr, lkbr = t.lkbr;
    // the tile's 16-token blocks (one token per lane: at most 4)
    const int mbs = (NS >> lkbr) < kTile / 16 ? NS >> lkbr : kTile / 16;
    const bool full = nv == 16 * mbs;               // uniform: no token masks needed
    const bool tok = lane < nv;                     // this lane's token is in the tile
    // this lane's token column in the probability table and the V-residual
    // tile (32-deep operand order: one 16-byte read per operand)
    const int ps = p_slot(lane);
    constexpr int EVS = ev_stride(GQ);

    // ---- scores, one token per lane: for slot i (block mb, channel block
    //      kb) the A rows 4 mb + j carry q' of head 4 u + j (hi and lo
    //      parts, read from the q' table; other rows read its zero block),
    //      the B operand the tokens' coefficients, so row 4 grp + j of
    //      accumulator u is (token lane, head 4 u + j)
    float4_t Sc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) Sc[u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // (the B operand's columns are tokens and every product adds 0 x B into
    // the other blocks' rows: channels past the rank and tokens past the
    // tile must be zeros, not whatever the arena holds there)
    half4_t qa[NS][NU][2];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int mb = i >> lkbr, kb = i & (kbr - 1);  // uniform
        const bool rows = (c16 >> 2) == mb;
        const half4_t *qp = s_qb + (rows ? kb : KB) * kWave + 16 * grp + (c16 & 3);
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) qa[i][u][hl] = qp[4 * u + 8 * hl];
    }
    lds_batch_end();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int mb = i >> lkbr, kb = i & (kbr - 1);  // uniform
        const bool col = mb < kTile / 16 && (full || 16 * mb + c16 < nv);
        const bool chan = 16 * kb + 4 * grp < r;
        half4_t bk = CB == 2 ? Dt.ka[i] : codes_h4(Dt.ka8[i]);
        if (!(col && chan)) bk = half4_t{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) Sc[u] = mma16(qa[i][u][hl], bk, Sc[u]);
    }

    // ---- residuals, one token per lane.  Entries past s are given index
    //      128 (a zero row of q, the spare row of the V-residual tile) and
    //      code 0, a whole record word at a time (s = 0: every entry).  K:
    //      logit terms from q gathered in LDS, added to the lane's scores.
    //      V: the token's cells of the dense LDS tile.
    float z[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) z[g] = Sc[g / 4][g % 4];
    if constexpr (CB == 1) {
        // 8-bit coefficients: the scores so far are q' . codes; times the
        // token's block scale
        const float kcs = h2f((uint16_t)Dt.kcs);
#pragma unroll
        for (int g = 0; g < GP; ++g) z[g] *= kcs;
    }
    const TierDesc &td = tiers[t.k];
    const uint32_t im0 = td.im0, im1 = td.im1, cm0 = td.cm0, cm1 = td.cm1;
    {
        const uint32_t ki0 = (Dt.ki0 & im0) | (0x80808080u & ~im0);
        const uint32_t ki1 = (Dt.ki1 & im1) | (0x80808080u & ~im1);
        const uint32_t kc0 = Dt.kc0 & cm0, kc1 = Dt.kc1 & cm1;
        float rk[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) rk[g] = 0.0f;
        // every gather requested before the first is used: one LDS round
        // trip for the token's entries, not one per entry
        float4_t qg[kMaxResid][GP / 4];
#pragma unroll
        for (int u = 0; u < kMaxResid; ++u)
#pragma unroll
            for (int p = 0; p < GP / 4; ++p)
                qg[u][p] = *reinterpret_cast<const float4_t *>(&s_qt[idx_at(ki0, ki1, u)][4 * p]);
        lds_batch_end();
#pragma unroll
        for (int u = 0; u < kMaxResid; ++u) {
            const float cv = code_at(kc0, kc1, u, bits);
#pragma unroll
            for (int g = 0; g < GP; ++g) rk[g] += cv * qg[u][g / 4][g % 4];
        }
        // (a tier without residuals has no scale array: its scale reads 0)
        const float sck = s > 0 ? h2f((uint16_t)Dt.ksc) : 0.0f;
#pragma unroll
        for (int g = 0; g < GQ; ++g) z[g] += rk[g] * sck;
    }
    // V cells of the lane's token (lanes past the tile leave their columns
    // zero)
    const uint32_t vi0 = (Dt.vi0 & im0) | (0x80808080u & ~im0);
    const uint32_t vi1 = (Dt.vi1 & im1) | (0x80808080u & ~im1);
    if (tok) {
        const uint32_t vc0 = Dt.vc0 & cm0, vc1 = Dt.vc1 & cm1;
        const _Float16 scv = s > 0 ? __builtin_bit_cast(_Float16, (uint16_t)Dt.vsc) : (_Float16)0.0f;
#pragma unroll
        for (int u = 0; u < kMaxResid; ++u) {
            const int pos = u * bits;
            const int code = (int)__builtin_amdgcn_sbfe((int)(pos < 32 ? vc0 : vc1), pos & 31, bits);
            ev[idx_at(vi0, vi1, u) * EVS + ps] = (_Float16)(int16_t)code * scv;
        }
    }
    wave_fence();
#pragma unroll
    for (int g = 0; g < GQ; ++g) z[g] = tok ? z[g] : -INFINITY;

    // ---- lazy running max: only when a logit passes its head's max by more
    //      than the lag are the max and every accumulator rescaled (rare)
    bool over = false;
#pragma unroll
    for (int g = 0; g < GQ; ++g) over |= z[g] > A.m[g] + kMaxLag;
    float f[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) f[g] = 1.0f;
    if (__builtin_amdgcn_ballot_w64(over)) {
        // (kept a branch: without the barrier the compiler computes the
        // reductions on every tile and selects their results)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
            const float tmax = wave_max(z[g]);
            // the same in every lane: kept in a scalar register
            const float nm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                                 int, tmax > A.m[g] + kMaxLag ? tmax : A.m[g])));
            f[g] = fast_exp2(A.m[g] - nm);
            A.m[g] = nm;
        }
    }
    // (the factors are applied every tile, 1 when the max held: accumulators
    // updated inside the branch make the compiler keep two copies of them).
    // Accumulator row 4 grp + j holds head (4 grp + j) % GP -- or nothing
    // (rows past the heads are zero, any factor keeps them so).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float fh = 1.0f;
        if constexpr (GP == 4) {
            if (j < GQ) fh = f[j];
        } else {
            // (both factors pinned first: a select between two elements of
            // f became an indexed load from scratch memory)
            float fa = f[j], fb = f[4 + j];
            asm volatile("" : "+v"(fa), "+v"(fb));
            fh = (grp & 1) ? fb : fa;
        }
#pragma unroll
        for (int a = 0; a < NA; ++a) A.O[a][j] *= fh;
#pragma unroll
        for (int nb = 0; nb < ND; ++nb) A.Ores[nb][j] *= fh;
    }
#pragma unroll
    for (int g = 0; g < GQ; ++g) A.l[g] *= f[g];

    // ---- probabilities: to LDS in operand order; the lane's normaliser
    //      terms are the same fp16 values
    {
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
            const _Float16 ph = (_Float16)fast_exp2(z[g] - A.m[g]);
            sP[g * kPStride + ps] = ph;
            A.l[g] += (float)ph;
        }
    }
    wave_fence();

    // ---- values: P x V coefficients in basis space.  Slot i adds its
    //      16 tokens x 16 channels into the packed accumulator of channel
    //      block kb: rows GP (kb % G4) + g are head g, the A rows of the
    //      lanes of other blocks read the zero row.  V coefficients of
    //      tokens past the tile are zeroed (they meet p = 0, but 0 x whatever
    //      the arena holds there need not be 0): whole-register masks.
    const int rq = c16 / GP, rh = c16 % GP;         // this lane's A row: block group, head
    half4_t va[NS];
    if constexpr (CB == 1) {
        // 8-bit coefficients: codes times the block scales of the lane's four
        // tokens of the slot's 16-token block (fp16 products, one rounding)
        // (the four scale pairs pinned in registers first: a select among
        // elements of the tile's array became an indexed load from a
        // scratch copy of the whole tile)
        u32x2_t w0 = Dt.vcs[0], w1 = Dt.vcs[1], w2 = Dt.vcs[2], w3 = Dt.vcs[3];
        asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int mb = i >> lkbr;                  // uniform
            const u32x2_t w = mb == 0 ? w0 : mb == 1 ? w1 : mb == 2 ? w2 : w3;
            va[i] = codes_h4(Dt.va8[i]) * __builtin_bit_cast(half4_t, w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NS; ++i) va[i] = Dt.va[i];
    }
    if (!full) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int t0 = 16 * (i >> lkbr) + 4 * grp;
            const uint32_t m0 = (t0 < nv ? 0xFFFFu : 0u) | (t0 + 1 < nv ? 0xFFFF0000u : 0u);
            const uint32_t m1 = (t0 + 2 < nv ? 0xFFFFu : 0u) | (t0 + 3 < nv ? 0xFFFF0000u : 0u);
            va[i] = keep_h4(va[i], m0, m1);
        }
    }
    half4_t pv[NS][NA];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int mb = i >> lkbr, kb = i & (kbr - 1);  // uniform
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const bool on = mb < kTile / 16 && a * G4 + rq == kb && rh < GQ;
            const _Float16 *pr = on ? sP + rh * kPStride + 32 * (mb >> 1) + 4 * (mb & 1) + 8 * grp
                                    : sP + GQ * kPStride + 8 * grp;
            pv[i][a] = *reinterpret_cast<const half4_t *>(pr);
        }
    }
    lds_batch_end();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int mb = i >> lkbr, kb = i & (kbr - 1);  // uniform
        half4_t bv = va[i];
        if (!(mb < kTile / 16 && 16 * kb + c16 < r)) bv = half4_t{0, 0, 0, 0};
#pragma unroll
        for (int a = 0; a < NA; ++a) A.O[a] = mma16(pv[i][a], bv, A.O[a]);
    }

    // ---- V residual mass: the dense tile times the probabilities (32-deep
    //      chunks; tokens past the tile have p = 0), then the written cells
    //      are cleared (after the reads: same wave, in order)
    {
        const _Float16 *prow = p_row<GQ>(sP, c16);
        half8_t PA[kTile / 32];
#pragma unroll
        for (int p = 0; p < kTile / 32; ++p) PA[p] = *reinterpret_cast<const half8_t *>(prow + 32 * p + 8 * grp);
        const _Float16 *evr = ev + c16 * EVS + 8 * grp;
        constexpr int NB = ND < 4 ? ND : 4;          // channel blocks per batch of reads
#pragma unroll
        for (int n0 = 0; n0 < ND; n0 += NB) {
            half8_t E[NB][kTile / 32];
#pragma unroll
            for (int q = 0; q < NB; ++q)
#pragma unroll
                for (int p = 0; p < kTile / 32; ++p) {
                    const _Float16 *e = evr + 16 * (n0 + q) * EVS + 32 * p;
                    if constexpr (EVS % 8 == 0)
                        E[q][p] = *reinterpret_cast<const half8_t *>(e);
                    else
                        E[q][p] = cat(*reinterpret_cast<const half4_t *>(e), *reinterpret_cast<const half4_t *>(e + 4));
                }
            if constexpr (NB == 4 && kTile / 32 == 2) hold8(E);
#pragma unroll
            for (int q = 0; q < NB; ++q)
#pragma unroll
                for (int p = 0; p < kTile / 32; ++p) A.Ores[n0 + q] = mma32(PA[p], E[q][p], A.Ores[n0 + q]);
        }
        wave_fence();
        if (tok) {
#pragma unroll
            for (int u = 0; u < kMaxResid; ++u) ev[idx_at(vi0, vi1, u) * EVS + ps] = (_Float16)0.0f;
        }
    }
}

// Publishes the appended token (tier count and position-map entry) from the
// last workgroup of its (sequence, KV head): every workgroup of the head has
// read the token counts by then.  The tier comes from the same input as the
// encoder's and the counts are the ones this workgroup read, so admission
// matches the encoder's.  Called by one wave; lane k of cnt_l holds tier k's count.
__device__ __forceinline__ void publish_token(const Layout &ly, uint8_t *arena, int layer, int b, int h,
                                              int tier_v, int cnt_l, int lane)
{
    const int tier = __builtin_amdgcn_readfirstlane(tier_v);
    int slot, n;
    if (append_admit(ly, tier, cnt_l, slot, n) == 0 && lane == 0) append_commit(ly, arena, layer, b, h, tier, slot, n);
}

template <int GQ, int KB, int D, int BITS, int CB>
__global__ __launch_bounds__(kBlock, 1) void decode_kernel(Layout ly, uint8_t *arena, int layer,
                                                           const uint16_t *q, float *out,
                                                           DecodeWorkspace ws, int S, double invS,
                                                           float qscale, AppendArgs ap)
{
    constexpr int GP = GQ < 4 ? 4 : GQ;           // query heads padded for 16-byte gathers
    constexpr int NS = kSlots * (KB / 4);          // operand slots per tile and Z
    constexpr int ND = D / 16;                     // channel blocks of the head
    constexpr int RMAX = 16 * KB;                  // largest rank this instance handles
    static_assert(KB <= kWaves, "one wave per block of q'");
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = uni(tid / kWave), lane = lane_id();
    const int c16 = lane & 15, grp = lane >> 4;
    const int R = ly.R;
    const int g0 = h * GQ;

    constexpr int EVW = ev_wave(GQ);
    __shared__ __attribute__((aligned(16))) _Float16 s_ev[kWaves * EVW];   // V-residual tiles
    __shared__ __attribute__((aligned(16))) float s_qt[kMaxHeadDim + 1][GP];   // q, base-2 units; zero rows
                                                                                // from D on (row 128: unused entries)
    // per-wave area: the tile probabilities in the loop, the merged sums after
    constexpr int kPBytes = (GQ + 1) * kPStride * 2;
    constexpr int kQpBytes = (GQ * (RMAX + D) * 4 / kWaves + 15) / 16 * 16;
    constexpr int kWvBytes = kPBytes > kQpBytes ? kPBytes : kQpBytes;
    __shared__ __attribute__((aligned(16))) uint8_t s_wv[kWaves * kWvBytes];
    __shared__ half4_t s_qb[(KB + 1) * kWave];     // score operand q', [channel block][lane]; block KB zero
    __shared__ float s_m[kWaves][GQ], s_l[kWaves][GQ];
    __shared__ float s_M[GQ], s_L[GQ];
    __shared__ int s_last;
    static_assert(GQ * (RMAX + D) * 4 <= sizeof(s_wv) && kPBytes % 16 == 0, "per-wave area");

    // ---- token counts first (one lane per tier), then the query in
    //      operand layout and, for waves 0..KB-1, one 16-row block of B_K
    const int T = ly.T;
    const int kl = lane < T ? lane : 0;
    // every per-tier value of lane k's tier, requested together and without
    // a branch, so the loads are in flight at once
    const int cnt_raw = counts_ptr(ly, arena, layer, b, h)[kl];
    const int r_l = ly.rank[kl];
    const int cost_l = ly.cost[kl];
    const double icb_l = ly.inv_cblk[kl];
    const int cnt_l = lane < T ? cnt_raw : 0;
    const int gq = c16 & 7;
    const uint16_t *qrow = q + ((int64_t)b * ly.Hq + g0 + (gq < GQ ? gq : 0)) * D;
    half4_t bq[ND], ak[ND];
#pragma unroll
    for (int kb = 0; kb < ND; ++kb) bq[kb] = *reinterpret_cast<const half4_t *>(qrow + 16 * kb + 4 * grp);
    // this thread's entries of the residual-gather table, requested now with
    // the counts (the table is written once the first tile is issued)
    constexpr int kQtEntries = (kMaxHeadDim + 1) * GP;
    constexpr int kQtPer = (kQtEntries + kBlock - 1) / kBlock;
    uint16_t qt_h[kQtPer];
#pragma unroll
    for (int e = 0; e < kQtPer; ++e) {
        const int i = tid + e * kBlock, j = i / GP, g = i % GP;
        qt_h[e] = i < kQtEntries && g < GQ && j < D ? q[((int64_t)b * ly.Hq + g0 + g) * D + j] : (uint16_t)0;
    }
    if (wave < KB) {
        const uint16_t *BK = basis_ptr(ly, arena, layer / ly.G, 0, h);
        const int row = 16 * wave + c16 < R ? 16 * wave + c16 : R - 1;
#pragma unroll
        for (int kb = 0; kb < ND; ++kb)
            ak[kb] = *reinterpret_cast<const half4_t *>(BK + (int64_t)row * D + 16 * kb + 4 * grp);
    }
    // With new tokens to append, waves 0 and 1 of the first workgroup of
    // each (sequence, KV head) encode them while the workgroup waits for its
    // first tiles; the token goes to its slot past the tier's counted tokens,
    // which no tile of this launch uses, and the last workgroup publishes it.
    const bool appending = ap.k != nullptr;
    const bool encoder = appending && split == 0;
    AppendRegs<D> app;
    if (encoder && wave < 2) append_fetch<D>(app, ly, arena, layer, b, h, wave, lane, ap);

    // ---- this workgroup's work-balanced run of 16-token blocks: lane k
    //      works out and keeps tier k's range
    const uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);
    // buffer resource on the block (reads past its end return zeros), built
    // from scalar registers so every load takes it directly
    const __amdgpu_buffer_rsrc_t rb = block_rsrc(blk, ly.head_block);
    // the transposed V basis (back-projection operand: row 16 w + c16 for wave w)
    const __amdgpu_buffer_rsrc_t rbv = block_rsrc(
        reinterpret_cast<const uint8_t *>(basis_vt_ptr(ly, arena, layer / ly.G, h)), (int64_t)R * D * 2);
    const uint32_t kbv = (uint32_t)((16 * (wave < ND ? wave : 0) + c16) * R + 4 * grp) * 2u;
    // ---- a first tile whose place needs no token count: tile (split, wave)
    //      of tier 0's first S * 8 tiles, its loads requested ahead of the
    //      work-balanced ranges (which need the counts).  Its valid tokens are
    //      known once the counts are (lanes past them are masked as in any
    //      tile; a tile with none is skipped), and the balanced runs below
    //      start after these tiles.  (Requesting it ahead of the counts
    //      themselves was slower: 2048 waves' tile loads then queue in front
    //      of the loads the prologue waits for.)
    TileData<NS> DA, DB;
    Tile ta;
    {
        const int r0 = ly.tier[0].rank;
        const int lkbr0 = (r0 > 16) + (r0 > 32) + (r0 > 64);
        const int mbs0 = lkbr0 == 0 && NS == 8 ? 4 : NS >> lkbr0;
        ta.valid = 1;
        ta.k = 0;
        ta.r = r0;
        ta.s = ly.tier[0].resid;
        ta.kbr = 1 << lkbr0;
        ta.lkbr = lkbr0;
        ta.blk0 = (split * kWaves + wave) * mbs0;
        ta.nv = 16 * mbs0;
    }
    issue_tile<NS, CB>(ta, DA, rb, rbv, kbv, ly, lane);
    const int static_blocks = S * kWaves * (ta.nv >> 4);   // tier 0's blocks the first tiles cover
    Ranges rg;
    {
        // (fp32: every workgroup evaluates the same expressions for a shared
        // boundary, so neighbours agree exactly; the first and last
        // boundaries are exact, so the runs cover every block once)
        const bool on = lane < T;
        const int nall_l = on ? (cnt_l + 15) >> 4 : 0;                // 16-token blocks of tier k
        const int bs_l = lane == 0 ? min(nall_l, static_blocks) : 0;  // of them, in the first tiles
        const int nb_l = nall_l - bs_l;                                // balanced over the splits
        const float wt_l = (float)nb_l * (16.0f * (float)cost_l);   // work of tier k's blocks
        float W = 0.0f, wk_l = 0.0f;                               // total; work of the tiers before k
#pragma unroll
        for (int k = 0; k < kMaxTiers; ++k) {
            const float wt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt_l), k));
            if (lane > k) wk_l += wt;
            W += wt;
        }
        // the encoding workgroup starts its share later: its boundaries
        // move down by the encoding's cost in balance units
        const float E = appending ? ap.enc_units : 0.0f;
        const float step = (W + E) * (float)invS;
        const float icb = (float)icb_l;
        const float x0 = fmaxf(floorf(step * (float)split) - E, 0.0f) - wk_l;
        const float x1 = fmaxf(floorf(step * (float)(split + 1)) - E, 0.0f) - wk_l;
        const int c0 = (int)fmaxf(ceilf(x0 * icb), 0.0f), c1 = (int)fmaxf(ceilf(x1 * icb), 0.0f);
        const int b0 = split == 0 ? 0 : (c0 < nb_l ? c0 : nb_l);
        const int b1 = split + 1 == S ? nb_l : (c1 < nb_l ? c1 : nb_l);
        const int lkbr = (r_l > 16) + (r_l > 32) + (r_l > 64);     // log2 of 16-channel blocks
        // log2 of 16-token blocks per tile: NS / (channel blocks), at most 4
        // (one token per lane)
        const int lmbs = lkbr == 0 ? 2 : (NS == 8 ? 3 : 2) - lkbr;
        const int nt_l = (b1 - b0 + (1 << lmbs) - 1) >> lmbs;
        rg.b0 = bs_l + b0;
        rg.b1 = bs_l + b1;
        rg.cnt = cnt_l;
        rg.nt = nt_l | (lkbr << 28);
    }

    // ---- the first balanced tile's loads; the first tile's valid tokens
    Cursor cur{0, wave};
    Tile tb = locate<NS>(rg, cur, ly);
    issue_tile<NS, CB>(tb, DB, rb, rbv, kbv, ly, lane);
    {
        const int left = __builtin_amdgcn_readlane(cnt_l, 0) - 16 * ta.blk0;
        ta.nv = left < 0 ? 0 : (left < ta.nv ? left : ta.nv);
    }

    // ---- query in base-2 logit units (LDS, for residual gathers); this
    //      wave's V-residual tile cleared
#pragma unroll
    for (int e = 0; e < kQtPer; ++e) {
        const int i = tid + e * kBlock;
        if (i < kQtEntries) s_qt[i / GP][i % GP] = qscale * h2f(qt_h[e]);
    }
    _Float16 *ev = s_ev + wave * EVW;
    constexpr int kAppendTiles = 4;                 // V-residual tiles the append scratch covers
    static_assert(kAppendLdsBytes <= kAppendTiles * EVW * sizeof(_Float16), "append scratch");
    if (!(encoder && wave < kAppendTiles)) {
        uint4 *e4 = reinterpret_cast<uint4 *>(ev);
        if constexpr (ev_stride(GQ) % 8 == 0) {
            // the cells the products read: channel rows 0..D-1, token columns
            // 0..63 (the spare row only ever receives zeros; the padding is
            // never read)
            constexpr int RW = ev_stride(GQ) / 8;   // 16-byte pieces per row
#pragma unroll 4
            for (int i = lane; i < D * (kTile / 8); i += kWave) e4[(i >> 3) * RW + (i & 7)] = uint4{0u, 0u, 0u, 0u};
        } else {
            for (int i = lane; i < EVW / 8; i += kWave) e4[i] = uint4{0u, 0u, 0u, 0u};
        }
    }

    // ---- score operand qb: q' = B_K q on the matrix cores, straight into
    //      operand layout (wave mb forms block mb, shared through LDS).
    //      Column c16 carries query head c16 % 8 -- as fp16(q') for c16 < 8
    //      and as the remainder fp16(q' - fp16(q')) above -- so that the fp16
    //      products reproduce q' to ~2^-22.  Products of fp16 inputs are
    //      exact and sums fp32: q' is fp32-accurate.
    if (wave < KB) {
        float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < ND; ++kb) acc = mma16(ak[kb], gq < GQ ? bq[kb] : half4_t{0, 0, 0, 0}, acc);
        half4_t v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x = 16 * wave + 4 * grp + j < R ? qscale * acc[j] : 0.0f;
            const _Float16 xh = (_Float16)x;
            const _Float16 xl = (_Float16)(x - (float)xh);
            v[j] = c16 < 8 ? xh : xl;
        }
        s_qb[wave * kWave + lane] = v;
    }
    if (wave == KB % kWaves) s_qb[KB * kWave + lane] = half4_t{0, 0, 0, 0};
    if (encoder && wave < 2) {
        int slot, n;
        append_encode<D>(app, ly, arena, layer, b, h, wave, lane, ap, carve_append_lds(s_ev), slot, n);
    }
    __syncthreads();
    if (encoder && wave < 2) {
        // both encodings are done: clear the V-residual tiles of waves 0..3
        // the append scratch spanned
#pragma unroll
        for (int t = 0; t < kAppendTiles / 2; ++t) {
            uint4 *e4 = reinterpret_cast<uint4 *>(s_ev + (wave + 2 * t) * EVW);
            for (int i = lane; i < EVW / 8; i += kWave) e4[i] = uint4{0u, 0u, 0u, 0u};
        }
    }
    if (encoder) __syncthreads();                  // waves 2, 3 write their tiles only after this
    // (the A operand of the scores for lane (c16, grp): q' (hi, lo) of head
    // 4 u + c16 % 4, channels 16 kb + 4 grp + 0..3, at s_qb[64 kb + 16 grp +
    // c16 % 4 + 4 u + 8 hl])
    // this wave's probability rows; row GQ (the padding heads' operand) zero
    _Float16 *sP = reinterpret_cast<_Float16 *>(s_wv + wave * kWvBytes);
    if (lane < kPStride / 8) reinterpret_cast<uint4 *>(sP + GQ * kPStride)[lane] = uint4{0u, 0u, 0u, 0u};

    // ---- main loop: two-deep pipeline over this wave's tiles
    WaveAcc<GQ, KB, D> A;
    constexpr int NA = KB * GP / 16;               // packed value accumulators
#pragma unroll
    for (int a = 0; a < NA; ++a) A.O[a] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) A.Ores[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
        A.l[g] = 0.0f;
        A.m[g] = -INFINITY;
    }
    // (the tile past a wave's last holds the B_V operand: copied out at the
    // loop's exits, not selected between the buffers after it)
    half4_t bvt[NS];
    if (ta.nv > 0) process_tile<GQ, KB, D, BITS, CB>(ta, DA, s_qb, A, s_qt, sP, ev, ly.tier, lane);
    while (true) {
        if (!tb.valid) {
#pragma unroll
            for (int i = 0; i < NS; ++i) bvt[i] = DB.ka[i];
            break;
        }
        cur.rem += kWaves;
        ta = locate<NS>(rg, cur, ly);
        issue_tile<NS, CB>(ta, DA, rb, rbv, kbv, ly, lane);
        process_tile<GQ, KB, D, BITS, CB>(tb, DB, s_qb, A, s_qt, sP, ev, ly.tier, lane);
        if (!ta.valid) {
#pragma unroll
            for (int i = 0; i < NS; ++i) bvt[i] = DA.ka[i];
            break;
        }
        cur.rem += kWaves;
        tb = locate<NS>(rg, cur, ly);
        issue_tile<NS, CB>(tb, DB, rb, rbv, kbv, ly, lane);
        process_tile<GQ, KB, D, BITS, CB>(ta, DA, s_qb, A, s_qt, sP, ev, ly.tier, lane);
    }

    // ---- merge the waves of this workgroup: each wave leaves its unscaled
    //      sums in its own (now idle) V-residual tile, then one barrier
    {
        float lw[GQ];
#pragma unroll
        for (int g = 0; g < GQ; ++g) lw[g] = wave_sum(A.l[g]);
        if (lane == 0) {
#pragma unroll
            for (int g = 0; g < GQ; ++g) {
                s_m[wave][g] = A.m[g];
                s_l[wave][g] = lw[g];
            }
        }
    }
    {
        float *part = reinterpret_cast<float *>(ev);            // [GQ][RMAX + D]
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 4 * grp + j;
            const int g = row % GP, kq = row / GP;                // packed row: head, block in group
            if (g < GQ) {
#pragma unroll
                for (int a = 0; a < NA; ++a) part[g * (RMAX + D) + 16 * (a * (16 / GP) + kq) + c16] = A.O[a][j];
            }
            if (row < GQ) {
#pragma unroll
                for (int nb = 0; nb < ND; ++nb) part[row * (RMAX + D) + RMAX + 16 * nb + c16] = A.Ores[nb][j];
            }
        }
    }
    __syncthreads();
    // weights 2^(m_w - M) in a fixed wave order (bitwise reproducible);
    // merged sums go to the K-residual area, idle now
    float *s_qp = reinterpret_cast<float *>(s_wv);                // [GQ][RMAX + D]
    static_assert((RMAX + D) % 4 == 0 && (EVW * 2) % 16 == 0, "float4 merge");
    static_assert(kWaves == 8, "one batch of eight wave parts");
    for (int i4 = 4 * tid; i4 < GQ * (RMAX + D); i4 += 4 * kBlock) {
        const int g = i4 / (RMAX + D);
        float4_t pw[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            pw[w] = *reinterpret_cast<const float4_t *>(reinterpret_cast<const float *>(s_ev + w * EVW) + i4);
        float mw[kWaves], lw[kWaves];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mw[w] = s_m[w][g];
            lw[w] = s_l[w][g];
            M = fmaxf(M, mw[w]);
        }
        hold8(pw);
        float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = M == -INFINITY ? 0.0f : fast_exp2(mw[w] - M);
            acc += f * pw[w];
            L += f * lw[w];
        }
        *reinterpret_cast<float4_t *>(s_qp + i4) = acc;
        if (i4 == g * (RMAX + D)) {
            s_M[g] = M;
            s_L[g] = L;
        }
    }
    __syncthreads();
    // one back-projection through B_V plus the residual mass, on the matrix
    // cores: wave w forms output channels 16w..16w+15 as
    // out[g][j] = res[g][j] + sum_i B_V[i][j] a[g][i], with B_V^T rows as the
    // A operand (exact fp16) and a as fp16 hi and lo parts in columns g and
    // 8 + g (products exact, sums fp32), the two halves added across lanes
    if (wave < ND) {
        float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        const int g = c16 & 7;
        const int gr = g < GQ ? g : 0;
        static_assert(NS == 4 || NS == 8, "back-projection batches");
        float4_t av[NS];
#pragma unroll
        for (int kb = 0; kb < NS; ++kb)
            av[kb] = *reinterpret_cast<const float4_t *>(&s_qp[gr * (RMAX + D) + 16 * kb + 4 * grp]);
        const float4_t res =
            *reinterpret_cast<const float4_t *>(&s_qp[gr * (RMAX + D) + RMAX + 16 * wave + 4 * grp]);
#pragma unroll
        for (int k0 = 0; k0 < NS; k0 += 4) hold4(*reinterpret_cast<float4_t (*)[4]>(&av[k0]));
#pragma unroll
        for (int kb = 0; kb < NS; ++kb) {
            half4_t bb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * kb + 4 * grp + j;
                const float x = g < GQ && i < R ? av[kb][j] : 0.0f;
                const _Float16 xh = (_Float16)x;
                bb[j] = c16 < 8 ? xh : (_Float16)(x - (float)xh);
            }
            acc = mma16(bvt[kb], bb, acc);
        }
        if (c16 < GQ) {
            float *po = ws.po + (((int64_t)b * ly.Hq + g0 + c16) * S + split) * D + 16 * wave + 4 * grp;
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = acc[j] + row_swap8(acc[j]) + res[j];
            st_agent2(po, o[0], o[1]);
            st_agent2(po + 2, o[2], o[3]);
        }
    }
    static_assert(GQ <= kMlNorm, "maxima and normalisers share a line");
    if (tid < GQ) {
        const int64_t ml = (((int64_t)b * ly.Hkv + h) * S + split) * kMlStride + tid;
        __hip_atomic_store(ws.pm + ml, s_M[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ws.pl + ml, s_L[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- the last workgroup of this (sequence, KV head) merges the splits.
    // Partials travel as agent-scope (cross-XCD coherent) relaxed stores and
    // loads; every store has completed (vmcnt 0) before the workgroup's
    // arrival is counted, so no cache-wide write-back or invalidate is needed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&ws.arrive[(b * ly.Hkv + h) * kArriveStride], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    // The appended token is published by the last wave once its share of
    // the merge is done, before the barrier.  Its tier is requested with the
    // partials, so publishing waits for no memory of its own.
    constexpr int kPubWave = kWaves - 1;
    const int app_tier_v = appending && wave == kPubWave ? ap.tier[b * ly.Hkv + h] : 0;
    // Each thread owns 4 adjacent outputs of one head and an interleaved
    // subset of the splits (part, part + parts, ...).  The partial vectors,
    // maxima and normalisers of its first splits are requested together, so
    // the merge waits for memory once up to 32 splits; the thread combines
    // its splits against their own largest max, and the parts are combined
    // through LDS after one barrier (fixed orders: bitwise reproducible).
    constexpr int quads = GQ * D / 4;
    constexpr int parts = kBlock / quads;
    constexpr int kFirst = 32 / parts > 8 ? 32 / parts : 8;
    static_assert(kBlock % quads == 0, "merge layout");
    static_assert(kBlock * (16 + 8) <= sizeof(s_ev), "merge scratch");
    const int qd = tid % quads, part = tid / quads;
    const int hq = (4 * qd) / D, j4 = (4 * qd) % D;
    const float *pob = ws.po + ((int64_t)b * ly.Hq + g0 + hq) * S * D + j4;
    const float *pmb = ws.pm + ((int64_t)b * ly.Hkv + h) * S * kMlStride + hq;
    float4_t pc[kFirst];
    float mc[kFirst], lc[kFirst];
#pragma unroll
    for (int c = 0; c < kFirst; ++c) {
        // (sp is the same in every lane of a wave: splits past S cost no load)
        const int sp = part + c * parts;
        pc[c] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        mc[c] = -INFINITY;
        lc[c] = 0.0f;
        if (sp < S) {
            pc[c] = ld_agent4(pob + (int64_t)sp * D);
            mc[c] = __hip_atomic_load(pmb + (int64_t)sp * kMlStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            lc[c] = __hip_atomic_load(pmb + (int64_t)sp * kMlStride + kMlNorm, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    float Mp = -INFINITY;
#pragma unroll
    for (int c = 0; c < kFirst; ++c) Mp = fmaxf(Mp, mc[c]);
    float Lp = 0.0f;
    float4_t accm = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < kFirst; ++c) {
        const float wgt = mc[c] == -INFINITY ? 0.0f : fast_exp2(mc[c] - Mp);
        accm += wgt * pc[c];
        Lp += wgt * lc[c];
    }
    // splits past the first batch (more than 32 splits): one at a time
    for (int sp = part + kFirst * parts; sp < S; sp += parts) {
        const float4_t o = ld_agent4(pob + (int64_t)sp * D);
        const float m = __hip_atomic_load(pmb + (int64_t)sp * kMlStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float l = __hip_atomic_load(pmb + (int64_t)sp * kMlStride + kMlNorm, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        const float nm = fmaxf(Mp, m);
        const float fa = Mp == -INFINITY ? 0.0f : fast_exp2(Mp - nm);
        const float fb = m == -INFINITY ? 0.0f : fast_exp2(m - nm);
        accm = fa * accm + fb * o;
        Lp = fa * Lp + fb * l;
        Mp = nm;
    }
    if (appending && wave == kPubWave) publish_token(ly, arena, layer, b, h, app_tier_v, rg.cnt, lane);
    float4_t *s_red = reinterpret_cast<float4_t *>(s_ev);                      // [parts][quads]
    float *s_mp = reinterpret_cast<float *>(s_red + kBlock);                    // [parts][quads] max, then normaliser
    s_red[tid] = accm;
    s_mp[tid] = Mp;
    s_mp[kBlock + tid] = Lp;
    __syncthreads();
    if (tid < quads) {
        float M = -INFINITY;
#pragma unroll
        for (int p2 = 0; p2 < parts; ++p2) M = fmaxf(M, s_mp[p2 * quads + tid]);
        float4_t o = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        float L = 0.0f;
#pragma unroll
        for (int p2 = 0; p2 < parts; ++p2) {
            const float mp = s_mp[p2 * quads + tid];
            const float wgt = mp == -INFINITY ? 0.0f : fast_exp2(mp - M);
            o += wgt * s_red[p2 * quads + tid];
            L += wgt * s_mp[kBlock + p2 * quads + tid];
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        *reinterpret_cast<float4_t *>(out + ((int64_t)b * ly.Hq + g0 + hq) * D + j4) = o * inv;
    }
    if (tid == 0) __hip_atomic_store(&ws.arrive[(b * ly.Hkv + h) * kArriveStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

}  // namespace dwkv
