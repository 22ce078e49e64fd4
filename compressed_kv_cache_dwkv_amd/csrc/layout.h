// Arena layout of a DepthWeave-KV compressed cache on the GPU.
//
// Decode attention is a sum over all cached tokens with no positional mask
// (every cached token precedes the decoding query), so tokens need not be
// stored in position order.  The arena keeps them grouped by rank tier: for
// every (layer, sequence, KV head) a contiguous block, and inside it one
// region per tier whose tokens all have the same coefficient rank r_k and the
// same residual channel count s_k.  A tier region is a structure of arrays,
// each array 16-byte aligned and unpadded per token:
//
//   coefK [cap][r_k] fp16                             (token-major rows)
//   coefV [cap/16][r_k][16] fp16                      (16-token blocks, channel-
//                                                      major inside a block)
//   idxK  [cap][is_k] u8    idxV  [cap][is_k] u8      (ascending channels)
//   valK  [cap][vs_k] u8    valV  [cap][vs_k] u8      (codes; 4-bit codes two
//                                                      per byte, element 2u in
//                                                      the low nibble of byte u)
//   scaleK [cap] fp16       scaleV [cap] fp16         (absent when s_k == 0)
//   cscaleK [cap] fp16      cscaleV [cap] fp16        (8-bit coefficients only:
//                                                      each token's block scale)
//
// With 8-bit blockwise coefficients coefK and coefV hold int8 codes in the
// same arrangement (one byte per coefficient).
// where is_k and vs_k are the s_k index bytes and s_k * bits / 8 code bytes
// of a token rounded up to whole 4-byte words (no rounding for the usual
// s_k = 4 or 8 with 8-bit, s_k = 8 with 4-bit codes), so a run of tokens of
// one tier is a few contiguous streams and every byte a decode step reads is
// a byte the method needs.  K coefficients are rows of
// a token x channel matrix and V coefficients columns of 16 tokens: both
// then load directly as operands of 16x16x16 matrix-core products (scores
// contract over channels, value sums over tokens).  Capacities are rounded
// up to whole 16-token blocks.  Besides the blocks the arena
// holds the sticky error word, token counts per (layer, sequence, KV head,
// tier), a position map per (layer, sequence, KV head) giving each position's
// (tier << 28 | slot), and the shared bases per (depth window, Z, KV head)
// as r_max rows of head_dim fp16 values.
#pragma once

#include <stdint.h>

#include "dwkv.h"

#if defined(__HIPCC__)
#define DWKV_HD __host__ __device__ __forceinline__
#else
#define DWKV_HD inline
#endif

namespace dwkv {

constexpr int kMaxTiers = DWKV_MAX_TIERS;
constexpr int kMaxHeadDim = 128;
constexpr int kMaxRank = 128;
constexpr int kMaxResid = 8;
constexpr int kMaxGroupQ = 8;
constexpr int kMaxSplits = 256;   // decode workgroups per (sequence, KV head)

// One tier as the decode kernel sees it: array offsets in bytes from the
// start of a (layer, sequence, KV head) block, and the tier's shape.
struct TierDesc {
    int32_t coefK, coefV, idxK, idxV, valK, valV, scaleK, scaleV;
    int32_t rank, resid, istride, vstride, weight, cscK, cscV, pad2;
    // A decode tile's operand slot i (16-token block i >> log2(kb), 16-channel
    // block i & (kb - 1), kb the rank's 16-channel blocks): its byte offset
    // from the tile's first K (koff) and V (voff) coefficient, for the
    // layout's coefficient width.
    int32_t koff[8], voff[8];
    // Masks keeping the first `resid` entries of a token's residual record
    // words: index bytes (im0, im1) and packed codes (cm0, cm1).
    uint32_t im0, im1, cm0, cm1;
};

struct Layout {
    int32_t L, G, Hq, Hkv, d, R, T, bits, Bmax, gq, s_max, qmax, num_groups;
    int32_t cb;                  // bytes per stored coefficient: 2 (fp16) or 1 (8-bit codes)
    int32_t rank[kMaxTiers];
    int32_t resid[kMaxTiers];
    int32_t vbytes[kMaxTiers];   // packed code bytes per token
    int32_t istride[kMaxTiers];  // stored index bytes per token (s rounded up to 4)
    int32_t vstride[kMaxTiers];  // stored code bytes per token (vbytes rounded up to 4)
    int32_t weight[kMaxTiers];   // algorithmic bytes per token (K and V)
    int32_t cost[kMaxTiers];     // decode work per token, the unit splits are balanced on
    double inv_cblk[kMaxTiers];  // 1 / (16 * cost): reciprocal of a 16-token block's cost
    int64_t cap[kMaxTiers];
    int64_t max_tokens;
    int64_t off_err, off_counts, off_posmap, off_basis, off_basisvt, off_basiskt, off_seg;
    int64_t basis_elems;         // Hkv * R * d  (one Z of one window)
    int64_t head_block;          // bytes of one (layer, b, h) block
    int64_t f_coefK[kMaxTiers], f_coefV[kMaxTiers];
    int64_t f_idxK[kMaxTiers], f_idxV[kMaxTiers];
    int64_t f_valK[kMaxTiers], f_valV[kMaxTiers];
    int64_t f_scaleK[kMaxTiers], f_scaleV[kMaxTiers];
    int64_t f_cscK[kMaxTiers], f_cscV[kMaxTiers];
    int64_t total;
    TierDesc tier[kMaxTiers];    // the same tiers, packed per tier (head blocks < 2 GiB)
};

// Kernels take the layout by value, beside a few hundred bytes of other
// arguments, within the 4 KiB a launch's arguments may occupy.
static_assert(sizeof(Layout) <= 3072, "layout too large for a kernel argument");

DWKV_HD int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

DWKV_HD uint8_t *head_block_ptr(const Layout &ly, uint8_t *arena, int layer, int b, int h)
{
    return arena + ly.off_seg + (((int64_t)layer * ly.Bmax + b) * ly.Hkv + h) * ly.head_block;
}

DWKV_HD int32_t *counts_ptr(const Layout &ly, uint8_t *arena, int layer, int b, int h)
{
    return reinterpret_cast<int32_t *>(arena + ly.off_counts) +
           (((int64_t)layer * ly.Bmax + b) * ly.Hkv + h) * ly.T;
}

DWKV_HD int32_t *posmap_ptr(const Layout &ly, uint8_t *arena, int layer, int b, int h)
{
    return reinterpret_cast<int32_t *>(arena + ly.off_posmap) +
           (((int64_t)layer * ly.Bmax + b) * ly.Hkv + h) * ly.max_tokens;
}

DWKV_HD uint32_t *err_ptr(const Layout &ly, uint8_t *arena)
{
    return reinterpret_cast<uint32_t *>(arena + ly.off_err);
}

// Basis of window m for Z (0 = K, 1 = V), KV head h: R rows of d fp16.
DWKV_HD uint16_t *basis_ptr(const Layout &ly, uint8_t *arena, int m, int z, int h)
{
    return reinterpret_cast<uint16_t *>(arena + ly.off_basis) +
           ((int64_t)m * 2 + z) * ly.basis_elems + (int64_t)h * ly.R * ly.d;
}

// Transposed V basis of window m, KV head h: d rows of R fp16 (row j holds
// component j of every basis vector), the operand layout of the decode's
// back-projection.
DWKV_HD uint16_t *basis_vt_ptr(const Layout &ly, uint8_t *arena, int m, int h)
{
    return reinterpret_cast<uint16_t *>(arena + ly.off_basisvt) + (int64_t)m * ly.basis_elems +
           (int64_t)h * ly.R * ly.d;
}

// Transposed K basis of window m, KV head h: d rows of R fp16 (the
// explicit reconstruction's matrix-core operand).
DWKV_HD uint16_t *basis_kt_ptr(const Layout &ly, uint8_t *arena, int m, int h)
{
    return reinterpret_cast<uint16_t *>(arena + ly.off_basiskt) + (int64_t)m * ly.basis_elems +
           (int64_t)h * ly.R * ly.d;
}

// Element (slot, i) of a tier's V coefficients, in fp16 units from the array
// start: 16-token blocks, each r channel rows of 16 tokens.
DWKV_HD int64_t coefV_index(int r, int64_t slot, int i)
{
    return ((slot >> 4) * r + i) * 16 + (slot & 15);
}

// Host-side construction and validation; returns DWKV_OK or an error code.
int build_layout(const dwkv_config *cfg, Layout *ly);

}  // namespace dwkv
