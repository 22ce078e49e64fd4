// Launchers of the HIP kernels (one translation unit per kernel family).
// Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>

#include "layout.h"

namespace dwkv {

// Decode workspace carve-up for `batch` sequences and `splits` workgroups per
// (sequence, KV head): arrival counters, then per (b, query head, split) the
// running max, the normaliser and the unnormalised output vector.  Each
// (sequence, KV head) counter, and the maxima and normalisers of each
// (sequence, KV head, split), have a 128-byte line of their own, so the
// stores and atomics of different workgroups do not queue on one line.
constexpr int kArriveStride = 32;   // uint32 per arrival counter
constexpr int kMlStride = 32;       // floats per split's maxima and normalisers
constexpr int kMlNorm = 16;         // offset of the normalisers in that line
struct DecodeWorkspace {
    uint32_t *arrive;   // [B][Hkv][kArriveStride], element 0 used
    float *pm;          // [B][Hkv][S][kMlStride], query head g of the group at g
    float *pl;          // pm + kMlNorm (same lines)
    float *po;          // [B][Hq][S][d]
};

// Inputs of one append call (device pointers).
struct AppendArgs {
    const uint16_t *k, *v;          // fp16 [B][Hkv][d]
    const uint8_t *tier;            // [B][Hkv], the router's rank tier
    const uint16_t *gateK, *gateV;  // fp16 [B][Hkv], or null for a gate of 1
    // one-launch decode step only: how much less of the tile work the
    // encoding workgroup of each (sequence, KV head) takes, in the units the
    // splits are balanced on (set by launch_decode)
    float enc_units = 0.0f;
};

size_t decode_workspace_bytes(const Layout &ly, int batch, int splits);
DecodeWorkspace carve_workspace(const Layout &ly, void *ws, int batch, int splits);

// Decode attention of one layer; with `ap` non-null the same launch also
// appends the new tokens: the first workgroup of each (sequence, KV head)
// encodes them into their slots, the last publishes them once every
// workgroup of that head has read the token counts.
hipError_t launch_decode(const Layout &ly, uint8_t *arena, int layer, const void *q, int batch,
                         float softmax_scale, float *out, const DecodeWorkspace &ws, int splits,
                         const AppendArgs *ap, hipStream_t stream);

// Dense fp16 decode (the uncompressed comparator): q fp16 [B][Hq][d]; k fp16
// [B][Hkv][n_cap][d] token rows; v fp16 [B][Hkv][n_cap/16][d][16]; n int32
// [B][Hkv] tokens per (sequence, KV head); out fp32 [B][Hq][d].
struct DenseArgs {
    const uint16_t *q, *k, *v;
    const int32_t *n;
    float *out;
    DecodeWorkspace ws;
    int B, Hq, Hkv, d;
    int64_t n_cap;
    float scale;
};
hipError_t launch_dense_decode(const DenseArgs &a, int splits, hipStream_t stream);

// A plain streaming read of `bytes` (a multiple of 16) with the given grid;
// a measurement aid.
hipError_t launch_stream_read(const void *src, int64_t bytes, int workgroups, int threads, uint32_t magic,
                              uint32_t *sink, hipStream_t stream);

// Writes the Eq. (1) reconstruction of every cached token of `layer` (batch
// sequences) into the dense layout above, in position order, and the tokens
// per (sequence, KV head) into n_out (int32 [batch][Hkv], may be null).
hipError_t launch_materialize(const Layout &ly, uint8_t *arena, int layer, int batch, uint16_t *kout,
                              uint16_t *vout, int64_t n_cap, int32_t *n_out, hipStream_t stream);

// Eq. (3) relative L2 error per (sequence, KV head) from the reference and
// compressed attention outputs o_ref, o_cmp (fp32 [nq][B][Hq][d]) into err
// (fp32 [B][Hkv]).
hipError_t launch_probe_error(const float *o_ref, const float *o_cmp, int nq, int B, int Hq, int Hkv, int d, float eps,
                              float *err, hipStream_t stream);

// The decode kernel's instances for 8-bit blockwise coefficients (ly.cb == 1);
// qscale is softmax_scale * log2(e).
hipError_t launch_decode8(const Layout &ly, uint8_t *arena, int layer, const uint16_t *q, int batch, float qscale,
                          float *out, const DecodeWorkspace &ws, int splits, const AppendArgs &ap,
                          hipStream_t stream);

hipError_t launch_append(const Layout &ly, uint8_t *arena, int layer, const void *k,
                         const void *v, const void *tier, const void *gateK, const void *gateV,
                         int batch, hipStream_t stream);

// Loads sequence b (n tokens) of `layer` from its logical form.
hipError_t launch_import(const Layout &ly, uint8_t *arena, int layer,
                         const dwkv_logical_layer &src, int b, int64_t n, hipStream_t stream);

hipError_t launch_export(const Layout &ly, uint8_t *arena, int layer,
                         const dwkv_logical_layer &dst, int32_t *counts, int32_t *slots,
                         int batch, hipStream_t stream);

// Writes the transposed bases of window m (basis_vt_ptr, basis_kt_ptr) from the arena's copies.
hipError_t launch_transpose_basis(const Layout &ly, uint8_t *arena, int m, hipStream_t stream);

// Prefill compression (prefill.hip).
constexpr int kGramMaxBatch = 1024;   // sequences per Gram call
constexpr int kGramMaxSplits = 128;   // workgroups per (Z, KV head) of a Gram call
constexpr int kMaxSketch = 72;        // sketch width k (LDS: two head_dim x k fp64 matrices)
constexpr int kJacobiMaxSweeps = 40;
constexpr int kSlotChunk = 1024;      // positions per chunk of the encoder's count and place passes
constexpr int kChunkStride = 16;      // ints per chunk record (tier counts, then the bad-tier flag)

// Number of 16x16 blocks on and above the diagonal of a head_dim^2 matrix.
constexpr int gram_pairs(int d) { return (d / 16) * (d / 16 + 1) / 2; }

struct GramArgs {
    const uint16_t *k, *v;        // fp16 [B][Hkv][n_cap][d]
    const int32_t *n_tokens;      // [B] prefill length per sequence
    int B, Hkv;
    int64_t n_cap;
    int S;                        // workgroups per (Z, KV head)
    int first;                    // 1: the window's sums start here
    float *part;                  // [2 Hkv][S][gram_pairs(d) * 256] partial sums
    double *acc;                  // the window's [2][Hkv][d][d] sums
};
hipError_t launch_gram(const Layout &ly, uint8_t *arena, const GramArgs &a, hipStream_t stream);

struct BasesArgs {
    const double *acc;            // [n_groups][2][Hkv][d][d] Gram sums of windows group0, ...
    const float *omega;           // [n_groups][2][Hkv][d][k] Gaussian sketches
    double *ritz;                 // [n_groups][2][Hkv][k] Ritz values in decreasing order, or null
    int k, power_iters, group0;
};
// Forms the bases of windows group0 .. group0 + n_groups - 1 and their
// transposed copies.
hipError_t launch_bases(const Layout &ly, uint8_t *arena, const BasesArgs &a, int n_groups, hipStream_t stream);

struct EncodeArgs {
    int layer;
    const uint16_t *k, *v;        // fp16 [B][Hkv][n_cap][d]
    const int32_t *n_tokens;      // [B]
    int64_t n_cap;
    const uint8_t *tier;          // [B][Hkv][n_cap]
    const uint16_t *gateK, *gateV;  // fp16 [B][Hkv][n_cap], or null
    int32_t *status;              // [B][Hkv] first position, or -1 if refused
    int32_t *cnt0, *tot;          // [B][Hkv][kMaxTiers] tier counts before the call, tokens added
    int32_t *inv;                 // [B][Hkv][max_tokens] the call's tokens listed by tier
    int32_t *cntc;                // [B][Hkv][n_chunks][kChunkStride] tier counts per chunk (+ a bad-tier flag)
    int n_chunks;                 // chunks of kSlotChunk positions the call's counts cover
    uint16_t *basis_blocks;       // the window's bases in blocks of 8 rows, fp16 [2][Hkv][kMaxRank / 8][d][8]
    bool copy_basis;              // (re)make basis_blocks from the arena first
};
hipError_t launch_prefill_encode(const Layout &ly, uint8_t *arena, const EncodeArgs &a, int batch,
                                 hipStream_t stream);

hipError_t launch_fill_u32(uint32_t *p, uint32_t value, int64_t count, hipStream_t stream);

}  // namespace dwkv
