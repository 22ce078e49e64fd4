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

hipError_t launch_append(const Layout &ly, uint8_t *arena, int layer, const void *k,
                         const void *v, const void *tier, const void *gateK, const void *gateV,
                         int batch, hipStream_t stream);

// Loads sequence b (n tokens) of `layer` from its logical form.
hipError_t launch_import(const Layout &ly, uint8_t *arena, int layer,
                         const dwkv_logical_layer &src, int b, int64_t n, hipStream_t stream);

hipError_t launch_export(const Layout &ly, uint8_t *arena, int layer,
                         const dwkv_logical_layer &dst, int32_t *counts, int32_t *slots,
                         int batch, hipStream_t stream);

// Writes the transposed V basis of window m (basis_vt_ptr) from the arena's copy.
hipError_t launch_transpose_basis(const Layout &ly, uint8_t *arena, int m, hipStream_t stream);

hipError_t launch_fill_u32(uint32_t *p, uint32_t value, int64_t count, hipStream_t stream);

}  // namespace dwkv
