// Decode attention over the compressed cache, fp16-coefficient instances
// and the dispatcher (the kernel is in decode_impl.h; the 8-bit coefficient
// instances are built in decode8.hip).
#include "decode_impl.h"

namespace dwkv {

namespace {

template <int GQ, int D>
hipError_t launch_gq(const Layout &ly, uint8_t *arena, int layer, const uint16_t *q, int batch,
                     float qs, float *out, const DecodeWorkspace &ws, int splits, const AppendArgs &ap,
                     hipStream_t stream)
{
    const dim3 grid(splits, ly.Hkv, batch);
    const double inv = 1.0 / splits;
    // (code widths 4 and 8, checked when the layout is built)
    if (ly.R <= 64 && ly.bits == 4)
        hipLaunchKernelGGL((decode_kernel<GQ, 4, D, 4, 2>), grid, dim3(kBlock), 0, stream, ly, arena, layer, q, out,
                           ws, splits, inv, qs, ap);
    else if (ly.R <= 64)
        hipLaunchKernelGGL((decode_kernel<GQ, 4, D, 8, 2>), grid, dim3(kBlock), 0, stream, ly, arena, layer, q, out,
                           ws, splits, inv, qs, ap);
    else if (ly.bits == 4)
        hipLaunchKernelGGL((decode_kernel<GQ, 8, D, 4, 2>), grid, dim3(kBlock), 0, stream, ly, arena, layer, q, out,
                           ws, splits, inv, qs, ap);
    else
        hipLaunchKernelGGL((decode_kernel<GQ, 8, D, 8, 2>), grid, dim3(kBlock), 0, stream, ly, arena, layer, q, out,
                           ws, splits, inv, qs, ap);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Layout &ly, uint8_t *arena, int layer, const uint16_t *q, int batch,
                    float qs, float *out, const DecodeWorkspace &ws, int splits, const AppendArgs &ap,
                    hipStream_t stream)
{
    switch (ly.gq) {
    case 1: return launch_gq<1, D>(ly, arena, layer, q, batch, qs, out, ws, splits, ap, stream);
    case 2: return launch_gq<2, D>(ly, arena, layer, q, batch, qs, out, ws, splits, ap, stream);
    case 4: return launch_gq<4, D>(ly, arena, layer, q, batch, qs, out, ws, splits, ap, stream);
    case 8: return launch_gq<8, D>(ly, arena, layer, q, batch, qs, out, ws, splits, ap, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// The append's encoding, done by the first workgroup of each (sequence, KV
// head) before its share of the tiles, in the units of the work balance
// (9216 per tile), from kernel-trace sweeps of the share on each workload
// shape: 250000 (about 27 tiles) with at most 4 query heads per KV head and
// many splits per head (the 64K workload); 30% less with 8 query heads per
// KV head, whose tiles take longer (the 128K 70B-shaped workload: 175000
// best); 40% more with at most 4 splits per head, where every encoder of the
// batch runs at once and each takes longer (the 32K x 16 workload: 350000
// best).
static float encode_units(const Layout &ly, int splits)
{
    float e = 250000.0f;
    if (ly.gq > 4) e *= 0.7f;
    if (splits <= 4) e *= 1.4f;
    return e;
}

hipError_t launch_decode(const Layout &ly, uint8_t *arena, int layer, const void *q, int batch,
                         float softmax_scale, float *out, const DecodeWorkspace &ws, int splits,
                         const AppendArgs *ap, hipStream_t stream)
{
    const float qs = softmax_scale * kLog2e;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const AppendArgs none{nullptr, nullptr, nullptr, nullptr, nullptr};
    AppendArgs a = ap ? *ap : none;
    if (ap) a.enc_units = encode_units(ly, splits);
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    if (ly.cb == 1) return launch_decode8(ly, arena, layer, qq, batch, qs, out, ws, splits, a, stream);
    if (ly.d == 64) return launch_d<64>(ly, arena, layer, qq, batch, qs, out, ws, splits, a, stream);
    if (ly.d == 128) return launch_d<128>(ly, arena, layer, qq, batch, qs, out, ws, splits, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace dwkv
