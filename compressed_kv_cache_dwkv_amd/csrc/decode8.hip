// Decode attention over the compressed cache with coefficients in the
// paper's 8-bit blockwise form (§3, second paragraph): the instances of the
// kernel in decode_impl.h for int8 codes with per-token block scales (bases
// of at most 64 vectors).  Built in a translation unit of its own, with the
// compiler's default instruction scheduler.
#include "decode_impl.h"

namespace dwkv {

namespace {

template <int GQ, int D>
hipError_t launch8_gq(const Layout &ly, uint8_t *arena, int layer, const uint16_t *q, int batch, float qs,
                      float *out, const DecodeWorkspace &ws, int splits, const AppendArgs &ap, hipStream_t stream)
{
    const dim3 grid(splits, ly.Hkv, batch);
    const double inv = 1.0 / splits;
    if (ly.bits == 4)
        hipLaunchKernelGGL((decode_kernel<GQ, 4, D, 4, 1>), grid, dim3(kBlock), 0, stream, ly, arena, layer, q, out,
                           ws, splits, inv, qs, ap);
    else
        hipLaunchKernelGGL((decode_kernel<GQ, 4, D, 8, 1>), grid, dim3(kBlock), 0, stream, ly, arena, layer, q, out,
                           ws, splits, inv, qs, ap);
    return hipGetLastError();
}

template <int D>
hipError_t launch8_d(const Layout &ly, uint8_t *arena, int layer, const uint16_t *q, int batch, float qs, float *out,
                     const DecodeWorkspace &ws, int splits, const AppendArgs &ap, hipStream_t stream)
{
    switch (ly.gq) {
    case 1: return launch8_gq<1, D>(ly, arena, layer, q, batch, qs, out, ws, splits, ap, stream);
    case 2: return launch8_gq<2, D>(ly, arena, layer, q, batch, qs, out, ws, splits, ap, stream);
    case 4: return launch8_gq<4, D>(ly, arena, layer, q, batch, qs, out, ws, splits, ap, stream);
    case 8: return launch8_gq<8, D>(ly, arena, layer, q, batch, qs, out, ws, splits, ap, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode8(const Layout &ly, uint8_t *arena, int layer, const uint16_t *q, int batch, float qscale,
                          float *out, const DecodeWorkspace &ws, int splits, const AppendArgs &ap, hipStream_t stream)
{
    if (ly.R > 64) return hipErrorInvalidValue;
    if (ly.d == 64) return launch8_d<64>(ly, arena, layer, q, batch, qscale, out, ws, splits, ap, stream);
    if (ly.d == 128) return launch8_d<128>(ly, arena, layer, q, batch, qscale, out, ws, splits, ap, stream);
    return hipErrorInvalidValue;
}

}  // namespace dwkv
