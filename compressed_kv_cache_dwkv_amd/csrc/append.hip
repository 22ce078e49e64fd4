// Append step as a kernel of its own: one workgroup per (sequence, KV head)
// runs the shared encoder (append_body.h; DepthWeave-KV paper, arXiv
// 2607.06523, §3 Method, second paragraph).  The file is built with
// -ffp-contract=off as well, so nothing outside the encoder's own fixed
// operation order is fused either.
#include <hip/hip_runtime.h>

#include "append_body.h"
#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

// One workgroup of two waves per (sequence, KV head): wave 0 encodes K,
// wave 1 encodes V; both write the same slot of the token's tier, and one
// thread publishes the token after both are done.
template <int D>
__global__ __launch_bounds__(2 * kWave) void append_kernel(Layout ly, uint8_t *arena, int layer,
                                                           AppendArgs ap)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_mem[kAppendLdsBytes];
    const int bh = blockIdx.x;
    const int b = bh / ly.Hkv, h = bh % ly.Hkv;
    const int tid = threadIdx.x, z = tid / kWave, lane = lane_id();
    AppendRegs<D> st;
    append_fetch<D>(st, ly, arena, layer, b, h, z, lane, ap);
    int slot, n;
    const int ok = append_encode<D>(st, ly, arena, layer, b, h, z, lane, ap, carve_append_lds(s_mem), slot, n);
    __syncthreads();
    if (tid == 0 && ok) append_commit(ly, arena, layer, b, h, st.k, slot, n);
}

}  // namespace

hipError_t launch_append(const Layout &ly, uint8_t *arena, int layer, const void *k,
                         const void *v, const void *tier, const void *gateK, const void *gateV,
                         int batch, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    const auto kern = ly.d == 64 ? append_kernel<64> : append_kernel<128>;
    const AppendArgs ap{static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                        static_cast<const uint8_t *>(tier), static_cast<const uint16_t *>(gateK),
                        static_cast<const uint16_t *>(gateV)};
    hipLaunchKernelGGL(kern, dim3(batch * ly.Hkv), dim3(2 * kWave), 0, stream, ly, arena, layer, ap);
    return hipGetLastError();
}

}  // namespace dwkv
