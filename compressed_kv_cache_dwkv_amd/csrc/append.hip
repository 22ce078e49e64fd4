// Append step: encodes the new token's K and V of every (sequence, KV head)
// into the compressed form and stores it in its tier (DepthWeave-KV paper,
// arXiv 2607.06523, §3 Method, second paragraph: coefficients by projection
// onto the current basis, residual kept on the router-chosen number of
// channels with low-bit group quantisation).
//
// The encoder makes integer decisions (kept channels, codes) from floating
// point values, so it follows one fixed IEEE fp32 operation order --
// sequential fused multiply-adds in ascending index order, correctly rounded
// division, round-to-nearest-even conversions -- and must be built with
// -ffp-contract=off so no other multiply-add is fused.
#include <hip/hip_runtime.h>

#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

// One workgroup of two waves per (sequence, KV head): wave 0 encodes K,
// wave 1 encodes V; both write the same slot of the token's tier.
__global__ __launch_bounds__(2 * kWave) void append_kernel(Layout ly, uint8_t *arena, int layer,
                                                           const uint16_t *kin, const uint16_t *vin,
                                                           const uint8_t *tier_in,
                                                           const uint16_t *gateK,
                                                           const uint16_t *gateV)
{
    const int bh = blockIdx.x;
    const int b = bh / ly.Hkv, h = bh % ly.Hkv;
    const int tid = threadIdx.x, z = tid / kWave, lane = lane_id();
    const int d = ly.d;

    __shared__ int s_ok, s_k, s_slot, s_n;
    __shared__ float s_x[2][kMaxHeadDim];
    __shared__ float s_c[2][kMaxRank];
    __shared__ float s_e[2][kMaxHeadDim];
    __shared__ float s_amax[2];
    __shared__ int8_t s_code[2][kMaxResid];
    __shared__ uint8_t s_idx[2][kMaxResid];

    int32_t *cnt = counts_ptr(ly, arena, layer, b, h);
    if (tid == 0) {
        uint32_t *err = err_ptr(ly, arena);
        int k = tier_in[bh];
        int ok = 1;
        int slot = 0;
        int64_t n = 0;
        if (k >= ly.T) {
            atomicOr(err, DWKV_DEVERR_BAD_TIER);
            ok = 0;
        } else {
            for (int kk = 0; kk < ly.T; ++kk) n += cnt[kk];
            slot = cnt[k];
            if (slot >= ly.cap[k]) {
                atomicOr(err, DWKV_DEVERR_TIER_FULL);
                ok = 0;
            }
            if (n >= ly.max_tokens) {
                atomicOr(err, DWKV_DEVERR_POS_FULL);
                ok = 0;
            }
        }
        s_ok = ok;
        s_k = k;
        s_slot = slot;
        s_n = (int)n;
    }
    __syncthreads();
    if (!s_ok) return;  // uniform across the workgroup
    const int k = s_k, slot = s_slot;
    const int r = ly.rank[k], s = ly.resid[k];
    uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);
    const uint16_t *B = basis_ptr(ly, arena, layer / ly.G, z, h);   // [R][d]
    const uint16_t *x = (z ? vin : kin) + (int64_t)bh * d;

    for (int j = lane; j < d; j += kWave) s_x[z][j] = h2f(x[j]);
    __syncthreads();

    // 1. coefficients c_i = fp16(sum_j B[i][j] x_j), sequential in j
    uint16_t *cdst = reinterpret_cast<uint16_t *>(blk + (z ? ly.f_coefV[k] : ly.f_coefK[k]));
    for (int i = lane; i < r; i += kWave) {
        const uint16_t *bi = B + (int64_t)i * d;
        float acc = 0.0f;
        for (int j = 0; j < d; ++j) acc = __builtin_fmaf(h2f(bi[j]), s_x[z][j], acc);
        const uint16_t c16 = f2h(acc);
        cdst[z ? coefV_index(r, slot, i) : (int64_t)slot * r + i] = c16;
        s_c[z][i] = h2f(c16);
    }
    __syncthreads();

    // 2. residual against the rounded coefficients, sequential in i
    for (int j = lane; j < d; j += kWave) {
        float acc = 0.0f;
        for (int i = 0; i < r; ++i) acc = __builtin_fmaf(h2f(B[(int64_t)i * d + j]), s_c[z][i], acc);
        s_e[z][j] = s_x[z][j] - acc;
    }
    __syncthreads();

    if (s > 0) {
        // 3. channel j is kept when fewer than s channels precede it in the
        //    order (larger |e| first, then smaller index)
        bool keep[2] = {false, false};
        for (int q = 0; q < 2; ++q) {
            const int j = lane + q * kWave;
            if (j >= d) continue;
            const float a = fabsf(s_e[z][j]);
            int before = 0;
            for (int jj = 0; jj < d; ++jj) {
                const float b2 = fabsf(s_e[z][jj]);
                before += (b2 > a) || (b2 == a && jj < j);
            }
            keep[q] = before < s;
            if (before == 0) s_amax[z] = a;
        }
        const uint64_t m0 = __ballot(keep[0]);
        const uint64_t m1 = __ballot(keep[1]);
        __syncthreads();
        // 4. one fp16 scale per token: max kept |e| / qmax, correctly rounded
        const uint16_t s16 = f2h(__fdiv_rn(s_amax[z], (float)ly.qmax));
        const float sf = h2f(s16);
        // 5. codes, placed in ascending channel order
        for (int q = 0; q < 2; ++q) {
            if (!keep[q]) continue;
            const int j = lane + q * kWave;
            const int pos = q == 0 ? __popcll(m0 & lanemask_lt())
                                   : __popcll(m0) + __popcll(m1 & lanemask_lt());
            float v = 0.0f;
            if (sf != 0.0f) {
                v = rintf(__fdiv_rn(s_e[z][j], sf));
                v = fminf(fmaxf(v, -(float)ly.qmax), (float)ly.qmax);
            }
            s_code[z][pos] = static_cast<int8_t>(v);
            s_idx[z][pos] = static_cast<uint8_t>(j);
        }
        __syncthreads();
        const int vb = ly.vbytes[k];
        uint8_t *idst = blk + (z ? ly.f_idxV[k] : ly.f_idxK[k]) + (int64_t)slot * ly.istride[k];
        uint8_t *vdst = blk + (z ? ly.f_valV[k] : ly.f_valK[k]) + (int64_t)slot * ly.vstride[k];
        if (lane < s) idst[lane] = s_idx[z][lane];
        if (ly.bits == 8) {
            if (lane < s) vdst[lane] = static_cast<uint8_t>(s_code[z][lane]);
        } else if (lane < vb) {
            const int lo = s_code[z][2 * lane] & 0xF;
            const int hi = (2 * lane + 1 < s) ? (s_code[z][2 * lane + 1] & 0xF) : 0;
            vdst[lane] = static_cast<uint8_t>(lo | (hi << 4));
        }
        // 6. the gate folds into the stored scale
        if (lane == 0) {
            const uint16_t *gp = z ? gateV : gateK;
            const uint16_t g = gp ? gp[bh] : uint16_t(0x3C00);
            const uint16_t stored = (g == 0x3C00) ? s16 : f2h(h2f(g) * sf);
            reinterpret_cast<uint16_t *>(blk + (z ? ly.f_scaleV[k] : ly.f_scaleK[k]))[slot] = stored;
        }
    }
    __syncthreads();
    if (tid == 0) {
        cnt[k] = slot + 1;
        posmap_ptr(ly, arena, layer, b, h)[s_n] = (k << 28) | slot;
    }
}

}  // namespace

hipError_t launch_append(const Layout &ly, uint8_t *arena, int layer, const void *k,
                         const void *v, const void *tier, const void *gateK, const void *gateV,
                         int batch, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    hipLaunchKernelGGL(append_kernel, dim3(batch * ly.Hkv), dim3(2 * kWave), 0, stream, ly, arena,
                       layer, static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                       static_cast<const uint8_t *>(tier), static_cast<const uint16_t *>(gateK),
                       static_cast<const uint16_t *>(gateV));
    return hipGetLastError();
}

}  // namespace dwkv
