// Bulk load of a layer from its logical (position-ordered) form into the
// tier-grouped arena, and the inverse read-back.  Not on the decode hot
// path: they stand in for the prefill that builds the cache, and let tests
// read appended tokens back.
#include <hip/hip_runtime.h>

#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace dwkv {

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

// One workgroup per KV head of sequence b.  Tokens are visited in position
// order, 256 at a time; each tier's slots are handed out in that order, so a
// tier region keeps its tokens sorted by position.
__global__ __launch_bounds__(kBlock) void import_kernel(Layout ly, uint8_t *arena, int layer,
                                                        dwkv_logical_layer src, int b, int64_t n)
{
    const int h = blockIdx.x;
    const int tid = threadIdx.x, wave = tid / kWave;
    __shared__ int s_base[kMaxTiers];
    __shared__ int s_cnt[kWaves][kMaxTiers];
    if (tid < kMaxTiers) s_base[tid] = 0;
    uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);
    int32_t *pmap = posmap_ptr(ly, arena, layer, b, h);
    uint32_t *err = err_ptr(ly, arena);
    const int64_t row0 = ((int64_t)b * ly.Hkv + h) * src.n_max;
    const uint8_t *tier_in = static_cast<const uint8_t *>(src.tier) + row0;
    __syncthreads();

    for (int64_t c0 = 0; c0 < n; c0 += kBlock) {
        const int64_t t = c0 + tid;
        bool valid = t < n;
        int k = valid ? tier_in[t] : 0;
        if (valid && k >= ly.T) {
            atomicOr(err, DWKV_DEVERR_BAD_TIER);
            valid = false;
        }
        int rank_in_wave = 0;
        for (int kk = 0; kk < ly.T; ++kk) {
            uint64_t m = __ballot(valid && k == kk);
            if (valid && k == kk) rank_in_wave = __popcll(m & lanemask_lt());
            if (lane_id() == 0) s_cnt[wave][kk] = __popcll(m);
        }
        __syncthreads();
        if (valid) {
            int slot = s_base[k] + rank_in_wave;
            for (int w = 0; w < wave; ++w) slot += s_cnt[w][k];
            if (slot >= ly.cap[k]) {
                atomicOr(err, DWKV_DEVERR_TIER_FULL);
            } else {
                const int r = ly.rank[k], s = ly.resid[k], vb = ly.vbytes[k];
                const int is = ly.istride[k], vs = ly.vstride[k];
                const int64_t tr = row0 + t;
                if (ly.cb == 2) {
                    const uint16_t *ck = static_cast<const uint16_t *>(src.coefK) + tr * ly.R;
                    const uint16_t *cv = static_cast<const uint16_t *>(src.coefV) + tr * ly.R;
                    uint16_t *dk = reinterpret_cast<uint16_t *>(blk + ly.f_coefK[k]) + (int64_t)slot * r;
                    uint16_t *dv = reinterpret_cast<uint16_t *>(blk + ly.f_coefV[k]);
                    for (int i = 0; i < r; ++i) {
                        dk[i] = ck[i];
                        dv[coefV_index(r, slot, i)] = cv[i];
                    }
                } else {
                    const int8_t *ck = static_cast<const int8_t *>(src.coefK) + tr * ly.R;
                    const int8_t *cv = static_cast<const int8_t *>(src.coefV) + tr * ly.R;
                    int8_t *dk = reinterpret_cast<int8_t *>(blk + ly.f_coefK[k]) + (int64_t)slot * r;
                    int8_t *dv = reinterpret_cast<int8_t *>(blk + ly.f_coefV[k]);
                    for (int i = 0; i < r; ++i) {
                        dk[i] = ck[i];
                        dv[coefV_index(r, slot, i)] = cv[i];
                    }
                    reinterpret_cast<uint16_t *>(blk + ly.f_cscK[k])[slot] = static_cast<const uint16_t *>(src.cscaleK)[tr];
                    reinterpret_cast<uint16_t *>(blk + ly.f_cscV[k])[slot] = static_cast<const uint16_t *>(src.cscaleV)[tr];
                }
                if (s > 0) {
                    for (int z = 0; z < 2; ++z) {
                        const uint8_t *ix = static_cast<const uint8_t *>(z ? src.idxV : src.idxK) +
                                            tr * ly.s_max;
                        const int8_t *vx = static_cast<const int8_t *>(z ? src.valV : src.valK) +
                                           tr * ly.s_max;
                        const uint16_t *sx = static_cast<const uint16_t *>(z ? src.scaleV : src.scaleK);
                        uint8_t *di = blk + (z ? ly.f_idxV[k] : ly.f_idxK[k]) + (int64_t)slot * is;
                        uint8_t *dvl = blk + (z ? ly.f_valV[k] : ly.f_valK[k]) + (int64_t)slot * vs;
                        uint16_t *ds = reinterpret_cast<uint16_t *>(blk + (z ? ly.f_scaleV[k] : ly.f_scaleK[k]));
                        for (int u = 0; u < s; ++u) {
                            int j = ix[u];
                            if (j >= ly.d) {   // decode trusts indices < head_dim
                                atomicOr(err, DWKV_DEVERR_BAD_INDEX);
                                j = ly.d - 1;
                            }
                            di[u] = static_cast<uint8_t>(j);
                        }
                        if (ly.bits == 8) {
                            for (int u = 0; u < s; ++u) dvl[u] = static_cast<uint8_t>(vx[u]);
                        } else {
                            for (int u = 0; u < vb; ++u) {
                                int lo = vx[2 * u] & 0xF;
                                int hi = (2 * u + 1 < s) ? (vx[2 * u + 1] & 0xF) : 0;
                                dvl[u] = static_cast<uint8_t>(lo | (hi << 4));
                            }
                        }
                        ds[slot] = sx[tr];
                    }
                }
                pmap[t] = (k << 28) | slot;
            }
        }
        __syncthreads();
        if (tid < ly.T) {
            int add = 0;
            for (int w = 0; w < kWaves; ++w) add += s_cnt[w][tid];
            s_base[tid] += add;
        }
        __syncthreads();
    }
    if (tid < ly.T) {
        int64_t c = s_base[tid];
        counts_ptr(ly, arena, layer, b, h)[tid] = (int32_t)(c < ly.cap[tid] ? c : ly.cap[tid]);
    }
}

// One workgroup per (sequence, KV head): every position of the layer written
// back in logical form through the position map.
__global__ __launch_bounds__(kBlock) void export_kernel(Layout ly, uint8_t *arena, int layer,
                                                        dwkv_logical_layer dst, int32_t *counts,
                                                        int32_t *slots)
{
    const int b = blockIdx.x / ly.Hkv, h = blockIdx.x % ly.Hkv;
    const int tid = threadIdx.x;
    uint8_t *blk = head_block_ptr(ly, arena, layer, b, h);
    const int32_t *pmap = posmap_ptr(ly, arena, layer, b, h);
    const int32_t *cnt = counts_ptr(ly, arena, layer, b, h);
    int64_t n = 0;
    for (int k = 0; k < ly.T; ++k) n += cnt[k];
    if (tid < ly.T) counts[((int64_t)b * ly.Hkv + h) * ly.T + tid] = cnt[tid];
    if (n > dst.n_max) n = dst.n_max;
    const int64_t row0 = ((int64_t)b * ly.Hkv + h) * dst.n_max;
    for (int64_t t = tid; t < n; t += kBlock) {
        const int pm = pmap[t];
        const int k = pm >> 28, slot = pm & 0x0FFFFFFF;
        const int r = ly.rank[k], s = ly.resid[k];
        const int is = ly.istride[k], vs = ly.vstride[k];
        const int64_t tr = row0 + t;
        static_cast<uint8_t *>(dst.tier)[tr] = static_cast<uint8_t>(k);
        if (slots) slots[tr] = slot;
        if (ly.cb == 2) {
            const uint16_t *sk = reinterpret_cast<const uint16_t *>(blk + ly.f_coefK[k]) + (int64_t)slot * r;
            const uint16_t *sv = reinterpret_cast<const uint16_t *>(blk + ly.f_coefV[k]);
            uint16_t *ck = static_cast<uint16_t *>(dst.coefK) + tr * ly.R;
            uint16_t *cv = static_cast<uint16_t *>(dst.coefV) + tr * ly.R;
            for (int i = 0; i < ly.R; ++i) {
                ck[i] = i < r ? sk[i] : 0;
                cv[i] = i < r ? sv[coefV_index(r, slot, i)] : 0;
            }
        } else {
            const int8_t *sk = reinterpret_cast<const int8_t *>(blk + ly.f_coefK[k]) + (int64_t)slot * r;
            const int8_t *sv = reinterpret_cast<const int8_t *>(blk + ly.f_coefV[k]);
            int8_t *ck = static_cast<int8_t *>(dst.coefK) + tr * ly.R;
            int8_t *cv = static_cast<int8_t *>(dst.coefV) + tr * ly.R;
            for (int i = 0; i < ly.R; ++i) {
                ck[i] = i < r ? sk[i] : 0;
                cv[i] = i < r ? sv[coefV_index(r, slot, i)] : 0;
            }
            static_cast<uint16_t *>(dst.cscaleK)[tr] = reinterpret_cast<const uint16_t *>(blk + ly.f_cscK[k])[slot];
            static_cast<uint16_t *>(dst.cscaleV)[tr] = reinterpret_cast<const uint16_t *>(blk + ly.f_cscV[k])[slot];
        }
        if (ly.s_max == 0) continue;
        for (int z = 0; z < 2; ++z) {
            uint8_t *ix = static_cast<uint8_t *>(z ? dst.idxV : dst.idxK) + tr * ly.s_max;
            int8_t *vx = static_cast<int8_t *>(z ? dst.valV : dst.valK) + tr * ly.s_max;
            uint16_t *sx = static_cast<uint16_t *>(z ? dst.scaleV : dst.scaleK);
            const uint8_t *si = blk + (z ? ly.f_idxV[k] : ly.f_idxK[k]) + (int64_t)slot * is;
            const uint8_t *svl = blk + (z ? ly.f_valV[k] : ly.f_valK[k]) + (int64_t)slot * vs;
            for (int u = 0; u < ly.s_max; ++u) {
                ix[u] = u < s ? si[u] : 0;
                vx[u] = u < s ? static_cast<int8_t>(unpack_code(svl, u, ly.bits)) : 0;
            }
            sx[tr] = s > 0 ? reinterpret_cast<const uint16_t *>(blk + (z ? ly.f_scaleV[k] : ly.f_scaleK[k]))[slot] : 0;
        }
    }
}

__global__ void fill_u32_kernel(uint32_t *p, uint32_t value, int64_t count)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

}  // namespace

hipError_t launch_import(const Layout &ly, uint8_t *arena, int layer,
                         const dwkv_logical_layer &src, int b, int64_t n, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    hipLaunchKernelGGL(import_kernel, dim3(ly.Hkv), dim3(kBlock), 0, stream, ly, arena, layer, src,
                       b, n);
    return hipGetLastError();
}

hipError_t launch_export(const Layout &ly, uint8_t *arena, int layer,
                         const dwkv_logical_layer &dst, int32_t *counts, int32_t *slots,
                         int batch, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    hipLaunchKernelGGL(export_kernel, dim3(batch * ly.Hkv), dim3(kBlock), 0, stream, ly, arena,
                       layer, dst, counts, slots);
    return hipGetLastError();
}

namespace {

// One thread per element of the window's V bases: dst[h][j][i] = src[h][i][j].
__global__ void transpose_basis_kernel(Layout ly, uint8_t *arena, int m)
{
    const int64_t n = ly.basis_elems;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const int h = (int)(e / ((int64_t)ly.R * ly.d));
        const int64_t rem = e - (int64_t)h * ly.R * ly.d;
        const int j = (int)(rem / ly.R), i = (int)(rem % ly.R);
        basis_vt_ptr(ly, arena, m, h)[(int64_t)j * ly.R + i] = basis_ptr(ly, arena, m, 1, h)[(int64_t)i * ly.d + j];
        basis_kt_ptr(ly, arena, m, h)[(int64_t)j * ly.R + i] = basis_ptr(ly, arena, m, 0, h)[(int64_t)i * ly.d + j];
    }
}

}  // namespace

hipError_t launch_transpose_basis(const Layout &ly, uint8_t *arena, int m, hipStream_t stream)
{
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    const int64_t blocks = (ly.basis_elems + 255) / 256;
    hipLaunchKernelGGL(transpose_basis_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream,
                       ly, arena, m);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, uint32_t value, int64_t count, hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, value,
                       count);
    return hipGetLastError();
}

}  // namespace dwkv
