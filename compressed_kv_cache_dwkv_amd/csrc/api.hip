// C ABI of libdwkv: argument validation, arena layout, launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>

#include "dwkv.h"
#include "kernels.h"
#include "layout.h"

struct dwkv_handle {
    dwkv_config cfg;
    dwkv::Layout ly;
    uint8_t *arena;
    int splits;
};

namespace dwkv {

// Decode work of a token, in the unit splits are balanced on.  The decode
// kernel cuts each tier into tiles of about 2 KiB of coefficients per K and
// V (64 tokens at rank <= 16, 32 at rank 32, 16 at rank 64; twice that when
// the basis is wider than 64).  Workgroup times on the 64K-token
// Llama-3-8B shape are set by their tile count alone (about 0.45 us of a
// compute unit per tile, whatever its rank and number of tokens): a token
// weighs its share of a tile.
static int token_cost(int r, int r_max)
{
    const int slots = r_max <= 64 ? 4 : 8;                 // 16x16 operand blocks per tile
    const int kbr = r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8;
    const int blocks = slots / kbr;                        // 16-token blocks, at most 4 (one token per lane)
    const int tokens_per_tile = 16 * (blocks < 4 ? blocks : 4);
    return 9216 / tokens_per_tile;
}
constexpr int64_t kArenaTail = 8192;

int build_layout(const dwkv_config *c, Layout *ly)
{
    if (!c || !ly) return DWKV_ERR_INVALID_ARG;
    std::memset(ly, 0, sizeof(*ly));
    if (c->num_layers <= 0 || c->layers_per_group <= 0 || c->num_q_heads <= 0 ||
        c->num_kv_heads <= 0 || c->head_dim <= 0 || c->r_max <= 0 || c->num_tiers <= 0 ||
        c->max_batch <= 0 || c->max_tokens < 0 || c->decode_splits < 0)
        return DWKV_ERR_INVALID_ARG;
    if (c->num_tiers > kMaxTiers) return DWKV_ERR_UNSUPPORTED;
    if (c->num_q_heads % c->num_kv_heads != 0) return DWKV_ERR_INVALID_ARG;
    const int gq = c->num_q_heads / c->num_kv_heads;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8) return DWKV_ERR_UNSUPPORTED;
    if (c->head_dim != 64 && c->head_dim != 128) return DWKV_ERR_UNSUPPORTED;
    if (c->r_max % 4 != 0 || c->r_max > kMaxRank) return DWKV_ERR_UNSUPPORTED;
    if (c->resid_bits != 4 && c->resid_bits != 8) return DWKV_ERR_UNSUPPORTED;
    if (c->max_tokens >= (int64_t(1) << 31)) return DWKV_ERR_UNSUPPORTED;
    if (c->decode_splits > kMaxSplits) return DWKV_ERR_UNSUPPORTED;
    int prev = 0, smax = 0;
    for (int k = 0; k < c->num_tiers; ++k) {
        int r = c->tier_rank[k], s = c->tier_resid[k];
        if (r <= 0 || r > c->r_max || r % 4 != 0) return DWKV_ERR_UNSUPPORTED;
        if (r <= prev) return DWKV_ERR_INVALID_ARG;  // ranks strictly ascending
        prev = r;
        if (s < 0 || s > kMaxResid || s > c->head_dim) return DWKV_ERR_UNSUPPORTED;
        if (c->tier_capacity[k] < 0 || c->tier_capacity[k] >= (int64_t(1) << 28))
            return DWKV_ERR_UNSUPPORTED;
        if (s > smax) smax = s;
    }
    ly->L = c->num_layers;
    ly->G = c->layers_per_group;
    ly->Hq = c->num_q_heads;
    ly->Hkv = c->num_kv_heads;
    ly->d = c->head_dim;
    ly->R = c->r_max;
    ly->T = c->num_tiers;
    ly->bits = c->resid_bits;
    ly->Bmax = c->max_batch;
    ly->gq = gq;
    ly->s_max = smax;
    ly->qmax = c->resid_bits == 4 ? 7 : 127;
    ly->num_groups = (c->num_layers + c->layers_per_group - 1) / c->layers_per_group;
    ly->max_tokens = c->max_tokens;

    int64_t blk = 0;
    for (int k = 0; k < c->num_tiers; ++k) {
        const int64_t cap = align_up(c->tier_capacity[k], 16);  // whole 16-token blocks
        const int r = c->tier_rank[k], s = c->tier_resid[k];
        const int vb = (s * c->resid_bits + 7) / 8;
        ly->rank[k] = r;
        ly->resid[k] = s;
        const int is = (s + 3) & ~3, vs = (vb + 3) & ~3;
        ly->vbytes[k] = vb;
        ly->istride[k] = is;
        ly->vstride[k] = vs;
        ly->cap[k] = c->tier_capacity[k];
        ly->weight[k] = 4 * r + (s > 0 ? 2 * (is + vs + 2) : 0);
        ly->cost[k] = token_cost(r, c->r_max);
        ly->inv_cblk[k] = 1.0 / (16.0 * ly->cost[k]);
        blk = align_up(blk, 256);
        ly->f_coefK[k] = blk; blk = align_up(blk + cap * r * 2, 16);
        ly->f_coefV[k] = blk; blk = align_up(blk + cap * r * 2, 16);
        ly->f_idxK[k] = blk;  blk = align_up(blk + cap * is, 16);
        ly->f_idxV[k] = blk;  blk = align_up(blk + cap * is, 16);
        ly->f_valK[k] = blk;  blk = align_up(blk + cap * vs, 16);
        ly->f_valV[k] = blk;  blk = align_up(blk + cap * vs, 16);
        ly->f_scaleK[k] = blk; blk = align_up(blk + (s > 0 ? cap * 2 : 0), 16);
        ly->f_scaleV[k] = blk; blk = align_up(blk + (s > 0 ? cap * 2 : 0), 16);
    }
    // 16 spare bytes: fixed-width residual reads may run past the last token
    ly->head_block = align_up(blk + 16, 256);
    if (ly->head_block > INT32_MAX) return DWKV_ERR_UNSUPPORTED;   // offsets are 32-bit
    for (int k = 0; k < c->num_tiers; ++k) {
        TierDesc &t = ly->tier[k];
        t.coefK = (int32_t)ly->f_coefK[k];
        t.coefV = (int32_t)ly->f_coefV[k];
        t.idxK = (int32_t)ly->f_idxK[k];
        t.idxV = (int32_t)ly->f_idxV[k];
        t.valK = (int32_t)ly->f_valK[k];
        t.valV = (int32_t)ly->f_valV[k];
        t.scaleK = (int32_t)ly->f_scaleK[k];
        t.scaleV = (int32_t)ly->f_scaleV[k];
        t.rank = ly->rank[k];
        t.resid = ly->resid[k];
        t.istride = ly->istride[k];
        t.vstride = ly->vstride[k];
        t.weight = ly->weight[k];
        t.pad0 = t.pad1 = t.pad2 = 0;
    }
    const int64_t heads = (int64_t)ly->L * ly->Bmax * ly->Hkv;
    int64_t off = 0;
    ly->off_err = off;      off = align_up(off + 4, 256);
    ly->off_counts = off;   off = align_up(off + heads * ly->T * 4, 256);
    ly->off_posmap = off;   off = align_up(off + heads * ly->max_tokens * 4, 256);
    ly->basis_elems = (int64_t)ly->Hkv * ly->R * ly->d;
    ly->off_basis = off;    off = align_up(off + (int64_t)ly->num_groups * 2 * ly->basis_elems * 2, 256);
    ly->off_basisvt = off;  off = align_up(off + (int64_t)ly->num_groups * ly->basis_elems * 2, 256);
    ly->off_seg = off;      off = off + heads * ly->head_block;
    // spare tail: the decode kernel's fixed-shape tile loads may read up to
    // a few KiB past the last token of the last head block
    ly->total = align_up(off + kArenaTail, 256);
    return DWKV_OK;
}

// Workgroups per (sequence, KV head) for decode.  A decode workgroup fills
// one compute unit (8 waves, more than half the LDS), so the grid aims at
// one workgroup per compute unit of the 256, while leaving each workgroup at
// least 1024 token slots (16 tiles of 64) of its head.
static int plan_splits(const dwkv_config &c, const Layout &ly)
{
    if (c.decode_splits > 0) return c.decode_splits;
    int64_t slots = 0;
    for (int k = 0; k < ly.T; ++k) slots += ly.cap[k];
    const int64_t heads = (int64_t)ly.Bmax * ly.Hkv;
    int64_t s = (256 + heads - 1) / heads;
    const int64_t by_tokens = slots / 1024;
    if (s > by_tokens) s = by_tokens;
    if (s < 1) s = 1;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int)s;
}

size_t decode_workspace_bytes(const Layout &ly, int batch, int splits)
{
    const int64_t B = batch;
    int64_t off = align_up(B * ly.Hkv * kArriveStride * 4, 256);
    off += align_up(B * ly.Hkv * splits * kMlStride * 4, 256);
    off += align_up(B * ly.Hq * splits * (int64_t)ly.d * 4, 256);
    return (size_t)off;
}

DecodeWorkspace carve_workspace(const Layout &ly, void *ws, int batch, int splits)
{
    const int64_t B = batch;
    uint8_t *p = static_cast<uint8_t *>(ws);
    DecodeWorkspace w;
    w.arrive = reinterpret_cast<uint32_t *>(p);
    p += align_up(B * ly.Hkv * kArriveStride * 4, 256);
    w.pm = reinterpret_cast<float *>(p);
    w.pl = w.pm + kMlNorm;
    p += align_up(B * ly.Hkv * splits * kMlStride * 4, 256);
    w.po = reinterpret_cast<float *>(p);
    return w;
}

}  // namespace dwkv

using dwkv::Layout;

static thread_local char g_hip_detail[160];

static int hip_status(hipError_t e)
{
    if (e == hipSuccess) return DWKV_OK;
    std::snprintf(g_hip_detail, sizeof g_hip_detail, "%s (%d)", hipGetErrorString(e), (int)e);
    return DWKV_ERR_HIP;
}

static bool valid_handle(const dwkv_handle *h) { return h && h->arena; }

extern "C" {

int dwkv_arena_bytes(const dwkv_config *cfg, size_t *bytes)
{
    if (!cfg || !bytes) return DWKV_ERR_INVALID_ARG;
    Layout ly;
    int rc = dwkv::build_layout(cfg, &ly);
    if (rc != DWKV_OK) return rc;
    *bytes = (size_t)ly.total;
    return DWKV_OK;
}

int dwkv_create(const dwkv_config *cfg, void *arena, size_t arena_bytes, dwkv_handle **out)
{
    if (!cfg || !arena || !out) return DWKV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(arena) % 256 != 0) return DWKV_ERR_INVALID_ARG;
    Layout ly;
    int rc = dwkv::build_layout(cfg, &ly);
    if (rc != DWKV_OK) return rc;
    if (arena_bytes < (size_t)ly.total) return DWKV_ERR_WORKSPACE;
    dwkv_handle *h = new (std::nothrow) dwkv_handle;
    if (!h) return DWKV_ERR_INVALID_ARG;
    h->cfg = *cfg;
    h->ly = ly;
    h->arena = static_cast<uint8_t *>(arena);
    h->splits = dwkv::plan_splits(*cfg, ly);
    *out = h;
    return DWKV_OK;
}

int dwkv_destroy(dwkv_handle *h)
{
    if (!h) return DWKV_ERR_INVALID_ARG;
    delete h;
    return DWKV_OK;
}

int dwkv_reset(dwkv_handle *h, void *stream)
{
    if (!valid_handle(h)) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // error word and the counts are contiguous words at the arena start
    int64_t words = (ly.off_counts + (int64_t)ly.L * ly.Bmax * ly.Hkv * ly.T * 4) / 4;
    return hip_status(dwkv::launch_fill_u32(reinterpret_cast<uint32_t *>(h->arena), 0u, words, s));
}

int dwkv_set_basis(dwkv_handle *h, int group, const void *basisK, const void *basisV,
                   void *stream)
{
    if (!valid_handle(h) || !basisK || !basisV) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (group < 0 || group >= ly.num_groups) return DWKV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    size_t bytes = (size_t)ly.basis_elems * 2;
    hipError_t e = hipMemcpyAsync(dwkv::basis_ptr(ly, h->arena, group, 0, 0), basisK, bytes,
                                  hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(dwkv::basis_ptr(ly, h->arena, group, 1, 0), basisV, bytes,
                           hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = dwkv::launch_transpose_basis(ly, h->arena, group, s);
    return hip_status(e);
}

static bool logical_ok(const dwkv_logical_layer *L, int s_max)
{
    if (!L || L->n_max < 0) return false;
    if (!L->tier || !L->coefK || !L->coefV) return false;
    if (s_max > 0 && (!L->idxK || !L->idxV || !L->valK || !L->valV || !L->scaleK || !L->scaleV))
        return false;
    return true;
}

int dwkv_import_layer(dwkv_handle *h, int layer, const dwkv_logical_layer *src,
                      const int64_t *n_tokens, int batch, void *stream)
{
    if (!valid_handle(h) || !n_tokens) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    if (!logical_ok(src, ly.s_max)) return DWKV_ERR_INVALID_ARG;
    for (int b = 0; b < batch; ++b) {
        if (n_tokens[b] < 0 || n_tokens[b] > src->n_max) return DWKV_ERR_INVALID_ARG;
        if (n_tokens[b] > ly.max_tokens) return DWKV_ERR_CAPACITY;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int b = 0; b < batch; ++b) {
        hipError_t e = dwkv::launch_import(ly, h->arena, layer, *src, b, n_tokens[b], s);
        if (e != hipSuccess) return hip_status(e);
    }
    return DWKV_OK;
}

int dwkv_export_layer(dwkv_handle *h, int layer, const dwkv_logical_layer *dst, int32_t *counts,
                      int32_t *slots, int batch, void *stream)
{
    if (!valid_handle(h) || !counts) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    if (!logical_ok(dst, ly.s_max)) return DWKV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(dwkv::launch_export(ly, h->arena, layer, *dst, counts, slots, batch, s));
}

int dwkv_read_counts(dwkv_handle *h, int layer, int batch, int32_t *host_counts, void *stream)
{
    if (!valid_handle(h) || !host_counts) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    size_t bytes = (size_t)batch * ly.Hkv * ly.T * 4;
    hipError_t e = hipMemcpyAsync(host_counts, dwkv::counts_ptr(ly, h->arena, layer, 0, 0), bytes,
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return hip_status(e);
}

int dwkv_workspace_bytes(const dwkv_config *cfg, int batch, size_t *bytes)
{
    if (!cfg || !bytes) return DWKV_ERR_INVALID_ARG;
    Layout ly;
    int rc = dwkv::build_layout(cfg, &ly);
    if (rc != DWKV_OK) return rc;
    if (batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    *bytes = dwkv::decode_workspace_bytes(ly, batch, dwkv::plan_splits(*cfg, ly));
    return DWKV_OK;
}

int dwkv_decode_attn(dwkv_handle *h, int layer, const void *q, int batch, float softmax_scale,
                     float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!valid_handle(h) || !q || !out || !workspace) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return DWKV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return DWKV_ERR_INVALID_ARG;
    if (workspace_bytes < dwkv::decode_workspace_bytes(ly, batch, h->splits))
        return DWKV_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    dwkv::DecodeWorkspace ws = dwkv::carve_workspace(ly, workspace, batch, h->splits);
    return hip_status(
        dwkv::launch_decode(ly, h->arena, layer, q, batch, softmax_scale, out, ws, h->splits, nullptr, s));
}

int dwkv_decode_step(dwkv_handle *h, int layer, const void *q, int batch, float softmax_scale,
                     float *out, void *workspace, size_t workspace_bytes, const void *k,
                     const void *v, const void *tier, const void *gateK, const void *gateV,
                     void *stream)
{
    if (!valid_handle(h) || !q || !out || !workspace || !k || !v || !tier) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return DWKV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return DWKV_ERR_INVALID_ARG;
    if (workspace_bytes < dwkv::decode_workspace_bytes(ly, batch, h->splits))
        return DWKV_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    dwkv::DecodeWorkspace ws = dwkv::carve_workspace(ly, workspace, batch, h->splits);
    const dwkv::AppendArgs ap{static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                              static_cast<const uint8_t *>(tier), static_cast<const uint16_t *>(gateK),
                              static_cast<const uint16_t *>(gateV)};
    return hip_status(
        dwkv::launch_decode(ly, h->arena, layer, q, batch, softmax_scale, out, ws, h->splits, &ap, s));
}

int dwkv_append(dwkv_handle *h, int layer, const void *k, const void *v, const void *tier,
                const void *gateK, const void *gateV, int batch, void *stream)
{
    if (!valid_handle(h) || !k || !v || !tier) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(dwkv::launch_append(ly, h->arena, layer, k, v, tier, gateK, gateV, batch, s));
}

int dwkv_check_errors(dwkv_handle *h, void *stream, uint32_t *bits)
{
    if (!valid_handle(h)) return DWKV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t word = 0;
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess)
        e = hipMemcpy(&word, dwkv::err_ptr(h->ly, h->arena), 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    if (bits) *bits = word;
    return word ? DWKV_ERR_DEVICE : DWKV_OK;
}

int dwkv_clear_errors(dwkv_handle *h, void *stream)
{
    if (!valid_handle(h)) return DWKV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(dwkv::launch_fill_u32(dwkv::err_ptr(h->ly, h->arena), 0u, 1, s));
}

const char *dwkv_last_hip_error(void) { return g_hip_detail; }

const char *dwkv_strerror(int code)
{
    switch (code) {
    case DWKV_OK: return "ok";
    case DWKV_ERR_INVALID_ARG: return "invalid argument";
    case DWKV_ERR_UNSUPPORTED: return "unsupported shape";
    case DWKV_ERR_WORKSPACE: return "workspace or arena too small";
    case DWKV_ERR_CAPACITY: return "capacity exceeded";
    case DWKV_ERR_HIP: return "HIP runtime error";
    case DWKV_ERR_DEVICE: return "device error word set";
    default: return "unknown error";
    }
}

}  // extern "C"
