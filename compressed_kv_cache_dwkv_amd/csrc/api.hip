// C ABI of libdwkv: argument validation, arena layout, launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "dwkv.h"
#include "kernels.h"
#include "layout.h"

struct dwkv_handle {
    dwkv_config cfg;
    dwkv::Layout ly;
    uint8_t *arena;
    int splits;
    uint64_t serial;                       // unique in the process
    // bases written per window so far (dwkv_set_basis, dwkv_prefill_bases)
    std::vector<uint64_t> basis_version;
};

namespace {

// The window bases a prefill workspace's block copy holds: made by handle
// `serial` for window `group` at basis version `version`, in the stream
// capture `capture` (0: not captured).  An encode reuses the copy only with
// every field equal, so a captured graph never relies on a copy made outside
// it, nor an eager call on one made inside a graph.
struct CopyTag {
    uint64_t serial;
    int group;
    uint64_t version;
    unsigned long long capture;
};
std::mutex g_copy_mu;
std::unordered_map<const void *, CopyTag> g_copy_tags;
std::atomic<uint64_t> g_next_serial{1};

}  // namespace

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
    if (c->coef_bits != 0 && c->coef_bits != 8 && c->coef_bits != 16) return DWKV_ERR_UNSUPPORTED;
    if (c->coef_bits == 8 && c->r_max > 64) return DWKV_ERR_UNSUPPORTED;
    int prev = 0, smax = 0;
    for (int k = 0; k < c->num_tiers; ++k) {
        int r = c->tier_rank[k], s = c->tier_resid[k];
        if (r <= 0 || r > c->r_max || r % 4 != 0) return DWKV_ERR_UNSUPPORTED;
        if (r < prev) return DWKV_ERR_INVALID_ARG;   // ranks non-decreasing (equal ranks: tiers that
                                                     // differ only in their residual channels)
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
    ly->cb = c->coef_bits == 8 ? 1 : 2;
    const int cb = ly->cb;
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
        ly->weight[k] = 2 * cb * r + (cb == 1 ? 4 : 0) + (s > 0 ? 2 * (is + vs + 2) : 0);
        ly->cost[k] = token_cost(r, c->r_max);
        ly->inv_cblk[k] = 1.0 / (16.0 * ly->cost[k]);
        blk = align_up(blk, 256);
        ly->f_coefK[k] = blk; blk = align_up(blk + cap * r * cb, 16);
        ly->f_coefV[k] = blk; blk = align_up(blk + cap * r * cb, 16);
        ly->f_idxK[k] = blk;  blk = align_up(blk + cap * is, 16);
        ly->f_idxV[k] = blk;  blk = align_up(blk + cap * is, 16);
        ly->f_valK[k] = blk;  blk = align_up(blk + cap * vs, 16);
        ly->f_valV[k] = blk;  blk = align_up(blk + cap * vs, 16);
        ly->f_scaleK[k] = blk; blk = align_up(blk + (s > 0 ? cap * 2 : 0), 16);
        ly->f_scaleV[k] = blk; blk = align_up(blk + (s > 0 ? cap * 2 : 0), 16);
        ly->f_cscK[k] = blk; blk = align_up(blk + (cb == 1 ? cap * 2 : 0), 16);
        ly->f_cscV[k] = blk; blk = align_up(blk + (cb == 1 ? cap * 2 : 0), 16);
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
        t.cscK = (int32_t)ly->f_cscK[k];
        t.cscV = (int32_t)ly->f_cscV[k];
        t.pad2 = 0;
        // operand slots of a decode tile (the rank's 16-channel blocks, at
        // most 8 slots) and the residual record masks
        const int r = ly->rank[k], sk = ly->resid[k];
        const int lkbr = (r > 16) + (r > 32) + (r > 64);
        for (int i = 0; i < 8; ++i) {
            const int mb = i >> lkbr, kb = i & ((1 << lkbr) - 1);
            t.koff[i] = (16 * mb * r + 16 * kb) * ly->cb;
            t.voff[i] = (mb * r + 16 * kb) * 16 * ly->cb;
        }
        auto low_bits = [](int n) -> uint32_t { return n >= 32 ? 0xFFFFFFFFu : n <= 0 ? 0u : (1u << n) - 1u; };
        t.im0 = low_bits(8 * sk);
        t.im1 = low_bits(8 * sk - 32);
        t.cm0 = low_bits(ly->bits * sk);
        t.cm1 = low_bits(ly->bits * sk - 32);
    }
    const int64_t heads = (int64_t)ly->L * ly->Bmax * ly->Hkv;
    int64_t off = 0;
    ly->off_err = off;      off = align_up(off + 4, 256);
    ly->off_counts = off;   off = align_up(off + heads * ly->T * 4, 256);
    ly->off_posmap = off;   off = align_up(off + heads * ly->max_tokens * 4, 256);
    ly->basis_elems = (int64_t)ly->Hkv * ly->R * ly->d;
    ly->off_basis = off;    off = align_up(off + (int64_t)ly->num_groups * 2 * ly->basis_elems * 2, 256);
    ly->off_basisvt = off;  off = align_up(off + (int64_t)ly->num_groups * ly->basis_elems * 2, 256);
    ly->off_basiskt = off;  off = align_up(off + (int64_t)ly->num_groups * ly->basis_elems * 2, 256);
    ly->off_seg = off;      off = off + heads * ly->head_block;
    // spare tail: the decode kernel's fixed-shape tile loads may read up to
    // a few KiB past the last token of the last head block
    ly->total = align_up(off + kArenaTail, 256);
    return DWKV_OK;
}

// Workgroups per (sequence, KV head) for decode.  A decode workgroup fills
// one compute unit (8 waves, more than half the LDS), so the grid aims at
// Compute units of the current device (read once per process; 256, the
// MI355X's, when no device answers, as in host-only use).
static int device_cus()
{
    static int cus = 0;
    static std::once_flag once;
    std::call_once(once, [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
        (void)hipGetLastError();
    });
    return cus;
}

// one workgroup per compute unit of the device, while leaving each
// workgroup at least 1024 token slots (16 tiles of 64) of its head.
static int plan_splits(const dwkv_config &c, const Layout &ly)
{
    if (c.decode_splits > 0) return c.decode_splits;
    int64_t slots = 0;
    for (int k = 0; k < ly.T; ++k) slots += ly.cap[k];
    const int64_t heads = (int64_t)ly.Bmax * ly.Hkv;
    const int64_t cus = device_cus();
    int64_t s = (cus + heads - 1) / heads;
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

// The decode workspace of dwkv_decode_step_noalloc: a fixed region of
// arrival counters at the start (so that no call's partials ever overlap
// another call's counters, whatever their batch), then the per-split maxima,
// normalisers and output vectors as in a caller workspace.
constexpr int64_t kScratchCounterBytes = (int64_t)DWKV_NOALLOC_MAX_PAIRS * kArriveStride * 4;

static size_t noalloc_workspace_bytes(const Layout &ly, int batch, int splits)
{
    const int64_t B = batch;
    int64_t off = kScratchCounterBytes;
    off += align_up(B * ly.Hkv * splits * kMlStride * 4, 256);
    off += align_up(B * ly.Hq * splits * (int64_t)ly.d * 4, 256);
    return (size_t)off;
}

static DecodeWorkspace carve_noalloc(const Layout &ly, uint8_t *p, int batch, int splits)
{
    DecodeWorkspace w;
    w.arrive = reinterpret_cast<uint32_t *>(p);
    p += kScratchCounterBytes;
    w.pm = reinterpret_cast<float *>(p);
    w.pl = w.pm + kMlNorm;
    p += align_up((int64_t)batch * ly.Hkv * splits * kMlStride * 4, 256);
    w.po = reinterpret_cast<float *>(p);
    return w;
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

// Scratch memory of dwkv_decode_step_noalloc.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names
// a host-side stand-in, never device memory: kernels and copies take the
// device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[DWKV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];      // device address of `scratch` per device, once set up
}  // namespace

// The current device's scratch address, set up on the first call on that
// device: the address is looked up, and the arrival counters are cleared by
// a kernel queued on `stream` ahead of the caller's first decode (each
// decode leaves them at zero for the next).
static int noalloc_scratch(hipStream_t stream, uint8_t **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return DWKV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!ptr) return DWKV_ERR_HIP;
        e = dwkv::launch_fill_u32(static_cast<uint32_t *>(ptr), 0u, dwkv::kScratchCounterBytes / 4, stream);
        if (e != hipSuccess) return hip_status(e);
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<uint8_t *>(g_scratch_ptr[dev]);
    return DWKV_OK;
}


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
    h->serial = g_next_serial.fetch_add(1);
    try {
        h->basis_version.assign((size_t)ly.num_groups, 0);
    } catch (...) {
        delete h;
        return DWKV_ERR_INVALID_ARG;
    }
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
    ++h->basis_version[group];
    size_t bytes = (size_t)ly.basis_elems * 2;
    hipError_t e = hipMemcpyAsync(dwkv::basis_ptr(ly, h->arena, group, 0, 0), basisK, bytes,
                                  hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(dwkv::basis_ptr(ly, h->arena, group, 1, 0), basisV, bytes,
                           hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = dwkv::launch_transpose_basis(ly, h->arena, group, s);
    return hip_status(e);
}

int dwkv_get_basis(dwkv_handle *h, int group, void *basisK, void *basisV, void *stream)
{
    if (!valid_handle(h) || !basisK || !basisV) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (group < 0 || group >= ly.num_groups) return DWKV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t bytes = (size_t)ly.basis_elems * 2;
    hipError_t e = hipMemcpyAsync(basisK, dwkv::basis_ptr(ly, h->arena, group, 0, 0), bytes,
                                  hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(basisV, dwkv::basis_ptr(ly, h->arena, group, 1, 0), bytes, hipMemcpyDeviceToDevice, s);
    return hip_status(e);
}

static bool logical_ok(const dwkv_logical_layer *L, int s_max, int cb)
{
    if (!L || L->n_max < 0) return false;
    if (!L->tier || !L->coefK || !L->coefV) return false;
    if (s_max > 0 && (!L->idxK || !L->idxV || !L->valK || !L->valV || !L->scaleK || !L->scaleV))
        return false;
    if (cb == 1 && (!L->cscaleK || !L->cscaleV)) return false;
    return true;
}

int dwkv_import_layer(dwkv_handle *h, int layer, const dwkv_logical_layer *src,
                      const int64_t *n_tokens, int batch, void *stream)
{
    if (!valid_handle(h) || !n_tokens) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    if (!logical_ok(src, ly.s_max, ly.cb)) return DWKV_ERR_INVALID_ARG;
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
    if (!logical_ok(dst, ly.s_max, ly.cb)) return DWKV_ERR_INVALID_ARG;
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

int dwkv_decode_splits(const dwkv_handle *h, int *splits)
{
    if (!valid_handle(h) || !splits) return DWKV_ERR_INVALID_ARG;
    *splits = h->splits;
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

int dwkv_decode_step_noalloc(dwkv_handle *h, int layer, const void *q, int batch, float softmax_scale,
                             float *out, const void *k, const void *v, const void *tier,
                             const void *gateK, const void *gateV, void *stream)
{
    if (!valid_handle(h) || !q || !out || !k || !v || !tier) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return DWKV_ERR_INVALID_ARG;
    if ((int64_t)batch * ly.Hkv > DWKV_NOALLOC_MAX_PAIRS) return DWKV_ERR_WORKSPACE;
    if (dwkv::noalloc_workspace_bytes(ly, batch, h->splits) > (size_t)DWKV_NOALLOC_SCRATCH_BYTES)
        return DWKV_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *base = nullptr;
    const int rc = noalloc_scratch(s, &base);
    if (rc != DWKV_OK) return rc;
    dwkv::DecodeWorkspace ws = dwkv::carve_noalloc(ly, base, batch, h->splits);
    const dwkv::AppendArgs ap{static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                              static_cast<const uint8_t *>(tier), static_cast<const uint16_t *>(gateK),
                              static_cast<const uint16_t *>(gateV)};
    return hip_status(
        dwkv::launch_decode(ly, h->arena, layer, q, batch, softmax_scale, out, ws, h->splits, &ap, s));
}

int dwkv_materialize_layer(dwkv_handle *h, int layer, int batch, void *k_out, void *v_out, int64_t n_cap,
                           int32_t *n_out, void *stream)
{
    if (!valid_handle(h) || !k_out || !v_out) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax) return DWKV_ERR_INVALID_ARG;
    if (n_cap <= 0 || n_cap % 64 != 0 || n_cap < ly.max_tokens || n_cap / 64 > INT32_MAX) return DWKV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(dwkv::launch_materialize(ly, h->arena, layer, batch, static_cast<uint16_t *>(k_out),
                                               static_cast<uint16_t *>(v_out), n_cap, n_out, s));
}

static bool dense_shape_ok(int batch, int num_q_heads, int num_kv_heads, int head_dim, int splits)
{
    if (batch <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0) return false;
    const int gq = num_q_heads / num_kv_heads;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8) return false;
    if (head_dim != 64 && head_dim != 128) return false;
    return splits >= 1 && splits <= dwkv::kMaxSplits;
}

static size_t dense_ws_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim, int splits)
{
    const int64_t B = batch;
    int64_t off = dwkv::align_up(B * num_kv_heads * dwkv::kArriveStride * 4, 256);
    off += dwkv::align_up(B * num_kv_heads * splits * dwkv::kMlStride * 4, 256);
    off += dwkv::align_up(B * num_q_heads * (int64_t)splits * head_dim * 4, 256);
    return (size_t)off;
}

int dwkv_dense_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim, int splits,
                               size_t *bytes)
{
    if (!bytes || !dense_shape_ok(batch, num_q_heads, num_kv_heads, head_dim, splits)) return DWKV_ERR_INVALID_ARG;
    *bytes = dense_ws_bytes(batch, num_q_heads, num_kv_heads, head_dim, splits);
    return DWKV_OK;
}

int dwkv_stream_probe(const void *src, int64_t bytes, int workgroups, int threads, uint32_t magic, uint32_t *sink,
                      void *stream)
{
    if (!src || !sink) return DWKV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return DWKV_ERR_INVALID_ARG;
    if (bytes <= 0 || bytes % 16 != 0) return DWKV_ERR_INVALID_ARG;
    if (workgroups < 1 || workgroups > 65535 || threads < 64 || threads > 1024 || threads % 64 != 0)
        return DWKV_ERR_INVALID_ARG;
    return hip_status(dwkv::launch_stream_read(src, bytes, workgroups, threads, magic, sink,
                                               static_cast<hipStream_t>(stream)));
}

int dwkv_dense_decode(const void *q, const void *k, const void *v, const int32_t *n_tokens, int batch,
                      int num_q_heads, int num_kv_heads, int head_dim, int64_t n_cap, int splits,
                      float softmax_scale, float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !n_tokens || !out || !workspace) return DWKV_ERR_INVALID_ARG;
    if (!dense_shape_ok(batch, num_q_heads, num_kv_heads, head_dim, splits)) return DWKV_ERR_INVALID_ARG;
    if (n_cap <= 0 || n_cap % 64 != 0 || n_cap >= (int64_t(1) << 31)) return DWKV_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return DWKV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return DWKV_ERR_INVALID_ARG;
    if (workspace_bytes < dense_ws_bytes(batch, num_q_heads, num_kv_heads, head_dim, splits))
        return DWKV_ERR_WORKSPACE;
    uint8_t *p = static_cast<uint8_t *>(workspace);
    dwkv::DenseArgs a;
    a.ws.arrive = reinterpret_cast<uint32_t *>(p);
    p += dwkv::align_up((int64_t)batch * num_kv_heads * dwkv::kArriveStride * 4, 256);
    a.ws.pm = reinterpret_cast<float *>(p);
    a.ws.pl = a.ws.pm + dwkv::kMlNorm;
    p += dwkv::align_up((int64_t)batch * num_kv_heads * splits * dwkv::kMlStride * 4, 256);
    a.ws.po = reinterpret_cast<float *>(p);
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.n = n_tokens;
    a.out = out;
    a.B = batch;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.d = head_dim;
    a.n_cap = n_cap;
    a.scale = softmax_scale;
    return hip_status(dwkv::launch_dense_decode(a, splits, static_cast<hipStream_t>(stream)));
}

// Probe workspace: the compressed decode's, the dense decode's, then the
// two attention outputs of every probed query.
static size_t probe_ws_bytes(const Layout &ly, int splits, int batch, int n_queries, int dense_splits)
{
    const size_t a = dwkv::align_up((int64_t)dwkv::decode_workspace_bytes(ly, batch, splits), 256);
    const size_t b = dwkv::align_up((int64_t)dense_ws_bytes(batch, ly.Hq, ly.Hkv, ly.d, dense_splits), 256);
    const size_t o = dwkv::align_up((int64_t)n_queries * batch * ly.Hq * ly.d * 4, 256);
    return a + b + 2 * o;
}

int dwkv_probe_workspace_bytes(const dwkv_config *cfg, int batch, int n_queries, int dense_splits, size_t *bytes)
{
    if (!cfg || !bytes) return DWKV_ERR_INVALID_ARG;
    Layout ly;
    int rc = dwkv::build_layout(cfg, &ly);
    if (rc != DWKV_OK) return rc;
    if (batch <= 0 || batch > ly.Bmax || n_queries <= 0 || dense_splits < 1 || dense_splits > dwkv::kMaxSplits)
        return DWKV_ERR_INVALID_ARG;
    *bytes = probe_ws_bytes(ly, dwkv::plan_splits(*cfg, ly), batch, n_queries, dense_splits);
    return DWKV_OK;
}

int dwkv_probe_error(dwkv_handle *h, int layer, const void *q, int n_queries, int batch, const void *k_ref,
                     const void *v_ref, const int32_t *n_ref, int64_t n_cap, int dense_splits, float softmax_scale,
                     float eps, float *err, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!valid_handle(h) || !q || !k_ref || !v_ref || !n_ref || !err || !workspace) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax || n_queries <= 0) return DWKV_ERR_INVALID_ARG;
    if (dense_splits < 1 || dense_splits > dwkv::kMaxSplits) return DWKV_ERR_INVALID_ARG;
    if (n_cap <= 0 || n_cap % 64 != 0 || n_cap >= (int64_t(1) << 31)) return DWKV_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale) || !(eps >= 0.0f)) return DWKV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return DWKV_ERR_INVALID_ARG;
    if (workspace_bytes < probe_ws_bytes(ly, h->splits, batch, n_queries, dense_splits)) return DWKV_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *p = static_cast<uint8_t *>(workspace);
    const dwkv::DecodeWorkspace wc = dwkv::carve_workspace(ly, p, batch, h->splits);
    p += dwkv::align_up((int64_t)dwkv::decode_workspace_bytes(ly, batch, h->splits), 256);
    uint8_t *pd = p;
    p += dwkv::align_up((int64_t)dense_ws_bytes(batch, ly.Hq, ly.Hkv, ly.d, dense_splits), 256);
    const int64_t out_elems = (int64_t)batch * ly.Hq * ly.d;
    float *o_cmp = reinterpret_cast<float *>(p);
    float *o_ref = reinterpret_cast<float *>(p + dwkv::align_up((int64_t)n_queries * out_elems * 4, 256));
    dwkv::DenseArgs a;
    a.ws.arrive = reinterpret_cast<uint32_t *>(pd);
    pd += dwkv::align_up((int64_t)batch * ly.Hkv * dwkv::kArriveStride * 4, 256);
    a.ws.pm = reinterpret_cast<float *>(pd);
    a.ws.pl = a.ws.pm + dwkv::kMlNorm;
    pd += dwkv::align_up((int64_t)batch * ly.Hkv * dense_splits * dwkv::kMlStride * 4, 256);
    a.ws.po = reinterpret_cast<float *>(pd);
    a.k = static_cast<const uint16_t *>(k_ref);
    a.v = static_cast<const uint16_t *>(v_ref);
    a.n = n_ref;
    a.B = batch;
    a.Hq = ly.Hq;
    a.Hkv = ly.Hkv;
    a.d = ly.d;
    a.n_cap = n_cap;
    a.scale = softmax_scale;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    for (int i = 0; i < n_queries; ++i) {
        const uint16_t *qi = qq + i * out_elems;
        hipError_t e = dwkv::launch_decode(ly, h->arena, layer, qi, batch, softmax_scale, o_cmp + i * out_elems, wc,
                                           h->splits, nullptr, s);
        if (e != hipSuccess) return hip_status(e);
        a.q = qi;
        a.out = o_ref + i * out_elems;
        e = dwkv::launch_dense_decode(a, dense_splits, s);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(dwkv::launch_probe_error(o_ref, o_cmp, n_queries, batch, ly.Hq, ly.Hkv, ly.d, eps, err, s));
}

int dwkv_probe_update(float *tau, int32_t *below, int n_windows, const float *err, float tol, float step,
                      int patience, float tau_min, float tau_max)
{
    if (!tau || !below || !err || n_windows <= 0 || patience <= 0 || !(tau_min <= tau_max) || !(step >= 0.0f))
        return DWKV_ERR_INVALID_ARG;
    for (int m = 0; m < n_windows; ++m) {
        float t = tau[m];
        if (err[m] > tol) {
            t = t - step;
            below[m] = 0;
        } else {
            below[m] += 1;
            if (below[m] >= patience) {
                t = t + step;
                below[m] = 0;
            }
        }
        tau[m] = t < tau_min ? tau_min : (t > tau_max ? tau_max : t);
    }
    return DWKV_OK;
}

// ------------------------------------------------------------------ prefill

// Gram workgroups per (Z, KV head): about two workgroups per compute unit.
static int gram_splits(const Layout &ly)
{
    const int want = 2 * dwkv::device_cus();
    int s = (want + 2 * ly.Hkv - 1) / (2 * ly.Hkv);
    return s < 1 ? 1 : (s > dwkv::kGramMaxSplits ? dwkv::kGramMaxSplits : s);
}

// Prefill workspace: the Gram sums of every window (fp64, first, so that
// their offset is 0), the Gram partials, then the encoder's per-(sequence,
// KV head) status, tier counts and tier-ordered token lists, and the
// window's bases in fp32.
struct PrefillWs {
    double *acc;
    float *part;
    int32_t *status, *cnt0, *tot, *inv, *cntc;
    int n_chunks;
    uint16_t *bblocks;
    size_t bytes;
};

static PrefillWs carve_prefill(const Layout &ly, void *base)
{
    PrefillWs w;
    uint8_t *p = static_cast<uint8_t *>(base);
    size_t off = 0;
    auto take = [&](int64_t bytes) {
        uint8_t *q = p ? p + off : nullptr;
        off += (size_t)dwkv::align_up(bytes, 256);
        return q;
    };
    const int64_t dd = (int64_t)ly.d * ly.d;
    w.acc = reinterpret_cast<double *>(take((int64_t)ly.num_groups * 2 * ly.Hkv * dd * 8));
    w.part = reinterpret_cast<float *>(take((int64_t)2 * ly.Hkv * gram_splits(ly) * dwkv::gram_pairs(ly.d) * 256 * 4));
    w.status = reinterpret_cast<int32_t *>(take((int64_t)ly.Bmax * ly.Hkv * 4));
    w.cnt0 = reinterpret_cast<int32_t *>(take((int64_t)ly.Bmax * ly.Hkv * dwkv::kMaxTiers * 4));
    w.tot = reinterpret_cast<int32_t *>(take((int64_t)ly.Bmax * ly.Hkv * dwkv::kMaxTiers * 4));
    w.inv = reinterpret_cast<int32_t *>(take((int64_t)ly.Bmax * ly.Hkv * ly.max_tokens * 4));
    w.n_chunks = (int)((ly.max_tokens + dwkv::kSlotChunk - 1) / dwkv::kSlotChunk) + 1;
    w.cntc = reinterpret_cast<int32_t *>(take((int64_t)ly.Bmax * ly.Hkv * w.n_chunks * dwkv::kChunkStride * 4));
    w.bblocks = reinterpret_cast<uint16_t *>(take((int64_t)2 * ly.Hkv * ly.d * dwkv::kMaxRank * 2));
    w.bytes = off;
    return w;
}

int dwkv_prefill_workspace_bytes(const dwkv_config *cfg, size_t *bytes)
{
    if (!cfg || !bytes) return DWKV_ERR_INVALID_ARG;
    Layout ly;
    const int rc = dwkv::build_layout(cfg, &ly);
    if (rc != DWKV_OK) return rc;
    *bytes = carve_prefill(ly, nullptr).bytes;
    return DWKV_OK;
}

static int prefill_common(const dwkv_handle *h, int layer, const void *k, const void *v, const int32_t *n_tokens,
                          int batch, int64_t n_cap, void *ws, size_t ws_bytes)
{
    if (!valid_handle(h) || !k || !v || !n_tokens || !ws) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (layer < 0 || layer >= ly.L || batch <= 0 || batch > ly.Bmax || batch > dwkv::kGramMaxBatch)
        return DWKV_ERR_INVALID_ARG;
    if (n_cap <= 0 || n_cap >= (int64_t(1) << 31)) return DWKV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return DWKV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(k) % 16 != 0 || reinterpret_cast<uintptr_t>(v) % 16 != 0)
        return DWKV_ERR_INVALID_ARG;
    if (ws_bytes < carve_prefill(ly, nullptr).bytes) return DWKV_ERR_WORKSPACE;
    return DWKV_OK;
}

int dwkv_prefill_gram(dwkv_handle *h, int layer, const void *k, const void *v, const int32_t *n_tokens, int batch,
                      int64_t n_cap, int first, void *workspace, size_t workspace_bytes, void *stream)
{
    const int rc = prefill_common(h, layer, k, v, n_tokens, batch, n_cap, workspace, workspace_bytes);
    if (rc != DWKV_OK) return rc;
    const Layout &ly = h->ly;
    // the Gram kernel addresses a sequence's rows with 32-bit byte offsets
    if ((n_cap + 256) * ly.d * 2 > (int64_t)UINT32_MAX) return DWKV_ERR_UNSUPPORTED;
    const PrefillWs w = carve_prefill(ly, workspace);
    dwkv::GramArgs a;
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.n_tokens = n_tokens;
    a.B = batch;
    a.Hkv = ly.Hkv;
    a.n_cap = n_cap;
    a.S = gram_splits(ly);
    a.first = first ? 1 : 0;
    a.part = w.part;
    a.acc = w.acc + (int64_t)(layer / ly.G) * 2 * ly.Hkv * ly.d * ly.d;
    return hip_status(dwkv::launch_gram(ly, h->arena, a, static_cast<hipStream_t>(stream)));
}

int dwkv_prefill_bases(dwkv_handle *h, int group0, int n_groups, const float *omega, int sketch, int power_iters,
                       double *ritz, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!valid_handle(h) || !omega || !workspace) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    if (group0 < 0 || n_groups <= 0 || group0 + n_groups > ly.num_groups) return DWKV_ERR_INVALID_ARG;
    if (sketch < ly.R || sketch > ly.d || power_iters < 0 || power_iters > 16) return DWKV_ERR_INVALID_ARG;
    if (sketch > dwkv::kMaxSketch) return DWKV_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return DWKV_ERR_INVALID_ARG;
    if (workspace_bytes < carve_prefill(ly, nullptr).bytes) return DWKV_ERR_WORKSPACE;
    const PrefillWs w = carve_prefill(ly, workspace);
    dwkv::BasesArgs a;
    a.acc = w.acc + (int64_t)group0 * 2 * ly.Hkv * ly.d * ly.d;
    a.omega = omega;
    a.ritz = ritz;
    a.k = sketch;
    a.power_iters = power_iters;
    a.group0 = group0;
    for (int g = group0; g < group0 + n_groups; ++g) ++h->basis_version[g];
    return hip_status(dwkv::launch_bases(ly, h->arena, a, n_groups, static_cast<hipStream_t>(stream)));
}

int dwkv_prefill_encode(dwkv_handle *h, int layer, const void *k, const void *v, const int32_t *n_tokens, int batch,
                        int64_t n_cap, const void *tier, const void *gate_k, const void *gate_v, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    const int rc = prefill_common(h, layer, k, v, n_tokens, batch, n_cap, workspace, workspace_bytes);
    if (rc != DWKV_OK) return rc;
    if (!tier) return DWKV_ERR_INVALID_ARG;
    const Layout &ly = h->ly;
    const PrefillWs w = carve_prefill(ly, workspace);
    dwkv::EncodeArgs a;
    a.layer = layer;
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.n_tokens = n_tokens;
    a.n_cap = n_cap;
    a.tier = static_cast<const uint8_t *>(tier);
    a.gateK = static_cast<const uint16_t *>(gate_k);
    a.gateV = static_cast<const uint16_t *>(gate_v);
    a.status = w.status;
    a.cnt0 = w.cnt0;
    a.tot = w.tot;
    a.inv = w.inv;
    a.basis_blocks = w.bblocks;
    a.cntc = w.cntc;
    {
        const int64_t need = (n_cap + dwkv::kSlotChunk - 1) / dwkv::kSlotChunk;
        a.n_chunks = (int)(need < w.n_chunks ? (need < 1 ? 1 : need) : w.n_chunks);
    }
    // the window's block copy of its bases is made once per basis version
    // (and per stream capture)
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int m = layer / ly.G;
    unsigned long long capture = 0;
    hipStreamCaptureStatus cst = hipStreamCaptureStatusNone;
    if (hipStreamGetCaptureInfo(s, &cst, &capture) != hipSuccess) {
        (void)hipGetLastError();
        cst = hipStreamCaptureStatusNone;
    }
    if (cst != hipStreamCaptureStatusActive) capture = 0;
    const CopyTag want{h->serial, m, h->basis_version[m], capture};
    {
        std::lock_guard<std::mutex> lock(g_copy_mu);
        auto it = g_copy_tags.find(workspace);
        a.copy_basis = !(it != g_copy_tags.end() && it->second.serial == want.serial && it->second.group == want.group &&
                         it->second.version == want.version && it->second.capture == want.capture);
        if (it != g_copy_tags.end()) g_copy_tags.erase(it);
    }
    const int rc2 = hip_status(dwkv::launch_prefill_encode(ly, h->arena, a, batch, s));
    if (rc2 == DWKV_OK) {
        std::lock_guard<std::mutex> lock(g_copy_mu);
        g_copy_tags[workspace] = want;
    }
    return rc2;
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
