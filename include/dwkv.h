/*
 * dwkv.h -- C ABI of libdwkv: decode-time attention over a DepthWeave-KV
 * compressed cache, and the per-token append, on AMD Instinct MI355X (gfx950).
 *
 * The cache (DepthWeave-KV paper, arXiv 2607.06523, §3 Method, Eq. (1)):
 * for every layer l, KV head h, token t and Z in {K, V}
 *
 *     X^Z_{l,h,t} = A^Z_{l,h,t} B^Z_{m,h} + g^Z_{l,h,t} R^Z_{l,h,t}
 *
 * where m = l / layers_per_group is the depth window, B^Z_{m,h} the window's
 * shared basis (r_max vectors of head_dim fp16 values), A the token's fp16
 * coefficient vector holding only the first r_k entries of its rank tier k
 * (the tier is the token-conditional router's decision, Eq. (2)), and g R a
 * sparse residual: s_k channel indices (ascending), s_k integer codes in
 * [-qmax, qmax] (qmax = 7 for 4-bit, 127 for 8-bit codes) and one fp16 scale
 * into which the gate g is folded.
 *
 * The two hot-path calls follow the decode procedure of the zhichai.net
 * DepthWeave-KV summary (Ch. 1.2): for the new token, compute its query,
 * attend over every cached key/value (dwkv_decode_attn), then append the new
 * key/value to the cache (dwkv_append).  Decode never materialises K^ or V^
 * in memory (paper §3, last paragraph before Fig. 2): scores are taken in
 * the basis' coordinate space and values accumulated there before a single
 * back-projection.
 *
 * Conventions for every entry point:
 *   - Return value: DWKV_OK (0) or a negative DWKV_ERR_* code.  Arguments
 *     are validated on the host before any GPU work is queued; on an error
 *     nothing is queued.
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary CPU memory.  The library never allocates, frees
 *     or retains device memory beyond the arena the caller hands to
 *     dwkv_create, and keeps only host metadata.
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is queued asynchronously and ordered by the stream; only
 *     dwkv_check_errors, dwkv_read_counts and dwkv_export_layer's caller-side
 *     copies synchronise.
 *   - A handle is not thread-safe; calls on one handle must be ordered by a
 *     single stream (or by the caller).
 *   - Query head g reads KV head g / (num_q_heads / num_kv_heads).
 */
#ifndef DWKV_H
#define DWKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DWKV_MAX_TIERS 8

/* Error codes. */
#define DWKV_OK 0
#define DWKV_ERR_INVALID_ARG (-1) /* null pointer, index out of range, bad size   */
#define DWKV_ERR_UNSUPPORTED (-2) /* shape outside what the kernels implement     */
#define DWKV_ERR_WORKSPACE (-3)   /* workspace or arena smaller than required     */
#define DWKV_ERR_CAPACITY (-4)    /* host-visible capacity exceeded               */
#define DWKV_ERR_HIP (-5)         /* a HIP runtime call or launch failed          */
#define DWKV_ERR_DEVICE (-6)      /* the device error word is set (check_errors)  */

/* Bits of the sticky device error word. */
#define DWKV_DEVERR_TIER_FULL 1u  /* a token did not fit its tier's capacity      */
#define DWKV_DEVERR_POS_FULL 2u   /* a position beyond max_tokens                 */
#define DWKV_DEVERR_BAD_TIER 4u   /* a tier index >= num_tiers in device input    */
#define DWKV_DEVERR_BAD_INDEX 8u  /* a residual channel index >= head_dim on import
                                     (stored as head_dim - 1)                     */

/*
 * Static shape of one cache.  Supported: head_dim 64 or 128; r_max a multiple
 * of 4 in [4, 128]; 1..8 tiers with ranks ascending, each a multiple of 4 and
 * <= r_max; tier_resid[k] (channels kept per token) in [0, 8]; resid_bits 4
 * or 8; num_q_heads a multiple of num_kv_heads with at most 8 query heads per
 * KV head.  tier_capacity[k] is the number of token slots per (layer,
 * sequence, KV head) reserved for tier k; max_tokens bounds the total tokens
 * per (layer, sequence, KV head).  decode_splits: workgroups per (sequence,
 * KV head) for dwkv_decode_attn, 0 = chosen from the capacities.
 */
typedef struct dwkv_config {
    int32_t num_layers;
    int32_t layers_per_group;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t r_max;
    int32_t num_tiers;
    int32_t tier_rank[DWKV_MAX_TIERS];
    int32_t tier_resid[DWKV_MAX_TIERS];
    int32_t resid_bits;
    int32_t max_batch;
    int32_t decode_splits;
    int64_t tier_capacity[DWKV_MAX_TIERS];
    int64_t max_tokens;
} dwkv_config;

typedef struct dwkv_handle dwkv_handle;

/*
 * One layer of the cache in logical form: tokens in position order, every
 * array device memory, token stride n_max.  Used to bulk-load a layer
 * (dwkv_import_layer) and to read it back (dwkv_export_layer).
 *   tier   uint8 [B][H_kv][n_max]
 *   coefK  fp16  [B][H_kv][n_max][r_max]   (entries >= the tier's rank ignored
 *   coefV                                     on import, written 0 on export)
 *   idxK   uint8 [B][H_kv][n_max][s_max]   (s_max = max tier_resid; entries
 *   idxV                                      >= the tier's s ignored / zero)
 *   valK   int8  [B][H_kv][n_max][s_max]   codes in [-qmax, qmax]
 *   valV
 *   scaleK fp16  [B][H_kv][n_max]
 *   scaleV
 */
typedef struct dwkv_logical_layer {
    int64_t n_max;
    void *tier;
    void *coefK, *coefV;
    void *idxK, *idxV;
    void *valK, *valV;
    void *scaleK, *scaleV;
} dwkv_logical_layer;

/* Bytes of device memory one cache needs (host only, no GPU call). */
int dwkv_arena_bytes(const dwkv_config *cfg, size_t *bytes);

/*
 * Binds a cache to a caller-owned device arena of at least
 * dwkv_arena_bytes bytes, 256-byte aligned.  Host only: the arena is not
 * touched; call dwkv_reset before first use.  *out receives the handle.
 */
int dwkv_create(const dwkv_config *cfg, void *arena, size_t arena_bytes, dwkv_handle **out);

/* Frees the handle's host memory (the arena stays the caller's). */
int dwkv_destroy(dwkv_handle *h);

/* Empties every layer and clears the device error word (queued on stream). */
int dwkv_reset(dwkv_handle *h, void *stream);

/*
 * Copies the shared bases of depth window `group` (paper §3: one basis per
 * window, head and Z) into the arena.  basisK, basisV: device fp16
 * [H_kv][r_max][head_dim], basis vector i of head h at [h][i][:].
 */
int dwkv_set_basis(dwkv_handle *h, int group, const void *basisK, const void *basisV,
                   void *stream);

/*
 * Replaces the content of `layer` by the logical cache `src` (device arrays,
 * see dwkv_logical_layer) holding n_tokens[b] tokens for sequence b < batch
 * (n_tokens: host int64 [batch]).  Tokens keep their position order inside
 * each tier.  Host-checked: n_tokens[b] <= min(n_max, max_tokens).
 * Device-checked (error word): tier indices, residual channel indices and
 * per-tier capacity.
 */
int dwkv_import_layer(dwkv_handle *h, int layer, const dwkv_logical_layer *src,
                      const int64_t *n_tokens, int batch, void *stream);

/*
 * Writes `layer` back in logical form into `dst` (device arrays, n_max >=
 * the longest sequence) and the per-(sequence, KV head, tier) token counts
 * into counts (device int32 [batch][H_kv][num_tiers]).  Slot of each token
 * inside its tier: slots (device int32 [batch][H_kv][n_max], may be NULL).
 */
int dwkv_export_layer(dwkv_handle *h, int layer, const dwkv_logical_layer *dst, int32_t *counts,
                      int32_t *slots, int batch, void *stream);

/* Synchronises the stream and copies the token counts of `layer` to host
 * int32 [batch][H_kv][num_tiers]. */
int dwkv_read_counts(dwkv_handle *h, int layer, int batch, int32_t *host_counts, void *stream);

/*
 * Device workspace dwkv_decode_attn needs for `batch` sequences.  It must be
 * zero-filled once before its first use; every decode call leaves it ready
 * for the next one (its arrival counters return to zero).
 */
int dwkv_workspace_bytes(const dwkv_config *cfg, int batch, size_t *bytes);

/*
 * Decode attention of one layer (the hot path; paper §3 last paragraph, and
 * the decode procedure of the zhichai.net summary Ch. 1.2):
 *   out[b][g][:] = sum_t softmax_t(softmax_scale * q[b][g] . K^_t) V^_t
 * over every token currently cached for (layer, b, g's KV head), with K^, V^
 * the Eq. (1) reconstructions.  No K^/V^ is written to memory.
 *   q:   device fp16 [batch][num_q_heads][head_dim]
 *   out: device fp32 [batch][num_q_heads][head_dim]; zero for an empty cache
 *   softmax_scale: > 0 (1/sqrt(head_dim) for standard attention)
 *   workspace: device, >= dwkv_workspace_bytes(cfg, batch), see above.
 */
int dwkv_decode_attn(dwkv_handle *h, int layer, const void *q, int batch, float softmax_scale,
                     float *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Appends one new token per (b, KV head) to `layer` (paper §3 second
 * paragraph: coefficients by projecting the vector onto the current basis,
 * residual kept on the router-chosen number of channels, low-bit group
 * quantisation).  For Z in {K, V}, x = the fp16 input vector, tier k, r = r_k,
 * s = s_k, all in IEEE fp32 with this fixed operation order:
 *   1. c_i = fp16_rne(fma-chain over j ascending of B[i][j] * x_j), i < r
 *   2. e_j = x_j - (fma-chain over i ascending of B[i][j] * c_i), j < d
 *   3. keep the s channels of largest |e_j|, ties to the smaller j
 *   4. s16 = fp16_rne(max kept |e_j| / qmax)      (correctly rounded divide)
 *   5. code_j = clamp(rint(e_j / s16), -qmax, qmax), 0 if s16 == 0
 *   6. stored scale = s16, or fp16_rne(gate * s16) if the gate is not 1
 * The token takes slot counts[layer][b][h][k] of its tier and position
 * n = total tokens of (layer, b, h).  A full tier or position map sets the
 * device error word and drops the token.
 *   k, v:   device fp16 [batch][H_kv][head_dim]
 *   tier:   device uint8 [batch][H_kv] (the router's rank tier)
 *   gateK, gateV: device fp16 [batch][H_kv], or NULL for a gate of 1
 */
int dwkv_append(dwkv_handle *h, int layer, const void *k, const void *v, const void *tier,
                const void *gateK, const void *gateV, int batch, void *stream);

/*
 * One whole decode step of a layer in a single launch: exactly
 * dwkv_decode_attn(q) over the cache as it stands, then dwkv_append(k, v,
 * tier, gates) -- the order of the zhichai.net summary's decode procedure
 * (Ch. 1.2: attend over the cached keys and values, then append the new
 * token's).  The cache afterwards is bit-identical to what the two calls
 * made in sequence leave; the attention output equals theirs up to
 * rounding (the tiles are split differently among workgroups, and each
 * rounds its probabilities to fp16 against its own running max).  For each (b, KV
 * head) the first decode workgroup encodes the new token into its slot past
 * the tier's counted tokens before taking a smaller share of the tiles, and
 * the workgroup that finishes last publishes it (tier count, position map)
 * once every workgroup of that head has read the counts.  Arguments,
 * layouts, errors and the workspace as for the two calls.
 */
int dwkv_decode_step(dwkv_handle *h, int layer, const void *q, int batch, float softmax_scale,
                     float *out, void *workspace, size_t workspace_bytes, const void *k,
                     const void *v, const void *tier, const void *gateK, const void *gateV,
                     void *stream);

/* Synchronises the stream; returns DWKV_ERR_DEVICE if the device error word
 * is set (its bits in *bits if non-NULL), else DWKV_OK. */
int dwkv_check_errors(dwkv_handle *h, void *stream, uint32_t *bits);

/* Clears the device error word (queued on stream). */
int dwkv_clear_errors(dwkv_handle *h, void *stream);

/* Static text for an error code. */
const char *dwkv_strerror(int code);

/* Text of the HIP error behind the calling thread's last DWKV_ERR_HIP
 * ("" if none); valid until the thread's next failing call. */
const char *dwkv_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DWKV_H */
