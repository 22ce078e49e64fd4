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
#define DWKV_DEVERR_BAD_LENGTH 16u /* a prefill length outside [0, n_cap]           */

/*
 * Static shape of one cache.  Supported: head_dim 64 or 128; r_max a multiple
 * of 4 in [4, 128]; 1..8 tiers with ranks non-decreasing (tiers of one rank
 * that differ in tier_resid give the paper's fixed coefficient width with
 * router-chosen residual channels), each a multiple of 4 and
 * <= r_max; tier_resid[k] (channels kept per token) in [0, 8]; resid_bits 4
 * or 8; num_q_heads a multiple of num_kv_heads with at most 8 query heads per
 * KV head.  tier_capacity[k] is the number of token slots per (layer,
 * sequence, KV head) reserved for tier k; max_tokens bounds the total tokens
 * per (layer, sequence, KV head).  decode_splits: workgroups per (sequence,
 * KV head) for dwkv_decode_attn, 0 = chosen from the capacities.
 * coef_bits selects the coefficient form (paper §3, second paragraph:
 * coefficients are stored in 8-bit blockwise quantised form; one block is
 * one token's r_k coefficients).
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
    int32_t coef_bits;   /* 16 (or 0): fp16 coefficients; 8: the paper's 8-bit blockwise form
                            (int8 codes in [-127, 127] and one fp16 scale per token and Z) */
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
 * With coef_bits 8, coefK/coefV hold int8 codes [B][H_kv][n_max][r_max] and
 *   cscaleK fp16  [B][H_kv][n_max]   each token's coefficient block scale
 *   cscaleV
 * (unused, may be NULL, with fp16 coefficients).
 */
typedef struct dwkv_logical_layer {
    int64_t n_max;
    void *tier;
    void *coefK, *coefV;
    void *idxK, *idxV;
    void *valK, *valV;
    void *scaleK, *scaleV;
    void *cscaleK, *cscaleV;
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

/* Copies the shared bases of window `group` out of the arena, in
 * dwkv_set_basis's layout (device fp16 [H_kv][r_max][head_dim] each). */
int dwkv_get_basis(dwkv_handle *h, int group, void *basisK, void *basisV, void *stream);

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
 * Workgroups per (sequence, KV head) that dwkv_decode_attn and
 * dwkv_decode_step launch with this handle (the config's decode_splits, or
 * the count chosen from the capacities when that is 0).  Host only.
 */
int dwkv_decode_splits(const dwkv_handle *h, int *splits);

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

/*
 * dwkv_decode_step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials and arrival counters
 * live in a static device array of DWKV_NOALLOC_SCRATCH_BYTES per GPU,
 * which the library holds until the process ends; nothing is allocated or
 * freed.  The first call on a device looks the array up and queues a
 * kernel on `stream` that clears its counters; every call leaves them at
 * zero for the next.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other threads, other handles)
 * race and give wrong results.  DWKV_ERR_WORKSPACE when batch * num_kv_heads
 * exceeds DWKV_NOALLOC_MAX_PAIRS or the partials of batch sequences at the
 * handle's split count exceed the array.  Otherwise as dwkv_decode_step.
 */
#define DWKV_NOALLOC_SCRATCH_BYTES (4 << 20)
#define DWKV_NOALLOC_MAX_PAIRS 1024
int dwkv_decode_step_noalloc(dwkv_handle *h, int layer, const void *q, int batch, float softmax_scale,
                             float *out, const void *k, const void *v, const void *tier,
                             const void *gateK, const void *gateV, void *stream);

/*
 * The explicit reconstruction an unfused decode performs before attention
 * (paper §3 Eq. (1); the zhichai.net summary's Ch. 3.3 names base lookup and
 * residual dequantisation as separate launches, and the paper's §5 ablation
 * measures decode without the fused kernel): every cached token of `layer`
 * for sequences b < batch, written as dense fp16 K^ and V^ in position order.
 *   k_out: device fp16 [batch][H_kv][n_cap][head_dim] (token rows)
 *   v_out: device fp16 [batch][H_kv][n_cap/16][head_dim][16] (16-token blocks,
 *          channel-major inside a block)
 *   n_cap: a multiple of 64, >= the config's max_tokens; positions past a
 *          sequence's length up to the next multiple of 64 are written 0,
 *          later ones are not written
 *   n_out: device int32 [batch][H_kv] (tokens per sequence and KV head), or NULL
 * Each element is the fp32 sum of the exact fp16 products plus the residual
 * channels, rounded once to fp16.
 */
int dwkv_materialize_layer(dwkv_handle *h, int layer, int batch, void *k_out, void *v_out, int64_t n_cap,
                           int32_t *n_out, void *stream);

/* Device workspace of dwkv_dense_decode (host only).  Zero-fill it once
 * before its first use; every call leaves it ready for the next. */
int dwkv_dense_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim, int splits,
                               size_t *bytes);

/*
 * Decode attention over a dense (uncompressed) fp16 K/V cache, the baseline
 * the compressed cache is measured against (paper §4) and the attention
 * launch of an unfused decode:
 *   out[b][g][:] = sum_{t < n_tokens[b][h]} softmax_t(softmax_scale q[b][g] . K_t) V_t
 * with h = g / (num_q_heads / num_kv_heads).
 *   q: device fp16 [batch][num_q_heads][head_dim]
 *   k, v: device, the layouts of dwkv_materialize_layer's k_out and v_out
 *   n_tokens: device int32 [batch][num_kv_heads], each <= n_cap
 *   splits: workgroups per (sequence, KV head), 1..256
 *   out: device fp32 [batch][num_q_heads][head_dim]; zero for an empty context
 * head_dim 64 or 128; 1, 2, 4 or 8 query heads per KV head.
 */
int dwkv_dense_decode(const void *q, const void *k, const void *v, const int32_t *n_tokens, int batch,
                      int num_q_heads, int num_kv_heads, int head_dim, int64_t n_cap, int splits,
                      float softmax_scale, float *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Measurement aid, not a step of the method: a plain streaming read of
 * `bytes` of device memory at src by `workgroups` workgroups of `threads`
 * threads (workgroup w reads the w-th contiguous share, 16 bytes per load,
 * four loads in flight per thread).  It computes nothing the method needs;
 * timed like a decode launch of the same size and grid, it gives the
 * bandwidth a single launch of that shape can reach on this device.
 *   src: device, 16-byte aligned; bytes: a positive multiple of 16
 *   workgroups: 1..65535; threads: a multiple of 64 in 64..1024
 *   magic, sink: the folded word of the loaded data is stored to sink[0]
 *          (device, 4 bytes) only if it equals magic; sink may be
 *          written, nothing else is
 * Returns DWKV_ERR_INVALID_ARG for a null or misaligned pointer or a size
 * or grid outside these ranges.
 */
int dwkv_stream_probe(const void *src, int64_t bytes, int workgroups, int threads, uint32_t magic, uint32_t *sink,
                      void *stream);

/* Device workspace of dwkv_probe_error for batch sequences and n_queries
 * probed query positions (host only).  Zero-fill it once before its first
 * use; every call leaves it ready for the next. */
int dwkv_probe_workspace_bytes(const dwkv_config *cfg, int batch, int n_queries, int dense_splits, size_t *bytes);

/*
 * The attention-output probe of the paper's §3 (Eq. (3)): for each
 * (sequence b, KV head h) of `layer`,
 *   err[b][h] = || Attn(Q, K, V) - Attn(Q, K^, V^) ||_2 / (|| Attn(Q, K, V) ||_2 + eps)
 * where K^, V^ is the compressed cache (dwkv_decode_attn over it), K, V a
 * higher-fidelity dense fp16 copy of the same tokens (dwkv_dense_decode over
 * it) and Q the n_queries recent query vectors; the norms run over every
 * query position, every query head of the KV head and every channel.
 *   q: device fp16 [n_queries][batch][num_q_heads][head_dim]
 *   k_ref, v_ref, n_ref, n_cap, dense_splits: the dense cache as for
 *          dwkv_dense_decode
 *   err: device fp32 [batch][num_kv_heads]
 * The reference cache is the caller's: the paper materialises it
 * temporarily for the probed window.  Which heads and positions to probe,
 * and how often, is the caller's schedule.
 */
int dwkv_probe_error(dwkv_handle *h, int layer, const void *q, int n_queries, int batch, const void *k_ref,
                     const void *v_ref, const int32_t *n_ref, int64_t n_cap, int dense_splits, float softmax_scale,
                     float eps, float *err, void *workspace, size_t workspace_bytes, void *stream);

/*
 * One probe interval of the router thresholds tau_m of n_windows depth
 * windows (the paper's §3, the paragraph after Eq. (3)), host memory only:
 * for window m, an error err[m] above tol lowers tau[m] by step (more tokens
 * of the window take higher residual rank) and resets below[m]; otherwise
 * below[m] counts the intervals in a row under tolerance and, when it
 * reaches patience, tau[m] rises by step (less residual storage) and
 * below[m] restarts.  tau stays in [tau_min, tau_max].  The pages give no
 * values for the tolerance, step or patience: they are the caller's.
 */
int dwkv_probe_update(float *tau, int32_t *below, int n_windows, const float *err, float tol, float step,
                      int patience, float tau_min, float tau_max);

/*
 * Prefill compression (the paper's §3 Method: the shared bases are
 * initialised after prefill from a randomized low-rank sketch of the cached
 * keys and values, per depth window, KV head and Z; every prefill token is
 * then projected onto its window's basis and its residual quantised at the
 * router's channel count -- the data path of Fig. 2).  Three calls, in this
 * order for each window m (layers m * layers_per_group ...):
 *
 *   dwkv_prefill_gram   once per layer of the window (first != 0 for the
 *                       first one): adds the layer's prefill vectors to the
 *                       window's Gram matrices C^Z_h = sum x x^T;
 *   dwkv_prefill_bases  forms the bases of one or more windows from their
 *                       Gram matrices and writes them into the cache (as
 *                       dwkv_set_basis would);
 *   dwkv_prefill_encode once per layer: appends its prefill tokens.
 *
 * Prefill keys and values k, v: device fp16 [batch][num_kv_heads][n_cap]
 * [head_dim] (16-byte aligned), the first n_tokens[b] positions of sequence
 * b valid; n_tokens: device int32 [batch] (a length outside [0, n_cap] sets
 * DWKV_DEVERR_BAD_LENGTH and counts as 0).  Every window's Gram sums pool
 * all layers of the window, all sequences of the batch and every valid
 * position (the bases are shared by the batch).
 *
 * Workspace: device memory of dwkv_prefill_workspace_bytes(cfg) bytes,
 * 256-byte aligned, zero-filled by the caller before its first use and left
 * ready for the next call; one workspace per stream of concurrent prefill
 * work, with one exception: dwkv_prefill_bases reads only its windows' Gram
 * sums and writes only their bases, so it may run on another stream, with
 * the same workspace, concurrently with Gram calls of other windows and
 * encode calls of layers of other windows (the caller orders each window's
 * Gram calls before its bases and its bases before its encodes, for
 * instance with events).  Its first num_groups * 2 * num_kv_heads * head_dim^2 * 8 bytes hold
 * the Gram sums, fp64 [window][Z][KV head][head_dim][head_dim] (row-major,
 * exactly symmetric), for inspection.
 */
int dwkv_prefill_workspace_bytes(const dwkv_config *cfg, size_t *bytes);

/* The window of `layer` gets layer's contribution.  The matrix-core partial
 * sums are fp32 per workgroup (a fixed share of the 64-token tiles of the
 * layer), added in fp64 in workgroup order: the result is deterministic.
 * DWKV_ERR_UNSUPPORTED when (n_cap + 256) * head_dim * 2 exceeds 2^32 - 1
 * (a sequence's rows are addressed with 32-bit byte offsets). */
int dwkv_prefill_gram(dwkv_handle *h, int layer, const void *k, const void *v, const int32_t *n_tokens, int batch,
                      int64_t n_cap, int first, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bases of windows group0 .. group0 + n_groups - 1 (one workgroup per
 * window, Z and KV head, fp64), by the randomized range finder with power
 * iterations and a Rayleigh-Ritz step (Halko, Martinsson and Tropp, SIAM
 * Review 2011, §4.5 and §5.3) on the window's Gram matrix C:
 *   1. Y = C Omega            (Omega: the caller's Gaussian sketch)
 *   2. Q = orth(Y)            (Gram-Schmidt twice per column over [Y | I],
 *                              a column skipped when its norm falls to
 *                              2^-40 of its norm before; the first k kept)
 *   3. power_iters times Q = orth(C Q)
 *   4. T = Q^T C Q = U diag(theta) U^T (cyclic Jacobi)
 *   5. the Ritz vectors Q U in decreasing theta (ties: lower index first),
 *      each with its first largest-magnitude entry made positive
 *   6. the first r_max of them, rounded once to fp16, as the basis rows.
 * omega: device fp32 [n_groups][2][num_kv_heads][head_dim][sketch] (Z = K,
 * V); sketch in [r_max, min(head_dim, 72)]; power_iters in [0, 16].  ritz:
 * device fp64 [n_groups][2][num_kv_heads][sketch] (theta in decreasing
 * order), or NULL.
 */
int dwkv_prefill_bases(dwkv_handle *h, int group0, int n_groups, const float *omega, int sketch, int power_iters,
                       double *ritz, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Appends layer's prefill tokens, in position order after the tokens it
 * already holds: token t of sequence b, KV head h is encoded exactly as
 * dwkv_append would encode it (same bits) at tier tier[b][h][t] with gates
 * gate_k/gate_v[b][h][t].  tier: device uint8 [batch][num_kv_heads][n_cap];
 * gate_k, gate_v: device fp16 [batch][num_kv_heads][n_cap] or NULL (a gate
 * of 1).  Admission is per (sequence, KV head), all or nothing: a tier >=
 * num_tiers, a full tier region or a full position map sets the device
 * error word and leaves that (sequence, KV head) unchanged.  The encoder
 * reads the window's bases from a copy in the workspace, which a call
 * makes unless the workspace's last copy was made by this handle, for this
 * window, since its last dwkv_set_basis or dwkv_prefill_bases, and in the
 * same stream capture (or outside any capture, as this call is): a captured
 * graph never relies on a copy made outside it.  Bases written into the
 * arena by other means are not seen by such a reusing call.
 */
int dwkv_prefill_encode(dwkv_handle *h, int layer, const void *k, const void *v, const int32_t *n_tokens, int batch,
                        int64_t n_cap, const void *tier, const void *gate_k, const void *gate_v, void *workspace,
                        size_t workspace_bytes, void *stream);

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
