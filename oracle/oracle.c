/*
 * DepthWeave-KV CPU oracle -- TEST INFRASTRUCTURE, not part of the product.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code with the HIP library: its own
 * fp16 codec, its own loops, no layout of the GPU cache.  It works on the
 * logical (token-position ordered) cache that the seeded input generator
 * produces.
 *
 * What it computes, and from which passage:
 *
 *  oracle_decode -- decode-time attention over the compressed cache.
 *    Reconstruction: DepthWeave-KV paper (arXiv 2607.06523) §3 Method,
 *    Eq. (1): X^_t = A_t B + g R_t for Z in {K, V}; A_t is the token's
 *    coefficient vector at its routed rank (the first r_tier basis vectors),
 *    B the depth window's shared basis, g R_t the gated sparse residual whose
 *    gate is folded into the stored fp16 scale.  Attention: the textbook
 *    softmax attention the zhichai.net summary recalls in Ch. 1.1 and whose
 *    decode procedure Ch. 1.2 gives (query of the new token against every
 *    cached key, weighted sum of the cached values).  Everything is done in
 *    fp64: fp16 inputs are exact in fp64, so the only error is the final
 *    rounding order of fp64 sums.
 *
 *  oracle_materialize -- the Eq. (1) reconstruction of every cached token,
 *    the explicit K^/V^ that a decode without the fused kernel writes out.
 *
 *  oracle_dense_decode -- textbook decode attention over a dense fp16 K/V
 *    cache (the uncompressed baseline).
 *
 *  oracle_encode_tokens -- the prefill's bulk encoding: each token exactly
 *    as one oracle_append (below), tokens independent of one another.
 *
 *  oracle_append -- encoding one new K or V vector into the compressed form
 *    (paper §3 Method, second paragraph: coefficients by projection onto the
 *    current basis; residual kept only on the routed channels, with low-bit
 *    group quantisation).  The pages fix neither the precision nor the order
 *    of operations; this oracle takes the reading that the encoder works in
 *    IEEE fp32 in one fixed order (sequential fused multiply-adds, ascending
 *    index), because the encoding makes integer decisions (which channels,
 *    which codes) that must be identical on both sides:
 *      1. c_i = fp16_rne( sum_j B[i][j] * x_j )            i < r
 *      2. e_j = x_j - sum_i B[i][j] * c_i                  j < d
 *      3. S   = the s channels of largest |e_j| (ties: smaller j first)
 *      4. s16 = fp16_rne( max_{j in S} |e_j| / qmax )
 *      5. v_j = clamp( rint(e_j / s16), -qmax, qmax )     (0 if s16 == 0)
 *      6. stored scale = s16, or fp16_rne(gate * s16) when gate != 1
 *    This file must be compiled with -ffp-contract=off (no implicit fusion).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ fp16 */

/* IEEE binary16 bit pattern -> exact double. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                  /* zero / subnormal */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), ex - 25);    /* 1.man * 2^(ex-15) */
    return sign ? -v : v;
}

/* fp32 -> binary16, round to nearest, ties to even. */
uint16_t oracle_float_to_half(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return sign | 0x7e00;
    double v = fabs((double)f);
    if (v >= 65520.0)                /* halfway to 2^16 and above round to inf */
        return sign | 0x7c00;
    if (v == 0.0)
        return sign;
    int ex;
    frexp(v, &ex);
    int e = ex - 1;                  /* floor(log2 v) */
    if (e < -14)
        e = -14;                     /* subnormal range shares the 2^-24 step */
    double step = ldexp(1.0, e - 10);
    double m = nearbyint(v / step);  /* exact quotient, rounded half-even */
    double r = m * step;
    if (r == 0.0)
        return sign;
    frexp(r, &ex);
    e = ex - 1;
    if (e < -14)
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    uint16_t man = (uint16_t)(r / ldexp(1.0, e - 10) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | man;
}

static float h2f(uint16_t h) { return (float)oracle_half_to_double(h); }

void oracle_half_to_double_array(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_half_to_double(in[i]);
}

void oracle_float_to_half_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_float_to_half(in[i]);
}

/* ---------------------------------------------------------------- decode */

typedef struct oracle_shape {
    int32_t batch, num_q_heads, num_kv_heads, head_dim, r_max, s_max;
    int64_t n_max;                   /* token stride of the logical arrays */
    int32_t num_tiers;
    int32_t tier_rank[8];
    int32_t tier_resid[8];
    int32_t coef_bits;               /* 16: fp16 coefficients; 8: int8 codes times a per-token fp16 scale */
} oracle_shape;

/* Coefficient i of the token whose row starts at element tt * r_max of the
 * coefficient array: fp16, or (8-bit blockwise form, paper §3 second
 * paragraph) the token's fp16 block scale times an int8 code. */
static double coef_at(const oracle_shape *sh, const void *coef, const uint16_t *cscale, int64_t tt, int i)
{
    if (sh->coef_bits == 8)
        return oracle_half_to_double(cscale[tt]) * (double)((const int8_t *)coef)[tt * sh->r_max + i];
    return oracle_half_to_double(((const uint16_t *)coef)[tt * sh->r_max + i]);
}

/* Rebuild one cached vector (K or V) of token tt in fp64 (Eq. (1)).
 * basis: the window's basis already decoded to fp64, [r_max][d]. */
static void reconstruct(const oracle_shape *sh, const double *basis /* [r_max][d] */,
                        const void *coef, const uint16_t *cscale, int64_t tt, const uint8_t *idx,
                        const int8_t *val, uint16_t scale, int tier, double *x /* [d] */)
{
    int d = sh->head_dim;
    int r = sh->tier_rank[tier];
    int s = sh->tier_resid[tier];
    for (int j = 0; j < d; ++j)
        x[j] = 0.0;
    for (int i = 0; i < r; ++i) {
        double c = coef_at(sh, coef, cscale, tt, i);
        const double *bi = basis + (int64_t)i * d;
        for (int j = 0; j < d; ++j)
            x[j] += c * bi[j];
    }
    double g = oracle_half_to_double(scale);
    for (int u = 0; u < s; ++u)
        x[idx[u]] += g * (double)val[u];
}

/*
 * out[b][g][:] for every query head g of the selected (b, KV head) pairs.
 * Query head g reads KV head g / (H_q / H_kv) (contiguous grouping).
 * pairs: NULL for all, else n_pairs (b, h) pairs.  Empty context -> zeros.
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_decode(const oracle_shape *sh, const int64_t *n_tokens, const uint8_t *tier,
                  const uint16_t *basisK, const uint16_t *basisV,
                  const void *coefK, const void *coefV,
                  const uint8_t *idxK, const uint8_t *idxV,
                  const int8_t *valK, const int8_t *valV,
                  const uint16_t *scaleK, const uint16_t *scaleV,
                  const uint16_t *cscaleK, const uint16_t *cscaleV,
                  const uint16_t *q, double alpha, double *out,
                  const int32_t *pairs, int n_pairs, int nthreads)
{
    const int B = sh->batch, Hq = sh->num_q_heads, Hkv = sh->num_kv_heads;
    const int d = sh->head_dim, R = sh->r_max, S = sh->s_max;
    const int64_t NM = sh->n_max;
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || d > 256 || R <= 0 || sh->num_tiers <= 0 ||
        sh->num_tiers > 8)
        return -1;
    const int gq = Hq / Hkv;
    int total = pairs ? n_pairs : B * Hkv;
    int bad = 0;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int p = 0; p < total; ++p) {
        int b = pairs ? pairs[2 * p] : p / Hkv;
        int h = pairs ? pairs[2 * p + 1] : p % Hkv;
        if (b < 0 || b >= B || h < 0 || h >= Hkv) {
            bad = 1;
            continue;
        }
        int64_t n = n_tokens[b];
        double *o = out + ((int64_t)b * Hq + (int64_t)h * gq) * d;
        for (int64_t i = 0; i < (int64_t)gq * d; ++i)
            o[i] = 0.0;
        if (n <= 0)
            continue;
        int64_t base = ((int64_t)b * Hkv + h) * NM;
        double *bK = (double *)malloc(sizeof(double) * (size_t)R * d);
        double *bV = (double *)malloc(sizeof(double) * (size_t)R * d);
        oracle_half_to_double_array(basisK + (int64_t)h * R * d, bK, (int64_t)R * d);
        oracle_half_to_double_array(basisV + (int64_t)h * R * d, bV, (int64_t)R * d);
        double *z = (double *)malloc(sizeof(double) * (size_t)(gq * n));
        double *x = (double *)malloc(sizeof(double) * (size_t)d);
        double *qd = (double *)malloc(sizeof(double) * (size_t)(gq * d));
        for (int g = 0; g < gq; ++g)
            for (int j = 0; j < d; ++j)
                qd[g * d + j] = oracle_half_to_double(q[((int64_t)b * Hq + h * gq + g) * d + j]);

        /* logits z_t = alpha * q . K^_t */
        for (int64_t t = 0; t < n; ++t) {
            int64_t tt = base + t;
            int k = tier[tt];
            if (k >= sh->num_tiers) { bad = 1; k = 0; }
            reconstruct(sh, bK, coefK, cscaleK, tt, idxK + tt * S, valK + tt * S, scaleK[tt], k, x);
            for (int g = 0; g < gq; ++g) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j)
                    acc += qd[g * d + j] * x[j];
                z[g * n + t] = alpha * acc;
            }
        }
        /* softmax weights w_t = exp(z_t - max z), normalised at the end */
        double *mx = (double *)malloc(sizeof(double) * gq);
        double *den = (double *)malloc(sizeof(double) * gq);
        for (int g = 0; g < gq; ++g) {
            double m = -INFINITY;
            for (int64_t t = 0; t < n; ++t)
                if (z[g * n + t] > m) m = z[g * n + t];
            mx[g] = m;
            den[g] = 0.0;
        }
        for (int64_t t = 0; t < n; ++t) {
            int64_t tt = base + t;
            int k = tier[tt];
            if (k >= sh->num_tiers) k = 0;
            reconstruct(sh, bV, coefV, cscaleV, tt, idxV + tt * S, valV + tt * S, scaleV[tt], k, x);
            for (int g = 0; g < gq; ++g) {
                double w = exp(z[g * n + t] - mx[g]);
                den[g] += w;
                for (int j = 0; j < d; ++j)
                    o[g * d + j] += w * x[j];
            }
        }
        for (int g = 0; g < gq; ++g)
            for (int j = 0; j < d; ++j)
                o[g * d + j] /= den[g];
        free(mx); free(den); free(z); free(x); free(qd); free(bK); free(bV);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------- materialisation */

/*
 * Kout, Vout[b][h][t][:] = the Eq. (1) reconstruction of token t (fp64) for
 * t < n_tokens[b], zero beyond; arrays [B][H_kv][n_max][d].  Follows the
 * paper's Eq. (1) (the basis combination of the token's coefficients plus
 * its gated sparse residual), the step a decode without the fused kernel
 * performs before attention (the topic page's Ch. 3.3: base lookup and
 * residual dequantisation as launches of their own).
 */
int oracle_materialize(const oracle_shape *sh, const int64_t *n_tokens, const uint8_t *tier,
                       const uint16_t *basisK, const uint16_t *basisV,
                       const void *coefK, const void *coefV,
                       const uint8_t *idxK, const uint8_t *idxV,
                       const int8_t *valK, const int8_t *valV,
                       const uint16_t *scaleK, const uint16_t *scaleV,
                       const uint16_t *cscaleK, const uint16_t *cscaleV,
                       double *Kout, double *Vout, int nthreads)
{
    const int B = sh->batch, Hkv = sh->num_kv_heads;
    const int d = sh->head_dim, R = sh->r_max, S = sh->s_max;
    const int64_t NM = sh->n_max;
    if (Hkv <= 0 || d <= 0 || d > 256 || R <= 0 || sh->num_tiers <= 0 || sh->num_tiers > 8)
        return -1;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int p = 0; p < B * Hkv; ++p) {
        int b = p / Hkv, h = p % Hkv;
        int64_t base = ((int64_t)b * Hkv + h) * NM;
        double *bK = (double *)malloc(sizeof(double) * (size_t)R * d);
        double *bV = (double *)malloc(sizeof(double) * (size_t)R * d);
        oracle_half_to_double_array(basisK + (int64_t)h * R * d, bK, (int64_t)R * d);
        oracle_half_to_double_array(basisV + (int64_t)h * R * d, bV, (int64_t)R * d);
        for (int64_t t = 0; t < NM; ++t) {
            double *xk = Kout + (base + t) * d, *xv = Vout + (base + t) * d;
            if (t >= n_tokens[b]) {
                for (int j = 0; j < d; ++j)
                    xk[j] = xv[j] = 0.0;
                continue;
            }
            int64_t tt = base + t;
            int k = tier[tt];
            if (k >= sh->num_tiers) { bad = 1; k = 0; }
            reconstruct(sh, bK, coefK, cscaleK, tt, idxK + tt * S, valK + tt * S, scaleK[tt], k, xk);
            reconstruct(sh, bV, coefV, cscaleV, tt, idxV + tt * S, valV + tt * S, scaleV[tt], k, xv);
        }
        free(bK); free(bV);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------ dense decode */

/*
 * Textbook decode attention over a dense fp16 cache (the uncompressed
 * baseline the paper compares against, §4): out[b][g][:] =
 * sum_t softmax_t(alpha q_g . K_t) V_t over t < n_tokens[b], query head g
 * reading KV head g / (H_q / H_kv).  K, V fp16 [B][H_kv][n_max][d] token
 * rows; q fp16 [B][H_q][d]; out fp64.  Empty context -> zeros.  Every sum
 * in fp64.
 */
int oracle_dense_decode(int B, int Hq, int Hkv, int d, int64_t n_max, const int64_t *n_tokens,
                        const uint16_t *K, const uint16_t *V, const uint16_t *q, double alpha,
                        double *out, int nthreads)
{
    if (B <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || d > 256)
        return -1;
    const int gq = Hq / Hkv;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int p = 0; p < B * Hq; ++p) {
        int b = p / Hq, g = p % Hq, h = g / gq;
        int64_t n = n_tokens[b];
        double *o = out + (int64_t)p * d;
        for (int j = 0; j < d; ++j)
            o[j] = 0.0;
        if (n <= 0)
            continue;
        const uint16_t *Kb = K + ((int64_t)b * Hkv + h) * n_max * d;
        const uint16_t *Vb = V + ((int64_t)b * Hkv + h) * n_max * d;
        double qd[256];
        for (int j = 0; j < d; ++j)
            qd[j] = oracle_half_to_double(q[(int64_t)p * d + j]);
        double *z = (double *)malloc(sizeof(double) * (size_t)n);
        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += qd[j] * oracle_half_to_double(Kb[t * d + j]);
            z[t] = alpha * acc;
            if (z[t] > m) m = z[t];
        }
        double den = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            double w = exp(z[t] - m);
            den += w;
            for (int j = 0; j < d; ++j)
                o[j] += w * oracle_half_to_double(Vb[t * d + j]);
        }
        for (int j = 0; j < d; ++j)
            o[j] /= den;
        free(z);
    }
    return 0;
}

/* ---------------------------------------------------------------- append */

/*
 * Encode one fp16 vector x[d] against basis[r_max][d] at rank r with s
 * residual channels and range qmax (7 for 4-bit, 127 for 8-bit codes).
 * gate: fp16 bit pattern of the residual gate (0x3c00 = 1).
 * Outputs: c_out[r] fp16 bits, idx_out[s] ascending, val_out[s], *scale_out
 * fp16 bits (0 when s == 0).  Returns 0, or -1 on an invalid argument.
 */
/* Steps 1-2: the coefficients (fp16 when coef_bits is 16; else int8 codes
 * in c8 with one fp16 block scale *cs16) -- and, if sum is not NULL, the
 * fp32 projection sums they come from -- and the fp32 residual e[d] against
 * the stored coefficients. */
static void project(int d, const uint16_t *basis, const uint16_t *x, int r, int coef_bits, uint16_t *c16,
                    int8_t *c8, uint16_t *cs16, float *sum, float *e)
{
    float c[256], acc1[256];
    for (int i = 0; i < r; ++i) {
        float acc = 0.0f;                                         /* step 1 */
        for (int j = 0; j < d; ++j)
            acc = fmaf(h2f(basis[(int64_t)i * d + j]), h2f(x[j]), acc);
        if (sum)
            sum[i] = acc;
        acc1[i] = acc;
    }
    if (coef_bits == 8) {
        /* 8-bit blockwise form: one block per token; scale = fp16(max |sum| /
         * 127), codes rint(sum / scale) in [-127, 127] (0 for a zero scale);
         * the stored coefficient is code * scale, exact in fp32 */
        float amax = 0.0f;
        for (int i = 0; i < r; ++i)
            if (fabsf(acc1[i]) > amax) amax = fabsf(acc1[i]);
        *cs16 = oracle_float_to_half(amax / 127.0f);
        float sf = h2f(*cs16);
        for (int i = 0; i < r; ++i) {
            float q = 0.0f;
            if (sf != 0.0f) {
                q = rintf(acc1[i] / sf);
                if (q > 127.0f) q = 127.0f;
                if (q < -127.0f) q = -127.0f;
            }
            c8[i] = (int8_t)q;
            c[i] = q * sf;
        }
    } else {
        for (int i = 0; i < r; ++i) {
            c16[i] = oracle_float_to_half(acc1[i]);
            c[i] = h2f(c16[i]);
        }
    }
    for (int j = 0; j < d; ++j) {
        float acc = 0.0f;                                         /* step 2 */
        for (int i = 0; i < r; ++i)
            acc = fmaf(h2f(basis[(int64_t)i * d + j]), c[i], acc);
        e[j] = h2f(x[j]) - acc;
    }
}

/*
 * Encode one fp16 vector x[d] against basis[r_max][d] at rank r with s
 * residual channels and range qmax (7 for 4-bit, 127 for 8-bit codes).
 * gate: fp16 bit pattern of the residual gate (0x3c00 = 1).
 * Outputs: c_out[r] fp16 bits, idx_out[s] ascending, val_out[s], *scale_out
 * fp16 bits (0 when s == 0).  Returns 0, or -1 on an invalid argument.
 */
int oracle_append_ex(int d, int r_max, const uint16_t *basis, const uint16_t *x, int r, int s,
                     int qmax, uint16_t gate, int coef_bits, void *c_out, uint16_t *cscale_out,
                     uint8_t *idx_out, int8_t *val_out, uint16_t *scale_out)
{
    if (d <= 0 || d > 256 || r < 0 || r > r_max || s < 0 || s > d || qmax <= 0 ||
        (coef_bits != 8 && coef_bits != 16))
        return -1;
    float e[256];
    uint16_t cs = 0;
    project(d, basis, x, r, coef_bits, (uint16_t *)c_out, (int8_t *)c_out, &cs, NULL, e);
    if (cscale_out)
        *cscale_out = cs;
    *scale_out = 0;
    if (s == 0)
        return 0;
    /* 3. the s largest |e_j|; a strict '>' keeps the smaller j on ties */
    char taken[256];
    memset(taken, 0, sizeof taken);
    int first = -1;
    for (int u = 0; u < s; ++u) {
        int best = -1;
        for (int j = 0; j < d; ++j) {
            if (taken[j]) continue;
            if (best < 0 || fabsf(e[j]) > fabsf(e[best]))
                best = j;
        }
        taken[best] = 1;
        if (u == 0) first = best;
    }
    /* 4. one fp16 scale for the group of kept channels */
    float amax = fabsf(e[first]);
    uint16_t s16 = oracle_float_to_half(amax / (float)qmax);
    float sf = h2f(s16);
    /* 5. integer codes, stored in ascending channel order */
    int u = 0;
    for (int j = 0; j < d; ++j) {
        if (!taken[j]) continue;
        float v = 0.0f;
        if (sf != 0.0f) {
            v = rintf(e[j] / sf);
            if (v > (float)qmax) v = (float)qmax;
            if (v < -(float)qmax) v = -(float)qmax;
        }
        idx_out[u] = (uint8_t)j;
        val_out[u] = (int8_t)v;
        ++u;
    }
    /* 6. gate folded into the stored scale */
    if (gate == 0x3c00)
        *scale_out = s16;
    else
        *scale_out = oracle_float_to_half(h2f(gate) * sf);
    return 0;
}

int oracle_append(int d, int r_max, const uint16_t *basis, const uint16_t *x, int r, int s,
                  int qmax, uint16_t gate, uint16_t *c_out, uint8_t *idx_out, int8_t *val_out,
                  uint16_t *scale_out)
{
    return oracle_append_ex(d, r_max, basis, x, r, s, qmax, gate, 16, c_out, NULL, idx_out, val_out,
                            scale_out);
}

/* Residual vector e of step 2 (for the quantisation-bound checks). */
int oracle_append_residual(int d, int r_max, const uint16_t *basis, const uint16_t *x, int r,
                           float *e_out)
{
    if (d <= 0 || d > 256 || r < 0 || r > r_max)
        return -1;
    uint16_t c16[256];
    project(d, basis, x, r, 16, c16, NULL, NULL, NULL, e_out);
    return 0;
}

/* Residual e of step 2 for either coefficient form (coef_bits 16 or 8). */
int oracle_append_residual_ex(int d, int r_max, const uint16_t *basis, const uint16_t *x, int r, int coef_bits,
                              float *e_out)
{
    if (d <= 0 || d > 256 || r < 0 || r > r_max || (coef_bits != 8 && coef_bits != 16))
        return -1;
    uint16_t c16[256], cs;
    int8_t c8[256];
    project(d, basis, x, r, coef_bits, c16, c8, &cs, NULL, e_out);
    return 0;
}

/* The fp32 sums of step 1 before their fp16 rounding (for the checks of the
 * fixed operation order). */
int oracle_append_projection(int d, int r_max, const uint16_t *basis, const uint16_t *x, int r,
                             float *sum_out)
{
    if (d <= 0 || d > 256 || r < 0 || r > r_max)
        return -1;
    uint16_t c16[256];
    float e[256];
    project(d, basis, x, r, 16, c16, NULL, NULL, sum_out, e);
    return 0;
}

/*
 * Bulk encoding of prefill tokens (paper §3 Method, the data-path paragraph
 * with Fig. 2: during prefill every cached vector is projected onto its
 * window's basis and its residual quantised at the routed channel count).
 * The prefill holds no arithmetic of its own: token u of the count vectors
 * x[u][d] is encoded exactly as one append (oracle_append_ex) at rank
 * ranks[u], resid[u] kept channels and gate gates[u] (NULL: a gate of 1).
 * Outputs per token, at strides r_stride / s_stride: c_out (fp16 bits, or
 * int8 codes with coef_bits 8), cs_out (block scales, 8-bit form only),
 * idx_out, val_out, scale_out.  Returns 0, or -1 if any token's arguments
 * are invalid.
 */
int oracle_encode_tokens(int d, int r_max, const uint16_t *basis, int64_t count, const uint16_t *x,
                         const int32_t *ranks, const int32_t *resid, const uint16_t *gates, int qmax,
                         int coef_bits, int r_stride, int s_stride, void *c_out, uint16_t *cs_out,
                         uint8_t *idx_out, int8_t *val_out, uint16_t *scale_out, int nthreads)
{
    if (coef_bits != 8 && coef_bits != 16)
        return -1;
    const int eb = coef_bits / 8;
    int bad = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : bad)
#endif
    for (int64_t u = 0; u < count; ++u) {
        if (ranks[u] > r_stride || resid[u] > s_stride) {
            bad |= 1;
            continue;
        }
        uint8_t *c = (uint8_t *)c_out + u * r_stride * eb;
        const int rc = oracle_append_ex(d, r_max, basis, x + u * d, ranks[u], resid[u], qmax,
                                        gates ? gates[u] : (uint16_t)0x3c00, coef_bits, c,
                                        cs_out ? cs_out + u : NULL, idx_out + u * s_stride,
                                        val_out + u * s_stride, scale_out + u);
        bad |= rc != 0;
    }
    return bad ? -1 : 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
