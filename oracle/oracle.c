/*
 * CPU oracle for one routed-expert FP4 MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The GPU product
 * shares no code with it: no kernel, header, table or helper.
 *
 * It is the plain definition, slow and obvious: double accumulation, one
 * element at a time, a library sort for the router.  Sources (DeepSeek-V4.1-
 * Flash pages):
 *   - 10100.com page, section on the MoE expert-capacity bottleneck: 384
 *     routed experts per layer, 6 active per token, each with w1/w2/w3 held as
 *     FP4 E2M1 codes (two per byte) plus UE8M0 scales; shapes
 *     w1/w3 [2304, 2560 B] + scale [2304, 160], w2 [5120, 1152 B] + scale
 *     [5120, 72], i.e. one scale byte per 32 consecutive inputs of a row.
 *   - ai-shiz.ru page, section "what the model is": hidden 5120, 384 routed
 *     experts, the router takes 6 per token; one expert is three 5120 x 2304
 *     matrices.
 * Readings where the pages are silent (each is listed in the design notes):
 *   - FFN is SwiGLU: y_e = W2 (silu(W1 x) * (W3 x)), silu(z) = z / (1 + e^-z);
 *   - the hidden activation h is rounded once to bf16 (nearest, ties to even)
 *     after silu(G)*U; G and U are not rounded;
 *   - low nibble of a byte = even element; scale group = 32 consecutive inputs;
 *   - E2M1 code c: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
 *     exponent field 0 is subnormal (0.5 * mantissa);  UE8M0 byte e = 2^(e-127);
 *   - routing: experts ranked by logit descending, ties to the lower index,
 *     -0 equal to +0, NaN below every number; gates are a softmax over the k
 *     selected logits; the output is the gate-weighted sum over the k experts
 *     taken in rank order, applied after w2.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ formats */

/* E2M1 code -> value, from the bit fields of the format. */
double oracle_e2m1(int code) {
    int s = (code >> 3) & 1, E = (code >> 1) & 3, m = code & 1;
    double mag = (E == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);
    return s ? -mag : mag;
}

/* UE8M0 byte -> scale 2^(e-127); 255 is NaN in the OCP MX format. */
double oracle_ue8m0(int e) {
    if (e == 255) return NAN;
    return ldexp(1.0, e - 127);
}

/* bf16 bit pattern -> value */
double oracle_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double straight to bf16 (8 significant bits, round to nearest, ties
 * to even; overflow to inf, NaN kept), return the bit pattern.  One rounding
 * step: never through float, which would round twice. */
uint16_t oracle_double_to_bf16(double v) {
    float f;
    uint32_t u;
    if (isnan(v)) return 0x7FC0;
    if (v == 0.0 || isinf(v)) {
        f = (float)v;
    } else {
        int ex;
        frexp(v, &ex);                    /* |v| = m * 2^ex, m in [0.5, 1) */
        int qexp = ex - 8;                /* 8 significant bits */
        if (qexp < -133) qexp = -133;     /* bf16 subnormal quantum 2^-133 */
        double r = nearbyint(ldexp(v, -qexp)) ;  /* default mode: ties to even */
        double q = ldexp(r, qexp);
        if (fabs(q) >= ldexp(1.0, 128)) q = copysign(INFINITY, v);
        f = (float)q;                     /* exact: q is a bf16 value */
    }
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ MXFP8
 * The optional prefill mode feeds the matrix cores FP8 activations in the OCP
 * MX layout (blocks of 32 values sharing one UE8M0 scale).  Readings: E4M3 as
 * in the OCP FP8 format; the shared exponent is floor(log2(amax)) minus 8, the
 * largest E4M3 exponent; elements round to nearest, ties to even, and saturate
 * to +-448; the sign of a value that rounds to zero is kept. */

/* E4M3 code -> value: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits
 * 2..0; exponent field 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN. */
double oracle_e4m3(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* r -> E4M3 code: round to nearest, ties to even, saturate to 448. */
static int e4m3_code(double r) {
    int s = signbit(r) ? 1 : 0;
    double a = fabs(r), q;
    if (a >= ldexp(1.0, -6)) {
        int e;
        frexp(a, &e);                          /* a in [2^(e-1), 2^e) */
        double quantum = ldexp(1.0, e - 1 - 3); /* 3 mantissa bits */
        q = nearbyint(a / quantum) * quantum;
    } else {
        q = nearbyint(a / ldexp(1.0, -9)) * ldexp(1.0, -9);
    }
    if (q > 448.0) q = 448.0;
    int code;
    if (q == 0.0) {
        code = 0;
    } else if (q < ldexp(1.0, -6)) {
        code = (int)(q / ldexp(1.0, -9));      /* subnormal: m * 2^-9 */
    } else {
        int e;
        frexp(q, &e);                          /* q in [2^(e-1), 2^e) */
        int m = (int)(ldexp(q, -(e - 1)) * 8.0 - 8.0);
        code = ((e - 1 + 7) << 3) | m;
    }
    return (s << 7) | code;
}

/* Quantise n values (n a multiple of 32) to MXFP8 blocks of 32: scales[b] is
 * the UE8M0 byte of block b, codes[i] the E4M3 code of v[i] / 2^(byte - 127).
 * A block of zeros gets byte 0 and zero codes. */
void oracle_mx8_quant(int n, const double *v, uint8_t *codes, uint8_t *scales) {
    for (int b = 0; b < n / 32; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[32 * b + i]));
        int se = 0;
        if (amax > 0.0) {
            int e;
            frexp(amax, &e);                   /* amax in [2^(e-1), 2^e) */
            se = (e - 1) - 8 + 127;
            if (se < 0) se = 0;
            if (se > 254) se = 254;
        }
        scales[b] = (uint8_t)se;
        for (int i = 0; i < 32; ++i) {
            double r = v[32 * b + i] / ldexp(1.0, se - 127);
            codes[32 * b + i] = (uint8_t)e4m3_code(r);
        }
    }
}

/* v <- dequantised MXFP8 of v (in place), blocks of 32. */
static void mx8_round_trip(int n, double *v) {
    uint8_t *c = (uint8_t *)malloc((size_t)n);
    uint8_t *s = (uint8_t *)malloc((size_t)n / 32);
    oracle_mx8_quant(n, v, c, s);
    for (int i = 0; i < n; ++i) v[i] = oracle_e4m3(c[i]) * ldexp(1.0, s[i / 32] - 127);
    free(s);
    free(c);
}

/* ------------------------------------------------------------------ weights */

/* ------------------------------------------------------------------ router */

typedef struct { float v; int e; } okey;

/* Total order of the router: larger logit first, then lower expert index.
 * -0 and +0 compare equal; NaN ranks below everything. */
static int key_cmp(const void *a, const void *b) {
    const okey *x = (const okey *)a, *y = (const okey *)b;
    int xn = isnan(x->v), yn = isnan(y->v);
    if (xn != yn) return xn ? 1 : -1;
    if (!xn) {
        if (x->v > y->v) return -1;
        if (x->v < y->v) return 1;
    }
    return (x->e < y->e) ? -1 : (x->e > y->e);
}

/* Per token: the k best experts by the total order, and gates = softmax over
 * those k logits (computed in double, stored as float). */
void oracle_route(int T, int E, int k, const float *logits, int32_t *idx, float *gates) {
    okey *keys = (okey *)malloc(sizeof(okey) * (size_t)E);
    double *ex = (double *)malloc(sizeof(double) * (size_t)k);
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) { keys[e].v = logits[(size_t)t * E + e]; keys[e].e = e; }
        qsort(keys, (size_t)E, sizeof(okey), key_cmp);
        double l0 = keys[0].v, den = 0.0;
        for (int j = 0; j < k; ++j) {
            idx[(size_t)t * k + j] = keys[j].e;
            ex[j] = exp((double)keys[j].v - l0);
            den += ex[j];
        }
        for (int j = 0; j < k; ++j) gates[(size_t)t * k + j] = (float)(ex[j] / den);
    }
    free(ex);
    free(keys);
}

/* Router logits (the step before routing; the router is one of the layer's
 * resident dense weights, 10100.com page, section on the MoE expert-capacity
 * bottleneck; its format is not given and is read as bf16):
 *   logits[t][e] = sum_c x[t][c] * wr[e][c], x [T][H] and wr [E][H] bf16 bits.
 * Summed in double (bf16 products are exact).  bound[t][e] is the standard
 * bound on an fp32 evaluation of the same sum in any order,
 * gamma_H * sum_c |x[t][c] * wr[e][c]| with gamma_H = H u / (1 - H u),
 * u = 2^-24 (Higham). */
void oracle_router_logits(int T, int H, int E, const uint16_t *x, const uint16_t *wr,
                          double *logits, double *bound) {
    const double u = ldexp(1.0, -24), gam = H * u / (1.0 - H * u);
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double s = 0.0, a = 0.0;
            for (int c = 0; c < H; ++c) {
                const double xv = oracle_bf16_to_double(x[(size_t)t * H + c]);
                const double wv = oracle_bf16_to_double(wr[(size_t)e * H + c]);
                s += xv * wv;
                a += fabs(xv * wv);
            }
            logits[(size_t)t * E + e] = s;
            bound[(size_t)t * E + e] = gam * a;
        }
}

/* Token permutation grouped by expert.  Pair p = t*k + j.  counts[e] = pairs
 * routed to e; offsets = exclusive prefix sum (E+1 entries); sorted_pairs lists
 * pair ids expert by expert, ascending p inside an expert; pair_slot is the
 * inverse (slot of pair p in sorted_pairs). */
void oracle_permute(int T, int E, int k, const int32_t *idx, int32_t *counts, int32_t *offsets,
                    int32_t *sorted_pairs, int32_t *pair_slot) {
    int P = T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int p = 0; p < P; ++p) counts[idx[p]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int s = 0;
    for (int e = 0; e < E; ++e)
        for (int p = 0; p < P; ++p)
            if (idx[p] == e) { sorted_pairs[s] = p; pair_slot[p] = s; ++s; }
}

/* ------------------------------------------------------------------ expert FFN */

typedef struct {
    /* per-expert base pointers of the six tensors (NULL = not provided) */
    const uint8_t **w1, **s1, **w3, **s3, **w2, **s2;
} oracle_weights;

/* Row r of a matrix with `cols` inputs per row, decoded to doubles:
 * out[c] = E2M1(nibble c of row r) * 2^(scale of group c/32 - 127).
 * The element of row r, input c of a [rows][cols/2] nibble tensor with a
 * [rows][cols/32] scale tensor. */
static void decode_row(const uint8_t *w, const uint8_t *s, int cols, int r, double *out) {
    double table[16];
    for (int c = 0; c < 16; ++c) table[c] = oracle_e2m1(c);
    for (int g = 0; g < cols / 32; ++g) {
        double sc = oracle_ue8m0(s[(size_t)r * (cols / 32) + g]);
        for (int c = 32 * g; c < 32 * g + 32; ++c) {
            uint8_t byte = w[(size_t)r * (cols / 2) + (c >> 1)];
            int code = (c & 1) ? (byte >> 4) : (byte & 0xF);
            out[c] = table[code] * sc;
        }
    }
}

/* silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z). */
static double dsilu(double z) {
    const double s = 1.0 / (1.0 + exp(-z));
    return s * (1.0 + z * (1.0 - s));
}

/* How far an fp32 evaluation of h = silu(G) * U can stray from the exact
 * value, when the evaluation's G' and U' are within dG and dU of G and U
 * (acc_bound below).  Then
 *   |silu(G') U' - silu(G) U| <= |silu(G') - silu(G)| |U'| + |silu(G)| |U' - U|
 *                             <= M dG (|U| + dU) + |silu(G)| dU
 * with M the largest |silu'| on [G - dG, G + dG] (mean value theorem).
 * silu' is monotone between its two extremes, at z = +-2.3994 (where
 * z tanh(z/2) = 2), with values 1.0998 and -0.0998; so M is the larger of
 * |silu'| at the two ends, or 1.1 (0.1) if the interval reaches the extreme
 * near +2.4 (-2.4).  The fp32 evaluation of silu(G') U' itself (an
 * exponential within 2 ulps, a division within 2.5 ulps and three more
 * roundings) adds a relative 16 u, u = 2^-24, and an fp32 subnormal result an
 * absolute 2^-149. */
static double h_bound(double G, double U, double dG, double dU) {
    const double u32 = ldexp(1.0, -24);
    const double lo = G - dG, hi = G + dG;
    double M = fmax(fabs(dsilu(lo)), fabs(dsilu(hi)));
    if (lo <= 2.41 && hi >= 2.39) M = fmax(M, 1.1);
    if (lo <= -2.39 && hi >= -2.41) M = fmax(M, 0.1);
    const double silu = G / (1.0 + exp(-G));
    const double e = M * dG * (fabs(U) + dU) + fabs(silu) * dU;
    return e + 16.0 * u32 * (fabs(silu * U) + e) + ldexp(1.0, -149);
}

/* The accumulation model of the fp32 evaluation that an h bound is for:
 * an evaluation of a sum S of exact products p_c (c ascending, as the oracle
 * sums them) is within
 *     sum * A + prefix * P,   A = sum_c |p_c|,
 *                             P = sum_{j >= 1} |p_0 + ... + p_{jB-1}|
 * of S, B = block (P: the magnitudes of the exact partial sums at the block
 * boundaries jB inside the row).  The plain worst case of any summation order
 * is sum = gamma_K = K u / (1 - K u), prefix = 0; an evaluation that takes
 * the inputs in ascending blocks of B, each block through m instructions that
 * err by at most eps relative to the absolute sum of their terms (the
 * accumulator included), satisfies sum = (m + 1) e, prefix = m e with
 * e = eps / (1 - N eps), N instructions in all (the accumulator before an
 * instruction of block j is at most |P_j| + the block's absolute sum away
 * from zero). */
typedef struct {
    double sum, prefix;
    int block;
} oracle_acc;

/* The bound of an evaluation of G (U likewise) under `acc` (NULL, or sum <= 0
 * with prefix <= 0: gamma_K).  A: sum of |terms|; P: prefix mass as above. */
static double acc_bound(const oracle_acc *am, int K, double A, double P) {
    const double u32 = ldexp(1.0, -24);
    if (!am || (am->sum <= 0.0 && am->prefix <= 0.0)) return K * u32 / (1.0 - K * u32) * A;
    return am->sum * A + am->prefix * P;
}

/* Sums of one row: S = sum_c p_c, A = sum_c |p_c| and the prefix mass P for
 * blocks of B (B <= 0: P = 0), all in ascending c, p_c = x_c * w_c. */
static void row_sums(int K, const double *x, const double *w, int B, double *S, double *A, double *P) {
    double s = 0.0, a = 0.0, pm = 0.0;
    for (int c = 0; c < K; ++c) {
        if (B > 0 && c > 0 && c % B == 0) pm += fabs(s);
        s += x[c] * w[c];
        a += fabs(x[c] * w[c]);
    }
    *S = s;
    *A = a;
    *P = pm;
}

/* One token through one expert.
 *   G_n = sum_c x_c W1[n][c],  U_n = sum_c x_c W3[n][c]           (double)
 *   h_n = bf16(silu(G_n) * U_n)                                    (one rounding)
 *   Y_m = sum_n h_n W2[m][n]                                       (double)
 * Sums run over ascending c (resp. n).  hpre (optional) receives silu(G)*U
 * before rounding.  hbound (optional) receives h_bound() of each element, G
 * and U evaluated under the accumulation model `acc` (see oracle_acc). */
static void expert_ffn(int H, int I, const double *x, const uint8_t *w1, const uint8_t *s1,
                       const uint8_t *w3, const uint8_t *s3, const uint8_t *w2, const uint8_t *s2,
                       int mx8, const oracle_acc *am, uint16_t *h, double *hpre, double *hbound,
                       double *Y) {
    const int B = am ? am->block : 0;
    double *hv = (double *)malloc(sizeof(double) * (size_t)I);
    #pragma omp parallel
    {
        double *r1 = (double *)malloc(sizeof(double) * (size_t)H);
        double *r3 = (double *)malloc(sizeof(double) * (size_t)H);
        #pragma omp for schedule(static)
        for (int n = 0; n < I; ++n) {
            decode_row(w1, s1, H, n, r1);
            decode_row(w3, s3, H, n, r3);
            double G, U, Ga, Ua, Gp, Up;
            row_sums(H, x, r1, B, &G, &Ga, &Gp);
            row_sums(H, x, r3, B, &U, &Ua, &Up);
            double a = G / (1.0 + exp(-G)) * U;
            if (hpre) hpre[n] = a;
            if (hbound) hbound[n] = h_bound(G, U, acc_bound(am, H, Ga, Gp), acc_bound(am, H, Ua, Up));
            h[n] = oracle_double_to_bf16(a);
            hv[n] = oracle_bf16_to_double(h[n]);
        }
        free(r3);
        free(r1);
    }
    if (mx8) mx8_round_trip(I, hv);  /* the bf16 h, quantised to MXFP8 along I */
    #pragma omp parallel
    {
        double *r2 = (double *)malloc(sizeof(double) * (size_t)I);
        #pragma omp for schedule(static)
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            decode_row(w2, s2, I, m, r2);
            for (int n = 0; n < I; ++n) acc += hv[n] * r2[n];
            Y[m] = acc;
        }
        free(r2);
    }
    free(hv);
}

/* Forward of the layer for the tokens listed in `tok` (n_tok of them; NULL =
 * all T in order).  Routing and permutation are computed for all T tokens.
 *   x      [T][H] bf16 bits          logits [T][E] float
 *   y      [n_tok][H] float           y[i] = sum_j g[t][j] * Y_(t,j), j ascending
 *   h_out  optional [T*k][I] bf16 (pair order; only pairs of listed tokens set)
 *   hpre   optional [T*k][I] double (same, before rounding)
 *   hbound optional [T*k][I] double (fp32 evaluation bound of hpre, see expert_ffn)
 *   idx, gates optional [T*k] outputs of the router
 * Returns 0, or -1 if a selected expert's weights were not provided. */
static int forward_impl(int T, int H, int I, int E, int k, const uint16_t *x, const float *logits,
                        const oracle_weights *W, int n_tok, const int32_t *tok, float *y,
                        uint16_t *h_out, double *hpre, double *hbound, int32_t *idx_out,
                        float *gates_out, int mx8, const oracle_acc *am) {
    int P = T * k;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
    float *g = (float *)malloc(sizeof(float) * (size_t)P);
    oracle_route(T, E, k, logits, idx, g);
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)P);
    if (gates_out) memcpy(gates_out, g, sizeof(float) * (size_t)P);
    if (tok == NULL) n_tok = T;
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *Y = (double *)malloc(sizeof(double) * (size_t)H);
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
    double *hp = (double *)malloc(sizeof(double) * (size_t)I);
    double *hb = (double *)malloc(sizeof(double) * (size_t)I);
    int rc = 0;
    for (int i = 0; i < n_tok && rc == 0; ++i) {
        int t = tok ? tok[i] : i;
        for (int c = 0; c < H; ++c) xd[c] = oracle_bf16_to_double(x[(size_t)t * H + c]);
        if (mx8) mx8_round_trip(H, xd);  /* x quantised to MXFP8 along H */
        for (int m = 0; m < H; ++m) acc[m] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = idx[(size_t)t * k + j];
            if (!W->w1[e] || !W->s1[e] || !W->w3[e] || !W->s3[e] || !W->w2[e] || !W->s2[e]) {
                rc = -1;
                break;
            }
            expert_ffn(H, I, xd, W->w1[e], W->s1[e], W->w3[e], W->s3[e], W->w2[e], W->s2[e], mx8,
                       am, h, hp, hbound ? hb : NULL, Y);
            size_t p = (size_t)t * k + j;
            if (h_out) memcpy(h_out + p * I, h, sizeof(uint16_t) * (size_t)I);
            if (hpre) memcpy(hpre + p * I, hp, sizeof(double) * (size_t)I);
            if (hbound) memcpy(hbound + p * I, hb, sizeof(double) * (size_t)I);
            double gj = (double)g[p];
            for (int m = 0; m < H; ++m) acc[m] += gj * Y[m];
        }
        for (int m = 0; m < H; ++m) y[(size_t)i * H + m] = (float)acc[m];
    }
    free(hb); free(hp); free(h); free(acc); free(Y); free(xd); free(g); free(idx);
    return rc;
}

/* The layer.  hbound (optional) bounds an evaluation of G and U under the
 * accumulation model `acc` (NULL: gamma_H, see oracle_acc). */
int oracle_forward(int T, int H, int I, int E, int k, const uint16_t *x, const float *logits,
                   const oracle_weights *W, int n_tok, const int32_t *tok, float *y,
                   uint16_t *h_out, double *hpre, double *hbound, int32_t *idx_out,
                   float *gates_out, const oracle_acc *am) {
    return forward_impl(T, H, I, E, k, x, logits, W, n_tok, tok, y, h_out, hpre, hbound, idx_out,
                        gates_out, 0, am);
}

/* The MXFP8 mode: as oracle_forward, with x quantised to MXFP8 along H before
 * w1/w3 and the bf16 h quantised to MXFP8 along I before w2.  hbound as in
 * oracle_forward. */
int oracle_forward_mx8(int T, int H, int I, int E, int k, const uint16_t *x, const float *logits,
                       const oracle_weights *W, int n_tok, const int32_t *tok, float *y,
                       uint16_t *h_out, double *hpre, double *hbound, int32_t *idx_out,
                       float *gates_out, const oracle_acc *am) {
    return forward_impl(T, H, I, E, k, x, logits, W, n_tok, tok, y, h_out, hpre, hbound, idx_out,
                        gates_out, 1, am);
}

/* Expert saliency, the pruning signal of the 10100.com page (section on
 * choosing experts, frequency against saliency): the router weight times the
 * L2 norm of the expert's output, summed over the tokens.  Read as: for each
 * listed expert e, sal[i] = sum over the pairs (t, j) with idx[t][j] = e, t
 * ascending, of g[t][j] * ||Y_(t,j)||_2, with Y the expert's output before the
 * gate (double throughout).  mx8 selects the MXFP8 activations of
 * oracle_forward_mx8.  Returns 0, or -1 if a listed expert's weights are
 * missing. */
int oracle_saliency(int T, int H, int I, int E, int k, const uint16_t *x, const float *logits,
                    const oracle_weights *W, int n_exp, const int32_t *list, double *sal,
                    int mx8) {
    int P = T * k;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
    float *g = (float *)malloc(sizeof(float) * (size_t)P);
    oracle_route(T, E, k, logits, idx, g);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *Y = (double *)malloc(sizeof(double) * (size_t)H);
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
    double *hp = (double *)malloc(sizeof(double) * (size_t)I);
    int rc = 0;
    for (int i = 0; i < n_exp && rc == 0; ++i) {
        int e = list[i];
        sal[i] = 0.0;
        if (!W->w1[e] || !W->s1[e] || !W->w3[e] || !W->s3[e] || !W->w2[e] || !W->s2[e]) {
            rc = -1;
            break;
        }
        for (int p = 0; p < P; ++p) {
            if (idx[p] != e) continue;
            int t = p / k;
            for (int c = 0; c < H; ++c) xd[c] = oracle_bf16_to_double(x[(size_t)t * H + c]);
            if (mx8) mx8_round_trip(H, xd);
            expert_ffn(H, I, xd, W->w1[e], W->s1[e], W->w3[e], W->s3[e], W->w2[e], W->s2[e], mx8,
                       NULL, h, hp, NULL, Y);
            double ss = 0.0;
            for (int m = 0; m < H; ++m) ss += Y[m] * Y[m];
            sal[i] += (double)g[p] * sqrt(ss);
        }
    }
    free(hp); free(h); free(Y); free(xd); free(g); free(idx);
    return rc;
}

/* ------------------------------------------------------------------ shared expert */

/* The shared expert (one per layer beside the 384 routed ones: ai-shiz.ru
 * page, section "what the model is"; kept in FP8 by the 10100.com page, plan
 * two; main weights as FP8 in 32 x 32 blocks, ai-shiz.ru page, same section).
 * Read as: SwiGLU of the routed experts' form with intermediate size I,
 *   W1[n][c] = E4M3(w1[n][c]) * 2^(s1[n/32][c/32] - 127)   w1, w3 [I][H], s1, s3 [I/32][H/32]
 *   W2[m][n] = E4M3(w2[m][n]) * 2^(s2[m/32][n/32] - 127)   w2 [H][I], s2 [H/32][I/32]
 * h = bf16(silu(W1 x) * (W3 x)) rounded once, y_s = W2 h, added to the
 * layer's output without a gate.  y [T][H] double; h, hpre, hbound [T][I]
 * optional, as in expert_ffn, hbound under the accumulation model `acc`
 * (NULL: gamma_H). */
static double fp8w(const uint8_t *w, const uint8_t *s, int cols, int r, int c) {
    const int si = (r / 32) * (cols / 32) + c / 32;
    return oracle_e4m3(w[(size_t)r * cols + c]) * oracle_ue8m0(s[si]);
}

void oracle_shared(int T, int H, int I, const uint16_t *x, const uint8_t *w1, const uint8_t *s1,
                   const uint8_t *w3, const uint8_t *s3, const uint8_t *w2, const uint8_t *s2,
                   double *y, uint16_t *h_out, double *hpre, double *hbound, const oracle_acc *am) {
    const int B = am ? am->block : 0;
    for (int t = 0; t < T; ++t) {
        double *hv = (double *)malloc(sizeof(double) * (size_t)I);
        #pragma omp parallel
        {
        double *xr = (double *)malloc(sizeof(double) * (size_t)H);
        double *r1 = (double *)malloc(sizeof(double) * (size_t)H);
        double *r3 = (double *)malloc(sizeof(double) * (size_t)H);
        for (int c = 0; c < H; ++c) xr[c] = oracle_bf16_to_double(x[(size_t)t * H + c]);
        #pragma omp for schedule(static)
        for (int n = 0; n < I; ++n) {
            for (int c = 0; c < H; ++c) {
                r1[c] = fp8w(w1, s1, H, n, c);
                r3[c] = fp8w(w3, s3, H, n, c);
            }
            double G, U, Ga, Ua, Gp, Up;
            row_sums(H, xr, r1, B, &G, &Ga, &Gp);
            row_sums(H, xr, r3, B, &U, &Ua, &Up);
            const double a = G / (1.0 + exp(-G)) * U;
            const size_t o = (size_t)t * I + n;
            if (hpre) hpre[o] = a;
            if (hbound) hbound[o] = h_bound(G, U, acc_bound(am, H, Ga, Gp), acc_bound(am, H, Ua, Up));
            const uint16_t hb = oracle_double_to_bf16(a);
            if (h_out) h_out[o] = hb;
            hv[n] = oracle_bf16_to_double(hb);
        }
        free(r3);
        free(r1);
        free(xr);
        }
        #pragma omp parallel for schedule(static)
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            for (int n = 0; n < I; ++n)
                acc += hv[n] * fp8w(w2, s2, I, m, n);
            y[(size_t)t * H + m] = acc;
        }
        free(hv);
    }
}

/* Pre-normalisation of the layer stack: u = bf16(x / sqrt(mean(x^2) + eps)). */
void oracle_prenorm(int T, int H, const float *x, double eps, uint16_t *u) {
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int m = 0; m < H; ++m) ss += (double)x[(size_t)t * H + m] * x[(size_t)t * H + m];
        double r = sqrt(ss / H + eps);
        for (int m = 0; m < H; ++m) u[(size_t)t * H + m] = oracle_double_to_bf16(x[(size_t)t * H + m] / r);
    }
}

/* One layer of the residual stack: x <- x + moe(prenorm(x)), float storage.
 * x [T][H] float is updated in place. */
int oracle_stack_layer(int T, int H, int I, int E, int k, float *x, const float *logits,
                       const oracle_weights *W) {
    uint16_t *u = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * H);
    float *y = (float *)malloc(sizeof(float) * (size_t)T * H);
    oracle_prenorm(T, H, x, 1e-6, u);
    int rc = oracle_forward(T, H, I, E, k, u, logits, W, T, NULL, y, NULL, NULL, NULL, NULL, NULL, NULL);
    if (rc == 0)
        for (size_t i = 0; i < (size_t)T * H; ++i) x[i] = (float)((double)x[i] + (double)y[i]);
    free(y);
    free(u);
    return rc;
}

/* Threads the oracle's parallel loops use. */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the threads of the oracle's parallel loops (n >= 1). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
