/*
 * moe_oracle.c -- plain, slow CPU oracle for the fused MoE expert forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or helper with the
 * HIP library; the only thing both sides share is the seeded input generator.
 *
 * Sources (page title, section):
 *   [FG]  "fused_moe.py analysis" (FlagDoc, flaggems/fused_moe.md):
 *         1.1 MoE math, 1.2 routed-item form, 1.3 block GEMM over routed items,
 *         "moe_align_block_size", "fused_moe_kernel" (fp32 accumulator, cast at
 *         the end), "FP8 W8A8" (block-wise scales per K block).
 *   [DG]  "DeepGEMM FusedMoE on Blackwell (vLLM)": 1.1 six-step table,
 *         2.6.1 aligned M bound, 2.6.2 permute / inv_perm, 2.6.4 SwiGLU +
 *         per-128 dynamic quant, 2.6.5 ep_gather (fp32 weighted sum, then cast).
 *   [MK]  "vLLM modular_kernel.py notes" (aicoding.csdn.net): section 3
 *         (fused_topk: softmax then top-k, renormalize flag, fp32 weights,
 *         int32 ids), 7.3.3 (weights sum to 1 when renormalised).
 *
 * Readings where the pages leave a step open (each one is listed with its
 * reason in the design notes):
 *   - top-k is taken on the logits (softmax is strictly increasing); equal
 *     logits go to the lower expert index; slots are in descending order.
 *   - rows [0, I) of w13 are the gate, rows [I, 2I) the up projection;
 *     z = SiLU(gate) * up; no biases.
 *   - apply_router_weight_on_input multiplies z (the second GEMM's input);
 *     the final weighted sum then uses weight 1.
 *   - bf16 rounding (round-to-nearest-even) at h, z, o and y; accumulation
 *     here is in double, so it is the exact sum up to one fp64 rounding.
 *   - padding entries of sorted_token_ids hold R = M*topk; expert_ids beyond
 *     the used blocks hold -1; inside an expert segment routed items ascend.
 *   - fp8: OCP E4M3FN (max 448), scale = amax/448 in fp32, code =
 *     RNE(clamp(v/scale)), an all-zero group gives scale 0 and code 0.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the parallel loops below use (reported beside CPU timings). */
int oracle_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits. */
/* ------------------------------------------------------------------------ */

double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to the nearest bf16, ties to even, directly (one rounding). */
uint16_t oracle_f64_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    /* quantum: spacing of bf16 numbers at the magnitude of a */
    double q;
    if (a >= ldexp(1.0, -126)) {
        int ex;
        frexp(a, &ex); /* a in [2^(ex-1), 2^ex) */
        q = ldexp(1.0, ex - 1 - 7);
    } else {
        q = ldexp(1.0, -133); /* subnormal spacing */
    }
    double r = rint(a / q) * q; /* a/q is exact (power of two); rint = ties-to-even */
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounds above it is inf */
    if (r > ldexp(255.0, 120)) return sign | 0x7F80;
    float rf = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity; */
/* S.1111.111 is NaN; largest finite is 1.75 * 2^8 = 448.                     */
/* ------------------------------------------------------------------------ */

double oracle_e4m3_to_f64(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9)                    /* m/8 * 2^-6 */
                        : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round a float to the nearest e4m3 value, ties to even, saturating at 448. */
uint8_t oracle_f32_to_e4m3(float f)
{
    if (isnan(f)) return 0x7F;
    uint8_t sign = signbit(f) ? 0x80 : 0;
    double a = fabs((double)f);
    double q;
    if (a >= ldexp(1.0, -6)) {
        int ex;
        frexp(a, &ex);
        q = ldexp(1.0, ex - 1 - 3);
    } else {
        q = ldexp(1.0, -9);
    }
    double r = rint(a / q) * q;
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    /* encode r, which is on the e4m3 grid */
    if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));
    int ex;
    double fr = frexp(r, &ex);        /* r = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1 + 7;               /* biased exponent of 1.mmm * 2^(ex-1) */
    int m = (int)((fr * 2.0 - 1.0) * 8.0);
    return sign | (uint8_t)(e << 3) | (uint8_t)m;
}

/* Array forms of the codecs, for the tests. */
void oracle_bf16_to_f64_n(const uint16_t *b, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(b[i]);
}
void oracle_f64_to_bf16_n(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(v[i]);
}
void oracle_e4m3_to_f64_n(const uint8_t *c, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f64(c[i]);
}
void oracle_f32_to_e4m3_n(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(v[i]);
}

/* Dynamic per-group quantisation of n fp32 values, one group per 128 values
 * ([DG] 2.5 / 2.6.4: per-token, per-128-column fp32 scales; [FG] "FP8 W8A8").
 * scale = amax / 448 (fp32 division); code = e4m3(clamp(v / scale)). */
void oracle_quant_groups_fp8(const float *v, int64_t n, uint8_t *q, float *scale)
{
    for (int64_t g = 0; g * 128 < n; ++g) {
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float a = fabsf(v[g * 128 + i]);
            if (a > amax) amax = a;
        }
        float s = amax / 448.0f;
        scale[g] = s;
        for (int i = 0; i < 128; ++i) {
            if (amax == 0.0f) {
                q[g * 128 + i] = 0;
                continue;
            }
            float t = v[g * 128 + i] / s;
            if (t > 448.0f) t = 448.0f;
            if (t < -448.0f) t = -448.0f;
            q[g * 128 + i] = oracle_f32_to_e4m3(t);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MX block scaling ([DG] TL;DR and section 4: MXFP8 1x32 with E8M0 scales on */
/* weights and dynamic activations; W4A8: E2M1 weights with E8M0/32 scales;  */
/* the "UE8M0" / "CEIL_UE8M0" scale formats). E8M0 code c means 2^(c - 127); */
/* 255 is NaN. A block of 32 values takes the smallest power-of-two scale s  */
/* with max|v| <= fmax * s (fmax 448 for E4M3, 6 for E2M1), clamped to the   */
/* E8M0 range; the codes are the element format's RNE(v / s). An all-zero   */
/* block gets code 0 and zero elements.                                      */
/* ------------------------------------------------------------------------ */

static double silu(double g);

double oracle_e8m0_to_f64(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

/* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_to_f64(uint8_t c)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[c & 7];
    return (c & 8) ? -v : v;
}

/* nearest E2M1 value, ties to the even code (mantissa bit 0), saturating at 6 */
uint8_t oracle_f32_to_e2m1(float f)
{
    uint8_t sign = signbit(f) ? 8 : 0;
    double a = fabs((double)f);
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - oracle_e2m1_to_f64((uint8_t)c)), db = fabs(a - oracle_e2m1_to_f64((uint8_t)best));
        if (d < db || (d == db && (c & 1) == 0)) best = c;
    }
    return sign | (uint8_t)best;
}

/* the E8M0 code of the smallest s = 2^e with a <= fmax * s */
static uint8_t mx_scale_code(double a, double fmax)
{
    if (a == 0.0) return 0;
    int e;
    frexp(a / fmax, &e);            /* a / fmax in [2^(e-1), 2^e): the answer is e-1 or e */
    while (e > -127 && a <= fmax * ldexp(1.0, e - 1)) --e;
    while (a > fmax * ldexp(1.0, e)) ++e;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (uint8_t)(e + 127);
}

/* n values (n a multiple of 32) -> E4M3 codes q[n] and E8M0 codes sc[n / 32] */
void oracle_quant_mx_fp8(const float *v, int64_t n, uint8_t *q, uint8_t *sc)
{
    for (int64_t b = 0; b < n / 32; ++b) {
        double a = 0.0;
        for (int i = 0; i < 32; ++i) a = fmax(a, fabs((double)v[b * 32 + i]));
        sc[b] = mx_scale_code(a, 448.0);
        double s = oracle_e8m0_to_f64(sc[b]);
        for (int i = 0; i < 32; ++i)
            q[b * 32 + i] = a == 0.0 ? 0 : oracle_f32_to_e4m3((float)(v[b * 32 + i] / s));
    }
}

/* n values -> E2M1 codes, two per byte (element 2i in the low nibble), and E8M0 scales */
void oracle_quant_mx_fp4(const float *v, int64_t n, uint8_t *q, uint8_t *sc)
{
    for (int64_t b = 0; b < n / 32; ++b) {
        double a = 0.0;
        for (int i = 0; i < 32; ++i) a = fmax(a, fabs((double)v[b * 32 + i]));
        sc[b] = mx_scale_code(a, 6.0);
        double s = oracle_e8m0_to_f64(sc[b]);
        for (int i = 0; i < 32; i += 2) {
            uint8_t lo = a == 0.0 ? 0 : oracle_f32_to_e2m1((float)(v[b * 32 + i] / s));
            uint8_t hi = a == 0.0 ? 0 : oracle_f32_to_e2m1((float)(v[b * 32 + i + 1] / s));
            q[(b * 32 + i) / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* out[n] = bf16( sum over 32-blocks b of (sum_{c in b} qa_c * qw[n, c]) * sa_b * sw[n, b] ),
 * fp64 accumulation. fmt_w 0: E4M3 weights [N, K]; 1: E2M1 weights [N, K/2]. The
 * activation side is E4M3 with E8M0 scales (mx_a = 1), or with one fp32 scale per
 * 128 columns (mx_a = 0, sa holds K/128 floats; W4A8's FP8 activations). */
void oracle_gemm_mx(const uint8_t *qa, const void *sa, int mx_a, const uint8_t *qw, const uint8_t *sw,
                    int fmt_w, int N, int K, uint16_t *out)
{
    for (int n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int b = 0; b < K / 32; ++b) {
            double part = 0.0;
            for (int c = b * 32; c < b * 32 + 32; ++c) {
                double w = fmt_w == 0 ? oracle_e4m3_to_f64(qw[(int64_t)n * K + c])
                                      : oracle_e2m1_to_f64((qw[((int64_t)n * K + c) / 2] >> (4 * (c & 1))) & 15);
                part += oracle_e4m3_to_f64(qa[c]) * w;
            }
            double a_scale = mx_a ? oracle_e8m0_to_f64(((const uint8_t *)sa)[b])
                                  : (double)((const float *)sa)[b / 4];
            acc += part * a_scale * oracle_e8m0_to_f64(sw[(int64_t)n * (K / 32) + b]);
        }
        out[n] = oracle_f64_to_bf16(acc);
    }
}

/* MXFP8 layer: activations and z quantised to MXFP8 per 32 columns; weights E4M3
 * with E8M0 scales [E, N, K/32] ([DG] TL;DR: MXFP8 (1x32), weights and dynamic
 * activations). W4A8 layer (mx_w4 = 1): weights E2M1 [E, N, K/2] with E8M0
 * scales, activations and z as in the FP8 block recipe (E4M3, fp32 scale per
 * 128 columns) ([DG] TL;DR: MXFP4 weights x FP8 activations (128)). */
int oracle_fused_experts_mx(int64_t M, int H, int I, int E, int k, int mx_w4,
                            const uint16_t *x, const uint8_t *w13q, const uint8_t *w13e,
                            const uint8_t *w2q, const uint8_t *w2e,
                            const int32_t *ids, const float *weights, int on_input,
                            int64_t t0, int64_t t1, uint16_t *y, double *acc_out)
{
    (void)M;
    int bad = 0;
    int64_t wb13 = mx_w4 ? (int64_t)I * H : (int64_t)2 * I * H;   /* bytes per expert */
    int64_t wb2 = mx_w4 ? (int64_t)H * I / 2 : (int64_t)H * I;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = t0; t < t1; ++t) {
        float *xf = malloc(sizeof(float) * (size_t)H);
        uint8_t *xq = malloc((size_t)H);
        uint8_t *xs8 = malloc((size_t)(H / 32));
        float *xs = malloc(sizeof(float) * (size_t)(H / 128));
        uint16_t *h = malloc(sizeof(uint16_t) * 2 * (size_t)I);
        float *zf = malloc(sizeof(float) * (size_t)I);
        uint8_t *zq = malloc((size_t)I);
        uint8_t *zs8 = malloc((size_t)(I / 32));
        float *zs = malloc(sizeof(float) * (size_t)(I / 128));
        uint16_t *o = malloc(sizeof(uint16_t) * (size_t)H);
        double *acc = calloc((size_t)H, sizeof(double));
        for (int c = 0; c < H; ++c) xf[c] = (float)oracle_bf16_to_f64(x[t * H + c]);
        if (mx_w4) oracle_quant_groups_fp8(xf, H, xq, xs);
        else oracle_quant_mx_fp8(xf, H, xq, xs8);
        for (int j = 0; j < k; ++j) {
            int e = ids[t * k + j];
            if (e < 0 || e >= E) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            double alpha = weights[t * k + j];
            oracle_gemm_mx(xq, mx_w4 ? (const void *)xs : (const void *)xs8, !mx_w4, w13q + e * wb13,
                           w13e + (int64_t)e * 2 * I * (H / 32), mx_w4, 2 * I, H, h);
            double a1 = on_input ? alpha : 1.0;
            for (int i = 0; i < I; ++i) {
                double g = oracle_bf16_to_f64(h[i]), u = oracle_bf16_to_f64(h[I + i]);
                zf[i] = (float)(a1 * silu(g) * u);
            }
            if (mx_w4) oracle_quant_groups_fp8(zf, I, zq, zs);
            else oracle_quant_mx_fp8(zf, I, zq, zs8);
            oracle_gemm_mx(zq, mx_w4 ? (const void *)zs : (const void *)zs8, !mx_w4, w2q + e * wb2,
                           w2e + (int64_t)e * H * (I / 32), mx_w4, H, I, o);
            double a2 = on_input ? 1.0 : alpha;
            for (int n = 0; n < H; ++n) acc[n] += a2 * oracle_bf16_to_f64(o[n]);
        }
        for (int n = 0; n < H; ++n) {
            y[t * H + n] = oracle_f64_to_bf16(acc[n]);
            if (acc_out) acc_out[t * H + n] = acc[n];
        }
        free(xf); free(xq); free(xs8); free(xs); free(h); free(zf); free(zq); free(zs8); free(zs);
        free(o); free(acc);
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Router ([MK] section 3; [FG] 1.1): p = softmax(s) over all E experts,       */
/* S = TopK(p, k), weights renormalised over S when `renormalize` is set.     */
/* ------------------------------------------------------------------------ */

/* A NaN logit is read as -inf: it ranks below every number, so it is chosen
 * only when fewer than k experts have another value, and then by the
 * lower-index rule; its softmax term is 0. (The pages do not say what a NaN
 * score does; this reading keeps every chosen id in [0, E).) A token whose
 * logits are all NaN or -inf has an undefined softmax: its weights come out
 * NaN from the arithmetic below (exp(-inf - -inf)). */
static void load_scores(const float *logits, int E, float *s)
{
    for (int e = 0; e < E; ++e) s[e] = isnan(logits[e]) ? -INFINITY : logits[e];
}

int oracle_topk(const float *logits, int64_t M, int E, int k, int renormalize,
                int32_t *ids, float *weights)
{
    if (k < 1 || k > E || E > 1024 || k > 64) return 1;
    for (int64_t t = 0; t < M; ++t) {
        float s[1024];
        load_scores(logits + t * E, E, s);
        double smax = -INFINITY;
        for (int e = 0; e < E; ++e)
            if (s[e] > smax) smax = s[e];
        double denom = 0.0;
        for (int e = 0; e < E; ++e) denom += exp((double)s[e] - smax);

        /* k rounds of "largest remaining logit, lowest index on ties" */
        char taken[1024];
        memset(taken, 0, sizeof taken);
        double p[64];
        double psum = 0.0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || s[e] > s[best])) best = e;
            taken[best] = 1;
            ids[t * k + j] = best;
            p[j] = exp((double)s[best] - smax) / denom;
            psum += p[j];
        }
        for (int j = 0; j < k; ++j)
            weights[t * k + j] = (float)(renormalize ? p[j] / psum : p[j]);
    }
    return 0;
}

/* Grouped / sigmoid router ([MK] section 3, fused_topk scoring_func softmax or
 * sigmoid; [MK] 11.x apply_monolithic: num_expert_group, topk_group,
 * e_score_correction_bias, routed_scaling_factor). The pages name the knobs;
 * the steps follow their plain meaning:
 *   1. score u_e: softmax over the E logits, or sigmoid(s_e);
 *   2. selection key: the logit itself (both scores increase with it), or with
 *      a correction bias (sigmoid only) the fp32 sum u_e + b_e, u_e being the
 *      sigmoid evaluated in double and rounded to fp32;
 *   3. groups of E / G consecutive experts; a group's score is its largest key,
 *      or with a bias the fp32 sum of its two largest keys; the topk_group
 *      best groups are kept (ties to the lower group index);
 *   4. the k largest keys among the kept groups' experts, in descending order
 *      (ties to the lower expert index);
 *   5. weights are the unbiased scores u (softmax over all E, or sigmoid),
 *      divided by their sum over the k chosen when `renormalize` is set, then
 *      multiplied by routed_scaling_factor.
 * G = 1 (or topk_group = G) is plain top-k. */
static float sigmoid_f32(float s) { return (float)(1.0 / (1.0 + exp(-(double)s))); }

int oracle_topk_grouped(const float *logits, int64_t M, int E, int k, int scoring,
                        int renormalize, int G, int topk_group, const float *bias,
                        float scale, int32_t *ids, float *weights)
{
    if (k < 1 || E > 1024 || k > 64 || G < 1 || E % G || topk_group < 1 || topk_group > G) return 1;
    int gs = E / G;
    if (k > topk_group * gs || (bias && (scoring != 1 || gs < 2))) return 1;
    for (int64_t t = 0; t < M; ++t) {
        float s[1024];
        load_scores(logits + t * E, E, s);
        float key[1024];
        for (int e = 0; e < E; ++e) key[e] = bias ? sigmoid_f32(s[e]) + bias[e] : s[e];
        char allowed[1024];
        memset(allowed, 0, sizeof allowed);
        char gtaken[1024];
        memset(gtaken, 0, sizeof gtaken);
        for (int r = 0; r < topk_group; ++r) {
            int bg = -1;
            float bscore = 0.0f;
            for (int g = 0; g < G; ++g) {
                if (gtaken[g]) continue;
                float m1 = -INFINITY, m2 = -INFINITY;   /* two largest keys of group g */
                for (int e = g * gs; e < (g + 1) * gs; ++e) {
                    if (key[e] > m1) { m2 = m1; m1 = key[e]; }
                    else if (key[e] > m2) m2 = key[e];
                }
                float score = bias ? m1 + m2 : m1;
                if (bg < 0 || score > bscore) { bg = g; bscore = score; }
            }
            gtaken[bg] = 1;
            for (int e = bg * gs; e < (bg + 1) * gs; ++e) allowed[e] = 1;
        }
        double smax = -INFINITY;
        for (int e = 0; e < E; ++e)
            if (s[e] > smax) smax = s[e];
        double denom = 0.0;
        for (int e = 0; e < E; ++e) denom += exp((double)s[e] - smax);
        double u[64], usum = 0.0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (allowed[e] && (best < 0 || key[e] > key[best])) best = e;
            allowed[best] = 0;
            ids[t * k + j] = best;
            u[j] = scoring == 1 ? (double)sigmoid_f32(s[best]) : exp((double)s[best] - smax) / denom;
            usum += u[j];
        }
        for (int j = 0; j < k; ++j)
            weights[t * k + j] = (float)((renormalize ? u[j] / usum : u[j]) * (double)scale);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Align ([FG] "moe_align_block_size"; [DG] 2.6.1, 2.6.2).                     */
/* ------------------------------------------------------------------------ */

/* Upper bound on the padded row count ([DG] 2.6.1, no per-expert counts on
 * the host): R + min(R, E) * (B - 1), rounded up to B. */
int64_t oracle_align_capacity(int64_t M, int k, int E, int B)
{
    int64_t R = M * k;
    int64_t bound = R + (R < E ? R : E) * (int64_t)(B - 1);
    return (bound + B - 1) / B * B;
}

/* The expert an item is computed with on this shard ([MK] "expert_map": a
 * global-to-local table with -1 for experts held by another rank; [DG] 2.6.2
 * ep_scatter skips items whose expert is not local). Without a map the ids
 * are local already. Returns -2 for an id outside the routing range. */
static int local_expert(int id, const int32_t *emap, int E_global, int E)
{
    if (!emap) return (id < 0 || id >= E) ? -2 : id;
    if (id < 0 || id >= E_global) return -2;
    return emap[id] >= 0 && emap[id] < E ? emap[id] : -1;
}

/* Routed item r = t*k + j. Items are grouped by expert in ascending expert
 * order; each expert's segment holds its items in ascending r, padded with the
 * sentinel R up to a multiple of B. expert_ids[b] is the expert of block b
 * (-1 past the used blocks); inv_perm[r] is the row that item r landed in.
 * With an expert map (emap, E_global entries), ids are global, segments are
 * those of the local experts, and items of remote experts get no row
 * (inv_perm = -1). */
int oracle_align(const int32_t *ids, int64_t M, int k, int E, int B, int64_t cap,
                 const int32_t *emap, int E_global,
                 int32_t *sorted, int32_t *expert_ids, int32_t *npp, int32_t *inv_perm)
{
    int64_t R = M * k;
    int64_t *count = calloc((size_t)E, sizeof(int64_t));
    int64_t *start = calloc((size_t)E + 1, sizeof(int64_t));
    int64_t *fill = calloc((size_t)E, sizeof(int64_t));
    for (int64_t r = 0; r < R; ++r) {
        int e = local_expert(ids[r], emap, E_global, E);
        if (e == -2) { free(count); free(start); free(fill); return 1; }
        if (e >= 0) count[e]++;
    }
    start[0] = 0;
    for (int e = 0; e < E; ++e) start[e + 1] = start[e] + (count[e] + B - 1) / B * B;
    if (start[E] > cap) { free(count); free(start); free(fill); return 2; }
    for (int64_t pos = 0; pos < cap; ++pos) sorted[pos] = (int32_t)R;
    for (int64_t b = 0; b < cap / B; ++b) expert_ids[b] = -1;
    for (int64_t r = 0; r < R; ++r) {
        int e = local_expert(ids[r], emap, E_global, E);
        if (e < 0) { inv_perm[r] = -1; continue; }
        int64_t pos = start[e] + fill[e]++;
        sorted[pos] = (int32_t)r;
        inv_perm[r] = (int32_t)pos;
    }
    for (int e = 0; e < E; ++e)
        for (int64_t b = start[e] / B; b < start[e + 1] / B; ++b) expert_ids[b] = e;
    *npp = (int32_t)start[E];
    free(count); free(start); free(fill);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* One expert applied to one token ([FG] 1.2: h = W1^T x, z = phi(h),          */
/* o = W2^T z; [DG] 1.1 step 7: gated SwiGLU).                                 */
/* ------------------------------------------------------------------------ */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* h[n] = bf16(sum_c x[c] * w13[n, c]), n < 2I */
void oracle_gemm1_bf16(const uint16_t *x, const uint16_t *w13e, int H, int I, uint16_t *h)
{
    for (int n = 0; n < 2 * I; ++n) {
        const uint16_t *w = w13e + (int64_t)n * H;
        double acc = 0.0;
        for (int c = 0; c < H; ++c) acc += oracle_bf16_to_f64(x[c]) * oracle_bf16_to_f64(w[c]);
        h[n] = oracle_f64_to_bf16(acc);
    }
}

/* z[i] = bf16(alpha * SiLU(h[i]) * h[I + i]) */
void oracle_act_bf16(const uint16_t *h, int I, double alpha, uint16_t *z)
{
    for (int i = 0; i < I; ++i) {
        double g = oracle_bf16_to_f64(h[i]), u = oracle_bf16_to_f64(h[I + i]);
        z[i] = oracle_f64_to_bf16(alpha * silu(g) * u);
    }
}

/* o[n] = bf16(sum_i z[i] * w2[n, i]), n < H */
void oracle_gemm2_bf16(const uint16_t *z, const uint16_t *w2e, int H, int I, uint16_t *o)
{
    for (int n = 0; n < H; ++n) {
        const uint16_t *w = w2e + (int64_t)n * I;
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += oracle_bf16_to_f64(z[i]) * oracle_bf16_to_f64(w[i]);
        o[n] = oracle_f64_to_bf16(acc);
    }
}

/* Block-scaled fp8 product ([FG] "FP8 W8A8", block-wise): for each 128-wide K
 * group g, the integer-grid dot product of the codes is scaled by the
 * activation's group scale and the weight block's scale, then summed.
 * out[n] = bf16(sum_g (sum_{c in g} qa[c] * qw[n, c]) * sa[g] * sw[n/128, g]) */
void oracle_gemm_fp8(const uint8_t *qa, const float *sa, const uint8_t *qwe, const float *swe,
                     int N, int K, uint16_t *out)
{
    int G = K / 128;
    for (int n = 0; n < N; ++n) {
        const uint8_t *w = qwe + (int64_t)n * K;
        double acc = 0.0;
        for (int g = 0; g < G; ++g) {
            double part = 0.0;
            for (int c = g * 128; c < g * 128 + 128; ++c)
                part += oracle_e4m3_to_f64(qa[c]) * oracle_e4m3_to_f64(w[c]);
            acc += part * (double)sa[g] * (double)swe[(int64_t)(n / 128) * G + g];
        }
        out[n] = oracle_f64_to_bf16(acc);
    }
}

/* fp8 activation step ([DG] 2.6.4: SwiGLU and dynamic quant in one pass, so z
 * is not rounded to bf16 before it is quantised): zf = fp32(alpha*SiLU(g)*u),
 * then per-128 quantisation. */
void oracle_act_fp8(const uint16_t *h, int I, double alpha, uint8_t *zq, float *zs)
{
    float *zf = malloc(sizeof(float) * (size_t)I);
    for (int i = 0; i < I; ++i) {
        double g = oracle_bf16_to_f64(h[i]), u = oracle_bf16_to_f64(h[I + i]);
        zf[i] = (float)(alpha * silu(g) * u);
    }
    oracle_quant_groups_fp8(zf, I, zq, zs);
    free(zf);
}

/* ------------------------------------------------------------------------ */
/* The layer, per token ([FG] 1.1 / 1.4: y_t = sum over the token's top-k     */
/* slots of alpha_{t,j} * f_{e_{t,j}}(x_t); [DG] 2.6.5: the weighted sum is    */
/* accumulated at high precision and cast to bf16 once).                      */
/* ------------------------------------------------------------------------ */

/* bf16 weights. tokens [t0, t1) of y are written; acc (optional, [M, H]) gets
 * the unrounded weighted sums. With an expert map the weights are the E local
 * experts' and only slots whose expert is local contribute ([DG] 2.6.5:
 * ep_gather skips the slots of experts on other ranks). */
int oracle_fused_experts_bf16(int64_t M, int H, int I, int E, int k,
                              const uint16_t *x, const uint16_t *w13, const uint16_t *w2,
                              const int32_t *ids, const float *weights, int on_input,
                              const int32_t *emap, int E_global,
                              int64_t t0, int64_t t1, uint16_t *y, double *acc_out)
{
    (void)M;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = t0; t < t1; ++t) {
        uint16_t *h = malloc(sizeof(uint16_t) * 2 * (size_t)I);
        uint16_t *z = malloc(sizeof(uint16_t) * (size_t)I);
        uint16_t *o = malloc(sizeof(uint16_t) * (size_t)H);
        double *acc = calloc((size_t)H, sizeof(double));
        for (int j = 0; j < k; ++j) {
            int e = local_expert(ids[t * k + j], emap, E_global, E);
            if (e == -2) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            if (e < 0) continue;  /* computed on another rank */
            double alpha = weights[t * k + j];
            oracle_gemm1_bf16(x + t * H, w13 + (int64_t)e * 2 * I * H, H, I, h);
            oracle_act_bf16(h, I, on_input ? alpha : 1.0, z);
            oracle_gemm2_bf16(z, w2 + (int64_t)e * H * I, H, I, o);
            double a2 = on_input ? 1.0 : alpha;
            for (int n = 0; n < H; ++n) acc[n] += a2 * oracle_bf16_to_f64(o[n]);
        }
        for (int n = 0; n < H; ++n) {
            y[t * H + n] = oracle_f64_to_bf16(acc[n]);
            if (acc_out) acc_out[t * H + n] = acc[n];
        }
        free(h); free(z); free(o); free(acc);
    }
    return bad;
}

/* fp8 W8A8 with 128x128 weight blocks and per-token per-128 activation
 * groups ([DG] 1.1 steps 4-8, 2.6.4; [FG] "FP8 W8A8"). */
int oracle_fused_experts_fp8(int64_t M, int H, int I, int E, int k,
                             const uint16_t *x, const uint8_t *w13q, const float *w13s,
                             const uint8_t *w2q, const float *w2s,
                             const int32_t *ids, const float *weights, int on_input,
                             const int32_t *emap, int E_global,
                             int64_t t0, int64_t t1, uint16_t *y, double *acc_out)
{
    (void)M;
    int bad = 0;
    int64_t s13 = (int64_t)(2 * I / 128) * (H / 128), s2 = (int64_t)(H / 128) * (I / 128);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = t0; t < t1; ++t) {
        float *xf = malloc(sizeof(float) * (size_t)H);
        uint8_t *xq = malloc((size_t)H);
        float *xs = malloc(sizeof(float) * (size_t)(H / 128));
        uint16_t *h = malloc(sizeof(uint16_t) * 2 * (size_t)I);
        uint8_t *zq = malloc((size_t)I);
        float *zs = malloc(sizeof(float) * (size_t)(I / 128));
        uint16_t *o = malloc(sizeof(uint16_t) * (size_t)H);
        double *acc = calloc((size_t)H, sizeof(double));
        for (int c = 0; c < H; ++c) xf[c] = (float)oracle_bf16_to_f64(x[t * H + c]);
        oracle_quant_groups_fp8(xf, H, xq, xs);
        for (int j = 0; j < k; ++j) {
            int e = local_expert(ids[t * k + j], emap, E_global, E);
            if (e == -2) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            if (e < 0) continue;  /* computed on another rank */
            double alpha = weights[t * k + j];
            oracle_gemm_fp8(xq, xs, w13q + (int64_t)e * 2 * I * H, w13s + e * s13, 2 * I, H, h);
            oracle_act_fp8(h, I, on_input ? alpha : 1.0, zq, zs);
            oracle_gemm_fp8(zq, zs, w2q + (int64_t)e * H * I, w2s + e * s2, H, I, o);
            double a2 = on_input ? 1.0 : alpha;
            for (int n = 0; n < H; ++n) acc[n] += a2 * oracle_bf16_to_f64(o[n]);
        }
        for (int n = 0; n < H; ++n) {
            y[t * H + n] = oracle_f64_to_bf16(acc[n]);
            if (acc_out) acc_out[t * H + n] = acc[n];
        }
        free(xf); free(xq); free(xs); free(h); free(zq); free(zs); free(o); free(acc);
    }
    return bad;
}

/* Dense form: every expert is evaluated for every token and weighted by its
 * routing weight, which is 0 for experts outside the token's top-k ([FG] 1.1:
 * unselected experts contribute nothing). Experts are summed in index order. */
int oracle_dense_experts_bf16(int64_t M, int H, int I, int E, int k,
                              const uint16_t *x, const uint16_t *w13, const uint16_t *w2,
                              const int32_t *ids, const float *weights,
                              uint16_t *y, double *acc_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < M; ++t) {
        uint16_t *h = malloc(sizeof(uint16_t) * 2 * (size_t)I);
        uint16_t *z = malloc(sizeof(uint16_t) * (size_t)I);
        uint16_t *o = malloc(sizeof(uint16_t) * (size_t)H);
        double *acc = calloc((size_t)H, sizeof(double));
        for (int e = 0; e < E; ++e) {
            double w = 0.0;
            for (int j = 0; j < k; ++j)
                if (ids[t * k + j] == e) w += weights[t * k + j];
            oracle_gemm1_bf16(x + t * H, w13 + (int64_t)e * 2 * I * H, H, I, h);
            oracle_act_bf16(h, I, 1.0, z);
            oracle_gemm2_bf16(z, w2 + (int64_t)e * H * I, H, I, o);
            for (int n = 0; n < H; ++n) acc[n] += w * oracle_bf16_to_f64(o[n]);
        }
        for (int n = 0; n < H; ++n) {
            y[t * H + n] = oracle_f64_to_bf16(acc[n]);
            if (acc_out) acc_out[t * H + n] = acc[n];
        }
        free(h); free(z); free(o); free(acc);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Batched-experts form ([MK] 6.x, 7.1: after a low-latency dispatch the      */
/* activations arrive as [E, max_M, K], one batch per local expert, with the  */
/* per-expert token counts; [DG] 2.5: the masked grouped GEMM computes only   */
/* the first count rows of each batch, and the combine applies the weights).  */
/* ------------------------------------------------------------------------ */

/* out[e, i] = W2_e(SiLU(G_e a[e, i]) * U_e a[e, i]) in bf16 for i < counts[e]
 * (clamped to max_M), unweighted; other rows are set to 0. Returns 1 if a
 * count is negative. */
int oracle_batched_experts_bf16(int E, int64_t max_M, int H, int I, const uint16_t *a,
                                const int32_t *counts, const uint16_t *w13, const uint16_t *w2,
                                uint16_t *out)
{
    for (int e = 0; e < E; ++e)
        if (counts[e] < 0) return 1;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int e = 0; e < E; ++e) {
        for (int64_t i = 0; i < max_M; ++i) {
            uint16_t *row = out + ((int64_t)e * max_M + i) * H;
            if (i >= counts[e]) {
                for (int n = 0; n < H; ++n) row[n] = 0;
                continue;
            }
            uint16_t *h = malloc(sizeof(uint16_t) * 2 * (size_t)I);
            uint16_t *z = malloc(sizeof(uint16_t) * (size_t)I);
            oracle_gemm1_bf16(a + ((int64_t)e * max_M + i) * H, w13 + (int64_t)e * 2 * I * H, H, I, h);
            oracle_act_bf16(h, I, 1.0, z);
            oracle_gemm2_bf16(z, w2 + (int64_t)e * H * I, H, I, row);
            free(h); free(z);
        }
    }
    return 0;
}

/* The same with e4m3 weights and 128x128 block scales: each row is quantised
 * per 128 columns, and z again after SiLU-and-mul (as in the routed form). */
int oracle_batched_experts_fp8(int E, int64_t max_M, int H, int I, const uint16_t *a,
                               const int32_t *counts, const uint8_t *w13q, const float *w13s,
                               const uint8_t *w2q, const float *w2s, uint16_t *out)
{
    for (int e = 0; e < E; ++e)
        if (counts[e] < 0) return 1;
    int64_t s13 = (int64_t)(2 * I / 128) * (H / 128), s2 = (int64_t)(H / 128) * (I / 128);
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int e = 0; e < E; ++e) {
        for (int64_t i = 0; i < max_M; ++i) {
            uint16_t *row = out + ((int64_t)e * max_M + i) * H;
            if (i >= counts[e]) {
                for (int n = 0; n < H; ++n) row[n] = 0;
                continue;
            }
            const uint16_t *x = a + ((int64_t)e * max_M + i) * H;
            float *xf = malloc(sizeof(float) * (size_t)H);
            uint8_t *xq = malloc((size_t)H);
            float *xs = malloc(sizeof(float) * (size_t)(H / 128));
            uint16_t *h = malloc(sizeof(uint16_t) * 2 * (size_t)I);
            uint8_t *zq = malloc((size_t)I);
            float *zs = malloc(sizeof(float) * (size_t)(I / 128));
            for (int c = 0; c < H; ++c) xf[c] = (float)oracle_bf16_to_f64(x[c]);
            oracle_quant_groups_fp8(xf, H, xq, xs);
            oracle_gemm_fp8(xq, xs, w13q + (int64_t)e * 2 * I * H, w13s + e * s13, 2 * I, H, h);
            oracle_act_fp8(h, I, 1.0, zq, zs);
            oracle_gemm_fp8(zq, zs, w2q + (int64_t)e * H * I, w2s + e * s2, H, I, row);
            free(xf); free(xq); free(xs); free(h); free(zq); free(zs);
        }
    }
    return 0;
}
