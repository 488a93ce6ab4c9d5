/*
 * Plain, slow, obviously correct CPU oracle for the small-batch MoE decode
 * layer.  TEST INFRASTRUCTURE ONLY: it is built and called by the test suite,
 * by the smoke check and by the benchmark's CPU-baseline leg, never by the
 * product path.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (warp-decode write-ups: "Better MoE model inference with
 * warp decode", TL;DR and section "How the two kernels work"; the Chinese
 * summary "Cursor推出MoE推理加速方法Warp Decode", section 技术原理 with its
 * Gate/Up and Down kernel subsections):
 *
 *     y[b] = sum_k w[b,k] * Down_e( SiLU(Gate_e x[b]) (.) Up_e x[b] ),  e = ids[b,k]
 *
 * with MXFP8 weights (E4M3 codes, one E8M0 scale per 32 elements along the
 * reduction axis), BF16 activations and the intermediate written once as BF16
 * between the gate/up and the down projection.  The warp-decode method reaches
 * this plain result by reordering the sums (the router weight commutes into the
 * accumulator by linearity: Key claims, section "How the two kernels work", and
 * the summary's "Why it's interesting"); the oracle therefore writes out the
 * plain definition, in FP64, summing in index order:
 *
 *   deq(c, s)     = E4M3(c) * 2^(s - 127)                      (exact in FP64)
 *   g[b,k,j]      = sum_h deq(Wgu[e,j,h],   Sgu[e,j,h/32])   * x[b,h]
 *   u[b,k,j]      = sum_h deq(Wgu[e,I+j,h], Sgu[e,I+j,h/32]) * x[b,h]
 *   act[b,k,j]    = BF16_RNE( FP32_RNE( g * sigmoid(g) * u ) )
 *   y[b,h]        = sum_k w[b,k] * sum_i deq(Wd[e,h,i], Sd[e,h,i/32]) * act[b,k,i]
 *
 * The router that produces topk_ids / topk_w from logits is oracle_route
 * (end of file).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - gate rows are 0..I-1 and up rows I..2I-1 of the [E,2I,H] tensor;
 *   - MXFP8 is OCP MX: E4M3 "FN" elements (no infinities, S.1111.111 = NaN,
 *     max 448), E8M0 scales 2^(s-127) with s = 255 = NaN;
 *   - the intermediate is an FP32 value rounded to BF16, nearest-even;
 *   - the router weight is used as given (no renormalisation);
 *   - y is returned unrounded (FP64); callers may round it to BF16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element formats ------------------------------------------------- */

/* OCP 8-bit floating point, E4M3 "FN": sign bit 7, exponent bits 6..3 with
 * bias 7, mantissa bits 2..0.  Exponent field 0 is subnormal m/8 * 2^-6.
 * Exponent 15 with mantissa 7 is NaN; there is no infinity. */
double oracle_e4m3_value(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* OCP E8M0 scale: an unsigned biased exponent, value 2^(s-127); 255 is NaN. */
double oracle_e8m0_value(uint8_t s) {
    if (s == 0xFF) return NAN;
    return ldexp(1.0, (int)s - 127);
}

void oracle_e4m3_table(double *out) { for (int c = 0; c < 256; ++c) out[c] = oracle_e4m3_value((uint8_t)c); }
void oracle_e8m0_table(double *out) { for (int s = 0; s < 256; ++s) out[s] = oracle_e8m0_value((uint8_t)s); }

/* One MXFP8 element: code times block scale (a product of two powers-of-two
 * scaled small integers, exact in FP64). */
double oracle_dequant(uint8_t code, uint8_t scale) {
    return oracle_e4m3_value(code) * oracle_e8m0_value(scale);
}

/* ---- BF16 ------------------------------------------------------------- */

double oracle_bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* FP64 -> FP32, round to nearest even (the C conversion under the default
 * rounding mode). */
float oracle_round_f32(double v) { return (float)v; }

/* FP32 -> BF16 by round-to-nearest-even on the 16 dropped bits.  NaN maps to
 * a quiet NaN with the same sign; overflow past the largest finite BF16 goes
 * to infinity, as IEEE rounding does. */
uint16_t oracle_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16, lower = u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
    return (uint16_t)upper;
}

/* SiLU(g) = g * sigmoid(g), sigmoid evaluated without overflow. */
double oracle_silu(double g) {
    if (g >= 0) return g / (1.0 + exp(-g));
    double t = exp(g);
    return g * t / (1.0 + t);
}

/* ---- the layer -------------------------------------------------------- */

static int check(const int32_t *ids, int B, int K, int E, int H, int I) {
    if (B < 0 || K < 1 || E < 1 || H < 32 || I < 32 || H % 32 || I % 32) return -2;
    for (long t = 0; t < (long)B * K; ++t)
        if (ids[t] < 0 || ids[t] >= E) return -3;
    return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Gate/up projection and activation.  act[B,K,I] receives BF16 bits;
 * gate/up (optional, may be NULL) receive the FP64 dot products g and u. */
int oracle_gate_up(const uint16_t *x, const int32_t *ids,
                   const uint8_t *wgu, const uint8_t *sgu,
                   int B, int K, int E, int H, int I,
                   uint16_t *act, double *gate, double *up, int nthreads) {
    int rc = check(ids, B, K, E, H, I);
    if (rc) return rc;
    set_threads(nthreads);
    const long nb = H / 32;
    long total = (long)B * K * I;
#pragma omp parallel for schedule(static)
    for (long t = 0; t < total; ++t) {
        long b = t / ((long)K * I), k = (t / I) % K, j = t % I;
        long e = ids[b * K + k];
        const uint8_t *cg = wgu + (e * 2 * I + j) * (long)H;
        const uint8_t *cu = wgu + (e * 2 * I + I + j) * (long)H;
        const uint8_t *sg = sgu + (e * 2 * I + j) * nb;
        const uint8_t *su = sgu + (e * 2 * I + I + j) * nb;
        double g = 0.0, u = 0.0;
        for (long h = 0; h < H; ++h) {
            double xv = oracle_bf16_value(x[b * H + h]);
            g += oracle_dequant(cg[h], sg[h / 32]) * xv;
            u += oracle_dequant(cu[h], su[h / 32]) * xv;
        }
        double a = oracle_silu(g) * u;
        act[t] = oracle_bf16_rne(oracle_round_f32(a));
        if (gate) gate[t] = g;
        if (up) up[t] = u;
    }
    return 0;
}

/* Weighted down projection of a given intermediate act[B,K,I] (BF16 bits). */
int oracle_down(const uint16_t *act, const int32_t *ids, const float *w,
                const uint8_t *wd, const uint8_t *sd,
                int B, int K, int E, int H, int I, double *y, int nthreads) {
    int rc = check(ids, B, K, E, H, I);
    if (rc) return rc;
    set_threads(nthreads);
    const long nb = I / 32;
    long total = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long t = 0; t < total; ++t) {
        long b = t / H, h = t % H;
        double acc = 0.0;
        for (long k = 0; k < K; ++k) {
            long e = ids[b * K + k];
            const uint8_t *c = wd + (e * H + h) * (long)I;
            const uint8_t *s = sd + (e * H + h) * nb;
            const uint16_t *a = act + (b * K + k) * (long)I;
            double part = 0.0;
            for (long i = 0; i < I; ++i)
                part += oracle_dequant(c[i], s[i / 32]) * oracle_bf16_value(a[i]);
            acc += (double)w[b * K + k] * part;
        }
        y[t] = acc;
    }
    return 0;
}

/* Whole layer: gate/up, then down on the oracle's own intermediate.
 * act (optional scratch [B,K,I] bits) may be NULL only if B*K*I == 0. */
int oracle_moe_decode(const uint16_t *x, const int32_t *ids, const float *w,
                      const uint8_t *wgu, const uint8_t *sgu,
                      const uint8_t *wd, const uint8_t *sd,
                      int B, int K, int E, int H, int I,
                      uint16_t *act, double *y, int nthreads) {
    int rc = oracle_gate_up(x, ids, wgu, sgu, B, K, E, H, I, act, 0, 0, nthreads);
    if (rc) return rc;
    return oracle_down(act, ids, w, wd, sd, B, K, E, H, I, y, nthreads);
}

/* ---- accuracy experiment ----------------------------------------------

 * The warp-decode write-ups claim their output is 1.4x closer to a full
 * FP32 reference than the conventional path's, because the conventional
 * path rounds BF16 activations to MXFP8 and back (the English summary, Key claims,
 * "Improved accuracy"; the Chinese summary, section 性能与精度 2), and writes
 * per-expert outputs to a BF16 buffer that a combine step sums (the English summary,
 * "Buffer elimination").  These functions give the reference and the
 * conventional path's numerics in FP64. */

/* Nearest E4M3 "FN" code of a value already limited to |v| <= 448 (OCP 8-bit
 * FP: subnormal step 2^-9 below 2^-6, 3 mantissa bits above), ties to even. */
uint8_t oracle_e4m3_encode(double v) {
    if (v != v) return 0x7F;
    uint8_t sign = v < 0 ? 0x80 : 0x00;
    double a = fabs(v);
    if (a > 448.0) a = 448.0;
    if (a < ldexp(1.0, -6)) {                       /* subnormal: m * 2^-9, m = 0..8 */
        double q = a / ldexp(1.0, -9);
        double m = floor(q);
        double r = q - m;
        if (r > 0.5 || (r == 0.5 && fmod(m, 2.0) == 1.0)) m += 1.0;
        if (m >= 8.0) return sign | 0x08;           /* rounds up to the smallest normal 2^-6 */
        return sign | (uint8_t)m;
    }
    int e;
    double f = frexp(a, &e);                        /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;                                          /* a = (2f) * 2^e, 2f in [1, 2) */
    double q = (2.0 * f - 1.0) * 8.0;               /* mantissa in eighths */
    double m = floor(q);
    double r = q - m;
    if (r > 0.5 || (r == 0.5 && fmod(m, 2.0) == 1.0)) m += 1.0;
    if (m >= 8.0) { m = 0.0; e += 1; }
    if (e > 8 || (e == 8 && m > 6.0)) return sign | 0x7E;   /* saturate at 448 */
    return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* OCP MX quantization of n values (n a multiple of 32): per 32-block the
 * shared exponent floor(log2 amax) - 8 (E4M3's largest binade), stored biased
 * by 127 and clamped to [0, 254]; an all-zero block gets byte 0.  Elements
 * are v / 2^shared, limited to +-448 and rounded to the nearest E4M3. */
void oracle_mxfp8_quantize(const double *v, long n, uint8_t *codes, uint8_t *scales) {
    for (long blk = 0; blk < n / 32; ++blk) {
        const double *p = v + blk * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(p[i]));
        int sb = 0;
        if (amax > 0.0) {
            int ex;
            frexp(amax, &ex);
            sb = (ex - 1) - 8 + 127;
            if (sb < 0) sb = 0;
            if (sb > 254) sb = 254;
        }
        scales[blk] = (uint8_t)sb;
        for (int i = 0; i < 32; ++i) codes[blk * 32 + i] = oracle_e4m3_encode(ldexp(p[i], -(sb - 127)));
    }
}

/* Reference: the layer in FP64 with the exact MXFP8 weights and the given x,
 * no rounding of the intermediate or the output. */
int oracle_moe_decode_exact(const uint16_t *x, const int32_t *ids, const float *w,
                            const uint8_t *wgu, const uint8_t *sgu, const uint8_t *wd, const uint8_t *sd,
                            int B, int K, int E, int H, int I, double *y, int nthreads) {
    int rc = check(ids, B, K, E, H, I);
    if (rc) return rc;
    set_threads(nthreads);
    const long nbh = H / 32, nbi = I / 32;
#pragma omp parallel for schedule(static)
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < H; ++h) y[b * H + h] = 0.0;
        for (long k = 0; k < K; ++k) {
            long e = ids[b * K + k];
            double wk = (double)w[b * K + k];
            for (long j = 0; j < I; ++j) {
                const uint8_t *cg = wgu + (e * 2 * I + j) * (long)H, *cu = wgu + (e * 2 * I + I + j) * (long)H;
                const uint8_t *sg = sgu + (e * 2 * I + j) * nbh, *su = sgu + (e * 2 * I + I + j) * nbh;
                double g = 0.0, u = 0.0;
                for (long h = 0; h < H; ++h) {
                    double xv = oracle_bf16_value(x[b * H + h]);
                    g += oracle_dequant(cg[h], sg[h / 32]) * xv;
                    u += oracle_dequant(cu[h], su[h / 32]) * xv;
                }
                double a = oracle_silu(g) * u;
                for (long h = 0; h < H; ++h)
                    y[b * H + h] += wk * oracle_dequant(wd[(e * H + h) * (long)I + j], sd[(e * H + h) * nbi + j / 32]) * a;
            }
        }
    }
    return 0;
}

/* The conventional path's numerics: x rounded to MXFP8 (per 32 along H)
 * before the gate/up projection; the intermediate rounded to BF16 and then
 * to MXFP8 (per 32 along I) before the down projection; each expert's output
 * rounded to BF16 (the per-expert buffer); the combine sums w_k times those
 * in FP64 and the result is rounded to BF16.  y receives that BF16 value. */
int oracle_moe_decode_conventional(const uint16_t *x, const int32_t *ids, const float *w,
                                   const uint8_t *wgu, const uint8_t *sgu, const uint8_t *wd,
                                   const uint8_t *sd, int B, int K, int E, int H, int I, double *y,
                                   int nthreads) {
    int rc = check(ids, B, K, E, H, I);
    if (rc) return rc;
    set_threads(nthreads);
    const long nbh = H / 32, nbi = I / 32;
    if (H > 8192 || I > 16384) return -2;
    int bad_alloc = 0;
#pragma omp parallel for schedule(static) reduction(| : bad_alloc)
    for (long b = 0; b < B; ++b) {
        double *xv = malloc(sizeof(double) * (size_t)(2 * H + 2 * I));
        uint8_t *xc = malloc((size_t)(H + H / 32 + I + I / 32));
        if (!xv || !xc) { free(xv); free(xc); bad_alloc = 1; continue; }
        double *xq = xv + H, *av = xq + H, *aq = av + I;
        uint8_t *xs = xc + H, *ac = xs + H / 32, *as = ac + I;
        for (long h = 0; h < H; ++h) xv[h] = oracle_bf16_value(x[b * H + h]);
        oracle_mxfp8_quantize(xv, H, xc, xs);
        for (long h = 0; h < H; ++h) xq[h] = oracle_dequant(xc[h], xs[h / 32]);
        for (long h = 0; h < H; ++h) y[b * H + h] = 0.0;
        for (long k = 0; k < K; ++k) {
            long e = ids[b * K + k];
            for (long j = 0; j < I; ++j) {
                const uint8_t *cg = wgu + (e * 2 * I + j) * (long)H, *cu = wgu + (e * 2 * I + I + j) * (long)H;
                const uint8_t *sg = sgu + (e * 2 * I + j) * nbh, *su = sgu + (e * 2 * I + I + j) * nbh;
                double g = 0.0, u = 0.0;
                for (long h = 0; h < H; ++h) {
                    g += oracle_dequant(cg[h], sg[h / 32]) * xq[h];
                    u += oracle_dequant(cu[h], su[h / 32]) * xq[h];
                }
                av[j] = oracle_bf16_value(oracle_bf16_rne(oracle_round_f32(oracle_silu(g) * u)));
            }
            oracle_mxfp8_quantize(av, I, ac, as);
            for (long j = 0; j < I; ++j) aq[j] = oracle_dequant(ac[j], as[j / 32]);
            for (long h = 0; h < H; ++h) {
                double o = 0.0;
                for (long j = 0; j < I; ++j)
                    o += oracle_dequant(wd[(e * H + h) * (long)I + j], sd[(e * H + h) * nbi + j / 32]) * aq[j];
                y[b * H + h] += (double)w[b * K + k] * oracle_bf16_value(oracle_bf16_rne(oracle_round_f32(o)));
            }
        }
        for (long h = 0; h < H; ++h) y[b * H + h] = oracle_bf16_value(oracle_bf16_rne(oracle_round_f32(y[b * H + h])));
        free(xv);
        free(xc);
    }
    return bad_alloc ? -4 : 0;
}

/* ---- router ------------------------------------------------------------

 * Top-k gating ahead of the layer (the pages name it only as routing each
 * token to 8 of 128 experts: the Chinese summary, section 传统路径的困境;
 * the English summary, Method).  Plain definition: the K largest logits of a
 * token (larger first; equal logits: the lower expert index first), and
 * weights = softmax over the full row renormalised to the chosen K, which is
 * the softmax of the chosen logits: w_k = exp(l_k - l_max) / sum_j exp(l_j - l_max).
 * FP64 throughout.  Logits must be finite. */
int oracle_route(const float *logits, int B, int E, int K, int32_t *ids, double *w) {
    if (B < 0 || E < 1 || K < 1 || K > E) return -2;
    for (long b = 0; b < B; ++b) {
        const float *l = logits + b * (long)E;
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int j = 0; j < k; ++j) taken |= ids[b * K + j] == e;
                if (taken) continue;
                if (best < 0 || l[e] > l[best]) best = e;     /* strict: ties keep the lower index */
            }
            ids[b * K + k] = best;
        }
        const double lmax = (double)l[ids[b * K]];
        double z = 0.0;
        for (int k = 0; k < K; ++k) z += exp((double)l[ids[b * K + k]] - lmax);
        for (int k = 0; k < K; ++k) w[b * K + k] = exp((double)l[ids[b * K + k]] - lmax) / z;
    }
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
