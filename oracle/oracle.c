/*
 * CPU oracle for the forward pass of one sparse token-choice MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plainly written reference
 * that the HIP path is checked against.  Only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may load it; the product path never
 * does.  It shares no code, header, table or constant generator with the HIP
 * path: the canonical scalar functions below are written here from their
 * mathematical definitions, independently of the device versions.
 *
 * Precision.  The pages fix one precision: the router runs in fp32 (CS336
 * lecture 4 notes, section 11 "stability": router computed entirely in
 * float32; awesome-ai-roadmap ch. 19, section 19.6.2 table "Router higher
 * precision").  Everything that decides an integer (router logits, noisy
 * scores, sigmoid affinities, the top-k keys) is therefore computed in fp32
 * with one stated operation order ("canonical arithmetic"):
 *   - dot products: acc = 0; acc = fmaf(a[i], b[i], acc) for i = 0..n-1;
 *   - exp / log / log1p / softplus / sigmoid / sin / cos: the polynomial
 *     schemes written out below (Cody-Waite reduction + Taylor / atanh
 *     series), with correctly rounded fp32 division and square root;
 *   - compiled with -ffp-contract=off and without fast-math.
 * Everything else (gates, router probabilities, expert FFNs, the combine) is
 * computed in fp64 and only rounded where the layer stores a tensor in its
 * activation dtype (bf16 round-to-nearest-even or fp32).
 *
 * Random numbers.  Shazeer's noisy gate adds standard-normal noise.  The noise
 * is either passed in by the caller, or drawn here from Philox4x32-10
 * (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
 * SC'11) followed by the Box-Muller transform, with a fixed counter mapping.
 *
 * Parity pins are documented with the tests that apply them.  The Philox
 * generator is pinned to the published known-answer vectors of Philox4x32-10
 * (stored with their citation among the test fixtures); the Gaussian draws
 * made from it are pinned statistically.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OC_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* configuration                                                             */
/* ------------------------------------------------------------------------ */

enum { OC_RELU = 0, OC_SWIGLU = 1 };
enum { OC_SOFTMAX_TOPK = 0, OC_SOFTMAX_FULL = 1, OC_NOISY_TOPK = 2, OC_SIGMOID_BIAS = 3, OC_EXPERT_CHOICE = 4,
       OC_HASH = 5, OC_HIERARCHICAL = 6 };

typedef struct {
    int32_t T, d, F, E, k;
    int32_t act_bf16;            /* 1: activations and expert weights are bf16 (uint16 bits) */
    int32_t act;                 /* OC_RELU | OC_SWIGLU */
    int32_t gate;                /* OC_SOFTMAX_TOPK | ... */
    double capacity_factor;      /* <= 0: dropless */
    int32_t residual;            /* add x to the output */
    int32_t n_shared, F_shared;  /* 0 or 1 always-on SwiGLU expert of width F_shared */
    int32_t round_intermediates; /* 1: round h, y, shared, out to the activation dtype */
    int32_t pad_;
    uint64_t seed, noise_offset; /* Philox key and counter offset for the noisy gate */
    int32_t n_groups, group_k;   /* hierarchical gate: groups, and groups picked per token */
} oc_config;

/* ------------------------------------------------------------------------ */
/* bit helpers and dtype conversion                                          */
/* ------------------------------------------------------------------------ */

static inline uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static inline float bf16_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

/* Load element i of an activation-dtype vector as fp32 (exact). */
static inline float act_load(const void* p, int act_bf16, size_t i) {
    return act_bf16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

/* Round a double to the nearest bf16 value (ties to even), returned as a
 * double.  Written directly from the format: 8 significant bits, exponent
 * range of fp32, so no intermediate rounding to fp32 happens. */
static double round_to_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    double m = frexp(v, &e);           /* v = m * 2^e, 0.5 <= |m| < 1 */
    if (e < -125) {                    /* bf16 subnormals: fixed quantum 2^-133 */
        double q = ldexp(1.0, -133);
        return nearbyint(v / q) * q;
    }
    double r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    if (fabs(r) > 3.3895313892515355e38) return v > 0 ? INFINITY : -INFINITY;
    return r;
}

static inline double round_act(double v, int act_bf16) {
    return act_bf16 ? round_to_bf16(v) : (double)(float)v;
}

/* ------------------------------------------------------------------------ */
/* canonical fp32 scalar functions                                           */
/* ------------------------------------------------------------------------ */

#define C_LOG2E   0x1.715476p+0f   /* log2(e) rounded to fp32 */
#define C_LN2_HI  0x1.62e400p-1f   /* ln 2 cut to 17 significant bits */
#define C_LN2_LO  0x1.7f7d1cp-20f  /* ln 2 - C_LN2_HI, rounded */

/* e^x.  Reduction x = n ln2 + r with n = rint(x log2 e) (Cody & Waite 1980),
 * r by two fmas against the split ln 2, e^r by its Taylor series to degree 7
 * in Horner form, then scaling by 2^n through the exponent field.  Inputs
 * below -87 give 0 and inputs above 88 give +inf, so every finite result is a
 * normal number. */
OC_EXPORT float oc_exp(float x) {
    if (x != x) return x;
    if (x > 88.0f) return INFINITY;
    if (x < -87.0f) return 0.0f;
    float n = rintf(x * C_LOG2E);
    float r = fmaf(-n, C_LN2_HI, x);
    r = fmaf(-n, C_LN2_LO, r);
    float p = 0x1.a01a02p-13f;         /* 1/7! */
    p = fmaf(p, r, 0x1.6c16c2p-10f);   /* 1/6! */
    p = fmaf(p, r, 0x1.111112p-7f);    /* 1/5! */
    p = fmaf(p, r, 0x1.555556p-5f);    /* 1/4! */
    p = fmaf(p, r, 0x1.555556p-3f);    /* 1/3! */
    p = fmaf(p, r, 0x1.000000p-1f);    /* 1/2! */
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int ni = (int)n;
    return p * u2f((uint32_t)(ni + 127) << 23);
}

/* ln x for x > 0.  x = m 2^e with m in [sqrt(1/2), sqrt(2)] by bit
 * manipulation; ln m = 2 atanh(s), s = (m-1)/(m+1), by the odd series
 * s + s^3/3 + ... + s^13/13 in Horner form in s^2; result e ln2 + ln m with
 * ln 2 split in two parts. */
OC_EXPORT float oc_log(float x) {
    if (x != x) return x;
    if (x < 0.0f) return NAN;
    if (x == 0.0f) return -INFINITY;
    if (isinf(x)) return x;
    int adj = 0;
    if (x < 0x1p-126f) { x = x * 0x1p+23f; adj = -23; }
    uint32_t u = f2u(x);
    int e = (int)(u >> 23) - 127 + adj;
    float m = u2f((u & 0x007fffffu) | 0x3f800000u);
    if (m > 0x1.6a09e6p+0f) { m = m * 0.5f; e += 1; }
    float s = (m - 1.0f) / (m + 1.0f);
    float s2 = s * s;
    float q = 0x1.3b13b2p-4f;          /* 1/13 */
    q = fmaf(q, s2, 0x1.745d18p-4f);   /* 1/11 */
    q = fmaf(q, s2, 0x1.c71c72p-4f);   /* 1/9 */
    q = fmaf(q, s2, 0x1.24924ap-3f);   /* 1/7 */
    q = fmaf(q, s2, 0x1.99999ap-3f);   /* 1/5 */
    q = fmaf(q, s2, 0x1.555556p-2f);   /* 1/3 */
    q = fmaf(q, s2, 1.0f);
    float lm = (2.0f * s) * q;
    float ef = (float)e;
    return fmaf(ef, C_LN2_HI, fmaf(ef, C_LN2_LO, lm));
}

/* ln(1+y) for y >= 0: y - y^2/2 for tiny y, otherwise ln(u) * (y / (u-1))
 * with u = 1+y, which cancels the rounding error of forming u. */
OC_EXPORT float oc_log1p(float y) {
    if (y < 0x1p-12f && y > -0x1p-12f) return fmaf(-0.5f * y, y, y);
    float u = 1.0f + y;
    return oc_log(u) * (y / (u - 1.0f));
}

/* softplus(t) = ln(1 + e^t) (Shazeer notes, section 2.2: Softplus keeps the
 * noise scale non-negative). */
OC_EXPORT float oc_softplus(float t) {
    if (t > 15.0f) return t;
    if (t < -15.0f) return oc_exp(t);
    return oc_log1p(oc_exp(t));
}

/* sigmoid(z) = 1 / (1 + e^-z) (DeepSeek-V3 affinity, CS336 lecture 4 notes,
 * section 12). */
OC_EXPORT float oc_sigmoid(float z) {
    return 1.0f / (1.0f + oc_exp(-z));
}

/* sin and cos of theta in [0, 2 pi]: quadrant q = rint(theta 2/pi), r by two
 * fmas against the split pi/2, Taylor polynomials of degree 9 (sin) and 8
 * (cos) on |r| <= pi/4, then the quadrant rotation. */
OC_EXPORT void oc_sincos(float th, float* s_out, float* c_out) {
    float q = rintf(th * 0x1.45f306p-1f);
    float r = fmaf(-q, 0x1.921fb6p+0f, th);
    r = fmaf(-q, -0x1.777a5cp-25f, r);
    float r2 = r * r;
    float ps = 0x1.71de3ap-19f;           /* 1/9! */
    ps = fmaf(ps, r2, -0x1.a01a02p-13f);  /* -1/7! */
    ps = fmaf(ps, r2, 0x1.111112p-7f);    /* 1/5! */
    ps = fmaf(ps, r2, -0x1.555556p-3f);   /* -1/3! */
    float sr = fmaf(r2 * r, ps, r);
    float pc = 0x1.a01a02p-16f;           /* 1/8! */
    pc = fmaf(pc, r2, -0x1.6c16c2p-10f);  /* -1/6! */
    pc = fmaf(pc, r2, 0x1.555556p-5f);    /* 1/4! */
    pc = fmaf(pc, r2, -0.5f);             /* -1/2! */
    float cr = fmaf(pc, r2, 1.0f);
    switch (((int)q) & 3) {
        case 0: *s_out = sr; *c_out = cr; break;
        case 1: *s_out = cr; *c_out = -sr; break;
        case 2: *s_out = -sr; *c_out = -cr; break;
        default: *s_out = -cr; *c_out = sr; break;
    }
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 and the Gaussian noise stream                              */
/* ------------------------------------------------------------------------ */

/* Philox4x32 with 10 rounds (Salmon et al., SC'11): per round two 32x32->64
 * multiplies by the published constants, the high halves xored with the other
 * two counter words and the key, then the key is bumped by the Weyl
 * increments. */
OC_EXPORT void oc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Box-Muller on two 32-bit words: u1 in (0,1], u2 in [0,1) from the top 24
 * bits, radius sqrt(-2 ln u1), angle 2 pi u2.  which = 0 gives r cos, 1 gives
 * r sin. */
static float box_muller(uint32_t w0, uint32_t w1, int which) {
    float u1 = (float)((w0 >> 8) + 1u) * 0x1p-24f;
    float u2 = (float)(w1 >> 8) * 0x1p-24f;
    float rad = sqrtf(-2.0f * oc_log(u1));
    float th = 0x1.921fb6p+2f * u2;
    float s, c;
    oc_sincos(th, &s, &c);
    return which ? rad * s : rad * c;
}

/* Standard-normal draw for flat element i = t*E + e of the [T][E] noise
 * matrix: Philox counter (i>>2 low, i>>2 high, offset low, offset high), key
 * (seed low, seed high); words (0,1) feed elements 0 and 1 of the group of 4,
 * words (2,3) feed elements 2 and 3; even elements take the cosine branch. */
OC_EXPORT float oc_normal(uint64_t seed, uint64_t offset, uint64_t i) {
    uint64_t g = i >> 2;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oc_philox4x32_10(ctr, key, w);
    int j = (int)(i & 3u);
    return j < 2 ? box_muller(w[0], w[1], j & 1) : box_muller(w[2], w[3], j & 1);
}

/* Hash-routing key (CS336 notes section 4, hash routing: a fixed hash of the
 * token, not a learned score, picks its experts).  For token id u and expert
 * e the element is i = u*E + e of the same counter layout as the noise
 * stream: Philox block (i>>2 low, i>>2 high, offset low, offset high) under
 * key (seed low, seed high), word i & 3; the key is that word's top 24 bits,
 * an integer, exact in fp32. */
OC_EXPORT float oc_hash_key(uint64_t seed, uint64_t offset, uint64_t i) {
    uint64_t g = i >> 2;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oc_philox4x32_10(ctr, key, w);
    return (float)(w[i & 3u] >> 8);
}

/* ------------------------------------------------------------------------ */
/* batch wrappers used by the tests of the scalar functions                 */
/* ------------------------------------------------------------------------ */

OC_EXPORT void oc_map_f32(int32_t fn, const float* x, float* y, int64_t n) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float s, c;
        switch (fn) {
            case 0: y[i] = oc_exp(x[i]); break;
            case 1: y[i] = oc_log(x[i]); break;
            case 2: y[i] = oc_log1p(x[i]); break;
            case 3: y[i] = oc_softplus(x[i]); break;
            case 4: y[i] = oc_sigmoid(x[i]); break;
            case 5: oc_sincos(x[i], &s, &c); y[i] = s; break;
            case 6: oc_sincos(x[i], &s, &c); y[i] = c; break;
            default: y[i] = NAN; break;
        }
    }
}

OC_EXPORT void oc_normal_batch(uint64_t seed, uint64_t offset, uint64_t first, int64_t n, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oc_normal(seed, offset, first + (uint64_t)i);
}

/* ------------------------------------------------------------------------ */
/* route                                                                    */
/* ------------------------------------------------------------------------ */

/* Canonical fp32 dot product of an activation row with an fp32 weight row. */
static float dot_c(const void* xrow, int act_bf16, const float* w, int n) {
    float acc = 0.0f;
    for (int i = 0; i < n; ++i) acc = fmaf(act_load(xrow, act_bf16, (size_t)i), w[i], acc);
    return acc;
}

/* Total order on fp32 keys: larger key first; -0 equals +0; NaN below -inf. */
static inline int32_t order_key(float f) {
    if (f != f) return INT32_MIN;
    if (f == 0.0f) return 0;
    int32_t i;
    memcpy(&i, &f, 4);
    return i >= 0 ? i : (int32_t)(i ^ 0x7fffffff);
}

/*
 * Router, top-k selection, gates and router probabilities for every token.
 *
 * Logits z = W_r x in fp32 (CS25 "Lecture29" notes, section "Top-two
 * routing", eq. z = W_r x; the per-expert logit bias, when given, is added to
 * z).  The key used for selection depends on the gate:
 *   SOFTMAX_TOPK / SOFTMAX_FULL: key = z.
 *   NOISY_TOPK: key = H = z + n * softplus(x W_noise) (Shazeer notes,
 *     section 2.2 symbol table for H, W_noise and Softplus; CS336 notes,
 *     section 8 noisy top-K listing), with n ~ N(0,1) per (token, expert).
 *   SIGMOID_BIAS: s = sigmoid(z), key = s + b (awesome-ai-roadmap 19.3.4:
 *     the bias corrects only the score used for top-k selection; CS336 notes
 *     section 12: V3 uses sigmoid affinities).
 *   HASH: key = oc_hash_key(seed, noise_offset, id_t * E + e) from the token
 *     ids; x and the router are not read and the logits are 0.
 *   HIERARCHICAL (Shazeer notes, appendix B: a primary gate picks groups, a
 *     secondary gate inside each picked group picks experts): the E experts
 *     form A = n_groups groups of B = E / A consecutive experts; the primary
 *     logits zp = W_group x (no bias) pick the group_k largest groups, then
 *     in each picked group the keys z of its B experts pick ks = k / group_k
 *     experts; slot order is group rank, then expert rank.
 * S = the k largest keys, ordered by key descending, ties to the lower
 * expert index.  Gates (fp64):
 *   SOFTMAX_TOPK: softmax over the selected logits (Lecture29, eq. g_i).
 *   SOFTMAX_FULL: full softmax over all E logits, read at the selected
 *     experts, no renormalisation (CS336 notes section 5 listing; Switch
 *     lesson: the chosen expert's output times the router probability).
 *   NOISY_TOPK: softmax over the selected H (Shazeer notes 2.2: the rest set
 *     to -inf before the softmax).
 *   SIGMOID_BIAS: raw affinities s of the selected experts renormalised to
 *     sum to 1 (awesome-ai-roadmap 19.3.4: mixing weights come from the
 *     original affinity, not the bias).
 *   HASH: 1 for every selected expert: the outputs are summed (CS336 notes
 *     section 4: some implementations add the expert outputs directly).
 *   HIERARCHICAL: softmax over the picked primary logits times softmax over
 *     the picked logits of the expert's group (appendix B: the output is the
 *     sum over groups and experts of the product of the two gates).
 * Router probabilities p_t (fp64), whose batch mean is P_i
 * (awesome-ai-roadmap 19.3.3; CS336 notes section 9): softmax(z) for the two
 * softmax gates, softmax(H) for the noisy gate, s / sum(s) for the sigmoid,
 * for HASH the selection itself, 1/k on each selected expert, and for
 * HIERARCHICAL softmax(zp)_g times the softmax of group g's logits.
 *
 * Outputs: idx [T][k], gates [T][k], optional keys [T][E] (fp32), optional
 * logits [T][E] (fp32), optional probs [T][E], P [E], and for the noisy gate
 * the optional noise scale softplus(x W_noise) [T][E] (fp32).  *status gets
 * bit 0 if any key was not finite.
 */
OC_EXPORT int oc_route(const oc_config* cfg, const void* x, const float* w_router,
                       const float* logit_bias, const float* sel_bias, const float* w_noise,
                       const float* noise, int32_t* idx, double* gates, float* keys_out,
                       float* logits_out, double* probs_out, double* P, int32_t* status,
                       float* noise_scale_out, const int32_t* token_ids, const float* w_group) {
    const int T = cfg->T, d = cfg->d, E = cfg->E, k = cfg->k;
    const int hashed = cfg->gate == OC_HASH;
    const int hier = cfg->gate == OC_HIERARCHICAL;
    const int A = hier ? cfg->n_groups : 1, KP = hier ? cfg->group_k : 1;
    if (hier && (A < 1 || A > 64 || KP < 1 || KP > A || E % A != 0 || k % KP != 0 || k / KP > E / A || k > 16 ||
                 !w_group))
        return -1;
    const int B = E / A, KS = k / KP;
    if (k < 1 || k > E) return -1;
    if (cfg->gate == OC_NOISY_TOPK && !w_noise) return -1;
    if (hashed && T > 0 && !token_ids) return -1;
    double* Psum = (double*)calloc((size_t)E, sizeof(double));
    int32_t bad = 0;
    #pragma omp parallel
    {
        float* z = (float*)malloc(sizeof(float) * (size_t)E);
        float* key = (float*)malloc(sizeof(float) * (size_t)E);
        double* prob = (double*)malloc(sizeof(double) * (size_t)E);
        double* Ploc = (double*)calloc((size_t)E, sizeof(double));
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        int32_t badloc = 0;
        #pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            const void* xr = cfg->act_bf16 ? (const void*)((const uint16_t*)x + (size_t)t * d)
                                           : (const void*)((const float*)x + (size_t)t * d);
            for (int e = 0; e < E; ++e) {
                if (hashed) {
                    z[e] = 0.0f;
                    key[e] = oc_hash_key(cfg->seed, cfg->noise_offset,
                                         (uint64_t)(uint32_t)token_ids[t] * (uint64_t)E + (uint64_t)e);
                    if (keys_out) keys_out[(size_t)t * E + e] = key[e];
                    if (logits_out) logits_out[(size_t)t * E + e] = 0.0f;
                    continue;
                }
                float ze = dot_c(xr, cfg->act_bf16, w_router + (size_t)e * d, d);
                if (logit_bias) ze = ze + logit_bias[e];
                z[e] = ze;
                float ke = ze;
                if (cfg->gate == OC_NOISY_TOPK) {
                    float zn = dot_c(xr, cfg->act_bf16, w_noise + (size_t)e * d, d);
                    float n = noise ? noise[(size_t)t * E + e]
                                    : oc_normal(cfg->seed, cfg->noise_offset, (uint64_t)t * (uint64_t)E + (uint64_t)e);
                    const float sc = oc_softplus(zn);
                    if (noise_scale_out) noise_scale_out[(size_t)t * E + e] = sc;
                    ke = fmaf(n, sc, ze);
                } else if (cfg->gate == OC_SIGMOID_BIAS) {
                    float s = oc_sigmoid(ze);
                    ke = sel_bias ? s + sel_bias[e] : s;
                }
                if (!isfinite(ke)) badloc = 1;
                key[e] = ke;
                if (keys_out) keys_out[(size_t)t * E + e] = ke;
                if (logits_out) logits_out[(size_t)t * E + e] = ze;
            }
            /* top-k: k passes of a strict arg-max over the experts not yet taken */
            memset(taken, 0, (size_t)E);
            double hg[16];               /* hierarchical gates of the k slots */
            if (hier) {
                /* primary logits, picked groups, then experts inside each group */
                double zp[64], pp[64];
                int gtaken[64] = {0};
                for (int g = 0; g < A; ++g) zp[g] = (double)dot_c(xr, cfg->act_bf16, w_group + (size_t)g * d, d);
                for (int g = 0; g < A; ++g) if (!isfinite(zp[g])) badloc = 1;
                int gsel[16];
                for (int j = 0; j < KP; ++j) {
                    int best = -1;
                    for (int g = 0; g < A; ++g) {
                        if (gtaken[g]) continue;
                        if (best < 0 || order_key((float)zp[g]) > order_key((float)zp[best])) best = g;
                    }
                    gtaken[best] = 1;
                    gsel[j] = best;
                }
                double mpk = zp[gsel[0]], spk = 0.0, gpk[16];
                for (int j = 0; j < KP; ++j) { gpk[j] = exp(zp[gsel[j]] - mpk); spk += gpk[j]; }
                for (int j = 0; j < KP; ++j) {
                    const int g = gsel[j];
                    int esel[16];
                    for (int q = 0; q < KS; ++q) {
                        int best = -1;
                        for (int e = g * B; e < (g + 1) * B; ++e) {
                            if (taken[e]) continue;
                            if (best < 0 || order_key(key[e]) > order_key(key[best])) best = e;
                        }
                        taken[best] = 1;
                        esel[q] = best;
                        idx[(size_t)t * k + j * KS + q] = best;
                    }
                    double ms = (double)key[esel[0]], ss = 0.0, gs[16];
                    for (int q = 0; q < KS; ++q) { gs[q] = exp((double)key[esel[q]] - ms); ss += gs[q]; }
                    for (int q = 0; q < KS; ++q) hg[j * KS + q] = (gpk[j] / spk) * (gs[q] / ss);
                }
                /* probabilities: softmax(zp)_g times the softmax of group g's logits */
                double mpa = -INFINITY, spa = 0.0;
                for (int g = 0; g < A; ++g) if (zp[g] > mpa) mpa = zp[g];
                for (int g = 0; g < A; ++g) { pp[g] = exp(zp[g] - mpa); spa += pp[g]; }
                for (int g = 0; g < A; ++g) {
                    double mg = -INFINITY, sg = 0.0;
                    for (int e = g * B; e < (g + 1) * B; ++e) if ((double)z[e] > mg) mg = (double)z[e];
                    for (int e = g * B; e < (g + 1) * B; ++e) sg += exp((double)z[e] - mg);
                    for (int e = g * B; e < (g + 1) * B; ++e) prob[e] = (pp[g] / spa) * (exp((double)z[e] - mg) / sg);
                }
            } else {
                for (int j = 0; j < k; ++j) {
                    int best = -1;
                    for (int e = 0; e < E; ++e) {
                        if (taken[e]) continue;
                        if (best < 0 || order_key(key[e]) > order_key(key[best])) best = e;
                    }
                    taken[best] = 1;
                    idx[(size_t)t * k + j] = best;
                }
            }
            /* router probabilities over all experts, fp64 */
            if (hier) {
                /* computed with the selection above */
            } else if (hashed) {
                for (int e = 0; e < E; ++e) prob[e] = taken[e] ? 1.0 / (double)k : 0.0;
            } else if (cfg->gate == OC_SIGMOID_BIAS) {
                double ssum = 0.0;
                for (int e = 0; e < E; ++e) { prob[e] = 1.0 / (1.0 + exp(-(double)z[e])); ssum += prob[e]; }
                for (int e = 0; e < E; ++e) prob[e] /= ssum;
            } else {
                const float* src = cfg->gate == OC_NOISY_TOPK ? key : z;
                double m = -INFINITY;
                for (int e = 0; e < E; ++e) if ((double)src[e] > m) m = (double)src[e];
                double sum = 0.0;
                for (int e = 0; e < E; ++e) { prob[e] = exp((double)src[e] - m); sum += prob[e]; }
                for (int e = 0; e < E; ++e) prob[e] /= sum;
            }
            for (int e = 0; e < E; ++e) Ploc[e] += prob[e];
            if (probs_out) for (int e = 0; e < E; ++e) probs_out[(size_t)t * E + e] = prob[e];
            /* gates, fp64 */
            const int32_t* sel = idx + (size_t)t * k;
            double* g = gates + (size_t)t * k;
            if (hashed) {
                for (int j = 0; j < k; ++j) g[j] = 1.0;
            } else if (hier) {
                for (int j = 0; j < k; ++j) g[j] = hg[j];
            } else if (cfg->gate == OC_SOFTMAX_FULL) {
                for (int j = 0; j < k; ++j) g[j] = prob[sel[j]];
            } else if (cfg->gate == OC_SIGMOID_BIAS) {
                double sum = 0.0;
                for (int j = 0; j < k; ++j) { g[j] = 1.0 / (1.0 + exp(-(double)z[sel[j]])); sum += g[j]; }
                for (int j = 0; j < k; ++j) g[j] /= sum;
            } else {
                const float* src = cfg->gate == OC_NOISY_TOPK ? key : z;
                double m = -INFINITY;
                for (int j = 0; j < k; ++j) if ((double)src[sel[j]] > m) m = (double)src[sel[j]];
                double sum = 0.0;
                for (int j = 0; j < k; ++j) { g[j] = exp((double)src[sel[j]] - m); sum += g[j]; }
                for (int j = 0; j < k; ++j) g[j] /= sum;
            }
        }
        #pragma omp critical
        {
            for (int e = 0; e < E; ++e) Psum[e] += Ploc[e];
            if (badloc) bad = 1;
        }
        free(z); free(key); free(prob); free(Ploc); free(taken);
    }
    for (int e = 0; e < E; ++e) P[e] = Psum[e] / (double)T;
    free(Psum);
    if (status) *status = bad ? 1 : 0;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* dispatch                                                                 */
/* ------------------------------------------------------------------------ */

/* Expert capacity C = ceil(alpha * T * k / E) (Lecture29, section "Inference
 * load balance"; Switch lesson: capacity = capacity factor x average tokens
 * per expert).  The capacity factor alpha is a decimal quantity (1.0, 1.25,
 * 1.1, ...), so it is read as the rational q / 10^6 with q the nearest
 * integer to alpha * 10^6 (halves up), and the ceiling is taken in exact
 * integer arithmetic: for every factor written with at most six decimals
 * this is the printed formula with the factor as written, with no binary
 * rounding of the factor.  The result is clamped to `cap` (a larger
 * capacity has no effect). */
static int64_t decimal_capacity(double cf, int64_t T, int64_t k, int64_t E, int64_t cap) {
    const double qd = floor(cf * 1e6 + 0.5);
    if (!(qd < 9.0e18)) return cap;               /* beyond any integer C: nothing is cut */
    const unsigned __int128 num = (unsigned __int128)(uint64_t)qd * (uint64_t)T * (uint64_t)k;
    const unsigned __int128 den = (unsigned __int128)1000000u * (uint64_t)E;
    const unsigned __int128 C = (num + den - 1) / den;
    return C < (unsigned __int128)cap ? (int64_t)C : cap;
}

/* Token choice: -1 when dropless (factor <= 0); else the capacity above,
 * at most T * k. */
OC_EXPORT int64_t oc_capacity(const oc_config* cfg) {
    if (!(cfg->capacity_factor > 0.0)) return -1;
    return decimal_capacity(cfg->capacity_factor, cfg->T, cfg->k, cfg->E, (int64_t)cfg->T * cfg->k);
}

/*
 * Capacity reroute (Lecture29, "Inference load balance": an expert that
 * receives more than C tokens may drop, reroute or delay the extra ones).
 * Reading: the assignments are taken in (t, j) order; the first C of an
 * expert stay; every later one, in that same order, moves to the best other
 * expert of its token (largest selection key, ties to the lower index) that
 * is not already among the token's current experts and still has room; with
 * none it stays and dispatch drops it.  The slot keeps its gate.  idx [T][k]
 * is rewritten in place; keys [T][E] are the selection keys of the route.
 * Returns the number of moved assignments (0 when dropless).
 */
OC_EXPORT int64_t oc_reroute(const oc_config* cfg, const float* keys, int32_t* idx) {
    const int T = cfg->T, E = cfg->E, k = cfg->k;
    const int64_t C = oc_capacity(cfg);
    if (C < 0 || T <= 0) return 0;
    int64_t* n = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    unsigned char* over = (unsigned char*)calloc((size_t)T * k, 1);
    for (int64_t a = 0; a < (int64_t)T * k; ++a) {
        const int e = idx[a];
        if (e < 0 || e >= E) continue;
        if (n[e] < C) n[e] += 1;
        else over[a] = 1;
    }
    int64_t moved = 0;
    for (int64_t a = 0; a < (int64_t)T * k; ++a) {
        if (!over[a]) continue;
        const int64_t t = a / k;
        const int32_t* cur = idx + t * k;
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (n[e] >= C) continue;
            int mine = 0;
            for (int j = 0; j < k; ++j) if (cur[j] == e) mine = 1;
            if (mine) continue;
            if (best < 0 || order_key(keys[t * E + e]) > order_key(keys[t * E + best])) best = e;
        }
        if (best >= 0) {
            idx[a] = best;
            n[best] += 1;
            moved += 1;
        }
    }
    free(n);
    free(over);
    return moved;
}

/*
 * Counting sort of the T*k assignments (t, j) by expert, stable in (t, j)
 * order (Lecture29, "Top-k routing semantics": tokens are re-arranged by
 * expert, run in batches, and inverse-permuted).  Assignment a = t*k + j.
 * With a capacity C, the first C assignments of each expert in that order are
 * kept and the rest are dropped (slot_pos = -1): the expert branch then
 * contributes nothing and the residual passes through (CS336 notes, section
 * 10; Switch lesson token-drop answer).
 *   counts[e] = assignments to e before drops; kept[e] = min(counts[e], C);
 *   offsets = exclusive prefix sum of kept (E+1 entries);
 *   perm_src[row] = a for the assignment stored in row; slot_pos[a] = row.
 * Returns the number of kept rows R = offsets[E].
 */
OC_EXPORT int64_t oc_dispatch(const oc_config* cfg, const int32_t* idx, int32_t* counts, int32_t* kept,
                              int32_t* offsets, int32_t* perm_src, int32_t* slot_pos) {
    const int T = cfg->T, E = cfg->E, k = cfg->k;
    if (E <= 0 || k <= 0 || T < 0) return -1;
    int64_t C = oc_capacity(cfg);
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < (int64_t)T * k; ++a)
        if (idx[a] >= 0 && idx[a] < E) counts[idx[a]] += 1;   /* other ids: no assignment */
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        kept[e] = (C >= 0 && counts[e] > C) ? (int32_t)C : counts[e];
        offsets[e + 1] = offsets[e] + kept[e];
    }
    int32_t* rank = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int64_t a = 0; a < (int64_t)T * k; ++a) {
        int e = idx[a];
        if (e < 0 || e >= E) { slot_pos[a] = -1; continue; }
        int32_t r = rank[e]++;
        if (C >= 0 && r >= C) { slot_pos[a] = -1; continue; }
        int32_t row = offsets[e] + r;
        perm_src[row] = (int32_t)a;
        slot_pos[a] = row;
    }
    free(rank);
    return offsets[E];
}

/* x_perm[row] = x[perm_src[row] / k], copied in the activation dtype. */
OC_EXPORT void oc_gather_rows(const oc_config* cfg, const void* x, const int32_t* perm_src, int64_t R,
                              void* x_perm) {
    const size_t rowbytes = (size_t)cfg->d * (cfg->act_bf16 ? 2 : 4);
    for (int64_t r = 0; r < R; ++r) {
        int64_t t = perm_src[r] / cfg->k;
        memcpy((char*)x_perm + (size_t)r * rowbytes, (const char*)x + (size_t)t * rowbytes, rowbytes);
    }
}

/* ------------------------------------------------------------------------ */
/* experts                                                                  */
/* ------------------------------------------------------------------------ */

/*
 * One expert applied to n rows a[n][d] (activation dtype), fp64 arithmetic.
 *   SWIGLU: y = W2 (SiLU(W1 a) . W3 a), SiLU(v) = v / (1 + e^-v)
 *           (Lecture29, "Dense baseline": the SwiGLU MLP; W1 = gate,
 *           W3 = up, W2 = down).
 *   RELU:   y = W2 relu(W1 a) (Shazeer notes 2.2: each expert is a
 *           feed-forward net with one ReLU hidden layer, 512->1024->512).
 * w1 (and w3) are [F][d], w2 is [d][F] (row = output unit).  The hidden
 * vector h and the output are rounded to the activation dtype when
 * round_intermediates is set, as the layer stores them there.
 * y_out is [n][d] fp64.
 */
OC_EXPORT void oc_expert_ffn(const oc_config* cfg, int32_t F, const void* a, int64_t n, const void* w1,
                             const void* w3, const void* w2, double* y_out) {
    const int d = cfg->d, bf = cfg->act_bf16, rnd = cfg->round_intermediates;
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * (size_t)F);
        double* ar = (double*)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            for (int i = 0; i < d; ++i) ar[i] = (double)act_load(a, bf, (size_t)r * d + i);
            for (int f = 0; f < F; ++f) {
                double g = 0.0;
                for (int i = 0; i < d; ++i) g += ar[i] * (double)act_load(w1, bf, (size_t)f * d + i);
                double hv;
                if (cfg->act == OC_SWIGLU) {
                    double u = 0.0;
                    for (int i = 0; i < d; ++i) u += ar[i] * (double)act_load(w3, bf, (size_t)f * d + i);
                    hv = g / (1.0 + exp(-g)) * u;
                } else {
                    hv = g > 0.0 ? g : 0.0;
                }
                h[f] = rnd ? round_act(hv, bf) : hv;
            }
            for (int o = 0; o < d; ++o) {
                double y = 0.0;
                for (int f = 0; f < F; ++f) y += h[f] * (double)act_load(w2, bf, (size_t)o * F + f);
                y_out[(size_t)r * d + o] = rnd ? round_act(y, bf) : y;
            }
        }
        free(h); free(ar);
    }
}

/* ------------------------------------------------------------------------ */
/* combine and statistics                                                   */
/* ------------------------------------------------------------------------ */

/*
 * out[t] = (residual ? x[t] : 0) + (shared ? shared[t] : 0)
 *          + sum over kept slots j of gates[t][j] * y[slot_pos[t][j]]
 * (Lecture29, eq. y = sum_i g_i(x) Expert_i(x); CS336 notes section 5
 * listing adds the residual; the shared expert is always on, weight 1,
 * awesome-ai-roadmap 19.5).  A dropped slot contributes nothing.  fp64,
 * rounded to the activation dtype when round_intermediates is set.
 * tokens lists which tokens to produce (NULL = all T); y is [R][d] fp64,
 * shared is [T][d] fp64 or NULL; out is [ntok][d].
 */
OC_EXPORT void oc_combine(const oc_config* cfg, const int32_t* tokens, int64_t ntok, const int32_t* slot_pos,
                          const double* gates, const double* y, const void* x, const double* shared,
                          double* out) {
    const int d = cfg->d, k = cfg->k;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < ntok; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        for (int o = 0; o < d; ++o) {
            double acc = 0.0;
            if (cfg->residual) acc += (double)act_load(x, cfg->act_bf16, (size_t)t * d + o);
            if (shared) acc += shared[(size_t)t * d + o];
            for (int j = 0; j < k; ++j) {
                int32_t row = slot_pos[t * k + j];
                if (row < 0) continue;
                acc += gates[t * k + j] * y[(size_t)row * d + o];
            }
            out[(size_t)i * d + o] = cfg->round_intermediates ? round_act(acc, cfg->act_bf16) : acc;
        }
    }
}

/*
 * Load statistics.  f_i = fraction of the assignments (T*k for token choice)
 * routed to expert i before capacity drops, so sum f = 1 (awesome-ai-roadmap
 * 19.3.3; CS336 notes section 9); aux = E * sum_i f_i P_i, the Switch balance
 * term without its coefficient; imbalance I = max_i n_i / (mean n)
 * (Lecture29, "Myth 3").
 */
OC_EXPORT void oc_stats(const oc_config* cfg, const int32_t* counts, const int32_t* kept, const double* P,
                        double* f, int64_t* n_dropped, double* imbalance, double* aux) {
    const int E = cfg->E;
    /* the assignments that exist: T k for token choice, E C for expert choice */
    double tk = 0.0;
    for (int e = 0; e < E; ++e) tk += (double)counts[e];
    int64_t kept_sum = 0;
    int32_t nmax = 0;
    double a = 0.0;
    for (int e = 0; e < E; ++e) {
        f[e] = (double)counts[e] / tk;
        kept_sum += kept[e];
        if (counts[e] > nmax) nmax = counts[e];
        a += f[e] * P[e];
    }
    *n_dropped = (int64_t)tk - kept_sum;
    *imbalance = (double)nmax / (tk / (double)E);
    *aux = (double)E * a;
}

/* ------------------------------------------------------------------------ */
/* balance and stability statistics                                         */
/* ------------------------------------------------------------------------ */

/* Standard normal CDF, Phi(x) = erfc(-x / sqrt(2)) / 2 (fp64 libm). */
static double oc_phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/*
 * Statistics the pages attach to the router, computed from the route's
 * per-token outputs (logits z [T][E], selection keys [T][E], the noisy
 * gate's noise scale softplus(x W_noise) [T][E] or NULL, probabilities
 * p [T][E], idx and gates [T][slots]: slots = k for token choice, E for
 * expert choice, whose untaken slots hold id -1 and are skipped).  All fp64.
 *
 *   z_loss = mean_t (log sum_e exp z_t,e)^2: the router z-loss, the squared
 *     log of the softmax normaliser (CS336 notes section 11; awesome-ai-
 *     roadmap 19.6.2 table: the squared logsumexp of the logits).  Taken
 *     over the clean logits z for every gate.
 *   importance_e = sum_t G(x_t)_e, the gate values an expert receives
 *     (Shazeer notes: Importance, balanced through CV^2); importance_cv2 =
 *     Var/mean^2 over the experts (CV = std / mean, population std).
 *   load_e = sum_t P(x_t, e) for the noisy gate, with
 *     P(x, e) = Phi((z_e - kth_excluding(H(x), k, e)) / softplus((x W_noise)_e))
 *     (Shazeer notes, Load(X) and Phi, eq. 9): kth_excluding is the k-th
 *     largest noisy score other than e's own, i.e. the (k+1)-th largest of H
 *     when e is among the top k and the k-th largest otherwise; with k = E
 *     every expert is always chosen and P = 1.  load_cv2 as above.  Left
 *     untouched when noise_scale is NULL.
 *   seq_aux = mean over sequences of E * sum_e f_e^s P_e^s, the balance term
 *     counted per sequence (CS336 notes section 9: V3 keeps a complementary
 *     sequence-level auxiliary loss; awesome-ai-roadmap 19.3.4), with
 *     f_e^s = n_e^s / (L k) from the selections of the sequence's L tokens
 *     (k = top_k, the mean experts per token, also under expert choice)
 *     and P_e^s their mean probability; seq_len <= 0 means one sequence of
 *     all T tokens (then seq_aux equals the batch aux).
 * Returns -1 when seq_len does not divide T.
 */
OC_EXPORT int oc_balance(const oc_config* cfg, int32_t seq_len, const float* logits, const float* keys,
                         const float* noise_scale, const double* probs, const int32_t* idx, const double* gates,
                         double* z_loss, double* importance, double* importance_cv2, double* load, double* load_cv2,
                         double* seq_aux) {
    const int T = cfg->T, E = cfg->E, k = cfg->k;
    const int slots = cfg->gate == OC_EXPERT_CHOICE ? E : k;
    const int L = seq_len > 0 ? seq_len : T;
    if (T > 0 && (L <= 0 || T % L != 0)) return -1;
    double zsum = 0.0;
    for (int e = 0; e < E; ++e) { importance[e] = 0.0; if (noise_scale) load[e] = 0.0; }
    unsigned char* sel = (unsigned char*)malloc((size_t)(E > 0 ? E : 1));
    for (int t = 0; t < T; ++t) {
        const float* z = logits + (size_t)t * E;
        double m = -INFINITY;
        for (int e = 0; e < E; ++e) if ((double)z[e] > m) m = (double)z[e];
        double s = 0.0;
        for (int e = 0; e < E; ++e) s += exp((double)z[e] - m);
        const double lse = m + log(s);
        zsum += lse * lse;
        for (int j = 0; j < slots; ++j) {
            const int32_t e = idx[(size_t)t * slots + j];
            if (e >= 0 && e < E) importance[e] += gates[(size_t)t * slots + j];
        }
        if (noise_scale) {
            const float* h = keys + (size_t)t * E;
            memset(sel, 0, (size_t)E);
            for (int j = 0; j < k; ++j) sel[idx[(size_t)t * k + j]] = 1;
            /* k-th largest key = the smallest selected one; (k+1)-th = the
               largest unselected one */
            double kth = INFINITY, next = -INFINITY;
            for (int e = 0; e < E; ++e) {
                if (sel[e]) { if ((double)h[e] < kth) kth = (double)h[e]; }
                else if ((double)h[e] > next) next = (double)h[e];
            }
            for (int e = 0; e < E; ++e) {
                double pe;
                if (k >= E) pe = 1.0;
                else {
                    const double thr = sel[e] ? next : kth;
                    pe = oc_phi(((double)z[e] - thr) / (double)noise_scale[(size_t)t * E + e]);
                }
                load[e] += pe;
            }
        }
    }
    free(sel);
    *z_loss = T > 0 ? zsum / (double)T : 0.0;
    /* CV^2 = population variance / mean^2 */
    for (int pass = 0; pass < 2; ++pass) {
        const double* v = pass == 0 ? importance : load;
        double* out = pass == 0 ? importance_cv2 : load_cv2;
        if (pass == 1 && !noise_scale) break;
        double mean = 0.0;
        for (int e = 0; e < E; ++e) mean += v[e];
        mean /= (double)E;
        double var = 0.0;
        for (int e = 0; e < E; ++e) var += (v[e] - mean) * (v[e] - mean);
        var /= (double)E;
        *out = mean != 0.0 ? var / (mean * mean) : 0.0;
    }
    /* sequence-wise balance term */
    double acc = 0.0;
    const int nseq = T > 0 ? T / L : 0;
    double* Ps = (double*)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
    int64_t* ns = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E > 0 ? E : 1));
    for (int sq = 0; sq < nseq; ++sq) {
        for (int e = 0; e < E; ++e) { Ps[e] = 0.0; ns[e] = 0; }
        for (int t = sq * L; t < (sq + 1) * L; ++t) {
            for (int e = 0; e < E; ++e) Ps[e] += probs[(size_t)t * E + e];
            for (int j = 0; j < slots; ++j) {
                const int32_t e = idx[(size_t)t * slots + j];
                if (e >= 0 && e < E) ns[e] += 1;
            }
        }
        double a = 0.0;
        for (int e = 0; e < E; ++e) a += ((double)ns[e] / ((double)L * k)) * (Ps[e] / (double)L);
        acc += (double)E * a;
    }
    free(Ps); free(ns);
    *seq_aux = nseq > 0 ? acc / (double)nseq : 0.0;
    return 0;
}

/*
 * Auxiliary-loss-free balancing (CS336 notes section 9; awesome-ai-roadmap
 * 19.3.4): after a batch, every expert's selection bias moves by gamma
 * towards balance, up when the expert received fewer assignments than the
 * mean, down when more, unchanged when equal:
 *   b_e += gamma * sign(mean - n_e),  mean = sum_e n_e / E.
 * The comparison n_e * E <=> sum n is exact in integers.  The bias only
 * enters the selection keys, never the gates.
 */
OC_EXPORT void oc_update_bias(int32_t E, const int32_t* counts, float gamma, float* bias) {
    int64_t total = 0;
    for (int e = 0; e < E; ++e) total += counts[e];
    for (int e = 0; e < E; ++e) {
        const int64_t c = (int64_t)counts[e] * E;
        if (c < total) bias[e] = bias[e] + gamma;
        else if (c > total) bias[e] = bias[e] - gamma;
    }
}

/* ------------------------------------------------------------------------ */
/* expert choice                                                            */
/* ------------------------------------------------------------------------ */

/* Tokens per expert under expert choice: C = ceil(cf * T * k / E) with the
 * capacity factor cf (1 when not set) read as a six-place decimal as for
 * token choice, and k the mean number of experts per token, at most T. */
OC_EXPORT int64_t oc_ec_capacity(const oc_config* cfg) {
    const double cf = cfg->capacity_factor > 0.0 ? cfg->capacity_factor : 1.0;
    return decimal_capacity(cf, cfg->T, cfg->k, cfg->E, cfg->T);
}

/*
 * Expert-choice routing (CS336 notes section 4: every expert scores all
 * tokens and takes its top K, "top-K along the rows", so every expert gets
 * exactly the same number of tokens; awesome-ai-roadmap 19.6.1: experts each
 * take a fixed number of tokens and a token may be processed by a varying
 * number of experts).  Reading: the score of token t for expert e is its
 * router probability S = softmax over the experts of the logits z (fp32:
 * m = max_e z, s = sum over e = 0..E-1 in order of exp(z_e - m) with the
 * canonical exp, S_e = exp(z_e - m) / s correctly rounded); expert e takes the
 * C tokens with the largest S[., e], ties to the lower token index; the gate
 * of a chosen (t, e) is S[t, e].
 * Outputs, with E slots per token: idx[t][e] = e if e took t, else -1;
 * gates[t][e] = S[t][e] or 0; scores [T][E] = S (fp32, optional); logits
 * [T][E] = z (fp32, optional); P_e = mean_t S[t][e].
 */
OC_EXPORT int oc_route_ec(const oc_config* cfg, const void* x, const float* w_router, const float* logit_bias,
                          int32_t* idx, double* gates, float* scores_out, float* logits_out, double* P) {
    const int T = cfg->T, d = cfg->d, E = cfg->E;
    if (E < 1 || cfg->k < 1 || cfg->k > E) return -1;
    const int64_t C = oc_ec_capacity(cfg);
    float* S = (float*)malloc(sizeof(float) * (size_t)T * (size_t)E + 1);
    #pragma omp parallel
    {
        float* z = (float*)malloc(sizeof(float) * (size_t)E);
        #pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            const void* xr = cfg->act_bf16 ? (const void*)((const uint16_t*)x + (size_t)t * d)
                                           : (const void*)((const float*)x + (size_t)t * d);
            float m = -INFINITY;
            for (int e = 0; e < E; ++e) {
                float ze = dot_c(xr, cfg->act_bf16, w_router + (size_t)e * d, d);
                if (logit_bias) ze = ze + logit_bias[e];
                z[e] = ze;
                if (logits_out) logits_out[(size_t)t * E + e] = ze;
                if (ze > m) m = ze;
            }
            float s = 0.0f;
            for (int e = 0; e < E; ++e) s = s + oc_exp(z[e] - m);
            for (int e = 0; e < E; ++e) S[(size_t)t * E + e] = oc_exp(z[e] - m) / s;
        }
        free(z);
    }
    for (size_t i = 0; i < (size_t)T * E; ++i) { idx[i] = -1; gates[i] = 0.0; }
    int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    for (int e = 0; e < E; ++e) {
        /* the C first tokens in the order (S descending, index ascending) */
        double psum = 0.0;
        for (int t = 0; t < T; ++t) psum += (double)S[(size_t)t * E + e];
        P[e] = T > 0 ? psum / (double)T : 0.0;
        for (int t = 0; t < T; ++t) order[t] = t;
        /* plain bottom-up merge sort of the token indices */
        for (int width = 1; width < T; width *= 2) {
            for (int lo = 0; lo < T; lo += 2 * width) {
                int mid = lo + width < T ? lo + width : T, hi = lo + 2 * width < T ? lo + 2 * width : T;
                int i = lo, j = mid, n = 0;
                int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(hi - lo + 1));
                while (i < mid || j < hi) {
                    int take_left;
                    if (i >= mid) take_left = 0;
                    else if (j >= hi) take_left = 1;
                    else {
                        const float a = S[(size_t)order[i] * E + e], b = S[(size_t)order[j] * E + e];
                        take_left = order_key(a) > order_key(b) || (order_key(a) == order_key(b) && order[i] < order[j]);
                    }
                    tmp[n++] = take_left ? order[i++] : order[j++];
                }
                memcpy(order + lo, tmp, sizeof(int32_t) * (size_t)(hi - lo));
                free(tmp);
            }
        }
        for (int64_t r = 0; r < C; ++r) {
            const int t = order[r];
            idx[(size_t)t * E + e] = e;
            gates[(size_t)t * E + e] = (double)S[(size_t)t * E + e];
        }
    }
    if (scores_out) memcpy(scores_out, S, sizeof(float) * (size_t)T * E);
    free(order);
    free(S);
    return 0;
}
