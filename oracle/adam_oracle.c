/*
 * Oracle for the fused multi-tensor Adam / AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct CPU
 * statement of what the GPU path computes.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the product
 * path never does.  It shares no code, header, table or constant with the HIP
 * library.
 *
 * Sources (all on the web pages this project follows):
 *   [P1] apex patch "Enhance Distributed Fused Adam (#1794)",
 *        hunk of multi_tensor_distopt_adam_kernel.cu:
 *        DistAdamCapturableFunctor::local_step (the per-element update) and
 *        DistAdamCapturableFunctor::operator() (noop return, bias correction,
 *        the static_cast to the param-out type).
 *   [P2] apex distributed_fused_adam.py (master): _bf16_rem_to_fp32 (the
 *        bf16 + int16 remainder encoding), _local_step_with_param_remainders,
 *        step() (step counter handling), _load_state_dict_v2 (remainder =
 *        low int16 half of the fp32 word).
 *
 * Precision: the pages compute the update in `float` with `float` state, so
 * every operation here is a single IEEE binary32 operation, rounded to
 * nearest-even, evaluated in the order the expressions are printed.  Build
 * with -ffp-contract=off (no fused multiply-add) and without -ffast-math (no
 * reassociation, no flush-to-zero).  On x86-64 `float` arithmetic is SSE, so
 * there is no excess precision.
 *
 * Readings where the pages leave a step open (listed again in the design doc):
 *   - lerp(beta, x, m) is used but never defined; it is read as the Adam
 *     moment average beta*m + (1-beta)*x: two rounded products and a rounded
 *     sum, with 1-beta itself rounded in float.
 *   - pow(beta, step) has unstated precision; it is read as beta (the float
 *     argument, widened exactly to double) raised to the integer step by
 *     binary exponentiation in double, then 1 - beta^t in double, rounded
 *     once to float.  For t <= 0 beta^t is taken as 1.
 *   - the float -> bf16 static_cast is read as IEEE round-to-nearest-even,
 *     with NaN kept NaN (quiet bit set, sign kept).
 *   - the remainder functor's body is not shown; it is read as decode ->
 *     the float update above -> encode, where encode is the unique inverse
 *     of the decoder _bf16_rem_to_fp32 prints.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float f32_from_bits(uint32_t b)
{
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

static uint32_t bits_from_f32(float f)
{
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return b;
}

/* ---------------------------------------------------------------------- */
/* Bias correction: [P1] operator(), the bias_correction == 1 branch.      */
/* ---------------------------------------------------------------------- */

/* beta^t in double for integer t, by square-and-multiply over the bits of t.
 * t <= 0 gives 1. */
double oracle_pow_int(double beta, int32_t t)
{
    double result = 1.0;
    double square = beta;
    uint32_t e = t > 0 ? (uint32_t)t : 0u;
    while (e != 0u) {
        if (e & 1u)
            result = result * square;
        square = square * square;
        e >>= 1;
    }
    return result;
}

/* bc1 = 1 - beta1^t and bc2 = 1 - beta2^t, rounded to float; both are 1 when
 * bias correction is off (bias_correction == 0). */
void oracle_bias_corrections(float beta1, float beta2, int32_t t,
                             int32_t bias_correction, float *bc1, float *bc2)
{
    if (bias_correction == 1) {
        *bc1 = (float)(1.0 - oracle_pow_int((double)beta1, t));
        *bc2 = (float)(1.0 - oracle_pow_int((double)beta2, t));
    } else {
        *bc1 = 1.0f;
        *bc2 = 1.0f;
    }
}

/* ---------------------------------------------------------------------- */
/* bf16 and remainder encodings.                                           */
/* ---------------------------------------------------------------------- */

/* float -> bf16 bits, round to nearest, ties to even ([P1] static_cast to
 * PARAM_OUT_T).  The decision is made on the exact value: keep the top 16
 * bits, and add one unit when the dropped 16 bits exceed half a unit, or
 * equal half a unit and the kept bits are odd.  NaN keeps its sign and top
 * payload bits and gets the quiet bit. */
uint16_t oracle_bf16_rne(float x)
{
    uint32_t b = bits_from_f32(x);
    if (isnan(x))
        return (uint16_t)((b >> 16) | 0x0040u);
    uint32_t kept = b >> 16;
    uint32_t dropped = b & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;  /* may carry into the exponent: that is the rounding */
    return (uint16_t)kept;
}

/* bf16 bits -> float (exact: the bf16 value is the top half of a float). */
float oracle_bf16_to_f32(uint16_t h)
{
    return f32_from_bits((uint32_t)h << 16);
}

/* [P2] _bf16_rem_to_fp32: the high half of the fp32 word is the bf16 bits
 * minus one when the remainder is negative (as a signed int16), the low half
 * is the remainder; 16-bit arithmetic wraps. */
float oracle_rem_decode(uint16_t bf16, int16_t rem)
{
    uint16_t high = (uint16_t)(bf16 - (rem < 0 ? 1u : 0u));
    uint16_t low = (uint16_t)rem;
    return f32_from_bits(((uint32_t)high << 16) | (uint32_t)low);
}

/* Inverse of oracle_rem_decode: the remainder is the low half of the fp32
 * word ([P2] _load_state_dict_v2 takes int16 element 0 of the fp32 state),
 * and the bf16 bits are the high half plus one when that remainder is
 * negative, wrapping mod 2^16. */
void oracle_rem_encode(float x, uint16_t *bf16, int16_t *rem)
{
    uint32_t b = bits_from_f32(x);
    uint16_t low = (uint16_t)(b & 0xFFFFu);
    uint16_t high = (uint16_t)(b >> 16);
    int16_t r;
    memcpy(&r, &low, sizeof r);
    *rem = r;
    *bf16 = (uint16_t)(high + (r < 0 ? 1u : 0u));
}

/* Array forms, used by the exhaustive encoding tests. */
void oracle_bf16_rne_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(x[i]);
}

void oracle_rem_encode_array(const float *x, uint16_t *bf16, int16_t *rem,
                             int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        oracle_rem_encode(x[i], &bf16[i], &rem[i]);
}

void oracle_rem_decode_array(const uint16_t *bf16, const int16_t *rem,
                             float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_rem_decode(bf16[i], rem[i]);
}

/* ---------------------------------------------------------------------- */
/* The per-element update: [P1] local_step, both branches.                 */
/* ---------------------------------------------------------------------- */

/* Moment average beta*m + (1-beta)*x (the reading of lerp). */
static float moment_average(float beta, float x, float m)
{
    float keep = beta * m;
    float one_minus_beta = 1.0f - beta;
    float take = one_minus_beta * x;
    return keep + take;
}

/* Scalars of one call.  mode 0 = L2 (decay folded into the gradient),
 * mode 1 = AdamW (decay added to the update), as the pages encode it. */
struct oracle_scalars {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    float bc1;
    float bc2;
    float grad_scale;
    int32_t mode;
};

/* Updates one element.  P, G are the param and gradient as float; *M, *V are
 * the moments, updated in place.  Returns the new param. */
static float adam_element(float P, float G, float *M, float *V,
                          const struct oracle_scalars *s)
{
    float scaled_grad;
    if (s->mode == 0) {
        /* L2: the decay term joins the gradient before the moments. */
        float grad_part = G * s->grad_scale;
        float decay_part = s->weight_decay * P;
        scaled_grad = grad_part + decay_part;
    } else {
        scaled_grad = G * s->grad_scale;
    }
    float next_m = moment_average(s->beta1, scaled_grad, *M);
    float grad_sq = scaled_grad * scaled_grad;
    float next_v = moment_average(s->beta2, grad_sq, *V);
    float m_unbiased = next_m / s->bc1;
    float v_unbiased = next_v / s->bc2;
    float denom = sqrtf(v_unbiased) + s->eps;  /* eps outside the root */
    float update = m_unbiased / denom;
    if (s->mode == 1) {
        /* AdamW: decoupled decay uses the param from before this step. */
        float decay_part = s->weight_decay * P;
        update = update + decay_part;
    }
    *M = next_m;
    *V = next_v;
    float step = s->lr * update;
    return P - step;
}

static float load_grad(const void *g, int32_t g_is_bf16, int64_t i)
{
    if (g_is_bf16)
        return oracle_bf16_to_f32(((const uint16_t *)g)[i]);
    return ((const float *)g)[i];
}

/* fp32 params: p, m, v updated in place over n elements; g is float or bf16
 * bits; p_out (nullable) receives round-to-nearest-even bf16 of the new p. */
void oracle_adam_f32(float *p, float *m, float *v, const void *g,
                     int32_t g_is_bf16, uint16_t *p_out, int64_t n,
                     float lr, float beta1, float beta2, float eps,
                     float weight_decay, int32_t mode, float bc1, float bc2,
                     float grad_scale)
{
    struct oracle_scalars s = {lr, beta1, beta2, eps, weight_decay,
                               bc1, bc2, grad_scale, mode};
    for (int64_t i = 0; i < n; ++i) {
        float M = m[i];
        float V = v[i];
        float P_new = adam_element(p[i], load_grad(g, g_is_bf16, i), &M, &V, &s);
        p[i] = P_new;
        m[i] = M;
        v[i] = V;
        if (p_out)
            p_out[i] = oracle_bf16_rne(P_new);
    }
}

/* bf16 params with int16 remainders (the implicit fp32 master): each element
 * is decoded to float, updated exactly as above, and encoded back; p_out
 * (nullable) receives the new bf16 param bits. */
void oracle_adam_remainder(uint16_t *p, int16_t *rem, float *m, float *v,
                           const void *g, int32_t g_is_bf16, uint16_t *p_out,
                           int64_t n, float lr, float beta1, float beta2,
                           float eps, float weight_decay, int32_t mode,
                           float bc1, float bc2, float grad_scale)
{
    struct oracle_scalars s = {lr, beta1, beta2, eps, weight_decay,
                               bc1, bc2, grad_scale, mode};
    for (int64_t i = 0; i < n; ++i) {
        float P = oracle_rem_decode(p[i], rem[i]);
        float M = m[i];
        float V = v[i];
        float P_new = adam_element(P, load_grad(g, g_is_bf16, i), &M, &V, &s);
        oracle_rem_encode(P_new, &p[i], &rem[i]);
        m[i] = M;
        v[i] = V;
        if (p_out)
            p_out[i] = p[i];
    }
}

/* ---------------------------------------------------------------------- */
/* Sum of squares of the gradients, exactly, rounded once to double        */
/* (the local part of the gradient norm: [P2] grad_norm squares and sums   */
/* the per-bucket L2 norms of the gradient shards).                        */
/* ---------------------------------------------------------------------- */

/* Every square of a float (or bf16) is a double of the form M * 2^E with M a
 * 53-bit integer and E >= -350 (the smallest float denormal is 2^-149, its
 * square 2^-298).  The accumulator is one big fixed-point integer whose
 * lowest bit is worth 2^-400, in 64-bit words; adding M * 2^E is an exact
 * integer addition.  Inf and NaN are tracked apart. */
#define ACC_WORDS 14
#define ACC_LSB_EXP (-400)

struct oracle_acc {
    uint64_t w[ACC_WORDS];
    int32_t has_inf;
    int32_t has_nan;
};

void oracle_acc_clear(struct oracle_acc *a)
{
    memset(a, 0, sizeof *a);
}

static void acc_add_bits(struct oracle_acc *a, int word, uint64_t lo, uint64_t hi)
{
    /* adds (hi:lo) << (64 * word) with carry */
    uint64_t s = a->w[word] + lo;
    uint64_t carry = s < lo;
    a->w[word] = s;
    int k = word + 1;
    uint64_t add = hi;
    while (k < ACC_WORDS && (add != 0 || carry != 0)) {
        uint64_t t = a->w[k] + add;
        uint64_t c1 = t < add;
        uint64_t t2 = t + carry;
        uint64_t c2 = t2 < carry;
        a->w[k] = t2;
        carry = c1 + c2;
        add = 0;
        ++k;
    }
}

static void acc_add_double(struct oracle_acc *a, double x)
{
    if (isnan(x)) {
        a->has_nan = 1;
        return;
    }
    if (isinf(x)) {
        a->has_inf = 1;
        return;
    }
    if (x == 0.0)
        return;
    int e;
    double frac = frexp(x, &e);            /* x = frac * 2^e, 0.5 <= frac < 1 */
    uint64_t m = (uint64_t)ldexp(frac, 53); /* exact 53-bit integer */
    int shift = (e - 53) - ACC_LSB_EXP;    /* bit position of m's lowest bit */
    int word = shift / 64;
    int bit = shift % 64;
    uint64_t lo = m << bit;
    uint64_t hi = bit == 0 ? 0 : m >> (64 - bit);
    acc_add_bits(a, word, lo, hi);
}

void oracle_acc_add_squares(struct oracle_acc *a, const void *g, int32_t g_is_bf16, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)load_grad(g, g_is_bf16, i);
        acc_add_double(a, x * x);          /* exact: at most 48 significant bits */
    }
}

void oracle_acc_merge(struct oracle_acc *into, const struct oracle_acc *from)
{
    for (int k = 0; k < ACC_WORDS; ++k)
        acc_add_bits(into, k, from->w[k], 0);
    into->has_inf |= from->has_inf;
    into->has_nan |= from->has_nan;
}

/* The accumulated value rounded to the nearest double, ties to even. */
double oracle_acc_value(const struct oracle_acc *a)
{
    if (a->has_nan)
        return NAN;
    if (a->has_inf)
        return INFINITY;
    int top = -1;
    for (int k = ACC_WORDS - 1; k >= 0 && top < 0; --k)
        if (a->w[k] != 0)
            top = k * 64 + 63 - __builtin_clzll(a->w[k]);
    if (top < 0)
        return 0.0;
    /* the 53 bits from `top` down, then round on the bits below */
    uint64_t m = 0;
    for (int b = top; b > top - 53; --b) {
        m <<= 1;
        if (b >= 0 && ((a->w[b / 64] >> (b % 64)) & 1u))
            m |= 1u;
    }
    int below = top - 53;                  /* highest bit not kept */
    int round_up = 0;
    if (below >= 0 && ((a->w[below / 64] >> (below % 64)) & 1u)) {
        int sticky = 0;
        for (int b = below - 1; b >= 0 && !sticky; --b)
            if ((a->w[b / 64] >> (b % 64)) & 1u)
                sticky = 1;
        round_up = sticky || (m & 1u);
    }
    if (round_up)
        m += 1;                            /* may become 2^53: still exact */
    return ldexp((double)m, top - 52 + ACC_LSB_EXP);
}

size_t oracle_acc_size(void)
{
    return sizeof(struct oracle_acc);
}
