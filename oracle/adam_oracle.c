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
 *        low int16 half of the fp32 word), _local_step_with_scaled_states
 *        and _apply_state_scale (per-tensor scaled 16-bit optimizer state),
 *        _check_params_shard_dtypes (param-sync cast).
 *
 * Precision: the pages compute the update in `float` with `float` state, so
 * every operation here is a single IEEE binary32 operation, rounded to
 * nearest-even, evaluated in the order the expressions are printed.  Build
 * with -ffp-contract=off (no fused multiply-add) and without -ffast-math (no
 * reassociation, no flush-to-zero).  On x86-64 `float` arithmetic is SSE, so
 * there is no excess precision.
 *
 * Readings where the pages leave a step open:
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
 *   - float -> binary16 casts (fp16 param-out, fp16 scaled state) round to
 *     nearest even with IEEE overflow to infinity and subnormals kept.
 *   - scaled state: torch.reciprocal and the float division of the scale are
 *     correctly rounded float operations.
 *   - a 16-bit state type T (bf16 or fp16 params and moments): the functor's
 *     update of its T arrays (`p -= lr * update`, `m = next_m`, ...) is read
 *     as the float result rounded once to T, nearest even; the param-out
 *     cast starts from the new T value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types of the gradient, param-out and scaled-state buffers. */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2 };

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

/* float -> IEEE binary16 bits, round to nearest, ties to even, from the
 * definition of the format: near |x| in [2^e, 2^(e+1)) the binary16 values
 * are spaced 2^(e-10) apart (e >= -14; below 2^-14 the subnormals are spaced
 * 2^-24).  |x| divided by that spacing (exact in double) is rounded to an
 * integer with ties to even (rint in the default rounding mode); a result of
 * 2^16 or more overflows to infinity.  NaN stays NaN (quiet, sign kept). */
uint16_t oracle_f16_rne(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    if (isinf(x))
        return (uint16_t)(sign | 0x7C00u);
    double a = fabs((double)x);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                       /* a in [2^(e-1), 2^e) */
    int low = e - 1 < -14 ? -14 : e - 1;
    double spacing = ldexp(1.0, low - 10);
    double r = rint(a / spacing) * spacing;
    if (r >= 65536.0)
        return (uint16_t)(sign | 0x7C00u);
    if (r < ldexp(1.0, -14))            /* subnormal (or zero): count of 2^-24 */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    int re;
    double f = frexp(r, &re);           /* r = f * 2^re, f in [0.5, 1) */
    uint16_t exponent = (uint16_t)(re - 1 + 15);
    uint16_t fraction = (uint16_t)((2.0 * f - 1.0) * 1024.0);
    return (uint16_t)(sign | (exponent << 10) | fraction);
}

/* binary16 bits -> float (exact): (-1)^s * 2^(e-15) * (1 + f/1024), or
 * f * 2^-24 for e == 0; e == 31 is infinity or NaN. */
float oracle_f16_to_f32(uint16_t h)
{
    int negative = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double mag;
    if (e == 0x1F)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, -24);
    else
        mag = ldexp(1024.0 + f, e - 25);
    return (float)(negative ? -mag : mag);
}

/* Array forms, used by the exhaustive encoding tests. */
void oracle_f16_rne_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_rne(x[i]);
}

void oracle_f16_to_f32_array(const uint16_t *h, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f32(h[i]);
}

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

/* Gradient element i as float (g_type: ORACLE_F32, ORACLE_BF16, ORACLE_F16). */
static float load_grad(const void *g, int32_t g_type, int64_t i)
{
    if (g_type == ORACLE_F32)
        return ((const float *)g)[i];
    uint16_t h = ((const uint16_t *)g)[i];
    return g_type == ORACLE_F16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);
}

/* The param-out cast (out_type ORACLE_BF16 or ORACLE_F16), nearest even. */
static uint16_t cast_out(float x, int32_t out_type)
{
    return out_type == ORACLE_F16 ? oracle_f16_rne(x) : oracle_bf16_rne(x);
}

/* The param-out store ([P1] operator(): the new param cast to PARAM_OUT_T):
 * out_type ORACLE_F32 stores the float, ORACLE_BF16 / ORACLE_F16 its
 * nearest-even 16-bit value. */
static void store_out(void *p_out, int64_t i, float x, int32_t out_type)
{
    if (out_type == ORACLE_F32)
        ((float *)p_out)[i] = x;
    else
        ((uint16_t *)p_out)[i] = cast_out(x, out_type);
}

/* A 16-bit value of the state type (ORACLE_BF16 or ORACLE_F16) as float
 * (exact), and a float rounded to that type (nearest even). */
static float state_to_f32(uint16_t h, int32_t type)
{
    return type == ORACLE_F16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);
}

static uint16_t f32_to_state(float x, int32_t type)
{
    return type == ORACLE_F16 ? oracle_f16_rne(x) : oracle_bf16_rne(x);
}

/* fp32 params: p, m, v updated in place over n elements; g is float, bf16 or
 * fp16 (g_type); p_out (nullable) receives the new p as float, bf16 or fp16
 * (out_type), round to nearest even. */
void oracle_adam_f32(float *p, float *m, float *v, const void *g,
                     int32_t g_type, void *p_out, int32_t out_type, int64_t n,
                     float lr, float beta1, float beta2, float eps,
                     float weight_decay, int32_t mode, float bc1, float bc2,
                     float grad_scale)
{
    struct oracle_scalars s = {lr, beta1, beta2, eps, weight_decay,
                               bc1, bc2, grad_scale, mode};
    for (int64_t i = 0; i < n; ++i) {
        float M = m[i];
        float V = v[i];
        float P_new = adam_element(p[i], load_grad(g, g_type, i), &M, &V, &s);
        p[i] = P_new;
        m[i] = M;
        v[i] = V;
        if (p_out)
            store_out(p_out, i, P_new, out_type);
    }
}

/* 16-bit state: [P1] operator() takes the type T of the param and both
 * moments from the param tensor list (float, half or bfloat16; apex's
 * optimizer passes its state dtype as T).  For T = bf16 or fp16
 * (state_type) p, m and v hold T values: each is widened to float (exact),
 * updated as above, and assigned back to T (round to nearest even, once, as
 * the functor's stores of its float results into T arrays do); p_out
 * (nullable) receives the static_cast of the new param, which the functor
 * takes from its T array, so from the rounded T value (out_type float, bf16
 * or fp16). */
void oracle_adam_state16(uint16_t *p, uint16_t *m, uint16_t *v, int32_t state_type,
                         const void *g, int32_t g_type, void *p_out, int32_t out_type,
                         int64_t n, float lr, float beta1, float beta2, float eps,
                         float weight_decay, int32_t mode, float bc1, float bc2,
                         float grad_scale)
{
    struct oracle_scalars s = {lr, beta1, beta2, eps, weight_decay,
                               bc1, bc2, grad_scale, mode};
    for (int64_t i = 0; i < n; ++i) {
        float P = state_to_f32(p[i], state_type);
        float M = state_to_f32(m[i], state_type);
        float V = state_to_f32(v[i], state_type);
        float P_new = adam_element(P, load_grad(g, g_type, i), &M, &V, &s);
        m[i] = f32_to_state(M, state_type);
        v[i] = f32_to_state(V, state_type);
        p[i] = f32_to_state(P_new, state_type);
        if (p_out)
            store_out(p_out, i, state_to_f32(p[i], state_type), out_type);
    }
}

/* bf16 params with int16 remainders (the implicit fp32 master): each element
 * is decoded to float, updated exactly as above, and encoded back; p_out
 * (nullable) receives the new bf16 param bits. */
void oracle_adam_remainder(uint16_t *p, int16_t *rem, float *m, float *v,
                           const void *g, int32_t g_type, uint16_t *p_out,
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
        float P_new = adam_element(P, load_grad(g, g_type, i), &M, &V, &s);
        oracle_rem_encode(P_new, &p[i], &rem[i]);
        m[i] = M;
        v[i] = V;
        if (p_out)
            p_out[i] = p[i];
    }
}

/* ---------------------------------------------------------------------- */
/* Per-tensor scaled 16-bit optimizer state: [P2]                          */
/* _local_step_with_scaled_states, _apply_state_scale,                     */
/* _check_params_shard_dtypes.                                             */
/* ---------------------------------------------------------------------- */

/* Half the largest finite value of the state type (torch.finfo(dtype).max
 * / 2, exact in float): the magnitude the largest scaled element is mapped
 * to.  binary16: (2 - 2^-10) * 2^15 / 2; bfloat16: (2 - 2^-7) * 2^127 / 2. */
float oracle_scaled_state_limit(int32_t type)
{
    if (type == ORACLE_F16)
        return ldexpf(2.0f - ldexpf(1.0f, -10), 14);
    return ldexpf(2.0f - ldexpf(1.0f, -7), 126);
}

/* max(-min(x), max(x)) over a float buffer, NaN when any element is NaN (the
 * minimum and maximum reductions propagate NaN). */
static float abs_max(const float *x, int64_t n)
{
    float lo = x[0], hi = x[0];
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(x[i]))
            return NAN;
        if (x[i] < lo)
            lo = x[i];
        if (x[i] > hi)
            hi = x[i];
    }
    float neg_lo = -lo;
    return neg_lo > hi ? neg_lo : hi;
}

/* _apply_state_scale, then the copy into the state type: scale = absmax /
 * limit, every element multiplied by 1/scale (0 when scale is not positive)
 * and cast to the state type.  Returns the new scale.  n must be > 0. */
float oracle_rescale_store(const float *x, uint16_t *out, int64_t n, int32_t type)
{
    float absmax = abs_max(x, n);
    float scale = absmax / oracle_scaled_state_limit(type);
    float rscale = scale > 0.0f ? 1.0f / scale : 0.0f;
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_state(x[i] * rscale, type);
    return scale;
}

/* One step of one tensor with scaled state.  p, m, v hold 16-bit values of
 * state_type (bf16 or fp16) and scales[0..2] their float scales; all are
 * updated in place.  In the pages' order: the state is copied to float and
 * multiplied by its scale; the float update runs with the param as its own
 * output; the param-sync copy p_out (nullable, bf16 or fp16) is the new float
 * param cast to its type; then each of param, exp_avg, exp_avg_sq gets a new
 * scale from its largest magnitude and is stored scaled.  An empty tensor
 * is left alone (it holds no fragment of the local shard).  Returns 0, or -1
 * when the float work buffers cannot be allocated. */
int oracle_adam_scaled(uint16_t *p, uint16_t *m, uint16_t *v, int32_t state_type,
                       float *scales, const void *g, int32_t g_type,
                       uint16_t *p_out, int32_t out_type, int64_t n,
                       float lr, float beta1, float beta2, float eps,
                       float weight_decay, int32_t mode, float bc1, float bc2,
                       float grad_scale)
{
    if (n <= 0)
        return 0;
    float *P = malloc(sizeof(float) * (size_t)n * 3);
    if (P == NULL)
        return -1;
    float *M = P + n;
    float *V = P + 2 * n;
    for (int64_t i = 0; i < n; ++i) {
        P[i] = state_to_f32(p[i], state_type) * scales[0];
        M[i] = state_to_f32(m[i], state_type) * scales[1];
        V[i] = state_to_f32(v[i], state_type) * scales[2];
    }
    struct oracle_scalars s = {lr, beta1, beta2, eps, weight_decay,
                               bc1, bc2, grad_scale, mode};
    for (int64_t i = 0; i < n; ++i)
        P[i] = adam_element(P[i], load_grad(g, g_type, i), &M[i], &V[i], &s);
    if (p_out)
        for (int64_t i = 0; i < n; ++i)
            p_out[i] = cast_out(P[i], out_type);
    scales[0] = oracle_rescale_store(P, p, n, state_type);
    scales[1] = oracle_rescale_store(M, m, n, state_type);
    scales[2] = oracle_rescale_store(V, v, n, state_type);
    free(P);
    return 0;
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

void oracle_acc_add_squares(struct oracle_acc *a, const void *g, int32_t g_type, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)load_grad(g, g_type, i);
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
