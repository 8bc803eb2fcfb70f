/*
 * FP64 CPU oracle: packed variable-length width-4 depthwise causal
 * convolution followed by SiLU, training forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference the GPU
 * path is checked against.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the library itself never
 * calls it, and it shares no code, header or table with the HIP sources.
 *
 * Sources (documentation pages of flashinfer.cake_causal_conv1d_train):
 *   [F] cake_causal_conv1d_train_forward  - Parameters, Returns
 *   [B] cake_causal_conv1d_train_backward - Description, Parameters, Returns
 *
 * Everything is evaluated in IEEE double.  Inputs arrive already decoded to
 * double (see orc_decode_bf16 / orc_decode_f32); the only rounding to a
 * narrower format the method itself prescribes inside the computation is the
 * BF16 rounding of the preactivation under the "bf16" SiLU-derivative policy
 * ([B] Parameters, silu_grad_preactivation), done by orc_bf16_rne.
 *
 * Layout: x, dy, p, y, dpre, dx are row-major [S][C] (row t = token t);
 * w is [C][4] with w[c][3] on the current token and w[c][0] three tokens
 * back ([F] Parameters, weight); b is [C] or NULL; cu is [D+1] int32 prefix
 * sums of document lengths with cu[0] = 0 and cu[D] = S, repeated values
 * being empty documents ([F] Parameters, cu_seqlens).
 *
 * Status codes: 0 ok, -1 malformed cu_seqlens (the oracle checks the
 * precondition the GPU path may not read on the host), -2 bad sizes,
 * -3 out of memory, -4 unknown policy.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_POLICY_BF16 0 /* SiLU' at the BF16-rounded preactivation */
#define ORC_POLICY_FP32 1 /* SiLU' at the unrounded preactivation   */

/* ---- exact decoders ---------------------------------------------------- */

/* A bfloat16 value is, bit for bit, the upper half of an IEEE binary32. */
void orc_decode_bf16(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) {
        uint32_t u = (uint32_t)in[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = (double)f;
    }
}

void orc_decode_f32(const float *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = (double)in[i];
}

/* ---- double -> bfloat16, round to nearest, ties to even ----------------- */

/*
 * Rounds v directly to the nearest bfloat16 (8 significant bits, binary32
 * exponent range, subnormal quantum 2^-133), ties to even, with no
 * intermediate binary32 step.  |v| is scaled by the quantum of its binade,
 * rounded to an integer with nearbyint() (round-half-even in the default
 * rounding mode), and scaled back; both scalings are exact powers of two.
 */
uint16_t orc_bf16_rne(double v)
{
    if (isnan(v))
        return 0x7fc0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                  /* a = m * 2^e with m in [0.5, 1) */
    int qexp = e - 8;              /* 8 significant bits per binade */
    if (qexp < -133)
        qexp = -133;               /* subnormal quantum */
    double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    if (r >= ldexp(1.0, 128))      /* rounds past the largest finite */
        return sign | 0x7f80;
    float f = (float)r;            /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

void orc_bf16_rne_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_bf16_rne(in[i]);
}

static double bf16_round_value(double v)
{
    uint16_t h = orc_bf16_rne(v);
    double r;
    orc_decode_bf16(&h, &r, 1);
    return r;
}

/* ---- the scalar functions ------------------------------------------------ */

/* Logistic sigmoid; exp() overflowing to +inf gives exactly 0. */
static double sigmoid(double z)
{
    return 1.0 / (1.0 + exp(-z));
}

/* SiLU(z) = z * sigmoid(z). */
static double silu(double z)
{
    return z * sigmoid(z);
}

/* d/dz SiLU(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z))). */
static double silu_grad(double z)
{
    double s = sigmoid(z);
    return s * (1.0 + z * (1.0 - s));
}

/* ---- helpers ------------------------------------------------------------- */

/* [F] Parameters, cu_seqlens: cu[0] = 0, cu[D] = S, non-decreasing. */
static int check_cu(const int32_t *cu, int64_t D, int64_t S)
{
    if (D < 0)
        return -2;
    if (D == 0)
        return S == 0 ? 0 : -1;
    if (cu[0] != 0 || (int64_t)cu[D] != S)
        return -1;
    for (int64_t d = 0; d < D; d++)
        if (cu[d + 1] < cu[d])
            return -1;
    return 0;
}

/* Neumaier compensated summation. */
typedef struct { double sum, comp; } nsum;

static void nsum_add(nsum *a, double v)
{
    double t = a->sum + v;
    if (fabs(a->sum) >= fabs(v))
        a->comp += (a->sum - t) + v;
    else
        a->comp += (v - t) + a->sum;
    a->sum = t;
}

static double nsum_value(const nsum *a)
{
    return a->sum + a->comp;
}

/*
 * Preactivation of token t, channel c, inside a document starting at s:
 * p = sum over the taps k = 0..3 whose source token t-3+k lies in the same
 * document of w[c][k] * x[t-3+k][c], then + b[c] ([F] Returns; the bias is
 * added after the taps, [F] Parameters, bias).  *pabs receives the same sum
 * with every term replaced by its absolute value (used by the tests to size
 * the rounding-error allowance of a binary32 evaluation).
 */
static double preact(const double *x, const double *w, const double *b,
                     int64_t C, int64_t s, int64_t t, int64_t c, double *pabs)
{
    double p = 0.0, pa = 0.0;
    for (int k = 0; k < 4; k++) {
        int64_t src = t - 3 + k;
        if (src < s)
            continue;      /* zero history before the document's first token */
        double term = w[c * 4 + k] * x[src * C + c];
        p += term;
        pa += fabs(term);
    }
    if (b) {
        p += b[c];
        pa += fabs(b[c]);
    }
    if (pabs)
        *pabs = pa;
    return p;
}

/* ---- forward ([F] Returns) ------------------------------------------------ */

/*
 * p_out, pabs_out, y_out: [S][C], each may be NULL.  y_out is the unrounded
 * SiLU(p); the product rounds it to BF16, the tests compare against it.
 */
int orc_forward(int64_t S, int64_t C, const double *x, const double *w,
                const double *b, const int32_t *cu, int64_t D,
                double *p_out, double *pabs_out, double *y_out)
{
    if (S < 0 || C <= 0)
        return -2;
    int rc = check_cu(cu, D, S);
    if (rc)
        return rc;
    for (int64_t d = 0; d < D; d++) {
        int64_t s = cu[d], e = cu[d + 1];
        for (int64_t t = s; t < e; t++)
            for (int64_t c = 0; c < C; c++) {
                double pa;
                double p = preact(x, w, b, C, s, t, c, &pa);
                if (p_out)
                    p_out[t * C + c] = p;
                if (pabs_out)
                    pabs_out[t * C + c] = pa;
                if (y_out)
                    y_out[t * C + c] = silu(p);
            }
    }
    return 0;
}

/* ---- backward ([B] Description, Parameters, Returns) ---------------------- */

/*
 * dpre[t][c] = dy[t][c] * SiLU'(z) with z the recomputed preactivation,
 * rounded to BF16 under ORC_POLICY_BF16 and left as is under ORC_POLICY_FP32
 * ([B] Parameters, silu_grad_preactivation).  dpre is the gradient at the
 * preactivation; the Returns formulas sum it against the taps:
 *   dx[t][c]    = sum_k w[c][k] * dpre[t+3-k][c], over taps whose token
 *                 t+3-k lies in t's document;
 *   dw[c][k]    = sum_t dpre[t][c] * x[t-3+k][c], over tokens whose tap
 *                 source t-3+k lies in t's document;
 *   db[c]       = sum_t dpre[t][c].
 * dx_out is the unrounded value.  The sums over t use Neumaier summation.
 * dpre_out, dx_out: [S][C]; dw_out: [C][4]; db_out: [C]; each may be NULL.
 */
int orc_backward(int64_t S, int64_t C, const double *x, const double *w,
                 const double *b, const int32_t *cu, int64_t D,
                 const double *dy, int policy,
                 double *dpre_out, double *dx_out, double *dw_out,
                 double *db_out)
{
    if (S < 0 || C <= 0)
        return -2;
    if (policy != ORC_POLICY_BF16 && policy != ORC_POLICY_FP32)
        return -4;
    int rc = check_cu(cu, D, S);
    if (rc)
        return rc;

    double *dpre = dpre_out;
    if (!dpre) {
        dpre = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S * C : 1));
        if (!dpre)
            return -3;
    }
    nsum *acc = (nsum *)calloc((size_t)C * 5, sizeof(nsum)); /* [C][4 taps + bias] */
    if (!acc) {
        if (!dpre_out)
            free(dpre);
        return -3;
    }

    for (int64_t d = 0; d < D; d++) {
        int64_t s = cu[d], e = cu[d + 1];
        /* dpre over the document */
        for (int64_t t = s; t < e; t++)
            for (int64_t c = 0; c < C; c++) {
                double p = preact(x, w, b, C, s, t, c, NULL);
                double z = policy == ORC_POLICY_BF16 ? bf16_round_value(p) : p;
                dpre[t * C + c] = dy[t * C + c] * silu_grad(z);
            }
        /* dx: taps reaching forward, stopping at the document's end */
        if (dx_out)
            for (int64_t t = s; t < e; t++)
                for (int64_t c = 0; c < C; c++) {
                    double v = 0.0;
                    for (int k = 0; k < 4; k++) {
                        int64_t src = t + 3 - k;
                        if (src >= e)
                            continue;
                        v += w[c * 4 + k] * dpre[src * C + c];
                    }
                    dx_out[t * C + c] = v;
                }
        /* dweight, dbias */
        for (int64_t t = s; t < e; t++)
            for (int64_t c = 0; c < C; c++) {
                double g = dpre[t * C + c];
                for (int k = 0; k < 4; k++) {
                    int64_t src = t - 3 + k;
                    if (src < s)
                        continue;
                    nsum_add(&acc[c * 5 + k], g * x[src * C + c]);
                }
                nsum_add(&acc[c * 5 + 4], g);
            }
    }

    for (int64_t c = 0; c < C; c++) {
        if (dw_out)
            for (int k = 0; k < 4; k++)
                dw_out[c * 4 + k] = nsum_value(&acc[c * 5 + k]);
        if (db_out)
            db_out[c] = nsum_value(&acc[c * 5 + 4]);
    }
    free(acc);
    if (!dpre_out)
        free(dpre);
    return 0;
}

/* Scalar entry points, so the tests can pin the SiLU pieces on their own. */
double orc_silu(double z) { return silu(z); }
double orc_silu_grad(double z) { return silu_grad(z); }
