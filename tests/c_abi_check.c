/*
 * c_abi_check - a plain C program that drives libvdc.so through
 * include/vdc.h alone (device memory and a stream from the HIP runtime, no
 * Python, no PyTorch) and checks what it computes against the FP64 oracle
 * (oracle/vdc_oracle.c, linked as liboracle.so).
 *
 * TEST INFRASTRUCTURE: tests/test_c_abi.py runs it.  Exit status 0 when
 * every check passes, 1 when one fails, 77 when no GPU is present.
 *
 * The inputs are positive (x, dy, weight, bias), so neither the taps of the
 * preactivation nor those of dx cancel and SiLU' stays away from its zero,
 * and x, weight and bias lie on a grid that makes p exact in binary32:
 * y and dx must then be within one BF16 ulp of the FP64 values
 * (cake_causal_conv1d_train_backward, Parameters silu_grad_preactivation),
 * and dweight / dbias within the policy's rel-L2 bound (3e-5 for "bf16",
 * 2e-7 for "fp32").  The document lengths include empty and short documents
 * (cake_causal_conv1d_train_forward, Parameters cu_seqlens); C = 136 is a
 * multiple of 8 whose rows are not a multiple of 128 bytes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "vdc.h"

/* The oracle's entry points (oracle/vdc_oracle.c). */
void orc_decode_bf16(const uint16_t *in, double *out, int64_t n);
uint16_t orc_bf16_rne(double v);
int orc_forward(int64_t S, int64_t C, const double *x, const double *w, const double *b,
                const int32_t *cu, int64_t D, double *p_out, double *pabs_out, double *y_out);
int orc_backward(int64_t S, int64_t C, const double *x, const double *w, const double *b,
                 const int32_t *cu, int64_t D, const double *dy, int policy, double *dpre_out,
                 double *dx_out, double *dw_out, double *db_out);

enum { S = 3000, C = 136, D = 8 };
static const int32_t kLengths[D] = {0, 1, 2, 3, 700, 5, 1289, 1000};

static int failures = 0;

#define HIP_CHECK(call)                                                            \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s:%d: %s failed: %s\n", __FILE__, __LINE__, #call,   \
                    hipGetErrorString(e_));                                        \
            exit(1);                                                               \
        }                                                                          \
    } while (0)

static void expect(int ok, const char *what)
{
    printf("%s %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok)
        failures++;
}

/* Uniform in [0, 1) from a 32-bit linear congruential generator. */
static double uniform(uint32_t *state)
{
    *state = *state * 1664525u + 1013904223u;
    return (double)(*state >> 8) / 16777216.0;
}

/* Spacing of BF16 numbers at |v|: 2^(floor(log2 |v|) - 7), at least 2^-133. */
static double ulp_bf16(double v)
{
    int e;
    if (v == 0.0)
        return ldexp(1.0, -133);
    frexp(fabs(v), &e);
    return e - 8 < -133 ? ldexp(1.0, -133) : ldexp(1.0, e - 8);
}

/* Elements of a BF16 [S][C] result farther than one BF16 ulp from ref. */
static int64_t beyond_one_ulp(const uint16_t *got, const double *ref, int64_t n)
{
    int64_t bad = 0;
    for (int64_t i = 0; i < n; i++) {
        double g;
        orc_decode_bf16(&got[i], &g, 1);
        if (!(fabs(g - ref[i]) <= ulp_bf16(ref[i])))
            bad++;
    }
    return bad;
}

static double rel_l2(const float *got, const double *ref, int64_t n)
{
    double num = 0.0, den = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double d = (double)got[i] - ref[i];
        num += d * d;
        den += ref[i] * ref[i];
    }
    return sqrt(num / den);
}

int main(void)
{
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
        fprintf(stderr, "c_abi_check: no GPU\n");
        return 77;
    }
    HIP_CHECK(hipSetDevice(0));

    /* Host inputs: BF16 x, dy; FP32 weight, bias; int32 cu_seqlens. */
    const int64_t n = (int64_t)S * C;
    uint16_t *x = malloc(n * 2), *dy = malloc(n * 2), *y = malloc(n * 2), *dx = malloc(n * 2);
    uint16_t *dx2 = malloc(n * 2);
    float w[C * 4], b[C], dw[C * 4], db[C], dw2[C * 4], db2[C];
    int32_t cu[D + 1];
    double *x64 = malloc(n * 8), *dy64 = malloc(n * 8), *y64 = malloc(n * 8), *dx64 = malloc(n * 8);
    double w64[C * 4], b64[C], dw64[C * 4], db64[C];
    if (!x || !dy || !y || !dx || !dx2 || !x64 || !dy64 || !y64 || !dx64) {
        fprintf(stderr, "c_abi_check: out of host memory\n");
        return 1;
    }
    /* x, weight and bias are multiples of 2^-8 below 1: every product and
     * partial sum of the preactivation is then exact in binary32, so the
     * library's FP32 p equals the oracle's and its BF16 rounding (the "bf16"
     * policy's SiLU' argument) cannot land on the other side of a tie. */
    uint32_t seed = 12345u;
    for (int64_t i = 0; i < n; i++) {
        x[i] = orc_bf16_rne((13 + (int)(243 * uniform(&seed))) / 256.0);
        dy[i] = orc_bf16_rne(0.05 + uniform(&seed));
    }
    for (int i = 0; i < C * 4; i++) {
        w[i] = (float)((13 + (int)(51 * uniform(&seed))) / 256.0);
        w64[i] = w[i];
    }
    for (int i = 0; i < C; i++) {
        b[i] = (float)((int)(26 * uniform(&seed)) / 256.0);
        b64[i] = b[i];
    }
    cu[0] = 0;
    for (int d = 0; d < D; d++)
        cu[d + 1] = cu[d] + kLengths[d];
    orc_decode_bf16(x, x64, n);
    orc_decode_bf16(dy, dy64, n);

    /* Device buffers; the caller owns all of them, workspace included. */
    void *d_x, *d_dy, *d_y, *d_dx, *d_w, *d_b, *d_cu, *d_dw, *d_db, *d_ws, *d_dx2, *d_dw2, *d_db2;
    const size_t ws = workspace_bytes(VDC_BWD, S, C);
    expect(ws > 0 && workspace_bytes(VDC_FWD, S, C) == 0, "workspace_bytes");
    HIP_CHECK(hipMalloc(&d_x, n * 2));
    HIP_CHECK(hipMalloc(&d_dy, n * 2));
    HIP_CHECK(hipMalloc(&d_y, n * 2));
    HIP_CHECK(hipMalloc(&d_dx, n * 2));
    HIP_CHECK(hipMalloc(&d_w, sizeof w));
    HIP_CHECK(hipMalloc(&d_b, sizeof b));
    HIP_CHECK(hipMalloc(&d_cu, sizeof cu));
    HIP_CHECK(hipMalloc(&d_dw, sizeof dw));
    HIP_CHECK(hipMalloc(&d_db, sizeof db));
    HIP_CHECK(hipMalloc(&d_ws, ws));
    HIP_CHECK(hipMalloc(&d_dx2, n * 2));
    HIP_CHECK(hipMalloc(&d_dw2, sizeof dw2));
    HIP_CHECK(hipMalloc(&d_db2, sizeof db2));
    HIP_CHECK(hipMemcpy(d_x, x, n * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_dy, dy, n * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_b, b, sizeof b, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_cu, cu, sizeof cu, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_CHECK(hipStreamCreate(&stream));

    /* A refused call enqueues nothing and reports why. */
    int rc = conv1d_fwd(d_x, d_w, VDC_F32, d_b, VDC_F32, d_cu, D, S, 12, d_y, NULL, 0, stream);
    expect(rc == VDC_EINVAL && conv1d_status_string(rc) != NULL, "C = 12 refused (EINVAL)");
    rc = conv1d_bwd(d_x, d_w, VDC_F32, d_b, VDC_F32, d_cu, D, d_dy, S, C, VDC_SILU_GRAD_BF16,
                    d_dx, d_dw, VDC_F32, d_db, VDC_F32, d_ws, ws - 8, stream);
    expect(rc == VDC_EWORKSPACE, "short workspace refused (EWORKSPACE)");

    /* Forward. */
    rc = conv1d_fwd(d_x, d_w, VDC_F32, d_b, VDC_F32, d_cu, D, S, C, d_y, NULL, 0, stream);
    expect(rc == VDC_OK, "conv1d_fwd returns VDC_OK");
    HIP_CHECK(hipStreamSynchronize(stream));
    HIP_CHECK(hipMemcpy(y, d_y, n * 2, hipMemcpyDeviceToHost));
    if (orc_forward(S, C, x64, w64, b64, cu, D, NULL, NULL, y64) != 0) {
        fprintf(stderr, "c_abi_check: oracle forward failed\n");
        return 1;
    }
    int64_t bad = beyond_one_ulp(y, y64, n);
    printf("     y: %lld of %lld elements beyond one BF16 ulp\n", (long long)bad, (long long)n);
    expect(bad == 0, "y within one BF16 ulp of the FP64 oracle");

    /* Backward under both SiLU' policies, FP32 gradient outputs. */
    static const struct { int policy; const char *name; double bound; } kPolicies[2] = {
        {VDC_SILU_GRAD_BF16, "bf16", 3e-5}, {VDC_SILU_GRAD_FP32, "fp32", 2e-7}};
    for (int q = 0; q < 2; q++) {
        char what[128];
        rc = conv1d_bwd(d_x, d_w, VDC_F32, d_b, VDC_F32, d_cu, D, d_dy, S, C, kPolicies[q].policy,
                        d_dx, d_dw, VDC_F32, d_db, VDC_F32, d_ws, ws, stream);
        snprintf(what, sizeof what, "conv1d_bwd (%s) returns VDC_OK", kPolicies[q].name);
        expect(rc == VDC_OK, what);
        HIP_CHECK(hipStreamSynchronize(stream));
        HIP_CHECK(hipMemcpy(dx, d_dx, n * 2, hipMemcpyDeviceToHost));
        HIP_CHECK(hipMemcpy(dw, d_dw, sizeof dw, hipMemcpyDeviceToHost));
        HIP_CHECK(hipMemcpy(db, d_db, sizeof db, hipMemcpyDeviceToHost));
        if (orc_backward(S, C, x64, w64, b64, cu, D, dy64, kPolicies[q].policy, NULL, dx64, dw64,
                         db64) != 0) {
            fprintf(stderr, "c_abi_check: oracle backward failed\n");
            return 1;
        }
        bad = beyond_one_ulp(dx, dx64, n);
        printf("     dx (%s): %lld of %lld elements beyond one BF16 ulp\n", kPolicies[q].name,
               (long long)bad, (long long)n);
        snprintf(what, sizeof what, "dx (%s) within one BF16 ulp", kPolicies[q].name);
        expect(bad == 0, what);
        const double rw = rel_l2(dw, dw64, C * 4), rb = rel_l2(db, db64, C);
        printf("     dweight rel-L2 %.3e, dbias rel-L2 %.3e (bound %.0e)\n", rw, rb,
               kPolicies[q].bound);
        snprintf(what, sizeof what, "dweight and dbias (%s) within the rel-L2 bound",
                 kPolicies[q].name);
        expect(rw <= kPolicies[q].bound && rb <= kPolicies[q].bound, what);

        /* The no-allocation entry point: the library's own workspace, the
         * same kernels and plan, so bitwise the same outputs. */
        expect(ws <= conv1d_noalloc_scratch_bytes(), "workspace fits the no-allocation array");
        rc = conv1d_bwd_noalloc(d_x, d_w, VDC_F32, d_b, VDC_F32, d_cu, D, d_dy, S, C,
                                kPolicies[q].policy, d_dx2, d_dw2, VDC_F32, d_db2, VDC_F32, stream);
        snprintf(what, sizeof what, "conv1d_bwd_noalloc (%s) returns VDC_OK", kPolicies[q].name);
        expect(rc == VDC_OK, what);
        HIP_CHECK(hipStreamSynchronize(stream));
        HIP_CHECK(hipMemcpy(dx2, d_dx2, n * 2, hipMemcpyDeviceToHost));
        HIP_CHECK(hipMemcpy(dw2, d_dw2, sizeof dw2, hipMemcpyDeviceToHost));
        HIP_CHECK(hipMemcpy(db2, d_db2, sizeof db2, hipMemcpyDeviceToHost));
        snprintf(what, sizeof what, "conv1d_bwd_noalloc (%s) bitwise equal to conv1d_bwd",
                 kPolicies[q].name);
        expect(memcmp(dx2, dx, n * 2) == 0 && memcmp(dw2, dw, sizeof dw) == 0 &&
                   memcmp(db2, db, sizeof db) == 0, what);
    }

    HIP_CHECK(hipStreamDestroy(stream));
    void *bufs[] = {d_x, d_dy, d_y, d_dx, d_w, d_b, d_cu, d_dw, d_db, d_ws, d_dx2, d_dw2, d_db2};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++)
        HIP_CHECK(hipFree(bufs[i]));
    free(x); free(dy); free(y); free(dx); free(dx2);
    free(x64); free(dy64); free(y64); free(dx64);
    printf("%s\n", failures ? "c_abi_check: FAILED" : "c_abi_check: all checks passed");
    return failures ? 1 : 0;
}
