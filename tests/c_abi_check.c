/*
 * c_abi_check.c -- test infrastructure: a plain C99 program that uses the SP
 * region library through include/sp_region.h alone (the HIP runtime API only
 * for device memory), and compares its forward and backward with the C oracle
 * (oracle/sp_oracle.c) on seeded inputs.
 *
 * Three shards are checked, one per dgamma schedule: a short LayerNorm shard
 * (column workgroups, one row segment, no workspace), a 1024-row RMSNorm shard
 * (column workgroups over several row segments, called twice on the one
 * zero-filled workspace: the second call must give the same bits) and a long
 * RMSNorm shard (partial rows and the finish kernel).  Bar: mask and h byte-identical; y,
 * d_residual, dP, dgamma, dbeta within 1e-2 relative (plus 1e-2 of the rms of
 * the reference); rstd and mean within 1e-5.  Exit status 0 = pass.
 * --any-schedule: do not check which dgamma schedule each shard gets.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sp_region.h"

/* The oracle's entry points and descriptor (oracle/sp_oracle.c). */
typedef struct {
    int64_t S, B, H;
    int32_t T, j, dtype, norm;
    float eps, p;
    uint64_t seed;
} spo_desc;
int sp_oracle_fwd(const spo_desc* d, int64_t row0, int64_t nrows, const void* const* P,
                  const void* residual, const double* gamma, const double* beta, void* h, void* y,
                  uint8_t* mask, double* mean, double* rstd);
int sp_oracle_bwd(const spo_desc* d, int64_t row0, int64_t nrows, const void* dY, const void* h,
                  const uint8_t* mask, const double* mean, const double* rstd, const double* gamma,
                  const void* dR, void* d_res, void* dP, double* dgamma, double* dbeta);

#define CHECK_HIP(x)                                                                 \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);         \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

/* splitmix64: seeded input values only, none of the method's arithmetic */
static uint64_t g_state;
static uint64_t next_u64(void)
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
/* roughly normal (sum of four uniforms, centred), times `scale` */
static float rnd(float scale)
{
    double s = 0.0;
    int i;
    for (i = 0; i < 4; ++i) s += (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0);
    return (float)((s - 2.0) * 1.7320508 * scale);
}
/* a bf16 value: the upper half of a float's bits (the data is only data) */
static uint16_t bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static double bf16_val(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static int failures = 0;
static int any_schedule = 0; /* --any-schedule: a build that forces one dgamma schedule */

static void close_to(const char* what, const double* got, const double* ref, int64_t n, double rtol)
{
    double ms = 0.0, worst = 0.0;
    int64_t i, bad = 0;
    for (i = 0; i < n; ++i) ms += ref[i] * ref[i];
    ms = n > 0 ? sqrt(ms / (double)n) : 0.0;
    for (i = 0; i < n; ++i) {
        const double err = fabs(got[i] - ref[i]);
        if (!(err <= rtol * fabs(ref[i]) + rtol * ms)) ++bad;
        if (err > worst) worst = err;
    }
    if (bad) {
        fprintf(stderr, "  %s: %lld of %lld outside tolerance (worst error %.3e)\n", what, (long long)bad,
                (long long)n, worst);
        ++failures;
    }
}

static void* dev_copy(const void* host, size_t bytes)
{
    void* d = NULL;
    CHECK_HIP(hipMalloc(&d, bytes > 0 ? bytes : 16));
    if (bytes && host) CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* expect: 0 = partial rows, 1 = column workgroups with one row segment, 2 = with several */
static void check_shard(int64_t S, int64_t B, int64_t H, int32_t T, int32_t j, int32_t norm, int expect)
{
    const int ln = norm == SP_LAYERNORM;
    const int64_t R = (S / T) * B, N = R * H, full = S * B * H;
    const float eps = ln ? 1e-5f : 1e-6f, p = 0.1f;
    const uint64_t seed = 1234;
    sp_desc_t d;
    spo_desc od;
    uint16_t *Ph[SP_MAX_T], *res, *dY, *h_g, *y_g, *h_o, *y_o, *dres_g, *dP_g, *dres_o, *dP_o;
    uint8_t *m_g, *m_o;
    float *gam, *bet, *rs_g, *mu_g, *dgam_g, *dbet_g, *dgam_first = NULL;
    double *gam64, *bet64, *rs_o, *mu_o, *rs_o32, *mu_o32, *dgam_o, *dbet_o, *a, *b;
    void *Pd[SP_MAX_T], *res_d, *dY_d, *gam_d, *bet_d, *h_d, *y_d, *m_d, *mu_d, *rs_d;
    void *dres_d, *dP_d, *dgam_d, *dbet_d, *ws_d = NULL;
    const void* Pshard[SP_MAX_T];
    size_t ws;
    int64_t i;
    int t, rc, sched;

    printf("[case] S=%lld B=%lld H=%lld T=%d j=%d %s\n", (long long)S, (long long)B, (long long)H, T, j,
           ln ? "LayerNorm" : "RMSNorm");
    fflush(stdout);
    memset(&d, 0, sizeof d);
    d.S = S; d.B = B; d.H = H; d.T = T; d.j = j; d.dtype = SP_BF16; d.norm = norm;
    d.eps = eps; d.p = p; d.seed = seed;
    memset(&od, 0, sizeof od);
    od.S = S; od.B = B; od.H = H; od.T = T; od.j = j; od.dtype = 1; od.norm = norm;
    od.eps = eps; od.p = p; od.seed = seed;

    /* inputs */
    for (t = 0; t < T; ++t) {
        Ph[t] = (uint16_t*)malloc((size_t)full * 2);
        for (i = 0; i < full; ++i) Ph[t][i] = bf16_bits(rnd((float)(1.0 / sqrt((double)T))));
    }
    res = (uint16_t*)malloc((size_t)N * 2);
    dY = (uint16_t*)malloc((size_t)N * 2);
    for (i = 0; i < N; ++i) res[i] = bf16_bits(rnd(1.0f));
    for (i = 0; i < N; ++i) dY[i] = bf16_bits(rnd(1.0f));
    gam = (float*)malloc((size_t)H * 4);
    bet = (float*)malloc((size_t)H * 4);
    gam64 = (double*)malloc((size_t)H * 8);
    bet64 = (double*)malloc((size_t)H * 8);
    for (i = 0; i < H; ++i) {
        gam[i] = 1.0f + rnd(0.02f);
        bet[i] = rnd(0.02f);
        gam64[i] = gam[i];
        bet64[i] = bet[i];
    }

    /* the library */
    for (t = 0; t < T; ++t) Pd[t] = dev_copy(Ph[t], (size_t)full * 2);
    res_d = dev_copy(res, (size_t)N * 2);
    dY_d = dev_copy(dY, (size_t)N * 2);
    gam_d = dev_copy(gam, (size_t)H * 4);
    bet_d = dev_copy(bet, (size_t)H * 4);
    h_d = dev_copy(NULL, (size_t)N * 2);
    y_d = dev_copy(NULL, (size_t)N * 2);
    m_d = dev_copy(NULL, (size_t)N);
    mu_d = dev_copy(NULL, (size_t)R * 4);
    rs_d = dev_copy(NULL, (size_t)R * 4);
    dres_d = dev_copy(NULL, (size_t)N * 2);
    dP_d = dev_copy(NULL, (size_t)N * 2);
    dgam_d = dev_copy(NULL, (size_t)H * 4);
    dbet_d = dev_copy(NULL, (size_t)H * 4);
    rc = sp_region_fwd(&d, (const void* const*)Pd, res_d, (const float*)gam_d, ln ? (const float*)bet_d : NULL,
                       h_d, y_d, (uint8_t*)m_d, ln ? (float*)mu_d : NULL, (float*)rs_d, NULL);
    if (rc != SP_OK) {
        fprintf(stderr, "  sp_region_fwd: %s\n", sp_region_strerror(rc));
        ++failures;
        return;
    }
    ws = sp_region_bwd_workspace_size(&d);
    sched = sp_region_bwd_schedule(&d);
    if (sched < 0 || (sched == 1) != (ws == 0)) {
        fprintf(stderr, "  schedule %d with a workspace of %zu bytes\n", sched, ws);
        ++failures;
    }
    if (!any_schedule && (sched > 2 ? 2 : sched) != expect) {
        fprintf(stderr, "  dgamma schedule %d, expected %d\n", sched, expect);
        ++failures;
    }
    if (ws > 0) {
        CHECK_HIP(hipMalloc(&ws_d, ws));
        CHECK_HIP(hipMemset(ws_d, 0, ws));
    }
    for (t = 0; t < 2; ++t) {  /* twice on one workspace: the second call must repeat the first */
        rc = sp_region_bwd(&d, dY_d, h_d, (const uint8_t*)m_d, ln ? (const float*)mu_d : NULL,
                           (const float*)rs_d, (const float*)gam_d, NULL, dres_d, dP_d, (float*)dgam_d,
                           ln ? (float*)dbet_d : NULL, ws_d, ws, NULL);
        if (rc != SP_OK) {
            fprintf(stderr, "  sp_region_bwd: %s\n", sp_region_strerror(rc));
            ++failures;
            return;
        }
        CHECK_HIP(hipDeviceSynchronize());
        if (t == 0) {
            dgam_first = (float*)malloc((size_t)H * 4);
            CHECK_HIP(hipMemcpy(dgam_first, dgam_d, (size_t)H * 4, hipMemcpyDeviceToHost));
        }
    }
    h_g = (uint16_t*)malloc((size_t)N * 2);
    y_g = (uint16_t*)malloc((size_t)N * 2);
    dres_g = (uint16_t*)malloc((size_t)N * 2);
    dP_g = (uint16_t*)malloc((size_t)N * 2);
    m_g = (uint8_t*)malloc((size_t)N);
    rs_g = (float*)malloc((size_t)R * 4);
    mu_g = (float*)malloc((size_t)R * 4);
    dgam_g = (float*)malloc((size_t)H * 4);
    dbet_g = (float*)malloc((size_t)H * 4);
    CHECK_HIP(hipMemcpy(h_g, h_d, (size_t)N * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(y_g, y_d, (size_t)N * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(m_g, m_d, (size_t)N, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(rs_g, rs_d, (size_t)R * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(mu_g, mu_d, (size_t)R * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(dres_g, dres_d, (size_t)N * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(dP_g, dP_d, (size_t)N * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(dgam_g, dgam_d, (size_t)H * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(dbet_g, dbet_d, (size_t)H * 4, hipMemcpyDeviceToHost));
    if (memcmp(dgam_first, dgam_g, (size_t)H * 4) != 0) {
        fprintf(stderr, "  dgamma of the second call on the workspace differs from the first\n");
        ++failures;
    }

    /* the oracle, on the shard's rows */
    for (t = 0; t < T; ++t) Pshard[t] = Ph[t] + (int64_t)j * N;
    h_o = (uint16_t*)malloc((size_t)N * 2);
    y_o = (uint16_t*)malloc((size_t)N * 2);
    m_o = (uint8_t*)malloc((size_t)N);
    rs_o = (double*)malloc((size_t)R * 8);
    mu_o = (double*)malloc((size_t)R * 8);
    rs_o32 = (double*)malloc((size_t)R * 8);
    mu_o32 = (double*)malloc((size_t)R * 8);
    dres_o = (uint16_t*)malloc((size_t)N * 2);
    dP_o = (uint16_t*)malloc((size_t)N * 2);
    dgam_o = (double*)malloc((size_t)H * 8);
    dbet_o = (double*)malloc((size_t)H * 8);
    if (sp_oracle_fwd(&od, 0, R, Pshard, res, gam64, ln ? bet64 : NULL, h_o, y_o, m_o, ln ? mu_o : NULL, rs_o)) {
        fprintf(stderr, "  oracle forward refused the descriptor\n");
        ++failures;
        return;
    }
    for (i = 0; i < R; ++i) { /* the saved statistics are fp32 on both sides */
        rs_o32[i] = (double)(float)rs_o[i];
        mu_o32[i] = ln ? (double)(float)mu_o[i] : 0.0;
    }
    if (sp_oracle_bwd(&od, 0, R, dY, h_o, m_o, ln ? mu_o32 : NULL, rs_o32, gam64, NULL, dres_o, dP_o, dgam_o,
                      ln ? dbet_o : NULL)) {
        fprintf(stderr, "  oracle backward refused the descriptor\n");
        ++failures;
        return;
    }

    if (memcmp(m_g, m_o, (size_t)N) != 0) {
        fprintf(stderr, "  mask differs\n");
        ++failures;
    }
    if (memcmp(h_g, h_o, (size_t)N * 2) != 0) {
        fprintf(stderr, "  h is not bit-identical\n");
        ++failures;
    }
    a = (double*)calloc((size_t)N, 8);
    b = (double*)calloc((size_t)N, 8);
    for (i = 0; i < N; ++i) { a[i] = bf16_val(y_g[i]); b[i] = bf16_val(y_o[i]); }
    close_to("y", a, b, N, 1e-2);
    for (i = 0; i < N; ++i) { a[i] = bf16_val(dres_g[i]); b[i] = bf16_val(dres_o[i]); }
    close_to("d_residual", a, b, N, 1e-2);
    for (i = 0; i < N; ++i) { a[i] = bf16_val(dP_g[i]); b[i] = bf16_val(dP_o[i]); }
    close_to("dP", a, b, N, 1e-2);
    for (i = 0; i < R; ++i) a[i] = rs_g[i];
    close_to("rstd", a, rs_o, R, 1e-5);
    if (ln) {
        for (i = 0; i < R; ++i) {
            const double scale = fabs(mu_o[i]) + 1.0 / rs_o[i];
            if (!(fabs((double)mu_g[i] - mu_o[i]) <= 1e-5 * scale)) {
                fprintf(stderr, "  mean of row %lld differs\n", (long long)i);
                ++failures;
                break;
            }
        }
    }
    for (i = 0; i < H; ++i) a[i] = dgam_g[i];
    close_to("dgamma", a, dgam_o, H, 1e-2);
    if (ln) {
        for (i = 0; i < H; ++i) a[i] = dbet_g[i];
        close_to("dbeta", a, dbet_o, H, 1e-2);
    }

    for (t = 0; t < T; ++t) {
        CHECK_HIP(hipFree(Pd[t]));
        free(Ph[t]);
    }
    CHECK_HIP(hipFree(res_d)); CHECK_HIP(hipFree(dY_d)); CHECK_HIP(hipFree(gam_d)); CHECK_HIP(hipFree(bet_d));
    CHECK_HIP(hipFree(h_d)); CHECK_HIP(hipFree(y_d)); CHECK_HIP(hipFree(m_d)); CHECK_HIP(hipFree(mu_d));
    CHECK_HIP(hipFree(rs_d)); CHECK_HIP(hipFree(dres_d)); CHECK_HIP(hipFree(dP_d));
    CHECK_HIP(hipFree(dgam_d)); CHECK_HIP(hipFree(dbet_d));
    if (ws_d) CHECK_HIP(hipFree(ws_d));
    free(res); free(dY); free(gam); free(bet); free(gam64); free(bet64);
    free(h_g); free(y_g); free(dres_g); free(dP_g); free(m_g); free(rs_g); free(mu_g); free(dgam_g); free(dbet_g); free(dgam_first);
    free(h_o); free(y_o); free(m_o); free(rs_o); free(mu_o); free(rs_o32); free(mu_o32);
    free(dres_o); free(dP_o); free(dgam_o); free(dbet_o); free(a); free(b);
}

int main(int argc, char** argv)
{
    sp_desc_t bad;
    g_state = 1234;
    any_schedule = argc > 1 && strcmp(argv[1], "--any-schedule") == 0;
    if (sp_region_version() <= 0) {
        fprintf(stderr, "bad version\n");
        return 1;
    }
    /* an argument error comes back synchronously, with its text */
    memset(&bad, 0, sizeof bad);
    bad.S = 10; bad.B = 1; bad.H = 64; bad.T = 4; bad.j = 0; bad.dtype = SP_BF16; bad.norm = SP_RMSNORM;
    bad.eps = 1e-6f; bad.p = 0.1f;
    if (sp_region_fwd(&bad, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != SP_ESHAPE ||
        sp_region_strerror(SP_ESHAPE) == NULL) {
        fprintf(stderr, "S %% T != 0 was not reported as SP_ESHAPE\n");
        return 1;
    }
    check_shard(64, 2, 256, 2, 1, SP_LAYERNORM, 1);    /* 64 rows: columns, one segment */
    check_shard(2048, 1, 1024, 2, 1, SP_RMSNORM, 2);   /* 1024 rows: columns, four segments */
    check_shard(16384, 1, 1024, 2, 1, SP_RMSNORM, 0);  /* 8192 rows: partial rows + finish */
    if (failures) {
        fprintf(stderr, "c_abi_check: %d failure(s)\n", failures);
        return 1;
    }
    printf("c_abi_check: the C ABI matches the oracle\n");
    return 0;
}
