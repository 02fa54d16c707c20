/*
 * sp_oracle.c -- plain, slow CPU oracle for the sequence-parallel (SP) region.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (one rank's sequence shard j of an [S,B,H] activation, the
 * region between two tensor-parallel regions):
 *
 *   "MiniMind-tron: Sequence Parallelism" (anker661.github.io), section 3.1 and
 *   3.2.1: every TP rank t holds a full-shape partial P_t:[S,B,H]; after the
 *   reduce-scatter, rank j owns Y^(j) = sum over t of P_t^(j), a contiguous
 *   [S/T,B,H] block of the sequence axis (section 3.2.4, S % T == 0).
 *   Section 3.2.2: dropout, residual add and RMSNorm then run on that shard.
 *
 *   "Sequence Parallel" (formulaic.cloudchewie.com), section "MLP activation
 *   size": dropout is Z = Z' (.) M with a 0/1 mask stored as one byte per
 *   element, and its backward multiplies the incoming gradient by M; section
 *   "basic idea": LayerNorm(x) = gamma (x - mu) / sqrt(sigma^2 + eps) + beta with
 *   mu and sigma^2 taken along the hidden axis, and the dropout mask must stay
 *   consistent along the sequence.
 *
 *   "MiniMind-tron: SP optimisation" (anker661.github.io), section 4.2.1.1: the
 *   RMSNorm casts the bf16 stream to fp32, multiplies by the weight in fp32 and
 *   casts back to the activation type.
 *
 * Readings taken where the pages leave a step open:
 *   - order: sum of partials -> dropout -> + residual -> norm; outputs are the
 *     residual stream h and the normalised y.
 *   - element-wise arithmetic of the bf16/fp32 modes is fp32 with one rounding
 *     of h (round to nearest even), partials summed with t ascending.
 *   - inverted dropout: kept elements are scaled by 1/(1-p), dropped ones are +0.
 *   - keep mask from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 *     Numbers: As Easy as 1, 2, 3", SC'11): element with global index gi into the
 *     full [S,B,H] tensor uses counter (lo32(gi>>2), hi32(gi>>2), 0, 0), key
 *     (lo32(seed), hi32(seed)) and output word gi & 3; kept iff
 *     word >= floor(p * 2^32).
 *   - RMSNorm: x / sqrt(mean(x^2) + eps), gamma only; LayerNorm variance biased.
 *   - row statistics and all reductions in fp64 (the oracle is more precise than
 *     any kernel); mean/rstd are returned in fp64.
 *   - backward: the standard derivatives of the above (the pages print none);
 *     pinned by central finite differences in the fp64 mode.
 *
 * Modes: SPO_F32 and SPO_BF16 take activations as float / uint16 bf16 bit
 * patterns and follow the rounding rules above; SPO_F64 takes doubles and rounds
 * nothing (used for finite differences).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SPO_F32 0
#define SPO_BF16 1
#define SPO_F64 2
#define SPO_RMSNORM 0
#define SPO_LAYERNORM 1

typedef struct {
    int64_t S, B, H;   /* full activation [S,B,H] */
    int32_t T, j;      /* number of partials, shard index */
    int32_t dtype;     /* SPO_F32 / SPO_BF16 / SPO_F64 */
    int32_t norm;      /* SPO_RMSNORM / SPO_LAYERNORM */
    float eps;
    float p;           /* dropout probability */
    uint64_t seed;     /* Philox key */
} spo_desc;

/* ------------------------------------------------------------------ */
/* Philox4x32-10, written from the SC'11 paper's description: ten rounds, each
 * round multiplies counter words 0 and 2 by two fixed odd constants, keeps the
 * 64-bit products split into high and low halves, and mixes the high halves
 * with the other two counter words and the round key by XOR; the two key words
 * advance by the Weyl increments (golden ratio and sqrt(3)-1 in 32-bit fixed
 * point) between rounds. */
static const uint32_t PHILOX_MUL0 = 0xD2511F53u;
static const uint32_t PHILOX_MUL1 = 0xCD9E8D57u;
static const uint32_t PHILOX_WEYL0 = 0x9E3779B9u;
static const uint32_t PHILOX_WEYL1 = 0xBB67AE85u;

static void philox4x32_10(const uint32_t counter[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = counter[0], x1 = counter[1], x2 = counter[2], x3 = counter[3];
    uint32_t k0 = key[0], k1 = key[1];
    int round;
    for (round = 0; round < 10; ++round) {
        uint64_t prod0, prod1;
        uint32_t n0, n1, n2, n3;
        if (round > 0) {
            k0 += PHILOX_WEYL0;
            k1 += PHILOX_WEYL1;
        }
        prod0 = (uint64_t)PHILOX_MUL0 * (uint64_t)x0;
        prod1 = (uint64_t)PHILOX_MUL1 * (uint64_t)x2;
        n0 = (uint32_t)(prod1 >> 32) ^ x1 ^ k0;
        n1 = (uint32_t)prod1;
        n2 = (uint32_t)(prod0 >> 32) ^ x3 ^ k1;
        n3 = (uint32_t)prod0;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* The 32-bit uniform word for global element index gi. */
static uint32_t uniform_word(uint64_t seed, uint64_t gi)
{
    uint32_t counter[4], key[2], out[4];
    uint64_t block = gi >> 2;
    counter[0] = (uint32_t)block;
    counter[1] = (uint32_t)(block >> 32);
    counter[2] = 0u;
    counter[3] = 0u;
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    philox4x32_10(counter, key, out);
    return out[gi & 3u];
}

/* floor(p * 2^32) in double; p in [0, 1). */
static uint64_t keep_threshold(float p)
{
    return (uint64_t)floor((double)p * 4294967296.0);
}

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32.  bf16 is the upper half of an IEEE binary32.  Rounding to
 * nearest, ties to even: add 0x7FFF plus the lowest kept bit, then truncate.
 * NaNs map to the canonical quiet NaN 0x7FC0. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Element access by mode.  Values are handed around as double; in the
 * fp32/bf16 modes they are exactly representable floats. */
static double load_elem(const void* base, int64_t idx, int dtype)
{
    if (dtype == SPO_BF16) return (double)bf16_to_f32(((const uint16_t*)base)[idx]);
    if (dtype == SPO_F32) return (double)((const float*)base)[idx];
    return ((const double*)base)[idx];
}

/* Round a value once to the activation type and store it. */
static void store_elem(void* base, int64_t idx, int dtype, double v)
{
    if (dtype == SPO_BF16) ((uint16_t*)base)[idx] = f32_to_bf16((float)v);
    else if (dtype == SPO_F32) ((float*)base)[idx] = (float)v;
    else ((double*)base)[idx] = v;
}

/* The value a store then a load would give back (the rounded h). */
static double round_to_dtype(double v, int dtype)
{
    if (dtype == SPO_BF16) return (double)bf16_to_f32(f32_to_bf16((float)v));
    if (dtype == SPO_F32) return (double)(float)v;
    return v;
}

static int check_desc(const spo_desc* d)
{
    if (!d) return -1;
    if (d->S <= 0 || d->B <= 0 || d->H <= 0) return -2;
    if (d->T < 1 || d->j < 0 || d->j >= d->T) return -2;
    if (d->S % d->T != 0) return -2;
    if (d->dtype != SPO_F32 && d->dtype != SPO_BF16 && d->dtype != SPO_F64) return -3;
    if (d->norm != SPO_RMSNORM && d->norm != SPO_LAYERNORM) return -4;
    if (!(d->p >= 0.0f && d->p < 1.0f)) return -4;
    if (!(d->eps >= 0.0f)) return -4;
    return 0;
}

/* Token rows in one shard: (S/T) * B. */
static int64_t shard_rows(const spo_desc* d) { return (d->S / d->T) * d->B; }

/* ------------------------------------------------------------------ */
/* Forward over rows [row0, row0+nrows) of shard j.
 *
 * P[t]      : T pointers, each to the nrows x H block of P_t^(j) starting at
 *             shard row row0 (the caller slices the full [S,B,H] buffers).
 * residual  : nrows x H, same rows.
 * gamma,beta: H doubles (beta NULL for RMSNorm).
 * h, y      : nrows x H outputs in the activation type.
 * mask      : nrows x H bytes, 1 = kept.
 * mean      : nrows doubles (LayerNorm only; NULL for RMSNorm).
 * rstd      : nrows doubles.
 * Returns 0 or a negative code for a bad descriptor or row range. */
int sp_oracle_fwd(const spo_desc* d, int64_t row0, int64_t nrows,
                  const void* const* P, const void* residual,
                  const double* gamma, const double* beta,
                  void* h, void* y, uint8_t* mask, double* mean, double* rstd)
{
    int rc = check_desc(d);
    int64_t H, R, r, k;
    uint64_t thr;
    double scale64;
    float scale32;
    double* hrow;
    if (rc) return rc;
    H = d->H;
    R = shard_rows(d);
    if (row0 < 0 || nrows < 0 || row0 + nrows > R) return -2;
    if (d->norm == SPO_LAYERNORM && (!beta || !mean)) return -1;
    thr = keep_threshold(d->p);
    scale64 = 1.0 / (1.0 - (double)d->p);
    scale32 = (float)scale64;
    hrow = (double*)malloc(sizeof(double) * (size_t)H);
    if (!hrow) return -1;

    for (r = 0; r < nrows; ++r) {
        double sum = 0.0, sumsq = 0.0, mu = 0.0, var, rs;
        for (k = 0; k < H; ++k) {
            int64_t i = r * H + k;
            uint64_t gi = (uint64_t)((d->j * R + row0 + r) * H + k);
            int keep = uniform_word(d->seed, gi) >= thr;
            double hv;
            mask[i] = (uint8_t)keep;
            if (d->dtype == SPO_F64) {
                /* exact-arithmetic mode: no roundings anywhere */
                double acc = 0.0, z;
                int t;
                for (t = 0; t < d->T; ++t) acc += load_elem(P[t], i, SPO_F64);
                z = keep ? acc * scale64 : 0.0;
                hv = load_elem(residual, i, SPO_F64) + z;
            } else {
                /* fp32 element-wise, t ascending, one rounding of h */
                float acc = (float)load_elem(P[0], i, d->dtype);
                float z, hf;
                int t;
                for (t = 1; t < d->T; ++t) acc = acc + (float)load_elem(P[t], i, d->dtype);
                z = keep ? acc * scale32 : 0.0f;
                hf = (float)load_elem(residual, i, d->dtype) + z;
                hv = round_to_dtype((double)hf, d->dtype);
            }
            store_elem(h, i, d->dtype, hv);
            hrow[k] = hv;
        }
        if (d->norm == SPO_RMSNORM) {
            for (k = 0; k < H; ++k) sumsq += hrow[k] * hrow[k];
            rs = 1.0 / sqrt(sumsq / (double)H + (double)d->eps);
            for (k = 0; k < H; ++k)
                store_elem(y, r * H + k, d->dtype, gamma[k] * (hrow[k] * rs));
        } else {
            for (k = 0; k < H; ++k) sum += hrow[k];
            mu = sum / (double)H;
            for (k = 0; k < H; ++k) sumsq += (hrow[k] - mu) * (hrow[k] - mu);
            var = sumsq / (double)H;
            rs = 1.0 / sqrt(var + (double)d->eps);
            for (k = 0; k < H; ++k)
                store_elem(y, r * H + k, d->dtype, gamma[k] * ((hrow[k] - mu) * rs) + beta[k]);
            mean[r] = mu;
        }
        rstd[r] = rs;
    }
    free(hrow);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Backward over rows [row0, row0+nrows) of shard j.
 *
 * Inputs : dY, h (nrows x H, activation type), mask (bytes), mean (LayerNorm;
 *          NULL for RMSNorm) and rstd (nrows doubles), gamma (H doubles),
 *          dR (optional nrows x H extra gradient of the residual stream h;
 *          NULL = none).
 * Outputs: d_res = dL/dh (the residual input's gradient), dP = d_res scaled by
 *          mask/(1-p) (the same gradient for every partial P_t: the backward of
 *          a sum copies the gradient to each addend), dgamma / dbeta = sums
 *          over these rows only (dbeta NULL for RMSNorm).
 * Derivation: x^ = (h - mu) * rstd, g = dY * gamma,
 *   RMSNorm  : dh = rstd * (g - x^ * mean(g x^))
 *   LayerNorm: dh = rstd * (g - mean(g) - x^ * mean(g x^))
 *   dgamma   = sum over rows of dY x^,  dbeta = sum over rows of dY. */
int sp_oracle_bwd(const spo_desc* d, int64_t row0, int64_t nrows,
                  const void* dY, const void* h, const uint8_t* mask,
                  const double* mean, const double* rstd, const double* gamma,
                  const void* dR,
                  void* d_res, void* dP, double* dgamma, double* dbeta)
{
    int rc = check_desc(d);
    int64_t H, R, r, k;
    double scale;
    double *xhat, *g;
    if (rc) return rc;
    H = d->H;
    R = shard_rows(d);
    if (row0 < 0 || nrows < 0 || row0 + nrows > R) return -2;
    if (d->norm == SPO_LAYERNORM && (!mean || !dbeta)) return -1;
    /* the element-wise modes scale by the fp32 value of 1/(1-p) */
    scale = 1.0 / (1.0 - (double)d->p);
    if (d->dtype != SPO_F64) scale = (double)(float)scale;
    xhat = (double*)malloc(sizeof(double) * (size_t)H);
    g = (double*)malloc(sizeof(double) * (size_t)H);
    if (!xhat || !g) { free(xhat); free(g); return -1; }

    for (k = 0; k < H; ++k) {
        dgamma[k] = 0.0;
        if (dbeta) dbeta[k] = 0.0;
    }
    for (r = 0; r < nrows; ++r) {
        double mu = (d->norm == SPO_LAYERNORM) ? mean[r] : 0.0;
        double rs = rstd[r];
        double c1 = 0.0, c2 = 0.0;
        for (k = 0; k < H; ++k) {
            int64_t i = r * H + k;
            double dy = load_elem(dY, i, d->dtype);
            xhat[k] = (load_elem(h, i, d->dtype) - mu) * rs;
            g[k] = dy * gamma[k];
            c1 += g[k];
            c2 += g[k] * xhat[k];
            dgamma[k] += dy * xhat[k];
            if (dbeta) dbeta[k] += dy;
        }
        c1 /= (double)H;
        c2 /= (double)H;
        for (k = 0; k < H; ++k) {
            int64_t i = r * H + k;
            double dh;
            if (d->norm == SPO_LAYERNORM) dh = rs * (g[k] - c1 - xhat[k] * c2);
            else dh = rs * (g[k] - xhat[k] * c2);
            if (dR) dh += load_elem(dR, i, d->dtype);
            store_elem(d_res, i, d->dtype, dh);
            store_elem(dP, i, d->dtype, mask[i] ? dh * scale : 0.0);
        }
    }
    free(xhat);
    free(g);
    (void)R;
    return 0;
}

/* ------------------------------------------------------------------ */
/* The raw 32-bit words for global indices start .. start+n-1 (for pinning the
 * generator against an independent implementation). */
void sp_oracle_uniform_words(uint64_t seed, uint64_t start, int64_t n, uint32_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = uniform_word(seed, start + (uint64_t)i);
}

/* Keep mask for global indices start .. start+n-1 at probability p. */
void sp_oracle_keep_mask(uint64_t seed, float p, uint64_t start, int64_t n, uint8_t* out)
{
    uint64_t thr = keep_threshold(p);
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)(uniform_word(seed, start + (uint64_t)i) >= thr);
}

/* fp32 -> bf16 round-to-nearest-even on an array (pinned against a library cast). */
void sp_oracle_f32_to_bf16(const float* in, int64_t n, uint16_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}
