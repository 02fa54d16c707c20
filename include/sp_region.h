/*
 * sp_region.h -- C ABI of the sequence-parallel (SP) region kernels for MI355X (gfx950).
 *
 * The SP region is the stretch of a transformer block between two
 * tensor-parallel (TP) regions that runs on a sequence shard.
 *
 *   "MiniMind-tron: Sequence Parallelism" (anker661.github.io), sections 3.1,
 *   3.2.1 and 3.2.4: a row-parallel linear leaves each of the T TP ranks with a
 *   full-shape partial P_t:[S,B,H]; a reduce-scatter hands rank j the summed
 *   block Y^(j) = sum_t P_t^(j) of S/T consecutive sequence positions
 *   ([S/T,B,H], S % T == 0); dropout, residual add and RMSNorm then run on that
 *   shard (section 3.2.2).
 *   "Sequence Parallel" (formulaic.cloudchewie.com), sections "basic idea" and
 *   "MLP activation size": LayerNorm over the hidden axis; dropout keeps a
 *   one-byte 0/1 mask and its backward multiplies the gradient by that mask.
 *   "MiniMind-tron: SP optimisation", section 4.2.1.1: the norm is computed in
 *   fp32 and cast back to the activation type.
 *
 * One call processes shard j of one rank with all T partials resident in this
 * GPU's memory: it performs the local arithmetic of the reduce-scatter plus the
 * region's element-wise and per-token work, forward or backward, in one pass
 * over HBM.
 *
 * Conventions for every entry point
 *   Layout     Activations are [S,B,H] row-major; shard j is the contiguous slab
 *              of R = (S/T)*B token rows starting at element j*R*H.  Tensors
 *              named "shard" below are R x H; "full" ones are S*B x H.
 *   Memory     Every tensor pointer is a DEVICE pointer; P is a HOST array of T
 *              device pointers.  The caller owns all memory; the library never
 *              allocates, frees or synchronises.
 *   Alignment  Tensor pointers must be 16-byte aligned and H * element_size a
 *              multiple of 16 bytes (else SP_EALIGN / SP_ESHAPE).
 *   Aliasing   Outputs may not overlap inputs or each other (SP_EINVAL).
 *   Streams    `stream` is a hipStream_t (NULL = the default stream).  Work is
 *              enqueued and the call returns; outputs are valid once the stream
 *              reaches that point.
 *   Errors     Argument errors are returned synchronously, before anything is
 *              enqueued.  A failed launch returns SP_EHIP (the text is kept for
 *              sp_region_strerror).  Calls are thread-safe.  The library keeps
 *              no state of its own apart from the per-GPU scratch array of
 *              sp_region_bwd_noalloc; the backward's workspace carries arrival
 *              counts from call to call (see sp_region_bwd).
 *   Empty      S == 0 or B == 0 is an empty shard: the forward enqueues
 *              nothing, the backward writes zeros to dgamma/dbeta.
 */
#ifndef SP_REGION_H
#define SP_REGION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SP_MAX_T 64          /* largest number of partials */
#define SP_MAX_H_BYTES 131072 /* largest row: H * element_size */
#define SP_NOALLOC_SCRATCH_BYTES (32u << 20) /* scratch held by sp_region_bwd_noalloc, per GPU */

/* activation element type */
enum { SP_F32 = 0, SP_BF16 = 1 };
/* normalisation */
enum { SP_RMSNORM = 0, SP_LAYERNORM = 1 };
/* descriptor flags */
enum {
    /* Keep no mask tensor: the forward stores none (mask_out must be NULL) and the
     * backward regenerates the keep flags from (seed, global index) (mask must be
     * NULL).  Saves one byte per element in each direction; the flags are the same
     * bits either way. */
    SP_FLAG_RECOMPUTE_MASK = 1
};
/* status codes */
enum {
    SP_OK = 0,
    SP_EINVAL = -1,      /* NULL / overlapping / inconsistent pointer arguments */
    SP_ESHAPE = -2,      /* bad S, B, H, T or j */
    SP_EDTYPE = -3,      /* unknown dtype */
    SP_EPARAM = -4,      /* bad norm, p, eps */
    SP_EALIGN = -5,      /* pointer not 16-byte aligned */
    SP_EWORKSPACE = -6,  /* workspace missing or too small */
    SP_EHIP = -7,        /* the HIP runtime refused the launch */
    SP_ESCRATCH = -8     /* sp_region_bwd_noalloc: the shape needs more than SP_NOALLOC_SCRATCH_BYTES */
};

typedef struct sp_desc {
    int64_t S, B, H;   /* full activation [S,B,H]; S >= 0, B >= 0, H > 0 */
    int32_t T;         /* number of partials = TP size, 1 <= T <= SP_MAX_T, S % T == 0 */
    int32_t j;         /* shard index, 0 <= j < T */
    int32_t dtype;     /* SP_F32 or SP_BF16, for every activation tensor */
    int32_t norm;      /* SP_RMSNORM (gamma only) or SP_LAYERNORM (gamma, beta) */
    float eps;         /* added to the mean square / variance; finite, >= 0 */
    float p;           /* dropout probability, 0 <= p < 1 */
    uint64_t seed;     /* dropout generator key */
    uint32_t flags;    /* SP_FLAG_* bits; unknown bits are rejected (SP_EPARAM) */
    uint32_t reserved; /* must be 0 */
} sp_desc_t;

/*
 * Forward of the SP region on shard j.
 *
 * For each token row r of the shard and hidden index k, with i = r*H + k and
 * global index gi = j*R*H + i into the full [S,B,H] tensor:
 *   y32  = P_0[gi] + P_1[gi] + ... + P_{T-1}[gi]     fp32, t ascending
 *   keep = word(seed, gi) >= floor(p * 2^32)          Philox4x32-10, Salmon et
 *          al. SC'11: counter (lo, hi of gi >> 2, 0, 0), key (lo, hi of seed),
 *          output word gi & 3 -- the mask depends only on (seed, gi), so it is
 *          the same whatever T and j are
 *   h    = round(residual[i] + (keep ? y32 * (1/(1-p)) : +0))   fp32, one rounding
 *   RMSNorm  : rstd = 1/sqrt(mean_k h^2 + eps),              y = gamma * h * rstd
 *   LayerNorm: mean = mean_k h, rstd = 1/sqrt(var_k h + eps), y = gamma * (h - mean) * rstd + beta
 * Statistics use the rounded h, in fp32; y is rounded once.
 *
 * P         HOST array of T device pointers, each a full [S,B,H] partial;
 *           only its rows of shard j are read.
 * residual  shard, activation type.
 * gamma     [H] fp32.  beta: [H] fp32 for LayerNorm, NULL for RMSNorm.
 * h_out     shard: the residual stream after the add (saved for the backward).
 * y_out     shard: the normalised output (what the next all-gather consumes).
 * mask_out  shard of bytes, 1 = kept, 0 = dropped (NULL with SP_FLAG_RECOMPUTE_MASK).
 * mean_out  [R] fp32 for LayerNorm, NULL for RMSNorm.
 * rstd_out  [R] fp32.
 */
int sp_region_fwd(const sp_desc_t* d, const void* const* P, const void* residual,
                  const float* gamma, const float* beta,
                  void* h_out, void* y_out, uint8_t* mask_out,
                  float* mean_out, float* rstd_out, void* stream);

/*
 * Backward of the SP region on shard j: the derivative of the forward above.
 *
 *   "Sequence Parallel" (formulaic.cloudchewie.com), section "MLP activation
 *   size": the backward of dropout multiplies the incoming gradient by the
 *   saved 0/1 mask (here with the forward's 1/(1-p) scale, inverted dropout).
 *   "MiniMind-tron: Sequence Parallelism", section 3.3.3.1: the forward sums
 *   the partials, and the backward of a sum hands every addend the same
 *   gradient, so one dP serves all T partials P_t.  Section 3.4.2.1: the norm
 *   weights are replicated while each rank sees only its S/T tokens, so the
 *   dgamma / dbeta of one shard are partial sums that still have to be summed
 *   over the T ranks (outside this call).
 *   The norm derivatives themselves are not printed on the pages; they are the
 *   standard ones of the forward's formulas:
 *
 *   xhat = (h - mean) * rstd  (mean = 0 for RMSNorm),  g = dY * gamma
 *   RMSNorm  : dh = rstd * (g - xhat * mean_k(g * xhat))
 *   LayerNorm: dh = rstd * (g - mean_k(g) - xhat * mean_k(g * xhat))
 *   dh += dR (when given)
 *   d_residual = round(dh);  dP = round(keep ? dh * (1/(1-p)) : +0)
 *   dgamma[k] = sum_r dY * xhat;  dbeta[k] = sum_r dY   (this shard's rows only)
 *
 * dY        shard gradient of y.  h, mask (NULL with SP_FLAG_RECOMPUTE_MASK), mean
 *           (LayerNorm; NULL for RMSNorm), rstd: as saved by sp_region_fwd.
 *           gamma: [H] fp32.
 * dR        optional shard: an extra gradient of the residual stream h from its
 *           other consumer (the next residual add); NULL = none.
 * d_residual, dP   shard outputs, activation type.
 * dgamma    [H] fp32, overwritten.  dbeta: [H] fp32 for LayerNorm, NULL for RMSNorm.
 * workspace device scratch of at least sp_region_bwd_workspace_size(d) bytes,
 *           16-byte aligned, zero-filled before the first call that uses it.
 *           Its first 4096 bytes hold arrival counts; each count wraps back to
 *           zero on the last arrival of every call, so one zero fill at
 *           allocation serves every later call, for any descriptor, as long as
 *           only sp_region_bwd writes the buffer.  The rest is scratch.  Calls
 *           that share a workspace must be ordered on one stream: calls that
 *           overlap in time race on it.  A call that never completes (its
 *           kernel stopped part way) can leave counts that are not zero; the
 *           next call on that workspace may then return dgamma / dbeta computed
 *           from stale scratch, or NaN where a count is out of range.  Zero the
 *           workspace again after such an event.  When the size is 0 the
 *           workspace is not touched and may be NULL.
 *
 * dgamma / dbeta are fp32 sums in a fixed order, so repeated calls give the same
 * bits.  Two schedules exist, chosen from the shape (sp_region_bwd_schedule):
 * per-workgroup partial rows in the workspace summed by a second kernel, or
 * column workgroups inside the one launch, each summing a strip of columns over
 * a segment of rows; where a strip has several segments, the workgroup that
 * completes it adds them in segment order.  That hand-over between workgroups
 * uses device-scope atomic stores, a drain of the stores (s_waitcnt) and an
 * integer atomic count, and relies on gfx950 performing device-scope accesses
 * at the device's point of coherence; it uses no release/acquire fence.
 */
int sp_region_bwd(const sp_desc_t* d, const void* dY, const void* h, const uint8_t* mask,
                  const float* mean, const float* rstd, const float* gamma,
                  const void* dR,
                  void* d_residual, void* dP, float* dgamma, float* dbeta,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * sp_region_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments, outputs and results are those of
 * sp_region_bwd (bit for bit); the scratch comes from a static device array of
 * SP_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until
 * the process ends, looked up on the first call on each device (that call also
 * clears its arrival counts, with a kernel on `stream`).  The call itself
 * allocates nothing.
 *
 * Returns SP_ESCRATCH, before anything is enqueued, when the descriptor needs
 * more than SP_NOALLOC_SCRATCH_BYTES (sp_region_bwd_workspace_size(d) says how
 * much it needs); then use sp_region_bwd with a workspace of that size.
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * contents: calls that overlap in time on one GPU (other streams, other host
 * threads) race on it and must be ordered by the caller.
 */
int sp_region_bwd_noalloc(const sp_desc_t* d, const void* dY, const void* h, const uint8_t* mask,
                          const float* mean, const float* rstd, const float* gamma,
                          const void* dR,
                          void* d_residual, void* dP, float* dgamma, float* dbeta, void* stream);

/* Bytes of workspace sp_region_bwd needs for this descriptor: 0 when it needs
 * none (then the workspace may be NULL) and on a bad descriptor.  Host only;
 * the layout of the workspace is described at sp_region_bwd. */
size_t sp_region_bwd_workspace_size(const sp_desc_t* d);

/* The dgamma / dbeta schedule sp_region_bwd takes for this descriptor: 0 =
 * partial rows plus a finish kernel; k >= 1 = column workgroups with k row
 * segments per strip (k = 1 needs no workspace); a negative status for a bad
 * descriptor.  Host only; for tests and tuning. */
int sp_region_bwd_schedule(const sp_desc_t* d);

/*
 * Algorithmic HBM bytes of one call: every input read once and every output
 * written once (fwd: T partial slabs, residual, h, y, mask, stats, gamma/beta;
 * bwd: dY, h, mask, stats, gamma, d_residual, dP, dgamma/dbeta; dR not counted;
 * no mask bytes with SP_FLAG_RECOMPUTE_MASK).
 *
 *   "MiniMind-tron: SP optimisation", section 4.2.1: the pages count memory in
 *   units of F = 2 bytes x S*B*H, one full-sequence bf16 [S,B,H] tensor (6 MiB
 *   for B=2, S=2048, H=768).  One shard's tensor is F/T; a bf16 forward moves
 *   (2T+7) bytes per shard element and the backward 9, so fwd = (T+3.5) F/T and
 *   bwd = 4.5 F/T, plus the [R] statistics and [H] parameters.
 *
 * Returns SP_OK or the validation error of the descriptor; fwd_bytes and
 * bwd_bytes must be non-NULL (SP_EINVAL).
 */
int sp_region_traffic_bytes(const sp_desc_t* d, uint64_t* fwd_bytes, uint64_t* bwd_bytes);

/* Static text for a status code (for SP_EHIP: the text of the last launch error
 * this thread saw from the library).  The library never calls hipGetLastError,
 * so an error left pending by the caller's own work stays pending for it. */
const char* sp_region_strerror(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int sp_region_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SP_REGION_H */
