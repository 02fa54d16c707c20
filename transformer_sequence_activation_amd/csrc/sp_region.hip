// sp_region.hip -- sequence-parallel region kernels for MI355X (gfx950, CDNA4).
//
// What is computed is defined in include/sp_region.h (with the passages of the
// pages it follows).  This file is the device code and the C-ABI host side.
//
// Design (gfx950):
//   * One HBM pass per direction.  A token row of H elements is owned by a
//     "row group" of TPR lanes (16..64 lanes of one wavefront, or 2..16 whole
//     wavefronts); each lane owns CPT 16-byte chunks of the row (8 bf16 or 4
//     fp32 elements), so every global load and store is a coalesced dwordx4.
//   * All T partial chunks and the residual chunk are loaded before any of them
//     is used, so a lane keeps (T+1)*CPT 16-byte loads in flight.
//   * The row statistics are reduced in registers: DPP quad_perm / row mirrors
//     inside 16-lane rows, ds_swizzle across 32 lanes, ds_bpermute across the
//     wavefront, and a few LDS words only when a row spans several wavefronts.
//     Every lane of a row ends with bit-identical statistics.
//   * The dropout mask is a counter-based Philox4x32-10 keyed on (seed, global
//     element index): one generator call gives the four words of four
//     consecutive elements, so a bf16 chunk costs two calls and no state is
//     kept between launches.
//   * dgamma/dbeta have two schedules, chosen per shape by the host.  Column
//     workgroups: the first workgroups of the backward launch each sum a
//     128-byte column strip over one segment of rows (dY and h read a second
//     time); with several segments per strip, the last segment to arrive adds
//     them (an integer arrival count in the workspace, no second launch).
//     Partial rows: the row workgroups accumulate their columns in registers,
//     write one fp32 partial row each, and a second small kernel sums those
//     rows.  Every sum has a fixed order: no float atomics, results are
//     run-to-run identical.
//   * No MFMA: nothing here is a contraction; the path is bound by HBM.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "sp_region.h"

#ifndef SP_BWD_TARGET_BLOCKS
#define SP_BWD_TARGET_BLOCKS 0  // > 0: workgroups the backward aims for; 0 = the variant's own figure
#endif

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Activation element types: a 16-byte chunk holds E elements.

template <int DT>
struct Act;

template <>
struct Act<SP_BF16> {
    static constexpr int E = 8;
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ void unpack(const u32x4 v, float (&f)[8]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f[2 * m] = __uint_as_float(v[m] << 16);
            f[2 * m + 1] = __uint_as_float(v[m] & 0xFFFF0000u);
        }
    }
    // fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 under the default
    // rounding mode), two elements per instruction.
    static __device__ __forceinline__ u32x4 pack(const float (&f)[8]) {
        u32x4 v;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x2 pr = {f[2 * m], f[2 * m + 1]};
            v[m] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
        }
        return v;
    }
};

template <>
struct Act<SP_F32> {
    static constexpr int E = 4;
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ void unpack(const u32x4 v, float (&f)[4]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) f[m] = __uint_as_float(v[m]);
    }
    static __device__ __forceinline__ u32x4 pack(const float (&f)[4]) {
        u32x4 v;
#pragma unroll
        for (int m = 0; m < 4; ++m) v[m] = __float_as_uint(f[m]);
        return v;
    }
};

// Streaming 16-byte accesses: every activation byte is touched once per launch.
#ifndef SP_NT_LOADS
#define SP_NT_LOADS 1
#endif
#ifndef SP_NT_STORES
#define SP_NT_STORES 1
#endif
#ifndef SP_EARLY_FLAGS
#define SP_EARLY_FLAGS 1  // forward with T <= 2: keep flags made while the loads are in flight
#endif
#ifndef SP_EARLY_FLAGS_MAX_T
#define SP_EARLY_FLAGS_MAX_T 2  // the largest fixed T whose forward makes its flags early
#endif
#ifndef SP_BWD_EARLY_FLAGS
#define SP_BWD_EARLY_FLAGS 1  // mask-free backward, 2+ rows in flight: the same for its flags
#endif
__device__ __forceinline__ u32x4 ld16(const void* base, int64_t byte_off) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + byte_off);
#if SP_NT_LOADS
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
// dY and h in the backward.  Under the column schedule they are read twice (by
// the row and by the column workgroups), so both reads use ordinary loads,
// which leave the lines in the caches for the other read; otherwise the row
// workgroups stream them like every other tensor.
#ifndef SP_COL_NT
#define SP_COL_NT 0
#endif
#ifndef SP_ROWS_NT
#define SP_ROWS_NT 1  // partial-row schedule: dY and h by streaming loads
#endif
#ifndef SP_COL_FIRST
#define SP_COL_FIRST 1  // column workgroups take the first blockIdx values of the backward grid
#endif
constexpr bool kColFirst = SP_COL_FIRST != 0;
template <bool NT>
__device__ __forceinline__ u32x4 ld16_policy(const void* base, int64_t byte_off) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + byte_off);
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
__device__ __forceinline__ u32x4 ld16_col(const void* base, int64_t byte_off) {
    return ld16_policy<SP_COL_NT != 0>(base, byte_off);
}
__device__ __forceinline__ void st16(void* base, int64_t byte_off, u32x4 v) {
    u32x4* p = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + byte_off);
#if SP_NT_STORES
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64
// multiplies whose halves are mixed into the other counter words with the round
// key; the key advances by two Weyl constants between rounds.  Counter words 2
// and 3 are zero here.

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ void philox10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1,
                                         uint32_t (&w)[4]) {
    uint32_t x0 = c0, x1 = c1, x2 = 0u, x3 = 0u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        const uint64_t p0 = (uint64_t)kPhiloxM0 * x0;
        const uint64_t p1 = (uint64_t)kPhiloxM1 * x2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        x1 = (uint32_t)p1;
        x3 = (uint32_t)p0;
        x0 = n0;
        x2 = n2;
    }
    w[0] = x0;
    w[1] = x1;
    w[2] = x2;
    w[3] = x3;
}

// Keep flags of the E elements starting at global index gi0 (a multiple of E).
template <int E>
__device__ __forceinline__ void keep_flags(uint64_t gi0, uint32_t thr, uint32_t k0, uint32_t k1,
                                           bool (&keep)[E]) {
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
        const uint64_t c = (gi0 >> 2) + (uint64_t)q;
        uint32_t w[4];
        philox10((uint32_t)c, (uint32_t)(c >> 32), k0, k1, w);
#pragma unroll
        for (int m = 0; m < 4; ++m) keep[4 * q + m] = w[m] >= thr;
    }
}

// ---------------------------------------------------------------------------
// Reductions over a row group of TPR lanes; every lane gets the same bits.

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int TPR>
__device__ __forceinline__ float lanes_sum(float v) {
    static_assert(TPR >= 16, "row groups span at least one 16-lane DPP row");
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp<0x141>(v);  // row_half_mirror: the other quad of the 8
    v += dpp<0x140>(v);  // row_mirror: the other 8 of the 16
    if constexpr (TPR >= 32)
        v += __builtin_bit_cast(
            float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));  // lane ^ 16
    if constexpr (TPR >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Sum NV values over the TPR lanes of each row group of a BLOCK-thread block.
// Must be reached by every thread of the block (it may synchronise).
// REUSE: the LDS words are written again later in the kernel, so wait for every
// wavefront to have read them before returning.
template <int TPR, int BLOCK, int NV, bool REUSE = true>
__device__ __forceinline__ void group_sum(float (&v)[NV]) {
    if constexpr (TPR > kWave && TPR % kWave != 0) {
        // Row groups of a multiple of 32 lanes that wavefronts do not tile (96):
        // each aligned 32-lane group sums its lanes, then the groups of a row are
        // added in order through LDS.
        static_assert(TPR % 32 == 0, "row groups are whole 32-lane groups");
        constexpr int NG = TPR / 32;
        constexpr int RPW = BLOCK / TPR;
        __shared__ float red[RPW * NG * NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = lanes_sum<32>(v[i]);
        const int tid = threadIdx.x;
        const int rg = tid / TPR;
        const int g = (tid % TPR) / 32;
        if ((tid & 31) == 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i) red[(rg * NG + g) * NV + i] = v[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float t = red[(rg * NG) * NV + i];
#pragma unroll
            for (int q = 1; q < NG; ++q) t += red[(rg * NG + q) * NV + i];
            v[i] = t;
        }
        if constexpr (REUSE) __syncthreads();
        return;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = lanes_sum<TPR>(v[i]);
    if constexpr (TPR > kWave) {
        constexpr int NW = TPR / kWave;
        constexpr int RPW = BLOCK / TPR;
        __shared__ float red[RPW * NW * NV];
        const int tid = threadIdx.x;
        const int rg = tid / TPR;
        const int w = (tid % TPR) / kWave;
        if ((tid & (kWave - 1)) == 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i) red[(rg * NW + w) * NV + i] = v[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float s = red[(rg * NW) * NV + i];
#pragma unroll
            for (int q = 1; q < NW; ++q) s += red[(rg * NW + q) * NV + i];
            v[i] = s;
        }
        if constexpr (REUSE) __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Forward.

struct FwdArgs {
    const void* P[SP_MAX_T];  // each points at the first element of shard j of P_t
    const void* residual;
    const float* gamma;
    const float* beta;
    void* h;
    void* y;
    uint8_t* mask;   // NULL: keep no mask
    float* mean;
    float* rstd;
    int64_t R;       // token rows in the shard
    uint64_t base;   // global index of the shard's first element (j * R * H)
    int32_t H;
    int32_t nchunk;  // H / E
    int32_t T;
    int32_t norm;
    uint32_t thr;    // keep iff word >= thr
    uint32_t key0, key1;
    float scale;     // 1 / (1 - p) in fp32
    float eps;
    float inv_h;
};

// h = round(residual + (keep ? sum * scale : +0)), fp32 and unfused, so that
// the product and the sum each round once.
template <int E>
__device__ __forceinline__ void residual_add(const float (&acc)[E], const float (&res)[E],
                                             const bool (&keep)[E], float scale, float (&hf)[E]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float z = keep[e] ? acc[e] * scale : 0.0f;
        hf[e] = res[e] + z;
    }
}

template <int E>
struct MaskWord;
template <>
struct MaskWord<8> {
    typedef uint2 type;
    static __device__ __forceinline__ uint2 make(const bool (&k)[8]) {
        uint2 m;
        m.x = (uint32_t)k[0] | ((uint32_t)k[1] << 8) | ((uint32_t)k[2] << 16) | ((uint32_t)k[3] << 24);
        m.y = (uint32_t)k[4] | ((uint32_t)k[5] << 8) | ((uint32_t)k[6] << 16) | ((uint32_t)k[7] << 24);
        return m;
    }
    static __device__ __forceinline__ void unmake(uint2 m, bool (&k)[8]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            k[e] = (m.x >> (8 * e)) & 0xFFu;
            k[4 + e] = (m.y >> (8 * e)) & 0xFFu;
        }
    }
};
template <>
struct MaskWord<4> {
    typedef uint32_t type;
    static __device__ __forceinline__ uint32_t make(const bool (&k)[4]) {
        return (uint32_t)k[0] | ((uint32_t)k[1] << 8) | ((uint32_t)k[2] << 16) | ((uint32_t)k[3] << 24);
    }
    static __device__ __forceinline__ void unmake(uint32_t m, bool (&k)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) k[e] = (m >> (8 * e)) & 0xFFu;
    }
};

template <int E>
__device__ __forceinline__ void load_vec_f32(const float* p, int64_t idx, float (&f)[E]) {
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p + idx + 4 * q);
#pragma unroll
        for (int m = 0; m < 4; ++m) f[4 * q + m] = v[m];
    }
}

// TT: number of partials fixed at compile time (0 = read a.T at run time).
// RPT: rows a row group takes at once (all their loads in flight together).
template <int DT, int TT, int TPR, int CPT, int BLOCK, int RPT>
__global__ __launch_bounds__(BLOCK) void sp_fwd_kernel(const FwdArgs a) {
    using A = Act<DT>;
    constexpr int E = A::E;
    constexpr int EB = A::kBytes;
    constexpr int RPW = BLOCK / TPR;
    using MW = MaskWord<E>;

    const int tid = threadIdx.x;
    const int rg = tid / TPR;
    const int l = tid % TPR;
    const int64_t row0 = ((int64_t)blockIdx.x * RPW + rg) * RPT;

    int col[CPT];
    bool ok[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int c = l + k * TPR;
        ok[k] = c < a.nchunk;
        col[k] = (ok[k] ? c : a.nchunk - 1) * E;
    }

    if constexpr (BLOCK > 512 && CPT > 2) {
        // Rows too long for every partial chunk to sit in registers at once: the
        // chunks go through in batches of KB and h stays packed (16 bytes per
        // chunk) for the statistics and y.  Same arithmetic, same order.
        static_assert(RPT == 1, "long rows are taken one at a time");
        const int64_t row = row0;
        const bool row_ok = row < a.R;
        const int64_t rowc = row_ok ? row : a.R - 1;  // loads stay in bounds; stores are predicated
        const int64_t row_elem = rowc * (int64_t)a.H;
        constexpr int KB = (TT > 0 && TT < 4) ? 2 : 1;
        u32x4 hp[CPT];
        float s1 = 0.0f;  // LayerNorm: sum of h; RMSNorm: sum of h^2
#pragma unroll
        for (int k0 = 0; k0 < CPT; k0 += KB) {
            float acc[KB][E], res[KB][E];
            if constexpr (TT > 0) {
                u32x4 pv[KB][TT], rv[KB];
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    if (k0 + kk >= CPT) continue;
                    const int64_t off = (row_elem + col[k0 + kk]) * EB;
#pragma unroll
                    for (int t = 0; t < TT; ++t) pv[kk][t] = ld16(a.P[t], off);
                    rv[kk] = ld16(a.residual, off);
                }
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    if (k0 + kk >= CPT) continue;
                    A::unpack(pv[kk][0], acc[kk]);
#pragma unroll
                    for (int t = 1; t < TT; ++t) {
                        float f[E];
                        A::unpack(pv[kk][t], f);
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[kk][e] = acc[kk][e] + f[e];
                    }
                    A::unpack(rv[kk], res[kk]);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    if (k0 + kk >= CPT) continue;
                    const int64_t off = (row_elem + col[k0 + kk]) * EB;
                    const u32x4 rv = ld16(a.residual, off);
                    A::unpack(ld16(a.P[0], off), acc[kk]);
                    for (int t = 1; t < a.T; ++t) {
                        float f[E];
                        A::unpack(ld16(a.P[t], off), f);
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[kk][e] = acc[kk][e] + f[e];
                    }
                    A::unpack(rv, res[kk]);
                }
            }
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int k = k0 + kk;
                if (k >= CPT) continue;
                const int64_t idx = row_elem + col[k];
                bool keep[E];
                keep_flags<E>(a.base + (uint64_t)idx, a.thr, a.key0, a.key1, keep);
                float hf[E], hv[E];
                residual_add<E>(acc[kk], res[kk], keep, a.scale, hf);
                hp[k] = A::pack(hf);
                A::unpack(hp[k], hv);
                if (row_ok && ok[k]) {
                    st16(a.h, idx * EB, hp[k]);
                    if (a.mask) *reinterpret_cast<typename MW::type*>(a.mask + idx) = MW::make(keep);
                }
                if (ok[k]) {
#pragma unroll
                    for (int e = 0; e < E; ++e) s1 += a.norm == SP_LAYERNORM ? hv[e] : hv[e] * hv[e];
                }
            }
        }
        float mu = 0.0f, rs;
        float q[1] = {s1};
        if (a.norm == SP_LAYERNORM) {
            group_sum<TPR, BLOCK, 1>(q);
            mu = q[0] * a.inv_h;
            q[0] = 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                if (!ok[k]) continue;
                float hv[E];
                A::unpack(hp[k], hv);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float dlt = hv[e] - mu;
                    q[0] += dlt * dlt;
                }
            }
        }
        group_sum<TPR, BLOCK, 1, false>(q);
        rs = rsqrtf(q[0] * a.inv_h + a.eps);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float hv[E], gm[E], yv[E];
            A::unpack(hp[k], hv);
            load_vec_f32<E>(a.gamma, col[k], gm);
            if (a.norm == SP_LAYERNORM) {
                float bt[E];
                load_vec_f32<E>(a.beta, col[k], bt);
#pragma unroll
                for (int e = 0; e < E; ++e) yv[e] = gm[e] * ((hv[e] - mu) * rs) + bt[e];
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) yv[e] = gm[e] * (hv[e] * rs);
            }
            if (row_ok && ok[k]) st16(a.y, (row_elem + col[k]) * EB, A::pack(yv));
        }
        if (row_ok && l == 0) {
            a.rstd[row] = rs;
            if (a.norm == SP_LAYERNORM) a.mean[row] = mu;
        }
        return;
    }

    // ---- loads: every partial chunk and the residual of the RPT rows, issued together ----
    bool rok[RPT];
    int64_t relem[RPT];  // first element of each row (a valid row: loads stay in bounds)
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int64_t r = row0 + p;
        rok[p] = r < a.R;
        relem[p] = (rok[p] ? r : a.R - 1) * (int64_t)a.H;
    }
    float acc[RPT][CPT][E];
    float res[RPT][CPT][E];
    // With few partials the generator is a visible share of the work: its flags
    // (one bit per element) are then made while the loads are in flight.
    constexpr bool kEarlyFlags = SP_EARLY_FLAGS && TT > 0 && TT <= SP_EARLY_FLAGS_MAX_T;
    uint32_t kbits[RPT][CPT];
    if constexpr (TT > 0) {
        u32x4 pv[RPT][CPT][TT];
        u32x4 rv[RPT][CPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p)
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                const int64_t off = (relem[p] + col[k]) * EB;
#pragma unroll
                for (int t = 0; t < TT; ++t) pv[p][k][t] = ld16(a.P[t], off);
                rv[p][k] = ld16(a.residual, off);
            }
        if constexpr (kEarlyFlags) {
#pragma unroll
            for (int p = 0; p < RPT; ++p)
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    bool kf[E];
                    keep_flags<E>(a.base + (uint64_t)(relem[p] + col[k]), a.thr, a.key0, a.key1, kf);
                    kbits[p][k] = 0;
#pragma unroll
                    for (int e = 0; e < E; ++e) kbits[p][k] |= (uint32_t)kf[e] << e;
                }
        }
#pragma unroll
        for (int p = 0; p < RPT; ++p)
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                A::unpack(pv[p][k][0], acc[p][k]);
#pragma unroll
                for (int t = 1; t < TT; ++t) {
                    float f[E];
                    A::unpack(pv[p][k][t], f);
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[p][k][e] = acc[p][k][e] + f[e];
                }
                A::unpack(rv[p][k], res[p][k]);
            }
    } else {
        u32x4 rv[RPT][CPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p)
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                const int64_t off = (relem[p] + col[k]) * EB;
                rv[p][k] = ld16(a.residual, off);
                A::unpack(ld16(a.P[0], off), acc[p][k]);
            }
        for (int t = 1; t < a.T; ++t) {
#pragma unroll
            for (int p = 0; p < RPT; ++p)
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    float f[E];
                    A::unpack(ld16(a.P[t], (relem[p] + col[k]) * EB), f);
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[p][k][e] = acc[p][k][e] + f[e];
                }
        }
#pragma unroll
        for (int p = 0; p < RPT; ++p)
#pragma unroll
            for (int k = 0; k < CPT; ++k) A::unpack(rv[p][k], res[p][k]);
    }

    // gamma / beta for the normalisation, loaded early
    float gam[CPT][E], bet[CPT][E];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        load_vec_f32<E>(a.gamma, col[k], gam[k]);
        if (a.norm == SP_LAYERNORM) load_vec_f32<E>(a.beta, col[k], bet[k]);
    }

    // ---- dropout + residual add, one rounding of h ----
    float hv[RPT][CPT][E];
#pragma unroll
    for (int p = 0; p < RPT; ++p)
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t idx = relem[p] + col[k];
            bool keep[E];
            if constexpr (kEarlyFlags) {
#pragma unroll
                for (int e = 0; e < E; ++e) keep[e] = (kbits[p][k] >> e) & 1u;
            } else {
                keep_flags<E>(a.base + (uint64_t)idx, a.thr, a.key0, a.key1, keep);
            }
            float hf[E];
            residual_add<E>(acc[p][k], res[p][k], keep, a.scale, hf);
            const u32x4 hp = A::pack(hf);
            A::unpack(hp, hv[p][k]);  // the rounded h the norm sees
            if (rok[p] && ok[k]) {
                st16(a.h, idx * EB, hp);
                if (a.mask) *reinterpret_cast<typename MW::type*>(a.mask + idx) = MW::make(keep);
            }
        }

    // ---- per-token statistics (the RPT rows' sums reduced together) ----
    float mu[RPT], rs[RPT];
    if (a.norm == SP_LAYERNORM) {
        float s[RPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            s[p] = 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
                if (ok[k])
#pragma unroll
                    for (int e = 0; e < E; ++e) s[p] += hv[p][k][e];
        }
        group_sum<TPR, BLOCK, RPT>(s);
        float q[RPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            mu[p] = s[p] * a.inv_h;
            q[p] = 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
                if (ok[k])
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float dlt = hv[p][k][e] - mu[p];
                        q[p] += dlt * dlt;
                    }
        }
        group_sum<TPR, BLOCK, RPT, false>(q);
#pragma unroll
        for (int p = 0; p < RPT; ++p) rs[p] = rsqrtf(q[p] * a.inv_h + a.eps);
    } else {
        float q[RPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            mu[p] = 0.0f;
            q[p] = 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
                if (ok[k])
#pragma unroll
                    for (int e = 0; e < E; ++e) q[p] += hv[p][k][e] * hv[p][k][e];
        }
        group_sum<TPR, BLOCK, RPT, false>(q);
#pragma unroll
        for (int p = 0; p < RPT; ++p) rs[p] = rsqrtf(q[p] * a.inv_h + a.eps);
    }

    // ---- y = gamma * xhat (+ beta), one rounding ----
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float yv[E];
            if (a.norm == SP_LAYERNORM) {
#pragma unroll
                for (int e = 0; e < E; ++e) yv[e] = gam[k][e] * ((hv[p][k][e] - mu[p]) * rs[p]) + bet[k][e];
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) yv[e] = gam[k][e] * (hv[p][k][e] * rs[p]);
            }
            if (rok[p] && ok[k]) st16(a.y, (relem[p] + col[k]) * EB, A::pack(yv));
        }
        if (rok[p] && l == 0) {
            a.rstd[row0 + p] = rs[p];
            if (a.norm == SP_LAYERNORM) a.mean[row0 + p] = mu[p];
        }
    }
}

// ---------------------------------------------------------------------------
// Backward.

struct BwdArgs {
    const void* dY;
    const void* h;
    const uint8_t* mask;
    const float* mean;
    const float* rstd;
    const float* gamma;
    const void* dR;
    void* dres;
    void* dP;
    float* ws;            // [G][nacc][H] fp32 partial sums of dgamma (, dbeta) per row workgroup,
                          // or [segments][nacc][H] per column segment
    uint32_t* col_count;  // [strips] arrivals of a strip's column segments, zero between calls
    float* dgamma;        // [H] outputs, written directly by the column workgroups
    float* dbeta;
    uint64_t base;        // global index of the shard's first element (mask regeneration)
    uint32_t thr, key0, key1;
    int64_t R;
    int64_t rows_per_block;
    int32_t H;
    int32_t nchunk;
    int32_t norm;
    int32_t nacc;         // 1 (RMSNorm) or 2 (LayerNorm)
    int32_t col_blocks;   // leading workgroups that sum dgamma / dbeta by columns (0 = partial rows)
    int32_t col_strips;   // column strips; col_blocks / col_strips segments of rows per strip
    int64_t col_seg_rows; // rows per segment
    float scale;
    float inv_h;
};

// One token row's backward inputs as loaded (packed).
template <int CPT, int E>
struct BwdRow {
    u32x4 dy[CPT];
    u32x4 hh[CPT];
    u32x4 dr[CPT];
    typename MaskWord<E>::type m[CPT];
    float mu, rs;
};

template <int DT, bool LN, int CPT, bool HAS_DR, bool REGEN, bool NT>
__device__ __forceinline__ void bwd_load(const BwdArgs& a, int64_t rowc, const int (&col)[CPT],
                                         BwdRow<CPT, Act<DT>::E>& b) {
    using A = Act<DT>;
    constexpr int E = A::E;
    constexpr int EB = A::kBytes;
    const int64_t row_elem = rowc * (int64_t)a.H;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int64_t idx = row_elem + col[k];
        b.dy[k] = ld16_policy<NT && SP_NT_LOADS>(a.dY, idx * EB);
        b.hh[k] = ld16_policy<NT && SP_NT_LOADS>(a.h, idx * EB);
        if constexpr (HAS_DR) b.dr[k] = ld16(a.dR, idx * EB);
        if constexpr (!REGEN) b.m[k] = *reinterpret_cast<const typename MaskWord<E>::type*>(a.mask + idx);
    }
    b.rs = a.rstd[rowc];
    b.mu = LN ? a.mean[rowc] : 0.0f;
}

// The PF rows one row group takes in step `it` (rows past the tile's end are
// loaded from a valid row and never stored).
template <int DT, bool LN, int CPT, int PF, bool HAS_DR, bool REGEN, bool NT>
__device__ __forceinline__ void bwd_load_step(const BwdArgs& a, int64_t row0, int64_t row_end,
                                              const int (&col)[CPT],
                                              BwdRow<CPT, Act<DT>::E> (&rows)[PF]) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int64_t r = row0 + p;
        bwd_load<DT, LN, CPT, HAS_DR, REGEN, NT>(a, r < row_end ? r : a.R - 1, col, rows[p]);
    }
}

// dgamma / dbeta by columns.  A column workgroup owns one strip of kSeg adjacent
// 16-byte chunks (128 bytes of every row, lanes kSeg apart share a chunk) and
// one segment of contiguous rows, and sums dY * xhat (and dY) over them: its
// BLOCK / kSeg row offsets each take every (BLOCK / kSeg)-th row in ascending
// order, then the offsets are added in a fixed tree (lane butterfly inside a
// wavefront, wavefronts in order through LDS).  With one segment per strip
// that sum is dgamma.  With several, each segment publishes its sums and counts
// itself in (the count wraps back to zero on the last arrival); the workgroup
// that completes the strip adds the segments in segment order.  The order of every addition
// is fixed, whichever workgroup finishes last.  Needs no second launch, at the
// cost of reading dY and h a second time.
#ifndef SP_COL_BATCH
#define SP_COL_BATCH 8
#endif
constexpr int kColBatch = SP_COL_BATCH;
// 1024-lane workgroups have half the registers per lane: half the batch (the
// same rows per batch, as there are twice the row offsets).
constexpr int col_batch(int block) { return block > 512 ? (kColBatch + 1) / 2 : kColBatch; }
#ifndef SP_COL_SEG
#define SP_COL_SEG 8
#endif
constexpr int kSeg = SP_COL_SEG;  // lanes per row segment (16 bytes each)

template <int DT, bool LN, int BLOCK>
__device__ __forceinline__ void bwd_columns(const BwdArgs& a, int wg) {
    using A = Act<DT>;
    constexpr int E = A::E;
    constexpr int EB = A::kBytes;
    constexpr int NACC = LN ? 2 : 1;
    constexpr int kRO = BLOCK / kSeg;  // row offsets
    constexpr int kB = col_batch(BLOCK);  // steps whose loads are in flight together
    constexpr int NW = BLOCK / kWave;
    __shared__ float cred[NW][NACC][kSeg * E];
    __shared__ uint32_t arrived;

    const int strip = wg % a.col_strips;
    const int seg = wg / a.col_strips;
    const int nseg = a.col_blocks / a.col_strips;
    const int64_t row_lo = (int64_t)seg * a.col_seg_rows;
    const int64_t row_hi = min(row_lo + a.col_seg_rows, a.R);
    const int tid = threadIdx.x;
    const int ch = tid % kSeg;
    const int ro = tid / kSeg;
    const int c = strip * kSeg + ch;
    const bool cok = c < a.nchunk;
    const int col = (cok ? c : a.nchunk - 1) * E;
    float dg[E], db[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        dg[e] = 0.0f;
        db[e] = 0.0f;
    }
    for (int64_t r0 = row_lo; r0 < row_hi; r0 += (int64_t)kRO * kB) {
        u32x4 dy[kB], hh[kB];
        float mu[kB], rs[kB];
        bool rok[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            const int64_t row = r0 + (int64_t)b * kRO + ro;
            rok[b] = row < row_hi;
            const int64_t rr = rok[b] ? row : row_hi - 1;
            const int64_t off = (rr * a.H + col) * EB;
            dy[b] = ld16_col(a.dY, off);
            hh[b] = ld16_col(a.h, off);
            rs[b] = a.rstd[rr];
            mu[b] = LN ? a.mean[rr] : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            float dyv[E], hv[E];
            A::unpack(dy[b], dyv);
            A::unpack(hh[b], hv);
            if (rok[b]) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = (hv[e] - mu[b]) * rs[b];
                    dg[e] += dyv[e] * x;
                    if constexpr (LN) db[e] += dyv[e];
                }
            }
        }
    }
    // the row offsets inside a wavefront (lanes kSeg, 2 kSeg, ... apart), then the wavefronts
#pragma unroll
    for (int m = kSeg; m < kWave; m *= 2) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            dg[e] += __shfl_xor(dg[e], m);
            if constexpr (LN) db[e] += __shfl_xor(db[e], m);
        }
    }
    const int w = tid / kWave;
    if (tid % kWave < kSeg) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            cred[w][0][ch * E + e] = dg[e];
            if constexpr (LN) cred[w][1][ch * E + e] = db[e];
        }
    }
    __syncthreads();
    const bool mine = tid < NACC * kSeg * E;
    const int acc = tid / (kSeg * E);
    const int gcol = strip * kSeg * E + tid % (kSeg * E);
    const bool live = mine && gcol < a.H;
    float v = 0.0f;
    if (mine) {
        const int cc = tid % (kSeg * E);
        v = cred[0][acc][cc];
#pragma unroll
        for (int q = 1; q < NW; ++q) v += cred[q][acc][cc];
    }
    float* const out = acc == 0 ? a.dgamma : a.dbeta;
    if (nseg == 1) {  // uniform over the grid
        if (live) out[gcol] = v;
        return;
    }
    // Several segments: publish this one's sums, then count in.  The sums go
    // out as device-scope (agent) atomic stores and every wave drains them
    // (s_waitcnt) before the barrier, so they have reached the device's point of
    // coherence before the count is taken; the workgroup that completes the
    // strip reads them back with device-scope atomic loads, issued after its
    // count returned.  This relies on gfx950 performing device-scope stores and
    // loads at that point (they bypass the XCD-private caches), not on a
    // release/acquire pair: a device fence would write back every dirty line of
    // the XCD's L2, the d_residual and dP tiles included (on 2048 rows of 768
    // the backward took 20.5 us with fences, 8.7 us without).
    float* const part = a.ws + ((int64_t)seg * NACC + acc) * a.H + gcol;
    if (live) __hip_atomic_store(part, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // The count wraps to zero on the strip's last arrival (atomicInc with bound
    // nseg - 1), so every completed call leaves it at zero.  A count above
    // nseg - 1 can only be left by a call that never completed, or by calls of
    // different shapes racing on one workspace: the strip's outputs are then
    // NaN instead of sums read from segments that may be stale.
    if (tid == 0) arrived = atomicInc(a.col_count + strip, (uint32_t)(nseg - 1));
    __syncthreads();
    const uint32_t before = arrived;  // uniform over the workgroup
    if (before < (uint32_t)(nseg - 1)) return;
    if (before > (uint32_t)(nseg - 1)) {
        if (live) out[gcol] = __builtin_nanf("");
        return;
    }
    if (live) {
        // every segment's sum, in segment order; the loads of a batch are in
        // flight together
        const float* src = a.ws + (int64_t)acc * a.H + gcol;
        const int64_t stride = (int64_t)NACC * a.H;
        constexpr int kRead = 8;
        float t = 0.0f;
        for (int q0 = 0; q0 < nseg; q0 += kRead) {
            float sv[kRead];
#pragma unroll
            for (int b = 0; b < kRead; ++b)
                sv[b] = q0 + b < nseg
                            ? __hip_atomic_load(src + (q0 + b) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0.0f;
#pragma unroll
            for (int b = 0; b < kRead; ++b) {
                if (q0 + b == 0) t = sv[b];
                else if (q0 + b < nseg) t += sv[b];
            }
        }
        out[gcol] = t;
    }
}

// A workgroup holds RG row groups of TPR lanes and walks a tile of
// rows_per_block rows.  In each step every row group takes PF rows whose loads
// are all in flight together, reduces the PF rows' two sums in one pass, then
// writes their gradients.  Without COLS, dgamma (and dbeta) accumulate in
// registers and each workgroup writes one partial row; with COLS the first
// col_blocks workgroups are column workgroups (bwd_columns) and the row
// workgroups leave dgamma alone.  With REGEN the keep flags are generated again
// from (seed, global index) instead of read from a mask tensor.
template <int DT, int NORM, int TPR, int CPT, int RG, int PF, bool HAS_DR, bool REGEN, bool COLS>
__global__ __launch_bounds__(RG* TPR) void sp_bwd_kernel(const BwdArgs a) {
    using A = Act<DT>;
    constexpr bool LN = NORM == SP_LAYERNORM;
    constexpr int E = A::E;
    constexpr int EB = A::kBytes;
    constexpr int BLOCK = RG * TPR;
    constexpr int STEP = RG * PF;  // rows per step of the workgroup
    constexpr int NACC = LN ? 2 : 1;
    using MW = MaskWord<E>;
    extern __shared__ float comb[];  // [RG][NACC][H] when RG > 1

    const int tid = threadIdx.x;
    const int rg = tid / TPR;
    const int l = tid % TPR;
    // the column workgroups come first in the grid, or after the row workgroups
    const int nrow_wg = (int)gridDim.x - a.col_blocks;
    const int col_wg = kColFirst ? (int)blockIdx.x : (int)blockIdx.x - nrow_wg;
    const int row_wg = kColFirst ? (int)blockIdx.x - a.col_blocks : (int)blockIdx.x;
    if constexpr (COLS) {
        if (col_wg >= 0 && col_wg < a.col_blocks) {  // uniform over the workgroup
            bwd_columns<DT, LN, BLOCK>(a, col_wg);
            return;
        }
    }
    constexpr bool partial_rows = !COLS;
    const int64_t row_begin = (int64_t)row_wg * a.rows_per_block;
    const int64_t row_end = min(row_begin + a.rows_per_block, a.R);
    const int iters = (int)((a.rows_per_block + STEP - 1) / STEP);  // uniform over the grid

    int col[CPT];
    bool ok[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const int c = l + k * TPR;
        ok[k] = c < a.nchunk;
        col[k] = (ok[k] ? c : a.nchunk - 1) * E;
    }
    // gamma: held in registers, or (long rows, 1024-lane workgroups) read again
    // where it is used -- a small array that stays in the caches
    constexpr bool kGammaRegs = !(BLOCK > 512 && CPT > 2);
    float gam[CPT][E];
    if constexpr (kGammaRegs) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) load_vec_f32<E>(a.gamma, col[k], gam[k]);
    }

    float dg[CPT][E], db[CPT][LN ? E : 1];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
#pragma unroll
        for (int e = 0; e < E; ++e) dg[k][e] = 0.0f;
#pragma unroll
        for (int e = 0; e < (LN ? E : 1); ++e) db[k][e] = 0.0f;
    }

    BwdRow<CPT, E> rows[PF];
    // streaming loads of dY and h unless the column workgroups read them again
    auto load_step = [&](int64_t r0, BwdRow<CPT, E>(&dst)[PF]) {
        bwd_load_step<DT, LN, CPT, PF, HAS_DR, REGEN, !COLS && SP_ROWS_NT>(a, r0, row_end, col, dst);
    };
    // regenerated keep flags (one bit per element), made right after a step's
    // loads are issued so that the generator runs while they are in flight;
    // measured to pay where several rows are in flight per row group
    constexpr bool kEarly = REGEN && SP_BWD_EARLY_FLAGS && PF >= 2;
    uint32_t kb[kEarly ? PF : 1][kEarly ? CPT : 1];
    auto gen_flags = [&](int64_t r0) {
        if constexpr (kEarly) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                const int64_t row = r0 + p;
                const int64_t re = (row < row_end ? row : 0) * (int64_t)a.H;
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    bool kf[E];
                    keep_flags<E>(a.base + (uint64_t)(re + col[k]), a.thr, a.key0, a.key1, kf);
                    kb[p][k] = 0;
#pragma unroll
                    for (int e = 0; e < E; ++e) kb[p][k] |= (uint32_t)kf[e] << e;
                }
            }
        }
    };
    load_step(row_begin + (int64_t)rg * PF, rows);
    gen_flags(row_begin + (int64_t)rg * PF);
    for (int it = 0; it < iters; ++it) {
        const int64_t row0 = row_begin + (int64_t)it * STEP + (int64_t)rg * PF;
        // pass 1: the two row sums of every row, and the dgamma / dbeta terms
        float s[2 * PF];
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const bool row_ok = row0 + p < row_end;
            s[2 * p] = 0.0f;
            s[2 * p + 1] = 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float dyv[E], hv[E], gk[E];
                A::unpack(rows[p].dy[k], dyv);
                A::unpack(rows[p].hh[k], hv);
                if constexpr (!kGammaRegs) load_vec_f32<E>(a.gamma, col[k], gk);
                if (ok[k]) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float x = (hv[e] - rows[p].mu) * rows[p].rs;
                        const float g = dyv[e] * (kGammaRegs ? gam[k][e] : gk[e]);
                        if constexpr (LN) s[2 * p] += g;
                        s[2 * p + 1] += g * x;
                        if (row_ok && partial_rows) {
                            dg[k][e] += dyv[e] * x;
                            if constexpr (LN) db[k][e] += dyv[e];
                        }
                    }
                }
            }
        }
        group_sum<TPR, BLOCK, 2 * PF>(s);
        // pass 2: dh, d_residual, dP
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int64_t row = row0 + p;
            const bool row_ok = row < row_end;
            const float c1 = LN ? s[2 * p] * a.inv_h : 0.0f;
            const float c2 = s[2 * p + 1] * a.inv_h;
            const int64_t row_elem = (row_ok ? row : 0) * (int64_t)a.H;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float dyv[E], hv[E], drv[E], dh[E], dp[E], gk[E];
                bool keep[E];
                A::unpack(rows[p].dy[k], dyv);
                A::unpack(rows[p].hh[k], hv);
                if constexpr (!kGammaRegs) load_vec_f32<E>(a.gamma, col[k], gk);
                if constexpr (HAS_DR) A::unpack(rows[p].dr[k], drv);
                if constexpr (kEarly) {
#pragma unroll
                    for (int e = 0; e < E; ++e) keep[e] = (kb[p][k] >> e) & 1u;
                } else if constexpr (REGEN) {
                    keep_flags<E>(a.base + (uint64_t)(row_elem + col[k]), a.thr, a.key0, a.key1, keep);
                } else {
                    MW::unmake(rows[p].m[k], keep);
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = (hv[e] - rows[p].mu) * rows[p].rs;
                    const float g = dyv[e] * (kGammaRegs ? gam[k][e] : gk[e]);
                    float v = rows[p].rs * (g - c1 - x * c2);
                    if constexpr (HAS_DR) v += drv[e];
                    dh[e] = v;
                    dp[e] = keep[e] ? v * a.scale : 0.0f;
                }
                if (row_ok && ok[k]) {
                    const int64_t off = (row_elem + col[k]) * EB;
                    st16(a.dres, off, A::pack(dh));
                    st16(a.dP, off, A::pack(dp));
                }
            }
        }
        if (it + 1 < iters) {
            load_step(row0 + STEP, rows);
            gen_flags(row0 + STEP);
        }
    }

    // ---- this workgroup's partial dgamma / dbeta row ----
    if constexpr (COLS) return;
    float* out = a.ws + (int64_t)row_wg * NACC * a.H;
    if constexpr (RG == 1) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            if (!ok[k]) continue;
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                f32x4 v = {dg[k][4 * q], dg[k][4 * q + 1], dg[k][4 * q + 2], dg[k][4 * q + 3]};
                *reinterpret_cast<f32x4*>(out + col[k] + 4 * q) = v;
                if constexpr (LN) {
                    f32x4 w = {db[k][4 * q], db[k][4 * q + 1], db[k][4 * q + 2], db[k][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(out + a.H + col[k] + 4 * q) = w;
                }
            }
        }
    } else {
        const int H = a.H;
        float* mine = comb + (int64_t)rg * NACC * H;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            if (!ok[k]) continue;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                mine[col[k] + e] = dg[k][e];
                if constexpr (LN) mine[H + col[k] + e] = db[k][e];
            }
        }
        __syncthreads();
        const int n = NACC * H;
        for (int c = tid; c < n; c += BLOCK) {
            float v = comb[c];
#pragma unroll
            for (int q = 1; q < RG; ++q) v += comb[(int64_t)q * n + c];
            out[c] = v;
        }
    }
}

// dgamma[k] (and dbeta[k]) = sum over the G workgroup partials, in a fixed
// order.  A block covers kFinGroups groups of four adjacent columns (one 16-byte
// load each) and splits the G partial rows into kFinSlices contiguous slices, one
// per lane; a lane issues all of its slice's loads before adding them in order,
// then the slices are added in a fixed tree (lane butterfly inside a wavefront,
// the wavefronts in order through LDS).
#ifndef SP_FIN_SLICES
#define SP_FIN_SLICES 32
#endif
#ifndef SP_FIN_GROUPS
#define SP_FIN_GROUPS 8
#endif
constexpr int kFinGroups = SP_FIN_GROUPS;
constexpr int kFinSlices = SP_FIN_SLICES;
static_assert(kWave % kFinGroups == 0 && (kFinGroups * kFinSlices) % kWave == 0,
              "a wavefront holds whole slices of every column group");
constexpr int kFinBatch = 8;

__global__ __launch_bounds__(kFinGroups* kFinSlices) void sp_dgamma_finish_kernel(
    const float* ws, int64_t G, int32_t H, int32_t nacc, float* dgamma, float* dbeta) {
    constexpr int NW = kFinGroups * kFinSlices / kWave;
    __shared__ f32x4 part[NW][kFinGroups];
    const int n = nacc * H;  // a multiple of 4
    const int cg = threadIdx.x % kFinGroups;
    const int sl = threadIdx.x / kFinGroups;
    const int c = (blockIdx.x * kFinGroups + cg) * 4;
    const int64_t per = (G + kFinSlices - 1) / kFinSlices;
    const int64_t g0 = sl * per;
    const int64_t g1 = min(g0 + per, G);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c < n) {
        const float* src = ws + c;
        int64_t g = g0;
        for (; g + kFinBatch <= g1; g += kFinBatch) {
            f32x4 v[kFinBatch];
#pragma unroll
            for (int b = 0; b < kFinBatch; ++b)
                v[b] = *reinterpret_cast<const f32x4*>(src + (g + b) * n);
#pragma unroll
            for (int b = 0; b < kFinBatch; ++b) acc += v[b];
        }
        for (; g < g1; ++g) acc += *reinterpret_cast<const f32x4*>(src + g * n);
    }
    // the slices of one wavefront by a lane butterfly, then the wavefronts in order
#pragma unroll
    for (int m = kFinGroups; m < kWave; m *= 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], m);
    }
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave < kFinGroups) part[w][cg] = acc;
    __syncthreads();
    if (threadIdx.x < kFinGroups && c < n) {
        f32x4 t = part[0][cg];
#pragma unroll
        for (int q = 1; q < NW; ++q) t += part[q][cg];
        float* dst = c < H ? dgamma + c : dbeta + (c - H);
        *reinterpret_cast<f32x4*>(dst) = t;
    }
}

// Zero n words (the arrival counts of a workspace that starts in an unknown
// state); a kernel rather than a memset, so that it can sit in a captured graph.
__global__ __launch_bounds__(256) void sp_clear_counts_kernel(uint32_t* p, int32_t n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Launch layouts: (lanes per row, chunks per lane) by row length in chunks.

struct Layout {
    int tpr, cpt, limit;  // the default choice for rows of up to `limit` chunks
};
// X(lanes per row, chunks per lane, longest row it is chosen for, ...), in
// increasing limit: the first whose limit holds the row is used.  One chunk per
// lane wherever a row fills most of a power-of-two lane group (more wavefronts
// per SIMD to hide the arithmetic); rows of 113-128 chunks measured faster at
// two chunks per lane.  The host table and the kernel tables below are both
// generated from this list.
#define SP_LAYOUT_LIST(X, ...)                                                                  \
    X(16, 1, 16, __VA_ARGS__), X(32, 1, 32, __VA_ARGS__), X(64, 1, 64, __VA_ARGS__),            \
        X(128, 1, 88, __VA_ARGS__), X(96, 1, 96, __VA_ARGS__), X(128, 1, 112, __VA_ARGS__),     \
        X(64, 2, 128, __VA_ARGS__), X(256, 1, 256, __VA_ARGS__),                                 \
        X(512, 1, 512, __VA_ARGS__), X(512, 2, 1024, __VA_ARGS__), X(512, 4, 2048, __VA_ARGS__), \
        X(1024, 4, 4096, __VA_ARGS__), X(1024, 8, 8192, __VA_ARGS__)
#define SP_LAYOUT_STRUCT(TPR, CPT, LIMIT, ...) Layout{TPR, CPT, LIMIT}
constexpr Layout kLayouts[] = {SP_LAYOUT_LIST(SP_LAYOUT_STRUCT, 0)};
constexpr int kNumLayouts = sizeof(kLayouts) / sizeof(kLayouts[0]);
constexpr bool layouts_ok() {
    for (int i = 0; i < kNumLayouts; ++i) {
        if (kLayouts[i].tpr * kLayouts[i].cpt < kLayouts[i].limit) return false;
        if (i > 0 && kLayouts[i].limit <= kLayouts[i - 1].limit) return false;
    }
    return kLayouts[kNumLayouts - 1].limit == SP_MAX_H_BYTES / 16;
}
static_assert(layouts_ok(), "each layout holds its rows; limits increase up to the longest row");
#ifndef SP_SUBWAVE_BLOCK
#define SP_SUBWAVE_BLOCK 256
#endif
constexpr int kSubWaveBlock = SP_SUBWAVE_BLOCK;  // block size of the layouts whose rows fit in one wavefront

// Row groups larger than a wavefront take one row per workgroup, except the
// 96-lane ones, which take two (three whole wavefronts).
constexpr int block_of(int tpr) { return tpr <= kWave ? kSubWaveBlock : (tpr % kWave ? 2 * tpr : tpr); }

// Compile-time overrides (layout indices) used when tuning; -1 = default choice.
#ifndef SP_FWD_LAYOUT
#define SP_FWD_LAYOUT -1
#endif
#ifndef SP_FWD_RPT
#define SP_FWD_RPT 1  // rows per forward row group (tuning builds: 2)
#endif
#ifndef SP_BWD_VARIANT
#define SP_BWD_VARIANT -1
#endif

// Backward launch variants: X(lanes per row, chunks per lane, row groups per
// workgroup, rows in flight per row group, workgroups aimed for, ...).  The
// first twelve are the default choices in increasing capacity; the last serves
// the column schedule.  The host table and the kernel tables are both generated
// from this list.
struct BwdVariant {
    int tpr, cpt, rg, pf, blocks;
};
#define SP_BWD_LIST(X, ...)                                                                          \
    X(16, 1, 16, 1, 256, __VA_ARGS__), X(32, 1, 8, 1, 256, __VA_ARGS__), X(64, 1, 4, 1, 256, __VA_ARGS__), \
        X(32, 3, 8, 1, 256, __VA_ARGS__), X(64, 2, 4, 1, 256, __VA_ARGS__),                                \
        X(64, 3, 4, 1, 256, __VA_ARGS__), X(64, 4, 4, 1, 256, __VA_ARGS__),                                \
        X(512, 1, 1, 2, 256, __VA_ARGS__), X(512, 2, 1, 1, 512, __VA_ARGS__),                              \
        X(512, 4, 1, 1, 256, __VA_ARGS__), X(1024, 4, 1, 1, 256, __VA_ARGS__),                             \
        X(1024, 8, 1, 1, 256, __VA_ARGS__), X(512, 1, 1, 4, 256, __VA_ARGS__)
#define SP_BWD_STRUCT(TPR, CPT, RG, PF, BLOCKS, ...) BwdVariant{TPR, CPT, RG, PF, BLOCKS}
constexpr BwdVariant kBwdVariants[] = {SP_BWD_LIST(SP_BWD_STRUCT, 0)};
constexpr int kNumBwdVariants = sizeof(kBwdVariants) / sizeof(kBwdVariants[0]);
constexpr int kNumBwdDefault = 12;
// Under the column schedule the (512, 1) rows take 4 rows in flight instead of 2.
constexpr int kBwdCol512From = 7, kBwdCol512To = 12;
static_assert(kBwdVariants[kBwdCol512From].tpr == 512 && kBwdVariants[kBwdCol512From].cpt == 1 &&
                  kBwdVariants[kBwdCol512To].tpr == 512 && kBwdVariants[kBwdCol512To].cpt == 1 &&
                  kBwdVariants[kBwdCol512To].rg == kBwdVariants[kBwdCol512From].rg,
              "the column-schedule swap keeps the row layout and block size");
#ifndef SP_COL_MIN_SEGS
#define SP_COL_MIN_SEGS 1  // row segments per column strip at least (tuning)
#endif
#ifndef SP_COL_ROW_BLOCKS
#define SP_COL_ROW_BLOCKS 256  // row + column workgroups the column schedule aims for
#endif
#ifndef SP_COL_ROW_BLOCKS_SMALL
#define SP_COL_ROW_BLOCKS_SMALL 256  // the same for workgroups of 256 lanes or fewer
#endif
constexpr int64_t col_row_blocks(int block) { return block <= 256 ? SP_COL_ROW_BLOCKS_SMALL : SP_COL_ROW_BLOCKS; }

typedef void (*FwdKernel)(FwdArgs);
typedef void (*BwdKernel)(BwdArgs);

// Rows too long to keep every partial chunk in registers are taken one at a time,
// in batches of chunks; every other layout may take several rows per row group.
constexpr bool fwd_batched(int tpr, int cpt) { return block_of(tpr) > 512 && cpt > 2; }
constexpr int fwd_rpt(int tpr, int cpt, int rpt) { return fwd_batched(tpr, cpt) ? 1 : rpt; }
#define SP_FWD_ENTRY(TPR, CPT, LIMIT, DT, TT, RPT) \
    &sp_fwd_kernel<DT, TT, TPR, CPT, block_of(TPR), fwd_rpt(TPR, CPT, RPT)>
#define SP_BWD_ENTRY(TPR, CPT, RG, PF, BLOCKS, DT, NORM, HDR, REGEN, COLS) \
    &sp_bwd_kernel<DT, NORM, TPR, CPT, RG, PF, HDR, REGEN, COLS>

// [fixed T: run time, 1, 2, 4, 8][layout]
const FwdKernel kFwdBf16[5][kNumLayouts] = {
    {SP_LAYOUT_LIST(SP_FWD_ENTRY, SP_BF16, 0, SP_FWD_RPT)}, {SP_LAYOUT_LIST(SP_FWD_ENTRY, SP_BF16, 1, SP_FWD_RPT)},
    {SP_LAYOUT_LIST(SP_FWD_ENTRY, SP_BF16, 2, SP_FWD_RPT)}, {SP_LAYOUT_LIST(SP_FWD_ENTRY, SP_BF16, 4, SP_FWD_RPT)},
    {SP_LAYOUT_LIST(SP_FWD_ENTRY, SP_BF16, 8, SP_FWD_RPT)},
};
const FwdKernel kFwdF32[kNumLayouts] = {SP_LAYOUT_LIST(SP_FWD_ENTRY, SP_F32, 0, SP_FWD_RPT)};
// [dtype][norm][has dR][mask regenerated][column schedule][variant]
#define SP_BWD_BY_REGEN(DT, NORM, HDR, REGEN)                      \
    {{SP_BWD_LIST(SP_BWD_ENTRY, DT, NORM, HDR, REGEN, false)},     \
     {SP_BWD_LIST(SP_BWD_ENTRY, DT, NORM, HDR, REGEN, true)}}
#define SP_BWD_BY_DR(DT, NORM, HDR) \
    {SP_BWD_BY_REGEN(DT, NORM, HDR, false), SP_BWD_BY_REGEN(DT, NORM, HDR, true)}
#define SP_BWD_BY_NORM(DT)                                                                       \
    {{SP_BWD_BY_DR(DT, SP_RMSNORM, false), SP_BWD_BY_DR(DT, SP_RMSNORM, true)},                  \
     {SP_BWD_BY_DR(DT, SP_LAYERNORM, false), SP_BWD_BY_DR(DT, SP_LAYERNORM, true)}}
const BwdKernel kBwd[2][2][2][2][2][kNumBwdVariants] = {SP_BWD_BY_NORM(SP_F32), SP_BWD_BY_NORM(SP_BF16)};

// ---------------------------------------------------------------------------
// Host-side validation.

thread_local char g_hip_error[256] = "no HIP error recorded";

inline int elem_bytes(int dtype) { return dtype == SP_BF16 ? 2 : 4; }
inline int elems_per_chunk(int dtype) { return 16 / elem_bytes(dtype); }

int check_desc(const sp_desc_t* d) {
    if (!d) return SP_EINVAL;
    if (d->dtype != SP_F32 && d->dtype != SP_BF16) return SP_EDTYPE;
    if (d->norm != SP_RMSNORM && d->norm != SP_LAYERNORM) return SP_EPARAM;
    if (!(d->p >= 0.0f && d->p < 1.0f)) return SP_EPARAM;
    if (!(d->eps >= 0.0f) || !isfinite(d->eps)) return SP_EPARAM;
    if ((d->flags & ~(uint32_t)SP_FLAG_RECOMPUTE_MASK) != 0 || d->reserved != 0) return SP_EPARAM;
    if (d->S < 0 || d->B < 0 || d->H <= 0) return SP_ESHAPE;
    if (d->T < 1 || d->T > SP_MAX_T) return SP_ESHAPE;
    if (d->j < 0 || d->j >= d->T) return SP_ESHAPE;
    if (d->S % d->T != 0) return SP_ESHAPE;
    const int64_t eb = elem_bytes(d->dtype);
    if ((d->H * eb) % 16 != 0 || d->H * eb > SP_MAX_H_BYTES) return SP_ESHAPE;
    // element indices of the full tensor must fit in 63 bits
    if (d->S > 0 && d->B > 0 && (d->B > INT64_MAX / d->S || d->S * d->B > INT64_MAX / d->H / eb))
        return SP_ESHAPE;
    return SP_OK;
}

inline int64_t shard_rows(const sp_desc_t* d) { return (d->S / d->T) * d->B; }

// keep iff word >= floor(p * 2^32), the product taken in double; p < 1 keeps it below 2^32.
inline uint32_t keep_threshold(float p) { return (uint32_t)floor((double)p * 4294967296.0); }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};
inline Span span(const void* p, int64_t bytes) {
    return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Every output span against every other span.
bool any_overlap(const Span* outs, int nout, const Span* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int k = i + 1; k < nout; ++k)
            if (overlap(outs[i], outs[k])) return true;
        for (int k = 0; k < nin; ++k)
            if (overlap(outs[i], ins[k])) return true;
    }
    return false;
}

int capacity(int li) { return kLayouts[li].tpr * kLayouts[li].cpt; }

int pick_layout(int64_t nchunk, int forced) {
    if (forced >= 0 && forced < kNumLayouts && nchunk <= capacity(forced)) return forced;
    for (int i = 0; i < kNumLayouts; ++i)
        if (nchunk <= kLayouts[i].limit) return i;
    return -1;
}

int fwd_tt_index(int T) {
    switch (T) {
        case 1: return 1;
        case 2: return 2;
        case 4: return 3;
        case 8: return 4;
        default: return 0;
    }
}

int pick_bwd_variant(int64_t nchunk, int forced) {
    auto cap = [](int v) { return kBwdVariants[v].tpr * kBwdVariants[v].cpt; };
    if (forced >= 0 && forced < kNumBwdVariants && nchunk <= cap(forced)) return forced;
    for (int i = 0; i < kNumBwdDefault; ++i)
        if (nchunk <= cap(i)) return i;
    return -1;
}

struct BwdPlan {
    int variant;
    int64_t rows_per_block;
    int64_t blocks;
    int block;
    int nacc;
    size_t ws_bytes;
    size_t lds_bytes;
    int64_t col_blocks;  // > 0: dgamma / dbeta by column workgroups, no finish launch
    int64_t col_strips;
    int64_t col_seg_rows;
};

// A workspace starts with one arrival count per column strip (zero between
// calls, written only by column segments); partial sums follow.
constexpr size_t kWsCountBytes = 4096;
static_assert((size_t)SP_MAX_H_BYTES / 16 / kSeg * sizeof(uint32_t) <= kWsCountBytes,
              "a count for every strip of the longest row");

// dgamma / dbeta strategy: 0 = by estimated bytes, 1 = partial rows + finish
// kernel, 2 = column workgroups.
#ifndef SP_BWD_DG
#define SP_BWD_DG 0
#endif
// Rows a column workgroup takes in one batch of loads: one segment at most, so
// that no column walk becomes the critical path of the launch.
constexpr int64_t col_segment_rows(int block) { return (int64_t)(block / kSeg) * col_batch(block); }

// Column workgroups read dY and h a second time (2 R H e bytes), but need no
// partial rows and no second launch; a strip's segments are joined inside the
// launch by the workgroup that completes it.  That pays where the second read
// is small enough to be served largely from the caches, a row holds a few
// strips and the rows fit in a few segments.  Measured on bf16 shards, over
// buffer sets larger than the Infinity Cache (backward us, partial rows ->
// columns): 2048 x 768 RMS 7.8 -> 7.3; a second read of 67 MB (2048 x 8192
// RMS) 36.8 -> 38.3 and of 134 MB (4096 x 8192 RMS) 65.3 -> 77.2 keep the
// partial rows; so do rows of two strips (4096 x 128 LN 6.3 / 6.5) and many
// segments (8192 x 1024 RMS, 32 segments: 19.3 / 19.4), unless all rows fit
// in one segment.  Rows of 1024-lane workgroups always take columns: there the
// partial-row schedule's per-lane dgamma / dbeta accumulators spill.
#ifndef SP_COL_MIN_STRIPS
#define SP_COL_MIN_STRIPS 4
#endif
#ifndef SP_COL_MAX_SEGS
#define SP_COL_MAX_SEGS 16
#endif
constexpr int64_t kColMaxReread = (int64_t)32 << 20;
bool use_columns(int64_t R, int64_t H, int eb, int block) {
    if (SP_BWD_DG == 1 || R == 0) return false;
    if (SP_BWD_DG == 2 || block > 512) return true;
    const int64_t strips = (H * eb / 16 + kSeg - 1) / kSeg;
    const int64_t segs = (R + col_segment_rows(block) - 1) / col_segment_rows(block);
    if (segs == 1) return true;  // no workspace, no second launch, a small re-read
    return strips >= SP_COL_MIN_STRIPS && segs <= SP_COL_MAX_SEGS && 2 * R * H * eb <= kColMaxReread;
}

BwdPlan plan_bwd(const sp_desc_t* d) {
    BwdPlan p{};
    const int64_t R = shard_rows(d), H = d->H;
    const int64_t nchunk = H / elems_per_chunk(d->dtype);
    p.nacc = d->norm == SP_LAYERNORM ? 2 : 1;
    p.variant = pick_bwd_variant(nchunk, SP_BWD_VARIANT);
    if (p.variant < 0) return p;  // unreachable for a validated descriptor
    auto tile_rows = [&](int64_t target_blocks) {
        const BwdVariant v = kBwdVariants[p.variant];
        const int step = v.rg * v.pf;  // rows a workgroup takes per step
        int64_t rpb = (R + target_blocks - 1) / target_blocks;
        rpb = ((rpb + step - 1) / step) * step;
        if (rpb < step) rpb = step;
        p.block = v.rg * v.tpr;
        p.rows_per_block = rpb;
        p.blocks = R > 0 ? (R + rpb - 1) / rpb : 0;
    };
    tile_rows(SP_BWD_TARGET_BLOCKS > 0 ? SP_BWD_TARGET_BLOCKS : kBwdVariants[p.variant].blocks);
    if (use_columns(R, H, elem_bytes(d->dtype), p.block)) {
        // Rows split into equal segments of at most one batch each.
        const int64_t most = col_segment_rows(p.block);
        int64_t segs = (R + most - 1) / most;
        if (segs < SP_COL_MIN_SEGS) segs = R < SP_COL_MIN_SEGS ? R : SP_COL_MIN_SEGS;
        p.col_seg_rows = (R + segs - 1) / segs;
        segs = (R + p.col_seg_rows - 1) / p.col_seg_rows;  // no empty segment
        p.col_strips = (nchunk + kSeg - 1) / kSeg;
        p.col_blocks = p.col_strips * segs;
        if (segs > 1)
            p.ws_bytes = kWsCountBytes + (size_t)segs * (size_t)p.nacc * (size_t)H * sizeof(float);
        // Column kernels are register-heavy (the 512-lane one fits one workgroup
        // per CU): size the row tiles so that row and column workgroups together
        // number one per CU, with all of a row workgroup's rows in flight where a
        // variant allows it.
        if (2 * p.col_blocks <= col_row_blocks(p.block)) {
            if (SP_BWD_VARIANT < 0 && p.variant == kBwdCol512From) p.variant = kBwdCol512To;
            tile_rows(col_row_blocks(p.block) - p.col_blocks);
        }
        return p;
    }
    const BwdVariant v = kBwdVariants[p.variant];
    if (p.blocks > 0) p.ws_bytes = kWsCountBytes + (size_t)p.blocks * (size_t)p.nacc * (size_t)H * sizeof(float);
    p.lds_bytes = v.rg > 1 ? (size_t)v.rg * (size_t)p.nacc * (size_t)H * sizeof(float) : 0;
    return p;
}

int record_hip(hipError_t e) {
    snprintf(g_hip_error, sizeof(g_hip_error), "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return SP_EHIP;
}

// Enqueue a kernel; its status comes from the launch call itself, so an error
// that earlier work left pending for the caller is neither cleared nor taken
// for this launch's.
int launch(const void* kernel, unsigned grid, unsigned block, size_t lds, void* stream, void** args) {
    const hipError_t e = hipLaunchKernel(kernel, dim3(grid), dim3(block), args, lds, (hipStream_t)stream);
    return e == hipSuccess ? SP_OK : record_hip(e);
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI.

extern "C" int sp_region_version(void) { return 100; }

extern "C" const char* sp_region_strerror(int status) {
    switch (status) {
        case SP_OK: return "success";
        case SP_EINVAL: return "invalid, missing or overlapping pointer argument";
        case SP_ESHAPE: return "invalid shape (S, B, H, T or j)";
        case SP_EDTYPE: return "unknown activation dtype";
        case SP_EPARAM: return "invalid norm, dropout probability or eps";
        case SP_EALIGN: return "tensor pointer not 16-byte aligned";
        case SP_EWORKSPACE: return "workspace missing or smaller than sp_region_bwd_workspace_size";
        case SP_EHIP: return g_hip_error;
        case SP_ESCRATCH: return "the shape needs more backward scratch than SP_NOALLOC_SCRATCH_BYTES";
        default: return "unknown status";
    }
}

extern "C" int sp_region_traffic_bytes(const sp_desc_t* d, uint64_t* fwd_bytes, uint64_t* bwd_bytes) {
    const int rc = check_desc(d);
    if (rc != SP_OK) return rc;
    if (!fwd_bytes || !bwd_bytes) return SP_EINVAL;
    const uint64_t R = (uint64_t)shard_rows(d), H = (uint64_t)d->H, T = (uint64_t)d->T;
    const uint64_t N = R * H, e = (uint64_t)elem_bytes(d->dtype);
    const uint64_t ln = d->norm == SP_LAYERNORM ? 1 : 0;
    const uint64_t stats = R * 4 * (1 + ln);    // rstd (+ mean)
    const uint64_t params = H * 4 * (1 + ln);   // gamma (+ beta) / dgamma (+ dbeta)
    const uint64_t mask = (d->flags & SP_FLAG_RECOMPUTE_MASK) ? 0 : N;
    // fwd: T partial slabs + residual in; h, y, mask, stats out; gamma/beta in
    *fwd_bytes = T * N * e + N * e + N * e + N * e + mask + stats + params;
    // bwd: dY, h, mask, stats, gamma in; d_residual, dP, dgamma/dbeta out
    *bwd_bytes = N * e + N * e + mask + stats + H * 4 + N * e + N * e + params;
    return SP_OK;
}

extern "C" size_t sp_region_bwd_workspace_size(const sp_desc_t* d) {
    if (check_desc(d) != SP_OK) return 0;
    return plan_bwd(d).ws_bytes;
}

extern "C" int sp_region_bwd_schedule(const sp_desc_t* d) {
    const int rc = check_desc(d);
    if (rc != SP_OK) return rc;
    const BwdPlan p = plan_bwd(d);
    return p.col_blocks > 0 ? (int)(p.col_blocks / p.col_strips) : 0;
}

extern "C" int sp_region_fwd(const sp_desc_t* d, const void* const* P, const void* residual,
                             const float* gamma, const float* beta, void* h_out, void* y_out,
                             uint8_t* mask_out, float* mean_out, float* rstd_out, void* stream) {
    int rc = check_desc(d);
    if (rc != SP_OK) return rc;
    const bool ln = d->norm == SP_LAYERNORM;
    const int64_t R = shard_rows(d), H = d->H, N = R * H;
    const int eb = elem_bytes(d->dtype);
    const int64_t base = (int64_t)d->j * N;
    // [H] parameters are always required; shard-sized tensors only when the shard has rows
    if (!gamma || ln != (beta != nullptr)) return SP_EINVAL;
    const bool regen = (d->flags & SP_FLAG_RECOMPUTE_MASK) != 0;
    if (regen && mask_out) return SP_EINVAL;
    if (R > 0) {
        if (!P || !residual || !h_out || !y_out || (!regen && !mask_out) || !rstd_out) return SP_EINVAL;
        if (ln != (mean_out != nullptr)) return SP_EINVAL;
        for (int t = 0; t < d->T; ++t)
            if (!P[t]) return SP_EINVAL;
    } else if (!ln && mean_out) {
        return SP_EINVAL;
    }
    if (R > 0)
        for (int t = 0; t < d->T; ++t)
            if (!aligned16(P[t])) return SP_EALIGN;
    if (!aligned16(residual) || !aligned16(gamma) || (beta && !aligned16(beta)) ||
        !aligned16(h_out) || !aligned16(y_out) || !aligned16(mask_out) ||
        (mean_out && !aligned16(mean_out)) || !aligned16(rstd_out))
        return SP_EALIGN;
    if (R == 0) return SP_OK;
    Span ins[SP_MAX_T + 3];
    int nin = 0;
    for (int t = 0; t < d->T; ++t)
        ins[nin++] = span((const char*)P[t] + base * eb, N * eb);
    ins[nin++] = span(residual, N * eb);
    ins[nin++] = span(gamma, H * 4);
    if (beta) ins[nin++] = span(beta, H * 4);
    Span outs[5];
    int nout = 0;
    outs[nout++] = span(h_out, N * eb);
    outs[nout++] = span(y_out, N * eb);
    if (mask_out) outs[nout++] = span(mask_out, N);
    outs[nout++] = span(rstd_out, R * 4);
    if (mean_out) outs[nout++] = span(mean_out, R * 4);
    if (any_overlap(outs, nout, ins, nin)) return SP_EINVAL;

    FwdArgs a;
    memset(&a, 0, sizeof(a));
    for (int t = 0; t < d->T; ++t) a.P[t] = (const char*)P[t] + base * eb;
    a.residual = residual;
    a.gamma = gamma;
    a.beta = beta;
    a.h = h_out;
    a.y = y_out;
    a.mask = mask_out;
    a.mean = mean_out;
    a.rstd = rstd_out;
    a.R = R;
    a.base = (uint64_t)base;
    a.H = (int32_t)H;
    a.nchunk = (int32_t)(H / elems_per_chunk(d->dtype));
    a.T = d->T;
    a.norm = d->norm;
    a.thr = keep_threshold(d->p);
    a.key0 = (uint32_t)d->seed;
    a.key1 = (uint32_t)(d->seed >> 32);
    a.scale = (float)(1.0 / (1.0 - (double)d->p));
    a.eps = d->eps;
    a.inv_h = (float)(1.0 / (double)H);

    const int li = pick_layout(a.nchunk, SP_FWD_LAYOUT);
    if (li < 0) return SP_ESHAPE;
    const Layout L = kLayouts[li];
    const int block = block_of(L.tpr);
    const int64_t rows_per_wg = (int64_t)(block / L.tpr) * fwd_rpt(L.tpr, L.cpt, SP_FWD_RPT);
    const int64_t grid = (R + rows_per_wg - 1) / rows_per_wg;
    if (grid > INT32_MAX) return SP_ESHAPE;
    const FwdKernel k = d->dtype == SP_BF16 ? kFwdBf16[fwd_tt_index(d->T)][li] : kFwdF32[li];
    void* args[] = {&a};
    return launch((const void*)k, (unsigned)grid, (unsigned)block, 0, stream, args);
}

namespace {

// The backward on a given workspace.  clear_counts: zero the workspace's
// arrival counts (a small fill kernel on the same stream) before the backward.
int bwd_enqueue(const sp_desc_t* d, const void* dY, const void* h, const uint8_t* mask, const float* mean,
                const float* rstd, const float* gamma, const void* dR, void* d_residual, void* dP, float* dgamma,
                float* dbeta, void* workspace, size_t workspace_bytes, void* stream, bool clear_counts) {
    int rc = check_desc(d);
    if (rc != SP_OK) return rc;
    const bool ln = d->norm == SP_LAYERNORM;
    // [H] tensors are always required; shard-sized tensors only when the shard has rows
    if (!gamma || !dgamma || ln != (dbeta != nullptr)) return SP_EINVAL;
    const bool regen = (d->flags & SP_FLAG_RECOMPUTE_MASK) != 0;
    if (regen && mask) return SP_EINVAL;
    if (shard_rows(d) > 0) {
        if (!dY || !h || (!regen && !mask) || !rstd || !d_residual || !dP) return SP_EINVAL;
        if (ln != (mean != nullptr)) return SP_EINVAL;
    } else if (!ln && mean) {
        return SP_EINVAL;
    }
    if (!aligned16(dY) || !aligned16(h) || !aligned16(mask) || (mean && !aligned16(mean)) ||
        !aligned16(rstd) || !aligned16(gamma) || (dR && !aligned16(dR)) || !aligned16(d_residual) ||
        !aligned16(dP) || !aligned16(dgamma) || (dbeta && !aligned16(dbeta)))
        return SP_EALIGN;
    const BwdPlan plan = plan_bwd(d);
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes)) return SP_EWORKSPACE;
    if (workspace && !aligned16(workspace)) return SP_EALIGN;
    const int64_t R = shard_rows(d), H = d->H, N = R * H;
    const int eb = elem_bytes(d->dtype);
    Span ins[8];
    int nin = 0;
    ins[nin++] = span(dY, N * eb);
    ins[nin++] = span(h, N * eb);
    if (mask) ins[nin++] = span(mask, N);
    ins[nin++] = span(rstd, R * 4);
    ins[nin++] = span(gamma, H * 4);
    if (mean) ins[nin++] = span(mean, R * 4);
    if (dR) ins[nin++] = span(dR, N * eb);
    Span outs[5];
    int nout = 0;
    outs[nout++] = span(d_residual, N * eb);
    outs[nout++] = span(dP, N * eb);
    outs[nout++] = span(dgamma, H * 4);
    if (dbeta) outs[nout++] = span(dbeta, H * 4);
    if (plan.ws_bytes > 0) outs[nout++] = span(workspace, (int64_t)plan.ws_bytes);
    if (any_overlap(outs, nout, ins, nin)) return SP_EINVAL;

    BwdArgs a;
    memset(&a, 0, sizeof(a));
    a.dY = dY;
    a.h = h;
    a.mask = mask;
    a.mean = mean;
    a.rstd = rstd;
    a.gamma = gamma;
    a.dR = dR;
    a.dres = d_residual;
    a.dP = dP;
    a.col_count = plan.ws_bytes > 0 ? (uint32_t*)workspace : nullptr;
    a.ws = plan.ws_bytes > 0 ? (float*)((char*)workspace + kWsCountBytes) : nullptr;
    a.dgamma = dgamma;
    a.dbeta = dbeta;
    a.col_blocks = (int32_t)plan.col_blocks;
    a.col_strips = (int32_t)plan.col_strips;
    a.col_seg_rows = plan.col_seg_rows;
    a.R = R;
    a.rows_per_block = plan.rows_per_block;
    a.H = (int32_t)H;
    a.nchunk = (int32_t)(H / elems_per_chunk(d->dtype));
    a.norm = d->norm;
    a.nacc = plan.nacc;
    a.scale = (float)(1.0 / (1.0 - (double)d->p));
    a.inv_h = (float)(1.0 / (double)H);
    a.base = (uint64_t)((int64_t)d->j * N);
    a.thr = keep_threshold(d->p);
    a.key0 = (uint32_t)d->seed;
    a.key1 = (uint32_t)(d->seed >> 32);

    if (plan.variant < 0) return SP_ESHAPE;
    if (plan.blocks + plan.col_blocks > INT32_MAX) return SP_ESHAPE;
    if (clear_counts) {
        uint32_t* counts = (uint32_t*)workspace;
        int32_t n = (int32_t)(kWsCountBytes / sizeof(uint32_t));
        void* args[] = {&counts, &n};
        rc = launch((const void*)sp_clear_counts_kernel, (unsigned)((n + 255) / 256), 256u, 0, stream, args);
        if (rc != SP_OK) return rc;
    }
    if (plan.blocks > 0) {
        const BwdKernel k = kBwd[d->dtype == SP_BF16 ? 1 : 0][d->norm == SP_LAYERNORM ? 1 : 0][dR ? 1 : 0]
                                [regen ? 1 : 0][plan.col_blocks > 0 ? 1 : 0][plan.variant];
        void* args[] = {&a};
        rc = launch((const void*)k, (unsigned)(plan.col_blocks + plan.blocks), (unsigned)plan.block,
                    plan.lds_bytes, stream, args);
        if (rc != SP_OK) return rc;
    }
    if (plan.col_blocks > 0) return SP_OK;  // the column workgroups wrote dgamma / dbeta
    const int ncols = plan.nacc * (int)H;
    const unsigned fin_grid = (unsigned)((ncols / 4 + kFinGroups - 1) / kFinGroups);
    const float* fin_ws = a.ws;
    int64_t fin_g = plan.blocks;
    int32_t fin_h = (int32_t)H, fin_nacc = (int32_t)plan.nacc;
    void* args[] = {&fin_ws, &fin_g, &fin_h, &fin_nacc, &dgamma, &dbeta};
    return launch((const void*)sp_dgamma_finish_kernel, fin_grid, (unsigned)(kFinGroups * kFinSlices), 0, stream,
                  args);
}

// ---------------------------------------------------------------------------
// Scratch of the backward entry point that allocates nothing: a device array
// of SP_NOALLOC_SCRATCH_BYTES, one copy per GPU, alive until the process ends.
// Host code never uses its name as an address: the address of each device's
// copy is looked up once, with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[SP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag looked_up;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
    std::atomic<bool> counts_cleared{false};
};
ScratchSlot g_scratch[kMaxDevices];

int scratch_of_current_device(ScratchSlot** slot) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return record_hip(e);
    if (dev < 0 || dev >= kMaxDevices) {
        snprintf(g_hip_error, sizeof(g_hip_error), "device %d is past the %d devices the scratch serves", dev,
                 kMaxDevices);
        return SP_EHIP;
    }
    ScratchSlot& s = g_scratch[dev];
    std::call_once(s.looked_up, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    if (s.err != hipSuccess) return record_hip(s.err);
    *slot = &s;
    return SP_OK;
}

}  // namespace

extern "C" int sp_region_bwd(const sp_desc_t* d, const void* dY, const void* h, const uint8_t* mask,
                             const float* mean, const float* rstd, const float* gamma, const void* dR,
                             void* d_residual, void* dP, float* dgamma, float* dbeta, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return bwd_enqueue(d, dY, h, mask, mean, rstd, gamma, dR, d_residual, dP, dgamma, dbeta, workspace,
                       workspace_bytes, stream, false);
}

extern "C" int sp_region_bwd_noalloc(const sp_desc_t* d, const void* dY, const void* h, const uint8_t* mask,
                                     const float* mean, const float* rstd, const float* gamma, const void* dR,
                                     void* d_residual, void* dP, float* dgamma, float* dbeta, void* stream) {
    const int rc = check_desc(d);
    if (rc != SP_OK) return rc;
    if (plan_bwd(d).ws_bytes > (size_t)SP_NOALLOC_SCRATCH_BYTES) return SP_ESCRATCH;
    ScratchSlot* s = nullptr;
    const int rs = scratch_of_current_device(&s);
    if (rs != SP_OK) return rs;
    // the arrival counts start at zero: cleared by this device's first call
    // (they wrap back to zero at the end of every call after that)
    const bool first = !s->counts_cleared.load();
    const int rb = bwd_enqueue(d, dY, h, mask, mean, rstd, gamma, dR, d_residual, dP, dgamma, dbeta, s->ptr,
                               (size_t)SP_NOALLOC_SCRATCH_BYTES, stream, first);
    if (rb == SP_OK && first) s->counts_cleared.store(true);
    return rb;
}
