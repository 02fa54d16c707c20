// stream_probe.hip -- streaming-bandwidth ceilings on MI355X (measurement tool, not the library).
//
// Times, with hipEvents over rotating disjoint buffers (cold HBM every launch), kernels
// that move bytes and do no arithmetic:
//   copy : one 16-byte nontemporal load and store per lane, grid-stride loop, at several
//          sizes and grid sizes;
//   fwd  : the SP forward's access pattern -- T partial streams and the residual read, two
//          16-byte streams and one 8-byte stream written;
//   bwd  : the SP backward's pattern -- two 16-byte streams and one 8-byte stream read, two
//          16-byte streams written.
// The fwd / bwd patterns are swept over the launch shape: chunks per lane (a workgroup of
// BLOCK lanes takes BLOCK*CPL consecutive 16-byte chunks, lane i the chunks i, i+BLOCK, ...),
// workgroup size, and the cache policy of the loads and stores (nontemporal or not), at the
// stream sizes of the LayerNorm T=8 H=4096 shard (4 MiB per stream), the MiniMind T=2
// shard (3 MiB) and the large-hidden T=8 H=8192 B=2 shard (32 MiB).
// Prints one JSON object per measurement.  Usage: stream_probe [max_buffer_GiB]
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define CHECK(x)                                                                           \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                       \
        }                                                                                  \
    } while (0)

template <bool NT, class V>
__device__ __forceinline__ V ld(const V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, class V>
__device__ __forceinline__ void st(V* p, V v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

// n chunks per stream; p holds T consecutive streams, r one more.  Every load is issued
// before any store.
template <int T, int CPL, int BLOCK, bool NTL, bool NTS>
__global__ __launch_bounds__(BLOCK) void fwd_pattern(const u32x4* __restrict__ p, const u32x4* __restrict__ r,
                                                     u32x4* __restrict__ h, u32x4* __restrict__ y,
                                                     u32x2* __restrict__ m, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * BLOCK * CPL + threadIdx.x;
    u32x4 acc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        int64_t i = base + (int64_t)k * BLOCK;
        if (i >= n) i = n - 1;
        acc[k] = ld<NTL>(r + i);
#pragma unroll
        for (int t = 0; t < T; ++t) acc[k] ^= ld<NTL>(p + t * n + i);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int64_t i = base + (int64_t)k * BLOCK;
        if (i < n) {
            st<NTS>(h + i, acc[k]);
            st<NTS>(y + i, acc[k] + 1u);
            const u32x2 mm = {acc[k].x, acc[k].y};
            st<false>(m + i, mm);
        }
    }
}

template <int CPL, int BLOCK, bool NTL, bool NTS>
__global__ __launch_bounds__(BLOCK) void bwd_pattern(const u32x4* __restrict__ dy, const u32x4* __restrict__ hh,
                                                     const u32x2* __restrict__ m, u32x4* __restrict__ o1,
                                                     u32x4* __restrict__ o2, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * BLOCK * CPL + threadIdx.x;
    u32x4 a[CPL], b[CPL];
    u32x2 mm[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        int64_t i = base + (int64_t)k * BLOCK;
        if (i >= n) i = n - 1;
        a[k] = ld<NTL>(dy + i);
        b[k] = ld<NTL>(hh + i);
        mm[k] = ld<NTL>(m + i);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int64_t i = base + (int64_t)k * BLOCK;
        a[k].x ^= mm[k].x;
        b[k].y ^= mm[k].y;
        if (i < n) {
            st<NTS>(o1 + i, a[k] ^ b[k]);
            st<NTS>(o2 + i, a[k] + b[k]);
        }
    }
}

struct Timer {
    hipEvent_t e0, e1;
    Timer() {
        CHECK(hipEventCreate(&e0));
        CHECK(hipEventCreate(&e1));
    }
    template <class F>
    double us_per_launch(F launch, int reps) {
        for (int w = 0; w < 3; ++w) launch(w);
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0));
        for (int k = 0; k < reps; ++k) launch(k + 3);  // the warm-up sets are not reused
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipGetLastError());
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        return ms * 1e3 / reps;
    }
};

static char *A, *B;
static int64_t CAP;
static Timer* TM;
constexpr int kReps = 60;

static int rotations(int64_t bytes) {
    int64_t r = CAP / bytes;
    // one set per launch where the buffers allow (3 warm-up + kReps timed): more than the
    // 256 MB Infinity Cache is cycled between two uses of a set
    return (int)(r > kReps + 3 ? kReps + 3 : r);
}

template <int T, int CPL, int BLOCK, bool NTL, bool NTS>
void fwd_case(int64_t sb) {
    const int64_t n = sb / 16, per = BLOCK * CPL;
    const int grid = (int)((n + per - 1) / per);
    const int64_t rin = (T + 1) * sb, rout = 3 * sb;
    const int nrot = rotations(rin > rout ? rin : rout);
    const double us = TM->us_per_launch(
        [&](int k) {
            char* a = A + (int64_t)(k % nrot) * rin;
            char* b = B + (int64_t)(k % nrot) * rout;
            fwd_pattern<T, CPL, BLOCK, NTL, NTS><<<grid, BLOCK>>>((const u32x4*)a, (const u32x4*)(a + T * sb),
                                                                  (u32x4*)b, (u32x4*)(b + sb),
                                                                  (u32x2*)(b + 2 * sb), n);
        },
        kReps);
    const double moved = (T + 1.0) * sb + 2.5 * sb;
    printf("{\"probe\": \"fwd_pattern\", \"T\": %d, \"stream_bytes\": %lld, \"chunks_per_lane\": %d, \"block\": %d, "
           "\"grid\": %d, \"nt_loads\": %d, \"nt_stores\": %d, \"us\": %.3f, \"GBs\": %.1f}\n",
           T, (long long)sb, CPL, BLOCK, grid, (int)NTL, (int)NTS, us, moved / us / 1e3);
    fflush(stdout);
}

template <int CPL, int BLOCK, bool NTL, bool NTS>
void bwd_case(int64_t sb) {
    const int64_t n = sb / 16, per = BLOCK * CPL;
    const int grid = (int)((n + per - 1) / per);
    const int64_t rin = 5 * sb / 2, rout = 2 * sb;
    const int nrot = rotations(rin);
    const double us = TM->us_per_launch(
        [&](int k) {
            char* a = A + (int64_t)(k % nrot) * rin;
            char* b = B + (int64_t)(k % nrot) * rout;
            bwd_pattern<CPL, BLOCK, NTL, NTS><<<grid, BLOCK>>>((const u32x4*)a, (const u32x4*)(a + sb),
                                                               (const u32x2*)(a + 2 * sb), (u32x4*)b,
                                                               (u32x4*)(b + sb), n);
        },
        kReps);
    printf("{\"probe\": \"bwd_pattern\", \"stream_bytes\": %lld, \"chunks_per_lane\": %d, \"block\": %d, \"grid\": %d, "
           "\"nt_loads\": %d, \"nt_stores\": %d, \"us\": %.3f, \"GBs\": %.1f}\n",
           (long long)sb, CPL, BLOCK, grid, (int)NTL, (int)NTS, us, 4.5 * sb / us / 1e3);
    fflush(stdout);
}

template <int T>
void fwd_sweep(int64_t sb) {
    fwd_case<T, 1, 128, true, true>(sb);
    fwd_case<T, 1, 256, true, true>(sb);
    fwd_case<T, 1, 512, true, true>(sb);
    fwd_case<T, 1, 1024, true, true>(sb);
    fwd_case<T, 2, 256, true, true>(sb);
    fwd_case<T, 2, 512, true, true>(sb);
    fwd_case<T, 4, 256, true, true>(sb);
    fwd_case<T, 1, 512, false, true>(sb);
    fwd_case<T, 1, 512, true, false>(sb);
    fwd_case<T, 1, 512, false, false>(sb);
    fwd_case<T, 2, 512, false, true>(sb);
}

void bwd_sweep(int64_t sb) {
    bwd_case<1, 128, true, true>(sb);
    bwd_case<1, 256, true, true>(sb);
    bwd_case<1, 512, true, true>(sb);
    bwd_case<1, 1024, true, true>(sb);
    bwd_case<2, 256, true, true>(sb);
    bwd_case<2, 512, true, true>(sb);
    bwd_case<4, 256, true, true>(sb);
    bwd_case<4, 128, true, true>(sb);
    bwd_case<1, 512, false, true>(sb);
    bwd_case<1, 512, true, false>(sb);
    bwd_case<1, 512, false, false>(sb);
    bwd_case<1, 256, false, true>(sb);
    bwd_case<4, 256, false, true>(sb);
    bwd_case<2, 512, false, true>(sb);
}

int main(int argc, char** argv) {
    CAP = (int64_t)(argc > 1 ? atoi(argv[1]) : 1) << 30;  // bytes per buffer
    CHECK(hipMalloc(&A, CAP));
    CHECK(hipMalloc(&B, CAP));
    CHECK(hipMemset(A, 1, CAP));
    CHECK(hipMemset(B, 0, CAP));
    TM = new Timer();

    const int64_t sizes[] = {(int64_t)24 << 20, (int64_t)64 << 20, (int64_t)256 << 20};
    const int grids[] = {1024, 4096, 16384};
    for (int64_t bytes : sizes) {
        if (bytes > CAP) continue;
        const int64_t n = bytes / 16;
        const int nrot = rotations(bytes);
        for (int g : grids) {
            const double us = TM->us_per_launch(
                [&](int k) {
                    const int64_t off = (int64_t)(k % nrot) * bytes;
                    copy_kernel<<<g, 256>>>((const u32x4*)(A + off), (u32x4*)(B + off), n);
                },
                kReps);
            printf("{\"probe\": \"copy\", \"bytes_each_way\": %lld, \"grid\": %d, \"us\": %.3f, \"GBs\": %.1f}\n",
                   (long long)bytes, g, us, 2.0 * bytes / us / 1e3);
            fflush(stdout);
        }
    }
    const int64_t S4 = (int64_t)4 << 20, S3 = (int64_t)3 << 20, S32 = (int64_t)32 << 20;
    fwd_sweep<8>(S4);
    fwd_sweep<2>(S3);
    bwd_sweep(S4);
    bwd_sweep(S3);
    if (9 * S32 <= CAP) {
        fwd_case<8, 1, 512, true, true>(S32);
        fwd_case<8, 2, 512, true, true>(S32);
        fwd_case<8, 1, 256, true, true>(S32);
        bwd_case<1, 512, true, true>(S32);
        bwd_case<2, 512, true, true>(S32);
        bwd_case<4, 256, true, true>(S32);
        bwd_case<1, 512, false, true>(S32);
    }
    CHECK(hipFree(A));
    CHECK(hipFree(B));
    return 0;
}
