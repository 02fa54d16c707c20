// stream_probe.hip -- streaming-bandwidth reference for MI355X (measurement tool).
//
// Times, with hipEvents over rotating disjoint buffers, kernels that move bytes
// with no arithmetic:
//   copy    : one 16-byte nontemporal load and store per lane, grid-stride loop,
//             at several sizes and grid sizes (the achievable-bandwidth ceiling);
//   fwd_pat : the forward's access pattern: T partial streams (T = 8 or 2) +
//             residual read, two 16-byte streams and one 8-byte stream written;
//   bwd_pat : the backward's pattern: two 16-byte streams and one 8-byte stream
//             read, two 16-byte streams written.
// Prints one JSON object per measurement.  Usage: stream_probe [max_buffer_GiB]
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define CHECK(x)                                                                        \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                    \
        }                                                                               \
    } while (0)

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b,
                                                   int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

// n chunks per stream; p holds T consecutive streams, r one more
template <int T>
__global__ __launch_bounds__(512) void fwd_pattern_kernel(const u32x4* __restrict__ p, const u32x4* __restrict__ r,
                                                          u32x4* __restrict__ h, u32x4* __restrict__ y,
                                                          u32x2* __restrict__ m, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    u32x4 acc = __builtin_nontemporal_load(r + i);
#pragma unroll
    for (int t = 0; t < T; ++t) acc ^= __builtin_nontemporal_load(p + t * n + i);
    __builtin_nontemporal_store(acc, h + i);
    __builtin_nontemporal_store(acc + 1u, y + i);
    const u32x2 mm = {acc.x, acc.y};
    __builtin_nontemporal_store(mm, m + i);
}

__global__ __launch_bounds__(512) void bwd_pattern_kernel(const u32x4* __restrict__ dy, const u32x4* __restrict__ hh,
                                                          const u32x2* __restrict__ m, u32x4* __restrict__ o1,
                                                          u32x4* __restrict__ o2, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    u32x4 a = __builtin_nontemporal_load(dy + i);
    u32x4 b = __builtin_nontemporal_load(hh + i);
    const u32x2 mm = __builtin_nontemporal_load(m + i);
    a.x ^= mm.x;
    b.y ^= mm.y;
    __builtin_nontemporal_store(a ^ b, o1 + i);
    __builtin_nontemporal_store(a + b, o2 + i);
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
        for (int k = 0; k < reps; ++k) launch(k);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        return ms * 1e3 / reps;
    }
};

int main(int argc, char** argv) {
    const int64_t cap = (int64_t)(argc > 1 ? atoi(argv[1]) : 4) << 30;  // bytes per buffer
    char *A, *B;
    CHECK(hipMalloc(&A, cap));
    CHECK(hipMalloc(&B, cap));
    CHECK(hipMemset(A, 1, cap));
    CHECK(hipMemset(B, 0, cap));
    Timer tm;
    const int reps = 40;

    const int64_t sizes[] = {(int64_t)24 << 20, (int64_t)64 << 20, (int64_t)256 << 20, (int64_t)1 << 30};
    const int grids[] = {1024, 2048, 4096, 16384};
    for (int64_t bytes : sizes) {
        const int64_t n = bytes / 16;
        int nrot = (int)(cap / bytes);
        if (nrot > 16) nrot = 16;
        for (int g : grids) {
            const double us = tm.us_per_launch(
                [&](int k) {
                    const int64_t off = (int64_t)(k % nrot) * bytes;
                    copy_kernel<<<g, 256>>>((const u32x4*)(A + off), (u32x4*)(B + off), n);
                },
                reps);
            printf("{\"probe\": \"copy\", \"bytes_each_way\": %lld, \"grid\": %d, \"us\": %.3f, \"GBs\": %.1f}\n",
                   (long long)bytes, g, us, 2.0 * bytes / us / 1e3);
        }
    }
    // stream sizes of the MiniMind T=2 shard (3 MiB bf16 per stream), the LayerNorm
    // T=8 H=4096 shard (4 MiB) and the large-hidden T=8 H=8192 B=2 shard (32 MiB)
    struct Case {
        int T;
        int64_t sb;
    };
    const Case cases[] = {{2, (int64_t)3 << 20}, {8, (int64_t)4 << 20}, {8, (int64_t)32 << 20}};
    for (const Case& c : cases) {
        const int64_t sb = c.sb;
        const int64_t n = sb / 16;
        const int g = (int)((n + 511) / 512);
        {
            const int64_t rin = (c.T + 1) * sb, rout = 3 * sb;
            int nrot = (int)(cap / rin);
            if (nrot > 16) nrot = 16;
            const double us = tm.us_per_launch(
                [&](int k) {
                    char* a = A + (int64_t)(k % nrot) * rin;
                    char* b = B + (int64_t)(k % nrot) * rout;
                    if (c.T == 2)
                        fwd_pattern_kernel<2><<<g, 512>>>((const u32x4*)a, (const u32x4*)(a + 2 * sb), (u32x4*)b,
                                                          (u32x4*)(b + sb), (u32x2*)(b + 2 * sb), n);
                    else
                        fwd_pattern_kernel<8><<<g, 512>>>((const u32x4*)a, (const u32x4*)(a + 8 * sb), (u32x4*)b,
                                                          (u32x4*)(b + sb), (u32x2*)(b + 2 * sb), n);
                },
                reps);
            const double moved = (c.T + 1.0) * sb + 2.5 * sb;
            printf("{\"probe\": \"fwd_pattern\", \"T\": %d, \"stream_bytes\": %lld, \"us\": %.3f, \"GBs\": %.1f}\n",
                   c.T, (long long)sb, us, moved / us / 1e3);
        }
        if (c.T == 8 || sb == ((int64_t)3 << 20)) {
            const int64_t rin = 5 * sb / 2, rout = 2 * sb;
            int nrot = (int)(cap / rin);
            if (nrot > 16) nrot = 16;
            const double us = tm.us_per_launch(
                [&](int k) {
                    char* a = A + (int64_t)(k % nrot) * rin;
                    char* b = B + (int64_t)(k % nrot) * rout;
                    bwd_pattern_kernel<<<g, 512>>>((const u32x4*)a, (const u32x4*)(a + sb), (const u32x2*)(a + 2 * sb),
                                                   (u32x4*)b, (u32x4*)(b + sb), n);
                },
                reps);
            const double moved = 2.5 * sb + 2.0 * sb;
            printf("{\"probe\": \"bwd_pattern\", \"stream_bytes\": %lld, \"us\": %.3f, \"GBs\": %.1f}\n",
                   (long long)sb, us, moved / us / 1e3);
        }
    }
    CHECK(hipFree(A));
    CHECK(hipFree(B));
    return 0;
}
