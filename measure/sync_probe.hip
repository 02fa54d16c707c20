// sync_probe.hip -- what it costs workgroups of one launch to wait for each other on MI355X
// (measurement tool, not the library).
//
//   empty_kernel      : back-to-back launches of a kernel that does nothing (launch floor);
//   atomic_roundtrip  : one lane, dependent device-scope atomic adds on one word;
//   group_barrier     : 256 workgroups in groups of Cb; in each of `steps` steps every
//                       workgroup publishes 8 floats (device-scope stores), drains them,
//                       counts itself in, one lane waits (bounded) for the group's count, and
//                       the group's floats are read back -- the exchange a kernel needs when a
//                       token row is split over several workgroups;
//   last_arriver      : G workgroups store W floats each, count in, and the last one to
//                       arrive reads all G*W (device-scope loads, 16 in flight per lane) --
//                       a reduction finished inside the launch instead of by a second one.
// Every wait is bounded (a count that never arrives is reported, not waited for), and the
// grids fit the device at once.  Prints one JSON object per measurement.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#define CHECK(x)                                                                           \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                       \
        }                                                                                  \
    } while (0)

constexpr int kSpin = 1 << 14;  // polls before a wait gives up

__global__ void empty_kernel(int* x) {
    if (x && threadIdx.x == 9999) x[0] = 1;
}

// each add's address depends on the previous add's result (mask is 0 at run time)
__global__ void atomic_chain(uint32_t* c, int n, uint32_t mask, uint32_t* out) {
    if (threadIdx.x != 0) return;
    uint32_t v = 0;
    for (int i = 0; i < n; ++i) v = atomicAdd(c + (v & mask), 1u);
    out[0] = v;
}

__global__ __launch_bounds__(256) void group_barrier(float* data, uint32_t* counters, int Cb, int steps,
                                                     uint32_t call, uint32_t* timeouts, float* sink) {
    __shared__ float red[64];
    const int g = blockIdx.x;
    const int cb = g % Cb, grp = g / Cb;
    float acc = 0.0f;
    for (int s = 0; s < steps; ++s) {
        float* blk = data + ((int64_t)(grp * steps + s) * Cb) * 8;
        if (threadIdx.x < 8)
            __hip_atomic_store(blk + cb * 8 + threadIdx.x, (float)(g + s), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        uint32_t* cnt = counters + grp * 64;
        if (threadIdx.x == 0) {
            __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t target = (call * (uint32_t)steps + (uint32_t)s + 1u) * (uint32_t)Cb;
            int it = 0;
            for (; it < kSpin; ++it) {
                const uint32_t v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((int32_t)(v - target) >= 0) break;
                __builtin_amdgcn_s_sleep(1);
            }
            if (it == kSpin) atomicAdd(timeouts, 1u);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            float v = 0.0f;
            if (threadIdx.x < 8 * Cb)
                v = __hip_atomic_load(blk + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            red[threadIdx.x] = v;
        }
        __syncthreads();
        float t = 0.0f;
        for (int q = 0; q < 64; ++q) t += red[q];
        acc += t;
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[g] = acc;
}

__global__ __launch_bounds__(256) void last_arriver(float* part, uint32_t* count, float* out, int W, int G,
                                                    int chain) {
    __shared__ uint32_t last;
    const int g = blockIdx.x;
    for (int c = threadIdx.x; c < W; c += 256)
        __hip_atomic_store(part + (int64_t)g * W + c, (float)(g + c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!chain) return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) last = atomicInc(count, (uint32_t)(G - 1)) == (uint32_t)(G - 1);
    __syncthreads();
    if (!last) return;
    constexpr int NB = 16;
    for (int c = threadIdx.x; c < W; c += 256) {
        float s = 0.0f;
        for (int q0 = 0; q0 < G; q0 += NB) {
            float v[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                v[b] = q0 + b < G ? __hip_atomic_load(part + (int64_t)(q0 + b) * W + c, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                  : 0.0f;
#pragma unroll
            for (int b = 0; b < NB; ++b) s += v[b];
        }
        out[c] = s;
    }
}

template <class F>
double us_per_launch(F launch, int reps) {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int w = 0; w < 3; ++w) launch();
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int k = 0; k < reps; ++k) launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipGetLastError());
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    return ms * 1e3 / reps;
}

int main() {
    for (int g : {1, 256}) {
        const double us = us_per_launch([&] { empty_kernel<<<g, 256>>>(nullptr); }, 200);
        printf("{\"probe\": \"empty_kernel\", \"grid\": %d, \"us\": %.3f}\n", g, us);
    }
    uint32_t *cnt, *out, *tmo;
    CHECK(hipMalloc(&cnt, 1 << 20));
    CHECK(hipMalloc(&out, 4096));
    CHECK(hipMalloc(&tmo, 4096));
    CHECK(hipMemset(cnt, 0, 1 << 20));
    CHECK(hipMemset(tmo, 0, 4096));
    {
        const int n = 2000;
        const double t1 = us_per_launch([&] { atomic_chain<<<1, 64>>>(cnt, 1, 0u, out); }, 50);
        const double tn = us_per_launch([&] { atomic_chain<<<1, 64>>>(cnt, n, 0u, out); }, 5);
        printf("{\"probe\": \"atomic_roundtrip\", \"ns\": %.1f}\n", (tn - t1) * 1e3 / (n - 1));
    }
    float *data, *sink;
    CHECK(hipMalloc(&data, (size_t)16 << 20));
    CHECK(hipMalloc(&sink, 1 << 20));
    const int G = 256;
    for (int steps : {1, 4}) {
        for (int Cb : {2, 4, 8, 16}) {
            CHECK(hipMemset(cnt, 0, 1 << 20));
            uint32_t call = 0;
            const double us = us_per_launch(
                [&] { group_barrier<<<G, 256>>>(data, cnt, Cb, steps, call++, tmo, sink); }, 50);
            uint32_t t = 0;
            CHECK(hipMemcpy(&t, tmo, 4, hipMemcpyDeviceToHost));
            printf("{\"probe\": \"group_barrier\", \"workgroups\": %d, \"group\": %d, \"steps\": %d, \"us\": %.3f, "
                   "\"waits_given_up\": %u}\n",
                   G, Cb, steps, us, t);
            fflush(stdout);
        }
    }
    float* part;
    CHECK(hipMalloc(&part, (size_t)256 * 8192 * 4));
    CHECK(hipMemset(cnt, 0, 1 << 20));
    for (int G2 : {64, 256}) {
        for (int W : {768, 8192}) {
            const double t0 = us_per_launch([&] { last_arriver<<<G2, 256>>>(part, cnt, sink, W, G2, 0); }, 50);
            const double t1 = us_per_launch([&] { last_arriver<<<G2, 256>>>(part, cnt, sink, W, G2, 1); }, 50);
            printf("{\"probe\": \"last_arriver\", \"workgroups\": %d, \"floats_each\": %d, \"store_only_us\": %.3f, "
                   "\"with_last_arriver_read_us\": %.3f}\n",
                   G2, W, t0, t1);
            fflush(stdout);
        }
    }
    CHECK(hipFree(part));
    CHECK(hipFree(data));
    CHECK(hipFree(sink));
    CHECK(hipFree(cnt));
    CHECK(hipFree(out));
    CHECK(hipFree(tmo));
    return 0;
}
