// Practical HBM ceilings of the box, as context for the rooflines of the
// HBM-bound kernels: streams with 16-byte accesses over 2 GiB (well past the
// 256 MB last-level cache).
//   read      grid-stride, every thread reads and folds its pieces
//   read nt   each workgroup reads one contiguous chunk with non-temporal
//             loads, U pieces per lane in flight (the decode kernel's kind
//             of access: contiguous, non-temporal); the fastest read found
//   write     grid-stride, every thread writes its pieces
//   read1:2   reads 512 MiB, writes 1 GiB (the embedding gather's mix:
//             one int8 byte in, one float16 out)
//   size      "read nt" at the sizes of single decode launches (90, 346 and
//             997 MB), back to back over rotating windows of the buffer,
//             and at 346 MB with 8 pieces per lane in flight (the decode
//             kernel's 8 KB per wave)
// A measurement tool, not part of the library (the library build does not
// compile it). Build and run it by hand:
//   mkdir -p workloads/_build && hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       workloads/stream_ceiling.hip -o workloads/_build/stream_ceiling
// then run workloads/_build/stream_ceiling on one MI355X.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                               \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

__global__ __launch_bounds__(256) void stream_read(const u32x4 *__restrict__ p, size_t n, unsigned *__restrict__ out) {
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    unsigned acc = 0;
    for (size_t i = tid; i < n; i += stride) {
        const u32x4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[tid] = acc;
}

// workgroup b reads elements [b * per, (b + 1) * per), per = n / gridDim
// rounded down to whole steps of U * 256 (so no access leaves the chunk)
template <int U>
__global__ __launch_bounds__(256) void stream_read_nt(const u32x4 *__restrict__ p, size_t n, unsigned *__restrict__ out) {
    const size_t per = n / gridDim.x / (U * 256) * (U * 256);
    const u32x4 *q = p + (size_t)blockIdx.x * per;
    unsigned acc = 0;
    for (size_t i = threadIdx.x; i < per; i += U * 256) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(q + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void stream_write(u32x4 *__restrict__ p, size_t n) {
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = tid; i < n; i += stride) p[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
}

// src[0, n) in, dst[0, 2n) out
__global__ __launch_bounds__(256) void stream_read1_write2(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                           size_t n) {
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = tid; i < n; i += stride) {
        const u32x4 v = src[i];
        dst[2 * i] = v;
        dst[2 * i + 1] = v + 1u;
    }
}

template <typename F>
static double time_ms(F launch, int reps) {
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    for (int w = 0; w < 3; ++w) launch();
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(a));
    for (int r = 0; r < reps; ++r) launch();
    CHECK(hipEventRecord(b));
    CHECK(hipEventSynchronize(b));
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, a, b));
    CHECK(hipEventDestroy(a));
    CHECK(hipEventDestroy(b));
    return ms / reps;
}

int main() {
    const size_t bytes = (size_t)2 << 30;
    const size_t n = bytes / 16;
    const int reps = 20;
    const int max_blocks = 4096;
    u32x4 *d;
    unsigned *out;
    CHECK(hipMalloc(&d, bytes));
    CHECK(hipMemset(d, 1, bytes));
    CHECK(hipMalloc(&out, (size_t)max_blocks * 256 * sizeof(unsigned)));
    for (int blocks : {768, 1024, 1536}) {
        const size_t per2 = n / blocks / 512 * 512, per4 = n / blocks / 1024 * 1024;
        const double r2 = time_ms([&] { stream_read_nt<2><<<blocks, 256>>>(d, n, out); }, reps);
        const double r4 = time_ms([&] { stream_read_nt<4><<<blocks, 256>>>(d, n, out); }, reps);
        printf("blocks %5d  read nt, contiguous chunks: %6.0f GB/s (2 in flight)  %6.0f GB/s (4 in flight)\n", blocks,
               per2 * blocks * 16.0 / (r2 * 1e-3) / 1e9, per4 * blocks * 16.0 / (r4 * 1e-3) / 1e9);
    }
    // Reads the size of one decode launch (the LM head alone, the 0.6B and
    // the 1.7B steps), back to back, each launch reading the next window of
    // the buffer so that no launch finds its bytes in the last-level cache.
    for (size_t mb : {90, 346, 997}) {
        const size_t wn = mb * 1000000 / 16, windows = n / wn;
        int r = 0;
        const int blocks = 768;
        const size_t per = wn / blocks / 512 * 512;
        const double ms = time_ms(
            [&] {
                stream_read_nt<2><<<blocks, 256>>>(d + (size_t)(r++ % windows) * wn, wn, out);
            },
            reps * 4);
        printf("size %4zu MB  read nt, contiguous chunks, 768 blocks: %6.0f GB/s (%.1f us per launch)\n", mb,
               per * blocks * 16.0 / (ms * 1e-3) / 1e9, ms * 1e3);
    }
    // the decode kernel's depth: 8 pieces (8 KB per wave) in flight, then
    // all of them used, at the 0.6B step's size
    {
        const size_t wn = (size_t)346 * 1000000 / 16, windows = n / wn;
        int r = 0;
        const int blocks = 768;
        const size_t per = wn / blocks / 2048 * 2048;
        const double ms = time_ms(
            [&] {
                stream_read_nt<8><<<blocks, 256>>>(d + (size_t)(r++ % windows) * wn, wn, out);
            },
            reps * 4);
        printf("size  346 MB  read nt, 8 in flight, 768 blocks:         %6.0f GB/s (%.1f us per launch)\n",
               per * blocks * 16.0 / (ms * 1e-3) / 1e9, ms * 1e3);
    }
    for (int blocks : {1024, 2048, 4096}) {
        const double r = time_ms([&] { stream_read<<<blocks, 256>>>(d, n, out); }, reps);
        const double w = time_ms([&] { stream_write<<<blocks, 256>>>(d, n); }, reps);
        // 512 MiB source, 1 GiB destination, disjoint parts of the buffer
        const double rw = time_ms([&] { stream_read1_write2<<<blocks, 256>>>(d, d + n / 4, n / 4); }, reps);
        printf("blocks %5d  read %6.0f GB/s  write %6.0f GB/s  read1:write2 %6.0f GB/s\n", blocks,
               bytes / (r * 1e-3) / 1e9, bytes / (w * 1e-3) / 1e9, (bytes / 4 * 3) / (rw * 1e-3) / 1e9);
    }
    CHECK(hipFree(d));
    CHECK(hipFree(out));
    return 0;
}
