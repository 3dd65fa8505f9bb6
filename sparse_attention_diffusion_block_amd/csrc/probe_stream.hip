// HBM streaming probe for gfx950: the rate at which plain kernels move data with and without the
// non-temporal cache policy.  A standalone measurement program (not part of librettn.so); it backs
// the streaming floor the sparse step is judged against.
//
// Three access patterns, each as a grid-stride loop of 16-byte accesses per lane (x1 or unrolled
// x4), with the default policy and with the nt bit on every load and store:
//   * read:  one 4 GiB buffer, read only (an XOR that is never stored, so nothing is written);
//   * copy:  one 136.5 MB buffer copied into another;
//   * mix:   four 136.5 MB buffers read and a fifth written, element by element: the traffic of
//            the sparse step (Q, K, V and R read, O written), sized like one of its tensors
//            at B = 2, H = 30, L = 17776, d = 64 in bfloat16.
// Before every timed launch a 4 GiB fill evicts the 256 MB last-level cache, so each sample reads
// from HBM.  20 samples per row (HIP events around one launch); best and mean.  With --mix-json it
// runs only the non-temporal mix (unrolled x1, 2 work-groups per CU) and prints one JSON line.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <string>

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                               \
    do {                                                                                       \
        hipError_t e_ = (x);                                                                   \
        if (e_ != hipSuccess) {                                                                \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
            exit(1);                                                                           \
        }                                                                                      \
    } while (0)

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4 v, u32x4* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <int U, bool NT>
__global__ void __launch_bounds__(256) read_kernel(const u32x4* __restrict__ a, size_t n, u32x4* __restrict__ sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld<NT>(a + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n; i += stride) acc ^= a[i];
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[threadIdx.x] = acc;   // never true for the fill
}

template <int U, bool NT>
__global__ void __launch_bounds__(256) copy_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ o, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld<NT>(a + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) st<NT>(v[u], o + i + u * stride);
    }
    for (; i < n; i += stride) o[i] = a[i];
}

template <int U, bool NT>
__global__ void __launch_bounds__(256) mix_kernel(const u32x4* __restrict__ a, const u32x4* __restrict__ b,
                                                  const u32x4* __restrict__ c, const u32x4* __restrict__ d,
                                                  u32x4* __restrict__ o, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 va[U], vb[U], vc[U], vd[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t j = i + u * stride;
            va[u] = ld<NT>(a + j);
            vb[u] = ld<NT>(b + j);
            vc[u] = ld<NT>(c + j);
            vd[u] = ld<NT>(d + j);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) st<NT>(va[u] ^ vb[u] ^ vc[u] ^ vd[u], o + i + u * stride);
    }
    for (; i < n; i += stride) o[i] = a[i] ^ b[i] ^ c[i] ^ d[i];
}

int main(int argc, char** argv) {
    const bool mix_json = argc > 1 && std::string(argv[1]) == "--mix-json";
    const size_t bytes = (size_t)2 * 30 * 17776 * 64 * 2;   // one bfloat16 tensor of the video workload
    const size_t n = bytes / 16;
    const size_t big_bytes = (size_t)4 << 30;
    u32x4 *a, *b, *c, *d, *o, *sink, *big;
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&b, bytes));
    CHECK(hipMalloc(&c, bytes));
    CHECK(hipMalloc(&d, bytes));
    CHECK(hipMalloc(&o, bytes));
    CHECK(hipMalloc(&sink, 256 * sizeof(u32x4)));
    CHECK(hipMalloc(&big, big_bytes));
    for (u32x4* p : {a, b, c, d, o}) CHECK(hipMemset(p, 1, bytes));
    CHECK(hipMemset(big, 1, big_bytes));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    int dev = 0, cus = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, dev));
    if (!mix_json) {
        printf("device: %s, %d CUs\n\n", prop.gcnArchName, cus);
        printf("| pattern | policy | unroll | work-groups per CU | bytes moved | best us | best GB/s | mean us | mean GB/s |\n");
        printf("|---|---|---|---|---|---|---|---|---|\n");
    }

    auto row = [&](const char* pattern, bool nt, int unroll, int per_cu, double moved, auto launch) {
        for (int w = 0; w < 3; ++w) launch();
        CHECK(hipDeviceSynchronize());
        float best = 1e30f, total = 0.f;
        const int samples = 20;
        for (int r = 0; r < samples; ++r) {
            CHECK(hipMemset(big, r + 2, big_bytes));   // evicts the last-level cache
            CHECK(hipEventRecord(e0));
            launch();
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms = 0.f;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            best = ms < best ? ms : best;
            total += ms;
        }
        const float mean = total / samples;
        if (mix_json)
            printf("{\"pattern\": \"%s\", \"policy\": \"%s\", \"unroll\": %d, \"workgroups_per_cu\": %d, "
                   "\"bytes\": %.0f, \"best_us\": %.1f, \"mean_us\": %.1f, \"best_gbs\": %.0f, \"samples\": %d}\n",
                   pattern, nt ? "nt" : "default", unroll, per_cu, moved, best * 1e3, mean * 1e3, moved / (best * 1e6),
                   samples);
        else
            printf("| %s | %s | x%d | %d | %.0f | %.1f | %.0f | %.1f | %.0f |\n", pattern, nt ? "nt" : "default", unroll,
                   per_cu, moved, best * 1e3, moved / (best * 1e6), mean * 1e3, moved / (mean * 1e6));
    };
    if (mix_json) {
        const dim3 grid(cus * 2), blk(256);
        row("mix 4R+1W", true, 1, 2, 5.0 * bytes,
            [&] { hipLaunchKernelGGL((mix_kernel<1, true>), grid, blk, 0, 0, a, b, c, d, o, n); });
        CHECK(hipGetLastError());
        return 0;
    }

    for (int per_cu : {2, 4, 8}) {
        const dim3 grid(cus * per_cu), blk(256);
        row("read", false, 4, per_cu, (double)big_bytes,
            [&] { hipLaunchKernelGGL((read_kernel<4, false>), grid, blk, 0, 0, big, big_bytes / 16, sink); });
        row("read", true, 4, per_cu, (double)big_bytes,
            [&] { hipLaunchKernelGGL((read_kernel<4, true>), grid, blk, 0, 0, big, big_bytes / 16, sink); });
        row("copy", false, 4, per_cu, 2.0 * bytes,
            [&] { hipLaunchKernelGGL((copy_kernel<4, false>), grid, blk, 0, 0, a, o, n); });
        row("copy", true, 4, per_cu, 2.0 * bytes,
            [&] { hipLaunchKernelGGL((copy_kernel<4, true>), grid, blk, 0, 0, a, o, n); });
        row("mix 4R+1W", false, 1, per_cu, 5.0 * bytes,
            [&] { hipLaunchKernelGGL((mix_kernel<1, false>), grid, blk, 0, 0, a, b, c, d, o, n); });
        row("mix 4R+1W", false, 4, per_cu, 5.0 * bytes,
            [&] { hipLaunchKernelGGL((mix_kernel<4, false>), grid, blk, 0, 0, a, b, c, d, o, n); });
        row("mix 4R+1W", true, 1, per_cu, 5.0 * bytes,
            [&] { hipLaunchKernelGGL((mix_kernel<1, true>), grid, blk, 0, 0, a, b, c, d, o, n); });
        row("mix 4R+1W", true, 4, per_cu, 5.0 * bytes,
            [&] { hipLaunchKernelGGL((mix_kernel<4, true>), grid, blk, 0, 0, a, b, c, d, o, n); });
        CHECK(hipGetLastError());
    }
    printf("\nprobe done\n");
    return 0;
}
