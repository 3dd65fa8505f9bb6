// Issue-cost probe for gfx950: what one SIMD pays for matrix and vector instructions, alone and
// mixed, at 1-3 resident waves per SIMD, and the arithmetic ceiling of the calibration's inner
// loop with no memory traffic.  A standalone measurement program (not part of librettn.so); it
// backs the cost model the attention kernels are designed against.
//
// Every kernel runs independent instruction streams on registers only (no loads or stores inside
// the timed loop).  One launch places one 4-wave work-group per CU per resident wave slot, so
// "w waves per SIMD" is a grid of 256 * w work-groups of 256 threads; the register count of every
// kernel's occupancy is asked of the runtime, and a wave count that does not fit is skipped.
// Time comes from HIP events around 5 back-to-back launches, after one warm-up launch.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                               \
    do {                                                                                       \
        hipError_t e_ = (x);                                                                   \
        if (e_ != hipSuccess) {                                                                \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
            exit(1);                                                                           \
        }                                                                                      \
    } while (0)

constexpr int kCUs = 256;
constexpr int kIters = 1024;

// ---------------------------------------------------------------- mixes: per group, NM MFMAs
// (4 independent chains) and NV independent vector instructions of one kind per MFMA
// KIND 0: v_fma_f32, 1: v_exp_f32
template <int NM, int NV, int KIND>
__global__ void __launch_bounds__(256) mix_kernel(float* out, float x0) {
    f32x16 acc[4] = {};
    bf16x8 m = {};
    for (int i = 0; i < 8; ++i) m[i] = (__bf16)(x0 * 0.5f + i);
    float a[16];
    for (int i = 0; i < 16; ++i) a[i] = x0 + i * 0.001f + threadIdx.x * 1e-6f;
    for (int it = 0; it < kIters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (NM) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(m, m, acc[j], 0, 0, 0);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int i = (j * NV + v) & 15;
                if (KIND == 0) a[i] = fmaf(a[i], 0.999f, 0.001f);
                else a[i] = __builtin_amdgcn_exp2f(a[i]);
            }
        }
        asm volatile("" ::: "memory");
    }
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += a[i];
    for (int j = 0; j < 4; ++j)
        for (int i = 0; i < 16; ++i) s += acc[j][i];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

// ---------------------------------------------------------------- the calibration's tile, registers only:
// S^T = K Q^T (8 bf16 MFMAs in two chains), the softmax of its 32 scores per lane (fma, exp,
// packing to float16, float16 row sum), O^T += V^T P^T (8 fp16 MFMAs).  PIPE = 1 issues the next
// tile's S^T before this tile's softmax.
constexpr int kTileIters = 512;
__device__ __forceinline__ unsigned pack_rtz(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a, b));
}

template <int PIPE>
__global__ void __launch_bounds__(256) tile_kernel(float* out, float x0, float c) {
    bf16x8 kq[4];
    f16x8 vv[4];
    for (int k = 0; k < 4; ++k)
        for (int i = 0; i < 8; ++i) {
            kq[k][i] = (__bf16)(x0 * 0.01f * (i + k) + threadIdx.x * 1e-5f);
            vv[k][i] = (_Float16)(0.01f * i);
        }
    f32x16 o0 = {}, o1 = {}, s0 = {}, s1 = {};
    float m = 0.5f, dsum = 0.f;
    const h2 one = {(_Float16)1.f, (_Float16)1.f};
    auto scores = [&](f32x16& a, f32x16& b) {
        a = f32x16{};
        b = f32x16{};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[k], kq[(k + 1) & 3], a, 0, 0, 0);
            b = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[(k + 2) & 3], kq[(k + 1) & 3], b, 0, 0, 0);
        }
    };
    auto softmax = [&](const f32x16& a, const f32x16& b, u32x4 (&pf)[4]) {
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f32x16& sp = (t >> 1) ? b : a;
                const int o = 8 * (t & 1) + 2 * w;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sp[o], c, -m));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sp[o + 1], c, -m));
                pf[t][w] = pack_rtz(p0, p1);
                sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pf[t][w]), one, sum, false);
            }
        dsum += sum;
    };
    auto pv = [&](const u32x4 (&pf)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv[t], __builtin_bit_cast(f16x8, pf[t]), o0, 0, 0, 0);
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv[(t + 1) & 3], __builtin_bit_cast(f16x8, pf[t]), o1, 0, 0, 0);
        }
    };
    if (PIPE == 0) {
        for (int it = 0; it < kTileIters; ++it) {
            u32x4 pf[4];
            scores(s0, s1);
            softmax(s0, s1, pf);
            pv(pf);
            asm volatile("" ::: "memory");
        }
    } else {
        scores(s0, s1);
        for (int it = 0; it < kTileIters; ++it) {
            u32x4 pf[4];
            f32x16 n0, n1;
            scores(n0, n1);
            softmax(s0, s1, pf);
            pv(pf);
            s0 = n0;
            s1 = n1;
            asm volatile("" ::: "memory");
        }
    }
    float s = dsum;
    for (int i = 0; i < 16; ++i) s += o0[i] + o1[i];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

// ---------------------------------------------------------------- harness
static int regs_of(const void* kernel) {
    hipFuncAttributes at;
    CHECK(hipFuncGetAttributes(&at, kernel));
    return at.numRegs;
}

// resident 256-thread work-groups per CU = resident waves per SIMD (the runtime's own count,
// which includes the accumulation registers that numRegs leaves out)
static int waves_per_simd(const void* kernel) {
    int blocks = 0;
    CHECK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 256, 0));
    return blocks;
}

template <typename Launch>
static float time_ms(Launch launch) {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    launch();
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 5; ++r) launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    return ms / 5.f;
}


template <int NM, int NV, int KIND>
static void mix_row(const char* name, float* out) {
    const void* k = (const void*)mix_kernel<NM, NV, KIND>;
    const int regs = regs_of(k), wmax = waves_per_simd(k);
    printf("| %-22s |", name);
    for (int w = 1; w <= 3; ++w) {
        if (w > wmax) {
            printf(" (does not fit) |");
            continue;
        }
        const float ms = time_ms([&] {
            hipLaunchKernelGGL((mix_kernel<NM, NV, KIND>), dim3(kCUs * w), dim3(256), 0, 0, out, 0.5f);
        });
        const double groups = (double)w * kIters * 4;             // per SIMD
        printf(" %6.2f ns |", ms * 1e6 / groups);
    }
    printf(" %d (%d waves fit) |\n", regs, wmax);
}

template <int PIPE>
static void tile_row(const char* name, float* out) {
    const void* k = (const void*)tile_kernel<PIPE>;
    const int regs = regs_of(k), wmax = waves_per_simd(k);
    printf("| %-22s |", name);
    for (int w = 1; w <= 3; ++w) {
        if (w > wmax) {
            printf(" (does not fit) |");
            continue;
        }
        const float ms = time_ms([&] {
            hipLaunchKernelGGL((tile_kernel<PIPE>), dim3(kCUs * w), dim3(256), 0, 0, out, 0.5f, 0.18f);
        });
        const double flops = (double)kCUs * w * 4 * kTileIters * 16 * 32768.0;
        printf(" %5.1f%% |", flops / (ms * 1e-3) / 2.5e15 * 100.0);
    }
    printf(" %d (%d waves fit) |\n", regs, wmax);
}

int main() {
    int dev = 0;
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, dev));
    if (prop.multiProcessorCount != kCUs)
        printf("note: %d compute units (the grids assume %d)\n", prop.multiProcessorCount, kCUs);
    float* out = nullptr;
    CHECK(hipMalloc(&out, (size_t)kCUs * 3 * 256 * sizeof(float)));
    printf("device: %s, %d CUs\n\n", prop.gcnArchName, prop.multiProcessorCount);
    printf("Cost per SIMD of one group (ns); a group is one MFMA 32x32x16 bf16 and/or the vector\n");
    printf("instructions listed, 4 independent chains of each per wave.\n\n");
    printf("| group | 1 wave/SIMD | 2 waves/SIMD | 3 waves/SIMD | vector registers |\n|---|---|---|---|---|\n");
    mix_row<1, 0, 0>("MFMA", out);
    mix_row<0, 8, 0>("8 v_fma_f32", out);
    mix_row<0, 8, 1>("8 v_exp_f32", out);
    mix_row<1, 8, 0>("MFMA + 8 v_fma_f32", out);
    mix_row<1, 8, 1>("MFMA + 8 v_exp_f32", out);
    mix_row<1, 4, 1>("MFMA + 4 v_exp_f32", out);
    printf("\nThe calibration's tile with no memory traffic, %% of the 2.5 PFLOP/s bf16 MFMA peak:\n\n");
    printf("| tile | 1 wave/SIMD | 2 waves/SIMD | 3 waves/SIMD | vector registers |\n|---|---|---|---|---|\n");
    tile_row<0>("S, softmax, P*V", out);
    tile_row<1>("next S before softmax", out);
    CHECK(hipFree(out));
    printf("\nprobe done\n");
    return 0;
}
