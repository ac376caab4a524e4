// ceilings.hip -- micro-benchmarks of the rates the decoder's kernels are
// measured against: the matrix cores (independent MFMA chains, no memory
// traffic), LDS reads (conflict-free 16-byte reads), the vector ALU on the
// Snake activation the fused stages evaluate, and MFMA and Snake work issued
// together by the same waves, in separate blocks or interleaved.  The shader
// clock under each load is read from the wave's cycle counter against the
// constant 100 MHz counter.  Timing only: each kernel touches no memory but
// its own small output buffer (one record per wave) and its LDS array, and
// every loop runs a fixed number of iterations.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "snrvq_probes.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Snake as the library evaluates it: x + sin^2(2 pi r) / alpha with r the
// fractional part of x alpha / (2 pi), the hardware sine taking revolutions.
__device__ __forceinline__ float snake(float v, float alpha_rev, float inv_alpha)
{
#pragma clang fp contract(off)
    const float r = __builtin_amdgcn_fractf(alpha_rev * v);
    const float s = __builtin_amdgcn_sinf(r);
    return __builtin_fmaf(s * s, inv_alpha, v);
}

// per-wave record: cycle counter and 100 MHz counter at start and end
struct WaveRec {
    uint64_t t0, t1, r0, r1;
    float sink;
    float pad[7];
};

__device__ __forceinline__ void rec_start(uint64_t &t, uint64_t &r)
{
    r = __builtin_amdgcn_s_memrealtime();
    t = __builtin_amdgcn_s_memtime();
}

__device__ __forceinline__ void rec_end(WaveRec *out, uint64_t t0, uint64_t r0, float sink)
{
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if ((threadIdx.x & 63) == 0) {
        WaveRec *w = out + blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
        w->t0 = t0;
        w->t1 = t1;
        w->r0 = r0;
        w->r1 = r1;
        w->sink = sink;
    }
}

__device__ __forceinline__ h8 lane_h8(float base)
{
    h8 v;
#pragma unroll
    for (int i = 0; i < 8; i++)
        v[i] = (_Float16)(base + 0.001f * i);
    return v;
}

// 16 independent 16x16x32 chains (KIND 0) or 4 independent 32x32x16 chains
// updated twice per iteration (KIND 1) per wave, each accumulator updated in
// place (they start from `seed`, zeros in memory: accumulators that start at
// constants get copied between registers every iteration).
constexpr int MF_CHAINS = 16;
template <int KIND>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, const float *seed, WaveRec *out)
{
    const float l = (threadIdx.x & 63) * 1e-3f;
    const h8 a = lane_h8(0.5f + l), b = lane_h8(0.25f - l);
    uint64_t t0, r0;
    rec_start(t0, r0);
    float sink = 0.f;
    if constexpr (KIND == 0) {
        f4 acc[MF_CHAINS];
#pragma unroll
        for (int j = 0; j < MF_CHAINS; j++)
            acc[j] = *(const f4 *)(seed + 4 * j);
        for (int i = 0; i < iters; i++)
#pragma unroll
            for (int j = 0; j < MF_CHAINS; j++)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < MF_CHAINS; j++)
            sink += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
    } else {
        f16v acc[4];
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[j] = *(const f16v *)(seed + 16 * j);
        for (int i = 0; i < iters; i++)
#pragma unroll
            for (int r = 0; r < 2; r++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                sink += acc[j][e];
    }
    rec_end(out, t0, r0, sink);
}

// Conflict-free LDS reads: in each read the 64 lanes take 64 consecutive
// 16-byte slots; 8 reads per iteration at compile-time offsets from a base
// that moves with the iteration, folded into a running XOR (the empty asm
// with a memory clobber keeps reads of one iteration from being reused in
// the next).
// SLOTS 16-byte slots per work-group: 4096 (64 KiB, up to two work-groups
// per CU) or 1024 (16 KiB, up to eight).
template <int SLOTS>
__global__ __launch_bounds__(256) void lds_kernel(int iters, WaveRec *out)
{
    static_assert(SLOTS >= 1024 && SLOTS % 512 == 0, "slots");
    __shared__ u4 buf[SLOTS];
    for (int i = threadIdx.x; i < SLOTS; i += blockDim.x)
        buf[i] = u4{(uint32_t)i, (uint32_t)i * 3u, (uint32_t)i * 5u, (uint32_t)i * 7u};
    __syncthreads();
    const int lane = threadIdx.x & 63;
    u4 x = u4{0u, 0u, 0u, 0u};
    uint64_t t0, r0;
    rec_start(t0, r0);
    for (int i = 0; i < iters; i++) {
        // slots up to (SLOTS / 512 - 1) 256 + 63 + 7 * 64 = SLOTS / 2 + 255 < SLOTS
        const u4 *p = buf + (i & (SLOTS / 512 - 1)) * 256 + lane;
        u4 r[8];
#pragma unroll
        for (int j = 0; j < 8; j++)
            r[j] = p[j * 64];
        x ^= (r[0] ^ r[1]) ^ (r[2] ^ r[3]) ^ (r[4] ^ r[5]) ^ (r[6] ^ r[7]);
        __asm__ volatile("" ::: "memory");
    }
    rec_end(out, t0, r0, (float)(x[0] ^ x[1] ^ x[2] ^ x[3]));
}

// Global -> LDS direct loads (16 bytes per lane, the conv kernel's staging
// path) from a 256 KiB source that stays in L2: 8 loads of 1 KiB per wave
// per iteration into the wave's own 8 KiB of LDS, then a wait for all of
// them (vmcnt(0)) before the next iteration overwrites it.
constexpr int GL_CHUNKS = 256;  // 1 KiB chunks of the source
#define GLOBAL_PTR(p) ((const void __attribute__((address_space(1))) *)(p))
#define LDS_PTR(p) ((void __attribute__((address_space(3))) *)(p))
__global__ __launch_bounds__(256) void gload_kernel(int iters, const float *src, WaveRec *out)
{
    __shared__ u4 buf[4 * 8 * 64];  // 4 waves x 8 loads x 64 lanes x 16 bytes
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const char *sb = (const char *)src;
    uint64_t t0, r0;
    rec_start(t0, r0);
    for (int i = 0; i < iters; i++) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int c = ((i * 8 + j) * 4 + wave) & (GL_CHUNKS - 1);
            __builtin_amdgcn_global_load_lds(GLOBAL_PTR(sb + c * 1024 + lane * 16),
                                             LDS_PTR(buf + (wave * 8 + j) * 64), 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    }
    __syncthreads();
    const u4 v = buf[threadIdx.x];
    rec_end(out, t0, r0, (float)(v[0] ^ v[3]));
}

// HBM streaming: y = x + 1 over n float4 elements, grid-stride, 16 bytes per
// lane per load and store (read and write traffic equal).
__global__ __launch_bounds__(256) void stream_kernel(const f4 *x, f4 *y, long n)
{
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
        y[i] = x[i] + 1.0f;
}

// MFMA chains and Snake chains in the same waves.  MODE 0: Snakes only;
// 1: MFMAs only; 2: per iteration all MFMAs, then all Snakes (scheduling
// barriers keep the blocks apart); 3: the same work interleaved, one MFMA
// then SPM Snakes (a scheduling-group pattern).
constexpr int OV_MFMA = 16;  // MFMAs per iteration
constexpr int OV_SPM = 2;   // Snakes per MFMA
template <int MODE>
__global__ __launch_bounds__(256) void overlap_kernel(int iters, const float *seed, WaveRec *out)
{
    const float l = (threadIdx.x & 63) * 1e-3f;
    const h8 a = lane_h8(0.5f + l), b = lane_h8(0.25f - l);
    f4 acc[OV_MFMA];
#pragma unroll
    for (int j = 0; j < OV_MFMA; j++)
        acc[j] = *(const f4 *)(seed + 4 * j);
    constexpr int NS = OV_MFMA * OV_SPM;
    float v[NS];
#pragma unroll
    for (int j = 0; j < NS; j++)
        v[j] = 0.1f * j + l;
    const float ar = 0.3183f, ia = 1.7f;
    uint64_t t0, r0;
    rec_start(t0, r0);
    for (int i = 0; i < iters; i++) {
        if constexpr (MODE != 0) {
#pragma unroll
            for (int j = 0; j < OV_MFMA; j++)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
        }
        if constexpr (MODE == 2)
            __builtin_amdgcn_sched_barrier(0);
        if constexpr (MODE != 1) {
#pragma unroll
            for (int j = 0; j < NS; j++)
                v[j] = snake(v[j], ar, ia);
        }
        if constexpr (MODE == 2)
            __builtin_amdgcn_sched_barrier(0);
        if constexpr (MODE == 3) {
            // 0x8: MFMA, 0x2: VALU; a Snake is 5 VALU instructions
#pragma unroll
            for (int j = 0; j < OV_MFMA; j++) {
                __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x2, 5 * OV_SPM, 0);
            }
        }
    }
    float sink = 0.f;
#pragma unroll
    for (int j = 0; j < OV_MFMA; j++)
        sink += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
#pragma unroll
    for (int j = 0; j < NS; j++)
        sink += v[j];
    rec_end(out, t0, r0, sink);
}

int n_cu()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return n;
}

// Launches `launch` once untimed and `reps` times timed; fills the wall time
// of one launch and the mean shader clock of its waves.
template <typename L>
int timed(int blocks, int reps, L launch, probe_result *res)
{
    if (blocks <= 0 || reps <= 0 || !res)
        return 1;
    const size_t waves = (size_t)blocks * 4;
    // zeros the accumulators start from, and the direct-load probe's source
    constexpr size_t SEED = GL_CHUNKS * 1024 / sizeof(float);
    WaveRec *d = nullptr;
    if (hipMalloc((void **)&d, waves * sizeof(WaveRec) + SEED * sizeof(float)) != hipSuccess)
        return 2;
    float *seed = (float *)(d + waves);
    if (hipMemset(seed, 0, SEED * sizeof(float)) != hipSuccess) {
        (void)hipFree(d);
        return 3;
    }
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        (void)hipFree(d);
        return 3;
    }
    launch(d, seed);
    int rc = hipEventRecord(e0, 0) == hipSuccess ? 0 : 3;
    for (int i = 0; i < reps; i++)
        launch(d, seed);
    if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipGetLastError() != hipSuccess)
        rc = 3;
    float ms = 0.f;
    if (!rc && hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
        rc = 3;
    std::vector<WaveRec> h(waves);
    if (!rc && hipMemcpy(h.data(), d, waves * sizeof(WaveRec), hipMemcpyDeviceToHost) != hipSuccess)
        rc = 3;
    double clk = 0.0;
    size_t nclk = 0;
    for (const WaveRec &w : h)
        if (w.r1 > w.r0 && w.t1 > w.t0) {
            clk += (double)(w.t1 - w.t0) / (double)(w.r1 - w.r0) * 0.1;  // GHz
            nclk++;
        }
    res->us = 1000.0 * ms / reps;
    res->clock_ghz = nclk ? clk / nclk : 0.0;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(d);
    return rc;
}

}  // namespace

extern "C" {

int probe_cu_count(void) { return n_cu(); }

int probe_mfma(int kind, int waves_per_simd, int iters, int reps, probe_result *res)
{
    const int blocks = n_cu() * waves_per_simd;
    if (iters <= 0 || waves_per_simd < 1 || waves_per_simd > 8 || (kind != 0 && kind != 1))
        return 1;
    int rc = timed(blocks, reps, [&](WaveRec *d, const float *seed) {
        if (kind == 0)
            hipLaunchKernelGGL(mfma_kernel<0>, dim3(blocks), dim3(256), 0, 0, iters, seed, d);
        else
            hipLaunchKernelGGL(mfma_kernel<1>, dim3(blocks), dim3(256), 0, 0, iters, seed, d);
    }, res);
    // multiply-adds per MFMA: 16 * 16 * 32 = 8192, 32 * 32 * 16 = 16384
    const double mfmas = (double)blocks * 4 * iters * (kind == 0 ? MF_CHAINS : 8);
    if (!rc)
        res->rate = mfmas * 2.0 * (kind == 0 ? 8192.0 : 16384.0) / (res->us * 1e-6) / 1e12;
    return rc;
}

int probe_lds(int waves_per_simd, int iters, int reps, probe_result *res)
{
    const int blocks = n_cu() * waves_per_simd;
    if (iters <= 0 || waves_per_simd < 1 || waves_per_simd > 8)
        return 1;
    int rc = timed(blocks, reps, [&](WaveRec *d, const float *) {
        if (waves_per_simd <= 2)
            hipLaunchKernelGGL(lds_kernel<4096>, dim3(blocks), dim3(256), 0, 0, iters, d);
        else
            hipLaunchKernelGGL(lds_kernel<1024>, dim3(blocks), dim3(256), 0, 0, iters, d);
    }, res);
    const double bytes = (double)blocks * 256 * iters * 8 * 16;
    if (!rc)
        res->rate = bytes / (res->us * 1e-6) / 1e12;  // TB/s over all CUs
    return rc;
}

int probe_gload(int waves_per_simd, int iters, int reps, probe_result *res)
{
    const int blocks = n_cu() * waves_per_simd;
    if (iters <= 0 || waves_per_simd < 1 || waves_per_simd > 4)  // 32 KiB of LDS per block
        return 1;
    int rc = timed(blocks, reps, [&](WaveRec *d, const float *seed) {
        hipLaunchKernelGGL(gload_kernel, dim3(blocks), dim3(256), 0, 0, iters, seed, d);
    }, res);
    const double bytes = (double)blocks * 4 * iters * 8 * 1024;
    if (!rc)
        res->rate = bytes / (res->us * 1e-6) / 1e12;  // TB/s over all CUs
    return rc;
}

int probe_hbm(int mib, int blocks_per_cu, int reps, probe_result *res)
{
    if (mib < 64 || mib > 8192 || blocks_per_cu < 1 || blocks_per_cu > 32 || reps <= 0 || !res)
        return 1;
    const long n = (long)mib * (1L << 20) / 16;  // float4 elements per buffer
    f4 *x = nullptr, *y = nullptr;
    if (hipMalloc((void **)&x, n * 16) != hipSuccess)
        return 2;
    if (hipMalloc((void **)&y, n * 16) != hipSuccess) {
        (void)hipFree(x);
        return 2;
    }
    int rc = hipMemset(x, 0, n * 16) == hipSuccess ? 0 : 3;
    const int blocks = n_cu() * blocks_per_cu;
    hipEvent_t e0, e1;
    if (!rc && (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess))
        rc = 3;
    float ms = 0.f;
    if (!rc) {
        hipLaunchKernelGGL(stream_kernel, dim3(blocks), dim3(256), 0, 0, x, y, n);
        if (hipEventRecord(e0, 0) != hipSuccess)
            rc = 3;
        for (int i = 0; i < reps && !rc; i++)
            hipLaunchKernelGGL(stream_kernel, dim3(blocks), dim3(256), 0, 0, x, y, n);
        if (!rc && (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                    hipGetLastError() != hipSuccess ||
                    hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
            rc = 3;
        (void)hipEventDestroy(e0);
        (void)hipEventDestroy(e1);
    }
    if (!rc) {
        res->us = 1000.0 * ms / reps;
        res->rate = 2.0 * n * 16 / (res->us * 1e-6) / 1e9;  // GB/s, reads + writes
        res->clock_ghz = 0.0;
    }
    (void)hipFree(x);
    (void)hipFree(y);
    return rc;
}

int probe_overlap(int mode, int waves_per_simd, int iters, int reps, probe_result *res)
{
    const int blocks = n_cu() * waves_per_simd;
    if (iters <= 0 || waves_per_simd < 1 || waves_per_simd > 8 || mode < 0 || mode > 3)
        return 1;
    int rc = timed(blocks, reps, [&](WaveRec *d, const float *seed) {
        switch (mode) {
        case 0: hipLaunchKernelGGL(overlap_kernel<0>, dim3(blocks), dim3(256), 0, 0, iters, seed, d); break;
        case 1: hipLaunchKernelGGL(overlap_kernel<1>, dim3(blocks), dim3(256), 0, 0, iters, seed, d); break;
        case 2: hipLaunchKernelGGL(overlap_kernel<2>, dim3(blocks), dim3(256), 0, 0, iters, seed, d); break;
        default: hipLaunchKernelGGL(overlap_kernel<3>, dim3(blocks), dim3(256), 0, 0, iters, seed, d); break;
        }
    }, res);
    // rate: Snakes per second (modes 0, 2, 3) or TFLOP/s (mode 1)
    const double lanes = (double)blocks * 256 * iters;
    if (!rc)
        res->rate = mode == 1 ? lanes / 64 * OV_MFMA * 2.0 * 8192.0 / (res->us * 1e-6) / 1e12
                              : lanes * OV_MFMA * OV_SPM / (res->us * 1e-6);
    return rc;
}

}  // extern "C"
