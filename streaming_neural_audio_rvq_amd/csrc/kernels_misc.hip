// kernels_misc.hip -- the non-GEMM kernels of a decode step:
//   * halo fill / save: move each stream's left context between its state
//     slot and the halo rows of every extended conv input (all layers at
//     once; the fill shares one launch with the gather);
//   * RVQ gather-and-sum of the codebook rows of every frame;
//   * the final causal conv to one channel: on the matrix cores for fp16
//     operands (weights in row 0 of the A operand, 16 samples per MFMA
//     column block), an N = 1 VALU reduction for fp32;
//   * unextend: packed fp32 copy of an extended buffer (inspection only).
#include "internal.h"

namespace snrvq {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// blockIdx.x = batch index b, blockIdx.y = halo layer.
__global__ __launch_bounds__(256) void halo_save_kernel(HaloTable t, char *state,
                                                        const int32_t *cu, const int32_t *slot)
{
    halo_save_one(t, blockIdx.y, blockIdx.x, state, cu, slot, threadIdx.x, 256);
}

// 8 consecutive table values as fp32 (bf16 -> fp32 is exact: the bits move to
// the top half).
__device__ __forceinline__ void load8(const uint16_t *p, float *v)
{
    const u4 w = *(const u4 *)p;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float *v)
{
    const f4 a = *(const f4 *)p, b = *(const f4 *)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[i] = a[i];
        v[4 + i] = b[i];
    }
}
__device__ __forceinline__ void store8(half_t *p, const float *v)
{
    h8 h;
#pragma unroll
    for (int i = 0; i < 8; i++)
        h[i] = snrvq_f16(v[i]);
    *(h8 *)p = h;
}
__device__ __forceinline__ void store8(float *p, const float *v)
{
    *(f4 *)p = f4{v[0], v[1], v[2], v[3]};
    *(f4 *)(p + 4) = f4{v[4], v[5], v[6], v[7]};
}

// One thread owns 8 consecutive values of one frame's output row and sums
// the K selected codebook rows in codebook order, in fp32.  The codebooks are
// one contiguous [K][E][d_cb] array.  Codebooks are taken 16 at a time: all
// 16 codes are loaded, then all 16 rows, before any is added, so a step of up
// to 16 codebooks costs two dependent memory round trips (codes, rows).  The output row is out_ld wide:
// channels [0, d_cb) take the sum; with `one` set channel d_cb is 1 (the
// constant input that carries the projection bias through a folded input
// conv) and the rest zero.  out_H > 0: rows go to the extended buffer (stream
// b's frame f at row (b + 1) out_H + f).
template <typename CB, typename OUT>
__device__ __forceinline__ void rvq_gather_body(int blk, const CB *cb, const int32_t *codes, int F,
                                                int K, int E, int d_cb, int out_ld, int out_H,
                                                bool one, const int32_t *frame_stream, OUT *z,
                                                unsigned long long *bad)
{
    const int per_frame = out_ld / 8;
    const long g = (long)blk * 256 + threadIdx.x;
    const long f = g / per_frame;
    if (f >= F)
        return;
    const int d = (int)(g - f * per_frame) * 8;
    const long row = out_H ? (long)(frame_stream[f] + 1) * out_H + f : f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (d >= d_cb) {  // the constant channel and the zero padding
#pragma unroll
        for (int i = 0; i < 8; i++)
            acc[i] = one && d + i == d_cb ? 1.f : 0.f;
        store8(z + row * out_ld + d, acc);
        return;
    }
    const int32_t *cf = codes + f * K;
    constexpr int KB = 16;
    for (int k0 = 0; k0 < K; k0 += KB) {
        int e[KB];
#pragma unroll
        for (int j = 0; j < KB; j++)
            e[j] = k0 + j < K ? cf[k0 + j] : 0;
#pragma unroll
        for (int j = 0; j < KB; j++)
            if ((unsigned)e[j] >= (unsigned)E) {  // only reachable with device-resident codes
                if (d == 0 && k0 + j < K)
                    atomicAdd(bad, 1ull);
                e[j] = 0;
            }
        float v[KB][8];
#pragma unroll
        for (int j = 0; j < KB; j++)
            if (k0 + j < K)
                load8(cb + ((long)(k0 + j) * E + e[j]) * d_cb + d, v[j]);
#pragma unroll
        for (int j = 0; j < KB; j++)
            if (k0 + j < K)
#pragma unroll
                for (int i = 0; i < 8; i++)
                    acc[i] += v[j][i];
    }
    store8(z + row * out_ld + d, acc);
}

// The step's first launch: the gather in work-groups [0, gblocks), the halo
// fill of every layer and stream in the rest.  The two are independent, so
// one launch runs them side by side.  The fill is flat over (layer, stream,
// 16-byte chunk), each thread copying FILL_PER chunks (zeros for a fresh
// stream).  One chunk per thread: the copies are latency-bound (a stream's
// slot, then its state), so more threads in flight beat more work per thread
// (128-stream steps: 16.4 us per launch against 18.5 us with 4 chunks and
// 26.5 us with 8).
constexpr int FILL_PER = 1;
template <typename CB, typename OUT>
__global__ __launch_bounds__(256) void rvq_gather_fill_kernel(
    const CB *cb, const int32_t *codes, int F, int K, int E, int d_cb, int out_ld, int out_H,
    int one, OUT *z, unsigned long long *bad, int gblocks, HaloTable t, const char *state,
    const int32_t *frame_stream, const int32_t *cu, const int32_t *slot, const int32_t *fresh,
    int B)
{
    const int blk = blockIdx.x;
    if (blk < gblocks) {
        rvq_gather_body(blk, cb, codes, F, K, E, d_cb, out_ld, out_H, one != 0, frame_stream, z,
                        bad);
        return;
    }
    // consecutive threads take consecutive chunks (one 16-byte chunk per
    // thread per pass: every wave access is one contiguous 1 KB run)
#pragma unroll
    for (int q = 0; q < FILL_PER; q++) {
        int i = ((blk - gblocks) * FILL_PER + q) * 256 + (int)threadIdx.x;
        for (int l = 0; l < t.n; l++) {
            const HaloLayer &L = t.l[l];
            const int cpr = L.C * t.elem_bytes / 16;  // chunks per row
            const int per_stream = L.H * cpr;
            if (i >= per_stream * B) {
                i -= per_stream * B;
                continue;
            }
            const int b = i / per_stream;
            const int k = i - b * per_stream;
            char *dst = (char *)L.ext + (((long)b * L.H + (long)cu[b] * L.rate) * cpr + k) * 16;
            const char *src =
                state + ((long)slot[b] * t.slot_elems + L.state_off) * t.elem_bytes + (long)k * 16;
            *(u4 *)dst = fresh[b] ? u4{0u, 0u, 0u, 0u} : *(const u4 *)src;
            break;
        }
    }
}

// fp32 final conv: pcm[m] = b + sum_j sum_c w[j][c] A[row(m) - (6 - j)][c],
// one thread per output sample, fp32 accumulation.  The channels are split in
// four quarters, each summed taps-then-channels ascending, and combined as
// b + ((q0 + q1) + (q2 + q3)).
__global__ __launch_bounds__(256) void final_conv_kernel(const float *A, int A_H, int C, int rate,
                                                         const float *w, float bias, int tanh_out,
                                                         const int32_t *frame_stream, int M,
                                                         float *pcm)
{
    extern __shared__ float wsh[];  // [7][C]
    for (int i = threadIdx.x; i < 7 * C; i += blockDim.x) {
        int c = i / 7, j = i - c * 7;  // input layout [C][7]
        wsh[j * C + c] = w[i];
    }
    __syncthreads();
    long m = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M)
        return;
    int b = frame_stream[m / rate];
    long ext = (long)(b + 1) * A_H + m;
    const int CQ = C / 4;
    float q[4];
    for (int qp = 0; qp < 4; qp++) {
        float part = 0.f;
        for (int j = 0; j < 7; j++) {
            const float *row = A + (ext - (6 - j)) * C + qp * CQ;
            const float *wj = wsh + j * C + qp * CQ;
            for (int c = 0; c < CQ; c += 4) {
                const f4 v = *(const f4 *)(row + c);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    part += wj[c + e] * v[e];
            }
        }
        q[qp] = part;
    }
    const float acc = bias + ((q[0] + q[1]) + (q[2] + q[3]));
    pcm[m] = tanh_out ? tanhf(acc) : acc;
}

// fp16 final conv on v_mfma_f32_16x16x32_f16, C a multiple of 32.  A wave
// takes 16 consecutive packed samples (the B operand's columns); the A
// operand's row 0 holds the weights of one (tap, 32-channel) K step, its other
// rows zeros, so row 0 of the accumulator is the conv output.  K steps run
// tap-major, channel-minor; the fused last stage runs the same sequence.
__global__ __launch_bounds__(256) void final_conv_mfma_kernel(const half_t *A, int A_H, int C,
                                                              int rate, const float *w,
                                                              float bias, int tanh_out,
                                                              const int32_t *frame_stream, int M,
                                                              float *pcm)
{
    extern __shared__ float wsh[];  // fp16 [7][C]
    half_t *w16 = (half_t *)wsh;
    for (int i = threadIdx.x; i < 7 * C; i += blockDim.x) {
        int c = i / 7, j = i - c * 7;  // input layout [C][7]
        w16[j * C + c] = (half_t)w[i];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
    const long m0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16;
    if (m0 >= M)
        return;
    long m = m0 + l16;
    const bool ok = m < M;
    m = ok ? m : M - 1;
    const long ext = (long)(frame_stream[m / rate] + 1) * A_H + m;
    const h8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < 7; j++) {
        const half_t *row = A + (ext - (6 - j)) * C + lg * 8;
        for (int k0 = 0; k0 < C; k0 += 32) {
            const h8 wf = *(const h8 *)(w16 + j * C + k0 + lg * 8);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(l16 == 0 ? wf : zero,
                                                        *(const h8 *)(row + k0), acc, 0, 0, 0);
        }
    }
    if (lg == 0 && ok) {
        const float y = bias + acc[0];
        pcm[m] = tanh_out ? tanhf(y) : y;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void unextend_kernel(const T *ext, int H, int ld, int C,
                                                       int rate, const int32_t *frame_stream,
                                                       int M, float *dst)
{
    long g = (long)blockIdx.x * 256 + threadIdx.x;
    long total = (long)M * C;
    if (g >= total)
        return;
    long m = g / C;
    int c = (int)(g - m * C);
    int b = frame_stream[m / rate];
    dst[g] = (float)ext[((long)(b + 1) * H + m) * ld + c];
}

}  // namespace

hipError_t launch_halo_save(const HaloTable &t, void *state, const StepMeta &m, int B,
                            hipStream_t st)
{
    if (t.n == 0 || B == 0)
        return hipSuccess;
    hipLaunchKernelGGL(halo_save_kernel, dim3(B, t.n), dim3(256), 0, st, t, (char *)state, m.cu,
                       m.slot);
    return hipGetLastError();
}

hipError_t launch_rvq_gather_fill(const void *cb, int cb_dtype, const int32_t *codes, int F,
                                  int K, int E, int d_cb, int out_ld, int out_H, int one, void *z,
                                  int out_dtype, unsigned long long *bad, const HaloTable &t,
                                  void *state, const StepMeta &m, int B, hipStream_t st)
{
    if (F <= 0 || B <= 0)
        return hipSuccess;
    if (out_ld % 8 || d_cb % 8 || out_ld < d_cb + (one ? 1 : 0))
        return hipErrorInvalidValue;
    const long threads = (long)F * (out_ld / 8);
    const int gblocks = (int)((threads + 255) / 256);
    long chunks = 0;
    for (int l = 0; l < t.n; l++) {
        if ((long)t.l[l].C * t.elem_bytes % 16)
            return hipErrorInvalidValue;
        chunks += (long)B * t.l[l].H * t.l[l].C * t.elem_bytes / 16;
    }
    if (chunks >= (1L << 30))  // the fill indexes chunks in 32 bits
        return hipErrorInvalidValue;
    const long fblocks = (chunks + 256L * FILL_PER - 1) / (256L * FILL_PER);
    const dim3 grid((unsigned)(gblocks + fblocks));
    const char *sp = (const char *)state;
#define SNRVQ_GATHER(CBT, OT)                                                                      \
    hipLaunchKernelGGL((rvq_gather_fill_kernel<CBT, OT>), grid, dim3(256), 0, st,                  \
                       (const CBT *)cb, codes, F, K, E, d_cb, out_ld, out_H, one, (OT *)z, bad,    \
                       gblocks, t, sp, m.frame_stream, m.cu, m.slot, m.fresh, B)
    if (cb_dtype == 1 && out_dtype == 1)
        SNRVQ_GATHER(uint16_t, half_t);
    else if (cb_dtype == 0 && out_dtype == 0)
        SNRVQ_GATHER(float, float);
    else if (cb_dtype == 1 && out_dtype == 0)
        SNRVQ_GATHER(uint16_t, float);
    else
        SNRVQ_GATHER(float, half_t);
#undef SNRVQ_GATHER
    return hipGetLastError();
}

hipError_t launch_final_conv(const void *A, int dtype, int A_H, int C, int rate, const float *w,
                             float b, int final_tanh, const int32_t *frame_stream, int M,
                             float *pcm, hipStream_t st)
{
    if (M <= 0)
        return hipSuccess;
    dim3 grid((M + 255) / 256);
    size_t sh = sizeof(float) * 7 * C;
    // fp16 channel widths are multiples of 32 (the codec's configuration
    // check); fp32 ones multiples of 16, so C / 4 is a whole number of f4s
    if (dtype ? C % 32 : C % 16)
        return hipErrorInvalidValue;
    if (dtype)
        hipLaunchKernelGGL(final_conv_mfma_kernel, dim3((M + 63) / 64), dim3(256), sh, st,
                           (const half_t *)A, A_H, C, rate, w, b, final_tanh, frame_stream, M,
                           pcm);
    else
        hipLaunchKernelGGL(final_conv_kernel, grid, dim3(256), sh, st, (const float *)A, A_H, C,
                           rate, w, b, final_tanh, frame_stream, M, pcm);
    return hipGetLastError();
}

hipError_t launch_unextend(const void *ext, int dtype, int H, int ld, int C, int rate,
                           const int32_t *frame_stream, int M, float *dst, hipStream_t st)
{
    long total = (long)M * C;
    if (total <= 0)
        return hipSuccess;
    dim3 grid((unsigned)((total + 255) / 256));
    if (dtype)
        hipLaunchKernelGGL(unextend_kernel<half_t>, grid, dim3(256), 0, st, (const half_t *)ext, H,
                           ld, C, rate, frame_stream, M, dst);
    else
        hipLaunchKernelGGL(unextend_kernel<float>, grid, dim3(256), 0, st, (const float *)ext, H,
                           ld, C, rate, frame_stream, M, dst);
    return hipGetLastError();
}

}  // namespace snrvq
