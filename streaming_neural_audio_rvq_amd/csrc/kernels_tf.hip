// kernels_tf.hip -- the windowed causal transformer in front of the conv
// decoder (Fish-DAC-shaped workload): LayerNorm, rotary positions, attention
// of every new frame over its stream's last W frames (the earlier ones from
// the stream's K/V ring, the newer ones from this step), and the ring append.
// The dense projections (in/QKV/O/MLP/out) run on the implicit-GEMM kernel
// with k = 1, with bias, GELU and residual fused into its epilogue.
//
// K/V ring: per slot and layer, W-1 rows of post-rotary K and of V (fp32),
// the frame at absolute position p living in row p mod (W-1).
#include "internal.h"

namespace snrvq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

template <typename T>
__device__ __forceinline__ void st(T *p, float v);
template <>
__device__ __forceinline__ void st<half_t>(half_t *p, float v) { *p = snrvq_f16(v); }
template <>
__device__ __forceinline__ void st<float>(float *p, float v) { *p = v; }

// One wave per row: y = (x - mean) / sqrt(var + eps) * g + b, D % 64 == 0.
template <typename T>
__global__ __launch_bounds__(256) void layer_norm_kernel(const float *x, const float *g,
                                                         const float *b, int F, int D, T *y)
{
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= F)
        return;
    const float *xr = x + row * D;
    float s = 0.f;
    for (int i = lane; i < D; i += 64)
        s += xr[i];
    const float mean = wave_sum(s) / D;
    float v = 0.f;
    for (int i = lane; i < D; i += 64) {
        float d = xr[i] - mean;
        v += d * d;
    }
    const float inv = rsqrtf(wave_sum(v) / D + 1e-5f);
    for (int i = lane; i < D; i += 64)
        st<T>(y + row * D + i, (xr[i] - mean) * inv * g[i] + b[i]);
}

// Rotary embedding of q and k in place, rotate-half pairs (i, i + hd/2),
// angle = p * inv_freq[i] evaluated in fp64 and reduced before sin / cos.
__global__ __launch_bounds__(256) void rope_kernel(float *qkv, const double *inv_freq,
                                                   const int32_t *frame_stream,
                                                   const int32_t *cu, const int32_t *pos, int F,
                                                   int H, int hd)
{
    const int half = hd / 2;
    const int dm = H * hd;
    long g = (long)blockIdx.x * 256 + threadIdx.x;
    long total = (long)F * H * half;
    if (g >= total)
        return;
    int i = (int)(g % half);
    long fh = g / half;
    int h = (int)(fh % H);
    int f = (int)(fh / H);
    int b = frame_stream[f];
    long p = (long)pos[b] + (f - cu[b]);
    double ang = (double)p * inv_freq[i];
    double sn, cs;
    sincos(ang, &sn, &cs);
    float c = (float)cs, s = (float)sn;
    float *q = qkv + (long)f * 3 * dm + h * hd;
    float *k = q + dm;
    float a = q[i], bq = q[i + half];
    q[i] = a * c - bq * s;
    q[i + half] = bq * c + a * s;
    a = k[i];
    bq = k[i + half];
    k[i] = a * c - bq * s;
    k[i + half] = bq * c + a * s;
}

// One wave per (frame, head); lane e owns dimension e (hd == 64).  Keys
// j in [max(0, p - (W-1)), p], ascending: those before the stream's first
// frame of this step come from the ring, the rest from this step's qkv.
template <typename T>
__global__ __launch_bounds__(256) void window_attention_kernel(AttnArgs a)
{
    const int lane = threadIdx.x & 63;
    const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int H = a.H, hd = a.hd, dm = H * hd, W1 = a.W - 1;
    if (wid >= (long)a.F * H)
        return;
    const int h = (int)(wid % H);
    const int f = (int)(wid / H);
    const int b = a.frame_stream[f];
    const long p0 = a.pos[b];
    const long p = p0 + (f - a.cu[b]);
    const long jlo = p - W1 > 0 ? p - W1 : 0;
    const int nk = (int)(p - jlo + 1);
    const float q = a.qkv[(long)f * 3 * dm + h * hd + lane];
    const long ring_base = ((long)a.slot[b] * a.n_layers + a.layer) * W1 * dm;
    const float scale = 1.0f / sqrtf((float)hd);
    // key kk: ring slot (jlo + kk) mod (W-1) while j < p0, else this step's row
    const int nring = (int)(p0 - jlo > 0 ? p0 - jlo : 0);  // keys held in the ring
    const int slot0 = (int)(jlo % W1);
    const float *kr = a.kring + ring_base + h * hd + lane;
    const float *vr = a.vring + ring_base + h * hd + lane;
    const long row0 = (long)a.cu[b] * 3 * dm + h * hd + lane;  // this step's first frame
    float sc[SNRVQ_MAX_WINDOW];  // fully unrolled: stays in registers
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < SNRVQ_MAX_WINDOW; kk++) {
        if (kk < nk) {
            float kv;
            if (kk < nring) {
                int sl = slot0 + kk;
                sl = sl >= W1 ? sl - W1 : sl;
                kv = kr[(long)sl * dm];
            } else {
                kv = a.qkv[row0 + (long)(kk - nring + (jlo + nring - p0)) * 3 * dm + dm];
            }
            float s = wave_sum(q * kv) * scale;
            sc[kk] = s;
            mx = fmaxf(mx, s);
        }
    }
    float den = 0.f;
#pragma unroll
    for (int kk = 0; kk < SNRVQ_MAX_WINDOW; kk++) {
        if (kk < nk) {
            sc[kk] = expf(sc[kk] - mx);
            den += sc[kk];
        }
    }
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < SNRVQ_MAX_WINDOW; kk++) {
        if (kk < nk) {
            float vv;
            if (kk < nring) {
                int sl = slot0 + kk;
                sl = sl >= W1 ? sl - W1 : sl;
                vv = vr[(long)sl * dm];
            } else {
                vv = a.qkv[row0 + (long)(kk - nring + (jlo + nring - p0)) * 3 * dm + 2 * dm];
            }
            acc += sc[kk] * vv;
        }
    }
    st<T>((T *)a.att + (long)f * dm + h * hd + lane, acc / den);
}

// Ring append: the last min(n_b, W-1) frames of each stream's chunk.
__global__ __launch_bounds__(256) void kv_append_kernel(AttnArgs a)
{
    const int b = blockIdx.x;
    const int dm = a.H * a.hd, W1 = a.W - 1;
    const int n = a.cu[b + 1] - a.cu[b];
    const int keep = n < W1 ? n : W1;
    const long ring_base = ((long)a.slot[b] * a.n_layers + a.layer) * W1 * dm;
    int sl = (int)(((long)a.pos[b] + (n - keep)) % W1);  // ring slot of the first kept frame
    for (int t = n - keep; t < n; t++) {
        const long f = a.cu[b] + t;
        for (int c = threadIdx.x; c < dm; c += 256) {
            a.kring[ring_base + (long)sl * dm + c] = a.qkv[f * 3 * dm + dm + c];
            a.vring[ring_base + (long)sl * dm + c] = a.qkv[f * 3 * dm + 2 * dm + c];
        }
        sl = sl + 1 == W1 ? 0 : sl + 1;
    }
}

}  // namespace

hipError_t launch_layer_norm(const float *x, const float *g, const float *b, int F, int D,
                             void *y, int dtype, hipStream_t st)
{
    if (F <= 0)
        return hipSuccess;
    dim3 grid((F + 3) / 4);
    if (dtype)
        hipLaunchKernelGGL(layer_norm_kernel<half_t>, grid, dim3(256), 0, st, x, g, b, F, D,
                           (half_t *)y);
    else
        hipLaunchKernelGGL(layer_norm_kernel<float>, grid, dim3(256), 0, st, x, g, b, F, D,
                           (float *)y);
    return hipGetLastError();
}

hipError_t launch_rope(float *qkv, const double *inv_freq, const int32_t *frame_stream,
                       const int32_t *cu, const int32_t *pos, int F, int H, int hd,
                       hipStream_t st)
{
    long total = (long)F * H * (hd / 2);
    if (total <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, qkv,
                       inv_freq, frame_stream, cu, pos, F, H, hd);
    return hipGetLastError();
}

hipError_t launch_window_attention(const AttnArgs &a, hipStream_t st)
{
    long waves = (long)a.F * a.H;
    if (waves <= 0)
        return hipSuccess;
    dim3 grid((unsigned)((waves + 3) / 4));
    if (a.dtype)
        hipLaunchKernelGGL(window_attention_kernel<half_t>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(window_attention_kernel<float>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_kv_append(const AttnArgs &a, int B, hipStream_t st)
{
    if (B <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(kv_append_kernel, dim3(B), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace snrvq
