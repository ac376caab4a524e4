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
// Rows of at most 1024 values with D % 256 == 0 are read once, 16 bytes per
// lane per load, and kept in registers for the three passes.
template <typename T>
__global__ __launch_bounds__(256) void layer_norm_kernel(const float *x, const float *g,
                                                         const float *b, int F, int D, T *y)
{
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= F)
        return;
    const float *xr = x + row * D;
    if (D % 256 == 0 && D <= 1024) {
        const int nv = D / 256;
        f4 v[4];
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (i < nv) {
                v[i] = *(const f4 *)(xr + i * 256 + lane * 4);
                s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
            }
        const float mean = wave_sum(s) / D;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (i < nv)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float d = v[i][e] - mean;
                    q += d * d;
                }
        const float inv = rsqrtf(wave_sum(q) / D + 1e-5f);
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (i < nv) {
                const int c = i * 256 + lane * 4;
                const f4 gg = *(const f4 *)(g + c), bb = *(const f4 *)(b + c);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    st<T>(y + row * D + c + e, (v[i][e] - mean) * inv * gg[e] + bb[e]);
            }
        return;
    }
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

// One wave per (frame, head), hd == 64.  Keys j in [max(0, p - (W-1)), p],
// ascending: those before the stream's first frame of this step come from
// the ring, the rest from this step's qkv.  Scores: lane kk owns key kk and
// takes its dot product with q over the 64 dimensions itself (all keys' loads
// in flight at once, no per-key cross-lane reduction); softmax over the
// lanes; output: lane e owns dimension e and sums the value rows in key
// order with the probabilities broadcast from their lanes.
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
    const long ring_base = ((long)a.slot[b] * a.n_layers + a.layer) * W1 * dm + h * hd;
    const float scale = 1.0f / sqrtf((float)hd);
    // key kk: ring slot (jlo + kk) mod (W-1) while j < p0, else this step's row
    const int nring = (int)(p0 - jlo > 0 ? p0 - jlo : 0);  // keys held in the ring
    const int slot0 = W1 > 0 ? (int)(jlo % W1) : 0;
    const long row0 = (long)a.cu[b] * 3 * dm + h * hd;  // this step's first frame (q part)
    const long step0 = jlo + nring - p0;                 // step row of key nring
    // element offset of key kk's K row (V row: + dm) in kring / qkv
    auto key_row = [&](int kk, bool &in_ring) -> long {
        in_ring = kk < nring;
        if (in_ring) {
            int sl = slot0 + kk;
            sl = sl >= W1 ? sl - W1 : sl;
            return ring_base + (long)sl * dm;
        }
        return row0 + (step0 + kk - nring) * 3 * dm + dm;
    };

    // scores: lane kk < nk
    const int kk = lane < nk ? lane : nk - 1;
    bool k_in_ring;
    const long krow = key_row(kk, k_in_ring);
    const f4 *kp = (const f4 *)((k_in_ring ? a.kring : a.qkv) + krow);
    const f4 *qp = (const f4 *)(a.qkv + (long)f * 3 * dm + h * hd);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const f4 kv = kp[i], qv = qp[i];
        dot += qv[0] * kv[0] + qv[1] * kv[1] + qv[2] * kv[2] + qv[3] * kv[3];
    }
    const float s = lane < nk ? dot * scale : -INFINITY;
    float mx = s;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float pk = lane < nk ? expf(s - mx) : 0.f;
    const float den = wave_sum(pk);

    // output: lane e, value rows in key order (all W loads issued at once:
    // keys past nk read key nk - 1 and add nothing)
    float acc = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < SNRVQ_MAX_WINDOW; k2++) {
        const int kc = k2 < nk ? k2 : nk - 1;
        const float pr = __shfl(pk, kc, 64);
        bool v_in_ring;
        const long vrow = key_row(kc, v_in_ring);
        const float *vp = v_in_ring ? a.vring + vrow : a.qkv + vrow + dm;
        const float vv = vp[lane];
        acc += k2 < nk ? pr * vv : 0.f;
    }
    st<T>((T *)a.att + (long)f * dm + h * hd + lane, acc / den);
}

// Ring append: the last min(n_b, W-1) frames of each stream's chunk; block
// (b, t) copies the K and V rows of kept frame t of stream b, 16 bytes per
// thread per load (dm % 4 == 0).
__global__ __launch_bounds__(256) void kv_append_kernel(AttnArgs a)
{
    const int b = blockIdx.x, t = blockIdx.y;
    const int dm = a.H * a.hd, W1 = a.W - 1;
    const int n = a.cu[b + 1] - a.cu[b];
    const int keep = n < W1 ? n : W1;
    if (t >= keep)
        return;
    const long ring_base = ((long)a.slot[b] * a.n_layers + a.layer) * W1 * dm;
    const int sl = (int)(((long)a.pos[b] + (n - keep) + t) % W1);  // ring slot of the frame
    const long f = a.cu[b] + (n - keep) + t;
    const f4 *ks = (const f4 *)(a.qkv + f * 3 * dm + dm), *vs = ks + dm / 4;
    f4 *kd = (f4 *)(a.kring + ring_base + (long)sl * dm);
    f4 *vd = (f4 *)(a.vring + ring_base + (long)sl * dm);
    for (int c = threadIdx.x; c < dm / 4; c += 256) {
        kd[c] = ks[c];
        vd[c] = vs[c];
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
    if (B <= 0 || a.W <= 1)  // a window of one frame keeps no ring
        return hipSuccess;
    hipLaunchKernelGGL(kv_append_kernel, dim3(B, a.W - 1), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace snrvq
