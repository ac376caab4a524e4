// kernels_tf.hip -- the windowed causal transformer in front of the conv
// decoder (Fish-DAC-shaped workload): LayerNorm, rotary positions, attention
// of every new frame over its stream's last W frames (the earlier ones from
// the stream's K/V ring, the newer ones from this step), and the ring append.
// The dense projections (in/QKV/O/MLP/out) run on the implicit-GEMM kernel
// with k = 1, with bias, GELU and residual fused into its epilogue.  The
// rotary angles of the step's frames are tabulated once per step; q and k are
// rotated where they are read (attention) or stored (ring append, which rides
// on the launch of the layer's second LayerNorm).
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
__device__ __forceinline__ void layer_norm_block(int blk, const float *x, const float *g,
                                                 const float *b, int F, int D, T *y)
{
    const int lane = threadIdx.x & 63;
    const long row = (long)blk * 4 + (threadIdx.x >> 6);
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

// Rotary table of the step's frames: rot[f][i] = (cos, sin) of the angle
// p inv_freq[i] (p: the frame's absolute position in its stream), evaluated
// in fp64 and reduced before sin / cos.  One thread per (frame, i): the
// angles do not depend on the head.
__global__ __launch_bounds__(256) void rope_table_kernel(float *rot, const double *inv_freq,
                                                         const int32_t *frame_stream,
                                                         const int32_t *cu, const int32_t *pos,
                                                         int F, int half)
{
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= (long)F * half)
        return;
    const int i = (int)(g % half), f = (int)(g / half);
    const int b = frame_stream[f];
    const long p = (long)pos[b] + (f - cu[b]);
    double sn, cs;
    sincos((double)p * inv_freq[i], &sn, &cs);
    rot[2 * g] = (float)cs;
    rot[2 * g + 1] = (float)sn;
}

// Rotate-half pair (i, i + hd/2) of one q or k row: every rotation of the
// library (query, key in the attention, key into the ring) goes through this
// one expression, so a key has the same bits wherever it is rotated.
__device__ __forceinline__ void rope_pair(float a, float b, float c, float s, float &x, float &y)
{
#pragma clang fp contract(off)
    x = a * c - b * s;
    y = b * c + a * s;
}

// One wave per (frame, head), hd == 64.  Keys j in [max(0, p - (W-1)), p],
// ascending: those before the stream's first frame of this step come from
// the ring, the rest from this step's qkv.  Scores: lanes kk and kk + 32 own
// key kk and take its dot product with q over half the dimensions each (all
// keys' loads in flight at once, one cross-lane add per key); softmax over
// the lanes; output: lane e owns dimension e and sums the value rows in key
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

    // scores: key kk = lane mod 32 (W <= 32).  Lanes kk and kk + 32 split the
    // head's 32 rotate-half pairs (i, i + 32) between them, pairs 16u .. 16u + 15
    // for u = lane / 32, and add their two partial sums.  The query and this
    // step's keys are rotated here with their frames' table rows (the ring's
    // keys already are).
    const int u = lane >> 5;
    const int kk = (lane & 31) < nk ? (lane & 31) : nk - 1;
    bool k_in_ring;
    const long krow = key_row(kk, k_in_ring);
    const float *kp = (k_in_ring ? a.kring : a.qkv) + krow + 16 * u;
    const float *qp = a.qkv + (long)f * 3 * dm + h * hd + 16 * u;
    const float *rq = a.rot + (long)f * hd + 32 * u;  // (cos, sin) of pairs 16u ..
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {  // pairs 16u + 4i .. 16u + 4i + 3
        const f4 ql = *(const f4 *)(qp + 4 * i), qh = *(const f4 *)(qp + 32 + 4 * i);
        f4 kl = *(const f4 *)(kp + 4 * i), kh = *(const f4 *)(kp + 32 + 4 * i);
        const f4 r0 = *(const f4 *)(rq + 8 * i), r1 = *(const f4 *)(rq + 8 * i + 4);
        const float cq[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        if (!k_in_ring) {
            const float *rk = a.rot + ((long)a.cu[b] + (step0 + kk - nring)) * hd + 32 * u;
            const f4 t0 = *(const f4 *)(rk + 8 * i), t1 = *(const f4 *)(rk + 8 * i + 4);
            const float ck[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                float x, y;
                rope_pair(kl[e], kh[e], ck[2 * e], ck[2 * e + 1], x, y);
                kl[e] = x;
                kh[e] = y;
            }
        }
        float lo = 0.f, hi = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            float qx, qy;
            rope_pair(ql[e], qh[e], cq[2 * e], cq[2 * e + 1], qx, qy);
            lo += qx * kl[e];
            hi += qy * kh[e];
        }
        dot += lo + hi;
    }
    dot += __shfl_xor(dot, 32, 64);
    const float s = lane < nk ? dot * scale : -INFINITY;  // lanes >= 32: none
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

// Ring append of frame f: kept if it is among its stream's last min(n_b, W-1)
// frames of the step; its K row (rotated as in the attention) and V row go to
// ring row p(f) mod (W-1) of its slot and layer, 16 bytes per thread per load
// (dm % 4 == 0).
__device__ __forceinline__ void kv_append_frame(const AttnArgs &a, int f)
{
    const int dm = a.H * a.hd, W1 = a.W - 1;
    const int b = a.frame_stream[f];
    const int n = a.cu[b + 1] - a.cu[b];
    const int keep = n < W1 ? n : W1;
    const int t = f - a.cu[b];
    if (t < n - keep)
        return;
    const long ring_base = ((long)a.slot[b] * a.n_layers + a.layer) * W1 * dm;
    const int sl = (int)(((long)a.pos[b] + t) % W1);
    const f4 *ks = (const f4 *)(a.qkv + (long)f * 3 * dm + dm), *vs = ks + dm / 4;
    f4 *kd = (f4 *)(a.kring + ring_base + (long)sl * dm);
    f4 *vd = (f4 *)(a.vring + ring_base + (long)sl * dm);
    const int half = a.hd / 2;
    const float *rf = a.rot + (long)f * a.hd;
    for (int c = threadIdx.x; c < dm / 4; c += 256) {
        // dims d .. d + 3 of a head, paired with d + half .. (or d - half ..)
        const int d = (c * 4) % a.hd;
        const bool lo = d < half;
        const f4 own = ks[c], other = ks[lo ? c + half / 4 : c - half / 4];
        f4 out;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int i = (lo ? d : d - half) + e;
            float x, y;
            if (lo)
                rope_pair(own[e], other[e], rf[2 * i], rf[2 * i + 1], x, y);
            else
                rope_pair(other[e], own[e], rf[2 * i], rf[2 * i + 1], x, y);
            out[e] = lo ? x : y;
        }
        kd[c] = out;
        vd[c] = vs[c];
    }
}

// Four rows per work-group; with a ring, F more work-groups append frame
// blockIdx.x - ceil(F / 4) each.
template <typename T, bool APPEND>
__global__ __launch_bounds__(256) void layer_norm_kernel(const float *x, const float *g,
                                                         const float *b, int F, int D, T *y,
                                                         AttnArgs ring)
{
    const int nln = (F + 3) / 4;
    if (!APPEND || (int)blockIdx.x < nln)
        layer_norm_block<T>(blockIdx.x, x, g, b, F, D, y);
    else
        kv_append_frame(ring, blockIdx.x - nln);
}

}  // namespace

hipError_t launch_layer_norm(const float *x, const float *g, const float *b, int F, int D,
                             void *y, int dtype, hipStream_t st, const AttnArgs *ring)
{
    if (F <= 0)
        return hipSuccess;
    const bool app = ring && ring->W > 1;  // a window of one frame keeps no ring
    const AttnArgs r = app ? *ring : AttnArgs{};
    dim3 grid((F + 3) / 4 + (app ? F : 0));
    if (dtype) {
        if (app)
            hipLaunchKernelGGL((layer_norm_kernel<half_t, true>), grid, dim3(256), 0, st, x, g, b,
                               F, D, (half_t *)y, r);
        else
            hipLaunchKernelGGL((layer_norm_kernel<half_t, false>), grid, dim3(256), 0, st, x, g,
                               b, F, D, (half_t *)y, r);
    } else {
        if (app)
            hipLaunchKernelGGL((layer_norm_kernel<float, true>), grid, dim3(256), 0, st, x, g, b,
                               F, D, (float *)y, r);
        else
            hipLaunchKernelGGL((layer_norm_kernel<float, false>), grid, dim3(256), 0, st, x, g, b,
                               F, D, (float *)y, r);
    }
    return hipGetLastError();
}

hipError_t launch_rope_table(float *rot, const double *inv_freq, const int32_t *frame_stream,
                             const int32_t *cu, const int32_t *pos, int F, int hd,
                             hipStream_t st)
{
    const long total = (long)F * (hd / 2);
    if (total <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                       rot, inv_freq, frame_stream, cu, pos, F, hd / 2);
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

}  // namespace snrvq
