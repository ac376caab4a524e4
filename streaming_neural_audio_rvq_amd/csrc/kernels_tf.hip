// kernels_tf.hip -- the windowed causal transformer in front of the conv
// decoder (Fish-DAC-shaped workload): LayerNorm, rotary positions, attention
// of every new frame over its stream's last W frames (the earlier ones from
// the stream's K/V ring, the newer ones from this step), and the ring append.
// The dense projections (in/QKV/O/MLP/out) run on the implicit-GEMM kernel
// with k = 1, with bias, GELU and residual fused into its epilogue.  The
// rotary angles of the step's frames are tabulated once per step; q and k are
// rotated where they are read (attention) or stored (ring append, which rides
// on the launch of the layer's second LayerNorm).  The attention stages each
// block of frames' key window in LDS once.
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

// One work-group per (query block, head), hd == 64: the block's frames are
// up to SNRVQ_ATTN_QB consecutive frames of one stream (the host lists each
// block's frames, positions and slot), and frame f at absolute position p attends
// to keys j in [max(0, p - (W-1)), p], ascending.  The block first stages in
// LDS its frames' q rows (rotated) and the K (rotated) and V rows of every key
// they need -- keys before the stream's first frame of this step from the
// ring, the rest from this step's qkv, rotated here -- so the frames of a
// block share them.  Then wave w takes frames w, w + 4, ... of the block.
// Scores: lanes kk and kk + 32 own key kk and take its dot product with q over
// half the dimensions each (pairs 16u .. 16u + 15 of the rotate-half pairs
// (i, i + 32), u = lane / 32), adding the halves with one cross-lane add;
// softmax over the lanes; output: lane e owns dimension e and sums the value
// rows in key order with the probabilities broadcast from their lanes.
constexpr int ATT_KROWS = SNRVQ_ATTN_QB + SNRVQ_MAX_WINDOW - 1;  // keys a block can need
constexpr int ATT_KP = 68;  // LDS row pitch, floats: 16-byte reads of 16 rows on distinct banks

// Rotated f4 q4 (dims 4 q4 .. 4 q4 + 3) of a 64-wide q or K row r of frame
// row rf of the rotary table: dims below 32 pair with the f4 8 further on.
__device__ __forceinline__ f4 rope_f4(const float *r, const float *rf, int q4)
{
    const bool lo4 = q4 < 8;
    const f4 own = *(const f4 *)(r + 4 * q4);
    const f4 other = *(const f4 *)(r + 4 * (lo4 ? q4 + 8 : q4 - 8));
    f4 out;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const int i = 4 * (lo4 ? q4 : q4 - 8) + e;
        float x, y;
        if (lo4)
            rope_pair(own[e], other[e], rf[2 * i], rf[2 * i + 1], x, y);
        else
            rope_pair(other[e], own[e], rf[2 * i], rf[2 * i + 1], x, y);
        out[e] = lo4 ? x : y;
    }
    return out;
}

template <typename T>
__global__ __launch_bounds__(256) void window_attention_kernel(AttnArgs a)
{
    __shared__ __attribute__((aligned(16))) float ks[ATT_KROWS * ATT_KP];
    __shared__ __attribute__((aligned(16))) float vs[ATT_KROWS * ATT_KP];
    __shared__ __attribute__((aligned(16))) float qs[SNRVQ_ATTN_QB * ATT_KP];
    const int qb = blockIdx.x, h = blockIdx.y;
    const int32_t *e = a.attn_q + (long)qb * SNRVQ_ATTN_Q_INTS;
    const int f0 = e[0], nq = e[1];
    if (nq <= 0)  // graph launches size the grid for the most blocks a step can have
        return;
    const long pf0 = e[2];  // position of frame f0
    const long p0 = e[3];   // position of the stream's first frame of this step
    const int slot = e[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, hd = a.hd, dm = H * hd, W1 = a.W - 1;
    const int f1 = f0 + nq;
    const long jlo = pf0 - W1 > 0 ? pf0 - W1 : 0;  // first key staged
    const int nkeys = (int)(pf0 + nq - 1 - jlo + 1);
    const long ring_base = ((long)slot * a.n_layers + a.layer) * W1 * dm + h * hd;

    // stage the key rows jlo .. jlo + nkeys - 1 and the q rows f0 .. f1 - 1 of
    // head h, 16 f4 per row: item c < (nkeys + nq) 16 of thread c mod 256,
    // all of a thread's loads issued before its first LDS store
    constexpr int ITEMS = (ATT_KROWS + SNRVQ_ATTN_QB) * 16 / 256;
    static_assert((ATT_KROWS + SNRVQ_ATTN_QB) * 16 <= ITEMS * 256 + 255, "items");
    f4 kv[ITEMS + 1], vv[ITEMS + 1];
#pragma unroll
    for (int it = 0; it <= ITEMS; it++) {
        const int c = tid + it * 256;
        const int r = c >> 4, q4 = c & 15;
        if (c >= (nkeys + nq) * 16)
            continue;
        if (r >= nkeys) {  // q row of frame f0 + r - nkeys
            const long f = f0 + (r - nkeys);
            kv[it] = rope_f4(a.qkv + f * 3 * dm + h * hd, a.rot + f * hd, q4);
            continue;
        }
        const long j = jlo + r;
        if (j < p0) {  // in the ring (row j mod (W-1)), K already rotated
            const long o = ring_base + (j % W1) * dm + 4 * q4;
            kv[it] = *(const f4 *)(a.kring + o);
            vv[it] = *(const f4 *)(a.vring + o);
        } else {  // this step's frame, K rotated as in the ring append
            const long fk = f0 + (j - pf0);
            const float *kr = a.qkv + fk * 3 * dm + dm + h * hd;
            kv[it] = rope_f4(kr, a.rot + fk * hd, q4);
            vv[it] = *(const f4 *)(kr + dm + 4 * q4);
        }
    }
#pragma unroll
    for (int it = 0; it <= ITEMS; it++) {
        const int c = tid + it * 256;
        const int r = c >> 4, q4 = c & 15;
        if (c >= (nkeys + nq) * 16)
            continue;
        if (r >= nkeys) {
            *(f4 *)(qs + (r - nkeys) * ATT_KP + 4 * q4) = kv[it];
        } else {
            *(f4 *)(ks + r * ATT_KP + 4 * q4) = kv[it];
            *(f4 *)(vs + r * ATT_KP + 4 * q4) = vv[it];
        }
    }
    __syncthreads();

    const float scale = 1.0f / sqrtf((float)hd);
    const int u = lane >> 5;
    for (int f = f0 + wave; f < f1; f += 4) {
        const long p = pf0 + (f - f0);
        const long jf = p - W1 > 0 ? p - W1 : 0;
        const int nk = (int)(p - jf + 1);
        const int r0 = (int)(jf - jlo);  // LDS row of this frame's key 0
        const int kk = (lane & 31) < nk ? (lane & 31) : nk - 1;
        const float *kp = ks + (r0 + kk) * ATT_KP + 16 * u;
        const float *qp = qs + (f - f0) * ATT_KP + 16 * u;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {  // pairs 16u + 4i .. 16u + 4i + 3
            const f4 ql = *(const f4 *)(qp + 4 * i), qh = *(const f4 *)(qp + 32 + 4 * i);
            const f4 kl = *(const f4 *)(kp + 4 * i), kh = *(const f4 *)(kp + 32 + 4 * i);
            float lo2 = 0.f, hi2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                lo2 += ql[e] * kl[e];
                hi2 += qh[e] * kh[e];
            }
            dot += lo2 + hi2;
        }
        dot += __shfl_xor(dot, 32, 64);
        const float s = lane < nk ? dot * scale : -INFINITY;  // lanes >= 32: none
        float mx = s;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        const float pk = lane < nk ? expf(s - mx) : 0.f;
        const float den = wave_sum(pk);

        // output: lane e, value rows in key order (keys past nk read key
        // nk - 1 and add nothing)
        float acc = 0.f;
#pragma unroll
        for (int k2 = 0; k2 < SNRVQ_MAX_WINDOW; k2++) {
            const int kc = k2 < nk ? k2 : nk - 1;
            const float pr = __shfl(pk, kc, 64);
            const float vv = vs[(r0 + kc) * ATT_KP + lane];
            acc += k2 < nk ? pr * vv : 0.f;
        }
        st<T>((T *)a.att + (long)f * dm + h * hd + lane, acc / den);
    }
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
    const float *kr = a.qkv + (long)f * 3 * dm + dm;
    const float *rf = a.rot + (long)f * a.hd;
    f4 *kd = (f4 *)(a.kring + ring_base + (long)sl * dm);
    f4 *vd = (f4 *)(a.vring + ring_base + (long)sl * dm);
    for (int c = threadIdx.x; c < dm / 4; c += 256) {
        const int hh = c / 16, q4 = c % 16;  // head, f4 within its 64 dims
        kd[c] = rope_f4(kr + hh * 64, rf, q4);
        vd[c] = *(const f4 *)(kr + dm + 4 * c);
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
    if (a.F <= 0 || a.n_qblocks <= 0)
        return hipSuccess;
    if (a.hd != 64 || a.W < 1 || a.W > SNRVQ_MAX_WINDOW)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)a.n_qblocks, (unsigned)a.H);
    if (a.dtype)
        hipLaunchKernelGGL(window_attention_kernel<half_t>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(window_attention_kernel<float>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace snrvq
