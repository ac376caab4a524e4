// kernels_stage.hip -- one kernel per late upsample stage of the conv
// decoder: ConvTranspose1d -> residual unit (dilation 1) -> residual unit
// (dilation 3) [-> final conv to PCM, for the last stage], over time tiles
// of one stream.  Snake activations only (ELU decoders take the per-layer
// path).
//
// The per-layer path moves every intermediate through HBM (at the last stage
// of the Qwen-shaped decoder about 1.1 KB per output row).  Here a tile of T
// output rows recomputes the left halo its residual units need (6 rows for
// the dilation-1 conv, 18 for the dilation-3 conv, 6 more when the final
// conv is fused) and keeps the fp32 residual stream x, the activated conv
// inputs and the residual-unit intermediate in LDS.  HBM sees the stage's
// fp16 input rows and its fp16 output rows (or the PCM) only.
//
// Arithmetic is the per-layer path's, operation for operation: the same
// fp16 operands (each activation applied once, then rounded), the same K
// order (tap-major, channel-minor in steps of 32) on v_mfma_f32_16x16x32_f16,
// the same fp32 epilogues, so both paths give bit-identical PCM.
//
// Orientation: weights are the MFMA's A operand (16 output channels per
// block) and activations the B operand (16 time rows per block), so each
// lane's accumulator holds 4 consecutive channels of one time row.  Every
// epilogue then works on 4 channels at once: one 16-byte read and write of
// the fp32 residual, one 8-byte fp16 store, one address per 4 values.
//
// Left context: at a stream's first tile the rows before the chunk come
// from the halo rows that the step's halo fill wrote into the (otherwise
// unused) extended buffers of the per-layer path; the stream's last tile
// writes the new left contexts straight into its state slot.
//
// Work split (NW waves): ConvT work items of 16 input rows x up to 8 column
// blocks; residual-unit row blocks of 16 output rows, RB blocks per wave in
// flight so each weight fragment feeds RB MFMAs.  The dilated conv reads its
// 7 taps as row shifts of the LDS tile.  Per-channel parameters (biases,
// Snake alpha/2pi and 1/alpha) sit in LDS.  With WL the stage's weights also
// sit in LDS and one persistent work-group per CU walks the tiles.
#include "internal.h"

namespace snrvq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ f4 mma(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h4 snake4(f4 v, f4 ar, f4 ai)
{
    return h4{snrvq_f16(snrvq_snake(v[0], ar[0], ai[0])),
              snrvq_f16(snrvq_snake(v[1], ar[1], ai[1])),
              snrvq_f16(snrvq_snake(v[2], ar[2], ai[2])),
              snrvq_f16(snrvq_snake(v[3], ar[3], ai[3]))};
}

// fp32 residual rows in LDS: C floats per row, the 4-float slots of row r
// permuted by r mod (C/4), so 16 lanes reading 16 consecutive rows at one
// channel group hit 16 different bank groups.
template <int C>
__device__ __forceinline__ int xoff(int r, int c)
{
    return r * C + (c ^ ((r & (C / 4 - 1)) << 2));
}

// Per-channel parameter rows in LDS ([P_COUNT][C] fp32).
enum Prm {
    P_BT = 0,                                      // ConvT bias
    P_A1R0, P_A1I0, P_B70, P_A2R0, P_A2I0, P_B10,  // residual unit 0
    P_A1R1, P_A1I1, P_B71, P_A2R1, P_A2I1, P_B11,  // residual unit 1
    P_ANR, P_ANI,                                  // activation of the stage output
    P_COUNT
};

// One residual unit over output rows [lo, hi): conv7 (dilation D) of the
// activated input in LDS (row of time t at in + (t - in_t0) * CP), Snake,
// 1x1 conv, + bias + residual x (LDS fp32, row t - x_t0 of xs, see xoff);
// epi(t, c, v) receives channels c..c+3 of row t.
template <int C, int D, int RB, int NW, int U, class Epi>
__device__ __forceinline__ void residual_unit(const half_t *in, int in_t0, int lo, int hi,
                                              const half_t *W7, int ld7, const half_t *W1,
                                              int ld1, const float *prm, const float *xs,
                                              int x_t0, half_t *hsw, Epi epi)
{
    constexpr int CP = C + 8;
    constexpr int NB = C / 16;
    constexpr int K7 = 7 * C;
    constexpr int PB7 = U ? P_B71 : P_B70, PA2R = U ? P_A2R1 : P_A2R0,
                  PA2I = U ? P_A2I1 : P_A2I0, PB1 = U ? P_B11 : P_B10;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int nblk = (hi - lo + 15) / 16;
    for (int rb0 = wave; rb0 < nblk; rb0 += NW * RB) {
        f4 acc[RB][NB];
#pragma unroll
        for (int j = 0; j < RB; j++)
#pragma unroll
            for (int n = 0; n < NB; n++)
                acc[j][n] = f4{0.f, 0.f, 0.f, 0.f};
        int rowoff[RB];
#pragma unroll
        for (int j = 0; j < RB; j++) {
            int t = lo + (rb0 + j * NW) * 16 + l16;
            t = t < hi ? t : hi - 1;
            rowoff[j] = (t - in_t0) * CP + lg * 8;
        }
#pragma unroll 2
        for (int k0 = 0; k0 < K7; k0 += 32) {
            const int tap = k0 / C, c0 = k0 - tap * C;
            const int sh = (tap - 6) * D * CP + c0;
            h8 wf[NB];
#pragma unroll
            for (int n = 0; n < NB; n++)
                wf[n] = *(const h8 *)(W7 + (n * 16 + l16) * ld7 + k0 + lg * 8);
#pragma unroll
            for (int j = 0; j < RB; j++) {
                if (rb0 + j * NW < nblk) {
                    h8 xf = *(const h8 *)(in + rowoff[j] + sh);
#pragma unroll
                    for (int n = 0; n < NB; n++)
                        acc[j][n] = mma(wf[n], xf, acc[j][n]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < RB; j++) {
            const int blk = rb0 + j * NW;
            if (blk >= nblk)
                continue;
            // Snake(conv7 + b7) -> this wave's scratch, row l16, 4 channels per lane
#pragma unroll
            for (int n = 0; n < NB; n++) {
                const int c = n * 16 + lg * 4;
                const f4 b7 = *(const f4 *)(prm + PB7 * C + c);
                const f4 ar = *(const f4 *)(prm + PA2R * C + c);
                const f4 ai = *(const f4 *)(prm + PA2I * C + c);
                *(h4 *)(hsw + l16 * CP + c) = snake4(acc[j][n] + b7, ar, ai);
            }
            wave_lds_sync();
            f4 a2c[NB];
#pragma unroll
            for (int n = 0; n < NB; n++)
                a2c[n] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c0 = 0; c0 < C; c0 += 32) {
                const h8 hf = *(const h8 *)(hsw + l16 * CP + c0 + lg * 8);
#pragma unroll
                for (int n = 0; n < NB; n++) {
                    const h8 wf = *(const h8 *)(W1 + (n * 16 + l16) * ld1 + c0 + lg * 8);
                    a2c[n] = mma(wf, hf, a2c[n]);
                }
            }
            wave_lds_sync();
            const int t = lo + blk * 16 + l16;
            if (t < hi) {
#pragma unroll
                for (int n = 0; n < NB; n++) {
                    const int c = n * 16 + lg * 4;
                    const f4 b1 = *(const f4 *)(prm + PB1 * C + c);
                    const f4 xr = *(const f4 *)(xs + xoff<C>(t - x_t0, c));
                    epi(t, c, (a2c[n] + b1) + xr);
                }
            }
        }
    }
}

template <int C, int S, int T, bool FINAL, bool WL, int NW>
__global__ __launch_bounds__(NW * 64) void stage_kernel(StageArgs p)
{
    constexpr int NT_ = NW * 64;
    constexpr int E = FINAL ? 6 : 0;
    constexpr int HX = S * ((24 + E + S - 1) / S);  // ConvT rows recomputed before t0
    constexpr int NX = T + HX;                      // a1 rows: [t0 - HX, t0 + T)
    constexpr int NR = T + 18 + E;                  // x and a2 rows: [t0 - 18 - E, t0 + T)
    constexpr int CP = C + 8;
    constexpr int RB = NW >= 16 && C >= 64 ? 2 : 4;
    constexpr int CIN = 2 * C;
    constexpr int NT = S * C, KT = 2 * CIN, NBT = NT / 16;
    // ConvT column blocks per work item: 2 with 16 waves (enough items for
    // every wave), else the largest divisor of NBT <= 8 (fewer re-reads of
    // the item's input rows, which are loaded once, up front)
    constexpr int NG = NW >= 16 ? (NBT % 2 == 0 ? 2 : 1)
                                : (NBT % 8 == 0 ? 8 : NBT % 6 == 0 ? 6 : NBT % 4 == 0 ? 4 : NBT % 2 == 0 ? 2 : 1);
    constexpr int NGR = NBT / NG;
    constexpr int NKT = KT / 32;
    static_assert(T % S == 0 && NT % 16 == 0 && C % 32 == 0, "shape");

    __shared__ __attribute__((aligned(16))) float xs[NR * C];
    __shared__ __attribute__((aligned(16))) half_t a1s[NX * CP];  // a1, then a_out (FINAL)
    __shared__ __attribute__((aligned(16))) half_t a2s[NR * CP];
    __shared__ __attribute__((aligned(16))) half_t hs[NW * 16 * CP];
    __shared__ __attribute__((aligned(16))) float prm[P_COUNT * C];
    constexpr int LDT = KT + 8, LD7 = 7 * C + 8, LD1 = C + 8;
    constexpr int WBYTES = WL ? 2 * (NT * LDT + 2 * C * LD7 + 2 * C * LD1) : 16;
    __shared__ __attribute__((aligned(16))) char wsm[WBYTES];
    __shared__ float wout_s[FINAL ? 7 * C : 1];  // final conv weights, [tap][channel]
    half_t *const wTs = (half_t *)wsm;
    half_t *const w7s = wTs + NT * LDT;
    half_t *const w1s = w7s + 2 * C * LD7;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;

    {
        const float *src[P_COUNT] = {p.bT,      p.al1[0], p.ial1[0], p.b7[0], p.al2[0],
                                     p.ial2[0], p.b1[0],  p.al1[1], p.ial1[1], p.b7[1],
                                     p.al2[1],  p.ial2[1], p.b1[1],  p.al_next, p.ial_next};
        for (int i = tid; i < P_COUNT * C; i += NT_)
            prm[i] = src[i / C][i % C];
    }
    if (WL) {
        auto copy = [&](half_t *dst, int ld, const half_t *src, int rows, int cols) {
            const int cpr = cols / 8;
            for (int i = tid; i < rows * cpr; i += NT_) {
                const int r = i / cpr, c8 = (i - r * cpr) * 8;
                *(h8 *)(dst + r * ld + c8) = *(const h8 *)(src + (long)r * cols + c8);
            }
        };
        copy(wTs, LDT, p.WT, NT, KT);
        for (int j = 0; j < 2; j++) {
            copy(w7s + j * C * LD7, LD7, p.W7[j], C, 7 * C);
            copy(w1s + j * C * LD1, LD1, p.W1[j], C, C);
        }
    }
    if (FINAL) {
        for (int i = tid; i < 7 * C; i += NT_) {
            const int c = i / 7, j = i - c * 7;  // input layout [C][7]
            wout_s[j * C + c] = p.w_out[i];
        }
    }
    const half_t *const WT = WL ? wTs : p.WT;
    const int ldT = WL ? LDT : KT;
    const half_t *const W7a = WL ? w7s : p.W7[0];
    const half_t *const W7b = WL ? w7s + C * LD7 : p.W7[1];
    const half_t *const W1a = WL ? w1s : p.W1[0];
    const half_t *const W1b = WL ? w1s + C * LD1 : p.W1[1];
    const int ld7 = WL ? LD7 : 7 * C, ld1 = WL ? LD1 : C;
    __syncthreads();  // parameters and weights are in LDS

    for (int g = blockIdx.x; g < p.n_tiles; g += gridDim.x) {
        if (g != (int)blockIdx.x)
            __syncthreads();  // the previous tile's LDS reads are done
        const int f = g / p.tiles_per_frame;
        const int b = p.frame_stream[f];
        const int cu0 = p.cu[b];
        const int rows_b = (p.cu[b + 1] - cu0) * p.r_out;
        const int t0 = (g - cu0 * p.tiles_per_frame) * T;
        const bool first = t0 == 0, last = t0 + T == rows_b;
        half_t *hsw = hs + wave * 16 * CP;
        half_t *slot_state = p.state + (long)p.slot[b] * p.slot_elems;

        // ---- left context of a stream's first tile (written by the halo fill)
        if (first) {
            const half_t *s1 = p.a1_ext + ((long)b * 6 + (long)cu0 * p.r_out) * C;
            for (int i = tid; i < 6 * C / 8; i += NT_) {
                int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
                *(h8 *)(a1s + (HX - 6 + r) * CP + c8) = *(const h8 *)(s1 + r * C + c8);
            }
            const half_t *s2 = p.a2_ext + ((long)b * 18 + (long)cu0 * p.r_out) * C;
            for (int i = tid; i < 18 * C / 8; i += NT_) {
                int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
                *(h8 *)(a2s + (E + r) * CP + c8) = *(const h8 *)(s2 + r * C + c8);
            }
        }

        // ---- phase 1: transposed conv of input rows [qlo, qhi) -> x, a1
        {
            const int q0 = t0 / S;
            const int qlo = first ? 0 : q0 - HX / S;
            const int qhi = q0 + T / S;
            const int nbt = (qhi - qlo + 15) / 16;
            for (int item = wave; item < nbt * NGR; item += NW) {
                const int rb = item / NGR, ng = item - rb * NGR;
                f4 acc[NG];
#pragma unroll
                for (int n = 0; n < NG; n++)
                    acc[n] = f4{0.f, 0.f, 0.f, 0.f};
                int q = qlo + rb * 16 + l16;
                const bool qok = q < qhi;
                q = qok ? q : qhi - 1;
                const half_t *x1 =
                    p.aT + ((long)(b + 1) + (long)cu0 * p.r_in + q) * CIN + lg * 8;
                const half_t *x0 = x1 - CIN;
                const half_t *wt = WT + (ng * NG * 16 + l16) * ldT + lg * 8;
                h8 xf[NKT];
#pragma unroll
                for (int ks = 0; ks < NKT; ks++) {
                    const int k0 = ks * 32, tap = k0 / CIN, c0 = k0 - tap * CIN;
                    xf[ks] = *(const h8 *)((tap ? x1 : x0) + c0);
                }
#pragma unroll
                for (int ks = 0; ks < NKT; ks++) {
#pragma unroll
                    for (int n = 0; n < NG; n++) {
                        const h8 wf = *(const h8 *)(wt + n * 16 * ldT + ks * 32);
                        acc[n] = mma(wf, xf[ks], acc[n]);
                    }
                }
                if (qok) {
#pragma unroll
                    for (int n = 0; n < NG; n++) {
                        const int col = (ng * NG + n) * 16 + lg * 4;
                        const int r = col / C, c = col - r * C;
                        const int t = q * S + r;
                        const f4 v = acc[n] + *(const f4 *)(prm + P_BT * C + c);
                        if (t >= t0 - 18 - E)
                            *(f4 *)(xs + xoff<C>(t - (t0 - 18 - E), c)) = v;
                        *(h4 *)(a1s + (t - (t0 - HX)) * CP + c) =
                            snake4(v, *(const f4 *)(prm + P_A1R0 * C + c),
                                   *(const f4 *)(prm + P_A1I0 * C + c));
                    }
                }
            }
        }
        __syncthreads();

        // ---- phase 2: residual unit, dilation 1, rows [lo2, t0 + T)
        if (last) {  // new left context of the dilation-1 conv: last 6 rows of a1
            half_t *d = slot_state + p.off_a1;
            for (int i = tid; i < 6 * C / 8; i += NT_) {
                int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
                *(h8 *)(d + r * C + c8) = *(const h8 *)(a1s + (T + HX - 6 + r) * CP + c8);
            }
        }
        {
            const int lo2 = first ? 0 : t0 - 18 - E;
            const int xt0 = t0 - 18 - E;
            residual_unit<C, 1, RB, NW, 0>(a1s, t0 - HX, lo2, t0 + T, W7a, ld7, W1a, ld1, prm, xs,
                                           xt0, hsw, [&](int t, int c, f4 v) {
                                               *(f4 *)(xs + xoff<C>(t - xt0, c)) = v;
                                               *(h4 *)(a2s + (t - xt0) * CP + c) = snake4(
                                                   v, *(const f4 *)(prm + P_A1R1 * C + c),
                                                   *(const f4 *)(prm + P_A1I1 * C + c));
                                           });
        }
        __syncthreads();

        // ---- phase 3: residual unit, dilation 3, rows [lo3, t0 + T)
        if (last) {  // new left context of the dilation-3 conv: last 18 rows of a2
            half_t *d = slot_state + p.off_a2;
            for (int i = tid; i < 18 * C / 8; i += NT_) {
                int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
                *(h8 *)(d + r * C + c8) = *(const h8 *)(a2s + (T + E + r) * CP + c8);
            }
        }
        if (FINAL && first) {  // left context of the final conv into a_out rows 0..5
            const half_t *s3 = p.ao_ext + ((long)b * 6 + (long)cu0 * p.r_out) * C;
            for (int i = tid; i < 6 * C / 8; i += NT_) {
                int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
                *(h8 *)(a1s + r * CP + c8) = *(const h8 *)(s3 + r * C + c8);
            }
        }
        {
            const int lo3 = first ? 0 : t0 - E;
            const int xt0 = t0 - 18 - E;
            const long next_base = ((long)(b + 1) + (long)cu0 * p.r_out) * C;
            residual_unit<C, 3, RB, NW, 1>(a2s, xt0, lo3, t0 + T, W7b, ld7, W1b, ld1, prm, xs,
                                           xt0, hsw, [&](int t, int c, f4 v) {
                                               const h4 y = snake4(
                                                   v, *(const f4 *)(prm + P_ANR * C + c),
                                                   *(const f4 *)(prm + P_ANI * C + c));
                                               if (FINAL)
                                                   *(h4 *)(a1s + (t - (t0 - 6)) * CP + c) = y;
                                               else
                                                   *(h4 *)(p.next + next_base + (long)t * C + c) =
                                                       y;
                                           });
        }

        if (FINAL) {
            __syncthreads();
            if (last) {  // new left context of the final conv: last 6 rows of a_out
                half_t *d = slot_state + p.off_ao;
                for (int i = tid; i < 6 * C / 8; i += NT_) {
                    int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
                    *(h8 *)(d + r * C + c8) = *(const h8 *)(a1s + (T + r) * CP + c8);
                }
            }
            // ---- phase 4: final conv, four threads per output sample, each
            // over one quarter of the channels, combined as (q0+q1)+(q2+q3)
            for (int i = tid; i < 4 * T; i += NT_) {
                const int t = t0 + (i >> 2), qp = i & 3;
                float part = 0.f;
#pragma unroll
                for (int j = 0; j < 7; j++) {
                    const half_t *row = a1s + (t - t0 + j) * CP + qp * (C / 4);
                    const float *wj = wout_s + j * C + qp * (C / 4);
#pragma unroll
                    for (int c0 = 0; c0 < C / 4; c0 += 8) {
                        h8 v = *(const h8 *)(row + c0);
#pragma unroll
                        for (int e = 0; e < 8; e++)
                            part += wj[c0 + e] * (float)v[e];
                    }
                }
                part += __shfl_xor(part, 1, 64);
                part += __shfl_xor(part, 2, 64);
                if (qp == 0) {
                    const float y = p.b_out + part;
                    p.pcm[(long)cu0 * p.r_out + t] = p.final_tanh ? tanhf(y) : y;
                }
            }
        }
    }  // tile loop
}

template <int C, int S, int T, bool FINAL, bool WL, int NW>
hipError_t launch_stage_t(const StageArgs &a, int F, hipStream_t st)
{
    StageArgs b = a;
    b.tiles_per_frame = a.r_out / T;
    b.n_tiles = F * b.tiles_per_frame;
    // weights resident in LDS: one persistent work-group per CU walks the tiles
    int grid = WL ? (b.n_tiles < a.n_cu ? b.n_tiles : a.n_cu) : b.n_tiles;
    hipLaunchKernelGGL((stage_kernel<C, S, T, FINAL, WL, NW>), dim3(grid), dim3(NW * 64), 0, st,
                       b);
    return hipGetLastError();
}

}  // namespace

// (C, stride, rows per frame at the output, final) -> an instantiated tile
int stage_fused_tile(int C, int S, int r_out, bool final_stage)
{
    if (final_stage) {
        if (C == 32 && S == 4 && r_out % 192 == 0)
            return 192;
        if (C == 32 && S == 2 && r_out % 256 == 0)
            return 256;
    } else {
        if (C == 64 && S == 3 && r_out % 240 == 0)
            return 240;
        if (C == 64 && S == 4 && r_out % 128 == 0)
            return 128;
    }
    return 0;
}

hipError_t launch_stage_fused(const StageArgs &a, int C, int S, int T, bool final_stage, int F,
                              hipStream_t st)
{
    if (F <= 0)
        return hipSuccess;
    if (final_stage) {
        if (C == 32 && S == 4 && T == 192)
            return launch_stage_t<32, 4, 192, true, true, 16>(a, F, st);
        if (C == 32 && S == 2 && T == 256)
            return launch_stage_t<32, 2, 256, true, true, 16>(a, F, st);
    } else {
        if (C == 64 && S == 3 && T == 240)
            return launch_stage_t<64, 3, 240, false, false, 8>(a, F, st);
        if (C == 64 && S == 4 && T == 128)
            return launch_stage_t<64, 4, 128, false, false, 16>(a, F, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace snrvq
