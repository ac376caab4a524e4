// kernels_conv.hip -- implicit-GEMM causal convolutions on CDNA4 MFMA.
//
// One kernel template serves every dense contraction of the decoder:
//   * causal dilated Conv1d (k = 7, dilation 1 or 3): taps are row shifts of
//     the channels-last extended input, so the GEMM's K dimension is
//     (tap, channel) and the A operand rows are gathered per output row;
//   * ConvTranspose1d of stride s and kernel 2s in polyphase form: output
//     sample q s + r = b + W_r x[q] + W_{r+s} x[q-1], i.e. a 2-tap causal
//     conv with N = s C_out whose output, in channels-last layout, is the
//     plain row-major [q][s C_out] matrix;
//   * 1x1 convs and linear layers (k = 1).
// The epilogue adds the bias, optionally adds an fp32 residual and stores it
// (the residual stream), and stores the next layer's MFMA operand with the
// next activation (Snake / ELU / GELU) applied, into that layer's extended
// buffer.  So every activation is computed once per element, and every conv
// reads operands that are ready for the matrix cores.
//
// Tiles: 256 threads (4 waves of 64), BM x BN output tile, BK = 32 (fp16,
// v_mfma_f32_16x16x32_f16) or 16 (fp32, v_mfma_f32_16x16x4_f32).  Global
// loads are 16-byte chunks staged through double-buffered LDS; the epilogue
// goes through LDS so that every global store is a 16-byte chunk of a row.
// Work-groups are remapped so that each XCD (dispatch round-robin over 8)
// owns a contiguous range of tiles, N-tiles of one M-row block adjacent, so
// the A rows (re-read by every tap and every N-tile) stay in one L2.
#include "internal.h"

namespace snrvq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

typedef uint32_t Chunk __attribute__((ext_vector_type(4)));

template <typename T>
struct Traits;
template <>
struct Traits<half_t> {
    static constexpr int BK = 32;
};
template <>
struct Traits<float> {
    static constexpr int BK = 16;
};

__device__ __forceinline__ float act_fn(float v, int act, float a, float ia)
{
    if (act == ACT_SNAKE)
        return snrvq_snake(v, a, ia);
    if (act == ACT_ELU)
        return snrvq_elu(v);
    if (act == ACT_GELU)
        return 0.5f * v * (1.f + erff(v * 0.7071067811865475f));
    return v;
}

template <typename T>
__device__ __forceinline__ void store4(T *dst, f4 v);
template <>
__device__ __forceinline__ void store4<half_t>(half_t *dst, f4 v)
{
    h4 h = {snrvq_f16(v[0]), snrvq_f16(v[1]), snrvq_f16(v[2]), snrvq_f16(v[3])};
    *(h4 *)dst = h;
}
template <>
__device__ __forceinline__ void store4<float>(float *dst, f4 v)
{
    *(f4 *)dst = v;
}

// Contiguous tile range per XCD: bid % 8 is the XCD a work-group lands on.
__device__ __forceinline__ int xcd_remap(int bid, int total)
{
    const int nx = 8;
    int q = total / nx, r = total % nx;
    int x = bid % nx, i = bid / nx;
    return x * q + (x < r ? x : r) + i;
}

template <typename T, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void conv_gemm_kernel(ConvArgs p)
{
    constexpr int BK = Traits<T>::BK;
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int CPR = BK / VEC;  // 16-byte chunks per tile row (4)
    constexpr int LD = BK + VEC;   // padded LDS row, elements
    constexpr int A_CH = BM * CPR, B_CH = BN * CPR;
    constexpr int A_PT = (A_CH + 255) / 256, B_PT = (B_CH + 255) / 256;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    static_assert(WM * WN == 4, "4 waves");
    static_assert(FM >= 1 && FN >= 1 && TM % 16 == 0 && TN % 16 == 0, "wave tile");
    constexpr int AB_BYTES = 2 * (BM + BN) * LD * (int)sizeof(T);
    constexpr int ELD = BN + 4;
    constexpr int EPI_BYTES = BM * ELD * 4;
    constexpr int SMEM = AB_BYTES > EPI_BYTES ? AB_BYTES : EPI_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    T *As = (T *)smem;
    T *Bs = As + 2 * BM * LD;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntm = (p.M + BM - 1) / BM, ntn = p.N / BN;
    const int tile = xcd_remap(blockIdx.x, ntm * ntn);
    const int tm = tile / ntn, tn = tile - tm * ntn;
    const int m0 = tm * BM, n0 = tn * BN;
    const int Ktot = p.taps * p.Cin;
    const T *A = (const T *)p.A;
    const T *W = (const T *)p.Wt;

    const T *a_ptr[A_PT];
    int a_lds[A_PT];
#pragma unroll
    for (int i = 0; i < A_PT; i++) {
        int c = tid + i * 256;
        int row = c / CPR, kc = c % CPR;
        if (c >= A_CH)
            row = 0;
        int m = m0 + row;
        int mm = m < p.M ? m : p.M - 1;
        int b = p.frame_stream[mm / p.rate_in];
        long ext = (long)(b + 1) * p.A_H + mm;
        a_ptr[i] = A + ext * p.Cin + kc * VEC;
        a_lds[i] = row * LD + kc * VEC;
    }
    const T *b_ptr[B_PT];
    int b_lds[B_PT];
#pragma unroll
    for (int i = 0; i < B_PT; i++) {
        int c = tid + i * 256;
        int row = c / CPR, kc = c % CPR;
        if (c >= B_CH)
            row = 0;
        b_ptr[i] = W + (long)(n0 + row) * Ktot + kc * VEC;
        b_lds[i] = row * LD + kc * VEC;
    }

    Chunk ra[A_PT], rb[B_PT];
    auto gload = [&](int ks) {
        int k0 = ks * BK;
        int tap = k0 / p.Cin;
        int c0 = k0 - tap * p.Cin;
        long off = (long)c0 - (long)(p.taps - 1 - tap) * p.dil * p.Cin;
#pragma unroll
        for (int i = 0; i < A_PT; i++)
            if (A_CH % 256 == 0 || tid + i * 256 < A_CH)
                ra[i] = *(const Chunk *)(a_ptr[i] + off);
#pragma unroll
        for (int i = 0; i < B_PT; i++)
            if (B_CH % 256 == 0 || tid + i * 256 < B_CH)
                rb[i] = *(const Chunk *)(b_ptr[i] + k0);
    };
    auto sstore = [&](int buf) {
        T *Ab = As + buf * BM * LD;
        T *Bb = Bs + buf * BN * LD;
#pragma unroll
        for (int i = 0; i < A_PT; i++)
            if (A_CH % 256 == 0 || tid + i * 256 < A_CH)
                *(Chunk *)(Ab + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PT; i++)
            if (B_CH % 256 == 0 || tid + i * 256 < B_CH)
                *(Chunk *)(Bb + b_lds[i]) = rb[i];
    };

    f4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    const int wm = wave / WN, wn = wave % WN;
    const int rbase = wm * TM, cbase = wn * TN;
    const int lrow = lane & 15, lk = lane >> 4;

    const int nk = Ktot / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ks++) {
        const int buf = ks & 1;
        if (ks + 1 < nk)
            gload(ks + 1);
        const T *Ab = As + buf * BM * LD;
        const T *Bb = Bs + buf * BN * LD;
        if constexpr (sizeof(T) == 2) {
            h8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; i++)
                af[i] = *(const h8 *)(Ab + (rbase + i * 16 + lrow) * LD + lk * 8);
#pragma unroll
            for (int j = 0; j < FN; j++)
                bf[j] = *(const h8 *)(Bb + (cbase + j * 16 + lrow) * LD + lk * 8);
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0,
                                                                       0, 0);
        } else {
            f4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; i++)
                af[i] = *(const f4 *)(Ab + (rbase + i * 16 + lrow) * LD + lk * 4);
#pragma unroll
            for (int j = 0; j < FN; j++)
                bf[j] = *(const f4 *)(Bb + (cbase + j * 16 + lrow) * LD + lk * 4);
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][kk], bf[j][kk],
                                                                         acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < nk)
            sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: bias into an LDS tile, then row-contiguous 16-byte stores
    float *epi = (float *)smem;
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
            int c = cbase + j * 16 + lrow;
            float bv = p.bias[(n0 + c) % p.Cout];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                int r = rbase + i * 16 + lk * 4 + e;
                epi[r * ELD + c] = acc[i][j][e] + bv;
            }
        }
    __syncthreads();
    constexpr int QPR = BN / 4;
    for (int q = tid; q < BM * QPR; q += 256) {
        int r = q / QPR, cq = (q - r * QPR) * 4;
        int m = m0 + r;
        if (m >= p.M)
            continue;
        int n = n0 + cq;
        f4 v = *(const f4 *)(epi + r * ELD + cq);
        if (p.res) {
            f4 rr = *(const f4 *)(p.res + (long)m * p.Cout + n);
            v = v + rr;
        }
        long orow = (long)m * p.s;
        if (p.out32)
            *(f4 *)(p.out32 + orow * p.Cout + n) = v;
        if (p.out16) {
            int ch = n % p.Cout;
            f4 y;
            if (p.act == ACT_SNAKE) {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    y[e] = act_fn(v[e], ACT_SNAKE, p.alpha[ch + e], p.inv_alpha[ch + e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    y[e] = act_fn(v[e], p.act, 0.f, 0.f);
            }
            int b = p.frame_stream[m / p.rate_in];
            long base = ((long)(b + 1) * p.out_H + orow) * p.Cout + n;
            store4<T>((T *)p.out16 + base, y);
        }
    }
}

struct TileDesc {
    int BM, BN;
    const char *name;
};

// fp16 operand tiles, in order of preference
const TileDesc H_TILES[] = {
    {128, 128, "h128x128"}, {256, 64, "h256x64"}, {128, 64, "h128x64"}, {256, 32, "h256x32"},
    {64, 64, "h64x64"},     {128, 32, "h128x32"}, {32, 64, "h32x64"},   {64, 32, "h64x32"},
};
const TileDesc F_TILES[] = {
    {64, 64, "f64x64"}, {128, 32, "f128x32"}, {64, 32, "f64x32"}, {64, 16, "f64x16"},
};
constexpr int NH = sizeof(H_TILES) / sizeof(H_TILES[0]);
constexpr int NF = sizeof(F_TILES) / sizeof(F_TILES[0]);

template <typename T, int BM, int BN, int WM, int WN>
hipError_t launch_t(const ConvArgs &a, hipStream_t st)
{
    int ntm = (a.M + BM - 1) / BM, ntn = a.N / BN;
    hipLaunchKernelGGL((conv_gemm_kernel<T, BM, BN, WM, WN>), dim3(ntm * ntn), dim3(256), 0, st,
                       a);
    return hipGetLastError();
}

}  // namespace

int conv_gemm_tile_choice(const ConvArgs &a, int dtype)
{
    const TileDesc *t = dtype ? H_TILES : F_TILES;
    int n = dtype ? NH : NF;
    int best = -1;
    long best_tiles = -1;
    for (int i = 0; i < n; i++) {
        if (a.N % t[i].BN != 0)
            continue;
        long tiles = (long)((a.M + t[i].BM - 1) / t[i].BM) * (a.N / t[i].BN);
        if (tiles >= 512)
            return i;
        if (tiles > best_tiles) {
            best_tiles = tiles;
            best = i;
        }
    }
    return best;
}

const char *conv_gemm_tile_name(int dtype, int tile)
{
    if (tile < 0)
        return "none";
    return dtype ? H_TILES[tile].name : F_TILES[tile].name;
}

hipError_t launch_conv_gemm(const ConvArgs &a, int dtype, hipStream_t st, int tile)
{
    if (a.M <= 0)
        return hipSuccess;
    if (tile < 0)
        tile = conv_gemm_tile_choice(a, dtype);
    if (tile < 0)
        return hipErrorInvalidValue;
    if (dtype) {
        switch (tile) {
        case 0: return launch_t<half_t, 128, 128, 2, 2>(a, st);
        case 1: return launch_t<half_t, 256, 64, 4, 1>(a, st);
        case 2: return launch_t<half_t, 128, 64, 2, 2>(a, st);
        case 3: return launch_t<half_t, 256, 32, 4, 1>(a, st);
        case 4: return launch_t<half_t, 64, 64, 2, 2>(a, st);
        case 5: return launch_t<half_t, 128, 32, 4, 1>(a, st);
        case 6: return launch_t<half_t, 32, 64, 2, 2>(a, st);
        case 7: return launch_t<half_t, 64, 32, 4, 1>(a, st);
        }
    } else {
        switch (tile) {
        case 0: return launch_t<float, 64, 64, 2, 2>(a, st);
        case 1: return launch_t<float, 128, 32, 4, 1>(a, st);
        case 2: return launch_t<float, 64, 32, 4, 1>(a, st);
        case 3: return launch_t<float, 64, 16, 4, 1>(a, st);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace snrvq
