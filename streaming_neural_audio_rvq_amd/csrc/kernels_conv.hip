// kernels_conv.hip -- implicit-GEMM causal convolutions on CDNA4 MFMA.
//
// One kernel template serves every dense contraction of the per-layer path:
//   * causal dilated Conv1d (k = 7, dilation 1 or 3): taps are row shifts of
//     the channels-last extended input, so the GEMM's K dimension is
//     (tap, channel) and the A operand rows are gathered per output row;
//   * ConvTranspose1d of stride s and kernel 2s in polyphase form: output
//     sample q s + r = b + W_r x[q] + W_{r+s} x[q-1], i.e. a 2-tap causal
//     conv with N = s C_out whose output, in channels-last layout, is the
//     plain row-major [q][s C_out] matrix;
//   * 1x1 convs and linear layers (k = 1).
// The accumulators start at the bias; the epilogue optionally adds an fp32
// residual and stores it
// (the residual stream), and stores the next layer's MFMA operand with the
// next activation (Snake / ELU / GELU) applied, into that layer's extended
// buffer.  So every activation is computed once per element, and every conv
// reads operands that are ready for the matrix cores.
//
// Tiles: 256 threads (4 waves of 64), BM x BN output tile, K staged in steps
// of BK = 32 KSUB (fp16, v_mfma_f32_16x16x32_f16) or 16 (fp32,
// v_mfma_f32_16x16x4_f32).  K stages are double-buffered in LDS (three
// buffers for the 128 x 64 and 64 x 128 tiles of the frame-rate layers).  fp16
// stages go global -> LDS directly (16-byte global_load_lds: no register
// staging and no LDS store instructions, which would otherwise share the LDS
// port with the fragment reads), into unpadded rows with XOR-permuted 16-byte
// chunks so that fragment reads stay conflict-free.  The weights are the MFMA's A operand and the activation rows
// its B operand, so each lane's accumulator holds 4 consecutive output
// columns of one row and the epilogue stores straight from registers (4
// channels per lane, 16 lanes per row segment).  Work-groups are remapped so that each XCD
// (dispatch round-robin over 8) owns a contiguous range of tiles, N-tiles of
// one M-row block adjacent, so the A rows (re-read by every tap and every
// N-tile) stay in one L2.
//
// Split-K (layers whose M x N has fewer tiles than the GPU has CUs, e.g. the
// frame-rate layers at a few hundred frames): blockIdx.y selects a
// contiguous K range; each split writes its fp32 partial tile and a reduce
// kernel sums the splits in split order, then applies the same epilogue.
// No atomics: the result depends only on the shapes, never on timing.
#include "internal.h"
#include <type_traits>

namespace snrvq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

typedef uint32_t Chunk __attribute__((ext_vector_type(4)));
#define GLOBAL_PTR(p) ((const void __attribute__((address_space(1))) *)(p))
#define LDS_PTR(p) ((void __attribute__((address_space(3))) *)(p))

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

template <int ACT>
__device__ __forceinline__ f4 act4t(f4 v, f4 a, f4 ia)
{
    f4 y;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        if constexpr (ACT == ACT_SNAKE)
            y[e] = snrvq_snake(v[e], a[e], ia[e]);
        else if constexpr (ACT == ACT_ELU)
            y[e] = snrvq_elu(v[e]);
        else if constexpr (ACT == ACT_GELU)
            y[e] = 0.5f * v[e] * (1.f + erff(v[e] * 0.7071067811865475f));
        else
            y[e] = v[e];
    }
    return y;
}

// Activation of 4 values: one uniform branch, then 4 independent evaluations.
__device__ __forceinline__ f4 act4(f4 v, int act, f4 a, f4 ia)
{
    if (act == ACT_SNAKE)
        return act4t<ACT_SNAKE>(v, a, ia);
    if (act == ACT_ELU)
        return act4t<ACT_ELU>(v, a, ia);
    if (act == ACT_GELU)
        return act4t<ACT_GELU>(v, a, ia);
    return v;
}

// Calls f(std::integral_constant<int, act>) for the runtime activation, so a
// loop over a whole tile is compiled once per activation, branch-free inside.
template <typename F>
__device__ __forceinline__ void with_act(int act, F &&f)
{
    if (act == ACT_SNAKE)
        f(std::integral_constant<int, ACT_SNAKE>());
    else if (act == ACT_ELU)
        f(std::integral_constant<int, ACT_ELU>());
    else if (act == ACT_GELU)
        f(std::integral_constant<int, ACT_GELU>());
    else
        f(std::integral_constant<int, ACT_NONE>());
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

// m / rate_in for any 32-bit m: round-up multiply-shift division with the
// constants the launcher derives from the divisor.
__device__ __forceinline__ int frame_of(const ConvArgs &p, int m)
{
    const uint32_t t = __umulhi(p.div_m, (uint32_t)m);
    return (int)((t + (((uint32_t)m - t) >> p.div_s1)) >> p.div_s2);
}

// Output of 4 consecutive columns n..n+3 of packed input row m (stream b),
// bias included: + residual, fp32 store, activation and compute-type store.
// al / ial: Snake parameters of the 4 output channels.
template <typename T>
__device__ __forceinline__ void epilogue4(const ConvArgs &p, int m, int b, int n, f4 v, f4 al,
                                          f4 ial)
{
    if (p.res) {
        f4 rr = *(const f4 *)(p.res + (long)m * p.Cout + n);
        v = v + rr;
    }
    long orow = (long)m * p.s;
    if (p.out32)
        *(f4 *)(p.out32 + orow * p.Cout + n) = v;
    if (p.out16) {
        const f4 y = act4(v, p.act, al, ial);
        long base = ((long)(b + 1) * p.out_H + orow) * p.Cout + n;
        store4<T>((T *)p.out16 + base, y);
    }
}

__device__ __forceinline__ void snake_params(const ConvArgs &p, int ch, f4 &al, f4 &ial)
{
    al = f4{0.f, 0.f, 0.f, 0.f};
    ial = al;
    if (p.out16 && p.act == ACT_SNAKE) {
        al = *(const f4 *)(p.alpha + ch);
        ial = *(const f4 *)(p.inv_alpha + ch);
    }
}

// Contiguous tile range per XCD: bid % 8 is the XCD a work-group lands on.
__device__ __forceinline__ int xcd_remap(int bid, int total)
{
    const int nx = 8;
    int q = total / nx, r = total % nx;
    int x = bid % nx, i = bid / nx;
    return x * q + (x < r ? x : r) + i;
}

// MINW: waves per SIMD the register allocation must leave room for (the
// 128 x 128 and 160-row tiles ask for 2: left to itself the compiler gives
// them more than 256 registers, i.e. one work-group per CU)
template <typename T, int BM, int BN, int WM, int WN, int KSUB, bool RU = false, int NBUF = 2,
          int MINW = 1>
__global__ __launch_bounds__(256, MINW) void conv_gemm_kernel(ConvArgs p)
{
    constexpr int BK0 = Traits<T>::BK;
    constexpr int BK = BK0 * KSUB;
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int CPR = BK / VEC;  // 16-byte chunks per tile row
    // fp16 tiles load global -> LDS directly (no register staging, no LDS
    // store instructions) into unpadded rows whose 16-byte chunks are
    // XOR-permuted so that a fragment read (16 rows, one chunk) is
    // conflict-free; fp32 tiles stage through registers into padded rows
    constexpr bool DIRECT = sizeof(T) == 2;
    constexpr int LD = DIRECT ? BK : BK + VEC;  // LDS row, elements
    constexpr int A_CH = BM * CPR, B_CH = BN * CPR;
    constexpr int A_PT = (A_CH + 255) / 256, B_PT = (B_CH + 255) / 256;
    // direct: one instruction of a wave fills 1 KB = RPI whole rows
    constexpr int RPI = 64 / CPR;
    constexpr int A_NI = BM / RPI, B_NI = BN / RPI;  // instructions per tile
    static_assert(!DIRECT || (BM % RPI == 0 && BN % RPI == 0), "direct rows");
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    static_assert(WM * WN == 4, "4 waves");
    static_assert(FM >= 1 && FN >= 1 && TM % 16 == 0 && TN % 16 == 0, "wave tile");
    // one LDS object holds both stage buffers and the row table; the K loop
    // reads the current buffer while the next stage's direct loads are in
    // flight into the other, and waits for them (vmcnt(0)) only before the
    // barrier that publishes them
    constexpr int SMEM_BUF = (BM + BN) * LD * (int)sizeof(T);
    constexpr int SMEM_RU0 = RU ? BM * (BN + 8) * 2 : 0;  // h tile
    constexpr int SMEM_RU1 = RU ? 2 * BN * 72 * 2 : 0;    // 1x1 weight chunks
    // NBUF > 2 stage buffers (fp16 direct loads only): the loads of stage
    // ks + NBUF - 1 are issued while stage ks is multiplied, so a stage's
    // loads have NBUF - 1 stages of MFMA work to land in
    static_assert(NBUF == 2 || (DIRECT && !RU), "deep pipeline: fp16 direct loads");
    constexpr int SMEM0 = SMEM_BUF > SMEM_RU0 ? SMEM_BUF : SMEM_RU0;
    constexpr int SMEM1 = (SMEM_BUF > SMEM_RU1 ? SMEM_BUF : SMEM_RU1) + (NBUF - 2) * SMEM_BUF;
    __shared__ __attribute__((aligned(16))) char smem[SMEM0 + SMEM1 + BM * 4];
    char *const smem0 = smem, *const smem1 = smem + SMEM0;
    int *const rowb = (int *)(smem + SMEM0 + SMEM1);
    T *const A0 = (T *)smem0, *const B0 = A0 + BM * LD;
    T *const A1 = (T *)smem1, *const B1 = A1 + BM * LD;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntm = (p.M + BM - 1) / BM, ntn = p.N / BN;
    const int tile = xcd_remap(blockIdx.x, ntm * ntn);
    const int tm = tile / ntn, tn = tile - tm * ntn;
    const int m0 = tm * BM, n0 = tn * BN;
    const int Ktot = p.taps * p.Cin;
    const T *A = (const T *)p.A;
    const T *W = (const T *)p.Wt;

    // K range of this split (whole K without split-K)
    const int nk_all = Ktot / BK;
    const int per = (nk_all + p.splits - 1) / p.splits;
    const int ks0 = blockIdx.y * per;
    const int ks1 = ks0 + per < nk_all ? ks0 + per : nk_all;

    // physical chunk of logical chunk kc in row r: kc ^ swz(r); the 8 rows
    // one 128-byte LDS line pass spans land on 8 distinct chunks
    auto swz = [](int r) { return DIRECT ? (r * CPR / 8) & (CPR - 1) : 0; };

    // load slot i of this thread: tile row, logical chunk, LDS offset
    auto slot = [&](int i, int nrows, int &row, int &kc, int &lo) -> bool {
        if constexpr (DIRECT) {
            const int blk = i * 4 + wave;
            row = blk * RPI + lane / CPR;
            kc = (lane % CPR) ^ swz(row);
            lo = blk * RPI * LD;  // wave-uniform
            if (blk >= nrows / RPI) {
                row = 0;
                return false;
            }
            return true;
        } else {
            const int c = tid + i * 256;
            row = c / CPR;
            kc = c % CPR;
            lo = row * LD + kc * VEC;
            if (c >= nrows * CPR) {
                row = 0;
                return false;
            }
            return true;
        }
    };
    constexpr int A_N = DIRECT ? (A_NI + 3) / 4 : A_PT;
    constexpr int B_N = DIRECT ? (B_NI + 3) / 4 : B_PT;
    constexpr bool A_FULL = DIRECT ? A_NI % 4 == 0 : A_CH % 256 == 0;
    constexpr bool B_FULL = DIRECT ? B_NI % 4 == 0 : B_CH % 256 == 0;

    const T *a_ptr[A_N];
    int a_lds[A_N];
    bool a_ok[A_N];
#pragma unroll
    for (int i = 0; i < A_N; i++) {
        int row, kc;
        a_ok[i] = slot(i, BM, row, kc, a_lds[i]);
        int m = m0 + row;
        int mm = m < p.M ? m : p.M - 1;
        int b = p.frame_stream[frame_of(p, mm)];
        long ext = (long)(b + 1) * p.A_H + mm;
        a_ptr[i] = A + ext * p.Cin + kc * VEC;
        if (a_ok[i] && (DIRECT ? lane % CPR == 0 : kc == 0))
            rowb[row] = b;
    }
    const T *b_ptr[B_N];
    int b_lds[B_N];
    bool b_ok[B_N];
#pragma unroll
    for (int i = 0; i < B_N; i++) {
        int row, kc;
        b_ok[i] = slot(i, BN, row, kc, b_lds[i]);
        b_ptr[i] = W + (long)(n0 + row) * Ktot + kc * VEC;
    }

    Chunk ra[DIRECT ? 1 : A_N], rb[DIRECT ? 1 : B_N];
    // a K stage of BK never straddles two taps (C_in is a multiple of BK).
    // Stages are loaded in order, so the element offsets of the next stage's
    // loads advance by BK, and by dil Cin - Cin more where a tap ends (the A
    // rows of tap t sit (taps - 1 - t) dil rows back): a few scalar adds per
    // stage, no division or 64-bit multiply
    int g_c0, a_off, b_off = ks0 * BK;
    {
        const int tap0 = (ks0 * BK) / p.Cin;
        g_c0 = ks0 * BK - tap0 * p.Cin;
        a_off = g_c0 - (p.taps - 1 - tap0) * p.dil * p.Cin;
    }
    const int tap_jump = (p.dil - 1) * p.Cin;
    auto gload = [&](T *Ab, T *Bb) {
        const int off = a_off, k0 = b_off;
        a_off += BK;
        b_off += BK;
        g_c0 += BK;
        if (g_c0 == p.Cin) {
            g_c0 = 0;
            a_off += tap_jump;
        }
        if constexpr (DIRECT) {
#pragma unroll
            for (int i = 0; i < A_N; i++)
                if (A_FULL || a_ok[i])
                    __builtin_amdgcn_global_load_lds(GLOBAL_PTR(a_ptr[i] + off),
                                                     LDS_PTR(Ab + a_lds[i]), 16, 0, 0);
#pragma unroll
            for (int i = 0; i < B_N; i++)
                if (B_FULL || b_ok[i])
                    __builtin_amdgcn_global_load_lds(GLOBAL_PTR(b_ptr[i] + k0),
                                                     LDS_PTR(Bb + b_lds[i]), 16, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < A_N; i++)
                if (A_FULL || a_ok[i])
                    ra[i] = *(const Chunk *)(a_ptr[i] + off);
#pragma unroll
            for (int i = 0; i < B_N; i++)
                if (B_FULL || b_ok[i])
                    rb[i] = *(const Chunk *)(b_ptr[i] + k0);
        }
    };
    auto sstore = [&](T *Ab, T *Bb) {
        if constexpr (!DIRECT) {
#pragma unroll
            for (int i = 0; i < A_N; i++)
                if (A_FULL || a_ok[i])
                    *(Chunk *)(Ab + a_lds[i]) = ra[i];
#pragma unroll
            for (int i = 0; i < B_N; i++)
                if (B_FULL || b_ok[i])
                    *(Chunk *)(Bb + b_lds[i]) = rb[i];
        }
    };
    // the direct loads of a stage must have landed before the barrier that
    // publishes it
    auto loads_done = [&]() {
        if constexpr (DIRECT)
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    };

    const int wm = wave / WN, wn = wave % WN;
    const int rbase = wm * TM, cbase = wn * TN;
    const int lrow = lane & 15, lk = lane >> 4;
    const bool split = p.splits > 1;

    // accumulators start at the bias (of the k = 7 conv in a residual-unit
    // launch): the first MFMA of the K loop takes it as its C operand.
    // Split-K partials start at zero and the reduce adds the bias.
    // (loaded after the first stage's loads are issued, all four together)
    f4 binit[FN];
    auto load_bias = [&]() {
        if (split) {
#pragma unroll
            for (int j = 0; j < FN; j++)
                binit[j] = f4{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int ch = (n0 + cbase + j * 16 + lk * 4) % p.Cout;
                binit[j] = *(const f4 *)((RU ? p.bias7 : p.bias) + ch);
            }
        }
    };
    f4 acc[FM][FN];

    const int fsw = swz(lrow);  // fragment rows are lrow + multiples of 16
    auto mma_stage = [&](const T *Ab, const T *Bb, auto first) {
#pragma unroll
        for (int sub = 0; sub < KSUB; sub++) {
            // C operand: the bias for the first MFMA of each output
            auto cin = [&](int i, int j) {
                if constexpr (decltype(first)::value)
                    return sub == 0 ? binit[j] : acc[i][j];
                else
                    return acc[i][j];
            };
            if constexpr (sizeof(T) == 2) {
                h8 af[FM], bf[FN];
#pragma unroll
                for (int i = 0; i < FM; i++)
                    af[i] = *(const h8 *)(Ab + (rbase + i * 16 + lrow) * LD +
                                          ((sub * 4 + lk) ^ fsw) * 8);
#pragma unroll
                for (int j = 0; j < FN; j++)
                    bf[j] = *(const h8 *)(Bb + (cbase + j * 16 + lrow) * LD +
                                          ((sub * 4 + lk) ^ fsw) * 8);
                __builtin_amdgcn_s_setprio(1);  // keep the matrix pipe fed
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[j], af[i],
                                                                           cin(i, j), 0, 0, 0);
            } else {
                f4 af[FM], bf[FN];
#pragma unroll
                for (int i = 0; i < FM; i++)
                    af[i] = *(const f4 *)(Ab + (rbase + i * 16 + lrow) * LD + sub * 16 + lk * 4);
#pragma unroll
                for (int j = 0; j < FN; j++)
                    bf[j] = *(const f4 *)(Bb + (cbase + j * 16 + lrow) * LD + sub * 16 + lk * 4);
#pragma unroll
                for (int kk = 0; kk < 4; kk++)
#pragma unroll
                    for (int i = 0; i < FM; i++)
#pragma unroll
                        for (int j = 0; j < FN; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                bf[j][kk], af[i][kk], kk == 0 ? cin(i, j) : acc[i][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    if constexpr (NBUF > 2) {
        // stage j of this split sits in buffer j mod NBUF; every wave issues
        // the same LPS loads per stage, so "stage ks has landed" is a vmcnt
        // of LPS times the number of younger stages in flight
        static_assert(A_FULL && B_FULL, "uniform loads per wave");
        constexpr int LPS = A_N + B_N;
        // byte offsets of the buffer read next and of the one loaded next,
        // each stepping through the NBUF buffers in turn
        int rd = 0, wr = 0;
        auto step = [](int o) { return o + SMEM_BUF == NBUF * SMEM_BUF ? 0 : o + SMEM_BUF; };
        auto bufA = [&](int o) { return (T *)(smem + o); };
        auto bufB = [&](int o) { return bufA(o) + BM * LD; };
        load_bias();
        int issued = ks0;
#pragma unroll
        for (int i = 0; i < NBUF - 1; i++)
            if (issued < ks1) {
                gload(bufA(wr), bufB(wr));
                wr = step(wr);
                issued++;
            }
        if (ks0 >= ks1) {
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = binit[j];
        }
        // the row table written above must be in LDS before the first bare
        // barrier publishes it (lgkmcnt(0) only; the loads keep flying)
        __builtin_amdgcn_s_waitcnt(0xc07f);
        for (int ks = ks0; ks < ks1; ks++) {
            if (issued - ks - 1 == NBUF - 2)
                __builtin_amdgcn_s_waitcnt(0x3f70 | ((LPS * (NBUF - 2)) & 15) |
                                           (((LPS * (NBUF - 2)) >> 4) << 14));
            else
                __builtin_amdgcn_s_waitcnt(0x3f70);  // tail: everything
            // stage ks is visible to every wave, and the buffer of stage
            // ks - 1 is free (every wave is done with it).  A bare barrier:
            // __syncthreads() would also wait for the younger stages' loads
            // (its release fence waits for every outstanding memory op)
            __asm__ volatile("s_barrier" ::: "memory");
            if (issued < ks1) {
                gload(bufA(wr), bufB(wr));
                wr = step(wr);
                issued++;
            }
            if (ks == ks0)
                mma_stage(bufA(0), bufB(0), std::true_type());
            else
                mma_stage(bufA(rd), bufB(rd), std::false_type());
            rd = step(rd);
        }
    } else {  // two stage buffers
        if (ks0 < ks1) {
            gload(A0, B0);
            sstore(A0, B0);
        }
        load_bias();
        loads_done();
        __syncthreads();
        // first K stage (buffer 0) peeled: its MFMAs start from the bias
        if (ks0 < ks1) {
            if (ks0 + 1 < ks1)
                gload(A1, B1);
            mma_stage(A0, B0, std::true_type());
            if (ks0 + 1 < ks1)
                sstore(A1, B1);
            loads_done();
            __syncthreads();
        } else {
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = binit[j];
        }
        for (int ks = ks0 + 1; ks < ks1; ks++) {
            const int buf = (ks - ks0) & 1;
            T *const Ac = buf ? A1 : A0, *const Bc = buf ? B1 : B0;
            T *const An = buf ? A0 : A1, *const Bn = buf ? B0 : B1;
            if (ks + 1 < ks1)
                gload(An, Bn);
            mma_stage(Ac, Bc, std::false_type());
            if (ks + 1 < ks1)
                sstore(An, Bn);
            loads_done();
            __syncthreads();
        }
    }

    if constexpr (RU) {
        // ---- residual unit: h = act7(conv7 + b7) into LDS (the staging
        // buffers are free after the main loop's last barrier), then the 1x1
        // conv over h with its weights streamed through LDS in K chunks
        static_assert(sizeof(T) == 2, "fp16 operands");
        constexpr int HP = BN + 8;           // h row pitch
        constexpr int B1 = 64, LD1 = B1 + 8; // 1x1 K chunk and its pitch
        constexpr int NK1 = BN / B1;
        constexpr int W1_PT = BN * (B1 / 8) / 256;
        static_assert(BN * (B1 / 8) % 256 == 0 && BN % B1 == 0, "1x1 chunks");
        static_assert(BM * HP * 2 <= SMEM0 && 2 * BN * LD1 * 2 <= SMEM1, "LDS");
        half_t *hS = (half_t *)smem0;
        half_t *w1s = (half_t *)smem1;
        const half_t *W1 = (const half_t *)p.W1;
        Chunk wr[W1_PT];
        auto w1load = [&](int kc) {
#pragma unroll
            for (int i = 0; i < W1_PT; i++) {
                const int k = tid + i * 256, row = k / (B1 / 8), c8 = (k % (B1 / 8)) * 8;
                wr[i] = *(const Chunk *)(W1 + (long)row * BN + kc * B1 + c8);
            }
        };
        auto w1store = [&](int buf) {
#pragma unroll
            for (int i = 0; i < W1_PT; i++) {
                const int k = tid + i * 256, row = k / (B1 / 8), c8 = (k % (B1 / 8)) * 8;
                *(Chunk *)(w1s + buf * BN * LD1 + row * LD1 + c8) = wr[i];
            }
        };
        w1load(0);
        with_act(p.act7, [&](auto act) {
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int ch = cbase + j * 16 + lk * 4;  // one N tile: n0 == 0
                const f4 b1 = *(const f4 *)(p.bias + ch);
                f4 a7 = f4{0.f, 0.f, 0.f, 0.f}, ia7 = a7;
                if constexpr (decltype(act)::value == ACT_SNAKE) {
                    a7 = *(const f4 *)(p.alpha7 + ch);
                    ia7 = *(const f4 *)(p.inv_alpha7 + ch);
                }
#pragma unroll
                for (int i = 0; i < FM; i++) {
                    const f4 y = act4t<decltype(act)::value>(acc[i][j], a7, ia7);
                    store4<half_t>(hS + (rbase + i * 16 + lrow) * HP + ch, y);
                    acc[i][j] = b1;  // the 1x1 conv starts at its bias
                }
            }
        });
        w1store(0);
        __syncthreads();
        for (int kc = 0; kc < NK1; kc++) {
            if (kc + 1 < NK1)
                w1load(kc + 1);
            const half_t *Wb = w1s + (kc & 1) * BN * LD1;
#pragma unroll
            for (int sub = 0; sub < B1 / 32; sub++) {
                h8 af[FM], bf[FN];
#pragma unroll
                for (int i = 0; i < FM; i++)
                    af[i] = *(const h8 *)(hS + (rbase + i * 16 + lrow) * HP + kc * B1 + sub * 32 +
                                          lk * 8);
#pragma unroll
                for (int j = 0; j < FN; j++)
                    bf[j] = *(const h8 *)(Wb + (cbase + j * 16 + lrow) * LD1 + sub * 32 + lk * 8);
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[j], af[i],
                                                                           acc[i][j], 0, 0, 0);
            }
            if (kc + 1 < NK1)
                w1store((kc + 1) & 1);
            __syncthreads();
        }
    }

    // ---- epilogue straight from the accumulators: weights are the MFMA's A
    // operand, so acc[i][j] holds 4 consecutive output columns of one row
    f4 al4[FN], ial4[FN];
    int nj[FN], chj[FN];
#pragma unroll
    for (int j = 0; j < FN; j++) {
        nj[j] = n0 + cbase + j * 16 + lk * 4;
        chj[j] = nj[j] % p.Cout;
        snake_params(p, chj[j], al4[j], ial4[j]);
    }
    if (split) {
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int m = m0 + rbase + i * 16 + lrow;
            if (m < p.M)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    *(f4 *)(p.partial + ((long)blockIdx.y * p.M + m) * p.N + nj[j]) = acc[i][j];
        }
        return;
    }
    // one code path per activation.  The residual loads: where the epilogue
    // also writes the fp32 stream (the first residual unit of a stage), all
    // of the tile's are issued together before any is used, so they take one
    // memory round trip instead of one per row block (stage-2 residual unit
    // 75 -> 72 us at 128 streams); where it writes only the 16-bit
    // activation, those of one row block at a time (the batched form was
    // 2-3 us slower there)
    f4 rr[FM][FN];
    const bool res_all = p.res && p.out32;
    if (res_all) {
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int m = m0 + rbase + i * 16 + lrow;
            const int mc = m < p.M ? m : p.M - 1;  // loads stay in bounds
#pragma unroll
            for (int j = 0; j < FN; j++)
                rr[i][j] = *(const f4 *)(p.res + (long)mc * p.Cout + nj[j]);
        }
    }
    with_act(p.out16 ? p.act : ACT_NONE, [&](auto act) {
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int r = rbase + i * 16 + lrow;
            const int m = m0 + r;
            const int mc = m < p.M ? m : p.M - 1;  // loads stay in bounds
            f4 v[FN];
#pragma unroll
            for (int j = 0; j < FN; j++)
                v[j] = acc[i][j];  // bias included
            if (p.res) {
                if (!res_all) {
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        rr[i][j] = *(const f4 *)(p.res + (long)mc * p.Cout + nj[j]);
                }
#pragma unroll
                for (int j = 0; j < FN; j++)
                    v[j] = v[j] + rr[i][j];
            }
            if (m >= p.M)
                continue;
            const long orow = (long)m * p.s;
            if (p.out32)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    *(f4 *)(p.out32 + orow * p.Cout + nj[j]) = v[j];
            if (p.out16) {
                T *o = (T *)p.out16 + ((long)(rowb[r] + 1) * p.out_H + orow) * p.Cout;
#pragma unroll
                for (int j = 0; j < FN; j++)
                    store4<T>(o + nj[j], act4t<decltype(act)::value>(v[j], al4[j], ial4[j]));
            }
        }
    });
}

// Sum of the split-K partials in split order, + bias, then the epilogue.
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(ConvArgs p)
{
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    const long nq = (long)p.M * (p.N / 4);
    if (q >= nq)
        return;
    const int m = (int)(q / (p.N / 4));
    const int n = (int)(q - (long)m * (p.N / 4)) * 4;
    const long stride = (long)p.M * p.N;
    f4 v = *(const f4 *)(p.partial + (long)m * p.N + n);
    for (int s = 1; s < p.splits; s++)
        v = v + *(const f4 *)(p.partial + s * stride + (long)m * p.N + n);
    const int ch = n % p.Cout;
    v = v + *(const f4 *)(p.bias + ch);
    f4 al, ial;
    snake_params(p, ch, al, ial);
    epilogue4<T>(p, m, p.out16 ? p.frame_stream[frame_of(p, m)] : 0, n, v, al, ial);
}

struct TileDesc {
    int BM, BN, BK;
    const char *name;
    bool deep = false;  // three K stage buffers
};

// fp16 operand tiles, in order of preference
const TileDesc H_TILES[] = {
    {128, 128, 64, "h128x128k64"}, {128, 64, 64, "h128x64k64"}, {64, 128, 64, "h64x128k64"},
    {64, 64, 64, "h64x64k64"},     {256, 32, 32, "h256x32"},    {128, 32, 32, "h128x32"},
    {32, 64, 32, "h32x64"},        {64, 32, 32, "h64x32"},
    // three stage buffers: two work-groups per CU still fit (74 KB of LDS each)
    {128, 64, 64, "h128x64k64b3", true}, {64, 128, 64, "h64x128k64b3", true},
    // 160 rows: taken instead of 128 x 128 when that tile would leave a small
    // last round of work-groups (see tall_rows below)
    {160, 128, 64, "h160x128k64"},
};
constexpr int TILE_128 = 0, TILE_TALL = 10;
// fp16 tiles tried first, unsplit: 128 x 128 (double-buffered), then the
// three-buffer half tiles.  Timed alone on the 128-stream layer shapes, a
// half tile with its loads three stages deep beats a split 128 x 128 tile on
// the frame-rate layers (k = 7 conv 6352 x 512 x 3584: 35 us against 40 us
// split in two; transposed conv 794 x 4096 x 2048: 28 against 35 us), while
// on layers that fill the GPU unsplit the double-buffered 128 x 128 tile
// stays ahead of every deeper pipeline (31760 x 256 x 1792: 33 us against
// 42-50 us).  Each is taken from the work-groups per CU (in quarters) given
// beside it: 128 x 128 from 1.25 per CU, the half tiles from one per CU (at
// 512 frames, k = 7 conv 20480 x 256 x 1792: 29 us on 320 128 x 128 tiles
// against 37 us on 640 half tiles; transposed conv 512 x 4096 x 2048: 22 us on
// 256 three-buffer half tiles against 27 us on 128 x 128 tiles split in three).
const int H_UNSPLIT[][2] = {{0, 5}, {8, 4}, {9, 4}};
const TileDesc F_TILES[] = {
    {64, 64, 16, "f64x64"}, {128, 32, 16, "f128x32"}, {64, 32, 16, "f64x32"}, {64, 16, 16, "f64x16"},
};
constexpr int NH = sizeof(H_TILES) / sizeof(H_TILES[0]);
constexpr int NF = sizeof(F_TILES) / sizeof(F_TILES[0]);

template <typename T, int BM, int BN, int WM, int WN, int KSUB, bool RU = false, int NBUF = 2,
          int MINW = 1>
hipError_t launch_t(const ConvArgs &a, hipStream_t st)
{
    int ntm = (a.M + BM - 1) / BM, ntn = a.N / BN;
    hipLaunchKernelGGL((conv_gemm_kernel<T, BM, BN, WM, WN, KSUB, RU, NBUF, MINW>),
                       dim3(ntm * ntn, a.splits),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

void set_division(ConvArgs &a)
{
    // m / d == (t + ((m - t) >> s1)) >> s2, t = umulhi(mult, m), for all
    // 32-bit m (round-up reciprocal, l = ceil(log2 d))
    const uint32_t d = (uint32_t)a.rate_in;
    int l = 0;
    while ((1ull << l) < d)
        l++;
    a.div_m = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
    a.div_s1 = l < 1 ? l : 1;
    a.div_s2 = l > 1 ? l - 1 : 0;
}

}  // namespace

// Work-groups of the 128 x 128 tile (and of its 160-row variant) that a CU
// holds at once: two (66 and 74 KB of LDS, at most 256 registers per lane).
// A launch runs in rounds of 2 n_cu work-groups; when the 128-row tiles
// overflow a whole number of rounds by a few work-groups, those few run as
// a round of their own (at 848 frames per step the 128-stream stage-1 k7
// conv has 530 tiles: 52 us against 33 us at 500), so 160-row tiles are
// taken when they fit in the whole rounds (424 tiles: 37 us).  Timed alone:
// stage-1 ConvT / k7 / 1x1 convs at 848 frames 41 / 52 / 29 us -> 32 / 37 /
// 23 us; the stage-2 residual units (one launch each) 78 -> 75 us.
static bool tall_rows(const ConvArgs &a, int n_cu, int bn)
{
    if (!a.tall_allowed || a.N % bn != 0)
        return false;
    const long slots = 2L * n_cu;
    const long wg = (long)((a.M + 127) / 128) * (a.N / bn);
    const long tail = wg % slots;
    const long wg_tall = (long)((a.M + 159) / 160) * (a.N / bn);
    return tail > 0 && 4 * tail <= slots && wg_tall <= wg - tail;
}

// Tile and split count for a launch: the preferred tile that gives at least
// two work-groups per CU; failing that, split K (at least 8 K stages per
// split, partials within the workspace) until the CUs are covered.
ConvPlan conv_gemm_plan(const ConvArgs &a, int dtype, int n_cu, long partial_cap)
{
    // A larger tile reads fewer LDS and L2 bytes per MFMA (a 64 x 64 wave
    // tile half as many as a 32 x 32 one).  First the unsplit candidates
    // (H_UNSPLIT) are tried, then the rule for small problems below; then
    // the tiles largest first, and the first that
    // reaches 1.5 work-groups per CU -- alone, or with K split (>= 8 K stages
    // per split) -- is taken; failing all, the plan with the most work-groups.
    // A short K (at most 16 stages) is not split when a tile covers three
    // quarters of the CUs without it: there the reduce launch costs more than
    // the idle CUs (the 128-stream projection: 7 us unsplit at 64 x 64, 13 us
    // split at 128 x 32).
    const TileDesc *t = dtype ? H_TILES : F_TILES;
    const int n = dtype ? 8 : NF;  // tiles the split search walks, in order
    const int Ktot = a.taps * a.Cin;  // a K stage must not straddle two taps
    const long target = 3L * n_cu / 2;
    if (dtype) {
        for (const auto &u : H_UNSPLIT) {
            const int i = u[0];
            if (a.N % t[i].BN != 0 || a.Cin % t[i].BK != 0 || (t[i].deep && !a.deep_allowed))
                continue;
            if (4L * ((a.M + t[i].BM - 1) / t[i].BM) * (a.N / t[i].BN) >= (long)u[1] * n_cu)
                return ConvPlan{i == TILE_128 && tall_rows(a, n_cu, 128) ? TILE_TALL : i, 1};
        }
        // Little work (at most 32 64 x 64 x 64 tile stages per CU: the layers
        // of steps of a few frames): the 64 x 64 tile, which pads the fewest
        // rows, with K split up to 1.5 work-groups per CU as below, except a
        // K of at most 16 stages, where the reduce launch costs more than it
        // saves.  (Qwen-shaped decoder, one stream decoding one frame per
        // step: 230 us per step against 246 us with the largest tiles split;
        // 8 streams of 8 frames: 245 against 261 us.)
        if (a.N % t[3].BN == 0 && a.Cin % t[3].BK == 0) {
            const long t64 = (long)((a.M + t[3].BM - 1) / t[3].BM) * (a.N / t[3].BN);
            const int nk = Ktot / t[3].BK;
            if (t64 * nk <= 32L * n_cu) {
                int sp = 1;
                if (a.splits_allowed && partial_cap > 0 && nk > 16)
                    while (sp < 32 && t64 * sp < target && nk / (sp + 1) >= 8 &&
                           (long)(sp + 1) * a.M * a.N <= partial_cap)
                        sp++;
                return ConvPlan{3, sp};
            }
        }
    }
    ConvPlan best{-1, 1};
    long best_work = -1;
    int unsplit = -1;  // largest short-K tile reaching 3/4 of the CUs
    // the three-buffer 128 x 64 tile leads the split search (input conv at
    // 512 frames, 512 x 1024 x 7168, in the decode step: 28.2 us split in six
    // against 30.8 us for 128 x 128 split in twelve; at 794 frames no change)
    constexpr int NH = sizeof(H_TILES) / sizeof(H_TILES[0]);
    int order[(NH > NF ? NH : NF) + 1], no = 0;  // n <= max(8, NF) entries + 1
    if (dtype && a.deep_allowed)
        order[no++] = 8;
    for (int i = 0; i < n; i++)
        order[no++] = i;
    for (int oi = 0; oi < no; oi++) {
        const int i = order[oi];
        if (a.N % t[i].BN != 0 || a.Cin % t[i].BK != 0)
            continue;
        const long tiles = (long)((a.M + t[i].BM - 1) / t[i].BM) * (a.N / t[i].BN);
        if (tiles >= target)
            return ConvPlan{dtype && i == TILE_128 && tall_rows(a, n_cu, 128) ? TILE_TALL : i, 1};
        if (tiles > best_work) {
            best_work = tiles;
            best = ConvPlan{i, 1};
        }
        const int nk = Ktot / t[i].BK;
        if (unsplit < 0 && nk <= 16 && 4 * tiles >= 3L * n_cu)
            unsplit = i;
        if (!a.splits_allowed || partial_cap <= 0)
            continue;
        for (int sp = 2; sp <= 32; sp++) {
            if (nk / sp < 8 || (long)sp * a.M * a.N > partial_cap)
                break;
            if (tiles * sp >= target)
                return unsplit >= 0 ? ConvPlan{unsplit, 1} : ConvPlan{i, sp};
            if (tiles * sp > best_work) {
                best_work = tiles * sp;
                best = ConvPlan{i, sp};
            }
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

hipError_t launch_conv_gemm(const ConvArgs &a0, int dtype, hipStream_t st, ConvPlan plan)
{
    if (a0.M <= 0)
        return hipSuccess;
    if (plan.tile < 0)
        return hipErrorInvalidValue;
    ConvArgs a = a0;
    a.splits = plan.splits > 1 ? plan.splits : 1;
    set_division(a);
    hipError_t e = hipErrorInvalidValue;
    if (dtype) {
        switch (plan.tile) {
        case 0: e = launch_t<half_t, 128, 128, 2, 2, 2, false, 2, 2>(a, st); break;
        case 1: e = launch_t<half_t, 128, 64, 2, 2, 2>(a, st); break;
        case 2: e = launch_t<half_t, 64, 128, 2, 2, 2>(a, st); break;
        case 3: e = launch_t<half_t, 64, 64, 2, 2, 2>(a, st); break;
        case 4: e = launch_t<half_t, 256, 32, 4, 1, 1>(a, st); break;
        case 5: e = launch_t<half_t, 128, 32, 4, 1, 1>(a, st); break;
        case 6: e = launch_t<half_t, 32, 64, 2, 2, 1>(a, st); break;
        case 7: e = launch_t<half_t, 64, 32, 4, 1, 1>(a, st); break;
        case 8: e = launch_t<half_t, 128, 64, 2, 2, 2, false, 3>(a, st); break;
        case 9: e = launch_t<half_t, 64, 128, 2, 2, 2, false, 3>(a, st); break;
        case 10: e = launch_t<half_t, 160, 128, 2, 2, 2, false, 2, 2>(a, st); break;
        }
    } else {
        switch (plan.tile) {
        case 0: e = launch_t<float, 64, 64, 2, 2, 1>(a, st); break;
        case 1: e = launch_t<float, 128, 32, 4, 1, 1>(a, st); break;
        case 2: e = launch_t<float, 64, 32, 4, 1, 1>(a, st); break;
        case 3: e = launch_t<float, 64, 16, 4, 1, 1>(a, st); break;
        }
    }
    if (e != hipSuccess || a.splits == 1)
        return e;
    long nq = (long)a.M * (a.N / 4);
    dim3 grid((unsigned)((nq + 255) / 256));
    if (dtype)
        hipLaunchKernelGGL(splitk_reduce_kernel<half_t>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<float>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

bool ru_gemm_supported(int Cout, int dtype)
{
    // 256 channels would need a 64 x 256 tile at one work-group per CU, which
    // is slower than the two separate launches
    return dtype == 1 && Cout == 128;
}

hipError_t launch_ru_gemm(const ConvArgs &a0, int n_cu, hipStream_t st)
{
    if (a0.M <= 0)
        return hipSuccess;
    ConvArgs a = a0;
    a.splits = 1;
    set_division(a);
    if (a.N != a.Cout || a.s != 1 || a.Cin % 64 != 0)
        return hipErrorInvalidValue;
    if (a.Cout != 128)
        return hipErrorInvalidValue;
    // 160-row tiles by the same rule as the plain 128 x 128 tile (81 KB of
    // LDS: two still fit in a CU's 160 KB)
    if (tall_rows(a, n_cu, 128))
        return launch_t<half_t, 160, 128, 2, 2, 2, true, 2, 2>(a, st);
    return launch_t<half_t, 128, 128, 2, 2, 2, true, 2, 2>(a, st);
}

}  // namespace snrvq
