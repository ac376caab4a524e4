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
// conv is fused) and keeps everything between the stage input and output on
// chip: HBM sees the stage's fp16 input rows and its fp16 output rows (or
// the PCM) only.
//
// Arithmetic is the per-layer path's, operation for operation: the same fp16
// operands (each activation applied once, then rounded), the same K order
// (tap-major, channel-minor in steps of 32) on v_mfma_f32_16x16x32_f16 with
// the accumulators starting at the bias, the same fp32 epilogues, so both
// paths give bit-identical PCM.
//
// Work split.  The transposed conv maps input row q to output rows q S + r,
// r < S.  Wave w of a work-group owns q-block w of the tile (16 input rows)
// and with it the S "units" of 16 output rows {(q0 + j) S + r : j < 16}, all
// channels, through all three phases.  So the fp32 residual stream x never
// leaves the wave's registers: the MFMA accumulator layout of a unit (lane =
// row j and 4 consecutive channels) is the same in the transposed conv, both
// residual units and the output epilogue.  Only the activated conv inputs
// go through LDS (the k = 7 convs read neighbouring rows); each 1x1 conv
// takes its operand straight from the k = 7 conv's accumulators, whose
// output channels are ordered for it.  A tile spans 16 NW input rows, HQ of
// them recomputed halo, so every wave has one q-block.
//
// Weights are the MFMA's A operand (16 output channels per block), the
// activations its B operand (16 rows per block); a lane's accumulator holds
// 4 consecutive channels of one row, so every epilogue works on 4 channels
// at once.  With 32 channels the whole stage's weights (64 KiB) stay in LDS
// for the kernel's lifetime.  With 64 channels (229 KiB) the weights stream
// through three LDS buffers in K chunks, loaded cooperatively two chunks
// ahead straight from global memory into LDS; the chunk sequence runs on
// across phases and tiles.
//
// Work-groups are persistent (one per CU) and walk the step's tiles; a
// stream's rows are cut into tiles of T rows, the last one shorter.  The
// first tile of a stream reads the left contexts that the step's halo fill
// wrote into the per-layer path's extended buffers; the last tile writes the
// new left contexts straight into the stream's state slot.
#include "internal.h"

namespace snrvq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mma(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Output channel that A row `row` of channel block n of a k = 7 conv computes:
// blocks 2k and 2k+1 hold channels 32k..32k+31, so that lane lg of both holds
// channels 32k + 8 lg + 0..3 (block 2k) and + 4..7 (block 2k+1).
__device__ __forceinline__ int ch7(int n, int row)
{
    return 32 * (n >> 1) + 8 * (row >> 2) + 4 * (n & 1) + (row & 3);
}

// LDS row of the k = 7 weights of output channel c: 16 n + row for
// c == ch7(n, row), so that the 16 A rows of block n are consecutive in LDS
// (rows 8 apart would share banks) and block n's operand is rows 16 n ..
// 16 n + 15.
__device__ __forceinline__ int w7_row(int c)
{
    return 16 * (2 * (c >> 5) + ((c >> 2) & 1)) + 4 * ((c >> 3) & 3) + (c & 3);
}

// Chunk permutation of unpadded weight rows of 64 bytes (32 halves) and of
// 128 bytes (64 halves): element k of row r sits at k ^ x(r).
__device__ __forceinline__ int x64(int r) { return ((r >> 2) & 1) << 4; }
__device__ __forceinline__ int x128(int r) { return ((r >> 1) & 3) << 4; }
// and of 256-byte rows (128 halves)
__device__ __forceinline__ int x256(int r) { return (r & 7) << 4; }

__device__ __forceinline__ h4 snake4(f4 v, f4 ar, f4 ai)
{
    return h4{snrvq_f16(snrvq_snake(v[0], ar[0], ai[0])),
              snrvq_f16(snrvq_snake(v[1], ar[1], ai[1])),
              snrvq_f16(snrvq_snake(v[2], ar[2], ai[2])),
              snrvq_f16(snrvq_snake(v[3], ar[3], ai[3]))};
}

// fp16 activation rows in LDS, phase-major: row i of a buffer sits in plane
// i mod S at plane row i / S (+1: one spare row in front of every plane), rows
// padded to C + 16 elements.  The MFMA operand of a unit reads rows S apart,
// i.e. consecutive rows of one plane, and a k = 7 tap shifts them by a
// constant: so every operand address is a per-lane base plus a compile-time
// offset.  A 16-byte fragment read is served 16 lanes per cycle (lanes
// 8k..8k+7 with 8k+16..8k+23: 8 rows at two neighbouring 16-byte chunks) over
// 64 four-byte banks; a row stride of 6 (C = 32) or 10 (C = 64) 16-byte slots
// puts those 16 reads on distinct slots of a 256-byte line.
template <int C, int S, int NROWS>
struct Planes {
    static_assert(C == 32 || C == 64, "channels");
    static constexpr int P = C + 16;                      // row pitch, elements
    static constexpr int QR = (NROWS + S - 1) / S + 1;    // rows per plane
    static constexpr int PLANE = QR * P;
    static constexpr int ELEMS = S * PLANE;
    // element offset of channel c of row i >= 0
    __device__ static __forceinline__ int off(int i, int c)
    {
        return (i % S) * PLANE + (i / S + 1) * P + c;
    }
    // lane base of plane row q (rows S q + k are at base(q) + rel(k))
    __device__ static __forceinline__ int base(int q) { return (q + 1) * P; }
    // offset of row S q + k from base(q); k may be negative (down to -S q - S)
    __device__ static constexpr int rel(int k)
    {
        return (((k % S) + S) % S) * PLANE + ((k - (((k % S) + S) % S)) / S) * P;
    }
};

// Per-channel parameter rows in LDS ([P_COUNT][C] fp32).
enum Prm {
    P_BT = 0,                                      // ConvT bias
    P_A1R0, P_A1I0, P_B70, P_A2R0, P_A2I0, P_B10,  // residual unit 0
    P_A1R1, P_A1I1, P_B71, P_A2R1, P_A2I1, P_B11,  // residual unit 1
    P_ANR, P_ANI,                                  // activation of the stage output
    P_COUNT
};

template <int C, int S, int NW, bool FINAL>
struct StageShape {
    static constexpr int E = FINAL ? 6 : 0;          // rows of the final conv's context
    static constexpr int HQ = (24 + E + S - 1) / S;  // input rows of recomputed halo
    static constexpr int HX = HQ * S;                // output rows of recomputed halo
    static constexpr int T = S * (16 * NW - HQ);     // output rows per tile
    static constexpr int O2 = (18 + E + S - 1) / S * S;  // a2 rows before t0 (a multiple of S)
    static constexpr int OO = (6 + S - 1) / S * S;       // final conv input rows before t0
    static constexpr int NA1 = T + HX;                   // a1 rows: [t0 - HX, t0 + T)
    static constexpr int NA2 = T + O2;                   // a2 rows: [t0 - O2, t0 + T)
    static constexpr int NAO = FINAL ? T + OO : 0;       // a_out rows: [t0 - OO, t0 + T)
    static constexpr int NROWS = NA1 > NA2 ? (NA1 > NAO ? NA1 : NAO) : (NA2 > NAO ? NA2 : NAO);
};

// Work-groups per CU: two for the streamed shapes of at most 4 waves (their
// LDS fits twice), so one work-group's VALU phases overlap the other's
// matrix phases and barrier waits; one otherwise.
template <int NW, bool RES>
constexpr int stage_wg_per_cu()
{
    return !RES && NW <= 4 ? 2 : 1;
}

template <int C, int S, int NW, bool FINAL, bool RES>
__global__ __launch_bounds__(NW * 64, (stage_wg_per_cu<NW, RES>())) void stage_kernel(StageArgs p)
{
    using SH = StageShape<C, S, NW, FINAL>;
    using L = Planes<C, S, StageShape<C, S, NW, FINAL>::NROWS>;
    constexpr int NTH = NW * 64;
    constexpr int E = SH::E, HQ = SH::HQ, HX = SH::HX, T = SH::T, O2 = SH::O2, OO = SH::OO;
    constexpr int CIN = 2 * C, NT = S * C, KT = 2 * CIN, NB = C / 16, NKT = KT / 32;
    constexpr int K7 = 7 * C;
    static_assert(T > 0 && C % 32 == 0, "shape");

    // ---- weights: resident copies (RES) or streaming buffers
    // weight rows are read 16 at a time (A operand rows) at two neighbouring
    // chunks per cycle: resident ConvT / conv7 rows padded to a stride of 2
    // mod 16 slots; 64- and 128-byte rows unpadded with their chunks permuted
    // by row (x64 / x128 below)
    static_assert(!RES || C == 32, "resident weights: 32 channels");
    constexpr int LDT = KT + 16, LD7 = K7 + 48, LD1 = C;  // resident pitches
    // streamed (64 channels): ConvT chunks of CTW K columns (64 when three
    // buffers of it fit beside the activations, else 32); per residual unit
    // chunks of TPC conv7 taps, the last one tap 6 with the 1x1 weights.
    // Fewer, larger chunks mean fewer barriers: three taps at stride 3 (its
    // buffers are sized by the ConvT chunk anyway), two at stride 4 (three
    // would fill the LDS and spill registers: 14% slower; one: 6% slower)
    static_assert(RES || C == 64, "streamed weights: 64 channels");
    constexpr int CTW = NT * 64 <= 12288 ? 64 : 32;
    constexpr int TPC = S == 3 ? 3 : 2;
    constexpr int NCT = KT / CTW;         // ConvT chunks
    constexpr int NRC = 6 / TPC + 1;      // chunks per residual unit
    constexpr int NCH = NCT + 2 * NRC;    // chunks per tile (streamed)
    // chunk permutation of the rows of a conv7 chunk (TPC C columns)
    // (rows of 2 C halves: x256; of 3 C: x128, since 384-byte rows already
    // put odd rows half a bank line from even ones)
    auto xtap = [](int r) { return TPC == 2 ? x256(r) : x128(r); };
    constexpr int RES_ELEMS = NT * LDT + 2 * C * LD7 + 2 * C * LD1;
    constexpr int RU_BUF = C * (TPC > 2 ? TPC : 2) * C;  // one residual-unit chunk
    constexpr int CT_BUF = NT * CTW;   // one ConvT chunk
    constexpr int W_BUF = RU_BUF > CT_BUF ? RU_BUF : CT_BUF;

    // One activation buffer holds a1, then a2 (a1 is dead once the first
    // unit's conv7 is done), then a_out (FINAL; a2 is dead once the second
    // unit's conv7 is done).  Streamed weights (ConvT chunks included)
    // rotate through three buffers.
    constexpr int ACT_ELEMS = L::ELEMS;
    constexpr int W_ELEMS = RES ? RES_ELEMS : 3 * W_BUF;

    // Streamed weights arrive by direct global -> LDS loads.  The compiler
    // orders those against LDS reads per LDS variable: with one array it
    // leaves the waits to the kernel, with several it waits for every load in
    // flight before the first LDS read that follows them.  The streamed shapes
    // therefore carve their buffers out of one array (weights last: the
    // activation offsets stay within a DS instruction's offset field); the
    // resident shapes keep one array per buffer.
    constexpr int OFF_PRM = (ACT_ELEMS * 2 + 15) & ~15;
    constexpr int OFF_WOUT = OFF_PRM + P_COUNT * C * 4;
    // the step's tile and frame starts per stream, staged in LDS for steps of
    // up to TAB streams (larger ones search them in global memory)
    constexpr int TAB = 512;
    constexpr int OFF_TAB = OFF_WOUT + (((FINAL ? 7 * C / 2 : 8) * 4 + 15) & ~15);
    constexpr int OFF_W = OFF_TAB + ((2 * (TAB + 1) * 4 + 15) & ~15);
    static_assert(OFF_W % 16 == 0 && OFF_TAB % 16 == 0, "16-byte aligned LDS regions");
    __shared__ __attribute__((aligned(16))) char smem[RES ? 16 : OFF_W + W_ELEMS * 2];
    __shared__ __attribute__((aligned(16))) int tab_r[RES ? 2 * (TAB + 1) : 4];
    __shared__ __attribute__((aligned(16))) half_t acts_r[RES ? ACT_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) half_t wsm_r[RES ? W_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) float prm_r[RES ? P_COUNT * C : 4];
    __shared__ __attribute__((aligned(16))) h2 wout_r[RES && FINAL ? 7 * C / 2 : 8];
    half_t *const acts = RES ? acts_r : (half_t *)smem;
    half_t *const wsm = RES ? wsm_r : (half_t *)(smem + OFF_W);
    float *const prm = RES ? prm_r : (float *)(smem + OFF_PRM);
    int *const tcu_s = RES ? tab_r : (int *)(smem + OFF_TAB);  // tile starts [n_streams + 1]
    int *const cu_s = tcu_s + TAB + 1;                         // frame starts [n_streams + 1]
    const bool tab = p.n_streams <= TAB;
    h2 *const wout_s = RES ? wout_r : (h2 *)(smem + OFF_WOUT);  // final conv weights, fp16 [tap][channel]
    half_t *const a1s = acts, *const a2s = acts;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;

    {
        const float *src[P_COUNT] = {p.bT,      p.al1[0], p.ial1[0], p.b7[0], p.al2[0],
                                     p.ial2[0], p.b1[0],  p.al1[1], p.ial1[1], p.b7[1],
                                     p.al2[1],  p.ial2[1], p.b1[1],  p.al_next, p.ial_next};
        for (int i = tid; i < P_COUNT * C; i += NTH)
            prm[i] = src[i / C][i % C];
        if (tab)
            for (int i = tid; i <= p.n_streams; i += NTH) {
                tcu_s[i] = p.tile_cu[i];
                cu_s[i] = p.cu[i];
            }
    }
    if (FINAL) {
        for (int i = tid; i < 7 * C; i += NTH) {
            const int c = i / 7, j = i - c * 7;  // input layout [C][7]
            ((half_t *)wout_s)[j * C + c] = (half_t)p.w_out[i];
        }
    }
    half_t *const wTs = wsm;
    half_t *const w7s = wsm + NT * LDT;
    half_t *const w1s = w7s + 2 * C * LD7;
    if constexpr (RES) {
        // kind 0: plain rows, 1: conv7 rows (w7_row order), 2: 64-byte rows (x64)
        auto copy = [&](half_t *dst, int ld, const half_t *src, int rows, int cols, int kind) {
            const int cpr = cols / 8;
            for (int i = tid; i < rows * cpr; i += NTH) {
                const int r = i / cpr, c8 = (i - r * cpr) * 8;
                const int o = kind == 1 ? w7_row(r) * ld + c8
                                        : r * ld + (kind == 2 ? c8 ^ x64(r) : c8);
                *(h8 *)(dst + o) = *(const h8 *)(src + (long)r * cols + c8);
            }
        };
        copy(wTs, LDT, p.WT, NT, KT, 0);
        for (int j = 0; j < 2; j++) {
            copy(w7s + j * C * LD7, LD7, p.W7[j], C, K7, 1);
            copy(w1s + j * C * LD1, LD1, p.W1[j], C, C, 2);
        }
    }

    // ---- streamed weights: chunk j of the per-tile sequence
    //   [0, NCT): ConvT K columns [CTW j, CTW (j + 1)) (NT rows)
    //   then per residual unit u, chunk c < NRC - 1: conv7 taps TPC c ..
    //   TPC c + TPC - 1 (C rows in w7_row order, TPC C columns); the last
    //   chunk: tap 6 (C x C, w7_row order) followed by the 1x1 weights (C x C)
    // go global -> LDS directly (16 bytes per lane, no register staging) into
    // three buffers in turn: chunk jc is read from wsm + wcur while chunks
    // jc + 1 and jc + 2 are in flight.  In a wave's instruction i the 64 lanes
    // fill LDS pieces (i NW + wave) 64 .. + 63 (16 bytes each) of the chunk's
    // layout; each lane loads the global piece that belongs there.
    constexpr int CT_P = NT * CTW / 8, RU_P = C * TPC * C / 8, LAST_P = 2 * C * C / 8;
    constexpr int MAXP = CT_P > RU_P ? (CT_P > LAST_P ? CT_P : LAST_P) : (RU_P > LAST_P ? RU_P : LAST_P);
    constexpr int PPW = 64 * NW;  // pieces one instruction of every wave fills
    static_assert(RES || (CT_P % PPW == 0 && RU_P % PPW == 0 && LAST_P % PPW == 0), "pieces");
    constexpr int MAXL = MAXP / PPW;  // load instructions per wave and chunk, at most
    static_assert(RES || MAXL <= 3, "wait_vm below covers up to three loads per chunk");
    auto pieces = [](int jt) {
        return jt < NCT ? CT_P : ((jt - NCT) % NRC == NRC - 1 ? LAST_P : RU_P);
    };
    auto src_of = [&](int jt, int u) -> const half_t * {
        if (jt < NCT) {
            constexpr int ppr = CTW / 8;
            const int row = u / ppr, c8 = ((u % ppr) * 8) ^ (CTW == 64 ? x128(row) : x64(row));
            return p.WT + (long)row * KT + jt * CTW + c8;
        }
        const int unit = (jt - NCT) / NRC, c = (jt - NCT) % NRC;
        if (c < NRC - 1) {
            constexpr int ppr = TPC * C / 8;
            const int lr = u / ppr, c8 = ((u % ppr) * 8) ^ xtap(lr);
            return p.W7[unit] + (long)ch7(lr >> 4, lr & 15) * K7 + TPC * c * C + c8;
        }
        constexpr int ppr = C / 8, HALF = C * C / 8;
        if (u < HALF) {  // tap 6, rows in w7_row order
            const int lr = u / ppr, c8 = ((u % ppr) * 8) ^ x128(lr);
            return p.W7[unit] + (long)ch7(lr >> 4, lr & 15) * K7 + 6 * C + c8;
        }
        const int v = u - HALF, row = v / ppr, c8 = ((v % ppr) * 8) ^ x128(row);
        return p.W1[unit] + (long)row * C + c8;
    };
    auto dload = [&](int j, int off) {
        const int jt = j % NCH, np = pieces(jt);
#pragma unroll
        for (int i = 0; i < MAXL; i++)
            if (i * PPW < np) {
                const int blk = i * NW + wave;
                __builtin_amdgcn_global_load_lds(
                    (const void __attribute__((address_space(1))) *)src_of(jt, blk * 64 + lane),
                    (void __attribute__((address_space(3))) *)(wsm + off + blk * 512), 16, 0, 0);
            }
    };
    // wait until at most n (1 .. 3) vector memory operations are outstanding
    auto wait_vm = [](int n) {
        if (n <= 1)
            __builtin_amdgcn_s_waitcnt(0x3f71);
        else if (n == 2)
            __builtin_amdgcn_s_waitcnt(0x3f72);
        else
            __builtin_amdgcn_s_waitcnt(0x3f73);
    };
    // this thread is done with chunk jc: the loads of chunk jc + 2 start (into
    // the buffer of chunk jc - 1, free since the last barrier), chunk jc + 1
    // must have landed (its loads are older than jc + 2's), then the barrier
    int jc = 0, wcur = 0, wnext2 = 2 * W_BUF;
    auto rot3 = [](int o) { return o + W_BUF == 3 * W_BUF ? 0 : o + W_BUF; };
    auto lds_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
        __asm__ volatile("s_barrier" ::: "memory");
    };
    auto advance = [&]() {
        if constexpr (!RES) {
            dload(jc + 2, wnext2);
            wait_vm(pieces((jc + 2) % NCH) / PPW);
            lds_barrier();
            wcur = rot3(wcur);
            wnext2 = rot3(wnext2);
            jc++;
        } else {
            __syncthreads();
        }
    };

    if constexpr (!RES) {
        dload(0, 0);
        dload(1, W_BUF);
    }
    __syncthreads();  // parameters and weights are in LDS (chunk 1 landed too)

    const int n_tiles = p.tile_cu[p.n_streams];
    for (int g = blockIdx.x; g < n_tiles; g += gridDim.x) {
        // stream of tile g: the largest b with tile_cu[b] <= g.  From the LDS
        // table: tile starts rise with b (every stream has a tile), so b + 1
        // is the number of starts <= g, counted 64 at a time with a ballot
        // (128-stream steps: 4-6 us less per fused-stage launch than the
        // binary search's chain of dependent global loads)
        int b, cu0, cu1, tc0;
        if (tab) {
            int base = 0, c = 64;
            while (c == 64) {
                const int i = base + lane;
                const int v = tcu_s[i < p.n_streams ? i : p.n_streams];
                c = __popcll(__builtin_amdgcn_ballot_w64(i <= p.n_streams && v <= g));
                base += 64;
            }
            b = __builtin_amdgcn_readfirstlane(base - 64 + c - 1);
            cu0 = __builtin_amdgcn_readfirstlane(cu_s[b]);
            cu1 = __builtin_amdgcn_readfirstlane(cu_s[b + 1]);
            tc0 = __builtin_amdgcn_readfirstlane(tcu_s[b]);
        } else {
            int lo = 0, hi = p.n_streams;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (p.tile_cu[mid] <= g)
                    lo = mid;
                else
                    hi = mid;
            }
            b = lo;
            cu0 = p.cu[b];
            cu1 = p.cu[b + 1];
            tc0 = p.tile_cu[b];
        }
        const int rows_b = (cu1 - cu0) * p.r_out;
        const int t0 = (g - tc0) * T;
        const int tend = t0 + T < rows_b ? t0 + T : rows_b;  // rows [t0, tend)
        const bool first = t0 == 0, last = tend == rows_b;
        half_t *slot_state = p.state + (long)p.slot[b] * p.slot_elems;
        const int r1 = t0 - HX;  // stream row of a1 row 0
        const int r2 = t0 - O2;  // stream row of a2 row 0 (r1, r2: multiples of S)

        // ---- phase 1: transposed conv of this wave's 16 input rows
        const int q0 = t0 / S;
        const int qlo = first ? 0 : q0 - HQ;
        const int qhi = tend / S;
        int q = qlo + wave * 16 + l16;
        const bool qok = q < qhi;
        q = qok ? q : qhi - 1;
        f4 x[S][NB];  // the residual stream of this wave's units
        {
            const half_t *x1 = p.aT + ((long)(b + 1) + (long)cu0 * p.r_in + q) * CIN + lg * 8;
            const half_t *x0 = x1 - CIN;
            h8 xf[NKT];
#pragma unroll
            for (int ks = 0; ks < NKT; ks++) {
                const int k0 = ks * 32, tap = k0 / CIN, c0 = k0 - tap * CIN;
                xf[ks] = *(const h8 *)((tap ? x1 : x0) + c0);
            }
#pragma unroll
            for (int n = 0; n < NB; n++) {
                const f4 bt = *(const f4 *)(prm + P_BT * C + n * 16 + lg * 4);
#pragma unroll
                for (int r = 0; r < S; r++)
                    x[r][n] = bt;  // accumulators start at the bias
            }
#pragma unroll
            for (int ks = 0; ks < NKT; ks++) {
                // streamed: K step ks is columns (32 ks) mod CTW of chunk 32 ks / CTW
                const half_t *wp = RES ? wTs + ks * 32 : wsm + wcur;
                const int wld = RES ? LDT : CTW;
                const int wk = RES ? lg * 8
                                   : ((ks * 32) % CTW + lg * 8) ^ (CTW == 64 ? x128(l16) : x64(l16));
#pragma unroll
                for (int r = 0; r < S; r++)
#pragma unroll
                    for (int n = 0; n < NB; n++) {
                        const h8 wf = *(const h8 *)(wp + (r * C + n * 16 + l16) * wld + wk);
                        x[r][n] = mma(wf, xf[ks], x[r][n]);
                    }
                if (!RES && (ks + 1) * 32 % CTW == 0 && ks + 1 < NKT)
                    advance();
            }
            // epilogue: + bias -> x; Snake -> a1
            const int b1 = L::base(q - r1 / S) + lg * 4;  // a1 rows S q + r
#pragma unroll
            for (int r = 0; r < S; r++) {
#pragma unroll
                for (int n = 0; n < NB; n++) {
                    const int c = n * 16 + lg * 4;
                    if (qok)
                        *(h4 *)(a1s + b1 + L::rel(r) + n * 16) =
                            snake4(x[r][n], *(const f4 *)(prm + P_A1R0 * C + c),
                                   *(const f4 *)(prm + P_A1I0 * C + c));
                }
            }
            // left context of a stream's first tile (written by the halo fill)
            if (first) {
                const half_t *s1 = p.a1_ext + ((long)b * 6 + (long)cu0 * p.r_out) * C;
                for (int k = tid; k < 6 * C / 8; k += NTH) {
                    const int r = k / (C / 8), c8 = (k - r * (C / 8)) * 8;
                    *(h8 *)(a1s + L::off(HX - 6 + r, c8)) = *(const h8 *)(s1 + r * C + c8);
                }
            }
            advance();  // a1 complete, ConvT chunks no longer read
        }

        // ---- phases 2 and 3: the residual units on this wave's units
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int D = u ? 3 : 1;
            const half_t *in = u ? a2s : a1s;
            const int rin = u ? r2 : r1;
            const int rlo = first ? 0 : (u ? t0 - E : t0 - 18 - E);  // rows computed
            if (last) {  // new left context of this unit's conv7: the last 6 D rows of its input
                half_t *d = slot_state + (u ? p.off_a2 : p.off_a1);
                const int nr = 6 * D;
                for (int k = tid; k < nr * C / 8; k += NTH) {
                    const int r = k / (C / 8), c8 = (k - r * (C / 8)) * 8;
                    *(h8 *)(d + r * C + c8) = *(const h8 *)(in + L::off(tend - nr - rin + r, c8));
                }
            }
            bool rok[S];  // unit r's row of this lane is computed and kept
#pragma unroll
            for (int r = 0; r < S; r++) {
                const int t = q * S + r;
                rok[r] = qok && t >= rlo && t < tend;
            }
            // lane base of the input rows S qi + r.  Lanes with a kept row
            // have qi >= 6 D / S; the others are clamped there, so every row
            // they read lies at most one row before a plane, on its spare row.
            int qi = q - rin / S;
            qi = qi < 6 * D / S ? 6 * D / S : qi;
            const int bin = L::base(qi) + lg * 8;
            const int PB7 = u ? P_B71 : P_B70, PA2R = u ? P_A2R1 : P_A2R0,
                      PA2I = u ? P_A2I1 : P_A2I0, PB1 = u ? P_B11 : P_B10;
            f4 acc[S][NB];
#pragma unroll
            for (int n = 0; n < NB; n++) {
                const f4 b7 = *(const f4 *)(prm + PB7 * C + ch7(n, 4 * lg));
#pragma unroll
                for (int r = 0; r < S; r++)
                    acc[r][n] = b7;  // accumulators start at the bias
            }
            // one K step of 32 of the conv7 (dilation D) from weights wp (row
            // pitch wld, lane element wk); block n, A row l16 computes output
            // channel ch7(n, l16) (LDS row 16 n + l16); ro: offset of each
            // unit's input row for this step's tap from the lane base
            auto step7 = [&](int c0, const half_t *wp, int wld, int wk, const int (&ro)[S]) {
                h8 wf[NB];
#pragma unroll
                for (int n = 0; n < NB; n++)
                    wf[n] = *(const h8 *)(wp + (16 * n + l16) * wld + wk);
#pragma unroll
                for (int r = 0; r < S; r++) {
                    const h8 xf = *(const h8 *)(in + bin + ro[r] + c0);
#pragma unroll
                    for (int n = 0; n < NB; n++)
                        acc[r][n] = mma(wf[n], xf, acc[r][n]);
                }
            };
            auto tap_offsets = [&](int tap, int (&ro)[S]) {
#pragma unroll
                for (int r = 0; r < S; r++)
                    ro[r] = L::rel(r + (tap - 6) * D);
            };
            if constexpr (RES) {
#pragma unroll
                for (int tap = 0; tap < 7; tap++) {
                    int ro[S];
                    tap_offsets(tap, ro);
#pragma unroll
                    for (int c0 = 0; c0 < C; c0 += 32)
                        step7(c0, w7s + u * C * LD7 + tap * C + c0, LD7, lg * 8, ro);
                }
            } else {
#pragma unroll 1
                for (int c = 0; c < NRC - 1; c++) {  // taps TPC c .. TPC c + TPC - 1
                    const half_t *wb = wsm + wcur;
#pragma unroll 1
                    for (int t2 = 0; t2 < TPC; t2++) {
                        int ro[S];
                        tap_offsets(TPC * c + t2, ro);
#pragma unroll
                        for (int kin = 0; kin < C; kin += 32)
                            step7(kin, wb, TPC * C, (t2 * C + kin + lg * 8) ^ xtap(l16), ro);
                    }
                    advance();
                }
                // tap 6: first half of the unit's last chunk
                const half_t *wb = wsm + wcur;
                int ro[S];
                tap_offsets(6, ro);
#pragma unroll
                for (int kin = 0; kin < C; kin += 32)
                    step7(kin, wb, C, (kin + lg * 8) ^ x128(l16), ro);
            }
            // the unit's input is dead from here on: its rows take the next
            // activation, whose left context a stream's first tile reads from
            // the halo fill's buffers
            if constexpr (RES)
                __syncthreads();
            else
                lds_barrier();  // not waiting for the weight loads in flight
            if (first && (u == 0 || FINAL)) {
                const half_t *sx = u == 0 ? p.a2_ext + ((long)b * 18 + (long)cu0 * p.r_out) * C
                                          : p.ao_ext + ((long)b * 6 + (long)cu0 * p.r_out) * C;
                const int nr = u == 0 ? 18 : 6, r0 = u == 0 ? O2 - 18 : OO - 6;
                for (int k = tid; k < nr * C / 8; k += NTH) {
                    const int r = k / (C / 8), c8 = (k - r * (C / 8)) * 8;
                    *(h8 *)(acts + L::off(r0 + r, c8)) = *(const h8 *)(sx + r * C + c8);
                }
            }
            // per unit: Snake(conv7 + b7) -> 1x1 conv -> + b1 + x.  The lane's conv7
            // accumulators of blocks 2k, 2k+1 hold channels 32k + 8 lg + 0..7 of
            // its row: exactly its B operand of the 1x1 conv's K step k.
            const half_t *w1p = RES ? w1s + u * C * LD1 : wsm + wcur + C * C;
            const int w1ld = RES ? LD1 : C;
#pragma unroll
            for (int r = 0; r < S; r++) {
                h8 hb[NB / 2];
#pragma unroll
                for (int n = 0; n < NB; n++) {
                    const int c = ch7(n, 4 * lg);
                    const h4 hv = snake4(acc[r][n], *(const f4 *)(prm + PA2R * C + c),
                                         *(const f4 *)(prm + PA2I * C + c));
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        hb[n >> 1][(n & 1) * 4 + e] = hv[e];
                }
                f4 y[NB];
#pragma unroll
                for (int n = 0; n < NB; n++)
                    y[n] = *(const f4 *)(prm + PB1 * C + n * 16 + lg * 4);  // starts at the bias
#pragma unroll
                for (int kk = 0; kk < NB / 2; kk++) {
#pragma unroll
                    for (int n = 0; n < NB; n++) {
                        const h8 wf =
                            *(const h8 *)(w1p + (n * 16 + l16) * w1ld +
                                          ((kk * 32 + lg * 8) ^ (RES ? x64(l16) : x128(l16))));
                        y[n] = mma(wf, hb[kk], y[n]);
                    }
                }
                const int t = q * S + r;
                // a2 row t - r2 / a_out row t - (t0 - OO): plane row q - r2 / S
                // or q - (t0 - OO) / S, plane r
                const int bo = L::base(q - (u == 0 ? r2 : t0 - OO) / S) + L::rel(r) + lg * 4;
#pragma unroll
                for (int n = 0; n < NB; n++) {
                    const int c = n * 16 + lg * 4;
                    x[r][n] = y[n] + x[r][n];
                    if (!rok[r])
                        continue;
                    if (u == 0) {
                        *(h4 *)(a2s + bo + n * 16) =
                            snake4(x[r][n], *(const f4 *)(prm + P_A1R1 * C + c),
                                   *(const f4 *)(prm + P_A1I1 * C + c));
                    } else {
                        const h4 o = snake4(x[r][n], *(const f4 *)(prm + P_ANR * C + c),
                                            *(const f4 *)(prm + P_ANI * C + c));
                        if (FINAL)
                            *(h4 *)(a1s + bo + n * 16) = o;
                        else
                            *(h4 *)(p.next + ((long)(b + 1) + (long)cu0 * p.r_out + t) * C +
                                    c) = o;
                    }
                }
            }
            advance();  // a2 complete (u = 0) / a_out complete (u = 1)
        }

        if (FINAL) {
            if (last) {  // new left context of the final conv: the last 6 rows of a_out
                half_t *d = slot_state + p.off_ao;
                for (int k = tid; k < 6 * C / 8; k += NTH) {
                    const int r = k / (C / 8), c8 = (k - r * (C / 8)) * 8;
                    *(h8 *)(d + r * C + c8) =
                        *(const h8 *)(a1s + L::off(tend - 6 - (t0 - OO) + r, c8));
                }
            }
            // ---- phase 4: final conv on the matrix cores.  A block is 16
            // samples of one phase ph, S apart: tt = S (16 qb + l16) + ph, so
            // its tap-j rows are consecutive rows of one plane.  A row 0 holds
            // the weights of one (tap, 32 channels) K step, the other rows
            // zeros; K steps tap-major (the per-layer final conv's sequence).
            // All S phases of a block run together: the input row of (phase
            // ph, tap j) is ph + j rows on from the block's first, so the
            // (ph, j) pairs with equal ph + j share one operand read (the S
            // phases x 7 taps read S + 6 operands, not 7 S).  Each output
            // keeps the tap-major K sequence.
            const int nsamp = tend - t0;
            const h8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
            const int nqb = (nsamp + 16 * S - 1) / (16 * S);  // blocks per phase
            // lanes past the tile's last sample read the rows of the last
            // plane row that has one (still below the buffer's NROWS rows:
            // at most nsamp - 2 + S + OO), and store nothing
            const int qmax = (nsamp - 1) / S;
            for (int qb = wave; qb < nqb; qb += NW) {
                const int qq = 16 * qb + l16;
                const int bq = L::base(qq < qmax ? qq : qmax) + lg * 8;
                f4 acc[S];
#pragma unroll
                for (int ph = 0; ph < S; ph++)
                    acc[ph] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 7; j++) {
#pragma unroll
                    for (int k0 = 0; k0 < C; k0 += 32) {
                        const h8 wf = *(const h8 *)((const half_t *)wout_s + j * C + k0 + lg * 8);
                        const h8 wa = l16 == 0 ? wf : zero;
#pragma unroll
                        for (int ph = 0; ph < S; ph++)  // a_out row of sample tt, tap j: tt + j + OO - 6
                            acc[ph] = mma(wa, *(const h8 *)(a1s + bq + L::rel(ph + j + OO - 6) + k0),
                                          acc[ph]);
                    }
                }
                if (lg == 0) {
#pragma unroll
                    for (int ph = 0; ph < S; ph++) {
                        if (S * qq + ph < nsamp) {
                            const float yv = p.b_out + acc[ph][0];
                            p.pcm[(long)cu0 * p.r_out + t0 + S * qq + ph] =
                                p.final_tanh ? tanhf(yv) : yv;
                        }
                    }
                }
            }
            __syncthreads();  // a_out is read before the next tile writes a1
        }
    }  // tile loop
    if constexpr (!RES)
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): no load into LDS outlives the work-group

    // The last stage's work-groups also save the per-layer halos of the step
    // (every earlier layer's output is final by now; this kernel neither
    // reads those buffers' last rows nor writes their slot regions), so the
    // step needs no separate save launch and the work fills the tail left
    // by the last round of tiles.
    if constexpr (FINAL) {
        const int jobs = p.save.n * p.n_streams;
        for (int j = blockIdx.x; j < jobs; j += gridDim.x)
            halo_save_one(p.save, j / p.n_streams, j % p.n_streams, (char *)p.state, p.cu,
                          p.slot, tid, NTH);
    }
}

template <int C, int S, int NW, bool FINAL, bool RES>
hipError_t launch_stage_t(const StageArgs &a, hipStream_t st)
{
    const int slots = a.n_cu * stage_wg_per_cu<NW, RES>();
    const int grid = a.n_tiles < slots ? a.n_tiles : slots;
    if (grid <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((stage_kernel<C, S, NW, FINAL, RES>), dim3(grid), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

#ifndef NW_Q3
#define NW_Q3 8
#endif
#ifndef NW_Q4
#define NW_Q4 12
#endif
// instantiated shapes
struct StageInst {
    int C, S, NW;
    bool final_stage, res;
};
constexpr StageInst INSTS[] = {
    {64, 3, NW_Q3, false, false},  // Qwen-shaped stage 3, weights streamed
    {32, 4, NW_Q4, true, true},    // Qwen-shaped stage 4 + final conv, weights resident
    {64, 4, 8, false, false},  // Fish-shaped stage 3, weights streamed
    {32, 2, 16, true, true},   // Fish-shaped stage 4 + final conv, weights resident
};

constexpr int tile_rows(const StageInst &s)
{
    return s.S * (16 * s.NW - (24 + (s.final_stage ? 6 : 0) + s.S - 1) / s.S);
}

}  // namespace

int stage_fused_tile(int C, int S, bool final_stage)
{
    for (const StageInst &s : INSTS)
        if (s.C == C && s.S == S && s.final_stage == final_stage)
            return tile_rows(s);
    return 0;
}

hipError_t launch_stage_fused(const StageArgs &a, int C, int S, int T, bool final_stage,
                              hipStream_t st)
{
    if (C == 64 && S == 3 && !final_stage && T == tile_rows(INSTS[0]))
        return launch_stage_t<64, 3, NW_Q3, false, false>(a, st);
    if (C == 32 && S == 4 && final_stage && T == tile_rows(INSTS[1]))
        return launch_stage_t<32, 4, NW_Q4, true, true>(a, st);
    if (C == 64 && S == 4 && !final_stage && T == tile_rows(INSTS[2]))
        return launch_stage_t<64, 4, 8, false, false>(a, st);
    if (C == 32 && S == 2 && final_stage && T == tile_rows(INSTS[3]))
        return launch_stage_t<32, 2, 16, true, true>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace snrvq
