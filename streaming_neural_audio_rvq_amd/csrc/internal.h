// internal.h -- declarations shared by the library's host code and kernels.
//
// Activation layout.  Every activation is channels-last (one row per sample,
// C contiguous values).  Rows of all streams in a step are packed stream
// after stream ("packed rows"); at a layer running at r rows per frame,
// stream b owns packed rows [cu[b] r, cu[b+1] r).  A conv input buffer that
// needs left context is "extended": each stream's rows are preceded by H
// halo rows, so packed row m of stream b sits at extended row (b+1) H + m,
// and its halo rows are b H + cu[b] r .. + H.  The halo is filled from the
// stream's state slot before the step and the last H rows of every stream's
// extended segment are saved back after it, which also handles n r < H.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "snrvq.h"

namespace snrvq {

typedef _Float16 half_t;

enum Act : int { ACT_NONE = 0, ACT_SNAKE = 1, ACT_ELU = 2, ACT_GELU = 3 };

// Snake, applied once per element in fp32: v + sin^2(alpha v) / alpha.
// alpha_rev = alpha / 2pi (precomputed per channel), so alpha v in
// revolutions is one multiply; its fractional part is fed to the hardware
// sine, which takes revolutions.  Every Snake evaluation of the
// library goes through this one function, so fused and per-layer paths
// round identically.
// The rounding steps are spelled out (no contraction) so that every caller
// gets the same bits whatever the compiler does around it.
__device__ __forceinline__ float snrvq_snake(float v, float alpha_rev, float inv_alpha)
{
#pragma clang fp contract(off)
    const float r = __builtin_amdgcn_fractf(alpha_rev * v);  // exact reduction to [0, 1)
    const float s = __builtin_amdgcn_sinf(r);
    const float s2 = s * s;
    return __builtin_fmaf(s2, inv_alpha, v);
}
__device__ __forceinline__ float snrvq_elu(float v) { return v > 0.f ? v : expm1f(v); }

// fp32 -> fp16 (round to nearest even) of a materialized fp32 value.  The
// empty asm keeps the compiler from folding the conversion into the FMA that
// produced x (v_fma_mixlo_f16 rounds once, straight to fp16), so every
// kernel rounds the same way: to fp32 first, then to fp16.
__device__ __forceinline__ half_t snrvq_f16(float x)
{
    __asm__("" : "+v"(x));
    return (half_t)x;
}

// One implicit-GEMM convolution (also transposed conv in polyphase form,
// and plain GEMMs as k = 1 convs).
//   out[m, n] = bias[n % Cout] + sum_{tap, c} A_ext[row(m) - (taps-1-tap) dil, c] * Wt[n, tap Cin + c]
// where row(m) is the extended row of packed input row m.  For a transposed
// conv of stride s the output row of (m, n) is m s + n / Cout, channel n % Cout.
struct ConvArgs {
    const void *A;          // input, compute type, extended with A_H halo rows per stream
    const void *Wt;         // packed weights [N][taps Cin], compute type
    const float *bias;      // [Cout]
    const int32_t *frame_stream;  // [F] batch index of each packed frame
    const float *res;       // fp32 residual [M][Cout] (s == 1) or null
    float *out32;           // fp32 output [M s][Cout] or null
    void *out16;            // compute-type output, extended with out_H halo rows, or null
    const float *alpha;     // [Cout] activation parameter for out16
    const float *inv_alpha; // [Cout]
    int M;                  // packed input rows = F * rate_in
    int A_H, Cin, taps, dil, rate_in;
    int N, Cout, s;
    int out_H, act;
    int out_ld;             // row width of out16 / out32 (== Cout)
    uint32_t div_m;         // packed row -> frame: m / rate_in as a multiply-shift
    int div_s1, div_s2;     //   (set by the launcher)
    int splits;             // split-K count (set by the launcher)
    int splits_allowed;     // 1: the planner may split K
    int deep_allowed;       // 1: the planner may take the three-buffer tiles
    int tall_allowed;       // 1: the planner may take the 160-row tiles
    float *partial;         // split-K partials [splits][M][N] fp32
    // residual unit in one launch (k = 7 conv -> act7 -> 1x1 conv -> epilogue):
    // A, Wt describe the k = 7 conv, bias and everything after it the 1x1
    // conv's output side
    const void *W1;         // [Cout][Cout] 1x1 weights
    const float *bias7;     // [Cout] k = 7 conv bias
    const float *alpha7, *inv_alpha7;  // [Cout] activation between the convs
    int act7;
};

// Tile choice and split-K count of one conv launch.
struct ConvPlan {
    int tile, splits;
};

// Halo layers: fill before a step, save after it.
#define SNRVQ_MAX_HALO 24
struct HaloLayer {
    void *ext;        // extended buffer (compute type)
    int64_t state_off;// element offset of this layer inside one slot
    int H, C, rate, pad;
};
struct HaloTable {
    HaloLayer l[SNRVQ_MAX_HALO];
    int n;
    int elem_bytes;
    int64_t slot_elems;
};

// Saves the last H rows of stream b's extended segment of halo layer `layer`
// (they start at extended row b H + cu[b+1] rate) into its slot; threads
// tid of nthreads share the copy.
__device__ __forceinline__ void halo_save_one(const HaloTable &t, int layer, int b, char *state,
                                              const int32_t *cu, const int32_t *slot, int tid,
                                              int nthreads)
{
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const HaloLayer &L = t.l[layer];
    const long row_bytes = (long)L.C * t.elem_bytes;
    const long bytes = (long)L.H * row_bytes;
    const char *src = (const char *)L.ext + ((long)b * L.H + (long)cu[b + 1] * L.rate) * row_bytes;
    char *dst = state + ((long)slot[b] * t.slot_elems + L.state_off) * t.elem_bytes;
    for (long i = (long)tid * 16; i < bytes; i += (long)nthreads * 16)
        *(u4v *)(dst + i) = *(const u4v *)(src + i);
}

// Per-step device metadata (one H2D copy).
struct StepMeta {
    int32_t *codes;        // [F][K]
    int32_t *frame_stream; // [F]
    int32_t *cu;           // [B+1]
    int32_t *slot;         // [B]
    int32_t *fresh;        // [B]
    int32_t *pos;          // [B]
    int32_t *tile_cu[CODEC_MAX_STAGES];  // fused stage i: first tile of each stream [B+1]
    int32_t *attn_q;                      // attention query blocks, SNRVQ_ATTN_Q_INTS each (see AttnArgs)
    int B;                                // streams in the step
    int n_tiles[CODEC_MAX_STAGES];        // fused stage i: tiles in the step
    int n_qblocks;                        // attention query blocks (a bound for graphs)
};

// ---- launchers (kernels_*.hip) ----
// dtype: 0 = fp32 operands, 1 = fp16 operands
hipError_t launch_conv_gemm(const ConvArgs &a, int dtype, hipStream_t st, ConvPlan plan);
ConvPlan conv_gemm_plan(const ConvArgs &a, int dtype, int n_cu, long partial_cap);
// One residual unit x + conv1x1(act7(conv7(a))) with its epilogue, fp16
// operands; ru_gemm_supported says for which widths it runs.
bool ru_gemm_supported(int Cout, int dtype);
hipError_t launch_ru_gemm(const ConvArgs &a, int n_cu, hipStream_t st);
const char *conv_gemm_tile_name(int dtype, int tile);

hipError_t launch_halo_save(const HaloTable &t, void *state, const StepMeta &m, int B,
                            hipStream_t st);

// z[f][0, d_cb) = sum_k cb[k][codes[f][k]][:] (cb is one [K][E][d_cb] array),
// written in the compute type as rows of out_ld values: with `one`, value
// d_cb is 1 and the rest of the row zero (the constant input of a folded
// input conv).  out_H > 0 writes the rows into an extended buffer with out_H
// halo rows per stream.  cb_dtype: 0 fp32 tables, 1 bf16 tables.  out_dtype:
// 0 fp32, 1 fp16.  Codes outside [0, E) are counted in *bad and read as 0.
// The same launch fills the halo rows of every layer of table t from the
// streams' slots (zeros for fresh streams): the two are independent.
hipError_t launch_rvq_gather_fill(const void *cb, int cb_dtype, const int32_t *codes, int F,
                                  int K, int E, int d_cb, int out_ld, int out_H, int one, void *z,
                                  int out_dtype, unsigned long long *bad, const HaloTable &t,
                                  void *state, const StepMeta &m, int B, hipStream_t st);

// pcm[m] = b + sum_{j, c} w[c][j] A_ext[row(m) - (6 - j), c], m < M (k = 7, Cout = 1).
hipError_t launch_final_conv(const void *A, int dtype, int A_H, int C, int rate,
                             const float *w /*[C][7]*/, float b, int final_tanh,
                             const int32_t *frame_stream, int M, float *pcm, hipStream_t st);

// Copies the first C values of packed rows out of an extended buffer (rows
// of ld values, H halo rows per stream) as fp32 [M][C].
hipError_t launch_unextend(const void *ext, int dtype, int H, int ld, int C, int rate,
                           const int32_t *frame_stream, int M, float *dst, hipStream_t st);

// ---- fused upsample stage (kernels_stage.hip), fp16 operands only ----
struct StageArgs {
    const half_t *aT;                 // ConvT input, extended with 1 halo row, width 2C
    const half_t *WT;                 // polyphase ConvT weights [S C][2 * 2C]
    const float *bT;                  // [C]
    const half_t *W7[2], *W1[2];      // residual units: [C][7C], [C][C]
    const float *b7[2], *b1[2];
    const float *al1[2], *ial1[2];    // activation of each residual unit's input
    const float *al2[2], *ial2[2];    // activation inside each residual unit
    const float *al_next, *ial_next;  // activation of the stage output
    const half_t *a1_ext, *a2_ext, *ao_ext;  // halo sources (extended, H = 6, 18, 6)
    half_t *next;                     // next stage's ConvT input (extended, 1 halo row)
    float *pcm;                       // final stage: PCM [F hop]
    const float *w_out;               // final conv [C][7]
    float b_out;
    int final_tanh;
    half_t *state;                    // slot array, slot_elems per slot
    long slot_elems, off_a1, off_a2, off_ao;
    const int32_t *frame_stream, *cu, *slot;
    const int32_t *tile_cu;           // [n_streams + 1]: stream b's tiles start at tile_cu[b]
    int n_streams, n_tiles;
    int r_in, r_out, act;
    int n_cu;                         // compute units of the device
    HaloTable save;                   // last stage: the per-layer halos its work-groups save
                                      // once their tiles are done (n = 0: none)
};
// Output rows per tile of an instantiated fused stage, or 0 when the shape
// has none (then the per-layer path runs).  A stream's rows are cut into
// tiles of that many rows, the last one shorter.
int stage_fused_tile(int C, int S, bool final_stage);
hipError_t launch_stage_fused(const StageArgs &a, int C, int S, int T, bool final_stage,
                              hipStream_t st);

// ---- transformer ops (kernels_tf.hip) ----
#define SNRVQ_MAX_WINDOW 32  // keys per query, including its own frame
#define SNRVQ_ATTN_QB 16     // frames of one stream per attention work-group
#define SNRVQ_ATTN_Q_INTS 8  // per query block: first frame, frames (0: none), position of
                             // the first frame, of the stream's first frame of the step, slot
struct AttnArgs {
    float *qkv;               // [F][3 dm] fp32, bias included (q, k not rotated)
    const float *rot;         // [F][hd/2][2] cos, sin of each frame's rotary angles
    void *att;                // [F][dm] compute type
    float *kring, *vring;     // [slots][layers][W-1][dm] fp32; K rotated
    const int32_t *frame_stream, *cu, *slot, *pos;
    const int32_t *attn_q;    // [n_qblocks][SNRVQ_ATTN_Q_INTS] query blocks of the step
    int F, H, hd, W, layer, n_layers;
    int n_qblocks;            // query blocks launched
    int dtype;
};
// y[f] = LN(x[f]) in the compute type (x fp32 [F][D], D % 64 == 0).  With
// ring != nullptr the same launch also appends the layer's K (rotated) and V
// rows of each stream's last min(n_b, W-1) frames to the K/V ring (ring->
// layer); the caller orders it after that layer's attention.
hipError_t launch_layer_norm(const float *x, const float *g, const float *b, int F, int D,
                             void *y, int dtype, hipStream_t st,
                             const AttnArgs *ring = nullptr);
// rot[f][i] = (cos, sin) of pos(f) inv_freq[i], i < hd / 2 (the angle in
// fp64, reduced, then both rounded to fp32): the rotary table of the step's
// frames, applied to q and k inside the attention and the ring append.
hipError_t launch_rope_table(float *rot, const double *inv_freq, const int32_t *frame_stream,
                             const int32_t *cu, const int32_t *pos, int F, int hd,
                             hipStream_t st);
hipError_t launch_window_attention(const AttnArgs &a, hipStream_t st);

}  // namespace snrvq
