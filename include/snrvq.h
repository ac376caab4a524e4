/*
 * snrvq.h -- C ABI of the MI355X (gfx950) streaming RVQ codec decoder.
 *
 * The library is stage 1 of a two-stage TTS pipeline: it turns batched
 * per-stream multi-codebook RVQ frames into PCM.  Each stream keeps its
 * causal-conv left context (and, for configurations with one, its windowed
 * transformer's K/V), every call decodes only the new frames, and the
 * concatenated output of a stream equals the decode of its whole utterance
 * (AREX article on vLLM-Omni / Fish Audio Drama 3, section "two stages share
 * one card: one forward per frame, stateful streaming decode").
 *
 * Codes arrive as [T, Q] frames of Q codebook indices (AI-infra handbook,
 * "Qwen3-TTS" case, second stop, the stream output builder).  Reference-audio
 * codes prefixed once to a stream warm its left context without producing
 * audio (same case, self-test answer 4 and exercise 3): that is
 * stream_prefill.  The codec's weights, state slots and workspace are all
 * allocated when it is opened, before any decode (same case, topology: the
 * vocoder is built before the engine so its memory is resident first; and
 * the note that incremental-decode state slots cost GPU memory).
 *
 * Conventions
 *   - Every function returns CODEC_OK (0) or one of the CODEC_E* codes; the
 *     message of the last failure is returned by codec_last_error().
 *   - Every argument check runs before anything is enqueued: a call that
 *     fails changes no state, on the host or on the device.
 *   - Device work is enqueued on the caller's HIP stream (passed as an opaque
 *     codec_hip_stream, NULL = the default stream) and the call returns
 *     without waiting for it.  All calls on one codec must be ordered by the
 *     caller (one host thread at a time, one stream or explicit ordering).
 *   - Memory: host pointers are read during the call only; device pointers
 *     (pcm, capture destinations) are written asynchronously on the stream
 *     and belong to the caller.
 */
#ifndef SNRVQ_H
#define SNRVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define CODEC_OK 0
#define CODEC_EINVAL 1  /* null pointer, non-positive size, bad cfg or weight manifest, pcm too small */
#define CODEC_ESTREAM 2 /* unknown or closed stream id */
#define CODEC_EDUP 3    /* the same stream twice in one call */
#define CODEC_ERANGE 4  /* a code outside [0, E), e.g. an EOS id such as 2150 */
#define CODEC_ENOSLOT 5 /* every state slot is in use */
#define CODEC_ETOOBIG 6 /* more frames in one call than max_frames_per_call */
#define CODEC_ENOMEM 7  /* device or pinned allocation failed */
#define CODEC_EHIP 8    /* a HIP runtime error (its string is in the message) */

/* ---- enums -------------------------------------------------------------- */
#define CODEC_DTYPE_F32 0
#define CODEC_DTYPE_BF16 1
#define CODEC_DTYPE_F16 2

#define CODEC_ACT_SNAKE 0 /* x + sin^2(alpha x) / alpha, per-channel alpha */
#define CODEC_ACT_ELU 1   /* x > 0 ? x : exp(x) - 1 */

#define CODEC_MAX_STAGES 8

typedef struct codec codec_t;     /* opaque, owned by the library */
typedef void *codec_hip_stream;   /* a hipStream_t; NULL = default stream */

/* One named parameter in host memory.  dtype CODEC_DTYPE_F32 (float) or
 * CODEC_DTYPE_BF16 (uint16 bit patterns); row-major with the given shape. */
typedef struct {
    const char *name;
    int32_t dtype;
    int32_t ndim;
    int64_t shape[4];
    const void *host_data;
} codec_tensor;

/* Decoder shape.  Channels start at d_lat and halve at every upsample stage;
 * stage i upsamples by strides[i] with a transposed conv of kernel
 * 2 strides[i] followed by residual units of dilation 1 and 3; hop =
 * product of strides.  tf_layers = 0 means no transformer.  weight_dtype
 * F32 runs the fp32 path (fp32 MFMA operands); BF16 weights run on fp16 MFMA
 * operands with fp32 accumulation and an fp32 residual stream. */
typedef struct {
    int32_t K, E, d_cb, d_lat;
    int32_t n_stages;
    int32_t strides[CODEC_MAX_STAGES];
    int32_t sample_rate;
    int32_t act;        /* CODEC_ACT_* */
    int32_t final_tanh; /* 0: raw PCM out of the last conv */
    int32_t tf_layers, tf_heads, tf_head_dim, tf_window, tf_mlp;
    int32_t weight_dtype; /* CODEC_DTYPE_F32 or CODEC_DTYPE_BF16 */
    int32_t max_streams;
    int32_t max_frames_per_call;
    int32_t flags; /* CODEC_FLAG_* */
} codec_cfg;

/* Run every layer as its own launch instead of the fused per-stage kernels
 * (same arithmetic, bit-identical output; for testing and comparison), for
 * all stages or for upsample stage i only. */
#define CODEC_FLAG_PER_LAYER 1
#define CODEC_FLAG_PER_LAYER_STAGE(i) (1 << (8 + (i)))
/* Conv GEMM planner restrictions, for testing and comparison.  NO_SPLIT_K:
 * never split a contraction over K (a split sums partials in another order,
 * so without splits every tile choice gives bit-identical output).
 * TWO_STAGE_BUFFERS: only tiles that double-buffer their K stages (not the
 * three-buffer 128 x 64 / 64 x 128 tiles).  NO_TALL_TILES: never the
 * 160-row tiles that replace 128 x 128 ones where those would leave a small
 * last round of work-groups (the rows of a tile do not change any sum, so
 * this too gives bit-identical output). */
#define CODEC_FLAG_NO_SPLIT_K 2
#define CODEC_FLAG_TWO_STAGE_BUFFERS 4
#define CODEC_FLAG_NO_TALL_TILES 8

typedef struct {
    int32_t hop;                 /* PCM samples per frame */
    int32_t sample_rate;
    int32_t K, E;
    int32_t left_context_frames; /* frames of history an output frame depends on */
    int32_t max_streams, max_frames_per_call, open_streams;
    int32_t compute_dtype;       /* CODEC_DTYPE_F32 or CODEC_DTYPE_F16 (MFMA operands) */
    int64_t state_bytes_per_stream;
    int64_t weight_bytes;
    int64_t workspace_bytes;
    int64_t graph_captures;      /* decode_chunk_graph: graphs captured so far */
    int64_t graph_replays;       /* decode_chunk_graph: steps that replayed one */
} codec_info_t;

/* ---- lifetime ----------------------------------------------------------- */

/* Validates cfg and the weight manifest (every canonical parameter present
 * once with the right shape and dtype), uploads and repacks the weights into
 * library-owned device memory on the current HIP device, and preallocates
 * the state slots of max_streams streams and the workspace of
 * max_frames_per_call frames.  No device or pinned memory is allocated
 * later (decode_chunk_graph's first use of a bucket instantiates a graph,
 * a runtime object).  The caller's host arrays may be freed on return.
 * With BF16 weights the compute operands are fp16: CODEC_EINVAL if a conv
 * or linear weight lies outside fp16's finite range (|w| > 65504) or the
 * codebooks' largest entries could sum past it.  On failure *out is NULL
 * and the message is available from codec_last_error(NULL). */
int codec_open(const codec_tensor *weights, int32_t n_weights, const codec_cfg *cfg,
               codec_t **out);

/* Waits for the codec's device work, frees everything it owns. */
int codec_close(codec_t *codec);

int codec_info(const codec_t *codec, codec_info_t *out);

/* Message of the last failure on this codec, or of the calling thread's last
 * codec_open failure when codec is NULL.  Never NULL. */
const char *codec_last_error(const codec_t *codec);

/* ---- streams ------------------------------------------------------------ */

/* Takes a free state slot; the stream starts with all-zero left context and
 * position 0.  Host-only bookkeeping: the slot is cleared on the stream's
 * first decode.  Ids are positive and never reused by this codec. */
int stream_open(codec_t *codec, int32_t *stream_id_out);

/* Releases the stream's slot.  Later use of the id fails with CODEC_ESTREAM. */
int stream_close(codec_t *codec, int32_t stream_id);

/* Decodes n frames of codes [n][K] (host memory) into the stream's state and
 * discards the audio: reference-audio codes used as left context.  n may
 * exceed max_frames_per_call (it is split into several decodes). */
int stream_prefill(codec_t *codec, int32_t stream_id, const int32_t *codes, int32_t n,
                   codec_hip_stream stream);

/* ---- the hot path ------------------------------------------------------- */

/* One batched decode step over B distinct open streams.
 *   stream_ids [B]    streams in this step (no duplicates)
 *   n_frames  [B]     new frames per stream, each >= 1 (any mix of sizes)
 *   codes             host int32, packed stream after stream, then frame,
 *                     then codebook: [sum n][K]
 *   pcm               device float32, caller-owned, pcm_capacity elements;
 *                     stream b's n_b * hop samples are written at
 *                     pcm[hop * sum_{b' < b} n_b'], in stream order
 * The dense form decode_chunk(ids, codes[B, n, K]) is the case where every
 * n_frames[b] == n.  Checks: CODEC_EINVAL (nulls, B < 1, n < 1, capacity),
 * CODEC_ESTREAM, CODEC_EDUP, CODEC_ETOOBIG (sum n > max_frames_per_call),
 * CODEC_ERANGE (a code outside [0, E)). */
int decode_chunk(codec_t *codec, int32_t B, const int32_t *stream_ids, const int32_t *n_frames,
                 const int32_t *codes, float *pcm, int64_t pcm_capacity,
                 codec_hip_stream stream);

/* The same step with the codes already in device memory (as when stage 0
 * samples them on this GPU): codes_dev is device int32 [sum n][K], read on
 * the stream.  Host checks are those of decode_chunk except the code range,
 * which is checked on the device: an out-of-range code is counted (see
 * codec_device_status) and replaced by code 0, so no access leaves the
 * codebook; the PCM of that step is then not meaningful. */
int decode_chunk_device(codec_t *codec, int32_t B, const int32_t *stream_ids,
                        const int32_t *n_frames, const int32_t *codes_dev, float *pcm,
                        int64_t pcm_capacity, codec_hip_stream stream);

/* The same step as decode_chunk, replayed from a HIP graph (the pages'
 * streaming decoders capture CUDA graphs per input-shape bucket; AREX
 * article on Fish Audio Drama 3, "two stages share one card", and the
 * AI-infra handbook's Qwen3-TTS case, "third stop: the streaming vocoder").
 * A step of F = sum n frames runs as the graph of its bucket: Fb = the next
 * power of two for F <= 32, else the next multiple of 32.  The Fb - F extra
 * frames belong to an internal pad stream (zero state, code 0, output
 * discarded), so any mix of per-stream chunk sizes with the same B and
 * bucket replays one graph: the per-stream layout travels in the step's
 * metadata, copied before the launch from the codec's pinned buffers.  The
 * first call for a (B, bucket) captures the step's kernels (the capture
 * runs nothing) and instantiates the graph; up to 64 graphs are kept, the
 * least recently used evicted.  The PCM is written to a codec buffer by the
 * graph and copied to pcm after it, on the stream.  Results are those of
 * decode_chunk for the same step within the parity bound (the pad frames
 * change the step's size, hence possibly its K-split plan, never its
 * arithmetic); replays of one bucket are bitwise repeatable.  Checks and
 * errors are those of decode_chunk (CODEC_EHIP if capture or instantiation
 * fails).  Profiling events are not recorded for graph steps; codec_info
 * counts captures and replays. */
int decode_chunk_graph(codec_t *codec, int32_t B, const int32_t *stream_ids,
                       const int32_t *n_frames, const int32_t *codes, float *pcm,
                       int64_t pcm_capacity, codec_hip_stream stream);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): decode_chunk_device
 * with the step's scratch -- its metadata and the split-K partial sums --
 * taken from a static device array of 32 MiB per GPU (1 MiB of metadata,
 * 31 MiB of partials) instead of the codec's buffers.  It allocates nothing,
 * on the device, the host or pinned.  Weights, state slots and the
 * activation workspace are the codec's, allocated by codec_open.  Arguments,
 * checks and results are those of decode_chunk_device (within the parity
 * bound: the smaller partial space can change a layer's K split), plus
 * CODEC_ETOOBIG when the step's metadata exceeds the 1 MiB region (about
 * 250,000 frames).  Every codec on a GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap on one GPU (different
 * codecs or streams without ordering) race and give wrong results.
 * codec_debug_capture after such a step reads the metadata in the array. */
int decode_chunk_device_noalloc(codec_t *codec, int32_t B, const int32_t *stream_ids,
                                const int32_t *n_frames, const int32_t *codes_dev, float *pcm,
                                int64_t pcm_capacity, codec_hip_stream stream);

/* Waits for the codec's device work and returns through *bad_codes the
 * number of out-of-range codes seen by decode_chunk_device since the last
 * call (then resets it).  CODEC_ERANGE when it is nonzero. */
int codec_device_status(codec_t *codec, int64_t *bad_codes);

/* ---- inspection (tests) -------------------------------------------------- */

#define CODEC_CAPTURE_LATENT 0    /* projected RVQ sum, [sum n][d_lat] (decoders with a
                                     transformer; the step composes the projection into the
                                     transformer's input projection, so the capture runs the
                                     projection GEMM on the step's stored RVQ sum first, on
                                     `stream`.  Without a transformer the projection is folded
                                     into the input conv and this capture is refused) */
#define CODEC_CAPTURE_DEC_INPUT 1 /* input of the conv decoder (after the transformer) */
#define CODEC_CAPTURE_RVQ_SUM 2   /* the gathered codebook sum z, [sum n][d_cb] */
/* Conv operands of the decoder, in network order (S = n_stages):
 *   CODEC_CAPTURE_LAYER0 + 3 i          stage i's transposed-conv input,
 *                                       activated: [sum n * r_i][C_i]
 *   CODEC_CAPTURE_LAYER0 + 3 i + 1 + j  residual unit j's input of stage i,
 *                                       activated: [sum n * r_{i+1}][C_{i+1}]
 *   CODEC_CAPTURE_LAYER0 + 3 S          the final conv's input: [sum n * hop][C_S]
 * (r_i = prod of strides before stage i, C_i = d_lat / 2^i).  These are the
 * stored MFMA operands (fp16 for BF16 weights), widened to float32.  Inside
 * a fused stage kernel the residual-unit and final-conv inputs never reach
 * memory: capturing them needs a codec opened with CODEC_FLAG_PER_LAYER
 * (same arithmetic, every layer stored), else CODEC_EINVAL. */
#define CODEC_CAPTURE_LAYER0 3

/* Copies an intermediate of the last decode step (any decode entry point)
 * as float32, packed like the codes: stream after stream, rows of a stream
 * in time order, [rows][channels].  dst is device memory with capacity
 * elements; written asynchronously on the stream.  For layer-by-layer
 * parity against a reference decode of the same frames. */
int codec_debug_capture(codec_t *codec, int32_t what, float *dst, int64_t capacity,
                        codec_hip_stream stream);

/* Copies the state slot of an open stream to host memory after waiting for
 * the codec's device work: the conv left contexts ([H][C] per layer, in the
 * compute type, in layer order) followed by nothing else.  *bytes_out
 * receives the slot size; dst may be NULL to query it. */
int codec_debug_read_state(codec_t *codec, int32_t stream_id, void *dst, int64_t capacity,
                           int64_t *bytes_out);

/* Per-kernel-class device time of the decode steps since the last reset,
 * measured with HIP events on the decode stream while profiling is on.
 * names/ms/launches receive up to cap entries; returns the entry count
 * through *n_out. */
int codec_profile_enable(codec_t *codec, int32_t on);
int codec_profile_read(codec_t *codec, int32_t cap, const char **names, double *ms,
                       int64_t *launches, int64_t *units, int32_t *n_out);

/* ---- host-only chunk policy (no device needed) --------------------------- */

/* New-frame counts of the decodes of an utterance of `total` generated
 * frames arriving one at a time (AI-infra handbook, "Qwen3-TTS" case, third
 * stop: decode when the generated count reaches the next threshold; the
 * threshold grows by the ramp entries, each clamped to `steady`, then by
 * `steady`; the final chunk decodes the remainder).  initial > 0 replaces
 * the first ramp entry.  Writes up to cap values to out; *n_out receives the
 * number of decodes (CODEC_EINVAL when it exceeds cap or arguments are bad). */
int codec_chunk_plan(int32_t total, const int32_t *ramp, int32_t n_ramp, int32_t steady,
                     int32_t initial, int32_t *out, int32_t cap, int32_t *n_out);

/* First-chunk size of one request, in frames (same section: a request may
 * ask for its own first chunk).  has_request = 0 takes fallback instead of
 * requested.  The size must be >= 0 and is capped at steady, which must be
 * >= 1; CODEC_EINVAL otherwise (message via codec_last_error(NULL)). */
int codec_initial_chunk_size(int64_t requested, int32_t has_request, int32_t steady,
                             int32_t fallback, int32_t *out);

/* Test-only: the conv GEMM planner's choice for one launch shape -- host
 * logic only, no device or codec needed.  M output rows, N output columns,
 * Cin input channels per tap, taps; fp16 = 1 for fp16 operands (0: fp32);
 * n_cu compute units; flags: any of CODEC_FLAG_NO_SPLIT_K,
 * CODEC_FLAG_TWO_STAGE_BUFFERS and CODEC_FLAG_NO_TALL_TILES.  *tile receives the tile's name (a static
 * string; "none" when no tile fits the shape), *splits the number of K
 * splits (1: unsplit), for the split-K workspace every codec allocates.
 * CODEC_EINVAL for non-positive sizes or NULL outputs. */
int codec_debug_conv_plan(int32_t M, int32_t N, int32_t Cin, int32_t taps, int32_t fp16,
                          int32_t n_cu, int32_t flags, const char **tile, int32_t *splits);

#ifdef __cplusplus
}
#endif

#endif /* SNRVQ_H */
