// api.cpp -- the C ABI: validation, weight repacking, the state-slot store,
// the ragged batcher and the per-step launch sequence.
//
// Decode step (all on the caller's stream):
//   H2D of the packed step metadata (codes, frame->stream map, cu, slots,
//   fresh flags, positions) from a pinned staging arena;
//   one launch: the RVQ gather-and-sum of every frame beside the halo fill
//   (every conv layer's left context, all streams);
//   projection GEMM -> [windowed transformer] -> input conv -> per stage
//   [ConvT -> RU(d=1) -> RU(d=3)] -> final conv to PCM, where an RU is a conv7
//   launch and a conv1 launch with the residual add in its epilogue (one
//   launch at 128 channels), and the late stages run as one fused kernel
//   each, the last one with the final conv;
//   halo save (last rows of every extended input back into the slots).
// Every activation (Snake / ELU) is applied once, in the epilogue of the
// layer that produces its input, so the stored left context is exactly the
// operand the next conv multiplies.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <map>
#include <mutex>
#include <thread>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "internal.h"
#include "snrvq.h"

using namespace snrvq;

namespace {

thread_local std::string g_err = "";

constexpr long kSplitKCap = 16L << 20;  // split-K partials per codec: 64 MiB of fp32
// A graph step of F frames runs with Fb - F < kGraphPadMax pad frames.
constexpr int kGraphPadMax = 32;

int set_err(std::string *dst, int code, const char *fmt, ...)
{
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (dst)
        *dst = buf;
    g_err = buf;
    return code;
}

struct Lin {
    void *Wt = nullptr;
    float *bias = nullptr;
    int N = 0, Cout = 0, Cin = 0, taps = 1, dil = 1, s = 1;
};

struct ActP {
    float *alpha = nullptr, *ialpha = nullptr;
};

struct ProfRec {
    int cls;
    hipEvent_t a, b;
    int64_t units;
};

struct ParamSpec {
    std::string name;
    std::vector<int64_t> shape;
};

const int RU_DIL[2] = {1, 3};

}  // namespace

struct codec {
    codec_cfg cfg{};
    int dev = 0;
    int dtype = 1;  // 1: fp16 MFMA operands, 0: fp32
    int esz = 2;
    int S = 0, hop = 1;
    int ch[CODEC_MAX_STAGES + 1]{};
    int rate[CODEC_MAX_STAGES + 1]{};
    int left_ctx = 0;
    int maxF = 0, maxB = 0;
    int n_cu = 256;  // compute units of the device

    std::vector<void *> allocs;
    void *cb = nullptr;
    int cb_dtype = 0;
    Lin proj, in_conv, convT[CODEC_MAX_STAGES], conv7[CODEC_MAX_STAGES][2],
        conv1[CODEC_MAX_STAGES][2];
    ActP a_stage[CODEC_MAX_STAGES], a_ru1[CODEC_MAX_STAGES][2], a_ru2[CODEC_MAX_STAGES][2], a_out;
    float *out_w = nullptr;
    float out_b = 0.f;

    // windowed transformer (tf_layers > 0)
    int dm = 0;
    Lin tf_in, tf_out, tf_qkv[16], tf_o[16], tf_fc1[16], tf_fc2[16];
    float *ln1_g[16]{}, *ln1_b[16]{}, *ln2_g[16]{}, *ln2_b[16]{}, *lnf_g = nullptr,
          *lnf_b = nullptr;
    double *inv_freq = nullptr;
    void *u16 = nullptr, *a16 = nullptr, *att16 = nullptr, *f16 = nullptr;
    float *h32 = nullptr, *qkv32 = nullptr, *kring = nullptr, *vring = nullptr;
    float *rot = nullptr;  // [F][hd/2] (cos, sin) of the step's rotary angles

    // Decoders without a transformer fold the projection into the input conv
    // (fold): the gather writes z' = [z, 1, 0...] rows of dz values into the
    // extended buffer z, and the input conv's weights are W_in composed with
    // [W_p | b_p] (computed at open).  Otherwise z is the packed RVQ sum
    // (dz = d_cb) and the projection runs as its own GEMM into u_ext / u16.
    bool fold = false;
    int dz = 0;
    void *z = nullptr, *u_ext = nullptr, *aT[CODEC_MAX_STAGES]{}, *a1[CODEC_MAX_STAGES]{},
         *a2[CODEC_MAX_STAGES]{}, *h = nullptr, *a_outb = nullptr;
    float *x = nullptr, *pcm_scratch = nullptr;
    float *splitk_ws = nullptr;  // split-K partial sums
    long splitk_cap = 0;         // floats
    // buffers of the step being enqueued: the codec's own (above and
    // meta_dev), or the no-allocation entry point's static scratch
    float *partial_now = nullptr;
    long partial_cap_now = 0;
    void *meta_now = nullptr;

    void *state = nullptr;
    int64_t slot_elems = 0;
    HaloTable halo{};       // filled before every step
    HaloTable halo_save{};  // saved after it (fused stages write their own)
    int fuse_T[CODEC_MAX_STAGES]{};  // output rows per tile of a fused stage, 0 = per-layer
    // stages that have a fused kernel, whether or not it is used: their
    // per-layer convs run K in one pass, the fused kernel's summation order
    bool fusable[CODEC_MAX_STAGES]{};
    int64_t off_a1[CODEC_MAX_STAGES]{}, off_a2[CODEC_MAX_STAGES]{}, off_ao = 0;

    void *meta_dev = nullptr;
    size_t meta_cap = 0;  // int32 elements
    unsigned long long *bad_codes = nullptr;  // device counter (device-resident codes)
    // Pinned staging of the step metadata: an arena used as a ring.  Each
    // step takes the next span of it, and an event recorded after the step's
    // launches releases the span; the host waits only when the arena (or the
    // event pool) is full, so it can queue many steps ahead of the device
    // and a host-side pause does not leave the device idle.
    char *arena = nullptr;
    size_t arena_cap = 0, arena_head = 0;
    struct Span {
        size_t begin, end;
        hipEvent_t ev;
    };
    std::deque<Span> inflight;          // oldest first
    std::vector<hipEvent_t> ev_free;    // preallocated at open
    // Step graphs (decode_chunk_graph), keyed by (streams in the graph, frames
    // in the graph): a step of F frames runs as a graph of the next bucket of
    // Fb >= F frames, the difference decoded by the pad stream (slot pad_slot,
    // zero state, codes 0, its output discarded).  The graph holds kernels
    // only; the metadata copy before it and the PCM copy after it are plain
    // stream operations, so every graph shares the codec's buffers.
    struct GraphEntry {
        hipGraphExec_t exec = nullptr;
        hipEvent_t done = nullptr;
        uint64_t last_use = 0;
    };
    std::map<std::pair<int, int>, GraphEntry> graphs;
    uint64_t graph_clock = 0;
    int64_t graph_captures = 0, graph_replays = 0;
    bool capturing = false;
    hipStream_t cap_stream = nullptr;  // graphs are captured here, launched on the caller's
    int pad_slot = 0;                  // state slot of the graph pad stream (max_streams)
    int allocF = 0, allocB = 0;        // frames and streams the workspace holds
    StepMeta last_meta{};
    int lastF = 0, lastB = 0;

    std::unordered_map<int32_t, int> id2slot;
    std::vector<int> free_slots;
    std::vector<int64_t> slot_pos;
    std::vector<char> slot_fresh;
    int32_t next_id = 1;

    std::string err;
    int64_t weight_bytes = 0, workspace_bytes = 0;

    bool prof = false;
    std::vector<std::string> cls_names;
    std::vector<double> cls_ms;
    std::vector<int64_t> cls_launches, cls_units;
    std::vector<ProfRec> recs;
    std::vector<hipEvent_t> ev_pool;
};

namespace {

int fail(codec *c, int code, const char *fmt, ...)
{
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (c)
        c->err = buf;
    g_err = buf;
    return code;
}

#define HIPCHK(c, expr)                                                                        \
    do {                                                                                       \
        hipError_t e_ = (expr);                                                                \
        if (e_ != hipSuccess)                                                                  \
            return fail((c), CODEC_EHIP, "HIP error %s (%d) at %s", hipGetErrorString(e_),     \
                        (int)e_, #expr);                                                       \
    } while (0)

int dev_alloc(codec *c, void **p, size_t bytes, int64_t *counter)
{
    if (bytes == 0)
        bytes = 16;
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(c, CODEC_ENOMEM, "hipMalloc of %zu bytes failed: %s", bytes,
                    hipGetErrorString(e));
    }
    c->allocs.push_back(*p);
    if (counter)
        *counter += (int64_t)bytes;
    return CODEC_OK;
}

// ---- canonical parameter list ----------------------------------------------
std::vector<ParamSpec> param_specs(const codec_cfg &g, const int *ch)
{
    std::vector<ParamSpec> v;
    char n[128];
    for (int k = 0; k < g.K; k++) {
        snprintf(n, sizeof n, "rvq.codebook.%d", k);
        v.push_back({n, {g.E, g.d_cb}});
    }
    v.push_back({"rvq.proj.weight", {g.d_lat, g.d_cb}});
    v.push_back({"rvq.proj.bias", {g.d_lat}});
    if (g.tf_layers > 0) {
        int64_t dm = (int64_t)g.tf_heads * g.tf_head_dim, mlp = g.tf_mlp;
        v.push_back({"tf.in_proj.weight", {dm, g.d_lat}});
        v.push_back({"tf.in_proj.bias", {dm}});
        for (int l = 0; l < g.tf_layers; l++) {
            std::string p = "tf.layer." + std::to_string(l) + ".";
            v.push_back({p + "ln1.weight", {dm}});
            v.push_back({p + "ln1.bias", {dm}});
            v.push_back({p + "attn.qkv.weight", {3 * dm, dm}});
            v.push_back({p + "attn.qkv.bias", {3 * dm}});
            v.push_back({p + "attn.out.weight", {dm, dm}});
            v.push_back({p + "attn.out.bias", {dm}});
            v.push_back({p + "ln2.weight", {dm}});
            v.push_back({p + "ln2.bias", {dm}});
            v.push_back({p + "mlp.fc1.weight", {mlp, dm}});
            v.push_back({p + "mlp.fc1.bias", {mlp}});
            v.push_back({p + "mlp.fc2.weight", {dm, mlp}});
            v.push_back({p + "mlp.fc2.bias", {dm}});
        }
        v.push_back({"tf.ln_f.weight", {dm}});
        v.push_back({"tf.ln_f.bias", {dm}});
        v.push_back({"tf.out_proj.weight", {g.d_lat, dm}});
        v.push_back({"tf.out_proj.bias", {g.d_lat}});
    }
    v.push_back({"dec.in_conv.weight", {ch[0], g.d_lat, 7}});
    v.push_back({"dec.in_conv.bias", {ch[0]}});
    for (int i = 0; i < g.n_stages; i++) {
        int ci = ch[i], co = ch[i + 1], s = g.strides[i];
        snprintf(n, sizeof n, "dec.stage.%d.snake.alpha", i);
        v.push_back({n, {ci}});
        snprintf(n, sizeof n, "dec.stage.%d.convT.weight", i);
        v.push_back({n, {ci, co, 2 * s}});
        snprintf(n, sizeof n, "dec.stage.%d.convT.bias", i);
        v.push_back({n, {co}});
        for (int j = 0; j < 2; j++) {
            const char *parts[6] = {"snake1.alpha", "conv7.weight", "conv7.bias",
                                    "snake2.alpha", "conv1.weight", "conv1.bias"};
            std::vector<int64_t> shp[6] = {{co}, {co, co, 7}, {co}, {co}, {co, co, 1}, {co}};
            for (int q = 0; q < 6; q++) {
                snprintf(n, sizeof n, "dec.stage.%d.ru.%d.%s", i, j, parts[q]);
                v.push_back({n, shp[q]});
            }
        }
    }
    int cs = ch[g.n_stages];
    v.push_back({"dec.out.snake.alpha", {cs}});
    v.push_back({"dec.out.conv.weight", {1, cs, 7}});
    v.push_back({"dec.out.conv.bias", {1}});
    return v;
}

// Host values of a tensor as fp32 (bf16 widening is exact).
std::vector<float> host_f32(const codec_tensor &t, int64_t n)
{
    std::vector<float> out((size_t)n);
    if (t.dtype == CODEC_DTYPE_F32) {
        memcpy(out.data(), t.host_data, sizeof(float) * (size_t)n);
    } else {
        const uint16_t *b = (const uint16_t *)t.host_data;
        for (int64_t i = 0; i < n; i++) {
            uint32_t u = (uint32_t)b[i] << 16;
            memcpy(&out[(size_t)i], &u, 4);
        }
    }
    return out;
}

// Upload values in the compute type.
int upload_compute(codec *c, const std::vector<float> &v, void **dst)
{
    size_t n = v.size();
    int rc = dev_alloc(c, dst, n * c->esz, &c->weight_bytes);
    if (rc)
        return rc;
    if (c->dtype) {
        std::vector<half_t> h(n);
        for (size_t i = 0; i < n; i++)
            h[i] = (half_t)v[i];
        HIPCHK(c, hipMemcpy(*dst, h.data(), n * 2, hipMemcpyHostToDevice));
    } else {
        HIPCHK(c, hipMemcpy(*dst, v.data(), n * 4, hipMemcpyHostToDevice));
    }
    return CODEC_OK;
}

int upload_f32(codec *c, const std::vector<float> &v, float **dst)
{
    int rc = dev_alloc(c, (void **)dst, v.size() * 4, &c->weight_bytes);
    if (rc)
        return rc;
    HIPCHK(c, hipMemcpy(*dst, v.data(), v.size() * 4, hipMemcpyHostToDevice));
    return CODEC_OK;
}

// Snake parameters as the kernels use them: alpha / 2pi (the hardware sine
// takes revolutions) and 1 / alpha, both rounded once from fp64.
int upload_act(codec *c, const std::vector<float> &alpha, ActP *a)
{
    std::vector<float> rev(alpha.size()), inv(alpha.size());
    for (size_t i = 0; i < alpha.size(); i++) {
        rev[i] = (float)((double)alpha[i] / (2.0 * M_PI));
        inv[i] = (float)(1.0 / (double)alpha[i]);
    }
    int rc = upload_f32(c, rev, &a->alpha);
    if (rc)
        return rc;
    return upload_f32(c, inv, &a->ialpha);
}

// Conv1d weight W[Co][Ci][k] -> Wt[o][tap Ci + c].
std::vector<float> pack_conv(const std::vector<float> &W, int Co, int Ci, int k)
{
    std::vector<float> o((size_t)Co * Ci * k);
    for (int oc = 0; oc < Co; oc++)
        for (int c = 0; c < Ci; c++)
            for (int j = 0; j < k; j++)
                o[((size_t)oc * k + j) * Ci + c] = W[((size_t)oc * Ci + c) * k + j];
    return o;
}

// ConvTranspose1d weight W[Ci][Co][2s] -> polyphase Wt[r Co + o][tap Ci + c]:
// tap 0 multiplies x[q-1] (kernel index r + s), tap 1 multiplies x[q] (r).
std::vector<float> pack_convT(const std::vector<float> &W, int Ci, int Co, int s)
{
    std::vector<float> o((size_t)s * Co * 2 * Ci);
    int k = 2 * s;
    for (int r = 0; r < s; r++)
        for (int oc = 0; oc < Co; oc++)
            for (int c = 0; c < Ci; c++) {
                size_t n = (size_t)r * Co + oc;
                o[(n * 2 + 0) * Ci + c] = W[((size_t)c * Co + oc) * k + r + s];
                o[(n * 2 + 1) * Ci + c] = W[((size_t)c * Co + oc) * k + r];
            }
    return o;
}

// Input conv composed with the projection, for decoders whose projection
// feeds the input conv directly.  The conv of u = W_p z + b_p over a zero
// left context equals, tap by tap, a conv of z' = [z, 1, 0...] (zero left
// context too: the 1 is absent before the stream's first frame, exactly
// where the bias b_p is) with weights W_in[o][:, tap] [W_p | b_p]:
//   Wc[o][tap dz + c] = sum_m W_in[o][m][tap] W'[m][c],
//   W'[m][c] = W_p[m][c] (c < d_cb), b_p[m] (c = d_cb), 0 (c > d_cb).
// Summed in fp64 over m ascending, then rounded once to fp32.  Packed K-major
// ([o][tap][c]) for the implicit GEMM.  Rows split over host threads.
std::vector<float> fold_projection(const std::vector<float> &Win /*[Co][Dl][7]*/,
                                   const std::vector<float> &Wp /*[Dl][Dcb]*/,
                                   const std::vector<float> &bp /*[Dl]*/, int Co, int Dl, int Dcb,
                                   int dz)
{
    std::vector<double> wpx((size_t)Dl * dz, 0.0);
    for (int m = 0; m < Dl; m++) {
        for (int cc = 0; cc < Dcb; cc++)
            wpx[(size_t)m * dz + cc] = Wp[(size_t)m * Dcb + cc];
        wpx[(size_t)m * dz + Dcb] = bp[m];
    }
    std::vector<float> out((size_t)Co * 7 * dz);
    auto rows = [&](int o0, int o1) {
        std::vector<double> acc((size_t)7 * dz);
        for (int o = o0; o < o1; o++) {
            std::fill(acc.begin(), acc.end(), 0.0);
            for (int m = 0; m < Dl; m++) {
                const double *wr = wpx.data() + (size_t)m * dz;
                for (int tap = 0; tap < 7; tap++) {
                    const double w = Win[((size_t)o * Dl + m) * 7 + tap];
                    double *ar = acc.data() + (size_t)tap * dz;
                    for (int cc = 0; cc <= Dcb; cc++)
                        ar[cc] += w * wr[cc];
                }
            }
            for (size_t k = 0; k < acc.size(); k++)
                out[(size_t)o * 7 * dz + k] = (float)acc[k];
        }
    };
    unsigned nt = std::thread::hardware_concurrency();
    nt = nt < 1 ? 1 : (nt > 16 ? 16 : nt);
    std::vector<std::thread> th;
    const int per = (Co + (int)nt - 1) / (int)nt;
    for (unsigned t = 0; t < nt; t++) {
        const int o0 = (int)t * per, o1 = std::min(Co, o0 + per);
        if (o0 < o1)
            th.emplace_back(rows, o0, o1);
    }
    for (auto &x : th)
        x.join();
    return out;
}

// The transformer's input projection composed with the codebook-space
// projection (nothing between the two linear maps: the latent feeds only the
// transformer): h = W_in (W_p z + b_p) + b_in = (W_in W_p) z + (W_in b_p + b_in).
// Summed in fp64 over the latent index ascending, then rounded once to fp32.
// Wf: [Dm][Dcb] (row-major, the k = 1 GEMM's packed layout); bf: [Dm].
void fold_tf_input(const std::vector<float> &Win /*[Dm][Dl]*/, const std::vector<float> &bin,
                   const std::vector<float> &Wp /*[Dl][Dcb]*/, const std::vector<float> &bp,
                   int Dm, int Dl, int Dcb, std::vector<float> &Wf, std::vector<float> &bf)
{
    Wf.assign((size_t)Dm * Dcb, 0.f);
    bf.assign(Dm, 0.f);
    auto rows = [&](int o0, int o1) {
        std::vector<double> acc(Dcb);
        for (int o = o0; o < o1; o++) {
            std::fill(acc.begin(), acc.end(), 0.0);
            double bacc = 0.0;
            for (int m = 0; m < Dl; m++) {
                const double w = Win[(size_t)o * Dl + m];
                const float *wp = Wp.data() + (size_t)m * Dcb;
                for (int cc = 0; cc < Dcb; cc++)
                    acc[cc] += w * wp[cc];
                bacc += w * bp[m];
            }
            for (int cc = 0; cc < Dcb; cc++)
                Wf[(size_t)o * Dcb + cc] = (float)acc[cc];
            bf[o] = (float)(bacc + bin[o]);
        }
    };
    unsigned nt = std::thread::hardware_concurrency();
    nt = nt < 1 ? 1 : (nt > 16 ? 16 : nt);
    std::vector<std::thread> th;
    const int per = (Dm + (int)nt - 1) / (int)nt;
    for (unsigned t = 0; t < nt; t++) {
        const int o0 = (int)t * per, o1 = std::min(Dm, o0 + per);
        if (o0 < o1)
            th.emplace_back(rows, o0, o1);
    }
    for (auto &x : th)
        x.join();
}

int make_lin(codec *c, const std::vector<float> &packed, const std::vector<float> &bias, int N,
             int Cout, int Cin, int taps, int dil, int s, Lin *L)
{
    L->N = N;
    L->Cout = Cout;
    L->Cin = Cin;
    L->taps = taps;
    L->dil = dil;
    L->s = s;
    int rc = upload_compute(c, packed, &L->Wt);
    if (rc)
        return rc;
    return upload_f32(c, bias, &L->bias);
}

// Frames of history that one output frame depends on: walk back from every
// sample of a frame through the layers (causal conv: i - (k-1) d; transposed
// conv: floor(i / s) - 1).
int left_context_frames(const codec_cfg &g, int hop)
{
    int best = 0;
    for (long n = 4L * hop; n < 5L * hop; n++) {
        long i = n - 6;
        for (int st = g.n_stages - 1; st >= 0; st--) {
            i -= 18;
            i -= 6;
            long s = g.strides[st];
            i = (i >= 0 ? i / s : -((-i + s - 1) / s)) - 1;
        }
        i -= 6;
        i -= (long)g.tf_layers * (g.tf_window > 0 ? g.tf_window - 1 : 0);
        long L = n / hop - i;
        if (L > best)
            best = (int)L;
    }
    return best;
}

hipEvent_t get_ev(codec *c)
{
    if (c->ev_pool.empty()) {
        hipEvent_t e;
        (void)hipEventCreate(&e);
        return e;
    }
    hipEvent_t e = c->ev_pool.back();
    c->ev_pool.pop_back();
    return e;
}

int cls_id(codec *c, const std::string &name)
{
    for (size_t i = 0; i < c->cls_names.size(); i++)
        if (c->cls_names[i] == name)
            return (int)i;
    c->cls_names.push_back(name);
    c->cls_ms.push_back(0.0);
    c->cls_launches.push_back(0);
    c->cls_units.push_back(0);
    return (int)c->cls_names.size() - 1;
}

template <class Fn>
int timed(codec *c, const char *name, int64_t units, hipStream_t s, Fn &&fn)
{
    hipEvent_t a = nullptr, b = nullptr;
    const bool prof = c->prof && !c->capturing;
    if (prof) {
        a = get_ev(c);
        b = get_ev(c);
        (void)hipEventRecord(a, s);
    }
    hipError_t e = fn();
    if (prof) {
        (void)hipEventRecord(b, s);
        c->recs.push_back({cls_id(c, name), a, b, units});
    }
    if (e != hipSuccess)
        return fail(c, CODEC_EHIP, "kernel launch '%s' failed: %s", name, hipGetErrorString(e));
    return CODEC_OK;
}

ConvArgs conv_args(codec *c, const Lin &L, const void *A, int A_H, int rate_in, int M,
                   const StepMeta &m)
{
    ConvArgs a{};
    a.tall_allowed = !(c->cfg.flags & CODEC_FLAG_NO_TALL_TILES);
    a.A = A;
    a.Wt = L.Wt;
    a.bias = L.bias;
    a.frame_stream = m.frame_stream;
    a.M = M;
    a.A_H = A_H;
    a.Cin = L.Cin;
    a.taps = L.taps;
    a.dil = L.dil;
    a.rate_in = rate_in;
    a.N = L.N;
    a.Cout = L.Cout;
    a.s = L.s;
    a.out_ld = L.Cout;
    a.act = ACT_NONE;
    return a;
}

void set_act(codec *c, ConvArgs &a, const ActP &p)
{
    a.act = c->cfg.act == CODEC_ACT_ELU ? ACT_ELU : ACT_SNAKE;
    a.alpha = p.alpha;
    a.inv_alpha = p.ialpha;
}

int run_conv(codec *c, const char *name, const ConvArgs &a0, hipStream_t s, bool allow_split = true)
{
    ConvArgs a = a0;
    a.splits_allowed = allow_split && !(c->cfg.flags & CODEC_FLAG_NO_SPLIT_K);
    a.deep_allowed = !(c->cfg.flags & CODEC_FLAG_TWO_STAGE_BUFFERS);
    a.tall_allowed = !(c->cfg.flags & CODEC_FLAG_NO_TALL_TILES);
    a.partial = c->partial_now;
    const ConvPlan plan = conv_gemm_plan(a, c->dtype, c->n_cu, c->partial_cap_now);
    return timed(c, name, (int64_t)a.M, s,
                 [&] { return launch_conv_gemm(a, c->dtype, s, plan); });
}

size_t round4(size_t n) { return (n + 3) & ~(size_t)3; }

// Stage i as one fused kernel (ConvT + both residual units [+ final conv]).
int enqueue_fused_stage(codec *c, int i, int F, const StepMeta &m, float *pcm, hipStream_t s)
{
    const bool fin = i == c->S - 1;
    StageArgs a{};
    a.aT = (const half_t *)c->aT[i];
    a.WT = (const half_t *)c->convT[i].Wt;
    a.bT = c->convT[i].bias;
    for (int j = 0; j < 2; j++) {
        a.W7[j] = (const half_t *)c->conv7[i][j].Wt;
        a.b7[j] = c->conv7[i][j].bias;
        a.W1[j] = (const half_t *)c->conv1[i][j].Wt;
        a.b1[j] = c->conv1[i][j].bias;
        a.al1[j] = c->a_ru1[i][j].alpha;
        a.ial1[j] = c->a_ru1[i][j].ialpha;
        a.al2[j] = c->a_ru2[i][j].alpha;
        a.ial2[j] = c->a_ru2[i][j].ialpha;
    }
    const ActP &nx = fin ? c->a_out : c->a_stage[i + 1];
    a.al_next = nx.alpha;
    a.ial_next = nx.ialpha;
    a.a1_ext = (const half_t *)c->a1[i];
    a.a2_ext = (const half_t *)c->a2[i];
    a.ao_ext = (const half_t *)c->a_outb;
    a.next = fin ? nullptr : (half_t *)c->aT[i + 1];
    a.pcm = pcm;
    a.w_out = c->out_w;
    a.b_out = c->out_b;
    a.final_tanh = c->cfg.final_tanh;
    a.state = (half_t *)c->state;
    a.slot_elems = c->slot_elems;
    a.off_a1 = c->off_a1[i];
    a.off_a2 = c->off_a2[i];
    a.off_ao = c->off_ao;
    a.frame_stream = m.frame_stream;
    a.cu = m.cu;
    a.slot = m.slot;
    a.tile_cu = m.tile_cu[i];
    a.n_streams = m.B;
    a.n_tiles = m.n_tiles[i];
    a.r_in = c->rate[i];
    a.r_out = c->rate[i + 1];
    a.act = c->cfg.act == CODEC_ACT_ELU ? ACT_ELU : ACT_SNAKE;
    a.n_cu = c->n_cu;
    if (fin)
        a.save = c->halo_save;  // the step's halo save rides on the last stage
    char nm[32];
    snprintf(nm, sizeof nm, "s%d.fused", i);
    return timed(c, nm, (int64_t)F * c->rate[i + 1], s, [&] {
        return F > 0 ? launch_stage_fused(a, c->ch[i + 1], c->cfg.strides[i], c->fuse_T[i], fin, s)
                     : hipSuccess;
    });
}

// Windowed causal transformer over the F new frames of this step (pre-norm
// layers; the KV ring holds every stream's last W-1 frames per layer).
int enqueue_transformer(codec *c, int B, int F, const StepMeta &m, hipStream_t s)
{
    const codec_cfg &g = c->cfg;
    const int dm = c->dm;
    ConvArgs a = conv_args(c, c->tf_in, c->z, 0, 1, F, m);  // projection folded in
    a.out32 = c->h32;
    int rc = run_conv(c, "tf.in_proj", a, s);
    if (rc)
        return rc;
    AttnArgs at{};
    at.qkv = c->qkv32;
    at.rot = c->rot;
    at.att = c->att16;
    at.kring = c->kring;
    at.vring = c->vring;
    at.frame_stream = m.frame_stream;
    at.cu = m.cu;
    at.slot = m.slot;
    at.pos = m.pos;
    at.attn_q = m.attn_q;
    at.n_qblocks = m.n_qblocks;
    at.F = F;
    at.H = g.tf_heads;
    at.hd = g.tf_head_dim;
    at.W = g.tf_window;
    at.n_layers = g.tf_layers;
    at.dtype = c->dtype;
    // the rotary angles depend on the frame only: one table for every layer
    if ((rc = timed(c, "tf.rope", F, s, [&] {
             return launch_rope_table(c->rot, c->inv_freq, m.frame_stream, m.cu, m.pos, F,
                                      g.tf_head_dim, s);
         })))
        return rc;
    for (int l = 0; l < g.tf_layers; l++) {
        at.layer = l;
        if ((rc = timed(c, "tf.ln", F, s, [&] {
                 return launch_layer_norm(c->h32, c->ln1_g[l], c->ln1_b[l], F, dm, c->a16,
                                          c->dtype, s);
             })))
            return rc;
        a = conv_args(c, c->tf_qkv[l], c->a16, 0, 1, F, m);
        a.out32 = c->qkv32;
        if ((rc = run_conv(c, "tf.qkv", a, s)))
            return rc;
        if ((rc = timed(c, "tf.attention", F, s, [&] { return launch_window_attention(at, s); })))
            return rc;
        a = conv_args(c, c->tf_o[l], c->att16, 0, 1, F, m);
        a.res = c->h32;
        a.out32 = c->h32;
        if ((rc = run_conv(c, "tf.o_proj", a, s)))
            return rc;
        // the second LayerNorm's launch also appends this layer's K/V rows to
        // the ring (after the attention that read the ring's old rows)
        if ((rc = timed(c, "tf.ln+kv_append", F, s, [&] {
                 return launch_layer_norm(c->h32, c->ln2_g[l], c->ln2_b[l], F, dm, c->a16,
                                          c->dtype, s, &at);
             })))
            return rc;
        a = conv_args(c, c->tf_fc1[l], c->a16, 0, 1, F, m);
        a.out16 = c->f16;
        a.out_H = 0;
        a.act = ACT_GELU;
        if ((rc = run_conv(c, "tf.fc1", a, s)))
            return rc;
        a = conv_args(c, c->tf_fc2[l], c->f16, 0, 1, F, m);
        a.res = c->h32;
        a.out32 = c->h32;
        if ((rc = run_conv(c, "tf.fc2", a, s)))
            return rc;
    }
    if ((rc = timed(c, "tf.ln", F, s, [&] {
             return launch_layer_norm(c->h32, c->lnf_g, c->lnf_b, F, dm, c->a16, c->dtype, s);
         })))
        return rc;
    a = conv_args(c, c->tf_out, c->a16, 0, 1, F, m);
    a.out16 = c->u_ext;
    a.out_H = 6;
    return run_conv(c, "tf.out_proj", a, s);
}

// One decode step over B streams (slots[] / n[] / codes[] already validated).
// codes: host array (copied with the metadata) or, when codes_on_device,
// a device array read in place.
// Step metadata written into host buffer hp; m points into the device copy.
struct MetaLayout {
    size_t total = 0;  // int32 elements to copy
    StepMeta m{};
};

// Attention query blocks of a step of B streams and F frames, at most: each
// stream's frames in blocks of SNRVQ_ATTN_QB, the last shorter.
inline int attn_qblock_bound(int B, int F) { return (F + SNRVQ_ATTN_QB - 1) / SNRVQ_ATTN_QB + B; }

// Metadata layout of a step of B streams and F frames (int32 offsets).
struct MetaOffsets {
    size_t codes, fs, cu, slot, fresh, pos, tile[CODEC_MAX_STAGES], attn, total;
};
MetaOffsets meta_offsets(const codec *c, int B, int F, bool codes_on_device)
{
    MetaOffsets o{};
    const size_t ncodes = codes_on_device ? 0 : (size_t)F * c->cfg.K;
    o.codes = 0;
    o.fs = round4(o.codes + ncodes);
    o.cu = round4(o.fs + F);
    o.slot = round4(o.cu + B + 1);
    o.fresh = round4(o.slot + B);
    o.pos = round4(o.fresh + B);
    o.total = round4(o.pos + B);
    for (int i = 0; i < c->S; i++)
        if (c->fuse_T[i]) {
            o.tile[i] = o.total;
            o.total = round4(o.total + B + 1);
        }
    if (c->cfg.tf_layers) {
        o.attn = o.total;
        o.total = round4(o.total + SNRVQ_ATTN_Q_INTS * (size_t)attn_qblock_bound(B, F));
    }
    return o;
}

// Fills the step metadata into host buffer hp (its device copy goes to
// c->meta_now).  codes: host codes of the first code_frames frames (the rest,
// pad frames, get code 0), or with codes_on_device the device array itself.
// For a graph (tile_bound), the fused stages' tile counts in the launch
// arguments are the most any step of this (B, F) can have; the kernels read
// the step's own count from the metadata.
MetaLayout fill_meta(codec *c, int32_t *hp, int B, const int *slots, const int32_t *n,
                     const int32_t *codes, bool codes_on_device, int code_frames = -1,
                     bool tile_bound = false)
{
    const codec_cfg &g = c->cfg;
    int F = 0;
    for (int b = 0; b < B; b++)
        F += n[b];
    if (code_frames < 0)
        code_frames = F;
    const MetaOffsets o = meta_offsets(c, B, F, codes_on_device);
    if (!codes_on_device) {
        memcpy(hp + o.codes, codes, sizeof(int32_t) * (size_t)code_frames * g.K);
        memset(hp + o.codes + (size_t)code_frames * g.K, 0,
               sizeof(int32_t) * (size_t)(F - code_frames) * g.K);
    }
    int acc = 0;
    hp[o.cu] = 0;
    for (int b = 0; b < B; b++) {
        for (int f = 0; f < n[b]; f++)
            hp[o.fs + acc + f] = b;
        acc += n[b];
        hp[o.cu + b + 1] = acc;
        hp[o.slot + b] = slots[b];
        hp[o.fresh + b] = c->slot_fresh[slots[b]] ? 1 : 0;
        hp[o.pos + b] = (int32_t)c->slot_pos[slots[b]];
    }
    int32_t *dm = (int32_t *)c->meta_now;
    StepMeta m{codes_on_device ? (int32_t *)codes : dm + o.codes, dm + o.fs, dm + o.cu,
               dm + o.slot, dm + o.fresh, dm + o.pos};
    m.B = B;
    // fused stages: each stream's output rows in tiles of fuse_T rows, the last shorter
    for (int i = 0; i < c->S; i++) {
        if (!c->fuse_T[i])
            continue;
        int32_t *tc = hp + o.tile[i];
        tc[0] = 0;
        for (int b = 0; b < B; b++) {
            const int64_t rows = (int64_t)n[b] * c->rate[i + 1];
            tc[b + 1] = tc[b] + (int32_t)((rows + c->fuse_T[i] - 1) / c->fuse_T[i]);
        }
        m.tile_cu[i] = dm + o.tile[i];
        m.n_tiles[i] = tile_bound ? (int)(((int64_t)F * c->rate[i + 1] + c->fuse_T[i] - 1) /
                                              c->fuse_T[i] + B)
                                  : tc[B];
    }
    // attention: each stream's frames in query blocks of SNRVQ_ATTN_QB, the
    // last shorter; per block its first frame, frame count, the position of
    // its first frame and of the stream's first frame of the step, and the
    // stream's slot; blocks of no frames up to the bound
    if (g.tf_layers) {
        int32_t *aq = hp + o.attn;
        const int bound = attn_qblock_bound(B, F);
        int nq = 0, f0 = 0;
        for (int b = 0; b < B; b++) {
            const int32_t p0 = hp[o.pos + b];
            for (int q = 0; q < n[b]; q += SNRVQ_ATTN_QB, nq++) {
                int32_t *e = aq + (size_t)SNRVQ_ATTN_Q_INTS * nq;
                e[0] = f0 + q;
                e[1] = std::min(SNRVQ_ATTN_QB, n[b] - q);
                e[2] = p0 + q;
                e[3] = p0;
                e[4] = slots[b];
                e[5] = e[6] = e[7] = 0;
            }
            f0 += n[b];
        }
        for (int q = nq; q < bound; q++)
            for (int k = 0; k < SNRVQ_ATTN_Q_INTS; k++)
                aq[(size_t)SNRVQ_ATTN_Q_INTS * q + k] = 0;
        m.attn_q = dm + o.attn;
        m.n_qblocks = tile_bound ? bound : nq;
    }
    MetaLayout out;
    out.total = o.total;
    out.m = m;
    return out;
}

// The step's metadata copy from hp on stream s.
int enqueue_meta_copy(codec *c, const MetaLayout &ml, const int32_t *hp, hipStream_t s)
{
    return timed(c, "h2d_meta", (int64_t)ml.total * 4, s, [&] {
        return hipMemcpyAsync(c->meta_now, hp, ml.total * 4, hipMemcpyHostToDevice, s);
    });
}

// The step's kernels on stream s (reading the metadata already copied).
// Only asynchronous calls and no memset nodes, so that a graph can capture it.
int enqueue_kernels(codec *c, int B, int F, const MetaLayout &ml, float *pcm, hipStream_t s)
{
    const codec_cfg &g = c->cfg;
    const StepMeta &m = ml.m;
    int rc = CODEC_OK;

    // the gather and the halo fill of every layer share one launch
    rc = timed(c, "rvq_gather", F, s, [&] {
        return launch_rvq_gather_fill(c->cb, c->cb_dtype, m.codes, F, g.K, g.E, g.d_cb, c->dz,
                                      c->fold ? 6 : 0, c->fold ? 1 : 0, c->z, c->dtype,
                                      c->bad_codes, c->halo, c->state, m, B, s);
    });
    if (rc)
        return rc;

    // the codebook-space projection is folded into the next layer: the input
    // conv (decoders without a transformer) or the transformer's input projection
    ConvArgs a;
    if (g.tf_layers && (rc = enqueue_transformer(c, B, F, m, s)))
        return rc;

    a = conv_args(c, c->in_conv, c->fold ? c->z : c->u_ext, 6, 1, F, m);
    a.out16 = c->aT[0];
    a.out_H = 1;
    set_act(c, a, c->a_stage[0]);
    if ((rc = run_conv(c, "in_conv", a, s)))
        return rc;

    char nm[64];
    for (int i = 0; i < c->S; i++) {
        int ri = c->rate[i], ro = c->rate[i + 1];
        if (c->fuse_T[i]) {
            if ((rc = enqueue_fused_stage(c, i, F, m, pcm, s)))
                return rc;
            continue;
        }
        a = conv_args(c, c->convT[i], c->aT[i], 1, ri, F * ri, m);
        a.out32 = c->x;
        a.out16 = c->a1[i];
        a.out_H = 6;
        set_act(c, a, c->a_ru1[i][0]);
        snprintf(nm, sizeof nm, "s%d.convT", i);
        const bool split = !c->fusable[i];
        if ((rc = run_conv(c, nm, a, s, split)))
            return rc;
        for (int j = 0; j < 2; j++) {
            void *in = j == 0 ? c->a1[i] : c->a2[i];
            int inH = 6 * RU_DIL[j];
            // (with enough rows to fill the GPU without splitting K)
            if (!c->fusable[i] && ru_gemm_supported(c->ch[i + 1], c->dtype) &&
                (int64_t)F * ro >= 64LL * c->n_cu) {
                // the whole residual unit in one launch: h never leaves the chip
                a = conv_args(c, c->conv7[i][j], in, inH, ro, F * ro, m);
                a.W1 = c->conv1[i][j].Wt;
                a.bias7 = c->conv7[i][j].bias;
                a.act7 = c->cfg.act == CODEC_ACT_ELU ? ACT_ELU : ACT_SNAKE;
                a.alpha7 = c->a_ru2[i][j].alpha;
                a.inv_alpha7 = c->a_ru2[i][j].ialpha;
                a.bias = c->conv1[i][j].bias;
                a.res = c->x;
                if (j == 0) {
                    a.out32 = c->x;  // in place: each element is read then written by one thread
                    a.out16 = c->a2[i];
                    a.out_H = 18;
                    set_act(c, a, c->a_ru1[i][1]);
                } else if (i + 1 < c->S) {
                    a.out16 = c->aT[i + 1];
                    a.out_H = 1;
                    set_act(c, a, c->a_stage[i + 1]);
                } else {
                    a.out16 = c->a_outb;
                    a.out_H = 6;
                    set_act(c, a, c->a_out);
                }
                snprintf(nm, sizeof nm, "s%d.ru%d", i, j);
                if ((rc = timed(c, nm, (int64_t)a.M, s, [&] { return launch_ru_gemm(a, c->n_cu, s); })))
                    return rc;
                continue;
            }
            a = conv_args(c, c->conv7[i][j], in, inH, ro, F * ro, m);
            a.out16 = c->h;
            a.out_H = 0;
            set_act(c, a, c->a_ru2[i][j]);
            snprintf(nm, sizeof nm, "s%d.ru%d.conv7", i, j);
            if ((rc = run_conv(c, nm, a, s, split)))
                return rc;
            a = conv_args(c, c->conv1[i][j], c->h, 0, ro, F * ro, m);
            a.res = c->x;
            if (j == 0) {
                a.out32 = c->x;  // in place: each element is read then written by one thread
                a.out16 = c->a2[i];
                a.out_H = 18;
                set_act(c, a, c->a_ru1[i][1]);
            } else if (i + 1 < c->S) {
                a.out16 = c->aT[i + 1];
                a.out_H = 1;
                set_act(c, a, c->a_stage[i + 1]);
            } else {
                a.out16 = c->a_outb;
                a.out_H = 6;
                set_act(c, a, c->a_out);
            }
            snprintf(nm, sizeof nm, "s%d.ru%d.conv1", i, j);
            if ((rc = run_conv(c, nm, a, s, split)))
                return rc;
        }
    }
    if (!c->fuse_T[c->S - 1]) {
        rc = timed(c, "final_conv", (int64_t)F * c->hop, s, [&] {
            return launch_final_conv(c->a_outb, c->dtype, 6, c->ch[c->S], c->hop, c->out_w,
                                     c->out_b, g.final_tanh, m.frame_stream, F * c->hop, pcm, s);
        });
        if (rc)
            return rc;
    }
    if (!c->fuse_T[c->S - 1]) {  // else the fused last stage saved the halos
        rc = timed(c, "halo_save", B, s,
                   [&] { return launch_halo_save(c->halo_save, c->state, m, B, s); });
        if (rc)
            return rc;
    }
    c->last_meta = m;
    c->lastF = F;
    c->lastB = B;
    return CODEC_OK;
}

void graph_free(codec::GraphEntry &e)
{
    if (e.done)
        (void)hipEventSynchronize(e.done);
    if (e.exec)
        (void)hipGraphExecDestroy(e.exec);
    if (e.done)
        (void)hipEventDestroy(e.done);
    e = codec::GraphEntry{};
}

// Host bookkeeping of a step that has been enqueued.
void step_done(codec *c, int B, const int *slots, const int32_t *n)
{
    for (int b = 0; b < B; b++) {
        c->slot_pos[slots[b]] += n[b];
        c->slot_fresh[slots[b]] = 0;
    }
}

// Waits for (and releases) the oldest in-flight span of the staging arena.
int arena_retire_oldest(codec *c)
{
    const codec::Span sp = c->inflight.front();
    c->inflight.pop_front();
    c->ev_free.push_back(sp.ev);
    HIPCHK(c, hipEventSynchronize(sp.ev));
    return CODEC_OK;
}

// A span of `bytes` of the staging arena for the next step's metadata (the
// arena holds the largest step several times over).  Spans are taken in ring
// order; the in-flight spans that the new one overlaps are waited for first.
int arena_take(codec *c, size_t bytes, int32_t **out)
{
    bytes = (bytes + 255) & ~(size_t)255;
    if (bytes > c->arena_cap)
        return fail(c, CODEC_ETOOBIG, "step metadata of %zu bytes exceeds the staging arena",
                    bytes);
    // The in-flight spans form one circular run ending at the head, oldest
    // first, so the spans a new span overlaps are always the oldest ones --
    // except when wrapping to 0 while the run itself wraps: its oldest spans
    // then lie in [head, cap), which this lap gives up, and are retired first.
    const size_t at = c->arena_head + bytes <= c->arena_cap ? c->arena_head : 0;
    if (at == 0 && c->arena_head > 0)
        while (!c->inflight.empty() && c->inflight.front().begin >= c->arena_head) {
            int rc = arena_retire_oldest(c);
            if (rc)
                return rc;
        }
    while (!c->inflight.empty()) {
        const codec::Span &sp = c->inflight.front();
        const bool overlap = sp.begin < at + bytes && at < sp.end;
        if (!overlap && !c->ev_free.empty())
            break;
        int rc = arena_retire_oldest(c);
        if (rc)
            return rc;
    }
    *out = (int32_t *)(c->arena + at);
    c->arena_head = at + bytes;
    return CODEC_OK;
}

// Marks the span just taken as in flight until the work enqueued so far on s
// is done.  Recorded after the step's last launch (not right after the copy
// that reads the span): the record also hands the step's launches to the
// device, so a later wait on it never finds them still queued on the host.
int arena_commit(codec *c, const int32_t *hp, size_t bytes, hipStream_t s)
{
    bytes = (bytes + 255) & ~(size_t)255;
    hipEvent_t ev = c->ev_free.back();
    HIPCHK(c, hipEventRecord(ev, s));
    c->ev_free.pop_back();
    const size_t begin = (size_t)((const char *)hp - c->arena);
    c->inflight.push_back({begin, begin + bytes, ev});
    return CODEC_OK;
}

int enqueue_step(codec *c, int B, const int *slots, const int32_t *n, const int32_t *codes,
                 float *pcm, hipStream_t s, bool codes_on_device = false)
{
    int F = 0;
    for (int b = 0; b < B; b++)
        F += n[b];
    // batch assembly into the pinned staging arena, one H2D copy
    const size_t bytes = meta_offsets(c, B, F, codes_on_device).total * 4;
    int32_t *hp = nullptr;
    int rc = arena_take(c, bytes, &hp);
    if (rc)
        return rc;
    MetaLayout ml = fill_meta(c, hp, B, slots, n, codes, codes_on_device);
    if ((rc = enqueue_meta_copy(c, ml, hp, s)))
        return rc;
    if ((rc = enqueue_kernels(c, B, F, ml, pcm, s)))
        return rc;
    if ((rc = arena_commit(c, hp, bytes, s)))
        return rc;
    step_done(c, B, slots, n);
    return CODEC_OK;
}

// ---- static scratch of decode_chunk_device_noalloc ----
// One array per GPU the library runs on, held until the process ends: the
// step metadata in the first SNRVQ_SCRATCH_META_BYTES, the split-K partials
// after it.  Host code never uses the array's name as an address: the device
// address of each GPU's copy is looked up once per device (with that device
// current) and kept in g_scratch_dev.
constexpr size_t SNRVQ_SCRATCH_BYTES = (size_t)32 << 20;
constexpr size_t SNRVQ_SCRATCH_META_BYTES = (size_t)1 << 20;
constexpr int SNRVQ_MAX_DEVICES = 64;
void *g_scratch_dev[SNRVQ_MAX_DEVICES];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) char scratch[SNRVQ_SCRATCH_BYTES];

namespace {

// Resolves this codec's device's scratch address (once per device).
int scratch_setup(codec *c)
{
    if (c->dev < 0 || c->dev >= SNRVQ_MAX_DEVICES)
        return fail(c, CODEC_EINVAL, "device %d: the no-allocation scratch covers devices 0..%d",
                    c->dev, SNRVQ_MAX_DEVICES - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[c->dev])
        return CODEC_OK;
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
        return fail(c, CODEC_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", c->dev,
                    hipGetErrorString(e));
    g_scratch_dev[c->dev] = ptr;
    return CODEC_OK;
}

int check_cfg(const codec_cfg *g, int *ch, int *hop)
{
    if (g->K < 1 || g->K > 64 || g->E < 1 || g->d_cb < 1 || g->d_lat < 1)
        return set_err(nullptr, CODEC_EINVAL, "cfg: K=%d (1..64), E=%d, d_cb=%d, d_lat=%d", g->K,
                       g->E, g->d_cb, g->d_lat);
    if (g->n_stages < 1 || g->n_stages > CODEC_MAX_STAGES)
        return set_err(nullptr, CODEC_EINVAL, "cfg: n_stages=%d (1..%d)", g->n_stages,
                       CODEC_MAX_STAGES);
    if (g->act != CODEC_ACT_SNAKE && g->act != CODEC_ACT_ELU)
        return set_err(nullptr, CODEC_EINVAL, "cfg: act=%d", g->act);
    if (g->weight_dtype != CODEC_DTYPE_F32 && g->weight_dtype != CODEC_DTYPE_BF16)
        return set_err(nullptr, CODEC_EINVAL, "cfg: weight_dtype=%d (F32 or BF16)",
                       g->weight_dtype);
    if (g->max_streams < 1 || g->max_frames_per_call < 1)
        return set_err(nullptr, CODEC_EINVAL, "cfg: max_streams=%d, max_frames_per_call=%d",
                       g->max_streams, g->max_frames_per_call);
    int gran = g->weight_dtype == CODEC_DTYPE_BF16 ? 32 : 16;
    if (g->tf_layers < 0 || g->tf_layers > 16)
        return set_err(nullptr, CODEC_EINVAL, "cfg: tf_layers=%d (0..16)", g->tf_layers);
    if (g->tf_layers > 0) {
        if (g->tf_head_dim != 64 || g->tf_heads < 1 || g->tf_heads > 64)
            return set_err(nullptr, CODEC_EINVAL,
                           "cfg: tf_heads=%d tf_head_dim=%d (head_dim must be 64)", g->tf_heads,
                           g->tf_head_dim);
        if (g->tf_window < 1 || g->tf_window > SNRVQ_MAX_WINDOW)
            return set_err(nullptr, CODEC_EINVAL, "cfg: tf_window=%d (1..%d)", g->tf_window,
                           SNRVQ_MAX_WINDOW);
        if (g->tf_mlp < gran || g->tf_mlp % gran)
            return set_err(nullptr, CODEC_EINVAL, "cfg: tf_mlp=%d is not a multiple of %d",
                           g->tf_mlp, gran);
    }
    ch[0] = g->d_lat;
    *hop = 1;
    for (int i = 0; i < g->n_stages; i++) {
        if (g->strides[i] < 1 || g->strides[i] > 64)
            return set_err(nullptr, CODEC_EINVAL, "cfg: strides[%d]=%d", i, g->strides[i]);
        if (ch[i] % 2)
            return set_err(nullptr, CODEC_EINVAL, "cfg: channel width %d of stage %d is odd",
                           ch[i], i);
        ch[i + 1] = ch[i] / 2;
        *hop *= g->strides[i];
    }
    for (int i = 0; i <= g->n_stages; i++)
        if (ch[i] % gran)
            return set_err(nullptr, CODEC_EINVAL,
                           "cfg: channel width %d is not a multiple of %d (the MFMA K step of "
                           "this weight dtype)",
                           ch[i], gran);
    if (g->d_cb % gran)
        return set_err(nullptr, CODEC_EINVAL, "cfg: d_cb=%d is not a multiple of %d", g->d_cb,
                       gran);
    if ((int64_t)(g->max_frames_per_call + kGraphPadMax) * *hop >= (int64_t)1 << 31)
        return set_err(nullptr, CODEC_EINVAL, "cfg: max_frames_per_call * hop overflows int32");
    return CODEC_OK;
}

}  // namespace

// ============================================================================
extern "C" {

const char *codec_last_error(const codec_t *c)
{
    if (c)
        return c->err.c_str();
    return g_err.c_str();
}

int codec_open(const codec_tensor *weights, int32_t n_weights, const codec_cfg *cfg,
               codec_t **out)
{
    if (!out)
        return set_err(nullptr, CODEC_EINVAL, "codec_open: out is NULL");
    *out = nullptr;
    if (!cfg || (!weights && n_weights > 0) || n_weights < 0)
        return set_err(nullptr, CODEC_EINVAL, "codec_open: null cfg or weights");
    int ch[CODEC_MAX_STAGES + 1];
    int hop = 1;
    int rc = check_cfg(cfg, ch, &hop);
    if (rc)
        return rc;

    // ---- weight manifest: every canonical parameter exactly once ----
    std::vector<ParamSpec> specs = param_specs(*cfg, ch);
    std::unordered_map<std::string, int> by_name;
    for (int i = 0; i < n_weights; i++) {
        const codec_tensor &t = weights[i];
        if (!t.name || !t.host_data)
            return set_err(nullptr, CODEC_EINVAL, "weights[%d]: null name or data", i);
        if (by_name.count(t.name))
            return set_err(nullptr, CODEC_EINVAL, "weights: '%s' given twice", t.name);
        by_name[t.name] = i;
    }
    for (const ParamSpec &p : specs) {
        auto it = by_name.find(p.name);
        if (it == by_name.end())
            return set_err(nullptr, CODEC_EINVAL, "weights: '%s' missing", p.name.c_str());
        const codec_tensor &t = weights[it->second];
        bool ok = t.ndim == (int)p.shape.size();
        for (int d = 0; ok && d < t.ndim; d++)
            ok = t.shape[d] == p.shape[d];
        if (!ok) {
            std::string want, got;
            for (auto v : p.shape)
                want += std::to_string(v) + ",";
            for (int d = 0; d < t.ndim && d < 4; d++)
                got += std::to_string(t.shape[d]) + ",";
            return set_err(nullptr, CODEC_EINVAL, "weights: '%s' has shape (%s), expected (%s)",
                           p.name.c_str(), got.c_str(), want.c_str());
        }
        if (t.dtype != cfg->weight_dtype)
            return set_err(nullptr, CODEC_EINVAL, "weights: '%s' dtype %d, cfg weight_dtype %d",
                           p.name.c_str(), t.dtype, cfg->weight_dtype);
    }
    if ((size_t)n_weights != specs.size()) {
        std::unordered_set<std::string> known;
        for (auto &p : specs)
            known.insert(p.name);
        for (int i = 0; i < n_weights; i++)
            if (!known.count(weights[i].name))
                return set_err(nullptr, CODEC_EINVAL, "weights: unknown parameter '%s'",
                               weights[i].name);
    }

    // bf16 weights run as fp16 MFMA operands: a weight beyond fp16's finite
    // range, or codebook entries whose K-term sum could exceed it (the RVQ sum
    // is stored in fp16), cannot be represented; reject them here
    if (cfg->weight_dtype == CODEC_DTYPE_BF16) {
        const float kF16Max = 65504.f;
        auto bf16 = [](uint16_t b) {
            uint32_t u = (uint32_t)b << 16;
            float f;
            memcpy(&f, &u, 4);
            return f;
        };
        std::vector<float> cb_sum((size_t)cfg->d_cb, 0.f);
        for (const ParamSpec &p : specs) {
            const codec_tensor &t = weights[by_name[p.name]];
            int64_t nel = 1;
            for (auto v : p.shape)
                nel *= v;
            const uint16_t *b = (const uint16_t *)t.host_data;
            const bool codebook = p.name.rfind("rvq.codebook.", 0) == 0;
            const bool operand = p.name.size() > 7 &&
                                 p.name.compare(p.name.size() - 7, 7, ".weight") == 0 &&
                                 p.name.find(".ln") == std::string::npos;
            if (codebook) {
                std::vector<float> mx((size_t)cfg->d_cb, 0.f);
                for (int64_t i = 0; i < nel; i++) {
                    const float v = std::fabs(bf16(b[i]));
                    float &m = mx[(size_t)(i % cfg->d_cb)];
                    m = std::isnan(v) || v > m ? v : m;
                }
                for (int d = 0; d < cfg->d_cb; d++)
                    cb_sum[(size_t)d] += mx[(size_t)d];
            } else if (operand) {
                for (int64_t i = 0; i < nel; i++)
                    if (!(std::fabs(bf16(b[i])) <= kF16Max))
                        return set_err(nullptr, CODEC_EINVAL,
                                       "weights: '%s'[%lld] = %g is outside the fp16 range of "
                                       "the compute operands (|w| <= 65504)",
                                       p.name.c_str(), (long long)i, (double)bf16(b[i]));
            }
        }
        for (int d = 0; d < cfg->d_cb; d++)
            if (!(cb_sum[(size_t)d] <= kF16Max))
                return set_err(nullptr, CODEC_EINVAL,
                               "weights: codebook column %d can sum to %g over the %d codebooks, "
                               "beyond the fp16 range of the stored RVQ sum (65504)",
                               d, (double)cb_sum[(size_t)d], cfg->K);
    }

    int dev = 0;
    int ndev = 0;
    hipError_t he = hipGetDeviceCount(&ndev);
    if (he != hipSuccess || ndev < 1)
        return set_err(nullptr, CODEC_EHIP, "codec_open: no HIP device (%s)",
                       hipGetErrorString(he));
    he = hipGetDevice(&dev);
    if (he != hipSuccess)
        return set_err(nullptr, CODEC_EHIP, "codec_open: hipGetDevice: %s",
                       hipGetErrorString(he));

    codec *c = new codec();
    c->cfg = *cfg;
    c->dev = dev;
    {
        int ncu = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            ncu > 0)
            c->n_cu = ncu;
    }
    c->dtype = cfg->weight_dtype == CODEC_DTYPE_BF16 ? 1 : 0;
    c->esz = c->dtype ? 2 : 4;
    c->S = cfg->n_stages;
    c->hop = hop;
    memcpy(c->ch, ch, sizeof ch);
    c->rate[0] = 1;
    for (int i = 0; i < c->S; i++)
        c->rate[i + 1] = c->rate[i] * cfg->strides[i];
    c->left_ctx = left_context_frames(*cfg, hop);
    c->maxF = cfg->max_frames_per_call;
    c->maxB = cfg->max_streams;

    auto W = [&](const std::string &name) {
        const codec_tensor &t = weights[by_name[name]];
        int64_t n = 1;
        for (int d = 0; d < t.ndim; d++)
            n *= t.shape[d];
        return host_f32(t, n);
    };
    auto cleanup_fail = [&](int code) {
        std::string msg = c->err;
        codec_close(c);
        g_err = msg;
        return code;
    };
    char nm[128];
    const codec_cfg &g = *cfg;

    // ---- codebooks: one contiguous [K][E][d_cb] array in the given dtype ----
    {
        size_t per = (size_t)g.E * g.d_cb;
        c->cb_dtype = c->dtype;  // bf16 tables for the fp16 path, fp32 tables otherwise
        size_t esz = c->cb_dtype ? 2 : 4;
        if ((rc = dev_alloc(c, &c->cb, per * g.K * esz, &c->weight_bytes)))
            return cleanup_fail(rc);
        for (int k = 0; k < g.K; k++) {
            snprintf(nm, sizeof nm, "rvq.codebook.%d", k);
            const codec_tensor &t = weights[by_name[nm]];
            hipError_t e = hipMemcpy((char *)c->cb + per * esz * k, t.host_data, per * esz,
                                     hipMemcpyHostToDevice);
            if (e != hipSuccess) {
                fail(c, CODEC_EHIP, "codebook upload: %s", hipGetErrorString(e));
                return cleanup_fail(CODEC_EHIP);
            }
        }
    }
    // ---- dense layers, repacked K-major for the implicit GEMM ----
    c->fold = g.tf_layers == 0;
    c->dz = c->fold ? (g.d_cb + 1 + (c->dtype ? 63 : 15)) / (c->dtype ? 64 : 16) * (c->dtype ? 64 : 16)
                    : g.d_cb;
    if (!c->fold &&
        (rc = make_lin(c, W("rvq.proj.weight"), W("rvq.proj.bias"), g.d_lat, g.d_lat, g.d_cb, 1,
                       1, 1, &c->proj)))
        return cleanup_fail(rc);
    if (g.tf_layers) {
        const int dm = g.tf_heads * g.tf_head_dim, mlp = g.tf_mlp;
        c->dm = dm;
        // the input projection runs on the RVQ sum directly, the codebook-space
        // projection composed into it (c->proj stays for latent captures)
        std::vector<float> wf, bf;
        fold_tf_input(W("tf.in_proj.weight"), W("tf.in_proj.bias"), W("rvq.proj.weight"),
                      W("rvq.proj.bias"), dm, g.d_lat, g.d_cb, wf, bf);
        if ((rc = make_lin(c, wf, bf, dm, dm, g.d_cb, 1, 1, 1, &c->tf_in)))
            return cleanup_fail(rc);
        for (int l = 0; l < g.tf_layers; l++) {
            std::string p = "tf.layer." + std::to_string(l) + ".";
            if ((rc = upload_f32(c, W(p + "ln1.weight"), &c->ln1_g[l])) ||
                (rc = upload_f32(c, W(p + "ln1.bias"), &c->ln1_b[l])) ||
                (rc = upload_f32(c, W(p + "ln2.weight"), &c->ln2_g[l])) ||
                (rc = upload_f32(c, W(p + "ln2.bias"), &c->ln2_b[l])) ||
                (rc = make_lin(c, W(p + "attn.qkv.weight"), W(p + "attn.qkv.bias"), 3 * dm,
                               3 * dm, dm, 1, 1, 1, &c->tf_qkv[l])) ||
                (rc = make_lin(c, W(p + "attn.out.weight"), W(p + "attn.out.bias"), dm, dm, dm, 1,
                               1, 1, &c->tf_o[l])) ||
                (rc = make_lin(c, W(p + "mlp.fc1.weight"), W(p + "mlp.fc1.bias"), mlp, mlp, dm,
                               1, 1, 1, &c->tf_fc1[l])) ||
                (rc = make_lin(c, W(p + "mlp.fc2.weight"), W(p + "mlp.fc2.bias"), dm, dm, mlp, 1,
                               1, 1, &c->tf_fc2[l])))
                return cleanup_fail(rc);
        }
        if ((rc = upload_f32(c, W("tf.ln_f.weight"), &c->lnf_g)) ||
            (rc = upload_f32(c, W("tf.ln_f.bias"), &c->lnf_b)) ||
            (rc = make_lin(c, W("tf.out_proj.weight"), W("tf.out_proj.bias"), g.d_lat, g.d_lat,
                           dm, 1, 1, 1, &c->tf_out)))
            return cleanup_fail(rc);
        std::vector<double> inv(g.tf_head_dim / 2);
        for (size_t i = 0; i < inv.size(); i++)
            inv[i] = std::pow(10000.0, -(2.0 * (double)i) / g.tf_head_dim);
        if ((rc = dev_alloc(c, (void **)&c->inv_freq, inv.size() * 8, &c->weight_bytes)))
            return cleanup_fail(rc);
        HIPCHK(c, hipMemcpy(c->inv_freq, inv.data(), inv.size() * 8, hipMemcpyHostToDevice));
    }
    if (c->fold) {
        std::vector<float> wc =
            fold_projection(W("dec.in_conv.weight"), W("rvq.proj.weight"), W("rvq.proj.bias"),
                            ch[0], g.d_lat, g.d_cb, c->dz);
        if ((rc = make_lin(c, wc, W("dec.in_conv.bias"), ch[0], ch[0], c->dz, 7, 1, 1,
                           &c->in_conv)))
            return cleanup_fail(rc);
    } else if ((rc = make_lin(c, pack_conv(W("dec.in_conv.weight"), ch[0], g.d_lat, 7),
                              W("dec.in_conv.bias"), ch[0], ch[0], g.d_lat, 7, 1, 1,
                              &c->in_conv))) {
        return cleanup_fail(rc);
    }
    for (int i = 0; i < c->S; i++) {
        int ci = ch[i], co = ch[i + 1], s = g.strides[i];
        snprintf(nm, sizeof nm, "dec.stage.%d.snake.alpha", i);
        if ((rc = upload_act(c, W(nm), &c->a_stage[i])))
            return cleanup_fail(rc);
        snprintf(nm, sizeof nm, "dec.stage.%d.convT.weight", i);
        std::vector<float> wt = pack_convT(W(nm), ci, co, s);
        snprintf(nm, sizeof nm, "dec.stage.%d.convT.bias", i);
        if ((rc = make_lin(c, wt, W(nm), s * co, co, ci, 2, 1, s, &c->convT[i])))
            return cleanup_fail(rc);
        for (int j = 0; j < 2; j++) {
            std::string p = "dec.stage." + std::to_string(i) + ".ru." + std::to_string(j) + ".";
            if ((rc = upload_act(c, W(p + "snake1.alpha"), &c->a_ru1[i][j])))
                return cleanup_fail(rc);
            if ((rc = upload_act(c, W(p + "snake2.alpha"), &c->a_ru2[i][j])))
                return cleanup_fail(rc);
            if ((rc = make_lin(c, pack_conv(W(p + "conv7.weight"), co, co, 7), W(p + "conv7.bias"),
                               co, co, co, 7, RU_DIL[j], 1, &c->conv7[i][j])))
                return cleanup_fail(rc);
            if ((rc = make_lin(c, W(p + "conv1.weight"), W(p + "conv1.bias"), co, co, co, 1, 1, 1,
                               &c->conv1[i][j])))
                return cleanup_fail(rc);
        }
    }
    if ((rc = upload_act(c, W("dec.out.snake.alpha"), &c->a_out)))
        return cleanup_fail(rc);
    if ((rc = upload_f32(c, W("dec.out.conv.weight"), &c->out_w)))
        return cleanup_fail(rc);
    c->out_b = W("dec.out.conv.bias")[0];

    // ---- workspace for max_frames_per_call frames of max_streams streams,
    // plus a graph step's pad frames and pad stream ----
    c->allocF = c->maxF + kGraphPadMax;
    c->allocB = c->maxB + 1;
    c->pad_slot = c->maxB;
    const size_t F = (size_t)c->allocF, B = (size_t)c->allocB, es = (size_t)c->esz;
    int64_t *ws = &c->workspace_bytes;
    if (c->fold) {  // extended rows of dz values: the input conv's operand
        if ((rc = dev_alloc(c, &c->z, (B * 6 + F) * c->dz * es, ws)))
            return cleanup_fail(rc);
    } else {
        if ((rc = dev_alloc(c, &c->z, F * g.d_cb * es, ws)))
            return cleanup_fail(rc);
        if ((rc = dev_alloc(c, &c->u_ext, (B * 6 + F) * g.d_lat * es, ws)))
            return cleanup_fail(rc);
    }
    size_t hmax = 0;
    for (int i = 0; i < c->S; i++) {
        size_t ro = (size_t)c->rate[i + 1], co = (size_t)ch[i + 1];
        if ((rc = dev_alloc(c, &c->aT[i], (B * 1 + F * c->rate[i]) * ch[i] * es, ws)))
            return cleanup_fail(rc);
        if ((rc = dev_alloc(c, &c->a1[i], (B * 6 + F * ro) * co * es, ws)))
            return cleanup_fail(rc);
        if ((rc = dev_alloc(c, &c->a2[i], (B * 18 + F * ro) * co * es, ws)))
            return cleanup_fail(rc);
        hmax = std::max(hmax, F * ro * co);
    }
    if ((rc = dev_alloc(c, &c->h, hmax * es, ws)))
        return cleanup_fail(rc);
    if ((rc = dev_alloc(c, (void **)&c->x, hmax * 4, ws)))
        return cleanup_fail(rc);
    if ((rc = dev_alloc(c, &c->a_outb, (B * 6 + F * hop) * ch[c->S] * es, ws)))
        return cleanup_fail(rc);
    if (g.tf_layers) {
        const size_t dm = c->dm, W1 = g.tf_window - 1;
        if ((rc = dev_alloc(c, &c->u16, F * g.d_lat * es, ws)) ||
            (rc = dev_alloc(c, &c->a16, F * dm * es, ws)) ||
            (rc = dev_alloc(c, &c->att16, F * dm * es, ws)) ||
            (rc = dev_alloc(c, &c->f16, F * g.tf_mlp * es, ws)) ||
            (rc = dev_alloc(c, (void **)&c->h32, F * dm * 4, ws)) ||
            (rc = dev_alloc(c, (void **)&c->qkv32, F * 3 * dm * 4, ws)) ||
            (rc = dev_alloc(c, (void **)&c->rot, F * g.tf_head_dim * 4, ws)) ||
            (rc = dev_alloc(c, (void **)&c->kring, B * g.tf_layers * (W1 ? W1 : 1) * dm * 4, ws)) ||
            (rc = dev_alloc(c, (void **)&c->vring, B * g.tf_layers * (W1 ? W1 : 1) * dm * 4, ws)))
            return cleanup_fail(rc);
    }
    if ((rc = dev_alloc(c, (void **)&c->pcm_scratch, F * hop * 4, ws)))
        return cleanup_fail(rc);
    c->splitk_cap = kSplitKCap;
    if ((rc = dev_alloc(c, (void **)&c->splitk_ws, (size_t)c->splitk_cap * 4, ws)))
        return cleanup_fail(rc);

    // ---- halo table and state slots ----
    HaloTable &t = c->halo;
    t.elem_bytes = c->esz;
    int64_t off = 0;
    auto add = [&](void *ext, int H, int C, int rate) {
        HaloLayer &L = t.l[t.n++];
        L.ext = ext;
        L.H = H;
        L.C = C;
        L.rate = rate;
        L.state_off = off;
        off += (int64_t)H * C;
    };
    if (c->fold)
        add(c->z, 6, c->dz, 1);
    else
        add(c->u_ext, 6, g.d_lat, 1);
    for (int i = 0; i < c->S; i++) {
        add(c->aT[i], 1, ch[i], c->rate[i]);
        c->off_a1[i] = off;
        add(c->a1[i], 6, ch[i + 1], c->rate[i + 1]);
        c->off_a2[i] = off;
        add(c->a2[i], 18, ch[i + 1], c->rate[i + 1]);
    }
    c->off_ao = off;
    add(c->a_outb, 6, ch[c->S], hop);
    c->slot_elems = off;
    t.slot_elems = off;
    // fused stages (fp16 path): their residual-unit and final-conv left
    // contexts are written by the stage kernel itself, not by the halo save
    for (int i = 0; i < c->S; i++) {
        const int T = (c->dtype && g.act == CODEC_ACT_SNAKE)
                          ? stage_fused_tile(ch[i + 1], g.strides[i], i == c->S - 1)
                          : 0;
        c->fusable[i] = T != 0;
        c->fuse_T[i] = (g.flags & CODEC_FLAG_PER_LAYER) || (g.flags & CODEC_FLAG_PER_LAYER_STAGE(i)) ? 0 : T;
    }
    HaloTable &sv = c->halo_save;
    sv.elem_bytes = t.elem_bytes;
    sv.slot_elems = t.slot_elems;
    for (int k = 0; k < t.n; k++) {
        const void *e = t.l[k].ext;
        bool skip = false;
        for (int i = 0; i < c->S; i++)
            if (c->fuse_T[i] && (e == c->a1[i] || e == c->a2[i] ||
                                 (i == c->S - 1 && e == c->a_outb)))
                skip = true;
        if (!skip)
            sv.l[sv.n++] = t.l[k];
    }
    if ((rc = dev_alloc(c, &c->state, (size_t)c->allocB * off * es, ws)))
        return cleanup_fail(rc);

    // ---- step metadata: device buffer + pinned staging arena ----
    c->meta_cap = round4(F * g.K) + round4(F) + round4(B + 1) + 3 * round4(B) +
                  CODEC_MAX_STAGES * round4(B + 1) +
                  (g.tf_layers ? round4(SNRVQ_ATTN_Q_INTS * (size_t)attn_qblock_bound(B, F)) : 0) + 4;
    if ((rc = dev_alloc(c, &c->meta_dev, c->meta_cap * 4, ws)))
        return cleanup_fail(rc);
    if ((rc = dev_alloc(c, (void **)&c->bad_codes, sizeof(unsigned long long), ws)))
        return cleanup_fail(rc);
    HIPCHK(c, hipMemset(c->bad_codes, 0, sizeof(unsigned long long)));
    // staging arena: the largest step's metadata 16 times over, at least
    // 16 MiB; events for up to 1024 steps in flight
    c->arena_cap = std::max<size_t>((size_t)16 << 20, 16 * ((c->meta_cap * 4 + 255) & ~(size_t)255));
    {
        hipError_t e = hipHostMalloc((void **)&c->arena, c->arena_cap, hipHostMallocDefault);
        if (e != hipSuccess) {
            c->arena = nullptr;
            fail(c, CODEC_ENOMEM, "hipHostMalloc of the %zu-byte staging arena: %s",
                 c->arena_cap, hipGetErrorString(e));
            return cleanup_fail(CODEC_ENOMEM);
        }
        for (int i = 0; i < 1024; i++) {
            hipEvent_t ev = nullptr;
            e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
            if (e != hipSuccess) {
                fail(c, CODEC_EHIP, "hipEventCreate: %s", hipGetErrorString(e));
                return cleanup_fail(CODEC_EHIP);
            }
            c->ev_free.push_back(ev);
        }
    }

    c->slot_pos.assign(c->allocB, 0);
    c->slot_fresh.assign(c->allocB, 1);
    c->partial_now = c->splitk_ws;
    c->partial_cap_now = c->splitk_cap;
    c->meta_now = c->meta_dev;
    if ((rc = scratch_setup(c)))
        return cleanup_fail(rc);
    for (int i = c->maxB - 1; i >= 0; i--)
        c->free_slots.push_back(i);
    *out = c;
    return CODEC_OK;
}

int codec_close(codec_t *c)
{
    if (!c)
        return set_err(nullptr, CODEC_EINVAL, "codec_close: NULL codec");
    (void)hipDeviceSynchronize();
    for (auto &r : c->recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (auto e : c->ev_pool)
        (void)hipEventDestroy(e);
    for (auto &sp : c->inflight)
        (void)hipEventDestroy(sp.ev);
    for (auto e : c->ev_free)
        (void)hipEventDestroy(e);
    if (c->arena)
        (void)hipHostFree(c->arena);
    if (c->cap_stream)
        (void)hipStreamDestroy(c->cap_stream);
    for (auto &kv : c->graphs)
        graph_free(kv.second);
    for (void *p : c->allocs)
        (void)hipFree(p);
    delete c;
    return CODEC_OK;
}

int codec_info(const codec_t *c, codec_info_t *o)
{
    if (!c || !o)
        return set_err(nullptr, CODEC_EINVAL, "codec_info: NULL argument");
    memset(o, 0, sizeof *o);
    o->hop = c->hop;
    o->sample_rate = c->cfg.sample_rate;
    o->K = c->cfg.K;
    o->E = c->cfg.E;
    o->left_context_frames = c->left_ctx;
    o->max_streams = c->maxB;
    o->max_frames_per_call = c->maxF;
    o->open_streams = (int32_t)c->id2slot.size();
    o->compute_dtype = c->dtype ? CODEC_DTYPE_F16 : CODEC_DTYPE_F32;
    o->state_bytes_per_stream =
        c->slot_elems * c->esz +
        (c->cfg.tf_layers ? (int64_t)2 * c->cfg.tf_layers * (c->cfg.tf_window - 1) * c->dm * 4 : 0);
    o->weight_bytes = c->weight_bytes;
    o->workspace_bytes = c->workspace_bytes;
    o->graph_captures = c->graph_captures;
    o->graph_replays = c->graph_replays;
    return CODEC_OK;
}

int stream_open(codec_t *c, int32_t *id_out)
{
    if (!c || !id_out)
        return set_err(c ? &c->err : nullptr, CODEC_EINVAL, "stream_open: NULL argument");
    if (c->free_slots.empty())
        return fail(c, CODEC_ENOSLOT, "stream_open: all %d state slots are in use", c->maxB);
    if (c->next_id == INT32_MAX)
        return fail(c, CODEC_ENOSLOT, "stream_open: stream ids exhausted");
    int slot = c->free_slots.back();
    c->free_slots.pop_back();
    int32_t id = c->next_id++;
    c->id2slot[id] = slot;
    c->slot_pos[slot] = 0;
    c->slot_fresh[slot] = 1;
    *id_out = id;
    return CODEC_OK;
}

int stream_close(codec_t *c, int32_t id)
{
    if (!c)
        return set_err(nullptr, CODEC_EINVAL, "stream_close: NULL codec");
    auto it = c->id2slot.find(id);
    if (it == c->id2slot.end())
        return fail(c, CODEC_ESTREAM, "stream_close: stream %d is not open", id);
    c->free_slots.push_back(it->second);
    c->id2slot.erase(it);
    return CODEC_OK;
}

static int check_codes(codec *c, const int32_t *codes, int64_t F, const int32_t *ids,
                       const int32_t *n, int B)
{
    const int K = c->cfg.K, E = c->cfg.E;
    for (int64_t i = 0; i < F * K; i++) {
        uint32_t v = (uint32_t)codes[i];
        if (v >= (uint32_t)E) {
            int64_t f = i / K;
            int b = 0;
            int64_t acc = 0;
            while (b < B && acc + n[b] <= f)
                acc += n[b++];
            return fail(c, CODEC_ERANGE,
                        "code %d at stream %d frame %lld codebook %lld is outside [0, %d)",
                        codes[i], ids ? ids[b] : -1, (long long)(f - acc),
                        (long long)(i % K), E);
        }
    }
    return CODEC_OK;
}

static int check_step(codec_t *c, int32_t B, const int32_t *ids, const int32_t *n,
                      const int32_t *codes, float *pcm, int64_t pcm_capacity, bool on_device,
                      std::vector<int> &slots)
{
    if (B < 1 || !ids || !n || !codes || !pcm)
        return fail(c, CODEC_EINVAL,
                    "decode_chunk: B=%d (must be >= 1) and ids, n_frames, codes, pcm non-NULL", B);
    if (B > c->maxB)
        return fail(c, CODEC_ETOOBIG, "decode_chunk: B=%d exceeds max_streams=%d", B, c->maxB);
    int64_t F = 0;
    for (int b = 0; b < B; b++) {
        if (n[b] < 1)
            return fail(c, CODEC_EINVAL, "decode_chunk: n_frames[%d]=%d (must be >= 1)", b, n[b]);
        F += n[b];
    }
    slots.assign((size_t)B, 0);
    std::unordered_set<int32_t> seen;
    for (int b = 0; b < B; b++) {
        auto it = c->id2slot.find(ids[b]);
        if (it == c->id2slot.end())
            return fail(c, CODEC_ESTREAM, "decode_chunk: stream %d (index %d) is not open", ids[b],
                        b);
        if (!seen.insert(ids[b]).second)
            return fail(c, CODEC_EDUP, "decode_chunk: stream %d appears twice", ids[b]);
        slots[b] = it->second;
    }
    if (F > c->maxF)
        return fail(c, CODEC_ETOOBIG,
                    "decode_chunk: %lld frames in one call exceed max_frames_per_call=%d",
                    (long long)F, c->maxF);
    if (pcm_capacity < F * c->hop)
        return fail(c, CODEC_EINVAL, "decode_chunk: pcm capacity %lld < %lld samples",
                    (long long)pcm_capacity, (long long)(F * c->hop));
    if (on_device)
        return CODEC_OK;
    return check_codes(c, codes, F, ids, n, B);
}

int decode_chunk(codec_t *c, int32_t B, const int32_t *ids, const int32_t *n, const int32_t *codes,
                 float *pcm, int64_t pcm_capacity, codec_hip_stream stream)
{
    if (!c)
        return set_err(nullptr, CODEC_EINVAL, "decode_chunk: NULL codec");
    std::vector<int> slots;
    int rc = check_step(c, B, ids, n, codes, pcm, pcm_capacity, false, slots);
    if (rc)
        return rc;
    HIPCHK(c, hipSetDevice(c->dev));
    return enqueue_step(c, B, slots.data(), n, codes, pcm, (hipStream_t)stream);
}

int decode_chunk_device(codec_t *c, int32_t B, const int32_t *ids, const int32_t *n,
                        const int32_t *codes_dev, float *pcm, int64_t pcm_capacity,
                        codec_hip_stream stream)
{
    if (!c)
        return set_err(nullptr, CODEC_EINVAL, "decode_chunk_device: NULL codec");
    std::vector<int> slots;
    int rc = check_step(c, B, ids, n, codes_dev, pcm, pcm_capacity, true, slots);
    if (rc)
        return rc;
    HIPCHK(c, hipSetDevice(c->dev));
    return enqueue_step(c, B, slots.data(), n, codes_dev, pcm, (hipStream_t)stream, true);
}

#define SNRVQ_MAX_GRAPHS 64

// Frames a graph step of F frames is captured for: the next power of two up
// to kGraphPadMax frames, then the next multiple of kGraphPadMax.
static int graph_bucket(int F)
{
    if (F <= kGraphPadMax) {
        int b = 1;
        while (b < F)
            b <<= 1;
        return b;
    }
    return (F + kGraphPadMax - 1) / kGraphPadMax * kGraphPadMax;
}

int decode_chunk_graph(codec_t *c, int32_t B, const int32_t *ids, const int32_t *n,
                       const int32_t *codes, float *pcm, int64_t pcm_capacity,
                       codec_hip_stream stream)
{
    if (!c)
        return set_err(nullptr, CODEC_EINVAL, "decode_chunk_graph: NULL codec");
    std::vector<int> slots;
    int rc = check_step(c, B, ids, n, codes, pcm, pcm_capacity, false, slots);
    if (rc)
        return rc;
    HIPCHK(c, hipSetDevice(c->dev));
    hipStream_t s = (hipStream_t)stream;
    int F = 0;
    for (int b = 0; b < B; b++)
        F += n[b];
    // the graph's streams: the caller's, then the pad stream if the bucket
    // has frames to spare (fresh every step: zero state, position 0)
    const int Fb = graph_bucket(F), pad = Fb - F;
    std::vector<int> gslots(slots);
    std::vector<int32_t> gn(n, n + B);
    if (pad > 0) {
        gslots.push_back(c->pad_slot);
        gn.push_back(pad);
        c->slot_fresh[c->pad_slot] = 1;
        c->slot_pos[c->pad_slot] = 0;
    }
    const int Bt = (int)gslots.size();
    const std::pair<int, int> key{Bt, Fb};
    auto it = c->graphs.find(key);
    if (it == c->graphs.end()) {
        if (c->graphs.size() >= SNRVQ_MAX_GRAPHS) {  // evict the least recently used
            auto lru = c->graphs.begin();
            for (auto jt = c->graphs.begin(); jt != c->graphs.end(); ++jt)
                if (jt->second.last_use < lru->second.last_use)
                    lru = jt;
            graph_free(lru->second);
            c->graphs.erase(lru);
        }
        it = c->graphs.emplace(key, codec::GraphEntry{}).first;
    }
    codec::GraphEntry &e = it->second;
    e.last_use = ++c->graph_clock;

    // metadata through the codec's pinned staging arena, as for an eager step
    const size_t meta_bytes = meta_offsets(c, Bt, Fb, false).total * 4;
    int32_t *hp = nullptr;
    if ((rc = arena_take(c, meta_bytes, &hp)))
        return rc;
    MetaLayout ml = fill_meta(c, hp, Bt, gslots.data(), gn.data(), codes, false, F, true);
    if ((rc = enqueue_meta_copy(c, ml, hp, s)))
        return rc;

    if (!e.exec) {
        // capture on the codec's own stream (the caller's may be the null
        // stream, which cannot be captured); nothing runs during capture.
        // The PCM goes to the codec's buffer, so the graph does not depend
        // on the caller's pcm address.
        if (!c->cap_stream)
            HIPCHK(c, hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
        hipGraph_t graph = nullptr;
        c->capturing = true;
        hipError_t ce = hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal);
        if (ce != hipSuccess) {
            c->capturing = false;
            return fail(c, CODEC_EHIP, "decode_chunk_graph: capture failed: %s",
                        hipGetErrorString(ce));
        }
        rc = enqueue_kernels(c, Bt, Fb, ml, c->pcm_scratch, c->cap_stream);
        ce = hipStreamEndCapture(c->cap_stream, &graph);
        c->capturing = false;
        if (rc) {
            if (graph)
                (void)hipGraphDestroy(graph);
            return rc;
        }
        if (ce != hipSuccess)
            return fail(c, CODEC_EHIP, "decode_chunk_graph: capture failed: %s",
                        hipGetErrorString(ce));
        ce = hipGraphInstantiate(&e.exec, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (ce != hipSuccess) {
            e.exec = nullptr;
            return fail(c, CODEC_EHIP, "decode_chunk_graph: instantiate failed: %s",
                        hipGetErrorString(ce));
        }
        HIPCHK(c, hipEventCreateWithFlags(&e.done, hipEventDisableTiming));
        c->graph_captures++;
    } else {
        c->graph_replays++;
    }
    HIPCHK(c, hipGraphLaunch(e.exec, s));
    HIPCHK(c, hipEventRecord(e.done, s));
    HIPCHK(c, hipMemcpyAsync(pcm, c->pcm_scratch, sizeof(float) * (size_t)F * c->hop,
                             hipMemcpyDeviceToDevice, s));
    if ((rc = arena_commit(c, hp, meta_bytes, s)))
        return rc;
    step_done(c, B, slots.data(), n);
    c->last_meta = ml.m;  // the caller's streams are the first B of the graph's
    c->lastF = F;
    c->lastB = B;
    return CODEC_OK;
}

int decode_chunk_device_noalloc(codec_t *c, int32_t B, const int32_t *ids, const int32_t *n,
                                const int32_t *codes_dev, float *pcm, int64_t pcm_capacity,
                                codec_hip_stream stream)
{
    if (!c)
        return set_err(nullptr, CODEC_EINVAL, "decode_chunk_device_noalloc: NULL codec");
    std::vector<int> slots;
    int rc = check_step(c, B, ids, n, codes_dev, pcm, pcm_capacity, true, slots);
    if (rc)
        return rc;
    int F = 0;
    for (int b = 0; b < B; b++)
        F += n[b];
    const size_t meta_bytes = meta_offsets(c, B, F, true).total * 4;
    if (meta_bytes > SNRVQ_SCRATCH_META_BYTES)
        return fail(c, CODEC_ETOOBIG,
                    "decode_chunk_device_noalloc: the step's metadata takes %zu bytes, the "
                    "static scratch holds %zu",
                    meta_bytes, SNRVQ_SCRATCH_META_BYTES);
    void *base = c->dev >= 0 && c->dev < SNRVQ_MAX_DEVICES ? g_scratch_dev[c->dev] : nullptr;
    if (!base)
        return fail(c, CODEC_EHIP, "decode_chunk_device_noalloc: no scratch on device %d",
                    c->dev);
    HIPCHK(c, hipSetDevice(c->dev));
    c->meta_now = base;
    c->partial_now = (float *)((char *)base + SNRVQ_SCRATCH_META_BYTES);
    c->partial_cap_now = (long)((SNRVQ_SCRATCH_BYTES - SNRVQ_SCRATCH_META_BYTES) / sizeof(float));
    rc = enqueue_step(c, B, slots.data(), n, codes_dev, pcm, (hipStream_t)stream, true);
    c->meta_now = c->meta_dev;
    c->partial_now = c->splitk_ws;
    c->partial_cap_now = c->splitk_cap;
    return rc;
}

int codec_device_status(codec_t *c, int64_t *bad)
{
    if (!c || !bad)
        return set_err(c ? &c->err : nullptr, CODEC_EINVAL, "codec_device_status: NULL argument");
    HIPCHK(c, hipSetDevice(c->dev));
    HIPCHK(c, hipDeviceSynchronize());
    unsigned long long v = 0;
    HIPCHK(c, hipMemcpy(&v, c->bad_codes, sizeof v, hipMemcpyDeviceToHost));
    HIPCHK(c, hipMemset(c->bad_codes, 0, sizeof v));
    *bad = (int64_t)v;
    if (v)
        return fail(c, CODEC_ERANGE, "%llu out-of-range codes in device-resident steps", v);
    return CODEC_OK;
}

int stream_prefill(codec_t *c, int32_t id, const int32_t *codes, int32_t n,
                   codec_hip_stream stream)
{
    if (!c)
        return set_err(nullptr, CODEC_EINVAL, "stream_prefill: NULL codec");
    if (n < 0 || (n > 0 && !codes))
        return fail(c, CODEC_EINVAL, "stream_prefill: n=%d, codes=%p", n, (const void *)codes);
    auto it = c->id2slot.find(id);
    if (it == c->id2slot.end())
        return fail(c, CODEC_ESTREAM, "stream_prefill: stream %d is not open", id);
    int rc = check_codes(c, codes, n, &id, &n, 1);
    if (rc)
        return rc;
    HIPCHK(c, hipSetDevice(c->dev));
    int slot = it->second;
    for (int32_t at = 0; at < n;) {
        int32_t piece = std::min<int32_t>(n - at, c->maxF);
        rc = enqueue_step(c, 1, &slot, &piece, codes + (size_t)at * c->cfg.K, c->pcm_scratch,
                          (hipStream_t)stream);
        if (rc)
            return rc;
        at += piece;
    }
    return CODEC_OK;
}

int codec_debug_capture(codec_t *c, int32_t what, float *dst, int64_t capacity,
                        codec_hip_stream stream)
{
    if (!c || !dst)
        return set_err(c ? &c->err : nullptr, CODEC_EINVAL, "codec_debug_capture: NULL argument");
    if (c->lastF == 0)
        return fail(c, CODEC_EINVAL, "codec_debug_capture: no decode step yet");
    const void *ext = nullptr;
    int H = 0, C = 0, rate = 1;
    bool materialized = true;
    int ld = 0;  // row pitch of the source, 0: C
    if (what == CODEC_CAPTURE_LATENT || what == CODEC_CAPTURE_DEC_INPUT) {
        if (c->fold)
            return fail(c, CODEC_EINVAL,
                        "codec_debug_capture: without a transformer the projection is folded "
                        "into the input conv and the latent is never stored; capture "
                        "CODEC_CAPTURE_RVQ_SUM");
        const bool tf_latent = what == CODEC_CAPTURE_LATENT && c->cfg.tf_layers > 0;
        ext = tf_latent ? c->u16 : c->u_ext;
        H = tf_latent ? 0 : 6;
        C = c->cfg.d_lat;
        if (tf_latent && c->lastF <= c->allocF && c->lastB <= c->allocB) {
            // the step ran the projection folded into the transformer's input
            // projection: the latent is computed here, from the step's RVQ sum
            HIPCHK(c, hipSetDevice(c->dev));
            ConvArgs a = conv_args(c, c->proj, c->z, 0, 1, c->lastF, c->last_meta);
            a.out16 = c->u16;
            a.out_H = 0;
            const int rc = run_conv(c, "proj", a, (hipStream_t)stream);
            if (rc)
                return rc;
        }
    } else if (what == CODEC_CAPTURE_RVQ_SUM) {
        ext = c->z;
        H = c->fold ? 6 : 0;
        ld = c->dz;
        C = c->cfg.d_cb;
    } else if (what >= CODEC_CAPTURE_LAYER0 && what <= CODEC_CAPTURE_LAYER0 + 3 * c->S) {
        const int t = what - CODEC_CAPTURE_LAYER0, i = t / 3, k = t % 3;
        if (t == 3 * c->S) {  // the final conv's input
            ext = c->a_outb;
            H = 6;
            C = c->ch[c->S];
            rate = c->hop;
            materialized = !c->fuse_T[c->S - 1];
        } else if (k == 0) {  // stage i's transposed-conv input (written by every path)
            ext = c->aT[i];
            H = 1;
            C = c->ch[i];
            rate = c->rate[i];
        } else {  // residual unit k - 1 of stage i
            ext = k == 1 ? c->a1[i] : c->a2[i];
            H = k == 1 ? 6 : 18;
            C = c->ch[i + 1];
            rate = c->rate[i + 1];
            materialized = !c->fuse_T[i];
        }
    } else {
        return fail(c, CODEC_EINVAL, "codec_debug_capture: what=%d (0..%d)", what,
                    CODEC_CAPTURE_LAYER0 + 3 * c->S);
    }
    if (!materialized)
        return fail(c, CODEC_EINVAL,
                    "codec_debug_capture: layer %d runs inside a fused stage kernel and is never "
                    "stored; open the codec with CODEC_FLAG_PER_LAYER to capture it",
                    what);
    const int64_t need = (int64_t)c->lastF * rate * C;
    if (capacity < need)
        return fail(c, CODEC_EINVAL, "codec_debug_capture: capacity %lld < %lld",
                    (long long)capacity, (long long)need);
    if (c->lastF > c->allocF || c->lastB > c->allocB)  // the workspace holds the step
        return fail(c, CODEC_EINVAL, "codec_debug_capture: step of %d frames, %d streams",
                    c->lastF, c->lastB);
    HIPCHK(c, hipSetDevice(c->dev));
    HIPCHK(c, launch_unextend(ext, c->dtype, H, ld ? ld : C, C, rate, c->last_meta.frame_stream,
                              c->lastF * rate, dst, (hipStream_t)stream));
    return CODEC_OK;
}

int codec_debug_read_state(codec_t *c, int32_t id, void *dst, int64_t capacity,
                           int64_t *bytes_out)
{
    if (!c || !bytes_out)
        return set_err(c ? &c->err : nullptr, CODEC_EINVAL, "codec_debug_read_state: NULL argument");
    auto it = c->id2slot.find(id);
    if (it == c->id2slot.end())
        return fail(c, CODEC_ESTREAM, "codec_debug_read_state: stream %d is not open", id);
    const int64_t bytes = c->slot_elems * c->esz;
    *bytes_out = bytes;
    if (!dst)
        return CODEC_OK;
    if (capacity < bytes)
        return fail(c, CODEC_EINVAL, "codec_debug_read_state: capacity %lld < %lld",
                    (long long)capacity, (long long)bytes);
    HIPCHK(c, hipSetDevice(c->dev));
    HIPCHK(c, hipDeviceSynchronize());
    HIPCHK(c, hipMemcpy(dst, (char *)c->state + (size_t)it->second * bytes, (size_t)bytes,
                        hipMemcpyDeviceToHost));
    return CODEC_OK;
}

int codec_profile_enable(codec_t *c, int32_t on)
{
    if (!c)
        return set_err(nullptr, CODEC_EINVAL, "codec_profile_enable: NULL codec");
    c->prof = on != 0;
    return CODEC_OK;
}

int codec_profile_read(codec_t *c, int32_t cap, const char **names, double *ms, int64_t *launches,
                       int64_t *units, int32_t *n_out)
{
    if (!c || !n_out)
        return set_err(c ? &c->err : nullptr, CODEC_EINVAL, "codec_profile_read: NULL argument");
    for (auto &r : c->recs) {
        HIPCHK(c, hipEventSynchronize(r.b));
        float t = 0.f;
        HIPCHK(c, hipEventElapsedTime(&t, r.a, r.b));
        c->cls_ms[r.cls] += t;
        c->cls_launches[r.cls] += 1;
        c->cls_units[r.cls] += r.units;
        c->ev_pool.push_back(r.a);
        c->ev_pool.push_back(r.b);
    }
    c->recs.clear();
    int n = (int)c->cls_names.size();
    for (int i = 0; i < n && i < cap; i++) {
        if (names)
            names[i] = c->cls_names[i].c_str();
        if (ms)
            ms[i] = c->cls_ms[i];
        if (launches)
            launches[i] = c->cls_launches[i];
        if (units)
            units[i] = c->cls_units[i];
    }
    *n_out = n;
    // reset the accumulators for the next window (names stay valid)
    std::fill(c->cls_ms.begin(), c->cls_ms.end(), 0.0);
    std::fill(c->cls_launches.begin(), c->cls_launches.end(), 0);
    std::fill(c->cls_units.begin(), c->cls_units.end(), 0);
    return CODEC_OK;
}

int codec_chunk_plan(int32_t total, const int32_t *ramp, int32_t n_ramp, int32_t steady,
                     int32_t initial, int32_t *out, int32_t cap, int32_t *n_out)
{
    if (total < 0 || steady <= 0 || n_ramp < 0 || (n_ramp > 0 && !ramp) || !n_out ||
        (cap > 0 && !out))
        return set_err(nullptr, CODEC_EINVAL,
                       "codec_chunk_plan: total=%d steady=%d n_ramp=%d", total, steady, n_ramp);
    for (int i = 0; i < n_ramp; i++)
        if (ramp[i] <= 0)
            return set_err(nullptr, CODEC_EINVAL, "codec_chunk_plan: ramp[%d]=%d", i, ramp[i]);
    // stride sequence: initial (or ramp[0]), ramp[1..], then steady; each <= steady
    auto stride = [&](int i) -> int32_t {
        int32_t v;
        if (i == 0)
            v = initial > 0 ? initial : (n_ramp > 0 ? ramp[0] : steady);
        else if (i < n_ramp)
            v = ramp[i];
        else
            v = steady;
        return std::min(v, steady);
    };
    int cnt = 0, si = 0;
    int64_t threshold = stride(si++), done = 0;
    for (int64_t g = 1; g <= total; g++) {
        if (g >= threshold) {
            if (cnt < cap)
                out[cnt] = (int32_t)(g - done);
            cnt++;
            done = g;
            threshold = g + stride(si++);
        }
    }
    if (done < total) {
        if (cnt < cap)
            out[cnt] = (int32_t)(total - done);
        cnt++;
    }
    *n_out = cnt;
    if (cnt > cap)
        return set_err(nullptr, CODEC_EINVAL, "codec_chunk_plan: %d decodes exceed cap %d", cnt,
                       cap);
    return CODEC_OK;
}

int codec_debug_conv_plan(int32_t M, int32_t N, int32_t Cin, int32_t taps, int32_t fp16,
                          int32_t n_cu, int32_t flags, const char **tile, int32_t *splits)
{
    if (M <= 0 || N <= 0 || Cin <= 0 || taps <= 0 || n_cu <= 0 || !tile || !splits)
        return set_err(nullptr, CODEC_EINVAL,
                       "codec_debug_conv_plan: M=%d N=%d Cin=%d taps=%d n_cu=%d", M, N, Cin, taps,
                       n_cu);
    ConvArgs a{};
    a.M = M;
    a.N = N;
    a.Cout = N;
    a.Cin = Cin;
    a.taps = taps;
    a.dil = 1;
    a.s = 1;
    a.rate_in = 1;
    a.splits_allowed = !(flags & CODEC_FLAG_NO_SPLIT_K);
    a.deep_allowed = !(flags & CODEC_FLAG_TWO_STAGE_BUFFERS);
    a.tall_allowed = !(flags & CODEC_FLAG_NO_TALL_TILES);
    const int dt = fp16 ? 1 : 0;
    const ConvPlan p = conv_gemm_plan(a, dt, n_cu, kSplitKCap);
    *tile = conv_gemm_tile_name(dt, p.tile);
    *splits = p.tile < 0 ? 0 : p.splits;
    return CODEC_OK;
}

int codec_initial_chunk_size(int64_t requested, int32_t has_request, int32_t steady,
                             int32_t fallback, int32_t *out)
{
    if (!out)
        return set_err(nullptr, CODEC_EINVAL, "codec_initial_chunk_size: NULL out");
    if (steady < 1)
        return set_err(nullptr, CODEC_EINVAL, "steady chunk size %d is below one frame", steady);
    const int64_t frames = has_request ? requested : (int64_t)fallback;
    if (frames < 0)
        return set_err(nullptr, CODEC_EINVAL, "chunk size %lld is negative", (long long)frames);
    *out = frames > steady ? steady : (int32_t)frames;
    return CODEC_OK;
}

}  // extern "C"
