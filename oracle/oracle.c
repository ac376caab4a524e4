/*
 * oracle.c -- plain fp64 CPU oracle of the streaming RVQ codec decoder.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library, and nothing here is ever on the
 * product path.
 *
 * What it computes.  Stage 1 of a two-stage TTS pipeline: each stream's
 * multi-codebook frames are turned into PCM by an RVQ decode followed by a
 * causal upsampling decoder.  The stateful streaming form keeps, per stream,
 * the causal convolutions' left context and the windowed transformer's KV,
 * decodes only new frames, and its concatenated output equals the decode of
 * the whole utterance (AREX article on vLLM-Omni / Fish Audio Drama 3,
 * section "two stages share one card: one forward per frame, stateful
 * streaming decode").  The pages give no layer-level architecture; the
 * network below is the plainest reading of the workload descriptions
 * (codebook counts and sizes, latent widths, hop factors, residual units of
 * kernel 7 with dilations 1 and 3 and Snake, a 4-layer 8-head windowed
 * transformer of window 32), each reading listed with its reason in the
 * design notes of the repository.
 *
 * Arithmetic.  Everything is fp64.  Every output element is reduced serially
 * in one fixed order (bias first, then taps ascending, then channels
 * ascending; keys ascending in attention), independent of how many frames a
 * call decodes, so a streamed decode equals the full decode bit for bit.
 * Vectorisation is only ever across independent output elements.  Build with
 * -fno-fast-math -ffp-contract=off.  OpenMP splits work across output
 * channels and across streams only.
 *
 * Layouts.  Convolutions work on channels x time arrays with PyTorch weight
 * layouts: Conv1d W[Co][Ci][k], ConvTranspose1d W[Ci][Co][k].  Linear layers
 * use W[out][in].
 */
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_MAX_STAGES 8
#define ORC_MAX_TF_LAYERS 16

typedef struct {
    int K, E, d_cb, d_lat;
    int n_stages;
    int strides[ORC_MAX_STAGES];
    int act;        /* 0: Snake, 1: ELU */
    int final_tanh; /* 0: off */
    int tf_layers, tf_heads, tf_head_dim, tf_window, tf_mlp;
} orc_cfg;

typedef struct {
    double *a1, *w7, *b7, *a2, *w1, *b1;
} orc_ru;

typedef struct {
    double *alpha, *wT, *bT;
    orc_ru ru[2];
} orc_stage;

typedef struct {
    double *ln1_g, *ln1_b, *qkv_w, *qkv_b, *o_w, *o_b;
    double *ln2_g, *ln2_b, *fc1_w, *fc1_b, *fc2_w, *fc2_b;
} orc_tflayer;

typedef struct {
    char name[96];
    double **slot;
    long n;
} orc_param;

typedef struct orc_model {
    orc_cfg cfg;
    int ch[ORC_MAX_STAGES + 1];
    int hop;
    int dm; /* transformer width */
    double *codebook[64];
    double *proj_w, *proj_b;
    double *tf_in_w, *tf_in_b, *lnf_g, *lnf_b, *tf_out_w, *tf_out_b;
    orc_tflayer tl[ORC_MAX_TF_LAYERS];
    double *in_w, *in_b;
    orc_stage st[ORC_MAX_STAGES];
    double *out_alpha, *out_w, *out_b;
    orc_param params[512];
    int n_params;
} orc_model;

typedef struct orc_stream {
    const orc_model *m;
    long pos;                             /* absolute frame index of the next frame */
    double *h_in;                         /* [d_lat][6] */
    double *h_T[ORC_MAX_STAGES];          /* [C_i][1] */
    double *h_ru[ORC_MAX_STAGES][2];      /* [C_{i+1}][6 d] */
    double *h_out;                        /* [C_S][6] */
    double *kv_k[ORC_MAX_TF_LAYERS];      /* [(W-1)][dm], oldest first */
    double *kv_v[ORC_MAX_TF_LAYERS];
    int kv_n;                             /* valid rows in each ring */
} orc_stream;

static const int RU_DIL[2] = {1, 3};

/* ------------------------------------------------------------------------ */
/* Elementwise maps                                                          */
/* ------------------------------------------------------------------------ */

/* Snake with per-channel alpha: y = x + sin(alpha x)^2 / alpha.  x is [C][T]. */
void orc_snake(const double *x, const double *alpha, int C, long T, double *y)
{
    for (int c = 0; c < C; c++) {
        double a = alpha[c];
        for (long t = 0; t < T; t++) {
            double v = x[(long)c * T + t];
            double s = sin(a * v);
            y[(long)c * T + t] = v + (s * s) / a;
        }
    }
}

/* ELU with alpha = 1: y = x for x > 0, else exp(x) - 1. */
void orc_elu(const double *x, long n, double *y)
{
    for (long i = 0; i < n; i++)
        y[i] = x[i] > 0.0 ? x[i] : expm1(x[i]);
}

/* GELU, erf form: 0.5 x (1 + erf(x / sqrt 2)). */
void orc_gelu(const double *x, long n, double *y)
{
    for (long i = 0; i < n; i++)
        y[i] = 0.5 * x[i] * (1.0 + erf(x[i] / sqrt(2.0)));
}

/* Decoder activation selected by the configuration. */
static void act_apply(const orc_model *m, const double *x, const double *alpha, int C, long T,
                      double *y)
{
    if (m->cfg.act == 1)
        orc_elu(x, (long)C * T, y);
    else
        orc_snake(x, alpha, C, T, y);
}

/* LayerNorm over one vector of D values: biased variance, affine. */
void orc_layer_norm(const double *x, const double *g, const double *b, int D, double eps,
                    double *y)
{
    double mean = 0.0;
    for (int i = 0; i < D; i++)
        mean += x[i];
    mean /= D;
    double var = 0.0;
    for (int i = 0; i < D; i++) {
        double dv = x[i] - mean;
        var += dv * dv;
    }
    var /= D;
    double inv = 1.0 / sqrt(var + eps);
    for (int i = 0; i < D; i++)
        y[i] = (x[i] - mean) * inv * g[i] + b[i];
}

/* y[o] = b[o] + sum_i W[o][i] x[i], i ascending (b may be NULL). */
void orc_linear(const double *W, const double *b, const double *x, int O, int I, double *y)
{
#pragma omp parallel for schedule(static)
    for (int o = 0; o < O; o++) {
        double acc = b ? b[o] : 0.0;
        const double *w = W + (long)o * I;
        for (int i = 0; i < I; i++)
            acc += w[i] * x[i];
        y[o] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Convolutions                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Causal dilated convolution.  x is [Ci][Hh + T] where the first
 * Hh = (k-1) d columns are the left context (zeros at a stream's start):
 *   y[o][t] = b[o] + sum_j sum_c W[o][c][j] x[c][t - (k-1-j) d]
 * with t counted from the first new column.  Order: bias, j ascending,
 * c ascending.
 */
void orc_causal_conv(const double *x, int Ci, long T, const double *W, const double *b, int Co,
                     int k, int d, double *y)
{
    long Hh = (long)(k - 1) * d;
    long L = Hh + T;
#pragma omp parallel for schedule(static)
    for (int o = 0; o < Co; o++) {
        double *yo = y + (long)o * T;
        double b0 = b ? b[o] : 0.0;
        for (long t = 0; t < T; t++)
            yo[t] = b0;
        for (int j = 0; j < k; j++) {
            long sh = (long)(k - 1 - j) * d;
            for (int c = 0; c < Ci; c++) {
                double w = W[((long)o * Ci + c) * k + j];
                const double *xc = x + (long)c * L + Hh - sh;
                for (long t = 0; t < T; t++)
                    yo[t] += w * xc[t];
            }
        }
    }
}

/*
 * Transposed convolution with stride s and kernel 2s, causal by dropping the
 * right overhang.  x is [Ci][1 + T]: column 0 is input index -1 (the previous
 * chunk's last input sample, zero at a stream's start).  Definition:
 *   y[o][n] = b[o] + sum_{(i, j): i s + j = n} sum_c x[c][i] W[c][o][j],
 * for n in [0, T s).  Order: bias, j ascending (so j = n mod s, then
 * j = n mod s + s), c ascending.
 */
void orc_conv_transpose(const double *x, int Ci, long T, const double *W, const double *b,
                        int Co, int s, double *y)
{
    int k = 2 * s;
    long N = T * s;
    long L = T + 1;
#pragma omp parallel for schedule(static)
    for (int o = 0; o < Co; o++) {
        double *yo = y + (long)o * N;
        double b0 = b ? b[o] : 0.0;
        for (long n = 0; n < N; n++)
            yo[n] = b0;
        for (int j = 0; j < k; j++) {
            for (int c = 0; c < Ci; c++) {
                double w = W[((long)c * Co + o) * k + j];
                const double *xc = x + (long)c * L + 1; /* xc[i], i >= -1 */
                for (long i = -1; i < T; i++) {
                    long n = i * s + j;
                    if (n < 0 || n >= N)
                        continue;
                    yo[n] += w * xc[i];
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Rotary position embedding, rotate-half pairing (i, i + hd/2), theta 10000,
 * applied to H heads of width hd at absolute position pos.
 */
void orc_rope(double *x, int H, int hd, long pos)
{
    int half = hd / 2;
    for (int h = 0; h < H; h++) {
        double *v = x + (long)h * hd;
        for (int i = 0; i < half; i++) {
            double inv_freq = pow(10000.0, -(2.0 * i) / hd);
            double ang = (double)pos * inv_freq;
            double cs = cos(ang), sn = sin(ang);
            double a = v[i], b = v[i + half];
            v[i] = a * cs - b * sn;
            v[i + half] = b * cs + a * sn;
        }
    }
}

/*
 * One query position attending over n keys (oldest first, the last is the
 * query's own frame): per head, softmax(q . k_j / sqrt(hd)) weighted sum of
 * v_j.  keys / vals are [n][H hd].
 */
void orc_window_attention(const double *q, const double *keys, const double *vals, int n, int H,
                          int hd, double *out)
{
    int dm = H * hd;
    double *sc = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
    double scale = sqrt((double)hd);
    for (int h = 0; h < H; h++) {
        const double *qh = q + (long)h * hd;
        double mx = -INFINITY;
        for (int j = 0; j < n; j++) {
            const double *kj = keys + (long)j * dm + (long)h * hd;
            double dot = 0.0;
            for (int e = 0; e < hd; e++)
                dot += qh[e] * kj[e];
            sc[j] = dot / scale;
            if (sc[j] > mx)
                mx = sc[j];
        }
        double den = 0.0;
        for (int j = 0; j < n; j++) {
            sc[j] = exp(sc[j] - mx);
            den += sc[j];
        }
        for (int e = 0; e < hd; e++) {
            double acc = 0.0;
            for (int j = 0; j < n; j++)
                acc += sc[j] * vals[(long)j * dm + (long)h * hd + e];
            out[(long)h * hd + e] = acc / den;
        }
    }
    free(sc);
}

/* ------------------------------------------------------------------------ */
/* Model                                                                     */
/* ------------------------------------------------------------------------ */

static void reg(orc_model *m, double **slot, long n, const char *fmt, ...)
    __attribute__((format(printf, 4, 5)));

static void reg(orc_model *m, double **slot, long n, const char *fmt, ...)
{
    orc_param *p = &m->params[m->n_params++];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(p->name, sizeof p->name, fmt, ap);
    va_end(ap);
    p->slot = slot;
    p->n = n;
    *slot = NULL;
}

orc_model *orc_model_new(const orc_cfg *cfg)
{
    if (cfg->K < 1 || cfg->K > 64 || cfg->n_stages < 1 || cfg->n_stages > ORC_MAX_STAGES ||
        cfg->tf_layers < 0 || cfg->tf_layers > ORC_MAX_TF_LAYERS)
        return NULL;
    orc_model *m = (orc_model *)calloc(1, sizeof(orc_model));
    m->cfg = *cfg;
    m->ch[0] = cfg->d_lat;
    m->hop = 1;
    for (int i = 0; i < cfg->n_stages; i++) {
        m->ch[i + 1] = m->ch[i] / 2;
        m->hop *= cfg->strides[i];
    }
    long E = cfg->E, dcb = cfg->d_cb, dl = cfg->d_lat;
    for (int k = 0; k < cfg->K; k++)
        reg(m, &m->codebook[k], E * dcb, "rvq.codebook.%d", k);
    reg(m, &m->proj_w, dl * dcb, "rvq.proj.weight");
    reg(m, &m->proj_b, dl, "rvq.proj.bias");
    if (cfg->tf_layers) {
        long dm = (long)cfg->tf_heads * cfg->tf_head_dim, mlp = cfg->tf_mlp;
        m->dm = (int)dm;
        reg(m, &m->tf_in_w, dm * dl, "tf.in_proj.weight");
        reg(m, &m->tf_in_b, dm, "tf.in_proj.bias");
        for (int l = 0; l < cfg->tf_layers; l++) {
            orc_tflayer *t = &m->tl[l];
            reg(m, &t->ln1_g, dm, "tf.layer.%d.ln1.weight", l);
            reg(m, &t->ln1_b, dm, "tf.layer.%d.ln1.bias", l);
            reg(m, &t->qkv_w, 3 * dm * dm, "tf.layer.%d.attn.qkv.weight", l);
            reg(m, &t->qkv_b, 3 * dm, "tf.layer.%d.attn.qkv.bias", l);
            reg(m, &t->o_w, dm * dm, "tf.layer.%d.attn.out.weight", l);
            reg(m, &t->o_b, dm, "tf.layer.%d.attn.out.bias", l);
            reg(m, &t->ln2_g, dm, "tf.layer.%d.ln2.weight", l);
            reg(m, &t->ln2_b, dm, "tf.layer.%d.ln2.bias", l);
            reg(m, &t->fc1_w, mlp * dm, "tf.layer.%d.mlp.fc1.weight", l);
            reg(m, &t->fc1_b, mlp, "tf.layer.%d.mlp.fc1.bias", l);
            reg(m, &t->fc2_w, dm * mlp, "tf.layer.%d.mlp.fc2.weight", l);
            reg(m, &t->fc2_b, dm, "tf.layer.%d.mlp.fc2.bias", l);
        }
        reg(m, &m->lnf_g, dm, "tf.ln_f.weight");
        reg(m, &m->lnf_b, dm, "tf.ln_f.bias");
        reg(m, &m->tf_out_w, dl * dm, "tf.out_proj.weight");
        reg(m, &m->tf_out_b, dl, "tf.out_proj.bias");
    }
    reg(m, &m->in_w, (long)m->ch[0] * dl * 7, "dec.in_conv.weight");
    reg(m, &m->in_b, m->ch[0], "dec.in_conv.bias");
    for (int i = 0; i < cfg->n_stages; i++) {
        long ci = m->ch[i], co = m->ch[i + 1], s = cfg->strides[i];
        orc_stage *st = &m->st[i];
        reg(m, &st->alpha, ci, "dec.stage.%d.snake.alpha", i);
        reg(m, &st->wT, ci * co * 2 * s, "dec.stage.%d.convT.weight", i);
        reg(m, &st->bT, co, "dec.stage.%d.convT.bias", i);
        for (int j = 0; j < 2; j++) {
            orc_ru *r = &st->ru[j];
            reg(m, &r->a1, co, "dec.stage.%d.ru.%d.snake1.alpha", i, j);
            reg(m, &r->w7, co * co * 7, "dec.stage.%d.ru.%d.conv7.weight", i, j);
            reg(m, &r->b7, co, "dec.stage.%d.ru.%d.conv7.bias", i, j);
            reg(m, &r->a2, co, "dec.stage.%d.ru.%d.snake2.alpha", i, j);
            reg(m, &r->w1, co * co, "dec.stage.%d.ru.%d.conv1.weight", i, j);
            reg(m, &r->b1, co, "dec.stage.%d.ru.%d.conv1.bias", i, j);
        }
    }
    int cs = m->ch[cfg->n_stages];
    reg(m, &m->out_alpha, cs, "dec.out.snake.alpha");
    reg(m, &m->out_w, (long)cs * 7, "dec.out.conv.weight");
    reg(m, &m->out_b, 1, "dec.out.conv.bias");
    return m;
}

/* Copies one named parameter (fp64 values).  0 ok, -1 unknown name, -2 size. */
int orc_model_set(orc_model *m, const char *name, const double *data, long n)
{
    for (int i = 0; i < m->n_params; i++) {
        orc_param *p = &m->params[i];
        if (strcmp(p->name, name) != 0)
            continue;
        if (n != p->n)
            return -2;
        free(*p->slot);
        *p->slot = (double *)malloc(sizeof(double) * (size_t)n);
        memcpy(*p->slot, data, sizeof(double) * (size_t)n);
        return 0;
    }
    return -1;
}

/* Index of the first parameter not yet set, or -1 when all are set. */
int orc_model_missing(const orc_model *m)
{
    for (int i = 0; i < m->n_params; i++)
        if (!*m->params[i].slot)
            return i;
    return -1;
}

const char *orc_model_param_name(const orc_model *m, int i)
{
    return (i >= 0 && i < m->n_params) ? m->params[i].name : NULL;
}

int orc_model_n_params(const orc_model *m) { return m->n_params; }
int orc_model_hop(const orc_model *m) { return m->hop; }

void orc_model_free(orc_model *m)
{
    if (!m)
        return;
    for (int i = 0; i < m->n_params; i++)
        free(*m->params[i].slot);
    free(m);
}

/* ------------------------------------------------------------------------ */
/* Streams                                                                   */
/* ------------------------------------------------------------------------ */

static double *zalloc(long n) { return (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double)); }

/* A fresh stream: every left context is zero and the next frame has absolute
 * index pos0 (0 for a stream decoded from its start). */
orc_stream *orc_stream_new(const orc_model *m, long pos0)
{
    orc_stream *s = (orc_stream *)calloc(1, sizeof(orc_stream));
    const orc_cfg *c = &m->cfg;
    s->m = m;
    s->pos = pos0;
    s->h_in = zalloc((long)c->d_lat * 6);
    for (int i = 0; i < c->n_stages; i++) {
        s->h_T[i] = zalloc(m->ch[i]);
        for (int j = 0; j < 2; j++)
            s->h_ru[i][j] = zalloc((long)m->ch[i + 1] * 6 * RU_DIL[j]);
    }
    s->h_out = zalloc((long)m->ch[c->n_stages] * 6);
    for (int l = 0; l < c->tf_layers; l++) {
        s->kv_k[l] = zalloc((long)(c->tf_window - 1) * m->dm);
        s->kv_v[l] = zalloc((long)(c->tf_window - 1) * m->dm);
    }
    s->kv_n = 0;
    return s;
}

void orc_stream_free(orc_stream *s)
{
    if (!s)
        return;
    const orc_cfg *c = &s->m->cfg;
    free(s->h_in);
    for (int i = 0; i < c->n_stages; i++) {
        free(s->h_T[i]);
        for (int j = 0; j < 2; j++)
            free(s->h_ru[i][j]);
    }
    free(s->h_out);
    for (int l = 0; l < c->tf_layers; l++) {
        free(s->kv_k[l]);
        free(s->kv_v[l]);
    }
    free(s);
}

long orc_stream_pos(const orc_stream *s) { return s->pos; }

/*
 * Causal conv of new columns x [Ci][T] against the stream's left context
 * halo [Ci][(k-1) d]; afterwards halo holds the last (k-1) d input columns
 * of [halo | x], which also covers T < (k-1) d.
 */
static void conv_stream(double *halo, const double *x, int Ci, long T, const double *W,
                        const double *b, int Co, int k, int d, double *y)
{
    long Hh = (long)(k - 1) * d, L = Hh + T;
    double *ext = zalloc((long)Ci * L);
    for (int c = 0; c < Ci; c++) {
        if (Hh)
            memcpy(ext + (long)c * L, halo + (long)c * Hh, sizeof(double) * Hh);
        memcpy(ext + (long)c * L + Hh, x + (long)c * T, sizeof(double) * T);
    }
    orc_causal_conv(ext, Ci, T, W, b, Co, k, d, y);
    for (int c = 0; c < Ci; c++)
        if (Hh)
            memcpy(halo + (long)c * Hh, ext + (long)c * L + T, sizeof(double) * Hh);
    free(ext);
}

/* Transposed conv of new columns with a one-column left context. */
static void convT_stream(double *halo, const double *x, int Ci, long T, const double *W,
                         const double *b, int Co, int s, double *y)
{
    long L = T + 1;
    double *ext = zalloc((long)Ci * L);
    for (int c = 0; c < Ci; c++) {
        ext[(long)c * L] = halo[c];
        memcpy(ext + (long)c * L + 1, x + (long)c * T, sizeof(double) * T);
    }
    orc_conv_transpose(ext, Ci, T, W, b, Co, s, y);
    for (int c = 0; c < Ci; c++)
        halo[c] = ext[(long)c * L + T];
    free(ext);
}

/* RVQ decode of frames: z[t] = sum_k C_k[codes[t][k]], k ascending.
 * Returns -1 if a code is outside [0, E). */
int orc_rvq_sum(const orc_model *m, const int32_t *codes, int T, double *z)
{
    const orc_cfg *c = &m->cfg;
    for (int t = 0; t < T; t++) {
        double *zt = z + (long)t * c->d_cb;
        for (int d = 0; d < c->d_cb; d++)
            zt[d] = 0.0;
        for (int k = 0; k < c->K; k++) {
            int32_t e = codes[(long)t * c->K + k];
            if (e < 0 || e >= c->E)
                return -1;
            const double *row = m->codebook[k] + (long)e * c->d_cb;
            for (int d = 0; d < c->d_cb; d++)
                zt[d] += row[d];
        }
    }
    return 0;
}

/* One frame through the windowed causal transformer at absolute position
 * pos.  x [d_lat] -> y [d_lat]; appends this frame's K, V to the rings. */
static void tf_frame(orc_stream *s, const double *x, long pos, double *y)
{
    const orc_model *m = s->m;
    const orc_cfg *c = &m->cfg;
    int dm = m->dm, H = c->tf_heads, hd = c->tf_head_dim, W1 = c->tf_window - 1;
    double *h = zalloc(dm), *a = zalloc(dm), *qkv = zalloc(3L * dm), *att = zalloc(dm);
    double *o = zalloc(dm), *f1 = zalloc(c->tf_mlp), *f2 = zalloc(dm);
    double *keys = zalloc((long)(W1 + 1) * dm), *vals = zalloc((long)(W1 + 1) * dm);
    orc_linear(m->tf_in_w, m->tf_in_b, x, dm, c->d_lat, h);
    int nprev = s->kv_n;
    for (int l = 0; l < c->tf_layers; l++) {
        const orc_tflayer *t = &m->tl[l];
        orc_layer_norm(h, t->ln1_g, t->ln1_b, dm, 1e-5, a);
        orc_linear(t->qkv_w, t->qkv_b, a, 3 * dm, dm, qkv);
        double *q = qkv, *k = qkv + dm, *v = qkv + 2 * dm;
        orc_rope(q, H, hd, pos);
        orc_rope(k, H, hd, pos);
        memcpy(keys, s->kv_k[l], sizeof(double) * (size_t)nprev * dm);
        memcpy(vals, s->kv_v[l], sizeof(double) * (size_t)nprev * dm);
        memcpy(keys + (long)nprev * dm, k, sizeof(double) * dm);
        memcpy(vals + (long)nprev * dm, v, sizeof(double) * dm);
        orc_window_attention(q, keys, vals, nprev + 1, H, hd, att);
        orc_linear(t->o_w, t->o_b, att, dm, dm, o);
        for (int i = 0; i < dm; i++)
            h[i] = h[i] + o[i];
        orc_layer_norm(h, t->ln2_g, t->ln2_b, dm, 1e-5, a);
        orc_linear(t->fc1_w, t->fc1_b, a, c->tf_mlp, dm, f1);
        orc_gelu(f1, c->tf_mlp, f1);
        orc_linear(t->fc2_w, t->fc2_b, f1, dm, c->tf_mlp, f2);
        for (int i = 0; i < dm; i++)
            h[i] = h[i] + f2[i];
        /* ring update: keep the last W-1 frames, oldest first */
        int n1 = nprev + 1;
        const double *src_k = keys, *src_v = vals;
        if (n1 > W1) {
            src_k += (long)(n1 - W1) * dm;
            src_v += (long)(n1 - W1) * dm;
            n1 = W1;
        }
        memcpy(s->kv_k[l], src_k, sizeof(double) * (size_t)n1 * dm);
        memcpy(s->kv_v[l], src_v, sizeof(double) * (size_t)n1 * dm);
    }
    s->kv_n = nprev + 1 > W1 ? W1 : nprev + 1;
    orc_layer_norm(h, m->lnf_g, m->lnf_b, dm, 1e-5, a);
    orc_linear(m->tf_out_w, m->tf_out_b, a, c->d_lat, dm, y);
    free(h); free(a); free(qkv); free(att); free(o); free(f1); free(f2);
    free(keys); free(vals);
}

/*
 * Decode n new frames of one stream.  codes [n][K] (k = 0 is the first,
 * coarsest codebook); pcm receives n * hop samples.  Optional captures:
 * cap_u [n][d_lat] the projected latent, cap_x [n][d_lat] the decoder
 * input (after the transformer, equal to cap_u without one).
 * Returns 0, -1 for a code outside [0, E), -2 for n < 0.
 *
 * orc_stream_decode_tap also copies out one conv operand of the decoder
 * (the activated input a conv multiplies), time-major [rows][C], for
 * layer-by-layer comparisons: tap 3 i is the transposed conv input of stage
 * i, tap 3 i + 1 + j the input of residual unit j of stage i, tap 3 S the
 * final conv input.  Taking a tap changes nothing in the decode.
 */
static int stream_decode(orc_stream *s, const int32_t *codes, int n, double *pcm, double *cap_u,
                         double *cap_x, int tap, double *cap_tap);

static void tap_copy(const double *a, int C, long T, double *dst)
{
    for (long t = 0; t < T; t++)
        for (int c = 0; c < C; c++)
            dst[t * C + c] = a[(long)c * T + t];
}

int orc_stream_decode(orc_stream *s, const int32_t *codes, int n, double *pcm, double *cap_u,
                      double *cap_x)
{
    return stream_decode(s, codes, n, pcm, cap_u, cap_x, -1, NULL);
}

int orc_stream_decode_tap(orc_stream *s, const int32_t *codes, int n, double *pcm, int tap,
                          double *cap_tap)
{
    if (tap < 0 || tap > 3 * s->m->cfg.n_stages || !cap_tap)
        return -3;
    return stream_decode(s, codes, n, pcm, NULL, NULL, tap, cap_tap);
}

static int stream_decode(orc_stream *s, const int32_t *codes, int n, double *pcm, double *cap_u,
                         double *cap_x, int tap, double *cap_tap)
{
    const orc_model *m = s->m;
    const orc_cfg *c = &m->cfg;
    if (n < 0)
        return -2;
    if (n == 0)
        return 0;
    for (long i = 0; i < (long)n * c->K; i++)
        if (codes[i] < 0 || codes[i] >= c->E)
            return -1;
    int dl = c->d_lat;
    double *z = zalloc((long)n * c->d_cb);
    double *u = zalloc((long)n * dl); /* time-major [n][dl] */
    orc_rvq_sum(m, codes, n, z);
    for (int t = 0; t < n; t++)
        orc_linear(m->proj_w, m->proj_b, z + (long)t * c->d_cb, dl, c->d_cb, u + (long)t * dl);
    if (cap_u)
        memcpy(cap_u, u, sizeof(double) * (size_t)n * dl);
    if (c->tf_layers) {
        double *y = zalloc(dl);
        for (int t = 0; t < n; t++) {
            tf_frame(s, u + (long)t * dl, s->pos + t, y);
            memcpy(u + (long)t * dl, y, sizeof(double) * dl);
        }
        free(y);
    }
    if (cap_x)
        memcpy(cap_x, u, sizeof(double) * (size_t)n * dl);

    /* channels x time from here on */
    long T = n;
    double *x = zalloc((long)dl * T);
    for (int t = 0; t < n; t++)
        for (int ch = 0; ch < dl; ch++)
            x[(long)ch * T + t] = u[(long)t * dl + ch];
    double *y = zalloc((long)m->ch[0] * T);
    conv_stream(s->h_in, x, dl, T, m->in_w, m->in_b, m->ch[0], 7, 1, y);
    free(x);
    x = y; /* [C0][T] */

    for (int i = 0; i < c->n_stages; i++) {
        const orc_stage *st = &m->st[i];
        int ci = m->ch[i], co = m->ch[i + 1], sd = c->strides[i];
        double *a = zalloc((long)ci * T);
        act_apply(m, x, st->alpha, ci, T, a);
        if (tap == 3 * i)
            tap_copy(a, ci, T, cap_tap);
        long T2 = T * sd;
        double *xt = zalloc((long)co * T2);
        convT_stream(s->h_T[i], a, ci, T, st->wT, st->bT, co, sd, xt);
        free(a);
        free(x);
        x = xt;
        T = T2;
        for (int j = 0; j < 2; j++) {
            const orc_ru *r = &st->ru[j];
            double *a1 = zalloc((long)co * T), *h7 = zalloc((long)co * T);
            double *a2 = zalloc((long)co * T), *h1 = zalloc((long)co * T);
            act_apply(m, x, r->a1, co, T, a1);
            if (tap == 3 * i + 1 + j)
                tap_copy(a1, co, T, cap_tap);
            conv_stream(s->h_ru[i][j], a1, co, T, r->w7, r->b7, co, 7, RU_DIL[j], h7);
            act_apply(m, h7, r->a2, co, T, a2);
            orc_causal_conv(a2, co, T, r->w1, r->b1, co, 1, 1, h1);
            for (long e = 0; e < (long)co * T; e++)
                x[e] = x[e] + h1[e];
            free(a1); free(h7); free(a2); free(h1);
        }
    }
    int cs = m->ch[c->n_stages];
    double *a = zalloc((long)cs * T);
    act_apply(m, x, m->out_alpha, cs, T, a);
    if (tap == 3 * c->n_stages)
        tap_copy(a, cs, T, cap_tap);
    conv_stream(s->h_out, a, cs, T, m->out_w, m->out_b, 1, 7, 1, pcm);
    if (c->final_tanh)
        for (long e = 0; e < T; e++)
            pcm[e] = tanh(pcm[e]);
    free(a);
    free(x);
    free(z);
    free(u);
    s->pos += n;
    return 0;
}

/*
 * Decode one chunk for each of B independent streams in parallel (one
 * stream per thread; per-layer loops then run single-threaded).  codes and
 * pcm are packed stream after stream: stream b's frames start at frame
 * sum_{b' < b} n[b'].  Returns 0 or the first nonzero per-stream status.
 */
int orc_decode_batch(orc_stream **streams, int B, const int32_t *n, const int32_t *codes,
                     double *pcm)
{
    long *off = (long *)malloc(sizeof(long) * (size_t)(B + 1));
    off[0] = 0;
    for (int b = 0; b < B; b++)
        off[b + 1] = off[b] + n[b];
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; b++) {
        const orc_model *m = streams[b]->m;
        int rc = orc_stream_decode(streams[b], codes + off[b] * m->cfg.K, n[b],
                                   pcm + off[b] * m->hop, NULL, NULL);
        if (rc) {
#pragma omp critical
            if (!status)
                status = rc;
        }
    }
    free(off);
    return status;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
