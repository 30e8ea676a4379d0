/*
 * oracle.c - plain CPU reference of one batch-1 decode step (see oracle.h).
 *
 * TEST INFRASTRUCTURE ONLY.  Slow on purpose: every output element is one
 * loop in natural index order, in fp64, so that a reader can check each
 * function against its definition by eye.  OpenMP only splits independent
 * output elements across threads; it never changes an element's arithmetic,
 * so results do not depend on the thread count.
 *
 * Sources (web pages on batch-1 decode):
 *   [tiles]  "Decoding in tiles" (TileInfer), sec. 2 "Why decode has a lower
 *            bound" and sec. 4 "Tile-based static scheduling".
 *   [tiny]   "How I built an LLM inference engine from scratch in CUDA"
 *            (tinyinfer), sections "The speed limit is memory", "v0.1",
 *            "Round 2" and "How I knew it was still correct".
 *   [launch] "One launch per token", sections "The oracle, then the kernels"
 *            and "The attention trap".
 *   [flint]  flint README, the chat.py passage on half-split RoPE.
 *   [metal]  "LLAMA 1B Optimizing Kernels", sections "Grouped Query
 *            Attention", "RMSNorm" and "Kernel Fusion".
 * Readings where the pages are silent (epsilon, RoPE frequencies, attention
 * scale, nibble order) are the plainest ones and are listed in the design
 * notes; each function below states the one it takes.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* bf16: the top 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
double orc_f16_value(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return sign ? -v : v;
}

/* double -> fp32 (C cast, round to nearest even) -> bf16 round to nearest even. */
uint16_t orc_round_bf16(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t rest = u & 0xffffu;
    uint32_t top = u >> 16;
    if (rest > 0x8000u || (rest == 0x8000u && (top & 1u))) top += 1u;
    return (uint16_t)top;
}

/* ---------------------------------------------------------------- RMSNorm */

/* y_i = x_i / sqrt(mean_j x_j^2 + eps) * g_i.  RMSNorm is the norm the layer
 * applies before attention and before the MLP ([tiles] sec. 2, Fig. 3; [metal]
 * "RMSNorm": a reduction over the whole hidden vector).  eps is a config value. */
void orc_rmsnorm(const double* x, const uint16_t* gain, int32_t n, double eps, double* y) {
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int32_t i = 0; i < n; ++i) y[i] = x[i] * inv * orc_bf16_value(gain[i]);
}

/* ---------------------------------------------------------------- weights */

/* Weight (r, k) of a stored linear.  bf16: its value.  int4 ([tiny] "The speed
 * limit is memory": 4 bits plus one fp16 scale per 64 weights): scale * (u - 8),
 * where u is the 4-bit code of element k (byte k/2, low nibble for even k) and
 * the scale is the one of group k/64 of row r.  The product is exact in fp64. */
double orc_weight(const void* w, const uint16_t* s, int32_t fmt, int32_t cols, int64_t r, int32_t k) {
    if (fmt == ORC_WF_BF16) return orc_bf16_value(((const uint16_t*)w)[r * cols + k]);
    const uint8_t* row = (const uint8_t*)w + r * (cols / 2);
    uint8_t byte = row[k / 2];
    int u = (k % 2 == 0) ? (byte & 0xf) : (byte >> 4);
    double scale = orc_f16_value(s[r * (cols / 64) + k / 64]);
    return scale * (double)(u - 8);
}

/* y = W x: at batch one every projection is a matrix-vector product, each
 * weight used for one multiply-add ([tiles] sec. 2).  Row r of W is output r. */
void orc_linear(const void* w, const uint16_t* s, int32_t fmt, int32_t rows, int32_t cols,
                const double* x, double* y, int32_t nthreads) {
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int32_t r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int32_t k = 0; k < cols; ++k) acc += orc_weight(w, s, fmt, cols, r, k) * x[k];
        y[r] = acc;
    }
}

/* ---------------------------------------------------------------- RoPE */

/* Half-split (NeoX) rotary embedding of one head vector in place ([flint],
 * chat.py passage: out[i] = x[i] cos - x[i + d/2] sin; [launch]: rotate_half
 * from a gathered index).  Pair (i, i + d/2) turns by the angle pos * theta_i
 * with theta_i = base^(-2i/d), i < d/2; no frequency scaling. */
void orc_rope(double* v, int32_t d, int32_t pos, double base) {
    int32_t half = d / 2;
    for (int32_t i = 0; i < half; ++i) {
        double freq = pow(base, -2.0 * (double)i / (double)d);
        double ang = (double)pos * freq;
        double c = cos(ang), s = sin(ang);
        double a = v[i], b = v[i + half];
        v[i] = a * c - b * s;
        v[i + half] = b * c + a * s;
    }
}

/* ---------------------------------------------------------------- attention */

/* Decode attention of one query head over positions 0..n_pos-1 of its K/V head
 * ([tiles] sec. 2: of the step's costs only attention depends on the
 * position; [metal] "Flash Attention": at decode a single query row reads the
 * whole cache, so no causal mask applies).  Scores q.k / sqrt(d), softmax, weighted sum of V.
 * Plain two-pass softmax: max, then exponentials and their sum. */
void orc_attention(const double* q, const uint16_t* K, const uint16_t* V, int32_t n_pos,
                   int32_t d, double* out) {
    double* sc = (double*)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
    double scale = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int32_t t = 0; t < n_pos; ++t) {
        double dot = 0.0;
        for (int32_t i = 0; i < d; ++i) dot += q[i] * orc_bf16_value(K[(int64_t)t * d + i]);
        sc[t] = dot * scale;
        if (sc[t] > m) m = sc[t];
    }
    double l = 0.0;
    for (int32_t t = 0; t < n_pos; ++t) {
        sc[t] = exp(sc[t] - m);
        l += sc[t];
    }
    for (int32_t i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int32_t t = 0; t < n_pos; ++t) acc += sc[t] * orc_bf16_value(V[(int64_t)t * d + i]);
        out[i] = acc / l;
    }
    free(sc);
}

/* ---------------------------------------------------------------- SwiGLU */

/* SiLU(z) = z / (1 + e^-z); the MLP output is SiLU(gate) * up ([tiles] sec. 4
 * "FFN"; [metal] "RMSNorm + 2 GEMV (Up, Gate) + SwiGLU"). */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* ---------------------------------------------------------------- argmax */

/* Greedy selection ([tiles] sec. 5): the largest logit, the lowest token id
 * among ties; a non-finite logit is an error.  The comparison is made on the
 * logits rounded to fp32, the precision the GPU kernel decides in. */
int32_t orc_argmax(const double* logits, int32_t n, int32_t* nonfinite) {
    int32_t best = -1;
    float bv = 0.0f;
    int32_t bad = 0;
    for (int32_t i = 0; i < n; ++i) {
        float v = (float)logits[i];
        if (!isfinite(v)) { bad = 1; continue; }
        if (best < 0 || v > bv) { bv = v; best = i; }   /* strict: ties keep the lower id */
    }
    if (nonfinite) *nonfinite = bad;
    return best;
}

/* ---------------------------------------------------------------- MoE routing */

/* The router of a mixture-of-experts layer ("One launch per token", its 64-expert
 * MoE section): each token goes to a fixed number k of the E experts, chosen at
 * run time from the router's scores, and the experts' outputs are combined as a
 * weighted sum.  The pages fix neither the scores' normalisation nor the
 * weights; read plainly, as in the model they name, the weights are the softmax
 * of all E router logits taken at the k chosen experts (not renormalised over
 * the k), and the k chosen are those with the largest logits.  The choice is an
 * integer decided on floating point, so it is made on logits rounded to fp32,
 * the precision the GPU decides in; ties go to the lowest expert id. */
int32_t orc_route(const double* z, int32_t E, int32_t k, int32_t* ids, double* weights) {
    if (!z || !ids || !weights || E <= 0 || k <= 0 || k > E) return ORC_E_ARG;
    double m = z[0];
    for (int32_t e = 0; e < E; ++e) {
        if (!isfinite(z[e])) return ORC_E_NONFINITE;
        if (z[e] > m) m = z[e];
    }
    double sum = 0.0;
    for (int32_t e = 0; e < E; ++e) sum += exp(z[e] - m);
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        float bv = 0.0f;
        for (int32_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            float v = (float)z[e];
            if (best < 0 || bv < v) { bv = v; best = e; }   /* strict: ties keep the lower id */
        }
        taken[best] = 1;
        ids[j] = best;
        weights[j] = exp(z[best] - m) / sum;
    }
    free(taken);
    return ORC_OK;
}

/* Expert e's block of a stacked [E][rows][cols] linear and of its scales. */
static const void* expert_w(const void* w, int32_t fmt, int32_t e, int32_t rows, int32_t cols) {
    if (fmt == ORC_WF_INT4_G64) return (const uint8_t*)w + (int64_t)e * rows * (cols / 2);
    return (const uint16_t*)w + (int64_t)e * rows * cols;
}
static const uint16_t* expert_s(const uint16_t* s, int32_t fmt, int32_t e, int32_t rows, int32_t cols) {
    if (fmt != ORC_WF_INT4_G64 || !s) return NULL;
    return s + (int64_t)e * rows * (cols / 64);
}

/* ---------------------------------------------------------------- the step */

static int32_t check_cfg(const orc_config* c) {
    if (!c || c->n_layers <= 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
        c->head_dim <= 0 || (c->head_dim % 2) || c->intermediate <= 0 || c->vocab <= 0 ||
        c->max_ctx <= 0 || (c->n_q_heads % c->n_kv_heads))
        return ORC_E_ARG;
    if (c->weight_format == ORC_WF_INT4_G64 &&
        ((c->hidden % 64) || (c->intermediate % 64) || ((c->n_q_heads * c->head_dim) % 64)))
        return ORC_E_ARG;
    if (c->weight_format != ORC_WF_BF16 && c->weight_format != ORC_WF_INT4_G64) return ORC_E_ARG;
    if (c->n_experts < 0 || (c->n_experts > 0 && (c->top_k < 1 || c->top_k > c->n_experts))) return ORC_E_ARG;
    return ORC_OK;
}

int32_t orc_step_traced(const orc_config* c, const orc_weights* w, int32_t token, int32_t pos,
                        uint16_t* k_cache, uint16_t* v_cache, double* logits, int32_t nthreads,
                        const orc_trace* tr) {
    if (check_cfg(c) != ORC_OK || !w || !k_cache || !v_cache) return ORC_E_ARG;
    if (token < 0 || token >= c->vocab || pos < 0 || pos >= c->max_ctx) return ORC_E_ARG;
    const int32_t H = c->hidden, d = c->head_dim, nq = c->n_q_heads, nkv = c->n_kv_heads;
    const int32_t I = c->intermediate, V = c->vocab, fmt = c->weight_format;
    const int32_t qd = nq * d, kvd = nkv * d, rows_qkv = qd + 2 * kvd;
    const int32_t group = nq / nkv;
    const int64_t ctx = c->max_ctx;

    double* x = (double*)calloc((size_t)H, sizeof(double));
    double* h = (double*)calloc((size_t)H, sizeof(double));
    double* y = (double*)calloc((size_t)H, sizeof(double));
    double* qkv = (double*)calloc((size_t)rows_qkv, sizeof(double));
    double* att = (double*)calloc((size_t)qd, sizeof(double));
    double* gu = (double*)calloc((size_t)2 * I, sizeof(double));
    double* act = (double*)calloc((size_t)I, sizeof(double));

    /* 1. the input side reads one embedding row, no scaling ([tiles] sec. 2). */
    for (int32_t i = 0; i < H; ++i) x[i] = orc_bf16_value(w->embed[(int64_t)token * H + i]);
    if (tr && tr->x_in) memcpy(tr->x_in, x, sizeof(double) * H);

    for (int32_t l = 0; l < c->n_layers; ++l) {
        const orc_layer* L = &w->layers[l];
        uint16_t* Kl = k_cache + (int64_t)l * nkv * ctx * d;
        uint16_t* Vl = v_cache + (int64_t)l * nkv * ctx * d;

        /* 2. RMSNorm, then the stacked [Wq; Wk; Wv] projection ([tiles] sec. 4
         *    "QKV"; [launch]: bias added in the QKV epilogue). */
        orc_rmsnorm(x, L->attn_norm, H, c->rms_eps, h);
        orc_linear(L->w_qkv, L->s_qkv, fmt, rows_qkv, H, h, qkv, nthreads);
        if (c->qkv_bias && L->b_qkv)
            for (int32_t r = 0; r < rows_qkv; ++r) qkv[r] += orc_bf16_value(L->b_qkv[r]);

        /* 3. RoPE on every q and k head at this position. */
        for (int32_t hh = 0; hh < nq; ++hh) orc_rope(qkv + hh * d, d, pos, c->rope_theta);
        for (int32_t g = 0; g < nkv; ++g) orc_rope(qkv + qd + g * d, d, pos, c->rope_theta);
        if (tr && tr->qkv) memcpy(tr->qkv + (int64_t)l * rows_qkv, qkv, sizeof(double) * rows_qkv);

        /* 4. the new K and V rows go to the cache at `pos` ([tiles] sec. 4
         *    "Attention"; the cache is the only state kept across tokens). */
        for (int32_t g = 0; g < nkv; ++g)
            for (int32_t i = 0; i < d; ++i) {
                Kl[((int64_t)g * ctx + pos) * d + i] = orc_round_bf16(qkv[qd + g * d + i]);
                Vl[((int64_t)g * ctx + pos) * d + i] = orc_round_bf16(qkv[qd + kvd + g * d + i]);
            }

        /* 5. grouped-query attention: q head hh reads K/V head hh / group
         *    ([metal] "Grouped Query Attention": consecutive groups of query
         *    heads share one K/V head), over positions 0..pos read back from the
         *    cache. */
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
        for (int32_t hh = 0; hh < nq; ++hh) {
            int32_t g = hh / group;
            orc_attention(qkv + hh * d, Kl + (int64_t)g * ctx * d, Vl + (int64_t)g * ctx * d, pos + 1,
                          d, att + hh * d);
        }
        if (tr && tr->attn) memcpy(tr->attn + (int64_t)l * qd, att, sizeof(double) * qd);

        /* 6. output projection and residual add ([tiles] sec. 4 "Wo"). */
        orc_linear(L->w_o, L->s_o, fmt, H, qd, att, y, nthreads);
        for (int32_t i = 0; i < H; ++i) x[i] += y[i];
        if (tr && tr->x_mid) memcpy(tr->x_mid + (int64_t)l * H, x, sizeof(double) * H);

        /* 7. RMSNorm, gate and up projections, SiLU(gate) * up ([tiles] sec. 4 "FFN"). */
        orc_rmsnorm(x, L->mlp_norm, H, c->rms_eps, h);
        if (c->n_experts == 0) {
            orc_linear(L->w_gu, L->s_gu, fmt, 2 * I, H, h, gu, nthreads);
            for (int32_t r = 0; r < I; ++r) act[r] = orc_silu(gu[r]) * gu[I + r];
            if (tr && tr->act) memcpy(tr->act + (int64_t)l * I, act, sizeof(double) * I);

            /* 8. down projection and residual add ([metal] "GEMV (Down) + Residual Add"). */
            orc_linear(L->w_d, L->s_d, fmt, H, I, act, y, nthreads);
            for (int32_t i = 0; i < H; ++i) x[i] += y[i];
        } else {
            /* 7-8 (MoE, [launch] 64-expert section): the router scores the E experts,
             * the k chosen run the same SiLU-gated MLP on h, and their down
             * projections are added to the residual weighted by the router
             * probabilities, in the order chosen. */
            const int32_t E = c->n_experts, k = c->top_k;
            double* z = (double*)calloc((size_t)E, sizeof(double));
            double* ysum = (double*)calloc((size_t)H, sizeof(double));
            int32_t* ids = (int32_t*)calloc((size_t)k, sizeof(int32_t));
            double* wts = (double*)calloc((size_t)k, sizeof(double));
            int32_t rr = L->w_router ? ORC_OK : ORC_E_ARG;
            if (rr == ORC_OK) {
                orc_linear(L->w_router, NULL, ORC_WF_BF16, E, H, h, z, nthreads);
                rr = orc_route(z, E, k, ids, wts);
            }
            if (rr == ORC_OK) {
                for (int32_t j = 0; j < k; ++j) {
                    const int32_t e = ids[j];
                    orc_linear(expert_w(L->w_gu, fmt, e, 2 * I, H), expert_s(L->s_gu, fmt, e, 2 * I, H), fmt,
                               2 * I, H, h, gu, nthreads);
                    for (int32_t r = 0; r < I; ++r) act[r] = gu[I + r] * orc_silu(gu[r]);
                    orc_linear(expert_w(L->w_d, fmt, e, H, I), expert_s(L->s_d, fmt, e, H, I), fmt, H, I, act, y,
                               nthreads);
                    for (int32_t i = 0; i < H; ++i) ysum[i] += wts[j] * y[i];
                }
                for (int32_t i = 0; i < H; ++i) x[i] += ysum[i];
                if (tr && tr->expert_ids) memcpy(tr->expert_ids + (int64_t)l * k, ids, sizeof(int32_t) * k);
                if (tr && tr->expert_w) memcpy(tr->expert_w + (int64_t)l * k, wts, sizeof(double) * k);
            }
            free(z); free(ysum); free(ids); free(wts);
            if (rr != ORC_OK) {
                free(x); free(h); free(y); free(qkv); free(att); free(gu); free(act);
                return rr;
            }
        }
        if (tr && tr->x_out) memcpy(tr->x_out + (int64_t)l * H, x, sizeof(double) * H);
    }

    int32_t ret = 0;
    /* 9. final RMSNorm, the vocabulary-wide logits and the greedy token
     *    ([tiles] sec. 2 "lm_head" and sec. 5). */
    orc_rmsnorm(x, w->final_norm, H, c->rms_eps, h);
    if (tr && tr->h_final) memcpy(tr->h_final, h, sizeof(double) * H);
    if (logits) {
        orc_linear(w->head, NULL, ORC_WF_BF16, V, H, h, logits, nthreads);
        int32_t bad = 0;
        int32_t tok = orc_argmax(logits, V, &bad);
        ret = bad ? ORC_E_NONFINITE : tok;
    }
    free(x); free(h); free(y); free(qkv); free(att); free(gu); free(act);
    return ret;
}

int32_t orc_step(const orc_config* c, const orc_weights* w, int32_t token, int32_t pos,
                 uint16_t* k_cache, uint16_t* v_cache, double* logits, int32_t nthreads) {
    return orc_step_traced(c, w, token, pos, k_cache, v_cache, logits, nthreads, NULL);
}
