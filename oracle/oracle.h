/*
 * oracle.h - plain CPU reference of one batch-1 decode step of a Llama-style
 * decoder.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the GPU library never does.
 *
 * Everything is computed in fp64 from the stored weights (bf16, or 4-bit codes
 * with fp16 group scales), one output element at a time in natural index
 * order.  The only roundings on the path are the ones the stored formats
 * impose: the K/V cache rows are bf16, and the argmax is taken over logits
 * rounded to fp32 (the precision the GPU kernel decides in).
 *
 * Storage conventions (shared with the GPU library only as a documented data
 * format, never as code):
 *   bf16 linear  [rows][cols] uint16 bf16 bits, row r = output r.
 *   int4 linear  [rows][cols/2] bytes, element k in byte k/2, low nibble for
 *                even k; stored code u in 0..15 means q = u - 8; fp16 scale
 *                array [rows][cols/64]; weight = scale * q.
 *   K/V cache    [n_layers][n_kv_heads][max_ctx][head_dim] bf16 bits.
 */
#ifndef TD_ORACLE_H
#define TD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_WF_BF16 = 0, ORC_WF_INT4_G64 = 1 };
enum { ORC_OK = 0, ORC_E_ARG = -1, ORC_E_NONFINITE = -6 };

typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab, max_ctx;
    double rope_theta, rms_eps;
    int32_t weight_format; /* ORC_WF_* for the layer linears; embedding and head are bf16 */
    int32_t qkv_bias;      /* nonzero: b_qkv is added after the QKV projection */
    int32_t n_experts;     /* > 0: the MLP is a mixture of n_experts experts (0: dense) */
    int32_t top_k;         /* experts each token is routed to (MoE only) */
} orc_config;

typedef struct {
    const uint16_t* attn_norm;                 /* bf16 [H] */
    const void* w_qkv; const uint16_t* s_qkv;  /* [(nq+2nkv)d, H] */
    const uint16_t* b_qkv;                     /* bf16 [(nq+2nkv)d] or NULL */
    const void* w_o; const uint16_t* s_o;      /* [H, nq d] */
    const uint16_t* mlp_norm;                  /* bf16 [H] */
    const void* w_gu; const uint16_t* s_gu;    /* [2I, H]: gate rows then up rows */
    const void* w_d; const uint16_t* s_d;      /* [H, I] */
    const uint16_t* w_router;                  /* MoE: bf16 [E, H]; w_gu is [E][2I][H] and
                                                  w_d [E][H][I] (expert e's block at e * rows),
                                                  their scales likewise */
} orc_layer;

typedef struct {
    const uint16_t* embed;      /* bf16 [V, H] */
    const uint16_t* head;       /* bf16 [V, H] (may equal embed) */
    const uint16_t* final_norm; /* bf16 [H] */
    const orc_layer* layers;    /* n_layers entries */
} orc_weights;

/* value conversions of the stored formats */
double orc_bf16_value(uint16_t b);
double orc_f16_value(uint16_t h);
uint16_t orc_round_bf16(double v);   /* via fp32, both steps round to nearest even */

/* one step each; see oracle.c for the passage each follows */
void orc_rmsnorm(const double* x, const uint16_t* gain, int32_t n, double eps, double* y);
double orc_weight(const void* w, const uint16_t* s, int32_t fmt, int32_t cols, int64_t r, int32_t k);
void orc_linear(const void* w, const uint16_t* s, int32_t fmt, int32_t rows, int32_t cols,
                const double* x, double* y, int32_t nthreads);
void orc_rope(double* head_vec, int32_t head_dim, int32_t pos, double theta);
void orc_attention(const double* q, const uint16_t* K, const uint16_t* V, int32_t n_pos,
                   int32_t head_dim, double* out);
double orc_silu(double z);
int32_t orc_argmax(const double* logits, int32_t n, int32_t* nonfinite);
/* MoE routing of one token: the k experts with the largest router logits z[E]
 * (compared rounded to fp32; ties to the lowest id), in that order, into ids[k],
 * and their softmax probabilities over all E experts into weights[k].  Returns
 * ORC_OK, ORC_E_ARG, or ORC_E_NONFINITE when a logit is NaN or infinite. */
int32_t orc_route(const double* z, int32_t E, int32_t k, int32_t* ids, double* weights);

/* The whole step at position `pos` for input `token`: writes K/V row `pos` of
 * every layer into the caches, reads rows 0..pos, and (when logits != NULL)
 * writes the V logits.  Returns the greedy next token (lowest id among the
 * maxima of the fp32-rounded logits), ORC_E_NONFINITE if any logit is NaN/Inf,
 * ORC_E_ARG on bad arguments, or 0 when logits == NULL (prefill). */
int32_t orc_step(const orc_config* cfg, const orc_weights* w, int32_t token, int32_t pos,
                 uint16_t* k_cache, uint16_t* v_cache, double* logits, int32_t nthreads);

/* The same step with every intermediate vector written out (tests only):
 * x_in[H] (embedding), per layer: qkv[(nq+2nkv)d] after bias and RoPE,
 * attn[nq d], x_mid[H], act[I] (dense MLP only), x_out[H]; then h_final[H]; for a
 * MoE model each layer's routed expert ids and weights.  Any pointer may be NULL. */
typedef struct {
    double* x_in;
    double* qkv;    /* [n_layers][(nq+2nkv)d] */
    double* attn;   /* [n_layers][nq d] */
    double* x_mid;  /* [n_layers][H] */
    double* act;    /* [n_layers][I] */
    double* x_out;  /* [n_layers][H] */
    double* h_final;/* [H] */
    int32_t* expert_ids; /* MoE: [n_layers][top_k] routed experts */
    double* expert_w;    /* MoE: [n_layers][top_k] their weights */
} orc_trace;
int32_t orc_step_traced(const orc_config* cfg, const orc_weights* w, int32_t token, int32_t pos,
                        uint16_t* k_cache, uint16_t* v_cache, double* logits, int32_t nthreads,
                        const orc_trace* tr);

#ifdef __cplusplus
}
#endif
#endif
