/*
 * td.h - C ABI of the batch-1 decode-step library for MI355X (gfx950).
 *
 * One call runs one autoregressive decode step of a Llama-style decoder at
 * batch size one: embedding row, then per layer RMSNorm, the fused QKV
 * projection (+ optional bias), half-split RoPE and the K/V-cache write,
 * grouped-query attention over the cache, the output projection and residual,
 * RMSNorm, the gate/up projections with SiLU(gate)*up, the down projection and
 * residual; then the final RMSNorm, the vocabulary-wide logits and the greedy
 * token.  ("Decoding in tiles", sec. 2 lists the chain of steps and sec. 4 how
 * one layer becomes tiles; "One launch per token", "The oracle, then the
 * kernels", lists the same fused set; tinyinfer's "speed limit" section defines
 * the 4-bit format.)
 *
 * All pointers named d_* or described as "device" are device memory of the
 * current HIP device; nothing here allocates host-visible memory for the
 * caller.  Every function returns TD_OK (0) or a negative TD_E_* code and never
 * throws.  One context is used from one host thread and one stream at a time.
 */
#ifndef TD_H
#define TD_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ errors */
enum {
    TD_OK = 0,
    TD_E_INVALID_ARG = -1, /* a null pointer, a bad shape or an unknown option */
    TD_E_UNSUPPORTED = -2, /* the device is not a gfx950 with a CU count the plan handles, or the
                              config is outside what the kernels handle (see td_create) */
    TD_E_PLAN = -3,        /* the work plan failed its validation (bounds, single writer, order) */
    TD_E_RANGE = -4,       /* pos < 0, pos >= max_ctx, or a token id outside [0, vocab) */
    TD_E_HIP = -5,         /* a HIP runtime call failed; td_last_error() holds its message */
    TD_E_NONFINITE = -6,   /* a logit was NaN or Inf (reported by td_status) */
    TD_E_NOMEM = -7,       /* a device allocation failed */
    TD_E_TIMEOUT = -8      /* a grid-wide wait inside the kernel exceeded its time limit */
};

/* --------------------------------------------------------------- formats */
enum {
    TD_WF_BF16 = 0,     /* layer linears stored as bf16, row-major [rows][cols] */
    TD_WF_INT4_G64 = 1  /* layer linears stored as 4-bit codes, [rows][cols/2] bytes: element k in
                           byte k/2, low nibble for even k; code u in 0..15 stands for q = u - 8;
                           plus fp16 scales [rows][cols/64], one per 64 consecutive elements of a
                           row; weight = scale * q (tinyinfer: 4 bits plus one fp16 scale per 64
                           weights). The embedding and the head are bf16 in both formats. */
};

/* Executors behind the same td_decode_step. */
enum {
    TD_EXEC_MEGAKERNEL = 0, /* one persistent kernel over all CUs per step (the default) */
    TD_EXEC_PER_OP = 1,     /* one kernel launch per fused op (baseline) */
    TD_EXEC_GRAPH = 2       /* the per-op launches captured once into a hipGraph and replayed */
};

typedef struct td_config {
    int32_t n_layers;
    int32_t hidden;        /* H */
    int32_t n_q_heads;
    int32_t n_kv_heads;    /* divides n_q_heads; q head h uses kv head h / (n_q_heads / n_kv_heads) */
    int32_t head_dim;      /* d: 64 or 128 */
    int32_t intermediate;  /* I */
    int32_t vocab;         /* V */
    int32_t max_ctx;       /* K/V cache positions */
    float rope_theta;      /* RoPE base: pair (i, i + d/2) turns by pos * theta^(-2i/d) */
    float rms_eps;         /* RMSNorm: x / sqrt(mean(x^2) + eps) * gain */
    int32_t weight_format; /* TD_WF_* (layer linears) */
    int32_t qkv_bias;      /* nonzero: b_qkv is added after the QKV projection, before RoPE */
    int32_t n_experts;     /* 0: dense MLP.  > 0: the MLP is a mixture of n_experts experts of
                              intermediate size I ("One launch per token", its 64-expert MoE
                              section): a router scores the experts, the token goes to the top_k
                              best, and their outputs are added weighted by the router's softmax
                              probabilities (not renormalised over the top_k) */
    int32_t top_k;         /* experts per token (MoE only): 1 .. min(n_experts, TD_MAX_TOPK) */
} td_config;

/* Largest MoE shapes the kernels handle. */
#define TD_MAX_EXPERTS 256
#define TD_MAX_TOPK 16

/* Device pointers of one layer.  Shapes are [rows][cols], row = output.  Every
 * weight pointer (these and those of td_weights) must be 16-byte aligned: the
 * kernels read rows in 16-byte pieces (td_create returns TD_E_INVALID_ARG
 * otherwise; hipMalloc and torch allocations satisfy it). */
typedef struct td_layer_weights {
    const void* attn_norm;  /* bf16 [H] */
    const void* w_qkv;      /* [(nq + 2 nkv) d][H]: q rows, then k rows, then v rows */
    const void* s_qkv;      /* fp16 scales (INT4 only, else NULL) */
    const void* b_qkv;      /* bf16 [(nq + 2 nkv) d] when qkv_bias, else NULL */
    const void* w_o;        /* [H][nq d] */
    const void* s_o;
    const void* mlp_norm;   /* bf16 [H] */
    const void* w_gu;       /* [2 I][H]: gate rows, then up rows */
    const void* s_gu;
    const void* w_d;        /* [H][I] */
    const void* s_d;
    const void* w_router;   /* MoE: bf16 [n_experts][H], else NULL.  With experts, w_gu is
                               [n_experts][2 I][H] and w_d [n_experts][H][I] (expert e's block at
                               row 2 I e, resp. H e) and their int4 scales follow the same rows */
} td_layer_weights;

typedef struct td_weights {
    const void* embed;                /* bf16 [V][H] */
    const void* final_norm;           /* bf16 [H] */
    const void* head;                 /* bf16 [V][H]; may equal embed (tied) */
    const td_layer_weights* layers;   /* host array of n_layers entries */
} td_weights;

/* Caller-owned K/V cache: bf16 [n_layers][n_kv_heads][max_ctx][head_dim] each, 16-byte
 * aligned (the kernels move its rows in 16-byte pieces; TD_E_INVALID_ARG otherwise). */
typedef struct td_kv {
    void* k;
    void* v;
    int32_t max_ctx;  /* must equal the config's max_ctx */
} td_kv;

typedef struct td_ctx td_ctx;

/*
 * td_create: validates the config and the device, builds and validates the
 * work plan, and allocates the context's device scratch (activations, attention
 * partials, barrier words, the token and error words, the RoPE table).
 * `executor` is a TD_EXEC_* value.  The weight buffers are not copied: they
 * must stay valid and unchanged for the life of the context.
 * Errors: TD_E_INVALID_ARG (null pointer, shape not positive, n_kv_heads not
 * dividing n_q_heads, head_dim not 64 or 128, a dimension not a multiple of 64,
 * more than 8 query heads per kv head, missing scales or bias, a weight pointer
 * not 16-byte aligned), TD_E_UNSUPPORTED
 * (device is not gfx950, or its CU count is not a multiple of 8), TD_E_PLAN,
 * TD_E_NOMEM, TD_E_HIP.  On error *out is set to NULL.
 * A mixture-of-experts config ("One launch per token", its 64-expert MoE
 * section) runs on every executor.  On TD_EXEC_MEGAKERNEL the routing happens
 * inside the launch: a router stage publishes the E logits, every CU makes the
 * same top-k choice and streams the chosen experts' rows, gathered by id from
 * a packed copy of all experts (bf16 weights only: TD_E_UNSUPPORTED for int4
 * experts on this executor).  On TD_EXEC_PER_OP and TD_EXEC_GRAPH the router
 * writes the chosen ids to a device tensor and the expert kernels read their
 * weights through it, so one recorded graph replays whatever the routing.
 * Either way td_expert_ids reports the last step's routing.  TD_E_INVALID_ARG
 * for top_k outside [1, min(n_experts, TD_MAX_TOPK)], n_experts above
 * TD_MAX_EXPERTS, or a null w_router.
 */
int td_create(const td_config* cfg, const td_weights* w, int32_t executor, td_ctx** out);

/*
 * td_decode_step: one decode step at position `pos` for the token id stored at
 * the device address d_token (an int32 on the device, so greedy steps chain
 * without a host round trip: pass td_token_ptr(ctx) as the next d_token).
 * Writes K/V row `pos` of every layer into `kv`, reads rows 0..pos, writes the
 * fp32 logits [vocab] to d_logits_out (device, caller-owned) and the greedy
 * token (largest logit, lowest id among ties) to the device int32 at
 * td_token_ptr(ctx).  Asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream); no host synchronisation and no allocation.
 * Errors (before launch): TD_E_INVALID_ARG (null ctx/kv/logits/token, kv
 * max_ctx mismatch), TD_E_RANGE (pos outside [0, max_ctx)), TD_E_HIP.  Errors
 * found on the device (a non-finite logit, a token id out of range, a timed-out
 * grid wait) are reported by td_status.
 */
int td_decode_step(td_ctx* ctx, const int32_t* d_token, int32_t pos, const td_kv* kv, float* d_logits_out,
                   void* stream);

/* Device address of the context's int32 greedy-token word (valid for the ctx's life). */
const int32_t* td_token_ptr(const td_ctx* ctx);

/* MoE routing of the last step (device memory owned by the context, valid for
 * its life; NULL for a dense config): int32 ids [n_layers][top_k], each layer's
 * chosen experts in order of decreasing router logit (ties to the lower id), and
 * float weights [n_layers][top_k], their softmax probabilities over all experts. */
const int32_t* td_expert_ids(const td_ctx* ctx);
const float* td_expert_weights(const td_ctx* ctx);

/* Most steps one td_decode_loop call runs. */
#define TD_MAX_LOOP_STEPS 256

/*
 * td_decode_loop: up to n_steps greedy decode steps in one launch ("Decoding in
 * tiles", sec. 5 and Figure 10: the token loop runs inside the persistent
 * kernel and the workers pick the token themselves).  Step s runs at position
 * pos + s; step 0 takes the token at d_token, every later step the greedy token
 * of the step before, decided on the device: every CU reads every CU's
 * candidate and takes the same token, so the host never sees it.  The loop stops
 * after n_steps steps, after a step whose token is eos_id (eos_id = -1: never),
 * or after a step with a non-finite logit (reported by td_status as
 * TD_E_NONFINITE).  Each step computes exactly what td_decode_step computes:
 * the K/V rows of its position are written to `kv`, d_logits_out holds the last
 * step's fp32 logits [vocab], td_token_ptr(ctx) its token.
 * d_tokens_out (device int32 [n_steps], or NULL) receives the steps' tokens,
 * -1 past the last step run; d_count_out (device int32, or NULL) the number of
 * steps run.  Asynchronous on `stream`, no allocation.
 * Errors (before launch): TD_E_INVALID_ARG (null ctx/kv/logits/token, kv max_ctx
 * mismatch, n_steps outside [1, TD_MAX_LOOP_STEPS], eos_id outside [-1, vocab)),
 * TD_E_UNSUPPORTED (the context's executor is not TD_EXEC_MEGAKERNEL),
 * TD_E_RANGE (pos < 0 or pos + n_steps > max_ctx), TD_E_HIP.  Device-side
 * errors as for td_decode_step, through td_status.
 */
int td_decode_loop(td_ctx* ctx, const int32_t* d_token, int32_t pos, int32_t n_steps, int32_t eos_id,
                   const td_kv* kv, float* d_logits_out, int32_t* d_tokens_out, int32_t* d_count_out, void* stream);

/* Most tokens one td_forward_block call takes. */
#define TD_MAX_BLOCK 64

/*
 * td_forward_block: n consecutive tokens of one sequence through the decoder in
 * one pass over the weights, for a prompt (prefill) or to check drafted tokens
 * (the M = K + 1 verify of speculative decoding).  (tinyinfer, "What I'd tell
 * someone starting, and what's next": a prompt fed one token at a time costs a
 * full weight read per token, and a batch of prompt tokens turns the
 * matrix-vector products into matrix-matrix products on the matrix cores;
 * "Llama 1B: optimizing kernels", "Decode vs Prefill": prefill needs GEMM
 * kernels and its own attention; the flint page, past the MLP-path table: the
 * K + 1 positions of a draft are verified in one launch that reads the weights
 * once.)  Token i (the int32 at d_tokens[i], device) sits at
 * position pos0 + i and attends to positions 0 .. pos0 + i; the K/V rows of
 * positions pos0 .. pos0 + n - 1 of every layer are written to `kv` (rows
 * before pos0 must hold earlier tokens').  Row i of the result equals what
 * td_decode_step computes for token i at position pos0 + i, up to rounding:
 * the linears run as matrix-core products of bf16 weights with each input row
 * split into a bf16 high and low part, fp32 accumulation.
 * all_logits = 0: d_logits_out (device fp32 [vocab]) receives the logits of
 * the last token; nonzero: d_logits_out is [n][vocab], row i token i's.
 * d_argmax_out (device int32 [n] when all_logits, else [1]; or NULL) receives
 * the greedy token of each logits row (largest logit, lowest id among ties);
 * td_token_ptr(ctx) receives the last token's greedy token, so a decode loop
 * can follow without a host round trip.  Uses the context's own workspace:
 * asynchronous on `stream`, no allocation, and not concurrent with another call
 * on the same context.  Works with every executor.
 * Errors (before launch): TD_E_INVALID_ARG (null ctx/tokens/kv/logits, kv
 * max_ctx mismatch, n outside [1, TD_MAX_BLOCK]), TD_E_UNSUPPORTED (a
 * mixture-of-experts config), TD_E_RANGE (pos0 < 0 or pos0 + n > max_ctx),
 * TD_E_HIP.  A token id outside [0, vocab) or a
 * non-finite logit is reported by td_status.
 */
int td_forward_block(td_ctx* ctx, const int32_t* d_tokens, int32_t n, int32_t pos0, const td_kv* kv,
                     float* d_logits_out, int32_t all_logits, int32_t* d_argmax_out, void* stream);

/*
 * td_decode_step_noalloc: one decode step, as td_decode_step computes it on a
 * TD_EXEC_PER_OP context (the same per-op kernels, the same bits), for callers
 * that cannot allocate device memory: code under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc.  There is no context: the config and
 * the weights (as for td_create; device memory that must stay valid until the
 * step has run) are passed each call, and every piece of device scratch the
 * step uses (activations, attention partials, greedy candidates, the layer
 * pointer table, the step's RoPE row) lives in the library's own fixed device
 * array of TD_NOALLOC_SCRATCH_BYTES (4 MiB), one per GPU, held until the
 * process ends.  The call allocates nothing: no hipMalloc, no hipFree, no
 * pinned host memory.  The greedy token goes to d_token_out (device int32), the
 * fp32 logits to d_logits_out (device [vocab]), and d_error_out (device int32)
 * is cleared and then receives the device error bits of the step (1: a
 * non-finite logit, 2: a token id outside [0, vocab)).  Every call on a GPU
 * shares that GPU's array, which keeps the last call's contents: calls that
 * overlap on one GPU (several streams or host threads) race, so serialise them.
 * Asynchronous on `stream`.
 * Errors (before any launch): as td_create for the config and weights,
 * TD_E_INVALID_ARG (a null pointer, kv max_ctx mismatch, a cache pointer not
 * 16-byte aligned), TD_E_RANGE (pos outside [0, max_ctx)), TD_E_UNSUPPORTED
 * (the config needs more scratch than the array holds), TD_E_HIP.
 */
#define TD_NOALLOC_SCRATCH_BYTES (4u << 20)
int td_decode_step_noalloc(const td_config* cfg, const td_weights* w, const int32_t* d_token, int32_t pos,
                           const td_kv* kv, float* d_logits_out, int32_t* d_token_out, int32_t* d_error_out,
                           void* stream);

/*
 * td_status: synchronises the stream of the last td_decode_step, then returns
 * the device error word as a TD_* code (TD_OK, TD_E_NONFINITE, TD_E_RANGE,
 * TD_E_TIMEOUT) and clears it.  *device_error (optional) receives the same code.
 * A TD_E_TIMEOUT leaves the context unusable: destroy it.
 */
int td_status(td_ctx* ctx, int32_t* device_error);

/* Frees the context's own device memory (never the caller's weights, cache or logits). */
void td_destroy(td_ctx* ctx);

/* Static description of an error code. */
const char* td_strerror(int code);

/* The message of the last TD_E_HIP or TD_E_UNSUPPORTED raised in this thread. */
const char* td_last_error(void);

/* ------------------------------------------------------------ test hooks */
/* Each runs one device routine on caller device buffers on `stream`, then
 * synchronises; they exist so that tests can compare one routine with the
 * oracle.  Same error convention. */

/* The work plan without a device ("Decoding in tiles", sec. 4: the schedule is
 * built and checked once, before any launch, and an invalid one is refused).
 * td_plan_check builds the plan td_create would build on a gfx950 with ncu
 * CUs and 160 KiB of LDS per CU (the attention split, every GEMV stage's units
 * over the CUs, the LDS layout, the weight streams) and validates it: TD_OK,
 * or the code td_create would return (TD_E_PLAN for a partition that leaves a
 * unit or a row without an owner, gives one two owners, or leaves the
 * matrix; TD_E_UNSUPPORTED for a config the kernels cannot split, such as
 * more kv heads than CUs, or int4 expert weights; TD_E_INVALID_ARG for a bad
 * config).  With part non-NULL (host int32 [6][ncu + 1], part_len =
 * 6 (ncu + 1): for each unit space -- QKV row pairs, hidden rows,
 * intermediate rows, vocabulary rows, router rows (one per expert), expert
 * gate/up units (top_k slots of intermediate units; every CU's range inside
 * one slot, else TD_E_PLAN) -- the first unit of every CU, then the unit
 * count; the last two spaces are empty for a dense config) the plan uses
 * that partition instead of its own.  td_plan_partition writes the partition the
 * plan builds into part_out (same layout).  Host code only: no HIP call. */
int td_plan_partition(const td_config* cfg, int32_t ncu, int32_t* part_out, int32_t part_len);
int td_plan_check(const td_config* cfg, int32_t ncu, const int32_t* part, int32_t part_len);

/* y[rows] = W x for a bf16 or int4 linear (w, scales: device, row-major as in
 * td_layer_weights; d_x [cols], d_y [rows]: device fp32) through the step's
 * GEMV path: x zero-padded to whole chunks, each row chunk packed as the
 * weight streams pack it (an int4 chunk's codes and its 64-byte scale block)
 * and consumed by the step's chunk dot product.  cols <= 32768 (bf16: a
 * multiple of 8; int4: a multiple of 64, scales non-NULL). */
int td_test_gemv(int32_t weight_format, const void* w, const void* scales, int32_t rows, int32_t cols,
                 const float* d_x, float* d_y, void* stream);

/* One query head's attention over n_pos bf16 K/V rows ([n_pos][head_dim], device), fp32 q and
 * out [head_dim] (device): softmax(q . K^T / sqrt(d)) V with the decode step's own routines
 * ("One launch per token", "The attention trap": split-K partials merged with the
 * e^(m_c - M) rescale): the positions are cut into chunks of chunk_len (a multiple of 64; 0 =
 * one chunk for all), each chunk runs the step's 64-row tile routine over its tiles as
 * waves_per_head waves of one head do in the step (wave s takes rows [s 64 / W, (s + 1) 64 / W)
 * of every tile; the W states are then folded in wave order by the step's routine), and the
 * chunks' partials are merged by the step's merge routine in chunk order.  waves_per_head: 1, 2
 * or 4, or 8 at head_dim 128 (the step uses 8, or 4 at head_dim 64, for a model with one query
 * head per kv head, else 1).  At most 64 chunks (TD_E_INVALID_ARG otherwise, or for head_dim not
 * 64 or 128). */
int td_test_attention(const float* d_q, const void* k, const void* v, int32_t n_pos, int32_t head_dim,
                      int32_t chunk_len, int32_t waves_per_head, float* d_out, void* stream);

/* Half-split RoPE of n_heads vectors of head_dim fp32 values (d_x, d_out: device
 * [n_heads][head_dim]) at position pos, with the step's rotation and a table row
 * built as td_create builds its table (pair (i, i + d/2) turns by
 * pos * rope_theta^(-2i/d); angle, cosine and sine in double, rounded to fp32;
 * the flint page's chat.py passage on half-split RoPE). */
int td_test_rope(const float* d_x, int32_t n_heads, int32_t head_dim, int32_t pos, float rope_theta, float* d_out,
                 void* stream);

/* The greedy token of n fp32 logits (d_logits, device) by the step's selection
 * ("Decoding in tiles", sec. 5): `groups` workgroups (1 .. n) each take a
 * contiguous share of the vocabulary as the plan splits it among the CUs, lanes
 * of 8 waves run over their rows, and the candidates are reduced wave, then
 * workgroup, then across workgroups; the largest finite logit wins, the lowest
 * id among equal ones.  *d_token (device int32) receives it (0 if no logit is
 * finite), *d_nonfinite (device int32) 1 if any logit is NaN or infinite, else 0.
 * d_work: device scratch of at least 12 * groups bytes, caller-owned. */
int td_test_argmax(const float* d_logits, int32_t n, int32_t groups, void* d_work, int32_t* d_token,
                   int32_t* d_nonfinite, void* stream);

/* In-kernel stage trace (the per-worker timeline of one step).  td_trace_bytes
 * gives the size of the trace: for each CU and each stage of the step (5 per
 * layer plus the head), a record of 32 uint64 timestamps of the 100 MHz device
 * clock, four per compute wave w at [4 w .. 4 w + 3]: stage entered, inputs
 * staged (the workgroup rendezvous passed), first weight chunk in LDS (first
 * attention tile done), last output published; 0 where the wave had no part
 * in the stage.  td_set_trace(ctx, d_buf, bytes) makes every following step
 * write it to the device buffer d_buf (caller-owned, at least td_trace_bytes
 * bytes); d_buf = NULL turns it off.  TD_E_INVALID_ARG for a buffer that is
 * too small. */
int64_t td_trace_bytes(const td_ctx* ctx);
int td_set_trace(td_ctx* ctx, void* d_buf, int64_t bytes);

/* Per-step clock of the token loop.  td_set_step_clock(ctx, d_buf, n) makes
 * every following td_decode_loop (and td_decode_step on the persistent
 * kernel) write the device's 100 MHz clock into d_buf (device uint64 [n],
 * caller-owned, n >= 2): [0] when the launch starts, [s + 1] when step s's
 * greedy token has been decided (on the first CU; every CU decides it from
 * the same candidates at the same moment), for s + 1 < n.  Step s took
 * d_buf[s + 1] - d_buf[s] ticks.  d_buf = NULL turns it off. */
int td_set_step_clock(td_ctx* ctx, uint64_t* d_buf, int32_t n);

/* The stream-read yardstick ("Decoding in tiles", sec. 2: the measured rate
 * of a plain streaming read, against which a weight-read floor is set): one
 * warm-up pass and then `reps` timed passes of a kernel that reads `bytes`
 * (a multiple of 16; d_buf device, 16-byte aligned) with 16-byte
 * non-temporal loads, one workgroup per CU reading 32 KiB contiguous per
 * pass.  *ms_out (host) receives the time of the
 * `reps` passes; the rate is bytes * reps / time.  Synchronises `stream`. */
int td_measure_stream(const void* d_buf, int64_t bytes, int32_t reps, float* ms_out, void* stream);

/* Measured duration of the last megakernel step (HIP events on the step's own
 * stream), or a negative value when unavailable.  Timing is off unless enabled. */
int td_set_timing(td_ctx* ctx, int32_t enable);
float td_last_step_ms(td_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif
