// td_api.cpp - host side of the C ABI declared in include/td.h.
//
// td_create validates the config and the device, builds the static work plan
// (which CU and wave owns which rows of every stage, how the attention context
// is split, where everything sits in LDS), validates it, and allocates the
// context's scratch.  td_decode_step fills the per-step fields and launches the
// persistent kernel cooperatively: every workgroup must be resident at once,
// since each one spins on values that other workgroups publish (there is no
// grid barrier; the hand-offs are tagged values in global memory).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "td.h"
#include "td_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return TD_E_HIP;
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace

struct td_ctx {
  td_config cfg;
  int executor = TD_EXEC_MEGAKERNEL;
  int ncu = 0;
  int ring = 0;
  td_kparams kp{};
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  void* wstream = nullptr;      // packed weight streams (code chunks, then int4 scales)
  size_t wstream_bytes = 0;
  td_layer_dev* d_layers = nullptr;
  float* d_rope = nullptr;
  hipStream_t last_stream = nullptr;
  bool launched = false;
  bool timing = false;
  bool timed = false;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  // per-op and graph executors
  td_opparams op{};
  void* opbuf = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  hipStream_t cap_stream = nullptr;
  const void* g_kc = nullptr;  // the K/V cache and logits the captured graph was made for
  const void* g_vc = nullptr;
  const void* g_logits = nullptr;
  // block forward (td_forward_block): workspace and the layer pointers on the host
  void* blockbuf = nullptr;
  td_blockparams blk{};
  std::vector<td_layer_dev> layers_host;
};

namespace {

// One position's RoPE table row: pair i (i < d/2) turns by the angle
// pos * theta^(-2i/d); the angle, its cosine and its sine are computed in
// double and rounded to fp32 (cs[2 i] = cos, cs[2 i + 1] = sin).
void rope_row(float theta, int d, int pos, float* cs) {
  for (int i = 0; i < d / 2; ++i) {
    const double ang = (double)pos * std::pow((double)theta, -2.0 * i / d);
    cs[2 * i] = (float)std::cos(ang);
    cs[2 * i + 1] = (float)std::sin(ang);
  }
}

// Builds the partition table: CU c owns units [part[s][c], part[s][c + 1]) of
// unit space s, in proportion to the per-CU weights (all 1 unless a weighting
// is given), so that every unit has exactly one owner.
std::vector<int32_t> build_partition(const td_config& c, int ncu, const std::vector<double>& wt) {
  const int64_t E = c.n_experts > 0 ? c.n_experts : 0, k = E ? c.top_k : 0, I = c.intermediate;
  const int64_t U[TD_NSPACES] = {(int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim / 2, c.hidden,
                                 I, c.vocab, E, k * I};
  std::vector<double> cum(ncu + 1, 0.0);
  for (int i = 0; i < ncu; ++i) cum[i + 1] = cum[i] + wt[i];
  std::vector<int32_t> part((size_t)TD_NSPACES * (ncu + 1));
  for (int sp = 0; sp < TD_NSPACES; ++sp) {
    int32_t* t = part.data() + (size_t)sp * (ncu + 1);
    if (sp == TD_SP_EI && k > 0) {
      // slot j (the j-th chosen expert's I units) goes to CUs [j ncu / k, (j + 1) ncu / k):
      // no CU's range crosses a slot, so each wave streams one expert's rows
      for (int64_t j = 0; j < k; ++j) {
        const int64_t c0 = j * ncu / k, c1 = (j + 1) * ncu / k;
        for (int64_t i = c0; i < c1; ++i) t[i] = (int32_t)(j * I + (I * (i - c0)) / (c1 - c0));
      }
      t[ncu] = (int32_t)(k * I);
      continue;
    }
    for (int i = 0; i <= ncu; ++i)
      t[i] = i == ncu ? (int32_t)U[sp] : (int32_t)std::llround((double)U[sp] * cum[i] / cum[ncu]);
  }
  return part;
}

// Enumerates the row ownership of every GEMV stage exactly as the kernel
// derives it from the partition table and checks: every unit of every stage is
// owned by exactly one (CU, wave); every row is produced once; all rows are
// inside the matrix; a CU's residual rows fit the LDS area; a wave's QKV units
// fit one wavefront (their biases are held one per lane).
int validate_plan(const td_config& c, int ncu, const std::vector<int32_t>& part, int own_floats) {
  const int d = c.head_dim, H = c.hidden, I = c.intermediate, V = c.vocab;
  const int qkv_rows = (c.n_q_heads + 2 * c.n_kv_heads) * d;
  const int E = c.n_experts > 0 ? c.n_experts : 0, k = E ? c.top_k : 0;
  // the expert gate/up space (kind -1): unit u is slot u / I, rows (gate, up) of
  // row u % I of the slot's expert, counted here as 2 u and 2 u + 1
  struct St {
    int U, rpu, rows, kind, space;
  } st[] = {{qkv_rows / 2, 2, qkv_rows, TD_ST_QKV, TD_SP_QKV}, {H, 1, H, TD_ST_O, TD_SP_H},
            {I, 2, 2 * I, TD_ST_GU, TD_SP_I}, {H, 1, H, TD_ST_DOWN, TD_SP_H}, {V, 1, V, TD_ST_HEAD, TD_SP_V},
            {E, 1, E, TD_ST_ROUTER, TD_SP_E}, {k * I, 2, 2 * k * I, -1, TD_SP_EI}};
  for (const St& s : st) {
    std::vector<uint8_t> seen_row(s.rows, 0);
    std::vector<uint8_t> seen_unit(s.U, 0);
    const int32_t* t = part.data() + (size_t)s.space * (ncu + 1);
    if (t[0] != 0 || t[ncu] != s.U) return fail(TD_E_PLAN, "partition does not cover the unit space");
    for (int cu = 0; cu < ncu; ++cu) {
      const int u0 = t[cu], u1 = t[cu + 1];
      if (u0 < 0 || u1 > s.U || u1 < u0) return fail(TD_E_PLAN, "unit range out of bounds");
      if (s.space == TD_SP_H && u1 - u0 > own_floats) return fail(TD_E_PLAN, "residual rows exceed the LDS area");
      if (s.space == TD_SP_QKV && (u1 - u0 + TD_NW - 1) / TD_NW > 64)
        return fail(TD_E_UNSUPPORTED, "more than 64 QKV row pairs per compute wave");
      if (s.space == TD_SP_EI && u1 > u0 && u0 / I != (u1 - 1) / I)
        return fail(TD_E_PLAN, "a CU's expert units cross a slot");
      for (int wave = 0; wave < TD_NW; ++wave) {
        for (int u = u0 + wave; u < u1; u += TD_NW) {
          if (seen_unit[u]++) return fail(TD_E_PLAN, "unit owned twice");
          for (int r = 0; r < s.rpu; ++r) {
            int row;
            if (s.kind == TD_ST_QKV) {
              int half = d / 2, head = u / half, i = u - head * half;
              row = head * d + i + r * half;
            } else if (s.kind == TD_ST_GU) {
              row = u + r * I;
            } else if (s.kind == -1) {
              row = 2 * u + r;
            } else {
              row = u;
            }
            if (row < 0 || row >= s.rows) return fail(TD_E_PLAN, "row outside the matrix");
            if (seen_row[row]++) return fail(TD_E_PLAN, "row written twice");
          }
        }
      }
    }
    for (int r = 0; r < s.rows; ++r)
      if (!seen_row[r]) return fail(TD_E_PLAN, "row without a writer");
  }
  return TD_OK;
}

int check_config(const td_config* c) {
  if (!c) return fail(TD_E_INVALID_ARG, "null config");
  if (c->n_layers <= 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->intermediate <= 0 ||
      c->vocab <= 0 || c->max_ctx <= 0)
    return fail(TD_E_INVALID_ARG, "non-positive dimension");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(TD_E_INVALID_ARG, "head_dim must be 64 or 128");
  if (c->n_q_heads % c->n_kv_heads) return fail(TD_E_INVALID_ARG, "n_kv_heads must divide n_q_heads");
  if (c->n_q_heads / c->n_kv_heads > TD_MAX_GROUP) return fail(TD_E_INVALID_ARG, "more than 8 q heads per kv head");
  if (c->hidden % 256) return fail(TD_E_INVALID_ARG, "hidden must be a multiple of 256");
  if (c->intermediate % 64) return fail(TD_E_INVALID_ARG, "intermediate must be a multiple of 64");
  if (c->weight_format != TD_WF_BF16 && c->weight_format != TD_WF_INT4_G64)
    return fail(TD_E_INVALID_ARG, "unknown weight format");
  if (c->weight_format == TD_WF_INT4_G64 &&
      ((c->hidden % 128) || (c->intermediate % 128) || ((c->n_q_heads * c->head_dim) % 128)))
    return fail(TD_E_INVALID_ARG, "int4 needs every K to be a multiple of 128");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(TD_E_INVALID_ARG, "bad rope_theta or rms_eps");
  if (c->n_experts < 0 || c->n_experts > TD_MAX_EXPERTS) return fail(TD_E_INVALID_ARG, "n_experts out of range");
  if (c->n_experts > 0 && (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > TD_MAX_TOPK))
    return fail(TD_E_INVALID_ARG, "top_k out of range");
  return TD_OK;
}

int check_weights(const td_config* c, const td_weights* w) {
  if (!w || !w->embed || !w->final_norm || !w->head || !w->layers) return fail(TD_E_INVALID_ARG, "null weight pointer");
  const bool q4 = c->weight_format == TD_WF_INT4_G64;
  for (int l = 0; l < c->n_layers; ++l) {
    const td_layer_weights& L = w->layers[l];
    if (!L.attn_norm || !L.w_qkv || !L.w_o || !L.mlp_norm || !L.w_gu || !L.w_d)
      return fail(TD_E_INVALID_ARG, "null layer weight pointer");
    if (q4 && (!L.s_qkv || !L.s_o || !L.s_gu || !L.s_d)) return fail(TD_E_INVALID_ARG, "int4 layer without scales");
    if (c->qkv_bias && !L.b_qkv) return fail(TD_E_INVALID_ARG, "qkv_bias set but b_qkv is null");
    if (c->n_experts > 0 && !L.w_router) return fail(TD_E_INVALID_ARG, "MoE layer without router weights");
    for (const void* p : {L.attn_norm, L.w_qkv, L.s_qkv, L.b_qkv, L.w_o, L.s_o, L.mlp_norm, L.w_gu, L.s_gu, L.w_d,
                          L.s_d, L.w_router})
      if ((uintptr_t)p & 15) return fail(TD_E_INVALID_ARG, "layer weight pointer not 16-byte aligned");
  }
  for (const void* p : {w->embed, w->final_norm, w->head})
    if ((uintptr_t)p & 15) return fail(TD_E_INVALID_ARG, "weight pointer not 16-byte aligned");
  return TD_OK;
}

// The per-op executor's parameters and fp32 activation buffers (one allocation).
int setup_per_op(td_ctx* ctx, const td_kparams& kp) {
  td_opparams& op = ctx->op;
  op.L = kp.L;
  op.H = kp.H;
  op.nq = kp.nq;
  op.nkv = kp.nkv;
  op.d = kp.d;
  op.I = kp.I;
  op.V = kp.V;
  op.max_ctx = kp.max_ctx;
  op.wf = kp.wf;
  op.has_bias = kp.has_bias;
  op.qd = kp.qd;
  op.kvd = kp.kvd;
  op.qkv_rows = kp.qkv_rows;
  op.group = kp.group;
  op.eps = kp.eps;
  op.attn_scale = kp.attn_scale;
  op.chunk_len = kp.chunk_len;
  op.n_chunks_max = kp.n_chunks_max;
  op.E = ctx->cfg.n_experts;
  op.topk = op.E > 0 ? ctx->cfg.top_k : 0;
  op.layers = kp.layers;
  op.embed = kp.embed;
  op.head = kp.head;
  op.final_norm = kp.final_norm;
  op.rope_cs = kp.rope_cs;
  op.token_out = kp.token_out;
  op.err = kp.err;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  const size_t o_pos = take(4), o_x = take((size_t)op.H * 4), o_q = take((size_t)op.qd * 4);
  const size_t o_part = take((size_t)op.nkv * op.n_chunks_max * op.group * (op.d + 4) * 4);
  const size_t o_o = take((size_t)op.qd * 4), o_act = take((size_t)op.I * std::max(1, op.topk) * 4);
  const size_t o_cand = take((size_t)td_op_head_blocks(&op) * 16);
  const size_t o_rl = take((size_t)std::max(1, op.E) * 4), o_eid = take((size_t)op.L * std::max(1, op.topk) * 4);
  const size_t o_ew = take((size_t)op.L * std::max(1, op.topk) * 4);
  hipError_t e = hipMalloc(&ctx->opbuf, off);
  if (e != hipSuccess) return e == hipErrorOutOfMemory ? fail(TD_E_NOMEM, "hipMalloc of per-op buffers failed")
                                                       : hip_fail(e, "hipMalloc");
  e = hipMemset(ctx->opbuf, 0, off);
  if (e != hipSuccess) {
    (void)hipFree(ctx->opbuf);
    ctx->opbuf = nullptr;
    return hip_fail(e, "hipMemset");
  }
  uint8_t* b = (uint8_t*)ctx->opbuf;
  op.pos_word = (int32_t*)(b + o_pos);
  op.x = (float*)(b + o_x);
  op.q = (float*)(b + o_q);
  op.part = (float*)(b + o_part);
  op.o = (float*)(b + o_o);
  op.act = (float*)(b + o_act);
  op.cand = (uint32_t*)(b + o_cand);
  op.rlogits = (float*)(b + o_rl);
  op.expert_ids = op.E > 0 ? (int32_t*)(b + o_eid) : nullptr;
  op.expert_w = op.E > 0 ? (float*)(b + o_ew) : nullptr;
  int le = td_op_set_lds_limits(&op);
  if (le) {
    (void)hipFree(ctx->opbuf);
    ctx->opbuf = nullptr;
    return hip_fail((hipError_t)le, "hipFuncSetAttribute");
  }
  return TD_OK;
}

void drop_graph(td_ctx* ctx) {
  if (ctx->gexec) (void)hipGraphExecDestroy(ctx->gexec);
  if (ctx->graph) (void)hipGraphDestroy(ctx->graph);
  ctx->gexec = nullptr;
  ctx->graph = nullptr;
}

// Captures every launch after op_begin into a graph (once per K/V cache and
// logits buffer) on a private stream; no memset node is ever recorded.
int capture_graph(td_ctx* ctx) {
  drop_graph(ctx);
  hipError_t e = hipSuccess;
  if (!ctx->cap_stream) e = hipStreamCreateWithFlags(&ctx->cap_stream, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "hipStreamCreate");
  e = hipStreamBeginCapture(ctx->cap_stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
  const int le = td_launch_op_layers(&ctx->op, ctx->cap_stream);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(ctx->cap_stream, &g);
  if (le) {
    if (g) (void)hipGraphDestroy(g);
    return hip_fail((hipError_t)le, "launch during capture");
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  ctx->graph = g;
  e = hipGraphInstantiate(&ctx->gexec, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    drop_graph(ctx);
    return hip_fail(e, "hipGraphInstantiate");
  }
  ctx->g_kc = ctx->op.kc;
  ctx->g_vc = ctx->op.vc;
  ctx->g_logits = ctx->op.logits;
  return TD_OK;
}

// The static plan of the persistent kernel for a device of ncu CUs with
// lds_cap bytes of LDS per CU: the attention split, the partition of every
// GEMV stage's units over the CUs (part_in: a caller's table to validate
// instead, TD_NSPACES x (ncu + 1) entries), the LDS layout with the ring
// depth, and every compute wave's packed stream.  Host arithmetic only: no
// device call, so the plan and its validation can be tested without a GPU.
struct Plan {
  td_kparams kp{};
  int chunk_len = 0, n_chunks_max = 0;
  std::vector<int32_t> part;
  std::vector<td_wstream> ws;
  uint64_t stream_code_chunks = 0, stream_scale_blocks = 0;
};

// The attention split of a config on ncu CUs: at most one task per CU, chunks
// a multiple of the tile, at most 64 chunks per kv head, and the merge staging
// within the LDS the GEMV input area and the first K/V tile buffer already take
// (the attention area aliases the input area; the merge runs once the CU's own
// tiles are consumed, so its staging may run on into the tile buffer), at
// least 24 KiB: more chunks mean fewer tiles per CU, which a CU runs one by
// one.  No allocation.
int attention_split(const td_config& c, int ncu, int* chunk_len_out, int* n_chunks_out) {
  const int d = c.head_dim, H = c.hidden, I = c.intermediate;
  const int nq = c.n_q_heads, nkv = c.n_kv_heads, group = nq / nkv, qd = nq * d;
  if (nkv > ncu) return fail(TD_E_UNSUPPORTED, "more kv heads than CUs: the attention split needs a CU per kv head");
  const int cmax_by_cu = ncu / nkv;
  int chunk_len = (int)round_up(std::max<int64_t>(1, ((int64_t)c.max_ctx + cmax_by_cu - 1) / cmax_by_cu), TD_TILE);
  auto n_chunks_of = [&](int cl) { return (c.max_ctx + cl - 1) / cl; };
  const int64_t topk_i = c.n_experts > 0 ? (int64_t)td_moe_down_reach(c.top_k, I) : 0;
  const int64_t kpad_in = round_up(std::max<int64_t>({H, qd, I, topk_i}), 2048);
  const int64_t merge_budget = std::max<int64_t>(
      24 * 1024, kpad_in * 4 + td_tile_bytes(d) - (int64_t)td_attn_layout(d, group, 1, c.n_experts > 0).merge);
  while (n_chunks_of(chunk_len) > 64 || (int64_t)n_chunks_of(chunk_len) * group * (d + 4) * 4 > merge_budget)
    chunk_len += TD_TILE;
  const int n_chunks_max = n_chunks_of(chunk_len);
  if (n_chunks_max * nkv > ncu) return fail(TD_E_PLAN, "attention split exceeds the CU count");
  *chunk_len_out = chunk_len;
  *n_chunks_out = n_chunks_max;
  return TD_OK;
}

// persistent: the plan is for the persistent kernel (which refuses int4 expert
// weights); the per-op executors build it for the shapes and the attention split.
int build_plan(const td_config* cfg, int ncu, int64_t lds_cap, const int32_t* part_in, bool persistent, Plan& out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (ncu <= 0 || ncu % 8) return fail(TD_E_UNSUPPORTED, "CU count must be a positive multiple of 8");
  const td_config& c = *cfg;
  const int d = c.head_dim, H = c.hidden, I = c.intermediate, L = c.n_layers;
  const int nq = c.n_q_heads, nkv = c.n_kv_heads, group = nq / nkv;
  const int qd = nq * d;
  const int E = c.n_experts > 0 ? c.n_experts : 0, topk = E ? c.top_k : 0;
  if (persistent && E && c.weight_format != TD_WF_BF16)
    return fail(TD_E_UNSUPPORTED, "the persistent kernel runs mixture-of-experts layers on bf16 weights only");
  if (E && ncu < topk) return fail(TD_E_UNSUPPORTED, "fewer CUs than experts per token");

  int chunk_len = 0, n_chunks_max = 0;
  rc = attention_split(c, ncu, &chunk_len, &n_chunks_max);
  if (rc) return rc;

  // partition of every GEMV stage's units over the CUs (or the caller's, for the plan test)
  std::vector<int32_t> part = build_partition(c, ncu, std::vector<double>(ncu, 1.0));
  if (part_in) part.assign(part_in, part_in + part.size());
  int own_floats = 0;
  for (int i = 0; i < ncu; ++i)
    own_floats = std::max(own_floats, part[(size_t)TD_SP_H * (ncu + 1) + i + 1] - part[(size_t)TD_SP_H * (ncu + 1) + i]);
  own_floats = (int)round_up(std::max(own_floats, 1), 64);
  // the LDS output area holds a CU's dot products of one stage (rpu per unit)
  int out_floats = 0;
  for (int i = 0; i < ncu; ++i) {
    auto cnt = [&](int sp) { return part[(size_t)sp * (ncu + 1) + i + 1] - part[(size_t)sp * (ncu + 1) + i]; };
    out_floats = std::max({out_floats, 2 * cnt(TD_SP_QKV), cnt(TD_SP_H), 2 * cnt(TD_SP_I), cnt(TD_SP_V), cnt(TD_SP_E),
                           2 * cnt(TD_SP_EI)});
  }
  out_floats = (int)round_up(std::max(out_floats, 1), 64);

  // LDS layout: the rings take what the rest leaves, up to TD_RING_MAX slots per wave
  const td_attn_lds A = td_attn_layout(d, group, n_chunks_max, E > 0);
  // the GEMV input area holds the longest input: a MoE down stage's is top_k slots of I
  // (a MoE down stage reads its last slot's whole chunks: td_moe_down_reach)
  const int64_t kpad = round_up(std::max({H, qd, I, E ? td_moe_down_reach(topk, I) : 0}), 2048);
  // the attention area aliases the input area; its merge staging (used after the
  // CU's tiles) may run on into the first tile buffer, which follows
  const int64_t xin_bytes = std::max<int64_t>({kpad * 4, (int64_t)A.merge, A.bytes - td_tile_bytes(d)});
  td_kparams kp{};
  int64_t fixed = 0;
  const int64_t per_slot = (int64_t)TD_NW * (TD_CHUNK + (c.weight_format == TD_WF_INT4_G64 ? TD_SCHUNK : 0));
  // more K/V tile buffers (nb - 1 tiles in flight while one is consumed) when a
  // chunk spans at least nb tiles and the rings keep at least TD_RING_MIN2
  // (two buffers) or TD_RING_MIN3 (three) slots; three only at d = 64, where a
  // tile is 17 copy instructions and two tiles in flight stay within the wait
  // counts the sync wave uses (34)
  kp.tile_stride = (int32_t)round_up(td_tile_bytes(d), 256);
  kp.tile_bufs = 1;
  for (int nb = d == 64 ? 3 : 2; nb >= 1; --nb) {
    int64_t off = 0;
    kp.off_xin = kp.off_attn = (int32_t)off;
    off += round_up(xin_bytes, 1024);
    kp.off_tile = (int32_t)off;
    kp.merge_in_tile = A.bytes > kp.off_tile - kp.off_attn ? 1 : 0;
    off += (int64_t)nb * kp.tile_stride;
    kp.off_own = (int32_t)off;
    off += (int64_t)own_floats * 4;
    kp.off_out = (int32_t)off;
    off += (int64_t)out_floats * 4;
    kp.off_rope = (int32_t)off;
    off += round_up((int64_t)d * 4, 256);
    kp.off_ctl = (int32_t)off;
    off += TD_CTL_WORDS * 4;
    kp.off_route = (int32_t)off;
    if (E) off += (TD_MAX_EXPERTS + TD_NW * 2 * TD_MAX_TOPK) * 4;
    fixed = round_up(off, 1024);
    kp.tile_bufs = nb;
    if (nb == 1 || (chunk_len > (nb - 1) * TD_TILE && (lds_cap - fixed) / per_slot >= (nb == 3 ? TD_RING_MIN3 : TD_RING_MIN2)))
      break;
  }
  const int64_t ring = std::min<int64_t>(TD_RING_MAX, (lds_cap - fixed) / per_slot);
  if (ring < TD_RING_MIN) return fail(TD_E_UNSUPPORTED, "the LDS cannot hold the weight rings for this shape");
  {
    // rings first (1 KiB aligned), then the fixed areas shifted behind them
    const int32_t ring_bytes = (int32_t)((int64_t)TD_NW * ring * TD_CHUNK);
    const int32_t sring_bytes =
        c.weight_format == TD_WF_INT4_G64 ? (int32_t)round_up((int64_t)TD_NW * ring * TD_SCHUNK, 1024) : 0;
    kp.off_ring = 0;
    kp.off_sring = ring_bytes;
    const int32_t shift = ring_bytes + sring_bytes;
    kp.off_xin += shift;
    kp.off_attn += shift;
    kp.off_tile += shift;
    kp.off_own += shift;
    kp.off_out += shift;
    kp.off_rope += shift;
    kp.off_ctl += shift;
    kp.off_route += shift;
    kp.lds_bytes = (int32_t)(shift + fixed);
  }
  if (kp.lds_bytes > lds_cap) return fail(TD_E_UNSUPPORTED, "LDS layout exceeds the CU's LDS");
  // the greedy candidates of all CUs are gathered in the attention tile area
  if ((int64_t)ncu * 16 > td_tile_bytes(d)) return fail(TD_E_UNSUPPORTED, "too many CUs for the candidate area");
  kp.ring_slots = (int32_t)ring;


  rc = validate_plan(c, ncu, part, own_floats);
  if (rc) return rc;

  uint64_t stream_code_chunks = 0, stream_scale_blocks = 0;
  // every compute wave's packed stream, counted exactly as the kernel walks it:
  // stages in order (attention has no weights), for a MoE gate/up or down stage
  // every expert in turn (ne = E), the wave's units, their rows, the row's chunks
  std::vector<td_wstream> ws((size_t)ncu * TD_NW);
  {
    struct St {
      int space, rpu, K, fmt, ne;
    };
    std::vector<St> stages;
    for (int l = 0; l < L; ++l) {
      stages.push_back({TD_SP_QKV, 2, H, c.weight_format, 1});
      stages.push_back({TD_SP_H, 1, qd, c.weight_format, 1});
      if (E) {
        stages.push_back({TD_SP_E, 1, H, TD_WF_BF16, 1});
        stages.push_back({TD_SP_EI, 2, H, c.weight_format, E});
        stages.push_back({TD_SP_H, 1, I, c.weight_format, E});
      } else {
        stages.push_back({TD_SP_I, 2, H, c.weight_format, 1});
        stages.push_back({TD_SP_H, 1, I, c.weight_format, 1});
      }
    }
    stages.push_back({TD_SP_V, 1, H, TD_WF_BF16, 1});
    uint64_t code = 0, scal = 0;
    for (int cu = 0; cu < ncu; ++cu)
      for (int wave = 0; wave < TD_NW; ++wave) {
        uint64_t nt = 0, n4 = 0;
        for (const St& st : stages) {
          const int32_t* t = part.data() + (size_t)st.space * (ncu + 1);
          const int cnt = t[cu + 1] - t[cu];
          const int n = cnt > wave ? (cnt - wave + TD_NW - 1) / TD_NW : 0;
          const int row_bytes = st.fmt == TD_WF_BF16 ? st.K * 2 : st.K / 2;
          const uint64_t ch = (uint64_t)st.ne * n * st.rpu * ((row_bytes + TD_CHUNK - 1) / TD_CHUNK);
          nt += ch;
          if (st.fmt == TD_WF_INT4_G64) n4 += ch;
        }
        if (code + nt > 0xffffffffull || scal + n4 > 0xffffffffull) return fail(TD_E_UNSUPPORTED, "model too large");
        ws[(size_t)cu * TD_NW + wave] = {(uint32_t)code, (uint32_t)scal, (uint32_t)nt, (uint32_t)n4};
        code += nt;
        scal += n4;
      }
    stream_code_chunks = code;
    stream_scale_blocks = scal;
  }

  out.kp = kp;
  out.chunk_len = chunk_len;
  out.n_chunks_max = n_chunks_max;
  out.part = part;
  out.ws = ws;
  out.stream_code_chunks = stream_code_chunks;
  out.stream_scale_blocks = stream_scale_blocks;
  return TD_OK;
}

}  // namespace

extern "C" {

const char* td_strerror(int code) {
  switch (code) {
    case TD_OK: return "ok";
    case TD_E_INVALID_ARG: return "invalid argument";
    case TD_E_UNSUPPORTED: return "unsupported device or config";
    case TD_E_PLAN: return "work plan failed validation";
    case TD_E_RANGE: return "position or token id out of range";
    case TD_E_HIP: return "HIP runtime error";
    case TD_E_NONFINITE: return "non-finite logit";
    case TD_E_NOMEM: return "device allocation failed";
    case TD_E_TIMEOUT: return "grid-wide wait timed out";
    default: return "unknown error";
  }
}

const char* td_last_error(void) { return g_last_error.c_str(); }

int td_create(const td_config* cfg, const td_weights* w, int32_t executor, td_ctx** out) {
  if (!out) return fail(TD_E_INVALID_ARG, "null out pointer");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  rc = check_weights(cfg, w);
  if (rc) return rc;
  if (executor != TD_EXEC_MEGAKERNEL && executor != TD_EXEC_PER_OP && executor != TD_EXEC_GRAPH)
    return fail(TD_E_INVALID_ARG, "unknown executor");

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(TD_E_UNSUPPORTED, std::string("needs gfx950, found ") + prop.gcnArchName);
  const int ncu = prop.multiProcessorCount;
  if (ncu <= 0 || ncu % 8) return fail(TD_E_UNSUPPORTED, "CU count must be a positive multiple of 8");
  if (!prop.cooperativeLaunch) return fail(TD_E_UNSUPPORTED, "device lacks cooperative launch");

  Plan plan;
  rc = build_plan(cfg, ncu, std::min<int64_t>((int64_t)prop.maxSharedMemoryPerMultiProcessor, 160 * 1024), nullptr,
                  executor == TD_EXEC_MEGAKERNEL, plan);
  if (rc) return rc;
  td_kparams kp = plan.kp;
  if (executor == TD_EXEC_MEGAKERNEL) {
    int blocks = 0;
    const int oe = td_megakernel_occupancy(cfg->head_dim, cfg->weight_format, cfg->n_experts > 0, kp.lds_bytes, &blocks);
    if (oe != 0 || blocks < 1) return fail(TD_E_UNSUPPORTED, "the kernel does not fit one workgroup per CU");
  }
  const td_config& c = *cfg;
  const int d = c.head_dim, H = c.hidden, I = c.intermediate, V = c.vocab, L = c.n_layers;
  const int nq = c.n_q_heads, nkv = c.n_kv_heads, group = nq / nkv;
  const int qd = nq * d, kvd = nkv * d, qkv_rows = qd + 2 * kvd;
  const int E = c.n_experts > 0 ? c.n_experts : 0, topk = E ? c.top_k : 0;
  const int chunk_len = plan.chunk_len, n_chunks_max = plan.n_chunks_max;
  const std::vector<int32_t>& part = plan.part;
  const std::vector<td_wstream>& ws = plan.ws;
  const uint64_t stream_code_chunks = plan.stream_code_chunks, stream_scale_blocks = plan.stream_scale_blocks;
  (void)V;
  td_ctx* ctx = new (std::nothrow) td_ctx();
  if (!ctx) return fail(TD_E_NOMEM, "host allocation failed");
  ctx->cfg = c;
  ctx->executor = executor;
  ctx->ncu = ncu;
  ctx->ring = kp.ring_slots;

  // scratch: one allocation, 256-byte aligned pieces
  const int sync_words = TD_SY_WORDS;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  const size_t o_xmid = take((size_t)H * 8), o_xout = take((size_t)H * 8);
  const size_t o_q = take((size_t)(qd + 2 * kvd) * 8), o_o = take((size_t)qd * 8);
  const size_t o_act = take((size_t)std::max(I, topk * I) * 8);
  const size_t o_rl = take((size_t)(E + 2) * 8);  // pairs [0, E), padded to an even count
  const size_t o_eid = take((size_t)std::max(L * topk, 1) * 4), o_ew = take((size_t)std::max(L * topk, 1) * 4);
  const size_t o_part = take((size_t)nkv * n_chunks_max * group * (d + 4) * 8);
  const size_t o_cand = take((size_t)ncu * 4 * 8);
  const size_t o_sync = take((size_t)sync_words * 4);
  const size_t o_tok = take(4), o_err = take(4);
  const size_t o_rope = take((size_t)c.max_ctx * (d / 2) * 2 * 4);
  const size_t o_layers = take(sizeof(td_layer_dev) * L);
  const size_t o_ws = take(sizeof(td_wstream) * ws.size());
  const size_t o_ptab = take(sizeof(int32_t) * part.size());
  const size_t o_gains = take((size_t)(2 * L + 1) * H * 2);
  const size_t o_bias = c.qkv_bias ? take((size_t)L * qkv_rows * 2) : 0;
  const size_t o_bad = take(4);
  ctx->scratch_bytes = off;
  e = hipMalloc(&ctx->scratch, off);
  if (e != hipSuccess) {
    delete ctx;
    return e == hipErrorOutOfMemory ? fail(TD_E_NOMEM, "hipMalloc of scratch failed") : hip_fail(e, "hipMalloc");
  }
  uint8_t* base = (uint8_t*)ctx->scratch;
  e = hipMemset(base, 0, off);
  if (e != hipSuccess) {
    (void)hipFree(ctx->scratch);
    delete ctx;
    return hip_fail(e, "hipMemset");
  }

  // RoPE table: one row per position
  std::vector<float> rope((size_t)c.max_ctx * (d / 2) * 2);
  for (int p = 0; p < c.max_ctx; ++p) rope_row(c.rope_theta, d, p, rope.data() + (size_t)p * d);
  std::vector<td_layer_dev> layers(L);
  for (int l = 0; l < L; ++l) {
    const td_layer_weights& Lw = w->layers[l];
    td_layer_dev& Ld = layers[l];
    Ld.w[0] = (const uint8_t*)Lw.w_qkv;
    Ld.w[1] = (const uint8_t*)Lw.w_o;
    Ld.w[2] = (const uint8_t*)Lw.w_gu;
    Ld.w[3] = (const uint8_t*)Lw.w_d;
    Ld.s[0] = (const uint16_t*)Lw.s_qkv;
    Ld.s[1] = (const uint16_t*)Lw.s_o;
    Ld.s[2] = (const uint16_t*)Lw.s_gu;
    Ld.s[3] = (const uint16_t*)Lw.s_d;
    Ld.bias = c.qkv_bias ? (const uint16_t*)Lw.b_qkv : nullptr;
    Ld.attn_norm = (const uint16_t*)Lw.attn_norm;
    Ld.mlp_norm = (const uint16_t*)Lw.mlp_norm;
    Ld.router = c.n_experts > 0 ? (const uint16_t*)Lw.w_router : nullptr;
  }
  e = hipMemcpy(base + o_rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_layers, layers.data(), sizeof(td_layer_dev) * L, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_ws, ws.data(), sizeof(td_wstream) * ws.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_ptab, part.data(), sizeof(int32_t) * part.size(), hipMemcpyHostToDevice);
  // the RMSNorm gains and QKV biases, contiguous per layer: the kernel finds
  // them by arithmetic instead of through the per-layer pointer table
  for (int l = 0; l < L && e == hipSuccess; ++l) {
    const td_layer_weights& Lw = w->layers[l];
    e = hipMemcpy(base + o_gains + (size_t)(2 * l) * H * 2, Lw.attn_norm, (size_t)H * 2, hipMemcpyDeviceToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(base + o_gains + (size_t)(2 * l + 1) * H * 2, Lw.mlp_norm, (size_t)H * 2, hipMemcpyDeviceToDevice);
    if (e == hipSuccess && c.qkv_bias)
      e = hipMemcpy(base + o_bias + (size_t)l * qkv_rows * 2, Lw.b_qkv, (size_t)qkv_rows * 2, hipMemcpyDeviceToDevice);
  }
  if (e == hipSuccess)
    e = hipMemcpy(base + o_gains + (size_t)(2 * L) * H * 2, w->final_norm, (size_t)H * 2, hipMemcpyDeviceToDevice);
  if (e == hipSuccess) {
    // The launch epoch starts at a value of this context's own.  A hand-off
    // pair's tag is (epoch + step) n_stages + stage + 1, and this context's
    // scratch may sit where another context's kernels published and polled: a
    // copy of such a line left in some XCD's L2 must not carry a tag this
    // context expects, which a common starting epoch of 0 would allow.
    static std::atomic<uint32_t> n_created{0};
    uint64_t z = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                 ((uint64_t)n_created.fetch_add(1) << 32) ^ (uint64_t)(uintptr_t)ctx;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;  // SplitMix64's output mix
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    const uint32_t epoch0 = (uint32_t)(z ^ (z >> 31));
    e = hipMemcpy(base + o_sync + (size_t)TD_SY_EPOCH * 4, &epoch0, 4, hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    (void)hipFree(ctx->scratch);
    delete ctx;
    return hip_fail(e, "hipMemcpy");
  }

  kp.L = L;
  kp.H = H;
  kp.nq = nq;
  kp.nkv = nkv;
  kp.d = d;
  kp.I = I;
  kp.V = V;
  kp.max_ctx = c.max_ctx;
  kp.wf = c.weight_format;
  kp.has_bias = c.qkv_bias ? 1 : 0;
  kp.qd = qd;
  kp.kvd = kvd;
  kp.qkv_rows = qkv_rows;
  kp.group = group;
  kp.eps = c.rms_eps;
  kp.attn_scale = (float)(1.0 / std::sqrt((double)d));
  kp.chunk_len = chunk_len;
  kp.n_chunks_max = n_chunks_max;
  kp.layers = (const td_layer_dev*)(base + o_layers);
  kp.embed = (const uint16_t*)w->embed;
  kp.head = (const uint16_t*)w->head;
  kp.final_norm = (const uint16_t*)w->final_norm;
  kp.rope_cs = (const float*)(base + o_rope);
  kp.tx_mid = (uint2*)(base + o_xmid);
  kp.tx_out = (uint2*)(base + o_xout);
  kp.tq = (uint2*)(base + o_q);
  kp.to = (uint2*)(base + o_o);
  kp.tact = (uint2*)(base + o_act);
  kp.trl = (uint2*)(base + o_rl);
  kp.expert_ids = E ? (int32_t*)(base + o_eid) : nullptr;
  kp.expert_w = E ? (float*)(base + o_ew) : nullptr;
  kp.tpart = (uint2*)(base + o_part);
  kp.cand = (uint2*)(base + o_cand);
  kp.sync = (uint32_t*)(base + o_sync);
  kp.token_out = (int32_t*)(base + o_tok);
  kp.err = (int32_t*)(base + o_err);
  kp.E = E;
  kp.topk = topk;
  kp.spl = E ? 6 : 5;
  kp.n_stages = kp.spl * L + 1;
  kp.ws = (const td_wstream*)(base + o_ws);
  kp.part = (const int32_t*)(base + o_ptab);
  kp.gains = (const uint16_t*)(base + o_gains);
  kp.biases = c.qkv_bias ? (const uint16_t*)(base + o_bias) : nullptr;

  // block forward workspace: TD_MAX_BLOCK rows of every activation it keeps
  {
    const size_t R = TD_MAX_BLOCK, ymax = (size_t)std::max(qkv_rows, 2 * I);
    // split-K slices: the O and down projections always write slices (one when unsplit), the
    // others only when split
    size_t part_floats = 0;
    const int wf = c.weight_format;  // {rows, K, always sliced, format}: the logits GEMM is bf16
    const int gem[5][4] = {{qkv_rows, H, 0, wf}, {H, qd, 1, wf}, {2 * I, H, 0, wf}, {H, I, 1, wf}, {V, H, 0, TD_WF_BF16}};
    for (const auto& g : gem)
      for (int tile_rows : {64, 128}) {  // the GEMM's tile height depends on the block's rows
        int KS = 0;
        const int S = td_block_split(g[0], g[1], ncu, tile_rows, g[3], &KS);
        if (S > 1 || g[2]) part_floats = std::max(part_floats, (size_t)S * R * g[0]);
      }
    // the block attention's key splits use the same buffer (between the QKV
    // epilogue and the O GEMM, when it holds nothing)
    part_floats = std::max(part_floats, td_block_attn_part_floats(nkv, group, d, c.max_ctx, ncu));
    for (int gi = 0; gi < 4; ++gi) {  // the streamed GEMM's slices (bf16, all but the logits GEMM)
      const auto& g = gem[gi];
      if (g[3] != TD_WF_BF16) continue;
      int nt = 0, xc = 0;
      const int S = td_block_stream_plan(g[0], g[1], ncu, &nt, &xc);
      if (S > 1 || g[2]) part_floats = std::max(part_floats, (size_t)S * R * g[0]);
    }
    size_t bo = 0;
    auto btake = [&](size_t bytes) {
      size_t o = bo;
      bo += (size_t)round_up((int64_t)bytes, 256);
      return o;
    };
    const size_t b_x = btake(R * H * 4), b_xg = btake(R * H * 4), b_act = btake(R * I * 4);
    const size_t b_part = btake(part_floats * 4), b_ssq = btake(R * (H / 256) * 4);
    const size_t b_cand = btake(R * TD_BLOCK_ARGMAX_SLICES * 8);
    const size_t b_y = btake(R * ymax * 4), b_q = btake(R * qd * 4), b_ao = btake(R * qd * 4);
    e = hipMalloc(&ctx->blockbuf, bo);
    if (e != hipSuccess) {
      (void)hipFree(ctx->scratch);
      delete ctx;
      return e == hipErrorOutOfMemory ? fail(TD_E_NOMEM, "hipMalloc of the block workspace failed")
                                      : hip_fail(e, "hipMalloc");
    }
    const int pe = td_block_prepare();
    if (pe) {
      (void)hipFree(ctx->blockbuf);
      ctx->blockbuf = nullptr;
      (void)hipFree(ctx->scratch);
      delete ctx;
      return hip_fail((hipError_t)pe, "hipFuncSetAttribute (block GEMM)");
    }
    uint8_t* bb = (uint8_t*)ctx->blockbuf;
    ctx->blk.ncu = ncu;
    ctx->blk.x = (float*)(bb + b_x);
    ctx->blk.xg = (float*)(bb + b_xg);
    ctx->blk.act = (float*)(bb + b_act);
    ctx->blk.ssq = (float*)(bb + b_ssq);
    ctx->blk.cand = (uint2*)(bb + b_cand);
    ctx->blk.part = (float*)(bb + b_part);
    ctx->blk.y = (float*)(bb + b_y);
    ctx->blk.q = (float*)(bb + b_q);
    ctx->blk.ao = (float*)(bb + b_ao);
    ctx->layers_host = layers;
  }

  if (executor != TD_EXEC_MEGAKERNEL) {
    int rc2 = setup_per_op(ctx, kp);
    if (rc2) {
      td_destroy(ctx);
      return rc2;
    }
    ctx->kp = kp;
    *out = ctx;
    return TD_OK;
  }

  // pack the weights into the per-wave streams
  const size_t code_bytes = (size_t)stream_code_chunks * TD_CHUNK;
  ctx->wstream_bytes = code_bytes + (size_t)stream_scale_blocks * TD_SCHUNK + TD_CHUNK;
  e = hipMalloc(&ctx->wstream, ctx->wstream_bytes);
  if (e != hipSuccess) {
    ctx->wstream = nullptr;
    td_destroy(ctx);
    return e == hipErrorOutOfMemory ? fail(TD_E_NOMEM, "hipMalloc of the weight streams failed")
                                    : hip_fail(e, "hipMalloc");
  }
  kp.wcode = (const uint8_t*)ctx->wstream;
  kp.wscale = (const uint8_t*)ctx->wstream + code_bytes;
  int le = td_launch_repack(&kp, ncu, (uint8_t*)ctx->wstream, (uint8_t*)ctx->wstream + code_bytes, kp.ws,
                            (int*)(base + o_bad), nullptr);
  int bad = 0;
  if (le == 0) e = hipDeviceSynchronize();
  if (le == 0 && e == hipSuccess) e = hipMemcpy(&bad, base + o_bad, 4, hipMemcpyDeviceToHost);
  if (le != 0 || e != hipSuccess || bad) {
    td_destroy(ctx);
    if (le) return hip_fail((hipError_t)le, "repack launch");
    if (e != hipSuccess) return hip_fail(e, "repack");
    return fail(TD_E_PLAN, "packed weight stream disagrees with the plan");
  }
  ctx->kp = kp;
  *out = ctx;
  return TD_OK;
}

const int32_t* td_token_ptr(const td_ctx* ctx) { return ctx ? ctx->kp.token_out : nullptr; }

const int32_t* td_expert_ids(const td_ctx* ctx) {
  if (!ctx) return nullptr;
  return ctx->executor == TD_EXEC_MEGAKERNEL ? ctx->kp.expert_ids : ctx->op.expert_ids;
}

const float* td_expert_weights(const td_ctx* ctx) {
  if (!ctx) return nullptr;
  return ctx->executor == TD_EXEC_MEGAKERNEL ? ctx->kp.expert_w : ctx->op.expert_w;
}

int td_decode_step(td_ctx* ctx, const int32_t* d_token, int32_t pos, const td_kv* kv, float* d_logits_out,
                   void* stream) {
  if (!ctx || !d_token || !kv || !kv->k || !kv->v || !d_logits_out) return fail(TD_E_INVALID_ARG, "null argument");
  if (kv->max_ctx != ctx->cfg.max_ctx) return fail(TD_E_INVALID_ARG, "kv max_ctx differs from the config");
  if (((uintptr_t)kv->k | (uintptr_t)kv->v) & 15) return fail(TD_E_INVALID_ARG, "K/V cache pointer not 16-byte aligned");
  if (pos < 0 || pos >= ctx->cfg.max_ctx) return fail(TD_E_RANGE, "pos outside [0, max_ctx)");
  td_kparams p = ctx->kp;
  p.pos = pos;
  p.n_steps = 1;
  p.eos = -1;
  p.tokens_out = nullptr;
  p.count_out = nullptr;
  p.token_in = d_token;
  p.logits = d_logits_out;
  p.kc = (uint16_t*)kv->k;
  p.vc = (uint16_t*)kv->v;
  hipStream_t s = (hipStream_t)stream;
  if (ctx->executor != TD_EXEC_MEGAKERNEL) {
    ctx->op.kc = p.kc;
    ctx->op.vc = p.vc;
    ctx->op.logits = d_logits_out;
    if (ctx->executor == TD_EXEC_GRAPH &&
        (!ctx->gexec || ctx->g_kc != p.kc || ctx->g_vc != p.vc || ctx->g_logits != d_logits_out)) {
      int rc = capture_graph(ctx);
      if (rc) return rc;
    }
  }
  if (ctx->timing) (void)hipEventRecord(ctx->ev0, s);
  int le = 0;
  if (ctx->executor == TD_EXEC_MEGAKERNEL) {
    le = td_launch_megakernel(&p, ctx->ncu, stream);
  } else {
    le = td_launch_op_begin(&ctx->op, d_token, pos, stream);
    if (le == 0) {
      if (ctx->executor == TD_EXEC_PER_OP) le = td_launch_op_layers(&ctx->op, stream);
      else le = (int)hipGraphLaunch(ctx->gexec, s);
    }
  }
  if (le != 0) return hip_fail((hipError_t)le, "step launch");
  if (ctx->timing) {
    (void)hipEventRecord(ctx->ev1, s);
    ctx->timed = true;
  }
  ctx->last_stream = s;
  ctx->launched = true;
  return TD_OK;
}

int td_decode_loop(td_ctx* ctx, const int32_t* d_token, int32_t pos, int32_t n_steps, int32_t eos_id,
                   const td_kv* kv, float* d_logits_out, int32_t* d_tokens_out, int32_t* d_count_out, void* stream) {
  if (!ctx || !d_token || !kv || !kv->k || !kv->v || !d_logits_out) return fail(TD_E_INVALID_ARG, "null argument");
  if (ctx->executor != TD_EXEC_MEGAKERNEL) return fail(TD_E_UNSUPPORTED, "the step loop needs the megakernel executor");
  if (kv->max_ctx != ctx->cfg.max_ctx) return fail(TD_E_INVALID_ARG, "kv max_ctx differs from the config");
  if (((uintptr_t)kv->k | (uintptr_t)kv->v) & 15) return fail(TD_E_INVALID_ARG, "K/V cache pointer not 16-byte aligned");
  if (n_steps < 1 || n_steps > TD_MAX_LOOP_STEPS) return fail(TD_E_INVALID_ARG, "n_steps outside [1, TD_MAX_LOOP_STEPS]");
  if (eos_id < -1 || eos_id >= ctx->cfg.vocab) return fail(TD_E_INVALID_ARG, "eos_id outside [-1, vocab)");
  if (pos < 0 || (int64_t)pos + n_steps > ctx->cfg.max_ctx) return fail(TD_E_RANGE, "positions outside [0, max_ctx)");
  td_kparams p = ctx->kp;
  p.pos = pos;
  p.n_steps = n_steps;
  p.eos = eos_id;
  p.tokens_out = d_tokens_out;
  p.count_out = d_count_out;
  p.token_in = d_token;
  p.logits = d_logits_out;
  p.kc = (uint16_t*)kv->k;
  p.vc = (uint16_t*)kv->v;
  hipStream_t s = (hipStream_t)stream;
  if (ctx->timing) (void)hipEventRecord(ctx->ev0, s);
  const int le = td_launch_megakernel(&p, ctx->ncu, stream);
  if (le != 0) return hip_fail((hipError_t)le, "loop launch");
  if (ctx->timing) {
    (void)hipEventRecord(ctx->ev1, s);
    ctx->timed = true;
  }
  ctx->last_stream = s;
  ctx->launched = true;
  return TD_OK;
}

int td_forward_block(td_ctx* ctx, const int32_t* d_tokens, int32_t n, int32_t pos0, const td_kv* kv,
                     float* d_logits_out, int32_t all_logits, int32_t* d_argmax_out, void* stream) {
  if (!ctx || !d_tokens || !kv || !kv->k || !kv->v || !d_logits_out) return fail(TD_E_INVALID_ARG, "null argument");
  if (kv->max_ctx != ctx->cfg.max_ctx) return fail(TD_E_INVALID_ARG, "kv max_ctx differs from the config");
  if (((uintptr_t)kv->k | (uintptr_t)kv->v) & 15) return fail(TD_E_INVALID_ARG, "K/V cache pointer not 16-byte aligned");
  if (n < 1 || n > TD_MAX_BLOCK) return fail(TD_E_INVALID_ARG, "n outside [1, TD_MAX_BLOCK]");
  if (ctx->cfg.n_experts > 0) return fail(TD_E_UNSUPPORTED, "the block forward runs dense MLPs only");
  if (pos0 < 0 || (int64_t)pos0 + n > ctx->cfg.max_ctx) return fail(TD_E_RANGE, "positions outside [0, max_ctx)");
  td_kparams p = ctx->kp;
  p.kc = (uint16_t*)kv->k;
  p.vc = (uint16_t*)kv->v;
  td_blockparams B = ctx->blk;
  B.kp = &p;
  B.layers_host = ctx->layers_host.data();
  hipStream_t s = (hipStream_t)stream;
  if (ctx->timing) (void)hipEventRecord(ctx->ev0, s);
  const int le = td_launch_block(&B, d_tokens, n, pos0, all_logits ? 1 : 0, d_logits_out, d_argmax_out, stream);
  if (le != 0) return hip_fail((hipError_t)le, "block launch");
  if (ctx->timing) {
    (void)hipEventRecord(ctx->ev1, s);
    ctx->timed = true;
  }
  ctx->last_stream = s;
  ctx->launched = true;
  return TD_OK;
}

int td_decode_step_noalloc(const td_config* cfg, const td_weights* w, const int32_t* d_token, int32_t pos,
                           const td_kv* kv, float* d_logits_out, int32_t* d_token_out, int32_t* d_error_out,
                           void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  rc = check_weights(cfg, w);
  if (rc) return rc;
  if (!d_token || !kv || !kv->k || !kv->v || !d_logits_out || !d_token_out || !d_error_out)
    return fail(TD_E_INVALID_ARG, "null argument");
  if (kv->max_ctx != cfg->max_ctx) return fail(TD_E_INVALID_ARG, "kv max_ctx differs from the config");
  if (((uintptr_t)kv->k | (uintptr_t)kv->v) & 15) return fail(TD_E_INVALID_ARG, "K/V cache pointer not 16-byte aligned");
  if (pos < 0 || pos >= cfg->max_ctx) return fail(TD_E_RANGE, "pos outside [0, max_ctx)");
  const td_config& c = *cfg;
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (ncu <= 0 || ncu % 8) return fail(TD_E_UNSUPPORTED, "CU count must be a positive multiple of 8");
  int chunk_len = 0, n_chunks = 0;
  rc = attention_split(c, ncu, &chunk_len, &n_chunks);
  if (rc) return rc;
  void* base = nullptr;
  int se = td_noalloc_scratch(&base);
  if (se) return hip_fail((hipError_t)se, "hipGetSymbolAddress");

  // the per-op executor's parameters over the scratch array (no allocation)
  td_opparams op{};
  const int d = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  op.L = c.n_layers;
  op.H = c.hidden;
  op.nq = nq;
  op.nkv = nkv;
  op.d = d;
  op.I = c.intermediate;
  op.V = c.vocab;
  op.max_ctx = c.max_ctx;
  op.wf = c.weight_format;
  op.has_bias = c.qkv_bias ? 1 : 0;
  op.qd = nq * d;
  op.kvd = nkv * d;
  op.qkv_rows = op.qd + 2 * op.kvd;
  op.group = nq / nkv;
  op.eps = c.rms_eps;
  op.attn_scale = (float)(1.0 / std::sqrt((double)d));
  op.chunk_len = chunk_len;
  op.n_chunks_max = n_chunks;
  op.E = c.n_experts;
  op.topk = op.E > 0 ? c.top_k : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  const size_t o_layers = take(sizeof(td_layer_dev) * op.L), o_rope = take((size_t)d * 4), o_pos = take(4);
  const size_t o_x = take((size_t)op.H * 4), o_q = take((size_t)op.qd * 4);
  const size_t o_part = take((size_t)nkv * n_chunks * op.group * (d + 4) * 4);
  const size_t o_o = take((size_t)op.qd * 4), o_act = take((size_t)op.I * std::max(1, op.topk) * 4);
  const size_t o_cand = take((size_t)td_op_head_blocks(&op) * 16);
  const size_t o_rl = take((size_t)std::max(1, op.E) * 4), o_eid = take((size_t)op.L * std::max(1, op.topk) * 4);
  const size_t o_ew = take((size_t)op.L * std::max(1, op.topk) * 4);
  if (off > TD_NOALLOC_SCRATCH_BYTES)
    return fail(TD_E_UNSUPPORTED, "the config needs " + std::to_string(off) + " bytes of scratch, more than the " +
                                      std::to_string(TD_NOALLOC_SCRATCH_BYTES) + " of the no-allocation step");
  uint8_t* b = (uint8_t*)base;
  td_layer_dev* table = (td_layer_dev*)(b + o_layers);
  op.layers = table;
  op.rope_cs = (const float*)(b + o_rope);
  op.rope_pos0 = pos;
  op.pos_word = (int32_t*)(b + o_pos);
  op.x = (float*)(b + o_x);
  op.q = (float*)(b + o_q);
  op.part = (float*)(b + o_part);
  op.o = (float*)(b + o_o);
  op.act = (float*)(b + o_act);
  op.cand = (uint32_t*)(b + o_cand);
  op.rlogits = (float*)(b + o_rl);
  op.expert_ids = op.E > 0 ? (int32_t*)(b + o_eid) : nullptr;
  op.expert_w = op.E > 0 ? (float*)(b + o_ew) : nullptr;
  op.embed = (const uint16_t*)w->embed;
  op.head = (const uint16_t*)w->head;
  op.final_norm = (const uint16_t*)w->final_norm;
  op.kc = (uint16_t*)kv->k;
  op.vc = (uint16_t*)kv->v;
  op.logits = d_logits_out;
  op.token_out = d_token_out;
  op.err = d_error_out;
  int le = td_op_set_lds_limits(&op);
  if (le) return hip_fail((hipError_t)le, "hipFuncSetAttribute");
  // the layer table, the RoPE row of pos and the cleared error word, written by
  // kernels from their arguments (no copy from host memory)
  for (int l0 = 0; l0 < op.L; l0 += TD_NOALLOC_LAYERS_PER_LAUNCH) {
    td_noalloc_setup a{};
    a.first = l0;
    a.n = std::min(TD_NOALLOC_LAYERS_PER_LAUNCH, op.L - l0);
    for (int i = 0; i < a.n; ++i) {
      const td_layer_weights& Lw = w->layers[l0 + i];
      td_layer_dev& Ld = a.layers[i];
      Ld.w[0] = (const uint8_t*)Lw.w_qkv;
      Ld.w[1] = (const uint8_t*)Lw.w_o;
      Ld.w[2] = (const uint8_t*)Lw.w_gu;
      Ld.w[3] = (const uint8_t*)Lw.w_d;
      Ld.s[0] = (const uint16_t*)Lw.s_qkv;
      Ld.s[1] = (const uint16_t*)Lw.s_o;
      Ld.s[2] = (const uint16_t*)Lw.s_gu;
      Ld.s[3] = (const uint16_t*)Lw.s_d;
      Ld.bias = c.qkv_bias ? (const uint16_t*)Lw.b_qkv : nullptr;
      Ld.attn_norm = (const uint16_t*)Lw.attn_norm;
      Ld.mlp_norm = (const uint16_t*)Lw.mlp_norm;
      Ld.router = c.n_experts > 0 ? (const uint16_t*)Lw.w_router : nullptr;
    }
    a.d = d;
    a.write_rope = l0 == 0 ? 1 : 0;
    if (a.write_rope) rope_row(c.rope_theta, d, pos, a.rope.cs);
    le = td_launch_noalloc_setup(a, table, (float*)(b + o_rope), d_error_out, stream);
    if (le) return hip_fail((hipError_t)le, "setup launch");
  }
  le = td_launch_op_begin(&op, d_token, pos, stream);
  if (le == 0) le = td_launch_op_layers(&op, stream);
  if (le) return hip_fail((hipError_t)le, "step launch");
  return TD_OK;
}

int td_status(td_ctx* ctx, int32_t* device_error) {
  if (!ctx) return fail(TD_E_INVALID_ARG, "null ctx");
  hipError_t e = hipStreamSynchronize(ctx->last_stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int32_t bits = 0;
  e = hipMemcpy(&bits, ctx->kp.err, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  if (bits) {
    int32_t zero = 0;
    e = hipMemcpy(ctx->kp.err, &zero, 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  }
  int code = TD_OK;
  if (bits & TD_ERRBIT_NONFINITE) code = TD_E_NONFINITE;
  if (bits & TD_ERRBIT_RANGE) code = TD_E_RANGE;
  if (bits & TD_ERRBIT_TIMEOUT) code = TD_E_TIMEOUT;
  if (device_error) *device_error = code;
  return code;
}

void td_destroy(td_ctx* ctx) {
  if (!ctx) return;
  if (ctx->launched) (void)hipStreamSynchronize(ctx->last_stream);
  if (ctx->ev0) (void)hipEventDestroy(ctx->ev0);
  if (ctx->ev1) (void)hipEventDestroy(ctx->ev1);
  drop_graph(ctx);
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  if (ctx->scratch) (void)hipFree(ctx->scratch);
  if (ctx->wstream) (void)hipFree(ctx->wstream);
  if (ctx->opbuf) (void)hipFree(ctx->opbuf);
  if (ctx->blockbuf) (void)hipFree(ctx->blockbuf);
  delete ctx;
}

int td_set_step_clock(td_ctx* ctx, uint64_t* d_buf, int32_t n) {
  if (!ctx) return fail(TD_E_INVALID_ARG, "null ctx");
  if (d_buf && n < 2) return fail(TD_E_INVALID_ARG, "the step clock needs at least 2 entries");
  ctx->kp.step_clock = d_buf;
  ctx->kp.step_clock_n = d_buf ? n : 0;
  return TD_OK;
}

int td_measure_stream(const void* d_buf, int64_t bytes, int32_t reps, float* ms_out, void* stream) {
  if (!d_buf || bytes < 16 || (bytes & 15) || ((uintptr_t)d_buf & 15) || reps < 1 || !ms_out)
    return fail(TD_E_INVALID_ARG, "bad stream-read arguments");
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  int le = td_launch_stream_read(d_buf, bytes, ncu, stream);  // warm-up pass
  if (le == 0) e = hipEventRecord(e0, s);
  for (int r = 0; r < reps && le == 0 && e == hipSuccess; ++r) le = td_launch_stream_read(d_buf, bytes, ncu, stream);
  if (le == 0 && e == hipSuccess) e = hipEventRecord(e1, s);
  if (le == 0 && e == hipSuccess) e = hipEventSynchronize(e1);
  if (le == 0 && e == hipSuccess) e = hipEventElapsedTime(ms_out, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (le) return hip_fail((hipError_t)le, "stream-read launch");
  if (e != hipSuccess) return hip_fail(e, "stream-read timing");
  return TD_OK;
}

int td_set_timing(td_ctx* ctx, int32_t enable) {
  if (!ctx) return fail(TD_E_INVALID_ARG, "null ctx");
  if (enable && !ctx->ev0) {
    hipError_t e = hipEventCreate(&ctx->ev0);
    if (e == hipSuccess) e = hipEventCreate(&ctx->ev1);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  ctx->timing = enable != 0;
  ctx->timed = false;
  return TD_OK;
}

float td_last_step_ms(td_ctx* ctx) {
  if (!ctx || !ctx->timed) return -1.f;
  if (hipEventSynchronize(ctx->ev1) != hipSuccess) return -1.f;
  float ms = -1.f;
  if (hipEventElapsedTime(&ms, ctx->ev0, ctx->ev1) != hipSuccess) return -1.f;
  return ms;
}

int64_t td_trace_bytes(const td_ctx* ctx) {
  if (!ctx) return -1;
  return (int64_t)ctx->ncu * ctx->kp.n_stages * TD_TRACE_STAMPS * 8;
}

int td_set_trace(td_ctx* ctx, void* d_buf, int64_t bytes) {
  if (!ctx) return fail(TD_E_INVALID_ARG, "null ctx");
  if (d_buf && bytes < td_trace_bytes(ctx)) return fail(TD_E_INVALID_ARG, "trace buffer too small");
  ctx->kp.trace = (uint64_t*)d_buf;
  return TD_OK;
}

int td_plan_partition(const td_config* cfg, int32_t ncu, int32_t* part_out, int32_t part_len) {
  if (!cfg || !part_out) return fail(TD_E_INVALID_ARG, "null argument");
  int rc = check_config(cfg);
  if (rc) return rc;
  if (ncu <= 0 || ncu % 8) return fail(TD_E_UNSUPPORTED, "CU count must be a positive multiple of 8");
  if (part_len != TD_NSPACES * (ncu + 1)) return fail(TD_E_INVALID_ARG, "part_len must be 6 (ncu + 1)");
  const std::vector<int32_t> part = build_partition(*cfg, ncu, std::vector<double>(ncu, 1.0));
  std::copy(part.begin(), part.end(), part_out);
  return TD_OK;
}

int td_plan_check(const td_config* cfg, int32_t ncu, const int32_t* part, int32_t part_len) {
  if (!cfg) return fail(TD_E_INVALID_ARG, "null config");
  if (part && part_len != TD_NSPACES * (ncu + 1)) return fail(TD_E_INVALID_ARG, "part_len must be 6 (ncu + 1)");
  Plan plan;
  return build_plan(cfg, ncu, 160 * 1024, part, true, plan);
}

int td_test_rope(const float* d_x, int32_t n_heads, int32_t head_dim, int32_t pos, float rope_theta, float* d_out,
                 void* stream) {
  if (!d_x || !d_out || n_heads <= 0 || (head_dim != 64 && head_dim != 128) || pos < 0 || !(rope_theta > 0.f))
    return fail(TD_E_INVALID_ARG, "bad rope arguments");
  td_rope_row row{};
  rope_row(rope_theta, head_dim, pos, row.cs);
  int le = td_launch_test_rope(d_x, n_heads, head_dim, row, d_out, stream);
  if (le) return hip_fail((hipError_t)le, "rope launch");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  return e == hipSuccess ? TD_OK : hip_fail(e, "hipStreamSynchronize");
}

int td_test_argmax(const float* d_logits, int32_t n, int32_t groups, void* d_work, int32_t* d_token,
                   int32_t* d_nonfinite, void* stream) {
  if (!d_logits || !d_work || !d_token || !d_nonfinite || n <= 0 || groups <= 0 || groups > n)
    return fail(TD_E_INVALID_ARG, "bad argmax arguments");
  int le = td_launch_test_argmax(d_logits, n, groups, d_work, d_token, d_nonfinite, stream);
  if (le) return hip_fail((hipError_t)le, "argmax launch");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  return e == hipSuccess ? TD_OK : hip_fail(e, "hipStreamSynchronize");
}

int td_test_gemv(int32_t fmt, const void* w, const void* scales, int32_t rows, int32_t cols, const float* d_x,
                 float* d_y, void* stream) {
  if (!w || !d_x || !d_y || rows <= 0 || cols <= 0 || cols > 32768) return fail(TD_E_INVALID_ARG, "bad gemv arguments");
  if (fmt == TD_WF_BF16) {
    if (cols % 8) return fail(TD_E_INVALID_ARG, "bf16 cols must be a multiple of 8");
  } else if (fmt == TD_WF_INT4_G64) {
    if (cols % 64 || !scales) return fail(TD_E_INVALID_ARG, "int4 cols must be a multiple of 64, with scales");
  } else {
    return fail(TD_E_INVALID_ARG, "unknown format");
  }
  int le = td_launch_test_gemv(fmt, w, scales, rows, cols, d_x, d_y, stream);
  if (le) return hip_fail((hipError_t)le, "gemv launch");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  return e == hipSuccess ? TD_OK : hip_fail(e, "hipStreamSynchronize");
}

int td_test_attention(const float* d_q, const void* k, const void* v, int32_t n_pos, int32_t head_dim,
                      int32_t chunk_len, int32_t waves_per_head, float* d_out, void* stream) {
  if (!d_q || !k || !v || !d_out || n_pos <= 0 || (head_dim != 64 && head_dim != 128))
    return fail(TD_E_INVALID_ARG, "bad attention arguments");
  if (waves_per_head != 1 && waves_per_head != 2 && waves_per_head != 4 && !(waves_per_head == 8 && head_dim == 128))
    return fail(TD_E_INVALID_ARG, "waves_per_head must be 1, 2 or 4 (or 8 at head_dim 128)");
  if (chunk_len == 0) chunk_len = (int32_t)round_up(n_pos, TD_TILE);
  if (chunk_len < 0 || chunk_len % TD_TILE) return fail(TD_E_INVALID_ARG, "chunk_len must be a multiple of 64");
  if ((n_pos + chunk_len - 1) / chunk_len > 64) return fail(TD_E_INVALID_ARG, "more than 64 chunks");
  const float scale = (float)(1.0 / std::sqrt((double)head_dim));  // the decode kernel's attention scale
  int le = td_launch_test_attention(d_q, k, v, n_pos, head_dim, chunk_len, waves_per_head, scale, d_out, stream);
  if (le) return hip_fail((hipError_t)le, "attention launch");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  return e == hipSuccess ? TD_OK : hip_fail(e, "hipStreamSynchronize");
}


}  // extern "C"
