// td_internal.h - device-side parameter block and layout constants shared by
// the host API (td_api.cpp) and the kernels (td_kernels.hip, td_ops.hip).
#pragma once
#include <stddef.h>
#include <stdint.h>

#define TD_NW 8                       // compute waves per workgroup (waves 0..7)
#define TD_SYNC_WAVE 8                // attention tiles and the greedy-token reduction
#define TD_WAVE 64
#define TD_THREADS (9 * TD_WAVE)
#define TD_TILE 64                    // attention positions per LDS tile
#define TD_CHUNK 1024                 // bytes per wave-wide weight chunk (64 lanes x 16 B)
#define TD_SCHUNK 64                  // bytes of fp16 scales per int4 chunk (32 scales)
#define TD_MAX_GROUP 8                // query heads per kv head handled by one task
#define TD_SPIN_TICKS 100000000ull    // wait limit in 100 MHz ticks (1 s)
#define TD_RING_MIN 4                 // fewest ring slots per compute wave the plan accepts
#define TD_RING_MIN2 9                // fewest ring slots with which a second attention tile buffer is taken
#define TD_RING_MIN3 7                // fewest ring slots with which a third attention tile buffer is taken
#ifndef TD_RING_MAX
#define TD_RING_MAX 24
#endif

// stage kinds.  A dense layer runs QKV, ATTN, O, GU, DOWN; a mixture-of-experts
// layer runs QKV, ATTN, O, ROUTER, GU, DOWN (GU and DOWN then on the experts the
// router chose); the head follows the last layer
enum { TD_ST_QKV = 0, TD_ST_ATTN = 1, TD_ST_O = 2, TD_ST_GU = 3, TD_ST_DOWN = 4, TD_ST_HEAD = 5, TD_ST_ROUTER = 6 };

// unit spaces of the partition table: which units of a GEMV stage each CU owns.
// TD_SP_E: the router's rows (one per expert); TD_SP_EI: the expert gate/up
// units, top_k slots of I, a CU's range inside one slot.  Both are empty for a
// dense config.
enum { TD_SP_QKV = 0, TD_SP_H = 1, TD_SP_I = 2, TD_SP_V = 3, TD_SP_E = 4, TD_SP_EI = 5, TD_NSPACES = 6 };

// error bits of the device error word
enum { TD_ERRBIT_NONFINITE = 1, TD_ERRBIT_RANGE = 2, TD_ERRBIT_TIMEOUT = 4 };

// uint32 word offsets inside the sync area (each on its own 256-byte line)
enum {
  TD_SY_EPOCH = 0,    // steps completed (the tag base of the next launch's first step)
  TD_SY_ABORT = 64,   // set when a wait timed out
  TD_SY_WORDS = 128
};

// uint32 word offsets of the LDS control block (intra-workgroup hand-offs)
enum {
  TD_CTL_SUB = 0,        // [8] per query head: partial attention states its other waves have left (monotonic)
  TD_CTL_RV = 16,        // rendezvous arrivals of the compute waves (monotonic)
  TD_CTL_TREADY = 17,    // attention tiles made ready (monotonic)
  TD_CTL_TDONE = 18,     // attention tiles consumed, summed over the query-head waves
  TD_CTL_HEADDONE = 19,  // compute waves finished with the head stage (monotonic over the steps)
  TD_CTL_TOKEN = 20,     // the greedy token of the last step finished
  TD_CTL_TOKREADY = 21,  // steps whose token has been decided (monotonic)
  TD_CTL_STOP = 22,      // nonzero: the step just decided is the launch's last
  TD_CTL_SSQ = 24,       // [8] fp32 partial sums of squares of the RMSNorm input slices
  TD_CTL_CAND = 32,      // [8][4] per-wave greedy candidates: value bits, index, nonfinite, pad
  TD_CTL_WORDS = 64
};

// one position's RoPE table row: (cos, sin) of pair i at [2 i], [2 i + 1], i < d/2 <= 64
struct td_rope_row {
  float cs[128];
};

struct td_layer_dev {
  const uint8_t* w[4];     // QKV, O, GU, DOWN
  const uint16_t* s[4];    // fp16 scales (int4) or null
  const uint16_t* bias;    // bf16 QKV bias or null
  const uint16_t* attn_norm;
  const uint16_t* mlp_norm;
  const uint16_t* router;  // MoE: bf16 [E][H], else null (w[2], w[3] then hold all experts)
};

// One compute wave's weight stream: its chunks for the whole step, in the
// order it consumes them, packed contiguously (code_off in 1 KiB chunks), and
// for the leading n4 int4 chunks their scales (scale_off in 64-byte blocks).
struct td_wstream {
  uint32_t code_off, scale_off, n_tot, n4;
};

struct td_kparams {
  // shape
  int32_t L, H, nq, nkv, d, I, V, max_ctx, wf, has_bias;
  int32_t qd, kvd, qkv_rows, group;
  float eps, attn_scale;
  int32_t E, topk;  // MoE: experts and experts per token (E = 0: dense MLP)
  int32_t spl;      // stages per layer: 5 (dense) or 6 (MoE: with ROUTER)
  // attention split
  int32_t chunk_len, n_chunks_max;
  // steps: n_steps greedy steps at positions pos, pos + 1, ... in one launch,
  // stopping early after a step whose token is eos (eos < 0: none) or whose
  // logits were not all finite
  int32_t pos, n_steps, eos;
  // weights
  const td_layer_dev* layers;
  const uint16_t* embed;
  const uint16_t* head;
  const uint16_t* final_norm;
  const float* rope_cs;        // [max_ctx][d/2][2] (cos, sin)
  uint16_t* kc;                // caller K cache [L][nkv][max_ctx][d]
  uint16_t* vc;
  const int32_t* token_in;
  float* logits;
  int32_t* tokens_out;  // [n_steps] the steps' tokens, -1 past the last step run; or null
  int32_t* count_out;   // steps run; or null
  // scratch (ctx-owned).  Every value handed from one CU to another is
  // published as a (value bits, tag) pair written with one 8-byte agent-scope
  // store; tag = launch epoch * n_stages + stage + 1 names the producing stage,
  // and readers poll until every pair they need carries the tag they expect.
  uint2* tx_mid;   // [H] residual after the attention block
  uint2* tx_out;   // [H] residual after the MLP block
  uint2* tq;       // [nkv][(group + 2) d]: per kv head its rotated queries, then this
                   // position's K row (rotated) and V row (bf16 values)
  uint2* to;       // [nq d] attention output
  uint2* tact;     // [I] SiLU(gate) * up; MoE: [topk][I], slot j from the j-th chosen expert
  uint2* trl;      // MoE: [E] router logits (then -inf at [E] when E is odd: read in pairs)
  int32_t* expert_ids;  // MoE: [L][topk] the chosen experts of the last step (written by CU 0)
  float* expert_w;      // MoE: [L][topk] their router probabilities
  uint2* tpart;    // [nkv][group][n_chunks_max][d + 4] attention partials: acc[d], m, l, pad
  uint2* cand;     // [ncu][4] pairs: a CU's greedy candidate (value bits, index, nonfinite, 0)
  uint32_t* sync;
  int32_t* token_out;
  int32_t* err;
  const int32_t* part;  // [TD_NSPACES][ncu + 1] first unit of each CU in each unit space
  const uint16_t* gains;   // ctx copy of the RMSNorm gains, bf16 [L][2][H] (attention, MLP) then final [H]
  const uint16_t* biases;  // ctx copy of the QKV biases, bf16 [L][qkv_rows], or null
  // LDS layout (byte offsets into dynamic shared memory)
  int32_t off_ring, off_sring, off_xin, off_attn, off_tile, off_own, off_out, off_rope, off_ctl;
  int32_t off_route;  // MoE: router logits [TD_MAX_EXPERTS] floats, then per compute wave its choice
                      // (ids [TD_MAX_TOPK], weights [TD_MAX_TOPK]); 0 for a dense config
  int32_t tile_bufs, tile_stride;  // attention K/V tile buffers (1 or 2) and their spacing in bytes
  int32_t lds_bytes;
  int32_t n_stages;   // spl L + 1
  int32_t ring_slots; // S: LDS ring slots per compute wave
  uint64_t* trace;    // optional: [ncu][n_stages][TD_TRACE_STAMPS] 100 MHz timestamps, or null
  uint64_t* step_clock;  // optional: [step_clock_n] 100 MHz clock: [0] launch start, [s + 1] step s's token decided
  int32_t step_clock_n;
  // packed weight streams (built at create time)
  const uint8_t* wcode;
  const uint8_t* wscale;
  const td_wstream* ws;   // [ncu][TD_NW]
  int32_t merge_in_tile;  // the attention merge staging runs on into the first tile buffer
};

// Parameters of the per-op executor (td_ops.hip): the same weights, table and
// shapes; activations in plain fp32 device buffers ordered by kernel
// boundaries; the step's position in a device word so the launches after
// op_begin can be captured once and replayed.
struct td_opparams {
  int32_t L, H, nq, nkv, d, I, V, max_ctx, wf, has_bias;
  int32_t qd, kvd, qkv_rows, group;
  float eps, attn_scale;
  int32_t chunk_len, n_chunks_max;
  int32_t E, topk;   // MoE: experts and experts per token (E = 0: dense MLP)
  int32_t* pos_word;
  int32_t rope_pos0;  // position of rope_cs's first row (0: the full table; the no-allocation step keeps one row)
  const td_layer_dev* layers;
  const uint16_t* embed;
  const uint16_t* head;
  const uint16_t* final_norm;
  const float* rope_cs;
  uint16_t* kc;
  uint16_t* vc;
  float* logits;
  float* x;          // [H] residual
  float* q;          // [nq d] rotated queries times 1/sqrt(d)
  float* part;       // [nkv][group][n_chunks_max][d + 4] attention partials: acc[d], m, l, pad
  float* o;          // [nq d] attention output
  float* act;        // [I] SiLU(gate) * up; MoE: [topk][I], slot j of the j-th chosen expert
  float* rlogits;    // MoE: [E] router logits of the current layer
  int32_t* expert_ids;  // MoE: [L][topk] chosen experts (the routing tensor the expert ops read)
  float* expert_w;      // MoE: [L][topk] their router probabilities
  uint32_t* cand;    // [head blocks][4]: value bits, index, nonfinite
  int32_t* token_out;
  int32_t* err;
};

// Per (CU, stage) trace record of TD_TRACE_STAMPS uint64 timestamps (100 MHz):
// compute wave w writes [4 w + k]: k = 0 stage entered, 1 inputs staged (the
// workgroup rendezvous passed), 2 first weight chunk in LDS (or first attention
// tile done), 3 last output published; 0 where the wave had no part.
#define TD_TRACE_STAMPS 32

// LDS layout of the attention stage.  The K/V tile area is separate (it is
// filled while the QKV stage still uses the GEMV input area); the rest aliases
// the GEMV input area.  K rows are padded by 8 elements so that lanes reading
// different rows hit different banks.
#ifdef __HIPCC__
__host__ __device__
#endif
static inline int32_t td_tile_bytes(int d) {
  return TD_TILE * (d + 8) * 2 + TD_TILE * d * 2;
}

struct td_attn_lds {
  int32_t q, kvp, p, sub, merge, bytes;
};

// Compute waves per query head in the decode step's attention.  With one
// query head per kv head (group 1, the OLMoE layout) a CU's attention would run
// on one of its eight compute waves, so in a mixture-of-experts model W = 8
// waves share it (4 at head dim 64, where a wave's share of a tile, 64 / W
// rows, stays a multiple of 16): wave w takes query head w % group and rows
// [s 64 / W, (s + 1) 64 / W) of every tile, s = w / group, and the W partial
// states of a head are combined in wave order.  Measured on the OLMoE shape:
// 0.967 -> 0.954 ms per step.  Every other model keeps one wave per head, and
// the dense kernels are compiled without the split: two waves per head measured
// slower on the Llama-3.2-1B shapes (0.664 -> 0.682 ms per step), and the split's
// code alone, unused, cost the dense kernels 2 % in their GEMV loops.
#ifdef __HIPCC__
__host__ __device__
#endif
static inline int td_attn_waves(int d, int group, bool moe) { return moe && group == 1 ? (d == 64 ? 4 : 8) : 1; }

#ifdef __HIPCC__
__host__ __device__
#endif
static inline td_attn_lds td_attn_layout(int d, int group, int n_chunks_max, bool moe = false) {
  td_attn_lds a;
  const int W = td_attn_waves(d, group, moe);
  a.q = 0;                                          // group x d queries, then this
  a.kvp = a.q + group * d * 4;                      // position's K and V rows (2 d floats)
  a.p = a.kvp + 2 * d * 4;                          // group W x 64 probabilities / merge weights (one row a wave)
  a.sub = a.p + group * W * TD_TILE * 4;            // group x (W - 1) x (d + 4) partial states of a head's waves
  a.merge = a.sub + group * (W - 1) * (d + 4) * 4;  // group x (n_chunks_max - 1) x (d + 4) partials
  a.bytes = a.merge + group * (n_chunks_max > 1 ? n_chunks_max - 1 : 1) * (d + 4) * 4;
  a.bytes = (a.bytes + 255) & ~255;
  return a;
}

// How far into the LDS input area a mixture-of-experts down stage reads: slot j's
// activations start at j I, and a down row's whole chunks (512 bf16 weights
// each, zero weights past I) read 512 ceil(I / 512) activations from there, so
// the last slot reads up to (top_k - 1) I + 512 ceil(I / 512); the stage zeroes
// the input area from top_k I up to that point (0 x a stale NaN would be NaN).
#ifdef __HIPCC__
__host__ __device__
#endif
static inline int td_moe_down_reach(int top_k, int I) { return (top_k - 1) * I + (I + 511) / 512 * 512; }

// Input slice of compute wave w (of TD_NW) over a K-element vector, in whole
// (value, tag) pair units of two elements: [lo, hi).
#ifdef __HIPCC__
__host__ __device__
#endif
static inline void td_slice(int K, int w, int* lo, int* hi) {
  const int nu = K / 2;
  *lo = 2 * (int)(((int64_t)nu * w) / TD_NW);
  *hi = 2 * (int)(((int64_t)nu * (w + 1)) / TD_NW);
}

// Workspace and host-side views of the block forward (td_block.hip), for
// up to TD_MAX_BLOCK token rows (TD_MAX_BLOCK, the most rows, is declared in
// td.h).
struct td_blockparams {
  const td_kparams* kp;            // shapes, weights, cache, rope table, token and error words
  const td_layer_dev* layers_host; // [L] the layer pointers, host copy
  int ncu;                         // CUs of the device (split-K sizing)
  float* x;                        // [n][H] residual stream
  float* y;                        // [n][max(qkv_rows, 2 I)] QKV or gate/up output
  float* xg;                       // [n][H] x * gain of the next RMSNorm (a GEMM input)
  float* act;                      // [n][I] SiLU(gate) * up (a GEMM input)
  float* ssq;                      // [n][H / 256] block sums of squares of x (RMSNorm)
  uint2* cand;                     // [n][TD_BLOCK_ARGMAX_SLICES] greedy-token candidates
  float* part;                     // split-K partial slices, td_block_part_floats() floats
  float* q;                        // [n][qd] rotated, scaled queries
  float* ao;                       // [n][qd] attention output
};

#define TD_BLOCK_ARGMAX_SLICES 64  // column slices of a logits row searched in parallel

// Split-K plan of one block GEMM (N weight rows, K columns, tiles of
// tile_rows weight rows, weight format fmt): GEMMs with fewer tiles than two
// per CU cut K into S slices of KS columns (a multiple of 64), as many as keep
// the grid within two workgroups per CU (the most that are resident at once),
// but no more than leave every slice td_block_min_chunks(fmt) 64-column chunks:
// a shorter slice spends its time filling and draining its pipeline (measured:
// the 2048-column O projection took 14 us in 2-chunk slices, 10 us in 4).
// Returns S.
static inline int td_block_min_chunks(int fmt) { return fmt == TD_WF_INT4_G64 ? 6 : 4; }  // int4: 1/4 the bytes
static inline int td_block_split(int N, int K, int ncu, int tile_rows, int fmt, int* KS) {
  const int tiles = (N + tile_rows - 1) / tile_rows, chunks = K / 64;
  int s = tiles >= 2 * ncu ? 1 : (2 * ncu) / tiles;
  if (s > chunks / td_block_min_chunks(fmt)) s = chunks / td_block_min_chunks(fmt);
  if (s < 1) s = 1;
  const int per = (chunks + s - 1) / s;
  *KS = per * 64;
  return (chunks + per - 1) / per;
}

// The streamed block GEMM (bf16 weights, 49 to 64 token rows): workgroups of
// 16 nt weight rows (nt = 16 or 8) over K slices of 64 xc columns (xc = 8, 4
// or 2).  Among the plans whose grid fits one workgroup per CU (or, failing
// that, the fewest rounds), the one whose workgroup moves the fewest bytes: its
// weights, half the bytes of 64 input rows (they come from L2), a fixed fill
// cost and, when split, its partial output.  The plan does not depend on the
// block's row count, so the partial buffer sized for it fits every block.
// Measured on the Llama shapes: gate/up nt 16 xc 8, down nt 8 xc 8, QKV nt 8
// xc 4, O nt 8 xc 2.  Returns S, the number of K slices.
static inline int td_block_stream_plan(int N, int K, int ncu, int* nt, int* xc) {
  constexpr int M = 64;
  const int chunks = K / 64;
  double best = 1e300;
  int bs = 1;
  for (int t : {8, 16})
    for (int c : {8, 4, 2}) {
      const int nr = 16 * t, tiles = (N + nr - 1) / nr, S = (chunks + c - 1) / c;
      const long grid = (long)tiles * S, rounds = (grid + ncu - 1) / ncu;
      const double per_wg = (double)c * (nr * 128.0 + M * 128.0) + 49152.0 + (S > 1 ? 4.0 * M * nr : 0.0);
      const double sc = (double)rounds * per_wg;
      if (sc < best) {
        best = sc;
        *nt = t;
        *xc = c;
        bs = S;
      }
    }
  return bs;
}
static inline bool td_block_stream_ok(int fmt, int M) { return fmt == TD_WF_BF16 && M > 48 && M <= 64; }

// Key splits of the block attention: the workgroups of one split (base of
// them) use fewer than half the CUs and the keys span at least 64 tiles of 32
// (2048 positions), so more workgroups share the K/V reads; at most 4, and
// every split keeps 8 tiles (one per wave) or more.  Short prompts keep one
// launch (a split costs a merge launch).
static inline int td_block_attn_split(int base, int ntiles, int ncu) {
  if (ntiles < 64 || 2 * base > ncu) return 1;
  int s = ncu / base;
  if (s > 4) s = 4;
  if (s > ntiles / 8) s = ntiles / 8;
  return s < 1 ? 1 : s;
}
// scratch floats the block attention's splits need, the most over blocks of
// 1..TD_MAX_BLOCK rows: nsplit x nkv x rows x (D + 2)
static inline size_t td_block_attn_part_floats(int nkv, int group, int d, int max_ctx, int ncu) {
  size_t most = 0;
  for (int n = 1; n <= TD_MAX_BLOCK; ++n) {
    const int rows = n * group, nx = (rows + 15) / 16, s = td_block_attn_split(nx * nkv, max_ctx / 32 + 1, ncu);
    if (s > 1 && (size_t)s * nkv * rows * (d + 2) > most) most = (size_t)s * nkv * rows * (d + 2);
  }
  return most;
}

// launch entry points (td_kernels.hip)
int td_launch_megakernel(const td_kparams* p, int ncu, void* stream);
// block forward (td_block.hip): logits [n][V] (all_logits) or [V] of the last token
int td_launch_block(const td_blockparams* B, const int32_t* tokens, int n, int pos0, int all_logits, float* logits,
                    int32_t* argmax_out, void* stream);
// sets the dynamic LDS limit of the streamed block GEMM's instances (once per process)
int td_block_prepare();
int td_launch_repack(const td_kparams* p, int ncu, uint8_t* code, uint8_t* scale, const td_wstream* ws, int* bad,
                     void* stream);
int td_megakernel_occupancy(int head_dim, int weight_format, int moe, int lds_bytes, int* blocks_per_cu);
// per-op executor (td_ops.hip)
int td_op_head_blocks(const td_opparams* p);
// the no-allocation step (td_ops.hip): the device's copy of the file-scope
// scratch array and its size; the setup launch (layer table, RoPE row, error word)
#define TD_NOALLOC_LAYERS_PER_LAUNCH 16
struct td_noalloc_setup {
  td_layer_dev layers[TD_NOALLOC_LAYERS_PER_LAUNCH];
  td_rope_row rope;
  int32_t first, n, d, write_rope;
};
int td_noalloc_scratch(void** ptr);
int td_launch_noalloc_setup(const td_noalloc_setup& a, td_layer_dev* table, float* rope_row, int32_t* err,
                            void* stream);
size_t td_op_lds_bytes(const td_opparams* p);
int td_op_set_lds_limits(const td_opparams* p);
int td_launch_op_begin(const td_opparams* p, const int32_t* d_token, int32_t pos, void* stream);
int td_launch_op_layers(const td_opparams* p, void* stream);
int td_launch_test_gemv(int fmt, const void* w, const void* s, int rows, int cols, const float* x, float* y,
                        void* stream);
int td_launch_stream_read(const void* buf, int64_t bytes, int ncu, void* stream);
int td_launch_test_rope(const float* x, int n_heads, int d, const td_rope_row& row, float* y, void* stream);
int td_launch_test_argmax(const float* logits, int n, int groups, void* work, int* token, int* nonfinite,
                          void* stream);
size_t td_test_attention_lds(int d, int chunk_len, int n);
int td_launch_test_attention(const float* q, const void* k, const void* v, int n, int d, int chunk_len, int waves,
                             float scale, float* out, void* stream);
