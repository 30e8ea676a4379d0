// td_kernels.hip - the persistent decode-step megakernel for MI355X (gfx950)
// and the single-routine kernels behind the test hooks.
//
// One workgroup per CU runs the whole step as a fixed sequence of stages from
// a static plan ("Decoding in tiles", sec. 4; sec. 3: the next weights are
// fetched while a stage waits for its inputs).  Per layer:
//   QKV   RMSNorm + fused [Wq;Wk;Wv] GEMV (+bias), RoPE, K/V-cache write
//   ATTN  split-K grouped-query attention over the cache ("One launch per
//         token", "The attention trap": heads x chunks, merged with the
//         exp(m_local - m_global) rescale)
//   O     output projection + residual
//   GU    RMSNorm + gate/up GEMV + SiLU(gate) * up
//   DOWN  down projection + residual
// then HEAD: final RMSNorm, logits GEMV, greedy argmax (lowest id on ties,
// non-finite logit -> error word; "Decoding in tiles", sec. 5).
//
// Workgroup roles (9 waves; no s_barrier after the first instruction block:
// waves hand work to each other through counters in LDS):
//   8 compute waves  each streams its own weight chunks (1 KiB = 64 lanes x
//                 16 B) from HBM into its LDS ring with global_load_lds, in
//                 the order it consumes them, with a bounded number in flight
//                 (see "compute waves" below); polls one slice of the stage's
//                 input vector into LDS, meets the others at a rendezvous, then
//                 runs its rows from the ring and publishes its own outputs
//                 (bias, RoPE, K/V write, SiLU*up, residual, logits); in the
//                 attention stage, wave h < group runs query head h of the
//                 task and merges.
//   sync wave     loads the attention K/V tiles and reduces the greedy token.
// Cross-CU hand-off without grid barriers: every value handed to other CUs is
// a (value, tag) pair written with one 8-byte agent-scope (sc1) store, and a
// reader polls the pairs with sc1 loads until all carry the tag of the stage
// that produced them.  The data is its own ready signal, coherent across the 8
// XCDs without writing back or invalidating whole L2 caches, and a stage waits
// only for the values it reads.  Every wait is bounded in time.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "td.h"
#include "td_internal.h"

#include "td_device.h"

namespace {

// ------------------------------------------------------------ the plan
// A GEMV stage splits its "units" over the CUs by the partition table (CU c
// owns units [part[c], part[c+1]) of the stage's unit space) and round-robins
// a CU's units over its compute waves.  A unit is the set of rows one epilogue
// needs together: the two rows of a RoPE pair (i, i + d/2) of one head for QKV,
// the gate and up rows of one intermediate index for GU, one row otherwise.
// In a mixture-of-experts layer the GU units are top_k slots of I (slot j runs
// the j-th chosen expert), a DOWN unit's row is summed over the slots, and the
// packed stream holds every expert's rows of the wave's units (ne = E blocks,
// estride bytes apart in the stacked weights): the wave streams the blocks of
// the experts the router chose ("One launch per token", its 64-expert MoE
// section: the expert weights are gathered by id inside the same launch).
struct Gemv {
  const uint8_t* w;
  const uint16_t* s;
  int K, row_bytes, J, U, rpu, kind, fmt, space, ne;
  size_t estride;
};

template <bool MOE>
DEV void stage_of(const td_kparams& P, int seq, int& kind, int& layer) {
  constexpr int spl = MOE ? 6 : 5;
  if (seq >= spl * P.L) {
    kind = TD_ST_HEAD;
    layer = P.L;
  } else {
    layer = seq / spl;
    const int k = seq - layer * spl;
    kind = !MOE || k < 3 ? k : k == 3 ? TD_ST_ROUTER : k - 1;  // MoE: 3 ROUTER, 4 GU, 5 DOWN
  }
}
DEV void stage_of_any(const td_kparams& P, int seq, int& kind, int& layer) {
  if (P.E) stage_of<true>(P, seq, kind, layer);
  else stage_of<false>(P, seq, kind, layer);
}

DEV Gemv gemv_of(const td_kparams& P, int kind, int layer) {
  Gemv g;
  g.kind = kind;
  g.s = nullptr;
  g.ne = 1;
  g.estride = 0;
  if (kind == TD_ST_HEAD) {
    g.w = (const uint8_t*)P.head;
    g.K = P.H;
    g.U = P.V;
    g.rpu = 1;
    g.fmt = 0;
    g.space = TD_SP_V;
  } else if (kind == TD_ST_ROUTER) {  // bf16 [E][H]
    g.w = (const uint8_t*)P.layers[layer].router;
    g.K = P.H;
    g.U = P.E;
    g.rpu = 1;
    g.fmt = 0;
    g.space = TD_SP_E;
  } else {
    const td_layer_dev& Ld = P.layers[layer];
    int idx = kind == TD_ST_QKV ? 0 : kind == TD_ST_O ? 1 : kind == TD_ST_GU ? 2 : 3;
    g.w = Ld.w[idx];
    g.s = Ld.s[idx];
    g.fmt = P.wf;
    if (kind == TD_ST_QKV) { g.K = P.H; g.U = P.qkv_rows / 2; g.rpu = 2; g.space = TD_SP_QKV; }
    else if (kind == TD_ST_O) { g.K = P.qd; g.U = P.H; g.rpu = 1; g.space = TD_SP_H; }
    else if (kind == TD_ST_GU) { g.K = P.H; g.U = P.E ? P.topk * P.I : P.I; g.rpu = 2; g.space = P.E ? TD_SP_EI : TD_SP_I; }
    else { g.K = P.I; g.U = P.H; g.rpu = 1; g.space = TD_SP_H; }
  }
  g.row_bytes = g.fmt == 0 ? g.K * 2 : g.K / 2;
  g.J = (g.row_bytes + TD_CHUNK - 1) / TD_CHUNK;
  if (P.E && (kind == TD_ST_GU || kind == TD_ST_DOWN)) {  // all experts, stacked [E][rows][K]
    g.ne = P.E;
    g.estride = (size_t)(kind == TD_ST_GU ? 2 * P.I : P.H) * g.row_bytes;
  }
  return g;
}

// The shape of a GEMV stage from the plan's scalars alone (no memory access):
// what a compute wave needs to walk its rows.
struct Shape {
  int J, rpu, fmt, space;
};
template <bool MOE>
DEV Shape shape_of(const td_kparams& P, int kind) {
  Shape h;
  int K;
  if (kind == TD_ST_HEAD) { K = P.H; h.rpu = 1; h.fmt = 0; h.space = TD_SP_V; }
  else if (kind == TD_ST_ROUTER) { K = P.H; h.rpu = 1; h.fmt = 0; h.space = TD_SP_E; }
  else {
    h.fmt = P.wf;
    if (kind == TD_ST_QKV) { K = P.H; h.rpu = 2; h.space = TD_SP_QKV; }
    else if (kind == TD_ST_O) { K = P.qd; h.rpu = 1; h.space = TD_SP_H; }
    else if (kind == TD_ST_GU) { K = P.H; h.rpu = 2; h.space = MOE ? TD_SP_EI : TD_SP_I; }
    else { K = P.I; h.rpu = 1; h.space = TD_SP_H; }
  }
  const int row_bytes = h.fmt == 0 ? K * 2 : K / 2;
  h.J = (row_bytes + TD_CHUNK - 1) / TD_CHUNK;
  return h;
}

DEV int unit_row(const td_kparams& P, int kind, int u, int r) {
  if (kind == TD_ST_QKV) {
    int half = P.d >> 1;
    int head = u / half;
    int i = u - head * half;
    return head * P.d + i + r * half;
  }
  if (kind == TD_ST_GU) return (P.E ? u % P.I : u) + r * P.I;  // MoE: row u % I of slot u / I's expert
  return u;
}

DEV void cu_units(const td_kparams& P, int space, int cu, int ncu, int& u0, int& u1) {
  const int32_t* t = P.part + (size_t)space * (ncu + 1);
  u0 = t[cu];
  u1 = t[cu + 1];
}

DEV int wave_units(int cnt, int wave) { return cnt > wave ? (cnt - wave + TD_NW - 1) / TD_NW : 0; }

// position in one compute wave's chunk sequence over the whole step (weight packing)
struct Cursor {
  int seq;  // stage sequence number; == n_stages when done
  Gemv g;
  int u_first, n, e, k, r, j;
};

DEV void cur_enter(Cursor& c, const td_kparams& P, int wave, int cu, int ncu, int seq) {
  for (; seq < P.n_stages; ++seq) {
    int kind, layer;
    stage_of_any(P, seq, kind, layer);
    if (kind == TD_ST_ATTN) continue;
    Gemv g = gemv_of(P, kind, layer);
    int u0, u1;
    cu_units(P, g.space, cu, ncu, u0, u1);
    const int n = wave_units(u1 - u0, wave);
    if (n == 0) continue;
    c.seq = seq;
    c.g = g;
    c.u_first = u0 + wave;
    c.n = n;
    c.e = c.k = c.r = c.j = 0;
    return;
  }
  c.seq = P.n_stages;
}

DEV void cur_next(Cursor& c, const td_kparams& P, int wave, int cu, int ncu) {
  if (++c.j < c.g.J) return;
  c.j = 0;
  if (++c.r < c.g.rpu) return;
  c.r = 0;
  if (++c.k < c.n) return;
  c.k = 0;
  if (++c.e < c.g.ne) return;
  cur_enter(c, P, wave, cu, ncu, c.seq + 1);
}

// ------------------------------------------------------------ waits
// LDS control words are read and written with inline assembly: the compiler
// would otherwise make every such access wait for all of the wave's
// outstanding LDS DMAs (it cannot tell that the control block and the rings
// do not overlap), which would drain the weight stream at each hand-off.
DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
DEV uint32_t lds_ld(const uint32_t* p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
DEV void lds_st(uint32_t* p, uint32_t v) { asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory"); }
DEV void lds_add(uint32_t* p, uint32_t v) { asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory"); }
DEV void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// A wait that began at t0 (100 MHz clock) gives up once another wait has set
// the abort word or after TD_SPIN_TICKS.  The abort word is read only once the
// wait has lasted TD_ABORT_CHECK_TICKS: a hand-off normally completes in a few
// microseconds, and the read is a load the compiler tracks, whose wait (behind
// every weight chunk in flight) would otherwise stall each poll round that
// checks it.
#define TD_ABORT_CHECK_TICKS 10000ull  // 100 us
DEV bool wait_expired(const td_kparams& P, uint64_t t0) {
  const uint64_t el = wall_clock64() - t0;
  if (el < TD_ABORT_CHECK_TICKS) return false;
  if (ld_u(P.sync + TD_SY_ABORT)) return true;
  if (el > TD_SPIN_TICKS) {
    st_u(P.sync + TD_SY_ABORT, 1u);
    return true;
  }
  return false;
}

// Spins until the LDS word *p reaches at least `target`; returns the value
// seen (or 0 with ok cleared when the wait timed out or another wait did).
// (A compiler barrier follows every return, so that no LDS read of the data
// the word guards is moved above the wait.)
DEV uint32_t lds_wait_ge(const td_kparams& P, const uint32_t* p, uint32_t target, bool& ok) {
  uint32_t v = lds_ld(p);
  if (v < target) {
    const uint64_t t0 = wall_clock64();
    for (uint32_t it = 1;; ++it) {
      __builtin_amdgcn_s_sleep(1);
      v = lds_ld(p);
      if (v >= target) break;
      if ((it & 1023u) == 0u && uni(wait_expired(P, t0) ? 1 : 0)) {
        ok = false;
        v = 0;
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
  return v;
}

// ------------------------------------------------------------ cross-CU hand-off
#define TD_CPOL_SC1 16  // buffer-load cache policy: agent scope

DEV __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Loads whose completion the compiler does not track.  The compiler waits for
// a tracked load before its result is used, and when LDS-DMA chunks of a
// run-time count were issued after the load it can only wait for all of them
// (vmcnt(0)), which would hold every hand-off poll and every prefetched operand
// until the weight ring's newest chunks land.  With these, the kernel waits
// itself (vmcnt of exactly the loads issued after) and then fences the
// registers (reg_fence) so that no use is scheduled above that wait.
DEV u32x4 ld16_sc1_untracked(const void* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off sc1" : "=v"(v) : "v"(p) : "memory");
  return v;
}
DEV uint32_t ld4_untracked(const void* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
DEV uint32_t ld2_untracked(const void* p) {
  uint32_t v;
  asm volatile("global_load_ushort %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
template <class T>
DEV void reg_fence(T& v) {
  asm volatile("" : "+v"(v));
}

DEV void st_tag(uint2* p, float v, uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(w) : "memory");
}

// ------------------------------------------------------------ attention task
// Split-K decode attention: kv head g's positions 0..pos are cut into chunks of
// chunk_len; one CU per (g, chunk) computes a partial (m, l, acc) for each of
// g's query heads; on the CU of chunk 0 each query-head wave merges its head
// ("One launch per token", "The attention trap").  Task (g, c) runs on CU
// c nkv + g.  Workgroups are dealt to the 8 XCDs in turn, so with 8 (or 16)
// kv heads every chunk of head g, and its merge, run on one XCD, and the
// merge CUs sit on different XCDs at every position.  (The head-major order,
// CU g n_used + c, put two merge CUs on each of four XCDs whenever n_used was
// even: the O stage's hand-off then took about 1.2 us longer, and llama1b's
// steps at positions 576..639 17 us longer than at 512..575.)
struct AttnTask {
  int valid, g, c, t0, t1, ntiles, n_used;
};
DEV AttnTask attn_task(const td_kparams& P, int cu, int pos) {
  AttnTask t;
  t.n_used = (pos + P.chunk_len) / P.chunk_len;  // chunks covering positions 0..pos
  t.valid = cu < P.nkv * t.n_used;
  t.g = t.valid ? cu % P.nkv : 0;
  t.c = t.valid ? cu / P.nkv : 0;
  t.t0 = t.c * P.chunk_len;
  t.t1 = min(t.t0 + P.chunk_len, pos + 1);
  t.ntiles = t.valid ? (t.t1 - t.t0 + TD_TILE - 1) / TD_TILE : 0;
  return t;
}

// LDS buffer of the k-th tile (counted over the whole launch): with nb
// buffers, nb - 1 tiles are in flight while one is consumed.
DEV uint8_t* tile_buf(const td_kparams& P, uint8_t* lds, uint32_t k) {
  const uint32_t b = P.tile_bufs == 3 ? k % 3u : k & (uint32_t)(P.tile_bufs - 1);  // 1, 2 or 3 buffers
  return lds + P.off_tile + (int)b * P.tile_stride;
}

// K and V rows [tb, tb + nv) of the tile, except row pos (written during this
// very step; it comes from the published copy), into the LDS tile; rows past
// the chunk end read as zero.  The loads are agent-scope: rows written by an
// earlier step of the same launch come from other CUs.
DEV void load_tile(const td_kparams& P, uint8_t* buf, int layer, const AttnTask& T, int tile, int pos) {
  const int lane = lane_id();
  const int d = P.d;
  const int tb = T.t0 + tile * TD_TILE;
  const int nv = min(TD_TILE, T.t1 - tb);
  const size_t head_off = ((size_t)layer * P.nkv + T.g) * P.max_ctx;
  const __amdgpu_buffer_rsrc_t RK = rsrc(P.kc + (head_off + tb) * d, (uint32_t)(nv * d * 2));
  const __amdgpu_buffer_rsrc_t RV = rsrc(P.vc + (head_off + tb) * d, (uint32_t)(nv * d * 2));
  uint16_t* kt = (uint16_t*)buf;
  uint16_t* vt = kt + TD_TILE * (d + 8);
  const int q16 = d / 8;  // 16-byte pieces per row
  const int npiece = TD_TILE * q16;
  for (int i0 = 0; i0 < npiece; i0 += 8 * 64) {  // 8 K and 8 V loads in flight per lane (d = 64: one round)
    u32x4 kr[8], vr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t off = (uint32_t)(i0 + k * 64 + lane) * 16u;  // out of range reads 0
      kr[k] = __builtin_amdgcn_raw_buffer_load_b128(RK, off, 0, TD_CPOL_SC1);
      vr[k] = __builtin_amdgcn_raw_buffer_load_b128(RV, off, 0, TD_CPOL_SC1);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = i0 + k * 64 + lane;
      if (i < npiece) {
        const int row = i / q16, pc = i - row * q16;
        if (row >= nv || tb + row != pos) {
          *(u32x4*)(kt + row * (d + 8) + pc * 8) = kr[k];
          *(u32x4*)(vt + row * d + pc * 8) = vr[k];
        }
      }
    }
  }
}

// The same rows by LDS DMA (buffer_load ... lds, 16 bytes per lane, one KiB
// per instruction), so that the sync wave can keep several tiles in flight
// (three tile buffers; with fewer, load_tile's register path is as fast and
// does not share the LDS-DMA path with the weight streams): K rows
// at a pitch of 2 d + 16 bytes (a lane whose 16 bytes fall in a row's padding
// reads that row's first bytes again), then V rows unpadded.  Rows past the
// chunk end read as zero (the buffer's range ends there).  The loads are
// agent-scope: rows written by an earlier step of the same launch come from
// other CUs.  Row pos (written during this very step) arrives stale and is
// replaced from the published copy once the tile has landed (patch_pos_row).
// 17 instructions per tile at d = 64.
#define LDSPTR(p) ((__attribute__((address_space(3))) void*)(p))
DEV void issue_tile(const td_kparams& P, uint8_t* buf, int layer, const AttnTask& T, int tile) {
  const int lane = lane_id();
  const int d = P.d;
  const int tb = T.t0 + tile * TD_TILE;
  const int nv = min(TD_TILE, T.t1 - tb);
  const size_t head_off = ((size_t)layer * P.nkv + T.g) * P.max_ctx;
  const __amdgpu_buffer_rsrc_t RK = rsrc(P.kc + (head_off + tb) * d, (uint32_t)(nv * d * 2));
  const __amdgpu_buffer_rsrc_t RV = rsrc(P.vc + (head_off + tb) * d, (uint32_t)(nv * d * 2));
  const int kpitch = 2 * d + 16, kw = TD_TILE * kpitch / 1024, vw = TD_TILE * 2 * d / 1024;
  for (int w = 0; w < kw; ++w) {
    const int off = 1024 * w + 16 * lane, row = off / kpitch, in = off - row * kpitch;
    const uint32_t src = (uint32_t)(row * 2 * d + (in < 2 * d ? in : 0));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(RK, LDSPTR(buf + 1024 * w), 16, src, 0, 0, TD_CPOL_SC1);
  }
  uint8_t* vb = buf + TD_TILE * kpitch;
  for (int w = 0; w < vw; ++w)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(RV, LDSPTR(vb + 1024 * w), 16, (uint32_t)(1024 * w + 16 * lane), 0, 0,
                                             TD_CPOL_SC1);
}

// this position's K and V rows (LDS fp32 holding bf16 values) into the tile
// when the tile holds position pos
DEV void patch_pos_row(const td_kparams& P, uint8_t* lds, uint8_t* buf, const AttnTask& T, int tile, int pos) {
  const int tb = T.t0 + tile * TD_TILE;
  if (pos < tb || pos >= tb + TD_TILE || pos >= T.t1) return;
  const int d = P.d, row = pos - tb;
  const td_attn_lds A = td_attn_layout(d, P.group, P.n_chunks_max, false);  // (kvp: the same in every layout)
  const float* kvp = (const float*)(lds + P.off_attn + A.kvp);
  uint16_t* kt = (uint16_t*)buf;
  uint16_t* vt = kt + TD_TILE * (d + 8);
  for (int e = lane_id(); e < d; e += 64) {
    kt[row * (d + 8) + e] = (uint16_t)(__float_as_uint(kvp[e]) >> 16);
    vt[row * d + e] = (uint16_t)(__float_as_uint(kvp[d + e]) >> 16);
  }
}

// ------------------------------------------------------------ compute waves
// Each compute wave streams its own packed weight stream (one contiguous array
// per wave, built at create time in exactly the order consumed here) into its
// LDS ring of S slots with global_load_lds, keeping at most TD_FLIGHT chunks
// in flight: a CU serves its memory requests roughly in order, so every byte
// queued ahead of a hand-off (an epilogue store, an input poll) delays it,
// while a wave's own streaming rate is its bytes in flight over the load
// latency; 6 KiB per wave (48 KiB per CU) was the best of 3, 4 and 6 measured
// on the Llama-3.2-1B shape.  While a wave waits for a stage's inputs it tops
// the ring up toward its S slots, so the stream keeps going through the
// hand-offs and the next stage starts from chunks that are already in LDS.  A
// wave's loads complete in issue order, so "chunk t is in LDS" is "at most the
// loads issued after chunk t are outstanding"; the chunk loop waits only when
// the chunk is not already known to have landed.  A launch of several steps
// runs the stream once per step: once a step's stream is consumed the counts
// start over, and the next step's first chunks stream while its token is
// decided.  (The per-chunk path is kept free of any step logic: each
// instruction there is paid once per KiB streamed.)
#define TD_DMA_NT 2   // cache policy of the weight stream: non-temporal
#ifndef TD_FLIGHT
#define TD_FLIGHT 6   // chunks of its own stream a compute wave keeps in flight at most
#endif

struct CState {
  uint8_t* lds;
  uint32_t* ctl;
  float* xin;
  float* own;
  float* out;
  uint8_t* ring;
  uint8_t* sring;
  const uint8_t* fbase;  // the next chunk to issue (wave-uniform; a lane loads its 16 bytes)
  const uint8_t* sbase;  // the next int4 chunk's 64-byte scale block
  const uint8_t* fbase0;  // the stream's first chunk and first scale block
  const uint8_t* sbase0;
  uint32_t issued, n_tot, n4;  // chunks issued, stream length, leading int4 chunks
  uint32_t lk;                 // chunks [0, lk) are known to be in LDS
  int islot;                   // ring slot of the next chunk to issue
  uint32_t t;                  // chunks consumed
  int slot;                    // ring slot of chunk t
  uint32_t nrv;                // rendezvous passed
  // The stream in consumption order is a sequence of runs of contiguous
  // chunks; the chunk issued next belongs to the run that ends before chunk
  // run_end.  A dense model's step is one run.  A MoE layer is three kinds of
  // run: its fixed part (QKV, O, router rows), then the gate/up block of the
  // expert in this CU's slot and the down blocks of the chosen experts in slot
  // order, which can be issued only once the wave has that layer's routing.
  uint32_t run_end;
  int rl, rp;                  // MoE: layer and phase of the current run (0 fixed, 1 gate/up, 2 + j down slot j)
  int route_layer;             // MoE: the layer whose routing this wave holds (-1: none yet in this step)
  int ids_v;                   // MoE: lane j < top_k: the j-th chosen expert
  float wts_v;                 //      and its router probability
  uint32_t m_fixed, m_gu, m_down, m_head, m_stride, m_slot;  // MoE: run lengths (chunks), layer stride, GU slot
  float inv_mlp;               // MoE: the MLP RMSNorm factor of the layer (the router stage computes it)
  bool ok;
  int ranges;                  // lane 2 s: this CU's first unit of unit space s; lane 2 s + 1: its count
  DEV int unit_lo(int sp) const { return __builtin_amdgcn_readlane(ranges, 2 * sp); }
  DEV int unit_n(int sp) const { return __builtin_amdgcn_readlane(ranges, 2 * sp + 1); }
};
// The state's type says whether the model has MoE layers, so that a dense
// model's kernel is compiled without the routed-run logic on its chunk path.
template <bool M>
struct CStateT : CState {
  static constexpr bool kMoe = M;
};

// loads of chunks [a, b): an int4 chunk is two (its codes and its scales)
DEV uint32_t ops_of(const CState& C, uint32_t a, uint32_t b) {
  const uint32_t hi4 = min(b, C.n4);
  return (b - a) + (hi4 > a ? hi4 - a : 0u);
}
// s_waitcnt vmcnt(n) for a run-time n (values past the table wait for
// everything, which is only more conservative)
DEV void vmcnt_rt(uint32_t n) {
  switch (n) {
    case 1: vmcnt_wait<1>(); break;
    case 2: vmcnt_wait<2>(); break;
    case 3: vmcnt_wait<3>(); break;
    case 4: vmcnt_wait<4>(); break;
    case 5: vmcnt_wait<5>(); break;
    case 6: vmcnt_wait<6>(); break;
    case 7: vmcnt_wait<7>(); break;
    case 8: vmcnt_wait<8>(); break;
    case 9: vmcnt_wait<9>(); break;
    case 10: vmcnt_wait<10>(); break;
    case 11: vmcnt_wait<11>(); break;
    case 12: vmcnt_wait<12>(); break;
    case 13: vmcnt_wait<13>(); break;
    case 14: vmcnt_wait<14>(); break;
    case 15: vmcnt_wait<15>(); break;
    case 16: vmcnt_wait<16>(); break;
    case 17: vmcnt_wait<17>(); break;
    case 18: vmcnt_wait<18>(); break;
    case 19: vmcnt_wait<19>(); break;
    case 20: vmcnt_wait<20>(); break;
    case 21: vmcnt_wait<21>(); break;
    case 22: vmcnt_wait<22>(); break;
    case 23: vmcnt_wait<23>(); break;
    case 24: vmcnt_wait<24>(); break;
    default: vmcnt_wait<0>(); break;
  }
}
static_assert(TD_FLIGHT >= 1 && 4 * TD_FLIGHT <= 24, "vmcnt_rt covers the waits of up to 2 TD_FLIGHT int4 chunks");
// Waits until no load older than chunk a is outstanding (chunks [a, issued)
// may still be in flight).  The steady-state case, the newest TD_FLIGHT - 1
// chunks all of one format, is one compile-time wait.
DEV void wait_older_than(const CState& C, uint32_t a) {
  const uint32_t m = C.issued - a;
  if (m == TD_FLIGHT - 1 && a >= C.n4) vmcnt_wait<TD_FLIGHT - 1>();
  else if (m == TD_FLIGHT - 1 && C.issued <= C.n4) vmcnt_wait<2 * TD_FLIGHT - 2>();
  else vmcnt_rt(ops_of(C, a, C.issued));
}

DEV void issue_chunk(const td_kparams& P, CState& C) {
  const int lane = lane_id();
  __builtin_amdgcn_global_load_lds((const void*)(C.fbase + lane * 16), LDSPTR(C.ring + C.islot * TD_CHUNK), 16, 0,
                                   TD_DMA_NT);
  C.fbase += TD_CHUNK;
  if (C.issued < C.n4) {  // the chunk's 32 fp16 scales: 16 lanes x 4 bytes
    if (lane < 16)
      __builtin_amdgcn_global_load_lds((const void*)(C.sbase + lane * 4), LDSPTR(C.sring + C.islot * TD_SCHUNK), 4,
                                       0, TD_DMA_NT);
    C.sbase += TD_SCHUNK;
  }
  ++C.issued;
  C.islot = C.islot + 1 == P.ring_slots ? 0 : C.islot + 1;
}
// MoE: moves the issue position to the next non-empty run; false (and no
// change) if that run needs routing the wave does not have yet.
DEV bool run_advance(const td_kparams& P, CState& C) {
  if (!P.E) return false;
#pragma unroll 1
  for (;;) {
    int l = C.rl, p = C.rp + 1;
    if (p > 1 + P.topk) {
      ++l;
      p = 0;
    }
    if (l > P.L) return false;
    size_t off = (size_t)l * C.m_stride;
    uint32_t len;
    if (p == 0) {
      len = l < P.L ? C.m_fixed : C.m_head;
    } else {
      len = p == 1 ? C.m_gu : C.m_down;
      if (len && C.route_layer != l) return false;
      if (p == 1) off += C.m_fixed + (uint32_t)__builtin_amdgcn_readlane(C.ids_v, (int)C.m_slot) * C.m_gu;
      else off += C.m_fixed + (size_t)P.E * C.m_gu + (uint32_t)__builtin_amdgcn_readlane(C.ids_v, p - 2) * C.m_down;
    }
    C.rl = l;
    C.rp = p;
    C.fbase = C.fbase0 + off * TD_CHUNK;
    C.run_end = C.issued + len;
    if (len) return true;
  }
}
template <class CS>
DEV bool ring_room(const td_kparams& P, CS& C) {
  if (C.issued >= C.n_tot || C.issued >= C.t + (uint32_t)P.ring_slots) return false;
  if constexpr (CS::kMoe) return C.issued < C.run_end || run_advance(P, C);
  return true;
}
// After a chunk is consumed: one more chunk in flight if its slot is free, first
// waiting (only if needed) until at most TD_FLIGHT - 1 chunks are outstanding.
template <class CS>
DEV void refill(const td_kparams& P, CS& C) {
  if (!ring_room(P, C)) return;
  if (C.issued - C.lk >= TD_FLIGHT) {
    wait_older_than(C, C.issued - (TD_FLIGHT - 1));
    C.lk = C.issued - (TD_FLIGHT - 1);
  }
  issue_chunk(P, C);
}
// During a wait: up to TD_FLIGHT more chunks into free slots, without waiting
// (so up to 2 TD_FLIGHT chunks can be in flight for a while; the waits below
// count loads, not an assumed depth).
template <class CS>
DEV void topup(const td_kparams& P, CS& C) {
#pragma unroll 1
  for (int k = 0; k < TD_FLIGHT && ring_room(P, C); ++k) issue_chunk(P, C);
}
// The next chunk of the stream, once it is in LDS.
template <class CS>
DEV const uint8_t* chunk_wait(CS& C) {
  if (C.t >= C.lk) {
    wait_older_than(C, C.t + 1);
    C.lk = C.t + 1;
  }
  return C.ring + C.slot * TD_CHUNK;
}
// (REFILL false: the slot stays free until a later top-up)
template <class CS, bool REFILL = true>
DEV void chunk_release(const td_kparams& P, CS& C) {
  lds_fence();  // the slot has been read out
  ++C.t;
  C.slot = C.slot + 1 == P.ring_slots ? 0 : C.slot + 1;
  if (REFILL) refill(P, C);
}


// Waits until the pairs [lo, hi) of src (lo, hi even) all carry `tag` and
// copies their values to dst[lo, hi) (LDS).  Each round loads up to W 16-byte
// units (two pairs) per lane and re-polls the units still missing.  After a
// round's loads are issued, the (compute) wave tops its weight ring up (with
// TOPUP): those chunk loads are younger than the poll's, so waiting for the
// poll never waits for them, and every chunk issued before the round has
// landed once the round's results are in.  Without TOPUP the CU's memory queue
// stays short, so the next round's loads come back sooner: for a poll on the
// critical path of only a few CUs, whose streaming is not worth the delay.
// false: the wait timed out (or another wait did).
template <int W, bool TOPUP = true, class CS>
DEV bool poll_pairs(const td_kparams& P, const uint2* src, int lo, int hi, uint32_t tag, float* dst, CS& C) {
  const int lane = lane_id();
  const int nu = (hi - lo) >> 1;
  if (nu <= 0) {
    vm_drain();  // the operands prefetched ahead of the poll have landed
    return true;
  }
  const uint8_t* base = (const uint8_t*)(src + lo);
  float* d = dst + lo;
  const uint64_t t0 = wall_clock64();
  for (int b0 = 0; b0 < nu; b0 += W * 64) {
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < W; ++k)
      if (b0 + k * 64 + lane < nu) pend |= 1u << k;
    for (uint32_t it = 0;; ++it) {
      const uint32_t landed_before = C.issued;
      u32x4 r[W];
#pragma unroll
      for (int k = 0; k < W; ++k)  // past the slice: its last unit again (ignored)
        r[k] = ld16_sc1_untracked(base + (size_t)min(b0 + k * 64 + lane, nu - 1) * 16u);
      if (TOPUP) topup(P, C);
      // only the top-up's loads may still be outstanding: the poll's, and every
      // load issued before the round, are complete
      vmcnt_rt(ops_of(C, landed_before, C.issued));
#pragma unroll
      for (int k = 0; k < W; ++k) reg_fence(r[k]);
      if (C.lk < landed_before) C.lk = landed_before;
#pragma unroll
      for (int k = 0; k < W; ++k) {
        if (((pend >> k) & 1u) && r[k].y == tag && r[k].w == tag) {
          const int u = b0 + k * 64 + lane;
          d[2 * u] = __uint_as_float(r[k].x);
          d[2 * u + 1] = __uint_as_float(r[k].z);
          pend &= ~(1u << k);
        }
      }
      if (!__any(pend != 0u)) break;
      if ((it & 3u) == 3u && uni(wait_expired(P, t0) ? 1 : 0)) return false;
    }
  }
  return true;
}

DEV void rendezvous(const td_kparams& P, CState& C) {
  ++C.nrv;
  lds_fence();
  if (lane_id() == 0) lds_add(C.ctl + TD_CTL_RV, 1u);
  (void)lds_wait_ge(P, C.ctl + TD_CTL_RV, TD_NW * C.nrv, C.ok);
}

// One row of the current stage: J chunks of the stream against xin.  The
// format is a template parameter so that each chunk loop is compiled for one
// format only: every instruction in it is paid once per KiB streamed.
template <int FMT, bool QUIET = false, class CS>
DEV float gemv_row(const td_kparams& P, CS& C, int J, const float* x, int qfrom = 0) {
  const int lane = lane_id();
  float acc = 0.f;
  for (int j = 0; j < J; ++j) {
    const uint8_t* ch = chunk_wait(C);
    const u32x4 w = *(const u32x4*)(ch + lane * 16);
    if (FMT == 0) {
      acc += dot_bf16(w, x + j * 512 + lane * 8);
    } else {
      const uint2 sc = int4_lane_scales(C.sring + C.slot * TD_SCHUNK, lane);
      acc += dot_int4(w, x + j * 2048, lane, sc);
    }
    if (QUIET && j >= qfrom) chunk_release<CS, false>(P, C);
    else chunk_release(P, C);
  }
  return wave_sum(acc);
}

// The rows of a wave's n units (rpu rows each), their dot products to the LDS
// output area; `first` gets the time the first chunk was in LDS (when tracing).
// QUIET: the stage's last TD_FLIGHT chunks are consumed without refilling their
// slots, so that none of the wave's weight loads are still queued when the
// stage's stores go out; the caller tops the ring up behind those stores.  On
// the Llama-3.2-1B shape this measured 0.676 -> 0.664 ms per step; int4 streams
// (two loads a chunk, one chunk a row) measured slower with it and keep the
// plain form.
template <int FMT, bool QUIET, class CS>
DEV void gemv_rows(const td_kparams& P, CS& C, const Shape& g, int n, int wave, uint64_t& first) {
  if (P.trace && n > 0) {
    (void)chunk_wait(C);
    first = wall_clock64();
  }
  for (int k = 0; k < n; ++k) {
    const int idx = wave + k * TD_NW;  // u - u0
    float r0, r1 = 0.f;
    if (QUIET && k == n - 1) {  // the last unit: chunks from rpu J - TD_FLIGHT on leave their slots free
      r0 = gemv_row<FMT, true>(P, C, g.J, C.xin, g.rpu * g.J - TD_FLIGHT);
      if (g.rpu == 2) r1 = gemv_row<FMT, true>(P, C, g.J, C.xin, g.J - TD_FLIGHT);
    } else {
      r0 = gemv_row<FMT>(P, C, g.J, C.xin);
      if (g.rpu == 2) r1 = gemv_row<FMT>(P, C, g.J, C.xin);
    }
    if (lane_id() == 0) {
      C.out[idx * g.rpu] = r0;
      if (g.rpu == 2) C.out[idx * 2 + 1] = r1;
    }
  }
}

// The MoE down stage of a wave's n units: for each slot j in order, the rows of
// the j-th chosen expert against slot j's activations (xin + j I), the dot
// products summed with the slot's router probability as y = fma(w_j, d_j, y)
// from y = 0 (the per-op executor's order, so the bits agree).
template <int FMT, class CS>
DEV void moe_down_rows(const td_kparams& P, CS& C, const Shape& g, int n, int wave, uint64_t& first) {
  if (P.trace && n > 0) {
    (void)chunk_wait(C);
    first = wall_clock64();
  }
  for (int j = 0; j < P.topk; ++j) {
    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(C.wts_v), j));
    const float* xj = C.xin + (size_t)j * P.I;
    for (int k = 0; k < n; ++k) {
      const int idx = wave + k * TD_NW;
      const float dk = gemv_row<FMT>(P, C, g.J, xj);
      if (lane_id() == 0) C.out[idx] = fmaf(wj, dk, j == 0 ? 0.f : C.out[idx]);
    }
  }
}

// The wave's routing of a MoE layer from the staged router logits: its own
// moe_select (every wave computes the same bits), kept one expert per lane;
// CU 0's wave 0 reports it (expert ids and weights of the layer) and raises the
// error bit on a non-finite router logit.
DEV void moe_route(const td_kparams& P, CState& C, uint8_t* lds, int wave, int layer) {
  const float* zs = (const float*)(lds + P.off_route);
  int32_t* ids = (int32_t*)(lds + P.off_route + TD_MAX_EXPERTS * 4) + wave * 2 * TD_MAX_TOPK;
  float* wts = (float*)(ids + TD_MAX_TOPK);
  const bool bad = moe_select(P.E, P.topk, zs, ids, wts);
  lds_fence();
  const int lane = lane_id();
  C.ids_v = lane < P.topk ? ids[lane] : 0;
  C.wts_v = lane < P.topk ? wts[lane] : 0.f;
  C.route_layer = layer;
  if (blockIdx.x == 0 && wave == 0) {
    if (lane < P.topk) {
      P.expert_ids[layer * P.topk + lane] = C.ids_v;
      P.expert_w[layer * P.topk + lane] = C.wts_v;
    }
    if (bad && lane == 0) atomicOr(P.err, TD_ERRBIT_NONFINITE);
  }
}

// Input slice of a GEMV stage into xin: the published vector (polled), or the
// bf16 embedding row for the first layer.  With gains (the RMSNorm stages) the
// slice's sum of squares goes to the control block and the slice is multiplied
// by the gains.  The last wave zeroes the tail up to the chunk multiple.
template <class CS>
DEV void stage_gemv_input(const td_kparams& P, CS& C, int wave, int kind, int K, const uint2* src,
                          const uint16_t* erow, uint32_t tag, uint32_t g0, uint32_t g1, uint32_t g2, uint32_t g3,
                          const uint16_t* gain) {
  int lo, hi;
  td_slice(K, wave, &lo, &hi);
  if (erow) {
    for (int u = (lo >> 1) + lane_id(); u < (hi >> 1); u += 64) {
      const uint32_t e = *(const uint32_t*)(erow + 2 * u);
      C.xin[2 * u] = bf_lo(e);
      C.xin[2 * u + 1] = bf_hi(e);
    }
    vm_drain();  // the gains and biases loaded ahead (no input poll waits for them here)
  } else {
    C.ok &= poll_pairs<8>(P, src, lo, hi, tag, C.xin, C);
  }
  reg_fence(g0);
  reg_fence(g1);
  reg_fence(g2);
  reg_fence(g3);
  if (gain) {
    lds_fence();
    const float ss = slice_ssq(C.xin, lo, hi);
    if (lane_id() == 0) ((float*)C.ctl)[TD_CTL_SSQ + wave] = ss;
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // the gains fetched ahead of the rendezvous
      const int u = (lo >> 1) + lane_id() + 64 * k;
      const uint32_t g = k == 0 ? g0 : k == 1 ? g1 : k == 2 ? g2 : g3;
      if (u < (hi >> 1)) {
        C.xin[2 * u] *= bf_lo(g);
        C.xin[2 * u + 1] *= bf_hi(g);
      }
    }
    for (int u = (lo >> 1) + lane_id() + 256; u < (hi >> 1); u += 64) {
      const uint32_t g = *(const uint32_t*)(gain + 2 * u);
      C.xin[2 * u] *= bf_lo(g);
      C.xin[2 * u + 1] *= bf_hi(g);
    }
  }
  if (wave == TD_NW - 1) {  // the zero activations the padded tail of a row's last chunk meets
    const int ce = P.wf && kind != TD_ST_HEAD ? 2048 : 512;
    int kp = (K + ce - 1) / ce * ce;
    if constexpr (CS::kMoe)
      if (kind == TD_ST_DOWN) kp = max(kp, td_moe_down_reach(P.topk, P.I));  // bf16 expert rows
    for (int i = K + lane_id(); i < kp; i += 64) C.xin[i] = 0.f;
  }
}

// The GEMV part of a stage for one compute wave: the rows of its units (their
// dot products to the LDS output area), then the units' epilogues, one unit per
// lane, with every store of the stage issued after its last row: a store
// counts among the wave's outstanding loads, so a store issued between rows
// would make every following chunk wait for it.
template <int WF, class CS>
DEV void gemv_wave(const td_kparams& P, CS& C, int wave, int kind, int layer, int pos, uint32_t tag, float inv,
                   float bias_a, float bias_b, uint64_t& first) {
  const int lane = lane_id();
  const Shape g = shape_of<CS::kMoe>(P, kind);
  const int u0 = C.unit_lo(g.space), u1 = C.unit_lo(g.space) + C.unit_n(g.space);
  const int n = wave_units(u1 - u0, wave);
  bool routed = false;
  if constexpr (CS::kMoe) {  // the MoE down stage sums over the slots (bf16 only)
    if (kind == TD_ST_DOWN) {
      moe_down_rows<TD_WF_BF16>(P, C, g, n, wave, first);
      routed = true;
    }
  }
  if (routed) {
  } else if (WF == TD_WF_BF16 || kind == TD_ST_HEAD || kind == TD_ST_ROUTER) {
    gemv_rows<TD_WF_BF16, WF == TD_WF_BF16>(P, C, g, n, wave, first);
  } else {
    gemv_rows<TD_WF_INT4_G64, false>(P, C, g, n, wave, first);
  }
  lds_fence();
  float bv = -__builtin_inff();
  int bi = 0x7fffffff, bad = 0;
  for (int k = lane; k < n; k += 64) {
    const int idx = wave + k * TD_NW;
    const int u = u0 + idx;
    if (kind == TD_ST_QKV) {
      const int half = P.d >> 1;
      const int ra = unit_row(P, TD_ST_QKV, u, 0);
      const int i = ra % P.d;
      float a = C.out[2 * idx] * inv, b = C.out[2 * idx + 1] * inv;
      if (P.has_bias) {  // lane k fetched unit k's biases
        a += bias_a;
        b += bias_b;
      }
      if (ra < P.qd + P.kvd) {  // q or k: rotate the pair by pos * theta_i
        const float* cs = (const float*)(C.lds + P.off_rope);
        rope_pair(a, b, cs[2 * i], cs[2 * i + 1]);
      }
      const int gw = (P.group + 2) * P.d;  // published block of one kv head
      if (ra < P.qd) {
        const int h = ra / P.d, gg = h / P.group;
        uint2* pub = P.tq + (size_t)gg * gw + (h - gg * P.group) * P.d;
        st_tag(pub + i, a, tag);
        st_tag(pub + i + half, b, tag);
      } else {
        const bool isk = ra < P.qd + P.kvd;
        const int gg = (ra - P.qd - (isk ? 0 : P.kvd)) / P.d;
        const uint32_t ab = f2bf(a), bbits = f2bf(b);
        uint16_t* row = (isk ? P.kc : P.vc) + (((size_t)layer * P.nkv + gg) * P.max_ctx + pos) * P.d;
        st_u16_sc1(row + i, ab);  // agent scope: a later step of the launch reads it on other CUs
        st_u16_sc1(row + i + half, bbits);
        uint2* pub = P.tq + (size_t)gg * gw + (P.group + (isk ? 0 : 1)) * P.d;
        st_tag(pub + i, __uint_as_float(ab << 16), tag);
        st_tag(pub + i + half, __uint_as_float(bbits << 16), tag);
      }
    } else if (kind == TD_ST_O || kind == TD_ST_DOWN) {
      const float v = C.own[idx] + C.out[idx];
      C.own[idx] = v;
      st_tag((kind == TD_ST_O ? P.tx_mid : P.tx_out) + u, v, tag);
    } else if (kind == TD_ST_GU) {  // MoE: u is slot u / I's unit
      const float gt = C.out[2 * idx] * inv, up = C.out[2 * idx + 1] * inv;
      st_tag(P.tact + u, gt / (1.0f + expf(-gt)) * up, tag);
    } else if (kind == TD_ST_ROUTER) {
      st_tag(P.trl + u, C.out[idx] * inv, tag);
      // an odd expert count: the logits are read in pairs, the last one padded with -inf
      if ((P.E & 1) && u == P.E - 1) st_tag(P.trl + P.E, -__builtin_inff(), tag);
    } else {  // HEAD
      const float v = C.out[idx] * inv;
      P.logits[u] = v;
      if (!isfinite(v)) bad = 1;
      else if (cand_better(v, u, bv, bi)) { bv = v; bi = u; }
    }
  }
  if (WF == TD_WF_BF16) topup(P, C);  // the slots the quiet rows left free, behind the stores
  if (kind == TD_ST_HEAD) {
    cand_wave_max(bv, bi);
    bad = __any(bad);
    if (lane == 0) {
      uint32_t* cd = C.ctl + TD_CTL_CAND + 4 * wave;
      lds_st(cd + 0, __float_as_uint(bv));
      lds_st(cd + 1, (uint32_t)bi);
      lds_st(cd + 2, (uint32_t)bad);
    }
    lds_fence();
    if (lane == 0) lds_add(C.ctl + TD_CTL_HEADDONE, 1u);
  }
}

// Query-head wave h of an attention task: the tiles the sync wave makes ready,
// then either its partial (chunk c > 0) or, on the chunk-0 CU, the merge of all
// chunks' partials of its head, o = sum_c acc_c e^(m_c - M) / sum_c l_c e^(m_c - M)
// (the chunks summed in chunk order), published.
template <int D, class CS>
DEV void attn_wave_d(const td_kparams& P, CS& C, uint8_t* lds, int h, const AttnTask& T, uint32_t tag,
                     uint32_t& tiles_seen, uint64_t& first) {
  const int lane = lane_id();
  const int G = P.group;
  const td_attn_lds A = td_attn_layout(D, G, P.n_chunks_max);
  uint8_t* base = lds + P.off_attn;
  const float* qs = (const float*)(base + A.q) + h * D;
  float* ps = (float*)(base + A.p) + h * TD_TILE;
  float m = -__builtin_inff(), l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int tile = 0; tile < T.ntiles; ++tile) {
    const uint16_t* kt = (const uint16_t*)tile_buf(P, lds, tiles_seen);
    const uint16_t* vt = kt + TD_TILE * (D + 8);
    (void)lds_wait_ge(P, C.ctl + TD_CTL_TREADY, ++tiles_seen, C.ok);
    attn_tile<D>(qs, kt, vt, ps, min(TD_TILE, T.t1 - (T.t0 + tile * TD_TILE)), m, l, acc);
    lds_fence();
    if (lane == 0) lds_add(C.ctl + TD_CTL_TDONE, 1u);
    if (P.trace && !first) first = wall_clock64();
  }
  acc = attn_finish<D>(acc);
  constexpr int st = D + 4;
  uint2* myparts = P.tpart + ((size_t)T.g * G + h) * P.n_chunks_max * st;
  if (T.c > 0) {
    uint2* dst = myparts + (size_t)T.c * st;
    if (lane < D / 4) {
      st_tag(dst + 4 * lane + 0, acc.x, tag);
      st_tag(dst + 4 * lane + 1, acc.y, tag);
      st_tag(dst + 4 * lane + 2, acc.z, tag);
      st_tag(dst + 4 * lane + 3, acc.w, tag);
    }
    if (lane == 0) {
      st_tag(dst + D, m, tag);
      st_tag(dst + D + 1, l, tag);
      st_tag(dst + D + 2, 0.f, tag);
      st_tag(dst + D + 3, 0.f, tag);
    }
    return;
  }
  const int n = T.n_used;  // <= 64
  float* mb = (float*)(base + A.merge) + (size_t)h * (P.n_chunks_max - 1) * st;  // chunks 1..n-1
  // the merging CUs (one per kv head) poll without topping up: every CU's
  // O stage waits for their outputs.  Where the staging runs on into the K/V
  // tile buffer, it waits until every query-head wave is done with the tiles.
  if (P.merge_in_tile) (void)lds_wait_ge(P, C.ctl + TD_CTL_TDONE, (uint32_t)G * tiles_seen, C.ok);
  // (d = 128: 9 loads per lane, so that the nine chunks of a 576-position
  // context are polled in one round; measured faster than 8 or 12)
  if (n > 1) C.ok &= poll_pairs<D == 128 ? 9 : 8, false>(P, myparts + st, 0, (n - 1) * st, tag, mb, C);
  lds_fence();
  const f32x4 o = attn_merge<D>(acc, m, l, mb, n, ps);
  if (lane < D / 4) {
    uint2* dst = P.to + ((size_t)T.g * G + h) * D + 4 * lane;
    st_tag(dst + 0, o.x, tag);
    st_tag(dst + 1, o.y, tag);
    st_tag(dst + 2, o.z, tag);
    st_tag(dst + 3, o.w, tag);
  }
}

// The same for a MoE kernel, whose attention may spread a head over W waves
// (td_attn_waves): attention wave w of a task takes query head h = w % group
// and rows [s 64 / W,
// (s + 1) 64 / W) of every tile the sync wave makes ready (s = w / group, W
// waves a head).  A head's waves 1 .. W - 1 leave their states in LDS and are
// done; its first wave folds them in, in wave order, and publishes the chunk's
// partial (chunk c > 0) or, on the chunk-0 CU, merges all chunks' partials of
// its head, o = sum_c acc_c e^(m_c - M) / sum_c l_c e^(m_c - M) (the chunks
// summed in chunk order), and publishes o.  nattn counts the attention stages
// this wave has taken part in (the partial-state counters are monotonic).
template <int D, class CS>
DEV void attn_wave_split(const td_kparams& P, CS& C, uint8_t* lds, int w, const AttnTask& T, uint32_t tag,
                         uint32_t& tiles_seen, uint32_t& nattn, uint64_t& first) {
  const int lane = lane_id();
  const int G = P.group, W = td_attn_waves(D, G, true);
  const int h = w % G, s = w / G;
  const td_attn_lds A = td_attn_layout(D, G, P.n_chunks_max, true);
  uint8_t* base = lds + P.off_attn;
  const float* qs = (const float*)(base + A.q) + h * D;
  float* ps = (float*)(base + A.p) + w * TD_TILE;
  float m = -__builtin_inff(), l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  ++nattn;
  for (int tile = 0; tile < T.ntiles; ++tile) {
    const uint16_t* kt = (const uint16_t*)tile_buf(P, lds, tiles_seen);
    const uint16_t* vt = kt + TD_TILE * (D + 8);
    (void)lds_wait_ge(P, C.ctl + TD_CTL_TREADY, ++tiles_seen, C.ok);
    const int nv = min(TD_TILE, T.t1 - (T.t0 + tile * TD_TILE));
    attn_tile_part<D>(qs, kt, vt, ps, nv, W, s, m, l, acc);
    lds_fence();
    if (lane == 0) lds_add(C.ctl + TD_CTL_TDONE, 1u);
    if (P.trace && !first) first = wall_clock64();
  }
  acc = attn_finish<D>(acc);
  constexpr int st = D + 4;
  if (W > 1) {
    float* sub = (float*)(base + A.sub) + (size_t)h * (W - 1) * st;
    if (s > 0) {  // this wave's state for the head's first wave
      attn_sub_store<D>(sub + (s - 1) * st, acc, m, l);
      lds_fence();
      if (lane == 0) lds_add(C.ctl + TD_CTL_SUB + h, 1u);
      return;
    }
    (void)lds_wait_ge(P, C.ctl + TD_CTL_SUB + h, (uint32_t)(W - 1) * nattn, C.ok);
    attn_combine<D>(acc, m, l, sub, W);
  }
  uint2* myparts = P.tpart + ((size_t)T.g * G + h) * P.n_chunks_max * st;
  if (T.c > 0) {
    uint2* dst = myparts + (size_t)T.c * st;
    if (lane < D / 4) {
      st_tag(dst + 4 * lane + 0, acc.x, tag);
      st_tag(dst + 4 * lane + 1, acc.y, tag);
      st_tag(dst + 4 * lane + 2, acc.z, tag);
      st_tag(dst + 4 * lane + 3, acc.w, tag);
    }
    if (lane == 0) {
      st_tag(dst + D, m, tag);
      st_tag(dst + D + 1, l, tag);
      st_tag(dst + D + 2, 0.f, tag);
      st_tag(dst + D + 3, 0.f, tag);
    }
    return;
  }
  const int n = T.n_used;  // <= 64
  float* mb = (float*)(base + A.merge) + (size_t)h * (P.n_chunks_max - 1) * st;  // chunks 1..n-1
  // the merging CUs (one per kv head) poll without topping up: every CU's
  // O stage waits for their outputs.  Where the staging runs on into the K/V
  // tile buffer, it waits until every query-head wave is done with the tiles.
  if (P.merge_in_tile) (void)lds_wait_ge(P, C.ctl + TD_CTL_TDONE, (uint32_t)(G * W) * tiles_seen, C.ok);
  // (d = 128: 9 loads per lane, so that the nine chunks of a 576-position
  // context are polled in one round; measured faster than 8 or 12)
  if (n > 1) C.ok &= poll_pairs<D == 128 ? 9 : 8, false>(P, myparts + st, 0, (n - 1) * st, tag, mb, C);
  lds_fence();
  const f32x4 o = attn_merge<D>(acc, m, l, mb, n, ps);
  if (lane < D / 4) {
    uint2* dst = P.to + ((size_t)T.g * G + h) * D + 4 * lane;
    st_tag(dst + 0, o.x, tag);
    st_tag(dst + 1, o.y, tag);
    st_tag(dst + 2, o.z, tag);
    st_tag(dst + 3, o.w, tag);
  }
}

DEV void trace_rec(const td_kparams& P, int wave, int seq, uint64_t t0, uint64_t t1, uint64_t t2, uint64_t t3) {
  uint64_t* rec = P.trace + ((size_t)blockIdx.x * P.n_stages + seq) * TD_TRACE_STAMPS + 4 * wave;
  const int lane = lane_id();
  const uint64_t v = lane == 0 ? t0 : lane == 1 ? t1 : lane == 2 ? t2 : t3;
  if (lane < 4) rec[lane] = v;
}

// The wave's stream from its first chunk (ring slots and their order carry on).
template <class CS>
DEV void stream_start(const td_kparams& P, CS& C) {
  C.fbase = C.fbase0;
  C.sbase = C.sbase0;
  C.issued = C.t = C.lk = 0;
  if constexpr (CS::kMoe) {  // the first layer's fixed run; routing comes with each layer
    C.run_end = C.m_fixed;
    C.rl = C.rp = 0;
    C.route_layer = -1;
  }
}

// Spins until the LDS word *p reaches `target`, topping the weight ring up
// meanwhile (the next step's first chunks stream while its token is decided).
// The word is read as a wave-uniform value: the loop must not look divergent
// to the compiler, or the ring state it updates would leave scalar registers.
template <class CS>
DEV uint32_t lds_wait_ge_topup(const td_kparams& P, CS& C, const uint32_t* p, uint32_t target) {
  uint32_t v = (uint32_t)uni((int)lds_ld(p));
  if (v < target) {
    const uint64_t t0 = wall_clock64();
    for (uint32_t it = 1;; ++it) {
      topup(P, C);
      __builtin_amdgcn_s_sleep(1);
      v = (uint32_t)uni((int)lds_ld(p));
      if (v >= target) break;
      if ((it & 1023u) == 0u && uni(wait_expired(P, t0) ? 1 : 0)) {
        C.ok = false;
        v = 0;
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
  return v;
}

template <int D, int WF, bool MOE>
DEV void compute_wave(const td_kparams& P, uint8_t* lds, int wave) {
  const int lane = lane_id();
  const int cu = blockIdx.x, ncu = gridDim.x;
  CStateT<MOE> C;
  C.lds = lds;
  C.ctl = (uint32_t*)(lds + P.off_ctl);
  C.xin = (float*)(lds + P.off_xin);
  C.own = (float*)(lds + P.off_own);
  C.out = (float*)(lds + P.off_out);
  C.ring = lds + P.off_ring + wave * P.ring_slots * TD_CHUNK;
  C.sring = lds + P.off_sring + wave * P.ring_slots * TD_SCHUNK;
  {
    const td_wstream W = P.ws[cu * TD_NW + wave];
    C.fbase0 = P.wcode + (size_t)W.code_off * TD_CHUNK;
    C.sbase0 = P.wscale + (size_t)W.scale_off * TD_SCHUNK;
    C.n_tot = W.n_tot;
    C.n4 = WF == TD_WF_BF16 ? 0u : W.n4;  // a constant 0 for bf16 models
  }
  {
    C.ranges = 0;
    if (lane < 2 * TD_NSPACES) {
      const int32_t* t = P.part + (size_t)(lane >> 1) * (ncu + 1) + cu;
      C.ranges = (lane & 1) ? t[1] - t[0] : t[0];
    }
  }
  C.ids_v = 0;
  C.wts_v = 0.f;
  C.inv_mlp = 1.f;
  if constexpr (MOE) {  // the runs of a MoE step (bf16 rows of K elements take ceil(2 K / 1 KiB) chunks)
    auto chunks = [](int K) { return (uint32_t)((2 * K + TD_CHUNK - 1) / TD_CHUNK); };
    const uint32_t nqkv = wave_units(C.unit_n(TD_SP_QKV), wave), nh = wave_units(C.unit_n(TD_SP_H), wave);
    const uint32_t nr = wave_units(C.unit_n(TD_SP_E), wave), ng = wave_units(C.unit_n(TD_SP_EI), wave);
    const uint32_t nv = wave_units(C.unit_n(TD_SP_V), wave);
    C.m_fixed = nqkv * 2 * chunks(P.H) + nh * chunks(P.qd) + nr * chunks(P.H);
    C.m_gu = ng * 2 * chunks(P.H);
    C.m_down = nh * chunks(P.I);
    C.m_head = nv * chunks(P.H);
    C.m_stride = C.m_fixed + (uint32_t)P.E * (C.m_gu + C.m_down);
    C.m_slot = C.unit_n(TD_SP_EI) > 0 ? (uint32_t)(C.unit_lo(TD_SP_EI) / P.I) : 0u;
    C.n_tot = (uint32_t)P.L * (C.m_fixed + C.m_gu + (uint32_t)P.topk * C.m_down) + C.m_head;  // consumed per step
  }
  stream_start(P, C);
  C.islot = C.slot = 0;
  C.nrv = 0;
  C.ok = true;
  topup(P, C);  // the stream starts right away
  const uint32_t epoch = uni(ld_u(P.sync + TD_SY_EPOCH));
  if (ld_u(P.sync + TD_SY_ABORT)) C.ok = false;
  int tok = uni(*P.token_in);
  if (tok < 0 || tok >= P.V) tok = 0;  // the sync wave reports the range error
  uint32_t tiles_seen = 0, nattn = 0;
  const int attn_waves = P.group * (MOE ? td_attn_waves(D, P.group, true) : 1);  // waves taking part in attention
  bool first_stage = true;
  for (int step = 0;; ++step) {
    const int pos = P.pos + step;
    const uint32_t tag0 = (epoch + (uint32_t)step) * (uint32_t)P.n_stages;  // stage seq publishes tag0 + seq + 1
    const uint16_t* erow = P.embed + (size_t)tok * P.H;
    {  // this wave's residual rows start as the embedding row; wave 0 stages the RoPE row of pos
      const int r0 = C.unit_lo(TD_SP_H), r1 = r0 + C.unit_n(TD_SP_H);
      for (int r = r0 + wave + lane * TD_NW; r < r1; r += 64 * TD_NW) C.own[r - r0] = bf16f(erow[r]);
      if (wave == 0) {
        float* cs = (float*)(lds + P.off_rope);
        for (int i = lane; i < P.d; i += 64) cs[i] = P.rope_cs[(size_t)pos * P.d + i];
      }
    }
    const AttnTask T = attn_task(P, cu, pos);
    for (int seq = 0; seq < P.n_stages; ++seq) {
      int kind, layer;
      stage_of<MOE>(P, seq, kind, layer);
      if (kind == TD_ST_ATTN && !T.valid) continue;
      const uint32_t tag_in = tag0 + (uint32_t)seq, tag = tag_in + 1u;
      uint64_t ts0 = 0, ts1 = 0, ts2 = 0;
      if (P.trace) ts0 = wall_clock64();
      // operands fetched ahead of the rendezvous: this slice's gains, this wave's QKV biases
      const uint16_t* gain = kind == TD_ST_QKV ? P.gains + (size_t)(2 * layer) * P.H
                           : (kind == TD_ST_GU && !MOE) || kind == TD_ST_ROUTER ? P.gains + (size_t)(2 * layer + 1) * P.H
                           : kind == TD_ST_HEAD ? P.gains + (size_t)(2 * P.L) * P.H : nullptr;
      uint32_t g0 = 0u, g1 = 0u, g2 = 0u, g3 = 0u;
      if (gain) {
        int lo, hi;
        td_slice(P.H, wave, &lo, &hi);
        const int u = (lo >> 1) + lane;
        if (u < (hi >> 1)) g0 = ld4_untracked(gain + 2 * u);
        if (u + 64 < (hi >> 1)) g1 = ld4_untracked(gain + 2 * (u + 64));
        if (u + 128 < (hi >> 1)) g2 = ld4_untracked(gain + 2 * (u + 128));
        if (u + 192 < (hi >> 1)) g3 = ld4_untracked(gain + 2 * (u + 192));
      }
      uint32_t bias_a = 0u, bias_b = 0u;  // bf16 bits
      if (kind == TD_ST_QKV && P.has_bias) {
        const int u0 = C.unit_lo(TD_SP_QKV);
        if (lane < wave_units(C.unit_n(TD_SP_QKV), wave)) {
          const uint16_t* bl = P.biases + (size_t)layer * P.qkv_rows;
          const int ra = unit_row(P, TD_ST_QKV, u0 + wave + lane * TD_NW, 0);
          bias_a = ld2_untracked(bl + ra);
          bias_b = ld2_untracked(bl + ra + (P.d >> 1));
        }
      }
      if (!first_stage) rendezvous(P, C);  // every wave is done reading the previous stage's inputs
      first_stage = false;
      if (kind == TD_ST_ATTN) {
        // the kv head's block: its query heads (scaled by 1/sqrt(d)), then this position's K and V rows
        const td_attn_lds A = td_attn_layout(P.d, P.group, P.n_chunks_max, MOE);
        float* qs = (float*)(lds + P.off_attn + A.q);
        const int nqv = P.group * P.d, nb = nqv + 2 * P.d;
        int lo, hi;
        td_slice(nb, wave, &lo, &hi);
        // (dense models: no top-up, so that the CU's tile copies and partial
        // stores queue behind none of its weight loads; measured 0.7-1.4 %
        // faster on the dense workloads and 1.8 % slower on the OLMoE shape)
        C.ok &= poll_pairs<8, !MOE>(P, P.tq + (size_t)T.g * nb, lo, hi, tag_in, qs, C);
        lds_fence();
        for (int i = lo + lane; i < min(hi, nqv); i += 64) qs[i] *= P.attn_scale;
        rendezvous(P, C);
        if (P.trace) ts1 = wall_clock64();
        if constexpr (MOE) {
          if (wave < attn_waves) attn_wave_split<D>(P, C, lds, wave, T, tag, tiles_seen, nattn, ts2);
        } else {
          if (wave < P.group) attn_wave_d<D>(P, C, lds, wave, T, tag, tiles_seen, ts2);
        }
      } else if (MOE && kind == TD_ST_GU) {
        // MoE gate/up: the router logits (all E, from every CU) next to the
        // input the router stage staged, the wave's routing, then its slot's
        // expert rows, which can stream from here on
        float* zs = (float*)(lds + P.off_route);
        int lo, hi;
        td_slice((P.E + 1) & ~1, wave, &lo, &hi);
        C.ok &= poll_pairs<8>(P, P.trl, lo, hi, tag_in, zs, C);
        rendezvous(P, C);
        if (P.trace) ts1 = wall_clock64();
        moe_route(P, C, lds, wave, layer);
        topup(P, C);
        gemv_wave<WF>(P, C, wave, kind, layer, pos, tag, C.inv_mlp, 0.f, 0.f, ts2);
      } else {
        const int K = kind == TD_ST_O ? P.qd : kind == TD_ST_DOWN ? (MOE ? P.topk * P.I : P.I) : P.H;
        const uint2* src = kind == TD_ST_O ? P.to : kind == TD_ST_DOWN ? P.tact
                         : kind == TD_ST_GU || kind == TD_ST_ROUTER ? P.tx_mid : P.tx_out;
        stage_gemv_input(P, C, wave, kind, K, src, kind == TD_ST_QKV && layer == 0 ? erow : nullptr, tag_in, g0, g1,
                         g2, g3, gain);
        reg_fence(bias_a);  // landed: loaded ahead of the input poll, whose wait covers them
        reg_fence(bias_b);
        rendezvous(P, C);
        if (P.trace) ts1 = wall_clock64();
        float inv = 1.0f;
        if (gain) {  // norm_inv over the slices' sums of squares, in slice order
          u32x4 a, b;
          asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
                       : "=v"(a), "=v"(b)
                       : "v"(lds_addr(C.ctl + TD_CTL_SSQ))
                       : "memory");
          float ss = __uint_as_float(a.x);
          ss += __uint_as_float(a.y);
          ss += __uint_as_float(a.z);
          ss += __uint_as_float(a.w);
          ss += __uint_as_float(b.x);
          ss += __uint_as_float(b.y);
          ss += __uint_as_float(b.z);
          ss += __uint_as_float(b.w);
          inv = 1.0f / sqrtf(ss / (float)P.H + P.eps);
        }
        if (kind == TD_ST_ROUTER) C.inv_mlp = inv;  // the MoE gate/up stage reuses the staged input
        gemv_wave<WF>(P, C, wave, kind, layer, pos, tag, inv, bf16f((uint16_t)bias_a), bf16f((uint16_t)bias_b), ts2);
      }
      if (P.trace) trace_rec(P, wave, seq, ts0, ts1, ts2, wall_clock64());
    }
    // the step's stream is consumed (every chunk issued has been read): the
    // next step's starts over and streams while the sync wave decides the
    // token (and whether another step follows)
    if (step + 1 < P.n_steps) stream_start(P, C);
    (void)lds_wait_ge_topup(P, C, C.ctl + TD_CTL_TOKREADY, (uint32_t)step + 1u);
    if (!C.ok || uni((int)lds_ld(C.ctl + TD_CTL_STOP))) break;
    tok = (int)uni((int)lds_ld(C.ctl + TD_CTL_TOKEN));
  }
  vm_drain();
  if (!C.ok && lane == 0) atomicOr(P.err, TD_ERRBIT_TIMEOUT);
}

// ------------------------------------------------------------ sync wave
// Rendezvous count of the compute waves once they have staged the inputs of
// the k-th stage of a step they take part in (k from 0), where `base` counts
// the rendezvous of the earlier steps: one per stage for the staged inputs and
// one before staging, except before the launch's very first stage.
DEV uint32_t staged_target(uint32_t base, int k) { return (uint32_t)TD_NW * (base + (uint32_t)(2 * k + 1)); }

// Waits until the pairs [0, n) of src (n even) all carry `tag` and copies their
// values to dst[0, n) (LDS); the sync wave's form of the input poll (it has no
// weight ring to top up).  false: the wait timed out (or another wait did).
DEV bool poll_pairs_plain(const td_kparams& P, const uint2* src, int n, uint32_t tag, float* dst) {
  const int lane = lane_id();
  const int nu = n >> 1;
  const __amdgpu_buffer_rsrc_t R = rsrc(src, (uint32_t)nu * 16u);
  const uint64_t t0 = wall_clock64();
  for (int b0 = 0; b0 < nu; b0 += 8 * 64) {
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (b0 + k * 64 + lane < nu) pend |= 1u << k;
    for (uint32_t it = 0;; ++it) {
      u32x4 r[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        r[k] = __builtin_amdgcn_raw_buffer_load_b128(R, (uint32_t)(b0 + k * 64 + lane) * 16u, 0, TD_CPOL_SC1);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (((pend >> k) & 1u) && r[k].y == tag && r[k].w == tag) {
          const int u = b0 + k * 64 + lane;
          dst[2 * u] = __uint_as_float(r[k].x);
          dst[2 * u + 1] = __uint_as_float(r[k].z);
          pend &= ~(1u << k);
        }
      }
      if (!__any(pend != 0u)) break;
      if ((it & 3u) == 3u && uni(wait_expired(P, t0) ? 1 : 0)) return false;
    }
  }
  return true;
}

DEV void cand_max(float& bv, int& bi) { cand_wave_max(bv, bi); }

template <bool MOE>
DEV void sync_wave(const td_kparams& P, uint8_t* lds) {
  constexpr int SPL = MOE ? 6 : 5;  // stages per layer
  const int lane = lane_id();
  const int cu = blockIdx.x, ncu = gridDim.x;
  uint32_t* ctl = (uint32_t*)(lds + P.off_ctl);
  bool ok = true;
  const uint32_t epoch = uni(ld_u(P.sync + TD_SY_EPOCH));
  {
    const int tok = uni(*P.token_in);
    if ((tok < 0 || tok >= P.V) && lane == 0 && cu == 0) atomicOr(P.err, TD_ERRBIT_RANGE);
  }
  const int G = P.group * (MOE ? td_attn_waves(P.d, P.group, true) : 1);  // the attention waves, each consuming every tile
  uint32_t tiles_ready = 0, tiles_issued = 0, rv_base = 0;
  if (P.step_clock && cu == 0 && lane == 0) P.step_clock[0] = wall_clock64();
  for (int step = 0;; ++step) {
    const int pos = P.pos + step;
    const AttnTask T = attn_task(P, cu, pos);
    // a tile's buffer is free once the tile tile_bufs places earlier is
    // consumed; tiles [tiles_ready, tiles_issued) have their copies in flight
    const uint32_t nb = (uint32_t)P.tile_bufs;
    auto buf_free = [&](uint32_t k) { return (uint32_t)G * (k + 1u > nb ? k + 1u - nb : 0u); };
    const bool dma = nb >= 3 && P.d == 64;  // (the waits below count 17 copies a tile)
    auto issue = [&](int layer, int tile) {
      (void)lds_wait_ge(P, ctl + TD_CTL_TDONE, buf_free(tiles_issued), ok);
      if (dma) issue_tile(P, tile_buf(P, lds, tiles_issued), layer, T, tile);
      else load_tile(P, tile_buf(P, lds, tiles_issued), layer, T, tile, pos);  // (in LDS on return)
      ++tiles_issued;
    };
    // the oldest tile in flight: landed (only the copies issued after it may
    // be outstanding), its position row replaced, published to the compute waves
    auto ready = [&](int tile) {
      if (dma) {  // three buffers (d = 64, 17 copies a tile): at most two later tiles in flight
        const uint32_t later = tiles_issued - tiles_ready - 1u;
        if (later >= 2u) vmcnt_wait<34>();
        else if (later == 1u) vmcnt_wait<17>();
        else vmcnt_wait<0>();
      }
      patch_pos_row(P, lds, tile_buf(P, lds, tiles_ready), T, tile, pos);
      lds_fence();
      lds_st(ctl + TD_CTL_TREADY, ++tiles_ready);
    };
    // A layer's first tiles (as many as there are buffers) are issued ahead:
    // rows before pos are final, and row pos is patched when the tile is made
    // ready.  Within the layer a tile is issued once tile r, the next to be
    // made ready, needs it (one buffer) or while it is fewer than nb - 1 tiles
    // ahead of r: its buffer's previous tile, two behind r, is consumed by then
    // or soon, and the compute waves already hold tile r - 1.  (One issue site
    // per phase keeps the loaders' code from being inlined more often.)
    for (int layer = -1; T.valid && layer < P.L; ++layer) {
      if (layer >= 0) {
        // ATTN of this layer is the (spl layer + 1)-th stage the compute waves take part in
        (void)lds_wait_ge(P, ctl + TD_CTL_RV, staged_target(rv_base, SPL * layer + 1), ok);
        int next = min(T.ntiles, (int)nb), r = 0;
        while (r < T.ntiles) {
          if (next < T.ntiles && (next <= r || next < r + (int)nb - 1)) issue(layer, next++);
          else ready(r++);
        }
      }
      if (layer + 1 < P.L) {
        // the next layer's first tiles once the stage after O (GU, or the
        // router of a MoE layer), whose input poll is on the critical path, has
        // its inputs (every tile of this layer is consumed by then)
        if (layer >= 0) (void)lds_wait_ge(P, ctl + TD_CTL_RV, staged_target(rv_base, SPL * layer + 3), ok);
        for (int tile = 0; tile < T.ntiles && tile < (int)nb; ++tile) issue(layer + 1, tile);
      }
    }
    // every tile consumed: the tile area takes the candidates below
    (void)lds_wait_ge(P, ctl + TD_CTL_TDONE, (uint32_t)G * tiles_ready, ok);
    rv_base += 2u * (uint32_t)(P.n_stages - (T.valid ? 0 : P.L));
    // HEAD: the compute waves' candidates -> this CU's candidate, published;
    // then every CU reads all CUs' candidates and takes the same token
    (void)lds_wait_ge(P, ctl + TD_CTL_HEADDONE, (uint32_t)TD_NW * (uint32_t)(step + 1), ok);
    float bv = -__builtin_inff();
    int bi = 0x7fffffff, bad = 0;
    if (lane < TD_NW) {
      bv = __uint_as_float(ctl[TD_CTL_CAND + 4 * lane]);
      bi = (int)ctl[TD_CTL_CAND + 4 * lane + 1];
      bad = (int)ctl[TD_CTL_CAND + 4 * lane + 2];
    }
    cand_max(bv, bi);
    bad = __any(bad);
    const uint32_t tag = (epoch + (uint32_t)step) * (uint32_t)P.n_stages + (uint32_t)P.n_stages;
    if (lane == 0) {
      uint2* mine = P.cand + (size_t)cu * 4;
      st_tag(mine + 0, __uint_as_float(__float_as_uint(bv)), tag);
      st_tag(mine + 1, __uint_as_float((uint32_t)bi), tag);
      st_tag(mine + 2, __uint_as_float((uint32_t)bad), tag);
      st_tag(mine + 3, 0.f, tag);
    }
    float* cands = (float*)(lds + P.off_tile);  // the tiles are consumed
    ok &= poll_pairs_plain(P, P.cand, 4 * ncu, tag, cands);
    lds_fence();
    float fv = -__builtin_inff();
    int fi = 0x7fffffff, fbad = 0;
    for (int c = lane; c < ncu; c += 64) {
      const float v = cands[4 * c];
      const int i = (int)__float_as_uint(cands[4 * c + 1]);
      fbad |= (int)__float_as_uint(cands[4 * c + 2]);
      if (cand_better(v, i, fv, fi)) { fv = v; fi = i; }
    }
    cand_max(fv, fi);
    fbad = __any(fbad);
    const int token = uni(fi == 0x7fffffff ? 0 : fi);
    const bool stop = !ok || fbad || token == P.eos || step + 1 >= P.n_steps;
    if (cu == 0 && lane == 0) {
      *P.token_out = token;
      if (P.tokens_out) P.tokens_out[step] = token;
      if (fbad) atomicOr(P.err, TD_ERRBIT_NONFINITE);
    }
    lds_st(ctl + TD_CTL_TOKEN, (uint32_t)token);
    lds_st(ctl + TD_CTL_STOP, stop ? 1u : 0u);
    lds_fence();
    lds_st(ctl + TD_CTL_TOKREADY, (uint32_t)step + 1u);
    if (P.step_clock && cu == 0 && lane == 0 && step + 1 < P.step_clock_n) P.step_clock[step + 1] = wall_clock64();
    if (stop) {
      // every CU has read the epoch: all candidates of this step carry its tag
      if (cu == 0 && lane == 0) {
        if (P.count_out) *P.count_out = step + 1;
        st_u(P.sync + TD_SY_EPOCH, epoch + (uint32_t)step + 1u);
      }
      if (cu == 0 && P.tokens_out)
        for (int s = step + 1 + lane; s < P.n_steps; s += 64) P.tokens_out[s] = -1;
      break;
    }
  }
  if (!ok && lane == 0) atomicOr(P.err, TD_ERRBIT_TIMEOUT);
}

// ------------------------------------------------------------ the kernel
// D: the head dimension (64 or 128), a template parameter so that only one
// attention tile routine is compiled into each kernel; WF: the format of the
// layer linears (TD_WF_*), so that each chunk loop is compiled for one format.
template <int D, int WF, bool MOE>
__global__ void __launch_bounds__(TD_THREADS, 1) td_megakernel(td_kparams P) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  uint32_t* ctl = (uint32_t*)(lds + P.off_ctl);
  if (threadIdx.x < TD_CTL_WORDS) ctl[threadIdx.x] = 0u;
  // MoE: the router logits area is padded with -inf past E (the choice reads it in fours)
  if (MOE && threadIdx.x < TD_MAX_EXPERTS) ((float*)(lds + P.off_route))[threadIdx.x] = -__builtin_inff();
  __syncthreads();  // the only workgroup barrier: the control block is clear
  const int wave = uni((int)(threadIdx.x >> 6));
  if (wave < TD_NW) compute_wave<D, WF, MOE>(P, lds, wave);
  else sync_wave<MOE>(P, lds);
}

// ------------------------------------------------------------ weight packing
// One wave per (CU, compute wave): walks the same cursor as the plan and copies
// each chunk of its stream from the caller's row-major weights (zero-padding
// the tail of a row that is not a whole chunk: bf16 0, or the 4-bit code of 0),
// plus, for int4 chunks, the chunk's 32 fp16 scales.  A stream whose length
// disagrees with the host plan raises bit 0 of *bad and is cut short.
__global__ void __launch_bounds__(256) td_repack_kernel(td_kparams P, int ncu, uint8_t* code, uint8_t* scale,
                                                        const td_wstream* ws, int* bad) {
  const int gw = uni((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (gw >= ncu * TD_NW) return;
  const int cu = gw / TD_NW, wave = gw - cu * TD_NW;
  const int lane = lane_id();
  const td_wstream W = ws[gw];
  uint8_t* dst = code + (size_t)W.code_off * TD_CHUNK;
  uint8_t* sdst = scale + (size_t)W.scale_off * TD_SCHUNK;
  Cursor c;
  cur_enter(c, P, wave, cu, ncu, 0);
  uint32_t n = 0, n4 = 0;
  while (c.seq < P.n_stages && n < W.n_tot) {
    const int u = c.u_first + c.k * TD_NW;
    const int row = unit_row(P, c.g.kind, u, c.r);
    const uint8_t* rp = c.g.w + (size_t)c.e * c.g.estride + (size_t)row * c.g.row_bytes;
    u32x4 v;
    if (c.g.fmt == 0) {
      const int boff = c.j * TD_CHUNK + lane * 16;
      v = boff < c.g.row_bytes ? *(const u32x4*)(rp + boff) : (u32x4){0u, 0u, 0u, 0u};
    } else {  // the lane's four words, from their places in the row (zero weights past its end)
      v = int4_words(rp, c.g.row_bytes, c.j, lane);
    }
    *(u32x4*)(dst + lane * 16) = v;
    dst += TD_CHUNK;
    if (c.g.fmt == 1) {
      if (n4 >= W.n4) break;
      if (lane < 32)
        *(uint16_t*)(sdst + lane * 2) = int4_block_scale(c.g.s + (size_t)row * (c.g.K / 64), c.g.K / 64, c.j, lane);
      sdst += TD_SCHUNK;
      ++n4;
    }
    cur_next(c, P, wave, cu, ncu);
    ++n;
  }
  if (lane == 0 && (c.seq < P.n_stages || n != W.n_tot || n4 != W.n4)) atomicOr(bad, 1);
}

// ------------------------------------------------------------ stream-read yardstick
// Reads `bytes` (a multiple of 16) once with 16-byte non-temporal loads, four
// in flight per lane, over a grid of one workgroup of 512 threads per CU: the
// HBM read rate the weight stream can hope for on this part ("Decoding in
// tiles", sec. 2: the measured streaming rate, not the nominal one, is the
// floor's denominator).  Each lane folds its loaded words into one value that
// an empty asm statement consumes, so no load is dead.
__global__ void __launch_bounds__(512) td_stream_read_kernel(const u32x4* p, int64_t n16) {
  // a workgroup reads 32 KiB contiguous per pass (four 16-byte loads per lane in
  // flight), the passes strided over the grid; the best of the layouts, grid
  // sizes and cache policies measured on MI355X (1 workgroup per CU, non-temporal)
  constexpr int U = 4;
  const int64_t blk = (int64_t)U * 512;
  const int64_t gstride = (int64_t)gridDim.x * blk;
  uint32_t acc = 0;
  int64_t b = (int64_t)blockIdx.x * blk;
  for (; b + blk <= n16; b += gstride) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(p + b + k * 512 + threadIdx.x);
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (b < n16)  // the ragged last block
    for (int64_t i = b + threadIdx.x; i < n16; i += 512) {
      const u32x4 a = __builtin_nontemporal_load(p + i);
      acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
  asm volatile("" ::"v"(acc));  // every lane's folded value is kept, so none of its loads is dead
}

// ------------------------------------------------------------ test hooks
// y = W x through the packed-stream layout and the step's chunk arithmetic:
// x is staged into LDS zero-padded to whole chunks (as the step stages its
// input), and each chunk of a row is first packed into an LDS chunk buffer by
// the routines that build the packed streams (a lane's 16 bytes: its four
// int4 words or its 8 bf16 weights, zero weights past the row's end; an int4
// chunk's 64-byte scale block) and then consumed as the step consumes a ring
// slot.  One wave per row, 4 rows per workgroup.
__global__ void __launch_bounds__(256) td_gemv_kernel(int fmt, const uint8_t* w, const uint16_t* s, int rows,
                                                      int cols, int kpad, const float* x, float* y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* xs = (float*)lds;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  uint8_t* cbuf = lds + (size_t)kpad * 4 + wave * (TD_CHUNK + TD_SCHUNK);
  uint8_t* sbuf = cbuf + TD_CHUNK;
  for (int i = threadIdx.x; i < kpad; i += 256) xs[i] = i < cols ? x[i] : 0.f;
  __syncthreads();
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const int row_bytes = fmt == 0 ? cols * 2 : cols / 2;
  const int J = (row_bytes + TD_CHUNK - 1) / TD_CHUNK;
  const uint8_t* rp = w + (size_t)row * row_bytes;
  float acc = 0.f;
  for (int j = 0; j < J; ++j) {
    u32x4 v;
    if (fmt == 0) {
      const int boff = j * TD_CHUNK + lane * 16;
      v = boff < row_bytes ? *(const u32x4*)(rp + boff) : (u32x4){0u, 0u, 0u, 0u};
    } else {
      v = int4_words(rp, row_bytes, j, lane);
      if (lane < 32)
        *(uint16_t*)(sbuf + lane * 2) = int4_block_scale(s + (size_t)row * (cols / 64), cols / 64, j, lane);
    }
    *(u32x4*)(cbuf + lane * 16) = v;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const u32x4 wv = *(const u32x4*)(cbuf + lane * 16);
    if (fmt == 0) acc += dot_bf16(wv, xs + j * 512 + lane * 8);
    else acc += dot_int4(wv, xs + j * 2048, lane, int4_lane_scales(sbuf, lane));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  const float r = wave_sum(acc);
  if (lane == 0) y[row] = r;
}

// One query head over n bf16 K/V rows with the decode kernel's own attention
// routines: the positions cut into chunks of chunk_len (a multiple of the
// 64-row tile), each chunk's tiles staged into LDS in the kernel's tile layout
// (K rows padded to D + 8, rows past the chunk's end zero) and taken by
// attn_tile, the chunk's state finished by attn_finish, and the chunks merged
// by attn_merge, chunk 0 holding its own state as on the merging CU.  q is
// scaled by 1/sqrt(d) in fp32 first, as the kernel scales its staged queries.
// One wave; LDS: q [D], p [64], the tile, the partials of chunks 1 .. n-1.
template <int D>
__global__ void __launch_bounds__(64) td_attention_kernel(const float* q, const uint16_t* k, const uint16_t* v,
                                                          int n, int chunk_len, int W, float scale, float* out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int st = D + 4;
  float* qs = (float*)lds;
  float* ps = qs + D;
  uint16_t* kt = (uint16_t*)(ps + TD_TILE);
  uint16_t* vt = kt + TD_TILE * (D + 8);
  float* sub = (float*)(vt + TD_TILE * D);  // the states of waves 1 .. W - 1 of the head
  float* mb = sub + 7 * st;
  const int lane = lane_id();
  for (int i = lane; i < D; i += 64) qs[i] = q[i] * scale;
  const int nch = (n + chunk_len - 1) / chunk_len;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f};
  float m0 = -__builtin_inff(), l0 = 0.f;
  for (int c = 0; c < nch; ++c) {
    const int t0 = c * chunk_len, t1 = min(t0 + chunk_len, n);
    float m[8], l[8];
    f32x4 acc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      m[s] = -__builtin_inff();
      l[s] = 0.f;
      acc[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    for (int tb = t0; tb < t1; tb += TD_TILE) {
      const int nv = min(TD_TILE, t1 - tb);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      for (int i = lane; i < TD_TILE * (D / 8); i += 64) {
        const int row = i / (D / 8), pc = i - row * (D / 8);
        u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (row < nv) {
          kv = *(const u32x4*)(k + (size_t)(tb + row) * D + pc * 8);
          vv = *(const u32x4*)(v + (size_t)(tb + row) * D + pc * 8);
        }
        *(u32x4*)(kt + row * (D + 8) + pc * 8) = kv;
        *(u32x4*)(vt + row * D + pc * 8) = vv;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int s = 0; s < 8; ++s)  // the head's W waves, one after another
        if (s < W) {
          attn_tile_part<D>(qs, kt, vt, ps, nv, W, s, m[s], l[s], acc[s]);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < W) {
        acc[s] = attn_finish<D>(acc[s]);
        if (s > 0) attn_sub_store<D>(sub + (s - 1) * st, acc[s], m[s], l[s]);
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (W > 1) attn_combine<D>(acc[0], m[0], l[0], sub, W);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (c == 0) {
      acc0 = acc[0];
      m0 = m[0];
      l0 = l[0];
    } else {
      attn_sub_store<D>(mb + (size_t)(c - 1) * st, acc[0], m[0], l[0]);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const f32x4 o = attn_merge<D>(acc0, m0, l0, mb, nch, ps);
  if (lane < D / 4) *(f32x4*)(out + 4 * lane) = o;
}

// Half-split RoPE of n_heads vectors of d values at one position, with the
// step's pair rotation and a table row built as the step's table is (cs: d/2
// (cos, sin) pairs).  Thread (head, i) rotates pair (i, i + d/2) of its head.
__global__ void __launch_bounds__(256) td_rope_kernel(const float* x, int n_heads, int d, td_rope_row row, float* y) {
  const int t = blockIdx.x * 256 + threadIdx.x, half = d / 2;
  if (t >= n_heads * half) return;
  const int h = t / half, i = t - h * half;
  float a = x[h * d + i], b = x[h * d + i + half];
  rope_pair(a, b, row.cs[2 * i], row.cs[2 * i + 1]);
  y[h * d + i] = a;
  y[h * d + i + half] = b;
}

// The greedy token of n logits in the step's three levels: every one of the
// `groups` workgroups (a CU's share of the vocabulary, split as the plan splits
// it) runs its 8 waves over its rows round robin, lane k of a wave over its
// rows k, k + 64, ...; each wave's candidate, then the workgroup's over its 8
// waves, go to cand; the last kernel takes the best of all workgroups'.  A
// non-finite logit is left out of the choice and raises the flag.
__global__ void __launch_bounds__(512) td_argmax_groups(const float* logits, int n, int groups, uint2* cand,
                                                        int* badw) {
  __shared__ float wv[TD_NW];
  __shared__ int wi[TD_NW], wb[TD_NW];
  const int g = blockIdx.x, wave = threadIdx.x >> 6, lane = lane_id();
  const int u0 = (int)((int64_t)n * g / groups), u1 = (int)((int64_t)n * (g + 1) / groups);
  float bv = -__builtin_inff();
  int bi = 0x7fffffff, bad = 0;
  for (int u = u0 + wave + lane * TD_NW; u < u1; u += 64 * TD_NW) {
    const float v = logits[u];
    if (!isfinite(v)) bad = 1;
    else if (cand_better(v, u, bv, bi)) { bv = v; bi = u; }
  }
  cand_wave_max(bv, bi);
  bad = __any(bad);
  if (lane == 0) {
    wv[wave] = bv;
    wi[wave] = bi;
    wb[wave] = bad;
  }
  __syncthreads();
  if (wave == 0) {
    float v = lane < TD_NW ? wv[lane] : -__builtin_inff();
    int i = lane < TD_NW ? wi[lane] : 0x7fffffff;
    const int b = __any(lane < TD_NW && wb[lane]);
    cand_wave_max(v, i);
    if (lane == 0) {
      cand[g] = make_uint2(__float_as_uint(v), (uint32_t)i);
      badw[g] = b;
    }
  }
}
__global__ void __launch_bounds__(64) td_argmax_final(const uint2* cand, const int* badw, int groups, int* token,
                                                      int* nonfinite) {
  const int lane = lane_id();
  float fv = -__builtin_inff();
  int fi = 0x7fffffff, fbad = 0;
  for (int c = lane; c < groups; c += 64) {
    const float v = __uint_as_float(cand[c].x);
    const int i = (int)cand[c].y;
    fbad |= badw[c];
    if (cand_better(v, i, fv, fi)) { fv = v; fi = i; }
  }
  cand_wave_max(fv, fi);
  fbad = __any(fbad);
  if (lane == 0) {
    *token = fi == 0x7fffffff ? 0 : fi;
    *nonfinite = fbad;
  }
}

}  // namespace

// ------------------------------------------------------------ launchers
namespace {
// MoE layers run on bf16 weights only (the plan refuses the others)
const void* megakernel_of(int d, int wf, bool moe) {
  if (moe) return d == 64 ? (const void*)td_megakernel<64, 0, true> : (const void*)td_megakernel<128, 0, true>;
  if (d == 64) return wf ? (const void*)td_megakernel<64, 1, false> : (const void*)td_megakernel<64, 0, false>;
  return wf ? (const void*)td_megakernel<128, 1, false> : (const void*)td_megakernel<128, 0, false>;
}
}  // namespace

int td_megakernel_occupancy(int d, int wf, int moe, int lds_bytes, int* blocks) {
  const void* f = megakernel_of(d, wf, moe != 0);
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, f, TD_THREADS, lds_bytes);
  return (int)e;
}

int td_launch_megakernel(const td_kparams* p, int ncu, void* stream) {
  void* args[] = {(void*)p};
  const void* f = megakernel_of(p->d, p->wf, p->E > 0);
  return (int)hipLaunchCooperativeKernel(f, dim3(ncu), dim3(TD_THREADS), args, (unsigned)p->lds_bytes,
                                         (hipStream_t)stream);
}

int td_launch_repack(const td_kparams* p, int ncu, uint8_t* code, uint8_t* scale, const td_wstream* ws, int* bad,
                     void* stream) {
  const int waves = ncu * TD_NW;
  td_repack_kernel<<<(waves + 3) / 4, 256, 0, (hipStream_t)stream>>>(*p, ncu, code, scale, ws, bad);
  return (int)hipGetLastError();
}

int td_launch_test_gemv(int fmt, const void* w, const void* s, int rows, int cols, const float* x, float* y,
                        void* stream) {
  const int ce = fmt ? 2048 : 512;
  const int kpad = (cols + ce - 1) / ce * ce;
  const size_t lds = (size_t)kpad * 4 + 4 * (TD_CHUNK + TD_SCHUNK);
  hipError_t e = hipFuncSetAttribute((const void*)td_gemv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return (int)e;
  td_gemv_kernel<<<(rows + 3) / 4, 256, lds, (hipStream_t)stream>>>(fmt, (const uint8_t*)w, (const uint16_t*)s, rows,
                                                                     cols, kpad, x, y);
  return (int)hipGetLastError();
}

int td_launch_stream_read(const void* buf, int64_t bytes, int ncu, void* stream) {
  td_stream_read_kernel<<<ncu, 512, 0, (hipStream_t)stream>>>((const u32x4*)buf, bytes / 16);
  return (int)hipGetLastError();
}

int td_launch_test_rope(const float* x, int n_heads, int d, const td_rope_row& row, float* y, void* stream) {
  const int n = n_heads * (d / 2);
  td_rope_kernel<<<(n + 255) / 256, 256, 0, (hipStream_t)stream>>>(x, n_heads, d, row, y);
  return (int)hipGetLastError();
}

int td_launch_test_argmax(const float* logits, int n, int groups, void* work, int* token, int* nonfinite,
                          void* stream) {
  uint2* cand = (uint2*)work;
  int* badw = (int*)(cand + groups);
  td_argmax_groups<<<groups, 512, 0, (hipStream_t)stream>>>(logits, n, groups, cand, badw);
  td_argmax_final<<<1, 64, 0, (hipStream_t)stream>>>(cand, badw, groups, token, nonfinite);
  return (int)hipGetLastError();
}

size_t td_test_attention_lds(int d, int chunk_len, int n) {
  const int nch = (n + chunk_len - 1) / chunk_len;
  return (size_t)(d + TD_TILE) * 4 + (size_t)TD_TILE * (d + 8) * 2 + (size_t)TD_TILE * d * 2 + (size_t)7 * (d + 4) * 4 +
         (size_t)(nch > 1 ? nch - 1 : 1) * (d + 4) * 4;
}

int td_launch_test_attention(const float* q, const void* k, const void* v, int n, int d, int chunk_len, int waves,
                             float scale, float* out, void* stream) {
  const size_t lds = td_test_attention_lds(d, chunk_len, n);
  const void* f = d == 64 ? (const void*)td_attention_kernel<64> : (const void*)td_attention_kernel<128>;
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return (int)e;
  if (d == 64)
    td_attention_kernel<64><<<1, 64, lds, (hipStream_t)stream>>>(q, (const uint16_t*)k, (const uint16_t*)v, n,
                                                                  chunk_len, waves, scale, out);
  else
    td_attention_kernel<128><<<1, 64, lds, (hipStream_t)stream>>>(q, (const uint16_t*)k, (const uint16_t*)v, n,
                                                                   chunk_len, waves, scale, out);
  return (int)hipGetLastError();
}
