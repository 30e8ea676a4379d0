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
// Workgroup roles:
//   8 compute waves stream weight chunks (1 KiB = 64 lanes x 16 B) from HBM
//     straight into a per-wave LDS ring with global_load_lds_dwordx4.  Each
//     wave's chunks are packed at create time in the order it consumes them,
//     and the ring runs S chunks ahead across stage boundaries: weights never
//     depend on the token, so the next stage's loads are in flight while the
//     CU waits for that stage's inputs.  These waves issue no other global
//     memory operation, so vmcnt counts only ring loads.
//   1 sync wave does all activation traffic: it stages a stage's inputs in
//     LDS (with the RMSNorm applied), runs the epilogues (bias, RoPE, K/V
//     write, SiLU*up, residual, merge, argmax) and publishes the outputs.
// Cross-CU hand-off without grid barriers: every value handed to other CUs is
// a (value, tag) pair written with one 8-byte agent-scope (sc1) store, and a
// reader polls the pairs with sc1 loads until all carry the tag of the stage
// that produced them.  The data is its own ready signal, coherent across the 8
// XCDs without writing back or invalidating whole L2 caches, and a stage waits
// only for the values it reads.  Every wait is bounded in time.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "td_internal.h"

#include "td_device.h"

namespace {

// ------------------------------------------------------------ the plan
// A GEMV stage splits its "units" evenly over the CUs (equal bytes per CU up
// to one unit) and round-robins a CU's units over its compute waves.  A unit
// is the set of rows one epilogue needs together: the two rows of a RoPE pair
// (i, i + d/2) of one head for QKV, the gate and up rows of one intermediate
// index for GU, one row otherwise.
struct Gemv {
  const uint8_t* w;
  const uint16_t* s;
  int K, row_bytes, J, U, rpu, kind, fmt;
};

DEV void stage_of(const td_kparams& P, int seq, int& kind, int& layer) {
  if (seq >= 5 * P.L) {
    kind = TD_ST_HEAD;
    layer = P.L;
  } else {
    layer = seq / 5;
    kind = seq - layer * 5;
  }
}

DEV Gemv gemv_of(const td_kparams& P, int kind, int layer) {
  Gemv g;
  g.kind = kind;
  g.s = nullptr;
  if (kind == TD_ST_HEAD) {
    g.w = (const uint8_t*)P.head;
    g.K = P.H;
    g.U = P.V;
    g.rpu = 1;
    g.fmt = 0;
  } else {
    const td_layer_dev& Ld = P.layers[layer];
    int idx = kind == TD_ST_QKV ? 0 : kind == TD_ST_O ? 1 : kind == TD_ST_GU ? 2 : 3;
    g.w = Ld.w[idx];
    g.s = Ld.s[idx];
    g.fmt = P.wf;
    if (kind == TD_ST_QKV) { g.K = P.H; g.U = P.qkv_rows / 2; g.rpu = 2; }
    else if (kind == TD_ST_O) { g.K = P.qd; g.U = P.H; g.rpu = 1; }
    else if (kind == TD_ST_GU) { g.K = P.H; g.U = P.I; g.rpu = 2; }
    else { g.K = P.I; g.U = P.H; g.rpu = 1; }
  }
  g.row_bytes = g.fmt == 0 ? g.K * 2 : g.K / 2;
  g.J = (g.row_bytes + TD_CHUNK - 1) / TD_CHUNK;
  return g;
}

DEV int unit_row(const td_kparams& P, int kind, int u, int r) {
  if (kind == TD_ST_QKV) {
    int half = P.d >> 1;
    int head = u / half;
    int i = u - head * half;
    return head * P.d + i + r * half;
  }
  if (kind == TD_ST_GU) return u + r * P.I;
  return u;
}

DEV void cu_units(int U, int cu, int ncu, int& u0, int& u1) {
  u0 = (int)(((int64_t)U * cu) / ncu);
  u1 = (int)(((int64_t)U * (cu + 1)) / ncu);
}

// position in one compute wave's chunk sequence over the whole step
struct Cursor {
  int seq;  // stage sequence number; == n_stages when done
  Gemv g;
  int u_first, n, k, r, j;
};

DEV void cur_enter(Cursor& c, const td_kparams& P, int wave, int cu, int ncu, int seq) {
  for (; seq < P.n_stages; ++seq) {
    int kind, layer;
    stage_of(P, seq, kind, layer);
    if (kind == TD_ST_ATTN) continue;
    Gemv g = gemv_of(P, kind, layer);
    int u0, u1;
    cu_units(g.U, cu, ncu, u0, u1);
    int cnt = u1 - u0;
    int n = cnt > wave ? (cnt - wave + TD_NW - 1) / TD_NW : 0;
    if (n == 0) continue;
    c.seq = seq;
    c.g = g;
    c.u_first = u0 + wave;
    c.n = n;
    c.k = c.r = c.j = 0;
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
  cur_enter(c, P, wave, cu, ncu, c.seq + 1);
}

// ------------------------------------------------------------ hand-off of activations
// A value handed to other CUs is a (value bits, tag) pair written with one
// 8-byte agent-scope store; readers poll the pairs with agent-scope loads until
// every one carries the tag they expect.  The data is its own ready signal, so
// a stage waits exactly for the values it reads (no grid-wide barrier), and a
// buffer is only rewritten after every reader of its previous contents has
// provably moved on (each stage reads the complete output of the one before).
#define TD_CPOL_SC1 16  // buffer-load cache policy: agent scope

DEV __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

DEV void st_tag(uint2* p, float v, uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(w) : "memory");
}

DEV bool wait_expired(const td_kparams& P, uint64_t t0) {
  if (ld_u(P.sync + TD_SY_ABORT)) return true;
  if (wall_clock64() - t0 > TD_SPIN_TICKS) {
    st_u(P.sync + TD_SY_ABORT, 1u);
    return true;
  }
  return false;
}

// Waits until the n pairs at src (n even) all carry `tag` and copies their
// values to dst (LDS).  Each round loads W 16-byte units per lane and re-polls
// the units still missing.  false: the wait timed out (or another wait did).
template <int W>
DEV bool poll_vec_w(const td_kparams& P, const uint2* src, int n, uint32_t tag, float* dst) {
  const int lane = lane_id();
  const int nu = n >> 1;  // 16-byte units of two pairs
  const __amdgpu_buffer_rsrc_t R = rsrc(src, (uint32_t)nu * 16u);
  const uint64_t t0 = wall_clock64();
  for (int b0 = 0; b0 < nu; b0 += W * 64) {
    uint32_t pend = 0;
#pragma unroll
    for (int k = 0; k < W; ++k)
      if (b0 + k * 64 + lane < nu) pend |= 1u << k;
    for (uint32_t it = 0;; ++it) {
      u32x4 r[W];
#pragma unroll
      for (int k = 0; k < W; ++k)
        r[k] = __builtin_amdgcn_raw_buffer_load_b128(R, (uint32_t)(b0 + k * 64 + lane) * 16u, 0, TD_CPOL_SC1);
#pragma unroll
      for (int k = 0; k < W; ++k) {
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

DEV bool poll_vec(const td_kparams& P, const uint2* src, int n, uint32_t tag, float* dst) {
  return poll_vec_w<16>(P, src, n, tag, dst);
}

// ------------------------------------------------------------ attention task
// Split-K decode attention: kv head g's positions 0..pos are cut into chunks of
// chunk_len; one CU per (g, chunk) computes a partial (m, l, acc) for the g's
// query heads; the CU of chunk 0 merges the partials ("One launch per token",
// "The attention trap").
struct AttnTask {
  int valid, g, c, t0, t1, ntiles, n_used;
};
DEV AttnTask attn_task(const td_kparams& P, int cu) {
  AttnTask t;
  t.n_used = (P.pos + P.chunk_len) / P.chunk_len;  // chunks covering positions 0..pos
  t.valid = cu < P.nkv * t.n_used;
  t.g = t.valid ? cu / t.n_used : 0;
  t.c = t.valid ? cu - t.g * t.n_used : 0;
  t.t0 = t.c * P.chunk_len;
  t.t1 = min(t.t0 + P.chunk_len, P.pos + 1);
  t.ntiles = t.valid ? (t.t1 - t.t0 + TD_TILE - 1) / TD_TILE : 0;
  return t;
}

// compute waves: wave h < group handles query head g * group + h, one 64-row
// tile at a time (attn_tile).  Rows past the chunk end are zero in the tile
// and get p = 0.  Returns the trace stamp taken after the first tile (0
// without a trace).
template <int D>
DEV uint64_t attn_compute_d(const td_kparams& P, uint8_t* lds, int wave, const AttnTask& T) {
  const int lane = lane_id();
  const td_attn_lds A = td_attn_layout(D, P.group, P.n_chunks_max);
  uint8_t* base = lds + P.off_attn;
  const bool active = wave < P.group;
  const float* qs = (const float*)(base + A.q) + (active ? wave : 0) * D;
  const uint16_t* kt = (const uint16_t*)(lds + P.off_tile);
  const uint16_t* vt = kt + TD_TILE * (D + 8);
  float* ps = (float*)(base + A.p) + (active ? wave : 0) * TD_TILE;
  const int ntiles = T.ntiles, t0 = T.t0, t1 = T.t1;
  uint64_t stamp = 0;
  float m = -__builtin_inff(), l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int tile = 0; tile < ntiles; ++tile) {
    wg_bar();  // tile in LDS
    if (active) {
      attn_tile<D>(qs, kt, vt, ps, min(TD_TILE, t1 - (t0 + tile * TD_TILE)), m, l, acc);
      if (P.trace && tile == 0) stamp = wall_clock64();
    }
    wg_bar();  // tile consumed
  }
  if (active) {
    acc = attn_finish<D>(acc);
    float* pr = (float*)(base + A.part) + wave * (D + 4);
    if (lane < D / 4) *(f32x4*)(pr + 4 * lane) = acc;
    if (lane == 0) *(f32x4*)(pr + D) = f32x4{m, l, 0.f, 0.f};
  }
  return stamp;
}

DEV uint64_t attn_compute(const td_kparams& P, uint8_t* lds, int wave) {
  const AttnTask T = attn_task(P, blockIdx.x);
  if (!T.valid) return 0;
  return P.d == 64 ? attn_compute_d<64>(P, lds, wave, T) : attn_compute_d<128>(P, lds, wave, T);
}

// sync wave: K and V rows [tb, tb + nv) of the tile, except row pos (written
// during this very step; it comes from the published copy), into the LDS tile
DEV void load_tile(const td_kparams& P, uint8_t* lds, int layer, const AttnTask& T, int tile) {
  const int lane = lane_id();
  const int d = P.d;
  const int tb = T.t0 + tile * TD_TILE;
  const int nv = min(TD_TILE, T.t1 - tb);
  const size_t head_off = ((size_t)layer * P.nkv + T.g) * P.max_ctx;
  const __amdgpu_buffer_rsrc_t RK = rsrc(P.kc + (head_off + tb) * d, (uint32_t)(nv * d * 2));
  const __amdgpu_buffer_rsrc_t RV = rsrc(P.vc + (head_off + tb) * d, (uint32_t)(nv * d * 2));
  uint16_t* kt = (uint16_t*)(lds + P.off_tile);
  uint16_t* vt = kt + TD_TILE * (d + 8);
  const int q16 = d / 8;  // 16-byte pieces per row
  const int npiece = TD_TILE * q16;  // the whole tile: rows >= nv read as zero
  for (int i0 = 0; i0 < npiece; i0 += 8 * 64) {
    u32x4 kr[8], vr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t off = (uint32_t)(i0 + k * 64 + lane) * 16u;  // out of range reads 0
      kr[k] = __builtin_amdgcn_raw_buffer_load_b128(RK, off, 0, 0);
      vr[k] = __builtin_amdgcn_raw_buffer_load_b128(RV, off, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = i0 + k * 64 + lane;
      if (i < npiece) {
        const int row = i / q16, pc = i - row * q16;
        if (row >= nv || tb + row != P.pos) {  // row pos comes from the published copy
          *(u32x4*)(kt + row * (d + 8) + pc * 8) = kr[k];
          *(u32x4*)(vt + row * d + pc * 8) = vr[k];
        }
      }
    }
  }
}

// writes this position's K and V rows (from LDS, fp32 holding bf16 values)
// into the tile when the tile holds position pos
DEV void patch_pos_row(const td_kparams& P, uint8_t* lds, const AttnTask& T, int tile) {
  const int tb = T.t0 + tile * TD_TILE;
  if (P.pos < tb || P.pos >= tb + TD_TILE || P.pos >= T.t1) return;
  const int d = P.d, row = P.pos - tb;
  const td_attn_lds A = td_attn_layout(d, P.group, P.n_chunks_max);
  const float* kvp = (const float*)(lds + P.off_attn + A.kvp);
  uint16_t* kt = (uint16_t*)(lds + P.off_tile);
  uint16_t* vt = kt + TD_TILE * (d + 8);
  for (int e = lane_id(); e < d; e += 64) {
    kt[row * (d + 8) + e] = (uint16_t)(__float_as_uint(kvp[e]) >> 16);
    vt[row * d + e] = (uint16_t)(__float_as_uint(kvp[d + e]) >> 16);
  }
}

// ------------------------------------------------------------ compute waves
// A compute wave walks its packed weight stream (one contiguous array per wave,
// built at create time in exactly the order consumed here): chunk t lands in
// ring slot t % S, and the DMA of chunk t + S is issued as soon as chunk t has
// been read out of its slot.  The DMA never waits for a stage boundary, so the
// next stage's weights stream in while this CU waits at the grid barrier.
#define TD_DMA_NT 2  // cache policy of the weight stream: non-temporal
#define LDSPTR(p) ((__attribute__((address_space(3))) void*)(p))

template <int S>
DEV void compute_wave(const td_kparams& P, uint8_t* lds, int wave) {
  const int lane = lane_id();
  const int cu = blockIdx.x, ncu = gridDim.x;
  uint8_t* ring = lds + P.off_ring + wave * S * TD_CHUNK;
  uint8_t* sring = lds + P.off_sring + wave * S * TD_SCHUNK;
  const float* xin = (const float*)(lds + P.off_xin);
  float* out = (float*)(lds + P.off_out);
  const td_wstream& W = P.ws[cu * TD_NW + wave];
  const uint32_t n_tot = W.n_tot, n4 = W.n4;
  const uint8_t* fptr = P.wcode + (size_t)W.code_off * TD_CHUNK + lane * 16;
  const uint8_t* sptr = P.wscale + (size_t)W.scale_off * TD_SCHUNK + lane * 4;
  uint32_t issued = 0;
  auto issue = [&](int slot) {
    __builtin_amdgcn_global_load_lds((const void*)fptr, LDSPTR(ring + slot * TD_CHUNK), 16, 0, TD_DMA_NT);
    fptr += TD_CHUNK;
    if (issued < n4) {  // the chunk's 32 fp16 scales: 16 lanes x 4 bytes
      if (lane < 16)
        __builtin_amdgcn_global_load_lds((const void*)sptr, LDSPTR(sring + slot * TD_SCHUNK), 4, 0, TD_DMA_NT);
      sptr += TD_SCHUNK;
    }
    ++issued;
  };
#pragma unroll
  for (int t = 0; t < S; ++t)
    if (issued < n_tot) issue(t);

  uint32_t t = 0;  // chunks consumed
  int slot = 0;
  wg_bar();  // stage 0 inputs staged
  for (int seq = 0; seq < P.n_stages; ++seq) {
    if (seq) wg_bar();  // stage seq inputs staged
    int kind, layer;
    stage_of(P, seq, kind, layer);
    uint64_t w0 = 0, w1 = 0;
    if (P.trace) w0 = wall_clock64();
    if (kind == TD_ST_ATTN) {
      w1 = attn_compute(P, lds, wave);
    } else {
      const Gemv g = gemv_of(P, kind, layer);
      int u0, u1;
      cu_units(g.U, cu, ncu, u0, u1);
      const int cnt = u1 - u0;
      const int n = cnt > wave ? (cnt - wave + TD_NW - 1) / TD_NW : 0;
      const int nrows = n * g.rpu;
      for (int row = 0; row < nrows; ++row) {
        float acc = 0.f;
        for (int j = 0; j < g.J; ++j) {
          // chunk t is complete once at most the ops issued after it are pending
          const uint32_t after = issued - 1u - t;
          if (after >= (uint32_t)(S - 1)) {
            if (t < n4 && issued - 1u < n4) vmcnt_wait<2 * S - 2>();
            else vmcnt_wait<S - 1>();
          } else {
            vmcnt_wait<0>();
          }
          if (P.trace && row == 0 && j == 0) w1 = wall_clock64();
          const u32x4 w = *(const u32x4*)(ring + slot * TD_CHUNK + lane * 16);
          if (g.fmt == 0) {
            acc += dot_bf16(w, xin + j * 512 + lane * 8);
          } else {
            const float sc = f16f(*(const uint16_t*)(sring + slot * TD_SCHUNK + (lane >> 1) * 2));
            acc += dot_int4(w, xin + j * 2048 + lane * 32, sc);
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slot read out: refill it
          if (issued < n_tot) issue(slot);
          slot = slot + 1 == S ? 0 : slot + 1;
          ++t;
        }
        const float r = wave_sum(acc);
        const int k = g.rpu == 2 ? row >> 1 : row, rr = g.rpu == 2 ? row & 1 : 0;
        if (lane == 0) out[(wave + k * TD_NW) * g.rpu + rr] = r;
      }
    }
    if (P.trace) {
      uint64_t* wt = (uint64_t*)(lds + P.off_wtrace) + wave * 4;
      const uint64_t w2 = wall_clock64();
      if (lane == 0) {
        wt[0] = w0;
        wt[1] = w1;
        wt[2] = (w1 || kind == TD_ST_ATTN) ? w2 : 0;
      }
    }
    wg_bar();  // stage seq outputs in LDS
  }
}

// ------------------------------------------------------------ sync wave
// zero LDS floats [from, to): the tail of the last chunk of a GEMV input
DEV void zero_tail(float* x, int from, int to) {
  for (int i = from + lane_id(); i < to; i += 64) x[i] = 0.f;
}

DEV int chunk_elems(int fmt) { return fmt ? 2048 : 512; }

// RMSNorm of the residual stream into LDS: xin = x / sqrt(mean(x^2) + eps) * gain.
// The source is the published residual (tagged), or the bf16 embedding row; the
// bf16 gains were DMA'd into LDS when the previous stage ended.
DEV bool norm_input(const td_kparams& P, uint8_t* lds, const uint2* xsrc, uint32_t tag, const uint16_t* esrc,
                    int fmt) {
  const int lane = lane_id();
  float* xin = (float*)(lds + P.off_xin);
  const uint16_t* gain = (const uint16_t*)(lds + P.off_gain);
  const int H = P.H;  // multiple of 256
  bool ok = true;
  if (esrc) {
    for (int i = lane * 4; i < H; i += 256) {
      uint2 e = *(const uint2*)(esrc + i);
      f32x4 v = {bf_lo(e.x), bf_hi(e.x), bf_lo(e.y), bf_hi(e.y)};
      *(f32x4*)(xin + i) = v;
    }
  } else {
    ok = poll_vec(P, xsrc, H, tag, xin);
  }
  vm_drain();  // the gains' DMA into LDS
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float ss = 0.f;
  for (int i = lane * 4; i < H; i += 256) {
    f32x4 v = *(const f32x4*)(xin + i);
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)H + P.eps);
  for (int i = lane * 4; i < H; i += 256) {
    f32x4 v = *(const f32x4*)(xin + i);
    uint2 g = *(const uint2*)(gain + i);
    v.x = v.x * inv * bf_lo(g.x);
    v.y = v.y * inv * bf_hi(g.x);
    v.z = v.z * inv * bf_lo(g.y);
    v.w = v.w * inv * bf_hi(g.y);
    *(f32x4*)(xin + i) = v;
  }
  const int ce = chunk_elems(fmt);
  zero_tail(xin, H, (H + ce - 1) / ce * ce);
  return ok;
}

// Issued as soon as a stage's epilogue is out: the DMA of the next stage's
// bf16 norm gains into LDS, and the QKV bias of this CU's units.
DEV void preload(const td_kparams& P, uint8_t* lds, int kind, int layer, float& ba, float& bb) {
  const int lane = lane_id();
  const uint16_t* g = kind == TD_ST_QKV ? P.layers[layer].attn_norm
                    : kind == TD_ST_GU ? P.layers[layer].mlp_norm
                    : kind == TD_ST_HEAD ? P.final_norm : nullptr;
  if (g) {
    const int bytes = P.H * 2;
    for (int off = 0; off < bytes; off += TD_CHUNK)
      if (off + lane * 16 < bytes)
        __builtin_amdgcn_global_load_lds((const void*)((const uint8_t*)g + off + lane * 16),
                                         LDSPTR(lds + P.off_gain + off), 16, 0, 0);
  }
  if (kind == TD_ST_QKV && P.has_bias) {
    int u0, u1;
    cu_units(P.qkv_rows / 2, blockIdx.x, gridDim.x, u0, u1);
    if (lane < u1 - u0) {
      const int ra = unit_row(P, TD_ST_QKV, u0 + lane, 0);
      ba = bf16f(P.layers[layer].bias[ra]);
      bb = bf16f(P.layers[layer].bias[ra + (P.d >> 1)]);
    }
  }
}

// The chunk-0 CU of kv head g: combine every chunk's partial,
// o = sum_c acc_c e^(m_c - M) / sum_c l_c e^(m_c - M), and publish o.  The
// weights w[h][c] go to LDS first; then lane i owns 4 consecutive outputs
// (head i / (D/4)) and sums over the chunks in chunk order.
template <int D>
DEV void attn_merge_d(const td_kparams& P, uint8_t* lds, const AttnTask& T, uint32_t tag) {
  const int lane = lane_id();
  const int G = P.group, n = T.n_used;
  constexpr int st = D + 4;
  const td_attn_lds A = td_attn_layout(D, G, P.n_chunks_max);
  const float* own = (const float*)(lds + P.off_attn + A.part);
  const float* mb = (const float*)(lds + P.off_attn + A.merge);
  float* wl = (float*)(lds + P.off_attn + A.p);  // [G][64]: free once the tiles are consumed
  for (int h = 0; h < G; ++h) {
    const bool have = lane < n;  // n <= 64
    const float* pc = lane == 0 ? own + h * st : mb + ((have ? lane - 1 : 0) * G + h) * st;
    const float m = have ? pc[D] : -__builtin_inff();
    const float l = have ? pc[D + 1] : 0.f;
    const float M = wave_max(m);
    const float w0 = have ? __expf(m - M) : 0.f;
    wl[h * 64 + lane] = w0 / wave_sum(l * w0);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  for (int i = lane; i < G * (D / 4); i += 64) {
    const int h = i / (D / 4), e = 4 * (i - h * (D / 4));
    const float w00 = wl[h * 64];
    f32x4 o = *(const f32x4*)(own + h * st + e);
    o.x *= w00; o.y *= w00; o.z *= w00; o.w *= w00;
    for (int c = 1; c < n; ++c) {
      const f32x4 v = *(const f32x4*)(mb + ((c - 1) * G + h) * st + e);
      const float w = wl[h * 64 + c];
      o.x = fmaf(w, v.x, o.x);
      o.y = fmaf(w, v.y, o.y);
      o.z = fmaf(w, v.z, o.z);
      o.w = fmaf(w, v.w, o.w);
    }
    uint2* dst = P.to + ((size_t)T.g * G + h) * D + e;
    st_tag(dst + 0, o.x, tag);
    st_tag(dst + 1, o.y, tag);
    st_tag(dst + 2, o.z, tag);
    st_tag(dst + 3, o.w, tag);
  }
}

DEV bool attn_merge(const td_kparams& P, uint8_t* lds, const AttnTask& T, uint32_t tag) {
  const int d = P.d, G = P.group, st = d + 4;
  const td_attn_lds A = td_attn_layout(d, G, P.n_chunks_max);
  float* mb = (float*)(lds + P.off_attn + A.merge);
  bool ok = true;
  if (T.n_used > 1)
    ok = poll_vec(P, P.tpart + ((size_t)T.g * P.n_chunks_max + 1) * G * st, (T.n_used - 1) * G * st, tag, mb);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (P.trace && lane_id() == 0) ((uint64_t*)(lds + P.off_wtrace))[TD_NW * 4] = wall_clock64();
  if (d == 64) attn_merge_d<64>(P, lds, T, tag);
  else attn_merge_d<128>(P, lds, T, tag);
  return ok;
}

// stage outputs -> epilogue -> published values (tag: this stage's)
DEV bool sync_epilogue(const td_kparams& P, uint8_t* lds, int kind, int layer, uint32_t tag, uint32_t epoch,
                       const AttnTask& T, float ba, float bb) {
  const int lane = lane_id();
  const int cu = blockIdx.x, ncu = gridDim.x;
  const float* out = (const float*)(lds + P.off_out);
  float* own = (float*)(lds + P.off_own);
  bool ok = true;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (kind == TD_ST_QKV) {
    int u0, u1;
    cu_units(P.qkv_rows / 2, cu, ncu, u0, u1);
    const int half = P.d >> 1;
    const float* cs = (const float*)(lds + P.off_rope);
    if (lane < u1 - u0) {  // at most 64 units per CU (checked at create)
      const int u = u0 + lane;
      const int ra = unit_row(P, TD_ST_QKV, u, 0), rb = ra + half;
      float a = out[2 * lane], b = out[2 * lane + 1];
      if (P.has_bias) {
        a += ba;
        b += bb;
      }
      const int i = ra % P.d;  // < d/2
      if (ra < P.qd + P.kvd) {  // q or k: rotate the pair by pos * theta_i
        const float c = cs[2 * i], sn = cs[2 * i + 1];
        const float a2 = a * c - b * sn;
        const float b2 = b * c + a * sn;
        a = a2;
        b = b2;
      }
      const int gw = (P.group + 2) * P.d;  // published block of one kv head
      if (ra < P.qd) {
        const int h = ra / P.d, g = h / P.group;
        uint2* pub = P.tq + (size_t)g * gw + (h - g * P.group) * P.d;
        st_tag(pub + i, a, tag);
        st_tag(pub + i + half, b, tag);
      } else {
        const bool isk = ra < P.qd + P.kvd;
        const int g = (ra - P.qd - (isk ? 0 : P.kvd)) / P.d;
        const uint32_t ab = f2bf(a), bbits = f2bf(b);
        uint16_t* row = (isk ? P.kc : P.vc) + (((size_t)layer * P.nkv + g) * P.max_ctx + P.pos) * P.d;
        row[i] = (uint16_t)ab;
        row[i + half] = (uint16_t)bbits;
        uint2* pub = P.tq + (size_t)g * gw + (P.group + (isk ? 0 : 1)) * P.d;
        st_tag(pub + i, __uint_as_float(ab << 16), tag);
        st_tag(pub + i + half, __uint_as_float(bbits << 16), tag);
      }
    }
  } else if (kind == TD_ST_O || kind == TD_ST_DOWN) {
    int r0, r1;
    cu_units(P.H, cu, ncu, r0, r1);
    uint2* dst = kind == TD_ST_O ? P.tx_mid : P.tx_out;
    for (int k = lane; k < r1 - r0; k += 64) {
      const float v = own[k] + out[k];
      own[k] = v;
      st_tag(dst + r0 + k, v, tag);
    }
  } else if (kind == TD_ST_GU) {
    int u0, u1;
    cu_units(P.I, cu, ncu, u0, u1);
    for (int k = lane; k < u1 - u0; k += 64) {
      const float gt = out[2 * k], up = out[2 * k + 1];
      st_tag(P.tact + u0 + k, gt / (1.0f + expf(-gt)) * up, tag);
    }
  } else if (kind == TD_ST_ATTN) {
    if (T.valid) {
      if (T.c == 0) {
        ok = attn_merge(P, lds, T, tag);
      } else {
        const int st = P.d + 4;
        const td_attn_lds A = td_attn_layout(P.d, P.group, P.n_chunks_max);
        const float* pr = (const float*)(lds + P.off_attn + A.part);
        uint2* gp = P.tpart + ((size_t)T.g * P.n_chunks_max + T.c) * P.group * st;
        for (int i = lane; i < P.group * st; i += 64) st_tag(gp + i, pr[i], tag);
      }
    }
  } else {  // HEAD: logits, per-CU candidate, last arriver picks the token
    int u0, u1;
    cu_units(P.V, cu, ncu, u0, u1);
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    int bad = 0;
    for (int k = lane; k < u1 - u0; k += 64) {
      const float v = out[k];
      P.logits[u0 + k] = v;
      if (!isfinite(v)) bad = 1;
      else if (v > bv) { bv = v; bi = u0 + k; }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    bad = __any(bad);
    if (lane == 0) {
      st_u(P.cand + cu * 4 + 0, __float_as_uint(bv));
      st_u(P.cand + cu * 4 + 1, (uint32_t)bi);
      st_u(P.cand + cu * 4 + 2, (uint32_t)bad);
    }
    vm_drain();
    int last = 0;
    if (lane == 0) last = atomicAdd(P.sync + TD_SY_FINAL, 1u) + 1u == (uint32_t)ncu;
    if (uni(last)) {
      float fv = -__builtin_inff();
      int fi = 0x7fffffff, fbad = 0;
      for (int c = lane; c < ncu; c += 64) {
        const float v = __uint_as_float(ld_u(P.cand + c * 4 + 0));
        const int i = (int)ld_u(P.cand + c * 4 + 1);
        fbad |= (int)ld_u(P.cand + c * 4 + 2);
        if (v > fv || (v == fv && i < fi)) { fv = v; fi = i; }
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(fv, off);
        const int oi = __shfl_xor(fi, off);
        if (ov > fv || (ov == fv && oi < fi)) { fv = ov; fi = oi; }
      }
      fbad = __any(fbad);
      if (lane == 0) {
        *P.token_out = fi == 0x7fffffff ? 0 : fi;
        if (fbad) atomicOr(P.err, TD_ERRBIT_NONFINITE);
        st_u(P.sync + TD_SY_FINAL, 0u);
        st_u(P.sync + TD_SY_EPOCH, epoch + 1u);
      }
    }
  }
  return ok;
}

DEV void sync_wave(const td_kparams& P, uint8_t* lds) {
  const int lane = lane_id();
  const int cu = blockIdx.x, ncu = gridDim.x;
  const uint32_t epoch = uni(ld_u(P.sync + TD_SY_EPOCH));
  const uint32_t tag0 = epoch * (uint32_t)P.n_stages;  // stage seq publishes tag0 + seq + 1
  bool ok = true;
  if (ld_u(P.sync + TD_SY_ABORT)) ok = false;
  int tok = uni(*P.token_in);
  if (tok < 0 || tok >= P.V) {
    if (lane == 0 && cu == 0) atomicOr(P.err, TD_ERRBIT_RANGE);
    tok = 0;
  }
  const uint16_t* erow = P.embed + (size_t)tok * P.H;
  {  // this CU's residual rows start as the embedding row; the RoPE row of pos
    int r0, r1;
    cu_units(P.H, cu, ncu, r0, r1);
    float* own = (float*)(lds + P.off_own);
    for (int k = lane; k < r1 - r0; k += 64) own[k] = bf16f(erow[r0 + k]);
    float* cs = (float*)(lds + P.off_rope);
    for (int i = lane; i < P.d; i += 64) cs[i] = P.rope_cs[(size_t)P.pos * P.d + i];
  }
  const AttnTask T = attn_task(P, cu);
  const td_attn_lds A = td_attn_layout(P.d, P.group, P.n_chunks_max);
  float ba = 0.f, bb = 0.f;
  preload(P, lds, TD_ST_QKV, 0, ba, bb);
  uint64_t* tr = P.trace ? P.trace + (size_t)cu * P.n_stages * TD_TRACE_STAMPS : nullptr;
  for (int seq = 0; seq < P.n_stages; ++seq) {
    int kind, layer;
    stage_of(P, seq, kind, layer);
    const uint32_t tag_in = tag0 + (uint32_t)seq, tag = tag_in + 1u;
    uint64_t ts[TD_TRACE_STAMPS > 5 ? 5 : TD_TRACE_STAMPS] = {0, 0, 0, 0, 0};
    if (tr) ts[0] = wall_clock64();
    if (kind == TD_ST_QKV) {
      ok &= norm_input(P, lds, P.tx_out, tag_in, layer == 0 ? erow : nullptr, P.wf);
    } else if (kind == TD_ST_GU) {
      ok &= norm_input(P, lds, P.tx_mid, tag_in, nullptr, P.wf);
    } else if (kind == TD_ST_HEAD) {
      ok &= norm_input(P, lds, P.tx_out, tag_in, nullptr, 0);
    } else if (kind == TD_ST_O || kind == TD_ST_DOWN) {
      float* xin = (float*)(lds + P.off_xin);
      const int K = kind == TD_ST_O ? P.qd : P.I;
      ok &= poll_vec(P, kind == TD_ST_O ? P.to : P.tact, K, tag_in, xin);
      const int ce = chunk_elems(P.wf);
      zero_tail(xin, K, (K + ce - 1) / ce * ce);
    } else if (T.valid) {  // ATTN: the task's query heads (pre-scaled by 1/sqrt(d)), and row pos
      // the kv head's block: its query heads, then this position's K and V rows
      float* qs = (float*)(lds + P.off_attn + A.q);
      const int n = P.group * P.d;
      ok &= poll_vec(P, P.tq + (size_t)T.g * (n + 2 * P.d), n + 2 * P.d, tag_in, qs);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      for (int i = lane; i < n; i += 64) qs[i] *= P.attn_scale;
      if (T.t1 == P.pos + 1) patch_pos_row(P, lds, T, 0);
    }
    wg_bar();  // inputs ready
    if (tr) ts[1] = wall_clock64();
    if (kind == TD_ST_QKV && T.valid) {
      load_tile(P, lds, layer, T, 0);  // this layer's first attention tile, ahead of time
    } else if (kind == TD_ST_ATTN && T.valid) {
      for (int tile = 0; tile < T.ntiles; ++tile) {
        if (tile) {
          load_tile(P, lds, layer, T, tile);
          patch_pos_row(P, lds, T, tile);
        }
        wg_bar();  // tile in LDS
        wg_bar();  // tile consumed
      }
    }
    wg_bar();  // outputs ready
    if (tr) ts[2] = wall_clock64();
    ok &= sync_epilogue(P, lds, kind, layer, tag, epoch, T, ba, bb);
    if (tr) ts[3] = wall_clock64();
    if (seq + 1 < P.n_stages) {
      int nkind, nlayer;
      stage_of(P, seq + 1, nkind, nlayer);
      preload(P, lds, nkind, nlayer, ba, bb);
    }
    if (tr) {
      ts[4] = wall_clock64();
      uint64_t* rec = tr + (size_t)seq * TD_TRACE_STAMPS;
      if (lane < TD_TRACE_STAMPS) {
        const uint64_t* wt = (const uint64_t*)(lds + P.off_wtrace);
        uint64_t v = 0;
        if (lane < 5) v = ts[lane];
        else if (lane == 5) v = kind == TD_ST_ATTN && T.valid && T.c == 0 ? wt[TD_NW * 4] : 0;
        else if (lane >= 8 && lane < 8 + 3 * TD_NW) v = wt[((lane - 8) / 3) * 4 + (lane - 8) % 3];
        rec[lane] = v;
      }
    }
  }
  if (!ok && lane == 0) atomicOr(P.err, TD_ERRBIT_TIMEOUT);
}

template <int S>
__global__ void __launch_bounds__(TD_THREADS, 1) td_megakernel(td_kparams P) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int wave = uni((int)(threadIdx.x >> 6));
  if (wave < TD_NW) compute_wave<S>(P, lds, wave);
  else sync_wave(P, lds);
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
    const int boff = c.j * TD_CHUNK + lane * 16;
    u32x4 v;
    if (boff < c.g.row_bytes) {
      v = *(const u32x4*)(c.g.w + (size_t)row * c.g.row_bytes + boff);
    } else {
      const uint32_t z = c.g.fmt ? 0x88888888u : 0u;
      v = (u32x4){z, z, z, z};
    }
    *(u32x4*)(dst + lane * 16) = v;
    dst += TD_CHUNK;
    if (c.g.fmt == 1) {
      if (n4 >= W.n4) break;
      if (lane < 16) {
        const int si = c.j * 32 + lane * 2;
        uint32_t sv = 0;
        if (si < c.g.K / 64) sv = *(const uint32_t*)(c.g.s + (size_t)row * (c.g.K / 64) + si);
        *(uint32_t*)(sdst + lane * 4) = sv;
      }
      sdst += TD_SCHUNK;
      ++n4;
    }
    cur_next(c, P, wave, cu, ncu);
    ++n;
  }
  if (lane == 0 && (c.seq < P.n_stages || n != W.n_tot || n4 != W.n4)) atomicOr(bad, 1);
}

// ------------------------------------------------------------ test hooks
// y = W x, one wave per row, same chunk arithmetic as the megakernel.
__global__ void __launch_bounds__(256) td_gemv_kernel(int fmt, const uint8_t* w, const uint16_t* s, int rows,
                                                      int cols, const float* x, float* y) {
  const int lane = lane_id();
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int row_bytes = fmt == 0 ? cols * 2 : cols / 2;
  const int J = (row_bytes + TD_CHUNK - 1) / TD_CHUNK;
  float acc = 0.f;
  for (int j = 0; j < J; ++j) {
    const int boff = j * TD_CHUNK + lane * 16;
    if (boff < row_bytes) {
      const u32x4 wv = *(const u32x4*)(w + (size_t)row * row_bytes + boff);
      if (fmt == 0) {
        acc += dot_bf16(wv, x + j * 512 + lane * 8);
      } else {
        const int si = (j * 2048 + lane * 32) / 64;
        acc += dot_int4(wv, x + j * 2048 + lane * 32, f16f(s[(size_t)row * (cols / 64) + si]));
      }
    }
  }
  const float r = wave_sum(acc);
  if (lane == 0) y[row] = r;
}

// one query head over n bf16 K/V rows: scores, softmax, weighted V (one wave, lane = dim)
__global__ void __launch_bounds__(64) td_attention_kernel(const float* q, const uint16_t* k, const uint16_t* v,
                                                          int n, int d, float* out) {
  const int lane = lane_id();
  const float scale = 1.0f / sqrtf((float)d);
  float m = -__builtin_inff(), l = 0.f, a0 = 0.f, a1 = 0.f;
  for (int t = 0; t < n; ++t) {
    float part = 0.f;
    for (int e = lane; e < d; e += 64) part = fmaf(q[e], bf16f(k[(size_t)t * d + e]), part);
    const float s = wave_sum(part) * scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn), p = expf(s - mn);
    l = l * corr + p;
    a0 = a0 * corr + p * bf16f(v[(size_t)t * d + lane]);
    if (d > 64) a1 = a1 * corr + p * bf16f(v[(size_t)t * d + 64 + lane]);
    m = mn;
  }
  out[lane] = a0 / l;
  if (d > 64) out[64 + lane] = a1 / l;
}

}  // namespace

// ------------------------------------------------------------ launchers
#define TD_RING_CASES(X) X(8) X(12) X(16)

int td_megakernel_occupancy(int ring_slots, int lds_bytes, int* blocks) {
  hipError_t e = hipErrorInvalidValue;
#define OCC(S)                                                                                          \
  if (ring_slots == S) {                                                                                \
    e = hipFuncSetAttribute((const void*)td_megakernel<S>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                            lds_bytes);                                                                 \
    if (e == hipSuccess)                                                                                \
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, td_megakernel<S>, TD_THREADS, lds_bytes); \
  }
  TD_RING_CASES(OCC)
#undef OCC
  return (int)e;
}

int td_launch_megakernel(const td_kparams* p, int ncu, int ring_slots, void* stream) {
  void* args[] = {(void*)p};
  hipError_t e = hipErrorInvalidValue;
#define LAUNCH(S)                                                                                           \
  if (ring_slots == S)                                                                                      \
    e = hipLaunchCooperativeKernel((const void*)td_megakernel<S>, dim3(ncu), dim3(TD_THREADS), args,        \
                                   (unsigned)p->lds_bytes, (hipStream_t)stream);
  TD_RING_CASES(LAUNCH)
#undef LAUNCH
  return (int)e;
}

int td_launch_repack(const td_kparams* p, int ncu, uint8_t* code, uint8_t* scale, const td_wstream* ws, int* bad,
                     void* stream) {
  const int waves = ncu * TD_NW;
  td_repack_kernel<<<(waves + 3) / 4, 256, 0, (hipStream_t)stream>>>(*p, ncu, code, scale, ws, bad);
  return (int)hipGetLastError();
}

int td_launch_test_gemv(int fmt, const void* w, const void* s, int rows, int cols, const float* x, float* y,
                        void* stream) {
  td_gemv_kernel<<<(rows + 3) / 4, 256, 0, (hipStream_t)stream>>>(fmt, (const uint8_t*)w, (const uint16_t*)s, rows,
                                                                   cols, x, y);
  return (int)hipGetLastError();
}

int td_launch_test_attention(const float* q, const void* k, const void* v, int n, int d, float* out, void* stream) {
  td_attention_kernel<<<1, 64, 0, (hipStream_t)stream>>>(q, (const uint16_t*)k, (const uint16_t*)v, n, d, out);
  return (int)hipGetLastError();
}
