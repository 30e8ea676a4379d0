// td_kernels.hip - the persistent decode-step megakernel for MI355X (gfx950)
// and the single-routine kernels behind the test hooks.
//
// One workgroup per CU runs the whole step as a fixed sequence of stages
// separated by grid barriers ("Decoding in tiles", sec. 4: a static plan of
// waves; sec. 3: prefetching the next weights while waiting).  Per layer:
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
//     straight into a per-wave LDS ring with global_load_lds_dwordx4.  The
//     ring runs S chunks ahead of the arithmetic across stage boundaries and
//     grid barriers: weights never depend on the token, so the loads for the
//     next stage are in flight while the grid waits.  These waves issue no
//     other global memory operation, so vmcnt counts only ring loads.
//   1 sync wave does all activation traffic: it stages the stage inputs in
//     LDS (with the RMSNorm applied), runs the epilogues (bias, RoPE, K/V
//     write, SiLU*up, residual), publishes the stage outputs and takes part in
//     the grid barrier.
// Cross-CU data: written with agent-scope (sc1) stores, the writer waits for
// them (vmcnt(0)) before it arrives at the barrier, and readers use sc1 loads.
// This keeps values coherent across the 8 XCDs without writing back or
// invalidating whole L2 caches.  The barrier is two-level: 32 arrivals on a
// per-XCD counter, the last of them arrives on a global counter, then
// releases its XCD through a per-XCD word.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "td_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define DEV __device__ __forceinline__

DEV int lane_id() { return (int)__lane_id(); }
DEV int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------------ memory helpers
DEV uint32_t ld_u(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV float ld_f(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st_u(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void st_f(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void st_u16_sc1(uint16_t* p, uint32_t v) {
  asm volatile("global_store_short %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
DEV void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// workgroup barrier that waits for LDS traffic only (never for the ring loads)
DEV void wg_bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
template <int N>
DEV void vmcnt_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 8 agent-scope 16-byte loads, completed before the block ends
DEV void ld8x4_sc1(const void* const (&a)[8], u32x4 (&r)[8]) {
  asm volatile(
      "global_load_dwordx4 %0, %8, off sc1\n\t"
      "global_load_dwordx4 %1, %9, off sc1\n\t"
      "global_load_dwordx4 %2, %10, off sc1\n\t"
      "global_load_dwordx4 %3, %11, off sc1\n\t"
      "global_load_dwordx4 %4, %12, off sc1\n\t"
      "global_load_dwordx4 %5, %13, off sc1\n\t"
      "global_load_dwordx4 %6, %14, off sc1\n\t"
      "global_load_dwordx4 %7, %15, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// ------------------------------------------------------------ number formats
DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
DEV float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
DEV uint32_t f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
DEV float f16f(uint32_t h) { return __half2float(__ushort_as_half((unsigned short)(h & 0xffffu))); }

// ------------------------------------------------------------ wave reductions (DPP)
template <int CTRL, int RM = 0xf>
DEV float dpp(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, RM, 0xf, false));
}
DEV float wave_sum(float v) {
  v += dpp<0x111>(0.f, v);  // row_shr:1
  v += dpp<0x112>(0.f, v);  // row_shr:2
  v += dpp<0x114>(0.f, v);  // row_shr:4
  v += dpp<0x118>(0.f, v);  // row_shr:8  -> lane 15 of each row holds the row sum
  v += dpp<0x142, 0xa>(0.f, v);  // row_bcast:15 -> rows 1, 3
  v += dpp<0x143, 0xc>(0.f, v);  // row_bcast:31 -> rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
DEV float wave_max(float v) {
  const float ninf = -__builtin_inff();
  v = fmaxf(v, dpp<0x111>(ninf, v));
  v = fmaxf(v, dpp<0x112>(ninf, v));
  v = fmaxf(v, dpp<0x114>(ninf, v));
  v = fmaxf(v, dpp<0x118>(ninf, v));
  v = fmaxf(v, dpp<0x142, 0xa>(ninf, v));
  v = fmaxf(v, dpp<0x143, 0xc>(ninf, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ------------------------------------------------------------ chunk arithmetic
// bf16 chunk: lane holds 8 consecutive weights of the row, x holds the 8
// matching activations.
DEV float dot_bf16(u32x4 w, const float* x) {
  f32x4 a = *(const f32x4*)x;
  f32x4 b = *(const f32x4*)(x + 4);
  float s = bf_lo(w.x) * a.x;
  s = fmaf(bf_hi(w.x), a.y, s);
  s = fmaf(bf_lo(w.y), a.z, s);
  s = fmaf(bf_hi(w.y), a.w, s);
  s = fmaf(bf_lo(w.z), b.x, s);
  s = fmaf(bf_hi(w.z), b.y, s);
  s = fmaf(bf_lo(w.w), b.z, s);
  s = fmaf(bf_hi(w.w), b.w, s);
  return s;
}
// int4 chunk: lane holds 32 consecutive 4-bit codes (element 2i in the low
// nibble of byte i), all in one scale group; weight = scale * (code - 8).
DEV float dot_int4_word(uint32_t q, const float* x) {
  f32x4 a = *(const f32x4*)x;
  f32x4 b = *(const f32x4*)(x + 4);
  float s = ((float)(q & 15u) - 8.f) * a.x;
  s = fmaf((float)((q >> 4) & 15u) - 8.f, a.y, s);
  s = fmaf((float)((q >> 8) & 15u) - 8.f, a.z, s);
  s = fmaf((float)((q >> 12) & 15u) - 8.f, a.w, s);
  s = fmaf((float)((q >> 16) & 15u) - 8.f, b.x, s);
  s = fmaf((float)((q >> 20) & 15u) - 8.f, b.y, s);
  s = fmaf((float)((q >> 24) & 15u) - 8.f, b.z, s);
  s = fmaf((float)(q >> 28) - 8.f, b.w, s);
  return s;
}
DEV float dot_int4(u32x4 w, const float* x, float scale) {
  float s = dot_int4_word(w.x, x);
  s += dot_int4_word(w.y, x + 8);
  s += dot_int4_word(w.z, x + 16);
  s += dot_int4_word(w.w, x + 24);
  return s * scale;
}

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

// Start the DMA of the cursor's chunk into one ring slot.  Lanes past the end
// of the row (K not a multiple of the chunk) fetch the row start instead and
// are masked out of the arithmetic.
DEV void issue_chunk(const Cursor& c, const td_kparams& P, uint8_t* slot, uint8_t* sslot, int lane) {
  int u = c.u_first + c.k * TD_NW;
  int row = unit_row(P, c.g.kind, u, c.r);
  int boff = c.j * TD_CHUNK + lane * 16;
  bool valid = boff < c.g.row_bytes;
  const uint8_t* src = c.g.w + (size_t)row * c.g.row_bytes + (valid ? boff : 0);
  __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)slot, 16, 0, 0);
  if (c.g.fmt == 1) {
    // scale pair (2m, 2m + 1) with m = 16 j + lane / 4 holds this lane's scale
    int sw = valid ? c.j * 16 + (lane >> 2) : 0;
    const uint32_t* ss = (const uint32_t*)(c.g.s + (size_t)row * (c.g.K / 64)) + sw;
    __builtin_amdgcn_global_load_lds((const void*)ss, (__attribute__((address_space(3))) void*)sslot, 4, 0, 0);
  }
}

// ------------------------------------------------------------ grid barrier
DEV int spin_ge(uint32_t* p, uint32_t target, uint32_t* abortf) {
  uint64_t t0 = wall_clock64();
  for (uint32_t it = 0;; ++it) {
    if ((int32_t)(ld_u(p) - target) >= 0) return 1;
    if ((it & 63u) == 63u) {
      if (ld_u(abortf)) return 0;
      if (wall_clock64() - t0 > TD_SPIN_TICKS) {
        st_u(abortf, 1u);
        return 0;
      }
    }
  }
}

// gen: this barrier's global generation number (launch epoch * barriers per launch + index)
DEV bool grid_barrier(const td_kparams& P, uint32_t gen) {
  uint32_t* S = P.sync;
  int ok = 1;
  if (lane_id() == 0) {
    uint32_t x = blockIdx.x & 7u;
    uint32_t per = gridDim.x >> 3;
    uint32_t old = atomicAdd(S + TD_SY_XCTR + x * 64u, 1u);
    if (old + 1u == (gen + 1u) * per) {
      atomicAdd(S + TD_SY_GCTR, 1u);
      ok = spin_ge(S + TD_SY_GCTR, (gen + 1u) * 8u, S + TD_SY_ABORT);
      st_u(S + TD_SY_XREL + x * 64u, gen + 1u);
    } else {
      ok = spin_ge(S + TD_SY_XREL + x * 64u, gen + 1u, S + TD_SY_ABORT);
    }
  }
  return uni(ok) != 0;
}

// ------------------------------------------------------------ attention task
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

// compute waves: wave h < group handles query head g * group + h
DEV void attn_compute(const td_kparams& P, uint8_t* lds, int wave) {
  const AttnTask T = attn_task(P, blockIdx.x);
  if (!T.valid) return;
  const int lane = lane_id();
  const int d = P.d;
  const td_attn_lds A = td_attn_layout(d, P.group);
  uint8_t* base = lds + P.off_attn;
  const float* qs = (const float*)(base + A.q) + wave * d;
  const uint16_t* kt = (const uint16_t*)(base + A.k);
  const uint16_t* vt = (const uint16_t*)(base + A.v);
  float* ps = (float*)(base + A.p) + wave * TD_TILE;
  float m = -__builtin_inff(), l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int tile = 0; tile < T.ntiles; ++tile) {
    wg_bar();  // tile in LDS
    if (wave < P.group) {
      const int nv = min(TD_TILE, T.t1 - (T.t0 + tile * TD_TILE));
      float s = -__builtin_inff();
      if (lane < nv) {
        const uint16_t* kr = kt + lane * (d + 8);
        float a = 0.f;
        for (int e = 0; e < d; e += 8) {
          u32x4 kw = *(const u32x4*)(kr + e);
          a = fmaf(bf_lo(kw.x), qs[e + 0], a);
          a = fmaf(bf_hi(kw.x), qs[e + 1], a);
          a = fmaf(bf_lo(kw.y), qs[e + 2], a);
          a = fmaf(bf_hi(kw.y), qs[e + 3], a);
          a = fmaf(bf_lo(kw.z), qs[e + 4], a);
          a = fmaf(bf_hi(kw.z), qs[e + 5], a);
          a = fmaf(bf_lo(kw.w), qs[e + 6], a);
          a = fmaf(bf_hi(kw.w), qs[e + 7], a);
        }
        s = a;
      }
      const float mt = wave_max(s);
      const float mn = fmaxf(m, mt);
      const float p = lane < nv ? expf(s - mn) : 0.f;
      const float corr = expf(m - mn);
      l = l * corr + wave_sum(p);
      m = mn;
      ps[lane] = p;
      acc0 *= corr;
      acc1 *= corr;
      for (int t = 0; t < nv; ++t) {
        const float pt = ps[t];
        acc0 = fmaf(pt, bf16f(vt[t * d + lane]), acc0);
        if (d > 64) acc1 = fmaf(pt, bf16f(vt[t * d + 64 + lane]), acc1);
      }
    }
    wg_bar();  // tile consumed
  }
  if (wave < P.group) {
    float* pr = (float*)(base + A.part) + wave * (d + 2);
    pr[lane] = acc0;
    if (d > 64) pr[64 + lane] = acc1;
    if (lane == 0) {
      pr[d] = m;
      pr[d + 1] = l;
    }
  }
}

// sync wave: loads the K and V rows of each tile into LDS
DEV void attn_load_tiles(const td_kparams& P, uint8_t* lds, int layer) {
  const AttnTask T = attn_task(P, blockIdx.x);
  if (!T.valid) return;
  const int lane = lane_id();
  const int d = P.d;
  const td_attn_lds A = td_attn_layout(d, P.group);
  uint8_t* base = lds + P.off_attn;
  const size_t head_off = ((size_t)layer * P.nkv + T.g) * P.max_ctx;
  const uint16_t* kg = P.kc + head_off * d;
  const uint16_t* vg = P.vc + head_off * d;
  const int q16 = d / 8;  // 16-byte pieces per row
  for (int tile = 0; tile < T.ntiles; ++tile) {
    const int tb = T.t0 + tile * TD_TILE;
    const int nv = min(TD_TILE, T.t1 - tb);
    const int npiece = nv * q16;
    for (int i0 = 0; i0 < npiece; i0 += 8 * 64) {
      const void* ka[8];
      const void* va[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        int i = i0 + k * 64 + lane;
        int ii = i < npiece ? i : 0;
        int row = ii / q16, pc = ii - row * q16;
        ka[k] = kg + (size_t)(tb + row) * d + pc * 8;
        va[k] = vg + (size_t)(tb + row) * d + pc * 8;
      }
      u32x4 kr[8], vr[8];
      ld8x4_sc1(ka, kr);
      ld8x4_sc1(va, vr);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        int i = i0 + k * 64 + lane;
        if (i < npiece) {
          int row = i / q16, pc = i - row * q16;
          *(u32x4*)(base + A.k + (row * (d + 8) + pc * 8) * 2) = kr[k];
          *(u32x4*)(base + A.v + (row * d + pc * 8) * 2) = vr[k];
        }
      }
    }
    wg_bar();  // tile in LDS
    wg_bar();  // tile consumed
  }
}

// ------------------------------------------------------------ compute waves
template <int S>
DEV void compute_transition(const td_kparams& P, uint8_t* lds, int wave, int from, int to) {
  for (int s = from; s < to; ++s) {
    wg_bar();  // end of stage s: outputs in LDS
    if (s + 1 >= P.n_stages) return;
    wg_bar();  // stage s + 1 inputs in LDS
    int kind, layer;
    stage_of(P, s + 1, kind, layer);
    if (kind == TD_ST_ATTN) attn_compute(P, lds, wave);
  }
}

template <int S>
DEV void compute_wave(const td_kparams& P, uint8_t* lds, int wave) {
  const int lane = lane_id();
  const int cu = blockIdx.x, ncu = gridDim.x;
  uint8_t* ring = lds + P.off_ring + wave * S * TD_CHUNK;
  uint8_t* sring = lds + P.off_sring + wave * S * TD_SCHUNK;
  const float* xin = (const float*)(lds + P.off_xin);
  float* out = (float*)(lds + P.off_out);

  Cursor use, fe;
  cur_enter(use, P, wave, cu, ncu, 0);
  fe = use;
  int issued = 0;
  int last_int4 = 0;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    if (fe.seq < P.n_stages) {
      issue_chunk(fe, P, ring + t * TD_CHUNK, sring + t * TD_SCHUNK, lane);
      last_int4 = fe.g.fmt;
      cur_next(fe, P, wave, cu, ncu);
      ++issued;
    }
  }

  int cur = 0;
  wg_bar();  // stage 0 inputs in LDS
  float acc = 0.f;
  int slot = 0;
  for (int t = 0; use.seq < P.n_stages; ++t) {
    if (use.seq != cur) {
      compute_transition<S>(P, lds, wave, cur, use.seq);
      cur = use.seq;
    }
    // chunk t is complete once at most `after` newer DMA operations are pending
    const int after = issued - 1 - t;
    if (after >= S - 1) {
      if (use.g.fmt == 1 && last_int4) vmcnt_wait<2 * S - 2>();
      else vmcnt_wait<S - 1>();
    } else {
      vmcnt_wait<0>();
    }
    const uint8_t* sp = ring + slot * TD_CHUNK;
    const u32x4 w = *(const u32x4*)(sp + lane * 16);
    const bool valid = use.j * TD_CHUNK + lane * 16 < use.g.row_bytes;
    float c = 0.f;
    if (use.g.fmt == 0) {
      const float* xp = xin + use.j * 512 + lane * 8;
      c = dot_bf16(w, xp);
    } else {
      const uint32_t sw = *(const uint32_t*)(sring + slot * TD_SCHUNK + lane * 4);
      const float sc = f16f(((lane >> 1) & 1) ? (sw >> 16) : sw);
      const float* xp = xin + use.j * 2048 + lane * 32;
      c = dot_int4(w, xp, sc);
    }
    acc += valid ? c : 0.f;
    // the slot's data is in registers: refill it with the chunk S ahead
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (fe.seq < P.n_stages) {
      issue_chunk(fe, P, ring + slot * TD_CHUNK, sring + slot * TD_SCHUNK, lane);
      last_int4 = fe.g.fmt;
      cur_next(fe, P, wave, cu, ncu);
      ++issued;
    }
    if (use.j == use.g.J - 1) {
      const float r = wave_sum(acc);
      if (lane == 0) out[(wave + use.k * TD_NW) * use.g.rpu + use.r] = r;
      acc = 0.f;
    }
    cur_next(use, P, wave, cu, ncu);
    slot = slot + 1 == S ? 0 : slot + 1;
  }
  compute_transition<S>(P, lds, wave, cur, P.n_stages);
}

// ------------------------------------------------------------ sync wave
// Loads n fp32 values (n % 4 == 0) published by other CUs into LDS.
DEV void load_vec_sc1(const float* src, int n, float* dst) {
  const int lane = lane_id();
  for (int i0 = 0; i0 < n; i0 += 8 * 256) {
    const void* a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int i = i0 + (k * 64 + lane) * 4;
      a[k] = src + (i < n ? i : 0);
    }
    u32x4 r[8];
    ld8x4_sc1(a, r);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int i = i0 + (k * 64 + lane) * 4;
      if (i < n) *(u32x4*)(dst + i) = r[k];
    }
  }
}

// RMSNorm of the residual stream into LDS: xin = x / sqrt(mean(x^2) + eps) * gain.
// The source is the published fp32 residual, or the bf16 embedding row.
DEV void norm_input(const td_kparams& P, uint8_t* lds, const float* xsrc, const uint16_t* esrc,
                    const uint16_t* gain) {
  const int lane = lane_id();
  float* xin = (float*)(lds + P.off_xin);
  const int H = P.H;  // multiple of 256
  if (esrc) {
    for (int i = lane * 4; i < H; i += 256) {
      uint2 e = *(const uint2*)(esrc + i);
      f32x4 v = {bf_lo(e.x), bf_hi(e.x), bf_lo(e.y), bf_hi(e.y)};
      *(f32x4*)(xin + i) = v;
    }
  } else {
    load_vec_sc1(xsrc, H, xin);
  }
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
}

DEV void sync_prepare(const td_kparams& P, uint8_t* lds, int kind, int layer) {
  if (kind == TD_ST_QKV) {
    norm_input(P, lds, P.x, nullptr, P.layers[layer].attn_norm);
  } else if (kind == TD_ST_GU) {
    norm_input(P, lds, P.x, nullptr, P.layers[layer].mlp_norm);
  } else if (kind == TD_ST_HEAD) {
    norm_input(P, lds, P.x, nullptr, P.final_norm);
  } else if (kind == TD_ST_O) {
    load_vec_sc1(P.o, P.qd, (float*)(lds + P.off_xin));
  } else if (kind == TD_ST_DOWN) {
    load_vec_sc1(P.act, P.I, (float*)(lds + P.off_xin));
  } else {  // ATTN: the task's query heads, pre-scaled by 1/sqrt(d)
    const AttnTask T = attn_task(P, blockIdx.x);
    if (T.valid) {
      const td_attn_lds A = td_attn_layout(P.d, P.group);
      float* qs = (float*)(lds + P.off_attn + A.q);
      const int n = P.group * P.d;
      load_vec_sc1(P.q + (size_t)T.g * n, n, qs);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      for (int i = lane_id(); i < n; i += 64) qs[i] *= P.attn_scale;
    }
  }
}

// stage outputs -> epilogue -> published values
DEV void sync_epilogue(const td_kparams& P, uint8_t* lds, int kind, int layer, uint32_t epoch) {
  const int lane = lane_id();
  const int cu = blockIdx.x, ncu = gridDim.x;
  const float* out = (const float*)(lds + P.off_out);
  float* own = (float*)(lds + P.off_own);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (kind == TD_ST_QKV) {
    int u0, u1;
    cu_units(P.qkv_rows / 2, cu, ncu, u0, u1);
    const int half = P.d >> 1;
    const td_layer_dev& Ld = P.layers[layer];
    for (int k = lane; k < u1 - u0; k += 64) {
      const int u = u0 + k;
      const int ra = unit_row(P, TD_ST_QKV, u, 0), rb = ra + half;
      float a = out[2 * k], b = out[2 * k + 1];
      if (P.has_bias) {
        a += bf16f(Ld.bias[ra]);
        b += bf16f(Ld.bias[rb]);
      }
      const int i = ra % P.d;  // < d/2
      if (ra < P.qd + P.kvd) {  // q or k: rotate the pair
        const float* cs = P.rope_cs + ((size_t)P.pos * half + i) * 2;
        const float c = cs[0], s = cs[1];
        const float a2 = a * c - b * s;
        const float b2 = b * c + a * s;
        a = a2;
        b = b2;
      }
      if (ra < P.qd) {
        st_f(P.q + ra, a);
        st_f(P.q + rb, b);
      } else {
        const bool isk = ra < P.qd + P.kvd;
        const int g = (ra - P.qd - (isk ? 0 : P.kvd)) / P.d;
        uint16_t* cache = isk ? P.kc : P.vc;
        uint16_t* row = cache + (((size_t)layer * P.nkv + g) * P.max_ctx + P.pos) * P.d;
        st_u16_sc1(row + i, f2bf(a));
        st_u16_sc1(row + i + half, f2bf(b));
      }
    }
  } else if (kind == TD_ST_O || kind == TD_ST_DOWN) {
    int r0, r1;
    cu_units(P.H, cu, ncu, r0, r1);
    for (int k = lane; k < r1 - r0; k += 64) {
      float v = own[k] + out[k];
      own[k] = v;
      st_f(P.x + r0 + k, v);
    }
  } else if (kind == TD_ST_GU) {
    int u0, u1;
    cu_units(P.I, cu, ncu, u0, u1);
    for (int k = lane; k < u1 - u0; k += 64) {
      const float gt = out[2 * k], up = out[2 * k + 1];
      st_f(P.act + u0 + k, gt / (1.0f + expf(-gt)) * up);
    }
  } else if (kind == TD_ST_ATTN) {
    const AttnTask T = attn_task(P, cu);
    if (T.valid) {
      const int d = P.d, G = P.group;
      const td_attn_lds A = td_attn_layout(d, G);
      const float* pr = (const float*)(lds + P.off_attn + A.part);
      float* gp = P.part + ((size_t)T.g * P.n_chunks_max + T.c) * G * (d + 2);
      for (int i = lane; i < G * (d + 2); i += 64) st_f(gp + i, pr[i]);
      vm_drain();
      uint32_t* ctr = P.sync + TD_SY_MERGE + layer * P.nkv + T.g;
      int last = 0;
      if (lane == 0) last = atomicAdd(ctr, 1u) + 1u == (uint32_t)T.n_used;
      if (uni(last)) {
        // merge the n_used partials of this kv head: o = sum_c acc_c e^(m_c - M) / sum_c l_c e^(m_c - M)
        const float* base = P.part + (size_t)T.g * P.n_chunks_max * G * (d + 2);
        for (int h = 0; h < G; ++h) {
          float M = -__builtin_inff();
          for (int c = 0; c < T.n_used; ++c) M = fmaxf(M, ld_f(base + ((size_t)c * G + h) * (d + 2) + d));
          float Lsum = 0.f, o0 = 0.f, o1 = 0.f;
          for (int c = 0; c < T.n_used; ++c) {
            const float* pc = base + ((size_t)c * G + h) * (d + 2);
            const float wgt = expf(ld_f(pc + d) - M);
            Lsum = fmaf(ld_f(pc + d + 1), wgt, Lsum);
            o0 = fmaf(ld_f(pc + lane), wgt, o0);
            if (d > 64) o1 = fmaf(ld_f(pc + 64 + lane), wgt, o1);
          }
          float* dst = P.o + ((size_t)T.g * G + h) * d;
          st_f(dst + lane, o0 / Lsum);
          if (d > 64) st_f(dst + 64 + lane, o1 / Lsum);
        }
        if (lane == 0) st_u(ctr, 0u);
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
}

DEV void sync_wave(const td_kparams& P, uint8_t* lds) {
  const int lane = lane_id();
  const int cu = blockIdx.x, ncu = gridDim.x;
  const uint32_t epoch = uni(ld_u(P.sync + TD_SY_EPOCH));
  const uint32_t nbar = (uint32_t)(P.n_stages - 1);
  uint32_t gen = epoch * nbar;
  if (ld_u(P.sync + TD_SY_ABORT) && lane == 0) atomicOr(P.err, TD_ERRBIT_TIMEOUT);
  int tok = uni(*P.token_in);
  if (tok < 0 || tok >= P.V) {
    if (lane == 0 && cu == 0) atomicOr(P.err, TD_ERRBIT_RANGE);
    tok = 0;
  }
  const uint16_t* erow = P.embed + (size_t)tok * P.H;
  {  // this CU's residual rows start as the embedding row
    int r0, r1;
    cu_units(P.H, cu, ncu, r0, r1);
    float* own = (float*)(lds + P.off_own);
    for (int k = lane; k < r1 - r0; k += 64) own[k] = bf16f(erow[r0 + k]);
  }
  bool timed_out = false;
  for (int seq = 0; seq < P.n_stages; ++seq) {
    int kind, layer;
    stage_of(P, seq, kind, layer);
    if (kind == TD_ST_QKV && layer == 0) norm_input(P, lds, nullptr, erow, P.layers[0].attn_norm);
    else sync_prepare(P, lds, kind, layer);
    wg_bar();  // inputs ready
    if (kind == TD_ST_ATTN) attn_load_tiles(P, lds, layer);
    wg_bar();  // outputs ready
    sync_epilogue(P, lds, kind, layer, epoch);
    if (seq + 1 < P.n_stages) {
      vm_drain();
      if (!grid_barrier(P, gen)) timed_out = true;
      ++gen;
    }
  }
  if (timed_out && lane == 0) atomicOr(P.err, TD_ERRBIT_TIMEOUT);
}

template <int S>
__global__ void __launch_bounds__(TD_THREADS, 1) td_megakernel(td_kparams P) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int wave = uni((int)(threadIdx.x >> 6));
  if (wave < TD_NW) compute_wave<S>(P, lds, wave);
  else sync_wave(P, lds);
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
