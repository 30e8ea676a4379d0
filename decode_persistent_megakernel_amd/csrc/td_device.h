// td_device.h - device helpers shared by the persistent decode kernel
// (td_kernels.hip) and the per-op kernels (td_ops.hip): number formats, wave
// reductions, the chunk dot products and the attention tile update.  Both
// paths compute a GEMV row or an attention tile with exactly these routines.
#ifndef TD_DEVICE_H
#define TD_DEVICE_H
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "td.h"
#include "td_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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

// ------------------------------------------------------------ RMSNorm pieces
// RMSNorm is applied as y = inv * (W . (x * g)) with inv = 1 / sqrt(mean(x^2) +
// eps): the gains multiply the input elementwise, and the scalar inv multiplies
// each dot product.  mean(x^2) is summed in a fixed order: the input is cut
// into TD_NW slices (td_slice); within a slice, lane l adds the squares of the
// element pairs l, l + 64, ... in order and the lanes are summed by wave_sum;
// the slice sums are then added in slice order (norm_inv).
DEV float slice_ssq(const float* x, int lo, int hi) {
  float ss = 0.f;
  for (int u = (lo >> 1) + lane_id(); u < (hi >> 1); u += 64) {
    const float a = x[2 * u], b = x[2 * u + 1];
    ss = fmaf(a, a, ss);
    ss = fmaf(b, b, ss);
  }
  return wave_sum(ss);
}
DEV float norm_inv(const float* ssq, int H, float eps) {
  float s = ssq[0];
#pragma unroll
  for (int w = 1; w < TD_NW; ++w) s += ssq[w];
  return 1.0f / sqrtf(s / (float)H + eps);
}

// ------------------------------------------------------------ RoPE and greedy candidates
// Half-split rotary embedding of one pair (x_i, x_{i + d/2}) by the angle whose
// cosine and sine are c and sn (fp32, from the host-built table): the flint
// page's chat.py passage, out_i = x_i cos - x_{i + d/2} sin and
// out_{i + d/2} = x_{i + d/2} cos + x_i sin; products and sums rounded apart.
DEV void rope_pair(float& a, float& b, float c, float sn) {
  const float a2 = a * c - b * sn;
  const float b2 = b * c + a * sn;
  a = a2;
  b = b2;
}
// Greedy candidates ("Decoding in tiles", sec. 5: the largest logit, the lowest
// id among equal ones): (v, i) replaces (bv, bi) when it is better.
DEV bool cand_better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }
// The best candidate of the wave, on every lane.
DEV void cand_wave_max(float& bv, int& bi) {
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (cand_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
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
// 8 codes of one 32-bit word (element 2i in the low nibble of byte i) against
// the 8 matching activations; weight = scale * (code - 8), the scale applied by
// the caller.  The unpack makes two codes at a time into half-precision values
// without a conversion instruction: a code u placed in the low mantissa bits
// of the half-precision number 1024 (bits 0x6400) gives exactly 1024 + u, and
// one packed half-precision subtraction of 1032 leaves u - 8 exactly (the
// exponent-bit trick of tinyinfer's "v0.1" section, here on a pair of 16-bit
// halves).  Codes k and k + 4 of the word sit 16 bits apart, so one mask picks
// both.  Each fused multiply-add then takes its half-precision operand as is
// (v_fma_mix_f32: f32(u - 8) * x + s, one rounding).  Per word: 3 shifts, 4
// and-or, 4 packed subtractions and 8 multiply-adds, 19 vector instructions for
// 8 weights (2.4 per weight; a shift, a conversion, a subtraction and a
// multiply-add per weight before).  The products are added in element order,
// so the result is bit for bit the sum of fl((u_k - 8) x_k) in that order.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
DEV uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {  // (a & m) | c in one instruction
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}
DEV float dot_int4_word(uint32_t q, const float* x) {
  f32x4 a = *(const f32x4*)x;
  f32x4 b = *(const f32x4*)(x + 4);
  const uint32_t m = 0x000F000Fu, bias = 0x64006400u;
  const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 p0 = __builtin_bit_cast(f16x2, and_or(q, m, bias)) - off;        // codes 0, 4
  const f16x2 p1 = __builtin_bit_cast(f16x2, and_or(q >> 4, m, bias)) - off;   // codes 1, 5
  const f16x2 p2 = __builtin_bit_cast(f16x2, and_or(q >> 8, m, bias)) - off;   // codes 2, 6
  const f16x2 p3 = __builtin_bit_cast(f16x2, and_or(q >> 12, m, bias)) - off;  // codes 3, 7
  float s = (float)p0.x * a.x;
  s = fmaf((float)p1.x, a.y, s);
  s = fmaf((float)p2.x, a.z, s);
  s = fmaf((float)p3.x, a.w, s);
  s = fmaf((float)p0.y, b.x, s);
  s = fmaf((float)p1.y, b.y, s);
  s = fmaf((float)p2.y, b.z, s);
  s = fmaf((float)p3.y, b.w, s);
  return s;
}
// int4 chunk (2048 elements of a row): lane l holds four 8-code words, word w
// covering elements [512 w + 8 l, 512 w + 8 l + 8) (so the lanes of a wave read
// consecutive activations, free of LDS bank conflicts), in scale group
// 8 w + l / 8 of the chunk.  xc: the chunk's 2048 activations; sc: the lane's
// four scales as fp16 pairs (word 0 | word 1, word 2 | word 3).
DEV float dot_int4(u32x4 q, const float* xc, int lane, uint2 sc) {
  const float* x = xc + lane * 8;
  float s = f16f(sc.x) * dot_int4_word(q.x, x);
  s = fmaf(f16f(sc.x >> 16), dot_int4_word(q.y, x + 512), s);
  s = fmaf(f16f(sc.y), dot_int4_word(q.z, x + 1024), s);
  s = fmaf(f16f(sc.y >> 16), dot_int4_word(q.w, x + 1536), s);
  return s;
}
// Byte offset of word w of lane l inside an int4 chunk of a row-major row, and
// the scale group (within the chunk) of that word.
DEV int int4_word_off(int w, int lane) { return w * 256 + lane * 4; }
DEV int int4_word_group(int w, int lane) { return w * 8 + (lane >> 3); }
// A lane's four words of chunk j of a row-major int4 row of row_bytes bytes
// (code 8, a zero weight, past the row's end), and their four scales from the
// row's ngroups fp16 scales (0 past the end).
DEV u32x4 int4_words(const uint8_t* row, int row_bytes, int j, int lane) {
  uint32_t wd[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int off = j * 1024 + int4_word_off(w, lane);
    wd[w] = off < row_bytes ? *(const uint32_t*)(row + off) : 0x88888888u;
  }
  return (u32x4){wd[0], wd[1], wd[2], wd[3]};
}
// The packed stream keeps an int4 chunk's 32 scales in a 64-byte block ordered
// for the consumer: position p (0..31) holds the scale of word p & 3 of lanes
// 8 (p >> 2) .. 8 (p >> 2) + 7, so a lane's four scales are 8 consecutive bytes.
// int4_block_scale is the packing side (one position), int4_lane_scales the
// consuming side (word 0 | word 1 << 16, word 2 | word 3 << 16).
DEV uint16_t int4_block_scale(const uint16_t* srow, int ngroups, int j, int p) {
  const int g = j * 32 + int4_word_group(p & 3, (p >> 2) * 8);
  return g < ngroups ? srow[g] : (uint16_t)0;
}
DEV uint2 int4_lane_scales(const uint8_t* block, int lane) { return *(const uint2*)(block + (lane >> 3) * 8); }
DEV uint2 int4_scales(const uint16_t* srow, int ngroups, int j, int lane) {
  uint32_t h[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int g = j * 32 + int4_word_group(w, lane);
    h[w] = g < ngroups ? srow[g] : 0u;
  }
  return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

// ------------------------------------------------------------ attention tile
// One query head against one 64-row K/V tile in LDS (K rows padded to D + 8
// elements, V rows D elements, rows past nv zero), updating the online softmax
// state (m, l) and the unnormalised output ("One launch per token", "The
// attention trap"; "How I built an LLM inference engine", attention section).
// Scores: lane tau takes position tau.  P.V: lane (cg, pg) owns columns
// 4 cg .. 4 cg + 3 over the rows of position group pg; p is broadcast from LDS
// (ps, 64 floats of this wave); attn_finish sums the groups.
#define TD_TILE_ROWS 64
template <int D>
DEV void attn_tile(const float* qs, const uint16_t* kt, const uint16_t* vt, float* ps, int nv, float& m, float& l,
                   f32x4& acc) {
  constexpr int LPR = D / 4, NG = 64 / LPR, RPG = TD_TILE_ROWS / NG;
  const int lane = lane_id();
  const uint16_t* kr = kt + lane * (D + 8);
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < D; e += 8) {
    const u32x4 kw = *(const u32x4*)(kr + e);
    const f32x4 q0 = *(const f32x4*)(qs + e), q1 = *(const f32x4*)(qs + e + 4);
    a = fmaf(bf_lo(kw.x), q0.x, a);
    a = fmaf(bf_hi(kw.x), q0.y, a);
    a = fmaf(bf_lo(kw.y), q0.z, a);
    a = fmaf(bf_hi(kw.y), q0.w, a);
    a = fmaf(bf_lo(kw.z), q1.x, a);
    a = fmaf(bf_hi(kw.z), q1.y, a);
    a = fmaf(bf_lo(kw.w), q1.z, a);
    a = fmaf(bf_hi(kw.w), q1.w, a);
  }
  const float s = lane < nv ? a : -__builtin_inff();
  const float mn = fmaxf(m, wave_max(s));  // finite: nv >= 1
  const float p = __expf(s - mn);
  const float corr = __expf(m - mn);
  l = l * corr + wave_sum(p);
  m = mn;
  acc *= corr;
  ps[lane] = p;
  const int cg = lane % LPR, pg = lane / LPR;
  const uint16_t* vrow = vt + pg * RPG * D + cg * 4;
  const float* prow = ps + pg * RPG;
#pragma unroll
  for (int t = 0; t < RPG; t += 4) {
    const f32x4 p4 = *(const f32x4*)(prow + t);
    u32x2 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = *(const u32x2*)(vrow + (t + k) * D);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float pk = k == 0 ? p4.x : k == 1 ? p4.y : k == 2 ? p4.z : p4.w;
      acc.x = fmaf(pk, bf_lo(v[k].x), acc.x);
      acc.y = fmaf(pk, bf_hi(v[k].x), acc.y);
      acc.z = fmaf(pk, bf_lo(v[k].y), acc.z);
      acc.w = fmaf(pk, bf_hi(v[k].y), acc.w);
    }
  }
}

// The same update by one of W waves sharing a query head: this wave takes the
// tile's rows [s R, (s + 1) R), R = 64 / W, of which the first min(R, nv - s R)
// are positions (the caller skips a tile with none).  Scores: lane (r, part)
// with r = lane % R sums the dimensions [part D / W, (part + 1) D / W) of row
// s R + r, the W parts then added by butterfly shuffles; P.V as attn_tile over
// the wave's R rows (lane groups of RPG = R / (64 / (D / 4)) rows).
template <int D, int W>
DEV void attn_tile_w(const float* qs, const uint16_t* kt, const uint16_t* vt, float* ps, int nv, int s, float& m,
                     float& l, f32x4& acc) {
  constexpr int R = TD_TILE_ROWS / W, DPL = D / W, LPR = D / 4, NG = 64 / LPR, RPG = R / NG;
  static_assert(DPL % 8 == 0 && RPG % 4 == 0, "a wave's rows and dimensions come in whole loop steps");
  const int lane = lane_id();
  const int r0 = s * R, nr = min(R, nv - r0);
  const int r = lane % R, part = lane / R;
  const uint16_t* kr = kt + (r0 + r) * (D + 8) + part * DPL;
  const float* qp = qs + part * DPL;
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; e += 8) {
    const u32x4 kw = *(const u32x4*)(kr + e);
    const f32x4 q0 = *(const f32x4*)(qp + e), q1 = *(const f32x4*)(qp + e + 4);
    a = fmaf(bf_lo(kw.x), q0.x, a);
    a = fmaf(bf_hi(kw.x), q0.y, a);
    a = fmaf(bf_lo(kw.y), q0.z, a);
    a = fmaf(bf_hi(kw.y), q0.w, a);
    a = fmaf(bf_lo(kw.z), q1.x, a);
    a = fmaf(bf_hi(kw.z), q1.y, a);
    a = fmaf(bf_lo(kw.w), q1.z, a);
    a = fmaf(bf_hi(kw.w), q1.w, a);
  }
#pragma unroll
  for (int off = R; off < 64; off <<= 1) a += __shfl_xor(a, off);
  const float sc = r < nr ? a : -__builtin_inff();
  const float mn = fmaxf(m, wave_max(sc));  // finite: nr >= 1
  const float p = __expf(sc - mn);
  const float corr = __expf(m - mn);
  l = l * corr + wave_sum(part == 0 ? p : 0.f);
  m = mn;
  acc *= corr;
  if (part == 0) ps[r] = p;
  const int cg = lane % LPR, pg = lane / LPR;
  const uint16_t* vrow = vt + (r0 + pg * RPG) * D + cg * 4;
  const float* prow = ps + pg * RPG;
#pragma unroll
  for (int t = 0; t < RPG; t += 4) {
    const f32x4 p4 = *(const f32x4*)(prow + t);
    u32x2 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = *(const u32x2*)(vrow + (t + k) * D);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float pk = k == 0 ? p4.x : k == 1 ? p4.y : k == 2 ? p4.z : p4.w;
      acc.x = fmaf(pk, bf_lo(v[k].x), acc.x);
      acc.y = fmaf(pk, bf_hi(v[k].x), acc.y);
      acc.z = fmaf(pk, bf_lo(v[k].y), acc.z);
      acc.w = fmaf(pk, bf_hi(v[k].y), acc.w);
    }
  }
}
// One tile by wave s of W (W = 1: attn_tile itself); a wave whose share of the
// tile holds no position leaves its state as it is.
template <int D>
DEV void attn_tile_part(const float* qs, const uint16_t* kt, const uint16_t* vt, float* ps, int nv, int W, int s,
                        float& m, float& l, f32x4& acc) {
  if (W == 1) {
    attn_tile<D>(qs, kt, vt, ps, nv, m, l, acc);
  } else if (s * (TD_TILE_ROWS / W) < nv) {
    if (W == 2) attn_tile_w<D, 2>(qs, kt, vt, ps, nv, s, m, l, acc);
    else if (W == 4) attn_tile_w<D, 4>(qs, kt, vt, ps, nv, s, m, l, acc);
    else if constexpr (D >= 128) attn_tile_w<D, 8>(qs, kt, vt, ps, nv, s, m, l, acc);
  }
}

// Sums the position groups: afterwards lanes 0 .. D/4 - 1 hold the columns
// 4 lane .. 4 lane + 3.
template <int D>
DEV f32x4 attn_finish(f32x4 acc) {
#pragma unroll
  for (int off = D / 4; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  return acc;
}

// A wave's finished state (after attn_finish) for the head's first wave: D
// columns, then m and l, at st (LDS, D + 4 floats).
template <int D>
DEV void attn_sub_store(float* st, f32x4 acc, float m, float l) {
  const int lane = lane_id();
  if (lane < D / 4) *(f32x4*)(st + 4 * lane) = acc;
  if (lane == 0) {
    st[D] = m;
    st[D + 1] = l;
  }
}
// The head's first wave folds the states of waves 1 .. W - 1 (at sub, D + 4
// floats apart) into its own, in wave order, as one chunk's unnormalised state:
// M the largest m, acc = sum_s acc_s e^(m_s - M), l = sum_s l_s e^(m_s - M) (a
// wave without positions has m = -inf and adds nothing; the first wave always
// has some, so M is finite).  Lanes 0 .. D/4 - 1 carry acc.
template <int D>
DEV void attn_combine(f32x4& acc, float& m, float& l, const float* sub, int W) {
  const int lane = lane_id();
  float M = m;
  for (int k = 1; k < W; ++k) M = fmaxf(M, sub[(k - 1) * (D + 4) + D]);
  const float c0 = __expf(m - M);
  acc *= c0;
  float ls = l * c0;
  for (int k = 1; k < W; ++k) {
    const float* st = sub + (k - 1) * (D + 4);
    const float ck = __expf(st[D] - M);
    ls = fmaf(st[D + 1], ck, ls);
    if (lane < D / 4) {
      const f32x4 v = *(const f32x4*)(st + 4 * lane);
      acc.x = fmaf(ck, v.x, acc.x);
      acc.y = fmaf(ck, v.y, acc.y);
      acc.z = fmaf(ck, v.z, acc.z);
      acc.w = fmaf(ck, v.w, acc.w);
    }
  }
  m = M;
  l = ls;
}

// Split-K merge of one query head's chunk partials ("One launch per token",
// "The attention trap": each chunk's unnormalised output is rescaled by
// e^(m_c - M), M the largest chunk maximum, and divided by the rescaled sum of
// the l_c).  Chunk 0's state (acc, m, l) is the wave's own, after attn_finish;
// chunks 1 .. n-1 (n <= 64) are at mb + (c - 1) * (D + 4) in LDS: D output
// columns, then m and l.  ps (64 floats of LDS) takes the merge weights.
// Returns, on lanes 0 .. D/4 - 1, the merged output columns 4 lane .. 4 lane + 3;
// the chunks are added in chunk order.
template <int D>
DEV f32x4 attn_merge(f32x4 acc, float m, float l, const float* mb, int n, float* ps) {
  constexpr int st = D + 4;
  const int lane = lane_id();
  const bool have = lane < n;
  const float* pc = mb + (have && lane > 0 ? lane - 1 : 0) * st;
  const float mc = lane == 0 ? m : have ? pc[D] : -__builtin_inff();
  const float lc = lane == 0 ? l : have ? pc[D + 1] : 0.f;
  const float M = wave_max(mc);
  const float w0 = have ? __expf(mc - M) : 0.f;
  ps[lane] = w0 / wave_sum(lc * w0);  // the weights leave the lanes before the loop below
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (lane < D / 4) {
    const int e = 4 * lane;
    const float wc0 = ps[0];
    o.x = acc.x * wc0;
    o.y = acc.y * wc0;
    o.z = acc.z * wc0;
    o.w = acc.w * wc0;
    for (int c = 1; c < n; ++c) {
      const float wc = ps[c];
      const f32x4 v = *(const f32x4*)(mb + (c - 1) * st + e);
      o.x = fmaf(wc, v.x, o.x);
      o.y = fmaf(wc, v.y, o.y);
      o.z = fmaf(wc, v.z, o.z);
      o.w = fmaf(wc, v.w, o.w);
    }
  }
  return o;
}

// ------------------------------------------------------------ MoE routing
// moe_select (one wave): the router's choice from the E logits zs (LDS,
// padded with -inf to a multiple of 4).  The topk largest logits in decreasing
// order, the lower id first among equals: expert e takes slot rank(e), the
// number of experts with a larger logit or an equal one and a lower id, if that
// is below topk.  Their softmax probabilities over all E experts (max
// subtracted, the sum reduced in a fixed lane order) go to wts.  A non-finite
// logit gives ids 0 .. topk - 1 with weight 0 (every later read stays in
// bounds) and returns true.  Every caller computes the same bits from the same
// logits.
DEV bool moe_select(int E, int topk, const float* zs, int32_t* ids, float* wts) {
  constexpr int PER = TD_MAX_EXPERTS / 64;
  const int lane = lane_id();
  float z[PER];
  float m = -__builtin_inff();
  int bad = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    z[i] = zs[e];
    if (e < E && !isfinite(z[i])) bad = 1;
    if (e < E) m = fmaxf(m, z[i]);
  }
  bad = __any(bad);
  m = wave_max(m);
  float ssum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + 64 * i < E) ssum += expf(z[i] - m);
  ssum = wave_sum(ssum);
  if (bad) {
    if (lane < topk) {
      ids[lane] = lane;
      wts[lane] = 0.f;
    }
    return true;
  }
  const int E4 = (E + 3) & ~3;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (64 * i >= E) break;
    const int e = lane + 64 * i;
    int rank = 0;
    for (int c = 0; c < E4; c += 4) {  // the same address in every lane: a broadcast read
      const f32x4 q = *(const f32x4*)(zs + c);
      rank += (q.x > z[i] || (q.x == z[i] && c < e)) + (q.y > z[i] || (q.y == z[i] && c + 1 < e)) +
              (q.z > z[i] || (q.z == z[i] && c + 2 < e)) + (q.w > z[i] || (q.w == z[i] && c + 3 < e));
    }
    if (e < E && rank < topk) {
      ids[rank] = e;
      wts[rank] = expf(z[i] - m) / ssum;
    }
  }
  return false;
}


}  // namespace

#endif
