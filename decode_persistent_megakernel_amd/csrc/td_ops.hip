// td_ops.hip - the per-op executor: the decode step as one kernel launch per
// fused op, the baseline the persistent kernel is measured against ("Decoding
// in tiles", sec. 1 and 6: one kernel per step with launch gaps and tails;
// "One launch per token": the same ops captured in a graph).  The arithmetic
// is the persistent kernel's own: the same chunk dot products over the same
// 1 KiB chunks in the same order, the same RMSNorm, RoPE, attention tile,
// merge and argmax, so both executors give the same bits.  Activations live
// in plain device buffers; kernel boundaries order the ops.
//
// Per layer: op_qkv (RMSNorm + QKV GEMV + bias + RoPE + K/V write), op_attn
// (split-K partials), op_merge, op_o (+ residual), op_gu (RMSNorm + gate/up +
// SwiGLU), op_down (+ residual); then op_head (final RMSNorm + logits + block
// candidates) and op_argmax.  A mixture-of-experts layer replaces op_gu and
// op_down with op_router (RMSNorm + router logits), op_moe_gu (top-k choice +
// the chosen experts' gate/up + SwiGLU) and op_moe_down (the chosen experts'
// down rows, weighted, + residual).  op_begin (token, range check, embedding row,
// position word) runs first and is the only launch that carries the step's
// arguments, so the rest can be captured once and replayed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "td.h"
#include "td_internal.h"
#include "td_device.h"

namespace {

constexpr int OP_WAVES = 4;  // waves per workgroup of the GEMV ops

// Staging into LDS.  A thread's share of a vector is the 4-float groups
// t, t + T, ... (T threads); all of a thread's loads of a batch of NV groups
// are issued before its first LDS store, from clamped addresses so every load
// is unconditional, and a block pays one load round trip per batch instead of
// one per element.  Lengths are multiples of 4 floats and buffers 16-byte
// aligned (the config and weight checks enforce both).

// RMSNorm of x [H] in the persistent kernel's form: xs = x * gain in LDS, and
// the returned inv = 1 / sqrt(mean(x^2) + eps) (the caller multiplies each dot
// product by it), mean(x^2) summed over the same TD_NW slices in the same order
// (slice_ssq, norm_inv).  With H <= 4 NV T the gains are loaded with x and
// held in registers across the sum of squares.  With zsrc, wave 0 also copies
// the zn router logits zsrc to zs [TD_MAX_EXPERTS], padded with -inf, their
// loads in flight with its share of x.  Needs blockDim.x >= 64.
template <int NV>
DEV float op_norm_to_lds_n(const float* x, const uint16_t* gain, int H, float eps, float* xs, float* red,
                           const float* zsrc, int zn, float* zs) {
  constexpr int ZPER = TD_MAX_EXPERTS / 64;
  const int t = threadIdx.x, T = blockDim.x, wave = t >> 6, nwaves = T >> 6;
  const int n4 = H >> 2;
  f32x4 v[NV];
  uint2 g[NV];
  float z[ZPER];
  for (int b = 0; b < n4; b += NV * T) {
    if (b == 0 && zsrc && wave == 0) {
#pragma unroll
      for (int i = 0; i < ZPER; ++i) z[i] = zsrc[min(t + 64 * i, zn - 1)];
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int i = min(b + u * T + t, n4 - 1);
      v[u] = *(const f32x4*)(x + 4 * i);
      g[u] = *(const uint2*)(gain + 4 * i);
    }
#pragma unroll
    for (int u = 0; u < NV; ++u)
      if (b + u * T + t < n4) *(f32x4*)(xs + 4 * (b + u * T + t)) = v[u];
    if (b == 0 && zsrc && wave == 0) {
#pragma unroll
      for (int i = 0; i < ZPER; ++i) zs[t + 64 * i] = t + 64 * i < zn ? z[i] : -__builtin_inff();
    }
  }
  __syncthreads();
  for (int w = wave; w < TD_NW; w += nwaves) {
    int lo, hi;
    td_slice(H, w, &lo, &hi);
    const float ss = slice_ssq(xs, lo, hi);
    if (lane_id() == 0) red[w] = ss;
  }
  __syncthreads();  // every slice sum is in red and no wave reads xs again
  const float inv = norm_inv(red, H, eps);
  for (int b = 0; b < n4; b += NV * T) {
    if (n4 > NV * T) {  // several batches: the gains and x of this one again
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int i = min(b + u * T + t, n4 - 1);
        v[u] = *(const f32x4*)(xs + 4 * i);
        g[u] = *(const uint2*)(gain + 4 * i);
      }
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int i = b + u * T + t;
      if (i >= n4) continue;
      f32x4 a = v[u];
      a.x *= bf_lo(g[u].x);
      a.y *= bf_hi(g[u].x);
      a.z *= bf_lo(g[u].y);
      a.w *= bf_hi(g[u].y);
      *(f32x4*)(xs + 4 * i) = a;
    }
  }
  return inv;
}

DEV float op_norm_to_lds(const float* x, const uint16_t* gain, int H, float eps, float* xs, float* red,
                         const float* zsrc = nullptr, int zn = 0, float* zs = nullptr) {
  const int per = (H / 4 + (int)blockDim.x - 1) / (int)blockDim.x;
  if (per <= 2) return op_norm_to_lds_n<2>(x, gain, H, eps, xs, red, zsrc, zn, zs);
  if (per <= 4) return op_norm_to_lds_n<4>(x, gain, H, eps, xs, red, zsrc, zn, zs);
  return op_norm_to_lds_n<8>(x, gain, H, eps, xs, red, zsrc, zn, zs);
}

// Copies `rows` vectors of n floats (row j at src + j n) to LDS at xs + j kp,
// each zero-filled from n up to kp.
template <int NV>
DEV void op_stage_rows_n(const float* src, int rows, int n, int kp, float* xs) {
  const int t = threadIdx.x, T = blockDim.x;
  const int n4 = n >> 2, k4 = kp >> 2, tot = rows * k4;
  for (int b = 0; b < tot; b += NV * T) {
    f32x4 v[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int i = min(b + u * T + t, tot - 1);
      const int r = i / k4, c = i - r * k4;
      v[u] = *(const f32x4*)(src + (size_t)r * n + 4 * min(c, n4 - 1));
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int i = b + u * T + t;
      if (i >= tot) continue;
      const int r = i / k4, c = i - r * k4;
      *(f32x4*)(xs + 4 * i) = c < n4 ? v[u] : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  }
}

DEV void op_stage_rows(const float* src, int rows, int n, int kp, float* xs) {
  const int per = (rows * (kp >> 2) + (int)blockDim.x - 1) / (int)blockDim.x;
  if (per <= 2) op_stage_rows_n<2>(src, rows, n, kp, xs);
  else if (per <= 4) op_stage_rows_n<4>(src, rows, n, kp, xs);
  else op_stage_rows_n<8>(src, rows, n, kp, xs);
}

DEV void op_zero_tail(float* xs, int from, int to) {
  for (int i = from + (int)threadIdx.x; i < to; i += blockDim.x) xs[i] = 0.f;
}

DEV int op_kpad(int K, int fmt) {
  const int ce = fmt ? 2048 : 512;
  return (K + ce - 1) / ce * ce;
}

// One row of a stored linear against xs (LDS): the chunk loop of the
// persistent kernel, reading the row's chunks straight from the caller's
// row-major weights (a chunk column past the row end reads as zero weights).
template <int fmt>
DEV float op_row_f(const uint8_t* w, const uint16_t* s, int row, int K, const float* xs) {
  const int lane = lane_id();
  const int row_bytes = fmt == 0 ? K * 2 : K / 2;
  const int J = (row_bytes + TD_CHUNK - 1) / TD_CHUNK;
  const uint8_t* rp = w + (size_t)row * row_bytes;
  float acc = 0.f;
  for (int j0 = 0; j0 < J; j0 += 4) {
    u32x4 c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (fmt == 0) {
        const int boff = (j0 + u) * TD_CHUNK + lane * 16;
        c[u] = (j0 + u < J && boff < row_bytes) ? __builtin_nontemporal_load((const u32x4*)(rp + boff))
                                                : (u32x4){0u, 0u, 0u, 0u};
      } else {
        c[u] = int4_words(rp, row_bytes, j0 + u, lane);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u;
      if (j >= J) break;
      if (fmt == 0) acc += dot_bf16(c[u], xs + j * 512 + lane * 8);
      else acc += dot_int4(c[u], xs + j * 2048, lane, int4_scales(s + (size_t)row * (K / 64), K / 64, j, lane));
    }
  }
  return wave_sum(acc);
}

// the format as a template parameter: each chunk loop is compiled for one format
DEV float op_row(int fmt, const uint8_t* w, const uint16_t* s, int row, int K, const float* xs) {
  return fmt ? op_row_f<1>(w, s, row, K, xs) : op_row_f<0>(w, s, row, K, xs);
}

// Row `row` of nr <= NR different matrices w[i] (scales s[i]) against nr
// different LDS vectors xs + i xs_stride, their chunks loaded together (two
// chunks of every row per round) so that one wave keeps NR rows in flight;
// each dot product adds its chunks in the order op_row_f does (same bits).
// Every w[i] must point at a valid matrix (callers repeat a valid one past nr):
// the bf16 loads are unconditional from clamped addresses and the unused
// values are zeroed afterwards, so the compiler's wait counts stay exact and
// all loads of a round are in flight together.
template <int fmt, int NR>
DEV void op_rows_multi(const uint8_t* const (&w)[NR], const uint16_t* const (&s)[NR], int nr, int row, int K,
                       const float* xs, int xs_stride, float (&out)[NR]) {
  const int lane = lane_id();
  const int row_bytes = fmt == 0 ? K * 2 : K / 2;
  const int J = (row_bytes + TD_CHUNK - 1) / TD_CHUNK;
  float acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < J; j0 += 2) {
    u32x4 c[NR][2];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const uint8_t* rp = w[i] + (size_t)row * row_bytes;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + u;
        const bool ok = i < nr && j < J;
        if (fmt == 0) {
          const int boff = j * TD_CHUNK + lane * 16;
          const u32x4 v = __builtin_nontemporal_load((const u32x4*)(rp + min(boff, row_bytes - 16)));
          const bool use = ok && boff < row_bytes;
          c[i][u] = (u32x4){use ? v.x : 0u, use ? v.y : 0u, use ? v.z : 0u, use ? v.w : 0u};
        } else {
          c[i][u] = ok ? int4_words(rp, row_bytes, j, lane) : (u32x4){0x88888888u, 0x88888888u, 0x88888888u,
                                                                      0x88888888u};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + u;
        if (i >= nr || j >= J) continue;
        const float* x = xs + (size_t)i * xs_stride;
        if (fmt == 0) acc[i] += dot_bf16(c[i][u], x + j * 512 + lane * 8);
        else acc[i] += dot_int4(c[i][u], x + j * 2048, lane, int4_scales(s[i] + (size_t)row * (K / 64), K / 64, j, lane));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) out[i] = wave_sum(acc[i]);
}

DEV int op_unit_row_qkv(const td_opparams& P, int u, int r) {
  const int half = P.d >> 1;
  const int head = u / half;
  const int i = u - head * half;
  return head * P.d + i + r * half;
}

// --------------------------------------------------------------- op_begin
__global__ void __launch_bounds__(256) op_begin(td_opparams P, const int32_t* d_token, int32_t pos) {
  __shared__ int tok_s;
  if (threadIdx.x == 0) {
    int tok = *d_token;
    if (tok < 0 || tok >= P.V) {
      atomicOr(P.err, TD_ERRBIT_RANGE);
      tok = 0;
    }
    tok_s = tok;
    *P.pos_word = pos;
  }
  __syncthreads();
  const uint16_t* e = P.embed + (size_t)tok_s * P.H;
  for (int i = threadIdx.x; i < P.H; i += blockDim.x) P.x[i] = bf16f(e[i]);
}

// --------------------------------------------------------------- op_qkv
__global__ void __launch_bounds__(256) op_qkv(td_opparams P, int layer, int R) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* xs = (float*)lds;
  const td_layer_dev& Ld = P.layers[layer];
  const float inv = op_norm_to_lds(P.x, Ld.attn_norm, P.H, P.eps, xs, xs + op_kpad(P.H, P.wf));
  op_zero_tail(xs, P.H, op_kpad(P.H, P.wf));
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int pos = *P.pos_word;
  const int half = P.d >> 1;
  const int U = P.qkv_rows / 2;
  for (int k = 0; k < R; ++k) {
    const int u = (blockIdx.x * OP_WAVES + wave) * R + k;
    if (u >= U) break;
    const int ra = op_unit_row_qkv(P, u, 0), rb = ra + half;
    float a = op_row(P.wf, Ld.w[0], Ld.s[0], ra, P.H, xs) * inv;
    float b = op_row(P.wf, Ld.w[0], Ld.s[0], rb, P.H, xs) * inv;
    if (lane != 0) continue;
    if (P.has_bias) {
      a += bf16f(Ld.bias[ra]);
      b += bf16f(Ld.bias[rb]);
    }
    const int i = ra % P.d;
    if (ra < P.qd + P.kvd) {  // q or k: rotate the pair by pos * theta_i
      const size_t rr = (size_t)(pos - P.rope_pos0) * half + i;
      rope_pair(a, b, P.rope_cs[rr * 2], P.rope_cs[rr * 2 + 1]);
    }
    if (ra < P.qd) {
      P.q[ra] = a * P.attn_scale;
      P.q[rb] = b * P.attn_scale;
    } else {
      const bool isk = ra < P.qd + P.kvd;
      const int g = (ra - P.qd - (isk ? 0 : P.kvd)) / P.d;
      uint16_t* row = (isk ? P.kc : P.vc) + (((size_t)layer * P.nkv + g) * P.max_ctx + pos) * P.d;
      row[i] = (uint16_t)f2bf(a);
      row[i + half] = (uint16_t)f2bf(b);
    }
  }
}

// --------------------------------------------------------------- op_attn
// Workgroup (g, c): kv head g, positions of chunk c; all 8 waves load the
// tiles, and wave w < group W runs rows [s 64 / W, (s + 1) 64 / W) of every
// tile for query head g * group + w % group (s = w / group; W = td_attn_waves,
// as in the persistent kernel: 1 but for a MoE model with one query head per kv
// head), the head's W states then folded in wave order by its first wave: the
// persistent kernel's routines in its order.
template <int D>
__global__ void __launch_bounds__(512) op_attn(td_opparams P, int layer) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int pos = *P.pos_word;
  const int G = P.group;
  const int g = blockIdx.x / P.n_chunks_max, c = blockIdx.x - g * P.n_chunks_max;
  const int n_used = (pos + P.chunk_len) / P.chunk_len;
  if (c >= n_used) return;
  const int t0 = c * P.chunk_len, t1 = min(t0 + P.chunk_len, pos + 1);
  const int W = td_attn_waves(D, G, P.E > 0);
  float* qs = (float*)lds;                                             // [G][D]
  float* ps = qs + G * D;                                              // [G W][64]
  uint16_t* kt = (uint16_t*)(ps + G * W * TD_TILE_ROWS);               // [64][D + 8]
  uint16_t* vt = kt + TD_TILE_ROWS * (D + 8);                          // [64][D]
  float* sub = (float*)(vt + TD_TILE_ROWS * D);                        // [G][W - 1][D + 4]
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int h = wave % G, s = wave / G;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) qs[i] = P.q[(size_t)g * G * D + i];
  const size_t head_off = ((size_t)layer * P.nkv + g) * P.max_ctx;
  float m = -__builtin_inff(), l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int Q16 = D / 8;  // 16-byte pieces per row
  for (int tb = t0; tb < t1; tb += TD_TILE_ROWS) {
    const int nv = min(TD_TILE_ROWS, t1 - tb);
    __syncthreads();  // previous tile consumed
    for (int i = threadIdx.x; i < TD_TILE_ROWS * Q16; i += blockDim.x) {
      const int row = i / Q16, pc = i - row * Q16;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (row < nv) {
        kv = *(const u32x4*)(P.kc + (head_off + tb + row) * D + pc * 8);
        vv = *(const u32x4*)(P.vc + (head_off + tb + row) * D + pc * 8);
      }
      *(u32x4*)(kt + row * (D + 8) + pc * 8) = kv;
      *(u32x4*)(vt + row * D + pc * 8) = vv;
    }
    __syncthreads();  // tile in LDS
    if (wave < G * W) attn_tile_part<D>(qs + h * D, kt, vt, ps + wave * TD_TILE_ROWS, nv, W, s, m, l, acc);
  }
  if (wave < G * W) acc = attn_finish<D>(acc);
  if (W > 1) {
    if (wave < G * W && s > 0) attn_sub_store<D>(sub + ((size_t)h * (W - 1) + s - 1) * (D + 4), acc, m, l);
    __syncthreads();
    if (wave < G) attn_combine<D>(acc, m, l, sub + (size_t)h * (W - 1) * (D + 4), W);
  }
  if (wave < G) {
    float* pr = P.part + (((size_t)g * G + wave) * P.n_chunks_max + c) * (D + 4);
    if (lane < D / 4) *(f32x4*)(pr + 4 * lane) = acc;
    if (lane == 0) *(f32x4*)(pr + D) = f32x4{m, l, 0.f, 0.f};
  }
}

// --------------------------------------------------------------- op_merge
// Workgroup g, wave h: o = sum_c acc_c w_c with w_c = e^(m_c - M) / sum l e^(m - M),
// chunk 0 first, the others fused in chunk order.
template <int D>
__global__ void __launch_bounds__(512) op_merge(td_opparams P) {
  const int pos = *P.pos_word;
  const int G = P.group, g = blockIdx.x, h = threadIdx.x >> 6, lane = lane_id();
  if (h >= G) return;
  const int n = (pos + P.chunk_len) / P.chunk_len;  // <= 64
  const float* base = P.part + ((size_t)g * G + h) * P.n_chunks_max * (D + 4);
  auto part = [&](int c) { return base + (size_t)c * (D + 4); };
  const bool have = lane < n;
  const float* own = part(have ? lane : 0);
  const float mm = have ? own[D] : -__builtin_inff();
  const float ll = have ? own[D + 1] : 0.f;
  const float M = wave_max(mm);
  const float w0 = have ? __expf(mm - M) : 0.f;
  __shared__ float wl[8][64];  // the weights leave the lanes before the loop below diverges
  wl[h][lane] = w0 / wave_sum(ll * w0);
  for (int e = lane * 4; e < D; e += 256) {
    const float wc0 = wl[h][0];
    const f32x4 p0 = *(const f32x4*)(part(0) + e);
    f32x4 o;
    o.x = p0.x * wc0;
    o.y = p0.y * wc0;
    o.z = p0.z * wc0;
    o.w = p0.w * wc0;
    for (int c = 1; c < n; ++c) {
      const float wc = wl[h][c];
      const f32x4 v = *(const f32x4*)(part(c) + e);
      o.x = fmaf(wc, v.x, o.x);
      o.y = fmaf(wc, v.y, o.y);
      o.z = fmaf(wc, v.z, o.z);
      o.w = fmaf(wc, v.w, o.w);
    }
    *(f32x4*)(P.o + ((size_t)g * G + h) * D + e) = o;
  }
}

// --------------------------------------------------------------- op_o / op_down
// x[r] += W[r] . in (in = o for the output projection, act for the down projection)
__global__ void __launch_bounds__(256) op_resid(td_opparams P, int layer, int which, int R) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* xs = (float*)lds;
  const td_layer_dev& Ld = P.layers[layer];
  const int K = which == 1 ? P.qd : P.I;
  op_stage_rows(which == 1 ? P.o : P.act, 1, K, op_kpad(K, P.wf), xs);
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  for (int k = 0; k < R; ++k) {
    const int r = (blockIdx.x * OP_WAVES + wave) * R + k;
    if (r >= P.H) break;
    const float y = op_row(P.wf, Ld.w[which], Ld.s[which], r, K, xs);
    if (lane_id() == 0) P.x[r] = P.x[r] + y;
  }
}

// --------------------------------------------------------------- op_gu
__global__ void __launch_bounds__(256) op_gu(td_opparams P, int layer, int R) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* xs = (float*)lds;
  const td_layer_dev& Ld = P.layers[layer];
  const float inv = op_norm_to_lds(P.x, Ld.mlp_norm, P.H, P.eps, xs, xs + op_kpad(P.H, P.wf));
  op_zero_tail(xs, P.H, op_kpad(P.H, P.wf));
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  for (int k = 0; k < R; ++k) {
    const int u = (blockIdx.x * OP_WAVES + wave) * R + k;
    if (u >= P.I) break;
    const float gt = op_row(P.wf, Ld.w[2], Ld.s[2], u, P.H, xs) * inv;
    const float up = op_row(P.wf, Ld.w[2], Ld.s[2], u + P.I, P.H, xs) * inv;
    if (lane_id() == 0) P.act[u] = gt / (1.0f + expf(-gt)) * up;
  }
}

// --------------------------------------------------------------- MoE
// A mixture-of-experts MLP ("One launch per token", its 64-expert section):
// the router writes the chosen expert ids into a fixed device tensor and the
// expert kernels read their weights through it, so the launches (and a graph
// recorded from them) never change while the routing does.

// op_router: z[e] = W_router[e] . RMSNorm(x) for every expert e (bf16 rows,
// the chunk arithmetic of the other GEMVs), one expert per wave.
__global__ void __launch_bounds__(256) op_router(td_opparams P, int layer) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* xs = (float*)lds;
  const td_layer_dev& Ld = P.layers[layer];
  const float inv = op_norm_to_lds(P.x, Ld.mlp_norm, P.H, P.eps, xs, xs + op_kpad(P.H, 0));
  op_zero_tail(xs, P.H, op_kpad(P.H, 0));
  __syncthreads();
  const int e = blockIdx.x * OP_WAVES + (threadIdx.x >> 6);
  if (e >= P.E) return;
  const float z = op_row(0, (const uint8_t*)Ld.router, nullptr, e, P.H, xs) * inv;
  if (lane_id() == 0) P.rlogits[e] = z;
}

// Expert e's block of a stacked [E][rows][K] linear (codes and scales).
DEV const uint8_t* expert_w(const uint8_t* w, int fmt, int e, int rows, int K) {
  return w + (size_t)e * rows * (fmt ? (size_t)(K / 2) : (size_t)K * 2);
}
DEV const uint16_t* expert_s(const uint16_t* s, int fmt, int e, int rows, int K) {
  return fmt ? s + (size_t)e * rows * (K / 64) : nullptr;
}

// op_moe_gu: unit u = j I + r: row r of the j-th chosen expert's gate and up
// projections of RMSNorm(x), act[j][r] = SiLU(gate) * up.  Wave 0 of every
// block stages the router logits with x and makes the router's choice
// (moe_select) while the other waves finish the norm;
// block 0 publishes it in expert_ids[layer] and expert_w[layer] for op_moe_down
// and the caller, and raises the error bit on a non-finite router logit.
__global__ void __launch_bounds__(256) op_moe_gu(td_opparams P, int layer, int R) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ __attribute__((aligned(16))) float zs[TD_MAX_EXPERTS];
  __shared__ int32_t sid[TD_MAX_TOPK];
  __shared__ float swt[TD_MAX_TOPK];
  float* xs = (float*)lds;
  const td_layer_dev& Ld = P.layers[layer];
  const int wave = threadIdx.x >> 6;
  const float inv = op_norm_to_lds(P.x, Ld.mlp_norm, P.H, P.eps, xs, xs + op_kpad(P.H, P.wf), P.rlogits, P.E, zs);
  bool bad = false;
  if (wave == 0) bad = moe_select(P.E, P.topk, zs, sid, swt);
  op_zero_tail(xs, P.H, op_kpad(P.H, P.wf));
  __syncthreads();
  if (blockIdx.x == 0 && wave == 0) {
    const int lane = lane_id();
    if (lane < P.topk) {
      P.expert_ids[layer * P.topk + lane] = sid[lane];
      P.expert_w[layer * P.topk + lane] = swt[lane];
    }
    if (bad && lane == 0) atomicOr(P.err, TD_ERRBIT_NONFINITE);
  }
  for (int k = 0; k < R; ++k) {
    const int u = (blockIdx.x * OP_WAVES + wave) * R + k;
    if (u >= P.topk * P.I) break;
    const int j = u / P.I, r = u - j * P.I;
    const int e = uni(sid[j]);
    const uint8_t* w = expert_w(Ld.w[2], P.wf, e, 2 * P.I, P.H);
    const uint16_t* sc = expert_s(Ld.s[2], P.wf, e, 2 * P.I, P.H);
    const float gt = op_row(P.wf, w, sc, r, P.H, xs) * inv;
    const float up = op_row(P.wf, w, sc, r + P.I, P.H, xs) * inv;
    if (lane_id() == 0) P.act[u] = gt / (1.0f + expf(-gt)) * up;
  }
}

// op_moe_down: x[r] += sum over the chosen experts j (in order) of
// w_j (W_down of expert j, row r) . act[j].
__global__ void __launch_bounds__(256) op_moe_down(td_opparams P, int layer, int R) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* xs = (float*)lds;
  const td_layer_dev& Ld = P.layers[layer];
  const int kp = op_kpad(P.I, P.wf);
  op_stage_rows(P.act, P.topk, P.I, kp, xs);
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  const int32_t* ids = P.expert_ids + layer * P.topk;
  const float* wts = P.expert_w + layer * P.topk;
  for (int k = 0; k < R; ++k) {
    const int r = (blockIdx.x * OP_WAVES + wave) * R + k;
    if (r >= P.H) break;
    float y = 0.f;
    for (int g0 = 0; g0 < P.topk; g0 += 8) {  // eight experts' rows in flight at a time
      const int nr = min(8, P.topk - g0);
      const uint8_t* wp[8];
      const uint16_t* sp[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = uni(ids[min(g0 + i, P.topk - 1)]);
        wp[i] = expert_w(Ld.w[3], P.wf, e, P.H, P.I);
        sp[i] = expert_s(Ld.s[3], P.wf, e, P.H, P.I);
      }
      float d[8];
      if (P.wf) op_rows_multi<1, 8>(wp, sp, nr, r, P.I, xs + (size_t)g0 * kp, kp, d);
      else op_rows_multi<0, 8>(wp, sp, nr, r, P.I, xs + (size_t)g0 * kp, kp, d);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < nr) y = fmaf(wts[g0 + i], d[i], y);
    }
    if (lane_id() == 0) P.x[r] = P.x[r] + y;
  }
}

// --------------------------------------------------------------- op_head / op_argmax
__global__ void __launch_bounds__(256) op_head(td_opparams P, int R) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* xs = (float*)lds;
  __shared__ float cv[OP_WAVES];
  __shared__ int ci[OP_WAVES], cb[OP_WAVES];
  const float inv = op_norm_to_lds(P.x, P.final_norm, P.H, P.eps, xs, xs + op_kpad(P.H, 0));
  op_zero_tail(xs, P.H, op_kpad(P.H, 0));
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = lane_id();
  float bv = -__builtin_inff();
  int bi = 0x7fffffff, bad = 0;
  for (int k = 0; k < R; ++k) {
    const int r = (blockIdx.x * OP_WAVES + wave) * R + k;
    if (r >= P.V) break;
    const float v = op_row(0, (const uint8_t*)P.head, nullptr, r, P.H, xs) * inv;
    if (lane == 0) P.logits[r] = v;
    if (!isfinite(v)) bad = 1;
    else if (v > bv) { bv = v; bi = r; }
  }
  if (lane == 0) {
    cv[wave] = bv;
    ci[wave] = bi;
    cb[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < OP_WAVES; ++w) {
      if (cv[w] > bv || (cv[w] == bv && ci[w] < bi)) { bv = cv[w]; bi = ci[w]; }
      bad |= cb[w];
    }
    P.cand[blockIdx.x * 4 + 0] = __float_as_uint(bv);
    P.cand[blockIdx.x * 4 + 1] = (uint32_t)bi;
    P.cand[blockIdx.x * 4 + 2] = (uint32_t)bad;
  }
}

__global__ void __launch_bounds__(64) op_argmax(td_opparams P, int nblocks) {
  const int lane = lane_id();
  float fv = -__builtin_inff();
  int fi = 0x7fffffff, fbad = 0;
  for (int c = lane; c < nblocks; c += 64) {
    const float v = __uint_as_float(P.cand[c * 4 + 0]);
    const int i = (int)P.cand[c * 4 + 1];
    fbad |= (int)P.cand[c * 4 + 2];
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
  }
}

// --------------------------------------------------------------- the no-allocation step
// Writes one launch's share of the layer table (and, with write_rope, the
// step's RoPE row and a cleared error word) into the scratch array.
__global__ void __launch_bounds__(64) op_noalloc_setup(td_noalloc_setup a, td_layer_dev* table, float* rope_row,
                                                       int32_t* err) {
  const int t = threadIdx.x;
  if (t < a.n) table[a.first + t] = a.layers[t];
  if (a.write_rope) {
    for (int i = t; i < a.d; i += 64) rope_row[i] = a.rope.cs[i];
    if (t == 0) *err = 0;
  }
}

}  // namespace

// The scratch of td_decode_step_noalloc: activations, attention partials,
// greedy candidates, the layer table and the step's RoPE row of the per-op
// kernels, for callers that cannot allocate.  Each device holds its own copy
// for the life of the process; host code reaches it only through the address
// hipGetSymbolAddress returns on that device (the array's name is a host-side
// stand-in, not a device address).  Every call on a device shares the copy, so
// calls that overlap on one device race.
static __device__ __align__(256) uint8_t scratch[TD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int TD_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[TD_MAX_DEVICES] = {};
}  // namespace

// This device's copy of the scratch array (looked up once per device, with the
// device current).
int td_noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= TD_MAX_DEVICES) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

int td_launch_noalloc_setup(const td_noalloc_setup& a, td_layer_dev* table, float* rope_row, int32_t* err,
                            void* stream) {
  op_noalloc_setup<<<1, 64, 0, (hipStream_t)stream>>>(a, table, rope_row, err);
  return (int)hipGetLastError();
}

// --------------------------------------------------------------- launchers
namespace {
constexpr int R_QKV = 1, R_RESID = 1, R_GU = 4, R_HEAD = 16, R_MOE_GU = 2, R_MOE_DOWN = 1;
int blocks_for(int units, int r) { return (units + OP_WAVES * r - 1) / (OP_WAVES * r); }
}  // namespace

int td_op_head_blocks(const td_opparams* p) { return blocks_for(p->V, R_HEAD); }

// op_attn's LDS: queries, one probability row a wave, the tile, the head's wave
// states (td_attn_waves).  It has its own size, so that the other kernels' LDS
// (and their workgroups per CU) does not grow with the wave split.
static size_t op_attn_lds_bytes(const td_opparams* p, size_t W) {
  const size_t D = (size_t)p->d, G = (size_t)p->group;
  return G * D * 4 + G * W * TD_TILE_ROWS * 4 + TD_TILE_ROWS * (D + 8) * 2 + TD_TILE_ROWS * D * 2 +
         G * (W - 1) * (D + 4) * 4;
}
static size_t op_attn_lds_bytes(const td_opparams* p) {
  return op_attn_lds_bytes(p, (size_t)td_attn_waves(p->d, p->group, p->E > 0));
}

size_t td_op_lds_bytes(const td_opparams* p) {
  auto kp = [](int K, int f) { return (size_t)((K + (f ? 2047 : 511)) / (f ? 2048 : 512) * (f ? 2048 : 512)); };
  size_t x = std::max({kp(p->H, p->wf), kp(p->qd, p->wf), kp(p->I, p->wf), kp(p->H, 0)}) * 4 + TD_NW * 4;
  if (p->topk > 0) x = std::max(x, (size_t)p->topk * kp(p->I, p->wf) * 4);
  return std::max(x, op_attn_lds_bytes(p, 1));  // (the one-wave attention layout, as before the split)
}

int td_launch_op_begin(const td_opparams* p, const int32_t* d_token, int32_t pos, void* stream) {
  op_begin<<<1, 256, 0, (hipStream_t)stream>>>(*p, d_token, pos);
  return (int)hipGetLastError();
}

// Every launch of the step after op_begin, in order.
int td_launch_op_layers(const td_opparams* p, void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  const td_opparams& P = *p;
  const size_t lds = td_op_lds_bytes(p), alds = op_attn_lds_bytes(p);
  const int U = P.qkv_rows / 2;
  for (int l = 0; l < P.L; ++l) {
    op_qkv<<<blocks_for(U, R_QKV), 256, lds, s>>>(P, l, R_QKV);
    if (P.d == 64) {
      op_attn<64><<<P.nkv * P.n_chunks_max, 512, alds, s>>>(P, l);
      op_merge<64><<<P.nkv, 512, 0, s>>>(P);
    } else {
      op_attn<128><<<P.nkv * P.n_chunks_max, 512, alds, s>>>(P, l);
      op_merge<128><<<P.nkv, 512, 0, s>>>(P);
    }
    op_resid<<<blocks_for(P.H, R_RESID), 256, lds, s>>>(P, l, 1, R_RESID);
    if (P.E > 0) {
      op_router<<<blocks_for(P.E, 1), 256, lds, s>>>(P, l);
      op_moe_gu<<<blocks_for(P.topk * P.I, R_MOE_GU), 256, lds, s>>>(P, l, R_MOE_GU);
      op_moe_down<<<blocks_for(P.H, R_MOE_DOWN), 256, lds, s>>>(P, l, R_MOE_DOWN);
    } else {
      op_gu<<<blocks_for(P.I, R_GU), 256, lds, s>>>(P, l, R_GU);
      op_resid<<<blocks_for(P.H, R_RESID), 256, lds, s>>>(P, l, 3, R_RESID);
    }
  }
  const int hb = blocks_for(P.V, R_HEAD);
  op_head<<<hb, 256, lds, s>>>(P, R_HEAD);
  op_argmax<<<1, 64, 0, s>>>(P, hb);
  return (int)hipGetLastError();
}

int td_op_set_lds_limits(const td_opparams* p) {
  const int lds = (int)td_op_lds_bytes(p), alds = (int)op_attn_lds_bytes(p);
  hipError_t e = hipSuccess;
  const void* fns[] = {(const void*)op_qkv, (const void*)op_resid, (const void*)op_gu, (const void*)op_head,
                       (const void*)op_router, (const void*)op_moe_gu, (const void*)op_moe_down};
  for (const void* f : fns)
    if (e == hipSuccess) e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  for (const void* f : {(const void*)op_attn<64>, (const void*)op_attn<128>})
    if (e == hipSuccess) e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, alds);
  return (int)e;
}
