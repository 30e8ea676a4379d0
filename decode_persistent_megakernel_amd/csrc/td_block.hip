// td_block.hip - the block forward: n <= TD_MAX_BLOCK consecutive tokens of
// one sequence through the decoder in one pass over the weights, for a prompt
// (prefill) or for checking drafted tokens (the M = K + 1 verify of
// speculative decoding).  With M tokens the weight-streaming GEMVs of the
// decode step become GEMMs, Y[M][N] = X[M][K] W[N][K]^T, and run on the matrix
// cores.  Token i sits at position pos0 + i and attends to positions
// 0 .. pos0 + i; its K/V rows are written to the cache.
//
// Arithmetic: the GEMM inputs stay fp32.  When a workgroup stages a chunk of
// them into LDS it splits every value into three bf16 parts, hi + mid + lo,
// which hold its 24 significant bits (each part takes the rounding residue of
// the one before), and multiplies all three with the bf16 weights by
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation: the products are those of
// fp32 inputs with bf16 weights, as in the decode step, up to the order of the
// sums.  int4 codes minus 8 are exact in bf16; the fp16 scale of a 64-column
// group multiplies that group's partial.  The residual stream, RMSNorm, RoPE,
// softmax and SiLU are fp32 as in the decode step.
//
// One kernel launch per op (the prompt path is not latency-bound like a decode
// step).  Per layer: residual update + RMSNorm statistics, QKV GEMM (the norm
// applied while staging), QKV epilogue (bias, RoPE, K/V write), attention, O
// GEMM, residual update + statistics, gate/up GEMM (the norm applied while
// staging), SwiGLU, down GEMM; then the final residual update + statistics, the
// logits GEMM (normalised while staging; the last row or every row) and the
// greedy token of each logits row.  GEMMs with fewer
// 64-row weight tiles than CUs split K into slices whose partial sums are
// added by their consumer in slice order (deterministic results).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "td.h"
#include "td_internal.h"
#include "td_device.h"

namespace {

typedef short s8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

// Sum over the workgroup of one value per thread, in a fixed order (the same
// bits on every run): wave sums, then the waves' sums in wave order.
DEV float block_sum(float v, float* red) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  if (lane_id() == 0) red[wave] = v;
  __syncthreads();
  float s = red[0];
  for (int w = 1; w < nw; ++w) s += red[w];
  __syncthreads();
  return s;
}

// ------------------------------------------------------------ elementwise
// x[i][:] = the bf16 embedding row of token i (fp32); an id outside [0, V)
// raises the range bit and reads row 0.
__global__ void __launch_bounds__(256) blk_embed(const uint16_t* embed, const int32_t* tokens, int H, int V, float* x,
                                                 int32_t* err) {
  const int i = blockIdx.x;
  int t = tokens[i];
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0) atomicOr(err, TD_ERRBIT_RANGE);
    t = 0;
  }
  const uint16_t* row = embed + (size_t)t * H;
  float* xi = x + (size_t)i * H;
  for (int e = threadIdx.x; e < H; e += blockDim.x) xi[e] = bf16f(row[e]);
}

// Columns 256 b .. + 256 of row i of the residual stream: x += the S partial
// sums of the producing GEMM (slice order; S = 0 adds nothing); xg = x * gain,
// the input of the GEMM that consumes RMSNorm(x); the block's sum of squares
// of the updated values goes to ssq[i][b] (wave sums in wave order), from
// which that GEMM forms the row's 1 / rms.
__global__ void __launch_bounds__(256) blk_resid(float* x, const float* part, int S, size_t sstride, int H,
                                                 const uint16_t* gain, float* xg, float* ssq) {
  __shared__ float red[4];
  const int i = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  const size_t o = (size_t)i * H + e;
  float v = x[o];
  if (S) {
#pragma unroll 4
    for (int s = 0; s < S; ++s) v += part[s * sstride + o];
    x[o] = v;
  }
  xg[o] = v * bf16f(gain[e]);
  const float ss = block_sum(v * v, red);
  if (threadIdx.x == 0) ssq[i * gridDim.x + blockIdx.x] = ss;
}

// act = SiLU(gate) * up from the gate/up GEMM output [gate I | up I] (the sum
// of its S slices in slice order when split), columns 256 b .. of row i.
__global__ void __launch_bounds__(256) blk_swiglu(const float* src, int S, size_t sstride, int I, float* act) {
  const int i = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e >= I) return;
  const float* yi = src + (size_t)i * 2 * I;
  float g = yi[e], u = yi[I + e];
#pragma unroll 4
  for (int s = 1; s < S; ++s) {
    g += yi[s * sstride + e];
    u += yi[s * sstride + I + e];
  }
  act[(size_t)i * I + e] = g / (1.0f + expf(-g)) * u;
}

// logits[r][:] = the sum of the S slices of a split logits GEMM (slice order).
__global__ void __launch_bounds__(256) blk_sum_parts(const float* part, int S, size_t sstride, int N, float* y) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= N) return;
  const size_t o = (size_t)blockIdx.y * N + e;
  float v = part[o];
  for (int s = 1; s < S; ++s) v += part[s * sstride + o];
  y[o] = v;
}

// ------------------------------------------------------------ GEMM
// Y[M][N] = X[M][K] W[N][K]^T over the K slice [KS blockIdx.y, + KS) for
// M <= 16 MT, X fp32 with row pitch ldx.  A workgroup of 4 waves takes 64
// weight rows, 16 per wave; all waves share the X chunk (64 columns of every
// token row) that the workgroup stages into LDS, split into three bf16 parts,
// two chunks deep.  Each wave streams its rows' weights through a ring of D
// chunks held in registers (D - 1 chunks in flight ahead of the one being
// multiplied).  Every load is issued unconditionally (rows past M read row
// M - 1, chunks past the slice re-read its last chunk, results unused), so
// the number of loads between any two points is fixed and each wait for a
// chunk leaves the later loads in flight.
//
// The split is exact: hi = v with the low 16 bits cleared, mid = the same of
// v - hi, lo = v - hi - mid; each part carries 8 of v's 24 significant bits,
// so hi + mid + lo = v and the three products with a bf16 weight sum to the
// fp32 product.
//
// MFMA 16x16x32 bf16 operands: lane l holds row l % 16 of A (token rows) and
// of B (weight rows) at 8 columns of the 32-column step selected by l / 16;
// the result lane l holds token rows 4 (l / 16) + e, weight row l % 16.  For
// bf16 weights lane l takes columns 32 j + 8 (l / 16) of the chunk at step j;
// for int4 columns 16 (l / 16) + 8 j (the chunk is one scale group and a lane
// reads its 16 codes as one 8-byte word).  A and B take the same columns, so
// each step's products are a dot product over 32 distinct columns.
constexpr int XP = 72;  // LDS row pitch of a staged part, bf16 elements (144 B: conflict-free 16-B reads)

// Thread t stages groups g = t + 256 i (i < MT) of a chunk: 4 consecutive
// columns 4 (g % 16) of token row g / 16.
template <int MT>
DEV void stage_load(float4 (&v)[MT], const float* X, int ldx, int M, int k0) {
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int g = threadIdx.x + 256 * i, m = min(g >> 4, M - 1), c = (g & 15) * 4;
    v[i] = *(const float4*)(X + (size_t)m * ldx + k0 + c);
  }
}

DEV uint32_t hi_pair(float a, float b) {  // the high halves of a and b, a in the low half
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
DEV float drop_hi(float a) { return a - __uint_as_float(__float_as_uint(a) & 0xffff0000u); }

template <int MT>
DEV void stage_store(uint16_t* xs, const float4 (&v)[MT]) {
  constexpr int PART = MT * 16 * XP;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int g = threadIdx.x + 256 * i, m = g >> 4, c = (g & 15) * 4;
    float a[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint16_t* dst = xs + m * XP + c;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      *(uint2*)(dst + p * PART) = make_uint2(hi_pair(a[0], a[1]), hi_pair(a[2], a[3]));
      if (p < 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = drop_hi(a[e]);
      }
    }
  }
}

template <int FMT>
struct WChunk;
template <>
struct WChunk<TD_WF_BF16> {
  u32x4 w[2];
};
template <>
struct WChunk<TD_WF_INT4_G64> {
  u32x2 w;
  uint32_t s;
};

template <int FMT>
DEV void load_chunk(WChunk<FMT>& c, const uint8_t* wrow, const uint16_t* srow, int ch, int q) {
  if constexpr (FMT == TD_WF_BF16) {
    c.w[0] = *(const u32x4*)(wrow + ch * 128 + q * 16);
    c.w[1] = *(const u32x4*)(wrow + ch * 128 + 64 + q * 16);
  } else {
    c.w = *(const u32x2*)(wrow + ch * 32 + q * 8);
    c.s = srow[ch];
  }
}

DEV s8v int4_bf16x8(uint32_t c) {
  s8v b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (short)(__float_as_uint((float)((c >> (4 * e)) & 15u) - 8.f) >> 16);  // exact
  return b;
}

// One chunk for NB weight tiles: each 64-column chunk's products are summed by
// the MFMAs into a fresh partial (parts lo, mid, hi in that order), which a
// VALU add (round to nearest) then adds to the running sum; the running sum
// never passes through the matrix unit's accumulator.  Each A fragment read
// from LDS serves all NB weight tiles.
template <int FMT, int MT, int NB>
DEV void mul_chunk(f32x4 (&acc)[MT][NB], const WChunk<FMT> (&c)[NB], const uint16_t* xs, int r, int q) {
  constexpr int PART = MT * 16 * XP;
  f32x4 pr[MT][NB];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pr[t][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bf8v b[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (FMT == TD_WF_BF16) b[nb] = __builtin_bit_cast(bf8v, c[nb].w[j]);
      else b[nb] = __builtin_bit_cast(bf8v, int4_bf16x8(j ? c[nb].w.y : c[nb].w.x));
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint16_t* a = xs + (16 * t + r) * XP + (FMT == TD_WF_BF16 ? 32 * j + 8 * q : 16 * q + 8 * j);
#pragma unroll
      for (int p = 2; p >= 0; --p) {
        const bf8v av = *(const bf8v*)(a + p * PART);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          pr[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[nb], pr[t][nb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (FMT == TD_WF_BF16) {
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t][nb] += pr[t][nb];
    } else {
      // result lane l is weight row l % 16 of tile nb, the row whose scale this lane loaded
      const float sc = f16f(c[nb].s);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        acc[t][nb].x = fmaf(sc, pr[t][nb].x, acc[t][nb].x);
        acc[t][nb].y = fmaf(sc, pr[t][nb].y, acc[t][nb].y);
        acc[t][nb].z = fmaf(sc, pr[t][nb].z, acc[t][nb].z);
        acc[t][nb].w = fmaf(sc, pr[t][nb].w, acc[t][nb].w);
      }
    }
  }
}

// Chunk c's loads, weights and X, go into ring slot c % D together, D - 1
// chunks ahead of their use, X first: waiting for the X of chunk c + 1 (to
// stage it) then leaves the weights of chunks c + 1 .. c + D - 1 in flight.
template <int FMT, int MT, int NB>
struct Slot {
  WChunk<FMT> w[NB];
  float4 x[MT];
};

template <int FMT, int MT, int NB>
constexpr int ring_depth() {
  if (NB > 1) return FMT == TD_WF_BF16 ? 4 : 6;
  return FMT == TD_WF_BF16 ? (MT <= 2 ? 8 : 6) : (MT <= 2 ? 10 : 8);
}

// Weight tiles per wave: two (a workgroup covers 128 weight rows, halving the
// input reads per weight byte) when the token rows make the staged input as
// large as the weights it multiplies and the matrix still has a 64-row tile per
// CU; otherwise one, which keeps the split-K slices of short matrices long.
inline int nb_of(int mt, int N, int ncu) { return (mt >= 3 && N >= 64 * ncu) ? 2 : 1; }

// With NORM, X holds x * gain and the result is RMSNorm(x) W^T: row m of the
// product is multiplied by row m's 1 / rms, its sum of squares being the nbs
// block sums ssq[m nbs ..] of blk_resid added in block order (the decode step's
// form: the gains scale the input, 1 / rms the finished dot products).
template <int FMT, int MT, int NB, bool NORM>
__global__ void __launch_bounds__(256) blk_gemm(const float* X, int ldx, int M, int K, int KS, const uint8_t* W,
                                                const uint16_t* Sc, int N, float* Y, int ldy, size_t sstride,
                                                const float* ssq, int nbs, float eps) {
  constexpr int PART = MT * 16 * XP;
  constexpr int D = ring_depth<FMT, MT, NB>();
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][3 * PART];
  const int wave = threadIdx.x >> 6, lane = lane_id(), r = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 64 * NB + wave * 16 * NB + r;  // tile nb: row n0 + 16 nb
  const int kb = blockIdx.y * KS, nch = (min(K, kb + KS) - kb) >> 6;
  const uint8_t* wrow[NB];
  const uint16_t* srow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int nr = min(n0 + 16 * nb, N - 1);  // rows past N read row N - 1 and are not stored
    if constexpr (FMT == TD_WF_BF16) {
      wrow[nb] = W + ((size_t)nr * K + kb) * 2;
      srow[nb] = nullptr;
    } else {
      wrow[nb] = W + (size_t)nr * (K >> 1) + (kb >> 1);
      srow[nb] = Sc + (size_t)nr * (K >> 6) + (kb >> 6);
    }
  }
  const float* xb = X + kb;
  // NORM: thread t < M forms row t's 1 / rms.  Its first 8 block sums are
  // loaded before the weights of the prologue, so that waiting for them leaves
  // those in flight (every thread loads, from a clamped row, so that the wait
  // counts stay exact).
  __shared__ float invs[NORM ? 64 : 1];
  float sv[8];
  const int nrow = min((int)threadIdx.x, M - 1);
  if constexpr (NORM) {
#pragma unroll
    for (int u = 0; u < 8; ++u) sv[u] = ssq[nrow * nbs + min(u, nbs - 1)];
  }
  f32x4 acc[MT][NB];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[t][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  Slot<FMT, MT, NB> ring[D];
#pragma unroll
  for (int i = 0; i < D - 1; ++i) {
    const int ch = min(i, nch - 1);
    stage_load<MT>(ring[i].x, xb, ldx, M, 64 * ch);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) load_chunk<FMT>(ring[i].w[nb], wrow[nb], srow[nb], ch, q);
  }
  if constexpr (NORM) {
    float ss = sv[0];  // the block sums added in block order
#pragma unroll
    for (int u = 1; u < 8; ++u)
      if (u < nbs) ss += sv[u];
    for (int b = 8; b < nbs; ++b) ss += ssq[nrow * nbs + b];
    if (threadIdx.x < 64) invs[threadIdx.x] = 1.0f / sqrtf(ss / (float)K + eps);
  }
  stage_store<MT>(xs[0], ring[0].x);
  wg_bar();  // (also makes invs visible)
  for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int c = c0 + i;
      {
        Slot<FMT, MT, NB>& sl = ring[(i + D - 1) % D];  // chunk c - 1's slot, consumed
        const int ch = min(c + D - 1, nch - 1);
        stage_load<MT>(sl.x, xb, ldx, M, 64 * ch);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) load_chunk<FMT>(sl.w[nb], wrow[nb], srow[nb], ch, q);
      }
      if (c < nch) mul_chunk<FMT, MT, NB>(acc, ring[i].w, xs[c & 1], r, q);
      stage_store<MT>(xs[(c + 1) & 1], ring[(i + 1) % D].x);
      wg_bar();
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + 16 * nb;
    if (n >= N) continue;
    float* dst = Y + blockIdx.y * sstride + n;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float rv[4] = {acc[t][nb].x, acc[t][nb].y, acc[t][nb].z, acc[t][nb].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * t + 4 * q + e;
        if (m < M) dst[(size_t)m * ldy] = NORM ? rv[e] * invs[m] : rv[e];
      }
    }
  }
}

// ------------------------------------------------------------ streamed GEMM
// Y[M][N] = X[M][K] W[N][K]^T for bf16 weights and 49 <= M <= 64 token rows,
// over the K slice [KS blockIdx.y, + KS) of at most XC 64-column chunks.  A
// workgroup of 8 waves takes NR = 16 NT weight rows; wave w multiplies token
// rows 16 (w & 3) .. + 15 by weight tiles (w >> 2) NT / 2 .. + NT / 2 (two
// waves per SIMD, so one wave's matrix work covers the other's waits).
//
// The weights stream through a ring of SR LDS slots, one 64-column chunk
// (NR rows x 128 bytes) each: global_load_lds copies 8 whole 128-byte rows
// per instruction, and each wave copies 1/8 of every chunk.  Each wave loads
// its 16 token rows' 64 input columns of the chunk straight into registers and
// splits them into the three bf16 parts there.  A chunk's copies and input
// loads are issued together, SR - 1 chunks ahead of their use, so one counted
// wait covers both; the waves meet once per chunk, when all copies of the
// chunk have landed and the slot about to be refilled has been read out by
// all of them.  Compared with blk_gemm (weights in registers, input split in
// LDS) this reads every weight line whole and splits each input value once
// per pair of waves instead of staging it through LDS.
//
// The 16-byte units of weight row n sit in the LDS slot in the order
// u ^ (n & 7), so that a fragment read (16 rows at one column offset) spreads
// over the banks.  The fragments of each group of 4 tiles are read one group
// ahead with inline ds_reads and counted waits (the compiler would read each
// just before its use and stall on every read).
//
// The input and norm loads are inline-asm loads the wave waits for with an
// exact count: the compiler, unable to order them against the LDS copies,
// would otherwise wait for every copy in flight.  Such a load's destination
// must stay live until the load has been waited for (the compiler, which sees
// the value written at issue, may otherwise give a dead destination to another
// value while the load is still in flight): inputs are loaded only for
// chunks below XC, and every loaded register is consumed in its own
// iteration, after its wait, also past the end of the slice.
//
// The products, and the order in which each chunk's partial is formed (fresh
// per chunk, parts lo, mid, hi) and added to the running sum, are those of
// blk_gemm: the same bits.  Outputs are stored non-temporally (the partial
// slices are read once, by the next kernel).
template <int NT>
constexpr int stream_slots() {
  return (147456 / (NT * 2048)) < 5 ? 147456 / (NT * 2048) : 5;
}
template <int NT>
constexpr int stream_lds() {
  return stream_slots<NT>() * NT * 2048;
}

DEV u32x4 ld16_asm(const void* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// s_waitcnt vmcnt(n) for an n that the unrolled caller makes a constant
DEV void vm_wait_n(int n) {
  switch (n) {
#define TD_VW(k) \
  case k: vmcnt_wait<k>(); break;
    TD_VW(0) TD_VW(1) TD_VW(2) TD_VW(3) TD_VW(4) TD_VW(5) TD_VW(6) TD_VW(7) TD_VW(8) TD_VW(9) TD_VW(10) TD_VW(11)
    TD_VW(12) TD_VW(13) TD_VW(14) TD_VW(15) TD_VW(16) TD_VW(17) TD_VW(18) TD_VW(19) TD_VW(20) TD_VW(21) TD_VW(22)
    TD_VW(23) TD_VW(24) TD_VW(25) TD_VW(26) TD_VW(27) TD_VW(28) TD_VW(29) TD_VW(30) TD_VW(31) TD_VW(32)
#undef TD_VW
    default: vmcnt_wait<0>(); break;
  }
}

#define TD_LDSPTR(p) ((__attribute__((address_space(3))) void*)(p))

template <int NT, int XC, bool NORM>
__global__ void __launch_bounds__(512) blk_gemm_stream(const float* X, int ldx, int M, int K, int KS,
                                                       const uint16_t* W, int N, float* Y, int ldy, size_t sstride,
                                                       const float* ssq, int nbs, float eps) {
  constexpr int NR = 16 * NT, WB = NR * 128, SR = stream_slots<NT>(), WI = WB / 8192, NTW = NT / 2;
  static_assert(SR >= 3 && NTW % 4 == 0, "the ring keeps two chunks in flight; tiles go in groups of 4");
  extern __shared__ __attribute__((aligned(1024))) uint8_t ring[];
  __shared__ float invs[NORM ? 64 : 1];
  const int wave = threadIdx.x >> 6, lane = lane_id(), r = lane & 15, q = lane >> 4;
  const int tw = wave & 3, th = wave >> 2;
  const int n0 = blockIdx.x * NR;
  const int kb = blockIdx.y * KS, nch = (min(K, kb + KS) - kb) >> 6;
  const float* xr = X + (size_t)min(16 * tw + r, M - 1) * ldx + kb + 8 * q;
  // NORM: the first 8 block sums of row t's sum of squares, consumed in the first chunk's iteration
  uint32_t sv[8];
  const int nrow = min((int)threadIdx.x & 63, M - 1);
  if constexpr (NORM) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      asm volatile("global_load_dword %0, %1, off" : "=v"(sv[u]) : "v"(ssq + nrow * nbs + min(u, nbs - 1)) : "memory");
  }
  // copy sources: instruction WI wave + e of a chunk covers rows 8 (WI wave + e) + lane / 8
  const uint8_t* wsrc[WI];
#pragma unroll
  for (int e = 0; e < WI; ++e) {
    const int n = 8 * (WI * wave + e) + (lane >> 3), u = (lane & 7) ^ (n & 7);
    wsrc[e] = (const uint8_t*)(W + (size_t)min(n0 + n, N - 1) * K + kb) + 16 * u;
  }
  u32x4 xq[XC][2][2];  // chunk c's inputs: columns 32 j + 8 q + 4 h of token row 16 tw + r
  auto issue = [&](int c) {
    const int ch = min(c, nch - 1);  // past the slice: its last chunk again (results unused)
    if (c < XC) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) xq[c][j][h] = ld16_asm(xr + 64 * ch + 32 * j + 4 * h);
    }
    uint8_t* base = ring + (c % SR) * WB + 1024 * WI * wave;
#pragma unroll
    for (int e = 0; e < WI; ++e)
      __builtin_amdgcn_global_load_lds((const void*)(wsrc[e] + ch * 128), TD_LDSPTR(base + 1024 * e), 16, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < SR - 1; ++i) issue(i);
  f32x4 acc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < XC; ++c) {
    if (c >= nch) {  // past the slice: everything lands, then this chunk's input registers are released
      vm_drain();
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) asm volatile("" ::"v"(xq[c][j][h]));
      continue;
    }
    {  // this wave's loads of chunk c have landed: later ones are chunks c + 1 .. c + SR - 2's
      int later = 0;
#pragma unroll
      for (int k = c + 1; k <= c + SR - 2; ++k) later += WI + (k < XC ? 4 : 0);
      vm_wait_n(later);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(xq[c][j][h]));
    if (NORM && c == 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) asm volatile("" : "+v"(sv[u]));
      float ss = __uint_as_float(sv[0]);  // the block sums added in block order
#pragma unroll
      for (int u = 1; u < 8; ++u)
        if (u < nbs) ss += __uint_as_float(sv[u]);
      for (int b = 8; b < nbs; ++b) ss += ssq[nrow * nbs + b];
      if (threadIdx.x < 64) invs[threadIdx.x] = 1.0f / sqrtf(ss / (float)K + eps);
    }
    wg_bar();  // every wave's copies of chunk c; and chunk c - 1's slot has been read out
    issue(c + SR - 1);
    // A fragments: step j, part p (hi, mid, lo)
    bf8v xa[2][3];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float a[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = __uint_as_float(xq[c][j][0][e]);
        a[4 + e] = __uint_as_float(xq[c][j][1][e]);
      }
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        u32x4 hh;
        hh.x = hi_pair(a[0], a[1]);
        hh.y = hi_pair(a[2], a[3]);
        hh.z = hi_pair(a[4], a[5]);
        hh.w = hi_pair(a[6], a[7]);
        xa[j][p] = __builtin_bit_cast(bf8v, hh);
        if (p < 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = drop_hi(a[e]);
        }
      }
    }
    // B fragments: weight row 16 (NTW th + t) + r, columns 32 j + 8 q (unit 4 j + q); steps
    // s = (j, group of 4 tiles), each read one step ahead
    constexpr int GPJ = NTW / 4, NS = 2 * GPJ;
    u32x4 bq[NS][4];
    const uint32_t wsa = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(ring + (c % SR) * WB) +
                         r * 128 + 2048 * NTW * th;
    auto rd = [&](int s) {
      const int j = s / GPJ, g = s % GPJ;
      const uint32_t a = wsa + 16 * ((4 * j + q) ^ (r & 7)) + 2048 * 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("ds_read_b128 %0, %1" : "=v"(bq[s][i]) : "v"(a + 2048 * i));
    };
    f32x4 pr[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) pr[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    rd(0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + 1 < NS) {
        rd(s + 1);
        asm volatile("s_waitcnt lgkmcnt(4)" ::: "memory");
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(bq[s][i]));
      const int j = s / GPJ, g = s % GPJ;
#pragma unroll
      for (int p = 2; p >= 0; --p)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pr[4 * g + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j][p], __builtin_bit_cast(bf8v, bq[s][i]),
                                                                  pr[4 * g + i], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] += pr[t];
  }
  vm_drain();  // the copies past the slice have landed before the workgroup ends
  wg_bar();    // invs
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int n = n0 + 16 * (NTW * th + t) + r;
    if (n >= N) continue;
    float* dst = Y + blockIdx.y * sstride + n;
    const float rv[4] = {acc[t].x, acc[t].y, acc[t].z, acc[t].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mm = 16 * tw + 4 * q + e;
      if (mm < M) __builtin_nontemporal_store(NORM ? rv[e] * invs[mm] : rv[e], dst + (size_t)mm * ldy);
    }
  }
}

// ------------------------------------------------------------ QKV epilogue
// Token i (blockIdx.y), row pair u (256 per block): the sum of the S QKV
// partial slices, bias, RoPE of the q and k row pairs at position pos0 + i, q
// (times 1/sqrt(d)) to qout [n][qd], k and v rows to the cache as bf16.
__global__ void __launch_bounds__(256) blk_qkv_post(const float* part, int S, size_t sstride, int qkv_rows, int qd,
                                                    int kvd, int d, int nkv, int max_ctx, int layer, int pos0,
                                                    const uint16_t* bias, const float* rope_cs, float attn_scale,
                                                    float* qout, uint16_t* kc, uint16_t* vc) {
  const int i = blockIdx.y;
  const int pos = pos0 + i;
  const int half = d >> 1;
  const float* yi = part + (size_t)i * qkv_rows;
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u < qkv_rows / 2) {
    const int head = u / half, j = u - head * half;
    const int ra = head * d + j, rb = ra + half;
    float a = yi[ra], b = yi[rb];
#pragma unroll 4
    for (int s = 1; s < S; ++s) {
      a += yi[s * sstride + ra];
      b += yi[s * sstride + rb];
    }
    if (bias) {
      a += bf16f(bias[ra]);
      b += bf16f(bias[rb]);
    }
    if (ra < qd + kvd) {
      const float c = rope_cs[((size_t)pos * half + j) * 2], sn = rope_cs[((size_t)pos * half + j) * 2 + 1];
      const float a2 = a * c - b * sn;
      const float b2 = b * c + a * sn;
      a = a2;
      b = b2;
    }
    if (ra < qd) {
      qout[(size_t)i * qd + ra] = a * attn_scale;
      qout[(size_t)i * qd + rb] = b * attn_scale;
    } else {
      const bool isk = ra < qd + kvd;
      const int g = (ra - qd - (isk ? 0 : kvd)) / d;
      uint16_t* row = (isk ? kc : vc) + (((size_t)layer * nkv + g) * max_ctx + pos) * d;
      row[j] = (uint16_t)f2bf(a);
      row[j + half] = (uint16_t)f2bf(b);
    }
  }
}

// ------------------------------------------------------------ attention on the matrix cores
// Workgroup (x, g): kv head g and 16 of its query rows, the (token, head)
// pairs r0 .. r0 + 15 (r0 = 16 x) of the block's n tokens and the group's
// heads, row = token * group + head.  The scores come out transposed, S^T =
// K Q^T, so that each lane holds one query's scores for 8 keys:
// v_mfma_f32_16x16x32_bf16 with the keys' K rows (bf16, straight from the
// cache) as A and the queries (fp32, split into three bf16 parts as in the
// GEMMs: exact products) as B; result lane l holds keys 4 (l / 16) + e of a
// 16-key block for query l % 16.  The online softmax then needs only the
// lane's own values and the 3 other lanes of its query (two shuffles), and
// O^T += V^T P^T takes P^T straight from those registers (split into three
// parts) as B; the A operand, V^T, gathers each lane's 8 keys for one
// dimension from the wave's V tile in LDS.  The MFMA's K index of lane group
// a is the key set {4 a + e, 16 + 4 a + e}, the same in both operands.
// Keys come in tiles of 32; wave w takes tiles w, w + 8, ... (loads of its
// next tile in flight during this one), keeps its running max m, sum l and
// O^T, and the 8 waves' states merge in wave order at the end
// (deterministic).  Keys after a query's position get probability 0; loads
// past the workgroup's last key read that key instead.
//
// Long contexts split the key tiles over nsplit workgroups per (rows, head),
// contiguous ranges in split order: each writes its merged (O, m, l) to
// part[sp][g][row] (O unnormalised, relative to m) and blk_attn_merge combines
// the splits in split order.  With nsplit = 1 the output is written here.
template <int D>
__global__ void __launch_bounds__(512) blk_attn_mma(const float* q, const uint16_t* kc, const uint16_t* vc, int nq,
                                                    int group, int nkv, int max_ctx, int layer, int pos0, int n,
                                                    int nsplit, float* part, float* out) {
  constexpr int NS = D / 32, DB = D / 16, VP = D + 8, SEG = D / 8, VL = 32 * SEG / 64;
  // the V tiles, and after the key loop the waves' output states in the same bytes
  constexpr int VT_BYTES = 8 * 32 * VP * 2, OST_BYTES = 8 * 16 * (D + 1) * 4;
  static_assert(OST_BYTES <= VT_BYTES, "the output states fit the V tiles' bytes");
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[VT_BYTES];
  __shared__ float mst[8][16], lst[8][16];
  uint16_t(*vt)[32][VP] = (uint16_t(*)[32][VP])lds_v;
  float(*ost)[16][D + 1] = (float(*)[16][D + 1])lds_v;
  const int wave = threadIdx.x >> 6, lane = lane_id(), r = lane & 15, a = lane >> 4;
  // workgroup L of a 1-D grid: kv head L % nkv, rows 16 x, key split sp with
  // x + nx sp = L / nkv; the dispatcher deals workgroups to the 8 XCDs in
  // turn, so all workgroups of a head land on the same XCDs and share their
  // L2's copy of its K/V rows
  const int rows = n * group, nx = (rows + 15) / 16, g = blockIdx.x % nkv;
  const int r0 = (blockIdx.x / nkv % nx) * 16, sp = blockIdx.x / nkv / nx;
  const int qr = min(r0 + r, rows - 1), ti = qr / group, hh = qr - ti * group;
  const int pos_q = pos0 + ti;
  const int last = pos0 + min(r0 + 15, rows - 1) / group;  // the workgroup's last key
  const int ntiles_all = last / 32 + 1;
  const int t_lo = ntiles_all * sp / nsplit, ntiles = ntiles_all * (sp + 1) / nsplit;  // this split: [t_lo, ntiles)
  // B fragments of Q^T: columns 32 s + 8 a .. + 8 of query qr, in three parts
  bf8v qf[NS][3];
  {
    const float* qp = q + ((size_t)ti * nq + g * group + hh) * D + 8 * a;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 x0 = *(const f32x4*)(qp + 32 * s), x1 = *(const f32x4*)(qp + 32 * s + 4);
      float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        u32x4 h;
        h.x = hi_pair(v[0], v[1]);
        h.y = hi_pair(v[2], v[3]);
        h.z = hi_pair(v[4], v[5]);
        h.w = hi_pair(v[6], v[7]);
        qf[s][p] = __builtin_bit_cast(bf8v, h);
        if (p < 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = drop_hi(v[e]);
        }
      }
    }
  }
  const uint16_t* K = kc + ((size_t)layer * nkv + g) * max_ctx * D;
  const uint16_t* V = vc + ((size_t)layer * nkv + g) * max_ctx * D;
  // a tile's loads: K fragments (key k0 + 16 b + r, columns 32 s + 8 a) and
  // this lane's pieces of the V rows (piece lane + 64 u of the tile)
  auto load_k = [&](int t, u32x4 (&kf)[2][NS]) {
    const int k0 = 32 * t;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        kf[b][s] = *(const u32x4*)(K + (size_t)min(k0 + 16 * b + r, last) * D + 32 * s + 8 * a);
  };
  auto load_v = [&](int t, u32x4 (&vr)[VL]) {
    const int k0 = 32 * t;
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      const int idx = lane + 64 * u;
      vr[u] = *(const u32x4*)(V + (size_t)min(k0 + idx / SEG, last) * D + 8 * (idx % SEG));
    }
  };
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;
  // each tile's loads are issued during the previous tile: V right after the
  // previous V went to LDS, K right after the previous scores (past the last
  // tile: the last one again, unused)
  u32x4 kb[2][NS], vb[VL];
  load_k(max(min(t_lo + wave, ntiles - 1), 0), kb);
  load_v(max(min(t_lo + wave, ntiles - 1), 0), vb);
  // one key tile t with its loads in kf, vr; then tile tn's loads into them
  auto tile = [&](int t, u32x4 (&kf)[2][NS], u32x4 (&vr)[VL], int tn) {
    const int k0 = 32 * t;
    // the V tile into LDS (this wave's own area; its reads below follow in order)
#pragma unroll
    for (int u = 0; u < VL; ++u) {
      const int idx = lane + 64 * u;
      *(u32x4*)&vt[wave][idx / SEG][8 * (idx % SEG)] = vr[u];
    }
    load_v(tn, vr);
    // S^T blocks: keys k0 + 16 b .. + 16 against the 16 queries
    f32x4 sb[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int p = 2; p >= 0; --p)
          sb[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, kf[b][s]), qf[s][p], sb[b], 0, 0, 0);
    load_k(tn, kf);
    // causal mask and the tile's max over the query's 32 keys
    float sv[8], mt = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + 16 * b + 4 * a + e;
        sv[4 * b + e] = key <= pos_q ? sb[b][e] : -__builtin_inff();
        mt = fmaxf(mt, sv[4 * b + e]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    const float corr = m == -__builtin_inff() ? 0.f : expf(m - mn);
    float pv[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = sv[e] == -__builtin_inff() ? 0.f : expf(sv[e] - mn);
      ps += pv[e];
    }
    l = l * corr + ps;
    m = mn;
    // P^T in three parts; K index 8 a + e' is key 4 a + e' (e' < 4) or 16 + 4 a + e' - 4
    bf8v pp[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      u32x4 h;
      h.x = hi_pair(pv[0], pv[1]);
      h.y = hi_pair(pv[2], pv[3]);
      h.z = hi_pair(pv[4], pv[5]);
      h.w = hi_pair(pv[6], pv[7]);
      pp[p] = __builtin_bit_cast(bf8v, h);
      if (p < 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = drop_hi(pv[e]);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      o[db] *= corr;
      // A fragment of V^T: dimension 16 db + r at the lane group's 8 keys
      const int d = 16 * db + r;
      u32x4 w;
      w.x = (uint32_t)vt[wave][4 * a][d] | ((uint32_t)vt[wave][4 * a + 1][d] << 16);
      w.y = (uint32_t)vt[wave][4 * a + 2][d] | ((uint32_t)vt[wave][4 * a + 3][d] << 16);
      w.z = (uint32_t)vt[wave][16 + 4 * a][d] | ((uint32_t)vt[wave][16 + 4 * a + 1][d] << 16);
      w.w = (uint32_t)vt[wave][16 + 4 * a + 2][d] | ((uint32_t)vt[wave][16 + 4 * a + 3][d] << 16);
#pragma unroll
      for (int p = 2; p >= 0; --p)
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, w), pp[p], o[db], 0, 0, 0);
    }
  };
  for (int t = t_lo + wave; t < ntiles; t += 8) tile(t, kb, vb, min(t + 8, ntiles - 1));
  // the query's sum over its 4 lanes; the wave's state to LDS
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (a == 0) {
    mst[wave][r] = m;
    lst[wave][r] = l;
  }
  __syncthreads();  // every wave is done with its V tile: the bytes now hold the output states
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) ost[wave][r][16 * db + 4 * a + e] = o[db][e];
  __syncthreads();
  // merge in wave order; output (row r0 + qq, dimension d)
  for (int idx = threadIdx.x; idx < 16 * D; idx += 512) {
    const int qq = idx / D, d = idx - qq * D, row = r0 + qq;
    if (row >= rows) continue;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 8; ++w) M = fmaxf(M, mst[w][qq]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      if (mst[w][qq] == -__builtin_inff()) continue;
      const float f = expf(mst[w][qq] - M);
      L = fmaf(lst[w][qq], f, L);
      O = fmaf(ost[w][qq][d], f, O);
    }
    if (nsplit == 1) {
      const int i = row / group, h = row - i * group;
      out[((size_t)i * nq + g * group + h) * D + d] = O / L;
    } else {
      float* ps = part + (((size_t)sp * nkv + g) * rows + row) * (D + 2);
      ps[d] = O;
      if (d == 0) {
        ps[D] = M;
        ps[D + 1] = L;
      }
    }
  }
}

// The key splits of blk_attn_mma combined in split order: thread (row, d) of
// kv head g (blockIdx.y) over rows 512 / D blockIdx.x ...
template <int D>
__global__ void __launch_bounds__(512) blk_attn_merge(const float* part, int nsplit, int nq, int group, int nkv, int n,
                                                      float* out) {
  const int g = blockIdx.y, rows = n * group;
  const int row = blockIdx.x * (512 / D) + (int)threadIdx.x / D, d = threadIdx.x % D;
  if (row >= rows) return;
  auto at = [&](int s) { return part + (((size_t)s * nkv + g) * rows + row) * (D + 2); };
  float M = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, at(s)[D]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* ps = at(s);
    if (ps[D] == -__builtin_inff()) continue;
    const float f = expf(ps[D] - M);
    L = fmaf(ps[D + 1], f, L);
    O = fmaf(ps[d], f, O);
  }
  const int i = row / group, h = row - i * group;
  out[((size_t)i * nq + g * group + h) * D + d] = O / L;
}

// ------------------------------------------------------------ greedy token
// Phase 1, workgroup (b, r): the largest value of columns [CH b, CH (b + 1))
// of logits row r (lowest id among equals) as (value bits, id) in
// cand[r][b]; id TD_ARGMAX_NONE when the slice is empty, TD_ARGMAX_BAD (and
// the error bit) when it holds a NaN or an infinity.
constexpr uint32_t TD_ARGMAX_NONE = 0x7fffffffu, TD_ARGMAX_BAD = 0xfffffffeu;
__global__ void __launch_bounds__(256) blk_argmax_part(const float* logits, int V, int CH, uint2* cand,
                                                       int32_t* err) {
  __shared__ float bvs[4];
  __shared__ int bis[4], bads[4];
  const int r = blockIdx.y, b = blockIdx.x;
  const float* x = logits + (size_t)r * V;
  const int e1 = min(V, CH * (b + 1));
  float bv = -__builtin_inff();
  int bi = (int)TD_ARGMAX_NONE, bad = 0;
  for (int e = CH * b + threadIdx.x; e < e1; e += 256) {
    const float v = x[e];
    if (!isfinite(v)) bad = 1;
    else if (v > bv || (v == bv && e < bi)) { bv = v; bi = e; }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  bad = __any(bad);
  const int wave = threadIdx.x >> 6;
  if (lane_id() == 0) {
    bvs[wave] = bv;
    bis[wave] = bi;
    bads[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  for (int w = 1; w < 4; ++w) {
    if (bvs[w] > bv || (bvs[w] == bv && bis[w] < bi)) { bv = bvs[w]; bi = bis[w]; }
    bad |= bads[w];
  }
  if (bad) atomicOr(err, TD_ERRBIT_NONFINITE);
  cand[r * gridDim.x + b] = make_uint2(__float_as_uint(bv), bad ? TD_ARGMAX_BAD : (uint32_t)bi);
}

// Phase 2, one thread per row r: the slices' candidates in slice order (ids
// ascend with the slice, so the first of equal values has the lowest id);
// token 0 when the row held a non-finite value.  The last row's token also
// goes to token_word.
__global__ void __launch_bounds__(64) blk_argmax_final(const uint2* cand, int nb, int rows, int32_t* tokens,
                                                       int32_t* token_word) {
  const int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= rows) return;
  float bv = -__builtin_inff();
  uint32_t bi = TD_ARGMAX_NONE;
  bool bad = false;
  for (int b0 = 0; b0 < nb; b0 += 16) {  // 16 candidates loaded together, then taken in slice order
    uint2 cs[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) cs[u] = cand[r * nb + min(b0 + u, nb - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint2 c = cs[u];
      if (b0 + u >= nb) continue;
      if (c.y == TD_ARGMAX_BAD) bad = true;
      else if (c.y != TD_ARGMAX_NONE && (__uint_as_float(c.x) > bv || bi == TD_ARGMAX_NONE)) {
        bv = __uint_as_float(c.x);
        bi = c.y;
      }
    }
  }
  const int tok = (bad || bi == TD_ARGMAX_NONE) ? 0 : (int)bi;
  if (tokens) tokens[r] = tok;
  if (r == rows - 1) *token_word = tok;
}

// RMSNorm by row scaling of the product (ssq non-null) or none.
struct NormArgs {
  const float* ssq;
  int nbs;
  float eps;
};

template <int FMT, bool NORM>
int launch_gemm_n(int S, int NB, int N, hipStream_t st, const float* X, int ldx, int M, int K, int KS,
                  const uint8_t* W, const uint16_t* Sc, float* Y, int ldy, size_t sstride, const NormArgs& a) {
  const dim3 block(256), grid((N + 64 * NB - 1) / (64 * NB), S);
  const int mt = (M + 15) / 16;
#define TD_GEMM(MT_, NB_)                                                                                      \
  blk_gemm<FMT, MT_, NB_, NORM><<<grid, block, 0, st>>>(X, ldx, M, K, KS, W, Sc, N, Y, ldy, sstride, a.ssq, a.nbs, \
                                                        a.eps)
  if (mt == 1) TD_GEMM(1, 1);
  else if (mt == 2) TD_GEMM(2, 1);
  else if (mt == 3 && NB == 1) TD_GEMM(3, 1);
  else if (mt == 3) TD_GEMM(3, 2);
  else if (NB == 1) TD_GEMM(4, 1);
  else TD_GEMM(4, 2);
#undef TD_GEMM
  return (int)hipGetLastError();
}

template <int FMT>
int launch_gemm_f(int S, int NB, int N, hipStream_t st, const float* X, int ldx, int M, int K, int KS,
                  const uint8_t* W, const uint16_t* Sc, float* Y, int ldy, size_t sstride, const NormArgs& a) {
  return a.ssq ? launch_gemm_n<FMT, true>(S, NB, N, st, X, ldx, M, K, KS, W, Sc, Y, ldy, sstride, a)
                : launch_gemm_n<FMT, false>(S, NB, N, st, X, ldx, M, K, KS, W, Sc, Y, ldy, sstride, a);
}

template <int NT, int XC>
int launch_stream(dim3 grid, hipStream_t st, const float* X, int ldx, int M, int K, int KS, const uint8_t* W, int N,
                  float* Y, int ldy, size_t sstride, const NormArgs& a) {
  if (a.ssq)
    blk_gemm_stream<NT, XC, true><<<grid, 512, stream_lds<NT>(), st>>>(X, ldx, M, K, KS, (const uint16_t*)W, N, Y,
                                                                       ldy, sstride, a.ssq, a.nbs, a.eps);
  else
    blk_gemm_stream<NT, XC, false><<<grid, 512, stream_lds<NT>(), st>>>(X, ldx, M, K, KS, (const uint16_t*)W, N, Y,
                                                                        ldy, sstride, nullptr, 0, 0.f);
  return (int)hipGetLastError();
}

template <int NT, int XC>
int prepare_stream() {
  for (const void* f : {(const void*)blk_gemm_stream<NT, XC, true>, (const void*)blk_gemm_stream<NT, XC, false>}) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, stream_lds<NT>());
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

// X W^T (with norm.ssq, X = x * gain and the rows scaled to RMSNorm(x) W^T),
// N columns with row pitch ldy.  With
// one K slice the result goes to Y; with S > 1 slices, slice s goes to
// part + s M ldy and the consumer adds them in slice order.  *S_out receives S.
// stream: the streamed GEMM may serve (bf16, 49..64 rows); the logits GEMM
// keeps blk_gemm, so that its last row's bits match the last-row-only call.
int gemm(int fmt, int ncu, const float* X, int ldx, int M, int K, const uint8_t* W, const uint16_t* Sc, int N,
         float* Y, float* part, int ldy, int* S_out, hipStream_t st, const NormArgs& norm, bool stream = true) {
  int KS = 0;
  if (stream && td_block_stream_ok(fmt, M)) {
    int nt = 0, xc = 0;
    const int S = td_block_stream_plan(N, K, ncu, &nt, &xc);
    KS = 64 * xc;
    *S_out = S;
    float* dst = S == 1 ? Y : part;
    const size_t sstride = (size_t)M * ldy;
    const dim3 grid((N + 16 * nt - 1) / (16 * nt), S);
    if (nt == 16)
      return xc == 8   ? launch_stream<16, 8>(grid, st, X, ldx, M, K, KS, W, N, dst, ldy, sstride, norm)
             : xc == 4 ? launch_stream<16, 4>(grid, st, X, ldx, M, K, KS, W, N, dst, ldy, sstride, norm)
                       : launch_stream<16, 2>(grid, st, X, ldx, M, K, KS, W, N, dst, ldy, sstride, norm);
    return xc == 8   ? launch_stream<8, 8>(grid, st, X, ldx, M, K, KS, W, N, dst, ldy, sstride, norm)
           : xc == 4 ? launch_stream<8, 4>(grid, st, X, ldx, M, K, KS, W, N, dst, ldy, sstride, norm)
                     : launch_stream<8, 2>(grid, st, X, ldx, M, K, KS, W, N, dst, ldy, sstride, norm);
  }
  const int NB = nb_of((M + 15) / 16, N, ncu);
  const int S = td_block_split(N, K, ncu, 64 * NB, fmt, &KS);
  *S_out = S;
  float* dst = S == 1 ? Y : part;
  const size_t sstride = (size_t)M * ldy;
  return fmt ? launch_gemm_f<TD_WF_INT4_G64>(S, NB, N, st, X, ldx, M, K, KS, W, Sc, dst, ldy, sstride, norm)
             : launch_gemm_f<TD_WF_BF16>(S, NB, N, st, X, ldx, M, K, KS, W, Sc, dst, ldy, sstride, norm);
}

template <int D>
int launch_attn(const td_kparams& P, const td_blockparams* B, int n, int l, int pos0, hipStream_t st) {
  const int rows = n * P.group, nx = (rows + 15) / 16;
  const int nsplit = td_block_attn_split(nx * P.nkv, (pos0 + n - 1) / 32 + 1, B->ncu);
  blk_attn_mma<D><<<dim3(nx * P.nkv * nsplit), 512, 0, st>>>(B->q, P.kc, P.vc, P.nq, P.group, P.nkv, P.max_ctx, l,
                                                             pos0, n, nsplit, B->part, B->ao);
  if (nsplit > 1)
    blk_attn_merge<D><<<dim3((rows + 512 / D - 1) / (512 / D), P.nkv), 512, 0, st>>>(B->part, nsplit, P.nq, P.group,
                                                                                     P.nkv, n, B->ao);
  return (int)hipGetLastError();
}

}  // namespace

int td_block_prepare() {
  static int rc = -1;  // once per process (the attribute belongs to the function, on every device)
  if (rc < 0) {
    rc = prepare_stream<16, 8>();
    if (!rc) rc = prepare_stream<16, 4>();
    if (!rc) rc = prepare_stream<16, 2>();
    if (!rc) rc = prepare_stream<8, 8>();
    if (!rc) rc = prepare_stream<8, 4>();
    if (!rc) rc = prepare_stream<8, 2>();
  }
  return rc;
}

int td_launch_block(const td_blockparams* B, const int32_t* tokens, int n, int pos0, int all_logits,
                    float* logits, int32_t* argmax_out, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const td_kparams& P = *B->kp;
  const int H = P.H, I = P.I, d = P.d, qd = P.qd, L = P.L, ncu = B->ncu;
  float* part = B->part;
  int e = 0, S = 0, S_prev = 0;
#define TD_CK(x)                      \
  do {                                \
    x;                                \
    e = (int)hipGetLastError();       \
    if (e) return e;                  \
  } while (0)
  const int hb = H / 256;  // column blocks of the residual stream (H is a multiple of 256)
  const dim3 rgrid(hb, n);
  const NormArgs no_norm{nullptr, 0, 0.f}, norm{B->ssq, hb, P.eps};
  TD_CK((blk_embed<<<n, 256, 0, st>>>(P.embed, tokens, H, P.V, B->x, P.err)));
  for (int l = 0; l < L; ++l) {
    const td_layer_dev& Ld = B->layers_host[l];
    // x += the previous layer's down-projection slices; attention RMSNorm
    TD_CK((blk_resid<<<rgrid, 256, 0, st>>>(B->x, part, S_prev, (size_t)n * H, H, Ld.attn_norm, B->xg, B->ssq)));
    if ((e = gemm(P.wf, ncu, B->xg, H, n, H, Ld.w[0], Ld.s[0], P.qkv_rows, B->y, part, P.qkv_rows, &S, st, norm)))
      return e;
    TD_CK((blk_qkv_post<<<dim3((P.qkv_rows / 2 + 255) / 256, n), 256, 0, st>>>(
        S == 1 ? B->y : part, S, (size_t)n * P.qkv_rows, P.qkv_rows, qd, P.kvd, d, P.nkv, P.max_ctx, l, pos0, Ld.bias,
        P.rope_cs, P.attn_scale, B->q, P.kc, P.vc)));
    if ((e = d == 64 ? launch_attn<64>(P, B, n, l, pos0, st) : launch_attn<128>(P, B, n, l, pos0, st))) return e;
    // the O and down projections always land in part (slice 0 when unsplit)
    if ((e = gemm(P.wf, ncu, B->ao, qd, n, qd, Ld.w[1], Ld.s[1], H, part, part, H, &S, st, no_norm))) return e;
    TD_CK((blk_resid<<<rgrid, 256, 0, st>>>(B->x, part, S, (size_t)n * H, H, Ld.mlp_norm, B->xg, B->ssq)));
    if ((e = gemm(P.wf, ncu, B->xg, H, n, H, Ld.w[2], Ld.s[2], 2 * I, B->y, part, 2 * I, &S, st, norm))) return e;
    TD_CK((blk_swiglu<<<dim3((I + 255) / 256, n), 256, 0, st>>>(S == 1 ? B->y : part, S, (size_t)n * 2 * I, I,
                                                               B->act)));
    if ((e = gemm(P.wf, ncu, B->act, I, n, I, Ld.w[3], Ld.s[3], H, part, part, H, &S_prev, st, no_norm))) return e;
  }
  TD_CK((blk_resid<<<rgrid, 256, 0, st>>>(B->x, part, S_prev, (size_t)n * H, H, P.final_norm, B->xg, B->ssq)));
  const int r0 = all_logits ? 0 : n - 1, rows = all_logits ? n : 1;
  if ((e = gemm(TD_WF_BF16, ncu, B->xg + (size_t)r0 * H, H, rows, H, (const uint8_t*)P.head, nullptr, P.V, logits,
                part, P.V, &S, st, NormArgs{B->ssq + (size_t)r0 * hb, hb, P.eps}, false)))
    return e;
  if (S > 1) TD_CK((blk_sum_parts<<<dim3((P.V + 255) / 256, rows), 256, 0, st>>>(part, S, (size_t)rows * P.V, P.V,
                                                                                 logits)));
  const int ch = (P.V + TD_BLOCK_ARGMAX_SLICES - 1) / TD_BLOCK_ARGMAX_SLICES;
  TD_CK((blk_argmax_part<<<dim3(TD_BLOCK_ARGMAX_SLICES, rows), 256, 0, st>>>(logits, P.V, ch, B->cand, P.err)));
  TD_CK((blk_argmax_final<<<(rows + 63) / 64, 64, 0, st>>>(B->cand, TD_BLOCK_ARGMAX_SLICES, rows, argmax_out,
                                                           P.token_out)));
#undef TD_CK
  return 0;
}
