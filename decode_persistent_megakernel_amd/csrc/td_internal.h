// td_internal.h - device-side parameter block and layout constants shared by
// the host API (td_api.cpp) and the kernels (td_kernels.hip).
#pragma once
#include <stdint.h>

#define TD_NW 8                       // compute waves per workgroup
#define TD_WAVE 64
#define TD_THREADS ((TD_NW + 1) * TD_WAVE)  // + one sync wave
#define TD_TILE 64                    // attention positions per LDS tile
#define TD_CHUNK 1024                 // bytes per wave-wide weight chunk (64 lanes x 16 B)
#define TD_SCHUNK 256                 // bytes per int4 scale chunk (64 lanes x 4 B)
#define TD_MAX_GROUP 8                // query heads per kv head handled by one task
#define TD_SPIN_TICKS 100000000ull    // grid-wait limit in 100 MHz ticks (1 s)

// stage kinds, in layer order; the head follows the last layer
enum { TD_ST_QKV = 0, TD_ST_ATTN = 1, TD_ST_O = 2, TD_ST_GU = 3, TD_ST_DOWN = 4, TD_ST_HEAD = 5 };

// error bits of the device error word
enum { TD_ERRBIT_NONFINITE = 1, TD_ERRBIT_RANGE = 2, TD_ERRBIT_TIMEOUT = 4 };

// uint32 word offsets inside the sync area; each group on its own 256 B line(s)
enum {
  TD_SY_EPOCH = 0,
  TD_SY_GCTR = 64,
  TD_SY_XCTR = 128,            // 8 lines: per-XCD arrival counters
  TD_SY_XREL = 128 + 8 * 64,   // 8 lines: per-XCD release words
  TD_SY_ABORT = 128 + 16 * 64,
  TD_SY_FINAL = TD_SY_ABORT + 64,
  TD_SY_MERGE = TD_SY_FINAL + 64  // n_layers * n_kv_heads attention-merge counters
};

struct td_layer_dev {
  const uint8_t* w[4];     // QKV, O, GU, DOWN
  const uint16_t* s[4];    // fp16 scales (int4) or null
  const uint16_t* bias;    // bf16 QKV bias or null
  const uint16_t* attn_norm;
  const uint16_t* mlp_norm;
};

struct td_kparams {
  // shape
  int32_t L, H, nq, nkv, d, I, V, max_ctx, wf, has_bias;
  int32_t qd, kvd, qkv_rows, group;
  float eps, attn_scale;
  // attention split
  int32_t chunk_len, n_chunks_max;
  // step
  int32_t pos;
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
  // scratch (ctx-owned)
  float* x;      // [H] residual stream
  float* q;      // [nq d]
  float* o;      // [nq d] merged attention output
  float* act;    // [I]
  float* part;   // [nkv][n_chunks_max][group][d + 2]
  uint32_t* cand;  // [ncu][4]: value bits, index, nonfinite
  uint32_t* sync;
  int32_t* token_out;
  int32_t* err;
  // LDS layout (byte offsets into dynamic shared memory)
  int32_t off_ring, off_sring, off_xin, off_out, off_own, off_attn;
  int32_t lds_bytes;
  int32_t n_stages;   // 5 L + 1
};

// LDS offsets inside the attention area (bytes, relative to off_attn)
struct td_attn_lds {
  int32_t q, k, v, p, part, bytes;
};

#ifdef __HIPCC__
__host__ __device__
#endif
static inline td_attn_lds td_attn_layout(int d, int group) {
  td_attn_lds a;
  a.q = 0;
  a.k = a.q + group * d * 4;
  a.v = a.k + TD_TILE * (d + 8) * 2;
  a.p = a.v + TD_TILE * d * 2;
  a.part = a.p + group * TD_TILE * 4;
  a.bytes = a.part + group * (d + 2) * 4;
  a.bytes = (a.bytes + 255) & ~255;
  return a;
}

// launch entry points (td_kernels.hip)
int td_launch_megakernel(const td_kparams* p, int ncu, int ring_slots, void* stream);
int td_megakernel_occupancy(int ring_slots, int lds_bytes, int* blocks_per_cu);
int td_launch_test_gemv(int fmt, const void* w, const void* s, int rows, int cols, const float* x, float* y,
                        void* stream);
int td_launch_test_attention(const float* q, const void* k, const void* v, int n, int d, float* out,
                             void* stream);
