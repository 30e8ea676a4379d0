// td_bench: native driver of the decode step on one GPU, with no Python and
// no PyTorch in the process.  It builds the same seeded random-init model as
// the Python workloads (through libsynth), uploads it, fills the K/V cache
// (prompt prefilled through the decode step itself, or a random prefix), then
// runs W untimed and K timed greedy decode steps and prints one JSON line with
// the mean step time measured by HIP events on the step's stream.
//
// It exists so that a kernel profiler can be attached to a process that holds
// nothing but the HIP runtime and this library.
//
// --copy-calibration adds one plain 1 GiB device-to-device copy after the
// timed steps: a transfer of known size, against which hardware byte
// counters read on the decode kernel can be scaled.
//
// --executor megakernel|per_op|graph picks the executor behind td_decode_step.
//
// --loop N runs the steps through td_decode_loop, N greedy steps per launch
// (the last launch takes the remainder), instead of one td_decode_step each
// (persistent executor only).
//
// --block N fills the prompt through td_forward_block, N tokens per call,
// instead of one decode step per token, and times that prefill (one untimed
// pass, then three timed passes over the same positions) on its own JSON line.
// A workload with a random cache prefix and no prompt times one block of N
// tokens at the first decode position instead (the shape of a draft verify).
//
// --maps FILE writes the process's memory map (/proc/self/maps) to FILE at the
// end of main, so that addresses in a crash report from the exit-time
// teardown can be matched to the library they fall in.
//
//   td_bench [--config NAME] [--steps K] [--warmup W] [--executor E] [--loop N] [--block N]
//            [--copy-calibration] [--print-config] [--maps FILE]
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "td.h"

extern "C" {
uint64_t synth_key(uint64_t seed, int32_t layer, const char* name);
void synth_fill_bf16_normal(uint16_t* out, int64_t n, uint64_t key, double mean, double std);
void synth_fill_bf16_const(uint16_t* out, int64_t n, float v);
void synth_fill_f16_absnormal(uint16_t* out, int64_t n, uint64_t key, double std);
void synth_fill_u8_uniform(uint8_t* out, int64_t n, uint64_t key);
void synth_fill_i32_uniform(int32_t* out, int64_t n, uint64_t key, int32_t hi);
}

namespace {

struct Workload {
  const char* name;
  int layers, hidden, nq, nkv, d, inter, vocab;
  double theta, eps;
  int wf, bias, tied, prompt, kv_prefix, steps, max_ctx, seed;
  int n_experts = 0, top_k = 0;  // mixture of experts (0: dense MLP)
};

// The workloads (same shapes, formats and seeds as the Python definitions).
const Workload kWorkloads[] = {
    {"tiny", 2, 256, 4, 2, 64, 1024, 4096, 10000.0, 1e-5, TD_WF_BF16, 0, 1, 16, 0, 16, 32, 1000},
    {"llama1b", 16, 2048, 32, 8, 64, 8192, 128256, 500000.0, 1e-5, TD_WF_BF16, 0, 1, 512, 0, 128, 640, 1001},
    {"tinyllama_int4", 22, 2048, 32, 4, 64, 5632, 32000, 10000.0, 1e-5, TD_WF_INT4_G64, 0, 0, 256, 0, 128, 384,
     1002},
    {"qwen1p5b", 28, 1536, 12, 2, 128, 8960, 151936, 1e6, 1e-6, TD_WF_BF16, 1, 1, 1024, 0, 64, 1088, 1003},
    {"llama1b_int4_long", 16, 2048, 32, 8, 64, 8192, 128256, 500000.0, 1e-5, TD_WF_INT4_G64, 0, 1, 0, 8192, 64,
     8256, 1004},
    {"olmoe", 16, 2048, 16, 16, 128, 1024, 50304, 10000.0, 1e-5, TD_WF_BF16, 0, 0, 0, 512, 64, 576, 1005, 64, 8},
};

constexpr double kWeightStd = 0.02, kScaleStd = 0.003, kKvStd = 1.0;

#define CK(x)                                                                                  \
  do {                                                                                         \
    hipError_t e_ = (x);                                                                       \
    if (e_ != hipSuccess) {                                                                    \
      fprintf(stderr, "td_bench: %s failed: %s\n", #x, hipGetErrorString(e_));                 \
      exit(1);                                                                                 \
    }                                                                                          \
  } while (0)
#define TD(x)                                                                                  \
  do {                                                                                         \
    int r_ = (x);                                                                              \
    if (r_ != TD_OK) {                                                                         \
      fprintf(stderr, "td_bench: %s -> %s (%s)\n", #x, td_strerror(r_), td_last_error());      \
      exit(1);                                                                                 \
    }                                                                                          \
  } while (0)

std::vector<void*> g_allocs;

void* upload(const void* host, size_t bytes) {
  void* d = nullptr;
  CK(hipMalloc(&d, bytes));
  CK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  g_allocs.push_back(d);
  return d;
}

void* bf16_normal_dev(int64_t n, uint64_t key, double std) {
  std::vector<uint16_t> h(n);
  synth_fill_bf16_normal(h.data(), n, key, 0.0, std);
  return upload(h.data(), n * 2);
}

void* bf16_const_dev(int64_t n, float v) {
  std::vector<uint16_t> h(n);
  synth_fill_bf16_const(h.data(), n, v);
  return upload(h.data(), n * 2);
}

// One linear layer [rows][cols]: bf16 N(0, 0.02), or int4 codes plus fp16 scales.
void linear_dev(const Workload& w, int layer, const char* name, int64_t rows, int64_t cols, const void** wp,
                const void** sp) {
  const uint64_t k = synth_key(w.seed, layer, name);
  if (w.wf == TD_WF_BF16) {
    *wp = bf16_normal_dev(rows * cols, k, kWeightStd);
    *sp = nullptr;
    return;
  }
  std::vector<uint8_t> codes(rows * cols / 2);
  synth_fill_u8_uniform(codes.data(), (int64_t)codes.size(), k);
  *wp = upload(codes.data(), codes.size());
  std::vector<uint16_t> sc(rows * cols / 64);
  const std::string sname = std::string(name) + ".scale";
  synth_fill_f16_absnormal(sc.data(), (int64_t)sc.size(), synth_key(w.seed, layer, sname.c_str()), kScaleStd);
  *sp = upload(sc.data(), sc.size() * 2);
}

void print_config(const Workload& w) {
  printf("{\"name\": \"%s\", \"n_layers\": %d, \"hidden\": %d, \"n_q_heads\": %d, \"n_kv_heads\": %d, "
         "\"head_dim\": %d, \"intermediate\": %d, \"vocab\": %d, \"rope_theta\": %.17g, \"rms_eps\": %.17g, "
         "\"weight_format\": %d, \"qkv_bias\": %d, \"tied\": %d, \"prompt_len\": %d, \"kv_prefix\": %d, "
         "\"decode_steps\": %d, \"max_ctx\": %d, \"seed\": %d, \"n_experts\": %d, \"top_k\": %d}\n",
         w.name, w.layers, w.hidden, w.nq, w.nkv, w.d, w.inter, w.vocab, w.theta, w.eps, w.wf, w.bias, w.tied,
         w.prompt, w.kv_prefix, w.steps, w.max_ctx, w.seed, w.n_experts, w.top_k);
}

}  // namespace

int main(int argc, char** argv) {
  std::string name = "llama1b";
  int steps = 128, warmup = 8;
  bool only_config = false, copy_cal = false;
  std::string maps_path;
  int loop_n = 0, block_n = 0;
  int executor = TD_EXEC_MEGAKERNEL;
  std::string ex_name = "megakernel";
  for (int i = 1; i < argc; ++i) {
    const std::string a = argv[i];
    if (a == "--config" && i + 1 < argc) name = argv[++i];
    else if (a == "--steps" && i + 1 < argc) steps = atoi(argv[++i]);
    else if (a == "--warmup" && i + 1 < argc) warmup = atoi(argv[++i]);
    else if (a == "--print-config") only_config = true;
    else if (a == "--copy-calibration") copy_cal = true;
    else if (a == "--loop" && i + 1 < argc) loop_n = atoi(argv[++i]);
    else if (a == "--block" && i + 1 < argc) block_n = atoi(argv[++i]);
    else if (a == "--maps" && i + 1 < argc) maps_path = argv[++i];
    else if (a == "--executor" && i + 1 < argc) {
      ex_name = argv[++i];
      if (ex_name == "megakernel") executor = TD_EXEC_MEGAKERNEL;
      else if (ex_name == "per_op") executor = TD_EXEC_PER_OP;
      else if (ex_name == "graph") executor = TD_EXEC_GRAPH;
      else {
        fprintf(stderr, "td_bench: unknown executor %s\n", ex_name.c_str());
        return 2;
      }
    }
    else {
      fprintf(stderr, "usage: td_bench [--config NAME] [--steps K] [--warmup W] [--executor E] [--loop N] "
                      "[--block N] [--copy-calibration] [--print-config]\n");
      return 2;
    }
  }
  const Workload* wp = nullptr;
  for (const Workload& w : kWorkloads)
    if (name == w.name) wp = &w;
  if (!wp) {
    fprintf(stderr, "td_bench: unknown workload %s\n", name.c_str());
    return 2;
  }
  const Workload& w = *wp;
  if (w.n_experts > 0 && block_n > 0) {
    fprintf(stderr, "td_bench: --block runs dense models only\n");
    return 2;
  }
  if (only_config) {
    print_config(w);
    return 0;
  }
  const int start = w.prompt + w.kv_prefix;
  if (block_n < 0 || block_n > TD_MAX_BLOCK) {
    fprintf(stderr, "td_bench: --block takes 1..%d\n", TD_MAX_BLOCK);
    return 2;
  }
  if (steps < 1 || warmup < 0 || start + steps > w.max_ctx || start + warmup > w.max_ctx) {
    fprintf(stderr, "td_bench: steps/warmup do not fit the cache (%d positions after the prefix)\n",
            w.max_ctx - start);
    return 2;
  }

  // model
  const int64_t H = w.hidden, I = w.inter, V = w.vocab, qd = (int64_t)w.nq * w.d;
  const int64_t qkv_rows = (int64_t)(w.nq + 2 * w.nkv) * w.d;
  td_config cfg{};
  cfg.n_layers = w.layers;
  cfg.hidden = w.hidden;
  cfg.n_q_heads = w.nq;
  cfg.n_kv_heads = w.nkv;
  cfg.head_dim = w.d;
  cfg.intermediate = w.inter;
  cfg.vocab = w.vocab;
  cfg.max_ctx = w.max_ctx;
  cfg.rope_theta = (float)w.theta;
  cfg.rms_eps = (float)w.eps;
  cfg.weight_format = w.wf;
  cfg.qkv_bias = w.bias;
  cfg.n_experts = w.n_experts;
  cfg.top_k = w.top_k;
  const int64_t E = std::max(1, w.n_experts);
  td_weights tw{};
  tw.embed = bf16_normal_dev(V * H, synth_key(w.seed, -1, "embed"), kWeightStd);
  tw.head = w.tied ? tw.embed : bf16_normal_dev(V * H, synth_key(w.seed, -1, "head"), kWeightStd);
  tw.final_norm = bf16_const_dev(H, 1.0f);
  std::vector<td_layer_weights> layers(w.layers);
  for (int l = 0; l < w.layers; ++l) {
    td_layer_weights& L = layers[l];
    L.attn_norm = bf16_const_dev(H, 1.0f);
    L.mlp_norm = bf16_const_dev(H, 1.0f);
    L.b_qkv = w.bias ? bf16_normal_dev(qkv_rows, synth_key(w.seed, l, "qkv_bias"), kWeightStd) : nullptr;
    linear_dev(w, l, "qkv", qkv_rows, H, &L.w_qkv, &L.s_qkv);
    linear_dev(w, l, "o", H, qd, &L.w_o, &L.s_o);
    linear_dev(w, l, "gate_up", E * 2 * I, H, &L.w_gu, &L.s_gu);
    linear_dev(w, l, "down", E * H, I, &L.w_d, &L.s_d);
    L.w_router = w.n_experts ? bf16_normal_dev(E * H, synth_key(w.seed, l, "router"), kWeightStd) : nullptr;
  }
  tw.layers = layers.data();

  // K/V cache [L][nkv][max_ctx][d], zero, with a random prefix when asked
  const size_t head_rows = (size_t)w.max_ctx * w.d;
  const size_t kv_elems = (size_t)w.layers * w.nkv * head_rows;
  void *kc = nullptr, *vc = nullptr;
  CK(hipMalloc(&kc, kv_elems * 2));
  CK(hipMalloc(&vc, kv_elems * 2));
  g_allocs.push_back(kc);
  g_allocs.push_back(vc);
  CK(hipMemset(kc, 0, kv_elems * 2));
  CK(hipMemset(vc, 0, kv_elems * 2));
  if (w.kv_prefix) {
    std::vector<uint16_t> h((size_t)w.kv_prefix * w.d);
    for (int l = 0; l < w.layers; ++l)
      for (int g = 0; g < w.nkv; ++g) {
        const size_t off = ((size_t)l * w.nkv + g) * head_rows * 2;
        synth_fill_bf16_normal(h.data(), (int64_t)h.size(), synth_key(w.seed, l * 1000 + g, "k_prefix"), 0.0,
                               kKvStd);
        CK(hipMemcpy((uint8_t*)kc + off, h.data(), h.size() * 2, hipMemcpyHostToDevice));
        synth_fill_bf16_normal(h.data(), (int64_t)h.size(), synth_key(w.seed, l * 1000 + g, "v_prefix"), 0.0,
                               kKvStd);
        CK(hipMemcpy((uint8_t*)vc + off, h.data(), h.size() * 2, hipMemcpyHostToDevice));
      }
  }
  td_kv kv{kc, vc, w.max_ctx};

  td_ctx* ctx = nullptr;
  TD(td_create(&cfg, &tw, executor, &ctx));
  hipStream_t stream;
  CK(hipStreamCreate(&stream));
  float* logits = nullptr;
  int32_t* tok = nullptr;
  CK(hipMalloc(&logits, V * 4));
  CK(hipMalloc(&tok, 4));
  g_allocs.push_back(logits);
  g_allocs.push_back(tok);

  // the prompt in blocks (timed), through the decode step, or the first token after a random prefix
  if (block_n > 0) {
    const int n_tok = w.prompt ? w.prompt : block_n;
    const int p0 = w.prompt ? 0 : start;
    if (p0 + n_tok > w.max_ctx) {
      fprintf(stderr, "td_bench: the block does not fit the cache\n");
      return 2;
    }
    std::vector<int32_t> toks(n_tok);
    if (w.prompt) synth_fill_i32_uniform(toks.data(), n_tok, synth_key(w.seed, -1, "prompt"), w.vocab);
    else synth_fill_i32_uniform(toks.data(), n_tok, synth_key(w.seed, -1, "block"), w.vocab);
    int32_t* d_toks = nullptr;
    CK(hipMalloc(&d_toks, (size_t)n_tok * 4));
    g_allocs.push_back(d_toks);
    CK(hipMemcpy(d_toks, toks.data(), (size_t)n_tok * 4, hipMemcpyHostToDevice));
    auto pass = [&]() {
      for (int i = 0; i < n_tok; i += block_n)
        TD(td_forward_block(ctx, d_toks + i, std::min(block_n, n_tok - i), p0 + i, &kv, logits, 0, nullptr, stream));
    };
    pass();
    CK(hipStreamSynchronize(stream));
    TD(td_status(ctx, nullptr));
    hipEvent_t b0, b1;
    CK(hipEventCreate(&b0));
    CK(hipEventCreate(&b1));
    const int reps = 3;
    CK(hipEventRecord(b0, stream));
    for (int r = 0; r < reps; ++r) pass();
    CK(hipEventRecord(b1, stream));
    CK(hipStreamSynchronize(stream));
    TD(td_status(ctx, nullptr));
    float ms = 0.f;
    CK(hipEventElapsedTime(&ms, b0, b1));
    ms /= reps;
    printf("{\"workload\": \"%s\", \"block_rows\": %d, \"tokens\": %d, \"positions\": [%d, %d], "
           "\"ms_per_pass\": %.4f, \"tokens_per_s\": %.1f}\n",
           w.name, block_n, n_tok, p0, p0 + n_tok - 1, ms, n_tok / (ms / 1e3));
    fflush(stdout);
    CK(hipEventDestroy(b0));
    CK(hipEventDestroy(b1));
    if (!w.prompt) {
      int32_t first = 0;
      synth_fill_i32_uniform(&first, 1, synth_key(w.seed, -1, "first_token"), w.vocab);
      CK(hipMemcpy(tok, &first, 4, hipMemcpyHostToDevice));
    }
  } else if (w.prompt) {
    std::vector<int32_t> prompt(w.prompt);
    synth_fill_i32_uniform(prompt.data(), w.prompt, synth_key(w.seed, -1, "prompt"), w.vocab);
    for (int i = 0; i < w.prompt; ++i) {
      CK(hipMemcpyAsync(tok, &prompt[i], 4, hipMemcpyHostToDevice, stream));
      CK(hipStreamSynchronize(stream));
      TD(td_decode_step(ctx, tok, i, &kv, logits, stream));
    }
  } else {
    int32_t first = 0;
    synth_fill_i32_uniform(&first, 1, synth_key(w.seed, -1, "first_token"), w.vocab);
    CK(hipMemcpy(tok, &first, 4, hipMemcpyHostToDevice));
  }
  CK(hipStreamSynchronize(stream));
  TD(td_status(ctx, nullptr));
  int32_t first_tok = 0;
  CK(hipMemcpy(&first_tok, w.prompt ? td_token_ptr(ctx) : tok, 4, hipMemcpyDeviceToHost));
  CK(hipMemcpy(tok, &first_tok, 4, hipMemcpyHostToDevice));

  // one launch per step, or loops of loop_n steps; events bracket every launch
  auto launches_of = [&](int n) { return loop_n > 0 ? (n + loop_n - 1) / loop_n : n; };
  auto run = [&](int n, std::vector<hipEvent_t>* ev) {
    int li = 0;
    for (int i = 0; i < n; ++li) {
      const int m = loop_n > 0 ? std::min(loop_n, n - i) : 1;
      if (ev) CK(hipEventRecord((*ev)[2 * li], stream));
      const int32_t* t = i == 0 ? tok : td_token_ptr(ctx);
      if (loop_n > 0) TD(td_decode_loop(ctx, t, start + i, m, -1, &kv, logits, nullptr, nullptr, stream));
      else TD(td_decode_step(ctx, t, start + i, &kv, logits, stream));
      if (ev) CK(hipEventRecord((*ev)[2 * li + 1], stream));
      i += m;
    }
  };
  run(warmup, nullptr);
  CK(hipStreamSynchronize(stream));
  TD(td_status(ctx, nullptr));
  const int nl = launches_of(steps);
  std::vector<hipEvent_t> ev(2 * nl);
  for (auto& e : ev) CK(hipEventCreate(&e));
  run(steps, &ev);
  CK(hipStreamSynchronize(stream));
  TD(td_status(ctx, nullptr));
  double total = 0.0;
  for (int i = 0; i < nl; ++i) {
    float ms = 0.f;
    CK(hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]));
    total += ms;
  }
  printf("{\"workload\": \"%s\", \"executor\": \"%s\", \"steps\": %d, \"warmup\": %d, \"steps_per_launch\": %d, "
         "\"positions\": [%d, %d], \"ms_per_step\": %.4f, \"tokens_per_s\": %.2f}\n",
         w.name, ex_name.c_str(), steps, warmup, loop_n > 0 ? loop_n : 1, start, start + steps - 1, total / steps,
         steps / (total / 1e3));
  fflush(stdout);

  if (copy_cal) {
    const size_t bytes = (size_t)1 << 30;
    void *a = nullptr, *b = nullptr;
    CK(hipMalloc(&a, bytes));
    CK(hipMalloc(&b, bytes));
    CK(hipMemsetAsync(a, 1, bytes, stream));
    CK(hipMemcpyAsync(b, a, bytes, hipMemcpyDeviceToDevice, stream));
    CK(hipStreamSynchronize(stream));
    CK(hipFree(a));
    CK(hipFree(b));
    printf("{\"copy_calibration_bytes\": %zu}\n", bytes);
    fflush(stdout);
  }
  for (auto& e : ev) CK(hipEventDestroy(e));
  td_destroy(ctx);
  CK(hipStreamDestroy(stream));
  for (void* p : g_allocs) CK(hipFree(p));
  if (!maps_path.empty()) {  // the process's mappings at the end of main (which library sits where)
    FILE* in = fopen("/proc/self/maps", "r");
    FILE* out = fopen(maps_path.c_str(), "w");
    if (in && out) {
      char line[4096];
      while (fgets(line, sizeof line, in)) fputs(line, out);
    }
    if (in) fclose(in);
    if (out) fclose(out);
  }
  return 0;
}
