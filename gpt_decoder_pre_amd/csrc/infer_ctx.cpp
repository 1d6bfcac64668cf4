// Decoding context (gpt2_infer.h): prefill and one-token steps through the
// step's forward kernels with a key / value cache, and the sampler.
#include "gpt2_infer.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>

#include "common.h"
#include "infer_kernels.h"
#include "kernels.h"

using namespace gpt2k;

struct gpt2_infer {
  gpt2_config cfg;
  bool ops16;  // 16-bit MFMA operands and activations (bf16; decoding has no fp16 mode)
  int L, C, NH, V, Vp, Bmax, Tmax;
  int64_t act;
  const float* params;
  const char* pbf16;
  std::map<std::string, int64_t> off;  // tensor name -> element offset
  std::map<std::string, int64_t> per;  // elements of one block's tensor
  hipStream_t stream;
  char* cache;
  // workspace
  float *x0, *x1, *mean, *rstd, *lse;
  char *ln, *qkv, *atty, *fcgd, *fcg, *lnf, *last;
  int32_t* ids;
  int* err;
  int B = 0, len = -1;

  bool has(const char* n) const { return off.count(n) > 0; }
  const float* P(const char* n, int l = 0) const { return params + off.at(n) + (int64_t)l * per.at(n); }
  const void* W(const char* n, int l = 0) const {
    const int64_t o = off.at(n) + (int64_t)l * per.at(n);
    return ops16 ? (const void*)(pbf16 + 2 * o) : (const void*)(params + o);
  }
  char* cache_l(int l) const { return cache + (int64_t)l * Bmax * Tmax * 2 * C * act; }
};

namespace {

int64_t plan(gpt2_infer* c, char* base) {
  const int64_t M = (int64_t)c->Bmax * c->Tmax, C = c->C, A = c->act;
  int64_t o = 0;
  auto take = [&](int64_t bytes) -> char* {
    char* p = base ? base + o : nullptr;
    o += (bytes + 255) / 256 * 256;
    return p;
  };
  c->x0 = (float*)take(M * C * 4);
  c->x1 = (float*)take(M * C * 4);
  c->mean = (float*)take(M * 4);
  c->rstd = (float*)take(M * 4);
  c->lse = (float*)take(M * c->NH * 4);
  c->ln = take(M * C * A);
  c->qkv = take(M * 3 * C * A);
  c->atty = take(M * C * A);
  c->fcgd = take(M * 4 * C * A);
  c->fcg = take(M * 4 * C * A);
  c->lnf = take(M * C * A);
  c->last = take((int64_t)c->Bmax * C * A);
  c->ids = (int32_t*)take(M * 4);
  c->err = (int*)take(256);
  return o;
}

GemmArgs args(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K, void* Cp, int64_t ldc) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = A;
  a.B = B;
  a.lda = lda;
  a.ldb = ldb;
  a.M = M;
  a.N = N;
  a.K = K;
  a.C = Cp;
  a.ldc = ldc;
  a.splits = 1;
  a.k_per_split = K;
  return a;
}

int hip_ok() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    fprintf(stderr, "gpt2_infer: HIP error: %s\n", hipGetErrorString(e));
    return GPT2_ERR_HIP;
  }
  return GPT2_OK;
}

// A product of the forward pass: the skinny kernel for the few rows of a
// decoding step in bf16 mode, else the step's GEMM.
bool product(gpt2_infer* c, GemmEpilogue epi, const GemmArgs& g, hipStream_t s) {
  if (c->ops16 && g.M <= 32 && gemm_skinny(epi, g, s)) return true;
  return gemm(LAYOUT_NT, epi, c->ops16, g, s);
}

// The blocks, final LayerNorm and lm_head over M = B T rows (prefill, T > 1
// or len == 0) or B rows at position len (decode), from x0 (the embeddings).
template <typename TA>
int forward(gpt2_infer* c, int B, int T, bool decode, float* d_logits) {
  hipStream_t s = c->stream;
  const int C = c->C, M = B * T;
  const bool bf = c->ops16;
  float* xa = c->x0;
  float* xb = c->x1;
  TA* ln = (TA*)c->ln;
  TA* qkv = (TA*)c->qkv;
  TA* atty = (TA*)c->atty;
  // a bf16 decoding step of at most 16 sequences forms each LayerNorm in the
  // prologue of the product that reads it, from the fp32 residual rows
  const bool ln_pro = decode && bf && M <= 16;
  for (int l = 0; l < c->L; ++l) {
    GemmArgs g = args(ln, C, c->W("qkv_w", l), C, M, 3 * C, C, qkv, 3 * C);
    g.bias = c->has("qkv_b") ? c->P("qkv_b", l) : nullptr;
    TA* cache = (TA*)c->cache_l(l);
    // a bf16 decoding step stores the new keys and values from the QKV
    // product's epilogue
    bool kv_fused = ln_pro && gemm_skinny_ln(EPI_ACT, g, xa, c->P("ln1_w", l), c->P("ln1_b", l), s, (h16*)cache,
                                             c->Tmax, c->len, C);
    if (!kv_fused) {
      layernorm_fwd<TA>(xa, c->P("ln1_w", l), c->P("ln1_b", l), ln, c->mean, c->rstd, M, C, s);
      kv_fused = decode && bf && M <= 32 && gemm_skinny(EPI_ACT, g, s, (h16*)cache, c->Tmax, c->len, C);
      if (!kv_fused && !product(c, EPI_ACT, g, s)) return GPT2_ERR_ARG;
    }
    if (decode) {
      if (!kv_fused) kv_store<TA>(qkv, cache, B, 1, c->len, c->Tmax, C, s);
      if (!decode_attn<TA>(qkv, cache, atty, B, c->len + 1, c->Tmax, C, c->NH, s)) return GPT2_ERR_ARG;
    } else {
      kv_store<TA>(qkv, cache, B, T, 0, c->Tmax, C, s);
      if (bf) attn_fwd_bf16(qkv, atty, c->lse, B, T, c->NH, C, s);
      else attn_fwd_f32((const float*)qkv, (float*)atty, c->lse, B, T, c->NH, C, s);
    }
    g = args(atty, C, c->W("proj_w", l), C, M, C, C, xb, C);
    g.bias = c->P("proj_b", l);
    g.resid = xa;
    if (!product(c, EPI_RESID, g, s)) return GPT2_ERR_ARG;
    g = args(ln, C, c->W("fc_w", l), C, M, 4 * C, C, c->fcgd, 4 * C);
    g.bias = c->P("fc_b", l);
    g.C2 = c->fcg;
    if (!(ln_pro && gemm_skinny_ln(EPI_GELU, g, xb, c->P("ln2_w", l), c->P("ln2_b", l), s))) {
      layernorm_fwd<TA>(xb, c->P("ln2_w", l), c->P("ln2_b", l), ln, c->mean, c->rstd, M, C, s);
      if (!product(c, EPI_GELU, g, s)) return GPT2_ERR_ARG;
    }
    g = args(c->fcg, 4 * C, c->W("fcproj_w", l), 4 * C, M, C, 4 * C, xa, C);
    g.bias = c->P("fcproj_b", l);
    g.resid = xb;
    if (!product(c, EPI_RESID, g, s)) return GPT2_ERR_ARG;
  }
  // the final LayerNorm stays a launch of its own: lm_head's thousands of
  // workgroups would each re-read and normalise the rows
  const void* head_w = c->W(c->has("lm_head") ? "lm_head" : "wte");
  layernorm_fwd<TA>(xa, c->P("lnf_w"), c->P("lnf_b"), (TA*)c->lnf, c->mean, c->rstd, M, C, s);
  const void* hrows = c->lnf;
  if (!decode && T > 1) {
    last_rows<TA>((const TA*)c->lnf, (TA*)c->last, B, T, C, s);
    hrows = c->last;
  }
  GemmArgs g = args(hrows, C, head_w, C, B, c->Vp, C, d_logits, c->Vp);
  if (!product(c, EPI_F32, g, s)) return GPT2_ERR_ARG;
  return hip_ok();
}

}  // namespace

extern "C" {

int gpt2_infer_init(const gpt2_config* cfg, const float* d_params, const void* d_params_bf16, void* d_cache,
                    void* d_workspace, void* hip_stream, gpt2_infer_sizes* sizes, gpt2_infer** out) {
  if (!cfg) return GPT2_ERR_ARG;
  gpt2_sizes ps;
  if (gpt2_init(cfg, nullptr, nullptr, &ps, nullptr) != GPT2_OK) return GPT2_ERR_ARG;
  if (cfg->n_embd / cfg->n_head > 256) return GPT2_ERR_ARG;
  if (cfg->precision == GPT2_FP16) return GPT2_ERR_ARG;  // decoding runs in fp32 or bf16
  gpt2_infer probe;
  probe.cfg = *cfg;
  probe.ops16 = cfg->precision == GPT2_BF16;
  probe.act = probe.ops16 ? 2 : 4;
  probe.L = cfg->n_layer;
  probe.C = cfg->n_embd;
  probe.NH = cfg->n_head;
  probe.V = cfg->vocab_size;
  probe.Vp = cfg->padded_vocab_size;
  probe.Bmax = cfg->max_batch;
  probe.Tmax = cfg->block_size;
  const int64_t cache_bytes = (int64_t)probe.L * probe.Bmax * probe.Tmax * 2 * probe.C * probe.act;
  const int64_t ws = plan(&probe, nullptr);
  if (sizes) {
    sizes->cache_bytes = cache_bytes;
    sizes->workspace_bytes = ws;
  }
  if (!d_cache) return GPT2_OK;
  if (!out || !d_params || !d_workspace || (probe.ops16 && !d_params_bf16)) return GPT2_ERR_ARG;
  gpt2_infer* c = new gpt2_infer(probe);
  c->params = d_params;
  c->pbf16 = (const char*)d_params_bf16;
  c->stream = (hipStream_t)hip_stream;
  c->cache = (char*)d_cache;
  plan(c, (char*)d_workspace);
  for (int i = 0;; ++i) {
    const char* name = nullptr;
    int64_t o = 0, n = 0, dims[3];
    int32_t nd = 0;
    if (gpt2_tensor_info(cfg, i, &name, &o, &n, &nd, dims) != GPT2_OK) break;
    c->off[name] = o;
    // per-block tensors have L as their leading dimension
    const bool block = strncmp(name, "ln1", 3) == 0 || strncmp(name, "ln2", 3) == 0 || strncmp(name, "qkv", 3) == 0 ||
                       strncmp(name, "proj", 4) == 0 || strncmp(name, "fc", 2) == 0;
    c->per[name] = block ? n / c->L : n;
  }
  fill_f32((float*)c->err, 1, 0.f, c->stream);
  const int st = hip_ok();
  if (st != GPT2_OK) {
    delete c;
    return st;
  }
  *out = c;
  return GPT2_OK;
}

int gpt2_infer_prefill(gpt2_infer* c, const int32_t* d_idx, int B, int T, float* d_logits) {
  if (!c || !d_idx || !d_logits) return GPT2_ERR_ARG;
  if (T > c->Tmax) return GPT2_ERR_SEQ_TOO_LONG;
  if (B < 1 || B > c->Bmax || T < 1) return GPT2_ERR_BATCH;
  embed_fwd(d_idx, c->P("wte"), c->P("wpe"), c->x0, c->ids, B * T, T, c->C, c->V, c->err, c->stream);
  c->len = 0;
  const int e = c->ops16 ? forward<h16>(c, B, T, false, d_logits) : forward<float>(c, B, T, false, d_logits);
  if (e != GPT2_OK) {
    c->len = -1;
    return e;
  }
  c->B = B;
  c->len = T;
  return GPT2_OK;
}

int gpt2_infer_decode(gpt2_infer* c, const int32_t* d_tokens, float* d_logits) {
  if (!c || !d_tokens || !d_logits) return GPT2_ERR_ARG;
  if (c->len < 0) return GPT2_ERR_STATE;
  if (c->len >= c->Tmax) return GPT2_ERR_SEQ_TOO_LONG;
  const int B = c->B;
  // one position: wpe row len for every sequence
  embed_fwd(d_tokens, c->P("wte"), c->P("wpe") + (int64_t)c->len * c->C, c->x0, c->ids, B, 1, c->C, c->V, c->err,
            c->stream);
  const int e = c->ops16 ? forward<h16>(c, B, 1, true, d_logits) : forward<float>(c, B, 1, true, d_logits);
  if (e != GPT2_OK) return e;
  c->len += 1;
  return GPT2_OK;
}

int gpt2_infer_length(const gpt2_infer* c) { return c ? c->len : -1; }

int gpt2_sample(const float* d_logits, int64_t ld, int B, int vocab_size, float temperature, int top_k, float top_p,
                const float* d_uniform, int32_t* d_tokens, void* hip_stream) {
  if (!d_logits || !d_uniform || !d_tokens || B < 1 || ld < vocab_size) return GPT2_ERR_ARG;
  if (!sample(d_logits, ld, B, vocab_size, temperature, top_k, top_p, d_uniform, d_tokens, (hipStream_t)hip_stream))
    return GPT2_ERR_ARG;
  return hip_ok();
}

int gpt2_infer_sync_status(gpt2_infer* c) {
  if (!c) return GPT2_ERR_ARG;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
  int flag = 0;
  if (hipMemcpy(&flag, c->err, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return GPT2_ERR_HIP;
  if (flag) {
    fill_f32((float*)c->err, 1, 0.f, c->stream);
    if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
    return GPT2_ERR_TOKEN;
  }
  return hip_ok();
}

void gpt2_infer_destroy(gpt2_infer* c) { delete c; }

}  // extern "C"
