// C ABI of the GPT-2 step: workspace plan, launch sequence of the forward,
// backward, accumulation and clip + AdamW, and the helpers declared in gpt2.h.
#include "gpt2.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"
#include "gpt2_train.h"
#include "kernels.h"

// This file is compiled twice: as the library's C ABI (16-bit operands in
// bfloat16), and with GPT2_OPS_F16 against the kernels built for IEEE half
// (namespace gpt2k_f16), where every entry point takes an f16_ prefix.  The
// ABI entry points hand contexts and configs of the fp16 mode to those.
#ifdef GPT2_OPS_F16
#define GPT2_NAME(name) f16_##name
#define GPT2_API(name) __attribute__((visibility("hidden"))) GPT2_NAME(name)
#define GPT2_TO_F16(cond, call)
#else
#define GPT2_NAME(name) name
#define GPT2_API(name) name
#define GPT2_TO_F16(cond, call) \
  if (cond) return call
extern "C" {
int f16_gpt2_init(const gpt2_config*, const gpt2_buffers*, void*, gpt2_sizes*, gpt2_ctx**);
int f16_gpt2_forward_loss(gpt2_ctx*, const int32_t*, const int32_t*, int, int, float, float*);
int f16_gpt2_backward(gpt2_ctx*);
int f16_gpt2_accumulate(gpt2_ctx*, const int32_t*, const int32_t*, int, int, int, float*);
int f16_gpt2_clip_adamw_step(gpt2_ctx*, float, float, float, float, float, float, float*, int32_t*);
int f16_gpt2_sync_params(gpt2_ctx*);
int f16_gpt2_checkpoint_load(gpt2_ctx*, const char*, int64_t*, int*);
int f16_gpt2_embedding_backward(gpt2_ctx*, const int32_t*, const float*, int, int);
}
#endif

using namespace gpt2k;

namespace {

// micro-batches whose ids gpt2_accumulate sorts in one launch (the sort
// buffers hold this many)
constexpr int kSortBatch = 4;
// parameters gpt2_clip_adamw_step_static takes at most (its AdamW grid of
// n / 1024 workgroups stays within the 32-bit grid dimension)
constexpr int64_t kStaticMaxParams = (int64_t)1 << 40;

enum TensorId {
  T_WTE = 0, T_WPE, T_LN1W, T_LN1B, T_QKVW, T_QKVB, T_PROJW, T_PROJB,
  T_LN2W, T_LN2B, T_FCW, T_FCB, T_FCPW, T_FCPB, T_LNFW, T_LNFB, T_LMHEAD, T_COUNT
};
const char* const kTensorNames[T_COUNT] = {"wte", "wpe", "ln1_w", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b",
                                           "ln2_w", "ln2_b", "fc_w", "fc_b", "fcproj_w", "fcproj_b", "lnf_w",
                                           "lnf_b", "lm_head"};

struct TensorDesc {
  int64_t off, numel, per_layer;  // per_layer: elements of one block's tensor (numel if global)
  int ndim;
  int64_t dims[3];
  bool decay;
  bool present;  // false: the variant has no such tensor (numel 0)
};

bool config_ok(const gpt2_config& c) {
  if (c.n_layer < 1 || c.n_head < 1 || c.n_embd < 8 || c.block_size < 1 || c.vocab_size < 1) return false;
  if (c.n_embd % c.n_head || c.n_embd % 8 || c.n_embd > 2048) return false;
  if (c.padded_vocab_size < c.vocab_size || c.max_batch < 1) return false;
  if (c.precision != GPT2_FP32 && c.precision != GPT2_BF16 && c.precision != GPT2_FP16) return false;
  if (c.variant & ~(GPT2_UNTIED_HEAD | GPT2_NO_QKV_BIAS)) return false;
  if (c.precision != GPT2_FP32 && (c.n_embd / c.n_head != 64 || c.padded_vocab_size % 8)) return false;
  if (c.precision == GPT2_FP32 && c.n_embd / c.n_head > 256) return false;
  if ((int64_t)c.max_batch * c.block_size > (1 << 26)) return false;
  return true;
}

void tensor_table(const gpt2_config& c, TensorDesc t[T_COUNT]) {
  const int64_t C = c.n_embd, L = c.n_layer, Vp = c.padded_vocab_size;
  struct S { int ndim; int64_t d0, d1; bool layer; } sh[T_COUNT] = {
      {2, Vp, C, false},    {2, c.block_size, C, false}, {1, C, 0, true},     {1, C, 0, true},
      {2, 3 * C, C, true},  {1, 3 * C, 0, true},         {2, C, C, true},     {1, C, 0, true},
      {1, C, 0, true},      {1, C, 0, true},             {2, 4 * C, C, true}, {1, 4 * C, 0, true},
      {2, C, 4 * C, true},  {1, C, 0, true},             {1, C, 0, false},    {1, C, 0, false},
      {2, Vp, C, false}};
  int64_t off = 0;
  for (int i = 0; i < T_COUNT; ++i) {
    const int64_t per = sh[i].ndim == 2 ? sh[i].d0 * sh[i].d1 : sh[i].d0;
    TensorDesc& d = t[i];
    d.present = !((i == T_QKVB && (c.variant & GPT2_NO_QKV_BIAS)) || (i == T_LMHEAD && !(c.variant & GPT2_UNTIED_HEAD)));
    d.off = off;
    d.per_layer = d.present ? per : 0;
    d.numel = d.present ? (sh[i].layer ? per * L : per) : 0;
    d.decay = sh[i].ndim >= 2;  // weight decay on tensors of two or more dimensions
    if (sh[i].layer) {
      d.ndim = sh[i].ndim + 1;
      d.dims[0] = L;
      d.dims[1] = sh[i].d0;
      d.dims[2] = sh[i].d1;
    } else {
      d.ndim = sh[i].ndim;
      d.dims[0] = sh[i].d0;
      d.dims[1] = sh[i].d1;
      d.dims[2] = 0;
    }
    off += d.numel;
  }
}

int64_t total_params(const TensorDesc t[T_COUNT]) { return t[T_COUNT - 1].off + t[T_COUNT - 1].numel; }

// Workspace plan: a list of 256-byte aligned regions.
struct Plan {
  int64_t bytes = 0;
  int64_t take(int64_t n) {
    const int64_t o = bytes;
    bytes += (n + 255) / 256 * 256;
    return o;
  }
};

}  // namespace

struct gpt2_ctx {
  gpt2_config cfg;
  gpt2_buffers buf;
  hipStream_t stream;
  TensorDesc t[T_COUNT];
  int64_t n_params;
  bool ops16;  // 16-bit MFMA operands (bf16, or fp16 in the fp16 build)
  bool f16;    // fp16 mode: this context runs on the f16_ build
  int64_t act;  // bytes per activation element
  int64_t Mmax;
  int L, C, NH, Vp, V;
  int id_bits;
  int head;        // tensor of the lm_head weight: T_WTE (tied) or T_LMHEAD
  bool qkv_bias;   // the QKV projection has a bias

  // workspace regions
  float* res;
  char* ln1;
  float *ln1_mean, *ln1_rstd;
  char* qkv;
  char* atty;
  float* lse;
  char* ln2;
  float *ln2_mean, *ln2_rstd;
  char* fcgd;  // gelu'(u) of the MLP pre-activation u, the only use of u in the backward
  char* fcg;
  char* lnf;
  float *lnf_mean, *lnf_rstd;
  char* logits;
  float* row_loss;
  int32_t* ids;
  float* dres;
  char* dres_act;
  float* dh;
  char* dbig;
  char* dqkv;
  char* dy;
  float* attnD;
  // gpt2_accumulate sorts the ids of up to kSortBatch micro-batches in one
  // launch; presorted >= 0: the backward's sorted ids are slice presorted
  int presorted = -1;
  float* splitk;
  int64_t splitk_elems;
  float* colpart;
  int32_t *sort_ka, *sort_va, *sort_kb, *sort_vb;
  float* run_sums;
  double* norm_part;
  float* clip_scale;
  int* err_flag;
  int32_t* amp_found;  // fp16 mode: 1 when the last step found a non-finite gradient

  // Dynamic loss scaling (fp16 mode): the loss gradient is formed times
  // amp_scale, so the gradients accumulate scaled; the clip + AdamW step
  // unscales them, and skips the update (parameters, moments and step count
  // unchanged) when one is not finite.  Then the scale is multiplied by
  // amp_backoff after a skipped step and by amp_growth after amp_interval
  // consecutive good ones.
  bool amp = false;
  float amp_scale = 65536.f, amp_growth = 2.f, amp_backoff = 0.5f;
  int amp_interval = 2000, amp_good = 0, amp_skipped = 0;

  // state
  bool have_fwd = false;
  int B = 0, T = 0;
  int64_t step = 0;

  // timing
  std::string site;
  bool timing = false;
  std::vector<hipEvent_t> ev;
  std::vector<double> ev_flops, ev_bytes;
  std::vector<const char*> ev_site;  // launch-site name of each bracketed launch
  std::vector<int> ev_cfg;           // its GEMM tile configuration (-1: not a GEMM)
  size_t ev_used = 0;
  bool ev_overflow = false;

  // helpers
  int64_t MC() const { return Mmax * C; }
  char* layer_act(char* base, int l, int64_t cols) const { return base + (int64_t)l * Mmax * cols * act; }
  const void* W(int id, int l = 0) const {
    const int64_t o = t[id].off + (int64_t)l * t[id].per_layer;
    return ops16 ? (const void*)((const char*)buf.params_bf16 + o * 2) : (const void*)(buf.params + o);
  }
  const float* P(int id, int l = 0) const { return buf.params + t[id].off + (int64_t)l * t[id].per_layer; }
  float* G(int id, int l = 0) const { return buf.grads + t[id].off + (int64_t)l * t[id].per_layer; }
  float* resid(int i) const { return res + (int64_t)i * MC(); }
};

namespace {

// True when `prefix` is `site` or a leading run of its dot-separated parts
// ("gemm.fwd" matches "gemm.fwd.fc"; "gemm.fwd.fc" does not match "gemm.fwd.fcproj").
bool site_matches(const char* site, const std::string& prefix) {
  if (strncmp(site, prefix.c_str(), prefix.size()) != 0) return false;
  const char next = site[prefix.size()];
  return next == '\0' || next == '.' || prefix.empty();
}

// GEMM tile configuration recorded for the grouped weight-gradient launch
constexpr int kCfgGrouped = -2;

// Brackets one launch with HIP events when its site matches the enabled prefix.
// site must be a string literal (its address is kept).
struct Timed {
  gpt2_ctx* c;
  bool on = false;
  size_t slot = 0;
  Timed(gpt2_ctx* ctx, const char* site, double flops, double bytes, int cfg = -1) : c(ctx) {
    if (!c->timing || !site_matches(site, c->site)) return;
    if (c->ev_used * 2 + 2 > c->ev.size()) {
      if (c->ev.size() >= 2 * 8192) {
        c->ev_overflow = true;
        return;
      }
      for (int i = 0; i < 256; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        c->ev.push_back(e);
      }
    }
    slot = c->ev_used++;
    c->ev_flops.resize(c->ev_used);
    c->ev_bytes.resize(c->ev_used);
    c->ev_site.resize(c->ev_used);
    c->ev_cfg.resize(c->ev_used);
    c->ev_flops[slot] = flops;
    c->ev_bytes[slot] = bytes;
    c->ev_site[slot] = site;
    c->ev_cfg[slot] = cfg;
    (void)hipEventRecord(c->ev[2 * slot], c->stream);
    on = true;
  }
  ~Timed() {
    if (on) (void)hipEventRecord(c->ev[2 * slot + 1], c->stream);
  }
};

bool gemm_site(gpt2_ctx* c, const char* site, GemmLayout lay, GemmEpilogue epi, const GemmArgs& a, double bytes) {
  Timed tm(c, site, 2.0 * a.M * (double)a.N * a.K, bytes,
           c->timing ? gemm_resolve_config(-1, lay, epi, c->ops16, a) : -1);
  return gemm(lay, epi, c->ops16, a, c->stream);
}

GemmArgs gargs(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K, void* C, int64_t ldc) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = A;
  a.B = B;
  a.lda = lda;
  a.ldb = ldb;
  a.M = M;
  a.N = N;
  a.K = K;
  a.C = C;
  a.ldc = ldc;
  a.splits = 1;
  a.k_per_split = K;
  return a;
}

// Weight gradient: out[Mo][N] += A^T B with A stored [K][Mo], B stored [K][N].
// The token dimension K is split when the output has too few tiles to fill
// the chip; the splits write fp32 partials that a second kernel adds in split
// order (deterministic).  Tile configuration and split count minimise the
// modelled GEMM time plus the partials' HBM traffic.
bool weight_grad(gpt2_ctx* c, const char* site, float* out, const void* A, int64_t lda, const void* B, int64_t ldb,
                 int Mo, int N, int K) {
  const int64_t outn = (int64_t)Mo * N;
  GemmArgs a = gargs(A, lda, B, ldb, Mo, N, K, out, N);
  int best_cfg = -1, best_splits = 1, best_kps = K;
  if (c->ops16) {
    double best = 1e30;
    for (int cfg = 0; cfg < kGemmConfigs; ++cfg) {
      for (int sp = 1; sp <= 16; sp *= 2) {
        int kps = (K + sp - 1) / sp;
        kps = (kps + 63) / 64 * 64;
        const int splits = (K + kps - 1) / kps;
        if (splits > 1 && (int64_t)splits * outn > c->splitk_elems) continue;
        GemmArgs t = a;
        t.splits = splits;
        t.k_per_split = splits > 1 ? kps : K;
        if (!gemm_config_usable(cfg, LAYOUT_TN, t)) continue;
        double time = gemm_model_time(cfg, t, true);
        if (splits > 1) time += (2.0 * splits + 2.0) * outn * 4.0 / 4.0e12;
        if (time < best) {
          best = time;
          best_cfg = cfg;
          best_splits = splits;
          best_kps = t.k_per_split;
        }
      }
    }
  } else {
    const int64_t tiles = (int64_t)((Mo + 63) / 64) * ((N + 63) / 64);
    int sp = (int)std::min<int64_t>(16, std::max<int64_t>(1, (512 + tiles - 1) / tiles));
    int kps = ((K + sp - 1) / sp + 63) / 64 * 64;
    sp = (K + kps - 1) / kps;
    if (sp > 1 && sp * outn > c->splitk_elems) sp = 1;
    best_splits = sp;
    best_kps = sp > 1 ? kps : K;
  }
  const double bytes = (double)c->act * ((double)K * Mo + (double)K * N) + 8.0 * outn;
  if (!c->ops16) best_cfg = kGemmCfgF32;
  if (best_splits == 1) {
    Timed tm(c, site, 2.0 * a.M * (double)a.N * a.K, bytes, best_cfg);
    return gemm_cfg(best_cfg, LAYOUT_TN, EPI_F32_ACC, c->ops16, a, c->stream);
  }
  a.C = c->splitk;
  a.splits = best_splits;
  a.k_per_split = best_kps;
  a.split_stride = outn;
  {
    Timed tm(c, site, 2.0 * a.M * (double)a.N * a.K, bytes, best_cfg);
    if (!gemm_cfg(best_cfg, LAYOUT_TN, EPI_PARTIAL, c->ops16, a, c->stream)) return false;
  }
  splitk_reduce_add(out, c->splitk, best_splits, outn, outn, c->stream);
  return true;
}

int hip_status() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    fprintf(stderr, "gpt2: HIP error: %s\n", hipGetErrorString(e));
    return GPT2_ERR_HIP;
  }
  return GPT2_OK;
}

template <typename TA>
int forward_impl(gpt2_ctx* c, const int32_t* d_idx, const int32_t* d_tgt, int B, int T, float loss_scale,
                 float* d_loss, bool accumulate) {
  hipStream_t s = c->stream;
  const int M = B * T, C = c->C, L = c->L, Vp = c->Vp;
  const double a = (double)c->act;
  embed_fwd(d_idx, c->P(T_WTE), c->P(T_WPE), c->resid(0), c->ids, M, T, C, c->V, c->err_flag, s);
  for (int l = 0; l < L; ++l) {
    float* x_in = c->resid(2 * l);
    float* x_mid = c->resid(2 * l + 1);
    float* x_out = c->resid(2 * l + 2);
    TA* ln1 = (TA*)c->layer_act(c->ln1, l, C);
    TA* qkv = (TA*)c->layer_act(c->qkv, l, 3 * C);
    TA* atty = (TA*)c->layer_act(c->atty, l, C);
    TA* ln2 = (TA*)c->layer_act(c->ln2, l, C);
    TA* fcgd = (TA*)c->layer_act(c->fcgd, l, 4 * C);
    TA* fcg = (TA*)c->layer_act(c->fcg, l, 4 * C);
    float* lse = c->lse + (int64_t)l * c->Mmax * c->NH;
    {
      Timed tm(c, "ln.fwd", 0, (double)M * C * (4 + a) + 8.0 * M);
      layernorm_fwd<TA>(x_in, c->P(T_LN1W, l), c->P(T_LN1B, l), ln1, c->ln1_mean + (int64_t)l * c->Mmax,
                        c->ln1_rstd + (int64_t)l * c->Mmax, M, C, s);
    }
    GemmArgs g = gargs(ln1, C, c->W(T_QKVW, l), C, M, 3 * C, C, qkv, 3 * C);
    g.bias = c->qkv_bias ? c->P(T_QKVB, l) : nullptr;
    if (!gemm_site(c, "gemm.fwd.qkv", LAYOUT_NT, EPI_ACT, g, a * ((double)M * C + 3.0 * C * C + 3.0 * M * C)))
      return GPT2_ERR_ARG;
    {
      Timed tm(c, "attn.fwd", 4.0 * B * c->NH * ((double)T * (T + 1) / 2) * (C / c->NH),
               a * (4.0 * M * C) + 4.0 * M * c->NH);
      if (c->ops16) attn_fwd_bf16(qkv, atty, lse, B, T, c->NH, C, s);
      else attn_fwd_f32((const float*)qkv, (float*)atty, lse, B, T, c->NH, C, s);
    }
    g = gargs(atty, C, c->W(T_PROJW, l), C, M, C, C, x_mid, C);
    g.bias = c->P(T_PROJB, l);
    g.resid = x_in;
    if (!gemm_site(c, "gemm.fwd.proj", LAYOUT_NT, EPI_RESID, g, a * ((double)M * C + (double)C * C) + 8.0 * M * C))
      return GPT2_ERR_ARG;
    {
      Timed tm(c, "ln.fwd", 0, (double)M * C * (4 + a) + 8.0 * M);
      layernorm_fwd<TA>(x_mid, c->P(T_LN2W, l), c->P(T_LN2B, l), ln2, c->ln2_mean + (int64_t)l * c->Mmax,
                        c->ln2_rstd + (int64_t)l * c->Mmax, M, C, s);
    }
    g = gargs(ln2, C, c->W(T_FCW, l), C, M, 4 * C, C, fcgd, 4 * C);
    g.bias = c->P(T_FCB, l);
    g.C2 = fcg;
    if (!gemm_site(c, "gemm.fwd.fc", LAYOUT_NT, EPI_GELU, g, a * ((double)M * C + 4.0 * C * C + 8.0 * M * C)))
      return GPT2_ERR_ARG;
    g = gargs(fcg, 4 * C, c->W(T_FCPW, l), 4 * C, M, C, 4 * C, x_out, C);
    g.bias = c->P(T_FCPB, l);
    g.resid = x_mid;
    if (!gemm_site(c, "gemm.fwd.fcproj", LAYOUT_NT, EPI_RESID, g,
                   a * (4.0 * M * C + 4.0 * C * C) + 8.0 * M * C))
      return GPT2_ERR_ARG;
  }
  {
    Timed tm(c, "ln.fwd", 0, (double)M * C * (4 + a) + 8.0 * M);
    layernorm_fwd<TA>(c->resid(2 * L), c->P(T_LNFW), c->P(T_LNFB), (TA*)c->lnf, c->lnf_mean, c->lnf_rstd, M, C, s);
  }
  GemmArgs g = gargs(c->lnf, C, c->W(c->head), C, M, Vp, C, c->logits, Vp);
  if (!gemm_site(c, "gemm.fwd.lmhead", LAYOUT_NT, EPI_LOGITS, g, a * ((double)M * C + (double)Vp * C + (double)M * Vp)))
    return GPT2_ERR_ARG;
  {
    Timed tm(c, "xent", 0, 2.0 * a * M * Vp + 8.0 * M);
    const float seed = c->amp ? loss_scale * c->amp_scale : loss_scale;  // gradient of the (scaled) loss
    xent_fwd_bwd<TA>((TA*)c->logits, d_tgt, c->row_loss, M, Vp, c->V, seed / (float)M, c->err_flag, s);
  }
  loss_reduce(c->row_loss, M, loss_scale / (float)M, accumulate, d_loss, s);
  c->have_fwd = true;
  c->B = B;
  c->T = T;
  return hip_status();
}

template <typename TA>
int backward_impl(gpt2_ctx* c) {
  hipStream_t s = c->stream;
  const int B = c->B, T = c->T, M = B * T, C = c->C, L = c->L, Vp = c->Vp;
  const double a = (double)c->act;
  // Column partials (LayerNorm gain / shift and bias gradients): every
  // producer writes its own region; one batched launch at the end of the
  // pass reduces them all (each output has exactly one job).
  float* part = c->colpart;
  std::vector<ColJob> jobs;
  jobs.reserve(4 * L + 1);
  // arrays: partial arrays the producer wrote (3 for LayerNorm, 1 for a sum)
  auto defer = [&](float* o0, float* o1, float* o2, int chunks, int n, int arrays) {
    const int nout = o2 ? 3 : (o1 ? 2 : 1);
    jobs.push_back(ColJob{{o0, o1, o2}, part, chunks, n, nout});
    part += (int64_t)arrays * chunks * n;
  };
  // Weight gradients: in bf16 mode with whole 64-token k-tiles they are
  // collected and run as one grouped launch at the end of the pass (enough
  // output tiles to fill the GPU without split-K); otherwise each runs here.
  const bool group_dw = c->ops16 && M % 64 == 0;
  std::vector<GemmProblem> dw;
  auto wgrad = [&](const char* site, float* out, const void* A, int64_t lda, const void* Bop, int64_t ldb, int Mo,
                   int N) -> bool {
    if (group_dw) {
      const GemmProblem pr{A, Bop, out, Mo, N, M, (int)lda, (int)ldb};
      if (gemm_group_ok(pr)) {
        dw.push_back(pr);
        return true;
      }
    }
    return weight_grad(c, site, out, A, lda, Bop, ldb, Mo, N, M);
  };
  // residual-gradient slots (bf16 copy): 2L + 1 is the lm_head side, 2l + 1
  // the gradient at x_mid of block l, 2l the gradient at x_in of block l
  const bool per_layer = c->ops16;
  auto dres_slot = [&](int i) -> TA* {
    return (TA*)(c->dres_act + (per_layer ? (int64_t)i * c->Mmax * C * c->act : 0));
  };
  // lm_head (tied): dlnf = dz wte; dwte += dz^T lnf
  // dh: gradient at a LayerNorm output, in the activation type (bf16 in bf16
  // mode, like every other matmul output of the mixed-precision step)
  TA* dh = (TA*)c->dh;
  GemmArgs g = gargs(c->logits, Vp, c->W(c->head), C, M, C, Vp, dh, C);
  if (!gemm_site(c, "gemm.bwd.lmhead.dx", LAYOUT_NN, EPI_ACT, g, a * ((double)M * Vp + (double)Vp * C + (double)M * C)))
    return GPT2_ERR_ARG;
  if (!wgrad("gemm.bwd.lmhead.dw", c->G(c->head), c->logits, Vp, c->lnf, C, Vp, C)) return GPT2_ERR_ARG;
  int ch;
  {
    Timed tm(c, "ln.bwd", 0, (double)M * C * (8 + 2 * a) + 8.0 * M);
    ch = layernorm_bwd<TA>(dh, c->resid(2 * L), c->lnf_mean, c->lnf_rstd, c->P(T_LNFW), c->dres, false,
                           dres_slot(2 * L), part, M, C, s);
  }
  defer(c->G(T_LNFW), c->G(T_LNFB), c->G(T_FCPB, L - 1), ch, C, 3);

  for (int l = L - 1; l >= 0; --l) {
    TA* ln1 = (TA*)c->layer_act(c->ln1, l, C);
    TA* qkv = (TA*)c->layer_act(c->qkv, l, 3 * C);
    TA* atty = (TA*)c->layer_act(c->atty, l, C);
    TA* ln2 = (TA*)c->layer_act(c->ln2, l, C);
    TA* fcgd = (TA*)c->layer_act(c->fcgd, l, 4 * C);
    TA* fcg = (TA*)c->layer_act(c->fcg, l, 4 * C);
    float* lse = c->lse + (int64_t)l * c->Mmax * c->NH;
    TA* dres_out = dres_slot(2 * l + 2);  // gradient at x_out of this block
    TA* dres_mid = dres_slot(2 * l + 1);
    TA* dbig = (TA*)(per_layer ? c->layer_act(c->dbig, l, 4 * C) : c->dbig);
    TA* dqkv = (TA*)(per_layer ? c->layer_act(c->dqkv, l, 3 * C) : c->dqkv);
    TA* dy = (TA*)c->dy;

    // MLP output projection: x_out = x_mid + g Wfp^T + bfp
    if (!wgrad("gemm.bwd.fcproj.dw", c->G(T_FCPW, l), dres_out, C, fcg, 4 * C, C, 4 * C)) return GPT2_ERR_ARG;
    g = gargs(dres_out, C, c->W(T_FCPW, l), 4 * C, M, 4 * C, C, dbig, 4 * C);
    g.aux = fcgd;
    g.colsum = part;  // fc bias gradient partials, 64 rows per chunk
    if (!gemm_site(c, "gemm.bwd.fcproj.dx", LAYOUT_NN, EPI_GELU_BWD, g, a * ((double)M * C + 4.0 * C * C + 8.0 * M * C)))
      return GPT2_ERR_ARG;
    ch = (M + 63) / 64;
    defer(c->G(T_FCB, l), nullptr, nullptr, ch, 4 * C, 1);
    // MLP input projection: u = LN2(x_mid) Wfc^T + bfc
    if (!wgrad("gemm.bwd.fc.dw", c->G(T_FCW, l), dbig, 4 * C, ln2, C, 4 * C, C)) return GPT2_ERR_ARG;
    g = gargs(dbig, 4 * C, c->W(T_FCW, l), C, M, C, 4 * C, dh, C);
    if (!gemm_site(c, "gemm.bwd.fc.dx", LAYOUT_NN, EPI_ACT, g, a * (4.0 * M * C + 4.0 * C * C + (double)M * C)))
      return GPT2_ERR_ARG;
    {
      Timed tm(c, "ln.bwd", 0, (double)M * C * (12 + 2 * a) + 8.0 * M);
      ch = layernorm_bwd<TA>(dh, c->resid(2 * l + 1), c->ln2_mean + (int64_t)l * c->Mmax,
                             c->ln2_rstd + (int64_t)l * c->Mmax, c->P(T_LN2W, l), c->dres, true, dres_mid, part, M,
                             C, s);
    }
    defer(c->G(T_LN2W, l), c->G(T_LN2B, l), c->G(T_PROJB, l), ch, C, 3);
    // attention output projection: x_mid = x_in + y Wp^T + bp
    if (!wgrad("gemm.bwd.proj.dw", c->G(T_PROJW, l), dres_mid, C, atty, C, C, C)) return GPT2_ERR_ARG;
    g = gargs(dres_mid, C, c->W(T_PROJW, l), C, M, C, C, dy, C);
    if (!gemm_site(c, "gemm.bwd.proj.dx", LAYOUT_NN, EPI_ACT, g, a * (2.0 * M * C + (double)C * C)))
      return GPT2_ERR_ARG;
    bool fused = false;
    {
      Timed tm(c, "attn.bwd", 10.0 * B * c->NH * ((double)T * (T + 1) / 2) * (C / c->NH),
               a * (9.0 * M * C) + 8.0 * M * c->NH);
      // the qkv bias gradient partials come from the attention kernels when
      // they can form them (64-token chunks within a sequence)
      if (c->ops16)
        fused = attn_bwd_bf16(qkv, atty, dy, lse, c->attnD, dqkv, B, T, c->NH, C, c->qkv_bias ? part : nullptr, s);
      else attn_bwd_f32((const float*)qkv, (const float*)atty, (const float*)dy, lse, c->attnD, (float*)dqkv, B, T,
                        c->NH, C, s);
    }
    if (c->qkv_bias) {
      ch = fused ? M / 64 : colsum_partials<TA>(dqkv, M, 3 * C, part, s);
      defer(c->G(T_QKVB, l), nullptr, nullptr, ch, 3 * C, 1);
    }
    // QKV projection: qkv = LN1(x_in) Wqkv^T + bqkv
    if (!wgrad("gemm.bwd.qkv.dw", c->G(T_QKVW, l), dqkv, 3 * C, ln1, C, 3 * C, C)) return GPT2_ERR_ARG;
    g = gargs(dqkv, 3 * C, c->W(T_QKVW, l), C, M, C, 3 * C, dh, C);
    if (!gemm_site(c, "gemm.bwd.qkv.dx", LAYOUT_NN, EPI_ACT, g, a * (3.0 * M * C + 3.0 * C * C + (double)M * C)))
      return GPT2_ERR_ARG;
    {
      Timed tm(c, "ln.bwd", 0, (double)M * C * (12 + 2 * a) + 8.0 * M);
      ch = layernorm_bwd<TA>(dh, c->resid(2 * l), c->ln1_mean + (int64_t)l * c->Mmax,
                             c->ln1_rstd + (int64_t)l * c->Mmax, c->P(T_LN1W, l), c->dres, true, dres_slot(2 * l), part, M,
                             C, s);
    }
    // the shift's third output is the previous block's MLP output bias
    if (l > 0) defer(c->G(T_LN1W, l), c->G(T_LN1B, l), c->G(T_FCPB, l - 1), ch, C, 3);
    else defer(c->G(T_LN1W, l), c->G(T_LN1B, l), nullptr, ch, C, 3);
  }
  colpart_reduce_batch(jobs.data(), (int)jobs.size(), s);
  if (!dw.empty()) {
    double fl = 0.0, by = 0.0;
    for (const GemmProblem& pr : dw) {
      fl += 2.0 * pr.M * (double)pr.N * pr.K;
      by += a * ((double)pr.K * pr.M + (double)pr.K * pr.N) + 8.0 * pr.M * (double)pr.N;
    }
    Timed tm(c, "gemm.bwd.dw", fl, by, kCfgGrouped);
    gemm_group_tn_acc(dw.data(), (int)dw.size(), c->splitk, c->splitk_elems, s);  // split-K scratch is free here
  }
  // embedding: x0 = wte[idx] + wpe[t]
  {
    Timed tm(c, "embed.bwd", 0, 12.0 * M * C);
    embed_wpe_grad(c->dres, c->G(T_WPE), B, T, C, s);
    int32_t* keys = c->sort_ka;
    int32_t* vals = c->sort_va;
    if (c->presorted >= 0) {
      keys += (int64_t)c->presorted * M;
      vals += (int64_t)c->presorted * M;
    } else {
      embed_sort(c->ids, M, c->Vp, c->id_bits, c->sort_ka, c->sort_va, c->sort_kb, c->sort_vb, s);
    }
    embed_scatter(keys, vals, c->dres, c->run_sums, c->G(T_WTE), M, C, s);
  }
  c->have_fwd = false;
  return hip_status();
}

int check_bt(const gpt2_ctx* c, int B, int T) {
  if (T > c->cfg.block_size) return GPT2_ERR_SEQ_TOO_LONG;
  if (B < 1 || T < 1 || B > c->cfg.max_batch) return GPT2_ERR_BATCH;
  // bf16 weight gradients contract over the B*T tokens in 16-byte rows
  if (c->ops16 && ((int64_t)B * T) % 8) return GPT2_ERR_BATCH;
  return GPT2_OK;
}

int64_t plan_workspace(gpt2_ctx* c, Plan& p, bool assign) {
  const int64_t M = c->Mmax, C = c->C, L = c->L, A = c->act, Vp = c->Vp, NH = c->NH;
  char* base = (char*)c->buf.workspace;
  auto at = [&](int64_t bytes) -> char* {
    const int64_t o = p.take(bytes);
    return assign ? base + o : nullptr;
  };
  c->res = (float*)at((2 * L + 1) * M * C * 4);
  c->ln1 = at(L * M * C * A);
  c->ln1_mean = (float*)at(L * M * 4);
  c->ln1_rstd = (float*)at(L * M * 4);
  c->qkv = at(L * M * 3 * C * A);
  c->atty = at(L * M * C * A);
  c->lse = (float*)at(L * M * NH * 4);
  c->ln2 = at(L * M * C * A);
  c->ln2_mean = (float*)at(L * M * 4);
  c->ln2_rstd = (float*)at(L * M * 4);
  c->fcgd = at(L * M * 4 * C * A);
  c->fcg = at(L * M * 4 * C * A);
  c->lnf = at(M * C * A);
  c->lnf_mean = (float*)at(M * 4);
  c->lnf_rstd = (float*)at(M * 4);
  c->logits = at(M * Vp * A);
  c->row_loss = (float*)at(M * 4);
  c->ids = (int32_t*)at(M * 4);
  c->dres = (float*)at(M * C * 4);
  // bf16: the gradients the weight-gradient GEMMs read stay until the end of
  // the backward pass (one grouped launch there): 2L + 1 residual-gradient
  // slots, L slots of du and of dqkv.  fp32: one of each.
  const int64_t slots = c->ops16 ? L : 1;
  c->dres_act = at((2 * slots + 1) * M * C * A);
  c->dh = (float*)at(M * C * 4);
  c->dbig = at(slots * M * 4 * C * A);
  c->dqkv = at(slots * M * 3 * C * A);
  c->dy = at(M * C * A);
  c->attnD = (float*)at(2 * M * NH * 4);  // D, then the exp2-domain log-sum-exp (bf16 backward)
  c->splitk_elems = std::max<int64_t>(16 * 4 * C * C, 2 * Vp * C);
  c->splitk = (float*)at(c->splitk_elems * 4);
  // one region per column-partial producer of a backward pass: 2L + 1
  // LayerNorm backwards (3 x M/32 rows of C) and the qkv and fc bias sums
  // (M/64 rows of 3C and 4C)
  const int64_t col_elems = (2 * L + 1) * 3 * ((M + 31) / 32) * C + L * ((M + 63) / 64) * 7 * C;
  c->colpart = (float*)at(col_elems * 4);
  c->sort_ka = (int32_t*)at(kSortBatch * M * 4);
  c->sort_va = (int32_t*)at(kSortBatch * M * 4);
  c->sort_kb = (int32_t*)at(M * 4);
  c->sort_vb = (int32_t*)at(M * 4);
  c->run_sums = (float*)at(M * C * 4);
  c->norm_part = (double*)at(1024 * 8);
  c->clip_scale = (float*)at(256);
  c->err_flag = (int*)at(256);
  c->amp_found = (int32_t*)at(256);
  return p.bytes;
}

void fill_layout(gpt2_ctx* c, const gpt2_config& cfg) {
  c->cfg = cfg;
  tensor_table(cfg, c->t);
  c->n_params = total_params(c->t);
  c->ops16 = cfg.precision != GPT2_FP32;
  c->f16 = cfg.precision == GPT2_FP16;
  c->amp = c->f16;
  c->act = c->ops16 ? 2 : 4;
  c->Mmax = (int64_t)cfg.max_batch * cfg.block_size;
  c->L = cfg.n_layer;
  c->C = cfg.n_embd;
  c->NH = cfg.n_head;
  c->Vp = cfg.padded_vocab_size;
  c->V = cfg.vocab_size;
  int bits = 1;
  while ((1 << bits) < cfg.padded_vocab_size) ++bits;
  c->id_bits = bits;
  c->head = (cfg.variant & GPT2_UNTIED_HEAD) ? T_LMHEAD : T_WTE;
  c->qkv_bias = !(cfg.variant & GPT2_NO_QKV_BIAS);
}

}  // namespace

extern "C" {

int GPT2_API(gpt2_init)(const gpt2_config* cfg, const gpt2_buffers* bufs, void* hip_stream, gpt2_sizes* sizes,
                        gpt2_ctx** out) {
  if (!cfg || !config_ok(*cfg)) return GPT2_ERR_ARG;
  GPT2_TO_F16(cfg->precision == GPT2_FP16, f16_gpt2_init(cfg, bufs, hip_stream, sizes, out));
  gpt2_ctx probe;
  fill_layout(&probe, *cfg);
  Plan plan;
  const int64_t ws = plan_workspace(&probe, plan, false);
  if (sizes) {
    sizes->n_params = probe.n_params;
    sizes->workspace_bytes = ws;
    sizes->params_bf16_bytes = probe.ops16 ? probe.n_params * 2 : 0;
  }
  if (!bufs) return GPT2_OK;
  if (!out || !bufs->params || !bufs->grads || !bufs->adam_m || !bufs->adam_v || !bufs->workspace)
    return GPT2_ERR_ARG;
  if (probe.ops16 && !bufs->params_bf16) return GPT2_ERR_ARG;
  if (((uintptr_t)bufs->workspace) % 256) return GPT2_ERR_ARG;
  gpt2_ctx* c = new gpt2_ctx();
  fill_layout(c, *cfg);
  c->buf = *bufs;
  if (!c->ops16) c->buf.params_bf16 = nullptr;
  c->stream = (hipStream_t)hip_stream;
  Plan p2;
  plan_workspace(c, p2, true);
  fill_f32(c->buf.grads, c->n_params, 0.f, c->stream);
  fill_f32(c->buf.adam_m, c->n_params, 0.f, c->stream);
  fill_f32(c->buf.adam_v, c->n_params, 0.f, c->stream);
  fill_f32((float*)c->err_flag, 1, 0.f, c->stream);
  if (c->ops16) to_bf16(c->buf.params, c->buf.params_bf16, c->n_params, c->stream);
  const int st = hip_status();
  if (st != GPT2_OK) {
    delete c;
    return st;
  }
  *out = c;
  return GPT2_OK;
}

int GPT2_API(gpt2_forward_loss)(gpt2_ctx* c, const int32_t* d_idx, const int32_t* d_targets, int B, int T,
                                float loss_scale, float* d_loss) {
  if (!c || !d_idx || !d_targets || !d_loss) return GPT2_ERR_ARG;
  GPT2_TO_F16(c->f16, f16_gpt2_forward_loss(c, d_idx, d_targets, B, T, loss_scale, d_loss));
  const int e = check_bt(c, B, T);
  if (e != GPT2_OK) return e;
  return c->ops16 ? forward_impl<h16>(c, d_idx, d_targets, B, T, loss_scale, d_loss, false)
                 : forward_impl<float>(c, d_idx, d_targets, B, T, loss_scale, d_loss, false);
}

int GPT2_API(gpt2_backward)(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  GPT2_TO_F16(c->f16, f16_gpt2_backward(c));
  if (!c->have_fwd) return GPT2_ERR_STATE;
  return c->ops16 ? backward_impl<h16>(c) : backward_impl<float>(c);
}

int GPT2_API(gpt2_accumulate)(gpt2_ctx* c, const int32_t* d_idx, const int32_t* d_targets, int k, int B, int T,
                              float* d_mean_loss) {
  if (!c || !d_idx || !d_targets || !d_mean_loss) return GPT2_ERR_ARG;
  GPT2_TO_F16(c->f16, f16_gpt2_accumulate(c, d_idx, d_targets, k, B, T, d_mean_loss));
  if (k < 1) return GPT2_ERR_BATCH;
  int e = check_bt(c, B, T);
  if (e != GPT2_OK) return e;
  fill_f32(c->buf.grads, c->n_params, 0.f, c->stream);
  const int64_t stride = (int64_t)B * T;
  bool batched = false;
  for (int i = 0; i < k; ++i) {
    // the embedding gradient's sort of the ids, for kSortBatch micro-batches
    // at a time (one workgroup each, side by side, instead of one per backward)
    if (i % kSortBatch == 0) {
      Timed tm(c, "embed.bwd", 0, 8.0 * stride * std::min(kSortBatch, k - i));
      batched = embed_sort_batch(d_idx + i * stride, (int)stride, std::min(kSortBatch, k - i), c->V, c->sort_ka,
                                 c->sort_va, c->stream);
    }
    e = c->ops16 ? forward_impl<h16>(c, d_idx + i * stride, d_targets + i * stride, B, T, 1.0f / k, d_mean_loss,
                                     i > 0)
                : forward_impl<float>(c, d_idx + i * stride, d_targets + i * stride, B, T, 1.0f / k, d_mean_loss,
                                      i > 0);
    if (e != GPT2_OK) return e;
    c->presorted = batched ? i % kSortBatch : -1;
    e = GPT2_NAME(gpt2_backward)(c);
    c->presorted = -1;
    if (e != GPT2_OK) return e;
  }
  return GPT2_OK;
}

namespace {

static DecaySegments decay_segments(const TensorDesc t[T_COUNT], int64_t n_params) {
  DecaySegments seg;
  memset(&seg, 0, sizeof(seg));
  for (int i = 0; i < T_COUNT; ++i) {
    if (!t[i].present) continue;
    if (seg.n == 0 || seg.decay[seg.n - 1] != (int)t[i].decay) {
      seg.start[seg.n] = t[i].off;
      seg.decay[seg.n] = t[i].decay;
      ++seg.n;
    }
  }
  seg.start[seg.n] = n_params;
  return seg;
}

// Norm, clip decision and AdamW at step t on the flat vectors of bufs, with
// the norm partials and the clip factor in (norm_part, clip_scale).
static void clip_adamw_launch(gpt2_ctx* c, const gpt2_buffers& b, int64_t n_params, const DecaySegments& seg,
                              int64_t t, double* norm_part, float* clip_scale, float lr, float beta1, float beta2,
                              float eps, float weight_decay, float max_norm, float* d_norm, int32_t* d_clipped,
                              hipStream_t s) {
  {
    Timed tm(c, "norm", 0, 4.0 * n_params);
    const int nblk = sumsq_partials(b.grads, n_params, norm_part, s);
    clip_finalize(norm_part, nblk, max_norm, d_norm, d_clipped, clip_scale, c->amp ? 1.0f / c->amp_scale : 1.0f,
                  c->amp ? c->amp_found : nullptr, s);
  }
  const double bc1 = 1.0 - std::pow((double)beta1, (double)t);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)t);
  {
    Timed tm(c, "adamw", 0, (b.params_bf16 ? 30.0 : 28.0) * n_params);
    adamw(b.params, b.grads, b.adam_m, b.adam_v, b.params_bf16, n_params, seg, clip_scale,
          c->amp ? c->amp_found : nullptr, lr, beta1, beta2, eps, weight_decay, (float)(1.0 / bc1),
          (float)(1.0 / bc2), s);
  }
}

}  // namespace

int GPT2_API(gpt2_clip_adamw_step)(gpt2_ctx* c, float lr, float beta1, float beta2, float eps, float weight_decay,
                         float max_norm, float* d_norm, int32_t* d_clipped) {
  if (!c || !d_norm || !d_clipped) return GPT2_ERR_ARG;
  GPT2_TO_F16(c->f16, f16_gpt2_clip_adamw_step(c, lr, beta1, beta2, eps, weight_decay, max_norm, d_norm, d_clipped));
  c->step += 1;
  clip_adamw_launch(c, c->buf, c->n_params, decay_segments(c->t, c->n_params), c->step, c->norm_part, c->clip_scale,
                    lr, beta1, beta2, eps, weight_decay, max_norm, d_norm, d_clipped, c->stream);
  if (c->amp) {  // the scale update needs the device's overflow flag of this step
    int32_t found = 0;
    if (hipMemcpyAsync(&found, c->amp_found, sizeof(found), hipMemcpyDeviceToHost, c->stream) != hipSuccess ||
        hipStreamSynchronize(c->stream) != hipSuccess)
      return GPT2_ERR_HIP;
    c->amp_skipped = found ? 1 : 0;
    if (found) {
      c->step -= 1;
      c->amp_scale *= c->amp_backoff;
      c->amp_good = 0;
    } else if (++c->amp_good >= c->amp_interval) {
      // a growth that would overflow fp32 is not taken (an infinite scale
      // could never back off again)
      if (std::isfinite(c->amp_scale * c->amp_growth)) c->amp_scale *= c->amp_growth;
      c->amp_good = 0;
    }
  }
  return hip_status();
}

int GPT2_API(gpt2_clip_adamw_step_static)(const gpt2_config* cfg, const gpt2_buffers* bufs, void* hip_stream, int64_t t,
                                float lr, float beta1, float beta2, float eps, float weight_decay, float max_norm,
                                float* d_norm, int32_t* d_clipped) {
  if (!cfg || !config_ok(*cfg) || !bufs || !bufs->params || !bufs->grads || !bufs->adam_m || !bufs->adam_v ||
      !d_norm || !d_clipped || t < 1)
    return GPT2_ERR_ARG;
  TensorDesc td[T_COUNT];
  tensor_table(*cfg, td);
  const int64_t n = total_params(td);
  if (n > kStaticMaxParams) {
    fprintf(stderr, "gpt2_clip_adamw_step_static: %lld parameters exceed the limit of %lld\n", (long long)n,
            (long long)kStaticMaxParams);
    return GPT2_ERR_ARG;
  }
  if (cfg->precision == GPT2_FP16) return GPT2_ERR_ARG;  // loss scaling needs the context's scaler
  gpt2_buffers b = *bufs;
  if (cfg->precision != GPT2_BF16) b.params_bf16 = nullptr;
  else if (!b.params_bf16) return GPT2_ERR_ARG;
  double* part = nullptr;
  float* clip_scale = nullptr;
  int nblk = 0;
  if (static_scratch(&part, &clip_scale, &nblk) != 0) return GPT2_ERR_HIP;
  gpt2_ctx none;  // no timing
  clip_adamw_launch(&none, b, n, decay_segments(td, n), t, part, clip_scale, lr, beta1, beta2, eps, weight_decay,
                    max_norm, d_norm, d_clipped, (hipStream_t)hip_stream);
  return hip_status();
}

void GPT2_API(gpt2_destroy)(gpt2_ctx* c) {
  if (!c) return;
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  delete c;
}

int GPT2_API(gpt2_sync_status)(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
  int flag = 0;
  if (hipMemcpy(&flag, c->err_flag, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return GPT2_ERR_HIP;
  if (flag) {
    fill_f32((float*)c->err_flag, 1, 0.f, c->stream);
    if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
    return GPT2_ERR_TOKEN;
  }
  return hip_status();
}

int GPT2_API(gpt2_sync_params)(gpt2_ctx* c) {
  if (!c) return GPT2_ERR_ARG;
  GPT2_TO_F16(c->f16, f16_gpt2_sync_params(c));
  if (c->ops16) to_bf16(c->buf.params, c->buf.params_bf16, c->n_params, c->stream);
  return hip_status();
}

int64_t GPT2_API(gpt2_get_step)(const gpt2_ctx* c) { return c ? c->step : -1; }

int GPT2_API(gpt2_set_step)(gpt2_ctx* c, int64_t t) {
  if (!c || t < 0) return GPT2_ERR_ARG;
  c->step = t;
  return GPT2_OK;
}

int GPT2_API(gpt2_tensor_info)(const gpt2_config* cfg, int index, const char** name, int64_t* offset, int64_t* numel,
                     int32_t* ndim, int64_t* dims) {
  if (!cfg || !config_ok(*cfg) || index < 0) return GPT2_ERR_ARG;
  TensorDesc t[T_COUNT];
  tensor_table(*cfg, t);
  int id = -1;
  for (int i = 0, k = 0; i < T_COUNT; ++i)
    if (t[i].present && k++ == index) {
      id = i;
      break;
    }
  if (id < 0) return GPT2_ERR_ARG;
  if (name) *name = kTensorNames[id];
  if (offset) *offset = t[id].off;
  if (numel) *numel = t[id].numel;
  if (ndim) *ndim = t[id].ndim;
  if (dims)
    for (int i = 0; i < 3; ++i) dims[i] = i < t[id].ndim ? t[id].dims[i] : 0;
  return GPT2_OK;
}

int GPT2_API(gpt2_activation)(gpt2_ctx* c, const char* name, int layer, void** ptr, int64_t* numel,
                              int32_t* dtype) {
  if (!c || !name || !ptr || !numel || !dtype) return GPT2_ERR_ARG;
  const int64_t M = (int64_t)c->B * c->T, C = c->C;
  const int32_t at = c->f16 ? 3 : c->ops16 ? 1 : 0;
  const bool lay_ok = layer >= 0 && layer < c->L;
  auto ret = [&](void* p, int64_t n, int32_t d) {
    *ptr = p;
    *numel = n;
    *dtype = d;
    return GPT2_OK;
  };
  const std::string n(name);
  if (n == "resid" && layer >= 0 && layer <= 2 * c->L) return ret(c->resid(layer), M * C, 0);
  if (n == "lnf") return ret(c->lnf, M * C, at);
  if (n == "logits") return ret(c->logits, M * c->Vp, at);
  if (n == "row_loss") return ret(c->row_loss, M, 0);
  if (n == "dresid") return ret(c->dres, M * C, 0);
  if (n == "emb_sorted_ids") return ret(c->sort_ka, M, 2);
  if (n == "emb_sorted_pos") return ret(c->sort_va, M, 2);
  if (!lay_ok) return GPT2_ERR_ARG;
  if (n == "ln1") return ret(c->layer_act(c->ln1, layer, C), M * C, at);
  if (n == "ln1_mean") return ret(c->ln1_mean + (int64_t)layer * c->Mmax, M, 0);
  if (n == "ln1_rstd") return ret(c->ln1_rstd + (int64_t)layer * c->Mmax, M, 0);
  if (n == "qkv") return ret(c->layer_act(c->qkv, layer, 3 * C), M * 3 * C, at);
  if (n == "atty") return ret(c->layer_act(c->atty, layer, C), M * C, at);
  if (n == "lse") return ret(c->lse + (int64_t)layer * c->Mmax * c->NH, M * c->NH, 0);
  if (n == "ln2") return ret(c->layer_act(c->ln2, layer, C), M * C, at);
  if (n == "fcgd") return ret(c->layer_act(c->fcgd, layer, 4 * C), M * 4 * C, at);
  if (n == "fcg") return ret(c->layer_act(c->fcg, layer, 4 * C), M * 4 * C, at);
  return GPT2_ERR_ARG;
}

int GPT2_API(gpt2_timing_enable)(gpt2_ctx* c, const char* site) {
  if (!c) return GPT2_ERR_ARG;
  c->ev_used = 0;
  c->ev_overflow = false;
  c->ev_flops.clear();
  c->ev_bytes.clear();
  c->ev_site.clear();
  c->ev_cfg.clear();
  c->timing = site != nullptr;
  c->site = site ? site : "";
  return GPT2_OK;
}

int GPT2_API(gpt2_timing_read)(gpt2_ctx* c, double* total_ms, int64_t* launches, double* flops, double* bytes) {
  if (!c || !total_ms || !launches || !flops || !bytes) return GPT2_ERR_ARG;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
  double ms = 0, f = 0, b = 0;
  for (size_t i = 0; i < c->ev_used; ++i) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, c->ev[2 * i], c->ev[2 * i + 1]) != hipSuccess) return GPT2_ERR_HIP;
    ms += t;
    f += c->ev_flops[i];
    b += c->ev_bytes[i];
  }
  *total_ms = ms;
  *launches = (int64_t)c->ev_used;
  *flops = f;
  *bytes = b;
  return c->ev_overflow ? GPT2_ERR_ARG : GPT2_OK;
}

// ---- checkpoints ------------------------------------------------------------------
// File: "GPT2CKP1", the gpt2_config, int64 step, n_params, n_extra, the extra
// words, then params, adam_m and adam_v as fp32 (little-endian, as in memory).
namespace {
constexpr char kCkptMagic[8] = {'G', 'P', 'T', '2', 'C', 'K', 'P', '1'};
constexpr int kCkptExtraMax = 16;
constexpr int64_t kCkptChunk = (int64_t)1 << 24;  // floats per staged copy

static bool same_model(const gpt2_config& a, const gpt2_config& b) {
  return a.n_layer == b.n_layer && a.n_head == b.n_head && a.n_embd == b.n_embd && a.block_size == b.block_size &&
         a.vocab_size == b.vocab_size && a.padded_vocab_size == b.padded_vocab_size && a.precision == b.precision &&
         a.variant == b.variant;
}
}  // namespace

int GPT2_API(gpt2_checkpoint_save)(gpt2_ctx* c, const char* path, const int64_t* extra, int n_extra) {
  if (!c || !path || n_extra < 0 || n_extra > kCkptExtraMax || (n_extra > 0 && !extra)) return GPT2_ERR_ARG;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
  const std::string tmp = std::string(path) + ".tmp";
  FILE* f = fopen(tmp.c_str(), "wb");
  if (!f) return GPT2_ERR_IO;
  const int64_t head[3] = {c->step, c->n_params, (int64_t)n_extra};
  uint32_t scale_bits;
  memcpy(&scale_bits, &c->amp_scale, 4);
  const int64_t amp_words[2] = {(int64_t)scale_bits, (int64_t)c->amp_good};  // fp16 mode: the loss scaler
  bool ok = fwrite(kCkptMagic, 1, 8, f) == 8 && fwrite(&c->cfg, sizeof(gpt2_config), 1, f) == 1 &&
            fwrite(head, sizeof(int64_t), 3, f) == 3 &&
            (n_extra == 0 || fwrite(extra, sizeof(int64_t), n_extra, f) == (size_t)n_extra) &&
            (!c->amp || fwrite(amp_words, sizeof(int64_t), 2, f) == 2);
  std::vector<float> stage((size_t)std::min<int64_t>(kCkptChunk, c->n_params));
  const float* src[3] = {c->buf.params, c->buf.adam_m, c->buf.adam_v};
  int err = GPT2_ERR_IO;
  for (int a = 0; a < 3 && ok; ++a) {
    for (int64_t o = 0; o < c->n_params && ok; o += kCkptChunk) {
      const int64_t n = std::min<int64_t>(kCkptChunk, c->n_params - o);
      if (hipMemcpy(stage.data(), src[a] + o, n * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) {
        ok = false;
        err = GPT2_ERR_HIP;
        break;
      }
      ok = fwrite(stage.data(), sizeof(float), n, f) == (size_t)n;
    }
  }
  ok = (fclose(f) == 0) && ok;
  if (!ok || rename(tmp.c_str(), path) != 0) {
    remove(tmp.c_str());
    return ok ? GPT2_ERR_IO : err;
  }
  return GPT2_OK;
}

int GPT2_API(gpt2_checkpoint_load)(gpt2_ctx* c, const char* path, int64_t* extra, int* n_extra) {
  if (!c || !path || !n_extra || *n_extra < 0 || (*n_extra > 0 && !extra)) return GPT2_ERR_ARG;
  GPT2_TO_F16(c->f16, f16_gpt2_checkpoint_load(c, path, extra, n_extra));
  FILE* f = fopen(path, "rb");
  if (!f) return GPT2_ERR_IO;
  char magic[8];
  gpt2_config cfg;
  int64_t head[3];
  if (fread(magic, 1, 8, f) != 8 || memcmp(magic, kCkptMagic, 8) != 0 || fread(&cfg, sizeof(cfg), 1, f) != 1 ||
      fread(head, sizeof(int64_t), 3, f) != 3 || head[2] < 0 || head[2] > kCkptExtraMax || head[0] < 0) {
    fclose(f);
    return GPT2_ERR_IO;
  }
  if (!same_model(cfg, c->cfg) || head[1] != c->n_params) {
    fclose(f);
    return GPT2_ERR_ARG;
  }
  int64_t ex[kCkptExtraMax], amp_words[2] = {0, 0};
  if ((head[2] > 0 && fread(ex, sizeof(int64_t), head[2], f) != (size_t)head[2]) ||
      (c->amp && fread(amp_words, sizeof(int64_t), 2, f) != 2)) {
    fclose(f);
    return GPT2_ERR_IO;
  }
  if (hipStreamSynchronize(c->stream) != hipSuccess) {
    fclose(f);
    return GPT2_ERR_HIP;
  }
  std::vector<float> stage((size_t)std::min<int64_t>(kCkptChunk, c->n_params));
  float* dst[3] = {c->buf.params, c->buf.adam_m, c->buf.adam_v};
  for (int a = 0; a < 3; ++a) {
    for (int64_t o = 0; o < c->n_params; o += kCkptChunk) {
      const int64_t n = std::min<int64_t>(kCkptChunk, c->n_params - o);
      if (fread(stage.data(), sizeof(float), n, f) != (size_t)n) {
        fclose(f);
        return GPT2_ERR_IO;
      }
      if (hipMemcpy(dst[a] + o, stage.data(), n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) {
        fclose(f);
        return GPT2_ERR_HIP;
      }
    }
  }
  fclose(f);
  c->step = head[0];
  if (c->amp) {
    const uint32_t scale_bits = (uint32_t)amp_words[0];
    memcpy(&c->amp_scale, &scale_bits, 4);
    c->amp_good = (int)amp_words[1];
  }
  const int nx = (int)std::min<int64_t>(head[2], *n_extra);
  for (int i = 0; i < nx; ++i) extra[i] = ex[i];
  *n_extra = nx;
  if (c->ops16) to_bf16(c->buf.params, c->buf.params_bf16, c->n_params, c->stream);
  return hip_status();
}

int GPT2_API(gpt2_embedding_backward)(gpt2_ctx* c, const int32_t* d_idx, const float* d_dx0, int B, int T) {
  if (!c || !d_idx || !d_dx0) return GPT2_ERR_ARG;
  GPT2_TO_F16(c->f16, f16_gpt2_embedding_backward(c, d_idx, d_dx0, B, T));
  if (T > c->cfg.block_size) return GPT2_ERR_SEQ_TOO_LONG;
  if (B < 1 || T < 1 || B > c->cfg.max_batch) return GPT2_ERR_BATCH;
  hipStream_t s = c->stream;
  const int M = B * T;
  Timed tm(c, "embed.bwd", 0, 12.0 * M * c->C);
  embed_wpe_grad(d_dx0, c->G(T_WPE), B, T, c->C, s);
  embed_sort(d_idx, M, c->Vp, c->id_bits, c->sort_ka, c->sort_va, c->sort_kb, c->sort_vb, s);
  embed_scatter(c->sort_ka, c->sort_va, d_dx0, c->run_sums, c->G(T_WTE), M, c->C, s);
  return hip_status();
}

int GPT2_API(gpt2_timing_site)(gpt2_ctx* c, int index, const char** site, double* total_ms, int64_t* launches,
                     double* flops, double* bytes, int32_t* gemm_cfg) {
  if (!c || index < 0 || !site || !total_ms || !launches || !flops || !bytes || !gemm_cfg) return GPT2_ERR_ARG;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return GPT2_ERR_HIP;
  // distinct sites in order of first launch
  std::vector<const char*> names;
  for (size_t i = 0; i < c->ev_used; ++i) {
    bool seen = false;
    for (const char* n : names) seen = seen || strcmp(n, c->ev_site[i]) == 0;
    if (!seen) names.push_back(c->ev_site[i]);
  }
  if ((size_t)index >= names.size()) return GPT2_ERR_ARG;
  double ms = 0, f = 0, b = 0;
  int64_t n = 0;
  int cfg = -1;
  for (size_t i = 0; i < c->ev_used; ++i) {
    if (strcmp(names[index], c->ev_site[i]) != 0) continue;
    float t = 0.f;
    if (hipEventElapsedTime(&t, c->ev[2 * i], c->ev[2 * i + 1]) != hipSuccess) return GPT2_ERR_HIP;
    ms += t;
    f += c->ev_flops[i];
    b += c->ev_bytes[i];
    cfg = c->ev_cfg[i];
    ++n;
  }
  *site = names[index];
  *total_ms = ms;
  *launches = n;
  *flops = f;
  *bytes = b;
  *gemm_cfg = cfg;
  return GPT2_OK;
}

int GPT2_API(gpt2_loss_scaler)(gpt2_ctx* c, float scale, float growth_factor, float backoff_factor,
                               int32_t growth_interval, int32_t good_steps) {
  if (!c || !c->amp) return GPT2_ERR_STATE;
  if (!(scale > 0.f) || !std::isfinite(scale) || !(growth_factor >= 1.f) || !(backoff_factor > 0.f) ||
      !(backoff_factor <= 1.f) || growth_interval < 1 || good_steps < 0 || good_steps >= growth_interval)
    return GPT2_ERR_ARG;
  c->amp_scale = scale;
  c->amp_growth = growth_factor;
  c->amp_backoff = backoff_factor;
  c->amp_interval = growth_interval;
  c->amp_good = good_steps;
  return GPT2_OK;
}

int GPT2_API(gpt2_loss_scaler_state)(const gpt2_ctx* c, float* scale, int32_t* good_steps, int32_t* skipped) {
  if (!c || !scale || !good_steps || !skipped) return GPT2_ERR_ARG;
  if (!c->amp) return GPT2_ERR_STATE;
  *scale = c->amp_scale;
  *good_steps = c->amp_good;
  *skipped = c->amp_skipped;
  return GPT2_OK;
}

}  // extern "C"
