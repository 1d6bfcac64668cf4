// Host-side launchers of the gfx950 kernels of the GPT-2 step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt2k {

// ---- GEMM ---------------------------------------------------------------------
// C[m][n] = sum_k A(m, k) B(k, n), fp32 accumulation, then an epilogue.
enum GemmLayout {
  LAYOUT_NT = 0,  // A stored [M][K], B stored [N][K]   (forward: x W^T)
  LAYOUT_NN = 1,  // A stored [M][K], B stored [K][N]   (input gradient: dY W)
  LAYOUT_TN = 2,  // A stored [K][M], B stored [K][N]   (weight gradient: dY^T X)
};
enum GemmEpilogue {
  EPI_ACT = 0,       // C (activation type) = acc (+ bias[n] if bias)
  EPI_F32 = 1,       // C (fp32) = acc
  EPI_F32_ACC = 2,   // C (fp32) += acc
  EPI_RESID = 3,     // C (fp32) = resid + acc + bias[n]
  EPI_GELU = 4,      // u = acc + bias[n]: gelu'(u) -> C (act), gelu(u) -> C2 (act)
  EPI_GELU_BWD = 5,  // C (act) = acc * aux[m][n]  (aux = the stored gelu'(u))
  EPI_PARTIAL = 6,   // C (fp32) + split * split_stride = acc (split-K partial)
  EPI_LOGITS = 7,    // C (activation type) = acc; the lm_head product (its own kernel symbol)
};
struct GemmArgs {
  const void* A;
  const void* B;
  int M, N, K;
  int64_t lda, ldb, ldc;
  void* C;
  void* C2;
  const float* bias;
  const float* resid;
  const void* aux;
  int splits;
  int k_per_split;
  int64_t split_stride;
  int group_m;     // tile-rows walked together (0: default 8)
  int no_xcd_map;  // 1: keep the hardware block order (no per-XCD renumbering)
  // EPI_GELU_BWD only (or null): column sums of C per 64-row chunk, fp32
  // [ceil(M/64)][N] with ldc == N, each chunk's rows added in ascending order
  // (formed in the epilogue where the tile allows it, else by a pass over C)
  float* colsum;
};
// One product of a grouped launch: fp32 C[M][N] += A^T B with A stored
// [K][M] (lda) and B stored [K][N] (ldb), bf16 operands.
struct GemmProblem {
  const void* A;
  const void* B;
  void* C;        // ldc = N
  int M, N, K;
  int lda, ldb;
};
constexpr int kGroupMax = 64;
constexpr int kGroupXcds = 8;     // workgroups are dealt to the XCDs round-robin
constexpr int kGroupTailMax = 16;  // split tail tiles per XCD
struct GemmGroup {
  GemmProblem prob[kGroupMax];
  int first[kGroupMax];  // first tile of each problem
  int n;
  // per XCD: its contiguous range of tiles, and how many of the last ones
  // are computed as two K halves into part (slot x * kGroupTailMax + i, two
  // 256 x 256 fp32 blocks each) and added into C by a second kernel
  int xstart[kGroupXcds], xcount[kGroupXcds], xsplit[kGroupXcds];
  float* part;
};
static_assert(sizeof(GemmGroup) <= 4096, "kernel argument size");
// Whether a problem can go into a grouped launch (K a multiple of 64, M and N
// multiples of 8).
bool gemm_group_ok(const GemmProblem& p);
// All problems in as few launches as kGroupMax allows, with about equal tile
// counts per launch (256 x 256 tiles; each tile adds its whole-K product into
// C).  Problems must not overlap in C.  Where an XCD's last round of tiles
// would leave most of its CUs idle, those tiles run as two K halves into
// scratch (part, part_elems fp32; null: never) and a fixed-order pass adds
// both halves into C, so the result stays deterministic.
void gemm_group_tn_acc(const GemmProblem* probs, int n, float* part, int64_t part_elems, hipStream_t s);
// The tile configuration gemm_cfg launches for these arguments (cfg < 0:
// the automatic choice), kGemmCfgF32 in fp32 mode, or -1 if the shape breaks
// a kernel precondition.
constexpr int kGemmCfgF32 = 100;
int gemm_resolve_config(int cfg, GemmLayout layout, GemmEpilogue epi, bool bf16_mode, const GemmArgs& a);
// Returns false if the shape breaks a kernel precondition.
bool gemm(GemmLayout layout, GemmEpilogue epi, bool bf16_mode, const GemmArgs& a, hipStream_t s);
// Same with an explicit bf16 tile configuration (cfg < 0: automatic choice).
bool gemm_cfg(int cfg, GemmLayout layout, GemmEpilogue epi, bool bf16_mode, const GemmArgs& a, hipStream_t s);
// The tile configuration the automatic choice takes for these shapes, and the
// modelled time of a configuration (seconds).
int gemm_pick_config(const GemmArgs& a, GemmLayout layout);
double gemm_model_time(int cfg, const GemmArgs& a, bool transposed_a);
// Whether a configuration can run these shapes.
bool gemm_config_usable(int cfg, GemmLayout layout, const GemmArgs& a);
constexpr int kGemmConfigs = 23;
// Block tile of a configuration.
void gemm_config_tile(int cfg, int* bm, int* bn);
// out[i] += sum_{s < splits} part[s * stride + i], i < count (fixed order).
void splitk_reduce_add(float* out, const float* part, int splits, int64_t stride, int64_t count,
                       hipStream_t s);

// ---- embedding ---------------------------------------------------------------
// x[m][:] = wte[idx[m]][:] + wpe[m % T][:]; out-of-range ids set *err and use row 0;
// ids_out[m] receives the id used.
void embed_fwd(const int32_t* idx, const float* wte, const float* wpe, float* x, int32_t* ids_out, int M, int T,
               int C, int vocab, int* err, hipStream_t s);
// Stable sort of (idx[m], m) by id into (keys_a, vals_a): a bitonic sort in
// LDS for M <= 32768 and ids below 65535, else an LSD radix sort (4-bit
// digits, one workgroup, keys_b / vals_b as the other buffer).
void embed_sort(const int32_t* idx, int M, int vocab, int id_bits, int32_t* keys_a, int32_t* vals_a,
                int32_t* keys_b, int32_t* vals_b, hipStream_t s);
// The bitonic sort of nb independent arrays of M ids at once (array b at
// idx + b M into keys / vals + b M; out-of-range ids sort as id 0), one
// workgroup each.  Returns false (nothing launched) where the bitonic sort
// does not apply.
bool embed_sort_batch(const int32_t* idx, int M, int nb, int vocab, int32_t* keys, int32_t* vals, hipStream_t s);
// dwte[id] += sum over positions with that id of dx[pos] (in position order);
// run_sums: M x C fp32 scratch.
void embed_scatter(const int32_t* sorted_ids, const int32_t* sorted_pos, const float* dx, float* run_sums,
                   float* dwte, int M, int C, hipStream_t s);
// dwpe[t] += sum_b dx[b * T + t].
void embed_wpe_grad(const float* dx, float* dwpe, int B, int T, int C, hipStream_t s);

// ---- LayerNorm -------------------------------------------------------------------
template <typename TA>
void layernorm_fwd(const float* x, const float* w, const float* b, TA* y, float* mean, float* rstd, int M,
                   int C, hipStream_t s);
// dres (fp32, in place) = (dres_in ? dres : 0) + dx;  dres_act = dres as TA.
// Partial column sums per row chunk: part[0][chunk][C] = sum dy*xhat, part[1] = sum dy,
// part[2] = sum dres_out.  Returns the number of chunks.
template <typename TA>
int layernorm_bwd(const TA* dy, const float* x, const float* mean, const float* rstd, const float* w,
                  float* dres, bool dres_in, TA* dres_act, float* part, int M, int C, hipStream_t s);
// A column-partial reduction deferred to one batched launch: out[k][n] +=
// sum over the chunks of part[k][chunk][n] for k < nout (fixed chunk order).
struct ColJob {
  float* out[3];
  const float* part;
  int chunks, N, nout;
};
constexpr int kColJobsMax = 64;
struct ColJobs {
  ColJob job[kColJobsMax];
  int first[kColJobsMax];  // first block of each job
  int n;
};
static_assert(sizeof(ColJobs) <= 4096, "kernel argument size");
// Launches the jobs (kColJobsMax per launch); each output is written by one job.
// N a multiple of 4, part and the outputs 16-byte aligned.
void colpart_reduce_batch(const ColJob* jobs, int n, hipStream_t s);
// Column sums of an activation matrix (M x N, row-major) into partials [chunks][N];
// returns the number of chunks.
template <typename TA>
int colsum_partials(const TA* x, int M, int N, float* part, hipStream_t s);

// ---- attention ---------------------------------------------------------------------
// qkv: [B*T][3C]; y: [B*T][C]; lse: [B][NH][T] (natural log).
void attn_fwd_bf16(const void* qkv, void* y, float* lse, int B, int T, int NH, int C, hipStream_t s);
// colsum (or null): column sums of dqkv per 64-token chunk, fp32 [M/64][3C],
// each chunk's tokens added in ascending order; formed only when T % 64 == 0
// (the return value says whether they were).  Dbuf: 2 B NH T floats of
// scratch (D = rowsum(dO o O), then the log-sum-exp in the exp2 domain).
bool attn_bwd_bf16(const void* qkv, const void* y, const void* dy, const float* lse, float* Dbuf, void* dqkv,
                   int B, int T, int NH, int C, float* colsum, hipStream_t s);
void attn_fwd_f32(const float* qkv, float* y, float* lse, int B, int T, int NH, int C, hipStream_t s);
void attn_bwd_f32(const float* qkv, const float* y, const float* dy, const float* lse, float* Dbuf,
                  float* dqkv, int B, int T, int NH, int C, hipStream_t s);

// ---- cross-entropy ---------------------------------------------------------------
// Per row: loss_row = logsumexp(z) - z[y]; z <- (softmax(z) - onehot(y)) * grad_scale in place.
template <typename TA>
void xent_fwd_bwd(TA* logits, const int32_t* targets, float* row_loss, int M, int V, int vocab,
                  float grad_scale, int* err, hipStream_t s);
// *out = (accumulate ? *out : 0) + scale * sum(row_loss[0..M)) (fixed order).
void loss_reduce(const float* row_loss, int M, float scale, bool accumulate, float* out, hipStream_t s);

// ---- optimizer ---------------------------------------------------------------------
void fill_f32(float* p, int64_t n, float v, hipStream_t s);
void to_bf16(const float* src, void* dst, int64_t n, hipStream_t s);
// Sum of squares into nblk fp64 partials; returns nblk.
int sumsq_partials(const float* g, int64_t n, double* part, hipStream_t s);
// norm = sqrt(sum part); coef = max_norm / (norm + 1e-6); clipped = coef < 1.
// With gradients held times a loss scale S (inv_loss_scale = 1/S, else 1) the
// norm is that of the unscaled gradients, scale_out includes 1/S, and
// found_inf (or null) is set to whether the norm is finite.
void clip_finalize(const double* part, int nblk, float max_norm, float* d_norm, int32_t* d_clipped,
                   float* scale_out, float inv_loss_scale, int32_t* found_inf, hipStream_t s);
struct DecaySegments {
  int n;
  int64_t start[24];  // segment i covers [start[i], start[i+1]) (start[n] = total)
  int decay[24];
};
// The current device's copy of the library's static scratch: room for the
// sumsq_partials of any n (nblk of them) and one clip factor.  Returns 0, or
// -1 if the device address cannot be found.
int static_scratch(double** partials, float** clip_scale, int* nblk);
// skip (or null): when *skip is nonzero the update is skipped (nothing written).
void adamw(float* p, const float* g, float* m, float* v, void* p_bf16, int64_t n, const DecaySegments& seg,
           const float* grad_scale, const int32_t* skip, float lr, float beta1, float beta2, float eps, float wd,
           float inv_bc1, float inv_bc2, hipStream_t s);

}  // namespace gpt2k
