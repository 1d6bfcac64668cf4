// Host-side launchers of the decoding kernels (infer.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace gpt2k {

// cache[(b Tmax + t0 + t)][0 : 2C] = qkv[b T + t][C : 3C] (the keys and values of
// rows (b, t) of a (B, T, 3C) QKV activation into a (B, Tmax, 2C) cache).
template <typename TA>
void kv_store(const TA* qkv, TA* cache, int B, int T, int t0, int Tmax, int C, hipStream_t s);
// dst (B, C) = the rows (b, T - 1) of src (B, T, C).
template <typename TA>
void last_rows(const TA* src, TA* dst, int B, int T, int C, hipStream_t s);
// y (B, C) = causal attention of the single query of each sequence (qkv
// (B, 3C)) over keys and values 0 .. n_keys - 1 of its cache rows (the last
// one its own).  Returns false for shapes the kernel does not take.
template <typename TA>
bool decode_attn(const TA* qkv, const TA* cache, TA* y, int B, int n_keys, int Tmax, int C, int NH, hipStream_t s);
// bf16 C = epilogue(A B^T) for M <= 32 rows with the weights read once (the
// one-token decoding step); epilogues EPI_ACT, EPI_F32, EPI_RESID (C fp32 =
// resid + acc + bias, resid with C's row stride) and EPI_GELU.  Returns false
// (nothing launched) for shapes it does not take: M > 32, K % 16, unaligned
// rows.  With a cache (EPI_ACT, N = 3C: the QKV product of a decoding step)
// the key and value columns of output row m also go to row (m, pos) of that
// (B, Tmax, 2C) cache.
bool gemm_skinny(GemmEpilogue epi, const GemmArgs& a, hipStream_t s, h16* cache = nullptr, int Tmax = 0,
                 int pos = 0, int C = 0);
// The same product for M <= 16 rows with A = LayerNorm(x): x fp32 (M x K, row
// stride a.lda), gain w and shift b (K); each row normalised as
// (x - mean) rstd w + b and rounded to bf16 in the prologue (a.A unused).
// Epilogues EPI_ACT (with the cache as above), EPI_F32 and EPI_GELU.  Returns
// false (nothing launched) for shapes it does not take (M > 16, K % 32, K > 2048).
bool gemm_skinny_ln(GemmEpilogue epi, const GemmArgs& a, const float* x, const float* w, const float* b,
                    hipStream_t s, h16* cache = nullptr, int Tmax = 0, int pos = 0, int C = 0);
// out[b] = a column of logits row b (fp32, row stride ld) among [0, V):
// temperature <= 0 or top_k == 1: the first largest; else z = logits / T,
// columns below the k-th largest z dropped (top_k > 0), p = softmax(z),
// columns outside the smallest most-probable set of mass >= top_p dropped
// (0 < top_p < 1; ties at the threshold kept), and the column where the
// running sum of the kept p in column order first exceeds uniform[b] times
// their total.
bool sample(const float* logits, int64_t ld, int B, int V, float temperature, int top_k, float top_p,
            const float* uniform, int32_t* out, hipStream_t s);

}  // namespace gpt2k
