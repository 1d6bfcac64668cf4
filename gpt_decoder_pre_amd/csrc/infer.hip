// Autoregressive decoding on the step's kernels: the key / value cache, the
// attention of one new query per sequence over its cached keys, and
// temperature / top-k / top-p sampling.
#include "common.h"
#include "infer_kernels.h"
#include "kernels.h"

namespace gpt2k {

// cache[(b * Tmax + t0 + t)][0 : 2C] = qkv[b * T + t][C : 3C] (keys | values)
template <typename TA>
__global__ void kv_store_kernel(const TA* __restrict__ qkv, TA* __restrict__ cache, int B, int T, int t0, int Tmax,
                                int C) {
  constexpr int V = 16 / sizeof(TA);  // elements per 16-byte chunk
  const int chunks = 2 * C / V;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * T * chunks) return;
  const int64_t row = i / chunks;
  const int c = (int)(i % chunks) * V;
  const int b = (int)(row / T), t = (int)(row % T);
  const u32x4 v = *reinterpret_cast<const u32x4*>(qkv + row * 3 * C + C + c);
  *reinterpret_cast<u32x4*>(cache + ((int64_t)b * Tmax + t0 + t) * 2 * C + c) = v;
}

template <typename TA>
void kv_store(const TA* qkv, TA* cache, int B, int T, int t0, int Tmax, int C, hipStream_t s) {
  const int64_t n = (int64_t)B * T * (2 * C / (16 / (int)sizeof(TA)));
  kv_store_kernel<TA><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(qkv, cache, B, T, t0, Tmax, C);
}

// dst[b] = src[b * T + T - 1] (the last position of every sequence)
template <typename TA>
__global__ void last_rows_kernel(const TA* __restrict__ src, TA* __restrict__ dst, int B, int T, int C) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * C) return;
  const int b = (int)(i / C), c = (int)(i % C);
  dst[i] = src[((int64_t)b * T + T - 1) * C + c];
}

template <typename TA>
void last_rows(const TA* src, TA* dst, int B, int T, int C, hipStream_t s) {
  const int64_t n = (int64_t)B * C;
  last_rows_kernel<TA><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src, dst, B, T, C);
}

// One new query per sequence against its n_keys cached keys (the query's own
// key and value are the last of them): workgroup (head, sequence).  A key's
// row is read by TPK threads, 16 bytes each, so a pass covers KP = 256 / TPK
// keys; each thread issues the loads of KR passes before it uses any of them,
// so that a round trip to memory is paid once per KR passes.  The scores go
// to LDS, then the block's softmax, then the same threads sum p_j v_j for
// every KP-th key and the KP partial rows are added in order.
template <typename TA, int TPK>
__global__ __launch_bounds__(256) void decode_attn_kernel(const TA* __restrict__ qkv, const TA* __restrict__ cache,
                                                          TA* __restrict__ y, int n_keys, int Tmax, int C, int NH,
                                                          float scale) {
  extern __shared__ float sm[];  // [n_keys] scores, then [KP][hd] partial rows
  __shared__ float red[16];
  constexpr int V = 16 / sizeof(TA);  // elements per 16-byte chunk
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  constexpr int hd = TPK * V;
  constexpr int tpk = TPK;       // threads per key row (a power of two)
  constexpr int kp = 256 / tpk;  // keys per pass
  const int sub = tid % tpk, kq = tid / tpk;
  float q[V];
  {
    const TA* qr = qkv + (int64_t)b * 3 * C + h * hd + sub * V;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(qr);
    unpack16<TA>(raw, q);
  }
  const TA* kb = cache + (int64_t)b * Tmax * 2 * C + h * hd + sub * V;
  constexpr int KR = 16;  // passes whose rows are loaded together
  const u32x4 zero = {0u, 0u, 0u, 0u};
  float mx = -INFINITY;
  for (int j0 = 0; j0 < n_keys; j0 += KR * kp) {
    u32x4 raw[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int j = j0 + r * kp + kq;
      raw[r] = j < n_keys ? *reinterpret_cast<const u32x4*>(kb + (int64_t)j * 2 * C) : zero;
    }
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int j = j0 + r * kp + kq;
      float k[V];
      unpack16<TA>(raw[r], k);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) part = fmaf(q[e], k[e], part);
      for (int o = tpk / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
      if (j < n_keys && sub == 0) {
        sm[j] = part * scale;
        mx = fmaxf(mx, part * scale);
      }
    }
  }
  mx = block_max(mx, red);
  float l = 0.f;
  for (int j = tid; j < n_keys; j += blockDim.x) {
    const float pj = expf(sm[j] - mx);
    sm[j] = pj;
    l += pj;
  }
  l = block_sum(l, red);  // its barriers also order the writes of the probabilities
  __syncthreads();
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  for (int j0 = 0; j0 < n_keys; j0 += KR * kp) {
    u32x4 raw[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int j = j0 + r * kp + kq;
      raw[r] = j < n_keys ? *reinterpret_cast<const u32x4*>(kb + C + (int64_t)j * 2 * C) : zero;
    }
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int j = j0 + r * kp + kq;
      if (j < n_keys) {
        float v[V];
        unpack16<TA>(raw[r], v);
        const float pj = sm[j];
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = fmaf(pj, v[e], acc[e]);
      }
    }
  }
  float* part = sm + n_keys;
#pragma unroll
  for (int e = 0; e < V; ++e) part[kq * hd + sub * V + e] = acc[e];
  __syncthreads();
  if (tid < hd) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kp; ++i) sum += part[i * hd + tid];
    y[(int64_t)b * C + h * hd + tid] = from_f32<TA>(sum / l);
  }
}

template <typename TA>
bool decode_attn(const TA* qkv, const TA* cache, TA* y, int B, int n_keys, int Tmax, int C, int NH, hipStream_t s) {
  const int hd = C / NH;
  constexpr int V = 16 / sizeof(TA);
  const int tpk = hd / V;
  // 16-byte rows chunks: hd a multiple of V, tpk a power of two that fits a wavefront
  if (hd % V || tpk < 1 || tpk > 64 || (tpk & (tpk - 1)) || C % V || n_keys < 1 || n_keys > Tmax) return false;
  const int kp = 256 / tpk;
  const size_t lds = (size_t)(n_keys + kp * hd) * sizeof(float);
  if (lds > 60 * 1024) return false;
  const dim3 grid(NH, B);
  const float scale = 1.0f / sqrtf((float)hd);
#define GPT2_DECODE_ATTN(T) decode_attn_kernel<TA, T><<<grid, 256, lds, s>>>(qkv, cache, y, n_keys, Tmax, C, NH, scale)
  switch (tpk) {
    case 1: GPT2_DECODE_ATTN(1); break;
    case 2: GPT2_DECODE_ATTN(2); break;
    case 4: GPT2_DECODE_ATTN(4); break;
    case 8: GPT2_DECODE_ATTN(8); break;
    case 16: GPT2_DECODE_ATTN(16); break;
    case 32: GPT2_DECODE_ATTN(32); break;
    default: GPT2_DECODE_ATTN(64); break;
  }
#undef GPT2_DECODE_ATTN
  return true;
}


// ------------------------------------------------------------- skinny GEMM ----
// C = epilogue(A B^T) for at most 32 rows (the one-token decoding step): A
// (M x K, bf16, row stride lda), B (N x K, bf16, row stride ldb: a weight
// matrix (out, in)).  A workgroup owns 32 output columns; its NW waves (4, or
// 16 for long K) take every NW-th 16-wide k-step, one v_mfma_f32_32x32x16_bf16
// each (rows past M and columns past N read as zero), then add their 32 x 32
// partial products in LDS in wave order and apply the epilogue.  The weights
// stream from HBM once; the rows of A stay in L2.  KV (the QKV product of a
// decoding step): the key and value columns [C, 3C) of output row m also go to
// row (m, pos) of the layer's (B, Tmax, 2C) cache, so the step needs no
// separate cache store.
struct SkinnyKv {
  h16* cache;
  int Tmax, pos, C;
};
// A of a product formed as LayerNorm(x) in the prologue (skinny16)
struct SkinnyLnA {
  const float* x;
  const float* w;
  const float* b;
};
constexpr int kSkinnyU = 6;      // k-steps per wave whose loads are issued together
constexpr int kSkinnyULn16 = 4;  // the same for the sixteen-wave LayerNorm form

// output (m, n) = v plus the bias, through the epilogue
template <int EPI, bool KV>
DEVI void skinny_store(const GemmArgs& a, const SkinnyKv& kv, int m, int n, float v) {
  const float bias = a.bias ? a.bias[n] : 0.f;
  const int64_t idx = (int64_t)m * a.ldc + n;
  if constexpr (EPI == EPI_ACT) {
    const h16 out = (h16)(v + bias);
    reinterpret_cast<h16*>(a.C)[idx] = out;
    if constexpr (KV) {
      if (n >= kv.C) kv.cache[((int64_t)m * kv.Tmax + kv.pos) * 2 * kv.C + (n - kv.C)] = out;
    }
  } else if constexpr (EPI == EPI_F32) {
    reinterpret_cast<float*>(a.C)[idx] = v + bias;
  } else if constexpr (EPI == EPI_RESID) {
    reinterpret_cast<float*>(a.C)[idx] = a.resid[idx] + (v + bias);
  } else if constexpr (EPI == EPI_GELU) {
    float g, d;
    gelu_and_grad(v + bias, g, d);
    reinterpret_cast<h16*>(a.C)[idx] = (h16)d;
    reinterpret_cast<h16*>(a.C2)[idx] = (h16)g;
  }
}

template <int EPI, int NW, bool KV>
__global__ __launch_bounds__(64 * NW) void skinny_gemm_kernel(GemmArgs a, SkinnyKv kv) {
  __shared__ float red[NW][32 * 33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 32;
  const int col = lane & 31, kh = lane >> 5;
  const h16* A = reinterpret_cast<const h16*>(a.A);
  const h16* B = reinterpret_cast<const h16*>(a.B);
  const bool row_ok = col < a.M, col_ok = n0 + col < a.N;
  const h16* ar = A + (int64_t)(row_ok ? col : 0) * a.lda + 8 * kh;
  const h16* br = B + (int64_t)(col_ok ? n0 + col : 0) * a.ldb + 8 * kh;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int steps = a.K / 16;
  int ks = wave;
  for (; ks + 3 * NW < steps; ks += 4 * NW) {  // four steps per round, their loads first
    h16x8 af[4], bfr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      af[u] = __builtin_bit_cast(h16x8, ld16_or_zero(ar + 16 * (ks + NW * u), row_ok));
      bfr[u] = __builtin_bit_cast(h16x8, ld16_or_zero(br + 16 * (ks + NW * u), col_ok));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[u], bfr[u], acc, 0, 0, 0);
  }
  for (; ks < steps; ks += NW) {
    const h16x8 af = __builtin_bit_cast(h16x8, ld16_or_zero(ar + 16 * ks, row_ok));
    const h16x8 bfr = __builtin_bit_cast(h16x8, ld16_or_zero(br + 16 * ks, col_ok));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc, 0, 0, 0);
  }
  // acc[r] = partial C[row 8 (r / 4) + 4 kh + r % 4][column n0 + col]
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][(8 * (r >> 2) + 4 * kh + (r & 3)) * 33 + col] = acc[r];
  __syncthreads();
  for (int o = tid; o < 32 * 32; o += 64 * NW) {
    const int m = o >> 5, c = o & 31, n = n0 + c;
    if (m >= a.M || n >= a.N) continue;
    float v = red[0][m * 33 + c];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w][m * 33 + c];
    skinny_store<EPI, KV>(a, kv, m, n, v);
  }
}

// The same product for at most 16 rows on v_mfma_f32_16x16x32_bf16: a
// workgroup owns 16 output columns (twice the workgroups of the 32-row form,
// none of the MFMA rows wasted when a decoding batch has 16 sequences).  Each
// wave takes every NW-th 32-wide k-step and issues the loads of all its steps
// (up to U) before the first product.
//
// LNA: A = LayerNorm(x) (fp32 rows, K <= 32 U NW).  The workgroup's A loads
// then cover its M rows whole: lane (row, kq) holds eight columns of each of
// its wave's steps, so the row sums (then the sums of squared deviations) are
// added over the lane's steps, the four lanes of the row and the waves in
// LDS, and the lane normalises its values in registers as
// (x - mean) rstd w + b, rounded to bf16 for the MFMA.
//
// CW: output columns per workgroup (16, or 8 / 4 for products with few
// columns: more workgroups share the weight stream, the MFMA's other columns
// come from zero rows of B and are not stored).
template <int EPI, int NW, bool KV, bool LNA = false, int CW = 16>
__global__ __launch_bounds__(64 * NW) void skinny16_gemm_kernel(GemmArgs a, SkinnyKv kv, SkinnyLnA ln = {}) {
  // sixteen waves have 128 registers each: fewer steps per wave, and the
  // LayerNorm's gain and shift loaded after the statistics
  constexpr int U = (LNA && NW > 4) ? kSkinnyULn16 : kSkinnyU;
  constexpr bool PRE = NW <= 4;
  __shared__ float red[NW][16 * 17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  static_assert(CW == 16 || CW == 8 || CW == 4, "columns per workgroup");
  const int n0 = blockIdx.x * CW;
  const int col = lane & 15, kq = lane >> 4;
  const h16* A = reinterpret_cast<const h16*>(a.A);
  const h16* B = reinterpret_cast<const h16*>(a.B);
  const bool row_ok = col < a.M, col_ok = col < CW && n0 + col < a.N;
  const h16* br = B + (int64_t)(col_ok ? n0 + col : 0) * a.ldb + 8 * kq;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int steps = a.K / 32;
  if constexpr (LNA) {
    __shared__ float stat[2][NW][16];
    const float* xr = ln.x + (int64_t)(row_ok ? col : 0) * a.lda + 8 * kq;
    float xv[U][8], ww[U][8], bb[U][8];
    h16x8 bfr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = wave + NW * u;
      bfr[u] = __builtin_bit_cast(h16x8, ld16_or_zero(br + 32 * ks, col_ok && ks < steps));
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[u][e] = ww[u][e] = bb[u][e] = 0.f;
      if (row_ok && ks < steps) {
        load4(xr + 32 * ks, xv[u]);
        load4(xr + 32 * ks + 4, xv[u] + 4);
      }
      if (PRE && ks < steps) {  // the gain and shift come with the rows, not after the statistics
        load4(ln.w + 32 * ks + 8 * kq, ww[u]);
        load4(ln.w + 32 * ks + 8 * kq + 4, ww[u] + 4);
        load4(ln.b + 32 * ks + 8 * kq, bb[u]);
        load4(ln.b + 32 * ks + 8 * kq + 4, bb[u] + 4);
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      sum += ((xv[u][0] + xv[u][1]) + (xv[u][2] + xv[u][3])) + ((xv[u][4] + xv[u][5]) + (xv[u][6] + xv[u][7]));
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    if (kq == 0) stat[0][wave][col] = sum;
    __syncthreads();
    float mean = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) mean += stat[0][w][col];
    mean /= (float)a.K;
    float sq = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (wave + NW * u < steps) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = xv[u][e] - mean;
          sq += d * d;
        }
      }
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    if (kq == 0) stat[1][wave][col] = sq;
    __syncthreads();
    float var = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) var += stat[1][w][col];
    const float rs = 1.0f / sqrtf(var / (float)a.K + kLnEps);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = wave + NW * u;
      if (ks < steps) {
        if (!PRE) {
          load4(ln.w + 32 * ks + 8 * kq, ww[u]);
          load4(ln.w + 32 * ks + 8 * kq + 4, ww[u] + 4);
          load4(ln.b + 32 * ks + 8 * kq, bb[u]);
          load4(ln.b + 32 * ks + 8 * kq + 4, bb[u] + 4);
        }
        h16x8 af;
#pragma unroll
        for (int e = 0; e < 8; ++e) af[e] = (h16)((xv[u][e] - mean) * rs * ww[u][e] + bb[u][e]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[u], acc, 0, 0, 0);
      }
    }
  }
  const h16* ar = A + (int64_t)(row_ok ? col : 0) * a.lda + 8 * kq;
  for (int ks0 = wave; !LNA && ks0 < steps; ks0 += U * NW) {
    h16x8 af[U], bfr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + NW * u;
      af[u] = __builtin_bit_cast(h16x8, ld16_or_zero(ar + 32 * ks, row_ok && ks < steps));
      bfr[u] = __builtin_bit_cast(h16x8, ld16_or_zero(br + 32 * ks, col_ok && ks < steps));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u], bfr[u], acc, 0, 0, 0);
  }
  // acc[r] = partial C[row 4 kq + r][column n0 + col]
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][(4 * kq + r) * 17 + col] = acc[r];
  __syncthreads();
  for (int o = tid; o < 16 * 16; o += 64 * NW) {
    const int m = o >> 4, c = o & 15, n = n0 + c;
    if (m >= a.M || c >= CW || n >= a.N) continue;
    float v = red[0][m * 17 + c];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w][m * 17 + c];
    skinny_store<EPI, KV>(a, kv, m, n, v);
  }
}

template <int EPI, int NW, bool KV>
void skinny_go(const GemmArgs& a, const SkinnyKv& kv, hipStream_t s) {
  if (a.M <= 16 && a.K % 32 == 0) {
    // at most 16 rows: 16 columns per workgroup, or 8 where 16 would leave
    // too few workgroups to keep the weight stream going (the 768-column
    // products of a GPT-2 124M decoding step: 96 workgroups instead of 48;
    // measured on MI355X, 16 sequences: 34.0-34.4k -> 35.1-35.6k tokens/s,
    // and 4 columns no faster)
    if (a.N <= 1024)
      skinny16_gemm_kernel<EPI, NW, KV, false, 8><<<(unsigned)((a.N + 7) / 8), 64 * NW, 0, s>>>(a, kv);
    else
      skinny16_gemm_kernel<EPI, NW, KV><<<(unsigned)((a.N + 15) / 16), 64 * NW, 0, s>>>(a, kv);
  } else
    skinny_gemm_kernel<EPI, NW, KV><<<(unsigned)((a.N + 31) / 32), 64 * NW, 0, s>>>(a, kv);
}

template <int NW>
bool skinny_launch(GemmEpilogue epi, const GemmArgs& a, const SkinnyKv& kv, hipStream_t s) {
  if (kv.cache) {
    if (epi != EPI_ACT) return false;
    skinny_go<EPI_ACT, NW, true>(a, kv, s);
    return true;
  }
  switch (epi) {
    case EPI_ACT: skinny_go<EPI_ACT, NW, false>(a, kv, s); return true;
    case EPI_F32: skinny_go<EPI_F32, NW, false>(a, kv, s); return true;
    case EPI_RESID: skinny_go<EPI_RESID, NW, false>(a, kv, s); return true;
    case EPI_GELU: skinny_go<EPI_GELU, NW, false>(a, kv, s); return true;
    default: return false;
  }
}

template <int NW>
bool skinny_ln_launch(GemmEpilogue epi, const GemmArgs& a, const SkinnyKv& kv, const SkinnyLnA& ln, hipStream_t s) {
  const unsigned grid = (unsigned)((a.N + 15) / 16);
  if (kv.cache) {
    if (epi != EPI_ACT) return false;
    skinny16_gemm_kernel<EPI_ACT, NW, true, true><<<grid, 64 * NW, 0, s>>>(a, kv, ln);
    return true;
  }
  switch (epi) {
    case EPI_ACT: skinny16_gemm_kernel<EPI_ACT, NW, false, true><<<grid, 64 * NW, 0, s>>>(a, kv, ln); return true;
    case EPI_F32: skinny16_gemm_kernel<EPI_F32, NW, false, true><<<grid, 64 * NW, 0, s>>>(a, kv, ln); return true;
    case EPI_GELU: skinny16_gemm_kernel<EPI_GELU, NW, false, true><<<grid, 64 * NW, 0, s>>>(a, kv, ln); return true;
    default: return false;
  }
}

bool gemm_skinny_ln(GemmEpilogue epi, const GemmArgs& a, const float* x, const float* w, const float* b,
                    hipStream_t s, h16* cache, int Tmax, int pos, int C) {
  if (a.M < 1 || a.M > 16 || a.N < 1 || a.K < 32 || a.K % 32 || a.lda % 4 || a.ldb % 8 || !x || !w || !b)
    return false;
  if (cache && (epi != EPI_ACT || a.N != 3 * C || pos < 0 || pos >= Tmax)) return false;
  const SkinnyKv kv{cache, Tmax, pos, C};
  const SkinnyLnA ln{x, w, b};
  const int steps = a.K / 32;
  if (steps <= kSkinnyU * 4) return skinny_ln_launch<4>(epi, a, kv, ln, s);
  if (steps <= kSkinnyULn16 * 16) return skinny_ln_launch<16>(epi, a, kv, ln, s);
  return false;
}

bool gemm_skinny(GemmEpilogue epi, const GemmArgs& a, hipStream_t s, h16* cache, int Tmax, int pos, int C) {
  if (a.M < 1 || a.M > 32 || a.N < 1 || a.K < 16 || a.K % 16 || a.lda % 8 || a.ldb % 8) return false;
  if (cache && (epi != EPI_ACT || a.N != 3 * C || pos < 0 || pos >= Tmax)) return false;
  const SkinnyKv kv{cache, Tmax, pos, C};
  // long K over few columns (the MLP's output projection): sixteen waves share
  // the k-steps, so that a workgroup's chain of dependent steps stays short
  if (a.K > 1024 && a.N <= 4096) return skinny_launch<16>(epi, a, kv, s);
  return skinny_launch<4>(epi, a, kv, s);
}

// ---------------------------------------------------------------- sampling ----
// One workgroup of 1024 threads (16 waves) per row.  Loads are coalesced:
// lane l of wave w holds the columns 4096 w + 64 i + l, i = 0 .. 63, so column
// order is (wave, i, lane).  Thresholds are found by bitwise searches over
// ordered 32-bit keys or float bit patterns (exact), so nothing is sorted.
//
// Top-k with 2 <= k <= 1024 first bounds the k-th largest value from below by
// the k-th largest of the 1024 per-thread maxima (k threads each hold a value
// at least that large).  When at most 1024 columns reach the bound, they are
// gathered in column order into LDS and one wave finishes the row -- the
// exact k-th value, the softmax, top-p and the inverse CDF -- with no block
// barrier.  Otherwise the block works on the whole row in registers.
constexpr int kSampleThreads = 1024;
constexpr int kSampleNPT = 64;                     // columns per thread: vocabularies up to 65,536
constexpr int kSampleWaveCols = 64 * kSampleNPT;   // consecutive columns of one wave
constexpr int kSampleCand = 1024;                  // gathered candidates of the top-k path

// block-wide integer sum with one barrier: consecutive calls alternate between
// the two halves of scratch (32 entries), so a half is rewritten only after
// every thread has passed the barrier of the call in between
DEVI int block_count_alt(int v, int* scratch, int parity) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  int* half = scratch + 16 * parity;
  if ((threadIdx.x & 63) == 0) half[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += half[w];
  return r;
}

// exclusive prefix sum over the block's threads in thread order (every
// thread gets its own; blockDim.x a multiple of 64, at most 1024)
DEVI int block_excl_scan(int v, int* scratch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  __syncthreads();
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += scratch[i];
  return off + incl - v;
}

// block-wide integer sum (every thread gets it)
DEVI int block_count(int v, int* scratch) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += scratch[w];
  return r;
}

// order-preserving map of a float to an unsigned key (-inf lowest), and back.
// Without -0 and NaN among the values, key(x) >= K  <=>  x >= key_float(K) for
// every K the threshold search visits.
DEVI uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DEVI float key_float(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

// inclusive prefix sum of a float over the wave's lanes
DEVI float wave_incl_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// wave sum, the same bits in every lane: DPP exchanges inside rows of 16
// lanes (each lane adds the same pairs), then the four row sums in a fixed order
DEVI float read_lane(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
DEVI int read_lane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
template <int CTRL>
DEVI float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
DEVI int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <typename T>
DEVI T wave_sum_rows(T v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x141>(v);  // row_half_mirror: the other quad of each eight
  v += dpp_mov<0x140>(v);  // row_mirror: the other eight of each sixteen
  const T r0 = read_lane(v, 0), r1 = read_lane(v, 16), r2 = read_lane(v, 32), r3 = read_lane(v, 48);
  return (r0 + r1) + (r2 + r3);
}

DEVI int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// the thread's columns c0 + 64 i of one row (-inf past V), coalesced; with
// SCALE each is divided by the temperature as z inv_t + 0 (the + 0 turns -0
// into +0)
template <bool SCALE>
DEVI void load_row(float (&z)[kSampleNPT], const float* row, int c0, int w, int V, float inv_t) {
  if ((w + 1) * kSampleWaveCols <= V) {  // the wave's columns all lie below V
#pragma unroll
    for (int i = 0; i < kSampleNPT; ++i) {
      const float v = row[c0 + 64 * i];
      z[i] = SCALE ? v * inv_t + 0.0f : v;
    }
  } else {  // branch-free: clamped addresses, then -inf past the end
#pragma unroll
    for (int i = 0; i < kSampleNPT; ++i) {
      float v = row[min(c0 + 64 * i, V - 1)];
      if (SCALE) v = v * inv_t + 0.0f;
      z[i] = c0 + 64 * i < V ? v : -INFINITY;
    }
  }
}

// The top-k row finished by wave 0 on n <= 64 NC candidates cv (values after
// the temperature) and ci (their columns), both in column order; candidate j
// sits in lane j % 64 of chunk j / 64.
template <int NC>
DEVI void sample_candidates(const float* cv, const int* ci, int n, int top_k, float top_p, float u, int32_t* out) {
  const int lane = threadIdx.x & 63;
  float x[NC];
  uint32_t kx[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j = 64 * c + lane;
    x[c] = j < n ? cv[j] : -INFINITY;
    kx[c] = j < n ? order_key(x[c]) : 0u;  // key 0 lies below every key the search visits
  }
  // the exact k-th largest key: every column at or above it is a candidate
  uint32_t kth = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = kth | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) cnt += __popcll(__ballot(kx[c] >= cand));
    if (cnt >= top_k) kth = cand;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < NC; ++c) mx = fmaxf(mx, x[c]);
  mx = wave_max(mx);
  float e[NC], part = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    e[c] = kx[c] >= kth ? expf(x[c] - mx) : 0.f;
    part += e[c];
  }
  if (top_p > 0.f && top_p < 1.f) {
    // the largest e-threshold whose kept mass reaches top_p Z (e <= 1: bit 30 is clear)
    const float need = top_p * wave_sum_rows(part);
    uint32_t thr = 0;
    for (int bit = 29; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      const float cf = __uint_as_float(cand);
      float sp = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) sp += e[c] >= cf ? e[c] : 0.f;
      if (wave_sum_rows(sp) >= need) thr = cand;
    }
    const float cf = __uint_as_float(thr);
#pragma unroll
    for (int c = 0; c < NC; ++c) e[c] = e[c] >= cf ? e[c] : 0.f;
  }
  // inverse CDF in column order: per-chunk scans chained by their last lanes
  float cum[NC], carry = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    cum[c] = carry + wave_incl_scan(e[c]);
    carry = read_lane(cum[c], 63);
  }
  const float target = u * carry;
  int sel = -1;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint64_t m = __ballot(cum[c] > target && e[c] > 0.f);
    if (sel < 0 && m) sel = 64 * c + __builtin_ctzll(m);
  }
  if (sel < 0) {  // the target fell at or past the rounded total: the last kept column
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint64_t m = __ballot(e[c] > 0.f);
      if (m) sel = 64 * c + 63 - __builtin_clzll(m);
    }
  }
  if (lane == 0) *out = ci[sel >= 0 ? sel : 0];  // sel < 0 only for NaN input
}

// bitwise OR over the wave, the same in every lane
DEVI uint32_t wave_or(uint32_t v) {
  v |= (uint32_t)dpp_mov<0xB1>((int)v);
  v |= (uint32_t)dpp_mov<0x4E>((int)v);
  v |= (uint32_t)dpp_mov<0x141>((int)v);
  v |= (uint32_t)dpp_mov<0x140>((int)v);
  return (uint32_t)(read_lane((int)v, 0) | read_lane((int)v, 16) | read_lane((int)v, 32) | read_lane((int)v, 48));
}

__global__ __launch_bounds__(kSampleThreads) void sample_kernel(const float* __restrict__ logits, int64_t ld, int V,
                                                                float temperature, int top_k, float top_p,
                                                                const float* __restrict__ uniform,
                                                                int32_t* __restrict__ out) {
  __shared__ float redf[16];
  __shared__ int redi[16];
  __shared__ int redi2[32];
  __shared__ uint32_t bound_key;
  // 64 rows of 65: a wave's 4096 columns transposed (padded against bank
  // conflicts); its front also holds the gathered candidates
  __shared__ float big[kSampleNPT * 65];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float* row = logits + (int64_t)b * ld;
  const int c0 = w * kSampleWaveCols + lane;  // column of z[i]: c0 + 64 i
  float z[kSampleNPT];
  if (temperature <= 0.f || top_k == 1) {  // greedy: the first largest logit
    load_row<false>(z, row, c0, w, V, 1.0f);
    const int nv = c0 < V ? (V - c0 + 63) >> 6 : 0;  // this thread's columns below V
    float best = -INFINITY;
    int bi = V;  // past the end: no candidate yet
#pragma unroll
    for (int i = 0; i < kSampleNPT; ++i)
      if (i < nv && (z[i] > best || bi == V)) {
        best = z[i];
        bi = c0 + 64 * i;
      }
    // block arg-max with the lowest index on ties
    const float m = block_max(best, redf);
    int cand = (best == m) ? bi : V;
    for (int o = 32; o >= 1; o >>= 1) cand = min(cand, __shfl_xor(cand, o, 64));
    __syncthreads();
    if (lane == 0) redi[w] = cand;
    __syncthreads();
    if (t == 0) {
      int r = V;
      for (int v = 0; v < kSampleThreads / 64; ++v) r = min(r, redi[v]);
      out[b] = r;
    }
    return;
  }
  const float inv_t = 1.0f / temperature;
  if (top_k > 1 && top_k <= kSampleCand && top_k < V) {
    load_row<true>(z, row, c0, w, V, inv_t);
    // lower bound: the k-th largest of the per-thread maxima
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < kSampleNPT; ++i) tmax = fmaxf(tmax, z[i]);
    uint32_t* tkey = reinterpret_cast<uint32_t*>(big + 2 * kSampleCand);
    tkey[t] = order_key(tmax);
    __syncthreads();
    if (w == 0) {
      uint32_t k16[kSampleThreads / 64];
#pragma unroll
      for (int c = 0; c < kSampleThreads / 64; ++c) k16[c] = tkey[64 * c + lane];
      // the top 16 bits of the k-th largest key, the rest zero: still a lower bound
      uint32_t lb = 0;
      for (int bit = 31; bit >= 16; --bit) {
        const uint32_t cand = lb | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int c = 0; c < kSampleThreads / 64; ++c) cnt += __popcll(__ballot(k16[c] >= cand));
        if (cnt >= top_k) lb = cand;
      }
      if (lane == 0) bound_key = lb;
    }
    __syncthreads();
    // a bound of -inf (fewer than k threads hold a finite value) leaves the
    // whole row (its truncated key reads as NaN); otherwise the padded
    // columns (-inf) fall below it.  mk: bit i set when column c0 + 64 i is a
    // candidate.
    const float lbf = key_float(bound_key);
    uint64_t mk = 0;
    int wc = kSampleCand + 1;
    if (lbf > -INFINITY) {
#pragma unroll
      for (int i = 0; i < kSampleNPT; ++i) mk |= (uint64_t)(z[i] >= lbf ? 1 : 0) << i;
      wc = wave_sum_rows((int)__popcll(mk));
    }
    if (lane == 0) redi[w] = wc;
    __syncthreads();
    int n = 0, off = 0;
    for (int v = 0; v < kSampleThreads / 64; ++v) {
      if (v == w) off = n;
      n += redi[v];
    }
    if (n <= kSampleCand) {
      float* cv = big;
      int* ci = reinterpret_cast<int*>(big + kSampleCand);
      // the columns i with a candidate in some lane of the wave
      const uint64_t any = ((uint64_t)wave_or((uint32_t)(mk >> 32)) << 32) | wave_or((uint32_t)mk);
      // a copy of c0 the compiler cannot match with the load addresses, so
      // that it recomputes each column here instead of keeping 64 of them
      int cb = c0;
      asm volatile("" : "+v"(cb));
#pragma unroll
      for (int i = 0; i < kSampleNPT; ++i) {
        if ((any >> i) & 1) {
          const bool p = (mk >> i) & 1;
          const uint64_t m = __ballot(p);
          if (p) {
            const int j = off + lanes_below(m);
            cv[j] = z[i];
            ci[j] = cb + 64 * i;
          }
          off += __popcll(m);
        }
      }
      __syncthreads();
      if (w == 0) {
        const float ub = uniform[b];
        if (n <= 64) sample_candidates<1>(cv, ci, n, top_k, top_p, ub, out + b);
        else if (n <= 128) sample_candidates<2>(cv, ci, n, top_k, top_p, ub, out + b);
        else if (n <= 256) sample_candidates<4>(cv, ci, n, top_k, top_p, ub, out + b);
        else if (n <= 512) sample_candidates<8>(cv, ci, n, top_k, top_p, ub, out + b);
        else sample_candidates<16>(cv, ci, n, top_k, top_p, ub, out + b);
      }
      return;
    }
    __syncthreads();  // redi is reused below
  }

  // the whole row.  It is loaded again (from L2): the registers of the first
  // load are then free over this part, which needs more of them.
  {
    const float* again = row;
    asm volatile("" : "+s"(again));  // a pointer the compiler cannot match with row
    load_row<true>(z, again, c0, w, V, inv_t);
  }
  // top-k: the k-th largest key; columns below it drop out
  uint32_t kth = 0;
  if (top_k > 0 && top_k < V) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = kth | (1u << bit);
      const float cf = key_float(cand);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < kSampleNPT; ++i) cnt += z[i] >= cf ? 1 : 0;
      if (block_count_alt(cnt, redi2, bit & 1) >= top_k) kth = cand;
    }
  }
  float mx = -INFINITY;
  const float kth_f = key_float(kth);
#pragma unroll
  for (int i = 0; i < kSampleNPT; ++i) {
    if (z[i] < kth_f) z[i] = -INFINITY;  // the padded columns hold -inf already
    mx = fmaxf(mx, z[i]);
  }
  mx = block_max(mx, redf);
  // unnormalised probabilities e = exp(z - max) of the kept columns
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < kSampleNPT; ++i) {
    z[i] = expf(z[i] - mx);
    part += z[i];
  }
  const float Z = block_sum(part, redf);
  // top-p: the largest e-threshold whose kept mass reaches top_p Z
  if (top_p > 0.f && top_p < 1.f) {
    const float need = top_p * Z;
    // few columns left: gather them and give each its mass at or above it,
    // S(e) = sum of the kept e' >= e; the threshold is the largest e with
    // S(e) >= need
    int mine_n = 0;
#pragma unroll
    for (int i = 0; i < kSampleNPT; ++i) mine_n += z[i] > 0.f ? 1 : 0;
    const int nk = block_count(mine_n, redi);
    if (nk <= kSampleThreads) {
      float* scan = big;
      int pos = block_excl_scan(mine_n, redi);
#pragma unroll
      for (int i = 0; i < kSampleNPT; ++i)
        if (z[i] > 0.f) scan[pos++] = z[i];
      __syncthreads();
      float thr_e = 0.f;
      if (t < nk) {
        const float mine_e = scan[t];
        float sum = 0.f;
        for (int j = 0; j < nk; ++j) sum += scan[j] >= mine_e ? scan[j] : 0.f;
        if (sum >= need) thr_e = mine_e;
      }
      const float c = block_max(thr_e, redf);
#pragma unroll
      for (int i = 0; i < kSampleNPT; ++i) z[i] = z[i] >= c ? z[i] : 0.f;
      __syncthreads();  // big[] is reused below
    } else {
      uint32_t thr = 0;
      for (int bit = 29; bit >= 0; --bit) {  // e <= 1: bit 30 is clear
        const uint32_t cand = thr | (1u << bit);
        const float c = __uint_as_float(cand);
        float sp = 0.f;
#pragma unroll
        for (int i = 0; i < kSampleNPT; ++i) sp += z[i] >= c ? z[i] : 0.f;
        if (block_sum(sp, redf) >= need) thr = cand;
      }
      const float c = __uint_as_float(thr);
#pragma unroll
      for (int i = 0; i < kSampleNPT; ++i) z[i] = z[i] >= c ? z[i] : 0.f;
    }
  }
  // inverse CDF in column order.  A fixed-order scan over the 16 wave sums
  // (each wave covers consecutive columns) finds the wave whose range holds
  // u * total; that wave transposes its columns through LDS so that lane l
  // holds the 64 consecutive ones 64 l .. 64 l + 63, scans the lanes' sums and
  // the lane holding the target walks its columns.
  float mine = 0.f;
#pragma unroll
  for (int i = 0; i < kSampleNPT; ++i) mine += z[i];
  const float ws = wave_sum(mine);
  __syncthreads();
  if (lane == 0) redf[w] = ws;
  __syncthreads();
  float before = 0.f, total = 0.f;
  for (int v = 0; v < kSampleThreads / 64; ++v) {
    if (v == w) before = total;
    total += redf[v];
  }
  const float target = uniform[b] * total;
  if (target < total) {
    if (target >= before && target < before + ws) {  // this wave (the same for all its lanes)
#pragma unroll
      for (int i = 0; i < kSampleNPT; ++i) big[65 * i + lane] = z[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float* mycols = big + 65 * lane;  // columns w 4096 + 64 lane + m
      float ls = 0.f;
      for (int m = 0; m < kSampleNPT; ++m) ls += mycols[m];
      const float incl = wave_incl_scan(ls);
      float excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = 0.f;
      uint64_t hit = __ballot(before + incl > target && ls > 0.f);
      const bool walk_all = hit == 0;  // rounding at the wave's end: its last kept column
      if (walk_all) hit = __ballot(ls > 0.f);
      const int L = walk_all ? 63 - __builtin_clzll(hit) : __builtin_ctzll(hit);
      if (lane == L) {
        int sel = -1, last = -1;
        float c = before + excl;
        for (int m = 0; m < kSampleNPT; ++m) {
          const float e = mycols[m];
          if (e > 0.f) {
            last = m;
            if (sel < 0 && !walk_all) {
              c += e;
              if (target < c) sel = m;
            }
          }
        }
        out[b] = w * kSampleWaveCols + 64 * L + (sel >= 0 ? sel : last);
      }
    }
    return;
  }
  // the target fell at or past the rounded total: the last kept column
  int li = -1;
#pragma unroll
  for (int i = 0; i < kSampleNPT; ++i)
    if (z[i] > 0.f) li = i;
  int last = li >= 0 ? c0 + 64 * li : -1;
  for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (lane == 0) redi[w] = last;
  __syncthreads();
  if (t == 0) {
    int r = -1;
    for (int v = 0; v < kSampleThreads / 64; ++v) r = max(r, redi[v]);
    out[b] = r;
  }
}

bool sample(const float* logits, int64_t ld, int B, int V, float temperature, int top_k, float top_p,
            const float* uniform, int32_t* out, hipStream_t s) {
  if (V < 1 || V > kSampleThreads * kSampleNPT || B < 1) return false;
  sample_kernel<<<B, kSampleThreads, 0, s>>>(logits, ld, V, temperature, top_k, top_p, uniform, out);
  return true;
}

template void kv_store<float>(const float*, float*, int, int, int, int, int, hipStream_t);
template void kv_store<h16>(const h16*, h16*, int, int, int, int, int, hipStream_t);
template void last_rows<float>(const float*, float*, int, int, int, hipStream_t);
template void last_rows<h16>(const h16*, h16*, int, int, int, hipStream_t);
template bool decode_attn<float>(const float*, const float*, float*, int, int, int, int, int, hipStream_t);
template bool decode_attn<h16>(const h16*, const h16*, h16*, int, int, int, int, int, hipStream_t);

}  // namespace gpt2k
