// Global gradient norm, clip decision and one multi-tensor AdamW pass over the
// flat fp32 parameter vector (HBM-bound).
#include "common.h"
#include "kernels.h"

namespace gpt2k {

__global__ void fill_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = n >> 2;
  if (i < n4) {
    float t[4] = {v, v, v, v};
    store4(p + 4 * i, t);
  } else if (i - n4 < (n & 3)) {
    p[4 * n4 + (i - n4)] = v;
  }
}

void fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  const int64_t work = (n >> 2) + 4;
  fill_kernel<<<(unsigned)((work + 255) / 256), 256, 0, s>>>(p, n, v);
}

__global__ void to_bf16_kernel(const float* __restrict__ src, bf16* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i + 3 < n) {
    float v[4];
    load4(src + 4 * i, v);
    store4(dst + 4 * i, v);
  } else {
    for (int64_t j = 4 * i; j < n; ++j) dst[j] = (bf16)src[j];
  }
}

void to_bf16(const float* src, void* dst, int64_t n, hipStream_t s) {
  const int64_t work = (n + 3) / 4;
  to_bf16_kernel<<<(unsigned)((work + 255) / 256), 256, 0, s>>>(src, reinterpret_cast<bf16*>(dst), n);
}

constexpr int kNormBlocks = 1024;

__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ g, int64_t n, double* part) {
  __shared__ double red[16];
  const int64_t n4 = n >> 2;
  double acc = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    float v[4];
    load4(g + 4 * i, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += (double)v[e] * (double)v[e];
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const double v = g[4 * n4 + threadIdx.x];
    acc += v * v;
  }
  acc = block_sum(acc, red);
  if (threadIdx.x == 0) part[blockIdx.x] = acc;
}

int sumsq_partials(const float* g, int64_t n, double* part, hipStream_t s) {
  sumsq_kernel<<<kNormBlocks, 256, 0, s>>>(g, n, part);
  return kNormBlocks;
}

__global__ __launch_bounds__(256) void clip_finalize_kernel(const double* __restrict__ part, int nblk,
                                                            float max_norm, float* d_norm, int32_t* d_clipped,
                                                            float* scale_out) {
  __shared__ double red[16];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) s += part[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) {
    const double norm = sqrt(s);
    const double coef = (double)max_norm / (norm + 1e-6);
    const bool clip = coef < 1.0;
    *d_norm = (float)norm;
    *d_clipped = clip ? 1 : 0;
    *scale_out = clip ? (float)coef : 1.0f;
  }
}

void clip_finalize(const double* part, int nblk, float max_norm, float* d_norm, int32_t* d_clipped,
                   float* scale_out, hipStream_t s) {
  clip_finalize_kernel<<<1, 256, 0, s>>>(part, nblk, max_norm, d_norm, d_clipped, scale_out);
}

template <bool BF16>
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16* __restrict__ pb, int64_t n4, DecaySegments seg,
                                                    const float* __restrict__ grad_scale, float lr, float beta1,
                                                    float beta2, float eps, float wd, float inv_bc1,
                                                    float inv_bc2) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const int64_t e0 = 4 * i;
  int decay = 0;
  for (int k = 0; k < seg.n; ++k)
    if (e0 >= seg.start[k] && e0 < seg.start[k + 1]) decay = seg.decay[k];
  const float gs = *grad_scale;
  float pp[4], gg[4], mm[4], vv[4];
  load4(p + e0, pp);
  load4(g + e0, gg);
  load4(m + e0, mm);
  load4(v + e0, vv);
  const float shrink = decay ? 1.0f - lr * wd : 1.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float gr = gg[e] * gs;
    mm[e] = beta1 * mm[e] + (1.0f - beta1) * gr;
    vv[e] = beta2 * vv[e] + (1.0f - beta2) * gr * gr;
    const float denom = sqrtf(vv[e] * inv_bc2) + eps;
    pp[e] = pp[e] * shrink - lr * (mm[e] * inv_bc1) / denom;
  }
  store4(p + e0, pp);
  store4(m + e0, mm);
  store4(v + e0, vv);
  if constexpr (BF16) store4(pb + e0, pp);
}

void adamw(float* p, const float* g, float* m, float* v, void* p_bf16, int64_t n, const DecaySegments& seg,
           const float* grad_scale, float lr, float beta1, float beta2, float eps, float wd, float inv_bc1,
           float inv_bc2, hipStream_t s) {
  const int64_t n4 = n / 4;
  const unsigned grid = (unsigned)((n4 + 255) / 256);
  if (p_bf16)
    adamw_kernel<true><<<grid, 256, 0, s>>>(p, g, m, v, reinterpret_cast<bf16*>(p_bf16), n4, seg, grad_scale, lr,
                                            beta1, beta2, eps, wd, inv_bc1, inv_bc2);
  else
    adamw_kernel<false><<<grid, 256, 0, s>>>(p, g, m, v, nullptr, n4, seg, grad_scale, lr, beta1, beta2, eps, wd,
                                             inv_bc1, inv_bc2);
}

}  // namespace gpt2k
