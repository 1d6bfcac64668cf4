// Global gradient norm, clip decision and one multi-tensor AdamW pass over the
// flat fp32 parameter vector (HBM-bound).
#include <cstdio>
#include <mutex>

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

__global__ void to_bf16_kernel(const float* __restrict__ src, h16* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i + 3 < n) {
    float v[4];
    load4(src + 4 * i, v);
    store4(dst + 4 * i, v);
  } else {
    for (int64_t j = 4 * i; j < n; ++j) dst[j] = (h16)src[j];
  }
}

void to_bf16(const float* src, void* dst, int64_t n, hipStream_t s) {
  const int64_t work = (n + 3) / 4;
  to_bf16_kernel<<<(unsigned)((work + 255) / 256), 256, 0, s>>>(src, reinterpret_cast<h16*>(dst), n);
}

constexpr int kNormBlocks = 1024;

// Each thread keeps four 16-byte loads in flight per round (a read-only
// stream needs that many bytes outstanding per CU to cover the HBM latency).
__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ g, int64_t n, double* part) {
  __shared__ double red[16];
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  double acc = 0.0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    float v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) load4(g + 4 * (i + u * stride), v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += (double)v[u][e] * (double)v[u][e];
  }
  for (; i < n4; i += stride) {
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
                                                            float* scale_out, float inv_loss_scale,
                                                            int32_t* found_inf) {
  __shared__ double red[16];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) s += part[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) {
    // gradients held times the loss scale: the norm of the true gradients is
    // the scaled norm over the scale, and the update multiplies by both
    // factors (the clip factor, then the unscale)
    const double norm = sqrt(s) * (double)inv_loss_scale;
    const double coef = (double)max_norm / (norm + 1e-6);
    const bool clip = coef < 1.0;
    *d_norm = (float)norm;
    *d_clipped = clip ? 1 : 0;
    *scale_out = (clip ? (float)coef : 1.0f) * inv_loss_scale;
    if (found_inf) *found_inf = isfinite(norm) ? 0 : 1;
  }
}

void clip_finalize(const double* part, int nblk, float max_norm, float* d_norm, int32_t* d_clipped,
                   float* scale_out, float inv_loss_scale, int32_t* found_inf, hipStream_t s) {
  clip_finalize_kernel<<<1, 256, 0, s>>>(part, nblk, max_norm, d_norm, d_clipped, scale_out, inv_loss_scale,
                                         found_inf);
}

template <bool BF16>
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    h16* __restrict__ pb, int64_t n4, DecaySegments seg,
                                                    const float* __restrict__ grad_scale,
                                                    const int32_t* __restrict__ skip, float lr, float beta1,
                                                    float beta2, float eps, float wd, float inv_bc1,
                                                    float inv_bc2) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  if (skip && *skip) return;  // a skipped step (non-finite gradient under loss scaling)
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
  if constexpr (BF16) {
    // the 16-bit copy rounds the stored fp32 value, as to_bf16 does (for
    // fp16 the compiler would otherwise fuse the rounding into the update's
    // fma, v_fma_mix, and a copy rebuilt from the fp32 weights, as after a
    // checkpoint, would differ from it)
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(pp[e]));
    store4(pb + e0, pp);
  }
}

void adamw(float* p, const float* g, float* m, float* v, void* p_bf16, int64_t n, const DecaySegments& seg,
           const float* grad_scale, const int32_t* skip, float lr, float beta1, float beta2, float eps, float wd,
           float inv_bc1, float inv_bc2, hipStream_t s) {
  const int64_t n4 = n / 4;
  const unsigned grid = (unsigned)((n4 + 255) / 256);
  if (p_bf16)
    adamw_kernel<true><<<grid, 256, 0, s>>>(p, g, m, v, reinterpret_cast<h16*>(p_bf16), n4, seg, grad_scale, skip,
                                            lr, beta1, beta2, eps, wd, inv_bc1, inv_bc2);
  else
    adamw_kernel<false><<<grid, 256, 0, s>>>(p, g, m, v, nullptr, n4, seg, grad_scale, skip, lr, beta1, beta2,
                                             eps, wd, inv_bc1, inv_bc2);
}

// ---- scratch in device memory that nothing allocates ----------------------------
// The norm's fp64 partials (kNormBlocks) and the clip factor for callers that
// cannot allocate.  Each device holds its own copy from module load until the
// process ends; the host-side name of the array is not a device address, so
// host code only ever uses the address hipGetSymbolAddress returns for the
// current device.
constexpr int kStaticScratchDoubles = kNormBlocks + 32;
static __device__ __align__(256) double scratch[kStaticScratchDoubles];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int static_scratch(double** partials, float** clip_scale, int* nblk) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fprintf(stderr, "gpt2: hipGetSymbolAddress(scratch) failed on device %d: %s\n", dev, hipGetErrorString(e));
      return -1;
    }
    g_scratch_ptr[dev] = ptr;
  }
  double* base = static_cast<double*>(g_scratch_ptr[dev]);
  *partials = base;
  *clip_scale = reinterpret_cast<float*>(base + kNormBlocks);
  *nblk = kNormBlocks;
  return 0;
}

}  // namespace gpt2k
