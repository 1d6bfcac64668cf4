// HBM stream probes: plain read-only, write-only and copy streams over fp32
// buffers.  They are the reference rates for the HBM-bound kernels of the
// step (what this part sustains for each mix of reads and writes), not part
// of the step itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "gpt2.h"

namespace gpt2k {

// One launch walks the buffer once: workgroup g owns the contiguous 16-byte
// chunks [g 256 U, (g + 1) 256 U), thread t the chunks g 256 U + t + 256 u,
// u < U (a grid of one workgroup per chunk range; measured on MI355X, this
// streams reads at ~5.6 TB/s, writes at ~6.9 and copies at ~6.2, where
// 2,048 workgroups walking the buffer grid-stride reach 5.2, 4.3 and 4.4).
constexpr int kProbeThreads = 256, kReadU = 8, kWriteU = 1, kCopyU = 1;

// all U loads in flight before any is used; one partial sum per wave
template <int U>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const f32x4* __restrict__ src, int64_t n4,
                                                                    float* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * kProbeThreads * U + threadIdx.x;
  f32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    v[u] = b + u * kProbeThreads < n4 ? src[b + u * kProbeThreads] : z;
  }
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) acc += (v[u][0] + v[u][1]) + (v[u][2] + v[u][3]);
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

template <int U>
__global__ __launch_bounds__(kProbeThreads) void stream_write_kernel(f32x4* __restrict__ dst, int64_t n4,
                                                                     float value) {
  const int64_t b = (int64_t)blockIdx.x * kProbeThreads * U + threadIdx.x;
  const f32x4 v = {value, value, value, value};
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (b + u * kProbeThreads < n4) dst[b + u * kProbeThreads] = v;
}

template <int U>
__global__ __launch_bounds__(kProbeThreads) void stream_copy_kernel(const f32x4* __restrict__ src,
                                                                    f32x4* __restrict__ dst, int64_t n4) {
  const int64_t b = (int64_t)blockIdx.x * kProbeThreads * U + threadIdx.x;
  f32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (b + u * kProbeThreads < n4) v[u] = src[b + u * kProbeThreads];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (b + u * kProbeThreads < n4) dst[b + u * kProbeThreads] = v[u];
}

static int64_t blocks_for(int64_t n4, int u) { return (n4 + (int64_t)kProbeThreads * u - 1) / ((int64_t)kProbeThreads * u); }

}  // namespace gpt2k

extern "C" int gpt2_stream_probe(int mode, const float* d_src, float* d_dst, int64_t n, void* stream) {
  using namespace gpt2k;
  if (n <= 0 || n % 4 || mode < 0 || mode > 2) return GPT2_ERR_ARG;
  if ((mode != 1 && !d_src) || !d_dst) return GPT2_ERR_ARG;
  if (((uintptr_t)d_src | (uintptr_t)d_dst) & 15) return GPT2_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t n4 = n / 4;
  const f32x4* src = reinterpret_cast<const f32x4*>(d_src);
  f32x4* dst = reinterpret_cast<f32x4*>(d_dst);
  if (blocks_for(n4, 1) > INT32_MAX) return GPT2_ERR_ARG;
  if (mode == 0)
    stream_read_kernel<kReadU><<<(unsigned)blocks_for(n4, kReadU), kProbeThreads, 0, s>>>(src, n4, d_dst);
  else if (mode == 1)
    stream_write_kernel<kWriteU><<<(unsigned)blocks_for(n4, kWriteU), kProbeThreads, 0, s>>>(dst, n4, 0.5f);
  else
    stream_copy_kernel<kCopyU><<<(unsigned)blocks_for(n4, kCopyU), kProbeThreads, 0, s>>>(src, dst, n4);
  return hipGetLastError() == hipSuccess ? GPT2_OK : GPT2_ERR_HIP;
}
