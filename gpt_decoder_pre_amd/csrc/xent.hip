// Softmax cross-entropy over the padded vocabulary, fused with its gradient.
//
// One workgroup per row of logits.  The row's max and sum of exponentials are
// combined across the block (fp32 even for bf16 logits) into its
// log-sum-exp, and the logits are overwritten with
// (softmax - onehot(target)) * grad_scale.  bf16 rows stay in registers
// between the two uses (one HBM read, one write); other rows are read twice.
#include "common.h"
#include "kernels.h"

namespace gpt2k {

// General path (any V): two passes over the row.
template <typename TA, int VEC>
__global__ __launch_bounds__(256) void xent_kernel(TA* __restrict__ logits, const int32_t* __restrict__ targets,
                                                   float* __restrict__ row_loss, int V, int vocab,
                                                   float grad_scale, int* __restrict__ err) {
  __shared__ float red[16];
  __shared__ float red2[16];
  const int row = blockIdx.x;
  TA* z = logits + (int64_t)row * V;
  int y = targets[row];
  if (y < 0 || y >= vocab) {
    if (threadIdx.x == 0) *err = 1;
    y = 0;
  }
  float m = -INFINITY, s = 0.f;
  const int nv = V / VEC;
  for (int i = threadIdx.x; i < nv; i += blockDim.x) {
    float v[VEC];
    if constexpr (VEC == 8) {
      load4(z + i * 8, v);
      load4(z + i * 8 + 4, v + 4);
    } else {
      v[0] = to_f32(z[i]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (v[e] > m) {
        s = s * exp_fast(m - v[e]) + 1.f;
        m = v[e];
      } else {
        s += exp_fast(v[e] - m);
      }
    }
  }
  const float M = block_max(m, red);
  const float S = block_sum(m == -INFINITY ? 0.f : s * exp_fast(m - M), red2);
  const float lse = M + logf(S);
  const float zy = to_f32(z[y]);
  if (threadIdx.x == 0) row_loss[row] = lse - zy;
  __syncthreads();
  for (int i = threadIdx.x; i < nv; i += blockDim.x) {
    float v[VEC];
    if constexpr (VEC == 8) {
      load4(z + i * 8, v);
      load4(z + i * 8 + 4, v + 4);
    } else {
      v[0] = to_f32(z[i]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int col = i * VEC + e;
      v[e] = (exp_fast(v[e] - lse) - (col == y ? 1.f : 0.f)) * grad_scale;
    }
    if constexpr (VEC == 8) {
      store4(z + i * 8, v);
      store4(z + i * 8 + 4, v + 4);
    } else {
      z[i] = from_f32<TA>(v[0]);
    }
  }
}

// bf16 rows of up to NT x NCH x 8 elements: the row is read once into
// registers (16-byte chunks, NCH per thread), the statistics come from the
// registers, and the gradient is written from them: one read, one write.
// The register budget (64 VGPRs) keeps two rows resident per CU, so one row's
// loads overlap the other's arithmetic and stores.
template <int NCH, int NT>
__global__ __launch_bounds__(NT, 8 * NT / 1024) void xent_bf16_resident_kernel(h16* __restrict__ logits,
                                                                 const int32_t* __restrict__ targets,
                                                                 float* __restrict__ row_loss, int V, int vocab,
                                                                 float grad_scale, int* __restrict__ err) {
  __shared__ float red[16];
  __shared__ float red2[16];
  const int row = blockIdx.x;
  h16* z = logits + (int64_t)row * V;
  int y = targets[row];
  if (y < 0 || y >= vocab) {
    if (threadIdx.x == 0) *err = 1;
    y = 0;
  }
  const int nchunk = V / 8;
  u32x4 r[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + i * NT;
    r[i] = ld16_or_zero(z + 8 * c, c < nchunk);
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nchunk) {
      const h16x8 v = __builtin_bit_cast(h16x8, r[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, (float)v[e]);
    }
  }
  const float M = block_max(m, red);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nchunk) {
      const h16x8 v = __builtin_bit_cast(h16x8, r[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += exp2_fast(((float)v[e] - M) * kLog2e);
    }
  }
  const float S = block_sum(s, red2);
  const float lse = M + logf(S);
  if (threadIdx.x == (y / 8) % NT) {
    float zy = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (i == (y / 8) / NT) {
        const h16x8 v = __builtin_bit_cast(h16x8, r[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e == y % 8) zy = (float)v[e];
      }
    }
    row_loss[row] = lse - zy;
  }
  const float l2 = lse * kLog2e;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nchunk) {
      const h16x8 v = __builtin_bit_cast(h16x8, r[i]);
      h16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2_fast((float)v[e] * kLog2e - l2);
        o[e] = (h16)((p - (8 * c + e == y ? 1.f : 0.f)) * grad_scale);
      }
      *reinterpret_cast<h16x8*>(z + 8 * c) = o;
    }
  }
}

template <typename TA>
void xent_fwd_bwd(TA* logits, const int32_t* targets, float* row_loss, int M, int V, int vocab, float grad_scale,
                  int* err, hipStream_t s) {
  if constexpr (sizeof(TA) == 2) {
    if (V % 8 == 0 && V <= 1024 * 8 * 8) {
      const int nch = (V / 8 + 1023) / 1024;
      if (nch <= 2) {
        xent_bf16_resident_kernel<2, 1024><<<M, 1024, 0, s>>>(logits, targets, row_loss, V, vocab, grad_scale, err);
      } else if (nch <= 4) {
        xent_bf16_resident_kernel<4, 1024><<<M, 1024, 0, s>>>(logits, targets, row_loss, V, vocab, grad_scale, err);
      } else if (nch <= 7) {
        xent_bf16_resident_kernel<7, 1024><<<M, 1024, 0, s>>>(logits, targets, row_loss, V, vocab, grad_scale, err);
      } else {
        xent_bf16_resident_kernel<8, 1024><<<M, 1024, 0, s>>>(logits, targets, row_loss, V, vocab, grad_scale, err);
      }
      return;
    }
  }
  if (V % 8 == 0) xent_kernel<TA, 8><<<M, 256, 0, s>>>(logits, targets, row_loss, V, vocab, grad_scale, err);
  else xent_kernel<TA, 1><<<M, 256, 0, s>>>(logits, targets, row_loss, V, vocab, grad_scale, err);
}
template void xent_fwd_bwd<float>(float*, const int32_t*, float*, int, int, int, float, int*, hipStream_t);
template void xent_fwd_bwd<h16>(h16*, const int32_t*, float*, int, int, int, float, int*, hipStream_t);

__global__ __launch_bounds__(1024) void loss_reduce_kernel(const float* __restrict__ row_loss, int M, float scale,
                                                           int accumulate, float* out) {
  __shared__ double red[16];
  // four independent partial sums per thread (loads in flight together),
  // combined in a fixed order
  double s4[4] = {0.0, 0.0, 0.0, 0.0};
  const int step = 4 * blockDim.x;
  int i = threadIdx.x;
  for (; i + 3 * (int)blockDim.x < M; i += step) {
#pragma unroll
    for (int u = 0; u < 4; ++u) s4[u] += (double)row_loss[i + u * blockDim.x];
  }
  for (int u = 0; i < M; i += blockDim.x, ++u) s4[u] += (double)row_loss[i];
  double s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  s = block_sum(s, red);
  if (threadIdx.x == 0) {
    const float v = (float)(s * (double)scale);
    *out = accumulate ? *out + v : v;
  }
}

void loss_reduce(const float* row_loss, int M, float scale, bool accumulate, float* out, hipStream_t s) {
  loss_reduce_kernel<<<1, 1024, 0, s>>>(row_loss, M, scale, accumulate ? 1 : 0, out);
}

}  // namespace gpt2k
