// LayerNorm forward / backward and column-sum reductions (HBM-bound).
//
// Rows stay in registers (up to C = 2048): the forward takes one or two rows
// per wavefront in chunks of eight values, the backward one row per
// wavefront in float4s; mean and variance are wavefront-shuffle reductions,
// biased variance, eps = 1e-5.  Column sums (gain / shift / bias gradients) are
// deterministic: fixed row chunks per block write partial rows, a second
// kernel adds the partials in chunk order.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gpt2k {

// Eight consecutive values of a row: two float4 loads; eight outputs in one
// 16-byte store (bf16) or two (fp32).
DEVI void store8(float* p, const float o[8]) {
  store4(p, o);
  store4(p + 4, o + 4);
}
DEVI void store8(h16* p, const float o[8]) {
  h16x8 t;
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (h16)o[e];
  *reinterpret_cast<h16x8*>(p) = t;
}

// Each wavefront normalises R rows together (their loads in flight at once,
// their shuffle reductions interleaved), the rows in registers.  The R rows
// are taken end to end as R C / 8 chunks of eight values; lane l holds
// chunks l, l + 64, ..., NP of them, so every lane reads 32 bytes and writes
// one 16-byte bf16 group per chunk.  C % 8 == 0.
template <typename TA, int NP, int R>
__global__ __launch_bounds__(256) void ln_fwd_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ b, TA* __restrict__ y,
                                                     float* __restrict__ mean, float* __restrict__ rstd, int M,
                                                     int C) {
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  const int P = C >> 3;  // chunks per row
  float v[NP][8];
  int rk[NP];  // which of the R rows chunk k belongs to (-1: past them)
  float mu[R], rs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) mu[r] = 0.f;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int p = lane + 64 * k;
    const int r = p / P;
    rk[k] = p < R * P ? r : -1;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[k][e] = 0.f;
    if (rk[k] >= 0) {
      const float* xr = x + (int64_t)min(row0 + r, M - 1) * C + 8 * (p - r * P);
      load4(xr, v[k]);
      load4(xr + 4, v[k] + 4);
      const float t = ((v[k][0] + v[k][1]) + (v[k][2] + v[k][3])) + ((v[k][4] + v[k][5]) + (v[k][6] + v[k][7]));
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
        if (rr == r) mu[rr] += t;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    mu[r] = wave_sum(mu[r]) / (float)C;
    rs[r] = 0.f;
  }
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    if (rk[k] >= 0) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
        if (rr == rk[k]) {
          float q = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float d = v[k][e] - mu[rr];
            q += d * d;
          }
          rs[rr] += q;
        }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) rs[r] = 1.0f / sqrtf(wave_sum(rs[r]) / (float)C + kLnEps);
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int r = rk[k];
    if (r >= 0 && row0 + r < M) {
      const int c = 8 * (lane + 64 * k - r * P);
      float ww[8], bb[8], o[8];
      load4(w + c, ww);
      load4(w + c + 4, ww + 4);
      load4(b + c, bb);
      load4(b + c + 4, bb + 4);
      float m = mu[0], sd = rs[0];
#pragma unroll
      for (int rr = 1; rr < R; ++rr)
        if (rr == r) m = mu[rr], sd = rs[rr];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[k][e] - m) * sd * ww[e] + bb[e];
      store8(y + (int64_t)(row0 + r) * C + c, o);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (row0 + r < M) {
        mean[row0 + r] = mu[r];
        rstd[row0 + r] = rs[r];
      }
    }
  }
}

template <typename TA>
void layernorm_fwd(const float* x, const float* w, const float* b, TA* y, float* mean, float* rstd, int M,
                   int C, hipStream_t s) {
  // two rows per wavefront up to C = 1024, one beyond (register budget);
  // NP = chunks of eight per lane over those rows
#define GPT2_LN_FWD(NP, R) ln_fwd_kernel<TA, NP, R><<<(M + 4 * R - 1) / (4 * R), 256, 0, s>>>(x, w, b, y, mean, rstd, M, C)
  const int R = C <= 1024 ? 2 : 1;
  switch ((R * (C / 8) + 63) / 64) {
    case 1: if (R == 2) GPT2_LN_FWD(1, 2); else GPT2_LN_FWD(1, 1); break;
    case 2: if (R == 2) GPT2_LN_FWD(2, 2); else GPT2_LN_FWD(2, 1); break;
    case 3: if (R == 2) GPT2_LN_FWD(3, 2); else GPT2_LN_FWD(3, 1); break;
    case 4: if (R == 2) GPT2_LN_FWD(4, 2); else GPT2_LN_FWD(4, 1); break;
    default: GPT2_LN_FWD(4, 1); break;  // C <= 2048
  }
#undef GPT2_LN_FWD
}
template void layernorm_fwd<float>(const float*, const float*, const float*, float*, float*, float*, int, int,
                                   hipStream_t);
template void layernorm_fwd<h16>(const float*, const float*, const float*, h16*, float*, float*, int, int,
                                  hipStream_t);

// dx = rstd (dxhat - mean(dxhat) - xhat mean(dxhat xhat)), dxhat = dy w.
//
// A block of W wavefronts owns rows_per_block consecutive rows; each
// wavefront takes every W-th of them.  For rows of up to 768 columns W = 8 at
// no more than 128 VGPRs, so two blocks (four rows per SIMD) are resident and
// their row loads overlap; wider rows need more registers and use W = 4.  The
// per-wavefront column sums (gain, shift, residual gradient) are combined by
// a fixed pairwise tree in LDS, then written as the block's partial row.
template <int NV> constexpr int ln_bwd_waves() { return NV <= 3 ? 8 : 4; }

template <typename TA, int NV>
struct LnBwdRow {
  float g[NV][4], xv[NV][4], o[NV][4];
  float mu, rs;
  DEVI void load(const TA* dy, const float* x, const float* dres, int dres_in, const float* mean,
                 const float* rstd, int row, int lane, int C) {
    const int C4 = C >> 2;
    mu = mean[row];
    rs = rstd[row];
    const TA* dyr = dy + (int64_t)row * C;
    const float* xr = x + (int64_t)row * C;
    const float* dr = dres + (int64_t)row * C;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c4 = lane + i * 64;
#pragma unroll
      for (int e = 0; e < 4; ++e) g[i][e] = xv[i][e] = o[i][e] = 0.f;
      if (c4 < C4) {
        load4(dyr + 4 * c4, g[i]);
        load4(xr + 4 * c4, xv[i]);
        if (dres_in) load4(dr + 4 * c4, o[i]);
      }
    }
  }
};

template <typename TA, int NV, int W = ln_bwd_waves<NV>()>
__global__ __launch_bounds__(64 * W, W == 8 ? 4 : 1) void ln_bwd_kernel(
    const TA* __restrict__ dy, const float* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const float* __restrict__ w, float* __restrict__ dres, int dres_in,
    TA* __restrict__ dres_act, float* __restrict__ part, int M, int C, int rows_per_block, int chunks) {
  __shared__ float red[W / 2][3][NV * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C4 = C >> 2;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(M, r0 + rows_per_block);
  float aw[NV][4], ab[NV][4], ar[NV][4], ww[NV][4];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c4 = lane + i * 64;
#pragma unroll
    for (int e = 0; e < 4; ++e) aw[i][e] = ab[i][e] = ar[i][e] = ww[i][e] = 0.f;
    if (c4 < C4) load4(w + 4 * c4, ww[i]);
  }
  for (int row = r0 + wave; row < r1; row += W) {
    LnBwdRow<TA, NV> cur;
    cur.load(dy, x, dres, dres_in, mean, rstd, row, lane, C);
    float xh[NV][4];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xh[i][e] = (cur.xv[i][e] - cur.mu) * cur.rs;
        const float d = cur.g[i][e] * ww[i][e];
        s1 += d;
        s2 += d * xh[i][e];
        aw[i][e] += cur.g[i][e] * xh[i][e];
        ab[i][e] += cur.g[i][e];
      }
    }
    const float m1 = wave_sum(s1) / (float)C, m2 = wave_sum(s2) / (float)C;
    float* dr = dres + (int64_t)row * C;
    TA* da = dres_act + (int64_t)row * C;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c4 = lane + i * 64;
      if (c4 < C4) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = cur.o[i][e] + cur.rs * (cur.g[i][e] * ww[i][e] - m1 - xh[i][e] * m2);
          ar[i][e] += o[e];
        }
        store4(dr + 4 * c4, o);
        store4(da + 4 * c4, o);
      }
    }
  }
  // fixed pairwise tree: wave w += wave w + h for h = W/2, ..., 2, 1
#pragma unroll
  for (int h = W / 2; h >= 1; h >>= 1) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 4 * (lane + i * 64) + e;
          red[wave - h][0][c] = aw[i][e];
          red[wave - h][1][c] = ab[i][e];
          red[wave - h][2][c] = ar[i][e];
        }
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 4 * (lane + i * 64) + e;
          aw[i][e] += red[wave][0][c];
          ab[i][e] += red[wave][1][c];
          ar[i][e] += red[wave][2][c];
        }
    }
    __syncthreads();
  }
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c4 = lane + i * 64;
      if (c4 < C4) {
        store4(part + ((int64_t)0 * chunks + blockIdx.x) * C + 4 * c4, aw[i]);
        store4(part + ((int64_t)1 * chunks + blockIdx.x) * C + 4 * c4, ab[i]);
        store4(part + ((int64_t)2 * chunks + blockIdx.x) * C + 4 * c4, ar[i]);
      }
    }
  }
}

template <typename TA>
int layernorm_bwd(const TA* dy, const float* x, const float* mean, const float* rstd, const float* w,
                  float* dres, bool dres_in, TA* dres_act, float* part, int M, int C, hipStream_t s) {
  const int rpb = 32;
  const int chunks = (M + rpb - 1) / rpb;
#define GPT2_LN_BWD(NV)                                                                          \
  ln_bwd_kernel<TA, NV><<<chunks, 64 * ln_bwd_waves<NV>(), 0, s>>>(dy, x, mean, rstd, w, dres, dres_in ? 1 : 0, \
                                                                   dres_act, part, M, C, rpb, chunks)
  switch ((C / 4 + 63) / 64) {
    case 1: GPT2_LN_BWD(1); break;
    case 2: GPT2_LN_BWD(2); break;
    case 3: GPT2_LN_BWD(3); break;
    case 4: GPT2_LN_BWD(4); break;
    case 5: GPT2_LN_BWD(5); break;
    case 6: GPT2_LN_BWD(6); break;
    case 7: GPT2_LN_BWD(7); break;
    default: GPT2_LN_BWD(8); break;
  }
#undef GPT2_LN_BWD
  return chunks;
}
template int layernorm_bwd<float>(const float*, const float*, const float*, const float*, const float*, float*,
                                  bool, float*, float*, int, int, hipStream_t);
template int layernorm_bwd<h16>(const h16*, const float*, const float*, const float*, const float*, float*,
                                 bool, h16*, float*, int, int, hipStream_t);

// Many column-partial reductions in one launch: block b belongs to the job j
// with jobs.first[j] <= b < jobs.first[j + 1] and reduces 256 of that job's
// columns, four per lane (16-byte accesses).  Each of 16 lane groups adds
// every 16th chunk in chunk order, then the groups are added in order: a
// fixed order for every column.
__global__ __launch_bounds__(1024) void colpart_reduce_batch_kernel(ColJobs jobs) {
  __shared__ f32x4 red[16][64];
  int j = 0;
  while (j + 1 < jobs.n && (int)blockIdx.x >= jobs.first[j + 1]) ++j;
  const ColJob& job = jobs.job[j];
  const int local = blockIdx.x - jobs.first[j];
  const int cblocks = (job.N + 255) / 256;  // 256 columns per block, four per lane
  const int k = local / cblocks;
  float* out = job.out[k];
  const int col = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int n = (local % cblocks) * 256 + 4 * col;
  const float* p = job.part + (int64_t)k * job.chunks * job.N;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  if (n < job.N) {
#pragma unroll 8
    for (int c = grp; c < job.chunks; c += 16) sum += *reinterpret_cast<const f32x4*>(p + (int64_t)c * job.N + n);
  }
  red[grp][col] = sum;
  __syncthreads();
  if (grp == 0 && n < job.N) {
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 16; ++g) t += red[g][col];
    f32x4* o = reinterpret_cast<f32x4*>(out + n);
    *o += t;
  }
}

void colpart_reduce_batch(const ColJob* jobs, int n, hipStream_t s) {
  for (int j0 = 0; j0 < n; j0 += kColJobsMax) {
    ColJobs b;
    b.n = std::min(kColJobsMax, n - j0);
    int blocks = 0;
    for (int j = 0; j < b.n; ++j) {
      b.job[j] = jobs[j0 + j];
      b.first[j] = blocks;
      blocks += (b.job[j].N + 255) / 256 * b.job[j].nout;
    }
    colpart_reduce_batch_kernel<<<blocks, 1024, 0, s>>>(b);
  }
}

// Partial column sums: block `chunk` covers rows_per_chunk rows and all N
// columns; each lane owns W = 16 bytes of consecutive columns (one 16-byte
// load per row, eight rows in flight) and loops over column groups if the row
// is wider than the block.
template <typename TA>
__global__ __launch_bounds__(1024) void colsum_kernel(const TA* __restrict__ x, int M, int N, int rows_per_chunk,
                                                      float* __restrict__ part) {
  constexpr int W = 16 / sizeof(TA);
  const int r0 = blockIdx.x * rows_per_chunk, r1 = min(M, r0 + rows_per_chunk);
  for (int c = threadIdx.x * W; c < N; c += blockDim.x * W) {
    float s[W];
#pragma unroll
    for (int e = 0; e < W; ++e) s[e] = 0.f;
    int r = r0;
    for (; r + 8 <= r1; r += 8) {
      u32x4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const u32x4*>(x + (int64_t)(r + k) * N + c);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float f[W];
        unpack16<TA>(v[k], f);
#pragma unroll
        for (int e = 0; e < W; ++e) s[e] += f[e];
      }
    }
    for (; r < r1; ++r) {
      float f[W];
      unpack16<TA>(*reinterpret_cast<const u32x4*>(x + (int64_t)r * N + c), f);
#pragma unroll
      for (int e = 0; e < W; ++e) s[e] += f[e];
    }
#pragma unroll
    for (int e = 0; e < W; e += 4) store4(part + (int64_t)blockIdx.x * N + c + e, s + e);
  }
}

template <typename TA>
int colsum_partials(const TA* x, int M, int N, float* part, hipStream_t s) {
  constexpr int W = 16 / sizeof(TA);
  const int rpc = 64;
  const int chunks = (M + rpc - 1) / rpc;
  const int groups = N / W;
  const int threads = std::min(1024, (groups + 63) / 64 * 64);
  colsum_kernel<TA><<<chunks, threads, 0, s>>>(x, M, N, rpc, part);
  return chunks;
}
template int colsum_partials<float>(const float*, int, int, float*, hipStream_t);
template int colsum_partials<h16>(const h16*, int, int, float*, hipStream_t);

}  // namespace gpt2k
