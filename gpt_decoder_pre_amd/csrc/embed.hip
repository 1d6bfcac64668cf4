// Token + position embedding: forward gather and deterministic backward scatter.
//
// Backward: the (id, position) pairs are sorted by id with a stable LSD radix
// sort (4-bit digits, one workgroup), so the gradient of every wte row is the
// sum of its positions' rows in position order.  The sum is split into runs of
// at most 64 sorted entries (one block each) and the runs of a segment are
// then added in order: no atomics, the same bits on every run.
#include "common.h"
#include "kernels.h"

namespace gpt2k {

__global__ void embed_fwd_kernel(const int32_t* __restrict__ idx, const float* __restrict__ wte,
                                 const float* __restrict__ wpe, float* __restrict__ x, int32_t* __restrict__ ids_out,
                                 int M, int T, int C, int vocab, int* __restrict__ err) {
  const int C4 = C >> 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * C4) return;
  const int m = (int)(i / C4), c = (int)(i % C4) * 4;
  int id = idx[m];
  if (id < 0 || id >= vocab) {
    *err = 1;
    id = 0;
  }
  if (c == 0) ids_out[m] = id;
  float a[4], b[4];
  load4(wte + (int64_t)id * C + c, a);
  load4(wpe + (int64_t)(m % T) * C + c, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] += b[e];
  store4(x + (int64_t)m * C + c, a);
}

void embed_fwd(const int32_t* idx, const float* wte, const float* wpe, float* x, int32_t* ids_out, int M, int T,
               int C, int vocab, int* err, hipStream_t s) {
  const int64_t n = (int64_t)M * (C / 4);
  embed_fwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(idx, wte, wpe, x, ids_out, M, T, C, vocab, err);
}

// Stable LSD radix sort of (key = idx[m], value = m).  Thread t owns the
// contiguous range [t*chunk, (t+1)*chunk) of the input order, which keeps the
// scatter stable.  Out-of-range ids are sorted as id 0 (the forward already
// flagged them).
__global__ __launch_bounds__(256) void radix_sort_kernel(const int32_t* __restrict__ idx, int M, int vocab,
                                                         int passes, int32_t* ka, int32_t* va, int32_t* kb,
                                                         int32_t* vb) {
  __shared__ int hist[16][256];
  __shared__ int tsum[256];
  const int t = threadIdx.x;
  const int chunk = (M + 255) / 256;
  const int lo = min(M, t * chunk), hi = min(M, lo + chunk);
  for (int pass = 0; pass < passes; ++pass) {
    // the last pass writes (ka, va)
    const bool out_b = ((passes - 1 - pass) & 1) != 0;
    const int32_t* kin = out_b ? ka : kb;
    const int32_t* vin = out_b ? va : vb;
    int32_t* kout = out_b ? kb : ka;
    int32_t* vout = out_b ? vb : va;
    const int shift = 4 * pass;
    int cnt[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) cnt[d] = 0;
    for (int i = lo; i < hi; ++i) {
      int key;
      if (pass == 0) {
        key = idx[i];
        if (key < 0 || key >= vocab) key = 0;
      } else {
        key = kin[i];
      }
      ++cnt[(key >> shift) & 15];
    }
#pragma unroll
    for (int d = 0; d < 16; ++d) hist[d][t] = cnt[d];
    __syncthreads();
    // exclusive scan in (digit, thread) order; thread t scans flat entries [16t, 16t+16)
    const int dd = t >> 4, t0 = (t & 15) * 16;
    int loc[16], s = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      loc[j] = hist[dd][t0 + j];
      s += loc[j];
    }
    tsum[t] = s;
    __syncthreads();
    if (t == 0) {
      int run = 0;
      for (int i = 0; i < 256; ++i) {
        const int v = tsum[i];
        tsum[i] = run;
        run += v;
      }
    }
    __syncthreads();
    int run = tsum[t];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      hist[dd][t0 + j] = run;
      run += loc[j];
    }
    __syncthreads();
    int off[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) off[d] = hist[d][t];
    for (int i = lo; i < hi; ++i) {
      int key, val;
      if (pass == 0) {
        key = idx[i];
        if (key < 0 || key >= vocab) key = 0;
        val = i;
      } else {
        key = kin[i];
        val = vin[i];
      }
      const int d = (key >> shift) & 15;
      const int dst = off[d]++;
      kout[dst] = key;
      vout[dst] = val;
    }
    __threadfence();
    __syncthreads();
  }
}

// The same order from one workgroup: position m and id idx[m] packed as
// (id << 16) | m are distinct words, so sorting the words (a bitonic network
// over 1024 E words, padded with all-ones words) gives the stable order by
// id.  Thread t holds the E consecutive words t E .. t E + E - 1: stages whose
// partners are less than E apart run in registers, those within a wavefront
// exchange by lane shuffles, and only the stages across wavefronts go through
// LDS with barriers.  For M <= 32768 and ids below 65535.  Workgroup b sorts
// the b-th of several independent arrays of M ids (b M .. b M + M - 1).
constexpr int kBitonicMax = 32768;
template <int E>
__global__ __launch_bounds__(1024) void bitonic_sort_kernel(const int32_t* __restrict__ idx, int M, int vocab,
                                                            int32_t* __restrict__ keys, int32_t* __restrict__ vals) {
  constexpr int N = 1024 * E;
  __shared__ uint32_t w[N];
  const int t = threadIdx.x;
  idx += (int64_t)blockIdx.x * M;
  keys += (int64_t)blockIdx.x * M;
  vals += (int64_t)blockIdx.x * M;
  uint32_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = t * E + e;
    if (i < M) {
      int key = idx[i];
      if (key < 0 || key >= vocab) key = 0;
      x[e] = ((uint32_t)key << 16) | (uint32_t)i;
    } else {
      x[e] = 0xffffffffu;
    }
  }
  for (int k = 2; k <= N; k <<= 1) {
    // partners j >= E apart: in another thread
    for (int j = k >> 1; j >= E; j >>= 1) {
      const int m = j / E;  // partner thread = t ^ m
      const bool low = (t & m) == 0;
      if (m < 64) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t y = (uint32_t)__shfl_xor((int)x[e], m, 64);
          const bool asc = ((t * E + e) & k) == 0;
          x[e] = (asc == low) ? min(x[e], y) : max(x[e], y);
        }
      } else {
        __syncthreads();  // the previous exchange's reads are done
#pragma unroll
        for (int e = 0; e < E; ++e) w[t * E + e] = x[e];
        __syncthreads();
        const int p = t ^ m;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t y = w[p * E + e];
          const bool asc = ((t * E + e) & k) == 0;
          x[e] = (asc == low) ? min(x[e], y) : max(x[e], y);
        }
      }
    }
    // partners j < E apart: in this thread's registers
#pragma unroll
    for (int j = E / 2; j > 0; j >>= 1) {
      if (j < k) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & j) == 0) {
            const bool asc = ((t * E + e) & k) == 0;
            const uint32_t a = x[e], b = x[e | j];
            if ((a > b) == asc) {
              x[e] = b;
              x[e | j] = a;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = t * E + e;
    if (i < M) {
      keys[i] = (int32_t)(x[e] >> 16);
      vals[i] = (int32_t)(x[e] & 0xffffu);
    }
  }
}

bool embed_sort_batch(const int32_t* idx, int M, int nb, int vocab, int32_t* keys, int32_t* vals, hipStream_t s) {
  if (M > kBitonicMax || vocab >= 65535 || nb < 1) return false;
  const int e = (M + 1023) / 1024;
#define GPT2_BITONIC(E) bitonic_sort_kernel<E><<<nb, 1024, 0, s>>>(idx, M, vocab, keys, vals)
  if (e <= 1) GPT2_BITONIC(1);
  else if (e <= 2) GPT2_BITONIC(2);
  else if (e <= 4) GPT2_BITONIC(4);
  else if (e <= 8) GPT2_BITONIC(8);
  else if (e <= 16) GPT2_BITONIC(16);
  else GPT2_BITONIC(32);
#undef GPT2_BITONIC
  return true;
}

void embed_sort(const int32_t* idx, int M, int vocab, int id_bits, int32_t* keys_a, int32_t* vals_a,
                int32_t* keys_b, int32_t* vals_b, hipStream_t s) {
  if (M <= kBitonicMax && vocab < 65535) {
    const int e = (M + 1023) / 1024;  // words per thread, rounded up to a power of two
#define GPT2_BITONIC(E) bitonic_sort_kernel<E><<<1, 1024, 0, s>>>(idx, M, vocab, keys_a, vals_a)
    if (e <= 1) GPT2_BITONIC(1);
    else if (e <= 2) GPT2_BITONIC(2);
    else if (e <= 4) GPT2_BITONIC(4);
    else if (e <= 8) GPT2_BITONIC(8);
    else if (e <= 16) GPT2_BITONIC(16);
    else GPT2_BITONIC(32);
#undef GPT2_BITONIC
    return;
  }
  const int passes = (id_bits + 3) / 4;
  radix_sort_kernel<<<1, 256, 0, s>>>(idx, M, vocab, passes, keys_a, vals_a, keys_b, vals_b);
}

constexpr int kRun = 64;

// Runs: within each chunk of 64 sorted entries, consecutive equal ids form a run;
// the run's row sum is stored at the index of its first entry.  The rows go
// out eight at a time (their loads in flight together) and are added in
// sorted order.
__global__ __launch_bounds__(256) void run_sum_kernel(const int32_t* __restrict__ sid,
                                                      const int32_t* __restrict__ spos,
                                                      const float* __restrict__ dx, float* __restrict__ runs,
                                                      int M, int C) {
  constexpr int U = 8;
  const int base = blockIdx.x * kRun, end = min(M, base + kRun);
  const int C4 = C >> 2;
  for (int c4 = threadIdx.x; c4 < C4; c4 += blockDim.x) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int start = base;
    for (int i0 = base; i0 < end; i0 += U) {
      float v[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u < end) load4(dx + (int64_t)spos[i0 + u] * C + 4 * c4, v[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u;
        if (i >= end) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += v[u][e];
        if (i + 1 == end || sid[i + 1] != sid[i]) {
          store4(runs + (int64_t)start * C + 4 * c4, acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = 0.f;
          start = i + 1;
        }
      }
    }
  }
}

// One wavefront per sorted entry; entries that start a segment add the
// segment's runs (in order) into their wte row.  A lane takes up to three
// 4-column groups at once and the runs of a long segment come eight at a
// time, so that a frequent token's row costs a few round trips to memory
// instead of one per run; the additions keep the run order.
__global__ __launch_bounds__(256) void segment_add_kernel(const int32_t* __restrict__ sid,
                                                          const float* __restrict__ runs, float* __restrict__ dwte,
                                                          int M, int C) {
  constexpr int U = 8, NB = 3;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= M) return;
  const int id = sid[i];
  if (i > 0 && sid[i - 1] == id) return;
  const int C4 = C >> 2;
  for (int cb = 0; cb < C4; cb += 64 * NB) {
    float s[NB][4];
    bool col[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c4 = cb + b * 64 + lane;
      col[b] = c4 < C4;
      if (col[b]) load4(runs + (int64_t)i * C + 4 * c4, s[b]);
    }
    // the segment's later runs (the first entry of each later chunk)
    int j = (i / kRun + 1) * kRun;
    while (j < M && sid[j] == id) {
      float v[U][NB][4];
      bool in[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jj = j + u * kRun;
        in[u] = jj < M && sid[jj] == id && (u == 0 || in[u - 1]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (in[u] && col[b]) load4(runs + (int64_t)jj * C + 4 * (cb + b * 64 + lane), v[u][b]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (in[u]) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            if (col[b]) {
#pragma unroll
              for (int e = 0; e < 4; ++e) s[b][e] += v[u][b][e];
            }
        }
      j += U * kRun;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (col[b]) {
        float* o = dwte + (int64_t)id * C + 4 * (cb + b * 64 + lane);
        float a4[4];
        load4(o, a4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] += s[b][e];
        store4(o, a4);
      }
  }
}

void embed_scatter(const int32_t* sorted_ids, const int32_t* sorted_pos, const float* dx, float* run_sums,
                   float* dwte, int M, int C, hipStream_t s) {
  run_sum_kernel<<<(M + kRun - 1) / kRun, 256, 0, s>>>(sorted_ids, sorted_pos, dx, run_sums, M, C);
  segment_add_kernel<<<(M + 3) / 4, 256, 0, s>>>(sorted_ids, run_sums, dwte, M, C);
}

__global__ void wpe_grad_kernel(const float* __restrict__ dx, float* __restrict__ dwpe, int B, int T, int C) {
  const int C4 = C >> 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * C4) return;
  const int t = (int)(i / C4), c = (int)(i % C4) * 4;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < B; ++b) {
    float v[4];
    load4(dx + ((int64_t)b * T + t) * C + c, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += v[e];
  }
  float* o = dwpe + (int64_t)t * C + c;
  float a[4];
  load4(o, a);
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] += s[e];
  store4(o, a);
}

void embed_wpe_grad(const float* dx, float* dwpe, int B, int T, int C, hipStream_t s) {
  const int64_t n = (int64_t)T * (C / 4);
  wpe_grad_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dx, dwpe, B, T, C);
}

}  // namespace gpt2k
