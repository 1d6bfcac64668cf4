// Causal multi-head attention, forward and backward.
//
// bf16 path (head dim 64): flash attention on v_mfma_f32_32x32x16_bf16.  A
// workgroup owns 128 queries (four waves of 32); keys and values stream
// through LDS in tiles of 64.  Scores are computed transposed, S^T = K Q^T,
// so that every lane owns one query: the online-softmax statistics (running
// max and sum, in the exp2 domain) are per-lane registers, and a row max needs
// a single exchange with the lane 32 apart.  The probabilities are fed back
// to the MFMA as the B operand of O^T = V^T P^T with the key order permuted
// to match the accumulator layout (the contraction order is free), so P never
// leaves registers; V is stored transposed in LDS for that product.
// Backward recomputes P from the saved log-sum-exp: one kernel per query tile
// computes D = rowsum(dO o O) (stored with the log-sum-exp in the exp2 domain
// for the next kernel) and accumulates dQ over key tiles, then one per key
// tile accumulates dK and dV over query tiles (no atomics).
//
// fp32 path: one wavefront per query (forward, dQ) or key (dK, dV) row with the
// scores of the row in LDS; plain fp32 arithmetic for the exact-mode step.
#include <type_traits>

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds_tile.h"

namespace gpt2k {

constexpr int HD = 64;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

DEVI h16x8 as_h16x8(u32x4 v) { return __builtin_bit_cast(h16x8, v); }

DEVI h16x8 pack8(const f32x16& v, int base) {
  h16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (h16)v[base + e];
  return r;
}

// ------------------------------------------------------------------ forward ----
// Workgroup: 128 queries of one (sequence, head); wave w owns queries
// q0 + 32 w + lane%32.  K and V tiles of 64 keys go from HBM straight to LDS
// (global_load_lds), two stages deep, and the loop runs two tiles per trip so
// that the stage offsets are compile-time constants.  Each tile in turn:
// scores, softmax on the vector ALUs, and the probabilities feed the V
// product from registers.  At 120 VGPRs and 32 KB of LDS four workgroups
// share a CU, and their waves overlap one another's MFMA and softmax phases
// (measured on MI355X: 4-7% faster than three workgroups of a form that
// multiplied tile j+1's scores during tile j's softmax, with the same results).
//
// Softmax in the exp2 domain with a lazily updated running max: the max m is
// raised only when a tile's max exceeds it by more than kLazy (then o and l
// are rescaled), so exponents stay below 2^kLazy and most tiles skip the
// rescale.  The result is the same up to rounding: o and l share the factor.

constexpr int ATILE = 64 * 64;     // one 64 x 64 bf16 tile, swizzled, unpadded
constexpr int ASTAGE = 2 * ATILE;  // K | V (or Q | dO)
constexpr float kLazy = 8.0f;

// Every attention tile (64 rows of one head: keys or queries by 64 dims,
// 128 bytes a row) is read both row-wise (ds_read_b128: eight dims of one row
// per lane, 16 consecutive rows per 256-byte slice) and transposed
// (ds_read_b64_tr_b16: four consecutive rows of one dim column).  Chunk c of
// row r is stored at chunk c ^ bswz(r), bswz(r) = 4 r1 + 2 r2 + r3 (r_i the
// bits of r): a bijection over bits 1..3 spreads the row-wise slices over all
// banks, and rows r and r + 2 land in opposite chunk halves, which spreads the
// transposed reads.
DEVI int bswz(int r) { return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1); }

// This wave's two 1 KB loads of a tile (rows r0.. of a [T][ld] matrix).  The
// per-lane byte offsets within a tile do not depend on r0, so they are formed
// once; a tile adds the wave-uniform r0 * ld to the scalar base.  Rows past T
// (only in a partial last tile) are clamped to T - 1.
struct AttnTileLoader {
  uint32_t off[2];  // lane byte offsets of the two loads, relative to row r0
  int64_t ld;       // row stride of the source (elements)
  DEVI static void place(int wave, int lane, int j, int& r, int& c8) {
    const int byte = (2 * wave + j) * 1024 + lane * 16;
    r = byte >> 7;
    c8 = 8 * (((byte >> 4) & 7) ^ bswz(r));
  }
  DEVI void init(int64_t ld_, int wave, int lane) {
    ld = ld_;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int r, c8;
      place(wave, lane, j, r, c8);
      off[j] = (uint32_t)(2 * ((int64_t)r * ld + c8));
    }
  }
  DEVI void issue(const h16* g, int r0, int T, uint32_t lds_tile, int wave, int lane) const {
    if (r0 + 64 <= T) {
      const h16* b = uniform_ptr(g + (int64_t)r0 * ld);
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16s(b, off[j], lds_tile + (2 * wave + j) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int r, c8;
        place(wave, lane, j, r, c8);
        dma16(g + (int64_t)min(r0 + r, T - 1) * ld + c8, lds_tile + (2 * wave + j) * 1024);
      }
    }
  }
};

// MFMA operand rows row0 + lane%32 of a tile, dims 16 kk + 8 hl .. + 7.
DEVI h16x8 row_frag(const h16* tile, int row0, int kk, int lane) {
  const int r = row0 + (lane & 31);
  const int c = 2 * kk + (lane >> 5);
  return *reinterpret_cast<const h16x8*>(tile + r * 64 + 8 * (c ^ bswz(r)));
}

// A operand of a product over the tile's rows, read transposed: rows
// (dims) mbase + lane%32, and the eight tile rows of the 16-row step kbase in
// the order the score accumulators hold them: kbase + 4 hl + {0..3} and
// kbase + 8 + 4 hl + {0..3}.  ds_read_b64_tr_b16 hands lane j of each 16-lane
// group element i of source lane 4i + j/4's 8-byte row, so source lane 4i + q
// points at (row kb + i, dims m16 + 4q .. + 3).
DEVI h16x8 tr_frag_keys(const h16* tile, int kbase, int mbase, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int k = kbase + 4 * (g >> 1) + (s >> 2);
  const int m = mbase + 16 * (g & 1) + 4 * (s & 3);
  const int c = m >> 3, o = m & 7;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + k * 64 + 8 * (c ^ bswz(k)) + o));
  const i16x4 b =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + (k + 8) * 64 + 8 * (c ^ bswz(k + 8)) + o));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  u32x4 r = {ua[0], ua[1], ub[0], ub[1]};
  return as_h16x8(r);
}

// acc + the sum of eight 16-bit values (four dot2 against ones)
DEVI float sum_h16x8(h16x8 v, float acc) {
  const h16x2 one = {(h16)1.0f, (h16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const h16x2 pair = {v[2 * e], v[2 * e + 1]};
    acc = dot2(pair, one, acc);
  }
  return acc;
}

// Block -> (tile index within the head, head, sequence).  Causal tiles carry
// very different work (the first key tile of a head sees every query tile,
// the last one a single one), so the tile index is the slowest-varying part
// of the block index: every head's longest tile is dispatched first, then
// every head's second longest, and so on.  Taken in this order, greedy
// dispatch leaves a short tail; head by head, a long tile dispatched near
// the end would run alone (about a third longer in all).  Workgroups go to
// the eight XCDs round-robin in launch order, so when B NH is a multiple of 8
// every tile of a head runs on the same XCD and shares its L2 (the tiles
// re-read the same K and V, or Q and dO).
DEVI void attn_block(int T, int NH, int& tile, int& h, int& b) {
  const int nq = (T + 127) / 128;
  const int bh_count = gridDim.x / nq;
  tile = blockIdx.x / bh_count;
  const int bh = blockIdx.x - tile * bh_count;
  h = bh % NH;
  b = bh / NH;
}

// qkv bias gradient partials from a backward kernel's stored outputs (T a
// multiple of 64).  Each wave holds a 64-dim x 32-token block (acc[t][r]:
// dim 32 t + 8 (r/4) + 4 hl + r%4, token lane%32) of bf16-rounded values;
// the block's four waves write theirs to LDS, then thread (c, d) of the
// first 128 adds dim d over the 64 tokens of chunk c (waves 2c and 2c + 1,
// tokens ascending) into out[chunk][d], out = colsum + column offset.  The
// caller has synchronised so that red may be overwritten.
DEVI void chunk_colsums(const f32x16 (&acc)[2], float scale, bool tok_ok, float* red, float* out, int64_t chunk0,
                        int64_t ldo, int tok0, int T) {
  const int tid = threadIdx.x, lane = tid & 63, lc = lane & 31, hl = lane >> 5, wave = tid >> 6;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = t * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
      red[(wave * 64 + d) * 33 + lc] = tok_ok ? (float)(h16)(acc[t][r] * scale) : 0.f;
    }
  __syncthreads();
  if (tid < 128) {
    const int c = tid >> 6, d = tid & 63;
    if (tok0 + 64 * c < T) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll 8
        for (int q = 0; q < 32; ++q) sum += red[((2 * c + w) * 64 + d) * 33 + q];
      out[(chunk0 + c) * ldo + d] = sum;
    }
  }
}

// max / sum of a value and its copy in the lane 32 apart (same query row)
DEVI float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
DEVI float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(256, 4) void flash_fwd_kernel(const h16* __restrict__ qkv, h16* __restrict__ y,
                                                           float* __restrict__ lse, int T, int NH, int C,
                                                           float sl2) {
  __shared__ __attribute__((aligned(1024))) h16 smem[2 * ASTAGE];  // [stage][K | V]
  int qt, h, b;
  attn_block(T, NH, qt, h, b);
  qt = (T + 127) / 128 - 1 - qt;  // tile 0: the most key tiles
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = qt * 128;
  const int wq0 = q0 + wave * 32;
  const int myq = wq0 + (lane & 31);
  const int64_t ld = 3 * (int64_t)C;
  const h16* Q = qkv + (int64_t)b * T * ld + h * HD;
  const h16* K = Q + C;
  const h16* V = Q + 2 * C;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
  const int nkt = (min(T, q0 + 128) + 63) / 64;
  AttnTileLoader tl;
  tl.init(ld, wave, lane);
  auto load = [&](int j, int stg) {
    const uint32_t base = lds0 + stg * (ASTAGE * 2);
    tl.issue(K, j * 64, T, base, wave, lane);
    tl.issue(V, j * 64, T, base + ATILE * 2, wave, lane);
  };
  load(0, 0);
  h16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = as_h16x8(ld16_or_zero(Q + (int64_t)myq * ld + kk * 16 + hl * 8, myq < T));
  f32x16 o[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) o[0][r] = o[1][r] = 0.f;
  float mrow = -INFINITY, lrow = 0.f;
  const int qlim = min(myq, T - 1);
  // Tile j: wait for its loads, barrier (every wave past tile j-1, whose
  // stage the loads of tile j+1 then take), scores, softmax, O += P V.
  auto step = [&](int j, auto stgc) {
    constexpr int stg = decltype(stgc)::value;
    wait_vmcnt<0>();
    lds_barrier();
    if (j + 1 < nkt) load(j + 1, stg ^ 1);
    const h16* Ks = smem + stg * ASTAGE;
    f32x16 cur[2];
#pragma unroll
    for (int js = 0; js < 2; ++js) {
#pragma unroll
      for (int r = 0; r < 16; ++r) cur[js][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) cur[js] = mfma32(row_frag(Ks, js * 32, kk, lane), qf[kk], cur[js]);
    }
    const int k0 = j * 64;
    if (k0 + 63 > wq0 || k0 + 64 > T) {
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        const int lim = qlim - (k0 + 32 * js + 4 * hl);
#pragma unroll
        for (int r = 0; r < 16; ++r) cur[js][r] = (8 * (r >> 2) + (r & 3) <= lim) ? cur[js][r] : -INFINITY;
      }
    }
    float mx = cur[0][0];
#pragma unroll
    for (int js = 0; js < 2; ++js)
#pragma unroll
      for (int r = (js == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, cur[js][r]);
    const float mx2 = halves_max(mx) * sl2;
    const bool need = mx2 > mrow + kLazy;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mnew = need ? mx2 : mrow;
      const float alpha = exp2_fast(mrow - mnew);
      lrow *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[0][r] *= alpha;
        o[1][r] *= alpha;
      }
      mrow = mnew;
    }
#pragma unroll
    for (int js = 0; js < 2; ++js)
#pragma unroll
      for (int r = 0; r < 16; ++r) cur[js][r] = exp2_fast(fmaf(cur[js][r], sl2, -mrow));
    const h16* Vs = smem + stg * ASTAGE + ATILE;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const h16x8 pf = pack8(cur[st >> 1], 8 * (st & 1));
#pragma unroll
      for (int i = 0; i < 2; ++i) o[i] = mfma32(tr_frag_keys(Vs, st * 16, i * 32, lane), pf, o[i]);
      lrow = sum_h16x8(pf, lrow);
    }
  };
  for (int j = 0; j < nkt; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < nkt) step(j + 1, std::integral_constant<int, 1>{});
  }
  const float ltot = halves_sum(lrow);
  if (myq < T) {
    const float inv = 1.0f / ltot;
    h16* yr = y + ((int64_t)b * T + myq) * C + h * HD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4] = {o[i][4 * q] * inv, o[i][4 * q + 1] * inv, o[i][4 * q + 2] * inv, o[i][4 * q + 3] * inv};
        store4(yr + i * 32 + 8 * q + 4 * hl, v);
      }
    if (hl == 0) lse[((int64_t)b * NH + h) * T + myq] = (mrow + log2f(ltot)) * kLn2;
  }
}

// ---------------------------------------------------------- backward: dK, dV ----
// Workgroup: 128 keys of one (sequence, head); wave w owns keys key0 + 32 w +
// lane%32 and accumulates dK^T and dV^T over the query tiles (64 queries)
// that can see them, one 32-query half at a time (scores, P and dS of that
// half, then its dV / dK products), which keeps the kernel at 168 VGPRs and
// three workgroups per CU.  Q / dO tiles and their LSE / D rows go through a
// two-stage LDS ring, two q-tiles per loop trip (compile-time stage offsets).
// Measured on MI355X (dQ + dK/dV at 16 x 12 x 1024 x 64): two workgroups per
// CU with both halves' P and dS held 142-144 us, three with a three-stage
// ring 138.5, three with two stages 130; the same products in the same order.  Q and dO tiles stream from HBM straight into a
// three-stage LDS ring, and the tile's log-sum-exp (exp2 domain) and D rows
// beside them (written by the dQ kernel).
__global__ __launch_bounds__(256, 3) void flash_bwd_dkdv_kernel(const h16* __restrict__ qkv,
                                                                const h16* __restrict__ dy,
                                                                const float* __restrict__ lse,
                                                                const float* __restrict__ Dd,
                                                                h16* __restrict__ dqkv, int T, int NH, int C,
                                                                float sl2, float scale, float* __restrict__ colsum) {
  // [stage][Q | dO], two stages; sized for the column sums' staging after the loop (33 KB)
  __shared__ __attribute__((aligned(1024))) h16 smem[(4 * 64 * 33 * 4 + 1) / 2 > 2 * ASTAGE ? (4 * 64 * 33 * 4 + 1) / 2 : 2 * ASTAGE];
  __shared__ __attribute__((aligned(16))) float rowv[2][2][64];     // [stage][lse log2e | D]
  int kt, h, b;
  attn_block(T, NH, kt, h, b);
  const int tid = threadIdx.x, lane = tid & 63, lc = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int key0 = kt * 128;  // tile 0: the most query tiles
  const int wk0 = key0 + wave * 32;
  const int mykey = wk0 + lc;
  const int64_t ld = 3 * (int64_t)C;
  const h16* Q = qkv + (int64_t)b * T * ld + h * HD;
  const h16* K = Q + C;
  const h16* V = Q + 2 * C;
  const h16* G = dy + (int64_t)b * T * C + h * HD;
  const float* D_b = Dd + ((int64_t)b * NH + h) * T;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);

  const int nqt = (T - key0 + 63) / 64;
  AttnTileLoader tlq, tlg;  // Q rows are 3C apart, dO rows C apart
  tlq.init(ld, wave, lane);
  tlg.init(C, wave, lane);
  // waves 0 and 1 bring the tile's lse (exp2 domain) and D rows into LDS
  // beside it, one 4-byte element per lane
  const float* L2_b = Dd + (int64_t)(gridDim.x / ((T + 127) / 128)) * T + ((int64_t)b * NH + h) * T;
  const uint32_t rows0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)&rowv[0][0][0]);
  auto load = [&](int it, int stg) {
    const int q0 = key0 + it * 64;
    const uint32_t base = lds0 + stg * (ASTAGE * 2);
    tlq.issue(Q, q0, T, base, wave, lane);
    tlg.issue(G, q0, T, base + ATILE * 2, wave, lane);
    if (wave < 2) dma4((wave == 0 ? L2_b : D_b) + min(q0 + lane, T - 1), rows0 + (stg * 2 + wave) * 256);
  };
  h16x8 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    kf[kk] = as_h16x8(ld16_or_zero(K + (int64_t)mykey * ld + kk * 16 + hl * 8, mykey < T));
    vf[kk] = as_h16x8(ld16_or_zero(V + (int64_t)mykey * ld + kk * 16 + hl * 8, mykey < T));
  }
  f32x16 dk[2], dv[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) dk[0][r] = dk[1][r] = dv[0][r] = dv[1][r] = 0.f;

  // Prologue: tile 0 in flight.  Step it waits for tile it, barrier (tile it
  // resident for every wave, every wave past step it-1), loads tile it+1
  // into the stage tile it-1 used, then uses tile it.
  load(0, 0);
  auto step = [&](int it, auto stgc) {
    constexpr int stg = decltype(stgc)::value;
    wait_vmcnt<0>();
    lds_barrier();
    if (it + 1 < nqt) load(it + 1, stg ^ 1);
    const int q0 = key0 + it * 64;
    const h16* Qs = smem + stg * ASTAGE;
    const h16* Gs = Qs + ATILE;
    if (q0 + 63 >= wk0) {  // some query of the tile sees a key of this wave
      const bool diag = q0 < wk0 + 31 || q0 + 64 > T;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f32x16 sv, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = dp[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          sv = mfma32(row_frag(Qs, i * 32, kk, lane), kf[kk], sv);
          dp = mfma32(row_frag(Gs, i * 32, kk, lane), vf[kk], dp);
        }
        // sv[r]: query q0 + 32 i + 8 (r/4) + 4 hl + r%4, key mykey.  Queries
        // before the key or past T get score -inf (probability exactly 0).
        if (diag) {
          const int lo = mykey - q0 - 4 * hl, span = T - q0 - 4 * hl - lo;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = i * 32 + 8 * (r >> 2) + (r & 3);
            sv[r] = ((unsigned)(c - lo) < (unsigned)span) ? sv[r] : -INFINITY;
          }
        }
        f32x16 P, dS;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qg = i * 32 + 8 * g4 + 4 * hl;  // four consecutive queries
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&rowv[stg][0][qg]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&rowv[stg][1][qg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            const float p = exp2_fast(fmaf(sv[r], sl2, -l4[e]));
            P[r] = p;
            dS[r] = p * (dp[r] - d4[e]);
          }
        }
        // this half's 16-query steps of dV^T += dO^T P and dK^T += Q^T dS
        // (transposed operands read from the natural tiles)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const int st = 2 * i + sh;
          const h16x8 pb = pack8(P, 8 * sh);
          const h16x8 sb = pack8(dS, 8 * sh);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            dv[t] = mfma32(tr_frag_keys(Gs, st * 16, t * 32, lane), pb, dv[t]);
            dk[t] = mfma32(tr_frag_keys(Qs, st * 16, t * 32, lane), sb, dk[t]);
          }
        }
      }
    }
  };
  for (int it = 0; it < nqt; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < nqt) step(it + 1, std::integral_constant<int, 1>{});
  }
  if (mykey < T) {
    h16* o = dqkv + ((int64_t)b * T + mykey) * ld + h * HD;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float a[4] = {dk[t][4 * q] * scale, dk[t][4 * q + 1] * scale, dk[t][4 * q + 2] * scale,
                      dk[t][4 * q + 3] * scale};
        float c[4] = {dv[t][4 * q], dv[t][4 * q + 1], dv[t][4 * q + 2], dv[t][4 * q + 3]};
        store4(o + C + t * 32 + 8 * q + 4 * hl, a);
        store4(o + 2 * C + t * 32 + 8 * q + 4 * hl, c);
      }
  }
  if (colsum) {  // K and V parts of the qkv bias gradient
    float* red = reinterpret_cast<float*>(smem);
    const int64_t chunk0 = ((int64_t)b * T + key0) / 64;
    __syncthreads();  // every wave is done with the Q / dO stages
    chunk_colsums(dk, scale, mykey < T, red, colsum + C + h * HD, chunk0, 3 * (int64_t)C, key0, T);
    __syncthreads();
    chunk_colsums(dv, 1.0f, mykey < T, red, colsum + 2 * C + h * HD, chunk0, 3 * (int64_t)C, key0, T);
  }
}

// --------------------------------------------------------------- backward: dQ ----
// Workgroup: 128 queries; wave w owns queries q0 + 32 w + lane%32, forms D
// for them from the dO and O rows (and stores it for the dK / dV kernel), and
// accumulates dQ^T over the key tiles (64 keys) it sees; K and V tiles stream
// into a two-stage LDS ring as in the forward kernel, two tiles per loop trip.
// A key tile past every query of a wave is computed fully masked (it adds
// zeros) rather than branched around: the branch made the compiler copy the
// dQ accumulators between register sets every tile.
__global__ __launch_bounds__(256, 3) void flash_bwd_dq_kernel(const h16* __restrict__ qkv,
                                                              const h16* __restrict__ y,
                                                              const h16* __restrict__ dy,
                                                              const float* __restrict__ lse, float* __restrict__ Dd,
                                                              h16* __restrict__ dqkv, int T, int NH, int C, float sl2,
                                                              float scale, float* __restrict__ colsum) {
  // [stage][K | V], two stages; sized for the column sums' staging after the loop (33 KB)
  __shared__ __attribute__((aligned(1024))) h16 smem[(4 * 64 * 33 * 4 + 1) / 2 > 2 * ASTAGE ? (4 * 64 * 33 * 4 + 1) / 2 : 2 * ASTAGE];
  int qt, h, b;
  attn_block(T, NH, qt, h, b);
  qt = (T + 127) / 128 - 1 - qt;  // tile 0: the most key tiles
  const int tid = threadIdx.x, lane = tid & 63, lc = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = qt * 128;
  const int wq0 = q0 + wave * 32;
  const int myq = wq0 + lc;
  const int64_t ld = 3 * (int64_t)C;
  const h16* Q = qkv + (int64_t)b * T * ld + h * HD;
  const h16* K = Q + C;
  const h16* V = Q + 2 * C;
  const h16* G = dy + (int64_t)b * T * C + h * HD;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
  const int nkt = (min(T, q0 + 128) + 63) / 64;
  AttnTileLoader tl;
  tl.init(ld, wave, lane);
  auto load = [&](int j, int stg) {
    const uint32_t base = lds0 + stg * (ASTAGE * 2);
    tl.issue(K, j * 64, T, base, wave, lane);
    tl.issue(V, j * 64, T, base + ATILE * 2, wave, lane);
  };
  load(0, 0);

  const bool qok = myq < T;
  const float lse2 = qok ? lse[((int64_t)b * NH + h) * T + myq] * kLog2e : 0.f;
  h16x8 qf[4], gf[4];
  float dsum = 0.f;  // this lane's half of D = sum_d dO O for its query
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qf[kk] = as_h16x8(ld16_or_zero(Q + (int64_t)myq * ld + kk * 16 + hl * 8, qok));
    gf[kk] = as_h16x8(ld16_or_zero(G + (int64_t)myq * C + kk * 16 + hl * 8, qok));
    const h16x8 of = as_h16x8(ld16_or_zero(y + ((int64_t)b * T + myq) * C + h * HD + kk * 16 + hl * 8, qok));
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = fmaf((float)gf[kk][e], (float)of[e], dsum);
  }
  // D for the dK / dV kernel (launched after this one) and for this one
  const float Dq = halves_sum(dsum);
  if (qok && hl == 0) {
    const int64_t rows = (int64_t)(gridDim.x / ((T + 127) / 128)) * T;  // B NH T
    Dd[((int64_t)b * NH + h) * T + myq] = Dq;
    Dd[rows + ((int64_t)b * NH + h) * T + myq] = lse2;
  }
  f32x16 dq[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) dq[0][r] = dq[1][r] = 0.f;
  const int qlim = min(myq, T - 1);

  // Key tile kt: wait for its loads, barrier (every wave past tile kt-1,
  // whose stage the loads of tile kt+1 then take), then use it.
  auto step = [&](int kt, auto stgc) {
    constexpr int stg = decltype(stgc)::value;
    wait_vmcnt<0>();
    lds_barrier();
    if (kt + 1 < nkt) load(kt + 1, stg ^ 1);
    const int k0 = kt * 64;
    const h16* Ks = smem + stg * ASTAGE;
    const h16* Vs = Ks + ATILE;
    {  // a key tile past every query of the wave is masked whole (adds zeros)
      const bool diag = k0 + 63 > wq0 || k0 + 64 > T;
      h16x8 sb[4];  // dS^T in bf16, 16-key steps st = 0..3
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        f32x16 sv, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = dp[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          sv = mfma32(row_frag(Ks, js * 32, kk, lane), qf[kk], sv);
          dp = mfma32(row_frag(Vs, js * 32, kk, lane), gf[kk], dp);
        }
        if (diag) {
          const int lim = qlim - (k0 + 32 * js + 4 * hl);
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = (8 * (r >> 2) + (r & 3) <= lim) ? sv[r] : -INFINITY;
        }
        f32x16 ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(fmaf(sv[r], sl2, -lse2));
          ds[r] = p * (dp[r] - Dq);
        }
        sb[2 * js] = pack8(ds, 0);
        sb[2 * js + 1] = pack8(ds, 8);
      }
      // dQ^T += K^T dS^T (K read transposed, keys in the accumulator order)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int t = 0; t < 2; ++t) dq[t] = mfma32(tr_frag_keys(Ks, st * 16, t * 32, lane), sb[st], dq[t]);
      }
    }
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nkt) step(kt + 1, std::integral_constant<int, 1>{});
  }
  if (qok) {
    h16* o = dqkv + ((int64_t)b * T + myq) * ld + h * HD;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float a[4] = {dq[t][4 * q] * scale, dq[t][4 * q + 1] * scale, dq[t][4 * q + 2] * scale,
                      dq[t][4 * q + 3] * scale};
        store4(o + t * 32 + 8 * q + 4 * hl, a);
      }
  }
  if (colsum) {  // Q part of the qkv bias gradient
    __syncthreads();  // every wave is done with the K / V stages
    chunk_colsums(dq, scale, qok, reinterpret_cast<float*>(smem), colsum + h * HD, ((int64_t)b * T + q0) / 64,
                  3 * (int64_t)C, q0, T);
  }
}

void attn_fwd_bf16(const void* qkv, void* y, float* lse, int B, int T, int NH, int C, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)HD);
  const unsigned grid = (unsigned)((T + 127) / 128 * NH * B);
  flash_fwd_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<const h16*>(qkv), reinterpret_cast<h16*>(y), lse, T, NH,
                                        C, scale * kLog2e);
}

bool attn_bwd_bf16(const void* qkv, const void* y, const void* dy, const float* lse, float* Dbuf, void* dqkv, int B,
                   int T, int NH, int C, float* colsum, hipStream_t s) {
  if (T % 64) colsum = nullptr;  // chunks would straddle sequences
  const float scale = 1.0f / sqrtf((float)HD);
  const unsigned grid = (unsigned)((T + 127) / 128 * NH * B);
  // dQ first: it also writes D = rowsum(dO o O), which dK / dV reads
  flash_bwd_dq_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<const h16*>(qkv), reinterpret_cast<const h16*>(y),
                                           reinterpret_cast<const h16*>(dy), lse, Dbuf,
                                           reinterpret_cast<h16*>(dqkv), T, NH, C, scale * kLog2e, scale, colsum);
  flash_bwd_dkdv_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<const h16*>(qkv), reinterpret_cast<const h16*>(dy),
                                             lse, Dbuf, reinterpret_cast<h16*>(dqkv), T, NH, C, scale * kLog2e,
                                             scale, colsum);
  return colsum != nullptr;
}

// ------------------------------------------------------------------ fp32 path ----
// One wavefront per (query, head, sequence); scores of the row in LDS.
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(const float* __restrict__ qkv, float* __restrict__ y,
                                                          float* __restrict__ lse, int T, int NH, int C) {
  extern __shared__ float sc[];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int hd = C / NH;
  const int64_t ld = 3 * (int64_t)C;
  const float* base = qkv + (int64_t)b * T * ld + h * hd;
  const float* q = base + (int64_t)i * ld;
  const float scale = 1.0f / sqrtf((float)hd);
  float mx = -INFINITY;
  for (int j = lane; j <= i; j += 64) {
    const float* k = base + C + (int64_t)j * ld;
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s = fmaf(q[d], k[d], s);
    s *= scale;
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int j = lane; j <= i; j += 64) {
    const float p = expf(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  __syncthreads();
  for (int d = lane; d < hd; d += 64) {
    float acc = 0.f;
    for (int j = 0; j <= i; ++j) acc = fmaf(sc[j], base[2 * C + (int64_t)j * ld + d], acc);
    y[((int64_t)b * T + i) * C + h * hd + d] = acc / sum;
  }
  if (lane == 0) lse[((int64_t)b * NH + h) * T + i] = mx + logf(sum);
}

// dQ for query i, and D_i = dO_i . O_i kept for the dK/dV kernel.
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(const float* __restrict__ qkv,
                                                             const float* __restrict__ y,
                                                             const float* __restrict__ dy,
                                                             const float* __restrict__ lse, float* __restrict__ Dd,
                                                             float* __restrict__ dqkv, int T, int NH, int C) {
  extern __shared__ float sc[];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int hd = C / NH;
  const int64_t ld = 3 * (int64_t)C;
  const float* base = qkv + (int64_t)b * T * ld + h * hd;
  const float* q = base + (int64_t)i * ld;
  const float* g = dy + ((int64_t)b * T + i) * C + h * hd;
  const float* o = y + ((int64_t)b * T + i) * C + h * hd;
  const float scale = 1.0f / sqrtf((float)hd);
  float dsum = 0.f;
  for (int d = lane; d < hd; d += 64) dsum = fmaf(g[d], o[d], dsum);
  const float Di = wave_sum(dsum);
  const float L = lse[((int64_t)b * NH + h) * T + i];
  for (int j = lane; j <= i; j += 64) {
    const float* k = base + C + (int64_t)j * ld;
    const float* v = base + 2 * C + (int64_t)j * ld;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < hd; ++d) {
      s = fmaf(q[d], k[d], s);
      dp = fmaf(g[d], v[d], dp);
    }
    const float p = expf(s * scale - L);
    sc[j] = p * (dp - Di);
  }
  __syncthreads();
  for (int d = lane; d < hd; d += 64) {
    float acc = 0.f;
    for (int j = 0; j <= i; ++j) acc = fmaf(sc[j], base[C + (int64_t)j * ld + d], acc);
    dqkv[((int64_t)b * T + i) * ld + h * hd + d] = acc * scale;
  }
  if (lane == 0) Dd[((int64_t)b * NH + h) * T + i] = Di;
}

// dK, dV for key j.
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(const float* __restrict__ qkv,
                                                               const float* __restrict__ dy,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ Dd,
                                                               float* __restrict__ dqkv, int T, int NH, int C) {
  extern __shared__ float sc[];  // [2][T]
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int hd = C / NH;
  const int64_t ld = 3 * (int64_t)C;
  const float* base = qkv + (int64_t)b * T * ld + h * hd;
  const float* k = base + C + (int64_t)j * ld;
  const float* v = base + 2 * C + (int64_t)j * ld;
  const float scale = 1.0f / sqrtf((float)hd);
  float* P = sc;
  float* S = sc + T;
  for (int i = j + lane; i < T; i += 64) {
    const float* q = base + (int64_t)i * ld;
    const float* g = dy + ((int64_t)b * T + i) * C + h * hd;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < hd; ++d) {
      s = fmaf(q[d], k[d], s);
      dp = fmaf(g[d], v[d], dp);
    }
    const int64_t r = ((int64_t)b * NH + h) * T + i;
    const float p = expf(s * scale - lse[r]);
    P[i] = p;
    S[i] = p * (dp - Dd[r]);
  }
  __syncthreads();
  for (int d = lane; d < hd; d += 64) {
    float a = 0.f, c = 0.f;
    for (int i = j; i < T; ++i) {
      a = fmaf(S[i], base[(int64_t)i * ld + d], a);
      c = fmaf(P[i], dy[((int64_t)b * T + i) * C + h * hd + d], c);
    }
    float* out = dqkv + ((int64_t)b * T + j) * ld + h * hd + d;
    out[C] = a * scale;
    out[2 * C] = c;
  }
}

void attn_fwd_f32(const float* qkv, float* y, float* lse, int B, int T, int NH, int C, hipStream_t s) {
  dim3 grid(T, NH, B);
  attn_fwd_f32_kernel<<<grid, 64, T * sizeof(float), s>>>(qkv, y, lse, T, NH, C);
}

void attn_bwd_f32(const float* qkv, const float* y, const float* dy, const float* lse, float* Dbuf, float* dqkv,
                  int B, int T, int NH, int C, hipStream_t s) {
  dim3 grid(T, NH, B);
  attn_bwd_dq_f32_kernel<<<grid, 64, T * sizeof(float), s>>>(qkv, y, dy, lse, Dbuf, dqkv, T, NH, C);
  attn_bwd_dkdv_f32_kernel<<<grid, 64, 2 * T * sizeof(float), s>>>(qkv, dy, lse, Dbuf, dqkv, T, NH, C);
}

}  // namespace gpt2k
