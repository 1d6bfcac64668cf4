// GEMMs of the GPT-2 step: C = A B with fused epilogues.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on LDS-staged tiles.  Both operand
// tiles are kept in LDS with k contiguous per row, so every MFMA fragment is a
// single 16-byte LDS read; operands stored with k strided in HBM (the
// transposed operands of the backward GEMMs) are transposed in registers
// (8x8 bf16 blocks, v_perm_b32) between the coalesced global load and the
// LDS store.  Global loads of tile k+1 are in flight while tile k is
// multiplied (two LDS buffers, one barrier per k-tile).
//
// fp32 path: LDS-tiled FMA GEMM (64x64 tile, 4x4 outputs per thread).
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds_tile.h"

namespace gpt2k {

// ---------------------------------------------------------------- epilogue ----
template <int EPI, typename TA>
DEVI void epi_store4(const GemmArgs& p, int m, int n, float v[4], int split) {
  const int64_t off = (int64_t)m * p.ldc + n;
  if constexpr (EPI == EPI_LOGITS) {
    store4(reinterpret_cast<TA*>(p.C) + off, v);
  } else if constexpr (EPI == EPI_ACT) {
    if (p.bias) {
      float b[4];
      load4(p.bias + n, b);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += b[i];
    }
    store4(reinterpret_cast<TA*>(p.C) + off, v);
  } else if constexpr (EPI == EPI_F32) {
    store4(reinterpret_cast<float*>(p.C) + off, v);
  } else if constexpr (EPI == EPI_F32_ACC) {
    float o[4];
    float* c = reinterpret_cast<float*>(p.C) + off;
    load4(c, o);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += o[i];
    store4(c, v);
  } else if constexpr (EPI == EPI_RESID) {
    float r[4], b[4] = {0.f, 0.f, 0.f, 0.f};
    load4(p.resid + off, r);
    if (p.bias) load4(p.bias + n, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r[i] + (v[i] + b[i]);
    store4(reinterpret_cast<float*>(p.C) + off, v);
  } else if constexpr (EPI == EPI_GELU) {
    float b[4] = {0.f, 0.f, 0.f, 0.f}, g[4], d[4];
    if (p.bias) load4(p.bias + n, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) gelu_and_grad(v[i] + b[i], g[i], d[i]);
    store4(reinterpret_cast<TA*>(p.C) + off, d);
    store4(reinterpret_cast<TA*>(p.C2) + off, g);
  } else if constexpr (EPI == EPI_GELU_BWD) {
    float d[4];
    load4(reinterpret_cast<const TA*>(p.aux) + off, d);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= d[i];
    store4(reinterpret_cast<TA*>(p.C) + off, v);
  } else {  // EPI_PARTIAL
    store4(reinterpret_cast<float*>(p.C) + (int64_t)split * p.split_stride + off, v);
  }
}

// One element (fp32 path, shapes that are not multiples of four).
template <int EPI, typename TA>
DEVI void epi_store1(const GemmArgs& p, int m, int n, float v, int split) {
  const int64_t off = (int64_t)m * p.ldc + n;
  if constexpr (EPI == EPI_LOGITS) {
    reinterpret_cast<TA*>(p.C)[off] = from_f32<TA>(v);
  } else if constexpr (EPI == EPI_ACT) {
    reinterpret_cast<TA*>(p.C)[off] = from_f32<TA>(p.bias ? v + p.bias[n] : v);
  } else if constexpr (EPI == EPI_F32) {
    reinterpret_cast<float*>(p.C)[off] = v;
  } else if constexpr (EPI == EPI_F32_ACC) {
    reinterpret_cast<float*>(p.C)[off] += v;
  } else if constexpr (EPI == EPI_RESID) {
    reinterpret_cast<float*>(p.C)[off] = p.resid[off] + (v + p.bias[n]);
  } else if constexpr (EPI == EPI_GELU) {
    float g, d;
    gelu_and_grad(v + p.bias[n], g, d);
    reinterpret_cast<TA*>(p.C)[off] = from_f32<TA>(d);
    reinterpret_cast<TA*>(p.C2)[off] = from_f32<TA>(g);
  } else if constexpr (EPI == EPI_GELU_BWD) {
    reinterpret_cast<TA*>(p.C)[off] = from_f32<TA>(v * to_f32(reinterpret_cast<const TA*>(p.aux)[off]));
  } else {
    reinterpret_cast<float*>(p.C)[(int64_t)split * p.split_stride + off] = v;
  }
}

// ------------------------------------------------------------ bf16 MFMA GEMM ----
// Stages an R x BK operand tile (rows r0.., k in [k0, kend)) through registers
// into LDS laid out [R][BK + 8] (k contiguous, 16-byte row padding: the
// fragment reads of eight consecutive rows hit distinct banks).
template <bool KMAJ, int R, int BK, int NT>
struct TileLoader {
  static constexpr int LDS = BK + 8;
  static constexpr int NCH = KMAJ ? (R * BK / 8) : (R * BK / 64);
  static constexpr int PER = (NCH + NT - 1) / NT;
  static constexpr int REGS = KMAJ ? PER : PER * 8;
  u32x4 r[REGS];

  DEVI void load(const h16* g, int64_t ld, int r0, int rmax, int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      if (NCH % NT == 0 || c < NCH) {
        if constexpr (KMAJ) {
          // g is [rows][k]: 16-byte chunks along k, eight lanes per 128-byte row
          const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
          const bool ok = (r0 + row < rmax) && (k0 + kc < kend);
          r[i] = ld16_or_zero(g + (int64_t)(r0 + row) * ld + k0 + kc, ok);
        } else {
          // g is [k][rows]: an 8 (k) x 8 (rows) block; consecutive lanes take
          // consecutive k blocks so that the transposed LDS rows they write
          // are contiguous
          const int kb = c % (BK / 8), rb = c / (BK / 8);
          const int rr = r0 + rb * 8;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int k = k0 + kb * 8 + j;
            r[i * 8 + j] = ld16_or_zero(g + (int64_t)k * ld + rr, (k < kend) && (rr < rmax));
          }
        }
      }
    }
  }
  DEVI void store(h16* s, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      if (NCH % NT == 0 || c < NCH) {
        if constexpr (KMAJ) {
          const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
          *reinterpret_cast<u32x4*>(s + row * LDS + kc) = r[i];
        } else {
          const int kb = c % (BK / 8), rb = c / (BK / 8);
          u32x4 t[8];
          transpose8x8(&r[i * 8], t);
#pragma unroll
          for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(s + (rb * 8 + e) * LDS + kb * 8) = t[e];
        }
      }
    }
  }
};

// Tile t of one k-split: groups of GM tile-rows are walked column by column,
// so that neighbouring tiles share operand rows and columns.
DEVI void tile_walk(const GemmArgs& p, int tiles_m, int tiles_n, int t, int& tm, int& tn) {
  const int GM = p.group_m > 0 ? p.group_m : 8;
  const int per_group = GM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int w = t - g * per_group;
  tm = first_m + w % gm;
  tn = w / gm;
}

// Tile order.  The dispatcher deals workgroups round-robin to the eight XCDs
// (each with its own L2) in linear block order, so the linear id is first
// renumbered to give every XCD a contiguous range; that range is walked
// split by split, and within a split in groups of GM tile-rows so that
// neighbouring tiles share A rows and B columns in that XCD's L2.
DEVI void tile_coords(const GemmArgs& p, int tiles_m, int tiles_n, int b, int nblk, int& tm, int& tn,
                      int& split) {
  constexpr int NX = 8;
  int t = b;
  if (!p.no_xcd_map) {
    const int xcd = b % NX, idx = b / NX;
    const int q = nblk / NX, rem = nblk % NX;
    t = xcd * q + min(xcd, rem) + idx;
  }
  const int tiles = tiles_m * tiles_n;
  split = t / tiles;
  t -= split * tiles;
  tile_walk(p, tiles_m, tiles_n, t, tm, tn);
}

template <bool A_K, bool B_K, int BM, int BN, int BK, int WGM, int WGN, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int LDS = BK + 8;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is a multiple of 32");
  __shared__ __attribute__((aligned(16))) h16 smem[2 * (BM + BN) * LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int lc = lane & 31, hl = lane >> 5;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn, split;
  tile_coords(p, tiles_m, tiles_n, blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nkt = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const h16* A = reinterpret_cast<const h16*>(p.A);
  const h16* B = reinterpret_cast<const h16*>(p.B);

  h16* sA0 = smem;
  h16* sB0 = smem + BM * LDS;
  h16* sA1 = smem + (BM + BN) * LDS;
  h16* sB1 = sA1 + BM * LDS;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  TileLoader<A_K, BM, BK, NT> la;
  TileLoader<B_K, BN, BK, NT> lb;
  if (nkt > 0) {
    la.load(A, p.lda, m0, p.M, kbeg, kend, tid);
    lb.load(B, p.ldb, n0, p.N, kbeg, kend, tid);
    la.store(sA0, tid);
    lb.store(sB0, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) {
      la.load(A, p.lda, m0, p.M, kbeg + (kt + 1) * BK, kend, tid);
      lb.load(B, p.ldb, n0, p.N, kbeg + (kt + 1) * BK, kend, tid);
    }
    const h16* a_s = ((kt & 1) ? sA1 : sA0) + (wm * WTM + lc) * LDS + hl * 8;
    const h16* b_s = ((kt & 1) ? sB1 : sB0) + (wn * WTN + lc) * LDS + hl * 8;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      h16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const h16x8*>(a_s + i * 32 * LDS + kk * 16);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const h16x8*>(b_s + j * 32 * LDS + kk * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          // first operand supplies the output rows (n), second the columns (m)
          acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
    }
    if (more) {
      la.store((kt & 1) ? sA0 : sA1, tid);
      lb.store((kt & 1) ? sB0 : sB1, tid);
    }
    __syncthreads();
  }

  // acc[i][j][4q + e] is C[m][n] with m = .. + lc, n = .. + 8q + 4hl + e
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WTM + i * 32 + lc;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * hl;
        if (n < p.N) {
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          epi_store4<EPI, h16>(p, m, n, v, split);
        }
      }
    }
  }
}

// --------------------------------------------- bf16 MFMA GEMM, LDS-direct ----
// Operand tiles go from HBM to LDS with global_load_lds_dwordx4 (each lane
// moves 16 bytes; a wave instruction fills 1 KB of LDS), NST stages deep, so
// tiles kt+1 .. kt+NST-2 are in flight while tile kt is multiplied and no
// VGPRs or LDS-store instructions are spent on staging.
//   * k-contiguous operand: LDS rows of BK elements; the 16-byte chunks of a
//     row are XOR-swizzled by the row so that the ds_read_b128 fragment reads
//     of 16 consecutive rows hit distinct banks;
//   * transposed operand (stored [k][rows] in HBM): LDS rows are k, laid out
//     as in HBM (chunks swizzled by 2 (k mod 4)); fragments come from pairs of
//     ds_read_b64_tr_b16, which hand each lane four consecutive k of one row.
// Tiles are not zero-filled: rows past M or N are clamped to the last row
// (their outputs are discarded), so K must be a multiple of BK.

// This wave's share of the direct loads of one R x BK operand tile.  The
// per-lane source addresses are formed once; each k-tile adds its offset.
template <bool KMAJ, int R, int BK, int NW>
struct DirectLoader {
  static constexpr int BYTES = R * BK * 2;
  static constexpr int INSTR = BYTES / 1024;         // wave instructions per tile
  // every wave issues the same number of loads (the vmcnt accounting is per
  // wave); surplus loads repeat the tile's last chunk (same bytes, same place)
  static constexpr int PER_WAVE = (INSTR + NW - 1) / NW;
  static_assert(BYTES % 1024 == 0, "whole 1 KB wave loads");
  const h16* src[PER_WAVE];
  uint32_t lds[PER_WAVE];
  int64_t kstep;  // elements between consecutive k-tiles

  DEVI void init(const h16* g, int64_t ld, int r0, int rmax, int kbeg, const h16* lds_tile, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int J = min(wave * PER_WAVE + j, INSTR - 1);
      const int byte = J * 1024 + lane * 16;
      if constexpr (KMAJ) {
        const int r = byte / (BK * 2), pc = (byte % (BK * 2)) / 16;
        const int c = pc ^ kswz<BK>(r);
        const int row = min(r0 + r, rmax - 1);
        src[j] = g + (int64_t)row * ld + kbeg + 8 * c;
      } else {
        const int k = byte / (R * 2), pc = (byte % (R * 2)) / 16;
        const int c = pc ^ tswz<R>(k);
        const int col = min(r0 + 8 * c, rmax - 8);
        src[j] = g + (int64_t)(kbeg + k) * ld + col;
      }
      lds[j] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(lds_tile + J * 512));
    }
    kstep = KMAJ ? (int64_t)BK : (int64_t)BK * ld;
  }
  // loads k-tile kt into the stage whose LDS byte offset from stage 0 is stage_off
  DEVI void issue(int kt, uint32_t stage_off) const {
    const int64_t off = kt * kstep;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) dma16(src[j] + off, __builtin_amdgcn_readfirstlane(lds[j] + stage_off));
  }
};

// ----------------------------------------------------------- epilogue ----
// Writes one wave's FM x FN accumulator tiles (rows mb.., columns nb..).
// acc[i][j][4q + e] holds C[mb + 32 i + lane % 32][nb + 32 j + 8 q + 4 (lane / 32) + e].
// bf16 outputs are staged through this wave's LDS region (RB rows of
// 32 FN + 8 elements: the whole wave tile, or one 32-row block of it at a
// time) so that every store instruction writes whole row segments (16 bytes
// per lane along n) instead of 16 bytes into each of 32 rows; lines then
// reach L2 complete.  Other outputs go straight from the registers.
template <int EPI>
constexpr bool epi_staged() {
  return EPI == EPI_ACT || EPI == EPI_LOGITS || EPI == EPI_GELU || EPI == EPI_GELU_BWD;
}

// aux_pre (EPI_GELU_BWD, staged, or null): this wave's aux tile already in
// registers, chunk `it` of the staging loop below in aux_pre[it].
template <int EPI, int FM, int FN, bool STAGED, int RB = 32 * FM>
DEVI void gemm_epilogue(const GemmArgs& p, f32x16 (&acc)[FM][FN], h16* region, int mb, int nb, int lane, int split,
                        const u32x4* aux_pre = nullptr) {
  constexpr int WTM = 32 * FM, WTN = 32 * FN;
  const int lc = lane & 31, hl = lane >> 5;
  if constexpr (STAGED) {
    // RB rows of the wave tile per pass (the region holds RB rows of WTN + 8
    // elements): the whole tile, or 32-row blocks where LDS is short.
    constexpr int SLD = WTN + 8;  // staged row stride (elements)
    constexpr int NOUT = EPI == EPI_GELU ? 2 : 1;
    constexpr int CPR = WTN / 8;       // 16-byte chunks per staged row
    constexpr int RBF = RB / 32;       // accumulator row blocks per pass
    constexpr int ITB = RB * CPR / 64;  // 16-byte chunks per lane for one pass
    static_assert(RB % 32 == 0 && WTM % RB == 0, "whole 32-row blocks per pass");
    static_assert(WTN / 2 <= 64, "one column pair per lane for the column sums");
    // The 16-byte chunk it * 64 + lane of a pass is row q / CPR, chunk q % CPR
    // of the staged rows.  That pattern repeats every PER iterations, RPP rows
    // further down, so the divisions are taken once for the first PER
    // iterations and the rest add a constant row step: RPP rows of the
    // staging region (an immediate) and of the output (one 32-bit add).
    constexpr int G = (CPR & -CPR) < 64 ? (CPR & -CPR) : 64;  // gcd(64, CPR): CPR's power-of-two part
    constexpr int PER = CPR / G, RPP = 64 / G;
    static_assert(ITB % PER == 0 && RB % RPP == 0, "whole periods per pass");
    int rb[PER], cb[PER];
    uint32_t ob[PER];  // element offset of chunk b from the pass's first output element
#pragma unroll
    for (int b = 0; b < PER; ++b) {
      rb[b] = (b * 64 + lane) / CPR;
      cb[b] = (b * 64 + lane) % CPR;
      ob[b] = (uint32_t)rb[b] * (uint32_t)p.ldc + 8u * (uint32_t)cb[b];
    }
    const uint32_t ostep = (uint32_t)RPP * (uint32_t)p.ldc;  // RPP output rows, wave-uniform
    auto row_of = [&](int it) { return (it / PER) * RPP + rb[it % PER]; };
    auto chunk_of = [&](int it) { return cb[it % PER]; };
    auto goff = [&](int it) { return ob[it % PER] + (uint32_t)(it / PER) * ostep; };
    float cs0 = 0.f, cs1 = 0.f;  // GELU', 32-row passes: this lane's column pair, current 64-row chunk
#pragma unroll
    for (int pb = 0; pb < WTM / RB; ++pb) {
      const int mi = mb + RB * pb;
      if constexpr (EPI == EPI_GELU_BWD) {
        // the gelu'(u) rows come in whole row segments too
        const h16* aux = reinterpret_cast<const h16*>(p.aux) + (mi * p.ldc + nb);
#pragma unroll
        for (int it = 0; it < ITB; ++it) {
          const int r = row_of(it), c = chunk_of(it);
          *reinterpret_cast<u32x4*>(region + r * SLD + 8 * c) =
              aux_pre ? aux_pre[pb * ITB + it] : ld16_or_zero(aux + goff(it), mi + r < p.M && nb + 8 * c < p.N);
          if (it % 8 == 7) __builtin_amdgcn_sched_barrier(0);  // bounded loads in flight
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
      }
#pragma unroll
      for (int o = 0; o < NOUT; ++o) {
#pragma unroll
        for (int ib = 0; ib < RBF; ++ib) {
          const int i = pb * RBF + ib;
          const int rl = ib * 32 + lc;  // this lane's staged row
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int nl = j * 32 + 8 * q + 4 * hl;
              const int n = nb + nl;
              float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              if constexpr (EPI == EPI_ACT || EPI == EPI_GELU) {
                if (o == 0 && p.bias && n < p.N) {
                  float bb[4];
                  load4(p.bias + n, bb);
#pragma unroll
                  for (int e = 0; e < 4; ++e) v[e] += bb[e];
                }
              }
              if constexpr (EPI == EPI_GELU) {
                // pass 0 writes gelu'(u) and leaves gelu(u) in the accumulators
                // for pass 1: one sigmoid per element
                if (o == 0) {
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    float g;
                    gelu_and_grad(v[e], g, v[e]);
                    acc[i][j][4 * q + e] = g;
                  }
                }
              }
              if constexpr (EPI == EPI_GELU_BWD) {
                float d[4];
                load4(region + rl * SLD + nl, d);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= d[e];
              }
              store4(region + rl * SLD + nl, v);
              // one accumulator block at a time: the scheduler must not copy
              // every accumulator out of the AGPRs at once
              if (q == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        h16* out = reinterpret_cast<h16*>(o == 0 ? p.C : p.C2) + (mi * p.ldc + nb);
#pragma unroll
        for (int it = 0; it < ITB; ++it) {
          const int r = row_of(it), c = chunk_of(it);
          if (mi + r < p.M && nb + 8 * c < p.N)
            *reinterpret_cast<u32x4*>(out + goff(it)) = *reinterpret_cast<const u32x4*>(region + r * SLD + 8 * c);
        }
        if constexpr (EPI == EPI_GELU_BWD && WTM % 64 == 0) {
          // column sums of the staged (bf16) rows per 64-row chunk: the bias
          // gradient of the layer whose pre-activation gradient this is.  Rows
          // are added in ascending order, as a separate column-sum pass over C
          // would.
          if (p.colsum && lane < WTN / 2) {
            const int n = nb + 2 * lane;
            auto sum_rows = [&](int r0, int rows) {
              const h16* col = region + r0 * SLD + 2 * lane;
#pragma unroll 8
              for (int r = 0; r < rows; ++r) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(col + r * SLD);
                cs0 += lo16_f32(w);
                cs1 += hi16_f32(w);
              }
            };
            auto flush = [&](int c0) {  // chunk of rows c0 .. c0 + 63
              if (n < p.N) {
                float* cp = p.colsum + (int64_t)(c0 >> 6) * p.N + n;
                cp[0] = cs0;
                cp[1] = cs1;
              }
              cs0 = cs1 = 0.f;
            };
            if constexpr (RB >= 64) {
#pragma unroll
              for (int c = 0; c < RB / 64; ++c) {
                const int c0 = mi + 64 * c;
                if (c0 >= p.M) break;  // wave-uniform
                sum_rows(64 * c, min(64, p.M - c0));
                flush(c0);
              }
            } else {
              sum_rows(0, min(32, p.M - mi));  // wave-uniform; none past M
              if ((pb & 1) && mi - 32 < p.M) flush(mi - 32);
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
      }
    }
  } else if constexpr (EPI == EPI_RESID && FM * FN <= 6) {
    // the residual tile is loaded whole first (one round trip instead of FM)
    f32x4 rv[FM][FN][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = mb + i * 32 + lc, n = nb + j * 32 + 8 * q + 4 * hl;
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          rv[i][j][q] = (m < p.M && n < p.N) ? *reinterpret_cast<const f32x4*>(p.resid + (int64_t)m * p.ldc + n) : z;
        }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = mb + i * 32 + lc;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb + j * 32 + 8 * q + 4 * hl;
          if (n < p.N) {
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.bias) load4(p.bias + n, b);
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = rv[i][j][q][e] + (acc[i][j][4 * q + e] + b[e]);
            store4(reinterpret_cast<float*>(p.C) + (int64_t)m * p.ldc + n, v);
          }
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = mb + i * 32 + lc;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb + j * 32 + 8 * q + 4 * hl;
          if (n < p.N) {
            float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            epi_store4<EPI, h16>(p, m, n, v, split);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <bool A_K, bool B_K, int BM, int BN, int BK, int WGM, int WGN, int NST, int EPI, int OCC = 1>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void gemm_lds_kernel(GemmArgs p) {
  static_assert(NST >= 2 && NST <= 4, "two to four stages");
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int STAGE = (BM + BN) * BK;
  using LA = DirectLoader<A_K, BM, BK, NW>;
  using LB = DirectLoader<B_K, BN, BK, NW>;
  constexpr int LPW = LA::PER_WAVE + LB::PER_WAVE;  // loads per wave per tile
  // One array per stage: every LDS access names its stage at compile time, so
  // the compiler can tell the reads of stage s from the loads into the others.
  __shared__ __attribute__((aligned(1024))) h16 st0[STAGE];
  __shared__ __attribute__((aligned(1024))) h16 st1[STAGE];
  __shared__ __attribute__((aligned(1024))) h16 st2[NST > 2 ? STAGE : 1];
  __shared__ __attribute__((aligned(1024))) h16 st3[NST > 3 ? STAGE : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn, split;
  tile_coords(p, tiles_m, tiles_n, blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nkt = kend > kbeg ? (kend - kbeg) / BK : 0;
  const h16* A = reinterpret_cast<const h16*>(p.A);
  const h16* B = reinterpret_cast<const h16*>(p.B);

  auto stage = [&](auto S) -> h16* {
    constexpr int s = decltype(S)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else return st3;
  };
  LA la;
  LB lb;
  la.init(A, p.lda, m0, p.M, kbeg, st0, wave, lane);
  lb.init(B, p.ldb, n0, p.N, kbeg, st0 + BM * BK, wave, lane);
  const uint32_t base0 = (uint32_t)(uintptr_t)(lds_void*)st0;
  auto issue = [&](auto S, int kt) {
    const uint32_t off = (uint32_t)(uintptr_t)(lds_void*)stage(S) - base0;
    la.issue(kt, off);
    lb.issue(kt, off);
  };

  // Epilogues that add a per-column bias start the accumulators from it
  // (acc[i][j][4q + e] is column n0 + wn WTN + 32 j + 8 q + 4 hl + e), so the
  // epilogue neither loads nor adds it.
  constexpr bool kBiasInit = EPI == EPI_ACT || EPI == EPI_GELU || EPI == EPI_RESID;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float b[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kBiasInit) {
        const int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);
        if (p.bias && n < p.N && split == 0) load4(p.bias + n, b);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = b[e];
    }

  // one k-tile on stage S: wait for its loads, free the oldest stage, refill it, multiply
  auto step = [&](auto S, int kt) {
    constexpr int s = decltype(S)::value;
    const int ahead = min(nkt - 1, kt + NST - 2) - kt;
    if constexpr (NST >= 4) {
      if (ahead >= 2) wait_vmcnt<2 * LPW>();
      else if (ahead == 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
    } else if constexpr (NST == 3) {
      if (ahead >= 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();  // every wave's loads of tile kt landed; the stage of tile kt-1 is free
    if (kt + NST - 1 < nkt) issue(std::integral_constant<int, (s + NST - 1) % NST>{}, kt + NST - 1);
    const h16* sa = stage(S);
    const h16* sb = sa + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      h16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = frag<A_K, BM, BK>(sa, wm * WTM + i * 32, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = frag<B_K, BN, BK>(sb, wn * WTN + j * 32, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
    }
  };

  if (0 < nkt) issue(std::integral_constant<int, 0>{}, 0);
  if (1 < nkt && NST > 2) issue(std::integral_constant<int, 1>{}, 1);
  if constexpr (NST > 3)
    if (2 < nkt) issue(std::integral_constant<int, 2>{}, 2);

  for (int kt = 0; kt < nkt; kt += NST) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nkt) step(std::integral_constant<int, 1>{}, kt + 1);
    if constexpr (NST > 2)
      if (kt + 2 < nkt) step(std::integral_constant<int, 2>{}, kt + 2);
    if constexpr (NST > 3)
      if (kt + 3 < nkt) step(std::integral_constant<int, 3>{}, kt + 3);
  }

  GemmArgs pe = p;
  if constexpr (kBiasInit) pe.bias = nullptr;  // already in the accumulators
  constexpr int SLD = WTN + 8;
  constexpr int WPA = (NW + 1) / 2;  // waves per stage array
  if constexpr (epi_staged<EPI>() && WPA * WTM * SLD <= STAGE) {
    __syncthreads();  // all waves are done reading the operand stages
    h16* region = (wave < WPA ? st0 : st1) + (wave % WPA) * WTM * SLD;
    gemm_epilogue<EPI, FM, FN, true>(pe, acc, region, m0 + wm * WTM, n0 + wn * WTN, lane, split);
  } else {
    gemm_epilogue<EPI, FM, FN, false>(pe, acc, nullptr, m0 + wm * WTM, n0 + wn * WTN, lane, split);
  }
}

// ------------------------------------------------------- one wave per SIMD ----
// 2 x 2 waves, each owning a (BM/2) x (BN/2) accumulator tile (up to 256
// accumulators, which live in AGPRs), BK = 64, two LDS stages filled by
// global_load_lds.  With one wave per SIMD nothing hides a stall behind
// another wave, so the k-loop is scheduled explicitly: after every MFMA the
// wave issues at most one fragment read for the next 16-k step (double-
// buffered fragment registers) and a share of the direct loads of a later
// k-tile (the schedule is described in w4_tiles).  A k-tile's only
// barrier sits before its last 16-k step, once every wave holds that step's
// fragments.  Measured on MI355X the loop runs at about 95% of the MFMA peak
// without the operand loads; with them it is bound by the operand stream
// (about 40-48 GB/s per CU from L2).

// A k-tile's direct loads go out in two halves (measured: 0.6% faster over
// the whole step than one burst; three or four chunks leave the last one too
// little time before the barrier that waits for it).
constexpr int kW4LoadChunks = 2;

// This wave's share of one R x 64 operand tile, in the SADDR form: a wave-
// uniform base (advanced per k-tile) plus a 32-bit per-lane byte offset.
template <bool KMAJ, int R, int NW>
struct SaddrLoader {
  static constexpr int INSTR = R * 64 * 2 / 1024;  // 1 KB wave instructions per k-tile
  static constexpr int PER_WAVE = INSTR / NW;
  static_assert(INSTR % NW == 0, "whole instructions per wave");
  const h16* base;
  uint32_t voff[PER_WAVE];
  uint32_t lds[PER_WAVE];
  int64_t kstep;

  // Rows past rmax are clamped to the last row (their outputs are discarded).
  DEVI void init(const h16* g, int64_t ld, int r0, int rmax, int kbeg, const h16* lds_tile, int wave, int lane) {
    base = uniform_ptr(KMAJ ? g + (int64_t)r0 * ld + kbeg : g + (int64_t)kbeg * ld + r0);
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int J = wave * PER_WAVE + j;
      const int byte = J * 1024 + lane * 16;
      if constexpr (KMAJ) {
        const int r = byte / 128, pc = (byte % 128) / 16;
        const int c = pc ^ kswz<64>(r);
        const int row = min(r0 + r, rmax - 1);
        voff[j] = (uint32_t)(((int64_t)(row - r0) * ld + 8 * c) * 2);
      } else {
        const int k = byte / (R * 2), pc = (byte % (R * 2)) / 16;
        const int c = pc ^ tswz<R>(k);
        const int col = min(r0 + 8 * c, rmax - 8);
        voff[j] = (uint32_t)(((int64_t)k * ld + (col - r0)) * 2);
      }
      lds[j] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(lds_tile + J * 512));
    }
    kstep = KMAJ ? (int64_t)64 : (int64_t)64 * ld;
  }
  DEVI void issue(int j, int kt, uint32_t stage_off) const {
    dma16s(base + kt * kstep, voff[j], lds[j] + stage_off);
  }
};

// LDS elements of the tile: two operand stages; the staged epilogue of a
// single tile takes the whole wave tile at once (over both stages), that of
// a persistent workgroup 32-row blocks from the second stage on (the first
// is then receiving the next tile's loads).
template <int BM, int BN, bool PERSIST, int NW = 4>
constexpr int w4_lds_elems() {
  constexpr int STAGE = (BM + BN) * 64, SLD = BN / 2 + 8;
  constexpr int EPI_ELEMS = PERSIST ? STAGE + NW * 32 * SLD : 2 * BM * SLD;
  return 2 * STAGE > EPI_ELEMS ? 2 * STAGE : EPI_ELEMS;
}

// A sequence of BM x BN output tiles of p, one after the other in this
// workgroup: next(tm, tn, split) gives the coordinates of the next tile
// (tile row tm, column tn, k-split split) or returns false.  Between two
// tiles the loads of the next tile's first k-tile go out before the
// epilogue of the current one (which stages through the other stage), so
// that their latency is spent storing instead of waiting.
template <bool A_K, bool B_K, int BM, int BN, int EPI, bool PERSIST, int NW, class Next>
DEVI void w4_tiles(const GemmArgs& p, h16* smem, Next next) {
  constexpr int BK = 64;
  constexpr int WTM = BM / (NW / 2), WTN = BN / 2;  // NW / 2 x 2 waves
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "whole 32 x 32 accumulator blocks");
  // 64-row tiles (one accumulator row block per wave) computed a wrong step
  // in the residual epilogue and are not supported
  static_assert(BM >= 128, "tiles of at least 128 rows");
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int STAGE = (BM + BN) * BK;  // elements
  constexpr int SLD = WTN + 8;           // staged epilogue row stride
  using LA = SaddrLoader<A_K, BM, NW>;
  using LB = SaddrLoader<B_K, BN, NW>;
  constexpr int LPW = LA::PER_WAVE + LB::PER_WAVE;
  constexpr int G = FM * FN;  // MFMAs per 16-k step

  int tm, tn, split;
  if (!next(tm, tn, split)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int m0, n0, kbeg, nkt;
  LA la;
  LB lb;
  // operand loaders of tile (tm, tn, split)
  auto setup = [&]() {
    m0 = tm * BM;
    n0 = tn * BN;
    kbeg = split * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    nkt = kend > kbeg ? (kend - kbeg) / BK : 0;
    la.init(reinterpret_cast<const h16*>(p.A), p.lda, m0, p.M, kbeg, smem, wave, lane);
    lb.init(reinterpret_cast<const h16*>(p.B), p.ldb, n0, p.N, kbeg, smem + BM * BK, wave, lane);
  };
  constexpr uint32_t kStageBytes = STAGE * 2;
  // direct load number d (A loads first) of k-tile kt into the stage at stage_off
  auto dma = [&](int d, int kt, uint32_t stage_off) {
    if (d < LA::PER_WAVE) la.issue(d, kt, stage_off);
    else lb.issue(d - LA::PER_WAVE, kt, stage_off);
  };

  constexpr bool kBiasInit = EPI == EPI_ACT || EPI == EPI_GELU || EPI == EPI_RESID;
  f32x16 acc[FM][FN];
  h16x8 fa[2][FM], fb[2][FN];
  auto read_a = [&](int buf, int i, const h16* st, int kk) {
    fa[buf][i] = frag<A_K, BM, BK>(st, wm * WTM + i * 32, kk, lane);
  };
  auto read_b = [&](int buf, int j, const h16* st, int kk) {
    fb[buf][j] = frag<B_K, BN, BK>(st + BM * BK, wn * WTN + j * 32, kk, lane);
  };

  // GELU': the wave's gelu'(u) tile (read by the epilogue) is loaded into
  // registers during the k-loop, a share after each k-tile barrier (which
  // waits for the share before), so that its HBM reads overlap the MFMAs
  // instead of following them.  Only where the registers allow it.
  constexpr int CPR = WTN / 8, NA = WTM * CPR / 64;  // 16-byte loads per lane
  constexpr bool kAuxPre = EPI == EPI_GELU_BWD && 4 * NA <= 48;
  u32x4 auxr[kAuxPre ? NA : 1];
  auto aux_load = [&](int j) {
    const int q = j * 64 + lane, r = q / CPR, c = q % CPR;
    const int m = m0 + wm * WTM + r, n = n0 + wn * WTN + 8 * c;
    auxr[j] = ld16_or_zero(reinterpret_cast<const h16*>(p.aux) + (int64_t)m * p.ldc + n, m < p.M && n < p.N);
  };
  auto aux_share = [&](int kt) {  // k-tiles 0 .. nkt-2 each load their share
    const int lo = kt * NA / (nkt - 1), hi = (kt + 1) * NA / (nkt - 1);
#pragma unroll
    for (int j = 0; j < NA; ++j)
      if (j >= lo && j < hi) aux_load(j);
  };

  // A k-tile's direct loads go out in S chunks: chunk 0 in the last 16-k step
  // of the k-tile two before it (its stage has just been freed), chunks 1..S-1
  // in the first S-1 16-k steps of the k-tile before it (before that k-tile's
  // barrier, which waits for them).  Spreading them smooths the request
  // stream into L2: a whole k-tile of loads from every CU at once queues up
  // there and raises the load latency.
  constexpr int S = kW4LoadChunks;
  // first load of chunk c (chunk 0 holds C0 loads)
  constexpr int C0 = LPW / S;
  auto chunk_lo = [](int c) { return c * LPW / S; };
  auto dma_chunk = [&](int c, int g, int kt_load, uint32_t stage_off) {
    const int lo = chunk_lo(c), hi = chunk_lo(c + 1);
#pragma unroll
    for (int d = lo + g * (hi - lo) / G; d < lo + (g + 1) * (hi - lo) / G; ++d) dma(d, kt_load, stage_off);
  };

  // One k-tile.  NEXT: k-tile kt + 1 exists (its chunks 1..S-1 are loaded in
  // the first 16-k steps, its fragments read in the last one); LOAD: k-tile
  // kt + 2 exists (its chunk 0 is loaded into this k-tile's stage once every
  // wave is past the barrier).
  auto ktile = [&](auto next_c, auto load_c, int kt) {
    constexpr bool NEXT = decltype(next_c)::value, LOAD = decltype(load_c)::value;
    const h16* cur = smem + (kt & 1) * STAGE;
    const h16* nxt = smem + ((kt + 1) & 1) * STAGE;
    const uint32_t cur_off = (kt & 1) * kStageBytes, nxt_off = ((kt + 1) & 1) * kStageBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cb = kk & 1;
      if (kk == 3 && NEXT) {
        // k-tile kt + 1 has landed for every wave, and every wave holds the
        // fragments of this last 16-k step: the stage of k-tile kt is free
        wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xc07f);
        lds_barrier();
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int i = g / FN, j = g % FN;
        acc[i][j] = mfma32(fb[cb][j], fa[cb][i], acc[i][j]);
        if (kk < 3) {
          if (g < FM) read_a(cb ^ 1, g, cur, kk + 1);
          else if (g < FM + FN) read_b(cb ^ 1, g - FM, cur, kk + 1);
          if (NEXT && kk < S - 1) dma_chunk(kk + 1, g, kt + 1, nxt_off);
        } else if (NEXT) {
          if (g < FM) read_a(cb ^ 1, g, nxt, 0);
          else if (g < FM + FN) read_b(cb ^ 1, g - FM, nxt, 0);
          if (LOAD) dma_chunk(0, g, kt + 2, cur_off);
          if constexpr (kAuxPre) {
            if (g == G - 1) aux_share(kt);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // every split has at least one k-tile (the host requires K = splits x
  // k_per_split with k_per_split a positive multiple of 64).  First tile:
  // k-tile 0 whole, chunk 0 of k-tile 1 (the rest follows in k-tile 0's
  // steps).
  setup();
#pragma unroll
  for (int d = 0; d < LPW; ++d) dma(d, 0, 0);
  if (nkt > 1) {
#pragma unroll
    for (int d = 0; d < C0; ++d) dma(d, 1, kStageBytes);
  }
  for (;;) {
    // k-tile 0 has landed (and the previous tile's stores have gone out)
    if (nkt > 1) wait_vmcnt<C0>();
    else wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kBiasInit) {
          const int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);
          if (p.bias && n < p.N && split == 0) load4(p.bias + n, b);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = b[e];
      }
#pragma unroll
    for (int i = 0; i < FM; ++i) read_a(0, i, smem, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) read_b(0, j, smem, 0);
    int kt = 0;
    for (; kt + 2 < nkt; ++kt) ktile(std::true_type{}, std::true_type{}, kt);
    if (kt + 1 < nkt) ktile(std::true_type{}, std::false_type{}, kt++);
    ktile(std::false_type{}, std::false_type{}, kt);

    GemmArgs pe = p;
    if constexpr (kBiasInit) pe.bias = nullptr;  // already in the accumulators
    const int am0 = m0 + wm * WTM, an0 = n0 + wn * WTN, esplit = split;
    const bool more = next(tm, tn, split);
    __syncthreads();  // all waves are done reading the operand stages
    if constexpr (kAuxPre) {
      if (nkt < 2) {  // no k-tile barrier carried the loads
#pragma unroll
        for (int j = 0; j < NA; ++j) aux_load(j);
      }
    }
    if (more) {  // the next tile's first k-tile, into stage 0
      setup();
#pragma unroll
      for (int d = 0; d < LPW; ++d) dma(d, 0, 0);
    }
    if constexpr (epi_staged<EPI>()) {
      const u32x4* aux_pre = nullptr;
      if constexpr (kAuxPre) aux_pre = auxr;
      if constexpr (PERSIST)
        gemm_epilogue<EPI, FM, FN, true, 32>(pe, acc, smem + STAGE + wave * 32 * SLD, am0, an0, lane, esplit, aux_pre);
      else
        gemm_epilogue<EPI, FM, FN, true>(pe, acc, smem + wave * WTM * SLD, am0, an0, lane, esplit, aux_pre);
    } else {
      gemm_epilogue<EPI, FM, FN, false>(pe, acc, nullptr, am0, an0, lane, esplit);
    }
    if (!more) break;
    // the loaders again: the same values, but nothing of them stays live
    // across the epilogue
    setup();
    if (nkt > 1) {
      __syncthreads();  // every wave is done with its staging rows in stage 1
#pragma unroll
      for (int d = 0; d < C0; ++d) dma(d, 1, kStageBytes);
    }
  }
}

// The single tile (tm, tn, split).
struct OneTile {
  int tm, tn, split;
  bool done;
  DEVI bool operator()(int& a, int& b, int& s) {
    if (done) return false;
    a = tm;
    b = tn;
    s = split;
    done = true;
    return true;
  }
};

template <bool A_K, bool B_K, int BM, int BN, int EPI, int OCC = 1, int NW = 4>
__global__ __launch_bounds__(64 * NW, OCC) void gemm_w4_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) h16 smem[w4_lds_elems<BM, BN, false, NW>()];
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn, split;
  tile_coords(p, tiles_m, tiles_n, blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y, tm, tn, split);
  w4_tiles<A_K, B_K, BM, BN, EPI, false, NW>(p, smem, OneTile{tm, tn, split, false});
}

// Persistent form (one k-split): a grid of 8 n workgroups, n per XCD (they
// are dealt to the XCDs round-robin).  XCD x owns the contiguous range of
// tiles tile_coords gives it; its workgroup w takes the tiles w, w + n,
// w + 2n, ... of that range, so that at any moment the XCD works on
// neighbouring tiles as the one-tile-per-workgroup grid does.
template <bool A_K, bool B_K, int BM, int BN, int EPI, int OCC = 1, int NW = 4>
__global__ __launch_bounds__(64 * NW, OCC) void gemm_w4p_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) h16 smem[w4_lds_elems<BM, BN, true, NW>()];
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  constexpr int NX = 8;
  const int x = blockIdx.x % NX, w = blockIdx.x / NX, nw = gridDim.x / NX;
  const int start = x * (total / NX) + min(x, total % NX);
  const int count = total / NX + (x < total % NX ? 1 : 0);
  int j = 0;
  auto next = [&](int& tm, int& tn, int& split) {
    const int local = w + j * nw;
    if (local >= count) return false;
    ++j;
    tile_walk(p, tiles_m, tiles_n, start + local, tm, tn);
    split = 0;
    return true;
  };
  w4_tiles<A_K, B_K, BM, BN, EPI, true, NW>(p, smem, next);
}

// The grouped launch runs eight waves per workgroup, two per SIMD, each a
// 64 x 128 block of the shared 256 x 256 tile (measured on MI355X: 1.4%
// faster than four waves of 128 x 128; the products are bitwise the same).
constexpr int kGroupWaves = 8;

// Many independent products in one launch (weight gradients of a whole
// backward pass: fp32 C += A^T B, both operands stored [K][rows]).  Each XCD
// works through a contiguous range of the tiles; tile t belongs to the
// problem with first[j] <= t < first[j + 1].
//
// Tile t of a grouped launch: its problem's arguments and tile coordinates
// (within a problem, tiles walk groups of GM tile-rows as in tile_coords).
template <int BM, int BN>
DEVI void group_tile(const GemmGroup& grp, int t, GemmArgs& p, int& tm, int& tn) {
  int j = 0;
  while (j + 1 < grp.n && t >= grp.first[j + 1]) ++j;
  const GemmProblem& pr = grp.prob[j];
  p = {};
  p.A = pr.A;
  p.B = pr.B;
  p.C = pr.C;
  p.M = pr.M;
  p.N = pr.N;
  p.K = pr.K;
  p.lda = pr.lda;
  p.ldb = pr.ldb;
  p.ldc = pr.N;
  p.splits = 1;
  p.k_per_split = pr.K;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int local = t - grp.first[j];
  constexpr int GM = 8;
  const int g = local / (GM * tiles_n);
  const int first_m = g * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int w = local - g * GM * tiles_n;
  tm = first_m + w % gm;
  tn = w / gm;
}

template <int BM, int BN>
__global__ __launch_bounds__(64 * kGroupWaves, 1) void gemm_w4_group_kernel(GemmGroup grp) {
  __shared__ __attribute__((aligned(1024))) h16 smem[w4_lds_elems<BM, BN, false, kGroupWaves>()];
  // block b runs on XCD b % 8 as that XCD's idx-th workgroup: its whole
  // tiles first, then the K halves of its split tail tiles
  const int x = blockIdx.x % kGroupXcds, idx = blockIdx.x / kGroupXcds;
  const int whole = grp.xcount[x] - grp.xsplit[x];
  GemmArgs p;
  int tm, tn;
  if (idx < whole) {
    group_tile<BM, BN>(grp, grp.xstart[x] + idx, p, tm, tn);
    w4_tiles<false, false, BM, BN, EPI_F32_ACC, false, kGroupWaves>(p, smem, OneTile{tm, tn, 0, false});
  } else if (idx < whole + 2 * grp.xsplit[x]) {
    const int u = idx - whole, half = u & 1;
    group_tile<BM, BN>(grp, grp.xstart[x] + whole + (u >> 1), p, tm, tn);
    // the tile as tile (0, 0) of the BM x BN problem at its origin (both
    // operands are stored [K][rows]), its half's partial into a dense
    // BM x BN block of its slot
    const int64_t slot = (int64_t)x * kGroupTailMax + (u >> 1);
    p.A = reinterpret_cast<const h16*>(p.A) + (int64_t)tm * BM;
    p.B = reinterpret_cast<const h16*>(p.B) + (int64_t)tn * BN;
    p.M = min(BM, p.M - tm * BM);
    p.N = min(BN, p.N - tn * BN);
    p.splits = 2;
    p.k_per_split = p.K / 2;
    p.ldc = BN;
    p.split_stride = (int64_t)BM * BN;
    p.C = grp.part + slot * 2 * BM * BN;
    w4_tiles<false, false, BM, BN, EPI_PARTIAL, false, kGroupWaves>(p, smem, OneTile{0, 0, half, false});
  }
}

// C += first half + second half, for every split tail tile (fixed order);
// kTailRowBlocks workgroups per tile, each a band of rows
constexpr int kTailRowBlocks = 8;
template <int BM, int BN>
__global__ __launch_bounds__(256) void group_tail_reduce_kernel(GemmGroup grp) {
  const int band = blockIdx.x % kTailRowBlocks, slot = blockIdx.x / kTailRowBlocks;
  const int x = slot / kGroupTailMax, i = slot % kGroupTailMax;
  if (i >= grp.xsplit[x]) return;
  GemmArgs p;
  int tm, tn;
  group_tile<BM, BN>(grp, grp.xstart[x] + grp.xcount[x] - grp.xsplit[x] + i, p, tm, tn);
  const float* p0 = grp.part + ((int64_t)x * kGroupTailMax + i) * 2 * BM * BN;
  const float* p1 = p0 + BM * BN;
  float* c = reinterpret_cast<float*>(p.C);
  constexpr int ROWS = BM / kTailRowBlocks;
  for (int e = threadIdx.x; e < ROWS * BN / 4; e += blockDim.x) {
    const int r = band * ROWS + e / (BN / 4), c4 = (e % (BN / 4)) * 4;
    const int m = tm * BM + r, n = tn * BN + c4;
    if (m < p.M && n < p.N) {
      float a[4], b[4], o[4];
      load4(p0 + r * BN + c4, a);
      load4(p1 + r * BN + c4, b);
      float* cp = c + (int64_t)m * p.N + n;
      load4(cp, o);
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] += a[k] + b[k];
      store4(cp, o);
    }
  }
}

// -------------------------------------------------------------- fp32 GEMM ----
template <bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  constexpr int BT = 64, BK = 16;
  __shared__ float As[BK][BT + 4];
  __shared__ float Bs[BK][BT + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (p.N + BT - 1) / BT;
  const int m0 = (blockIdx.x / tiles_n) * BT, n0 = (blockIdx.x % tiles_n) * BT;
  const int split = blockIdx.y;
  const int kbeg = split * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const float* A = reinterpret_cast<const float*>(p.A);
  const float* B = reinterpret_cast<const float*>(p.B);
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = tid + 256 * r;
      int mm, kk, nn, kb;
      if (A_K) { mm = e / BK; kk = e % BK; } else { mm = e % BT; kk = e / BT; }
      const int gm = m0 + mm, gk = k0 + kk;
      float av = 0.f;
      if (gm < p.M && gk < kend) av = A_K ? A[(int64_t)gm * p.lda + gk] : A[(int64_t)gk * p.lda + gm];
      As[kk][mm] = av;
      if (B_K) { nn = e / BK; kb = e % BK; } else { nn = e % BT; kb = e / BT; }
      const int gn = n0 + nn, gk2 = k0 + kb;
      float bv = 0.f;
      if (gn < p.N && gk2 < kend) bv = B_K ? B[(int64_t)gn * p.ldb + gk2] : B[(int64_t)gk2 * p.ldb + gn];
      Bs[kb][nn] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const bool vec = (p.ldc % 4 == 0) && (p.N % 4 == 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i, n = n0 + tx * 4;
    if (m >= p.M || n >= p.N) continue;
    if (vec) {
      epi_store4<EPI, float>(p, m, n, acc[i], split);
    } else {
      for (int j = 0; j < 4 && n + j < p.N; ++j) epi_store1<EPI, float>(p, m, n + j, acc[i][j], split);
    }
  }
}

// ----------------------------------------------------------- split-K reduce ----
__global__ void splitk_reduce_kernel(float* out, const float* part, int splits, int64_t stride, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  float a[4];
  load4(out + 4 * i, a);
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < splits; ++k) {
    float t[4];
    load4(part + k * stride + 4 * i, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += t[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] += s[e];
  store4(out + 4 * i, a);
}

void splitk_reduce_add(float* out, const float* part, int splits, int64_t stride, int64_t count,
                       hipStream_t s) {
  const int64_t n4 = count / 4;
  splitk_reduce_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(out, part, splits, stride, n4);
}

// ---------------------------------------------------------------- dispatch ----
namespace {
constexpr int kBK = 64;

// Tile configurations (block tile BM x BN, wave grid WGM x WGN).
#ifndef GPT2_W4_PERSIST
#define GPT2_W4_PERSIST 1
#endif
// Workgroups per XCD of the persistent one-wave-per-SIMD launch (one per
// resident slot: CUs per XCD x occupancy), or 0 for the one-tile-per-
// workgroup grid: k-splits, the hardware block order, or fewer than two
// tiles per workgroup (nothing to overlap).
// The GELU' epilogue keeps the one-tile grid: its persistent form either
// spills registers (gelu'(u) carried through the k-loop) or, loading those
// rows in the epilogue, ran 6% slower on MI355X.  So does the residual add
// on the largest tile (it spills).
template <int EPI, int BM, int BN>
constexpr bool w4_persist_ok() {
  return EPI != EPI_GELU_BWD && !(EPI == EPI_RESID && BM * BN > 256 * 192);
}
int w4_persistent_per_xcd(int occ, int tiles, const GemmArgs& a) {
  if (!GPT2_W4_PERSIST || a.splits != 1 || a.no_xcd_map) return 0;
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n = 256;
    cus = n;
  }
  const int nw = std::max(1, cus / 8) * occ;
  return tiles >= 2 * 8 * nw ? nw : 0;
}

template <bool A_K, bool B_K, int EPI>
void launch_bf16_cfg(int cfg, const GemmArgs& a, hipStream_t s) {
#define GPT2_GEMM_CFG(ID, BM, BN, WGM, WGN)                                                     \
  case ID: {                                                                                   \
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);                           \
    gemm_bf16_kernel<A_K, B_K, BM, BN, kBK, WGM, WGN, EPI><<<dim3(tiles, a.splits), 64 * WGM * WGN, 0, s>>>(a); \
    break;                                                                                     \
  }
  switch (cfg) {
    GPT2_GEMM_CFG(0, 128, 128, 2, 2)
    GPT2_GEMM_CFG(1, 256, 128, 2, 2)
    GPT2_GEMM_CFG(2, 256, 256, 2, 2)
    GPT2_GEMM_CFG(3, 256, 192, 2, 2)
    GPT2_GEMM_CFG(4, 256, 256, 2, 4)
    GPT2_GEMM_CFG(5, 128, 256, 2, 2)
    default: break;
  }
#undef GPT2_GEMM_CFG
#define GPT2_GEMM_LDS(ID, BM, BN, BK, WGM, WGN, NST, OCC)                                       \
  case ID: {                                                                                   \
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);                           \
    gemm_lds_kernel<A_K, B_K, BM, BN, BK, WGM, WGN, NST, EPI, OCC>                             \
        <<<dim3(tiles, a.splits), 64 * WGM * WGN, 0, s>>>(a);                                  \
    break;                                                                                     \
  }
  switch (cfg) {
    GPT2_GEMM_LDS(6, 256, 256, 32, 2, 2, 4, 1)
    GPT2_GEMM_LDS(7, 256, 256, 32, 2, 4, 4, 1)
    GPT2_GEMM_LDS(8, 256, 256, 64, 2, 4, 2, 1)
    GPT2_GEMM_LDS(9, 256, 128, 32, 2, 2, 4, 1)
    GPT2_GEMM_LDS(10, 128, 256, 32, 2, 2, 4, 1)
    GPT2_GEMM_LDS(11, 256, 192, 32, 2, 2, 4, 1)
    GPT2_GEMM_LDS(12, 128, 128, 32, 2, 2, 4, 1)
    GPT2_GEMM_LDS(13, 256, 256, 64, 2, 2, 2, 1)
    GPT2_GEMM_LDS(14, 256, 256, 32, 2, 4, 3, 1)
    GPT2_GEMM_LDS(15, 256, 192, 64, 4, 2, 2, 1)
    GPT2_GEMM_LDS(16, 256, 128, 64, 4, 2, 3, 1)
    GPT2_GEMM_LDS(17, 128, 256, 64, 2, 4, 3, 1)
    GPT2_GEMM_LDS(18, 256, 256, 64, 4, 2, 2, 1)
    GPT2_GEMM_LDS(19, 128, 192, 64, 2, 2, 2, 2)  // two workgroups per CU
    default: break;
  }
#undef GPT2_GEMM_LDS
#define GPT2_GEMM_W4(ID, BM, BN, OCC, NW)                                                       \
  case ID: {                                                                                   \
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);                           \
    if constexpr (w4_persist_ok<EPI, BM, BN>()) {                                             \
      const int nw = w4_persistent_per_xcd(OCC, tiles, a);                                    \
      if (nw > 0) {                                                                            \
        gemm_w4p_kernel<A_K, B_K, BM, BN, EPI, OCC, NW><<<dim3(8 * nw), 64 * NW, 0, s>>>(a);   \
        break;                                                                                 \
      }                                                                                        \
    }                                                                                          \
    gemm_w4_kernel<A_K, B_K, BM, BN, EPI, OCC, NW><<<dim3(tiles, a.splits), 64 * NW, 0, s>>>(a); \
    break;                                                                                     \
  }
  switch (cfg) {
    GPT2_GEMM_W4(20, 256, 256, 1, 4)
    GPT2_GEMM_W4(21, 256, 192, 1, 4)
    GPT2_GEMM_W4(22, 128, 192, 2, 4)  // two workgroups per CU
    default: break;
  }
#undef GPT2_GEMM_W4
}
constexpr int kNumCfg = 23;
constexpr int kFirstLds = 6;
const int kCfgBM[kNumCfg] = {128, 256, 256, 256, 256, 128, 256, 256, 256, 256, 128, 256, 128, 256, 256, 256, 256, 128, 256, 128, 256, 256, 128};
const int kCfgBN[kNumCfg] = {128, 128, 256, 192, 256, 256, 256, 256, 256, 128, 256, 192, 128, 256, 256, 192, 128, 256, 256, 192, 256, 192, 192};
const int kCfgBK[kNumCfg] = {64, 64, 64, 64, 64, 64, 32, 32, 64, 32, 32, 32, 32, 64, 32, 64, 64, 64, 64, 64, 64, 64, 64};

template <bool A_K, bool B_K, int EPI>
void launch_f32(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + 63) / 64) * ((a.N + 63) / 64);
  dim3 grid(tiles, a.splits);
  gemm_f32_kernel<A_K, B_K, EPI><<<grid, 256, 0, s>>>(a);
}
template <bool A_K, bool B_K, int EPI>
void launch(bool bf16_mode, int cfg, const GemmArgs& a, hipStream_t s) {
  if (bf16_mode) launch_bf16_cfg<A_K, B_K, EPI>(cfg, a, s);
  else launch_f32<A_K, B_K, EPI>(a, s);
}

// Picks the tile configuration with the least modelled time: a sustained
// rate per configuration (measured on MI355X for these kernels) scaled by the
// fill of the last wave of blocks over the 256 CUs and by the padding of
// partial tiles.
double model_time(int c, const GemmArgs& a, bool transposed_a) {
  // sustained TFLOP/s at full waves; 13 spills registers and is never chosen;
  // 22 is never chosen for weight gradients (measured slower in the step
  // than in isolation: its split-K partials compete with the other
  // workgroup on the CU)
  static const double tf_k[kNumCfg] = {560, 480, 650, 720, 750, 500, 750, 800, 880, 650, 650, 930, 820,
                                        1, 820, 1020, 760, 760, 900, 1, 1090, 1060, 1040};  // A k-contiguous
  static const double tf_t[kNumCfg] = {450, 460, 660, 560, 640, 380, 860, 880, 950, 740, 740, 900, 820,
                                        1, 950, 930, 850, 900, 930, 1, 1080, 1000, 1};   // A transposed
  const int64_t tm = (a.M + kCfgBM[c] - 1) / kCfgBM[c], tn = (a.N + kCfgBN[c] - 1) / kCfgBN[c];
  const double waves = (double)(tm * tn * a.splits) / 256.0;
  const double fill = waves / std::ceil(waves);
  const double used = (double)a.M * a.N / ((double)tm * kCfgBM[c] * tn * kCfgBN[c]);
  const double flops = 2.0 * a.M * (double)a.N * a.K;
  return flops / ((transposed_a ? tf_t[c] : tf_k[c]) * 1e12 * fill * used);
}
int choose_cfg(const GemmArgs& a, GemmLayout layout) {
  int pick = 0;
  double best = 1e30;
  for (int c = 0; c < kNumCfg; ++c) {
    if (!gemm_config_usable(c, layout, a)) continue;
    const double t = model_time(c, a, layout == LAYOUT_TN);
    if (t < best) {
      best = t;
      pick = c;
    }
  }
  return pick;
}
}  // namespace

bool gemm_group_ok(const GemmProblem& p) {
  return p.M > 0 && p.N > 0 && p.K > 0 && p.K % 64 == 0 && p.M % 8 == 0 && p.N % 8 == 0 && p.lda % 8 == 0 &&
         p.ldb % 8 == 0;
}

// 256 x 256 tiles: fewer operand bytes per flop than 256 x 192 (the stream
// from L2 bounds these long-K products), at a slightly coarser last wave.
constexpr int kGroupBM = 256, kGroupBN = 256;

// CUs per XCD of the current device (256 CUs in 8 XCDs on MI355X)
static int cus_per_xcd() {
  static int v = 0;
  if (v == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    v = std::max(1, cus / kGroupXcds);
  }
  return v;
}

void gemm_group_tn_acc(const GemmProblem* probs, int n, float* part, int64_t part_elems, hipStream_t s) {
  auto tiles_of = [](const GemmProblem& p) {
    return ((p.M + kGroupBM - 1) / kGroupBM) * ((p.N + kGroupBN - 1) / kGroupBN);
  };
  int64_t total = 0;
  for (int j = 0; j < n; ++j) total += tiles_of(probs[j]);
  const int cpx = cus_per_xcd();
  const int64_t tail_cap = part ? part_elems / (2LL * kGroupBM * kGroupBN) / kGroupXcds : 0;
  const int tail_max = (int)std::min<int64_t>(kGroupTailMax, tail_cap);
  // launches of at most kGroupMax problems, each cut once its running tile
  // count passes an equal share (a launch with a few tiles would idle most
  // CUs) but never leaving more problems than the later launches can take
  const int launches = (n + kGroupMax - 1) / kGroupMax;
  int j0 = 0;
  int64_t done = 0;
  for (int li = 0; li < launches; ++li) {
    const int64_t target = total * (li + 1) / launches;
    const int min_count = std::max(1, (n - j0) - (launches - 1 - li) * kGroupMax);
    const int max_count = std::min(kGroupMax, n - j0);
    GemmGroup g;
    g.n = 0;
    int tiles = 0;
    bool halves_ok = true;  // every K splits into two whole-k-tile halves
    while (g.n < max_count && (g.n < min_count || done < target || li == launches - 1)) {
      g.prob[g.n] = probs[j0 + g.n];
      g.first[g.n] = tiles;
      tiles += tiles_of(probs[j0 + g.n]);
      done += tiles_of(probs[j0 + g.n]);
      halves_ok = halves_ok && probs[j0 + g.n].K % (2 * kBK) == 0;
      ++g.n;
    }
    j0 += g.n;
    if (tiles == 0) break;
    // each XCD takes a contiguous range of tiles; a last round of r <= cpx/2
    // tiles becomes 2r K halves, which finish in about half a round
    g.part = part;
    int per_xcd = 0;
    bool any_split = false;
    for (int x = 0; x < kGroupXcds; ++x) {
      g.xstart[x] = x * (tiles / kGroupXcds) + std::min(x, tiles % kGroupXcds);
      g.xcount[x] = tiles / kGroupXcds + (x < tiles % kGroupXcds ? 1 : 0);
      const int r = g.xcount[x] % cpx;
      g.xsplit[x] = (halves_ok && r > 0 && 2 * r <= cpx && r <= tail_max) ? r : 0;
      any_split = any_split || g.xsplit[x] > 0;
      per_xcd = std::max(per_xcd, g.xcount[x] + g.xsplit[x]);
    }
    gemm_w4_group_kernel<kGroupBM, kGroupBN><<<per_xcd * kGroupXcds, 64 * kGroupWaves, 0, s>>>(g);
    if (any_split)
      group_tail_reduce_kernel<kGroupBM, kGroupBN><<<kGroupXcds * kGroupTailMax * kTailRowBlocks, 256, 0, s>>>(g);
  }
}

int gemm_pick_config(const GemmArgs& a, GemmLayout layout) { return choose_cfg(a, layout); }

bool gemm_config_usable(int cfg, GemmLayout layout, const GemmArgs& a) {
  if (cfg < 0 || cfg >= kNumCfg || cfg == 13) return false;
  if (cfg >= kFirstLds) {
    // whole k-tiles, and every split the same length (the persistent walk
    // gives each tile the same number of k-steps)
    if (a.K % kCfgBK[cfg] || a.k_per_split % kCfgBK[cfg]) return false;
    if (a.splits > 1 && a.K != a.splits * a.k_per_split) return false;
    // the staged epilogue addresses a pass of at most 256 output rows with
    // 32-bit element offsets
    if (a.ldc >= (int64_t(1) << 24)) return false;
  }
  return true;
}

double gemm_model_time(int cfg, const GemmArgs& a, bool transposed_a) { return model_time(cfg, a, transposed_a); }

void gemm_config_tile(int cfg, int* bm, int* bn) {
  *bm = (cfg >= 0 && cfg < kNumCfg) ? kCfgBM[cfg] : 128;
  *bn = (cfg >= 0 && cfg < kNumCfg) ? kCfgBN[cfg] : 128;
}

int gemm_resolve_config(int cfg, GemmLayout layout, GemmEpilogue epi, bool bf16_mode, const GemmArgs& a0) {
  GemmArgs a = a0;
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return -1;
  if (a.splits < 1) a.splits = 1;
  if (a.splits == 1) a.k_per_split = a.K;
  if (a.splits > 1 && (a.k_per_split % kBK) != 0) return -1;
  if (!bf16_mode) return kGemmCfgF32;
  // 16-byte operand accesses: k-contiguous and transposed dims are multiples of 8;
  // the epilogue writes four columns at a time.
  if (a.K % 8 || a.N % 8 || a.ldc % 4 || a.lda % 8 || a.ldb % 8) return -1;
  if (layout == LAYOUT_TN && a.M % 8) return -1;
  if (cfg < 0) {
    // Epilogues that do per-element work on bf16 activations (bias, GELU,
    // GELU') and short-K products (K <= 1024: a dozen k-tiles per output
    // tile) are bound by the time outside the k-loop; the 128 x 192 tile at
    // two workgroups per CU (config 22) lets one workgroup's prologue and
    // epilogue run beside the other's k-loop (measured on MI355X: 3-10%
    // faster than config 19 and 5-18% faster than the one-workgroup tiles
    // for these GEMMs).  So does the residual add (its fp32 read-modify-
    // write epilogue; measured on MI355X with K = 4C: 3.8% faster than the
    // 256 x 192 tile).  The lm_head product (K = C but 50k columns) keeps
    // the one-workgroup tiles, and so do the long-K input gradients (the
    // 128 x 192 tile measured 5% slower on the lm_head one).
    const bool heavy_epi =
        (epi == EPI_ACT && a.bias) || epi == EPI_GELU || epi == EPI_GELU_BWD || epi == EPI_RESID;
    const bool short_k = a.K <= 1024 && epi != EPI_LOGITS;
    if ((heavy_epi || short_k) && gemm_config_usable(22, layout, a)) cfg = 22;
    else if (heavy_epi && gemm_config_usable(19, layout, a)) cfg = 19;
    else cfg = choose_cfg(a, layout);
  }
  return gemm_config_usable(cfg, layout, a) ? cfg : -1;
}

bool gemm_cfg(int cfg, GemmLayout layout, GemmEpilogue epi, bool bf16_mode, const GemmArgs& a0, hipStream_t s) {
  cfg = gemm_resolve_config(cfg, layout, epi, bf16_mode, a0);
  if (cfg < 0) return false;
  GemmArgs a = a0;
  if (a.splits < 1) a.splits = 1;
  if (a.splits == 1) a.k_per_split = a.K;
  // column-sum partials: formed in the epilogue by the one-wave-per-SIMD
  // tiles (their wave tiles span whole 64-row chunks), else by a pass over C
  float* const colsum = epi == EPI_GELU_BWD ? a.colsum : nullptr;
  if (colsum && a.ldc != a.N) return false;
  const bool fused_colsum = colsum && bf16_mode && cfg >= 20 && cfg <= 22;
  if (!fused_colsum) a.colsum = nullptr;
  switch (layout) {
    case LAYOUT_NT:
      if (epi == EPI_ACT) launch<true, true, EPI_ACT>(bf16_mode, cfg, a, s);
      else if (epi == EPI_LOGITS) launch<true, true, EPI_LOGITS>(bf16_mode, cfg, a, s);
      else if (epi == EPI_RESID) launch<true, true, EPI_RESID>(bf16_mode, cfg, a, s);
      else if (epi == EPI_GELU) launch<true, true, EPI_GELU>(bf16_mode, cfg, a, s);
      else if (epi == EPI_F32) launch<true, true, EPI_F32>(bf16_mode, cfg, a, s);
      else return false;
      break;
    case LAYOUT_NN:
      if (epi == EPI_F32) launch<true, false, EPI_F32>(bf16_mode, cfg, a, s);
      else if (epi == EPI_GELU_BWD) launch<true, false, EPI_GELU_BWD>(bf16_mode, cfg, a, s);
      else if (epi == EPI_ACT) launch<true, false, EPI_ACT>(bf16_mode, cfg, a, s);
      else return false;
      break;
    case LAYOUT_TN:
      if (epi == EPI_PARTIAL) launch<false, false, EPI_PARTIAL>(bf16_mode, cfg, a, s);
      else if (epi == EPI_F32_ACC) launch<false, false, EPI_F32_ACC>(bf16_mode, cfg, a, s);
      else if (epi == EPI_F32) launch<false, false, EPI_F32>(bf16_mode, cfg, a, s);
      else return false;
      break;
  }
  if (colsum && !fused_colsum) {
    if (bf16_mode) colsum_partials<h16>(reinterpret_cast<const h16*>(a.C), a.M, a.N, colsum, s);
    else colsum_partials<float>(reinterpret_cast<const float*>(a.C), a.M, a.N, colsum, s);
  }
  return true;
}

bool gemm(GemmLayout layout, GemmEpilogue epi, bool bf16_mode, const GemmArgs& a, hipStream_t s) {
  return gemm_cfg(-1, layout, epi, bf16_mode, a, s);
}

}  // namespace gpt2k
