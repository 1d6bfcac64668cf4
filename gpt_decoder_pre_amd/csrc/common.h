// Device helpers shared by the gfx950 kernels of the GPT-2 step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// h16: the 16-bit operand type of the MFMA kernels (GEMM operands,
// attention operands, the activations kept for the backward, logits).  It is
// bfloat16, except in the translation units compiled for the fp16 mode
// (GPT2_OPS_F16 defined, namespace gpt2k_f16), where it is IEEE binary16.
#ifdef GPT2_OPS_F16
typedef _Float16 h16;
#else
typedef __bf16 h16;
#endif
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define GPT2_WAVE 64
#define DEVI __device__ __forceinline__

// ---- conversions -----------------------------------------------------------
DEVI float to_f32(float x) { return x; }
DEVI float to_f32(h16 x) { return (float)x; }
template <typename T> DEVI T from_f32(float x);
template <> DEVI float from_f32<float>(float x) { return x; }
template <> DEVI h16 from_f32<h16>(float x) { return (h16)x; }  // round to nearest even

// Load / store four consecutive elements as fp32.
DEVI void load4(const float* p, float v[4]) {
  f32x4 t = *reinterpret_cast<const f32x4*>(p);
  v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
}
DEVI void load4(const h16* p, float v[4]) {
  h16x4 t = *reinterpret_cast<const h16x4*>(p);
  v[0] = (float)t[0]; v[1] = (float)t[1]; v[2] = (float)t[2]; v[3] = (float)t[3];
}
DEVI void store4(float* p, const float v[4]) {
  f32x4 t = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p) = t;
}
DEVI void store4(h16* p, const float v[4]) {
  h16x4 t = {(h16)v[0], (h16)v[1], (h16)v[2], (h16)v[3]};
  *reinterpret_cast<h16x4*>(p) = t;
}

// The two 16-bit values of a 32-bit word (element 0 in the low half) as fp32.
DEVI float lo16_f32(uint32_t w) {
  if constexpr (__is_same(h16, __bf16)) return __builtin_bit_cast(float, w << 16);
  else return (float)__builtin_bit_cast(h16, (uint16_t)(w & 0xffffu));
}
DEVI float hi16_f32(uint32_t w) {
  if constexpr (__is_same(h16, __bf16)) return __builtin_bit_cast(float, w & 0xffff0000u);
  else return (float)__builtin_bit_cast(h16, (uint16_t)(w >> 16));
}

// c + a b on the 32 x 32 x 16 MFMA of the operand type (v_mfma_f32_32x32x16_bf16
// or _f16; fp32 accumulation either way).
DEVI f32x16 mfma32(bf16x8_t a, bf16x8_t b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
DEVI f32x16 mfma32(f16x8_t a, f16x8_t b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }

// acc + a0 b0 + a1 b1 in fp32 (v_dot2c_f32_bf16 / v_dot2_f32_f16)
DEVI float dot2(bf16x2_t a, bf16x2_t b, float acc) { return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false); }
DEVI float dot2(f16x2_t a, f16x2_t b, float acc) { return __builtin_amdgcn_fdot2(a, b, acc, false); }

// Sixteen bytes as fp32 values: four floats, or eight 16-bit values (element
// 2i in the low half of word i).
template <typename T> DEVI void unpack16(u32x4 v, float* f);
template <> DEVI void unpack16<float>(u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // through a scalar: __builtin_bit_cast of a vector element subscript
    // yields element 0 with this compiler
    const uint32_t u = v[i];
    f[i] = __builtin_bit_cast(float, u);
  }
}
template <> DEVI void unpack16<h16>(u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = v[i];
    f[2 * i] = lo16_f32(u);
    f[2 * i + 1] = hi16_f32(u);
  }
}

// ---- math --------------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;   // log2(e)
constexpr float kLn2 = 0.6931471805599453f;     // ln(2)

DEVI float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
DEVI float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

DEVI float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }  // v_rcp_f32

// tanh-form GELU, 0.5 u (1 + tanh(k (u + 0.044715 u^3))), k = sqrt(2/pi),
// evaluated as u * sigmoid(z) with z = 2 k (u + 0.044715 u^3), because
// 0.5 (1 + tanh(z / 2)) = sigmoid(z):  one exp2 and one reciprocal.
// Large |u| saturate cleanly: exp2 -> inf gives sigmoid 0, exp2 -> 0 gives 1.
constexpr float kGeluK = 0.7978845608028654f;  // sqrt(2 / pi)
constexpr float kGeluA = 0.044715f;
constexpr float kGeluZ1 = -2.0f * kGeluK * kLog2e;           // -z / ln 2 per unit u
constexpr float kGeluZ3 = -2.0f * kGeluK * kGeluA * kLog2e;  // ... per unit u^3
DEVI float gelu_sigmoid(float u) {
  const float t = u * u;
  return rcp_fast(1.0f + exp2_fast(u * fmaf(kGeluZ3, t, kGeluZ1)));
}
// gelu(u) and its derivative from one sigmoid:
// d/du [u sigmoid(z)] = s + u s (1 - s) dz/du,  dz/du = 2 k (1 + 3 * 0.044715 u^2)
DEVI void gelu_and_grad(float u, float& g, float& d) {
  const float s = gelu_sigmoid(u);
  const float dz = 2.0f * kGeluK * fmaf(3.0f * kGeluA, u * u, 1.0f);
  g = u * s;
  d = fmaf(g * (1.0f - s), dz, s);
}

// LayerNorm's epsilon inside the square root
constexpr float kLnEps = 1e-5f;

// ---- wave / block reductions ---------------------------------------------------
DEVI float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEVI float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
DEVI double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide sum (blockDim.x a multiple of 64, at most 1024); every thread gets the result.
template <typename T>
DEVI T block_sum(T v, T* scratch /* >= 16 entries */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if constexpr (sizeof(T) == 8) v = wave_sum_d(v); else v = wave_sum(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  T r = 0;
  for (int i = 0; i < nw; ++i) r += scratch[i];  // fixed order
  return r;
}
DEVI float block_max(float v, float* scratch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  float r = -INFINITY;
  for (int i = 0; i < nw; ++i) r = fmaxf(r, scratch[i]);
  return r;
}

// ---- 8x8 16-bit transpose in registers ------------------------------------------
// in[j] holds 8 bf16 of row j (elements 0..7 of that row).  out[e] receives
// the 8 bf16 of column e (element j from row j).
DEVI void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // low half from row 2d, high half from row 2d+1
      out[e][d] = __builtin_amdgcn_perm(in[2 * d + 1][e >> 1], in[2 * d][e >> 1], sel);
    }
  }
}

// 16-byte global load with zero fill when the predicate is false.
DEVI u32x4 ld16_or_zero(const void* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}
