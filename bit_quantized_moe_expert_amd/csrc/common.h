// Device-side helpers shared by the gfx950 kernels of libnf4moe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Decode tables (index = 4-bit code).
// NF4: the 16-entry NormalFloat codebook, i.e. the QLoRA construction (normal
// quantiles at offset 0.9677083, 8 positive, 7 negative, plus 0, divided by
// the largest), rounded to fp32. The pages name this codebook (grouped-nf4-gemm
// PKG-INFO intro; "How do I run a grouped GEMM directly on NF4 packed MoE
// expert weights ...", section "Why it happens") without printing it.
// MXFP4: OCP e2m1 values; bit 3 = sign ("The MXFP4 native-byte lane").
// ---------------------------------------------------------------------------
__host__ __device__ constexpr float nf4_value(int code) {
  constexpr float t[16] = {
      -0x1.000000p+0f, -0x1.647362p-1f, -0x1.0cd65cp-1f, -0x1.94653cp-2f,
      -0x1.234496p-2f, -0x1.7a6a7ap-3f, -0x1.74f0d2p-4f, 0.0f,
      0x1.45f602p-4f,  0x1.4995bep-3f,  0x1.f809b4p-3f,  0x1.5a066cp-2f,
      0x1.c3496ap-2f,  0x1.200f52p-1f,  0x1.722760p-1f,  0x1.000000p+0f};
  return t[code & 15];
}

__host__ __device__ constexpr float e2m1_value(int code) {
  constexpr float t[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                           -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};
  return t[code & 15];
}

// Value of the code stored at even k (first) and odd k (second) of a byte.
// NF4 keeps the even-k code in the high nibble, MXFP4 in the low nibble.
template <int FMT>
__host__ __device__ constexpr float even_value(uint32_t byte) {
  return FMT == 0 ? nf4_value(byte >> 4) : e2m1_value(byte & 15);
}
template <int FMT>
__host__ __device__ constexpr float odd_value(uint32_t byte) {
  return FMT == 0 ? nf4_value(byte & 15) : e2m1_value(byte >> 4);
}

// Block size of the scale along K and bytes per scale.
template <int FMT> struct Fmt;
template <> struct Fmt<0> { static constexpr int kBlock = 64; };
template <> struct Fmt<1> { static constexpr int kBlock = 32; };

// Scale of one block as an fp32 multiplier. NF4: the stored fp32 absmax.
// MXFP4: 2^(e8m0 - 127), e8m0 = 255 -> NaN.
__device__ inline float e8m0_to_f32(uint32_t e) {
  if (e == 255u) return __builtin_nanf("");
  if (e == 0u) return 0x1p-127f;               // the one subnormal power of two
  return __uint_as_float(e << 23);
}

// ---------------------------------------------------------------------------
// bf16 helpers (bf16 tensors cross the ABI as uint16 bit patterns)
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ inline float bf16lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ inline float bf16hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ inline uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;   // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes). Every lane receives the result.
// ---------------------------------------------------------------------------
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Max over the 32-lane half a lane belongs to.
__device__ inline float half_max(float v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ inline uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------------------
// LDS decode table: byte -> (value of even-k code, value of odd-k code) as two
// fp32, replicated kRep times so the lanes of one LDS access read distinct
// banks. Entry (byte b, replica r) lives at float2 index b * kRep + r.
// ---------------------------------------------------------------------------
template <int FMT, int kRep>
__device__ inline void build_pair_table(float2 *tab) {
  for (int i = threadIdx.x; i < 256 * kRep; i += blockDim.x) {
    const uint32_t b = (uint32_t)i / kRep;
    tab[i] = make_float2(even_value<FMT>(b), odd_value<FMT>(b));
  }
}

}  // namespace nf4moe
