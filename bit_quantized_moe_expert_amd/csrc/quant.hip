// Quantize fp32 weights to NF4 / MXFP4 and decode them back (off the timed path).
//
// NF4 (grouped-nf4-gemm PKG-INFO, "Try it on CPU right now", block 1): per row
// and 64-element K block, absmax = max |w| kept in fp32; each weight becomes
// the code of the nearest codebook value of w / absmax; two codes per byte,
// even k in the high nibble. The nearest code is decided exactly: code =
// #{ i : m_i * absmax < w } with m_i = (c_i + c_{i+1}) / 2, evaluated in fp64
// where both the midpoint and its product with absmax are exact, so a weight
// on a midpoint takes the lower code.
// MXFP4 (same section, block 2; OCP MX v1.0): X = floor(log2 amax) - 2 clamped
// to [-127, 127], e8m0 = X + 127, code = nearest e2m1 of w / 2^X with ties to
// the even code, saturating at 6; code bit 3 is w's sign bit; even k in the
// low nibble.
#include "common.h"
#include "internal.h"

namespace nf4moe {

// One wave per 64-element NF4 block, one lane per element. BF16ABS: the
// absmax is stored as bf16, rounded up to the nearest bf16 value when it is
// not one (exact, and the same codes as the fp32 form, for bf16-source
// weights, whose block maximum is itself a bf16 value), and the codes are
// chosen against that stored value.
template <bool BF16ABS>
__global__ __launch_bounds__(256) void k_quant_nf4(const float *__restrict__ w, int64_t nblocks,
                                                   uint8_t *__restrict__ packed,
                                                   void *__restrict__ absmax) {
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;  // the whole wave leaves together
  const int lane = threadIdx.x & 63;
  const float v = w[blk * 64 + lane];
  float a = wave_max(fabsf(v));
  if (BF16ABS) a = __uint_as_float(bf16_round_up_bits(__float_as_uint(a)) << 16);
  uint32_t code = 7;
  if (a != 0.0f) {
    const double wd = (double)v, ad = (double)a;
    code = 0;
#pragma unroll
    for (int i = 0; i < 15; ++i) {
      const double mid = ((double)nf4_value(i) + (double)nf4_value(i + 1)) * 0.5;
      code += (mid * ad < wd) ? 1u : 0u;
    }
  }
  const uint32_t odd = __shfl_xor(code, 1, kWave);
  if ((lane & 1) == 0) packed[blk * 32 + (lane >> 1)] = (uint8_t)((code << 4) | odd);
  if (lane == 0) {
    if (BF16ABS)
      reinterpret_cast<uint16_t *>(absmax)[blk] = (uint16_t)(__float_as_uint(a) >> 16);
    else
      reinterpret_cast<float *>(absmax)[blk] = a;
  }
}

// fp32 absmax -> bf16 (rounded up when not exact); counts the inexact ones.
__global__ __launch_bounds__(256) void k_absmax_bf16(const float *__restrict__ a, int64_t n,
                                                     uint16_t *__restrict__ out, int32_t *__restrict__ inexact) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = i < n;
  const uint32_t b = live ? __float_as_uint(a[i]) : 0u;
  if (live) out[i] = (uint16_t)bf16_round_up_bits(b);
  const uint64_t bad = __ballot(live && (b & 0xffffu) != 0u);
  if ((threadIdx.x & 63) == 0 && bad) atomicAdd(inexact, (int32_t)__popcll(bad));
}

// One half-wave per 32-element MXFP4 block.
__global__ __launch_bounds__(256) void k_quant_mxfp4(const float *__restrict__ w, int64_t nblocks,
                                                     uint8_t *__restrict__ packed,
                                                     uint8_t *__restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int lane = threadIdx.x & 63;
  const bool live = blk < nblocks;
  const float v = live ? w[blk * 32 + (lane & 31)] : 0.0f;
  const float amax = half_max(fabsf(v));
  // floor(log2(amax)) from the exponent field; subnormal or zero amax gives an
  // exponent at or below -127, which clamps to X = -127 anyway.
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xff);
  int X = (ebits == 0 ? -127 : ebits - 127) - 2;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  const double q = fabs((double)v * __builtin_ldexp(1.0, -X));  // exact
  uint32_t mag = (q > 0.25) + (q >= 0.75) + (q > 1.25) + (q >= 1.75) + (q > 2.5) + (q >= 3.5) +
                 (q > 5.0);
  const uint32_t code = mag | ((__float_as_uint(v) >> 31) << 3);
  const uint32_t odd = __shfl_xor(code, 1, kWave);
  if (live) {
    if ((lane & 1) == 0) packed[blk * 16 + ((lane & 31) >> 1)] = (uint8_t)(code | (odd << 4));
    if ((lane & 31) == 0) scales[blk] = (uint8_t)(X + 127);
  }
}

// Decode: one thread per packed byte -> two fp32 values.
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t *__restrict__ packed,
                                                 const void *__restrict__ scale, int64_t nbytes,
                                                 float2 *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nbytes) return;
  const uint32_t b = packed[i];
  const int64_t k = 2 * i;                       // flat element index of the even element
  if (Fmt<FMT>::kNF4) {
    const float a = Fmt<FMT>::value(Fmt<FMT>::raw(scale, k / 64));
    out[i] = make_float2(even_value<FMT>(b) * a, odd_value<FMT>(b) * a);
  } else {
    const uint32_t e = reinterpret_cast<const uint8_t *>(scale)[k / 32];
    if (e == 255u) {
      out[i] = make_float2(__builtin_nanf(""), __builtin_nanf(""));
    } else {
      const double s = __builtin_ldexp(1.0, (int)e - 127);
      out[i] = make_float2((float)((double)even_value<1>(b) * s), (float)((double)odd_value<1>(b) * s));
    }
  }
}

// Large tensors are processed in pieces so every grid stays well inside the
// 32-bit limits of a dispatch.
static constexpr int64_t kPiece = int64_t(1) << 28;   // elements per launch (multiple of 64)

hipError_t launch_quantize(int fmt, const float *w, int64_t rows, int64_t K, uint8_t *packed,
                           void *scale, hipStream_t s) {
  const int64_t n = rows * K;
  for (int64_t e0 = 0; e0 < n; e0 += kPiece) {
    const int64_t m = (n - e0) < kPiece ? (n - e0) : kPiece;
    if (fmt == 0) {
      const int64_t nb = m / 64;
      hipLaunchKernelGGL(k_quant_nf4<false>, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, s, w + e0, nb,
                         packed + e0 / 2, (void *)((float *)scale + e0 / 64));
    } else if (fmt == 2) {
      const int64_t nb = m / 64;
      hipLaunchKernelGGL(k_quant_nf4<true>, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, s, w + e0, nb,
                         packed + e0 / 2, (void *)((uint16_t *)scale + e0 / 64));
    } else {
      const int64_t nb = m / 32;
      hipLaunchKernelGGL(k_quant_mxfp4, dim3((unsigned)((nb + 7) / 8)), dim3(256), 0, s, w + e0,
                         nb, packed + e0 / 2, (uint8_t *)scale + e0 / 32);
    }
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, const uint8_t *packed, const void *scale, int64_t rows,
                             int64_t K, float *out, hipStream_t s) {
  const int64_t n = rows * K;
  for (int64_t e0 = 0; e0 < n; e0 += kPiece) {
    const int64_t m = (n - e0) < kPiece ? (n - e0) : kPiece;
    const int64_t nbytes = m / 2;
    const dim3 grid((unsigned)((nbytes + 255) / 256));
    if (fmt == 0)
      hipLaunchKernelGGL(k_dequant<0>, grid, dim3(256), 0, s, packed + e0 / 2,
                         (const void *)((const float *)scale + e0 / 64), nbytes,
                         (float2 *)(out + e0));
    else if (fmt == 2)
      hipLaunchKernelGGL(k_dequant<2>, grid, dim3(256), 0, s, packed + e0 / 2,
                         (const void *)((const uint16_t *)scale + e0 / 64), nbytes,
                         (float2 *)(out + e0));
    else
      hipLaunchKernelGGL(k_dequant<1>, grid, dim3(256), 0, s, packed + e0 / 2,
                         (const void *)((const uint8_t *)scale + e0 / 32), nbytes,
                         (float2 *)(out + e0));
  }
  return hipGetLastError();
}

hipError_t launch_absmax_bf16(const float *a, int64_t n, uint16_t *out, int32_t *inexact, hipStream_t s) {
  for (int64_t i0 = 0; i0 < n; i0 += kPiece) {
    const int64_t m = (n - i0) < kPiece ? (n - i0) : kPiece;
    hipLaunchKernelGGL(k_absmax_bf16, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, a + i0, m, out + i0,
                       inexact);
  }
  return hipGetLastError();
}

}  // namespace nf4moe
