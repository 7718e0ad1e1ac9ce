// A measurement aid: one plain streaming read of a buffer, to put a measured
// single-launch HBM read rate beside the decode kernels' at the same byte
// counts (the spec peak is not reachable by one short launch). Each thread
// issues a fixed number of independent 16-byte loads (1 to 16, a launch
// parameter, so the caller can take the fastest shape), all before the first
// use, and folds them into one XOR that its workgroup writes out, so no load
// can be dropped.
#include "common.h"
#include "internal.h"
#include "probe.h"

namespace nf4moe {

constexpr int kStreamThreads = 256;

// Each thread issues LOADS independent 16-byte loads, all before the first use.
template <int LOADS>
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const uint4 *__restrict__ src, int64_t n16,
                                                                uint32_t *__restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (kStreamThreads * LOADS) + threadIdx.x;
  uint4 v[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int64_t j = base + (int64_t)i * kStreamThreads;
    v[i] = src[j < n16 ? j : n16 - 1];
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  __shared__ uint32_t red[kStreamThreads / 64];
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

bool stream_read_loads_ok(int loads) { return loads == 1 || loads == 2 || loads == 4 || loads == 8 || loads == 16; }

int64_t stream_read_grid(int64_t bytes, int loads) { return cdiv(bytes / 16, (int64_t)kStreamThreads * loads); }

template <int LOADS>
static void launch_stream_t(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read<LOADS>, dim3((unsigned)stream_read_grid(bytes, LOADS)), dim3(kStreamThreads), 0,
                     s, reinterpret_cast<const uint4 *>(src), bytes / 16, sink);
}

hipError_t launch_stream_read(const void *src, int64_t bytes, int loads, uint32_t *sink, hipStream_t s) {
  switch (loads) {
    case 1: launch_stream_t<1>(src, bytes, sink, s); break;
    case 2: launch_stream_t<2>(src, bytes, sink, s); break;
    case 4: launch_stream_t<4>(src, bytes, sink, s); break;
    case 8: launch_stream_t<8>(src, bytes, sink, s); break;
    case 16: launch_stream_t<16>(src, bytes, sink, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// A second measurement aid: the bf16 matrix-core rate this GPU sustains with
// every SIMD busy, to put beside the published dense peak. Each wave runs
// `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on operands held
// in registers (no memory traffic). The operands are pseudo-random finite bf16
// values (random signs and significands, exponents within 2^-3 .. 2^4), so
// the matrix cores toggle as they do on real data; the rate they sustain is
// the clock the chip holds under that load times the published flops per
// clock. Each thread writes the sum of its accumulators to sink, so no MFMA
// can be dropped.
typedef __bf16 pk_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float pk_f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kPeakThreads = 512;
constexpr int kPeakChains = 8;

__device__ inline uint32_t peak_hash(uint32_t x) {  // a 32-bit integer mix (xorshift-multiply)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ inline uint32_t peak_bf16x2(uint32_t r) {  // two finite bf16: sign, exponent 124..131, significand
  const uint32_t lo = (r & 0x807fu) | ((124u + ((r >> 7) & 7u)) << 7);
  const uint32_t hi = ((r >> 16) & 0x807fu) | ((124u + ((r >> 23) & 7u)) << 7);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(kPeakThreads) void k_mfma_peak(int iters, uint32_t seed, float *__restrict__ sink) {
  const uint32_t t = blockIdx.x * kPeakThreads + threadIdx.x;
  pk_bf16x8_t a[2], b[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4 v = make_uint4(peak_bf16x2(peak_hash(seed ^ (t * 16u + 4u * i))),
                               peak_bf16x2(peak_hash(seed ^ (t * 16u + 4u * i + 1u))),
                               peak_bf16x2(peak_hash(seed ^ (t * 16u + 4u * i + 2u))),
                               peak_bf16x2(peak_hash(seed ^ (t * 16u + 4u * i + 3u))));
    a[i] = __builtin_bit_cast(pk_bf16x8_t, v);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = make_uint4(peak_bf16x2(peak_hash(~seed ^ (t * 16u + 4u * i))),
                               peak_bf16x2(peak_hash(~seed ^ (t * 16u + 4u * i + 1u))),
                               peak_bf16x2(peak_hash(~seed ^ (t * 16u + 4u * i + 2u))),
                               peak_bf16x2(peak_hash(~seed ^ (t * 16u + 4u * i + 3u))));
    b[i] = __builtin_bit_cast(pk_bf16x8_t, v);
  }
  pk_f32x16_t c[kPeakChains];
#pragma unroll
  for (int j = 0; j < kPeakChains; ++j) c[j] = pk_f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kPeakChains; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 1], b[j >> 1], c[j], 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kPeakChains; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) sum += c[j][v];
  sink[t] = sum;
}

int64_t mfma_peak_flops(int workgroups, int iters) {
  return (int64_t)workgroups * (kPeakThreads / 64) * iters * kPeakChains * (2LL * 32 * 32 * 16);
}

hipError_t launch_mfma_peak(int workgroups, int iters, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_peak, dim3((unsigned)workgroups), dim3(kPeakThreads), 0, s, iters, 0x5eed1234u, sink);
  return hipGetLastError();
}

}  // namespace nf4moe
