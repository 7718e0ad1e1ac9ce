// A measurement aid: one plain streaming read of a buffer, to put a measured
// single-launch HBM read rate beside the decode kernels' at the same byte
// counts (the spec peak is not reachable by one short launch). Each thread
// issues a fixed number of independent 16-byte loads (1 to 16, a launch
// parameter, so the caller can take the fastest shape), all before the first
// use, and folds them into one XOR that its workgroup writes out, so no load
// can be dropped.
#include "common.h"
#include "internal.h"

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

}  // namespace nf4moe
