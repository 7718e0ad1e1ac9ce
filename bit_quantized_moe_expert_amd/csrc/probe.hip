// A measurement aid: one plain streaming read of a buffer, to put a measured
// single-launch HBM read rate beside the decode kernels' at the same byte
// counts (the spec peak is not reachable by one short launch). Each thread
// issues kStreamLoads independent 16-byte loads, all before the first use, and
// folds them into one XOR that its workgroup writes out, so no load can be
// dropped.
#include "common.h"
#include "internal.h"

namespace nf4moe {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 4;

__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const uint4 *__restrict__ src, int64_t n16,
                                                                uint32_t *__restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (kStreamThreads * kStreamLoads) + threadIdx.x;
  uint4 v[kStreamLoads];
#pragma unroll
  for (int i = 0; i < kStreamLoads; ++i) {
    const int64_t j = base + (int64_t)i * kStreamThreads;
    v[i] = src[j < n16 ? j : n16 - 1];
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kStreamLoads; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  __shared__ uint32_t red[kStreamThreads / 64];
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

int64_t stream_read_grid(int64_t bytes) { return cdiv(bytes / 16, kStreamThreads * kStreamLoads); }

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t grid = stream_read_grid(bytes);
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(kStreamThreads), 0, s,
                     reinterpret_cast<const uint4 *>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace nf4moe
