// Grouped dgrad (input gradient of the grouped GEMM) -- internal interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4moe {

struct DgradArgs {
  int fmt;
  const uint16_t *dc;       // bf16 [R, N], rows in group order
  const uint8_t *B;         // [E, N, K/2]
  const void *B_scale;      // NF4 fp32 [E, N, K/64]; MXFP4 e8m0 [E, N, K/32]
  int64_t N, K;             // N % 64 == 0
  const int4 *tiles;        // (expert, row0, rows, group rows) tiles of <= 128 rows
  const int32_t *n_tiles;
  int max_tiles;
  void *da;                 // [R, K] fp32 or bf16
  int da_bf16;
};

hipError_t launch_dgrad(const DgradArgs &a, hipStream_t s);

}  // namespace nf4moe
