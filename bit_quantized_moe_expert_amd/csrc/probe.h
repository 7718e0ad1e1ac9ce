// The matrix-core rate probe (a measurement aid), shared by probe.hip and the
// C-ABI in api.hip.
#pragma once
#include <cstdint>

#include <hip/hip_runtime.h>

namespace nf4moe {

// workgroups of 512 threads, each wave `iters` rounds of 8 bf16 MFMAs (32x32x16)
// on register operands; sink[workgroups * 512] floats.
int64_t mfma_peak_flops(int workgroups, int iters);
hipError_t launch_mfma_peak(int workgroups, int iters, float *sink, hipStream_t s);

}  // namespace nf4moe
