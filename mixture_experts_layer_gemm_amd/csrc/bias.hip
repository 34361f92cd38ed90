// Hard-count feedback controller of auxiliary-loss-free balancing ("Section 10: Routing,
// Capacity, and Load Balancing", Eq. 36-37): over one feedback window of requested
// counts C, every expert's persistent selection bias moves by gamma toward the mean,
//   b_i <- b_i + gamma sign(mean(C) - C_i),
// applied outside any gradient. The sign is decided exactly in 64-bit integers as
// sign(sum_j C_j - N C_i); an expert exactly at the mean keeps its bias bit for bit.
// One workgroup, one expert per thread (N <= 256); the total is a fixed-order tree sum.
#include "common.h"

using namespace moe;

namespace {

constexpr int BU_THREADS = 256;

__global__ void __launch_bounds__(BU_THREADS)
bias_update_kernel(int N, float gamma, int32_t* __restrict__ count_accum,
                   float* __restrict__ expert_bias, int reset) {
  __shared__ long long red[BU_THREADS];
  const int tid = threadIdx.x;
  const long long c = tid < N ? count_accum[tid] : 0;
  red[tid] = c;
  __syncthreads();
  for (int off = BU_THREADS / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const long long diff = red[0] - static_cast<long long>(N) * c;
  if (tid < N) {
    if (diff != 0) expert_bias[tid] = expert_bias[tid] + (diff > 0 ? gamma : -gamma);
    if (reset) count_accum[tid] = 0;
  }
}

}  // namespace

hipError_t launch_bias_update(int N, float gamma, int32_t* count_accum, float* expert_bias,
                              int reset, hipStream_t stream) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(BU_THREADS), 0, stream, N, gamma,
                     count_accum, expert_bias, reset);
  return hipGetLastError();
}
