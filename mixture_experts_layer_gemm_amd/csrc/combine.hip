// Combine: y = sum_{i in S(x), kept} r_i f_i(x) + s(x) g(x)
// ("Section 21: Merging Routed and Shared Expert Activations", Eq. 80; dropped routes
// are masked and the kept coefficients are not renormalized, "Section 10: Routing,
// Capacity, and Load Balancing", Section 10.3).
//
// HBM-bound weighted gather: one wave per token, each lane owns 16-byte pieces of the
// row; the K packed expert rows and the shared row are read once with coalesced
// 16-byte loads, four slots' loads in flight together, accumulated in fp32 in slot
// order, and y is written once.
#include "common.h"

using namespace moe;

namespace {

constexpr int WAVES = 4;

constexpr int KG = 4;  // slots whose loads are in flight together

// a 16-byte piece as floats: 8 bf16 or 4 fp32
template <bool BF16>
__device__ __forceinline__ void unpack16(const u32x4& u, float* v) {
  if (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(u[i]);
  }
}

template <bool BF16>
__global__ void __launch_bounds__(WAVES * kWave)
combine_kernel(int T, int d, int K, const void* __restrict__ f_perm,
               const int32_t* __restrict__ dest_row, const float* __restrict__ topk_r,
               const void* __restrict__ g, float s, const float* __restrict__ s_tok,
               void* __restrict__ y) {
  constexpr int EPP = BF16 ? 8 : 4;  // elements per 16-byte piece
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * WAVES + (threadIdx.x >> 6);
  if (t >= T) return;
  int dk = -1;
  float rk = 0.f;
  if (lane < K) {
    dk = dest_row[static_cast<size_t>(t) * K + lane];
    rk = topk_r != nullptr ? topk_r[static_cast<size_t>(t) * K + lane] : 1.0f;
  }
  const float st = (s_tok != nullptr) ? s_tok[t] : s;
  const char* fb = static_cast<const char*>(f_perm);
  const char* gb = static_cast<const char*>(g);
  const size_t rowb = static_cast<size_t>(d) * (BF16 ? 2 : 4);
  const int npc = d / EPP;
  for (int j = lane; j < npc; j += kWave) {
    float acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.f;
    // slots in groups of KG: the group's loads (and the shared row's, with the first
    // group) are all issued before the first is used; accumulation stays in slot order
    u32x4 gv = u32x4{0u, 0u, 0u, 0u};
    if (g != nullptr) gv = *reinterpret_cast<const u32x4*>(gb + static_cast<size_t>(t) * rowb + j * 16);
    for (int k0 = 0; k0 < K; k0 += KG) {
      int row[KG];
      float rr[KG];
      u32x4 fv[KG];
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        row[q] = k0 + q < K ? __shfl(dk, k0 + q, kWave) : -1;
        rr[q] = __shfl(rk, min(k0 + q, K - 1), kWave);
        if (row[q] >= 0)
          fv[q] = *reinterpret_cast<const u32x4*>(fb + static_cast<size_t>(row[q]) * rowb + j * 16);
      }
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        if (row[q] < 0) continue;
        float v[EPP];
        unpack16<BF16>(fv[q], v);
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc[e] = fmaf(rr[q], v[e], acc[e]);
      }
    }
    if (g != nullptr) {
      float v[EPP];
      unpack16<BF16>(gv, v);
#pragma unroll
      for (int e = 0; e < EPP; ++e) acc[e] = fmaf(st, v[e], acc[e]);
    }
    if (BF16) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + static_cast<size_t>(t) * d + j * EPP) = o;
    } else {
      *reinterpret_cast<floatx4*>(static_cast<float*>(y) + static_cast<size_t>(t) * d + j * EPP) =
          floatx4{acc[0], acc[1], acc[2], acc[3]};
    }
  }
}

}  // namespace

hipError_t launch_combine(int T, int d_model, int K, int dt, const void* f_perm,
                          const int32_t* dest_row, const float* topk_r, const void* g,
                          float s, const float* s_tok, void* y, hipStream_t stream) {
  const int grid = (T + WAVES - 1) / WAVES;
  if (dt == 1)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(WAVES * kWave), 0, stream, T,
                       d_model, K, f_perm, dest_row, topk_r, g, s, s_tok, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(WAVES * kWave), 0, stream, T,
                       d_model, K, f_perm, dest_row, topk_r, g, s, s_tok, y);
  return hipGetLastError();
}
