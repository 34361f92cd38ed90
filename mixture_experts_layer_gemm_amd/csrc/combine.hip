// Combine: y = sum_{i in S(x), kept} r_i f_i(x) + s(x) g(x)
// ("Section 21: Merging Routed and Shared Expert Activations", Eq. 80; dropped routes
// are masked and the kept coefficients are not renormalized, "Section 10: Routing,
// Capacity, and Load Balancing", Section 10.3).
//
// HBM-bound weighted gather: one wave per token, each lane owns 16-byte pieces of the
// row; the K packed expert rows and the shared row are read once with coalesced
// 16-byte loads (up to four slots times four pieces per lane in flight together; the
// expert rows, read once, non-temporal), accumulated in fp32 in slot order, and y is
// written once with non-temporal stores.
#include "common.h"

using namespace moe;

namespace {

constexpr int WAVES = 4;

constexpr int JU = 4;  // 16-byte pieces per lane whose loads are in flight together

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

// KG: slots whose loads are issued together (min(K, 4)). Every load is unconditional and
// in bounds, so none waits on another: a dropped route reads the token's own y row and a
// slot past K the last slot's row again (both replaced by zeros), a piece past the row
// end the row's last piece (not stored).
template <bool BF16, int KG>
__global__ void __launch_bounds__(WAVES * kWave)
combine_kernel(int T, int d, int K, const void* __restrict__ f_perm,
               const int32_t* __restrict__ dest_row, const float* __restrict__ topk_r,
               const void* __restrict__ g, float s, const float* __restrict__ s_tok,
               void* __restrict__ y) {
  constexpr int EPP = BF16 ? 8 : 4;  // elements per 16-byte piece
  const int lane = threadIdx.x & 63;
  // wave-uniform token: its row addresses are scalar, every load a scalar base + offset
  const int t = blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  int dk = -1;
  float rk = 0.f;
  if (lane < K) {
    dk = dest_row[static_cast<size_t>(t) * K + lane];
    rk = topk_r != nullptr ? topk_r[static_cast<size_t>(t) * K + lane] : 1.0f;
  }
  const float st = (s_tok != nullptr) ? s_tok[t] : s;
  const size_t rowb = static_cast<size_t>(d) * (BF16 ? 2 : 4);
  const int npc = d / EPP;
  char* yrow = static_cast<char*>(y) + static_cast<size_t>(t) * rowb;
  const bool has_g = g != nullptr;
  const char* grow = has_g ? static_cast<const char*>(g) + static_cast<size_t>(t) * rowb : yrow;
  const char* fb = static_cast<const char*>(f_perm);
  // lane's pieces j0 + 64 u (u < JU) together; per element the slots are accumulated in
  // slot order, then the shared row
  for (int jb = 0; jb < npc; jb += kWave * JU) {  // wave-uniform trip count
    const int j0 = jb + lane;
    uint32_t off[JU];
#pragma unroll
    for (int u = 0; u < JU; ++u) off[u] = static_cast<uint32_t>(min(j0 + u * kWave, npc - 1)) * 16u;
    u32x4 gv[JU];
#pragma unroll
    for (int u = 0; u < JU; ++u) gv[u] = *reinterpret_cast<const u32x4*>(grow + off[u]);
    float acc[JU][EPP];
#pragma unroll
    for (int u = 0; u < JU; ++u)
#pragma unroll
      for (int e = 0; e < EPP; ++e) acc[u][e] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KG) {
      int row[KG];
      float rr[KG];
      const char* fr[KG];
      u32x4 fv[KG][JU];
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        // wave-uniform: the slot's row and coefficient live in scalar registers
        const int k = min(k0 + q, K - 1);
        const int rw = __builtin_amdgcn_readfirstlane(__shfl(dk, k, kWave));
        row[q] = k0 + q < K ? rw : -1;
        rr[q] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                    __builtin_bit_cast(int, __shfl(rk, k, kWave))));
        fr[q] = rw >= 0 ? fb + static_cast<size_t>(rw) * rowb : yrow;
#pragma unroll
        for (int u = 0; u < JU; ++u)  // each expert output row is read once: non-temporal
          fv[q][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(fr[q] + off[u]));
      }
      // a dropped or absent slot adds exact zeros (selected bits, not a branch, so that
      // no load is sunk into a conditional block and waited for on its own)
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        const bool live = row[q] >= 0;
#pragma unroll
        for (int u = 0; u < JU; ++u) {
          float v[EPP];
          const u32x4 z = u32x4{0u, 0u, 0u, 0u};
          unpack16<BF16>(live ? fv[q][u] : z, v);
#pragma unroll
          for (int e = 0; e < EPP; ++e) acc[u][e] = fmaf(rr[q], v[e], acc[u][e]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < JU; ++u) {
      const int j = j0 + u * kWave;
      if (j >= npc) continue;
      if (has_g) {
        float v[EPP];
        unpack16<BF16>(gv[u], v);
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc[u][e] = fmaf(st, v[e], acc[u][e]);
      }
      u32x4 o;
      if (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[u][2 * i], acc[u][2 * i + 1]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[u][i]);
      }
      // y is written once and not read back here
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(yrow + j * 16));
    }
  }
}

template <bool BF16>
hipError_t launch_dt(int T, int d_model, int K, const void* f_perm, const int32_t* dest_row,
                     const float* topk_r, const void* g, float s, const float* s_tok, void* y,
                     hipStream_t stream) {
  const int grid = (T + WAVES - 1) / WAVES;
#define MOE_COMBINE_KG(KG_)                                                                  \
  hipLaunchKernelGGL((combine_kernel<BF16, KG_>), dim3(grid), dim3(WAVES * kWave), 0, stream, \
                     T, d_model, K, f_perm, dest_row, topk_r, g, s, s_tok, y)
  if (K == 1) MOE_COMBINE_KG(1);
  else if (K == 2) MOE_COMBINE_KG(2);
  else if (K == 3) MOE_COMBINE_KG(3);
  else MOE_COMBINE_KG(4);
#undef MOE_COMBINE_KG
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(int T, int d_model, int K, int dt, const void* f_perm,
                          const int32_t* dest_row, const float* topk_r, const void* g,
                          float s, const float* s_tok, void* y, hipStream_t stream) {
  if (dt == 1)
    return launch_dt<true>(T, d_model, K, f_perm, dest_row, topk_r, g, s, s_tok, y, stream);
  return launch_dt<false>(T, d_model, K, f_perm, dest_row, topk_r, g, s, s_tok, y, stream);
}
