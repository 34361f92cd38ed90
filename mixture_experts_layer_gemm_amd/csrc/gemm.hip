// Grouped GEMM over densely packed expert segments, with a fused SwiGLU epilogue.
//
// Expert i owns rows [o_i, o_{i+1}) of the packed activation (real-count offsets,
// "Section 10: Routing, Capacity, and Load Balancing", Eq. 26); no padding rows are
// computed. The two passes of the SwiGLU expert ("Section 20: One Shared Expert Is All
// You Need", Eq. 74) are:
//   swiglu = true : h = SiLU(a W_g^T) * (a W_u^T)  (gate and up tiles in one workgroup)
//   swiglu = false: out = a W^T                     (the down projection)
//
// bf16 path (gfx950 MFMA, v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * tile = 128 packed rows x 256 weight rows (swiglu: 128 gate + 128 up rows, i.e.
//     128 output columns; plain: 256 output columns), k-step 32, 4 waves;
//   * the product is formed transposed (weights as the MFMA A operand, rows as B) so
//     each lane ends up holding 4 consecutive output columns of one row: 8-byte stores;
//   * LDS stages are double buffered through registers; 16-byte chunks are XOR
//     swizzled by row so MFMA operand reads and the staging writes avoid bank conflicts;
//   * the tile map is rebuilt on the device from the offsets (no host sync): every
//     workgroup scans the per-group m-tile counts in LDS; the tile order is
//     (group, m-tile, n-tile) and is laid out XCD-major, so the tiles sharing a weight
//     slab or an activation slab run together on one XCD and hit its L2.
// f32 path: a plain LDS-tiled FMA kernel with the same tile map (small fp32 layers).
#include "common.h"

using namespace moe;

namespace {

constexpr int BM = 128;                 // packed rows per tile
constexpr int BNW = 256;                // weight rows per tile
constexpr int BK = 32;                  // k per stage
constexpr int THREADS = 256;
constexpr int A_BYTES = BM * BK * 2;
constexpr int W_BYTES = BNW * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + W_BYTES;

// byte offset of 16-byte chunk kc (0..3) of row r in a [rows][BK] bf16 LDS tile;
// the XOR pattern spreads 8 (or 16) consecutive rows over distinct banks.
__device__ __forceinline__ int swz(int r, int kc) {
  const int f = (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1);
  return r * (BK * 2) + ((kc ^ f) << 4);
}

struct TileMap {
  int g, row0, rows, nt;
};

// Builds the (group, m-tile) prefix in LDS and decodes this workgroup's tile.
// Returns false for a spare workgroup. All threads must call it.
__device__ bool decode_tile(const int32_t* __restrict__ offsets, int G, int max_rows, int bm,
                            int n_tiles, int* s_off, int* s_mstart, TileMap& tm) {
  const int tid = threadIdx.x;
  for (int g = tid; g <= G; g += blockDim.x)
    s_off[g] = (offsets != nullptr) ? offsets[g] : (g == 0 ? 0 : max_rows);
  __syncthreads();
  // inclusive scan of m-tile counts (G <= 256 = blockDim)
  const int cnt = (tid < G) ? ceil_div(s_off[tid + 1] - s_off[tid], bm) : 0;
  s_mstart[tid + 1] = cnt;
  if (tid == 0) s_mstart[0] = 0;
  __syncthreads();
  for (int off = 1; off < THREADS; off <<= 1) {
    const int v = (tid >= off) ? s_mstart[tid + 1 - off] : 0;
    __syncthreads();
    s_mstart[tid + 1] += v;
    __syncthreads();
  }
  const int total_m = s_mstart[G];
  const int tile = xcd_remap(blockIdx.x, total_m * n_tiles);
  if (tile < 0) return false;
  const int mt = tile / n_tiles;
  tm.nt = tile - mt * n_tiles;
  int lo = 0, hi = G - 1;  // largest g with s_mstart[g] <= mt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_mstart[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  tm.g = lo;
  tm.row0 = s_off[lo] + (mt - s_mstart[lo]) * bm;
  tm.rows = min(bm, s_off[lo + 1] - tm.row0);
  return true;
}

// GROUPED = false: one group over rows [0, max_rows) (the shared MLP); a separate
// instantiation so that profiles tell the routed and the shared launches apart.
template <bool SWIGLU, bool GROUPED>
__global__ void __launch_bounds__(THREADS, 2)
gemm_bf16_kernel(int G, int Kd, int Nd, const uint16_t* __restrict__ a,
                 const int32_t* __restrict__ offsets, int max_rows,
                 const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1,
                 uint16_t* __restrict__ out) {
  __shared__ int s_off[kMaxN + 1];
  __shared__ int s_mstart[THREADS + 1];
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE_BYTES];

  constexpr int COLS = SWIGLU ? BNW / 2 : BNW;  // output columns per tile
  const int n_tiles = ceil_div(Nd, COLS);
  TileMap tm;
  if (!decode_tile(GROUPED ? offsets : nullptr, G, max_rows, BM, n_tiles, s_off, s_mstart, tm))
    return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n0 = tm.nt * COLS;
  const size_t wstride = static_cast<size_t>(Nd) * Kd;
  const uint16_t* wg = w0 + tm.g * wstride;
  const uint16_t* wu = SWIGLU ? (w1 + tm.g * wstride) : nullptr;

  // staging assignment: A 2 chunks/thread, W 4 chunks/thread
  const uint16_t* asrc[2];
  int alds[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * THREADS;
    const int r = c >> 2, kc = c & 3;
    const int src = tm.row0 + min(r, tm.rows - 1);
    asrc[i] = a + static_cast<size_t>(src) * Kd + kc * 8;
    alds[i] = swz(r, kc);
  }
  const uint16_t* wsrc[4];
  int wlds[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * THREADS;
    const int r = c >> 2, kc = c & 3;
    const uint16_t* base;
    int n;
    if (SWIGLU) {
      base = (r < BNW / 2) ? wg : wu;
      n = n0 + (r & (BNW / 2 - 1));
    } else {
      base = wg;
      n = n0 + r;
    }
    n = min(n, Nd - 1);
    wsrc[i] = base + static_cast<size_t>(n) * Kd + kc * 8;
    wlds[i] = A_BYTES + swz(r, kc);
  }

  // wave roles: two 32-row weight blocks x four 32-row activation blocks
  const int wb0 = SWIGLU ? 32 * w : 64 * w;
  const int wb1 = SWIGLU ? BNW / 2 + 32 * w : 64 * w + 32;
  const int ncol0 = SWIGLU ? n0 + 32 * w : n0 + 64 * w;        // output column of block 0
  const int ncol1 = SWIGLU ? ncol0 : ncol0 + 32;
  const bool wv0 = ncol0 < Nd;
  const bool wv1 = ncol1 < Nd;
  const int xblocks = ceil_div(tm.rows, 32);

  floatx16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  u32x4 ra[2], rw[4];
  const int nk = Kd / BK;
  auto gload = [&](int ks) {
    const int ko = ks * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) ra[i] = *reinterpret_cast<const u32x4*>(asrc[i] + ko);
#pragma unroll
    for (int i = 0; i < 4; ++i) rw[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + ko);
  };
  auto lstore = [&](int buf) {
    char* base = lds + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(base + alds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(base + wlds[i]) = rw[i];
  };

  gload(0);
  lstore(0);
  __syncthreads();
  const int lr = lane & 31;
  const int lh = lane >> 5;
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) gload(ks + 1);
    const char* base = lds + (ks & 1) * STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kc = 2 * s + lh;
      const bf16x8 wa0 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(base + A_BYTES + swz(wb0 + lr, kc)));
      const bf16x8 wa1 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(base + A_BYTES + swz(wb1 + lr, kc)));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < xblocks) {
          const bf16x8 xb = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(base + swz(32 * j + lr, kc)));
          if (wv0) acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa0, xb, acc[0][j], 0, 0, 0);
          if (wv1) acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa1, xb, acc[1][j], 0, 0, 0);
        }
      }
    }
    if (ks + 1 < nk) lstore((ks + 1) & 1);
    __syncthreads();
  }

  // epilogue: lane holds row (32 j + lr) and columns 8 q + 4 lh + {0..3} of each block
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 32 * j + lr;
    if (m >= tm.rows) continue;
    uint16_t* orow = out + static_cast<size_t>(tm.row0 + m) * Nd;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (SWIGLU) {
        if (!wv0) continue;
        const int n = ncol0 + 8 * q + 4 * lh;
        float h[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) h[u] = silu_f(acc[0][j][4 * q + u]) * acc[1][j][4 * q + u];
        *reinterpret_cast<u32x2*>(orow + n) = u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bool ok = i == 0 ? wv0 : wv1;
          if (!ok) continue;
          const int n = (i == 0 ? ncol0 : ncol1) + 8 * q + 4 * lh;
          const floatx16& c = acc[i][j];
          *reinterpret_cast<u32x2*>(orow + n) =
              u32x2{pack_bf16x2(c[4 * q], c[4 * q + 1]), pack_bf16x2(c[4 * q + 2], c[4 * q + 3])};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// f32: 64 x 64 output tile, 256 threads with 4 x 4 outputs each, k-step 16
// ---------------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool SWIGLU>
__global__ void __launch_bounds__(THREADS)
gemm_f32_kernel(int G, int Kd, int Nd, const float* __restrict__ a,
                const int32_t* __restrict__ offsets, int max_rows, const float* __restrict__ w0,
                const float* __restrict__ w1, float* __restrict__ out) {
  __shared__ int s_off[kMaxN + 1];
  __shared__ int s_mstart[THREADS + 1];
  __shared__ float sa[FBK][FBM + 4];
  __shared__ float sg[FBK][FBN + 4];
  __shared__ float su[FBK][FBN + 4];
  const int n_tiles = ceil_div(Nd, FBN);
  TileMap tm;
  if (!decode_tile(offsets, G, max_rows, FBM, n_tiles, s_off, s_mstart, tm)) return;
  const int tid = threadIdx.x;
  const int n0 = tm.nt * FBN;
  const size_t wstride = static_cast<size_t>(Nd) * Kd;
  const float* wg = w0 + tm.g * wstride;
  const float* wu = SWIGLU ? w1 + tm.g * wstride : nullptr;
  const int tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
  float cg[4][4] = {}, cu[4][4] = {};
  for (int k0 = 0; k0 < Kd; k0 += FBK) {
    for (int i = tid; i < FBM * FBK; i += THREADS) {
      const int r = i / FBK, k = i % FBK;
      sa[k][r] = a[static_cast<size_t>(tm.row0 + min(r, tm.rows - 1)) * Kd + k0 + k];
      const int n = min(n0 + r, Nd - 1);
      sg[k][r] = wg[static_cast<size_t>(n) * Kd + k0 + k];
      if (SWIGLU) su[k][r] = wu[static_cast<size_t>(n) * Kd + k0 + k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FBK; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cg[i][j] = fmaf(sa[k][tr + i], sg[k][tc + j], cg[i][j]);
          if (SWIGLU) cu[i][j] = fmaf(sa[k][tr + i], su[k][tc + j], cu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (tr + i >= tm.rows) continue;
    float* orow = out + static_cast<size_t>(tm.row0 + tr + i) * Nd;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tc + j;
      if (n < Nd) orow[n] = SWIGLU ? silu_f(cg[i][j]) * cu[i][j] : cg[i][j];
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(bool swiglu, int G, int Kd, int Nd, int dt, const void* a,
                               const int32_t* offsets, int max_rows, const void* w0,
                               const void* w1, void* out, hipStream_t stream) {
  const int bm = dt == 1 ? BM : FBM;
  const int cols = dt == 1 ? (swiglu ? BNW / 2 : BNW) : FBN;
  const int n_tiles = (Nd + cols - 1) / cols;
  const long max_m = static_cast<long>(max_rows) / bm + G + 1;
  long grid = max_m * n_tiles;
  grid = (grid + 7) / 8 * 8;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  const dim3 g(static_cast<unsigned>(grid)), b(THREADS);
  if (dt == 1) {
    const uint16_t* A = static_cast<const uint16_t*>(a);
    const uint16_t* W0 = static_cast<const uint16_t*>(w0);
    const uint16_t* W1 = static_cast<const uint16_t*>(w1);
    uint16_t* O = static_cast<uint16_t*>(out);
    const bool grouped = offsets != nullptr;
    if (swiglu && grouped)
      hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), g, b, 0, stream, G, Kd, Nd, A, offsets, max_rows, W0, W1, O);
    else if (swiglu)
      hipLaunchKernelGGL((gemm_bf16_kernel<true, false>), g, b, 0, stream, G, Kd, Nd, A, offsets, max_rows, W0, W1, O);
    else if (grouped)
      hipLaunchKernelGGL((gemm_bf16_kernel<false, true>), g, b, 0, stream, G, Kd, Nd, A, offsets, max_rows, W0, W1, O);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), g, b, 0, stream, G, Kd, Nd, A, offsets, max_rows, W0, W1, O);
  } else {
    const float* A = static_cast<const float*>(a);
    const float* W0 = static_cast<const float*>(w0);
    const float* W1 = static_cast<const float*>(w1);
    float* O = static_cast<float*>(out);
    if (swiglu)
      hipLaunchKernelGGL(gemm_f32_kernel<true>, g, b, 0, stream, G, Kd, Nd, A, offsets, max_rows, W0, W1, O);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<false>, g, b, 0, stream, G, Kd, Nd, A, offsets, max_rows, W0, W1, O);
  }
  return hipGetLastError();
}
