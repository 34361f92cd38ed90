// Grouped GEMM over densely packed expert segments, with a fused SwiGLU epilogue.
//
// Expert i owns rows [o_i, o_{i+1}) of the packed activation (real-count offsets,
// "Section 10: Routing, Capacity, and Load Balancing", Eq. 26); no padding rows are
// computed. The two passes of the SwiGLU expert ("Section 20: One Shared Expert Is All
// You Need", Eq. 74) are:
//   swiglu = true : h = SiLU(a W_g^T) * (a W_u^T)  (gate and up tiles in one workgroup)
//   swiglu = false: out = a W^T                     (the down projection)
//
// bf16 path (gfx950, v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * workgroup tile = 128 packed rows x 512 weight rows (swiglu: 256 gate + 256 up
//     rows = 256 output columns; plain: 512 output columns), 4 waves, one per SIMD,
//     each wave a 128 x 128 block of 4 x 4 MFMA tiles (256 fp32 accumulators): large
//     wave tiles keep LDS traffic per MFMA low;
//   * the k loop streams 32-wide stages through a 3-deep LDS ring filled by
//     global_load_lds_dwordx4 (gfx950 direct-to-LDS loads, no register staging): each
//     stage is issued two iterations before it is consumed, so ~80 KB per CU stays in
//     flight to HBM while the MFMAs run; one barrier per stage;
//   * 16-byte chunks are XOR-swizzled by row so MFMA operand reads are bank-conflict
//     free; the DMA lane -> (row, chunk) mapping writes that swizzled layout directly;
//   * the product is formed transposed (weights are the MFMA A operand, rows the B
//     operand), so each lane holds 4 consecutive output columns of one row;
//   * the tile map is rebuilt on the device from the offsets (no host sync); tiles are
//     ordered (group, n-tile, m-tile) and laid out XCD-major so the m-tiles that share
//     a weight slab run side by side on one XCD and share its L2.
// f32 path: a plain LDS-tiled FMA kernel with the same tile map (small fp32 layers).
#include "gemm_common.h"

using namespace moe;

namespace {

constexpr int THREADS = 256;
constexpr int BM = 128;                    // packed rows per tile
constexpr int BN = 512;                    // weight rows per tile
constexpr int BK = 32;                     // k per stage
constexpr int STAGES = 3;
constexpr int ROWB = BK * 2;               // bytes per LDS row (4 chunks of 16 B)
constexpr int X_BYTES = BM * ROWB;         // 8 KB
constexpr int W_BYTES = BN * ROWB;         // 32 KB
constexpr int STAGE_BYTES = X_BYTES + W_BYTES;
constexpr int DMA_BLOCKS = STAGE_BYTES / 1024;      // 1 KB per wave-wide DMA instruction
constexpr int DMA_PER_WAVE = DMA_BLOCKS / 4;         // 10
static_assert(DMA_BLOCKS % 4 == 0, "stage must split evenly over 4 waves");

// physical 16-byte chunk of logical chunk c (0..3) in LDS row r: bijective per row and
// spreads 8 (32 banks) or 16 (64 banks) consecutive rows over distinct banks
__device__ __forceinline__ int swz_chunk(int r, int c) {
  const int f = (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1);
  return c ^ f;
}
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + (swz_chunk(r, c) << 4); }

// GROUPED = false: one group over rows [0, max_rows) (the shared MLP); a separate
// instantiation so that profiles tell the routed and the shared launches apart.
template <bool SWIGLU, bool GROUPED>
__global__ void __launch_bounds__(THREADS, 1)
gemm_bf16_kernel(int G, int Kd, int Nd, const uint16_t* __restrict__ a,
                 const int32_t* __restrict__ row_index, const int32_t* __restrict__ offsets,
                 int max_rows,
                 const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1,
                 uint16_t* __restrict__ out) {
  __shared__ int s_off[kMaxN + 1];
  __shared__ int s_tstart[THREADS + 1];
  __shared__ __attribute__((aligned(1024))) char lds[STAGES * STAGE_BYTES];

  constexpr int COLS = SWIGLU ? BN / 2 : BN;  // output columns per tile
  const int n_tiles = ceil_div(Nd, COLS);
  TileMap tm;
  if (!decode_tile(GROUPED ? offsets : nullptr, G, max_rows, BM, n_tiles, s_off, s_tstart, tm))
    return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n0 = __builtin_amdgcn_readfirstlane(tm.nt * COLS);
  const size_t wstride = static_cast<size_t>(Nd) * Kd;
  const uint16_t* wg = w0 + tm.g * wstride;
  const uint16_t* wu = SWIGLU ? (w1 + tm.g * wstride) : nullptr;

  // DMA sources: instruction i of wave w fills 1 KB block b = 4 i + w of a stage;
  // lane j of it writes 16-byte slot 64 b + j, i.e. (row, physical chunk).
  const uint16_t* src[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int slot = (4 * i + w) * 64 + lane;
    if (slot < X_BYTES / 16) {
      const int r = slot >> 2;
      const int c = swz_chunk(r, slot & 3);
      int row = tm.row0 + min(r, tm.rows - 1);
      if (row_index != nullptr) row = row_index[row];
      src[i] = a + static_cast<size_t>(row) * Kd + c * 8;
    } else {
      const int ws = slot - X_BYTES / 16;
      const int r = ws >> 2;
      const int c = swz_chunk(r, ws & 3);
      const uint16_t* base;
      int n;
      if (SWIGLU) {
        base = (r < BN / 2) ? wg : wu;
        n = n0 + (r & (BN / 2 - 1));
      } else {
        base = wg;
        n = n0 + r;
      }
      src[i] = base + static_cast<size_t>(min(n, Nd - 1)) * Kd + c * 8;
    }
  }
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds_base = static_cast<uint32_t>((size_t)((lds_char*)lds));  // LDS byte offset
  auto issue = [&](int ks) {
    const uint32_t st = lds_base + (ks % STAGES) * STAGE_BYTES + w * 1024;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) dma16(src[i] + ks * BK, st + i * 4096);
  };

  // wave roles: 4 weight blocks of 32 rows x 4 activation blocks of 32 rows
  int wrow[4], ncol[4];
  bool wv[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    wrow[b] = SWIGLU ? ((b < 2) ? 64 * w + 32 * b : BN / 2 + 64 * w + 32 * (b - 2)) : 128 * w + 32 * b;
    ncol[b] = SWIGLU ? n0 + 64 * w + 32 * (b & 1) : n0 + 128 * w + 32 * b;
    wv[b] = ncol[b] < Nd;
  }
  const int xblocks = __builtin_amdgcn_readfirstlane(ceil_div(tm.rows, 32));

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = Kd / BK;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  issue(0);
  if (nk > 1) issue(1);
  for (int ks = 0; ks < nk; ++ks) {
    // stage ks landed (only stage ks + 1 may still be in flight), visible to all waves;
    // the barrier also retires every read of the slot that stage ks + 2 overwrites
    if (ks + 1 < nk) wait_vmcnt<DMA_PER_WAVE>(); else wait_vmcnt<0>();
    __syncthreads();
    if (ks + 2 < nk) issue(ks + 2);
    const char* st = lds + (ks % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kc = 2 * s + lh;
      bf16x8 wa[4], xb[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        wa[b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + X_BYTES + swz(wrow[b] + lr, kc)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xb[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + swz(32 * j + lr, kc)));
      // weight blocks past N_dim hold clamped rows: computed, never stored
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j >= xblocks) break;  // wave-uniform: activation blocks past the tile's rows
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[b], xb[j], acc[b][j], 0, 0, 0);
      }
    }
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
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (!wv[b]) continue;
          const int n = ncol[b] + 8 * q + 4 * lh;
          float h[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) h[u] = silu_f(acc[b][j][4 * q + u]) * acc[b + 2][j][4 * q + u];
          *reinterpret_cast<u32x2*>(orow + n) = u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (!wv[b]) continue;
          const int n = ncol[b] + 8 * q + 4 * lh;
          const floatx16& c = acc[b][j];
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
                const int32_t* __restrict__ row_index, const int32_t* __restrict__ offsets,
                int max_rows, const float* __restrict__ w0,
                const float* __restrict__ w1, float* __restrict__ out) {
  __shared__ int s_off[kMaxN + 1];
  __shared__ int s_tstart[THREADS + 1];
  __shared__ float sa[FBK][FBM + 4];
  __shared__ float sg[FBK][FBN + 4];
  __shared__ float su[FBK][FBN + 4];
  const int n_tiles = ceil_div(Nd, FBN);
  TileMap tm;
  if (!decode_tile(offsets, G, max_rows, FBM, n_tiles, s_off, s_tstart, tm)) return;
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
      int row = tm.row0 + min(r, tm.rows - 1);
      if (row_index != nullptr) row = row_index[row];
      sa[k][r] = a[static_cast<size_t>(row) * Kd + k0 + k];
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
                               const int32_t* row_index, const int32_t* offsets, int max_rows,
                               const void* w0,
                               const void* w1, void* out, hipStream_t stream) {
  const int bm = dt == 1 ? BM : FBM;
  const int cols = dt == 1 ? (swiglu ? BN / 2 : BN) : FBN;
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
      hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
    else if (swiglu)
      hipLaunchKernelGGL((gemm_bf16_kernel<true, false>), g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
    else if (grouped)
      hipLaunchKernelGGL((gemm_bf16_kernel<false, true>), g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
  } else {
    const float* A = static_cast<const float*>(a);
    const float* W0 = static_cast<const float*>(w0);
    const float* W1 = static_cast<const float*>(w1);
    float* O = static_cast<float*>(out);
    if (swiglu)
      hipLaunchKernelGGL(gemm_f32_kernel<true>, g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<false>, g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
  }
  return hipGetLastError();
}
