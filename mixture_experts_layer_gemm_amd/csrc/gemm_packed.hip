// Grouped GEMM with fused SwiGLU over packed ("MFMA-operand order") weights.
//
// Same operation and tile map as the row-major kernels in gemm.hip (expert i owns rows
// [o_i, o_{i+1}), "Section 10: Routing, Capacity, and Load Balancing", Eq. 26; the
// SwiGLU expert of "Section 20: One Shared Expert Is All You Need", Eq. 74), but the
// weights are first stored once in the order in which v_mfma_f32_32x32x16_bf16 consumes
// them as its A operand:
//     packed[g][nb][kb][lane][8] = W[g][32 nb + (lane & 31)][16 kb + 8 (lane >> 5) + 0..7]
// so that one wave-wide 16-byte-per-lane load brings one 32 x 16 operand block (1 KB,
// contiguous) straight into registers. Each wave then streams its four 32-row weight
// blocks as four sequential HBM streams, with no LDS staging, no bank conflicts and no
// barrier on the weight path; a ring of PW k16-steps of weight registers is kept in
// flight. Only the activation tile, shared by the 4 waves, goes through LDS (64-wide
// k stages, 4-deep ring filled by global_load_lds_dwordx4, one barrier per stage).
//
// Workgroup tile: 128 packed rows x 512 weight rows (swiglu: 256 gate + 256 up rows,
// 256 output columns; plain: 512 output columns); wave tile 128 x 128 (256 fp32
// accumulators). The number of active 32-row activation blocks (1..4) is a
// template parameter picked once per tile, so the k loop has no per-block branches.
#include "gemm_common.h"

using namespace moe;

namespace {

constexpr int THREADS = 256;
constexpr int BM = 128;                     // packed rows per tile
constexpr int BN = 512;                     // weight rows per tile
constexpr int BKX = 64;                     // k per activation stage
constexpr int XSTAGES = 4;
constexpr int PW = BKX / 16;                // k16 steps per stage = weight ring depth
constexpr int ROWB = BKX * 2;               // activation row bytes per stage (8 chunks)
constexpr int XSTAGE = BM * ROWB;           // 16 KB
constexpr int XDPW = XSTAGE / 4096;         // DMA instructions per wave per stage

// physical 16-byte chunk of logical chunk c (0..7) of activation row r: conflict-free
// MFMA B-operand reads for both 8-lane (32-bank) and 16-lane (64-bank) LDS phases
__device__ __forceinline__ int xswz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

template <bool SWIGLU, int XBLK>
__device__ __forceinline__ void tile_body(const TileMap& tm, int Kd, int Nd, int lane, int w, int n0,
                                          const u32x4* const* ws, const uint16_t* const* xsrc,
                                          char* lds, uint16_t* __restrict__ out) {
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds_base = static_cast<uint32_t>((size_t)((lds_char*)lds));
  const int lr = lane & 31, lh = lane >> 5;
  const int KB = Kd / 16;
  const int nst = Kd / BKX;
  auto issue_x = [&](int st) {
    const uint32_t dst = lds_base + (st % XSTAGES) * XSTAGE + w * 1024;
#pragma unroll
    for (int i = 0; i < XDPW; ++i) dma16(xsrc[i] + st * BKX, dst + i * 4096);
  };
  floatx16 acc[4][XBLK];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < XBLK; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  for (int p = 0; p < XSTAGES - 1 && p < nst; ++p) issue_x(p);
  u32x4 wr[PW][4];
#pragma unroll
  for (int u = 0; u < PW; ++u)
#pragma unroll
    for (int b = 0; b < 4; ++b) wr[u][b] = ws[b][(size_t)u * 64];

  for (int st = 0; st < nst; ++st) {
    // activation stage st has landed (later stages and the weight loads issued during
    // the previous stage may still be in flight); the barrier publishes it and retires
    // every read of the slot that stage st + XSTAGES - 1 overwrites
    const int ahead = min(nst - 1 - st, XSTAGES - 2);
    if (ahead >= 2) wait_vmcnt<2 * XDPW + 4 * PW>();
    else if (ahead == 1) wait_vmcnt<XDPW + 4 * PW>();
    else wait_vmcnt<4 * PW>();
    __syncthreads();
    if (st + XSTAGES - 1 < nst) issue_x(st + XSTAGES - 1);
    const char* xs = lds + (st % XSTAGES) * XSTAGE;
    const int nbase = min((st + 1) * PW, KB - PW);   // refill target, clamped (no branch)
    auto xread = [&](int u, bf16x8* xb) {
      const int kc = 2 * u + lh;
#pragma unroll
      for (int j = 0; j < XBLK; ++j) {
        const int r = 32 * j + lr;
        xb[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + r * ROWB + (xswz(r, kc) << 4)));
      }
    };
    bf16x8 xb[2][XBLK];
    xread(0, xb[0]);
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int cur = u & 1;
      if (u + 1 < PW) xread(u + 1, xb[cur ^ 1]);
      __builtin_amdgcn_sched_barrier(0);  // keep the next step's LDS reads ahead of these MFMAs
#pragma unroll
      for (int j = 0; j < XBLK; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wr[u][b]),
                                                              xb[cur][j], acc[b][j], 0, 0, 0);
#pragma unroll
      for (int b = 0; b < 4; ++b) wr[u][b] = ws[b][(size_t)(nbase + u) * 64];
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: lane holds row (32 j + lr) and columns 8 q + 4 lh + {0..3} of each block
#pragma unroll
  for (int j = 0; j < XBLK; ++j) {
    const int m = 32 * j + lr;
    if (m >= tm.rows) continue;
    uint16_t* orow = out + static_cast<size_t>(tm.row0 + m) * Nd;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (SWIGLU) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int n = n0 + 64 * w + 32 * b + 8 * q + 4 * lh;
          if (n >= Nd) continue;
          float h[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) h[u] = silu_f(acc[b][j][4 * q + u]) * acc[b + 2][j][4 * q + u];
          *reinterpret_cast<u32x2*>(orow + n) = u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int n = n0 + 128 * w + 32 * b + 8 * q + 4 * lh;
          if (n >= Nd) continue;
          const floatx16& c = acc[b][j];
          *reinterpret_cast<u32x2*>(orow + n) =
              u32x2{pack_bf16x2(c[4 * q], c[4 * q + 1]), pack_bf16x2(c[4 * q + 2], c[4 * q + 3])};
        }
      }
    }
  }
}

// GROUPED = false: one group over rows [0, max_rows) (the shared MLP).
template <bool SWIGLU, bool GROUPED>
__global__ void __launch_bounds__(THREADS, 1)
gemm_packed_kernel(int G, int Kd, int Nd, const uint16_t* __restrict__ a,
                   const int32_t* __restrict__ row_index, const int32_t* __restrict__ offsets,
                   int max_rows,
                   const uint16_t* __restrict__ w0p, const uint16_t* __restrict__ w1p,
                   uint16_t* __restrict__ out) {
  __shared__ int s_off[kMaxN + 1];
  __shared__ int s_tstart[THREADS + 1];
  __shared__ __attribute__((aligned(1024))) char lds[XSTAGES * XSTAGE];
  constexpr int COLS = SWIGLU ? BN / 2 : BN;
  const int n_tiles = ceil_div(Nd, COLS);
  TileMap tm;
  if (!decode_tile(GROUPED ? offsets : nullptr, G, max_rows, BM, n_tiles, s_off, s_tstart, tm))
    return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = __builtin_amdgcn_readfirstlane(tm.nt * COLS);
  const int KB = Kd / 16;
  const size_t gstride = static_cast<size_t>(Nd) * Kd;
  // this wave's four weight streams (32-row blocks); blocks past N_dim are clamped and
  // their results never stored
  const u32x4* ws[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint16_t* base;
    int nb;
    if (SWIGLU) {
      base = (b < 2 ? w0p : w1p) + tm.g * gstride;
      nb = n0 / 32 + 2 * w + (b & 1);
    } else {
      base = w0p + tm.g * gstride;
      nb = n0 / 32 + 4 * w + b;
    }
    nb = min(nb, Nd / 32 - 1);
    ws[b] = reinterpret_cast<const u32x4*>(base) + static_cast<size_t>(nb) * KB * 64 + lane;
  }
  // activation DMA: instruction i of wave w fills 1 KB block 4 i + w of a stage; with a
  // row index the packed row r is gathered from activation row row_index[r]
  const uint16_t* xsrc[XDPW];
#pragma unroll
  for (int i = 0; i < XDPW; ++i) {
    const int slot = (4 * i + w) * 64 + lane;
    const int r = slot >> 3, c = xswz(r, slot & 7);
    int src = tm.row0 + min(r, tm.rows - 1);
    if (row_index != nullptr) src = row_index[src];
    xsrc[i] = a + static_cast<size_t>(src) * Kd + c * 8;
  }
  const int xblocks = __builtin_amdgcn_readfirstlane(ceil_div(tm.rows, 32));
  switch (xblocks) {
    case 1: tile_body<SWIGLU, 1>(tm, Kd, Nd, lane, w, n0, ws, xsrc, lds, out); break;
    case 2: tile_body<SWIGLU, 2>(tm, Kd, Nd, lane, w, n0, ws, xsrc, lds, out); break;
    case 3: tile_body<SWIGLU, 3>(tm, Kd, Nd, lane, w, n0, ws, xsrc, lds, out); break;
    default: tile_body<SWIGLU, 4>(tm, Kd, Nd, lane, w, n0, ws, xsrc, lds, out); break;
  }
}

// [G][N][K] row-major -> [G][N/32][K/16][64][8]
__global__ void __launch_bounds__(256)
pack_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ p, long pieces, int N, int K) {
  const int KB = K / 16, NB = N / 32;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < pieces; i += (long)gridDim.x * 256) {
    const int lane = static_cast<int>(i & 63);
    long blk = i >> 6;
    const int kb = static_cast<int>(blk % KB);
    blk /= KB;
    const int nb = static_cast<int>(blk % NB);
    const long g = blk / NB;
    const int row = nb * 32 + (lane & 31), k = kb * 16 + (lane >> 5) * 8;
    reinterpret_cast<u32x4*>(p)[i] = *reinterpret_cast<const u32x4*>(w + (g * N + row) * static_cast<long>(K) + k);
  }
}

}  // namespace

hipError_t launch_grouped_gemm_packed(bool swiglu, int G, int Kd, int Nd, const void* a,
                                      const int32_t* row_index, const int32_t* offsets,
                                      int max_rows, const void* w0p,
                                      const void* w1p, void* out, hipStream_t stream) {
  const int cols = swiglu ? BN / 2 : BN;
  const int n_tiles = (Nd + cols - 1) / cols;
  const long max_m = static_cast<long>(max_rows) / BM + G + 1;
  long grid = (max_m * n_tiles + 7) / 8 * 8;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  const dim3 g(static_cast<unsigned>(grid)), b(THREADS);
  const uint16_t* A = static_cast<const uint16_t*>(a);
  const uint16_t* W0 = static_cast<const uint16_t*>(w0p);
  const uint16_t* W1 = static_cast<const uint16_t*>(w1p);
  uint16_t* O = static_cast<uint16_t*>(out);
  const bool grouped = offsets != nullptr;
  if (swiglu && grouped)
    hipLaunchKernelGGL((gemm_packed_kernel<true, true>), g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
  else if (swiglu)
    hipLaunchKernelGGL((gemm_packed_kernel<true, false>), g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
  else if (grouped)
    hipLaunchKernelGGL((gemm_packed_kernel<false, true>), g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
  else
    hipLaunchKernelGGL((gemm_packed_kernel<false, false>), g, b, 0, stream, G, Kd, Nd, A, row_index, offsets, max_rows, W0, W1, O);
  return hipGetLastError();
}

hipError_t launch_pack_weights(int G, int N, int K, const void* w, void* w_packed, hipStream_t stream) {
  const long pieces = static_cast<long>(G) * N * K / 8;
  long grid = (pieces + 255) / 256;
  if (grid > 16384) grid = 16384;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(w), static_cast<uint16_t*>(w_packed), pieces, N, K);
  return hipGetLastError();
}
