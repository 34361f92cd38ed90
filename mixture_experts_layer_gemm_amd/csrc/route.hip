// Router: logits z = x W_r^T (+ b), scores, top-K selection and routed coefficients.
//
// Follows "Section 21: Merging Routed and Shared Expert Activations" (Eq. 80, 83) and
// "Appendix E: Expert-Merge Normalization in Public MoE Models" (Table 52) for the
// score rules, and the router projection of "Shared and Fine-Grained Experts" (a
// bias-free linear layer from d_model to N).
//
// One workgroup owns BT tokens. Phase 1 computes the BT x N logit tile in one of three
// ways: for bf16 with 33 to 128 logit columns, 16 tokens and 16 waves with both operands
// staged through an LDS ring (logits_lds); for 128 < N <= 256 without a gate, split-K
// partial logits from a separate kernel (logits_split_kernel), added here in a fixed
// order; otherwise (16 tokens and 8 waves up to 128 columns, 32 tokens and 4 waves
// beyond) v_mfma_f32_16x16x32_bf16 with the d_model reduction split round-robin over the
// waves in 32-wide steps, operands loaded straight from global memory into the MFMA lane
// layout several steps at a time, and the per-wave partial tiles summed in LDS in a fixed
// order. Phase 2 gives each wave BT / waves tokens: top-K by ranks of packed
// (ordered float key, inverted expert index) 64-bit values, which put the lowest index
// first on ties, then the coefficients in the lanes k < K. For N > 64 (several keys per
// lane) the ranks are counted only among the keys at or above a threshold: the K-th
// largest of the 64 per-lane maxima. K distinct keys reach it, so the K largest keys all
// do, and at most K lanes, hence K * N / 64 keys, can hold keys that reach it.
//
// Auxiliary-loss-free balancing ("Section 10: Routing, Capacity, and Load Balancing",
// Eq. 35): with a persistent expert bias b the keys become z + b (softmax rules) or
// sigmoid(z) + b (sigmoid affinities), summed in fp32, while the coefficients are still
// computed from the unbiased logits of the selected experts.
#include <utility>

#include "common.h"
#include "gemm_common.h"

using namespace moe;

namespace {


// Order-preserving map float -> uint32 (larger float, larger key); -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord_key(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Butterfly sum: every lane ends with the same, run-to-run deterministic value
// (each stage adds a + b on one lane and b + a on its partner, which are equal).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float sigmoid_f(float v) { return 1.0f / (1.0f + expf(-v)); }

// orders this wave's LDS writes before its later LDS reads (lanes of one wave only)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Writes the experts of the K largest packed keys to sel[0..K-1], largest first. Lane l
// holds the keys of experts l + 64 j in mine[j] (0 where l + 64 j >= N; every valid key
// is nonzero and all valid keys are distinct). key is this wave's LDS scratch of kMaxN
// entries; sel is read back after a wave_lds_sync().
__device__ __forceinline__ void select_topk(const uint64_t (&mine)[kMaxN / kWave], int N, int K,
                                            int lane, uint64_t* key, int* sel) {
  if (N <= kWave) {  // one key per lane: rank among all N
    key[lane] = mine[0];
    wave_lds_sync();
    int rank = 0;
#pragma unroll 8
    for (int i = 0; i < N; ++i) rank += key[i] > mine[0] ? 1 : 0;  // broadcast reads
    if (lane < N && rank < K) sel[rank] = lane;
    return;
  }
  // threshold: the K-th largest of the per-lane maxima (every lane holds a valid key)
  uint64_t lmax = mine[0];
#pragma unroll
  for (int j = 1; j < kMaxN / kWave; ++j) lmax = mine[j] > lmax ? mine[j] : lmax;
  key[lane] = lmax;
  wave_lds_sync();
  int r = 0;
#pragma unroll 8
  for (int i = 0; i < kWave; ++i) r += key[i] > lmax ? 1 : 0;
  if (r == K - 1) key[kWave] = lmax;  // slot 64: read by no lane above
  wave_lds_sync();
  const uint64_t theta = key[kWave];
  // candidates (keys >= theta, at most K * (kMaxN / 64) <= 64) packed into slots 128..
  uint64_t* cand = key + 2 * kWave;
  int nc = 0;
#pragma unroll
  for (int j = 0; j < kMaxN / kWave; ++j) {
    const bool c = mine[j] >= theta;
    const uint64_t b = __ballot(c);
    if (c) cand[nc + __popcll(b & ((1ull << lane) - 1ull))] = mine[j];
    nc += __popcll(b);
  }
  wave_lds_sync();
  if (lane < nc) {
    const uint64_t mk = cand[lane];
    int rank = 0;
    for (int i = 0; i < nc; ++i) rank += cand[i] > mk ? 1 : 0;
    if (rank < K) sel[rank] = static_cast<int>(~static_cast<uint32_t>(mk));
  }
}

// ---- phase 1, bf16: MFMA logits into part[w][BT][ldz] -----------------------------
// Wave w owns the 32-wide k steps w, w + WAVES, ...; U steps at a time it first issues
// every operand load (x rows and router rows, straight into the MFMA lane layout), then
// the MFMAs, so U * (RB + NB) 16-byte loads per lane are in flight at once.
template <int BT, int NBT, int WAVES, int U>
__device__ void logits_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                            const uint16_t* __restrict__ wgate, int T, int d, int N, int NB,
                            int t0, float* part, int ldz) {
  constexpr int RB = BT / 16;  // 16-row token blocks
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int row = lane & 15;
  const int kq = (lane >> 4) * 8;
  const uint16_t* xr[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    xr[rb] = x + static_cast<size_t>(min(t0 + 16 * rb + row, T - 1)) * d + kq;
  const uint16_t* br[NBT];
#pragma unroll
  for (int nb = 0; nb < NBT; ++nb) {
    const int n = nb * 16 + row;
    const uint16_t* p = wr;  // padding columns read row 0; their results are dropped
    if (n < N) p = wr + static_cast<size_t>(n) * d;
    else if (n == N && wgate != nullptr) p = wgate;
    br[nb] = p + kq;
  }
  floatx4 acc[RB][NBT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NBT; ++nb) acc[rb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nks = d / 32;
  for (int ks0 = w; ks0 < nks; ks0 += WAVES * U) {
    u32x4 av[U][RB], bv[U][NBT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = min(ks0 + u * WAVES, nks - 1);  // clamped re-read, results skipped below
      const int k0 = ks * 32;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) av[u][rb] = *reinterpret_cast<const u32x4*>(xr[rb] + k0);
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb)
        if (nb < NB) bv[u][nb] = *reinterpret_cast<const u32x4*>(br[nb] + k0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ks0 + u * WAVES >= nks) break;
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb) {
        if (nb < NB) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, av[u][rb]), __builtin_bit_cast(bf16x8, bv[u][nb]),
                acc[rb][nb], 0, 0, 0);
        }
      }
    }
  }
  // D layout of 16x16: lane holds column (lane & 15), rows 4*(lane >> 4) + j.
  float* pw = part + w * BT * ldz;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NBT; ++nb) {
      if (nb < NB) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pw[(16 * rb + (lane >> 4) * 4 + j) * ldz + nb * 16 + row] = acc[rb][nb][j];
      }
    }
}

// ---- phase 1, f32: one wave per (token, column) dot product -----------------------
template <int BT, int WAVES>
__device__ void logits_f32(const float* __restrict__ x, const float* __restrict__ wr,
                           const float* __restrict__ wgate, int T, int d, int N, int ncol,
                           int t0, float* z, int ldz) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int p = w; p < BT * ncol; p += WAVES) {
    const int t = p / ncol, n = p % ncol;
    const int tok = min(t0 + t, T - 1);
    const float* xr = x + static_cast<size_t>(tok) * d;
    const float* wrow = (n < N) ? wr + static_cast<size_t>(n) * d : wgate;
    float acc = 0.f;
    for (int k = lane; k < d; k += kWave) acc = fmaf(xr[k], wrow[k], acc);
    acc = wave_sum(acc);
    if (lane == 0) z[t * ldz + n] = acc;
  }
}

// ---- phase 1 for many experts (128 < N <= 256, bf16): split-K logits ----------------
// Each workgroup of 4 waves computes partial logits of LS_BT tokens x all N experts over
// one of P equal slices of d_model; the route kernel then adds the P slices in a fixed
// order. Wave w owns experts 64 w .. 64 w + 63 (two 32-row blocks of W_r, packed once per
// call into the MFMA operand layout and loaded straight from global memory into
// v_mfma_f32_32x32x16_bf16 A-operand registers, four stages ahead, 1 KB per load)
// against all LS_BT tokens (x staged through a 4-stage LDS ring by direct-to-LDS loads,
// XOR-swizzled chunks). Every W_r byte of a slice enters a compute unit once per 128
// tokens instead of once per 32. Every stage issues the same loads (past the last stage
// the last stage's addresses again), so one vmcnt wait per stage covers what it reads.
constexpr int kRouteMaxSlices = 4;                   // d_model slices (partial logits)
constexpr int LS_BT = 128;                           // tokens per workgroup
constexpr int LS_BK = 64;                            // k per stage
constexpr int LS_XS = 4;                             // x ring depth (stages)
constexpr int LS_XSTAGE = LS_BT * LS_BK * 2;         // bytes per x stage
constexpr int LS_XDPW = LS_XSTAGE / (1024 * 4);      // direct-to-LDS loads per wave per stage
constexpr int LS_WPS = 2 * (LS_BK / 16);             // W_r loads per wave per stage
constexpr int LS_PER = LS_XDPW + LS_WPS;
constexpr int LS_RS = 4;                             // W_r stages in flight
// ops issued after the W_r (resp. x) loads of stage s when stage s begins
constexpr int LS_WAITN = (LS_RS - 1) * LS_PER < LS_WPS + (LS_XS - 2) * LS_PER
                             ? (LS_RS - 1) * LS_PER : LS_WPS + (LS_XS - 2) * LS_PER;
static_assert(LS_WAITN <= 63, "vmcnt range");

__device__ __forceinline__ int ls_swz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

// (non-temporal: x is read once, so it should not push W_r out of L2)
__device__ __forceinline__ void ls_dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
// 16-byte load into registers the compiler does not track (read after the stage wait)
template <int OFF>
__device__ __forceinline__ void ls_ldg16(u32x4& dst, const void* sbase, uint32_t voff) {
  asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3"
               : "=v"(dst)
               : "v"(voff), "s"(sbase), "i"(OFF)
               : "memory");
}
template <typename F, int... I>
__device__ __forceinline__ void ls_unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void ls_unroll(F&& f) {
  ls_unroll_impl(f, std::make_integer_sequence<int, N>{});
}

// grid (ceil(T / LS_BT), P); part[p][t][n] = sum over slice p of x[t][k] W_r[n][k];
// N a multiple of 64, kslice = d / P a multiple of LS_RS LS_BK; wpk is W_r in the
// moe_pack_weights layout (the A operand of v_mfma_f32_32x32x16_bf16, 1 KB per 32 rows
// x 16 k, contiguous along k for each 32-row block)
__global__ void __launch_bounds__(256, 1)
logits_split_kernel(int T, int d, int N, int kslice, const uint16_t* __restrict__ x,
                    const uint16_t* __restrict__ wpk, float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) char lds[LS_XS * LS_XSTAGE];
  typedef __attribute__((address_space(3))) char lds_char;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * LS_BT;
  const int kp = blockIdx.y;
  const int nst = kslice / LS_BK;
  const uint32_t lds_base = static_cast<uint32_t>((size_t)((lds_char*)lds));
  const uint32_t rowb = static_cast<uint32_t>(d) * 2u;
  const char* xs0 = reinterpret_cast<const char*>(x) + static_cast<size_t>(kp) * kslice * 2;
  // this slice's first 16-wide k step within each packed 32-row block
  const char* ws0 = reinterpret_cast<const char*>(wpk) + static_cast<size_t>(kp) * (kslice / 16) * 1024;
  // x: load i of wave w brings tile rows 8 (4 i + w) .. + 7, lane j row 8 (4 i + w) + (j >> 3),
  // physical chunk j & 7 (rows past T repeat row T - 1)
  uint32_t xo[LS_XDPW];
#pragma unroll
  for (int i = 0; i < LS_XDPW; ++i) {
    const int row = (4 * i + wv) * 8 + (lane >> 3);
    xo[i] = static_cast<uint32_t>(min(t0 + row, T - 1)) * rowb +
            static_cast<uint32_t>(ls_swz(row, lane & 7) << 4);
  }
  // W_r: block b of this wave is packed 32-row block 2 w + b (past N: the last block,
  // computed and never stored); each k16 step of a block is 1 KB, 16 bytes per lane
  uint32_t wo[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
    wo[b] = static_cast<uint32_t>(min(2 * wv + b, N / 32 - 1)) * 32u * rowb +
            static_cast<uint32_t>(lane) * 16u;
  // LDS byte offset of this lane's x fragment for k16 step u (token block 0)
  uint32_t xoff[LS_BK / 16];
#pragma unroll
  for (int u = 0; u < LS_BK / 16; ++u)
    xoff[u] = static_cast<uint32_t>(lr * (LS_BK * 2) + (ls_swz(lr, 2 * u + lh) << 4));

  auto issue_x = [&](int ks, int slot) {
    const char* sb = xs0 + static_cast<size_t>(ks) * (LS_BK * 2);
    const uint32_t dst = lds_base + slot * LS_XSTAGE + wv * 1024;
#pragma unroll
    for (int i = 0; i < LS_XDPW; ++i) ls_dma16(xo[i], sb, dst + i * 4096);
  };
  u32x4 wrg[LS_RS][LS_BK / 16][2];
  auto issue_w = [&](u32x4 (&dst)[LS_BK / 16][2], int ks, auto uc) {
    constexpr int u = decltype(uc)::value;
    const char* sb = ws0 + static_cast<size_t>(ks) * ((LS_BK / 16) * 1024);
    ls_ldg16<u * 1024>(dst[u][0], sb, wo[0]);
    ls_ldg16<u * 1024>(dst[u][1], sb, wo[1]);
  };
  // prologue: the loads of virtual stages -V..-1 (targets clamped to the last stage), in
  // the order a steady stage issues them
  constexpr int V = (LS_XS - 1) > LS_RS ? (LS_XS - 1) : LS_RS;
  ls_unroll<V>([&](auto vc) {
    constexpr int v = decltype(vc)::value - V;
    constexpr int xs_t = v + LS_XS - 1;
    if constexpr (xs_t >= 0) issue_x(min(xs_t, nst - 1), xs_t);
    constexpr int ws_t = v + LS_RS;
    if constexpr (ws_t >= 0) {
      const int ks = min(ws_t, nst - 1);
      ls_unroll<LS_BK / 16>([&](auto uc) { issue_w(wrg[ws_t], ks, uc); });
    }
  });

  floatx16 acc[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[b][j][v] = 0.f;

  for (int s0 = 0; s0 < nst; s0 += LS_RS) {
    ls_unroll<LS_RS>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      const int s = s0 + r;
      wait_vmcnt<LS_WAITN>();
      __syncthreads();
      // past the end: the last stage again (loaded, never read)
      issue_x(min(s + LS_XS - 1, nst - 1), (s + LS_XS - 1) % LS_XS);
      const int ts = min(s + LS_RS, nst - 1);
      const char* xt = lds + (s % LS_XS) * LS_XSTAGE;
      bf16x8 xv[2][4];
      auto xread = [&](int u, bf16x8* v) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[j] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(xt + xoff[u] + j * (32 * LS_BK * 2)));
      };
      xread(0, xv[0]);
      ls_unroll<LS_BK / 16>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u + 1 < LS_BK / 16) xread(u + 1, xv[(u + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, wrg[r][u][b]), xv[u & 1][j], acc[b][j], 0, 0, 0);
        issue_w(wrg[r], ts, uc);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  }
  wait_vmcnt<0>();  // no load may land after the workgroup ends
  // lane (lr, lh) holds token 32 j + lr, experts 64 w + 32 b + 8 q + 4 lh + {0..3}. N is a
  // multiple of 64, so a wave's experts are all real or (past N) all absent: absent ones
  // store nothing (their rows would land in the next token's)
  if (64 * wv >= N) return;
  float* pp = part + static_cast<size_t>(kp) * T * N;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 32 * j + lr;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 64 * wv + 32 * b + 8 * q + 4 * lh;
        *reinterpret_cast<floatx4*>(pp + static_cast<size_t>(t) * N + n) =
            floatx4{acc[b][j][4 * q], acc[b][j][4 * q + 1], acc[b][j][4 * q + 2],
                    acc[b][j][4 * q + 3]};
      }
  }
}


// ---- phase 1, bf16, up to 128 logit columns: both operands staged through LDS ------------
// The 16 x rows and the (padded) router rows of a k stage are brought into an LDS ring by
// direct-to-LDS loads of whole row pieces (16-byte chunks XOR-swizzled by row), several
// stages ahead, each load moving 1 KB of full row pieces; wave w then runs
// v_mfma_f32_16x16x32_bf16 on k32 step (w mod KS) of each stage for every (WAVES / KS)-th
// column block from LDS. The KS per-step partial tiles are added in a fixed order into
// the logits tile.
constexpr int LP_BT = 16;             // tokens per workgroup
constexpr int LP_BK = 128;            // k per stage
constexpr int LP_ROWB = LP_BK * 2;    // bytes per staged row piece
constexpr int LP_CPR = LP_ROWB / 16;  // 16-byte chunks per row piece
constexpr int LP_RPL = 64 / LP_CPR;   // row pieces per 1 KB load
constexpr int LP_KS = LP_BK / 32;     // k32 steps per stage
static_assert(LP_CPR >= 16 && LP_CPR <= 64 && LP_KS <= 8, "stage width");

template <int NBT, int WAVES>
struct LpCfg {
  static constexpr int WPQ = WAVES / LP_KS;     // waves per k32 step
  static constexpr int NC = NBT * 16;           // staged router rows (padded)
  static constexpr int ROWS = LP_BT + NC;       // staged rows per stage
  static constexpr int STAGE = ROWS * LP_ROWB;  // bytes per stage
  static constexpr int NI = ROWS / LP_RPL;      // 1 KB loads per stage
  static constexpr int M = (NI + WAVES - 1) / WAVES;  // loads per wave per stage
  static constexpr int S = NBT <= 4 ? 4 : 3;    // ring depth (stages)
  static constexpr int WAITN = (S - 2) * M;     // loads still in flight when a stage starts
  static constexpr int LDZ = NC + 1;
  static constexpr int RING = S * STAGE;
  static constexpr int NJ = (NBT + WPQ - 1) / WPQ;  // column blocks per wave
  static_assert(WAVES % LP_KS == 0, "whole k32 steps per wave group");
  static_assert((LP_KS + 1) * LP_BT * LDZ * 4 <= RING, "partial tiles and logits fit the ring");
  static_assert(WAITN < 64, "vmcnt range");
};

// bf16 logits of tokens t0 .. t0 + 15 into z = ring + KS partial tiles ([16][LDZ] floats,
// columns < ncol valid); d a multiple of LP_BK; returns z
template <int NBT, int WAVES>
__device__ float* logits_lds(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                             const uint16_t* __restrict__ wgate, const float* __restrict__ logit_bias,
                             int T, int d, int N, int NB, int ncol, int t0, char* ring) {
  typedef LpCfg<NBT, WAVES> C;
  typedef __attribute__((address_space(3))) char lds_char;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nst = d / LP_BK;
  const uint32_t ring_base = static_cast<uint32_t>((size_t)((lds_char*)ring));
  // this lane's source of each of its M loads: load i = w + WAVES u (past NI: load NI - 1
  // again, the same bytes to the same place) brings staged rows RPL i .. RPL i + RPL - 1,
  // lane l row RPL i + l / CPR, physical chunk l % CPR = logical chunk (l % CPR) ^ (row & 15)
  const char* src[C::M];
  uint32_t dst[C::M];
#pragma unroll
  for (int u = 0; u < C::M; ++u) {
    const int i = min(w + WAVES * u, C::NI - 1);
    const int row = LP_RPL * i + lane / LP_CPR;
    const int lc = (lane % LP_CPR) ^ (row & 15);
    const uint16_t* rp;
    if (row < LP_BT) {
      rp = x + static_cast<size_t>(min(t0 + row, T - 1)) * d;
    } else {
      const int n = row - LP_BT;  // padding rows read router row 0; their columns are dropped
      rp = n < N ? wr + static_cast<size_t>(n) * d : (n == N && wgate != nullptr ? wgate : wr);
    }
    src[u] = reinterpret_cast<const char*>(rp) + lc * 16;
    dst[u] = ring_base + static_cast<uint32_t>(i) * 1024u;
  }
  // workgroup b walks the k stages from stage b mod nst (wrapping), so workgroups running
  // side by side read different k ranges of W_r
  const int skew = static_cast<int>(blockIdx.x % static_cast<unsigned>(nst));
  auto issue = [&](int ks, int slot) {
    const int kk = ks + skew < nst ? ks + skew : ks + skew - nst;
#pragma unroll
    for (int u = 0; u < C::M; ++u)
      dma16(src[u] + static_cast<size_t>(kk) * LP_ROWB, dst[u] + slot * C::STAGE);
  };
  // operand LDS offset (within a stage) of this lane for its k32 step q
  const int q = w % LP_KS, cb0 = w / LP_KS;
  const int lr = lane & 15, lcq = q * 4 + (lane >> 4);
  const uint32_t a_off = static_cast<uint32_t>(lr * LP_ROWB + ((lcq ^ lr) << 4));
  floatx4 acc[C::NJ];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < C::S - 1; ++v) issue(min(v, nst - 1), v);
  for (int s = 0; s < nst; ++s) {
    wait_vmcnt<C::WAITN>();
    __syncthreads();
    // past the end: the last stage again into a slot no stage still needs
    issue(min(s + C::S - 1, nst - 1), (s + C::S - 1) % C::S);
    const char* st = ring + (s % C::S) * C::STAGE;
    const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + a_off));
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int nb = cb0 + C::WPQ * j;
      if (nb < NB) {
        const bf16x8 bv = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(st + (LP_BT + 16 * nb) * LP_ROWB + a_off));
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[j], 0, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();  // the repeated last-stage loads too
  __syncthreads();
  // partial tile of k32 step q: lane holds column (lane & 15), rows 4 (lane >> 4) + j
  float* part = reinterpret_cast<float*>(ring);
  float* pq = part + q * LP_BT * C::LDZ;
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    const int nb = cb0 + C::WPQ * j;
    if (nb < NB) {
#pragma unroll
      for (int e = 0; e < 4; ++e) pq[(4 * (lane >> 4) + e) * C::LDZ + nb * 16 + lr] = acc[j][e];
    }
  }
  __syncthreads();
  float* z = part + LP_KS * LP_BT * C::LDZ;
  for (int i = tid; i < LP_BT * ncol; i += blockDim.x) {
    const int t = i / ncol, n = i % ncol;
    const int o = t * C::LDZ + n;
    float v = part[o];  // fixed order: k32 steps 0, 1, ...
#pragma unroll
    for (int qq = 1; qq < LP_KS; ++qq) v += part[qq * LP_BT * C::LDZ + o];
    if (n < N && logit_bias != nullptr) v += logit_bias[n];
    z[o] = v;
  }
  return z;
}

// TILE_ONLY: logits come from memory (logits_mode 1 or 2), so LDS holds the one final
// tile instead of a partial tile per wave
// LDSP: bf16 logits by logits_lds (16 tokens), the tile and partials in its ring
template <int BT, int NBT, int WAVES, int U, bool TILE_ONLY = false, bool LDSP = false>
__global__ void __launch_bounds__(WAVES * 64)
route_kernel(int T, int d, int N, int K, int score, int renorm, float alpha, int dt,
             const void* __restrict__ x, const void* __restrict__ w_router,
             const float* __restrict__ logit_bias, const float* __restrict__ sel_bias,
             const void* __restrict__ w_gate_vec,
             float* __restrict__ logits, int logits_mode, int32_t* __restrict__ topk_idx,
             float* __restrict__ topk_r, float* __restrict__ s_tok,
             const float* __restrict__ part, int nparts, int32_t* __restrict__ hist,
             int32_t* __restrict__ loc_rank) {
  constexpr int THREADS = WAVES * 64;
  static_assert(BT <= 32, "one 32-bit token mask per expert");
  constexpr int ldz = NBT * 16 + 1;
  static_assert(!LDSP || BT == LP_BT, "staged logits: 16 tokens");
  // bf16 path: a partial tile per wave; TILE_ONLY: the one tile; staged path: the LDS ring
  // (partials and tile in it)
  __shared__ float smem[LDSP ? 1 : (TILE_ONLY ? 1 : WAVES) * BT * ldz];
  __shared__ __attribute__((aligned(1024))) char ring[LDSP ? LpCfg<NBT, WAVES>::RING : 16];
  float* z = smem;  // final logits tile [BT][ldz]
  const int t0 = blockIdx.x * BT;
  const int tid = threadIdx.x;
  const bool has_gate = (w_gate_vec != nullptr) && logits_mode == 0;
  const int ncol = N + (has_gate ? 1 : 0);
  // the tile's count (hist != nullptr): a 32-bit token mask per expert, OR-ed in LDS
  __shared__ uint32_t s_mask[kMaxN];
  __shared__ int s_tsel[BT][kMaxK];
  if (hist != nullptr)
    for (int i = tid; i < kMaxN; i += THREADS) s_mask[i] = 0u;

  if (logits_mode == 1) {
    for (int i = tid; i < BT * N; i += THREADS) {
      const int t = i / N, n = i % N;
      if (t0 + t < T) z[t * ldz + n] = logits[static_cast<size_t>(t0 + t) * N + n];
    }
  } else if (logits_mode == 2) {
    // the split-K slices of logits_split_kernel, added in slice order, then the bias; a
    // thread's loads for EPT elements of every slice are all issued before any sum
    constexpr int EPT = 8;
    const size_t slice = static_cast<size_t>(T) * N;
    for (int i0 = tid; i0 < BT * N; i0 += THREADS * EPT) {
      float pv[kRouteMaxSlices][EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = i0 + e * THREADS;
        const bool ok = i < BT * N && t0 + i / N < T;
        const size_t o = ok ? static_cast<size_t>(t0) * N + i : 0;
#pragma unroll
        for (int q = 0; q < kRouteMaxSlices; ++q)
          pv[q][e] = (ok && q < nparts) ? part[q * slice + o] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = i0 + e * THREADS;
        if (i < BT * N && t0 + i / N < T) {
          const int t = i / N, n = i % N;
          float v = pv[0][e];
#pragma unroll
          for (int q = 1; q < kRouteMaxSlices; ++q)
            if (q < nparts) v += pv[q][e];
          if (logit_bias != nullptr) v += logit_bias[n];
          z[t * ldz + n] = v;
        }
      }
    }
  } else if (TILE_ONLY) {
    return;  // not launched for logits computed here
  } else if (LDSP) {
    z = logits_lds<NBT, WAVES>(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                        static_cast<const uint16_t*>(w_gate_vec), logit_bias, T, d, N,
                        (ncol + 15) / 16, ncol, t0, ring);
  } else if (dt == 1) {
    const int NB = (ncol + 15) / 16;
    logits_bf16<BT, NBT, WAVES, U>(static_cast<const uint16_t*>(x),
                                   static_cast<const uint16_t*>(w_router),
                                   static_cast<const uint16_t*>(w_gate_vec), T, d, N, NB, t0,
                                   smem, ldz);
    __syncthreads();
    const int S = BT * ldz;
    for (int i = tid; i < BT * ncol; i += THREADS) {
      const int t = i / ncol, n = i % ncol;
      const int o = t * ldz + n;
      float v = smem[o];  // fixed summation order: wave 0, 1, 2, ...
#pragma unroll
      for (int q = 1; q < WAVES; ++q) v += smem[q * S + o];
      if (n < N && logit_bias != nullptr) v += logit_bias[n];
      z[o] = v;
    }
  } else {
    logits_f32<BT, WAVES>(static_cast<const float*>(x), static_cast<const float*>(w_router),
                          static_cast<const float*>(w_gate_vec), T, d, N, ncol, t0, z, ldz);
    __syncthreads();
    if (logit_bias != nullptr)
      for (int i = tid; i < BT * N; i += THREADS) z[(i / N) * ldz + i % N] += logit_bias[i % N];
  }
  __syncthreads();

  if (logits_mode != 1 && logits != nullptr) {
    for (int i = tid; i < BT * N; i += THREADS) {
      const int t = i / N, n = i % N;
      if (t0 + t < T) logits[static_cast<size_t>(t0 + t) * N + n] = z[t * ldz + n];
    }
  }

  // ---- phase 2: top-K and coefficients, one wave per token --------------------------
  // Selection by rank (select_topk): packed keys go to LDS, each lane counts the keys
  // above its own (all comparisons independent, no cross-lane chains), and the expert of
  // rank k < K lands in slot k. Equal float keys are ordered by the packed inverted
  // index, so the lower index ranks first.
  const int lane = tid & 63;
  const int w = tid >> 6;
  const bool biased = sel_bias != nullptr;
  __shared__ uint64_t s_key[WAVES][kMaxN];
  __shared__ int s_sel[WAVES][kMaxK];
  float bias_r[kMaxN / kWave];
#pragma unroll
  for (int j = 0; j < kMaxN / kWave; ++j) {
    const int e = lane + j * kWave;
    bias_r[j] = (biased && e < N) ? sel_bias[e] : 0.f;
  }
  for (int t = w; t < BT; t += WAVES) {
    const int tok = t0 + t;
    if (tok >= T) break;
    const float* zr = z + t * ldz;
    uint64_t mine[kMaxN / kWave];
#pragma unroll
    for (int j = 0; j < kMaxN / kWave; ++j) {
      const int e = lane + j * kWave;
      mine[j] = 0ull;
      if (e < N) {
        float key = zr[e];
        if (biased) key = (score == 1 ? sigmoid_f(key) : key) + bias_r[j];
        mine[j] = (static_cast<uint64_t>(ord_key(key)) << 32) |
                  static_cast<uint64_t>(~static_cast<uint32_t>(e));
      }
    }
    select_topk(mine, N, K, lane, s_key[w], s_sel[w]);
    wave_lds_sync();
    const int sele = lane < K ? s_sel[w][lane] : 0;
    const float selz = lane < K ? zr[sele] : 0.f;
    const bool act = lane < K;
    float r;
    if (score == 1) {  // sigmoid affinities
      const float a = act ? sigmoid_f(selz) : 0.f;
      r = renorm ? alpha * a / wave_sum(a) : alpha * a;
    } else {
      // max over all N logits: the top-1 key unless a bias reordered the selection
      float m;
      if (biased) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMaxN / kWave; ++j) {
          const int ee = lane + j * kWave;
          if (ee < N) mx = fmaxf(mx, zr[ee]);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
        m = mx;
      } else {
        m = __shfl(selz, 0, kWave);
      }
      const float e = act ? expf(selz - m) : 0.f;
      if (score == 0 && !renorm) {
        float zsum = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxN / kWave; ++j) {
          const int ee = lane + j * kWave;
          if (ee < N) zsum += expf(zr[ee] - m);
        }
        r = alpha * e / wave_sum(zsum);
      } else {
        r = alpha * e / wave_sum(e);
      }
    }
    if (act) {
      topk_idx[static_cast<size_t>(tok) * K + lane] = sele;
      topk_r[static_cast<size_t>(tok) * K + lane] = r;
      if (hist != nullptr) s_tsel[t][lane] = sele;
    }
    if (has_gate && s_tok != nullptr && lane == 0) s_tok[tok] = sigmoid_f(zr[N]);
  }
  // ---- epilogue: this tile's histogram row and each route's rank within the row ------
  // (the K experts of a token are distinct, so each token sets one bit per expert; OR is
  // order-free and the rank is the popcount of the mask below the token)
  if (hist != nullptr) {
    const int nt = min(BT, T - t0);
    __syncthreads();
    for (int i = tid; i < nt * K; i += THREADS) atomicOr(&s_mask[s_tsel[i / K][i % K]], 1u << (i / K));
    __syncthreads();
    for (int i = tid; i < nt * K; i += THREADS) {
      const int t = i / K;
      loc_rank[static_cast<size_t>(t0) * K + i] = __popc(s_mask[s_tsel[t][i % K]] & ((1u << t) - 1u));
    }
    for (int e = tid; e < N; e += THREADS)
      hist[static_cast<size_t>(blockIdx.x) * N + e] = __popc(s_mask[e]);
  }
}

template <int BT, int NBT, int WAVES, int U, bool TILE_ONLY = false, bool LDSP = false>
hipError_t launch_cfg(int T, int d, int N, int K, int score, int renorm, float alpha, int dt,
                      const void* x, const void* w_router, const float* logit_bias,
                      const float* sel_bias, const void* w_gate_vec, float* logits, int logits_mode, int32_t* topk_idx,
                      float* topk_r, float* s_tok, const float* part, int nparts,
                      int32_t* hist, int32_t* loc_rank, hipStream_t stream) {
  const int grid = (T + BT - 1) / BT;
  hipLaunchKernelGGL((route_kernel<BT, NBT, WAVES, U, TILE_ONLY, LDSP>), dim3(grid), dim3(WAVES * 64), 0, stream,
                     T, d, N, K, score, renorm, alpha, dt, x, w_router, logit_bias, sel_bias,
                     w_gate_vec,
                     logits, logits_mode, topk_idx, topk_r, s_tok, part, nparts, hist, loc_rank);
  return hipGetLastError();
}

}  // namespace

// d_model slices of the split-K logits for this router, or 0 when the fused single-pass
// router runs (few experts, fp32, a shared-gate column, or logits given as input)
int route_split_slices(int N, int d_model, int dt, int logits_mode, bool has_gate) {
  if (logits_mode != 0 || dt != 1 || has_gate || N <= 128 || N > 256 || N % 64 != 0) return 0;
  // up to 4 slices: 256 workgroups of 128 tokens at 8192 tokens
  for (int P = kRouteMaxSlices; P >= 1; P >>= 1)
    if (d_model % (P * LS_RS * LS_BK) == 0) return P;
  return 0;
}

// scratch of the split-K path: the partial logit slices, then W_r packed (256-byte aligned)
size_t route_scratch_bytes(int T, int d_model, int N) {
  if (N <= 128) return 0;
  const size_t part = (static_cast<size_t>(kRouteMaxSlices) * T * N * sizeof(float) + 255) / 256 * 256;
  return part + static_cast<size_t>(N) * d_model * 2;
}

namespace {

}  // namespace

// tokens per router workgroup, i.e. per histogram row of the router's own count
int route_tile_tokens(int N, int d_model, int dt, int logits_mode, bool has_gate) {
  if (route_split_slices(N, d_model, dt, logits_mode, has_gate) > 0) return 32;
  const int ncol = N + ((has_gate && logits_mode == 0) ? 1 : 0);
  return (ncol + 15) / 16 <= 8 ? 16 : 32;
}

hipError_t launch_route(int T, int d_model, int N, int K, int score, int renorm, float alpha,
                        int dt, const void* x, const void* w_router, const float* logit_bias,
                        const float* expert_bias, const void* w_shared_gate, float* logits, int logits_mode,
                        int32_t* topk_idx, float* topk_r, float* s_tok, void* scratch,
                        int32_t* hist, int32_t* loc_rank, hipStream_t stream) {
  const int ncol = N + ((w_shared_gate != nullptr && logits_mode == 0) ? 1 : 0);
  const int NB = (ncol + 15) / 16;
  const int P = route_split_slices(N, d_model, dt, logits_mode, w_shared_gate != nullptr);
  if (P > 0) {  // pack W_r, split-K logits into slices, top-K over their fixed-order sum
    if (scratch == nullptr) return hipErrorInvalidValue;
    float* partials = static_cast<float*>(scratch);
    char* wpk = static_cast<char*>(scratch) +
                (static_cast<size_t>(kRouteMaxSlices) * T * N * sizeof(float) + 255) / 256 * 256;
    hipError_t e = launch_pack_weights(1, N, d_model, w_router, wpk, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(logits_split_kernel, dim3((T + LS_BT - 1) / LS_BT, P), dim3(256), 0,
                       stream, T, d_model, N, d_model / P, static_cast<const uint16_t*>(x),
                       reinterpret_cast<const uint16_t*>(wpk), partials);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_cfg<32, 17, 16, 1, true>(T, d_model, N, K, score, renorm, alpha, dt, nullptr,
                                          nullptr, logit_bias, expert_bias, nullptr, logits, 2,
                                          topk_idx, topk_r, nullptr, partials, P, hist, loc_rank,
                                          stream);
  }
  // bf16, 33 to 128 logit columns: the LDS-staged logits (with fewer columns the x rows
  // dominate and the register-direct loads below stream them as fast)
  if (dt == 1 && logits_mode == 0 && NB >= 3 && NB <= 8 && d_model % LP_BK == 0) {
#define MOE_ROUTE_LDS(NBT_)                                                                  \
  if (NB <= NBT_)                                                                            \
    return launch_cfg<16, NBT_, 16, 1, false, true>(T, d_model, N, K, score, renorm, alpha,  \
                                                   dt, x, w_router, logit_bias, expert_bias, \
                                                   w_shared_gate, logits, logits_mode,       \
                                                   topk_idx, topk_r, s_tok, nullptr, 0, hist, \
                                                   loc_rank, stream);
    MOE_ROUTE_LDS(4)
    MOE_ROUTE_LDS(8)
#undef MOE_ROUTE_LDS
  }
  // (tokens per workgroup, column blocks, waves, k steps in flight per wave): small N
  // uses 16 tokens and 8 waves; large N 32 tokens (router rows re-read half as often)
#define MOE_ROUTE_CASE(BT_, NBT_, W_, U_)                                                    \
  if (NB <= NBT_)                                                                            \
    return launch_cfg<BT_, NBT_, W_, U_>(T, d_model, N, K, score, renorm, alpha, dt, x,      \
                                         w_router, logit_bias, expert_bias, w_shared_gate,   \
                                         logits, logits_mode, topk_idx, topk_r, s_tok,       \
                                         nullptr, 0, hist, loc_rank, stream);
  MOE_ROUTE_CASE(16, 1, 8, 8)
  MOE_ROUTE_CASE(16, 2, 8, 8)
  MOE_ROUTE_CASE(16, 4, 8, 4)
  MOE_ROUTE_CASE(16, 8, 8, 2)
  MOE_ROUTE_CASE(32, 17, 4, 2)
#undef MOE_ROUTE_CASE
  return hipErrorInvalidValue;
}
