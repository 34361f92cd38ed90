// Persistent grouped GEMM with fused SwiGLU over packed weights; the weight stream is
// prefetched several stages ahead and continues across tile boundaries.
//
// Operation and weight layout are those of gemm_packed.hip (expert i owns packed rows
// [o_i, o_{i+1}), "Section 10: Routing, Capacity, and Load Balancing", Eq. 26; the SwiGLU
// expert of "Section 20: One Shared Expert Is All You Need", Eq. 74; weights in the
// v_mfma_f32_32x32x16_bf16 A-operand order written by moe_pack_weights). One launch
// serves up to two problems: a grouped one (the routed experts over their real-count
// segments, activation rows optionally gathered through a row index) and a dense one
// (the shared MLP over all tokens), so the shared expert fills the routed pass's tail.
//
// Schedule (one workgroup of 4 waves per compute unit):
//   * tiles are ordered (problem, group, n-tile, m-tile); 8 contiguous parts of that list
//     of equal cost go to the 8 XCDs (workgroup b runs on XCD b % 8) and the workgroups
//     of an XCD take every (grid / 8)-th tile of its part, so the row tiles that share a
//     weight block run at the same time behind the same L2. A tile's cost is its bytes
//     through the compute unit's vector L1 per k stage, in units of one 32-row activation
//     block: 2 per wave for the weight blocks (fetched whatever the tile's rows) plus one
//     per active 32-row block, times the k stages;
//   * every wave streams its NBW weight blocks straight into registers, RS stages
//     (64 k each) ahead, in a register ring; activations go through a 4-stage LDS ring
//     filled by direct-to-LDS loads; in the last stages of a tile both rings are already
//     refilled with the next tile's first stages, so the pipeline never drains;
//   * these loads are not visible to the compiler (inline asm): every stage issues the
//     same number of them, and one explicit s_waitcnt vmcnt per stage, before the stage
//     barrier, covers the weights and activations that stage consumes. Other memory
//     operations (epilogue stores, row-index loads) only add to the count, which can
//     only make that wait stricter.
// Wave w of a tile owns weight blocks (32 rows each) w * NBW .. w * NBW + NBW - 1 of the
// tile's 128 NBW weight rows (SwiGLU: NBW / 2 gate blocks and the matching up blocks)
// and all BM = 32 XBM activation rows.
#include <atomic>
#include <utility>

#include "gemm_common.h"
#include "gemm_stream.h"

using namespace moe;

namespace {

constexpr int SK_GT = 256;           // threads that build the group tables (<= 256 groups)
constexpr int SK_BKX = 64;           // k per stage
constexpr int SK_XS = 4;             // activation ring depth (stages)
constexpr int SK_SPS = SK_BKX / 16;  // k16 steps per stage

// physical 16-byte chunk of logical chunk c (0..7) of activation row r in a stage:
// conflict-free MFMA operand reads
__device__ __forceinline__ int sk_swz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

// direct-to-LDS loads (uniform base + 32-bit per-lane byte offset; lane j lands at
// lds_addr + j * size)
__device__ __forceinline__ void sk_dma16(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void sk_dma4(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
// 16-byte load into registers that the compiler does not track: the register is read
// only after the stage wait that covers it
__device__ __forceinline__ void sk_ldg16(u32x4& dst, const void* sbase, uint32_t voff) {
  asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(dst) : "v"(voff), "s"(sbase) : "memory");
}

template <typename F, int... I>
__device__ __forceinline__ void sk_unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in order
template <int N, typename F>
__device__ __forceinline__ void sk_unroll(F&& f) {
  sk_unroll_impl(f, std::make_integer_sequence<int, N>{});
}

// RH row halves: wave v takes weight position v % 4 and tile rows (v / 4) * 32 XBM ..
// + 32 XBM - 1; the waves of one position load the same weight blocks
template <int NBW, int XBM, int RS, int RH>
struct SK {
  static constexpr int WAVES = 4 * RH;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int HROWS = 32 * XBM;            // rows per row half
  static constexpr int BM = HROWS * RH;             // rows per tile
  static constexpr int COLS_SWIGLU = 64 * NBW;   // output columns of a SwiGLU tile
  static constexpr int COLS_PLAIN = 128 * NBW;
  static constexpr int XSTAGE = BM * SK_BKX * 2;  // bytes
  static constexpr int XDPW = XSTAGE / (1024 * WAVES);  // direct-to-LDS loads per wave per stage
  static constexpr int WPS = SK_SPS * NBW;        // weight loads per wave per stage
  static constexpr int PER = XDPW + WPS;          // vector memory ops per wave per stage
  // ops issued after the weights (resp. activations) of stage s when stage s begins
  static constexpr int AFTER_W = (RS - 1) * PER;
  static constexpr int AFTER_X = WPS + (SK_XS - 2) * PER;
  static constexpr int WAITN = AFTER_W < AFTER_X ? AFTER_W : AFTER_X;
  static_assert(WAITN <= 63, "vmcnt range");
  static_assert(XDPW * 1024 * WAVES == XSTAGE, "whole direct-to-LDS loads per stage");
  static_assert(BM <= 256, "row index buffer");
};

// one tile, all fields uniform
struct SkTile {
  int p;     // problem
  int g;     // group within the problem
  int row0;  // first packed row
  int rows;  // packed rows (1..BM)
  int n0;    // first output column
  int nst;   // k stages
};

// MODE: SK_PLAIN, SK_SWIGLU, or SK_SWIGLU_BWD (gate and up products as in SK_SWIGLU; the
// epilogue takes dH and writes H = SiLU(A) B and [dA | dB] instead of SiLU(A) B alone)
constexpr int SK_PLAIN = 0, SK_SWIGLU = 1, SK_SWIGLU_BWD = 2;

template <int NBW, int XBM, int RS, int RH, int MODE>
__global__ void __launch_bounds__(64 * 4 * RH, 1)
gemm_stream_kernel(StreamProblem p0, StreamProblem p1) {
  using C = SK<NBW, XBM, RS, RH>;
  constexpr bool SWIGLU = MODE != SK_PLAIN;
  constexpr int COLS = SWIGLU ? C::COLS_SWIGLU : C::COLS_PLAIN;
  __shared__ int s_off[kMaxN + 2];     // packed row offsets of the groups (p1 last)
  __shared__ int s_tstart[SK_GT + 1];
  __shared__ int s_cstart[SK_GT + 1];
  __shared__ int s_rows[2][256];       // gathered activation rows of the current / next tile
  __shared__ __attribute__((aligned(1024))) char lds[SK_XS * C::XSTAGE];
  // SwiGLU backward: the tile's dH rows ([BM][COLS] bf16, 16-byte chunks of row r permuted
  // by r & 15), brought in by direct-to-LDS loads during the tile's last stage
  constexpr int DH_ROWB = COLS * 2;
  __shared__ __attribute__((aligned(1024))) char dhbuf[MODE == SK_SWIGLU_BWD ? C::BM * DH_ROWB : 16];
  typedef __attribute__((address_space(3))) char lds_char;
  const int tid = threadIdx.x;
  const int G0 = p0.G;
  const int NG = G0 + (p1.rows > 0 ? 1 : 0);  // groups over both problems (<= 256)

  // ---- tile list: per-group tile counts and costs, prefix-summed in LDS ----
  // cost of a tile = (KW + active 32-row blocks) x k stages; a group's tiles cost
  // n-tiles x (KW x m-tiles + ceil(rows / 32)) x stages in all
  constexpr int KW = 2 * C::WAVES;  // weight bytes per stage, in 32-row activation blocks
  for (int g = tid; g <= G0; g += C::THREADS)
    s_off[g] = (p0.offsets != nullptr) ? p0.offsets[g] : (g == 0 ? 0 : p0.rows);
  __syncthreads();
  if (tid == 0) s_off[G0 + 1] = s_off[G0] + p1.rows;
  __syncthreads();
  if (tid < SK_GT) {
    int cnt = 0, cost = 0;
    if (tid < NG) {
      const StreamProblem& P = tid < G0 ? p0 : p1;
      const int nrows = s_off[tid + 1] - s_off[tid];
      cnt = ceil_div(nrows, C::BM) * (P.Nd / COLS);
      cost = (P.Nd / COLS) * (KW * ceil_div(nrows, C::BM) + ceil_div(nrows, 32)) * (P.Kd / SK_BKX);
    }
    s_tstart[tid + 1] = cnt;
    s_cstart[tid + 1] = cost;
  }
  if (tid == 0) {
    s_tstart[0] = 0;
    s_cstart[0] = 0;
  }
  __syncthreads();
  for (int off = 1; off < SK_GT; off <<= 1) {  // inclusive scans over <= 256 groups
    const bool gt = tid < SK_GT;
    const int v = (gt && tid >= off) ? s_tstart[tid + 1 - off] : 0;
    const int c = (gt && tid >= off) ? s_cstart[tid + 1 - off] : 0;
    __syncthreads();
    if (gt) {
      s_tstart[tid + 1] += v;
      s_cstart[tid + 1] += c;
    }
    __syncthreads();
  }
  const int total = s_tstart[NG];
  // this XCD's contiguous share of the tile list: from the first tile whose cost prefix
  // reaches xcd / 8 of the total cost to the first that reaches (xcd + 1) / 8
  auto first_tile_at_cost = [&](long target) -> int {
    if (target <= 0) return 0;
    if (target >= s_cstart[NG]) return total;
    int lo = 0, hi = NG - 1;  // group with s_cstart[g] < target <= s_cstart[g + 1]
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_cstart[mid + 1] < target) lo = mid + 1; else hi = mid;
    }
    const StreamProblem& P = lo < G0 ? p0 : p1;
    const int nrows = s_off[lo + 1] - s_off[lo];
    const int mtiles = ceil_div(nrows, C::BM);
    const int cn = KW * mtiles + ceil_div(nrows, 32);  // per n-tile, per stage
    const int nst = P.Kd / SK_BKX;
    const long u = (target - s_cstart[lo] + nst - 1) / nst;  // cost per stage into the group
    int nt = static_cast<int>(u / cn);
    const int rem = static_cast<int>(u - static_cast<long>(nt) * cn);
    // every m-tile but the last costs KW + BM / 32: the first m-tile whose prefix reaches rem
    int mt = ceil_div(rem, KW + C::BM / 32);
    if (mt >= mtiles) {
      ++nt;
      mt = 0;
    }
    return min(total, s_tstart[lo] + nt * mtiles + mt);
  };
  const int step = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const long ctot = s_cstart[NG];
  const int t_beg = __builtin_amdgcn_readfirstlane(first_tile_at_cost(ctot * xcd / 8));
  const int t_end = __builtin_amdgcn_readfirstlane(first_tile_at_cost(ctot * (xcd + 1) / 8));
  int t = t_beg + (blockIdx.x >> 3);
  if (t >= t_end) return;

  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave
  const int w = wv & 3;                                    // weight position
  const int rh = wv >> 2;                                  // row half
  const uint32_t lds_base = static_cast<uint32_t>((size_t)((lds_char*)lds));
  const uint32_t rows_base = static_cast<uint32_t>((size_t)((lds_char*)(&s_rows[0][0])));
  const uint32_t dh_base = static_cast<uint32_t>((size_t)((lds_char*)dhbuf));

  auto tile_at = [&](int ti) -> SkTile {
    int lo = 0, hi = NG - 1;  // largest g with s_tstart[g] <= ti (a non-empty group)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tstart[mid] <= ti) lo = mid; else hi = mid - 1;
    }
    const bool second = lo >= G0;
    const int base = second ? 0 : s_off[lo];
    const int nrows = s_off[lo + 1] - s_off[lo];
    const int local = ti - s_tstart[lo];
    const int mtiles = ceil_div(nrows, C::BM);
    const int nt = local / mtiles;
    const int mt = local - nt * mtiles;
    SkTile k;
    k.p = __builtin_amdgcn_readfirstlane(second ? 1 : 0);
    k.g = __builtin_amdgcn_readfirstlane(second ? 0 : lo);
    k.row0 = __builtin_amdgcn_readfirstlane(base + mt * C::BM);
    k.rows = __builtin_amdgcn_readfirstlane(min(C::BM, nrows - mt * C::BM));
    k.n0 = __builtin_amdgcn_readfirstlane(nt * COLS);
    k.nst = __builtin_amdgcn_readfirstlane((second ? p1.Kd : p0.Kd) / SK_BKX);
    return k;
  };
  auto prob = [&](const SkTile& k) -> const StreamProblem& { return k.p ? p1 : p0; };
  // uniform base of weight block b of this wave for tile k
  auto wbase = [&](const SkTile& k, int b) -> const char* {
    const StreamProblem& P = prob(k);
    const size_t gstride = static_cast<size_t>(P.Nd) * P.Kd;
    const uint16_t* base;
    int nb;
    if (SWIGLU) {
      base = (b < NBW / 2 ? P.w0 : P.w1) + k.g * gstride;
      nb = k.n0 / 32 + w * (NBW / 2) + (b % (NBW / 2));
    } else {
      base = P.w0 + k.g * gstride;
      nb = k.n0 / 32 + w * NBW + b;
    }
    return reinterpret_cast<const char*>(base + static_cast<size_t>(nb) * 32 * P.Kd);
  };
  // packed row (within the tile) behind this lane's DMA slot i
  auto slot_row = [&](int i) -> int { return ((C::WAVES * i + wv) * 64 + lane) >> 3; };
  // direct-to-LDS copy of tile k's gathered activation rows into row buffer `slot`
  // (rows past the tile repeat its last row)
  auto fetch_rows = [&](const SkTile& k, int slot) {
    const StreamProblem& P = prob(k);
    if (P.row_index != nullptr && wv * 64 < C::BM) {
      const int r = k.row0 + min(wv * 64 + lane, k.rows - 1);
      sk_dma4(static_cast<uint32_t>(r) * 4u, P.row_index, rows_base + slot * 1024 + wv * 256);
    }
  };
  // activation row of each of this lane's DMA slots for tile k
  auto rows_of = [&](const SkTile& k, int slot, uint32_t* xr) {
    const bool gathered = prob(k).row_index != nullptr;
#pragma unroll
    for (int i = 0; i < C::XDPW; ++i) {
      const int r = min(slot_row(i), k.rows - 1);
      xr[i] = static_cast<uint32_t>(gathered ? s_rows[slot][r] : k.row0 + r);
    }
  };
  auto issue_x = [&](const SkTile& k, const uint32_t* xr, int ks, int ring_slot) {
    const StreamProblem& P = prob(k);
    const uint32_t kbytes = static_cast<uint32_t>(P.Kd) * 2u;
    const uint32_t dst = lds_base + ring_slot * C::XSTAGE + wv * 1024;
#pragma unroll
    for (int i = 0; i < C::XDPW; ++i) {
      const int s = (C::WAVES * i + wv) * 64 + lane;
      const uint32_t off = xr[i] * kbytes +
                           static_cast<uint32_t>(sk_swz(s >> 3, s & 7) * 16 + ks * (SK_BKX * 2));
      sk_dma16(off, P.a, dst + i * (1024 * C::WAVES));
    }
  };

  // dH of tile k into dhbuf: wave w brings tile rows 32 w .. 32 w + 31 (rows past the tile
  // repeat its last row), lane j of load i row 32 w + 4 i + (j >> 4), chunk j & 15
  auto issue_dh = [&](const SkTile& k) {
    static_assert(MODE != SK_SWIGLU_BWD || (C::BM == 128 && DH_ROWB == 256),
                  "dH staging assumes 128 rows of 256 bytes");
    const StreamProblem& P = prob(k);
    const uint32_t rowb = static_cast<uint32_t>(P.Nd) * 2u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 32 * w + 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ (rr & 15);
      const uint32_t off = static_cast<uint32_t>(k.row0 + min(rr, k.rows - 1)) * rowb +
                           static_cast<uint32_t>(k.n0 + 8 * c) * 2u;
      sk_dma16(off, P.dh, dh_base + (32 * w + 4 * i) * DH_ROWB);
    }
  };

  SkTile cur = tile_at(t);
  bool has_n = t + step < t_end;
  SkTile nxt = has_n ? tile_at(t + step) : cur;
  const char* wc[NBW];
  const char* wn[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    wc[b] = wbase(cur, b);
    wn[b] = wbase(nxt, b);
  }
  int kslot = 0;  // row buffer of the current tile
  fetch_rows(cur, 0);
  wait_vmcnt<0>();
  __syncthreads();
  uint32_t xc[C::XDPW];
  rows_of(cur, 0, xc);

  // prologue: the loads of virtual stages -V..-1, in the order a steady stage issues them
  u32x4 wr[RS][SK_SPS][NBW];
  constexpr int V = (SK_XS - 1) > RS ? (SK_XS - 1) : RS;
  sk_unroll<V>([&](auto vc) {
    constexpr int v = decltype(vc)::value - V;
    constexpr int xs_t = v + SK_XS - 1;
    if constexpr (xs_t >= 0) issue_x(cur, xc, xs_t, xs_t);
    constexpr int ws_t = v + RS;
    if constexpr (ws_t >= 0) {
#pragma unroll
      for (int u = 0; u < SK_SPS; ++u)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
          sk_ldg16(wr[ws_t][u][b], wc[b],
                   static_cast<uint32_t>(((ws_t * SK_SPS + u) * 64 + lane) * 16));
    }
  });

  int gs = 0;  // stages completed by this workgroup (activation ring position)
  for (;;) {
    fetch_rows(nxt, kslot ^ 1);  // published by the stage barriers before its first use
    const bool has_nn = t + 2 * step < t_end;
    const SkTile nn = has_nn ? tile_at(t + 2 * step) : nxt;
    // 32-row blocks of this wave's row half that hold rows of the tile
    const int xb = __builtin_amdgcn_readfirstlane(
        min(XBM, max(0, ceil_div(cur.rows - rh * C::HROWS, 32))));
    const int nst = cur.nst;

    floatx16 acc[NBW][XBM];
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
      for (int j = 0; j < XBM; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][j][v] = 0.f;

    for (int s0 = 0; s0 < nst; s0 += RS) {
      sk_unroll<RS>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int s = s0 + r;
        // this stage's weights and activations have landed in this wave's registers and
        // LDS part; the barrier publishes the activations and retires every read of the
        // slot that stage s + XS - 1 overwrites
        wait_vmcnt<C::WAITN>();
        __syncthreads();
        // (the previous tile's epilogue read of dhbuf is behind this barrier)
        if constexpr (MODE == SK_SWIGLU_BWD) {
          if (s == nst - 1) issue_dh(cur);
        }
        {
          const int ts = s + SK_XS - 1;
          uint32_t xr[C::XDPW];
          if (ts < nst) {
#pragma unroll
            for (int i = 0; i < C::XDPW; ++i) xr[i] = xc[i];
            issue_x(cur, xr, ts, (gs + SK_XS - 1) % SK_XS);
          } else {
            rows_of(nxt, kslot ^ 1, xr);
            issue_x(nxt, xr, ts - nst, (gs + SK_XS - 1) % SK_XS);
          }
        }
        const char* xs = lds + (gs % SK_XS) * C::XSTAGE;
        const int tw = s + RS;  // weight refill target stage (the next tile's past the end)
        const bool w_in_cur = tw < nst;
        const int kw = (w_in_cur ? tw : tw - nst) * SK_SPS;
        auto xread = [&](int u, bf16x8* xv) {
          const int kc = 2 * u + lh;
#pragma unroll
          for (int j = 0; j < XBM; ++j) {
            const int row = rh * C::HROWS + 32 * j + lr;
            xv[j] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(xs + row * (SK_BKX * 2) + (sk_swz(row, kc) << 4)));
          }
        };
        // double-buffered activation fragments with one row half; with two (half the
        // registers per wave) one set at a time
        constexpr int XV = RH == 1 ? 2 : 1;
        bf16x8 xv[XV][XBM];
        if (XV == 2) xread(0, xv[0]);
#pragma unroll
        for (int u = 0; u < SK_SPS; ++u) {
          const int cb = XV == 2 ? (u & 1) : 0;
          if (XV == 2 && u + 1 < SK_SPS) xread(u + 1, xv[cb ^ 1]);
          if (XV == 1) xread(u, xv[0]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < XBM; ++j) {
            if (j >= xb) break;  // uniform: rows past the tile are never computed
#pragma unroll
            for (int b = 0; b < NBW; ++b)
              acc[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, wr[r][u][b]), xv[cb][j], acc[b][j], 0, 0, 0);
          }
#pragma unroll
          for (int b = 0; b < NBW; ++b)
            sk_ldg16(wr[r][u][b], w_in_cur ? wc[b] : wn[b],
                     static_cast<uint32_t>(((kw + u) * 64 + lane) * 16));
          __builtin_amdgcn_sched_barrier(0);
        }
        ++gs;
      });
    }

    // epilogue: lane (lr, lh) holds row 32 j + lr, columns 8 q + 4 lh + {0..3} of each
    // 32-wide block; one exchange between lane halves gives each lane two 16-byte pieces
    // per row and block (columns 8 lh..+7 and 16 + 8 lh..+7)
    if constexpr (MODE == SK_SWIGLU_BWD) {
      // the last stage issued exactly PER loads after the dH loads
      wait_vmcnt<C::PER>();
      __syncthreads();
    }
    {
      const StreamProblem& P = prob(cur);
      constexpr int OB = SWIGLU ? NBW / 2 : NBW;  // output blocks per wave
      // packed bf16 pieces pk[q] (columns 8 q + 4 lh + {0..3}) -> row dst, columns n..n+31
      auto put = [&](const u32x2* pk, uint16_t* dst, bool ok) {
        // lh = 0 keeps q = 0, 2 and receives the partner's; lh = 1 keeps q = 1, 3
        const u32x2 s0v = lh ? pk[0] : pk[1], s1v = lh ? pk[2] : pk[3];
        u32x2 r0, r1;
        r0[0] = __shfl_xor(s0v[0], 32, kWave);
        r0[1] = __shfl_xor(s0v[1], 32, kWave);
        r1[0] = __shfl_xor(s1v[0], 32, kWave);
        r1[1] = __shfl_xor(s1v[1], 32, kWave);
        const u32x4 ca = lh ? u32x4{r0[0], r0[1], pk[1][0], pk[1][1]}
                            : u32x4{pk[0][0], pk[0][1], r0[0], r0[1]};
        const u32x4 cb = lh ? u32x4{r1[0], r1[1], pk[3][0], pk[3][1]}
                            : u32x4{pk[2][0], pk[2][1], r1[0], r1[1]};
        if (ok) {
          *reinterpret_cast<u32x4*>(dst + 8 * lh) = ca;
          *reinterpret_cast<u32x4*>(dst + 16 + 8 * lh) = cb;
        }
      };
#pragma unroll
      for (int j = 0; j < XBM; ++j) {
        if (j >= xb) break;
        const int m = rh * C::HROWS + 32 * j + lr;
        const bool ok = m < cur.rows;
        const size_t prow = static_cast<size_t>(cur.row0 + (ok ? m : 0));
        uint16_t* orow = P.out + prow * P.Nd;
#pragma unroll
        for (int ob = 0; ob < OB; ++ob) {
          const int n = cur.n0 + 32 * (SWIGLU ? w * (NBW / 2) + ob : w * NBW + ob);
          if constexpr (MODE == SK_SWIGLU_BWD) {
            // dH of this lane's 16 elements (from dhbuf); A, B are the fp32 sums
            u32x2 gh[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = (n - cur.n0) / 8 + q;  // logical 16-byte chunk of the tile row
              gh[q] = *reinterpret_cast<const u32x2*>(dhbuf + m * DH_ROWB +
                                                      ((c ^ (m & 15)) << 4) + 8 * lh);
            }
            uint16_t* abrow = P.dab + prow * 2 * P.Nd + n;
            // H = SiLU(A) B (as the forward's SwiGLU epilogue), dA = dH B sg (1 + A (1 - sg)),
            // dB = dH A sg, with sg = sigmoid(A)
            u32x2 ph[4], pa[4], pb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float oh[4], oa[4], ob2[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float a = acc[ob][j][4 * q + e];
                const float b = acc[ob + NBW / 2][j][4 * q + e];
                const uint32_t gw = gh[q][e >> 1];
                const float g = __uint_as_float((e & 1) ? (gw & 0xFFFF0000u) : (gw << 16));
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
                const float sa = a * sg;
                oh[e] = sa * b;
                oa[e] = g * b * sg * (1.0f + a * (1.0f - sg));
                ob2[e] = g * sa;
              }
              ph[q] = u32x2{pack_bf16x2(oh[0], oh[1]), pack_bf16x2(oh[2], oh[3])};
              pa[q] = u32x2{pack_bf16x2(oa[0], oa[1]), pack_bf16x2(oa[2], oa[3])};
              pb[q] = u32x2{pack_bf16x2(ob2[0], ob2[1]), pack_bf16x2(ob2[2], ob2[3])};
            }
            put(ph, orow + n, ok);
            put(pa, abrow, ok);
            put(pb, abrow + P.Nd, ok);
          } else {
            // two halves of the block (columns 0..15, 16..31), one exchange each, so that
            // only half a block's packed values are live at a time
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              u32x2 pk[2];
#pragma unroll
              for (int qq = 0; qq < 2; ++qq) {
                const int q = 2 * hf + qq;
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  h[e] = SWIGLU ? silu_f(acc[ob][j][4 * q + e]) * acc[ob + NBW / 2][j][4 * q + e]
                                : acc[ob][j][4 * q + e];
                pk[qq] = u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
              }
              // lh = 0 keeps q = 2 hf and receives the partner's; lh = 1 keeps q = 2 hf + 1
              const u32x2 sv = lh ? pk[0] : pk[1];
              u32x2 rv;
              rv[0] = __shfl_xor(sv[0], 32, kWave);
              rv[1] = __shfl_xor(sv[1], 32, kWave);
              const u32x4 c = lh ? u32x4{rv[0], rv[1], pk[1][0], pk[1][1]}
                                 : u32x4{pk[0][0], pk[0][1], rv[0], rv[1]};
              if (ok) *reinterpret_cast<u32x4*>(orow + n + 16 * hf + 8 * lh) = c;
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);  // one block's values live at a time
        }
      }
    }

    if (!has_n) break;
    cur = nxt;
    nxt = nn;
    has_n = has_nn;
    t += step;
    kslot ^= 1;
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      wc[b] = wn[b];
      wn[b] = wbase(nxt, b);
    }
    rows_of(cur, kslot, xc);
  }
  wait_vmcnt<0>();  // no direct-to-LDS load may land after the workgroup ends
}

// tile shapes: 2 weight blocks per wave, 128 rows per row half. One row half (4 waves)
// with 4 stages of weights in flight; for few experts with many rows each (at least
// kRowsRH2 per group), two row halves (8 waves, 2 waves per SIMD, so 2 stages of weights
// in flight) that share every weight block fetched into the CU.
constexpr int kNBW = 2, kXBM = 4, kRS = 4, kRS2 = 2, kRowsRH2 = 1024;

bool fits(int mode, const StreamProblem& P) {
  const bool swiglu = mode != SK_PLAIN;
  if (P.rows <= 0) return true;
  if (mode == SK_SWIGLU_BWD && (P.dh == nullptr || P.dab == nullptr)) return false;
  using C = SK<kNBW, kXBM, kRS, 1>;  // both row-half shapes share COLS and the stage rule
  const int cols = swiglu ? C::COLS_SWIGLU : C::COLS_PLAIN;
  const int nst = P.Kd / SK_BKX;
  if (P.G <= 0 || P.G > kMaxN || P.a == nullptr || P.w0 == nullptr || P.out == nullptr)
    return false;
  if (swiglu && P.w1 == nullptr) return false;
  if (P.Nd % cols != 0 || P.Kd % SK_BKX != 0 || nst % kRS != 0 || nst < kRS + SK_XS) return false;
  // 32-bit byte offsets into the activations and the row index
  const long a_rows = P.row_index != nullptr ? P.a_rows : P.rows;
  if (a_rows <= 0 || a_rows * P.Kd * 2L >= (1L << 32)) return false;
  if (P.rows * 4L >= (1L << 32)) return false;
  if (mode == SK_SWIGLU_BWD && P.rows * P.Nd * 2L >= (1L << 32)) return false;  // dH offsets
  return true;
}

}  // namespace

// upper bound of the kernel's summed tile cost (32-bit prefix sums in LDS) for any split
// of a problem's rows into its G groups: every group adds at most one m-tile and one
// 32-row block to the unsplit count
static long cost_bound(int mode, const StreamProblem& P) {
  if (P.rows <= 0) return 0;
  using C = SK<kNBW, kXBM, kRS, 1>;
  const long cols = mode != SK_PLAIN ? C::COLS_SWIGLU : C::COLS_PLAIN;
  const long kw = 2 * 8, bm = 128;  // the larger weight cost (two row halves), the smaller tile
  const long mt = (P.rows + bm - 1) / bm + P.G, rb = (P.rows + 31) / 32 + P.G;
  return (P.Nd / cols) * (kw * mt + rb) * (P.Kd / SK_BKX);
}

static bool supported(int mode, const StreamProblem& p0, const StreamProblem& p1) {
  if (p0.rows <= 0 || !fits(mode, p0) || !fits(mode, p1)) return false;
  if (p1.rows > 0 && (p1.offsets != nullptr || p1.G != 1 || p0.G + 1 > SK_GT)) return false;
  if (cost_bound(mode, p0) + cost_bound(mode, p1) >= (1L << 31)) return false;
  return true;
}

static hipError_t launch(int mode, const StreamProblem& p0, const StreamProblem& p1,
                         hipStream_t stream) {
  if (!supported(mode, p0, p1)) return hipErrorNotSupported;
  // compute units per device, looked up once (host threads may race to store the same value)
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n_cu = cus[dev].load(std::memory_order_relaxed);
  if (n_cu == 0) {
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    cus[dev].store(n_cu, std::memory_order_relaxed);
  }
  const int grid = n_cu / 8 * 8;
  if (grid <= 0) return hipErrorNotSupported;
  const bool rh2 = mode != SK_SWIGLU_BWD && p0.rows >= static_cast<long>(kRowsRH2) * p0.G;
  const dim3 block(rh2 ? 512 : 256);
  if (mode == SK_SWIGLU && rh2)
    hipLaunchKernelGGL((gemm_stream_kernel<kNBW, kXBM, kRS2, 2, SK_SWIGLU>), dim3(grid), block,
                       0, stream, p0, p1);
  else if (mode == SK_SWIGLU)
    hipLaunchKernelGGL((gemm_stream_kernel<kNBW, kXBM, kRS, 1, SK_SWIGLU>), dim3(grid), block,
                       0, stream, p0, p1);
  else if (mode == SK_SWIGLU_BWD)
    hipLaunchKernelGGL((gemm_stream_kernel<kNBW, kXBM, kRS, 1, SK_SWIGLU_BWD>), dim3(grid),
                       block, 0, stream, p0, p1);
  else if (rh2)
    hipLaunchKernelGGL((gemm_stream_kernel<kNBW, kXBM, kRS2, 2, SK_PLAIN>), dim3(grid), block,
                       0, stream, p0, p1);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<kNBW, kXBM, kRS, 1, SK_PLAIN>), dim3(grid), block,
                       0, stream, p0, p1);
  return hipGetLastError();
}

bool stream_gemm_supported(bool swiglu, const StreamProblem& p0, const StreamProblem& p1) {
  return supported(swiglu ? SK_SWIGLU : SK_PLAIN, p0, p1);
}

hipError_t launch_stream_gemm(bool swiglu, const StreamProblem& p0, const StreamProblem& p1,
                              hipStream_t stream) {
  return launch(swiglu ? SK_SWIGLU : SK_PLAIN, p0, p1, stream);
}

bool stream_swiglu_bwd_supported(const StreamProblem& p0, const StreamProblem& p1) {
  return supported(SK_SWIGLU_BWD, p0, p1);
}

hipError_t launch_stream_swiglu_bwd(const StreamProblem& p0, const StreamProblem& p1,
                                    hipStream_t stream) {
  return launch(SK_SWIGLU_BWD, p0, p1, stream);
}
