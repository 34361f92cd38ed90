// Backward of the layer with the router held fixed ("Section 21: Merging Routed and
// Shared Expert Activations", Eq. 80 and Section 21.3's fixed-router gradients; the
// SwiGLU expert of "Section 20: One Shared Expert Is All You Need", Eq. 74).
//
// With A = X W_g^T, B = X W_u^T, S = SiLU(A), H = S * B and F = H W_d^T per expert, and
// the upstream gradient dF of each kept route's row equal to r dy (s dy for the shared
// branch), the chain rule gives
//   dH = dF W_d,  dA = dH * B * SiLU'(A),  dB = dH * S,  dX = [dA dB] [W_g; W_u],
//   dW_d = dF^T H,  dW_g = dA^T X,  dW_u = dB^T X.
// The data-gradient contractions (dH, dX) and the recomputation of A and B run on the
// forward's persistent grouped GEMM over weights packed in MFMA-operand order (the
// transposed weights come from transpose_pack_kernel). This file holds the rest:
//   transpose_pack_kernel  packs W^T (optionally two matrices stacked along the
//                          contraction) in the MFMA-operand order, through an LDS tile
//   grad_rows_kernel       dF rows (r dy gathered into the packed expert order) and the
//                          shared branch's s dy, one wave per token
//   swiglu_bwd_kernel      dA | dB and H from dH, A, B (fp32 math, bf16 out)
//   wgrad_kernel           weight gradients, a grouped GEMM contracting over each
//                          expert's ragged row segment: rows reach LDS by direct-to-LDS
//                          loads in a 4-stage ring and the MFMA fragments come out with the
//                          LDS transpose read (ds_read_b64_tr_b16).
#include "gemm_common.h"

using namespace moe;

namespace {

// ---- transpose into the packed operand order ----------------------------------------
// dst[g][nb][kb][lane][8] = Wt[g][32 nb + (lane & 31)][16 kb + 8 (lane >> 5) + 0..7], with
// Wt[g][n][k] = S[g][k][n] and S = [A; B] stacked along k (A has Ka rows, B the rest).
constexpr int TP = 64;        // tile edge (k and n)
constexpr int TP_LD = TP + 8; // padded LDS row (n)

__global__ void __launch_bounds__(256)
transpose_pack_kernel(int Nn, int Kk, int Ka, const uint16_t* __restrict__ A,
                      const uint16_t* __restrict__ B, uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[TP][TP_LD];
  const int kt = Kk / TP, nt = Nn / TP;
  const int bid = blockIdx.x;
  const int n_tile = bid % nt;
  const int k_tile = (bid / nt) % kt;
  const long g = bid / (nt * kt);
  const int k0 = k_tile * TP, n0 = n_tile * TP;
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {  // 64 rows x 8 pieces of 16 bytes
    const int piece = tid + h * 256;
    const int kr = piece >> 3, c = (piece & 7) * 8;
    const int k = k0 + kr;
    const uint16_t* src = k < Ka ? A + (g * Ka + k) * static_cast<long>(Nn)
                                 : B + (g * (Kk - Ka) + (k - Ka)) * static_cast<long>(Nn);
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + n0 + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[kr][c + 2 * i] = static_cast<uint16_t>(v[i] & 0xFFFFu);
      tile[kr][c + 2 * i + 1] = static_cast<uint16_t>(v[i] >> 16);
    }
  }
  __syncthreads();
  const int KB = Kk / 16, NB = Nn / 32;
#pragma unroll
  for (int h = 0; h < 2; ++h) {  // 2 n-blocks x 4 k-blocks x 64 lanes
    const int piece = tid + h * 256;
    const int lane = piece & 63, blk = piece >> 6;
    const int nbl = blk >> 2, kbl = blk & 3;
    const int nl = 32 * nbl + (lane & 31), kl = 16 * kbl + 8 * (lane >> 5);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = static_cast<uint32_t>(tile[kl + 2 * i][nl]) |
             (static_cast<uint32_t>(tile[kl + 2 * i + 1][nl]) << 16);
    const long nb = n0 / 32 + nbl, kb = k0 / 16 + kbl;
    reinterpret_cast<u32x4*>(dst)[((g * NB + nb) * KB + kb) * 64 + lane] = o;
  }
}

// ---- upstream gradient rows ---------------------------------------------------------
constexpr int GR_WAVES = 4;

__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 u, float c) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(u[i] << 16) * c;
    const float hi = __uint_as_float(u[i] & 0xFFFF0000u) * c;
    o[i] = pack_bf16x2(lo, hi);
  }
  return o;
}

// dF[dest_row[t][k]] = r[t][k] dy[t] for kept routes; dG[t] = s_t dy[t] when dG != null
__global__ void __launch_bounds__(GR_WAVES * kWave)
grad_rows_kernel(int T, int d, int K, const uint16_t* __restrict__ dy,
                 const int32_t* __restrict__ dest_row, const float* __restrict__ topk_r,
                 float s, const float* __restrict__ s_tok, uint16_t* __restrict__ dF,
                 uint16_t* __restrict__ dG) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * GR_WAVES + (threadIdx.x >> 6);
  if (t >= T) return;
  int dk = -1;
  float rk = 0.f;
  if (lane < K) {
    dk = dest_row[static_cast<size_t>(t) * K + lane];
    rk = topk_r[static_cast<size_t>(t) * K + lane];
  }
  const float st = s_tok != nullptr ? s_tok[t] : s;
  const int npc = d / 8;
  for (int j = lane; j < npc; j += kWave) {
    const u32x4 u = reinterpret_cast<const u32x4*>(dy + static_cast<size_t>(t) * d)[j];
    for (int k = 0; k < K; ++k) {
      const int row = __shfl(dk, k, kWave);
      const float rr = __shfl(rk, k, kWave);
      if (row < 0) continue;
      reinterpret_cast<u32x4*>(dF + static_cast<size_t>(row) * d)[j] = scale_bf16x8(u, rr);
    }
    if (dG != nullptr)
      reinterpret_cast<u32x4*>(dG + static_cast<size_t>(t) * d)[j] = scale_bf16x8(u, st);
  }
}

// ---- SwiGLU backward ----------------------------------------------------------------
// rows [0, rows_dev ? *rows_dev : rows): dAB[j] = [dA | dB] (2 d_ff wide), H[j] = S * B
__global__ void __launch_bounds__(256)
swiglu_bwd_kernel(int rows, const int32_t* __restrict__ rows_dev, int dff,
                  const uint16_t* __restrict__ dH, const uint16_t* __restrict__ Av,
                  const uint16_t* __restrict__ Bv, uint16_t* __restrict__ dAB,
                  uint16_t* __restrict__ H) {
  const int R = rows_dev != nullptr ? min(rows, *rows_dev) : rows;
  const int per_row = dff / 8;
  const long total = static_cast<long>(R) * per_row;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += static_cast<long>(gridDim.x) * 256) {
    const long j = i / per_row;
    const int c = static_cast<int>(i % per_row) * 8;
    const size_t o = static_cast<size_t>(j) * dff + c;
    const u32x4 uh = *reinterpret_cast<const u32x4*>(dH + o);
    const u32x4 ua = *reinterpret_cast<const u32x4*>(Av + o);
    const u32x4 ub = *reinterpret_cast<const u32x4*>(Bv + o);
    u32x4 oa, ob, oh;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float da[2], db[2], hh[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float g = __uint_as_float(h ? (uh[q] & 0xFFFF0000u) : (uh[q] << 16));
        const float a = __uint_as_float(h ? (ua[q] & 0xFFFF0000u) : (ua[q] << 16));
        const float b = __uint_as_float(h ? (ub[q] & 0xFFFF0000u) : (ub[q] << 16));
        const float sg = 1.0f / (1.0f + expf(-a));
        const float sa = a * sg;
        db[h] = g * sa;
        da[h] = g * b * sg * (1.0f + a * (1.0f - sg));
        hh[h] = sa * b;
      }
      oa[q] = pack_bf16x2(da[0], da[1]);
      ob[q] = pack_bf16x2(db[0], db[1]);
      oh[q] = pack_bf16x2(hh[0], hh[1]);
    }
    const size_t o2 = static_cast<size_t>(j) * 2 * dff + c;
    *reinterpret_cast<u32x4*>(dAB + o2) = oa;
    *reinterpret_cast<u32x4*>(dAB + o2 + dff) = ob;
    *reinterpret_cast<u32x4*>(H + o) = oh;
  }
}

// ---- weight gradients: out[g][m][n] = sum_{j in segment g} P[j][m] Q[row(j)][n] ---------
// Both operands are k-major (k = the row j of a segment), while v_mfma_f32_32x32x16_bf16
// wants 8 consecutive k of one column per lane. The rows go to LDS as they are, by
// direct-to-LDS loads into a ring of W2_XS stages (32 rows each), and the fragments come out
// with ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i & 3 of the
// 8-byte pieces that lanes (i >> 2), 4 + (i >> 2), 8 + (i >> 2), 12 + (i >> 2) of the
// group point at; pointing lane s at column block 4 (s & 3) of row s >> 2 therefore hands
// lane i four consecutive rows of one column. An 8-byte-unit XOR swizzle per row keeps
// those reads free of bank conflicts.
constexpr int W2_BM = 256, W2_BN = 128;       // output tile (M: P columns, N: Q columns)
constexpr int W2_BK = 32;                     // segment rows per stage
constexpr int W2_XS = 2;                      // ring depth (stages)
static_assert(W2_XS == 2 || W2_XS == 3, "the stage waits are written for 2 or 3 stages");
constexpr int W2_ROWP = W2_BM * 2;            // LDS bytes per stage row of P (256 bf16)
constexpr int W2_ROWQ = W2_BN * 2;            // LDS bytes per stage row of Q (128 bf16)
constexpr int W2_OPP = W2_BK * W2_ROWP;       // bytes of P per stage
constexpr int W2_STAGE = W2_BK * (W2_ROWP + W2_ROWQ);
constexpr int W2_DPP = W2_OPP / (1024 * 4);   // direct-to-LDS loads of P per wave per stage
constexpr int W2_DPQ = W2_BK * W2_ROWQ / (1024 * 4);
constexpr int W2_DPW = W2_DPP + W2_DPQ;       // loads per wave per stage
constexpr int W2_RPP = 1024 / W2_ROWP;        // P rows per load
constexpr int W2_CPP = W2_ROWP / 16;          // 16-byte chunks per P row
constexpr int W2_PB = W2_BM / 64;             // 32-column P blocks per wave (half the tile)
constexpr int W2_EROWS = 64;                  // epilogue rows per pass through the ring
static_assert(W2_XS * W2_STAGE >= W2_EROWS * W2_BN * 4, "the epilogue reuses the ring");
static_assert(W2_DPP * W2_RPP == 8 && W2_DPQ == 2, "each wave loads 8 rows of each operand per stage");

struct WgradProblem {
  const uint16_t* P;      // [rows][ldp], columns [0, M) used
  int ldp;
  const uint16_t* Q;      // [*][ldq], row j or row_index[j]; columns [0, Nc)
  int ldq;
  const int32_t* row_index;
  const int32_t* offsets; // [G+1] device, or null: one segment [0, rows)
  int rows;
  int G, M, Nc;
  float* out;             // [G][M][Nc]
};

// physical 16-byte chunk of logical chunk c in stage row r (the low 4 bits are permuted,
// so the map stays inside every 16-chunk block of a row)
__device__ __forceinline__ int w2_swz(int r, int c) {
  const int q = r & 3;
  return c ^ (2 * q + 8 * (q & 1));
}

__device__ __forceinline__ void w2_dma16(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

typedef short w2_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) w2_v4s w2_lv4s;

__global__ void __launch_bounds__(256, 3)
wgrad_kernel(WgradProblem q0, WgradProblem q1, int s_per, int r_per) {
  __shared__ __attribute__((aligned(1024))) char ring[W2_XS * W2_STAGE];
  typedef __attribute__((address_space(3))) char lds_char;
  // consecutive workgroups land on different XCDs: give each XCD a contiguous range of
  // tiles so that the tiles of one expert share an L2. The second problem (the shared
  // MLP: few tiles, each contracting over every token) comes first in every XCD's range,
  // so its long tiles start first and the short expert tiles fill in around them.
  const int b = blockIdx.x;
  const int xcd = b % 8, local = b / 8;
  const bool second = local < s_per;
  const int tile = second ? xcd * s_per + local : xcd * r_per + (local - s_per);
  // the tile's problem, field by field (a reference to either argument would be copied
  // to scratch)
  WgradProblem pb;
  pb.P = second ? q1.P : q0.P;
  pb.ldp = second ? q1.ldp : q0.ldp;
  pb.Q = second ? q1.Q : q0.Q;
  pb.ldq = second ? q1.ldq : q0.ldq;
  pb.row_index = second ? q1.row_index : q0.row_index;
  pb.offsets = second ? q1.offsets : q0.offsets;
  pb.rows = second ? q1.rows : q0.rows;
  pb.G = second ? q1.G : q0.G;
  pb.M = second ? q1.M : q0.M;
  pb.Nc = second ? q1.Nc : q0.Nc;
  pb.out = second ? q1.out : q0.out;
  const int tiles_m = (pb.M + W2_BM - 1) / W2_BM, tiles_n = (pb.Nc + W2_BN - 1) / W2_BN;
  const int total = pb.G * tiles_m * tiles_n;
  if ((second ? local : local - s_per) >= (second ? s_per : r_per) || tile >= total) return;
  const int tn = tile % tiles_n;
  const int tm = (tile / tiles_n) % tiles_m;
  const int g = tile / (tiles_n * tiles_m);
  const int m0 = tm * W2_BM, n0 = tn * W2_BN;
  const int j0 = __builtin_amdgcn_readfirstlane(pb.offsets != nullptr ? pb.offsets[g] : 0);
  const int j1 = __builtin_amdgcn_readfirstlane(pb.offsets != nullptr ? pb.offsets[g + 1] : pb.rows);
  const int nst = (j1 - j0 + W2_BK - 1) / W2_BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const uint32_t lds0 = static_cast<uint32_t>((size_t)((lds_char*)ring));
  const int32_t* gather = pb.row_index;
  const int rb = 8 * w;  // wave w brings stage rows rb .. rb + 7 of both operands

  // one stage: P rows as 2 rows x 32 chunks per load (lane j -> row rb + 2 i + (j >> 5),
  // physical chunk j & 31), Q rows as 4 rows x 16 chunks (row rb + 4 i + (j >> 4),
  // physical chunk j & 15); rows past the segment are clamped to its last row and zeroed
  // after landing, columns past the matrix read column 0 and are never stored
  auto issue = [&](int s, int slot) {
    const int jr = j0 + s * W2_BK + rb;
    const uint32_t sb = lds0 + slot * W2_STAGE;
#pragma unroll
    for (int i = 0; i < W2_DPP; ++i) {
      const int row = rb + W2_RPP * i + lane / W2_CPP;
      const int grow = min(jr + W2_RPP * i + lane / W2_CPP, j1 - 1);
      int col = m0 + 8 * w2_swz(row, lane % W2_CPP);
      if (col >= pb.M) col = 0;
      const uint32_t off = static_cast<uint32_t>((static_cast<long>(grow) * pb.ldp + col) * 2);
      w2_dma16(off, pb.P, sb + (rb + W2_RPP * i) * W2_ROWP);
    }
#pragma unroll
    for (int i = 0; i < W2_DPQ; ++i) {
      // row indices: uniform addresses, so scalar loads, which the direct-to-LDS
      // accounting (vector memory) does not see
      const int sel = lane >> 4;
      const int row = rb + 4 * i + sel;
      const int ja = min(jr + 4 * i, j1 - 1), jb = min(jr + 4 * i + 1, j1 - 1);
      const int jc = min(jr + 4 * i + 2, j1 - 1), jd = min(jr + 4 * i + 3, j1 - 1);
      int ra = ja, rbv = jb, rc = jc, rd = jd;
      if (gather != nullptr) {
        // the row index is read-only for the whole launch: constant address space, so the
        // uniform loads become scalar loads
        typedef const __attribute__((address_space(4))) int32_t cint;
        cint* cg = (cint*)(gather);
        ra = cg[ja];
        rbv = cg[jb];
        rc = cg[jc];
        rd = cg[jd];
      }
      const int grow = sel == 0 ? ra : (sel == 1 ? rbv : (sel == 2 ? rc : rd));
      int col = n0 + 8 * w2_swz(row, lane & 15);
      if (col >= pb.Nc) col = 0;
      const uint32_t off = static_cast<uint32_t>((static_cast<long>(grow) * pb.ldq + col) * 2);
      w2_dma16(off, pb.Q, sb + W2_OPP + (rb + 4 * i) * W2_ROWQ);
    }
  };

  // fragment of the 32 columns [cb, cb + 32) of an operand (rows of rowb bytes) for k16
  // step t: lane l holds column cb + (l & 31), stage rows 16 t + 8 (l >> 5) + 0..7
  auto frag = [&](uint32_t opbase, int rowb, int cb, int t) -> bf16x8 {
    const int gq = lane >> 4, sl = lane & 15;
    const int col = cb + 16 * (gq & 1) + 4 * (sl & 3);
    const int u = col >> 2;
    w2_v4s part[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * t + 8 * (gq >> 1) + 4 * h + (sl >> 2);
      const int q = row & 3;
      const uint32_t addr = opbase + row * rowb + ((u ^ (4 * q + 16 * (q & 1))) << 3);
      part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((w2_lv4s*)((lds_char*)nullptr + addr));
    }
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s both = {part[0][0], part[0][1], part[0][2], part[0][3],
                      part[1][0], part[1][1], part[1][2], part[1][3]};
    return __builtin_bit_cast(bf16x8, both);
  };

  // wave (wm, wn) owns tile rows wm * BM / 2 .. + BM / 2 - 1 (PB blocks of 32) and
  // columns wn * 64 .. + 63 (2 blocks of 32)
  floatx16 acc[W2_PB][2];
#pragma unroll
  for (int i = 0; i < W2_PB; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;

#pragma unroll
  for (int v = 0; v < W2_XS - 1; ++v)
    if (v < nst) issue(v, v);
  for (int s = 0; s < nst; ++s) {
    // this stage's loads have landed; the stages issued after it (min(XS - 2, nst - 1 - s)
    // of them: stage s + XS - 2 was issued during stage s - 1) may still be in flight
    if constexpr (W2_XS == 2) {
      wait_vmcnt<0>();
    } else {
      if (s + 1 < nst) wait_vmcnt<W2_DPW>();
      else wait_vmcnt<0>();
    }
    const uint32_t sb = lds0 + (s % W2_XS) * W2_STAGE;
    // rows past the segment (last stage only) read as zero: each wave clears its own rows
    if (j0 + (s + 1) * W2_BK > j1) {
      const int r = rb + (lane >> 3);
      if (j0 + s * W2_BK + r >= j1) {
        typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
        lds_u32x4* zp = (lds_u32x4*)((lds_char*)nullptr + sb + r * W2_ROWP + (lane & 7) * (W2_ROWP / 8));
        lds_u32x4* zq = (lds_u32x4*)((lds_char*)nullptr + sb + W2_OPP + r * W2_ROWQ + (lane & 7) * 32);
#pragma unroll
        for (int c = 0; c < W2_ROWP / 128; ++c) zp[c] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 2; ++c) zq[c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();  // publishes this stage; every wave is done with stage s - 1's slot
    if (s + W2_XS - 1 < nst) issue(s + W2_XS - 1, (s + W2_XS - 1) % W2_XS);
#pragma unroll
    for (int t = 0; t < W2_BK / 16; ++t) {
      // the Q fragments stay, one P fragment at a time (registers for a third workgroup)
      bf16x8 bf[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) bf[jj] = frag(sb + W2_OPP, W2_ROWQ, wn * 64 + jj * 32, t);
#pragma unroll
      for (int i = 0; i < W2_PB; ++i) {
        const bf16x8 af = frag(sb, W2_ROWP, wm * (W2_BM / 2) + i * 32, t);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[jj], acc[i][jj], 0, 0, 0);
      }
    }
  }
  // epilogue through LDS (the ring is free once every wave is past the last stage), in
  // passes of 64 tile rows: the rows go in as 128 fp32 each and leave as whole 16-byte
  // row pieces. 4-float pieces are swizzled by 8 (row / 4 odd), so the two rows that one
  // accumulator store writes (4 apart) fall 32 banks apart.
  float* tileo = (float*)ring;
  float* out = pb.out + static_cast<size_t>(g) * pb.M * pb.Nc;
  const int pc = tid & 31;  // 4-float column piece of this thread
  const int n = n0 + 4 * pc;
#pragma unroll
  for (int ps = 0; ps < W2_BM / W2_EROWS; ++ps) {
    __syncthreads();
    // pass ps holds tile rows 64 ps .. + 63: the waves' 32-row blocks wm PB + i with
    // (wm PB + i) / 2 = ps
#pragma unroll
    for (int i = 0; i < W2_PB; ++i) {
      const int gb = wm * W2_PB + i;
      if (gb / 2 == ps) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int vv = 0; vv < 16; ++vv) {
            // lane holds row 8 (v / 4) + 4 (lane / 32) + v % 4, column lane % 32 of the block
            const int m = (gb & 1) * 32 + 8 * (vv >> 2) + 4 * (lane >> 5) + (vv & 3);
            const int nn = wn * 64 + jj * 32 + (lane & 31);
            tileo[m * W2_BN + 4 * ((nn >> 2) ^ (8 * ((m >> 2) & 1))) + (nn & 3)] = acc[i][jj][vv];
          }
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int r = tid >> 5; r < W2_EROWS; r += 8) {
      const int m = m0 + ps * W2_EROWS + r;
      // M and Nc are multiples of 64: a piece is wholly inside or wholly outside
      // written once and not read back here: non-temporal, so the stream of fp32
      // gradients does not evict the operand rows from L2
      if (m < pb.M && n < pb.Nc)
        __builtin_nontemporal_store(
            *reinterpret_cast<const floatx4*>(tileo + r * W2_BN + 4 * (pc ^ (8 * ((r >> 2) & 1)))),
            reinterpret_cast<floatx4*>(out + static_cast<size_t>(m) * pb.Nc + n));
    }
  }
}

}  // namespace

hipError_t launch_transpose_pack(int G, int Nn, int Kk, int Ka, const void* A, const void* B,
                                 void* dst, hipStream_t stream) {
  const long grid = static_cast<long>(G) * (Kk / TP) * (Nn / TP);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_pack_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     stream, Nn, Kk, Ka, static_cast<const uint16_t*>(A),
                     static_cast<const uint16_t*>(B), static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_grad_rows(int T, int d, int K, const void* dy, const int32_t* dest_row,
                            const float* topk_r, float s, const float* s_tok, void* dF,
                            void* dG, hipStream_t stream) {
  const int grid = (T + GR_WAVES - 1) / GR_WAVES;
  hipLaunchKernelGGL(grad_rows_kernel, dim3(grid), dim3(GR_WAVES * kWave), 0, stream, T, d, K,
                     static_cast<const uint16_t*>(dy), dest_row, topk_r, s, s_tok,
                     static_cast<uint16_t*>(dF), static_cast<uint16_t*>(dG));
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int rows, const int32_t* rows_dev, int dff, const void* dH,
                             const void* A, const void* B, void* dAB, void* H,
                             hipStream_t stream) {
  const long total = static_cast<long>(rows) * (dff / 8);
  if (total <= 0) return hipSuccess;
  long grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                     rows, rows_dev, dff, static_cast<const uint16_t*>(dH),
                     static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B),
                     static_cast<uint16_t*>(dAB), static_cast<uint16_t*>(H));
  return hipGetLastError();
}

hipError_t launch_wgrad(int G, int M, int Nc, const void* P, int ldp, const void* Q, int ldq,
                        const int32_t* row_index, const int32_t* offsets, int rows, float* out,
                        int M1, int Nc1, const void* P1, int ldp1, const void* Q1, int ldq1,
                        int rows1, float* out1, hipStream_t stream) {
  WgradProblem q0{static_cast<const uint16_t*>(P), ldp, static_cast<const uint16_t*>(Q), ldq,
                  row_index, offsets, rows, G, M, Nc, out};
  WgradProblem q1{static_cast<const uint16_t*>(P1), ldp1, static_cast<const uint16_t*>(Q1), ldq1,
                  nullptr, nullptr, rows1, out1 != nullptr ? 1 : 0, M1, Nc1, out1};
  auto tiles = [](const WgradProblem& q) -> long {
    return static_cast<long>(q.G) * ((q.M + W2_BM - 1) / W2_BM) * ((q.Nc + W2_BN - 1) / W2_BN);
  };
  const long t0 = tiles(q0), t1 = out1 != nullptr ? tiles(q1) : 0;
  if (t0 + t1 <= 0) return hipSuccess;
  // 32-bit byte offsets of the direct-to-LDS loads
  auto fits = [](long rows_, int ld_) { return rows_ * ld_ * 2L < (1L << 32); };
  if (!fits(rows, ldp) || !fits(rows, ldq) || (out1 != nullptr && (!fits(rows1, ldp1) || !fits(rows1, ldq1))))
    return hipErrorNotSupported;
  if (t0 + t1 > 0x3fffffffL) return hipErrorInvalidValue;
  const long s_per = (t1 + 7) / 8, r_per = (t0 + 7) / 8;
  const long grid = 8 * (s_per + r_per);
  hipLaunchKernelGGL(wgrad_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, q0,
                     q1, static_cast<int>(s_per), static_cast<int>(r_per));
  return hipGetLastError();
}
