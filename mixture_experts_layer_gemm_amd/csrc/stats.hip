// Router balance statistics and drop diagnostics of one routed batch (forward values).
//
// "Section 10: Routing, Capacity, and Load Balancing": the requested-route fractions
// f_i = C_i^req / (K T) and mean normalized router scores P_i (Eq. 38), the Switch-style
// scalar N f.P (Eq. 30), max/mean imbalance (Eq. 22, 39), normalized entropy deficit,
// coefficient of variation and never-selected count (Section 10.2), the route-drop
// fraction (Eq. 27) and the per-token drop measures Section 10.3 asks for (tokens losing
// at least one and all K routes, selected coefficient mass removed). With destination
// groups of g consecutive experts, also max/mean imbalance of the requested and kept
// destination totals (Eq. 20-22).
//
// stats_partial_kernel: 4 waves per workgroup, `tpb` tokens per workgroup (16 or more,
// chosen so that at most 128 workgroups write partials). A wave loads four tokens' logits
// at once, normalizes each token's N scores (full softmax of the logits, or sigmoid
// affinities divided by their sum) with butterfly reductions and adds them to per-lane
// column sums; lanes k < K accumulate the dropped slots and their coefficients. The four
// waves' partials are added in a fixed order and written per workgroup.
// stats_final_kernel: 256 threads add the partials column by column (threads split the
// workgroups of each expert, eight independent loads in flight, then a fixed-order sum in
// fp64); wave 0 then derives every statistic with fp64 butterfly reductions over the
// experts. No atomics: results are bitwise repeatable.
#include <cmath>

#include "../../include/moe.h"
#include "common.h"

using namespace moe;

namespace {

constexpr int ST_WAVES = 4;
constexpr int ST_BATCH = 4;              // tokens a wave loads at once
constexpr int ST_MAXBLK = 128;           // partial workgroups at most
constexpr int ST_COLS = kMaxN / kWave;   // score columns per lane

__device__ __forceinline__ float st_wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ float st_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ double st_wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ double st_wave_max_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, kWave));
  return v;
}

int stats_tokens_per_block(int T) {
  int tpb = ST_WAVES * ST_BATCH;
  while ((T + tpb - 1) / tpb > ST_MAXBLK) tpb *= 2;
  return tpb;
}

// partial layout per workgroup b: colsum[b][N] (float), then drops[b][4] (float):
// tokens losing >= 1 route, tokens losing all K, dropped coefficient sum, coefficient sum
__global__ void __launch_bounds__(ST_WAVES * kWave)
stats_partial_kernel(int T, int N, int K, int score, int tpb, const float* __restrict__ logits,
                     const int32_t* __restrict__ dest_row, const float* __restrict__ topk_r,
                     float* __restrict__ colsum, float* __restrict__ drops) {
  __shared__ float s_col[ST_WAVES][kMaxN];
  __shared__ float s_drop[ST_WAVES][4];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t0 = blockIdx.x * tpb;
  const int t_end = min(T, t0 + tpb);
  float acc[ST_COLS];
#pragma unroll
  for (int j = 0; j < ST_COLS; ++j) acc[j] = 0.f;
  float lost_any = 0.f, lost_all = 0.f, w_drop = 0.f, w_sel = 0.f;
  for (int base = t0 + w * ST_BATCH; base < t_end; base += ST_WAVES * ST_BATCH) {
    float v[ST_BATCH][ST_COLS];
    int dropped[ST_BATCH];
    float rk[ST_BATCH];
#pragma unroll
    for (int u = 0; u < ST_BATCH; ++u) {  // every load of the batch first
      const int t = base + u;
      const bool ok = t < t_end;
      const float* z = logits + static_cast<size_t>(ok ? t : 0) * N;
#pragma unroll
      for (int j = 0; j < ST_COLS; ++j) {
        const int e = lane + j * kWave;
        v[u][j] = (ok && e < N) ? z[e] : -INFINITY;
      }
      const bool slot = ok && lane < K;
      const size_t tk = static_cast<size_t>(ok ? t : 0) * K + lane;
      dropped[u] = slot ? (dest_row[tk] < 0) : 0;
      rk[u] = slot ? topk_r[tk] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < ST_BATCH; ++u) {
      if (base + u >= t_end) break;  // uniform across the wave
      float sum = 0.f;
      if (score == MOE_SCORE_SIGMOID) {
#pragma unroll
        for (int j = 0; j < ST_COLS; ++j) {
          const int e = lane + j * kWave;
          v[u][j] = e < N ? 1.0f / (1.0f + expf(-v[u][j])) : 0.f;
          sum += v[u][j];
        }
      } else {
        float m = v[u][0];
#pragma unroll
        for (int j = 1; j < ST_COLS; ++j) m = fmaxf(m, v[u][j]);
        m = st_wave_max(m);
#pragma unroll
        for (int j = 0; j < ST_COLS; ++j) {
          const int e = lane + j * kWave;
          v[u][j] = e < N ? expf(v[u][j] - m) : 0.f;
          sum += v[u][j];
        }
      }
      const float inv = 1.0f / st_wave_sum(sum);
#pragma unroll
      for (int j = 0; j < ST_COLS; ++j) acc[j] += v[u][j] * inv;
      const int nd = __popcll(__ballot(dropped[u]));
      lost_any += nd > 0 ? 1.f : 0.f;
      lost_all += nd == K ? 1.f : 0.f;
      w_drop += dropped[u] ? rk[u] : 0.f;
      w_sel += rk[u];
    }
  }
  w_drop = st_wave_sum(w_drop);
  w_sel = st_wave_sum(w_sel);
#pragma unroll
  for (int j = 0; j < ST_COLS; ++j) {
    const int e = lane + j * kWave;
    if (e < N) s_col[w][e] = acc[j];
  }
  if (lane == 0) {
    s_drop[w][0] = lost_any;
    s_drop[w][1] = lost_all;
    s_drop[w][2] = w_drop;
    s_drop[w][3] = w_sel;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += ST_WAVES * kWave) {
    float s = s_col[0][e];
#pragma unroll
    for (int q = 1; q < ST_WAVES; ++q) s += s_col[q][e];  // fixed order
    colsum[static_cast<size_t>(blockIdx.x) * N + e] = s;
  }
  if (threadIdx.x < 4) {
    float s = s_drop[0][threadIdx.x];
#pragma unroll
    for (int q = 1; q < ST_WAVES; ++q) s += s_drop[q][threadIdx.x];
    drops[blockIdx.x * 4 + threadIdx.x] = s;
  }
}

constexpr int SF_THREADS = 256;

__global__ void __launch_bounds__(SF_THREADS)
stats_final_kernel(int T, int N, int K, int group, int nblk, int NP,
                   const float* __restrict__ colsum, const float* __restrict__ drops,
                   const int32_t* __restrict__ C_req, const int32_t* __restrict__ C_keep,
                   float* __restrict__ P_out, float* __restrict__ stats) {
  __shared__ double part[SF_THREADS];
  __shared__ double dpart[64];
  __shared__ double s_P[kMaxN], s_req[kMaxN], s_keep[kMaxN];
  const int tid = threadIdx.x;
  // column sums: thread (e, q) adds workgroups [q per, (q+1) per) of expert e
  {
    const int Q = SF_THREADS / NP;
    const int e = tid % NP, q = tid / NP;
    const int per = (nblk + Q - 1) / Q;
    const int b0 = min(q * per, nblk), b1 = min(b0 + per, nblk);
    double acc = 0.0;
    if (e < N) {
      int b = b0;
      for (; b + 8 <= b1; b += 8) {
        float h[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) h[u] = colsum[static_cast<size_t>(b + u) * N + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += h[u];
      }
      for (; b < b1; ++b) acc += colsum[static_cast<size_t>(b) * N + e];
    }
    part[tid] = acc;
  }
  // drop partials: 16 runs of workgroups for each of the 4 values
  if (tid < 64) {
    const int v = tid & 3, q = tid >> 2;
    const int per = (nblk + 15) / 16;
    const int b0 = min(q * per, nblk), b1 = min(b0 + per, nblk);
    double acc = 0.0;
    for (int b = b0; b < b1; ++b) acc += drops[b * 4 + v];
    dpart[tid] = acc;
  }
  __syncthreads();
  if (tid < N) {
    const int Q = SF_THREADS / NP;
    double P = 0.0;
    for (int q = 0; q < Q; ++q) P += part[q * NP + tid];  // fixed order
    P /= T;
    s_P[tid] = P;
    s_req[tid] = C_req[tid];
    s_keep[tid] = C_keep[tid];
    P_out[tid] = static_cast<float>(P);
  }
  __syncthreads();
  if (tid >= kWave) return;
  // wave 0: lane l owns experts l, l + 64, ...
  const int lane = tid;
  const double KT = static_cast<double>(K) * T;
  double fP = 0.0, sreq = 0.0, skeep = 0.0, never = 0.0, mreq = 0.0, mkeep = 0.0;
  for (int e = lane; e < N; e += kWave) {
    fP += s_req[e] / KT * s_P[e];
    sreq += s_req[e];
    skeep += s_keep[e];
    never += s_req[e] == 0.0 ? 1.0 : 0.0;
    mreq = fmax(mreq, s_req[e]);
    mkeep = fmax(mkeep, s_keep[e]);
  }
  fP = st_wave_sum_d(fP);
  sreq = st_wave_sum_d(sreq);
  skeep = st_wave_sum_d(skeep);
  never = st_wave_sum_d(never);
  mreq = st_wave_max_d(mreq);
  mkeep = st_wave_max_d(mkeep);
  const double mean_req = sreq / N, mean_keep = skeep / N;
  double hreq = 0.0, hkeep = 0.0, vreq = 0.0, vkeep = 0.0;
  for (int e = lane; e < N; e += kWave) {
    if (s_req[e] > 0.0) hreq -= (s_req[e] / sreq) * log(s_req[e] / sreq);
    if (s_keep[e] > 0.0) hkeep -= (s_keep[e] / skeep) * log(s_keep[e] / skeep);
    vreq += (s_req[e] - mean_req) * (s_req[e] - mean_req);
    vkeep += (s_keep[e] - mean_keep) * (s_keep[e] - mean_keep);
  }
  hreq = st_wave_sum_d(hreq);
  hkeep = st_wave_sum_d(hkeep);
  vreq = st_wave_sum_d(vreq) / N;
  vkeep = st_wave_sum_d(vkeep) / N;
  // destination totals R_q: lane l sums destinations l, l + 64, ... (experts in order)
  const int M = group > 0 ? N / group : 0;
  double mrreq = 0.0, mrkeep = 0.0;
  for (int q = lane; q < M; q += kWave) {
    double rq = 0.0, rk = 0.0;
    for (int j = q * group; j < (q + 1) * group; ++j) {
      rq += s_req[j];
      rk += s_keep[j];
    }
    mrreq = fmax(mrreq, rq);
    mrkeep = fmax(mrkeep, rk);
  }
  mrreq = st_wave_max_d(mrreq);
  mrkeep = st_wave_max_d(mrkeep);
  double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
  for (int q = 0; q < 16; ++q) {  // fixed order
    d0 += dpart[q * 4];
    d1 += dpart[q * 4 + 1];
    d2 += dpart[q * 4 + 2];
    d3 += dpart[q * 4 + 3];
  }
  if (lane == 0) {
    const double nan = __builtin_nan("");
    const double logn = log(static_cast<double>(N));
    stats[MOE_STAT_LBL] = static_cast<float>(N * fP);
    stats[MOE_STAT_IMAX_REQ] = static_cast<float>(sreq > 0 ? N * mreq / sreq : nan);
    stats[MOE_STAT_IMAX_KEEP] = static_cast<float>(skeep > 0 ? N * mkeep / skeep : nan);
    // one expert: log N = 0, the load is balanced by construction and the deficit is 0
    stats[MOE_STAT_IH_REQ] = static_cast<float>(sreq > 0 ? (N > 1 ? 1.0 - hreq / logn : 0.0) : nan);
    stats[MOE_STAT_IH_KEEP] = static_cast<float>(skeep > 0 ? (N > 1 ? 1.0 - hkeep / logn : 0.0) : nan);
    stats[MOE_STAT_CV_REQ] = static_cast<float>(mean_req > 0 ? sqrt(vreq) / mean_req : nan);
    stats[MOE_STAT_CV_KEEP] = static_cast<float>(mean_keep > 0 ? sqrt(vkeep) / mean_keep : nan);
    stats[MOE_STAT_NEVER_SELECTED] = static_cast<float>(never);
    stats[MOE_STAT_DELTA_ROUTE] = static_cast<float>((KT - skeep) / KT);
    stats[MOE_STAT_TOKENS_LOST_ANY] = static_cast<float>(d0);
    stats[MOE_STAT_TOKENS_LOST_ALL] = static_cast<float>(d1);
    stats[MOE_STAT_WEIGHT_REMOVED] = static_cast<float>(d3 > 0 ? d2 / d3 : nan);
    // destination totals sum to the expert totals
    stats[MOE_STAT_IMAX_RANK_REQ] = static_cast<float>(M > 0 && sreq > 0 ? M * mrreq / sreq : nan);
    stats[MOE_STAT_IMAX_RANK_KEEP] = static_cast<float>(M > 0 && skeep > 0 ? M * mrkeep / skeep : nan);
  }
}

}  // namespace

size_t stats_workspace_bytes(int T, int N) {
  const int tpb = stats_tokens_per_block(T);
  const size_t nblk = (static_cast<size_t>(T) + tpb - 1) / tpb;
  return nblk * (static_cast<size_t>(N) + 4) * sizeof(float);
}

hipError_t launch_balance_stats(int T, int N, int K, int score, int group, const float* logits,
                                const int32_t* dest_row, const float* topk_r,
                                const int32_t* C_req, const int32_t* C_keep, float* P,
                                float* stats, void* workspace, hipStream_t stream) {
  const int tpb = stats_tokens_per_block(T);
  const int nblk = (T + tpb - 1) / tpb;
  float* colsum = static_cast<float*>(workspace);
  float* drops = colsum + static_cast<size_t>(nblk) * N;
  int NP = 1;
  while (NP < N) NP <<= 1;
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(ST_WAVES * kWave), 0, stream, T, N,
                     K, score, tpb, logits, dest_row, topk_r, colsum, drops);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(SF_THREADS), 0, stream, T, N, K, group,
                     nblk, NP, colsum, drops, C_req, C_keep, P, stats);
  return hipGetLastError();
}
