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
// stats_partial_kernel: one wave per token, 4 waves per workgroup, TPB tokens per
// workgroup. A wave normalizes its token's N scores (full softmax of the logits, or
// sigmoid affinities divided by their sum) with butterfly reductions and adds them to
// per-lane column sums; lanes k < K count the dropped slots and their coefficients. The
// four waves' partials are added in a fixed order and written per workgroup.
// stats_final_kernel: one workgroup adds the partials in workgroup order in fp64 and
// derives every statistic. No atomics: results are bitwise repeatable.
#include <cmath>

#include "../../include/moe.h"
#include "common.h"

using namespace moe;

namespace {

constexpr int ST_WAVES = 4;
constexpr int ST_TPB = 64;           // tokens per workgroup
constexpr int ST_COLS = kMaxN / kWave;  // score columns per lane

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

// partial layout per workgroup b: colsum[b][N] (float), then drops[b][4] (float):
// tokens losing >= 1 route, tokens losing all K, dropped coefficient sum, coefficient sum
__global__ void __launch_bounds__(ST_WAVES * kWave)
stats_partial_kernel(int T, int N, int K, int score, const float* __restrict__ logits,
                     const int32_t* __restrict__ dest_row, const float* __restrict__ topk_r,
                     float* __restrict__ colsum, float* __restrict__ drops) {
  __shared__ float s_col[ST_WAVES][kMaxN];
  __shared__ float s_drop[ST_WAVES][4];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t0 = blockIdx.x * ST_TPB;
  float acc[ST_COLS];
#pragma unroll
  for (int j = 0; j < ST_COLS; ++j) acc[j] = 0.f;
  float lost_any = 0.f, lost_all = 0.f, w_drop = 0.f, w_sel = 0.f;
  for (int t = t0 + w; t < min(T, t0 + ST_TPB); t += ST_WAVES) {
    const float* z = logits + static_cast<size_t>(t) * N;
    float v[ST_COLS];
#pragma unroll
    for (int j = 0; j < ST_COLS; ++j) {
      const int e = lane + j * kWave;
      v[j] = e < N ? z[e] : -INFINITY;
    }
    float sum = 0.f;
    if (score == MOE_SCORE_SIGMOID) {
#pragma unroll
      for (int j = 0; j < ST_COLS; ++j) {
        const int e = lane + j * kWave;
        v[j] = e < N ? 1.0f / (1.0f + expf(-v[j])) : 0.f;
        sum += v[j];
      }
    } else {
      float m = v[0];
#pragma unroll
      for (int j = 1; j < ST_COLS; ++j) m = fmaxf(m, v[j]);
      m = st_wave_max(m);
#pragma unroll
      for (int j = 0; j < ST_COLS; ++j) {
        const int e = lane + j * kWave;
        v[j] = e < N ? expf(v[j] - m) : 0.f;
        sum += v[j];
      }
    }
    const float inv = 1.0f / st_wave_sum(sum);
#pragma unroll
    for (int j = 0; j < ST_COLS; ++j) acc[j] += v[j] * inv;
    // dropped slots of this token (lanes k < K)
    int dropped = 0;
    float rk = 0.f;
    if (lane < K) {
      const size_t tk = static_cast<size_t>(t) * K + lane;
      dropped = dest_row[tk] < 0;
      rk = topk_r[tk];
    }
    const int nd = __popcll(__ballot(dropped));
    lost_any += nd > 0 ? 1.f : 0.f;
    lost_all += nd == K ? 1.f : 0.f;
    w_drop += st_wave_sum(dropped ? rk : 0.f);
    w_sel += st_wave_sum(rk);
  }
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

// fixed-order tree sum / max over the workgroup (fp64)
__device__ double sf_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int off = SF_THREADS / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}
__device__ double sf_max(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int off = SF_THREADS / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmax(red[tid], red[tid + off]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(SF_THREADS)
stats_final_kernel(int T, int N, int K, int group, int nblk, const float* __restrict__ colsum,
                   const float* __restrict__ drops, const int32_t* __restrict__ C_req,
                   const int32_t* __restrict__ C_keep, float* __restrict__ P_out,
                   float* __restrict__ stats) {
  __shared__ double red[SF_THREADS];
  __shared__ double s_req[SF_THREADS], s_keep[SF_THREADS];
  const int tid = threadIdx.x;
  const double KT = static_cast<double>(K) * T;
  // P_i and per-expert terms (N <= 256: one expert per thread)
  double P = 0.0, creq = 0.0, ckeep = 0.0;
  const bool act = tid < N;
  if (act) {
    for (int b = 0; b < nblk; ++b) P += colsum[static_cast<size_t>(b) * N + tid];
    P /= T;
    creq = C_req[tid];
    ckeep = C_keep[tid];
    P_out[tid] = static_cast<float>(P);
  }
  const double f = creq / KT;
  const double lbl = N * sf_sum(act ? f * P : 0.0, red);
  const double sreq = sf_sum(creq, red), skeep = sf_sum(ckeep, red);
  const double mreq = sf_max(act ? creq : 0.0, red), mkeep = sf_max(act ? ckeep : 0.0, red);
  const double never = sf_sum(act && creq == 0.0 ? 1.0 : 0.0, red);
  auto plogp = [](double x, double tot) { return x > 0.0 ? (x / tot) * log(x / tot) : 0.0; };
  const double hreq = sreq > 0 ? -sf_sum(act ? plogp(creq, sreq) : 0.0, red) : 0.0;
  const double hkeep = skeep > 0 ? -sf_sum(act ? plogp(ckeep, skeep) : 0.0, red) : 0.0;
  const double mean_req = sreq / N, mean_keep = skeep / N;
  const double vreq = sf_sum(act ? (creq - mean_req) * (creq - mean_req) : 0.0, red) / N;
  const double vkeep = sf_sum(act ? (ckeep - mean_keep) * (ckeep - mean_keep) : 0.0, red) / N;
  // destination totals R_q (thread q < N / group sums its group's experts in order)
  s_req[tid] = creq;
  s_keep[tid] = ckeep;
  __syncthreads();
  const int M = group > 0 ? N / group : 0;
  double rreq = 0.0, rkeep = 0.0;
  if (tid < M)
    for (int j = tid * group; j < (tid + 1) * group; ++j) {
      rreq += s_req[j];
      rkeep += s_keep[j];
    }
  const double mrreq = sf_max(rreq, red), mrkeep = sf_max(rkeep, red);
  // drop partials, in workgroup order
  double d[4] = {0.0, 0.0, 0.0, 0.0};
  if (tid < 4)
    for (int b = 0; b < nblk; ++b) d[tid] += drops[b * 4 + tid];
  red[tid] = tid < 4 ? d[tid] : 0.0;
  __syncthreads();
  if (tid == 0) {
    const double nan = __builtin_nan("");
    const double logn = log(static_cast<double>(N));
    stats[MOE_STAT_LBL] = static_cast<float>(lbl);
    stats[MOE_STAT_IMAX_REQ] = static_cast<float>(sreq > 0 ? N * mreq / sreq : nan);
    stats[MOE_STAT_IMAX_KEEP] = static_cast<float>(skeep > 0 ? N * mkeep / skeep : nan);
    // one expert: log N = 0, the load is balanced by construction and the deficit is 0
    stats[MOE_STAT_IH_REQ] = static_cast<float>(sreq > 0 ? (N > 1 ? 1.0 - hreq / logn : 0.0) : nan);
    stats[MOE_STAT_IH_KEEP] = static_cast<float>(skeep > 0 ? (N > 1 ? 1.0 - hkeep / logn : 0.0) : nan);
    stats[MOE_STAT_CV_REQ] = static_cast<float>(mean_req > 0 ? sqrt(vreq) / mean_req : nan);
    stats[MOE_STAT_CV_KEEP] = static_cast<float>(mean_keep > 0 ? sqrt(vkeep) / mean_keep : nan);
    stats[MOE_STAT_NEVER_SELECTED] = static_cast<float>(never);
    stats[MOE_STAT_DELTA_ROUTE] = static_cast<float>((KT - skeep) / KT);
    stats[MOE_STAT_TOKENS_LOST_ANY] = static_cast<float>(red[0]);
    stats[MOE_STAT_TOKENS_LOST_ALL] = static_cast<float>(red[1]);
    stats[MOE_STAT_WEIGHT_REMOVED] = static_cast<float>(red[3] > 0 ? red[2] / red[3] : nan);
    // destination totals sum to the expert totals
    stats[MOE_STAT_IMAX_RANK_REQ] = static_cast<float>(M > 0 && sreq > 0 ? M * mrreq / sreq : nan);
    stats[MOE_STAT_IMAX_RANK_KEEP] = static_cast<float>(M > 0 && skeep > 0 ? M * mrkeep / skeep : nan);
  }
}

}  // namespace

size_t stats_workspace_bytes(int T, int N) {
  const size_t nblk = (static_cast<size_t>(T) + ST_TPB - 1) / ST_TPB;
  return nblk * (static_cast<size_t>(N) + 4) * sizeof(float);
}

hipError_t launch_balance_stats(int T, int N, int K, int score, int group, const float* logits,
                                const int32_t* dest_row, const float* topk_r,
                                const int32_t* C_req, const int32_t* C_keep, float* P,
                                float* stats, void* workspace, hipStream_t stream) {
  const int nblk = (T + ST_TPB - 1) / ST_TPB;
  float* colsum = static_cast<float*>(workspace);
  float* drops = colsum + static_cast<size_t>(nblk) * N;
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(ST_WAVES * kWave), 0, stream, T, N,
                     K, score, logits, dest_row, topk_r, colsum, drops);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(SF_THREADS), 0, stream, T, N, K, group,
                     nblk, colsum, drops, C_req, C_keep, P, stats);
  return hipGetLastError();
}
