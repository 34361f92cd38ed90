// Requested counts, capacity admission, offsets and the packed row copy.
//
// Follows "Section 10: Routing, Capacity, and Load Balancing": requested counts
// (Eq. 19), kept counts M_i and drops (Eq. 21), and the real-count offsets
// o_j = sum_{i<=j} M_i of the densely packed expert segments (Eq. 26). Two capacity
// policies: the independent per-expert limit (Eq. 25), admitting routes first come by
// token index, and the rank-wide budget of Eq. 23 / Section 10.3, shared by each group
// of `group` consecutive experts (a destination). The rank-wide admission order is
// local-expert-major, then source rank, with a prefix of each split kept; the batch's
// sources are contiguous token shards in rank order, so that order is (expert, token)
// and expert e keeps M_e = clamp(B - sum_{e' < e in its group} C_e'^req, 0, C_e^req):
// either way the kept routes of an expert are its first M_e routes in token order.
//
// Deterministic by construction: no atomic decides a position. A histogram row holds
// the per-expert route counts of R consecutive tokens (R = 64 from count_kernel, or the
// router's own 16- or 32-token tile when the router counts in its epilogue), and each
// route's rank among its row's routes to the same expert.
//   count   one wave per 64-token chunk: each expert's 64-bit token mask is built with
//           LDS OR (order-free), so a route's rank inside the chunk is a popcount of
//           the mask below its lane and the chunk histogram is the mask's popcount.
//   place   one launch: every 1024-thread workgroup re-reduces the whole histogram
//           (per-expert totals C^req, and the prefix before its own rows), applies the
//           capacity policy and the exclusive scan over experts itself, then writes the
//           restoration map of its 64 tokens (and copies their rows when asked). Used
//           while the histogram is small enough to re-read per workgroup (<= 64 Ki
//           entries), so no grid-wide wait is needed.
//   scan    otherwise, one workgroup: per-expert running sums over rows, split over up to
//           1024 threads (row base ranks and C^req), C^keep from the capacity policy, and
//           an exclusive scan over experts -> offsets; then
//   scatter one wave per token: rank = row base + rank in row; kept iff rank < C^keep;
//           the token's row is read once (16-byte lanes, coalesced) and written to each
//           kept destination (map: the same without the copy, one thread per route).
#include "common.h"

using namespace moe;

namespace {

constexpr int CNT_WAVES = 4;

__global__ void __launch_bounds__(CNT_WAVES * kWave)
count_kernel(int T, int N, int K, const int32_t* __restrict__ topk_idx,
             int32_t* __restrict__ hist, int32_t* __restrict__ loc_rank) {
  extern __shared__ unsigned long long masks[];  // [CNT_WAVES][N]
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int chunk = blockIdx.x * CNT_WAVES + w;
  const int nchunks = (T + kChunk - 1) / kChunk;
  unsigned long long* m = masks + static_cast<size_t>(w) * N;
  for (int e = lane; e < N; e += kWave) m[e] = 0ull;
  __syncthreads();
  const int t = chunk * kChunk + lane;
  const bool valid = chunk < nchunks && t < T;
  if (valid) {
    for (int k = 0; k < K; ++k) {
      const int e = topk_idx[static_cast<size_t>(t) * K + k];
      atomicOr(&m[e], 1ull << lane);
    }
  }
  __syncthreads();
  if (valid) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int k = 0; k < K; ++k) {
      const int e = topk_idx[static_cast<size_t>(t) * K + k];
      loc_rank[static_cast<size_t>(t) * K + k] = __popcll(m[e] & below);
    }
  }
  if (chunk < nchunks)
    for (int e = lane; e < N; e += kWave)
      hist[static_cast<size_t>(chunk) * N + e] = __popcll(m[e]);
}

constexpr int SCAN_THREADS = 1024;

// Single workgroup. hist[c][e] (chunk counts) is overwritten with the exclusive
// running sum over chunks, i.e. the rank of chunk c's first route to expert e.
// Thread t owns expert e = t % NP and the p-th contiguous run of chunks, p = t / NP
// (NP = N rounded up to a power of two): its loads are independent and coalesced
// across the experts; a scan over the P runs of each expert then gives the bases.
__global__ void __launch_bounds__(SCAN_THREADS)
scan_kernel(int nchunks, int N, int NP, int capacity, int group, int32_t* __restrict__ hist,
            int32_t* __restrict__ C_req, int32_t* __restrict__ C_keep,
            int32_t* __restrict__ offsets, int32_t* __restrict__ count_accum) {
  __shared__ int32_t part[SCAN_THREADS];
  __shared__ int32_t req[kMaxN];
  __shared__ int32_t keep[kMaxN];
  const int tid = threadIdx.x;
  const int P = SCAN_THREADS / NP;
  const int e = tid % NP, p = tid / NP;
  const int per = (nchunks + P - 1) / P;
  const int c0 = min(p * per, nchunks), c1 = min(c0 + per, nchunks);
  int local = 0;
  if (e < N) {
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = hist[static_cast<size_t>(c + u) * N + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) local += h[u];
    }
    for (; c < c1; ++c) local += hist[static_cast<size_t>(c) * N + e];
  }
  part[tid] = local;
  __syncthreads();
  // exclusive prefix over the runs p' < p of the same expert (P <= 256, serial is fine
  // for the few runs; done by each thread over its own expert's column of part[])
  int base = 0;
  for (int q = 0; q < p; ++q) base += part[q * NP + e];
  if (e < N) {
    int run = base;
    int c = c0;
    for (; c + 8 <= c1; c += 8) {  // batches of independent loads, then the stores
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = hist[static_cast<size_t>(c + u) * N + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        hist[static_cast<size_t>(c + u) * N + e] = run;
        run += h[u];
      }
    }
    for (; c < c1; ++c) {
      const size_t o = static_cast<size_t>(c) * N + e;
      const int h = hist[o];
      hist[o] = run;
      run += h;
    }
    if (p == P - 1) {
      C_req[e] = run;
      req[e] = run;
      if (count_accum != nullptr) count_accum[e] += run;
    }
  }
  __syncthreads();
  // kept counts (thread tid owns expert tid)
  if (tid < N) {
    const int r = req[tid];
    int kk = r;
    if (capacity >= 0) {
      if (group > 0) {  // shared destination budget, earlier local experts first
        int before = 0;
        for (int q = tid - tid % group; q < tid; ++q) before += req[q];
        kk = min(r, max(capacity - before, 0));
      } else {
        kk = min(r, capacity);
      }
    }
    C_keep[tid] = kk;
    keep[tid] = kk;
  }
  __syncthreads();
  // exclusive scan of C_keep over experts (N <= 256): Hillis-Steele in part[0..N)
  if (tid < kMaxN) part[tid] = (tid < N) ? keep[tid] : 0;
  __syncthreads();
  for (int off = 1; off < kMaxN; off <<= 1) {
    const int v = (tid < kMaxN && tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    if (tid < kMaxN) part[tid] += v;
    __syncthreads();
  }
  if (tid < N) offsets[tid] = part[tid] - keep[tid];
  if (tid == 0) offsets[N] = part[kMaxN - 1];
}

constexpr int SC_WAVES = 4;

template <int EB>  // bytes per element
__global__ void __launch_bounds__(SC_WAVES * kWave)
scatter_kernel(int T, int d, int N, int K, int R, const void* __restrict__ x,
               const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ base,
               const int32_t* __restrict__ loc_rank, const int32_t* __restrict__ C_keep,
               const int32_t* __restrict__ offsets, int32_t* __restrict__ dest_row,
               int32_t* __restrict__ row_token, void* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * SC_WAVES + (threadIdx.x >> 6);
  if (t >= T) return;
  int dest = -1;
  if (lane < K) {
    const size_t tk = static_cast<size_t>(t) * K + lane;
    const int e = topk_idx[tk];
    const int rank = base[static_cast<size_t>(t / R) * N + e] + loc_rank[tk];
    if (rank < C_keep[e]) dest = offsets[e] + rank;
    dest_row[tk] = dest;
    if (dest >= 0) row_token[dest] = t;
  }
  const int n16 = d * EB / 16;  // 16-byte pieces per row
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(x) +
                                                    static_cast<size_t>(t) * d * EB);
  char* dst0 = static_cast<char*>(x_perm);
  for (int j0 = 0; j0 < n16; j0 += 4 * kWave) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kWave + lane;
      if (j < n16) v[u] = src[j];
    }
    for (int k = 0; k < K; ++k) {
      const int dk = __shfl(dest, k, kWave);
      if (dk < 0) continue;
      u32x4* dst = reinterpret_cast<u32x4*>(dst0 + static_cast<size_t>(dk) * d * EB);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * kWave + lane;
        if (j < n16) dst[j] = v[u];
      }
    }
  }
}

// restoration map only (no row copy): one thread per (token, slot)
__global__ void __launch_bounds__(256)
map_kernel(int T, int N, int K, int R, const int32_t* __restrict__ topk_idx,
           const int32_t* __restrict__ base, const int32_t* __restrict__ loc_rank,
           const int32_t* __restrict__ C_keep, const int32_t* __restrict__ offsets,
           int32_t* __restrict__ dest_row, int32_t* __restrict__ row_token) {
  const size_t tk = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tk >= static_cast<size_t>(T) * K) return;
  const int t = static_cast<int>(tk / K);
  const int e = topk_idx[tk];
  const int rank = base[static_cast<size_t>(t / R) * N + e] + loc_rank[tk];
  int dest = -1;
  if (rank < C_keep[e]) dest = offsets[e] + rank;
  dest_row[tk] = dest;
  if (dest >= 0) row_token[dest] = t;
}

// ---- place: capacity, offsets and restoration map in one launch ----------------------
constexpr int PL_THREADS = 1024;
constexpr int PL_TOK = 64;                // tokens placed per workgroup
constexpr int PL_MAXP = 32;               // row runs per expert (reduced by one thread)
constexpr int PL_ROWS = PL_TOK / 16;      // histogram rows per workgroup (rows of >= 16)
constexpr int PL_PART = 4096;             // partial sums: runs x experts
static_assert(PL_TOK * kMaxK <= PL_THREADS, "one route per thread");
constexpr int kPlaceMaxHist = 64 * 1024;  // histogram entries each workgroup re-reads

template <int V>
struct IntV;
template <>
struct IntV<1> {
  typedef int type;
  static __device__ __forceinline__ int at(const int& v, int) { return v; }
};
template <>
struct IntV<4> {
  typedef int __attribute__((ext_vector_type(4))) type;
  static __device__ __forceinline__ int at(const type& v, int i) { return v[i]; }
};

// V experts per load (4 when N % 4 == 0); EB bytes per element of x, 0: no row copy.
// Run p of expert group g covers histogram rows [p per, (p + 1) per); the sums over the
// runs are taken in run order, so every workgroup derives the same C^req, C^keep and
// offsets (workgroup 0 writes them).
template <int V, int EB>
__global__ void __launch_bounds__(PL_THREADS)
place_kernel(int T, int d, int N, int K, int R, int nrows, int capacity, int group,
             const int32_t* __restrict__ hist, const int32_t* __restrict__ topk_idx,
             const int32_t* __restrict__ loc_rank, int32_t* __restrict__ C_req,
             int32_t* __restrict__ C_keep, int32_t* __restrict__ offsets,
             int32_t* __restrict__ count_accum, int32_t* __restrict__ dest_row,
             int32_t* __restrict__ row_token, const void* __restrict__ x,
             void* __restrict__ x_perm) {
  typedef typename IntV<V>::type vec;
  __shared__ int32_t s_tot[PL_PART];
  __shared__ int32_t s_pre[PL_PART];
  __shared__ int32_t s_base[PL_ROWS][kMaxN];
  __shared__ int32_t s_req[kMaxN];
  __shared__ int32_t s_keep[kMaxN];
  __shared__ int32_t s_scan[kMaxN];
  __shared__ int32_t s_dest[EB > 0 ? PL_TOK * kMaxK : 1];
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.x * PL_TOK;
  const int ntok = min(PL_TOK, T - tok0);
  const int r0 = tok0 / R;             // PL_TOK is a multiple of R
  const int nr = (ntok + R - 1) / R;   // this workgroup's rows
  const int G = (N + V - 1) / V;
  const int P = min(PL_THREADS / G, PL_MAXP);
  const int g = tid % G, p = tid / G;
  // this thread's route (64 tokens x K <= 1024 threads: one each) and this workgroup's
  // own rows of expert tid, loaded up front beside the runs' loads
  const bool has_route = tid < ntok * K;
  const size_t tk = static_cast<size_t>(tok0) * K + tid;
  const int my_e = has_route ? topk_idx[tk] : 0;
  const int my_rank = has_route ? loc_rank[tk] : 0;
  int own[PL_ROWS];
#pragma unroll
  for (int ri = 0; ri < PL_ROWS; ++ri)
    own[ri] = (tid < N && ri < nr) ? hist[static_cast<size_t>(r0 + ri) * N + tid] : 0;
  // 1. each run: sums over all its rows and over its rows before r0
  if (p < P) {
    const int per = (nrows + P - 1) / P;
    const int c0 = min(p * per, nrows), c1 = min(c0 + per, nrows);
    int tot[V], pre[V];
#pragma unroll
    for (int v = 0; v < V; ++v) tot[v] = pre[v] = 0;
    const int32_t* hg = hist + g * V;
    int c = c0;
    for (; c + 8 <= c1; c += 8) {  // batches of independent loads
      vec h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = *reinterpret_cast<const vec*>(hg + static_cast<size_t>(c + u) * N);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int hv = IntV<V>::at(h[u], v);
          tot[v] += hv;
          pre[v] += (c + u < r0) ? hv : 0;
        }
    }
    for (; c < c1; ++c) {
      const vec h = *reinterpret_cast<const vec*>(hg + static_cast<size_t>(c) * N);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        tot[v] += IntV<V>::at(h, v);
        pre[v] += (c < r0) ? IntV<V>::at(h, v) : 0;
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      s_tot[p * N + g * V + v] = tot[v];
      s_pre[p * N + g * V + v] = pre[v];
    }
  }
  __syncthreads();
  // 2. per expert: C^req, and the base rank of each of this workgroup's rows
  if (tid < N) {
    int tt = 0, pp = 0;
    for (int q = 0; q < P; ++q) {
      tt += s_tot[q * N + tid];
      pp += s_pre[q * N + tid];
    }
    s_req[tid] = tt;
    int b = pp;
#pragma unroll
    for (int ri = 0; ri < PL_ROWS; ++ri) {
      s_base[ri][tid] = b;
      b += own[ri];
    }
  }
  __syncthreads();
  // 3. kept counts (thread tid owns expert tid), then their exclusive scan
  int req = 0, kk = 0;
  if (tid < N) {
    req = s_req[tid];
    kk = req;
    if (capacity >= 0) {
      if (group > 0) {  // shared destination budget, earlier local experts first
        int before = 0;
        for (int q = tid - tid % group; q < tid; ++q) before += s_req[q];
        kk = min(req, max(capacity - before, 0));
      } else {
        kk = min(req, capacity);
      }
    }
    s_keep[tid] = kk;
  }
  // inclusive scan of the kept counts over experts: within each of the first four waves
  // by shuffles, then each wave adds the totals of the waves before it
  __shared__ int32_t s_wsum[kMaxN / kWave];
  int inc = kk;  // zero past N
  if (tid < kMaxN) {
    const int lane = tid & 63;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += v;
    }
    if (lane == kWave - 1) s_wsum[tid >> 6] = inc;
  }
  __syncthreads();
  if (tid < kMaxN) {
    for (int q = 0; q < (tid >> 6); ++q) inc += s_wsum[q];
    s_scan[tid] = inc;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < N) {
      C_req[tid] = req;
      C_keep[tid] = kk;
      offsets[tid] = s_scan[tid] - kk;
      if (count_accum != nullptr) count_accum[tid] += req;
    }
    if (tid == 0) offsets[N] = s_scan[kMaxN - 1];
  }
  // 4. restoration map of this workgroup's routes
  if (has_route) {
    const int t = tok0 + tid / K;
    const int rank = s_base[t / R - r0][my_e] + my_rank;
    int dest = -1;
    if (rank < s_keep[my_e]) dest = s_scan[my_e] - s_keep[my_e] + rank;
    dest_row[tk] = dest;
    if (dest >= 0) row_token[dest] = t;
    if constexpr (EB > 0) s_dest[tid] = dest;
  }
  // 5. row copy: wave w copies tokens w, w + 16, ... to their kept destinations
  if constexpr (EB > 0) {
    __syncthreads();
    const int lane = tid & 63, w = tid >> 6;
    const int n16 = d * EB / 16;
    char* dst0 = static_cast<char*>(x_perm);
    for (int tl = w; tl < ntok; tl += PL_THREADS / kWave) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(x) +
                                                        static_cast<size_t>(tok0 + tl) * d * EB);
      for (int j0 = 0; j0 < n16; j0 += 4 * kWave) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = j0 + u * kWave + lane;
          if (j < n16) v[u] = src[j];
        }
        for (int k = 0; k < K; ++k) {
          const int dk = s_dest[tl * K + k];
          if (dk < 0) continue;
          u32x4* dst = reinterpret_cast<u32x4*>(dst0 + static_cast<size_t>(dk) * d * EB);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = j0 + u * kWave + lane;
            if (j < n16) dst[j] = v[u];
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_count(int T, int N, int K, const int32_t* topk_idx, int32_t* hist,
                        int32_t* loc_rank, hipStream_t stream) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int grid = (nchunks + CNT_WAVES - 1) / CNT_WAVES;
  const size_t shm = sizeof(unsigned long long) * CNT_WAVES * N;
  hipLaunchKernelGGL(count_kernel, dim3(grid), dim3(CNT_WAVES * kWave), shm, stream, T, N, K,
                     topk_idx, hist, loc_rank);
  return hipGetLastError();
}

hipError_t launch_scan(int nrows, int N, int capacity, int group, int32_t* hist,
                       int32_t* C_req, int32_t* C_keep, int32_t* offsets, int32_t* count_accum,
                       hipStream_t stream) {
  int NP = 1;
  while (NP < N) NP <<= 1;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, stream, nrows, N, NP,
                     capacity, group, hist, C_req, C_keep, offsets, count_accum);
  return hipGetLastError();
}

hipError_t launch_scatter(int T, int d_model, int N, int K, int R, int dt, const void* x,
                          const int32_t* topk_idx, const int32_t* hist_base,
                          const int32_t* loc_rank, const int32_t* C_keep,
                          const int32_t* offsets, int32_t* dest_row, int32_t* row_token,
                          void* x_perm, hipStream_t stream) {
  if (x_perm == nullptr) {
    const size_t n = static_cast<size_t>(T) * K;
    hipLaunchKernelGGL(map_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       stream, T, N, K, R, topk_idx, hist_base, loc_rank, C_keep, offsets,
                       dest_row, row_token);
    return hipGetLastError();
  }
  const int grid = (T + SC_WAVES - 1) / SC_WAVES;
  if (dt == 1)
    hipLaunchKernelGGL(scatter_kernel<2>, dim3(grid), dim3(SC_WAVES * kWave), 0, stream, T,
                       d_model, N, K, R, x, topk_idx, hist_base, loc_rank, C_keep, offsets,
                       dest_row, row_token, x_perm);
  else
    hipLaunchKernelGGL(scatter_kernel<4>, dim3(grid), dim3(SC_WAVES * kWave), 0, stream, T,
                       d_model, N, K, R, x, topk_idx, hist_base, loc_rank, C_keep, offsets,
                       dest_row, row_token, x_perm);
  return hipGetLastError();
}

bool place_fused(int T, int N, int R) {
  return static_cast<size_t>((T + R - 1) / R) * N <= static_cast<size_t>(kPlaceMaxHist);
}

hipError_t launch_place(int T, int d_model, int N, int K, int R, int capacity, int group,
                        int dt, const void* x, const int32_t* topk_idx, int32_t* hist,
                        const int32_t* loc_rank, int32_t* C_req, int32_t* C_keep,
                        int32_t* offsets, int32_t* count_accum, int32_t* dest_row,
                        int32_t* row_token, void* x_perm, hipStream_t stream) {
  if (R < 16 || PL_TOK % R != 0) return hipErrorInvalidValue;
  const int nrows = (T + R - 1) / R;
  if (!place_fused(T, N, R)) {  // one scan workgroup, then the map / row copy
    hipError_t e = launch_scan(nrows, N, capacity, group, hist, C_req, C_keep, offsets,
                               count_accum, stream);
    if (e != hipSuccess) return e;
    return launch_scatter(T, d_model, N, K, R, dt, x, topk_idx, hist, loc_rank, C_keep, offsets,
                          dest_row, row_token, x_perm, stream);
  }
  const dim3 grid((T + PL_TOK - 1) / PL_TOK), block(PL_THREADS);
#define MOE_PLACE(V_, EB_)                                                                   \
  hipLaunchKernelGGL((place_kernel<V_, EB_>), grid, block, 0, stream, T, d_model, N, K, R,     \
                     nrows, capacity, group, hist, topk_idx, loc_rank, C_req, C_keep, offsets, \
                     count_accum, dest_row, row_token, x, x_perm)
  const int eb = x_perm == nullptr ? 0 : (dt == 1 ? 2 : 4);
  // four experts per 16-byte load where the rows stay 16-byte aligned
  if (N % 4 == 0 && (reinterpret_cast<uintptr_t>(hist) & 15u) == 0) {
    if (eb == 0) MOE_PLACE(4, 0);
    else if (eb == 2) MOE_PLACE(4, 2);
    else MOE_PLACE(4, 4);
  } else {
    if (eb == 0) MOE_PLACE(1, 0);
    else if (eb == 2) MOE_PLACE(1, 2);
    else MOE_PLACE(1, 4);
  }
#undef MOE_PLACE
  return hipGetLastError();
}
