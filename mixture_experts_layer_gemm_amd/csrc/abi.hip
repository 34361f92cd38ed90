// C ABI of the MoE layer library: argument validation, workspace carving and the
// per-stage launch sequence. Declarations and the contract of every entry point are in
// include/moe.h. Nothing here allocates device memory or synchronizes the stream.
#include <climits>
#include <cmath>
#include <cstddef>
#include <mutex>

#include "../../include/moe.h"
#include "common.h"
#include "gemm_stream.h"

namespace {

constexpr size_t kAlign = 256;

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

int nchunks_of(int T) { return (T + moe::kChunk - 1) / moe::kChunk; }
int rows_of(int T, int R) { return (T + R - 1) / R; }

int check_router_dims(int T, int d_model, int N, int K) {
  if (T < 0 || d_model <= 0 || N <= 0 || K <= 0 || K > N) return MOE_ERR_INVALID_ARG;
  if (K > moe::kMaxK || N > moe::kMaxN || d_model % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// experts per destination group: 0 = none, else a divisor of N (every destination owns
// the same number of experts)
int check_group(int N, int group) {
  if (group < 0 || (group > 0 && N % group != 0)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_dtype(int dt) { return (dt == MOE_F32 || dt == MOE_BF16) ? MOE_OK : MOE_ERR_INVALID_ARG; }

size_t esize(int dt) { return dt == MOE_BF16 ? 2 : 4; }

#define MOE_TRY(expr)                        \
  do {                                       \
    const int st_ = (expr);                  \
    if (st_ != MOE_OK) return st_;           \
  } while (0)
#define MOE_HIP(expr)                                  \
  do {                                                 \
    if ((expr) != hipSuccess) return MOE_ERR_HIP;      \
  } while (0)

// Workspace layout shared by moe_route and moe_permute: chunk histograms and
// in-chunk ranks, then (route only) scratch for C_keep/offsets and the split-K logit
// slices of routers with many experts.
struct CountWs {
  int32_t* hist;
  int32_t* loc_rank;
  int32_t* c_keep;
  int32_t* offsets;
  void* route_scratch;  // split-K logits of many experts (moe_route only)
};

// d_model < 0: no route scratch (moe_permute, histogram rows of kChunk tokens); else the
// router counts in its epilogue, in rows of 16 or 32 tokens (sized for 16)
size_t carve_count(void* ws, int T, int d_model, int N, int K, CountWs* out) {
  Carver c(ws);
  CountWs w;
  const bool route = d_model >= 0;
  w.hist = c.take<int32_t>(static_cast<size_t>(route ? rows_of(T, 16) : nchunks_of(T)) * N);
  w.loc_rank = c.take<int32_t>(static_cast<size_t>(T) * K);
  w.c_keep = route ? c.take<int32_t>(N) : nullptr;
  w.offsets = route ? c.take<int32_t>(N + 1) : nullptr;
  const size_t rb = route ? route_scratch_bytes(T, d_model, N) : 0;
  w.route_scratch = rb ? static_cast<void*>(c.take<char>(rb)) : nullptr;
  if (out) *out = w;
  return c.off;
}

struct FwdWs {
  float* topk_r;
  int32_t* topk_idx;
  float* s_tok;
  int32_t *hist, *loc_rank, *C_req, *C_keep, *offsets, *dest_row, *row_token;
  void *x_perm, *h_perm, *f_perm, *g, *h_shared;
  float* logits;     // needed by the balance statistics
  void* stats_ws;
  void* route_scratch;  // split-K logits of routers with many experts
};

size_t carve_forward(const moe_forward_args* a, void* ws, FwdWs* out) {
  Carver c(ws);
  FwdWs w;
  const size_t T = a->T, K = a->K, N = a->N, d = a->d_model;
  const size_t rows =
      static_cast<size_t>(moe_max_rows(a->T, a->N, a->K, a->capacity, a->capacity_group));
  const size_t es = esize(a->dt);
  const bool gate = a->w_shared_gate != nullptr;
  w.topk_idx = a->topk_idx ? a->topk_idx : c.take<int32_t>(T * K);
  w.topk_r = a->topk_r ? a->topk_r : c.take<float>(T * K);
  w.s_tok = !gate ? nullptr : (a->s_tok ? a->s_tok : c.take<float>(T));
  w.hist = c.take<int32_t>(static_cast<size_t>(rows_of(a->T, 16)) * N);  // router rows
  w.loc_rank = c.take<int32_t>(T * K);
  w.C_req = a->C_req ? a->C_req : c.take<int32_t>(N);
  w.C_keep = a->C_keep ? a->C_keep : c.take<int32_t>(N);
  w.offsets = a->offsets ? a->offsets : c.take<int32_t>(N + 1);
  w.dest_row = a->dest_row ? a->dest_row : c.take<int32_t>(T * K);
  w.row_token = a->row_token ? a->row_token : c.take<int32_t>(rows);
  w.x_perm = a->x_perm;  // the gate/up pass gathers rows of x; a copy only on request
  w.h_perm = a->h_perm ? a->h_perm : static_cast<void*>(c.take<char>(rows * a->d_r * es));
  w.f_perm = a->f_perm ? a->f_perm : static_cast<void*>(c.take<char>(rows * d * es));
  if (a->d_s > 0) {
    w.g = a->g ? a->g : static_cast<void*>(c.take<char>(T * d * es));
    w.h_shared = c.take<char>(T * static_cast<size_t>(a->d_s) * es);
  } else {
    w.g = nullptr;
    w.h_shared = nullptr;
  }
  const bool stats = a->balance_P != nullptr && a->balance_stats != nullptr;
  w.logits = a->logits ? a->logits : (stats ? c.take<float>(T * N) : nullptr);
  w.stats_ws = stats ? static_cast<void*>(c.take<char>(stats_workspace_bytes(a->T, a->N))) : nullptr;
  const size_t rb = route_split_slices(a->N, a->d_model, a->dt, 0, a->w_shared_gate != nullptr) > 0
                        ? route_scratch_bytes(a->T, a->d_model, a->N) : 0;
  w.route_scratch = rb ? static_cast<void*>(c.take<char>(rb)) : nullptr;
  if (out) *out = w;
  return c.off;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or option";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int moe_capacity_from_factor(double c, int K, int T, int N) {
  if (c < 0.0 || N <= 0) return -1;
  const double v = std::ceil(c * K * T / N);
  return v >= static_cast<double>(INT_MAX) ? INT_MAX : static_cast<int>(v);
}

int moe_rank_capacity_from_factor(double c, int K, int T_s) {
  if (c < 0.0) return -1;
  const double v = std::ceil(c * K * T_s);
  if (v < 1.0) return 1;
  return v >= static_cast<double>(INT_MAX) ? INT_MAX : static_cast<int>(v);
}

int moe_max_rows(int T, int N, int K, int capacity, int capacity_group) {
  const long kt = static_cast<long>(K) * (T > 0 ? T : 0);
  long r = kt;
  if (capacity >= 0) {
    const long budgets = capacity_group > 0 ? N / capacity_group : N;
    const long nc = budgets * capacity;
    r = nc < kt ? nc : kt;
  }
  return r > INT_MAX ? INT_MAX : static_cast<int>(r);
}

size_t moe_route_workspace_size(int T, int d_model, int N, int K) {
  if (T <= 0 || d_model <= 0 || N <= 0 || K <= 0) return 0;
  return carve_count(nullptr, T, d_model, N, K, nullptr);
}

int moe_route(int T, int d_model, int N, int K, int score, int renorm, float alpha, int dt,
              const void* x, const void* w_router, const float* logit_bias,
              const float* expert_bias, const void* w_shared_gate, float* logits,
              int logits_mode, int32_t* topk_idx, float* topk_r, float* s_tok, int32_t* C_req,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_router_dims(T, d_model, N, K));
  MOE_TRY(check_dtype(dt));
  if (score < MOE_SCORE_SOFTMAX || score > MOE_SCORE_SOFTMAX_SELECTED) return MOE_ERR_INVALID_ARG;
  if (logits_mode != 0 && logits_mode != 1) return MOE_ERR_INVALID_ARG;
  if (!topk_idx || !topk_r) return MOE_ERR_INVALID_ARG;
  if (logits_mode == 0 && (!x || !w_router)) return MOE_ERR_INVALID_ARG;
  if (logits_mode == 1 && (!logits || s_tok)) return MOE_ERR_INVALID_ARG;
  if (logits_mode == 0 && ((w_shared_gate != nullptr) != (s_tok != nullptr)))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  CountWs w{};
  const bool split =
      route_split_slices(N, d_model, dt, logits_mode, logits_mode == 0 && w_shared_gate) > 0;
  if (C_req || split) {
    if (!workspace || workspace_bytes < moe_route_workspace_size(T, d_model, N, K))
      return MOE_ERR_WORKSPACE;
    carve_count(workspace, T, d_model, N, K, &w);
  }
  const void* gate = logits_mode == 0 ? w_shared_gate : nullptr;
  MOE_HIP(launch_route(T, d_model, N, K, score, renorm, alpha, dt, x, w_router, logit_bias,
                       expert_bias, gate, logits, logits_mode, topk_idx, topk_r, s_tok,
                       w.route_scratch, C_req ? w.hist : nullptr, C_req ? w.loc_rank : nullptr,
                       stream));
  if (C_req) {  // the router counted its tiles; the per-expert sums of those rows
    const int R = route_tile_tokens(N, d_model, dt, logits_mode, gate != nullptr);
    MOE_HIP(launch_scan(rows_of(T, R), N, -1, 0, w.hist, C_req, w.c_keep, w.offsets, nullptr,
                        stream));
  }
  return MOE_OK;
}

size_t moe_permute_workspace_size(int T, int N, int K) {
  if (T <= 0 || N <= 0 || K <= 0) return 0;
  return carve_count(nullptr, T, -1, N, K, nullptr);
}

int moe_permute(int T, int d_model, int N, int K, int capacity, int capacity_group, int dt,
                const void* x, const int32_t* topk_idx, int32_t* C_req, int32_t* C_keep,
                int32_t* offsets, int32_t* dest_row, int32_t* row_token, void* x_perm,
                int max_rows, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_router_dims(T, d_model, N, K));
  MOE_TRY(check_dtype(dt));
  MOE_TRY(check_group(N, capacity_group));
  if (!x || !topk_idx || !C_req || !C_keep || !offsets || !dest_row || !row_token)
    return MOE_ERR_INVALID_ARG;
  if (max_rows < moe_max_rows(T, N, K, capacity, capacity_group)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!workspace || workspace_bytes < moe_permute_workspace_size(T, N, K)) return MOE_ERR_WORKSPACE;
  CountWs w{};
  carve_count(workspace, T, -1, N, K, &w);
  MOE_HIP(launch_count(T, N, K, topk_idx, w.hist, w.loc_rank, stream));
  MOE_HIP(launch_place(T, d_model, N, K, moe::kChunk, capacity, capacity_group, dt, x, topk_idx,
                       w.hist, w.loc_rank, C_req, C_keep, offsets, nullptr, dest_row, row_token,
                       x_perm, stream));
  return MOE_OK;
}

// ---- allocation-free permute: scratch in a fixed device array ----------------------
// Each device the library runs on holds its own copy of `scratch` (one code object per
// device). Host code never passes the array's name to a kernel (on the host that name is
// a stand-in, not a device address): the device address of each copy is looked up once,
// with that device current, and kept per device.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// device address of the current device's scratch array, or nullptr
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

int moe_permute_noalloc(int T, int d_model, int N, int K, int capacity, int capacity_group,
                        int dt, const void* x, const int32_t* topk_idx, int32_t* C_req,
                        int32_t* C_keep, int32_t* offsets, int32_t* dest_row,
                        int32_t* row_token, void* x_perm, int max_rows, hipStream_t stream) {
  MOE_TRY(check_router_dims(T, d_model, N, K));
  MOE_TRY(check_dtype(dt));
  MOE_TRY(check_group(N, capacity_group));
  if (!x || !topk_idx || !C_req || !C_keep || !offsets || !dest_row || !row_token)
    return MOE_ERR_INVALID_ARG;
  if (max_rows < moe_max_rows(T, N, K, capacity, capacity_group)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (moe_permute_workspace_size(T, N, K) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (ws == nullptr) return MOE_ERR_HIP;
  CountWs w{};
  carve_count(ws, T, -1, N, K, &w);
  MOE_HIP(launch_count(T, N, K, topk_idx, w.hist, w.loc_rank, stream));
  MOE_HIP(launch_place(T, d_model, N, K, moe::kChunk, capacity, capacity_group, dt, x, topk_idx,
                       w.hist, w.loc_rank, C_req, C_keep, offsets, nullptr, dest_row, row_token,
                       x_perm, stream));
  return MOE_OK;
}

static StreamProblem problem(const void* a, int a_rows, const int32_t* row_index,
                             const int32_t* offsets, int G, int rows, int Kd, int Nd,
                             const void* w0, const void* w1, void* out) {
  StreamProblem p;
  p.a = static_cast<const uint16_t*>(a);
  p.row_index = row_index;
  p.offsets = offsets;
  p.G = G;
  p.rows = rows;
  p.a_rows = row_index != nullptr ? a_rows : rows;
  p.Kd = Kd;
  p.Nd = Nd;
  p.w0 = static_cast<const uint16_t*>(w0);
  p.w1 = static_cast<const uint16_t*>(w1);
  p.out = static_cast<uint16_t*>(out);
  p.dh = nullptr;
  p.dab = nullptr;
  return p;
}

// one grouped GEMM pass: the persistent packed-weight kernel where the shape fits it,
// else the per-tile packed kernel, or the row-major kernels for row-major weights
static hipError_t gemm_pass(bool swiglu, bool packed, int G, int Kd, int Nd, int dt,
                            const void* a, int a_rows, const int32_t* row_index,
                            const int32_t* offsets, int max_rows, const void* w0, const void* w1,
                            void* out, hipStream_t stream) {
  if (packed) {
    const StreamProblem p0 = problem(a, a_rows, row_index, offsets, G, max_rows, Kd, Nd, w0, w1, out);
    StreamProblem none{};
    if (stream_gemm_supported(swiglu, p0, none)) return launch_stream_gemm(swiglu, p0, none, stream);
    return launch_grouped_gemm_packed(swiglu, G, Kd, Nd, a, row_index, offsets, max_rows, w0, w1,
                                      out, stream);
  }
  return launch_grouped_gemm(swiglu, G, Kd, Nd, dt, a, row_index, offsets, max_rows, w0, w1, out,
                             stream);
}

// The routed experts over their segments (rows gathered from x through row_token) and
// the shared MLP over all T tokens: pass 1 = gate/up, 2 = down, 0 = both. With packed
// weights and shapes that fit, each pass is one persistent launch holding both problems.
static hipError_t expert_passes(int N, int d, int d_r, int d_s, int dt, bool pk, const void* x,
                                int T, const int32_t* row_token, const int32_t* offsets,
                                int rows, const void* w_gate, const void* w_up,
                                const void* w_down, const void* ws_gate, const void* ws_up,
                                const void* ws_down, void* h_perm, void* f_perm, void* h_shared,
                                void* g, int pass, hipStream_t stream) {
  const bool up = pass != 2, down = pass != 1;
  if (pk && rows > 0 && d_s > 0) {
    const StreamProblem gu0 = problem(x, T, row_token, offsets, N, rows, d, d_r, w_gate, w_up, h_perm);
    const StreamProblem gu1 = problem(x, T, nullptr, nullptr, 1, T, d, d_s, ws_gate, ws_up, h_shared);
    const StreamProblem dn0 = problem(h_perm, rows, nullptr, offsets, N, rows, d_r, d, w_down,
                                      nullptr, f_perm);
    const StreamProblem dn1 = problem(h_shared, T, nullptr, nullptr, 1, T, d_s, d, ws_down,
                                      nullptr, g);
    if (stream_gemm_supported(true, gu0, gu1) && stream_gemm_supported(false, dn0, dn1)) {
      if (up) {
        const hipError_t e = launch_stream_gemm(true, gu0, gu1, stream);
        if (e != hipSuccess) return e;
      }
      if (down) return launch_stream_gemm(false, dn0, dn1, stream);
      return hipSuccess;
    }
  }
  hipError_t e = hipSuccess;
  if (rows > 0) {
    if (up)
      e = gemm_pass(true, pk, N, d, d_r, dt, x, T, row_token, offsets, rows, w_gate, w_up,
                    h_perm, stream);
    if (e == hipSuccess && down)
      e = gemm_pass(false, pk, N, d_r, d, dt, h_perm, rows, nullptr, offsets, rows, w_down,
                    nullptr, f_perm, stream);
  }
  if (e == hipSuccess && d_s > 0) {
    if (up)
      e = gemm_pass(true, pk, 1, d, d_s, dt, x, T, nullptr, nullptr, T, ws_gate, ws_up, h_shared,
                    stream);
    if (e == hipSuccess && down)
      e = gemm_pass(false, pk, 1, d_s, d, dt, h_shared, T, nullptr, nullptr, T, ws_down, nullptr,
                    g, stream);
  }
  return e;
}

int moe_grouped_swiglu(int G, int d_model, int d_ff, int dt, int packed, const void* a,
                       int a_rows, const int32_t* row_index, const int32_t* offsets,
                       int max_rows, const void* w_gate,
                       const void* w_up, const void* w_down, void* h, void* out,
                       hipStream_t stream) {
  MOE_TRY(check_dtype(dt));
  if (packed != 0 && packed != 1) return MOE_ERR_INVALID_ARG;
  if (packed && dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (G <= 0 || d_model <= 0 || d_ff <= 0 || max_rows < 0) return MOE_ERR_INVALID_ARG;
  if (G > moe::kMaxN || d_model % 64 != 0 || d_ff % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && G != 1) return MOE_ERR_INVALID_ARG;
  if (!a || !w_gate || !w_up || !w_down || !h || !out) return MOE_ERR_INVALID_ARG;
  if (row_index != nullptr && a_rows <= 0) return MOE_ERR_INVALID_ARG;
  if (max_rows == 0) return MOE_OK;
  MOE_HIP(gemm_pass(true, packed, G, d_model, d_ff, dt, a, a_rows, row_index, offsets, max_rows,
                    w_gate, w_up, h, stream));
  MOE_HIP(gemm_pass(false, packed, G, d_ff, d_model, dt, h, max_rows, nullptr, offsets, max_rows,
                    w_down, nullptr, out, stream));
  return MOE_OK;
}

int moe_pack_weights(int G, int N_dim, int K_dim, int dt, const void* w, void* w_packed,
                     hipStream_t stream) {
  MOE_TRY(check_dtype(dt));
  if (G <= 0 || N_dim <= 0 || K_dim <= 0 || !w || !w_packed) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16 || N_dim % 64 != 0 || K_dim % 64 != 0) return MOE_ERR_UNSUPPORTED;
  const size_t bytes = static_cast<size_t>(G) * N_dim * K_dim * 2;
  const char* src = static_cast<const char*>(w);
  char* dst = static_cast<char*>(w_packed);
  if (src < dst + bytes && dst < src + bytes) return MOE_ERR_INVALID_ARG;  // overlap
  MOE_HIP(launch_pack_weights(G, N_dim, K_dim, w, w_packed, stream));
  return MOE_OK;
}

int moe_grouped_gemm(int G, int K_dim, int N_dim, int dt, int swiglu, int packed,
                     const void* a, int a_rows, const int32_t* row_index,
                     const int32_t* offsets, int max_rows, const void* w0, const void* w1,
                     void* out, hipStream_t stream) {
  MOE_TRY(check_dtype(dt));
  if (G <= 0 || K_dim <= 0 || N_dim <= 0 || max_rows < 0) return MOE_ERR_INVALID_ARG;
  if (swiglu != 0 && swiglu != 1) return MOE_ERR_INVALID_ARG;
  if (packed != 0 && packed != 1) return MOE_ERR_INVALID_ARG;
  if (packed && dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (G > moe::kMaxN || K_dim % 64 != 0 || N_dim % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && G != 1) return MOE_ERR_INVALID_ARG;
  if (!a || !w0 || (swiglu && !w1) || !out) return MOE_ERR_INVALID_ARG;
  if (row_index != nullptr && a_rows <= 0) return MOE_ERR_INVALID_ARG;
  if (max_rows == 0) return MOE_OK;
  MOE_HIP(gemm_pass(swiglu == 1, packed == 1, G, K_dim, N_dim, dt, a, a_rows, row_index, offsets,
                    max_rows, w0, swiglu ? w1 : nullptr, out, stream));
  return MOE_OK;
}

int moe_experts(int N, int d_model, int d_r, int d_s, int dt, int packed, const void* x, int T,
                const int32_t* row_token, const int32_t* offsets, int max_rows,
                const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                const void* ws_up, const void* ws_down, void* h_perm, void* f_perm,
                void* h_shared, void* g, int pass, hipStream_t stream) {
  MOE_TRY(check_dtype(dt));
  if (packed != 0 && packed != 1) return MOE_ERR_INVALID_ARG;
  if (packed && dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (pass < 0 || pass > 2) return MOE_ERR_INVALID_ARG;
  if (N <= 0 || d_model <= 0 || d_r <= 0 || d_s < 0 || T < 0 || max_rows < 0)
    return MOE_ERR_INVALID_ARG;
  if (N > moe::kMaxN || d_model % 64 != 0 || d_r % 64 != 0 || d_s % 64 != 0)
    return MOE_ERR_UNSUPPORTED;
  if (max_rows > 0 && (!x || !row_token || !offsets || !w_gate || !w_up || !w_down || !h_perm ||
                       !f_perm || T <= 0))
    return MOE_ERR_INVALID_ARG;
  if (d_s > 0 && (!x || !ws_gate || !ws_up || !ws_down || !h_shared || !g))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  MOE_HIP(expert_passes(N, d_model, d_r, d_s, dt, packed == 1, x, T, row_token, offsets, max_rows,
                        w_gate, w_up, w_down, ws_gate, ws_up, ws_down, h_perm, f_perm, h_shared,
                        g, pass, stream));
  return MOE_OK;
}

int moe_combine(int T, int d_model, int K, int dt, const void* f_perm,
                const int32_t* dest_row, const float* topk_r, const void* g, float s,
                const float* s_tok, void* y, hipStream_t stream) {
  MOE_TRY(check_dtype(dt));
  if (T < 0 || d_model <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (K > moe::kMaxK || d_model % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (!f_perm || !dest_row || !topk_r || !y) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  MOE_HIP(launch_combine(T, d_model, K, dt, f_perm, dest_row, topk_r, g, s, s_tok, y, stream));
  return MOE_OK;
}

size_t moe_balance_stats_workspace_size(int T, int N) {
  if (T <= 0 || N <= 0) return 0;
  return stats_workspace_bytes(T, N);
}

int moe_balance_stats(int T, int N, int K, int score, int expert_group, const float* logits,
                      const int32_t* C_req, const int32_t* C_keep, const int32_t* dest_row,
                      const float* topk_r, float* P, float* stats, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || N <= 0 || K <= 0 || K > N) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_group(N, expert_group));
  if (N > moe::kMaxN || K > moe::kMaxK) return MOE_ERR_UNSUPPORTED;
  if (score < MOE_SCORE_SOFTMAX || score > MOE_SCORE_SOFTMAX_SELECTED) return MOE_ERR_INVALID_ARG;
  if (!logits || !C_req || !C_keep || !dest_row || !topk_r || !P || !stats)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!workspace || workspace_bytes < moe_balance_stats_workspace_size(T, N))
    return MOE_ERR_WORKSPACE;
  MOE_HIP(launch_balance_stats(T, N, K, score, expert_group, logits, dest_row, topk_r, C_req,
                               C_keep, P, stats, workspace, stream));
  return MOE_OK;
}

int moe_bias_update(int N, float gamma, int32_t* count_accum, float* expert_bias, int reset,
                    hipStream_t stream) {
  if (N <= 0 || !count_accum || !expert_bias || (reset != 0 && reset != 1))
    return MOE_ERR_INVALID_ARG;
  if (N > moe::kMaxN) return MOE_ERR_UNSUPPORTED;
  if (!std::isfinite(gamma)) return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_bias_update(N, gamma, count_accum, expert_bias, reset, stream));
  return MOE_OK;
}

size_t moe_forward_workspace_size(const moe_forward_args* a) {
  if (!a || a->T <= 0 || a->N <= 0 || a->K <= 0 || a->d_model <= 0) return 0;
  return carve_forward(a, nullptr, nullptr);
}

int moe_forward(const moe_forward_args* a, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_router_dims(a->T, a->d_model, a->N, a->K));
  MOE_TRY(check_dtype(a->dt));
  if (a->score < MOE_SCORE_SOFTMAX || a->score > MOE_SCORE_SOFTMAX_SELECTED) return MOE_ERR_INVALID_ARG;
  if (a->d_r <= 0 || a->d_s < 0) return MOE_ERR_INVALID_ARG;
  if (a->d_r % 64 != 0 || a->d_s % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (!a->x || !a->w_router || !a->w_gate || !a->w_up || !a->w_down || !a->y)
    return MOE_ERR_INVALID_ARG;
  if (a->d_s > 0 && (!a->ws_gate || !a->ws_up || !a->ws_down)) return MOE_ERR_INVALID_ARG;
  if (a->w_shared_gate && a->d_s == 0) return MOE_ERR_INVALID_ARG;
  if (a->weights_packed != 0 && a->weights_packed != 1) return MOE_ERR_INVALID_ARG;
  if (a->weights_packed && a->dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((a->balance_P == nullptr) != (a->balance_stats == nullptr)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_group(a->N, a->capacity_group));
  if (a->T == 0) return MOE_OK;
  if (!workspace || workspace_bytes < moe_forward_workspace_size(a)) return MOE_ERR_WORKSPACE;
  FwdWs w{};
  carve_forward(a, workspace, &w);
  const int T = a->T, d = a->d_model, N = a->N, K = a->K;
  const int rows = moe_max_rows(T, N, K, a->capacity, a->capacity_group);
  // the router also counts its tiles; placement then needs one launch (two past
  // place_fused's histogram size)
  MOE_HIP(launch_route(T, d, N, K, a->score, a->renorm, a->alpha, a->dt, a->x, a->w_router,
                       a->logit_bias, a->expert_bias, a->w_shared_gate, w.logits, 0, w.topk_idx,
                       w.topk_r, w.s_tok, w.route_scratch, w.hist, w.loc_rank, stream));
  const int R = route_tile_tokens(N, d, a->dt, 0, a->w_shared_gate != nullptr);
  MOE_HIP(launch_place(T, d, N, K, R, a->capacity, a->capacity_group, a->dt, a->x, w.topk_idx,
                       w.hist, w.loc_rank, w.C_req, w.C_keep, w.offsets, a->count_accum,
                       w.dest_row, w.row_token, w.x_perm, stream));
  MOE_HIP(expert_passes(N, d, a->d_r, a->d_s, a->dt, a->weights_packed == 1, a->x, T,
                        w.row_token, w.offsets, rows, a->w_gate, a->w_up, a->w_down, a->ws_gate,
                        a->ws_up, a->ws_down, w.h_perm, w.f_perm, w.h_shared, w.g, 0, stream));
  MOE_HIP(launch_combine(T, d, K, a->dt, w.f_perm, w.dest_row, w.topk_r, w.g, a->s, w.s_tok,
                         a->y, stream));
  if (w.stats_ws != nullptr)
    MOE_HIP(launch_balance_stats(T, N, K, a->score, a->capacity_group, w.logits, w.dest_row,
                                 w.topk_r, w.C_req, w.C_keep, a->balance_P, a->balance_stats,
                                 w.stats_ws, stream));
  return MOE_OK;
}

// ---- backward ------------------------------------------------------------------------
namespace {

struct BwdWs {
  uint16_t *dF, *A, *B, *dH, *dAB, *H, *dXp;          // routed: [rows][...]
  uint16_t *dG, *As, *Bs, *dHs, *dABs, *Hs, *dXs;     // shared: [T][...]
};

size_t carve_backward(const moe_backward_args* a, void* ws, BwdWs* out) {
  Carver c(ws);
  BwdWs w{};
  const size_t R = a->max_rows > 0 ? a->max_rows : 0, T = a->T, d = a->d_model;
  const size_t dr = a->d_r, ds = a->d_s;
  w.dF = c.take<uint16_t>(R * d);
  w.A = c.take<uint16_t>(R * dr);
  w.B = c.take<uint16_t>(R * dr);
  w.dH = c.take<uint16_t>(R * dr);
  w.dAB = c.take<uint16_t>(R * 2 * dr);
  w.H = c.take<uint16_t>(R * dr);
  w.dXp = c.take<uint16_t>(R * d);
  if (ds > 0) {
    w.dG = c.take<uint16_t>(T * d);
    w.As = c.take<uint16_t>(T * ds);
    w.Bs = c.take<uint16_t>(T * ds);
    w.dHs = c.take<uint16_t>(T * ds);
    w.dABs = c.take<uint16_t>(T * 2 * ds);
    w.Hs = c.take<uint16_t>(T * ds);
    w.dXs = c.take<uint16_t>(T * d);
  }
  if (out) *out = w;
  return c.off;
}

// one plain (no SwiGLU) contraction for the routed experts and, when given, the shared
// MLP: a single persistent launch when both fit it, else one pass each
hipError_t plain_pair(const StreamProblem& p0, const StreamProblem* p1, hipStream_t stream) {
  if (p1 != nullptr && p0.rows > 0 && stream_gemm_supported(false, p0, *p1))
    return launch_stream_gemm(false, p0, *p1, stream);
  hipError_t e = hipSuccess;
  if (p0.rows > 0)
    e = gemm_pass(false, true, p0.G, p0.Kd, p0.Nd, MOE_BF16, p0.a, p0.a_rows, p0.row_index,
                  p0.offsets, p0.rows, p0.w0, nullptr, p0.out, stream);
  if (e == hipSuccess && p1 != nullptr)
    e = gemm_pass(false, true, 1, p1->Kd, p1->Nd, MOE_BF16, p1->a, p1->a_rows, nullptr, nullptr,
                  p1->rows, p1->w0, nullptr, p1->out, stream);
  return e;
}

}  // namespace

int moe_pack_weights_transposed(int G, int N_dim, int K_dim, int K_a, int dt, const void* w_a,
                                const void* w_b, void* dst, hipStream_t stream) {
  MOE_TRY(check_dtype(dt));
  if (G <= 0 || N_dim <= 0 || K_dim <= 0 || K_a <= 0 || K_a > K_dim || !w_a || !dst)
    return MOE_ERR_INVALID_ARG;
  if ((K_a < K_dim) != (w_b != nullptr)) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16 || N_dim % 64 != 0 || K_dim % 64 != 0 || K_a % 64 != 0)
    return MOE_ERR_UNSUPPORTED;
  const size_t out_bytes = static_cast<size_t>(G) * N_dim * K_dim * 2;
  const size_t a_bytes = static_cast<size_t>(G) * K_a * N_dim * 2;
  const size_t b_bytes = static_cast<size_t>(G) * (K_dim - K_a) * N_dim * 2;
  const char* o = static_cast<const char*>(dst);
  const char* pa = static_cast<const char*>(w_a);
  const char* pb = static_cast<const char*>(w_b);
  if (pa < o + out_bytes && o < pa + a_bytes) return MOE_ERR_INVALID_ARG;  // overlap
  if (pb && pb < o + out_bytes && o < pb + b_bytes) return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_transpose_pack(G, N_dim, K_dim, K_a, w_a, w_b, dst, stream));
  return MOE_OK;
}

size_t moe_backward_workspace_size(const moe_backward_args* a) {
  if (!a || a->T <= 0 || a->d_model <= 0 || a->d_r <= 0 || a->d_s < 0) return 0;
  return carve_backward(a, nullptr, nullptr);
}

int moe_backward(const moe_backward_args* a, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_router_dims(a->T, a->d_model, a->N, a->K));
  MOE_TRY(check_dtype(a->dt));
  if (a->dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (a->d_r <= 0 || a->d_s < 0 || a->max_rows < 0) return MOE_ERR_INVALID_ARG;
  if (a->d_r % 64 != 0 || a->d_s % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (!a->x || !a->dy || !a->row_token || !a->offsets || !a->dest_row || !a->topk_r ||
      !a->w_gate || !a->w_up || !a->wt_down || !a->wt_gate_up || !a->dx || !a->dw_gate ||
      !a->dw_up || !a->dw_down)
    return MOE_ERR_INVALID_ARG;
  if (a->d_s > 0 && (!a->ws_gate || !a->ws_up || !a->wst_down || !a->wst_gate_up ||
                     !a->dws_gate || !a->dws_up || !a->dws_down))
    return MOE_ERR_INVALID_ARG;
  if (a->max_rows > static_cast<long>(a->K) * a->T) return MOE_ERR_INVALID_ARG;
  if (a->T == 0) return MOE_OK;
  if (!workspace || workspace_bytes < moe_backward_workspace_size(a)) return MOE_ERR_WORKSPACE;
  BwdWs w{};
  carve_backward(a, workspace, &w);
  const int T = a->T, d = a->d_model, N = a->N, K = a->K, dr = a->d_r, ds = a->d_s;
  const int R = a->max_rows;
  const bool sh = ds > 0;
  // upstream rows: dF = r dy in the packed expert order, dG = s dy
  MOE_HIP(launch_grad_rows(T, d, K, a->dy, a->dest_row, a->topk_r, a->s, a->s_tok, w.dF,
                           sh ? w.dG : nullptr, stream));
  // dH = dF W_d
  {
    const StreamProblem p0 = problem(w.dF, R, nullptr, a->offsets, N, R, d, dr, a->wt_down,
                                     nullptr, w.dH);
    const StreamProblem p1 = problem(w.dG, T, nullptr, nullptr, 1, T, d, ds, a->wst_down, nullptr,
                                     w.dHs);
    MOE_HIP(plain_pair(p0, sh ? &p1 : nullptr, stream));
  }
  // recompute A and B (rows gathered from x, as in the forward) and take the SwiGLU
  // backward: [dA | dB] and H. One persistent launch does both for the routed experts and
  // the shared MLP where the shapes fit it; otherwise A and B go through memory.
  {
    StreamProblem f0 = problem(a->x, T, a->row_token, a->offsets, N, R, d, dr, a->w_gate,
                               a->w_up, w.H);
    f0.dh = w.dH;
    f0.dab = w.dAB;
    StreamProblem f1{};
    if (sh) {
      f1 = problem(a->x, T, nullptr, nullptr, 1, T, d, ds, a->ws_gate, a->ws_up, w.Hs);
      f1.dh = w.dHs;
      f1.dab = w.dABs;
    }
    if (stream_swiglu_bwd_supported(f0, f1)) {
      MOE_HIP(launch_stream_swiglu_bwd(f0, f1, stream));
    } else {
      const StreamProblem pa = problem(a->x, T, a->row_token, a->offsets, N, R, d, dr,
                                       a->w_gate, nullptr, w.A);
      const StreamProblem pas = problem(a->x, T, nullptr, nullptr, 1, T, d, ds, a->ws_gate,
                                        nullptr, w.As);
      MOE_HIP(plain_pair(pa, sh ? &pas : nullptr, stream));
      const StreamProblem pb = problem(a->x, T, a->row_token, a->offsets, N, R, d, dr, a->w_up,
                                       nullptr, w.B);
      const StreamProblem pbs = problem(a->x, T, nullptr, nullptr, 1, T, d, ds, a->ws_up,
                                        nullptr, w.Bs);
      MOE_HIP(plain_pair(pb, sh ? &pbs : nullptr, stream));
      if (R > 0)
        MOE_HIP(launch_swiglu_bwd(R, a->offsets + N, dr, w.dH, w.A, w.B, w.dAB, w.H, stream));
      if (sh) MOE_HIP(launch_swiglu_bwd(T, nullptr, ds, w.dHs, w.As, w.Bs, w.dABs, w.Hs, stream));
    }
  }
  // dX = [dA dB] [W_g; W_u], then dx = sum over kept routes + shared
  {
    const StreamProblem p0 = problem(w.dAB, R, nullptr, a->offsets, N, R, 2 * dr, d,
                                     a->wt_gate_up, nullptr, w.dXp);
    const StreamProblem p1 = problem(w.dABs, T, nullptr, nullptr, 1, T, 2 * ds, d,
                                     a->wst_gate_up, nullptr, w.dXs);
    MOE_HIP(plain_pair(p0, sh ? &p1 : nullptr, stream));
  }
  MOE_HIP(launch_combine(T, d, K, MOE_BF16, w.dXp, a->dest_row, nullptr, sh ? w.dXs : nullptr,
                         1.0f, nullptr, a->dx, stream));
  // weight gradients, contracting over each expert's rows (zero for experts without rows)
  // (the shared MLP's gradients ride in the same launches: a dense second problem)
  MOE_HIP(launch_wgrad(N, d, dr, w.dF, d, w.H, dr, nullptr, a->offsets, R, a->dw_down,
                       d, ds, w.dG, d, w.Hs, ds, T, sh ? a->dws_down : nullptr, stream));
  MOE_HIP(launch_wgrad(N, dr, d, w.dAB, 2 * dr, a->x, d, a->row_token, a->offsets, R, a->dw_gate,
                       ds, d, w.dABs, 2 * ds, a->x, d, T, sh ? a->dws_gate : nullptr, stream));
  MOE_HIP(launch_wgrad(N, dr, d, w.dAB + dr, 2 * dr, a->x, d, a->row_token, a->offsets, R,
                       a->dw_up, ds, d, sh ? w.dABs + ds : nullptr, 2 * ds, a->x, d, T,
                       sh ? a->dws_up : nullptr, stream));
  return MOE_OK;
}

}  // extern "C"
