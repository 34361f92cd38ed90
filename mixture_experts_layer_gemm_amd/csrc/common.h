// Shared device helpers and kernel-launcher declarations of the MoE layer library.
// gfx950 (CDNA4) only: wave64, bf16 MFMA, 160 KB LDS per CU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxK = 16;     // experts selected per token
constexpr int kMaxN = 256;    // routed experts (router tile kept in LDS)
constexpr int kChunk = 64;    // tokens per count chunk (one 64-bit mask per expert)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Workload-group id -> logical tile id so that consecutive logical tiles run on the
// same XCD (the dispatcher hands workgroups to the 8 XCDs round-robin). Tiles that
// share weight or activation tiles then share that XCD's L2. Returns -1 for a spare
// workgroup. `grid` must be a multiple of 8 and >= 8 * ceil(total / 8).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = (total + 7) >> 3;
  const int slot = bid >> 3;
  if (slot >= per) return -1;
  const int t = (bid & 7) * per + slot;
  return t < total ? t : -1;
}

}  // namespace moe

// ---------------------------------------------------------------------------------
// launchers (enqueue only; return hipError_t of the launch)
// ---------------------------------------------------------------------------------
// expert_bias: selection-only bias b of auxiliary-loss-free balancing, or nullptr
// scratch: route_scratch_bytes(T, d_model, N) bytes for the split-K logits of many experts
// (route_split_slices > 0), else unused and may be nullptr
// hist, loc_rank (or nullptr): the router also counts its selections, one histogram row
// of N counts per workgroup of route_tile_tokens(...) tokens and each route's rank among
// its row's routes to the same expert (the input of launch_place with that R)
hipError_t launch_route(int T, int d_model, int N, int K, int score, int renorm, float alpha,
                        int dt, const void* x, const void* w_router, const float* logit_bias,
                        const float* expert_bias, const void* w_shared_gate, float* logits,
                        int logits_mode,
                        int32_t* topk_idx, float* topk_r, float* s_tok, void* scratch,
                        int32_t* hist, int32_t* loc_rank, hipStream_t stream);
int route_split_slices(int N, int d_model, int dt, int logits_mode, bool has_gate);
size_t route_scratch_bytes(int T, int d_model, int N);
int route_tile_tokens(int N, int d_model, int dt, int logits_mode, bool has_gate);

// histogram rows of kChunk tokens from given selections
hipError_t launch_count(int T, int N, int K, const int32_t* topk_idx, int32_t* hist,
                        int32_t* loc_rank, hipStream_t stream);

// capacity < 0: keep every route; group == 0: per-expert limit; group > 0: one budget
// `capacity` shared by each run of `group` consecutive experts. count_accum (or nullptr)
// gets C_req added (feedback-window counts of the bias controller). hist (nrows x N) is
// overwritten with each row's base ranks.
hipError_t launch_scan(int nrows, int N, int capacity, int group, int32_t* hist,
                       int32_t* C_req, int32_t* C_keep, int32_t* offsets, int32_t* count_accum,
                       hipStream_t stream);

// From histogram rows of R tokens (R in {16, 32, 64}): C_req, C_keep, offsets, the
// restoration map and, when x_perm != nullptr, the packed row copy. One launch while
// place_fused(T, N, R), else scan then map / scatter (hist overwritten).
bool place_fused(int T, int N, int R);
hipError_t launch_place(int T, int d_model, int N, int K, int R, int capacity, int group,
                        int dt, const void* x, const int32_t* topk_idx, int32_t* hist,
                        const int32_t* loc_rank, int32_t* C_req, int32_t* C_keep,
                        int32_t* offsets, int32_t* count_accum, int32_t* dest_row,
                        int32_t* row_token, void* x_perm, hipStream_t stream);

// b_i += gamma sign(sum_j C_j - N C_i); C zeroed when reset != 0
hipError_t launch_bias_update(int N, float gamma, int32_t* count_accum, float* expert_bias,
                              int reset, hipStream_t stream);

// x_perm == nullptr: restoration map only (no row copy); hist_base: base ranks of rows
// of R tokens (launch_scan's output)
hipError_t launch_scatter(int T, int d_model, int N, int K, int R, int dt, const void* x,
                          const int32_t* topk_idx, const int32_t* hist_base,
                          const int32_t* loc_rank, const int32_t* C_keep,
                          const int32_t* offsets, int32_t* dest_row, int32_t* row_token,
                          void* x_perm, hipStream_t stream);

size_t stats_workspace_bytes(int T, int N);
hipError_t launch_balance_stats(int T, int N, int K, int score, int group, const float* logits,
                                const int32_t* dest_row, const float* topk_r,
                                const int32_t* C_req, const int32_t* C_keep, float* P,
                                float* stats, void* workspace, hipStream_t stream);

hipError_t launch_grouped_gemm(bool swiglu, int G, int K_dim, int N_dim, int dt, const void* a,
                               const int32_t* row_index, const int32_t* offsets, int max_rows,
                               const void* w0, const void* w1, void* out, hipStream_t stream);

hipError_t launch_grouped_gemm_packed(bool swiglu, int G, int K_dim, int N_dim, const void* a,
                                      const int32_t* row_index, const int32_t* offsets,
                                      int max_rows, const void* w0p, const void* w1p, void* out,
                                      hipStream_t stream);

hipError_t launch_pack_weights(int G, int N_dim, int K_dim, const void* w, void* w_packed,
                               hipStream_t stream);

// backward (router held fixed)
hipError_t launch_transpose_pack(int G, int Nn, int Kk, int Ka, const void* A, const void* B,
                                 void* dst, hipStream_t stream);
hipError_t launch_grad_rows(int T, int d, int K, const void* dy, const int32_t* dest_row,
                            const float* topk_r, float s, const float* s_tok, void* dF,
                            void* dG, hipStream_t stream);
hipError_t launch_swiglu_bwd(int rows, const int32_t* rows_dev, int dff, const void* dH,
                             const void* A, const void* B, void* dAB, void* H,
                             hipStream_t stream);
// weight gradients of G grouped segments (offsets) and, when out1 != nullptr, of one dense
// problem over rows1 rows (the shared MLP) in the same launch
hipError_t launch_wgrad(int G, int M, int Nc, const void* P, int ldp, const void* Q, int ldq,
                        const int32_t* row_index, const int32_t* offsets, int rows, float* out,
                        int M1, int Nc1, const void* P1, int ldp1, const void* Q1, int ldq1,
                        int rows1, float* out1, hipStream_t stream);

// topk_r == nullptr: unit coefficients
hipError_t launch_combine(int T, int d_model, int K, int dt, const void* f_perm,
                          const int32_t* dest_row, const float* topk_r, const void* g,
                          float s, const float* s_tok, void* y, hipStream_t stream);
