/*
 * moe.h - C ABI of the MI355X (gfx950) forward pass of one mixture-of-experts layer.
 *
 * The layer, in the notation of the source pages:
 *   router   z = x W_r^T (+ b), scores, top-K selection S(x), routed coefficients r_i
 *            ("Section 21: Merging Routed and Shared Expert Activations", Eq. 80 and 83;
 *             "Appendix E: Expert-Merge Normalization in Public MoE Models", Table 52)
 *   capacity requested counts C^req, kept counts C^keep = M_i, offsets o_i
 *            ("Section 10: Routing, Capacity, and Load Balancing", Eq. 19, 21, 25, 26)
 *   experts  E(x) = [SiLU(x W_g) * (x W_u)] W_d, run as a grouped GEMM over the packed
 *            per-expert segments ("Section 20: One Shared Expert Is All You Need", Eq. 74)
 *   combine  y = sum_{i in S(x)} r_i f_i(x) + s(x) g(x)   (Section 21, Eq. 80)
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise. The caller owns every buffer;
 *     the library allocates and frees nothing, keeps no state between calls and is
 *     re-entrant. Scratch memory comes from a caller-provided workspace whose size is
 *     returned by the matching *_workspace_size() query.
 *   - Every call only enqueues kernels on `stream` and returns without synchronizing.
 *     Results are valid once the stream has completed.
 *   - Matrices are row-major. Weights use the layout of a PyTorch Linear weight, i.e.
 *     they are stored transposed with respect to the pages' row-vector notation, so the
 *     reduction dimension is contiguous: w_gate[i] = W_g,i^T with shape [d_ff][d_model],
 *     w_up[i] = W_u,i^T [d_ff][d_model], w_down[i] = W_d,i^T [d_model][d_ff],
 *     w_router = W_r^T [N][d_model].
 *   - dtype MOE_BF16: x, weights, packed rows, expert outputs and y are bfloat16 (uint16
 *     bit patterns); logits, coefficients, gates and every accumulator are float32.
 *     dtype MOE_F32: everything is float32.
 *   - Return value: MOE_OK, or a negative moe_status. Arguments are validated before any
 *     kernel is enqueued; on error nothing is enqueued. MOE_ERR_HIP reports a failed
 *     launch; faults inside a kernel surface when the stream is synchronized.
 *   - Limits: 1 <= K <= min(N, 16), N <= 256, d_model and d_ff multiples of 64.
 *     Inputs must be finite. Inputs and outputs must not alias.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* NULL pointer, negative size, K > N, bad enum, short buffer */
  MOE_ERR_UNSUPPORTED = -2, /* outside the limits listed above */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than the *_workspace_size() query */
  MOE_ERR_HIP = -4          /* a kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Router score functions (Appendix E, Table 52):
 *  SOFTMAX           q = softmax over all N logits; renorm: r_i = alpha q_i / sum_S q_j
 *                    (Olmo rule with alpha = K, Section 21 Eq. 83), else r_i = alpha q_i
 *                    (routed mass m_K(x) < 1, Qwen1.5/2 and OLMoE rows)
 *  SIGMOID           sigmoid affinities; renorm: r_i = alpha sigma_i / sum_S sigma_j
 *                    (DeepSeek-V3 row, alpha = 2.5), else r_i = alpha sigma_i
 *  SOFTMAX_SELECTED  softmax over the K selected logits, times alpha (Mixtral row)
 * Selection always ranks the float32 logit z (+ b): every score is monotone in it.
 * Ties go to the lower expert index; -0.0 ties +0.0. The K slots of a token are ordered
 * by descending logit, ties by ascending index. */
typedef enum {
  MOE_SCORE_SOFTMAX = 0,
  MOE_SCORE_SIGMOID = 1,
  MOE_SCORE_SOFTMAX_SELECTED = 2
} moe_score;

/* Host. Short static description of a status code. */
const char* moe_status_string(int status);

/* Host. Per-expert capacity ceil(c * K * T / N): the independent per-expert limit of
 * Section 10 Eq. 25 with T_route = K T routes and N_local = N experts on one GPU,
 * evaluated in double precision. Returns -1 when c < 0 (unlimited capacity). */
int moe_capacity_from_factor(double c, int K, int T, int N);

/* Host. Rank-wide budget max(1, ceil(c * K * T_s)) of Section 10 Eq. 23: one limit
 * shared by the experts of a destination, T_route = K T_s the routes of one source
 * shard of T_s tokens. Double precision; -1 when c < 0 (unlimited). */
int moe_rank_capacity_from_factor(double c, int K, int T_s);

/* Host. Rows needed for packed per-expert buffers: every kept route owns one row
 * (Section 10 Eq. 26), so min(K T, N capacity) under per-expert capacity
 * (capacity_group = 0), min(K T, (N / capacity_group) capacity) under rank-wide
 * capacity, and K T when capacity < 0. */
int moe_max_rows(int T, int N, int K, int capacity, int capacity_group);

/* ---------------------------------------------------------------------------------
 * moe_route: router logits, scores, top-K selection and routed coefficients, plus the
 * requested counts C_i^req = #{t : i in S_t} (Section 10 Eq. 19).
 *
 *   T, d_model, N, K   tokens, model width, routed experts, experts selected per token
 *   score, renorm      score function (moe_score) and selected renormalization (0/1);
 *                      renorm is ignored for SOFTMAX_SELECTED
 *   alpha              routed scale: r_i = alpha p_i (Appendix E)
 *   dt                 moe_dtype of x and w_router
 *   x                  [T][d_model]
 *   w_router           [N][d_model]
 *   logit_bias         [N] float32 added to every logit, or NULL
 *   expert_bias        [N] float32 persistent selection bias b of auxiliary-loss-free
 *                      balancing (Section 10 Eq. 35), or NULL: experts are selected by
 *                      TopK(a + b) with a = z (softmax rules) or sigmoid(z) (sigmoid
 *                      affinities), summed in float32; the coefficients still come from
 *                      the unbiased logits of the selected experts
 *   w_shared_gate      [d_model] (dtype dt) learned shared-gate vector w_s, or NULL;
 *                      when given, s_tok[t] = sigmoid(x_t . w_s) (Table 52, Qwen rows)
 *   logits             [T][N] float32: logits_mode 0 -> output (z + b), may be NULL;
 *                      logits_mode 1 -> input, and x, w_router, logit_bias and
 *                      w_shared_gate are ignored (s_tok must then be NULL)
 *   topk_idx           [T][K] int32 out: selected experts
 *   topk_r             [T][K] float32 out: routed coefficients r
 *   s_tok              [T] float32 out, or NULL (required iff w_shared_gate != NULL)
 *   C_req              [N] int32 out, or NULL
 *   workspace          moe_route_workspace_size(T, d_model, N, K) bytes; needed when C_req
 *                      is given, and for bf16 logits of more than 128 experts without a
 *                      shared gate (N a multiple of 64, d_model a multiple of 256): those
 *                      are computed split over d_model slices (partial logits, summed in
 *                      a fixed order) from a copy of w_router packed in the workspace
 * ------------------------------------------------------------------------------- */
size_t moe_route_workspace_size(int T, int d_model, int N, int K);
int moe_route(int T, int d_model, int N, int K, int score, int renorm, float alpha, int dt,
              const void* x, const void* w_router, const float* logit_bias,
              const float* expert_bias, const void* w_shared_gate, float* logits,
              int logits_mode, int32_t* topk_idx, float* topk_r, float* s_tok, int32_t* C_req,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_bias_update: one step of the hard-count controller of auxiliary-loss-free
 * balancing (Section 10 Eq. 36-37), outside any gradient:
 *   b_i <- b_i + gamma sign(mean_j C_j - C_i)
 * over the requested counts C accumulated during one feedback window (for example by
 * moe_forward_args.count_accum across the microbatches of a batch). The sign is decided
 * exactly in 64-bit integers; an expert exactly at the mean keeps its bias.
 *
 *   count_accum        [N] int32 device, in; set to zero afterwards when reset = 1
 *   expert_bias        [N] float32 device, updated in place
 * Returns MOE_ERR_INVALID_ARG for N <= 0, a NULL pointer, reset not 0/1 or a non-finite
 * gamma, MOE_ERR_UNSUPPORTED for N > 256.
 * ------------------------------------------------------------------------------- */
int moe_bias_update(int N, float gamma, int32_t* count_accum, float* expert_bias, int reset,
                    hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_permute: requested counts, capacity admission, offsets, restoration map and the
 * packed rows (Section 10 Eq. 19, 21, 23, 25, 26 and Section 10.3).
 *
 *   capacity           < 0: every route is kept. capacity_group = 0: routes kept per
 *                      expert, first come by token index (Eq. 25). capacity_group = g > 0:
 *                      experts [q g, (q+1) g) form destination q and share one budget of
 *                      `capacity` rows (Eq. 23), admitted local-expert-major with a
 *                      token-order prefix per expert (the batch's tokens are the source
 *                      shards in rank order); N must be a multiple of g, g = 1 is the
 *                      per-expert limit
 *   x                  [T][d_model] (dtype dt)
 *   topk_idx           [T][K] int32 in (each row holds K distinct experts in [0, N))
 *   C_req, C_keep      [N] int32 out: requested and kept counts (M_i = C_keep[i])
 *   offsets            [N+1] int32 out: o_0 = 0, o_{i+1} = o_i + M_i
 *   dest_row           [T][K] int32 out: packed row of each route, -1 when dropped
 *   row_token          [max_rows] int32 out: source token of packed rows [0, o_N)
 *   x_perm             [max_rows][d_model] out: x_perm[dest_row[t][k]] = x[t]; expert i
 *                      owns rows [o_i, o_{i+1}), rows in ascending token order; rows at
 *                      and beyond o_N are left untouched. May be NULL: then only the
 *                      counts and maps are written, and the grouped GEMM gathers its
 *                      rows from x through row_token instead (no packed copy in HBM)
 *   max_rows           >= moe_max_rows(T, N, K, capacity, capacity_group)
 *   workspace          moe_permute_workspace_size(T, N, K) bytes
 * ------------------------------------------------------------------------------- */
size_t moe_permute_workspace_size(int T, int N, int K);
int moe_permute(int T, int d_model, int N, int K, int capacity, int capacity_group, int dt,
                const void* x, const int32_t* topk_idx, int32_t* C_req, int32_t* C_keep,
                int32_t* offsets, int32_t* dest_row, int32_t* row_token, void* x_perm,
                int max_rows, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_permute_noalloc: moe_permute with its scratch (chunk histograms and in-chunk
 * ranks) in a fixed device array of the library instead of a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Arguments, outputs and errors are
 * those of moe_permute without `workspace` / `workspace_bytes`; nothing is allocated or
 * freed.
 *
 *   limit              moe_permute_workspace_size(T, N, K) = 4 N ceil(T / 64) + 4 T K
 *                      bytes (each part rounded up to 256) must not exceed
 *                      MOE_NOALLOC_SCRATCH_BYTES, else MOE_ERR_WORKSPACE (nothing is
 *                      enqueued); e.g. T = 65536 tokens at N = 256, K = 16 need 5 MiB.
 *   sharing            every GPU holds one such array from the library's first call on
 *                      it until the process ends; all calls on a GPU use it, so calls
 *                      that overlap on one GPU (other streams, other host threads)
 *                      race. Nothing in it needs clearing: each call writes the
 *                      histograms and ranks it reads.
 *   device             the array is resolved for the current device on the first call
 *                      there (hipGetSymbolAddress); a failure returns MOE_ERR_HIP.
 * ------------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int moe_permute_noalloc(int T, int d_model, int N, int K, int capacity, int capacity_group,
                        int dt, const void* x, const int32_t* topk_idx, int32_t* C_req,
                        int32_t* C_keep, int32_t* offsets, int32_t* dest_row,
                        int32_t* row_token, void* x_perm, int max_rows, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_grouped_swiglu: G SwiGLU experts over densely packed row segments, as a grouped
 * GEMM over the real counts (no padding rows):
 *   for each group g, rows r in [offsets[g], offsets[g+1]):
 *     h[r]   = SiLU(a[r] W_g,g) * (a[r] W_u,g)        [d_ff]     (Section 20 Eq. 74)
 *     out[r] = h[r] W_d,g                              [d_model]
 *
 *   G                  groups (routed experts; 1 for the shared MLP)
 *   a                  input rows: [max_rows][d_model] when row_index is NULL, else
 *                      [a_rows][d_model]
 *   a_rows             rows of a when row_index is given (> every entry), else ignored
 *   row_index          [max_rows] int32 DEVICE array or NULL: packed row r reads input row
 *                      a[row_index[r]] (the permutation of Section 10 fused into the
 *                      operand load; pass moe_permute's row_token with a = x), NULL = a[r].
 *                      Entries of rows in [offsets[0], offsets[G]) must index valid rows of a
 *   offsets            [G+1] int32 DEVICE array, non-decreasing, offsets[G] <= max_rows;
 *                      or NULL for one group covering rows [0, max_rows)
 *   w_gate, w_up       [G][d_ff][d_model]
 *   w_down             [G][d_model][d_ff]
 *   h                  [max_rows][d_ff] out (intermediate activation)
 *   out                [max_rows][d_model] out
 *   packed             0: weights row-major as above; 1: weights in the packed layout
 *                      written by moe_pack_weights (bf16 only; the fast path)
 * Rows outside [offsets[0], offsets[G]) are neither read nor written.
 * Several ungated shared experts are run as ONE group whose weights are the
 * concatenation of the gate/up rows and of the down columns (Section 20 Eq. 75-76).
 * ------------------------------------------------------------------------------- */
int moe_grouped_swiglu(int G, int d_model, int d_ff, int dt, int packed, const void* a,
                       int a_rows, const int32_t* row_index, const int32_t* offsets,
                       int max_rows, const void* w_gate,
                       const void* w_up, const void* w_down, void* h, void* out,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_grouped_gemm: ONE pass of the grouped SwiGLU expert, the building block that
 * moe_grouped_swiglu runs twice (packed as in moe_grouped_swiglu):
 *   swiglu = 1: out[r] = SiLU(a[r] W0_g^T) * (a[r] W1_g^T)   (w0 = w_gate, w1 = w_up,
 *               each [G][N_dim][K_dim]; out = h, [max_rows][N_dim])
 *   swiglu = 0: out[r] = a[r] W0_g^T                          (w0 = w_down [G][N_dim][K_dim],
 *               w1 unused)
 * for rows r of group g in [offsets[g], offsets[g+1]) (Section 20 Eq. 74 over the
 * real-count offsets of Section 10 Eq. 26). K_dim and N_dim are multiples of 64;
 * a, a_rows, row_index and offsets as in moe_grouped_swiglu (a[r] stands for a[row_index[r]]
 * when row_index is non-NULL).
 * ------------------------------------------------------------------------------- */
int moe_grouped_gemm(int G, int K_dim, int N_dim, int dt, int swiglu, int packed,
                     const void* a, int a_rows, const int32_t* row_index,
                     const int32_t* offsets, int max_rows, const void* w0, const void* w1,
                     void* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_pack_weights: one-time re-layout of G row-major bf16 weight matrices
 * w[G][N_dim][K_dim] into the order in which the bf16 MFMA consumes them:
 *   w_packed[g][nb][kb][lane][8] = w[g][32 nb + (lane & 31)][16 kb + 8 (lane >> 5) + 0..7]
 * (nb < N_dim / 32, kb < K_dim / 16, lane < 64). Same size as w; w and w_packed must
 * not overlap. Gate, up and down weights are each packed as they are passed to the GEMM
 * (w_gate and w_up with N_dim = d_ff, K_dim = d_model; w_down with N_dim = d_model,
 * K_dim = d_ff). N_dim and K_dim are multiples of 64. dt must be MOE_BF16.
 * ------------------------------------------------------------------------------- */
int moe_pack_weights(int G, int N_dim, int K_dim, int dt, const void* w, void* w_packed,
                     hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_experts: the expert stage of the layer, the routed experts over their real-count
 * segments together with the shared MLP (Section 20 Eq. 74-76 over the offsets of
 * Section 10 Eq. 26), as moe_forward runs it:
 *   routed, rows r of expert i in [offsets[i], offsets[i+1]), t = row_token[r]:
 *     h_perm[r] = SiLU(x[t] W_g,i^T) * (x[t] W_u,i^T),   f_perm[r] = h_perm[r] W_d,i^T
 *   shared (d_s > 0), every token t:
 *     h_shared[t] = SiLU(x[t] Ws_g^T) * (x[t] Ws_u^T),     g[t] = h_shared[t] Ws_d^T
 * With packed weights and widths that the persistent kernel takes (bf16; d_model and d_s
 * multiples of 256, >= 512; d_r a multiple of 256, >= 512) each pass is ONE launch that
 * holds both problems; otherwise the passes run as separate grouped GEMMs.
 *
 *   N, d_model, d_r    routed experts and widths; w_gate, w_up [N][d_r][d_model],
 *                      w_down [N][d_model][d_r]
 *   d_s                shared MLP width (0 = none); ws_gate, ws_up [d_s][d_model],
 *                      ws_down [d_model][d_s] (NULL when d_s == 0)
 *   packed             weights in the moe_pack_weights layout (1) or row-major (0)
 *   x                  [T][d_model]
 *   row_token, offsets moe_permute's restoration map and offsets ([max_rows], [N+1])
 *   h_perm, f_perm     [max_rows][d_r], [max_rows][d_model] out
 *   h_shared, g        [T][d_s], [T][d_model] out
 *   pass               1: gate/up only, 2: down only (reads h_perm, h_shared), 0: both
 * ------------------------------------------------------------------------------- */
int moe_experts(int N, int d_model, int d_r, int d_s, int dt, int packed, const void* x, int T,
                const int32_t* row_token, const int32_t* offsets, int max_rows,
                const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                const void* ws_up, const void* ws_down, void* h_perm, void* f_perm,
                void* h_shared, void* g, int pass, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_combine: y[t] = sum_{k : dest_row[t][k] >= 0} r[t][k] f_perm[dest_row[t][k]]
 *                     + s_t g[t]                                   (Section 21 Eq. 80)
 * Dropped routes contribute nothing and the kept coefficients are not renormalized
 * (Section 10.3). Accumulation is float32 in slot order k = 0..K-1, then the shared
 * term.
 *
 *   f_perm             [rows][d_model] packed expert outputs
 *   dest_row, topk_r   [T][K]
 *   g                  [T][d_model] shared-expert output, or NULL (no shared expert)
 *   s                  shared gain, used when s_tok == NULL
 *   s_tok              [T] float32 per-token shared gate, or NULL
 *   y                  [T][d_model] out
 * ------------------------------------------------------------------------------- */
int moe_combine(int T, int d_model, int K, int dt, const void* f_perm,
                const int32_t* dest_row, const float* topk_r, const void* g, float s,
                const float* s_tok, void* y, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_balance_stats: forward balance statistics and drop diagnostics of one routed
 * batch ("Section 10: Routing, Capacity, and Load Balancing"):
 *   P[i]   = (1/T) sum_t p_{t,i}, the mean of each token's scores normalized across all
 *            N experts (Eq. 38): full softmax of the logits for the softmax modes, sigmoid
 *            affinities divided by their sum for MOE_SCORE_SIGMOID
 *   stats[MOE_STAT_LBL]         N sum_i f_i P_i with f_i = C_req[i] / (K T)   (Eq. 30)
 *   stats[MOE_STAT_IMAX_REQ|KEEP]  N max_i C[i] / sum_i C[i]  (Eq. 39, Eq. 22)
 *   stats[MOE_STAT_IH_REQ|KEEP]    1 - H(C / sum C) / ln N, entropy deficit (Section 10.2);
 *                                  0 when N = 1 (one expert is balanced by construction)
 *   stats[MOE_STAT_CV_REQ|KEEP]    std / mean of the counts (population)
 *   stats[MOE_STAT_NEVER_SELECTED] experts with C_req = 0
 *   stats[MOE_STAT_DELTA_ROUTE]    (K T - sum C_keep) / (K T)                  (Eq. 27)
 *   stats[MOE_STAT_TOKENS_LOST_ANY|ALL] tokens with >= 1 / all K routes dropped (Sec. 10.3)
 *   stats[MOE_STAT_WEIGHT_REMOVED] dropped share of the selected coefficient mass sum r
 *   stats[MOE_STAT_IMAX_RANK_REQ|KEEP] Eq. 22 on destination totals R_q (Eq. 20, 21) when
 *                                  expert_group = g > 0 (destination q owns experts
 *                                  [q g, (q+1) g)); NaN when expert_group = 0
 * Ratios of an all-zero count vector are NaN. Sums run in a fixed order (repeatable).
 *
 *   logits             [T][N] float32 router logits as moe_route writes them (bias added)
 *   C_req, C_keep      [N] int32 (moe_permute); dest_row, topk_r [T][K]
 *   P                  [N] float32 out; stats [MOE_STAT_COUNT] float32 out
 *   workspace          moe_balance_stats_workspace_size(T, N) bytes
 * All buffers are device memory owned by the caller. Returns MOE_ERR_INVALID_ARG for
 * K > N, a non-positive size, an unknown score mode, a NULL buffer, a negative
 * expert_group or one that does not divide N, MOE_ERR_UNSUPPORTED
 * for N > 256 or K > 16, MOE_ERR_WORKSPACE for a short workspace; T = 0 enqueues nothing.
 * ------------------------------------------------------------------------------- */
enum moe_stat {
  MOE_STAT_LBL = 0,
  MOE_STAT_IMAX_REQ = 1,
  MOE_STAT_IMAX_KEEP = 2,
  MOE_STAT_IH_REQ = 3,
  MOE_STAT_IH_KEEP = 4,
  MOE_STAT_CV_REQ = 5,
  MOE_STAT_CV_KEEP = 6,
  MOE_STAT_NEVER_SELECTED = 7,
  MOE_STAT_DELTA_ROUTE = 8,
  MOE_STAT_TOKENS_LOST_ANY = 9,
  MOE_STAT_TOKENS_LOST_ALL = 10,
  MOE_STAT_WEIGHT_REMOVED = 11,
  MOE_STAT_IMAX_RANK_REQ = 12,
  MOE_STAT_IMAX_RANK_KEEP = 13,
  MOE_STAT_COUNT = 14
};
size_t moe_balance_stats_workspace_size(int T, int N);
int moe_balance_stats(int T, int N, int K, int score, int expert_group, const float* logits,
                      const int32_t* C_req, const int32_t* C_keep, const int32_t* dest_row,
                      const float* topk_r, float* P, float* stats, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_forward: the whole layer: route -> permute -> grouped SwiGLU experts -> shared
 * MLP -> combine, all enqueued on `stream` with no host synchronization (counts and
 * offsets stay on the device).
 * ------------------------------------------------------------------------------- */
typedef struct moe_forward_args {
  int T, d_model, N, K;
  int d_r;               /* routed expert width */
  int d_s;               /* shared MLP width (sum of the ungated shared widths), 0 = none */
  int score, renorm;     /* moe_score, 0/1 */
  float alpha;           /* routed scale */
  float s;               /* shared gain when w_shared_gate == NULL */
  int capacity;          /* < 0 = unlimited; per expert, or per destination group */
  int capacity_group;    /* 0: per-expert capacity; g > 0: rank-wide budget shared by each
                            group of g consecutive experts (as in moe_permute) */
  int dt;                /* moe_dtype */
  int weights_packed;    /* 1: w_gate/w_up/w_down and ws_* are in the moe_pack_weights
                            layout (bf16; the fast path), 0: row-major */
  const void* x;         /* [T][d_model] */
  const void* w_router;  /* [N][d_model] */
  const float* logit_bias;    /* [N] or NULL */
  const float* expert_bias;   /* [N] selection-only bias (moe_route), or NULL */
  const void* w_shared_gate;  /* [d_model] or NULL */
  const void* w_gate;    /* [N][d_r][d_model] */
  const void* w_up;      /* [N][d_r][d_model] */
  const void* w_down;    /* [N][d_model][d_r] */
  const void* ws_gate;   /* [d_s][d_model] (NULL when d_s == 0) */
  const void* ws_up;     /* [d_s][d_model] */
  const void* ws_down;   /* [d_model][d_s] */
  void* y;               /* [T][d_model] out */
  /* Optional outputs: when non-NULL the intermediate is written there, otherwise it
   * lives in the workspace. Shapes as in the per-stage entry points; `rows` below is
   * moe_max_rows(T, N, K, capacity, capacity_group). */
  float* logits;         /* [T][N] */
  int32_t* topk_idx;     /* [T][K] */
  float* topk_r;         /* [T][K] */
  float* s_tok;          /* [T] */
  int32_t* C_req;        /* [N] */
  int32_t* C_keep;       /* [N] */
  int32_t* offsets;      /* [N+1] */
  int32_t* dest_row;     /* [T][K] */
  int32_t* row_token;    /* [rows] */
  void* x_perm;          /* [rows][d_model]; only written when non-NULL: the gate/up pass
                            gathers its rows from x through row_token */
  void* h_perm;          /* [rows][d_r] */
  void* f_perm;          /* [rows][d_model] */
  void* g;               /* [T][d_model] shared output */
  /* Balance statistics (moe_balance_stats, expert_group = capacity_group) of the same
   * batch, computed after the combine when both are non-NULL (one without the other is
   * MOE_ERR_INVALID_ARG): */
  float* balance_P;      /* [N] */
  float* balance_stats;  /* [MOE_STAT_COUNT] */
  /* Feedback-window counts for moe_bias_update: C_req of this batch is added to it when
   * non-NULL ([N] int32, zeroed by the caller or by moe_bias_update's reset). */
  int32_t* count_accum;
} moe_forward_args;

size_t moe_forward_workspace_size(const moe_forward_args* args);
int moe_forward(const moe_forward_args* args, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_pack_weights_transposed: packs the transpose of a stack of two matrices in the
 * moe_pack_weights operand order, for the backward's data-gradient contractions:
 *   Wt[g][n][k] = k < K_a ? w_a[g][k][n] : w_b[g][k - K_a][n],   n < N_dim, k < K_dim
 * w_a is [G][K_a][N_dim] and w_b [G][K_dim - K_a][N_dim] (NULL when K_a = K_dim), all bf16
 * device memory; dst is [G][N_dim][K_dim] packed (same size) and must not overlap them.
 * Backward operands: pack(w_down^T) with w_a = w_down viewed [G][d_model][d_r] gives the
 * [G][d_r][d_model] operand of dH; w_a = w_gate, w_b = w_up ([G][d_r][d_model] each) give
 * the [G][d_model][2 d_r] operand of dX. N_dim, K_dim, K_a multiples of 64 (else
 * MOE_ERR_UNSUPPORTED); bf16 only.
 * ------------------------------------------------------------------------------- */
int moe_pack_weights_transposed(int G, int N_dim, int K_dim, int K_a, int dt, const void* w_a,
                                const void* w_b, void* dst, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * moe_backward: gradients of the layer output y (Section 21 Eq. 80 with Section 20
 * Eq. 74 experts) for an upstream gradient dy, with the router held fixed (the
 * fixed-router gradients of Section 21.3): the selection, the kept routes, r and the
 * shared gain are the forward's and are treated as constants. Each kept route's expert
 * row receives r dy and the shared MLP s dy; with A = X W_g^T, B = X W_u^T (recomputed),
 *   dH = dF W_d, dA = dH * B * SiLU'(A), dB = dH * SiLU(A), dX = dA W_g + dB W_u,
 *   dW_d = dF^T H, dW_g = dA^T X, dW_u = dB^T X,
 * and dx sums each token's kept routes' dX rows and the shared branch's. Experts with
 * no kept row get zero weight gradients. bf16 activations and weights (fp32
 * accumulation); weight gradients are written in fp32. Everything is enqueued on
 * `stream` without host synchronization.
 * Returns MOE_ERR_UNSUPPORTED unless dt = MOE_BF16 and the forward's size limits hold,
 * MOE_ERR_INVALID_ARG for a NULL required pointer or inconsistent sizes,
 * MOE_ERR_WORKSPACE for a short workspace; T = 0 enqueues nothing.
 * ------------------------------------------------------------------------------- */
typedef struct moe_backward_args {
  int T, d_model, N, K, d_r, d_s;
  int dt;                     /* MOE_BF16 */
  float s;                    /* shared gain when s_tok == NULL */
  int max_rows;               /* rows of the forward's packed buffers (moe_max_rows) */
  const void* x;              /* [T][d_model] the forward's input */
  const void* dy;             /* [T][d_model] upstream gradient */
  const int32_t* row_token;   /* [max_rows] } the forward's routing (moe_permute / */
  const int32_t* offsets;     /* [N+1]      } moe_forward outputs)                 */
  const int32_t* dest_row;    /* [T][K]     }                                       */
  const float* topk_r;        /* [T][K]     }                                       */
  const float* s_tok;         /* [T] per-token shared gate, or NULL */
  const void* w_gate;         /* [N][d_r][d_model] packed (moe_pack_weights) */
  const void* w_up;           /* [N][d_r][d_model] packed */
  const void* wt_down;        /* [N][d_r][d_model] packed transpose of w_down */
  const void* wt_gate_up;     /* [N][d_model][2 d_r] packed transpose of [w_gate; w_up] */
  const void* ws_gate;        /* [d_s][d_model] packed shared MLP (NULL when d_s = 0) */
  const void* ws_up;          /* [d_s][d_model] packed */
  const void* wst_down;       /* [d_s][d_model] packed transpose of ws_down */
  const void* wst_gate_up;    /* [d_model][2 d_s] packed transpose of [ws_gate; ws_up] */
  void* dx;                   /* [T][d_model] out, bf16 */
  float* dw_gate;             /* [N][d_r][d_model] out */
  float* dw_up;               /* [N][d_r][d_model] out */
  float* dw_down;             /* [N][d_model][d_r] out */
  float* dws_gate;            /* [d_s][d_model] out (NULL when d_s = 0) */
  float* dws_up;              /* [d_s][d_model] out */
  float* dws_down;            /* [d_model][d_s] out */
} moe_backward_args;

size_t moe_backward_workspace_size(const moe_backward_args* args);
int moe_backward(const moe_backward_args* args, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
