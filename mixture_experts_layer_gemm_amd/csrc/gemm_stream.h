// Host interface of the persistent grouped GEMM (gemm_stream.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// One GEMM problem of a launch, bf16 with weights in the moe_pack_weights layout.
//   swiglu: out[r] = SiLU(a[r] W0_g^T) * (a[r] W1_g^T)   (W0, W1: [G][Nd][Kd])
//   plain:  out[r] = a[r] W0_g^T                          (W0: [G][Nd][Kd])
// for packed rows r of group g; a[r] stands for a[row_index[r]] when row_index is set.
struct StreamProblem {
  const uint16_t* a;          // activation rows [a_rows][Kd]
  const int32_t* row_index;   // [rows] packed row -> activation row, or NULL (identity)
  const int32_t* offsets;     // [G + 1] device group offsets, or NULL (one group of `rows`)
  int G;                      // groups
  int rows;                   // packed rows (bound on offsets[G]); 0 = no problem
  int a_rows;                 // rows of a (every row_index entry is below it)
  int Kd;                     // reduction depth
  int Nd;                     // output columns
  const uint16_t* w0;
  const uint16_t* w1;         // SwiGLU only
  uint16_t* out;              // [rows][Nd]
  // SwiGLU backward only (else NULL): dh [rows][Nd] is the gradient of the SwiGLU
  // output; the launch writes out = SiLU(A) B and dab [rows][2 Nd] = [dA | dB]
  const uint16_t* dh;
  uint16_t* dab;
};

// Whether one persistent launch can run p0 (grouped or dense) together with p1 (dense,
// G = 1, no offsets; rows = 0 for none).
bool stream_gemm_supported(bool swiglu, const StreamProblem& p0, const StreamProblem& p1);

// Enqueues p0 and p1 as one launch; hipErrorNotSupported when the shapes do not fit.
hipError_t launch_stream_gemm(bool swiglu, const StreamProblem& p0, const StreamProblem& p1,
                              hipStream_t stream);

// The SwiGLU backward with the gate and up products recomputed: for each problem, with
// A = a W0^T and B = a W1^T, writes out = SiLU(A) B, dab = [dH B SiLU'(A) | dH SiLU(A)].
bool stream_swiglu_bwd_supported(const StreamProblem& p0, const StreamProblem& p1);
hipError_t launch_stream_swiglu_bwd(const StreamProblem& p0, const StreamProblem& p1,
                                    hipStream_t stream);
