// escha_launch.hpp -- argument blocks and host launchers shared between the
// kernels (escha_kernels.hip) and the validating C ABI (escha_api.cpp).
// Launchers assume validated arguments: every size check happens in the ABI
// layer before any of them is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace escha {

// Partial sums of a projection. Pair p uses token p / top_k and expert ids[p]
// (or fixed_expert when ids is null). The input row is either bf16 (x_bf16)
// or, when x_bf16 is null, the previous layer's fp32 output y_prev with its
// per-128-block sums of squares ss_prev: the kernel applies the RMSNorm
// (unit weight, eps) and rounds to bf16 itself, and writes those bf16 rows
// to x_out when x_out is not null. partial: fp32 [n_pairs][in_f/128][out_f].
struct InPartialArgs {
  const uint16_t* code;
  const uint16_t* rin;
  int32_t n_experts, in_f, out_f, n_pairs, top_k;
  const int32_t* ids;
  int32_t fixed_expert;
  const uint16_t* x_bf16;
  const float* y_prev;
  const float* ss_prev;
  float eps;
  uint16_t* x_out;
  float* partial;
};

// Partial sums of down_proj; the input h is produced from gate_up's partials
// (gu_partial fp32 [n_pairs][gu_chunks][2*in_f]). inter_out nullable.
struct DownPartialArgs {
  const uint16_t* code;
  const uint16_t* rin;
  int32_t n_experts, in_f, out_f, n_pairs;
  const int32_t* ids;
  const float* gu_partial;
  int32_t gu_chunks;
  const uint16_t* gu_rout;
  float* inter_out;
  float* partial;
};

// y[p] = rout (.) H_n(sum of partials) for one projection per pair.
struct FinishArgs {
  const float* partial;
  int32_t n_chunks;
  const uint16_t* rout;
  int32_t n_experts, out_f, n_pairs;
  const int32_t* ids;
  int32_t fixed_expert;
  float* y;
};

// Per-token weighted slot sum of down outputs. y fp32 [n_tokens][hidden];
// ss fp32 [n_tokens][hidden/128] receives each 128-block's sum of squares
// (the next layer's RMSNorm).
struct CombineArgs {
  const float* partial;
  int32_t n_chunks;
  const uint16_t* rout;
  const int32_t* ids;
  const float* w;
  int32_t n_experts, hidden, top_k, n_tokens;
  float* y;
  float* ss;
};

hipError_t launch_in_partial(const InPartialArgs& a, int k_bits, hipStream_t s);
hipError_t launch_down_partial(const DownPartialArgs& a, int k_bits, hipStream_t s);
hipError_t launch_proj_finish(const FinishArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_rmsnorm_bf16(const float* y, int n_tokens, int n, float eps, uint16_t* x,
                               hipStream_t s);
hipError_t launch_decode_tiles(const uint16_t* code_e, int in_f, int out_f, int k_bits,
                               uint16_t* w, hipStream_t s);
hipError_t launch_hadamard128(const float* x, int64_t rows, int n, float* y, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);
hipError_t launch_group(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* hist, int32_t* base, int32_t* rank,
                        hipStream_t s);

}  // namespace escha
