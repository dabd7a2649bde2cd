// escha_launch.hpp -- argument blocks and host launchers shared between the
// kernels (escha_kernels.hip) and the validating C ABI (escha_api.cpp).
// Launchers assume validated arguments: every size check happens in the ABI
// layer before any of them is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace escha {

// Output-transformed partial sums of a projection: for each 128-input chunk c,
// partial[p][c] = rout (.) H_n(W~[:, chunk c] x~[chunk c]); the projection's
// output is the fixed-order sum over c. Pair p uses token p / top_k and
// expert ids[p] (or fixed_expert when ids is null). The input row is either
// bf16 (x_bf16) or, when x_bf16 is null, the previous layer's fp32 output
// y_prev with its per-128-block sums of squares ss_prev: the kernel applies
// the RMSNorm (unit weight, eps) and rounds to bf16 itself, and writes those
// bf16 rows to x_out when x_out is not null. partial: fp32
// [n_pairs][in_f/128][out_f].
// Router step inside the streaming gate_up kernel: experts per lane of its
// top-k (n_experts <= 64 kRouteFusedPer).
constexpr int kRouteFusedPer = 4;
// The selections of a router step run inside a layer's first kernel: from
// logits ([n_tokens][n_experts]) to ids_out / w_out ([n_tokens][top_k]).
struct RouteOut {
  const float* logits;
  int top_k;
  int32_t* ids_out;
  float* w_out;
};

struct InPartialArgs {
  const uint16_t* code;
  const uint16_t* rin;
  const uint16_t* rout;
  int32_t n_experts, in_f, out_f, n_pairs, top_k;
  const int32_t* ids;
  int32_t fixed_expert;
  // logits non-null: the router step runs here (fp32 [n_pairs / top_k]
  // [n_experts]; ids is unused) and its selections go to ids_out / w_out
  // ([n_pairs], pair order)
  const float* logits;
  int32_t* ids_out;
  float* w_out;
  const uint16_t* x_bf16;
  const float* y_prev;
  const float* ss_prev;
  float eps;
  uint16_t* x_out;
  float* partial;
};

// Output-transformed partial sums of down_proj, already weighted by the
// router probability w[p] (w may be null: weight 1). The input h comes from
// gate_up's transformed partials (gu_partial fp32 [n_pairs][gu_chunks][2*in_f]):
// h = SiLU(sum gate) * (sum up). inter_out (nullable) receives h.
struct DownPartialArgs {
  const uint16_t* code;
  const uint16_t* rin;
  const uint16_t* rout;
  int32_t n_experts, in_f, out_f, n_pairs;
  const int32_t* ids;
  const float* w;
  const float* gu_partial;
  int32_t gu_chunks;
  float* inter_out;
  float* partial;
  const float* gu_bias;  // nullable fp32 [2*in_f]: gate and up biases, added before the SiLU
};

// y[p] = sum over the chunks of a pair's transformed partials.
struct FinishArgs {
  const float* partial;
  int32_t n_chunks, out_f, n_pairs;
  float* y;
  const float* bias;  // nullable fp32 [out_f], added to every row
};

// Per-token sum over slots (in order) and chunks of down's weighted partials.
// y fp32 [n_tokens][hidden]; ss fp32 [n_tokens][hidden/128] receives each
// 128-block's sum of squares (the next layer's RMSNorm).
struct CombineArgs {
  const float* partial;
  int32_t n_chunks, hidden, top_k, n_tokens;
  float* y;
  float* ss;
  const float* bias;  // nullable fp32 [hidden], added after the slot sum
};

// Grouped path (pairs sorted by expert; see escha_grouped.hip).
struct GatherArgs {
  const uint16_t* x_bf16;  // [T][hidden]
  const uint16_t* rin;     // gate_up rin [E][hidden]
  const int32_t* ids;      // [T*top_k]
  const int32_t* inv;      // pair -> sorted index (-1: the pair has no row)
  int32_t n_pairs, hidden, top_k;
  uint16_t* xg;            // fp16 [P][hidden] at the sorted index, row i scaled by 2^xg_exp[i]
  int32_t* xg_exp;         // [P]: each row's power-of-two exponent
};

// Activations enter the grouped kernels as fp16 with power-of-two
// exponents: gate_up's input rows one per row (x_exp_in [P]), down's input
// one per 128-channel block (x_exp_in [P][inter/128], written by gate_up
// into x_exp_out); the kernels undo them in their fp32 epilogues.
struct GroupedArgs {
  const uint16_t* code;     // this projection's codes
  const uint16_t* rout;     // this projection's rout
  const uint16_t* rin2;     // gate_up kernel: down's rin (for its epilogue)
  int32_t hidden, inter;
  const uint16_t* x_in;     // fp16 rows at the sorted index
  const int32_t* x_exp_in;  // their exponents (see above)
  int32_t* x_exp_out;       // gate_up: exponents of x_out's blocks [P][inter/128]
  uint16_t* x_out;          // gate_up: fp16 rotated down input [P][inter]
  float* y_out;             // down: fp32 weighted outputs [P][hidden]
  float* inter_out;         // nullable: h per pair, pair order
  const int32_t* perm;
  const float* w;           // router weights per pair
  const int32_t* t_expert;
  const int32_t* t_row0;
  const int32_t* t_rows;
  const int32_t* n_tiles;
  const float* bias;        // gate_up kernels: nullable fp32 [2*inter], added before the SiLU
};

// Combine of a layer's sorted pair outputs fused with the RMSNorm of the
// stack chain and the next layer's input gather/rotation (escha_grouped.hip).
struct CombineNextArgs {
  const float* rows;         // this layer's weighted pair outputs [P][hidden], sorted
  const int32_t* inv;        // this layer: pair -> sorted index (-1: none)
  int32_t hidden, top_k, n_tokens;
  float* y;                  // fp32 [T][hidden]
  float eps;
  uint16_t* x_out;           // nullable: bf16 RMSNorm(y) [T][hidden]
  const uint16_t* rin_next;  // next layer's gate_up rin [E][hidden]
  const int32_t* ids_next;   // next layer's [T][top_k]
  const int32_t* inv_next;   // next layer: pair -> sorted index
  uint16_t* xg_next;         // next layer's fp16 rotated inputs [P][hidden], sorted
  int32_t* xg_exp_next;      // their row exponents [P]
};

struct SortedCombineArgs {
  const float* rows;   // [P][hidden] at the sorted index
  const int32_t* inv;  // pair -> sorted index, -1 if the pair has none
  int32_t hidden, top_k, n_tokens;
  float* y;
  float* ss;           // nullable
  const float* bias;   // nullable fp32 [hidden], added after the slot sum
};

// Decode of a whole stack of layers in one launch (escha_stack.hip). Every
// layer has the same hidden/inter/top_k/n_experts and the same k_bits pair.
constexpr int kMaxStackLayers = 64;

struct StackLayer {
  const uint16_t* gu_code;
  const uint16_t* gu_rin;
  const uint16_t* gu_rout;
  const uint16_t* dn_code;
  const uint16_t* dn_rin;
  const uint16_t* dn_rout;
};

// Words handed between tasks are tagged 64-bit words {value, tag}; the tag
// of layer l's words is (epoch << 8) + l + 1, epoch being the call number
// that launch_flow_prepare advances before each launch.
struct FlowArgs {
  StackLayer layer[kMaxStackLayers];
  int32_t n_layers, n_tokens, top_k, hidden, inter, n_experts;
  int32_t p8;          // n_tokens * top_k rounded up to a multiple of 8
  float eps;
  const int32_t* ids;  // [n_layers][n_tokens * top_k]
  const float* w;      // same layout
  const uint16_t* x0;  // bf16 [n_tokens][hidden]
  float* y_last;       // fp32 [n_tokens][hidden]
  uint16_t* x_chain;   // nullable: bf16 [n_layers][n_tokens][hidden]
  uint64_t* gu_part;   // tagged [p8][hidden/512][2*inter], written and read on the pair's XCD
  uint64_t* dn_part;   // tagged, 2 copies of [p8][hidden]: each pair's weighted output
  int64_t dn_copy;     // words per copy
  uint64_t* ycb;       // tagged [n_tokens][8][hidden]: each XCD's copy of the layer output
  uint64_t* sscb;      // tagged [n_tokens][8][32]: its per-128-block sums of squares
  int32_t* dflag;      // [n_layers][p8][df_pair]: down task of output block g at g (its tag)
  int32_t df_pair;
  const int32_t* epoch;  // the call number
  int32_t* ticket;     // [8][32]: next task of each XCD (word 32x)
  int32_t* error;      // 1: a wait gave up
  int32_t fold;        // 1: the down tasks combine the pair outputs (no combine tasks)
  int32_t late;        // 1: tasks decode after their wait (three work-groups per compute unit)
  int32_t wide;        // 1: 4-wave tasks holding two chunks' operands per wave (decode before the
                       // wait, fold only; three work-groups per compute unit)
};
constexpr int kFlowSpare = 64;  // work-groups launched beyond the task count (8 per XCD)

int64_t flow_blocks_per_layer(int hidden, int inter, int top_k, int n_tokens, bool fold);
// Zero the n words of a control block except word 2, the call number, which
// it advances (modulo 2^24).
hipError_t launch_flow_prepare(int32_t* ctl, size_t n, hipStream_t s);
hipError_t launch_stack_flow(const FlowArgs& a, int k_gu, int k_dn, hipStream_t s);
// Work-groups of the one-launch kernel (late: the form that decodes after
// the wait; wide: the 4-wave form) that one compute unit holds at once.
hipError_t flow_groups_per_cu(int k_gu, int k_dn, bool late, bool wide, int* n);

// n_layers tile lists at once (layer l: offsets + l (E + 1), t_* + l max_tiles,
// n_tiles + l).
hipError_t launch_make_tiles(const int32_t* offsets, int E, int tm, int max_tiles, int32_t* t_expert,
                             int32_t* t_row0, int32_t* t_rows, int32_t* n_tiles, hipStream_t s,
                             int n_layers = 1);
hipError_t launch_xin_gather(const GatherArgs& a, int n_pairs, hipStream_t s);
hipError_t launch_grouped_gate_up(const GroupedArgs& a, int max_tiles, int k_bits, hipStream_t s);
hipError_t launch_grouped_down(const GroupedArgs& a, int max_tiles, int k_bits, hipStream_t s);
// Small tiles (at most 16 tokens of one expert; inter and hidden multiples
// of 256): weights decoded straight into matrix-core operands.
hipError_t launch_small_gate_up(const GroupedArgs& a, int max_tiles, int k_bits, hipStream_t s);
// Both small-tile projections of a layer in one launch (gate_up blocks,
// then down blocks that wait for their tile's gate_up blocks on the same
// XCD). ctl: the control block, kSmallCtlFlags + max_tiles * (inter / 128)
// words, zero before the launch; word kSmallCtlErr is 1 afterwards if a
// wait gave up.
constexpr int kSmallCtlErr = 256;
constexpr int kSmallCtlFlags = 288;
inline size_t small_ctl_words(int max_tiles, int inter) { return kSmallCtlFlags + (size_t)max_tiles * (inter / 128); }
hipError_t launch_small_layer(const GroupedArgs& gu, const GroupedArgs& dn, int max_tiles, int k_gu, int k_dn,
                              int32_t* ctl, hipStream_t s);
hipError_t launch_small_down(const GroupedArgs& a, int max_tiles, int k_bits, hipStream_t s);
hipError_t launch_combine_sorted(const SortedCombineArgs& a, hipStream_t s);
hipError_t launch_combine_next(const CombineNextArgs& a, hipStream_t s);

// The shared expert in its w8a16 form (escha_shared.hip): int8 weights with
// f32 scales per group of 128 inputs; gu_w [2*inter][hidden] (gate rows
// first), dn_w [hidden][inter]; gate fp16 [hidden]. h fp32 [T][inter] and
// glogit fp32 [T] are scratch; y fp32 [T][hidden] receives (accumulate: is
// increased by) sigmoid(gate . x) * down(SiLU(gate_x) * up_x).
// hidden % 1024 == 0, hidden <= kShMaxHidden (the gate_up work-group's waves
// take one or two 128-input groups each, at most 16 waves); inter % 512 == 0,
// inter <= kShMaxInter (the down work-group's waves take one group each).
constexpr int kShMaxHidden = 4096;
constexpr int kShMaxInter = 2048;
struct SharedArgs {
  const int8_t* gu_w;
  const float* gu_s;
  const int8_t* dn_w;
  const float* dn_s;
  const uint16_t* gate;
  int32_t hidden, inter, n_tokens;
  const uint16_t* x;
  float* h;
  float* glogit;
  float* y;
  int32_t accumulate;
};
hipError_t launch_shared_expert(const SharedArgs& a, hipStream_t s);

// The device-resident scratch array of escha_static.hip (one per device,
// kStaticScratchBytes): its device address on the current device, looked up
// on the first call there and kept for the process.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
hipError_t static_scratch(void** ptr);

// ids = 0 and weights = 1 for n pairs: the routing of the one-expert case.
hipError_t launch_fill_one_expert(int32_t* ids, float* w, int n, hipStream_t s);

hipError_t launch_in_partial(const InPartialArgs& a, int k_bits, hipStream_t s);
hipError_t launch_down_partial(const DownPartialArgs& a, int k_bits, hipStream_t s);
hipError_t launch_proj_finish(const FinishArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_rmsnorm_bf16(const float* y, int n_tokens, int n, float eps, uint16_t* x,
                               hipStream_t s);
hipError_t launch_decode_tiles(const uint16_t* code_e, int in_f, int out_f, int k_bits,
                               uint16_t* w, hipStream_t s);
// The fused kernels' decoders with their results written in [out][in] order:
// layout 1 = matrix-operand decode (decode_stage_mfma), 2 = LDS tiles
// (decode_to_lds read back through the matrix waves' addressing).
// in_f % 128 == 0, out_f % 256 == 0.
hipError_t launch_decode_operands(const uint16_t* code_e, int in_f, int out_f, int k_bits, int layout,
                                  uint16_t* w, hipStream_t s);
hipError_t launch_hadamard128(const float* x, int64_t rows, int n, float* y, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);
// Router logits (k_router_logits / k_router_reduce): x bf16 [T][H], gate
// fp16 [E][H], logits fp32 [T][E]; part: ksplit * T * E floats when
// ksplit > 1. H % 32 == 0 and (H / 32) % ksplit == 0.
struct RouterArgs {
  const uint16_t* x;
  const uint16_t* gate;
  int T, H, E;
  int ksplit;
  float* logits;
  float* part;
};
// input slices for a call: 1 up to 8 tokens (one wave per expert); else a
// power of two <= 32 dividing H / 32, as many as keep the grid within 4096
// waves
int router_ksplit(int T, int H, int E);
hipError_t launch_router_logits(const RouterArgs& a, hipStream_t s);
// inv (nullable): pair -> sorted index, -1 for a pair with an out-of-range id
// n_layers groupings at once: layer l reads ids + l P and uses counts + l E,
// offsets + l (E + 1), perm / inv / rank + l P, hist / base + l chunks E.
// One work-group per layer doing all of the grouping (and, with t_expert
// non-null, the tile list of launch_make_tiles) when group_small_ok(P, E).
bool group_small_ok(int P, int E);
// clear (nullable): n_clear words per layer zeroed as well (layer l's at
// clear + l n_clear), the small-tile layer kernel's control blocks.
hipError_t launch_group_small(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* inv, int tm, int max_tiles, int32_t* t_expert,
                              int32_t* t_row0, int32_t* t_rows, int32_t* n_tiles, hipStream_t s,
                              int n_layers = 1, int32_t* clear = nullptr, int n_clear = 0);
hipError_t launch_group(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* inv, int32_t* hist, int32_t* base, int32_t* rank,
                        hipStream_t s, int n_layers = 1);

}  // namespace escha
