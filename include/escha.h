/*
 * escha.h -- C ABI of libescha.so: the trellis-coded ("eschamoe",
 * EXL3-style) routed-expert path of a Qwen3.6-35B-A3B-class MoE layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The experts stay in their packed form and are decoded inside the kernels;
 * no entry point except escha_decode_tiles ever writes decoded weights to
 * memory.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller, contiguous,
 *    row-major, and at least 16-byte aligned. bf16 and fp16 values are passed
 *    as their uint16_t bit patterns.
 *  - `stream` is a hipStream_t passed as void*. All work is enqueued on it,
 *    asynchronously; nothing runs on the null stream unless the caller passes
 *    it. The caller keeps every buffer alive until the stream has finished.
 *  - The library allocates nothing and keeps no reference after a call
 *    returns. Scratch memory is the caller's `workspace`; its required size
 *    comes from the matching *_workspace_bytes function, and a larger
 *    workspace is accepted.
 *  - Every argument is validated on the host before anything is launched.
 *    The return value is ESCHA_OK (0) or a negative ESCHA_E_* code;
 *    escha_last_error() then holds a readable message for the calling
 *    thread. A validation failure launches nothing.
 *  - Expert ids read from device memory (topk_ids) are not visible to the
 *    host: the kernels skip an out-of-range id (its pair contributes zero)
 *    instead of reading outside the expert arrays.
 *
 * Sources (page title, section):
 *  [trellis-mlx] model card "Qwen3.6-35B-A3B-Escha-W2-trellis-mlx",
 *                exactness table and Hadamard note;
 *  [escha-card]  model card "Qwen3.6-35B-A3B-Escha-W2", Format notes;
 *  [hipfire]     PR "Escha-W2 port: 2-bit trellis decoded in the GEMV",
 *                commit notes and the closing summary "What it is".
 */
#ifndef ESCHA_H_
#define ESCHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ESCHA_API __attribute__((visibility("default")))
#else
#define ESCHA_API
#endif

enum escha_status {
  ESCHA_OK = 0,
  ESCHA_E_NULL = -1,        /* a required pointer is NULL */
  ESCHA_E_SHAPE = -2,       /* sizes inconsistent or not tile/block aligned */
  ESCHA_E_KBITS = -3,       /* k_bits is not 2 or 3 */
  ESCHA_E_WORKSPACE = -4,   /* workspace smaller than required */
  ESCHA_E_HIP = -5,         /* a HIP launch or runtime call failed */
  ESCHA_E_UNSUPPORTED = -6, /* valid request this build does not serve */
  ESCHA_E_ARG = -7,         /* scalar argument out of range */
};

/*
 * One coded projection, for every expert of a layer ([hipfire] "What it is";
 * [escha-card] Format notes):
 *   code  int16 [n_experts][in_features/16][out_features/16][16*k_bits]
 *         verbatim trellis words, input-tile index outermost. Each 16x16
 *         tile is a stream of 256*k_bits bits; weight i of the tile is the
 *         fp16 value of the 16-bit window starting at bit k_bits*i (windows
 *         wrap at the tile end), decoded by the hash of [trellis-mlx].
 *   rin   fp16  [n_experts][in_features]   input sign/scale vector
 *   rout  fp16  [n_experts][out_features]  output scale vector; a zero
 *         entry is a pruned channel and its output is exactly zero.
 *   k_bits must equal the code tensor's last dimension / 16 (2 or 3).
 * Alignment: in_features % 128 == 0 and out_features % 256 == 0.
 */
typedef struct escha_proj {
  const void* code;
  const void* rin;
  const void* rout;
  int32_t n_experts;
  int32_t in_features;
  int32_t out_features;
  int32_t k_bits;
} escha_proj_t;

/*
 * One MoE layer's routed experts: gate_up (hidden -> 2*inter; rows
 * [0, inter) are the gate, [inter, 2*inter) the up projection) and down
 * (inter -> hidden). [hipfire] commit notes: gate is the first half.
 */
typedef struct escha_moe_layer {
  escha_proj_t gate_up;
  escha_proj_t down;
  int32_t hidden;
  int32_t inter;
  int32_t top_k;
} escha_moe_layer_t;

/*
 * Decode every weight of one expert to fp16, bit-exact: the one entry point
 * that writes decoded weights, for checking the codec.
 * [trellis-mlx] exactness table (hash, two fp16 halves summed with
 * round-to-nearest-even); [hipfire] "What it is" (tiles and windows).
 *   w_f16  out: fp16 bits [out_features][in_features] of expert `expert`.
 */
ESCHA_API int escha_decode_tiles(const escha_proj_t* w, int32_t expert, uint16_t* w_f16, void* stream);

/*
 * The same decode as escha_decode_tiles, run through the decoder of one of
 * the fused kernels and written back in [out_features][in_features] order,
 * so that each kernel's decoder can be checked bit for bit against the
 * format ([trellis-mlx] exactness table; [hipfire] "What it is"):
 *   ESCHA_LAYOUT_QUARTER        the streaming kernels' decoder (four lanes
 *                               per tile); identical to escha_decode_tiles;
 *   ESCHA_LAYOUT_MFMA_OPERAND   the decoder of the one-launch stack (its K=3
 *                               down tasks) and the small-tile kernels (tiles
 *                               staged in LDS, weights decoded into
 *                               matrix-core A operands);
 *   ESCHA_LAYOUT_LDS_TILE       the decoder of the 128-token grouped kernels
 *                               (an eighth of a tile per lane, fp16 tiles in
 *                               LDS, read back with the matrix waves'
 *                               addressing);
 *   ESCHA_LAYOUT_MFMA_PAIRS     the K=2 decoder of the one-launch stack's
 *                               gate_up tasks (A operands holding output
 *                               columns c and c + 8 of one input row, both
 *                               states from one 32-bit window); K=2 codes
 *                               only, else ESCHA_E_ARG;
 *   ESCHA_LAYOUT_MFMA_TILE_PAIRS the K=2 decoder of the small-tile gate_up
 *                               kernel on tiles of at most 8 tokens (A
 *                               operands covering two output tiles, columns
 *                               c and c + 8 from one window); K=2 only.
 * w_f16 is 16-byte aligned (8 for ESCHA_LAYOUT_QUARTER). An unknown layout
 * returns ESCHA_E_ARG.
 */
enum escha_decode_layout {
  ESCHA_LAYOUT_QUARTER = 0,
  ESCHA_LAYOUT_MFMA_OPERAND = 1,
  ESCHA_LAYOUT_LDS_TILE = 2,
  ESCHA_LAYOUT_MFMA_PAIRS = 3,
  ESCHA_LAYOUT_MFMA_TILE_PAIRS = 4,
};
ESCHA_API int escha_decode_tiles_layout(const escha_proj_t* w, int32_t expert, int32_t layout,
                                        uint16_t* w_f16, void* stream);

/*
 * y = H_n x on each consecutive block of 128 values of every row, with H the
 * Sylvester-ordered 128-point Hadamard matrix and H_n = H / sqrt(128)
 * ([trellis-mlx] Hadamard note). x, y fp32 [rows][n]; n % 128 == 0; x and y
 * may alias.
 */
ESCHA_API int escha_hadamard128(const float* x, int64_t rows, int32_t n, float* y, void* stream);

/*
 * Router step: softmax over each row of fp32 logits [n_tokens][n_experts],
 * then the top_k experts by logit (ties to the lower expert index).
 * topk_ids int32 [n_tokens][top_k] in decreasing-logit order; topk_w fp32
 * [n_tokens][top_k] the selected softmax probabilities, not renormalised.
 * 1 <= top_k <= 32, top_k <= n_experts <= 1024.
 */
ESCHA_API int escha_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                     int32_t* topk_ids, float* topk_w, void* stream);

/*
 * Router logits, the step before escha_route_topk: logits[t][e] = the fp16
 * value nearest (ties to even) to the dot product of gate row e with the
 * hidden state of token t, returned as fp32. [trellis-mlx] exactness table:
 * the router gate (mlp.gate) is kept in fp16; [hipfire] review notes: the
 * logits are rounded to f16 before the top-k, which creates exact ties that
 * escha_route_topk then breaks to the lower expert index. The products of an
 * fp16 and a bf16 value are exact in fp32 and are added with IEEE fp32
 * operations in a fixed order that depends on the number of tokens:
 *   - up to 8 tokens: lane l of a 64-lane wave adds, with FMAs in input
 *     order, the inputs of 32-input chunks l, l + 64, l + 128, ...; the 64
 *     lane sums are then added pairwise in a butterfly (lanes 1, 2, 4, 8,
 *     16, 32 apart);
 *   - more tokens: the inputs are cut into ksplit consecutive slices (ksplit
 *     a power of two <= 32 chosen from the sizes); each slice is summed from
 *     zero with FMAs in input order, and the slice sums are then added in
 *     slice order.
 * A logit can therefore differ from the rounding of the exact sum by one f16
 * step only where that sum lies within the fp32 error of these orders of a
 * midpoint between two f16 values. The same call (sizes) always sums in the
 * same order: results are reproducible.
 *   x_bf16    bf16 [n_tokens][hidden], 16-byte aligned
 *   gate_f16  fp16 [n_experts][hidden], 16-byte aligned
 *   logits    out: fp32 [n_tokens][n_experts]
 * hidden % 32 == 0; 1 <= n_experts <= 1024; n_tokens >= 0 (0: no-op).
 * workspace >= escha_router_workspace_bytes(n_tokens, hidden, n_experts)
 * (partial sums when calls of more than 8 tokens split the inputs; 0 bytes
 * up to 8 tokens).
 */
ESCHA_API size_t escha_router_workspace_bytes(int32_t n_tokens, int32_t hidden, int32_t n_experts);
ESCHA_API int escha_router_logits(const uint16_t* x_bf16, int32_t n_tokens, int32_t hidden,
                                  const uint16_t* gate_f16, int32_t n_experts, float* logits,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Group the n_tokens*top_k (token, slot) pairs by expert ([hipfire] grouped
 * GEMM notes: expert_offsets and a permutation). counts int32 [n_experts];
 * offsets int32 [n_experts+1] exclusive prefix sums; perm int32
 * [n_tokens*top_k] pair indices t*top_k+j sorted by expert, stable in the
 * pair index. Ids out of range are not counted and are left out of perm;
 * perm's tail past offsets[n_experts] is then unspecified.
 * workspace >= escha_moe_group_workspace_bytes(n_tokens, top_k, n_experts).
 */
ESCHA_API size_t escha_moe_group_workspace_bytes(int32_t n_tokens, int32_t top_k, int32_t n_experts);
ESCHA_API int escha_moe_group(const int32_t* topk_ids, int32_t n_tokens, int32_t top_k, int32_t n_experts,
                    int32_t* counts, int32_t* offsets, int32_t* perm, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * One coded projection of one expert on n_tokens activations:
 *   y[t] = rout (.) H_n( W~ H_n( rin (.) x[t] ) )
 * with W~ the decoded [out][in] weights ([hipfire] "What it is": Hadamard on
 * both sides; rin applied before the input rotation, rout as the final
 * multiply). x bf16 [n_tokens][in_features]; y fp32 [n_tokens][out_features].
 */
ESCHA_API size_t escha_expert_gemv_workspace_bytes(const escha_proj_t* w, int32_t n_tokens);
ESCHA_API int escha_expert_gemv(const escha_proj_t* w, int32_t expert, const uint16_t* x_bf16,
                      int32_t n_tokens, float* y, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * One MoE layer: for every token t and slot j with e = topk_ids[t][j],
 *   g,u = split(gate_up_e(x[t]));  h = SiLU(g) * u;
 *   y[t] = sum_j topk_w[t][j] * down_e(h)       (summed in slot order).
 * x bf16 [n_tokens][hidden]; topk_ids int32 / topk_w fp32 [n_tokens][top_k];
 * y fp32 [n_tokens][hidden]; inter_out (nullable) fp32
 * [n_tokens*top_k][inter] receives h per pair, in pair order t*top_k+j.
 * _decode streams every pair's expert weights for fewer than 16 tokens,
 * and from 16 tokens on groups the pairs by expert like _prefill: with at
 * most 16 tokens per expert on average (and hidden, inter multiples of
 * 256) in tiles of up to 16 tokens whose weights are decoded straight into
 * matrix-core operands, otherwise in the 128-token tiles of _prefill;
 * _prefill groups the pairs by expert and decodes each weight tile once per
 * 128-token tile of an expert (long prompts). All compute the same function
 * (summation orders differ: results agree to rounding).
 * escha_moe_workspace_bytes(L, n_tokens, prefill) sizes the workspace of
 * the call that will be made (prefill = 1 for _prefill, 0 for _decode).
 */
ESCHA_API size_t escha_moe_workspace_bytes(const escha_moe_layer_t* L, int32_t n_tokens, int32_t prefill);
ESCHA_API int escha_moe_layer_decode(const escha_moe_layer_t* L, const uint16_t* x_bf16, int32_t n_tokens,
                           const int32_t* topk_ids, const float* topk_w, float* y,
                           float* inter_out, void* workspace, size_t workspace_bytes,
                           void* stream);
ESCHA_API int escha_moe_layer_prefill(const escha_moe_layer_t* L, const uint16_t* x_bf16, int32_t n_tokens,
                            const int32_t* topk_ids, const float* topk_w, float* y,
                            float* inter_out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * escha_moe_layer_decode with the router step inside: topk_ids / topk_w are
 * outputs, the selections escha_route_topk makes from the router logits
 * (fp32 [n_tokens][n_experts of the layer]), and the layer then runs on
 * them. Below 16 tokens, with at most 256 experts and top_k <= 8, every
 * streaming gate_up work-group selects its own pair's expert (and one per
 * token stores the selections), which saves the router step's own launch;
 * otherwise escha_route_topk's kernel runs first. topk_ids, topk_w and y
 * are the same bits as escha_route_topk followed by escha_moe_layer_decode
 * on the same inputs. Same workspace as escha_moe_layer_decode
 * (escha_moe_workspace_bytes(L, n_tokens, 0)); top_k <= 32.
 */
ESCHA_API int escha_moe_layer_decode_logits(const escha_moe_layer_t* L, const uint16_t* x_bf16,
                                            int32_t n_tokens, const float* logits, int32_t* topk_ids,
                                            float* topk_w, float* y, float* inter_out, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * escha_moe_layer_decode for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument. Its scratch is one array of
 * 8 MiB that the library holds on every device it runs on until the process
 * ends (escha_moe_workspace_bytes(L, n_tokens, 0) must not exceed it: with
 * hidden 2048, inter 512, top_k 8 that is 1 to 10 tokens, and 16 to 78
 * tokens through the grouped kernels; a larger request returns
 * ESCHA_E_WORKSPACE and launches nothing). The device address of that array
 * is looked up on the first call on a device. Same kernels, same results
 * as escha_moe_layer_decode. Every call on one device shares the one array:
 * calls that overlap on a device (different streams, not ordered) race and
 * must be serialised by the caller.
 */
ESCHA_API int escha_moe_layer_decode_static(const escha_moe_layer_t* L, const uint16_t* x_bf16,
                                            int32_t n_tokens, const int32_t* topk_ids,
                                            const float* topk_w, float* y, float* inter_out,
                                            void* stream);

/*
 * Dense coded projections: the one-expert case of the routed path, with the
 * additive output biases of an Escha dense export ([hipfire] commit notes:
 * a dense linear is served through the indexed contract as one expert, id 0,
 * weight 1; every coded projection of the dense export carries an additive
 * bias, which no weight absorbs; the gate/up biases land before the SwiGLU,
 * the down / out_proj bias on the output). Biases are fp32 and added after
 * rout, to the projection's output.
 *   gate_up, down  as in escha_moe_layer_t, each with n_experts == 1
 *   gate_up_bias   nullable fp32 [2*inter]
 *   down_bias      nullable fp32 [hidden]
 */
typedef struct escha_dense_mlp {
  escha_proj_t gate_up;
  escha_proj_t down;
  const float* gate_up_bias;
  const float* down_bias;
  int32_t hidden;
  int32_t inter;
} escha_dense_mlp_t;

/*
 * y[t] = down(SiLU(g + b_g) * (u + b_u)) + b_down with g, u the halves of
 * gate_up(x[t]); the same kernels as escha_moe_layer_decode / _prefill with
 * one expert (_decode: the streaming kernels below 16 tokens, the grouped
 * kernels from 16 on; _prefill: the 128-token grouped GEMMs, the expert's
 * token list being all n_tokens tokens, i.e. expert_offsets = [0, n]).
 * x bf16 [n_tokens][hidden]; y fp32 [n_tokens][hidden]; inter_out
 * (nullable) fp32 [n_tokens][inter] receives h.
 * workspace >= escha_dense_mlp_workspace_bytes(M, n_tokens, prefill).
 */
ESCHA_API size_t escha_dense_mlp_workspace_bytes(const escha_dense_mlp_t* M, int32_t n_tokens,
                                                 int32_t prefill);
ESCHA_API int escha_dense_mlp_decode(const escha_dense_mlp_t* M, const uint16_t* x_bf16, int32_t n_tokens,
                                     float* y, float* inter_out, void* workspace, size_t workspace_bytes,
                                     void* stream);
ESCHA_API int escha_dense_mlp_prefill(const escha_dense_mlp_t* M, const uint16_t* x_bf16,
                                      int32_t n_tokens, float* y, float* inter_out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * One dense coded projection (n_experts == 1) plus its bias (nullable fp32
 * [out_features]): y[t] = rout (.) H_n(W~ H_n(rin (.) x[t])) + bias, through
 * the streaming kernels of escha_expert_gemv, whose workspace size it takes
 * (escha_expert_gemv_workspace_bytes).
 */
ESCHA_API int escha_dense_gemv(const escha_proj_t* w, const float* bias, const uint16_t* x_bf16,
                               int32_t n_tokens, float* y, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * The MoE block's shared expert in its w8a16 form, and its gate
 * ([trellis-mlx] exactness table: the shared expert is int8 with f32 scales
 * per group of 128 inputs, its dequantised weight the f32 product
 * scale * w8; shared_expert_gate is fp16. [mtplx] improvements table: int8
 * weights applied by a fused matvec, never dequantised in memory):
 *   gate_up        int8 [2*inter][hidden]: gate rows [0, inter), up rows
 *                  [inter, 2*inter)
 *   gate_up_scale  f32  [2*inter][hidden/128]: row o, inputs 128 g ..
 *                  128 g + 127 use gate_up_scale[o][g]
 *   down           int8 [hidden][inter]
 *   down_scale     f32  [hidden][inter/128]
 *   gate           fp16 [hidden]: the shared_expert_gate row
 * hidden % 1024 == 0 and hidden <= 4096; inter % 512 == 0 and inter <= 2048.
 * int8 tensors 16-byte aligned; scales 4-byte aligned.
 */
typedef struct escha_shared_expert {
  const int8_t* gate_up;
  const float* gate_up_scale;
  const int8_t* down;
  const float* down_scale;
  const uint16_t* gate;
  int32_t hidden;
  int32_t inter;
} escha_shared_expert_t;

/*
 * For every token t: y[t] (+)= sigmoid(gate . x[t]) * down(SiLU(g) * u),
 * g, u = the gate and up halves of gate_up x[t], with weights
 * scale * w8 (binary32 products) and fp32 accumulation. x bf16
 * [n_tokens][hidden]; y fp32 [n_tokens][hidden]. accumulate != 0 adds into
 * y (the routed experts' output of escha_moe_layer_decode/_prefill on the
 * same stream: the MoE block's sum); 0 overwrites it. The gate's dot product
 * is not rounded to fp16 (the pages state that rounding for the router
 * logits only). workspace >= escha_shared_expert_workspace_bytes.
 */
ESCHA_API size_t escha_shared_expert_workspace_bytes(const escha_shared_expert_t* S, int32_t n_tokens);
ESCHA_API int escha_shared_expert(const escha_shared_expert_t* S, const uint16_t* x_bf16,
                                  int32_t n_tokens, float* y, int32_t accumulate, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Between stacked layers: x = bf16( y / sqrt(mean(y^2) + eps) ) per row,
 * unit weight, no residual. y fp32 [n_tokens][n]; x_bf16 [n_tokens][n];
 * n a multiple of 128, at most 16384. Bit-identical to the normalisation
 * escha_moe_stack_decode applies between its layers.
 */
ESCHA_API int escha_rmsnorm_bf16(const float* y, int32_t n_tokens, int32_t n, float eps, uint16_t* x_bf16,
                       void* stream);

/*
 * A stack of n_layers MoE layers applied in turn to n_tokens tokens:
 *   x_0 = x0_bf16; y_l = layer_l(x_l); x_{l+1} = rmsnorm_bf16(y_l).
 * Each layer does what escha_moe_layer_decode does for n_tokens tokens,
 * with the same arithmetic in the same order, and the normalisation is
 * escha_rmsnorm_bf16's, so the result equals those calls chained, bit for
 * bit (from 16 tokens on, one kernel per token links two layers: the
 * combine, the normalisation and the next layer's input rotation).
 * `layers` is a HOST array of n_layers descriptors (their tensors are on
 * the device). topk_ids int32 / topk_w fp32 [n_layers][n_tokens][top_k];
 * y_last fp32 [n_tokens][hidden] = y_{n_layers-1}; x_chain (nullable) bf16
 * [n_layers][n_tokens][hidden] receives each layer's input x_l.
 * All layers must share hidden, inter and top_k.
 * probe_events (nullable): a HOST array of 2*n_layers hipEvent_t handles;
 * events[2l] and events[2l+1] are recorded on `stream` right before layer
 * l's first kernel and right after its last one, so a caller can time each
 * layer inside a longer run. The library does not create or destroy them.
 * Under stream capture they are recorded as external event nodes, so every
 * replay of the graph stamps them.
 */
ESCHA_API size_t escha_moe_stack_workspace_bytes(const escha_moe_layer_t* layers, int32_t n_layers,
                                       int32_t n_tokens);
ESCHA_API int escha_moe_stack_decode(const escha_moe_layer_t* layers, int32_t n_layers,
                           const uint16_t* x0_bf16, int32_t n_tokens, const int32_t* topk_ids,
                           const float* topk_w, float eps, float* y_last, uint16_t* x_chain,
                           void* workspace, size_t workspace_bytes, void* const* probe_events,
                           void* stream);

/*
 * The same stack in ONE kernel launch (plus a small kernel that clears the
 * launch's flag words first). Same arguments and workspace size; the
 * results agree with escha_moe_stack_decode to rounding, not bit for bit
 * (each task sums over more inputs before its output transform, so the
 * fp32 summation order differs; both follow the same arithmetic). Every
 * task of every layer (gate_up and down pieces of one (token, expert) pair,
 * and for larger batches the per-token combine) is one work-group; a
 * work-group loads and decodes its codes before it waits for the outputs
 * it reads, so code streaming and decode of later layers overlap the
 * dependency chain of earlier ones. The tasks of one pair run on one XCD of
 * the device and exchange data through that XCD's L2.
 * Additional requirements: n_layers <= 64; every layer has the same
 * n_experts and the same gate_up and down k_bits; n_tokens <= 64;
 * hidden 1024 or 2048; inter <= 512; top_k * hidden / 256 <= 64.
 * The workspace must be zero-filled before its first use by this call (the
 * data handed between tasks carries a per-call tag kept in the workspace);
 * afterwards the library keeps it consistent from call to call.
 * probe_events (nullable): a HOST array of 2 hipEvent_t handles, recorded
 * right before and right after the kernel (external event nodes under
 * stream capture).
 * A dependency wait that exceeds its bound (half a second; it cannot happen
 * while the device makes progress) makes every work-group stop at its next
 * wait; the outputs are then incomplete and escha_moe_stack_status reports 1.
 * The return value cannot show this: ESCHA_OK only means the launch was
 * enqueued, before the kernel has run. A caller must read the status word
 * with escha_moe_stack_status after the stream has reached the call; the
 * Python binding does so by default (a synchronising read) and raises when
 * it is set.
 * Calls sharing one workspace must be ordered (same stream or synchronised).
 */
ESCHA_API int escha_moe_stack_decode_persistent(const escha_moe_layer_t* layers, int32_t n_layers,
                                      const uint16_t* x0_bf16, int32_t n_tokens,
                                      const int32_t* topk_ids, const float* topk_w, float eps,
                                      float* y_last, uint16_t* x_chain, void* workspace,
                                      size_t workspace_bytes, void* const* probe_events,
                                      void* stream);

/*
 * Status word of the last escha_moe_stack_decode_persistent call on this
 * workspace: waits for `stream`, then stores 0 (complete) or 1 (a wait gave
 * up) in *status (a HOST pointer).
 */
ESCHA_API int escha_moe_stack_status(const void* workspace, int32_t* status, void* stream);

/*
 * Measurement hook. With n_events == 2, every later layer call of the
 * calling thread (escha_moe_layer_decode / _prefill, and each layer of
 * escha_moe_stack_decode) records events[0] on its stream right before its
 * gate_up projection kernel and events[1] right after its down projection
 * kernel, so a caller can time the two projection kernels alone (and
 * escha_shared_expert around its two kernels); events
 * NULL or n_events == 0 removes the hook. The handles are hipEvent_t
 * created by the caller, who keeps them alive while the hook is set. Under
 * stream capture the records become external event nodes of the graph.
 */
ESCHA_API int escha_probe_events_set(void* const* events, int32_t n_events);

/* Message for the calling thread's last failed call ("" if none). */
ESCHA_API const char* escha_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ESCHA_H_ */
