// escha_api.cpp -- the C ABI of libescha.so (declared in include/escha.h):
// host-side validation, workspace layout and launch sequencing. No entry
// point allocates memory; every launch goes on the caller's stream.
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "escha.h"
#include "escha_launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(ESCHA_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// A probe event recorded on the stream. Under stream capture a plain record
// is not a node of the graph (a replay would never stamp the event), so an
// event-record node is added to the graph being captured, after the
// stream's current capture dependencies, and becomes the new dependency.
// A failure is returned and also cleared from the runtime's last-error
// state, so that later launch checks do not report it again.
hipError_t record_probe(hipEvent_t ev, hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipGraph_t graph = nullptr;
  const hipGraphNode_t* deps = nullptr;
  size_t n_deps = 0;
  hipError_t e = hipStreamGetCaptureInfo_v2(s, &st, nullptr, &graph, &deps, &n_deps);
  if (e == hipSuccess) {
    if (st != hipStreamCaptureStatusActive) {
      e = hipEventRecord(ev, s);
    } else {
      hipGraphNode_t node = nullptr;
      e = hipGraphAddEventRecordNode(&node, graph, deps, n_deps, ev);
      if (e == hipSuccess) e = hipStreamUpdateCaptureDependencies(s, &node, 1, hipStreamSetCaptureDependencies);
    }
  }
  if (e != hipSuccess) (void)hipGetLastError();
  return e;
}

// Events that escha_probe_events_set installs for this thread: recorded
// right before a layer call's gate_up projection kernel and right after its
// down projection kernel.
thread_local hipEvent_t g_proj_probe[2] = {nullptr, nullptr};

int probe_proj(int which, hipStream_t s) {
  if (!g_proj_probe[which]) return ESCHA_OK;
  const hipError_t e = record_probe(g_proj_probe[which], s);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "projection probe record");
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int32_t kMaxTopK = 64;
constexpr int32_t kMaxHidden = 16384;  // k_rmsnorm_bf16 keeps one sum per 128-block in LDS
constexpr int32_t kMaxExpertsRoute = 1024;
constexpr int32_t kMaxStackTokens = 64;  // persistent stack path

int check_proj(const escha_proj_t* w, const char* what) {
  if (!w) return fail(ESCHA_E_NULL, "%s: descriptor is NULL", what);
  if (!w->code || !w->rin || !w->rout) return fail(ESCHA_E_NULL, "%s: code/rin/rout is NULL", what);
  if (w->k_bits != 2 && w->k_bits != 3)
    return fail(ESCHA_E_KBITS, "%s: k_bits=%d, must be 2 or 3", what, (int)w->k_bits);
  if (w->n_experts < 1) return fail(ESCHA_E_SHAPE, "%s: n_experts=%d", what, (int)w->n_experts);
  if (w->in_features < 128 || w->in_features % 128)
    return fail(ESCHA_E_SHAPE, "%s: in_features=%d is not a positive multiple of 128", what,
                (int)w->in_features);
  if (w->out_features < 256 || w->out_features % 256)
    return fail(ESCHA_E_SHAPE, "%s: out_features=%d is not a positive multiple of 256", what,
                (int)w->out_features);
  if (!aligned(w->code, 16)) return fail(ESCHA_E_ARG, "%s: code is not 16-byte aligned", what);
  if (!aligned(w->rin, 2) || !aligned(w->rout, 2))
    return fail(ESCHA_E_ARG, "%s: rin/rout are not 2-byte aligned", what);
  return ESCHA_OK;
}

int check_layer(const escha_moe_layer_t* L) {
  if (!L) return fail(ESCHA_E_NULL, "layer descriptor is NULL");
  int rc = check_proj(&L->gate_up, "gate_up");
  if (rc) return rc;
  rc = check_proj(&L->down, "down");
  if (rc) return rc;
  if (L->gate_up.in_features != L->hidden || L->gate_up.out_features != 2 * L->inter ||
      L->down.in_features != L->inter || L->down.out_features != L->hidden)
    return fail(ESCHA_E_SHAPE,
                "layer shapes disagree: hidden=%d inter=%d gate_up %dx%d down %dx%d", L->hidden,
                L->inter, L->gate_up.in_features, L->gate_up.out_features, L->down.in_features,
                L->down.out_features);
  if (L->gate_up.n_experts != L->down.n_experts)
    return fail(ESCHA_E_SHAPE, "gate_up has %d experts, down has %d", L->gate_up.n_experts,
                L->down.n_experts);
  if (L->hidden > kMaxHidden) return fail(ESCHA_E_UNSUPPORTED, "hidden=%d > %d", L->hidden, kMaxHidden);
  if (L->top_k < 1 || L->top_k > kMaxTopK || L->top_k > L->gate_up.n_experts)
    return fail(ESCHA_E_ARG, "top_k=%d out of range", L->top_k);
  if (L->gate_up.n_experts > kMaxExpertsRoute)
    return fail(ESCHA_E_UNSUPPORTED, "n_experts=%d > %d", L->gate_up.n_experts, kMaxExpertsRoute);
  return ESCHA_OK;
}

// ---------------------------------------------------------------- decode ws
struct DecodeWs {
  float* gu_part;  // [P][hidden/128][2*inter]
  float* dn_part;  // [P][inter/128][hidden]
  float* ss;       // [T][hidden/128] per-block sums of squares of y
};

size_t decode_ws_bytes(const escha_moe_layer_t* L, int64_t T) {
  const int64_t P = T * L->top_k;
  const size_t gu = (size_t)P * (L->hidden / 128) * (2 * L->inter) * sizeof(float);
  const size_t dn = (size_t)P * (L->inter / 128) * L->hidden * sizeof(float);
  const size_t ss = (size_t)T * (L->hidden / 128) * sizeof(float);
  return round_up(gu) + round_up(dn) + round_up(ss);
}

DecodeWs decode_ws_carve(const escha_moe_layer_t* L, int64_t T, void* ws) {
  const int64_t P = T * L->top_k;
  const size_t gu = (size_t)P * (L->hidden / 128) * (2 * L->inter) * sizeof(float);
  const size_t dn = (size_t)P * (L->inter / 128) * L->hidden * sizeof(float);
  char* b = (char*)ws;
  DecodeWs d;
  d.gu_part = (float*)b;
  d.dn_part = (float*)(b + round_up(gu));
  d.ss = (float*)(b + round_up(gu) + round_up(dn));
  return d;
}

// Where a layer's input row comes from: bf16 rows, or the previous layer's
// fp32 output with its block sums of squares (RMSNorm applied on the fly).
struct LayerInput {
  const uint16_t* x_bf16;
  const float* y_prev;
  const float* ss_prev;
  float eps;
  uint16_t* x_out;  // nullable: the bf16 rows the layer consumed
};

// One layer over T tokens through the streaming kernels.
// gu_bias / dn_bias (nullable): the dense export's biases (one-expert case).
// route (nullable): the router step runs inside the first kernel, from
// route->logits, and its selections (route->ids_out / w_out) are the
// routing (ids and w are then unused).
int run_layer_decode(const escha_moe_layer_t* L, const LayerInput& in, int T, const int32_t* ids,
                     const float* w, float* y, float* inter_out, const DecodeWs& ws,
                     hipStream_t s, hipEvent_t probe_before = nullptr,
                     hipEvent_t probe_after = nullptr, const float* gu_bias = nullptr,
                     const float* dn_bias = nullptr, const escha::RouteOut* route = nullptr) {
  const int P = T * L->top_k;
  if (route) {
    ids = route->ids_out;
    w = route->w_out;
  }
  escha::InPartialArgs a{};
  a.code = (const uint16_t*)L->gate_up.code;
  a.rin = (const uint16_t*)L->gate_up.rin;
  a.rout = (const uint16_t*)L->gate_up.rout;
  a.n_experts = L->gate_up.n_experts;
  a.in_f = L->hidden;
  a.out_f = 2 * L->inter;
  a.n_pairs = P;
  a.top_k = L->top_k;
  a.ids = route ? nullptr : ids;
  a.fixed_expert = 0;
  if (route) {
    a.logits = route->logits;
    a.ids_out = route->ids_out;
    a.w_out = route->w_out;
  }
  a.x_bf16 = in.x_bf16;
  a.y_prev = in.y_prev;
  a.ss_prev = in.ss_prev;
  a.eps = in.eps;
  a.x_out = in.x_out;
  a.partial = ws.gu_part;
  hipError_t e;
  if (probe_before && (e = record_probe(probe_before, s)) != hipSuccess)
    return hip_fail(e, "probe event record");
  int rc = probe_proj(0, s);
  if (rc) return rc;
  e = escha::launch_in_partial(a, L->gate_up.k_bits, s);
  if (e != hipSuccess) return hip_fail(e, "gate_up partial launch");

  escha::DownPartialArgs d{};
  d.code = (const uint16_t*)L->down.code;
  d.rin = (const uint16_t*)L->down.rin;
  d.rout = (const uint16_t*)L->down.rout;
  d.n_experts = L->down.n_experts;
  d.in_f = L->inter;
  d.out_f = L->hidden;
  d.n_pairs = P;
  d.ids = ids;
  d.w = w;
  d.gu_partial = ws.gu_part;
  d.gu_chunks = L->hidden / 128;
  d.inter_out = inter_out;
  d.partial = ws.dn_part;
  d.gu_bias = gu_bias;
  e = escha::launch_down_partial(d, L->down.k_bits, s);
  if (e != hipSuccess) return hip_fail(e, "down partial launch");
  rc = probe_proj(1, s);
  if (rc) return rc;

  escha::CombineArgs c{};
  c.partial = ws.dn_part;
  c.n_chunks = L->inter / 128;
  c.hidden = L->hidden;
  c.top_k = L->top_k;
  c.n_tokens = T;
  c.y = y;
  c.ss = ws.ss;
  c.bias = dn_bias;
  e = escha::launch_combine(c, s);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  if (probe_after && (e = record_probe(probe_after, s)) != hipSuccess)
    return hip_fail(e, "probe event record");
  return ESCHA_OK;
}

// ---------------------------------------------------------------- grouped ws
// Decode calls (single layers and the layer-by-layer stack) with at least
// this many tokens take the grouped path: pairs sorted by expert, each
// weight tile decoded once for all of an expert's tokens in a tile.
constexpr int32_t kGroupedDecodeTokens = 16;
// One-launch stack: with top_k <= 8, from kFlowWideTokens to
// kFlowWideMaxTokens tokens its tasks are 4 waves holding two chunks'
// decoded operands per wave (three work-groups per compute unit; measured
// faster than both 8-wave forms there). Otherwise from kFlowLateTokens
// tokens its 8-wave tasks decode after their wait (three work-groups per
// compute unit), and below that before it (two).
constexpr int32_t kFlowWideTokens = 1;
constexpr int32_t kFlowWideMaxTokens = 16;
constexpr int32_t kFlowLateTokens = 8;
constexpr int32_t kTileTokens = 128;      // tokens per grouped tile (escha_grouped.hip)
constexpr int32_t kSmallTileTokens = 16;  // tokens per small tile

// Decode calls whose experts get at most 16 tokens on average take the small
// tiles (weights decoded straight into matrix-core operands); prefill calls
// and larger batches take the 128-token tiles, which decode each expert's
// weights once for up to 128 of its tokens.
bool grouped_small(const escha_moe_layer_t* L, int64_t T, bool prefill) {
  const int64_t P = T * L->top_k;
  return !prefill && L->inter % 256 == 0 && L->hidden % 256 == 0 && L->inter <= 2048 &&
         P <= (int64_t)kSmallTileTokens * L->gate_up.n_experts;
}

// Tile-list capacity: enough for either tile size.
int32_t grouped_max_tiles(const escha_moe_layer_t* L, int64_t T, bool small) {
  const int64_t P = T * L->top_k;
  const int64_t tm = small ? kSmallTileTokens : kTileTokens;
  return (int32_t)((P + tm - 1) / tm + L->gate_up.n_experts);
}

struct GroupedWs {
  int32_t *hist, *base, *rank;          // grouping scratch
  int32_t *counts, *offsets, *perm, *inv;
  int32_t *t_expert, *t_row0, *t_rows, *n_tiles;
  uint16_t* xg;     // fp16 [P][hidden], row i scaled by 2^xg_exp[i]
  uint16_t* xd;     // fp16 [P][inter], 128-block c of row i scaled by 2^xd_exp[i][c]
  float* yd;        // fp32 [P][hidden]
  int32_t* xg_exp;  // [P]
  int32_t* xd_exp;  // [P][inter/128]
  int32_t* sctl;    // control blocks of the one-launch small-tile layer kernel, sctl_words per layer
  int32_t sctl_words;
};

// Carves the grouped workspace; with ws == nullptr only sizes it. The
// grouping and tile-list arrays are held for n_layers layers (layer l's at
// the offsets that launch_group and launch_make_tiles use for layer l);
// the activation buffers once.
size_t grouped_ws(const escha_moe_layer_t* L, int64_t T, void* ws, GroupedWs* out,
                  int n_layers = 1) {
  const int64_t P = T * L->top_k;
  const int E = L->gate_up.n_experts;
  const int32_t mt = grouped_max_tiles(L, T, true);
  const size_t chunks = ((size_t)P + 63) / 64;
  const size_t nl = (size_t)n_layers;
  size_t off = 0;
  char* b = (char*)ws;
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += round_up(bytes);
    return p;
  };
  GroupedWs g{};
  g.hist = (int32_t*)take(nl * chunks * E * sizeof(int32_t));
  g.base = (int32_t*)take(nl * chunks * E * sizeof(int32_t));
  g.rank = (int32_t*)take(nl * (size_t)P * sizeof(int32_t));
  g.counts = (int32_t*)take(nl * (size_t)E * sizeof(int32_t));
  g.offsets = (int32_t*)take(nl * (size_t)(E + 1) * sizeof(int32_t));
  g.perm = (int32_t*)take(nl * (size_t)P * sizeof(int32_t));
  g.inv = (int32_t*)take(nl * (size_t)P * sizeof(int32_t));
  g.t_expert = (int32_t*)take(nl * (size_t)mt * sizeof(int32_t));
  g.t_row0 = (int32_t*)take(nl * (size_t)mt * sizeof(int32_t));
  g.t_rows = (int32_t*)take(nl * (size_t)mt * sizeof(int32_t));
  g.n_tiles = (int32_t*)take(nl * sizeof(int32_t));
  g.xg = (uint16_t*)take((size_t)P * L->hidden * sizeof(uint16_t));
  g.xd = (uint16_t*)take((size_t)P * L->inter * sizeof(uint16_t));
  g.yd = (float*)take((size_t)P * L->hidden * sizeof(float));
  g.xg_exp = (int32_t*)take((size_t)P * sizeof(int32_t));
  g.xd_exp = (int32_t*)take((size_t)P * (L->inter / 128) * sizeof(int32_t));
  g.sctl_words = (int32_t)round_up(escha::small_ctl_words(mt, L->inter) * sizeof(int32_t)) / sizeof(int32_t);
  g.sctl = (int32_t*)take(nl * (size_t)g.sctl_words * sizeof(int32_t));
  if (out) *out = g;
  return off;
}

// Layer l's grouping and tile-list arrays of a workspace carved for
// several layers.
GroupedWs grouped_layer(const GroupedWs& g, const escha_moe_layer_t* L, int64_t T, int l) {
  const int64_t P = T * L->top_k;
  const int E = L->gate_up.n_experts;
  const size_t chunks = ((size_t)P + 63) / 64;
  const int32_t mt = grouped_max_tiles(L, T, true);
  GroupedWs v = g;
  v.sctl += (size_t)l * g.sctl_words;
  v.hist += (size_t)l * chunks * E;
  v.base += (size_t)l * chunks * E;
  v.rank += (size_t)l * P;
  v.counts += (size_t)l * E;
  v.offsets += (size_t)l * (E + 1);
  v.perm += (size_t)l * P;
  v.inv += (size_t)l * P;
  v.t_expert += (size_t)l * mt;
  v.t_row0 += (size_t)l * mt;
  v.t_rows += (size_t)l * mt;
  v.n_tiles += l;
  return v;
}

// The grouping and tile lists of n_layers layers (ids [n_layers][T][top_k])
// into a workspace carved for n_layers layers.
int group_layers(const escha_moe_layer_t* L, int T, const int32_t* ids, const GroupedWs& g,
                 bool prefill, int n_layers, hipStream_t s) {
  const int P = T * L->top_k;
  const int E = L->gate_up.n_experts;
  const bool small = grouped_small(L, T, prefill);
  if (escha::group_small_ok(P, E)) {
    // also zeroes the layers' control blocks of the one-launch small-tile
    // layer kernel (run_layer_grouped uses it after this grouping only)
    const hipError_t e = escha::launch_group_small(
        ids, P, E, g.counts, g.offsets, g.perm, g.inv, small ? kSmallTileTokens : kTileTokens,
        grouped_max_tiles(L, T, true), g.t_expert, g.t_row0, g.t_rows, g.n_tiles, s, n_layers, g.sctl,
        g.sctl_words);
    return e == hipSuccess ? ESCHA_OK : hip_fail(e, "group launch");
  }
  hipError_t e = escha::launch_group(ids, P, E, g.counts, g.offsets, g.perm, g.inv, g.hist, g.base,
                                     g.rank, s, n_layers);
  if (e != hipSuccess) return hip_fail(e, "group launch");
  e = escha::launch_make_tiles(g.offsets, E, small ? kSmallTileTokens : kTileTokens,
                               grouped_max_tiles(L, T, true), g.t_expert, g.t_row0, g.t_rows,
                               g.n_tiles, s, n_layers);
  if (e != hipSuccess) return hip_fail(e, "tile list launch");
  return ESCHA_OK;
}

// One layer over T tokens through the grouped kernels: group the pairs by
// expert (unless `grouped`: g then already holds this layer's grouping),
// decode every weight tile once per tile of its expert's tokens, contract
// on the matrix cores, combine in slot order.
// grouped: the pairs are already grouped (by an up-front call for all
// layers); gather: rotate x into g.xg here (else it is already there);
// combine: add the pair outputs into y here (else the caller does).
int run_layer_grouped(const escha_moe_layer_t* L, const uint16_t* x, int T, const int32_t* ids,
                      const float* w, float* y, float* inter_out, const GroupedWs& g,
                      bool prefill, hipStream_t s, bool grouped = false, bool gather = true,
                      bool combine = true, const float* gu_bias = nullptr,
                      const float* dn_bias = nullptr) {
  const int P = T * L->top_k;
  const int E = L->gate_up.n_experts;
  const bool small = grouped_small(L, T, prefill);
  // grid bound: the tile count for this tile size never exceeds it (the
  // tile lists themselves are laid out for the small-tile bound)
  const int32_t max_tiles = grouped_max_tiles(L, T, small);
  hipError_t e;
  if (!grouped) {
    const int rc = group_layers(L, T, ids, g, prefill, 1, s);
    if (rc) return rc;
  }
  if (gather) {
    escha::GatherArgs ga{x, (const uint16_t*)L->gate_up.rin, ids, g.inv, P, L->hidden, L->top_k, g.xg,
                         g.xg_exp};
    e = escha::launch_xin_gather(ga, P, s);
    if (e != hipSuccess) return hip_fail(e, "input gather launch");
  }
  escha::GroupedArgs gu{};
  gu.code = (const uint16_t*)L->gate_up.code;
  gu.rout = (const uint16_t*)L->gate_up.rout;
  gu.rin2 = (const uint16_t*)L->down.rin;
  gu.hidden = L->hidden;
  gu.inter = L->inter;
  gu.x_in = g.xg;
  gu.x_exp_in = g.xg_exp;
  gu.x_exp_out = g.xd_exp;
  gu.x_out = g.xd;
  gu.inter_out = inter_out;
  gu.perm = g.perm;
  gu.w = w;
  gu.t_expert = g.t_expert;
  gu.t_row0 = g.t_row0;
  gu.t_rows = g.t_rows;
  gu.n_tiles = g.n_tiles;
  gu.bias = gu_bias;
  int rc = probe_proj(0, s);
  if (rc) return rc;
  // small tiles after the one-work-group grouping (which zeroed the control
  // block): both projections in one launch
  const bool one_launch = small && escha::group_small_ok(P, E);
  if (!one_launch) {
    e = small ? escha::launch_small_gate_up(gu, max_tiles, L->gate_up.k_bits, s)
              : escha::launch_grouped_gate_up(gu, max_tiles, L->gate_up.k_bits, s);
    if (e != hipSuccess) return hip_fail(e, "grouped gate_up launch");
  }
  escha::GroupedArgs dn = gu;
  dn.code = (const uint16_t*)L->down.code;
  dn.rout = (const uint16_t*)L->down.rout;
  dn.rin2 = nullptr;
  dn.x_in = g.xd;
  dn.x_exp_in = g.xd_exp;
  dn.x_exp_out = nullptr;
  dn.x_out = nullptr;
  dn.y_out = g.yd;
  dn.inter_out = nullptr;
  dn.bias = nullptr;
  if (one_launch) {
    e = escha::launch_small_layer(gu, dn, max_tiles, L->gate_up.k_bits, L->down.k_bits, g.sctl, s);
    if (e != hipSuccess) return hip_fail(e, "small-tile layer launch");
  } else {
    e = small ? escha::launch_small_down(dn, max_tiles, L->down.k_bits, s)
              : escha::launch_grouped_down(dn, max_tiles, L->down.k_bits, s);
    if (e != hipSuccess) return hip_fail(e, "grouped down launch");
  }
  rc = probe_proj(1, s);
  if (rc) return rc;
  if (!combine) return ESCHA_OK;
  escha::SortedCombineArgs c{g.yd, g.inv, L->hidden, L->top_k, T, y, nullptr, dn_bias};
  e = escha::launch_combine_sorted(c, s);
  if (e != hipSuccess) return hip_fail(e, "sorted combine launch");
  return ESCHA_OK;
}

int check_layer_call(const escha_moe_layer_t* L, const uint16_t* x, int32_t T, const int32_t* ids,
                     const float* w, const float* y) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", T);
  if (T > 0 && (!x || !ids || !w || !y)) return fail(ESCHA_E_NULL, "x/topk_ids/topk_w/y is NULL");
  return ESCHA_OK;
}


// ---------------------------------------------------------------- stack
// Control block at the start of a stack workspace: a 512-int header (word 1:
// status of the one-launch path; word 2: its call number; words 256 + 32x:
// XCD x's task ticket) and that path's flag words, one per (layer, pair,
// down output block). The tickets and flags are zeroed before every launch;
// each group of flag words that one XCD writes starts on a 128-byte line of
// its own.
constexpr int64_t kCtlHeaderInts = 512;

int64_t round32(int64_t n) { return (n + 31) / 32 * 32; }

struct FlowLayout {
  int64_t p8, df_pair;
  int64_t dflag, ctl_ints;  // offset / total, in ints
  size_t gu_part, dn_part, dn_copy, ycb, sscb, data_bytes;  // offsets in bytes from the data start
};

FlowLayout flow_layout(const escha_moe_layer_t* L, int64_t n_layers, int64_t T) {
  FlowLayout f{};
  const int64_t H = L->hidden, I = L->inter;
  f.p8 = (T * L->top_k + 7) / 8 * 8;
  f.df_pair = round32(H / 128);
  f.dflag = kCtlHeaderInts;
  f.ctl_ints = f.dflag + n_layers * f.p8 * f.df_pair;
  f.dn_copy = (size_t)f.p8 * H;
  size_t off = 0;
  f.gu_part = off;
  off += round_up((size_t)f.p8 * (H / 512) * (2 * I) * sizeof(uint64_t));
  f.dn_part = off;
  off += round_up(2 * f.dn_copy * sizeof(uint64_t));
  f.ycb = off;
  off += round_up((size_t)T * 8 * H * sizeof(uint64_t));
  f.sscb = off;
  off += round_up((size_t)T * 8 * 32 * sizeof(uint64_t));
  f.data_bytes = off;
  return f;
}

size_t stack_ctl_bytes(const escha_moe_layer_t* L, int64_t n_layers, int64_t T) {
  return round_up((size_t)flow_layout(L, n_layers, T).ctl_ints * sizeof(int32_t));
}

// The layer with the most experts (the grouped workspace is sized for it).
const escha_moe_layer_t* widest_layer(const escha_moe_layer_t* layers, int32_t n_layers) {
  const escha_moe_layer_t* w = &layers[0];
  for (int l = 1; l < n_layers; ++l)
    if (layers[l].gate_up.n_experts > w->gate_up.n_experts) w = &layers[l];
  return w;
}

// Buffers of the layer-by-layer stack path after the control block: the
// streaming kernels' workspace, or (at least kGroupedDecodeTokens tokens)
// the grouped kernels' plus two bf16 layer inputs; the fp32 layer output
// follows.
size_t stack_layered_bytes(const escha_moe_layer_t* layers, int32_t n_layers, int64_t T) {
  size_t a = decode_ws_bytes(&layers[0], T);
  if (T >= kGroupedDecodeTokens) {
    const size_t g = grouped_ws(widest_layer(layers, n_layers), T, nullptr, nullptr, n_layers) +
                     2 * round_up((size_t)T * layers[0].hidden * sizeof(uint16_t));
    if (g > a) a = g;
  }
  return a;
}

int check_stack_call(const escha_moe_layer_t* layers, int32_t n_layers, const uint16_t* x0_bf16,
                     int32_t n_tokens, const int32_t* topk_ids, const float* topk_w, float eps,
                     const float* y_last, const void* workspace, size_t workspace_bytes) {
  if (!layers) return fail(ESCHA_E_NULL, "layers is NULL");
  if (n_layers < 1) return fail(ESCHA_E_ARG, "n_layers=%d", n_layers);
  for (int l = 0; l < n_layers; ++l) {
    int rc = check_layer_call(&layers[l], x0_bf16, n_tokens, topk_ids, topk_w, y_last);
    if (rc) return rc;
    if (layers[l].hidden != layers[0].hidden || layers[l].inter != layers[0].inter ||
        layers[l].top_k != layers[0].top_k)
      return fail(ESCHA_E_SHAPE, "layer %d differs from layer 0 in hidden/inter/top_k", l);
  }
  if (!(eps >= 0.f)) return fail(ESCHA_E_ARG, "eps must be >= 0");
  if (n_tokens == 0) return ESCHA_OK;
  const size_t need = escha_moe_stack_workspace_bytes(layers, n_layers, n_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  return ESCHA_OK;
}

// One projection of one expert through the streaming kernels (validated
// arguments), plus an optional output bias.
int expert_gemv_call(const escha_proj_t* w, int32_t expert, const uint16_t* x_bf16, int32_t n_tokens,
                     float* y, void* workspace, const float* bias, hipStream_t s) {
  escha::InPartialArgs a{};
  a.code = (const uint16_t*)w->code;
  a.rin = (const uint16_t*)w->rin;
  a.rout = (const uint16_t*)w->rout;
  a.n_experts = w->n_experts;
  a.in_f = w->in_features;
  a.out_f = w->out_features;
  a.n_pairs = n_tokens;
  a.top_k = 1;
  a.ids = nullptr;
  a.fixed_expert = expert;
  a.x_bf16 = x_bf16;
  a.partial = (float*)workspace;
  hipError_t e = escha::launch_in_partial(a, w->k_bits, s);
  if (e != hipSuccess) return hip_fail(e, "expert_gemv partial launch");
  escha::FinishArgs f{};
  f.partial = (const float*)workspace;
  f.n_chunks = w->in_features / 128;
  f.out_f = w->out_features;
  f.n_pairs = n_tokens;
  f.y = y;
  f.bias = bias;
  e = escha::launch_proj_finish(f, s);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "expert_gemv finish launch");
}

// ---------------------------------------------------------------- dense

// The one-expert layer of a dense MLP, or an error.
int dense_layer(const escha_dense_mlp_t* M, escha_moe_layer_t* L) {
  if (!M) return fail(ESCHA_E_NULL, "dense MLP descriptor is NULL");
  if (M->gate_up.n_experts != 1 || M->down.n_experts != 1)
    return fail(ESCHA_E_SHAPE, "dense MLP: n_experts must be 1 (gate_up %d, down %d)", M->gate_up.n_experts,
                M->down.n_experts);
  *L = escha_moe_layer_t{M->gate_up, M->down, M->hidden, M->inter, 1};
  return check_layer(L);
}

size_t dense_route_bytes(int64_t T) { return 2 * round_up((size_t)T * sizeof(int32_t)); }

int dense_mlp_call(const escha_dense_mlp_t* M, const uint16_t* x_bf16, int32_t n_tokens, float* y,
                   float* inter_out, void* workspace, size_t workspace_bytes, void* stream,
                   bool prefill) {
  escha_moe_layer_t L;
  int rc = dense_layer(M, &L);
  if (rc) return rc;
  if (n_tokens < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", n_tokens);
  if (n_tokens == 0) return ESCHA_OK;
  if (!x_bf16 || !y) return fail(ESCHA_E_NULL, "x/y is NULL");
  const size_t need = escha_dense_mlp_workspace_bytes(M, n_tokens, prefill ? 1 : 0);
  if (!workspace || workspace_bytes < need)
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  // the routing of the one-expert case (id 0, weight 1) at the workspace's start
  int32_t* ids = (int32_t*)workspace;
  float* w = (float*)((char*)workspace + round_up((size_t)n_tokens * sizeof(int32_t)));
  void* rest = (char*)workspace + dense_route_bytes(n_tokens);
  hipError_t e = escha::launch_fill_one_expert(ids, w, n_tokens, s);
  if (e != hipSuccess) return hip_fail(e, "routing fill launch");
  if (prefill || n_tokens >= kGroupedDecodeTokens) {
    GroupedWs g;
    grouped_ws(&L, n_tokens, rest, &g);
    return run_layer_grouped(&L, x_bf16, n_tokens, ids, w, y, inter_out, g, prefill, s, false, true, true,
                             M->gate_up_bias, M->down_bias);
  }
  const DecodeWs ws = decode_ws_carve(&L, n_tokens, rest);
  const LayerInput in{x_bf16, nullptr, nullptr, 0.f, nullptr};
  return run_layer_decode(&L, in, n_tokens, ids, w, y, inter_out, ws, s, nullptr, nullptr,
                          M->gate_up_bias, M->down_bias);
}

}  // namespace

extern "C" {

const char* escha_last_error(void) { return g_err; }

int escha_probe_events_set(void* const* events, int32_t n_events) {
  if (!events || n_events == 0) {
    g_proj_probe[0] = g_proj_probe[1] = nullptr;
    return ESCHA_OK;
  }
  if (n_events != 2) return fail(ESCHA_E_ARG, "n_events=%d, must be 0 or 2", n_events);
  if (!events[0] || !events[1]) return fail(ESCHA_E_NULL, "a probe event is NULL");
  g_proj_probe[0] = (hipEvent_t)events[0];
  g_proj_probe[1] = (hipEvent_t)events[1];
  return ESCHA_OK;
}

int escha_decode_tiles(const escha_proj_t* w, int32_t expert, uint16_t* w_f16, void* stream) {
  int rc = check_proj(w, "decode_tiles");
  if (rc) return rc;
  if (expert < 0 || expert >= w->n_experts)
    return fail(ESCHA_E_ARG, "expert=%d out of [0, %d)", expert, w->n_experts);
  if (!w_f16) return fail(ESCHA_E_NULL, "w_f16 is NULL");
  if (!aligned(w_f16, 8)) return fail(ESCHA_E_ARG, "w_f16 is not 8-byte aligned");
  const size_t per_expert = (size_t)(w->in_features / 16) * (w->out_features / 16) * 16 * w->k_bits;
  const uint16_t* code_e = (const uint16_t*)w->code + (size_t)expert * per_expert;
  hipError_t e = escha::launch_decode_tiles(code_e, w->in_features, w->out_features, w->k_bits,
                                            w_f16, (hipStream_t)stream);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "decode_tiles launch");
}

int escha_decode_tiles_layout(const escha_proj_t* w, int32_t expert, int32_t layout, uint16_t* w_f16,
                              void* stream) {
  if (layout == ESCHA_LAYOUT_QUARTER) return escha_decode_tiles(w, expert, w_f16, stream);
  int rc = check_proj(w, "decode_tiles_layout");
  if (rc) return rc;
  if (layout != ESCHA_LAYOUT_MFMA_OPERAND && layout != ESCHA_LAYOUT_LDS_TILE &&
      layout != ESCHA_LAYOUT_MFMA_PAIRS && layout != ESCHA_LAYOUT_MFMA_TILE_PAIRS)
    return fail(ESCHA_E_ARG, "layout=%d is not one of the ESCHA_LAYOUT_* values", layout);
  if ((layout == ESCHA_LAYOUT_MFMA_PAIRS || layout == ESCHA_LAYOUT_MFMA_TILE_PAIRS) && w->k_bits != 2)
    return fail(ESCHA_E_ARG, "the column-pair layouts decode K=2 codes only (K=%d)", w->k_bits);
  if (expert < 0 || expert >= w->n_experts)
    return fail(ESCHA_E_ARG, "expert=%d out of [0, %d)", expert, w->n_experts);
  if (!w_f16) return fail(ESCHA_E_NULL, "w_f16 is NULL");
  if (!aligned(w_f16, 16)) return fail(ESCHA_E_ARG, "w_f16 is not 16-byte aligned");
  const size_t per_expert = (size_t)(w->in_features / 16) * (w->out_features / 16) * 16 * w->k_bits;
  const uint16_t* code_e = (const uint16_t*)w->code + (size_t)expert * per_expert;
  hipError_t e = escha::launch_decode_operands(code_e, w->in_features, w->out_features, w->k_bits, layout,
                                               w_f16, (hipStream_t)stream);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "decode_tiles_layout launch");
}

int escha_hadamard128(const float* x, int64_t rows, int32_t n, float* y, void* stream) {
  if (rows < 0 || n < 128 || n % 128) return fail(ESCHA_E_SHAPE, "rows=%lld n=%d", (long long)rows, n);
  if (rows == 0) return ESCHA_OK;
  if (!x || !y) return fail(ESCHA_E_NULL, "x/y is NULL");
  hipError_t e = escha::launch_hadamard128(x, rows, n, y, (hipStream_t)stream);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "hadamard128 launch");
}

int escha_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                     int32_t* topk_ids, float* topk_w, void* stream) {
  if (n_tokens < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", n_tokens);
  if (n_experts < 1 || n_experts > kMaxExpertsRoute)
    return fail(ESCHA_E_ARG, "n_experts=%d out of [1, %d]", n_experts, kMaxExpertsRoute);
  if (top_k < 1 || top_k > 32 || top_k > n_experts) return fail(ESCHA_E_ARG, "top_k=%d", top_k);
  if (n_tokens == 0) return ESCHA_OK;
  if (!logits || !topk_ids || !topk_w) return fail(ESCHA_E_NULL, "logits/topk_ids/topk_w is NULL");
  hipError_t e = escha::launch_route_topk(logits, n_tokens, n_experts, top_k, topk_ids, topk_w,
                                          (hipStream_t)stream);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "route_topk launch");
}

size_t escha_router_workspace_bytes(int32_t n_tokens, int32_t hidden, int32_t n_experts) {
  if (n_tokens <= 0 || hidden < 32 || hidden % 32 || n_experts < 1 || n_experts > kMaxExpertsRoute)
    return 0;
  const int ks = escha::router_ksplit(n_tokens, hidden, n_experts);
  return ks > 1 ? round_up((size_t)ks * n_tokens * n_experts * sizeof(float)) : 0;
}

int escha_router_logits(const uint16_t* x_bf16, int32_t n_tokens, int32_t hidden,
                        const uint16_t* gate_f16, int32_t n_experts, float* logits, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (n_tokens < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", n_tokens);
  if (hidden < 32 || hidden % 32) return fail(ESCHA_E_SHAPE, "hidden=%d is not a positive multiple of 32", hidden);
  if (n_experts < 1 || n_experts > kMaxExpertsRoute)
    return fail(ESCHA_E_ARG, "n_experts=%d out of [1, %d]", n_experts, kMaxExpertsRoute);
  if (n_tokens == 0) return ESCHA_OK;
  if (!x_bf16 || !gate_f16 || !logits) return fail(ESCHA_E_NULL, "x_bf16/gate_f16/logits is NULL");
  if (!aligned(x_bf16, 16) || !aligned(gate_f16, 16))
    return fail(ESCHA_E_ARG, "x_bf16/gate_f16 is not 16-byte aligned");
  const size_t need = escha_router_workspace_bytes(n_tokens, hidden, n_experts);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(ESCHA_E_WORKSPACE, "workspace %zu bytes < %zu", workspace ? workspace_bytes : 0, need);
  escha::RouterArgs a;
  a.x = x_bf16;
  a.gate = gate_f16;
  a.T = n_tokens;
  a.H = hidden;
  a.E = n_experts;
  a.ksplit = escha::router_ksplit(n_tokens, hidden, n_experts);
  a.logits = logits;
  a.part = (float*)workspace;
  hipError_t e = escha::launch_router_logits(a, (hipStream_t)stream);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "router_logits launch");
}

size_t escha_moe_group_workspace_bytes(int32_t n_tokens, int32_t top_k, int32_t n_experts) {
  if (n_tokens < 0 || top_k < 1 || n_experts < 1) return 0;
  const size_t P = (size_t)n_tokens * top_k;
  const size_t chunks = (P + 63) / 64;
  return 2 * round_up(chunks * n_experts * sizeof(int32_t)) + round_up(P * sizeof(int32_t)) + 256;
}

int escha_moe_group(const int32_t* topk_ids, int32_t n_tokens, int32_t top_k, int32_t n_experts,
                    int32_t* counts, int32_t* offsets, int32_t* perm, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (n_tokens < 0 || top_k < 1 || n_experts < 1 || n_experts > kMaxExpertsRoute)
    return fail(ESCHA_E_ARG, "n_tokens=%d top_k=%d n_experts=%d", n_tokens, top_k, n_experts);
  if ((int64_t)n_tokens * top_k > (int64_t)1 << 30) return fail(ESCHA_E_ARG, "too many pairs");
  if (!counts || !offsets) return fail(ESCHA_E_NULL, "counts/offsets is NULL");
  const int P = n_tokens * top_k;
  if (P > 0 && (!topk_ids || !perm)) return fail(ESCHA_E_NULL, "topk_ids/perm is NULL");
  const size_t need = escha_moe_group_workspace_bytes(n_tokens, top_k, n_experts);
  if (workspace_bytes < need || (!workspace && need))
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  const size_t chunks = ((size_t)P + 63) / 64;
  char* b = (char*)workspace;
  int32_t* hist = (int32_t*)b;
  int32_t* base = (int32_t*)(b + round_up(chunks * n_experts * sizeof(int32_t)));
  int32_t* rank = (int32_t*)(b + 2 * round_up(chunks * n_experts * sizeof(int32_t)));
  hipError_t e = escha::group_small_ok(P, n_experts)
                     ? escha::launch_group_small(topk_ids, P, n_experts, counts, offsets, perm, nullptr,
                                                 0, 0, nullptr, nullptr, nullptr, nullptr,
                                                 (hipStream_t)stream)
                     : escha::launch_group(topk_ids, P, n_experts, counts, offsets, perm, nullptr,
                                           hist, base, rank, (hipStream_t)stream);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "group launch");
}

size_t escha_expert_gemv_workspace_bytes(const escha_proj_t* w, int32_t n_tokens) {
  if (!w || n_tokens < 0 || w->in_features < 128 || w->out_features < 256) return 0;
  return round_up((size_t)n_tokens * (w->in_features / 128) * w->out_features * sizeof(float));
}

int escha_expert_gemv(const escha_proj_t* w, int32_t expert, const uint16_t* x_bf16,
                      int32_t n_tokens, float* y, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int rc = check_proj(w, "expert_gemv");
  if (rc) return rc;
  if (expert < 0 || expert >= w->n_experts)
    return fail(ESCHA_E_ARG, "expert=%d out of [0, %d)", expert, w->n_experts);
  if (n_tokens < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", n_tokens);
  if (n_tokens == 0) return ESCHA_OK;
  if (!x_bf16 || !y) return fail(ESCHA_E_NULL, "x/y is NULL");
  const size_t need = escha_expert_gemv_workspace_bytes(w, n_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  return expert_gemv_call(w, expert, x_bf16, n_tokens, y, workspace, nullptr, (hipStream_t)stream);
}



size_t escha_moe_workspace_bytes(const escha_moe_layer_t* L, int32_t n_tokens, int32_t prefill) {
  if (!L || n_tokens < 0 || L->top_k < 1 || L->hidden < 128 || L->inter < 128) return 0;
  if (prefill || n_tokens >= kGroupedDecodeTokens) return grouped_ws(L, n_tokens, nullptr, nullptr);
  return decode_ws_bytes(L, n_tokens);
}

int escha_moe_layer_decode(const escha_moe_layer_t* L, const uint16_t* x_bf16, int32_t n_tokens,
                           const int32_t* topk_ids, const float* topk_w, float* y,
                           float* inter_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int rc = check_layer_call(L, x_bf16, n_tokens, topk_ids, topk_w, y);
  if (rc) return rc;
  if (n_tokens == 0) return ESCHA_OK;
  const size_t need = escha_moe_workspace_bytes(L, n_tokens, 0);
  if (!workspace || workspace_bytes < need)
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (n_tokens >= kGroupedDecodeTokens) {
    GroupedWs g;
    grouped_ws(L, n_tokens, workspace, &g);
    return run_layer_grouped(L, x_bf16, n_tokens, topk_ids, topk_w, y, inter_out, g, false,
                             (hipStream_t)stream);
  }
  const DecodeWs ws = decode_ws_carve(L, n_tokens, workspace);
  const LayerInput in{x_bf16, nullptr, nullptr, 0.f, nullptr};
  return run_layer_decode(L, in, n_tokens, topk_ids, topk_w, y, inter_out, ws,
                          (hipStream_t)stream);
}

int escha_moe_layer_decode_logits(const escha_moe_layer_t* L, const uint16_t* x_bf16, int32_t n_tokens,
                                  const float* logits, int32_t* topk_ids, float* topk_w, float* y,
                                  float* inter_out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (n_tokens < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", n_tokens);
  if (n_tokens == 0) return ESCHA_OK;
  if (!x_bf16 || !logits || !topk_ids || !topk_w || !y)
    return fail(ESCHA_E_NULL, "x/logits/topk_ids/topk_w/y is NULL");
  if (L->top_k > 32) return fail(ESCHA_E_ARG, "top_k=%d > 32", L->top_k);
  const size_t need = escha_moe_workspace_bytes(L, n_tokens, 0);
  if (!workspace || workspace_bytes < need)
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  const int E = L->gate_up.n_experts;
  const escha::RouteOut route{logits, L->top_k, topk_ids, topk_w};
  // the router step inside the streaming gate_up kernel (below 16 tokens,
  // up to 256 experts and 8 slots); otherwise a kernel of its own first
  const bool fusable = n_tokens < kGroupedDecodeTokens && E <= 64 * escha::kRouteFusedPer && L->top_k <= 8;
  if (!fusable) {
    hipError_t e = escha::launch_route_topk(logits, n_tokens, E, L->top_k, topk_ids, topk_w, s);
    if (e != hipSuccess) return hip_fail(e, "route_topk launch");
  }
  if (n_tokens >= kGroupedDecodeTokens) {
    GroupedWs g;
    grouped_ws(L, n_tokens, workspace, &g);
    return run_layer_grouped(L, x_bf16, n_tokens, topk_ids, topk_w, y, inter_out, g, false, s);
  }
  const DecodeWs ws = decode_ws_carve(L, n_tokens, workspace);
  const LayerInput in{x_bf16, nullptr, nullptr, 0.f, nullptr};
  return run_layer_decode(L, in, n_tokens, topk_ids, topk_w, y, inter_out, ws, s, nullptr, nullptr, nullptr,
                          nullptr, fusable ? &route : nullptr);
}

int escha_moe_layer_decode_static(const escha_moe_layer_t* L, const uint16_t* x_bf16, int32_t n_tokens,
                                  const int32_t* topk_ids, const float* topk_w, float* y,
                                  float* inter_out, void* stream) {
  int rc = check_layer_call(L, x_bf16, n_tokens, topk_ids, topk_w, y);
  if (rc) return rc;
  if (n_tokens == 0) return ESCHA_OK;
  const size_t need = escha_moe_workspace_bytes(L, n_tokens, 0);
  if (need > escha::kStaticScratchBytes)
    return fail(ESCHA_E_WORKSPACE,
                "decode_static: %d tokens need %zu bytes of scratch, more than the library's "
                "%zu-byte array (call escha_moe_layer_decode with a workspace instead)",
                n_tokens, need, escha::kStaticScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = escha::static_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "static scratch address");
  // the same kernels, in the same order, as escha_moe_layer_decode with this
  // scratch as its workspace (nothing in it needs to start at zero)
  return escha_moe_layer_decode(L, x_bf16, n_tokens, topk_ids, topk_w, y, inter_out, scratch,
                                escha::kStaticScratchBytes, stream);
}

int escha_moe_layer_prefill(const escha_moe_layer_t* L, const uint16_t* x_bf16, int32_t n_tokens,
                            const int32_t* topk_ids, const float* topk_w, float* y,
                            float* inter_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  int rc = check_layer_call(L, x_bf16, n_tokens, topk_ids, topk_w, y);
  if (rc) return rc;
  if (n_tokens == 0) return ESCHA_OK;
  const size_t need = escha_moe_workspace_bytes(L, n_tokens, 1);
  if (!workspace || workspace_bytes < need)
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  GroupedWs g;
  grouped_ws(L, n_tokens, workspace, &g);
  return run_layer_grouped(L, x_bf16, n_tokens, topk_ids, topk_w, y, inter_out, g, true,
                           (hipStream_t)stream);
}

size_t escha_dense_mlp_workspace_bytes(const escha_dense_mlp_t* M, int32_t n_tokens, int32_t prefill) {
  if (!M || n_tokens < 0) return 0;
  const escha_moe_layer_t L{M->gate_up, M->down, M->hidden, M->inter, 1};
  return dense_route_bytes(n_tokens) + escha_moe_workspace_bytes(&L, n_tokens, prefill);
}

int escha_dense_mlp_decode(const escha_dense_mlp_t* M, const uint16_t* x_bf16, int32_t n_tokens, float* y,
                           float* inter_out, void* workspace, size_t workspace_bytes, void* stream) {
  return dense_mlp_call(M, x_bf16, n_tokens, y, inter_out, workspace, workspace_bytes, stream, false);
}

int escha_dense_mlp_prefill(const escha_dense_mlp_t* M, const uint16_t* x_bf16, int32_t n_tokens, float* y,
                            float* inter_out, void* workspace, size_t workspace_bytes, void* stream) {
  return dense_mlp_call(M, x_bf16, n_tokens, y, inter_out, workspace, workspace_bytes, stream, true);
}

int escha_dense_gemv(const escha_proj_t* w, const float* bias, const uint16_t* x_bf16, int32_t n_tokens,
                     float* y, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_proj(w, "dense_gemv");
  if (rc) return rc;
  if (w->n_experts != 1) return fail(ESCHA_E_SHAPE, "dense_gemv: n_experts=%d, must be 1", w->n_experts);
  if (n_tokens < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", n_tokens);
  if (n_tokens == 0) return ESCHA_OK;
  if (!x_bf16 || !y) return fail(ESCHA_E_NULL, "x/y is NULL");
  const size_t need = escha_expert_gemv_workspace_bytes(w, n_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  return expert_gemv_call(w, 0, x_bf16, n_tokens, y, workspace, bias, (hipStream_t)stream);
}

size_t escha_shared_expert_workspace_bytes(const escha_shared_expert_t* S, int32_t n_tokens) {
  if (!S || n_tokens < 0 || S->inter <= 0) return 0;
  return round_up((size_t)n_tokens * S->inter * sizeof(float)) + round_up((size_t)n_tokens * sizeof(float));
}

int escha_shared_expert(const escha_shared_expert_t* S, const uint16_t* x_bf16, int32_t n_tokens,
                        float* y, int32_t accumulate, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!S) return fail(ESCHA_E_NULL, "shared expert descriptor is NULL");
  if (!S->gate_up || !S->gate_up_scale || !S->down || !S->down_scale || !S->gate)
    return fail(ESCHA_E_NULL, "shared expert: a weight, scale or gate pointer is NULL");
  const int H = S->hidden, I = S->inter;
  if (H < 1024 || H % 1024 || H > escha::kShMaxHidden)
    return fail(ESCHA_E_SHAPE, "shared expert: hidden=%d is not a multiple of 1024 in [1024, %d]", H,
                escha::kShMaxHidden);
  if (I < 512 || I % 512 || I > escha::kShMaxInter)
    return fail(ESCHA_E_SHAPE, "shared expert: inter=%d is not a multiple of 512 in [512, %d]", I,
                escha::kShMaxInter);
  if (!aligned(S->gate_up, 16) || !aligned(S->down, 16) || !aligned(S->gate_up_scale, 4) ||
      !aligned(S->down_scale, 4) || !aligned(S->gate, 2))
    return fail(ESCHA_E_ARG, "shared expert: misaligned weights (int8 16 B, scales 4 B)");
  if (n_tokens < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", n_tokens);
  if (n_tokens == 0) return ESCHA_OK;
  if (!x_bf16 || !y) return fail(ESCHA_E_NULL, "x/y is NULL");
  if (!aligned(x_bf16, 16)) return fail(ESCHA_E_ARG, "x_bf16 is not 16-byte aligned");
  const size_t need = escha_shared_expert_workspace_bytes(S, n_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(ESCHA_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  escha::SharedArgs a{};
  a.gu_w = S->gate_up;
  a.gu_s = S->gate_up_scale;
  a.dn_w = S->down;
  a.dn_s = S->down_scale;
  a.gate = S->gate;
  a.hidden = H;
  a.inter = I;
  a.n_tokens = n_tokens;
  a.x = x_bf16;
  a.h = (float*)workspace;
  a.glogit = (float*)((char*)workspace + round_up((size_t)n_tokens * I * sizeof(float)));
  a.y = y;
  a.accumulate = accumulate ? 1 : 0;
  int rc = probe_proj(0, (hipStream_t)stream);
  if (rc) return rc;
  const hipError_t e = escha::launch_shared_expert(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "shared expert launch");
  return probe_proj(1, (hipStream_t)stream);
}

int escha_rmsnorm_bf16(const float* y, int32_t n_tokens, int32_t n, float eps, uint16_t* x_bf16,
                       void* stream) {
  if (n_tokens < 0) return fail(ESCHA_E_ARG, "n_tokens=%d", n_tokens);
  if (n < 128 || n % 128 || n > kMaxHidden)
    return fail(ESCHA_E_SHAPE, "n=%d is not a multiple of 128 in [128, %d]", n, kMaxHidden);
  if (!(eps >= 0.f)) return fail(ESCHA_E_ARG, "eps must be >= 0");
  if (n_tokens == 0) return ESCHA_OK;
  if (!y || !x_bf16) return fail(ESCHA_E_NULL, "y/x is NULL");
  hipError_t e = escha::launch_rmsnorm_bf16(y, n_tokens, n, eps, x_bf16, (hipStream_t)stream);
  return e == hipSuccess ? ESCHA_OK : hip_fail(e, "rmsnorm launch");
}

size_t escha_moe_stack_workspace_bytes(const escha_moe_layer_t* layers, int32_t n_layers,
                                       int32_t n_tokens) {
  if (!layers || n_layers < 1 || n_tokens < 0) return 0;
  const escha_moe_layer_t* L = &layers[0];
  // the control block, then the layer-by-layer path's buffers, then the
  // one-launch path's
  const size_t ybuf = round_up((size_t)n_tokens * L->hidden * sizeof(float));
  return stack_ctl_bytes(L, n_layers, n_tokens) + stack_layered_bytes(layers, n_layers, n_tokens) +
         ybuf + flow_layout(L, n_layers, n_tokens).data_bytes;
}

int escha_moe_stack_decode(const escha_moe_layer_t* layers, int32_t n_layers,
                           const uint16_t* x0_bf16, int32_t n_tokens, const int32_t* topk_ids,
                           const float* topk_w, float eps, float* y_last, uint16_t* x_chain,
                           void* workspace, size_t workspace_bytes, void* const* probe_events,
                           void* stream) {
  int rc = check_stack_call(layers, n_layers, x0_bf16, n_tokens, topk_ids, topk_w, eps, y_last,
                            workspace, workspace_bytes);
  if (rc || n_tokens == 0) return rc;
  const escha_moe_layer_t* L0 = &layers[0];
  const int H = L0->hidden, k = L0->top_k;
  char* b = (char*)workspace + stack_ctl_bytes(L0, n_layers, n_tokens);
  float* ytmp = (float*)(b + stack_layered_bytes(layers, n_layers, n_tokens));
  hipStream_t s = (hipStream_t)stream;
  const size_t xs = (size_t)n_tokens * H;
  if (x_chain) {
    hipError_t e =
        hipMemcpyAsync(x_chain, x0_bf16, xs * sizeof(uint16_t), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "x_chain copy");
  }
  if (n_tokens >= kGroupedDecodeTokens) {
    // grouped kernels per layer, the next layer's input by the RMSNorm
    // kernel; when every layer has the same number of experts, the pairs
    // of all layers are grouped up front (the routing is known for all)
    GroupedWs g;
    const escha_moe_layer_t* Lw = widest_layer(layers, n_layers);
    const size_t gb = grouped_ws(Lw, n_tokens, b, &g, n_layers);
    uint16_t* xbuf[2] = {(uint16_t*)(b + gb),
                         (uint16_t*)(b + gb + round_up(xs * sizeof(uint16_t)))};
    bool same_e = true;
    for (int l = 1; l < n_layers; ++l) same_e &= layers[l].gate_up.n_experts == L0->gate_up.n_experts;
    if (same_e) {
      const int rc = group_layers(L0, n_tokens, topk_ids, g, false, n_layers, s);
      if (rc) return rc;
    }
    // with the pairs grouped up front, one kernel per token links two
    // layers: combine, RMSNorm and the next layer's input gather/rotation
    const bool linked = same_e && H <= 2048;
    const uint16_t* x = x0_bf16;
    for (int l = 0; l < n_layers; ++l) {
      float* y = l == n_layers - 1 ? y_last : ytmp;
      hipError_t e;
      if (probe_events && (e = record_probe((hipEvent_t)probe_events[2 * l], s)) != hipSuccess)
        return hip_fail(e, "probe event record");
      const GroupedWs gl = same_e ? grouped_layer(g, Lw, n_tokens, l) : g;
      const bool link = linked && l + 1 < n_layers;
      int rc = run_layer_grouped(&layers[l], x, n_tokens, topk_ids + (size_t)l * n_tokens * k,
                                 topk_w + (size_t)l * n_tokens * k, y, nullptr, gl, false, s, same_e,
                                 !linked || l == 0, !link);
      if (rc) return rc;
      if (link) {
        const GroupedWs gn = grouped_layer(g, Lw, n_tokens, l + 1);
        escha::CombineNextArgs cn{};
        cn.rows = gl.yd;
        cn.inv = gl.inv;
        cn.hidden = H;
        cn.top_k = k;
        cn.n_tokens = n_tokens;
        cn.y = y;
        cn.eps = eps;
        cn.x_out = x_chain ? x_chain + (size_t)(l + 1) * xs : nullptr;
        cn.rin_next = (const uint16_t*)layers[l + 1].gate_up.rin;
        cn.ids_next = topk_ids + (size_t)(l + 1) * n_tokens * k;
        cn.inv_next = gn.inv;
        cn.xg_next = gn.xg;
        cn.xg_exp_next = gn.xg_exp;
        e = escha::launch_combine_next(cn, s);
        if (e != hipSuccess) return hip_fail(e, "combine/RMSNorm/gather launch");
      } else if (l + 1 < n_layers) {
        uint16_t* next = x_chain ? x_chain + (size_t)(l + 1) * xs : xbuf[l & 1];
        e = escha::launch_rmsnorm_bf16(y, n_tokens, H, eps, next, s);
        if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
        x = next;
      }
      if (probe_events && (e = record_probe((hipEvent_t)probe_events[2 * l + 1], s)) != hipSuccess)
        return hip_fail(e, "probe event record");
    }
    return ESCHA_OK;
  }
  const DecodeWs ws = decode_ws_carve(L0, n_tokens, b);
  for (int l = 0; l < n_layers; ++l) {
    // layer 0 reads x0; layer l > 0 reads RMSNorm(y_{l-1}) from ytmp, which
    // its own combine then overwrites with y_l (stream order)
    LayerInput in{};
    if (l == 0) {
      in.x_bf16 = x0_bf16;
    } else {
      in.y_prev = ytmp;
      in.ss_prev = ws.ss;
      in.eps = eps;
      in.x_out = x_chain ? x_chain + (size_t)l * xs : nullptr;
    }
    float* y = l == n_layers - 1 ? y_last : ytmp;
    hipEvent_t before = probe_events ? (hipEvent_t)probe_events[2 * l] : nullptr;
    hipEvent_t after = probe_events ? (hipEvent_t)probe_events[2 * l + 1] : nullptr;
    int rc = run_layer_decode(&layers[l], in, n_tokens, topk_ids + (size_t)l * n_tokens * k,
                              topk_w + (size_t)l * n_tokens * k, y, nullptr, ws, s, before, after);
    if (rc) return rc;
  }
  return ESCHA_OK;
}

int escha_moe_stack_decode_persistent(const escha_moe_layer_t* layers, int32_t n_layers,
                                      const uint16_t* x0_bf16, int32_t n_tokens,
                                      const int32_t* topk_ids, const float* topk_w, float eps,
                                      float* y_last, uint16_t* x_chain, void* workspace,
                                      size_t workspace_bytes, void* const* probe_events,
                                      void* stream) {
  int rc = check_stack_call(layers, n_layers, x0_bf16, n_tokens, topk_ids, topk_w, eps, y_last,
                            workspace, workspace_bytes);
  if (rc) return rc;
  if (n_layers > escha::kMaxStackLayers)
    return fail(ESCHA_E_UNSUPPORTED, "n_layers=%d > %d", n_layers, escha::kMaxStackLayers);
  if (n_tokens > kMaxStackTokens)
    return fail(ESCHA_E_UNSUPPORTED, "n_tokens=%d > %d", n_tokens, kMaxStackTokens);
  const escha_moe_layer_t* L0 = &layers[0];
  for (int l = 1; l < n_layers; ++l) {
    const escha_moe_layer_t* L = &layers[l];
    if (L->gate_up.n_experts != L0->gate_up.n_experts || L->gate_up.k_bits != L0->gate_up.k_bits ||
        L->down.k_bits != L0->down.k_bits)
      return fail(ESCHA_E_UNSUPPORTED,
                  "layer %d differs from layer 0 in n_experts or k_bits (one-launch path)", l);
  }
  const int64_t T = n_tokens, H = L0->hidden, I = L0->inter, k = L0->top_k;
  // task shapes of the one-launch kernel: gate_up tasks over 1024 inputs (two
  // parts at most), one down task over all channels (at most four
  // 128-blocks), one wave polling all the flags a task waits for
  if (H % 1024 != 0 || H > 2048 || I > 512 || k * (H / 256) > 64)
    return fail(ESCHA_E_UNSUPPORTED,
                "one-launch path needs hidden 1024 or 2048, inter <= 512 and "
                "top_k * hidden / 256 <= 64 (hidden=%lld inter=%lld top_k=%lld)",
                (long long)H, (long long)I, (long long)k);
  if (n_tokens == 0) return ESCHA_OK;
  // Small batches fold the combine into the down tasks, whose waits on each
  // other are deadlock-free only while one layer's down tasks of one XCD
  // can all be resident at once.
  int dev = 0, n_cu = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  // the 4-wave form between kFlowWideTokens and kFlowWideMaxTokens tokens;
  // otherwise from kFlowLateTokens tokens the tasks decode after their wait
  const bool wide = k <= 8 && n_tokens >= kFlowWideTokens && n_tokens <= kFlowWideMaxTokens;
  const bool late = !wide && n_tokens >= kFlowLateTokens;
  if (e == hipSuccess)
    e = escha::flow_groups_per_cu(L0->gate_up.k_bits, L0->down.k_bits, late, wide, &per_cu);
  if (e != hipSuccess) return hip_fail(e, "device query");
  const int64_t p8 = (T * k + 7) / 8 * 8;
  const bool fold = k <= 8 && (p8 / 8) * (H / 128) <= (int64_t)(n_cu / 8) * per_cu;
  const int64_t blocks =
      escha::flow_blocks_per_layer((int)H, (int)I, (int)k, (int)T, fold) * n_layers;
  if (blocks + escha::kFlowSpare > 0x7FFFFFFF)
    return fail(ESCHA_E_UNSUPPORTED, "%lld work-groups exceed one grid", (long long)blocks);

  hipStream_t s = (hipStream_t)stream;
  const FlowLayout f = flow_layout(L0, n_layers, T);
  int32_t* ctl = (int32_t*)workspace;
  char* data = (char*)workspace + stack_ctl_bytes(L0, n_layers, T) +
               stack_layered_bytes(layers, n_layers, T) + round_up((size_t)T * H * sizeof(float));

  escha::FlowArgs a{};
  for (int l = 0; l < n_layers; ++l) {
    a.layer[l].gu_code = (const uint16_t*)layers[l].gate_up.code;
    a.layer[l].gu_rin = (const uint16_t*)layers[l].gate_up.rin;
    a.layer[l].gu_rout = (const uint16_t*)layers[l].gate_up.rout;
    a.layer[l].dn_code = (const uint16_t*)layers[l].down.code;
    a.layer[l].dn_rin = (const uint16_t*)layers[l].down.rin;
    a.layer[l].dn_rout = (const uint16_t*)layers[l].down.rout;
  }
  a.n_layers = n_layers;
  a.n_tokens = n_tokens;
  a.top_k = (int32_t)k;
  a.hidden = (int32_t)H;
  a.inter = (int32_t)I;
  a.n_experts = L0->gate_up.n_experts;
  a.p8 = (int32_t)f.p8;
  a.eps = eps;
  a.ids = topk_ids;
  a.w = topk_w;
  a.x0 = x0_bf16;
  a.y_last = y_last;
  a.x_chain = x_chain;
  a.gu_part = (uint64_t*)(data + f.gu_part);
  a.dn_part = (uint64_t*)(data + f.dn_part);
  a.dn_copy = (int64_t)f.dn_copy;
  a.ycb = (uint64_t*)(data + f.ycb);
  a.sscb = (uint64_t*)(data + f.sscb);
  a.dflag = ctl + f.dflag;
  a.df_pair = (int32_t)f.df_pair;
  a.epoch = ctl + 2;
  a.ticket = ctl + 256;
  a.error = ctl + 1;
  a.fold = fold ? 1 : 0;
  a.late = late ? 1 : 0;
  a.wide = wide ? 1 : 0;

  // status, tickets and flags to zero, the call number one further
  e = escha::launch_flow_prepare(ctl, (size_t)f.ctl_ints, s);
  if (e != hipSuccess) return hip_fail(e, "flag clear launch");
  if (probe_events && (e = record_probe((hipEvent_t)probe_events[0], s)) != hipSuccess)
    return hip_fail(e, "probe event record");
  e = escha::launch_stack_flow(a, L0->gate_up.k_bits, L0->down.k_bits, s);
  if (e != hipSuccess) return hip_fail(e, "one-launch stack launch");
  if (probe_events && (e = record_probe((hipEvent_t)probe_events[1], s)) != hipSuccess)
    return hip_fail(e, "probe event record");
  return ESCHA_OK;
}

int escha_moe_stack_status(const void* workspace, int32_t* status, void* stream) {
  if (!workspace || !status) return fail(ESCHA_E_NULL, "workspace/status is NULL");
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, (const int32_t*)workspace + 1, sizeof(v), hipMemcpyDeviceToHost,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "status copy");
  e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "status copy");
  *status = v;
  return ESCHA_OK;
}

}  // extern "C"
