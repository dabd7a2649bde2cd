// escha_stack.hip -- decode of a whole stack of MoE layers in one launch
// (small batches: the token-by-token generation case).
//
// Every task of every layer is one work-group (8 waves, or 4 in the wide
// form; two or three work-groups share a compute unit), and the tasks are
// numbered in dependency order:
// layer by layer, first the layer's gate_up tasks, then its down tasks, then
// (larger batches only) its combine tasks.
//   gate_up (pair p, part hh = four 128-input chunks, 128-output block g):
//     the rotated inputs of the four chunks, the decode of their 32
//     tile-rows x 8 tiles (32 tiles per wave), the sum over the chunks and
//     the output transform of that sum;
//   down (p, 128-output block g): h = SiLU(gate) * up over all the
//     intermediate channels from gate_up's part sums, its rotation (one
//     128-block per chunk), the decode of every tile-row of the block, the
//     sum over the channels and the output transform, weighted by the
//     router probability: the pair's finished output for the block. For
//     small batches the down task then also combines: it adds the block's
//     outputs of all the token's pairs (its own included) once they carry
//     this layer's tag, and stores the sum and its sum of squares for the
//     next layer's gate_up tasks on its XCD;
//   combine (token t, XCD x, four 128-output blocks; larger batches): the
//     same sum for XCD x as a task of its own, once the down tasks flag.
// The arithmetic per projection is the method's (rin, H_n, the decoded
// weights with fp32 accumulation, H_n, rout); the summation order differs
// from the layer-by-layer kernels (here each task sums over more inputs
// before the transform), so the two paths agree to rounding, not bit for
// bit.
//
// A work-group first issues the loads of its codes and decodes them into
// registers -- none of which depends on other tasks -- and only then waits
// for the tasks whose outputs it reads. Work-groups start in index order
// (per XCD), and every wait is on a task with a smaller number, so the
// smallest unfinished task can always run; the device holds as many later
// work-groups as fit, and their decode overlaps the dependency chain of the
// earlier ones. The down tasks that combine also wait on down tasks of the
// same layer with larger numbers: the host enables that only when all of
// one layer's down tasks of one XCD fit on the XCD at once, which keeps
// the argument. Every wait is bounded all the same (by the constant 100 MHz
// clock): when one gives up it sets the error word, and every work-group
// leaves at its next wait.
//
// Placement. Every XCD of the device has its own L2. Tasks are numbered so
// that task i belongs to XCD i % 8 and all the tasks of pair p to XCD p % 8:
// gate_up -> down exchanges stay inside one L2. A work-group reads the XCD
// it runs on and claims that XCD's next task from a per-XCD ticket counter;
// work-groups are dealt to the XCDs round-robin, so each XCD receives as
// many work-groups as the grid's share (the grid has 8 per XCD to spare, and
// a surplus work-group finds no task and leaves). The claim order on an XCD
// is the order its work-groups start, which keeps the argument above. On this
// device, a plain store lands in the storing XCD's L2 and a load with the
// sc1 cache policy reads through the compute unit's cache to that L2 (or to
// memory), so inside one XCD a plain store followed by an sc1 load is a
// complete hand-off; a store with sc1 writes through to memory, which every
// XCD's sc1 loads see. The pair outputs of down and their flags cross XCDs
// (sc1 stores); everything else is XCD-local (plain stores). Every load of
// data written during the launch uses sc1.
//
// Buffers written during the launch and read by other work-groups are
// reused from layer to layer where the dependency chain makes that safe (a
// task that overwrites one waits, directly or transitively, for every task
// that reads the previous contents); the pair outputs, which the combining
// tasks of all XCDs read, alternate between two copies by layer parity.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "escha_device.hpp"
#include "escha_launch.hpp"
#include "escha_mfma.hpp"
#include "escha_stream.hpp"

namespace escha {

namespace {

constexpr long long kWaitTicks = 50000000;  // 0.5 s of the 100 MHz clock: a wait's bound

__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xF;  // HW_REG_XCC_ID, bits 3:0
}

// sc1 load: reads what other work-groups stored during this launch.
__device__ __forceinline__ int ld_fresh(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// sc1 store: written through to memory, for readers on other XCDs.
__device__ __forceinline__ void st_remote(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Tagged words: data that work-groups hand to each other is stored as a
// 64-bit word {value bits, tag} with one store, so a reader sees a value
// together with the tag written with it; the tag names the call and the
// layer, so a reader recognises the word the current layer's producer
// stored without any flag or store completion in between.
__device__ __forceinline__ uint64_t tag_word(float v, uint32_t tag) {
  return (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
}
__device__ __forceinline__ uint64_t ld_fresh64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_remote64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bound of every wait: true while the wait may go on; false once the error
// word is set or the bound has passed (then this wave sets the error word).
__device__ __forceinline__ bool keep_waiting(int it, long long t0, int32_t* err) {
  if ((it & 15) == 15) {
    if (ld_fresh(err)) return false;
    if (wall_clock64() - t0 > kWaitTicks) {
      st_remote(err, 1);
      return false;
    }
  }
  __builtin_amdgcn_s_sleep(2);
  return true;
}

// Wave-level fetch of N tagged words per lane (word i at p(i); words i >=
// n are not read) until every word the wave reads carries `tag`; out[i]
// receives the values. False when a wait gives up. Whole wave.
template <int N, class F>
__device__ bool wave_fetch(F p, int n, uint32_t tag, float (&out)[N], int32_t* err) {
  const long long t0 = wall_clock64();
  for (int it = 0;; ++it) {
    uint64_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = i < n ? ld_fresh64(p(i)) : tag_word(0.f, tag);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && (uint32_t)(v[i] >> 32) == tag;
    if (__ballot(!ok) == 0) {
#pragma unroll
      for (int i = 0; i < N; ++i) out[i] = __uint_as_float((uint32_t)v[i]);
      return true;
    }
    if (!keep_waiting(it, t0, err)) return false;
  }
}

// Wave-level fetch of up to two groups of four tagged words per lane (word
// 4j + c at p(4j + c), groups j < n), added in group order to `start` once
// every word the wave reads carries `tag`: sum.c = start.c + w(0, c) + ... +
// w(n - 1, c). False when a wait gives up. Whole wave.
template <class F>
__device__ bool wave_fetch_sum4(F p, int n, uint32_t tag, float4 start, float4& sum, int32_t* err) {
  constexpr int kGroups = 2;  // n <= kGroups
  const long long t0 = wall_clock64();
  for (int it = 0;; ++it) {
    uint64_t v[4 * kGroups];
#pragma unroll
    for (int i = 0; i < 4 * kGroups; ++i) v[i] = (i >> 2) < n ? ld_fresh64(p(i)) : tag_word(0.f, tag);
    bool ok = true;
    float4 s = start;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ok = ok && (uint32_t)(v[4 * j + c] >> 32) == tag;
      if (j < n) {
        s.x += __uint_as_float((uint32_t)v[4 * j + 0]);
        s.y += __uint_as_float((uint32_t)v[4 * j + 1]);
        s.z += __uint_as_float((uint32_t)v[4 * j + 2]);
        s.w += __uint_as_float((uint32_t)v[4 * j + 3]);
      }
    }
    if (__ballot(!ok) == 0) {
      sum = s;
      return true;
    }
    if (!keep_waiting(it, t0, err)) return false;
  }
}

// Wave-level wait: lane i (with a non-null `mine`) polls one flag word until
// every polled word equals `want`. False when the wait gives up.
__device__ bool wave_wait(const int32_t* mine, int want, int32_t* err) {
  const long long t0 = wall_clock64();
  for (int it = 0;; ++it) {
    const int v = mine ? ld_fresh(mine) : want;
    if (__ballot(v != want) == 0) return true;
    if (!keep_waiting(it, t0, err)) return false;
  }
}

// Keep decoded weights where they are: an empty asm that claims to modify
// each register, so the compiler cannot sink the decode past the wait (it
// would otherwise recompute it there to shorten register live ranges).
template <int NKT>
__device__ __forceinline__ void pin_decoded(h16x2 (&wv)[NKT][32]) {
#pragma unroll
  for (int j = 0; j < NKT; ++j)
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      uint32_t u = __builtin_bit_cast(uint32_t, wv[j][i]);
      asm volatile("" : "+v"(u));
      wv[j][i] = __builtin_bit_cast(h16x2, u);
    }
}

constexpr int kWaves = 8;    // waves per work-group (two work-groups per compute unit)
constexpr int kChunks = 4;   // 128-input chunks of a gate_up task; channel chunks of a down task

// SiLU from the hardware exponential and reciprocal (each within about one
// ulp): g / (1 + e^-g), within a few ulp of the correctly rounded value.
// Large negative g gives e^-g = inf and a zero (signed) result.
__device__ __forceinline__ float silu_fast(float g) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

struct Lds {
  uint32_t code[kWaves * Stage<3>::kDw];                   // each wave's staged codes
  _Float16 xh[kChunks][128] __attribute__((aligned(16)));  // rotated inputs (high fp16 parts) per chunk
  _Float16 xl[kChunks][128] __attribute__((aligned(16)));  // and their low parts
  float xe[kChunks];                                       // undo factor of each chunk's scale
  float red[2][kChunks * 128] __attribute__((aligned(16)));  // per-chunk sums of the task's outputs
                                                             // (two input-row sets in the pair layout)
  float rin[kChunks][128];                                 // input scales of the task's chunks
  float rout[128];                                         // output scales of its block
  float4 part[kChunks][64];                                // down: second-half gate_up part sums
  int skip[kChunks];
  int ok[kWaves];
  int task;
  float wt;  // down: the pair's router weight (kept here across the wait)
};

// True when no wave of the group recorded a failed wait; after a barrier.
__device__ __forceinline__ bool all_ok(const Lds& sh) {
  int ok = 1;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ok &= sh.ok[w];
  return ok != 0;
}

// Contract a wave's decoded tiles (8 tile-rows of 128-block cl x 4 output
// tiles 4nq..4nq+3) with the block's activations on the matrix cores and
// leave the 64 sums in sh.red[0][stride * cl + 16 (4nq + j) + n] (output
// 16 (4nq + j) + n of the task).
// OPS: the operands of tile-row pair pp, OPS(pp, A4) (decoded beforehand,
// or just now when the task decodes after its wait).
// LEAN: each B operand is read from LDS just before its pair's MFMAs
// instead of all four up front (12 fewer registers live at the start of
// the contraction, for a form that holds 128 registers of operands).
template <bool LEAN = false, class OPS>
__device__ __forceinline__ void mfma_block(Lds& sh, OPS&& ops, int cl, int nq, int stride, int lane) {
  // B operands of the four tile-row pairs: column 0 of B = high parts,
  // column 1 = low parts, other columns zero; only the lanes of columns 0
  // and 1 read LDS
  const int col = lane & 15;
  const _Float16* src = (col == 0 ? sh.xh[cl] : sh.xl[cl]) + 8 * (lane >> 4);
  auto load_b = [&](int pp) {
    return col < 2 ? *reinterpret_cast<const h16x8*>(src + 32 * pp) : h16x8{};
  };
  h16x8 B[4];
  if constexpr (!LEAN) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) B[pp] = h16x8{};
    if (col < 2) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) B[pp] = *reinterpret_cast<const h16x8*>(src + 32 * pp);
    }
  }
  f32x4 D[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) D[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    h16x8 A[4];
    ops(pp, A);
    const h16x8 Bp = LEAN ? load_b(pp) : B[pp];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      D[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[j], Bp, D[j], 0, 0, 0);
  }
  float4 zr[4];
  finish_mfma(D, sh.xe[cl], zr);
  if ((lane & 15) == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(&sh.red[0][stride * cl + 16 * (4 * nq + j) + 4 * (lane >> 4)]) = zr[j];
  }
}

// The same contraction for operands in the column-pair layout (PairDecoder,
// K = 2): B's column 2 q + h (q = 2 set + parity, h: 0 high, 1 low part)
// holds the activations of the set's input rows at the B rows of that
// parity (8 g + 2 i + parity) and zeros at the others, so that
// D[m][2 q + h] with m = 8 set + c collects output column c (parity 0) or
// c + 8 (parity 1) over the set's input rows. The two sets' sums go to
// sh.red[set] and are added in sum_transform_store.
template <bool LEAN = false, class OPS>
__device__ __forceinline__ void mfma_pairs(Lds& sh, OPS&& ops, int cl, int nq, int lane) {
  const int col = lane & 15;
  const int g = lane >> 4;
  const int set = col >> 2, par = (col >> 1) & 1;
  // input rows 8 set + 4 (g & 1) + i of tile-row 2 pp + (g >> 1): inputs
  // 32 pp + 16 (g >> 1) + 8 set + 4 (g & 1) + i of the chunk
  const _Float16* src = ((col & 1) ? sh.xl[cl] : sh.xh[cl]) + 16 * (g >> 1) + 8 * set + 4 * (g & 1);
  // LEAN: the four pairs' activations kept packed (2 registers each) and
  // spread into B just before use
  u32x2 Braw[4];
  h16x8 B[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    Braw[pp] = u32x2{0u, 0u};
    B[pp] = h16x8{};
  }
  if (col < 8) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      Braw[pp] = *reinterpret_cast<const u32x2*>(src + 32 * pp);
      if constexpr (!LEAN) B[pp] = parity_operand(Braw[pp], par);
    }
  }
  f32x4 D[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) D[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    h16x8 A[4];
    ops(pp, A);
    const h16x8 Bp = LEAN ? (col < 8 ? parity_operand(Braw[pp], par) : h16x8{}) : B[pp];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      D[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[j], Bp, D[j], 0, 0, 0);
  }
  // high + low part into the even columns (finish_mfma), then lanes (col
  // 4 set + 2 parity, g) with set = g >> 1 hold outputs 8 parity + 4 (g &
  // 1) .. + 3 of each tile for that set
  float4 zr[4];
  finish_mfma(D, sh.xe[cl], zr);
  if ((col & 9) == 0 && (col >> 2) == (g >> 1)) {
    const int set = col >> 2;
    const int off = 128 * cl + 8 * ((col >> 1) & 1) + 4 * (g & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<float4*>(&sh.red[set][off + 16 * (4 * nq + j)]) = zr[j];
  }
}

// Tile-row pair pp's operands from a decoder whose decode takes the pair
// as a template argument (pp is a constant once the callers are unrolled).
template <class DEC>
__device__ __forceinline__ void decode_pp(const DEC& dec, int pp, h16x8 (&A)[4]) {
  switch (pp) {
    case 0: dec.template decode<0>(A); break;
    case 1: dec.template decode<1>(A); break;
    case 2: dec.template decode<2>(A); break;
    default: dec.template decode<3>(A); break;
  }
}

// Output transform of the task's 128 outputs (wave 0): the sum over the
// first nb input chunks (in chunk order), H_n, rout (sh.rout) and the
// weight, stored as tagged words (REMOTE: sc1 stores).
template <bool REMOTE, bool PAIRS = false>
__device__ __forceinline__ void sum_transform_store(const Lds& sh, int nb, float wt,
                                                    uint64_t* __restrict__ out, uint32_t tag,
                                                    int wave, int lane) {
  if (wave == 0) {
    const int o = lane;
    // chunk by chunk (in order), each chunk's two sets first in the pair layout
    auto part = [&](int b, int oo) {
      return PAIRS ? sh.red[0][128 * b + oo] + sh.red[1][128 * b + oo] : sh.red[0][128 * b + oo];
    };
    float z0 = part(0, o), z1 = part(0, o + 64);
    for (int b = 1; b < nb; ++b) {
      z0 += part(b, o);
      z1 += part(b, o + 64);
    }
    fwht128(z0, z1);
    const float o0 = z0 * kInvSqrt128 * sh.rout[o] * wt;
    const float o1 = z1 * kInvSqrt128 * sh.rout[o + 64] * wt;
    if constexpr (REMOTE) {
      st_remote64(out + o, tag_word(o0, tag));
      st_remote64(out + o + 64, tag_word(o1, tag));
    } else {
      out[o] = tag_word(o0, tag);
      out[o + 64] = tag_word(o1, tag);
    }
  }
}

// A combined 128-block of a token's layer output (y0, y1: outputs lane and
// lane + 64 of block b): in the last layer the output y; otherwise XCD x's
// copy of it and the block's sum of squares, tagged. Whole wave.
__device__ __forceinline__ void store_combined(const FlowArgs& a, bool last, int t, int x, int b,
                                               int lane, float y0, float y1, uint32_t tag) {
  const int H = a.hidden;
  if (last) {
    a.y_last[(size_t)t * H + 128 * b + lane] = y0;
    a.y_last[(size_t)t * H + 128 * b + lane + 64] = y1;
  } else {
    uint64_t* yo = a.ycb + ((size_t)t * 8 + x) * H + 128 * b + lane;
    yo[0] = tag_word(y0, tag);
    yo[64] = tag_word(y1, tag);
    const float sq = wave_sum(__builtin_fmaf(y0, y0, y1 * y1));
    if (lane == 0) a.sscb[((size_t)t * 8 + x) * 32 + b] = tag_word(sq, tag);
  }
}

}  // namespace

// LATE: a task stages its codes before its wait but decodes them only
// after it, each tile-row pair just before its MFMAs, so that it holds 32
// rather than 64 registers of operands while it waits and three work-groups
// fit on a compute unit (larger batches, where a layer's tasks are many
// times the device's slots, so decode ahead of the chain matters little).
// WIDE (decode before the wait, top_k <= 8): a task is 4 waves, each
// holding the decoded operands of two chunks (128 registers), and three
// work-groups share a compute unit: the device then holds 1.5 times the
// decoded weights of the 8-wave form (two work-groups of 8 waves with 64
// registers of operands each).
template <int KG, int KD, bool LATE, bool WIDE = false>
__global__ __launch_bounds__(WIDE ? 256 : 64 * kWaves, LATE ? 6 : (WIDE ? 3 : 4)) void k_stack_flow(
    const FlowArgs a) {
  static_assert(!(LATE && WIDE), "the wide form decodes before its wait");
  constexpr int CPW = WIDE ? 2 : 1;  // chunks per wave
  __shared__ Lds sh;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int H = a.hidden, I = a.inter, k = a.top_k, T = a.n_tokens;
  const int P = T * k, P8 = a.p8;
  const int ncg = H / 128, ngb = (2 * I) / 128;  // gate_up input chunks / output blocks
  const int nh = ncg / kChunks;                  // gate_up input parts (kChunks chunks each)
  const int ncd = I / 128, ngd = H / 128;        // down chunks (<= kChunks) / output blocks
  const int nb_gu = nh * ngb * P8, nb_dn = ngd * P8;
  const int nb = H / 128, nhf = (nb + 3) / 4;   // output blocks / combine tasks per (token, XCD)
  const int per_layer = nb_gu + nb_dn + (a.fold ? 0 : T * nhf * 8);

  // claim this XCD's next task: the j-th work-group to start on XCD x runs
  // task 8j + x (the grid holds at least as many work-groups per XCD as the
  // XCD has tasks; the surplus finds no task and leaves)
  if (tid == 0) {
    const int x = xcc_id();
    const int j = x < 8 ? __hip_atomic_fetch_add(a.ticket + 32 * x, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                        : a.n_layers * per_layer;
    sh.task = x < 8 ? 8 * j + x : a.n_layers * per_layer;
  }
  __syncthreads();
  const int bid = sh.task;
  if (bid >= a.n_layers * per_layer) return;
  const int l = bid / per_layer;
  int r = bid - l * per_layer;
  // tag of the words this layer's tasks write (the call's number, written
  // by the kernel that precedes this launch, and the layer)
  const uint32_t epoch = (uint32_t)a.epoch[0];
  const uint32_t tag = (epoch << 8) + (uint32_t)l + 1u;
  if (tid < kWaves) sh.ok[tid] = 1;
  const StackLayer& Ly = a.layer[l];


  if (r < nb_gu) {
    // ------------------------------------------------------------ gate_up
    // task (pair p, inputs 512 hh .. 512 hh + 511, outputs 128 g .. 128 g +
    // 127); wave w: input chunk cl = w / 2 of the four (its 8 tile-rows),
    // output tiles 4 nq .. 4 nq + 3 (nq = w % 2) of the block (WIDE: input
    // chunks 2 (w / 2) and 2 (w / 2) + 1)
    const int cl = WIDE ? 2 * (wave >> 1) : wave >> 1;  // first chunk of the wave
    const int nq = wave & 1;
    const int p = r % P8;
    if (p >= P) return;
    r /= P8;
    const int g = r % ngb;
    const int hh = r / ngb;
    const int c = kChunks * hh + cl;  // this wave's (first) input chunk
    const int t = p / k;
    const int x = p & 7;
    const int e = a.ids[(size_t)l * P + p];
    const bool valid = e >= 0 && e < a.n_experts;
    const int n_nt = (2 * I) / 16;
    uint64_t* out = a.gu_part + ((size_t)p * nh + hh) * (2 * I) + g * 128;

    // an out-of-range id is decoded as expert 0 and its result discarded,
    // which keeps the register state the same on every path
    const int es = valid ? e : 0;
    const uint16_t* code_e = Ly.gu_code + (size_t)es * (size_t)ncg * 8 * n_nt * (16 * KG);
    u32x4 cv[CPW][Stage<KG>::kPerLane];
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci) stage_issue<KG>(code_e, n_nt, 8 * (c + ci), 8 * g + 4 * nq, lane, cv[ci]);
    // the chunk's input scales and the block's output scales, kept in LDS
    // until they are needed (WIDE: wave w loads chunk w's, wave 1 also the
    // output scales)
    const int cn = WIDE ? wave : cl;  // the chunk this wave normalises (nq == 0 or WIDE)
    const uint16_t* rr = Ly.gu_rin + (size_t)es * H + (kChunks * hh + cn) * 128;
    const uint16_t* ro = Ly.gu_rout + (size_t)es * (2 * I) + g * 128;
    const uint16_t* rs = (WIDE || nq == 0) ? rr : ro;
    const uint16_t s0 = rs[lane], s1 = rs[lane + 64];
    uint16_t o0 = 0, o1 = 0;
    if (WIDE && wave == 1) {
      o0 = ro[lane];
      o1 = ro[lane + 64];
    }
    uint32_t* stage = sh.code + CPW * wave * Stage<KG>::kDw;
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci) stage_store<KG>(stage + ci * Stage<KG>::kDw, lane, cv[ci]);
    float* sd = (WIDE || nq == 0) ? sh.rin[cn] : sh.rout;
    if (WIDE || nq == 0 || wave == 1) {
      sd[lane] = f16_to_f32(s0);
      sd[lane + 64] = f16_to_f32(s1);
    }
    if (WIDE && wave == 1) {
      sh.rout[lane] = f16_to_f32(o0);
      sh.rout[lane + 64] = f16_to_f32(o1);
    }
    h16x8 A[CPW][4][4];
    if constexpr (!LATE) {
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        if constexpr (KG == 2) {  // column-pair layout: 9 VALU operations per pair of weights
          const PairDecoder dec(stage + ci * Stage<KG>::kDw, lane);
          dec.template decode<0>(A[ci][0]);
          dec.template decode<1>(A[ci][1]);
          dec.template decode<2>(A[ci][2]);
          dec.template decode<3>(A[ci][3]);
        } else {
          decode_stage_mfma<KG>(stage + ci * Stage<KG>::kDw, lane, A[ci]);
        }
        pin_operands(A[ci]);
      }
    }
    // arguments the normalisation needs, read now rather than after the wait
    float eps = a.eps;
    float inv_h = __int_as_float((96 + __builtin_clz(H)) << 23);  // 1 / H (a power of two)
    uint16_t* x_chain = a.x_chain;
    asm volatile("" : "+s"(eps), "+s"(inv_h), "+s"(x_chain));
    __syncthreads();  // sh.ok initialised
    if (WIDE || nq == 0) {  // one wave per chunk: x~ = H_n(rin (.) x)
      const int cc = kChunks * hh + cn;
      float x0, x1;
      if (l == 0) {
        const uint16_t* xr = a.x0 + (size_t)t * H + cc * 128;
        x0 = bf16_to_f32(xr[lane]);
        x1 = bf16_to_f32(xr[lane + 64]);
      } else {
        // the previous layer's combine tasks of this token on this XCD wrote
        // the chunk's outputs y and every block's sum of squares: RMSNorm,
        // rounded to bf16
        const uint64_t* yr = a.ycb + ((size_t)t * 8 + x) * H + cc * 128 + lane;
        const uint64_t* sr = a.sscb + ((size_t)t * 8 + x) * 32 + (lane < ncg ? lane : 0);
        float v[3];
        const bool ok = wave_fetch<3>([&](int i) { return i < 2 ? yr + 64 * i : sr; }, 3, tag - 1u, v,
                                      a.error);
        if (lane == 0) sh.ok[wave] = ok ? 1 : 0;
        __builtin_amdgcn_s_setprio(3);
        // the blocks' sums of squares (lane b: block b) summed across the
        // wave, the same bits in every lane and every task of the token
        const float tot = wave_sum(lane < ncg ? v[2] : 0.f);
        const float inv = 1.0f / sqrtf(tot * inv_h + eps);
        const uint16_t b0 = f32_to_bf16_rne(v[0] * inv);
        const uint16_t b1 = f32_to_bf16_rne(v[1] * inv);
        x0 = bf16_to_f32(b0);
        x1 = bf16_to_f32(b1);
      }
      if (x_chain && g == 0 && p % k == 0) {  // the layer input, recorded by one pair per token
        uint16_t* xo = x_chain + ((size_t)l * T + t) * H + cc * 128;
        xo[lane] = f32_to_bf16_rne(x0);
        xo[lane + 64] = f32_to_bf16_rne(x1);
      }
      float v0 = x0 * sh.rin[cn][lane];
      float v1 = x1 * sh.rin[cn][lane + 64];
      fwht128(v0, v1);
      const float xe = split_hilo(v0 * kInvSqrt128, v1 * kInvSqrt128, sh.xh[cn], sh.xl[cn], lane);
      if (lane == 0) sh.xe[cn] = xe;
    }
    __syncthreads();
    if (!all_ok(sh)) return;
    __builtin_amdgcn_s_setprio(3);
    if (valid) {  // uniform over the group
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        auto held = [&](int pp, h16x8(&A4)[4]) {
#pragma unroll
          for (int j = 0; j < 4; ++j) A4[j] = A[ci][pp][j];
        };
        if constexpr (KG == 2) {
          if constexpr (LATE) {
            const PairDecoder dec(stage, lane);
            mfma_pairs(sh, [&](int pp, h16x8(&A4)[4]) { decode_pp(dec, pp, A4); }, cl, nq, lane);
          } else {
            mfma_pairs<WIDE>(sh, held, cl + ci, nq, lane);
          }
        } else {
          if constexpr (LATE) {
            const OperandDecoder<KG> dec(stage, lane);
            mfma_block(sh, [&](int pp, h16x8(&A4)[4]) { decode_pp(dec, pp, A4); }, cl, nq, 128, lane);
          } else {
            mfma_block<WIDE>(sh, held, cl + ci, nq, 128, lane);
          }
        }
      }
      __syncthreads();
      sum_transform_store<false, KG == 2>(sh, kChunks, 1.0f, out, tag, wave, lane);
    } else if (wave == 0) {  // an out-of-range expert id contributes nothing
      out[lane] = tag_word(0.f, tag);
      out[lane + 64] = tag_word(0.f, tag);
    }
  } else if ((r -= nb_gu) < nb_dn) {
    // --------------------------------------------------------------- down
    // task (pair p, outputs 128 g .. 128 g + 127); wave w: channel chunk
    // cl = w / 2 (its 8 tile-rows), output tiles 4 nq .. 4 nq + 3 (nq = w % 2)
    // (WIDE: channel chunks 2 (w / 2) and 2 (w / 2) + 1)
    const int cl = WIDE ? 2 * (wave >> 1) : wave >> 1;
    const int nq = wave & 1;
    const int p = r % P8;
    if (p >= P) return;
    const int g = r / P8;
    const int e = a.ids[(size_t)l * P + p];
    const bool valid = e >= 0 && e < a.n_experts;
    const bool active = cl < ncd;  // this wave has tile-rows (of its first chunk)
    const int cn = WIDE ? wave : cl;  // the chunk this wave forms h of (nq == 0 or WIDE)
    const bool nactive = cn < ncd;
    const int n_nt = H / 16;
    uint64_t* out = a.dn_part + (size_t)(l & 1) * a.dn_copy + (size_t)p * H + g * 128;

    const int es = valid ? e : 0;
    const uint16_t* code_e = Ly.dn_code + (size_t)es * (size_t)ncd * 8 * n_nt * (16 * KD);
    u32x4 cv[CPW][Stage<KD>::kPerLane];
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci)
      if (cl + ci < ncd) stage_issue<KD>(code_e, n_nt, 8 * (cl + ci), 8 * g + 4 * nq, lane, cv[ci]);
    const uint16_t* rr = Ly.dn_rin + (size_t)es * I + (nactive ? cn : 0) * 128;
    const uint16_t* ro = Ly.dn_rout + (size_t)es * H + g * 128;
    const uint16_t* rs = (WIDE || nq == 0) ? rr : ro;
    const uint16_t s0 = rs[lane], s1 = rs[lane + 64];
    uint16_t o0 = 0, o1 = 0;
    if (WIDE && wave == 1) {
      o0 = ro[lane];
      o1 = ro[lane + 64];
    }
    const float wt_ld = a.w[(size_t)l * P + p];
    uint32_t* stage = sh.code + CPW * wave * Stage<KD>::kDw;
    h16x8 A[CPW][4][4];
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci)
      if (cl + ci < ncd) stage_store<KD>(stage + ci * Stage<KD>::kDw, lane, cv[ci]);
    float* sd = (WIDE || nq == 0) ? sh.rin[cn] : sh.rout;
    if (((WIDE || nq == 0) && nactive) || (!WIDE && wave == 1)) {
      sd[lane] = f16_to_f32(s0);
      sd[lane + 64] = f16_to_f32(s1);
    }
    if (WIDE && wave == 1) {
      sh.rout[lane] = f16_to_f32(o0);
      sh.rout[lane + 64] = f16_to_f32(o1);
    }
    if constexpr (!LATE) {
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        if (cl + ci < ncd) decode_stage_mfma<KD>(stage + ci * Stage<KD>::kDw, lane, A[ci]);
        pin_operands(A[ci]);
      }
    }
    if (tid == 0) sh.wt = wt_ld;
    __syncthreads();  // sh.ok and sh.wt initialised
    // gate and up sums of the chunk's channels over gate_up's input parts,
    // once every gate_up task of this pair has written them: the chunk's
    // wave nq fetches parts 2 nq and 2 nq + 1, and the sum is (part 0 +
    // part 1) + (part 2 + part 3)
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    // parts 2 h and 2 h + 1 of chunk ch's gate and up sums, from 0
    auto fetch_half = [&](int ch, int h, float4& out) {
      const uint64_t* src = a.gu_part + ((size_t)p * nh + 2 * h) * (2 * I) + 128 * ch + lane;
      auto word = [&](int i) {  // part 2 h + i / 4; gate, gate + 64, up, up + 64
        return src + (size_t)(i >> 2) * (2 * I) + ((i & 1) ? 64 : 0) + ((i & 2) ? I : 0);
      };
      return wave_fetch_sum4(word, nh - 2 * h < 2 ? nh - 2 * h : 2, tag, make_float4(0.f, 0.f, 0.f, 0.f),
                             out, a.error);
    };
    float4 second = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (WIDE) {
      // one wave per chunk fetches both halves
      if (nactive && valid) {
        bool ok = fetch_half(cn, 0, sum);
        if (nh > 2) {
          ok = ok && fetch_half(cn, 1, second);
          sum.x += second.x;
          sum.y += second.y;
          sum.z += second.z;
          sum.w += second.w;
          second = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (lane == 0) sh.ok[wave] = ok ? 1 : 0;
      }
    } else {
      if (active && valid && 2 * nq < nh) {
        const bool ok = fetch_half(cl, nq, sum);
        if (lane == 0) sh.ok[wave] = ok ? 1 : 0;
        if (nq == 1) sh.part[cl][lane] = sum;
      }
      if (nh > 2) __syncthreads();  // second halves in LDS
      if (nq == 0 && active && valid && nh > 2) second = sh.part[cl][lane];
    }
    if ((WIDE || nq == 0) && nactive) {  // one wave per 128-channel chunk
      int skip = 1;
      if (valid) {
        __builtin_amdgcn_s_setprio(3);
        if (!WIDE && nh > 2) {
          const float4 q = second;
          sum.x += q.x;
          sum.y += q.y;
          sum.z += q.z;
          sum.w += q.w;
        }
        const float g0 = sum.x, g1 = sum.y, u0 = sum.z, u1 = sum.w;
        const float h0 = silu_fast(g0) * u0;
        const float h1 = silu_fast(g1) * u1;
        skip = __ballot((h0 != 0.f) || (h1 != 0.f)) == 0;
        float v0 = h0 * sh.rin[cn][lane];
        float v1 = h1 * sh.rin[cn][lane + 64];
        fwht128(v0, v1);
        const float xe = split_hilo(v0 * kInvSqrt128, v1 * kInvSqrt128, sh.xh[cn], sh.xl[cn], lane);
        if (lane == 0) sh.xe[cn] = xe;
      }
      // a chunk whose h is all zero contributes exactly zero: its MAC is skipped
      if (lane == 0) sh.skip[cn] = skip;
    }
    __syncthreads();
    if (!all_ok(sh)) return;
    __builtin_amdgcn_s_setprio(3);
    if (valid) {  // uniform over the group
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        const int ch = cl + ci;
        if (ch < ncd && !sh.skip[ch]) {
          if constexpr (LATE) {
            const OperandDecoder<KD> dec(stage, lane);
            mfma_block(sh, [&](int pp, h16x8(&A4)[4]) { decode_pp(dec, pp, A4); }, cl, nq, 128, lane);
          } else {
            mfma_block<WIDE>(
                sh,
                [&](int pp, h16x8(&A4)[4]) {
#pragma unroll
                  for (int j = 0; j < 4; ++j) A4[j] = A[ci][pp][j];
                },
                ch, nq, 128, lane);
          }
        } else if (ch < ncd && (lane & 15) == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4*>(&sh.red[0][128 * ch + 16 * (4 * nq + j) + 4 * (lane >> 4)]) =
                make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      __syncthreads();
      sum_transform_store<true>(sh, ncd, sh.wt, out, tag, wave, lane);
    } else if (wave == 0) {  // an out-of-range expert id contributes nothing
      st_remote64(out + lane, tag_word(0.f, tag));
      st_remote64(out + lane + 64, tag_word(0.f, tag));
    }
    if (a.fold) {
      // the combine of this output block for the token's copy on this XCD:
      // wave 0 (lanes outputs lane and lane + 64) adds the outputs of the
      // token's pairs in slot order as soon as every one carries this
      // layer's tag. The pair of slot j < 8 is the token's only pair on its
      // XCD; in the last layer only slot 0 runs it, to write y.
      const int t = p / k;
      const int j = p - t * k;
      if (wave == 0 && (l == a.n_layers - 1 ? j == 0 : j < 8)) {
        const int b = g;
        const uint64_t* pp = a.dn_part + (size_t)(l & 1) * a.dn_copy + (size_t)t * k * H + 128 * b + lane;
        float v[16];
        if (wave_fetch<16>([&](int i) { return pp + (size_t)(i >> 1) * H + ((i & 1) ? 64 : 0); },
                           2 * k, tag, v, a.error)) {
          float y0 = 0.f, y1 = 0.f;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj)
            if (jj < k) {
              y0 += v[2 * jj];
              y1 += v[2 * jj + 1];
            }
          store_combined(a, l == a.n_layers - 1, t, p & 7, b, lane, y0, y1, tag);
        }
      }
    } else {
      // flag for the combine tasks (a hint: the tags decide)
      __syncthreads();
      if (tid == 0) st_remote(a.dflag + ((size_t)l * P8 + p) * a.df_pair + g, (int)tag);
    }
  } else {
    // ------------------------------------------------------------ combine
    // task (token t, XCD x, outputs 512 hf .. 512 hf + 511): the sum of
    // the token's pair outputs and the sums of squares of its 128-blocks,
    // for the next layer's gate_up tasks on XCD x. Waves 2i and 2i + 1 take
    // block 4 hf + i, lanes its outputs lane and lane + 64; the even wave
    // sums the first half of the slots in order, the odd wave the second
    // half, and the two halves are added (first + second).
    r -= nb_dn;
    const int x = r & 7;
    r >>= 3;
    const int hf = r % nhf;
    const int t = r / nhf;
    // combine tasks run only on XCDs that hold a pair of the token (the
    // next layer's gate_up tasks there read them); in the last layer only
    // the XCD of the token's first pair runs them, to write y_last
    const int x_first = (t * k) & 7;
    const bool last = l == a.n_layers - 1;
    if (last ? x != x_first : (k < 8 && ((x - x_first) & 7) >= k)) return;
    const int b = 4 * hf + (WIDE ? wave : wave >> 1);  // this wave's 128-block
    if (wave == 0) {
      // the down tasks of the token's pairs for these outputs have flagged
      const int32_t* df = a.dflag + ((size_t)l * P8 + (size_t)t * k) * a.df_pair + 4 * hf;
      const int32_t* mine =
          lane < 4 * k ? df + (size_t)(lane >> 2) * a.df_pair + (lane & 3) : nullptr;
      const bool ok = wave_wait(mine, (int)tag, a.error);
      if (lane == 0) sh.ok[0] = ok ? 1 : 0;
    }
    __syncthreads();
    if (!all_ok(sh)) return;
    __builtin_amdgcn_s_setprio(3);
    const int half = (k + 1) / 2;
    if constexpr (WIDE) {
      // one wave per block (top_k <= 8): both halves of the slots, each
      // summed from zero in order, then added (first + second)
      if (b < nb) {
        const uint64_t* pp = a.dn_part + (size_t)(l & 1) * a.dn_copy + (size_t)(t * k) * H + 128 * b + lane;
        float v[16];
        const bool ok = wave_fetch<16>([&](int i) { return pp + (size_t)(i >> 1) * H + ((i & 1) ? 64 : 0); },
                                       2 * k, tag, v, a.error);
        float f0 = 0.f, f1 = 0.f, s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < half) {
            f0 += v[2 * j];
            f1 += v[2 * j + 1];
          } else if (j < k) {
            s0 += v[2 * j];
            s1 += v[2 * j + 1];
          }
        }
        if (ok) store_combined(a, last, t, x, b, lane, f0 + s0, f1 + s1, tag);
      }
      return;
    }
    const int j0 = (wave & 1) ? half : 0;  // this wave's slots j0 .. j1 - 1
    const int j1 = (wave & 1) ? k : half;
    const uint64_t* pp =
        a.dn_part + (size_t)(l & 1) * a.dn_copy + (size_t)(t * k + j0) * H + 128 * b + lane;
    float y0 = 0.f, y1 = 0.f;
    bool ok = true;
    if (b < nb) {
      float v[16];
      ok = wave_fetch<16>([&](int i) { return pp + (size_t)(i >> 1) * H + ((i & 1) ? 64 : 0); },
                          2 * (j1 - j0), tag, v, a.error);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < j1 - j0) {
          y0 += v[2 * j];
          y1 += v[2 * j + 1];
        }
      if (wave & 1) {  // second half of the slots to LDS
        sh.red[0][128 * (wave >> 1) + lane] = y0;
        sh.red[0][128 * (wave >> 1) + 64 + lane] = y1;
      }
    }
    if (lane == 0 && !ok) sh.ok[wave] = 0;
    __syncthreads();
    if (!all_ok(sh)) return;
    if (!(wave & 1) && b < nb) {
      y0 += sh.red[0][128 * (wave >> 1) + lane];
      y1 += sh.red[0][128 * (wave >> 1) + 64 + lane];
      store_combined(a, last, t, x, b, lane, y0, y1, tag);
    }
  }
}

// Before a launch: zero the control block's n words except word 2, the call
// number, which advances.
__global__ __launch_bounds__(256) void k_flow_prepare(int32_t* __restrict__ ctl, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    if (i != 2) ctl[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) ctl[2] = (int32_t)(((uint32_t)ctl[2] + 1u) & 0xFFFFFFu);
}

hipError_t launch_flow_prepare(int32_t* ctl, size_t n, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_flow_prepare, dim3((unsigned)blocks), dim3(256), 0, s, ctl, n);
  return hipGetLastError();
}

int64_t flow_blocks_per_layer(int hidden, int inter, int top_k, int n_tokens, bool fold) {
  const int64_t P8 = ((int64_t)n_tokens * top_k + 7) / 8 * 8;
  return (int64_t)(hidden / 512) * (2 * inter / 128) * P8 + (int64_t)(hidden / 128) * P8 +
         (fold ? 0 : (int64_t)n_tokens * ((hidden / 128 + 3) / 4) * 8);
}

template <bool LATE, bool WIDE>
const void* flow_kernel(int k_gu, int k_dn) {
  return k_gu == 2 && k_dn == 3   ? (const void*)k_stack_flow<2, 3, LATE, WIDE>
         : k_gu == 2 && k_dn == 2 ? (const void*)k_stack_flow<2, 2, LATE, WIDE>
         : k_gu == 3 && k_dn == 3 ? (const void*)k_stack_flow<3, 3, LATE, WIDE>
         : k_gu == 3 && k_dn == 2 ? (const void*)k_stack_flow<3, 2, LATE, WIDE>
                                  : nullptr;
}

const void* flow_kernel(int k_gu, int k_dn, bool late, bool wide) {
  return late ? flow_kernel<true, false>(k_gu, k_dn)
              : (wide ? flow_kernel<false, true>(k_gu, k_dn) : flow_kernel<false, false>(k_gu, k_dn));
}

hipError_t flow_groups_per_cu(int k_gu, int k_dn, bool late, bool wide, int* n) {
  if (late && wide) return hipErrorInvalidValue;
  const void* f = flow_kernel(k_gu, k_dn, late, wide);
  if (!f) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, f, wide ? 256 : 64 * kWaves, 0);
}

hipError_t launch_stack_flow(const FlowArgs& a, int k_gu, int k_dn, hipStream_t s) {
  // the wide form decodes before its wait, and its combine tasks take top_k <= 8
  if (a.wide && (a.late || a.top_k > 8)) return hipErrorInvalidValue;
  const int64_t blocks =
      flow_blocks_per_layer(a.hidden, a.inter, a.top_k, a.n_tokens, a.fold != 0) * a.n_layers +
      kFlowSpare;
  const void* f = flow_kernel(k_gu, k_dn, a.late != 0, a.wide != 0);
  if (!f) return hipErrorInvalidValue;
  FlowArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(f, dim3((unsigned)blocks), dim3(a.wide ? 256 : 64 * kWaves), args, 0, s);
}

}  // namespace escha
