// escha_grouped.hip -- the grouped path: pairs sorted by expert, each weight
// tile decoded once per tile of tokens of the same expert and contracted on
// the matrix cores with fp32 accumulation. Used by the prefill entry point
// and by decode calls with enough tokens. Kernels: the rotated-input gather;
// the 128-token tile kernels below (weights decoded into LDS as fp16,
// v_mfma_f32_32x32x16_f16); the small-tile kernels (<= 16 tokens, weights
// decoded straight into v_mfma_f32_16x16x32_f16 operands); the sorted
// combine, and the kernel that links two layers of the stack (combine,
// RMSNorm, next layer's gather).
//
// Sources: hipfire PR "Escha-W2 port: 2-bit trellis decoded in the GEMV",
// grouped-GEMM notes (expert_offsets + permutation; each weight tile
// decoded once and reused by several activation tiles). Activations enter
// the contraction as fp16 (the decoded weights are exactly fp16).
//
// Layout in one work-group (16 waves, four per SIMD):
//  - waves 0-7 decode: lane = 8*tile + o, tile = 16*kt_local + nt_local: 64
//    tiles (4 tile-rows x 16 output tiles) = one 64-input step for 256
//    outputs, written to LDS one step ahead of the matrix waves; lane o of a
//    tile's eight decodes input rows 2o and 2o+1 (32 weights), so every SIMD
//    has two decoder waves to hide the decode's latencies;
//  - LDS W fp16 in 16-byte k-chunks: element (row, k) of a step sits at
//    halves ((k/8)*256 + pi(row))*8 + k%8, pi(row) = row ^ ((row>>4) & 15).
//    A decode store (a 4-byte row pair of one output column per lane) then
//    spreads over all 32 banks, and an MFMA operand read (32 consecutive
//    rows) uses each 16-byte slot exactly twice. Two buffers, one barrier
//    per step;
//  - the decoder waves also stage the step's activation tile (fp16,
//    [k/8][token][8]) in LDS; codes and activations are issued two steps
//    ahead of their use;
//  - waves 8-15 run the matrix cores on the current step from LDS, so decode
//    (VALU) and contraction (MFMA) overlap on every SIMD, and each SIMD has
//    two matrix waves, one issuing MFMAs while the other waits for its LDS
//    operands;
//  - matrix wave (wo, wt) owns outputs 64wo..64wo+63 (two 32-row MFMA
//    tiles) for tokens 64wt..64wt+63 (two 32-token MFMA tiles): 4
//    accumulators of 16 fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "escha_device.hpp"
#include "escha_launch.hpp"
#include "escha_mfma.hpp"

namespace escha {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDecWaves = 8;     // decoder waves per work-group
constexpr int kMatWaves = 8;    // matrix waves per work-group
constexpr int kMT = 16 / kMatWaves;  // 32-row output tiles of a matrix wave
constexpr int kThreads = 64 * (kDecWaves + kMatWaves);
constexpr int kWaves = kThreads / 64;
constexpr int kTM = 128;         // tokens per tile
constexpr int kStep = 64;        // inputs per step (4 tile-rows)
constexpr int kWBuf = 256 * kStep;  // halves per W buffer (32 KiB)
constexpr int kXBuf = kTM * kStep;  // halves per activation buffer (16 KiB)
constexpr int kEPitch = 260;     // LDS row pitch of the epilogue (floats; rows 16-byte aligned)
constexpr int kMainBytes = 2 * (kWBuf + kXBuf) * 2;  // 96 KiB of main-loop buffers
constexpr int kEpiBytes = kTM * kEPitch * 4;        // 130 KiB: the whole tile's outputs
constexpr int kSmemBytes = kMainBytes > kEpiBytes ? kMainBytes : kEpiBytes;

// ------------------------------------------------------------------------
// Tile list: for every expert, ceil(count / tm) tiles of consecutive sorted
// pairs (tm tokens each, the last one shorter). One block of 1024 threads;
// n_experts <= 1024.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_make_tiles(const int32_t* __restrict__ offsets, int E,
                                                     int tm, int max_tiles,
                                                     int32_t* __restrict__ t_expert,
                                                     int32_t* __restrict__ t_row0,
                                                     int32_t* __restrict__ t_rows,
                                                     int32_t* __restrict__ n_tiles) {
  __shared__ int32_t scan[1024];
  const int e = threadIdx.x;
  const size_t ly = blockIdx.y;  // layer of a batch of tile lists
  offsets += ly * (E + 1);
  t_expert += ly * max_tiles;
  t_row0 += ly * max_tiles;
  t_rows += ly * max_tiles;
  n_tiles += ly;
  int32_t cnt = 0, nt = 0;
  if (e < E) {
    cnt = offsets[e + 1] - offsets[e];
    nt = (cnt + tm - 1) / tm;
  }
  scan[e] = nt;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t v = e >= d ? scan[e - d] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  const int32_t base = scan[e] - nt;
  for (int i = 0; i < nt; ++i) {
    const int32_t ti = base + i;
    if (ti < max_tiles) {
      t_expert[ti] = e;
      t_row0[ti] = offsets[e] + i * tm;
      t_rows[ti] = cnt - i * tm < tm ? cnt - i * tm : tm;
    }
  }
  if (e == 1023) *n_tiles = scan[1023] < max_tiles ? scan[1023] : max_tiles;
}

// ------------------------------------------------------------------------
// Rotated gate_up inputs per sorted pair: Xg[i] = fp16(2^e H_n(rin_e (.) x_t))
// with the row's power-of-two exponent e (xg_exp[i]). Every rotated value
// is at most 16 max|rin (.) x| in magnitude (the 128 terms of a row of
// H_n each have magnitude 1/sqrt(128) < 16/128), so e is taken from that
// bound: 2^13 <= 16 max|rin (.) x| 2^e < 2^14, and the rotated values stay
// below 2^14. One wave per pair, kGatherRows consecutive pairs per
// work-group (with top_k 8, one token's: its input row is fetched once and
// read by the group from the cache), each written to its sorted row: lane l
// takes inputs 8 l .. 8 l + 7 of every 512-input chunk, so each 16 lanes
// hold one 128-input block; rows of up to kGatherHeld chunks stay in
// registers between the row maximum and the transform (every load issued
// up front), longer rows are read twice.
// ------------------------------------------------------------------------
constexpr int kGatherRows = 8;
constexpr int kGatherHeld = 4;
constexpr int kGatherSmallPairs = 8192;  // below: k_xin_gather_small

__global__ __launch_bounds__(64 * kGatherRows) void k_xin_gather(GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int p = kGatherRows * blockIdx.x + (threadIdx.x >> 6);
  if (p >= a.n_pairs) return;  // uniform over the wave
  const int i = a.inv[p];
  if (i < 0) return;  // an out-of-range expert id: no row
  const int e = a.ids[p];
  const int t = p / a.top_k;
  const int H = a.hidden;
  const int nch = (H + 511) / 512;
  const uint16_t* xrow = a.x_bf16 + (size_t)t * H;
  const uint16_t* rrow = a.rin + (size_t)e * H;
  auto load8 = [&](int base, float (&v)[8]) {
    const u32x4 xq = *reinterpret_cast<const u32x4*>(xrow + base);
    const u32x4 rq = *reinterpret_cast<const u32x4*>(rrow + base);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_to_f32((uint16_t)(xq[q] & 0xFFFFu)) * f16_to_f32((uint16_t)(rq[q] & 0xFFFFu));
      v[2 * q + 1] = bf16_to_f32((uint16_t)(xq[q] >> 16)) * f16_to_f32((uint16_t)(rq[q] >> 16));
    }
  };
  // The butterflies run in fwht128's order (bit 6, then bits 0-5), so the
  // rounded results are the same: bit 6 and bits 3-5 across lanes, bits
  // 0-2 inside the lane. The 16 lanes of a block are all in or all out of
  // the row (hidden is a multiple of 128).
  const float s1 = lane_sign(lane, 1), s2 = lane_sign(lane, 2), s4 = lane_sign(lane, 4);
  const float s8 = lane_sign(lane, 8);
  auto transform_store = [&](int base, float (&v)[8], float scale) {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = butterfly<8>(v[q], s8);  // bit 6
#pragma unroll
    for (int h = 1; h <= 4; h <<= 1)  // bits 0-2
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (!(q & h)) {
          const float lo = v[q], hi = v[q + h];
          v[q] = lo + hi;
          v[q + h] = lo - hi;
        }
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = butterfly<4>(butterfly<2>(butterfly<1>(v[q], s1), s2), s4);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const _Float16 lo = (_Float16)(v[2 * q] * scale);
      const _Float16 hi = (_Float16)(v[2 * q + 1] * scale);
      o[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<u32x4*>(a.xg + (size_t)i * H + base) = o;
  };
  // the row's largest |rin (.) x| -> its exponent
  auto row_scale = [&](float m) {
    m = wave_max(m);
    int ex = fp16_block_exp(16.0f * m);
    if (ex == kExpZeroBlock) ex = 0;
    if (lane == 0) a.xg_exp[i] = ex;
    return kInvSqrt128 * exp2i(ex);
  };
  if (nch <= kGatherHeld) {
    float v[kGatherHeld][8];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < kGatherHeld; ++j) {
      const int base = 8 * lane + 512 * j;
      if (j < nch && base < H) {
        load8(base, v[j]);
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[j][q]));
      }
    }
    const float scale = row_scale(m);
#pragma unroll
    for (int j = 0; j < kGatherHeld; ++j) {
      const int base = 8 * lane + 512 * j;
      if (j < nch && base < H) transform_store(base, v[j], scale);
    }
  } else {
    float m = 0.f;
    for (int base = 8 * lane; base < H; base += 512) {
      float v[8];
      load8(base, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
    }
    const float scale = row_scale(m);
    for (int base = 8 * lane; base < H; base += 512) {
      float v[8];
      load8(base, v);
      transform_store(base, v, scale);
    }
  }
}

// The same rows for small batches, where the work-groups of k_xin_gather
// would be too few to spread over the device: one work-group of 256 threads
// per pair (16 lanes per 128-input block, 8 inputs per lane), the row
// maximum across the four waves in LDS; the same arithmetic in the same
// order.
__global__ __launch_bounds__(256) void k_xin_gather_small(GatherArgs a) {
  __shared__ float wmax[4];
  const int p = blockIdx.x;
  const int i = a.inv[p];
  if (i < 0) return;  // uniform: an out-of-range expert id has no row
  const int e = a.ids[p];
  const int t = p / a.top_k;
  const int lane = threadIdx.x & 63;
  const int H = a.hidden;
  const uint16_t* xrow = a.x_bf16 + (size_t)t * H;
  const uint16_t* rrow = a.rin + (size_t)e * H;
  auto load8 = [&](int base, float (&v)[8]) {
    const u32x4 xq = *reinterpret_cast<const u32x4*>(xrow + base);
    const u32x4 rq = *reinterpret_cast<const u32x4*>(rrow + base);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_to_f32((uint16_t)(xq[q] & 0xFFFFu)) * f16_to_f32((uint16_t)(rq[q] & 0xFFFFu));
      v[2 * q + 1] = bf16_to_f32((uint16_t)(xq[q] >> 16)) * f16_to_f32((uint16_t)(rq[q] >> 16));
    }
  };
  float m = 0.f;
  for (int base = 8 * threadIdx.x; base < H; base += 8 * 256) {
    float v[8];
    load8(base, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
  }
  m = wave_max(m);
  if (lane == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  int ex = fp16_block_exp(16.0f * m);
  if (ex == kExpZeroBlock) ex = 0;
  if (threadIdx.x == 0) a.xg_exp[i] = ex;
  const float scale = kInvSqrt128 * exp2i(ex);
  const float s1 = lane_sign(lane, 1), s2 = lane_sign(lane, 2), s4 = lane_sign(lane, 4);
  const float s8 = lane_sign(lane, 8);
  for (int base = 8 * threadIdx.x; base < H; base += 8 * 256) {
    float v[8];
    load8(base, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = butterfly<8>(v[q], s8);  // bit 6
#pragma unroll
    for (int h = 1; h <= 4; h <<= 1)  // bits 0-2
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (!(q & h)) {
          const float lo = v[q], hi = v[q + h];
          v[q] = lo + hi;
          v[q + h] = lo - hi;
        }
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = butterfly<4>(butterfly<2>(butterfly<1>(v[q], s1), s2), s4);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const _Float16 lo = (_Float16)(v[2 * q] * scale);
      const _Float16 hi = (_Float16)(v[2 * q + 1] * scale);
      o[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<u32x4*>(a.xg + (size_t)i * H + base) = o;
  }
}

// ------------------------------------------------------------------------
// Shared main loop: acc[mt][tt] += W[256 outputs][K] * X[128 tokens][K]^T.
// Wave (wo, wt) = (wave >> 1, wave & 1) owns outputs 32*kMT*wo + 32*mt (mt < kMT)
// and tokens 64*wt + 32*tt (tt 0..1). Step s's matrix-core work is issued
// in the same loop body as the decode of step s+1 (into the other LDS
// buffer), so the VALU decode and the MFMAs overlap; codes run two steps
// and activations one step ahead.
// out_tile(j) maps the local output tile j (0..15) to its global tile index.
// ------------------------------------------------------------------------
// A lane's eighth of a tile: stream bits 32K*o .. 32K*o + 32K - 1 (input
// rows 2o and 2o+1), K dwords, plus the first dword of the next eighth (the
// windows reach at most 15 bits into it).
template <int K>
__device__ __forceinline__ void load_eighth(const uint16_t* te, uint32_t (&d)[K]) {
  if constexpr (K == 2) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(te));
    d[0] = v.x;
    d[1] = v.y;
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(te);
#pragma unroll
    for (int i = 0; i < K; ++i) d[i] = __builtin_nontemporal_load(p + i);
  }
}

// Offset (in halves) of the 16-byte chunk holding inputs 8kc .. 8kc + 7 of
// row `row` (0..255) of a step's W buffer: chunks of one kc are 256 rows
// apart, and rows are permuted as row ^ ((row >> 4) & 15) (see the header).
__device__ __forceinline__ int w_slot(int kc, int row) {
  return (kc * 256 + (row ^ ((row >> 4) & 15))) * 8;
}

// Decode the lane's 32 weights (input rows 2o, 2o+1 of tile (dkt, dnt) of
// the step, all 16 output columns) and store them to the W buffer at
// w_slot's positions.
template <int K>
__device__ __forceinline__ void decode_to_lds(const uint32_t (&raw)[K], int dkt, int dnt, int o,
                                              int lane, _Float16* wb) {
  uint32_t d[K + 1];
#pragma unroll
  for (int i = 0; i < K; ++i) d[i] = raw[i];
  // first dword of the next eighth of the same tile: lane 8t + (o+1) % 8
  d[K] = (uint32_t)__builtin_amdgcn_ds_bpermute(((lane & ~7) | ((lane + 1) & 7)) << 2, (int)raw[0]);
  uint32_t lo[8], hi[8];  // columns n and n+8: rows (2o, 2o+1)
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const uint32_t w0 = __builtin_bit_cast(uint32_t, cba_decode_pair(row_state_pair<K>(d, 0, n)));
    const uint32_t w1 = __builtin_bit_cast(uint32_t, cba_decode_pair(row_state_pair<K>(d, 1, n)));
    lo[n] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
    hi[n] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
  }
  // rows 16*dnt + n and 16*dnt + n + 8, inputs 16*dkt + 2o, +1 (one 4-byte pair)
  _Float16* chunk = wb + (2 * dkt + (o >> 2)) * (256 * 8) + 2 * (o & 3);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    *reinterpret_cast<uint32_t*>(chunk + (16 * dnt + (n ^ dnt)) * 8) = lo[n];
    *reinterpret_cast<uint32_t*>(chunk + (16 * dnt + ((n + 8) ^ dnt)) * 8) = hi[n];
  }
}

// One step's operands as held by a decoder lane between issue and use: its
// eighth of one code tile and two 16-byte chunks of the activation tile.
template <int K>
struct StepLoads {
  uint32_t raw[K];
  h8 x[2];
  int eb;  // exponent of the activations' 128-input block (rescaling loops)
};

// The matrix waves' part of every step: NT live 32-token sub-tiles (1 or 2)
// against kMT 32-row output tiles; operands of sub-step ks+1 are read from
// LDS while sub-step ks's MFMAs issue. One barrier per step, matching the
// decoder waves'.
template <int NT>
__device__ __forceinline__ void mma_steps(const _Float16* wl, const _Float16* xl, int n_steps, int wo,
                                          int wt, int lane, f32x16 (&acc)[kMT][2]) {
  constexpr int kKs = kStep / 16;
  const int l32 = lane & 31;
  const int khi = lane >> 5;
  int wrow[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) wrow[mt] = 32 * kMT * wo + 32 * mt + l32;
  for (int s = 0; s < n_steps; ++s) {
    const _Float16* wb = wl + (s & 1) * kWBuf;
    const _Float16* xb = xl + (s & 1) * kXBuf;
    auto load_ops = [&](int ks, h8 (&a)[kMT], h8 (&b)[2]) {
      const int kc = 2 * ks + khi;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
        b[tt] = *reinterpret_cast<const h8*>(xb + (kc * kTM + 64 * wt + 32 * tt + l32) * 8);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) a[mt] = *reinterpret_cast<const h8*>(wb + w_slot(kc, wrow[mt]));
    };
    h8 a0[kMT], b0[2], a1[kMT], b1[2];
    load_ops(0, a0, b0);
    // the scheduling barriers keep each sub-step's reads ahead of the
    // previous sub-step's MFMAs (left alone, the compiler sinks them to just
    // before their use to save registers and exposes every read's latency)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kKs; ks += 2) {
      load_ops(ks + 1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          acc[mt][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[mt], b0[tt], acc[mt][tt], 0, 0, 0);
      if (ks + 2 < kKs) load_ops(ks + 2, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          acc[mt][tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[mt], b1[tt], acc[mt][tt], 0, 0, 0);
    }
    __syncthreads();
  }
}

// The main loop runs over n_steps of the projection's 64-input steps:
// step i of the loop is input step step_of(i) (all steps in order for
// gate_up; the down kernel leaves out steps whose 128-channel block is zero
// for every token of the tile). RESCALE: the activation rows are stored
// with a power-of-two exponent per 128-input block (xexp [row][nblk]); each
// 16-byte chunk is rescaled to its row's exponent (row_exp) before it goes
// to LDS, so that a whole row enters the contraction at one scale.
// rexp_out (RESCALE, LDS): each token row's exponent, for the epilogue.
template <int K, bool RESCALE, class OutTile, class StepOf>
__device__ __forceinline__ void grouped_mainloop(const uint16_t* __restrict__ code_e, int n_nt,
                                                 int n_steps, StepOf step_of,
                                                 const _Float16* __restrict__ X, int x_pitch,
                                                 const int32_t* __restrict__ xexp, int nblk,
                                                 int row0, int rows, OutTile out_tile,
                                                 _Float16* wl, _Float16* xl,
                                                 f32x16 (&acc)[kMT][2], int* rexp_out = nullptr) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: uniform per wave
  const int lane = tid & 63;
  const bool decoder = wave < kDecWaves;

  if (decoder) {
    // waves 0-7: codes and activations of step i+2 are issued at step i
    // (two steps of latency cover); at step i the lane decodes step i+1's
    // eighth of a tile into W and copies its activation chunks into the X
    // tile.
    const int o = tid & 7;
    const int dtile = tid >> 3;
    const int dkt = dtile >> 4;  // tile-row inside the step
    const int dnt = dtile & 15;  // output tile inside the group
    const int gnt = out_tile(dnt);
    const int xtok = tid & 127;        // activation row of this lane
    const int xkc0 = 2 * (tid >> 7);   // first of its two 16-byte k-chunks
    const int xr = row0 + (xtok < rows ? xtok : rows - 1);
    const _Float16* xrow = X + (size_t)xr * x_pitch + 8 * xkc0;
    const int32_t* erow = RESCALE ? xexp + (size_t)xr * nblk : nullptr;
    const int e_row = RESCALE ? row_exp(erow, nblk) : 0;
    if (RESCALE && rexp_out && tid < kTM) rexp_out[xtok] = e_row;  // for the epilogue
    auto issue = [&](int i, StepLoads<K>& L) {
      const int st = step_of(i);
      load_eighth<K>(code_e + ((size_t)(4 * st + dkt) * n_nt + gnt) * (16 * K) + o * (2 * K), L.raw);
#pragma unroll
      for (int j = 0; j < 2; ++j) L.x[j] = *reinterpret_cast<const h8*>(xrow + st * kStep + 8 * j);
      if constexpr (RESCALE) L.eb = erow[(st * kStep) >> 7];
    };
    auto consume = [&](int i, StepLoads<K>& L) {
      decode_to_lds<K>(L.raw, dkt, dnt, o, lane, wl + (i & 1) * kWBuf);
      _Float16* xb = xl + (i & 1) * kXBuf;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        h8 v = L.x[j];
        if constexpr (RESCALE) v = rescale_h8(v, block_shift(e_row, L.eb));
        *reinterpret_cast<h8*>(xb + ((xkc0 + j) * kTM + xtok) * 8) = v;
      }
    };
    StepLoads<K> ring[2];
    if (n_steps > 0) {
      issue(0, ring[0]);
      if (n_steps > 1) issue(1, ring[1]);
      consume(0, ring[0]);
      if (n_steps > 2) issue(2, ring[0]);
    }
    __syncthreads();
    // step i consumes ring[(i+1)&1] (issued two steps earlier) and reuses it
    for (int i = 0; i < n_steps; i += 2) {
      if (i + 1 < n_steps) {
        consume(i + 1, ring[1]);
        if (i + 3 < n_steps) issue(i + 3, ring[1]);
      }
      __syncthreads();
      if (i + 1 < n_steps) {
        if (i + 2 < n_steps) {
          consume(i + 2, ring[0]);
          if (i + 4 < n_steps) issue(i + 4, ring[0]);
        }
        __syncthreads();
      }
    }
  } else {
    // the other waves: matrix cores on step i from LDS. (wo, wt): outputs
    // 32*kMT*wo + 32*mt, tokens 64*wt + 32*tt. Token sub-tiles without a real
    // token are skipped (uniform per wave); padded columns of a live
    // sub-tile hold a clamped row and are never stored.
    const int mw = wave - kDecWaves;
    const int wo = mw >> 1, wt = mw & 1;
    const int live = 64 * wt + 32 < rows ? 2 : (64 * wt < rows ? 1 : 0);
    __syncthreads();
    if (live == 2)
      mma_steps<2>(wl, xl, n_steps, wo, wt, lane, acc);
    else if (live == 1)
      mma_steps<1>(wl, xl, n_steps, wo, wt, lane, acc);
    else
      for (int i = 0; i < n_steps; ++i) __syncthreads();
  }
}

// Accumulators of every matrix wave -> LDS E[128 tokens][256 outputs]
// (fp32; token 64 wt + 32 tt + column).
__device__ __forceinline__ void acc_to_lds(const f32x16 (&acc)[kMT][2], float* el) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave < kDecWaves) return;
  const int wo = (wave - kDecWaves) >> 1, wt = (wave - kDecWaves) & 1;
  const int j = 64 * wt + (lane & 31);  // token of column lane & 31
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        // rows 8 r4 + 4 (lane >> 5) .. + 3 of the 32x32 tile: one 16-byte store
        const int i = 8 * r4 + 4 * (lane >> 5);
        *reinterpret_cast<f32x4*>(&el[(32 * tt + j) * kEPitch + 32 * kMT * wo + 32 * mt + i]) =
            f32x4{acc[mt][tt][4 * r4], acc[mt][tt][4 * r4 + 1], acc[mt][tt][4 * r4 + 2],
                  acc[mt][tt][4 * r4 + 3]};
      }
}

// ------------------------------------------------------------------------
// Work-group -> (tile, output block) so that all nb blocks of a tile run on
// one XCD, one after another in its dispatch order: the hardware deals
// work-groups to the 8 XCDs in turn (block b to XCD b % 8), so XCD x takes
// tiles x, x + 8, ... and each tile's activations come from HBM into that
// XCD's L2 once, not once per block. The grid is a multiple of 8 nb
// covering every tile (grouped_grid).
// ------------------------------------------------------------------------
__device__ __forceinline__ void xcd_tile_block(int nb, int& tile, int& blk) {
  const int b = blockIdx.x;
  const int slot = b >> 3;  // the slot-th work-group of XCD b % 8
  tile = 8 * (slot / nb) + (b & 7);
  blk = slot % nb;
}
__host__ __device__ constexpr unsigned grouped_grid(int max_tiles, int nb) {
  return (unsigned)(((max_tiles + 7) / 8) * 8 * nb);
}

// ------------------------------------------------------------------------
// gate_up, grouped. grid.x = grouped_grid(max_tiles, inter / 128), block = kThreads.
// A work-group takes the gate rows and the up rows of one 128-channel block
// c (256 outputs) for one tile; its epilogue undoes the input rows'
// exponents, finishes h = SiLU(gate) * up for those channels and writes
// down's rotated fp16 input block c with the block's own exponent.
// ------------------------------------------------------------------------

// Down's rotated input block (v0 at channel lane, v1 at lane + 64, before
// the 1/sqrt(128) of H_n) of sorted row i, as fp16 scaled by the block's
// exponent, and the exponent. Whole wave.
__device__ __forceinline__ void store_down_input(const GroupedArgs& a, int i, int c, float v0, float v1,
                                                 int lane) {
  const bool nan = __ballot(v0 != v0 || v1 != v1) != 0;
  const float m = wave_max(fmaxf(fabsf(v0), fabsf(v1))) * kInvSqrt128;
  int ex = nan ? 0 : fp16_block_exp(m);
  const float scale = kInvSqrt128 * exp2i(ex == kExpZeroBlock ? 0 : ex);
  _Float16* xo = reinterpret_cast<_Float16*>(a.x_out) + (size_t)i * a.inter + 128 * c;
  xo[lane] = (_Float16)(v0 * scale);
  xo[lane + 64] = (_Float16)(v1 * scale);
  if (lane == 0) a.x_exp_out[(size_t)i * (a.inter / 128) + c] = ex;
}

template <int K>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_grouped_gate_up(GroupedArgs a) {
  const int nb = a.inter / 128;
  int c, tile;
  xcd_tile_block(nb, tile, c);
  if (tile >= *a.n_tiles) return;  // uniform
  const int e = a.t_expert[tile];
  const int row0 = a.t_row0[tile];
  const int rows = a.t_rows[tile];
  const int n_nt = 2 * a.inter / 16;
  const int gate_nt0 = 8 * c, up_nt0 = a.inter / 16 + 8 * c;
  const uint16_t* code_e = a.code + (size_t)e * (size_t)(a.hidden / 16) * n_nt * (16 * K);

  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __shared__ int rexp[kTM];  // the tile's input row exponents (read after the main loop's barriers)
  if (threadIdx.x < rows) rexp[threadIdx.x] = a.x_exp_in[row0 + threadIdx.x];
  _Float16* wl = reinterpret_cast<_Float16*>(smem);
  _Float16* xl = wl + 2 * kWBuf;
  f32x16 acc[kMT][2];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][tt][r] = 0.f;
  grouped_mainloop<K, false>(code_e, n_nt, a.hidden / kStep, [](int i) { return i; },
                             reinterpret_cast<const _Float16*>(a.x_in), a.hidden, nullptr, 0, row0,
                             rows, [&](int j) { return j < 8 ? gate_nt0 + j : up_nt0 + j - 8; }, wl,
                             xl, acc);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint16_t* rg = a.rout + (size_t)e * (2 * a.inter) + 128 * c;
  const uint16_t* ru = rg + a.inter;
  const uint16_t* rd = a.rin2 + (size_t)e * a.inter + 128 * c;
  const float rg0 = f16_to_f32(rg[lane]), rg1 = f16_to_f32(rg[lane + 64]);
  const float ru0 = f16_to_f32(ru[lane]), ru1 = f16_to_f32(ru[lane + 64]);
  const float rd0 = f16_to_f32(rd[lane]), rd1 = f16_to_f32(rd[lane + 64]);
  // the dense export's gate/up biases (zero for routed experts)
  const float* bg = a.bias ? a.bias + 128 * c : nullptr;
  const float bg0 = bg ? bg[lane] : 0.f, bg1 = bg ? bg[lane + 64] : 0.f;
  const float bu0 = bg ? bg[a.inter + lane] : 0.f, bu1 = bg ? bg[a.inter + lane + 64] : 0.f;
  float* el = reinterpret_cast<float*>(smem);
  // every wave takes tokens wave, wave + kWaves, ... of the tile, two at a time
  // (two independent butterfly chains in flight)
  auto two_tokens = [&](int tla) {
    bool ok[2];
    float g0[2], g1[2], u0[2], u1[2], us[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tl = tla + kWaves * q;
      ok[q] = tl < kTM && tl < rows;  // uniform over the wave
      const float* er = el + (ok[q] ? tl : 0) * kEPitch;
      g0[q] = er[lane];
      g1[q] = er[lane + 64];
      u0[q] = er[128 + lane];
      u1[q] = er[192 + lane];
      us[q] = exp2i(-rexp[ok[q] ? tl : 0]);  // undo the input row's scale
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      fwht128(g0[q], g1[q]);
      fwht128(u0[q], u1[q]);
    }
    float v0[2], v1[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float h0 = silu(g0[q] * (kInvSqrt128 * rg0) * us[q] + bg0) * (u0[q] * (kInvSqrt128 * ru0) * us[q] + bu0);
      const float h1 = silu(g1[q] * (kInvSqrt128 * rg1) * us[q] + bg1) * (u1[q] * (kInvSqrt128 * ru1) * us[q] + bu1);
      if (ok[q] && a.inter_out) {
        float* io = a.inter_out + (size_t)a.perm[row0 + tla + kWaves * q] * a.inter + 128 * c;
        io[lane] = h0;
        io[lane + 64] = h1;
      }
      v0[q] = h0 * rd0;
      v1[q] = h1 * rd1;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) fwht128(v0[q], v1[q]);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!ok[q]) continue;
      store_down_input(a, row0 + tla + kWaves * q, c, v0[q], v1[q], lane);
    }
  };
  acc_to_lds(acc, el);
  __syncthreads();
  for (int tla = wave; tla < kTM; tla += 2 * kWaves) two_tokens(tla);
}

// The 128-channel blocks of down's input that are nonzero for some token
// of the tile (rows row0 .. row0 + rows - 1), as the list of their 64-input
// steps in order: steps[0 .. n) in LDS; returns n. A block that is exactly
// zero for every token contributes exactly zero, so its codes are neither
// loaded nor decoded. Whole work-group (ends with a barrier).
__device__ __forceinline__ int live_down_steps(const int32_t* __restrict__ xexp, int nblk, int row0,
                                               int rows, int* live_blk, int* steps) {
  for (int c = threadIdx.x; c < nblk; c += blockDim.x) live_blk[c] = 0;
  __syncthreads();
  for (int idx = threadIdx.x; idx < rows * nblk; idx += blockDim.x)
    if (xexp[(size_t)(row0 + idx / nblk) * nblk + idx % nblk] != kExpZeroBlock) live_blk[idx % nblk] = 1;
  __syncthreads();
  int n = 0;
  for (int c = 0; c < nblk; ++c)
    if (live_blk[c]) n += 128 / kStep;
  if (threadIdx.x == 0) {
    int j = 0;
    for (int c = 0; c < nblk; ++c)
      if (live_blk[c])
        for (int q = 0; q < 128 / kStep; ++q) steps[j++] = c * (128 / kStep) + q;
  }
  __syncthreads();
  return n;
}

// ------------------------------------------------------------------------
// down, grouped. grid.x = grouped_grid(max_tiles, hidden / 256), block = kThreads. The
// epilogue undoes the row's exponent, applies H_n, rout and the pair's
// router weight and stores the pair's 256 outputs (fp32) at its sorted index.
// ------------------------------------------------------------------------
constexpr int kMaxDownBlocks = 64;  // inter <= 8192 for the zero-block skip

template <int K>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_grouped_down(GroupedArgs a) {
  const int ng = a.hidden / 256;
  int r, tile;
  xcd_tile_block(ng, tile, r);
  if (tile >= *a.n_tiles) return;
  const int e = a.t_expert[tile];
  const int row0 = a.t_row0[tile];
  const int rows = a.t_rows[tile];
  const int n_nt = a.hidden / 16;
  const int nblk = a.inter / 128;
  const uint16_t* code_e = a.code + (size_t)e * (size_t)(a.inter / 16) * n_nt * (16 * K);

  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __shared__ int live_blk[kMaxDownBlocks];
  __shared__ int steps[kMaxDownBlocks * (128 / kStep)];
  __shared__ int rexp[kTM];  // the tile's row exponents (written in the main loop)
  int n_steps = a.inter / kStep;
  const bool skip = nblk <= kMaxDownBlocks;  // uniform
  if (skip) n_steps = live_down_steps(a.x_exp_in, nblk, row0, rows, live_blk, steps);
  _Float16* wl = reinterpret_cast<_Float16*>(smem);
  _Float16* xl = wl + 2 * kWBuf;
  f32x16 acc[kMT][2];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mt][tt][q] = 0.f;
  grouped_mainloop<K, true>(code_e, n_nt, n_steps, [&](int i) { return skip ? steps[i] : i; },
                            reinterpret_cast<const _Float16*>(a.x_in), a.inter, a.x_exp_in, nblk, row0,
                            rows, [&](int j) { return 16 * r + j; }, wl, xl, acc, rexp);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint16_t* ro = a.rout + (size_t)e * a.hidden + 256 * r;
  const float r00 = f16_to_f32(ro[lane]), r01 = f16_to_f32(ro[lane + 64]);
  const float r10 = f16_to_f32(ro[128 + lane]), r11 = f16_to_f32(ro[192 + lane]);
  float* el = reinterpret_cast<float*>(smem);
  // every wave takes tokens wave, wave + kWaves, ... of the tile, two at a time
  auto two_tokens = [&](int tla) {
    bool ok[2];
    float z0[2], z1[2], z2[2], z3[2], wt[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tl = tla + kWaves * q;
      ok[q] = tl < kTM && tl < rows;  // uniform over the wave
      const float* er = el + (ok[q] ? tl : 0) * kEPitch;
      z0[q] = er[lane];
      z1[q] = er[lane + 64];
      z2[q] = er[128 + lane];
      z3[q] = er[192 + lane];
      // the router weight, with the row's input exponent undone
      wt[q] = ok[q] ? a.w[a.perm[row0 + tl]] * exp2i(-rexp[tl]) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      fwht128(z0[q], z1[q]);
      fwht128(z2[q], z3[q]);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!ok[q]) continue;
      const int i = row0 + tla + kWaves * q;
      float* yo = a.y_out + (size_t)i * a.hidden + 256 * r;
      yo[lane] = z0[q] * kInvSqrt128 * r00 * wt[q];
      yo[lane + 64] = z1[q] * kInvSqrt128 * r01 * wt[q];
      yo[128 + lane] = z2[q] * kInvSqrt128 * r10 * wt[q];
      yo[192 + lane] = z3[q] * kInvSqrt128 * r11 * wt[q];
    }
  };
  acc_to_lds(acc, el);
  __syncthreads();
  for (int tla = wave; tla < kTM; tla += 2 * kWaves) two_tokens(tla);
}

// ------------------------------------------------------------------------
// Small tiles (decode calls with few tokens per expert): a tile holds at
// most 16 pairs of one expert, and every wave decodes its share of the
// expert's weights straight into the A operands of v_mfma_f32_16x16x32_f16
// (no LDS copy of the weights, no barrier per step); B holds the tile's
// fp16 activations, one column per token. Wave w takes output quad w % 4
// (four 16-output tiles) and input half w / 4; the halves are added in LDS
// (half 0 + half 1) before the epilogue. Work-group: 8 waves.
// ------------------------------------------------------------------------
constexpr int kSmallTM = 16;
constexpr int kSmallMaxBlocks = 16;  // small tiles: inter <= 2048 (the host checks)

struct SmallLds {
  uint32_t stage[8 * Stage<3>::kDw];  // each wave's staged codes
  float red[2][kSmallTM][256];        // per input half: [token][output]
  int rexp[kSmallTM];                 // down: each token's row exponent
};

// The wave's partial sums over chunks c0 .. c0 + nch - 1 of the 16 output
// columns nt0 .. nt0 + 3; the tile's token rows are rows row0 .. row0 +
// rows - 1 of X (pitch x_pitch; the columns of tokens >= rows read row row0
// and are never stored); lane (n, g) ends with outputs 16j + 4g + q of tile
// j for token n in D[j][q]. RESCALE: X carries an exponent per 128-input
// block (xexp [row][nblk]); a chunk that is zero for every token of the
// tile is skipped, and each chunk's activations are rescaled to the row's
// exponent before their contraction; the lanes n < 16 store the row
// exponent of token n at rexp_out[n] when rexp_out is not null.
template <int K, bool RESCALE, bool FRESH = false>
__device__ __forceinline__ void small_mainloop(const uint16_t* __restrict__ code_e, int n_nt, int c0,
                                               int nch, int nt0, const _Float16* __restrict__ X,
                                               int x_pitch, const int32_t* __restrict__ xexp, int nblk,
                                               int row0, int rows, uint32_t* stage, int lane,
                                               f32x4 (&D)[4], int* rexp_out) {
  const int n = lane & 15;
  const int gq = lane >> 4;
  const int xr = row0 + (n < rows ? n : 0);
  const _Float16* xrow = X + (size_t)xr * x_pitch;
#pragma unroll
  for (int j = 0; j < 4; ++j) D[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int cend = c0 + nch;
  // the first chunk's codes go out before anything else
  u32x4 cv[Stage<K>::kPerLane];
  stage_issue<K>(code_e, n_nt, 8 * c0, nt0, lane, cv);
  // the row's block exponents, loaded together once (nblk <= kSmallMaxBlocks):
  // the row exponent (stored at rexp_out[n] by the lanes n < 16 when
  // rexp_out is given), which chunks of this half are live for some token of
  // the tile (a bit per chunk, uniform), and each chunk's shift to the row
  // exponent, packed as -shift / 8 in four bits per chunk (7: the block
  // rounds to zero). Nothing else of the exponents stays live in the loop,
  // which runs at the register limit.
  uint32_t live_bits = 0xFFFFFFFFu;
  uint32_t sh_pack = 0;
  if constexpr (RESCALE) {
    const int32_t* erow = xexp + (size_t)xr * nblk;
    // clamped indices: every load is issued unconditionally, back to back
    // (a load under a branch would be waited for before the branch)
    auto ld = [&](int b) {  // FRESH: past the compute unit's cache (written during this launch)
      if constexpr (FRESH)
        return __hip_atomic_load(const_cast<int32_t*>(erow + b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        return erow[b];
    };
    int eb_all[kSmallMaxBlocks], eb_half[kSmallMaxBlocks / 2];
#pragma unroll
    for (int b = 0; b < kSmallMaxBlocks; ++b) eb_all[b] = ld(b < nblk ? b : nblk - 1);
#pragma unroll
    for (int ch = 0; ch < kSmallMaxBlocks / 2; ++ch) eb_half[ch] = ld(c0 + (ch < nch ? ch : 0));
    int emin = kExpZeroBlock;
#pragma unroll
    for (int b = 0; b < kSmallMaxBlocks; ++b) emin = eb_all[b] < emin ? eb_all[b] : emin;
    const int e_row = emin == kExpZeroBlock ? 0 : emin;
    if (rexp_out != nullptr && lane < kSmallTM) rexp_out[lane] = e_row;  // lane n: token n
    live_bits = 0;
#pragma unroll
    for (int ch = 0; ch < kSmallMaxBlocks / 2; ++ch) {
      if (__ballot(ch < nch && n < rows && eb_half[ch] != kExpZeroBlock) != 0) live_bits |= 1u << ch;
      const int q = -block_shift(e_row, eb_half[ch]) >> 3;  // exponents are multiples of 8
      sh_pack |= (uint32_t)(q < 7 ? q : 7) << (4 * ch);
    }
  }
  auto live = [&](int c) { return ((live_bits >> (c - c0)) & 1u) != 0; };  // uniform
  auto next_live = [&](int c) {  // first live chunk after c, or cend
    for (++c; c < cend && !live(c); ++c) {
    }
    return c;
  };
  // the first chunk is always contracted (its codes are already on the
  // way; a dead first chunk only adds zeros), later dead chunks are skipped
  int c = c0;
  do {
    const int cn = next_live(c);
    stage_store<K>(stage, lane, cv);
    // the chunk's activations, then the next chunk's codes (past the last
    // chunk: this chunk's again, never used), all in flight during the
    // decode; issued unconditionally, so that the wait before the MFMAs
    // leaves the codes outstanding
    h16x8 B[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
      B[pp] = *reinterpret_cast<const h16x8*>(xrow + 128 * c + 32 * pp + 8 * gq);
    const int sh = RESCALE ? -8 * (int)((sh_pack >> (4 * (c - c0))) & 7u) : 0;
    stage_issue<K>(code_e, n_nt, 8 * (cn < cend ? cn : c), nt0, lane, cv);
    // the chunk's activations at the row's exponent (this waits for their
    // loads only: the next chunk's codes stay in flight)
    if constexpr (RESCALE) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) B[pp] = rescale_h8(B[pp], sh);
    }
    // tile-row pairs decoded one ahead of their MFMAs into two operand sets
    // (32 VGPRs instead of 64): pair pp's MFMAs run on the matrix core while
    // pair pp + 1 (then pp + 2, into pp's freed set) is decoded
    const OperandDecoder<K> dec(stage, lane);
    h16x8 A0[4], A1[4];
    dec.template decode<0>(A0);
    dec.template decode<1>(A1);
    auto mfma4 = [&](const h16x8 (&A)[4], const h16x8& b) {
#pragma unroll
      for (int j = 0; j < 4; ++j) D[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[j], b, D[j], 0, 0, 0);
    };
    mfma4(A0, B[0]);
    dec.template decode<2>(A0);
    mfma4(A1, B[1]);
    dec.template decode<3>(A1);
    mfma4(A0, B[2]);
    mfma4(A1, B[3]);
    c = cn;
  } while (c < cend);
}

// D of a wave (output quad nq, input half kh) -> sh.red[kh][token][output].
__device__ __forceinline__ void small_to_lds(const f32x4 (&D)[4], SmallLds& sh, int kh, int nq,
                                             int lane) {
  const int n = lane & 15;
  const int gq = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<float4*>(&sh.red[kh][n][16 * (4 * nq + j) + 4 * gq]) =
        make_float4(D[j][0], D[j][1], D[j][2], D[j][3]);
}

// The gate_up main loop for tiles of at most 8 tokens at K = 2, in the
// tile-pair layout (TilePairDecoder: 9 VALU operations per pair of weights
// instead of 11): the wave's partial sums over chunks c0 .. c0 + nch - 1 of
// output tiles nt0 .. nt0 + 3, D[jp] for the tile pair (2 jp, 2 jp + 1). The
// tile's rows are row0 .. row0 + rows - 1 of X (rows <= 8; the columns of
// tokens >= rows read row row0 and are never stored).
__device__ __forceinline__ void small_mainloop_pairs(const uint16_t* __restrict__ code_e, int n_nt, int c0,
                                                     int nch, int nt0, const _Float16* __restrict__ X,
                                                     int x_pitch, int row0, int rows, uint32_t* stage,
                                                     int lane, f32x4 (&D)[2]) {
  const int tk = lane & 7;          // B column 8 par + tk: token tk
  const int par = (lane >> 3) & 1;
  const _Float16* xrow = X + (size_t)(row0 + (tk < rows ? tk : 0)) * x_pitch + 4 * (lane >> 4);
  D[0] = D[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 cv[Stage<2>::kPerLane];
  stage_issue<2>(code_e, n_nt, 8 * c0, nt0, lane, cv);
  const TilePairDecoder dec(stage, lane);
  for (int c = c0; c < c0 + nch; ++c) {
    stage_store<2>(stage, lane, cv);
    // the chunk's activations (inputs 16 tr + 4 g .. + 3 of token tk), then
    // the next chunk's codes, in flight during the decode
    u32x2 xa[8];
#pragma unroll
    for (int tr = 0; tr < 8; ++tr) xa[tr] = *reinterpret_cast<const u32x2*>(xrow + 128 * c + 16 * tr);
    const int cn = c + 1 < c0 + nch ? c + 1 : c;
    stage_issue<2>(code_e, n_nt, 8 * cn, nt0, lane, cv);
    auto step = [&](auto trc) {
      constexpr int TR = decltype(trc)::value;
      const h16x8 B = parity_operand(xa[TR], par);
      D[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dec.template decode<TR, 0>(), B, D[0], 0, 0, 0);
      D[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dec.template decode<TR, 1>(), B, D[1], 0, 0, 0);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 7>{});
  }
}

// Accumulators of small_mainloop_pairs -> sh.red[kh][token][output]: lane
// (8 par + tk, g) holds rows 4 g .. 4 g + 3 of D[jp], i.e. columns 4 (g & 1)
// + r + 8 par of tile 2 jp + (g >> 1) for token tk.
__device__ __forceinline__ void small_pairs_to_lds(const f32x4 (&D)[2], SmallLds& sh, int kh, int nq, int lane) {
  const int tk = lane & 7, par = (lane >> 3) & 1, g = lane >> 4;
#pragma unroll
  for (int jp = 0; jp < 2; ++jp)
    *reinterpret_cast<float4*>(&sh.red[kh][tk][16 * (4 * nq + 2 * jp + (g >> 1)) + 8 * par + 4 * (g & 1)]) =
        make_float4(D[jp][0], D[jp][1], D[jp][2], D[jp][3]);
}

// gate_up, small tiles. grid.x = max_tiles * (inter / 128), block = 512.
// A work-group takes gate block c and up block c (256 outputs, quads 0-1
// and 2-3) of one tile; its epilogue is the big tile kernel's: the input
// rows' exponents undone, h = SiLU(gate) * up for the block's channels,
// then down's rotated input with the block's exponent.
template <int K>
__device__ __forceinline__ void small_gate_up_block(const GroupedArgs& a, int tile, int c, SmallLds& sh) {
  const int e = a.t_expert[tile];
  const int row0 = a.t_row0[tile];
  const int rows = a.t_rows[tile];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nq = wave & 3, kh = wave >> 2;
  const int n_nt = 2 * a.inter / 16;
  const int ncg = a.hidden / 128;
  const int nt0 = nq < 2 ? 8 * c + 4 * nq : a.inter / 16 + 8 * c + 4 * (nq - 2);
  const uint16_t* code_e = a.code + (size_t)e * (size_t)ncg * 8 * n_nt * (16 * K);
  if (threadIdx.x < rows) sh.rexp[threadIdx.x] = a.x_exp_in[row0 + threadIdx.x];  // read after the barrier below
  bool pairs = false;
  if constexpr (K == 2) pairs = rows <= 8;  // uniform
  if (pairs) {
    f32x4 D[2];
    small_mainloop_pairs(code_e, n_nt, kh * (ncg / 2), ncg / 2, nt0, reinterpret_cast<const _Float16*>(a.x_in),
                         a.hidden, row0, rows, sh.stage + wave * Stage<K>::kDw, lane, D);
    small_pairs_to_lds(D, sh, kh, nq, lane);
  } else {
    f32x4 D[4];
    small_mainloop<K, false>(code_e, n_nt, kh * (ncg / 2), ncg / 2, nt0,
                             reinterpret_cast<const _Float16*>(a.x_in), a.hidden, nullptr, 0, row0, rows,
                             sh.stage + wave * Stage<K>::kDw, lane, D, nullptr);
    small_to_lds(D, sh, kh, nq, lane);
  }
  __syncthreads();
  const uint16_t* rg = a.rout + (size_t)e * (2 * a.inter) + 128 * c;
  const uint16_t* ru = rg + a.inter;
  const uint16_t* rd = a.rin2 + (size_t)e * a.inter + 128 * c;
  const float rg0 = f16_to_f32(rg[lane]), rg1 = f16_to_f32(rg[lane + 64]);
  const float ru0 = f16_to_f32(ru[lane]), ru1 = f16_to_f32(ru[lane + 64]);
  const float rd0 = f16_to_f32(rd[lane]), rd1 = f16_to_f32(rd[lane + 64]);
  const float* bg = a.bias ? a.bias + 128 * c : nullptr;  // dense gate/up biases
  const float bg0 = bg ? bg[lane] : 0.f, bg1 = bg ? bg[lane + 64] : 0.f;
  const float bu0 = bg ? bg[a.inter + lane] : 0.f, bu1 = bg ? bg[a.inter + lane + 64] : 0.f;
  for (int tok = 2 * wave; tok < 2 * wave + 2; ++tok) {
    if (tok >= rows) break;  // uniform over the wave
    const int i = row0 + tok;
    const float us = exp2i(-sh.rexp[tok]);  // undo the input row's scale
    const float* r0 = sh.red[0][tok];
    const float* r1 = sh.red[1][tok];
    float g0 = r0[lane] + r1[lane], g1 = r0[lane + 64] + r1[lane + 64];
    float u0 = r0[128 + lane] + r1[128 + lane], u1 = r0[192 + lane] + r1[192 + lane];
    fwht128(g0, g1);
    fwht128(u0, u1);
    g0 = g0 * (kInvSqrt128 * rg0) * us + bg0;
    g1 = g1 * (kInvSqrt128 * rg1) * us + bg1;
    u0 = u0 * (kInvSqrt128 * ru0) * us + bu0;
    u1 = u1 * (kInvSqrt128 * ru1) * us + bu1;
    const float h0 = silu(g0) * u0;
    const float h1 = silu(g1) * u1;
    if (a.inter_out) {
      float* io = a.inter_out + (size_t)a.perm[i] * a.inter + 128 * c;
      io[lane] = h0;
      io[lane + 64] = h1;
    }
    float v0 = h0 * rd0, v1 = h1 * rd1;
    fwht128(v0, v1);
    store_down_input(a, i, c, v0, v1, lane);
  }
}

template <int K>
__global__ __launch_bounds__(512, 4) void k_small_gate_up(GroupedArgs a) {
  const int nb = a.inter / 128;
  const int c = blockIdx.x % nb;
  const int tile = blockIdx.x / nb;
  if (tile >= *a.n_tiles) return;  // uniform
  __shared__ SmallLds sh;
  small_gate_up_block<K>(a, tile, c, sh);
}

// down, small tiles. grid.x = max_tiles * (hidden / 256), block = 512. The
// epilogue undoes the row's exponent, applies H_n, rout and the pair's
// router weight and stores the pair's 256 outputs (fp32) at its sorted
// index. 128-channel blocks that are zero for every token of the tile are
// skipped.
// FRESH: down's input exponents were written during this launch (by the
// gate_up blocks of the one-launch layer kernel), so they are read with
// loads that go past the compute unit's cache.
template <int K, bool FRESH = false>
__device__ __forceinline__ void small_down_block(const GroupedArgs& a, int tile, int r, SmallLds& sh) {
  const int e = a.t_expert[tile];
  const int row0 = a.t_row0[tile];
  const int rows = a.t_rows[tile];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nq = wave & 3, kh = wave >> 2;
  const int n_nt = a.hidden / 16;
  const int ncd = a.inter / 128;
  const uint16_t* code_e = a.code + (size_t)e * (size_t)ncd * 8 * n_nt * (16 * K);
  f32x4 D[4];
  small_mainloop<K, true, FRESH>(code_e, n_nt, kh * (ncd / 2), ncd / 2, 16 * r + 4 * nq,
                          reinterpret_cast<const _Float16*>(a.x_in), a.inter, a.x_exp_in, ncd, row0, rows,
                          sh.stage + wave * Stage<K>::kDw, lane, D, wave == 0 ? sh.rexp : nullptr);
  small_to_lds(D, sh, kh, nq, lane);
  __syncthreads();
  const uint16_t* ro = a.rout + (size_t)e * a.hidden + 256 * r;
  const float r00 = f16_to_f32(ro[lane]), r01 = f16_to_f32(ro[lane + 64]);
  const float r10 = f16_to_f32(ro[128 + lane]), r11 = f16_to_f32(ro[192 + lane]);
  for (int tok = 2 * wave; tok < 2 * wave + 2; ++tok) {
    if (tok >= rows) break;
    const int i = row0 + tok;
    // the router weight, with the row's input exponent undone
    const float wt = a.w[a.perm[i]] * exp2i(-sh.rexp[tok]);
    const float* q0 = sh.red[0][tok];
    const float* q1 = sh.red[1][tok];
    float z0 = q0[lane] + q1[lane], z1 = q0[lane + 64] + q1[lane + 64];
    float z2 = q0[128 + lane] + q1[128 + lane], z3 = q0[192 + lane] + q1[192 + lane];
    fwht128(z0, z1);
    fwht128(z2, z3);
    float* yo = a.y_out + (size_t)i * a.hidden + 256 * r;
    yo[lane] = z0 * kInvSqrt128 * r00 * wt;
    yo[lane + 64] = z1 * kInvSqrt128 * r01 * wt;
    yo[128 + lane] = z2 * kInvSqrt128 * r10 * wt;
    yo[192 + lane] = z3 * kInvSqrt128 * r11 * wt;
  }
}

template <int K>
__global__ __launch_bounds__(512, 4) void k_small_down(GroupedArgs a) {
  const int ng = a.hidden / 256;
  const int r = blockIdx.x % ng;
  const int tile = blockIdx.x / ng;
  if (tile >= *a.n_tiles) return;  // uniform
  __shared__ SmallLds sh;
  small_down_block<K>(a, tile, r, sh);
}

// ------------------------------------------------------------------------
// One small-tile layer in one launch: the gate_up blocks of every tile and
// then its down blocks, as tasks that the work-groups of each XCD claim in
// order from the XCD's ticket (task 8 j + x is the j-th claim on XCD x). All
// of tile t's tasks run on XCD t % 8, so the hand-off of down's input stays
// in that XCD's L2: a gate_up block stores its part of the input, waits
// until the stores are done and sets its flag with a plain store (which
// lands in the L2); a down block polls the tile's flags with loads that
// read the L2 and then reads the input. No compute unit can hold a stale
// copy of that input in its cache: each 1 KiB row belongs to one tile and
// is read only after the tile's flags, and the exponents (16 bytes per row,
// several tiles to a cache line) are read past the cache. A down block
// waits only for gate_up blocks, which have smaller numbers on the same XCD
// and are claimed first, so the smallest unfinished task can always run.
// Waits are bounded (0.5 s of the 100 MHz clock) and set the error word
// when they give up. The down blocks of the first tiles run while the last
// gate_up blocks do, where two launches would leave the device part idle.
// Control block, zeroed before the launch (by the grouping kernel): ticket
// of XCD x at word 32 x, the error word at kSmallCtlErr, and from
// kSmallCtlFlags the flag of tile t's gate_up block c at t * (inter / 128) + c.
// ------------------------------------------------------------------------
constexpr long long kSmallWaitTicks = 50000000;

__device__ __forceinline__ int xcd_of_this_wave() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xF;  // HW_REG_XCC_ID, bits 3:0
}

template <int KG, int KD>
__global__ __launch_bounds__(512, 4) void k_small_layer(GroupedArgs gu, GroupedArgs dn, int32_t* ctl) {
  __shared__ SmallLds sh;
  __shared__ int claim[2];
  if (threadIdx.x == 0) {
    const int x = xcd_of_this_wave();
    const int nt = *gu.n_tiles;
    const int j = x < 8 ? __hip_atomic_fetch_add(ctl + 32 * x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    claim[0] = x < 8 ? 8 * j + x : -1;
    claim[1] = nt;
  }
  __syncthreads();
  const int task = claim[0], nt = claim[1];
  const int nb = gu.inter / 128, ng = dn.hidden / 256;
  const int n8 = (nt + 7) / 8;
  const int n_gu = 8 * nb * n8, n_dn = 8 * ng * n8;
  if (task < 0 || task >= n_gu + n_dn) return;  // uniform: a surplus work-group
  int32_t* flags = ctl + kSmallCtlFlags;
  if (task < n_gu) {
    const int j = task >> 3;
    const int tile = 8 * (j / nb) + (task & 7);
    const int c = j % nb;
    if (tile >= nt) return;
    small_gate_up_block<KG>(gu, tile, c, sh);
    // every wave's stores of down's input are done, then the flag
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) *(volatile int32_t*)(flags + tile * nb + c) = 1;
  } else {
    const int t2 = task - n_gu;
    const int j = t2 >> 3;
    const int tile = 8 * (j / ng) + (t2 & 7);
    const int r = j % ng;
    if (tile >= nt) return;
    if (threadIdx.x < 64) {  // wave 0: lane c < nb polls gate_up block c's flag
      int32_t* f = flags + tile * nb + (threadIdx.x < nb ? threadIdx.x : 0);
      const long long t0 = wall_clock64();
      for (int it = 0;; ++it) {
        const int v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__ballot(v == 0) == 0) break;
        if ((it & 15) == 15 && wall_clock64() - t0 > kSmallWaitTicks) {
          if (threadIdx.x == 0) __hip_atomic_store(ctl + kSmallCtlErr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    small_down_block<KD, true>(dn, tile, r, sh);
  }
}

// ------------------------------------------------------------------------
// Combine from sorted rows: y[t] = sum over slots j (in order) of the row of
// pair t*k+j (skipped if the pair has no row). grid.x = n_tokens *
// (hidden / 128), block = 64.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_combine_sorted(SortedCombineArgs a) {
  const int nb = a.hidden / 128;
  const int b = blockIdx.x % nb;
  const int t = blockIdx.x / nb;
  const int lane = threadIdx.x;
  float acc0 = 0.f, acc1 = 0.f;
  // slots in groups of 8: every load of a group issued before its adds (a
  // slot without a row reads row 0 and adds nothing)
  const int k = a.top_k;
  for (int j0 = 0; j0 < k; j0 += 8) {
    int iv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) iv[q] = j0 + q < k ? a.inv[t * k + j0 + q] : -1;
    float v0[8], v1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float* yr = a.rows + (size_t)(iv[q] >= 0 ? iv[q] : 0) * a.hidden + 128 * b;
      v0[q] = yr[lane];
      v1[q] = yr[lane + 64];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (iv[q] >= 0) {
        acc0 += v0[q];
        acc1 += v1[q];
      }
  }
  if (a.bias) {  // the dense export's output bias, after the sum
    acc0 += a.bias[128 * b + lane];
    acc1 += a.bias[128 * b + lane + 64];
  }
  float* y = a.y + (size_t)t * a.hidden + 128 * b;
  y[lane] = acc0;
  y[lane + 64] = acc1;
  if (a.ss) {
    const float ss = wave_sum(__builtin_fmaf(acc0, acc0, acc1 * acc1));
    if (lane == 0) a.ss[(size_t)t * nb + b] = ss;
  }
}

// ------------------------------------------------------------------------
// Stack chain between two grouped layers, one work-group per token (wave b
// = 128-input block b, hidden <= 2048): the slot-ordered combine of the
// token's sorted pair outputs (as k_combine_sorted), the RMSNorm to bf16 (as
// k_rmsnorm_bf16: per-block sums of squares over the wave, blocks added in
// order), then, for each of the token's pairs in the next layer, that
// pair's rotated fp16 input H_n(rin (.) x) at its sorted index (as
// k_xin_gather). Each step keeps the arithmetic and order of the kernel it
// replaces, so the chain's values are the same bits.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_combine_next(CombineNextArgs a) {
  __shared__ float block_ss[16];
  __shared__ float pmax[16][8];  // [block][pair of a group]: largest |rin (.) x|
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int b = threadIdx.x >> 6;
  const int nb = a.hidden / 128;
  const int k = a.top_k;
  const bool mine = b < nb;
  const int32_t* __restrict__ inv = a.inv + (size_t)t * k;
  const int32_t* __restrict__ inv_next = a.inv_next + (size_t)t * k;
  const int32_t* __restrict__ ids_next = a.ids_next + (size_t)t * k;
  // the next layer's pairs of the first group and their input scales: a
  // chain of dependent loads that does not depend on the combine, issued
  // first so that it overlaps it
  int dst[8];
  uint16_t r0[8], r1[8];
  auto load_group = [&](int j0) {
    // clamped indices: the loads are issued unconditionally, back to back
    int id[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int jq = j0 + q < k ? j0 + q : k - 1;
      dst[q] = inv_next[jq];
      id[q] = ids_next[jq];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (j0 + q >= k) dst[q] = -1;
      const int e = dst[q] >= 0 ? id[q] : 0;  // a pair without a row may carry an invalid id
      const uint16_t* rr = a.rin_next + (size_t)e * a.hidden + 128 * (mine ? b : 0);
      r0[q] = rr[lane];
      r1[q] = rr[lane + 64];
    }
  };
  load_group(0);
  // slots in groups of 8: every load of a group issued before its use (a
  // slot without a row reads row 0 and adds nothing)
  float acc0 = 0.f, acc1 = 0.f;
  if (mine) {
    for (int j0 = 0; j0 < k; j0 += 8) {
      float v0[8], v1[8];
      bool ok[8];
      int iv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) iv[q] = inv[j0 + q < k ? j0 + q : k - 1];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = j0 + q < k ? iv[q] : -1;
        ok[q] = i >= 0;
        const float* yr = a.rows + (size_t)(ok[q] ? i : 0) * a.hidden + 128 * b;
        v0[q] = yr[lane];
        v1[q] = yr[lane + 64];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (ok[q]) {
          acc0 += v0[q];
          acc1 += v1[q];
        }
    }
    float* y = a.y + (size_t)t * a.hidden + 128 * b;
    y[lane] = acc0;
    y[lane + 64] = acc1;
    const float ss = wave_sum(__builtin_fmaf(acc0, acc0, acc1 * acc1));
    if (lane == 0) block_ss[b] = ss;
  }
  __syncthreads();
  float tot = 0.f;
  for (int q = 0; q < nb; ++q) tot += block_ss[q];
  const float rs = 1.0f / sqrtf(tot / (float)a.hidden + a.eps);
  const uint16_t x0 = f32_to_bf16_rne(acc0 * rs), x1 = f32_to_bf16_rne(acc1 * rs);
  if (mine && a.x_out) {
    uint16_t* xr = a.x_out + (size_t)t * a.hidden + 128 * b;
    xr[lane] = x0;
    xr[lane + 64] = x1;
  }
  const float xf0 = bf16_to_f32(x0), xf1 = bf16_to_f32(x1);
  // the next layer's inputs of the token's pairs, as k_xin_gather forms
  // them: each pair's row scaled by the power of two taken from 16 times
  // its largest |rin (.) x| (the blocks' maxima meet in LDS)
  for (int j0 = 0; j0 < k; j0 += 8) {
    if (j0 > 0) load_group(j0);
    float v0[8], v1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      v0[q] = xf0 * f16_to_f32(r0[q]);
      v1[q] = xf1 * f16_to_f32(r1[q]);
      const float m = wave_max(fmaxf(fabsf(v0[q]), fabsf(v1[q])));
      if (mine && lane == 0) pmax[b][q] = m;
    }
    __syncthreads();
    // lane q < 8: pair q's largest magnitude over the blocks
    float mq = 0.f;
    if (lane < 8)
      for (int bb = 0; bb < nb; ++bb) mq = fmaxf(mq, pmax[bb][lane]);
    __syncthreads();  // pmax is rewritten by the next group
    if (!mine) continue;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (dst[q] < 0) continue;  // uniform over the work-group
      const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mq), q));
      int ex = fp16_block_exp(16.0f * m);
      if (ex == kExpZeroBlock) ex = 0;
      if (b == 0 && lane == 0) a.xg_exp_next[dst[q]] = ex;
      const float scale = kInvSqrt128 * exp2i(ex);
      fwht128(v0[q], v1[q]);
      _Float16* xo = reinterpret_cast<_Float16*>(a.xg_next) + (size_t)dst[q] * a.hidden + 128 * b;
      xo[lane] = (_Float16)(v0[q] * scale);
      xo[lane + 64] = (_Float16)(v1[q] * scale);
    }
  }
}

// ------------------------------------------------------------------------
// The decoders of the fused kernels, with their results written back in
// [out][in] order, so that every decode layout can be checked bit for bit
// against the format (escha_decode_tiles_layout).
//
// MFMA-operand layout (the one-launch stack and the small-tile kernels):
// one wave per region of 8 tile-rows x 4 output tiles, staged and decoded
// by exactly the routines those kernels run (stage_issue, stage_store,
// decode_stage_mfma). Lane (n, g) holds in A[pp][j] the weights of output
// column n of tile nt0 + j, input rows 8 (g & 1) + i (i = 0..7) of
// tile-row kt0 + 2 pp + (g >> 1). grid.x = (in/128) * (out/64), block = 64.
// ------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(64) void k_decode_operands_mfma(const uint16_t* __restrict__ code_e,
                                                             int in_f, int out_f,
                                                             uint16_t* __restrict__ w) {
  __shared__ uint32_t stage[Stage<K>::kDw];
  const int n_nt = out_f / 16;
  const int nq = n_nt / 4;
  const int kt0 = 8 * (blockIdx.x / nq);
  const int nt0 = 4 * (blockIdx.x % nq);
  const int lane = threadIdx.x;
  u32x4 cv[Stage<K>::kPerLane];
  stage_issue<K>(code_e, n_nt, kt0, nt0, lane, cv);
  stage_store<K>(stage, lane, cv);
  h16x8 A[4][4];
  decode_stage_mfma<K>(stage, lane, A);
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * (nt0 + j) + n;
      const int col = 16 * (kt0 + 2 * pp + (g >> 1)) + 8 * (g & 1);
      *reinterpret_cast<h16x8*>(w + (size_t)row * in_f + col) = A[pp][j];
    }
}

// Column-pair layout (PairDecoder, K = 2: the one-launch kernel's gate_up
// tasks): the same staged region; lane (m, g) holds in register i of
// A[pp][j] the weights of output columns c = m & 7 and c + 8 of tile nt0 + j,
// input row 8 (m >> 3) + 4 (g & 1) + i of tile-row kt0 + 2 pp + (g >> 1).
// grid.x = (in/128) * (out/64), block = 64.
__global__ __launch_bounds__(64) void k_decode_operands_pairs(const uint16_t* __restrict__ code_e, int in_f,
                                                              int out_f, uint16_t* __restrict__ w) {
  __shared__ uint32_t stage[Stage<2>::kDw];
  const int n_nt = out_f / 16;
  const int nq = n_nt / 4;
  const int kt0 = 8 * (blockIdx.x / nq);
  const int nt0 = 4 * (blockIdx.x % nq);
  const int lane = threadIdx.x;
  u32x4 cv[Stage<2>::kPerLane];
  stage_issue<2>(code_e, n_nt, kt0, nt0, lane, cv);
  stage_store<2>(stage, lane, cv);
  const PairDecoder dec(stage, lane);
  h16x8 A[4][4];
  dec.decode<0>(A[0]);
  dec.decode<1>(A[1]);
  dec.decode<2>(A[2]);
  dec.decode<3>(A[3]);
  const int m = lane & 15, g = lane >> 4;
  const int c = m & 7;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * (nt0 + j) + c;  // output c (and c + 8 eight rows on)
      const int col0 = 16 * (kt0 + 2 * pp + (g >> 1)) + 8 * (m >> 3) + 4 * (g & 1);
      const u32x4 v = __builtin_bit_cast(u32x4, A[pp][j]);  // register i: (column c, column c + 8)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[(size_t)row * in_f + col0 + i] = (uint16_t)(v[i] & 0xFFFFu);
        w[(size_t)(row + 8) * in_f + col0 + i] = (uint16_t)(v[i] >> 16);
      }
    }
}

// Tile-pair layout (TilePairDecoder, K = 2: the small-tile gate_up kernel on
// tiles of at most 8 tokens): the same staged region; lane (m, g) holds in
// register i of the operand of tile-row tr and tile pair jp the weights of
// output columns c = m & 7 and c + 8 of tile nt0 + 2 jp + (m >> 3), input row
// 4 g + i of tile-row kt0 + tr. grid.x = (in/128) * (out/64), block = 64.
__global__ __launch_bounds__(64) void k_decode_operands_tilepairs(const uint16_t* __restrict__ code_e,
                                                                  int in_f, int out_f,
                                                                  uint16_t* __restrict__ w) {
  __shared__ uint32_t stage[Stage<2>::kDw];
  const int n_nt = out_f / 16;
  const int nq = n_nt / 4;
  const int kt0 = 8 * (blockIdx.x / nq);
  const int nt0 = 4 * (blockIdx.x % nq);
  const int lane = threadIdx.x;
  u32x4 cv[Stage<2>::kPerLane];
  stage_issue<2>(code_e, n_nt, kt0, nt0, lane, cv);
  stage_store<2>(stage, lane, cv);
  const TilePairDecoder dec(stage, lane);
  const int m = lane & 15, g = lane >> 4;
  auto put = [&](int tr, int jp, h16x8 A) {
    const u32x4 v = __builtin_bit_cast(u32x4, A);  // register i: (column c, column c + 8)
    const int row = 16 * (nt0 + 2 * jp + (m >> 3)) + (m & 7);
    const int col0 = 16 * (kt0 + tr) + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[(size_t)row * in_f + col0 + i] = (uint16_t)(v[i] & 0xFFFFu);
      w[(size_t)(row + 8) * in_f + col0 + i] = (uint16_t)(v[i] >> 16);
    }
  };
  auto both = [&](auto trc) {
    constexpr int TR = decltype(trc)::value;
    put(TR, 0, dec.template decode<TR, 0>());
    put(TR, 1, dec.template decode<TR, 1>());
  };
  both(std::integral_constant<int, 0>{});
  both(std::integral_constant<int, 1>{});
  both(std::integral_constant<int, 2>{});
  both(std::integral_constant<int, 3>{});
  both(std::integral_constant<int, 4>{});
  both(std::integral_constant<int, 5>{});
  both(std::integral_constant<int, 6>{});
  both(std::integral_constant<int, 7>{});
}

// LDS-tile layout (the 128-token grouped kernels): one work-group of eight
// waves -- the decoder waves of those kernels -- per 64-input step and
// group of 16 output tiles; each lane loads and decodes its eighth of a
// tile with load_eighth and decode_to_lds, and the W buffer is then read
// back through w_slot, the addressing of the matrix waves' operand reads.
// grid.x = (in/64) * (out/256), block = 512.
template <int K>
__global__ __launch_bounds__(512) void k_decode_operands_lds(const uint16_t* __restrict__ code_e,
                                                             int in_f, int out_f,
                                                             uint16_t* __restrict__ w) {
  __shared__ __attribute__((aligned(16))) _Float16 wb[kWBuf];
  const int n_nt = out_f / 16;
  const int ng = out_f / 256;
  const int s = blockIdx.x / ng;
  const int grp = blockIdx.x % ng;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int o = tid & 7;
  const int dtile = tid >> 3;
  const int dkt = dtile >> 4, dnt = dtile & 15;
  uint32_t raw[K];
  load_eighth<K>(code_e + ((size_t)(4 * s + dkt) * n_nt + 16 * grp + dnt) * (16 * K) + o * (2 * K), raw);
  decode_to_lds<K>(raw, dkt, dnt, o, lane, wb);
  __syncthreads();
  for (int idx = tid; idx < 256 * (kStep / 8); idx += 512) {
    const int row = idx / (kStep / 8);
    const int kc = idx % (kStep / 8);
    const h8 v = *reinterpret_cast<const h8*>(wb + w_slot(kc, row));
    *reinterpret_cast<h8*>(w + (size_t)(256 * grp + row) * in_f + kStep * s + 8 * kc) = v;
  }
}

hipError_t launch_decode_operands(const uint16_t* code_e, int in_f, int out_f, int k_bits, int layout,
                                  uint16_t* w, hipStream_t s) {
  if (layout == 1) {
    const unsigned grid = (unsigned)((in_f / 128) * (out_f / 64));
    if (k_bits == 2)
      hipLaunchKernelGGL(k_decode_operands_mfma<2>, dim3(grid), dim3(64), 0, s, code_e, in_f, out_f, w);
    else
      hipLaunchKernelGGL(k_decode_operands_mfma<3>, dim3(grid), dim3(64), 0, s, code_e, in_f, out_f, w);
  } else if (layout == 3 || layout == 4) {
    if (k_bits != 2) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((in_f / 128) * (out_f / 64));
    if (layout == 3)
      hipLaunchKernelGGL(k_decode_operands_pairs, dim3(grid), dim3(64), 0, s, code_e, in_f, out_f, w);
    else
      hipLaunchKernelGGL(k_decode_operands_tilepairs, dim3(grid), dim3(64), 0, s, code_e, in_f, out_f, w);
  } else if (layout == 2) {
    const unsigned grid = (unsigned)((in_f / kStep) * (out_f / 256));
    if (k_bits == 2)
      hipLaunchKernelGGL(k_decode_operands_lds<2>, dim3(grid), dim3(512), 0, s, code_e, in_f, out_f, w);
    else
      hipLaunchKernelGGL(k_decode_operands_lds<3>, dim3(grid), dim3(512), 0, s, code_e, in_f, out_f, w);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// Launchers.
// ------------------------------------------------------------------------
hipError_t launch_make_tiles(const int32_t* offsets, int E, int tm, int max_tiles, int32_t* t_expert,
                             int32_t* t_row0, int32_t* t_rows, int32_t* n_tiles, hipStream_t s,
                             int n_layers) {
  hipLaunchKernelGGL(k_make_tiles, dim3(1, (unsigned)n_layers), dim3(1024), 0, s, offsets, E, tm,
                     max_tiles, t_expert, t_row0, t_rows, n_tiles);
  return hipGetLastError();
}

hipError_t launch_xin_gather(const GatherArgs& a, int n_pairs, hipStream_t s) {
  if (n_pairs <= 0) return hipSuccess;
  if (n_pairs < kGatherSmallPairs)
    hipLaunchKernelGGL(k_xin_gather_small, dim3((unsigned)n_pairs), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_xin_gather, dim3((unsigned)((n_pairs + kGatherRows - 1) / kGatherRows)),
                       dim3(64 * kGatherRows), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_gate_up(const GroupedArgs& a, int max_tiles, int k_bits, hipStream_t s) {
  const unsigned grid = grouped_grid(max_tiles, a.inter / 128);
  if (k_bits == 2)
    hipLaunchKernelGGL(k_grouped_gate_up<2>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_grouped_gate_up<3>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_down(const GroupedArgs& a, int max_tiles, int k_bits, hipStream_t s) {
  const unsigned grid = grouped_grid(max_tiles, a.hidden / 256);
  if (k_bits == 2)
    hipLaunchKernelGGL(k_grouped_down<2>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_grouped_down<3>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_small_gate_up(const GroupedArgs& a, int max_tiles, int k_bits, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)max_tiles * (a.inter / 128));
  if (k_bits == 2)
    hipLaunchKernelGGL(k_small_gate_up<2>, dim3(grid), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(k_small_gate_up<3>, dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

unsigned small_layer_grid(int max_tiles, int inter, int hidden) {
  return (unsigned)(8 * ((max_tiles + 7) / 8) * (inter / 128 + hidden / 256) + 64);
}

hipError_t launch_small_layer(const GroupedArgs& gu, const GroupedArgs& dn, int max_tiles, int k_gu, int k_dn,
                              int32_t* ctl, hipStream_t s) {
  const dim3 grid(small_layer_grid(max_tiles, gu.inter, dn.hidden)), block(512);
  if (k_gu == 2 && k_dn == 3)
    hipLaunchKernelGGL((k_small_layer<2, 3>), grid, block, 0, s, gu, dn, ctl);
  else if (k_gu == 2 && k_dn == 2)
    hipLaunchKernelGGL((k_small_layer<2, 2>), grid, block, 0, s, gu, dn, ctl);
  else if (k_gu == 3 && k_dn == 3)
    hipLaunchKernelGGL((k_small_layer<3, 3>), grid, block, 0, s, gu, dn, ctl);
  else if (k_gu == 3 && k_dn == 2)
    hipLaunchKernelGGL((k_small_layer<3, 2>), grid, block, 0, s, gu, dn, ctl);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_small_down(const GroupedArgs& a, int max_tiles, int k_bits, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)max_tiles * (a.hidden / 256));
  if (k_bits == 2)
    hipLaunchKernelGGL(k_small_down<2>, dim3(grid), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(k_small_down<3>, dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine_next(const CombineNextArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_combine_next, dim3((unsigned)a.n_tokens), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine_sorted(const SortedCombineArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)a.n_tokens * (a.hidden / 128));
  hipLaunchKernelGGL(k_combine_sorted, dim3(grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace escha
