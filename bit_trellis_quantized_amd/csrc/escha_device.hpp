// escha_device.hpp -- device routines shared by the gfx950 kernels of
// libescha: the trellis tile decoder, the in-wave 128-point Hadamard and
// number-format helpers.
//
// Format (sources: model card "Qwen3.6-35B-A3B-Escha-W2-trellis-mlx",
// exactness table; hipfire PR "Escha-W2 port: 2-bit trellis decoded in the
// GEMV", closing summary "What it is"):
//  - a 16x16 tile is 16*K little-endian uint16 words = a 256*K-bit stream,
//    bit b being bit b%16 of word b/16;
//  - weight i (input row i/16, output column i%16 of the tile) is the
//    16-bit window of the stream starting at bit K*i, first bit least
//    significant, wrapping at the end of the tile;
//  - a state s decodes as r = (s*0xCBAC1FED mod 2^32 & 0x8FFF8FFF) ^
//    0x3B603B60, weight = fp16(lo16 r) + fp16(hi16 r) rounded to nearest
//    even.
//
// Work split inside a wave: four lanes share one tile. Lane q of the four
// holds a quarter of the stream (16 B at K=2, 24 B at K=3) plus the first
// dword of the next quarter, and decodes the 64 weights whose windows start
// in its quarter: input rows 4q..4q+3 of the tile, all 16 output columns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace escha {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kInvSqrt128 = 0.08838834764831845f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Decode the two 16-bit states packed in V (low and high half) into two fp16
// weights packed the same way.
//
// With C = C1*2^16 + C0 (C1 = 0xCBAC, C0 = 0x1FED), s*C mod 2^32 has low half
// lo16(s*C0) and high half hi16(s*C0) + lo16(s*C1) (mod 2^16). The two
// 16x16->32 products s*C0 are the only full-width multiplies; the rest runs
// on packed 16-bit lanes, and one packed fp16 add (round-to-nearest-even,
// the hardware default) forms both weights.
__device__ __forceinline__ h16x2 cba_decode_pair(uint32_t V) {
  const uint32_t a = V & 0xFFFFu;
  const uint32_t b = V >> 16;
  const uint32_t ma = a * 0x1FEDu;
  const uint32_t mb = b * 0x1FEDu;
  uint32_t lo = __builtin_amdgcn_perm(mb, ma, 0x05040100u);        // lo16(ma) | lo16(mb) << 16
  const uint32_t zh = __builtin_amdgcn_perm(mb, ma, 0x07060302u);  // hi16(ma) | hi16(mb) << 16
  const u16x2 c1 = {(unsigned short)0xCBAC, (unsigned short)0xCBAC};
  const u16x2 hv = __builtin_bit_cast(u16x2, V) * c1 + __builtin_bit_cast(u16x2, zh);
  uint32_t hi = __builtin_bit_cast(uint32_t, hv);
  lo = (lo & 0x8FFF8FFFu) ^ 0x3B603B60u;
  hi = (hi & 0x8FFF8FFFu) ^ 0x3B603B60u;
  return __builtin_bit_cast(h16x2, lo) + __builtin_bit_cast(h16x2, hi);
}

// 32 stream bits starting at bit `o` of the lane's dwords d[] (o known at
// compile time after unrolling).
template <int O>
__device__ __forceinline__ uint32_t window32(const uint32_t* d) {
  if constexpr (O % 32 == 0) {
    return d[O / 32];
  } else {
    return __builtin_amdgcn_alignbit(d[O / 32 + 1], d[O / 32], O % 32);
  }
}

// Packed states of weights (kk, n) and (kk, n+8) of the lane's quarter:
// relative stream offsets K*(16*kk + n) and that + 8*K.
template <int K, int KK, int N>
__device__ __forceinline__ uint32_t quarter_state_pair(const uint32_t* d) {
  constexpr int o = K * (16 * KK + N);
  if constexpr (K == 2) {
    // the partner window starts 16 bits later: one 32-bit window holds both
    return window32<o>(d);
  } else {
    // the partner starts 24 bits later: take its 16 bits from the window
    // that begins 8 bits after ours (its bits 16..31)
    const uint32_t w0 = window32<o>(d);
    const uint32_t w1 = window32<o + 8>(d);
    return __builtin_amdgcn_perm(w1, w0, 0x07060100u);
  }
}

// Packed states of weights (row kk, column n) and (row kk, column n + 8) of
// a lane's stream piece d (offsets K*(16*kk + n) and that + 8*K).
template <int K>
__device__ __forceinline__ uint32_t row_state_pair(const uint32_t* d, int kk, int n) {
  const int o = K * (16 * kk + n);
  const uint32_t w0 = __builtin_amdgcn_alignbit(d[(o >> 5) + 1], d[o >> 5], o & 31);
  if constexpr (K == 2) return w0;
  const int o1 = o + 8;
  const uint32_t w1 = __builtin_amdgcn_alignbit(d[(o1 >> 5) + 1], d[o1 >> 5], o1 & 31);
  return __builtin_amdgcn_perm(w1, w0, 0x07060100u);
}

// Number of dwords a lane holds: its quarter (2K) plus the next quarter's
// first dword (the wrap reaches at most 15 bits into it).
template <int K>
struct Quarter {
  static constexpr int kOwn = 2 * K;
  static constexpr int kAll = 2 * K + 1;
};

// Decode the lane's 64 weights and hand each packed pair to f(kk, n, w):
// w.x = weight (row 4q+kk, column n), w.y = weight (row 4q+kk, column n+8).
template <int K, int KK = 0, int N = 0, class F>
__device__ __forceinline__ void decode_quarter(const uint32_t* d, F&& f) {
  if constexpr (KK < 4) {
    if constexpr (N < 8) {
      const h16x2 w = cba_decode_pair(quarter_state_pair<K, KK, N>(d));
      f(KK, N, w);
      decode_quarter<K, KK, N + 1>(d, f);
    } else {
      decode_quarter<K, KK + 1, 0>(d, f);
    }
  }
}

// Load the lane's quarter of a tile. `tq` points at the quarter's first
// word (16-byte aligned at K=2, 8-byte aligned at K=3).
template <int K>
__device__ __forceinline__ void load_quarter(const uint16_t* tq, uint32_t* d) {
  if constexpr (K == 2) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tq));
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  } else {
    const u32x2* p = reinterpret_cast<const u32x2*>(tq);
    const u32x2 a = __builtin_nontemporal_load(p + 0);
    const u32x2 b = __builtin_nontemporal_load(p + 1);
    const u32x2 c = __builtin_nontemporal_load(p + 2);
    d[0] = a.x;
    d[1] = a.y;
    d[2] = b.x;
    d[3] = b.y;
    d[4] = c.x;
    d[5] = c.y;
  }
}

// First dword of the next quarter of the same tile (lanes 4t..4t+3 share a
// tile; lane 4t+3 wraps to lane 4t). quad_perm [1,2,3,0].
__device__ __forceinline__ uint32_t next_quarter_dword(uint32_t d0) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0x39, 0xF, 0xF, false);
}

// ---- cross-lane data movement inside one wave (no LDS traffic) ----------

// DPP move: lane i receives src from the lane selected by CTRL.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kQuadXor3 = 0x1B;     // quad_perm [3,2,1,0]
constexpr int kHalfMirror = 0x141;  // lane i <- lane 7-i inside each group of 8
constexpr int kRowRor8 = 0x128;     // rotate by 8 inside each row of 16 = xor 8

// Value of lane i^H for H = 1, 2, 4, 8.
template <int H>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (H == 1) return dpp<kQuadXor1>(v);
  if constexpr (H == 2) return dpp<kQuadXor2>(v);
  if constexpr (H == 4) return dpp<kHalfMirror>(dpp<kQuadXor3>(v));  // (i^3)^7 = i^4
  if constexpr (H == 8) return dpp<kRowRor8>(v);
}

// One butterfly across lanes i and i^H: low lane gets low+high, high lane
// gets low-high. s = +1 on low lanes, -1 on high lanes; fma(+-1, a, b) is the
// exactly rounded b +- a, identical to an add or a subtract.
template <int H>
__device__ __forceinline__ float butterfly(float v, float s) {
  if constexpr (H <= 8) {
    return __builtin_fmaf(s, v, xor_lane<H>(v));
  } else {
    // rows 16 apart (H = 16) or halves 32 apart (H = 32): swap the odd
    // rows / upper half of a copy with the even rows / lower half of
    // another copy; r[0] then holds the low element and r[1] the high one
    // on both sides of the pair.
    const unsigned u = __float_as_uint(v);
    unsigned a, b;
    if constexpr (H == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      a = r[0];
      b = r[1];
    } else {
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      a = r[0];
      b = r[1];
    }
    return __builtin_fmaf(s, __uint_as_float(b), __uint_as_float(a));
  }
}

__device__ __forceinline__ float lane_sign(int lane, int h) { return (lane & h) ? -1.0f : 1.0f; }

// 128-point Sylvester Walsh-Hadamard transform (unscaled) across one wave:
// element i of the block is v0 of lane i for i < 64 and v1 of lane i-64
// otherwise. Butterflies: bit 6 inside the lane, bits 0..5 across lanes.
// The butterflies of different bits commute, so the order is free.
__device__ __forceinline__ void fwht128(float& v0, float& v1) {
  const float a = v0 + v1;
  const float b = v0 - v1;
  const int lane = threadIdx.x & 63;
  const float s1 = lane_sign(lane, 1), s2 = lane_sign(lane, 2), s4 = lane_sign(lane, 4);
  const float s8 = lane_sign(lane, 8), s16 = lane_sign(lane, 16), s32 = lane_sign(lane, 32);
  v0 = butterfly<32>(butterfly<16>(butterfly<8>(butterfly<4>(butterfly<2>(butterfly<1>(a, s1), s2), s4), s8), s16), s32);
  v1 = butterfly<32>(butterfly<16>(butterfly<8>(butterfly<4>(butterfly<2>(butterfly<1>(b, s1), s2), s4), s8), s16), s32);
}

// Sum over the 64 lanes; every lane gets the same bits.
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane<1>(v);
  v += xor_lane<2>(v);
  v += xor_lane<4>(v);
  v += xor_lane<8>(v);
  {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// Largest value over the 64 lanes (NaN lanes are ignored by fmaxf); every
// lane gets the same result.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lane<1>(v));
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<4>(v));
  v = fmaxf(v, xor_lane<8>(v));
  {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}

// ---- power-of-two scaling of activations rounded to fp16 ---------------
//
// Activations that enter a matrix-core contraction as fp16 are first
// multiplied by 2^e, e a multiple of 8 chosen from the largest magnitude m
// of the block they belong to so that m 2^e lies in [2^6, 2^14): far from
// fp16's overflow (65504) and 20 binades above its subnormals (below
// 2^-14), whatever the magnitude of the input. The fp32 result is
// multiplied by 2^-e. A power of two scales exactly, so wherever the
// unscaled values would have been normal fp16 numbers the results carry the
// same bits as without scaling. The coarse steps make neighbouring blocks of
// a row share their exponent unless their maxima straddle a step, so the
// rescaling to a row's common exponent is mostly not needed.

// Exponent marker of a block whose values are all exactly zero (+0 or -0,
// no NaN): the block contributes exactly zero to any contraction.
constexpr int kExpZeroBlock = 1 << 20;

// 2^e for |e| < 126 (exact).
__device__ __forceinline__ float exp2i(int e) { return __int_as_float((e + 127) << 23); }

// e, a multiple of 8, with 2^6 <= m 2^e < 2^14 for a finite m > 0; 0 for
// an infinite or NaN m (no scaling); kExpZeroBlock for m == 0. Clamped to
// |e| <= 96.
__device__ __forceinline__ int fp16_block_exp(float m) {
  if (m == 0.0f) return kExpZeroBlock;
  if (!(m <= 3.0e38f)) return 0;
  int ex;
  frexpf(m, &ex);                 // 2^(ex - 1) <= m < 2^ex
  int e = (14 - ex) & ~7;         // floor to a multiple of 8: m 2^e in [2^6, 2^14)
  return e < -96 ? -96 : (e > 96 ? 96 : e);
}

// The exponent of a row whose blocks carry exponents ex[0..n): the
// smallest (the scale of its largest block); zero blocks do not count, and a
// row of zero blocks gets 0.
__device__ __forceinline__ int row_exp(const int32_t* __restrict__ ex, int n) {
  int e = kExpZeroBlock;
  for (int c0 = 0; c0 < n; c0 += 8) {
    // eight loads in flight at once (clamped indices: no load under a branch)
    int v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = ex[c0 + q < n ? c0 + q : n - 1];
#pragma unroll
    for (int q = 0; q < 8; ++q) e = v[q] < e ? v[q] : e;
  }
  return e == kExpZeroBlock ? 0 : e;
}

// Shift that brings fp16 values of a block with exponent eb to the exponent
// er of their row (er <= eb, so the shift is <= 0); 0 for a zero block.
__device__ __forceinline__ int block_shift(int er, int eb) {
  return eb == kExpZeroBlock ? 0 : er - eb;
}

// 8 fp16 values times 2^sh (sh <= 0, a multiple of 8): one packed multiply
// per pair by 2^sh, an fp16 number down to 2^-24 (subnormal below 2^-14), so
// each value is rounded once to nearest even. A block more than 2^24 below
// its row (sh < -24) gives zeros: its values are then below 2^-24 of the
// row's largest, under the resolution of the fp32 sums they would join.
// Branch-free: the callers run at their register limit, where a branch here
// costs the LDS pipelining of the loop around it.
typedef _Float16 h16x8v __attribute__((ext_vector_type(8)));
__device__ __forceinline__ _Float16 f16_pow2(int sh) {  // -24 <= sh <= 0
  return __builtin_bit_cast(_Float16, sh >= -14 ? (uint16_t)((sh + 15) << 10)
                                                : (uint16_t)(1u << (sh + 24)));
}
__device__ __forceinline__ h16x8v rescale_h8(h16x8v v, int sh) {
  const _Float16 f = sh < -24 ? (_Float16)0 : f16_pow2(sh);
  return v * h16x8v{f, f, f, f, f, f, f, f};
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

}  // namespace escha
