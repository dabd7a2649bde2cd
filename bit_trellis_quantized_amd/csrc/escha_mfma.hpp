// escha_mfma.hpp -- decode of trellis tiles straight into the operand layout
// of the gfx950 matrix instruction v_mfma_f32_16x16x32_f16, and the
// contraction of decoded tiles with activations on the matrix cores.
//
// Operand layouts of v_mfma_f32_16x16x32_f16 (D[16][16] += A[16][32] B[32][16]),
// lane l of the wave: A[l % 16][8 (l / 16) + i] and B[8 (l / 16) + i][l % 16]
// for i = 0..7 (8 halves, 4 registers); D[4 (l / 16) + j][l % 16] for
// j = 0..3 (4 floats).
//
// Mapping: A is a pair of vertically adjacent 16x16 tiles (input tile-rows
// kt and kt+1, output tile nt) with A's row m = output column n of the
// tiles and A's k = 16 * (tile of the pair) + input row inside the tile; B
// holds the 32 activations of those inputs, split into a high and a low
// fp16 part in B's columns 0 and 1 (all other columns zero), so that
// D[n][0] + D[n][1] is the fp32-accurate dot product of output n's weights
// with the fp32 activations (the products of two fp16 values are exact in
// fp32, and hi + lo carries 22 significant bits of each activation).
//
// A lane (n, g = l / 16) needs the 8 weights (input rows 8 (g & 1) + i of
// tile g >> 1, column n): their states are the 16-bit windows at stream
// bits K (16 (8 (g & 1) + i) + n). The codes of a wave's tiles are staged in
// LDS first (one 16-byte load per lane and chunk, coalesced), each tile
// followed by a copy of its first dword so that windows that run past the
// end of the tile wrap without a special case.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "escha_device.hpp"

namespace escha {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS staging of one wave's 8 tile-rows x 4 tiles.
template <int K>
struct Stage {
  static constexpr int kTileDw = 8 * K;                 // dwords of a tile (16K words)
  static constexpr int kStride = kTileDw + 1;           // + the wrap dword
  static constexpr int kDw = 8 * 4 * kStride;           // dwords per wave
  static constexpr int kChunks = 8 * 4 * kTileDw / 4;   // 16-byte chunks per wave
  static constexpr int kPerLane = kChunks / 64;         // 2 (K=2) or 3 (K=3)
};

// Issue the global loads of tile-rows kt0..kt0+7, tiles nt0..nt0+3 (each
// tile-row's four tiles are contiguous). Nothing waits for the data here.
template <int K>
__device__ __forceinline__ void stage_issue(const uint16_t* __restrict__ code_e, int n_nt, int kt0,
                                            int nt0, int lane,
                                            u32x4 (&v)[Stage<K>::kPerLane]) {
  constexpr int kRowChunks = Stage<K>::kTileDw;  // 4 tiles x kTileDw dwords / 4 dwords per chunk
#pragma unroll
  for (int m = 0; m < Stage<K>::kPerLane; ++m) {
    const int c = lane + 64 * m;
    const int r = c / kRowChunks;
    const int cc = c - r * kRowChunks;
    const uint16_t* src = code_e + ((size_t)(kt0 + r) * n_nt + nt0) * (16 * K) + 8 * cc;
    v[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  }
}

// LDS position (in tiles) of tile-row r, tile j of a wave's region of NT
// tiles per row: the odd tile-rows after the even ones, so that the 4 NT
// tiles a lane decodes (rows of one parity) are contiguous.
template <int NT = 4>
__device__ __forceinline__ int stage_slot(int r, int j) {
  return (r & 1) * (4 * NT) + (r >> 1) * NT + j;
}

// Store the loaded chunks to the wave's LDS region (tile (r, j) at dword
// stage_slot(r, j) * kStride) with each tile's wrap dword; the wave can read
// them back once this returns.
template <int K>
__device__ __forceinline__ void stage_store(uint32_t* lds, int lane,
                                            const u32x4 (&v)[Stage<K>::kPerLane]) {
  constexpr int kRowChunks = Stage<K>::kTileDw;
  constexpr int kTileChunks = Stage<K>::kTileDw / 4;
#pragma unroll
  for (int m = 0; m < Stage<K>::kPerLane; ++m) {
    const int c = lane + 64 * m;
    const int r = c / kRowChunks;
    const int cc = c - r * kRowChunks;
    const int j = cc / kTileChunks;
    const int d = 4 * (cc - j * kTileChunks);
    uint32_t* t = lds + stage_slot(r, j) * Stage<K>::kStride;
    t[d + 0] = v[m].x;
    t[d + 1] = v[m].y;
    t[d + 2] = v[m].z;
    t[d + 3] = v[m].w;
    if (d == 0) t[Stage<K>::kTileDw] = v[m].x;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Lane-dependent part of the operand decode of a staged region (NT tiles per
// row, at stage_slot<NT>): the two window base addresses of each half of the
// tile-row pairs and the two window shifts.
template <int K, int NT = 4>
struct OperandDecoder {
  const uint32_t* base;
  int a0, a1, a0h, a1h;
  uint32_t s0, s1;

  __device__ __forceinline__ OperandDecoder(const uint32_t* lds, int lane) {
    const int n = lane & 15;
    const int g = lane >> 4;
    const int h = g & 1;
    // tile of the pair: rows 2pp + (g >> 1)
    base = lds + stage_slot<NT>(g >> 1, 0) * Stage<K>::kStride;
    if constexpr (K == 2) {
      // window i at bit 256h + 32i + 2n: dword 8h + i, shift 2n
      a0 = a1 = 8 * h;
      s0 = s1 = 2 * n;
    } else {
      // window i at bit 384h + 48i + 3n; for i = 2m: dword 12h + 3m + (3n >> 5),
      // shift 3n & 31; for i = 2m + 1: dword 12h + 3m + ((48 + 3n) >> 5),
      // shift (16 + 3n) & 31
      a0 = 12 * h + ((3 * n) >> 5);
      a1 = 12 * h + ((48 + 3 * n) >> 5);
      s0 = (3 * n) & 31;
      s1 = (16 + 3 * n) & 31;
    }
    // the tiles of pairs 2 and 3 through second base addresses (opaque to
    // the compiler, so that it keeps them instead of adding a constant
    // before every read: LDS read offsets reach 255 dwords)
    a0h = a0 + 2 * NT * Stage<K>::kStride;
    a1h = a1 + 2 * NT * Stage<K>::kStride;
    asm volatile("" : "+v"(a0h), "+v"(a1h));
  }

  // This lane's 8 weights of tile j of tile-row pair PP (rows 2PP, 2PP+1)
  // in the A-operand layout, for every j.
  template <int PP>
  __device__ __forceinline__ void decode(h16x8 (&A)[NT]) const {
    const uint32_t* p0 = base + (PP < 2 ? a0 : a0h);
    const uint32_t* p1 = base + (PP < 2 ? a1 : a1h);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int toff = (stage_slot<NT>(2 * (PP & 1), j) - stage_slot<NT>(0, 0)) * Stage<K>::kStride;
      uint32_t win[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ci = K == 2 ? i : 3 * (i >> 1);
        const uint32_t* p = (i & 1) ? p1 : p0;
        win[i] = __builtin_amdgcn_alignbit(p[toff + ci + 1], p[toff + ci], (i & 1) ? s1 : s0);
      }
      h16x8 a;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        // states of rows 8h + i and 8h + i + 1 (low halves of two windows)
        const h16x2 w = cba_decode_pair(__builtin_amdgcn_perm(win[i + 1], win[i], 0x05040100u));
        a[i] = w.x;
        a[i + 1] = w.y;
      }
      A[j] = a;
    }
  }
};

// Column-pair operand layout (K = 2 only; the one-launch kernel's gate_up
// tasks, whose contraction has one token): lane (m, g), c = m & 7, set =
// m >> 3, decodes of tile j of tile-row pair PP the weights of output
// columns c and c + 8 in input rows 8 set + 4 (g & 1) + i (i = 0..3) of
// tile-row 2 PP + (g >> 1). At K = 2 those two states are 16 stream bits
// apart, so one 32-bit window (one v_alignbit) holds both, packed as the
// hash wants them: a pair of weights costs the window and the hash, 9
// VALU operations instead of 11. Register i of A[j] holds (w(row_i, c),
// w(row_i, c + 8)); the contraction puts each set's activations into its
// own B columns (mfma_pairs in the one-launch kernel).
struct PairDecoder {
  const uint32_t* base;
  int a0, a0h;
  uint32_t sh;

  __device__ __forceinline__ PairDecoder(const uint32_t* lds, int lane) {
    const int m = lane & 15;
    const int g = lane >> 4;
    base = lds + stage_slot<4>(g >> 1, 0) * Stage<2>::kStride;
    // row r of a tile is dword r (16 weights x 2 bits); the window of
    // columns (c, c + 8) of row r starts at bit 2 c of it
    a0 = 8 * (m >> 3) + 4 * (g & 1);
    sh = 2 * (m & 7);
    a0h = a0 + 2 * 4 * Stage<2>::kStride;  // tile-rows 4..7: second base (see OperandDecoder)
    asm volatile("" : "+v"(a0h));
  }

  template <int PP>
  __device__ __forceinline__ void decode(h16x8 (&A)[4]) const {
    const uint32_t* p = base + (PP < 2 ? a0 : a0h);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int toff = (stage_slot<4>(2 * (PP & 1), j) - stage_slot<4>(0, 0)) * Stage<2>::kStride;
      uint32_t r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = __builtin_bit_cast(uint32_t,
                                  cba_decode_pair(__builtin_amdgcn_alignbit(p[toff + i + 1], p[toff + i], sh)));
      A[j] = __builtin_bit_cast(h16x8, u32x4{r[0], r[1], r[2], r[3]});
    }
  }
};

// Tile-pair operand layout (K = 2 only; the small-tile gate_up kernel on
// tiles of at most 8 tokens): one A operand covers output tiles 2 jp (A rows
// 0..7) and 2 jp + 1 (rows 8..15) of one input tile-row tr; lane (m, g), t =
// m >> 3, c = m & 7, holds in register i the weights of columns c and c + 8
// of tile 2 jp + t at input row 4 g + i of the tile (one window each, as in
// PairDecoder). With B column 8 par + tk holding token tk's activation of
// input row 4 g + i at B row 8 g + 2 i + par (zeros at the other parity),
// D[m][8 par + tk] is output column c + 8 par of tile 2 jp + t for token tk.
struct TilePairDecoder {
  const uint32_t* base;
  uint32_t sh;

  __device__ __forceinline__ TilePairDecoder(const uint32_t* lds, int lane) {
    const int m = lane & 15;
    base = lds + (m >> 3) * Stage<2>::kStride + 4 * (lane >> 4);
    sh = 2 * (m & 7);
  }

  // the operand of tile-row tr and tile pair jp (tiles 2 jp, 2 jp + 1)
  template <int TR, int JP>
  __device__ __forceinline__ h16x8 decode() const {
    const uint32_t* p = base + stage_slot<4>(TR, 2 * JP) * Stage<2>::kStride;
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_bit_cast(uint32_t, cba_decode_pair(__builtin_amdgcn_alignbit(p[i + 1], p[i], sh)));
    return __builtin_bit_cast(h16x8, u32x4{r[0], r[1], r[2], r[3]});
  }
};

// B operand of the parity layouts from four fp16 activations (two words):
// at the even B rows of the lane's group (parity 0) or the odd ones.
__device__ __forceinline__ h16x8 parity_operand(u32x2 v, int par) {
  const u32x4 d = par == 0 ? u32x4{v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16}
                           : u32x4{v.x << 16, v.x & 0xFFFF0000u, v.y << 16, v.y & 0xFFFF0000u};
  return __builtin_bit_cast(h16x8, d);
}

// Decode, for every pair pp of adjacent tile-rows (2pp, 2pp+1) and tile j of
// the staged region (NT tiles per row, at stage_slot<NT>), this lane's 8
// weights into A[pp][j] (A-operand layout).
template <int K, int NT = 4>
__device__ __forceinline__ void decode_stage_mfma(const uint32_t* lds, int lane,
                                                  h16x8 (&A)[4][NT]) {
  const OperandDecoder<K, NT> dec(lds, lane);
  dec.template decode<0>(A[0]);
  dec.template decode<1>(A[1]);
  dec.template decode<2>(A[2]);
  dec.template decode<3>(A[3]);
}

// Keep decoded operands where they are: an empty asm that claims to modify
// each register, so the compiler neither sinks the decode past a later
// point (a wait, the contraction) nor recomputes it there.
template <int NT>
__device__ __forceinline__ void pin_operands(h16x8 (&A)[4][NT]) {
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int j = 0; j < NT; ++j) asm volatile("" : "+v"(A[pp][j]));
}

static __device__ __noinline__ float2 scale_block(float m);

// Split a wave's 128 rotated activations (v0 at position lane, v1 at
// lane + 64) into fp16 high and low parts for B, scaled by a power of two
// that keeps both parts inside fp16's normal range: 1 unless the largest
// magnitude exceeds 2^14 or is below 2^-8 (then it is brought into
// [2^13, 2^14)). Returns the factor that undoes the scale.
__device__ __forceinline__ float split_hilo(float v0, float v1, _Float16* xh, _Float16* xl,
                                            int lane) {
  float m = fmaxf(fabsf(v0), fabsf(v1));
  float scale = 1.0f, unscale = 1.0f;
  // rare: large values, or a block whose values are all small
  if (__ballot(!(m <= 16384.0f)) != 0 || __ballot(m >= 0.00390625f) == 0) {
    const float2 su = scale_block(m);
    scale = su.x;
    unscale = su.y;
  }
  const float a0 = v0 * scale, a1 = v1 * scale;
  const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
  xh[lane] = h0;
  xh[lane + 64] = h1;
  xl[lane] = (_Float16)(a0 - (float)h0);
  xl[lane + 64] = (_Float16)(a1 - (float)h1);
  return unscale;
}

// The power-of-two scale of split_hilo for a block whose largest magnitude
// exceeds 2^14 or lies below 2^-8 (m: this lane's largest magnitude; NaN,
// infinity and an all-zero block leave the scale at 1): {scale, its
// inverse}.
static __device__ __noinline__ float2 scale_block(float m) {
  m = fmaxf(m, xor_lane<1>(m));
  m = fmaxf(m, xor_lane<2>(m));
  m = fmaxf(m, xor_lane<4>(m));
  m = fmaxf(m, xor_lane<8>(m));
  {
    const unsigned u = __float_as_uint(m);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const unsigned u = __float_as_uint(m);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  float scale = 1.0f, unscale = 1.0f;
  if ((m > 16384.0f && m <= 3.0e38f) || (m < 0.00390625f && m > 0.0f)) {
    int ex;
    frexpf(m * (1.0f / 16384.0f), &ex);
    scale = ldexpf(1.0f, -ex);
    unscale = ldexpf(1.0f, ex);
  }
  return make_float2(scale, unscale);
}

// z of the 4 tiles x 16 outputs of a wave from its accumulators: lane
// 16g (g = 0..3) receives outputs 4g .. 4g+3 of tile j in zr[j] (high part
// plus low part, times the unscale factor); other lanes' zr are unspecified.
__device__ __forceinline__ void finish_mfma(const f32x4 (&D)[4], float unscale, float4 (&zr)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = (D[j][q] + dpp<0xF5>(D[j][q])) * unscale;  // + lane l+1 (column 1)
    zr[j] = make_float4(r[0], r[1], r[2], r[3]);
  }
}

}  // namespace escha
