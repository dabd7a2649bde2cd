// escha_kernels.hip -- gfx950 kernels of the trellis-coded expert path and
// their host-side launchers (called by escha_api.cpp after validation).
//
// Streaming-decode kernels (small batches): one work-group per (pair, group
// of 16 output tiles = 256 outputs, chunk of 128 inputs = one Hadamard
// block). Each wave first issues the loads of its tile-rows of codes (one
// 16-byte load per lane per tile-row at K=2; the codes do not depend on the
// activations), then wave 0 rotates the chunk's 128 inputs in registers
// while the bytes are in flight; every wave then decodes in registers and
// accumulates in fp32. The waves' sums meet in LDS and splits over the
// input dimension land in a partial buffer that the next kernel reduces in
// a fixed order, so results are bit-reproducible with no atomics.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "escha_device.hpp"
#include "escha_launch.hpp"
#include "escha_stream.hpp"

namespace escha {

// ------------------------------------------------------------------------
// Router: softmax + top-k of a row of logits, one wave per row; each lane
// holds kMaxPer logits (E <= 64 kMaxPer). The wave-wide reductions run on
// DPP and permlane swaps (no LDS round trips): the max, the sum of the
// exponentials, and per selected expert an argmax.
// ------------------------------------------------------------------------

// (ov, oi) replaces (bv, bi) when it ranks higher: larger value, then
// smaller index.
__device__ __forceinline__ void take_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

// The highest-ranking (value, index) pair of the wave, in every lane.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  auto within_rows = [&](auto h) {
    constexpr int H = decltype(h)::value;
    const float ov = xor_lane<H>(bv);
    const int oi = __float_as_int(xor_lane<H>(__int_as_float(bi)));
    take_better(bv, bi, ov, oi);
  };
  within_rows(std::integral_constant<int, 1>{});
  within_rows(std::integral_constant<int, 2>{});
  within_rows(std::integral_constant<int, 4>{});
  within_rows(std::integral_constant<int, 8>{});
  // rows 16 apart, then halves 32 apart: both lanes of a pair see the same
  // two candidates (r[0], r[1]) and keep the same one
  {
    const auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto ri = __builtin_amdgcn_permlane16_swap((unsigned)bi, (unsigned)bi, false, false);
    bv = __uint_as_float(rv[0]);
    bi = (int)ri[0];
    take_better(bv, bi, __uint_as_float(rv[1]), (int)ri[1]);
  }
  {
    const auto rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto ri = __builtin_amdgcn_permlane32_swap((unsigned)bi, (unsigned)bi, false, false);
    bv = __uint_as_float(rv[0]);
    bi = (int)ri[0];
    take_better(bv, bi, __uint_as_float(rv[1]), (int)ri[1]);
  }
}

// The first `rounds` selections of the softmax top-k of row l (E logits),
// in decreasing-logit order, ties to the lower index: sel(r, expert,
// probability) is called in every lane for selection r (the same values in
// every lane; the probability is computed only WITH_W, else 0). Whole wave.
template <int kMaxPer, bool WITH_W = true, class F>
__device__ __forceinline__ void wave_topk(const float* __restrict__ l, int E, int rounds, int lane, F&& sel) {
  float v[kMaxPer];
  uint32_t taken = 0;
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? l[e] : -INFINITY;
    m = fmaxf(m, v[j]);
    if (e >= E) taken |= 1u << j;
  }
  float s = 0.f;
  if constexpr (WITH_W) {
    m = wave_max(m);
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
      if (lane + 64 * j < E) s += expf(v[j] - m);
    s = wave_sum(s);
  }
  for (int r = 0; r < rounds; ++r) {
    // lane-local best untaken, then the wave's
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
      if (!(taken & (1u << j))) take_better(bv, bi, v[j], lane + 64 * j);
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if constexpr (WITH_W)
      sel(r, bi, expf(bv - m) / s);
    else
      sel(r, bi, 0.f);
  }
}

// ------------------------------------------------------------------------
// gate_up (or any single projection): transformed partial sums over one
// 128-input chunk. grid.x = n_pairs * n_chunks * n_groups; block = 4 waves,
// wave w streams tile-rows 8c+2w and 8c+2w+1 of the 16 output tiles of
// group g.
// ------------------------------------------------------------------------
template <int K, bool FROM_Y>
__global__ __launch_bounds__(256) void k_in_partial(InPartialArgs a) {
  constexpr int kOwn = Quarter<K>::kOwn;
  const int n_groups = a.out_f / 256;
  const int n_chunks = a.in_f / 128;
  int bid = blockIdx.x;
  const int g = bid % n_groups;
  bid /= n_groups;
  const int c = bid % n_chunks;
  const int p = bid / n_chunks;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  float* out = a.partial + ((size_t)p * n_chunks + c) * a.out_f + g * 256;
  int e;
  if (a.logits) {
    // the router step inside: every wave selects the top (j + 1) of the
    // token's logits for its pair (slot j) as the standalone router step
    // does; the work-group of slot 0 (first chunk and group) stores all
    // top_k selections for the kernels that follow
    const int tt = p / a.top_k, j = p - tt * a.top_k;
    const bool writer = j == 0 && c == 0 && g == 0 && wave == 0;
    int32_t* ido = a.ids_out + (size_t)tt * a.top_k;
    float* wo = a.w_out + (size_t)tt * a.top_k;
    const float* lt = a.logits + (size_t)tt * a.n_experts;
    int ej = 0;
    if (writer) {
      wave_topk<kRouteFusedPer>(lt, a.n_experts, a.top_k, lane, [&](int r, int er, float wr) {
        if (r == 0) ej = er;
        if (lane == 0) {
          ido[r] = er;
          wo[r] = wr;
        }
      });
    } else {  // the selection only (no softmax weights)
      wave_topk<kRouteFusedPer, false>(lt, a.n_experts, j + 1, lane, [&](int r, int er, float) {
        if (r == j) ej = er;
      });
    }
    e = __builtin_amdgcn_readfirstlane(ej);
  } else {
    e = a.ids ? a.ids[p] : a.fixed_expert;
  }
  const bool valid = e >= 0 && e < a.n_experts;  // uniform over the block
  const int t = p / a.top_k;
  const int q = lane & 3;
  const int nt = g * 16 + (lane >> 2);
  const int n_nt = a.out_f / 16;

  // 1. the codes do not depend on the activations: start streaming them now
  uint32_t raw[2][kOwn];
  if (valid) {
    const uint16_t* code_e = a.code + (size_t)e * (size_t)(a.in_f / 16) * n_nt * (16 * K);
    issue_rows<K, 2>(code_e, n_nt, 8 * c + 2 * wave, nt, q, raw);
  }

  // 2. rotated inputs of this chunk: x~ = H_n(rin (.) x)
  __shared__ __attribute__((aligned(16))) float xs[128];
  __shared__ __attribute__((aligned(16))) float zs[256];
  __shared__ float4 red[4][64];
  if (wave == 0) {
    float x0, x1;
    if constexpr (FROM_Y) {
      // RMSNorm of the previous layer's output row, rounded to bf16
      const int nb = a.in_f / 128;
      const float* ss = a.ss_prev + (size_t)t * nb;
      // the blocks' sums of squares added in block order, the loads of each
      // group of 16 issued before its adds
      float tot = 0.f;
      for (int b0 = 0; b0 < nb; b0 += 16) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = ss[b0 + q < nb ? b0 + q : nb - 1];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (b0 + q < nb) tot += v[q];
      }
      const float inv = 1.0f / sqrtf(tot / (float)a.in_f + a.eps);
      const float* yr = a.y_prev + (size_t)t * a.in_f + c * 128;
      const uint16_t b0 = f32_to_bf16_rne(yr[lane] * inv);
      const uint16_t b1 = f32_to_bf16_rne(yr[lane + 64] * inv);
      if (a.x_out && g == 0 && p % a.top_k == 0) {
        uint16_t* xo = a.x_out + (size_t)t * a.in_f + c * 128;
        xo[lane] = b0;
        xo[lane + 64] = b1;
      }
      x0 = bf16_to_f32(b0);
      x1 = bf16_to_f32(b1);
    } else {
      const uint16_t* xr = a.x_bf16 + (size_t)t * a.in_f + c * 128;
      x0 = bf16_to_f32(xr[lane]);
      x1 = bf16_to_f32(xr[lane + 64]);
    }
    if (!valid) {  // an out-of-range expert id contributes nothing
      reinterpret_cast<float4*>(out)[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    const uint16_t* rr = a.rin + (size_t)e * a.in_f + c * 128;
    float v0 = x0 * f16_to_f32(rr[lane]);
    float v1 = x1 * f16_to_f32(rr[lane + 64]);
    fwht128(v0, v1);
    xs[lane] = v0 * kInvSqrt128;
    xs[lane + 64] = v1 * kInvSqrt128;
  }
  if (!valid) return;
  __syncthreads();

  // 3. decode and accumulate this wave's two tile-rows
  float acc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) acc[n] = 0.f;
  mac_rows<K, 2>(raw, 2 * wave, q, xs, acc);
  red[wave][lane] = quad_reduce_pick(acc, q);
  __syncthreads();

  // 4. fixed-order sum over the four waves, then the output transform
  if (wave == 0) {
    float4 r = red[0][lane];
    r = f4add(r, red[1][lane]);
    r = f4add(r, red[2][lane]);
    r = f4add(r, red[3][lane]);
    reinterpret_cast<float4*>(zs)[lane] = r;
  }
  __syncthreads();
  transform_store(zs, a.rout + (size_t)e * a.out_f + g * 256, 1.0f, out, wave, lane);
}

// ------------------------------------------------------------------------
// down: transformed, router-weighted partial sums over one 128-channel
// chunk of the inter dimension. grid.x = n_pairs * n_chunks * n_groups;
// block = 8 waves, wave w streams tile-row 8c+w. Wave 0 forms the chunk's
// h = SiLU(gate) * up from gate_up's transformed partials, then rin and
// H128 of down. A chunk whose 128 h values are all exactly zero (every
// channel pruned) contributes exactly zero: its decode is skipped.
// ------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(512) void k_down_partial(DownPartialArgs a) {
  constexpr int kOwn = Quarter<K>::kOwn;
  const int n_groups = a.out_f / 256;
  const int n_chunks = a.in_f / 128;  // in_f = inter
  // Work-groups are dealt to the 8 XCDs round-robin by index. All groups of
  // one (pair, chunk) read the same gate_up partials, so they are placed on
  // one XCD, whose L2 then fetches those partials once instead of 8 times.
  const int bid = blockIdx.x;
  const int n_pc = a.n_pairs * n_chunks;
  int g, pc;
  if (n_pc % 8 == 0) {
    const int i = bid >> 3;
    g = i % n_groups;
    pc = (i / n_groups) * 8 + (bid & 7);
  } else {
    g = bid % n_groups;
    pc = bid / n_groups;
  }
  const int c = pc % n_chunks;
  const int p = pc / n_chunks;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  float* out = a.partial + ((size_t)p * n_chunks + c) * a.out_f + g * 256;
  const int e = a.ids[p];
  if (e < 0 || e >= a.n_experts) {
    if (wave == 0) reinterpret_cast<float4*>(out)[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const int inter = a.in_f;
  const int g2 = 2 * inter;
  const int q = lane & 3;
  const int nt = g * 16 + (lane >> 2);
  const int n_nt = a.out_f / 16;
  const uint16_t* code_e = a.code + (size_t)e * (size_t)(inter / 16) * n_nt * (16 * K);

  uint32_t raw[1][kOwn];
  issue_rows<K, 1>(code_e, n_nt, 8 * c + wave, nt, q, raw);

  __shared__ __attribute__((aligned(16))) float xs[128];
  __shared__ __attribute__((aligned(16))) float zs[256];
  __shared__ float4 red[8][64];
  __shared__ int skip;
  if (wave == 0) {
    float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f;
    const float* gp = a.gu_partial + (size_t)p * a.gu_chunks * g2 + 128 * c;
#pragma unroll 16
    for (int cc = 0; cc < a.gu_chunks; ++cc) {
      const float* b = gp + (size_t)cc * g2;
      g0 += b[lane];
      g1 += b[lane + 64];
      u0 += b[inter + lane];
      u1 += b[inter + lane + 64];
    }
    if (a.gu_bias) {  // the dense export's gate/up biases, before the SiLU
      g0 += a.gu_bias[128 * c + lane];
      g1 += a.gu_bias[128 * c + lane + 64];
      u0 += a.gu_bias[inter + 128 * c + lane];
      u1 += a.gu_bias[inter + 128 * c + lane + 64];
    }
    const float h0 = silu(g0) * u0;
    const float h1 = silu(g1) * u1;
    if (a.inter_out && g == 0) {
      float* io = a.inter_out + (size_t)p * inter + 128 * c;
      io[lane] = h0;
      io[lane + 64] = h1;
    }
    const bool all_zero = __ballot((h0 != 0.f) || (h1 != 0.f)) == 0;
    const uint16_t* rr = a.rin + (size_t)e * inter + 128 * c;
    float v0 = h0 * f16_to_f32(rr[lane]);
    float v1 = h1 * f16_to_f32(rr[lane + 64]);
    fwht128(v0, v1);
    xs[lane] = v0 * kInvSqrt128;
    xs[lane + 64] = v1 * kInvSqrt128;
    if (lane == 0) skip = all_zero ? 1 : 0;
  }
  __syncthreads();
  if (skip) {  // uniform over the block
    if (wave == 0) reinterpret_cast<float4*>(out)[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  float acc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) acc[n] = 0.f;
  mac_rows<K, 1>(raw, wave, q, xs, acc);
  red[wave][lane] = quad_reduce_pick(acc, q);
  __syncthreads();
  if (wave == 0) {
    float4 r = red[0][lane];
#pragma unroll
    for (int w = 1; w < 8; ++w) r = f4add(r, red[w][lane]);
    reinterpret_cast<float4*>(zs)[lane] = r;
  }
  __syncthreads();
  const float wt = a.w ? a.w[p] : 1.0f;
  transform_store(zs, a.rout + (size_t)e * a.out_f + g * 256, wt, out, wave, lane);
}

// ------------------------------------------------------------------------
// Finish one projection per pair: the fixed-order sum of its chunks.
// grid.x = n_pairs * (out_f / 128), block = 64.
constexpr int kCombineRows = 32;  // partial rows whose loads are all issued before the first add

// ------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_proj_finish(FinishArgs a) {
  const int nb = a.out_f / 128;
  const int b = blockIdx.x % nb;
  const int p = blockIdx.x / nb;
  const int lane = threadIdx.x;
  float z0 = 0.f, z1 = 0.f;
  const float* pp = a.partial + (size_t)p * a.n_chunks * a.out_f + 128 * b;
  // every load of a group of kCombineRows chunks issued before the adds
  for (int c0 = 0; c0 < a.n_chunks; c0 += kCombineRows) {
    float v0[kCombineRows], v1[kCombineRows];
#pragma unroll
    for (int q = 0; q < kCombineRows; ++q) {
      const int cc = c0 + q < a.n_chunks ? c0 + q : a.n_chunks - 1;  // clamped: read, not added
      v0[q] = pp[(size_t)cc * a.out_f + lane];
      v1[q] = pp[(size_t)cc * a.out_f + lane + 64];
    }
#pragma unroll
    for (int q = 0; q < kCombineRows; ++q)
      if (c0 + q < a.n_chunks) {
        z0 += v0[q];
        z1 += v1[q];
      }
  }
  if (a.bias) {
    z0 += a.bias[128 * b + lane];
    z1 += a.bias[128 * b + lane + 64];
  }
  float* y = a.y + (size_t)p * a.out_f + 128 * b;
  y[lane] = z0;
  y[lane + 64] = z1;
}

// ------------------------------------------------------------------------
// Combine: one wave per (token, 128-block of hidden): the sum over slots (in
// order) and chunks (in order) of down's weighted, transformed partials,
// plus the block's sum of squares. grid.x = n_tokens * (hidden / 128).
// ------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_combine(CombineArgs a) {
  const int nb = a.hidden / 128;
  const int b = blockIdx.x % nb;
  const int t = blockIdx.x / nb;
  const int lane = threadIdx.x;
  const int n = a.top_k * a.n_chunks;  // partial rows of this token, in order
  const float* pp = a.partial + (size_t)t * n * a.hidden + 128 * b;
  float acc0 = 0.f, acc1 = 0.f;
  // groups of kCombineRows rows: every load of a group issued first (one
  // round trip per group), then the adds in row order
  for (int r0 = 0; r0 < n; r0 += kCombineRows) {
    float v0[kCombineRows], v1[kCombineRows];
#pragma unroll
    for (int q = 0; q < kCombineRows; ++q) {
      const int r = r0 + q < n ? r0 + q : n - 1;  // clamped: the row is read, not added
      v0[q] = pp[(size_t)r * a.hidden + lane];
      v1[q] = pp[(size_t)r * a.hidden + lane + 64];
    }
#pragma unroll
    for (int q = 0; q < kCombineRows; ++q)
      if (r0 + q < n) {
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
  const float ss = wave_sum(__builtin_fmaf(acc0, acc0, acc1 * acc1));
  if (lane == 0) a.ss[(size_t)t * nb + b] = ss;
}

// ------------------------------------------------------------------------
// Standalone RMSNorm -> bf16, with the same arithmetic as the fused path of
// the layer stack (block sums of squares as in k_combine, summed over the
// blocks in order, then the scale as in k_in_partial). grid.x = n_tokens,
// block = 1024 (wave w handles 128-blocks w, w+16, ..).
// ------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_rmsnorm_bf16(const float* __restrict__ y, int n, float eps,
                                                       uint16_t* __restrict__ x) {
  __shared__ float block_ss[128];  // n <= 16384
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nb = n / 128;
  const float* yr = y + (size_t)blockIdx.x * n;
  for (int b = wave; b < nb; b += 16) {
    const float a0 = yr[128 * b + lane], a1 = yr[128 * b + lane + 64];
    const float ss = wave_sum(__builtin_fmaf(a0, a0, a1 * a1));
    if (lane == 0) block_ss[b] = ss;
  }
  __syncthreads();
  float tot = 0.f;
  for (int b = 0; b < nb; ++b) tot += block_ss[b];
  const float inv = 1.0f / sqrtf(tot / (float)n + eps);
  uint16_t* xr = x + (size_t)blockIdx.x * n;
  for (int i = threadIdx.x; i < n; i += 1024) xr[i] = f32_to_bf16_rne(yr[i] * inv);
}

// ------------------------------------------------------------------------
// Decode one expert's weights to fp16 [out][in] (bit-exact export).
// grid.x = (in/16) * (out/256), block = 64.
// ------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(64) void k_decode_tiles(const uint16_t* __restrict__ code_e, int in_f,
                                                     int out_f, uint16_t* __restrict__ w) {
  const int n_groups = out_f / 256;
  const int g = blockIdx.x % n_groups;
  const int kt = blockIdx.x / n_groups;
  const int lane = threadIdx.x;
  const int q = lane & 3;
  const int nt = g * 16 + (lane >> 2);
  const int n_nt = out_f / 16;
  constexpr int kOwn = Quarter<K>::kOwn;
  uint32_t d[kOwn + 1];
  load_quarter<K>(code_e + ((size_t)kt * n_nt + nt) * (16 * K) + q * (4 * K), d);
  d[kOwn] = next_quarter_dword(d[0]);
  uint32_t cols[16][2];  // per output column n: rows 4q..4q+3 as two packed pairs
  decode_quarter<K>(d, [&](int kk, int n, h16x2 wv) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, wv);
    const uint32_t lo = bits & 0xFFFFu, hi = bits >> 16;
    uint32_t& c0 = cols[n][kk >> 1];
    uint32_t& c8 = cols[n + 8][kk >> 1];
    if (kk & 1) {
      c0 |= lo << 16;
      c8 |= hi << 16;
    } else {
      c0 = lo;
      c8 = hi;
    }
  });
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    uint16_t* dst = w + (size_t)(16 * nt + n) * in_f + 16 * kt + 4 * q;
    *reinterpret_cast<uint2*>(dst) = make_uint2(cols[n][0], cols[n][1]);
  }
}

// ------------------------------------------------------------------------
// y = H_n x per 128-block. grid.x = rows * (n/128), block = 64.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_hadamard128(const float* x, int n, float* y) {
  const int nb = n / 128;
  const size_t r = blockIdx.x / nb;
  const int b = blockIdx.x % nb;
  const int lane = threadIdx.x;
  const float* xr = x + r * n + 128 * b;
  float v0 = xr[lane], v1 = xr[lane + 64];
  fwht128(v0, v1);
  float* yr = y + r * n + 128 * b;
  yr[lane] = v0 * kInvSqrt128;
  yr[lane + 64] = v1 * kInvSqrt128;
}

// ------------------------------------------------------------------------
// Router logits: logit[t][e] = fp16(gate[e] . x[t]) (gate fp16 [E][H], x
// bf16 [T][H]; the model card's exactness table keeps the router gate in
// fp16, and the port's review notes round the logits to f16 before the
// top-k). The product of an fp16 and a bf16 value is exact in fp32; each
// lane adds its products with IEEE fp32 FMAs in input order, so the sum's
// error follows the textbook bound of sequential summation (the order of
// additions inside a matrix-core instruction is not specified).
// One wave per (32-expert tile, 32-token tile, input slice): lane (r, h)
// loads inputs 32c + 16q + 8h .. + 7 (q = 0, 1) of gate row 32et + r and of
// token 32tt + r for chunk c (16-byte loads, one chunk ahead of its use;
// rows past the end are clamped to the last row and their results
// dropped), converts them to fp32 into LDS ([input][row]), and then
// accumulates token r against experts 8p + 4h + m (p, m = 0..3) of the
// tile. With one slice the kernel rounds and stores the logits; otherwise
// it stores fp32 partial sums [slice][T][E], which k_router_reduce adds in
// slice order. grid.x = n_tiles * ksplit (slice fastest), block = 64.
// ------------------------------------------------------------------------

// A lane's operands of one 32-input chunk.
struct RouterChunk {
  u32x4 g[2], x[2];
};

__device__ __forceinline__ void router_load(const uint16_t* gp, const uint16_t* xp, int c,
                                            RouterChunk& o) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    o.g[q] = *reinterpret_cast<const u32x4*>(gp + 32 * c + 16 * q);
    o.x[q] = *reinterpret_cast<const u32x4*>(xp + 32 * c + 16 * q);
  }
}

__global__ __launch_bounds__(64) void k_router_logits(RouterArgs a) {
  __shared__ __attribute__((aligned(16))) float gs[32][32];  // [input][expert of the tile]
  __shared__ float xs[32][32];                               // [input][token of the tile]
  const int lane = threadIdx.x;
  const int ne = (a.E + 31) / 32;
  int b = blockIdx.x;
  const int ks = b % a.ksplit;
  b /= a.ksplit;
  const int et = b % ne, tt = b / ne;
  const int r = lane & 31, h = lane >> 5;
  const int er = 32 * et + r < a.E ? 32 * et + r : a.E - 1;
  const int tr = 32 * tt + r < a.T ? 32 * tt + r : a.T - 1;
  const int per = (a.H / 32) / a.ksplit;
  const int c0 = ks * per, c1 = c0 + per;
  const uint16_t* gp = a.gate + (size_t)er * a.H + 8 * h;
  const uint16_t* xp = a.x + (size_t)tr * a.H + 8 * h;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  RouterChunk cur;
  router_load(gp, xp, c0, cur);
  for (int c = c0; c < c1; ++c) {
    __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = 16 * q + 8 * h + j;
        gs[k][r] = f16_to_f32((uint16_t)(cur.g[q][j >> 1] >> (16 * (j & 1))));
        xs[k][r] = bf16_to_f32((uint16_t)(cur.x[q][j >> 1] >> (16 * (j & 1))));
      }
    // the next chunk's loads (past the slice: this chunk's again, unused)
    router_load(gp, xp, c + 1 < c1 ? c + 1 : c, cur);
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      const float xv = xs[k][r];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float4 g4 = *reinterpret_cast<const float4*>(&gs[k][8 * p + 4 * h]);
        acc[4 * p + 0] = __builtin_fmaf(g4.x, xv, acc[4 * p + 0]);
        acc[4 * p + 1] = __builtin_fmaf(g4.y, xv, acc[4 * p + 1]);
        acc[4 * p + 2] = __builtin_fmaf(g4.z, xv, acc[4 * p + 2]);
        acc[4 * p + 3] = __builtin_fmaf(g4.w, xv, acc[4 * p + 3]);
      }
    }
  }
  // lane holds token r, experts 8p + 4h + m (i = 4p + m) of the tile
  const int t = 32 * tt + r;
  if (t >= a.T) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = 32 * et + 8 * (i >> 2) + 4 * h + (i & 3);
    if (e < a.E) {
      if (a.ksplit == 1)
        a.logits[(size_t)t * a.E + e] = (float)(_Float16)acc[i];
      else
        a.part[((size_t)ks * a.T + t) * a.E + e] = acc[i];
    }
  }
}

// Router logits for a few tokens (T <= 8): one wave per expert; lane l
// sums inputs 32c .. 32c + 31 (c = l, l + 64, ...) of every token in input
// order with IEEE fp32 FMAs, and the wave adds its 64 lane sums in a fixed
// butterfly order; one RNE rounding to f16. No partial sums in memory.
// grid.x = ceil(E / 4), block = 256.
constexpr int kRouterGemvTokens = 8;

__global__ __launch_bounds__(256) void k_router_gemv(RouterArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = 4 * blockIdx.x + wave;
  if (e >= a.E) return;  // uniform over the wave
  float acc[kRouterGemvTokens];
#pragma unroll
  for (int t = 0; t < kRouterGemvTokens; ++t) acc[t] = 0.f;
  for (int c = lane; c < a.H / 32; c += 64) {
    const u32x4* gp = reinterpret_cast<const u32x4*>(a.gate + (size_t)e * a.H + 32 * c);
    float gf[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 g = gp[q];
#pragma unroll
      for (int j = 0; j < 8; ++j) gf[8 * q + j] = f16_to_f32((uint16_t)(g[j >> 1] >> (16 * (j & 1))));
    }
#pragma unroll
    for (int t = 0; t < kRouterGemvTokens; ++t) {
      if (t < a.T) {  // uniform
        const u32x4* xp = reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.H + 32 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 xv = xp[q];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[t] = __builtin_fmaf(gf[8 * q + j], bf16_to_f32((uint16_t)(xv[j >> 1] >> (16 * (j & 1)))),
                                    acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterGemvTokens; ++t) {
    if (t < a.T) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) a.logits[(size_t)t * a.E + e] = (float)(_Float16)s;
    }
  }
}

// Partial sums of the input slices added in slice order, then rounded to
// fp16 (round to nearest even). One thread per logit.
__global__ __launch_bounds__(256) void k_router_reduce(const float* __restrict__ part, int ksplit,
                                                       size_t n, float* __restrict__ logits) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // every slice's partial in flight at once (ksplit <= 32), then added in
  // slice order
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) v[k] = k < ksplit ? part[(size_t)k * n + i] : 0.f;
  float s = v[0];
#pragma unroll
  for (int k = 1; k < 32; ++k)
    if (k < ksplit) s += v[k];
  logits[i] = (float)(_Float16)s;
}

// Router step on its own: one wave per token. grid.x = n_tokens, block = 64.
template <int kMaxPer>
__global__ __launch_bounds__(64) void k_route_topk(const float* __restrict__ logits, int E, int k,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  wave_topk<kMaxPer>(logits + (size_t)t * E, E, k, lane, [&](int r, int e, float wr) {
    if (lane == 0) {
      ids[(size_t)t * k + r] = e;
      w[(size_t)t * k + r] = wr;
    }
  });
}

// ------------------------------------------------------------------------
// Grouping pairs by expert (counting sort, stable in the pair index).
// Pass 1: per chunk of 64 pairs, per-expert counts and in-chunk ranks.
// Pass 2: one block scans the chunk counts per expert and the totals.
// Pass 3: scatter.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_group_count(const int32_t* __restrict__ ids, int P, int E,
                                                    int32_t* __restrict__ hist,
                                                    int32_t* __restrict__ rank) {
  const int chunk = blockIdx.x;
  const int lane = threadIdx.x;
  // layer blockIdx.y of a batch of groupings (gridDim.x = chunks per layer)
  const size_t ly = blockIdx.y;
  ids += ly * P;
  hist += ly * gridDim.x * E;
  rank += ly * P;
  const int i = chunk * 64 + lane;
  const int e = i < P ? ids[i] : -1;
  const bool valid = e >= 0 && e < E;
  int r = 0;
  for (int s = 0; s < 64; ++s) {
    const int es = __shfl(e, s, 64);
    if (s < lane && es == e) ++r;
  }
  int32_t* hrow = hist + (size_t)chunk * E;
  for (int x = lane; x < E; x += 64) hrow[x] = 0;
  __syncthreads();
  // the last lane of each run of equal experts (highest rank) writes the count
  bool last = valid;
  for (int s = 0; s < 64; ++s) {
    const int es = __shfl(e, s, 64);
    if (s > lane && es == e) last = false;
  }
  if (valid && last) hrow[e] = r + 1;
  if (i < P) rank[i] = valid ? r : -1;
}

// Pass 2a: one block per expert: exclusive scan of its chunk counts.
__global__ __launch_bounds__(256) void k_group_scan(const int32_t* __restrict__ hist, int n_chunks,
                                                    int E, int32_t* __restrict__ base,
                                                    int32_t* __restrict__ counts) {
  __shared__ int32_t part[256];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t ly = blockIdx.y;  // layer of a batch of groupings
  hist += ly * n_chunks * E;
  base += ly * n_chunks * E;
  counts += ly * E;
  // each thread owns a contiguous run of chunks
  const int per = (n_chunks + 255) / 256;
  const int c0 = tid * per;
  int32_t run = 0;
  for (int c = c0; c < c0 + per && c < n_chunks; ++c) run += hist[(size_t)c * E + e];
  part[tid] = run;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int32_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t acc = part[tid] - run;  // exclusive prefix of this thread's run
  for (int c = c0; c < c0 + per && c < n_chunks; ++c) {
    base[(size_t)c * E + e] = acc;
    acc += hist[(size_t)c * E + e];
  }
  if (tid == 255) counts[e] = part[255];
}

// Pass 2b: offsets = exclusive prefix sums of the counts (E <= 1024).
__global__ __launch_bounds__(1024) void k_group_offsets(const int32_t* __restrict__ counts, int E,
                                                        int32_t* __restrict__ offsets) {
  __shared__ int32_t scan[1024];
  const int e = threadIdx.x;
  const size_t ly = blockIdx.y;  // layer of a batch of groupings
  counts += ly * E;
  offsets += ly * (E + 1);
  const int32_t v0 = e < E ? counts[e] : 0;
  scan[e] = v0;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int32_t v = e >= d ? scan[e - d] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e] = scan[e] - v0;
  if (e == 0) offsets[E] = scan[1023];
}

__global__ __launch_bounds__(64) void k_group_scatter(const int32_t* __restrict__ ids, int P, int E,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ inv) {
  const size_t ly = blockIdx.y;  // layer of a batch of groupings
  ids += ly * P;
  base += ly * gridDim.x * E;
  rank += ly * P;
  offsets += ly * (E + 1);
  perm += ly * P;
  if (inv) inv += ly * P;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= P) return;
  const int e = ids[i];
  if (e < 0 || e >= E) {
    if (inv) inv[i] = -1;
    return;
  }
  const int pos = offsets[e] + base[(size_t)blockIdx.x * E + e] + rank[i];
  perm[pos] = i;
  if (inv) inv[i] = pos;
}

// ------------------------------------------------------------------------
// Grouping of up to kGroupSmallPairs pairs in one work-group of 1024 threads
// (one launch instead of count, scan, offsets, scatter and tile list): the
// same results as the multi-pass path -- counts, offsets, the stable
// permutation (sorted index -> pair, ties in pair order), its inverse, and
// optionally the tile list (tiles of tm
// consecutive sorted pairs of one expert, experts in order). Pairs are
// taken 1024 at a time; inside a wave, the lanes holding the same expert
// are found with one ballot per bit of the expert index; a wave's count per
// expert goes to LDS, and the rank of a pair is the expert's running count
// before this chunk + the counts of the earlier waves of the chunk + its
// rank among the wave's lanes with that expert. grid.y = layer of a batch.
// ------------------------------------------------------------------------
constexpr int kGroupSmallPairs = 8192;
constexpr int kGroupSmallExperts = 256;  // wave-count table in LDS: 16 waves x 256 experts

__global__ __launch_bounds__(1024) void k_group_small(const int32_t* __restrict__ ids, int P, int E,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                      int tm, int max_tiles, int32_t* __restrict__ t_expert,
                                                      int32_t* __restrict__ t_row0,
                                                      int32_t* __restrict__ t_rows,
                                                      int32_t* __restrict__ n_tiles,
                                                      int32_t* __restrict__ clear, int n_clear) {
  __shared__ int32_t cnt[kGroupSmallExperts];       // per expert: running count, then its offset
  __shared__ int32_t wc[16][kGroupSmallExperts];    // per wave of the chunk and expert: its count
  __shared__ int32_t scan[1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;  // bits of the largest expert index
  const size_t ly = blockIdx.y;
  ids += ly * P;
  counts += ly * E;
  offsets += ly * (E + 1);
  perm += ly * P;
  if (inv) inv += ly * P;
  // the layer's control block of the one-launch small-tile layer kernel
  if (clear)
    for (int i = tid; i < n_clear; i += 1024) clear[ly * n_clear + i] = 0;
  // pass 1: counts (LDS atomics on integers: exact, order-free)
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  for (int i = tid; i < P; i += 1024) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // offsets: exclusive scan of the counts
  const int32_t c0 = tid < E ? cnt[tid] : 0;
  scan[tid] = c0;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int32_t v = tid >= d ? scan[tid - d] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int32_t off = scan[tid] - c0;
  if (tid < E) {
    counts[tid] = c0;
    offsets[tid] = off;
    cnt[tid] = off;  // now: the next free sorted index of the expert
  }
  if (tid == 0) offsets[E] = scan[1023];
  // the tile list: ceil(count / tm) tiles per expert, experts in order
  if (t_expert) {
    __syncthreads();
    const int32_t nt = tid < E ? (c0 + tm - 1) / tm : 0;
    scan[tid] = nt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int32_t v = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    t_expert += ly * max_tiles;
    t_row0 += ly * max_tiles;
    t_rows += ly * max_tiles;
    const int32_t b = scan[tid] - nt;
    for (int q = 0; q < nt; ++q)
      if (b + q < max_tiles) {
        t_expert[b + q] = tid;
        t_row0[b + q] = off + q * tm;
        t_rows[b + q] = c0 - q * tm < tm ? c0 - q * tm : tm;
      }
    if (tid == 1023) n_tiles[ly] = scan[1023] < max_tiles ? scan[1023] : max_tiles;
  }
  // pass 2: the stable scatter, 1024 pairs at a time
  for (int i0 = 0; i0 < P; i0 += 1024) {
    for (int q = tid; q < 16 * kGroupSmallExperts; q += 1024) (&wc[0][0])[q] = 0;
    __syncthreads();
    const int i = i0 + tid;
    const int e = i < P ? ids[i] : -1;
    const bool valid = e >= 0 && e < E;
    // lanes of this wave holding the same expert: one ballot per index bit
    uint64_t same = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t ones = __ballot(valid && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? ones : ~ones;
    }
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int r_wave = __popcll(same & below);
    if (valid && r_wave == __popcll(same) - 1) wc[wave][e] = __popcll(same);  // the last such lane
    __syncthreads();
    if (valid) {
      int pos = cnt[e] + r_wave;
      for (int w = 0; w < wave; ++w) pos += wc[w][e];
      perm[pos] = i;
      if (inv) inv[i] = pos;
    } else if (i < P && inv) {
      inv[i] = -1;
    }
    __syncthreads();
    // advance the experts' cursors by this chunk's counts
    if (tid < E) {
      int add = 0;
      for (int w = 0; w < 16; ++w) add += wc[w][tid];
      cnt[tid] += add;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_fill_one_expert(int32_t* __restrict__ ids, float* __restrict__ w,
                                                        int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    ids[i] = 0;
    w[i] = 1.0f;
  }
}

// ------------------------------------------------------------------------
// Host launchers.
// ------------------------------------------------------------------------
static hipError_t last_launch() { return hipGetLastError(); }

hipError_t launch_fill_one_expert(int32_t* ids, float* w, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_one_expert, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids, w, n);
  return last_launch();
}

hipError_t launch_in_partial(const InPartialArgs& a, int k_bits, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)a.n_pairs * (a.in_f / 128) * (a.out_f / 256));
  const bool from_y = a.x_bf16 == nullptr;
  if (k_bits == 2) {
    if (from_y)
      hipLaunchKernelGGL((k_in_partial<2, true>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_in_partial<2, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (from_y)
      hipLaunchKernelGGL((k_in_partial<3, true>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_in_partial<3, false>), dim3(grid), dim3(256), 0, s, a);
  }
  return last_launch();
}

hipError_t launch_down_partial(const DownPartialArgs& a, int k_bits, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)a.n_pairs * (a.in_f / 128) * (a.out_f / 256));
  if (k_bits == 2)
    hipLaunchKernelGGL(k_down_partial<2>, dim3(grid), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(k_down_partial<3>, dim3(grid), dim3(512), 0, s, a);
  return last_launch();
}

hipError_t launch_proj_finish(const FinishArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)a.n_pairs * (a.out_f / 128));
  hipLaunchKernelGGL(k_proj_finish, dim3(grid), dim3(64), 0, s, a);
  return last_launch();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)a.n_tokens * (a.hidden / 128));
  hipLaunchKernelGGL(k_combine, dim3(grid), dim3(64), 0, s, a);
  return last_launch();
}

hipError_t launch_rmsnorm_bf16(const float* y, int n_tokens, int n, float eps, uint16_t* x,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm_bf16, dim3(n_tokens), dim3(1024), 0, s, y, n, eps, x);
  return last_launch();
}

hipError_t launch_decode_tiles(const uint16_t* code_e, int in_f, int out_f, int k_bits,
                               uint16_t* w, hipStream_t s) {
  const unsigned grid = (unsigned)((in_f / 16) * (out_f / 256));
  if (k_bits == 2)
    hipLaunchKernelGGL(k_decode_tiles<2>, dim3(grid), dim3(64), 0, s, code_e, in_f, out_f, w);
  else
    hipLaunchKernelGGL(k_decode_tiles<3>, dim3(grid), dim3(64), 0, s, code_e, in_f, out_f, w);
  return last_launch();
}

hipError_t launch_hadamard128(const float* x, int64_t rows, int n, float* y, hipStream_t s) {
  const size_t blocks = (size_t)rows * (n / 128);
  const size_t max_grid = 0x7FFFFFFFu;
  // split very tall inputs into several launches of whole rows
  const int64_t rows_per = (int64_t)(max_grid / (n / 128));
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per) {
    const int64_t nr = rows - r0 < rows_per ? rows - r0 : rows_per;
    hipLaunchKernelGGL(k_hadamard128, dim3((unsigned)(nr * (n / 128))), dim3(64), 0, s,
                       x + r0 * n, n, y + r0 * n);
    const hipError_t err = last_launch();
    if (err != hipSuccess) return err;
  }
  (void)blocks;
  return hipSuccess;
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s) {
  if (E <= 256)
    hipLaunchKernelGGL(k_route_topk<4>, dim3(T), dim3(64), 0, s, logits, E, k, ids, w);
  else if (E <= 512)
    hipLaunchKernelGGL(k_route_topk<8>, dim3(T), dim3(64), 0, s, logits, E, k, ids, w);
  else
    hipLaunchKernelGGL(k_route_topk<16>, dim3(T), dim3(64), 0, s, logits, E, k, ids, w);
  return last_launch();
}

int router_ksplit(int T, int H, int E) {
  if (T <= kRouterGemvTokens) return 1;  // k_router_gemv
  const int tiles = ((E + 31) / 32) * ((T + 31) / 32);
  const int nch = H / 32;
  int ks = 1;
  while (ks < 32 && nch % (2 * ks) == 0 && tiles * 2 * ks <= 4096) ks *= 2;
  return ks;
}

hipError_t launch_router_logits(const RouterArgs& a, hipStream_t s) {
  if (a.T <= kRouterGemvTokens) {
    hipLaunchKernelGGL(k_router_gemv, dim3((unsigned)((a.E + 3) / 4)), dim3(256), 0, s, a);
    return last_launch();
  }
  const unsigned grid = (unsigned)(((a.E + 31) / 32) * ((a.T + 31) / 32) * a.ksplit);
  hipLaunchKernelGGL(k_router_logits, dim3(grid), dim3(64), 0, s, a);
  hipError_t err = last_launch();
  if (err != hipSuccess || a.ksplit == 1) return err;
  const size_t n = (size_t)a.T * a.E;
  hipLaunchKernelGGL(k_router_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.part,
                     a.ksplit, n, a.logits);
  return last_launch();
}

bool group_small_ok(int P, int E) { return P <= kGroupSmallPairs && E <= kGroupSmallExperts; }

hipError_t launch_group_small(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* inv, int tm, int max_tiles, int32_t* t_expert,
                              int32_t* t_row0, int32_t* t_rows, int32_t* n_tiles, hipStream_t s, int n_layers,
                              int32_t* clear, int n_clear) {
  hipLaunchKernelGGL(k_group_small, dim3(1, (unsigned)n_layers), dim3(1024), 0, s, ids, P, E, counts, offsets,
                     perm, inv, tm, max_tiles, t_expert, t_row0, t_rows, n_tiles, clear, n_clear);
  return last_launch();
}

hipError_t launch_group(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* inv, int32_t* hist, int32_t* base, int32_t* rank,
                        hipStream_t s, int n_layers) {
  const int n_chunks = (P + 63) / 64;
  const unsigned L = (unsigned)n_layers;
  if (n_chunks > 0) {
    hipLaunchKernelGGL(k_group_count, dim3(n_chunks, L), dim3(64), 0, s, ids, P, E, hist, rank);
    hipError_t err = last_launch();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_group_scan, dim3(E, L), dim3(256), 0, s, hist, n_chunks, E, base, counts);
  hipError_t err = last_launch();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_group_offsets, dim3(1, L), dim3(1024), 0, s, counts, E, offsets);
  err = last_launch();
  if (err != hipSuccess || n_chunks == 0) return err;
  hipLaunchKernelGGL(k_group_scatter, dim3(n_chunks, L), dim3(64), 0, s, ids, P, E, base, rank,
                     offsets, perm, inv);
  return last_launch();
}

}  // namespace escha
