// escha_shared.hip -- the shared expert of the MoE block in its w8a16 form
// and its gate: int8 weights with f32 scales per group of 128 inputs
// (weight = scale * w8), applied to the bf16 hidden state with fp32
// accumulation; the
// shared_expert_gate (one fp16 row) scales the expert's output through a
// sigmoid, and the result is added to the routed experts' output.
// Sources: model card "Qwen3.6-35B-A3B-Escha-W2-trellis-mlx", exactness
// table (shared expert in affine Q8 group-128 with f32 scales, bit-exact to
// the int8 w8a16 contract with dequantisation scale * w8; router gates,
// shared_expert_gate among them, in fp16); PR "serve Qwen3.6-35B-A3B-
// Escha-W2 natively", improvements table (int8 non-experts run as a fused
// matvec, never dequantised at load).
//
// The contraction runs on the matrix cores in bf16 with fp32 accumulation:
// an int8 weight is exactly a bf16 number and the hidden state is bf16, so
// v_mfma_f32_16x16x32_bf16 forms the exact products w8 * x; each group of
// 128 inputs is summed on its own and multiplied by its f32 scale in the
// fp32 accumulation (sum over groups of scale * sum(w8 * x), the same sum
// as sum(scale * w8 * x) up to fp32 rounding). The down projection's input
// h (fp32) enters as two bf16 parts, h = hi + lo (hi = bf16(h), lo =
// bf16(h - hi)), i.e. 16 significant bits, in two contractions.
//
// Work split: a work-group owns 16 output channels and up to 32 tokens;
// its waves split the inputs (one or two whole 128-input groups each, all
// of a wave's loads issued before its first contraction), their partial
// sums are added in LDS in wave order, and the work-group finishes its
// outputs (gate_up: h = SiLU(gate) * up; down: the sigmoid gate and the add
// into y).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "escha_device.hpp"
#include "escha_launch.hpp"

namespace escha {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kShTile = 32;           // tokens per work-group
constexpr int kShSub = kShTile / 16;  // 16-token sub-tiles
constexpr int kShMaxWaves = 16;       // waves per work-group (one or two 128-input groups each)

// 8 int8 weights (one 8-byte word pair) as 8 bf16 values (exact).
__device__ __forceinline__ bf16x8 w8_to_bf16(u32x2 w) {
  bf16x8 r;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint32_t word = b < 4 ? w.x : w.y;
    r[b] = (__bf16)(float)(int)(int8_t)((word >> (8 * (b & 3))) & 0xFFu);
  }
  return r;
}

// 8 of the 16 bytes of a weight word: bytes 8 hf .. 8 hf + 7.
__device__ __forceinline__ u32x2 half_words(u32x4 w, int hf) {
  return hf ? u32x2{w.z, w.w} : u32x2{w.x, w.y};
}

// The MFMA B operand of sub-tile st: lane (n, g) holds inputs k .. k + 7
// (k: the lane's own) of token t0 + 16 st + n (zeros past the last token).
__device__ __forceinline__ bf16x8 x_operand(const uint16_t* __restrict__ x, int H, int T, int t0, int st,
                                            int k, int lane) {
  const int t = t0 + 16 * st + (lane & 15);
  const int tc = t < T ? t : T - 1;
  u32x4 v = *reinterpret_cast<const u32x4*>(x + (size_t)tc * H + k);
  if (t >= T) v = u32x4{0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, v);
}

// The B operands of sub-tile st from fp32 h (inputs k .. k + 7 of the
// lane's token): high and low bf16 parts.
__device__ __forceinline__ void h_operands(const float* __restrict__ h, int I, int T, int t0, int st, int k,
                                           int lane, bf16x8& hi, bf16x8& lo) {
  const int t = t0 + 16 * st + (lane & 15);
  const int tc = t < T ? t : T - 1;
  const float* hp = h + (size_t)tc * I + k;
  const float4 v0 = *reinterpret_cast<const float4*>(hp);
  const float4 v1 = *reinterpret_cast<const float4*>(hp + 4);
  const float hv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const float v = t < T ? hv[b] : 0.f;
    hi[b] = (__bf16)v;
    lo[b] = (__bf16)(v - (float)hi[b]);
  }
}

// Scale the group's sums of a 16-row tile (rows row0 + 4 g + r of lane
// (n, g)) by their group scales and add them to acc.
__device__ __forceinline__ void add_scaled(const float* __restrict__ sc, int ngrp, int row0, int grp,
                                           const f32x4v (&part)[kShSub], f32x4v (&acc)[kShSub], int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float s = sc[(size_t)(row0 + 4 * g + r) * ngrp + grp];
#pragma unroll
    for (int st = 0; st < kShSub; ++st) acc[st][r] = __builtin_fmaf(s, part[st][r], acc[st][r]);
  }
}

}  // namespace

// gate_up of the shared expert and its gate logits. grid = (inter / 16 + 1,
// ceil(T / 32)), block = 64 * (hidden / 128 / GPW): work-group (j, tt) <
// inter / 16 owns channels 16 j .. 16 j + 15 (gate rows 16 j + n, up rows
// inter + 16 j + n) for tokens 32 tt ..; wave w sums the GPW 128-input
// groups from w GPW on (every load of the wave is issued before its first
// contraction). The last work-group of each token tile computes the gate
// logits (fp16 gate . bf16 x, fp32, wave w: tokens w, w + waves, ..).
template <int GPW>
__global__ __launch_bounds__(64 * kShMaxWaves) void k_shared_gate_up(SharedArgs a) {
  __shared__ float red[kShMaxWaves][2][kShSub][64][4];  // 64 KiB
  const int H = a.hidden, I = a.inter, T = a.n_tokens;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int t0 = kShTile * blockIdx.y;
  const int nt = T - t0 < kShTile ? T - t0 : kShTile;
  if (blockIdx.x == (unsigned)(I / 16)) {
    // gate logits: lane l holds the 8-value chunks l, l + 64, .. of the row
    // (all of them loaded before the first product; at most kShMaxHidden / 512)
    constexpr int kGateChunks = kShMaxHidden / 512;
    const int nch = H / 512;
    u32x4 gv[kGateChunks];
#pragma unroll
    for (int m = 0; m < kGateChunks; ++m)
      if (m < nch) gv[m] = *reinterpret_cast<const u32x4*>(a.gate + 8 * (lane + 64 * m));
    for (int tl = wave; tl < nt; tl += nw) {
      const uint16_t* xr = a.x + (size_t)(t0 + tl) * H;
      u32x4 xv[kGateChunks];
#pragma unroll
      for (int m = 0; m < kGateChunks; ++m)
        if (m < nch) xv[m] = *reinterpret_cast<const u32x4*>(xr + 8 * (lane + 64 * m));
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < kGateChunks; ++m)
        if (m < nch) {
#pragma unroll
          for (int b = 0; b < 8; ++b)
            acc = __builtin_fmaf(f16_to_f32((uint16_t)(gv[m][b >> 1] >> (16 * (b & 1)))),
                                 bf16_to_f32((uint16_t)(xv[m][b >> 1] >> (16 * (b & 1)))), acc);
        }
      acc = wave_sum(acc);
      if (lane == 0) a.glogit[t0 + tl] = acc;
    }
    return;
  }
  const int c0 = 16 * blockIdx.x;
  const int ngrp = H / 128;
  const int kb = 128 * GPW * wave;
  // every weight word and activation operand of the wave, then the
  // contractions. Inside a group, contraction step ks takes inputs 32 g +
  // 8 ks .. + 7 in lane group g (the same order for weights and
  // activations), so that a lane reads 32 contiguous bytes of each weight
  // row and 64 of each activation row per group.
  u32x4 wg[GPW][2], wu[GPW][2];
  bf16x8 B[GPW][4][kShSub];
#pragma unroll
  for (int q = 0; q < GPW; ++q) {
    const int kq = kb + 128 * q + 32 * g;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      wg[q][h2] = *reinterpret_cast<const u32x4*>(a.gu_w + (size_t)(c0 + n) * H + kq + 16 * h2);
      wu[q][h2] = *reinterpret_cast<const u32x4*>(a.gu_w + (size_t)(I + c0 + n) * H + kq + 16 * h2);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int st = 0; st < kShSub; ++st) B[q][ks][st] = x_operand(a.x, H, T, t0, st, kq + 8 * ks, lane);
  }
  f32x4v dg[kShSub], du[kShSub];
#pragma unroll
  for (int st = 0; st < kShSub; ++st) dg[st] = du[st] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < GPW; ++q) {
    f32x4v pg[kShSub], pu[kShSub];
#pragma unroll
    for (int st = 0; st < kShSub; ++st) pg[st] = pu[st] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 Ag = w8_to_bf16(half_words(wg[q][ks >> 1], ks & 1));
      const bf16x8 Au = w8_to_bf16(half_words(wu[q][ks >> 1], ks & 1));
#pragma unroll
      for (int st = 0; st < kShSub; ++st) {
        pg[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ag, B[q][ks][st], pg[st], 0, 0, 0);
        pu[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Au, B[q][ks][st], pu[st], 0, 0, 0);
      }
    }
    const int grp = GPW * wave + q;
    add_scaled(a.gu_s, ngrp, c0, grp, pg, dg, lane);
    add_scaled(a.gu_s, ngrp, I + c0, grp, pu, du, lane);
  }
#pragma unroll
  for (int st = 0; st < kShSub; ++st) {
    *reinterpret_cast<f32x4v*>(red[wave][0][st][lane]) = dg[st];
    *reinterpret_cast<f32x4v*>(red[wave][1][st][lane]) = du[st];
  }
  __syncthreads();
  // (channel c0 + cl, token t0 + tl) per thread: the waves' sums added in
  // wave order, then h = SiLU(gate) * up
  for (int idx = threadIdx.x; idx < 16 * kShTile; idx += blockDim.x) {
    const int cl = idx & 15, tl = idx >> 4;
    if (tl >= nt) break;
    const int st = tl >> 4, ln = 16 * (cl >> 2) + (tl & 15), r = cl & 3;
    float gs = red[0][0][st][ln][r], us = red[0][1][st][ln][r];
#pragma unroll
    for (int w = 1; w < kShMaxWaves; ++w)
      if (w < nw) {
        gs += red[w][0][st][ln][r];
        us += red[w][1][st][ln][r];
      }
    a.h[(size_t)(t0 + tl) * I + c0 + cl] = silu(gs) * us;
  }
}

// down of the shared expert, the sigmoid gate and the add into y. grid =
// (hidden / 16, ceil(T / 32)), block = 64 * (inter / 128): work-group (o, tt)
// owns output rows 16 o .. 16 o + 15 for tokens 32 tt ..; wave w sums
// channel group w with h split into bf16 high and low parts.
__global__ __launch_bounds__(64 * kShMaxWaves) void k_shared_down(SharedArgs a) {
  __shared__ float red[kShMaxWaves][kShSub][64][4];  // 32 KiB
  const int H = a.hidden, I = a.inter, T = a.n_tokens;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int t0 = kShTile * blockIdx.y;
  const int nt = T - t0 < kShTile ? T - t0 : kShTile;
  const int r0 = 16 * blockIdx.x;
  const int kq = 128 * wave + 32 * g;  // the lane's inputs of the group (steps as in gate_up)
  u32x4 wd[2];
  bf16x8 hi[4][kShSub], lo[4][kShSub];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) wd[h2] = *reinterpret_cast<const u32x4*>(a.dn_w + (size_t)(r0 + n) * I + kq + 16 * h2);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int st = 0; st < kShSub; ++st) h_operands(a.h, I, T, t0, st, kq + 8 * ks, lane, hi[ks][st], lo[ks][st]);
  f32x4v p[kShSub], d[kShSub];
#pragma unroll
  for (int st = 0; st < kShSub; ++st) p[st] = d[st] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 A = w8_to_bf16(half_words(wd[ks >> 1], ks & 1));
#pragma unroll
    for (int st = 0; st < kShSub; ++st) {
      p[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, hi[ks][st], p[st], 0, 0, 0);
      p[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, lo[ks][st], p[st], 0, 0, 0);
    }
  }
  add_scaled(a.dn_s, I / 128, r0, wave, p, d, lane);
#pragma unroll
  for (int st = 0; st < kShSub; ++st) *reinterpret_cast<f32x4v*>(red[wave][st][lane]) = d[st];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * kShTile; idx += blockDim.x) {
    const int ol = idx & 15, tl = idx >> 4;
    if (tl >= nt) break;
    const int st = tl >> 4, ln = 16 * (ol >> 2) + (tl & 15), r = ol & 3;
    float s = red[0][st][ln][r];
#pragma unroll
    for (int w = 1; w < kShMaxWaves; ++w)
      if (w < nw) s += red[w][st][ln][r];
    const float gt = 1.0f / (1.0f + expf(-a.glogit[t0 + tl]));
    float* yp = a.y + (size_t)(t0 + tl) * H + r0 + ol;
    *yp = a.accumulate ? *yp + gt * s : gt * s;
  }
}

hipError_t launch_shared_expert(const SharedArgs& a, hipStream_t s) {
  if (a.n_tokens <= 0) return hipSuccess;
  const unsigned tiles = (unsigned)((a.n_tokens + kShTile - 1) / kShTile);
  const int ngrp = a.hidden / 128;  // 8, 16 or 32 (hidden 1024 .. 4096)
  const int gpw = ngrp > kShMaxWaves ? 2 : 1;
  const dim3 gu_grid((unsigned)(a.inter / 16 + 1), tiles), gu_block((unsigned)(64 * (ngrp / gpw)));
  if (gpw == 1)
    hipLaunchKernelGGL(k_shared_gate_up<1>, gu_grid, gu_block, 0, s, a);
  else
    hipLaunchKernelGGL(k_shared_gate_up<2>, gu_grid, gu_block, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_shared_down, dim3((unsigned)(a.hidden / 16), tiles), dim3((unsigned)(64 * (a.inter / 128))),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace escha
