// escha_shared.hip -- the shared expert of the MoE block in its w8a16 form
// and its gate: int8 weights with f32 scales per group of 128 inputs,
// dequantised in registers (weight = scale * w8, one binary32 multiply) and
// applied to the bf16 hidden state with fp32 accumulation; the
// shared_expert_gate (one fp16 row) scales the expert's output through a
// sigmoid, and the result is added to the routed experts' output.
// Sources: model card "Qwen3.6-35B-A3B-Escha-W2-trellis-mlx", exactness
// table (shared expert in affine Q8 group-128 with f32 scales, bit-exact to
// the int8 w8a16 contract with dequantisation scale * w8; router gates,
// shared_expert_gate among them, in fp16); PR "serve Qwen3.6-35B-A3B-
// Escha-W2 natively", improvements table (int8 non-experts run as a fused
// matvec, never dequantised at load).
//
// Decode-sized batches: the weights stream once per group of 8 tokens, each
// wave owns one output channel (gate_up: gate row c and up row inter + c, so
// that h = SiLU(gate) * up is finished in the wave; down: one hidden row),
// lanes split the inputs in 16-byte (gate_up) / 8-byte (down) chunks, and
// the 64 lane sums of a token are added in a fixed butterfly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "escha_device.hpp"
#include "escha_launch.hpp"

namespace escha {

namespace {

constexpr int kShTok = 8;  // tokens per pass over the weights

// Dequantised int8 lane of a packed dword (byte b, sign-extended) times its
// group scale: one binary32 multiply.
__device__ __forceinline__ float dq(uint32_t word, int b, float scale) {
  const int q = (int)(int8_t)((word >> (8 * b)) & 0xFFu);
  return scale * (float)q;
}

}  // namespace

// gate_up of the shared expert and its gate logits. grid.x = inter / 4 + 1,
// block = 256: wave w of work-group b < inter / 4 owns channel c = 4 b + w;
// the last work-group computes the gate logits (wave w: tokens w, w + 4, ..).
// The token tile's bf16 inputs are staged in LDS (dynamic, 2 * 8 * hidden
// bytes). Lane l holds the 16-byte chunks l, l + 64, .. of its two rows.
__global__ __launch_bounds__(256) void k_shared_gate_up(SharedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [kShTok][hidden]
  const int H = a.hidden, I = a.inter, T = a.n_tokens;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = H / 16;            // 16-input chunks of a weight row
  const int per = (nch + 63) / 64;   // chunks per lane (<= kShMaxChunks)
  const bool gate_block = blockIdx.x == (unsigned)(I / 4);
  const int c = 4 * blockIdx.x + wave;
  // the lane's weight chunks of the gate row and the up row, and their scales
  u32x4 wg[kShMaxChunks], wu[kShMaxChunks];
  float sg[kShMaxChunks], su[kShMaxChunks];
  // the gate work-group: the lane's 8-value chunks l, l + 64, .. of the
  // fp16 gate row, loaded before anything waits
  constexpr int kGateChunks = 2 * kShMaxChunks;
  u32x4 gv[kGateChunks];
  if (gate_block) {
#pragma unroll
    for (int m = 0; m < kGateChunks; ++m)
      if (lane + 64 * m < H / 8) gv[m] = *reinterpret_cast<const u32x4*>(a.gate + 8 * (lane + 64 * m));
  } else {
#pragma unroll
    for (int m = 0; m < kShMaxChunks; ++m) {
      const int j = lane + 64 * m;
      if (m < per && j < nch) {
        wg[m] = *reinterpret_cast<const u32x4*>(a.gu_w + (size_t)c * H + 16 * j);
        wu[m] = *reinterpret_cast<const u32x4*>(a.gu_w + (size_t)(I + c) * H + 16 * j);
        sg[m] = a.gu_s[(size_t)c * (H / 128) + j / 8];
        su[m] = a.gu_s[(size_t)(I + c) * (H / 128) + j / 8];
      }
    }
  }
  for (int t0 = 0; t0 < T; t0 += kShTok) {
    const int nt = T - t0 < kShTok ? T - t0 : kShTok;
    __syncthreads();  // the previous tile's reads are done
    for (int i = threadIdx.x; i < nt * (H / 8); i += 256) {  // 16-byte chunks of x
      const int t = i / (H / 8), k = i % (H / 8);
      *reinterpret_cast<u32x4*>(xs + (size_t)t * H + 8 * k) =
          *reinterpret_cast<const u32x4*>(a.x + (size_t)(t0 + t) * H + 8 * k);
    }
    __syncthreads();
    if (gate_block) {
      // logit of token t: gate (fp16) . x (bf16), fp32 sum in a fixed order
      for (int t = wave; t < nt; t += 4) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < kGateChunks; ++m) {
          const int j = lane + 64 * m;
          if (j >= H / 8) break;
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + (size_t)t * H + 8 * j);
#pragma unroll
          for (int b = 0; b < 8; ++b)
            acc = __builtin_fmaf(f16_to_f32((uint16_t)(gv[m][b >> 1] >> (16 * (b & 1)))),
                                 bf16_to_f32((uint16_t)(xv[b >> 1] >> (16 * (b & 1)))), acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) a.glogit[t0 + t] = acc;
      }
      continue;
    }
    float ag[kShTok], au[kShTok];
#pragma unroll
    for (int t = 0; t < kShTok; ++t) ag[t] = au[t] = 0.f;
#pragma unroll
    for (int m = 0; m < kShMaxChunks; ++m) {
      const int j = lane + 64 * m;
      if (m >= per || j >= nch) continue;
      float g16[16], u16[16];
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        g16[b] = dq(wg[m][b >> 2], b & 3, sg[m]);
        u16[b] = dq(wu[m][b >> 2], b & 3, su[m]);
      }
#pragma unroll
      for (int t = 0; t < kShTok; ++t) {
        if (t >= nt) break;
        const u32x4* xp = reinterpret_cast<const u32x4*>(xs + (size_t)t * H + 16 * j);
        const u32x4 x0 = xp[0], x1 = xp[1];
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const uint32_t word = b < 8 ? x0[b >> 1] : x1[(b - 8) >> 1];
          const float xv = bf16_to_f32((uint16_t)(word >> (16 * (b & 1))));
          ag[t] = __builtin_fmaf(g16[b], xv, ag[t]);
          au[t] = __builtin_fmaf(u16[b], xv, au[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kShTok; ++t) {
      if (t >= nt) break;
      const float g = wave_sum(ag[t]);
      const float u = wave_sum(au[t]);
      if (lane == 0) a.h[(size_t)(t0 + t) * I + c] = silu(g) * u;
    }
  }
}

// down of the shared expert, the sigmoid gate and the add into y.
// grid.x = hidden / 8, block = 512: wave w of work-group b owns output row
// o = 8 b + w; lane l holds the 8-byte chunks l, l + 64, .. of the row. The
// token tile's h is staged in LDS (dynamic, 4 * 8 * inter bytes).
__global__ __launch_bounds__(512) void k_shared_down(SharedArgs a) {
  extern __shared__ __attribute__((aligned(16))) float hs[];  // [kShTok][inter]
  const int H = a.hidden, I = a.inter, T = a.n_tokens;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int o = 8 * blockIdx.x + wave;
  const int nch = I / 8;
  const int per = (nch + 63) / 64;
  u32x2 wd[kShMaxChunks];
  float sd[kShMaxChunks];
#pragma unroll
  for (int m = 0; m < kShMaxChunks; ++m) {
    const int j = lane + 64 * m;
    if (m < per && j < nch) {
      wd[m] = *reinterpret_cast<const u32x2*>(a.dn_w + (size_t)o * I + 8 * j);
      sd[m] = a.dn_s[(size_t)o * (I / 128) + j / 16];
    }
  }
  for (int t0 = 0; t0 < T; t0 += kShTok) {
    const int nt = T - t0 < kShTok ? T - t0 : kShTok;
    __syncthreads();
    for (int i = threadIdx.x; i < nt * I / 4; i += 512) {
      const int t = i / (I / 4), k = i % (I / 4);
      *reinterpret_cast<float4*>(hs + (size_t)t * I + 4 * k) =
          *reinterpret_cast<const float4*>(a.h + (size_t)(t0 + t) * I + 4 * k);
    }
    __syncthreads();
    float acc[kShTok];
#pragma unroll
    for (int t = 0; t < kShTok; ++t) acc[t] = 0.f;
#pragma unroll
    for (int m = 0; m < kShMaxChunks; ++m) {
      const int j = lane + 64 * m;
      if (m >= per || j >= nch) continue;
      float w8[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) w8[b] = dq(wd[m][b >> 2], b & 3, sd[m]);
#pragma unroll
      for (int t = 0; t < kShTok; ++t) {
        if (t >= nt) break;
        const float4 h0 = *reinterpret_cast<const float4*>(hs + (size_t)t * I + 8 * j);
        const float4 h1 = *reinterpret_cast<const float4*>(hs + (size_t)t * I + 8 * j + 4);
        const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[t] = __builtin_fmaf(w8[b], hv[b], acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < kShTok; ++t) {
      if (t >= nt) break;
      const float s = wave_sum(acc[t]);
      if (lane == 0) {
        const float gl = a.glogit[t0 + t];
        const float g = 1.0f / (1.0f + expf(-gl));
        float* yp = a.y + (size_t)(t0 + t) * H + o;
        *yp = a.accumulate ? *yp + g * s : g * s;
      }
    }
  }
}

hipError_t launch_shared_expert(const SharedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_gate_up, dim3((unsigned)(a.inter / 4 + 1)), dim3(256),
                     (size_t)2 * kShTok * a.hidden, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_shared_down, dim3((unsigned)(a.hidden / 8)), dim3(512),
                     (size_t)4 * kShTok * a.inter, s, a);
  return hipGetLastError();
}

}  // namespace escha
