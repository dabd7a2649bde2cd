// escha_stream.hpp -- pieces shared by the streaming decode kernels
// (escha_kernels.hip) and the persistent layer-stack kernel
// (escha_stack.hip): loading a wave's tile-rows of codes, decoding them and
// accumulating against the rotated inputs, the quad reduction and the
// output transform. Both users go through these routines so that the two
// paths perform the same floating-point operations in the same order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "escha_device.hpp"

namespace escha {

// ------------------------------------------------------------------------
// Loading, decoding and accumulating tile-rows.
// ------------------------------------------------------------------------

// Issue the loads of NKT consecutive tile-rows (kt0, kt0+1, ..) of output
// tile nt, this lane's quarter. Nothing here waits for the data.
template <int K, int NKT>
__device__ __forceinline__ void issue_rows(const uint16_t* __restrict__ code_e, int n_nt, int kt0,
                                           int nt, int q, uint32_t (&raw)[NKT][Quarter<K>::kOwn]) {
#pragma unroll
  for (int j = 0; j < NKT; ++j) {
    const uint16_t* tq = code_e + ((size_t)(kt0 + j) * n_nt + nt) * (16 * K) + q * (4 * K);
    load_quarter<K>(tq, raw[j]);
  }
}

// Decode the loaded rows and accumulate: acc[n] += W[.., n] * x~[k] over this
// lane's 4 input rows of each tile-row. xs: the 128 rotated inputs of the
// chunk (LDS); j0: index of the first row inside the chunk.
template <int K, int NKT>
__device__ __forceinline__ void mac_rows(const uint32_t (&raw)[NKT][Quarter<K>::kOwn], int j0, int q,
                                         const float* xs, float (&acc)[16]) {
  constexpr int kOwn = Quarter<K>::kOwn;
#pragma unroll
  for (int j = 0; j < NKT; ++j) {
    uint32_t d[kOwn + 1];
#pragma unroll
    for (int i = 0; i < kOwn; ++i) d[i] = raw[j][i];
    d[kOwn] = next_quarter_dword(raw[j][0]);
    const float4 xv = *reinterpret_cast<const float4*>(xs + 16 * (j0 + j) + 4 * q);
    const float xk[4] = {xv.x, xv.y, xv.z, xv.w};
    decode_quarter<K>(d, [&](int kk, int n, h16x2 w) {
      acc[n] = __builtin_fmaf((float)w.x, xk[kk], acc[n]);
      acc[n + 8] = __builtin_fmaf((float)w.y, xk[kk], acc[n + 8]);
    });
  }
}

// Sum the four quarter-lanes' column sums (DPP inside each quad; all four
// lanes get the same bits). Lane q then owns output columns 4q..4q+3 of its
// tile, i.e. outputs 4*lane .. 4*lane+3 of the wave's 256.
__device__ __forceinline__ float4 quad_reduce_pick(float (&acc)[16], int q) {
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    acc[n] += xor_lane<1>(acc[n]);
    acc[n] += xor_lane<2>(acc[n]);
  }
  float4 r;
  r.x = q == 0 ? acc[0] : q == 1 ? acc[4] : q == 2 ? acc[8] : acc[12];
  r.y = q == 0 ? acc[1] : q == 1 ? acc[5] : q == 2 ? acc[9] : acc[13];
  r.z = q == 0 ? acc[2] : q == 1 ? acc[6] : q == 2 ? acc[10] : acc[14];
  r.w = q == 0 ? acc[3] : q == 1 ? acc[7] : q == 2 ? acc[11] : acc[15];
  return r;
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Agent-scope (device-coherent) 32-bit accesses: the store writes through to
// the point where every compute unit of the device sees it, the load reads
// from there. Used for data that work-groups of one launch exchange.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Output transform of one 256-output group held in LDS (zs, in output
// order): waves 0 and 1 each take one 128-block, apply H_n, multiply by
// rout (and the weight wt) and store. out points at the group's first
// output; ro0/ro1 are rout at this lane's two outputs of the wave's block.
// AGENT: store with agent-scope stores (same values).
template <bool AGENT = false>
__device__ __forceinline__ void transform_store_rv(const float* zs, float ro0, float ro1, float wt,
                                                   float* __restrict__ out, int wave, int lane) {
  if (wave < 2) {
    float z0 = zs[128 * wave + lane];
    float z1 = zs[128 * wave + lane + 64];
    fwht128(z0, z1);
    const float o0 = z0 * kInvSqrt128 * ro0 * wt;
    const float o1 = z1 * kInvSqrt128 * ro1 * wt;
    if constexpr (AGENT) {
      st_agent(out + 128 * wave + lane, o0);
      st_agent(out + 128 * wave + lane + 64, o1);
    } else {
      out[128 * wave + lane] = o0;
      out[128 * wave + lane + 64] = o1;
    }
  }
}

__device__ __forceinline__ void transform_store(const float* zs, const uint16_t* __restrict__ rout_g,
                                                float wt, float* __restrict__ out, int wave,
                                                int lane) {
  if (wave < 2) {
    const uint16_t* ro = rout_g + 128 * wave;
    transform_store_rv(zs, f16_to_f32(ro[lane]), f16_to_f32(ro[lane + 64]), wt, out, wave, lane);
  }
}

// Decode ahead of the activations: the lane's 64 weights of each loaded
// tile-row, kept as packed pairs (index 8*kk + n holds columns n and n+8 of
// input row 4q+kk).
template <int K, int NKT>
__device__ __forceinline__ void decode_rows(const uint32_t (&raw)[NKT][Quarter<K>::kOwn],
                                            h16x2 (&wv)[NKT][32]) {
  constexpr int kOwn = Quarter<K>::kOwn;
#pragma unroll
  for (int j = 0; j < NKT; ++j) {
    uint32_t d[kOwn + 1];
#pragma unroll
    for (int i = 0; i < kOwn; ++i) d[i] = raw[j][i];
    d[kOwn] = next_quarter_dword(raw[j][0]);
    decode_quarter<K>(d, [&](int kk, int n, h16x2 w) { wv[j][8 * kk + n] = w; });
  }
}

// Accumulate decoded rows against the rotated inputs: the same multiply-adds
// in the same order as mac_rows, so both give identical sums. jrow: index of
// the tile-row inside the 128-input chunk.
__device__ __forceinline__ void mac_decoded_row(const h16x2 (&wr)[32], int jrow, int q,
                                                const float* xs, float (&acc)[16]) {
  const float4 xv = *reinterpret_cast<const float4*>(xs + 16 * jrow + 4 * q);
  const float xk[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const h16x2 w = wr[8 * kk + n];
      acc[n] = __builtin_fmaf((float)w.x, xk[kk], acc[n]);
      acc[n + 8] = __builtin_fmaf((float)w.y, xk[kk], acc[n + 8]);
    }
  }
}

}  // namespace escha
