// escha_stack.hip -- decode of a whole stack of MoE layers in one persistent
// launch (small batches, the token-by-token generation case).
//
// The work of every layer is the same set of tasks as the streaming kernels
// (escha_kernels.hip) perform, in the same arithmetic:
//   gate_up task (pair p, 128-input chunk c, 256-output group g): the
//     rotated inputs of the chunk (RMSNorm of the previous layer's output
//     for layers after the first), the decode of 8 tile-rows x 16 tiles and
//     the output transform of the partial sums;
//   down task (p, 128-channel chunk c of the intermediate, group g): h =
//     SiLU(gate) * up from gate_up's partials, its rotation, the decode and
//     the transform weighted by the router probability;
//   combine (token t, group g): the fixed-order sum of the token's down
//     partials, done by whichever down task of (t, g) finishes last.
// Tasks are numbered layer by layer (gate_up before down, pair-major) and
// handed out through one atomic ticket counter. A work-group claims a task,
// issues the loads of its codes and decodes them into registers -- none of
// which depends on earlier tasks -- and only then waits for the counters of
// the tasks whose outputs it reads, so the decode of later work overlaps
// the waits of the dependency chain. Past the wait the group claims its
// next task and runs at raised issue priority until the task ends. Every
// dependency of a task has a smaller number, and a number is only ever
// claimed by a running work-group, so the smallest unfinished task can
// always proceed: the scheme needs no co-residency guarantee. Each wait is
// bounded all the same: when one gives up, the kernel sets an error word
// and every work-group leaves at its next wait.
//
// Cross-work-group data is written with agent-scope (device-coherent)
// stores, and every wave waits for its stores to complete before the
// group's counter increment; no cache needs a write-back. Two kinds of
// buffers, two ways of reading:
//  - the partial sums (gate_up's and down's) are reused from layer to
//    layer, which the dependency chain makes safe (a task that overwrites
//    one waits, directly or transitively, for every task of the previous
//    layer that reads it); they are read with agent-scope loads, since a
//    cache may still hold the previous layer's lines;
//  - each layer's output and its sums of squares, which every gate_up task
//    of the next layer reads, have an address of their own (256-byte
//    aligned) written once per launch: no cache can hold an older copy
//    (caches start clean at a kernel launch, and nothing reads these lines
//    before their counter is complete), so plain loads, served from the
//    caches after the first miss, are exact.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "escha_device.hpp"
#include "escha_launch.hpp"
#include "escha_stream.hpp"

namespace escha {

namespace {

constexpr int kSpinLimit = 1 << 21;  // polls before a wait gives up
constexpr int kGroupsPerCu = 2;      // persistent work-groups per compute unit

__device__ __forceinline__ int ld_relaxed(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_relaxed(int32_t* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's stores have completed (with agent-scope stores:
// until they are visible device-wide); also a compiler barrier.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Poll until *ctr >= target. False when the wait gave up (and raised the
// error word) or another work-group has raised it.
__device__ bool wait_count(const int32_t* ctr, int target, int32_t* err) {
  for (int it = 0;; ++it) {
    if (ld_relaxed(ctr) >= target) return true;
    if ((it & 63) == 63) {
      if (ld_relaxed(err)) return false;
      if (it >= kSpinLimit) {
        st_relaxed(err, 1);
        return false;
      }
    }
    // back off: a task claimed far ahead of the chain polls less often
    if (it < 8)
      __builtin_amdgcn_s_sleep(1);
    else if (it < 32)
      __builtin_amdgcn_s_sleep(4);
    else
      __builtin_amdgcn_s_sleep(12);
  }
}

// Work-group wait: thread 0 polls, everyone learns the outcome after the
// barrier; the group's reads of the producers' data (agent-scope loads) all
// come after it. Must be reached by all threads of the group.
__device__ __forceinline__ bool group_wait(const int32_t* ctr, int target, int32_t* err, int* sh_ok) {
  if (threadIdx.x == 0) *sh_ok = wait_count(ctr, target, err) ? 1 : 0;
  __syncthreads();
  return *sh_ok != 0;
}

// Every wave waits for its agent-scope stores to complete, then thread 0
// counts the task as done. Returns the counter's previous value (to thread
// 0; other threads get 0).
__device__ __forceinline__ int group_signal(int32_t* ctr) {
  stores_done();
  __syncthreads();
  int old = 0;
  if (threadIdx.x == 0) old = add_relaxed(ctr, 1);
  return old;
}

// Sum of p[i * stride] for i = 0 .. n-1, added in index order from 0.f (the
// order of the streaming kernels' loops); the loads of each batch of 16 are
// issued back to back before the first is used.
__device__ __forceinline__ float ordered_sum_agent(const float* p, size_t stride, int n) {
  float s = 0.f;
  for (int b0 = 0; b0 < n; b0 += 16) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = b0 + i < n ? ld_agent(p + (size_t)(b0 + i) * stride) : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (b0 + i < n) s += v[i];
  }
  return s;
}

// Zero outputs 4*lane .. 4*lane+3 of a 256-output group.
__device__ __forceinline__ void zero4_agent(float* out, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) st_agent(out + 4 * lane + i, 0.f);
}

// Past its wait, a task is on the dependency chain: claim the group's next
// task now (its number is needed only when this one ends; claiming earlier
// would tie a later task to this one's wait) and raise the waves' issue
// priority above the groups that are still decoding ahead.
__device__ __forceinline__ void claim_next(int32_t* ticket, int& next) {
  if (threadIdx.x == 0) next = add_relaxed(ticket, 1);
  __builtin_amdgcn_s_setprio(3);
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

// group_signal on each of the kYRep copies of a counter (waiters poll one
// copy each, which spreads the polling over kYRep memory locations).
__device__ __forceinline__ void group_signal_rep(int32_t* ctr0) {
  stores_done();
  __syncthreads();
  if (threadIdx.x < kYRep) add_relaxed(ctr0 + threadIdx.x * kPollStride, 1);
}

struct Lds {
  float xs[128] __attribute__((aligned(16)));
  float zs[256] __attribute__((aligned(16)));
  float4 red[8][64];
  int tk, ok, go, last;
};

}  // namespace

template <int KG, int KD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_stack_decode(
    const StackArgs a) {
  constexpr int kOwnG = Quarter<KG>::kOwn;
  constexpr int kOwnD = Quarter<KD>::kOwn;
  __shared__ Lds sh;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int q = lane & 3;
  const int H = a.hidden, I = a.inter, k = a.top_k, T = a.n_tokens;
  const int P = T * k;
  const int ncg = H / 128, ngg = (2 * I) / 256;  // gate_up chunks / groups
  const int ncd = I / 128, ngd = H / 256;        // down chunks / groups
  const int n_gu = P * ncg * ngg;
  const int per_layer = n_gu + P * ncd * ngd;

  if (tid == 0) sh.tk = add_relaxed(a.ticket, 1);
  __syncthreads();
  int tk = sh.tk;
  while (tk < a.n_tasks) {
    int next = 0;

    const int l = tk / per_layer;
    int r = tk - l * per_layer;
    const StackLayer& Ly = a.layer[l];
    if (r < n_gu) {
      // ---------------------------------------------------------- gate_up
      const int p = r / (ncg * ngg);
      r -= p * (ncg * ngg);
      const int c = r / ngg;
      const int g = r - c * ngg;
      const int t = p / k;
      const int e = a.ids[(size_t)l * P + p];
      const bool valid = e >= 0 && e < a.n_experts;
      const int n_nt = (2 * I) / 16;
      const int nt = g * 16 + (lane >> 2);
      float* out = a.gu_part + ((size_t)p * ncg + c) * (2 * I) + g * 256;

      // an out-of-range id is decoded as expert 0 and its result discarded,
      // which keeps the register state the same on every path
      const int es = valid ? e : 0;
      uint32_t raw[2][kOwnG];
      h16x2 wv[2][32];
      const uint16_t* code_e = Ly.gu_code + (size_t)es * (size_t)ncg * 8 * n_nt * (16 * KG);
      issue_rows<KG, 2>(code_e, n_nt, 8 * c + 2 * wave, nt, q, raw);
      const uint16_t* rr = Ly.gu_rin + (size_t)es * H + c * 128;
      const float rin0 = f16_to_f32(rr[lane]);
      const float rin1 = f16_to_f32(rr[lane + 64]);
      const uint16_t* ro = Ly.gu_rout + (size_t)es * (2 * I) + g * 256 + 128 * (wave & 1);
      const float ro0 = f16_to_f32(ro[lane]);
      const float ro1 = f16_to_f32(ro[lane + 64]);
      decode_rows<KG, 2>(raw, wv);
      pin_decoded(wv);
      if (l > 0 &&
          !group_wait(a.y_done + (((size_t)(l - 1) * T + t) * kYRep + blockIdx.x % kYRep) * kPollStride,
                      ngd, a.error, &sh.ok))
        return;
      claim_next(a.ticket, next);

      if (wave == 0) {
        float x0, x1;
        uint16_t* xo = nullptr;
        if (a.x_chain && g == 0 && p % k == 0)
          xo = a.x_chain + ((size_t)l * T + t) * H + c * 128;
        if (l == 0) {
          const uint16_t* xr = a.x0 + (size_t)t * H + c * 128;
          const uint16_t b0 = xr[lane], b1 = xr[lane + 64];
          if (xo) {
            xo[lane] = b0;
            xo[lane + 64] = b1;
          }
          x0 = bf16_to_f32(b0);
          x1 = bf16_to_f32(b1);
        } else {
          // RMSNorm of the previous layer's output row, rounded to bf16
          // written once per launch at this address, so plain (cached) loads
          // see the final values
          const float* yr = a.y_layers + ((size_t)(l - 1) * T + t) * H + c * 128;
          const float* ss = a.ss_layers + (size_t)(l - 1) * a.ss_stride + (size_t)t * a.ss_tok;
          const float y0 = yr[lane];
          const float y1 = yr[lane + 64];
          float tot = 0.f;
          for (int b = 0; b < ncg; ++b) tot += ss[b];
          const float inv = 1.0f / sqrtf(tot / (float)H + a.eps);
          const uint16_t b0 = f32_to_bf16_rne(y0 * inv);
          const uint16_t b1 = f32_to_bf16_rne(y1 * inv);
          if (xo) {
            xo[lane] = b0;
            xo[lane + 64] = b1;
          }
          x0 = bf16_to_f32(b0);
          x1 = bf16_to_f32(b1);
        }
        if (valid) {
          float v0 = x0 * rin0;
          float v1 = x1 * rin1;
          fwht128(v0, v1);
          sh.xs[lane] = v0 * kInvSqrt128;
          sh.xs[lane + 64] = v1 * kInvSqrt128;
        } else {  // an out-of-range expert id contributes nothing
          zero4_agent(out, lane);
        }
      }
      if (valid) {  // uniform over the group
        __syncthreads();
        float acc[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[n] = 0.f;
        mac_decoded_row(wv[0], 2 * wave, q, sh.xs, acc);
        mac_decoded_row(wv[1], 2 * wave + 1, q, sh.xs, acc);
        sh.red[wave][lane] = quad_reduce_pick(acc, q);
        __syncthreads();
        if (wave == 0) {
          float4 s = sh.red[0][lane];
          s = f4add(s, sh.red[1][lane]);
          s = f4add(s, sh.red[2][lane]);
          s = f4add(s, sh.red[3][lane]);
          reinterpret_cast<float4*>(sh.zs)[lane] = s;
        }
        __syncthreads();
        transform_store_rv<true>(sh.zs, ro0, ro1, 1.0f, out, wave, lane);
      }
      group_signal(a.gu_done + ((size_t)l * P + p) * kPollStride);
    } else {
      // ------------------------------------------------------------- down
      r -= n_gu;
      const int p = r / (ncd * ngd);
      r -= p * (ncd * ngd);
      const int c = r / ngd;
      const int g = r - c * ngd;
      const int t = p / k;
      const int e = a.ids[(size_t)l * P + p];
      const bool valid = e >= 0 && e < a.n_experts;
      const int n_nt = H / 16;
      const int nt = g * 16 + (lane >> 2);
      float* out = a.dn_part + ((size_t)p * ncd + c) * H + g * 256;

      const int es = valid ? e : 0;
      uint32_t raw[2][kOwnD];
      h16x2 wv[2][32];
      const uint16_t* code_e = Ly.dn_code + (size_t)es * (size_t)ncd * 8 * n_nt * (16 * KD);
      issue_rows<KD, 2>(code_e, n_nt, 8 * c + 2 * wave, nt, q, raw);
      const uint16_t* rr = Ly.dn_rin + (size_t)es * I + c * 128;
      const float rin0 = f16_to_f32(rr[lane]);
      const float rin1 = f16_to_f32(rr[lane + 64]);
      const uint16_t* ro = Ly.dn_rout + (size_t)es * H + g * 256 + 128 * (wave & 1);
      const float ro0 = f16_to_f32(ro[lane]);
      const float ro1 = f16_to_f32(ro[lane + 64]);
      const float wt = a.w[(size_t)l * P + p];
      decode_rows<KD, 2>(raw, wv);
      pin_decoded(wv);
      if (!group_wait(a.gu_done + ((size_t)l * P + p) * kPollStride, ncg * ngg, a.error, &sh.ok))
        return;
      claim_next(a.ticket, next);

      // gate and up sums of this chunk's 128 channels: thread i sums value i
      // (gate channel i, or up channel i-128) over gate_up's chunks
      if (valid) {
        const int col = tid < 128 ? 128 * c + tid : I + 128 * c + (tid - 128);
        sh.zs[tid] = ordered_sum_agent(a.gu_part + (size_t)p * ncg * (2 * I) + col, 2 * I, ncg);
      }
      __syncthreads();
      if (wave == 0) {
        int skip = 1;
        if (valid) {
          const float h0 = silu(sh.zs[lane]) * sh.zs[128 + lane];
          const float h1 = silu(sh.zs[lane + 64]) * sh.zs[192 + lane];
          skip = __ballot((h0 != 0.f) || (h1 != 0.f)) == 0;
          float v0 = h0 * rin0;
          float v1 = h1 * rin1;
          fwht128(v0, v1);
          sh.xs[lane] = v0 * kInvSqrt128;
          sh.xs[lane + 64] = v1 * kInvSqrt128;
        }
        // an invalid expert, or a chunk whose h is all zero, contributes zero
        if (skip) zero4_agent(out, lane);
        if (lane == 0) sh.go = skip ? 0 : 1;
      }
      __syncthreads();
      if (sh.go) {  // uniform over the group
        float acc0[16], acc1[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) acc0[n] = acc1[n] = 0.f;
        mac_decoded_row(wv[0], 2 * wave, q, sh.xs, acc0);
        mac_decoded_row(wv[1], 2 * wave + 1, q, sh.xs, acc1);
        sh.red[2 * wave][lane] = quad_reduce_pick(acc0, q);
        sh.red[2 * wave + 1][lane] = quad_reduce_pick(acc1, q);
        __syncthreads();
        if (wave == 0) {
          float4 s = sh.red[0][lane];
#pragma unroll
          for (int w = 1; w < 8; ++w) s = f4add(s, sh.red[w][lane]);
          reinterpret_cast<float4*>(sh.zs)[lane] = s;
        }
        __syncthreads();
        transform_store_rv<true>(sh.zs, ro0, ro1, wt, out, wave, lane);
      }
      const int n_rows = k * ncd;  // down partial rows of one token
      const int old = group_signal(a.c_done + (((size_t)l * T + t) * ngd + g) * kCtrStride);
      if (tid == 0) sh.last = old == n_rows - 1;
      __syncthreads();
      if (sh.last) {
        // ------------------------------------------ combine of (t, group g)
        // thread i sums output column 256g + i over the token's rows in order
        const float* pp = a.dn_part + (size_t)t * n_rows * H + 256 * g + tid;
        const float col_sum = ordered_sum_agent(pp, H, n_rows);
        float* y = (l == a.n_layers - 1 ? a.y_last : a.y_layers + (size_t)l * T * H) +
                   (size_t)t * H + 256 * g;
        st_agent(y + tid, col_sum);
        sh.zs[tid] = col_sum;
        __syncthreads();
        if (wave < 2 && l < a.n_layers - 1) {  // block 2g + wave: its sum of squares
          const float s0 = sh.zs[128 * wave + lane];
          const float s1 = sh.zs[128 * wave + lane + 64];
          const float sq = wave_sum(__builtin_fmaf(s0, s0, s1 * s1));
          if (lane == 0)
            st_agent(a.ss_layers + (size_t)l * a.ss_stride + (size_t)t * a.ss_tok + 2 * g + wave, sq);
        }
        group_signal_rep(a.y_done + ((size_t)l * T + t) * kYRep * kPollStride);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (tid == 0) sh.tk = next;
    __syncthreads();
    tk = sh.tk;
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(int32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

namespace {

template <int KG, int KD>
hipError_t resident(int* groups) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stack_decode<KG, KD>, 256, 0);
  if (e != hipSuccess) return e;
  // two groups per compute unit measured fastest at batch 1 (more groups
  // decode further ahead but poll more and lengthen every memory round trip)
  if (per_cu > kGroupsPerCu) per_cu = kGroupsPerCu;
  *groups = cus * per_cu;
  return hipSuccess;
}

}  // namespace

hipError_t stack_resident_groups(int k_gu, int k_dn, int* groups) {
  if (k_gu == 2 && k_dn == 3) return resident<2, 3>(groups);
  if (k_gu == 2 && k_dn == 2) return resident<2, 2>(groups);
  if (k_gu == 3 && k_dn == 3) return resident<3, 3>(groups);
  if (k_gu == 3 && k_dn == 2) return resident<3, 2>(groups);
  return hipErrorInvalidValue;
}

hipError_t launch_fill_zero(int32_t* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_stack_decode(const StackArgs& a, int k_gu, int k_dn, int groups, hipStream_t s) {
  const dim3 grid(groups), block(256);
  if (k_gu == 2 && k_dn == 3)
    hipLaunchKernelGGL((k_stack_decode<2, 3>), grid, block, 0, s, a);
  else if (k_gu == 2 && k_dn == 2)
    hipLaunchKernelGGL((k_stack_decode<2, 2>), grid, block, 0, s, a);
  else if (k_gu == 3 && k_dn == 3)
    hipLaunchKernelGGL((k_stack_decode<3, 3>), grid, block, 0, s, a);
  else if (k_gu == 3 && k_dn == 2)
    hipLaunchKernelGGL((k_stack_decode<3, 2>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace escha
