// Router of a mixture of experts on gfx950 (TurboSparse-Mixtral; nubint.ai PowerInfer-2 review,
// section on the models it runs; citnews.com.cn PowerInfer-2 article): every token picks its
// top-K experts by the logits l_e = R[e] . x, ties going to the lower expert index, and weighs
// them by the softmax over the chosen logits.
//
// One workgroup of eight waves per token.  The routing decision never leaves the device: the workgroup copies
// the chosen experts' weight records (from the table passed by value in the kernel arguments)
// into per-slot records in the workspace, and the expert kernels that follow take their weight
// pointers from those records.
#include <hip/hip_ext.h>

#include "common.h"
#include "launch.h"

namespace ffn {

constexpr int RT_THREADS = 512;
constexpr int RT_NW = RT_THREADS / WAVE;
constexpr int RT_EPW = (MOE_MAX_E + RT_NW - 1) / RT_NW;   // experts per wave
constexpr int RT_CPL = 8;                                  // chunks per lane in flight

template <int XK>
__device__ __forceinline__ void route_token(const RouterArgs& a, int b) {
  constexpr int EPC = Kind<XK>::EPC;
  __shared__ float s_logit[MOE_MAX_E];
  __shared__ int s_ids[MOE_MAX_K];
  __shared__ float s_w[MOE_MAX_K];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int nch = a.d / EPC;
  const char* xb = static_cast<const char*>(a.x) + (size_t)b * nch * 16;
  const char* R = static_cast<const char*>(a.R);

  // logits: wave w takes experts w and w + RT_NW; lanes split the rows in 16-byte chunks, and a
  // lane's chunks of the token and of both rows are requested together (one round trip at
  // d = 4096 fp16)
  float acc[RT_EPW] = {};
  for (int c0 = 0; c0 < nch; c0 += RT_CPL * WAVE) {
    u32x4 xv[RT_CPL], w[RT_EPW][RT_CPL];
#pragma unroll
    for (int k = 0; k < RT_CPL; ++k) {
      const int c = min(c0 + lane + k * WAVE, nch - 1);
      xv[k] = ld16(xb + (size_t)c * 16);
#pragma unroll
      for (int j = 0; j < RT_EPW; ++j) {
        const int e = min(wave + j * RT_NW, a.E - 1);
        w[j][k] = ld16(R + ((size_t)e * nch + c) * 16);
      }
    }
    issue_fence();
#pragma unroll
    for (int k = 0; k < RT_CPL; ++k) {
      if (c0 + lane + k * WAVE < nch) {
#pragma unroll
        for (int j = 0; j < RT_EPW; ++j) {
          if constexpr (XK == WK_F16) acc[j] = dot8_f16(w[j][k], xv[k], acc[j]);
          else acc[j] = dot4_f32(w[j][k], xv[k], acc[j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < RT_EPW; ++j) {
    const float l = wave_sum(acc[j]);
    if (lane == 0 && wave + j * RT_NW < a.E) s_logit[wave + j * RT_NW] = l;
  }
  __syncthreads();

  if (tid == 0) {
    // top-K by repeated arg-max over the experts not yet taken (strict >: ties keep the lower
    // index), then the softmax over the chosen logits (the first is the largest)
    unsigned taken = 0u;
    for (int t = 0; t < a.K; ++t) {
      int best = -1;
      for (int e = 0; e < a.E; ++e)
        if (!(taken >> e & 1u) && (best < 0 || s_logit[e] > s_logit[best])) best = e;
      taken |= 1u << best;
      s_ids[t] = best;
    }
    const float mx = s_logit[s_ids[0]];
    float den = 0.0f;
    for (int t = 0; t < a.K; ++t) den += expf(s_logit[s_ids[t]] - mx);
    for (int t = 0; t < a.K; ++t) {
      s_w[t] = expf(s_logit[s_ids[t]] - mx) / den;
      if (a.ids_out) a.ids_out[b * a.K + t] = s_ids[t];
      if (a.w_out) a.w_out[b * a.K + t] = s_w[t];
    }
  }
  __syncthreads();

  // per-slot records: the chosen expert's pointers, then (routing weight, expert id)
  constexpr int NPTR = offsetof(ExpertW, wgt) / 8;
  static_assert(sizeof(ExpertW) == (NPTR + 1) * 8, "ExpertW: pointers, then wgt and expert");
  if (tid < a.K * (NPTR + 1)) {
    const int t = tid / (NPTR + 1), j = tid % (NPTR + 1);
    uint64_t v;
    if (j < NPTR) {
      v = reinterpret_cast<const uint64_t*>(&a.tab.e[s_ids[t]])[j];
    } else {
      v = (uint64_t)__float_as_uint(s_w[t]) | ((uint64_t)(uint32_t)s_ids[t] << 32);
    }
    reinterpret_cast<uint64_t*>(&a.slots[(size_t)b * a.K + t])[j] = v;
  }
}

// Router and predictor stage 1 of every expert in one launch.  Blocks [0, B) route token b
// (above); each further block runs eight P1 rows, a wave per row (token b, expert e, row k of
// the flattened (b, e, k) order): 16-byte chunks per lane, all loads issued before use, wave sum.
// Computing stage 1 for the experts the router is about to drop costs P1 bytes of E instead of
// top_k experts, but takes the routing decision off the path to the predictor's second stage.
template <int XK, int CPL>
__global__ __launch_bounds__(RT_THREADS) void k_route_z(RouterArgs a) {
  if ((int)blockIdx.x < a.B) {
    route_token<XK>(a, blockIdx.x);
    return;
  }
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int q = ((int)blockIdx.x - a.B) * RT_NW + wave;
  if (q >= a.B * a.E * a.rank) return;                // whole waves
  const int k = q % a.rank, e = (q / a.rank) % a.E, b = q / (a.rank * a.E);
  const int nch = a.d / Kind<XK>::EPC;
  XRegs<XK, CPL> xr;
  load_x<XK, CPL>(xr, static_cast<const char*>(a.x) + (size_t)b * nch * 16, nch, lane);
  u32x4 w[CPL];
  float sc[CPL];
  load_row<XK, CPL>(w, sc, a.tab.e[e].p1, nullptr, k, nch, lane);
  issue_fence();
  finish_x<XK, CPL>(xr, nch, lane);
  const float acc = wave_sum(row_dot<XK, CPL>(w, sc, xr));
  if (lane == 0) a.zall[q] = acc + (a.tab.e[e].c1 ? a.tab.e[e].c1[k] : 0.0f);
}

hipError_t launch_route_z(const RouterArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid(a.B + (a.B * a.E * a.rank + RT_NW - 1) / RT_NW);
#define RZ(X, C)                                                                                \
  do {                                                                                        \
    if (ev0 && ev1)                                                                           \
      hipExtLaunchKernelGGL((k_route_z<X, C>), grid, dim3(RT_THREADS), 0, st, ev0, ev1, 0, a); \
    else                                                                                      \
      hipLaunchKernelGGL((k_route_z<X, C>), grid, dim3(RT_THREADS), 0, st, a);                \
  } while (0)
#define RZ_CASE(C) \
  case C: if (a.x_f16) RZ(WK_F16, C); else RZ(WK_F32, C); break;
  switch (a.cpl) {
    RZ_CASE(1) RZ_CASE(2) RZ_CASE(3) RZ_CASE(4) RZ_CASE(6) RZ_CASE(8) RZ_CASE(12) RZ_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef RZ_CASE
#undef RZ
  return hipGetLastError();
}

}  // namespace ffn
