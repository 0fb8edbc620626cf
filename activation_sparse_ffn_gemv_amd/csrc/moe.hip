// Router of a mixture of experts on gfx950 (TurboSparse-Mixtral; nubint.ai PowerInfer-2 review,
// section on the models it runs; citnews.com.cn PowerInfer-2 article): every token picks its
// top-K experts by the logits l_e = R[e] . x, ties going to the lower expert index, and weighs
// them by the softmax over the chosen logits.
//
// One workgroup per token.  The routing decision never leaves the device: the workgroup copies
// the chosen experts' weight records (from the table passed by value in the kernel arguments)
// into per-slot records in the workspace, and the expert kernels that follow take their weight
// pointers from those records.
#include "common.h"
#include "launch.h"

namespace ffn {

constexpr int RT_THREADS = 256;
constexpr int RT_NW = RT_THREADS / WAVE;

template <int XK>
__global__ __launch_bounds__(RT_THREADS) void k_router(RouterArgs a) {
  constexpr int EPC = Kind<XK>::EPC;
  __shared__ float s_logit[MOE_MAX_E];
  __shared__ int s_ids[MOE_MAX_K];
  __shared__ float s_w[MOE_MAX_K];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int nch = a.d / EPC;
  const char* xb = static_cast<const char*>(a.x) + (size_t)b * nch * 16;
  const char* R = static_cast<const char*>(a.R);

  // logits: wave w takes experts w, w + RT_NW, ...; lanes split the row in 16-byte chunks
  for (int e = wave; e < a.E; e += RT_NW) {
    float acc = 0.0f;
#pragma unroll 4
    for (int c = lane; c < nch; c += WAVE) {
      const u32x4 w = ld16(R + ((size_t)e * nch + c) * 16);
      const u32x4 xv = ld16(xb + (size_t)c * 16);
      if constexpr (XK == WK_F16) acc = dot8_f16(w, xv, acc);
      else acc = dot4_f32(w, xv, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) s_logit[e] = acc;
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

hipError_t launch_router(const RouterArgs& a, int B, hipStream_t st) {
  if (a.x_f16)
    hipLaunchKernelGGL(k_router<WK_F16>, dim3(B), dim3(RT_THREADS), 0, st, a);
  else
    hipLaunchKernelGGL(k_router<WK_F32>, dim3(B), dim3(RT_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace ffn
