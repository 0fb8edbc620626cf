// Router of a mixture of experts on gfx950 (TurboSparse-Mixtral; nubint.ai PowerInfer-2 review,
// section on the models it runs; citnews.com.cn PowerInfer-2 article): every token picks its
// top-K experts by the logits l_e = R[e] . x, ties going to the lower expert index, and weighs
// them by the softmax over the chosen logits.
//
// One workgroup of four waves per token.  The routing decision never leaves the device: the
// workgroup copies the chosen experts' weight records (from the table passed by value in the
// kernel arguments) into per-slot records in the workspace, and the expert kernels that follow
// take their weight pointers from those records.
#include <hip/hip_ext.h>

#include "common.h"
#include "launch.h"

namespace ffn {

constexpr int RT_THREADS = 256;
constexpr int RT_NW = RT_THREADS / WAVE;

// Experts per wave of the logits (a template parameter: 1, 2 or 4 for up to 4, 8 or 16
// experts), so that every row load is unconditional: a load under a branch makes the compiler
// wait for the loads before it where the paths join, and the token's round trip would become
// one per expert.
constexpr int rt_epw(int E) { return E <= RT_NW ? 1 : E <= 2 * RT_NW ? 2 : 4; }
static_assert(MOE_MAX_E <= 4 * RT_NW, "four experts per wave at most");

// Logits of token b over every expert (into s_logit) and its top-K (repeated arg-max over the
// experts not yet taken, strict >: ties keep the lower index) into ids[0, K) of every thread.
// xr holds the token's chunks as load_x requested them (lane l: chunks l, l + 64, ...; they may
// still be in flight).  Wave w takes experts w, w + RT_NW, ... (EPW of them; a slot past the last
// expert reads the last expert's row again and is not used); a lane requests its chunks of all its
// rows at once, so the token and the rows take one round trip.  Every workgroup that needs the
// decision runs this same code on the same data, so all of them reach the same experts.
template <int XK, int CPL, int EPW>
__device__ __forceinline__ void route_decide(const RouterArgs& a, const XRegs<XK, CPL>& xr,
                                             float* s_logit, int (&ids)[MOE_MAX_K]) {
  constexpr int EPC = Kind<XK>::EPC;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int nch = a.d / EPC;
  const char* R = static_cast<const char*>(a.R);
  u32x4 w[EPW][CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = min(lane + k * WAVE, nch - 1);
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
      const int e = min(wave + j * RT_NW, a.E - 1);
      w[j][k] = ld16(R + ((size_t)e * nch + c) * 16);
    }
  }
  issue_fence();
  float acc[EPW] = {};
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    if (lane + k * WAVE < nch) {
#pragma unroll
      for (int j = 0; j < EPW; ++j) {
        if constexpr (XK == WK_F16) acc[j] = dot8_f16(w[j][k], xr.v[k][0], acc[j]);
        else acc[j] = dot4_f32(w[j][k], xr.v[k][0], acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < EPW; ++j) {
    const float l = wave_sum(acc[j]);
    if (lane == 0 && wave + j * RT_NW < a.E) s_logit[wave + j * RT_NW] = l;
  }
  __syncthreads();
  // every thread takes the top-K from the E logits itself (the same comparisons everywhere): no
  // serial step on one thread and no second barrier
  float lg[MOE_MAX_E];
#pragma unroll
  for (int e = 0; e < MOE_MAX_E; ++e) lg[e] = e < a.E ? s_logit[e] : 0.0f;
  unsigned taken = 0u;
#pragma unroll
  for (int t = 0; t < MOE_MAX_K; ++t) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int e = 0; e < MOE_MAX_E; ++e)
      if (e < a.E && !(taken >> e & 1u) && (bi < 0 || lg[e] > bv)) {
        bv = lg[e];
        bi = e;
      }
    if (t < a.K) {
      taken |= 1u << bi;
      ids[t] = bi;
    }
  }
}

template <int XK, int CPL, int EPW>
__device__ __forceinline__ void route_token(const RouterArgs& a, int b) {
  __shared__ float s_logit[MOE_MAX_E];
  __shared__ int s_ids[MOE_MAX_K];
  __shared__ float s_w[MOE_MAX_K];
  const int tid = threadIdx.x;
  const int nch = a.d / Kind<XK>::EPC;
  XRegs<XK, CPL> xr;
  load_x<XK, CPL>(xr, static_cast<const char*>(a.x) + (size_t)b * nch * 16, nch, tid & (WAVE - 1));
  int ids[MOE_MAX_K];
  route_decide<XK, CPL, EPW>(a, xr, s_logit, ids);
  if (tid == 0) {
    // the softmax over the chosen logits (the first is the largest)
    const float mx = s_logit[ids[0]];
    float den = 0.0f;
#pragma unroll
    for (int t = 0; t < MOE_MAX_K; ++t)
      if (t < a.K) den += expf(s_logit[ids[t]] - mx);
#pragma unroll
    for (int t = 0; t < MOE_MAX_K; ++t) {
      if (t < a.K) {
        s_ids[t] = ids[t];
        s_w[t] = expf(s_logit[ids[t]] - mx) / den;
        if (a.ids_out) a.ids_out[b * a.K + t] = ids[t];
        if (a.w_out) a.w_out[b * a.K + t] = s_w[t];
      }
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

// Router and predictor stage 1 of the chosen experts in one launch.  Blocks [0, B) route token b
// (above) and write its slot records; each further block runs four P1 rows of one token's chosen
// experts, a wave per row (rows in (token b, slot t, row k) order; rank is a multiple of eight, so
// a block's rows share the token and the slot).  Four waves per block rather than eight: the
// chosen experts' P1 rows spread over twice as many CUs.  Such a block first reaches the token's routing
// decision itself (the same code as the routing block, so the same experts), then reads the P1
// rows of the experts chosen and no others: 16-byte chunks per lane, all loads issued before use,
// wave sum.  The rows land at zall[(b * E + e) * rank + k], where the stage-2 kernels look for
// the slot's expert e.
template <int XK, int CPL, int EPW>
__global__ __launch_bounds__(RT_THREADS) void k_route_z(RouterArgs a) {
  if ((int)blockIdx.x < a.B) {
    route_token<XK, CPL, EPW>(a, blockIdx.x);
    return;
  }
  __shared__ float s_logit[MOE_MAX_E];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int q = ((int)blockIdx.x - a.B) * RT_NW + wave;
  const int b = (((int)blockIdx.x - a.B) * RT_NW) / (a.K * a.rank);
  const int nch = a.d / Kind<XK>::EPC;
  XRegs<XK, CPL> xr;
  load_x<XK, CPL>(xr, static_cast<const char*>(a.x) + (size_t)b * nch * 16, nch, lane);
  int ids[MOE_MAX_K];
  route_decide<XK, CPL, EPW>(a, xr, s_logit, ids);
  const int k = q % a.rank, t = (q / a.rank) % a.K;
  int e = ids[0];
#pragma unroll
  for (int j = 1; j < MOE_MAX_K; ++j) e = t == j ? ids[j] : e;
  e = __builtin_amdgcn_readfirstlane(e);
  u32x4 w[CPL];
  float sc[CPL];
  load_row<XK, CPL>(w, sc, a.tab.e[e].p1, nullptr, k, nch, lane);
  issue_fence();
  finish_x<XK, CPL>(xr, nch, lane);
  const float acc = wave_sum(row_dot<XK, CPL>(w, sc, xr));
  if (lane == 0)
    a.zall[((size_t)b * a.E + e) * a.rank + k] = acc + (a.tab.e[e].c1 ? a.tab.e[e].c1[k] : 0.0f);
}

template <int XK, int CPL>
static void launch_route_z_t(const RouterArgs& a, dim3 grid, hipStream_t st, hipEvent_t ev0,
                             hipEvent_t ev1) {
  const int epw = rt_epw(a.E);
  auto kern = epw == 1 ? k_route_z<XK, CPL, 1> : epw == 2 ? k_route_z<XK, CPL, 2>
                                                          : k_route_z<XK, CPL, 4>;
  if (ev0 && ev1)
    hipExtLaunchKernelGGL(kern, grid, dim3(RT_THREADS), 0, st, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL(kern, grid, dim3(RT_THREADS), 0, st, a);
}

hipError_t launch_route_z(const RouterArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.rank % RT_NW) return hipErrorInvalidValue;   // a block's rows share one token
  if (a.E < 1 || a.E > MOE_MAX_E) return hipErrorInvalidValue;
  const dim3 grid(a.B + a.B * a.K * a.rank / RT_NW);
#define RZ_CASE(C)                                                              \
  case C:                                                                       \
    if (a.x_f16) launch_route_z_t<WK_F16, C>(a, grid, st, ev0, ev1);            \
    else launch_route_z_t<WK_F32, C>(a, grid, st, ev0, ev1);                    \
    break;
  switch (a.cpl) {
    RZ_CASE(1) RZ_CASE(2) RZ_CASE(3) RZ_CASE(4) RZ_CASE(6) RZ_CASE(8) RZ_CASE(12) RZ_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef RZ_CASE
  return hipGetLastError();
}

}  // namespace ffn
