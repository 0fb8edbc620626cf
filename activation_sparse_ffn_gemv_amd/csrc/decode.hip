// Batch-1 decode path of the activation-sparse FFN on gfx950.
//
// Per token and layer, three launches on the caller's stream:
//   k_pred_z     z = P1 x + c1                                   (predictor stage 1)
//   k_main       per neuron chunk: s = P2 z + c2, threshold, ballot compaction of the chunk's
//                active neurons, gathered up/gate rows -> activation -> h, and the transposed
//                down rows scaled by h, reduced across the workgroup's waves in LDS into one
//                fp32 partial of y per chunk
//   k_reduce     y = b_down + sum over chunks of the partials, in a fixed order
// Nothing is accumulated with global atomics, so y is bit-reproducible run to run.
//
// The method (PowerInfer, unite.ai: "Adaptive sparse predictor", "Neuron-aware operator";
// nearauto.com Fig. 8; citnews.com.cn "Dynamic neuron cache") computes only the predicted
// neurons' rows of up / gate and of the transposed down projection.
#include <hip/hip_ext.h>

#include "common.h"
#include "launch.h"

namespace ffn {

// ---------------------------------------------------------------------------------------------
// Token slice held in registers: lane `l` owns 16-byte chunks l, l+64, l+128, ... of a row.
template <int WK, int CPL>
struct XRegs {
  u32x4 v[CPL][Kind<WK>::XW];
};

template <int WK, int CPL>
__device__ __forceinline__ void load_x(XRegs<WK, CPL>& xr, const void* x, int nch, int lane) {
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    int c = lane + k * WAVE;
#pragma unroll
    for (int q = 0; q < Kind<WK>::XW; ++q) {
      if (c < nch) {
        // fp32 / fp16 tokens: 16 bytes per chunk.  int4 rows: 32 fp16 token values per chunk.
        xr.v[k][q] = ld16(static_cast<const char*>(x) + (size_t)c * 16 * Kind<WK>::XW + q * 16);
      } else {
        xr.v[k][q] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (WK == WK_I4) i4_perm_x(xr.v[k]);
  }
}

// Dot product of one weight row with the register-resident token (partial per lane).
template <int WK, int CPL>
__device__ __forceinline__ float row_dot(const u32x4 (&w)[CPL], const float (&sc)[CPL],
                                         const XRegs<WK, CPL>& xr) {
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    if constexpr (WK == WK_F32) acc = dot4_f32(w[k], xr.v[k][0], acc);
    else if constexpr (WK == WK_F16) acc = dot8_f16(w[k], xr.v[k][0], acc);
    else acc = dot32_i4(w[k], xr.v[k], sc[k], acc);
  }
  return acc;
}

template <int WK, int CPL>
__device__ __forceinline__ void load_row(u32x4 (&w)[CPL], float (&sc)[CPL], const void* base,
                                         const void* scales, size_t row, int nch, int lane) {
  const char* rp = static_cast<const char*>(base) + row * (size_t)nch * 16;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    int c = lane + k * WAVE;
    w[k] = c < nch ? ld16(rp + (size_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
    if constexpr (WK == WK_I4) {
      const _Float16* sp = static_cast<const _Float16*>(scales) + row * (size_t)nch;
      sc[k] = c < nch ? (float)sp[c] : 0.0f;
    } else {
      sc[k] = 0.0f;
    }
  }
}

// acc[k][e] += h * w (row chunk k, element e); int4 elements are decoded exactly (scale * q).
template <int WK, int CPL>
__device__ __forceinline__ void axpy_row(float (&acc)[CPL][Kind<WK>::EPC], float h,
                                         const u32x4 (&w)[CPL], const float (&sc)[CPL]) {
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    if constexpr (WK == WK_F32) {
      f32x4 a = __builtin_bit_cast(f32x4, w[k]);
      acc[k][0] = __builtin_fmaf(h, a.x, acc[k][0]);
      acc[k][1] = __builtin_fmaf(h, a.y, acc[k][1]);
      acc[k][2] = __builtin_fmaf(h, a.z, acc[k][2]);
      acc[k][3] = __builtin_fmaf(h, a.w, acc[k][3]);
    } else if constexpr (WK == WK_F16) {
      uint32_t ww[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[k][2 * q] = __builtin_fmaf(h, h_lo(ww[q]), acc[k][2 * q]);
        acc[k][2 * q + 1] = __builtin_fmaf(h, h_hi(ww[q]), acc[k][2 * q + 1]);
      }
    } else {
      float hs = h * sc[k];
      uint32_t ww[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          int nib = (ww[q] >> (4 * b)) & 0xF;
          int qv = nib >= 8 ? nib - 16 : nib;
          acc[k][8 * q + b] = __builtin_fmaf(hs, (float)qv, acc[k][8 * q + b]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Predictor stage 1: one wave per row of P1.  z[k] = c1[k] + P1[k] . x
template <int PK, int CPL>
__global__ __launch_bounds__(256) void k_pred_z(const void* __restrict__ p1,
                                                const float* __restrict__ c1,
                                                const void* __restrict__ x,
                                                float* __restrict__ z, int d, int rank) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int row = blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
  if (row >= rank) return;
  const int nch = d / Kind<PK>::EPC;
  XRegs<PK, CPL> xr;
  load_x<PK, CPL>(xr, x, nch, lane);
  u32x4 w[CPL];
  float sc[CPL];
  load_row<PK, CPL>(w, sc, p1, nullptr, row, nch, lane);
  float acc = wave_sum(row_dot<PK, CPL>(w, sc, xr));
  if (lane == 0) z[row] = acc + (c1 ? c1[row] : 0.0f);
}

// ---------------------------------------------------------------------------------------------
// Main kernel.  Workgroup = one chunk of `nc` consecutive neurons; MW waves.
// Waves per workgroup: 8, or 4 when the token, three rows and the accumulators of a wave need
// more than the 256 registers a lane gets at two waves per SIMD.
constexpr int waves_for(int cpl) { return cpl >= 12 ? 4 : 8; }
int main_waves(int cpl) { return waves_for(cpl); }

template <int WK, int CPL, int MAIN_WAVES>
__global__ __launch_bounds__(MAIN_WAVES * WAVE) void k_main(MainArgs a) {
  extern __shared__ float smem[];
  // LDS layout: acc[d] | z[rank] | score[nc] | h[nc] | list[nc] | count
  float* s_acc = smem;
  float* s_z = s_acc + a.d;
  float* s_score = s_z + a.rank;
  float* s_h = s_score + a.nc;
  int* s_list = reinterpret_cast<int*>(s_h + a.nc);
  int* s_m = s_list + a.nc;

  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wave = tid / WAVE;
  const int chunk = blockIdx.x;
  const int i0 = chunk * a.nc;
  const int n = min(a.nc, a.ffn - i0);
  const int nch = a.d / Kind<WK>::EPC;

  // Token in registers (every wave needs all of it).
  XRegs<WK, CPL> xr;
  load_x<WK, CPL>(xr, a.x, nch, lane);

  for (int j = tid; j < a.d; j += blockDim.x) s_acc[j] = 0.0f;

  if (a.mask == nullptr) {
    // ---- predictor stage 2 over this chunk's neurons
    for (int k = tid; k < a.rank; k += blockDim.x) s_z[k] = a.z[k];
    __syncthreads();
    const int pe = a.p_f16 ? 8 : 4;                 // P2 elements per 16-byte chunk
    const int pch = a.rank / pe;                    // 16-byte chunks per P2 row
    int L = 64;                                     // lanes per row: next pow2 >= pch, <= 64
    while (L > 1 && (L >> 1) >= pch) L >>= 1;
    const int rpw = WAVE / L;                       // rows per wave per pass
    const int g = lane / L, gl = lane % L;
    for (int base = wave * rpw; base < n; base += MAIN_WAVES * rpw) {
      const int r = base + g;
      float acc = 0.0f;
      if (r < n) {
        const char* rp = static_cast<const char*>(a.p2) + (size_t)(i0 + r) * a.rank * (a.p_f16 ? 2 : 4);
        for (int c = gl; c < pch; c += L) {
          u32x4 w = ld16(rp + (size_t)c * 16);
          const float* zp = s_z + c * pe;
          if (a.p_f16) {
            uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc = __builtin_fmaf(h_lo(ww[q]), zp[2 * q], acc);
              acc = __builtin_fmaf(h_hi(ww[q]), zp[2 * q + 1], acc);
            }
          } else {
            f32x4 wf = __builtin_bit_cast(f32x4, w);
            acc = __builtin_fmaf(wf.x, zp[0], acc);
            acc = __builtin_fmaf(wf.y, zp[1], acc);
            acc = __builtin_fmaf(wf.z, zp[2], acc);
            acc = __builtin_fmaf(wf.w, zp[3], acc);
          }
        }
      }
      acc = group_sum(acc, L);
      if (r < n && gl == 0) {
        float s = acc + (a.c2 ? a.c2[i0 + r] : 0.0f);
        s_score[r] = s;
        if (a.scores) a.scores[i0 + r] = s;
      }
    }
    __syncthreads();
    // ---- compaction: ascending local list of neurons with score > thr (wave 0, ballots)
    if (wave == 0) {
      int m = 0;
      for (int b = 0; b < n; b += WAVE) {
        const int r = b + lane;
        const bool on = r < n && s_score[r] > a.thr;
        const unsigned long long bal = __ballot(on);
        const int pos = m + __popcll(bal & ((1ull << lane) - 1ull));
        if (on) s_list[pos] = i0 + r;
        m += __popcll(bal);
      }
      if (lane == 0) *s_m = m;
    }
  } else {
    // ---- caller's mask replaces the predictor
    if (wave == 0) {
      int m = 0;
      for (int b = 0; b < n; b += WAVE) {
        const int r = b + lane;
        const bool on = r < n && a.mask[i0 + r] != 0;
        const unsigned long long bal = __ballot(on);
        const int pos = m + __popcll(bal & ((1ull << lane) - 1ull));
        if (on) s_list[pos] = i0 + r;
        m += __popcll(bal);
      }
      if (lane == 0) *s_m = m;
    }
  }
  __syncthreads();
  const int m = *s_m;
  if (tid == 0) a.chunk_cnt[chunk] = m;
  for (int k = tid; k < m; k += blockDim.x) a.chunk_list[i0 + k] = s_list[k];

  // ---- gathered rows: wave w takes active neurons w, w + MW, ...  Up, gate and down rows of a
  // neuron are all requested before any of them is used.
  float acc[CPL][Kind<WK>::EPC];
#pragma unroll
  for (int k = 0; k < CPL; ++k)
#pragma unroll
    for (int e = 0; e < Kind<WK>::EPC; ++e) acc[k][e] = 0.0f;

  for (int t = wave; t < m; t += MAIN_WAVES) {
    const size_t i = (size_t)s_list[t];
    u32x4 wu[CPL], wg[CPL], wd[CPL];
    float su[CPL], sg[CPL], sd[CPL];
    load_row<WK, CPL>(wu, su, a.w_up, a.s_up, i, nch, lane);
    if (a.has_gate) load_row<WK, CPL>(wg, sg, a.w_gate, a.s_gate, i, nch, lane);
    load_row<WK, CPL>(wd, sd, a.w_dn, a.s_dn, i, nch, lane);
    float u = wave_sum(row_dot<WK, CPL>(wu, su, xr)) + (a.b_up ? a.b_up[i] : 0.0f);
    float h;
    if (a.act == FFN_ACT_RELU) {
      h = fmaxf(u, 0.0f);
    } else {
      float gv = wave_sum(row_dot<WK, CPL>(wg, sg, xr)) + (a.b_gate ? a.b_gate[i] : 0.0f);
      float gr = fmaxf(gv, 0.0f);
      h = a.act == FFN_ACT_REGLU ? gr * u : gr * fmaxf(u, 0.0f);
    }
    axpy_row<WK, CPL>(acc, h, wd, sd);
  }

  // ---- cross-wave reduction in LDS, fixed wave order, then one partial row per chunk
  const int active_waves = min(m, MAIN_WAVES);
  for (int w = 0; w < active_waves; ++w) {
    __syncthreads();
    if (wave == w) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = lane + k * WAVE;
        if (c < nch) {
#pragma unroll
          for (int e = 0; e < Kind<WK>::EPC; ++e) s_acc[c * Kind<WK>::EPC + e] += acc[k][e];
        }
      }
    }
  }
  __syncthreads();
  float* prow = a.part + (size_t)chunk * a.d;
  for (int j = tid * 4; j < a.d; j += blockDim.x * 4)
    *reinterpret_cast<f32x4*>(prow + j) = *reinterpret_cast<const f32x4*>(s_acc + j);
}

// ---------------------------------------------------------------------------------------------
// y[j] = b_down[j] + sum_c part[c][j].  Block = 64 columns x 16 chunk groups.
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int n_chunks,
                                                const float* __restrict__ b_down,
                                                float* __restrict__ y, int d) {
  __shared__ f32x4 s[16][16];
  const int q = threadIdx.x & 15;        // float4 column within the tile
  const int cg = threadIdx.x >> 4;       // chunk group
  const int j = (blockIdx.x * 16 + q) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (j < d) {
    for (int c = cg; c < n_chunks; c += 16)
      acc += *reinterpret_cast<const f32x4*>(part + (size_t)c * d + j);
  }
  s[cg][q] = acc;
  __syncthreads();
  if (cg == 0 && j < d) {
    f32x4 t = s[0][q];
#pragma unroll
    for (int k = 1; k < 16; ++k) t += s[k][q];
    if (b_down) t += *reinterpret_cast<const f32x4*>(b_down + j);
    *reinterpret_cast<f32x4*>(y + j) = t;
  }
}

// Global ascending index list from the per-chunk lists (test hook; not on the timed path).
__global__ __launch_bounds__(256) void k_write_idx(const int* __restrict__ ccnt,
                                                   const int* __restrict__ clist, int n_chunks,
                                                   int nc, int* __restrict__ idx,
                                                   int* __restrict__ cnt) {
  __shared__ int s_off;
  const int chunk = blockIdx.x;
  if (threadIdx.x == 0) {
    int off = 0;
    for (int c = 0; c < chunk; ++c) off += ccnt[c];
    s_off = off;
    if (chunk == n_chunks - 1 && cnt) *cnt = off + ccnt[chunk];
  }
  __syncthreads();
  const int m = ccnt[chunk];
  if (idx)
    for (int k = threadIdx.x; k < m; k += blockDim.x) idx[s_off + k] = clist[chunk * nc + k];
}

// ---------------------------------------------------------------------------------------------
// Host launchers.
template <int PK, int CPL>
static hipError_t launch_pred_z_t(const void* p1, const float* c1, const void* x, float* z,
                                  int d, int rank, hipStream_t st) {
  const int wpb = 4;
  dim3 grid((rank + wpb - 1) / wpb);
  hipLaunchKernelGGL((k_pred_z<PK, CPL>), grid, dim3(wpb * WAVE), 0, st, p1, c1, x, z, d, rank);
  return hipGetLastError();
}

#define CPL_SWITCH(cpl, F)                                                                    \
  switch (cpl) {                                                                              \
    case 1: return F(1); case 2: return F(2); case 3: return F(3); case 4: return F(4);       \
    case 6: return F(6); case 8: return F(8); case 12: return F(12); case 16: return F(16);   \
    default: return hipErrorInvalidValue;                                                     \
  }

hipError_t launch_pred_z(int p_f16, int cpl, const void* p1, const float* c1, const void* x,
                         float* z, int d, int rank, hipStream_t st) {
  if (p_f16) {
#define F16Z(c) launch_pred_z_t<WK_F16, c>(p1, c1, x, z, d, rank, st)
    CPL_SWITCH(cpl, F16Z)
#undef F16Z
  } else {
#define F32Z(c) launch_pred_z_t<WK_F32, c>(p1, c1, x, z, d, rank, st)
    CPL_SWITCH(cpl, F32Z)
#undef F32Z
  }
}

size_t main_lds_bytes(int d, int rank, int nc) {
  return (size_t)(d + rank + 3 * nc + 1) * 4;
}

template <int WK, int CPL>
static hipError_t launch_main_t(const MainArgs& a, int n_chunks, hipStream_t st,
                                hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int MW = waves_for(CPL);
  size_t lds = main_lds_bytes(a.d, a.rank, a.nc);
  if (ev0 && ev1) {
    // events attached to the dispatch: their elapsed time is this launch's execution time
    hipExtLaunchKernelGGL((k_main<WK, CPL, MW>), dim3(n_chunks), dim3(MW * WAVE), lds, st, ev0,
                          ev1, 0, a);
  } else {
    hipLaunchKernelGGL((k_main<WK, CPL, MW>), dim3(n_chunks), dim3(MW * WAVE), lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_main(int wk, int cpl, const MainArgs& a, int n_chunks, hipStream_t st,
                       hipEvent_t ev0, hipEvent_t ev1) {
  if (wk == WK_F32) {
#define M32(c) launch_main_t<WK_F32, c>(a, n_chunks, st, ev0, ev1)
    CPL_SWITCH(cpl, M32)
#undef M32
  } else if (wk == WK_F16) {
#define M16(c) launch_main_t<WK_F16, c>(a, n_chunks, st, ev0, ev1)
    CPL_SWITCH(cpl, M16)
#undef M16
  } else {
    // int4 rows: 32 elements per chunk, so d <= 8192 needs at most 4 chunks per lane
    switch (cpl) {
      case 1: return launch_main_t<WK_I4, 1>(a, n_chunks, st, ev0, ev1);
      case 2: return launch_main_t<WK_I4, 2>(a, n_chunks, st, ev0, ev1);
      case 3: return launch_main_t<WK_I4, 3>(a, n_chunks, st, ev0, ev1);
      case 4: return launch_main_t<WK_I4, 4>(a, n_chunks, st, ev0, ev1);
      default: return hipErrorInvalidValue;
    }
  }
}

hipError_t launch_reduce(const float* part, int n_chunks, const float* b_down, float* y, int d,
                         hipStream_t st) {
  dim3 grid((d / 4 + 15) / 16);
  hipLaunchKernelGGL(k_reduce, grid, dim3(256), 0, st, part, n_chunks, b_down, y, d);
  return hipGetLastError();
}

hipError_t launch_write_idx(const int* ccnt, const int* clist, int n_chunks, int nc, int* idx,
                            int* cnt, hipStream_t st) {
  hipLaunchKernelGGL(k_write_idx, dim3(n_chunks), dim3(256), 0, st, ccnt, clist, n_chunks, nc,
                     idx, cnt);
  return hipGetLastError();
}

}  // namespace ffn
