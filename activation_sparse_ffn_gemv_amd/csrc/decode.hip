// Batch-1 decode path of the activation-sparse FFN on gfx950.
//
// Per token and layer, four launches on the caller's stream; each spreads its bytes evenly over
// all the CUs (a CU can only keep so many requests in flight, so an uneven split leaves the
// busiest CU setting the time):
//   k_pred_z   z = P1 x + c1                            (predictor stage 1; one wave per P1 row)
//   k_pred_s   s = P2 z + c2, active iff s > logit(tau); one word of the active bitmap per 32
//              neurons, built with a wave ballot                       (predictor stage 2)
//   k_gather   256 workgroups split the active neurons evenly by rank; each reads the up, gate
//              and transposed-down rows of its neurons in one trip (every thread the same column
//              chunks of every row), forms u, g, h from workgroup-wide sums and adds one
//              contiguous-row axpy per neuron into its partial of y
//   k_reduce   y = b_down + sum of the partials, in a fixed order
// No global atomics anywhere, so y is bit-reproducible run to run.
//
// The method (PowerInfer, unite.ai: "Adaptive sparse predictor", "Neuron-aware operator";
// nearauto.com Fig. 8; citnews.com.cn "Dynamic neuron cache") reads only the predicted
// neurons' rows of up / gate and of the transposed down projection.
#include <hip/hip_ext.h>

#include "common.h"
#include "index.h"
#include "launch.h"

namespace ffn {

#ifdef FFN_TRACE
__device__ unsigned long long* g_trace;
extern "C" hipError_t ffn_trace_set_buffer(void* p) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_trace), &p, sizeof(p));
}
#endif

// ---------------------------------------------------------------------------------------------
// Predictor stage 1: one 64-thread workgroup per row of P1.  z[k] = c1[k] + P1[k] . x
template <int PK, int CPL>
__global__ __launch_bounds__(64) void k_pred_z(const void* __restrict__ p1,
                                               const float* __restrict__ c1,
                                               const void* __restrict__ x,
                                               float* __restrict__ z, int d, int rank,
                                               const ExpertW* __restrict__ slot, int zstride) {
  FFN_TS(0, 0);
  if (slot) {
    slot += blockIdx.y;                         // expert slots side by side
    z += (size_t)blockIdx.y * zstride;
    p1 = slot->p1;
    c1 = slot->c1;
  }
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int nch = d / Kind<PK>::EPC;
  XRegs<PK, CPL> xr;
  load_x<PK, CPL>(xr, x, nch, lane);
  u32x4 w[CPL];
  float sc[CPL];
  load_row<PK, CPL>(w, sc, p1, nullptr, row, nch, lane);
  issue_fence();
  finish_x<PK, CPL>(xr, nch, lane);
  const float acc = wave_sum(row_dot<PK, CPL>(w, sc, xr));
  FFN_TS(0, 1);
  if (lane == 0) z[row] = acc + (c1 ? c1[row] : 0.0f);
  FFN_TS(0, 2);
}

// ---------------------------------------------------------------------------------------------
// Predictor stage 2 + threshold + bitmap.  Workgroup of 256 threads = 32 neurons = one word of
// the active bitmap.  A P2 row (rank values) is split over L lanes (L = next power of two >= its
// 16-byte chunk count, 4..64; CPR chunks per lane beyond 64 chunks); all passes' loads are issued
// before any is used.
constexpr int PS_THREADS = 256;
constexpr int PS_MAXP = 8;

// MAXP: the passes the rank needs (1, 2, 4 or 8), so that no registers sit idle.
template <int PK, int CPR, int MAXP>
__global__ __launch_bounds__(PS_THREADS) void k_pred_s(PredArgs a) {
  constexpr int PE = Kind<PK>::EPC;           // predictor elements per 16-byte chunk
  __shared__ float s_score[32];
  const int tid = threadIdx.x;
  const int pch = a.rank / PE;
  int L = 64;
  while (L > 4 && (L >> 1) >= pch) L >>= 1;
  const int R = PS_THREADS / L;               // rows per pass
  const int P = (32 + R - 1) / R;             // passes (<= 8)
  const int g = tid / L, gl = tid % L;
  const int i0 = blockIdx.x * 32;
  FFN_TS(3, 0);
  if (a.slot) {
    a.slot += blockIdx.y;                       // expert slots side by side
    a.z = a.zall ? a.zall + (size_t)a.slot->expert * a.rank : a.z + (size_t)blockIdx.y * a.zstride;
    a.bitmap += (size_t)blockIdx.y * a.bstride;
    a.p2 = a.slot->p2;
    a.c2 = a.slot->c2;
  }
  if ((int)blockIdx.x < a.head_words) {         // hot head: always active, no score computed
    if (tid == 0) a.bitmap[blockIdx.x] = ~0u;
    return;
  }
  const float c2v = (tid < 32 && a.c2) ? a.c2[i0 + tid] : 0.0f;
  f32x4 zr[CPR][PE / 4];                      // this lane's z slice, fixed across rows
#pragma unroll
  for (int k = 0; k < CPR; ++k) {
    const int c = gl + k * L;
    const int cc = min(c, pch - 1);
#pragma unroll
    for (int q = 0; q < PE / 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.z + cc * PE + 4 * q);
      zr[k][q] = c < pch ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // every pass's loads in one straight run (rows clamped into the word, so a pass past P just
  // re-reads a row of it): a per-pass branch here would make each pass wait for its own loads
  u32x4 w[MAXP][CPR];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int r = min(p * R + g, 31);
#pragma unroll
    for (int k = 0; k < CPR; ++k) {
      const int cc = min(gl + k * L, pch - 1);
      w[p][k] = ld16(static_cast<const char*>(a.p2) + ((size_t)(i0 + r) * pch + cc) * 16);
    }
  }
  issue_fence();
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if (p < P) {                              // uniform
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < CPR; ++k) {
      if (gl + k * L >= pch) continue;        // lane past the row end (small ranks)
      const float* zf = reinterpret_cast<const float*>(&zr[k][0]);
      if constexpr (PK == WK_F16) {
        const uint32_t ww[4] = {w[p][k].x, w[p][k].y, w[p][k].z, w[p][k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc = __builtin_fmaf(h_lo(ww[q]), zf[2 * q], acc);
          acc = __builtin_fmaf(h_hi(ww[q]), zf[2 * q + 1], acc);
        }
      } else {
        const f32x4 wf = __builtin_bit_cast(f32x4, w[p][k]);
        acc = __builtin_fmaf(wf.x, zf[0], acc);
        acc = __builtin_fmaf(wf.y, zf[1], acc);
        acc = __builtin_fmaf(wf.z, zf[2], acc);
        acc = __builtin_fmaf(wf.w, zf[3], acc);
      }
    }
    acc = group_sum_last(acc, L);
    const int r = p * R + g;
    if (gl == L - 1 && r < 32) s_score[r] = acc;
    }
  }
  __syncthreads();
  if (tid < WAVE) {
    bool on = false;
    if (tid < 32) {
      const float sc = s_score[tid] + c2v;
      on = sc > a.thr;
      if (a.scores) a.scores[i0 + tid] = sc;
    }
    const unsigned long long bal = __ballot(on);
    if (tid == 0) a.bitmap[blockIdx.x] = (uint32_t)bal;
  }
  FFN_TS(3, 5);
}

// Caller-supplied mask -> bitmap: one wave builds two 32-bit words.  mask == nullptr sets every
// bit (the dense FFN over all neurons).
__global__ __launch_bounds__(256) void k_mask_bits(const unsigned char* __restrict__ mask,
                                                   uint32_t* __restrict__ bitmap, int words) {
  const int w = blockIdx.x * 4 + threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  const int word = w * 2 + (lane >> 5);
  const bool on = word < words && (!mask || mask[(size_t)word * 32 + (lane & 31)] != 0);
  const unsigned long long bal = __ballot(on);
  if (lane == 0 && word < words) bitmap[word] = (uint32_t)bal;
  if (lane == 32 && word < words) bitmap[word] = (uint32_t)(bal >> 32);
}

// ---------------------------------------------------------------------------------------------
// Balanced gather.  GA_BLOCKS workgroups of 512 threads split the active neurons evenly by
// rank: workgroup g owns ranks [g*|A|/G, (g+1)*|A|/G).
//   1. the bitmap (two words per thread) is prefix-summed over the workgroup; the threads whose
//      words hold the workgroup's ranks write those neurons to an LDS list;
//   2. the threads form SLOTS groups of TPR = 512 / SLOTS (SLOTS > 1 when a row has fewer
//      16-byte chunks than the workgroup has threads); thread (slot, c) owns the column chunks
//      c, c + TPR, ... of every row.  Rounds of up to SLOTS * RN neurons, neuron q of a round on
//      slot q % SLOTS: every thread requests its chunks of the up, gate and transposed-down rows
//      of its slot's neurons at once (the neurons' biases with them), forms partial dot products
//      with its slice of the token; the partials are summed over the slot (DPP wave sums, then
//      the slot's waves in order) into u, g and h; each thread adds h * (its down chunks) to its
//      own accumulator: one contiguous-row axpy per active neuron;
//   3. the slots' accumulators are summed through LDS (fixed order) and form the workgroup's
//      partial of y (written only when it owns a rank).
// Every workgroup and every thread does the same work, so the load is even over the CUs.
constexpr int GA_THREADS = 512;
constexpr int GA_NW = GA_THREADS / WAVE;
constexpr int GA_BLOCKS = 256;
constexpr int GA_MAXW = 2;            // bitmap words per thread: ffn <= 32768
constexpr int GA_LIST = 64;           // ranks resolved per batch

// Neurons per slot and round: as many as the registers hold, and every round fits the rank batch.
template <int WK, int CPT, int SLOTS> struct Round {
  static constexpr int BASE = WK == WK_I4 ? 8 : 16 / CPT;
  static constexpr int RN = BASE * SLOTS <= GA_LIST ? BASE : GA_LIST / SLOTS;
};

// CACHED: the neuron-cache variant (fp16 rows): the ranks' neurons and row sources come from
// the cache plan instead of the bitmap, and rows read from host memory are also written to
// their cache slot.
template <int WK, int CPT, int SLOTS, bool CACHED = false>
__global__ __launch_bounds__(GA_THREADS) void k_gather(GatherArgs a) {
  constexpr int NT = GA_THREADS;
  constexpr int TPR = NT / SLOTS;                 // threads per row
  constexpr int WPS = TPR / WAVE;                 // waves per slot
  constexpr int RN = Round<WK, CPT, SLOTS>::RN;   // neurons per slot and round
  constexpr int RQ = RN * SLOTS;                  // neurons per round
  constexpr int EPC = Kind<WK>::EPC;
  static_assert(RQ <= GA_LIST && GA_LIST % RQ == 0, "rounds tile the rank batch");
  static_assert(!CACHED || WK == WK_F16, "the neuron cache holds fp16 rows");
  static_assert(32 * GA_MAXW < (1 << 7), "a thread's count fits the prefix's seven bit planes");
  __shared__ int s_wsum[GA_NW];
  __shared__ int s_list[GA_LIST];
  __shared__ int s_src[CACHED ? GA_LIST : 1];
  __shared__ int s_vic[CACHED ? GA_LIST : 1];
  __shared__ float s_red[GA_NW][2 * RN];
  __shared__ float s_h[RQ];
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int slot = tid / TPR, ct = tid % TPR;
  const int nch = a.d / EPC;
  FFN_TS(1, 0);
  if (a.slot) {
    a.slot += blockIdx.y;                       // expert slots side by side
    a.bitmap += (size_t)blockIdx.y * a.bstride;
    a.cnt += (size_t)blockIdx.y * a.cstride;
    a.part += (size_t)blockIdx.y * a.pstride;
    const ExpertW& e = *a.slot;
    a.w_up = e.w_up;
    a.w_gate = e.w_gate;
    a.w_dn = e.w_dn;
    a.s_up = e.s_up;
    a.s_gate = e.s_gate;
    a.s_dn = e.s_dn;
    a.b_up = e.b_up;
    a.b_gate = e.b_gate;
  }

  // this thread's chunks of the token (chunk ct + k*TPR)
  u32x4 xr[CPT][Kind<WK>::XW];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = ct + k * TPR;
    const int cc = min(c, nch - 1);
#pragma unroll
    for (int q = 0; q < Kind<WK>::XW; ++q) {
      const u32x4 v = ld16(static_cast<const char*>(a.x) + (size_t)cc * 16 * Kind<WK>::XW + q * 16);
      xr[k][q] = c < nch ? v : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (WK == WK_I4) i4_perm_x(xr[k]);
  }

  // 1. word prefix of the bitmap: thread t owns words 2t, 2t+1 (consecutive)
  const int words = a.ffn / 32;
  const uint32_t nblk = gridDim.x;
  uint32_t b[GA_MAXW];
  int local = 0, total = 0, run0 = 0;
  if constexpr (CACHED) {
    total = *a.cnt;                              // written by the cache plan
  } else {
#pragma unroll
  for (int k = 0; k < GA_MAXW; ++k) {
    const int w = tid * GA_MAXW + k;
    b[k] = w < words ? a.bitmap[w] : 0u;
    local += __popc(b[k]);
  }
  // the grid size (a hidden kernel argument, on its own scalar-cache line) is waited for here,
  // while the token and bitmap loads are in flight, rather than after the barrier below
  asm volatile("" ::"s"(nblk));
  // local <= 32 * GA_MAXW = 64: seven bit planes
  int wtot;
  const int before = wave_prefix_small<7>(local, wtot);
  if (lane == 0) s_wsum[wave] = wtot;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int k = 0; k < GA_NW; ++k) {
    base += k < wave ? s_wsum[k] : 0;
    total += s_wsum[k];
  }
  run0 = base + before;                          // rank of this thread's first active neuron
  }
  int r0, r1;
  gather_rank_range((uint32_t)total, blockIdx.x, nblk, r0, r1);
  FFN_TS(1, 1);

  float acc[CPT][EPC];
#pragma unroll
  for (int k = 0; k < CPT; ++k)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[k][e] = 0.0f;

  for (int l0 = r0; l0 < r1; l0 += GA_LIST) {
    const int nl = min(GA_LIST, r1 - l0);
    // owners of ranks [l0, l0 + nl): every thread whose words hold some of them writes those
    // (no search: a thread knows the ranks of its own active neurons)
    if constexpr (CACHED) {
      if (tid < nl) {
        s_list[tid] = a.rank_nid[l0 + tid];
        s_src[tid] = a.rank_src[l0 + tid];
        s_vic[tid] = a.rank_vic[l0 + tid];
      }
    } else if (run0 < l0 + nl && run0 + local > l0) {
      int pos = run0;
#pragma unroll
      for (int k = 0; k < GA_MAXW; ++k) {
        uint32_t bb = b[k];
        const int nbase = (tid * GA_MAXW + k) * 32;
        while (bb) {
          if (pos >= l0 && pos < l0 + nl) s_list[pos - l0] = nbase + __builtin_ctz(bb);
          bb &= bb - 1;
          ++pos;
        }
      }
    }
    __syncthreads();
    FFN_TS(1, 2);
    for (int t0 = 0; t0 < nl; t0 += RQ) {
      u32x4 wu[RN][CPT], wg[RN][CPT], wd[RN][CPT];
      uint32_t su[RN][CPT], sg[RN][CPT], sd[RN][CPT];        // words holding int4 group scales
      // the biases of the round's neurons travel with the rows (thread q < RQ: neuron q)
      float bu = 0.0f, bgt = 0.0f;
      if (tid < RQ && t0 + tid < nl) {
        const int nq = s_list[t0 + tid];
        if (a.b_up) bu = a.b_up[nq];
        if (a.b_gate) bgt = a.b_gate[nq];
      }
#pragma unroll
      for (int r = 0; r < RN; ++r) {
        const int q = r * SLOTS + slot;                      // this slot's r-th neuron
        const bool live_r = t0 + q < nl;                     // uniform across the slot's waves
        const size_t nr = (size_t)s_list[min(t0 + q, nl - 1)];
        // row bases: the neuron's rows, or (cache) its slot's rows when it is resident
        size_t row = nr;
        const char* pu = static_cast<const char*>(a.w_up);
        const char* pg = static_cast<const char*>(a.w_gate);
        const char* pd = static_cast<const char*>(a.w_dn);
        if constexpr (CACHED) {
          const int sr = s_src[min(t0 + q, nl - 1)];
          if (sr >= 0) {
            row = (size_t)sr;
            pu = static_cast<const char*>(a.c_up);
            pg = static_cast<const char*>(a.c_gate);
            pd = static_cast<const char*>(a.c_dn);
          }
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          const int cc = min(ct + k * TPR, nch - 1);
          const size_t off = (row * nch + cc) * 16;
          wu[r][k] = wg[r][k] = wd[r][k] = u32x4{0u, 0u, 0u, 0u};
          su[r][k] = sg[r][k] = sd[r][k] = 0u;
          if (live_r) {
            wu[r][k] = ld16(pu + off);
            if (a.has_gate) wg[r][k] = ld16(pg + off);
            wd[r][k] = ld16(pd + off);
            if constexpr (WK == WK_I4) {
              // (ffn is a multiple of 32, so the word of the last scale is inside the array)
              su[r][k] = ldh_word(a.s_up, nr * nch + cc);
              if (a.has_gate) sg[r][k] = ldh_word(a.s_gate, nr * nch + cc);
              sd[r][k] = ldh_word(a.s_dn, nr * nch + cc);
            }
          }
        }
      }
      issue_fence();
#pragma unroll
      for (int r = 0; r < RN; ++r) {
        if (t0 + r * SLOTS + slot < nl) {                    // uniform across the wave
          float pu = 0.0f, pg = 0.0f;
#pragma unroll
          for (int k = 0; k < CPT; ++k) {
            if constexpr (WK == WK_F32) {
              pu = dot4_f32(wu[r][k], xr[k][0], pu);
              if (a.has_gate) pg = dot4_f32(wg[r][k], xr[k][0], pg);
            } else if constexpr (WK == WK_F16) {
              pu = dot8_f16(wu[r][k], xr[k][0], pu);
              if (a.has_gate) pg = dot8_f16(wg[r][k], xr[k][0], pg);
            } else {
              const size_t si = (size_t)s_list[min(t0 + r * SLOTS + slot, nl - 1)] * nch +
                                min(ct + k * TPR, nch - 1);
              pu = dot32_i4(wu[r][k], xr[k], pick_h(su[r][k], si), pu);
              if (a.has_gate) pg = dot32_i4(wg[r][k], xr[k], pick_h(sg[r][k], si), pg);
            }
          }
          pu = wave_sum(pu);
          if (a.has_gate) pg = wave_sum(pg);
          if (lane == 0) {
            s_red[wave][2 * r] = pu;
            s_red[wave][2 * r + 1] = pg;
          }
          if constexpr (CACHED) {
            // a row read from host memory goes to its cache slot as well
            const int vs = s_vic[t0 + r * SLOTS + slot];
            if (vs >= 0) {
#pragma unroll
              for (int k = 0; k < CPT; ++k) {
                if (ct + k * TPR < nch) {
                  const size_t off = ((size_t)vs * nch + ct + k * TPR) * 16;
                  *reinterpret_cast<u32x4*>(static_cast<char*>(a.c_up) + off) = wu[r][k];
                  if (a.has_gate) *reinterpret_cast<u32x4*>(static_cast<char*>(a.c_gate) + off) = wg[r][k];
                  *reinterpret_cast<u32x4*>(static_cast<char*>(a.c_dn) + off) = wd[r][k];
                }
              }
            }
          }
        }
      }
      __syncthreads();
      if (tid < RQ) {
        const int q = tid, qs = q % SLOTS, qr = q / SLOTS;
        float u = 0.0f, g = 0.0f, h = 0.0f;
        if (t0 + q < nl) {
#pragma unroll
          for (int w = 0; w < WPS; ++w) {
            u += s_red[qs * WPS + w][2 * qr];
            g += s_red[qs * WPS + w][2 * qr + 1];
          }
          u += bu;
          if (a.act == FFN_ACT_RELU) {
            h = fmaxf(u, 0.0f);
          } else {
            g = fmaxf(g + bgt, 0.0f);
            h = a.act == FFN_ACT_REGLU ? g * u : g * fmaxf(u, 0.0f);
          }
        }
        s_h[q] = h;                                          // 0 for slots past the list
      }
      __syncthreads();
      FFN_TS(1, 3);
#pragma unroll
      for (int r = 0; r < RN; ++r) {
        if (t0 + r * SLOTS + slot >= nl) break;              // uniform; later slots are dead too
        const float h = s_h[r * SLOTS + slot];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          if constexpr (WK == WK_F32) {
            const f32x4 q = __builtin_bit_cast(f32x4, wd[r][k]);
            acc[k][0] = __builtin_fmaf(h, q.x, acc[k][0]);
            acc[k][1] = __builtin_fmaf(h, q.y, acc[k][1]);
            acc[k][2] = __builtin_fmaf(h, q.z, acc[k][2]);
            acc[k][3] = __builtin_fmaf(h, q.w, acc[k][3]);
          } else if constexpr (WK == WK_F16) {
            const uint32_t ww[4] = {wd[r][k].x, wd[r][k].y, wd[r][k].z, wd[r][k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[k][2 * q] = __builtin_fmaf(h, h_lo(ww[q]), acc[k][2 * q]);
              acc[k][2 * q + 1] = __builtin_fmaf(h, h_hi(ww[q]), acc[k][2 * q + 1]);
            }
          } else {
            const size_t si = (size_t)s_list[min(t0 + r * SLOTS + slot, nl - 1)] * nch +
                              min(ct + k * TPR, nch - 1);
            const float hs = h * pick_h(sd[r][k], si);
            const uint32_t ww[4] = {wd[r][k].x, wd[r][k].y, wd[r][k].z, wd[r][k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int bb = 0; bb < 8; ++bb)
                acc[k][8 * q + bb] = __builtin_fmaf(hs, (float)((int)(ww[q] << (28 - 4 * bb)) >> 28),
                                                    acc[k][8 * q + bb]);
          }
        }
      }
      __syncthreads();                                       // s_red / s_h reused
    }
  }
  FFN_TS(1, 4);
  if (r1 > r0) {
    if constexpr (SLOTS > 1) {
      // sum the slots' accumulators: slots 1.. park theirs in LDS (16-byte vectors, consecutive
      // threads at consecutive addresses), slot 0 adds them in slot order
      extern __shared__ __align__(16) f32x4 s_acc[];         // [SLOTS-1][CPT][EPC/4][TPR]
      if (slot > 0) {
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
          for (int e = 0; e < EPC; e += 4)
            s_acc[(((slot - 1) * CPT + k) * (EPC / 4) + e / 4) * TPR + ct] =
                f32x4{acc[k][e], acc[k][e + 1], acc[k][e + 2], acc[k][e + 3]};
      }
      __syncthreads();
      if (slot == 0) {
#pragma unroll
        for (int o = 1; o < SLOTS; ++o)
#pragma unroll
          for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int e = 0; e < EPC; e += 4) {
              const f32x4 t = s_acc[(((o - 1) * CPT + k) * (EPC / 4) + e / 4) * TPR + ct];
              acc[k][e] += t.x;
              acc[k][e + 1] += t.y;
              acc[k][e + 2] += t.z;
              acc[k][e + 3] += t.w;
            }
      }
    }
    // partial of y, tile-major: part[col / RD_TW][workgroup][col % RD_TW], so that the reduce
    // reads one contiguous block per tile
    if (slot == 0) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int c = ct + k * TPR;
        if (c < nch) {
#pragma unroll
          for (int e = 0; e < EPC; e += 4) {
            float* dst = a.part + part_offset(c * EPC + e, blockIdx.x, nblk);
            // streaming store: the partial is read once, by the next kernel
            __builtin_nontemporal_store(f32x4{acc[k][e], acc[k][e + 1], acc[k][e + 2], acc[k][e + 3]},
                                        reinterpret_cast<f32x4*>(dst));
          }
        }
      }
    }
  }
  // stored last: a store ahead of a barrier would hold this workgroup at the barrier
  if (!CACHED && blockIdx.x == 0 && tid == 0) *a.cnt = total;
  FFN_TRACE_SYNC();
  FFN_TS(1, 5);
  FFN_TV(1, 6, r1 - r0);
}

// ---------------------------------------------------------------------------------------------
// Fused predictor stage 2 + gather (batch-1 decode variant).  A workgroup of 512 threads owns 64
// consecutive neurons (two bitmap words; the last may own 32):
//   1. s = P2 z + c2 for its rows (as k_pred_s: a P2 row split over L lanes, all passes' loads
//      in flight together with the token's), threshold, a 64-lane ballot -> the two bitmap words
//      and the ascending local list of its active neurons;
//   2. rounds of up to RN of those neurons exactly as in k_gather (thread t owns column chunks
//      t, t + 512, ...; workgroup sums through DPP and LDS; one row axpy per neuron);
//   3. its partial of y (written only when one of its neurons fired).
// No rank balancing: the workgroups' loads differ with the token's set, but the predictor's
// second stage and the gather share one launch and no scan is needed.
constexpr int FU_THREADS = 512;
constexpr int FU_NW = FU_THREADS / WAVE;
constexpr int FU_ROWS = 64;

template <int WK, int CPT, int CPR>
__global__ __launch_bounds__(FU_THREADS) void k_fused(FusedArgs f) {
  constexpr int NT = FU_THREADS;
  constexpr int RN = 16 / CPT;
  constexpr int EPC = Kind<WK>::EPC;
  constexpr int PK = WK == WK_F32 ? WK_F32 : WK_F16;    // predictor storage = token storage
  constexpr int PE = Kind<PK>::EPC;
  __shared__ float s_score[FU_ROWS];
  __shared__ int s_list[FU_ROWS];
  __shared__ int s_m;
  __shared__ float s_red[FU_NW][2 * RN];
  __shared__ float s_h[RN];
  const PredArgs& p = f.pa;
  const GatherArgs& a = f.ga;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int i0 = blockIdx.x * FU_ROWS;
  const int n = min(FU_ROWS, p.ffn - i0);               // 64, or 32 for the last workgroup
  const int nh = min(max(32 * p.head_words - i0, 0), n); // hot-head rows: on, no score
  const int nch = a.d / EPC;
  FFN_TS(1, 0);

  // this thread's chunks of the token (chunk tid + k*NT)
  u32x4 xr[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = tid + k * NT;
    const u32x4 v = ld16(static_cast<const char*>(a.x) + (size_t)min(c, nch - 1) * 16);
    xr[k] = c < nch ? v : u32x4{0u, 0u, 0u, 0u};
  }

  // 1. scores of the workgroup's rows
  const int pch = p.rank / PE;
  int L = 64;
  while (L > 4 && (L >> 1) >= pch) L >>= 1;
  const int R = NT / L;                                 // rows per pass
  const int P = (n + R - 1) / R;                        // passes (<= PS_MAXP)
  const int g = tid / L, gl = tid % L;
  const float c2v = (tid >= nh && tid < n && p.c2) ? p.c2[i0 + tid] : 0.0f;
  f32x4 zr[CPR][PE / 4];
#pragma unroll
  for (int k = 0; k < CPR; ++k) {
    const int c = gl + k * L;
    const int cc = min(c, pch - 1);
#pragma unroll
    for (int q = 0; q < PE / 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p.z + cc * PE + 4 * q);
      zr[k][q] = c < pch ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // every pass's loads in one straight run (rows clamped into the workgroup's): a per-pass branch
  // here would make each pass wait for its own loads
  u32x4 w[PS_MAXP][CPR];
  if (nh < n) {                                         // uniform: not a whole-head workgroup
#pragma unroll
    for (int pp = 0; pp < PS_MAXP; ++pp) {
      const int r = min(pp * R + g, n - 1);
#pragma unroll
      for (int k = 0; k < CPR; ++k) {
        const int cc = min(gl + k * L, pch - 1);
        w[pp][k] = ld16(static_cast<const char*>(p.p2) + ((size_t)(i0 + r) * pch + cc) * 16);
      }
    }
  }
  issue_fence();
#pragma unroll
  for (int pp = 0; pp < PS_MAXP; ++pp) {
    if (pp < P && nh < n) {                             // uniform
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < CPR; ++k) {
      if (gl + k * L >= pch) continue;                 // lane past the row end (small ranks)
      const float* zf = reinterpret_cast<const float*>(&zr[k][0]);
      if constexpr (PK == WK_F16) {
        const uint32_t ww[4] = {w[pp][k].x, w[pp][k].y, w[pp][k].z, w[pp][k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc = __builtin_fmaf(h_lo(ww[q]), zf[2 * q], acc);
          acc = __builtin_fmaf(h_hi(ww[q]), zf[2 * q + 1], acc);
        }
      } else {
        const f32x4 wf = __builtin_bit_cast(f32x4, w[pp][k]);
        acc = __builtin_fmaf(wf.x, zf[0], acc);
        acc = __builtin_fmaf(wf.y, zf[1], acc);
        acc = __builtin_fmaf(wf.z, zf[2], acc);
        acc = __builtin_fmaf(wf.w, zf[3], acc);
      }
    }
    acc = group_sum_last(acc, L);
    const int r = pp * R + g;
    if (gl == L - 1 && r < n) s_score[r] = acc;
    }
  }
  __syncthreads();
  FFN_TS(1, 1);
  if (wave == 0) {
    bool on = false;
    if (lane < nh) {
      on = true;
    } else if (lane < n) {
      const float sc = s_score[lane] + c2v;
      on = sc > p.thr;
      if (p.scores) p.scores[i0 + lane] = sc;
    }
    const unsigned long long bal = __ballot(on);
    if (on) s_list[__popcll(bal & ((1ull << lane) - 1ull))] = i0 + lane;
    if (lane == 0) {
      p.bitmap[blockIdx.x * 2] = (uint32_t)bal;
      if (n > 32) p.bitmap[blockIdx.x * 2 + 1] = (uint32_t)(bal >> 32);
      s_m = __popcll(bal);
    }
  }
  __syncthreads();
  FFN_TS(1, 2);
  const int m = s_m;

  float acc[CPT][EPC];
#pragma unroll
  for (int k = 0; k < CPT; ++k)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[k][e] = 0.0f;

  for (int t0 = 0; t0 < m; t0 += RN) {
    u32x4 wu[RN][CPT], wg[RN][CPT], wd[RN][CPT];
    float bu = 0.0f, bgt = 0.0f;
    if (tid < RN && t0 + tid < m) {
      const int nq = s_list[t0 + tid];
      if (a.b_up) bu = a.b_up[nq];
      if (a.b_gate) bgt = a.b_gate[nq];
    }
#pragma unroll
    for (int r = 0; r < RN; ++r) {
      const bool live_r = t0 + r < m;                   // uniform across the workgroup
      const size_t nr = (size_t)s_list[min(t0 + r, m - 1)];
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const size_t off = (nr * nch + min(tid + k * NT, nch - 1)) * 16;
        wu[r][k] = wg[r][k] = wd[r][k] = u32x4{0u, 0u, 0u, 0u};
        if (live_r) {
          wu[r][k] = ld16(static_cast<const char*>(a.w_up) + off);
          if (a.has_gate) wg[r][k] = ld16(static_cast<const char*>(a.w_gate) + off);
          wd[r][k] = ld16(static_cast<const char*>(a.w_dn) + off);
        }
      }
    }
    issue_fence();
#pragma unroll
    for (int r = 0; r < RN; ++r) {
      if (t0 + r < m) {                                  // uniform across the workgroup
        float pu = 0.0f, pg = 0.0f;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          if constexpr (WK == WK_F32) {
            pu = dot4_f32(wu[r][k], xr[k], pu);
            if (a.has_gate) pg = dot4_f32(wg[r][k], xr[k], pg);
          } else {
            pu = dot8_f16(wu[r][k], xr[k], pu);
            if (a.has_gate) pg = dot8_f16(wg[r][k], xr[k], pg);
          }
        }
        pu = wave_sum(pu);
        if (a.has_gate) pg = wave_sum(pg);
        if (lane == 0) {
          s_red[wave][2 * r] = pu;
          s_red[wave][2 * r + 1] = pg;
        }
      }
    }
    __syncthreads();
    if (tid < RN) {
      float u = 0.0f, gg = 0.0f, h = 0.0f;
      if (t0 + tid < m) {
#pragma unroll
        for (int ww = 0; ww < FU_NW; ++ww) {
          u += s_red[ww][2 * tid];
          gg += s_red[ww][2 * tid + 1];
        }
        u += bu;
        if (a.act == FFN_ACT_RELU) {
          h = fmaxf(u, 0.0f);
        } else {
          gg = fmaxf(gg + bgt, 0.0f);
          h = a.act == FFN_ACT_REGLU ? gg * u : gg * fmaxf(u, 0.0f);
        }
      }
      s_h[tid] = h;
    }
    __syncthreads();
    FFN_TS(1, 3);
#pragma unroll
    for (int r = 0; r < RN; ++r) {
      if (t0 + r < m) {                                  // uniform
      const float h = s_h[r];
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        if constexpr (WK == WK_F32) {
          const f32x4 q = __builtin_bit_cast(f32x4, wd[r][k]);
          acc[k][0] = __builtin_fmaf(h, q.x, acc[k][0]);
          acc[k][1] = __builtin_fmaf(h, q.y, acc[k][1]);
          acc[k][2] = __builtin_fmaf(h, q.z, acc[k][2]);
          acc[k][3] = __builtin_fmaf(h, q.w, acc[k][3]);
        } else {
          const uint32_t ww[4] = {wd[r][k].x, wd[r][k].y, wd[r][k].z, wd[r][k].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[k][2 * q] = __builtin_fmaf(h, h_lo(ww[q]), acc[k][2 * q]);
            acc[k][2 * q + 1] = __builtin_fmaf(h, h_hi(ww[q]), acc[k][2 * q + 1]);
          }
        }
      }
      }
    }
    __syncthreads();                                     // s_red / s_h reused
  }
  FFN_TS(1, 4);
  if (m > 0) {
    const int nparts = gridDim.x;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = tid + k * NT;
      if (c < nch) {
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
          float* dst = a.part + part_offset(c * EPC + e, blockIdx.x, nparts);
          __builtin_nontemporal_store(f32x4{acc[k][e], acc[k][e + 1], acc[k][e + 2], acc[k][e + 3]},
                                      reinterpret_cast<f32x4*>(dst));
        }
      }
    }
  }
  FFN_TRACE_SYNC();
  FFN_TS(1, 5);
  FFN_TV(1, 6, m);
}

// ---------------------------------------------------------------------------------------------
// y = b_down + sum of the gather partials, in workgroup order.  Workgroup j owns the RD_TW
// columns of tile j; the partials are stored tile-major, so it reads one contiguous block of
// GA_BLOCKS * RD_TW floats (every thread four 16-byte pieces at once).  Partials of gather
// workgroups that owned no rank were not written and are skipped (their ranges follow from |A|).
// Workgroup 0 also writes the ascending index list and the count when the caller asks for them.
constexpr int RD_THREADS = 256;
constexpr int RD_Q = RD_TW / 4;                        // float4 columns per tile
constexpr int RD_G = RD_THREADS / RD_Q;                // partial groups
constexpr int RD_UNROLL = 4;                           // partials per thread in flight

// MODE 0: one token, balanced gather (GA_BLOCKS partials, existence from |A| and the rank
// split); MODE 1: one token, fused variant (existence from the bitmap words); MODE 2: expert
// slots side by side (slot-major (slot, partial) items, routing-weighted).
template <int MODE>
__global__ __launch_bounds__(RD_THREADS) void k_reduce(ReduceArgs a) {
  __shared__ f32x4 s[RD_THREADS / WAVE][RD_Q];
  const int q = threadIdx.x % RD_Q;          // float4 column within the tile
  const int g = threadIdx.x / RD_Q;          // items g, g + RD_G, ...
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int tile = blockIdx.x;
  const int j = tile * RD_TW + q * 4;
  FFN_TS(2, 0);
  const int nslot = MODE == 2 ? a.nslot : 1;
  // b_down.  One layer: the load goes out now and is first used after the loop, so it does not
  // hold up the partials' loads.  Expert slots: each slot's routing weight, |A| and b_down come
  // from its record, all requested at once ahead of the partials (the weighted biases are added
  // after the loop: their loads depend on the records).
  f32x4 bias = {0.f, 0.f, 0.f, 0.f};
  float sw[MOE_MAX_K];
  uint32_t stot[MOE_MAX_K];
  const float* sbd[MOE_MAX_K];
  if constexpr (MODE == 2) {
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k) {
      const int kk = min(k, nslot - 1);
      sw[k] = a.slot[kk].wgt;
      sbd[k] = a.slot[kk].b_down;
      stot[k] = (uint32_t)a.cnt[(size_t)kk * a.cstride];
    }
  } else if (threadIdx.x < RD_Q && j < a.d && a.b_down) {
    bias = ldg(reinterpret_cast<const f32x4*>(a.b_down + j), 0);
  }
  const uint32_t np = MODE == 0 ? (uint32_t)GA_BLOCKS : (uint32_t)a.n_part;
  const uint32_t items = (uint32_t)nslot * np;
  const uint32_t total0 = MODE == 0 ? (uint32_t)a.cnt[0] : 0u;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // expert slots: nslot * n_part <= RD_G * RD_UNROLL (the gather's workgroups are shared between
  // the slots), so one pass, which lets the slots' constants arrive while the partials load
  const uint32_t passes = MODE == 2 ? 1u : (items + RD_G * RD_UNROLL - 1) / (RD_G * RD_UNROLL);
  for (uint32_t ip = 0; ip < passes; ++ip) {
    const uint32_t i0 = ip * RD_G * RD_UNROLL;
    f32x4 v[RD_UNROLL];
    float wt[RD_UNROLL];
    uint32_t ks[RD_UNROLL], cs[RD_UNROLL];
    // the partials' loads first (their addresses need no loaded value), then the weights
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) {
      const uint32_t it = min(i0 + g + u * RD_G, items - 1);
      ks[u] = MODE == 2 ? it / np : 0u;
      cs[u] = it - ks[u] * np;
      v[u] = *reinterpret_cast<const f32x4*>(a.part + (size_t)ks[u] * a.pstride +
                                             part_offset(tile * RD_TW + q * 4, cs[u], np));
    }
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) {
      const uint32_t k = ks[u], c = cs[u];
      // the slot's weight and |A| (a select over the slots, not a per-lane load)
      float wk = 1.0f;
      uint32_t total = total0;
      if constexpr (MODE == 2) {
        wk = sw[0];
        total = stot[0];
#pragma unroll
        for (int s2 = 1; s2 < MOE_MAX_K; ++s2) {
          wk = k == (uint32_t)s2 ? sw[s2] : wk;
          total = k == (uint32_t)s2 ? stot[s2] : total;
        }
      }
      bool on;
      if (MODE == 1) {
        on = (a.bitmap[2 * c] | (2 * c + 1 < (uint32_t)a.ffn / 32 ? a.bitmap[2 * c + 1] : 0u)) != 0u;
      } else {
        // partial c exists iff gather workgroup c owned at least one rank
        on = gather_wrote_partial(total, c, np);
      }
      on = on && i0 + g + u * RD_G < items;
      wt[u] = on ? wk : 0.0f;
    }
    issue_fence();
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) {
      // partials that were not written hold stale bytes: skipped, never multiplied by 0
      if (wt[u] != 0.0f) acc += MODE == 2 ? wt[u] * v[u] : v[u];
    }
  }
  if constexpr (MODE == 2) {
    if (threadIdx.x < RD_Q && j < a.d) {
#pragma unroll
      for (int k = 0; k < MOE_MAX_K; ++k)
        if (k < nslot && sbd[k]) bias += sw[k] * *reinterpret_cast<const f32x4*>(sbd[k] + j);
    }
  }
  // fixed-order tree over the groups: within each wave by lane exchange (lane = 4 g' + q), then
  // the waves' sums through LDS
#pragma unroll
  for (int o = RD_Q; o < WAVE; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o, WAVE);
    acc.y += __shfl_xor(acc.y, o, WAVE);
    acc.z += __shfl_xor(acc.z, o, WAVE);
    acc.w += __shfl_xor(acc.w, o, WAVE);
  }
  if (lane < RD_Q) s[wave][lane] = acc;
  __syncthreads();
  if (threadIdx.x < RD_Q && j < a.d) {
    f32x4 t = s[0][q];
#pragma unroll
    for (int w = 1; w < RD_THREADS / WAVE; ++w) t += s[w][q];
    *reinterpret_cast<f32x4*>(a.y + j) = t + bias;
  }
  if (MODE == 2) {
    // expert slots: each slot's |A| (written by the gather) in slot order
    if (blockIdx.x == 0 && a.cnt_out && (int)threadIdx.x < nslot)
      a.cnt_out[threadIdx.x] = a.cnt[(size_t)threadIdx.x * a.cstride];
  } else if (blockIdx.x == 0 && (a.idx_out || a.cnt_out)) {
    write_index_list<RD_THREADS>(a.bitmap, a.ffn / 32, a.idx_out, a.cnt_out);
  }
  FFN_TS(2, 5);
}

// ---------------------------------------------------------------------------------------------
// Host launchers.
#define CPL_SWITCH(cpl, F)                                                                    \
  switch (cpl) {                                                                              \
    case 1: return F(1); case 2: return F(2); case 3: return F(3); case 4: return F(4);       \
    case 6: return F(6); case 8: return F(8); case 12: return F(12); case 16: return F(16);   \
    default: return hipErrorInvalidValue;                                                     \
  }

template <int PK, int CPL>
static hipError_t launch_pred_z_t(const void* p1, const float* c1, const void* x, float* z,
                                  int d, int rank, const ExpertW* slot, int nslot, int zstride,
                                  hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid(rank, slot ? nslot : 1);
  if (ev0 && ev1)
    hipExtLaunchKernelGGL((k_pred_z<PK, CPL>), grid, dim3(WAVE), 0, st, ev0, ev1, 0, p1, c1, x,
                          z, d, rank, slot, zstride);
  else
    hipLaunchKernelGGL((k_pred_z<PK, CPL>), grid, dim3(WAVE), 0, st, p1, c1, x, z, d, rank, slot,
                       zstride);
  return hipGetLastError();
}

hipError_t launch_pred_z(int p_f16, int cpl, const void* p1, const float* c1, const void* x,
                         float* z, int d, int rank, const ExpertW* slot, int nslot, int zstride,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (p_f16) {
#define F16Z(c) launch_pred_z_t<WK_F16, c>(p1, c1, x, z, d, rank, slot, nslot, zstride, st, ev0, ev1)
    CPL_SWITCH(cpl, F16Z)
#undef F16Z
  } else {
#define F32Z(c) launch_pred_z_t<WK_F32, c>(p1, c1, x, z, d, rank, slot, nslot, zstride, st, ev0, ev1)
    CPL_SWITCH(cpl, F32Z)
#undef F32Z
  }
}

int pred_s_cpr(int p_f16, int rank) {
  const int pch = rank / (p_f16 ? 8 : 4);
  if (pch <= 64) return 1;
  if (pch <= 128) return 2;
  if (pch <= 256) return 4;
  return -1;
}

template <int PK, int CPR, int MAXP>
static hipError_t launch_pred_s_t(const PredArgs& a, hipStream_t st, hipEvent_t ev0,
                                  hipEvent_t ev1) {
  const dim3 grid(a.ffn / 32, a.slot ? a.nslot : 1);
  if (ev0 && ev1)
    hipExtLaunchKernelGGL((k_pred_s<PK, CPR, MAXP>), grid, dim3(PS_THREADS), 0, st, ev0, ev1, 0,
                          a);
  else
    hipLaunchKernelGGL((k_pred_s<PK, CPR, MAXP>), grid, dim3(PS_THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pred_s(int p_f16, const PredArgs& a, hipStream_t st, hipEvent_t ev0,
                         hipEvent_t ev1) {
  const int cpr = pred_s_cpr(p_f16, a.rank);
  const int pch = a.rank / (p_f16 ? 8 : 4);
  int L = 64;
  while (L > 4 && (L >> 1) >= pch) L >>= 1;
  const int passes = (32 * L + PS_THREADS - 1) / PS_THREADS;     // 1, 2, 4 or 8
#define PS_CASE(K, C, P) \
  if (cpr == C && passes == P) return launch_pred_s_t<K, C, P>(a, st, ev0, ev1);
  if (p_f16) {
    PS_CASE(WK_F16, 1, 1) PS_CASE(WK_F16, 1, 2) PS_CASE(WK_F16, 1, 4) PS_CASE(WK_F16, 1, 8)
    PS_CASE(WK_F16, 2, 8) PS_CASE(WK_F16, 4, 8)
  } else {
    PS_CASE(WK_F32, 1, 1) PS_CASE(WK_F32, 1, 2) PS_CASE(WK_F32, 1, 4) PS_CASE(WK_F32, 1, 8)
    PS_CASE(WK_F32, 2, 8) PS_CASE(WK_F32, 4, 8)
  }
#undef PS_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_mask_bits(const unsigned char* mask, uint32_t* bitmap, int words,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_mask_bits, dim3((words + 7) / 8), dim3(256), 0, st, mask, bitmap, words);
  return hipGetLastError();
}

// Threads per row of the gather kernel: the smallest multiple of 64 lanes, a power-of-two
// fraction of the workgroup, that covers the row's 16-byte chunks once or twice.
static int gather_slots(int nch) {
  int slots = 1;
  while (slots < 8 && GA_THREADS / (slots * 2) >= nch) slots *= 2;
  return slots;
}

// 16-byte chunks of a weight row per thread of the gather kernel
int gather_cpt(int wk, int d) {
  const int nch = d / (wk == WK_F32 ? 4 : wk == WK_F16 ? 8 : 32);
  const int tpr = GA_THREADS / gather_slots(nch);
  return (nch + tpr - 1) / tpr;
}
// Workgroups per gather launch and slot: expert slots running side by side share the GPU's
// one wave of resident workgroups.
int gather_blocks(int nslot) { return GA_BLOCKS / (nslot < 1 ? 1 : nslot); }

template <int WK, int CPT, int SLOTS, bool CACHED = false>
static hipError_t launch_gather_t(const GatherArgs& a, hipStream_t st, hipEvent_t ev0,
                                  hipEvent_t ev1) {
  // LDS for the slots' accumulator sum (dynamic: only multi-slot variants use it)
  const size_t lds = SLOTS > 1 ? (size_t)(SLOTS - 1) * (GA_THREADS / SLOTS) * CPT *
                                     Kind<WK>::EPC * sizeof(float) : 0;
  if (ev0 && ev1)
    hipExtLaunchKernelGGL((k_gather<WK, CPT, SLOTS, CACHED>),
                          dim3(gather_blocks(a.slot ? a.nslot : 1), a.slot ? a.nslot : 1),
                          dim3(GA_THREADS), lds, st, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL((k_gather<WK, CPT, SLOTS, CACHED>),
                       dim3(gather_blocks(a.slot ? a.nslot : 1), a.slot ? a.nslot : 1),
                       dim3(GA_THREADS), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_gather(int wk, const GatherArgs& a, hipStream_t st, hipEvent_t ev0,
                         hipEvent_t ev1) {
  const int nch = a.d / (wk == WK_F32 ? 4 : wk == WK_F16 ? 8 : 32);
  const int slots = gather_slots(nch);
  const int cpt = gather_cpt(wk, a.d);
#define GA_CASE(W, C, S) \
  if (cpt == C && slots == S) return launch_gather_t<W, C, S>(a, st, ev0, ev1);
  if (wk == WK_F32) {
    GA_CASE(WK_F32, 1, 1) GA_CASE(WK_F32, 2, 1) GA_CASE(WK_F32, 1, 2) GA_CASE(WK_F32, 1, 4)
    GA_CASE(WK_F32, 1, 8)
  } else if (wk == WK_F16) {
    GA_CASE(WK_F16, 1, 1) GA_CASE(WK_F16, 2, 1) GA_CASE(WK_F16, 1, 2) GA_CASE(WK_F16, 1, 4)
    GA_CASE(WK_F16, 1, 8)
  } else {
    GA_CASE(WK_I4, 1, 1) GA_CASE(WK_I4, 1, 2) GA_CASE(WK_I4, 1, 4) GA_CASE(WK_I4, 1, 8)
  }
#undef GA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gather_cached(const GatherArgs& a, hipStream_t st, hipEvent_t ev0,
                                hipEvent_t ev1) {
  const int nch = a.d / 8;
  const int slots = gather_slots(nch);
  const int cpt = gather_cpt(WK_F16, a.d);
#define GC_CASE(C, S) \
  if (cpt == C && slots == S) return launch_gather_t<WK_F16, C, S, true>(a, st, ev0, ev1);
  GC_CASE(1, 1) GC_CASE(2, 1) GC_CASE(1, 2) GC_CASE(1, 4) GC_CASE(1, 8)
#undef GC_CASE
  return hipErrorInvalidValue;
}

int reduce_tiles(int d) { return (d + RD_TW - 1) / RD_TW; }

int fused_blocks(int ffn) { return (ffn + FU_ROWS - 1) / FU_ROWS; }

// fp32 / fp16 rows of 64 to 1024 16-byte chunks (one or two chunks per thread; threads past a
// narrower row load a clamped chunk, multiply it by a zero token slice and store nothing)
bool fused_supported(int wk, int d) {
  if (wk == WK_I4) return false;
  const int nch = d / (wk == WK_F32 ? 4 : 8);
  return nch >= WAVE && nch <= 2 * FU_THREADS;
}

template <int WK, int CPT, int CPR>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t st, hipEvent_t ev0,
                                 hipEvent_t ev1) {
  const dim3 grid(fused_blocks(a.pa.ffn));
  if (ev0 && ev1)
    hipExtLaunchKernelGGL((k_fused<WK, CPT, CPR>), grid, dim3(FU_THREADS), 0, st, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL((k_fused<WK, CPT, CPR>), grid, dim3(FU_THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fused(int wk, const FusedArgs& a, hipStream_t st, hipEvent_t ev0,
                        hipEvent_t ev1) {
  if (!fused_supported(wk, a.ga.d)) return hipErrorInvalidValue;
  const int nch = a.ga.d / (wk == WK_F32 ? 4 : 8);
  const int cpt = (nch + FU_THREADS - 1) / FU_THREADS;
  const int cpr = pred_s_cpr(wk == WK_F16, a.pa.rank);
#define FU_CASE(W, C, R) \
  if (cpt == C && cpr == R) return launch_fused_t<W, C, R>(a, st, ev0, ev1);
  if (wk == WK_F32) {
    FU_CASE(WK_F32, 1, 1) FU_CASE(WK_F32, 1, 2) FU_CASE(WK_F32, 1, 4)
    FU_CASE(WK_F32, 2, 1) FU_CASE(WK_F32, 2, 2) FU_CASE(WK_F32, 2, 4)
  } else {
    FU_CASE(WK_F16, 1, 1) FU_CASE(WK_F16, 1, 2) FU_CASE(WK_F16, 1, 4)
    FU_CASE(WK_F16, 2, 1) FU_CASE(WK_F16, 2, 2) FU_CASE(WK_F16, 2, 4)
  }
#undef FU_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid(reduce_tiles(a.d)), block(RD_THREADS);
  auto kern = a.slot ? k_reduce<2> : a.fused ? k_reduce<1> : k_reduce<0>;
  if (!a.slot && !a.fused && a.n_part != GA_BLOCKS) return hipErrorInvalidValue;
  // expert slots: every (slot, partial) item in the reduce's one pass
  if (a.slot && (a.nslot < 1 || a.nslot > MOE_MAX_K ||
                 (long long)a.nslot * a.n_part > RD_G * RD_UNROLL))
    return hipErrorInvalidValue;
  if (ev0 && ev1)
    hipExtLaunchKernelGGL(kern, grid, block, 0, st, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL(kern, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace ffn
