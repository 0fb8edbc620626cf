// Self-attention block of one token with a head-level active set (gfx950, wave64).
//
// PowerInfer (unite.ai), section "Adaptive sparse predictor": besides the FFN's, every layer has a
// predictor for its self-attention block; section "Online stage": only what is predicted active
// is computed.  The unit predicted here is a head (its query rows, its scores over the cache and
// its rows of the transposed output projection); keys and values are made for every head, so
// the cache stays that of the dense model.  Per token, five launches on the caller's stream:
//   k_pred_z       z = P1 x + c1                      (the FFN's predictor stage 1, shared)
//   k_attn_proj    query rows of the active heads (by rank) and key / value rows of every
//                  key/value head, two rows per wave; every query workgroup first scores all
//                  heads itself (s = P2 z + c2, active iff s > logit(tau)) and ranks the active
//                  ones, so no launch sits between the predictor and the projections; keys and
//                  values go to the cache at the token's position (fp16), queries (fp32) to the
//                  workspace.  Query workgroups come first in dispatch order: their path is one
//                  round trip longer.
//   k_attn_part    per (active head, chunk of positions): scores, a running softmax and the
//                  weighted sum of values over the chunk -> the chunk's (o, max, sum)
//   k_attn_out     256 workgroups split the active heads' output-projection rows evenly by
//                  rank; each merges its heads' chunk records into o and adds one contiguous-row
//                  axpy per channel into its partial of y
//   k_attn_reduce  y = sum of the 256 partials in a fixed order
// No global atomics: y is bit-reproducible run to run.
#include <hip/hip_ext.h>
#include <math.h>

#include "common.h"
#include "index.h"
#include "launch.h"

namespace ffn {

constexpr int AP_THREADS = 256;           // k_attn_proj: 4 waves x 2 rows
constexpr int AP_ROWS = 8;
constexpr int AT_THREADS = 256;           // k_attn_part
constexpr int AO_THREADS = 256;           // k_attn_out
constexpr int AR_THREADS = 256;           // k_attn_reduce: 8 float4 columns x 32 groups of 8
constexpr int AT_UNROLL = 4;              // steps of k_attn_part whose loads are in flight at once

// Sum over aligned groups of W lanes (W a power of two, 2..64); valid in every lane for W <= 16,
// in the group's last lane for W = 32, 64.
template <int W>
__device__ __forceinline__ float lanes_sum(float v) {
  if constexpr (W >= 2) v += dpp<0xb1>(v);          // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp<0x4e>(v);          // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp<0x141>(v);         // row_half_mirror
  if constexpr (W >= 16) v += dpp<0x140>(v);        // row_mirror
  if constexpr (W >= 32) v += dpp<0x142, 0xa>(v);   // row_bcast15
  if constexpr (W >= 64) v += dpp<0x143, 0xc>(v);   // row_bcast31
  return v;
}

__device__ __forceinline__ void unpack8(u32x4 w, float (&f)[8]) {
  f[0] = h_lo(w.x); f[1] = h_hi(w.x); f[2] = h_lo(w.y); f[3] = h_hi(w.y);
  f[4] = h_lo(w.z); f[5] = h_hi(w.z); f[6] = h_lo(w.w); f[7] = h_hi(w.w);
}

// 8 fp16 weights times 8 fp32 values from LDS, fp32 accumulate.
__device__ __forceinline__ float dot8_hz(u32x4 w, const float* z, float acc) {
  float f[8];
  unpack8(w, f);
  const f32x4 za = *reinterpret_cast<const f32x4*>(z);
  const f32x4 zb = *reinterpret_cast<const f32x4*>(z + 4);
  acc = __builtin_fmaf(f[0], za.x, acc);
  acc = __builtin_fmaf(f[1], za.y, acc);
  acc = __builtin_fmaf(f[2], za.z, acc);
  acc = __builtin_fmaf(f[3], za.w, acc);
  acc = __builtin_fmaf(f[4], zb.x, acc);
  acc = __builtin_fmaf(f[5], zb.y, acc);
  acc = __builtin_fmaf(f[6], zb.z, acc);
  return __builtin_fmaf(f[7], zb.w, acc);
}

// ---------------------------------------------------------------------------------------------
// The head set, computed by one workgroup: bits of the active heads (128-bit, two words).  With a
// predictor, TPH lanes share one head: each takes every TPH-th 16-byte chunk of the head's P2 row
// against z (staged in LDS) and the group's sum is the head's score.  Workgroup 0 also writes
// the set's outputs (bitmap, ranked list, count, scores).
template <int TPH>
__device__ void head_set(const AttnArgs& a, unsigned long long& lo, unsigned long long& hi) {
  __shared__ float s_z[ATTN_MAX_RANK];
  __shared__ unsigned long long s_wm[AP_THREADS / WAVE];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  constexpr int HPW = WAVE / TPH;                   // heads per wave
  const int h = wave * HPW + lane / TPH, sub = lane % TPH;
  bool on = false;
  float s = 0.0f;
  if (a.mask) {
    on = sub == 0 && h < a.H && a.mask[h] != 0;
  } else {
    const int pch = a.rank / 8;                     // 16-byte chunks of a P2 row (fp16)
    const int hh = min(h, a.H - 1);
    const char* prow = static_cast<const char*>(a.p2) + (size_t)hh * a.rank * 2;
    // the first P2 chunks are requested before z is staged (independent round trips)
    constexpr int NPRE = 8;
    u32x4 pre[NPRE];
#pragma unroll
    for (int i = 0; i < NPRE; ++i) pre[i] = ld16(prow + (size_t)min(sub + i * TPH, pch - 1) * 16);
    for (int z0 = tid * 4; z0 < a.rank; z0 += AP_THREADS * 4)
      *reinterpret_cast<f32x4*>(&s_z[z0]) = ldg(reinterpret_cast<const f32x4*>(a.z), z0 / 4);
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NPRE; ++i)
      if (sub + i * TPH < pch) acc = dot8_hz(pre[i], &s_z[(sub + i * TPH) * 8], acc);
    for (int c = sub + NPRE * TPH; c < pch; c += TPH)
      acc = dot8_hz(ld16(prow + (size_t)c * 16), &s_z[c * 8], acc);
    acc = lanes_sum<TPH>(acc);
    // the group's sum sits in every lane for TPH <= 16, in its last lane otherwise
    const int src = TPH <= 16 ? lane : (lane | (TPH - 1));
    s = __shfl(acc, src, WAVE) + (a.c2 ? a.c2[hh] : 0.0f);
    on = sub == 0 && h < a.H && s > a.thr;
    if (blockIdx.x == 0 && a.scores_out && sub == 0 && h < a.H) a.scores_out[h] = s;
  }
  // ballot bit (lane) -> head bit (lane / TPH)
  const unsigned long long b = __ballot(on);
  unsigned long long m = 0;
#pragma unroll
  for (int g = 0; g < HPW; ++g) m |= ((b >> (g * TPH)) & 1ull) << g;
  if (lane == 0) s_wm[wave] = m;
  __syncthreads();
  lo = hi = 0;
#pragma unroll
  for (int w = 0; w < AP_THREADS / WAVE; ++w) {
    const int sh = w * HPW;                         // HPW <= 32: a wave's bits never straddle
    if (sh < 64) lo |= s_wm[w] << sh;
    else hi |= s_wm[w] << (sh - 64);
  }
  if (blockIdx.x == 0) {
    // outputs: bitmap words, the active heads in ascending order (= by rank) and their count
    if (tid < 4) a.bits[tid] = (uint32_t)((tid < 2 ? lo : hi) >> (32 * (tid & 1)));
    if (tid < a.H) {
      const bool act = tid < 64 ? (lo >> tid) & 1 : (hi >> (tid - 64)) & 1;
      if (act) {
        const int k = tid < 64 ? __popcll(lo & ((1ull << tid) - 1))
                               : __popcll(lo) + __popcll(hi & ((1ull << (tid - 64)) - 1));
        a.alist[k] = tid;
        if (a.idx_out) a.idx_out[k] = tid;
      }
    }
    if (tid == 0) {
      const int n = __popcll(lo) + __popcll(hi);
      *a.cnt = n;
      if (a.cnt_out) *a.cnt_out = n;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Projections.  Workgroups [0, H e / 8) compute query rows by rank (8 rows = 8 channels of one
// head); the rest compute key rows, then value rows, of every key/value head.
template <int CPL, int TPH>
__global__ __launch_bounds__(AP_THREADS) void k_attn_proj(AttnArgs a) {
  __shared__ float s_out[AP_ROWS];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int nch = a.d / 8;
  const int nqb = a.H * a.e / AP_ROWS;
  const bool is_q = (int)blockIdx.x < nqb;
  XRegs<WK_F16, CPL> xr;
  load_x<WK_F16, CPL>(xr, a.x, nch, lane);
  const void* W;
  int row0, k = 0;
  if (is_q) {
    unsigned long long lo, hi;
    head_set<TPH>(a, lo, hi);
    k = (int)blockIdx.x * AP_ROWS / a.e;            // rank of the head of this workgroup's rows
    if (k >= __popcll(lo) + __popcll(hi)) return;   // uniform over the workgroup
    // the head of rank k: the k-th set bit
    unsigned long long m = lo;
    int kk = k, base = 0;
    if (kk >= __popcll(lo)) {
      kk -= __popcll(lo);
      m = hi;
      base = 64;
    }
    for (int i = 0; i < kk; ++i) m &= m - 1;
    const int h = base + __builtin_ctzll(m);
    row0 = h * a.e + ((int)blockIdx.x * AP_ROWS) % a.e;
    W = a.wq;
  } else {
    const int r = ((int)blockIdx.x - nqb) * AP_ROWS;
    const int kv = a.G * a.e;
    W = r < kv ? a.wk : a.wv;
    row0 = r < kv ? r : r - kv;
  }
  u32x4 w0[CPL], w1[CPL];
  float sc[CPL];
  load_row<WK_F16, CPL>(w0, sc, W, nullptr, (size_t)row0 + 2 * wave, nch, lane);
  load_row<WK_F16, CPL>(w1, sc, W, nullptr, (size_t)row0 + 2 * wave + 1, nch, lane);
  issue_fence();
  finish_x<WK_F16, CPL>(xr, nch, lane);
  const float v0 = wave_sum(row_dot<WK_F16, CPL>(w0, sc, xr));
  const float v1 = wave_sum(row_dot<WK_F16, CPL>(w1, sc, xr));
  if (lane == 0) {
    s_out[2 * wave] = v0;
    s_out[2 * wave + 1] = v1;
  }
  __syncthreads();
  if (tid == 0) {
    if (is_q) {
      f32x4* q = reinterpret_cast<f32x4*>(a.q + (size_t)k * a.e + row0 % a.e);
      q[0] = f32x4{s_out[0], s_out[1], s_out[2], s_out[3]};
      q[1] = f32x4{s_out[4], s_out[5], s_out[6], s_out[7]};
    } else {
      const int r = ((int)blockIdx.x - nqb) * AP_ROWS;
      void* cache = r < a.G * a.e ? a.kc : a.vc;
      const int g = row0 / a.e, c0 = row0 % a.e;
      u32x4 pk;
      h2 t;
      t.x = (_Float16)s_out[0]; t.y = (_Float16)s_out[1]; pk.x = __builtin_bit_cast(uint32_t, t);
      t.x = (_Float16)s_out[2]; t.y = (_Float16)s_out[3]; pk.y = __builtin_bit_cast(uint32_t, t);
      t.x = (_Float16)s_out[4]; t.y = (_Float16)s_out[5]; pk.z = __builtin_bit_cast(uint32_t, t);
      t.x = (_Float16)s_out[6]; t.y = (_Float16)s_out[7]; pk.w = __builtin_bit_cast(uint32_t, t);
      *reinterpret_cast<u32x4*>(static_cast<_Float16*>(cache) +
                                ((size_t)g * a.S + a.pos) * a.e + c0) = pk;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Scores and values of one chunk of positions for one active head.  A position's e channels are
// read by LPR = e / 8 lanes (16 bytes each); a wave covers 64 / LPR positions per step and the
// workgroup 4 times that.  Each lane keeps a running (max, sum, o-slice) over the positions its
// lane row sees; rows, then waves, are merged at the end.
__device__ __forceinline__ void merge_run(float& m, float& l, float (&o)[8], float m2, float l2,
                                          const float (&o2)[8]) {
  const float M = fmaxf(m, m2);
  const float f1 = m == -INFINITY ? 0.0f : __expf(m - M);
  const float f2 = m2 == -INFINITY ? 0.0f : __expf(m2 - M);
  l = l * f1 + l2 * f2;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = o[i] * f1 + o2[i] * f2;
  m = M;
}

template <int E, bool PIPE>
__global__ __launch_bounds__(AT_THREADS) void k_attn_part(AttnArgs a) {
  constexpr int LPR = E / 8;                        // lanes per position
  constexpr int PPW = WAVE / LPR;                   // positions per wave and step
  constexpr int PB = PPW * (AT_THREADS / WAVE);     // positions per workgroup and step
  constexpr int U = AT_UNROLL;
  __shared__ float s_rec[AT_THREADS / WAVE][LPR][10];
  const int k = blockIdx.y;
  // |A| and the head of rank k requested together (an entry past |A| is stale and unused)
  const int n = *a.cnt;
  const int h = a.alist[k];
  if (k >= n) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int pg = lane / LPR, ci = lane % LPR;
  const int g = h / (a.H / a.G);
  const int j0 = (int)blockIdx.x * a.lc;
  const int j1 = min(j0 + a.lc, a.pos + 1);
  const char* kb = static_cast<const char*>(a.kc) + (size_t)g * a.S * E * 2 + ci * 16;
  const char* vb = static_cast<const char*>(a.vc) + (size_t)g * a.S * E * 2 + ci * 16;
  const f32x4 qa = ldg(reinterpret_cast<const f32x4*>(a.q + (size_t)k * E + ci * 8), 0);
  const f32x4 qb = ldg(reinterpret_cast<const f32x4*>(a.q + (size_t)k * E + ci * 8), 1);
  float m = -INFINITY, l = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // keys and values of U steps from position s0 (clamped to the chunk, so never predicated)
  auto load_batch = [&](u32x4 (&kr)[U], u32x4 (&vr)[U], int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t jj = (size_t)min(s0 + u * PB + wave * PPW + pg, j1 - 1);
      kr[u] = ld16(kb + jj * E * 2);
      vr[u] = ld16(vb + jj * E * 2);
    }
  };
  // the running softmax over those steps (positions past the chunk weigh nothing)
  auto run_batch = [&](const u32x4 (&kr)[U], const u32x4 (&vr)[U], int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool val = s0 + u * PB + wave * PPW + pg < j1;
      float kf[8], vf[8];
      unpack8(kr[u], kf);
      float dp = qa.x * kf[0];
      dp = __builtin_fmaf(qa.y, kf[1], dp);
      dp = __builtin_fmaf(qa.z, kf[2], dp);
      dp = __builtin_fmaf(qa.w, kf[3], dp);
      dp = __builtin_fmaf(qb.x, kf[4], dp);
      dp = __builtin_fmaf(qb.y, kf[5], dp);
      dp = __builtin_fmaf(qb.z, kf[6], dp);
      dp = __builtin_fmaf(qb.w, kf[7], dp);
      const float sc = lanes_sum<LPR>(dp) * a.scale;  // LPR <= 16: every lane of the row
      const float sv = val ? sc : -INFINITY;
      const float mn = fmaxf(m, sv);
      const float corr = mn == m ? 1.0f : __expf(m - mn);
      const float p = val ? __expf(sv - mn) : 0.0f;
      unpack8(vr[u], vf);
      l = __builtin_fmaf(l, corr, p);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = __builtin_fmaf(o[i], corr, p * vf[i]);
      m = mn;
    }
  };
  if constexpr (!PIPE) {
    for (int s0 = j0; s0 < j1; s0 += U * PB) {
      u32x4 kr[U], vr[U];
      load_batch(kr, vr, s0);
      issue_fence();
      run_batch(kr, vr, s0);
    }
  } else {
    // chunks of two batches or more: the next batch's loads are in flight while one is used
    u32x4 k0[U], v0[U], k1[U], v1[U];
    load_batch(k0, v0, j0);
    for (int s0 = j0; s0 < j1; s0 += 2 * U * PB) {
      load_batch(k1, v1, s0 + U * PB);
      issue_fence();
      run_batch(k0, v0, s0);
      load_batch(k0, v0, s0 + 2 * U * PB);
      issue_fence();
      run_batch(k1, v1, s0 + U * PB);
    }
  }
  // merge the wave's position rows (lanes with the same ci), fixed order
#pragma unroll
  for (int sh = LPR; sh < WAVE; sh <<= 1) {
    float o2[8];
    const float m2 = __shfl_xor(m, sh, WAVE), l2 = __shfl_xor(l, sh, WAVE);
#pragma unroll
    for (int i = 0; i < 8; ++i) o2[i] = __shfl_xor(o[i], sh, WAVE);
    merge_run(m, l, o, m2, l2, o2);
  }
  if (pg == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s_rec[wave][ci][i] = o[i];
    s_rec[wave][ci][8] = m;
    s_rec[wave][ci][9] = l;
  }
  __syncthreads();
  if (wave == 0 && pg == 0) {
    for (int w = 1; w < AT_THREADS / WAVE; ++w) {
      float o2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o2[i] = s_rec[w][ci][i];
      merge_run(m, l, o, s_rec[w][ci][8], s_rec[w][ci][9], o2);
    }
    float* rec = a.rec + attn_rec_offset(k, blockIdx.x, E, ATTN_MAX_CHUNKS);
    f32x4* ro = reinterpret_cast<f32x4*>(rec + ci * 8);
    ro[0] = f32x4{o[0], o[1], o[2], o[3]};
    ro[1] = f32x4{o[4], o[5], o[6], o[7]};
    if (ci == 0) {
      rec[E] = m;
      rec[E + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Output projection: workgroup b takes ranked rows [n e b / 256, n e (b+1) / 256) of the active
// heads' W_o_t rows (n = |A|; at most 64 rows, so at most two heads); thread t owns 16-byte
// column chunks t, t + 256, ... of every row.  The first rows' loads are issued before the
// channels' outputs are merged from the chunk records, so the merge hides under them: per head
// the chunks' maxima and sums are reduced by the whole workgroup, then each row's weighted sum
// over the chunks is split over 256 / rows threads and added up in a fixed order.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

template <int CPT>
__global__ __launch_bounds__(AO_THREADS) void k_attn_out(AttnArgs a) {
  constexpr int RB = 8;                             // rows whose loads are in flight at once
  constexpr int NW = AO_THREADS / WAVE;
  __shared__ float s_a[ATTN_OUT_MAXR];
  __shared__ int s_alist[ATTN_MAX_HEADS];
  __shared__ float s_f[2][ATTN_MAX_CHUNKS];
  __shared__ float s_red[2][NW][2];
  __shared__ float s_part[AO_THREADS];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int e = a.e, nch = a.d / 8, nc = a.nchunk;
  const int n = *a.cnt;
  if (tid < a.H) s_alist[tid] = a.alist[tid];       // entries past |A| are stale and unused
  int r0, r1;
  attn_out_rows(n * e, blockIdx.x, ATTN_OUT_BLOCKS, r0, r1);
  const int nr = r1 - r0;
  float* part = a.part + (size_t)blockIdx.x * a.d;
  if (nr == 0) {                                    // no rows: a zero partial (uniform branch)
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cc = tid + i * AO_THREADS;
      if (cc < nch) {
        f32x4* p = reinterpret_cast<f32x4*>(part + (size_t)cc * 8);
        __builtin_nontemporal_store(f32x4{0.0f, 0.0f, 0.0f, 0.0f}, p);
        __builtin_nontemporal_store(f32x4{0.0f, 0.0f, 0.0f, 0.0f}, p + 1);
      }
    }
    return;
  }
  const int k0 = r0 / e, k1 = (r1 - 1) / e;         // k1 <= k0 + 1
  // Requests before the first rows' loads (the load counter retires in order, so a value
  // requested after them could only be used once they have all landed): the heads' chunk maxima
  // and sums, and this thread's share of its row's channel values (row i, chunks j, j + tpr, ..)
  float m[2], l[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const float* rc = a.rec + attn_rec_offset(min(k0 + hh, k1), min(tid, nc - 1), e,
                                              ATTN_MAX_CHUNKS);
    m[hh] = rc[e];
    l[hh] = rc[e + 1];
  }
  const int tpr = AO_THREADS / nr;
  const int ri = tid % nr, rj = tid / nr;
  const int rrow = r0 + ri, rhh = rrow / e - k0;
  const float* rco = a.rec + attn_rec_offset(rrow / e, 0, e, ATTN_MAX_CHUNKS) + rrow % e;
  constexpr int NPRE = 2;
  float ov[NPRE];
#pragma unroll
  for (int u = 0; u < NPRE; ++u) ov[u] = rco[(size_t)min(rj + u * tpr, nc - 1) * (e + 4)];
  __syncthreads();                                  // s_alist
  u32x4 w[RB][CPT];
  auto issue = [&](int rb) {
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int row = r0 + min(rb + u, nr - 1);
      const char* rp = static_cast<const char*>(a.wo) +
                       (size_t)(s_alist[row / e] * e + row % e) * nch * 16;
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        w[u][i] = ld16(rp + (size_t)min(tid + i * AO_THREADS, nch - 1) * 16);
    }
  };
  issue(0);
  // per head: M = max over the chunks, f_ch = exp(m_ch - M), L = sum l_ch f_ch
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const float v = wave_max(tid < nc ? m[hh] : -INFINITY);
    if (lane == 0) s_red[hh][wave][0] = v;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float M = s_red[hh][0][0];
#pragma unroll
    for (int q = 1; q < NW; ++q) M = fmaxf(M, s_red[hh][q][0]);
    const float f = tid < nc ? __expf(m[hh] - M) : 0.0f;
    if (tid < nc) s_f[hh][tid] = f;
    const float sl = wave_sum(l[hh] * f);
    if (lane == 0) s_red[hh][wave][1] = sl;
  }
  __syncthreads();
  // each row's weighted sum over the chunks, tpr threads per row, then in a fixed order
  if (tid < nr * tpr) {
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < NPRE; ++u)
      if (rj + u * tpr < nc) acc = __builtin_fmaf(ov[u], s_f[rhh][rj + u * tpr], acc);
    for (int ch = rj + NPRE * tpr; ch < nc; ch += tpr)
      acc = __builtin_fmaf(rco[(size_t)ch * (e + 4)], s_f[rhh][ch], acc);
    s_part[tid] = acc;
  }
  __syncthreads();
  if (tid < nr) {
    const int hh = (r0 + tid) / e - k0;
    float acc = s_part[tid];
    for (int j = 1; j < tpr; ++j) acc += s_part[j * nr + tid];
    float L = s_red[hh][0][1];
#pragma unroll
    for (int q = 1; q < NW; ++q) L += s_red[hh][q][1];
    s_a[tid] = acc / L;
  }
  __syncthreads();
  float acc[CPT][8];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  for (int rb = 0; rb < nr; rb += RB) {
    if (rb) issue(rb);
    issue_fence();
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const float coef = rb + u < nr ? s_a[rb + u] : 0.0f;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        float f[8];
        unpack8(w[u][i], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(coef, f[j], acc[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int cc = tid + i * AO_THREADS;
    if (cc < nch) {
      f32x4* p = reinterpret_cast<f32x4*>(part + (size_t)cc * 8);
      __builtin_nontemporal_store(f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]}, p);
      __builtin_nontemporal_store(f32x4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]}, p + 1);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// y = sum of the ATTN_OUT_BLOCKS partials: a workgroup per 8 float4 columns; thread (group gi,
// column ci) sums partials 8 gi .. 8 gi + 7, then the 32 groups are summed in order.
__global__ __launch_bounds__(AR_THREADS) void k_attn_reduce(AttnArgs a) {
  __shared__ f32x4 s_red[AR_THREADS / 8][8];
  const int tid = threadIdx.x, ci = tid & 7, gi = tid >> 3;
  const int n4 = a.d / 4;
  const int col = (int)blockIdx.x * 8 + ci;
  const int cc = min(col, n4 - 1);
  const f32x4* part = reinterpret_cast<const f32x4*>(a.part);
  f32x4 v[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) v[p] = ldg(part, (size_t)(gi * 8 + p) * n4 + cc);
  f32x4 s = v[0];
#pragma unroll
  for (int p = 1; p < 8; ++p) s += v[p];
  s_red[gi][ci] = s;
  __syncthreads();
  if (gi == 0 && col < n4) {
    f32x4 t = s_red[0][ci];
    for (int q = 1; q < AR_THREADS / 8; ++q) t += s_red[q][ci];
    reinterpret_cast<f32x4*>(a.y)[col] = t;
  }
}

static_assert(ATTN_OUT_BLOCKS == (AR_THREADS / 8) * 8, "k_attn_reduce sums 32 groups of 8");

// ---------------------------------------------------------------------------------------------
template <int CPL, int TPH>
static hipError_t launch_proj_t(const AttnArgs& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const int grid = (a.H + 2 * a.G) * a.e / AP_ROWS;
  if (e0 && e1)
    hipExtLaunchKernelGGL((k_attn_proj<CPL, TPH>), dim3(grid), dim3(AP_THREADS), 0, st, e0, e1, 0,
                          a);
  else
    hipLaunchKernelGGL((k_attn_proj<CPL, TPH>), dim3(grid), dim3(AP_THREADS), 0, st, a);
  return hipGetLastError();
}

template <int CPL>
static hipError_t launch_proj_c(const AttnArgs& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  // lanes per head: 64 / (heads per wave), heads per wave = the power of two >= H / 4
  const int hpw = attn_heads_per_wave(a.H);
  switch (WAVE / hpw) {
    case 2: return launch_proj_t<CPL, 2>(a, st, e0, e1);
    case 4: return launch_proj_t<CPL, 4>(a, st, e0, e1);
    case 8: return launch_proj_t<CPL, 8>(a, st, e0, e1);
    case 16: return launch_proj_t<CPL, 16>(a, st, e0, e1);
    case 32: return launch_proj_t<CPL, 32>(a, st, e0, e1);
    case 64: return launch_proj_t<CPL, 64>(a, st, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

int attn_heads_per_wave(int H) {
  int hpw = 1;
  while (hpw * (AP_THREADS / WAVE) < H) hpw <<= 1;
  return hpw;
}

hipError_t launch_attn_proj(int cpl, const AttnArgs& a, hipStream_t st, hipEvent_t e0,
                            hipEvent_t e1) {
  switch (cpl) {
    case 1: return launch_proj_c<1>(a, st, e0, e1);
    case 2: return launch_proj_c<2>(a, st, e0, e1);
    case 3: return launch_proj_c<3>(a, st, e0, e1);
    case 4: return launch_proj_c<4>(a, st, e0, e1);
    case 6: return launch_proj_c<6>(a, st, e0, e1);
    case 8: return launch_proj_c<8>(a, st, e0, e1);
    case 12: return launch_proj_c<12>(a, st, e0, e1);
    case 16: return launch_proj_c<16>(a, st, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

int attn_step_positions(int e) { return (WAVE / (e / 8)) * (AT_THREADS / WAVE); }

hipError_t launch_attn_part(const AttnArgs& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(a.nchunk, a.H);
  // two batches of loads in flight once a chunk holds two batches or more
  const bool pipe = a.lc >= 2 * AT_UNROLL * attn_step_positions(a.e);
#define ATT_L(E, P)                                                                            \
  do {                                                                                         \
    if (e0 && e1)                                                                              \
      hipExtLaunchKernelGGL((k_attn_part<E, P>), grid, dim3(AT_THREADS), 0, st, e0, e1, 0, a); \
    else                                                                                       \
      hipLaunchKernelGGL((k_attn_part<E, P>), grid, dim3(AT_THREADS), 0, st, a);               \
  } while (0)
  if (a.e == 64 && pipe) ATT_L(64, true);
  else if (a.e == 64) ATT_L(64, false);
  else if (a.e == 128 && pipe) ATT_L(128, true);
  else if (a.e == 128) ATT_L(128, false);
  else return hipErrorInvalidValue;
#undef ATT_L
  return hipGetLastError();
}

hipError_t launch_attn_out(const AttnArgs& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const int nch = a.d / 8;
  const int cpt = (nch + AO_THREADS - 1) / AO_THREADS;
#define ATO_L(C)                                                                               \
  do {                                                                                         \
    if (e0 && e1)                                                                              \
      hipExtLaunchKernelGGL((k_attn_out<C>), dim3(ATTN_OUT_BLOCKS), dim3(AO_THREADS), 0, st,   \
                            e0, e1, 0, a);                                                     \
    else                                                                                       \
      hipLaunchKernelGGL((k_attn_out<C>), dim3(ATTN_OUT_BLOCKS), dim3(AO_THREADS), 0, st, a);  \
  } while (0)
  if (cpt == 1) ATO_L(1);
  else if (cpt == 2) ATO_L(2);
  else if (cpt <= 4) ATO_L(4);
  else return hipErrorInvalidValue;
#undef ATO_L
  return hipGetLastError();
}

hipError_t launch_attn_reduce(const AttnArgs& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const int grid = (a.d / 4 + 7) / 8;
  if (e0 && e1)
    hipExtLaunchKernelGGL(k_attn_reduce, dim3(grid), dim3(AR_THREADS), 0, st, e0, e1, 0, a);
  else
    hipLaunchKernelGGL(k_attn_reduce, dim3(grid), dim3(AR_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace ffn
