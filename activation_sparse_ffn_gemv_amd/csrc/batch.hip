// Batched path of the activation-sparse FFN on gfx950 (fp16 layers, 2..32 tokens per pass).
//
// Every token keeps its own active set; the rows read are those of the union U of the tokens'
// sets, each read once per pass (nearauto.com, experiments, Fig. 14: batches; the pages' method
// per token is the neuron-aware operator of PowerInfer, unite.ai "神经元感知运算符").  With up to
// 32 tokens the per-row work is a skinny matrix product, so the contractions run on the MFMA
// units (32x32 tiles, M = the pass's tokens, zero-padded):
//   k_bz     Z = X P1^T, split over K            (predictor stage 1; partial sums per K slice)
//   k_bzr    z = sum of the K slices + c1, split into fp16 hi + lo parts (z = hi + lo to ~2^-22)
//   k_bs     S = Z P2^T + c2 (hi and lo MFMAs) for 128 neurons per workgroup, Z streamed through
//            LDS; per-token bitmap words by ballot; union words
//   k_bug    for 32 union neurons (by rank) per workgroup: U = X W_up^T, G = X W_gate^T;
//            h = act(u, g), zero where the token's own set excludes the neuron; H in fp16
//   k_bdown  Y_s = H[:, seg s] W_down_t[U_s]: split over union segments and 256-column tiles
//   k_bred   y = b_down + sum_s Y_s in segment order; per-token index lists and counts
// The fp16 rounding of h (relative 2^-11 per term) is the only precision given up against the
// batch-1 path.  No global atomics: the result is reproducible.
//
// MFMA lane layout (v_mfma_f32_32x32x16_f16 / 32x32x8_f16): lane l supplies row (l % 32) of A
// and column (l % 32) of B, each with the K elements 8*(l/32) .. +7 (x16) or 4*(l/32) .. +3
// (x8); accumulator element i of lane l is D[8*(i/4) + 4*(l/32) + i%4][l % 32].
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.h"
#include "index.h"
#include "launch.h"

namespace ffn {

constexpr int MB = BATCH_TILE;     // tokens per pass
constexpr int BT = 256;            // threads per workgroup: 4 waves
constexpr int BZ_GRP = 16;         // predictor stage 1: 16-k steps whose loads are issued together
constexpr int DN_CH = 512;         // union ranks staged in LDS at a time by k_bdown
constexpr int DN_COLS = 256;       // columns of y per k_bdown workgroup
constexpr int GRPD = 4;            // 8-rank steps whose loads k_bdown issues together

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mma16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, a),
                                                __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma8(u32x2 a, u32x2 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(h4v, a),
                                              __builtin_bit_cast(h4v, b), c, 0, 0, 0);
}

// Sum of the four waves' 32x32 accumulators in wave order; the result is valid in wave 0.
__device__ __forceinline__ f32x16 wg_sum4(f32x16 acc, float* red /* [3][16][64] */) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  __syncthreads();                      // red may still be read by a previous call
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[((wave - 1) * 16 + i) * WAVE + lane] = acc[i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += red[(w * 16 + i) * WAVE + lane];
  }
  return acc;
}

// Pass p of a multi-pass launch (by default blockIdx.z): the pass's tokens, buffers and count.
__device__ __forceinline__ void at_pass(BatchArgs& a, int p = blockIdx.z) {
  if (a.Btot > 0) a.B = min(MB, a.Btot - p * MB);      // (Btot 0: a one-pass launch)
  if (p == 0) return;
  const PassOffsets o = pass_offsets(p, MB, a.zpart_ps, a.zhl_ps, a.ubits_ps, a.uidx_ps,
                                     a.ypart_ps);
  a.x = static_cast<const char*>(a.x) + o.tok * a.d * 2;
  if (a.mask) a.mask += o.tok * a.ffn;
  a.bits += o.tok * (a.ffn / 32);
  if (a.scores) a.scores += o.tok * a.ffn;
  a.y += o.tok * a.d;
  if (a.idx_out) a.idx_out += o.tok * a.ffn;
  if (a.cnt_out) a.cnt_out += o.tok;
  a.zpart += o.zpart;
  a.zhl += o.zhl;
  a.ubits += o.ubits;
  a.ucnt += o.ucnt;
  a.uidx += o.uidx;
  a.H += o.tok * a.ffn;
  a.ypart += o.ypart;
}

// ---------------------------------------------------------------------------------------------
// Predictor stage 1: workgroup (tile of 32 P1 rows, K slice); wave w of slice k takes 16-k
// steps [(4k + w) * spw, ... + spw).
// Grid: one dimension of (P1 tile, K slice) blocks times passes (xcd_block_pass).
__global__ __launch_bounds__(BT) void k_bz(BatchArgs a) {
  const int tiles = (a.r + 31) / 32;
  int bx, pass;
  xcd_block_pass(blockIdx.x, tiles * a.ks, gridDim.x / (tiles * a.ks), bx, pass);
  at_pass(a, pass);
  const int tile = bx % tiles, slice = bx / tiles;
  __shared__ float red[3 * 16 * WAVE];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int n0 = tile * 32, row = lane & 31, g = lane >> 5;
  const int nchk = a.d / 8, nsteps = (nchk + 1) / 2;
  const int s0 = (slice * 4 + wave) * a.spw, s1 = min(nsteps, s0 + a.spw);
  const bool pok = n0 + row < a.r, xok = row < a.B;
  const char* pr = static_cast<const char*>(a.p1) + (size_t)min(n0 + row, a.r - 1) * a.d * 2;
  const char* xr = static_cast<const char*>(a.x) + (size_t)min(row, a.B - 1) * a.d * 2;
  f32x16 acc = {};
  for (int s = s0; s < s1; s += BZ_GRP) {
    u32x4 av[BZ_GRP], bv[BZ_GRP];
#pragma unroll
    for (int j = 0; j < BZ_GRP; ++j) {
      av[j] = bv[j] = u32x4{0u, 0u, 0u, 0u};
      if (s + j < s1) {                                   // uniform across the wave
        const int c = 2 * (s + j) + g;
        const int cc = min(c, nchk - 1);
        const u32x4 bl = ld16(pr + (size_t)cc * 16);
        const u32x4 al = ld16(xr + (size_t)cc * 16);
        bv[j] = (c < nchk && pok) ? bl : u32x4{0u, 0u, 0u, 0u};
        av[j] = (c < nchk && xok) ? al : u32x4{0u, 0u, 0u, 0u};
      }
    }
    issue_fence();
#pragma unroll
    for (int j = 0; j < BZ_GRP; ++j)
      if (s + j < s1) acc = mma16(av[j], bv[j], acc);
  }
  acc = wg_sum4(acc, red);
  if (wave == 0 && n0 + row < a.r) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      a.zpart[((size_t)slice * MB + acc_row(i, lane)) * a.r + n0 + row] = acc[i];
  }
}

// z = sum over the K slices (in order) + c1, stored as fp16 hi and lo planes.
__global__ __launch_bounds__(256) void k_bzr(BatchArgs a) {
  at_pass(a);
  const int e = blockIdx.x * 256 + threadIdx.x;       // m * r + k
  if (e >= MB * a.r) return;
  const int k = e % a.r;
  float z = 0.0f;
  // split-K slices in order, eight loads in flight at a time
  for (int q0 = 0; q0 < a.ks; q0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = q0 + u < a.ks ? a.zpart[(size_t)(q0 + u) * MB * a.r + e] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < a.ks) z += v[u];
  }
  if (a.c1) z += a.c1[k];
  const _Float16 hi = (_Float16)z;
  const _Float16 lo = (_Float16)(z - (float)hi);
  a.zhl[e] = hi;
  a.zhl[(size_t)MB * a.r + e] = lo;
  const int m = e / a.r;                                 // token of the pass
  if (a.zcat && m < a.B) {
    // the call's token (pass offset applied to x above): row of [hi | lo]
    const size_t row = (size_t)blockIdx.z * MB + m;
    a.zcat[row * 2 * a.r + k] = hi;
    a.zcat[row * 2 * a.r + a.r + k] = lo;
  }
}

// Predictor stage 2 for 128 neurons (four bitmap words per token) per workgroup:
// S = Z P2^T + c2.  Eight waves: waves w and w + 4 own the 32 neurons of word 4 b + w, each
// taking half of every chunk's rank steps (their two sums are added once, at the end).  Both
// operands stream through LDS in chunks of BS_KC ranks, loaded with whole contiguous row pieces
// (a wave's load instruction covers four P2 rows' 256 bytes), the next two chunks in flight
// while the current chunk's MFMAs run.
constexpr int BS_T = 512;                  // threads: 8 waves
constexpr int BS_N = 128;                  // neurons per workgroup
constexpr int BS_KC = 128;                 // ranks per chunk
constexpr int BS_PC = BS_KC / 8;           // 16-byte pieces of a row per chunk (16)
constexpr int BS_SW = BS_PC / 4;           // MFMA steps per wave and chunk (4: half the chunk)
constexpr int BS_LD = BS_PC + 1;           // padded LDS row
constexpr int BS_ZL = 2 * MB * BS_PC / BS_T;   // Z pieces per thread and chunk (2)
constexpr int BS_PL = BS_N * BS_PC / BS_T;     // P2 pieces per thread and chunk (4)

// Grid: one dimension of 128-neuron blocks times passes (xcd_block_pass).
__global__ __launch_bounds__(BS_T) void k_bs(BatchArgs a) {
  const int W = a.ffn / 32;
  const int nblk = (W + 3) / 4;
  int bx, pass;
  xcd_block_pass(blockIdx.x, nblk, gridDim.x / nblk, bx, pass);
  at_pass(a, pass);
  __shared__ u32x4 s_z[2][2][MB * BS_LD];  // [buffer][hi, lo][token row][piece]
  __shared__ u32x4 s_p[2][BS_N * BS_LD];   // [buffer][neuron][piece]
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int tw = wave & 3, kh = wave >> 2; // word of the workgroup, half of each chunk
  const int word = bx * 4 + tw;
  const bool head = word < a.head_words;   // hot head: every token's word set, no score
  const bool live = word < W && !head;     // uniform per wave
  if (kh == 0 && word < W && head) {
    if (lane < min(a.B, MB)) a.bits[(size_t)lane * W + word] = ~0u;
    if (lane == 0) a.ubits[word] = ~0u;
  }
  const int nb = bx * BS_N;                // first neuron of the workgroup
  const int row = lane & 31, g = lane >> 5;
  const int rch = a.r / 8;
  const int nchunk = (rch + BS_PC - 1) / BS_PC;
  const char* zb = reinterpret_cast<const char*>(a.zhl);
  const char* pb = static_cast<const char*>(a.p2);

  // Raw loads (clamped addresses, never predicated); what lies past the rank or the layer is
  // zeroed on the way into LDS, so that no load has to land before the loop turns.
  auto load = [&](int c, u32x4 (&z)[BS_ZL], u32x4 (&p)[BS_PL]) {
#pragma unroll
    for (int i = 0; i < BS_ZL; ++i) {
      const int e = tid + BS_T * i;        // (hl, token row, piece)
      const int hl = e / (MB * BS_PC), zr = (e / BS_PC) % MB, zc = e % BS_PC;
      const int pc = c * BS_PC + zc;
      z[i] = ld16(zb + (((size_t)hl * MB + zr) * a.r) * 2 + (size_t)min(pc, rch - 1) * 16);
    }
#pragma unroll
    for (int i = 0; i < BS_PL; ++i) {
      const int e = tid + BS_T * i;        // (neuron, piece)
      const int n = nb + e / BS_PC, pc = c * BS_PC + e % BS_PC;
      p[i] = ld16(pb + ((size_t)min(n, a.ffn - 1) * rch + min(pc, rch - 1)) * 16);
    }
  };
  auto store = [&](int buf, int c, const u32x4 (&z)[BS_ZL], const u32x4 (&p)[BS_PL]) {
#pragma unroll
    for (int i = 0; i < BS_ZL; ++i) {
      const int e = tid + BS_T * i;
      const int hl = e / (MB * BS_PC), zr = (e / BS_PC) % MB, zc = e % BS_PC;
      s_z[buf][hl][zr * BS_LD + zc] = c * BS_PC + zc < rch ? z[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < BS_PL; ++i) {
      const int e = tid + BS_T * i;
      const bool ok = nb + e / BS_PC < a.ffn && c * BS_PC + e % BS_PC < rch;
      s_p[buf][(e / BS_PC) * BS_LD + e % BS_PC] = ok ? p[i] : u32x4{0u, 0u, 0u, 0u};
    }
  };

  // Loads run two chunks ahead; LDS holds the current chunk and the next one.  The two register
  // sets swap roles by name each turn (chunk c+1 held for LDS in zh/qh, chunk c+2 arriving in
  // zr/qr), never by copy: copying a register that a load is still filling waits for the load.
  // Loads and LDS stores are unconditional (the last two turns re-read the last chunk, from L2,
  // and the last store writes zeros): a branch around either would merge a path with other
  // loads in flight, and the waits would then cover this turn's loads too.
  f32x16 acc = {};
  u32x4 zA[BS_ZL], zB[BS_ZL], qA[BS_PL], qB[BS_PL];
  load(0, zB, qB);
  load(min(1, nchunk - 1), zA, qA);
  store(0, 0, zB, qB);
  __syncthreads();
  auto step = [&](int c, const u32x4 (&zh)[BS_ZL], const u32x4 (&qh)[BS_PL], u32x4 (&zn)[BS_ZL],
                  u32x4 (&qn)[BS_PL]) {
    const int buf = c & 1;
    load(min(c + 2, nchunk - 1), zn, qn);
    issue_fence();                         // the loads go out first
    if (live) {
#pragma unroll
      for (int s = 0; s < BS_SW; ++s) {
        const int pcs = 2 * (kh * BS_SW + s) + g;
        const u32x4 ah = s_z[buf][0][row * BS_LD + pcs];
        const u32x4 al = s_z[buf][1][row * BS_LD + pcs];
        const u32x4 bv = s_p[buf][(tw * 32 + row) * BS_LD + pcs];
        acc = mma16(ah, bv, acc);
        acc = mma16(al, bv, acc);
      }
    }
    store(buf ^ 1, c + 1, zh, qh);         // past the last chunk: zeros nobody reads
    __syncthreads();
  };
  // pairs in the loop, an odd last chunk after it (an exit between the two steps would join the
  // loop head with loads in other registers in flight, and the head would wait for them all)
  int c0 = 0;
  for (; c0 + 2 <= nchunk; c0 += 2) {
    step(c0, zA, qA, zB, qB);
    step(c0 + 1, zB, qB, zA, qA);
  }
  if (c0 < nchunk) step(c0, zA, qA, zB, qB);
  // the second half's sums join the first's (the Z buffers are free now)
  float* red = reinterpret_cast<float*>(&s_p[0][0]);      // [4 words][16][64]
  static_assert(sizeof(s_p) >= 4 * 16 * WAVE * sizeof(float), "sums fit in the P2 buffers");
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(tw * 16 + i) * WAVE + lane] = acc[i];
  }
  __syncthreads();
  if (kh == 0 && live) {
    const int n0 = word * 32;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += red[(tw * 16 + i) * WAVE + lane];
    const float c2v = a.c2 ? a.c2[n0 + row] : 0.0f;
    uint32_t uw = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = acc_row(i, lane);
      const float sc = acc[i] + c2v;
      const bool on = sc > a.thr && m < a.B;
      if (a.scores && m < a.B) a.scores[(size_t)m * a.ffn + n0 + row] = sc;
      const unsigned long long bal = __ballot(on);
      const int m0 = 8 * (i >> 2) + (i & 3);          // lanes 0..31: token m0; 32..63: m0 + 4
      // rows of tokens past B are never read (and may lie past the caller's bitmap rows)
      if (lane == 0 && m0 < a.B) a.bits[(size_t)m0 * W + word] = (uint32_t)bal;
      if (lane == 32 && m0 + 4 < a.B) a.bits[(size_t)(m0 + 4) * W + word] = (uint32_t)(bal >> 32);
      uw |= (uint32_t)bal | (uint32_t)(bal >> 32);
    }
    if (lane == 0) a.ubits[word] = uw;
  }
}

// Caller masks -> per-token bitmap words and the union words (one thread per word).
__global__ __launch_bounds__(256) void k_bmask(BatchArgs a) {
  at_pass(a);
  const int w = blockIdx.x * 256 + threadIdx.x;
  const int W = a.ffn / 32;
  if (w >= W) return;
  uint32_t uw = 0u;
  for (int m = 0; m < a.B; ++m) {
    uint32_t bw = 0u;
    {
      if (a.mask) {
        const u32x4* mp = reinterpret_cast<const u32x4*>(a.mask + (size_t)m * a.ffn + w * 32);
        const u32x4 q0 = mp[0], q1 = mp[1];
        const uint32_t v[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if ((v[k] >> (8 * t)) & 0xffu) bw |= 1u << (4 * k + t);
      } else {
        bw = 0xffffffffu;                               // dense: every neuron
      }
    }
    a.bits[(size_t)m * W + w] = bw;
    uw |= bw;
  }
  a.ubits[w] = uw;
}

// Path choice on the device (nearauto.com / citnews.com.cn: prefill, where most neurons fire,
// runs dense; decode runs sparse): when the union holds more than dense_above neurons, the pass
// reads every neuron's rows; each token's h is still zeroed outside its own set, so the result
// is the same either way.
__global__ __launch_bounds__(1024) void k_bpath(BatchArgs a) {
  at_pass(a);
  __shared__ int s_total;
  if (a.run_if && *a.run_if != a.run_want) return;
  const int W = a.ffn / 32;
  const int w = threadIdx.x;                            // W <= 1024
  if (w == 0) s_total = 0;
  __syncthreads();
  if (w < W) atomicAdd(&s_total, __popc(a.ubits[w]));   // LDS atomic
  __syncthreads();
  if (s_total > a.dense_above && w < W) a.ubits[w] = 0xffffffffu;
}

// Union words of the pass's tokens from their bitmap words (bits written by an earlier step).
__global__ __launch_bounds__(256) void k_bunion(BatchArgs a) {
  at_pass(a);
  if (a.run_if && *a.run_if != a.run_want) return;
  const int w = blockIdx.x * 256 + threadIdx.x, W = a.ffn / 32;
  if (w >= W) return;
  uint32_t uw = 0u;
  for (int m = 0; m < a.B; ++m) uw |= a.bits[(size_t)m * W + w];
  a.ubits[w] = uw;
}

// Dense-or-sparse for a whole call: the union of its passes' union words against dense_above.
__global__ __launch_bounds__(1024) void k_dchoice(const uint32_t* __restrict__ ubits,
                                                  int passes, int W, int dense_above,
                                                  int* __restrict__ flag) {
  __shared__ int s_total;
  const int w = threadIdx.x;                            // W <= 1024
  if (w == 0) s_total = 0;
  __syncthreads();
  if (w < W) {
    uint32_t uw = 0u;
    for (int p0 = 0; p0 < passes; p0 += 8) {            // eight loads in flight at a time
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ubits[(size_t)min(p0 + u, passes - 1) * W + w];
#pragma unroll
      for (int u = 0; u < 8; ++u) uw |= v[u];           // a repeated last word changes nothing
    }
    atomicAdd(&s_total, __popc(uw));                    // LDS atomic
  }
  __syncthreads();
  if (w == 0) *flag = s_total > dense_above ? 1 : 0;
}

// Rows of NN union neurons (ranks [NN b, NN b + NN)): u, g on the MFMA units, then h.
// The rows stream through LDS in stages of UG_KC 16-byte chunks (a wave's load instruction
// covers two rows' 512 contiguous bytes), double-buffered; the waves split each stage's K
// between them for the MFMAs, and their 32x32 sums are added in wave order at the end.
constexpr int UG_KC = 32;                 // chunks per row per stage (256 k)
constexpr int UG_LD = UG_KC + 1;          // padded LDS row
constexpr int UG_WIDE_B = 16;             // ReLU batches above this take 64 neurons per workgroup

// NN = 32 or 64 neurons per workgroup (64: each token slice read from L2 serves twice the rows).
template <bool GATE, int NN>
__global__ __launch_bounds__(BT) void k_bug(BatchArgs a) {
  at_pass(a);
  constexpr int NMAT = GATE ? 2 : 1;
  constexpr int NTL = NN / 32;            // 32-neuron MFMA tiles
  constexpr int LPT = NN * UG_KC / BT;    // chunk loads per thread and matrix per stage
  __shared__ int s_wsum[BT / WAVE];
  __shared__ int s_nid[NN];
  // the row stages; after the last stage the same bytes hold the waves' sums (keeping the LDS
  // per workgroup small enough for four resident workgroups per CU)
  __shared__ u32x4 s_w[2][NMAT][NN * UG_LD];
  static_assert(sizeof(s_w) >= 3 * 16 * WAVE * sizeof(float), "sums fit in the stage buffers");
  float* red = reinterpret_cast<float*>(&s_w[0][0][0]);
  if (a.run_if && *a.run_if != a.run_want) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int W = a.ffn / 32;
  constexpr int WPT = 4;                                // bitmap words per thread (ffn <= 32768)
  // 1. union ranks: prefix of popcounts over the words (thread t owns words 4t .. 4t+3)
  uint32_t bw[WPT];
  int local = 0;
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int w = tid * WPT + k;
    bw[k] = w < W ? a.ubits[w] : 0u;
    local += __popc(bw[k]);
  }
  // local <= 32 * WPT = 128: eight bit planes
  static_assert(32 * WPT < (1 << 8), "a thread's count fits the prefix's eight bit planes");
  int wtot;
  const int before = wave_prefix_small<8>(local, wtot);
  if (lane == 0) s_wsum[wave] = wtot;
  if (tid < NN) s_nid[tid] = -1;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int k = 0; k < BT / WAVE; ++k) {
    base += k < wave ? s_wsum[k] : 0;
    total += s_wsum[k];
  }
  if (blockIdx.x == 0 && tid == 0) *a.ucnt = total;
  const int t0 = blockIdx.x * NN;
  if (t0 >= total) return;                              // uniform over the workgroup
  const int run0 = base + before;
  if (run0 < t0 + NN && run0 + local > t0) {
    int pos = run0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      uint32_t bb = bw[k];
      const int nb = (tid * WPT + k) * 32;
      while (bb) {
        if (pos >= t0 && pos < t0 + NN) {
          const int nid = nb + __builtin_ctz(bb);
          s_nid[pos - t0] = nid;
          a.uidx[pos] = nid;
        }
        bb &= bb - 1;
        ++pos;
      }
    }
  }
  __syncthreads();

  // 2. U = X W_up^T and G = X W_gate^T for the NN neurons
  const int row = lane & 31, g = lane >> 5;
  const int nchk = a.d / 8;
  const int nstage = (nchk + UG_KC - 1) / UG_KC;
  // cooperative row loads: element e = tid + BT * i -> (row e / UG_KC, chunk e % UG_KC)
  const char* wsrc[2] = {static_cast<const char*>(a.w_up),
                         static_cast<const char*>(GATE ? a.w_gate : a.w_up)};
  size_t lrow_off[LPT];
  int lch[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int e = tid + BT * i;
    lrow_off[i] = (size_t)max(s_nid[e / UG_KC], 0) * nchk * 16;
    lch[i] = e % UG_KC;
  }
  // Loads are raw (clamped addresses, never predicated); chunks past the row end are zeroed where
  // the values are next used (LDS store, MFMA operand), so that no load of a stage two ahead has
  // to land before the loop turns.
  auto load_w = [&](int st, u32x4 (&r)[NMAT][LPT]) {
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int c = st * UG_KC + lch[i];
        r[mt][i] = ld16(wsrc[mt] + lrow_off[i] + (size_t)min(c, nchk - 1) * 16);
      }
  };
  auto store_w = [&](int buf, int st, const u32x4 (&r)[NMAT][LPT]) {
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int e = tid + BT * i;
        s_w[buf][mt][(e / UG_KC) * UG_LD + e % UG_KC] =
            st * UG_KC + lch[i] < nchk ? r[mt][i] : u32x4{0u, 0u, 0u, 0u};
      }
  };
  // token operand straight from global: wave w takes the stage's 16-k steps 4w .. 4w+3
  constexpr int SPW = UG_KC / 2 / 4;                    // steps per wave and stage
  const char* xr = static_cast<const char*>(a.x) + (size_t)min(row, a.B - 1) * a.d * 2;
  const bool xok = row < a.B;
  auto load_x = [&](int st, u32x4 (&xv)[SPW]) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int c = st * UG_KC + 2 * (wave * SPW + j) + g;
      xv[j] = ld16(xr + (size_t)min(c, nchk - 1) * 16);
    }
  };

  // Loads run two stages ahead.  Register sets rotate by name, not by copy (a copy of a register
  // that a load is still filling waits for that load): the token slices over three sets (stage
  // st in xa, st+1 held, st+2 arriving in xc), the row chunks over two (stage st+1 in wb, bound
  // for LDS this turn; st+2 arriving in wc), so the loop body is written out for six stages.
  // Loads and LDS stores are unconditional (the last two turns re-read the last stage, from L2,
  // and the last store writes zeros): a branch around either would merge a path with other
  // loads in flight, and the waits would then cover this turn's loads too.
  f32x16 au[NTL], ag[NTL];
#pragma unroll
  for (int t = 0; t < NTL; ++t) au[t] = ag[t] = f32x16{};
  u32x4 wA[NMAT][LPT], wB[NMAT][LPT], xA[SPW], xB[SPW], xC[SPW];
  load_w(0, wB);
  load_x(0, xA);
  load_w(min(1, nstage - 1), wA);
  load_x(min(1, nstage - 1), xB);
  store_w(0, 0, wB);
  __syncthreads();
  auto step = [&](int st, const u32x4 (&xa)[SPW], u32x4 (&xc)[SPW], const u32x4 (&wb)[NMAT][LPT],
                  u32x4 (&wc)[NMAT][LPT]) {
    const int buf = st & 1;
    load_w(min(st + 2, nstage - 1), wc);
    load_x(min(st + 2, nstage - 1), xc);
    issue_fence();                                      // the loads go out first
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const bool ok = xok && st * UG_KC + 2 * (wave * SPW + j) + g < nchk;
      const u32x4 xj = ok ? xa[j] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const int idx = (t * 32 + row) * UG_LD + 2 * (wave * SPW + j) + g;
        au[t] = mma16(xj, s_w[buf][0][idx], au[t]);
        if constexpr (GATE) ag[t] = mma16(xj, s_w[buf][NMAT - 1][idx], ag[t]);
      }
    }
    store_w(buf ^ 1, st + 1, wb);                       // past the last stage: zeros, unread
    __syncthreads();
  };
  // whole rounds of six in the loop, the rest after it (an exit between the steps would join the
  // loop head with loads in other registers in flight, and the head would wait for them all)
  int st0 = 0;
  for (; st0 + 6 <= nstage; st0 += 6) {
    step(st0, xA, xC, wA, wB);
    step(st0 + 1, xB, xA, wB, wA);
    step(st0 + 2, xC, xB, wA, wB);
    step(st0 + 3, xA, xC, wB, wA);
    step(st0 + 4, xB, xA, wA, wB);
    step(st0 + 5, xC, xB, wB, wA);
  }
  const int rest = nstage - st0;
  if (rest > 0) {
    step(st0, xA, xC, wA, wB);
    if (rest > 1) {
      step(st0 + 1, xB, xA, wB, wA);
      if (rest > 2) {
        step(st0 + 2, xC, xB, wA, wB);
        if (rest > 3) {
          step(st0 + 3, xA, xC, wB, wA);
          if (rest > 4) step(st0 + 4, xB, xA, wA, wB);
        }
      }
    }
  }
  // the tokens' own bitmap words for phase 3, all loads issued at once (clamped addresses, so
  // unconditional), their latency hidden behind the cross-wave sums
  uint32_t ob[NTL][16];
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    const int nc = max(s_nid[t * 32 + row], 0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      ob[t][i] = ldg(a.bits, (size_t)min(acc_row(i, lane), a.B - 1) * W + (nc >> 5));
  }
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    au[t] = wg_sum4(au[t], red);
    if constexpr (GATE) ag[t] = wg_sum4(ag[t], red);
  }

  // 3. h per (token, neuron), masked by the token's own set; H column = union rank
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const int nid = s_nid[t * 32 + row];
      const float bu = (nid >= 0 && a.b_up) ? a.b_up[nid] : 0.0f;
      const float bg = (nid >= 0 && a.b_gate) ? a.b_gate[nid] : 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = acc_row(i, lane);
        const float u = au[t][i] + bu;
        float h;
        if constexpr (!GATE) {
          h = fmaxf(u, 0.0f);
        } else {
          const float gg = fmaxf(ag[t][i] + bg, 0.0f);
          h = a.act == FFN_ACT_REGLU ? gg * u : gg * fmaxf(u, 0.0f);
        }
        const bool on = nid >= 0 && m < a.B && ((ob[t][i] >> (nid & 31)) & 1u);
        if (t0 + t * 32 + row < a.ffn) a.H[(size_t)m * a.ffn + t0 + t * 32 + row] = (_Float16)(on ? h : 0.0f);
      }
    }
  }
}

// Y_s[:, c0 .. c0+256) = H[:, U_s] W_down_t[U_s, c0 .. c0+256); K (union ranks) split over the
// waves, each rank's down row read as 16-byte column chunks.  Lane (p, g) loads columns
// c0 + 8p .. c0 + 8p + 7 of four rows; element b of those chunks feeds MFMA block b, whose
// output column p is y column c0 + 8p + b.
__global__ __launch_bounds__(BT) void k_bdown(BatchArgs a) {
  at_pass(a);
  __shared__ int s_nid[DN_CH];
  __shared__ float s_y[MB * DN_COLS];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  if (a.run_if && *a.run_if != a.run_want) return;
  const int total = *a.ucnt;
  int r0, r1;
  seg_range(total, blockIdx.y, a.S, r0, r1);
  if (r0 >= r1) return;                                 // uniform: segment is empty
  const int c0 = blockIdx.x * DN_COLS, p = lane & 31, g = lane >> 5;
  const int col = min(c0 + 8 * p, a.d - 8);
  const char* dn = static_cast<const char*>(a.w_dn) + (size_t)col * 2;
  const char* hr = reinterpret_cast<const char*>(a.H + (size_t)p * a.ffn);
  f32x16 acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = f32x16{};
  for (int q0 = r0; q0 < r1; q0 += DN_CH) {
    const int nq = min(DN_CH, r1 - q0);                 // a multiple of 8
    __syncthreads();
    for (int t = tid; t < nq; t += BT) s_nid[t] = q0 + t < total ? a.uidx[q0 + t] : 0;
    __syncthreads();
    const int nst = nq / 8;
    for (int s0 = wave; s0 < nst; s0 += 4 * GRPD) {
      u32x2 av[GRPD];
      u32x4 bv[GRPD][4];
#pragma unroll
      for (int j = 0; j < GRPD; ++j) {
        const int s = s0 + 4 * j;
        const bool ok = s < nst;
        const int kb = 8 * min(s, nst - 1) + 4 * g;     // rank offset within the chunk
        const u32x2 hl = *reinterpret_cast<const u32x2*>(hr + (size_t)(q0 + kb) * 2);
        av[j] = ok ? hl : u32x2{0u, 0u};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          bv[j][jj] = ld16(dn + (size_t)s_nid[kb + jj] * a.d * 2);
      }
      issue_fence();
#pragma unroll
      for (int j = 0; j < GRPD; ++j) {
        const uint32_t w0[4] = {bv[j][0].x, bv[j][0].y, bv[j][0].z, bv[j][0].w};
        const uint32_t w1[4] = {bv[j][1].x, bv[j][1].y, bv[j][1].z, bv[j][1].w};
        const uint32_t w2[4] = {bv[j][2].x, bv[j][2].y, bv[j][2].z, bv[j][2].w};
        const uint32_t w3[4] = {bv[j][3].x, bv[j][3].y, bv[j][3].z, bv[j][3].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // column 8p + 2q (low halves) and 8p + 2q + 1 (high halves) of the four rows
          const u32x2 blo = {__builtin_amdgcn_perm(w1[q], w0[q], 0x05040100u),
                             __builtin_amdgcn_perm(w3[q], w2[q], 0x05040100u)};
          const u32x2 bhi = {__builtin_amdgcn_perm(w1[q], w0[q], 0x07060302u),
                             __builtin_amdgcn_perm(w3[q], w2[q], 0x07060302u)};
          acc[2 * q] = mma8(av[j], blo, acc[2 * q]);
          acc[2 * q + 1] = mma8(av[j], bhi, acc[2 * q + 1]);
        }
      }
    }
  }
  // sum the waves' tiles in wave order through LDS, then write this segment's partial
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float& dst = s_y[acc_row(i, lane) * DN_COLS + 8 * p + b];
          dst = w == 0 ? acc[b][i] : dst + acc[b][i];
        }
    }
    __syncthreads();
  }
  for (int e = tid; e < MB * DN_COLS / 4; e += BT) {
    const int m = e / (DN_COLS / 4), c4 = e % (DN_COLS / 4);
    const int cc = c0 + 4 * c4;
    if (m < a.B && cc < a.d)
      *reinterpret_cast<f32x4*>(a.ypart + ((size_t)blockIdx.y * MB + m) * a.d + cc) =
          *reinterpret_cast<const f32x4*>(&s_y[m * DN_COLS + 4 * c4]);
  }
}

// y = b_down + sum of the non-empty segments' partials (in segment order); workgroup (0, m)
// also writes token m's ascending index list and count.
__global__ __launch_bounds__(256) void k_bred(BatchArgs a) {
  at_pass(a);
  if (a.run_if && *a.run_if != a.run_want) return;
  const int m = blockIdx.y;
  if (m >= a.B) return;                                 // the last pass of a call may be short
  const int col = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int total = *a.ucnt;
  if (col < a.d) {
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    const f32x4 bd = a.b_down ? *reinterpret_cast<const f32x4*>(a.b_down + col) : t;
    // segments in order, eight loads in flight at a time; empty segments were not written
    for (int s0 = 0; s0 < a.S; s0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = min(s0 + u, a.S - 1);
        v[u] = *reinterpret_cast<const f32x4*>(a.ypart + ((size_t)s * MB + m) * a.d + col);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int r0, r1;
        seg_range(total, s0 + u, a.S, r0, r1);
        if (s0 + u < a.S && r0 < r1) t += v[u];
      }
    }
    if (a.b_down) t += bd;
    *reinterpret_cast<f32x4*>(a.y + (size_t)m * a.d + col) = t;
  }
  if (blockIdx.x == 0 && (a.idx_out || a.cnt_out))
    write_index_list<256>(a.bits + (size_t)m * (a.ffn / 32), a.ffn / 32,
                          a.idx_out ? a.idx_out + (size_t)m * a.ffn : nullptr,
                          a.cnt_out ? a.cnt_out + m : nullptr);
}

// ---------------------------------------------------------------------------------------------
// Host side.
BatchShape batch_shape(int d, int ffn, int r) {
  BatchShape s{};
  const int tiles = (r + 31) / 32;
  const int nsteps = (d / 8 + 1) / 2;
  s.ks = r > 0 ? std::max(1, std::min({32, 256 / std::max(tiles, 1), nsteps / 4})) : 1;
  s.spw = (nsteps + s.ks * 4 - 1) / (s.ks * 4);
  const int ctiles = (d + DN_COLS - 1) / DN_COLS;
  s.S = std::max(1, std::min(64, 256 / ctiles));
  s.zpart_bytes = (size_t)s.ks * MB * std::max(r, 1) * 4;
  s.zhl_bytes = (size_t)2 * MB * std::max(r, 1) * 2;
  s.bits_bytes = (size_t)MB * (ffn / 32) * 4;
  s.ubits_bytes = (size_t)(ffn / 32) * 4;
  s.uidx_bytes = (size_t)ffn * 4;
  s.H_bytes = (size_t)MB * ffn * 2;
  s.ypart_bytes = (size_t)s.S * MB * d * 4;
  return s;
}

hipError_t launch_batch_sets(const BatchArgs& a, int use_predictor, hipStream_t st,
                             int passes) {
  const int W = a.ffn / 32;
  if (use_predictor) {
    hipLaunchKernelGGL(k_bz, dim3((a.r + 31) / 32 * a.ks * passes), dim3(BT), 0, st, a);
    hipLaunchKernelGGL(k_bzr, dim3((MB * a.r + 255) / 256, 1, passes), dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_bs, dim3((W + 3) / 4 * passes), dim3(BS_T), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_bmask, dim3((W + 255) / 256, 1, passes), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_batch_stage1(const BatchArgs& a, hipStream_t st, int passes) {
  hipLaunchKernelGGL(k_bz, dim3((a.r + 31) / 32 * a.ks * passes), dim3(BT), 0, st, a);
  hipLaunchKernelGGL(k_bzr, dim3((MB * a.r + 255) / 256, 1, passes), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_batch_zsum(const BatchArgs& a, hipStream_t st, int passes) {
  hipLaunchKernelGGL(k_bzr, dim3((MB * a.r + 255) / 256, 1, passes), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_batch_union(const BatchArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_bunion, dim3((a.ffn / 32 + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_batch_rows(const BatchArgs& a, int choose_path, hipStream_t st,
                             hipEvent_t (*ev)[2], int passes) {
  const int W = a.ffn / 32;
  if (choose_path) hipLaunchKernelGGL(k_bpath, dim3(1), dim3(1024), 0, st, a);
  // ReLU layers at larger batches take 64 union neurons per workgroup: each token slice then
  // serves twice the rows (at small batches the union is too small to fill the chip that way,
  // and the gate's second tile would not fit the LDS of several resident workgroups)
  if (a.has_gate) {
    if (ev && ev[0][0])
      hipExtLaunchKernelGGL((k_bug<true, 32>), dim3(W, 1, passes), dim3(BT), 0, st, ev[0][0],
                            ev[0][1], 0, a);
    else
      hipLaunchKernelGGL((k_bug<true, 32>), dim3(W, 1, passes), dim3(BT), 0, st, a);
  } else if (a.B > UG_WIDE_B) {
    const dim3 g2((W + 1) / 2, 1, passes);
    if (ev && ev[0][0])
      hipExtLaunchKernelGGL((k_bug<false, 64>), g2, dim3(BT), 0, st, ev[0][0], ev[0][1], 0, a);
    else
      hipLaunchKernelGGL((k_bug<false, 64>), g2, dim3(BT), 0, st, a);
  } else {
    if (ev && ev[0][0])
      hipExtLaunchKernelGGL((k_bug<false, 32>), dim3(W, 1, passes), dim3(BT), 0, st, ev[0][0],
                            ev[0][1], 0, a);
    else
      hipLaunchKernelGGL((k_bug<false, 32>), dim3(W, 1, passes), dim3(BT), 0, st, a);
  }
  const dim3 gd((a.d + DN_COLS - 1) / DN_COLS, a.S, passes);
  if (ev && ev[1][0])
    hipExtLaunchKernelGGL(k_bdown, gd, dim3(BT), 0, st, ev[1][0], ev[1][1], 0, a);
  else
    hipLaunchKernelGGL(k_bdown, gd, dim3(BT), 0, st, a);
  hipLaunchKernelGGL(k_bred, dim3((a.d + 1023) / 1024, passes > 1 ? MB : a.B, passes), dim3(256),
                     0, st, a);
  return hipGetLastError();
}

int batch_segments_mp(int d, int passes) {
  const int ctiles = (d + DN_COLS - 1) / DN_COLS;
  const int S = std::max(1, std::min(64, 256 / ctiles));
  return std::max(1, std::min(S, 2048 / (ctiles * std::max(passes, 1))));
}

hipError_t launch_batch(const BatchArgs& a, int use_predictor, int choose_path, hipStream_t st,
                        hipEvent_t (*ev)[2]) {
  hipError_t e = launch_batch_sets(a, use_predictor, st);
  if (e != hipSuccess) return e;
  return launch_batch_rows(a, choose_path, st, ev);
}

hipError_t launch_dense_choice(const uint32_t* ubits, int passes, int ffn, int dense_above,
                               int* flag, hipStream_t st) {
  hipLaunchKernelGGL(k_dchoice, dim3(1), dim3(1024), 0, st, ubits, passes, ffn / 32, dense_above,
                     flag);
  return hipGetLastError();
}

}  // namespace ffn
