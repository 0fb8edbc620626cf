// Dense fallback of the FFN on gfx950's matrix cores (fp16 layers, many tokens: prefill).
//
// When most neurons fire -- a prompt of many tokens -- the pages run the FFN as large dense
// blocks instead of per-neuron work (citnews.com.cn PowerInfer-2 article, neuron-cluster
// computation: prefill as one big cluster, decode as small sparse ones).  Here that is two GEMMs
// with fp32 accumulation on v_mfma_f32_32x32x16_f16:
//   k_dup    H = act(X W_up^T + b_up [, X W_gate^T + b_gate]), zeroed where a token's set
//            (if given) excludes the neuron; H stored fp16, [M][ffn]
//   k_ddq / k_ddown  Y_k = H[:, K slice k] W_down_t[K slice k, :]   (split over ffn when the
//            tiles alone do not fill the GPU; k_ddq with 256-token tiles, k_ddown with 128-token
//            ones where those pad the tokens less)
//   k_dred   y = b_down + sum_k Y_k (in slice order)
// k_dupq and k_ddq copy both operands straight into LDS (global_load_lds_dwordx4, a four-slot
// ring); k_dup and k_ddown stage the weight tile in LDS from registers and read the token-side
// operand straight into registers.  Tiles are mapped to the eight XCDs so that the M tiles
// sharing a weight tile run on the same XCD one after another (its L2 serves the repeats).
//
// W_down_t is stored [ffn][d] (d contiguous): for the second GEMM the MFMA needs 8 consecutive
// ffn values per lane and column, so a lane reads 16-byte pieces of 8 rows (8 columns each) and
// regroups them in registers: element b of those pieces feeds MFMA block b, whose output column
// p is y column 8p + b of the tile.
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.h"
#include "index.h"
#include "launch.h"

namespace ffn {

namespace {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mma16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, a),
                                                __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}
constexpr int DT = 256;            // threads per workgroup: 4 waves
// k_ddown: DD_M tokens x DD_N columns per tile (8 MFMA blocks of 32 x 8; index.h)
constexpr int DD_K = 32;           // k_ddown: ffn rows per stage
constexpr int DD_LD = DD_N / 8 + 1;

// this workgroup's tile (consecutive tile ids run on one XCD; ids >= total are idle)
__device__ __forceinline__ int xcd_tile(int total) { return xcd_tile_of(blockIdx.x, total); }

}  // namespace

// k_dup: 256 tokens x 256 neurons (ReLU) or 256 x 128 neurons with their gate rows per
// workgroup of 8 waves; both operands staged through LDS per K stage of 64, double-buffered, with
// the global loads of the next stage in flight during the current one's MFMAs.  Wave w owns
// tokens 64 (w / 2) .. +63 and half of the tile's neurons (w % 2).
constexpr int UP_T = 512;                  // threads
constexpr int UP_M = 256;                  // tokens per tile
constexpr int UP_KC = 8;                   // 16-byte chunks per row per stage (K = 64)
constexpr int UP_LD = UP_KC + 1;           // padded LDS row

template <bool GATE>
__global__ __launch_bounds__(UP_T) void k_dup(DenseArgs a) {
  constexpr int NMAT = GATE ? 2 : 1;
  constexpr int UP_N = GATE ? 128 : 256;   // neurons per tile
  constexpr int BROWS = UP_N * NMAT;       // weight rows per stage (up rows, then gate rows)
  constexpr int NSUB = UP_N / 2 / 32;      // 32-neuron MFMA blocks per wave
  constexpr int LA = UP_M * UP_KC / UP_T;  // A chunk loads per thread and stage (4)
  constexpr int LB = BROWS * UP_KC / UP_T; // B chunk loads per thread and stage (4)
  __shared__ u32x4 sA[2][UP_M * UP_LD];
  __shared__ u32x4 sB[2][BROWS * UP_LD];
  if (a.run_if && *a.run_if != a.run_want) return;
  const int nb_m = (a.M + UP_M - 1) / UP_M, nb_n = (a.ffn + UP_N - 1) / UP_N;
  const int tile = xcd_tile(nb_m * nb_n);
  if (tile >= nb_m * nb_n) return;
  const int m0 = (tile % nb_m) * UP_M, n0 = (tile / nb_m) * UP_N;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int nchk = a.d / 8;

  // cooperative loads: element e = tid + UP_T * i -> (row e / UP_KC, chunk e % UP_KC)
  const char* xsrc = static_cast<const char*>(a.x);
  size_t aoff[LA], boff[LB];
  bool aok[LA];
  int ach[LA], bch[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int e = tid + UP_T * i, row = e / UP_KC;
    aok[i] = m0 + row < a.M;
    aoff[i] = (size_t)min(m0 + row, a.M - 1) * nchk * 16;
    ach[i] = e % UP_KC;
  }
  const char* bsrc[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int e = tid + UP_T * i, row = e / UP_KC;
    const int mat = row / UP_N, n = min(n0 + row % UP_N, a.ffn - 1);
    bsrc[i] = static_cast<const char*>(mat == 0 ? a.w_up : a.w_gate);
    boff[i] = (size_t)n * nchk * 16;
    bch[i] = e % UP_KC;
  }
  // Raw loads (clamped addresses, never predicated); rows past the tokens and chunks past the
  // row end are zeroed on the way into LDS, so that no load has to land before the loop turns.
  auto load = [&](int st, u32x4 (&ra)[LA], u32x4 (&rb)[LB]) {
#pragma unroll
    for (int i = 0; i < LA; ++i)
      ra[i] = ld16(xsrc + aoff[i] + (size_t)min(st * UP_KC + ach[i], nchk - 1) * 16);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      rb[i] = ld16(bsrc[i] + boff[i] + (size_t)min(st * UP_KC + bch[i], nchk - 1) * 16);
  };
  auto store = [&](int buf, int st, const u32x4 (&ra)[LA], const u32x4 (&rb)[LB]) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int e = tid + UP_T * i;
      const bool ok = aok[i] && st * UP_KC + ach[i] < nchk;
      sA[buf][(e / UP_KC) * UP_LD + e % UP_KC] = ok ? ra[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int e = tid + UP_T * i;
      const bool ok = st * UP_KC + bch[i] < nchk;
      sB[buf][(e / UP_KC) * UP_LD + e % UP_KC] = ok ? rb[i] : u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x16 acc[2][NSUB][NMAT];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt) acc[ms][ns][mt] = f32x16{};

  // Loads run two stages ahead, LDS holds the current and the next stage.  The two register sets
  // swap roles by name each turn (stage s+1 held for LDS, stage s+2 arriving), never by copy: a
  // copy of a register that a load is still filling waits for the load.  Loads and LDS stores are
  // unconditional (the last two turns re-read the last stage, from L2, and the last store writes
  // zeros nobody reads), and the loop holds whole pairs of stages: a branch around a load or an
  // exit between the pair would join paths with other loads in flight, and the waits would then
  // cover this turn's loads too.
  const int nstage = (nchk + UP_KC - 1) / UP_KC;
  u32x4 raA[LA], rbA[LB], raB[LA], rbB[LB];
  load(0, raB, rbB);
  load(min(1, nstage - 1), raA, rbA);
  store(0, 0, raB, rbB);
  __syncthreads();
  auto step = [&](int s, const u32x4 (&rah)[LA], const u32x4 (&rbh)[LB], u32x4 (&ran)[LA],
                  u32x4 (&rbn)[LB]) {
    const int buf = s & 1;
    load(min(s + 2, nstage - 1), ran, rbn);
    issue_fence();                                      // the loads go out first
#pragma unroll
    for (int kk = 0; kk < UP_KC / 2; ++kk) {
      u32x4 af[2];
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
        af[ms] = sA[buf][(wm * 64 + ms * 32 + r32) * UP_LD + 2 * kk + g];
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
          const u32x4 bf = sB[buf][(mt * UP_N + wn * (UP_N / 2) + ns * 32 + r32) * UP_LD + 2 * kk + g];
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) acc[ms][ns][mt] = mma16(af[ms], bf, acc[ms][ns][mt]);
        }
    }
    store(buf ^ 1, s + 1, rah, rbh);
    __syncthreads();
  };
  int s0 = 0;
  for (; s0 + 2 <= nstage; s0 += 2) {
    step(s0, raA, rbA, raB, rbB);
    step(s0 + 1, raB, rbB, raA, rbA);
  }
  if (s0 < nstage) step(s0, raA, rbA, raB, rbB);

  // the tile's words of the tokens' bitmaps, staged in LDS (the stage buffers are free now) by
  // one round of loads, instead of one dependent load per output element
  constexpr int TW = UP_N / 32;                         // bitmap words per token row
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(&sA[0][0]);
  static_assert(sizeof(sA) >= UP_M * TW * sizeof(uint32_t), "bitmap words fit in the A stages");
  const int W = a.ffn / 32;
  if (a.bits) {
    constexpr int BL = UP_M * TW / UP_T;
    uint32_t bw[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int e = tid + UP_T * i, row = e / TW, wc = e % TW;
      bw[i] = ldg(a.bits, (size_t)min(m0 + row, a.M - 1) * W + min(n0 / 32 + wc, W - 1));
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) s_bits[tid + UP_T * i] = bw[i];
    __syncthreads();
  }

  // epilogue: h per (token, neuron), masked by the token's set, to H (fp16)
#pragma unroll
  for (int ns = 0; ns < NSUB; ++ns) {
    const int n = n0 + wn * (UP_N / 2) + ns * 32 + r32;
    const int nc = min(n, a.ffn - 1);
    const float bu = a.b_up ? a.b_up[nc] : 0.0f;
    const float bg = (GATE && a.b_gate) ? a.b_gate[nc] : 0.0f;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * 64 + ms * 32 + acc_row(i, lane);
        const float u = acc[ms][ns][0][i] + bu;
        float h;
        if constexpr (!GATE) {
          h = fmaxf(u, 0.0f);
        } else {
          const float gg = fmaxf(acc[ms][ns][NMAT - 1][i] + bg, 0.0f);
          h = a.act == FFN_ACT_REGLU ? gg * u : gg * fmaxf(u, 0.0f);
        }
        if (m < a.M && n < a.ffn) {
          if (a.bits && !((s_bits[(m - m0) * TW + (n - n0) / 32] >> (n & 31)) & 1u)) h = 0.0f;
          a.H[(size_t)m * a.ffn + n] = (_Float16)h;
        }
      }
  }
}

// k_dupq: the same tile and wave split as k_dup, with both operands copied from global memory
// straight into LDS by gfx950's global_load_lds_dwordx4 (no register staging: the registers
// the staging took hold a second set of MFMA fragments instead).  K stages of 32 (four 16-byte
// chunks per row), a ring of four LDS slots, the copies for stage s + 3 issued once every wave
// has finished stage s - 1.  A row's four chunks sit in its 64 LDS bytes in an order swizzled by
// the row, (chunk ^ (row / 4) % 4), so that the fragment reads of 16 consecutive rows meet no bank
// twice.  Rows past the tokens or neurons are clamped copies (their outputs are never stored);
// d must be a multiple of 32 (no partial stage).
constexpr int UQ_DK = 4;                   // chunks per row per stage (K = 32)
constexpr int UQ_NS = 4;                   // LDS ring slots

__device__ __forceinline__ constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xf) | (0x7 << 4) | ((lgkm & 0xf) << 8) | (((vm >> 4) & 0x3) << 14);
}
// the target builtins sit in device helpers (a kernel template that names them directly gets
// no host-side launch stub)
__device__ __forceinline__ void lds_copy16(const void* src, u32x4* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, LGKM));
}
__device__ __forceinline__ void barrier_only() { __builtin_amdgcn_s_barrier(); }
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <int MASK, int N>
__device__ __forceinline__ void sched_group() { __builtin_amdgcn_sched_group_barrier(MASK, N, 0); }

// EPI 0: the FFN's up projection (h = act, masked, to H).  EPI 1: predictor stage 2 of a
// large call (scores against the threshold into bitmap and union words; GATE false).  EPI 2:
// predictor stage 1 of a large call, split over K (a.kslices slices of d): each slice's fp32
// partial of Z = X P1^T, in the per-pass layout [pass][slice][32 tokens][rank] that the batched
// path's fixed-order sum (k_bzr) reads.  TM x TN: the tile (tokens x neurons); the stage-1 GEMM
// takes ZP_M x ZP_N (its rank columns give few 256 x 256 tiles, which the K split would have to
// make up for with more partials).
constexpr int EPI_FFN = 0, EPI_SCORE = 1, EPI_ZPART = 2;

template <bool GATE, int EPI = EPI_FFN, int TM = UP_M, int TN = 256>
__global__ __launch_bounds__(UP_T) void k_dupq(DenseArgs a) {
  static_assert(EPI == EPI_FFN || !GATE, "the predictor GEMMs have no gate rows");
  static_assert((TM == UP_M && TN == 256) || EPI == EPI_ZPART, "smaller tiles: stage-1 GEMM only");
  constexpr int NMAT = GATE ? 2 : 1;
  constexpr int UP_N = GATE ? 128 : TN;    // neurons per tile
  constexpr int MS = TM / 4 / 32;          // 32-token MFMA blocks per wave (wave rows: TM / 4)
  constexpr int BROWS = UP_N * NMAT;       // weight rows per stage (up rows, then gate rows)
  constexpr int NSUB = UP_N / 2 / 32;      // 32-neuron MFMA blocks per wave
  constexpr int NW = UP_T / WAVE;          // 8 waves
  constexpr int AI = TM / 16 / NW;         // A copy instructions per wave and stage (2)
  constexpr int BI = BROWS / 16 / NW;      // B copy instructions per wave and stage (2)
  constexpr int NB = NSUB * NMAT;
  static_assert(AI * NW * 16 == TM && BI * NW * 16 == BROWS, "whole copy instructions");
  // one array per ring slot (not one indexed array): the compiler then sees that a stage's reads
  // and the copies in flight into the other slots touch different memory, and does not make the
  // reads wait for those copies
  __shared__ u32x4 sA0[TM * UQ_DK], sA1[TM * UQ_DK], sA2[TM * UQ_DK], sA3[TM * UQ_DK];
  __shared__ u32x4 sB0[BROWS * UQ_DK], sB1[BROWS * UQ_DK], sB2[BROWS * UQ_DK], sB3[BROWS * UQ_DK];
  static_assert(UQ_NS == 4, "four ring slots");
  if (a.run_if && *a.run_if != a.run_want) return;
  const int nb_m = (a.M + TM - 1) / TM, nb_n = (a.ffn + UP_N - 1) / UP_N;
  const int nks = EPI == EPI_ZPART ? a.kslices : 1;
  const int tile = xcd_tile(nb_m * nb_n * nks);
  if (tile >= nb_m * nb_n * nks) return;
  int mt, nt, kslice;
  gemm_tile(tile, nb_m, nb_n, mt, nt, kslice);
  const int m0 = mt * TM, n0 = nt * UP_N;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int wave = wave_uniform(tid / WAVE);             // scalar: the copies' LDS base
  const int r32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int nchk = a.d / 8, nst_all = nchk / UQ_DK;
  // this workgroup's K stages: all of them, or its slice's [sbase, sbase + nst)
  int sbase, nst;
  slice_stages(nst_all, kslice, nks, sbase, nst);
  const size_t rowb = (size_t)nchk * 16;

  // copy sources: instruction i of this wave covers rows 16 (wave * AI + i) .. +15 of the tile,
  // lane l row + l / 4 and LDS position l % 4, which holds chunk (l % 4) ^ (row / 4) % 4
  const char* asrc[AI];
  const char* bsrc[BI];
  const int pos = lane & 3;
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (wave * AI + i) * 16 + (lane >> 2);
    asrc[i] = static_cast<const char*>(a.x) + (size_t)min(m0 + row, a.M - 1) * rowb +
              (size_t)(pos ^ ((row >> 2) & 3)) * 16;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = (wave * BI + i) * 16 + (lane >> 2);
    const int mat = row / UP_N, n = min(n0 + row % UP_N, a.ffn - 1);
    bsrc[i] = static_cast<const char*>(mat == 0 ? a.w_up : a.w_gate) +
              (size_t)n * (EPI == EPI_SCORE ? a.b_rowb : rowb) +
              (size_t)(pos ^ ((row >> 2) & 3)) * 16;
  }
  auto copy = [&](int st, u32x4* dA, u32x4* dB) {   // stage st (clamped) into a ring slot
    const int sc = sbase + min(st, nst - 1);
    const size_t kb = (size_t)sc * UQ_DK * 16;
    // the score GEMM's B operand repeats its K (the hi, then the lo half of z meet P2 again)
    const size_t kbb = EPI == EPI_SCORE ? (size_t)(sc % a.bwrap) * UQ_DK * 16 : kb;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      lds_copy16(asrc[i] + kb, dA + (wave * AI + i) * 64);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      lds_copy16(bsrc[i] + kbb, dB + (wave * BI + i) * 64);
  };
  constexpr int PER_STAGE = AI + BI;       // copy instructions per wave and stage

  f32x16 acc[MS][NSUB][NMAT];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt) acc[ms][ns][mt] = f32x16{};

  // fragment (row, chunk) of a slot, at the row's swizzled position
  auto frag = [&](const u32x4* base, int row, int c) {
    return base[row * UQ_DK + (c ^ ((row >> 2) & 3))];
  };
  copy(0, sA0, sB0);
  copy(1, sA1, sB1);
  copy(2, sA2, sB2);
  // stage st lives in slot st % 4; the turn reads it and copies stage st + 3 into the slot of
  // stage st - 1 (slots named statically, four turns per loop round)
  auto step = [&](int st, const u32x4* pa, const u32x4* pb, u32x4* nA, u32x4* nB) {
    // this wave's copies of stage st have landed (stages st + 1, st + 2 may still be in
    // flight) and its reads of stage st - 1 are done; after the barrier every wave's are
    wait_counts<2 * PER_STAGE, 0>();
    barrier_only();
    issue_fence();
    copy(st + 3, nA, nB);
    issue_fence();
    u32x4 fa[2][MS], fb[2][NB];
#pragma unroll
    for (int kk = 0; kk < UQ_DK / 2; ++kk) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) fa[kk][ms] = frag(pa, wm * (TM / 4) + ms * 32 + r32, 2 * kk + g);
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
          fb[kk][ns * NMAT + mt] = frag(pb, mt * UP_N + wn * (UP_N / 2) + ns * 32 + r32, 2 * kk + g);
    }
#pragma unroll
    for (int kk = 0; kk < UQ_DK / 2; ++kk)
#pragma unroll
      for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
            acc[ms][ns][mt] = mma16(fa[kk][ms], fb[kk][ns * NMAT + mt], acc[ms][ns][mt]);
    // every fragment read of the stage first, then the MFMAs (the second step's reads land
    // while the first step's MFMAs run)
    sched_group<0x100, UQ_DK / 2 * (MS + NB)>();
    sched_group<0x008, UQ_DK / 2 * MS * NB>();
  };
  int st = 0;
  for (; st + 4 <= nst; st += 4) {
    step(st, sA0, sB0, sA3, sB3);
    step(st + 1, sA1, sB1, sA0, sB0);
    step(st + 2, sA2, sB2, sA1, sB1);
    step(st + 3, sA3, sB3, sA2, sB2);
  }
  if (st < nst) {
    step(st, sA0, sB0, sA3, sB3);
    if (st + 1 < nst) {
      step(st + 1, sA1, sB1, sA0, sB0);
      if (st + 2 < nst) step(st + 2, sA2, sB2, sA1, sB1);
    }
  }
  // every copy (the clamped ones past the last stage included) has landed before the slots
  // are reused for the bitmap words
  wait_counts<0, 0>();
  __syncthreads();

  if constexpr (EPI == EPI_ZPART) {
    const int N = a.ffn;                                  // the rank
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          int m, n;
          zpart_store_pos(m0, n0, TM, UP_N, wave, ms, ns, i, lane, m, n);
          if (m < a.M && n < N) a.zpart_out[zpart_offset(m, kslice, n, N, a.zpart_ps)] = acc[ms][ns][0][i];
        }
    return;
  }

  if constexpr (EPI == EPI_SCORE) {
    // s = acc + c2; a neuron is on iff s > logit(tau) (hot-head words: always, unscored).
    // Accumulator element i of a lane holds token row 8 (i / 4) + 4 (lane / 32) + i % 4 of the
    // wave's 32-row block and neuron (lane % 32) of its 32-neuron block, so a ballot over the
    // wave gives the bitmap word of two token rows; the OR over the block's 16 elements is the
    // union word of the block's 32 tokens (one pass).
    const int W = a.ffn / 32;
#pragma unroll
    for (int ns = 0; ns < NSUB; ++ns) {
      const int nb32 = n0 + wn * (UP_N / 2) + ns * 32;    // the block's first neuron
      if (nb32 >= a.ffn) continue;                        // uniform: ffn % 32 == 0
      const int word = nb32 / 32, n = nb32 + r32;
      const bool head = word < a.head_words;
      const float c2v = a.c2 ? a.c2[n] : 0.0f;
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) {
        const int mb = m0 + wm * 64 + ms * 32;            // the block's first token (a pass)
        if (mb >= a.M) continue;                          // uniform
        uint32_t uw = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = mb + acc_row(i, lane);
          const float s = acc[ms][ns][0][i] + c2v;
          const bool on = m < a.M && (head || s > a.thr);
          if (a.scores && !head && m < a.M) a.scores[(size_t)m * a.ffn + n] = s;
          const unsigned long long bal = __ballot(on);
          const int mr = mb + 8 * (i >> 2) + (i & 3);     // lanes 0..31: row mr; 32..63: mr + 4
          if (lane == 0 && mr < a.M) a.bits_out[(size_t)mr * W + word] = (uint32_t)bal;
          if (lane == 32 && mr + 4 < a.M)
            a.bits_out[(size_t)(mr + 4) * W + word] = (uint32_t)(bal >> 32);
          uw |= (uint32_t)bal | (uint32_t)(bal >> 32);
        }
        if (lane == 0) a.ubits_out[(size_t)(mb / 32) * W + word] = uw;
      }
    }
    return;
  }

  constexpr int TW = UP_N / 32;                         // bitmap words per token row
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(&sA0[0]);
  static_assert(sizeof(sA0) >= UP_M * TW * sizeof(uint32_t), "bitmap words fit in an A slot");
  const int W = a.ffn / 32;
  if (a.bits) {
    constexpr int BL = UP_M * TW / UP_T;
    uint32_t bw[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int e = tid + UP_T * i, row = e / TW, wc = e % TW;
      bw[i] = ldg(a.bits, (size_t)min(m0 + row, a.M - 1) * W + min(n0 / 32 + wc, W - 1));
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) s_bits[tid + UP_T * i] = bw[i];
    __syncthreads();
  }
#pragma unroll
  for (int ns = 0; ns < NSUB; ++ns) {
    const int n = n0 + wn * (UP_N / 2) + ns * 32 + r32;
    const int nc = min(n, a.ffn - 1);
    const float bu = a.b_up ? a.b_up[nc] : 0.0f;
    const float bg = (GATE && a.b_gate) ? a.b_gate[nc] : 0.0f;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * 64 + ms * 32 + acc_row(i, lane);
        const float u = acc[ms][ns][0][i] + bu;
        float h;
        if constexpr (!GATE) {
          h = fmaxf(u, 0.0f);
        } else {
          const float gg = fmaxf(acc[ms][ns][NMAT - 1][i] + bg, 0.0f);
          h = a.act == FFN_ACT_REGLU ? gg * u : gg * fmaxf(u, 0.0f);
        }
        if (m < a.M && n < a.ffn) {
          if (a.bits && !((s_bits[(m - m0) * TW + (n - n0) / 32] >> (n & 31)) & 1u)) h = 0.0f;
          a.H[(size_t)m * a.ffn + n] = (_Float16)h;
        }
      }
  }
}

__global__ __launch_bounds__(DT, 2) void k_ddown(DenseArgs a) {
  __shared__ u32x4 s_b[2][DD_K * DD_LD];             // [buffer][k row * DD_LD + column chunk]
  if (a.run_if && *a.run_if != a.run_want) return;
  const int nb_m = (a.M + DD_M - 1) / DD_M, nb_n = (a.d + DD_N - 1) / DD_N;
  const int total = nb_m * nb_n * a.ks;
  const int tile = xcd_tile(total);
  if (tile >= total) return;
  int mt, nt, kslice;
  gemm_tile(tile, nb_m, nb_n, mt, nt, kslice);
  const int m0 = mt * DD_M, c0 = nt * DD_N;
  // this slice's ffn rows, in whole stages
  const int nst_all = a.ffn / DD_K;
  int st0, nsl;
  slice_stages(nst_all, kslice, a.ks, st0, nsl);
  const int st1 = st0 + nsl;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int p = lane & 31, g = lane >> 5;
  const int dch = a.d / 8;

  const int am = m0 + wave * 32 + p;
  const bool aok = am < a.M;
  const char* arow = reinterpret_cast<const char*>(a.H + (size_t)min(am, a.M - 1) * a.ffn);
  const char* dn = static_cast<const char*>(a.w_dn);

  // weight tile loads: 32 rows x 32 chunks, four per thread (a row's 512 bytes by 32 threads)
  auto load_w = [&](int k0, u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * DT;
      const int row = e / (DD_N / 8), ch = e % (DD_N / 8);
      const int col = min(c0 / 8 + ch, dch - 1);
      v[i] = ld16(dn + ((size_t)(k0 + row) * dch + col) * 16);
    }
  };
  auto store_w = [&](int buf, const u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * DT;
      s_b[buf][(e / (DD_N / 8)) * DD_LD + e % (DD_N / 8)] = v[i];
    }
  };
  // raw loads of the token rows; rows past the tokens are zeroed where they feed the MFMAs
  auto load_a = [&](int k0, u32x4 (&v)[2]) {
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) v[ss] = ld16(arow + (size_t)(k0 + 16 * ss + 8 * g) * 2);
  };

  f32x16 acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = f32x16{};

  if (st0 < st1) {
    // Loads run two stages ahead, LDS holds the current and the next stage of weights.  Three
    // register sets of each operand swap roles by name (stage t in use / held for LDS, stage
    // t+2 arriving), never by copy: a copy of a register that a load is still filling waits for
    // the load.  Loads and LDS stores are unconditional (the last two turns re-read the slice's
    // last stage, from L2; the last store is never read), and the loop holds whole rounds of
    // three: a branch around a load or an exit inside the round would join paths with other
    // loads in flight, and the waits would then cover this turn's loads too.
    const int nst = st1 - st0;
    u32x4 w0[4], w1[4], w2[4], a0[2], a1[2], a2[2];
    auto kof = [&](int t) { return (st0 + min(t, nst - 1)) * DD_K; };
    load_w(kof(0), w0);
    load_a(kof(0), a0);
    load_w(kof(1), w1);
    load_a(kof(1), a1);
    store_w(0, w0);
    __syncthreads();
    auto step = [&](int t, const u32x4 (&acur)[2], u32x4 (&arecv)[2], const u32x4 (&whold)[4],
                    u32x4 (&wrecv)[4]) {
      const int buf = t & 1;
      load_w(kof(t + 2), wrecv);
      load_a(kof(t + 2), arecv);
      issue_fence();                                    // the loads go out first
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const u32x4 av = aok ? acur[ss] : u32x4{0u, 0u, 0u, 0u};
        // rows 16 ss + 8 g + j (j = 0..7), columns 8p .. 8p+7 of the tile
        uint32_t r[8][4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4 v = s_b[buf][(16 * ss + 8 * g + j) * DD_LD + p];
          r[j][0] = v.x;
          r[j][1] = v.y;
          r[j][2] = v.z;
          r[j][3] = v.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // block 2q: low halves (column 8p + 2q), block 2q + 1: high halves (column 8p + 2q + 1)
          u32x4 lo, hi;
          lo.x = __builtin_amdgcn_perm(r[1][q], r[0][q], 0x05040100u);
          lo.y = __builtin_amdgcn_perm(r[3][q], r[2][q], 0x05040100u);
          lo.z = __builtin_amdgcn_perm(r[5][q], r[4][q], 0x05040100u);
          lo.w = __builtin_amdgcn_perm(r[7][q], r[6][q], 0x05040100u);
          hi.x = __builtin_amdgcn_perm(r[1][q], r[0][q], 0x07060302u);
          hi.y = __builtin_amdgcn_perm(r[3][q], r[2][q], 0x07060302u);
          hi.z = __builtin_amdgcn_perm(r[5][q], r[4][q], 0x07060302u);
          hi.w = __builtin_amdgcn_perm(r[7][q], r[6][q], 0x07060302u);
          acc[2 * q] = mma16(av, lo, acc[2 * q]);
          acc[2 * q + 1] = mma16(av, hi, acc[2 * q + 1]);
        }
      }
      store_w(buf ^ 1, whold);
      __syncthreads();
    };
    int t0 = 0;
    for (; t0 + 3 <= nst; t0 += 3) {
      step(t0, a0, a2, w1, w2);
      step(t0 + 1, a1, a0, w2, w0);
      step(t0 + 2, a2, a1, w0, w1);
    }
    if (t0 < nst) {
      step(t0, a0, a2, w1, w2);
      if (t0 + 1 < nst) step(t0 + 1, a1, a0, w2, w0);
    }
  }

  // write the slice's partial: each wave's 32 x 256 tile through LDS (the weight buffers),
  // one wave after another, as rows of contiguous columns
  float* sy = reinterpret_cast<float*>(&s_b[0][0]);        // 32 x 256 floats = 32 KiB
  static_assert(sizeof(s_b) >= 32 * DD_N * 4, "staging fits in the weight buffers");
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) sy[acc_row(i, lane) * DD_N + 8 * p + b] = acc[b][i];
    }
    __syncthreads();
    for (int e = tid; e < 32 * DD_N / 4; e += DT) {
      const int row = e / (DD_N / 4), c4 = e % (DD_N / 4);
      int m, col;
      ddown_store_pos(m0, c0, w, e, m, col);
      if (m < a.M && col < a.d)
        *reinterpret_cast<f32x4*>(a.ypart + ((size_t)kslice * a.M + m) * a.d + col) =
            *reinterpret_cast<const f32x4*>(&sy[row * DD_N + 4 * c4]);
    }
    __syncthreads();
  }
}

// k_ddq: the down projection with k_dupq's structure: 8 waves, a tile of 256 tokens x 256
// columns (wave w: tokens 64 (w / 2) .. +63, columns 128 (w % 2) .. +127), K stages of 32 ffn rows
// copied straight into a four-slot LDS ring by global_load_lds_dwordx4 (H rows swizzled as in
// k_dupq; W_down_t rows as they are, 512 bytes per row and stage).  The B fragment of a column
// needs 8 consecutive ffn rows: a lane reads 8 bytes (4 columns) from each of 8 rows and
// regroups them in registers, so MFMA block b (b = 0..3) holds columns 4p + b of the wave's
// 128 (p = lane % 32), and each B fragment serves both of the wave's 32-token blocks (12 LDS
// bytes per lane and MFMA against k_ddown's 16).  Only LDS copies are in flight inside the loop,
// so the count-based wait covers exactly the copies of the stages it names.

__global__ __launch_bounds__(UP_T) void k_ddq(DenseArgs a) {
  constexpr int NW = UP_T / WAVE;                        // 8 waves
  constexpr int AI = DQ_M / 16 / NW;                     // A copies per wave and stage (2)
  constexpr int BI = 32 / 2 / NW;                        // B copies (two K rows each) (2)
  constexpr int PER_STAGE = AI + BI;
  __shared__ u32x4 sA0[DQ_M * UQ_DK], sA1[DQ_M * UQ_DK], sA2[DQ_M * UQ_DK], sA3[DQ_M * UQ_DK];
  __shared__ u32x4 sB0[32 * 32], sB1[32 * 32], sB2[32 * 32], sB3[32 * 32];
  if (a.run_if && *a.run_if != a.run_want) return;
  const int nb_m = (a.M + DQ_M - 1) / DQ_M, nb_n = (a.d + DQ_N - 1) / DQ_N;
  const int total = nb_m * nb_n * a.ks;
  const int tile = xcd_tile(total);
  if (tile >= total) return;
  int mt, nt, kslice;
  gemm_tile(tile, nb_m, nb_n, mt, nt, kslice);
  const int m0 = mt * DQ_M, c0 = nt * DQ_N;
  const int nst_all = a.ffn / 32;
  int sbase, nst;
  slice_stages(nst_all, kslice, a.ks, sbase, nst);
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int wave = wave_uniform(tid / WAVE);
  const int r32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int dch = a.d / 8;
  const size_t hrow = (size_t)a.ffn * 2;

  const char* asrc[AI];
  const char* bsrc[BI];
  const int pos = lane & 3;
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (wave * AI + i) * 16 + (lane >> 2);
    asrc[i] = reinterpret_cast<const char*>(a.H) + (size_t)min(m0 + row, a.M - 1) * hrow +
              (size_t)(pos ^ ((row >> 2) & 3)) * 16;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int krow = (wave * BI + i) * 2 + (lane >> 5);
    bsrc[i] = static_cast<const char*>(a.w_dn) +
              ((size_t)krow * dch + min(c0 / 8 + (lane & 31), dch - 1)) * 16;
  }
  auto copy = [&](int st, u32x4* dA, u32x4* dB) {
    const int sc = sbase + min(st, nst - 1);
#pragma unroll
    for (int i = 0; i < AI; ++i)
      lds_copy16(asrc[i] + (size_t)sc * 64, dA + (wave * AI + i) * 64);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      lds_copy16(bsrc[i] + (size_t)sc * 32 * dch * 16, dB + (wave * BI + i) * 64);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[ms][b] = f32x16{};

  auto frag = [&](const u32x4* base, int row, int c) {
    return base[row * UQ_DK + (c ^ ((row >> 2) & 3))];
  };
  if (nst > 0) {
    copy(0, sA0, sB0);
    copy(1, sA1, sB1);
    copy(2, sA2, sB2);
    auto step = [&](int st, const u32x4* pa, const u32x4* pb, u32x4* nA, u32x4* nB) {
      wait_counts<2 * PER_STAGE, 0>();
      barrier_only();
      issue_fence();
      copy(st + 3, nA, nB);
      issue_fence();
      const uint2* pb2 = reinterpret_cast<const uint2*>(pb);
      u32x4 fa[2][2];
      uint2 r[2][8];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) fa[kk][ms] = frag(pa, wm * 64 + ms * 32 + r32, 2 * kk + g);
#pragma unroll
        for (int j = 0; j < 8; ++j) r[kk][j] = pb2[(16 * kk + 8 * g + j) * 64 + wn * 32 + r32];
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          u32x4 lo, hi;
          uint32_t w[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = q ? r[kk][j].y : r[kk][j].x;
          lo.x = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
          lo.y = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
          lo.z = __builtin_amdgcn_perm(w[5], w[4], 0x05040100u);
          lo.w = __builtin_amdgcn_perm(w[7], w[6], 0x05040100u);
          hi.x = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
          hi.y = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
          hi.z = __builtin_amdgcn_perm(w[5], w[4], 0x07060302u);
          hi.w = __builtin_amdgcn_perm(w[7], w[6], 0x07060302u);
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) {
            acc[ms][2 * q] = mma16(fa[kk][ms], lo, acc[ms][2 * q]);
            acc[ms][2 * q + 1] = mma16(fa[kk][ms], hi, acc[ms][2 * q + 1]);
          }
        }
      }
    };
    int st = 0;
    for (; st + 4 <= nst; st += 4) {
      step(st, sA0, sB0, sA3, sB3);
      step(st + 1, sA1, sB1, sA0, sB0);
      step(st + 2, sA2, sB2, sA1, sB1);
      step(st + 3, sA3, sB3, sA2, sB2);
    }
    if (st < nst) {
      step(st, sA0, sB0, sA3, sB3);
      if (st + 1 < nst) {
        step(st + 1, sA1, sB1, sA0, sB0);
        if (st + 2 < nst) step(st + 2, sA2, sB2, sA1, sB1);
      }
    }
    wait_counts<0, 0>();
  }
  // the slice's partial: element i of block b is token row acc_row(i) of the 32-token block and
  // column 4p + b, so a lane's four blocks give 16 contiguous bytes of a row
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int m, col;
      ddq_store_pos(m0, c0, wave, ms, i, lane, m, col);
      if (m < a.M && col < a.d) {
        const f32x4 v = {acc[ms][0][i], acc[ms][1][i], acc[ms][2][i], acc[ms][3][i]};
        *reinterpret_cast<f32x4*>(a.ypart + ((size_t)kslice * a.M + m) * a.d + col) = v;
      }
    }
}

__global__ __launch_bounds__(256) void k_dred(DenseArgs a) {
  if (a.run_if && *a.run_if != a.run_want) return;
  const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;     // m * d + col
  if (e >= (size_t)a.M * a.d) return;
  const int col = (int)(e % a.d);
  const f32x4 bd = a.b_down ? *reinterpret_cast<const f32x4*>(a.b_down + col) : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 t = *reinterpret_cast<const f32x4*>(a.ypart + e);
  // K slices in order, eight loads in flight at a time
  for (int k0 = 1; k0 < a.ks; k0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const f32x4*>(a.ypart + (size_t)min(k0 + u, a.ks - 1) * a.M * a.d + e);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < a.ks) t += v[u];
  }
  if (a.b_down) t += bd;
  *reinterpret_cast<f32x4*>(a.y + e) = t;
}

// Index list and count of every token from its bitmap (one workgroup per token).
__global__ __launch_bounds__(256) void k_dlists(DenseArgs a) {
  if (a.run_if && *a.run_if != a.run_want) return;
  const int m = blockIdx.x, W = a.ffn / 32;
  write_index_list<256>(a.bits + (size_t)m * W, W, a.idx_out ? a.idx_out + (size_t)m * a.ffn : nullptr,
                        a.cnt_out ? a.cnt_out + m : nullptr);
}

// ---------------------------------------------------------------------------------------------

int dense_ks(int M, int d, int ffn) {
  if (dense_down_wide(M)) {
    // one workgroup per CU: split ffn until the grid reaches 256
    const int t = ((M + DQ_M - 1) / DQ_M) * ((d + DQ_N - 1) / DQ_N);
    return std::max(1, std::min({8, (256 + t - 1) / t, ffn / 32}));
  }
  const int tiles = ((M + DD_M - 1) / DD_M) * ((d + DD_N - 1) / DD_N);
  // two workgroups per CU (the kernel's occupancy): split ffn until the grid reaches 512
  const int ks = std::max(1, std::min({8, (512 + tiles - 1) / tiles, ffn / DD_K}));
  return ks;
}

hipError_t launch_dense_zpart(const DenseArgs& a, hipStream_t st) {
  if (a.d % (8 * UQ_DK) || a.kslices < 1 || a.kslices > a.d / (8 * UQ_DK) || a.has_gate)
    return hipErrorInvalidValue;
  const int t = ((a.M + ZP_M - 1) / ZP_M) * ((a.ffn + ZP_N - 1) / ZP_N) * a.kslices;
  hipLaunchKernelGGL((k_dupq<false, EPI_ZPART, ZP_M, ZP_N>), dim3(8 * ((t + 7) / 8)), dim3(UP_T), 0,
                     st, a);
  return hipGetLastError();
}

int zpart_kslices(int M, int d, int rank) {
  const int tiles = ((M + ZP_M - 1) / ZP_M) * ((rank + ZP_N - 1) / ZP_N);
  return std::max(1, std::min({ZPART_MAX_KS, (256 + tiles - 1) / tiles, d / (8 * UQ_DK)}));
}

hipError_t launch_dense_scores(const DenseArgs& a, hipStream_t st) {
  if (a.d % (8 * UQ_DK) || a.bwrap < 1 || a.has_gate) return hipErrorInvalidValue;
  const int t = ((a.M + UP_M - 1) / UP_M) * ((a.ffn + 255) / 256);
  hipLaunchKernelGGL((k_dupq<false, EPI_SCORE>), dim3(8 * ((t + 7) / 8)), dim3(UP_T), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dense(const DenseArgs& a, hipStream_t st, hipEvent_t (*ev)[2]) {
  const int up_n = a.has_gate ? 128 : 256;
  const int t_up = ((a.M + UP_M - 1) / UP_M) * ((a.ffn + up_n - 1) / up_n);
  const bool wide = dense_down_wide(a.M);
  const int t_dn = wide ? ((a.M + DQ_M - 1) / DQ_M) * ((a.d + DQ_N - 1) / DQ_N) * a.ks
                        : ((a.M + DD_M - 1) / DD_M) * ((a.d + DD_N - 1) / DD_N) * a.ks;
  const dim3 g_up(8 * ((t_up + 7) / 8)), g_dn(8 * ((t_dn + 7) / 8));
  const dim3 g_red((unsigned)(((size_t)a.M * a.d / 4 + 255) / 256));
  // rows in whole 32-wide K stages take the LDS-copy kernel
  const bool q = a.d % (8 * UQ_DK) == 0;
#define UP_LAUNCH(K)                                                                      \
  do {                                                                                    \
    if (ev && ev[0][0])                                                                   \
      hipExtLaunchKernelGGL(K, g_up, dim3(UP_T), 0, st, ev[0][0], ev[0][1], 0, a);        \
    else                                                                                  \
      hipLaunchKernelGGL(K, g_up, dim3(UP_T), 0, st, a);                                  \
  } while (0)
  if (a.has_gate) {
    if (q) UP_LAUNCH(k_dupq<true>);
    else UP_LAUNCH(k_dup<true>);
  } else {
    if (q) UP_LAUNCH(k_dupq<false>);
    else UP_LAUNCH(k_dup<false>);
  }
#undef UP_LAUNCH
  if (wide) {
    if (ev && ev[1][0])
      hipExtLaunchKernelGGL(k_ddq, g_dn, dim3(UP_T), 0, st, ev[1][0], ev[1][1], 0, a);
    else
      hipLaunchKernelGGL(k_ddq, g_dn, dim3(UP_T), 0, st, a);
  } else if (ev && ev[1][0]) {
    hipExtLaunchKernelGGL(k_ddown, g_dn, dim3(DT), 0, st, ev[1][0], ev[1][1], 0, a);
  } else {
    hipLaunchKernelGGL(k_ddown, g_dn, dim3(DT), 0, st, a);
  }
  if (ev && ev[2][0])
    hipExtLaunchKernelGGL(k_dred, g_red, dim3(256), 0, st, ev[2][0], ev[2][1], 0, a);
  else
    hipLaunchKernelGGL(k_dred, g_red, dim3(256), 0, st, a);
  if (a.bits && (a.idx_out || a.cnt_out))
    hipLaunchKernelGGL(k_dlists, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ffn
