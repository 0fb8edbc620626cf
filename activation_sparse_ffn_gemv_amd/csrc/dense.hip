// Dense fallback of the FFN on gfx950's matrix cores (fp16 layers, many tokens: prefill).
//
// When most neurons fire -- a prompt of many tokens -- the pages run the FFN as large dense
// blocks instead of per-neuron work (citnews.com.cn PowerInfer-2 article, neuron-cluster
// computation: prefill as one big cluster, decode as small sparse ones).  Here that is two GEMMs
// with fp32 accumulation on v_mfma_f32_32x32x16_f16:
//   k_dup    H = act(X W_up^T + b_up [, X W_gate^T + b_gate]), zeroed where a token's set
//            (if given) excludes the neuron; H stored fp16, [M][ffn]
//   k_ddown  Y_k = H[:, K slice k] W_down_t[K slice k, :]     (split over ffn when the tiles
//            alone do not fill the GPU)
//   k_dred   y = b_down + sum_k Y_k (in slice order)
// Both GEMMs stage the weight tile in LDS (double-buffered) and read the token-side operand
// straight into registers; each wave owns 32 tokens.  Tiles are mapped to the eight XCDs so that
// the M tiles sharing a weight tile run on the same XCD one after another (its L2 serves the
// repeats).
//
// W_down_t is stored [ffn][d] (d contiguous): for the second GEMM the MFMA needs 8 consecutive
// ffn values per lane and column, so a lane reads 16-byte pieces of 8 rows (8 columns each) and
// regroups them in registers: element b of those pieces feeds MFMA block b, whose output column
// p is y column 8p + b of the tile.
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace ffn {

namespace {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mma16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, a),
                                                __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

constexpr int DT = 256;            // threads per workgroup: 4 waves
constexpr int DU_M = 128;          // k_dup: tokens per tile (32 per wave)
constexpr int DU_N = 128;          // k_dup: neurons per tile (4 MFMA blocks)
constexpr int DU_KC = 4;           // k_dup: 16-byte chunks (8 k) per row per stage: K = 32
constexpr int DU_LD = DU_KC + 1;   // padded LDS row (chunks)
constexpr int DD_M = 128;          // k_ddown: tokens per tile
constexpr int DD_N = 256;          // k_ddown: columns per tile (8 MFMA blocks of 32 x 8)
constexpr int DD_K = 32;           // k_ddown: ffn rows per stage
constexpr int DD_LD = DD_N / 8 + 1;

// blockIdx -> linear tile id such that consecutive ids run on one XCD (workgroups are dealt to
// the eight XCDs round-robin); ids >= total are idle.
__device__ __forceinline__ int xcd_tile(int total) {
  const int per = (total + 7) / 8;
  return (blockIdx.x % 8) * per + blockIdx.x / 8;
}

}  // namespace

template <bool GATE>
__global__ __launch_bounds__(DT) void k_dup(DenseArgs a) {
  constexpr int NMAT = GATE ? 2 : 1;
  __shared__ u32x4 s_b[2][NMAT][DU_N * DU_LD];       // [buffer][up, gate][row * DU_LD + chunk]
  if (a.run_if && *a.run_if != a.run_want) return;
  const int nb_m = (a.M + DU_M - 1) / DU_M, nb_n = (a.ffn + DU_N - 1) / DU_N;
  const int tile = xcd_tile(nb_m * nb_n);
  if (tile >= nb_m * nb_n) return;
  const int m0 = (tile % nb_m) * DU_M, n0 = (tile / nb_m) * DU_N;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r32 = lane & 31, g = lane >> 5;
  const int nchk = a.d / 8;

  // token row of this lane (A operand), clamped; rows past M read zeros
  const int am = m0 + wave * 32 + r32;
  const bool aok = am < a.M;
  const char* arow = static_cast<const char*>(a.x) + (size_t)min(am, a.M - 1) * a.d * 2;
  // weight tile loads: 128 rows x 4 chunks per matrix, two per thread
  const char* wsrc[2] = {static_cast<const char*>(a.w_up),
                         static_cast<const char*>(GATE ? a.w_gate : a.w_up)};
  int lrow[2], lch[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lrow[i] = tid / DU_KC + i * (DT / DU_KC);
    lch[i] = tid % DU_KC;
  }

  auto load_w = [&](int k0c, u32x4 (&v)[NMAT][2]) {
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = k0c + lch[i];
        const size_t row = (size_t)min(n0 + lrow[i], a.ffn - 1);
        const u32x4 t = ld16(wsrc[mt] + (row * nchk + min(c, nchk - 1)) * 16);
        v[mt][i] = c < nchk ? t : u32x4{0u, 0u, 0u, 0u};
      }
  };
  auto load_a = [&](int k0c, u32x4 (&v)[2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = k0c + 2 * kk + g;
      const u32x4 t = ld16(arow + (size_t)min(c, nchk - 1) * 16);
      v[kk] = (aok && c < nchk) ? t : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_w = [&](int buf, const u32x4 (&v)[NMAT][2]) {
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
      for (int i = 0; i < 2; ++i) s_b[buf][mt][lrow[i] * DU_LD + lch[i]] = v[mt][i];
  };

  f32x16 au[4], ag[GATE ? 4 : 1];
#pragma unroll
  for (int t = 0; t < 4; ++t) au[t] = f32x16{};
#pragma unroll
  for (int t = 0; t < (GATE ? 4 : 1); ++t) ag[t] = f32x16{};

  const int nstage = (nchk + DU_KC - 1) / DU_KC;
  u32x4 wv[NMAT][2], av[2];
  load_w(0, wv);
  load_a(0, av);
  store_w(0, wv);
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    const int buf = s & 1;
    u32x4 an[2];
    const bool more = s + 1 < nstage;
    if (more) {
      load_w((s + 1) * DU_KC, wv);
      load_a((s + 1) * DU_KC, an);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int idx = (t * 32 + r32) * DU_LD + 2 * kk + g;
        au[t] = mma16(av[kk], s_b[buf][0][idx], au[t]);
        if constexpr (GATE) ag[t] = mma16(av[kk], s_b[buf][NMAT - 1][idx], ag[t]);
      }
    if (more) {
      store_w(buf ^ 1, wv);
      av[0] = an[0];
      av[1] = an[1];
    }
    __syncthreads();
  }

  // epilogue: h per (token, neuron), masked by the token's set, to H (fp16)
  const int W = a.ffn / 32;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = n0 + t * 32 + r32;
    const int nc = min(n, a.ffn - 1);
    const float bu = a.b_up ? a.b_up[nc] : 0.0f;
    const float bg = a.b_gate ? a.b_gate[nc] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + wave * 32 + acc_row(i, lane);
      const float u = au[t][i] + bu;
      float h;
      if constexpr (!GATE) {
        h = fmaxf(u, 0.0f);
      } else {
        const float gg = fmaxf(ag[t][i] + bg, 0.0f);
        h = a.act == FFN_ACT_REGLU ? gg * u : gg * fmaxf(u, 0.0f);
      }
      if (m < a.M && n < a.ffn) {
        if (a.bits && !((a.bits[(size_t)m * W + (n >> 5)] >> (n & 31)) & 1u)) h = 0.0f;
        a.H[(size_t)m * a.ffn + n] = (_Float16)h;
      }
    }
  }
}

__global__ __launch_bounds__(DT) void k_ddown(DenseArgs a) {
  __shared__ u32x4 s_b[2][DD_K * DD_LD];             // [buffer][k row * DD_LD + column chunk]
  if (a.run_if && *a.run_if != a.run_want) return;
  const int nb_m = (a.M + DD_M - 1) / DD_M, nb_n = (a.d + DD_N - 1) / DD_N;
  const int total = nb_m * nb_n * a.ks;
  const int tile = xcd_tile(total);
  if (tile >= total) return;
  const int mt = tile % nb_m, rest = tile / nb_m;
  const int nt = rest % nb_n, kslice = rest / nb_n;
  const int m0 = mt * DD_M, c0 = nt * DD_N;
  // this slice's ffn rows, in whole stages
  const int nst_all = a.ffn / DD_K;
  const int st0 = (int)((long long)nst_all * kslice / a.ks);
  const int st1 = (int)((long long)nst_all * (kslice + 1) / a.ks);
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
  auto load_a = [&](int k0, u32x4 (&v)[2]) {
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(arow + (size_t)(k0 + 16 * ss + 8 * g) * 2);
      v[ss] = aok ? t : u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x16 acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = f32x16{};

  if (st0 < st1) {
    u32x4 wv[4], av[2];
    load_w(st0 * DD_K, wv);
    load_a(st0 * DD_K, av);
    store_w(0, wv);
    __syncthreads();
    for (int s = st0; s < st1; ++s) {
      const int buf = (s - st0) & 1;
      const bool more = s + 1 < st1;
      u32x4 an[2];
      if (more) {
        load_w((s + 1) * DD_K, wv);
        load_a((s + 1) * DD_K, an);
      }
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
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
          acc[2 * q] = mma16(av[ss], lo, acc[2 * q]);
          acc[2 * q + 1] = mma16(av[ss], hi, acc[2 * q + 1]);
        }
      }
      if (more) {
        store_w(buf ^ 1, wv);
        av[0] = an[0];
        av[1] = an[1];
      }
      __syncthreads();
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
      const int m = m0 + w * 32 + row, col = c0 + 4 * c4;
      if (m < a.M && col < a.d)
        *reinterpret_cast<f32x4*>(a.ypart + ((size_t)kslice * a.M + m) * a.d + col) =
            *reinterpret_cast<const f32x4*>(&sy[row * DD_N + 4 * c4]);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_dred(DenseArgs a) {
  if (a.run_if && *a.run_if != a.run_want) return;
  const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;     // m * d + col
  if (e >= (size_t)a.M * a.d) return;
  const int col = (int)(e % a.d);
  f32x4 t = *reinterpret_cast<const f32x4*>(a.ypart + e);
  for (int k = 1; k < a.ks; ++k) t += *reinterpret_cast<const f32x4*>(a.ypart + (size_t)k * a.M * a.d + e);
  if (a.b_down) t += *reinterpret_cast<const f32x4*>(a.b_down + col);
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
  const int tiles = ((M + DD_M - 1) / DD_M) * ((d + DD_N - 1) / DD_N);
  // two workgroups per CU (the kernel's occupancy): split ffn until the grid reaches 512
  const int ks = std::max(1, std::min({8, (512 + tiles - 1) / tiles, ffn / DD_K}));
  return ks;
}

hipError_t launch_dense(const DenseArgs& a, hipStream_t st, hipEvent_t (*ev)[2]) {
  const int t_up = ((a.M + DU_M - 1) / DU_M) * ((a.ffn + DU_N - 1) / DU_N);
  const int t_dn = ((a.M + DD_M - 1) / DD_M) * ((a.d + DD_N - 1) / DD_N) * a.ks;
  const dim3 g_up(8 * ((t_up + 7) / 8)), g_dn(8 * ((t_dn + 7) / 8));
  const dim3 g_red((unsigned)(((size_t)a.M * a.d / 4 + 255) / 256));
  if (a.has_gate) {
    if (ev && ev[0][0])
      hipExtLaunchKernelGGL(k_dup<true>, g_up, dim3(DT), 0, st, ev[0][0], ev[0][1], 0, a);
    else
      hipLaunchKernelGGL(k_dup<true>, g_up, dim3(DT), 0, st, a);
  } else {
    if (ev && ev[0][0])
      hipExtLaunchKernelGGL(k_dup<false>, g_up, dim3(DT), 0, st, ev[0][0], ev[0][1], 0, a);
    else
      hipLaunchKernelGGL(k_dup<false>, g_up, dim3(DT), 0, st, a);
  }
  if (ev && ev[1][0])
    hipExtLaunchKernelGGL(k_ddown, g_dn, dim3(DT), 0, st, ev[1][0], ev[1][1], 0, a);
  else
    hipLaunchKernelGGL(k_ddown, g_dn, dim3(DT), 0, st, a);
  if (ev && ev[2][0])
    hipExtLaunchKernelGGL(k_dred, g_red, dim3(256), 0, st, ev[2][0], ev[2][1], 0, a);
  else
    hipLaunchKernelGGL(k_dred, g_red, dim3(256), 0, st, a);
  if (a.bits && (a.idx_out || a.cnt_out))
    hipLaunchKernelGGL(k_dlists, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ffn
