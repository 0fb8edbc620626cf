// Internal device helpers and the plan object of libffn_sparse (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ffn_sparse.h"

namespace ffn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Storage kinds of a weight row.  Every row is read in 16-byte chunks: 4 fp32, 8 fp16 or
// 32 int4 elements (one int4 group of 32 = one chunk, so each chunk has exactly one scale).
enum { WK_F32 = 0, WK_F16 = 1, WK_I4 = 2 };

template <int WK> struct Kind;
template <> struct Kind<WK_F32> { static constexpr int EPC = 4;  static constexpr int XW = 1; };
template <> struct Kind<WK_F16> { static constexpr int EPC = 8;  static constexpr int XW = 1; };
// int4 chunk: 32 elements; the matching token slice is 32 fp16 = four 16-byte words.
template <> struct Kind<WK_I4>  { static constexpr int EPC = 32; static constexpr int XW = 4; };

constexpr int WAVE = 64;

// Optional timeline trace (builds with -DFFN_TRACE only): thread 0 of every workgroup stores the
// 100 MHz real-time counter at a few points of a kernel into trace[(kernel * 4096 + block) * 8 +
// point] (kernel 0 predictor stage 1, 3 stage 2, 1 gather, 2 reduce).  The buffer is set with
// ffn_trace_set_buffer (declared in the trace build only).
#ifdef FFN_TRACE
extern __device__ unsigned long long* g_trace;
#define FFN_TS(K, PH)                                                                          \
  do {                                                                                         \
    if (threadIdx.x == 0 && g_trace)                                                           \
      g_trace[((K) * 4096 + blockIdx.x) * 8 + (PH)] = __builtin_amdgcn_s_memrealtime();        \
  } while (0)
#define FFN_TV(K, PH, V)                                                                       \
  do {                                                                                         \
    if (threadIdx.x == 0 && g_trace) g_trace[((K) * 4096 + blockIdx.x) * 8 + (PH)] = (V);      \
  } while (0)
#define FFN_TRACE_SYNC() __syncthreads()
#else
#define FFN_TS(K, PH) ((void)0)
#define FFN_TV(K, PH, V) ((void)0)
#define FFN_TRACE_SYNC() ((void)0)
#endif

// DPP lane exchange (gfx9 data-parallel primitives): lanes of rows outside ROW_MASK read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, false));
}

// Sum over aligned groups of 16 lanes; every lane of the group gets the sum.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xb1>(v);
  v += dpp<0x4e>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

// Sum over the 64 lanes of a wave, returned to every lane (row sums, then row_bcast15 into rows
// 1 and 3, row_bcast31 into rows 2 and 3: lane 63 holds the total).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += dpp<0x142, 0xa>(v);
  v += dpp<0x143, 0xc>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over aligned groups of `width` lanes (a power of two, 4 <= width <= 64).  The sum is valid
// in the last lane of each group (lane % width == width - 1); for width <= 16 in every lane.
__device__ __forceinline__ float group_sum_last(float v, int width) {
  v += dpp<0xb1>(v);
  v += dpp<0x4e>(v);
  if (width >= 8) v += dpp<0x141>(v);
  if (width >= 16) v += dpp<0x140>(v);
  if (width >= 32) v += dpp<0x142, 0xa>(v);
  if (width >= 64) v += dpp<0x143, 0xc>(v);
  return v;
}

// Scheduling fence: the compiler may not move instructions across it.  Placed between the
// instructions that issue a batch of loads and the first use of their results, so that the
// whole batch is in flight before the wave waits (instead of load / wait / use one by one).
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// 16-byte load from device (or mapped host) memory, issued as a global load.  Pointers fetched
// from memory (expert slot records) are generic to the compiler, and generic loads both count
// against the LDS counter and make it wait early, so every weight / token read goes through here.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *(const __attribute__((address_space(1))) u32x4*)p;
}

// Element i of a device array, as a global load.
template <class T>
__device__ __forceinline__ T ldg(const T* p, size_t i) {
  return ((const __attribute__((address_space(1))) T*)p)[i];
}

// The 32-bit word holding fp16 element i (an int4 group scale) of an array of an even number of
// elements, as a global load; pick_h takes the element out of it once the value is needed.
// A 16-bit load would be merged into a register half as soon as it lands, which needs a wait.
__device__ __forceinline__ uint32_t ldh_word(const void* p, size_t i) {
  return ((const __attribute__((address_space(1))) uint32_t*)p)[i >> 1];
}

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// fp16 x fp16 pairs, fp32 accumulate (v_dot2_f32_f16: the products are exact in fp32).
__device__ __forceinline__ float dot8_f16(u32x4 w, u32x4 x, float acc) {
  acc = __builtin_amdgcn_fdot2(as_h2(w.x), as_h2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(w.y), as_h2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(w.z), as_h2(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(w.w), as_h2(x.w), acc, false);
  return acc;
}

__device__ __forceinline__ float dot4_f32(u32x4 w, u32x4 x, float acc) {
  f32x4 a = __builtin_bit_cast(f32x4, w), b = __builtin_bit_cast(f32x4, x);
  acc = __builtin_fmaf(a.x, b.x, acc);
  acc = __builtin_fmaf(a.y, b.y, acc);
  acc = __builtin_fmaf(a.z, b.z, acc);
  acc = __builtin_fmaf(a.w, b.w, acc);
  return acc;
}

__device__ __forceinline__ float h_lo(uint32_t v) { return (float)as_h2(v).x; }
__device__ __forceinline__ float h_hi(uint32_t v) { return (float)as_h2(v).y; }
__device__ __forceinline__ float pick_h(uint32_t v, size_t i) { return i & 1 ? h_hi(v) : h_lo(v); }

// int4 group: 16 bytes = 32 signed nibbles, element 2k in the low nibble of byte k.
// Decoding: flipping the sign bit of each nibble gives n' = q + 8 in [0, 15]; the fp16 with bit
// pattern 0x6400 | n' equals 1024 + n', so subtracting 1032 gives q exactly.  Even and odd
// elements are split with masks, so the fp16 pairs hold elements (4m, 4m+2) and (4m+1, 4m+3);
// the token slice is pre-permuted into the same pair order once (see i4_perm_x).
__device__ __forceinline__ float dot32_i4(u32x4 w, const u32x4* xp, float scale, float acc) {
  const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  float part = 0.0f;
  uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t t = words[k] ^ 0x88888888u;
    uint32_t ev = t & 0x0F0F0F0Fu;          // elements 8k+0, +2, +4, +6 (one per byte)
    uint32_t od = (t >> 4) & 0x0F0F0F0Fu;   // elements 8k+1, +3, +5, +7
    // byte-interleave with 0x64: pairs (e0,e2) (e4,e6) (o1,o3) (o5,o7)
    uint32_t p0 = __builtin_amdgcn_perm(0x64646464u, ev, 0x07010700u);
    uint32_t p1 = __builtin_amdgcn_perm(0x64646464u, ev, 0x07030702u);
    uint32_t p2 = __builtin_amdgcn_perm(0x64646464u, od, 0x07010700u);
    uint32_t p3 = __builtin_amdgcn_perm(0x64646464u, od, 0x07030702u);
    u32x4 xv = xp[k];
    part = __builtin_amdgcn_fdot2(as_h2(p0) - bias, as_h2(xv.x), part, false);
    part = __builtin_amdgcn_fdot2(as_h2(p1) - bias, as_h2(xv.y), part, false);
    part = __builtin_amdgcn_fdot2(as_h2(p2) - bias, as_h2(xv.z), part, false);
    part = __builtin_amdgcn_fdot2(as_h2(p3) - bias, as_h2(xv.w), part, false);
  }
  return __builtin_fmaf(part, scale, acc);
}

// Reorder a 32-element fp16 token slice (four 16-byte words, natural order) into the pair order
// dot32_i4 consumes: per 8 elements e0..e7 -> (e0,e2) (e4,e6) (e1,e3) (e5,e7).
__device__ __forceinline__ void i4_perm_x(u32x4* xs) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x4 v = xs[k];  // halves: v.x = (e0,e1), v.y = (e2,e3), v.z = (e4,e5), v.w = (e6,e7)
    u32x4 o;
    o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (e0, e2)
    o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (e4, e6)
    o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (e1, e3)
    o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (e5, e7)
    xs[k] = o;
  }
}

// Token slice held in registers: lane `l` owns 16-byte row chunks l, l+64, l+128, ...
template <int WK, int CPL>
struct XRegs {
  u32x4 v[CPL][Kind<WK>::XW];
};

// Raw loads only (clamped, so never predicated): finish_x, called once every load of the caller
// is issued, zeroes the chunks past the row end and puts int4 slices in nibble order.  Doing that
// here would make the wave wait for the token before it issues its weight loads.
template <int WK, int CPL>
__device__ __forceinline__ void load_x(XRegs<WK, CPL>& xr, const void* x, int nch, int lane) {
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int cc = min(lane + k * WAVE, nch - 1);
#pragma unroll
    for (int q = 0; q < Kind<WK>::XW; ++q)
      // fp32 / fp16 rows: 16 token bytes per chunk.  int4 rows: 32 fp16 token values per chunk.
      xr.v[k][q] = ld16(static_cast<const char*>(x) + (size_t)cc * 16 * Kind<WK>::XW + q * 16);
  }
}

template <int WK, int CPL>
__device__ __forceinline__ void finish_x(XRegs<WK, CPL>& xr, int nch, int lane) {
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const bool in = lane + k * WAVE < nch;
#pragma unroll
    for (int q = 0; q < Kind<WK>::XW; ++q)
      xr.v[k][q] = in ? xr.v[k][q] : u32x4{0u, 0u, 0u, 0u};
    if constexpr (WK == WK_I4) i4_perm_x(xr.v[k]);
  }
}

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
  // Chunks past the row end (ragged d) re-read the last chunk and meet a zero token slice.
  const char* rp = static_cast<const char*>(base) + row * (size_t)nch * 16;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int cc = min(lane + k * WAVE, nch - 1);
    w[k] = ld16(rp + (size_t)cc * 16);
    if constexpr (WK == WK_I4) {
      const _Float16* sp = static_cast<const _Float16*>(scales) + row * (size_t)nch;
      sc[k] = (float)sp[cc];
    } else {
      sc[k] = 0.0f;
    }
  }
}


// Exclusive prefix sum over the wave of v, for 0 <= v < 2^BITS, and the wave's total, without
// lane exchanges: bit j of v is counted by a ballot of that bit and the lanes below this one in it
// (mbcnt), weighted 2^j.  Every lane of the wave must be active.
template <int BITS>
__device__ __forceinline__ int wave_prefix_small(int v, int& total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < BITS; ++j) {
    const unsigned long long m = __ballot((v >> j) & 1);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    pre += (int)below << j;
    tot += __popcll(m) << j;
  }
  total = tot;
  return pre;
}

// Ascending list of the set bits of bitmap[0 .. words) (neuron w*32 + b for bit b of word w) and
// its length, written by one workgroup of NT threads.  idx_out / cnt_out may each be nullptr.
template <int NT>
__device__ void write_index_list(const uint32_t* __restrict__ bitmap, int words,
                                 int* __restrict__ idx_out, int* __restrict__ cnt_out) {
  __shared__ int s_ws[NT / WAVE];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  int before = 0;
  for (int w0 = 0; w0 < words; w0 += NT) {
    const int w = w0 + tid;
    const uint32_t b = w < words ? bitmap[w] : 0u;
    const int c = __popc(b);
    int v = c;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
      const int u = __shfl_up(v, o, WAVE);
      if (lane >= o) v += u;
    }
    __syncthreads();
    if (lane == WAVE - 1) s_ws[wave] = v;
    __syncthreads();
    int base = before, tot = 0;
    for (int k = 0; k < NT / WAVE; ++k) {
      base += k < wave ? s_ws[k] : 0;
      tot += s_ws[k];
    }
    if (idx_out) {
      int pos = base + v - c;
      uint32_t bb = b;
      while (bb) {
        idx_out[pos++] = w * 32 + __builtin_ctz(bb);
        bb &= bb - 1;
      }
    }
    before += tot;
  }
  if (tid == 0 && cnt_out) *cnt_out = before;
}

}  // namespace ffn

// ----------------------------------------------------------------------------------------------
// Host-side plan.
struct ffn_plan {
  ffn_layer_desc desc;
  ffn_layer_weights w;
  char* ws;
  size_t ws_bytes;
  int cpl_w;         // 16-byte chunks per lane for a weight row
  int cpl_p;         // 16-byte chunks per lane for a predictor P1 row
  float thr;         // logit(threshold): active iff score > thr
  size_t off_z, off_bits, off_cnt, off_part;
  size_t off_batch;  // batched-path region (fp16 layers with max_batch > 1), else 0
  size_t off_dense;  // dense-GEMM region (fp16 layers with max_batch >= 64), else 0
  size_t dense_ypart_rows;      // rows of the dense partial buffer (max over M of ks * M)
  float crossover_density[13];  // per batch bucket 1, 2, 4, ..., 4096
  int dense_min_batch;          // AUTO takes the dense path from this batch size on
  hipEvent_t ev[9][2];          // instrumentation events attached to each stage's dispatch
  int decode_variant;           // batch-1 decode: 0 rank-balanced gather, 1 fused predictor + gather
  int head_words;               // hot head: neurons [0, 32 head_words) always active
  int cache_cap;                // neuron cache slots (host-resident rows), 0: rows resident
  size_t off_cache;             // the cache region of the workspace
};
