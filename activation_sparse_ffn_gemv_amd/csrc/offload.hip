// Neuron cache for FFN rows kept in host memory (PowerInfer-2, citnews.com.cn article, sections
// "Dynamic neuron cache" -- an in-memory pool of neurons under LRU replacement, segmented by
// weight type -- and neuron-cluster pipelining -- while some neurons wait for I/O, others are
// computed).  Here the "memory" is HBM and the "storage" is pinned host memory read over PCIe:
// the predictor segment (P1, P2, c1, c2) and the biases stay resident, and a pool of `capacity`
// slots holds the up / gate / down rows of recently used neurons.
//
// Per token, after the predictor's bitmap:
//   k_cache_plan  (one workgroup) ranks the active neurons, looks each up (hit: its slot, whose
//                 last use becomes the token's stamp), gives the misses -- in rank order -- the
//                 free or least recently used slots not used by this token (ascending (last
//                 use, slot), by a bitonic sort in LDS), evicts their previous neurons and
//                 updates the tables; misses beyond those slots are read but not admitted;
//   k_gather<..., CACHED> reads a hit's rows from its slot in HBM and a miss's rows from host
//                 memory, in the same rank-balanced rounds as the resident gather (so the
//                 arithmetic, and y, are bit-identical to the resident layer), and writes an
//                 admitted miss's rows into its slot on the way: the PCIe reads of the misses
//                 overlap the HBM reads of the hits inside every workgroup.
// No atomics: one workgroup owns the tables, and a slot is written only by the gather
// workgroup that owns its (single) admitted neuron.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace ffn {

constexpr int CP_THREADS = 1024;
constexpr int CP_NW = CP_THREADS / WAVE;
constexpr uint32_t CP_PINNED = 0xFFFFFFFFu;

// Exclusive prefix of v over the workgroup (fixed order); total in *sum.
__device__ __forceinline__ int block_scan(int v, int* s_wsum, int* sum) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  int incl = v;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const int u = __shfl_up(incl, o, WAVE);
    if (lane >= o) incl += u;
  }
  __syncthreads();                                   // s_wsum may still be read
  if (lane == WAVE - 1) s_wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < CP_NW; ++w) {
    base += w < wave ? s_wsum[w] : 0;
    tot += s_wsum[w];
  }
  *sum = tot;
  return base + incl - v;
}

__global__ __launch_bounds__(CP_THREADS) void k_cache_plan(CacheArgs a) {
  __shared__ unsigned long long s_key[CACHE_MAX_SLOTS];
  __shared__ int s_wsum[CP_NW];
  const int tid = threadIdx.x;
  const uint32_t stamp = *a.stamp + 1u;

  // 1. ranks: thread t owns bitmap word t (ffn <= 32768)
  const int W = a.ffn / 32;
  const uint32_t bw = tid < W ? a.bitmap[tid] : 0u;
  int total = 0;
  int pos = block_scan(__popc(bw), s_wsum, &total);
  for (uint32_t bb = bw; bb; bb &= bb - 1) a.rank_nid[pos++] = tid * 32 + __builtin_ctz(bb);
  __syncthreads();                                   // rank_nid written by other threads

  // 2. hits: the slot they are read from, touched with the stamp; misses get their miss index
  // (rank order) in rank_vic for now
  int misses = 0, hits = 0;
  for (int j0 = 0; j0 < total; j0 += CP_THREADS) {
    const int j = j0 + tid;
    int s = -1;
    if (j < total) {
      s = a.slot_of[a.rank_nid[j]];
      a.rank_src[j] = s;
      if (s >= 0 && a.last_use[s] != CP_PINNED) a.last_use[s] = stamp;
    }
    const bool miss = j < total && s < 0;
    int m = 0;
    const int q = block_scan(miss ? 1 : 0, s_wsum, &m);
    if (miss) a.rank_vic[j] = misses + q;
    else if (j < total) a.rank_vic[j] = -1;
    misses += m;
    hits += min(CP_THREADS, total - j0) - m;
  }
  __syncthreads();                                   // last_use of the hits

  // 3. the evictable slots (not used by this token, not pinned: last use < stamp) in ascending
  // (last use, slot) order
  int avail = 0;
  if (misses > 0) {                                  // uniform
    int npad = 1;
    while (npad < a.cap) npad <<= 1;
    int mine = 0;
    for (int i = tid; i < npad; i += CP_THREADS) {
      unsigned long long k = ~0ull;
      if (i < a.cap) {
        const uint32_t lu = a.last_use[i];
        if (lu < stamp) {
          k = ((unsigned long long)lu << 32) | (unsigned)i;
          ++mine;
        }
      }
      s_key[i] = k;
    }
    block_scan(mine, s_wsum, &avail);                // also orders the key stores
    for (int k = 2; k <= npad; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < npad; i += CP_THREADS) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const unsigned long long x = s_key[i], y = s_key[ixj];
            if ((x > y) == ((i & k) == 0)) {
              s_key[i] = y;
              s_key[ixj] = x;
            }
          }
        }
        __syncthreads();
      }

    // 4. admissions: miss q takes the q-th evictable slot; evictions first, then the new
    // mappings (an evicted neuron is not active this token, so the two never collide)
    for (int j = tid; j < total; j += CP_THREADS) {
      const int q = a.rank_vic[j];
      if (q >= 0) {
        const int v = q < avail ? (int)(s_key[q] & 0xFFFFFFFFull) : -1;
        a.rank_vic[j] = v;
        if (v >= 0) {
          const int old = a.neuron_of[v];
          if (old >= 0) a.slot_of[old] = -1;
        }
      }
    }
    __syncthreads();
    for (int j = tid; j < total; j += CP_THREADS) {
      const int v = a.rank_vic[j];
      if (v >= 0) {
        const int n = a.rank_nid[j];
        a.slot_of[n] = v;
        a.neuron_of[v] = n;
        a.last_use[v] = stamp;
      }
    }
  }
  if (tid == 0) {
    *a.stamp = stamp;
    *a.cnt = total;
    const int st[4] = {hits, misses, min(misses, avail), total};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a.stats[i] = st[i];
      a.stats[4 + i] = (int)((uint32_t)a.stats[4 + i] + (uint32_t)st[i]);   // running totals
    }
  }
}

// Tables of a new cache: neurons [0, n_pinned) pinned in slots [0, n_pinned), the rest free.
__global__ __launch_bounds__(256) void k_cache_init(CacheArgs a, int n_pinned) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < a.ffn) a.slot_of[i] = i < n_pinned ? i : -1;
  if (i < a.cap) {
    a.neuron_of[i] = i < n_pinned ? i : -1;
    a.last_use[i] = i < n_pinned ? CP_PINNED : 0u;
  }
  if (i < 8) a.stats[i] = 0;
  if (i == 0) *a.stamp = 0u;
}

hipError_t launch_cache_plan(const CacheArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_cache_plan, dim3(1), dim3(CP_THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_cache_init(const CacheArgs& a, int n_pinned, hipStream_t st) {
  const int n = std::max(a.ffn, a.cap);
  hipLaunchKernelGGL(k_cache_init, dim3((n + 255) / 256), dim3(256), 0, st, a, n_pinned);
  return hipGetLastError();
}

}  // namespace ffn
