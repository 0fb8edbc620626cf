// Index arithmetic of the kernels that split work between workgroups and exchange partial
// results through the workspace (and the GEMMs' tile and K-slice maps), as host-and-device functions: the kernels call them, and a CPU
// build of the same functions (tests/index_check.cpp) walks every workgroup and thread of the
// launch shapes the library uses and checks that each index stays inside its buffer, that
// writers and readers agree, and that the 32-bit products never wrap.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ffn {

// Columns of y per tile of the batch-1 partial sums: the gather stores its partial tile-major,
// part[col / RD_TW][workgroup][col % RD_TW], so the reduce reads one contiguous block per tile.
constexpr int RD_TW = 16;

// Ranks [r0, r1) of the active set owned by gather workgroup b of nblk (an even split).
// 32-bit exact for total <= 32768 and nblk <= 512: total * nblk < 2^24.
__host__ __device__ inline void gather_rank_range(uint32_t total, uint32_t b, uint32_t nblk,
                                                  int& r0, int& r1) {
  r0 = (int)((total * b) / nblk);
  r1 = (int)((total * (b + 1)) / nblk);
}

// Whether gather workgroup b of nblk owned a rank (so wrote a partial).
__host__ __device__ inline bool gather_wrote_partial(uint32_t total, uint32_t b, uint32_t nblk) {
  return (total * (b + 1)) / nblk > (total * b) / nblk;
}

// Element offset of column col of workgroup blk's partial (nblk partials), tile-major.
__host__ __device__ inline size_t part_offset(int col, int blk, int nblk) {
  return ((size_t)(col / RD_TW) * nblk + blk) * RD_TW + col % RD_TW;
}

// Union ranks [r0, r1) of segment s of S of the batched down projection: segments are cut at
// multiples of 8 ranks (one 8-deep MFMA step).  32-bit exact: total <= 32768 (so at most 4096
// units) and s + 1 <= S <= 64.
__host__ __device__ inline void seg_range(int total, int s, int S, int& r0, int& r1) {
  const uint32_t units = ((uint32_t)total + 7u) / 8u;
  r0 = (int)(8u * (units * (uint32_t)s / (uint32_t)S));
  r1 = (int)(8u * (units * (uint32_t)(s + 1) / (uint32_t)S));
}

// Workgroup id -> (weight block, pass) for a launch over nb weight blocks and `passes` passes.
// Workgroup id runs on XCD id % 8 (consecutive workgroups go to the eight XCDs in turn); the
// passes of one block go to consecutive workgroups of one XCD, so that they run side by side and
// read the block's weights from that XCD's L2 instead of once per pass from HBM.  nb not a
// multiple of 8: plain block-major order.
__host__ __device__ inline void xcd_block_pass(int id, int nb, int passes, int& bx, int& p) {
  if (passes == 1) {
    bx = id;
    p = 0;
  } else if (nb % 8) {
    bx = id % nb;
    p = id / nb;
  } else {
    const int k = id / 8;
    p = k % passes;
    bx = (k / passes) * 8 + id % 8;
  }
}

// Element offsets of pass p's share of the batched path's buffers when the passes of one call
// run in one launch (tokens [32 p, 32 p + 32)); strides per pass in elements.
struct PassOffsets {
  size_t tok;                 // tokens before the pass
  size_t zpart, zhl, ubits, ucnt, uidx, ypart;
};
__host__ __device__ inline PassOffsets pass_offsets(int p, int tile, size_t zpart_ps,
                                                    size_t zhl_ps, size_t ubits_ps,
                                                    size_t uidx_ps, size_t ypart_ps) {
  PassOffsets o;
  o.tok = (size_t)p * tile;
  o.zpart = (size_t)p * zpart_ps;
  o.zhl = (size_t)p * zhl_ps;
  o.ubits = (size_t)p * ubits_ps;
  o.ucnt = (size_t)p;
  o.uidx = (size_t)p * uidx_ps;
  o.ypart = (size_t)p * ypart_ps;
  return o;
}

// Row (within its 32-row block) of accumulator element i of lane `lane` of a 32 x 32 MFMA
// output block: lanes 0-31 hold rows 8 (i / 4) + i % 4, lanes 32-63 the rows four further on.
__host__ __device__ inline int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// Workgroup b of a GEMM grid of 8 ceil(total / 8) workgroups -> its tile id, such that
// consecutive ids run on one XCD (workgroup b runs on XCD b % 8); ids >= total are idle.
__host__ __device__ inline int xcd_tile_of(int b, int total) {
  const int per = (total + 7) / 8;
  return (b % 8) * per + b / 8;
}

// K stages [s0, s0 + n) of slice k of ks over nst_all stages (an even split; n >= 1 when
// ks <= nst_all).
__host__ __device__ inline void slice_stages(int nst_all, int k, int ks, int& s0, int& n) {
  s0 = (int)((long long)nst_all * k / ks);
  n = (int)((long long)nst_all * (k + 1) / ks) - s0;
}

// Tile id -> (token tile mt, column tile nt, K slice k) of the dense GEMMs, token tiles fastest:
// the token tiles that share a weight tile have consecutive ids, so they run on one XCD.
__host__ __device__ inline void gemm_tile(int tile, int nb_m, int nb_n, int& mt, int& nt,
                                          int& k) {
  mt = tile % nb_m;
  nt = tile / nb_m % nb_n;
  k = tile / (nb_m * nb_n);
}

// Down-projection tiles: k_ddown 128 tokens x 256 columns, k_ddq 256 x 256.  k_ddq takes the
// token counts whose 256-token tiles pad no more than 128-token ones.
constexpr int DD_M = 128, DD_N = 256;
constexpr int DQ_M = 256, DQ_N = 256;
__host__ __device__ inline bool dense_down_wide(int M) {
  return (M + DQ_M - 1) / DQ_M * DQ_M == (M + DD_M - 1) / DD_M * DD_M;
}

// Predictor stage 1 of a large call (Z = X P1^T, rank columns): 128 tokens x 128 columns per
// tile, so that the GPU fills with fewer K slices (fewer fp32 partials to write and sum).
constexpr int ZP_M = 128, ZP_N = 128;

// Stage-1 GEMM epilogue: accumulator element i of lane's block (ms, ns) of wave `wave` (8 waves,
// 2 per row of the tile) in the tm x tn tile at (m0, n0) -> token m, rank column n.
__host__ __device__ inline void zpart_store_pos(int m0, int n0, int tm, int tn, int wave, int ms,
                                                int ns, int i, int lane, int& m, int& n) {
  m = m0 + (wave >> 1) * (tm / 4) + ms * 32 + acc_row(i, lane);
  n = n0 + (wave & 1) * (tn / 2) + ns * 32 + (lane & 31);
}
// Offset of (token m, K slice k, column n) of the stage-1 partials, per-pass layout
// [pass = m / 32][slice][m % 32][N] with zpart_ps elements per pass.
__host__ __device__ inline size_t zpart_offset(int m, int k, int n, int N, size_t zpart_ps) {
  return (size_t)(m / 32) * zpart_ps + ((size_t)k * 32 + m % 32) * N + n;
}

// k_ddq's partial-sum store of lane `lane` of wave `wave`, 32-token block ms, accumulator
// element i: token m and the first of the lane's four consecutive columns col (MFMA block b
// holds column 4 (lane % 32) + b of the wave's 128).
__host__ __device__ inline void ddq_store_pos(int m0, int c0, int wave, int ms, int i, int lane,
                                              int& m, int& col) {
  m = m0 + (wave >> 1) * 64 + ms * 32 + acc_row(i, lane);
  col = c0 + (wave & 1) * 128 + 4 * (lane & 31);
}

// k_ddown's partial-sum store: wave w's 32 x 256 tile staged through LDS, element e of the
// workgroup's pass over it (four columns each): token m and first column col.
__host__ __device__ inline void ddown_store_pos(int m0, int c0, int w, int e, int& m, int& col) {
  m = m0 + w * 32 + e / (DD_N / 4);
  col = c0 + 4 * (e % (DD_N / 4));
}

// Attention block.  Chunks of a context of n positions for the score kernel: about 1024 / H
// chunks per head (so that half the heads active give ~512 workgroups), each a whole number of
// the kernel's steps of `step` positions, at most max_chunks; every chunk holds >= 1 position.
__host__ __device__ inline void attn_chunk_split(int H, int step, int n, int max_chunks, int& lc,
                                                 int& nchunk) {
  int target = (1024 + H - 1) / H;
  target = target < 1 ? 1 : target > max_chunks ? max_chunks : target;
  int per = (n + target - 1) / target;
  per = (per + step - 1) / step * step;
  lc = per;
  nchunk = (n + per - 1) / per;
}

// Output-projection rows [r0, r1) of workgroup b of nblk (an even split of `rows` ranked rows).
// 32-bit exact for rows <= 16384 and nblk <= 256 (rows * nblk < 2^23).
__host__ __device__ inline void attn_out_rows(int rows, int b, int nblk, int& r0, int& r1) {
  r0 = (int)((uint32_t)rows * (uint32_t)b / (uint32_t)nblk);
  r1 = (int)((uint32_t)rows * (uint32_t)(b + 1) / (uint32_t)nblk);
}

// Element offset of chunk ch's record (e values of o, then max and sum) of the head of rank k.
__host__ __device__ inline size_t attn_rec_offset(int k, int ch, int e, int max_chunks) {
  return ((size_t)k * max_chunks + ch) * (size_t)(e + 4);
}

}  // namespace ffn
