// CPU build of the kernels' index arithmetic (activation_sparse_ffn_gemv_amd/csrc/index.h, the
// functions the kernels call) under AddressSanitizer / UndefinedBehaviorSanitizer, walked over
// every workgroup and thread of the launch shapes the library uses: every index must stay inside
// its buffer, the gather's partial writes and the reduce's reads must address the same elements,
// the work splits must partition their ranges exactly, and no 32-bit product may wrap.  The
// shapes come from the built library's own host functions (workgroup counts, tiles, the batched
// path's buffer shapes, the dense down projection's and the stage-1 GEMM's K slices, the
// attention kernels' steps).  Exit status 0 and "index check: OK" when every check holds.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "../activation_sparse_ffn_gemv_amd/csrc/index.h"
#include "../activation_sparse_ffn_gemv_amd/csrc/launch.h"

using namespace ffn;

static long checks = 0, failures = 0;

#define CHECK(cond, ...)                                                  \
  do {                                                                    \
    ++checks;                                                             \
    if (!(cond)) {                                                        \
      if (failures < 20) {                                                \
        printf("FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond);            \
        printf(__VA_ARGS__);                                              \
        printf("\n");                                                     \
      }                                                                   \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

// Batch-1 gather -> reduce: nblk workgroups split `total` ranks; each writes the partial of all
// d columns (16-byte pieces of 4 floats); the reduce reads tile by tile.
static void check_partials(int d, int ffn, int nblk) {
  const int tiles = reduce_tiles(d);
  const size_t region = (size_t)nblk * tiles * RD_TW;           // the layout's partial block
  std::vector<unsigned char> written(region, 0);
  for (int blk = 0; blk < nblk; ++blk)
    for (int col = 0; col < d; col += 4) {                       // the gather's f32x4 stores
      const size_t o = part_offset(col, blk, nblk);
      CHECK(o + 3 < region, "d %d nblk %d blk %d col %d offset %zu region %zu", d, nblk, blk,
            col, o, region);
      if (o + 3 < region)
        for (int e = 0; e < 4; ++e) {
          CHECK(!written[o + e], "element written twice: d %d blk %d col %d", d, blk, col);
          written[o + e] = 1;
        }
    }
  for (int tile = 0; tile < tiles; ++tile)                       // the reduce's f32x4 reads
    for (int c = 0; c < nblk; ++c)
      for (int q = 0; q < RD_TW / 4; ++q) {
        const int col = tile * RD_TW + q * 4;
        const size_t o = part_offset(col, c, nblk);
        CHECK(o + 3 < region, "reduce read out of the region: d %d tile %d c %d", d, tile, c);
        if (col < d && o + 3 < region)                           // columns the reduce stores
          CHECK(written[o] && written[o + 3], "reduce reads an unwritten column %d", col);
      }
  // rank split: consecutive, covering [0, total) exactly, balanced; the existence test agrees
  const int totals[] = {0, 1, 7, nblk - 1, nblk, nblk + 1, 1093, ffn / 2, ffn - 1, ffn};
  for (int total : totals) {
    if (total < 0 || total > ffn) continue;
    int prev = 0;
    for (int b = 0; b < nblk; ++b) {
      int r0, r1;
      gather_rank_range((uint32_t)total, (uint32_t)b, (uint32_t)nblk, r0, r1);
      const long long e0 = (long long)total * b / nblk, e1 = (long long)total * (b + 1) / nblk;
      CHECK(r0 == e0 && r1 == e1, "32-bit rank split wraps: total %d b %d nblk %d", total, b,
            nblk);
      CHECK(r0 == prev && r1 >= r0, "ranks not consecutive: total %d b %d", total, b);
      CHECK(r1 - r0 <= (total + nblk - 1) / nblk, "unbalanced split: total %d b %d", total, b);
      CHECK(gather_wrote_partial((uint32_t)total, (uint32_t)b, (uint32_t)nblk) == (r1 > r0),
            "existence test disagrees: total %d b %d", total, b);
      prev = r1;
    }
    CHECK(prev == total, "split does not cover [0, %d)", total);
  }
}

// Batched down projection: S segments of the union ranks, cut at multiples of 8.
static void check_segments() {
  for (int S = 1; S <= 64; ++S)
    for (int total = 0; total <= 32768; total += (total < 300 ? 1 : 97)) {
      int prev = 0;
      const long long units = (total + 7) / 8;
      for (int s = 0; s < S; ++s) {
        int r0, r1;
        seg_range(total, s, S, r0, r1);
        CHECK(r0 == 8 * (units * s / S) && r1 == 8 * (units * (s + 1) / S),
              "32-bit segment split wraps: total %d S %d s %d", total, S, s);
        CHECK(r0 == prev && r1 >= r0 && r0 % 8 == 0, "segments not consecutive: %d %d", S, s);
        prev = r1;
      }
      CHECK(prev == 8 * units, "segments do not cover the union: total %d S %d", total, S);
    }
}

// (block, pass) order of a multi-pass launch: a bijection onto [0, nb) x [0, passes).
static void check_xcd_order() {
  const int passes_list[] = {1, 2, 3, 16, 128};
  for (int nb = 1; nb <= 520; ++nb)
    for (int passes : passes_list) {
      std::vector<unsigned char> seen((size_t)nb * passes, 0);
      for (int id = 0; id < nb * passes; ++id) {
        int bx, p;
        xcd_block_pass(id, nb, passes, bx, p);
        CHECK(bx >= 0 && bx < nb && p >= 0 && p < passes, "nb %d passes %d id %d -> %d %d", nb,
              passes, id, bx, p);
        if (bx >= 0 && bx < nb && p >= 0 && p < passes) {
          CHECK(!seen[(size_t)p * nb + bx], "pair given twice: nb %d passes %d", nb, passes);
          seen[(size_t)p * nb + bx] = 1;
        }
      }
    }
}

// The passes of one call in one launch: each pass's share of every buffer lies inside the
// region laid out for ceil(max_batch / 32) passes, and the kernels' largest index inside a pass
// stays below the pass's stride.
static void check_passes(int d, int ffn, int r, int max_batch) {
  const BatchShape s = batch_shape(d, ffn, r);
  const int P = (max_batch + BATCH_TILE - 1) / BATCH_TILE;
  const int S = batch_segments_mp(d, P);
  const size_t zpart_ps = s.zpart_bytes / 4, zhl_ps = s.zhl_bytes / 2, ubits_ps = ffn / 32,
               uidx_ps = ffn, ypart_ps = (size_t)S * BATCH_TILE * d;
  // largest element index each kernel touches inside one pass
  CHECK((size_t)(s.ks - 1) * BATCH_TILE * r + (size_t)(BATCH_TILE - 1) * r + (r - 1) < zpart_ps,
        "predictor stage-1 partials overflow a pass: d %d r %d", d, r);
  CHECK((size_t)BATCH_TILE * r + (size_t)BATCH_TILE * r - 1 < zhl_ps + 0, "z hi/lo overflow");
  CHECK(((size_t)(S - 1) * BATCH_TILE + BATCH_TILE - 1) * d + (d - 1) < ypart_ps,
        "segment partials overflow a pass: d %d S %d", d, S);
  CHECK(S >= 1 && S <= 64, "segments per pass %d", S);
  for (int B = 64; B <= max_batch; B += (B < 200 ? 1 : 61)) {
    const int Pc = (B + BATCH_TILE - 1) / BATCH_TILE;
    CHECK(Pc <= P, "a call of %d tokens needs %d passes, the region holds %d", B, Pc, P);
    for (int p = 0; p < Pc; ++p) {
      const PassOffsets o = pass_offsets(p, BATCH_TILE, zpart_ps, zhl_ps, ubits_ps, uidx_ps,
                                         ypart_ps);
      const int Bp = std::min(BATCH_TILE, B - p * BATCH_TILE);
      CHECK(Bp >= 1 && o.tok + Bp <= (size_t)B, "pass %d of %d tokens: tokens out of range", p, B);
      CHECK(o.zpart + zpart_ps <= (size_t)P * zpart_ps, "zpart");
      CHECK(o.zhl + zhl_ps <= (size_t)P * zhl_ps, "zhl");
      CHECK(o.ubits + ubits_ps <= (size_t)P * ubits_ps, "ubits");
      CHECK(o.ucnt + 1 <= (size_t)P, "ucnt");
      CHECK(o.uidx + uidx_ps <= (size_t)P * uidx_ps, "uidx");
      CHECK(o.ypart + ypart_ps <= (size_t)P * ypart_ps, "ypart");
      // H rows of the pass (every one of its 32 rows is written, the last pass's too)
      CHECK(o.tok + BATCH_TILE <= (size_t)P * BATCH_TILE, "H rows");
    }
  }
}


// Dense down projection (k_ddq or k_ddown by the token count): the grid's tiles are each
// (token tile, column tile, K slice) once, the K slices split the ffn stages with none empty,
// and every (slice, token, column) element of the partial-sum buffer [ks][M][d] is stored exactly
// once by the epilogue's index arithmetic, inside the buffer.
static void check_dense_down(int M, int d, int ffn) {
  const bool wide = dense_down_wide(M);
  const int TM = wide ? DQ_M : DD_M, TN = wide ? DQ_N : DD_N;
  const int ks = dense_ks(M, d, ffn), nst_all = ffn / 32;
  CHECK(ks >= 1 && ks <= nst_all, "M %d d %d ffn %d: %d K slices over %d stages", M, d, ffn, ks,
        nst_all);
  if (ks < 1 || ks > nst_all) return;
  const int nb_m = (M + TM - 1) / TM, nb_n = (d + TN - 1) / TN, total = nb_m * nb_n * ks;
  const int grid = 8 * ((total + 7) / 8);
  const size_t nel = (size_t)ks * M * d;
  std::vector<unsigned char> seen(total, 0), el(nel / 4, 0);
  for (int b = 0; b < grid; ++b) {
    const int tile = xcd_tile_of(b, total);
    CHECK(tile >= 0 && tile < grid, "tile id %d of grid %d", tile, grid);
    if (tile < 0 || tile >= total) continue;
    CHECK(!seen[tile], "tile %d given twice (M %d d %d)", tile, M, d);
    seen[tile] = 1;
    int mt, nt, k;
    gemm_tile(tile, nb_m, nb_n, mt, nt, k);
    CHECK(mt < nb_m && nt < nb_n && k < ks, "tile %d decodes outside the grid", tile);
    int s0, n;
    slice_stages(nst_all, k, ks, s0, n);
    CHECK(n >= 1 && s0 >= 0 && s0 + n <= nst_all, "slice %d of %d: stages [%d, %d)", k, ks, s0,
          s0 + n);
    const int m0 = mt * TM, c0 = nt * TN;
    auto store = [&](int m, int col) {
      if (m >= M || col >= d) return;                     // the kernels' own guard
      CHECK(m >= 0 && col >= 0 && col % 4 == 0 && col + 3 < d, "store at m %d col %d", m, col);
      const size_t off = ((size_t)k * M + m) * d + col;
      CHECK(off + 3 < nel, "store past the partials: M %d d %d off %zu", M, d, off);
      if (off + 3 < nel && col % 4 == 0) {
        CHECK(!el[off / 4], "element stored twice: M %d d %d k %d m %d col %d", M, d, k, m, col);
        el[off / 4] = 1;
      }
    };
    if (wide) {
      for (int wave = 0; wave < 8; ++wave)
        for (int ms = 0; ms < 2; ++ms)
          for (int i = 0; i < 16; ++i)
            for (int lane = 0; lane < 64; ++lane) {
              int m, col;
              ddq_store_pos(m0, c0, wave, ms, i, lane, m, col);
              store(m, col);
            }
    } else {
      for (int w = 0; w < 4; ++w)
        for (int e = 0; e < 32 * DD_N / 4; ++e) {
          int m, col;
          ddown_store_pos(m0, c0, w, e, m, col);
          store(m, col);
        }
    }
  }
  for (int t = 0; t < total; ++t) CHECK(seen[t], "tile %d never given (M %d d %d)", t, M, d);
  size_t missing = 0;
  for (unsigned char v : el) missing += !v;
  CHECK(missing == 0, "M %d d %d ffn %d: %zu partial elements never stored", M, d, ffn, missing);
  int prev = 0;
  for (int k = 0; k < ks; ++k) {
    int s0, n;
    slice_stages(nst_all, k, ks, s0, n);
    CHECK(s0 == prev, "slices not consecutive: M %d k %d", M, k);
    prev = s0 + n;
  }
  CHECK(prev == nst_all, "slices do not cover the ffn stages: M %d", M);
}

// Predictor stage 1 of a large call (the GEMM's ZP_M x ZP_N tiles, split over d): the grid's
// tiles are each (token tile, rank tile, K slice) once, the slices split d's 32-wide stages with
// none empty, and every (token, slice, rank column) element of the per-pass partials
// [pass][slice][32][rank] is stored exactly once, inside the passes' buffer.
static void check_zpart(int M, int d, int rank) {
  const int ks = zpart_kslices(M, d, rank), nst_all = d / 32;
  CHECK(ks >= 1 && ks <= ZPART_MAX_KS && ks <= nst_all, "M %d d %d rank %d: %d K slices", M, d,
        rank, ks);
  if (ks < 1 || ks > nst_all) return;
  const int nb_m = (M + ZP_M - 1) / ZP_M, nb_n = (rank + ZP_N - 1) / ZP_N;
  const int total = nb_m * nb_n * ks, grid = 8 * ((total + 7) / 8);
  const size_t zpart_ps = (size_t)ks * 32 * rank, passes = (M + 31) / 32;
  const size_t nel = passes * zpart_ps;
  std::vector<unsigned char> seen(total, 0), el(nel, 0);
  for (int b = 0; b < grid; ++b) {
    const int tile = xcd_tile_of(b, total);
    if (tile < 0 || tile >= total) continue;
    CHECK(!seen[tile], "tile %d given twice (M %d rank %d)", tile, M, rank);
    seen[tile] = 1;
    int mt, nt, k;
    gemm_tile(tile, nb_m, nb_n, mt, nt, k);
    int s0, n;
    slice_stages(nst_all, k, ks, s0, n);
    CHECK(n >= 1 && s0 >= 0 && s0 + n <= nst_all, "slice %d of %d: stages [%d, %d)", k, ks, s0,
          s0 + n);
    for (int wave = 0; wave < 8; ++wave)
      for (int ms = 0; ms < ZP_M / 4 / 32; ++ms)
        for (int ns = 0; ns < ZP_N / 2 / 32; ++ns)
          for (int i = 0; i < 16; ++i)
            for (int lane = 0; lane < 64; ++lane) {
              int m, c;
              zpart_store_pos(mt * ZP_M, nt * ZP_N, ZP_M, ZP_N, wave, ms, ns, i, lane, m, c);
              if (m >= M || c >= rank) continue;             // the kernel's own guard
              const size_t off = zpart_offset(m, k, c, rank, zpart_ps);
              CHECK(off < nel, "store past the partials: M %d rank %d off %zu", M, rank, off);
              if (off < nel) {
                CHECK(!el[off], "element stored twice: M %d k %d m %d c %d", M, k, m, c);
                el[off] = 1;
              }
            }
  }
  for (int t = 0; t < total; ++t) CHECK(seen[t], "tile %d never given (M %d rank %d)", t, M, rank);
  size_t missing = 0;
  for (size_t e = 0; e < nel; ++e) {
    const size_t p = e / zpart_ps, m = p * 32 + e % zpart_ps / rank % 32;
    if (m < (size_t)M) missing += !el[e];                    // rows past the last token: unused
  }
  CHECK(missing == 0, "M %d d %d rank %d: %zu partial elements never stored", M, d, rank, missing);
}

// Attention block, for H heads of width e (G key/value heads), d columns and contexts of n
// positions: the projection workgroups' rows stay inside their matrices; the score kernel's
// chunks cover [0, n) exactly, each non-empty and a whole number of steps, at most the record
// slots; the output projection's row split partitions the active heads' rows, at most
// ATTN_OUT_MAXR rows and two heads per workgroup, with every record and partial index in range.
static void check_attn(int H, int G, int e, int d, int S) {
  const int step = attn_step_positions(e);
  const size_t rec_size = (size_t)H * ATTN_MAX_CHUNKS * (e + 4);
  for (int b = 0; b < H * e / 8; ++b) {               // query workgroups: rank, channels
    const int k = b * 8 / e, c0 = b * 8 % e;
    CHECK(k < H && c0 + 8 <= e && (k * e + c0) / e == k, "q block %d", b);
  }
  for (int b = 0; b < 2 * G * e / 8; ++b) {           // key then value workgroups
    const int r = b * 8, row0 = r < G * e ? r : r - G * e;
    CHECK(row0 + 8 <= G * e && row0 / e == (row0 + 7) / e, "kv block %d", b);
  }
  for (int n = 1; n <= S; n += (n < 300 ? 1 : 97)) {
    int lc, nc;
    attn_chunk_split(H, step, n, ATTN_MAX_CHUNKS, lc, nc);
    CHECK(lc > 0 && lc % step == 0 && nc >= 1 && nc <= ATTN_MAX_CHUNKS, "H %d n %d", H, n);
    CHECK((long)(nc - 1) * lc < n && (long)nc * lc >= n, "H %d n %d lc %d nc %d", H, n, lc, nc);
    for (int k = 0; k < H; k += H - 1 > 0 ? H - 1 : 1)
      CHECK(attn_rec_offset(k, nc - 1, e, ATTN_MAX_CHUNKS) + e + 2 <= rec_size, "rec H %d", H);
  }
  for (int act = 0; act <= H; ++act) {
    const int rows = act * e;
    int prev = 0;
    for (int b = 0; b < ATTN_OUT_BLOCKS; ++b) {
      int r0, r1;
      attn_out_rows(rows, b, ATTN_OUT_BLOCKS, r0, r1);
      CHECK(r0 == prev && r1 >= r0, "rows %d b %d", rows, b);
      CHECK(r1 - r0 <= ATTN_OUT_MAXR, "rows %d b %d: %d rows", rows, b, r1 - r0);
      if (r1 > r0) {
        CHECK((r1 - 1) / e - r0 / e <= 1, "rows %d b %d spans >2 heads", rows, b);
        CHECK((size_t)b * d + (size_t)d <= (size_t)ATTN_OUT_BLOCKS * d, "part b %d", b);
        CHECK((r1 - 1) / e < act, "rows %d b %d past |A|", rows, b);
      }
      prev = r1;
    }
    CHECK(prev == rows, "rows %d not covered (%d)", rows, prev);
  }
}

int main() {
  const int ds[] = {64, 256, 512, 768, 776, 1024, 4096, 4104, 8192};
  const int ffns[] = {256, 1024, 3072, 11008, 14336, 32768};
  for (int d : ds)
    for (int ffn : ffns) {
      const int nblks[] = {gather_blocks(1), gather_blocks(2), gather_blocks(3), gather_blocks(4),
                           fused_blocks(ffn)};
      for (int nblk : nblks) check_partials(d, ffn, nblk);
    }
  check_segments();
  check_xcd_order();
  const int shapes[][4] = {{4096, 11008, 256, 64}, {4096, 14336, 512, 100},
                           {8192, 32768, 1024, 512}, {256, 1024, 32, 4096}, {512, 2048, 64, 70},
                           {1024, 4096, 64, 256}};
  for (const auto& sh : shapes) check_passes(sh[0], sh[1], sh[2], sh[3]);
  const int dshapes[][3] = {{64, 256, 1024},   {70, 264, 1056},   {129, 264, 2048},
                            {130, 512, 2048},  {256, 256, 1024},  {300, 768, 3072},
                            {385, 4096, 11008}, {512, 8192, 32768}, {1000, 1024, 4096},
                            {4096, 512, 2048}};
  for (const auto& sh : dshapes) check_dense_down(sh[0], sh[1], sh[2]);
  const int zshapes[][3] = {{128, 4096, 256}, {130, 4096, 512}, {512, 8192, 1024},
                            {300, 768, 64}, {4096, 2048, 2048}, {1000, 512, 96}};
  for (const auto& sh : zshapes) check_zpart(sh[0], sh[1], sh[2]);
  const int ashapes[][5] = {{32, 32, 128, 4096, 4096}, {32, 8, 128, 4096, 32768},
                            {12, 12, 64, 768, 2048}, {128, 8, 64, 1024, 8192},
                            {128, 1, 128, 8192, 4096}, {1, 1, 64, 64, 300},
                            {6, 3, 64, 328, 33}, {16, 1, 128, 1024, 300}};
  for (const auto& sh : ashapes) check_attn(sh[0], sh[1], sh[2], sh[3], sh[4]);
  if (failures) {
    printf("index check: %ld of %ld checks failed\n", failures, checks);
    return 1;
  }
  printf("index check: OK (%ld checks)\n", checks);
  return 0;
}
