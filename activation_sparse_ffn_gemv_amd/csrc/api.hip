// C ABI of libffn_sparse: validation, workspace layout, path choice and launch sequencing.
// Kernels live in decode.hip (batch-1 decode), batch.hip (several tokens), dense.hip (MFMA
// GEMMs), moe.hip (router) and attn.hip (attention block).  Nothing here allocates device memory or synchronises, except
// ffn_sparse_plan with calibrate = 1.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <mutex>
#include <new>
#include <vector>

#include "common.h"
#include "index.h"
#include "launch.h"

using namespace ffn;

namespace {

thread_local char g_err[512] = "";

ffn_status fail(ffn_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ffn_status fail(ffn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ffn_status hip_fail(hipError_t e, const char* what) {
  return fail(FFN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int elems_per_chunk(int dt) { return dt == FFN_F32 ? 4 : dt == FFN_F16 ? 8 : 32; }

int cpl_for(int nch) {
  static const int ok[] = {1, 2, 3, 4, 6, 8, 12, 16};
  int need = (nch + WAVE - 1) / WAVE;
  for (int c : ok)
    if (c >= need) return c;
  return -1;
}

struct Layout {
  int cpl_w, cpl_p;
  size_t off_z, off_bits, off_cnt, off_part, scratch_end, off_batch, off_dense, dense_rows, total;
};

// Dense-GEMM region (fp16 layers that may see DENSE_MIN_M tokens or more): dbits [max_batch]
// [ffn/32] | flag | H [max_batch][ffn] fp16 | partials [rows][d] fp32.
size_t dense_rows_for(const ffn_layer_desc* d) {
  size_t rows = 0;
  for (int M = DENSE_MIN_M; M <= d->max_batch; ++M)
    rows = std::max(rows, (size_t)dense_ks(M, d->d, d->ffn) * M);
  return rows;
}

// The batched kernels (MFMA) cover fp16 layers; other storage types run B > 1 token by token.
bool batched(const ffn_layer_desc* d) { return d->w_dtype == FFN_F16; }

// The dense region, from byte `base` of the workspace: per-token bitmaps [max_batch][ffn/32] |
// the path flag | H [passes * 32][ffn] fp16 (the dense GEMMs' H, and the batched kernels' H of
// a call whose passes share one launch: only one of the two runs per call) | the dense GEMMs'
// partials [rows][d] | for `passes` = ceil(max_batch / 32) passes: predictor stage-1 partials,
// z (hi, lo), union words, |U|, union ranks and the down projection's segment partials.
struct DenseRegion {
  size_t bits, flag, H, ypart, zpart, zhl, ubits, ucnt, uidx, mpart, zcat, end;
  int passes, S;
};

DenseRegion dense_region(const ffn_layer_desc* d, size_t base) {
  DenseRegion R{};
  const BatchShape s = batch_shape(d->d, d->ffn, d->rank);
  R.passes = (d->max_batch + BATCH_TILE - 1) / BATCH_TILE;
  R.S = batch_segments_mp(d->d, R.passes);
  const size_t P = (size_t)R.passes, W = (size_t)d->ffn / 32;
  size_t off = base;
  R.bits = off;   off = round_up(off + (size_t)d->max_batch * W * 4, 256);
  R.flag = off;   off = round_up(off + 4, 256);
  R.H = off;      off = round_up(off + P * BATCH_TILE * d->ffn * 2, 256);
  R.ypart = off;  off = round_up(off + dense_rows_for(d) * d->d * 4, 256);
  // (stage-1 partials of either the batched kernels or the stage-1 GEMM's K slices)
  R.zpart = off;
  off = round_up(off + P * std::max(s.zpart_bytes, (size_t)ZPART_MAX_KS * BATCH_TILE *
                                                       std::max(d->rank, 1) * 4), 256);
  R.zhl = off;    off = round_up(off + P * s.zhl_bytes, 256);
  R.ubits = off;  off = round_up(off + P * W * 4, 256);
  R.ucnt = off;   off = round_up(off + P * 4, 256);
  R.uidx = off;   off = round_up(off + P * d->ffn * 4, 256);
  R.mpart = off;  off = round_up(off + P * R.S * BATCH_TILE * d->d * 4, 256);
  R.zcat = off;   off = round_up(off + P * BATCH_TILE * std::max(d->rank, 1) * 2 * 2, 256);
  R.end = off;
  return R;
}

ffn_status check_desc(const ffn_layer_desc* d) {
  if (!d) return fail(FFN_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->d <= 0 || d->ffn <= 0 || d->rank < 0 || d->max_batch <= 0)
    return fail(FFN_ERR_INVALID_ARGUMENT, "d, ffn, max_batch must be > 0 and rank >= 0");
  if (d->act < FFN_ACT_RELU || d->act > FFN_ACT_DRELU)
    return fail(FFN_ERR_INVALID_ARGUMENT, "act %d is not an ffn_act", d->act);
  if (d->w_dtype < FFN_F32 || d->w_dtype > FFN_I4G32 || d->x_dtype < FFN_F32 ||
      d->x_dtype > FFN_F16 || d->p_dtype < FFN_F32 || d->p_dtype > FFN_F16)
    return fail(FFN_ERR_INVALID_ARGUMENT, "bad dtype (w %d, x %d, p %d)", d->w_dtype,
                d->x_dtype, d->p_dtype);
  if (!(d->threshold > 0.0f && d->threshold <= 1.0f))
    return fail(FFN_ERR_INVALID_ARGUMENT, "threshold must lie in (0, 1]");
  const int want_x = d->w_dtype == FFN_F32 ? FFN_F32 : FFN_F16;
  if (d->x_dtype != want_x)
    return fail(FFN_ERR_UNSUPPORTED, "x_dtype must be %s for this w_dtype",
                want_x == FFN_F32 ? "FFN_F32" : "FFN_F16");
  if (d->rank > 0 && d->p_dtype != d->x_dtype)
    return fail(FFN_ERR_UNSUPPORTED, "p_dtype must equal x_dtype");
  if (d->d % 8 || (d->w_dtype == FFN_I4G32 && d->d % 32))
    return fail(FFN_ERR_UNSUPPORTED, "d must be a multiple of 8 (32 for int4)");
  if (d->d > 8192) return fail(FFN_ERR_UNSUPPORTED, "d > 8192");
  if (d->ffn % 32 || d->ffn > 32768)
    return fail(FFN_ERR_UNSUPPORTED, "ffn must be a multiple of 32 and <= 32768");
  if (d->rank % 8 || (d->rank > 0 && pred_s_cpr(d->p_dtype == FFN_F16, d->rank) < 0))
    return fail(FFN_ERR_UNSUPPORTED, "rank must be a multiple of 8 and <= 2048 (fp16) / 1024 (fp32)");
  const int wk = d->w_dtype == FFN_F32 ? WK_F32 : d->w_dtype == FFN_F16 ? WK_F16 : WK_I4;
  if (gather_cpt(wk, d->d) > (wk == WK_I4 ? 1 : 2))
    return fail(FFN_ERR_UNSUPPORTED, "d > %d for this w_dtype", wk == WK_F32 ? 4096 : 8192);
  if (d->max_batch > 4096) return fail(FFN_ERR_UNSUPPORTED, "max_batch > 4096");
  return FFN_OK;
}

// Workspace of one token in flight (tokens of a batch reuse it one after another):
// z [rank] f32 | bitmap [ffn/32] u32 | |A| i32 | partials [gather workgroups][d] f32
Layout layout_for(const ffn_layer_desc* d) {
  Layout L{};
  L.cpl_w = cpl_for(d->d / elems_per_chunk(d->w_dtype));
  L.cpl_p = d->rank > 0 ? cpl_for(d->d / elems_per_chunk(d->p_dtype)) : 1;
  size_t off = 0;
  L.off_z = off;      off = round_up(off + (size_t)std::max(d->rank, 1) * 4, 256);
  L.off_bits = off;   off = round_up(off + (size_t)d->ffn / 32 * 4, 256);
  L.off_cnt = off;    off = round_up(off + 4, 256);
  L.off_part = off;
  off = round_up(off + (size_t)std::max(gather_blocks(), fused_blocks(d->ffn)) *
                           reduce_tiles(d->d) * 16 * 4, 256);
  L.scratch_end = off;              // end of one token's decode scratch
  L.off_batch = 0;
  if (batched(d)) {
    // batched region: zpart | zhl | bits | ubits | ucnt | uidx | H | ypart
    const BatchShape s = batch_shape(d->d, d->ffn, d->rank);
    L.off_batch = off;
    off = round_up(off + s.zpart_bytes, 256);
    off = round_up(off + s.zhl_bytes, 256);
    off = round_up(off + s.bits_bytes, 256);
    off = round_up(off + s.ubits_bytes, 256);
    off = round_up(off + 4, 256);
    off = round_up(off + s.uidx_bytes, 256);
    off = round_up(off + s.H_bytes, 256);
    off = round_up(off + s.ypart_bytes, 256);
  }
  L.off_dense = 0;
  L.dense_rows = 0;
  if (batched(d) && d->max_batch >= DENSE_MIN_M) {
    L.off_dense = off;
    L.dense_rows = dense_rows_for(d);
    off = dense_region(d, off).end;
  }
  L.total = off;
  return L;
}

struct DenseBufs {
  uint32_t* bits;
  int* flag;
  _Float16* H;
  float* ypart;
  // the batched kernels' buffers for all passes of one call (grid.z = pass)
  float* zpart;
  _Float16* zhl;
  uint32_t* ubits;
  int* ucnt;
  int* uidx;
  float* mpart;
  _Float16* zcat;
  int passes, S;
};

DenseBufs dense_bufs(char* ws, const ffn_plan* p) {
  const DenseRegion R = dense_region(&p->desc, p->off_dense);
  DenseBufs b{};
  b.bits = reinterpret_cast<uint32_t*>(ws + R.bits);
  b.flag = reinterpret_cast<int*>(ws + R.flag);
  b.H = reinterpret_cast<_Float16*>(ws + R.H);
  b.ypart = reinterpret_cast<float*>(ws + R.ypart);
  b.zpart = reinterpret_cast<float*>(ws + R.zpart);
  b.zhl = reinterpret_cast<_Float16*>(ws + R.zhl);
  b.ubits = reinterpret_cast<uint32_t*>(ws + R.ubits);
  b.ucnt = reinterpret_cast<int*>(ws + R.ucnt);
  b.uidx = reinterpret_cast<int*>(ws + R.uidx);
  b.mpart = reinterpret_cast<float*>(ws + R.mpart);
  b.zcat = reinterpret_cast<_Float16*>(ws + R.zcat);
  b.passes = R.passes;
  b.S = R.S;
  return b;
}

DenseArgs dense_args(const ffn_plan* p, const DenseBufs& db, const void* x, int M, float* y) {
  const ffn_layer_desc& D = p->desc;
  DenseArgs a{};
  a.x = x;
  a.w_up = p->w.w_up;
  a.w_gate = p->w.w_gate;
  a.w_dn = p->w.w_down_t;
  a.b_up = p->w.b_up;
  a.b_gate = p->w.b_gate;
  a.b_down = p->w.b_down;
  a.H = db.H;
  a.ypart = db.ypart;
  a.y = y;
  a.M = M;
  a.d = D.d;
  a.ffn = D.ffn;
  a.act = D.act;
  a.has_gate = D.act != FFN_ACT_RELU;
  a.ks = dense_ks(M, D.d, D.ffn);
  return a;
}

// The batched region's buffers, in the order layout_for reserves them.
BatchArgs batch_bufs(char* ws, const ffn_plan* p) {
  const ffn_layer_desc& D = p->desc;
  const BatchShape s = batch_shape(D.d, D.ffn, D.rank);
  BatchArgs a{};
  size_t off = p->off_batch;
  a.zpart = reinterpret_cast<float*>(ws + off);        off = round_up(off + s.zpart_bytes, 256);
  a.zhl = reinterpret_cast<_Float16*>(ws + off);       off = round_up(off + s.zhl_bytes, 256);
  a.bits = reinterpret_cast<uint32_t*>(ws + off);      off = round_up(off + s.bits_bytes, 256);
  a.ubits = reinterpret_cast<uint32_t*>(ws + off);     off = round_up(off + s.ubits_bytes, 256);
  a.ucnt = reinterpret_cast<int*>(ws + off);           off = round_up(off + 4, 256);
  a.uidx = reinterpret_cast<int*>(ws + off);           off = round_up(off + s.uidx_bytes, 256);
  a.H = reinterpret_cast<_Float16*>(ws + off);         off = round_up(off + s.H_bytes, 256);
  a.ypart = reinterpret_cast<float*>(ws + off);
  a.ks = s.ks;
  a.spw = s.spw;
  a.S = s.S;
  a.p1 = p->w.p1;
  a.p2 = p->w.p2;
  a.c1 = p->w.c1;
  a.c2 = p->w.c2;
  a.w_up = p->w.w_up;
  a.w_gate = p->w.w_gate;
  a.w_dn = p->w.w_down_t;
  a.b_up = p->w.b_up;
  a.b_gate = p->w.b_gate;
  a.b_down = p->w.b_down;
  a.head_words = p->head_words;
  a.d = D.d;
  a.ffn = D.ffn;
  a.r = D.rank;
  a.act = D.act;
  a.has_gate = D.act != FFN_ACT_RELU;
  a.thr = p->thr;
  return a;
}


// Workspace of a mixture: one decode scratch (z, bitmap, |A|, partials: the front of an
// expert's layout) per expert slot, then the per-slot expert records [max_batch][top_k].
struct MoeLayout {
  size_t slot_stride, off_slots, off_zall, total;
};

// slots' decode scratch | slot records [max_batch][top_k] | stage-1 results [max_batch][E][rank]
MoeLayout moe_layout(const ffn_plan* e0, int n_experts, int top_k) {
  MoeLayout L{};
  const ffn_layer_desc& D = e0->desc;
  L.slot_stride = round_up(layout_for(&D).scratch_end, 256);
  L.off_slots = L.slot_stride * top_k;
  L.off_zall = round_up(L.off_slots + (size_t)D.max_batch * top_k * sizeof(ExpertW), 256);
  L.total = round_up(L.off_zall + (size_t)D.max_batch * n_experts * D.rank * 4, 256);
  return L;
}

}  // namespace

ffn_status calibrate_crossover(ffn_plan* p, hipStream_t st);

struct ffn_moe {
  int n_experts, top_k;
  const void* router;
  const ffn_plan* e0;             // shapes and threshold (every expert shares them)
  char* ws;
  MoeLayout L;
  ExpertTable tab;                // every expert's weight pointers, passed to the router
};

namespace {

// Scratch of the token in flight inside a workspace laid out by layout_for.
struct TokenBufs {
  float* z;
  uint32_t* bits;
  int* cnt;
  float* part;
};

TokenBufs token_bufs(char* ws, const ffn_plan* p) {
  return TokenBufs{reinterpret_cast<float*>(ws + p->off_z),
                   reinterpret_cast<uint32_t*>(ws + p->off_bits),
                   reinterpret_cast<int*>(ws + p->off_cnt),
                   reinterpret_cast<float*>(ws + p->off_part)};
}

// The neuron-cache region: c_up | c_gate | c_dn [cap][d] fp16 | slot_of [ffn] | neuron_of [cap] |
// last_use [cap] | stamp | rank_nid, rank_src, rank_vic [ffn] | stats [4].
size_t cache_region_bytes(const ffn_layer_desc& D, int cap) {
  const size_t rows = round_up((size_t)cap * D.d * 2, 256);
  return 3 * rows + round_up((size_t)D.ffn * 4, 256) + 2 * round_up((size_t)cap * 4, 256) + 256 +
         3 * round_up((size_t)D.ffn * 4, 256) + 256;
}

struct CacheBufs {
  char* c_up;
  char* c_gate;
  char* c_dn;
  CacheArgs a;
};

CacheBufs cache_bufs(const ffn_plan* p) {
  const ffn_layer_desc& D = p->desc;
  const int cap = p->cache_cap;
  const size_t rows = round_up((size_t)cap * D.d * 2, 256);
  char* b = p->ws + p->off_cache;
  CacheBufs c{};
  c.c_up = b;
  c.c_gate = b + rows;
  c.c_dn = b + 2 * rows;
  size_t off = 3 * rows;
  c.a.ffn = D.ffn;
  c.a.cap = cap;
  c.a.slot_of = reinterpret_cast<int*>(b + off);         off += round_up((size_t)D.ffn * 4, 256);
  c.a.neuron_of = reinterpret_cast<int*>(b + off);       off += round_up((size_t)cap * 4, 256);
  c.a.last_use = reinterpret_cast<uint32_t*>(b + off);   off += round_up((size_t)cap * 4, 256);
  c.a.stamp = reinterpret_cast<uint32_t*>(b + off);      off += 256;
  c.a.rank_nid = reinterpret_cast<int*>(b + off);        off += round_up((size_t)D.ffn * 4, 256);
  c.a.rank_src = reinterpret_cast<int*>(b + off);        off += round_up((size_t)D.ffn * 4, 256);
  c.a.rank_vic = reinterpret_cast<int*>(b + off);        off += round_up((size_t)D.ffn * 4, 256);
  c.a.stats = reinterpret_cast<int*>(b + off);
  return c;
}

// The launches of one token: active set (predictor or caller mask) -> balanced gather -> reduce.
// slot != nullptr: the experts are chosen on the device; the kernels take their weights from
// the nslot consecutive slot records (p then only supplies shapes and the threshold) and run
// the slots side by side, slot k's scratch at slot_stride bytes past slot k-1's; the reduce
// writes the routing-weighted sum of the slots.
ffn_status enqueue_token(const ffn_plan* p, const TokenBufs& wb, const void* xb,
                         const uint8_t* maskb, float* yb, int* idxb, int* cntb, float* scoresb,
                         const ExpertW* slot, int nslot, size_t slot_stride, hipStream_t st,
                         bool all_neurons = false, const float* zall = nullptr) {
  const ffn_layer_desc& D = p->desc;
  const int wk = D.w_dtype == FFN_F32 ? WK_F32 : D.w_dtype == FFN_F16 ? WK_F16 : WK_I4;
  const int es = (int)(slot_stride / 4);      // the same stride in 4-byte elements
  hipError_t e;
  const bool fused = !maskb && !all_neurons && !slot && p->decode_variant == 1 &&
                     fused_supported(wk, D.d) && p->cache_cap == 0;
  if (maskb || all_neurons) {
    e = launch_mask_bits(maskb, wb.bits, D.ffn / 32, st);
    if (e != hipSuccess) return hip_fail(e, "mask launch");
  } else {
    if (!zall) {                                 // (a mixture ran stage 1 with its router)
      e = launch_pred_z(D.p_dtype == FFN_F16, p->cpl_p, p->w.p1, p->w.c1, xb, wb.z, D.d, D.rank,
                        slot, nslot, es, st, p->ev[FFN_STAGE_PRED_Z][0],
                        p->ev[FFN_STAGE_PRED_Z][1]);
      if (e != hipSuccess) return hip_fail(e, "predictor stage 1 launch");
    }
    PredArgs pa{};
    pa.p2 = p->w.p2;
    pa.c2 = p->w.c2;
    pa.z = wb.z;
    pa.scores = scoresb;
    pa.bitmap = wb.bits;
    pa.ffn = D.ffn;
    pa.rank = D.rank;
    pa.thr = p->thr;
    pa.slot = slot;
    pa.nslot = nslot;
    pa.zstride = es;
    pa.bstride = es;
    pa.head_words = slot ? 0 : p->head_words;
    pa.zall = zall;
    if (!fused) {
      e = launch_pred_s(D.p_dtype == FFN_F16, pa, st, p->ev[FFN_STAGE_PRED_S][0],
                        p->ev[FFN_STAGE_PRED_S][1]);
      if (e != hipSuccess) return hip_fail(e, "predictor stage 2 launch");
    } else {
      FusedArgs fa{};
      fa.pa = pa;
      fa.ga.w_up = p->w.w_up;
      fa.ga.w_gate = p->w.w_gate;
      fa.ga.w_dn = p->w.w_down_t;
      fa.ga.b_up = p->w.b_up;
      fa.ga.b_gate = p->w.b_gate;
      fa.ga.x = xb;
      fa.ga.part = wb.part;
      fa.ga.d = D.d;
      fa.ga.ffn = D.ffn;
      fa.ga.act = D.act;
      fa.ga.has_gate = D.act != FFN_ACT_RELU;
      e = launch_fused(wk, fa, st, p->ev[FFN_STAGE_GATHER][0], p->ev[FFN_STAGE_GATHER][1]);
      if (e != hipSuccess) return hip_fail(e, "fused predictor + gather launch");
    }
  }
  GatherArgs ga{};
  ga.w_up = p->w.w_up;
  ga.w_gate = p->w.w_gate;
  ga.w_dn = p->w.w_down_t;
  ga.s_up = p->w.s_up;
  ga.s_gate = p->w.s_gate;
  ga.s_dn = p->w.s_down_t;
  ga.b_up = p->w.b_up;
  ga.b_gate = p->w.b_gate;
  ga.x = xb;
  ga.bitmap = wb.bits;
  ga.part = wb.part;
  ga.cnt = wb.cnt;
  ga.d = D.d;
  ga.ffn = D.ffn;
  ga.act = D.act;
  ga.has_gate = D.act != FFN_ACT_RELU;
  ga.slot = slot;
  ga.nslot = nslot;
  ga.bstride = es;
  ga.cstride = es;
  ga.pstride = (size_t)es;
  if (p->cache_cap > 0 && !slot) {
    // host-resident rows: the cache plan ranks the set and picks each row's source, then the
    // gather reads hits from the cache and misses from host memory (admitting them)
    CacheBufs cb = cache_bufs(p);
    cb.a.bitmap = wb.bits;
    cb.a.cnt = wb.cnt;
    if ((e = launch_cache_plan(cb.a, st)) != hipSuccess) return hip_fail(e, "cache plan launch");
    ga.rank_nid = cb.a.rank_nid;
    ga.rank_src = cb.a.rank_src;
    ga.rank_vic = cb.a.rank_vic;
    ga.c_up = cb.c_up;
    ga.c_gate = cb.c_gate;
    ga.c_dn = cb.c_dn;
    e = launch_gather_cached(ga, st, p->ev[FFN_STAGE_GATHER][0], p->ev[FFN_STAGE_GATHER][1]);
    if (e != hipSuccess) return hip_fail(e, "cached gather launch");
  } else if (!fused) {
    e = launch_gather(wk, ga, st, p->ev[FFN_STAGE_GATHER][0], p->ev[FFN_STAGE_GATHER][1]);
    if (e != hipSuccess) return hip_fail(e, "gather launch");
  }
  ReduceArgs ra{};
  ra.part = wb.part;
  ra.cnt = wb.cnt;
  ra.bitmap = wb.bits;
  ra.b_down = p->w.b_down;
  ra.y = yb;
  ra.idx_out = idxb;
  ra.cnt_out = cntb;
  ra.d = D.d;
  ra.ffn = D.ffn;
  ra.n_part = fused ? fused_blocks(D.ffn) : gather_blocks(slot ? nslot : 1);
  ra.fused = fused;
  ra.slot = slot;
  ra.nslot = nslot;
  ra.cstride = es;
  ra.pstride = (size_t)es;
  e = launch_reduce(ra, st, p->ev[FFN_STAGE_REDUCE][0], p->ev[FFN_STAGE_REDUCE][1]);
  if (e != hipSuccess) return hip_fail(e, "reduce launch");
  return FFN_OK;
}

// Measured crossover (ffn_sparse_plan with calibrate = 1).  For each batch bucket B = 2, 4, 8,
// ... up to max_batch, the plan's own kernels are timed on its own weights: the dense path
// (every neuron's rows) and the sparse path over caller sets in which every token has the same
// random set of density rho, for rho on a grid.  The crossover is the density at which the
// sparse time reaches the dense time (linear between grid points; 1 when the sparse path is
// never slower).  Synchronous; the scratch buffers are allocated and freed here.
ffn_status time_call(hipStream_t st, hipEvent_t e0, hipEvent_t e1, float* ms,
                     const std::function<ffn_status()>& f) {
  float best = 1e30f;
  for (int rep = 0; rep < 4; ++rep) {
    hipError_t e = hipEventRecord(e0, st);
    if (e != hipSuccess) return hip_fail(e, "calibration event");
    ffn_status s = f();
    if (s != FFN_OK) return s;
    if ((e = hipEventRecord(e1, st)) != hipSuccess || (e = hipEventSynchronize(e1)) != hipSuccess)
      return hip_fail(e, "calibration event");
    float t = 0.0f;
    if ((e = hipEventElapsedTime(&t, e0, e1)) != hipSuccess) return hip_fail(e, "calibration");
    if (rep > 0) best = std::min(best, t);        // the first call warms up
  }
  *ms = best;
  return FFN_OK;
}

}  // namespace

ffn_status calibrate_crossover(ffn_plan* p, hipStream_t st) {
  const ffn_layer_desc& D = p->desc;
  const int Bmax = D.max_batch;
  void *x = nullptr, *y = nullptr, *mask = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  ffn_status res = FFN_OK;
  std::vector<unsigned char> hm((size_t)Bmax * D.ffn);
  static const float grid[] = {0.0625f, 0.125f, 0.25f, 0.5f, 0.75f, 1.0f};
  constexpr int NG = sizeof(grid) / sizeof(grid[0]);
  hipError_t e;
  if ((e = hipMalloc(&x, (size_t)Bmax * D.d * 2)) != hipSuccess ||
      (e = hipMalloc(&y, (size_t)Bmax * D.d * 4)) != hipSuccess ||
      (e = hipMalloc(&mask, hm.size())) != hipSuccess ||
      (e = hipMemsetAsync(x, 0, (size_t)Bmax * D.d * 2, st)) != hipSuccess ||
      (e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess) {
    res = hip_fail(e, "calibration setup");
  }
  for (int k = 1; res == FFN_OK && k < 13 && (1 << k) <= Bmax; ++k) {
    const int B = 1 << k;
    float t_dense = 0.0f, t_sp[NG];
    res = time_call(st, e0, e1, &t_dense, [&] {
      return ffn_dense_forward(p, x, B, static_cast<float*>(y), nullptr, st);
    });
    for (int gi = 0; res == FFN_OK && gi < NG; ++gi) {
      // the same random set for every token: union density = grid[gi]
      uint64_t h = 0x9e3779b97f4a7c15ull * (gi + 1);
      for (int i = 0; i < D.ffn; ++i) {
        h ^= h >> 33;
        h *= 0xff51afd7ed558ccdull;
        h ^= h >> 29;
        hm[i] = (double)(h >> 11) * (1.0 / 9007199254740992.0) < grid[gi] ? 1 : 0;
      }
      for (int b = 1; b < B; ++b) memcpy(&hm[(size_t)b * D.ffn], &hm[0], D.ffn);
      if ((e = hipMemcpy(mask, hm.data(), (size_t)B * D.ffn, hipMemcpyHostToDevice)) !=
          hipSuccess) {
        res = hip_fail(e, "calibration mask upload");
        break;
      }
      res = time_call(st, e0, e1, &t_sp[gi], [&] {
        return ffn_sparse_forward(p, x, B, static_cast<float*>(y),
                                  static_cast<const uint8_t*>(mask), nullptr, nullptr, nullptr,
                                  FFN_PATH_SPARSE, st);
      });
    }
    if (res != FFN_OK) break;
    float rho = 1.0f;
    for (int gi = 0; gi < NG; ++gi) {
      if (t_sp[gi] >= t_dense) {
        if (gi == 0) {
          rho = 0.0f;
        } else {
          const float f = (t_dense - t_sp[gi - 1]) / std::max(t_sp[gi] - t_sp[gi - 1], 1e-6f);
          rho = grid[gi - 1] + f * (grid[gi] - grid[gi - 1]);
        }
        break;
      }
    }
    p->crossover_density[k] = rho;
    // buckets above the largest measured batch inherit its value
    for (int kk = k + 1; kk < 13; ++kk) p->crossover_density[kk] = rho;
  }
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  if (x) hipFree(x);
  if (y) hipFree(y);
  if (mask) hipFree(mask);
  return res;
}

namespace {

ffn_status check_weights(const ffn_layer_desc* desc, const ffn_layer_weights* w);
void init_plan(ffn_plan* p, const ffn_layer_desc* desc, const ffn_layer_weights* w,
               void* workspace, size_t workspace_bytes);

// Scratch of the plan-less entry point (ffn_sparse_forward_static): one token's decode scratch
// (z, bitmap, |A|, the gather's partial sums of y) in a file-scope device array instead of a
// caller workspace.  Every GPU the library runs on holds its own copy until the process ends;
// its device address is looked up once per device (host code never uses the array's name as an
// address) and kept here.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)(4u << 20) + (64u << 10);
__device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];
constexpr int STATIC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[STATIC_MAX_DEVICES];

ffn_status scratch_of_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= STATIC_MAX_DEVICES)
    return fail(FFN_ERR_UNSUPPORTED, "device %d: the static scratch covers devices 0..%d", dev,
                STATIC_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return FFN_OK;
}

}  // namespace

extern "C" {

const char* ffn_last_error(void) { return g_err; }

const char* ffn_status_string(ffn_status s) {
  // A C caller may pass any int; reading a value outside the enumerators through the enum type
  // is undefined in C++, so the value is taken from the argument's bytes.
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case FFN_OK: return "FFN_OK";
    case FFN_ERR_INVALID_ARGUMENT: return "FFN_ERR_INVALID_ARGUMENT";
    case FFN_ERR_UNSUPPORTED: return "FFN_ERR_UNSUPPORTED";
    case FFN_ERR_WORKSPACE_TOO_SMALL: return "FFN_ERR_WORKSPACE_TOO_SMALL";
    case FFN_ERR_HIP: return "FFN_ERR_HIP";
    case FFN_ERR_INTERNAL: return "FFN_ERR_INTERNAL";
  }
  return "FFN_STATUS_UNKNOWN";
}

ffn_status ffn_workspace_size(const ffn_layer_desc* desc, size_t* bytes) {
  ffn_status st = check_desc(desc);
  if (st != FFN_OK) return st;
  if (!bytes) return fail(FFN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Layout L = layout_for(desc);
  if (L.cpl_w < 0 || L.cpl_p < 0) return fail(FFN_ERR_UNSUPPORTED, "d too large");
  *bytes = L.total;
  g_err[0] = 0;
  return FFN_OK;
}

ffn_status ffn_sparse_plan(const ffn_layer_desc* desc, const ffn_layer_weights* w,
                           void* workspace, size_t workspace_bytes, void* stream,
                           int32_t calibrate, ffn_plan** out) {
  ffn_status st = check_desc(desc);
  if (st != FFN_OK) return st;
  if (!w || !out) return fail(FFN_ERR_INVALID_ARGUMENT, "weights / out is NULL");
  *out = nullptr;
  if ((st = check_weights(desc, w)) != FFN_OK) return st;
  if (!aligned16(workspace)) return fail(FFN_ERR_INVALID_ARGUMENT, "pointer not 16-byte aligned");
  size_t need = 0;
  if ((st = ffn_workspace_size(desc, &need)) != FFN_OK) return st;
  if (!workspace) return fail(FFN_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(FFN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);

  ffn_plan* p = new (std::nothrow) ffn_plan();
  if (!p) return fail(FFN_ERR_INTERNAL, "out of host memory");
  init_plan(p, desc, w, workspace, workspace_bytes);
  if (calibrate && batched(desc) && desc->max_batch >= 2) {
    st = calibrate_crossover(p, static_cast<hipStream_t>(stream));
    if (st != FFN_OK) {
      delete p;
      return st;
    }
  }
  *out = p;
  g_err[0] = 0;
  return FFN_OK;
}

}  // extern "C"

namespace {

// Every weight pointer the descriptor needs is present and every pointer 16-byte aligned.
ffn_status check_weights(const ffn_layer_desc* desc, const ffn_layer_weights* w) {
  const bool i4 = desc->w_dtype == FFN_I4G32;
  const bool gate = desc->act != FFN_ACT_RELU;
  if (!w->w_up || !w->w_down_t || (gate && !w->w_gate))
    return fail(FFN_ERR_INVALID_ARGUMENT, "w_up, w_down_t (and w_gate unless ReLU) required");
  if (i4 && (!w->s_up || !w->s_down_t || (gate && !w->s_gate)))
    return fail(FFN_ERR_INVALID_ARGUMENT, "int4 weights need their fp16 scales");
  if (desc->rank > 0 && (!w->p1 || !w->p2))
    return fail(FFN_ERR_INVALID_ARGUMENT, "rank > 0 needs p1 and p2");
  const void* ptrs[] = {w->w_up, gate ? w->w_gate : nullptr, w->w_down_t,
                        i4 ? w->s_up : nullptr, (i4 && gate) ? w->s_gate : nullptr,
                        i4 ? w->s_down_t : nullptr, w->b_up, gate ? w->b_gate : nullptr,
                        w->b_down, w->p1, w->p2, w->c1, w->c2};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(FFN_ERR_INVALID_ARGUMENT, "pointer not 16-byte aligned");
  return FFN_OK;
}

// A plan's fields for a checked descriptor and weights over `workspace` (no allocation).
void init_plan(ffn_plan* p, const ffn_layer_desc* desc, const ffn_layer_weights* w,
               void* workspace, size_t workspace_bytes) {
  const bool gate = desc->act != FFN_ACT_RELU;
  p->desc = *desc;
  p->w = *w;
  if (!gate) { p->w.w_gate = nullptr; p->w.s_gate = nullptr; p->w.b_gate = nullptr; }
  p->ws = static_cast<char*>(workspace);
  p->ws_bytes = workspace_bytes;
  Layout L = layout_for(desc);
  p->cpl_w = L.cpl_w;
  p->cpl_p = L.cpl_p;
  p->off_z = L.off_z;
  p->off_bits = L.off_bits;
  p->off_cnt = L.off_cnt;
  p->off_part = L.off_part;
  p->off_batch = L.off_batch;
  p->off_dense = L.off_dense;
  p->dense_ypart_rows = L.dense_rows;
  const double tau = desc->threshold;
  p->thr = tau >= 1.0 ? INFINITY : (float)log(tau / (1.0 - tau));
  // built-in table, by row bytes: below DENSE_MIN_M tokens a pass reads the union of its
  // tokens' rows once, never more than every row (crossover 1); from DENSE_MIN_M tokens on the
  // sparse passes (BATCH_TILE tokens each) read the union ceil(B / BATCH_TILE) times against the
  // dense GEMMs' one read of every row, so dense wins above a union density of
  // 1 / ceil(B / BATCH_TILE) (B = the bucket's smallest batch)
  for (int k = 0; k < 13; ++k) {
    const int B = 1 << k;
    p->crossover_density[k] =
        B < DENSE_MIN_M ? 1.0f : 1.0f / (float)((B + BATCH_TILE - 1) / BATCH_TILE);
  }
  p->dense_min_batch = 2;
  p->decode_variant = 0;
  p->head_words = 0;
  p->cache_cap = 0;
  p->off_cache = 0;
}

}  // namespace

extern "C" {

ffn_status ffn_offload_workspace_size(const ffn_layer_desc* desc, int32_t capacity,
                                      size_t* bytes) {
  if (!desc || !bytes) return fail(FFN_ERR_INVALID_ARGUMENT, "desc / bytes is NULL");
  ffn_layer_desc d1 = *desc;
  d1.max_batch = 1;
  size_t main_bytes = 0;
  ffn_status st = ffn_workspace_size(&d1, &main_bytes);
  if (st != FFN_OK) return st;
  if (desc->w_dtype != FFN_F16 || desc->x_dtype != FFN_F16 || desc->rank == 0)
    return fail(FFN_ERR_UNSUPPORTED, "the neuron cache holds fp16 rows of a layer with a predictor");
  if (capacity < 32 || capacity > CACHE_MAX_SLOTS || capacity % 32 || capacity > desc->ffn)
    return fail(FFN_ERR_INVALID_ARGUMENT, "capacity %d: a multiple of 32 in [32, min(ffn, %d)]",
                capacity, CACHE_MAX_SLOTS);
  *bytes = round_up(main_bytes, 256) + cache_region_bytes(d1, capacity);
  g_err[0] = 0;
  return FFN_OK;
}

// A host pointer the kernels may read: pinned (hipHostMalloc) host memory, mapped for the GPU.
static const void* mapped_host(const void* h) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, h) != hipSuccess) {
    (void)hipGetLastError();                      // unregistered memory: clear the error
    return nullptr;
  }
  if (at.type != hipMemoryTypeHost) return nullptr;
  return at.devicePointer ? at.devicePointer : h;
}

ffn_status ffn_offload_plan(const ffn_layer_desc* desc, const ffn_layer_weights* w,
                            int32_t capacity, int32_t n_pinned, void* workspace,
                            size_t workspace_bytes, void* stream, ffn_plan** out) {
  if (!desc || !w || !out) return fail(FFN_ERR_INVALID_ARGUMENT, "desc / weights / out is NULL");
  *out = nullptr;
  size_t need = 0;
  ffn_status st = ffn_offload_workspace_size(desc, capacity, &need);
  if (st != FFN_OK) return st;
  if (n_pinned < 0 || n_pinned > capacity)
    return fail(FFN_ERR_INVALID_ARGUMENT, "n_pinned %d not in [0, capacity]", n_pinned);
  if (!workspace) return fail(FFN_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(FFN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  const bool gate = desc->act != FFN_ACT_RELU;
  if (!w->w_up || !w->w_down_t || (gate && !w->w_gate))
    return fail(FFN_ERR_INVALID_ARGUMENT, "w_up, w_down_t (and w_gate unless ReLU) required");
  ffn_layer_weights wd = *w;
  wd.w_up = mapped_host(w->w_up);
  wd.w_gate = gate ? mapped_host(w->w_gate) : nullptr;
  wd.w_down_t = mapped_host(w->w_down_t);
  if (!wd.w_up || !wd.w_down_t || (gate && !wd.w_gate))
    return fail(FFN_ERR_INVALID_ARGUMENT, "w_up / w_gate / w_down_t must be pinned host memory "
                "(hipHostMalloc) for a neuron-cache plan");
  ffn_layer_desc d1 = *desc;
  d1.max_batch = 1;
  ffn_plan* p = nullptr;
  if ((st = ffn_sparse_plan(&d1, &wd, workspace, workspace_bytes, stream, 0, &p)) != FFN_OK)
    return st;
  size_t main_bytes = 0;
  ffn_workspace_size(&d1, &main_bytes);
  p->cache_cap = capacity;
  p->off_cache = round_up(main_bytes, 256);
  // tables, and the pinned head's rows copied into slots [0, n_pinned)
  hipStream_t s = static_cast<hipStream_t>(stream);
  CacheBufs cb = cache_bufs(p);
  hipError_t e = launch_cache_init(cb.a, n_pinned, s);
  const size_t hb = (size_t)n_pinned * d1.d * 2;
  if (e == hipSuccess && hb) e = hipMemcpyAsync(cb.c_up, wd.w_up, hb, hipMemcpyDefault, s);
  if (e == hipSuccess && hb && gate) e = hipMemcpyAsync(cb.c_gate, wd.w_gate, hb, hipMemcpyDefault, s);
  if (e == hipSuccess && hb) e = hipMemcpyAsync(cb.c_dn, wd.w_down_t, hb, hipMemcpyDefault, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "neuron cache initialisation");
  }
  *out = p;
  g_err[0] = 0;
  return FFN_OK;
}

ffn_status ffn_offload_tables(const ffn_plan* p, const int32_t** slot_of,
                              const int32_t** neuron_of, const uint32_t** last_use,
                              const int32_t** stats) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (p->cache_cap == 0) return fail(FFN_ERR_INVALID_ARGUMENT, "not a neuron-cache plan");
  const CacheBufs cb = cache_bufs(p);
  if (slot_of) *slot_of = cb.a.slot_of;
  if (neuron_of) *neuron_of = cb.a.neuron_of;
  if (last_use) *last_use = cb.a.last_use;
  if (stats) *stats = cb.a.stats;
  return FFN_OK;
}

}  // extern "C"

namespace {

// fp16 call with a dense region and B >= DENSE_MIN_M: every token's set goes to the region's
// bitmaps first (predictor or caller masks, 32 tokens per pass), then the rows run as dense
// GEMMs (DENSE), as sparse passes (SPARSE), or as whichever the device picks from the union
// density of the whole call (AUTO: both are enqueued, each gated on the device flag).
// Calls of at least this many tokens run predictor stage 2 as one GEMM (launch_dense_scores)
// instead of the batched kernels' per-pass products.
constexpr int SCORE_GEMM_MIN = 128;

ffn_status run_large(ffn_plan* p, const void* x, int32_t B, float* y, const uint8_t* mask,
                     int32_t* idx, int32_t* cnt, float* scores, int32_t path, hipStream_t st,
                     bool dense_only) {
  const ffn_layer_desc& D = p->desc;
  const int W = D.ffn / 32;
  const DenseBufs db = dense_bufs(p->ws, p);
  const bool sets = !dense_only || mask;         // dense FFN without a mask needs no sets
  hipError_t e;
  // every pass of BATCH_TILE tokens in one launch per kernel (grid.z = pass), each pass with its
  // own buffers in the dense region
  const int P = (B + BATCH_TILE - 1) / BATCH_TILE;
  const BatchShape bs = batch_shape(D.d, D.ffn, D.rank);
  BatchArgs a = batch_bufs(p->ws, p);            // shapes, weights, threshold
  a.Btot = B;
  a.B = std::min(BATCH_TILE, B);
  a.x = x;
  a.mask = mask;
  a.bits = db.bits;
  a.scores = scores;
  a.y = y;
  a.idx_out = idx;
  a.cnt_out = cnt;
  a.zpart = db.zpart;
  a.zhl = db.zhl;
  a.ubits = db.ubits;
  a.ucnt = db.ucnt;
  a.uidx = db.uidx;
  a.H = db.H;
  a.ypart = db.mpart;
  a.S = db.S;
  a.zpart_ps = bs.zpart_bytes / 4;
  a.zhl_ps = bs.zhl_bytes / 2;
  a.ubits_ps = (size_t)W;
  a.uidx_ps = (size_t)D.ffn;
  a.ypart_ps = (size_t)db.S * BATCH_TILE * D.d;
  if (sets && !mask && B >= SCORE_GEMM_MIN && D.rank % 32 == 0) {
    // many tokens: predictor stage 2 as one GEMM on the matrix cores (z as [B][2 rank], hi then
    // lo, against P2 twice), its epilogue writing the bitmap and union words
    a.zcat = db.zcat;
    if (D.d % 32 == 0) {
      // stage 1 as a GEMM too, split over d; the batched path's fixed-order sum adds the slices
      DenseArgs za{};
      za.x = x;
      za.w_up = p->w.p1;
      za.M = B;
      za.d = D.d;
      za.ffn = D.rank;
      za.kslices = zpart_kslices(B, D.d, D.rank);
      za.zpart_out = db.zpart;
      za.zpart_ps = (size_t)za.kslices * BATCH_TILE * D.rank;
      a.ks = za.kslices;
      a.zpart_ps = za.zpart_ps;
      if ((e = launch_dense_zpart(za, st)) != hipSuccess ||
          (e = launch_batch_zsum(a, st, P)) != hipSuccess)
        return hip_fail(e, "stage-1 launch");
    } else if ((e = launch_batch_stage1(a, st, P)) != hipSuccess) {
      return hip_fail(e, "stage-1 launch");
    }
    DenseArgs sa{};
    sa.x = db.zcat;
    sa.w_up = p->w.p2;
    sa.M = B;
    sa.d = 2 * D.rank;
    sa.ffn = D.ffn;
    sa.c2 = p->w.c2;
    sa.thr = p->thr;
    sa.bits_out = db.bits;
    sa.ubits_out = db.ubits;
    sa.scores = scores;
    sa.head_words = p->head_words;
    sa.b_rowb = (size_t)D.rank * 2;
    sa.bwrap = D.rank / 32;
    if ((e = launch_dense_scores(sa, st)) != hipSuccess) return hip_fail(e, "score launch");
  } else if (sets && (e = launch_batch_sets(a, mask == nullptr, st, P)) != hipSuccess) {
    return hip_fail(e, "active-set launch");
  }
  const int* flag = nullptr;
  if (path == FFN_PATH_AUTO) {
    float rho = 1.0f;
    ffn_plan_crossover(p, B, &rho);
    const int dense_above = rho >= 1.0f ? D.ffn : (int)(rho * D.ffn);
    if ((e = launch_dense_choice(db.ubits, P, D.ffn, dense_above, db.flag, st)) != hipSuccess)
      return hip_fail(e, "path choice launch");
    flag = db.flag;
  }
  if (path != FFN_PATH_SPARSE) {
    DenseArgs da = dense_args(p, db, x, B, y);
    da.bits = sets ? db.bits : nullptr;
    da.idx_out = idx;
    da.cnt_out = cnt;
    da.run_if = flag;
    da.run_want = 1;
    if ((e = launch_dense(da, st, p->ev + FFN_STAGE_DENSE_UP)) != hipSuccess)
      return hip_fail(e, "dense launch");
  }
  if (path != FFN_PATH_DENSE) {
    a.run_if = flag;
    a.run_want = 0;
    if ((e = launch_batch_rows(a, 0, st, p->ev + FFN_STAGE_BATCH_UPGATE, P)) != hipSuccess)
      return hip_fail(e, "batched launch");
  }
  g_err[0] = 0;
  return FFN_OK;
}

}  // namespace

extern "C" {

ffn_status ffn_sparse_forward(ffn_plan* p, const void* x, int32_t B, float* y,
                              const uint8_t* mask, int32_t* idx, int32_t* cnt, float* scores,
                              int32_t path, void* stream) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!x || !y) return fail(FFN_ERR_INVALID_ARGUMENT, "x / y is NULL");
  const ffn_layer_desc& D = p->desc;
  if (B < 1 || B > D.max_batch)
    return fail(FFN_ERR_INVALID_ARGUMENT, "B = %d outside [1, %d]", B, D.max_batch);
  if (!mask && D.rank == 0)
    return fail(FFN_ERR_INVALID_ARGUMENT, "no predictor (rank 0) and no mask");
  if (path < FFN_PATH_AUTO || path > FFN_PATH_DENSE)
    return fail(FFN_ERR_INVALID_ARGUMENT, "path %d is not an ffn_path", path);
  if (!aligned16(x) || !aligned16(y) || !aligned16(mask))
    return fail(FFN_ERR_INVALID_ARGUMENT, "x / y / mask not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t xbytes = (size_t)D.d * (D.x_dtype == FFN_F32 ? 4 : 2);
  // Paths.  fp32 / int4 layers always run the per-token kernels (they have no MFMA path; a
  // dense request gives the same result over the same sets).  fp16:
  //  - B >= DENSE_MIN_M (and a dense region): sets first, then dense GEMMs / sparse passes /
  //    the device's choice between them (run_large);
  //  - otherwise SPARSE runs the batch-1 kernels for one token and the batched kernels for
  //    more; DENSE and AUTO run the batched kernels, widening the pass's union to every neuron
  //    (DENSE: always; AUTO: when it exceeds the crossover density).
  if (batched(&D) && p->off_dense && B >= DENSE_MIN_M)
    return run_large(p, x, B, y, mask, idx, cnt, scores, path, st, false);
  if (batched(&D) && (B > 1 || path == FFN_PATH_DENSE)) {
    int choose = 0, dense_above = 0;
    if (path == FFN_PATH_DENSE) {
      choose = 1;
      dense_above = -1;
    } else if (path == FFN_PATH_AUTO && B >= p->dense_min_batch) {
      float rho = 1.0f;
      ffn_plan_crossover(p, std::min(B, BATCH_TILE), &rho);
      choose = rho < 1.0f;
      dense_above = (int)(rho * D.ffn);
    }
    for (int b0 = 0; b0 < B; b0 += BATCH_TILE) {
      BatchArgs a = batch_bufs(p->ws, p);
      a.B = std::min(BATCH_TILE, B - b0);
      a.x = static_cast<const char*>(x) + b0 * xbytes;
      a.mask = mask ? mask + (size_t)b0 * D.ffn : nullptr;
      a.y = y + (size_t)b0 * D.d;
      a.scores = scores ? scores + (size_t)b0 * D.ffn : nullptr;
      a.idx_out = idx ? idx + (size_t)b0 * D.ffn : nullptr;
      a.cnt_out = cnt ? cnt + b0 : nullptr;
      a.dense_above = dense_above;
      hipError_t e = launch_batch(a, mask == nullptr, choose, st, p->ev + FFN_STAGE_BATCH_UPGATE);
      if (e != hipSuccess) return hip_fail(e, "batched launch");
    }
    g_err[0] = 0;
    return FFN_OK;
  }
  const TokenBufs wb = token_bufs(p->ws, p);
  for (int b = 0; b < B; ++b) {
    ffn_status s = enqueue_token(p, wb, static_cast<const char*>(x) + b * xbytes,
                                 mask ? mask + (size_t)b * D.ffn : nullptr, y + (size_t)b * D.d,
                                 idx ? idx + (size_t)b * D.ffn : nullptr, cnt ? cnt + b : nullptr,
                                 scores ? scores + (size_t)b * D.ffn : nullptr, nullptr, 1, 0, st);
    if (s != FFN_OK) return s;
  }
  g_err[0] = 0;
  return FFN_OK;
}

ffn_status ffn_sparse_forward_static(const ffn_layer_desc* desc, const ffn_layer_weights* w,
                                     const void* x, int32_t B, float* y, const uint8_t* mask,
                                     int32_t* idx, int32_t* cnt, void* stream) {
  ffn_status st = check_desc(desc);
  if (st != FFN_OK) return st;
  if (!w) return fail(FFN_ERR_INVALID_ARGUMENT, "weights is NULL");
  if ((st = check_weights(desc, w)) != FFN_OK) return st;
  if (!x || !y) return fail(FFN_ERR_INVALID_ARGUMENT, "x / y is NULL");
  if (B < 1 || B > desc->max_batch)
    return fail(FFN_ERR_INVALID_ARGUMENT, "B = %d outside [1, %d]", B, desc->max_batch);
  if (!mask && desc->rank == 0)
    return fail(FFN_ERR_INVALID_ARGUMENT, "no predictor (rank 0) and no mask");
  if (!aligned16(x) || !aligned16(y) || !aligned16(mask))
    return fail(FFN_ERR_INVALID_ARGUMENT, "x / y / mask not 16-byte aligned");
  // one token's scratch: z | bitmap | |A| | partials of the balanced gather's workgroups
  const Layout L = layout_for(desc);
  const size_t need =
      L.off_part + (size_t)gather_blocks() * reduce_tiles(desc->d) * 16 * 4;
  if (need > STATIC_SCRATCH_BYTES)
    return fail(FFN_ERR_WORKSPACE_TOO_SMALL,
                "d = %d, ffn = %d, rank = %d needs %zu bytes of scratch; the static scratch "
                "holds %zu (d <= 4096)", desc->d, desc->ffn, desc->rank, need,
                STATIC_SCRATCH_BYTES);
  char* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != FFN_OK) return st;
  ffn_plan p{};                                   // on the stack: nothing is allocated
  init_plan(&p, desc, w, ws, STATIC_SCRATCH_BYTES);
  hipStream_t sm = static_cast<hipStream_t>(stream);
  const size_t xbytes = (size_t)desc->d * (desc->x_dtype == FFN_F32 ? 4 : 2);
  const TokenBufs wb = token_bufs(ws, &p);
  for (int b = 0; b < B; ++b) {
    st = enqueue_token(&p, wb, static_cast<const char*>(x) + b * xbytes,
                       mask ? mask + (size_t)b * desc->ffn : nullptr, y + (size_t)b * desc->d,
                       idx ? idx + (size_t)b * desc->ffn : nullptr, cnt ? cnt + b : nullptr,
                       nullptr, nullptr, 1, 0, sm);
    if (st != FFN_OK) return st;
  }
  g_err[0] = 0;
  return FFN_OK;
}

ffn_status ffn_dense_forward(ffn_plan* p, const void* x, int32_t B, float* y,
                             const uint8_t* mask, void* stream) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!x || !y) return fail(FFN_ERR_INVALID_ARGUMENT, "x / y is NULL");
  const ffn_layer_desc& D = p->desc;
  if (B < 1 || B > D.max_batch)
    return fail(FFN_ERR_INVALID_ARGUMENT, "B = %d outside [1, %d]", B, D.max_batch);
  if (!aligned16(x) || !aligned16(y) || !aligned16(mask))
    return fail(FFN_ERR_INVALID_ARGUMENT, "x / y / mask not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t xbytes = (size_t)D.d * (D.x_dtype == FFN_F32 ? 4 : 2);
  if (batched(&D) && p->off_dense && B >= DENSE_MIN_M)
    return run_large(p, x, B, y, mask, nullptr, nullptr, nullptr, FFN_PATH_DENSE, st, true);
  if (batched(&D)) {
    for (int b0 = 0; b0 < B; b0 += BATCH_TILE) {
      BatchArgs a = batch_bufs(p->ws, p);
      a.B = std::min(BATCH_TILE, B - b0);
      a.x = static_cast<const char*>(x) + b0 * xbytes;
      a.mask = mask ? mask + (size_t)b0 * D.ffn : nullptr;
      a.y = y + (size_t)b0 * D.d;
      a.dense_above = -1;                  // every neuron's rows
      hipError_t e = launch_batch(a, 0, 1, st, p->ev + FFN_STAGE_BATCH_UPGATE);
      if (e != hipSuccess) return hip_fail(e, "dense launch");
    }
  } else {
    // fp32 / int4: the per-token kernels over every neuron (or the caller's sets)
    const TokenBufs wb = token_bufs(p->ws, p);
    for (int b = 0; b < B; ++b) {
      ffn_status s = enqueue_token(p, wb, static_cast<const char*>(x) + b * xbytes,
                                   mask ? mask + (size_t)b * D.ffn : nullptr, y + (size_t)b * D.d,
                                   nullptr, nullptr, nullptr, nullptr, 1, 0, st, true);
      if (s != FFN_OK) return s;
    }
  }
  g_err[0] = 0;
  return FFN_OK;
}

ffn_status ffn_plan_crossover(const ffn_plan* p, int32_t B, float* density) {
  if (!p || !density) return fail(FFN_ERR_INVALID_ARGUMENT, "plan / density is NULL");
  if (B < 1) return fail(FFN_ERR_INVALID_ARGUMENT, "B < 1");
  int k = 0;
  while (k < 12 && (1 << (k + 1)) <= B) ++k;
  *density = p->crossover_density[k];
  return FFN_OK;
}

ffn_status ffn_plan_set_crossover(ffn_plan* p, int32_t B, float density) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (B < 1) return fail(FFN_ERR_INVALID_ARGUMENT, "B < 1");
  if (!(density >= 0.0f && density <= 1.0f))
    return fail(FFN_ERR_INVALID_ARGUMENT, "density must lie in [0, 1]");
  int k = 0;
  while (k < 12 && (1 << (k + 1)) <= B) ++k;
  p->crossover_density[k] = density;
  return FFN_OK;
}

ffn_status ffn_plan_path_flag(const ffn_plan* p, const int32_t** flag) {
  if (!p || !flag) return fail(FFN_ERR_INVALID_ARGUMENT, "plan / flag is NULL");
  if (!p->off_dense)
    return fail(FFN_ERR_UNSUPPORTED, "the plan has no dense GEMMs (fp16 rows, max_batch >= %d)",
                DENSE_MIN_M);
  *flag = dense_bufs(p->ws, p).flag;
  return FFN_OK;
}

ffn_status ffn_plan_set_decode_variant(ffn_plan* p, int32_t variant) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (variant < 0 || variant > 1)
    return fail(FFN_ERR_INVALID_ARGUMENT, "variant %d is not 0 or 1", variant);
  const ffn_layer_desc& D = p->desc;
  const int wk = D.w_dtype == FFN_F32 ? WK_F32 : D.w_dtype == FFN_F16 ? WK_F16 : WK_I4;
  if (variant == 1 && p->cache_cap > 0)
    return fail(FFN_ERR_UNSUPPORTED, "the fused decode variant does not read a neuron cache");
  if (variant == 1 && (!fused_supported(wk, D.d) || D.rank == 0))
    return fail(FFN_ERR_UNSUPPORTED, "the fused decode variant needs fp32 / fp16 rows of "
                "%d..%d chunks and a predictor", 64, 1024);
  p->decode_variant = variant;
  return FFN_OK;
}

ffn_status ffn_plan_set_hot_head(ffn_plan* p, int32_t n_hot) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (n_hot < 0 || n_hot > p->desc.ffn || n_hot % 32 != 0)
    return fail(FFN_ERR_INVALID_ARGUMENT, "n_hot %d must be a multiple of 32 in [0, %d]", n_hot,
                p->desc.ffn);
  p->head_words = n_hot / 32;
  return FFN_OK;
}

ffn_status ffn_plan_set_timing_events(ffn_plan* p, int32_t stage, void* start, void* stop) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (stage < FFN_STAGE_PRED_Z || stage > FFN_STAGE_DENSE_REDUCE)
    return fail(FFN_ERR_INVALID_ARGUMENT, "stage %d is not an ffn_stage", stage);
  if ((start == nullptr) != (stop == nullptr))
    return fail(FFN_ERR_INVALID_ARGUMENT, "start and stop must both be set or both be NULL");
  p->ev[stage][0] = static_cast<hipEvent_t>(start);
  p->ev[stage][1] = static_cast<hipEvent_t>(stop);
  return FFN_OK;
}

ffn_status ffn_plan_destroy(ffn_plan* p) {
  delete p;
  return FFN_OK;
}

ffn_status ffn_moe_workspace_size(int32_t n_experts, int32_t top_k, const ffn_plan* e0,
                                  size_t* bytes) {
  if (!e0 || !bytes) return fail(FFN_ERR_INVALID_ARGUMENT, "expert0 / bytes is NULL");
  if (n_experts < 1 || n_experts > MOE_MAX_E)
    return fail(FFN_ERR_UNSUPPORTED, "n_experts must lie in [1, %d]", MOE_MAX_E);
  if (top_k < 1 || top_k > MOE_MAX_K || top_k > n_experts)
    return fail(FFN_ERR_UNSUPPORTED, "top_k must lie in [1, min(n_experts, %d)]", MOE_MAX_K);
  *bytes = moe_layout(e0, n_experts, top_k).total;
  g_err[0] = 0;
  return FFN_OK;
}

ffn_status ffn_moe_plan(int32_t n_experts, int32_t top_k, const void* w_router,
                        ffn_plan* const* experts, void* workspace, size_t workspace_bytes,
                        ffn_moe** out) {
  if (!out) return fail(FFN_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (!experts || !w_router || !workspace)
    return fail(FFN_ERR_INVALID_ARGUMENT, "experts / w_router / workspace is NULL");
  for (int e = 0; e < n_experts && e < MOE_MAX_E; ++e)
    if (!experts[e]) return fail(FFN_ERR_INVALID_ARGUMENT, "expert plan %d is NULL", e);
  size_t need = 0;
  ffn_status st = ffn_moe_workspace_size(n_experts, top_k, experts[0], &need);
  if (st != FFN_OK) return st;
  const ffn_layer_desc& D = experts[0]->desc;
  if (D.rank == 0) return fail(FFN_ERR_INVALID_ARGUMENT, "experts need a predictor (rank > 0)");
  for (int e = 0; e < n_experts && e < MOE_MAX_E; ++e)
    if (experts[e]->cache_cap > 0)
      return fail(FFN_ERR_UNSUPPORTED, "expert %d is a neuron-cache plan", e);
  for (int e = 1; e < n_experts; ++e) {
    const ffn_layer_desc& E = experts[e]->desc;
    if (E.d != D.d || E.ffn != D.ffn || E.rank != D.rank || E.act != D.act ||
        E.w_dtype != D.w_dtype || E.x_dtype != D.x_dtype || E.p_dtype != D.p_dtype ||
        E.threshold != D.threshold || E.max_batch != D.max_batch)
      return fail(FFN_ERR_INVALID_ARGUMENT, "expert %d differs from expert 0 in its descriptor", e);
  }
  if (!aligned16(w_router) || !aligned16(workspace))
    return fail(FFN_ERR_INVALID_ARGUMENT, "pointer not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(FFN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  ffn_moe* m = new (std::nothrow) ffn_moe();
  if (!m) return fail(FFN_ERR_INTERNAL, "out of host memory");
  m->n_experts = n_experts;
  m->top_k = top_k;
  m->router = w_router;
  m->e0 = experts[0];
  m->ws = static_cast<char*>(workspace);
  m->L = moe_layout(experts[0], n_experts, top_k);
  for (int e = 0; e < n_experts; ++e) {
    const ffn_layer_weights& w = experts[e]->w;
    ExpertW& r = m->tab.e[e];
    r.p1 = w.p1;
    r.p2 = w.p2;
    r.c1 = w.c1;
    r.c2 = w.c2;
    r.w_up = w.w_up;
    r.w_gate = w.w_gate;
    r.w_dn = w.w_down_t;
    r.s_up = w.s_up;
    r.s_gate = w.s_gate;
    r.s_dn = w.s_down_t;
    r.b_up = w.b_up;
    r.b_gate = w.b_gate;
    r.b_down = w.b_down;
    r.wgt = 0.0f;
    r.expert = e;
  }
  *out = m;
  g_err[0] = 0;
  return FFN_OK;
}

ffn_status ffn_moe_forward(ffn_moe* m, const void* x, int32_t B, float* y, int32_t* expert_idx,
                           float* expert_w, int32_t* expert_cnt, void* stream) {
  if (!m) return fail(FFN_ERR_INVALID_ARGUMENT, "moe is NULL");
  if (!x || !y) return fail(FFN_ERR_INVALID_ARGUMENT, "x / y is NULL");
  const ffn_plan* p = m->e0;
  const ffn_layer_desc& D = p->desc;
  if (B < 1 || B > D.max_batch)
    return fail(FFN_ERR_INVALID_ARGUMENT, "B = %d outside [1, %d]", B, D.max_batch);
  if (!aligned16(x) || !aligned16(y))
    return fail(FFN_ERR_INVALID_ARGUMENT, "x / y not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  ExpertW* slots = reinterpret_cast<ExpertW*>(m->ws + m->L.off_slots);
  RouterArgs ra{};
  ra.R = m->router;
  ra.x = x;
  ra.ids_out = expert_idx;
  ra.w_out = expert_w;
  ra.slots = slots;
  ra.d = D.d;
  ra.E = m->n_experts;
  ra.K = m->top_k;
  ra.x_f16 = D.x_dtype == FFN_F16;
  ra.tab = m->tab;
  float* zall = reinterpret_cast<float*>(m->ws + m->L.off_zall);
  ra.zall = zall;
  ra.rank = D.rank;
  ra.cpl = p->cpl_p;
  ra.B = B;
  // timed as the plan's stage-1 stage (it is the mixture's stage 1, with the router)
  hipError_t e = launch_route_z(ra, st, p->ev[FFN_STAGE_PRED_Z][0], p->ev[FFN_STAGE_PRED_Z][1]);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  const size_t xbytes = (size_t)D.d * (D.x_dtype == FFN_F32 ? 4 : 2);
  const TokenBufs wb = token_bufs(m->ws, p);
  for (int b = 0; b < B; ++b) {
    // the token's top_k experts run side by side, one launch per stage
    ffn_status s = enqueue_token(p, wb, static_cast<const char*>(x) + b * xbytes, nullptr,
                                 y + (size_t)b * D.d, nullptr,
                                 expert_cnt ? expert_cnt + (size_t)b * m->top_k : nullptr, nullptr,
                                 slots + (size_t)b * m->top_k, m->top_k, m->L.slot_stride, st,
                                 false, zall + (size_t)b * m->n_experts * D.rank);
    if (s != FFN_OK) return s;
  }
  g_err[0] = 0;
  return FFN_OK;
}

ffn_status ffn_moe_destroy(ffn_moe* m) {
  delete m;
  return FFN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Attention block with a head-level active set (kernels in attn.hip).
struct ffn_attn {
  ffn_attn_desc desc;
  ffn_attn_weights w;
  char* ws;
  size_t off_z, off_hdr, off_alist, off_q, off_rec, off_part;
  int cpl_w;
  hipEvent_t ev[FFN_STAGE_ATTN_REDUCE + 1][2];
};

namespace {

ffn_status check_attn_desc(const ffn_attn_desc* d) {
  if (!d) return fail(FFN_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->d <= 0 || d->d % 8 || d->d > 8192)
    return fail(FFN_ERR_UNSUPPORTED, "d = %d: need d %% 8 == 0 and d <= 8192", d->d);
  if (d->heads < 1 || d->heads > ATTN_MAX_HEADS)
    return fail(FFN_ERR_UNSUPPORTED, "heads = %d: need 1..%d", d->heads, ATTN_MAX_HEADS);
  if (d->kv_heads < 1 || d->heads % d->kv_heads)
    return fail(FFN_ERR_UNSUPPORTED, "kv_heads = %d must divide heads = %d", d->kv_heads,
                d->heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(FFN_ERR_UNSUPPORTED, "head_dim = %d: need 64 or 128", d->head_dim);
  if (d->heads * d->head_dim > ATTN_OUT_BLOCKS * ATTN_OUT_MAXR)
    return fail(FFN_ERR_UNSUPPORTED, "heads * head_dim = %d exceeds %d",
                d->heads * d->head_dim, ATTN_OUT_BLOCKS * ATTN_OUT_MAXR);
  if (d->rank < 0 || d->rank % 8 || d->rank > ATTN_MAX_RANK)
    return fail(FFN_ERR_UNSUPPORTED, "rank = %d: need rank %% 8 == 0 and rank <= %d", d->rank,
                ATTN_MAX_RANK);
  if (d->max_seq < 1) return fail(FFN_ERR_INVALID_ARGUMENT, "max_seq = %d", d->max_seq);
  if (!(d->threshold > 0.0f && d->threshold <= 1.0f))
    return fail(FFN_ERR_INVALID_ARGUMENT, "threshold %g not in (0, 1]", (double)d->threshold);
  if (cpl_for(d->d / 8) < 0) return fail(FFN_ERR_UNSUPPORTED, "d too large");
  return FFN_OK;
}

size_t attn_layout(const ffn_attn_desc* d, ffn_attn* p) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  const size_t z = take(sizeof(float) * std::max(d->rank, 8));
  const size_t hdr = take(64);
  const size_t alist = take(sizeof(int) * ATTN_MAX_HEADS);
  const size_t q = take(sizeof(float) * (size_t)d->heads * d->head_dim);
  const size_t rec = take(sizeof(float) * (size_t)d->heads * ATTN_MAX_CHUNKS * (d->head_dim + 4));
  const size_t part = take(sizeof(float) * (size_t)ATTN_OUT_BLOCKS * d->d);
  if (p) {
    p->off_z = z;
    p->off_hdr = hdr;
    p->off_alist = alist;
    p->off_q = q;
    p->off_rec = rec;
    p->off_part = part;
  }
  return off;
}

}  // namespace

extern "C" {

ffn_status ffn_attn_workspace_size(const ffn_attn_desc* desc, size_t* bytes) {
  ffn_status st = check_attn_desc(desc);
  if (st != FFN_OK) return st;
  if (!bytes) return fail(FFN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = attn_layout(desc, nullptr);
  return FFN_OK;
}

ffn_status ffn_attn_plan(const ffn_attn_desc* desc, const ffn_attn_weights* w, void* workspace,
                         size_t workspace_bytes, ffn_attn** out) {
  ffn_status st = check_attn_desc(desc);
  if (st != FFN_OK) return st;
  if (!w || !out) return fail(FFN_ERR_INVALID_ARGUMENT, "weights or out is NULL");
  if (!w->w_q || !w->w_k || !w->w_v || !w->w_o_t)
    return fail(FFN_ERR_INVALID_ARGUMENT, "w_q, w_k, w_v and w_o_t are required");
  if (desc->rank > 0 && (!w->p1 || !w->p2))
    return fail(FFN_ERR_INVALID_ARGUMENT, "rank > 0 needs p1 and p2");
  const void* ptrs[] = {w->w_q, w->w_k, w->w_v, w->w_o_t, w->p1, w->p2, w->c1, w->c2, workspace};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(FFN_ERR_INVALID_ARGUMENT, "pointer not 16-byte aligned");
  if (!workspace) return fail(FFN_ERR_INVALID_ARGUMENT, "workspace is NULL");
  const size_t need = attn_layout(desc, nullptr);
  if (workspace_bytes < need)
    return fail(FFN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                need);
  ffn_attn* p = new (std::nothrow) ffn_attn();
  if (!p) return fail(FFN_ERR_INTERNAL, "out of host memory");
  p->desc = *desc;
  p->w = *w;
  p->ws = static_cast<char*>(workspace);
  attn_layout(desc, p);
  p->cpl_w = cpl_for(desc->d / 8);
  *out = p;
  return FFN_OK;
}

ffn_status ffn_attn_forward(ffn_attn* p, const void* x, int32_t pos, void* k_cache,
                            void* v_cache, float* y, const uint8_t* mask, int32_t* idx,
                            int32_t* cnt, float* scores, void* stream) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  const ffn_attn_desc& D = p->desc;
  if (!x || !y || !k_cache || !v_cache)
    return fail(FFN_ERR_INVALID_ARGUMENT, "x, y, k_cache and v_cache are required");
  if (!aligned16(x) || !aligned16(y) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(FFN_ERR_INVALID_ARGUMENT, "x, y and the caches must be 16-byte aligned");
  if (pos < 0 || pos >= D.max_seq)
    return fail(FFN_ERR_INVALID_ARGUMENT, "pos = %d not in [0, %d)", pos, D.max_seq);
  if (!mask && D.rank == 0)
    return fail(FFN_ERR_INVALID_ARGUMENT, "no predictor (rank 0): a mask is required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = p->ws;
  AttnArgs a{};
  a.wq = p->w.w_q;
  a.wk = p->w.w_k;
  a.wv = p->w.w_v;
  a.wo = p->w.w_o_t;
  a.p2 = p->w.p2;
  a.c2 = p->w.c2;
  a.z = reinterpret_cast<const float*>(ws + p->off_z);
  a.mask = mask;
  a.x = x;
  a.kc = k_cache;
  a.vc = v_cache;
  a.q = reinterpret_cast<float*>(ws + p->off_q);
  a.bits = reinterpret_cast<uint32_t*>(ws + p->off_hdr);
  a.cnt = reinterpret_cast<int*>(ws + p->off_hdr + 16);
  a.alist = reinterpret_cast<int*>(ws + p->off_alist);
  a.rec = reinterpret_cast<float*>(ws + p->off_rec);
  a.part = reinterpret_cast<float*>(ws + p->off_part);
  a.y = y;
  a.scores_out = mask ? nullptr : scores;
  a.idx_out = idx;
  a.cnt_out = cnt;
  a.d = D.d;
  a.H = D.heads;
  a.G = D.kv_heads;
  a.e = D.head_dim;
  a.S = D.max_seq;
  a.pos = pos;
  a.rank = D.rank;
  attn_chunk_split(D.heads, attn_step_positions(D.head_dim), pos + 1, ATTN_MAX_CHUNKS, a.lc,
                   a.nchunk);
  const double tau = D.threshold;
  a.thr = tau >= 1.0 ? INFINITY : (float)log(tau / (1.0 - tau));
  a.scale = 1.0f / sqrtf((float)D.head_dim);
  hipError_t e = hipSuccess;
  if (!mask) {
    e = launch_pred_z(1, p->cpl_w, p->w.p1, p->w.c1, x, reinterpret_cast<float*>(ws + p->off_z),
                      D.d, D.rank, nullptr, 1, 0, st, p->ev[FFN_STAGE_PRED_Z][0],
                      p->ev[FFN_STAGE_PRED_Z][1]);
    if (e != hipSuccess) return hip_fail(e, "attention predictor stage 1");
  }
  e = launch_attn_proj(p->cpl_w, a, st, p->ev[FFN_STAGE_ATTN_PROJ][0],
                       p->ev[FFN_STAGE_ATTN_PROJ][1]);
  if (e != hipSuccess) return hip_fail(e, "attention projections");
  e = launch_attn_part(a, st, p->ev[FFN_STAGE_ATTN_SCORES][0], p->ev[FFN_STAGE_ATTN_SCORES][1]);
  if (e != hipSuccess) return hip_fail(e, "attention scores");
  e = launch_attn_out(a, st, p->ev[FFN_STAGE_ATTN_OUT][0], p->ev[FFN_STAGE_ATTN_OUT][1]);
  if (e != hipSuccess) return hip_fail(e, "attention output projection");
  e = launch_attn_reduce(a, st, p->ev[FFN_STAGE_ATTN_REDUCE][0], p->ev[FFN_STAGE_ATTN_REDUCE][1]);
  if (e != hipSuccess) return hip_fail(e, "attention reduce");
  return FFN_OK;
}

ffn_status ffn_attn_set_timing_events(ffn_attn* p, int32_t stage, void* start, void* stop) {
  if (!p) return fail(FFN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (stage != FFN_STAGE_PRED_Z && (stage < FFN_STAGE_ATTN_PROJ || stage > FFN_STAGE_ATTN_REDUCE))
    return fail(FFN_ERR_INVALID_ARGUMENT, "stage %d is not an attention stage", stage);
  if ((start == nullptr) != (stop == nullptr))
    return fail(FFN_ERR_INVALID_ARGUMENT, "start and stop must both be set or both be NULL");
  p->ev[stage][0] = static_cast<hipEvent_t>(start);
  p->ev[stage][1] = static_cast<hipEvent_t>(stop);
  return FFN_OK;
}

ffn_status ffn_attn_destroy(ffn_attn* p) {
  delete p;
  return FFN_OK;
}

}  // extern "C"
