// Launchers shared between the kernel translation units and the C-ABI layer (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ffn {

// One expert's weights as the kernels read them when the expert is chosen on the device (a
// mixture of experts): the router copies the chosen experts' records into per-slot records in
// the workspace, and a kernel given such a record takes its weight pointers from it instead of
// from its arguments.  wgt is the slot's routing weight.
struct ExpertW {
  const void *p1, *p2;
  const float *c1, *c2;
  const void *w_up, *w_gate, *w_dn, *s_up, *s_gate, *s_dn;
  const float *b_up, *b_gate, *b_down;
  float wgt;
  int expert;
};
constexpr int MOE_MAX_E = 16;
constexpr int MOE_MAX_K = 4;
struct ExpertTable {
  ExpertW e[MOE_MAX_E];
};

// Router of a mixture of experts (B tokens, one workgroup each).
struct RouterArgs {
  const void* R;              // [E][d] x dtype
  const void* x;              // [B][d]
  int* ids_out;               // [B][K] or nullptr
  float* w_out;               // [B][K] or nullptr
  ExpertW* slots;             // [B][K] out
  int d, E, K, x_f16;
  ExpertTable tab;
  // predictor stage 1 of the chosen experts, computed in the router's launch (each stage-1
  // workgroup reaches its token's routing decision itself): zall[(b * E + e) * rank + k] =
  // c1_e[k] + P1_e[k] . x_b for the K experts e chosen for token b (the other rows untouched)
  float* zall;
  int rank, cpl, B;
};

// Predictor stage 2 (one token).
struct PredArgs {
  const void* p2;             // [ffn][rank] p_dtype
  const float* c2;            // [ffn] or nullptr
  const float* z;             // [rank] from stage 1
  float* scores;              // [ffn] or nullptr
  uint32_t* bitmap;           // [ffn/32] out
  int ffn, rank;
  float thr;                  // logit(threshold)
  const ExpertW* slot;        // device-chosen expert (p2, c2 from it), or nullptr
  int nslot;                  // expert slots run side by side (grid.y); slot k uses slot + k,
  int zstride, bstride;       //   z + k*zstride, bitmap + k*bstride (elements)
  int head_words;             // hot head: bitmap words [0, head_words) always set, their P2 rows
                              //   and c2 entries never read
  const float* zall;          // expert slots: the token's stage-1 results of every expert
                              //   ([E][rank]); slot k reads the row of its expert
};

// Balanced gather of the active rows (one token).
struct GatherArgs {
  const void* w_up;
  const void* w_gate;
  const void* w_dn;           // [ffn][d] transposed down rows
  const void* s_up;
  const void* s_gate;
  const void* s_dn;
  const float* b_up;
  const float* b_gate;
  const void* x;              // token, x_dtype
  const uint32_t* bitmap;     // [ffn/32]
  float* part;                // [GA_BLOCKS][d] out: partial of y per workgroup
  int* cnt;                   // [1] out: |A|
  int d, ffn, act, has_gate;
  const ExpertW* slot;        // device-chosen expert (rows, scales, biases from it), or nullptr
  int nslot;                  // expert slots side by side (grid.y): slot + k, bitmap + k*bstride,
  int bstride, cstride;       //   cnt + k*cstride, part + k*pstride (elements)
  size_t pstride;
  // neuron cache (host-resident rows): per rank the neuron, the cache slot its rows are read
  // from (-1: from w_up / w_gate / w_dn, which then point to host memory) and the slot they are
  // written to on the way (-1: none); |A| is read from cnt
  const int* rank_nid;
  const int* rank_src;
  const int* rank_vic;
  void* c_up;                 // cache rows [capacity][d]
  void* c_gate;
  void* c_dn;
};

// Neuron cache of host-resident rows (one token): tables and per-rank outputs.
constexpr int CACHE_MAX_SLOTS = 8192;
struct CacheArgs {
  const uint32_t* bitmap;     // [ffn/32] the token's active set
  int ffn, cap;               // neurons, cache slots
  int* slot_of;               // [ffn] slot holding the neuron, or -1
  int* neuron_of;             // [cap] neuron in the slot, or -1
  uint32_t* last_use;         // [cap] stamp of the last token that used the slot (pinned: ~0)
  uint32_t* stamp;            // [1] stamp of the last token
  int* cnt;                   // [1] out: |A|
  int* rank_nid;              // [ffn] out per rank: neuron, source slot (-1: host), admission slot
  int* rank_src;
  int* rank_vic;
  int* stats;                 // [8] out: hits, misses, admitted, |A|; then their running totals
};

// Sum of the gather partials (one token).
struct ReduceArgs {
  const float* part;          // [n_part][d]
  const int* cnt;             // [1] |A| (tells which gather workgroups wrote a partial)
  const uint32_t* bitmap;     // [ffn/32], for the index-list output
  const float* b_down;
  float* y;                   // [d]
  int* idx_out;               // [ffn] ascending active list, or nullptr (one token)
  int* cnt_out;               // [1] |A|, or nullptr; expert slots: [nslot], each slot's |A|
  int d, ffn, n_part;
  int fused;                  // partials from the fused kernel: partial c exists iff bitmap words
                              //   2c, 2c+1 are not both zero (else: from |A| and the rank split)
  const ExpertW* slot;        // device-chosen experts: b_down and the routing weights, or nullptr
  int nslot;                  // y = sum over the nslot slots (in order) of wgt_k * result_k;
  int cstride;                //   slot k's partials at part + k*pstride, its |A| at cnt + k*cstride
  size_t pstride;
};

// Fused predictor stage 2 + gather (the alternative batch-1 decode variant): a workgroup
// scores its own 64 neurons and gathers the active ones among them (no rank balancing, one
// launch fewer).  Partials: one per workgroup, tile-major like the balanced gather's.
struct FusedArgs {
  PredArgs pa;                // p2, c2, z, scores, bitmap, ffn, rank, thr
  GatherArgs ga;              // rows, scales, biases, x, part, d, act, has_gate
};
int fused_blocks(int ffn);
bool fused_supported(int wk, int d);
hipError_t launch_fused(int wk, const FusedArgs& a, hipStream_t st, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr);

hipError_t launch_pred_z(int p_f16, int cpl, const void* p1, const float* c1, const void* x,
                         float* z, int d, int rank, const ExpertW* slot, int nslot, int zstride,
                         hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
int pred_s_cpr(int p_f16, int rank);
hipError_t launch_pred_s(int p_f16, const PredArgs& a, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
hipError_t launch_mask_bits(const unsigned char* mask, uint32_t* bitmap, int words,
                            hipStream_t st);
int gather_cpt(int wk, int d);
int gather_blocks(int nslot = 1);
int reduce_tiles(int d);
hipError_t launch_gather(int wk, const GatherArgs& a, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
hipError_t launch_gather_cached(const GatherArgs& a, hipStream_t st, hipEvent_t ev0,
                                hipEvent_t ev1);
hipError_t launch_cache_plan(const CacheArgs& a, hipStream_t st);
hipError_t launch_cache_init(const CacheArgs& a, int n_pinned, hipStream_t st);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
hipError_t launch_route_z(const RouterArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

// Batched path (fp16 layers): up to BATCH_TILE tokens per pass share one read of the union of
// their active neurons' rows.
constexpr int BATCH_TILE = 32;

struct BatchArgs {
  const void* x;              // [B][d] fp16, this pass's tokens
  const uint8_t* mask;        // [B][ffn] caller sets (k_bmask; nullptr there = every neuron)
  const void *p1, *p2;
  const float *c1, *c2;
  const void *w_up, *w_gate, *w_dn;
  const float *b_up, *b_gate, *b_down;
  float* zpart;               // [ks][BATCH_TILE][r] partial sums of predictor stage 1
  _Float16* zhl;              // [2][BATCH_TILE][r] z as fp16 hi + lo
  uint32_t* bits;             // [BATCH_TILE][ffn/32] per-token active bitmaps
  uint32_t* ubits;            // [ffn/32] union bitmap
  int* ucnt;                  // [1] |U|
  int* uidx;                  // [ffn] union neurons by rank
  _Float16* H;                // [BATCH_TILE][ffn] h per token, column = union rank
  float* ypart;               // [S][BATCH_TILE][d] per-segment partials of y
  float* y;                   // [B][d]
  float* scores;              // [B][ffn] or nullptr
  int* idx_out;               // [B][ffn] or nullptr
  int* cnt_out;               // [B] or nullptr
  int B, d, ffn, r, act, has_gate;
  int ks, spw, S;
  float thr;
  int dense_above;            // path choice: union larger than this -> every neuron's row
  const int* run_if;          // device flag: the row kernels run only if *run_if == run_want
  int run_want;               //   (nullptr: always)
  int head_words;             // hot head (as PredArgs)
  _Float16* zcat;             // k_bzr: also z as [tokens][2 r] (hi then lo) for the stage-2 GEMM,
                              //   or nullptr
  // Several passes in one launch (grid.z = pass p, tokens [32p, 32p + 32) of the call): every
  // per-token pointer above advances by 32 tokens per pass, the per-pass buffers by the strides
  // below (elements), and B = min(32, Btot - 32p).  One pass: Btot = 0 and the strides unused.
  int Btot;
  size_t zpart_ps, zhl_ps, ubits_ps, uidx_ps, ypart_ps;
};

struct BatchShape {
  int ks, spw, S;
  size_t zpart_bytes, zhl_bytes, bits_bytes, ubits_bytes, uidx_bytes, H_bytes, ypart_bytes;
};
BatchShape batch_shape(int d, int ffn, int r);
// use_predictor: predictor kernels (else caller masks); choose_path: run k_bpath, which widens
// the union to every neuron when it holds more than dense_above neurons (-1: always).
// ev: (start, stop) pairs for k_bug and k_bdown (entries may be null), or nullptr.
hipError_t launch_batch(const BatchArgs& a, int use_predictor, int choose_path, hipStream_t st,
                        hipEvent_t (*ev)[2] = nullptr);
// The pieces: the pass's active sets (bits, scores, union) ...
hipError_t launch_batch_sets(const BatchArgs& a, int use_predictor, hipStream_t st,
                             int passes = 1);
// ... or only predictor stage 1 (z, and z as [tokens][2 r] when a.zcat is set) ...
hipError_t launch_batch_stage1(const BatchArgs& a, hipStream_t st, int passes);
// ... or only the fixed-order sum of stage 1's a.ks K-slice partials (k_bzr) ...
hipError_t launch_batch_zsum(const BatchArgs& a, hipStream_t st, int passes);
// ... the union recomputed from bits (when bits were written by an earlier step) ...
hipError_t launch_batch_union(const BatchArgs& a, hipStream_t st);
// ... and the rows (optional k_bpath, k_bug, k_bdown, k_bred).
hipError_t launch_batch_rows(const BatchArgs& a, int choose_path, hipStream_t st,
                             hipEvent_t (*ev)[2] = nullptr, int passes = 1);
// Device-side choice for a call whose passes' union words are in ubits[passes][ffn/32]: flag =
// 1 when the union of all of them holds more than dense_above neurons.
hipError_t launch_dense_choice(const uint32_t* ubits, int passes, int ffn, int dense_above,
                               int* flag, hipStream_t st);
// Segments of the down projection per pass when `passes` passes share one launch.
int batch_segments_mp(int d, int passes);

// Dense path (fp16 layers, many tokens): two MFMA GEMMs and a fixed-order reduce.
constexpr int DENSE_MIN_M = 64;   // token count from which the dense GEMMs replace the batched kernels

struct DenseArgs {
  const void* x;              // [M][d] fp16
  const uint32_t* bits;       // [M][ffn/32] per-token sets, or nullptr (every neuron)
  const void *w_up, *w_gate, *w_dn;
  const float *b_up, *b_gate, *b_down;
  _Float16* H;                // [M][ffn]
  float* ypart;               // [ks][M][d]
  float* y;                   // [M][d]
  int* idx_out;               // [M][ffn] or nullptr (from bits)
  int* cnt_out;               // [M] or nullptr
  int M, d, ffn, act, has_gate, ks;
  const int* run_if;          // device flag: run only if *run_if == run_want (nullptr: always)
  int run_want;
  // predictor stage 2 of a large call on the same GEMM kernel (launch_dense_scores):
  // S = [z_hi | z_lo] [P2 | P2]^T + c2 with x = [M][2 rank] fp16 (d = 2 rank), w_up = P2 (rows of
  // b_rowb bytes, its K repeating after bwrap stages), ffn = neurons; each token's bitmap words,
  // each pass's (32 tokens') union words and, optionally, the scores are written
  const float* c2;
  float thr;
  uint32_t* bits_out;         // [M][ffn/32]
  uint32_t* ubits_out;        // [passes][ffn/32]
  float* scores;              // [M][ffn] or nullptr
  int head_words;             // words [0, head_words): every neuron on, no score
  size_t b_rowb;
  int bwrap;
  // predictor stage 1 of a large call on the same GEMM kernel (launch_dense_zpart; tiles of
  // ZP_M x ZP_N): Z = X P1^T with x = X, w_up = P1, ffn = rank, split over d into kslices slices;
  // the fp32 partials go to zpart_out in the batched path's per-pass layout
  // ([pass][slice][32][rank], zpart_ps per pass)
  float* zpart_out;
  size_t zpart_ps;
  int kslices;
};
// K slices of the down projection for M tokens (k_ddq's or k_ddown's tiles: dense_down_wide).
int dense_ks(int M, int d, int ffn);
// K slices of the stage-1 GEMM for a call of M tokens (at most ZPART_MAX_KS).
constexpr int ZPART_MAX_KS = 16;
int zpart_kslices(int M, int d, int rank);
hipError_t launch_dense_zpart(const DenseArgs& a, hipStream_t st);
// Predictor stage 2 of a call of many tokens as one GEMM (fields above); rank % 32 == 0.
hipError_t launch_dense_scores(const DenseArgs& a, hipStream_t st);
// ev: three (start, stop) pairs for k_dup, k_ddown, k_dred (entries may be null), or nullptr
hipError_t launch_dense(const DenseArgs& a, hipStream_t st, hipEvent_t (*ev)[2]);

// Self-attention block of one token with a head-level active set (fp16 weights, token and
// cache).  Heads H <= ATTN_MAX_HEADS of width e in {64, 128}, G key/value heads (H % G == 0).
constexpr int ATTN_MAX_HEADS = 128;
constexpr int ATTN_MAX_RANK = 1024;
constexpr int ATTN_MAX_CHUNKS = 256;      // chunk records per head (positions per chunk: lc)
constexpr int ATTN_OUT_BLOCKS = 256;      // workgroups (and partials of y) of the output projection
constexpr int ATTN_OUT_MAXR = 64;         // rows per output workgroup: H e <= 256 * 64
struct AttnArgs {
  const void *wq, *wk, *wv, *wo;  // [H e][d], [G e][d], [G e][d], [H e][d] fp16 (wo transposed)
  const void* p2;                 // head predictor stage 2 [H][rank] fp16
  const float* c2;                // [H] or nullptr
  const float* z;                 // [rank] predictor stage 1
  const uint8_t* mask;            // [H] caller's head set, or nullptr (the predictor's)
  const void* x;                  // [d] fp16
  void *kc, *vc;                  // caches [G][S][e] fp16; position pos is written
  float* q;                       // [H][e] queries of the active heads, by rank
  uint32_t* bits;                 // [4] active-head bitmap
  int* cnt;                       // [1] |A|
  int* alist;                     // [H] active heads by rank
  float* rec;                     // [H][ATTN_MAX_CHUNKS][e + 4] chunk records: o, max, sum
  float* part;                    // [ATTN_OUT_BLOCKS][d] partials of y
  float* y;                       // [d]
  float* scores_out;              // [H] or nullptr (predictor scores)
  int* idx_out;                   // [H] or nullptr (ascending active heads)
  int* cnt_out;                   // [1] or nullptr
  int d, H, G, e, S, pos, rank;
  int lc, nchunk;                 // positions per chunk, chunks = ceil((pos + 1) / lc)
  float thr, scale;               // logit(tau), 1 / sqrt(e)
};
int attn_heads_per_wave(int H);
int attn_step_positions(int e);   // positions one k_attn_part step covers (lc is a multiple)
hipError_t launch_attn_proj(int cpl, const AttnArgs& a, hipStream_t st, hipEvent_t e0 = nullptr,
                            hipEvent_t e1 = nullptr);
hipError_t launch_attn_part(const AttnArgs& a, hipStream_t st, hipEvent_t e0 = nullptr,
                            hipEvent_t e1 = nullptr);
hipError_t launch_attn_out(const AttnArgs& a, hipStream_t st, hipEvent_t e0 = nullptr,
                           hipEvent_t e1 = nullptr);
hipError_t launch_attn_reduce(const AttnArgs& a, hipStream_t st, hipEvent_t e0 = nullptr,
                              hipEvent_t e1 = nullptr);

}  // namespace ffn
