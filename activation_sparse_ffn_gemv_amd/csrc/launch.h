// Launchers shared between the kernel translation units and the C-ABI layer (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ffn {

// Predictor stage 2 (one token).
struct PredArgs {
  const void* p2;             // [ffn][rank] p_dtype
  const float* c2;            // [ffn] or nullptr
  const float* z;             // [rank] from stage 1
  float* scores;              // [ffn] or nullptr
  uint32_t* bitmap;           // [ffn/32] out
  int ffn, rank;
  float thr;                  // logit(threshold)
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
};

// Sum of the gather partials (one token).
struct ReduceArgs {
  const float* part;          // [n_part][d]
  const int* cnt;             // [1] |A| (tells which gather workgroups wrote a partial)
  const uint32_t* bitmap;     // [ffn/32], for the index-list output
  const float* b_down;
  float* y;                   // [d]
  int* idx_out;               // [ffn] ascending active list, or nullptr
  int* cnt_out;               // [1], or nullptr
  int d, ffn, n_part;
};

hipError_t launch_pred_z(int p_f16, int cpl, const void* p1, const float* c1, const void* x,
                         float* z, int d, int rank, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
int pred_s_cpr(int p_f16, int rank);
hipError_t launch_pred_s(int p_f16, const PredArgs& a, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
hipError_t launch_mask_bits(const unsigned char* mask, uint32_t* bitmap, int words,
                            hipStream_t st);
int gather_cpt(int wk, int d);
int gather_blocks();
int reduce_tiles(int d);
hipError_t launch_gather(int wk, const GatherArgs& a, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);

}  // namespace ffn
