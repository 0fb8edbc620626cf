// Launchers shared between the kernel translation units and the C-ABI layer (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ffn {

// Arguments of the batch-1 main kernel (one token).
struct MainArgs {
  const void* w_up;
  const void* w_gate;
  const void* w_dn;
  const void* s_up;
  const void* s_gate;
  const void* s_dn;
  const float* b_up;
  const float* b_gate;
  const void* p2;
  const float* c2;
  const void* x;          // one token, x_dtype (fp16 for int4 rows)
  const float* z;         // predictor stage-1 output [rank]
  const unsigned char* mask;  // caller's set [ffn] or nullptr
  float* scores;          // [ffn] or nullptr
  int* chunk_cnt;         // [n_chunks]
  int* chunk_list;        // [ffn]: chunk c's ascending active list at c*nc
  float* part;            // [n_chunks][d]
  int d, ffn, rank, nc, act, has_gate, p_f16;
  float thr;
};

hipError_t launch_pred_z(int p_f16, int cpl, const void* p1, const float* c1, const void* x,
                         float* z, int d, int rank, hipStream_t st);
size_t main_lds_bytes(int d, int rank, int nc);
int main_waves(int cpl);
hipError_t launch_main(int wk, int cpl, const MainArgs& a, int n_chunks, hipStream_t st,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_reduce(const float* part, int n_chunks, const float* b_down, float* y, int d,
                         hipStream_t st);
hipError_t launch_write_idx(const int* ccnt, const int* clist, int n_chunks, int nc, int* idx,
                            int* cnt, hipStream_t st);

}  // namespace ffn
