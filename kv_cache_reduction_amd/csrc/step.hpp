// Host-side plan and launcher of the generation step's projection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace slim {

// [q | k] = x . [W_Q | W_K] as ks row blocks of kr rows of W, each workgroup
// 512 output columns of BG = bg sequences; partial sums [ks][B][2d] float.
struct StepPlan {
  bool mfma;  // bf16 W and B >= 8: the MFMA product (qk_mfma_kernel), else the vector one
  int bg, bgroups, ntile, ks, kr, nb;  // nb: row batches per wave (kr = 8 waves x batch rows x nb)
  size_t off_q;     // [B, d] float: the new queries
  size_t off_part;  // [ks, B, 2d] float
  size_t bytes;     // end of the step's workspace (from `base`)
};

bool make_step_plan(int B, int d, int ncu, bool w_bf16, size_t base, StepPlan* p);
hipError_t launch_step_qk(const StepPlan& p, const float* x, const void* WQ, const void* WK, bool w_bf16,
                          void* Kc, bool k_bf16, const int32_t* lengths, int32_t* lengths_next, int B,
                          int d, int T_max, char* ws, hipStream_t s);

}  // namespace slim
