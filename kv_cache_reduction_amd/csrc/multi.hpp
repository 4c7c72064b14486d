// Host-side plan and launcher of the many-queries-over-one-context path.
#pragma once

#include "internal.hpp"

namespace slim {

struct MultiPlan {
  int method;      // 1: V = K.W_KV formed, then softmax . V; 2: softmax . K, then W_KV
  int qw;          // waves (32 queries each) per workgroup
  int nsplit, Ts;  // context splits of Ts rows
  size_t off_v;    // option 1: [T, d] bf16 values
  DecodePlan fin;  // partial rows (option 2; option 1 with splits) and the merge / projection
  size_t bytes;
};

bool make_multi_plan(int n, int H, int dh, int T, int method, bool w_bf16, int ncu, MultiPlan* p);
hipError_t launch_multi(const MultiPlan& pl, const float* Q, const void* K, const int32_t* limits,
                        const void* W, bool w_bf16, float* out, int n, int H, int dh, int T, float scale,
                        char* ws, hipStream_t s);

// merge of a fixed number of slots per row (slot = row * ns + split), then
// the W_KV projection; the decode finish with its slot ranges replaced
hipError_t launch_finish_fixed(const DecodePlan& p, const DecodeArgs& a, int ns, hipStream_t s);

}  // namespace slim
