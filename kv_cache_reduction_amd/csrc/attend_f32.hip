// Slim-Attention decode, attend phase, fp32 K cache (VALU, fp32 throughout,
// no bf16 rounding of the softmax weights).  Same chunk/piece/slot scheme
// and partial format as the bf16 MFMA path, so the finish phase is shared.
//
// One workgroup of 256 threads per (token chunk, block of 256 columns of K).
// Per token: the row is staged in LDS; thread h < H forms the score of head
// h (log2 units) and updates its running max / normaliser; then thread t
// updates the accumulator column cb*256 + t of every head:
//   U[h, col] = alpha_h * U[h, col] + p_h * K[t, col].
// Every workgroup recomputes the scores of all heads (each needs all d
// columns of the row); this path serves small fp32 problems.
#include "common.hpp"
#include "internal.hpp"

namespace slim {

struct AttendF32Params {
  const float* q;
  const float* K;
  const int32_t* lengths;
  float* U;
  float* ml;
  int B, H, dh, d, T_max, nch, gcf, nslots;
  float qscale;
};

constexpr int kF32MaxHeads = 64;

__global__ void __launch_bounds__(256) attend_f32_kernel(AttendF32Params p) {
  extern __shared__ int smem[];
  int* tmp = smem;                                        // [4]
  float* ap = reinterpret_cast<float*>(smem + 4);         // [2][kF32MaxHeads] alpha, p
  float* row = ap + 2 * kF32MaxHeads;                     // [d]
  int* pre = reinterpret_cast<int*>(row + p.d);           // [B + 1]

  const int tid = threadIdx.x;
  const int c = blockIdx.x / p.gcf, cb = blockIdx.x % p.gcf;
  const int col = cb * 256 + tid;
  const bool col_ok = col < p.d;

  lengths_prefix(p.lengths, p.B, p.T_max, pre, tmp);
  const int total = pre[p.B];
  if (total == 0) return;
  const int Ts = chunk_tokens(total, p.nch);
  const int cbeg = c * Ts;
  if (cbeg >= total) return;
  const int cend = min(total, cbeg + Ts);

  for (int b = seq_of(pre, p.B, cbeg); b < p.B && pre[b] < cend; ++b) {
    const int s0 = pre[b], s1 = pre[b + 1];
    if (s1 == s0) continue;
    const int tb = max(cbeg, s0) - s0, te = min(cend, s1) - s0;
    const int slot = c + b;
    const float* qb = p.q + (size_t)b * p.d;

    float m = kNegInf, l = 0.f;  // head tid (tid < H)
    float acc[kF32MaxHeads];
#pragma unroll
    for (int h = 0; h < kF32MaxHeads; ++h) acc[h] = 0.f;

    for (int t = tb; t < te; ++t) {
      const float* kr = p.K + ((size_t)b * p.T_max + t) * p.d;
      for (int i = tid; i < p.d; i += 256) row[i] = kr[i];
      __syncthreads();
      if (tid < p.H) {
        float s = 0.f;
        for (int j = 0; j < p.dh; ++j) s = fmaf(qb[tid * p.dh + j], row[tid * p.dh + j], s);
        s *= p.qscale;
        const float m_new = fmaxf(m, s);
        const float a = (m_new == kNegInf) ? 1.f : fast_exp2(m - m_new);
        const float e = (m_new == kNegInf) ? 0.f : fast_exp2(s - m_new);
        l = a * l + e;
        m = m_new;
        ap[tid] = a;
        ap[kF32MaxHeads + tid] = e;
      }
      __syncthreads();
      if (col_ok) {
        const float kv = row[col];
#pragma unroll
        for (int h = 0; h < kF32MaxHeads; ++h)
          if (h < p.H) acc[h] = fmaf(ap[kF32MaxHeads + h], kv, ap[h] * acc[h]);
      }
      __syncthreads();
    }
    if (col_ok) {
#pragma unroll
      for (int h = 0; h < kF32MaxHeads; ++h)
        if (h < p.H) p.U[((size_t)h * p.nslots + slot) * p.d + col] = acc[h];
    }
    if (cb == 0 && tid < p.H) {
      p.ml[(size_t)slot * 2 * p.H + tid] = m;
      p.ml[(size_t)slot * 2 * p.H + p.H + tid] = l;
    }
  }
}

hipError_t launch_attend_f32(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  AttendF32Params p;
  p.q = a.q;
  p.K = static_cast<const float*>(a.K);
  p.lengths = a.lengths;
  p.U = reinterpret_cast<float*>(a.ws + pl.off_U);
  p.ml = reinterpret_cast<float*>(a.ws + pl.off_ml);
  p.B = a.B;
  p.H = a.H;
  p.dh = a.dh;
  p.d = a.d;
  p.T_max = a.T_max;
  p.nch = pl.nch;
  p.gcf = pl.gc;
  p.nslots = pl.nslots;
  p.qscale = a.scale * kLog2e;
  const size_t lds = (4 + 2 * kF32MaxHeads + (size_t)a.d + (size_t)a.B + 1) * 4;
  hipLaunchKernelGGL(attend_f32_kernel, dim3(pl.nch * pl.gc), dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace slim
