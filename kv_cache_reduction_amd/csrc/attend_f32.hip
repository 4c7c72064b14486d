// Slim-Attention decode, attend phase, fp32 K cache (VALU, fp32 throughout,
// no bf16 rounding of the softmax weights).  Same chunk/piece/slot scheme
// and partial format as the bf16 MFMA path, so the finish phase is shared.
//
// One workgroup of 256 threads per (token chunk, block of 256 columns of K).
// Rows are staged in LDS RB at a time (one load round per block, not per
// token).  Per block: thread (r, h) forms the score of row r for head h (log2
// units); thread h < H then walks the block's rows in order, updating its
// running max and normaliser and recording (alpha, p) per row; then thread t
// updates the accumulator column cb*256 + t of every head, row by row:
//   U[h, col] = alpha_h * U[h, col] + p_h * K[t, col].
// The per-row arithmetic and its order are those of a token-at-a-time loop.
// Every workgroup recomputes the scores of all heads (each needs all d
// columns of the row); this path serves small fp32 problems.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace slim {

struct AttendF32Params {
  const float* q;
  const float* K;
  const int32_t* lengths;
  float* U;
  float* ml;
  uint32_t* status;  // cleared here; the finish sets it if a piece is marked failed
  int B, H, dh, d, T_max, nch, gcf, nslots, rb;
  float qscale;
};

constexpr int kF32MaxHeads = 64;

// MAXH >= H bounds the per-thread head loops at compile time, so that the
// accumulators stay in registers and a small H does not walk (and branch
// over) all kF32MaxHeads of them.
template <int MAXH>
__global__ void __launch_bounds__(256) attend_f32_kernel(AttendF32Params p) {
  extern __shared__ int smem[];
  const int RB = p.rb;
  int* tmp = smem;                                        // [4]
  float* qs = reinterpret_cast<float*>(smem + 4);         // [d] the piece's query
  float* rows = qs + p.d;                                 // [RB][d]
  float* sc = rows + (size_t)RB * p.d;                    // [RB][H] scores, then weights p
  float* al = sc + RB * p.H;                              // [RB][H] rescale factors
  int* pre = reinterpret_cast<int*>(al + RB * p.H);       // [B + 1]

  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid == 0) *p.status = 0u;
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
    for (int i = tid; i < p.d; i += 256) qs[i] = p.q[(size_t)b * p.d + i];

    float m = kNegInf, l = 0.f;  // head tid (tid < H)
    float acc[MAXH];
#pragma unroll
    for (int h = 0; h < MAXH; ++h) acc[h] = 0.f;

    for (int t0 = tb; t0 < te; t0 += RB) {
      const int nr = min(RB, te - t0);
      const float* kr = p.K + ((size_t)b * p.T_max + t0) * p.d;
      for (int i = tid; i < nr * p.d; i += 256) rows[i] = kr[i];
      __syncthreads();
      for (int i = tid; i < nr * p.H; i += 256) {
        const int r = i / p.H, h = i % p.H;
        float s = 0.f;
        for (int j = 0; j < p.dh; ++j) s = fmaf(qs[h * p.dh + j], rows[(size_t)r * p.d + h * p.dh + j], s);
        sc[i] = s * p.qscale;
      }
      __syncthreads();
      if (tid < p.H) {
        for (int r = 0; r < nr; ++r) {
          const float s = sc[r * p.H + tid];
          const float m_new = fmaxf(m, s);
          const float a = (m_new == kNegInf) ? 1.f : fast_exp2(m - m_new);
          const float e = (m_new == kNegInf) ? 0.f : fast_exp2(s - m_new);
          l = a * l + e;
          m = m_new;
          al[r * p.H + tid] = a;
          sc[r * p.H + tid] = e;
        }
      }
      __syncthreads();
      if (col_ok) {
        for (int r = 0; r < nr; ++r) {
          const float kv = rows[(size_t)r * p.d + col];
#pragma unroll
          for (int h = 0; h < MAXH; ++h)
            if (h < p.H) acc[h] = fmaf(sc[r * p.H + h], kv, al[r * p.H + h] * acc[h]);
        }
      }
      __syncthreads();
    }
    if (col_ok) {
#pragma unroll
      for (int h = 0; h < MAXH; ++h)
        if (h < p.H) p.U[((size_t)h * p.nslots + slot) * p.d + col] = acc[h];
    }
    if (cb == 0 && tid < p.H) {
      p.ml[(size_t)slot * 2 * p.H + tid] = m;
      p.ml[(size_t)slot * 2 * p.H + p.H + tid] = l;
    }
  }
}

template <int MAXH>
static hipError_t launch_heads(const AttendF32Params& p, const DecodePlan& pl, size_t lds, hipStream_t s) {
  static std::atomic<int> granted[kMaxDevices];
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(attend_f32_kernel<MAXH>), lds, granted);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_f32_kernel<MAXH>, dim3(pl.nch * pl.gc), dim3(256), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_attend_f32(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  AttendF32Params p;
  p.q = a.q;
  p.K = static_cast<const float*>(a.K);
  p.lengths = a.lengths;
  p.U = reinterpret_cast<float*>(a.ws + pl.off_U);
  p.ml = reinterpret_cast<float*>(a.ws + pl.off_ml);
  p.status = a.status;
  p.B = a.B;
  p.H = a.H;
  p.dh = a.dh;
  p.d = a.d;
  p.T_max = a.T_max;
  p.nch = pl.nch;
  p.gcf = pl.gc;
  p.nslots = pl.nslots;
  p.qscale = a.scale * kLog2e;
  // rows per LDS block: at most 64, 32 KB of rows and 2048 (row, head) pairs
  int rb = 32768 / (4 * a.d);
  if (rb > 64) rb = 64;
  if (rb > 2048 / a.H) rb = 2048 / a.H;
  if (rb < 1) rb = 1;
  p.rb = rb;
  const size_t lds = (4 + (size_t)a.d + (size_t)rb * a.d + 2 * (size_t)rb * a.H + (size_t)a.B + 1) * 4;
  if (a.H <= 4) return launch_heads<4>(p, pl, lds, s);
  if (a.H <= 8) return launch_heads<8>(p, pl, lds, s);
  if (a.H <= 16) return launch_heads<16>(p, pl, lds, s);
  if (a.H <= 32) return launch_heads<32>(p, pl, lds, s);
  if (a.H <= kF32MaxHeads) return launch_heads<kF32MaxHeads>(p, pl, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace slim
