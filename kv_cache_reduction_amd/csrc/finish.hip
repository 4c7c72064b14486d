// Slim-Attention decode, finish phase: merge the per-chunk partials of each
// sequence and apply W_KV per head (Slim Attention article, localbendi.com,
// section "K-Cache is All You Need": V = K.W_KV, so head h's output is
// (softmax_h . K) . W_KV[:, h*dh:(h+1)*dh]).
//
// combine_proj: one workgroup per (head h, block of kProjRows rows of W_KV).
//   Its slice W_KV[rows, h*dh:(h+1)*dh] is loaded into registers once and
//   reused for every sequence.  For sequence b with partial slots s (running
//   max m_s in log2 units, normaliser l_s, unnormalised row U_s):
//     m* = max_s m_s,  l* = sum_s 2^(m_s - m*) l_s,
//     u[c] = sum_s 2^(m_s - m*) U_s[h, c] / l*          (log-sum-exp merge)
//     part[pc, b, h, j] = sum_{c in rows} u[c] W_KV[c, h*dh + j]
// proj_reduce: out[b, h, j] = sum_pc part[pc, b, h, j] (fixed order, so the
//   result does not depend on scheduling).
#include "common.hpp"
#include "internal.hpp"

namespace slim {

struct FinishParams {
  const int32_t* lengths;
  const float* U;
  const float* ml;
  const void* W;
  float* part;
  int B, H, d, T_max, nch, npc;
};

template <int DH, bool WBF16>
__global__ void __launch_bounds__(256) combine_proj_kernel(FinishParams p) {
  constexpr int NSUB = (256 / DH < kProjRows) ? 256 / DH : kProjRows;  // row subsets
  constexpr int RPS = kProjRows / NSUB;                                // rows per subset
  extern __shared__ int smem[];
  int* tmp = smem;                                    // [8]
  float* uh = reinterpret_cast<float*>(smem + 8);     // [kProjRows]
  float* red = uh + kProjRows;                        // [NSUB][DH]
  float* wts = red + 256;                             // [nch + 1]
  int* pre = reinterpret_cast<int*>(wts + p.nch + 1); // [B + 1]

  const int tid = threadIdx.x;
  const int h = blockIdx.x, pc = blockIdx.y;
  const int r0 = pc * kProjRows;
  const int nr = min(kProjRows, p.d - r0);
  const int j = tid % DH, sub = tid / DH;
  const bool proj_thread = sub < NSUB;

  float wr[RPS];
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    const int r = sub * RPS + i;
    float v = 0.f;
    if (proj_thread && r < nr) {
      const size_t idx = (size_t)(r0 + r) * p.d + (size_t)h * DH + j;
      if (WBF16) {
        const uint32_t bits = static_cast<const uint16_t*>(p.W)[idx];
        v = __uint_as_float(bits << 16);
      } else {
        v = static_cast<const float*>(p.W)[idx];
      }
    }
    wr[i] = v;
  }

  lengths_prefix(p.lengths, p.B, p.T_max, pre, tmp);
  const int total = pre[p.B];
  const int Ts = total > 0 ? chunk_tokens(total, p.nch) : 1;
  const size_t HD = (size_t)p.H * p.d;
  const size_t nout = (size_t)p.B * p.H * DH;

  for (int b = 0; b < p.B; ++b) {
    const int s0 = pre[b], s1 = pre[b + 1];
    float* dst = p.part + (size_t)pc * nout + ((size_t)b * p.H + h) * DH;
    if (s1 == s0) {
      if (tid < DH) dst[tid] = 0.f;
      continue;
    }
    const int cf = s0 / Ts, cl = (s1 - 1) / Ts;
    const int ns = cl - cf + 1, slot0 = cf + b;

    if (tid < 64) {  // weights of the slots, one wave
      float m = kNegInf;
      for (int i = tid; i < ns; i += 64) m = fmaxf(m, p.ml[(size_t)(slot0 + i) * 2 * p.H + h]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float l = 0.f;
      for (int i = tid; i < ns; i += 64) {
        const float* e = p.ml + (size_t)(slot0 + i) * 2 * p.H;
        l += fast_exp2(e[h] - m) * e[p.H + h];
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
      const float inv = 1.f / l;
      for (int i = tid; i < ns; i += 64)
        wts[i] = fast_exp2(p.ml[(size_t)(slot0 + i) * 2 * p.H + h] - m) * inv;
    }
    __syncthreads();
    if (tid < kProjRows) {
      // rows past d (d not a multiple of kProjRows) are zero: the projection
      // below reads all kProjRows entries
      float acc = 0.f;
      if (tid < nr) {
        const float* u = p.U + (size_t)slot0 * HD + (size_t)h * p.d + r0 + tid;
#pragma unroll 4
        for (int i = 0; i < ns; ++i) acc = fmaf(wts[i], u[(size_t)i * HD], acc);
      }
      uh[tid] = acc;
    }
    __syncthreads();
    if (proj_thread) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < RPS; ++i) acc = fmaf(uh[sub * RPS + i], wr[i], acc);
      red[sub * DH + j] = acc;
    }
    __syncthreads();
    if (tid < DH) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < NSUB; ++k) s += red[k * DH + tid];
      dst[tid] = s;
    }
    // uh, red and wts are rewritten for the next sequence only after the
    // barriers above have been passed by every thread
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) proj_reduce_kernel(const float* __restrict__ part,
                                                          float* __restrict__ out, int npc, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < npc; ++k) s += part[(size_t)k * n + i];
  out[i] = s;
}

template <int DH, bool WBF16>
static hipError_t launch_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  FinishParams p;
  p.lengths = a.lengths;
  p.U = reinterpret_cast<const float*>(a.ws + pl.off_U);
  p.ml = reinterpret_cast<const float*>(a.ws + pl.off_ml);
  p.W = a.W;
  p.part = reinterpret_cast<float*>(a.ws + pl.off_op);
  p.B = a.B;
  p.H = a.H;
  p.d = a.d;
  p.T_max = a.T_max;
  p.nch = pl.nch;
  p.npc = pl.npc;
  const size_t lds = (8 + kProjRows + 256 + (size_t)pl.nch + 1 + (size_t)a.B + 1) * 4;
  hipLaunchKernelGGL((combine_proj_kernel<DH, WBF16>), dim3(a.H, pl.npc), dim3(256), lds, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = a.B * a.H * DH;
  hipLaunchKernelGGL(proj_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                     (const float*)p.part, a.out, pl.npc, n);
  return hipGetLastError();
}

template <int DH>
static hipError_t launch_w(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  return a.w_bf16 ? launch_t<DH, true>(pl, a, s) : launch_t<DH, false>(pl, a, s);
}

hipError_t launch_finish(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  switch (a.dh) {
    case 1: return launch_w<1>(pl, a, s);
    case 2: return launch_w<2>(pl, a, s);
    case 4: return launch_w<4>(pl, a, s);
    case 8: return launch_w<8>(pl, a, s);
    case 16: return launch_w<16>(pl, a, s);
    case 32: return launch_w<32>(pl, a, s);
    case 64: return launch_w<64>(pl, a, s);
    case 128: return launch_w<128>(pl, a, s);
    case 256: return launch_w<256>(pl, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace slim
