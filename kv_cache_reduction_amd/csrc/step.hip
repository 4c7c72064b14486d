// Generation step, projection part: the new token's query q = x.W_Q and key
// k = x.W_K for every sequence, with k rounded to the cache format and
// written at row len_b (Slim Attention article, localbendi.com, section
// "K-Cache is All You Need", generation phase: the step first computes its
// query, attends against the K rows cached at earlier steps, and at the end
// adds its own k to the K cache for the next step).  The attention itself is
// the decode path; slim_step enqueues it between these kernels' output and
// the caller's next step.
//
// qk_proj   [q | k] = x . [W_Q | W_K] split over the reduction dimension:
//           grid (ceil(2d/512), ks, ceil(B/BG)), 512 threads.  A workgroup
//           owns 512 output columns (8 per lane, one 16-byte row segment of
//           bf16 W per load) and KR rows of W; its 8 waves take every 8th row
//           and meet in LDS at the end.  x[b, rows] for BG sequences sits in
//           LDS, read as broadcasts.  W is read once per BG sequences.
//           part[ks][B][2d] float.
// qk_finish sums the ks partials of every output in a fixed order; q goes to
//           the workspace in float32, k to K_cache[b, len_b, :] rounded to
//           the cache format (round to nearest even for bf16) when
//           len_b < T_max, and lengths_next[b] = len_b + 1 (T_max when full).
#include "common.hpp"
#include "step.hpp"

namespace slim {

constexpr int kQkCols = 512;  // output columns per workgroup (64 lanes x 8)
constexpr int kQkWaves = 8;

template <bool WBF16, int BG>
__global__ void __launch_bounds__(512) qk_proj_kernel(const float* __restrict__ x,
                                                      const void* __restrict__ WQ,
                                                      const void* __restrict__ WK,
                                                      float* __restrict__ part, int B, int d, int KR) {
  extern __shared__ __attribute__((aligned(16))) float qk_smem[];
  constexpr int CB = BG < 4 ? BG : 4;  // sequences per round of the cross-wave sum
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = blockIdx.y * KR, nk = min(KR, d - k0);
  const int b0 = blockIdx.z * BG;

  float* xs = qk_smem;  // [KR][BG]
  for (int i = tid; i < nk * BG; i += 512) {
    const int k = i / BG, bb = i - k * BG;
    xs[i] = b0 + bb < B ? x[(size_t)(b0 + bb) * d + k0 + k] : 0.f;
  }
  __syncthreads();

  const int col = blockIdx.x * kQkCols + lane * 8;  // column of [q | k]
  const bool live = col < 2 * d;
  const int wc = col < d ? col : col - d;
  const void* W = col < d ? WQ : WK;

  float acc[BG][8];
#pragma unroll
  for (int i = 0; i < BG; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  auto load_row = [&](int k, float (&w)[8]) {
    const size_t off = (size_t)(k0 + k) * d + wc;
    if constexpr (WBF16) {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + off);
      w[0] = bf_lo(v.x); w[1] = bf_hi(v.x); w[2] = bf_lo(v.y); w[3] = bf_hi(v.y);
      w[4] = bf_lo(v.z); w[5] = bf_hi(v.z); w[6] = bf_lo(v.w); w[7] = bf_hi(v.w);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + off);
      const float4 c = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + off + 4);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = c.x; w[5] = c.y; w[6] = c.z; w[7] = c.w;
    }
  };
  auto fma_row = [&](int k, const float (&w)[8]) {
    float xv[BG];
    if constexpr (BG % 4 == 0) {
#pragma unroll
      for (int i = 0; i < BG; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(xs + k * BG + i);
        xv[i] = v.x; xv[i + 1] = v.y; xv[i + 2] = v.z; xv[i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < BG; ++i) xv[i] = xs[k * BG + i];
    }
#pragma unroll
    for (int i = 0; i < BG; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xv[i], w[j], acc[i][j]);
  };

  if (live) {
    constexpr int U = BG >= 16 ? 4 : 8;  // rows in flight per lane
    int k = wave;
    for (; k + kQkWaves * (U - 1) < nk; k += kQkWaves * U) {
      float w[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) load_row(k + kQkWaves * u, w[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) fma_row(k + kQkWaves * u, w[u]);
    }
    for (; k < nk; k += kQkWaves) {
      float w[8];
      load_row(k, w);
      fma_row(k, w);
    }
  }
  __syncthreads();  // xs is dead; the space becomes the cross-wave buffer

  float* red = qk_smem;  // [kQkWaves][CB][512]
  const int n2 = 2 * d;
#pragma unroll
  for (int cb = 0; cb < BG; cb += CB) {
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      float4* dst = reinterpret_cast<float4*>(red + (wave * CB + i) * kQkCols + lane * 8);
      dst[0] = make_float4(acc[cb + i][0], acc[cb + i][1], acc[cb + i][2], acc[cb + i][3]);
      dst[1] = make_float4(acc[cb + i][4], acc[cb + i][5], acc[cb + i][6], acc[cb + i][7]);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < CB; ++r) {
      const int o = tid + 512 * r;  // < CB * 512
      const int i = o / kQkCols, c = o - i * kQkCols;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kQkWaves; ++w) s += red[(w * CB + i) * kQkCols + c];
      const int b = b0 + cb + i, oc = blockIdx.x * kQkCols + c;
      if (b < B && oc < n2) part[((size_t)blockIdx.y * B + b) * n2 + oc] = s;
    }
    __syncthreads();
  }
}

template <bool KBF16>
__global__ void __launch_bounds__(256) qk_finish_kernel(const float* __restrict__ part, int ks,
                                                        float* __restrict__ q, void* __restrict__ Kc,
                                                        const int32_t* __restrict__ lengths,
                                                        int32_t* __restrict__ lengths_next, int B, int d,
                                                        int T_max) {
  const int n2 = 2 * d;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)B * n2) return;
  const int b = (int)(i / n2), c = (int)(i - (long long)b * n2);
  float s = 0.f;
  for (int k = 0; k < ks; ++k) s += part[(size_t)k * B * n2 + i];
  int len = lengths[b];
  len = len < 0 ? 0 : (len > T_max ? T_max : len);
  if (c < d) {
    q[(size_t)b * d + c] = s;
  } else if (len < T_max) {
    const size_t off = ((size_t)b * T_max + len) * d + (c - d);
    if constexpr (KBF16) static_cast<uint16_t*>(Kc)[off] = (uint16_t)f32_to_bf16_rne(s);
    else static_cast<float*>(Kc)[off] = s;
  }
  if (c == 0) lengths_next[b] = len < T_max ? len + 1 : T_max;
}

bool make_step_plan(int B, int d, int ncu, size_t base, StepPlan* p) {
  if (B <= 0 || d <= 0 || d % 8 != 0) return false;
  p->bg = B >= 16 ? 16 : (B > 8 ? 16 : (B > 4 ? 8 : (B > 2 ? 4 : B)));
  const int ntile = (2 * d + kQkCols - 1) / kQkCols;
  const int bgroups = (B + p->bg - 1) / p->bg;
  long long ks = ((long long)ncu + (long long)ntile * bgroups - 1) / ((long long)ntile * bgroups);
  const int kmax = (d + 63) / 64;  // at least 64 rows (8 per wave) per workgroup
  if (ks > kmax) ks = kmax;
  if (ks < 1) ks = 1;
  int kr = (int)((d + ks - 1) / ks);
  kr = (kr + 7) / 8 * 8;
  const int kr_cap = 16384 / p->bg;  // x rows staged in LDS: at most 64 KB
  if (kr > kr_cap) kr = kr_cap;
  p->kr = kr;
  p->ks = (d + kr - 1) / kr;
  p->ntile = ntile;
  p->bgroups = bgroups;
  size_t off = (base + 255) & ~(size_t)255;
  p->off_q = off;
  off += ((size_t)B * d * sizeof(float) + 255) & ~(size_t)255;
  p->off_part = off;
  off += ((size_t)p->ks * B * 2 * d * sizeof(float) + 255) & ~(size_t)255;
  p->bytes = off;
  return true;
}

template <bool WBF16, int BG>
static hipError_t launch_proj(const StepPlan& p, const float* x, const void* WQ, const void* WK,
                              float* part, int B, int d, hipStream_t s) {
  constexpr int CB = BG < 4 ? BG : 4;
  const size_t xs = (size_t)p.kr * BG * sizeof(float);
  const size_t red = (size_t)kQkWaves * CB * kQkCols * sizeof(float);
  hipLaunchKernelGGL((qk_proj_kernel<WBF16, BG>), dim3(p.ntile, p.ks, p.bgroups), dim3(512),
                     xs > red ? xs : red, s, x, WQ, WK, part, B, d, p.kr);
  return hipGetLastError();
}

template <bool WBF16>
static hipError_t launch_proj_bg(const StepPlan& p, const float* x, const void* WQ, const void* WK,
                                 float* part, int B, int d, hipStream_t s) {
  switch (p.bg) {
    case 1: return launch_proj<WBF16, 1>(p, x, WQ, WK, part, B, d, s);
    case 2: return launch_proj<WBF16, 2>(p, x, WQ, WK, part, B, d, s);
    case 4: return launch_proj<WBF16, 4>(p, x, WQ, WK, part, B, d, s);
    case 8: return launch_proj<WBF16, 8>(p, x, WQ, WK, part, B, d, s);
    case 16: return launch_proj<WBF16, 16>(p, x, WQ, WK, part, B, d, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_step_qk(const StepPlan& p, const float* x, const void* WQ, const void* WK, bool w_bf16,
                          void* Kc, bool k_bf16, const int32_t* lengths, int32_t* lengths_next, int B,
                          int d, int T_max, char* ws, hipStream_t s) {
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  float* q = reinterpret_cast<float*>(ws + p.off_q);
  hipError_t e = w_bf16 ? launch_proj_bg<true>(p, x, WQ, WK, part, B, d, s)
                        : launch_proj_bg<false>(p, x, WQ, WK, part, B, d, s);
  if (e != hipSuccess) return e;
  const long long n = (long long)B * 2 * d;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (k_bf16)
    hipLaunchKernelGGL(qk_finish_kernel<true>, dim3(grid), dim3(256), 0, s, (const float*)part, p.ks, q, Kc,
                       lengths, lengths_next, B, d, T_max);
  else
    hipLaunchKernelGGL(qk_finish_kernel<false>, dim3(grid), dim3(256), 0, s, (const float*)part, p.ks, q,
                       Kc, lengths, lengths_next, B, d, T_max);
  return hipGetLastError();
}

}  // namespace slim
