// Slim-Attention decode, finish phase: merge the per-chunk partials of each
// sequence and apply W_KV per head (Slim Attention article, localbendi.com,
// section "K-Cache is All You Need": V = K.W_KV, so head h's output is
// (softmax_h . K) . W_KV[:, h*dh:(h+1)*dh]).
//
// Partials (written by the attend phase) are laid out U[h][slot][d] and
// ml[slot][2][H] (running max in log2 units, normaliser).
//
// combine  grid (H, d/512, B): for sequence b with slots s (log-sum-exp merge)
//            m* = max_s m_s,  l* = sum_s 2^(m_s - m*) l_s,
//            u[b, h, c] = sum_s 2^(m_s - m*) U_s[h, c] / l*
//          Each thread sums one float4 of columns over a strided subset of the
//          slots; the subsets meet in LDS.
// project  grid (H, d/R, ceil(B/8)) with R = proj_rows(dh): the workgroup
//          holds W_KV[R rows, h-slice] in registers (16-byte loads) and forms
//          the partial products of up to 8 sequences:
//            part[rb, b, h, j] = sum_{c in rows} u[b, h, c] W_KV[c, h*dh + j]
// reduce   out[b, h, j] = sum_rb part[rb, b, h, j] in a fixed order, so the
//          result does not depend on scheduling.
#include "common.hpp"
#include "internal.hpp"

namespace slim {

constexpr int kCombineCols = 512;  // columns per combine workgroup (128 threads x float4)
constexpr int kSeqPerProj = 8;     // sequences per projection workgroup

__global__ void __launch_bounds__(256) combine_kernel(const int32_t* __restrict__ lengths,
                                                      const float* __restrict__ U,
                                                      const float* __restrict__ ml,
                                                      float* __restrict__ u_out, int B, int H, int d,
                                                      int T_max, int nch, int nslots) {
  extern __shared__ int smem[];
  int* tmp = smem;                                   // [8]
  float* red = reinterpret_cast<float*>(smem + 8);   // [2][kCombineCols]
  float* wts = red + 2 * kCombineCols;               // [nch + 1]
  int* pre = reinterpret_cast<int*>(wts + nch + 1);  // [B + 1]
  const int tid = threadIdx.x;
  const int h = blockIdx.x, c0 = blockIdx.y * kCombineCols, b = blockIdx.z;

  lengths_prefix(lengths, B, T_max, pre, tmp);
  const int s0 = pre[b], s1 = pre[b + 1];
  float* dst = u_out + ((size_t)b * H + h) * d + c0;
  const int ncols = min(kCombineCols, d - c0);
  if (s1 == s0) {
    for (int i = tid; i < ncols; i += blockDim.x) dst[i] = 0.f;
    return;
  }
  const int Ts = chunk_tokens(pre[B], nch);
  const int cf = s0 / Ts, cl = (s1 - 1) / Ts, ns = cl - cf + 1, slot0 = cf + b;

  if (tid < 64) {  // slot weights 2^(m_s - m*) / l*, one wave
    float m = kNegInf;
    for (int i = tid; i < ns; i += 64) m = fmaxf(m, ml[(size_t)(slot0 + i) * 2 * H + h]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float l = 0.f;
    for (int i = tid; i < ns; i += 64) {
      const float* e = ml + (size_t)(slot0 + i) * 2 * H;
      const float w = fast_exp2(e[h] - m);
      wts[i] = w;
      l += w * e[H + h];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    const float inv = 1.f / l;
    for (int i = tid; i < ns; i += 64) wts[i] *= inv;
  }
  __syncthreads();

  const int j4 = tid & 127, g = tid >> 7;  // 128 float4 columns x 2 slot subsets
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* src = U + ((size_t)h * nslots + slot0) * d + c0 + 4 * j4;
  if ((d & 3) == 0 && 4 * j4 < ncols) {
#pragma unroll 16
    for (int i = g; i < ns; i += 2) {
      const float4 v = *reinterpret_cast<const float4*>(src + (size_t)i * d);
      const float w = wts[i];
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
  } else if (4 * j4 < ncols) {  // rows not 16-byte aligned (d % 4 != 0)
    for (int i = g; i < ns; i += 2) {
      const float* v = src + (size_t)i * d;
      const float w = wts[i];
      acc.x = fmaf(w, v[0], acc.x);
      if (4 * j4 + 1 < ncols) acc.y = fmaf(w, v[1], acc.y);
      if (4 * j4 + 2 < ncols) acc.z = fmaf(w, v[2], acc.z);
      if (4 * j4 + 3 < ncols) acc.w = fmaf(w, v[3], acc.w);
    }
  }
  float* r = red + g * kCombineCols + 4 * j4;
  r[0] = acc.x;
  r[1] = acc.y;
  r[2] = acc.z;
  r[3] = acc.w;
  __syncthreads();
  for (int i = tid; i < ncols; i += blockDim.x) dst[i] = red[i] + red[kCombineCols + i];
}

template <int DH, bool WBF16>
__global__ void __launch_bounds__(256) project_kernel(const float* __restrict__ u,
                                                      const void* __restrict__ W,
                                                      float* __restrict__ part, int B, int H, int d) {
  // thread t: JW output columns (group jq = t % JQ) over the rows of subset t / JQ
  constexpr int PR = proj_rows(DH);
  constexpr int JQ = DH >= 8 ? DH / 8 : 1;  // column groups per head
  constexpr int JW = DH >= 8 ? 8 : DH;      // columns per group
  constexpr int NRS = 256 / JQ;             // row subsets
  constexpr int RPT = PR / NRS;             // rows per thread
  static_assert(RPT >= 1 && RPT * NRS == PR, "row split");
  __shared__ float red[NRS * DH];
  __shared__ float us[kSeqPerProj][PR];
  const int tid = threadIdx.x;
  const int h = blockIdx.x, r0 = blockIdx.y * PR, b0 = blockIdx.z * kSeqPerProj;
  const int nr = min(PR, d - r0), nb = min(kSeqPerProj, B - b0);
  const int jq = tid % JQ, rs = tid / JQ;

  float w[RPT][JW];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rs * RPT + i;
    const size_t base = (size_t)(r0 + r) * d + (size_t)h * DH + jq * JW;
    if (r < nr) {
      if constexpr (WBF16 && JW == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + base);
        w[i][0] = bf_lo(v.x); w[i][1] = bf_hi(v.x); w[i][2] = bf_lo(v.y); w[i][3] = bf_hi(v.y);
        w[i][4] = bf_lo(v.z); w[i][5] = bf_hi(v.z); w[i][6] = bf_lo(v.w); w[i][7] = bf_hi(v.w);
      } else {
#pragma unroll
        for (int k = 0; k < JW; ++k) {
          if (WBF16) w[i][k] = __uint_as_float((uint32_t)static_cast<const uint16_t*>(W)[base + k] << 16);
          else w[i][k] = static_cast<const float*>(W)[base + k];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < JW; ++k) w[i][k] = 0.f;
    }
  }
  for (int i = tid; i < nb * PR; i += 256) {
    const int bb = i / PR, r = i % PR;
    us[bb][r] = r < nr ? u[((size_t)(b0 + bb) * H + h) * d + r0 + r] : 0.f;
  }
  __syncthreads();
  const size_t nout = (size_t)B * H * DH;
  for (int bb = 0; bb < nb; ++bb) {
    float acc[JW];
#pragma unroll
    for (int k = 0; k < JW; ++k) acc[k] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float x = us[bb][rs * RPT + i];
#pragma unroll
      for (int k = 0; k < JW; ++k) acc[k] = fmaf(x, w[i][k], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < JW; ++k) red[rs * DH + jq * JW + k] = acc[k];
    __syncthreads();
    if (tid < DH) {
      float s = 0.f;
#pragma unroll 8
      for (int k = 0; k < NRS; ++k) s += red[k * DH + tid];
      part[(size_t)blockIdx.y * nout + ((size_t)(b0 + bb) * H + h) * DH + tid] = s;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) proj_reduce_kernel(const float* __restrict__ part,
                                                          float* __restrict__ out, int npc, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
#pragma unroll 8
  for (int k = 0; k < npc; ++k) s += part[(size_t)k * n + i];
  out[i] = s;
}

template <int DH, bool WBF16>
static hipError_t launch_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  const float* U = reinterpret_cast<const float*>(a.ws + pl.off_U);
  const float* ml = reinterpret_cast<const float*>(a.ws + pl.off_ml);
  float* uo = reinterpret_cast<float*>(a.ws + pl.off_u);
  float* part = reinterpret_cast<float*>(a.ws + pl.off_op);
  const size_t lds = (8 + 2 * kCombineCols + (size_t)pl.nch + 1 + (size_t)a.B + 1) * 4;
  hipLaunchKernelGGL(combine_kernel, dim3(a.H, (a.d + kCombineCols - 1) / kCombineCols, a.B), dim3(256),
                     lds, s, a.lengths, U, ml, uo, a.B, a.H, a.d, a.T_max, pl.nch, pl.nslots);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((project_kernel<DH, WBF16>),
                     dim3(a.H, pl.npc, (a.B + kSeqPerProj - 1) / kSeqPerProj), dim3(256), 0, s,
                     (const float*)uo, a.W, part, a.B, a.H, a.d);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = a.B * a.H * DH;
  hipLaunchKernelGGL(proj_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, (const float*)part,
                     a.out, pl.npc, n);
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
