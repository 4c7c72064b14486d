// Prompt phase / append: K_cache[b, t0[b] + i, :] = round(X[b, i, :] . W)
// (Slim Attention article, localbendi.com, section "K-Cache is All You
// Need": the prompt phase computes K for every input token in parallel and
// caches it; the generation step appends the new k at its end).
//
// bf16: M = B*n rows, N = d, K = d on v_mfma_f32_32x32x8_bf16, fp32
// accumulation, round-to-nearest-even bf16 output.  Workgroup tile 128x128
// (four waves of 64x64, 2x2 MFMA tiles each), K-step 32 through LDS.  A is
// stored row-major [m][k]; B is stored transposed [n][k] so both MFMA
// operands are one 8-byte LDS read per lane.
// fp32: a plain LDS-tiled VALU GEMM (64x64 tiles, 4x4 outputs per thread).
#include "common.hpp"
#include "internal.hpp"

namespace slim {

constexpr int kPM = 128, kPN = 128, kPK = 32, kPKpad = kPK + 4;

__global__ void __launch_bounds__(256) prefill_bf16_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ W,
                                                           uint16_t* __restrict__ Kc, int B, int n,
                                                           int d, int T_max,
                                                           const int32_t* __restrict__ t0) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kPM * kPKpad];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kPN * kPKpad];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = B * n;
  const int m0 = blockIdx.y * kPM, n0 = blockIdx.x * kPN;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};

  for (int k0 = 0; k0 < d; k0 += kPK) {
    // A tile: 128 rows x 32 k, 16-byte chunks
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int ch = tid + r * 256;
      const int row = ch >> 2, kc = (ch & 3) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + row < M && k0 + kc < d) v = *reinterpret_cast<const uint4*>(X + (size_t)(m0 + row) * d + k0 + kc);
      uint2* dst = reinterpret_cast<uint2*>(As + row * kPKpad + kc);
      dst[0] = make_uint2(v.x, v.y);
      dst[1] = make_uint2(v.z, v.w);
    }
    // B tile: 32 k x 128 n from W[k][n], stored transposed [n][k]
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int ch = tid + r * 256;
      const int kr = ch >> 4, nc = (ch & 15) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k0 + kr < d && n0 + nc < d) v = *reinterpret_cast<const uint4*>(W + (size_t)(k0 + kr) * d + n0 + nc);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        Bs[(nc + i) * kPKpad + kr] = (uint16_t)((i & 1) ? (w4[i >> 1] >> 16) : (w4[i >> 1] & 0xffffu));
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kPK; kk += 8) {
      const int kq = kk + 4 * (lane >> 5);
      s16x4 a[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const s16x4*>(As + row * kPKpad + kq);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (lane & 31);
        bv[j] = *reinterpret_cast<const s16x4*>(Bs + col * kPKpad + kq);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= d) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m >= M) continue;
        const int b = m / n, r = m - b * n;
        const int t = (t0 ? t0[b] : 0) + r;
        if (t < 0 || t >= T_max) continue;
        Kc[((size_t)b * T_max + t) * d + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
      }
    }
}

__global__ void __launch_bounds__(256) prefill_f32_kernel(const float* __restrict__ X,
                                                          const float* __restrict__ W,
                                                          float* __restrict__ Kc, int B, int n, int d,
                                                          int T_max, const int32_t* __restrict__ t0) {
  __shared__ float As[64][17];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int M = B * n;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      const int r = i / 16, k = i % 16;
      As[r][k] = (m0 + r < M && k0 + k < d) ? X[(size_t)(m0 + r) * d + k0 + k] : 0.f;
      const int kr = i / 64, c = i % 64;
      Bs[kr][c] = (k0 + kr < d && n0 + c < d) ? W[(size_t)(k0 + kr) * d + n0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[ty * 4 + i][k], Bs[k][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    const int b = m / n, r = m - b * n;
    const int t = (t0 ? t0[b] : 0) + r;
    if (t < 0 || t >= T_max) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col < d) Kc[((size_t)b * T_max + t) * d + col] = acc[i][j];
    }
  }
}

hipError_t launch_prefill_bf16(const void* X, const void* W, void* Kc, int B, int n, int d,
                               int T_max, const int32_t* t0, hipStream_t s) {
  const long long M = (long long)B * n;
  dim3 grid((d + kPN - 1) / kPN, (unsigned)((M + kPM - 1) / kPM));
  hipLaunchKernelGGL(prefill_bf16_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(X),
                     static_cast<const uint16_t*>(W), static_cast<uint16_t*>(Kc), B, n, d, T_max, t0);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const void* X, const void* W, void* Kc, int B, int n, int d,
                              int T_max, const int32_t* t0, hipStream_t s) {
  const long long M = (long long)B * n;
  dim3 grid((d + 63) / 64, (unsigned)((M + 63) / 64));
  hipLaunchKernelGGL(prefill_f32_kernel, grid, dim3(256), 0, s, static_cast<const float*>(X),
                     static_cast<const float*>(W), static_cast<float*>(Kc), B, n, d, T_max, t0);
  return hipGetLastError();
}

}  // namespace slim
