// Prompt phase / append: K_cache[b, t0[b] + i, :] = round(X[b, i, :] . W)
// (Slim Attention article, localbendi.com, section "K-Cache is All You
// Need": the prompt phase computes K for every input token in parallel and
// caches it; the generation step appends the new k at its end).
//
// bf16: M = B*n rows, N = d, K = d on v_mfma_f32_32x32x8_bf16, fp32
// accumulation, round-to-nearest-even bf16 output.  Workgroup tile 128x128
// (four waves of 64x64, 2x2 MFMA tiles each; 64x128 with waves of 32x64
// when the 128-row grid would leave compute units idle), 64-deep k blocks.  Both
// operands sit in LDS in their natural row-major layouts: a lane's A
// fragment (4 consecutive k of one row) is one 8-byte read; its B fragment
// (4 consecutive k of one column) is one transpose read (ds_read_b64_tr_b16)
// of four W rows.  The next k block is loaded into registers while the
// current one is multiplied.
// fp32: a plain LDS-tiled VALU GEMM (64x64 tiles, 4x4 outputs per thread).
#include "common.hpp"
#include "internal.hpp"

namespace slim {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_p;

constexpr int kPN = 128, kPK = 64;
constexpr int kAPitch = kPK * 2 + 8;   // bytes per A row in LDS (rows 8 bytes apart in bank order)
constexpr int kBPitch = kPN * 2 + 16;  // bytes per W row in LDS

template <int PM>  // rows per workgroup: 128, or 64 when the 128-row grid would leave compute units idle
__global__ void __launch_bounds__(256) prefill_bf16_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ W,
                                                           uint16_t* __restrict__ Kc, int B, int n,
                                                           int d, int T_max,
                                                           const int32_t* __restrict__ t0) {
  constexpr int MI = PM / 64;  // 32-row MFMA tiles per wave (waves 2 x 2, each PM/2 x 64)
  constexpr int AC = PM / 32;  // 16-byte A chunks per thread and k block
  __shared__ __attribute__((aligned(16))) char As[PM * kAPitch];
  __shared__ __attribute__((aligned(16))) char Bs[kPK * kBPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
  const long long M = (long long)B * n;
  const long long m0 = (long long)blockIdx.y * PM;
  const int n0 = blockIdx.x * kPN;

  // staging: AC chunks of A (row c/8, k 8*(c%8)) and 4 of W (row c/16, col 8*(c%16))
  uint4 sa[AC], sb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i;
      const int ar = c >> 3, ak = (c & 7) * 8;
      sa[i] = make_uint4(0, 0, 0, 0);
      if (m0 + ar < M && k0 + ak < d) sa[i] = *reinterpret_cast<const uint4*>(X + (size_t)(m0 + ar) * d + k0 + ak);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int br = c >> 4, bc = (c & 15) * 8;
      sb[i] = make_uint4(0, 0, 0, 0);
      if (k0 + br < d && n0 + bc < d) sb[i] = *reinterpret_cast<const uint4*>(W + (size_t)(k0 + br) * d + n0 + bc);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i;
      const int ar = c >> 3, ak = (c & 7) * 8;
      char* pa = As + ar * kAPitch + ak * 2;
      *reinterpret_cast<uint2*>(pa) = make_uint2(sa[i].x, sa[i].y);
      *reinterpret_cast<uint2*>(pa + 8) = make_uint2(sa[i].z, sa[i].w);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int br = c >> 4, bc = (c & 15) * 8;
      *reinterpret_cast<uint4*>(Bs + br * kBPitch + bc * 2) = sb[i];
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};

  // A fragment: row wm*PM/2 + 32i + lane%32, k 8*kk + 4*h .. +3
  const char* a_base = As + (wm * (PM / 2) + (lane & 31)) * kAPitch + h * 8;
  // B fragment by transpose read: lane L points at columns
  // 16*((L/16)%2) + 4*(L%4) of W row 4*(L/32) + (L%16)/4 (within a 32-column
  // tile and an 8-row k step); lane l ends with column l%32 of rows 4*(l/32)..+3
  const uint32_t b_base = (uint32_t)(uintptr_t)Bs + (uint32_t)((4 * h + ((lane & 15) >> 2)) * kBPitch +
                                                               (wn * 64 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);

  load(0);
  for (int k0 = 0; k0 < d; k0 += kPK) {
    store();
    __syncthreads();
    if (k0 + kPK < d) load(k0 + kPK);
#pragma unroll
    for (int kk = 0; kk < kPK / 8; ++kk) {
      s16x4 a[MI], b[2];
#pragma unroll
      for (int i = 0; i < MI; ++i) a[i] = *reinterpret_cast<const s16x4*>(a_base + 32 * i * kAPitch + 16 * kk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_p*)(size_t)(b_base + (uint32_t)(8 * kk * kBPitch + 64 * j)));
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= d) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const long long m = m0 + wm * (PM / 2) + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m >= M) continue;
        const int b = (int)(m / n), r = (int)(m - (long long)b * n);
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
  const unsigned gx = (unsigned)((d + kPN - 1) / kPN);
  const long long g128 = (M + 127) / 128;
  if (g128 * gx >= 512 || g128 > 65535) {
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(gx, (unsigned)g128), dim3(256), 0, s,
                       static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W),
                       static_cast<uint16_t*>(Kc), B, n, d, T_max, t0);
  } else {
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(gx, (unsigned)((M + 63) / 64)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W),
                       static_cast<uint16_t*>(Kc), B, n, d, T_max, t0);
  }
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
