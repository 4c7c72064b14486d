// Prompt phase / append: K_cache[b, t0[b] + i, :] = round(X[b, i, :] . W)
// (Slim Attention article, localbendi.com, section "K-Cache is All You
// Need": the prompt phase computes K for every input token in parallel and
// caches it; the generation step appends the new k at its end).
//
// bf16: M = B*n rows, N = d, K = d on v_mfma_f32_32x32x16_bf16, fp32
// accumulation, round-to-nearest-even bf16 output.  Workgroup tile 128x128
// (four waves of 64x64, 2x2 MFMA tiles each; 64x128 with waves of 32x64
// when the 128-row grid would leave compute units idle, and 64x64 with
// waves of 32x32 when even that grid is below two workgroups per compute
// unit), 64-deep k blocks.  Both
// operands sit in LDS in their natural row-major layouts: a lane's A
// fragment (8 consecutive k of one row) is one 16-byte read; its B fragment
// (the same 8 k of one column) is two transpose reads (ds_read_b64_tr_b16)
// of four W rows each.  k blocks are staged through registers three deep
// (two for the 128-row tile) into two LDS buffers, one barrier per block;
// every load is issued unconditionally, so that the compiler's wait counts
// let the younger blocks stay in flight.
// fp32: a plain LDS-tiled VALU GEMM (64x64 tiles, 4x4 outputs per thread).
#include "common.hpp"
#include "mfma16.hpp"
#include "internal.hpp"

namespace slim {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_p;

constexpr int kPK = 64;
constexpr int kAPitch = kPK * 2 + 16;  // bytes per A row in LDS (16-byte reads of 8 rows on distinct banks)

// PM x PN tiles: 128 x 128; 64 x 128 when the 128-row grid would leave
// compute units idle; 64 x 64 when even that grid is below two workgroups
// per compute unit (small products: twice the workgroups to hide latency)
template <int PM, int PN>
__global__ void __launch_bounds__(256) prefill_bf16_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ W,
                                                           uint16_t* __restrict__ Kc, int B, int n,
                                                           int d, int T_max,
                                                           const int32_t* __restrict__ t0) {
  constexpr int MI = PM / 64;  // 32-row MFMA tiles per wave (waves 2 x 2, each PM/2 x PN/2)
  constexpr int NJ = PN / 64;  // 32-column MFMA tiles per wave
  constexpr int BPITCH = PN * 2 + 16;  // bytes per W row in LDS
  constexpr int BC = kPK * PN / 8 / 256;  // 16-byte W chunks per thread and k block
  constexpr int CPR = PN / 8;             // 16-byte chunks per W row
  // k blocks in flight in registers: three for the 64-row tile, two for the
  // 128-row one (whose accumulators would otherwise leave room for one wave
  // per SIMD only)
  constexpr int kPStages = PM == 64 ? 3 : 2;
  constexpr int AC = PM / 32;  // 16-byte A chunks per thread and k block
  constexpr int ABYTES = PM * kAPitch, BUF = ABYTES + kPK * BPITCH;
  __shared__ __attribute__((aligned(16))) char lds[2 * BUF];  // two buffers of [A rows | W rows]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
  const long long M = (long long)B * n;
  const long long m0 = (long long)blockIdx.y * PM;
  const int n0 = blockIdx.x * PN;
  const int nkb = (d + kPK - 1) / kPK;

  // staging: AC chunks of A (row c/8, k 8*(c%8)) and BC of W (row c/CPR, col 8*(c%CPR))
  struct Stage {
    uint4 a[AC], b[BC];
  };
  Stage st[kPStages];
  // Every load is issued (rows and columns past the matrix clamped to its
  // last ones), so that the compiler can count the loads in flight and wait
  // for one k block only.  Clamped rows of X and columns of W only feed
  // outputs that are not stored; k past d is zeroed when the block is put
  // into LDS.
  auto load = [&](Stage& g, int kb) {
    const int k0 = kb * kPK;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i;
      const int ar = c >> 3, ak = (c & 7) * 8;
      const long long row = m0 + ar < M ? m0 + ar : M - 1;
      g.a[i] = *reinterpret_cast<const uint4*>(X + (size_t)row * d + min(k0 + ak, d - 8));
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int c = tid + 256 * i;
      const int br = c / CPR, bc = (c % CPR) * 8;
      g.b[i] = *reinterpret_cast<const uint4*>(W + (size_t)min(k0 + br, d - 1) * d + min(n0 + bc, d - 8));
    }
  };
  auto keep = [](bool ok, const uint4& v) {  // component-wise (a select of the whole vector
    // would go through memory)
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
  };
  auto store = [&](const Stage& g, char* buf, int kb) {
    const int k0 = kb * kPK;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(buf + (c >> 3) * kAPitch + (c & 7) * 16) = keep(k0 + (c & 7) * 8 < d, g.a[i]);
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(buf + ABYTES + (c / CPR) * BPITCH + (c % CPR) * 16) = keep(k0 + c / CPR < d, g.b[i]);
    }
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{0};

  // A fragment: row wm*PM/2 + 32i + lane%32, k 16*kk + 8*h .. +7
  const uint32_t a_off = (uint32_t)((wm * (PM / 2) + (lane & 31)) * kAPitch + h * 16);
  // B fragment by two transpose reads: lane L points at columns
  // 16*((L/16)%2) + 4*(L%4) of W row 8*(L/32) + (L%16)/4 (within a 32-column
  // tile and a 16-row k step), and 4 rows further down for the second read;
  // lane l ends with column l%32 of rows 8*(l/32)..+3 and +4..+7, the same
  // k order as its A fragment
  const uint32_t b_off = (uint32_t)(ABYTES + (8 * h + ((lane & 15) >> 2)) * BPITCH +
                                    (wn * (PN / 2) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);

  // one k block: into LDS buffer kb % 2 from its stage, the stage then takes
  // block kb + kPStages, and the block is multiplied
  auto block = [&](int kb, Stage& g) {
    char* buf = lds + (kb & 1) * BUF;
    store(g, buf, kb);
    __syncthreads();
    load(g, min(kb + kPStages, nkb - 1));
    const uint32_t base = (uint32_t)(uintptr_t)buf;
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      bf16x8_t a[MI], b[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(buf + a_off + 32 * i * kAPitch + 32 * kk);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t o = base + b_off + (uint32_t)(16 * kk * BPITCH + 64 * j);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p*)(size_t)o);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p*)(size_t)(o + 4 * BPITCH));
        b[j] = join_bf16x8(lo, hi);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int j = 0; j < kPStages; ++j) load(st[j], min(j, nkb - 1));
  const int nfull = nkb / kPStages * kPStages;
  for (int kb = 0; kb < nfull; kb += kPStages) {
#pragma unroll
    for (int j = 0; j < kPStages; ++j) block(kb + j, st[j]);
  }
#pragma unroll
  for (int j = 0; j < kPStages - 1; ++j)
    if (nfull + j < nkb) block(nfull + j, st[j]);

  // destination rows: output row m is row r = m mod n of sequence b = m / n,
  // cache row t0[b] + r (skipped outside [0, T_max)); -1 marks a skipped row.
  // Unsigned 32-bit division while every row index fits (a 64-bit division
  // costs an order of magnitude more instructions, 16*MI times per lane).
  long long dst[MI][16];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const long long m = m0 + wm * (PM / 2) + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      long long b, r;
      if (M <= 0xffffffffLL) {
        const uint32_t mu = (uint32_t)m, bu = mu / (uint32_t)n;
        b = bu;
        r = mu - bu * (uint32_t)n;
      } else {
        b = m / n;
        r = m - b * n;
      }
      const long long t = (t0 && m < M ? t0[b] : 0) + r;
      dst[i][e] = (m < M && t >= 0 && t < T_max) ? b * T_max + t : -1;
    }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + wn * (PN / 2) + j * 32 + (lane & 31);
      if (col >= d) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (dst[i][e] >= 0) Kc[(size_t)dst[i][e] * d + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
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
  const unsigned gx = (unsigned)((d + 127) / 128), gx64 = (unsigned)((d + 63) / 64);
  const long long g128 = (M + 127) / 128, g64 = (M + 63) / 64;
  const uint16_t* Xp = static_cast<const uint16_t*>(X);
  const uint16_t* Wp = static_cast<const uint16_t*>(W);
  uint16_t* Kp = static_cast<uint16_t*>(Kc);
  if (g128 * gx >= 512 || g128 > 65535)
    hipLaunchKernelGGL((prefill_bf16_kernel<128, 128>), dim3(gx, (unsigned)g128), dim3(256), 0, s, Xp, Wp, Kp, B, n,
                       d, T_max, t0);
  else if (g64 * gx >= 512 || g64 > 65535)
    hipLaunchKernelGGL((prefill_bf16_kernel<64, 128>), dim3(gx, (unsigned)g64), dim3(256), 0, s, Xp, Wp, Kp, B, n, d,
                       T_max, t0);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<64, 64>), dim3(gx64, (unsigned)g64), dim3(256), 0, s, Xp, Wp, Kp, B, n,
                       d, T_max, t0);
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
