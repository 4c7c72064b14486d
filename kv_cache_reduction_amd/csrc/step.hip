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
//           in batches of 8 (4 for float32 W), two batches in flight, and
//           meet in LDS at the end.  x[b, rows] for BG sequences sits in
//           LDS, read as broadcasts.  W is read once per BG sequences.
//           part[ks][B][2d] float.
// qk_finish sums the ks partials of every output in a fixed order; q goes to
//           the workspace in float32, k to K_cache[b, len_b, :] rounded to
//           the cache format (round to nearest even for bf16) when
//           len_b < T_max, and lengths_next[b] = len_b + 1 (T_max when full).
#include "common.hpp"
#include "mfma16.hpp"
#include "step.hpp"

namespace slim {

constexpr int kQkCols = 512;  // output columns per workgroup (64 lanes x 8)
constexpr int kQkWaves = 8;

// Rows of W per batch and lane (the raw row segments, 4 registers per row
// for bf16 and 8 for float32, take 32 registers per batch; two batches are
// in flight next to the BG x 8 accumulators).
template <bool WBF16>
constexpr int qk_batch_rows() {
  return WBF16 ? 8 : 4;
}
// rows of W per workgroup: 8 waves x U rows x NB batches
template <bool WBF16, int NB>
constexpr int qk_block_rows() {
  return kQkWaves * qk_batch_rows<WBF16>() * NB;
}

// Straight-line code (NB batches unrolled, every load unconditional with
// its row clamped into the block) so that the compiler's wait counts let a
// batch arrive while the previous one is summed.
template <bool WBF16, int BG, int NB>
__global__ void __launch_bounds__(512) qk_proj_kernel(const float* __restrict__ x,
                                                      const void* __restrict__ WQ,
                                                      const void* __restrict__ WK,
                                                      float* __restrict__ part, int B, int d) {
  extern __shared__ __attribute__((aligned(16))) float qk_smem[];
  constexpr int CB = BG < 4 ? BG : 4;  // sequences per round of the cross-wave sum
  constexpr int U = qk_batch_rows<WBF16>();
  constexpr int KR = qk_block_rows<WBF16, NB>();
  constexpr int RW = WBF16 ? 1 : 2;    // 16-byte loads per row segment
  constexpr int XPT = (KR * BG + 511) / 512;  // x values staged per thread
  constexpr int esz = WBF16 ? 2 : 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = blockIdx.y * KR, nk = min(KR, d - k0);
  const int b0 = blockIdx.z * BG;

  // x[b0 + bb, k0 + k] for the block, loads first (indexes clamped; the
  // values outside are replaced by zero when stored)
  float xv_st[XPT];
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int i = tid + 512 * j, k = i / BG, bb = i - k * BG;
    const int kk = min(k, nk - 1), b = min(b0 + bb, B - 1);
    xv_st[j] = x[(size_t)b * d + k0 + kk];
  }

  const int col = blockIdx.x * kQkCols + lane * 8;  // column of [q | k]
  const bool live = col < 2 * d;
  const int cl = live ? col : 0;
  const int wc = cl < d ? cl : cl - d;
  const char* W = static_cast<const char*>(cl < d ? WQ : WK);

  uint4 buf[2][U][RW];
  auto load = [&](uint4 (&raw)[U][RW], int nb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(wave + kQkWaves * (nb * U + u), nk - 1);
#pragma unroll
      for (int v = 0; v < RW; ++v)
        raw[u][v] = *reinterpret_cast<const uint4*>(W + ((size_t)(k0 + r) * d + wc) * esz + 16 * v);
    }
  };
  load(buf[0], 0);
  if constexpr (NB > 1) load(buf[1], 1);

  float* xs = qk_smem;  // [KR][BG], padded to XPT * 512 so every thread stores
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int i = tid + 512 * j, k = i / BG, bb = i - k * BG;
    xs[i] = (k < nk && b0 + bb < B) ? xv_st[j] : 0.f;
  }
  __syncthreads();

  float acc[BG][8];
#pragma unroll
  for (int i = 0; i < BG; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint4 (&raw)[U][RW] = buf[nb & 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = wave + kQkWaves * (nb * U + u);
      if (r < nk) {
        float w[8];
        if constexpr (WBF16) {
          const uint4 v = raw[u][0];
          w[0] = bf_lo(v.x); w[1] = bf_hi(v.x); w[2] = bf_lo(v.y); w[3] = bf_hi(v.y);
          w[4] = bf_lo(v.z); w[5] = bf_hi(v.z); w[6] = bf_lo(v.w); w[7] = bf_hi(v.w);
        } else {
          w[0] = __uint_as_float(raw[u][0].x); w[1] = __uint_as_float(raw[u][0].y);
          w[2] = __uint_as_float(raw[u][0].z); w[3] = __uint_as_float(raw[u][0].w);
          w[4] = __uint_as_float(raw[u][1].x); w[5] = __uint_as_float(raw[u][1].y);
          w[6] = __uint_as_float(raw[u][1].z); w[7] = __uint_as_float(raw[u][1].w);
        }
        float xv[BG];
        if constexpr (BG % 4 == 0) {
#pragma unroll
          for (int i = 0; i < BG; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(xs + r * BG + i);
            xv[i] = v.x; xv[i + 1] = v.y; xv[i + 2] = v.z; xv[i + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int i = 0; i < BG; ++i) xv[i] = xs[r * BG + i];
        }
#pragma unroll
        for (int i = 0; i < BG; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xv[i], w[j], acc[i][j]);
      }
    }
    if (nb + 2 < NB) load(buf[nb & 1], nb + 2);
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

// Many sequences (B >= 8): the same product on MFMA.  x is fp32; it is
// split into three bf16 parts x = hi + mid + lo (together they carry fp32's
// 24 significant bits), each multiplied by bf16 W on 32x32x16 MFMA with fp32
// accumulation, so every product is exact and only the accumulation rounds,
// as on the vector path.  Workgroup: 32 sequences x 256 columns of [q | k]
// (four waves of 64) x KR rows of W in 64-row blocks; the W block sits in LDS
// row-major (two transpose reads give a B operand), the x block as its three
// bf16 parts (one 16-byte read per A operand).  Blocks are staged through
// registers three deep into two LDS buffers (one barrier per block); every
// load is issued with its indexes clamped, and rows past the workgroup's
// range are zeroed when the block is put into LDS, so that the compiler's
// wait counts leave the younger blocks in flight.
constexpr int kQmCols = 256, kQmRows = 64;
constexpr int kQmWPitch = kQmCols * 2 + 16;  // bytes per W row in LDS
constexpr int kQmXPitch = kQmRows * 2 + 16;  // bytes per x row (one part) in LDS
constexpr int kQmStages = 3;
constexpr int kQmWBytes = kQmRows * kQmWPitch, kQmBuf = kQmWBytes + 3 * 32 * kQmXPitch;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_q;

__global__ void __launch_bounds__(256) qk_mfma_kernel(const float* __restrict__ x, const uint16_t* __restrict__ WQ,
                                                      const uint16_t* __restrict__ WK, float* __restrict__ part,
                                                      int B, int d, int KR) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kQmBuf];  // two buffers of [W rows | x parts]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int n2 = 2 * d;
  const int c0 = blockIdx.x * kQmCols;
  const int k0 = blockIdx.y * KR, k1 = min(d, k0 + KR);
  const int b0 = blockIdx.z * 32;
  const int nkb = (k1 - k0 + kQmRows - 1) / kQmRows;

  // staging: 8 chunks of W (row c/32, 8 columns at 8*(c%32)) and 8 x values
  // (sequence c/64, row c%64); clamped sequences only feed outputs that are
  // not stored
  struct Stage {
    uint4 w[8];
    float x[8];
  };
  Stage st[kQmStages];
  auto load = [&](Stage& g, int kb) {
    const int kr = k0 + kb * kQmRows;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const int r = min(kr + (c >> 5), d - 1), col = min(c0 + (c & 31) * 8, n2 - 8);
      const uint16_t* Wm = col < d ? WQ : WK;
      const u32x4 v = *reinterpret_cast<const u32x4*>(Wm + (size_t)r * d + (col < d ? col : col - d));
      g.w[i] = make_uint4(v.x, v.y, v.z, v.w);
      const int xb = min(b0 + (c >> 6), B - 1), xk = min(kr + (c & 63), d - 1);
      g.x[i] = x[(size_t)xb * d + xk];
    }
  };
  auto store = [&](const Stage& g, char* buf, int kb) {
    const int kr = k0 + kb * kQmRows;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const bool wok = kr + (c >> 5) < k1;
      *reinterpret_cast<uint4*>(buf + (c >> 5) * kQmWPitch + (c & 31) * 16) =
          make_uint4(wok ? g.w[i].x : 0u, wok ? g.w[i].y : 0u, wok ? g.w[i].z : 0u, wok ? g.w[i].w : 0u);
      const int xb = c >> 6, xk = c & 63;
      const float v = kr + xk < k1 ? g.x[i] : 0.f;
      const uint32_t hi = f32_to_bf16_rne(v);
      const float r1 = v - __uint_as_float(hi << 16);
      const uint32_t mid = f32_to_bf16_rne(r1);
      const uint32_t lo = f32_to_bf16_rne(r1 - __uint_as_float(mid << 16));
      char* px = buf + kQmWBytes + xb * kQmXPitch + xk * 2;
      *reinterpret_cast<uint16_t*>(px) = (uint16_t)hi;
      *reinterpret_cast<uint16_t*>(px + 32 * kQmXPitch) = (uint16_t)mid;
      *reinterpret_cast<uint16_t*>(px + 64 * kQmXPitch) = (uint16_t)lo;
    }
  };

  f32x16 acc[2] = {f32x16{0}, f32x16{0}};
  // A operands: sequence lane%32, rows 16*kk + 8*h .. +7 of each part
  const uint32_t xa = (uint32_t)(kQmWBytes + (lane & 31) * kQmXPitch + h * 16);
  // B operands by two transpose reads (as in the prefill GEMM): lane L
  // points at columns 16*((L/16)%2) + 4*(L%4) of W row 8*(L/32) + (L%16)/4
  // of a 32-column tile and a 16-row step, and 4 rows further down
  const uint32_t wb = (uint32_t)((8 * h + ((lane & 15) >> 2)) * kQmWPitch +
                                 (wave * 64 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);
  auto block = [&](int kb, Stage& g) {
    char* buf = lds + (kb & 1) * kQmBuf;
    store(g, buf, kb);
    __syncthreads();
    load(g, min(kb + kQmStages, nkb - 1));
    const uint32_t base = (uint32_t)(uintptr_t)buf;
#pragma unroll
    for (int kk = 0; kk < kQmRows / 16; ++kk) {
      bf16x8_t a[3], bo[2];
#pragma unroll
      for (int p3 = 0; p3 < 3; ++p3)
        a[p3] = *reinterpret_cast<const bf16x8_t*>(buf + xa + p3 * 32 * kQmXPitch + 32 * kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t o = base + wb + (uint32_t)(16 * kk * kQmWPitch + 64 * j);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_q*)(size_t)o);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_q*)(size_t)(o + 4 * kQmWPitch));
        bo[j] = join_bf16x8(lo, hi);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int p3 = 0; p3 < 3; ++p3) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[p3], bo[j], acc[j], 0, 0, 0);
    }
  };
#pragma unroll
  for (int j = 0; j < kQmStages; ++j) load(st[j], min(j, nkb - 1));
  const int nfull = nkb / kQmStages * kQmStages;
  for (int kb = 0; kb < nfull; kb += kQmStages) {
#pragma unroll
    for (int j = 0; j < kQmStages; ++j) block(kb + j, st[j]);
  }
#pragma unroll
  for (int j = 0; j < kQmStages - 1; ++j)
    if (nfull + j < nkb) block(nfull + j, st[j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = c0 + wave * 64 + 32 * j + (lane & 31);
    if (col >= n2) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int b = b0 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (b < B) part[((size_t)blockIdx.y * B + b) * n2 + col] = acc[j][e];
    }
  }
}

constexpr int kQkSumBatch = 32;  // partials loaded together per output

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
  const size_t stride = (size_t)B * n2;
  float s = 0.f;
  for (int k = 0; k < ks; k += kQkSumBatch) {  // loads of a batch first, then the sum in order
    float v[kQkSumBatch];
#pragma unroll
    for (int j = 0; j < kQkSumBatch; ++j) v[j] = k + j < ks ? part[(size_t)(k + j) * stride + i] : 0.f;
#pragma unroll
    for (int j = 0; j < kQkSumBatch; ++j) s += v[j];
  }
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

bool make_step_plan(int B, int d, int ncu, bool w_bf16, size_t base, StepPlan* p) {
  if (B <= 0 || d <= 0 || d % 8 != 0) return false;
  p->mfma = w_bf16 && B >= 8;
  if (p->mfma) {  // 256-column tiles x 32 sequences; row blocks of 64 rows for about one round
    const int ntile = (2 * d + kQmCols - 1) / kQmCols, mg = (B + 31) / 32;
    const int nblk = (d + kQmRows - 1) / kQmRows;
    long long ks = (long long)ncu / ((long long)ntile * mg);
    if (ks < 1) ks = 1;
    if (ks > nblk) ks = nblk;
    p->kr = (int)((nblk + ks - 1) / ks) * kQmRows;
    p->ks = (d + p->kr - 1) / p->kr;
    p->ntile = ntile;
    p->bgroups = mg;
    p->bg = 32;
    p->nb = 0;
    size_t off = (base + 255) & ~(size_t)255;
    p->off_q = off;
    off += ((size_t)B * d * sizeof(float) + 255) & ~(size_t)255;
    p->off_part = off;
    off += ((size_t)p->ks * B * 2 * d * sizeof(float) + 255) & ~(size_t)255;
    p->bytes = off;
    return true;
  }
  p->bg = B >= 16 ? 16 : (B > 8 ? 16 : (B > 4 ? 8 : (B > 2 ? 4 : B)));
  const int ntile = (2 * d + kQkCols - 1) / kQkCols;
  const int bgroups = (B + p->bg - 1) / p->bg;
  // one round of workgroups where possible: two per compute unit for few
  // sequences (short, load-bound blocks), one for many (their partial sums
  // grow with B); the fewest batches per wave that fit
  const long long target = (long long)ncu * (p->bg <= 4 ? 2 : 1);
  const int rows1 = kQkWaves * (w_bf16 ? qk_batch_rows<true>() : qk_batch_rows<false>());
  p->nb = 4;
  for (int nb = 1; nb <= 4; nb *= 2) {
    const long long ks = (d + (long long)rows1 * nb - 1) / ((long long)rows1 * nb);
    if (ks * ntile * bgroups <= target) {
      p->nb = nb;
      break;
    }
  }
  p->kr = rows1 * p->nb;
  p->ks = (d + p->kr - 1) / p->kr;
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

template <bool WBF16, int BG, int NB>
static hipError_t launch_proj(const StepPlan& p, const float* x, const void* WQ, const void* WK,
                              float* part, int B, int d, hipStream_t s) {
  constexpr int CB = BG < 4 ? BG : 4;
  const size_t xs = (size_t)((qk_block_rows<WBF16, NB>() * BG + 511) / 512) * 512 * sizeof(float);
  const size_t red = (size_t)kQkWaves * CB * kQkCols * sizeof(float);
  hipLaunchKernelGGL((qk_proj_kernel<WBF16, BG, NB>), dim3(p.ntile, p.ks, p.bgroups), dim3(512),
                     xs > red ? xs : red, s, x, WQ, WK, part, B, d);
  return hipGetLastError();
}

template <bool WBF16, int BG>
static hipError_t launch_proj_nb(const StepPlan& p, const float* x, const void* WQ, const void* WK,
                                 float* part, int B, int d, hipStream_t s) {
  switch (p.nb) {
    case 1: return launch_proj<WBF16, BG, 1>(p, x, WQ, WK, part, B, d, s);
    case 2: return launch_proj<WBF16, BG, 2>(p, x, WQ, WK, part, B, d, s);
    case 4: return launch_proj<WBF16, BG, 4>(p, x, WQ, WK, part, B, d, s);
  }
  return hipErrorInvalidValue;
}

template <bool WBF16>
static hipError_t launch_proj_bg(const StepPlan& p, const float* x, const void* WQ, const void* WK,
                                 float* part, int B, int d, hipStream_t s) {
  switch (p.bg) {
    case 1: return launch_proj_nb<WBF16, 1>(p, x, WQ, WK, part, B, d, s);
    case 2: return launch_proj_nb<WBF16, 2>(p, x, WQ, WK, part, B, d, s);
    case 4: return launch_proj_nb<WBF16, 4>(p, x, WQ, WK, part, B, d, s);
    case 8: return launch_proj_nb<WBF16, 8>(p, x, WQ, WK, part, B, d, s);
    case 16: return launch_proj_nb<WBF16, 16>(p, x, WQ, WK, part, B, d, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_step_qk(const StepPlan& p, const float* x, const void* WQ, const void* WK, bool w_bf16,
                          void* Kc, bool k_bf16, const int32_t* lengths, int32_t* lengths_next, int B,
                          int d, int T_max, char* ws, hipStream_t s) {
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  float* q = reinterpret_cast<float*>(ws + p.off_q);
  hipError_t e;
  if (p.mfma) {
    hipLaunchKernelGGL(qk_mfma_kernel, dim3(p.ntile, p.ks, p.bgroups), dim3(256), 0, s, x,
                       static_cast<const uint16_t*>(WQ), static_cast<const uint16_t*>(WK), part, B, d, p.kr);
    e = hipGetLastError();
  } else {
    e = w_bf16 ? launch_proj_bg<true>(p, x, WQ, WK, part, B, d, s)
               : launch_proj_bg<false>(p, x, WQ, WK, part, B, d, s);
  }
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
