// Slim-Attention decode, finish phase: merge the per-chunk partials of each
// sequence and apply W_KV per head (Slim Attention article, localbendi.com,
// section "K-Cache is All You Need": V = K.W_KV, so head h's output is
// (softmax_h . K) . W_KV[:, h*dh:(h+1)*dh]).
//
// Partials (written by the attend phase) are laid out U[h][slot][d] and
// ml[slot][2][H] (running max in log2 units, normaliser).
//
// merge_project  grid (H, ceil(d/R), ceil(B/S)), R rows of W_KV per
//          workgroup (256, or 64 when that grid would be small) and S = 8
//          or 16 sequences (16 while that grid still fills the device, so
//          that W_KV is read half as often).  For each of its sequences b the
//          workgroup first merges the slots s of b over its R rows
//          (log-sum-exp):
//            m* = max_s m_s,  l* = sum_s 2^(m_s - m*) l_s,
//            u[r] = sum_s 2^(m_s - m*) U_s[h, r] / l*
//          (each thread over its own slots with a running max, then the
//          threads' sums combined the same way),
//          then multiplies by the W_KV rows it holds in registers:
//            part[rb, b, h, j] = sum_{r in rows} u[r] W_KV[r, h*dh + j].
//          With bf16 W_KV and at least 4 sequences per workgroup this
//          product runs on MFMA (16x16x16, the workgroup's sequences as the
//          16 rows of A; with fewer, the padding rows would dominate and
//          the vector ALU is faster): the W_KV rows go
//          through LDS in rounds of 64 and reach the B operand by transposing
//          reads; each merged value is split exactly into three bf16 parts
//          (u = hi + mid + lo), so the products are exact and only the fp32
//          accumulation rounds.  fp32 W_KV uses the vector ALU.
//          The partials are read once and W_KV once per S sequences.
// reduce   out[b, h, j] = sum_rb part[rb, b, h, j] in a fixed order, so the
//          result does not depend on scheduling (not launched when one row
//          block covers d: merge_project then writes out itself).
#include "common.hpp"
#include "internal.hpp"
#include "multi.hpp"

namespace slim {

constexpr int kMergeBatch = 8;  // slots whose loads a thread issues together
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// x = hi + mid + lo exactly, each a bf16 (its bits in the low 16 bits of the
// result): every part is the remaining value truncated to bf16, and what is
// left after two parts has at most 8 significant bits.
__device__ __forceinline__ void split3_bf16(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t hb = __float_as_uint(x) & 0xffff0000u;
  const float r = x - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(r) & 0xffff0000u;
  const float r2 = r - __uint_as_float(mb);
  hi = hb >> 16;
  mid = mb >> 16;
  lo = __float_as_uint(r2) >> 16;
}

template <int DH, bool WBF16, int PR, bool MFMA, bool UB>
__global__ void __launch_bounds__(256) merge_project_kernel(const int32_t* __restrict__ lengths,
                                                            const void* __restrict__ Uv,
                                                            const float* __restrict__ ml,
                                                            const void* __restrict__ W,
                                                            float* __restrict__ part,
                                                            uint32_t* __restrict__ status, int B, int H, int d,
                                                            int T_max, int nch, int nslots, int fixed_ns,
                                                            int spw) {
  // projection: thread t covers JW output columns (group jq = t % JQ) over the
  // rows of subset t / JQ
  constexpr int JQ = DH >= 8 ? DH / 8 : 1;  // column groups per head
  constexpr int JW = DH >= 8 ? 8 : DH;      // columns per group
  constexpr int NRS = 256 / JQ;             // row subsets
  constexpr int RPT = PR / NRS;             // rows per thread
  static_assert(RPT >= 1 && RPT * NRS == PR, "row split");
  // merge: float4 column c4 of a slot subset; 256 / C4 (sequence, subset)
  // pairs share the workgroup
  constexpr int C4 = PR / 4;
  constexpr int NSS = 256 / C4;
  static_assert(C4 * NSS == 256, "merge split");
  // MFMA projection (bf16 W_KV): W_KV rows through LDS, CR at a time
  constexpr bool MP = MFMA && WBF16 && DH >= 16 && DH % 16 == 0 && JW == 8;
  constexpr int CR = PR < 64 ? PR : 64;
  constexpr int PITCH = DH * 2 + 32;  // bytes per W_KV row in LDS (rows of a transposing read on distinct banks)
  constexpr int WL = MP ? CR * PITCH / 4 : 0;
  static_assert(!MP || (CR % 16 == 0 && CR % RPT == 0 && PR % CR == 0), "projection rounds");
  extern __shared__ int smem[];
  int* tmp = smem;                                       // [8]
  float* red = reinterpret_cast<float*>(smem + 8);       // [max(NSS * PR, NRS * DH)]
  constexpr int RED = NSS * PR > NRS * DH ? NSS * PR : NRS * DH;
  float* us = red + RED;                                 // [spw][PR]
  float* mstar = us + spw * PR;                          // [NSS][2]: running max, normaliser
  char* wl = reinterpret_cast<char*>(mstar + 2 * NSS);   // [CR][PITCH] bytes: W_KV rows of a round (MP)
  int* pre = reinterpret_cast<int*>(mstar + 2 * NSS + WL);  // [B + 1]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, r0 = blockIdx.y * PR, b0 = blockIdx.z * spw;
  const int nr = min(PR, d - r0), nb = min(spw, B - b0);

  // W_KV rows [r0, r0 + PR) of head h's columns, in registers.  The loads
  // are unconditional (rows past the block clamped, then zeroed) so that
  // they are all in flight together.
  const int jq = tid % JQ, rs = tid / JQ;
  float w[MP ? 1 : RPT][JW];  // vector-ALU projection: fp32 values
  uint4 wq[MP ? RPT : 1];     // MFMA projection: 8 packed bf16 per row
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rs * RPT + i;
    const bool live = r < nr;
    const size_t base = (size_t)(r0 + (live ? r : nr - 1)) * d + (size_t)h * DH + jq * JW;
    if constexpr (MP) {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + base);
      wq[i] = live ? v : make_uint4(0u, 0u, 0u, 0u);
      continue;
    } else if constexpr (WBF16 && JW == 8) {
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
    if constexpr (!MP) {
#pragma unroll
      for (int k = 0; k < JW; ++k) w[i][k] = live ? w[i][k] : 0.f;
    }
  }

  // slots of sequence b: the chunks its rows fall in (decode), or a fixed
  // count per row, slot = b * fixed_ns + split (many queries over one context)
  int Ts = 1;
  if (fixed_ns == 0) {
    lengths_prefix(lengths, B, T_max, pre, tmp);
    Ts = chunk_tokens(pre[B] > 0 ? pre[B] : 1, nch);
  }

  // merged rows u[bb][r] of head h, rows [r0, r0 + nr): G sequences at a
  // time, 256/G threads each (C4 float4 columns x nss slot subsets).  Each
  // thread merges its slots with a running max of its own (one pass over U
  // and ml); the subsets then meet in LDS with the usual rescaling.
  int G = nb >= 8 ? 8 : (nb >= 4 ? 4 : (nb >= 2 ? 2 : 1));
  if (G > NSS) G = NSS;
  const int tps = 256 / G, nss = tps / C4;
  const int g = tid / tps, c4 = (tid % tps) % C4, ss = (tid % tps) / C4;
  const bool aligned = (d & 3) == 0;
  for (int base = 0; base < nb; base += G) {
    const int bb = base + g;
    const int b = b0 + bb;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float m = kNegInf, l = 0.f;
    bool bad = false;
    if (bb < nb && (fixed_ns > 0 || pre[b + 1] > pre[b])) {
      int ns, slot0;
      if (fixed_ns > 0) {
        ns = fixed_ns;
        slot0 = b * fixed_ns;
      } else {
        const int s0 = pre[b], s1 = pre[b + 1], cf = s0 / Ts;
        ns = (s1 - 1) / Ts - cf + 1;
        slot0 = cf + b;
      }
      const bool cols = 4 * c4 < nr;
      const float* mls = ml + (size_t)slot0 * 2 * H + h;
      for (int i = ss; i < ns; i += kMergeBatch * nss) {  // a batch of slots per round, loads first
        // every load of the batch is issued unconditionally (slots past the
        // sequence clamped to its last one, columns past the block to the
        // first) so that all are in flight together; dead ones are zeroed
        // after
        float4 x[kMergeBatch];
        float ms[kMergeBatch], ls[kMergeBatch];
        const size_t col = (size_t)h * nslots * d + (size_t)slot0 * d + r0 + 4 * (cols ? c4 : 0);
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
          const int j = i + k * nss;
          const int jj = j < ns ? j : ns - 1;
          ms[k] = mls[(size_t)jj * 2 * H];
          ls[k] = mls[(size_t)jj * 2 * H + H];
          if constexpr (UB) {  // bf16 partials (d % 8 == 0: 8-byte aligned)
            const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(Uv) + col + (size_t)jj * d);
            x[k] = make_float4(bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y));
          } else if (aligned) {
            x[k] = *reinterpret_cast<const float4*>(static_cast<const float*>(Uv) + col + (size_t)jj * d);
          } else {  // rows not 16-byte aligned (d % 4 != 0)
            const float* v = static_cast<const float*>(Uv) + col + (size_t)jj * d;
            x[k].x = v[0];
            x[k].y = 4 * c4 + 1 < nr ? v[1] : 0.f;
            x[k].z = 4 * c4 + 2 < nr ? v[2] : 0.f;
            x[k].w = 4 * c4 + 3 < nr ? v[3] : 0.f;
          }
        }
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
          const bool ok = i + k * nss < ns;
          ms[k] = ok ? ms[k] : kNegInf;
          ls[k] = ok ? ls[k] : 0.f;
          x[k] = ok && cols ? x[k] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) bad |= ms[k] != ms[k];  // an attend piece marked NaN
        float mn = m;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) mn = fmaxf(mn, ms[k]);
        if (mn > kNegInf) {
          const float sc = fast_exp2(m - mn);
          acc.x *= sc;
          acc.y *= sc;
          acc.z *= sc;
          acc.w *= sc;
          l *= sc;
#pragma unroll
          for (int k = 0; k < kMergeBatch; ++k) {
            const float q = fast_exp2(ms[k] - mn);
            l = fmaf(q, ls[k], l);
            acc.x = fmaf(q, x[k].x, acc.x);
            acc.y = fmaf(q, x[k].y, acc.y);
            acc.z = fmaf(q, x[k].z, acc.z);
            acc.w = fmaf(q, x[k].w, acc.w);
          }
          m = mn;
        }
      }
    }
    const int slot_id = g * nss + ss;  // < NSS
    float* rr = red + slot_id * PR + 4 * c4;
    rr[0] = acc.x;
    rr[1] = acc.y;
    rr[2] = acc.z;
    rr[3] = acc.w;
    if (c4 == 0) {
      mstar[2 * slot_id] = m;
      mstar[2 * slot_id + 1] = bad ? __builtin_nanf("") : l;
    }
    if (bad && status) *status = 1u;  // an attend piece gave up: report it
    __syncthreads();
    for (int r = tid; r < G * PR; r += 256) {
      const int gg = r / PR, rw = r % PR;
      float mx = kNegInf;
      for (int k = 0; k < nss; ++k) mx = fmaxf(mx, mstar[2 * (gg * nss + k)]);
      float x = 0.f, lt = 0.f;
      for (int k = 0; k < nss; ++k)
        if (mstar[2 * (gg * nss + k) + 1] != mstar[2 * (gg * nss + k) + 1]) lt = __builtin_nanf("");
      if (mx > kNegInf) {
        for (int k = 0; k < nss; ++k) {
          const float q = fast_exp2(mstar[2 * (gg * nss + k)] - mx);
          x = fmaf(q, red[(gg * nss + k) * PR + rw], x);
          lt = fmaf(q, mstar[2 * (gg * nss + k) + 1], lt);
        }
      }
      if (base + gg < nb) us[(base + gg) * PR + rw] = (rw < nr && !(lt <= 0.f)) ? x / lt : 0.f;
    }
    __syncthreads();
  }

  const size_t nout = (size_t)B * H * DH;
  if constexpr (MP) {
    // D[m][n] = sum_k u[m][k] W[k][n] over this block's rows: m = sequence
    // (16 rows of A, those past nb zero), n = 16-column tile of the head.
    // Lane (g, j) = (lane / 16, lane % 16) holds A[j][4g..4g+3],
    // B[4g..4g+3][j] and D[4g..4g+3][j].
    constexpr int NT = DH / 16;
    constexpr int TPW = NT >= 4 ? NT / 4 : 1;  // tiles per wave
    const int g = lane >> 4, j = lane & 15;
    const uint32_t wl_s = (uint32_t)reinterpret_cast<uintptr_t>(wl);
    f32x4 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < PR / CR; ++c) {
      const int rr = rs * RPT - c * CR;  // this thread's rows, relative to the round
      if (rr >= 0 && rr < CR) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) *reinterpret_cast<uint4*>(wl + (rr + i) * PITCH + jq * 16) = wq[i];
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < CR / 16; ++ks) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < nb) x = *reinterpret_cast<const float4*>(us + j * PR + c * CR + ks * 16 + 4 * g);
        uint32_t h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
        split3_bf16(x.x, h0, m0, l0);
        split3_bf16(x.y, h1, m1, l1);
        split3_bf16(x.z, h2, m2, l2);
        split3_bf16(x.w, h3, m3, l3);
        const s16x4 ah = {(short)h0, (short)h1, (short)h2, (short)h3};
        const s16x4 am = {(short)m0, (short)m1, (short)m2, (short)m3};
        const s16x4 al = {(short)l0, (short)l1, (short)l2, (short)l3};
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const int nt = wave * TPW + t;
          if (nt < NT) {
            const lds_s16x4* bp = (const lds_s16x4*)(size_t)(
                wl_s + (uint32_t)((ks * 16 + 4 * g + (j >> 2)) * PITCH + (nt * 16 + 4 * (j & 3)) * 2));
            const s16x4 bv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(bp));
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bv, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(am, bv, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bv, acc[t], 0, 0, 0);
          }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int nt = wave * TPW + t;
      if (nt < NT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * g + i;
          if (m < nb) part[(size_t)blockIdx.y * nout + ((size_t)(b0 + m) * H + h) * DH + nt * 16 + j] = acc[t][i];
        }
      }
    }
    return;
  }
  // projection of each merged row block by the W_KV rows held in registers
  for (int bb = 0; bb < nb; ++bb) {
    float acc[JW];
#pragma unroll
    for (int k = 0; k < JW; ++k) acc[k] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float x = us[bb * PR + rs * RPT + i];
#pragma unroll
      for (int k = 0; k < JW; ++k) acc[k] = fmaf(x, w[i][k], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < JW; ++k) red[rs * DH + jq * JW + k] = acc[k];
    __syncthreads();
    for (int j = tid; j < DH; j += 256) {
      float s = 0.f;
#pragma unroll 8
      for (int k = 0; k < NRS; ++k) s += red[k * DH + j];
      part[(size_t)blockIdx.y * nout + ((size_t)(b0 + bb) * H + h) * DH + j] = s;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) proj_reduce_kernel(const float* __restrict__ part,
                                                          float* __restrict__ out, int npc, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k0 = 0; k0 < npc; k0 += 16) {  // a batch's loads first, then the sum in order
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = k0 + j < npc ? part[(size_t)(k0 + j) * n + i] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
  }
  out[i] = s;
}

template <int DH, bool WBF16, int PR>
static hipError_t launch_t(const DecodePlan& pl, const DecodeArgs& a, int fixed_ns, hipStream_t s) {
  constexpr int JQ = DH >= 8 ? DH / 8 : 1;
  constexpr int NRS = 256 / JQ;
  constexpr int NSS = 256 / (PR / 4);
  constexpr int RED = NSS * PR > NRS * DH ? NSS * PR : NRS * DH;
  const void* U = a.ws + pl.off_U;
  const float* ml = reinterpret_cast<const float*>(a.ws + pl.off_ml);
  // one row block covering all of d (small d): the workgroups write out directly
  float* part = pl.npc == 1 ? a.out : reinterpret_cast<float*>(a.ws + pl.off_op);
  const int spw = pl.spw == 16 ? 16 : 8;
  // MFMA projection when a workgroup has at least 4 sequences
  constexpr bool MFMA_OK = WBF16 && DH >= 16 && DH % 16 == 0;
  const bool mp = MFMA_OK && (a.B < spw ? a.B : spw) >= 4;
  const int WL = mp ? (PR < 64 ? PR : 64) * (DH * 2 + 32) / 4 : 0;
  const size_t lds =
      (8 + (size_t)RED + (size_t)spw * PR + 2 * NSS + WL + (fixed_ns > 0 ? 0 : (size_t)a.B + 1)) * 4;
  const dim3 grid(a.H, pl.npc, (a.B + spw - 1) / spw);
  // bf16 partials exist only for the bf16-cache head widths
  constexpr bool UB_OK = DH == 32 || DH == 64 || DH == 128;
  const bool ub = UB_OK && pl.ubf16;
  if (mp && ub)
    hipLaunchKernelGGL((merge_project_kernel<DH, WBF16, PR, MFMA_OK, UB_OK>), grid, dim3(256), lds, s, a.lengths, U,
                       ml, a.W, part, a.status, a.B, a.H, a.d, a.T_max, pl.nch, pl.nslots, fixed_ns, spw);
  else if (mp)
    hipLaunchKernelGGL((merge_project_kernel<DH, WBF16, PR, MFMA_OK, false>), grid, dim3(256), lds, s, a.lengths, U,
                       ml, a.W, part, a.status, a.B, a.H, a.d, a.T_max, pl.nch, pl.nslots, fixed_ns, spw);
  else if (ub)
    hipLaunchKernelGGL((merge_project_kernel<DH, WBF16, PR, false, UB_OK>), grid, dim3(256), lds, s, a.lengths, U,
                       ml, a.W, part, a.status, a.B, a.H, a.d, a.T_max, pl.nch, pl.nslots, fixed_ns, spw);
  else
    hipLaunchKernelGGL((merge_project_kernel<DH, WBF16, PR, false, false>), grid, dim3(256), lds, s, a.lengths, U,
                       ml, a.W, part, a.status, a.B, a.H, a.d, a.T_max, pl.nch, pl.nslots, fixed_ns, spw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.npc == 1) return e;
  const int n = a.B * a.H * DH;
  hipLaunchKernelGGL(proj_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, (const float*)part,
                     a.out, pl.npc, n);
  return hipGetLastError();
}

template <int DH>
static hipError_t launch_w(const DecodePlan& pl, const DecodeArgs& a, int fixed_ns, hipStream_t s) {
  constexpr int big = proj_rows(DH, true), small = proj_rows(DH, false);
  if (pl.proj_rows == big)
    return a.w_bf16 ? launch_t<DH, true, big>(pl, a, fixed_ns, s) : launch_t<DH, false, big>(pl, a, fixed_ns, s);
  if (pl.proj_rows == small)
    return a.w_bf16 ? launch_t<DH, true, small>(pl, a, fixed_ns, s)
                    : launch_t<DH, false, small>(pl, a, fixed_ns, s);
  return hipErrorInvalidValue;
}

hipError_t launch_finish_fixed(const DecodePlan& pl, const DecodeArgs& a, int fixed_ns, hipStream_t s) {
  switch (a.dh) {
    case 1: return launch_w<1>(pl, a, fixed_ns, s);
    case 2: return launch_w<2>(pl, a, fixed_ns, s);
    case 4: return launch_w<4>(pl, a, fixed_ns, s);
    case 8: return launch_w<8>(pl, a, fixed_ns, s);
    case 16: return launch_w<16>(pl, a, fixed_ns, s);
    case 32: return launch_w<32>(pl, a, fixed_ns, s);
    case 64: return launch_w<64>(pl, a, fixed_ns, s);
    case 128: return launch_w<128>(pl, a, fixed_ns, s);
    case 256: return launch_w<256>(pl, a, fixed_ns, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_finish(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  return launch_finish_fixed(pl, a, 0, s);
}

}  // namespace slim
