// Many queries over one context, on MFMA: shared-context cross-attention
// (n decoder queries over one encoder K) and the causal prompt phase (a
// prompt's n tokens over its own K rows).  Slim Attention article,
// localbendi.com, section "K-Cache is All You Need": only K is kept; the
// values follow from V = K.W_KV, either formed first (option 1) or applied
// after the softmax has been multiplied by K (option 2).
//
// multi_attend<DH, QW, OPT>  grid (column blocks, H x query groups, T splits;
// with row limits the query groups are taken heaviest first),
// QW waves of 64 lanes; wave w owns 32 queries of head h.
//  * Tiles of 64 context rows (32 for workgroups of fewer than four waves)
//    travel global -> registers -> LDS (two tiles
//    in flight in registers while a third is used from LDS; two LDS
//    buffers, one barrier per tile): head h's DH key columns for the scores
//    and the value block: 128 columns of K (option 2) or head h's DH columns
//    of V (option 1).  All waves of the workgroup share the tile.
//  * Scores on 32x32x16 bf16 MFMA, computed transposed (S^T = K_h . Q_h^T,
//    the tile's K rows as the A operand, Q as the B operand) with Q split
//    into bf16 high and low parts (two MFMAs per step), so the products keep
//    about 16 bits of Q; fp32 accumulation.  The reduction over the head's
//    DH dimensions is ordered so that a lane's A operand is one 16-byte LDS
//    read of its row: lanes 0-31 take dimensions [0, DH/2), lanes 32-63
//    [DH/2, DH), eight per step, and Q (in registers for the whole kernel)
//    follows the same order.
//  * The transposed result already has the A-operand layout of P . V (lane =
//    query, 16 context rows each, halves joined by a lane swap), where the
//    online softmax runs: rows past a query's limit are -inf; lazy rescaling keeps
//    a reference max m (log2 units; Q is pre-scaled by scale*log2 e) that
//    moves only when a score exceeds it by more than 8, so weights stay
//    below 2^8; the accumulator rows are then rescaled through LDS.
//  * P (bf16) . value block on 32x32x16 MFMA, each B operand from two
//    transpose reads (ds_read_b64_tr_b16) of the tile rows.  A 16-row step
//    takes, in lane half g, the context rows 4g..4g+3 and 8+4g..8+4g+3 of
//    its 16 (the order the transposed scores hold them in); the B operand
//    takes the same rows, and the MFMA sums over them in any order.
//  * Option 2 writes unnormalised partial rows U[h, q*nsplit + split, cols]
//    and (column block 0) m and the normaliser l, the layout the decode
//    finish merges and projects by W_KV.  Option 1 writes the normalised
//    output rows directly (one split) or partial rows of the head's dh
//    columns that multi_merge combines.
#include "common.hpp"
#include "mfma16.hpp"
#include "internal.hpp"
#include "multi.hpp"
#include "launch.hpp"

namespace slim {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_m;

constexpr int kMRows = 32;              // context rows per score MFMA block (and the plan's split unit)
constexpr float kMultiSlack = 8.f;      // log2 units
constexpr uint32_t kOnes2 = 0x3f803f80u;  // two bf16 1.0

struct MultiParams {
  const float* Q;          // [n, d]
  const uint16_t* K;       // [T, d] bf16
  const uint16_t* Vs;      // value rows [T, d] bf16: K (option 2) or V (option 1)
  const int32_t* limits;   // [n] or null (all T rows)
  float* U;                // option 2: [H][n * nsplit][d]
  float* ml;               // option 2: [n * nsplit][2][H]
  float* out;              // option 1: [n][H][DH]
  int n, H, d, T, nsplit, Ts, nslots;
  float qscale;
};

// The pair {x of lane l, x of lane l^32} in every lane (in some order):
// their max or sum is the reduction over the two halves of the wave.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DH, int QW, int OPT>
struct MultiShape {
  // score blocks per tile: two (64-row tiles) for four-wave workgroups,
  // whose per-tile staging and barrier then cover twice the rows; one where
  // the extra registers would not fit
  static constexpr int MB = QW >= 4 ? 2 : 1;
  static constexpr int MT = kMRows * MB;              // context rows per tile
  static constexpr int NCW = OPT == 2 ? 128 : DH;     // value columns per workgroup
  static constexpr int NCT = NCW / 32;                // 32-column MFMA tiles per wave
  static constexpr int SP = DH * 2 + 16;              // bytes per score row in LDS
  static constexpr int VP = NCW * 2 + 16;             // bytes per value row in LDS
  static constexpr int SCH = MT * DH / 8;             // 16-byte chunks of the score part
  static constexpr int VCH = MT * NCW / 8;            // 16-byte chunks of the value part
  static constexpr int TILE = MT * (SP + VP);         // bytes per tile buffer
};

template <int DH, int QW, int OPT>
__global__ void __launch_bounds__(64 * QW) multi_attend_kernel(MultiParams p) {
  using S = MultiShape<DH, QW, OPT>;
  constexpr int NT = 64 * QW;
  constexpr int kMBlocks = S::MB, kMTile = S::MT;
  constexpr int CPT = (S::SCH + S::VCH + NT - 1) / NT;  // chunks per thread and tile
  extern __shared__ __attribute__((aligned(16))) char msm[];
  char* tiles = msm;                                               // [2][TILE]
  float* rowv = reinterpret_cast<float*>(msm + 2 * S::TILE);       // [QW][32]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, m = lane & 31;
  const int nqg = (p.n + 32 * QW - 1) / (32 * QW);
  // (head, query group, split) of the workgroup.  With row limits (the
  // causal prompt, where later queries see more rows) the workgroups are
  // dispatched heaviest first: query groups in descending order, heads
  // innermost, so that the light ones come last and share CUs with the
  // others; any order is correct, this one shortens the tail.  Without
  // limits every workgroup has the same work.
  int h, qg, split;
  if (p.limits) {
    const int L = blockIdx.y + gridDim.y * blockIdx.z, rest = L / p.H;
    h = L - rest * p.H;
    qg = nqg - 1 - rest / p.nsplit;
    split = rest - (rest / p.nsplit) * p.nsplit;
  } else {
    h = blockIdx.y / nqg;
    qg = blockIdx.y - h * nqg;
    split = blockIdx.z;
  }
  const int d = p.d;
  const int c0 = OPT == 2 ? blockIdx.x * S::NCW : h * DH;  // first value column
  const int q = (qg * QW + wave) * 32 + m;                 // this lane's query row
  const bool qok = q < p.n;

  const int t_begin = split * p.Ts;
  const int q_first = qg * QW * 32;  // the workgroup's first query row

  // every load of the set-up is issued first, in the order the data is
  // needed, with clamped rows so that none sits under a branch and all are
  // in flight together: the query limits, this lane's q row, then the first
  // two context tiles
  constexpr int kLimLoads = (QW * 32 + 63) / 64;
  int lim_raw = p.T, wg_raw[kLimLoads];
  if (p.limits) {
    lim_raw = p.limits[qok ? q : 0];
#pragma unroll
    for (int i = 0; i < kLimLoads; ++i) wg_raw[i] = p.limits[min(q_first + 64 * i + lane, p.n - 1)];
  }
  u32x4 qraw[DH / 8];
  {
    const float* qr = p.Q + (size_t)(qok ? q : 0) * d + h * DH + hh * (DH / 2);
#pragma unroll
    for (int i = 0; i < DH / 8; ++i) qraw[i] = *reinterpret_cast<const u32x4*>(qr + 4 * i);
  }

  // tile loads: chunk c < SCH is score row c / (DH/8), 8 columns at
  // 8*(c % (DH/8)); the rest are value rows.  Each thread's chunks are fixed,
  // so their sources (row 0 of the tile), rows and LDS offsets are computed
  // once; rows past T are clamped (and masked later).
  const uint16_t* ch_src[CPT];
  int ch_row[CPT];
  uint32_t ch_lds[CPT];
  bool ch_ok[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + NT * i;
    ch_ok[i] = c < S::SCH + S::VCH;
    if (c < S::SCH) {
      const int r = c / (DH / 8), k8 = c - r * (DH / 8);
      ch_row[i] = r;
      ch_src[i] = p.K + h * DH + 8 * k8;
      ch_lds[i] = (uint32_t)(r * S::SP + 16 * k8);
    } else {
      const int cc = ch_ok[i] ? c - S::SCH : 0, r = cc / (S::NCW / 8), k8 = cc - r * (S::NCW / 8);
      ch_row[i] = r;
      ch_src[i] = p.Vs + min(c0 + 8 * k8, d - 8);
      ch_lds[i] = (uint32_t)(kMTile * S::SP + r * S::VP + 16 * k8);
    }
  }
  uint4 stage[2][CPT];  // tiles it+1 and it+2 in flight while tile it is used
  auto load_tile = [&](uint4 (&st)[CPT], int tb) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int row = min(tb + ch_row[i], p.T - 1);
      // always issued (unused chunks are never stored); loaded as a vector
      // value, so that the stage stays in registers
      const u32x4 v = *reinterpret_cast<const u32x4*>(ch_src[i] + (size_t)row * d);
      st[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  auto store_tile = [&](const uint4 (&st)[CPT], char* buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (ch_ok[i]) *reinterpret_cast<uint4*>(buf + ch_lds[i]) = st[i];
  };

  load_tile(stage[0], t_begin);
  load_tile(stage[1], t_begin + kMTile);

  // query limits: this lane's row (clamped to [0, T]), and the workgroup's
  // largest, where its tiles stop; each wave reduces all of the workgroup's
  // rows itself, so no barrier is needed
  const auto clamp_t = [&](int x) { return x < 0 ? 0 : (x > p.T ? p.T : x); };
  const int lim = qok ? clamp_t(lim_raw) : 0;
  int wg_lim = p.T;
  if (p.limits) {
    wg_lim = 0;
#pragma unroll
    for (int i = 0; i < kLimLoads; ++i)
      if (64 * i + lane < QW * 32 && q_first + 64 * i + lane < p.n) wg_lim = max(wg_lim, clamp_t(wg_raw[i]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wg_lim = max(wg_lim, __shfl_xor(wg_lim, off));
    wg_lim = __builtin_amdgcn_readfirstlane(wg_lim);
  }
  const int t_end = min(min(p.T, t_begin + p.Ts), wg_lim);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kMTile - 1) / kMTile : 0;

  // Q_h of this lane's row, scaled, as bf16 hi/lo in the score A-operand
  // order: step k takes dimensions hh*DH/2 + 4k .. +3; rows past n are zero
  bf16x8_t qh[DH / 16], ql[DH / 16];
#pragma unroll
  for (int k = 0; k < DH / 16; ++k) {
    s16x4 hv[2], lv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const u32x4 r = qraw[2 * k + e];
      const float4 v = make_float4(qok ? __uint_as_float(r.x) : 0.f, qok ? __uint_as_float(r.y) : 0.f,
                                   qok ? __uint_as_float(r.z) : 0.f, qok ? __uint_as_float(r.w) : 0.f);
      uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
      split_bf16(v.x * p.qscale, h0, l0);
      split_bf16(v.y * p.qscale, h1, l1);
      split_bf16(v.z * p.qscale, h2, l2);
      split_bf16(v.w * p.qscale, h3, l3);
      hv[e] = s16x4{(short)h0, (short)h1, (short)h2, (short)h3};
      lv[e] = s16x4{(short)l0, (short)l1, (short)l2, (short)l3};
    }
    qh[k] = join_bf16x8(hv[0], hv[1]);
    ql[k] = join_bf16x8(lv[0], lv[1]);
  }

  float* rv = rowv + wave * 32;
  // transpose-read offset of the value part: lane L reads 4 columns
  // 32s + 16*((L/16)%2) + 4*(L%4) of row 8k + 4*(L/32) + (L%16)/4; the
  // 16-lane transpose leaves lane l with column 32s + l%32 of rows
  // 8k + 4*(l/32) .. +3
  const int tr_off = kMTile * S::SP + (4 * (lane >> 5) + ((lane & 15) >> 2)) * S::VP +
                     (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  f32x16 acc[S::NCT];
#pragma unroll
  for (int s = 0; s < S::NCT; ++s) acc[s] = f32x16{0};
  float m_ref = kNegInf, l_half = 0.f;

  // one tile: into LDS from its stage, then the stage takes tile it + 2
  auto tile = [&](int it, uint4 (&st)[CPT]) {
    char* buf = tiles + (it & 1) * S::TILE;
    store_tile(st, buf);
    __syncthreads();
    const int tb = t_begin + it * kMTile;
    load_tile(st, tb + 2 * kMTile);

    // scores of the tile, transposed: S^T = K_h . Q_h^T with the K rows as
    // the A operand and Q (registers) as the B operand, one 32-row block at a
    // time.  The result layout leaves lane l with query l%32 at context rows
    // 32b + 8k + 4*hh + j (block b, register 4k + j), which is exactly the
    // A-operand layout of P . V below.
    float v[kMBlocks][16];
#pragma unroll
    for (int b = 0; b < kMBlocks; ++b) {
      f32x16 sc = f32x16{0};
      const char* srow = buf + (kMRows * b + m) * S::SP + hh * DH;  // context row, this half's dimensions
#pragma unroll
      for (int k = 0; k < DH / 16; ++k) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(srow + 16 * k);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[k], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ql[k], sc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) v[b][i] = sc[i];
    }
    // rows past a query's limit (or the split) are -inf; only tiles that
    // cross a limit of this wave need the per-element test
    if (__builtin_amdgcn_ballot_w64(tb + kMTile > min(lim, t_end)) != 0) {
#pragma unroll
      for (int b = 0; b < kMBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = kMRows * b + 8 * (i >> 2) + 4 * hh + (i & 3);
          v[b][i] = (tb + t < min(lim, t_end)) ? v[b][i] : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < kMBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, v[b][i]);
    mx = pair_max(mx);
    const bool up = mx > m_ref + kMultiSlack;
    if (__builtin_amdgcn_ballot_w64(up)) {  // some row moves its reference: rescale through LDS
      const float nref = up ? mx : m_ref;
      const float alpha = up ? (m_ref == kNegInf ? 0.f : fast_exp2(m_ref - nref)) : 1.f;
      if (hh == 0) rv[m] = alpha;
      l_half *= alpha;
      m_ref = nref;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = rv[8 * (i >> 2) + 4 * hh + (i & 3)];
#pragma unroll
        for (int s = 0; s < S::NCT; ++s) acc[s][i] *= a;
      }
    }
    // weights 2^(s - m) rounded to bf16 (hardware pack), and the normaliser
    // summed from the same rounded weights the MFMA uses; m is finite once
    // any score of the row was, masked scores give 0 either way
    const float mu = fmaxf(m_ref, -__FLT_MAX__);
    s16x4 pa[kMBlocks][4];
#pragma unroll
    for (int b = 0; b < kMBlocks; ++b)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x2_t p01 = {(__bf16)fast_exp2(v[b][4 * k] - mu), (__bf16)fast_exp2(v[b][4 * k + 1] - mu)};
        const bf16x2_t p23 = {(__bf16)fast_exp2(v[b][4 * k + 2] - mu), (__bf16)fast_exp2(v[b][4 * k + 3] - mu)};
        const uint32_t w0 = __builtin_bit_cast(uint32_t, p01), w1 = __builtin_bit_cast(uint32_t, p23);
        l_half = dot2_bf16(w1, kOnes2, dot2_bf16(w0, kOnes2, l_half));
        pa[b][k] = __builtin_bit_cast(s16x4, make_uint2(w0, w1));
      }
    // P . value block, 16 context rows per MFMA
#pragma unroll
    for (int k = 0; k < 2 * kMBlocks; ++k) {
      const bf16x8_t a = join_bf16x8(pa[k >> 1][2 * (k & 1)], pa[k >> 1][2 * (k & 1) + 1]);
      const lds_s16x4_m* r0 =
          (const lds_s16x4_m*)(size_t)((uint32_t)(uintptr_t)(buf + tr_off) + (uint32_t)(16 * k * S::VP));
      const lds_s16x4_m* r1 =
          (const lds_s16x4_m*)(size_t)((uint32_t)(uintptr_t)(buf + tr_off) + (uint32_t)((16 * k + 8) * S::VP));
#pragma unroll
      for (int s = 0; s < S::NCT; ++s) {
        const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4_m*>(r0 + 8 * s));
        const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4_m*>(r1 + 8 * s));
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, join_bf16x8(b0, b1), acc[s], 0, 0, 0);
      }
    }
  };
  for (int it = 0; it + 1 < ntiles; it += 2) {
    tile(it, stage[0]);
    tile(it + 1, stage[1]);
  }
  if (ntiles & 1) tile(ntiles - 1, stage[0]);

  const float l_row = pair_sum(l_half);
  const int qbase = (qg * QW + wave) * 32;
  if constexpr (OPT == 2) {
    const int slot_of = p.nsplit;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * hh + (i & 3), qq = qbase + r;
      if (qq >= p.n) continue;
      float* dst = p.U + ((size_t)h * p.nslots + (size_t)qq * slot_of + split) * d;
#pragma unroll
      for (int s = 0; s < S::NCT; ++s) {
        const int col = c0 + 32 * s + m;
        if (col < d) dst[col] = acc[s][i];
      }
    }
    if (blockIdx.x == 0 && hh == 0 && qok) {
      float* mls = p.ml + (size_t)(q * slot_of + split) * 2 * p.H;
      mls[h] = m_ref;
      mls[p.H + h] = l_row;
    }
  } else if (p.nsplit > 1) {  // option 1 over context splits: partial rows [h][slot][DH], m, l
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * hh + (i & 3), qq = qbase + r;
      if (qq >= p.n) continue;
      float* dst = p.U + ((size_t)h * p.nslots + (size_t)qq * p.nsplit + split) * DH;
#pragma unroll
      for (int s = 0; s < S::NCT; ++s) dst[32 * s + m] = acc[s][i];
    }
    if (hh == 0 && qok) {
      float* mls = p.ml + (size_t)(q * p.nsplit + split) * 2 * p.H;
      mls[h] = m_ref;
      mls[p.H + h] = l_row;
    }
  } else {
    __syncthreads();  // rv is reused for the normalisers
    if (hh == 0) rv[m] = l_row;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * hh + (i & 3), qq = qbase + r;
      if (qq >= p.n) continue;
      const float lr = rv[r];
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      float* dst = p.out + ((size_t)qq * p.H + h) * DH;
#pragma unroll
      for (int s = 0; s < S::NCT; ++s) dst[32 * s + m] = acc[s][i] * inv;
    }
  }
}

// Option 1 over context splits: out[q, h, j] = sum_s 2^(m_s - m*) U_s[h, j] /
// sum_s 2^(m_s - m*) l_s (log-sum-exp merge of the splits), zero for a query
// with no rows.
__global__ void __launch_bounds__(256) multi_merge_kernel(const float* __restrict__ U,
                                                          const float* __restrict__ ml,
                                                          float* __restrict__ out, int n, int H, int dh,
                                                          int ns, int nslots) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)n * H * dh) return;
  const int j = (int)(i % dh), h = (int)((i / dh) % H), q = (int)(i / ((long long)dh * H));
  float mx = kNegInf;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, ml[(size_t)(q * ns + s) * 2 * H + h]);
  float num = 0.f, den = 0.f;
  if (mx > kNegInf) {
    for (int s = 0; s < ns; ++s) {
      const float* mls = ml + (size_t)(q * ns + s) * 2 * H;
      const float w = fast_exp2(mls[h] - mx);
      den = fmaf(w, mls[H + h], den);
      num = fmaf(w, U[((size_t)h * nslots + (size_t)q * ns + s) * dh + j], num);
    }
  }
  out[i] = den > 0.f ? num / den : 0.f;
}

template <int DH, int QW, int OPT>
static hipError_t launch_mq(const MultiPlan& pl, const MultiParams& mp, hipStream_t s) {
  using S = MultiShape<DH, QW, OPT>;
  const size_t lds = 2 * (size_t)S::TILE + (size_t)QW * 32 * 4;
  auto kern = multi_attend_kernel<DH, QW, OPT>;
  static std::atomic<int> granted[kMaxDevices];
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern), lds, granted);
  if (e != hipSuccess) return e;
  const int nqg = (mp.n + 32 * QW - 1) / (32 * QW);
  const int ncb = OPT == 2 ? (mp.d + S::NCW - 1) / S::NCW : 1;
  hipLaunchKernelGGL(kern, dim3(ncb, mp.H * nqg, pl.nsplit), dim3(64 * QW), lds, s, mp);
  return hipGetLastError();
}

template <int DH, int OPT>
static hipError_t launch_mq_qw(const MultiPlan& pl, const MultiParams& mp, hipStream_t s) {
  switch (pl.qw) {
    case 1: return launch_mq<DH, 1, OPT>(pl, mp, s);
    case 2: return launch_mq<DH, 2, OPT>(pl, mp, s);
    case 4: return launch_mq<DH, 4, OPT>(pl, mp, s);
  }
  return hipErrorInvalidValue;
}

bool make_multi_plan(int n, int H, int dh, int T, int method, bool w_bf16, int ncu, MultiPlan* p) {
  const long long d = (long long)H * dh;
  if (n <= 0 || H <= 0 || T <= 0 || (dh != 64 && dh != 128) || d % 128 != 0 || d > 65536) return false;
  if (method == 0) {  // multiply-accumulate counts of the two options
    const double o1 = (double)T * d * d + (double)n * T * d;
    const double o2 = (double)n * H * T * d + (double)n * d * d;
    method = o1 < o2 ? 1 : 2;
  }
  if (method == 1 && !w_bf16) return false;  // V = K.W_KV is formed by the bf16 MFMA product
  p->method = method;
  p->qw = n > 64 ? 4 : (n > 32 ? 2 : 1);
  const long long nqg = (n + 32LL * p->qw - 1) / (32LL * p->qw);
  const long long ncb = method == 2 ? (d + 127) / 128 : 1;
  const long long wgs = ncb * H * nqg;
  // split the context while the grid is below two workgroups per compute unit
  int nsplit = 1;
  while (wgs * nsplit * 2 <= 2LL * ncu && (long long)nsplit * 2 * kMRows * 4 <= T) nsplit *= 2;
  p->nsplit = nsplit;
  p->Ts = ((T + nsplit - 1) / nsplit + kMRows - 1) / kMRows * kMRows;
  p->nsplit = (T + p->Ts - 1) / p->Ts;
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += (b + 255) & ~(size_t)255;
    return o;
  };
  p->fin = DecodePlan{};
  if (method == 2) {
    p->fin.nslots = n * p->nsplit;
    const int big = proj_rows(dh, true);
    p->fin.spw = finish_seqs(H, (d + big - 1) / big, n, ncu);
    const long long grid = (long long)H * ((d + big - 1) / big) * ((n + p->fin.spw - 1) / p->fin.spw);
    p->fin.proj_rows = grid * 2 >= ncu ? big : proj_rows(dh, false);
    p->fin.npc = (int)((d + p->fin.proj_rows - 1) / p->fin.proj_rows);
    p->fin.nch = 1;
    p->fin.off_U = take((size_t)H * p->fin.nslots * d * sizeof(float));
    p->fin.off_ml = take((size_t)p->fin.nslots * 2 * H * sizeof(float));
    p->fin.off_op = take((size_t)p->fin.npc * n * H * dh * sizeof(float));
    p->off_v = 0;
  } else {
    p->off_v = take((size_t)T * d * sizeof(uint16_t));
    if (p->nsplit > 1) {
      p->fin.nslots = n * p->nsplit;
      p->fin.off_U = take((size_t)H * p->fin.nslots * dh * sizeof(float));
      p->fin.off_ml = take((size_t)p->fin.nslots * 2 * H * sizeof(float));
    }
  }
  p->bytes = off;
  return true;
}

hipError_t launch_multi(const MultiPlan& pl, const float* Q, const void* K, const int32_t* limits,
                        const void* W, bool w_bf16, float* out, int n, int H, int dh, int T, float scale,
                        char* ws, hipStream_t s) {
  const int d = H * dh;
  MultiParams mp{};
  mp.Q = Q;
  mp.K = static_cast<const uint16_t*>(K);
  mp.limits = limits;
  mp.n = n;
  mp.H = H;
  mp.d = d;
  mp.T = T;
  mp.nsplit = pl.nsplit;
  mp.Ts = pl.Ts;
  mp.qscale = scale * kLog2e;
  hipError_t e;
  if (pl.method == 1) {
    uint16_t* V = reinterpret_cast<uint16_t*>(ws + pl.off_v);
    e = launch_prefill_bf16(K, W, V, 1, T, d, T, nullptr, s);  // V = K . W_KV, rounded to bf16
    if (e != hipSuccess) return e;
    mp.Vs = V;
    mp.out = out;
    if (pl.nsplit > 1) {
      mp.U = reinterpret_cast<float*>(ws + pl.fin.off_U);
      mp.ml = reinterpret_cast<float*>(ws + pl.fin.off_ml);
      mp.nslots = pl.fin.nslots;
    }
    e = dh == 64 ? launch_mq_qw<64, 1>(pl, mp, s) : launch_mq_qw<128, 1>(pl, mp, s);
    if (e != hipSuccess || pl.nsplit == 1) return e;
    const long long tot = (long long)n * H * dh;
    hipLaunchKernelGGL(multi_merge_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s,
                       (const float*)mp.U, (const float*)mp.ml, out, n, H, dh, pl.nsplit, pl.fin.nslots);
    return hipGetLastError();
  }
  mp.Vs = mp.K;
  mp.U = reinterpret_cast<float*>(ws + pl.fin.off_U);
  mp.ml = reinterpret_cast<float*>(ws + pl.fin.off_ml);
  mp.nslots = pl.fin.nslots;
  e = dh == 64 ? launch_mq_qw<64, 2>(pl, mp, s) : launch_mq_qw<128, 2>(pl, mp, s);
  if (e != hipSuccess) return e;
  DecodeArgs a{};
  a.q = Q;
  a.K = K;
  a.lengths = nullptr;
  a.W = W;
  a.out = out;
  a.B = n;
  a.H = H;
  a.dh = dh;
  a.d = d;
  a.T_max = T;
  a.nslots = pl.fin.nslots;
  a.scale = scale;
  a.w_bf16 = w_bf16;
  a.ws = ws;
  return launch_finish_fixed(pl.fin, a, pl.nsplit, s);
}

}  // namespace slim
