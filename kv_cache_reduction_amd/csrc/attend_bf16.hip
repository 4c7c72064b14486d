// Slim-Attention decode, attend phase, bf16 K cache: streams the K cache
// once and, per token chunk, forms scores, the online softmax and the
// softmax-times-K contraction of every head over all d columns (Slim
// Attention article, localbendi.com, section "K-Cache is All You Need",
// generation step, second option: softmax result times K first, W_KV later).
//
// Work decomposition (gfx950, wave64, two waves per SIMD):
//  * The live rows of all sequences, concatenated, are cut into `nch` token
//    chunks.  Each chunk is handled by `gc` workgroups (column groups of `dc`
//    columns of K).  A workgroup's accumulator is 32 head rows x dc columns
//    in fp32: 128 registers in each of its dc/256 waves.
//  * Wave w owns one 256-column unit of its column group.  Per 8-token step
//    each lane needs 4 tokens x 8 columns of the unit, exactly the register
//    layout of the MFMA B operand (lane l: columns 8*(l%32)..+7 of tokens
//    4*(l/32)..+3).  These bytes travel HBM -> LDS by buffer_load ... lds
//    (16 bytes per lane, two 512-byte contiguous segments per instruction)
//    into a ring private to the wave, `NST` steps ahead, so the registers
//    only hold the step being computed.  The wave waits for its own ring
//    slot with an explicit vmcnt; no other wave touches it.  Buffer
//    resources bound each load to the piece's live rows, so the ragged tail
//    reads as zeros without branches.
//  * Scores come from the same registers: 8 fp32 FMAs per token per lane,
//    then a DPP sum over the dh/8 lanes that share a head.  With gc == 2 each
//    wave also loads the matching units of the other column group, for the
//    scores only (every workgroup needs the softmax of all heads; the second
//    read of a tile is meant to hit the XCD's L2).
//  * Scores of all heads meet in a small double-buffered LDS array behind one
//    barrier per step.  Every wave then runs the online softmax of all 32
//    head rows (lane l: head l%32, tokens 4*(l/32)..+3, the MFMA A-operand
//    layout), rounds the weights to bf16 and issues one 32x32 bf16 MFMA per 32
//    output columns with B operands built by byte permutes (a 4x8 -> 8x4
//    transpose of 16-bit values in registers).
//  * Lazy rescaling: each head keeps a reference max m (log2 units) and the
//    accumulator holds sum_t 2^(s_t - m) K[t]; m only moves (and the
//    accumulator rows are rescaled) when a score exceeds it by more than 8,
//    so weights stay below 2^8 and the rescale is rare.
//  * Per piece (chunk x sequence) the workgroup writes its unnormalised
//    accumulator U[slot, h, cols] and (column group 0) m and the normaliser
//    l of every head.  q is pre-scaled by scale*log2(e); exponentials use
//    v_exp_f32.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

namespace slim {

struct AttendBf16Params {
  const float* q;
  const uint16_t* K;
  const int32_t* lengths;
  float* U;
  float* ml;
  int B, H, d, T_max, nch, dc, nslots;
  float qscale;
};

constexpr float kRescaleSlack = 8.f;  // log2 units

__device__ __forceinline__ float dot8(const float4& qa, const float4& qb, const uint4& k) {
  float s = qa.x * bf_lo(k.x);
  s = fmaf(qa.y, bf_hi(k.x), s);
  s = fmaf(qa.z, bf_lo(k.y), s);
  s = fmaf(qa.w, bf_hi(k.y), s);
  s = fmaf(qb.x, bf_lo(k.z), s);
  s = fmaf(qb.y, bf_hi(k.z), s);
  s = fmaf(qb.z, bf_lo(k.w), s);
  s = fmaf(qb.w, bf_hi(k.w), s);
  return s;
}

// q . k over 8 columns: q as packed bf16 hi/lo pairs (4 words each), k as
// 8 bf16 in 4 words; two dot2 per column pair.
__device__ __forceinline__ float dot8_split(const uint4& qh, const uint4& ql, const uint4& k) {
  float s = dot2_bf16(k.x, qh.x, 0.f);
  s = dot2_bf16(k.x, ql.x, s);
  s = dot2_bf16(k.y, qh.y, s);
  s = dot2_bf16(k.y, ql.y, s);
  s = dot2_bf16(k.z, qh.z, s);
  s = dot2_bf16(k.z, ql.z, s);
  s = dot2_bf16(k.w, qh.w, s);
  s = dot2_bf16(k.w, ql.w, s);
  return s;
}

__device__ __forceinline__ void split_q8(const float* qp, float scale, uint4& hi, uint4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_bf16(qp[i] * scale, h[i], l[i]);
  hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}

// Scores of 4 tokens (this lane's half-step) for the head owning this lane's
// 8 columns, written to Sb[head][4*half + t].
template <int DH>
__device__ __forceinline__ void head_scores(const uint4& qh, const uint4& ql, const uint4 (&D)[4], bool ok,
                                            int col, int lane, int half, float* Sb) {
  constexpr int LPH = DH / 8;
  float v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = dot8_split(qh, ql, D[k]);
  if constexpr (LPH == 16) {
    const float x = row16_sum4(v[0], v[1], v[2], v[3], lane);
    const int r = lane & 15;
    if (ok && r < 4) Sb[(col / DH) * 8 + half * 4 + 2 * (r & 1) + (r >> 1)] = x;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = group_sum<LPH>(v[k]);
    if (ok && ((lane & 31) % LPH) == 0)
      *reinterpret_cast<float4*>(Sb + (col / DH) * 8 + half * 4) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// acc[s] += P (32 heads x 8 tokens, A layout: lane l = head l%32, tokens
// 4*(l/32)..+3 packed in w0, w1) times K (8 tokens x 256 columns held as
// D[k] = 8 columns of token 4*(l/32)+k).  Column 8*(l%32) + s of the unit is
// MFMA s's output column l%32.  On gfx950 the 32x32x16 instruction runs at
// twice the rate of 32x32x8, so the 8 tokens fill half of its K=16 and the
// other half is zero.
#ifndef SLIM_MFMA_K8
__device__ __forceinline__ void mfma_pk(f32x16 (&acc)[8], uint32_t w0, uint32_t w1, const uint4 (&D)[4]) {
  const uint4 aw = make_uint4(w0, w1, 0u, 0u);
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, aw);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint32_t sel = (s & 1) ? kSelHi : kSelLo;
    const int wd = s >> 1;
    const uint4 bw = make_uint4(perm(word(D[1], wd), word(D[0], wd), sel),
                                perm(word(D[3], wd), word(D[2], wd), sel), 0u, 0u);
    acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bw), acc[s], 0, 0, 0);
  }
}
#else
__device__ __forceinline__ void mfma_pk(f32x16 (&acc)[8], uint32_t w0, uint32_t w1, const uint4 (&D)[4]) {
  uint2 aw = make_uint2(w0, w1);
  const s16x4 a = *reinterpret_cast<s16x4*>(&aw);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint32_t sel = (s & 1) ? kSelHi : kSelLo;
    const int wd = s >> 1;
    uint2 bw;
    bw.x = perm(word(D[1], wd), word(D[0], wd), sel);
    bw.y = perm(word(D[3], wd), word(D[2], wd), sel);
    const s16x4 bv = *reinterpret_cast<s16x4*>(&bw);
    acc[s] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, bv, acc[s], 0, 0, 0);
  }
}
#endif

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor (V#) for a raw byte range; loads beyond `bytes` return 0.
__device__ __forceinline__ i32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = (int)(uint32_t)a;
  r.y = (int)((uint32_t)(a >> 32) & 0xffffu);  // stride 0
  r.z = (int)bytes;
  r.w = 0x00020000;
  r.x = __builtin_amdgcn_readfirstlane(r.x);
  r.y = __builtin_amdgcn_readfirstlane(r.y);
  r.z = __builtin_amdgcn_readfirstlane(r.z);
  return r;
}

// One 16-byte-per-lane load from a buffer straight into LDS: lane i's bytes
// land at LDS byte address lds + 16*i.  Written as inline asm so that the
// compiler does not drain the vector-memory counter at every workgroup
// barrier (it treats LDS DMA as pending LDS stores); the kernel waits for
// each ring slot itself with wait_vmcnt.
__device__ __forceinline__ void dma16(uint32_t lds, const i32x4& rsrc, uint32_t voff) {
  // `lds` and `rsrc` are wave-uniform; readfirstlane places them in SGPRs
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

template <int DH, int GC, int NST>
__global__ void __launch_bounds__(512) attend_bf16_kernel(AttendBf16Params p) {
  constexpr int LPH = DH / 8;          // lanes per head in a 32-lane half
  constexpr int LPS = GC == 2 ? 8 : 4; // DMA instructions per step and wave
  constexpr int SB = LPS * 1024;       // ring slot bytes per wave
  extern __shared__ __attribute__((aligned(16))) int smem[];
  const int nw = blockDim.x >> 6;
  char* ring = reinterpret_cast<char*>(smem);                        // [nw][NST][SB]
  float* S = reinterpret_cast<float*>(ring + (size_t)nw * NST * SB);  // [2][32][8]
  int* tmp = reinterpret_cast<int*>(S + 512);                         // [16]
  int* pre = tmp + 16;                                                // [B+1]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  int c, cg;
  {
    const int bid = blockIdx.x;
    if (GC == 2 && (p.nch & 7) == 0) {
      // the two column groups of a chunk land on the same XCD (workgroups
      // are dealt round-robin over the 8 XCDs) so the second read of each
      // K tile can hit that XCD's L2
      const int xcd = bid & 7, k = bid >> 3;
      cg = k & 1;
      c = ((k >> 1) << 3) + xcd;
    } else {
      c = bid / GC;
      cg = bid % GC;
    }
  }

  lengths_prefix(p.lengths, p.B, p.T_max, pre, tmp);
  const int total = pre[p.B];
  if (total == 0) return;
  const int Ts = chunk_tokens(total, p.nch);
  const int cbeg = c * Ts;
  if (cbeg >= total) return;
  const int cend = min(total, cbeg + Ts);

  const int d = p.d;
  const int ub = wave * kMfmaUnitCols + 8 * l32;
  const int ocol = cg * p.dc + ub;
  const bool ook = ocol < min(d, (cg + 1) * p.dc);
  const int xcol = (1 - cg) * p.dc + ub;
  const bool xok = GC == 2 && xcol < min(d, (2 - cg) * p.dc);
  const bool score_lane = (l32 % LPH) == 0;
  const bool head_ok = l32 < p.H;
  const uint32_t ring_w = (uint32_t)reinterpret_cast<uintptr_t>(ring + (size_t)wave * NST * SB);
  const uint4* ring_rd = reinterpret_cast<const uint4*>(ring + (size_t)wave * NST * SB) + lane;

  int gstep = 0;  // step counter across pieces: parity selects the S buffer
  for (int b = seq_of(pre, p.B, cbeg); b < p.B && pre[b] < cend; ++b) {
    const int s0 = pre[b], s1 = pre[b + 1];
    if (s1 == s0) continue;
    const int tb = max(cbeg, s0) - s0;
    const int n = min(cend, s1) - s0 - tb;
    const int slot = c + b;

    uint4 qoh, qol, qxh, qxl;  // scaled query, bf16 hi/lo pairs, own and other unit
    {
      const float* qb = p.q + (size_t)b * d;
      split_q8(qb + (ook ? ocol : 0), p.qscale, qoh, qol);
      split_q8(qb + (xok ? xcol : 0), p.qscale, qxh, qxl);
    }

    const uint32_t nbytes = (uint32_t)n * (uint32_t)d * 2u;
    const i32x4 rs = buffer_desc(p.K + ((size_t)b * p.T_max + tb) * d, nbytes);
    // byte offset of this lane's row 4*half of step 0; columns outside the
    // column range point past the resource and read as zero
    const uint32_t row_bytes = (uint32_t)d * 2u;
    const uint32_t step_bytes = row_bytes * kStepTokens;
    const uint32_t ooff = ook ? ((uint32_t)(half * 4) * d + ocol) * 2u : nbytes;
    const uint32_t xoff = xok ? ((uint32_t)(half * 4) * d + xcol) * 2u : nbytes;
    const uint32_t ostep = ook ? step_bytes : 0u, xstep = xok ? step_bytes : 0u;

    auto issue = [&](int step, int stage) {
      const uint32_t dst = ring_w + stage * SB;
#pragma unroll
      for (int k = 0; k < 4; ++k) dma16(dst + k * 1024, rs, ooff + step * ostep + k * row_bytes);
      if (GC == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) dma16(dst + 4096 + k * 1024, rs, xoff + step * xstep + k * row_bytes);
      }
    };

    float m_ref = kNegInf, l_run = 0.f;  // head l32 (both halves hold copies)
    f32x16 acc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[s] = f32x16{0};

    const int nsteps = (n + kStepTokens - 1) / kStepTokens;
#pragma unroll
    for (int s = 0; s < NST; ++s) issue(s, s);  // steps past the end read zeros

    for (int st = 0; st < nsteps; ++st) {
      const int stage = st % NST;
      wait_vmcnt<(NST - 1) * LPS>();
      uint4 ko[4], kx[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) ko[k] = ring_rd[(stage * SB + k * 1024) / 16];
      if (GC == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) kx[k] = ring_rd[(stage * SB + 4096 + k * 1024) / 16];
      }
      wait_lgkmcnt0();
      issue(st + NST, stage);

      float* Sb = S + (gstep & 1) * 256;
      ++gstep;
      // 1. scores of the heads whose columns this lane holds
      head_scores<DH>(qoh, qol, ko, ook, ocol, lane, half, Sb);
      if (GC == 2) head_scores<DH>(qxh, qxl, kx, xok, xcol, lane, half, Sb);
      __syncthreads();

      // 2. online softmax, head l32, tokens 4*half..+3 of the step
      const float4 sv = *reinterpret_cast<const float4*>(Sb + l32 * 8 + half * 4);
      float sc[4] = {sv.x, sv.y, sv.z, sv.w};
      const int t0 = st * kStepTokens + half * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (!head_ok || t0 + k >= n) sc[k] = kNegInf;
      float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const bool grow = mt > m_ref + kRescaleSlack;
      if (__any(grow)) {  // rare: move the reference max and rescale
        const float m_new = grow ? mt : m_ref;
        const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
        l_run *= alpha;
        m_ref = m_new;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float ar = __shfl(alpha, 8 * (e >> 2) + 4 * half + (e & 3), 64);
#pragma unroll
          for (int s = 0; s < 8; ++s) acc[s][e] *= ar;
        }
      }
      float pk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pk[k] = (m_ref == kNegInf) ? 0.f : fast_exp2(sc[k] - m_ref);
      const uint32_t w0 = pack_bf16x2(pk[0], pk[1]);
      const uint32_t w1 = pack_bf16x2(pk[2], pk[3]);
      float ps = (bf_lo(w0) + bf_hi(w0)) + (bf_lo(w1) + bf_hi(w1));
      ps += __shfl_xor(ps, 32, 64);
      l_run += ps;

      // 3. softmax weights (A: heads x tokens) times K (B: tokens x columns)
      mfma_pk(acc, w0, w1, ko);
    }
    wait_vmcnt<0>();  // the loads issued past the end have landed before the ring is reused

    // 4. partial results of this piece
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * half + (e & 3);
      if (ook && row < p.H) {
        float* dst = p.U + ((size_t)row * p.nslots + slot) * d + ocol;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0][e], acc[1][e], acc[2][e], acc[3][e]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4][e], acc[5][e], acc[6][e], acc[7][e]);
      }
    }
    if (cg == 0 && wave == 0 && lane < p.H) {
      p.ml[(size_t)slot * 2 * p.H + lane] = m_ref;
      p.ml[(size_t)slot * 2 * p.H + p.H + lane] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// Pair kernel (two column groups): each workgroup of a pair forms the scores
// of its own heads only (the heads whose columns lie in its column group)
// from its own half of K, and the pair exchange those scores through memory
// once per step; both then run the softmax of all heads and multiply by their
// own columns.  K is read once, and the score work is not duplicated.
//
// Step pipeline (step i, global step counter g):
//   [A] scores of step i+1 (registers D_next) -> S[(g+1)%3] own heads; the
//       loading waves wait for ring slot of step i+2.
//   barrier
//   [B] wave 0 publishes its heads' scores of step i+1 (write-through stores,
//       its own vmcnt(0), then the step flag) and waits for the partner's
//       scores of step i, which it copies into S[g%3]; the loading waves refill
//       the ring slot of step i+1 with step i+1+NST.
//   barrier
//   [C] online softmax of step i over all heads, MFMA with D_cur, then
//       D_cur <- D_next, D_next <- ring slot of step i+2.
// Wave 0 issues no ring loads (wave nw/2 loads its unit), so its vmcnt covers
// only its own exchange stores.  Flags carry a per-launch epoch in the high
// 32 bits; waits are bounded and a timeout is recorded in `err` and turns the
// outputs into NaN instead of hanging.
constexpr int kExchSlots = 4;
constexpr uint32_t kSpinLimit = 1u << 22;

struct PairParams {
  AttendBf16Params a;
  unsigned long long* flags;  // [nch][2]
  float* xbuf;                // [nch][2][kExchSlots][32][8]
  int* err;
  uint32_t epoch;
};

__device__ __forceinline__ void store_wt(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_wt(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DH, int NST>
__global__ void __launch_bounds__(512) attend_pair_kernel(PairParams pp) {
  static_assert(NST >= 3, "pipeline needs three ring slots");
  constexpr int LPH = DH / 8;
  constexpr int SB = 4 * 1024;  // one 256-column unit x 8 tokens per wave and slot
  const AttendBf16Params& p = pp.a;
  extern __shared__ __attribute__((aligned(16))) int smem[];
  const int nw = blockDim.x >> 6;
  char* ring = reinterpret_cast<char*>(smem);                         // [nw][NST][SB]
  float* S = reinterpret_cast<float*>(ring + (size_t)nw * NST * SB);  // [3][32][8]
  int* tmp = reinterpret_cast<int*>(S + 3 * 256);                // [16]
  int* pre = tmp + 16;                                           // [B+1]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  int c, cg;
  {
    const int bid = blockIdx.x;
    if ((p.nch & 7) == 0) {
      const int xcd = bid & 7, k = bid >> 3;
      cg = k & 1;
      c = ((k >> 1) << 3) + xcd;
    } else {
      c = bid >> 1;
      cg = bid & 1;
    }
  }
  unsigned long long* my_flag = pp.flags + (size_t)c * 2 + cg;
  const unsigned long long* pa_flag = pp.flags + (size_t)c * 2 + (1 - cg);
  float* my_x = pp.xbuf + ((size_t)c * 2 + cg) * kExchSlots * 256;
  const float* pa_x = pp.xbuf + ((size_t)c * 2 + (1 - cg)) * kExchSlots * 256;
  const unsigned long long ep = (unsigned long long)pp.epoch << 32;

  lengths_prefix(p.lengths, p.B, p.T_max, pre, tmp);
  const int total = pre[p.B];
  if (total == 0) return;
  const int Ts = chunk_tokens(total, p.nch);
  const int cbeg = c * Ts;
  if (cbeg >= total) return;
  const int cend = min(total, cbeg + Ts);

  const int d = p.d;
  const int own_lo = cg * p.dc, own_hi = min(d, (cg + 1) * p.dc);
  const int ocol = own_lo + wave * kMfmaUnitCols + 8 * l32;
  const bool ook = ocol < own_hi;
  // heads whose columns lie in this column group, and the partner's
  const int h_lo = own_lo / DH, h_hi = own_hi / DH;
  const bool score_lane = (l32 % LPH) == 0;
  const bool head_ok = l32 < p.H;
  // ring loads: wave w loads its own unit; wave nw/2 also loads wave 0's
  const bool loader = wave != 0;
  const bool extra = wave == (nw >> 1);
  const int ocol0 = own_lo + 8 * l32;  // wave 0's columns (for wave 4)
  const bool ook0 = ocol0 < own_hi;
  const uint32_t ring_w = (uint32_t)reinterpret_cast<uintptr_t>(ring + (size_t)wave * NST * SB);
  const uint32_t ring_0 = (uint32_t)reinterpret_cast<uintptr_t>(ring);
  const uint4* ring_rd = reinterpret_cast<const uint4*>(ring + (size_t)wave * NST * SB) + lane;

  unsigned long long gstep = 0;  // steps published so far across pieces
  bool failed = false;
  for (int b = seq_of(pre, p.B, cbeg); b < p.B && pre[b] < cend; ++b) {
    const int s0 = pre[b], s1 = pre[b + 1];
    if (s1 == s0) continue;
    const int tb = max(cbeg, s0) - s0;
    const int n = min(cend, s1) - s0 - tb;
    const int slot = c + b;

    uint4 qh, ql;
    split_q8(p.q + (size_t)b * d + (ook ? ocol : 0), p.qscale, qh, ql);
    const uint32_t nbytes = (uint32_t)n * (uint32_t)d * 2u;
    const i32x4 rs = buffer_desc(p.K + ((size_t)b * p.T_max + tb) * d, nbytes);
    const uint32_t row_bytes = (uint32_t)d * 2u;
    const uint32_t step_bytes = row_bytes * kStepTokens;
    // lanes whose columns lie outside the group start past the resource, so
    // every later row of theirs stays out of range too (offsets stay < 2^32)
    const uint32_t ooff = ook ? ((uint32_t)(half * 4) * d + ocol) * 2u : nbytes;
    const uint32_t ooff0 = ook0 ? ((uint32_t)(half * 4) * d + ocol0) * 2u : nbytes;
    auto issue = [&](int step) {
      const int stage = step % NST;
      const uint32_t sb = (uint32_t)step * step_bytes;
      if (loader) {
#pragma unroll
        for (int k = 0; k < 4; ++k) dma16(ring_w + stage * SB + k * 1024, rs, ooff + sb + k * row_bytes);
      }
      if (extra) {
#pragma unroll
        for (int k = 0; k < 4; ++k) dma16(ring_0 + stage * SB + k * 1024, rs, ooff0 + sb + k * row_bytes);
      }
    };
    // wait until the ring slot of step `ahead` steps before the newest issued one has landed
    auto wait_ring = [&]() {
      if (extra) wait_vmcnt<(NST - 2) * 8>();
      else if (loader) wait_vmcnt<(NST - 2) * 4>();
    };
    auto read_ring = [&](int step, uint4 (&D)[4]) {
      const int stage = step % NST;
#pragma unroll
      for (int k = 0; k < 4; ++k) D[k] = ring_rd[(stage * SB + k * 1024) / 16];
    };
    auto scores = [&](int step, const uint4 (&D)[4], float* Sb) {
      head_scores<DH>(qh, ql, D, ook, ocol, lane, half, Sb);
    };
    // wave 0: publish own heads' scores of a step, then fetch the partner's
    auto publish = [&](const float* Sb, unsigned long long g) {
      float* dst = my_x + (g % kExchSlots) * 256;
      for (int i = lane; i < (h_hi - h_lo) * 8; i += 64) store_wt(dst + h_lo * 8 + i, Sb[h_lo * 8 + i]);
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      if (lane == 0) __hip_atomic_store(my_flag, ep | (g + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto fetch = [&](float* Sb, unsigned long long g) {
      bool ok = true;
      if (lane == 0) {
        uint32_t spins = 0;
        for (;;) {
          const unsigned long long f = __hip_atomic_load(const_cast<unsigned long long*>(pa_flag),
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((f >> 32) == pp.epoch && (f & 0xffffffffull) >= g + 1) break;
          if (++spins >= kSpinLimit) {
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      ok = __shfl(ok ? 1 : 0, 0, 64) != 0;
      if (!ok) failed = true;
      const float* src = pa_x + (g % kExchSlots) * 256;
      for (int i = lane; i < 256; i += 64) {
        const int hh = i >> 3;
        if (hh < h_lo || hh >= h_hi) Sb[i] = ok ? load_wt(src + i) : __builtin_nanf("");
      }
    };

    float m_ref = kNegInf, l_run = 0.f;
    f32x16 acc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[s] = f32x16{0};
    const int nsteps = (n + kStepTokens - 1) / kStepTokens;

    // prologue: ring slots for steps 0..NST-1, scores of step 0, publish it
#pragma unroll
    for (int s = 0; s < NST; ++s) issue(s);
    wait_ring();
    __syncthreads();
    uint4 Dc[4], Dn[4];
    read_ring(0, Dc);
    read_ring(1, Dn);
    scores(0, Dc, S + (gstep % 3) * 256);
    __syncthreads();
    issue(NST);  // refill the slot of step 0
    if (wave == 0) publish(S + (gstep % 3) * 256, gstep);

    for (int st = 0; st < nsteps; ++st) {
      const unsigned long long g = gstep + st;
      float* Sc = S + (g % 3) * 256;
      float* Sn = S + ((g + 1) % 3) * 256;
      // [A]
      if (st + 1 < nsteps) scores(st + 1, Dn, Sn);
      wait_ring();
      __syncthreads();
      // [B]
      if (wave == 0) {
        if (st + 1 < nsteps) publish(Sn, g + 1);
        fetch(Sc, g);
      }
      issue(st + 1 + NST);
      __syncthreads();
      // [C] online softmax over all heads, tokens 4*half..+3 of step st
      const float4 sv = *reinterpret_cast<const float4*>(Sc + l32 * 8 + half * 4);
      float sc[4] = {sv.x, sv.y, sv.z, sv.w};
      const int t0 = st * kStepTokens + half * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (!head_ok || t0 + k >= n) sc[k] = kNegInf;
      float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const bool grow = mt > m_ref + kRescaleSlack;
      if (__any(grow)) {
        const float m_new = grow ? mt : m_ref;
        const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
        l_run *= alpha;
        m_ref = m_new;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float ar = __shfl(alpha, 8 * (e >> 2) + 4 * half + (e & 3), 64);
#pragma unroll
          for (int s = 0; s < 8; ++s) acc[s][e] *= ar;
        }
      }
      float pk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pk[k] = (m_ref == kNegInf) ? 0.f : fast_exp2(sc[k] - m_ref);
      const uint32_t w0 = pack_bf16x2(pk[0], pk[1]);
      const uint32_t w1 = pack_bf16x2(pk[2], pk[3]);
      float ps = (bf_lo(w0) + bf_hi(w0)) + (bf_lo(w1) + bf_hi(w1));
      ps += __shfl_xor(ps, 32, 64);
      l_run += ps;
      mfma_pk(acc, w0, w1, Dc);
#pragma unroll
      for (int k = 0; k < 4; ++k) Dc[k] = Dn[k];
      if (st + 2 < nsteps) read_ring(st + 2, Dn);
    }
    gstep += nsteps;
    if (loader) wait_vmcnt<0>();  // loads issued past the end have landed before the ring is reused
    __syncthreads();

    if (failed && lane == 0) atomicExch(pp.err, 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * half + (e & 3);
      if (ook && row < p.H) {
        float* dst = p.U + ((size_t)row * p.nslots + slot) * d + ocol;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0][e], acc[1][e], acc[2][e], acc[3][e]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4][e], acc[5][e], acc[6][e], acc[7][e]);
      }
    }
    if (cg == 0 && wave == 0 && lane < p.H) {
      p.ml[(size_t)slot * 2 * p.H + lane] = failed ? __builtin_nanf("") : m_ref;
      p.ml[(size_t)slot * 2 * p.H + p.H + lane] = l_run;
    }
  }
}

template <int DH, int GC>
static hipError_t launch_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  constexpr int NST = GC == 2 ? 2 : 4;
  constexpr int SB = (GC == 2 ? 8 : 4) * 1024;
  AttendBf16Params p;
  p.q = a.q;
  p.K = static_cast<const uint16_t*>(a.K);
  p.lengths = a.lengths;
  p.U = reinterpret_cast<float*>(a.ws + pl.off_U);
  p.ml = reinterpret_cast<float*>(a.ws + pl.off_ml);
  p.B = a.B;
  p.H = a.H;
  p.d = a.d;
  p.T_max = a.T_max;
  p.nch = pl.nch;
  p.dc = pl.dc;
  p.nslots = pl.nslots;
  p.qscale = a.scale * kLog2e;
  const size_t lds = (size_t)pl.nw * NST * SB + (512 + 16 + (size_t)a.B + 1) * sizeof(int);
  auto kern = attend_bf16_kernel<DH, GC, NST>;
  static int lds_allowed = 0;  // largest dynamic LDS size already granted to this kernel
  if ((int)lds > lds_allowed) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_allowed = (int)lds;
  }
  hipLaunchKernelGGL(kern, dim3(pl.nch * GC), dim3(pl.nw * 64), lds, s, p);
  return hipGetLastError();
}

// Per-launch epoch of the pair exchange flags: distinct for every launch of
// the process, starting from a value unlikely to match stale workspace bytes.
static uint32_t next_epoch() {
  static std::atomic<uint32_t> ctr{0x5a17c0deu ^ (uint32_t)(reinterpret_cast<uintptr_t>(&ctr) >> 4)};
  uint32_t e = ctr.fetch_add(1) + 1;
  return e == 0 ? 1 : e;
}

// Returns hipSuccess when the pair kernel was launched, hipErrorNotSupported
// when the plan or device does not allow it (the caller then uses the
// two-column-group kernel that recomputes all scores in each workgroup).
template <int DH>
static hipError_t launch_pair(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  constexpr int NST = 4;
  constexpr int SB = 4 * 1024;
  if (pl.gc != 2 || pl.nw < 2 || !pl.pair || env_int("SLIM_PAIR", 0) == 0) return hipErrorNotSupported;
  PairParams pp;
  AttendBf16Params& p = pp.a;
  p.q = a.q;
  p.K = static_cast<const uint16_t*>(a.K);
  p.lengths = a.lengths;
  p.U = reinterpret_cast<float*>(a.ws + pl.off_U);
  p.ml = reinterpret_cast<float*>(a.ws + pl.off_ml);
  p.B = a.B;
  p.H = a.H;
  p.d = a.d;
  p.T_max = a.T_max;
  p.nch = pl.nch;
  p.dc = pl.dc;
  p.nslots = pl.nslots;
  p.qscale = a.scale * kLog2e;
  pp.flags = reinterpret_cast<unsigned long long*>(a.ws + pl.off_flags);
  pp.xbuf = reinterpret_cast<float*>(a.ws + pl.off_x);
  pp.err = reinterpret_cast<int*>(a.ws + pl.off_err);
  pp.epoch = next_epoch();
  const size_t lds = (size_t)pl.nw * NST * SB + (3 * 256 + 16 + (size_t)a.B + 1) * sizeof(int);
  auto kern = attend_pair_kernel<DH, NST>;
  static int lds_allowed = 0;
  if ((int)lds > lds_allowed) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return hipErrorNotSupported;
    lds_allowed = (int)lds;
  }
  // the two workgroups of a pair wait on each other: they must be resident
  // together, which a cooperative launch guarantees (or refuses)
  void* args[] = {&pp};
  hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(pl.nch * 2),
                                            dim3(pl.nw * 64), args, (unsigned)lds, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the refusal
    return hipErrorNotSupported;
  }
  return hipSuccess;
}

hipError_t launch_attend_bf16(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  if (pl.gc == 1) {
    switch (a.dh) {
      case 32: return launch_t<32, 1>(pl, a, s);
      case 64: return launch_t<64, 1>(pl, a, s);
      case 128: return launch_t<128, 1>(pl, a, s);
    }
  } else {
    hipError_t e = hipErrorNotSupported;
    switch (a.dh) {
      case 32: e = launch_pair<32>(pl, a, s); break;
      case 64: e = launch_pair<64>(pl, a, s); break;
      case 128: e = launch_pair<128>(pl, a, s); break;
    }
    if (e != hipErrorNotSupported) return e;
    switch (a.dh) {
      case 32: return launch_t<32, 2>(pl, a, s);
      case 64: return launch_t<64, 2>(pl, a, s);
      case 128: return launch_t<128, 2>(pl, a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace slim
