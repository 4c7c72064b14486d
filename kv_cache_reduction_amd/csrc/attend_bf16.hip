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
//    (16 bytes per lane, two 512-byte contiguous segments per instruction,
//    non-temporal) into a ring private to the wave, `NST` steps ahead.  The
//    wave waits for its own ring slot with an explicit vmcnt; no other wave
//    touches it.  The buffer resource of each step starts at that step's
//    first row and ends at the piece's last live row, so the ragged tail and
//    the steps past the end read as zeros without branches.
//  * Scores come from the same registers: split-q dot2 products (q as bf16
//    high + low parts, so the products keep fp32 accuracy), then a DPP sum
//    over the dh/8 lanes that share a head.  With gc == 2 each wave also
//    loads the matching unit of the other column group, for the scores only
//    (every workgroup needs the softmax of all heads; the second read of a
//    tile mostly hits the XCD's L2).
//  * Software pipeline, one barrier per step: in iteration i a wave reads
//    the ring slot of step i+1, forms its heads' scores of step i+1 into the
//    LDS score buffer S[(i+1)%2], and meanwhile runs the online softmax of
//    step i from S[i%2] (written before the previous barrier) and the MFMAs
//    of step i with the registers it read one iteration earlier.  The
//    independent halves fill each other's latency.
//  * Online softmax: lane l handles head l%32, tokens 4*(l/32)..+3 (the MFMA
//    A-operand layout); weights are rounded to bf16 and one 32x32x8 bf16
//    MFMA per 32 output columns takes the step's 8 tokens; its B operand
//    comes from one transpose read (ds_read_b64_tr_b16) of the ring slot.
//  * Lazy rescaling: each head keeps a reference max m (log2 units) and the
//    accumulator holds sum_t 2^(s_t - m) K[t]; m only moves (and the
//    accumulator rows are rescaled) when a score exceeds it by more than 8,
//    so weights stay below 2^8 and the rescale is rare.
//  * Per piece (chunk x sequence) the workgroup writes its unnormalised
//    accumulator U[h, slot, cols] and (column group 0) m and the normaliser
//    l of every head.  q is pre-scaled by scale*log2(e); exponentials use
//    v_exp_f32.
#include <atomic>
#include <chrono>
#include <random>

#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace slim {

struct AttendBf16Params {
  const float* q;
  const uint16_t* K;
  const int32_t* lengths;
  void* U;           // partials: bf16 (ubf16) or fp32
  float* ml;
  uint32_t* status;  // cleared here; the finish sets it if a piece is marked failed
  int B, H, d, T_max, nch, dc, nslots;
  bool ubf16;
  float qscale;
};

constexpr float kRescaleSlack = 8.f;         // log2 units
constexpr uint32_t kOutOfRange = 0x80000000u;  // byte offset beyond any buffer resource used here
constexpr uint32_t kOnesBf16x2 = 0x3f803f80u;  // two bf16 1.0
constexpr uint32_t kQuietNaN = 0x7fc00000u;

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

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Buffer descriptor (V#) for a raw byte range; loads at offsets >= `bytes`
// return 0.
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

// One 16-byte-per-lane non-temporal load from a buffer straight into LDS:
// lane i's bytes land at LDS byte address lds + 16*i.  Written as inline asm
// so that the compiler does not drain the vector-memory counter at every
// workgroup barrier (it treats LDS DMA as pending LDS stores); the kernel
// waits for each ring slot itself with wait_vmcnt.  No register is written.
__device__ __forceinline__ void dma16(uint32_t lds, const i32x4& rsrc, uint32_t voff) {
  // `lds` and `rsrc` are wave-uniform; readfirstlane places them in SGPRs
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// The same with 4 bytes per lane (lane i's dword at lds + 4*i): needs only
// 4-byte alignment of the source.
__device__ __forceinline__ void dma4(uint32_t lds, const i32x4& rsrc, uint32_t voff) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Both halves of the wave see the pair (x of lane l, x of lane l^32):
// max / sum of the two equals the reduction over the two halves.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// A piece's partials: MFMA s, lane l, element e holds head
// 8*(e/4) + 4*(l/32) + e%4 at unit column 32s + l%32; columns at or past
// `clim` are not stored.  bf16 partials are rounded to nearest even once,
// here; the accumulation before and the merge after are fp32.
__device__ __forceinline__ void store_partials(const AttendBf16Params& p, const f32x16 (&acc)[8], int slot, int col,
                                               int clim, int half) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = 8 * (e >> 2) + 4 * half + (e & 3);
    if (row < p.H) {
      const size_t base = ((size_t)row * p.nslots + slot) * p.d + col;
      if (p.ubf16) {
        __bf16* dst = static_cast<__bf16*>(p.U) + base;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (col + 32 * s < clim) dst[32 * s] = (__bf16)acc[s][e];
      } else {
        float* dst = static_cast<float*>(p.U) + base;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (col + 32 * s < clim) dst[32 * s] = acc[s][e];
      }
    }
  }
}

template <int DH, int GC, int NST>
__global__ void __launch_bounds__(512) attend_bf16_kernel(AttendBf16Params p) {
  static_assert(NST >= 2 && (NST & (NST - 1)) == 0, "ring slots: a power of two, at least 2");
  constexpr int LPS = GC == 2 ? 8 : 4;  // DMA instructions per step and wave
  constexpr int SB = LPS * 1024;        // ring slot bytes per wave (own unit, then other unit)
  constexpr int WB = NST * SB;          // ring bytes per wave
  extern __shared__ __attribute__((aligned(16))) int smem[];
  const int nw = blockDim.x >> 6;
  char* ring = reinterpret_cast<char*>(smem);                     // [nw][NST][SB]
  float* S = reinterpret_cast<float*>(ring + (size_t)nw * WB);     // [2][32][8]
  float* qbuf = S + 512;                                           // [nw][GC][256] q of the units
  int* tmp = reinterpret_cast<int*>(qbuf + nw * GC * kMfmaUnitCols);  // [16]
  int* pre = tmp + 16;                                             // [B+1]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  if (blockIdx.x == 0 && tid == 0) *p.status = 0u;

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

  // score rows of heads >= H are never written and stay -inf (weight 0)
  for (int i = tid; i < 512; i += blockDim.x) S[i] = kNegInf;
  lengths_prefix(p.lengths, p.B, p.T_max, pre, tmp);  // (ends with a barrier)
  // values read from LDS are uniform here; readfirstlane keeps the step
  // arithmetic on the scalar unit
  const int total = __builtin_amdgcn_readfirstlane(pre[p.B]);
  if (total == 0) return;
  const int Ts = chunk_tokens(total, p.nch);
  const int cbeg = c * Ts;
  if (cbeg >= total) return;
  const int cend = min(total, cbeg + Ts);

  const int d = p.d;
  const int ubase = cg * p.dc + wave * kMfmaUnitCols;  // first column of this wave's unit
  const int clim = min(d, (cg + 1) * p.dc);            // end of this column group
  const int ocol = ubase + 8 * l32;
  const bool ook = ocol < clim;
  const int xcol = (1 - cg) * p.dc + wave * kMfmaUnitCols + 8 * l32;
  const bool xok = GC == 2 && xcol < min(d, (2 - cg) * p.dc);
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const uint32_t step_bytes = row_bytes * kStepTokens;
  // byte offset of this lane's first row within a step (row k adds k rows);
  // columns outside the column range read as zero
  const uint32_t vo = ook ? (uint32_t)(half * 4) * row_bytes + (uint32_t)ocol * 2u : kOutOfRange;
  const uint32_t vx = xok ? (uint32_t)(half * 4) * row_bytes + (uint32_t)xcol * 2u : kOutOfRange;
  // LDS: a slot holds the step's 8 rows x 256 columns of the own unit (and
  // then of the other unit), row t at (t%4)*1024 + (t/4)*512, column c at +2c
  // (the order the DMA writes them)
  char* wring = ring + (size_t)wave * WB;
  const uint32_t wring_s = (uint32_t)reinterpret_cast<uintptr_t>(wring);  // LDS byte address
  const uint4* rd16 = reinterpret_cast<const uint4*>(wring) + lane;
  // transpose read (ds_read_b64_tr_b16) feeding MFMA s its B operand: lane
  // L points at 4 columns 32s + 16*((L/16)%2) + 4*(L%4).. of row
  // 4*(L/32) + (L%16)/4; the 16-lane transpose then leaves output lane l with
  // column 32s + l%32 of rows 4*(l/32)..+3
  const int tr_off = ((lane & 15) >> 2) * 1024 + (lane >> 5) * 512 + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;

  int gstep = 0;  // step counter across pieces: parity selects the S buffer
  for (int b = __builtin_amdgcn_readfirstlane(seq_of(pre, p.B, cbeg)); b < p.B; ++b) {
    const int s0 = __builtin_amdgcn_readfirstlane(pre[b]), s1 = __builtin_amdgcn_readfirstlane(pre[b + 1]);
    if (s0 >= cend) break;
    if (s1 == s0) continue;
    const int tb = max(cbeg, s0) - s0;
    const int n = min(cend, s1) - s0 - tb;
    const int slot = c + b;

    uint4 qoh, qol, qxh, qxl;  // scaled query, bf16 hi/lo pairs, own and other unit (prologue)

    const uint16_t* kbase = p.K + ((size_t)b * p.T_max + tb) * d;
    const uint32_t nbytes = (uint32_t)n * row_bytes;  // < 2^31 (launch plan)
    // ring slot `sl` <- step `step`; the buffer resource runs from the step's
    // first row to the piece's end (rows past the piece, and whole steps
    // past it, read as zeros)
    auto issue = [&](int step, int sl) {
      const uint32_t done = (uint32_t)step * step_bytes;
      const uint32_t left = nbytes > done ? nbytes - done : 0u;
      const i32x4 rs = buffer_desc(reinterpret_cast<const char*>(kbase) + (left ? done : 0u), left);
      const uint32_t dst = wring_s + sl * SB;
#pragma unroll
      for (int k = 0; k < 4; ++k) dma16(dst + k * 1024, rs, vo + k * row_bytes);
      if (GC == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) dma16(dst + 4096 + k * 1024, rs, vx + k * row_bytes);
      }
    };
    // scores of the step in slot `sl` (own and other unit) -> Sb
    auto scores = [&](int sl, float* Sb) {
      uint4 ko[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) ko[k] = rd16[(sl * SB + k * 1024) / 16];
      head_scores<DH>(qoh, qol, ko, ook, ocol, lane, half, Sb);
      if (GC == 2) {
        uint4 kx[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) kx[k] = rd16[(sl * SB + 4096 + k * 1024) / 16];
        head_scores<DH>(qxh, qxl, kx, xok, xcol, lane, half, Sb);
      }
    };
    // MFMA B operands of the step in slot `sl`
    auto b_operands = [&](int sl, s16x4 (&bop)[8]) {
      const lds_s16x4* a0 = (const lds_s16x4*)(size_t)(wring_s + (uint32_t)(sl * SB + tr_off));
#pragma unroll
      for (int s = 0; s < 8; ++s) bop[s] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(a0 + 8 * s));
    };

    float m_ref = kNegInf, l_half = 0.f;  // head l32; l_half sums this half's tokens
    f32x16 acc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[s] = f32x16{0};

    const int nsteps = (n + kStepTokens - 1) / kStepTokens;
    // prologue: the wave's q columns (own unit, then the other) travel to
    // LDS by DMA with steps 0..NST-1; scores and B operands of step 0; step
    // NST refills slot 0.  (q by plain loads here would make the compiler
    // wait for the whole burst: it does not see the DMA.)
    s16x4 bcur[8];
    {
      float* qw = qbuf + wave * GC * kMfmaUnitCols;
      const uint32_t qs = (uint32_t)reinterpret_cast<uintptr_t>(qw);
      const float* qb = p.q + (size_t)b * d;
      const int ubeg = ubase, uend = clim;                    // own unit's columns [ubeg, min(ubeg + 256, uend))
      const i32x4 ro = buffer_desc(qb + ubeg, (uint32_t)max(0, min(kMfmaUnitCols, uend - ubeg)) * 4u);
#pragma unroll
      for (int k = 0; k < 4; ++k) dma4(qs + k * 256, ro, 4u * (uint32_t)(64 * k + lane));
      if (GC == 2) {
        const int xbeg = (1 - cg) * p.dc + wave * kMfmaUnitCols, xend = min(d, (2 - cg) * p.dc);
        const i32x4 rx = buffer_desc(qb + (xbeg < d ? xbeg : 0), (uint32_t)max(0, min(kMfmaUnitCols, xend - xbeg)) * 4u);
#pragma unroll
        for (int k = 0; k < 4; ++k) dma4(qs + 1024 + k * 256, rx, 4u * (uint32_t)(64 * k + lane));
      }
#pragma unroll
      for (int s = 0; s < NST; ++s) issue(s, s);
      wait_vmcnt<NST * LPS>();
      split_q8(qw + 8 * l32, p.qscale, qoh, qol);
      split_q8(qw + (GC == 2 ? 256 : 0) + 8 * l32, p.qscale, qxh, qxl);
    }
    wait_vmcnt<(NST - 1) * LPS>();
    scores(0, S + (gstep & 1) * 256);
    b_operands(0, bcur);
    wait_lgkmcnt0();
    issue(NST, 0);
    __syncthreads();

    for (int st = 0; st < nsteps; ++st) {
      float* Sc = S + ((gstep + st) & 1) * 256;
      float* Sn = S + ((gstep + st + 1) & 1) * 256;
      const int sl = (st + 1) & (NST - 1);
      // slot sl holds step st+1 (past the end: zeros); steps st+2.. may
      // still be in flight.  Scores and B operands of step st+1, then the
      // slot goes back in flight with step st+1+NST.  S[st+1] was last read
      // before the previous barrier.
      wait_vmcnt<(NST - 1) * LPS>();
      scores(sl, Sn);
      s16x4 bnext[8];
      b_operands(sl, bnext);

      // online softmax of step st: head l32, tokens 4*half..+3
      const float4 sv = *reinterpret_cast<const float4*>(Sc + l32 * 8 + half * 4);
      float sc[4] = {sv.x, sv.y, sv.z, sv.w};
      if ((st + 1) * kStepTokens > n) {  // ragged last step
        const int t0 = st * kStepTokens + half * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) sc[k] = t0 + k < n ? sc[k] : kNegInf;
      }
      wait_lgkmcnt0();
      issue(st + 1 + NST, sl);

      float ma, mb;
      halves(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), ma, mb);
      const float mt = fmaxf(ma, mb);
      const bool grow = mt > m_ref + kRescaleSlack;
      if (__any(grow)) {  // rare: move the reference max and rescale
        const float m_new = grow ? mt : m_ref;
        const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
        l_half *= alpha;
        m_ref = m_new;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float ar = __shfl(alpha, 8 * (e >> 2) + 4 * half + (e & 3), 64);
#pragma unroll
          for (int s = 0; s < 8; ++s) acc[s][e] *= ar;
        }
      }
      // m_ref is finite once any score of the head was finite; masked
      // scores (-inf) give weight 0 either way
      const float mu = fmaxf(m_ref, -__FLT_MAX__);
      const bf16x2_t p01 = {(__bf16)fast_exp2(sc[0] - mu), (__bf16)fast_exp2(sc[1] - mu)};
      const bf16x2_t p23 = {(__bf16)fast_exp2(sc[2] - mu), (__bf16)fast_exp2(sc[3] - mu)};
      const uint32_t w0 = __builtin_bit_cast(uint32_t, p01);
      const uint32_t w1 = __builtin_bit_cast(uint32_t, p23);
      l_half = dot2_bf16(w1, kOnesBf16x2, dot2_bf16(w0, kOnesBf16x2, l_half));

      // softmax weights (A: 32 heads x 8 tokens) times K (B: 8 tokens x 32
      // columns), MFMA s covering columns 32s..32s+31 of the unit
      {
        uint2 aw = make_uint2(w0, w1);
        const s16x4 a = __builtin_bit_cast(s16x4, aw);
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[s] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, bcur[s], acc[s], 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) bcur[s] = bnext[s];
      __syncthreads();
    }
    gstep += nsteps + 1;
    wait_vmcnt<0>();  // the loads issued past the end have landed before the ring is reused

    // partial results of this piece: MFMA s, lane l, element e holds head
    // 8*(e/4) + 4*(l/32) + e%4 at unit column 32s + l%32
    float la, lb;
    halves(l_half, la, lb);
    store_partials(p, acc, slot, ubase + l32, clim, half);
    if (cg == 0 && wave == 0 && lane < p.H) {
      p.ml[(size_t)slot * 2 * p.H + lane] = m_ref;
      p.ml[(size_t)slot * 2 * p.H + p.H + lane] = la + lb;
    }
  }
}

// ---------------------------------------------------------------------------
// Exchange kernel (two equal column groups, dh = 128): each workgroup forms
// the scores of its own 16 heads only, from its own columns, and the two
// workgroups of a chunk swap them through memory.  K is then read once and
// no score is computed twice.
//
// Scores of step j are formed kXchgLook steps ahead (in step j-3) and
// published as 64-bit mailbox entries {tag, score}; the 32-bit tag holds 24
// bits of a per-launch epoch (seeded at random per process, so stale
// entries left in reused memory by another launch or process do not match)
// and 8 bits of the entry's use count in its ring slot (step / 8: a slot
// holds step j only after step j-8, and the two workgroups of a pair stay
// within a few steps of each other).  A reader thus tells a fresh entry from
// an old one without any ordering between entries (relaxed agent-scope
// atomics: no fences, no drain of the DMA queue).  In step i a wave
//   1. starts the load (LDS DMA) of the partner's entries of step i+1,
//   2. forms and publishes its own heads' scores of step i+3,
//   3. reads the MFMA B operands of step i+1 and refills that ring slot with
//      step i+5,
//   4. runs the softmax and MFMAs of step i,
//   5. waits for the load of step 1 and copies the partner's entries of step
//      i+1 into the score buffer,
// then the workgroup meets at a barrier.  At the wait of step 5 the wave's
// vector-memory queue holds, oldest first: poll(i+1), publish(i+3), the 4
// loads of step i+5, so vmcnt(5) means poll(i+1) has landed, and with it
// the older ring loads (step i+4's, which step i+1 publishes from).  The
// partner published step i+1 two steps earlier.  A late partner is waited
// for with a bounded spin;
// running out of it marks the piece's results NaN.  Workgroups take their
// roles in arrival order (see the kernel), so the two of a pair are
// resident together without a cooperative launch.
constexpr int kXchgLook = 3;
constexpr int kMboxDepth = 8;                  // mailbox ring depth in steps
constexpr uint32_t kPollSpinLimit = 1u << 19;  // re-polls (about a second) before giving up
constexpr uint32_t kEpochMask = 0x7fffffu;     // 23 bits: a tag never has its top bit set

struct XchgParams {
  AttendBf16Params a;
  unsigned long long* mbox;     // [nch][2][kMboxDepth][8 waves][16] {tag, score}
  unsigned long long* tickets;  // arrival counter (any initial value)
  uint32_t epoch;               // kEpochMask bits used
  uint32_t spin_limit;          // re-polls of one wait before the piece is marked failed
  uint32_t pub_skew;            // testing: added to the epoch of column group 1's entries
};

__device__ __forceinline__ void dma16_sc1(uint32_t lds, const i32x4& rsrc, uint32_t voff) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen sc1 lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

template <int NST>
__global__ void __launch_bounds__(512) attend_xchg_kernel(XchgParams xp) {
  constexpr int DH = 128;
  constexpr int LPS = 4;            // DMA instructions per step and wave (own unit only)
  // a ring slot holds the 4 DMA slabs of a step (rows k and 4+k, 1 KB),
  // each padded by 64 bytes so that the 8 rows a transpose read touches do
  // not all start on the same LDS bank
  constexpr int SLAB = 1024 + 64;
  constexpr int SB = 4 * SLAB;      // ring slot bytes per wave
  constexpr int NS = 4;             // score buffers (steps i .. i+3)
  static_assert(NST == 4, "ring: slots of steps i+1 .. i+4");
  const AttendBf16Params& p = xp.a;
  extern __shared__ __attribute__((aligned(16))) int smem[];
  const int nw = blockDim.x >> 6;  // 8
  char* ring = reinterpret_cast<char*>(smem);                                 // [nw][NST][SB]
  float* S = reinterpret_cast<float*>(ring + (size_t)nw * NST * SB);           // [NS][32][8]
  unsigned long long* pollbuf = reinterpret_cast<unsigned long long*>(S + NS * 256);  // [nw][2][16]
  float* qbuf = reinterpret_cast<float*>(pollbuf + nw * 32);                    // [nw][256] q of each unit
  int* tmp = reinterpret_cast<int*>(qbuf + nw * kMfmaUnitCols);                 // [16]
  int* pre = tmp + 16;                                                          // [B+1]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  if (blockIdx.x == 0 && tid == 0) *p.status = 0u;
  // Roles by arrival: role = (ticket mod grid size); roles 2c and 2c+1 form
  // chunk c's pair.  Any gridDim.x consecutive tickets cover every role
  // once, whatever the counter held before, and a workgroup's partner is
  // the next or previous arrival (one pair wraps from the first arrival to
  // the last), so a resident workgroup never waits on one that cannot be
  // scheduled.  (Taken in wave 1, so that its round trip overlaps wave 0's
  // read of the lengths.)
  if (tid == 64)
    tmp[15] = (int)(__hip_atomic_fetch_add(xp.tickets, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) %
                    (unsigned long long)gridDim.x);
  for (int i = tid; i < NS * 256; i += blockDim.x) S[i] = kNegInf;
  lengths_prefix(p.lengths, p.B, p.T_max, pre, tmp);  // (ends with a barrier; leaves tmp[15])
  const int role = __builtin_amdgcn_readfirstlane(tmp[15]);
  const int c = role >> 1, cg = role & 1;
  const int total = __builtin_amdgcn_readfirstlane(pre[p.B]);
  if (total == 0) return;
  const int Ts = chunk_tokens(total, p.nch);
  const int cbeg = c * Ts;
  if (cbeg >= total) return;
  const int cend = min(total, cbeg + Ts);

  const int d = p.d;
  const int ubase = cg * p.dc + wave * kMfmaUnitCols;
  const int ocol = ubase + 8 * l32;
  const int xbase = (1 - cg) * p.dc + wave * kMfmaUnitCols;  // partner wave's unit
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const uint32_t step_bytes = row_bytes * kStepTokens;
  const uint32_t vo = (uint32_t)(half * 4) * row_bytes + (uint32_t)ocol * 2u;
  char* wring = ring + (size_t)wave * NST * SB;
  const uint32_t wring_s = (uint32_t)reinterpret_cast<uintptr_t>(wring);
  const uint4* rd16 = reinterpret_cast<const uint4*>(wring) + lane;
  const int tr_off = ((lane & 15) >> 2) * SLAB + (lane >> 5) * 512 + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;
  // mailbox entries: this wave publishes entry e = 8*(head within unit) + token
  unsigned long long* mine = xp.mbox + ((size_t)(2 * c + cg) * kMboxDepth * 8 + wave) * 16;
  const unsigned long long* theirs = xp.mbox + ((size_t)(2 * c + 1 - cg) * kMboxDepth * 8 + wave) * 16;
  const uint32_t poll_lds = (uint32_t)reinterpret_cast<uintptr_t>(pollbuf + wave * 32);
  const uint32_t qbuf_s = (uint32_t)reinterpret_cast<uintptr_t>(qbuf + wave * kMfmaUnitCols);
  const int r16 = lane & 15;
  const int pub_e = (l32 >> 4) * 8 + half * 4 + 2 * (r16 & 1) + (r16 >> 1);  // valid for r16 < 4
  const uint32_t ep = (xp.epoch & kEpochMask) << 8;
  const uint32_t ep_pub = ((xp.epoch + (cg ? xp.pub_skew : 0u)) & kEpochMask) << 8;
  bool failed = false;

  int gstep = 0;  // step counter across pieces (tags, score buffers)
  for (int b = __builtin_amdgcn_readfirstlane(seq_of(pre, p.B, cbeg)); b < p.B; ++b) {
    const int s0 = __builtin_amdgcn_readfirstlane(pre[b]), s1 = __builtin_amdgcn_readfirstlane(pre[b + 1]);
    if (s0 >= cend) break;
    if (s1 == s0) continue;
    const int tb = max(cbeg, s0) - s0;
    const int n = min(cend, s1) - s0 - tb;
    const int slot = c + b;

    uint4 qh, ql;  // split in the prologue, from the wave's q columns brought to LDS

    const uint16_t* kbase = p.K + ((size_t)b * p.T_max + tb) * d;
    const uint32_t nbytes = (uint32_t)n * row_bytes;
    auto issue = [&](int step) {  // ring slot step % NST <- step
      const uint32_t done = (uint32_t)step * step_bytes;
      const uint32_t left = nbytes > done ? nbytes - done : 0u;
      const i32x4 rs = buffer_desc(reinterpret_cast<const char*>(kbase) + (left ? done : 0u), left);
      const uint32_t dst = wring_s + (step & (NST - 1)) * SB;
#pragma unroll
      for (int k = 0; k < 4; ++k) dma16(dst + k * SLAB, rs, vo + k * row_bytes);
    };
    // own heads' scores of `step` -> S and the mailbox
    auto publish = [&](int step) {
      const int gs = gstep + step;
      const int sl = step & (NST - 1);
      uint4 ko[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) ko[k] = rd16[(sl * SB + k * SLAB) / 16];
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = dot8_split(qh, ql, ko[k]);
      const float x = row16_sum4(v[0], v[1], v[2], v[3], lane);
      if (r16 < 4) {
        S[(gs & (NS - 1)) * 256 + (ocol / DH) * 8 + (pub_e & 7)] = x;
        const unsigned long long ent =
            ((unsigned long long)(ep_pub | (((uint32_t)gs / kMboxDepth) & 0xffu)) << 32) | __float_as_uint(x);
        __hip_atomic_store(mine + (size_t)((uint32_t)gs % kMboxDepth) * 8 * 16 + pub_e, ent, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    auto poll = [&](int step) {  // partner's entries of `step` -> pollbuf[step & 1]
      const int gs = gstep + step;
      if (lane < 8) {
        const i32x4 rs = buffer_desc(theirs + (size_t)((uint32_t)gs % kMboxDepth) * 8 * 16, 128u);
        dma16_sc1(poll_lds + (gs & 1) * 128, rs, 16u * lane);
      }
    };
    // copy the partner's scores of `step` into S if all 16 polled entries
    // carry the step's tag; returns false (S untouched) otherwise
    auto try_check = [&](int step) -> bool {
      const int gs = gstep + step;
      const uint32_t want = ep | (((uint32_t)gs / kMboxDepth) & 0xffu);
      const unsigned long long v = lane < 16 ? pollbuf[wave * 32 + (gs & 1) * 16 + lane] : 0ull;
      const bool ok = __all(lane >= 16 || (uint32_t)(v >> 32) == want);
      if (ok && lane < 16)
        S[(gs & (NS - 1)) * 256 + (xbase / DH + (lane >> 3)) * 8 + (lane & 7)] = __uint_as_float((uint32_t)v);
      return ok;
    };
    // the same, re-polling synchronously until the entries arrive (bounded)
    auto check = [&](int step) {
      const int gs = gstep + step;
      uint32_t tries = 0;
      while (!try_check(step)) {
        if (failed || ++tries > xp.spin_limit) {
          failed = true;
          if (lane < 16) S[(gs & (NS - 1)) * 256 + (xbase / DH + (lane >> 3)) * 8 + (lane & 7)] = __uint_as_float(kQuietNaN);
          break;
        }
        __builtin_amdgcn_s_sleep(4);
        wait_lgkmcnt0();
        poll(step);
        wait_vmcnt<0>();
      }
      wait_lgkmcnt0();  // the pollbuf read is done before the buffer is refilled
    };
    auto b_operands = [&](int step, s16x4 (&bop)[8]) {
      const lds_s16x4* a0 =
          (const lds_s16x4*)(size_t)(wring_s + (uint32_t)((step & (NST - 1)) * SB + tr_off));
#pragma unroll
      for (int s = 0; s < 8; ++s) bop[s] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(a0 + 8 * s));
    };
    auto barrier = [&]() {
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
    };

    float m_ref = kNegInf, l_half = 0.f;
    f32x16 acc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[s] = f32x16{0};
    const int nsteps = (n + kStepTokens - 1) / kStepTokens;

    // prologue: ring steps 0..3 landed; the own heads' scores of steps 0..2
    // published and the partner's of step 0 in S; B operands of step 0;
    // step 4 in flight.  The wave's 1 KB of q travels by DMA (4-byte
    // elements: q need only be 4-byte aligned) with the first ring steps,
    // and each step's scores go out as soon as that step has landed (the
    // waits count only the younger ring loads).
    s16x4 bcur[8];
    {
      const i32x4 rq = buffer_desc(p.q + (size_t)b * d + ubase, kMfmaUnitCols * 4u);
#pragma unroll
      for (int k = 0; k < 4; ++k) dma4(qbuf_s + k * 256, rq, 4u * (uint32_t)(64 * k + lane));
    }
#pragma unroll
    for (int s = 0; s < NST; ++s) issue(s);
    wait_vmcnt<NST * LPS>();
    split_q8(qbuf + wave * kMfmaUnitCols + 8 * l32, p.qscale, qh, ql);
    wait_vmcnt<3 * LPS>();
    publish(0);
    wait_vmcnt<2 * LPS>();
    publish(1);
    wait_vmcnt<LPS>();
    publish(2);
    wait_lgkmcnt0();
    poll(0);
    wait_vmcnt<0>();
    check(0);
    b_operands(0, bcur);
    wait_lgkmcnt0();
    issue(NST);
    barrier();

    for (int st = 0; st < nsteps; ++st) {
      // ring step st+3 has landed (the wait for poll(st) at the end of the
      // previous step covered it); the partner's step st+1 was published two
      // steps ago
      poll(st + 1);
      publish(st + 3);
      s16x4 bnext[8];
      b_operands(st + 1, bnext);
      const float4 sv = *reinterpret_cast<const float4*>(S + ((gstep + st) & (NS - 1)) * 256 + l32 * 8 + half * 4);
      float sc[4] = {sv.x, sv.y, sv.z, sv.w};
      if ((st + 1) * kStepTokens > n) {  // ragged last step
        const int t0 = st * kStepTokens + half * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) sc[k] = t0 + k < n ? sc[k] : kNegInf;
      }
      wait_lgkmcnt0();
      issue(st + 1 + NST);

      float ma, mb;
      halves(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), ma, mb);
      const float mt = fmaxf(ma, mb);
      const bool grow = mt > m_ref + kRescaleSlack;
      if (__any(grow)) {
        const float m_new = grow ? mt : m_ref;
        const float alpha = grow ? fast_exp2(m_ref - m_new) : 1.f;
        l_half *= alpha;
        m_ref = m_new;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float ar = __shfl(alpha, 8 * (e >> 2) + 4 * half + (e & 3), 64);
#pragma unroll
          for (int s = 0; s < 8; ++s) acc[s][e] *= ar;
        }
      }
      const float mu = fmaxf(m_ref, -__FLT_MAX__);
      const bf16x2_t p01 = {(__bf16)fast_exp2(sc[0] - mu), (__bf16)fast_exp2(sc[1] - mu)};
      const bf16x2_t p23 = {(__bf16)fast_exp2(sc[2] - mu), (__bf16)fast_exp2(sc[3] - mu)};
      const uint32_t w0 = __builtin_bit_cast(uint32_t, p01);
      const uint32_t w1 = __builtin_bit_cast(uint32_t, p23);
      l_half = dot2_bf16(w1, kOnesBf16x2, dot2_bf16(w0, kOnesBf16x2, l_half));
      {
        uint2 aw = make_uint2(w0, w1);
        const s16x4 a = __builtin_bit_cast(s16x4, aw);
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[s] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, bcur[s], acc[s], 0, 0, 0);
      }
      // the partner's scores of step st+1: poll(st+1) has landed once only
      // publish(st+3) and the 4 ring loads of step st+5 are younger
      wait_vmcnt<1 + LPS>();
      check(st + 1);
#pragma unroll
      for (int s = 0; s < 8; ++s) bcur[s] = bnext[s];
      barrier();
    }
    gstep += nsteps + kXchgLook;
    wait_vmcnt<0>();

    float la, lb;
    halves(l_half, la, lb);
    store_partials(p, acc, slot, ubase + l32, d, half);
    if (cg == 0 && wave == 0 && lane < p.H) {
      p.ml[(size_t)slot * 2 * p.H + lane] = failed ? __uint_as_float(kQuietNaN) : m_ref;
      p.ml[(size_t)slot * 2 * p.H + p.H + lane] = la + lb;
    }
  }
}

template <int DH, int GC>
static hipError_t launch_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  constexpr int NST = GC == 2 ? 2 : 4;
  constexpr int WB = NST * (GC == 2 ? 8 : 4) * 1024;
  AttendBf16Params p;
  p.q = a.q;
  p.K = static_cast<const uint16_t*>(a.K);
  p.lengths = a.lengths;
  p.U = a.ws + pl.off_U;
  p.ubf16 = pl.ubf16;
  p.ml = reinterpret_cast<float*>(a.ws + pl.off_ml);
  p.status = a.status;
  p.B = a.B;
  p.H = a.H;
  p.d = a.d;
  p.T_max = a.T_max;
  p.nch = pl.nch;
  p.dc = pl.dc;
  p.nslots = pl.nslots;
  p.qscale = a.scale * kLog2e;
  const size_t lds = (size_t)pl.nw * WB + (512 + (size_t)pl.nw * GC * kMfmaUnitCols + 16 + (size_t)a.B + 1) * sizeof(int);
  auto kern = attend_bf16_kernel<DH, GC, NST>;
  static std::atomic<int> granted[kMaxDevices];
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern), lds, granted);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.nch * GC), dim3(pl.nw * 64), lds, s, p);
  return hipGetLastError();
}

// Per-launch epoch of the mailbox tags (23 bits used): distinct for 2^23
// consecutive launches of the process, and started at a random value so
// that another process's entries left in reused device memory do not match.
static uint32_t epoch_seed() {
  std::random_device rd;
  return rd() ^ (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count();
}
static uint32_t next_epoch() {
  static std::atomic<uint32_t> ctr{epoch_seed()};
  return ctr.fetch_add(1) + 1;
}

// Sets every mailbox entry to all ones: a tag no launch writes (tags keep
// their top bit clear).
__global__ void __launch_bounds__(256) mbox_reset_kernel(unsigned long long* __restrict__ mbox, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) mbox[i] = ~0ull;
}

// Launches the exchange kernel when the shape allows it (two full column
// groups of dh = 128); returns hipErrorNotSupported otherwise, and the caller
// falls back.
//
// The epoch is a kernel argument.  A launch recorded into a graph replays
// with the same epoch, so entries left by the previous replay would carry
// the expected tags; while the stream is capturing, a reset of the mailbox
// is recorded in front of the attend, and every replay starts from entries
// no tag matches.
static hipError_t launch_xchg(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  constexpr int NST = 4;
  if (!pl.xchg || env_int("SLIM_XCHG", 1) == 0) return hipErrorNotSupported;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return hipErrorInvalidValue;
  XchgParams xp;
  AttendBf16Params& p = xp.a;
  p.q = a.q;
  p.K = static_cast<const uint16_t*>(a.K);
  p.lengths = a.lengths;
  p.U = a.ws + pl.off_U;
  p.ubf16 = pl.ubf16;
  p.ml = reinterpret_cast<float*>(a.ws + pl.off_ml);
  p.status = a.status;
  p.B = a.B;
  p.H = a.H;
  p.d = a.d;
  p.T_max = a.T_max;
  p.nch = pl.nch;
  p.dc = pl.dc;
  p.nslots = pl.nslots;
  p.qscale = a.scale * kLog2e;
  xp.mbox = reinterpret_cast<unsigned long long*>(a.ws + pl.off_mbox);
  xp.tickets = reinterpret_cast<unsigned long long*>(a.ws + pl.off_tickets);
  xp.epoch = next_epoch();
  // testing knobs: the wait bound, and a skew that keeps one column group's
  // entries from ever matching (every wait then runs out of its bound)
  const int spin = env_int("SLIM_XCHG_SPIN", -1);
  xp.spin_limit = spin >= 0 ? (uint32_t)spin : kPollSpinLimit;
  xp.pub_skew = (uint32_t)env_int("SLIM_XCHG_SKEW", 0);
  if (cap == hipStreamCaptureStatusActive) {
    const size_t n = (size_t)pl.nch * 2 * kMboxDepth * 8 * 16;
    const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(mbox_reset_kernel, dim3(blocks), dim3(256), 0, s, xp.mbox, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t lds = (size_t)pl.nw * NST * 4 * (1024 + 64) + 4 * 256 * sizeof(float) +
                     (size_t)pl.nw * 32 * sizeof(unsigned long long) + (size_t)pl.nw * kMfmaUnitCols * sizeof(float) +
                     (16 + (size_t)a.B + 1) * sizeof(int);
  auto kern = attend_xchg_kernel<NST>;
  static std::atomic<int> granted[kMaxDevices];
  if (allow_lds(reinterpret_cast<const void*>(kern), lds, granted) != hipSuccess) {
    (void)hipGetLastError();
    return hipErrorNotSupported;
  }
  hipLaunchKernelGGL(kern, dim3(pl.nch * 2), dim3(pl.nw * 64), lds, s, xp);
  return hipGetLastError();
}

hipError_t launch_attend_bf16(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
  if (pl.gc == 2 && a.dh == 128) {
    const hipError_t e = launch_xchg(pl, a, s);
    if (e != hipErrorNotSupported) return e;
  }
  if (pl.gc == 1) {
    switch (a.dh) {
      case 32: return launch_t<32, 1>(pl, a, s);
      case 64: return launch_t<64, 1>(pl, a, s);
      case 128: return launch_t<128, 1>(pl, a, s);
    }
  } else {
    switch (a.dh) {
      case 32: return launch_t<32, 2>(pl, a, s);
      case 64: return launch_t<64, 2>(pl, a, s);
      case 128: return launch_t<128, 2>(pl, a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace slim
