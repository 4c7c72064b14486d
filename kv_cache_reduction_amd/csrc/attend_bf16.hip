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
//    layout), rounds the weights to bf16 and issues v_mfma_f32_32x32x8_bf16
//    with B operands built by byte permutes (a 4x8 -> 8x4 transpose of
//    16-bit values in registers).
//  * Lazy rescaling: each head keeps a reference max m (log2 units) and the
//    accumulator holds sum_t 2^(s_t - m) K[t]; m only moves (and the
//    accumulator rows are rescaled) when a score exceeds it by more than 8,
//    so weights stay below 2^8 and the rescale is rare.
//  * Per piece (chunk x sequence) the workgroup writes its unnormalised
//    accumulator U[slot, h, cols] and (column group 0) m and the normaliser
//    l of every head.  q is pre-scaled by scale*log2(e); exponentials use
//    v_exp_f32.
#include "common.hpp"
#include "internal.hpp"

namespace slim {

struct AttendBf16Params {
  const float* q;
  const uint16_t* K;
  const int32_t* lengths;
  float* U;
  float* ml;
  int B, H, d, T_max, nch, dc;
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

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

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

    float4 qo0, qo1, qx0, qx1;
    {
      const float* qb = p.q + (size_t)b * d;
      const float* qpo = qb + (ook ? ocol : 0);
      const float* qpx = qb + (xok ? xcol : 0);
      qo0 = make_float4(qpo[0], qpo[1], qpo[2], qpo[3]);
      qo1 = make_float4(qpo[4], qpo[5], qpo[6], qpo[7]);
      qx0 = make_float4(qpx[0], qpx[1], qpx[2], qpx[3]);
      qx1 = make_float4(qpx[4], qpx[5], qpx[6], qpx[7]);
      const float sc = p.qscale;
      qo0.x *= sc; qo0.y *= sc; qo0.z *= sc; qo0.w *= sc;
      qo1.x *= sc; qo1.y *= sc; qo1.z *= sc; qo1.w *= sc;
      qx0.x *= sc; qx0.y *= sc; qx0.z *= sc; qx0.w *= sc;
      qx1.x *= sc; qx1.y *= sc; qx1.z *= sc; qx1.w *= sc;
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
      {
        float sc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) sc[k] = group_sum<LPH>(dot8(qo0, qo1, ko[k]));
        if (ook && score_lane)
          *reinterpret_cast<float4*>(Sb + (ocol / DH) * 8 + half * 4) = make_float4(sc[0], sc[1], sc[2], sc[3]);
      }
      if (GC == 2) {
        float sc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) sc[k] = group_sum<LPH>(dot8(qx0, qx1, kx[k]));
        if (xok && score_lane)
          *reinterpret_cast<float4*>(Sb + (xcol / DH) * 8 + half * 4) = make_float4(sc[0], sc[1], sc[2], sc[3]);
      }
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
      uint2 aw = make_uint2(w0, w1);
      const s16x4 a = *reinterpret_cast<s16x4*>(&aw);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t sel = (s & 1) ? kSelHi : kSelLo;
        const int wd = s >> 1;
        uint2 bw;
        bw.x = perm(word(ko[1], wd), word(ko[0], wd), sel);
        bw.y = perm(word(ko[3], wd), word(ko[2], wd), sel);
        const s16x4 bv = *reinterpret_cast<s16x4*>(&bw);
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, bv, acc[s], 0, 0, 0);
      }
    }
    wait_vmcnt<0>();  // the loads issued past the end have landed before the ring is reused

    // 4. partial results of this piece
    float* Us = p.U + (size_t)slot * p.H * d;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * half + (e & 3);
      if (ook && row < p.H) {
        float* dst = Us + (size_t)row * d + ocol;
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

hipError_t launch_attend_bf16(const DecodePlan& pl, const DecodeArgs& a, hipStream_t s) {
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
