// Comparator: standard MHA decode over explicit bf16 K and V caches (the
// K+V baseline that Slim Attention halves; Slim Attention article,
// localbendi.com, section "K-Cache is All You Need").  Split-T flash
// decoding with the same chunk/piece/slot scheme as the Slim path.
//
// Each lane owns 8 columns of one head: lane l of wave w serves head
// w*(64/L) + l/L (L = dh/8 lanes per head) and reads, per token, 16 bytes of
// K and 16 bytes of V at those columns straight into registers.  Scores are
// summed over the L lanes of the head; the online softmax and the weighted
// sum of V rows stay inside those lanes, so waves never wait on each other:
// there is no LDS tile and no barrier in the token loop.  Softmax weights
// stay in fp32.
#include "common.hpp"
#include "internal.hpp"

namespace slim {

struct KVParams {
  const float* q;
  const uint16_t* K;
  const uint16_t* V;
  const int32_t* lengths;
  float* O;    // [nslots, H, dh]
  float* ml;   // [nslots, 2, H]
  int B, H, d, T_max, nch;
  float qscale;
};

constexpr int kKVStep = 4;  // tokens per register batch

__device__ __forceinline__ uint4 ldkv(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ float dot8k(const float (&q)[8], const uint4& k) {
  float s = q[0] * bf_lo(k.x);
  s = fmaf(q[1], bf_hi(k.x), s);
  s = fmaf(q[2], bf_lo(k.y), s);
  s = fmaf(q[3], bf_hi(k.y), s);
  s = fmaf(q[4], bf_lo(k.z), s);
  s = fmaf(q[5], bf_hi(k.z), s);
  s = fmaf(q[6], bf_lo(k.w), s);
  s = fmaf(q[7], bf_hi(k.w), s);
  return s;
}

template <int DH>
__global__ void __launch_bounds__(512) mha_kv_split_kernel(KVParams p) {
  constexpr int L = DH / 8, HPW = 64 / L;
  extern __shared__ int smem[];
  int* tmp = smem;       // [16]
  int* pre = smem + 16;  // [B + 1]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = wave * HPW + lane / L;
  const bool hv = h < p.H;
  const int col = h * DH + 8 * (lane % L);
  const int c = blockIdx.x;

  lengths_prefix(p.lengths, p.B, p.T_max, pre, tmp);
  const int total = pre[p.B];
  if (total == 0) return;
  const int Ts = chunk_tokens(total, p.nch);
  const int cbeg = c * Ts;
  if (cbeg >= total) return;
  const int cend = min(total, cbeg + Ts);

  for (int b = seq_of(pre, p.B, cbeg); b < p.B && pre[b] < cend; ++b) {
    const int s0 = pre[b], s1 = pre[b + 1];
    if (s1 == s0) continue;
    const int tb = max(cbeg, s0) - s0;
    const int n = min(cend, s1) - s0 - tb;
    const int slot = c + b;
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = hv ? p.q[(size_t)b * p.d + col + i] * p.qscale : 0.f;
    const size_t base = ((size_t)b * p.T_max + tb) * p.d + col;
    const uint16_t* Kb = p.K + base;
    const uint16_t* Vb = p.V + base;

    float m = kNegInf, l = 0.f, o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;
    const int nsteps = (n + kKVStep - 1) / kKVStep;

    auto load = [&](int st, uint4 (&kr)[kKVStep], uint4 (&vr)[kKVStep]) {
#pragma unroll
      for (int k = 0; k < kKVStep; ++k) {
        const int t = st * kKVStep + k;
        const bool ok = hv && t < n;
        kr[k] = ok ? ldkv(Kb + (size_t)t * p.d) : make_uint4(0, 0, 0, 0);
        vr[k] = ok ? ldkv(Vb + (size_t)t * p.d) : make_uint4(0, 0, 0, 0);
      }
    };
    auto compute = [&](int st, const uint4 (&kr)[kKVStep], const uint4 (&vr)[kKVStep]) {
      float s[kKVStep];
      float mt = kNegInf;
#pragma unroll
      for (int k = 0; k < kKVStep; ++k) {
        s[k] = group_sum<L>(dot8k(qv, kr[k]));
        if (st * kKVStep + k >= n) s[k] = kNegInf;
        mt = fmaxf(mt, s[k]);
      }
      const float m_new = fmaxf(m, mt);
      const float a = fast_exp2(m - m_new);  // m_new is finite: step has a live token
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= a;
#pragma unroll
      for (int k = 0; k < kKVStep; ++k) {
        const float e = fast_exp2(s[k] - m_new);
        ps += e;
        o[0] = fmaf(e, bf_lo(vr[k].x), o[0]);
        o[1] = fmaf(e, bf_hi(vr[k].x), o[1]);
        o[2] = fmaf(e, bf_lo(vr[k].y), o[2]);
        o[3] = fmaf(e, bf_hi(vr[k].y), o[3]);
        o[4] = fmaf(e, bf_lo(vr[k].z), o[4]);
        o[5] = fmaf(e, bf_hi(vr[k].z), o[5]);
        o[6] = fmaf(e, bf_lo(vr[k].w), o[6]);
        o[7] = fmaf(e, bf_hi(vr[k].w), o[7]);
      }
      l = a * l + ps;
      m = m_new;
    };

    uint4 kA[kKVStep], vA[kKVStep], kB[kKVStep], vB[kKVStep];
    load(0, kA, vA);
    for (int st = 0;;) {
      if (st + 1 < nsteps) load(st + 1, kB, vB);
      compute(st, kA, vA);
      if (++st >= nsteps) break;
      if (st + 1 < nsteps) load(st + 1, kA, vA);
      compute(st, kB, vB);
      if (++st >= nsteps) break;
    }
    if (hv) {
      float* dst = p.O + ((size_t)slot * p.H + h) * DH + 8 * (lane % L);
      *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
      if (lane % L == 0) {
        p.ml[(size_t)slot * 2 * p.H + h] = m;
        p.ml[(size_t)slot * 2 * p.H + p.H + h] = l;
      }
    }
  }
}

// out[b, h, :] = sum_s 2^(m_s - m*) O_s[h, :] / sum_s 2^(m_s - m*) l_s
// One 512-thread block per (b, h); thread t sums the float4 column group
// t % (dh/4) over slot group t / (dh/4), then the groups are added in LDS.
__global__ void __launch_bounds__(512) mha_kv_combine_kernel(const int32_t* __restrict__ lengths,
                                                             const float* __restrict__ O,
                                                             const float* __restrict__ ml,
                                                             float* __restrict__ out, int B, int H,
                                                             int dh, int T_max, int nch) {
  extern __shared__ int smem[];
  int* tmp = smem;                                  // [8]
  float* red = reinterpret_cast<float*>(smem + 8);  // [2048]
  float* w = red + 2048;                            // [nch + 1]
  int* pre = reinterpret_cast<int*>(w + nch + 1);   // [B + 1]
  const int b = blockIdx.x / H, h = blockIdx.x % H, tid = threadIdx.x;
  lengths_prefix(lengths, B, T_max, pre, tmp);
  const int s0 = pre[b], s1 = pre[b + 1];
  float* dst = out + ((size_t)b * H + h) * dh;
  if (s1 == s0) {
    for (int j = tid; j < dh; j += blockDim.x) dst[j] = 0.f;
    return;
  }
  const int Ts = chunk_tokens(pre[B], nch);
  const int cf = s0 / Ts, cl = (s1 - 1) / Ts, ns = cl - cf + 1, slot0 = cf + b;
  __shared__ float inv_l;
  if (tid < 64) {
    float m = kNegInf;
    for (int i = tid; i < ns; i += 64) m = fmaxf(m, ml[(size_t)(slot0 + i) * 2 * H + h]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float l = 0.f;
    for (int i = tid; i < ns; i += 64) {
      const float* e = ml + (size_t)(slot0 + i) * 2 * H;
      const float wi = fast_exp2(e[h] - m);
      w[i] = wi;
      l += wi * e[H + h];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (tid == 0) inv_l = 1.f / l;
  }
  __syncthreads();
  const int c4 = dh / 4, ng = blockDim.x / c4;
  const int j4 = tid % c4, g = tid / c4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* src = O + ((size_t)slot0 * H + h) * dh + 4 * j4;
#pragma unroll 8
  for (int i = g; i < ns; i += ng) {
    const float4 v = *reinterpret_cast<const float4*>(src + (size_t)i * H * dh);
    const float wi = w[i];
    acc.x = fmaf(wi, v.x, acc.x);
    acc.y = fmaf(wi, v.y, acc.y);
    acc.z = fmaf(wi, v.z, acc.z);
    acc.w = fmaf(wi, v.w, acc.w);
  }
  reinterpret_cast<float4*>(red)[g * c4 + j4] = acc;
  __syncthreads();
  for (int j = tid; j < dh; j += blockDim.x) {
    float sum = 0.f;
    for (int k = 0; k < ng; ++k) sum += red[k * dh + j];
    dst[j] = sum * inv_l;
  }
}

bool make_kv_plan(int B, int H, int dh, int T_max, int ncu, KVPlan* p) {
  const int L = dh / 8, HPW = 64 / L;
  const int nw = (H + HPW - 1) / HPW;
  long long want = (long long)ncu * 16 / nw;  // about 16 waves per CU
  const long long tokens = (long long)B * T_max;
  long long cap = (tokens + 63) / 64;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  int nch = (int)want;
  const int ov = env_int("SLIM_KV_CHUNKS", 0);
  if (ov > 0) nch = ov;
  p->nch = nch;
  p->nslots = nch + B - 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p->off_o = take((size_t)p->nslots * H * dh * 4);
  p->off_ml = take((size_t)p->nslots * 2 * H * 4);
  p->bytes = off;
  return true;
}

template <int DH>
static hipError_t launch_kv_t(const KVPlan& pl, const float* q, const void* K, const void* V,
                              const int32_t* lengths, float* out, int B, int H, int T_max,
                              float scale, char* ws, hipStream_t s) {
  constexpr int L = DH / 8, HPW = 64 / L;
  KVParams p;
  p.q = q;
  p.K = static_cast<const uint16_t*>(K);
  p.V = static_cast<const uint16_t*>(V);
  p.lengths = lengths;
  p.O = reinterpret_cast<float*>(ws + pl.off_o);
  p.ml = reinterpret_cast<float*>(ws + pl.off_ml);
  p.B = B;
  p.H = H;
  p.d = H * DH;
  p.T_max = T_max;
  p.nch = pl.nch;
  p.qscale = scale * kLog2e;
  const int nw = (H + HPW - 1) / HPW;
  hipLaunchKernelGGL((mha_kv_split_kernel<DH>), dim3(pl.nch), dim3(nw * 64),
                     (16 + (size_t)B + 1) * 4, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mha_kv_combine_kernel, dim3(B * H), dim3(512),
                     (8 + 2048 + (size_t)pl.nch + 1 + (size_t)B + 1) * 4, s, lengths,
                     (const float*)p.O, (const float*)p.ml, out, B, H, DH, T_max, pl.nch);
  return hipGetLastError();
}

hipError_t launch_mha_kv(const KVPlan& pl, const float* q, const void* K, const void* V,
                         const int32_t* lengths, float* out, int B, int H, int dh, int T_max,
                         float scale, char* ws, hipStream_t s) {
  switch (dh) {
    case 32: return launch_kv_t<32>(pl, q, K, V, lengths, out, B, H, T_max, scale, ws, s);
    case 64: return launch_kv_t<64>(pl, q, K, V, lengths, out, B, H, T_max, scale, ws, s);
    case 128: return launch_kv_t<128>(pl, q, K, V, lengths, out, B, H, T_max, scale, ws, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace slim
