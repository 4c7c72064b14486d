// Device helpers shared by the libslim kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slim {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// bf16 <-> fp32 on packed words.  A bf16 value is the high half of an fp32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).  Both results
// are formed and one is selected, so that long unrolled runs of conversions
// stay free of branches and exec-mask changes.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet_nan = (u >> 16) | 0x40u;
  return (u & 0x7fffffffu) > 0x7f800000u ? quiet_nan : rounded;
}

// Two fp32 -> one word of two bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Byte permute: result byte i = byte sel_i of {hi:lo} (lo = bytes 0..3).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
constexpr uint32_t kSelLo = 0x05040100u;  // {lo.lo16, hi.lo16}
constexpr uint32_t kSelHi = 0x07060302u;  // {lo.hi16, hi.hi16}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP move of a float within rows of 16 lanes (all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N a power of two <= 16, groups inside
// one DPP row of 16), result in every lane of the group.  xor-1 and xor-2
// quad permutes give quad sums; the half-row mirror pairs quads 0<->1; the
// row mirror pairs the two halves of the row.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (N >= 16) v += dpp_f<0x140>(v); // row_mirror
  return v;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 value split into two bf16 parts, hi = bf16(x), lo = bf16(x - hi);
// hi + lo matches x to about 2^-16 relatively.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - __uint_as_float(hi << 16));
}

// acc + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs, fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         acc, false);
}

// Sums of four per-lane values over each aligned row of 16 lanes, one result
// per lane: lane r of the row ends with the total of value (2*(r&1) + ((r>>1)&1)).
// Two exchange levels halve the values held per lane (xor 1, xor 2 quad
// permutes), two row rotations (by 4 and by 8) finish the sums.
__device__ __forceinline__ float row16_sum4(float v0, float v1, float v2, float v3, int lane) {
  const bool b0 = lane & 1, b1 = (lane >> 1) & 1;
  const float s0 = b0 ? v0 : v2, s1 = b0 ? v1 : v3;
  const float k0 = b0 ? v2 : v0, k1 = b0 ? v3 : v1;
  const float a0 = k0 + dpp_f<0xB1>(s0);  // partner lane ^ 1
  const float a1 = k1 + dpp_f<0xB1>(s1);
  const float sb = b1 ? a0 : a1, kb = b1 ? a1 : a0;
  float x = kb + dpp_f<0x4E>(sb);         // partner lane ^ 2
  x += dpp_f<0x124>(x);                   // row_ror:4
  x += dpp_f<0x128>(x);                   // row_ror:8
  return x;
}

// Raw buffer resource over [base, base + bytes): loads at byte offsets
// outside the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Exclusive prefix sum of per-thread ints over a block of up to 1024
// threads; `tmp` needs blockDim/64 ints of shared memory.  Returns the
// exclusive prefix; `total` receives the block sum.  Contains barriers.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63 || threadIdx.x == blockDim.x - 1) tmp[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    int s = tmp[i];
    off += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

// pre[0..B] = exclusive prefix sums of clamp(lengths[b], 0, T_max) in shared
// memory (pre[B] = total).  All threads of the block participate.
__device__ __forceinline__ void lengths_prefix(const int32_t* __restrict__ lengths, int B, int T_max,
                                               int* pre, int* tmp) {
  int carry = 0;
  for (int base = 0; base < B; base += blockDim.x) {
    const int b = base + threadIdx.x;
    int v = 0;
    if (b < B) {
      v = lengths[b];
      v = v < 0 ? 0 : (v > T_max ? T_max : v);
    }
    int tot;
    const int ex = block_exclusive_scan(v, tmp, tot);
    if (b < B) pre[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) pre[B] = carry;
  __syncthreads();
}

// Largest b in [0, B) with pre[b] <= x < pre[b+1]; x must be < pre[B].
__device__ __forceinline__ int seq_of(const int* pre, int B, int x) {
  int lo = 0, hi = B;  // invariant: pre[lo] <= x < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Chunk size of the token stream: the concatenation of all sequences'
// live rows is cut into `nch` chunks of ceil(total / nch) tokens.  A chunk
// c and a sequence b that overlap form a "piece" whose partial result is
// stored in slot c + b (unique; at most nch + B - 1 slots).
__device__ __forceinline__ int chunk_tokens(int total, int nch) {
  return (total + nch - 1) / nch;
}

}  // namespace slim
