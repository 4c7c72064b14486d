// C ABI of libslim.so: argument checks, launch planning and dispatch.
// Every entry point validates its arguments on the host before enqueueing
// anything and maps failures to slim_status_t; no exception crosses the ABI.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "slim.h"
#include "internal.hpp"
#include "step.hpp"
#include "multi.hpp"
#include "launch.hpp"

namespace slim {

bool lu_solve_inplace(double* A, double* R, int d, int nr);
uint16_t f64_to_bf16_rne(double x);

int env_int(const char* name, int dflt) {
  const char* e = std::getenv(name);
  if (!e || !*e) return dflt;
  return std::atoi(e);
}

static int device_cus(int* ncu) {
  static std::atomic<int> cache[kMaxDevices];  // 0 = unknown
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *ncu = c;
      return 0;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  if (cached) cache[dev].store(n, std::memory_order_relaxed);
  *ncu = n;
  return 0;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool make_decode_plan(int B, int H, int dh, int T_max, bool bf16_k, int ncu, DecodePlan* p) {
  const int d = H * dh;
  p->bf16_k = bf16_k;
  const long long tokens = (long long)B * T_max;
  long long nch;
  if (bf16_k) {
    p->gc = d > 2048 ? 2 : 1;
    const int per = (d + p->gc - 1) / p->gc;
    p->dc = ((per + kMfmaUnitCols - 1) / kMfmaUnitCols) * kMfmaUnitCols;
    p->nw = p->dc / kMfmaUnitCols;  // one 256-column unit per wave
    // two waves per SIMD: 8 waves per CU, one wide workgroup or several narrow
    const int wg_per_cu = p->nw >= 8 ? 1 : 8 / p->nw;
    nch = ((long long)ncu * wg_per_cu + p->gc - 1) / p->gc;
    const long long cap = (tokens + 63) / 64;  // at least ~64 tokens per chunk
    if (nch > cap) nch = cap;
    // 32-bit buffer offsets: a chunk's bytes must stay below 2^31
    const long long need = ((long long)B * T_max * d * 2 >> 30) + 1;
    if (nch < need) nch = need;
    if (p->gc == 2 && nch >= 8) nch = (nch + 7) / 8 * 8;
  } else {
    p->gc = (d + 255) / 256;
    p->dc = 256;
    p->nw = 4;
    nch = ((long long)ncu * 2 + p->gc - 1) / p->gc;
    const long long cap = (tokens + 15) / 16;
    if (nch > cap) nch = cap;
  }
  if (nch < 1) nch = 1;
  const int ov = env_int("SLIM_CHUNKS", 0);
  if (ov > 0) nch = ov;
  if (bf16_k) {
    // 32-bit buffer offsets: a chunk's bytes must stay below 2^31 (also
    // under the override)
    const long long need = ((long long)B * T_max * d * 2 >> 30) + 1;
    if (nch < need) nch = need;
  }
  if (nch > (1 << 20)) return false;
  p->nch = (int)nch;
  p->nslots = p->nch + B - 1;
  {
    const int big = proj_rows(dh, true);
    p->spw = finish_seqs(H, (d + big - 1) / big, B, ncu);
    const long long grid = (long long)H * ((d + big - 1) / big) * ((B + p->spw - 1) / p->spw);
    p->proj_rows = grid * 2 >= ncu ? big : proj_rows(dh, false);
  }
  p->npc = (d + p->proj_rows - 1) / p->proj_rows;
  // control block first: status word, arrival counter
  p->off_status = 0;
  p->off_tickets = 8;
  size_t off = 256;
  // bf16 caches keep their chunk partials in bf16 (accumulated in fp32,
  // rounded once when stored); SLIM_PARTIALS=f32 keeps them in fp32
  const char* pe = std::getenv("SLIM_PARTIALS");
  p->ubf16 = bf16_k && !(pe && std::strcmp(pe, "f32") == 0);
  p->off_U = off;
  off += align256((size_t)p->nslots * H * d * (p->ubf16 ? 2 : 4));
  p->off_ml = off;
  off += align256((size_t)p->nslots * 2 * H * sizeof(float));
  p->off_op = off;
  off += align256((size_t)p->npc * B * H * dh * sizeof(float));
  p->xchg = bf16_k && p->gc == 2 && dh == 128 && 2 * p->dc == d && p->nw == 8;
  p->off_mbox = off;
  off += p->xchg ? align256((size_t)p->nch * 2 * 8 * 8 * 16 * sizeof(unsigned long long)) : 0;
  p->bytes = off;
  return true;
}

}  // namespace slim

using namespace slim;

// Workspace of slim_decode_noalloc: a file-scope device array, one copy per
// device, held until the process ends.  In host code `scratch` only names
// the symbol; its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SLIM_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; null on failure.
static void* scratch_ptr() {
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return nullptr;
  }
  cache[dev].store(p, std::memory_order_release);
  return p;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

extern "C" {

const char* slim_status_string(slim_status_t s) {
  switch (s) {
    case SLIM_OK: return "ok";
    case SLIM_ERR_INVALID: return "invalid argument";
    case SLIM_ERR_UNSUPPORTED: return "unsupported configuration";
    case SLIM_ERR_WORKSPACE: return "workspace too small";
    case SLIM_ERR_HIP: return "HIP runtime error";
    case SLIM_ERR_SINGULAR: return "W_K is singular";
    case SLIM_ERR_TIMEOUT: return "an attend workgroup gave up waiting for its partner";
  }
  return "unknown status";
}

slim_status_t slim_wkv(const double* W_K, const double* W_V, int d, void* W_KV_out,
                       slim_dtype_t out_dt) {
  if (!W_K || !W_V || !W_KV_out || d <= 0) return SLIM_ERR_INVALID;
  if (out_dt != SLIM_F32 && out_dt != SLIM_BF16) return SLIM_ERR_UNSUPPORTED;
  try {
    const size_t n = (size_t)d * d;
    std::vector<double> A(W_K, W_K + n), R(W_V, W_V + n);
    if (!lu_solve_inplace(A.data(), R.data(), d, d)) return SLIM_ERR_SINGULAR;
    if (out_dt == SLIM_F32) {
      float* o = static_cast<float*>(W_KV_out);
      for (size_t i = 0; i < n; ++i) o[i] = (float)R[i];
    } else {
      uint16_t* o = static_cast<uint16_t*>(W_KV_out);
      for (size_t i = 0; i < n; ++i) o[i] = f64_to_bf16_rne(R[i]);
    }
  } catch (const std::bad_alloc&) {
    return SLIM_ERR_INVALID;
  } catch (...) {
    return SLIM_ERR_INVALID;
  }
  return SLIM_OK;
}

slim_status_t slim_prefill(const void* X, slim_dtype_t x_dt, const void* W, slim_dtype_t w_dt,
                           void* K_cache, slim_dtype_t k_dt, int B, int n, int d, int T_max,
                           const int32_t* t0, hipStream_t stream) {
  if (!X || !W || !K_cache || B <= 0 || n <= 0 || d <= 0 || T_max <= 0 || n > T_max)
    return SLIM_ERR_INVALID;
  const bool all_bf16 = x_dt == SLIM_BF16 && w_dt == SLIM_BF16 && k_dt == SLIM_BF16;
  const bool all_f32 = x_dt == SLIM_F32 && w_dt == SLIM_F32 && k_dt == SLIM_F32;
  if (!all_bf16 && !all_f32) return SLIM_ERR_UNSUPPORTED;
  if (all_bf16 && (d % 8 != 0 || !aligned16(X) || !aligned16(W) || !aligned16(K_cache)))
    return SLIM_ERR_INVALID;
  const long long M = (long long)B * n;
  if ((M + 63) / 64 > 65535 || (long long)B * T_max * d > (1LL << 40)) return SLIM_ERR_UNSUPPORTED;
  hipError_t e = all_bf16 ? launch_prefill_bf16(X, W, K_cache, B, n, d, T_max, t0, stream)
                          : launch_prefill_f32(X, W, K_cache, B, n, d, T_max, t0, stream);
  return e == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

// Shape support of slim_decode; SLIM_OK when supported.
static slim_status_t decode_shape_ok(int B, int H, int dh, int T_max, slim_dtype_t k_dt) {
  if (B <= 0 || H <= 0 || dh <= 0 || T_max <= 0) return SLIM_ERR_INVALID;
  if (k_dt != SLIM_F32 && k_dt != SLIM_BF16) return SLIM_ERR_UNSUPPORTED;
  if (B > 4096 || (long long)H * dh > 65536) return SLIM_ERR_UNSUPPORTED;
  if (k_dt == SLIM_BF16) {
    if (H > 32 || (dh != 32 && dh != 64 && dh != 128)) return SLIM_ERR_UNSUPPORTED;
  } else {
    if (H > 64 || !is_pow2(dh) || dh > 256 || H * dh > 16384) return SLIM_ERR_UNSUPPORTED;
  }
  return SLIM_OK;
}

size_t slim_decode_workspace_bytes(int B, int H, int dh, int T_max, slim_dtype_t k_dt) {
  if (decode_shape_ok(B, H, dh, T_max, k_dt) != SLIM_OK) return 0;
  int ncu = 0;
  if (device_cus(&ncu) != 0) return 0;
  DecodePlan p;
  if (!make_decode_plan(B, H, dh, T_max, k_dt == SLIM_BF16, ncu, &p)) return 0;
  return p.bytes;
}

enum DecodeMode { kFull = 0, kAttend = 1, kFinish = 2 };

// Host checks and plan of a decode call, everything but the workspace size.
static slim_status_t decode_prepare(const float* q, const void* K_cache, slim_dtype_t k_dt,
                                    const int32_t* lengths, const void* W_KV, slim_dtype_t w_dt,
                                    float* out, int B, int H, int dh, int T_max, float scale,
                                    void* workspace, DecodePlan* plan, DecodeArgs* a) {
  if (!q || !K_cache || !lengths || !W_KV || !out || !workspace) return SLIM_ERR_INVALID;
  if (!std::isfinite(scale)) return SLIM_ERR_INVALID;
  slim_status_t st = decode_shape_ok(B, H, dh, T_max, k_dt);
  if (st != SLIM_OK) return st;
  if (w_dt != SLIM_F32 && w_dt != SLIM_BF16) return SLIM_ERR_UNSUPPORTED;
  if (!aligned16(workspace) || !aligned16(K_cache) || !aligned16(W_KV) || ((uintptr_t)q & 3u) ||
      ((uintptr_t)out & 3u) || ((uintptr_t)lengths & 3u))
    return SLIM_ERR_INVALID;
  int ncu = 0;
  if (device_cus(&ncu) != 0) return SLIM_ERR_HIP;
  if (!make_decode_plan(B, H, dh, T_max, k_dt == SLIM_BF16, ncu, plan)) return SLIM_ERR_UNSUPPORTED;
  a->q = q;
  a->K = K_cache;
  a->lengths = lengths;
  a->W = W_KV;
  a->out = out;
  a->B = B;
  a->H = H;
  a->dh = dh;
  a->d = H * dh;
  a->T_max = T_max;
  a->nslots = plan->nslots;
  a->scale = scale;
  a->w_bf16 = w_dt == SLIM_BF16;
  a->ws = static_cast<char*>(workspace);
  a->status = reinterpret_cast<uint32_t*>(a->ws + plan->off_status);
  return SLIM_OK;
}

static hipError_t decode_launch(int mode, const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (mode == kFull || mode == kAttend)
    e = plan.bf16_k ? launch_attend_bf16(plan, a, stream) : launch_attend_f32(plan, a, stream);
  if (e == hipSuccess && (mode == kFull || mode == kFinish)) e = launch_finish(plan, a, stream);
  return e;
}

static slim_status_t decode_common(int mode, const float* q, const void* K_cache, slim_dtype_t k_dt,
                                   const int32_t* lengths, const void* W_KV, slim_dtype_t w_dt,
                                   float* out, int B, int H, int dh, int T_max, float scale,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodePlan plan;
  DecodeArgs a;
  slim_status_t st = decode_prepare(q, K_cache, k_dt, lengths, W_KV, w_dt, out, B, H, dh, T_max, scale,
                                    workspace, &plan, &a);
  if (st != SLIM_OK) return st;
  if (workspace_bytes < plan.bytes) return SLIM_ERR_WORKSPACE;
  return decode_launch(mode, plan, a, stream) == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

slim_status_t slim_decode(const float* q, const void* K_cache, slim_dtype_t k_dt,
                          const int32_t* lengths, const void* W_KV, slim_dtype_t w_dt, float* out,
                          int B, int H, int dh, int T_max, float scale, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return decode_common(kFull, q, K_cache, k_dt, lengths, W_KV, w_dt, out, B, H, dh, T_max, scale,
                       workspace, workspace_bytes, stream);
}

slim_status_t slim_decode_noalloc(const float* q, const void* K_cache, slim_dtype_t k_dt,
                                  const int32_t* lengths, const void* W_KV, slim_dtype_t w_dt, float* out,
                                  int B, int H, int dh, int T_max, float scale, hipStream_t stream) {
  DecodePlan plan;
  DecodeArgs a;
  // the argument checks need a non-null, aligned workspace pointer: the
  // scratch address is looked up only once they pass
  static const char kProbe alignas(256) = 0;
  slim_status_t st = decode_prepare(q, K_cache, k_dt, lengths, W_KV, w_dt, out, B, H, dh, T_max, scale,
                                    const_cast<char*>(&kProbe), &plan, &a);
  if (st != SLIM_OK) return st;
  if (plan.bytes > (size_t)SLIM_NOALLOC_SCRATCH_BYTES) return SLIM_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return SLIM_ERR_HIP;
  a.ws = static_cast<char*>(ws);
  a.status = reinterpret_cast<uint32_t*>(a.ws + plan.off_status);
  return decode_launch(kFull, plan, a, stream) == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

slim_status_t slim_decode_attend(const float* q, const void* K_cache, slim_dtype_t k_dt,
                                 const int32_t* lengths, const void* W_KV, slim_dtype_t w_dt,
                                 float* out, int B, int H, int dh, int T_max, float scale,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(kAttend, q, K_cache, k_dt, lengths, W_KV, w_dt, out, B, H, dh, T_max, scale,
                       workspace, workspace_bytes, stream);
}

slim_status_t slim_decode_finish(const float* q, const void* K_cache, slim_dtype_t k_dt,
                                 const int32_t* lengths, const void* W_KV, slim_dtype_t w_dt,
                                 float* out, int B, int H, int dh, int T_max, float scale,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(kFinish, q, K_cache, k_dt, lengths, W_KV, w_dt, out, B, H, dh, T_max, scale,
                       workspace, workspace_bytes, stream);
}

slim_status_t slim_decode_status(const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || workspace_bytes < 256 || !aligned16(workspace)) return SLIM_ERR_INVALID;
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return SLIM_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SLIM_ERR_HIP;
  return word == 0 ? SLIM_OK : SLIM_ERR_TIMEOUT;
}

size_t slim_step_workspace_bytes(int B, int H, int dh, int T_max, slim_dtype_t k_dt) {
  if (decode_shape_ok(B, H, dh, T_max, k_dt) != SLIM_OK || (H * dh) % 8 != 0) return 0;
  int ncu = 0;
  if (device_cus(&ncu) != 0) return 0;
  DecodePlan p;
  StepPlan sp, sp2;
  if (!make_decode_plan(B, H, dh, T_max, k_dt == SLIM_BF16, ncu, &p)) return 0;
  if (!make_step_plan(B, H * dh, ncu, true, p.bytes, &sp) ||
      !make_step_plan(B, H * dh, ncu, false, p.bytes, &sp2))
    return 0;
  return sp.bytes > sp2.bytes ? sp.bytes : sp2.bytes;  // either weight dtype
}

slim_status_t slim_step(const float* x, const void* W_Q, const void* W_K, slim_dtype_t w_dt,
                        void* K_cache, slim_dtype_t k_dt, const int32_t* lengths, int32_t* lengths_next,
                        const void* W_KV, slim_dtype_t wkv_dt, float* out, int B, int H, int dh,
                        int T_max, float scale, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!x || !W_Q || !W_K || !lengths_next) return SLIM_ERR_INVALID;
  if (w_dt != SLIM_F32 && w_dt != SLIM_BF16) return SLIM_ERR_UNSUPPORTED;
  if (((uintptr_t)x & 3u) || !aligned16(W_Q) || !aligned16(W_K) || ((uintptr_t)lengths_next & 3u))
    return SLIM_ERR_INVALID;
  if (lengths_next == lengths) return SLIM_ERR_INVALID;
  if ((long long)H * dh % 8 != 0) return SLIM_ERR_UNSUPPORTED;
  DecodePlan plan;
  DecodeArgs a;
  // q is filled in below; any aligned non-null pointer passes the checks here
  slim_status_t st = decode_prepare(x, K_cache, k_dt, lengths, W_KV, wkv_dt, out, B, H, dh, T_max, scale,
                                    workspace, &plan, &a);
  if (st != SLIM_OK) return st;
  int ncu = 0;
  if (device_cus(&ncu) != 0) return SLIM_ERR_HIP;
  StepPlan sp;
  if (!make_step_plan(B, H * dh, ncu, w_dt == SLIM_BF16, plan.bytes, &sp)) return SLIM_ERR_UNSUPPORTED;
  if (workspace_bytes < sp.bytes) return SLIM_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipError_t e = launch_step_qk(sp, x, W_Q, W_K, w_dt == SLIM_BF16, K_cache, k_dt == SLIM_BF16, lengths,
                                lengths_next, B, H * dh, T_max, ws, stream);
  if (e != hipSuccess) return SLIM_ERR_HIP;
  a.q = reinterpret_cast<const float*>(ws + sp.off_q);
  return decode_launch(kFull, plan, a, stream) == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

static slim_status_t multi_shape_ok(int n, int H, int dh, int T, slim_dtype_t k_dt, slim_dtype_t w_dt,
                                    int option) {
  if (n <= 0 || H <= 0 || dh <= 0 || T <= 0) return SLIM_ERR_INVALID;
  if (option < 0 || option > 2) return SLIM_ERR_INVALID;
  if (k_dt != SLIM_BF16 || (w_dt != SLIM_BF16 && w_dt != SLIM_F32)) return SLIM_ERR_UNSUPPORTED;
  if ((dh != 64 && dh != 128) || (H * dh) % 128 != 0 || H * dh > 65536) return SLIM_ERR_UNSUPPORTED;
  if (n > (1 << 20) || T > 4000000 || (long long)H * ((n + 31) / 32) > 65535) return SLIM_ERR_UNSUPPORTED;
  return SLIM_OK;
}

// Multiply-accumulate counts of the two options, with option 1's V = K.W_KV
// weighted by kGemmWeight: it is one dense GEMM, which runs at about 1.5
// times the rate of the per-head contractions of the many-query kernel on
// this device (measured: 125-185 against 80-140 TFLOP/s on the Whisper- and
// GPT-2-shaped cases).  Ties go to option 2.
constexpr double kGemmWeight = 2.0 / 3.0;

int slim_multi_query_option(int n, int H, int dh, int T) {
  if (n <= 0 || H <= 0 || dh <= 0 || T <= 0) return 0;
  const double d = (double)H * dh;
  const double o1 = kGemmWeight * (double)T * d * d + (double)n * T * d;
  const double o2 = (double)n * H * T * d + (double)n * d * d;
  return o1 < o2 ? 1 : 2;
}

size_t slim_multi_query_workspace_bytes(int n, int H, int dh, int T, slim_dtype_t k_dt, slim_dtype_t w_dt,
                                        int option) {
  if (multi_shape_ok(n, H, dh, T, k_dt, w_dt, option) != SLIM_OK) return 0;
  int ncu = 0;
  if (device_cus(&ncu) != 0) return 0;
  MultiPlan p;
  if (!make_multi_plan(n, H, dh, T, option, w_dt == SLIM_BF16, ncu, &p)) return 0;
  return p.bytes;
}

slim_status_t slim_multi_query(const float* Q, const void* K, slim_dtype_t k_dt, const int32_t* limits,
                               const void* W_KV, slim_dtype_t w_dt, float* out, int n, int H, int dh, int T,
                               float scale, int option, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (!Q || !K || !W_KV || !out || !workspace) return SLIM_ERR_INVALID;
  if (!std::isfinite(scale)) return SLIM_ERR_INVALID;
  slim_status_t st = multi_shape_ok(n, H, dh, T, k_dt, w_dt, option);
  if (st != SLIM_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(W_KV) || !aligned16(workspace) || ((uintptr_t)out & 3u) ||
      ((uintptr_t)limits & 3u))
    return SLIM_ERR_INVALID;
  int ncu = 0;
  if (device_cus(&ncu) != 0) return SLIM_ERR_HIP;
  MultiPlan plan;
  if (!make_multi_plan(n, H, dh, T, option, w_dt == SLIM_BF16, ncu, &plan)) return SLIM_ERR_UNSUPPORTED;
  if (workspace_bytes < plan.bytes) return SLIM_ERR_WORKSPACE;
  hipError_t e = launch_multi(plan, Q, K, limits, W_KV, w_dt == SLIM_BF16, out, n, H, dh, T, scale,
                              static_cast<char*>(workspace), stream);
  return e == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

static slim_status_t kv_shape_ok(int B, int H, int dh, int T_max, slim_dtype_t kv_dt) {
  if (B <= 0 || H <= 0 || dh <= 0 || T_max <= 0) return SLIM_ERR_INVALID;
  if (kv_dt != SLIM_BF16 && kv_dt != SLIM_F32) return SLIM_ERR_UNSUPPORTED;
  if (kv_dt != SLIM_BF16) return SLIM_ERR_UNSUPPORTED;
  if (B > 4096 || (dh != 32 && dh != 64 && dh != 128)) return SLIM_ERR_UNSUPPORTED;
  const int hpw = 64 / (dh / 8);
  if ((H + hpw - 1) / hpw > 8) return SLIM_ERR_UNSUPPORTED;
  return SLIM_OK;
}

size_t mha_decode_kv_workspace_bytes(int B, int H, int dh, int T_max, slim_dtype_t kv_dt) {
  if (kv_shape_ok(B, H, dh, T_max, kv_dt) != SLIM_OK) return 0;
  int ncu = 0;
  if (device_cus(&ncu) != 0) return 0;
  KVPlan p;
  if (!make_kv_plan(B, H, dh, T_max, ncu, &p)) return 0;
  return p.bytes;
}

slim_status_t mha_decode_kv(const float* q, const void* K_cache, const void* V_cache,
                            slim_dtype_t kv_dt, const int32_t* lengths, float* out, int B, int H,
                            int dh, int T_max, float scale, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  if (!q || !K_cache || !V_cache || !lengths || !out || !workspace) return SLIM_ERR_INVALID;
  if (!std::isfinite(scale)) return SLIM_ERR_INVALID;
  slim_status_t st = kv_shape_ok(B, H, dh, T_max, kv_dt);
  if (st != SLIM_OK) return st;
  if (!aligned16(K_cache) || !aligned16(V_cache) || !aligned16(workspace) || ((uintptr_t)q & 3u) ||
      ((uintptr_t)out & 3u) || ((uintptr_t)lengths & 3u))
    return SLIM_ERR_INVALID;
  int ncu = 0;
  if (device_cus(&ncu) != 0) return SLIM_ERR_HIP;
  KVPlan plan;
  if (!make_kv_plan(B, H, dh, T_max, ncu, &plan)) return SLIM_ERR_UNSUPPORTED;
  if (workspace_bytes < plan.bytes) return SLIM_ERR_WORKSPACE;
  hipError_t e = launch_mha_kv(plan, q, K_cache, V_cache, lengths, out, B, H, dh, T_max, scale,
                               static_cast<char*>(workspace), stream);
  return e == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

int slim_probe_sink_floats(void) { return probe_sink_floats(); }

slim_status_t slim_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !aligned16(src)) return SLIM_ERR_INVALID;
  return launch_probe_read(src, bytes, sink, stream) == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

slim_status_t slim_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
    return SLIM_ERR_INVALID;
  return launch_probe_copy(dst, src, bytes, stream) == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

}  // extern "C"
