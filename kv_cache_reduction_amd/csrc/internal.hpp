// Host-side plan and launcher declarations shared by the libslim sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace slim {

// Launch plan of one slim_decode call.  The token stream (all sequences'
// live rows, concatenated) is cut into `nch` chunks; every chunk is handled
// by `gc` workgroups, one per column group of `dc` columns of K.  Partial
// results live in `nslots = nch + B - 1` slots of the workspace.
struct DecodePlan {
  bool bf16_k;     // MFMA path (bf16 cache) or fp32 VALU path
  int gc;          // column groups
  int dc;          // columns per group (multiple of 256 on the MFMA path)
  int nw;          // waves per workgroup (MFMA path)
  int nch;         // token chunks
  int nslots;      // partial slots
  int proj_rows;   // W_KV rows per finish workgroup (proj_rows(dh, large or not))
  int spw;         // sequences per finish workgroup (finish_seqs)
  int npc;         // W_KV row blocks of the finish (proj_rows rows each)
  bool ubf16;      // partials U stored in bf16 (bf16 caches), else fp32
  size_t off_U;    // [H, nslots, d] bf16 or float: unnormalised softmax.K rows per chunk
  size_t off_ml;   // [nslots, 2, H] float (running max in log2 units, normaliser)
  size_t off_op;   // [npc, B, H, dh] float (per-row-block projection partials)
  bool xchg;       // two equal column groups whose workgroups exchange scores
  size_t off_mbox; // [nch, 2, 8, 8, 16] u64 score mailboxes of the exchange
  size_t off_status;   // u32 status word (0 = ok); cleared by the attend, set by the finish
  size_t off_tickets;  // u64 arrival counter of the exchange workgroups
  size_t bytes;
};

struct DecodeArgs {
  const float* q;
  const void* K;
  const int32_t* lengths;
  const void* W;
  float* out;
  int B, H, dh, d, T_max, nslots;
  float scale;
  bool w_bf16;
  char* ws;
  uint32_t* status;  // workspace status word (decode and step), or null
};

// W_KV rows per finish workgroup: a multiple of the projection's row subsets
// (256 threads / (dh/8) column groups).  The large block (256 rows, 1 KB of
// a partial row per slot) is fastest when the grid fills the device; the
// small one (64 rows, or the row-subset count) gives small problems four
// times the workgroups.  dh = 256 keeps 64 rows to stay out of spills.
constexpr int proj_rows(int dh, bool large) {
  return dh > 128 ? 64 : (large ? 256 : (256 / (dh >= 8 ? dh / 8 : 1) > 64 ? 256 / (dh >= 8 ? dh / 8 : 1) : 64));
}
// Sequences per finish workgroup: 16 (W_KV read once per 16 sequences) while
// that grid still gives every compute unit two workgroups, else 8.
inline int finish_seqs(int H, int npc_big, long long B, int ncu) {
  return B > 8 && (long long)H * npc_big * ((B + 15) / 16) >= 2LL * ncu ? 16 : 8;
}
constexpr int kMfmaUnitCols = 256; // K columns per MFMA unit (32 lanes x 8 columns)
constexpr int kStepTokens = 8;     // tokens per MFMA step (32x32x8)

bool make_decode_plan(int B, int H, int dh, int T_max, bool bf16_k, int ncu, DecodePlan* p);

hipError_t launch_attend_bf16(const DecodePlan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_attend_f32(const DecodePlan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_finish(const DecodePlan& p, const DecodeArgs& a, hipStream_t s);

// comparator (explicit K and V caches)
struct KVPlan {
  int nch, nslots;
  size_t off_o, off_ml, bytes;
};
bool make_kv_plan(int B, int H, int dh, int T_max, int ncu, KVPlan* p);
hipError_t launch_mha_kv(const KVPlan& p, const float* q, const void* K, const void* V,
                         const int32_t* lengths, float* out, int B, int H, int dh, int T_max,
                         float scale, char* ws, hipStream_t s);

hipError_t launch_prefill_bf16(const void* X, const void* W, void* Kc, int B, int n, int d,
                               int T_max, const int32_t* t0, hipStream_t s);
hipError_t launch_prefill_f32(const void* X, const void* W, void* Kc, int B, int n, int d,
                              int T_max, const int32_t* t0, hipStream_t s);

int probe_sink_floats();
hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

int env_int(const char* name, int dflt);

}  // namespace slim
