// Internal declarations of librtp: device helpers, launch wrappers and the
// workspace planner.  Nothing here is part of the public C ABI (include/rtp.h).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/rtp.h"

#include <climits>
#include <cstddef>
#include <cstdint>

namespace rtp {

constexpr int kNB = 256;        // histogram bins per head (1 KB of fp32 masses)
constexpr int kR = 16;          // indexer size
constexpr int kD = 128;         // head size
constexpr int kMaxHkv = 64;     // KV heads per layer
constexpr int kMaxG = 64;       // query heads per KV head
constexpr int kThreads = 256;   // threads per block of the streaming kernels
constexpr int kSplit = 64;      // selected tokens per sparse-attention work item
constexpr int kWinSplit = 128;  // window rows per window-attention work item
constexpr int kMerge1 = 16;     // chunk partials merged by one first-level merge block
constexpr int kEmptyCell = INT_MIN;

typedef _Float16 f16;
typedef uint16_t bf16s;  // bfloat16 storage: the upper 16 bits of an fp32

__device__ __forceinline__ float bf16_to_f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
// round to nearest, ties to even (finite inputs)
__device__ __forceinline__ bf16s f_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return (bf16s)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Row space of the retrieval kernels: row = kr * G + g for packed retrieval KV head
// kr and query head g of that KV head.  `kv[kr]` is the KV head id in the layer, used
// to address q / q_idx / out, whose head index is kv * G + g.
struct HeadMap {
  int32_t n;
  int32_t kv[kMaxHkv];
};

// ---------------------------------------------------------------------------
// chunk geometry of the histogram pass
// ---------------------------------------------------------------------------
struct ChunkGeom {
  int tpt;     // tokens per thread (4, 8 or 16)
  int tc;      // tokens per chunk = kThreads * tpt
  int nchunk;  // chunks per row = ceil(Lmax / tc)
  int nsplit;  // first-level merge blocks per row = ceil(nchunk / kMerge1)
};
ChunkGeom chunk_geom(int64_t rows_times_batch, int64_t Lmax);

// ---------------------------------------------------------------------------
// device buffers of the selection pipeline (all inside the caller's workspace)
// ---------------------------------------------------------------------------
struct SelectBufs {
  float* part_mass;     // [BH, nchunk, 256] chunk-relative bin masses
  int32_t* part_A;      // [BH, nchunk] chunk top cell (kEmptyCell when no token)
  uint32_t* codes;      // [BH, nchunk, tc/4, 4 bytes] chunk-relative bin of each token
  double* mid_mass;     // [BH, nsplit, 256] first-level merged masses
  int32_t* mid_A;       // [BH, nsplit]
  int32_t* thr;         // [BH, 4] = {A, b*, valid, pad}
  int32_t* cnt;         // [BH, nchunk] selected tokens per chunk
};

struct AttnPartials {
  float* m;    // [rows, maxs] running max of the scaled logits
  float* l;    // [rows, maxs] sum of exp(s - m)
  float* acc;  // [rows, maxs, d] sum of exp(s - m) * v
};

// ---------------------------------------------------------------------------
// launch wrappers (each returns the hipError_t of its launch)
// ---------------------------------------------------------------------------
hipError_t launch_index_score(const float* q_idx, const void* k_idx, int k_dtype,
                              const int32_t* seq_lens, int B, int Hr, int G, int Lmax,
                              float scale_idx, float* z, hipStream_t st);

// Histogram partials; mode 0 reads logits z [B, H, Lmax], mode 1 computes them from
// q_idx / k_idx (rows kr*G+g; q_idx head index map.kv[kr]*G+g of a [B, Hq, r] array).
// counts: every token weighs one (fixed top-k) instead of its softmax mass.
hipError_t launch_hist_from_z(const float* z, const int32_t* seq_lens, int B, int H, int Lmax,
                              float bin_width, bool counts, const ChunkGeom& cg,
                              const SelectBufs& sb, hipStream_t st);
hipError_t launch_hist_from_kidx(const float* q_idx, const void* k_idx, int k_dtype,
                                 const int32_t* seq_lens, const HeadMap& map, int B, int Hq,
                                 int Hr, int G, int Lmax, float scale_idx, float bin_width,
                                 bool counts, const ChunkGeom& cg, const SelectBufs& sb,
                                 hipStream_t st);

// b* per row: the least bin whose cumulative mass reaches p Z (topk == 0), or whose
// cumulative count reaches topk (topk > 0, histograms built with counts = true).
hipError_t launch_threshold(const int32_t* seq_lens, int B, int H, int Lmax, double p, int topk,
                            float bin_width, const ChunkGeom& cg, const SelectBufs& sb,
                            float* hist_out, int32_t* thresh_out, const HeadMap* out_map,
                            int G, int Hq, hipStream_t st);

// force_window > 0 also keeps every token n < force_sinks or n >= L - force_window
// (retrieval heads that attend to the sinks and the window besides their selected set).
hipError_t launch_select(const int32_t* seq_lens, int B, int H, int Lmax, const ChunkGeom& cg,
                         const SelectBufs& sb, int32_t* sel_idx, int32_t* sel_count, int cap,
                         int32_t* count_out, const HeadMap* out_map, int G, int Hq,
                         hipStream_t st, int force_sinks = 0, int force_window = 0);

// Sparse attention partials over sel_idx rows; rows kr*G+g, q head map.kv[kr]*G+g.
hipError_t launch_sparse_partial(const void* q, const void* K, const void* V, int kv_dtype,
                                 const int32_t* sel_idx, const int32_t* sel_count, int cap,
                                 const HeadMap& map, int B, int Hq, int Hr, int G, int Lmax,
                                 float scale_attn, const AttnPartials& pa, int maxs,
                                 hipStream_t st);

hipError_t launch_window_partial(const void* q, const void* K, const void* V, int kv_dtype,
                                 const int32_t* seq_lens, const HeadMap& map, int B, int Hq,
                                 int Hl, int G, int window, int sinks, float scale_attn,
                                 const AttnPartials& pa, int maxs, hipStream_t st);

// Copy the selected sets of retrieval rows (row kr*G+g, cap_in entries each) into the
// per-query-head arrays out_idx [B, Hq, cap_out] / out_count [B, Hq].
hipError_t launch_export_sets(const int32_t* sel_idx, const int32_t* sel_count, int cap_in,
                              const HeadMap& map, int B, int Hq, int Hr, int G, int32_t* out_idx,
                              int32_t* out_count, int cap_out, hipStream_t st);

// Merge split partials into out [B, Hq, d] / lse [B, Hq].  For sparse rows the number of
// used splits comes from sel_count (ceil(min(count, cap) / kSplit)); otherwise all `maxs`.
hipError_t launch_merge(const AttnPartials& pa, int maxs, const int32_t* sel_count, int cap,
                        const HeadMap& map, int B, int Hq, int Hrows_kv, int G, float* out,
                        float* lse, hipStream_t st);

// Cache update of a decode step (projections of the new token and its K/V rows).
struct AppendArgs {
  int B, Hq, Hkv, G, Hret, Hloc, Lmax, window, sinks;
  const int32_t* seq_lens;  // lengths after the append
  const float* q_pre;       // [B, Hq, 128]
  const float* k_pre;       // [B, Hkv, 128]
  const float* Wq;          // [Hq, 128, 16]
  const float* Wk;          // [Hret, 128, 16]
  const void* k_new;        // [B, Hkv, 128] cache dtype
  const void* v_new;
  float* q_idx;             // [B, Hq, 16]
  void* k_idx;              // [B, Hret, Lmax, 16]
  void* K_ret;
  void* V_ret;              // [B, Hret, Lmax, 128]
  void* K_loc;
  void* V_loc;              // [B, Hloc, sinks + window, 128]
  int32_t is_ret[kMaxHkv];  // per KV head: 1 = retrieval
  int32_t rank[kMaxHkv];    // per KV head: index among the retrieval (or local) heads
};
hipError_t launch_append_project(const AppendArgs& a, int kv_dtype, hipStream_t st);

// Prefill of a prompt (fp16 prompt K/V and queries) and the decode state it leaves.
struct PrefillArgs {
  int B, Hq, Hkv, G, Hret, Hloc, Lmax, window, sinks;
  int ntile;  // query tiles per sequence (set by launch_prefill)
  const int32_t* seq_lens;  // prompt lengths
  const void* q;            // [B, Hq, Lmax, 128] fp16 or bf16 (the K/V type)
  const void* K;            // [B, Hkv, Lmax, 128]
  const void* V;
  float scale2;             // scale_attn * log2(e)
  float* out;               // [B, Hq, Lmax, 128]
  const float* k_pre;       // [B, Hkv, Lmax, 128] (with k_idx)
  const float* Wk;          // [Hret, 128, 16]
  void* k_idx;              // [B, Hret, Lmax, 16] or null (the K/V type)
  void* K_ret;              // [B, Hret, Lmax, 128] or null (with V_ret)
  void* V_ret;
  void* K_loc;              // [B, Hloc, sinks + window, 128] or null (with V_loc)
  void* V_loc;
  int32_t is_ret[kMaxHkv];
  int32_t rank[kMaxHkv];
};
hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, hipStream_t st);

// ---------------------------------------------------------------------------
// workspace planning
// ---------------------------------------------------------------------------
struct WsPlanner {
  size_t off = 0;
  template <typename T>
  size_t take(size_t n) {
    off = (off + 255) & ~size_t(255);
    size_t o = off;
    off += n * sizeof(T);
    return o;
  }
};

// ---------------------------------------------------------------------------
// fused decode step (fp16 caches, G <= 16): stage A (indexer score + chunk histograms),
// stage T (suffix tables), stage B (selection + sparse attention, window attention),
// stage M (merges)
// ---------------------------------------------------------------------------
struct StepFusedPlan {
  int G, Hret, Hloc;
  int tc, nt, nchunk;  // histogram chunk tokens, stage-A threads, chunks per row
  int nwd, tb, nblk;   // selection slices: code words per thread, tokens, slices per KV head
  int nparts;          // selection blocks per slice (they share its attention steps)
  int wrows, nws;      // window blocks: rows per block, blocks per local KV head
  int ncu;             // compute units of the device
  int rwnws, rwrows;   // retrieval window blocks per KV head and their rows (0: none)
  int tcpb, tseg;      // stage-T blocks: chunks per block, blocks per head row
  size_t suf, partA, codes, bstar, Aglob, sufq;
  size_t p1m, p1l, p1acc, p1cnt;
  size_t wpm, wpl, wpacc;
  size_t xlist, xn;  // set export: union lists per slice and their lengths (0: no export)
  bool exp;
  size_t bytes;
};

struct StepFusedArgs {
  int B, Hq, Lmax, window, sinks;
  int kv_dtype;  // 1: fp16, 2: bf16
  const int32_t* seq_lens;
  const void* q;
  const float* q_idx;
  const void *K_ret, *V_ret, *k_idx, *K_loc, *V_loc;
  HeadMap ret, loc;
  double p;
  int topk;        // > 0: fixed top-k (count bins) instead of top-p
  int ret_window;  // retrieval heads also attend to the sinks and the window
  float bin_width, scale_idx, scale_attn;
  float* out;
  float* lse;
  float* hist_out;
  int32_t* thresh_out;
  int32_t* count_out;
  int32_t* sel_idx;  // [B, Hq, sel_cap] or null: the exported sets
  int32_t* sel_count;
  int sel_cap;
  // cache update fused into stage A (app == null: none); the caches above are then written
  const rtp_step_append* app;
  int Hkv;
};

bool step_fused_supported(int kv_dtype, int G, int Hloc, int window, int sinks, int B, int Hret,
                          int Lmax, bool ret_window);
StepFusedPlan plan_step_fused(WsPlanner& wp, int B, int Hq, int G, int Lmax, int Hret, int Hloc,
                              int window, int sinks, bool ret_window, bool export_sets);
// ev (may be null): events bound to the execution of stage A ([0] start, [1] end) and of
// stage B ([2] start, [3] end), each pair only when both of its events are given
hipError_t launch_step_fused(const StepFusedPlan& sp, char* ws, const StepFusedArgs& a,
                             hipStream_t st, hipEvent_t* ev);

// rtp_decode_step on the workspace ws (validation, planning and launches); events may be
// null (see rtp_decode_step_profiled)
rtp_status decode_step_impl(const rtp_layer_desc* d, void* ws, size_t ws_bytes, void* stream,
                            void* const* events);

size_t plan_select(WsPlanner& wp, int B, int H, int Lmax, const ChunkGeom& cg, size_t offs[7]);
SelectBufs bind_select(char* ws, const size_t offs[7]);

}  // namespace rtp
