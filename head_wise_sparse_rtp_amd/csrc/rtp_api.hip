// C ABI of librtp (declared in include/rtp.h): argument validation, workspace
// planning and the launch sequence of each entry point.
#include "../../include/rtp.h"
#include "rtp_internal.h"

#include <cmath>
#include <cstring>

using namespace rtp;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }
bool opt_ptr_ok(const void* p) { return p == nullptr || aligned16(p); }
bool dtype_ok(int32_t t) { return t == RTP_F32 || t == RTP_F16 || t == RTP_BF16; }

bool pow2_width(float w) {
  if (!(w > 0.0f) || !std::isfinite(w)) return false;
  int e = 0;
  const float m = std::frexp(w, &e);
  return m == 0.5f && e >= -9 && e <= 1;  // 2^-10 .. 1
}

// the attention scale is a softmax temperature: positive and finite (the MFMA tile takes
// each row maximum on the raw products, which needs a positive scale)
bool scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }

rtp_status hip_status(hipError_t e) { return e == hipSuccess ? RTP_OK : RTP_EHIP; }

HeadMap identity_map(int n) {
  HeadMap m{};
  m.n = n;
  for (int i = 0; i < n && i < kMaxHkv; i++) m.kv[i] = i;
  return m;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Rows of query heads over the batch (B x heads) are a launch's y or z grid dimension, or a
// factor of its one-dimensional block count; 65535 bounds the former and keeps the latter
// far inside an int.
constexpr int64_t kMaxRows = 65535;
bool rows_ok(int64_t B, int64_t heads) { return B * heads <= kMaxRows; }

// --- shared size checks -------------------------------------------------------
rtp_status check_common(int32_t B, int32_t G, int32_t Lmax) {
  if (B < 1 || Lmax < 1) return RTP_EINVAL;
  if (G < 1 || G > kMaxG || Lmax > (1 << 24)) return RTP_EUNSUPPORTED;
  return RTP_OK;
}

// --- workspace layouts ----------------------------------------------------------
struct SelectPlan {
  ChunkGeom cg;
  size_t offs[7];
  size_t bytes;
};

SelectPlan plan_topp(int B, int H, int Lmax, int64_t units) {
  SelectPlan sp;
  sp.cg = chunk_geom(units, Lmax);
  WsPlanner wp;
  sp.bytes = round256(plan_select(wp, B, H, Lmax, sp.cg, sp.offs));
  return sp;
}

struct PartPlan {
  size_t m, l, acc, bytes;
};

PartPlan plan_parts(size_t base, size_t rows, int maxs) {
  WsPlanner wp;
  wp.off = base;
  PartPlan pp;
  pp.m = wp.take<float>(rows * maxs);
  pp.l = wp.take<float>(rows * maxs);
  pp.acc = wp.take<float>(rows * maxs * kD);
  pp.bytes = round256(wp.off);
  return pp;
}

AttnPartials bind_parts(char* ws, const PartPlan& pp) {
  AttnPartials a;
  a.m = reinterpret_cast<float*>(ws + pp.m);
  a.l = reinterpret_cast<float*>(ws + pp.l);
  a.acc = reinterpret_cast<float*>(ws + pp.acc);
  return a;
}

int sparse_maxs(int cap) { return cap < 1 ? 1 : (cap + kSplit - 1) / kSplit; }
int window_maxs(int window, int sinks) { return (window + sinks + kWinSplit - 1) / kWinSplit; }

// --- decode step plan -------------------------------------------------------------
struct StepPlan {
  int Hret = 0, Hloc = 0, G = 0;
  bool fused = false;
  StepFusedPlan fp{};
  HeadMap ret{}, loc{};
  SelectPlan sel{};
  size_t sel_idx = 0, sel_cnt = 0;
  PartPlan sparse{}, win{};
  int smaxs = 0, wmaxs = 0;
  size_t bytes = 0;
};

rtp_status plan_step(const rtp_layer_desc* d, StepPlan& sp) {
  if (!d) return RTP_EINVAL;
  if (d->Hkv < 1 || d->Hq < 1 || d->Hq % d->Hkv != 0) return RTP_EINVAL;
  if (d->Hkv > kMaxHkv) return RTP_EUNSUPPORTED;
  sp.G = d->Hq / d->Hkv;
  rtp_status s = check_common(d->B, sp.G, d->Lmax);
  if (s != RTP_OK) return s;
  if (!rows_ok(d->B, d->Hq)) return RTP_EUNSUPPORTED;
  if (d->r != kR || d->d != kD || !dtype_ok(d->kv_dtype)) return RTP_EUNSUPPORTED;
  if (!d->kv_is_retrieval) return RTP_EINVAL;
  sp.ret.n = sp.loc.n = 0;
  for (int h = 0; h < d->Hkv; h++) {
    if (d->kv_is_retrieval[h])
      sp.ret.kv[sp.ret.n++] = h;
    else
      sp.loc.kv[sp.loc.n++] = h;
  }
  sp.Hret = sp.ret.n;
  sp.Hloc = sp.loc.n;
  if (sp.Hloc > 0 && (d->window < 1 || d->sinks < 0)) return RTP_EINVAL;
  if (sp.Hloc > 0 && (int64_t)d->window + d->sinks > (1 << 24)) return RTP_EUNSUPPORTED;
  if (sp.Hret > 0 && d->ret_window && (d->window < 1 || d->sinks < 0)) return RTP_EINVAL;
  if (step_fused_supported(d->kv_dtype, sp.G, sp.Hloc, d->window, d->sinks, d->B, sp.Hret,
                           d->Lmax, d->ret_window != 0)) {
    sp.fused = true;
    WsPlanner wp;
    sp.fp = plan_step_fused(wp, d->B, d->Hq, sp.G, d->Lmax, sp.Hret, sp.Hloc, d->window,
                            d->sinks, d->ret_window != 0, d->sel_idx != nullptr);
    sp.bytes = sp.fp.bytes;
    return RTP_OK;
  }
  size_t off = 0;
  if (sp.Hret > 0) {
    const int H = sp.Hret * sp.G;
    sp.sel = plan_topp(d->B, H, d->Lmax, (int64_t)d->B * sp.Hret);
    WsPlanner wp;
    wp.off = sp.sel.bytes;
    sp.sel_idx = wp.take<int32_t>((size_t)d->B * H * d->Lmax);
    sp.sel_cnt = wp.take<int32_t>((size_t)d->B * H);
    sp.smaxs = sparse_maxs(d->Lmax);
    sp.sparse = plan_parts(round256(wp.off), (size_t)d->B * H, sp.smaxs);
    off = sp.sparse.bytes;
  }
  if (sp.Hloc > 0) {
    sp.wmaxs = window_maxs(d->window, d->sinks);
    sp.win = plan_parts(off, (size_t)d->B * sp.Hloc * sp.G, sp.wmaxs);
    off = sp.win.bytes;
  }
  sp.bytes = off < 256 ? 256 : off;
  return RTP_OK;
}

// The standalone cache update's arguments for a layer descriptor with an append group.
AppendArgs append_args_of(const rtp_layer_desc* d, const rtp_step_append* ap) {
  AppendArgs a{};
  a.B = d->B;
  a.Hq = d->Hq;
  a.Hkv = d->Hkv;
  a.G = d->Hq / d->Hkv;
  a.Lmax = d->Lmax;
  a.window = d->window;
  a.sinks = d->sinks;
  for (int h = 0; h < d->Hkv; h++) {
    a.is_ret[h] = d->kv_is_retrieval[h] ? 1 : 0;
    a.rank[h] = a.is_ret[h] ? a.Hret++ : a.Hloc++;
  }
  a.seq_lens = d->seq_lens;
  a.q_pre = ap->q_pre;
  a.k_pre = ap->k_pre;
  a.Wq = ap->Wq_idx;
  a.Wk = ap->Wk_idx;
  a.k_new = ap->k_new;
  a.v_new = ap->v_new;
  a.q_idx = const_cast<float*>(d->q_idx);
  a.k_idx = const_cast<void*>(d->k_idx);
  a.K_ret = const_cast<void*>(d->K_ret);
  a.V_ret = const_cast<void*>(d->V_ret);
  a.K_loc = const_cast<void*>(d->K_loc);
  a.V_loc = const_cast<void*>(d->V_loc);
  return a;
}

}  // namespace

extern "C" {

const char* rtp_status_string(rtp_status s) {
  switch (s) {
    case RTP_OK: return "RTP_OK: success";
    case RTP_EINVAL: return "RTP_EINVAL: invalid argument (null or misaligned pointer, bad size or parameter)";
    case RTP_EUNSUPPORTED: return "RTP_EUNSUPPORTED: unsupported shape or dtype (r must be 16, d 128, G <= 64, Lmax <= 2^24, B x query heads <= 65535)";
    case RTP_EWORKSPACE: return "RTP_EWORKSPACE: workspace smaller than the size query";
    case RTP_EHIP: return "RTP_EHIP: a HIP kernel launch failed";
    case RTP_ESCRATCH: return "RTP_ESCRATCH: the step needs more scratch than the library's fixed buffer holds (use rtp_decode_step with a workspace)";
    default: return "unknown rtp_status";
  }
}

int32_t rtp_abi_version(void) { return RTP_ABI_VERSION; }

rtp_status rtp_index_score(const float* q_idx, const void* k_idx, int32_t k_dtype,
                           const int32_t* seq_lens, int32_t B, int32_t Hr, int32_t G,
                           int32_t Lmax, int32_t r, float scale_idx, float* z, void* stream) {
  rtp_status s = check_common(B, G, Lmax);
  if (s != RTP_OK) return s;
  if (Hr < 1) return RTP_EINVAL;
  if (r != kR || !dtype_ok(k_dtype) || !rows_ok(B, (int64_t)Hr * G)) return RTP_EUNSUPPORTED;
  if (!ptr_ok(q_idx) || !ptr_ok(k_idx) || !ptr_ok(seq_lens) || !ptr_ok(z)) return RTP_EINVAL;
  if (!std::isfinite(scale_idx)) return RTP_EINVAL;
  return hip_status(launch_index_score(q_idx, k_idx, k_dtype, seq_lens, B, Hr, G, Lmax,
                                       scale_idx, z, (hipStream_t)stream));
}

size_t rtp_topp_select_workspace_size(int32_t B, int32_t H, int32_t Lmax) {
  if (B < 1 || H < 1 || Lmax < 1 || Lmax > (1 << 24) || !rows_ok(B, H)) return 0;
  return plan_topp(B, H, Lmax, (int64_t)B * H).bytes;
}

rtp_status rtp_topp_select(const float* z, const int32_t* seq_lens, int32_t B, int32_t H,
                           int32_t Lmax, double p, float bin_width, int32_t* sel_idx,
                           int32_t* sel_count, int32_t cap, float* hist, int32_t* thresh,
                           void* ws, size_t ws_bytes, void* stream) {
  if (B < 1 || H < 1 || Lmax < 1 || cap < 0) return RTP_EINVAL;
  if (Lmax > (1 << 24) || !rows_ok(B, H)) return RTP_EUNSUPPORTED;
  if (!(p > 0.0) || std::isnan(p)) return RTP_EINVAL;
  if (!pow2_width(bin_width)) return RTP_EINVAL;
  if (!ptr_ok(z) || !ptr_ok(seq_lens) || !ptr_ok(sel_count) || !ptr_ok(ws)) return RTP_EINVAL;
  if (cap > 0 && !ptr_ok(sel_idx)) return RTP_EINVAL;
  if (!opt_ptr_ok(hist) || !opt_ptr_ok(thresh)) return RTP_EINVAL;
  const SelectPlan sp = plan_topp(B, H, Lmax, (int64_t)B * H);
  if (ws_bytes < sp.bytes) return RTP_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const SelectBufs sb = bind_select(static_cast<char*>(ws), sp.offs);
  hipError_t e = launch_hist_from_z(z, seq_lens, B, H, Lmax, bin_width, false, sp.cg, sb, st);
  if (e == hipSuccess)
    e = launch_threshold(seq_lens, B, H, Lmax, p, 0, bin_width, sp.cg, sb, hist, thresh, nullptr,
                         1, H, st);
  if (e == hipSuccess)
    e = launch_select(seq_lens, B, H, Lmax, sp.cg, sb, sel_idx, sel_count, cap, nullptr, nullptr,
                      1, H, st);
  return hip_status(e);
}

size_t rtp_topk_select_workspace_size(int32_t B, int32_t H, int32_t Lmax) {
  return rtp_topp_select_workspace_size(B, H, Lmax);
}

rtp_status rtp_topk_select(const float* z, const int32_t* seq_lens, int32_t B, int32_t H,
                           int32_t Lmax, int32_t k, float bin_width, int32_t* sel_idx,
                           int32_t* sel_count, int32_t cap, float* hist, int32_t* thresh,
                           void* ws, size_t ws_bytes, void* stream) {
  if (B < 1 || H < 1 || Lmax < 1 || cap < 0 || k < 1) return RTP_EINVAL;
  if (Lmax > (1 << 24) || !rows_ok(B, H)) return RTP_EUNSUPPORTED;
  if (!pow2_width(bin_width)) return RTP_EINVAL;
  if (!ptr_ok(z) || !ptr_ok(seq_lens) || !ptr_ok(sel_count) || !ptr_ok(ws)) return RTP_EINVAL;
  if (cap > 0 && !ptr_ok(sel_idx)) return RTP_EINVAL;
  if (!opt_ptr_ok(hist) || !opt_ptr_ok(thresh)) return RTP_EINVAL;
  const SelectPlan sp = plan_topp(B, H, Lmax, (int64_t)B * H);
  if (ws_bytes < sp.bytes) return RTP_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const SelectBufs sb = bind_select(static_cast<char*>(ws), sp.offs);
  hipError_t e = launch_hist_from_z(z, seq_lens, B, H, Lmax, bin_width, true, sp.cg, sb, st);
  if (e == hipSuccess)
    e = launch_threshold(seq_lens, B, H, Lmax, 1.0, k, bin_width, sp.cg, sb, hist, thresh,
                         nullptr, 1, H, st);
  if (e == hipSuccess)
    e = launch_select(seq_lens, B, H, Lmax, sp.cg, sb, sel_idx, sel_count, cap, nullptr, nullptr,
                      1, H, st);
  return hip_status(e);
}

size_t rtp_sparse_decode_workspace_size(int32_t B, int32_t Hr, int32_t G, int32_t cap) {
  if (B < 1 || Hr < 1 || G < 1 || cap < 0 || !rows_ok(B, (int64_t)Hr * G)) return 0;
  return plan_parts(0, (size_t)B * Hr * G, sparse_maxs(cap)).bytes;
}

rtp_status rtp_sparse_decode(const void* q, const void* K, const void* V, int32_t kv_dtype,
                             const int32_t* sel_idx, const int32_t* sel_count, int32_t cap,
                             int32_t B, int32_t Hr, int32_t G, int32_t Lmax, int32_t d,
                             float scale_attn, float* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  rtp_status s = check_common(B, G, Lmax);
  if (s != RTP_OK) return s;
  if (Hr < 1 || cap < 0) return RTP_EINVAL;
  if (Hr > kMaxHkv || !rows_ok(B, (int64_t)Hr * G)) return RTP_EUNSUPPORTED;
  if (d != kD || !dtype_ok(kv_dtype)) return RTP_EUNSUPPORTED;
  if (!ptr_ok(q) || !ptr_ok(K) || !ptr_ok(V) || !ptr_ok(sel_count) || !ptr_ok(out) ||
      !ptr_ok(ws))
    return RTP_EINVAL;
  if (cap > 0 && !ptr_ok(sel_idx)) return RTP_EINVAL;
  if (!opt_ptr_ok(lse) || !scale_ok(scale_attn)) return RTP_EINVAL;
  const int maxs = sparse_maxs(cap);
  const PartPlan pp = plan_parts(0, (size_t)B * Hr * G, maxs);
  if (ws_bytes < pp.bytes) return RTP_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const AttnPartials pa = bind_parts(static_cast<char*>(ws), pp);
  const HeadMap map = identity_map(Hr);
  hipError_t e = launch_sparse_partial(q, K, V, kv_dtype, sel_idx, sel_count, cap, map, B, Hr * G,
                                       Hr, G, Lmax, scale_attn, pa, maxs, st);
  if (e == hipSuccess) e = launch_merge(pa, maxs, sel_count, cap, map, B, Hr * G, Hr, G, out, lse, st);
  return hip_status(e);
}

size_t rtp_window_decode_workspace_size(int32_t B, int32_t Hl, int32_t G, int32_t window,
                                        int32_t sinks) {
  if (B < 1 || Hl < 1 || G < 1 || window < 1 || sinks < 0 || !rows_ok(B, (int64_t)Hl * G)) return 0;
  return plan_parts(0, (size_t)B * Hl * G, window_maxs(window, sinks)).bytes;
}

rtp_status rtp_window_decode(const void* q, const void* K, const void* V, int32_t kv_dtype,
                             const int32_t* seq_lens, int32_t B, int32_t Hl, int32_t G,
                             int32_t d, int32_t window, int32_t sinks, float scale_attn,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (B < 1 || Hl < 1 || window < 1 || sinks < 0) return RTP_EINVAL;
  if (G < 1 || G > kMaxG || Hl > kMaxHkv || (int64_t)window + sinks > (1 << 24) ||
      !rows_ok(B, (int64_t)Hl * G))
    return RTP_EUNSUPPORTED;
  if (d != kD || !dtype_ok(kv_dtype)) return RTP_EUNSUPPORTED;
  if (!ptr_ok(q) || !ptr_ok(K) || !ptr_ok(V) || !ptr_ok(seq_lens) || !ptr_ok(out) || !ptr_ok(ws))
    return RTP_EINVAL;
  if (!opt_ptr_ok(lse) || !scale_ok(scale_attn)) return RTP_EINVAL;
  const int maxs = window_maxs(window, sinks);
  const PartPlan pp = plan_parts(0, (size_t)B * Hl * G, maxs);
  if (ws_bytes < pp.bytes) return RTP_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const AttnPartials pa = bind_parts(static_cast<char*>(ws), pp);
  const HeadMap map = identity_map(Hl);
  hipError_t e = launch_window_partial(q, K, V, kv_dtype, seq_lens, map, B, Hl * G, Hl, G, window,
                                       sinks, scale_attn, pa, maxs, st);
  if (e == hipSuccess) e = launch_merge(pa, maxs, nullptr, 0, map, B, Hl * G, Hl, G, out, lse, st);
  return hip_status(e);
}

rtp_status rtp_append_project(const rtp_append_desc* d, void* stream) {
  if (!d) return RTP_EINVAL;
  if (d->B < 1 || d->Lmax < 1 || d->Hkv < 1 || d->Hq < 1 || d->Hq % d->Hkv != 0)
    return RTP_EINVAL;
  const int G = d->Hq / d->Hkv;
  if (G > kMaxG || d->Hkv > kMaxHkv || d->Lmax > (1 << 24) || !rows_ok(d->B, d->Hq))
    return RTP_EUNSUPPORTED;
  if (d->r != kR || d->d != kD || !dtype_ok(d->kv_dtype)) return RTP_EUNSUPPORTED;
  if (!d->kv_is_retrieval) return RTP_EINVAL;
  AppendArgs a{};
  a.B = d->B;
  a.Hq = d->Hq;
  a.Hkv = d->Hkv;
  a.G = G;
  a.Lmax = d->Lmax;
  a.window = d->window;
  a.sinks = d->sinks;
  for (int h = 0; h < d->Hkv; h++) {
    a.is_ret[h] = d->kv_is_retrieval[h] ? 1 : 0;
    a.rank[h] = a.is_ret[h] ? a.Hret++ : a.Hloc++;
  }
  if (!ptr_ok(d->k_new) || !ptr_ok(d->v_new) || !ptr_ok(d->seq_lens)) return RTP_EINVAL;
  if (a.Hret > 0 && (!ptr_ok(d->q_pre) || !ptr_ok(d->k_pre) || !ptr_ok(d->Wq_idx) ||
                     !ptr_ok(d->Wk_idx) || !ptr_ok(d->q_idx) || !ptr_ok(d->k_idx) ||
                     !ptr_ok(d->K_ret) || !ptr_ok(d->V_ret)))
    return RTP_EINVAL;
  if (a.Hloc > 0) {
    if (d->window < 1 || d->sinks < 0) return RTP_EINVAL;
    if ((int64_t)d->window + d->sinks > (1 << 24)) return RTP_EUNSUPPORTED;
    if (!ptr_ok(d->K_loc) || !ptr_ok(d->V_loc)) return RTP_EINVAL;
  }
  a.seq_lens = d->seq_lens;
  a.q_pre = d->q_pre;
  a.k_pre = d->k_pre;
  a.Wq = d->Wq_idx;
  a.Wk = d->Wk_idx;
  a.k_new = d->k_new;
  a.v_new = d->v_new;
  a.q_idx = d->q_idx;
  a.k_idx = d->k_idx;
  a.K_ret = d->K_ret;
  a.V_ret = d->V_ret;
  a.K_loc = d->K_loc;
  a.V_loc = d->V_loc;
  return hip_status(launch_append_project(a, d->kv_dtype, (hipStream_t)stream));
}

rtp_status rtp_prefill(const rtp_prefill_desc* d, void* stream) {
  if (!d) return RTP_EINVAL;
  if (d->B < 1 || d->Lmax < 1 || d->Hkv < 1 || d->Hq < 1 || d->Hq % d->Hkv != 0)
    return RTP_EINVAL;
  const int G = d->Hq / d->Hkv;
  if (G > kMaxG || d->Hkv > kMaxHkv || d->Lmax > (1 << 24)) return RTP_EUNSUPPORTED;
  // its launches are one-dimensional, B * Hkv * (blocks per sequence) blocks: at most 2^31 - 1
  // with a block per 16 prompt rows
  if (!rows_ok(d->B, d->Hq) || (int64_t)d->B * d->Hkv * ((d->Lmax + 15) / 16) > INT32_MAX)
    return RTP_EUNSUPPORTED;
  if (d->r != kR || d->d != kD || (d->kv_dtype != RTP_F16 && d->kv_dtype != RTP_BF16))
    return RTP_EUNSUPPORTED;
  if (!d->kv_is_retrieval || !scale_ok(d->scale_attn)) return RTP_EINVAL;
  PrefillArgs a{};
  a.B = d->B;
  a.Hq = d->Hq;
  a.Hkv = d->Hkv;
  a.G = G;
  a.Lmax = d->Lmax;
  a.window = d->window;
  a.sinks = d->sinks;
  for (int h = 0; h < d->Hkv; h++) {
    a.is_ret[h] = d->kv_is_retrieval[h] ? 1 : 0;
    a.rank[h] = a.is_ret[h] ? a.Hret++ : a.Hloc++;
  }
  if (!ptr_ok(d->q) || !ptr_ok(d->K) || !ptr_ok(d->V) || !ptr_ok(d->seq_lens) || !ptr_ok(d->out))
    return RTP_EINVAL;
  if (a.Hloc > 0) {
    if (d->window < 1 || d->sinks < 0) return RTP_EINVAL;
    if ((int64_t)d->window + d->sinks > (1 << 24)) return RTP_EUNSUPPORTED;
  }
  // optional decode state: each group all present or all absent
  if (!opt_ptr_ok(d->k_idx) || !opt_ptr_ok(d->K_ret) || !opt_ptr_ok(d->V_ret) ||
      !opt_ptr_ok(d->K_loc) || !opt_ptr_ok(d->V_loc))
    return RTP_EINVAL;
  if ((d->K_ret == nullptr) != (d->V_ret == nullptr) || (d->K_loc == nullptr) != (d->V_loc == nullptr))
    return RTP_EINVAL;
  if (d->k_idx && (!ptr_ok(d->k_pre) || !ptr_ok(d->Wk_idx))) return RTP_EINVAL;
  a.seq_lens = d->seq_lens;
  a.q = d->q;
  a.K = d->K;
  a.V = d->V;
  a.scale2 = d->scale_attn * 1.4426950408889634f;
  a.out = d->out;
  a.k_pre = d->k_pre;
  a.Wk = d->Wk_idx;
  a.k_idx = a.Hret > 0 ? d->k_idx : nullptr;
  a.K_ret = a.Hret > 0 ? d->K_ret : nullptr;
  a.V_ret = a.Hret > 0 ? d->V_ret : nullptr;
  a.K_loc = a.Hloc > 0 ? d->K_loc : nullptr;
  a.V_loc = a.Hloc > 0 ? d->V_loc : nullptr;
  return hip_status(launch_prefill(a, d->kv_dtype, (hipStream_t)stream));
}

size_t rtp_decode_step_workspace_size(const rtp_layer_desc* desc) {
  StepPlan sp;
  if (plan_step(desc, sp) != RTP_OK) return 0;
  return sp.bytes;
}

}  // extern "C"

namespace rtp {

rtp_status decode_step_impl(const rtp_layer_desc* d, void* ws, size_t ws_bytes, void* stream,
                            void* const* events) {
  StepPlan sp;
  rtp_status s = plan_step(d, sp);
  if (s != RTP_OK) return s;
  if (!ptr_ok(d->q) || !ptr_ok(d->seq_lens) || !ptr_ok(d->out) || !ptr_ok(ws)) return RTP_EINVAL;
  if (!opt_ptr_ok(d->lse) || !opt_ptr_ok(d->thresh_out) || !opt_ptr_ok(d->count_out))
    return RTP_EINVAL;
  if (!scale_ok(d->scale_attn) || !std::isfinite(d->scale_idx)) return RTP_EINVAL;
  if (sp.Hret > 0) {
    if (!ptr_ok(d->q_idx) || !ptr_ok(d->K_ret) || !ptr_ok(d->V_ret) || !ptr_ok(d->k_idx))
      return RTP_EINVAL;
    if (d->topk < 0 || !pow2_width(d->bin_width)) return RTP_EINVAL;
    if (d->ret_window != 0 && d->ret_window != 1) return RTP_EINVAL;
    if (d->ret_window && (d->window < 1 || d->sinks < 0)) return RTP_EINVAL;
    if (d->topk == 0 && (!(d->p > 0.0) || std::isnan(d->p))) return RTP_EINVAL;
  }
  if (sp.Hloc > 0 && (!ptr_ok(d->K_loc) || !ptr_ok(d->V_loc))) return RTP_EINVAL;
  if ((d->sel_idx == nullptr) != (d->sel_count == nullptr)) return RTP_EINVAL;
  const rtp_step_append* ap = d->append;
  if (ap) {
    if (!ptr_ok(ap->k_new) || !ptr_ok(ap->v_new)) return RTP_EINVAL;
    if (sp.Hret > 0 && (!ptr_ok(ap->q_pre) || !ptr_ok(ap->k_pre) || !ptr_ok(ap->Wq_idx) ||
                        !ptr_ok(ap->Wk_idx)))
      return RTP_EINVAL;
  }
  if (d->sel_idx && (!ptr_ok(d->sel_idx) || !ptr_ok(d->sel_count) || d->sel_cap < 1))
    return RTP_EINVAL;
  if (ws_bytes < sp.bytes) return RTP_EWORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  hipError_t e = hipSuccess;
  const int G = sp.G;
  if (sp.fused) {
    StepFusedArgs a{};
    a.B = d->B;
    a.Hq = d->Hq;
    a.Lmax = d->Lmax;
    a.window = d->window;
    a.sinks = d->sinks;
    a.kv_dtype = d->kv_dtype;
    a.seq_lens = d->seq_lens;
    a.q = d->q;
    a.q_idx = d->q_idx;
    a.K_ret = d->K_ret;
    a.V_ret = d->V_ret;
    a.k_idx = d->k_idx;
    a.K_loc = d->K_loc;
    a.V_loc = d->V_loc;
    a.ret = sp.ret;
    a.loc = sp.loc;
    a.p = d->p;
    a.topk = d->topk;
    a.ret_window = d->ret_window;
    a.bin_width = d->bin_width;
    a.scale_idx = d->scale_idx;
    a.scale_attn = d->scale_attn;
    a.out = d->out;
    a.lse = d->lse;
    a.hist_out = nullptr;
    a.thresh_out = d->thresh_out;
    a.count_out = d->count_out;
    a.sel_idx = d->sel_idx;
    a.sel_count = d->sel_count;
    a.sel_cap = d->sel_cap;
    a.Hkv = d->Hkv;
    // the cache update runs inside stage A; without retrieval heads there is no stage A,
    // and the standalone update kernel runs first
    a.app = sp.Hret > 0 ? ap : nullptr;
    if (ap && sp.Hret == 0) {
      const hipError_t ea = launch_append_project(append_args_of(d, ap), d->kv_dtype, st);
      if (ea != hipSuccess) return RTP_EHIP;
    }
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (events)
      for (int i = 0; i < 4; i++) ev[i] = (hipEvent_t)events[i];
    return hip_status(launch_step_fused(sp.fp, w, a, st, events ? ev : nullptr));
  }
  auto mark = [&](int i) {
    if (e == hipSuccess && events && events[i]) e = hipEventRecord((hipEvent_t)events[i], st);
  };
  if (ap) e = launch_append_project(append_args_of(d, ap), d->kv_dtype, st);
  if (sp.Hloc > 0) {
    const AttnPartials pa = bind_parts(w, sp.win);
    if (e == hipSuccess)
      e = launch_window_partial(d->q, d->K_loc, d->V_loc, d->kv_dtype, d->seq_lens, sp.loc, d->B,
                              d->Hq, sp.Hloc, G, d->window, d->sinks, d->scale_attn, pa, sp.wmaxs,
                              st);
    if (e == hipSuccess)
      e = launch_merge(pa, sp.wmaxs, nullptr, 0, sp.loc, d->B, d->Hq, sp.Hloc, G, d->out, d->lse,
                       st);
  }
  if (e == hipSuccess && sp.Hret > 0) {
    const int H = sp.Hret * G;
    const SelectBufs sb = bind_select(w, sp.sel.offs);
    int32_t* sel_idx = reinterpret_cast<int32_t*>(w + sp.sel_idx);
    int32_t* sel_cnt = reinterpret_cast<int32_t*>(w + sp.sel_cnt);
    mark(0);
    if (e == hipSuccess)
      e = launch_hist_from_kidx(d->q_idx, d->k_idx, d->kv_dtype, d->seq_lens, sp.ret, d->B,
                                d->Hq, sp.Hret, G, d->Lmax, d->scale_idx, d->bin_width,
                                d->topk > 0, sp.sel.cg, sb, st);
    mark(1);
    if (e == hipSuccess)
      e = launch_threshold(d->seq_lens, d->B, H, d->Lmax, d->p, d->topk, d->bin_width, sp.sel.cg,
                           sb, nullptr, d->thresh_out, &sp.ret, G, d->Hq, st);
    if (e == hipSuccess)
      e = launch_select(d->seq_lens, d->B, H, d->Lmax, sp.sel.cg, sb, sel_idx, sel_cnt, d->Lmax,
                        d->count_out, &sp.ret, G, d->Hq, st, d->ret_window ? d->sinks : 0,
                        d->ret_window ? d->window : 0);
    const AttnPartials pa = bind_parts(w, sp.sparse);
    mark(2);
    if (e == hipSuccess)
      e = launch_sparse_partial(d->q, d->K_ret, d->V_ret, d->kv_dtype, sel_idx, sel_cnt, d->Lmax,
                                sp.ret, d->B, d->Hq, sp.Hret, G, d->Lmax, d->scale_attn, pa,
                                sp.smaxs, st);
    mark(3);
    if (e == hipSuccess)
      e = launch_merge(pa, sp.smaxs, sel_cnt, d->Lmax, sp.ret, d->B, d->Hq, sp.Hret, G, d->out,
                       d->lse, st);
    if (e == hipSuccess && d->sel_idx)
      e = launch_export_sets(sel_idx, sel_cnt, d->Lmax, sp.ret, d->B, d->Hq, sp.Hret, G,
                             d->sel_idx, d->sel_count, d->sel_cap, st);
  }
  return hip_status(e);
}

}  // namespace rtp

extern "C" {

rtp_status rtp_decode_step(const rtp_layer_desc* d, void* ws, size_t ws_bytes, void* stream) {
  return decode_step_impl(d, ws, ws_bytes, stream, nullptr);
}

rtp_status rtp_decode_step_profiled(const rtp_layer_desc* d, void* ws, size_t ws_bytes,
                                    void* stream, void* const events[4]) {
  return decode_step_impl(d, ws, ws_bytes, stream, events);
}



}  // extern "C"
