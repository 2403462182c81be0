/*
 * rtp.h -- C ABI of librtp.so: one RTPurbo decode step on an AMD Instinct MI355X (gfx950).
 *
 * The method (Full Attention Strikes Back: Transferring Full Attention into Sparse
 * within Hundred Training Steps; xllm-io.github.io paper review, section 三 技术架构):
 * retrieval heads score every cached token with a 16-dim pre-RoPE indexer, keep a
 * top-p set of tokens chosen through a 256-bin histogram without sorting, and run
 * exact softmax attention over that set; local heads attend over a sliding window
 * plus sink tokens (section 五, test-configuration table: window 8192, 4 sinks,
 * indexer size 16, p = 0.9, 15% retrieval heads).  A fixed top-k budget through the
 * same histogram (section 三, insight 3) is offered beside top-p.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer to a dense row-major array whose
 *     shape is given next to it; all base pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *     enqueue work: they never allocate, free or synchronise, and keep no mutable
 *     global state.  Calls on different streams must use different workspaces.
 *   - The caller owns every buffer.  Workspace sizes come from the matching
 *     *_workspace_size() query; a smaller `ws_bytes` returns RTP_EWORKSPACE.
 *   - Arguments are validated on the host before anything is enqueued; an invalid
 *     argument returns an error and enqueues nothing.  Device-resident values
 *     (seq_lens, sel_idx, sel_count) cannot be checked on the host: kernels clamp
 *     sequence lengths to [0, Lmax] and skip token indices outside [0, Lmax).
 *   - A launch failure returns RTP_EHIP.  A device fault surfaces at the caller's
 *     next synchronisation.
 *   - Supported shapes: r = 16 (indexer size), d = 128 (head size), 1 <= G <= 64,
 *     1 <= Lmax <= 2^24.  Inputs must be finite.
 *   - dtype codes: RTP_F32 (fp32), RTP_F16 (IEEE binary16) or RTP_BF16 (bfloat16: the
 *     upper half of an fp32).  q, K, V and k_idx use the given dtype; q_idx and every
 *     output are fp32; accumulation is fp32.  Every stored value converts to fp32
 *     exactly; values written in a cache dtype (rtp_append_project, rtp_prefill) are
 *     rounded to nearest, ties to even.
 *   - Attention scales (scale_attn, the softmax temperature 1/sqrt(d)) must be positive
 *     and finite; RTP_EINVAL otherwise.
 *   - Logits must satisfy |z / bin_width| < 2^30, so that their cells fit in int32.
 *   - A sequence with length 0 yields out = 0, lse = -inf, sel_count = 0.
 *   - Results are deterministic: repeated calls on the same inputs are bitwise equal.
 */
#ifndef RTP_H_
#define RTP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RTP_ABI_VERSION 3

typedef int32_t rtp_status;
enum {
  RTP_OK = 0,
  RTP_EINVAL = -1,        /* null/misaligned pointer, bad size or parameter */
  RTP_EUNSUPPORTED = -2,  /* r != 16, d != 128, G or Lmax out of range, B x query heads
                             above 65535 (a launch's grid dimension), bad dtype */
  RTP_EWORKSPACE = -3,    /* ws_bytes below the size query */
  RTP_EHIP = -4,          /* a HIP launch failed */
  RTP_ESCRATCH = -5       /* rtp_decode_step_noalloc: the step needs more than its fixed scratch */
};
enum { RTP_F32 = 0, RTP_F16 = 1, RTP_BF16 = 2 };

/* Static description of a status code. */
const char* rtp_status_string(rtp_status s);
/* RTP_ABI_VERSION of the loaded library. */
int32_t rtp_abi_version(void);

/*
 * Indexer score (section 三, 核心公式, adaptive sparse attention: the first
 * equation, s_h(m,n) = (W^Q_h q^pre)^T (W^K_h k^pre), on features projected to r
 * dims before RoPE).  For every query head h = kr*G + g of retrieval KV head kr and
 * every token n < L_b:
 *     a = +0;  for i = 0..r-1:  a = fmaf(q_idx[b,h,i], k_idx[b,kr,n,i], a)
 *     z[b,h,n] = fl32(scale_idx * a)
 * (the fp32 fused multiply-add chain in this order; fp16 keys convert exactly).
 *   q_idx   [B, Hr*G, r] fp32        k_idx [B, Hr, Lmax, r] (k_dtype)
 *   seq_lens[B] int32 (device)       z     [B, Hr*G, Lmax] fp32 out; entries n >= L_b untouched
 */
rtp_status rtp_index_score(const float* q_idx, const void* k_idx, int32_t k_dtype,
                           const int32_t* seq_lens, int32_t B, int32_t Hr, int32_t G,
                           int32_t Lmax, int32_t r, float scale_idx, float* z, void* stream);

/*
 * Top-p selection without sorting through a 256-bin histogram (section 三,
 * 硬件感知解码内核: 256 bins, 1 KB per head, independent of the sequence length;
 * the top-p set S_h(m) = Top-P(s_h(m,.), p) of the sparse-attention equation).
 * Per row (b, h) over n < L = L_b, with w = bin_width (a power of two):
 *     g_n = floor(z_n / w);  A = max_n g_n;  j_n = min(A - g_n, 255)
 *     mu_j = sum_{j_n = j} exp(z_n - (A+1) w);  Z = sum_j mu_j
 *     b* = 255 if p >= 1, else the least j with mu_0 + ... + mu_j >= p Z
 *     S = { n : j_n <= b* }  (ascending)
 * S contains the exact top-p set and holds softmax mass >= p.
 *   z        [B, H, Lmax] fp32            seq_lens [B] int32 (device)
 *   p        in (0, 1]; values >= 1 select every token
 *   sel_idx  [B, H, cap] int32 out: the first min(|S|, cap) indices of S, ascending
 *   sel_count[B, H] int32 out: |S| (may exceed cap: the caller checks overflow)
 *   hist     [B, H, 256] fp32 out or NULL: mu_j
 *   thresh   [B, H, 2] int32 out or NULL: {A, b*}
 * Masses are accumulated exactly per bin from fp32 exponentials and merged in fp64,
 * so b* can differ from an fp64 evaluation only when a cumulative mass lies within
 * about 1e-6 Z of p Z.
 */
size_t rtp_topp_select_workspace_size(int32_t B, int32_t H, int32_t Lmax);
rtp_status rtp_topp_select(const float* z, const int32_t* seq_lens, int32_t B, int32_t H,
                           int32_t Lmax, double p, float bin_width, int32_t* sel_idx,
                           int32_t* sel_count, int32_t cap, float* hist, int32_t* thresh,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Fixed top-k through the same histogram (section 三, insight 3 and its top-k vs top-p
 * table: fixed token budgets set against top-p).  The bins are those of rtp_topp_select;
 * every token weighs one instead of its softmax mass:
 *     c_j = #{ n < L : j_n = j }
 *     b* = the least j with c_0 + ... + c_j >= k, or 255 when L < k
 *     S = { n : j_n <= b* }  (ascending)
 * S holds at least min(k, L) tokens, including every token whose logit is at least the
 * k-th largest.  Counts are exact, so the result depends on z only through the cells.
 *   k        >= 1 (RTP_EINVAL otherwise)
 *   hist     [B, H, 256] fp32 out or NULL: c_j
 * Every other argument, the workspace size and the outputs are those of rtp_topp_select.
 */
size_t rtp_topk_select_workspace_size(int32_t B, int32_t H, int32_t Lmax);
rtp_status rtp_topk_select(const float* z, const int32_t* seq_lens, int32_t B, int32_t H,
                           int32_t Lmax, int32_t k, float bin_width, int32_t* sel_idx,
                           int32_t* sel_count, int32_t cap, float* hist, int32_t* thresh,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Exact softmax attention over a selected token set (section 三, 核心公式, the
 * sparse-attention equation):
 *     O[b,h] = sum_{n in S} exp(s_n - m) V[b,kr,n] / sum_{n in S} exp(s_n - m),
 *     s_n = scale_attn * q[b,h] . K[b,kr,n],  m = max s_n,  lse = m + log(sum exp(s_n - m))
 * with kr = h / G and S = sel_idx[b,h,0 : min(sel_count[b,h], cap)].
 *   q [B, Hr*G, d] (kv_dtype)   K, V [B, Hr, Lmax, d] (kv_dtype)
 *   out [B, Hr*G, d] fp32 out   lse [B, Hr*G] fp32 out or NULL
 * Split-K: fixed-size slices of S give partial (max, sum, weighted V) triples that a
 * second pass merges.
 */
size_t rtp_sparse_decode_workspace_size(int32_t B, int32_t Hr, int32_t G, int32_t cap);
rtp_status rtp_sparse_decode(const void* q, const void* K, const void* V, int32_t kv_dtype,
                             const int32_t* sel_idx, const int32_t* sel_count, int32_t cap,
                             int32_t B, int32_t Hr, int32_t G, int32_t Lmax, int32_t d,
                             float scale_attn, float* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Local heads: exact softmax attention over the sink tokens and a sliding window
 * (section 五, test-configuration table; gist.science summary, section 1: local heads
 * use a sliding window with attention sinks).  The token set of a sequence of length
 * L is { n < min(sinks, L) } united with { max(sinks, L - window) <= n < L } (the
 * current token included).  The cache is a ring: position n < sinks lives in slot n,
 * any later position n in slot sinks + (n mod window).
 *   q [B, Hl*G, d] (kv_dtype)   K, V [B, Hl, sinks + window, d] (kv_dtype)
 *   out [B, Hl*G, d] fp32       lse [B, Hl*G] fp32 or NULL
 */
size_t rtp_window_decode_workspace_size(int32_t B, int32_t Hl, int32_t G, int32_t window,
                                        int32_t sinks);
rtp_status rtp_window_decode(const void* q, const void* K, const void* V, int32_t kv_dtype,
                             const int32_t* seq_lens, int32_t B, int32_t Hl, int32_t G,
                             int32_t d, int32_t window, int32_t sinks, float scale_attn,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step of one attention layer: KV heads flagged in kv_is_retrieval run
 * indexer score -> histogram top-p -> sparse attention for each of their G query
 * heads; the other KV heads run window attention.  Retrieval heads keep the full
 * cache and local heads a window plus sinks (section 三, solution overview and
 * insight 1; section 五, test configuration).
 */
typedef struct {
  int32_t B, Hq, Hkv, d, r, Lmax, window, sinks, kv_dtype;
  const uint8_t* kv_is_retrieval; /* HOST [Hkv]: 1 = retrieval, 0 = local */
  const void* q;                  /* [B, Hq, d] (kv_dtype); query head h belongs to KV head h / G */
  const float* q_idx;             /* [B, Hq, r] fp32; rows of local heads are ignored */
  const void* K_ret;              /* [B, Hret, Lmax, d]: retrieval KV heads in ascending order */
  const void* V_ret;              /* [B, Hret, Lmax, d] */
  const void* k_idx;              /* [B, Hret, Lmax, r] (kv_dtype) */
  const void* K_loc;              /* [B, Hloc, sinks + window, d] ring (see rtp_window_decode) */
  const void* V_loc;              /* [B, Hloc, sinks + window, d] */
  const int32_t* seq_lens;        /* [B] device */
  double p;                       /* top-p mass in (0, 1]; ignored when topk > 0 */
  float bin_width, scale_idx, scale_attn;
  float* out;                     /* [B, Hq, d] fp32 out */
  float* lse;                     /* [B, Hq] fp32 out or NULL */
  int32_t* thresh_out;            /* [B, Hq, 2] {A, b*} for retrieval query heads, or NULL */
  int32_t* count_out;             /* [B, Hq] |S| for retrieval query heads, or NULL */
  int32_t topk;                   /* 0: top-p with p; > 0: fixed top-k (rtp_topk_select's rule)
                                   * for every retrieval query head; < 0: RTP_EINVAL */
  int32_t ret_window;             /* 0: retrieval heads attend to their selected set only;
                                   * 1: to that set united with { n < sinks } and
                                   * { n >= L - window } (the local heads' window, in the
                                   * full cache); count_out then counts the union */
  /* Optional export of the token sets the step attended to, per retrieval query head (the
   * lists the attention kernels consumed, not a recomputation): sel_idx[b,h,:] holds the
   * first min(n, sel_cap) indices of the set in ascending order and sel_count[b,h] = n.  The
   * set is S_h (top-p or top-k), united with the sink and window positions when
   * ret_window = 1.  Rows of local query heads are left as they are.  NULL (both) skips the
   * export; the workspace query accounts for it, so query the size with the pointers set. */
  int32_t* sel_idx;               /* [B, Hq, sel_cap] int32 out, or NULL */
  int32_t* sel_count;             /* [B, Hq] int32 out, or NULL (NULL exactly when sel_idx is) */
  int32_t sel_cap;                /* >= 1 when sel_idx is given */
  /* Optional cache update fused into the step (NULL: none).  The step first does exactly
   * what rtp_append_project does with these inputs -- the new token's indexer projections
   * into q_idx and k_idx[L-1], its K/V rows into K_ret/V_ret[L-1] or the local ring -- and
   * then attends over the updated caches; seq_lens holds the lengths after the append.
   * q_idx, k_idx, K_ret, V_ret, K_loc and V_loc are then written as well as read. */
  const struct rtp_step_append* append;
} rtp_layer_desc;

/* Inputs of the cache update fused into rtp_decode_step (rtp_append_project's inputs). */
typedef struct rtp_step_append {
  const float* q_pre;             /* [B, Hq, d] fp32 pre-RoPE queries (retrieval rows read) */
  const float* k_pre;             /* [B, Hkv, d] fp32 pre-RoPE keys of the new token */
  const float* Wq_idx;            /* [Hq, d, r] fp32 */
  const float* Wk_idx;            /* [Hret, d, r] fp32, retrieval KV heads in ascending order */
  const void* k_new;              /* [B, Hkv, d] (kv_dtype) key of the new token (post-RoPE) */
  const void* v_new;              /* [B, Hkv, d] (kv_dtype) */
} rtp_step_append;

/* fp16 and bf16 caches with G <= 16 run four kernels per call: indexer score + chunk
 * histograms; per-head suffix tables of the bin masses (token counts under top-k);
 * selection + sparse attention together with the window attention of local heads; merge of
 * the split partials (plus a fifth that writes the exported sets, when asked for).  With
 * desc->append, the first kernel also does the cache update (layers without retrieval
 * heads run rtp_append_project's kernel first).  Other shapes (fp32 caches, G > 16) run
 * the single-purpose kernels in sequence, after rtp_append_project's kernel when desc->append
 * is given.  The workspace needs no initialisation; calls that may overlap must not share
 * one. */
size_t rtp_decode_step_workspace_size(const rtp_layer_desc* desc);
rtp_status rtp_decode_step(const rtp_layer_desc* desc, void* ws, size_t ws_bytes, void* stream);

/* rtp_decode_step with kernel timing for a profiler: events[0..3] are hipEvent_t handles
 * (each may be NULL) created on the calling process's device.  On the four-kernel path,
 * events[0] and [1] (when both are given) are bound to the start and the end of the
 * indexer-score / histogram kernel's own execution, and events[2] and [3] to those of the
 * selection + attention kernel (not to their dispatch).  The single-purpose path records
 * [0] and [1] on `stream` around its histogram kernel and [2] and [3] around its sparse
 * attention kernel.  Everything else is rtp_decode_step's. */
rtp_status rtp_decode_step_profiled(const rtp_layer_desc* desc, void* ws, size_t ws_bytes,
                                    void* stream, void* const events[4]);

/* rtp_decode_step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels, on a
 * fixed scratch array that the library holds on each device it runs on (64 MiB, kept until
 * the process ends; resolved on the first call on a device) instead of a caller workspace.
 * The call allocates nothing.  A step whose rtp_decode_step_workspace_size exceeds 64 MiB
 * returns RTP_ESCRATCH and enqueues nothing (every step with B x (retrieval KV heads) x Lmax
 * up to 2^21 tokens fits, exported sets included).  All calls on one device share its array,
 * which keeps the last call's contents (the kernels need no particular contents): calls
 * that may overlap on one device -- on different streams, or from different threads --
 * race, and the caller must order them. */
rtp_status rtp_decode_step_noalloc(const rtp_layer_desc* desc, void* stream);

/*
 * Cache update of one decode step, before rtp_decode_step (section 三, 核心公式: the
 * indexer compares W^Q_h q^pre with W^K_h k^pre, both projected to r dims before RoPE;
 * section 五, test configuration: retrieval heads keep the whole cache, local heads a
 * window plus sinks).  For every sequence b with L = seq_lens[b] >= 1 the new token sits
 * at position n = L - 1 (seq_lens holds the lengths after the append, the same array the
 * following rtp_decode_step takes):
 *   retrieval KV head kv (the kr-th flagged head), every query head h = kv*G + g:
 *     q_idx[b,h,i] = a_i,  a <- +0;  for c = 0..d-1: a <- fmaf(q_pre[b,h,c], Wq_idx[h,c,i], a)
 *     k_idx[b,kr,n,i] = the same chain over k_pre[b,kv] and Wk_idx[kr], rounded to the
 *                       cache dtype (round to nearest even)
 *     K_ret[b,kr,n] = k_new[b,kv];  V_ret[b,kr,n] = v_new[b,kv]
 *   local KV head kv (the kl-th unflagged head):
 *     K_loc[b,kl,slot] = k_new[b,kv];  V_loc[b,kl,slot] = v_new[b,kv],  slot = n if n < sinks,
 *     else sinks + (n mod window)  (the ring of rtp_window_decode)
 * Rows of q_idx that belong to local heads, and every other cache row, are left as they
 * are; sequences with L = 0 are left alone.  No workspace; the call never allocates.
 */
typedef struct {
  int32_t B, Hq, Hkv, d, r, Lmax, window, sinks, kv_dtype;
  const uint8_t* kv_is_retrieval; /* HOST [Hkv]: 1 = retrieval, 0 = local */
  const float* q_pre;             /* [B, Hq, d] fp32 pre-RoPE queries (retrieval rows read) */
  const float* k_pre;             /* [B, Hkv, d] fp32 pre-RoPE keys of the new token */
  const float* Wq_idx;            /* [Hq, d, r] fp32 (rows of local heads' queries unread) */
  const float* Wk_idx;            /* [Hret, d, r] fp32, retrieval KV heads in ascending order */
  const void* k_new;              /* [B, Hkv, d] (kv_dtype) key of the new token (post-RoPE) */
  const void* v_new;              /* [B, Hkv, d] (kv_dtype) */
  const int32_t* seq_lens;        /* [B] device: lengths after the append */
  float* q_idx;                   /* [B, Hq, r] fp32 out */
  void* k_idx;                    /* [B, Hret, Lmax, r] (kv_dtype) in/out */
  void* K_ret;                    /* [B, Hret, Lmax, d] in/out */
  void* V_ret;
  void* K_loc;                    /* [B, Hloc, sinks + window, d] in/out */
  void* V_loc;
} rtp_append_desc;
rtp_status rtp_append_project(const rtp_append_desc* desc, void* stream);

/*
 * Prefill of a prompt (section 五, efficiency evaluation: local heads windowed and
 * retrieval heads dense during prefill; section 五, test configuration: window 8192,
 * 4 sinks).  For every sequence b, prompt position t < L = seq_lens[b] and query head
 * h = kv*G + g:
 *     out[b,h,t] = sum_{n in R} e^{s_n - m} V[b,kv,n] / sum_{n in R} e^{s_n - m},
 *     s_n = scale_attn * q[b,h,t] . K[b,kv,n],  m = max s_n,
 *     R = { n <= t } (retrieval KV head) or { n < min(sinks, t+1) } united with
 *         { max(sinks, t+1-window) <= n <= t } (local KV head: the decode window of a
 *         sequence of length t + 1).
 * fp16 or bf16 inputs (q, K, V of one type), fp32 accumulation; rows t >= L of out are
 * left as they are.
 * It also writes the decode state the prompt leaves, for each group whose pointers are
 * given (NULL skips the group):
 *   - k_idx[b,kr,n] = the fp32 fma chain of rtp_append_project over k_pre[b,kv,n] and
 *     Wk_idx[kr], rounded to the K/V type (nearest even), for n < L (retrieval KV head kv,
 *     the kr-th flagged);
 *   - K_ret/V_ret[b,kr,n] = K/V[b,kv,n] for n < L;
 *   - K_loc/V_loc[b,kl,slot(n)] = K/V[b,kv,n] for the positions n of the final window set
 *     (rtp_window_decode's ring; other slots are left as they are).
 * kv_dtype is RTP_F16 or RTP_BF16 (else RTP_EUNSUPPORTED); every cache written has that
 * type.  No workspace; the call never allocates.
 */
typedef struct {
  int32_t B, Hq, Hkv, d, r, Lmax, window, sinks, kv_dtype;
  const uint8_t* kv_is_retrieval; /* HOST [Hkv]: 1 = retrieval, 0 = local */
  const void* q;                  /* [B, Hq, Lmax, d] post-RoPE queries of the prompt */
  const void* K;                  /* [B, Hkv, Lmax, d] post-RoPE keys of the prompt */
  const void* V;                  /* [B, Hkv, Lmax, d] */
  const int32_t* seq_lens;        /* [B] device prompt lengths */
  float scale_attn;
  float* out;                     /* [B, Hq, Lmax, d] fp32 out */
  const float* k_pre;             /* [B, Hkv, Lmax, d] fp32 pre-RoPE keys (with k_idx) */
  const float* Wk_idx;            /* [Hret, d, r] fp32 (with k_idx) */
  void* k_idx;                    /* [B, Hret, Lmax, r] out, or NULL */
  void* K_ret;                    /* [B, Hret, Lmax, d] out, or NULL (together with V_ret) */
  void* V_ret;
  void* K_loc;                    /* [B, Hloc, sinks + window, d] out, or NULL (with V_loc) */
  void* V_loc;
} rtp_prefill_desc;
rtp_status rtp_prefill(const rtp_prefill_desc* desc, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RTP_H_ */
