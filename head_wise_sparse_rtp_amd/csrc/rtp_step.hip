// Decode step for fp16 and bf16 caches in four launches per layer.
//
//   K1 stage A  indexer score and per-chunk 256-bin histograms of every retrieval query
//               head (chunk-relative bin codes, suffix sums of the bin masses, top cell).
//   K2 stage T  per (head, group of 16 bins): the suffix sums of all chunks, shifted to
//               the head's top cell and added, giving the head's whole suffix table.
//   K3 stage B  selection blocks (retrieval KV head x slice of 2048-8192 tokens): b* from
//               the suffix table, the union over the query heads of the selected tokens
//               of the slice, masked softmax attention on the matrix cores over the
//               gathered K/V rows -> one partial per slice; window blocks (local KV head x
//               run of window entries) -> one partial per run.
//   K4 stage M  per (query head, 32 output dims): merge the partials.
// Blocks of one launch never wait for or read each other's results: on gfx950 a
// device-scope release fence writes back and invalidates the whole L2 of the XCD, so
// cross-block hand-offs go through kernel boundaries instead.
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 三:
// the indexer score and sparse-attention equations (核心公式) and the sort-free 256-bin
// histogram top-p (硬件感知解码内核); section 五 (test configuration) for the window
// of local heads.  The pages' kernels target another GPU; the tiling here is for
// 64-wide wavefronts and 16x16x32 fp16 MFMA on gfx950.
//
// Attention tile (one wavefront, 32 cache rows):
//   S^T = K_tile (32 x 128) . Q^T (128 x 16 heads) as two 16-row tiles of 4 MFMAs; the
//   accumulator layout gives lane l the logits of head l%16 for rows 4*(l/16)+t,
//   which is exactly the A-operand layout of P for O += P . V (8 MFMAs, one per 16
//   output columns).  Output column c of MFMA nb holds head-dim 8*c + nb, so each lane
//   loads 16 contiguous bytes of each V row it needs.
#include <hip/hip_ext.h>

#include "rtp_attn_tile.h"

#include <algorithm>
#include <cmath>

namespace rtp {

namespace {

constexpr int kBThreads = 256;           // threads of a stage-B block (two blocks per CU)
constexpr int kBWaves = kBThreads / 64;  // wavefronts of a stage-B block
constexpr int kMaxCPB = 4;               // histogram chunks per selection block (at most)
constexpr int kMSlice = 32;              // output dims per stage-M block
constexpr int kMSlices = kD / kMSlice;
constexpr int kMaxParts = 4096;          // partials merged per head (at most)

// Sequence length of batch row b through the scalar cache: a load through the constant
// address space at a uniform index is a scalar load, waited for at its first use with the
// scalar counter.  A vector load would be waited for with the in-order vector-memory
// counter, i.e. together with every load issued before it.  (The lengths are not written
// while a step runs.)
typedef const __attribute__((address_space(4))) int32_t cint32_t;
__device__ __forceinline__ int seq_len(const int32_t* seq_lens, int b) {
  return *((cint32_t*)seq_lens + __builtin_amdgcn_readfirstlane(b));
}

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int Lmax) {
  const int L = seq_len(seq_lens, b);
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

// Brings every 64-byte line of a kernel's argument block into the scalar cache at once: one
// scalar load per line, all in flight together, waited for here.  The fields read later then
// hit the cache instead of paying a round trip for each line they first touch (a block's
// early fields span several lines, and some are indexed by values read from the first).
template <class Params>
__device__ __forceinline__ void fetch_args(const Params& P) {
  constexpr int kLines = (int)((sizeof(Params) + 63) / 64);
  const int32_t* w = reinterpret_cast<const int32_t*>(&P);
  int32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kLines; i++) acc ^= w[16 * i];
  asm volatile("" ::"s"(acc));
}
// The same for the given lines only (a kernel whose first loads need few of them).
template <int... LINES, class Params>
__device__ __forceinline__ void fetch_arg_lines(const Params& P) {
  const int32_t* w = reinterpret_cast<const int32_t*>(&P);
  const int32_t acc = (w[16 * LINES] ^ ...);
  asm volatile("" ::"s"(acc));
}

// ---------------------------------------------------------------------------
// wavefront scans and reductions on DPP lane moves (no LDS round trip)
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float x) {
  // lanes whose source is out of range, or whose row is masked off, read 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

// minimum over the 64 lanes (every lane gets it): rotations inside the rows, then the
// rows through lanes 15 / 31 and a final read of lane 63
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x121, 0xf, 0xf, false));  // row_ror:1
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x122, 0xf, 0xf, false));  // row_ror:2
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x128, 0xf, 0xf, false));  // row_ror:8
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each row of 16,
// then lane 15 of rows 0/2 into rows 1/3 and lane 31 into rows 2/3
__device__ __forceinline__ float wave_incl_sum(float v) {
  v += dpp_f<0x111>(v);  // row_shr:1
  v += dpp_f<0x112>(v);  // row_shr:2
  v += dpp_f<0x114>(v);  // row_shr:4
  v += dpp_f<0x118>(v);  // row_shr:8
  v += dpp_f<0x142, 0xa>(v);  // row_bcast:15
  v += dpp_f<0x143, 0xc>(v);  // row_bcast:31
  return v;
}

// Combine the NWV wavefronts of a block into per-head partials (unnormalised), written
// to out_m/out_l/out_acc for heads < G.  Only the first `nact` wavefronts can hold rows
// (the others took no step); they pass through LDS in one round, then thread
// (head, DPT dims) combines them in wavefront order.  lds >= NWV*(32+2048) floats.
template <int NWV>
__device__ void block_combine(AttnState& st, int G, int nact, float* lds, float* out_m,
                              float* out_l, float* out_acc) {
  constexpr int NT = NWV * 64;
  constexpr int DPT = 16 * kD / NT;  // dims per combining thread
  constexpr int WS = 32 + 2048;      // LDS floats per wavefront
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int h = lane & 15;
  const int gq = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (wv < nact) {
    float* wm = lds + wv * WS;
    if (lane < 16) {
      wm[h] = st.m;
      wm[16 + h] = l;
    }
    if (4 * gq < G) {
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
#pragma unroll
        for (int t = 0; t < 4; t++) wm[32 + (4 * gq + t) * kD + 8 * h + nb] = st.o[nb][t];
      }
    }
  }
  __syncthreads();
  const int th = threadIdx.x / (kD / DPT);
  const int d0 = (threadIdx.x % (kD / DPT)) * DPT;
  if (th < G) {
    float M = -INFINITY;
    for (int w = 0; w < nact; w++) M = fmaxf(M, lds[w * WS + th]);
    float L = 0.0f, acc[DPT];
#pragma unroll
    for (int i = 0; i < DPT; i++) acc[i] = 0.0f;
    if (M != -INFINITY) {
      for (int w = 0; w < nact; w++) {
        const float* base = lds + w * WS;
        const float mw = base[th];
        if (mw == -INFINITY) continue;
        const float f = __builtin_amdgcn_exp2f(mw - M);
        L += base[16 + th] * f;
#pragma unroll
        for (int i = 0; i < DPT; i++) acc[i] += base[32 + th * kD + d0 + i] * f;
      }
    }
    if (d0 == 0) {
      out_m[th] = M;
      out_l[th] = L;
    }
    float4* dst = reinterpret_cast<float4*>(out_acc + th * kD + d0);
#pragma unroll
    for (int i = 0; i < DPT / 4; i++)
      dst[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
  }
}

// ---------------------------------------------------------------------------
// histogram block (retrieval): indexer score on the matrix cores, then the bins,
// masses and codes of the chunk-histogram kernel of rtp_score.hip, then suffix sums
// of the bin masses.
// ---------------------------------------------------------------------------
// histogram copies per head: lane bits 3..4 (512-thread blocks) or bit 3 (256-thread
// blocks); either way a copy takes at most 512 tokens of a head, so no counter overflows
template <int NT>
constexpr int copies_of() {
  return NT >= 512 ? 4 : 2;
}
constexpr int kPad = 1;
// A projection chain's LDS region (floats): half of a 128 x 16 matrix (64 rows), stored
// transposed (output i's 64 coefficients at i kRowT, the 4 floats of padding spread the
// outputs over the banks), then the 128-float input row.  The fused cache update stages one
// region per query head of the group (region g for head g) and a ninth for the new key, in
// the histogram's space before the histogram uses it.
constexpr int kRowT = kD / 2 + 4;
constexpr int kRgn = kR * kRowT + kD;
// stage-A LDS: histogram copies, the wavefronts' head maxima, the code-word staging; with
// the fused cache update the eight chain regions share that space, and the group's
// projected q_idx and the new token's key follow it (they live across the histogram's
// first use of its space)
__host__ __device__ constexpr int stage_a_base_lds(int nt) {
  return (int)sizeof(uint32_t) * (nt >= 512 ? 4 : 2) * 8 * (kNB + kPad) + (int)sizeof(float) * 8 * (nt / 64) +
         (int)sizeof(uint32_t) * (nt / 64) * 8 * 64;
}
__host__ __device__ constexpr int stage_a_qsh(int nt) {
  return stage_a_base_lds(nt) > (int)sizeof(float) * 9 * kRgn ? stage_a_base_lds(nt)
                                                             : (int)sizeof(float) * 9 * kRgn;
}
__host__ __device__ constexpr int stage_a_lds(int nt, bool app) {
  return app ? stage_a_qsh(nt) + (int)sizeof(float) * 9 * kR : stage_a_base_lds(nt);
}
// an LDS request above a third of a CU's 160 KB: at most two stage-A blocks per CU
constexpr size_t kStageALds2PerCu = 56 * 1024;
static_assert(3 * kStageALds2PerCu > 160 * 1024 && 2 * kStageALds2PerCu <= 160 * 1024, "two blocks per CU");
static_assert(stage_a_lds(512, true) <= (int)kStageALds2PerCu, "the floor only raises the request");
// y of a token past the sequence's end: finite and far below every cell, so that its
// mass is exactly zero and it lands in the tail bin (with unit weights it is taken back
// out of that bin after the pass)
constexpr float kMaskY = -3.0e38f;

struct StageAParams {
  // line 0 (read before the first loads): the key and query addresses
  const void* k_idx;  // fp16 or bf16 (the kernel's element type)
  const float* q_idx;
  const int32_t* seq_lens;
  float* suf;
  int Lmax, Hret, G, Hq;
  int nchunk;
  int counts;  // unit weight per token (fixed top-k); c_log2 is then 0
  float yscale, c_log2;
  // line 1
  int32_t* partA;
  uint32_t* codes;
  unsigned long long* sufq;  // zeroed here (rows of the unit, by its chunk-0 block)
  int B, ngg;
  double w;
  // cache update fused into the step (kernels instantiated with APP only)
  const float* q_pre;  // [B, Hq, 128]
  const float* k_pre;  // [B, Hkv, 128]
  const float* Wq;     // [Hq, 128, 16]
  const float* Wk;     // [Hret, 128, 16]
  const void* k_new;   // [B, Hkv, 128] (the kernel's element type)
  const void* v_new;
  float* q_idx_w;      // the q_idx cache: the chunk-0 blocks write the projections
  void* k_idx_w;       // row L-1 written by the block that holds the token
  void* K_ret_w;
  void* V_ret_w;
  void* K_loc_w;
  void* V_loc_w;
  int Hkv, Hloc, window, sinks;
  HeadMap ret;  // last: indexed by a computed head (a dependent read)
  HeadMap loc;
};

struct WinParams {
  const int32_t* seq_lens;
  const void* q;  // the kernel's element type, as K_loc and V_loc
  const void* K_loc;
  const void* V_loc;
  float* wpm;
  float* wpl;
  float* wpacc;
  int Hq, G;
  int Hloc, window, sinks, nws, wrows;
  float scale2;
  HeadMap loc;  // last: indexed by a computed head (a dependent read)
};

// Histogram block: chunk `chunk` (TC = 4*NT tokens) of up to 8 query heads g0.. of
// retrieval KV head kr.  Wavefront wv scores tokens [256 wv, 256 wv + 256) of the chunk
// in 8 groups of 32 on the matrix cores:
//   A (16 x 32): row i = [k_idx(token i) | k_idx(token i + 16)]
//   B (32 x 16): column j = head j%8 against the half j/8 (the other half zero), once
//                with the high and once with the low fp16 part of the head's q_idx
//   D = A.B_hi + A.B_lo: lane l holds head l%8 for the 4 consecutive tokens
//       16*((l%16)/8) + 4*(l/16) + t of the group, t = 0..3.
// q_idx is first scaled by a power of two so that its largest entry lies in
// [2^13, 2^14): hi + lo then carry 22 significant bits and the products stay in fp32
// range; the scale is undone exactly in the final multiply.  The four bin codes of a
// lane's tokens form one code word (byte t = token 4w + t of word w).
// Loads of one histogram unit (k_idx rows and the raw q_idx of the lane's head), issued
// without waiting.
template <typename T>
struct HistIn {
  v8<T> ka[8];
  float4 q[2];   // q_idx[8*(kq&1) .. +7] of the lane's head
  // with the fused update: the projection matrix (float4 lane + 64 j of its 128 x 16 floats)
  // and input row (floats 2 lane, 2 lane + 1) of the wave's query heads wv and wv + NWV
  float4 w[2][8];
  float2 x[2];
};

struct HistUnit {
  int chunk, grp, kr, b, nrows;
  size_t rowb;
};

// grid (chunk, head group, sequence x retrieval KV head): the unit needs no division
// but b = z / Hret, in scalar registers
template <int NT>
__device__ __forceinline__ HistUnit hist_unit(const StageAParams& P) {
  HistUnit u;
  u.chunk = blockIdx.x;
  u.grp = blockIdx.y;
  u.kr = blockIdx.z % P.Hret;
  u.b = blockIdx.z / P.Hret;
  u.nrows = min(8, P.G - u.grp * 8);
  u.rowb = (size_t)u.b * P.Hret * P.G + (size_t)u.kr * P.G + u.grp * 8;
  return u;
}

template <int NT, typename T, bool APP>
__device__ __forceinline__ void hist_fetch(const StageAParams& P, const HistUnit& u, HistIn<T>& in) {
  constexpr int TC = NT * 4;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int base = u.chunk * TC;
  const int kq = lane >> 4;
  const T* kb = static_cast<const T*>(P.k_idx) + ((size_t)u.b * P.Hret + u.kr) * (size_t)P.Lmax * kR;
  const int wbase = base + wv * 256;
  // issued before the sequence length is read: rows past Lmax re-read the last row, and
  // tokens past the sequence's end are masked in hist_block
  const int nlast = P.Lmax - 1;
  // q_idx first: vector loads complete in order, so q_idx, issued ahead of the keys, is
  // ready when they arrive and its operands are prepared while they are in flight.  With
  // the fused cache update the block projects q_idx itself: the wave's projection matrix
  // and input row take q_idx's place.
  const int hh = lane & 7;
  if constexpr (APP) {
    constexpr int NWV = NT / 64;
#pragma unroll
    for (int s = 0; s < 8 / NWV; s++) {
      const int g = wv + NWV * s;  // the wave's query heads of the group
      if (g < u.nrows) {
        const size_t qh = (size_t)P.ret.kv[u.kr] * P.G + u.grp * 8 + g;
        const float4* W = reinterpret_cast<const float4*>(P.Wq + qh * kD * kR);
#pragma unroll
        for (int j = 0; j < 8; j++) in.w[s][j] = W[lane + 64 * j];
        in.x[s] = reinterpret_cast<const float2*>(P.q_pre + ((size_t)u.b * P.Hq + qh) * kD)[lane];
      }
    }
    // every wavefront's matrix loads enter the CU's memory pipeline ahead of the block's
    // key loads (an execution barrier only: no load is waited for)
    __builtin_amdgcn_s_barrier();
  } else {
    const float4* qp = reinterpret_cast<const float4*>(
        P.q_idx + ((size_t)u.b * P.Hq + (size_t)P.ret.kv[u.kr] * P.G + u.grp * 8 + min(hh, u.nrows - 1)) * kR +
        8 * (kq & 1));
    in.q[0] = qp[0];
    in.q[1] = qp[1];
  }
#pragma unroll
  for (int gi = 0; gi < 8; gi++) {
    const int n = min(wbase + gi * 32 + (lane & 15) + 16 * (kq >> 1), nlast);
    // streamed once: nontemporal, so that the stream does not displace the lines the
    // rest of the step reads back (measured 0.8-2 us per step faster; the gathered K/V
    // rows, code words, suffix rows and partials measured no better or slower that way)
    in.ka[gi] = __builtin_nontemporal_load(reinterpret_cast<const v8<T>*>(kb + (size_t)n * kR + 8 * (kq & 1)));
  }
}

// Orders one wave's LDS accesses across its lanes: what a lane wrote before the call is
// seen by every lane of the wave after it.  Lanes of a wave issue LDS operations in order,
// so this only has to stop the compiler from moving accesses across it (without it, the
// lanes that skip a divergent read may write the next piece before the others read).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The indexer projection of a pre-RoPE vector, as the cache update defines it: one fp32
// chain per output i, a <- fma(x[c], W[c][i], a) for c = 0..127 in order.  A chain region
// holds half of the 128 x 16 matrix (64 rows) and the input row; every lane of the wave
// writes its share of a half before any lane reads it, so each chain makes two passes.

// Half h (rows 64 h .. 64 h + 63) of a matrix held as float4 lane + 64 j of the lanes'
// registers is the registers j = 4 h .. 4 h + 3: register j holds row (lane >> 2) + 16 j of
// the half, columns 4 (lane & 3) .. + 3, written here to the transposed rows.
__device__ __forceinline__ void chain_put(float* rgn, float4 w0, float4 w1, float4 w2, float4 w3) {
  const int lane = threadIdx.x & 63;
  float* t = rgn + 4 * (lane & 3) * kRowT + (lane >> 2);
  const float4 w[4] = {w0, w1, w2, w3};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    t[16 * j] = w[j].x;
    t[kRowT + 16 * j] = w[j].y;
    t[2 * kRowT + 16 * j] = w[j].z;
    t[3 * kRowT + 16 * j] = w[j].w;
  }
}
__device__ __forceinline__ void chain_put_x(float* rgn, float2 x) {
  reinterpret_cast<float2*>(rgn + kR * kRowT)[threadIdx.x & 63] = x;
}
// rows 64 h .. 64 h + 63 of output i's chain, four coefficients and four inputs per read
__device__ __forceinline__ float chain_half(const float* rgn, int h, int i, float a) {
  const float4* wt = reinterpret_cast<const float4*>(rgn + i * kRowT);
  const float4* xs = reinterpret_cast<const float4*>(rgn + kR * kRowT + 64 * h);
#pragma unroll
  for (int c4 = 0; c4 < 16; c4++) {
    const float4 w = wt[c4], x = xs[c4];
    a = __builtin_fmaf(x.x, w.x, a);
    a = __builtin_fmaf(x.y, w.y, a);
    a = __builtin_fmaf(x.z, w.z, a);
    a = __builtin_fmaf(x.w, w.w, a);
  }
  return a;
}

template <typename T>
__device__ __forceinline__ T to_elem(float x);
template <>
__device__ __forceinline__ f16 to_elem<f16>(float x) {
  return (f16)x;
}
template <>
__device__ __forceinline__ bf16e to_elem<bf16e>(float x) {
  return __builtin_bit_cast(bf16e, (uint16_t)f_to_bf16(x));
}

template <int NT, typename T, bool APP>
__device__ void hist_block(const StageAParams& P, const HistUnit& U, HistIn<T>& in,
                           unsigned char* smem) {
  constexpr int TC = NT * 4;
  constexpr int NWV = NT / 64;
  constexpr int GG = 8;
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem);
  constexpr int CP = copies_of<NT>();
  float* smax = reinterpret_cast<float*>(smem + sizeof(uint32_t) * CP * GG * (kNB + kPad));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int chunk = U.chunk;
  const int nrows = U.nrows;
  const size_t rowb = U.rowb;
  const int L = clamp_len(P.seq_lens, U.b, P.Lmax);
  const int base = chunk * TC;
  if (chunk == 0)
    for (int i = tid; i < nrows * kNB; i += NT) P.sufq[rowb * kNB + i] = 0ull;
  if (base >= L) {
    if (tid < nrows) P.partA[(rowb + tid) * P.nchunk + chunk] = kEmptyCell;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the unit's loads are still in flight
    return;
  }
  const bool full = base + TC <= L;
  const int hh = lane & 7;         // head of this lane (B column and D column)
  const int th = (lane >> 3) & 1;  // token half of the B column
  const int kq = lane >> 4;        // k-group of the A / B operands
  const int wbase = base + wv * 256;
  // ---- q operands of head hh (zero for heads past nrows); lanes l and l^16 hold the
  // two halves of the head's q_idx.  The parts of each entry sum to it exactly: two fp16
  // parts (22 bits) or three bf16 parts (24 bits)
  constexpr int NQP = __is_same(T, bf16e) ? 3 : 2;
  v8<T> qp[NQP];
#pragma unroll
  for (int k = 0; k < NQP; k++)
#pragma unroll
    for (int i = 0; i < 8; i++) qp[k][i] = (T)0.0f;
  float q[8] = {in.q[0].x, in.q[0].y, in.q[0].z, in.q[0].w,
                in.q[1].x, in.q[1].y, in.q[1].z, in.q[1].w};
  using u4t = uint32_t __attribute__((ext_vector_type(4)));
  const int n = L - 1;  // the new token
  // (uniform per wave) the fused update's key of the new token is this wave's
  const bool tokw = APP && n >= base && n < base + TC && (n - base) / 256 == wv;
  u4t kvr[4];  // its K/V rows, stored at the block's end: retrieval K, V, local K, V
  if constexpr (APP) {
    // the fused cache update: q_idx of the group's heads, then the indexer key of token n
    // in the wave whose tokens hold it, which also loads the new K/V rows.  Every wave
    // stages its heads' matrices (heads wv and wv + NWV), half by half; the chains then run
    // four to a wave (head c in lanes 16 (c & 3) .. + 15 of wave c / 4), so that the few
    // fma chains do not share the SIMDs with one another.
    constexpr int QPW = 8 / NWV;
    float* qsh = reinterpret_cast<float*>(smem + stage_a_qsh(NT));  // [8 heads][16], then the key
    float* rg = reinterpret_cast<float*>(smem);  // region of head c: rg + c kRgn
    const size_t kvq = (size_t)P.ret.kv[U.kr] * P.G + U.grp * 8;
    const int i16 = lane & 15;
    const int cl = 4 * wv + (lane >> 4);  // the head whose chain the lane runs
    const bool act = cl < nrows;           // (waves 0 and 1 only)
    const float* mr = rg + (act ? cl : 0) * kRgn;
#pragma unroll
    for (int s = 0; s < QPW; s++) {
      const int g = wv + NWV * s;
      if (g < nrows) {
        chain_put(rg + g * kRgn, in.w[s][0], in.w[s][1], in.w[s][2], in.w[s][3]);
        chain_put_x(rg + g * kRgn, in.x[s]);
      }
    }
    __syncthreads();
    float a = 0.0f;
    if (act) a = chain_half(mr, 0, i16, a);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < QPW; s++) {
      const int g = wv + NWV * s;
      if (g < nrows) chain_put(rg + g * kRgn, in.w[s][4], in.w[s][5], in.w[s][6], in.w[s][7]);
    }
    __syncthreads();
    if (act) {
      a = chain_half(mr, 1, i16, a);
      qsh[cl * kR + i16] = a;
      if (chunk == 0) P.q_idx_w[((size_t)U.b * P.Hq + kvq + cl) * kR + i16] = a;
    }
    if (tokw) {
      const int kv = P.ret.kv[U.kr];
      float4 w[8];
      const float4* W = reinterpret_cast<const float4*>(P.Wk + (size_t)U.kr * kD * kR);
#pragma unroll
      for (int j = 0; j < 8; j++) w[j] = W[lane + 64 * j];
      const float2 x = reinterpret_cast<const float2*>(P.k_pre + ((size_t)U.b * P.Hkv + kv) * kD)[lane];
      float* kr = rg + 8 * kRgn;  // the ninth region
      chain_put(kr, w[0], w[1], w[2], w[3]);
      chain_put_x(kr, x);
      wave_lds_sync();
      float ak = 0.0f;
      if (lane < kR) ak = chain_half(kr, 0, lane, ak);
      wave_lds_sync();
      chain_put(kr, w[4], w[5], w[6], w[7]);
      wave_lds_sync();
      float* ksh = qsh + 8 * kR;
      const size_t krow = ((size_t)U.b * P.Hret + U.kr) * (size_t)P.Lmax + n;
      if (lane < kR) {
        ak = chain_half(kr, 1, lane, ak);
        ksh[lane] = ak;
        if (U.grp == 0) static_cast<T*>(P.k_idx_w)[krow * kR + lane] = to_elem<T>(ak);
      }
      wave_lds_sync();
      // the token's key row in the score tile: lanes (r & 15) + 16 (2 (r >> 4) + half)
      const int r = (n - base) & 255;
      const int gin = r >> 5, rr = r & 31;
      if ((lane & 15) == (rr & 15) && ((lane >> 4) >> 1) == (rr >> 4)) {
        const int half = (lane >> 4) & 1;
#pragma unroll
        for (int gi = 0; gi < 8; gi++)
          if (gi == gin)
#pragma unroll
            for (int i = 0; i < 8; i++) in.ka[gi][i] = to_elem<T>(ksh[8 * half + i]);
      }
      if (U.grp == 0) {
        // the new K/V rows: retrieval cache row n (lanes 0..15), and with the first
        // retrieval head the ring slot of local head lane / 16 (the rest at the block's end)
        const u4t* kn = reinterpret_cast<const u4t*>(static_cast<const T*>(P.k_new) + ((size_t)U.b * P.Hkv + kv) * kD);
        const u4t* vn = reinterpret_cast<const u4t*>(static_cast<const T*>(P.v_new) + ((size_t)U.b * P.Hkv + kv) * kD);
        if (lane < 16) {
          kvr[0] = kn[lane];
          kvr[1] = vn[lane];
        }
        const int kl = lane >> 4;
        if (U.kr == 0 && kl < P.Hloc) {
          const int kvl = P.loc.kv[kl];
          kvr[2] = reinterpret_cast<const u4t*>(static_cast<const T*>(P.k_new) + ((size_t)U.b * P.Hkv + kvl) * kD)[lane & 15];
          kvr[3] = reinterpret_cast<const u4t*>(static_cast<const T*>(P.v_new) + ((size_t)U.b * P.Hkv + kvl) * kD)[lane & 15];
        }
      }
    }
    __syncthreads();  // every head's q_idx in LDS; the regions are free again
#pragma unroll
    for (int i = 0; i < 8; i++) q[i] = qsh[min(hh, nrows - 1) * kR + 8 * (kq & 1) + i];
  }
  float qm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) qm = fmaxf(qm, fabsf(q[i]));
  {  // lanes l and l^16 hold the two halves of the head's q_idx
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(qm), __float_as_uint(qm), false, false);
    qm = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
  int e = 0;
  (void)frexpf(qm, &e);  // qm < 2^e
  const float ysc = hh < nrows ? ldexpf(P.yscale, e - 14) : 0.0f;
  if (hh < nrows && (kq >> 1) == th) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float v = ldexpf(q[i], 14 - e);
#pragma unroll
      for (int k = 0; k < NQP; k++) {
        const T part = (T)v;
        qp[k][i] = part;
        v -= (float)part;
      }
    }
  }
  for (int i = tid; i < CP * GG * (kNB + kPad); i += NT) hist[i] = 0u;

  // ---- pass 1: y = fl32(a * scale) / w (exact: w is a power of two) and the top cell
  float y[8][4];
  float ym = -INFINITY;
#pragma unroll
  for (int gi = 0; gi < 8; gi++) {
    f4 d = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < NQP; k++) d = mfma32(in.ka[gi], qp[k], d);
#pragma unroll
    for (int t = 0; t < 4; t++) y[gi][t] = d[t] * ysc;
  }
  if (!full) {  // (uniform) the chunk runs past the sequence's end
#pragma unroll
    for (int gi = 0; gi < 8; gi++)
#pragma unroll
      for (int t = 0; t < 4; t++)
        if (wbase + gi * 32 + 16 * th + 4 * kq + t >= L) y[gi][t] = kMaskY;
  }
#pragma unroll
  for (int gi = 0; gi < 8; gi++)
#pragma unroll
    for (int t = 0; t < 4; t++) ym = fmaxf(ym, y[gi][t]);
  // lanes of one head differ in bits 3..5: rotate by 8 inside the row (bit 3), then the
  // permlane swaps (bits 4 and 5)
  ym = fmaxf(ym, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ym), 0x128, 0xf, 0xf, false)));
  ym = col_max(ym);
  if (lane < GG) smax[lane * NWV + wv] = ym;
  __syncthreads();
  float m = smax[hh * NWV];
#pragma unroll
  for (int k = 1; k < NWV; k++) m = fmaxf(m, smax[hh * NWV + k]);
  const float Acf = floorf(m);

  // ---- pass 2: per-bin sums of x * 2^22 (truncated to integers: at most 2^-22 / e^-w,
  // below 3e-7, relative to the token's mass; 512 tokens per copy cannot overflow 32
  // bits), x = exp(z - (g+1) w), and the bin codes.
  // With m = max(g, A_c - 255) (the cell, or the deepest bin's cell for the tail):
  //   bin j = A_c - m,  x = 2^((y - m - 1) c),  c = w log2(e).
  // y - m is exact (it is fract(y) unless the token is in the tail) and a token past the
  // end (y = kMaskY) lands in bin 255 with zero mass.  With c = 0 every token adds 2^22.
  const float c = P.c_log2;
  const float Kt = Acf - 255.0f;
  const float c22 = 22.0f - c;  // x * 2^22 = 2^((y - m - 1) c + 22)
  uint32_t* hrow = hist + (((lane >> 3) & (CP - 1)) * GG + hh) * (kNB + kPad);
  // code words pass through LDS ([wave][head][64 words]) so that the global stores
  // cover whole 256-byte runs per head
  uint32_t* cl = reinterpret_cast<uint32_t*>(smax + GG * NWV) + (wv * GG + hh) * 64 + 4 * th + kq;
  if (hh < nrows) {
#pragma unroll
    for (int gi = 0; gi < 8; gi++) {
      uint32_t cw = 0u;
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const float yv = y[gi][t];
        const float mc = fmaxf(floorf(yv), Kt);
        const float ex = __builtin_amdgcn_exp2f(__builtin_fmaf(yv - mc, c, c22));
        const uint32_t j = (uint32_t)(Acf - mc);
        atomicAdd(&hrow[j], (uint32_t)ex);
        cw |= j << (8 * t);
      }
      cl[gi * 8] = cw;
    }
  }
  {
    // lane l: head l/8, 16-byte pieces l%8 and l%8 + 8 of the head's 256 bytes
    const int h2 = lane >> 3;
    if (h2 < nrows) {
      const u4* src = reinterpret_cast<const u4*>(reinterpret_cast<uint32_t*>(smax + GG * NWV) +
                                                  (wv * GG + h2) * 64);
      u4* dst = reinterpret_cast<u4*>(P.codes + ((rowb + h2) * P.nchunk + chunk) * (size_t)(TC / 4) +
                                      wv * 64);
      __builtin_nontemporal_store(src[lane & 7], &dst[lane & 7]);
      __builtin_nontemporal_store(src[(lane & 7) + 8], &dst[(lane & 7) + 8]);
    }
  }
  __syncthreads();
  // suffix sums of the bin masses, one head per wavefront pass: lane k owns bins
  // jb..jb+3, jb = 4*(63-k), so a prefix scan over the lanes gives suffix sums (fp32:
  // every sum is a tree of at most ten roundings)
  const int jb = 4 * (63 - lane);
  const int ninv = full ? 0 : base + TC - L;  // tokens past the end, all in bin 255
  float fj[4];
#pragma unroll
  for (int u = 0; u < 4; u++) fj[u] = __builtin_amdgcn_exp2f(-(float)(jb + u) * c) * 2.384185791015625e-07f;
  for (int gg = wv; gg < nrows; gg += NWV) {
    float mloc[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      unsigned long long sum = 0ull;
#pragma unroll
      for (int cp = 0; cp < CP; cp++) sum += hist[(cp * GG + gg) * (kNB + kPad) + jb + u];
      if (P.counts && jb + u == kNB - 1) sum -= (unsigned long long)ninv << 22;
      const float sf = __builtin_fmaf((float)(uint32_t)(sum >> 32), 4294967296.0f, (float)(uint32_t)sum);
      mloc[u] = sf * fj[u];
    }
    const float part = (mloc[0] + mloc[1]) + (mloc[2] + mloc[3]);
    // exclusive scan: the inclusive one moved up by a lane
    const float incl = wave_incl_sum(part);
    float acc = dpp_f<0x138>(incl);  // wave_shr:1
    f4 outv;
    acc += mloc[3]; outv[3] = acc;
    acc += mloc[2]; outv[2] = acc;
    acc += mloc[1]; outv[1] = acc;
    acc += mloc[0]; outv[0] = acc;
    f4* dst = reinterpret_cast<f4*>(P.suf + ((rowb + gg) * P.nchunk + chunk) * kNB);
    __builtin_nontemporal_store(outv, &dst[63 - lane]);
    if (lane == 0) {
      float mm = smax[gg * NWV];
      for (int k = 1; k < NWV; k++) mm = fmaxf(mm, smax[gg * NWV + k]);
      P.partA[(rowb + gg) * P.nchunk + chunk] = (int)floorf(mm);
    }
  }
  if constexpr (APP) {
    if (tokw && U.grp == 0) {
      // the new K/V rows, loaded before the histogram: retrieval cache row n, and with the
      // first retrieval head the ring slot of every local head
      const size_t krow = ((size_t)U.b * P.Hret + U.kr) * (size_t)P.Lmax + n;
      if (lane < 16) {
        reinterpret_cast<u4t*>(static_cast<T*>(P.K_ret_w) + krow * kD)[lane] = kvr[0];
        reinterpret_cast<u4t*>(static_cast<T*>(P.V_ret_w) + krow * kD)[lane] = kvr[1];
      }
      if (U.kr == 0) {
        const int slot = n < P.sinks ? n : P.sinks + n % P.window;
        for (int kl = lane >> 4; kl < P.Hloc; kl += 4) {
          const size_t lrow = ((size_t)U.b * P.Hloc + kl) * (size_t)(P.sinks + P.window) + slot;
          u4t kv4 = kvr[2], vv4 = kvr[3];
          if (kl >= 4) {
            const int kvl = P.loc.kv[kl];
            kv4 = reinterpret_cast<const u4t*>(static_cast<const T*>(P.k_new) + ((size_t)U.b * P.Hkv + kvl) * kD)[lane & 15];
            vv4 = reinterpret_cast<const u4t*>(static_cast<const T*>(P.v_new) + ((size_t)U.b * P.Hkv + kvl) * kD)[lane & 15];
          }
          reinterpret_cast<u4t*>(static_cast<T*>(P.K_loc_w) + lrow * kD)[lane & 15] = kv4;
          reinterpret_cast<u4t*>(static_cast<T*>(P.V_loc_w) + lrow * kD)[lane & 15] = vv4;
        }
      }
    }
  }
}

// One histogram unit per block: two blocks per CU hide the latency of the histogram
// pass better than a block that prefetches a second unit.
template <int NT, typename T, bool APP>
__global__ __launch_bounds__(NT, NT >= 512 ? 2 : 4) void k_stage_a(StageAParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  // the first argument line and the line of the retrieval heads' KV map, which the q_idx
  // address reads (and with the fused cache update, the line of its input addresses)
  if constexpr (APP)  // the cache update's inputs too
    fetch_arg_lines<0, (int)(offsetof(StageAParams, q_pre) / 64), (int)(offsetof(StageAParams, ret) / 64)>(P);
  else
    fetch_arg_lines<0, (int)(offsetof(StageAParams, ret) / 64)>(P);
  const HistUnit U = hist_unit<NT>(P);
  HistIn<T> in;
  hist_fetch<NT, T, APP>(P, U, in);
  hist_block<NT, T, APP>(P, U, in, smem);
}

// Masked attention over the entries e = 0..n-1 of a row list: row_of(e) is the cache
// row, mask_of(e) the heads that take part (bit h).  The list is cut into 32-row steps;
// this block takes steps part, part + nparts, ... and its wavefront wv of NWV every NWV-th
// of those, in that order, with two steps' loads in flight.
//  - Default: steps in pairs, both loads issued before either step is computed.  The
//    second load sits behind a branch, so the wait before the first step's products must
//    also hold on the path that skipped it: the first step waits for both.
//  - ROLL (long lists): two buffers roll.  As soon as a step is computed, its buffer is
//    refilled with the step after next, and no load sits behind a branch of its own, so
//    the wait before a step's first use counts exactly the other buffer's younger loads.
//    A refill past the end reloads entry 0's row (cached) and is not used.  On lists of
//    one or two steps per wavefront the extra refills cost more than the overlap gains.
// NTL: nontemporal K/V loads.  The step order, and so the result, is the same either way.
template <int NWV, typename T, bool NTL = false, bool ROLL = false, class RowOf, class MaskOf>
__device__ __forceinline__ void attend_list(const T* __restrict__ Kb, const T* __restrict__ Vb,
                                            int n, RowOf row_of, MaskOf mask_of,
                                            const v8<T> (&qop)[4], float scale2, AttnState& st,
                                            int part = 0, int nparts = 1) {
  const int wv = threadIdx.x >> 6;
  const int nsteps = (n + kStep - 1) / kStep;
  const int stride = nparts * NWV;
  auto load = [&](int s, StepLoads<T>& ld) {
    const int e0 = s * kStep;
    step_load<NTL>(Kb, Vb, [&](int i) { return row_of(e0 + i < n ? e0 + i : 0); }, ld);
  };
  auto compute = [&](int s, const StepLoads<T>& ld) {
    const int e0 = s * kStep;
    step_compute(ld, qop, scale2,
                 [&](int i, int h) { return e0 + i < n && ((mask_of(e0 + i < n ? e0 + i : 0) >> h) & 1u); },
                 st);
  };
  int s = part + nparts * wv;
  if constexpr (!ROLL) {
    for (; s < nsteps; s += 2 * stride) {
      StepLoads<T> ld0, ld1;
      load(s, ld0);
      if (s + stride < nsteps) load(s + stride, ld1);
      compute(s, ld0);
      if (s + stride < nsteps) compute(s + stride, ld1);
    }
  } else {
    if (s >= nsteps) return;
    StepLoads<T> ld0, ld1;
    load(s, ld0);
    load(s + stride, ld1);
    for (;;) {
      compute(s, ld0);
      load(s + 2 * stride, ld0);
      s += stride;
      if (s >= nsteps) break;
      compute(s, ld1);
      load(s + 2 * stride, ld1);
      s += stride;
      if (s >= nsteps) break;
    }
  }
}

// ---------------------------------------------------------------------------
// window block (local KV head): entries [wsplit*wrows, +wrows) of the window set of
// sinks followed by the last `window` positions -> one partial per query head
// ---------------------------------------------------------------------------
// Window blocks share the launch with the selection blocks, whose first loads (suffix
// tables, code words) gate their whole chain.  With selection blocks present, a window
// block first waits about 2 us, so that its bulk K/V traffic lands while the selection
// blocks work on the VALU instead of ahead of their first loads (it still ends well before
// them).
template <typename T, bool HEAVY>
__device__ void window_block(const WinParams& P, int wb, float* lds, bool delay) {
  if (delay) __builtin_amdgcn_s_sleep(72);  // 72 x 64 cycles: about 1.9 us at 2.4 GHz
  const int wsplit = wb % P.nws;
  const int kl = (wb / P.nws) % P.Hloc;
  const int b = wb / (P.nws * P.Hloc);
  const int G = P.G;
  const int ring = P.sinks + P.window;
  v8<T> qop[4];  // in flight while the sequence length is read
  load_qop(static_cast<const T*>(P.q) + ((size_t)b * P.Hq + (size_t)P.loc.kv[kl] * G) * kD, G, qop);
  int L = seq_len(P.seq_lens, b);
  L = L < 0 ? 0 : L;
  const int ns = min(P.sinks, L);
  const int wstart = max(P.sinks, L - P.window);
  const int nwin = ns + max(0, L - wstart);
  const T* Kb = static_cast<const T*>(P.K_loc) + ((size_t)b * P.Hloc + kl) * (size_t)ring * kD;
  const T* Vb = static_cast<const T*>(P.V_loc) + ((size_t)b * P.Hloc + kl) * (size_t)ring * kD;
  AttnState st;
  attn_init(st);
  const int elo = wsplit * P.wrows;
  const int n = max(0, min(nwin - elo, P.wrows));
  const int sinks = P.sinks, window = P.window;
  // entry e >= ns is position wstart + (e - ns); its slot is sinks + (pos mod window), and
  // the positions span at most `window`, so one wrap test replaces the modulo
  const int wbase = wstart % window;
  auto slot_of = [&](int e) {
    e += elo;
    if (e < ns) return e;  // sink positions 0..ns-1 sit in their own slots
    int v = wbase + (e - ns);
    v -= v >= window ? window : 0;
    return sinks + v;
  };
  auto all_heads = [&](int) { return 0xFFFFu; };
  // heavy window blocks (HEAVY: over 256 rows, so their rows are the launch's bulk and a
  // wavefront has 8 or more steps) read them nontemporally through the rolling loop; light
  // ones do neither (measured: nontemporal C2 61.0 -> 59.2 us but C4 29.5 -> 30.2 us)
  if constexpr (HEAVY)
    attend_list<kBWaves, T, true, true>(Kb, Vb, n, slot_of, all_heads, qop, P.scale2, st);
  else
    attend_list<kBWaves>(Kb, Vb, n, slot_of, all_heads, qop, P.scale2, st);
  const size_t prow = ((size_t)(b * P.Hloc + kl) * P.nws + wsplit) * G;
  block_combine<kBWaves>(st, G, min(kBWaves, (n + kStep - 1) / kStep), lds, P.wpm + prow,
                         P.wpl + prow, P.wpacc + prow * kD);
}

// ---------------------------------------------------------------------------
// stage T: suffix table of every retrieval head row,
//   SUF_J = sum_c suf_c[max(J - s_c, 0)] * exp(-s_c w),  s_c = A - A_c,  A = max_c A_c,
// in fixed point (units of 2^-38 of the top cell's mass, unsigned 64-bit).  Block
// (row, segment) takes the chunks [seg*cpb, seg*cpb + cpb) of the row: their 1 KB suffix
// rows are loaded whole, together with the row's top cells, so the block waits on memory
// once; the shift by s_c happens in LDS.  Thread J sums its bin over the block's chunks
// in chunk order in fp64, rounds the sum down to a multiple of 2^-38 and adds it to the
// row's table with an integer atomic: integer sums do not depend on the order of the
// segments, so the table is the same on every run.  Per-block sums stay below 2^24
// (one unit of mass per token at most), far inside the 2^26 the format holds.  Stage A
// zeroes the table.
// ---------------------------------------------------------------------------
constexpr int kTMaxCPB = 32;                         // chunks per stage-T block (at most)
constexpr double kSufOne = 274877906944.0;           // 2^38: fixed-point unit of the table

struct StageTParams {
  const float* suf;
  const int32_t* partA;
  int nchunk, cpb, nseg;
  int maxshift;  // chunks more than this many cells below the top add exactly nothing
  float c_log2;
  unsigned long long* sufq;
  int32_t* Aglob;
};

// PPT: 16-byte suffix pieces per thread (the block takes at most 4*PPT chunks).  Every
// load is unconditional (indices clamped into the row) so that none waits on another.
template <int PPT>
__global__ __launch_bounds__(kThreads) void k_stage_t(StageTParams P) {
  fetch_args(P);
  __shared__ __align__(16) float sb[4 * PPT * kNB];  // the block's chunk suffix rows
  constexpr int NCA = 4 * PPT < 8 ? 8 : 4 * PPT;
  __shared__ __align__(16) int sAc[NCA];  // top cells of the block's chunks (kEmptyCell past nc)
  __shared__ int sAw[kThreads / 64];
  const int row = blockIdx.x / P.nseg;
  const int seg = blockIdx.x % P.nseg;
  const int nchunk = P.nchunk;
  const int c0 = seg * P.cpb;
  const int nc = min(P.cpb, nchunk - c0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  // ---- suffix rows (piece i = bins 4(i%64).. of chunk i/64), then the top cells
  const f4* src = reinterpret_cast<const f4*>(P.suf + ((size_t)row * nchunk + c0) * kNB);
  const int npiece = nc * (kNB / 4);
  f4 v[PPT];
#pragma unroll
  for (int u = 0; u < PPT; u++) v[u] = src[min(tid + kThreads * u, npiece - 1)];
  const int32_t* pa = P.partA + (size_t)row * nchunk;
  const int aown = pa[min(c0 + tid, nchunk - 1)];
  int A = kEmptyCell;
  for (int cb = 0; cb < nchunk; cb += 8 * kThreads) {
    int a[8];
#pragma unroll
    for (int u = 0; u < 8; u++) a[u] = pa[min(cb + tid + kThreads * u, nchunk - 1)];
#pragma unroll
    for (int u = 0; u < 8; u++) A = max(A, a[u]);  // repeated cells leave the maximum alone
  }
  f4* sb4 = reinterpret_cast<f4*>(sb);
#pragma unroll
  for (int u = 0; u < PPT; u++)
    if (tid + kThreads * u < npiece) sb4[tid + kThreads * u] = v[u];
  if (tid < NCA) sAc[tid] = tid < nc ? aown : kEmptyCell;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) A = max(A, __shfl_xor(A, o, 64));
  if (lane == 0) sAw[wv] = A;
  __syncthreads();
  A = max(max(sAw[0], sAw[1]), max(sAw[2], sAw[3]));
  if (seg == 0 && tid == 0) P.Aglob[row] = A;
  if (A == kEmptyCell) return;
  const int j = tid;  // bin
  double acc = 0.0;
  for (int cc = 0; cc < nc; cc += 8) {
    const int4 a0 = *reinterpret_cast<const int4*>(sAc + cc);
    const int4 a1 = *reinterpret_cast<const int4*>(sAc + cc + 4);
    const int ac[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    int sh[8];
#pragma unroll
    for (int u = 0; u < 8; u++)  // no token, or mass below the fp32 range: no contribution (-1)
      sh[u] = (ac[u] != kEmptyCell && A - ac[u] <= P.maxshift) ? A - ac[u] : -1;
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; u++) x[u] = sb[min(cc + u, nc - 1) * kNB + max(j - max(sh[u], 0), 0)];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const double f = (double)__builtin_amdgcn_exp2f(-(float)max(sh[u], 0) * P.c_log2);
      acc += sh[u] >= 0 ? (double)x[u] * f : 0.0;
    }
  }
  const unsigned long long qv = (unsigned long long)(acc * kSufOne);
  if (qv != 0ull) atomicAdd(P.sufq + (size_t)row * kNB + j, qv);
}

// ---------------------------------------------------------------------------
// stage B
// ---------------------------------------------------------------------------
// Kernel arguments are read through the scalar cache, one 64-byte line per miss: the
// fields a block needs before its first loads come first, in the first two lines, and the
// head map (indexed by a computed head, hence a dependent read) comes last.
struct StageBParams {
  // line 0: block kind, slice geometry and the selection inputs
  const unsigned long long* sufq;
  const uint32_t* codes;
  const int32_t* partA;
  const int32_t* Aglob;
  int nret_blocks;  // blocks below this index run the selection
  int nrw_end;      // blocks below this index (and from nret_blocks on) run the retrieval window
  int nparts, nblk, Hret, G, tc, nchunk;
  // line 1
  double p;
  int topk;  // > 0: b* from token counts (fixed top-k) instead of masses
  int want_count;
  int Lmax, B, Hq;
  // rw_window > 0: every head also attends to n < rw_sinks and n >= L - rw_window; those
  // rows are left out of the selection lists and taken by the retrieval window blocks
  // (rw_nws per KV head, rw_rows rows each), whose partials follow the selection partials
  int rw_window;
  const int32_t* seq_lens;
  const void* q;  // the kernel's element type, as K_ret and V_ret
  const void* K_ret;
  const void* V_ret;
  int rw_sinks, rw_nws, rw_rows;
  int np_row;  // partials per retrieval KV head: nblk * nparts + rw_nws
  float scale2;
  int32_t* bstar;
  float* p1m;
  float* p1l;
  float* p1acc;
  int32_t* p1cnt;
  // export of the attended sets: each slice's union list (part 0) and its length
  uint32_t* xlist;
  int32_t* xn;
  WinParams win;
  HeadMap ret;
};

// Selection block over the TB = 1024*NWD tokens [blk*TB, (blk+1)*TB) of retrieval KV
// head kr.  Code word w of a chunk holds the bins of tokens 4w + q, q = 0..3 (byte q);
// thread tid takes the block's words NWD*tid .. NWD*tid + NWD-1.
//
// A token is selected for head g iff its chunk-relative code j_c <= tau_g = b* - (A - A_c)
// (all tokens when b* = 255).  Four codes are tested at once: with the bytes of a word
// spread over two 16-bit lanes, (256 + tau) - j_c has bit 8 set iff j_c <= tau.
template <int NWD, int GMAX, typename T>
__device__ void select_attend_block(const StageBParams& P, unsigned char* smem) {
  constexpr int NT = kBThreads;
  constexpr int TB = NT * 4 * NWD;
  constexpr int HPW = (GMAX + kBWaves - 1) / kBWaves;  // heads per wavefront (b* search)
  __shared__ uint32_t s_T[kMaxCPB][kAttnG];  // SWAR constant of (chunk, head), 0: none
  __shared__ int s_bs[kAttnG];
  __shared__ int s_wsum[kBWaves];
  __shared__ int s_cnt[kAttnG];
  uint32_t* lst = reinterpret_cast<uint32_t*>(smem);  // [TB]: in-block token | head mask << 16
  float* lds = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int part = blockIdx.x % P.nparts;  // share of the attention steps of the slice
  const int blk = (blockIdx.x / P.nparts) % P.nblk;
  const int kr = (blockIdx.x / (P.nparts * P.nblk)) % P.Hret;
  const int b = blockIdx.x / (P.nparts * P.nblk * P.Hret);
  const int G = P.G;
  const size_t row0 = (size_t)b * P.Hret * G + (size_t)kr * G;
  const int tc = P.tc;
  const int WPC = tc >> 2;     // code words per chunk
  const int cpb = TB / tc;     // chunks per block
  const int chunk0 = blk * cpb;
  const int tok0 = blk * TB;
  const T* Kb = static_cast<const T*>(P.K_ret) + ((size_t)b * P.Hret + kr) * (size_t)P.Lmax * kD;
  const T* Vb = static_cast<const T*>(P.V_ret) + ((size_t)b * P.Hret + kr) * (size_t)P.Lmax * kD;

  // ---- phase 0: every input of the selection is in flight at once (the q operand last:
  // its address needs the head map, a dependent argument read)
  int Ac = kEmptyCell, Ag = kEmptyCell;
  if (tid < cpb * kAttnG) {
    const int cc = tid / kAttnG, g = tid % kAttnG;
    const int chunk = chunk0 + cc;
    if (g < G) {
      Ag = P.Aglob[row0 + g];
      if (chunk < P.nchunk) Ac = P.partA[(row0 + g) * P.nchunk + chunk];
    }
  }
  // suffix table of the wavefront's heads (fixed point): lane l holds SUF at bins
  // 4l+1 .. 4l+4
  unsigned long long sv[HPW][4], zv[HPW];
#pragma unroll
  for (int u = 0; u < HPW; u++) {
    const int g = wv + u * kBWaves;
    zv[u] = 0ull;
#pragma unroll
    for (int k = 0; k < 4; k++) sv[u][k] = 0ull;
    if (g < G && (P.topk > 0 || P.p < 1.0)) {
      const unsigned long long* sp = P.sufq + (row0 + g) * kNB;
      zv[u] = sp[0];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int J = 4 * lane + 1 + k;
        sv[u][k] = J < kNB ? sp[J] : 0ull;
      }
    }
  }
  // the block's chunks are consecutive, so its code words of head g are the words
  // [chunk0*WPC, (chunk0+cpb)*WPC) of the head's row; thread tid takes the NWD words
  // from NWD*tid on in one load (clamped at the row's end: those tokens are masked)
  uint32_t cw[NWD][GMAX];
  {
    const int rowwords = P.nchunk * WPC;
    const int off = min(chunk0 * WPC + NWD * tid, rowwords - NWD);
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
      const uint32_t* crow = P.codes + (row0 + (g < G ? g : 0)) * (size_t)rowwords + off;
      if constexpr (NWD == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(crow);
        cw[0][g] = v.x; cw[1][g] = v.y; cw[2][g] = v.z; cw[3][g] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(crow);
        cw[0][g] = v.x; cw[1][g] = v.y;
      }
    }
  }
  v8<T> qop[4];  // used by the attention only
  load_qop(static_cast<const T*>(P.q) + ((size_t)b * P.Hq + (size_t)P.ret.kv[kr] * G) * kD, G, qop);
  if (tid < kAttnG) s_cnt[tid] = 0;
  // the sequence length only now: its scalar load waits for itself, so the loads above
  // are already in flight while it does
  const int L = clamp_len(P.seq_lens, b, P.Lmax);
  // b*: least J < 255 with Z - SUF_{J+1} >= p Z (top-k: >= k tokens), else 255
#pragma unroll
  for (int u = 0; u < HPW; u++) {
    const int g = wv + u * kBWaves;
    if (g < G) {
      int J = kNB - 1;
      if (P.topk > 0 || P.p < 1.0) {
        // the table counts in units of 2^-38 of a token (exact for every count)
        const double pz = P.topk > 0 ? (double)P.topk * kSufOne : P.p * (double)zv[u];
#pragma unroll
        for (int k = 3; k >= 0; k--) {
          const int Jk = 4 * lane + k;
          if (Jk < kNB - 1 && (double)(zv[u] - sv[u][k]) >= pz) J = Jk;
        }
        J = wave_min_i(J);
      }
      if (lane == 0) {
        s_bs[g] = J;
        if (blk == 0 && part == 0) P.bstar[row0 + g] = J;
      }
    }
  }
  __syncthreads();
  if (tid < cpb * kAttnG) {
    const int cc = tid / kAttnG, g = tid % kAttnG;
    int tau = -1;
    if (g < G && Ag != kEmptyCell && Ac != kEmptyCell && (chunk0 + cc) * tc < L) {
      const int bs = s_bs[g];
      if (bs >= kNB - 1) {
        tau = kNB - 1;
      } else {
        const long long t = (long long)bs - ((long long)Ag - (long long)Ac);
        tau = t < 0 ? -1 : (int)t;
      }
    }
    s_T[cc][g] = tau < 0 ? 0u : 0x01000100u + (uint32_t)tau * 0x00010001u;
  }
  __syncthreads();

  // ---- phase 1: per-token head masks, union compacted into the LDS list
  // the thread's words lie in chunk cc (the same for the whole wavefront: its NWD*64
  // words are aligned inside one chunk)
  const int cc = (NWD * tid) / WPC;
  uint32_t Tv[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; g++) Tv[g] = __builtin_amdgcn_readfirstlane(s_T[cc][g]);
  uint32_t hm[NWD][4];
  const bool tail = tok0 + TB > L;
#pragma unroll
  for (int i = 0; i < NWD; i++) {
    const int w = NWD * tid + i - cc * WPC;
    uint32_t me = 0u, mo = 0u;
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
      const uint32_t Tc = Tv[g];
      if (Tc == 0u) continue;
      const uint32_t x = cw[i][g];
      const uint32_t de = Tc - (x & 0x00FF00FFu);
      const uint32_t dd = Tc - ((x >> 8) & 0x00FF00FFu);
      const uint32_t bit = 0x00010001u << g;
      if (g <= 8) {
        me |= (de >> (8 - g)) & bit;
        mo |= (dd >> (8 - g)) & bit;
      } else {
        me |= (de << (g - 8)) & bit;
        mo |= (dd << (g - 8)) & bit;
      }
    }
    hm[i][0] = me & 0xFFFFu;
    hm[i][1] = mo & 0xFFFFu;
    hm[i][2] = me >> 16;
    hm[i][3] = mo >> 16;
    if (tail) {
#pragma unroll
      for (int q = 0; q < 4; q++)
        if (tok0 + cc * tc + 4 * w + q >= L) hm[i][q] = 0u;
    }
    if (P.rw_window > 0) {  // the sinks and the window belong to the window blocks
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = tok0 + cc * tc + 4 * w + q;
        if (n < P.rw_sinks || n >= L - P.rw_window) hm[i][q] = 0u;
      }
    }
  }
  if (P.want_count) {
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
      int c = 0;
#pragma unroll
      for (int i = 0; i < NWD; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) c += (hm[i][q] >> g) & 1u;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
      if (lane == 0 && c) atomicAdd(&s_cnt[g], c);
    }
  }
  // compaction: slot (i, q) of the wavefront's lanes goes in lane order after the
  // earlier slots; wavefronts follow each other
  int wtot = 0;
#pragma unroll
  for (int i = 0; i < NWD; i++)
#pragma unroll
    for (int q = 0; q < 4; q++) wtot += __popcll(__ballot(hm[i][q] != 0u));
  if (lane == 0) s_wsum[wv] = wtot;
  __syncthreads();
  int pos = 0, U = 0;
#pragma unroll
  for (int k = 0; k < kBWaves; k++) {
    if (k < wv) pos += s_wsum[k];
    U += s_wsum[k];
  }
#pragma unroll
  for (int i = 0; i < NWD; i++) {
    const int w = NWD * tid + i - cc * WPC;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const unsigned long long bal = __ballot(hm[i][q] != 0u);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (hm[i][q]) lst[pos + below] = (uint32_t)(cc * tc + 4 * w + q) | (hm[i][q] << 16);
      pos += __popcll(bal);
    }
  }
  __syncthreads();
  if (P.xlist && part == 0) {  // the list the attention below consumes, for the set export
    const size_t xs = (size_t)(b * P.Hret + kr) * P.nblk + blk;
    uint32_t* dst = P.xlist + xs * TB;
    for (int e = tid; e < U; e += NT) dst[e] = lst[e];
    if (tid == 0) P.xn[xs] = U;
  }

  // ---- phase 2: masked MFMA attention over the listed rows
  AttnState st;
  attn_init(st);
  attend_list<kBWaves>(
      Kb, Vb, U, [&](int e) { return tok0 + (int)(lst[e] & 0xFFFFu); },
      [&](int e) { return lst[e] >> 16; }, qop, P.scale2, st, part, P.nparts);
  __syncthreads();

  // ---- phase 3: block partial
  // partial (slice, part); the selection counts go with part 0 only
  const int mysteps = max(0, ((U + kStep - 1) / kStep - part + P.nparts - 1) / P.nparts);
  const size_t s1p = ((size_t)(b * P.Hret + kr) * P.np_row + (size_t)blk * P.nparts + part) * G;
  block_combine<kBWaves>(st, G, min(kBWaves, mysteps), lds, P.p1m + s1p, P.p1l + s1p,
                         P.p1acc + s1p * kD);
  if (tid < G) P.p1cnt[s1p + tid] = part == 0 ? s_cnt[tid] : 0;
}

// Retrieval window block: the sink and window rows of a retrieval KV head (positions of
// the full cache, no ring), attended by all G query heads; its partial follows the
// head's selection partials, with the row count as its count.
template <typename T>
__device__ void ret_window_block(const StageBParams& P, int wb, float* lds) {
  const int wsplit = wb % P.rw_nws;
  const int kr = (wb / P.rw_nws) % P.Hret;
  const int b = wb / (P.rw_nws * P.Hret);
  const int G = P.G;
  const int L = clamp_len(P.seq_lens, b, P.Lmax);
  const int ns = min(P.rw_sinks, L);
  const int wstart = max(P.rw_sinks, L - P.rw_window);
  const int nwin = ns + max(0, L - wstart);
  const T* Kb = static_cast<const T*>(P.K_ret) + ((size_t)b * P.Hret + kr) * (size_t)P.Lmax * kD;
  const T* Vb = static_cast<const T*>(P.V_ret) + ((size_t)b * P.Hret + kr) * (size_t)P.Lmax * kD;
  v8<T> qop[4];
  load_qop(static_cast<const T*>(P.q) + ((size_t)b * P.Hq + (size_t)P.ret.kv[kr] * G) * kD, G, qop);
  AttnState st;
  attn_init(st);
  const int elo = wsplit * P.rw_rows;
  const int n = max(0, min(nwin - elo, P.rw_rows));
  attend_list<kBWaves>(
      Kb, Vb, n,
      [&](int e) {
        e += elo;
        return e < ns ? e : wstart + (e - ns);
      },
      [&](int) { return 0xFFFFu; }, qop, P.scale2, st);
  const size_t prow =
      ((size_t)(b * P.Hret + kr) * P.np_row + (size_t)P.nblk * P.nparts + wsplit) * G;
  block_combine<kBWaves>(st, G, min(kBWaves, (n + kStep - 1) / kStep), lds, P.p1m + prow,
                         P.p1l + prow, P.p1acc + prow * kD);
  if ((int)threadIdx.x < G) P.p1cnt[prow + threadIdx.x] = n;
}

// HEAVY: the local window blocks have over 256 rows each (chosen on the host from
// win.wrows).  It is a template argument so that the kernels with light window blocks
// carry none of the heavy blocks' code: with it present but unused, the selection blocks
// measured slower (C4 +0.7 us, 16M tokens +3.8 us).
template <int NWD, int GMAX, typename T, bool HEAVY>
__global__ __launch_bounds__(kBThreads, 2) void k_stage_b(StageBParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  // the lines of the fields every block type reads, the window parameters with the first
  // local heads' map entries, and the first retrieval heads' map entries (not the maps'
  // tails: waiting for them too measured slower)
  constexpr int kLocLine = (int)((offsetof(StageBParams, win) + offsetof(WinParams, loc)) / 64);
  constexpr int kRetLine = (int)(offsetof(StageBParams, ret) / 64);
  static_assert(kLocLine == 4 && kRetLine == 8, "argument layout");
  fetch_arg_lines<0, 1, 2, 3, kLocLine, kRetLine>(P);
  if ((int)blockIdx.x < P.nret_blocks)
    select_attend_block<NWD, GMAX, T>(P, smem);
  else if ((int)blockIdx.x < P.nrw_end)
    ret_window_block<T>(P, blockIdx.x - P.nret_blocks, reinterpret_cast<float*>(smem));
  else
    // local window blocks wait behind the selection blocks' first loads, unless the
    // retrieval heads' own window blocks already sit between them, or the window blocks
    // are heavy enough (over 256 rows each) that their K/V traffic is the launch's bulk
    // (both measured slower with the wait)
    window_block<T, HEAVY>(P.win, blockIdx.x - P.nrw_end, reinterpret_cast<float*>(smem),
                           !HEAVY && P.nret_blocks > 0 && P.nrw_end == P.nret_blocks);
}

template <bool HEAVY>
void (*stage_b_kernel(int nwd, int G, bool bf))(StageBParams) {
  if (G <= 8)
    return nwd == 2 ? (bf ? &k_stage_b<2, 8, bf16e, HEAVY> : &k_stage_b<2, 8, f16, HEAVY>)
                    : (bf ? &k_stage_b<4, 8, bf16e, HEAVY> : &k_stage_b<4, 8, f16, HEAVY>);
  return nwd == 2 ? (bf ? &k_stage_b<2, 16, bf16e, HEAVY> : &k_stage_b<2, 16, f16, HEAVY>)
                  : (bf ? &k_stage_b<4, 16, bf16e, HEAVY> : &k_stage_b<4, 16, f16, HEAVY>);
}

// ---------------------------------------------------------------------------
// stage M: block (query head, 32 output dims) merges the head's n partials
// (m, l at [k*G + g], acc at [(k*G + g)*128 + d]) in a fixed order.
// ---------------------------------------------------------------------------
struct StageMParams {
  // line 0: what a block needs to issue its loads
  const float* p1m;
  const float* p1l;
  const float* p1acc;
  const int32_t* p1cnt;
  int nblk, Hret, G, nret, nws, Hloc;
  // line 1
  const float* wpm;
  const float* wpl;
  const float* wpacc;
  float* out;
  float* lse;
  int32_t* count_out;
  int32_t* thresh_out;
  const int32_t* Aglob;
  const int32_t* bstar;
  int Hq;
  HeadMap ret;  // last: indexed by a computed head (a dependent read)
  HeadMap loc;
};

// Merge state of a set of partials: running maximum M (base-2 logits), L = sum of
// l_k 2^(m_k - M), a = sum of acc_k 2^(m_k - M) over four output dims, C = sum of counts.
struct MState {
  float M, L;
  float4 a;
  int C;
};

__device__ __forceinline__ void mstate_fold(MState& s, float m, float l, float4 x) {
  if (m == -INFINITY) return;  // an empty partial
  if (m > s.M) {
    const float f = s.M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s.M - m);
    s.L *= f;
    s.a.x *= f;
    s.a.y *= f;
    s.a.z *= f;
    s.a.w *= f;
    s.M = m;
  }
  const float f = __builtin_amdgcn_exp2f(m - s.M);
  s.L += l * f;
  s.a.x += x.x * f;
  s.a.y += x.y * f;
  s.a.z += x.z * f;
  s.a.w += x.w * f;
}

__device__ __forceinline__ MState mstate_merge(const MState& p, const MState& q) {
  MState r;
  r.M = fmaxf(p.M, q.M);
  r.C = p.C + q.C;
  const float fp = p.M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(p.M - r.M);
  const float fq = q.M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(q.M - r.M);
  r.L = p.L * fp + q.L * fq;
  r.a = make_float4(p.a.x * fp + q.a.x * fq, p.a.y * fp + q.a.y * fq, p.a.z * fp + q.a.z * fq,
                    p.a.w * fp + q.a.w * fq);
  return r;
}

__device__ __forceinline__ MState mstate_shfl_xor(const MState& s, int o) {
  MState r;
  r.M = __shfl_xor(s.M, o, 64);
  r.L = __shfl_xor(s.L, o, 64);
  r.a = make_float4(__shfl_xor(s.a.x, o, 64), __shfl_xor(s.a.y, o, 64), __shfl_xor(s.a.z, o, 64),
                    __shfl_xor(s.a.w, o, 64));
  r.C = __shfl_xor(s.C, o, 64);
  return r;
}

// Thread (sub = t/8, dq = t%8) folds partials sub, sub + 32, ... of float4 dq of the slice
// (each round's loads -- value rows, maxima, sums and counts -- issued together, so n <= 256
// partials take one memory round trip), then the 32 streams of each dq merge on wave
// shuffles and across the wavefronts through LDS (lds >= 4 * 8 * 8 floats).
// The output row (head-map read) is computed by orow_of() once the loads are issued.
template <class OrowOf>
__device__ __forceinline__ void merge_slice(const float* __restrict__ pm, const float* __restrict__ pl,
                            const float* __restrict__ pacc, const int32_t* __restrict__ pcnt,
                            int n, int G, int g, int slice, float* __restrict__ out,
                            float* __restrict__ lse, int32_t* __restrict__ count_out,
                            OrowOf orow_of, float* lds) {
  constexpr int NSUB = kThreads / (kMSlice / 4);  // 32
  constexpr int UPT = 8;                          // partials per thread and round
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int sub = tid >> 3;
  const int dq = tid & 7;
  const size_t kst = (size_t)G * (kD / 4);  // float4 stride between partials
  const float4* accb = reinterpret_cast<const float4*>(pacc + (size_t)g * kD + slice * kMSlice) + dq;
  MState s;
  s.M = -INFINITY;
  s.L = 0.0f;
  s.a = make_float4(0.f, 0.f, 0.f, 0.f);
  s.C = 0;
  for (int k0 = 0; k0 < n; k0 += NSUB * UPT) {
    float4 x[UPT];
    float mk[UPT], lk[UPT];
    int ck[UPT];
#pragma unroll
    for (int u = 0; u < UPT; u++) {
      const size_t k = (size_t)min(k0 + sub + NSUB * u, n - 1);
      x[u] = accb[k * kst];
      mk[u] = pm[k * G + g];
      lk[u] = pl[k * G + g];
      ck[u] = pcnt ? pcnt[k * G + g] : 0;
    }
#pragma unroll
    for (int u = 0; u < UPT; u++) {
      if (k0 + sub + NSUB * u < n) {
        mstate_fold(s, mk[u], lk[u], x[u]);
        s.C += ck[u];
      }
    }
  }
  const size_t orow = orow_of();
  // lanes l, l^8, l^16, l^32 hold the same dims
  s = mstate_merge(s, mstate_shfl_xor(s, 8));
  s = mstate_merge(s, mstate_shfl_xor(s, 16));
  s = mstate_merge(s, mstate_shfl_xor(s, 32));
  float* red = lds;  // [wave][dq][M, L, a.x, a.y, a.z, a.w, C, -]
  if (lane < 8) {
    float* r = red + (wv * 8 + lane) * 8;
    r[0] = s.M;
    r[1] = s.L;
    r[2] = s.a.x;
    r[3] = s.a.y;
    r[4] = s.a.z;
    r[5] = s.a.w;
    r[6] = __int_as_float(s.C);
  }
  __syncthreads();
  if (tid < kMSlice) {  // output dim 4*dq + comp of the slice
    const int oq = tid >> 2, comp = tid & 3;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kThreads / 64; w++) M = fmaxf(M, red[(w * 8 + oq) * 8]);
    float Lsum = 0.0f, v = 0.0f;
    int C = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; w++) {
      const float* r = red + (w * 8 + oq) * 8;
      const float f = r[0] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(r[0] - M);
      Lsum += r[1] * f;
      v += r[2 + comp] * f;
      C += __float_as_int(r[6]);
    }
    out[orow * kD + slice * kMSlice + tid] = Lsum > 0.0f ? v / Lsum : 0.0f;
    if (slice == 0 && tid == 0) {
      if (lse) lse[orow] = Lsum > 0.0f ? (M + __log2f(Lsum)) * 0.69314718055994531f : -INFINITY;
      if (count_out) count_out[orow] = C;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_stage_m(StageMParams P) {
  extern __shared__ __align__(16) float mlds[];
  // the fields' lines (the last one also holds the retrieval heads' map entries) and the
  // first local heads' map entries (not the maps' tails)
  constexpr int kRetLine = (int)((offsetof(StageMParams, ret) + offsetof(HeadMap, kv)) / 64);
  constexpr int kLocLine = (int)((offsetof(StageMParams, loc) + offsetof(HeadMap, kv)) / 64);
  static_assert(kRetLine == 2 && kLocLine == 6, "argument layout");
  fetch_arg_lines<0, 1, kRetLine, kLocLine>(P);
  const int G = P.G;
  const int slice = blockIdx.x % kMSlices;
  const int hb = blockIdx.x / kMSlices;
  const bool win = hb >= P.nret;
  const float *pm, *pl, *pacc;
  const int32_t* pcnt = nullptr;
  int n, g, b, kh;
  if (win) {
    const int wm = hb - P.nret;
    g = wm % G;
    kh = (wm / G) % P.Hloc;
    b = wm / (G * P.Hloc);
    const size_t p0 = (size_t)(b * P.Hloc + kh) * P.nws * G;
    pm = P.wpm + p0;
    pl = P.wpl + p0;
    pacc = P.wpacc + p0 * kD;
    n = P.nws;
  } else {
    g = hb % G;
    kh = (hb / G) % P.Hret;
    b = hb / (G * P.Hret);
    const size_t p0 = (size_t)(b * P.Hret + kh) * P.nblk * G;
    pm = P.p1m + p0;
    pl = P.p1l + p0;
    pacc = P.p1acc + p0 * kD;
    if (P.count_out) pcnt = P.p1cnt + p0;
    n = P.nblk;
  }
  auto orow_of = [&]() {
    return (size_t)b * P.Hq + (size_t)(win ? P.loc.kv[kh] : P.ret.kv[kh]) * G + g;
  };
  merge_slice(pm, pl, pacc, pcnt, n, G, g, slice, P.out, P.lse, win ? nullptr : P.count_out,
              orow_of, mlds);
  if (!win && slice == 0 && P.thresh_out && threadIdx.x == 0) {
    const size_t row = (size_t)b * P.Hret * G + (size_t)kh * G + g;
    const size_t orow = orow_of();
    const int A = P.Aglob[row];
    P.thresh_out[orow * 2 + 0] = A == kEmptyCell ? 0 : A;
    P.thresh_out[orow * 2 + 1] = A == kEmptyCell ? 0 : P.bstar[row];
  }
}

// ---------------------------------------------------------------------------
// stage X (only when the sets are exported): block (slice, head g, sequence x retrieval
// KV head) turns the slice's union list into head g's tokens in ascending order, at the
// offset given by the head's counts in the earlier slices.
// ---------------------------------------------------------------------------
struct StageXParams {
  const int32_t* seq_lens;
  int Hq, G, Hret, Lmax, nblk, nparts, np_row, tb;
  HeadMap ret;
  const uint32_t* xlist;
  const int32_t* xn;
  const int32_t* p1cnt;
  int rw_sinks, rw_window;  // rw_window > 0: the sink and window positions join every set
  int32_t* sel_idx;
  int32_t* sel_count;
  int cap;
};

__global__ __launch_bounds__(kThreads) void k_stage_x(StageXParams P) {
  constexpr int kMaxTB = 16 * kThreads;  // 16 token bits per thread
  __shared__ uint32_t bm[kMaxTB / 32];
  __shared__ int red[kThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int slice = blockIdx.x;
  const int g = blockIdx.y;
  const int u = blockIdx.z;  // b * Hret + kr
  const int b = u / P.Hret;
  const int kr = u % P.Hret;
  const int L = clamp_len(P.seq_lens, b, P.Lmax);
  const int TB = P.tb;
  const int tok0 = slice * TB;
  const bool rw = P.rw_window > 0;
  const int ns = min(P.rw_sinks, L);
  const int wstart = max(P.rw_sinks, L - P.rw_window);
  // window positions below x: |([0, ns) u [wstart, L)) n [0, x)|
  auto win_below = [&](int x) { return rw ? min(x, ns) + max(0, min(x, L) - wstart) : 0; };
  // ---- the head's tokens in the earlier slices
  int off = 0;
  for (int sl = tid; sl < slice; sl += kThreads)
    off += P.p1cnt[((size_t)u * P.np_row + (size_t)sl * P.nparts) * P.G + g];
  for (int o = 32; o > 0; o >>= 1) off += __shfl_xor(off, o, 64);
  for (int i = tid; i < kMaxTB / 32; i += kThreads) bm[i] = 0u;
  if (lane == 0) red[wv] = off;
  __syncthreads();
  off = red[0] + red[1] + red[2] + red[3] + win_below(tok0);
  // ---- bitmap of the slice's tokens that carry head g
  const size_t xs = (size_t)u * P.nblk + slice;
  const int U = P.xn[xs];
  const uint32_t* lst = P.xlist + xs * TB;
  for (int e = tid; e < U; e += kThreads) {
    const uint32_t v = lst[e];
    if ((v >> (16 + g)) & 1u) atomicOr(&bm[(v & 0xFFFFu) >> 5], 1u << (v & 31u));
  }
  __syncthreads();
  uint32_t bits = 0u;
  const int t0 = 16 * tid;
  if (t0 < TB) {
    bits = (bm[tid >> 1] >> (16 * (tid & 1))) & 0xFFFFu;
    if (rw)
      for (int k = 0; k < 16; k++) {
        const int n = tok0 + t0 + k;
        if (n < L && (n < ns || n >= wstart)) bits |= 1u << k;
      }
  }
  // ---- exclusive scan of the per-thread counts, then the ascending write
  const int c = __popc(bits);
  int incl = c;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  __syncthreads();
  if (lane == 63) red[wv] = incl;
  __syncthreads();
  int pos = incl - c;
  int total = 0;
  for (int k = 0; k < kThreads / 64; k++) {
    if (k < wv) pos += red[k];
    total += red[k];
  }
  const size_t orow = (size_t)b * P.Hq + (size_t)P.ret.kv[kr] * P.G + g;
  int idx = off + pos;
  while (bits) {
    const int k = __ffs(bits) - 1;
    bits &= bits - 1u;
    if (idx < P.cap) P.sel_idx[orow * P.cap + idx] = tok0 + t0 + k;
    idx++;
  }
  if (slice == P.nblk - 1 && tid == 0) P.sel_count[orow] = off + total;
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
int chunk_tokens(int B, int Hret, int Lmax) {
  // 2048-token chunks (stage-A blocks of 512 threads) unless that leaves fewer than 256
  // histogram blocks; then 1024-token chunks (256 threads)
  const int64_t units = (int64_t)B * (Hret > 0 ? Hret : 1);
  return units * ((Lmax + 2047) / 2048) >= 256 ? 2048 : 1024;
}
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}
// window blocks the stage-B grid can hold beside the selection blocks (4096 tokens each)
// at two blocks per CU, and at least 256
int64_t window_budget(int B, int Hret, int Lmax, int ncu) {
  const int64_t nsel = (int64_t)B * Hret * ((Lmax + 4095) / 4096);
  return std::max<int64_t>(256, 2 * (int64_t)ncu - nsel);
}
int window_rows(int B, int Hloc, int ring, int64_t budget) {
  // rows per window block: one step per wavefront unless that makes more window blocks
  // than the budget; then up to 16 steps per wavefront
  int wr = kBWaves * kStep;
  while (wr < 16 * kBWaves * kStep && (int64_t)B * Hloc * ((ring + wr - 1) / wr) > budget) wr *= 2;
  return wr;
}
}  // namespace

bool step_fused_supported(int kv_dtype, int G, int Hloc, int window, int sinks, int B, int Hret,
                          int Lmax, bool ret_window) {
  if ((kv_dtype != 1 && kv_dtype != 2) || G > kAttnG) return false;
  if (Hloc > 0) {
    const int ring = window + sinks;
    const int wr = window_rows(B, Hloc, ring, window_budget(B, Hret, Lmax, device_cus()));
    if ((ring + wr - 1) / wr > kMaxParts) return false;
  }
  if (Hret > 0 && ret_window) {
    const int ring = window + sinks;
    const int wr = window_rows(B, Hret, ring, 256);
    if ((ring + wr - 1) / wr + (Lmax + 2047) / 2048 > kMaxParts) return false;
  }
  if (Hret > 0 && (Lmax + 4095) / 4096 > kMaxParts) return false;  // stage-M LDS
  return true;
}

StepFusedPlan plan_step_fused(WsPlanner& wp, int B, int Hq, int G, int Lmax, int Hret, int Hloc,
                              int window, int sinks, bool ret_window, bool export_sets) {
  (void)Hq;
  StepFusedPlan sp{};
  sp.exp = export_sets && Hret > 0;
  sp.G = G;
  sp.Hret = Hret;
  sp.Hloc = Hloc;
  sp.tc = chunk_tokens(B, Hret, Lmax);
  sp.nt = sp.tc / 4;
  sp.ncu = device_cus();
  int nwin_blocks = 0;
  if (Hloc > 0) {
    sp.wrows = window_rows(B, Hloc, window + sinks, window_budget(B, Hret, Lmax, sp.ncu));
    sp.nws = (window + sinks + sp.wrows - 1) / sp.wrows;
    nwin_blocks = B * Hloc * sp.nws;
  }
  if (Hret > 0 && ret_window) {  // window blocks of the retrieval heads, sized the same way
    sp.rwrows = window_rows(B, Hret, window + sinks, 256);
    sp.rwnws = (window + sinks + sp.rwrows - 1) / sp.rwrows;
    nwin_blocks += B * Hret * sp.rwnws;
  }
  if (Hret > 0) {
    sp.nchunk = (Lmax + sp.tc - 1) / sp.tc;
    // tokens per selection block: 2048 if that grid, with the window blocks, fits two
    // blocks per CU, else 4096
    sp.nwd = 4;
    {
      const int64_t nb = (int64_t)B * Hret * ((Lmax + 2047) / 2048);
      if (sp.tc <= 2048 && nb + nwin_blocks <= 2 * sp.ncu) sp.nwd = 2;
    }
    sp.tb = 1024 * sp.nwd;
    sp.nblk = (Lmax + sp.tb - 1) / sp.tb;
    // few slices (short sequences): several blocks share a slice's attention steps, as
    // many as still fit two blocks per CU beside the window blocks (the selected tokens per
    // query head do not shrink with the sequence, so their attention would otherwise sit
    // on a few CUs)
    {
      const int64_t nsel = (int64_t)B * Hret * sp.nblk;
      sp.nparts = (int)std::max<int64_t>(1, std::min<int64_t>(16, (2 * (int64_t)sp.ncu - nwin_blocks) / nsel));
    }
    const int H = Hret * G;
    sp.suf = wp.take<float>((size_t)B * H * sp.nchunk * kNB);
    sp.partA = wp.take<int32_t>((size_t)B * H * sp.nchunk);
    sp.codes = wp.take<uint32_t>((size_t)B * H * sp.nchunk * (sp.tc / 4));
    sp.bstar = wp.take<int32_t>((size_t)B * H);
    sp.Aglob = wp.take<int32_t>((size_t)B * H);
    sp.sufq = wp.take<unsigned long long>((size_t)B * H * kNB);
    // stage-T blocks: chunks per block so that the grid is about one block per CU
    {
      const int64_t rc = (int64_t)B * H * sp.nchunk;
      sp.tcpb = (int)std::min<int64_t>(kTMaxCPB, std::max<int64_t>(1, (rc + sp.ncu - 1) / sp.ncu));
      sp.tseg = (sp.nchunk + sp.tcpb - 1) / sp.tcpb;
    }
    const size_t n1 = (size_t)B * Hret * ((size_t)sp.nblk * sp.nparts + sp.rwnws) * G;
    sp.p1m = wp.take<float>(n1);
    sp.p1l = wp.take<float>(n1);
    sp.p1acc = wp.take<float>(n1 * kD);
    sp.p1cnt = wp.take<int32_t>(n1);
    if (sp.exp) {
      sp.xlist = wp.take<uint32_t>((size_t)B * Hret * sp.nblk * sp.tb);
      sp.xn = wp.take<int32_t>((size_t)B * Hret * sp.nblk);
    }
  }
  if (Hloc > 0) {
    const size_t nw = (size_t)B * Hloc * sp.nws * G;
    sp.wpm = wp.take<float>(nw);
    sp.wpl = wp.take<float>(nw);
    sp.wpacc = wp.take<float>(nw * kD);
  }
  sp.bytes = (wp.off + 255) & ~size_t(255);
  if (sp.bytes == 0) sp.bytes = 256;
  return sp;
}

template <typename T>
static T* at(char* ws, size_t off) {
  return reinterpret_cast<T*>(ws + off);
}

// Launch of a one-argument kernel; with both events given they are bound to the kernel's
// own start and end (a profiler's view of its execution, not of its dispatch).
template <typename PT>
static hipError_t launch1(void (*fn)(PT), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                          PT& arg, hipEvent_t e0, hipEvent_t e1) {
  if (e0 && e1) {
    void* args[] = {&arg};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, args, lds, st, e0,
                              e1, 0);
  }
  fn<<<grid, block, lds, st>>>(arg);
  return hipGetLastError();
}

hipError_t launch_step_fused(const StepFusedPlan& sp, char* ws, const StepFusedArgs& a,
                             hipStream_t st, hipEvent_t* ev) {
  const int G = sp.G;
  const int B = a.B;
  const int H = sp.Hret * G;
  // profiling: events 0/1 bound to stage A's execution, 2/3 to stage B's
  hipEvent_t ea0 = ev ? ev[0] : nullptr, ea1 = ev ? ev[1] : nullptr;
  hipEvent_t eb0 = ev ? ev[2] : nullptr, eb1 = ev ? ev[3] : nullptr;
  const float scale2 = a.scale_attn * 1.4426950408889634f;
  // top-k weighs every token one: a zero exponent turns the bin masses into counts
  const float c_log2 = a.topk > 0 ? 0.0f : (float)((double)a.bin_width * 1.4426950408889634);
  hipError_t e = hipSuccess;
  // ---- K1: indexer score + chunk histograms
  StageAParams P{};
  if (sp.Hret > 0) {
    constexpr int GG = 8;
    P.seq_lens = a.seq_lens;
    P.B = B;
    P.Hq = a.Hq;
    P.G = G;
    P.Lmax = a.Lmax;
    P.q_idx = a.q_idx;
    P.k_idx = a.k_idx;
    P.ret = a.ret;
    P.Hret = sp.Hret;
    P.nchunk = sp.nchunk;
    P.ngg = (G + GG - 1) / GG;
    P.yscale = a.scale_idx / a.bin_width;
    P.c_log2 = c_log2;
    P.counts = a.topk > 0 ? 1 : 0;
    P.w = (double)a.bin_width;
    P.suf = at<float>(ws, sp.suf);
    P.partA = at<int32_t>(ws, sp.partA);
    P.codes = at<uint32_t>(ws, sp.codes);
    P.sufq = at<unsigned long long>(ws, sp.sufq);
    const bool app = a.app != nullptr;
    if (app) {
      P.q_pre = a.app->q_pre;
      P.k_pre = a.app->k_pre;
      P.Wq = a.app->Wq_idx;
      P.Wk = a.app->Wk_idx;
      P.k_new = a.app->k_new;
      P.v_new = a.app->v_new;
      P.q_idx_w = const_cast<float*>(a.q_idx);
      P.k_idx_w = const_cast<void*>(a.k_idx);
      P.K_ret_w = const_cast<void*>(a.K_ret);
      P.V_ret_w = const_cast<void*>(a.V_ret);
      P.K_loc_w = const_cast<void*>(a.K_loc);
      P.V_loc_w = const_cast<void*>(a.V_loc);
      P.Hkv = a.Hkv;
      P.Hloc = sp.Hloc;
      P.window = a.window;
      P.sinks = a.sinks;
      P.loc = a.loc;
    }
    const dim3 gA(sp.nchunk, P.ngg, B * sp.Hret);
    // 512-thread blocks take 48-49 KB of LDS, so three fit a CU's 160 KB.  On grids of 16 or
    // more blocks per CU (8M tokens and up at one retrieval head) two per CU stream the keys
    // faster: the LDS request is raised past a third of the CU's (8M 133.2 -> 129.0 us,
    // 16M 258.8 -> 244.9 us per step; at 4M, 8 blocks per CU, three per CU stay 0.5 us ahead)
    size_t ldsA = (size_t)stage_a_lds(sp.nt, app);
    if (sp.nt == 512 && (int64_t)gA.x * gA.y * gA.z >= 16 * (int64_t)sp.ncu)
      ldsA = std::max<size_t>(ldsA, kStageALds2PerCu);
    const bool bf = a.kv_dtype == 2;
    void (*fa)(StageAParams) = nullptr;
    if (sp.nt == 256)
      fa = app ? (bf ? &k_stage_a<256, bf16e, true> : &k_stage_a<256, f16, true>)
               : (bf ? &k_stage_a<256, bf16e, false> : &k_stage_a<256, f16, false>);
    else
      fa = app ? (bf ? &k_stage_a<512, bf16e, true> : &k_stage_a<512, f16, true>)
               : (bf ? &k_stage_a<512, bf16e, false> : &k_stage_a<512, f16, false>);
    e = launch1(fa, gA, dim3(sp.nt), ldsA, st, P, ea0, ea1);
    if (e != hipSuccess) return e;
  }
  // ---- K2: suffix tables
  StageTParams T{};
  if (sp.Hret > 0) {
    T.suf = P.suf;
    T.partA = P.partA;
    T.nchunk = sp.nchunk;
    T.cpb = sp.tcpb;
    // a chunk s cells below the top scales by exp2f(-s c): below 2^-150 that is exactly zero
    // in fp32, so chunks further down than that are skipped without changing the table
    // (counts under top-k never decay)
    T.maxshift = a.topk > 0 ? INT_MAX
                            : (int)std::min<double>(INT_MAX - 1, std::ceil(150.0 / (double)c_log2) + 1.0);
    T.nseg = sp.tseg;
    T.c_log2 = c_log2;
    T.sufq = P.sufq;
    T.Aglob = at<int32_t>(ws, sp.Aglob);
    const dim3 gT(B * H * sp.tseg);
    if (sp.tcpb <= 4)
      k_stage_t<1><<<gT, kThreads, 0, st>>>(T);
    else if (sp.tcpb <= 8)
      k_stage_t<2><<<gT, kThreads, 0, st>>>(T);
    else if (sp.tcpb <= 16)
      k_stage_t<4><<<gT, kThreads, 0, st>>>(T);
    else
      k_stage_t<8><<<gT, kThreads, 0, st>>>(T);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // ---- K3: selection + sparse attention (retrieval) and window attention (local)
  StageBParams Q{};
  Q.seq_lens = a.seq_lens;
  Q.B = B;
  Q.Hq = a.Hq;
  Q.G = G;
  Q.Lmax = a.Lmax;
  Q.Hret = sp.Hret;
  Q.scale2 = scale2;
  Q.nret_blocks = 0;
  if (sp.Hret > 0) {
    Q.nchunk = sp.nchunk;
    Q.tc = sp.tc;
    Q.nblk = sp.nblk;
    Q.nparts = sp.nparts;
    Q.p = a.p;
    Q.topk = a.topk;
    Q.rw_sinks = a.ret_window ? a.sinks : 0;
    Q.rw_window = a.ret_window ? a.window : 0;  // the plan holds rwnws > 0 blocks then
    Q.q = a.q;
    Q.K_ret = a.K_ret;
    Q.V_ret = a.V_ret;
    Q.ret = a.ret;
    Q.partA = P.partA;
    Q.codes = P.codes;
    Q.sufq = T.sufq;
    Q.Aglob = T.Aglob;
    Q.bstar = at<int32_t>(ws, sp.bstar);
    Q.p1m = at<float>(ws, sp.p1m);
    Q.p1l = at<float>(ws, sp.p1l);
    Q.p1acc = at<float>(ws, sp.p1acc);
    Q.p1cnt = at<int32_t>(ws, sp.p1cnt);
    Q.want_count = a.count_out != nullptr || sp.exp;
    Q.xlist = sp.exp ? at<uint32_t>(ws, sp.xlist) : nullptr;
    Q.xn = sp.exp ? at<int32_t>(ws, sp.xn) : nullptr;
    Q.nret_blocks = B * sp.Hret * sp.nblk * sp.nparts;
    Q.rw_nws = sp.rwnws;
    Q.rw_rows = sp.rwrows;
    Q.np_row = sp.nblk * sp.nparts + sp.rwnws;
  }
  const int nrw_blocks = Q.rw_window > 0 ? B * sp.Hret * sp.rwnws : 0;
  Q.nrw_end = Q.nret_blocks + nrw_blocks;
  int nwin_blocks = 0;
  if (sp.Hloc > 0) {
    WinParams& W = Q.win;
    W.seq_lens = a.seq_lens;
    W.Hq = a.Hq;
    W.G = G;
    W.q = a.q;
    W.K_loc = a.K_loc;
    W.V_loc = a.V_loc;
    W.loc = a.loc;
    W.Hloc = sp.Hloc;
    W.window = a.window;
    W.sinks = a.sinks;
    W.nws = sp.nws;
    W.wrows = sp.wrows;
    W.scale2 = scale2;
    W.wpm = at<float>(ws, sp.wpm);
    W.wpl = at<float>(ws, sp.wpl);
    W.wpacc = at<float>(ws, sp.wpacc);
    nwin_blocks = B * sp.Hloc * sp.nws;
  }
  const size_t ldsB = std::max<size_t>(kBWaves * (32 + 2048) * sizeof(float),
                                       sizeof(uint32_t) * (size_t)(sp.Hret > 0 ? sp.tb : 0));
  const int nB = Q.nret_blocks + nrw_blocks + nwin_blocks;
  {
    const bool bf = a.kv_dtype == 2;
    void (*fb)(StageBParams) = nwin_blocks > 0 && sp.wrows > 256
                                   ? stage_b_kernel<true>(sp.nwd, G, bf)
                                   : stage_b_kernel<false>(sp.nwd, G, bf);
    e = launch1(fb, dim3(nB), dim3(kBThreads), ldsB, st, Q, eb0, eb1);
    if (e != hipSuccess) return e;
  }
  // ---- K4: merges
  StageMParams M{};
  M.G = G;
  M.Hq = a.Hq;
  M.out = a.out;
  M.lse = a.lse;
  M.nret = sp.Hret > 0 ? B * sp.Hret * G : 0;
  if (sp.Hret > 0) {
    M.p1m = Q.p1m;
    M.p1l = Q.p1l;
    M.p1acc = Q.p1acc;
    M.p1cnt = Q.p1cnt;
    M.Aglob = Q.Aglob;
    M.bstar = Q.bstar;
    M.nblk = sp.nblk * sp.nparts + sp.rwnws;
    M.Hret = sp.Hret;
    M.ret = a.ret;
    M.count_out = a.count_out;
    M.thresh_out = a.thresh_out;
  }
  const int nwm = sp.Hloc > 0 ? B * sp.Hloc * G : 0;
  if (sp.Hloc > 0) {
    M.wpm = Q.win.wpm;
    M.wpl = Q.win.wpl;
    M.wpacc = Q.win.wpacc;
    M.nws = sp.nws;
    M.Hloc = sp.Hloc;
    M.loc = a.loc;
  }
  const size_t ldsM = sizeof(float) * (kThreads / 64) * 8 * 8;
  k_stage_m<<<(M.nret + nwm) * kMSlices, kThreads, ldsM, st>>>(M);
  e = hipGetLastError();
  if (e == hipSuccess && sp.exp) {
    StageXParams X{};
    X.seq_lens = a.seq_lens;
    X.Hq = a.Hq;
    X.G = G;
    X.Hret = sp.Hret;
    X.Lmax = a.Lmax;
    X.nblk = sp.nblk;
    X.nparts = sp.nparts;
    X.np_row = Q.np_row;
    X.tb = sp.tb;
    X.ret = a.ret;
    X.xlist = Q.xlist;
    X.xn = Q.xn;
    X.p1cnt = Q.p1cnt;
    X.rw_sinks = Q.rw_sinks;
    X.rw_window = Q.rw_window;
    X.sel_idx = a.sel_idx;
    X.sel_count = a.sel_count;
    X.cap = a.sel_cap;
    k_stage_x<<<dim3(sp.nblk, G, B * sp.Hret), kThreads, 0, st>>>(X);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace rtp
