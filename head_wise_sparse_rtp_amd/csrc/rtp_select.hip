// Histogram merge, threshold scan and ascending compaction of the top-p set.
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 三,
// 硬件感知解码内核 (256-bin histogram top-p without sorting) and the Top-P set of the
// sparse-attention equation; gist.science summary, section 3 (mass is accumulated
// until the cumulative threshold p is reached).
//
// A chunk partial anchored at top cell A_c moves to the global anchor A = max A_c by
// an integer shift s = A - A_c: chunk bin j lands in global bin j + s (the last bin
// when j + s >= 255) and its mass scales by exp(-s w).  Merges run in fp64, in a fixed
// order, so the result does not depend on scheduling.
#include "rtp_internal.h"

namespace rtp {

namespace {

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int Lmax) {
  int L = seq_lens[b];
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

// Deterministic block sum (fixed tree) of one double per thread; all threads get it.
__device__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// Shift-merge `n` partials (anchor cells A[i], masses m[i*256 + j], either precision)
// into the global anchor Ag.  Thread j returns global bin j (bin 255: the tail total).
// w = 0 merges token counts: no decay with the shift, and no partial is too far down.
template <typename MT>
__device__ double shift_merge(const int32_t* sA, const MT* __restrict__ m, int n, int Ag,
                              double w, double* red) {
  const int j = threadIdx.x;
  double acc = 0.0, tail = 0.0;
  for (int i = 0; i < n; i++) {
    const int Ai = sA[i];
    if (Ai == kEmptyCell) continue;
    const long long s = (long long)Ag - (long long)Ai;
    // exp(-s w) is exactly zero in fp64 beyond this: skipping such a partial changes nothing
    if (w > 0.0 && (double)s * w > 746.0) continue;
    const double f = exp(-(double)s * w);
    const MT* mi = m + (size_t)i * kNB;
    if (j < kNB - 1 && j - s >= 0) acc += (double)mi[j - s] * f;
    if (j + s >= kNB - 1) tail += (double)mi[j] * f;
  }
  tail = block_sum(tail, red);
  return j == kNB - 1 ? tail : acc;
}

// First level: merge up to kMerge1 consecutive chunk partials of one row.
__global__ __launch_bounds__(kThreads) void k_merge1(const float* __restrict__ part_mass,
                                                     const int32_t* __restrict__ part_A,
                                                     int nchunk, int nsplit, double w,
                                                     double* __restrict__ mid_mass,
                                                     int32_t* __restrict__ mid_A) {
  __shared__ int32_t sA[kMerge1];
  __shared__ double red[kThreads];
  const size_t row = blockIdx.y;
  const int split = blockIdx.x;
  const int c0 = split * kMerge1;
  const int n = min(kMerge1, nchunk - c0);
  if ((int)threadIdx.x < n) sA[threadIdx.x] = part_A[row * nchunk + c0 + threadIdx.x];
  __syncthreads();
  int Ag = kEmptyCell;
  for (int i = 0; i < n; i++) Ag = max(Ag, sA[i]);
  if (Ag == kEmptyCell) {
    if (threadIdx.x == 0) mid_A[row * nsplit + split] = kEmptyCell;
    return;
  }
  const double v = shift_merge<float>(sA, part_mass + (row * nchunk + c0) * kNB, n, Ag, w, red);
  mid_mass[(row * nsplit + split) * kNB + threadIdx.x] = v;
  if (threadIdx.x == 0) mid_A[row * nsplit + split] = Ag;
}

// Second level: merge the first-level partials of one row, scan, find b*: the least
// bin whose cumulative mass reaches p Z, or (topk > 0, count histograms) whose cumulative
// count reaches topk; 255 when none does.
__global__ __launch_bounds__(kThreads) void k_threshold(
    const double* __restrict__ mid_mass, const int32_t* __restrict__ mid_A, int nsplit,
    double w, double p, int topk, int32_t* __restrict__ thr, float* __restrict__ hist_out,
    int32_t* __restrict__ thresh_out, HeadMap omap, int H, int G, int Hq, int use_map) {
  extern __shared__ int32_t sA[];  // nsplit entries
  __shared__ double red[kThreads];
  __shared__ double scan[kNB];
  __shared__ int bstar_s;
  const int row = blockIdx.x;  // b * H + h
  const int b = row / H;
  const int h = row % H;
  size_t orow = (size_t)row;
  if (use_map) orow = (size_t)b * Hq + (size_t)omap.kv[h / G] * G + (h % G);
  for (int i = threadIdx.x; i < nsplit; i += kThreads) sA[i] = mid_A[(size_t)row * nsplit + i];
  __syncthreads();
  int Ag = kEmptyCell;
  for (int i = 0; i < nsplit; i++) Ag = max(Ag, sA[i]);
  const int j = threadIdx.x;
  if (Ag == kEmptyCell) {  // empty sequence: nothing selected
    if (hist_out) hist_out[orow * kNB + j] = 0.0f;
    if (j == 0) {
      thr[row * 4 + 0] = 0;
      thr[row * 4 + 1] = 0;
      thr[row * 4 + 2] = 0;
      thr[row * 4 + 3] = 0;
      if (thresh_out) {
        thresh_out[orow * 2 + 0] = 0;
        thresh_out[orow * 2 + 1] = 0;
      }
    }
    return;
  }
  const double mu = shift_merge<double>(sA, mid_mass + (size_t)row * nsplit * kNB, nsplit, Ag,
                                        w, red);
  // inclusive scan over the 256 bins (fixed Hillis-Steele order)
  scan[j] = mu;
  __syncthreads();
  for (int off = 1; off < kNB; off <<= 1) {
    const double add = j >= off ? scan[j - off] : 0.0;
    __syncthreads();
    scan[j] += add;
    __syncthreads();
  }
  if (j == 0) bstar_s = kNB - 1;
  __syncthreads();
  const double Z = scan[kNB - 1];
  if (topk > 0 || p < 1.0) {
    const double target = topk > 0 ? (double)topk : p * Z;
    const bool reach = scan[j] >= target;
    const bool prev = j > 0 ? scan[j - 1] >= target : false;
    if (reach && !prev) bstar_s = j;  // the cumulative sum is monotone: one thread at most
  }
  __syncthreads();
  if (hist_out) hist_out[orow * kNB + j] = (float)mu;
  if (j == 0) {
    thr[row * 4 + 0] = Ag;
    thr[row * 4 + 1] = bstar_s;
    thr[row * 4 + 2] = 1;
    thr[row * 4 + 3] = 0;
    if (thresh_out) {
      thresh_out[orow * 2 + 0] = Ag;
      thresh_out[orow * 2 + 1] = bstar_s;
    }
  }
}

// Tokens kept whatever their bin: the first fs positions and the last fw (fw > 0 only).
__device__ __forceinline__ bool forced(int n, int L, int fs, int fw) {
  return fw > 0 && (n < fs || n >= L - fw);
}

// Per-chunk selection test.  Returns the chunk threshold code: tokens with code <= tau
// are selected; tau = 256 selects every valid token; tau < 0 selects none.
__device__ __forceinline__ int chunk_tau(const int32_t* thr, const int32_t* part_A, size_t row,
                                         int nchunk, int chunk) {
  if (thr[row * 4 + 2] == 0) return -1;
  const int A = thr[row * 4 + 0];
  const int bs = thr[row * 4 + 1];
  const int Ac = part_A[row * nchunk + chunk];
  if (Ac == kEmptyCell) return -1;
  if (bs >= kNB - 1) return 256;
  const long long tau = (long long)bs - ((long long)A - (long long)Ac);
  return tau < 0 ? -1 : (int)tau;
}

template <int TPT>
__global__ __launch_bounds__(kThreads) void k_select_count(
    const int32_t* __restrict__ seq_lens, int H, int Lmax, int nchunk,
    const int32_t* __restrict__ thr, const int32_t* __restrict__ part_A,
    const uint32_t* __restrict__ codes, int32_t* __restrict__ cnt, int fs, int fw) {
  __shared__ int red[kThreads / 64];
  constexpr int TC = kThreads * TPT;
  const size_t row = blockIdx.y;
  const int chunk = blockIdx.x;
  const int b = (int)(row / H);
  const int L = clamp_len(seq_lens, b, Lmax);
  const int tau = chunk_tau(thr, part_A, row, nchunk, chunk);
  const int tid = threadIdx.x;
  int c = 0;
  if (tau >= 0 || fw > 0) {
    const uint32_t* cp = codes + (row * nchunk + chunk) * (size_t)(TC / 4);
#pragma unroll
    for (int qd = 0; qd < TPT / 4; qd++) {
      const uint32_t wd = cp[qd * kThreads + tid];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int n = chunk * TC + (4 * qd + i) * kThreads + tid;
        const int code = (wd >> (8 * i)) & 255;
        const bool s = (tau >= 0 && (tau == 256 || code <= tau)) || forced(n, L, fs, fw);
        c += (n < L && s) ? 1 : 0;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int i = 0; i < kThreads / 64; i++) s += red[i];
    cnt[row * nchunk + chunk] = s;
  }
}

template <int TPT>
__global__ __launch_bounds__(kThreads) void k_select_write(
    const int32_t* __restrict__ seq_lens, int H, int Lmax, int nchunk,
    const int32_t* __restrict__ thr, const int32_t* __restrict__ part_A,
    const uint32_t* __restrict__ codes, const int32_t* __restrict__ cnt,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count, int cap,
    int32_t* __restrict__ count_out, HeadMap omap, int G, int Hq, int use_map, int fs, int fw) {
  __shared__ int wsum[kThreads / 64];
  __shared__ int red[kThreads / 64];
  constexpr int TC = kThreads * TPT;
  const size_t row = blockIdx.y;
  const int chunk = blockIdx.x;
  const int b = (int)(row / H);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  // offset of this chunk = selected tokens of all earlier chunks
  long long off = 0;
  for (int c = tid; c < chunk; c += kThreads) off += cnt[row * nchunk + c];
  for (int o = 32; o > 0; o >>= 1) off += __shfl_xor(off, o, 64);
  if (lane == 0) red[wv] = (int)off;
  __syncthreads();
  long long base_off = 0;
  for (int i = 0; i < kThreads / 64; i++) base_off += red[i];
  const int mine = cnt[row * nchunk + chunk];
  if (chunk == nchunk - 1 && tid == 0) {
    const int total = (int)(base_off + mine);
    sel_count[row] = total;
    if (count_out) {
      const int h = (int)(row % H);
      const size_t orow =
          use_map ? (size_t)b * Hq + (size_t)omap.kv[h / G] * G + (h % G) : row;
      count_out[orow] = total;
    }
  }
  if (mine == 0) return;
  const int L = clamp_len(seq_lens, b, Lmax);
  const int tau = chunk_tau(thr, part_A, row, nchunk, chunk);
  const uint32_t* cp = codes + (row * nchunk + chunk) * (size_t)(TC / 4);
  int32_t* out = sel_idx + row * (size_t)cap;
  long long running = base_off;
  for (int t = 0; t < TPT; t++) {
    const int n = chunk * TC + t * kThreads + tid;
    const uint32_t wd = cp[(t >> 2) * kThreads + tid];
    const int code = (wd >> (8 * (t & 3))) & 255;
    const bool sel = n < L && ((tau >= 0 && (tau == 256 || code <= tau)) || forced(n, L, fs, fw));
    const unsigned long long bal = __ballot(sel);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wv] = __popcll(bal);
    __syncthreads();
    long long wbase = 0;
    int tot = 0;
    for (int i = 0; i < kThreads / 64; i++) {
      if (i < wv) wbase += wsum[i];
      tot += wsum[i];
    }
    const long long pos = running + wbase + before;
    if (sel && pos < cap) out[pos] = n;
    running += tot;
    __syncthreads();
  }
}

// Row (b, h) of the retrieval rows (h = kr*G + g): its set, already ascending, into the
// caller's per-query-head arrays.
__global__ __launch_bounds__(kThreads) void k_export_sets(
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_count, int cap_in,
    HeadMap map, int H, int G, int Hq, int32_t* __restrict__ out_idx,
    int32_t* __restrict__ out_count, int cap_out) {
  const size_t row = blockIdx.x;
  const int b = (int)(row / H);
  const int h = (int)(row % H);
  const size_t orow = (size_t)b * Hq + (size_t)map.kv[h / G] * G + (h % G);
  const int n = sel_count[row];
  const int m = min(min(n, cap_in), cap_out);
  for (int i = threadIdx.x; i < m; i += kThreads)
    out_idx[orow * cap_out + i] = sel_idx[row * cap_in + i];
  if (threadIdx.x == 0) out_count[orow] = n;
}

}  // namespace

hipError_t launch_export_sets(const int32_t* sel_idx, const int32_t* sel_count, int cap_in,
                              const HeadMap& map, int B, int Hq, int Hr, int G, int32_t* out_idx,
                              int32_t* out_count, int cap_out, hipStream_t st) {
  k_export_sets<<<B * Hr * G, kThreads, 0, st>>>(sel_idx, sel_count, cap_in, map, Hr * G, G, Hq,
                                                 out_idx, out_count, cap_out);
  return hipGetLastError();
}

hipError_t launch_threshold(const int32_t* seq_lens, int B, int H, int Lmax, double p, int topk,
                            float bin_width, const ChunkGeom& cg, const SelectBufs& sb,
                            float* hist_out, int32_t* thresh_out, const HeadMap* out_map,
                            int G, int Hq, hipStream_t st) {
  (void)seq_lens;
  (void)Lmax;
  const double w = topk > 0 ? 0.0 : (double)bin_width;
  dim3 g1(cg.nsplit, B * H);
  k_merge1<<<g1, kThreads, 0, st>>>(sb.part_mass, sb.part_A, cg.nchunk, cg.nsplit, w,
                                    sb.mid_mass, sb.mid_A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  HeadMap m{};
  if (out_map) m = *out_map;
  k_threshold<<<B * H, kThreads, sizeof(int32_t) * cg.nsplit, st>>>(
      sb.mid_mass, sb.mid_A, cg.nsplit, w, p, topk, sb.thr, hist_out, thresh_out, m, H, G, Hq,
      out_map ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_select(const int32_t* seq_lens, int B, int H, int Lmax, const ChunkGeom& cg,
                         const SelectBufs& sb, int32_t* sel_idx, int32_t* sel_count, int cap,
                         int32_t* count_out, const HeadMap* out_map, int G, int Hq,
                         hipStream_t st, int force_sinks, int force_window) {
  const int fs = force_sinks, fw = force_window;
  dim3 grid(cg.nchunk, B * H);
  HeadMap m{};
  if (out_map) m = *out_map;
  if (cg.tpt == 4) {
    k_select_count<4><<<grid, kThreads, 0, st>>>(seq_lens, H, Lmax, cg.nchunk, sb.thr,
                                                 sb.part_A, sb.codes, sb.cnt, fs, fw);
  } else {
    k_select_count<8><<<grid, kThreads, 0, st>>>(seq_lens, H, Lmax, cg.nchunk, sb.thr,
                                                 sb.part_A, sb.codes, sb.cnt, fs, fw);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (cg.tpt == 4) {
    k_select_write<4><<<grid, kThreads, 0, st>>>(seq_lens, H, Lmax, cg.nchunk, sb.thr,
                                                 sb.part_A, sb.codes, sb.cnt, sel_idx,
                                                 sel_count, cap, count_out, m, G, Hq,
                                                 out_map ? 1 : 0, fs, fw);
  } else {
    k_select_write<8><<<grid, kThreads, 0, st>>>(seq_lens, H, Lmax, cg.nchunk, sb.thr,
                                                 sb.part_A, sb.codes, sb.cnt, sel_idx,
                                                 sel_count, cap, count_out, m, G, Hq,
                                                 out_map ? 1 : 0, fs, fw);
  }
  return hipGetLastError();
}

size_t plan_select(WsPlanner& wp, int B, int H, int Lmax, const ChunkGeom& cg, size_t offs[7]) {
  (void)Lmax;
  const size_t BH = (size_t)B * H;
  offs[0] = wp.take<float>(BH * cg.nchunk * kNB);
  offs[1] = wp.take<int32_t>(BH * cg.nchunk);
  offs[2] = wp.take<uint32_t>(BH * cg.nchunk * (cg.tc / 4));
  offs[3] = wp.take<double>(BH * cg.nsplit * kNB);
  offs[4] = wp.take<int32_t>(BH * cg.nsplit);
  offs[5] = wp.take<int32_t>(BH * 4);
  offs[6] = wp.take<int32_t>(BH * cg.nchunk);
  return wp.off;
}

SelectBufs bind_select(char* ws, const size_t offs[7]) {
  SelectBufs sb;
  sb.part_mass = reinterpret_cast<float*>(ws + offs[0]);
  sb.part_A = reinterpret_cast<int32_t*>(ws + offs[1]);
  sb.codes = reinterpret_cast<uint32_t*>(ws + offs[2]);
  sb.mid_mass = reinterpret_cast<double*>(ws + offs[3]);
  sb.mid_A = reinterpret_cast<int32_t*>(ws + offs[4]);
  sb.thr = reinterpret_cast<int32_t*>(ws + offs[5]);
  sb.cnt = reinterpret_cast<int32_t*>(ws + offs[6]);
  return sb;
}

}  // namespace rtp
