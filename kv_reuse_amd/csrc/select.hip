// Token-level selection: the forced recent window plus the top-k older keys by
// importance, ties to the lower index (news page "两天两连更：小米提前亮出V3底牌",
// section "Token级选择：精准定位大海里的那根针"; importance is the largest
// probability that any query head of the GQA group gives the key).
//
// Two paths share the helpers below.
//
// A. Given float32 scores (hs2_topk_select).  Every candidate's key is the
//    order-preserving image of its score, so ranks are exact from the start:
//      scores_hist     2048-bin histogram of the keys' top 11 bits per row
//                      (LDS per work-group, then device atomics);
//      scores_compact  keys above the k-th key's bin b* and keys in b* go to
//                      two per-row lists (one atomic pair per work-group);
//      scores_finish   one work-group per row ranks bin b* exactly and emits.
//
// B. The fused step (hs2_cross_decoder_step), from the full layer's per-subtile
//    logit maxima.  For a subtile of 16 keys, ub = max_h(max_j s2_hj - lse2_h)
//    bounds the base-2 log-importance of each of its keys, and one of its keys
//    attains it.  Hence the k-th largest ub is at most the k-th largest
//    importance, and a key can be selected only if its subtile's ub reaches it:
//      subtile_hist    histogram of the subtiles' ub (fixed-point log2 key,
//                      bins of 1/32 octave);
//      subtile_score   subtiles whose ub is at or above the bin below the k-th
//                      (a one-bin margin absorbs float32 error) are candidates,
//                      about k of them; their keys' importances are recomputed
//                      in float32 on MFMA;
//      row_select      one work-group per row: the candidates' float32
//                      importances are binned again, keys of the bins around
//                      the k-th are re-ranked by their importance recomputed in
//                      float64 from the bf16 query and key, and the index list
//                      (ascending) plus the window is written.

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kThreads = 256;
constexpr int kHistThreads = 512;
constexpr int kRowThreads = 512;
constexpr int kSubKeys = 16;        // keys per subtile (the full kernel's maxima)
constexpr int kMaxSubChunk = 8192;  // subtiles per work-group (32 per thread)

__device__ __forceinline__ int row_pos(int r, int T, int Hkv, int64_t S) {
  const int t = (r / Hkv) % T;
  return static_cast<int>(S - T + t);
}

__device__ __forceinline__ int64_t row_first(int P, int w) {
  return max(static_cast<int64_t>(0), static_cast<int64_t>(P) - w + 1);
}

__device__ __forceinline__ uint32_t key_from_log2(float y, float ybase) {
  const float z = (y - ybase) * 67108864.0f;  // 2^32 / kYRange
  if (!(z > 0.f)) return 0u;
  if (z >= 4294967040.0f) return 0xFFFFFFFFu;
  return static_cast<uint32_t>(z);
}

// ---------------------------------------------------------------- helpers

// Run by the 64 lanes of one wave over an LDS histogram of kNB bins: the bin
// where the count from the top first reaches k, the count strictly above it
// and the count in it; found = false if the histogram holds fewer than k.
struct KthBin {
  int bstar;
  uint32_t above;
  uint32_t at;
  bool found;
};
__device__ KthBin kth_bin_wave(const uint32_t* lh, uint32_t k) {
  const int lane = threadIdx.x & 63;
  uint32_t lane_sum = 0;
  for (int i = 0; i < 32; ++i) lane_sum += lh[kNB - 1 - 32 * lane - i];
  uint32_t incl = lane_sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  KthBin res{0, __shfl(incl, 63), 0u, false};
  const uint64_t hit = __ballot(incl >= k);
  if (!hit) return res;
  const int owner = __builtin_ctzll(hit);
  int bs = 0;
  uint32_t above = 0, at = 0;
  if (lane == owner) {
    above = incl - lane_sum;
    bs = kNB - 1 - 32 * lane;
    const int bs_end = bs - 31;
    for (;; --bs) {
      at = lh[bs];
      if (above + at >= k || bs == bs_end) break;
      above += at;
    }
  }
  res.bstar = __shfl(bs, owner);
  res.above = __shfl(above, owner);
  res.at = __shfl(at, owner);
  res.found = true;
  return res;
}

// Add a work-group's LDS histogram to the row histogram.  The row's k-th
// largest key is at least this work-group's own k-th largest, so bins below
// (local k-th bin - 1) can never be needed and are not added: device-scope
// atomics are costly.  All threads call it.
__device__ void flush_hist(const uint32_t* lh, uint32_t* __restrict__ hr, uint32_t k,
                           int* s_lo) {
  __syncthreads();
  if (threadIdx.x < 64) {
    const KthBin kb = kth_bin_wave(lh, max(k, 1u));
    if (threadIdx.x == 0) *s_lo = kb.found ? max(0, kb.bstar - 1) : 0;
  }
  __syncthreads();
  for (int i = *s_lo + threadIdx.x; i < kNB; i += blockDim.x)
    if (lh[i]) atomicAdd(&hr[i], lh[i]);
}

// Block-wide exclusive offsets of two per-thread counts; thread 0 reserves the
// block totals with one device atomic each.  Returns this thread's first slots.
__device__ void reserve_two(uint32_t n0, uint32_t n1, uint32_t* ctr0, uint32_t* ctr1,
                            uint32_t (*s_cnt)[16], uint32_t* s_base, uint32_t& o0,
                            uint32_t& o1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  uint32_t i0 = n0, i1 = n1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t a = __shfl_up(i0, off), b = __shfl_up(i1, off);
    if (lane >= off) {
      i0 += a;
      i1 += b;
    }
  }
  if (lane == 63) {
    s_cnt[0][wave] = i0;
    s_cnt[1][wave] = i1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t0 = 0, t1 = 0;
    for (int wv = 0; wv < nwaves; ++wv) {
      const uint32_t a = s_cnt[0][wv], b = s_cnt[1][wv];
      s_cnt[0][wv] = t0;
      s_cnt[1][wv] = t1;
      t0 += a;
      t1 += b;
    }
    s_base[0] = (t0 && ctr0) ? atomicAdd(ctr0, t0) : 0u;
    s_base[1] = (t1 && ctr1) ? atomicAdd(ctr1, t1) : 0u;
    s_base[2] = t0;
    s_base[3] = t1;
  }
  __syncthreads();
  o0 = s_base[0] + s_cnt[0][wave] + i0 - n0;
  o1 = s_base[1] + s_cnt[1][wave] + i1 - n1;
}

struct Cand {
  uint64_t key;  // larger = better
  int32_t idx;   // ties: lower index first
  int32_t pad;
};
__device__ __forceinline__ bool before(const Cand& a, const Cand& b) {
  return a.key > b.key || (a.key == b.key && a.idx < b.idx);
}

// In-LDS bitonic sort of n (power of two) entries into "before" order.
__device__ void bitonic_sort_cands(Cand* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const Cand x = a[lo], y = a[hi];
        if (before(y, x) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Exact radix select over a band source: appends to sel[*s_count ...] the
// indices of the `take` best entries by (64-bit key desc, index asc).
// Source: get(i, key, idx) for i < n; false skips the entry.  All threads call.
template <typename Src>
__device__ void radix_select_band(const Src& src, int64_t n, uint32_t take, int32_t* sel,
                                  uint32_t* s_count, uint32_t* h256, uint64_t* s_thr_hi,
                                  uint32_t* s_thr_lo, uint32_t* s_need) {
  uint64_t thr_hi = 0, mask_hi = 0;
  uint32_t thr_lo = 0, mask_lo = 0;
  uint32_t need = take;
  for (int pass = 0; pass < 12; ++pass) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) h256[i] = 0u;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      uint64_t vhi;
      int32_t j;
      if (!src.get(i, vhi, j)) continue;
      const uint32_t vlo = ~static_cast<uint32_t>(j);
      if ((vhi & mask_hi) != thr_hi || (vlo & mask_lo) != thr_lo) continue;
      const uint32_t digit = pass < 8 ? static_cast<uint32_t>(vhi >> (56 - 8 * pass)) & 255u
                                      : (vlo >> (24 - 8 * (pass - 8))) & 255u;
      atomicAdd(&h256[digit], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t above = 0;
      int dsel = 255;
      for (; dsel > 0; --dsel) {
        if (above + h256[dsel] >= need) break;
        above += h256[dsel];
      }
      *s_need = need - above;
      if (pass < 8) {
        *s_thr_hi = thr_hi | (static_cast<uint64_t>(dsel) << (56 - 8 * pass));
        *s_thr_lo = thr_lo;
      } else {
        *s_thr_hi = thr_hi;
        *s_thr_lo = thr_lo | (static_cast<uint32_t>(dsel) << (24 - 8 * (pass - 8)));
      }
    }
    __syncthreads();
    need = *s_need;
    thr_hi = *s_thr_hi;
    thr_lo = *s_thr_lo;
    if (pass < 8) mask_hi |= 255ull << (56 - 8 * pass);
    else mask_lo |= 255u << (24 - 8 * (pass - 8));
    __syncthreads();
  }
  // every entry whose composite is >= the threshold composite: exactly `take`
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    uint64_t vhi;
    int32_t j;
    if (!src.get(i, vhi, j)) continue;
    const uint32_t vlo = ~static_cast<uint32_t>(j);
    if (vhi > thr_hi || (vhi == thr_hi && vlo >= thr_lo)) sel[atomicAdd(s_count, 1u)] = j;
  }
  __syncthreads();
}

// The best `take` of a band of n entries into sel[*s_count ...]: a bitonic
// sort in LDS when the band fits, the radix select otherwise.  keys/idx hold
// the band (any memory); all threads call it.
__device__ void take_best(const uint64_t* keys, const int32_t* idx, int64_t n, uint32_t take,
                          Cand* cands, int32_t* sel, uint32_t* s_count, uint32_t* h256,
                          uint64_t* s_thr_hi, uint32_t* s_thr_lo, uint32_t* s_need) {
  if (take == 0) return;
  if (n <= kUncCap) {
    const int n2 = next_pow2(static_cast<int>(n));
    for (int i = threadIdx.x; i < n2; i += blockDim.x)
      cands[i] = i < n ? Cand{keys[i], idx[i], 0} : Cand{0ull, 0x7FFFFFFF, 0};
    __syncthreads();
    bitonic_sort_cands(cands, n2);
    const uint32_t base = *s_count;
    for (uint32_t i = threadIdx.x; i < take; i += blockDim.x) sel[base + i] = cands[i].idx;
    __syncthreads();
    if (threadIdx.x == 0) *s_count = base + take;
    __syncthreads();
    return;
  }
  struct ListSrc {
    const uint64_t* k;
    const int32_t* x;
    __device__ bool get(int64_t i, uint64_t& key, int32_t& j) const {
      key = k[i];
      j = x[i];
      return true;
    }
  } src{keys, idx};
  radix_select_band(src, n, take, sel, s_count, h256, s_thr_hi, s_thr_lo, s_need);
}

// Write a row's output: the n_keep selected older keys of tmp sorted ascending
// (into sel; values are distinct, each goes to its rank), then the window
// [first, P], then -1 up to cap.  All threads call it.
__device__ void emit_row(const int32_t* tmp, int32_t* sel, int n_keep, int64_t first, int P,
                         int32_t* __restrict__ out, int32_t* __restrict__ nsel_out, int cap) {
  for (int i = threadIdx.x; i < n_keep; i += blockDim.x) {
    const int32_t v = tmp[i];
    int rank = 0;
    for (int j = 0; j < n_keep; ++j) rank += tmp[j] < v;
    sel[rank] = v;
  }
  __syncthreads();
  const int n_total = n_keep + static_cast<int>(static_cast<int64_t>(P) - first + 1);
  for (int i = threadIdx.x; i < cap; i += blockDim.x) {
    int32_t val = -1;
    if (i < n_keep) val = sel[i];
    else if (i < n_total) val = static_cast<int32_t>(first + (i - n_keep));
    out[i] = val;
  }
  if (threadIdx.x == 0) *nsel_out = n_total;
}

// ================================================================ path A

__global__ void scores_clear_kernel(uint32_t* __restrict__ hist, RowInfo* __restrict__ info) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kNB; i += blockDim.x) hist[static_cast<size_t>(r) * kNB + i] = 0u;
  if (threadIdx.x == 0) info[r] = RowInfo{0, 0, 0, 0, 0u, 0u, 0u, 0};
}

__global__ __launch_bounds__(kHistThreads) void scores_hist_kernel(
    const float* __restrict__ scores, uint32_t* __restrict__ ukey, uint32_t* __restrict__ hist,
    int64_t S, int64_t Spad, int T, int Hkv, int topk, int w, int chunk) {
  __shared__ uint32_t lh[kNB];
  __shared__ int s_lo;
  const int r = blockIdx.y;
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  for (int i = threadIdx.x; i < kNB; i += kHistThreads) lh[i] = 0u;
  __syncthreads();
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t j1 = min(first, j0 + chunk);
  const float* sr = scores + static_cast<size_t>(r) * S;
  uint32_t* ur = ukey + static_cast<size_t>(r) * Spad;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += kHistThreads) {
    const uint32_t u = ordered_u32(sr[j]);
    ur[j] = u;
    atomicAdd(&lh[u >> kBinShift], 1u);
  }
  flush_hist(lh, hist + static_cast<size_t>(r) * kNB, static_cast<uint32_t>(topk), &s_lo);
}

// Keys above bin b* go to the cert list, keys in bin b* to the band list.
__global__ __launch_bounds__(kThreads) void scores_compact_kernel(
    const uint32_t* __restrict__ ukey, const float* __restrict__ scores,
    const uint32_t* __restrict__ hist, RowInfo* __restrict__ info, int32_t* __restrict__ cert,
    int32_t* __restrict__ band_idx, uint64_t* __restrict__ band_key, int64_t S, int64_t Spad,
    int T, int Hkv, int topk, int w, int chunk, int capk) {
  __shared__ uint32_t lh[kNB];
  __shared__ int s_b;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  if (topk <= 0 || first <= topk) return;  // nothing to rank: the finish pass handles it
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t j1 = min(first, j0 + chunk);
  if (j0 >= j1) return;
  for (int i = tid; i < kNB; i += kThreads) lh[i] = hist[static_cast<size_t>(r) * kNB + i];
  __syncthreads();
  if (tid < 64) {
    const KthBin kb = kth_bin_wave(lh, static_cast<uint32_t>(topk));
    if (tid == 0) s_b = kb.bstar;
  }
  __syncthreads();
  const int bstar = s_b;
  const uint32_t* ur = ukey + static_cast<size_t>(r) * Spad;
  // thread t owns keys j0 + t + 256*i, i < 64 (chunk <= 16384)
  uint64_t mc = 0, mu = 0;
  for (int i = 0; i < 64; ++i) {
    const int64_t j = j0 + tid + static_cast<int64_t>(kThreads) * i;
    if (j >= j1) break;
    const int bn = static_cast<int>(ur[j] >> kBinShift);
    if (bn > bstar) mc |= 1ull << i;
    else if (bn == bstar) mu |= 1ull << i;
  }
  uint32_t oc, ou;
  reserve_two(__popcll(mc), __popcll(mu), &info[r].cert_count, &info[r].unc_count, s_cnt, s_base,
              oc, ou);
  for (uint64_t m = mc; m; m &= m - 1) {
    const int i = __builtin_ctzll(m);
    cert[static_cast<size_t>(r) * capk + oc++] = static_cast<int32_t>(j0 + tid + kThreads * i);
  }
  for (uint64_t m = mu; m; m &= m - 1) {
    const int i = __builtin_ctzll(m);
    const int64_t j = j0 + tid + kThreads * i;
    if (ou < static_cast<uint32_t>(kUncCap)) {
      band_idx[static_cast<size_t>(r) * kUncCap + ou] = static_cast<int32_t>(j);
      band_key[static_cast<size_t>(r) * kUncCap + ou] =
          static_cast<uint64_t>(ordered_u32(scores[static_cast<size_t>(r) * S + j]));
    }
    ++ou;
  }
}

__global__ __launch_bounds__(kRowThreads) void scores_finish_kernel(
    const uint32_t* __restrict__ ukey, const float* __restrict__ scores,
    const uint32_t* __restrict__ hist, const RowInfo* __restrict__ info,
    const int32_t* __restrict__ cert, const int32_t* __restrict__ band_idx,
    const uint64_t* __restrict__ band_key, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ nsel_out, int64_t S, int64_t Spad, int T, int Hkv, int topk, int w,
    int capk, int cap) {
  __shared__ uint32_t lh[kNB];
  __shared__ int32_t tmp[kMaxSel];
  __shared__ int32_t sel[kMaxSel];
  __shared__ Cand cands[kUncCap];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_count, s_tlo, s_need;
  __shared__ uint64_t s_thi;
  __shared__ int s_b;
  __shared__ uint32_t s_above;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = row_first(P, w);
  int n_keep = 0;
  if (topk > 0 && first > 0) {
    if (first <= topk) {
      n_keep = static_cast<int>(first);
      for (int i = tid; i < n_keep; i += kRowThreads) tmp[i] = i;
    } else {
      n_keep = topk;
      for (int i = tid; i < kNB; i += kRowThreads) lh[i] = hist[static_cast<size_t>(r) * kNB + i];
      __syncthreads();
      if (tid < 64) {
        const KthBin kb = kth_bin_wave(lh, static_cast<uint32_t>(topk));
        if (tid == 0) {
          s_b = kb.bstar;
          s_above = kb.above;
        }
      }
      __syncthreads();
      const int n_cert = static_cast<int>(s_above);
      for (int i = tid; i < n_cert; i += kRowThreads) tmp[i] = cert[static_cast<size_t>(r) * capk + i];
      if (tid == 0) s_count = static_cast<uint32_t>(n_cert);
      __syncthreads();
      const uint32_t take = static_cast<uint32_t>(topk - n_cert);
      const int64_t n_band = info[r].unc_count;
      if (n_band <= kUncCap) {
        take_best(band_key + static_cast<size_t>(r) * kUncCap,
                  band_idx + static_cast<size_t>(r) * kUncCap, n_band, take, cands, tmp,
                  &s_count, h256, &s_thi, &s_tlo, &s_need);
      } else {
        // the band overflowed its list: rank it by scanning the row
        struct ScanSrc {
          const uint32_t* ur;
          const float* sr;
          int b;
          __device__ bool get(int64_t i, uint64_t& key, int32_t& j) const {
            if (static_cast<int>(ur[i] >> kBinShift) != b) return false;
            key = static_cast<uint64_t>(ordered_u32(sr[i]));
            j = static_cast<int32_t>(i);
            return true;
          }
        } src{ukey + static_cast<size_t>(r) * Spad, scores + static_cast<size_t>(r) * S, s_b};
        radix_select_band(src, first, take, tmp, &s_count, h256, &s_thi, &s_tlo, &s_need);
      }
    }
  }
  __syncthreads();
  emit_row(tmp, sel, n_keep, first, P, idx_out + static_cast<size_t>(r) * cap, nsel_out + r, cap);
}

// ================================================================ path B

__device__ __forceinline__ float row_ybase(const float* __restrict__ ytop_h, int r) {
  float yt = -INFINITY;
  for (int h = 0; h < kG; ++h) yt = fmaxf(yt, ytop_h[static_cast<size_t>(r) * kG + h]);
  return yt - kYRange;
}

__device__ __forceinline__ float subtile_ub(const float* __restrict__ stmax_row, int64_t st,
                                            const float* lse2f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(stmax_row + st * kG);
  const f32x4 b = *reinterpret_cast<const f32x4*>(stmax_row + st * kG + 4);
  float u = a[0] - lse2f[0];
  u = fmaxf(u, a[1] - lse2f[1]);
  u = fmaxf(u, a[2] - lse2f[2]);
  u = fmaxf(u, a[3] - lse2f[3]);
  u = fmaxf(u, b[0] - lse2f[4]);
  u = fmaxf(u, b[1] - lse2f[5]);
  u = fmaxf(u, b[2] - lse2f[6]);
  u = fmaxf(u, b[3] - lse2f[7]);
  return u;
}

// Histogram of the fully-older subtiles' bounds ub (a subtile that reaches into
// the window is always a candidate and is not counted here).
__global__ __launch_bounds__(kThreads) void subtile_hist_kernel(
    const float* __restrict__ stmax, const double* __restrict__ lse2,
    const float* __restrict__ ytop_h, uint32_t* __restrict__ hist, int64_t S, int64_t Spad,
    int T, int Hkv, int topk, int w, int chunk) {
  __shared__ uint32_t lh[kNB];
  __shared__ float lse2f[kG];
  __shared__ float s_ybase;
  __shared__ int s_lo;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  const int64_t n_counted = first / kSubKeys;
  for (int i = tid; i < kNB; i += kThreads) lh[i] = 0u;
  if (tid < kG) lse2f[tid] = static_cast<float>(lse2[static_cast<size_t>(r) * kG + tid]);
  if (tid == 0) s_ybase = row_ybase(ytop_h, r);
  __syncthreads();
  const float ybase = s_ybase;
  const float* stmax_row = stmax + static_cast<size_t>(r) * (Spad / kSubKeys) * kG;
  const int64_t st0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t st1 = min(n_counted, st0 + chunk);
  for (int64_t st = st0 + tid; st < st1; st += kThreads)
    atomicAdd(&lh[key_from_log2(subtile_ub(stmax_row, st, lse2f), ybase) >> kBinShift], 1u);
  flush_hist(lh, hist + static_cast<size_t>(r) * kNB, static_cast<uint32_t>(topk), &s_lo);
}

// Candidate subtiles, then their keys' importances in float32 on MFMA: one wave
// per candidate subtile, S^T = K . Q^T over its 16 keys.
__global__ __launch_bounds__(kThreads) void subtile_score_kernel(
    const float* __restrict__ stmax, const double* __restrict__ lse2,
    const float* __restrict__ ytop_h, const uint32_t* __restrict__ hist,
    RowInfo* __restrict__ info, const u16* __restrict__ q, const u16* __restrict__ k,
    float* __restrict__ cand_y, int32_t* __restrict__ cand_idx, int64_t S, int64_t Spad,
    int T, int Hkv, int topk, int w, int chunk, float c2_hi, float c2_lo) {
  __shared__ uint32_t lh[kNB];
  __shared__ int32_t s_list[kMaxSubChunk];
  __shared__ float lse2f[kG];
  __shared__ float s_ybase;
  __shared__ int s_lo;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  if (topk <= 0 || first == 0) return;
  const int64_t n_counted = first / kSubKeys;
  const int64_t n_sub = (first + kSubKeys - 1) / kSubKeys;
  const int64_t st0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t st1 = min(n_sub, st0 + chunk);
  if (st0 >= st1) return;
  const bool all_mode = n_counted <= topk;
  if (tid < kG) lse2f[tid] = static_cast<float>(lse2[static_cast<size_t>(r) * kG + tid]);
  if (tid == 0) s_ybase = row_ybase(ytop_h, r);
  if (!all_mode)
    for (int i = tid; i < kNB; i += kThreads) lh[i] = hist[static_cast<size_t>(r) * kNB + i];
  __syncthreads();
  if (!all_mode && tid < 64) {
    const KthBin kb = kth_bin_wave(lh, static_cast<uint32_t>(topk));
    if (tid == 0) s_lo = max(0, kb.bstar - 1);
  }
  __syncthreads();
  const int lo_bin = all_mode ? 0 : s_lo;
  const float ybase = s_ybase;
  const float* stmax_row = stmax + static_cast<size_t>(r) * (Spad / kSubKeys) * kG;
  // ---- phase 1: which subtiles of the chunk are candidates
  uint32_t mine = 0;
  for (int i = 0; i < kMaxSubChunk / kThreads; ++i) {
    const int64_t st = st0 + tid + static_cast<int64_t>(kThreads) * i;
    if (st >= st1) break;
    const bool cand =
        all_mode || st >= n_counted ||
        static_cast<int>(key_from_log2(subtile_ub(stmax_row, st, lse2f), ybase) >> kBinShift) >=
            lo_bin;
    if (cand) mine |= 1u << i;
  }
  uint32_t o_list, o_dummy;
  reserve_two(__popc(mine), 0u, nullptr, nullptr, s_cnt, s_base, o_list, o_dummy);
  const uint32_t n_local = s_base[2];
  for (uint32_t m = mine; m; m &= m - 1)
    s_list[o_list++] = static_cast<int32_t>(st0 + tid + kThreads * __builtin_ctz(m));
  __syncthreads();
  if (tid == 0)
    s_base[1] = n_local ? atomicAdd(&info[r].cert_count, n_local * kSubKeys) : 0u;
  __syncthreads();
  const uint32_t base = s_base[1];
  // ---- phase 2: float32 importances of the candidates' keys
  const int col = lane & 15, grp = lane >> 4;
  bf16x8 qb[4];
  {
    const u16* qr = q + static_cast<size_t>(r) * kG * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qb[c] = col < kG ? as_bf16x8(load_u32x4(qr + col * kD + 32 * c + 8 * grp))
                       : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  const int b = r / (T * Hkv);
  const int g = r % Hkv;
  const u16* kr = k + (static_cast<size_t>(b) * Hkv + g) * static_cast<size_t>(S) * kD;
  float* cy = cand_y + static_cast<size_t>(r) * Spad;
  int32_t* ci = cand_idx + static_cast<size_t>(r) * Spad;
  for (uint32_t i = wave; i < n_local; i += kThreads / 64) {
    const int64_t key0 = static_cast<int64_t>(s_list[i]) * kSubKeys;
    int64_t key = key0 + col;
    key = key < S - 1 ? key : S - 1;
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc = mfma_16x16x32(as_bf16x8(load_u32x4(kr + key * kD + 32 * c + 8 * grp)), qb[c], acc);
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = col < kG ? fmaf(acc[e], c2_hi, acc[e] * c2_lo) - lse2f[col] : -INFINITY;
      v = fmaxf(v, __shfl_xor(v, 1));
      v = fmaxf(v, __shfl_xor(v, 2));
      v = fmaxf(v, __shfl_xor(v, 4));
      y[e] = v;
    }
    if (col == 0) {
      const size_t pos = base + static_cast<size_t>(i) * kSubKeys + 4 * grp;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t j = key0 + 4 * grp + e;
        const bool ok = j < first;
        cy[pos + e] = ok ? y[e] : -INFINITY;
        ci[pos + e] = ok ? static_cast<int32_t>(j) : -1;
      }
    }
  }
}

// One work-group per row: exact top-k among the candidates, then emit.
__global__ __launch_bounds__(kRowThreads) void row_select_kernel(
    const RowInfo* __restrict__ info, const float* __restrict__ cand_y,
    const int32_t* __restrict__ cand_idx, const float* __restrict__ ytop_h,
    const double* __restrict__ lse2, const u16* __restrict__ q, const u16* __restrict__ k,
    int32_t* __restrict__ band_idx, uint64_t* __restrict__ band_key,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ nsel_out, int64_t S, int64_t Spad,
    int T, int Hkv, int topk, int w, int cap, double c2) {
  __shared__ uint32_t lh[kNB];
  __shared__ int32_t tmp[kMaxSel];
  __shared__ int32_t sel[kMaxSel];
  __shared__ Cand cands[kUncCap];
  __shared__ double qd[kG * kD];
  __shared__ double l2s[kG];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_count, s_band, s_valid, s_tlo, s_need;
  __shared__ uint64_t s_thi;
  __shared__ int s_lo, s_hi;
  __shared__ float s_ybase;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = row_first(P, w);
  const int64_t n_list = min(static_cast<int64_t>(info[r].cert_count), Spad);
  const float* cy = cand_y + static_cast<size_t>(r) * Spad;
  const int32_t* ci = cand_idx + static_cast<size_t>(r) * Spad;
  int n_keep = 0;
  if (tid == 0) {
    s_count = 0u;
    s_band = 0u;
    s_valid = 0u;
    s_ybase = row_ybase(ytop_h, r);
  }
  for (int i = tid; i < kNB; i += kRowThreads) lh[i] = 0u;
  __syncthreads();
  if (topk > 0 && first > 0) {
    // ---- pass 1: histogram of the candidates' float32 importances
    const float ybase = s_ybase;
    uint32_t nv = 0;
    for (int64_t i = tid; i < n_list; i += kRowThreads) {
      if (ci[i] < 0) continue;
      ++nv;
      atomicAdd(&lh[key_from_log2(cy[i], ybase) >> kBinShift], 1u);
    }
    atomicAdd(&s_valid, nv);
    __syncthreads();
    const uint32_t n_valid = s_valid;
    if (n_valid <= static_cast<uint32_t>(topk)) {
      // every candidate key is kept
      for (int64_t i = tid; i < n_list; i += kRowThreads)
        if (ci[i] >= 0) tmp[atomicAdd(&s_count, 1u)] = ci[i];
      __syncthreads();
      n_keep = static_cast<int>(n_valid);
    } else {
      if (tid < 64) {
        const KthBin kb = kth_bin_wave(lh, static_cast<uint32_t>(topk));
        if (tid == 0) {
          s_lo = max(0, kb.bstar - 1);
          s_hi = min(kNB - 1, kb.bstar + 1);
        }
      }
      // the query heads in float64, for the exact re-ranking of the band
      const u16* qr = q + static_cast<size_t>(r) * kG * kD;
      for (int i = tid; i < kG * kD; i += kRowThreads) qd[i] = static_cast<double>(bf16_bits_to_f32(qr[i]));
      if (tid < kG) l2s[tid] = lse2[static_cast<size_t>(r) * kG + tid];
      __syncthreads();
      // ---- pass 2: bins above the band are selected; the band goes to the
      // row's scratch list
      const int lo = s_lo, hi = s_hi;
      int32_t* bi = band_idx + static_cast<size_t>(r) * Spad;
      uint64_t* bk = band_key + static_cast<size_t>(r) * Spad;
      for (int64_t i = tid; i < n_list; i += kRowThreads) {
        const int32_t j = ci[i];
        if (j < 0) continue;
        const int bn = static_cast<int>(key_from_log2(cy[i], ybase) >> kBinShift);
        if (bn > hi) tmp[atomicAdd(&s_count, 1u)] = j;
        else if (bn >= lo) bi[atomicAdd(&s_band, 1u)] = j;
      }
      __syncthreads();
      const uint32_t n_band = s_band;
      // exact importance of the band keys in float64 (bf16 products are exact)
      const int b = r / (T * Hkv);
      const int g = r % Hkv;
      const u16* kr = k + (static_cast<size_t>(b) * Hkv + g) * static_cast<size_t>(S) * kD;
      for (uint32_t i = tid; i < n_band; i += kRowThreads) {
        const int32_t j = bi[i];
        const u16* kj = kr + static_cast<size_t>(j) * kD;
        u32x4 raw[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) raw[c] = load_u32x4(kj + 8 * c);
        double acc[kG];
#pragma unroll
        for (int h = 0; h < kG; ++h) acc[h] = 0.0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint32_t word = raw[c][t >> 1];
            const double kv = static_cast<double>(
                __uint_as_float((t & 1) ? (word & 0xFFFF0000u) : (word << 16)));
#pragma unroll
            for (int h = 0; h < kG; ++h) acc[h] = fma(qd[h * kD + 8 * c + t], kv, acc[h]);
          }
          // keep the scheduler from hoisting the next chunk's LDS reads of the
          // query (it would run out of registers)
          __builtin_amdgcn_sched_barrier(0);
        }
        double y = -INFINITY;
#pragma unroll
        for (int h = 0; h < kG; ++h) y = fmax(y, c2 * acc[h] - l2s[h]);
        bk[i] = ordered_u64(y);
      }
      __syncthreads();
      const uint32_t take = static_cast<uint32_t>(topk) - s_count;
      take_best(bk, bi, n_band, take, cands, tmp, &s_count, h256, &s_thi, &s_tlo, &s_need);
      n_keep = topk;
    }
  }
  __syncthreads();
  emit_row(tmp, sel, n_keep, first, P, idx_out + static_cast<size_t>(r) * cap, nsel_out + r, cap);
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_scores_select(const Plan& p, const float* scores, int32_t* idx, int32_t* n_sel,
                                void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + p.off_hist);
  RowInfo* info = reinterpret_cast<RowInfo*>(w + p.off_info);
  uint32_t* ukey = reinterpret_cast<uint32_t*>(w + p.off_ukey);
  int32_t* cert = reinterpret_cast<int32_t*>(w + p.off_cert);
  int32_t* bidx = reinterpret_cast<int32_t*>(w + p.off_unc);
  uint64_t* bkey = reinterpret_cast<uint64_t*>(w + p.off_unck);
  const int capk = ((p.k + 63) / 64) * 64;
  hipLaunchKernelGGL(scores_clear_kernel, dim3(p.R), dim3(256), 0, st, hist, info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scores_hist_kernel, dim3(p.sel_nchunk, p.R), dim3(kHistThreads), 0, st,
                     scores, ukey, hist, p.S, p.Spad, p.T, p.Hkv, p.k, p.w, p.sel_chunk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scores_compact_kernel, dim3(p.sel_nchunk, p.R), dim3(kThreads), 0, st,
                     ukey, scores, hist, info, cert, bidx, bkey, p.S, p.Spad, p.T, p.Hkv, p.k,
                     p.w, p.sel_chunk, capk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scores_finish_kernel, dim3(p.R), dim3(kRowThreads), 0, st, ukey, scores,
                     hist, info, cert, bidx, bkey, idx, n_sel, p.S, p.Spad, p.T, p.Hkv, p.k, p.w,
                     capk, p.cap);
  return hipGetLastError();
}

hipError_t launch_fused_select(const Plan& p, const u16* q, const u16* k, int32_t* idx,
                               int32_t* n_sel, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const float* stmax = reinterpret_cast<const float*>(w + p.off_stmax);
  const double* lse2 = reinterpret_cast<const double*>(w + p.off_lse2);
  const float* ytop = reinterpret_cast<const float*>(w + p.off_ytop);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + p.off_hist);
  RowInfo* info = reinterpret_cast<RowInfo*>(w + p.off_info);
  float* cand_y = reinterpret_cast<float*>(w + p.off_cand_y);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(w + p.off_cand_idx);
  const double c2 = p.scale * 1.4426950408889634;  // scale * log2(e)
  const float c2_hi = static_cast<float>(c2);
  const float c2_lo = static_cast<float>(c2 - static_cast<double>(c2_hi));
  hipLaunchKernelGGL(subtile_hist_kernel, dim3(p.st_nchunk, p.R), dim3(kThreads), 0, st, stmax,
                     lse2, ytop, hist, p.S, p.Spad, p.T, p.Hkv, p.k, p.w, p.st_chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(subtile_score_kernel, dim3(p.st_nchunk, p.R), dim3(kThreads), 0, st, stmax,
                     lse2, ytop, hist, info, q, k, cand_y, cand_idx, p.S, p.Spad, p.T, p.Hkv,
                     p.k, p.w, p.st_chunk, c2_hi, c2_lo);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(row_select_kernel, dim3(p.R), dim3(kRowThreads), 0, st, info, cand_y,
                     cand_idx, ytop, lse2, q, k, reinterpret_cast<int32_t*>(w + p.off_band_idx),
                     reinterpret_cast<uint64_t*>(w + p.off_band_key), idx, n_sel, p.S, p.Spad,
                     p.T, p.Hkv, p.k, p.w, p.cap, c2);
  return hipGetLastError();
}

}  // namespace hs2
