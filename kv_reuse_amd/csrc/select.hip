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

#include <algorithm>

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


// Histogram bin of a candidate's exact log2 importance (monotone in y).
__device__ __forceinline__ int cand_bin(double y, float ybase) {
  return static_cast<int>(key_from_log2(static_cast<float>(y), ybase) >> kBinShift);
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
  return (a.key > b.key) | ((a.key == b.key) & (a.idx < b.idx));
}

// Exact radix select over a band source: appends to sel[*s_count ...] the
// indices of the `take` best entries by (64-bit key desc, index asc).
// Source: get(i, key, idx) for i < n; false skips the entry.  All threads call.
template <typename Src>
__device__ void radix_select_band(const Src& src, int64_t n, uint32_t take, int32_t* sel,
                                  uint32_t* s_count, uint32_t* h256, uint64_t* s_thr_hi,
                                  uint32_t* s_thr_lo, uint32_t* s_need) {
  const uint32_t limit = *s_count + take;   // sel has room up to here
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
    if (vhi > thr_hi || (vhi == thr_hi && vlo >= thr_lo)) {
      const uint32_t slot = atomicAdd(s_count, 1u);
      if (slot < limit) sel[slot] = j;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- block sort
// Bitonic sort of kRowThreads * E values held E per thread (thread t holds
// elements E*t .. E*t+E-1), into `less` order.  Stages whose partners lie in
// the same thread run in registers, those within a wave through lane
// shuffles, the few across waves through the LDS buffer `xch` (N values).
// All threads call it.
__device__ __forceinline__ int32_t shfl_xor_val(int32_t v, int m) { return __shfl_xor(v, m); }
__device__ __forceinline__ int32_t pick(bool c, int32_t a, int32_t b) { return c ? a : b; }
__device__ __forceinline__ Cand pick(bool c, const Cand& a, const Cand& b) {
  Cand r;
  r.key = c ? a.key : b.key;
  r.idx = c ? a.idx : b.idx;
  r.pad = 0;
  return r;
}
__device__ __forceinline__ Cand shfl_xor_val(const Cand& c, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(c.key), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(c.key >> 32), m);
  return Cand{(static_cast<uint64_t>(hi) << 32) | lo, __shfl_xor(c.idx, m), 0};
}

// The values are distinct except for padding copies of one value, so "swap
// iff the pair is out of order" needs one comparison and no branch.
template <int E, int J, typename T, typename Less>
__device__ __forceinline__ void bitonic_in_thread(T (&v)[E], int k, Less less) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int l = e ^ J;
    if (l > e) {
      const bool asc = ((E * static_cast<int>(threadIdx.x) + e) & k) == 0;
      const bool sw = less(v[l], v[e]) == asc;
      const T a = v[e], b = v[l];
      v[e] = pick(sw, b, a);
      v[l] = pick(sw, a, b);
    }
  }
}

// Sorts the first M = next_pow2(n) positions, which hold every real value
// (positions >= n hold padding that sorts last).
template <int E, typename T, typename Less>
__device__ __forceinline__ void block_bitonic(T (&v)[E], T* xch, int n, Less less) {
  static_assert(E == 4 || E == 8, "4 or 8 values per thread");
  constexpr int N = kRowThreads * E;
  int M = 2;
  while (M < n && M < N) M <<= 1;
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int k = 2; k <= M; k <<= 1) {
#pragma unroll 1
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < E) {
        if (j == 1) bitonic_in_thread<E, 1>(v, k, less);
        else if (j == 2) bitonic_in_thread<E, 2>(v, k, less);
        else bitonic_in_thread<E, E == 8 ? 4 : 2>(v, k, less);
      } else {
        const int tm = j / E;                  // partner thread = tid ^ tm
        const bool asc = ((E * tid) & k) == 0;
        const bool keep_min = ((tid & tm) == 0) == asc;
        T o[E];
        if (tm < 64) {
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = shfl_xor_val(v[e], tm);
        } else {
          __syncthreads();
#pragma unroll
          for (int e = 0; e < E; ++e) xch[E * tid + e] = v[e];
          __syncthreads();
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = xch[E * (tid ^ tm) + e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool take_o = less(o[e], v[e]) == keep_min;
          v[e] = pick(take_o, o[e], v[e]);
        }
      }
    }
  }
  __syncthreads();
}

struct CandBefore {
  __device__ bool operator()(const Cand& a, const Cand& b) const { return before(a, b); }
};
struct IntLess {
  __device__ bool operator()(int32_t a, int32_t b) const { return a < b; }
};

// The best `take` of a band of n entries into sel[*s_count ...], in order.  A
// band that fits in LDS is sorted (key desc, index asc) in one block sort; a
// larger one goes through the radix select.  keys/idx hold the band (any
// memory); all threads call it.
__device__ void take_best(const uint64_t* keys, const int32_t* idx, int64_t n, uint32_t take,
                          Cand* cands, int32_t* sel, uint32_t* s_count, uint32_t* h256,
                          uint64_t* s_thr_hi, uint32_t* s_thr_lo, uint32_t* s_need) {
  if (take == 0) return;
  if (n <= kUncCap) {
    constexpr int E = kUncCap / kRowThreads;
    Cand v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = E * threadIdx.x + e;
      v[e] = i < n ? Cand{keys[i], idx[i], 0} : Cand{0ull, 0x7FFFFFFF, 0};
    }
    const uint32_t base = *s_count;
    block_bitonic<E>(v, cands, static_cast<int>(n), CandBefore{});
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t i = E * threadIdx.x + e;
      if (i < take) sel[base + i] = v[e].idx;
    }
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

template <int E>
__device__ void sort_ascending(const int32_t* tmp, int32_t* xch, int n, int32_t* __restrict__ out) {
  int32_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = E * threadIdx.x + e;
    v[e] = i < n ? tmp[i] : 0x7FFFFFFF;
  }
  block_bitonic<E>(v, xch, n, IntLess{});
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = E * threadIdx.x + e;
    if (i < n) out[i] = v[e];
  }
}

// Write a row's output: the n_keep (<= kMaxSel) selected older keys of tmp in
// ascending order, then the window [first, P], then -1 up to cap.  xch is LDS
// room for kMaxSel values.  All threads call it.
__device__ void emit_row(const int32_t* tmp, int32_t* xch, int n_keep, int64_t first, int P,
                         int32_t* __restrict__ out, int32_t* __restrict__ nsel_out, int cap) {
  if (n_keep > 0) {
    if (n_keep <= 4 * kRowThreads) sort_ascending<4>(tmp, xch, n_keep, out);
    else sort_ascending<kMaxSel / kRowThreads>(tmp, xch, n_keep, out);
  }
  const int n_total = n_keep + static_cast<int>(static_cast<int64_t>(P) - first + 1);
  for (int i = n_keep + threadIdx.x; i < cap; i += blockDim.x)
    out[i] = i < n_total ? static_cast<int32_t>(first + (i - n_keep)) : -1;
  if (threadIdx.x == 0) *nsel_out = n_total;
}

// ================================================================ path A

__global__ void scores_clear_kernel(uint32_t* __restrict__ hist, RowInfo* __restrict__ info) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kNB; i += blockDim.x) hist[static_cast<size_t>(r) * kNB + i] = 0u;
  if (threadIdx.x == 0) info[r] = RowInfo{0u, 0u, 0u, 0u};
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
    if (oc < static_cast<uint32_t>(capk))
      cert[static_cast<size_t>(r) * capk + oc] = static_cast<int32_t>(j0 + tid + kThreads * i);
    ++oc;
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
  __shared__ __align__(16) int32_t tmp[kMaxSel + 4];
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
      const int n_cert = min(static_cast<int>(s_above), topk);
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
    const float* __restrict__ ytop_h, uint32_t* __restrict__ hist, uint32_t* __restrict__ hist_c,
    int64_t S, int64_t Spad, int T, int Hkv, int topk, int w, int chunk) {
  __shared__ uint32_t lh[kNB];
  __shared__ float lse2f[kG];
  __shared__ float s_ybase;
  __shared__ int s_lo;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  const int64_t n_counted = first / kSubKeys;
  // the candidate histogram is filled by the next kernel
  if (blockIdx.x == 0)
    for (int i = tid; i < kNB; i += kThreads) hist_c[static_cast<size_t>(r) * kNB + i] = 0u;
  for (int i = tid; i < kNB; i += kThreads) lh[i] = 0u;
  if (tid < kG) lse2f[tid] = static_cast<float>(lse2[static_cast<size_t>(r) * kG + tid]);
  if (tid == 0) s_ybase = row_ybase(ytop_h, r);
  __syncthreads();
  const float ybase = s_ybase;
  const float* stmax_row = stmax + static_cast<size_t>(r) * (Spad / kSubKeys) * kG;
  const int64_t st0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t st1 = min(n_counted, st0 + chunk);
  for (int64_t sb = st0 + tid; sb < st1; sb += 4 * kThreads) {
    float ub[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t st = sb + u * kThreads;
      ub[u] = st < st1 ? subtile_ub(stmax_row, st, lse2f) : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (sb + u * kThreads < st1)
        atomicAdd(&lh[key_from_log2(ub[u], ybase) >> kBinShift], 1u);
  }
  flush_hist(lh, hist + static_cast<size_t>(r) * kNB, static_cast<uint32_t>(topk), &s_lo);
}

// Candidate subtiles, then their keys' importances in float64 on MFMA (one wave
// per candidate subtile), appended to the row's candidate list, and their
// histogram added to the row's candidate histogram hist_c.
__global__ __launch_bounds__(kThreads) void subtile_score_kernel(
    const float* __restrict__ stmax, const double* __restrict__ lse2,
    const float* __restrict__ ytop_h, const uint32_t* __restrict__ hist,
    uint32_t* __restrict__ hist_c, RowInfo* __restrict__ info, const u16* __restrict__ q,
    const u16* __restrict__ k, double* __restrict__ cand_y, int32_t* __restrict__ cand_idx,
    int64_t S, int64_t Spad, int T, int Hkv, int topk, int w, int chunk, double c2) {
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
  for (int i0 = 0; i0 < kMaxSubChunk / kThreads; i0 += 4) {
    if (st0 + tid + static_cast<int64_t>(kThreads) * i0 >= st1) break;
    float ub[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t st = st0 + tid + static_cast<int64_t>(kThreads) * (i0 + u);
      ub[u] = (st < min(st1, n_counted) && !all_mode) ? subtile_ub(stmax_row, st, lse2f) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t st = st0 + tid + static_cast<int64_t>(kThreads) * (i0 + u);
      if (st >= st1) continue;
      const bool cand = all_mode || st >= n_counted ||
                        static_cast<int>(key_from_log2(ub[u], ybase) >> kBinShift) >= lo_bin;
      if (cand) mine |= 1u << (i0 + u);
    }
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
  // ---- phase 2: float64 importances of the candidates' keys on MFMA.  A
  // wave takes a subtile: D = K . Q^T over 16 keys x 16 (8 used) heads, the
  // contraction split as dim = 32*(lane/16) + step, 32 steps of 4 dims.  The
  // bf16 products are exact in float64.
  for (int i = tid; i < kNB; i += kThreads) lh[i] = 0u;
  const int col = lane & 15, grp = lane >> 4;
  double qd[32];
  {
    const u16* qr = q + static_cast<size_t>(r) * kG * kD + col * kD + 32 * grp;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w4 = col < kG ? load_u32x4(qr + 8 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t word = w4[t >> 1];
        qd[8 * c + t] = static_cast<double>(
            __uint_as_float((t & 1) ? (word & 0xFFFF0000u) : (word << 16)));
      }
    }
  }
  const double l2 = col < kG ? lse2[static_cast<size_t>(r) * kG + col] : 0.0;
  __syncthreads();
  const int b = r / (T * Hkv);
  const int g = r % Hkv;
  const u16* kr = k + (static_cast<size_t>(b) * Hkv + g) * static_cast<size_t>(S) * kD;
  double* cy = cand_y + static_cast<size_t>(r) * Spad;
  int32_t* ci = cand_idx + static_cast<size_t>(r) * Spad;
  auto load_sub = [&](uint32_t i, u32x4 (&ka)[4]) {
    int64_t key = static_cast<int64_t>(s_list[i]) * kSubKeys + col;
    key = key < S - 1 ? key : S - 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) ka[c] = load_u32x4(kr + key * kD + 32 * grp + 8 * c);
  };
  u32x4 ka_cur[4], ka_nxt[4];
  if (static_cast<uint32_t>(wave) < n_local) load_sub(wave, ka_cur);
  for (uint32_t i = wave; i < n_local; i += kThreads / 64) {
    const int64_t key0 = static_cast<int64_t>(s_list[i]) * kSubKeys;
    if (i + kThreads / 64 < n_local) load_sub(i + kThreads / 64, ka_nxt);
    // four independent accumulation chains (one per 8-dim slice of the lane's
    // 32 dims), summed at the end
    f64x4 part[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) part[c] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t word = ka_cur[c][t >> 1];
        const double kv = static_cast<double>(
            __uint_as_float((t & 1) ? (word & 0xFFFF0000u) : (word << 16)));
        part[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(kv, qd[8 * c + t], part[c], 0, 0, 0);
      }
    }
    const f64x4 acc = (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
    for (int c = 0; c < 4; ++c) ka_cur[c] = ka_nxt[c];
    // register e holds key grp + 4e against head col
    double y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      double v = col < kG ? c2 * acc[e] - l2 : -INFINITY;
      v = fmax(v, __shfl_xor(v, 1));
      v = fmax(v, __shfl_xor(v, 2));
      v = fmax(v, __shfl_xor(v, 4));
      y[e] = v;
    }
    if (col < 4) {
      const double ye = col == 0 ? y[0] : col == 1 ? y[1] : col == 2 ? y[2] : y[3];
      const int kk = grp + 4 * col;
      const int64_t j = key0 + kk;
      const bool ok = j < first;
      const size_t pos = base + static_cast<size_t>(i) * kSubKeys + kk;
      cy[pos] = ok ? ye : -INFINITY;
      ci[pos] = ok ? static_cast<int32_t>(j) : -1;
      if (ok) atomicAdd(&lh[cand_bin(ye, ybase)], 1u);
    }
  }
  __syncthreads();
  flush_hist(lh, hist_c + static_cast<size_t>(r) * kNB, static_cast<uint32_t>(topk), &s_lo);
}

// ---- the row's exact top-k from its candidate list, over many work-groups:
// split (above the k-th bin: selected; the k-th bin: band), rank the band,
// rank the selection by index.

constexpr int kSplitPerWG = 16 * kThreads;  // list entries per work-group round
constexpr int kSplitMaxWG = 32;             // work-groups per row (grid-stride)

// Entries in bins above the k-th bin b* of the row's candidate histogram are
// appended to the selection list, entries in b* to the band list.  When the
// histogram holds fewer than k entries every candidate is selected.
__global__ __launch_bounds__(kThreads) void cand_split_kernel(
    RowInfo* __restrict__ info, const uint32_t* __restrict__ hist_c,
    const double* __restrict__ cand_y, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ ytop_h, int32_t* __restrict__ sel_list,
    int32_t* __restrict__ band_idx, uint64_t* __restrict__ band_key, int64_t S, int64_t Spad,
    int T, int Hkv, int topk, int w) {
  __shared__ uint32_t lh[kNB];
  __shared__ int s_b;
  __shared__ float s_ybase;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  if (topk <= 0 || first == 0) return;
  const int64_t n_list = min(static_cast<int64_t>(info[r].cert_count), Spad);
  if (static_cast<int64_t>(blockIdx.x) * kSplitPerWG >= n_list) return;
  for (int i = tid; i < kNB; i += kThreads) lh[i] = hist_c[static_cast<size_t>(r) * kNB + i];
  if (tid == 0) s_ybase = row_ybase(ytop_h, r);
  __syncthreads();
  if (tid < 64) {
    const KthBin kb = kth_bin_wave(lh, static_cast<uint32_t>(topk));
    if (tid == 0) s_b = kb.found ? kb.bstar : -1;
  }
  __syncthreads();
  const int bstar = s_b;
  const float ybase = s_ybase;
  const double* cy = cand_y + static_cast<size_t>(r) * Spad;
  const int32_t* ci = cand_idx + static_cast<size_t>(r) * Spad;
  int32_t* sl = sel_list + static_cast<size_t>(r) * kMaxSel;
  int32_t* gbi = band_idx + static_cast<size_t>(r) * Spad;
  uint64_t* gbk = band_key + static_cast<size_t>(r) * Spad;
  for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * kSplitPerWG; c0 < n_list;
       c0 += static_cast<int64_t>(gridDim.x) * kSplitPerWG) {
    // the list holds whole subtiles: 16 consecutive entries per thread
    const int64_t i0 = c0 + 16 * tid;
    const bool live = i0 < n_list;
    double yv[16];
    int32_t cv[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int4 c4 = live ? *reinterpret_cast<const int4*>(ci + i0 + 4 * u) : int4{-1, -1, -1, -1};
      cv[4 * u] = c4.x;
      cv[4 * u + 1] = c4.y;
      cv[4 * u + 2] = c4.z;
      cv[4 * u + 3] = c4.w;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const double2 y2 = live ? *reinterpret_cast<const double2*>(cy + i0 + 2 * u) : double2{0.0, 0.0};
      yv[2 * u] = y2.x;
      yv[2 * u + 1] = y2.y;
    }
    uint32_t mu = 0, ma = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int bn = cand_bin(yv[e], ybase);
      const bool valid = cv[e] >= 0;
      mu |= static_cast<uint32_t>(valid && bn > bstar) << e;
      ma |= static_cast<uint32_t>(valid && bn == bstar) << e;
    }
    uint32_t ou, oa;
    reserve_two(__popc(mu), __popc(ma), &info[r].up_count, &info[r].unc_count, s_cnt, s_base,
                ou, oa);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if ((mu >> e) & 1u) {
        if (ou < static_cast<uint32_t>(kMaxSel)) sl[ou] = cv[e];
        ++ou;
      } else if ((ma >> e) & 1u) {
        if (oa < static_cast<uint64_t>(Spad)) {
          gbk[oa] = ordered_u64(yv[e]);
          gbi[oa] = cv[e];
        }
        ++oa;
      }
    }
  }
}

// Sizes the rank kernels agree on: selected above the band, band size, and
// how many band entries join the selection.
struct SelCounts {
  uint32_t n_up, n_band, take;
};
__device__ __forceinline__ SelCounts sel_counts(const RowInfo& inf, int topk) {
  SelCounts c;
  c.n_up = min(inf.up_count, static_cast<uint32_t>(topk));
  c.n_band = inf.unc_count;
  c.take = min(static_cast<uint32_t>(topk) - c.n_up, c.n_band);
  return c;
}

// Rank of each band entry by (importance desc, index asc) among the row's band:
// 64 entries per work-group (one per lane), the four waves each count over a
// quarter of the band.  Entries of rank < take join the selection list at
// n_up + rank.  A band above kBandRankMax entries is resolved by work-group 0
// with the radix select.
__global__ __launch_bounds__(kThreads) void band_rank_kernel(
    const RowInfo* __restrict__ info, const int32_t* __restrict__ band_idx,
    const uint64_t* __restrict__ band_key, int32_t* __restrict__ sel_list, int64_t S,
    int64_t Spad, int T, int Hkv, int topk, int w) {
  __shared__ uint32_t part[4][64];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_count, s_tlo, s_need;
  __shared__ uint64_t s_thi;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  if (topk <= 0 || first == 0) return;
  const SelCounts c = sel_counts(info[r], topk);
  if (c.take == 0) return;
  const int32_t* bi = band_idx + static_cast<size_t>(r) * Spad;
  const uint64_t* bk = band_key + static_cast<size_t>(r) * Spad;
  int32_t* sl = sel_list + static_cast<size_t>(r) * kMaxSel;
  if (c.n_band > static_cast<uint32_t>(kBandRankMax)) {
    if (blockIdx.x != 0) return;
    struct ListSrc {
      const uint64_t* k;
      const int32_t* x;
      __device__ bool get(int64_t i, uint64_t& key, int32_t& j) const {
        key = k[i];
        j = x[i];
        return true;
      }
    } src{bk, bi};
    if (tid == 0) s_count = c.n_up;
    __syncthreads();
    radix_select_band(src, min(static_cast<int64_t>(c.n_band), Spad), c.take, sl, &s_count,
                      h256, &s_thi, &s_tlo, &s_need);
    return;
  }
  const uint32_t e0 = blockIdx.x * 64u;
  if (e0 >= c.n_band) return;
  const uint32_t e = e0 + lane;
  const bool mine = e < c.n_band;
  const Cand me = mine ? Cand{bk[e], bi[e], 0} : Cand{0ull, 0x7FFFFFFF, 0};
  // quarters of whole 16-entry blocks; reads past the band stay inside the
  // row's list (n_band <= Spad, both multiples of 64 after rounding) and are
  // masked
  const uint32_t q = ((c.n_band + 3u) / 4u + 15u) & ~15u;
  const uint32_t f0 = wave * q, f1 = min(c.n_band, f0 + q);
  uint32_t beat = 0;
  for (uint32_t f = f0; f < f1; f += 16) {
    uint64_t ok[16];
    int32_t oi[16];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const ulonglong2 k2 = *reinterpret_cast<const ulonglong2*>(bk + f + 2 * u);
      ok[2 * u] = k2.x;
      ok[2 * u + 1] = k2.y;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int4 i4 = *reinterpret_cast<const int4*>(bi + f + 4 * u);
      oi[4 * u] = i4.x;
      oi[4 * u + 1] = i4.y;
      oi[4 * u + 2] = i4.z;
      oi[4 * u + 3] = i4.w;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      beat += static_cast<uint32_t>((f + u < f1) & before(Cand{ok[u], oi[u], 0}, me));
  }
  part[wave][lane] = beat;
  __syncthreads();
  if (wave == 0 && mine) {
    const uint32_t rank = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    if (rank < c.take) sl[c.n_up + rank] = me.idx;
  }
}

// The row's output: the selection in ascending index order (each entry goes to
// its rank; 64 entries per work-group, four waves over quarters of the list),
// then the window [first, P], then -1 up to cap, and the count.
__global__ __launch_bounds__(kThreads) void emit_rank_kernel(
    const RowInfo* __restrict__ info, const int32_t* __restrict__ sel_list,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ nsel_out, int64_t S, int T, int Hkv,
    int topk, int w, int cap) {
  __shared__ uint32_t part[4][64];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = row_first(P, w);
  uint32_t n_keep = 0;
  if (topk > 0 && first > 0) {
    const SelCounts c = sel_counts(info[r], topk);
    n_keep = c.n_up + c.take;
  }
  int32_t* out = idx_out + static_cast<size_t>(r) * cap;
  if (blockIdx.x == 0) {
    const int n_total = static_cast<int>(n_keep) + static_cast<int>(static_cast<int64_t>(P) - first + 1);
    for (int i = static_cast<int>(n_keep) + tid; i < cap; i += kThreads)
      out[i] = i < n_total ? static_cast<int32_t>(first + (i - static_cast<int>(n_keep))) : -1;
    if (tid == 0) nsel_out[r] = n_total;
  }
  const uint32_t e0 = blockIdx.x * 64u;
  if (e0 >= n_keep) return;
  const int32_t* sl = sel_list + static_cast<size_t>(r) * kMaxSel;
  const uint32_t e = e0 + lane;
  const bool mine = e < n_keep;
  const int32_t me = mine ? sl[e] : 0x7FFFFFFF;
  // quarters of whole 16-entry blocks (reads stay inside the row's kMaxSel
  // entries and are masked past n_keep)
  const uint32_t q = ((n_keep + 3u) / 4u + 15u) & ~15u;
  const uint32_t f0 = wave * q, f1 = min(n_keep, f0 + q);
  uint32_t below = 0;
  for (uint32_t f = f0; f < f1; f += 16) {
    int32_t o[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int4 i4 = *reinterpret_cast<const int4*>(sl + f + 4 * u);
      o[4 * u] = i4.x;
      o[4 * u + 1] = i4.y;
      o[4 * u + 2] = i4.z;
      o[4 * u + 3] = i4.w;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) below += static_cast<uint32_t>((f + u < f1) & (o[u] < me));
  }
  part[wave][lane] = below;
  __syncthreads();
  if (wave == 0 && mine) {
    const uint32_t rank = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    if (rank < n_keep) out[rank] = me;
  }
}

// ================================================================ prefill chunk

// One work-group per row (b, t, g) of a prefill chunk: the exact top-k of the
// row's older keys from their float32 log2 importance y and the row's
// complete histogram.  Bins above b*+1 are selected; keys in bins b*-1..b*+1
// (the float32 error of y is far below a bin) get their importance recomputed
// in float64 from exact bf16 products and are ranked (importance desc, index
// asc).  A band larger than band_cap is ranked by its float32 y instead.
__global__ __launch_bounds__(kRowThreads) void prefill_select_kernel(
    const float* __restrict__ ybuf, const uint32_t* __restrict__ hist,
    const float* __restrict__ ytop_h, const double* __restrict__ lse2, const u16* __restrict__ q,
    const u16* __restrict__ k, int32_t* __restrict__ band_idx, uint64_t* __restrict__ band_key,
    int64_t band_cap, int32_t* __restrict__ idx_out, int32_t* __restrict__ nsel_out, int64_t S,
    int64_t Spad, int T, int Hkv, int topk, int w, int cap, double c2) {
  __shared__ __align__(16) int32_t tmp[kMaxSel];
  __shared__ __align__(16) uint32_t sel_lh[kMaxSel];   // histogram first, emit scratch last
  __shared__ __align__(16) Cand cands[kUncCap];        // band (keys, indices), then sort scratch
  __shared__ double qd[kG * kD];
  __shared__ double l2s[kG];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_count, s_tlo, s_need;
  __shared__ uint64_t s_thi;
  __shared__ int s_b, s_lo, s_hi;
  __shared__ uint32_t s_nband;
  __shared__ float s_ybase;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  uint32_t* lh = sel_lh;
  uint64_t* lband_k = reinterpret_cast<uint64_t*>(cands);
  int32_t* lband_i = reinterpret_cast<int32_t*>(lband_k + kUncCap);
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = row_first(P, w);
  int n_keep = 0;
  if (topk > 0 && first > 0) {
    for (int i = tid; i < kNB; i += kRowThreads) lh[i] = hist[static_cast<size_t>(r) * kNB + i];
    if (tid == 0) s_ybase = row_ybase(ytop_h, r);
    __syncthreads();
    if (tid < 64) {
      const KthBin kb = kth_bin_wave(lh, static_cast<uint32_t>(topk));
      if (tid == 0) {
        s_b = kb.found ? kb.bstar : -1;
        if (kb.found) {
          const int lo = max(0, kb.bstar - 1), hi = min(kNB - 1, kb.bstar + 1);
          uint32_t nb = 0;
          for (int bb = lo; bb <= hi; ++bb) nb += lh[bb];
          s_lo = lo;
          s_hi = hi;
          s_nband = nb;
        }
      }
    }
    __syncthreads();
    if (s_b < 0) {
      // fewer older keys than top_k: all of them
      n_keep = static_cast<int>(min(first, static_cast<int64_t>(kMaxSel)));
      for (int i = tid; i < n_keep; i += kRowThreads) tmp[i] = i;
    } else {
      const int lo = s_lo, hi = s_hi;
      const uint32_t n_band_h = s_nband;
      const bool band_lds = n_band_h <= static_cast<uint32_t>(kUncCap);
      const bool band_glob = !band_lds && n_band_h <= static_cast<uint64_t>(band_cap);
      const float ybase = s_ybase;
      const float* yr = ybuf + static_cast<size_t>(r) * Spad;
      int32_t* gbi = band_idx + static_cast<size_t>(r) * band_cap;
      uint64_t* gbk = band_key + static_cast<size_t>(r) * band_cap;
      const u16* qr = q + static_cast<size_t>(r) * kG * kD;
      for (int i = tid; i < kG * kD; i += kRowThreads) qd[i] = static_cast<double>(bf16_bits_to_f32(qr[i]));
      if (tid < kG) l2s[tid] = lse2[static_cast<size_t>(r) * kG + tid];
      // ---- one pass over y: above the band -> tmp, band -> band list
      const int64_t rounds = (first + 16 * kRowThreads - 1) / (16 * kRowThreads);
      uint32_t cu = 0, ca = 0;
      for (int64_t rr = 0; rr < rounds; ++rr) {
        const int64_t i0 = 16 * (static_cast<int64_t>(tid) + rr * kRowThreads);
        float yv[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 y4 = i0 + 4 * u < first ? *reinterpret_cast<const f32x4*>(yr + i0 + 4 * u)
                                                : f32x4{0.f, 0.f, 0.f, 0.f};
          yv[4 * u] = y4[0];
          yv[4 * u + 1] = y4[1];
          yv[4 * u + 2] = y4[2];
          yv[4 * u + 3] = y4[3];
        }
        uint32_t mu = 0, ma = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool valid = i0 + e < first;
          const int bn = static_cast<int>(key_from_log2(yv[e], ybase) >> kBinShift);
          mu |= static_cast<uint32_t>(valid && bn > hi) << e;
          ma |= static_cast<uint32_t>(valid && bn >= lo && bn <= hi) << e;
        }
        uint32_t ou, oa;
        reserve_two(__popc(mu), __popc(ma), nullptr, nullptr, s_cnt, s_base, ou, oa);
        const uint32_t tu = s_base[2], ta = s_base[3];
        ou += cu;
        oa += ca;
        cu += tu;
        ca += ta;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int32_t j = static_cast<int32_t>(i0 + e);
          if ((mu >> e) & 1u) {
            if (ou < static_cast<uint32_t>(kMaxSel)) tmp[ou] = j;
            ++ou;
          } else if ((ma >> e) & 1u) {
            if (band_lds) {
              if (oa < static_cast<uint32_t>(kUncCap)) lband_i[oa] = j;
            } else if (band_glob) {
              if (oa < static_cast<uint64_t>(band_cap)) gbi[oa] = j;
            }
            ++oa;
          }
        }
      }
      __syncthreads();
      const uint32_t n_up = min(cu, static_cast<uint32_t>(topk));
      const uint32_t take = static_cast<uint32_t>(topk) - n_up;
      if (tid == 0) s_count = n_up;
      if (band_lds || band_glob) {
        const uint32_t n_band = band_lds ? min(ca, static_cast<uint32_t>(kUncCap))
                                         : static_cast<uint32_t>(min(static_cast<int64_t>(ca), band_cap));
        // exact importance of the band keys in float64 (bf16 products are exact)
        const int b = r / (T * Hkv);
        const int g = r % Hkv;
        const u16* kr = k + (static_cast<size_t>(b) * Hkv + g) * static_cast<size_t>(S) * kD;
        for (uint32_t i = tid; i < n_band; i += kRowThreads) {
          const int32_t j = band_lds ? lband_i[i] : gbi[i];
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
            // keep the next chunk's LDS reads of the query from being hoisted
            __builtin_amdgcn_sched_barrier(0);
          }
          double yy = -INFINITY;
#pragma unroll
          for (int h = 0; h < kG; ++h) yy = fmax(yy, c2 * acc[h] - l2s[h]);
          if (band_lds) lband_k[i] = ordered_u64(yy);
          else gbk[i] = ordered_u64(yy);
        }
        __syncthreads();
        take_best(band_lds ? lband_k : gbk, band_lds ? lband_i : gbi, n_band,
                  min(take, n_band), cands, tmp, &s_count, h256, &s_thi, &s_tlo, &s_need);
      } else {
        // the band is too large to list: rank it by its float32 importance
        __syncthreads();
        struct ScanSrc {
          const float* yr;
          float ybase;
          int lo, hi;
          __device__ bool get(int64_t i, uint64_t& key, int32_t& j) const {
            const float yy = yr[i];
            const int bn = static_cast<int>(key_from_log2(yy, ybase) >> kBinShift);
            if (bn < lo || bn > hi) return false;
            key = static_cast<uint64_t>(ordered_u32(yy));
            j = static_cast<int32_t>(i);
            return true;
          }
        } src{yr, ybase, lo, hi};
        radix_select_band(src, first, min(take, ca), tmp, &s_count, h256, &s_thi, &s_tlo, &s_need);
      }
      n_keep = static_cast<int>(min(s_count, static_cast<uint32_t>(topk)));
    }
  }
  __syncthreads();
  emit_row(tmp, reinterpret_cast<int32_t*>(sel_lh), n_keep, first, P,
           idx_out + static_cast<size_t>(r) * cap, nsel_out + r, cap);
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
  uint32_t* hist_c = reinterpret_cast<uint32_t*>(w + p.off_hist_c);
  RowInfo* info = reinterpret_cast<RowInfo*>(w + p.off_info);
  double* cand_y = reinterpret_cast<double*>(w + p.off_cand_y);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(w + p.off_cand_idx);
  const double c2 = p.scale * 1.4426950408889634;  // scale * log2(e)
  hipLaunchKernelGGL(subtile_hist_kernel, dim3(p.st_nchunk, p.R), dim3(kThreads), 0, st, stmax,
                     lse2, ytop, hist, hist_c, p.S, p.Spad, p.T, p.Hkv, p.k, p.w, p.st_chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(subtile_score_kernel, dim3(p.st_nchunk, p.R), dim3(kThreads), 0, st, stmax,
                     lse2, ytop, hist, hist_c, info, q, k, cand_y, cand_idx, p.S, p.Spad, p.T,
                     p.Hkv, p.k, p.w, p.st_chunk, c2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n_split = std::min<int64_t>((p.Spad + kSplitPerWG - 1) / kSplitPerWG, kSplitMaxWG);
  int32_t* sel_list = reinterpret_cast<int32_t*>(w + p.off_sel_list);
  int32_t* band_idx = reinterpret_cast<int32_t*>(w + p.off_band_idx);
  uint64_t* band_key = reinterpret_cast<uint64_t*>(w + p.off_band_key);
  hipLaunchKernelGGL(cand_split_kernel, dim3(static_cast<unsigned>(n_split), p.R), dim3(kThreads),
                     0, st, info, hist_c, cand_y, cand_idx, ytop, sel_list, band_idx, band_key,
                     p.S, p.Spad, p.T, p.Hkv, p.k, p.w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(band_rank_kernel, dim3(kBandRankMax / 64, p.R), dim3(kThreads), 0, st, info,
                     band_idx, band_key, sel_list, p.S, p.Spad, p.T, p.Hkv, p.k, p.w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(emit_rank_kernel, dim3(kMaxSel / 64, p.R), dim3(kThreads), 0, st, info,
                     sel_list, idx, n_sel, p.S, p.T, p.Hkv, p.k, p.w, p.cap);
  return hipGetLastError();
}

hipError_t launch_prefill_select(const Plan& p, const u16* q, const u16* k, int32_t* idx,
                                 int32_t* n_sel, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  hipLaunchKernelGGL(prefill_select_kernel, dim3(p.R), dim3(kRowThreads), 0, st,
                     reinterpret_cast<const float*>(w + p.off_ybuf),
                     reinterpret_cast<const uint32_t*>(w + p.off_hist),
                     reinterpret_cast<const float*>(w + p.off_ytop),
                     reinterpret_cast<const double*>(w + p.off_lse2), q, k,
                     reinterpret_cast<int32_t*>(w + p.off_band_idx),
                     reinterpret_cast<uint64_t*>(w + p.off_band_key), p.band_cap, idx, n_sel, p.S,
                     p.Spad, p.T, p.Hkv, p.k, p.w, p.cap, c2);
  return hipGetLastError();
}

}  // namespace hs2
