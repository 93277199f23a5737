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
#include <type_traits>

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kThreads = 256;
constexpr int kHistThreads = 512;
constexpr int kRowThreads = 512;
constexpr int kSubKeys = 16;        // keys per subtile (the full kernel's maxima)

__device__ __forceinline__ int row_pos(int r, int T, int Hkv, int64_t S) {
  const int t = (r / Hkv) % T;
  return static_cast<int>(S - T + t);
}

__device__ __forceinline__ int64_t row_first(int P, int w) {
  return max(static_cast<int64_t>(0), static_cast<int64_t>(P) - w + 1);
}


// Two packed 16-bit values.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Histogram bin of a candidate's exact log2 importance (monotone in y).
__device__ __forceinline__ int cand_bin(double y, float ybase) {
  return static_cast<int>(key_from_log2(static_cast<float>(y), ybase) >> kBinShift);
}

// ---------------------------------------------------------------- helpers

// Wave-wide scans and reductions on the VALU's cross-lane paths: DPP moves
// inside each row of 16 lanes, row broadcasts (GFX9 DPP) or the gfx950 row
// swaps across rows.  An LDS permute (ds_bpermute) costs a round trip through
// the LDS pipeline per step; these do not, which matters in the one-work-group
// per row kernels whose time is a chain of such steps.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  // lanes whose source is outside the row, or whose row is masked off, read 0
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, kRowMask, 0xF, true));
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_mov<0x111>(x);        // row_shr:1
  x += dpp_mov<0x112>(x);        // row_shr:2
  x += dpp_mov<0x114>(x);        // row_shr:4
  x += dpp_mov<0x118>(x);        // row_shr:8: each row now holds its own prefix sums
  x += dpp_mov<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_mov<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}
// v combined over all 64 lanes, in every lane (op associative and commutative).
template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce(uint32_t v, Op op) {
  v = op(v, dpp_mov<0xB1>(v));    // quad_perm [1,0,3,2]: lane ^ 1
  v = op(v, dpp_mov<0x4E>(v));    // quad_perm [2,3,0,1]: lane ^ 2
  v = op(v, dpp_mov<0x141>(v));   // row_half_mirror: the other quad of the 8
  v = op(v, dpp_mov<0x140>(v));   // row_mirror: the other half of the row
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);         // rows 0|1 and 2|3
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);      // rows 0-1 | 2-3
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a & b; });
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a | b; });
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  return wave_allreduce(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}
// Lane `src`'s value (src the same in every lane).
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int src) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), src));
}
__device__ __forceinline__ uint64_t lane_value64(uint64_t v, int src) {
  return (static_cast<uint64_t>(lane_value(static_cast<uint32_t>(v >> 32), src)) << 32) |
         lane_value(static_cast<uint32_t>(v), src);
}
template <int kCtrl>
__device__ __forceinline__ double dpp_mov_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint64_t lo = dpp_mov<kCtrl>(static_cast<uint32_t>(u));
  const uint64_t hi = dpp_mov<kCtrl>(static_cast<uint32_t>(u >> 32));
  return __longlong_as_double(static_cast<long long>((hi << 32) | lo));
}
// The other rows' values through the gfx950 row swaps: the largest of a double
// over lanes l, l ^ 16, l ^ 32, l ^ 48 (in every lane).
__device__ __forceinline__ double max_over_rows_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const auto l16 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u), static_cast<uint32_t>(u), false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u >> 32), static_cast<uint32_t>(u >> 32), false, false);
  auto join = [](uint32_t hi, uint32_t lo) {
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
  };
  v = fmax(join(h16[0], l16[0]), join(h16[1], l16[1]));
  const uint64_t w = static_cast<uint64_t>(__double_as_longlong(v));
  const auto l32 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(w), static_cast<uint32_t>(w), false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(w >> 32), static_cast<uint32_t>(w >> 32), false, false);
  return fmax(join(h32[0], l32[0]), join(h32[1], l32[1]));
}
// Sum over each group of 8 lanes (lane ^ 1, ^ 2, ^ 4 butterfly order), in
// every lane of the group.
__device__ __forceinline__ double oct_sum(double v) {
  v += dpp_mov_f64<0xB1>(v);
  v += dpp_mov_f64<0x4E>(v);
  v += dpp_mov_f64<0x141>(v);
  return v;
}
// Sum over each row of 16 lanes, in every lane of the row: the pairing tree of
// a lane ^ 1, ^ 2, ^ 4, ^ 8 butterfly, so every lane holds the same value.
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_mov_f64<0xB1>(v);    // lane ^ 1
  v += dpp_mov_f64<0x4E>(v);    // lane ^ 2
  v += dpp_mov_f64<0x141>(v);   // the other quad of the 8
  v += dpp_mov_f64<0x140>(v);   // the other half of the row
  return v;
}

// Run by the 64 lanes of one wave over an LDS histogram of kNB bins: the bin
// where the count from the top first reaches k, the count strictly above it
// and the count in it; found = false if the histogram holds fewer than k.
struct KthBin {
  int bstar;
  uint32_t above;
  uint32_t at;
  bool found;
};
template <int NB>
__device__ KthBin kth_bin_wave_n(const uint32_t* lh, uint32_t k) {
  constexpr int kPer = NB / 64;   // bins per lane at level 1
  static_assert(kPer >= 1 && kPer <= 64, "64..4096 bins");
  const int lane = threadIdx.x & 63;
  // level 1: lane l sums the kPer bins NB-1-kPer*l .. NB-kPer-kPer*l
  uint32_t lane_sum = 0;
  for (int i = 0; i < kPer; ++i) lane_sum += lh[NB - 1 - kPer * lane - i];
  const uint32_t incl = wave_incl_scan(lane_sum);
  KthBin res{0, lane_value(incl, 63), 0u, false};
  const uint64_t hit = __ballot(incl >= k);
  if (!hit) return res;
  const int owner = __builtin_ctzll(hit);
  const uint32_t above0 = lane_value(incl - lane_sum, owner);
  // level 2: lanes 0..kPer-1 take the owner's bins from the top
  const int bin = NB - 1 - kPer * owner - (lane % kPer);
  const uint32_t c = lane < kPer ? lh[bin] : 0u;
  const uint32_t inc2 = wave_incl_scan(c);
  const uint64_t hit2 = __ballot(lane < kPer && above0 + inc2 >= k);
  const int jj = __builtin_ctzll(hit2);   // the owner's group reaches k, so some lane hits
  res.bstar = NB - 1 - kPer * owner - jj;
  res.above = above0 + lane_value(inc2 - c, jj);
  res.at = lane_value(c, jj);
  res.found = true;
  return res;
}
__device__ __forceinline__ KthBin kth_bin_wave(const uint32_t* lh, uint32_t k) {
  return kth_bin_wave_n<kNB>(lh, k);
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
  const uint32_t i0 = wave_incl_scan(n0), i1 = wave_incl_scan(n1);
  if (lane == 63) {
    s_cnt[0][wave] = i0;
    s_cnt[1][wave] = i1;
  }
  __syncthreads();
  if (wave == 0) {
    // the waves' totals (at most 16) scanned by lanes 0 .. nwaves-1
    const uint32_t c0 = lane < nwaves ? s_cnt[0][lane] : 0u;
    const uint32_t c1 = lane < nwaves ? s_cnt[1][lane] : 0u;
    const uint32_t x0 = wave_incl_scan(c0), x1 = wave_incl_scan(c1);
    if (lane < nwaves) {
      s_cnt[0][lane] = x0 - c0;
      s_cnt[1][lane] = x1 - c1;
    }
    if (lane == nwaves - 1) {
      s_base[0] = (x0 && ctr0) ? atomicAdd(ctr0, x0) : 0u;
      s_base[1] = (x1 && ctr1) ? atomicAdd(ctr1, x1) : 0u;
      s_base[2] = x0;
      s_base[3] = x1;
    }
  }
  __syncthreads();
  o0 = s_base[0] + s_cnt[0][wave] + i0 - n0;
  o1 = s_base[1] + s_cnt[1][wave] + i1 - n1;
}

// Block-wide exclusive offsets of one or two per-thread counts with a single
// barrier: each wave's totals go to its slots of buf, and every thread then
// sums the slots before its wave.  Consecutive calls must alternate between
// two buffers, so that a wave running ahead into the next call never
// overwrites totals another wave is still reading.  NW = waves per block.
template <int NW>
__device__ __forceinline__ void block_offsets2(uint32_t n0, uint32_t n1, uint32_t (*buf)[NW],
                                               uint32_t& o0, uint32_t& o1, uint32_t& t0,
                                               uint32_t& t1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t i0 = wave_incl_scan(n0), i1 = wave_incl_scan(n1);
  if (lane == 63) {
    buf[0][wave] = i0;
    buf[1][wave] = i1;
  }
  __syncthreads();
  uint32_t b0 = 0, b1 = 0, a0 = 0, a1 = 0;
#pragma unroll
  for (int wv = 0; wv < NW; ++wv) {
    const uint32_t c0 = buf[0][wv], c1 = buf[1][wv];
    a0 += c0;
    a1 += c1;
    b0 += wv < wave ? c0 : 0u;
    b1 += wv < wave ? c1 : 0u;
  }
  o0 = b0 + i0 - n0;
  o1 = b1 + i1 - n1;
  t0 = a0;
  t1 = a1;
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
  if (threadIdx.x == 0) *nsel_out = min(n_total, cap);
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

// The candidate subtiles of a row, in ascending order: a subtile is a
// candidate when its bound's bin is at least (k-th bound bin - 1), since every
// key that can be selected lies in one.  grid (cc chunks, R); each work-group
// lists the candidates of its range of subtiles into its own region of the
// row's list and counts them in ccnt.  Work-group 0 of a row also writes the
// row's lower bin for the next kernel.  The same pass lists, in dlist / dcnt,
// the subtiles whose bound reaches the refinement's cut (refine_cut_wave): the
// ones the refinement of lse2 sums again.
// A list entry is the subtile's index with, in bits kQuadShift.., the mask of
// its quads (4 keys each; all four when the plan writes no quad distances)
// whose own bound (the subtile's maximum of head h
// less the quad's stored distance below it) reaches the bottom of the bin
// below the lower bin for some head: the only quads whose keys the scoring
// kernel's float32 filter can pass.  The stored distances are rounded down,
// so these bounds are never below the quads' maxima (the subtraction's
// rounding aside, far inside the filter's one-bin margin).
constexpr int kQuadShift = 27;   // subtile indices are below 2^31 / 16
constexpr int32_t kSubMask = (1 << kQuadShift) - 1;
__global__ __launch_bounds__(kThreads) void subtile_cand_kernel(
    const float* __restrict__ stmax, const unsigned char* __restrict__ qdiff,
    const double* __restrict__ lse2,
    const float* __restrict__ ytop_h, const uint32_t* __restrict__ hist,
    int32_t* __restrict__ clist, uint32_t* __restrict__ ccnt, int32_t* __restrict__ lo_out,
    int32_t* __restrict__ dlist, uint32_t* __restrict__ dcnt, float* __restrict__ cut_out,
    uint32_t budget, int64_t S, int64_t Spad, int T, int Hkv, int topk, int w, int chunk,
    int n_chunks) {
  __shared__ uint32_t lh[kNB];
  __shared__ float lse2f[kG];
  __shared__ float s_ybase;
  __shared__ int s_lo;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  __shared__ float s_cut;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  const int64_t n_counted = first / kSubKeys;
  const int64_t n_sub = (first + kSubKeys - 1) / kSubKeys;
  const int64_t st0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t st1 = min(n_sub, st0 + chunk);
  uint32_t* cnt = ccnt + static_cast<size_t>(r) * n_chunks + blockIdx.x;
  uint32_t* dct = dcnt + static_cast<size_t>(r) * n_chunks + blockIdx.x;
  if (topk <= 0 || first == 0 || st0 >= st1) {
    if (tid == 0) {
      *cnt = 0u;
      *dct = 0u;
      // rows without candidates: the refinement takes the window's subtiles
      // down to the lowest cut
      if (blockIdx.x == 0 && (topk <= 0 || first == 0)) cut_out[r] = kDomFloorLog2;
    }
    return;
  }
  const bool all_mode = n_counted <= topk;
  const float* stmax_row = stmax + static_cast<size_t>(r) * (Spad / kSubKeys) * kG;
  // ---- the first loads, together: histogram and the first round's maxima
  uint32_t hv[kNB / kThreads];
#pragma unroll
  for (int u = 0; u < kNB / kThreads; ++u)
    hv[u] = hist[static_cast<size_t>(r) * kNB + tid + kThreads * u];
  // no quad distances (qdiff null): every quad of a candidate is kept
  const bool use_quads = qdiff != nullptr;
  const unsigned char* qd_row = qdiff + (use_quads ? static_cast<size_t>(r) * (Spad / kSubKeys) * (4 * kG) : 0);
  f32x4 mx[2];
  u32x4 qd[2];   // quad q, head h: byte h % 4 of word 2 q + h / 4
  auto load_round = [&](int64_t st) {
    const bool ld = st < st1;
    mx[0] = ld ? *reinterpret_cast<const f32x4*>(stmax_row + st * kG) : f32x4{0.f, 0.f, 0.f, 0.f};
    mx[1] = ld ? *reinterpret_cast<const f32x4*>(stmax_row + st * kG + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u)
      qd[u] = ld && use_quads ? *reinterpret_cast<const u32x4*>(qd_row + st * (4 * kG) + 16 * u)
                              : u32x4{0u, 0u, 0u, 0u};
  };
  load_round(st0 + tid);
  if (tid < kG) lse2f[tid] = static_cast<float>(lse2[static_cast<size_t>(r) * kG + tid]);
  if (tid == 0) s_ybase = row_ybase(ytop_h, r);
#pragma unroll
  for (int u = 0; u < kNB / kThreads; ++u) lh[tid + kThreads * u] = hv[u];
  __syncthreads();
  if (tid < 64) {
    if (!all_mode) {
      const KthBin kb = kth_bin_wave(lh, static_cast<uint32_t>(topk));
      if (tid == 0) s_lo = max(0, kb.bstar - 1);
    }
  } else if (tid < 128) {   // the second wave, meanwhile
    const float cut = refine_cut_wave(lh, s_ybase, budget);
    if (tid == 64) s_cut = cut;
  }
  __syncthreads();
  const int lo_bin = all_mode ? 0 : s_lo;
  if (blockIdx.x == 0 && tid == 0) {
    lo_out[r] = lo_bin;
    cut_out[r] = s_cut;
  }
  const float ybase = s_ybase;
  const float cut = s_cut;
  float l2v[kG];
#pragma unroll
  for (int h = 0; h < kG; ++h) l2v[h] = lse2f[h];
  int32_t* out = clist + (static_cast<size_t>(r) * n_chunks + blockIdx.x) * chunk;
  int32_t* dout = dlist + (static_cast<size_t>(r) * n_chunks + blockIdx.x) * chunk;
  uint32_t written = 0, dwritten = 0;
  // a quad may hold a key the filter passes when, for some head, its bound
  // less lse2 reaches the bottom of the bin below lo_bin
  const float qthr = lo_bin - 1 <= 0 ? -INFINITY
                                     : ybase + static_cast<float>(lo_bin - 1) * (kYRange / kNB);
  for (int64_t sr0 = st0; sr0 < st1; sr0 += kThreads) {
    const int64_t st = sr0 + tid;
    if (sr0 != st0) load_round(st);
    bool cand = false, dom = false;
    uint32_t qmask = 0xFu;
    if (st < st1) {
      float ub = mx[0][0] - l2v[0];
      ub = fmaxf(ub, mx[0][1] - l2v[1]);
      ub = fmaxf(ub, mx[0][2] - l2v[2]);
      ub = fmaxf(ub, mx[0][3] - l2v[3]);
      ub = fmaxf(ub, mx[1][0] - l2v[4]);
      ub = fmaxf(ub, mx[1][1] - l2v[5]);
      ub = fmaxf(ub, mx[1][2] - l2v[6]);
      ub = fmaxf(ub, mx[1][3] - l2v[7]);
      cand = all_mode || st >= n_counted ||
             static_cast<int>(key_from_log2(ub, ybase) >> kBinShift) >= lo_bin;
      dom = ub >= cut;
      if (use_quads && cand && !all_mode && st < n_counted) {
        qmask = 0u;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          float qb = -INFINITY;
#pragma unroll
          for (int h = 0; h < kG; ++h) {
            const uint32_t word = qd[qq >> 1][2 * (qq & 1) + (h >> 2)];
            const float dq = static_cast<float>((word >> (8 * (h & 3))) & 0xFFu) *
                             (1.f / static_cast<float>(kQuadSteps));
            qb = fmaxf(qb, (mx[h >> 2][h & 3] - dq) - l2v[h]);
          }
          qmask |= static_cast<uint32_t>(qb >= qthr) << qq;
        }
      }
    }
    uint32_t o_list, o_dom;
    reserve_two(cand ? 1u : 0u, dom ? 1u : 0u, nullptr, nullptr, s_cnt, s_base, o_list, o_dom);
    if (cand)   // ascending: thread order
      out[written + o_list] = static_cast<int32_t>(st | (static_cast<int64_t>(qmask) << kQuadShift));
    if (dom) dout[dwritten + o_dom] = static_cast<int32_t>(st);
    written += s_base[2];
    dwritten += s_base[3];
  }
  if (tid == 0) {
    *cnt = written;
    *dct = dwritten;
  }
}

// The exact importance of the candidates' keys.  grid (NS, R): work-group w of
// a row takes the w-th equal share of the row's candidate list (the regions of
// the list kernel in order), so clustered candidates spread over all NS
// work-groups, in rounds of kScoreRound list entries:
//  * a wave takes a candidate subtile; its keys' importance (exact float64
//    for every key that can be kept, see below) is staged in LDS kStageSub
//    subtiles at a time;
//  * keys whose bin is below the row's lower bin can never be selected and
//    are dropped; the others are appended to the work-group's own region of
//    the row's candidate-key list in ascending key order, and counted in the
//    row's candidate histogram.  The region's length goes to cand_cnt.
// Each candidate subtile is first scored in float32 on the bf16 MFMA (16 keys
// against the 8 heads); only its keys that may reach the lower bin (float
// error is far below a bin) get the exact float64 importance, by plain fp64
// fmas over lanes (head, 16 dims).  Those keys' rows come from the MFMA
// operand registers through a small per-wave LDS slot, not from memory again,
// so the exact pass adds no memory round trip to the wave's chain.  Three
// work-groups fit a CU, and the grid is sized to be resident at once.
constexpr int kStageSub = 128;  // candidate subtiles staged per pass
static_assert(kStageSub / (kThreads / 64) <= 64, "a wave's subtiles of a pass fit one per lane");
__global__ __launch_bounds__(kThreads, 3) void subtile_score_kernel(
    const int32_t* __restrict__ lo_in, const int32_t* __restrict__ clist,
    const uint32_t* __restrict__ ccnt, const double* __restrict__ lse2,
    const RefinePart* __restrict__ ref_part, int ref_nparts, double* __restrict__ lse2r,
    float* __restrict__ lse_out, RefineStat* __restrict__ ref_stat,
    const float* __restrict__ ytop_h, uint32_t* __restrict__ hist_c, const u16* __restrict__ q,
    const u16* __restrict__ k, double* __restrict__ cand_y, int32_t* __restrict__ cand_idx,
    uint32_t* __restrict__ cand_cnt, int64_t S, int T, int Hkv, int topk, int w,
    int cc_chunk, int cc_nchunk, int chunk, int n_chunks, double c2, int64_t kvp) {
  __shared__ uint32_t lh[kNB];
  __shared__ uint32_t pre[kMaxChunks + 1];
  __shared__ int32_t s_list[kScoreRound];
  __shared__ double stage_y[kStageSub * kSubKeys];
  __shared__ u32x4 q_lds[2 * kG * kD / 8];   // 16 heads (8 real) x 128 dims, bf16
  __shared__ u32x4 k_slot[kThreads / 64][2][kD / 8];   // per wave: two key rows, bf16
  __shared__ float s_ybase;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  __shared__ double s_l2[kG];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  // wave index in a scalar register: the per-wave loops below are uniform
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int64_t first = row_first(row_pos(r, T, Hkv, S), w);
  uint32_t* cnt = cand_cnt + static_cast<size_t>(r) * n_chunks + blockIdx.x;
  // The refined lse2 that the keys are ranked with: lse2 + log2(1 + the
  // refinement's partial sums), in every work-group of the row (the same
  // arithmetic as the refinement's own finishing kernel); work-group 0 also
  // writes it, lse for the caller and the row's refinement statistics.
  {
    const RefinePart* pr = ref_part + static_cast<size_t>(r) * ref_nparts;
    for (int h = wave; h < kG; h += kThreads / 64) {
      const double c = refine_head_sum(pr, ref_nparts, h);
      if (lane == 0) s_l2[h] = lse2[static_cast<size_t>(r) * kG + h] + log1p(c) * M_LOG2E;
    }
    if (blockIdx.x == 0 && wave == 0) {
      uint32_t nd = 0, nb = 0;
      for (int i = lane; i < ref_nparts; i += 64) {
        nd += pr[i].n_dom;
        nb += pr[i].n_bad;
      }
      for (int off = 32; off > 0; off >>= 1) {
        nd += __shfl_xor(nd, off);
        nb += __shfl_xor(nb, off);
      }
      if (lane == 0) ref_stat[r] = RefineStat{nd, nb, 0u, 0u};
    }
    __syncthreads();
    if (blockIdx.x == 0 && tid < kG) {
      lse2r[static_cast<size_t>(r) * kG + tid] = s_l2[tid];
      if (lse_out) lse_out[static_cast<size_t>(r) * kG + tid] = static_cast<float>(s_l2[tid] * M_LN2);
    }
  }
  if (topk <= 0 || first == 0) {
    if (tid == 0) *cnt = 0u;
    return;
  }
  // ---- the row's list: region lengths, their exclusive prefix in pre
  constexpr int kPer = kMaxChunks / kThreads;
  uint32_t cl[kPer];
  uint32_t mysum = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = kPer * tid + u;
    cl[u] = c < cc_nchunk ? ccnt[static_cast<size_t>(r) * cc_nchunk + c] : 0u;
    mysum += cl[u];
  }
  // the query operand staged in LDS, packed bf16: lane (col, grp) of MFMA c
  // takes head col (zero for the padding heads), dims 32*grp + 8c .. +8
  for (int i = tid; i < 2 * kG * kD / 8; i += kThreads) {
    const int h = i / (kD / 8), d8 = i % (kD / 8);
    q_lds[i] = h < kG ? load_u32x4(q + (static_cast<size_t>(r) * kG + h) * kD + 8 * d8)
                      : u32x4{0u, 0u, 0u, 0u};
  }
  // float32 scale and the lse2 of heads 4 grp .. 4 grp + 3 for the filter; for
  // the exact pass lane (h, j) keeps head h's query dims 16 j .. +16 widened to
  // float64 and its lse2
  const float c2f = static_cast<float>(c2);
  float l2f[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) l2f[i] = 4 * grp + i < kG ? static_cast<float>(s_l2[4 * grp + i]) : 0.f;
  const double l2h = s_l2[lane >> 3];
  u32x4 qh2[2];   // packed bf16, widened at each use
  {
    const u16* qh = q + (static_cast<size_t>(r) * kG + (lane >> 3)) * kD + 16 * (lane & 7);
    qh2[0] = load_u32x4(qh);
    qh2[1] = load_u32x4(qh + 8);
  }
  const int lo_bin = lo_in[r];
  if (tid == 0) s_ybase = row_ybase(ytop_h, r);
  for (int i = tid; i < kNB; i += kThreads) lh[i] = 0u;   // the candidate histogram
  uint32_t off, dummy;
  reserve_two(mysum, 0u, nullptr, nullptr, s_cnt, s_base, off, dummy);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = kPer * tid + u;
    if (c < cc_nchunk) pre[c] = off;
    off += cl[u];
  }
  if (tid == 0) pre[cc_nchunk] = s_base[2];
  __syncthreads();
  const uint32_t n_c = pre[cc_nchunk];
  const uint32_t share = (n_c + n_chunks - 1) / n_chunks;
  const uint32_t p_begin = min(n_c, share * blockIdx.x);
  const uint32_t p_end = min(n_c, p_begin + share);
  const float ybase = s_ybase;
  // The float32 filter as one compare per head on the raw MFMA logit: a key
  // may reach the lower bin only if, for some head h, s2_h c2 - lse2_h is at
  // least the bottom of the bin below it (one bin of margin for the float
  // error), i.e. s2_h >= t_h = (that bound + lse2_h) / c2.  Lane (col, grp)
  // holds heads 4 grp .. 4 grp + 3 of key col; the padding heads never pass.
  float t4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    t4[i] = 4 * grp + i >= kG ? INFINITY
            : lo_bin - 1 <= 0 ? -INFINITY
                              : (ybase + static_cast<float>(lo_bin - 1) * (kYRange / kNB) + l2f[i]) / c2f;
  // lane (col, grp)'s part of a subtile: key col, dims 32 grp .. 32 grp + 31
  const uint32_t lane_off = static_cast<uint32_t>(col * kD + 32 * grp);
  const int b = r / (T * Hkv);
  const int g = r % Hkv;
  const u16* kr = k + (static_cast<size_t>(b) * Hkv + g) * static_cast<size_t>(kvp) * kD;
  const size_t region = (static_cast<size_t>(r) * n_chunks + blockIdx.x) * static_cast<size_t>(chunk) * kSubKeys;
  double* cy = cand_y + region;
  int32_t* ci = cand_idx + region;
  uint32_t written = 0;
  for (uint32_t pr0 = p_begin; pr0 < p_end; pr0 += kScoreRound) {
    const uint32_t n_local = min(static_cast<uint32_t>(kScoreRound), p_end - pr0);
    // ---- this round's candidate subtiles (list entry -> region of the list kernel)
    if (static_cast<uint32_t>(tid) < n_local) {
      const uint32_t pos = pr0 + tid;
      int lo = 0, hi = cc_nchunk - 1;   // the region of pos: largest c with pre[c] <= pos
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= pos) lo = mid;
        else hi = mid - 1;
      }
      s_list[tid] = clist[(static_cast<size_t>(r) * cc_nchunk + lo) * cc_chunk + (pos - pre[lo])];
    }
    __syncthreads();
    uint32_t o_dummy;
    for (uint32_t p0 = 0; p0 < n_local; p0 += kStageSub) {
      const uint32_t np = min(static_cast<uint32_t>(kStageSub), n_local - p0);
      // ---- float64 importance of the pass's candidates, one subtile per wave
      // list entry e: subtile e & kSubMask, its quad mask above kQuadShift.
      // The subtile's K rows (uniform base, fixed lane offsets); a subtile that
      // runs past the cache's rows reads the last row instead, and the lanes
      // of a masked quad read the head's row 0 (one cached row for all)
      auto load_sub = [&](int32_t e, u32x4 (&ka)[4]) {
        const int64_t key0 = static_cast<int64_t>(e & kSubMask) * kSubKeys;
        const bool use = ((static_cast<uint32_t>(e) >> (kQuadShift + (col >> 2))) & 1u) != 0u;
        if (key0 + kSubKeys <= kvp) {
          const u16* base = use ? kr + key0 * kD + lane_off : kr + 32 * grp;
#pragma unroll
          for (int c = 0; c < 4; ++c) ka[c] = load_u32x4(base + 8 * c);
        } else {
          const int64_t key = use ? min(key0 + col, kvp - 1) : 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) ka[c] = load_u32x4(kr + key * kD + 32 * grp + 8 * c);
        }
      };
      // the A operand (the query heads) in registers for the whole pass
      u32x4 qa[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) qa[c] = q_lds[(col * kD + 32 * grp + 8 * c) / 8];
      // Three register buffers per wave, used in turn, so that two subtiles
      // are always in flight behind the one being scored.  The loads are
      // unconditional (past the wave's last subtile they repeat it) and no
      // buffer is copied, so each wait is for the oldest buffer only.
      constexpr uint32_t kW = kThreads / 64;
      // pass entry i (this wave's entries i = wave + kW t) is subtile st
      auto score_sub = [&](uint32_t i, int32_t e, const u32x4 (&ka)[4]) {
        const int64_t key0 = static_cast<int64_t>(e & kSubMask) * kSubKeys;
        // ---- float32 logits of the 16 keys on the bf16 MFMA (Q . K^T, 16
        // heads of which 8 are used x 16 keys): lane (col, grp) gets heads
        // 4 grp + e against key col
        f32x4 sf = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sf = mfma_16x16x32(as_bf16x8(qa[c]),
                             as_bf16x8(ka[c]), sf);
        // keys that may reach the lower bin: key col passes in lane col
        // (heads 0..3) or lane 16 + col (heads 4..7)
        const uint64_t hit = __ballot(sf[0] >= t4[0] || sf[1] >= t4[1] || sf[2] >= t4[2] ||
                                      sf[3] >= t4[3]);
        uint32_t promising = static_cast<uint32_t>(hit | (hit >> 16)) & 0xFFFFu;
        // only the quads whose keys were loaded (the others cannot pass)
        const uint32_t qm = static_cast<uint32_t>(e) >> kQuadShift;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (!((qm >> qq) & 1u)) promising &= ~(0xFu << (4 * qq));
        // only keys before `first` are candidates
        const int64_t room = first - key0;
        if (room < kSubKeys) promising &= room <= 0 ? 0u : (1u << room) - 1u;
        // ---- exact float64 importance of the promising keys only, two at a
        // time: lane (h, j) = (lane >> 3, lane & 7) takes head h, dims 16 j .. +16.
        // Key e's row sits in the MFMA operand of lanes (col = e, grp = 0..3),
        // 32 dims each; those lanes copy it to the wave's LDS slot.
        if (lane < kSubKeys) stage_y[i * kSubKeys + lane] = -INFINITY;
        for (uint32_t m = promising; m; ) {
          int ek[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            ek[u] = m ? __builtin_ctz(m) : -1;
            if (m) m &= m - 1;
            if (col == ek[u]) {
#pragma unroll
              for (int c = 0; c < 4; ++c) k_slot[wave][u][4 * grp + c] = ka[c];
            }
          }
          lds_fence_wave();   // the slot's writes land before any lane reads them
          u32x4 kv4[2][2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            kv4[u][0] = k_slot[wave][u][2 * (lane & 7)];
            kv4[u][1] = k_slot[wave][u][2 * (lane & 7) + 1];
          }
          lds_fence_wave();   // and are read before the next pair overwrites them
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (ek[u] < 0) continue;
            double acc = 0.0;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
              const uint32_t word = kv4[u][t >> 3][(t >> 1) & 3];
              const double kvd = static_cast<double>(
                  __uint_as_float((t & 1) ? (word & 0xFFFF0000u) : (word << 16)));
              const uint32_t qw = qh2[t >> 3][(t >> 1) & 3];
              const double qvd = static_cast<double>(
                  __uint_as_float((t & 1) ? (qw & 0xFFFF0000u) : (qw << 16)));
              acc = fma(qvd, kvd, acc);
            }
            acc = oct_sum(acc);
            double yy = c2 * acc - l2h;
            yy = fmax(yy, dpp_mov_f64<0x140>(yy));   // the row's other head
            yy = max_over_rows_f64(yy);
            if (lane == 0) stage_y[i * kSubKeys + ek[u]] = yy;
          }
        }
      };
      // (the scheduling barriers keep the loads in program order: the oldest
      // buffer is the one scored next).  The wave's subtile numbers for the
      // pass sit one per lane, read out with a scalar lane read.
      if (static_cast<uint32_t>(wave) < np) {
        const uint32_t n_w = (np - 1 - wave) / kW + 1;   // <= kStageSub / kW <= 64
        const int32_t my_sub = static_cast<uint32_t>(lane) < n_w ? s_list[p0 + wave + kW * lane] : 0;
        auto sub_at = [&](uint32_t t) {
          return static_cast<int32_t>(lane_value(static_cast<uint32_t>(my_sub), static_cast<int>(min(t, n_w - 1))));
        };
        u32x4 kb0[4], kb1[4], kb2[4];
        load_sub(sub_at(0), kb0);
        __builtin_amdgcn_sched_barrier(0);
        load_sub(sub_at(1), kb1);
        __builtin_amdgcn_sched_barrier(0);
        // (no early exit from the trip: an exit path that leaves a buffer in
        // flight would make every trip wait for it)
        for (uint32_t t = 0; t < n_w; t += 3) {
          load_sub(sub_at(t + 2), kb2);
          __builtin_amdgcn_sched_barrier(0);
          score_sub(wave + kW * t, sub_at(t), kb0);
          load_sub(sub_at(t + 3), kb0);
          __builtin_amdgcn_sched_barrier(0);
          if (t + 1 < n_w) score_sub(wave + kW * (t + 1), sub_at(t + 1), kb1);
          load_sub(sub_at(t + 4), kb1);
          __builtin_amdgcn_sched_barrier(0);
          if (t + 2 < n_w) score_sub(wave + kW * (t + 2), sub_at(t + 2), kb2);
        }
      }
      // the prefetches past the end are never used: drain them here, once,
      // so that no wait for them lands inside the next pass's loop
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      __syncthreads();
      // ---- keep the keys that can still be selected, in order (thread t:
      // the 16 keys of the pass's t-th candidate subtile)
      uint32_t keep = 0;
      int64_t key0 = 0;
      if (static_cast<uint32_t>(tid) < np) {
        key0 = static_cast<int64_t>(s_list[p0 + tid] & kSubMask) * kSubKeys;
#pragma unroll
        for (int e = 0; e < kSubKeys; ++e) {
          const double yy = stage_y[tid * kSubKeys + e];
          const bool ok = key0 + e < first && cand_bin(yy, ybase) >= lo_bin;
          keep |= static_cast<uint32_t>(ok) << e;
        }
      }
      uint32_t o_keep;
      reserve_two(__popc(keep), 0u, nullptr, nullptr, s_cnt, s_base, o_keep, o_dummy);
      o_keep += written;
      written += s_base[2];
      for (uint32_t m = keep; m; m &= m - 1) {
        const int e = __builtin_ctz(m);
        const double yy = stage_y[tid * kSubKeys + e];
        cy[o_keep] = yy;
        ci[o_keep] = static_cast<int32_t>(key0 + e);
        atomicAdd(&lh[cand_bin(yy, ybase)], 1u);
        ++o_keep;
      }
      __syncthreads();   // stage_y is reused by the next pass
    }
  }
  for (int i = tid; i < kNB; i += kThreads)
    if (lh[i]) atomicAdd(&hist_c[static_cast<size_t>(r) * kNB + i], lh[i]);
  if (tid == 0) *cnt = written;
}


// ---- the row's exact top-k from its candidate list, one work-group per row.
//
// The list holds, in ascending key index, every key that can be selected with
// its exact importance.  Bins above the k-th bin b* of the row's candidate
// histogram are selected.  In b* (the band) a radix select over the 64-bit
// importance finds the threshold T: entries above T are selected, and of the
// entries equal to T the first ones in list order (the lowest indices) make up
// the count.  One more pass writes the selected indices in list order, i.e.
// ascending.  Each thread owns kPerThr consecutive list entries per sweep of
// the list; the first sweep stays in registers.

constexpr int kSelThreads = 1024;
constexpr int kPerThr = 2;
constexpr int kSweep = kSelThreads * kPerThr;
static_assert(kNB % kSelThreads == 0, "whole histogram rows per thread");
constexpr int kSmallBand = 64;   // bands up to this size are ranked by one wave

struct SelEntry {
  double y[kPerThr];
  int32_t j[kPerThr];
  int n;   // entries held (0..kPerThr)
};

// Load list positions [p0, p0 + kPerThr) ∩ [0, n_total) into e.
__device__ __forceinline__ void load_entries(SelEntry& e, const double* __restrict__ cy,
                                             const int32_t* __restrict__ ci, const uint32_t* pre,
                                             int n_chunks, size_t chunk_len, uint32_t p0,
                                             uint32_t n_total) {
  e.n = p0 < n_total ? static_cast<int>(min(static_cast<uint32_t>(kPerThr), n_total - p0)) : 0;
  size_t at[kPerThr];
  if (e.n > 0) {
    int lo = 0, hi = n_chunks - 1;   // the chunk of p0: the largest c with pre[c] <= p0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= p0) lo = mid;
      else hi = mid - 1;
    }
    int c = lo;
    uint32_t o = p0 - pre[c];
#pragma unroll
    for (int u = 0; u < kPerThr; ++u) {
      if (u < e.n) {
        while (o >= pre[c + 1] - pre[c]) {
          ++c;
          o = 0;
        }
        at[u] = static_cast<size_t>(c) * chunk_len + o;
        ++o;
      } else {
        at[u] = u > 0 ? at[0] : 0;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kPerThr; ++u) {
    e.y[u] = u < e.n ? cy[at[u]] : -INFINITY;
    e.j[u] = u < e.n ? ci[at[u]] : -1;
  }
}

__global__ __launch_bounds__(kSelThreads) void row_select_kernel(
    const uint32_t* __restrict__ hist_c, const double* __restrict__ cand_y,
    const int32_t* __restrict__ cand_idx, const uint32_t* __restrict__ cand_cnt,
    const float* __restrict__ ytop_h, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ nsel_out, int64_t S, int T, int Hkv, int topk, int w, int cap,
    int chunk, int n_chunks) {
  __shared__ uint32_t lh[kNB];
  __shared__ uint32_t pre[kMaxChunks + 1];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_red[4];
  __shared__ uint64_t s_hi;
  __shared__ uint32_t s_need;
  __shared__ int s_done;
  __shared__ int s_b;
  __shared__ uint32_t s_above, s_at;
  __shared__ float s_ybase;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  __shared__ uint64_t s_bkey[kSmallBand];
  __shared__ uint32_t s_bpos[kSmallBand];
  __shared__ uint32_t s_nb;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = row_first(P, w);
  int32_t* out = idx_out + static_cast<size_t>(r) * cap;
  uint32_t n_keep = 0;
  if (topk > 0 && first > 0) {
    // ---- histogram and chunk lengths (exclusive prefix in pre); all of the
    // loads are issued before the first wait
    constexpr int kHv = kNB / kSelThreads;
    uint32_t hv[kHv];
#pragma unroll
    for (int u = 0; u < kHv; ++u) hv[u] = hist_c[static_cast<size_t>(r) * kNB + tid + u * kSelThreads];
    constexpr int kPer = kMaxChunks / kSelThreads;
    uint32_t cl[kPer];
    uint32_t mysum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = kPer * tid + u;
      cl[u] = c < n_chunks ? cand_cnt[static_cast<size_t>(r) * n_chunks + c] : 0u;
      mysum += cl[u];
    }
    if (tid == 0) s_ybase = row_ybase(ytop_h, r);
#pragma unroll
    for (int u = 0; u < kHv; ++u) lh[tid + u * kSelThreads] = hv[u];
    uint32_t off, dummy;
    reserve_two(mysum, 0u, nullptr, nullptr, s_cnt, s_base, off, dummy);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = kPer * tid + u;
      if (c < n_chunks) pre[c] = off;
      off += cl[u];
    }
    if (tid == 0) pre[n_chunks] = s_base[2];
    // the band's first radix round starts from cleared reductions
    if (tid < 4) s_red[tid] = tid < 2 ? 0xFFFFFFFFu : 0u;
    if (tid < 256) h256[tid] = 0u;
    if (tid == 0) s_nb = 0u;
    __syncthreads();
    // the list's first sweep is loaded while wave 0 finds the k-th bin
    const uint32_t n_total = pre[n_chunks];
    const size_t chunk_len = static_cast<size_t>(chunk) * kSubKeys;
    const size_t rbase = static_cast<size_t>(r) * n_chunks * chunk_len;
    const double* cy = cand_y + rbase;
    const int32_t* ci = cand_idx + rbase;
    const int n_sweeps = static_cast<int>((n_total + kSweep - 1) / kSweep);
    SelEntry e0;
    load_entries(e0, cy, ci, pre, n_chunks, chunk_len, kPerThr * tid, n_total);
    if (tid < 64) {
      const KthBin kb = kth_bin_wave(lh, static_cast<uint32_t>(topk));
      if (tid == 0) {
        s_b = kb.found ? kb.bstar : -1;
        s_above = kb.above;
        s_at = kb.at;
      }
    }
    __syncthreads();
    const int bstar = s_b;
    const float ybase = s_ybase;
    const bool all = bstar < 0;
    const uint32_t take = all ? 0u : static_cast<uint32_t>(topk) - s_above;
    const uint32_t n_band = all ? 0u : s_at;
    // sweep sw of the list as registers
    auto sweep = [&](int sw, SelEntry& e) {
      if (sw == 0) e = e0;
      else load_entries(e, cy, ci, pre, n_chunks, chunk_len, sw * kSweep + kPerThr * tid, n_total);
    };
    auto in_band = [&](const SelEntry& e, int u) {
      return u < e.n && cand_bin(e.y[u], ybase) == bstar;
    };
    // ---- threshold T of the band's importance (radix over the 64-bit key)
    uint64_t thr = 0;
    uint32_t nd_t = 0;      // entries equal to T taken, in list order
    bool incl = true;       // true: every band entry >= thr is taken
    if (!all && take < n_band && n_band <= kSmallBand) {
      // ---- a small band: its entries (key, list position) go to LDS and
      // wave 0 ranks them directly, larger key first and then lower position;
      // the best `take` are selected.  T is the key of the last one taken and
      // nd_t the taken entries equal to T, which are the first ties in list
      // order because the rank orders ties by position.
      for (int sw = 0; sw < n_sweeps; ++sw) {
        SelEntry e;
        sweep(sw, e);
#pragma unroll
        for (int u = 0; u < kPerThr; ++u) {
          if (!in_band(e, u)) continue;
          const uint32_t slot = atomicAdd(&s_nb, 1u);   // < n_band: the band's own count
          if (slot < static_cast<uint32_t>(kSmallBand)) {
            s_bkey[slot] = ordered_u64(e.y[u]);
            s_bpos[slot] = static_cast<uint32_t>(sw * kSweep + kPerThr * tid + u);
          }
        }
      }
      __syncthreads();
      if (tid < 64) {
        const bool have = static_cast<uint32_t>(lane) < n_band;
        const uint64_t kh = have ? s_bkey[lane] : 0ull;
        const uint32_t ph = have ? s_bpos[lane] : ~0u;
        uint32_t rank = 0;
        for (int j = 0; j < static_cast<int>(n_band); ++j) {
          const uint64_t kj = lane_value64(kh, j);
          const uint32_t pj = lane_value(ph, j);
          rank += (kj > kh || (kj == kh && pj < ph)) ? 1u : 0u;
        }
        const uint64_t last = __ballot(have && rank == take - 1);
        const uint64_t t_key = lane_value64(kh, last ? __builtin_ctzll(last) : 0);
        const uint64_t eq = __ballot(have && rank < take && kh == t_key);
        if (lane == 0) {
          s_hi = t_key;
          s_need = static_cast<uint32_t>(__popcll(eq));
        }
      }
      __syncthreads();
      thr = s_hi;
      nd_t = s_need;
      incl = false;
    } else if (!all && take < n_band) {
      // Each round: AND/OR of the keys in play -> barrier -> histogram of the
      // first digit where they differ -> barrier -> wave 0 picks the digit and
      // clears s_red / h256 for the next round -> barrier.  Every thread reads
      // s_red between the first two barriers and the round's result after the
      // third, so those single buffers are never rewritten while being read.
      uint64_t mask = 0;
      uint32_t nd = take;
      while (true) {
        uint32_t a0 = ~0u, a1 = ~0u, o0 = 0u, o1 = 0u;
        for (int sw = 0; sw < n_sweeps; ++sw) {
          SelEntry e;
          sweep(sw, e);
#pragma unroll
          for (int u = 0; u < kPerThr; ++u) {
            if (!in_band(e, u)) continue;
            const uint64_t kh = ordered_u64(e.y[u]);
            if ((kh & mask) != thr) continue;
            a0 &= static_cast<uint32_t>(kh >> 32);
            a1 &= static_cast<uint32_t>(kh);
            o0 |= static_cast<uint32_t>(kh >> 32);
            o1 |= static_cast<uint32_t>(kh);
          }
        }
        a0 = wave_and(a0);
        a1 = wave_and(a1);
        o0 = wave_or(o0);
        o1 = wave_or(o1);
        if (lane == 0) {
          atomicAnd(&s_red[0], a0);
          atomicAnd(&s_red[1], a1);
          atomicOr(&s_red[2], o0);
          atomicOr(&s_red[3], o1);
        }
        __syncthreads();
        const uint64_t and_k = (static_cast<uint64_t>(s_red[0]) << 32) | s_red[1];
        const uint64_t or_k = (static_cast<uint64_t>(s_red[2]) << 32) | s_red[3];
        const uint64_t diff = and_k ^ or_k;
        if (diff == 0) {
          // every entry still in play has the same importance: T, taken in order
          thr = and_k;
          nd_t = nd;
          incl = false;
          break;
        }
        const int d = __clzll(static_cast<long long>(diff)) / 8;   // first digit that differs
        mask = d == 0 ? 0ull : ~0ull << (64 - 8 * d);
        thr = and_k & mask;
        for (int sw = 0; sw < n_sweeps; ++sw) {
          SelEntry e;
          sweep(sw, e);
#pragma unroll
          for (int u = 0; u < kPerThr; ++u) {
            bool act = false;
            uint32_t dig = 0;
            if (in_band(e, u)) {
              const uint64_t kh = ordered_u64(e.y[u]);
              act = (kh & mask) == thr;
              dig = static_cast<uint32_t>(kh >> (56 - 8 * d)) & 255u;
            }
            const uint64_t m_act = __ballot(act);
            if (m_act) {
              const int leader = __builtin_ctzll(m_act);
              const uint32_t d0 = lane_value(dig, leader);
              if (__ballot(act && dig == d0) == m_act) {
                if (lane == leader) atomicAdd(&h256[d0], static_cast<uint32_t>(__popcll(m_act)));
              } else if (act) {
                atomicAdd(&h256[dig], 1u);
              }
            }
          }
        }
        __syncthreads();
        if (tid < 64) {
          // lane l holds bins 255-4l .. 252-4l; counts from the top
          uint32_t c4[4];
          uint32_t sum = 0;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            c4[u] = h256[255 - 4 * lane - u];
            sum += c4[u];
          }
          const uint32_t inc = wave_incl_scan(sum);
          const uint64_t hit = __ballot(inc >= nd);
          const int owner = hit ? __builtin_ctzll(hit) : 63;   // nd <= entries in play
          if (lane == owner) {
            uint32_t above = inc - sum;
            int u = 0;
            for (; u < 3; ++u) {
              if (above + c4[u] >= nd) break;
              above += c4[u];
            }
            const uint32_t left = nd - above;
            s_need = left;
            s_done = c4[u] == left;
            s_hi = thr | (static_cast<uint64_t>(255 - 4 * lane - u) << (56 - 8 * d));
          }
          // the next round's reductions start from cleared buffers (this
          // lane's reads of h256 above come first)
#pragma unroll
          for (int u = 0; u < 4; ++u) h256[255 - 4 * lane - u] = 0u;
          if (lane < 4) s_red[lane] = lane < 2 ? 0xFFFFFFFFu : 0u;
        }
        __syncthreads();
        nd = s_need;
        thr = s_hi;
        mask |= 255ull << (56 - 8 * d);
        if (s_done) break;   // every remaining entry of the bin is taken
      }
    }
    // ---- the selection in list order
    auto pick = [&](const SelEntry& e, int u, uint32_t& sel, uint32_t& tie) {
      sel = 0;
      tie = 0;
      if (u >= e.n) return;
      if (all) {
        sel = 1;
        return;
      }
      const int bn = cand_bin(e.y[u], ybase);
      if (bn != bstar) {
        sel = bn > bstar;
        return;
      }
      if (take >= n_band) {
        sel = 1;
        return;
      }
      const uint64_t kh = ordered_u64(e.y[u]);
      if (kh > thr || (incl && kh == thr)) sel = 1;
      else if (kh == thr) tie = 1;
    };
    // output position of an entry = selected entries before it + kept ties
    // before it, where the kept ties are the first nd_t ties: one block scan
    // of both counts gives both prefixes
    uint32_t sel_seen = 0, tie_seen = 0;
    for (int sw = 0; sw < n_sweeps; ++sw) {
      SelEntry e;
      sweep(sw, e);
      uint32_t ns = 0, nt = 0;
#pragma unroll
      for (int u = 0; u < kPerThr; ++u) {
        uint32_t sl, tl;
        pick(e, u, sl, tl);
        ns += sl;
        nt += tl;
      }
      uint32_t o_sel, o_tie;
      reserve_two(ns, nt, nullptr, nullptr, s_cnt, s_base, o_sel, o_tie);
      o_sel += sel_seen;
      o_tie += tie_seen;
      sel_seen += s_base[2];
      tie_seen += s_base[3];
#pragma unroll
      for (int u = 0; u < kPerThr; ++u) {
        uint32_t sl, tl;
        pick(e, u, sl, tl);
        if (sl) {
          const uint32_t at = o_sel + min(o_tie, nd_t);
          if (at < static_cast<uint32_t>(cap)) out[at] = e.j[u];
          ++o_sel;
        } else if (tl) {
          if (o_tie < nd_t && o_sel + o_tie < static_cast<uint32_t>(cap)) out[o_sel + o_tie] = e.j[u];
          ++o_tie;
        }
      }
    }
    const uint32_t written = sel_seen + min(tie_seen, nd_t);
    n_keep = min(written, static_cast<uint32_t>(topk));
  }
  // no barrier: the selection filled positions [0, n_keep) (exactly top-k of
  // them, or the whole list when it is shorter), the tail below starts at
  // n_keep, and n_keep is the same in every thread
  const int n_total_sel = static_cast<int>(n_keep) + static_cast<int>(static_cast<int64_t>(P) - first + 1);
  for (int i = static_cast<int>(n_keep) + tid; i < cap; i += kSelThreads)
    out[i] = i < n_total_sel ? static_cast<int32_t>(first + (i - static_cast<int>(n_keep))) : -1;
  if (tid == 0) nsel_out[r] = min(n_total_sel, cap);
}

// ================================================================ prefill chunk

// The threshold T of the best `need` of n 64-bit keys (larger is better): the
// keys above T are taken, and of the keys equal to T the first nd_t in array
// order (or, when incl, every key >= T).  MSB radix select in 8-bit digits:
// each round first finds the highest bit where the keys still in play differ
// (the bits they share are fixed at once, which skips exact ties), then takes
// a 256-bin histogram of that digit; it stops as soon as every remaining key
// of the chosen bin is needed.  keys: any memory, read several times.  All
// threads call it (blockDim a multiple of 64, >= 256); 1 <= need <= n.
struct KThr {
  uint64_t thr;
  uint32_t nd_t;
  bool incl;
};
__device__ __forceinline__ KThr key_threshold(const uint64_t* keys, uint32_t n, uint32_t need, uint32_t* h256,
                              uint32_t* s_red, uint64_t* s_hi, uint32_t* s_need, int* s_done) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  uint64_t thr = 0, mask = 0;
  uint32_t nd = need;
  while (true) {
    if (tid < 4) s_red[tid] = tid < 2 ? 0xFFFFFFFFu : 0u;
    __syncthreads();
    uint32_t a0 = ~0u, a1 = ~0u, o0 = 0u, o1 = 0u;
    for (uint32_t base = 0; base < n; base += blockDim.x) {
      const uint32_t i = base + tid;
      if (i < n) {
        const uint64_t kh = keys[i];
        if ((kh & mask) == thr) {
          a0 &= static_cast<uint32_t>(kh >> 32);
          a1 &= static_cast<uint32_t>(kh);
          o0 |= static_cast<uint32_t>(kh >> 32);
          o1 |= static_cast<uint32_t>(kh);
        }
      }
    }
    a0 = wave_and(a0);
    a1 = wave_and(a1);
    o0 = wave_or(o0);
    o1 = wave_or(o1);
    if (lane == 0) {
      atomicAnd(&s_red[0], a0);
      atomicAnd(&s_red[1], a1);
      atomicOr(&s_red[2], o0);
      atomicOr(&s_red[3], o1);
    }
    __syncthreads();
    const uint64_t and_k = (static_cast<uint64_t>(s_red[0]) << 32) | s_red[1];
    const uint64_t or_k = (static_cast<uint64_t>(s_red[2]) << 32) | s_red[3];
    const uint64_t diff = and_k ^ or_k;
    if (diff == 0) {
      __syncthreads();
      return KThr{and_k, nd, false};   // all keys in play equal: take the first nd
    }
    const int d = __clzll(static_cast<long long>(diff)) / 8;
    mask = d == 0 ? 0ull : ~0ull << (64 - 8 * d);
    thr = and_k & mask;
    if (tid < 256) h256[tid] = 0u;
    __syncthreads();
    for (uint32_t base = 0; base < n; base += blockDim.x) {
      const uint32_t i = base + tid;
      bool act = false;
      uint32_t dig = 0;
      if (i < n) {
        const uint64_t kh = keys[i];
        act = (kh & mask) == thr;
        dig = static_cast<uint32_t>(kh >> (56 - 8 * d)) & 255u;
      }
      const uint64_t m_act = __ballot(act);
      if (m_act) {
        const int leader = __builtin_ctzll(m_act);
        const uint32_t d0 = lane_value(dig, leader);
        if (__ballot(act && dig == d0) == m_act) {
          if (lane == leader) atomicAdd(&h256[d0], static_cast<uint32_t>(__popcll(m_act)));
        } else if (act) {
          atomicAdd(&h256[dig], 1u);
        }
      }
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t c4[4];
      uint32_t sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c4[u] = h256[255 - 4 * lane - u];
        sum += c4[u];
      }
      const uint32_t inc = wave_incl_scan(sum);
      const uint64_t hit = __ballot(inc >= nd);
      const int owner = hit ? __builtin_ctzll(hit) : 63;
      if (lane == owner) {
        uint32_t above = inc - sum;
        int u = 0;
        for (; u < 3; ++u) {
          if (above + c4[u] >= nd) break;
          above += c4[u];
        }
        const uint32_t left = nd - above;
        *s_need = left;
        *s_done = c4[u] == left;
        *s_hi = thr | (static_cast<uint64_t>(255 - 4 * lane - u) << (56 - 8 * d));
      }
    }
    __syncthreads();
    nd = *s_need;
    thr = *s_hi;
    mask |= 255ull << (56 - 8 * d);
    const bool done = *s_done != 0;
    __syncthreads();
    if (done) return KThr{thr, 0u, true};
  }
}

// Number of entries of the ascending array a[0..n) that are < v.
__device__ __forceinline__ uint32_t lower_bound_lds(const int32_t* a, uint32_t n, int32_t v) {
  uint32_t lo = 0, hi = n;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Rank a band of n_band keyed entries (bk[i] the key, bi[i] its payload, the
// entries in ascending payload order) and write the payloads of the best
// `take`, ascending, to win (at most win_cap of them); ties go to the earlier
// entry.  Returns how many won.  The band is only read.  All kRowThreads
// threads call it.
__device__ __forceinline__ uint32_t rank_band(const uint64_t* bk, const int32_t* bi, uint32_t n_band,
                              uint32_t take, int32_t* win, uint32_t win_cap, uint32_t* s_count,
                              uint32_t* h256, uint32_t* s_red, uint64_t* s_hi, uint32_t* s_need,
                              int* s_done, uint32_t (*s_cnt)[16], uint32_t* s_base) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (n_band <= 64) {
    // a small band: wave 0 ranks it directly.  Lane i holds entry i; its rank
    // counts the entries with a larger key, or an equal key and a lower
    // position; the best `take` win
    if (wave == 0) {
      const bool have = static_cast<uint32_t>(lane) < n_band;
      const uint64_t kh = have ? bk[lane] : 0ull;
      uint32_t rank = 0;
      for (int j = 0; j < static_cast<int>(n_band); ++j) {
        const uint64_t kj = lane_value64(kh, j);
        rank += (kj > kh || (kj == kh && j < lane)) ? 1u : 0u;
      }
      const bool won = have && rank < take;
      const uint64_t bal = __ballot(won);
      if (won) win[__popcll(bal & ((1ull << lane) - 1ull))] = bi[lane];
      if (lane == 0) *s_count = static_cast<uint32_t>(__popcll(bal));
    }
    __syncthreads();
    return *s_count;
  }
  // the band's share: all of it, or the best `take` by threshold
  KThr kt{0ull, 0u, true};
  const bool by_thr = take < n_band;
  if (by_thr && take > 0) kt = key_threshold(bk, n_band, take, h256, s_red, s_hi, s_need, s_done);
  // winners in band order, ties: the first kt.nd_t
  const uint32_t per = (n_band + kRowThreads - 1) / kRowThreads;
  const uint32_t q0 = min(n_band, tid * per), q1 = min(n_band, q0 + per);
  // class of entry i: 1 a winner, 2 a tie at the threshold, 0 out
  auto cls = [&](uint32_t i) -> uint32_t {
    if (!by_thr) return 1u;
    if (take == 0) return 0u;
    const uint64_t kh = bk[i];
    if (kh > kt.thr || (kt.incl && kh == kt.thr)) return 1u;
    return kh == kt.thr ? 2u : 0u;
  };
  uint32_t nwin = 0, ntie = 0;
  for (uint32_t i = q0; i < q1; ++i) {
    const uint32_t c = cls(i);
    nwin += c == 1u;
    ntie += c == 2u;
  }
  uint32_t o_tie, o_dummy;
  reserve_two(ntie, 0u, nullptr, nullptr, s_cnt, s_base, o_tie, o_dummy);
  uint32_t keep_tie = 0;
  for (uint32_t i = q0, ot = o_tie; i < q1; ++i)
    if (cls(i) == 2u) keep_tie += (ot++ < kt.nd_t);
  uint32_t o_w;
  reserve_two(nwin + keep_tie, 0u, nullptr, nullptr, s_cnt, s_base, o_w, o_dummy);
  const uint32_t n_w = s_base[2];
  for (uint32_t i = q0, ot = o_tie; i < q1; ++i) {
    const uint32_t c = cls(i);
    bool a = c == 1u;
    if (c == 2u) a = (ot++ < kt.nd_t);
    if (a) {
      if (o_w < win_cap) win[o_w] = bi[i];
      ++o_w;
    }
  }
  return n_w;
}

// One work-group per row (b, t, g) of a prefill chunk: the exact top-k of the
// row's older keys from their stored log2 importance v (16-bit fixed point,
// 2^-10 octave steps; bin = v >> 7 is an eighth of an octave).
//  * One pass over v, in rounds of 16 values per thread, keeps the row's
//    histogram of bins only at or above floor, the k-th largest bin of the
//    values seen so far: a subset's k-th largest never exceeds the whole
//    row's, so every bin at or above the row's k-th bin is counted exactly and
//    most values cost no atomic.  The values within reach of the band (below)
//    are listed in LDS (index and v), in key order.
//  * The k-th bin b* of the finished histogram and a 128-bucket count of the
//    listed values in b* give c, the k-th largest v exactly.
//  * E bounds twice the difference between a stored v and the exact float64
//    importance (the fixed-point rounding plus the float32 error of the
//    importance pass, from the largest |k| of the head and the row's |q|).
//    Keys with v > c + E are selected, keys with v < c - E are not, and the
//    band [c - E, c + E] is re-ranked on its importance recomputed in float64
//    from exact bf16 products: a radix threshold picks the band's share, ties
//    going to the lower index (the band list is in index order).
//  * The up list and the band winners, both ascending, are merged into the
//    output by rank; then the window, the padding and the count.
// A list longer than LDS holds is replaced by a second pass over v, with the
// band widened to [first value of b* - E, last value of b* + E]; a band larger
// than band_cap is ranked by v itself.
// Block-level selection (kBlocks, blocks of bs tokens) takes the same steps on
// the blocks' values, each the largest stored value of its tokens: one pass
// writes them (and their histogram) to LDS, c is the n_take-th largest, blocks
// above c + E are taken, and each band block's exact importance is the largest
// float64 importance of its tokens stored at or above (its value) - E, the only
// ones that can hold it.  The band is ranked exactly whatever its size (the
// plan gives every row a band list of one entry per block).
constexpr int kMaxBlocks = 16384;   // blocks per row (block-level selection)
constexpr int kMaxSelBlocks = kMaxSel / 16;   // blocks taken per row: top_k / block, block >= 16
constexpr int kPList = 4 * kUncCap;   // listed values per row held in LDS
constexpr int kPListPer = kPList / kRowThreads;
constexpr int kVBinShift = 16 - 9;    // v >> 7: the kPNB = 512 bins
static_assert(kPList % kRowThreads == 0, "list split evenly over the threads");
static_assert(2 * kMaxSel >= kPList, "the list's values fit in the up list's space");
static_assert(kPList >= 3 * kUncCap, "the band's keys and indices fit in the list's space");
static_assert(kPNB == 1 << (16 - kVBinShift), "bins are the top bits of v");

__device__ __forceinline__ uint32_t u16_at(const u32x4 (&v)[2], int e) {
  const uint32_t word = v[e >> 3][(e >> 1) & 3];
  return (e & 1) ? (word >> 16) : (word & 0xFFFFu);
}

template <bool kBlocks>
__global__ __launch_bounds__(kRowThreads, 2) void prefill_select_kernel(
    const u16* __restrict__ ybuf, const uint32_t* __restrict__ kmax, int n_ib,
    const double* __restrict__ lse2, double* __restrict__ lse2r, float* __restrict__ lse_out,
    const float* __restrict__ ytop_h, int32_t* __restrict__ dom_list, RefineStat* __restrict__ stat,
    const u16* __restrict__ q, const u16* __restrict__ k, int32_t* __restrict__ band_idx,
    uint64_t* __restrict__ band_key, int64_t band_cap, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ nsel_out, int64_t S, int64_t Spad, int T, int Hkv, int topk, int w,
    int cap, int bs, double c2, float c2_hi, float c2_lo, bool split_logits, int64_t kvp) {
  static_assert(kMaxBlocks * sizeof(uint16_t) <= kPList * sizeof(uint32_t), "block maxima fit the list");
  static_assert(3 * (kMaxSel / 4) + 2 * kMaxSelBlocks <= kMaxSel, "block lists fit bw");
  __shared__ __align__(16) int32_t up[kMaxSel];
  __shared__ __align__(16) int32_t bw[kMaxSel];        // band winners; first the histogram
  // the list's indices; after the split, the band (keys, then indices); the
  // list's values sit in the up list's space until the split
  __shared__ __align__(16) uint32_t pool[kPList];
  __shared__ double qd[kG * kD];
  __shared__ double l2s[kG];
  __shared__ double s_dl2[kG];
  __shared__ unsigned long long s_corr[kG];   // each head's refinement, fixed point 2^-60
  __shared__ uint32_t s_ndom;
  __shared__ float s_qn[2][kRowThreads / 64];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_red[4];
  __shared__ uint64_t s_hi;
  __shared__ uint32_t s_need, s_count, s_tlo;
  __shared__ uint64_t s_thi;
  __shared__ int s_done;
  __shared__ int s_b, s_floor, s_c, s_E;
  __shared__ uint32_t s_km;
  __shared__ uint32_t s_off[2][2][kRowThreads / 64];
  __shared__ uint32_t s_above;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  uint32_t* lh = reinterpret_cast<uint32_t*>(bw);
  uint16_t* lval = reinterpret_cast<uint16_t*>(up);
  int32_t* lidx = reinterpret_cast<int32_t*>(pool);
  uint64_t* lbk = reinterpret_cast<uint64_t*>(pool);
  int32_t* lbi = reinterpret_cast<int32_t*>(pool + 2 * kUncCap);
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = row_first(P, w);
  const int b = r / (T * Hkv);
  const int g = r % Hkv;
  int32_t* out = idx_out + static_cast<size_t>(r) * cap;
  const u16* qr = q + static_cast<size_t>(r) * kG * kD;
  const u16* kr = k + (static_cast<size_t>(b) * Hkv + g) * static_cast<size_t>(kvp) * kD;
  const u16* yr = ybuf + static_cast<size_t>(r) * Spad;
  // ---- refinement of lse2 over the row's dominant keys: those that some head
  // gives 2^kDomLog2 of its weight or more, found from the stored importance
  // (the pass below lists the older ones, refine_row the window's).  The
  // attention kernel summed 2^(a c2_hi - m) for each key, a the float32 MFMA
  // logit; each listed key's term is replaced by the one of its float64 logit
  // from exact bf16 products.  a is recomputed by the attention kernel's MFMA
  // sequence on the same operands (same bits wherever the element sits in the
  // tile).  The other keys, each below 2^kDomLog2 of the total, keep their
  // float32 terms: their independent logit errors average out in the
  // weighted sum.  The terms are summed as 64-bit fixed point (2^-60), so the
  // sum does not depend on the order the keys were listed in.  The stored
  // values were formed with the unrefined lse2, so the selection's band
  // allows for a change of up to kDl2Allow octave; a larger change is counted
  // in the row's statistics.
  for (int i = tid; i < kG * kD; i += kRowThreads)
    qd[i] = static_cast<double>(bf16_bits_to_f32(qr[i]));
  if (tid < kG) {
    l2s[tid] = lse2[static_cast<size_t>(r) * kG + tid];
    s_corr[tid] = 0ull;
  }
  if (tid == 0) s_ndom = 0u;
  // A key's importance in float64 (bf16 products are exact), the largest over
  // the heads of c2 q_h.k - lse2_h: 16 lanes per key, lane `part` of a group
  // taking dims 8 part .. 8 part + 7 of all the heads, then a sum over the
  // group (its 16 lanes must share the key).  Every lane returns the value.
  auto exact_importance = [&](int64_t key, int part) -> double {
    const u32x4 raw = load_u32x4(kr + static_cast<size_t>(key) * kD + 8 * part);
    double kv[8];
#pragma unroll
    for (int t2 = 0; t2 < 8; ++t2) {
      const uint32_t word = raw[t2 >> 1];
      kv[t2] = static_cast<double>(__uint_as_float((t2 & 1) ? (word & 0xFFFF0000u) : (word << 16)));
    }
    // one head at a time (a short live range)
    double yy = -INFINITY;
#pragma unroll 1
    for (int h = 0; h < kG; ++h) {
      const double* qh = qd + h * kD + 8 * part;
      double acc = 0.0;
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) acc = fma(qh[t2], kv[t2], acc);
      acc = row16_sum(acc);
      yy = fmax(yy, c2 * acc - l2s[h]);
    }
    return yy;
  };
  // the stored value of importance 2^kDomLog2 (as the importance pass stores:
  // 2^10 steps per octave above the row's top log-weight minus 64)
  int vdom;
  {
    float yt = -INFINITY;
    for (int h = 0; h < kG; ++h) yt = fmaxf(yt, ytop_h[static_cast<size_t>(r) * kG + h]);
    const float vd = (kDomLog2 - (yt - kYRange)) * static_cast<float>(1 << kYFixBits);
    vdom = static_cast<int>(fminf(fmaxf(floorf(vd), 0.f), 65536.f));
  }
  int32_t* dlr = dom_list + static_cast<size_t>(r) * kDomCap;
  auto list_dom = [&](int64_t key) {
    const uint32_t slot = atomicAdd(&s_ndom, 1u);
    if (slot < static_cast<uint32_t>(kDomCap)) dlr[slot] = static_cast<int32_t>(key);
  };
  auto refine_row = [&]() {
    // the window's dominant keys
    for (int64_t j = first + tid; j <= P; j += kRowThreads)
      if (static_cast<int>(yr[j]) >= vdom) list_dom(j);
    __syncthreads();
    const uint32_t n_raw = s_ndom;
    const uint32_t n_dom = min(n_raw, static_cast<uint32_t>(kDomCap));
    const int col = lane & 15, grp = lane >> 4;
    for (uint32_t gi = wave; 16 * gi < n_dom; gi += kRowThreads / 64) {
      // 16 keys as the A operand rows, the 8 heads as B columns (8 .. 15 zero)
      const int32_t key = dlr[min(16 * gi + col, n_dom - 1)];
      bf16x8 ka[4], qb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ka[c] = as_bf16x8(load_u32x4(kr + static_cast<size_t>(key) * kD + 32 * c + 8 * grp));
        qb[c] = col < kG ? as_bf16x8(load_u32x4(qr + col * kD + 32 * c + 8 * grp))
                         : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      }
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma_16x16x32(ka[c], qb[c], acc);
      // lane (head col, grp) holds keys 16 gi + 4 grp + i
      if (col < kG) {
        const double l2h = l2s[col];
        const double* qh = qd + col * kD;
#pragma unroll 1
        for (int i = 0; i < 4; ++i) {
          const uint32_t e = 16 * gi + 4 * grp + i;
          if (e >= n_dom) break;
          const u16* krow = kr + static_cast<size_t>(dlr[e]) * kD;
          double dot = 0.0;
#pragma unroll 2
          for (int d8 = 0; d8 < kD / 8; ++d8) {
            const u32x4 raw = load_u32x4(krow + 8 * d8);
#pragma unroll
            for (int t2 = 0; t2 < 8; ++t2) {
              const uint32_t word = raw[t2 >> 1];
              dot = fma(qh[8 * d8 + t2],
                        static_cast<double>(__uint_as_float((t2 & 1) ? (word & 0xFFFF0000u) : (word << 16))),
                        dot);
            }
          }
          // the term's change 2^(y - lse2) - 2^(a2 - lse2) = p (e^d - 1), d = (y - a2) ln 2,
          // p = 2^(a2 - lse2); |d| is below 1e-4, so d + d^2 / 2 leaves 2e-13 of p.
          // a2 is the base-2 logit as the full layer formed it: a c2_hi (exact
          // here) for a prefill chunk; for decode rows the split kernel's
          // two-term product, the same float32 operations
          const double a2 = split_logits
                                ? static_cast<double>(fmaf(acc[i], c2_hi, acc[i] * c2_lo))
                                : static_cast<double>(acc[i]) * static_cast<double>(c2_hi);
          const double dd = (c2 * dot - a2) * M_LN2;
          const float pw = __builtin_amdgcn_exp2f(static_cast<float>(a2 - l2h));
          const double term = static_cast<double>(pw) * (dd + 0.5 * dd * dd);
          atomicAdd(&s_corr[col], static_cast<unsigned long long>(llrint(term * 0x1p60)));
        }
      }
    }
    __syncthreads();
    if (tid < kG) {
      const double c = static_cast<double>(static_cast<long long>(s_corr[tid])) * 0x1p-60;
      const double d = log1p(c) * M_LOG2E;
      const double l2 = l2s[tid] + d;
      l2s[tid] = l2;
      s_dl2[tid] = d;
      lse2r[static_cast<size_t>(r) * kG + tid] = l2;
      if (lse_out) lse_out[static_cast<size_t>(r) * kG + tid] = static_cast<float>(l2 * M_LN2);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t big = 0;
      for (int h = 0; h < kG; ++h) big += fabs(s_dl2[h]) > kDl2Allow ? 1u : 0u;
      stat[r] = RefineStat{n_dom, big, n_raw - n_dom, 0u};
    }
  };
  uint32_t n_keep = 0;
  if (topk > 0 && first > 0) {
    for (int i = tid; i < kPNB; i += kRowThreads) lh[i] = 0u;
    if (tid == 0) {
      s_floor = 0;
      s_km = 0u;
    }
    __syncthreads();
    // the head's max |k|: the largest of the importance pass's block shares
    {
      const uint32_t* kp = kmax + (static_cast<size_t>(b) * Hkv + g) * n_ib;
      uint32_t m = 0u;
      for (int i = tid; i < n_ib; i += kRowThreads) m = max(m, kp[i]);
      m = wave_umax(m);
      if (lane == 0 && m) atomicMax(&s_km, m);
    }
    // each head's sum of |q| (thread t holds elements t and t + 512: heads
    // wave / 2 and 4 + wave / 2)
    {
      float qa[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = tid + u * kRowThreads;
        qa[u] = fabsf(bf16_bits_to_f32(qr[i]));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) qa[u] += __shfl_xor(qa[u], off);
      if (lane == 0) {
        s_qn[0][wave] = qa[0];
        s_qn[1][wave] = qa[1];
      }
    }
    __syncthreads();
    if (tid == 0) {
      // E: twice the largest |stored - exact| in steps of 2^-10 octave, plus
      // one.  Storing costs at most 1.5 steps (rounding, and clamping at the
      // top) and the float32 roundings of the per-head offset and of the fma
      // that forms the step count (below 2^17 in magnitude near any
      // threshold) 2^-6 steps each.  The float32 importance is off by at most
      // 2^-24 (130 |s|max c2 + 2 |lse2|) octaves: the MFMA's 128 float32
      // additions of exact bf16 products, the scale's dropped low part and
      // the fma each cost 2^-24 of |s| c2 <= max|k| sum|q_h| c2; lse2's
      // rounding to float32 costs 2^-24 |lse2|, counted twice.
      double qn = 0.0, l2m = 0.0;
      for (int h = 0; h < kG; ++h) {
        const int wv = 2 * (h & 3);
        const int u = h >> 2;
        qn = fmax(qn, static_cast<double>(s_qn[u][wv]) + static_cast<double>(s_qn[u][wv + 1]));
        l2m = fmax(l2m, fabs(l2s[h]));
      }
      const double km = static_cast<double>(bf16_bits_to_f32(static_cast<u16>(s_km)));
      // sum|q| was taken in float32: allow 2^-20 relative for its rounding.
      // The stored values were formed with lse2 before its refinement (after
      // the pass): its change, at most kDl2Allow (checked), adds to their
      // error against the exact importance ranked here.
      const double d32 = 0x1p-24 * (130.0 * km * qn * (1.0 + 0x1p-20) * c2 + 2.0 * l2m) + kDl2Allow;
      const double steps = 1.5 + 0x1p-5 + d32 * static_cast<double>(1 << kYFixBits);
      s_E = static_cast<int>(fmin(ceil(2.0 * steps) + 1.0, 65536.0));
    }
    __syncthreads();
    const int E = s_E;
    if (kBlocks) {
      // ---- block-level selection.  A block's stored value (the largest
      // stored value of its tokens) is within the same bound of its exact
      // importance (the largest float64 importance of its tokens) as a
      // token's, so the band argument carries over to blocks unchanged: with
      // c the n_take-th largest block value, blocks above c + E are taken,
      // blocks below c - E are not, and the band's blocks are ranked on their
      // exact importance.  Of a band block only the tokens stored at or above
      // (block value) - E can hold its exact maximum.
      uint16_t* bmx = reinterpret_cast<uint16_t*>(pool);   // a value per block
      const int nblk = static_cast<int>((first + bs - 1) / bs);
      const int bs_log2 = __builtin_ctz(static_cast<unsigned>(bs));
      const int n_take = min(topk >> bs_log2, nblk);
      {
        // the pass: 32 values per thread and round (an aligned run inside one
        // block when bs >= 32, two blocks' runs when bs = 16), block maxima
        // over bs / 32 neighbouring lanes, their histogram, and the older
        // dominant keys for the refinement
        constexpr int kV = 32;
        const int lpb = bs / kV;   // lanes per block (0: bs = 16)
        // (32-bit round counts: the loop's test stays a scalar compare)
        const int prounds = static_cast<int>((first + kV * kRowThreads - 1) / (kV * kRowThreads));
        // The row as a buffer resource of whole 16-byte groups (a load past its
        // end reads zeros) and two named register sets, loaded a round ahead:
        // no branch and no copy between a load and its use.
        const auto yrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<u16*>(yr), 0, static_cast<int>(2 * ((first + 7) & ~int64_t{7})), 0x00020000);
        auto load_pround = [&](int rr, u32x4 (&yv)[4]) {
          const int off = 2 * kV * (tid + rr * kRowThreads);
#pragma unroll
          for (int u = 0; u < 4; ++u) yv[u] = __builtin_amdgcn_raw_buffer_load_b128(yrs, off + 16 * u, 0, 0);
        };
        auto bround = [&](int rr, const u32x4 (&ycur)[4]) __attribute__((always_inline)) {
          const int64_t i0 = kV * (static_cast<int64_t>(tid) + static_cast<int64_t>(rr) * kRowThreads);
          const int nv = static_cast<int>(max(static_cast<int64_t>(0), min(static_cast<int64_t>(kV), first - i0)));
          uint32_t m0 = 0, m1 = 0, md = 0;
#pragma unroll
          for (int e = 0; e < kV; ++e) {
            const uint32_t word = ycur[e >> 3][(e >> 1) & 3];
            const uint32_t v = e < nv ? ((e & 1) ? (word >> 16) : (word & 0xFFFFu)) : 0u;
            if (e < 16) m0 = max(m0, v);
            else m1 = max(m1, v);
            md |= static_cast<uint32_t>(e < nv && static_cast<int>(v) >= vdom) << e;
          }
          for (uint32_t m = md; m; m &= m - 1) list_dom(i0 + __builtin_ctz(m));   // rare
          if (lpb == 0) {
            if (nv > 0) {
              bmx[i0 >> 4] = static_cast<uint16_t>(m0);
              atomicAdd(&lh[m0 >> kVBinShift], 1u);
            }
            if (nv > 16) {
              bmx[(i0 >> 4) + 1] = static_cast<uint16_t>(m1);
              atomicAdd(&lh[m1 >> kVBinShift], 1u);
            }
          } else {
            uint32_t m = max(m0, m1);
            for (int off = 1; off < lpb; off <<= 1)
              m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
            // the block's first lane: its run starts the block
            if ((lane & (lpb - 1)) == 0 && nv > 0) {
              bmx[i0 >> bs_log2] = static_cast<uint16_t>(m);
              atomicAdd(&lh[m >> kVBinShift], 1u);
            }
          }
        };
        // two rounds per iteration, no exit between them (an odd count's last
        // round lies past the row: every value masked)
        u32x4 ya[4], yb[4];
        load_pround(0, ya);
        for (int rr = 0; rr < prounds; rr += 2) {
          load_pround(rr + 1, yb);
          bround(rr, ya);
          load_pround(rr + 2, ya);
          bround(rr + 1, yb);
        }
      }
      refine_row();   // (l2s refined before the band is ranked with it)
      // LDS use from here: bw holds the band's keys (u64, at most kBandBlk),
      // its block indices, the band winners and the merged selection; up the
      // blocks taken outright
      constexpr int kBandBlk = kMaxSel / 4;   // band blocks held in LDS
      uint64_t* lbk_b = reinterpret_cast<uint64_t*>(bw);
      int32_t* lbi_b = bw + 2 * kBandBlk;
      int32_t* bwin = bw + 3 * kBandBlk;
      int32_t* sel = bw + 3 * kBandBlk + kMaxSelBlocks;
      if (n_take == nblk) {
        // every block: the selection is [0, first)
        for (int64_t i = tid; i < first; i += kRowThreads) out[i] = static_cast<int32_t>(i);
        n_keep = static_cast<uint32_t>(first);
      } else {
        if (tid < 128) h256[tid] = 0u;
        __syncthreads();
        if (tid < 64) {
          const KthBin kb = kth_bin_wave_n<kPNB>(lh, static_cast<uint32_t>(n_take));
          if (tid == 0) {
            s_b = kb.bstar;   // found: n_take < nblk, the number of values counted
            s_above = kb.above;
          }
        }
        __syncthreads();
        const int bstar = s_b;
        for (int c = tid; c < nblk; c += kRowThreads) {
          const uint32_t v = bmx[c];
          if (static_cast<int>(v >> kVBinShift) == bstar) atomicAdd(&h256[v & 127u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
          const KthBin kc = kth_bin_wave_n<128>(h256, static_cast<uint32_t>(n_take) - s_above);
          if (tid == 0) s_c = (bstar << kVBinShift) | kc.bstar;
        }
        __syncthreads();
        const int band_lo = max(0, s_c - E);
        const int band_hi = min(65535, s_c + E);
        // thread t classifies the blocks [t per, (t + 1) per), per <= 32
        const int per = (nblk + kRowThreads - 1) / kRowThreads;
        const int c0 = min(nblk, tid * per), c1 = min(nblk, c0 + per);
        uint32_t mu = 0, ma = 0;
        for (int j = 0; j < c1 - c0; ++j) {
          const int v = bmx[c0 + j];
          mu |= static_cast<uint32_t>(v > band_hi) << j;
          ma |= static_cast<uint32_t>(v >= band_lo && v <= band_hi) << j;
        }
        uint32_t ou, oa, cu, ca;
        block_offsets2<kRowThreads / 64>(__popc(mu), __popc(ma), s_off[0], ou, oa, cu, ca);
        // the band fits LDS or the row's global band list (the plan gives
        // block selection a list of at least one entry per block)
        const bool band_lds = ca <= static_cast<uint32_t>(kBandBlk);
        const uint32_t bcap = band_lds ? static_cast<uint32_t>(kBandBlk)
                                       : static_cast<uint32_t>(min(band_cap, static_cast<int64_t>(nblk)));
        for (uint32_t m = mu; m; m &= m - 1) {
          if (ou < static_cast<uint32_t>(kMaxSelBlocks)) up[ou] = c0 + __builtin_ctz(m);
          ++ou;
        }
        const uint32_t n_up = min(cu, static_cast<uint32_t>(n_take));
        const uint32_t take = static_cast<uint32_t>(n_take) - n_up;
        const uint32_t n_band = min(ca, bcap);
        // the band's blocks, their exact importance and their ranking: one copy
        // for a band in LDS and one for a band in global memory, so that each
        // access has a known memory (a pointer to either would be a flat one)
        auto band_blocks = [&](int32_t* bi, uint64_t* bk) -> uint32_t {
          for (uint32_t m = ma, o = oa; m; m &= m - 1) {
            if (o < bcap) bi[o] = c0 + __builtin_ctz(m);
            ++o;
          }
          __syncthreads();
          // ---- each band block's exact importance, a wave per block: its
          // tokens stored at or above (block value) - E, four at a time (16
          // lanes each), the largest key over the wave
          const int part = lane & 15, grp = lane >> 4;
          for (uint32_t i = wave; i < n_band; i += kRowThreads / 64) {
            const int blk = bi[i];
            const int64_t j0 = static_cast<int64_t>(blk) << bs_log2;
            const int64_t j1 = min(first, j0 + bs);
            const int thr = static_cast<int>(bmx[blk]) - E;
            uint64_t best = 0ull;
            for (int64_t jb = j0; jb < j1; jb += 64) {
              const int64_t j = jb + lane;
              uint64_t m = __ballot(j < j1 && static_cast<int>(yr[min(j, j1 - 1)]) >= thr);
              while (m) {
                uint64_t mg = m;   // this group's candidate: the grp-th of m
                for (int s = 0; s < grp; ++s) mg &= mg - 1;
                const int64_t key = jb + __builtin_ctzll(mg ? mg : m);
                const double yy = exact_importance(key, part);
                if (mg) best = max(best, ordered_u64(yy));
#pragma unroll
                for (int s = 0; s < 4; ++s) m &= m - 1;
              }
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
              const uint64_t o = (static_cast<uint64_t>(static_cast<uint32_t>(
                                      __shfl_xor(static_cast<int>(best >> 32), off))) << 32) |
                                 static_cast<uint32_t>(__shfl_xor(static_cast<int>(best), off));
              best = max(best, o);
            }
            if (lane == 0) bk[i] = best;
          }
          __syncthreads();
          return rank_band(bk, bi, n_band, take, bwin, kMaxSelBlocks, &s_count, h256, s_red,
                           &s_hi, &s_need, &s_done, s_cnt, s_base);
        };
        const uint32_t n_w = band_lds
                                 ? band_blocks(lbi_b, lbk_b)
                                 : band_blocks(band_idx + static_cast<size_t>(r) * band_cap,
                                               band_key + static_cast<size_t>(r) * band_cap);
        __syncthreads();
        // ---- merge the two ascending block lists by rank
        for (uint32_t i = tid; i < n_up; i += kRowThreads) {
          const int32_t v = up[i];
          const uint32_t rk = i + lower_bound_lds(bwin, n_w, v);
          if (rk < static_cast<uint32_t>(kMaxSelBlocks)) sel[rk] = v;
        }
        for (uint32_t i = tid; i < n_w; i += kRowThreads) {
          const int32_t v = bwin[i];
          const uint32_t rk = i + lower_bound_lds(up, n_up, v);
          if (rk < static_cast<uint32_t>(kMaxSelBlocks)) sel[rk] = v;
        }
        const uint32_t n_sb = min(n_up + n_w, static_cast<uint32_t>(n_take));
        __syncthreads();
        // the selected blocks' tokens in ascending order: every block but the
        // row's last is whole, and the last, if taken, comes last
        const uint32_t n_tok = n_sb << bs_log2;
        for (uint32_t i = tid; i < n_tok; i += kRowThreads) {
          const int64_t j = (static_cast<int64_t>(sel[i >> bs_log2]) << bs_log2) + (i & (bs - 1));
          if (j < first) out[i] = static_cast<int32_t>(j);
        }
        if (n_sb > 0 && sel[n_sb - 1] == nblk - 1) {
          n_keep = n_tok - static_cast<uint32_t>((static_cast<int64_t>(nblk) << bs_log2) - first);
        } else {
          n_keep = n_tok;
        }
      }
    } else {
      // 16 values per thread and round, as two 16-byte loads; the next round's
      // loads are issued before this round is processed
      const int64_t rounds = (first + 16 * kRowThreads - 1) / (16 * kRowThreads);
      auto load_round = [&](int64_t rr, u32x4 (&yv)[2]) {
        const int64_t i0 = 16 * (static_cast<int64_t>(tid) + rr * kRowThreads);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          yv[u] = i0 + 8 * u < first ? *reinterpret_cast<const u32x4*>(yr + i0 + 8 * u)
                                     : u32x4{0u, 0u, 0u, 0u};
      };
      // ---- the pass: histogram at or above floor, and the list of the values
      // at or above (first value of floor) - E.  One barrier per round: the
      // floor that wave 0 raises after it is read by the other waves whenever
      // they get to it (a stale floor is still a valid one: it only lists and
      // counts more).  The first round's values are counted before any are
      // listed, so that its floor already applies to them.
      uint32_t n_list = 0;
      {
        // 32 values per thread and round here (four 16-byte loads), so half as
        // many rounds, and barriers, as the second pass below
        constexpr int kV = 32;
        // (32-bit round counts: the loop's test stays a scalar compare)
        const int prounds = static_cast<int>((first + kV * kRowThreads - 1) / (kV * kRowThreads));
        // The row as a buffer resource of whole 16-byte groups: a load past
        // its end reads zeros, so the loads need no branch (values of the last
        // group past first are masked below).  The next round's loads go to
        // the other of two named register sets before this round is processed,
        // so that no copy and no branch stands between a load and its use and
        // the waits count only the loads they need.
        const auto yrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<u16*>(yr), 0, static_cast<int>(2 * ((first + 7) & ~int64_t{7})), 0x00020000);
        auto load_pround = [&](int rr, u32x4 (&yv)[4]) {
          const int off = 2 * kV * (tid + rr * kRowThreads);
#pragma unroll
          for (int u = 0; u < 4; ++u) yv[u] = __builtin_amdgcn_raw_buffer_load_b128(yrs, off + 16 * u, 0, 0);
        };
        auto val_at = [](const u32x4 (&yv)[4], int e) -> uint32_t {
          const uint32_t word = yv[e >> 3][(e >> 1) & 3];
          return (e & 1) ? (word >> 16) : (word & 0xFFFFu);
        };
        // The value at a position known only at run time (each lane its own):
        // a four-level select over the 16 words, then the half.  The words come
        // as vector values and every level selects between values (no array:
        // a select among loads from one would become a load from a selected
        // address, and the array would go to memory).
        auto val_pick = [](u32x4 y0, u32x4 y1, u32x4 y2, u32x4 y3, int e) -> uint32_t {
          // (scalar selects: a two-element vector would want an aligned
          // register pair, and the words would be copied into pairs)
          const int w = e >> 1;
          const bool s0 = w & 1, s1 = w & 2, s2 = w & 4, s3 = w & 8;
          const uint32_t a00 = s0 ? y0[1] : y0[0], a01 = s0 ? y0[3] : y0[2];
          const uint32_t a10 = s0 ? y1[1] : y1[0], a11 = s0 ? y1[3] : y1[2];
          const uint32_t a20 = s0 ? y2[1] : y2[0], a21 = s0 ? y2[3] : y2[2];
          const uint32_t a30 = s0 ? y3[1] : y3[0], a31 = s0 ? y3[3] : y3[2];
          const uint32_t b0 = s1 ? a01 : a00, b1 = s1 ? a11 : a10;
          const uint32_t b2 = s1 ? a21 : a20, b3 = s1 ? a31 : a30;
          const uint32_t c0 = s2 ? b1 : b0, c1 = s2 ? b3 : b2;
          const uint32_t word = s3 ? c1 : c0;
          return __builtin_amdgcn_ubfe(word, static_cast<uint32_t>(e & 1) << 4, 16);
        };
        // Bit e set where value e >= T, in packed 16-bit arithmetic: the
        // saturating difference v - (T - 1), capped at 1, is 1 exactly there
        // (two packed instructions per word, written out: the compiler would
        // otherwise turn them into a compare and a select per value).  Word w
        // gives bits w (its low value) and 16 + w (its high value); an outer
        // perfect shuffle of the 32 bits then puts value e at bit e.
        auto mask_ge = [](u32x4 y0, u32x4 y1, u32x4 y2, u32x4 y3, int T) -> uint32_t {
          const uint32_t t1 = static_cast<uint32_t>(min(max(T, 1), 65536) - 1);
          const uint32_t tt = t1 | (t1 << 16), one = 0x00010001u;
          uint32_t p = 0;
#pragma unroll
          for (int w = 0; w < 16; ++w) {
            const uint32_t word = (w < 4 ? y0 : w < 8 ? y1 : w < 12 ? y2 : y3)[w & 3];
            uint32_t d;
            asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "v"(word), "v"(tt));
            asm("v_pk_min_u16 %0, %1, %2" : "=v"(d) : "v"(d), "v"(one));
            p |= d << w;
          }
          uint32_t t;
          t = (p ^ (p >> 8)) & 0x0000FF00u;
          p ^= t ^ (t << 8);
          t = (p ^ (p >> 4)) & 0x00F000F0u;
          p ^= t ^ (t << 4);
          t = (p ^ (p >> 2)) & 0x0C0C0C0Cu;
          p ^= t ^ (t << 2);
          t = (p ^ (p >> 1)) & 0x22222222u;
          p ^= t ^ (t << 1);
          return T <= 0 ? 0xFFFFFFFFu : (T > 65535 ? 0u : p);
        };
        auto pround = [&](auto may_be_first, int rr, const u32x4 (&ycur)[4]) __attribute__((always_inline)) {
          const int64_t i0 = kV * (static_cast<int64_t>(tid) + static_cast<int64_t>(rr) * kRowThreads);
          const int nv = static_cast<int>(max(static_cast<int64_t>(0), min(static_cast<int64_t>(kV), first - i0)));
          const uint32_t valid = nv >= kV ? 0xFFFFFFFFu : ((1u << nv) - 1u);
          // (an LDS atomic read: a volatile one through a generic pointer would
          // be a flat load, and its wait would also wait for the prefetch)
          int fl = __hip_atomic_load(&s_floor, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          // the largest of the round's values, in packed 16-bit maxima: it
          // reads every register of the round outside any branch, so that
          // their loads are waited for here and none is left pending at the
          // loop's head; it also tells whether any value reaches vdom
          u16x2 m2{0, 0};
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // (a plain copy first: a vector element is not an object to
              // reinterpret in place)
              const uint32_t word = ycur[u][e];
              m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, word));
            }
          const int mx = max(static_cast<int>(m2[0]), static_cast<int>(m2[1]));
          const u32x4 y0 = ycur[0], y1 = ycur[1], y2 = ycur[2], y3 = ycur[3];
          if (decltype(may_be_first)::value && rr == 0) {
            // the first round counts every value (the floor starts at bin 0),
            // then sets the floor before anything is listed
            if (nv >= kV) {
#pragma unroll
              for (int e = 0; e < kV; ++e) atomicAdd(&lh[val_at(ycur, e) >> kVBinShift], 1u);
            } else {
              for (uint32_t m = valid; m; m &= m - 1)
                atomicAdd(&lh[val_pick(y0, y1, y2, y3, __builtin_ctz(m)) >> kVBinShift], 1u);
            }
            __syncthreads();
            if (wave == 0) {
              const KthBin kb = kth_bin_wave_n<kPNB>(lh, static_cast<uint32_t>(topk));
              if (lane == 0 && kb.found) s_floor = kb.bstar;
            }
            __syncthreads();
            fl = s_floor;
          }
          // the values to list (>= vmin) and the dominant ones (>= vdom); the
          // histogram's values (bin >= floor) are among the listed ones
          const int vmin = (fl << kVBinShift) - E;
          const uint32_t ml = mask_ge(y0, y1, y2, y3, vmin) & valid;
          const uint32_t md = mx >= vdom ? (mask_ge(y0, y1, y2, y3, vdom) & valid) : 0u;
          uint32_t ol, o_dummy, tot, t_dummy;
          block_offsets2<kRowThreads / 64>(__popc(ml), 0u, s_off[rr & 1], ol, o_dummy, tot, t_dummy);
          // raise the floor from the counts so far (this round's, counted
          // below, may be seen in part: any subset of the row's values gives
          // a k-th bin no higher than the row's own)
          if (wave == 0) {
            const KthBin kb = kth_bin_wave_n<kPNB>(lh, static_cast<uint32_t>(topk));
            if (lane == 0 && kb.found && kb.bstar > fl) atomicMax(&s_floor, kb.bstar);
          }
          ol += n_list;
          n_list += tot;
          // each lane walks its own selected values in key order: the wave
          // takes as many steps as its busiest lane has values, not kV
          for (uint32_t m = ml | md; m; m &= m - 1) {
            const int e = __builtin_ctz(m);
            const uint32_t v = val_pick(y0, y1, y2, y3, e);
            if ((ml >> e) & 1u) {
              if (rr > 0 && static_cast<int>(v >> kVBinShift) >= fl) atomicAdd(&lh[v >> kVBinShift], 1u);
              if (ol < static_cast<uint32_t>(kPList)) {
                lidx[ol] = static_cast<int32_t>(i0 + e);
                lval[ol] = static_cast<uint16_t>(v);
              }
              ++ol;
            }
            if ((md >> e) & 1u) list_dom(i0 + e);   // rare
          }
        };
        // A row of one round (a short row, where a large share of the values
        // are candidates once the floor is set): fixed loops over the 32
        // positions, each value read at a fixed place, cost less than the walk.
        // Every value is counted, the floor set, then the list written; the
        // count is whole before the k-th bin is read again after the pass.
        auto pround_single = [&](const u32x4 (&ycur)[4]) {
          const int64_t i0 = kV * static_cast<int64_t>(tid);
          const int nv = static_cast<int>(max(static_cast<int64_t>(0), min(static_cast<int64_t>(kV), first - i0)));
#pragma unroll
          for (int e = 0; e < kV; ++e)
            if (e < nv) atomicAdd(&lh[val_at(ycur, e) >> kVBinShift], 1u);
          __syncthreads();
          if (wave == 0) {
            const KthBin kb = kth_bin_wave_n<kPNB>(lh, static_cast<uint32_t>(topk));
            if (lane == 0 && kb.found) s_floor = kb.bstar;
          }
          __syncthreads();
          const int vmin = (s_floor << kVBinShift) - E;
          uint32_t ml = 0, md = 0;
#pragma unroll
          for (int e = 0; e < kV; ++e) {
            const int v = static_cast<int>(val_at(ycur, e));
            ml |= static_cast<uint32_t>(e < nv && v >= vmin) << e;
            md |= static_cast<uint32_t>(e < nv && v >= vdom) << e;
          }
          for (uint32_t m = md; m; m &= m - 1) list_dom(i0 + __builtin_ctz(m));   // rare
          uint32_t ol, o_dummy, tot, t_dummy;
          block_offsets2<kRowThreads / 64>(__popc(ml), 0u, s_off[0], ol, o_dummy, tot, t_dummy);
          n_list = tot;
#pragma unroll
          for (int e = 0; e < kV; ++e) {
            if (!((ml >> e) & 1u)) continue;
            if (ol < static_cast<uint32_t>(kPList)) {
              lidx[ol] = static_cast<int32_t>(i0 + e);
              lval[ol] = static_cast<uint16_t>(val_at(ycur, e));
            }
            ++ol;
          }
        };
        u32x4 ya[4], yb[4];
        load_pround(0, ya);
        // Two rounds per iteration and no exit between them, so that every
        // path back to the loop's head has used the loads it issued: with an
        // odd number of rounds the last one lies past the row, reads zeros and
        // counts and lists nothing (every value is masked), at the cost of
        // one barrier.
        if (prounds == 1) {
          pround_single(ya);
        } else {
          for (int rr = 0; rr < prounds; rr += 2) {
            load_pround(rr + 1, yb);
            pround(std::true_type{}, rr, ya);
            load_pround(rr + 2, ya);
            pround(std::false_type{}, rr + 1, yb);
          }
        }
      }
      refine_row();   // (l2s refined before the band is ranked with it)
      if (tid == 0) stat[r].pad = n_list;   // (thread 0 also wrote the rest)
      const bool listed = n_list <= static_cast<uint32_t>(kPList);
      if (tid < 128) h256[tid] = 0u;
      __syncthreads();
      if (tid < 64) {
        const KthBin kb = kth_bin_wave_n<kPNB>(lh, static_cast<uint32_t>(topk));
        if (tid == 0) {
          s_b = kb.found ? kb.bstar : -1;
          s_above = kb.above;
        }
      }
      __syncthreads();
      if (s_b < 0) {
        // fewer older keys than top_k: all of them, in order
        n_keep = static_cast<uint32_t>(min(first, static_cast<int64_t>(topk)));
        for (uint32_t i = tid; i < n_keep; i += kRowThreads) out[i] = static_cast<int32_t>(i);
      } else {
        const int bstar = s_b;
        int band_lo, band_hi;
        if (listed) {
          // ---- c: the k-th largest v, from the listed values in bin b*
          for (uint32_t i = tid; i < n_list; i += kRowThreads) {
            const uint32_t v = lval[i];
            if (static_cast<int>(v >> kVBinShift) == bstar) atomicAdd(&h256[v & 127u], 1u);
          }
          __syncthreads();
          if (tid < 64) {
            const KthBin kc = kth_bin_wave_n<128>(h256, static_cast<uint32_t>(topk) - s_above);
            if (tid == 0) s_c = (bstar << kVBinShift) | kc.bstar;
          }
          __syncthreads();
          band_lo = max(0, s_c - E);
          band_hi = min(65535, s_c + E);
        } else {
          band_lo = max(0, (bstar << kVBinShift) - E);
          band_hi = min(65535, (bstar << kVBinShift) + 127 + E);
        }
        int32_t* gbi = band_idx + static_cast<size_t>(r) * band_cap;
        uint64_t* gbk = band_key + static_cast<size_t>(r) * band_cap;
        bool band_lds = false, band_glob = false;
        uint32_t cu = 0, ca = 0;
        if (listed) {
          // ---- split the list: each thread takes kPListPer consecutive
          // entries into registers, so the band may overwrite the list
          const uint32_t q0 = static_cast<uint32_t>(tid) * kPListPer;
          int32_t li[kPListPer];
          uint32_t mu = 0, ma = 0;
#pragma unroll
          for (int j = 0; j < kPListPer; ++j) {
            const uint32_t i = q0 + j;
            li[j] = 0;
            if (i < n_list) {
              li[j] = lidx[i];
              const int v = lval[i];
              mu |= static_cast<uint32_t>(v > band_hi) << j;
              ma |= static_cast<uint32_t>(v >= band_lo && v <= band_hi) << j;
            }
          }
          uint32_t ou, oa;
          block_offsets2<kRowThreads / 64>(__popc(mu), __popc(ma), s_off[0], ou, oa, cu, ca);
          band_lds = ca <= static_cast<uint32_t>(kUncCap);
          band_glob = !band_lds && ca <= static_cast<uint64_t>(band_cap);
#pragma unroll
          for (int j = 0; j < kPListPer; ++j) {
            if ((mu >> j) & 1u) {
              if (ou < static_cast<uint32_t>(kMaxSel)) up[ou] = li[j];
              ++ou;
            }
            if ((ma >> j) & 1u) {
              if (band_lds) lbi[oa] = li[j];
              else if (band_glob) gbi[oa] = li[j];
              ++oa;
            }
          }
        } else {
          // ---- the list overflowed: a second pass over v, in key order; the
          // band goes to the global list (up to band_cap entries)
          u32x4 ycur[2], ynxt[2];
          if (rounds > 0) load_round(0, ycur);
          for (int64_t rr = 0; rr < rounds; ++rr) {
            const int64_t i0 = 16 * (static_cast<int64_t>(tid) + rr * kRowThreads);
            if (rr + 1 < rounds) load_round(rr + 1, ynxt);
            const int nv = static_cast<int>(min(static_cast<int64_t>(16), first - i0));
            uint32_t mu = 0, ma = 0;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int v = static_cast<int>(u16_at(ycur, e));
              mu |= static_cast<uint32_t>(e < nv && v > band_hi) << e;
              ma |= static_cast<uint32_t>(e < nv && v >= band_lo && v <= band_hi) << e;
            }
            uint32_t ou, oa;
            reserve_two(__popc(mu), __popc(ma), nullptr, nullptr, s_cnt, s_base, ou, oa);
            ou += cu;
            oa += ca;
            cu += s_base[2];
            ca += s_base[3];
            for (uint32_t m = mu; m; m &= m - 1) {
              if (ou < static_cast<uint32_t>(kMaxSel)) up[ou] = static_cast<int32_t>(i0 + __builtin_ctz(m));
              ++ou;
            }
            for (uint32_t m = ma; m; m &= m - 1) {
              if (oa < static_cast<uint64_t>(band_cap)) gbi[oa] = static_cast<int32_t>(i0 + __builtin_ctz(m));
              ++oa;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) ycur[u] = ynxt[u];
          }
          band_glob = ca <= static_cast<uint64_t>(band_cap);
        }
        __syncthreads();
        const uint32_t n_up = min(cu, static_cast<uint32_t>(topk));
        const uint32_t take = static_cast<uint32_t>(topk) - n_up;
        uint32_t n_w = 0;
        // ---- exact importance of the band keys, then their ranking: one copy
        // for a band in LDS and one for a band in global memory, so that each
        // access has a known memory (a pointer to either would be a flat one)
        auto band_rank = [&](int32_t* bi_, uint64_t* bk_, uint32_t n_band) -> uint32_t {
          for (uint32_t i = static_cast<uint32_t>(tid) >> 4; i < n_band; i += kRowThreads / 16) {
            const double yy = exact_importance(bi_[i], tid & 15);
            if ((tid & 15) == 0) bk_[i] = ordered_u64(yy);
          }
          __syncthreads();
          return rank_band(bk_, bi_, n_band, take, bw, kMaxSel, &s_count, h256, s_red, &s_hi,
                           &s_need, &s_done, s_cnt, s_base);
        };
        if (band_lds) {
          n_w = band_rank(lbi, lbk, min(ca, static_cast<uint32_t>(kUncCap)));
        } else if (band_glob) {
          n_w = band_rank(gbi, gbk, min(ca, static_cast<uint32_t>(band_cap)));
        } else if (take > 0) {
          // the band is too large to list: rank it by its stored importance
          // (unordered winners, then sorted)
          struct ScanSrc {
            const u16* yr;
            int lo, hi;
            __device__ bool get(int64_t i, uint64_t& key, int32_t& j) const {
              const int v = yr[i];
              if (v < lo || v > hi) return false;
              key = static_cast<uint64_t>(v);
              j = static_cast<int32_t>(i);
              return true;
            }
          } src{yr, band_lo, band_hi};
          if (tid == 0) s_count = 0u;
          __syncthreads();
          radix_select_band(src, first, min(take, ca), bw, &s_count, h256, &s_thi, &s_tlo, &s_need);
          n_w = min(s_count, static_cast<uint32_t>(kMaxSel));
          int32_t v[kMaxSel / kRowThreads];
#pragma unroll
          for (int e = 0; e < kMaxSel / kRowThreads; ++e) {
            const uint32_t ii = (kMaxSel / kRowThreads) * tid + e;
            v[e] = ii < n_w ? bw[ii] : 0x7FFFFFFF;
          }
          __syncthreads();
          block_bitonic<kMaxSel / kRowThreads>(v, bw, static_cast<int>(n_w), IntLess{});
#pragma unroll
          for (int e = 0; e < kMaxSel / kRowThreads; ++e) {
            const uint32_t ii = (kMaxSel / kRowThreads) * tid + e;
            if (ii < n_w) bw[ii] = v[e];
          }
        }
        __syncthreads();
        // ---- merge the two ascending lists by rank
        for (uint32_t i = tid; i < n_up; i += kRowThreads) {
          const int32_t v = up[i];
          const uint32_t rk = i + lower_bound_lds(bw, n_w, v);
          if (rk < static_cast<uint32_t>(cap)) out[rk] = v;
        }
        for (uint32_t i = tid; i < n_w; i += kRowThreads) {
          const int32_t v = bw[i];
          const uint32_t rk = i + lower_bound_lds(up, n_up, v);
          if (rk < static_cast<uint32_t>(cap)) out[rk] = v;
        }
        n_keep = min(n_up + n_w, static_cast<uint32_t>(topk));
      }
    }
  } else {
    __syncthreads();
    refine_row();
  }
  const int n_total = static_cast<int>(n_keep) + static_cast<int>(static_cast<int64_t>(P) - first + 1);
  for (int i = static_cast<int>(n_keep) + tid; i < cap; i += kRowThreads)
    out[i] = i < n_total ? static_cast<int32_t>(first + (i - static_cast<int>(n_keep))) : -1;
  if (tid == 0) nsel_out[r] = min(n_total, cap);
}

// ================================================================ block-level selection
//
// The previous generation's variant (news page, section "Token级选择：精准定位
// 大海里的那根针", which contrasts whole-block picks with token-level picks):
// the older tokens [0, first) are cut into aligned blocks of bs tokens (the
// last one ending at first), a block's importance is the largest importance of
// its tokens, and the top_k / bs best blocks are kept, ties to the lower block
// index; the window is forced as in the token-level selection.  Both kernels
// below (the fused decode step, from the candidate lists, and from given
// scores) fill one 64-bit key per block in LDS (0 = no key: below every real
// key), take the threshold with the radix select of the token path, and emit.
// A prefill chunk selects blocks in prefill_select_kernel<true>.

// Select from the block keys (LDS, one per block, 0 = no key) and write the
// row: the selected blocks' tokens in ascending order, the window, -1 padding,
// and the count.  The keyed blocks are first compacted in place (block order
// kept), so the radix select reads only them; the selected blocks' tokens are
// then written by all threads at once.  All threads call it.
__device__ __forceinline__ void emit_blocks(
    uint64_t* bkey, int nblk, int bs, int64_t first, int P, int topk, int cap, int32_t* out,
    int32_t* nsel_out, int r, uint32_t* sel_blk, uint32_t* sel_off, uint32_t* h256,
    uint32_t* s_red, uint64_t* s_hi, uint32_t* s_need, int* s_done, uint32_t (*s_cnt)[16],
    uint32_t* s_base) {
  constexpr int kOwn = kMaxBlocks / kSelThreads;   // blocks owned per thread, at most
  const int tid = threadIdx.x;
  // thread t owns the consecutive blocks [t * per, (t + 1) * per)
  const int per = (nblk + kSelThreads - 1) / kSelThreads;
  const int c0 = min(nblk, tid * per), c1 = min(nblk, c0 + per);
  uint32_t nzmask = 0;   // the owned blocks that have a key
  {
    uint64_t kr[kOwn];
#pragma unroll
    for (int u = 0; u < kOwn; ++u) {
      kr[u] = c0 + u < c1 ? bkey[c0 + u] : 0ull;
      nzmask |= (kr[u] != 0ull ? 1u : 0u) << u;
    }
    uint32_t p0, dummy;
    reserve_two(__popc(nzmask), 0u, nullptr, nullptr, s_cnt, s_base, p0, dummy);  // reads done
    uint32_t p = p0;
#pragma unroll
    for (int u = 0; u < kOwn; ++u)
      if (kr[u] != 0ull) bkey[p++] = kr[u];
  }
  // after compaction the owned keyed blocks sit at pos0, pos0 + 1, ... in block order
  uint32_t pos0, dummy;
  reserve_two(__popc(nzmask), 0u, nullptr, nullptr, s_cnt, s_base, pos0, dummy);
  const uint32_t n_nz = s_base[2];
  const uint32_t need = min(static_cast<uint32_t>(topk / bs), n_nz);
  const bool none = need == 0;
  const bool all = !none && need >= n_nz;
  KThr kt{0ull, 0u, true};
  if (!none && !all) kt = key_threshold(bkey, n_nz, need, h256, s_red, s_hi, s_need, s_done);
  // ties at the threshold go to the lowest blocks: rank them in block order
  uint32_t n_tie = 0;
  if (!none && !all && !kt.incl)
    for (uint32_t i = 0; i < static_cast<uint32_t>(__popc(nzmask)); ++i)
      n_tie += bkey[pos0 + i] == kt.thr ? 1u : 0u;
  uint32_t tie0;
  reserve_two(n_tie, 0u, nullptr, nullptr, s_cnt, s_base, tie0, dummy);
  uint32_t selmask = 0, nsb = 0, ntok = 0;
  {
    uint32_t tr = tie0, i = 0;
#pragma unroll
    for (int u = 0; u < kOwn; ++u) {
      if (!((nzmask >> u) & 1u)) continue;
      const uint64_t key = bkey[pos0 + i++];
      bool sel = false;
      if (!none) {
        if (all || key > kt.thr) sel = true;
        else if (key == kt.thr) sel = kt.incl || tr++ < kt.nd_t;
      }
      if (sel) {
        selmask |= 1u << u;
        ++nsb;
        ntok += static_cast<uint32_t>(
            min(static_cast<int64_t>(bs), first - static_cast<int64_t>(c0 + u) * bs));
      }
    }
  }
  uint32_t sb, at;
  reserve_two(nsb, ntok, nullptr, nullptr, s_cnt, s_base, sb, at);
  const uint32_t n_sb = s_base[2], n_keep = s_base[3];
  for (uint32_t m = selmask; m; m &= m - 1) {
    const int u = __builtin_ctz(m);
    sel_blk[sb] = static_cast<uint32_t>(c0 + u);
    sel_off[sb] = at;
    at += static_cast<uint32_t>(
        min(static_cast<int64_t>(bs), first - static_cast<int64_t>(c0 + u) * bs));
    ++sb;
  }
  if (tid == 0) sel_off[n_sb] = n_keep;
  __syncthreads();
  // the selected tokens, all threads: slot i lies in the last block whose offset is <= i
  for (uint32_t i = tid; i < n_keep && i < static_cast<uint32_t>(cap); i += kSelThreads) {
    uint32_t lo = 0, hi = n_sb - 1;
    while (lo < hi) {
      const uint32_t mid = (lo + hi + 1) >> 1;
      if (sel_off[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    out[i] = static_cast<int32_t>(sel_blk[lo] * static_cast<uint32_t>(bs) + (i - sel_off[lo]));
  }
  const int n_total =
      static_cast<int>(n_keep) + static_cast<int>(static_cast<int64_t>(P) - first + 1);
  for (int i = static_cast<int>(n_keep) + tid; i < cap; i += kSelThreads)
    out[i] = i < n_total ? static_cast<int32_t>(first + (i - static_cast<int>(n_keep))) : -1;
  if (tid == 0) nsel_out[r] = min(n_total, cap);
}

// Fused decode: the candidate lists hold the exact float64 importance of every
// key that can be the largest of a selectable block (such a block's best key
// is among the best top_k keys, all of which the lists keep); a block's key is
// the maximum over its listed keys.
__global__ __launch_bounds__(kSelThreads) void block_row_select_kernel(
    const double* __restrict__ cand_y, const int32_t* __restrict__ cand_idx,
    const uint32_t* __restrict__ cand_cnt, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ nsel_out, int64_t S, int T, int Hkv, int topk, int w, int cap,
    int chunk, int n_chunks, int bs) {
  __shared__ uint64_t bkey[kMaxBlocks];
  __shared__ uint32_t pre[kMaxChunks + 1];
  __shared__ uint32_t sel_blk[kMaxSelBlocks];
  __shared__ uint32_t sel_off[kMaxSelBlocks + 1];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_red[4];
  __shared__ uint64_t s_hi;
  __shared__ uint32_t s_need;
  __shared__ int s_done;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = row_first(P, w);
  const int nblk = static_cast<int>((first + bs - 1) / bs);
  for (int c = tid; c < nblk; c += kSelThreads) bkey[c] = 0ull;
  if (topk > 0 && first > 0) {
    // chunk lengths, then their exclusive prefix in pre
    constexpr int kPer = kMaxChunks / kSelThreads;
    uint32_t cl[kPer];
    uint32_t mysum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = kPer * tid + u;
      cl[u] = c < n_chunks ? cand_cnt[static_cast<size_t>(r) * n_chunks + c] : 0u;
      mysum += cl[u];
    }
    uint32_t off, dummy;
    reserve_two(mysum, 0u, nullptr, nullptr, s_cnt, s_base, off, dummy);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = kPer * tid + u;
      if (c < n_chunks) pre[c] = off;
      off += cl[u];
    }
    if (tid == 0) pre[n_chunks] = s_base[2];
    __syncthreads();
    const uint32_t n_total = pre[n_chunks];
    const size_t chunk_len = static_cast<size_t>(chunk) * kSubKeys;
    const size_t rbase = static_cast<size_t>(r) * n_chunks * chunk_len;
    // the entries spread evenly over the threads, four loads in flight each
    constexpr int kU = 4;
    for (uint32_t base = 0; base < n_total; base += kU * kSelThreads) {
      double y[kU];
      int32_t j[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t i = base + u * kSelThreads + tid;
        j[u] = -1;
        if (i < n_total) {
          int lo = 0, hi = n_chunks - 1;   // the chunk of entry i: largest c with pre[c] <= i
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= i) lo = mid;
            else hi = mid - 1;
          }
          const size_t at = rbase + static_cast<size_t>(lo) * chunk_len + (i - pre[lo]);
          y[u] = cand_y[at];
          j[u] = cand_idx[at];
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (j[u] >= 0 && j[u] < first)
          atomicMax(reinterpret_cast<unsigned long long*>(&bkey[j[u] / bs]),
                    static_cast<unsigned long long>(ordered_u64(y[u])));
    }
  }
  __syncthreads();
  emit_blocks(bkey, nblk, bs, first, P, topk, cap, idx_out + static_cast<size_t>(r) * cap,
              nsel_out, r, sel_blk, sel_off, h256, s_red, &s_hi, &s_need, &s_done, s_cnt,
              s_base);
}

// From given scores [R][S] (compared exactly as given): a block's key is the
// largest score of its older tokens.
__global__ __launch_bounds__(kSelThreads) void block_scores_select_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ nsel_out, int64_t S, int T, int Hkv, int topk, int w, int cap,
    int bs) {
  __shared__ uint64_t bkey[kMaxBlocks];
  __shared__ uint32_t sel_blk[kMaxSelBlocks];
  __shared__ uint32_t sel_off[kMaxSelBlocks + 1];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_red[4];
  __shared__ uint64_t s_hi;
  __shared__ uint32_t s_need;
  __shared__ int s_done;
  __shared__ uint32_t s_cnt[2][16];
  __shared__ uint32_t s_base[4];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = row_first(P, w);
  const int nblk = static_cast<int>((first + bs - 1) / bs);
  const float* sr = scores + static_cast<size_t>(r) * S;
  // each wave takes whole blocks: its lanes stride the block, then a wave max
  for (int c = wave; c < nblk; c += kSelThreads / 64) {
    const int64_t j0 = static_cast<int64_t>(c) * bs;
    const int64_t j1 = min(first, j0 + bs);
    uint32_t m = 0u;
    for (int64_t j = j0 + lane; j < j1; j += 64) m = max(m, ordered_u32(sr[j]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(m, off)));
    // the low bit marks a real key, so that no block compares equal to "no key"
    if (lane == 0) bkey[c] = (static_cast<uint64_t>(m) << 32) | 1ull;
  }
  __syncthreads();
  emit_blocks(bkey, nblk, bs, first, P, topk, cap, idx_out + static_cast<size_t>(r) * cap,
              nsel_out, r, sel_blk, sel_off, h256, s_red, &s_hi, &s_need, &s_done, s_cnt,
              s_base);
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_scores_select(const Plan& p, const float* scores, int32_t* idx, int32_t* n_sel,
                                void* ws, hipStream_t st) {
  if (p.bs > 0) {
    hipLaunchKernelGGL(block_scores_select_kernel, dim3(p.R), dim3(kSelThreads), 0, st, scores,
                       idx, n_sel, p.S, p.T, p.Hkv, p.k, p.w, p.cap, p.bs);
    return hipGetLastError();
  }
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

hipError_t launch_subtile_hist(const Plan& p, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  hipLaunchKernelGGL(subtile_hist_kernel, dim3(p.hs_nchunk, p.R), dim3(kThreads), 0, st,
                     reinterpret_cast<const float*>(w + p.off_stmax),
                     reinterpret_cast<const double*>(w + p.off_lse2),
                     reinterpret_cast<const float*>(w + p.off_ytop),
                     reinterpret_cast<uint32_t*>(w + p.off_hist),
                     reinterpret_cast<uint32_t*>(w + p.off_hist_c), p.S, p.Spad, p.T, p.Hkv, p.k,
                     p.w, p.hs_chunk);
  return hipGetLastError();
}

hipError_t launch_subtile_cand(const Plan& p, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  hipLaunchKernelGGL(subtile_cand_kernel, dim3(p.cc_nchunk, p.R), dim3(kThreads), 0, st,
                     reinterpret_cast<const float*>(w + p.off_stmax),
                     p.quads ? reinterpret_cast<const unsigned char*>(w + p.off_qdiff) : nullptr,
                     reinterpret_cast<const double*>(w + p.off_lse2),
                     reinterpret_cast<const float*>(w + p.off_ytop),
                     reinterpret_cast<const uint32_t*>(w + p.off_hist),
                     reinterpret_cast<int32_t*>(w + p.off_clist),
                     reinterpret_cast<uint32_t*>(w + p.off_ccnt),
                     reinterpret_cast<int32_t*>(w + p.off_lo),
                     reinterpret_cast<int32_t*>(w + p.off_dsub),
                     reinterpret_cast<uint32_t*>(w + p.off_dsub_cnt),
                     reinterpret_cast<float*>(w + p.off_cut), refine_budget(p.S), p.S, p.Spad,
                     p.T, p.Hkv, p.k, p.w, p.cc_chunk, p.cc_nchunk);
  return hipGetLastError();
}

hipError_t launch_fused_select(const Plan& p, const u16* q, const u16* k, int32_t* idx,
                               int32_t* n_sel, float* lse, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double* lse2 = reinterpret_cast<const double*>(w + p.off_lse2);
  const float* ytop = reinterpret_cast<const float*>(w + p.off_ytop);
  uint32_t* hist_c = reinterpret_cast<uint32_t*>(w + p.off_hist_c);
  double* cand_y = reinterpret_cast<double*>(w + p.off_cand_y);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(w + p.off_cand_idx);
  uint32_t* cand_cnt = reinterpret_cast<uint32_t*>(w + p.off_cand_cnt);
  const double c2 = p.scale * 1.4426950408889634;  // scale * log2(e)
  // the subtile-bound histogram, the candidate (and dominant) subtiles, then
  // the refinement of lse2 before anything ranks keys with it
  hipError_t e = launch_subtile_hist(p, ws, st);
  if (e != hipSuccess) return e;
  if ((e = launch_subtile_cand(p, ws, st)) != hipSuccess) return e;
  if ((e = launch_lse_refine(p, q, k, ws, st)) != hipSuccess) return e;
  int32_t* clist = reinterpret_cast<int32_t*>(w + p.off_clist);
  uint32_t* ccnt = reinterpret_cast<uint32_t*>(w + p.off_ccnt);
  int32_t* lo = reinterpret_cast<int32_t*>(w + p.off_lo);
  hipLaunchKernelGGL(subtile_score_kernel, dim3(p.sc_nchunk, p.R), dim3(kThreads), 0, st, lo,
                     clist, ccnt, lse2, reinterpret_cast<const RefinePart*>(w + p.off_ref_part),
                     p.ref_nwg, reinterpret_cast<double*>(w + p.off_lse2r), lse,
                     reinterpret_cast<RefineStat*>(w + p.off_ref_stat), ytop, hist_c, q, k,
                     cand_y, cand_idx, cand_cnt, p.S, p.T, p.Hkv, p.k, p.w, p.cc_chunk,
                     p.cc_nchunk, p.sc_chunk, p.sc_nchunk, c2, p.kvp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.bs > 0) {
    hipLaunchKernelGGL(block_row_select_kernel, dim3(p.R), dim3(kSelThreads), 0, st, cand_y,
                       cand_idx, cand_cnt, idx, n_sel, p.S, p.T, p.Hkv, p.k, p.w, p.cap,
                       p.sc_chunk, p.sc_nchunk, p.bs);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(row_select_kernel, dim3(p.R), dim3(kSelThreads), 0, st, hist_c, cand_y,
                     cand_idx, cand_cnt, ytop, idx, n_sel, p.S, p.T, p.Hkv, p.k, p.w, p.cap,
                     p.sc_chunk, p.sc_nchunk);
  return hipGetLastError();
}

hipError_t launch_prefill_select(const Plan& p, const u16* q, const u16* k, int32_t* idx,
                                 int32_t* n_sel, float* lse, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  const float c2_hi = static_cast<float>(c2);
  const float c2_lo = static_cast<float>(c2 - static_cast<double>(c2_hi));
  auto kern = p.bs > 0 ? prefill_select_kernel<true> : prefill_select_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(p.R), dim3(kRowThreads), 0, st,
                     reinterpret_cast<const u16*>(w + p.off_ybuf),
                     reinterpret_cast<const uint32_t*>(w + p.off_kmax), p.n_ib,
                     reinterpret_cast<const double*>(w + p.off_lse2),
                     reinterpret_cast<double*>(w + p.off_lse2r), lse,
                     reinterpret_cast<const float*>(w + p.off_ytop),
                     reinterpret_cast<int32_t*>(w + p.off_dom_list),
                     reinterpret_cast<RefineStat*>(w + p.off_ref_stat), q, k,
                     reinterpret_cast<int32_t*>(w + p.off_band_idx),
                     reinterpret_cast<uint64_t*>(w + p.off_band_key), p.band_cap, idx, n_sel, p.S,
                     p.Spad, p.T, p.Hkv, p.k, p.w, p.cap, p.bs, c2, c2_hi, c2_lo, p.T == 1, p.kvp);
  return hipGetLastError();
}

}  // namespace hs2
