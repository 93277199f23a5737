// Token-level selection: the forced recent window plus the top-k older keys
// by importance, ties to the lower index (news page "两天两连更：小米提前亮出V3底牌",
// section "Token级选择：精准定位大海里的那根针"; importance is the largest
// probability that any query head of the GQA group gives the key).
//
// Per row (batch, query token, KV head) with candidates [0, P-w+1):
//  1. select_hist: every candidate gets a 32-bit key that is monotone in its
//     importance; a 2048-bin histogram of the top 11 bits is built in LDS per
//     work-group and added to the row's histogram; the last work-group of the
//     row finds the bin b* that holds the k-th largest key.
//       - from logits (the fused step): importance is computed in float32 from
//         the stored logits and lse; the key is a fixed-point image of its
//         base-2 log over [top - 64, top], so a bin spans 1/32 of an octave.
//         float32 error is far below a bin, so bins >= b*+2 are certainly
//         selected, bins <= b*-2 certainly not, and bins b*-1..b*+1 are the
//         uncertain band.
//       - from given scores: the key is the order-preserving image of the
//         float32 score itself; only bin b* is uncertain.
//  2. select_compact: candidates of the certain bins and of the uncertain band
//     are appended to two per-row lists; a wave appends with one atomic, each
//     lane's slot coming from the wave's ballot and a masked bit count.
//  3. select_finish (one work-group per row): the uncertain keys are ranked by
//     their exact importance — recomputed in float64 from the bf16 query and
//     key (from logits), or the given score — and the best ones fill the k
//     slots; the selected indices are sorted ascending in LDS and the window
//     appended.  Bands too large for LDS go through a slower exact radix
//     select over the row.

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int row_pos(int r, int T, int Hkv, int64_t S) {
  const int t = (r / Hkv) % T;
  return static_cast<int>(S - T + t);
}

__device__ __forceinline__ uint32_t key_from_log2(float y, float ybase) {
  const float z = (y - ybase) * 67108864.0f;  // 2^32 / kYRange
  if (!(z > 0.f)) return 0u;
  if (z >= 4294967040.0f) return 0xFFFFFFFFu;
  return static_cast<uint32_t>(z);
}

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__global__ void select_clear_kernel(uint32_t* __restrict__ hist, RowInfo* __restrict__ info) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kNB; i += blockDim.x) hist[static_cast<size_t>(r) * kNB + i] = 0u;
  if (threadIdx.x == 0) info[r] = RowInfo{0, 0, 0, 0, 0u, 0u, 0u, 0};
}

template <bool FROM_LOGITS>
__global__ __launch_bounds__(kThreads) void select_hist_kernel(
    const float* __restrict__ logits, const double* __restrict__ lse2,
    const float* __restrict__ ytop, const float* __restrict__ scores_in,
    float* __restrict__ scores_out, uint32_t* __restrict__ ukey, uint32_t* __restrict__ hist,
    RowInfo* __restrict__ info, int64_t S, int64_t Spad, int T, int Hkv, int topk, int w,
    int chunk, int nchunk, int do_select) {
  __shared__ uint32_t lh[kNB];
  __shared__ float lse2f[kG];
  __shared__ int is_last;
  const int r = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t n_ctx = static_cast<int64_t>(P) + 1;
  const int64_t first = max(static_cast<int64_t>(0), static_cast<int64_t>(P) - w + 1);
  for (int i = tid; i < kNB; i += kThreads) lh[i] = 0u;
  float ybase = 0.f;
  if (FROM_LOGITS) {
    if (tid < kG) lse2f[tid] = static_cast<float>(lse2[static_cast<size_t>(r) * kG + tid]);
    ybase = ytop[r] - kYRange;
  }
  __syncthreads();
  const int64_t j0 = static_cast<int64_t>(c) * chunk;
  const int64_t j1 = min(S, j0 + chunk);
  const size_t rs = static_cast<size_t>(r) * S;
  for (int64_t j = j0 + tid; j < j1; j += kThreads) {
    if (j >= n_ctx) {
      if (scores_out) scores_out[rs + j] = 0.f;
      continue;
    }
    uint32_t u;
    if (FROM_LOGITS) {
      const float* lr = logits + static_cast<size_t>(r) * kG * Spad + j;
      float y = lr[0] - lse2f[0];
#pragma unroll
      for (int h = 1; h < kG; ++h) y = fmaxf(y, lr[static_cast<size_t>(h) * Spad] - lse2f[h]);
      if (scores_out) scores_out[rs + j] = exp2f(y);
      u = key_from_log2(y, ybase);
    } else {
      u = ordered_u32(scores_in[rs + j]);
    }
    if (do_select && j < first) {
      ukey[static_cast<size_t>(r) * Spad + j] = u;
      atomicAdd(&lh[u >> kBinShift], 1u);
    }
  }
  if (!do_select) return;
  __syncthreads();
  uint32_t* hr = hist + static_cast<size_t>(r) * kNB;
  for (int i = tid; i < kNB; i += kThreads)
    if (lh[i]) atomicAdd(&hr[i], lh[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = (atomicAdd(&info[r].arrive, 1u) == static_cast<uint32_t>(nchunk - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  // ---- the last work-group of the row: locate the k-th largest key's bin
  const int64_t n_cand = first;
  if (tid < 64) {
    int mode = kModeNormal;
    if (topk <= 0 || n_cand == 0) mode = kModeNone;
    else if (n_cand <= topk) mode = kModeAll;
    int bstar = 0, n_cert = 0, n_unc = 0;
    const int band = FROM_LOGITS ? 1 : 0;
    if (mode == kModeNormal) {
      // lane l owns bins [kNB-32(l+1), kNB-32l), scanned from the top
      const int lane = tid;
      uint32_t lane_sum = 0;
      for (int i = 0; i < 32; ++i)
        lane_sum += __hip_atomic_load(&hr[kNB - 1 - 32 * lane - i], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      uint32_t incl = lane_sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const uint32_t excl = incl - lane_sum;
      const uint64_t hit = __ballot(incl >= static_cast<uint32_t>(topk));
      const int owner = hit ? __builtin_ctzll(hit) : 63;
      if (lane == owner) {
        uint32_t above = excl;
        int bs = kNB - 1 - 32 * lane;
        const int bs_end = bs - 31;
        uint32_t cb = 0;
        for (;; --bs) {
          cb = __hip_atomic_load(&hr[bs], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (above + cb >= static_cast<uint32_t>(topk) || bs == bs_end) break;
          above += cb;
        }
        bstar = bs;
        n_cert = static_cast<int>(above);  // keys in bins above b*
        n_unc = static_cast<int>(cb);
      }
      bstar = __shfl(bstar, owner);
      n_cert = __shfl(n_cert, owner);
      n_unc = __shfl(n_unc, owner);
      if (band) {
        // widen the band by one bin on each side
        const uint32_t hu = (bstar + 1 < kNB)
                                ? __hip_atomic_load(&hr[bstar + 1], __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : 0u;
        const uint32_t hd = (bstar - 1 >= 0)
                                ? __hip_atomic_load(&hr[bstar - 1], __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : 0u;
        n_cert -= static_cast<int>(hu);
        n_unc += static_cast<int>(hu + hd);
      }
    }
    if (tid == 0) {
      info[r].bstar = bstar;
      info[r].n_cert = n_cert;
      info[r].n_unc = n_unc;
      info[r].mode = mode;
      info[r].band = band;
    }
  }
}

__global__ __launch_bounds__(kThreads) void select_compact_kernel(
    const uint32_t* __restrict__ ukey, RowInfo* __restrict__ info, int32_t* __restrict__ cert,
    int32_t* __restrict__ unc, int64_t S, int64_t Spad, int T, int Hkv, int w, int chunk,
    int capk) {
  const int r = blockIdx.y;
  const int c = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = max(static_cast<int64_t>(0), static_cast<int64_t>(P) - w + 1);
  const int mode = info[r].mode;
  if (mode == kModeNone) return;
  const int bstar = info[r].bstar;
  const int band = info[r].band;
  const int64_t j0 = static_cast<int64_t>(c) * chunk;
  const int64_t j1 = min(first, j0 + chunk);
  if (j0 >= j1) return;
  const uint32_t* ur = ukey + static_cast<size_t>(r) * Spad;
  // every lane of a wave runs the same number of iterations
  const int64_t wave_base = j0 + (threadIdx.x & ~63);
  for (int64_t jb = wave_base; jb < j1; jb += kThreads) {
    const int64_t j = jb + lane;
    bool is_cert = false, is_unc = false;
    if (j < j1) {
      if (mode == kModeAll) {
        is_cert = true;
      } else {
        const int b = static_cast<int>(ur[j] >> kBinShift);
        is_cert = b > bstar + band;
        is_unc = (b >= bstar - band) && (b <= bstar + band);
      }
    }
    const uint64_t mc = __ballot(is_cert);
    if (mc) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&info[r].cert_count, static_cast<uint32_t>(__popcll(mc)));
      base = __shfl(base, 0);
      if (is_cert) cert[static_cast<size_t>(r) * capk + base + lane_prefix(mc)] = static_cast<int32_t>(j);
    }
    const uint64_t mu = __ballot(is_unc);
    if (mu) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&info[r].unc_count, static_cast<uint32_t>(__popcll(mu)));
      base = __shfl(base, 0);
      const uint32_t slot = base + lane_prefix(mu);
      if (is_unc && slot < static_cast<uint32_t>(kUncCap))
        unc[static_cast<size_t>(r) * kUncCap + slot] = static_cast<int32_t>(j);
    }
  }
}

// ---- exact importance of one key (float64), from the bf16 query and key
struct ExactCtx {
  const double* qd;     // LDS [kG][kD] float64 queries
  const double* lse2;   // LDS [kG] base-2 log-sum-exp
  const u16* kr;        // key rows of this row's KV head
  double c2;            // scale * log2(e)
};

__device__ double exact_log2_importance(const ExactCtx& e, int64_t j) {
  double acc[kG];
#pragma unroll
  for (int h = 0; h < kG; ++h) acc[h] = 0.0;
  const u16* kj = e.kr + j * kD;
  for (int d0 = 0; d0 < kD; d0 += 8) {
    const u32x4 raw = load_u32x4(kj + d0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t word = raw[t >> 1];
      const double kv = static_cast<double>(
          __uint_as_float((t & 1) ? (word & 0xFFFF0000u) : (word << 16)));
#pragma unroll
      for (int h = 0; h < kG; ++h) acc[h] = fma(e.qd[h * kD + d0 + t], kv, acc[h]);
    }
  }
  double y = -INFINITY;
#pragma unroll
  for (int h = 0; h < kG; ++h) y = fmax(y, e.c2 * acc[h] - e.lse2[h]);
  return y;
}

struct Cand {
  uint64_t key;  // larger = better
  int32_t idx;   // ties: lower index first
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

__device__ void bitonic_sort_ints(int32_t* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int32_t x = a[lo], y = a[hi];
        if ((y < x) == up) {
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

template <bool FROM_LOGITS>
__global__ __launch_bounds__(kThreads) void select_finish_kernel(
    const RowInfo* __restrict__ info, const int32_t* __restrict__ cert,
    const int32_t* __restrict__ unc, const uint32_t* __restrict__ ukey,
    const float* __restrict__ scores_in, const u16* __restrict__ q, const u16* __restrict__ k,
    const double* __restrict__ lse2g, double c2, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ nsel_out, int64_t S, int64_t Spad, int T, int Hkv, int topk, int w,
    int capk, int cap) {
  __shared__ int32_t sel[kMaxSel];
  __shared__ Cand cands[kUncCap];
  __shared__ double qd[FROM_LOGITS ? kG * kD : 1];
  __shared__ double l2s[kG];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t s_sel_count;
  __shared__ uint64_t s_thr_hi;
  __shared__ uint32_t s_thr_lo;
  __shared__ uint32_t s_need;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = row_pos(r, T, Hkv, S);
  const int64_t first = max(static_cast<int64_t>(0), static_cast<int64_t>(P) - w + 1);
  const RowInfo inf = info[r];
  const int b = r / (T * Hkv);
  const int g = r % Hkv;
  const size_t kvrow = static_cast<size_t>(b) * Hkv + g;

  int n_keep = 0;  // selected older keys
  int r_take = 0;  // of which from the uncertain band
  if (inf.mode == kModeAll) {
    n_keep = static_cast<int>(first);
  } else if (inf.mode == kModeNormal) {
    n_keep = topk;
    r_take = topk - inf.n_cert;
  }
  const int n_cert = n_keep - r_take;
  for (int i = tid; i < n_cert; i += kThreads) sel[i] = cert[static_cast<size_t>(r) * capk + i];

  ExactCtx ex{};
  if (FROM_LOGITS && r_take > 0) {
    const u16* qr = q + static_cast<size_t>(r) * kG * kD;
    for (int i = tid; i < kG * kD; i += kThreads) qd[i] = static_cast<double>(bf16_bits_to_f32(qr[i]));
    if (tid < kG) l2s[tid] = lse2g[static_cast<size_t>(r) * kG + tid];
    __syncthreads();
    ex = ExactCtx{qd, l2s, k + kvrow * static_cast<size_t>(S) * kD, c2};
  }

  if (r_take > 0) {
    const int n_unc = static_cast<int>(inf.unc_count);
    if (n_unc <= kUncCap) {
      // ---- fast path: rank the whole band in LDS
      const int n2 = next_pow2(n_unc);
      for (int i = tid; i < n2; i += kThreads) {
        Cand cnd{0ull, 0x7FFFFFFF};
        if (i < n_unc) {
          const int32_t j = unc[static_cast<size_t>(r) * kUncCap + i];
          cnd.idx = j;
          if (FROM_LOGITS)
            cnd.key = ordered_u64(exact_log2_importance(ex, j));
          else
            cnd.key = ordered_u32(scores_in[static_cast<size_t>(r) * S + j]);
        }
        cands[i] = cnd;
      }
      __syncthreads();
      bitonic_sort_cands(cands, n2);
      for (int i = tid; i < r_take; i += kThreads) sel[n_cert + i] = cands[i].idx;
    } else {
      // ---- slow path: exact radix select over the band, scanning the row.
      // Composite key: 64-bit value, then 32-bit (~index) so lower indices win.
      const uint32_t* ur = ukey + static_cast<size_t>(r) * Spad;
      const int lo_bin = inf.bstar - inf.band, hi_bin = inf.bstar + inf.band;
      uint64_t thr_hi = 0, mask_hi = 0;
      uint32_t thr_lo = 0, mask_lo = 0;
      uint32_t need = static_cast<uint32_t>(r_take);
      for (int pass = 0; pass < 12; ++pass) {
        for (int i = tid; i < 256; i += kThreads) h256[i] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < first; j += kThreads) {
          const int bn = static_cast<int>(ur[j] >> kBinShift);
          if (bn < lo_bin || bn > hi_bin) continue;
          const uint64_t vhi = FROM_LOGITS ? ordered_u64(exact_log2_importance(ex, j))
                                           : static_cast<uint64_t>(ordered_u32(
                                                 scores_in[static_cast<size_t>(r) * S + j]));
          const uint32_t vlo = ~static_cast<uint32_t>(j);
          if ((vhi & mask_hi) != thr_hi || (vlo & mask_lo) != thr_lo) continue;
          const uint32_t digit = pass < 8 ? static_cast<uint32_t>(vhi >> (56 - 8 * pass)) & 255u
                                          : (vlo >> (24 - 8 * (pass - 8))) & 255u;
          atomicAdd(&h256[digit], 1u);
        }
        __syncthreads();
        if (tid == 0) {
          uint32_t above = 0;
          int dsel = 255;
          for (; dsel > 0; --dsel) {
            if (above + h256[dsel] >= need) break;
            above += h256[dsel];
          }
          s_need = need - above;
          if (pass < 8) {
            s_thr_hi = thr_hi | (static_cast<uint64_t>(dsel) << (56 - 8 * pass));
            s_thr_lo = thr_lo;
          } else {
            s_thr_hi = thr_hi;
            s_thr_lo = thr_lo | (static_cast<uint32_t>(dsel) << (24 - 8 * (pass - 8)));
          }
        }
        __syncthreads();
        need = s_need;
        thr_hi = s_thr_hi;
        thr_lo = s_thr_lo;
        if (pass < 8) mask_hi |= 255ull << (56 - 8 * pass);
        else mask_lo |= 255u << (24 - 8 * (pass - 8));
        __syncthreads();
      }
      // collect every band key whose composite is >= the threshold composite
      if (tid == 0) s_sel_count = 0u;
      __syncthreads();
      for (int64_t j = tid; j < first; j += kThreads) {
        const int bn = static_cast<int>(ur[j] >> kBinShift);
        if (bn < lo_bin || bn > hi_bin) continue;
        const uint64_t vhi = FROM_LOGITS ? ordered_u64(exact_log2_importance(ex, j))
                                         : static_cast<uint64_t>(ordered_u32(
                                               scores_in[static_cast<size_t>(r) * S + j]));
        const uint32_t vlo = ~static_cast<uint32_t>(j);
        if (vhi > thr_hi || (vhi == thr_hi && vlo >= thr_lo)) {
          const uint32_t slot = atomicAdd(&s_sel_count, 1u);
          if (slot < static_cast<uint32_t>(r_take)) sel[n_cert + slot] = static_cast<int32_t>(j);
        }
      }
    }
  }
  __syncthreads();
  // ---- emit: selected older keys ascending, then the window
  const int n2 = next_pow2(max(n_keep, 1));
  for (int i = n_keep + tid; i < n2; i += kThreads) sel[i] = 0x7FFFFFFF;
  __syncthreads();
  bitonic_sort_ints(sel, n2);
  const int64_t n_win = static_cast<int64_t>(P) - first + 1;
  const int n_total = n_keep + static_cast<int>(n_win);
  int32_t* out = idx_out + static_cast<size_t>(r) * cap;
  for (int i = tid; i < cap; i += kThreads) {
    int32_t val = -1;
    if (i < n_keep) val = sel[i];
    else if (i < n_total) val = static_cast<int32_t>(first + (i - n_keep));
    out[i] = val;
  }
  if (tid == 0) nsel_out[r] = n_total;
}

}  // namespace

hipError_t launch_select_clear(const Plan& p, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  hipLaunchKernelGGL(select_clear_kernel, dim3(p.R), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(w + p.off_hist),
                     reinterpret_cast<RowInfo*>(w + p.off_info));
  return hipGetLastError();
}

hipError_t launch_select_hist(const Plan& p, bool from_logits, const float* scores_in,
                              float* scores_out, bool do_select, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  dim3 grid(p.sel_nchunk, p.R);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, st,
                       reinterpret_cast<const float*>(w + p.off_logits),
                       reinterpret_cast<const double*>(w + p.off_lse2),
                       reinterpret_cast<const float*>(w + p.off_ytop), scores_in, scores_out,
                       reinterpret_cast<uint32_t*>(w + p.off_ukey),
                       reinterpret_cast<uint32_t*>(w + p.off_hist),
                       reinterpret_cast<RowInfo*>(w + p.off_info), p.S, p.Spad, p.T, p.Hkv, p.k,
                       p.w, p.sel_chunk, p.sel_nchunk, do_select ? 1 : 0);
  };
  if (from_logits) args(select_hist_kernel<true>);
  else args(select_hist_kernel<false>);
  return hipGetLastError();
}

hipError_t launch_select_compact(const Plan& p, bool /*from_logits*/, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  dim3 grid(p.sel_nchunk, p.R);
  hipLaunchKernelGGL(select_compact_kernel, grid, dim3(kThreads), 0, st,
                     reinterpret_cast<const uint32_t*>(w + p.off_ukey),
                     reinterpret_cast<RowInfo*>(w + p.off_info),
                     reinterpret_cast<int32_t*>(w + p.off_cert),
                     reinterpret_cast<int32_t*>(w + p.off_unc), p.S, p.Spad, p.T, p.Hkv, p.w,
                     p.sel_chunk, ((p.k + 63) / 64) * 64);
  return hipGetLastError();
}

hipError_t launch_select_finish(const Plan& p, bool from_logits, const float* scores_in,
                                const u16* q, const u16* k, int32_t* idx, int32_t* n_sel,
                                void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(p.R), dim3(kThreads), 0, st,
                       reinterpret_cast<const RowInfo*>(w + p.off_info),
                       reinterpret_cast<const int32_t*>(w + p.off_cert),
                       reinterpret_cast<const int32_t*>(w + p.off_unc),
                       reinterpret_cast<const uint32_t*>(w + p.off_ukey), scores_in, q, k,
                       reinterpret_cast<const double*>(w + p.off_lse2), c2, idx, n_sel, p.S,
                       p.Spad, p.T, p.Hkv, p.k, p.w, ((p.k + 63) / 64) * 64, p.cap);
  };
  if (from_logits) args(select_finish_kernel<true>);
  else args(select_finish_kernel<false>);
  return hipGetLastError();
}

}  // namespace hs2
