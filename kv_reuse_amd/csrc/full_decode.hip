// Full-attention layer of a Cross-Decoder group, decode (one query token per row).
//
// The group's full layer attends over the whole shared KV cache and its
// attention is what the selection is computed from (news page
// "两天两连更：小米提前亮出V3底牌", section "两级KV共享：让模型少跑一半", item
// KV Reuse; video page "小米 MiMo-V3 HySparse2 架构：读长文省一半", section
// "HySparse2 的解法：两派都用，还改了流程").
//
// Design (gfx950):
//  * A row is (batch, KV head): the 8 query heads of the GQA group share one
//    K/V stream.  The context is cut into splits; one work-group of 4 waves
//    streams one split, each wave taking every 4th tile of 32 keys, so the
//    work-group sweeps its split front to back.
//  * S^T = K . Q^T on MFMA 16x16x32 bf16: K rows are the A operand (16 keys per
//    MFMA, loaded straight from HBM with 16-byte non-temporal loads), the
//    group's queries padded to 16 heads are the B operand.  Half of the MFMA
//    columns are padding; the kernel is bound by HBM bytes, not by MFMA issue.
//  * O^T = V^T . P^T on MFMA: P^T comes out of the S^T accumulators already in
//    the B-operand lane layout (head = lane % 16), so only V needs a transpose;
//    it goes through a per-wave LDS tile (272-byte row pitch) and comes back
//    transposed with two ds_read_b64_tr_b16 per MFMA operand.
//  * Online softmax in base 2 with the running max rounded up to an integer:
//    every rescale factor is an exact power of two, and the normaliser l is
//    accumulated in float64, so the only error left in log-sum-exp comes from
//    the float32 logits themselves.
//  * The only per-key output is, for every subtile of 16 keys and every head,
//    the largest float32 base-2 logit (2 bytes per key row next to its 512
//    bytes of K/V).  Once lse is known this bounds every key's importance from
//    above, and the bound is attained by one of the subtile's own keys; the
//    selection uses that to find the few subtiles that can hold selected keys.
//    (Writing all logits, 32 bytes per key row, cost about 45% of the kernel's
//    time on MI355X: the write stream slows the 2 GiB read stream far more than
//    its byte count.)
//  * The next tile's K/V loads are issued before the current tile is processed
//    (two register buffers), so each wave keeps 16 KB of HBM reads in flight.

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;       // keys per wave iteration
constexpr int kVPitch = 136;    // u16 per V row in LDS: 272 bytes
constexpr int kStageKeys = 16384;  // splits up to this many keys stage their maxima in LDS

struct KVTile {
  bf16x8 ka[2][4];  // K as A operand: 2 sub-tiles of 16 keys x 4 chunks of 32 dims
  u32x4 vv[8];      // V: 8 pieces of 16 bytes of the 32 x 128 tile, natural layout
};

struct SoftmaxState {
  f32x4 o[8];  // O^T: d = 16*nb + 4*grp + i, head = lane % 16
  float m;     // running max (integer-valued), base 2
  double l;    // running sum of 2^(s - m) over this lane's keys
};

__device__ __forceinline__ void load_tile(KVTile& t, const u16* __restrict__ kr,
                                          const u16* __restrict__ vr, int64_t t0,
                                          int64_t key_last, int col, int grp) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    int64_t key = t0 + 16 * mt + col;
    key = key < key_last ? key : key_last;
    const u16* base = kr + key * kD + 8 * grp;
#pragma unroll
    for (int c = 0; c < 4; ++c) t.ka[mt][c] = as_bf16x8(load_u32x4_nt(base + 32 * c));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t key = t0 + grp + 4 * i;
    key = key < key_last ? key : key_last;
    t.vv[i] = load_u32x4_nt(vr + key * kD + 8 * col);
  }
}

// S^T for one tile: lane (col, grp) gets the base-2 logits of head col for keys
// t0 + 16*mt + 4*grp + i in sv[4*mt + i] (-inf past key_end).
__device__ __forceinline__ void tile_logits(const bf16x8 (&ka)[2][4], const bf16x8 (&qb)[4],
                                            int64_t t0, int64_t key_end, int grp, float c2_hi,
                                            float c2_lo, float (&sv)[8]) {
  f32x4 sacc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) sacc[mt] = mfma_16x16x32(ka[mt][c], qb[c], sacc[mt]);
  }
  // the scale is applied as a two-term product so that its float32 rounding
  // does not bias every logit of the row the same way
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = t0 + 16 * mt + 4 * grp + i;
      const float a = sacc[mt][i];
      sv[mt * 4 + i] = key < key_end ? fmaf(a, c2_hi, a * c2_lo) : -INFINITY;
    }
}

__device__ __forceinline__ void process_tile(const KVTile& t, SoftmaxState& st,
                                             const bf16x8 (&qb)[4], u16* __restrict__ vw,
                                             float* __restrict__ stmax_row, int64_t st_base,
                                             int64_t t0, int64_t key_end, int col, int grp,
                                             float c2_hi, float c2_lo) {
  float sv[8];
  tile_logits(t.ka, qb, t0, key_end, grp, c2_hi, c2_lo, sv);
  // per-subtile (16 keys) maxima of each head: lanes of one head are col + 16*grp
  float m0 = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  float m1 = fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7]));
  // one row swap serves both: rows 0 and 2 pair m0 across rows 0|1 and 2|3,
  // rows 1 and 3 pair m1; the second swap then joins 0-1 with 2-3, leaving
  // m0's subtile maximum in rows 0 and 2 and m1's in rows 1 and 3
  float mx;
  {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m0), __float_as_uint(m1), false, false);
    mx = max_xor32(fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
  }
  // subtile t0/16 + mt, head col: 64 contiguous bytes per tile (grp 0 and 1);
  // stmax_row is either the row's global array or the work-group's LDS stage
  // (then indexed from the split's first subtile)
  if (col < kG && grp < 2 && t0 + 16 * grp < key_end)
    stmax_row[(t0 / 16 + grp - st_base) * kG + col] = mx;   // row grp: subtile grp
  // ---- online softmax (per head = per lane % 16); the tile's maximum joins
  // the two subtiles' (rows 0|1 and 2|3)
  const float tm = max_xor16(mx);
  const float m_new = fmaxf(st.m, ceilf(tm));
  const float alpha = (st.m == -INFINITY) ? 0.f : ldexpf(1.f, static_cast<int>(st.m - m_new));
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(sv[e] - m_new);
  const float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  st.l = st.l * static_cast<double>(alpha) + static_cast<double>(ps);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) st.o[nb] *= alpha;
  st.m = m_new;
  // ---- V tile to LDS (natural layout), then V^T operands by transpose reads
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(vw + (grp + 4 * i) * kVPitch + 8 * col) = t.vv[i];
  lds_fence_wave();
  // P^T as B operand: lane holds keys {4grp+i} of sub-tile 0 then sub-tile 1
  const u32x4 pp{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                 pack_bf16x2(p[6], p[7])};
  const bf16x8 pb = as_bf16x8(pp);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    st.o[nb] = mfma_16x16x32(lds_vt_operand(vw, kVPitch, nb, col, grp), pb, st.o[nb]);
}

__device__ __forceinline__ void load_q_operand(const u16* __restrict__ qr, int col, int grp,
                                               bf16x8 (&qb)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qb[c] = col < kG ? as_bf16x8(load_u32x4(qr + col * kD + 32 * c + 8 * grp))
                     : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
}

__global__ __launch_bounds__(kWaves * 64, 2) void full_decode_split_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    float* __restrict__ stmax, float* __restrict__ part_m, double* __restrict__ part_l,
    float* __restrict__ part_o, int64_t S, int64_t Spad, int kps, int n_split, float c2_hi,
    float c2_lo, int64_t kvp) {
  // V tiles during the stream; reused for the cross-wave merge afterwards
  __shared__ __align__(16) unsigned char smem[kWaves * kTile * kVPitch * 2];
  __shared__ float sm_m[kWaves][kG];
  __shared__ double sm_l[kWaves][kG];
  // the split's subtile maxima, written to HBM in one burst at the end (when
  // the split is at most kStageKeys keys)
  __shared__ __align__(16) float st_stage[kStageKeys / 16 * kG];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int r = blockIdx.y;
  const int s = blockIdx.x;
  const int64_t key_begin = static_cast<int64_t>(s) * kps;
  const int64_t key_end = min(S, key_begin + kps);
  const u16* kr = k + static_cast<size_t>(r) * kvp * kD;
  const u16* vr = v + static_cast<size_t>(r) * kvp * kD;
  float* stmax_row = stmax + static_cast<size_t>(r) * (Spad / 16) * kG;
  const bool staged = kps <= kStageKeys;
  float* st_dst = staged ? st_stage : stmax_row;
  const int64_t st_base = staged ? key_begin / 16 : 0;
  u16* vw = reinterpret_cast<u16*>(smem) + wave * kTile * kVPitch;

  bf16x8 qb[4];
  load_q_operand(q + static_cast<size_t>(r) * kG * kD, col, grp, qb);

  SoftmaxState st;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) st.o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.0;

  const int64_t stride = kWaves * kTile;
  const int64_t key_last = key_end - 1;
  int64_t t0 = key_begin + wave * kTile;
  if (t0 < key_end) {
    KVTile ta, tb;
    load_tile(ta, kr, vr, t0, key_last, col, grp);
    while (true) {
      int64_t t1 = t0 + stride;
      bool more = t1 < key_end;
      if (more) load_tile(tb, kr, vr, t1, key_last, col, grp);
      process_tile(ta, st, qb, vw, st_dst, st_base, t0, key_end, col, grp, c2_hi, c2_lo);
      if (!more) break;
      t0 = t1;
      t1 = t0 + stride;
      more = t1 < key_end;
      if (more) load_tile(ta, kr, vr, t1, key_last, col, grp);
      process_tile(tb, st, qb, vw, st_dst, st_base, t0, key_end, col, grp, c2_hi, c2_lo);
      if (!more) break;
      t0 = t1;
    }
  }
  st.l = sum_rows(st.l);

  __syncthreads();  // all waves done with their V tiles (and the stage)
  if (staged) {
    // subtiles [key_begin/16, ceil(key_end/16)) of this split, 16 bytes a thread
    const int n4 = static_cast<int>((key_end - key_begin + 15) / 16) * kG / 4;
    float* dst = stmax_row + (key_begin / 16) * kG;
    for (int i = threadIdx.x; i < n4; i += blockDim.x)
      *reinterpret_cast<f32x4*>(dst + 4 * i) = *reinterpret_cast<const f32x4*>(st_stage + 4 * i);
  }
  float* sm_o = reinterpret_cast<float*>(smem);  // [kWaves][kG][kD]
  if (col < kG) {
    if (grp == 0) {
      sm_m[wave][col] = st.m;
      sm_l[wave][col] = st.l;
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[(wave * kG + col) * kD + 16 * nb + 4 * grp + i] = st.o[nb][i];
  }
  __syncthreads();
  const size_t pbase = static_cast<size_t>(r) * n_split + s;
  for (int idx = threadIdx.x; idx < kG * kD; idx += blockDim.x) {
    const int h = idx >> 7, d = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float acc = 0.f;
    double L = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][h];
      if (mw != -INFINITY) {
        const int e = static_cast<int>(mw - M);
        acc += sm_o[(w * kG + h) * kD + d] * ldexpf(1.f, e);
        L += sm_l[w][h] * ldexp(1.0, e);
      }
    }
    part_o[(pbase * kG + h) * kD + d] = acc;
    if (d == 0) {
      part_m[pbase * kG + h] = M;
      part_l[pbase * kG + h] = L;
    }
  }
}

// Merge of the splits, one work-group of 1024 threads per (head, row): the
// maximum M of the split maxima, L = sum_s l_s 2^(m_s - M) in float64 (fixed
// order), O = sum_s O_s 2^(m_s - M) / L (eight partial sums of 128 lanes,
// then in order).  Writes the output row (bf16), lse (natural log, when
// non-null), lse2 (float64, base 2) and the head's bound on log2 importance,
// max_j s2_j - lse2 = -log2(L).  It also clears the row's selection state.
constexpr int kCmbThreads = 1024;
__global__ __launch_bounds__(kCmbThreads) void full_combine_kernel(
    const float* __restrict__ part_m, const double* __restrict__ part_l,
    const float* __restrict__ part_o, int n_split, u16* __restrict__ out,
    float* __restrict__ lse_out, double* __restrict__ lse2, float* __restrict__ ytop_h,
    uint32_t* __restrict__ hist, RowInfo* __restrict__ info) {
  __shared__ float sm[kMaxSplits];
  __shared__ float sf[kMaxSplits];      // 2^(m_s - M)
  __shared__ double sl[kMaxSplits];
  __shared__ float po[8][kD];
  __shared__ float s_M;
  __shared__ double s_L;
  const int h = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x;
  const int d = tid & (kD - 1), part = tid >> 7;
  const size_t rb = static_cast<size_t>(r) * n_split;
  for (int s2 = tid; s2 < n_split; s2 += kCmbThreads) {
    sm[s2] = part_m[(rb + s2) * kG + h];
    sl[s2] = part_l[(rb + s2) * kG + h];
  }
  // fresh selection state for this row (each head clears a share)
  for (int i = tid; i < kNB / kG; i += kCmbThreads)
    hist[static_cast<size_t>(r) * kNB + h * (kNB / kG) + i] = 0u;
  if (h == 0 && tid == 0) info[r] = RowInfo{0u, 0u, 0u, 0u};
  __syncthreads();
  if (tid < 64) {
    float M = -INFINITY;
    for (int s2 = tid; s2 < n_split; s2 += 64) M = fmaxf(M, sm[s2]);
    M = max_xor32(max_xor16(M));
    M = fmaxf(M, dpp_f32<0x128>(M));   // row_ror:8, the other half of the row
    M = fmaxf(M, dpp_f32<0x141>(M));   // row_half_mirror, the other quad of 8
    M = fmaxf(M, dpp_f32<0x4E>(M));    // lane ^ 2
    M = fmaxf(M, dpp_f32<0xB1>(M));    // lane ^ 1
    // L in a fixed order: lane-strided partial sums, then the tree of a lane
    // ^ 32, ^ 16, ^ 8, ^ 4, ^ 2, ^ 1 butterfly.  After the ^ 8 step the row
    // repeats with period 8, so a rotation by 4 within the row reads lane ^ 4.
    double L = 0.0;
    for (int s2 = tid; s2 < n_split; s2 += 64)
      if (sm[s2] != -INFINITY) L += sl[s2] * ldexp(1.0, static_cast<int>(sm[s2] - M));
    L = sum_rows_f64(L);
    L += dpp_f64<0x128>(L);   // row_ror:8: lane ^ 8
    L += dpp_f64<0x124>(L);   // row_ror:4: lane ^ 4 (period 8)
    L += dpp_f64<0x4E>(L);    // lane ^ 2
    L += dpp_f64<0xB1>(L);    // lane ^ 1
    if (tid == 0) {
      s_M = M;
      s_L = L;
    }
  }
  __syncthreads();
  const float M = s_M;
  for (int s2 = tid; s2 < n_split; s2 += kCmbThreads)
    sf[s2] = sm[s2] == -INFINITY ? 0.f : ldexpf(1.f, static_cast<int>(sm[s2] - M));
  __syncthreads();
  // O: part p sums splits p, p + 8, ... (loads issued 8 at a time)
  float acc = 0.f;
  const float* po_base = part_o + (rb * kG + h) * kD + d;
  for (int s0 = part; s0 < n_split; s0 += 8 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s2 = s0 + 8 * u;
      v[u] = s2 < n_split ? po_base[static_cast<size_t>(s2) * kG * kD] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s2 = s0 + 8 * u;
      if (s2 < n_split) acc += v[u] * sf[s2];
    }
  }
  po[part][d] = acc;
  __syncthreads();
  if (part == 0) {
    float o = 0.f;
#pragma unroll
    for (int p2 = 0; p2 < 8; ++p2) o += po[p2][d];
    const double L = s_L;
    out[(static_cast<size_t>(r) * kG + h) * kD + d] = f32_to_bf16_rne(o * static_cast<float>(1.0 / L));
    if (d == 0) {
      const double l2 = static_cast<double>(M) + log2(L);
      lse2[static_cast<size_t>(r) * kG + h] = l2;
      if (lse_out) lse_out[static_cast<size_t>(r) * kG + h] = static_cast<float>(l2 * M_LN2);
      // every logit of this head is <= M, so its base-2 log-probability is <= M - lse2
      ytop_h[static_cast<size_t>(r) * kG + h] = static_cast<float>(-log2(L));
    }
  }
}

// Optional per-key importance for the caller (the step itself never needs all
// of them): recompute the logits tile by tile on MFMA and write
// max_h 2^(s2_h - lse2_h); entries past P are 0.  Reads K once more.
__global__ __launch_bounds__(256) void full_scores_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const double* __restrict__ lse2,
    float* __restrict__ scores, int64_t S, int kps, float c2_hi, float c2_lo, int64_t kvp) {
  __shared__ float l2f[kG];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int r = blockIdx.y;
  const int64_t key_begin = static_cast<int64_t>(blockIdx.x) * kps;
  const int64_t key_end = min(S, key_begin + kps);
  if (threadIdx.x < kG)
    l2f[threadIdx.x] = static_cast<float>(lse2[static_cast<size_t>(r) * kG + threadIdx.x]);
  __syncthreads();
  bf16x8 qb[4];
  load_q_operand(q + static_cast<size_t>(r) * kG * kD, col, grp, qb);
  const u16* kr = k + static_cast<size_t>(r) * kvp * kD;
  float* sr = scores + static_cast<size_t>(r) * S;
  for (int64_t t0 = key_begin + wave * kTile; t0 < key_end; t0 += 4 * kTile) {
    bf16x8 ka[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      int64_t key = t0 + 16 * mt + col;
      key = key < key_end - 1 ? key : key_end - 1;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        ka[mt][c] = as_bf16x8(load_u32x4(kr + key * kD + 8 * grp + 32 * c));
    }
    float sv[8];
    tile_logits(ka, qb, t0, key_end, grp, c2_hi, c2_lo, sv);
    // importance per key: max over the 8 real heads (lanes col 0..7 of a group)
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float yv = col < kG ? sv[e] - l2f[col] : -INFINITY;
      yv = fmaxf(yv, __shfl_xor(yv, 1));
      yv = fmaxf(yv, __shfl_xor(yv, 2));
      yv = fmaxf(yv, __shfl_xor(yv, 4));
      y[e] = yv;
    }
    if (col == 0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t key = t0 + 16 * mt + 4 * grp + i;
          if (key < key_end) sr[key] = exp2f(y[4 * mt + i]);
        }
    }
  }
}

}  // namespace

hipError_t launch_full_decode_split(const Plan& p, const u16* q, const u16* k, const u16* v,
                                    void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;  // scale * log2(e)
  const float c2_hi = static_cast<float>(c2);
  const float c2_lo = static_cast<float>(c2 - static_cast<double>(c2_hi));
  dim3 grid(p.n_split, p.R);
  hipLaunchKernelGGL(full_decode_split_kernel, grid, dim3(kWaves * 64), 0, st, q, k, v,
                     reinterpret_cast<float*>(w + p.off_stmax),
                     reinterpret_cast<float*>(w + p.off_part_m),
                     reinterpret_cast<double*>(w + p.off_part_l),
                     reinterpret_cast<float*>(w + p.off_part_o), p.S, p.Spad, p.kps, p.n_split,
                     c2_hi, c2_lo, p.kvp);
  return hipGetLastError();
}

hipError_t launch_full_combine(const Plan& p, u16* out, float* lse, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  hipLaunchKernelGGL(full_combine_kernel, dim3(kG, p.R), dim3(kCmbThreads), 0, st,
                     reinterpret_cast<const float*>(w + p.off_part_m),
                     reinterpret_cast<const double*>(w + p.off_part_l),
                     reinterpret_cast<const float*>(w + p.off_part_o), p.n_split, out, lse,
                     reinterpret_cast<double*>(w + p.off_lse2),
                     reinterpret_cast<float*>(w + p.off_ytop),
                     reinterpret_cast<uint32_t*>(w + p.off_hist),
                     reinterpret_cast<RowInfo*>(w + p.off_info));
  return hipGetLastError();
}

hipError_t launch_full_scores(const Plan& p, const u16* q, const u16* k, float* scores,
                              void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  const float c2_hi = static_cast<float>(c2);
  const float c2_lo = static_cast<float>(c2 - static_cast<double>(c2_hi));
  hipLaunchKernelGGL(full_scores_kernel, dim3(p.n_split, p.R), dim3(256), 0, st, q, k,
                     reinterpret_cast<const double*>(w + p.off_lse2), scores, p.S, p.kps, c2_hi,
                     c2_lo, p.kvp);
  return hipGetLastError();
}

}  // namespace hs2
