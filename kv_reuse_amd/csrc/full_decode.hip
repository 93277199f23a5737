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
//    Beside it, for each 4-key quad of the subtile, how far the quad's own
//    maximum lies below (one byte per quad and head, rounded down, so the
//    subtile maximum minus it still bounds the quad): the selection re-reads
//    only the quads that can reach its threshold.
//    (Writing all logits, 32 bytes per key row, cost about 45% of the kernel's
//    time on MI355X: the write stream slows the 2 GiB read stream far more than
//    its byte count.)
//  * The next tile's K/V loads are issued before the current tile is processed
//    (two register buffers), so each wave keeps 16 KB of HBM reads in flight.

#include <algorithm>

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;       // keys per wave iteration
constexpr int kVPitch = 136;    // u16 per V row in LDS: 272 bytes
constexpr int kStageKeys = 16384;  // splits up to this many keys stage their maxima in LDS
constexpr int kSubTileKeys = 16;   // keys per stored maximum

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

// The quad's distance below its subtile's maximum in 1/kQuadSteps octave
// steps, rounded down (so never more than the true distance), 255 at most.
__device__ __forceinline__ uint32_t quad_steps(float sub_max, float quad_max) {
  const float d = (sub_max - quad_max) * static_cast<float>(kQuadSteps);
  return static_cast<uint32_t>(__builtin_amdgcn_fmed3f(d, 0.f, 255.f));
}

template <bool kQuads>
__device__ __forceinline__ void process_tile(const KVTile& t, SoftmaxState& st,
                                             const bf16x8 (&qb)[4], u16* __restrict__ vw,
                                             float* __restrict__ stmax_row,
                                             unsigned char* __restrict__ qd_row, int64_t st_base,
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
  // m0 and m1 are quad grp's maxima in subtiles 0 and 1; a row swap of mx
  // gives every lane both subtiles' maxima (rows 0 and 2 hold subtile 0's)
  if (kQuads) {
    const auto sm = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    if (col < kG) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        if (t0 + 16 * mt < key_end)
          qd_row[(t0 / 16 + mt - st_base) * (4 * kG) + grp * kG + col] = static_cast<unsigned char>(
              quad_steps(__uint_as_float(sm[mt]), mt == 0 ? m0 : m1));
      }
    }
  }
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

// kStaged: the split is at most kStageKeys keys and its subtile maxima and
// quad distances go to LDS first.  A template parameter rather than a run-time
// choice, so that their stores are LDS stores: a vector-memory store among the
// stream's loads makes the compiler wait for every load in flight (the counter
// no longer drains in order), which serialises the prefetch with the tile.
// kQuads: the quads' distances are written too (the plan's choice: they pay
// where the selection re-reads many subtiles, and their write stream costs
// the full layer about 1% of its time).  The staged form with them holds
// about 100 KB of LDS, one work-group per CU (the plan launches one per CU).
template <bool kStaged, bool kQuads>
__global__ __launch_bounds__(kWaves * 64, kStaged && kQuads ? 1 : 2) void full_decode_split_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    float* __restrict__ stmax, unsigned char* __restrict__ qdiff, float* __restrict__ part_m,
    double* __restrict__ part_l, float* __restrict__ part_o, int64_t S, int64_t Spad, int kps,
    int n_split, float c2_hi, float c2_lo, int64_t kvp) {
  // V tiles during the stream; reused for the cross-wave merge afterwards
  __shared__ __align__(16) unsigned char smem[kWaves * kTile * kVPitch * 2];
  __shared__ float sm_m[kWaves][kG];
  __shared__ double sm_l[kWaves][kG];
  // the split's subtile maxima, written to HBM in one burst at the end (when
  // the split is at most kStageKeys keys)
  __shared__ __align__(16) float st_stage[kStageKeys / 16 * kG];
  __shared__ __align__(16) unsigned char qd_stage[kQuads ? kStageKeys / 16 * 4 * kG : 16];

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
  constexpr bool staged = kStaged;
  float* st_dst = staged ? st_stage : stmax_row;
  unsigned char* qd_row = qdiff + static_cast<size_t>(r) * (Spad / 16) * (4 * kG);
  unsigned char* qd_dst = staged ? qd_stage : qd_row;
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
    // The next tile is loaded whether or not it exists: past the split every
    // key clamps to key_last, so the wave reads that one row (512 bytes), and
    // with no branch around the loads the compiler does not wait for them
    // before the current tile's MFMAs (it does at the join of a conditional
    // prefetch).
    while (true) {
      int64_t t1 = t0 + stride;
      bool more = t1 < key_end;
      load_tile(tb, kr, vr, t1, key_last, col, grp);
      process_tile<kQuads>(ta, st, qb, vw, st_dst, qd_dst, st_base, t0, key_end, col, grp, c2_hi, c2_lo);
      if (!more) break;
      t0 = t1;
      t1 = t0 + stride;
      more = t1 < key_end;
      load_tile(ta, kr, vr, t1, key_last, col, grp);
      process_tile<kQuads>(tb, st, qb, vw, st_dst, qd_dst, st_base, t0, key_end, col, grp, c2_hi, c2_lo);
      if (!more) break;
      t0 = t1;
    }
  }
  st.l = sum_rows_f64(st.l);

  __syncthreads();  // all waves done with their V tiles (and the stage)
  if (staged) {
    // subtiles [key_begin/16, ceil(key_end/16)) of this split, 16 bytes a thread
    const int n4 = static_cast<int>((key_end - key_begin + 15) / 16) * kG / 4;
    float* dst = stmax_row + (key_begin / 16) * kG;
    for (int i = threadIdx.x; i < n4; i += blockDim.x)
      *reinterpret_cast<f32x4*>(dst + 4 * i) = *reinterpret_cast<const f32x4*>(st_stage + 4 * i);
    // and their quads' distances: 32 bytes per subtile
    if (kQuads) {
      const int n16 = static_cast<int>((key_end - key_begin + 15) / 16) * 2;
      unsigned char* qdst = qd_row + (key_begin / 16) * (4 * kG);
      for (int i = threadIdx.x; i < n16; i += blockDim.x)
        *reinterpret_cast<u32x4*>(qdst + 16 * i) = *reinterpret_cast<const u32x4*>(qd_stage + 16 * i);
    }
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

// ---------------------------------------------------------------- refinement of lse2
//
// lse2 above comes from float32 logits.  The bf16 MFMA's chained float32
// accumulation errs by up to a few units of 2^-24 sum_d |q_d k_d| per logit,
// and even a correctly rounded float32 logit of a large key is off by up to
// 2^-25 |s|.  A key that carries a large share of a head's softmax passes its
// logit error into lse2 at that share, and the selection's float64 ranking
// would shift every importance of that head by it.  So the (key, head) terms
// that carry weight are summed again: in every subtile whose stored maximum
// reaches 2^kDomLog2 of some head's normaliser, each pair whose term
// 2^(sv - lse2) reaches it, sv the very float32 logit the split kernel
// exponentiated, gets the term 2^(y - lse2) instead, y the float64 logit of
// exact bf16 products.  sv is recomputed by the split kernel's own MFMA
// sequence on the same operands, which gives the same bits (the MFMA result of
// an element does not depend on where in the tile it sits); the subtile
// maximum the split kernel stored is checked against it, and a mismatch is
// counted.  The change of a term is 2^(sv - lse2) (e^d - 1), d = (y - sv) ln 2
// below 1e-4 in size, taken as d + d^2 / 2.  What remains is the weighted mean
// of the other terms' logit errors, each term below 2^kDomLog2 of the total,
// in which independent errors average out, and the float32 exponentials and
// partial sums of the kept terms (a few units of 2^-24 of each).

constexpr int kRefThreads = 256;
constexpr int kRefWaves = kRefThreads / 64;

// bf16 bits of a 16-byte group, element t, widened to float64 (exact)
__device__ __forceinline__ double bf16_word_f64(const u32x4& raw, int t) {
  const uint32_t word = raw[t >> 1];
  return static_cast<double>(__uint_as_float((t & 1) ? (word & 0xFFFF0000u) : (word << 16)));
}

// Sum over each group of 8 lanes, in every lane of the group (the pairing of a
// lane ^ 1, ^ 2, ^ 4 butterfly).
__device__ __forceinline__ double group8_sum(double v) {
  v += dpp_f64<0xB1>(v);    // lane ^ 1
  v += dpp_f64<0x4E>(v);    // lane ^ 2
  v += dpp_f64<0x141>(v);   // the other quad of the 8
  return v;
}

// The float64 logit (unscaled dot product) of a bf16 key row and a query row,
// by the 8 lanes of a group: lane j takes dims 16 j .. 16 j + 15 (q_part its
// 16 query values, krow the key row in LDS), then the group's sum.
__device__ __forceinline__ double dot_group8(const double (&q_part)[16], const u16* __restrict__ krow,
                                             int j) {
  const u32x4 r0 = *reinterpret_cast<const u32x4*>(krow + 16 * j);
  const u32x4 r1 = *reinterpret_cast<const u32x4*>(krow + 16 * j + 8);
  double acc = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = fma(q_part[t], bf16_word_f64(r0, t), acc);
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = fma(q_part[8 + t], bf16_word_f64(r1, t), acc);
  return group8_sum(acc);
}

// grid (n_wg, R): work-group w of row r takes the w-th equal share of the row's
// dominant subtiles: the ones the selection's candidate kernel listed (their
// bound reaches the row's cut), region by region in ascending order, then
// every subtile reaching into the window (which that kernel does not see); a
// wave takes one subtile at a time.  Each work-group writes its partial sums
// to part[r][w].
__global__ __launch_bounds__(kRefThreads) void lse_refine_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const float* __restrict__ stmax,
    const double* __restrict__ lse2, const float* __restrict__ cut_row,
    const int32_t* __restrict__ dsub, const uint32_t* __restrict__ dsub_cnt,
    RefinePart* __restrict__ part, int64_t S, int64_t Spad, int w, int cc_chunk, int cc_nchunk,
    int n_wg, float c2_hi, float c2_lo, double c2, int64_t kvp) {
  __shared__ uint32_t pre[kMaxChunks + 1];
  __shared__ int32_t s_ids[kRefThreads];
  __shared__ uint32_t s_wsum[kRefWaves];
  __shared__ __align__(16) u16 s_k[kRefWaves][kSubTileKeys * kD];  // a wave's subtile of K rows
  __shared__ float s_sv[kRefWaves][kSubTileKeys * kG];             // its float32 logits [key][head]
  __shared__ double s_acc[kRefWaves][kG];
  __shared__ uint32_t s_bad[kRefWaves];
  __shared__ float s_cut;
  const int r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int h_l = lane >> 3, j = lane & 7;
  const int64_t first = max(static_cast<int64_t>(0), S - w);
  const int64_t n_sub = (first + kSubTileKeys - 1) / kSubTileKeys;
  const int64_t nst = (S + kSubTileKeys - 1) / kSubTileKeys;
  const u16* qr = q + static_cast<size_t>(r) * kG * kD;
  const u16* kr = k + static_cast<size_t>(r) * kvp * kD;
  const float* stmax_row = stmax + static_cast<size_t>(r) * (Spad / kSubTileKeys) * kG;
  // ---- the row's list: region lengths and their exclusive prefix
  constexpr int kPer = kMaxChunks / kRefThreads;
  uint32_t cl[kPer];
  uint32_t mysum = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = kPer * tid + u;
    cl[u] = c < cc_nchunk ? dsub_cnt[static_cast<size_t>(r) * cc_nchunk + c] : 0u;
    mysum += cl[u];
  }
  uint32_t incl = mysum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wsum[wave] = incl;
  if (tid == 0) s_cut = cut_row[r];
  __syncthreads();
  uint32_t base = incl - mysum;
  for (int w2 = 0; w2 < wave; ++w2) base += s_wsum[w2];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = kPer * tid + u;
    if (c < cc_nchunk) pre[c] = base;
    base += cl[u];
  }
  if (tid == kRefThreads - 1) pre[cc_nchunk] = base;
  __syncthreads();
  const uint32_t n_listed = pre[cc_nchunk];
  const uint32_t n_total = n_listed + static_cast<uint32_t>(nst - n_sub);
  const uint32_t share = (n_total + n_wg - 1) / n_wg;
  const uint32_t e0 = min(n_total, share * blockIdx.x);
  const uint32_t e1 = min(n_total, e0 + share);
  const float cut = s_cut;
  // lane (head h_l, dims 16 j ..): the query part in float64; lane (col, grp)
  // of the MFMA layout: the threshold of head col
  double q_part[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) q_part[t] = static_cast<double>(bf16_bits_to_f32(qr[h_l * kD + 16 * j + t]));
  const double l2h = lse2[static_cast<size_t>(r) * kG + h_l];
  const float thr_h = static_cast<float>(l2h) + cut;
  const float thr_c = col < kG ? static_cast<float>(lse2[static_cast<size_t>(r) * kG + col]) + cut
                               : INFINITY;
  bf16x8 qb[4];
  load_q_operand(qr, col, grp, qb);
  double corr = 0.0;   // lanes j = 0: head h_l's sum, subtile by subtile in list order
  uint32_t n_bad = 0;
  // the split kernel's K operand of a subtile (rows past S repeat the last) and,
  // in lanes (col < 8, grp 0), its stored maximum for head col
  auto load_sub = [&](int64_t sti, bf16x8 (&ka)[4], float& smax) {
    const int64_t key = min(sti * kSubTileKeys + col, S - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) ka[c] = as_bf16x8(load_u32x4(kr + key * kD + 8 * grp + 32 * c));
    smax = col < kG && grp == 0 ? stmax_row[sti * kG + col] : 0.f;
  };
  for (uint32_t b0 = e0; b0 < e1; b0 += kRefThreads) {
    // this round's subtiles, one list entry per thread (the regions of the
    // candidate kernel in order, then the window's subtiles)
    const uint32_t nb = min(static_cast<uint32_t>(kRefThreads), e1 - b0);
    __syncthreads();   // the previous round's ids are read
    if (static_cast<uint32_t>(tid) < nb) {
      const uint32_t e = b0 + tid;
      if (e < n_listed) {
        int lo = 0, hi = cc_nchunk - 1;   // the region of e: the largest c with pre[c] <= e
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= e) lo = mid;
          else hi = mid - 1;
        }
        s_ids[tid] = dsub[(static_cast<size_t>(r) * cc_nchunk + lo) * cc_chunk + (e - pre[lo])];
      } else {
        s_ids[tid] = static_cast<int32_t>(n_sub + (e - n_listed));
      }
    }
    __syncthreads();
    // one subtile ahead: its K rows and maxima load while the current one is processed
    bf16x8 ka_next[4];
    float smax_next = 0.f;
    if (static_cast<uint32_t>(wave) < nb) load_sub(s_ids[wave], ka_next, smax_next);
    for (uint32_t i = wave; i < nb; i += kRefWaves) {
      const int64_t sti = s_ids[i];
      bf16x8 ka[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) ka[c] = ka_next[c];
      const float smax = smax_next;
      if (i + kRefWaves < nb) load_sub(s_ids[i + kRefWaves], ka_next, smax_next);
      const int64_t key0 = sti * kSubTileKeys;
      // the split kernel's MFMA sequence for this subtile
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma_16x16x32(ka[c], qb[c], acc);
      float mx = -INFINITY;
      float sv[4];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float a = acc[i4];
        sv[i4] = key0 + 4 * grp + i4 < S ? fmaf(a, c2_hi, a * c2_lo) : -INFINITY;
        mx = fmaxf(mx, sv[i4]);
      }
      mx = max_xor32(max_xor16(mx));
      if (col < kG && grp == 0 && mx != smax) ++n_bad;
      // the K rows and the logits, staged for the float64 pass; the keys with a
      // dominant pair
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<bf16x8*>(s_k[wave] + col * kD + 32 * c + 8 * grp) = ka[c];
      uint32_t keys = 0;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        if (col < kG) s_sv[wave][(4 * grp + i4) * kG + col] = sv[i4];
        const uint64_t pb = __ballot(col < kG && sv[i4] >= thr_c);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          keys |= (((pb >> (16 * g4)) & 0xFFull) != 0 ? 1u : 0u) << (4 * g4 + i4);
      }
      lds_fence_wave();
      for (uint32_t m = keys; m; m &= m - 1) {
        const int ek = __builtin_ctz(m);
        const double dot = dot_group8(q_part, s_k[wave] + ek * kD, j);
        if (j == 0) {
          const float svf = s_sv[wave][ek * kG + h_l];
          if (svf >= thr_h) {
            const double svd = static_cast<double>(svf);
            const double dd = (c2 * dot - svd) * M_LN2;
            const float pw = __builtin_amdgcn_exp2f(static_cast<float>(svd - l2h));
            corr += static_cast<double>(pw) * (dd + 0.5 * dd * dd);
          }
        }
      }
      lds_fence_wave();   // the stage is read before the next subtile overwrites it
    }
  }
  n_bad = static_cast<uint32_t>(__popcll(__ballot(n_bad != 0)));   // lanes with a mismatch
  if (j == 0) s_acc[wave][h_l] = corr;
  if (lane == 0) s_bad[wave] = n_bad;
  __syncthreads();
  if (tid < kG) {
    double c = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < kRefWaves; ++w2) c += s_acc[w2][tid];
    RefinePart* pr = part + static_cast<size_t>(r) * n_wg + blockIdx.x;
    pr->corr[tid] = c;
    if (tid == 0) {
      uint32_t nb = 0;
#pragma unroll
      for (int w2 = 0; w2 < kRefWaves; ++w2) nb += s_bad[w2];
      pr->n_dom = e1 - e0;
      pr->n_bad = nb;
      pr->pad0 = 0u;
      pr->pad1 = 0u;
    }
  }
}

// One work-group of 8 waves per row, wave h for head h: the refined lse2 =
// lse2 + log2(1 + the head's partial sums) into lse2r, the natural-log lse for
// the caller, and the row's statistics.  (The heads' importance bounds keep
// the value they had: the selection's histograms are placed by them, and a
// bound off by the refinement's size stays a bound within a bin.)
__global__ __launch_bounds__(kG * 64) void lse_finalize_kernel(
    const RefinePart* __restrict__ part, int n_parts, const double* __restrict__ lse2,
    double* __restrict__ lse2r, float* __restrict__ lse_out, RefineStat* __restrict__ stat) {
  const int r = blockIdx.x, lane = threadIdx.x & 63, h = threadIdx.x >> 6;
  const RefinePart* pr = part + static_cast<size_t>(r) * n_parts;
  const double c = refine_head_sum(pr, n_parts, h);
  if (lane == 0) {
    const size_t o = static_cast<size_t>(r) * kG + h;
    const double l2 = lse2[o] + log1p(c) * M_LOG2E;
    lse2r[o] = l2;
    if (lse_out) lse_out[o] = static_cast<float>(l2 * M_LN2);
  }
  if (h == 0) {
    uint32_t nd = 0, nb = 0;
    for (int i = lane; i < n_parts; i += 64) {
      nd += pr[i].n_dom;
      nb += pr[i].n_bad;
    }
    for (int off = 32; off > 0; off >>= 1) {
      nd += __shfl_xor(nd, off);
      nb += __shfl_xor(nb, off);
    }
    if (lane == 0) stat[r] = RefineStat{nd, nb, 0u, 0u};
  }
}

// The largest of a double over lanes l, l ^ 8, l ^ 16, ..., l ^ 56 (in every lane).
__device__ __forceinline__ double max_over_groups8(double v) {
  v = fmax(v, dpp_f64<0x128>(v));   // row_ror:8, i.e. lane ^ 8 within the row of 16
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  auto join = [](uint32_t hi, uint32_t lo) {
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
  };
  const auto l16 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u), static_cast<uint32_t>(u), false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u >> 32), static_cast<uint32_t>(u >> 32), false, false);
  v = fmax(join(h16[0], l16[0]), join(h16[1], l16[1]));
  const uint64_t w = static_cast<uint64_t>(__double_as_longlong(v));
  const auto l32 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(w), static_cast<uint32_t>(w), false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(w >> 32), static_cast<uint32_t>(w >> 32), false, false);
  return fmax(join(h32[0], l32[0]), join(h32[1], l32[1]));
}

// Optional per-key importance for the caller (the step itself never needs all
// of them): every key's importance max_h 2^(y_h - lse2_h), y the float64 logit
// of exact bf16 products; one wave per subtile of 16 keys, lane (head h = lane
// >> 3, dims 16 (lane & 7) ..) as in the refinement.  grid (splits, R) over
// the split kernel's key ranges (multiples of 16 keys).
__global__ __launch_bounds__(kRefThreads) void full_scores_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const double* __restrict__ lse2,
    float* __restrict__ scores, int64_t S, int kps, double c2, int64_t kvp) {
  __shared__ __align__(16) u16 s_k[kRefWaves][kSubTileKeys * kD];
  const int r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int h = lane >> 3, j = lane & 7;
  const int64_t key_begin = static_cast<int64_t>(blockIdx.x) * kps;
  const int64_t key_end = min(S, key_begin + kps);
  const u16* qr = q + static_cast<size_t>(r) * kG * kD;
  const u16* kr = k + static_cast<size_t>(r) * kvp * kD;
  float* sr = scores + static_cast<size_t>(r) * S;
  double q_part[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) q_part[t] = static_cast<double>(bf16_bits_to_f32(qr[h * kD + 16 * j + t]));
  const double l2h = lse2[static_cast<size_t>(r) * kG + h];
  for (int64_t key0 = key_begin + kSubTileKeys * wave; key0 < key_end; key0 += kSubTileKeys * kRefWaves) {
    const int64_t key = min(key0 + col, key_end - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<u32x4*>(s_k[wave] + col * kD + 32 * c + 8 * grp) =
          load_u32x4(kr + key * kD + 32 * c + 8 * grp);
    lds_fence_wave();
    for (int e = 0; e < kSubTileKeys; ++e) {
      const double y = max_over_groups8(c2 * dot_group8(q_part, s_k[wave] + e * kD, j) - l2h);
      if (lane == 0 && key0 + e < key_end) sr[key0 + e] = static_cast<float>(exp2(y));
    }
    lds_fence_wave();
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
  const bool staged = p.kps <= kStageKeys;
  auto kern = p.quads ? (staged ? full_decode_split_kernel<true, true> : full_decode_split_kernel<false, true>)
                      : (staged ? full_decode_split_kernel<true, false> : full_decode_split_kernel<false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kWaves * 64), 0, st, q, k, v,
                     reinterpret_cast<float*>(w + p.off_stmax),
                     p.quads ? reinterpret_cast<unsigned char*>(w + p.off_qdiff) : nullptr,
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

hipError_t launch_lse_refine(const Plan& p, const u16* q, const u16* k, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  const float c2_hi = static_cast<float>(c2);
  const float c2_lo = static_cast<float>(c2 - static_cast<double>(c2_hi));
  hipLaunchKernelGGL(lse_refine_kernel, dim3(p.ref_nwg, p.R), dim3(kRefThreads), 0, st, q, k,
                     reinterpret_cast<const float*>(w + p.off_stmax),
                     reinterpret_cast<const double*>(w + p.off_lse2),
                     reinterpret_cast<const float*>(w + p.off_cut),
                     reinterpret_cast<const int32_t*>(w + p.off_dsub),
                     reinterpret_cast<const uint32_t*>(w + p.off_dsub_cnt),
                     reinterpret_cast<RefinePart*>(w + p.off_ref_part), p.S, p.Spad, p.w,
                     p.cc_chunk, p.cc_nchunk, p.ref_nwg, c2_hi, c2_lo, c2, p.kvp);
  return hipGetLastError();
}

hipError_t launch_lse_finalize(const Plan& p, float* lse, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  hipLaunchKernelGGL(lse_finalize_kernel, dim3(p.R), dim3(kG * 64), 0, st,
                     reinterpret_cast<const RefinePart*>(w + p.off_ref_part), p.ref_nwg,
                     reinterpret_cast<const double*>(w + p.off_lse2),
                     reinterpret_cast<double*>(w + p.off_lse2r), lse,
                     reinterpret_cast<RefineStat*>(w + p.off_ref_stat));
  return hipGetLastError();
}

hipError_t launch_full_scores(const Plan& p, const u16* q, const u16* k, float* scores,
                              void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  hipLaunchKernelGGL(full_scores_kernel, dim3(p.n_split, p.R), dim3(kRefThreads), 0, st, q, k,
                     reinterpret_cast<const double*>(w + p.off_lse2r), scores, p.S, p.kps, c2,
                     p.kvp);
  return hipGetLastError();
}

}  // namespace hs2
