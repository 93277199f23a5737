// Full-attention layer of a Cross-Decoder group over a chunk of T > 1 query
// tokens (prefill): causal attention of every chunk token over the shared KV
// cache, then each (token, KV head) row's log2 importance of every older key.
//
// The group's full layer and its attention-derived selection: news page
// "两天两连更：小米提前亮出V3底牌", section "两级KV共享：让模型少跑一半" (KV
// Reuse), video page "小米 MiMo-V3 HySparse2 架构：读长文省一半", section
// "HySparse2 的解法：两派都用，还改了流程".
//
// Design (gfx950):
//  * A work-group takes 16 consecutive chunk tokens of one (batch, KV head);
//    their 16 x 8 query heads are the 128 columns of S^T = K . Q^T.  Each of
//    the 4 waves owns 4 tokens = two 16-column query blocks (2 tokens x 8 heads
//    each), so no MFMA column is padding.
//  * Keys come in tiles of 64, staged once in LDS for all four waves (K and V,
//    272-byte row pitch); the next tile's global loads are in flight while the
//    current one is processed.
//  * S^T and O^T = V^T . P^T on MFMA 16x16x32 bf16; the P^T operand comes
//    straight from the S^T accumulators and V^T from ds_read_b64_tr_b16, as in
//    the decode kernel.  Online softmax in base 2 with an integer running
//    max (exact power-of-two rescales, skipped when no column's max moved)
//    and the normaliser accumulated in float64.
//  * Causality: token t (position P_t = S - T + t) sees keys 0..P_t; only the
//    last tiles of a work-group need the mask.
//  * Work-groups are numbered so that each of the 8 XCDs gets a contiguous
//    range of (batch, KV head, token block): the work-groups that share a KV
//    head's K/V run on one XCD and share its L2.
//  * The importance pass (second kernel) recomputes the logits with lse known
//    and writes y = max_h(s2_h - lse2_h) per (row, older key) as 16-bit fixed
//    point over the 64 octaves below the row's top log-weight (2^-10 octave
//    steps), and the largest |k| of each KV head, which bounds its float32
//    error for the selection.

#include <type_traits>

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kPThreads = 256;
// Attention: query blocks per wave.  Two keep the kernel at 244 VGPRs and two
// work-groups per CU; three or four halve the LDS operand reads per MFMA but
// drop to one wave per SIMD, and then measured 45-60% slower on the 4K-token
// chunk over 128K keys.
constexpr int kPrefillQB = 2;
constexpr int kPKeys = 64;      // keys per tile
// LDS row pitches, in u16.  K rows advance by 4 banks (68 dwords), so the
// 16-byte operand reads of 8 or 16 consecutive rows cover every bank once; V
// rows advance by 8 banks (72 dwords), so the transposing 8-byte reads (4 rows
// x 4 consecutive units per 16 lanes, 8 rows per 32) do.
constexpr int kPPitch = 136;
constexpr int kPVPitch = 144;

__device__ __forceinline__ int xcd_linear(int id, int n) {
  // hardware dispatch sends work-group id to XCD id % 8; renumber so that XCD x
  // processes the contiguous range [x * n/8, (x+1) * n/8)
  if (n % 8 != 0) return id;
  return (id & 7) * (n >> 3) + (id >> 3);
}

// One 64-key tile of K (and optionally V) from global memory into registers:
// thread t holds 64 bytes of key row t/4 (keys past `key_max` repeat it).
struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
};

template <bool kWithV>
__device__ __forceinline__ void tile_gload(TileRegs& r, const u16* __restrict__ kr,
                                           const u16* __restrict__ vr, int64_t key0,
                                           int64_t key_max) {
  const int tid = threadIdx.x;
  int64_t key = key0 + (tid >> 2);
  key = key < key_max ? key : key_max;
  const u16* ks = kr + key * kD + 32 * (tid & 3);
#pragma unroll
  for (int c = 0; c < 4; ++c) r.k[c] = load_u32x4(ks + 8 * c);
  if (kWithV) {
    const u16* vs = vr + key * kD + 32 * (tid & 3);
#pragma unroll
    for (int c = 0; c < 4; ++c) r.v[c] = load_u32x4(vs + 8 * c);
  }
}

template <bool kWithV>
__device__ __forceinline__ void tile_lstore(const TileRegs& r, u16* kt, u16* vt) {
  const int tid = threadIdx.x;
  u16* kd = kt + (tid >> 2) * kPPitch + 32 * (tid & 3);
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(kd + 8 * c) = r.k[c];
  if (kWithV) {
    u16* vd = vt + (tid >> 2) * kPVPitch + 32 * (tid & 3);
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(vd + 8 * c) = r.v[c];
  }
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// K as the A operand of S^T for key subtile kt (16 keys) and dims 32c..32c+31.
__device__ __forceinline__ bf16x8 lds_k_operand(const u16* kt, int sub, int c, int col, int grp) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(kt + (16 * sub + col) * kPPitch + 32 * c + 8 * grp));
}

// Make the compiler wait for a loaded operand here (an empty asm that reads
// it), so that the load is not left outstanding into a loop.
__device__ __forceinline__ void require_loaded(const bf16x8& x) {
  asm volatile("" : : "v"(__builtin_bit_cast(u32x4, x)));
}

// Q^T as the B operand: column col of a query block = (token tok, head col & 7).
__device__ __forceinline__ void load_q_block(const u16* __restrict__ qtok, int col, int grp,
                                             bf16x8 (&qb)[4]) {
  const u16* p = qtok + (col & 7) * kD + 8 * grp;
#pragma unroll
  for (int c = 0; c < 4; ++c) qb[c] = as_bf16x8(load_u32x4(p + 32 * c));
}

// grid: B * Hkv * ceil(T / (8 * QB)) work-groups of 256 threads; each wave
// owns QB query blocks (2 QB tokens), so every K/V operand read from LDS
// serves 16 QB query columns.
template <int QB>
__global__ __launch_bounds__(kPThreads, QB <= 2 ? 2 : 1) void full_prefill_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    u16* __restrict__ out, float* __restrict__ lse_out, double* __restrict__ lse2,
    float* __restrict__ ytop_h, int64_t S, int T, int Hkv, int n_tblk, float c2_hi,
    float c2_lo, int64_t kvp) {
  __shared__ __align__(16) u16 kt[kPKeys * kPPitch];
  __shared__ __align__(16) u16 vt[kPKeys * kPVPitch];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int lin = xcd_linear(blockIdx.x, gridDim.x);
  const int tb = lin % n_tblk;
  const int bg = lin / n_tblk;
  const int g = bg % Hkv, b = bg / Hkv;
  const int Hq = Hkv * kG;
  const u16* kr = k + static_cast<size_t>(bg) * kvp * kD;
  const u16* vr = v + static_cast<size_t>(bg) * kvp * kD;
  const int64_t pos0 = S - T;                      // position of chunk token 0
  constexpr int kTok = 8 * QB;                     // chunk tokens per work-group
  // this lane's columns: query block qbk covers tokens 2*QB*wave + 2*qbk + {0,1}
  int64_t pcol[QB];
  bf16x8 qop[QB][4];
#pragma unroll
  for (int qbk = 0; qbk < QB; ++qbk) {
    int t = tb * kTok + 2 * QB * wave + 2 * qbk + (col >> 3);
    t = t < T ? t : T - 1;                         // past the chunk: repeat the last token
    pcol[qbk] = pos0 + t;
    load_q_block(q + (static_cast<size_t>(b) * T + t) * Hq * kD + static_cast<size_t>(g) * kG * kD,
                 col, grp, qop[qbk]);
  }
  const int t_last = min(T - 1, tb * kTok + kTok - 1);
  const int64_t p_first = pos0 + tb * kTok;        // smallest position in the work-group
  const int64_t p_last = pos0 + t_last;
  const int n_tiles = static_cast<int>((p_last + kPKeys) / kPKeys);

  f32x4 o[QB][8];
  float m[QB];
  double l[QB];
#pragma unroll
  for (int qbk = 0; qbk < QB; ++qbk) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[qbk][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[qbk] = -INFINITY;
    l[qbk] = 0.0;
  }

  TileRegs regs;
  tile_gload<true>(regs, kr, vr, 0, p_last);
  tile_lstore<true>(regs, kt, vt);
  // the query operands must have landed before the loop: inside it only the
  // next tile's loads may be outstanding, or the first MFMAs of every tile
  // would wait for them
#pragma unroll
  for (int qbk = 0; qbk < QB; ++qbk)
#pragma unroll
    for (int c = 0; c < 4; ++c) require_loaded(qop[qbk][c]);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int64_t key0 = static_cast<int64_t>(it) * kPKeys;
    const bool more = it + 1 < n_tiles;
    if (more) tile_gload<true>(regs, kr, vr, key0 + kPKeys, p_last);
    // ---- S^T: 4 key subtiles x QB query blocks
    f32x4 sacc[QB][4];
#pragma unroll
    for (int qbk = 0; qbk < QB; ++qbk)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) sacc[qbk][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = lds_k_operand(kt, sub, c, col, grp);
#pragma unroll
        for (int qbk = 0; qbk < QB; ++qbk)
          sacc[qbk][sub] = mfma_16x16x32(a, qop[qbk][c], sacc[qbk][sub]);
      }
    // only the last tiles of a work-group reach past some token's position
    const bool masked = key0 + kPKeys - 1 > p_first;
    // The running max is taken over the raw dot products (the scale is
    // positive, and the rounded scaling is monotonic), and each exponent is
    // a * c2_hi - m in one fma: the product and the shift by the integer m are
    // exact inside it, so only the result rounds, and the scale's dropped low
    // part (below 2^-24 of a * c2) moves a probability by under 2e-7 of
    // itself, and lse2 by less: far inside the selection's tolerance (the
    // importance pass and the float64 re-ranking share this lse2).
    float p[QB][4][4];
#pragma unroll
    for (int qbk = 0; qbk < QB; ++qbk) {
      float sv[4][4];
      float amax = -INFINITY;
      if (!masked) {
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[sub][i] = sacc[qbk][sub][i];
            amax = fmaxf(amax, sv[sub][i]);
          }
      } else {
        // key0 + off is visible to the column iff off <= P - key0; a hidden
        // key gets a large finite negative product, whose exponent
        // underflows to 0
        const int lim = static_cast<int>(min(static_cast<int64_t>(kPKeys), pcol[qbk] - key0));
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[sub][i] = 16 * sub + 4 * grp + i <= lim ? sacc[qbk][sub][i] : -1.0e30f;
            amax = fmaxf(amax, sv[sub][i]);
          }
      }
      // the column's other keys sit in lanes ^ 16 and ^ 32: VALU row swaps
      {
        const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(amax),
                                                          __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
        const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax),
                                                          __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
      }
      // key 0 is visible to every token, so the running max is finite from the
      // first tile on
      const float tmax = fmaf(amax, c2_hi, amax * c2_lo);
      const float m_new = fmaxf(m[qbk], ceilf(tmax));
      const float alpha = m[qbk] == -INFINITY ? 0.f : ldexpf(1.f, static_cast<int>(m[qbk] - m_new));
      float ps = 0.f;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = sv[sub][i];
          p[qbk][sub][i] = __builtin_amdgcn_exp2f(fmaf(a, c2_hi, -m_new));
          ps += p[qbk][sub][i];
        }
      l[qbk] = l[qbk] * static_cast<double>(alpha) + static_cast<double>(ps);
      if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[qbk][nb] *= alpha;
      }
      m[qbk] = m_new;
    }
    // ---- O^T += V^T . P^T over two k-steps of 32 keys
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pb[QB];
#pragma unroll
      for (int qbk = 0; qbk < QB; ++qbk) {
        const u32x4 pp{pack_bf16x2(p[qbk][2 * ks][0], p[qbk][2 * ks][1]),
                       pack_bf16x2(p[qbk][2 * ks][2], p[qbk][2 * ks][3]),
                       pack_bf16x2(p[qbk][2 * ks + 1][0], p[qbk][2 * ks + 1][1]),
                       pack_bf16x2(p[qbk][2 * ks + 1][2], p[qbk][2 * ks + 1][3])};
        pb[qbk] = as_bf16x8(pp);
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x8 a = lds_vt_operand(vt + 32 * ks * kPVPitch, kPVPitch, nb, col, grp);
#pragma unroll
        for (int qbk = 0; qbk < QB; ++qbk) o[qbk][nb] = mfma_16x16x32(a, pb[qbk], o[qbk][nb]);
      }
    }
    __syncthreads();               // every wave is done with this tile
    if (more) {
      tile_lstore<true>(regs, kt, vt);
      __syncthreads();
    }
  }
  // ---- epilogue: normalise, write out and the row statistics
#pragma unroll
  for (int qbk = 0; qbk < QB; ++qbk) {
    double L = l[qbk];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    const int t = tb * kTok + 2 * QB * wave + 2 * qbk + (col >> 3);
    if (t >= T) continue;
    const int h = col & 7;
    const float inv = static_cast<float>(1.0 / L);
    u16* orow = out + ((static_cast<size_t>(b) * T + t) * Hq + static_cast<size_t>(g) * kG + h) * kD;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint2 pk{pack_bf16x2(o[qbk][nb][0] * inv, o[qbk][nb][1] * inv),
                     pack_bf16x2(o[qbk][nb][2] * inv, o[qbk][nb][3] * inv)};
      *reinterpret_cast<uint2*>(orow + 16 * nb + 4 * grp) = pk;
    }
    if (grp == 0) {
      const size_t row = (static_cast<size_t>(b) * T + t) * Hkv + g;
      const double l2 = static_cast<double>(m[qbk]) + log2(L);
      lse2[row * kG + h] = l2;
      if (lse_out) lse_out[row * kG + h] = static_cast<float>(l2 * M_LN2);
      ytop_h[row * kG + h] = static_cast<float>(-log2(L));
    }
  }
}

// Importance pass.  grid: B * Hkv * ceil(T / 64) work-groups of 8 waves; a
// work-group takes 64 chunk tokens, each wave 4 query blocks (2 tokens x 8
// heads each), so every K operand read from LDS serves 64 query rows.
// Here the MFMA computes S = Q . K^T (query rows, key columns): a lane holds 4
// heads of one token for one key, and the max over the token's 8 heads is 3
// in-lane steps and one exchange with the partner lane.
// The waves form two groups of four, one wave of each per SIMD, that take
// turns: while one group runs a tile's MFMAs the other turns its previous
// tile into importance values (VALU and stores), so the matrix cores stay
// fed during the epilogue.  Group B runs one phase behind group A; a barrier
// ends every phase.  K tiles (64 keys) are double-buffered in LDS; each wave
// stages 8 rows of the next tile through registers, loading them in one
// phase and writing them in the next.
// Writes, for every row (b, t, g) it owns:
//   y[row][j] = max_h(s2_h[j] - lse2_h) for older keys j < first_t, as
//               round((y - ybase) 2^10) clamped to 0..65535, with ybase the
//               row's top log-weight (over its 8 heads) minus 64 (when y is
//               non-null);
//   kmax[b][g][tb] = the largest |k| over this work-group's share of the KV
//               head's keys 0..S-1 (bf16 bits; when kmax is non-null): whole
//               key tile i belongs to token block i % n_tblk when that block
//               reads all of it, else to the last block, which reads every key.
constexpr int kIWaves = 8;
constexpr int kIThreads = 64 * kIWaves;
constexpr int kIQB = 4;                        // query blocks per wave
static_assert(kIWaves * 2 * kIQB == kImportanceTok, "64 chunk tokens per work-group");

// K tile in LDS as unpadded 256-byte rows, the 16-byte chunk c of row r at
// slot c ^ (r & 15): the operand reads of 16 consecutive rows (one chunk each)
// cover all banks once, and one LDS-direct load fills 4 whole rows.
__device__ __forceinline__ bf16x8 lds_k_swizzled(const u16* kt, int sub, int c, int col, int grp) {
  const int slot = (4 * c + grp) ^ col;
  return as_bf16x8(*reinterpret_cast<const u32x4*>(kt + (16 * sub + col) * kD + 8 * slot));
}

__device__ __forceinline__ void wait_lgkm_all() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), other counters untouched
}

// A work-group barrier that waits for no memory operation: the importance
// values' global stores stay in flight across it.  Whatever must be visible
// past it is waited for explicitly (the tile's LDS writes), and the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kIThreads, 1) void prefill_importance_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const double* __restrict__ lse2,
    const float* __restrict__ ytop_h, u16* __restrict__ y, uint32_t* __restrict__ kmax,
    int64_t S, int64_t Spad, int T, int Hkv, int w, int n_tblk, float c2_hi, int64_t kvp) {
  __shared__ __align__(16) u16 kbuf[2][kPKeys * kD];
  __shared__ uint32_t s_kmax[kIWaves];
  constexpr int QB = kIQB;
  constexpr int kTok = kImportanceTok;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // waves w and w + 4 share a SIMD; the group is wave-uniform (read as such)
  const bool group_b = __builtin_amdgcn_readfirstlane(wave) >= kIWaves / 2;
  const int col = lane & 15, grp = lane >> 4;
  const int lin = xcd_linear(blockIdx.x, gridDim.x);
  const int tb = lin % n_tblk;
  const int bg = lin / n_tblk;
  const int g = bg % Hkv, b = bg / Hkv;
  const int Hq = Hkv * kG;
  const u16* kr = k + static_cast<size_t>(bg) * kvp * kD;
  const int64_t pos0 = S - T;
  bf16x8 qop[QB][4];
  bool t_ok[QB];
  int64_t P[QB], first[QB];
  // y in fixed-point steps plus 0.5 is s c2 2^10 + (0.5 - 2^10 (lse2_h + ybase)):
  // one fma per head
  float nl2r[QB][4];     // 0.5 - 2^10 (lse2_h + ybase) for the lane's 4 heads
  u16* yrow[QB];
#pragma unroll
  for (int qbk = 0; qbk < QB; ++qbk) {
    // the A operand: query row col = (token .. + (col >> 3), head col & 7)
    int tq = tb * kTok + 2 * QB * wave + 2 * qbk + (col >> 3);
    tq = tq < T ? tq : T - 1;
    load_q_block(q + (static_cast<size_t>(b) * T + tq) * Hq * kD + static_cast<size_t>(g) * kG * kD,
                 col, grp, qop[qbk]);
    // this lane's rows of S: 4*grp + i = (token .. + (grp >> 1), head 4*(grp & 1) + i)
    int t = tb * kTok + 2 * QB * wave + 2 * qbk + (grp >> 1);
    t_ok[qbk] = t < T;
    t = t_ok[qbk] ? t : T - 1;
    P[qbk] = pos0 + t;
    first[qbk] = max(static_cast<int64_t>(0), P[qbk] - w + 1);
    const size_t row = (static_cast<size_t>(b) * T + t) * Hkv + g;
    float yt = -INFINITY;
    for (int h = 0; h < kG; ++h) yt = fmaxf(yt, ytop_h[row * kG + h]);
    const float ybase = yt - kYRange;
    // 2^10 ybase is exact, and so is its sum with 0.5 (|ybase| < 2^12)
    const float yoff = 0.5f - ybase * static_cast<float>(1 << kYFixBits);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      nl2r[qbk][i] = fmaf(-static_cast<float>(lse2[row * kG + 4 * (grp & 1) + i]),
                          static_cast<float>(1 << kYFixBits), yoff);
    yrow[qbk] = y ? y + row * Spad : nullptr;
  }
  const int t_last = min(T - 1, tb * kTok + kTok - 1);
  const int64_t p_last = pos0 + t_last;
  const int n_tiles = static_cast<int>((p_last + kPKeys) / kPKeys);
  // after the head max a lane owns key subtiles 2*(grp & 1) and 2*(grp & 1) + 1
  const int sub0 = 2 * (grp & 1);
  const float c2s = c2_hi * static_cast<float>(1 << kYFixBits);   // exact
  // this work-group's share of max |k|: whole tiles i with i % n_tblk == tb
  // (or, when that block does not read all of tile i, the last block's)
  auto owns_tile = [&](int i) {
    const int o = i % n_tblk;
    const int64_t o_last = pos0 + min(T - 1, o * kTok + kTok - 1);
    return (static_cast<int64_t>(i + 1) * kPKeys <= o_last + 1 ? o : n_tblk - 1) == tb;
  };
  u16x2 kabs{0, 0};

  // this wave's 8 rows of a tile, staged through registers: lane l holds
  // bytes 32 (l & 7) .. + 31 of row 8 wave + (l >> 3)
  const int srow_ = 8 * wave + (lane >> 3);
  const int sc0 = 2 * (lane & 7);
  u32x4 stg[2];
  auto stage_load = [&](int64_t key0) {
    const int64_t key = min(key0 + srow_, p_last);
    const u16* src = kr + key * kD + 8 * sc0;
    stg[0] = load_u32x4(src);
    stg[1] = load_u32x4(src + 8);
  };
  auto stage_store = [&](u16* kt, int tile) {
    u16* dst = kt + srow_ * kD;
    *reinterpret_cast<u32x4*>(dst + 8 * (sc0 ^ (srow_ & 15))) = stg[0];
    *reinterpret_cast<u32x4*>(dst + 8 * ((sc0 + 1) ^ (srow_ & 15))) = stg[1];
    if (kmax && tile < n_tiles && owns_tile(tile)) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kabs = __builtin_elementwise_max(kabs, __builtin_bit_cast(u16x2, stg[u][e] & 0x7FFF7FFFu));
    }
  };

  // prologue: tile 0 by every wave; group B loads its rows of tile 1 in the
  // phase it spends behind group A
  stage_load(0);
  stage_store(kbuf[0], 0);
#pragma unroll
  for (int qbk = 0; qbk < QB; ++qbk)
#pragma unroll
    for (int c = 0; c < 4; ++c) require_loaded(qop[qbk][c]);
  __syncthreads();
  // the tile loop, as a separate copy per group: each group's copy has only
  // its own loads and stores in flight, so the compiler waits on exactly those
  // a tile's MFMAs: S for this wave's 4 query blocks x 64 keys
  auto mfma_phase = [&](const u16* kt, f32x4 (&sacc)[QB][4]) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
#pragma unroll
      for (int qbk = 0; qbk < QB; ++qbk) sacc[qbk][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 kb = lds_k_swizzled(kt, sub, c, col, grp);
#pragma unroll
        for (int qbk = 0; qbk < QB; ++qbk)
          sacc[qbk][sub] = mfma_16x16x32(qop[qbk][c], kb, sacc[qbk][sub]);
      }
    }
  };
  // a tile's epilogue: importance values from S, and their stores
  auto epilogue = [&](const f32x4 (&sacc)[QB][4], int64_t key0) {
#pragma unroll
    for (int qbk = 0; qbk < QB; ++qbk) {
      // y per (token, key), in fixed-point steps plus 0.5: max over the 8
      // heads = 4 here x the partner lane.  One fma per head: the scale's low
      // part (below 1e-7 of s c2) is dropped; the selection allows for it and
      // re-ranks every key near its threshold in float64
      float yv[4];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaf(sacc[qbk][sub][i], c2s, nl2r[qbk][i]));
        // the partner lane (lane ^ 16) holds the other 4 heads: one VALU
        // row swap gives both lanes both halves
        const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m),
                                                         false, false);
        yv[sub] = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int sub = sub0 + u;
        const float yy = sub == 0 ? yv[0] : sub == 1 ? yv[1] : sub == 2 ? yv[2] : yv[3];
        const int64_t key = key0 + 16 * sub + col;
        // clamp to 0..65535, then truncate: rounds to nearest
        const u16 v = static_cast<u16>(static_cast<uint32_t>(__builtin_amdgcn_fmed3f(yy, 0.f, 65535.f)));
        // every lane stores (a fixed count of stores per phase, so the
        // tile loads can be waited for alone): keys at or past first_t
        // land in the row's unread tail (key < Spad), and a block past
        // the chunk's end repeats the last token, value for value
        yrow[qbk][key] = v;
      }
    }
  };
  // The tile loops, one per group, each laid out so that a tile's staging
  // loads and LDS writes fall in one loop iteration: the compiler then waits
  // for the loads alone, not for the importance stores issued after them.
  if (!group_b) {
    // phases 2 it (MFMAs of tile it, loads of tile it + 1) and 2 it + 1
    // (epilogue of tile it, LDS writes of tile it + 1)
    for (int it = 0; it < n_tiles; ++it) {
      const int64_t key0 = static_cast<int64_t>(it) * kPKeys;
      f32x4 sacc[QB][4];
      // past the last tile the rows repeat key p_last and the LDS writes land
      // in a buffer nobody reads again: unconditional, so every load is
      // waited for on every path
      stage_load(key0 + kPKeys);
      asm volatile("" ::: "memory");   // issue the loads before the phase's work
      mfma_phase(kbuf[it & 1], sacc);
      phase_barrier();
      stage_store(kbuf[(it & 1) ^ 1], it + 1);
      epilogue(sacc, key0);
      wait_lgkm_all();
      phase_barrier();
    }
    phase_barrier();   // group B's last phase
  } else {
    // phases 2 it (epilogue of tile it - 1, loads of tile it + 1) and 2 it + 1
    // (MFMAs of tile it, LDS writes of tile it + 1); the first of these phases
    // has no epilogue and puts group B one phase behind group A
    f32x4 sacc[QB][4];
    for (int it = 0; it < n_tiles; ++it) {
      const int64_t key0 = static_cast<int64_t>(it) * kPKeys;
      stage_load(key0 + kPKeys);
      if (it > 0) epilogue(sacc, key0 - kPKeys);
      phase_barrier();
      stage_store(kbuf[(it & 1) ^ 1], it + 1);
      mfma_phase(kbuf[it & 1], sacc);
      wait_lgkm_all();
      phase_barrier();
    }
    epilogue(sacc, static_cast<int64_t>(n_tiles - 1) * kPKeys);
    phase_barrier();
  }
  if (kmax) {
    uint32_t m = max(static_cast<uint32_t>(kabs[0]), static_cast<uint32_t>(kabs[1]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(m, off)));
    if (lane == 0) s_kmax[wave] = m;
    __syncthreads();
    if (tid == 0) {
      for (int wv = 1; wv < kIWaves; ++wv) m = max(m, s_kmax[wv]);
      kmax[static_cast<size_t>(bg) * n_tblk + tb] = m;
    }
  }
}

// Dense importance of a chunk for the caller (an optional output: the step
// itself never needs it), exactly: one work-group per row (b, t, g), the
// logits of keys 0..P_t in float64 from exact bf16 products, a first pass for
// each head's log-normaliser (an online max and sum in float64, combined in a
// fixed order), a second for max_h 2^(y_h - lse2_h); keys past P_t get 0.
constexpr int kXThreads = 256;
constexpr int kXWaves = kXThreads / 64;

__device__ __forceinline__ double dot_row_f64(const double* __restrict__ qh, const u16* __restrict__ krow) {
  double dot = 0.0;
#pragma unroll 4
  for (int d8 = 0; d8 < kD / 8; ++d8) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(krow + 8 * d8);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t word = raw[t >> 1];
      dot = fma(qh[8 * d8 + t],
                static_cast<double>(__uint_as_float((t & 1) ? (word & 0xFFFF0000u) : (word << 16))), dot);
    }
  }
  return dot;
}

__global__ __launch_bounds__(kXThreads) void prefill_scores_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, float* __restrict__ scores, int64_t S,
    int T, int Hkv, double c2, int64_t kvp) {
  __shared__ double s_q[kG * kD];
  __shared__ __align__(16) u16 s_k[kXWaves][16 * kD];
  __shared__ double s_m[kXWaves][kG], s_l[kXWaves][kG];
  __shared__ double s_l2[kG];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int t = (r / Hkv) % T, g = r % Hkv, b = r / (T * Hkv);
  const int64_t P = S - T + t;
  const u16* qr = q + static_cast<size_t>(r) * kG * kD;
  const u16* kr = k + (static_cast<size_t>(b) * Hkv + g) * static_cast<size_t>(kvp) * kD;
  float* sr = scores + static_cast<size_t>(r) * S;
  for (int i = tid; i < kG * kD; i += kXThreads) s_q[i] = static_cast<double>(bf16_bits_to_f32(qr[i]));
  __syncthreads();
  // lane (key e = (lane >> 3) + 8 u, head h = lane & 7) of each 16-key subtile
  const int h_l = lane & 7;
  const double* qh = s_q + h_l * kD;
  auto stage = [&](int64_t key0) {
    const int64_t key = min(key0 + col, P);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<u32x4*>(s_k[wave] + col * kD + 32 * c + 8 * grp) =
          load_u32x4(kr + key * kD + 32 * c + 8 * grp);
    lds_fence_wave();
  };
  double m = -INFINITY, l = 0.0;
  for (int64_t key0 = 16 * wave; key0 <= P; key0 += 16 * kXWaves) {
    stage(key0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = (lane >> 3) + 8 * u;
      if (key0 + e > P) continue;
      const double y = c2 * dot_row_f64(qh, s_k[wave] + e * kD);
      if (y > m) {
        l = l * exp2(m - y) + 1.0;
        m = y;
      } else {
        l += exp2(y - m);
      }
    }
    lds_fence_wave();
  }
  // each head over the lanes l with l & 7 = h (lane ^ 8, ^ 16, ^ 32), then the waves
  auto merge = [](double& m1, double& l1, double m2, double l2) {
    const double mm = fmax(m1, m2);
    if (mm == -INFINITY) return;
    l1 = (m1 == -INFINITY ? 0.0 : l1 * exp2(m1 - mm)) + (m2 == -INFINITY ? 0.0 : l2 * exp2(m2 - mm));
    m1 = mm;
  };
  {
    double m2 = dpp_f64<0x128>(m), l2 = dpp_f64<0x128>(l);   // lane ^ 8
    merge(m, l, m2, l2);
    m2 = __shfl_xor(m, 16);
    l2 = __shfl_xor(l, 16);
    merge(m, l, m2, l2);
    m2 = __shfl_xor(m, 32);
    l2 = __shfl_xor(l, 32);
    merge(m, l, m2, l2);
  }
  if (lane < kG) {
    s_m[wave][lane] = m;
    s_l[wave][lane] = l;
  }
  __syncthreads();
  if (tid < kG) {
    double mm = s_m[0][tid], ll = s_l[0][tid];
    for (int w2 = 1; w2 < kXWaves; ++w2) merge(mm, ll, s_m[w2][tid], s_l[w2][tid]);
    s_l2[tid] = mm + log2(ll);
  }
  __syncthreads();
  const double l2h = s_l2[h_l];
  for (int64_t key0 = 16 * wave; key0 <= P; key0 += 16 * kXWaves) {
    stage(key0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = (lane >> 3) + 8 * u;
      double y = c2 * dot_row_f64(qh, s_k[wave] + e * kD) - l2h;
      y = fmax(y, dpp_f64<0xB1>(y));    // lane ^ 1
      y = fmax(y, dpp_f64<0x4E>(y));    // lane ^ 2
      y = fmax(y, dpp_f64<0x141>(y));   // the other quad of the 8
      if (h_l == 0 && key0 + e <= P) sr[key0 + e] = static_cast<float>(exp2(y));
    }
    lds_fence_wave();
  }
  for (int64_t key = P + 1 + tid; key < S; key += kXThreads) sr[key] = 0.f;
}

}  // namespace

hipError_t launch_full_prefill(const Plan& p, const u16* q, const u16* k, const u16* v, u16* out,
                               float* lse, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;  // scale * log2(e)
  const float c2_hi = static_cast<float>(c2);
  const float c2_lo = static_cast<float>(c2 - static_cast<double>(c2_hi));
  constexpr int QB = kPrefillQB;
  const int n_tblk = (p.T + 8 * QB - 1) / (8 * QB);
  const int n_wg = p.B * p.Hkv * n_tblk;
  hipLaunchKernelGGL(full_prefill_kernel<QB>, dim3(n_wg), dim3(kPThreads), 0, st, q, k, v, out,
                     lse, reinterpret_cast<double*>(w + p.off_lse2),
                     reinterpret_cast<float*>(w + p.off_ytop), p.S, p.T, p.Hkv, n_tblk, c2_hi,
                     c2_lo, p.kvp);
  return hipGetLastError();
}

hipError_t launch_prefill_importance(const Plan& p, const u16* q, const u16* k, void* ws,
                                     hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  const float c2_hi = static_cast<float>(c2);
  const int n_tblk = (p.T + kImportanceTok - 1) / kImportanceTok;
  const int n_wg = p.B * p.Hkv * n_tblk;
  hipLaunchKernelGGL(prefill_importance_kernel, dim3(n_wg), dim3(kIThreads), 0, st, q, k,
                     reinterpret_cast<const double*>(w + p.off_lse2),
                     reinterpret_cast<const float*>(w + p.off_ytop),
                     reinterpret_cast<u16*>(w + p.off_ybuf),
                     reinterpret_cast<uint32_t*>(w + p.off_kmax), p.S, p.Spad, p.T, p.Hkv, p.w,
                     n_tblk, c2_hi, p.kvp);
  return hipGetLastError();
}

hipError_t launch_prefill_scores(const Plan& p, const u16* q, const u16* k, float* scores,
                                 hipStream_t st) {
  const double c2 = p.scale * 1.4426950408889634;
  hipLaunchKernelGGL(prefill_scores_kernel, dim3(p.R), dim3(kXThreads), 0, st, q, k, scores, p.S,
                     p.T, p.Hkv, c2, p.kvp);
  return hipGetLastError();
}

}  // namespace hs2
