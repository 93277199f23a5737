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
constexpr int kAttnQC = 1;   // attention: 32-column blocks per wave
constexpr int kPKeys = 64;      // keys per tile

__device__ __forceinline__ int xcd_linear(int id, int n) {
  // hardware dispatch sends work-group id to XCD id % 8; renumber so that XCD x
  // processes the contiguous range [x * n/8, (x+1) * n/8)
  if (n % 8 != 0) return id;
  return (id & 7) * (n >> 3) + (id >> 3);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Make the compiler wait for a loaded operand here (an empty asm that reads
// it), so that the load is not left outstanding into a loop.
__device__ __forceinline__ void require_loaded(const bf16x8& x) {
  asm volatile("" : : "v"(__builtin_bit_cast(u32x4, x)));
}

// ---- attention kernel
//
// grid: B * Hkv * ceil(T / 16) work-groups of 256 threads.  A work-group takes
// 16 consecutive chunk tokens of one (batch, KV head); each wave owns 4 of
// them, whose 4 x 8 query heads are the 32 columns of its S^T = K Q^T and
// O^T = V^T P^T, both on the 32x32x16 bf16 MFMA (which leaves the VALU more
// room beside each MFMA than the 16x16x32 form at the same rate).
//
// Lane l holds column n = l & 31 (token 4 wave + n / 8, head n % 8) and, of a
// 32-row accumulator block, rows 8 (r / 4) + 4 (l >> 5) + r % 4 in register r.
// A 64-key tile's logits are two such blocks (keys 32 kb + row).  The P^T
// operand of a 16-key step s is the 8 registers 8 (s & 1) .. of block s / 2,
// as bf16: its k-index 8 (l >> 5) + j is key 16 s + 8 (j / 4) + 4 (l >> 5) +
// j % 4, and V^T's operand takes the same key order (two transposing reads
// of 4 rows each).
//
// Software pipeline: step i turns tile i's logits S_i (computed in step
// i - 1) into probabilities while the MFMAs of tile i + 1's logits run, then
// adds V_i^T P_i to O.  So the wave's own VALU work (the softmax) sits
// between independent MFMAs instead of after them.  K and V tiles are
// double-buffered in LDS and filled by LDS-direct loads (16 bytes a lane) one
// step ahead, with one barrier per step.  Rows are 256 bytes, their 16-byte
// chunks XOR-swizzled so that both operand reads are bank-conflict-free: K's
// chunk c of row r sits at slot c ^ (r & 15) (the 16 rows of one K read hit 16
// different slots), V's at c ^ 4 (r & 3) (the 4 rows x 4 chunks x 2 halves
// that 32 lanes of a transposing read address hit 32 different 8-byte places).
typedef __attribute__((address_space(3))) void* lds_void_ptr;
// an LDS-direct load's destination: the wave-uniform start of its 1 KB
__device__ __forceinline__ lds_void_ptr lds_ptr(u16* tile, int byte_off) {
  return (lds_void_ptr)((__attribute__((address_space(3))) char*)tile + byte_off);
}
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// QC column blocks of 32 per wave: every K and V^T operand read from LDS
// then feeds QC MFMAs (LDS instruction issue, not bytes, is what bounds the
// operand reads: a transposing 8-byte read costs about as much as a 16-byte
// one).  QC = 2 needs more than 256 registers (O in accumulation registers),
// so one wave per SIMD; QC = 1 runs two.
template <int QC>
__global__ __launch_bounds__(kPThreads, QC == 1 ? 2 : 1) void full_prefill_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    u16* __restrict__ out, float* __restrict__ lse_out, double* __restrict__ lse2,
    float* __restrict__ ytop_h, int64_t S, int T, int Hkv, int n_tblk, float c2_hi,
    float c2_lo, int64_t kvp) {
  constexpr int kTok = 16 * QC;   // chunk tokens per work-group
  __shared__ __align__(16) u16 kb0[kPKeys * kD];
  __shared__ __align__(16) u16 kb1[kPKeys * kD];
  __shared__ __align__(16) u16 vb0[kPKeys * kD];
  __shared__ __align__(16) u16 vb1[kPKeys * kD];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int n = lane & 31, hf = lane >> 5;
  const int lin = xcd_linear(blockIdx.x, gridDim.x);
  const int tb = lin % n_tblk;
  const int bg = lin / n_tblk;
  const int g = bg % Hkv, b = bg / Hkv;
  const int Hq = Hkv * kG;
  const u16* kr = k + static_cast<size_t>(bg) * kvp * kD;
  const u16* vr = v + static_cast<size_t>(bg) * kvp * kD;
  // positions fit in 32 bits (the context is below 2^31 keys)
  const int pos0 = static_cast<int>(S) - T;        // position of chunk token 0
  // column block cb of this wave: tokens 4 (QC wave + cb) .. + 3 of the group
  int t_col[QC], pcol[QC];
  // Q^T as the B operand: k-step ks holds dims 16 ks + 8 hf .. + 7 of column n
  bf16x8 qop[QC][8];
#pragma unroll
  for (int cb = 0; cb < QC; ++cb) {
    t_col[cb] = tb * kTok + 4 * (QC * wave + cb) + (n >> 3);
    const int t_q = t_col[cb] < T ? t_col[cb] : T - 1;   // past the chunk: repeat the last token
    pcol[cb] = pos0 + t_q;
    const u16* qp = q + (static_cast<size_t>(b) * T + t_q) * Hq * kD +
                    (static_cast<size_t>(g) * kG + (n & 7)) * kD + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[cb][ks] = as_bf16x8(load_u32x4(qp + 16 * ks));
  }
  const int t_last = min(T - 1, tb * kTok + kTok - 1);
  const int p_first = pos0 + tb * kTok;            // smallest position in the work-group
  const int p_last = pos0 + t_last;
  const int n_tiles = (p_last + kPKeys) / kPKeys;

  // fills: wave w writes rows 16w .. 16w + 15 of a tile, 4 rows (1 KB) per
  // load, lane l at row r = 16w + 4j + (l >> 4), slot l & 15.  The source
  // chunk's byte offset in its 4 rows is f0 ^ (64 j) for K (swizzle r & 15 =
  // 4 j + (l >> 4)) and f0 for V (swizzle 4 (r & 3) = 4 (l >> 4)), f0 that of
  // j = 0.  A tile is filled from key kf = min(key0, p_last - 63), so that
  // every row it reads is a key at most p_last: the last tile of a
  // work-group then starts delta = key0 - kf rows early, and its softmax hides
  // those rows (their keys were the previous tile's).  With fewer than 64 keys
  // in all (a single tile) rows past p_last repeat it instead.
  const uint32_t fk0 = (lane >> 4) * 256u + 16u * ((lane & 15) ^ (lane >> 4));
  const uint32_t fv0 = (lane >> 4) * 256u + 16u * ((lane & 15) ^ (4 * (lane >> 4)));
  auto fill_base = [&](int key0) { return p_last >= kPKeys - 1 ? min(key0, p_last - (kPKeys - 1)) : 0; };
  auto fill_one = [&](const u16* src_head, u16* dst, int key0, uint32_t f0, bool is_v) {
    const int kf = fill_base(key0);
    const char* src = reinterpret_cast<const char*>(src_head + static_cast<size_t>(kf) * kD) +
                      (16 * wave_u) * 256;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t off = (is_v ? f0 : f0 ^ (64u * j)) + 1024u * j;
      // kept a 32-bit value here (not a hoisted 64-bit one), so that the load
      // takes the scalar base + 32-bit vector offset form
      asm volatile("" : "+v"(off));
      __builtin_amdgcn_global_load_lds(src + off, lds_ptr(dst, (16 * wave_u + 4 * j) * 256), 16, 0, 0);
    }
  };
  // the one-tile case with fewer than 64 keys: rows past p_last repeat it
  auto fill_short = [&](const u16* src_head, u16* dst, uint32_t f0, bool is_v) {
    const char* src = reinterpret_cast<const char*>(src_head);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * wave_u + 4 * j + (lane >> 4);
      const uint32_t off = static_cast<uint32_t>(min(r, p_last)) * 256u + ((is_v ? f0 : f0 ^ (64u * j)) & 255u);
      __builtin_amdgcn_global_load_lds(src + off, lds_ptr(dst, (16 * wave_u + 4 * j) * 256), 16, 0, 0);
    }
  };
  auto fill_k = [&](u16* dst, int key0) { fill_one(kr, dst, key0, fk0, false); };
  auto fill_v = [&](u16* dst, int key0) { fill_one(vr, dst, key0, fv0, true); };

  // operand reads, as byte offsets in a tile.  K's A operand of key block kb,
  // k-step ks: row 32 kb + n, chunk 2 ks + hf, at kbase ^ 32 ks (+ 8192 kb),
  // kbase = 256 n + 16 (hf ^ (n & 15)).  V^T's A operand of dim block db,
  // key step s: lane i = l & 15 of 16-lane group (l >> 4) reads 8 bytes of
  // row 16 s + 4 hf + (i >> 2) (+ 8 for the second read), chunk 4 db +
  // 2 ((l >> 4) & 1) + ((i & 3) >> 1), half i & 1: at vbase ^ 64 db
  // (+ 4096 s, + 2048), vbase = 256 (4 hf + (i >> 2)) + 64 (i >> 2) +
  // 16 (2 ((l >> 4) & 1) + ((i & 3) >> 1)) + 8 (i & 1).  The XORs are redone
  // in every step (a few VALU) rather than held in registers.
  const uint32_t kbase0 = 256u * n + 16u * (hf ^ (n & 15));
  const uint32_t li = lane & 15;
  const uint32_t vbase0 = 256u * (4 * hf + (li >> 2)) + 64u * (li >> 2) +
                          16u * (2 * ((lane >> 4) & 1) + ((li & 3) >> 1)) + 8u * (li & 1);
  uint32_t kbase = kbase0, vbase = vbase0;
  auto k_operand = [&](const u16* kt, int kb, int ks) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(kt) + 8192 * kb +
                                                     (kbase ^ (32u * ks))));
  };
  auto vt_operand = [&](const u16* vt, int db, int st) {
    const char* p0 = reinterpret_cast<const char*>(vt) + 4096 * st + (vbase ^ (64u * db));
    const uint2 lo = lds_read_tr16_b64(reinterpret_cast<const u16*>(p0));
    const uint2 hi = lds_read_tr16_b64(reinterpret_cast<const u16*>(p0 + 2048));
    return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
  };
  auto logits = [&](const u16* kt, f32x16 (&sacc)[QC][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int cb = 0; cb < QC; ++cb) sacc[cb][kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = k_operand(kt, kb, ks);
#pragma unroll
        for (int cb = 0; cb < QC; ++cb) sacc[cb][kb] = mfma_32x32x16(a, qop[cb][ks], sacc[cb][kb]);
      }
    }
  };

  f32x16 o[QC][4];
  float m[QC];
  double l[QC];
#pragma unroll
  for (int cb = 0; cb < QC; ++cb) {
#pragma unroll
    for (int db = 0; db < 4; ++db) o[cb][db] = f32x16{};
    m[cb] = -INFINITY;
    l[cb] = 0.0;
  }

  // The online softmax of a tile in two parts: tile_max takes the tile's
  // maximum and moves the running max m to m_new (alpha = 2^(m - m_new) is
  // the rescale of O and l it implies); tile_exp then turns the logits into
  // probabilities at m_new, their bf16 P^T operands (4 key steps) and l.  The
  // max is taken over the raw dot products (the scale is positive, and the
  // rounded scaling is monotonic), and each exponent is a * c2_hi - m in one
  // fma: the product and the shift by the integer m are exact inside it, so
  // only the result rounds, and the scale's dropped low part (below 2^-24 of
  // a * c2) moves a probability by under 2e-7 of itself, and lse2 by less:
  // far inside the selection's tolerance (the importance pass and the float64
  // re-ranking share this lse2).  kMasked: the tile reaches past some
  // column's position, or starts early (the last tile of a work-group, whose
  // first key0 - kf rows belong to the previous tile); otherwise no branch,
  // so that the work can be interleaved with MFMAs.
  auto masked_logits = [&](const f32x16 (&sacc)[2], int key0, int pc, float (&sv)[2][16]) {
    // row off (key kf + off) is new and visible to the column iff
    // key0 - kf <= off <= P - kf; a hidden key gets a large finite negative
    // product, whose exponent underflows to 0
    const int kf = fill_base(key0);
    const int lo = key0 - kf;
    const int lim = min(kPKeys, pc - kf);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
        sv[kb][r] = off <= lim && off >= lo ? sacc[kb][r] : -1.0e30f;
      }
  };
  auto tile_max = [&](const f32x16 (&sacc)[QC][2], int key0, float (&alpha)[QC], auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
    for (int cb = 0; cb < QC; ++cb) {
      float sv[2][16];
      if (kMasked) {
        masked_logits(sacc[cb], key0, pcol[cb], sv);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[kb][r] = sacc[cb][kb][r];
      }
      float mx[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        mx[u] = fmaxf(fmaxf(sv[u >> 2][4 * (u & 3)], sv[u >> 2][4 * (u & 3) + 1]),
                      fmaxf(sv[u >> 2][4 * (u & 3) + 2], sv[u >> 2][4 * (u & 3) + 3]));
      float amax = fmaxf(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])),
                         fmaxf(fmaxf(mx[4], mx[5]), fmaxf(mx[6], mx[7])));
      // the column's other 32 keys sit in lane ^ 32: one VALU row swap
      amax = max_xor32(amax);
      // key 0 is visible to every token, so the running max is finite from
      // the first tile on
      const float tmax = fmaf(amax, c2_hi, amax * c2_lo);
      const float m_new = fmaxf(m[cb], ceilf(tmax));
      alpha[cb] = m[cb] == -INFINITY ? 0.f : ldexpf(1.f, static_cast<int>(m[cb] - m_new));
      m[cb] = m_new;
    }
  };
  auto tile_exp = [&](const f32x16 (&sacc)[QC][2], int key0, const float (&alpha)[QC],
                      bf16x8 (&pb)[QC][4], auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
    for (int cb = 0; cb < QC; ++cb) {
      float sv[2][16];
      if (kMasked) {
        masked_logits(sacc[cb], key0, pcol[cb], sv);
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[kb][r] = sacc[cb][kb][r];
      }
      float p[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[kb][r] = __builtin_amdgcn_exp2f(fmaf(sv[kb][r], c2_hi, -m[cb]));
      // the tile's sum as a tree (short dependency chains)
      float ps8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        ps8[u] = (p[u >> 2][4 * (u & 3)] + p[u >> 2][4 * (u & 3) + 1]) +
                 (p[u >> 2][4 * (u & 3) + 2] + p[u >> 2][4 * (u & 3) + 3]);
      const float ps = ((ps8[0] + ps8[1]) + (ps8[2] + ps8[3])) + ((ps8[4] + ps8[5]) + (ps8[6] + ps8[7]));
      l[cb] = l[cb] * static_cast<double>(alpha[cb]) + static_cast<double>(ps);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float* q8 = &p[st >> 1][8 * (st & 1)];
        const u32x4 pp{pack_bf16x2(q8[0], q8[1]), pack_bf16x2(q8[2], q8[3]), pack_bf16x2(q8[4], q8[5]),
                       pack_bf16x2(q8[6], q8[7])};
        pb[cb][st] = as_bf16x8(pp);
      }
    }
  };
  auto rescale = [&](const float (&alpha)[QC]) {
#pragma unroll
    for (int cb = 0; cb < QC; ++cb)
      if (__ballot(alpha[cb] != 1.f) != 0) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o[cb][db] *= alpha[cb];
      }
  };
  auto accumulate = [&](const u16* vt, const bf16x8 (&pb)[QC][4]) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 a = vt_operand(vt, db, st);
#pragma unroll
        for (int cb = 0; cb < QC; ++cb) o[cb][db] = mfma_32x32x16(a, pb[cb][st], o[cb][db]);
      }
  };
  auto wait_fills = [] {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's tile loads landed
  };

  // tiles 0 .. n_full - 1 are visible to every column and start at key0; the
  // last one or two tiles of a work-group take the masked path
  const int n_full = min((p_first + 1) / kPKeys, n_tiles - 1);
  using Full = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  // prologue: K_0, V_0 and K_1 in LDS, S_0 computed
  if (p_last >= kPKeys - 1) {
    fill_k(kb0, 0);
    fill_v(vb0, 0);
  } else {
    fill_short(kr, kb0, fk0, false);
    fill_short(vr, vb0, fv0, true);
  }
  if (n_tiles > 1) fill_k(kb1, kPKeys);
  // the query operands and the first fills must have landed before the loop
#pragma unroll
  for (int cb = 0; cb < QC; ++cb)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) require_loaded(qop[cb][ks]);
  wait_fills();
  __syncthreads();
  f32x16 sa[QC][2], sbk[QC][2];
  logits(kb0, sa);

  // Step i: fills of K_{i+2} and V_{i+1} (into the buffers that tile i - 1's
  // reads are done with: the barrier before them); the logits of tile i + 1
  // from K_{i+1} beside tile i's softmax; O rescaled; O += V_i^T P_i; then
  // wait for the fills.  Even steps hold K_{i+1} in kb1, V_i in vb0, S_i in
  // sa; odd steps the other buffers.
  bf16x8 pb[QC][4];
  float alpha[QC];
  auto step = [&](int i, auto odd_tag) {
    constexpr bool kOdd = decltype(odd_tag)::value;
    u16* k_next = kOdd ? kb0 : kb1;
    u16* k_fill = kOdd ? kb1 : kb0;
    u16* v_cur = kOdd ? vb1 : vb0;
    u16* v_fill = kOdd ? vb0 : vb1;
    f32x16 (&s_cur)[QC][2] = kOdd ? sbk : sa;
    f32x16 (&s_next)[QC][2] = kOdd ? sa : sbk;
    const int key0 = i * kPKeys;
    // the operand bases, re-derived here so that their XORs stay in the step
    kbase = kbase0;
    vbase = vbase0;
    asm volatile("" : "+v"(kbase), "+v"(vbase));
    __syncthreads();
    if (i + 2 < n_tiles) fill_k(k_fill, key0 + 2 * kPKeys);
    if (i + 1 < n_tiles) fill_v(v_fill, key0 + kPKeys);
    if (i < n_full) {
      // the next tile's operand reads and MFMAs and this tile's softmax in
      // one basic block, for the scheduler to interleave
      logits(k_next, s_next);
      tile_max(s_cur, key0, alpha, Full{});
      tile_exp(s_cur, key0, alpha, pb, Full{});
    } else {
      if (i + 1 < n_tiles) logits(k_next, s_next);
      tile_max(s_cur, key0, alpha, Masked{});
      tile_exp(s_cur, key0, alpha, pb, Masked{});
    }
    rescale(alpha);
    // the MFMA phase at raised wave priority: the arbiter then prefers this
    // wave's MFMAs over the other wave's softmax on the SIMD (measured 4%
    // faster on the 4K-token chunk over 128K keys)
    __builtin_amdgcn_s_setprio(1);
    accumulate(v_cur, pb);
    __builtin_amdgcn_s_setprio(0);
    wait_fills();
  };
  using Even = std::integral_constant<bool, false>;
  using Odd = std::integral_constant<bool, true>;
  for (int i = 0; i < n_tiles; i += 2) {
    step(i, Even{});
    if (i + 1 >= n_tiles) break;
    step(i + 1, Odd{});
  }
  // ---- epilogue: normalise, write out and the row statistics
#pragma unroll
  for (int cb = 0; cb < QC; ++cb) {
    double L = l[cb];
    L += __shfl_xor(L, 32);
    if (t_col[cb] >= T) continue;
    const int h = n & 7;
    const float inv = static_cast<float>(1.0 / L);
    u16* orow = out + ((static_cast<size_t>(b) * T + t_col[cb]) * Hq + static_cast<size_t>(g) * kG + h) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 pk{pack_bf16x2(o[cb][db][4 * j] * inv, o[cb][db][4 * j + 1] * inv),
                       pack_bf16x2(o[cb][db][4 * j + 2] * inv, o[cb][db][4 * j + 3] * inv)};
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * j + 4 * hf) = pk;
      }
    if (hf == 0) {
      const size_t row = (static_cast<size_t>(b) * T + t_col[cb]) * Hkv + g;
      const double l2 = static_cast<double>(m[cb]) + log2(L);
      lse2[row * kG + h] = l2;
      if (lse_out) lse_out[row * kG + h] = static_cast<float>(l2 * M_LN2);
      ytop_h[row * kG + h] = static_cast<float>(-log2(L));
    }
  }
}

// Importance pass.  grid: B * Hkv * ceil(T / 64) work-groups of 8 waves; a
// work-group takes 64 chunk tokens, each wave 8 of them as two row blocks of
// 32 (4 tokens x 8 heads each), so every K operand read from LDS serves 64
// query rows.  The MFMA is the 32x32x16 bf16 form computing S = Q . K^T
// (query rows, key columns): a lane holds, for one key, 4 heads of each of its
// block's 4 tokens, and the max over a token's 8 heads is 3 in-lane steps and
// one exchange with the lane 32 away.  Beside a 32x32 MFMA the VALU has room
// for about four instructions, four times what the 16x16x32 form leaves at the
// same matrix rate, which is where the other group's epilogue runs.
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
//               row's top log-weight (over its 8 heads) minus 64;
//   kmax[b][g][tb] = the largest |k| over this work-group's share of the KV
//               head's keys 0..S-1 (bf16 bits; when kmax is non-null): whole
//               key tile i belongs to token block i % n_tblk when that block
//               reads all of it, else to the last block, which reads every key.
constexpr int kIWaves = 8;
constexpr int kIThreads = 64 * kIWaves;
constexpr int kIMB = 2;                        // 32-row blocks (4 tokens) per wave
static_assert(kIWaves * 4 * kIMB == kImportanceTok, "64 chunk tokens per work-group");

constexpr int kIRing = 4;                      // K tiles in LDS (3 in flight)
constexpr int kIAhead = 6;                     // K operand reads in flight per wave

// vmcnt waits (the other counters untouched): all of this wave's vector
// memory operations; all but the last 4 (the prologue's tiles 1 and 2: tile 0
// has landed); all but the last 16 (tile it + 1 landed, in the steady tile
// loop).  The counts hold only for the issue order the tile loop lays out, so
// no memory access may cross a wait (the empty asm statements).
template <int kImm>
__device__ __forceinline__ void wait_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kImm);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vm_all() { wait_vm<0x0F70>(); }
__device__ __forceinline__ void wait_vm_ring_start() { wait_vm<0x0F74>(); }
__device__ __forceinline__ void wait_vm_ring_steady() { wait_vm<0x4F70>(); }

// A work-group barrier that waits for no memory operation: the importance
// values' global stores stay in flight across it.  Whatever must be visible
// past it is waited for explicitly (the tile's LDS writes); the empty asm
// statements keep the compiler from moving memory accesses across it, and the
// scheduling barriers keep every other instruction on its side too (left to
// itself the scheduler sinks a phase's later MFMAs past the barrier, into the
// phase meant for the other group's).
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kIThreads, 1) void prefill_importance_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const double* __restrict__ lse2,
    const float* __restrict__ ytop_h, u16* __restrict__ y, uint32_t* __restrict__ kmax,
    int64_t S, int64_t Spad, int T, int Hkv, int w, int n_tblk, float c2_hi, int64_t kvp) {
  (void)w;
  // the ring of K tiles: four separate arrays, each named at compile time
  // wherever it is filled or read, so that the compiler can tell a tile's
  // reads from the fills in flight into the others (and waits for none)
  __shared__ __align__(16) u16 kq0[kPKeys * kD];
  __shared__ __align__(16) u16 kq1[kPKeys * kD];
  __shared__ __align__(16) u16 kq2[kPKeys * kD];
  __shared__ __align__(16) u16 kq3[kPKeys * kD];
  __shared__ uint32_t s_kmax[kIWaves];
  constexpr int MB = kIMB;
  constexpr int kTok = kImportanceTok;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // waves w and w + 4 share a SIMD; the group is wave-uniform
  const bool group_b = wave_u >= kIWaves / 2;
  const int n = lane & 31, hf = lane >> 5;
  const int lin = xcd_linear(blockIdx.x, gridDim.x);
  const int tb = lin % n_tblk;
  const int bg = lin / n_tblk;
  const int g = bg % Hkv, b = bg / Hkv;
  const int Hq = Hkv * kG;
  const u16* kr = k + static_cast<size_t>(bg) * kvp * kD;
  const int64_t pos0 = S - T;
  const int tw = tb * kTok + 4 * MB * wave;   // this wave's first token
  // Q as the A operand: row n of block mb = (token tw + 4 mb + (n >> 3),
  // head n & 7), k-step ks = dims 16 ks + 8 hf .. + 7
  bf16x8 qop[MB][8];
  // y in fixed-point steps plus 0.5 is s c2 2^10 + (0.5 - 2^10 (lse2_h + ybase)):
  // one fma per head.  nl2r[mb][j][i] is that offset for token tw + 4 mb + j,
  // head 4 hf + i (the lane's rows of S)
  float nl2r[MB][4][4];
  // after the head max the low half of the wave holds tokens 4 mb + {0, 2},
  // the high half 4 mb + {1, 3}: the rows this lane stores
  u16* yrow[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int tq = min(tw + 4 * mb + (n >> 3), T - 1);   // past the chunk: repeat the last token
    const u16* qp = q + (static_cast<size_t>(b) * T + tq) * Hq * kD +
                    (static_cast<size_t>(g) * kG + (n & 7)) * kD + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[mb][ks] = as_bf16x8(load_u32x4(qp + 16 * ks));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(tw + 4 * mb + j, T - 1);
      const size_t row = (static_cast<size_t>(b) * T + t) * Hkv + g;
      float yt = -INFINITY;
      for (int h = 0; h < kG; ++h) yt = fmaxf(yt, ytop_h[row * kG + h]);
      const float ybase = yt - kYRange;
      // 2^10 ybase is exact, and so is its sum with 0.5 (|ybase| < 2^12)
      const float yoff = 0.5f - ybase * static_cast<float>(1 << kYFixBits);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        nl2r[mb][j][i] = fmaf(-static_cast<float>(lse2[row * kG + 4 * hf + i]),
                              static_cast<float>(1 << kYFixBits), yoff);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = min(tw + 4 * mb + 2 * u + hf, T - 1);
      const size_t row = (static_cast<size_t>(b) * T + t) * Hkv + g;
      yrow[mb][u] = y + row * Spad + 2 * n;   // at the lane's keys 2 n, 2 n + 1
    }
  }
  const int t_last = min(T - 1, tb * kTok + kTok - 1);
  const int64_t p_last = pos0 + t_last;
  const int n_tiles = static_cast<int>((p_last + kPKeys) / kPKeys);
  const float c2s = c2_hi * static_cast<float>(1 << kYFixBits);   // exact
  // this work-group's share of max |k|: whole tiles i with i % n_tblk == tb
  // (or, when that block does not read all of tile i, the last block's)
  auto owns_tile = [&](int i) {
    const int o = i % n_tblk;
    const int64_t o_last = pos0 + min(T - 1, o * kTok + kTok - 1);
    return (static_cast<int64_t>(i + 1) * kPKeys <= o_last + 1 ? o : n_tblk - 1) == tb;
  };
  u16x2 kabs{0, 0};

  // Tiles travel straight from memory to LDS, kIRing - 1 tiles ahead of use
  // (tile i in buffer i % kIRing).  A tile is unpadded 256-byte rows, the
  // 16-byte chunk c of row r at slot c ^ (r & 15): the operand reads of 16
  // consecutive rows (one chunk each) cover all banks once.  Wave w fills
  // rows 8 w .. 8 w + 7, 4 rows (1 KB) per load: lane l writes slot l & 15 of
  // row 8 w + 4 j + (l >> 4), so it reads that row's chunk (l & 15) ^ (row &
  // 15).  Rows past p_last repeat it (their importance values land in the
  // unread tail), so every load stays inside the KV head's keys.  The loads
  // are the buffer form (a resource based at the tile's first row, 32-bit
  // offsets within it), not the flat-global one: while a flat load is
  // outstanding the compiler cannot count LDS reads and waits for all of
  // them, which would undo the operand prefetch in the MFMA phase.
  auto ring = [&](auto slot_tag) -> u16* {
    constexpr int kS = decltype(slot_tag)::value % kIRing;
    return kS == 0 ? kq0 : kS == 1 ? kq1 : kS == 2 ? kq2 : kq3;
  };
  // tile is in buffer kSlot (tile % kIRing)
  auto fill = [&](int tile, auto slot_tag) {
    u16* dst = ring(slot_tag);
    const int64_t key0 = static_cast<int64_t>(tile) * kPKeys;
    const int64_t kf = min(key0, p_last);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(kr + kf * kD), 0, kPKeys * kD * 2, 0x00020000);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 8 * wave_u + 4 * j + (lane >> 4);
      const int row = static_cast<int>(min(key0 + r, p_last) - kf);   // 0 .. 63
      const uint32_t off = 256u * row + 16u * ((lane & 15) ^ (r & 15));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(dst, (8 * wave_u + 4 * j) * 256), 16, off, 0, 0, 0);
    }
    asm volatile("" ::: "memory");   // issued before whatever follows (the waits count on it)
  };
  // this work-group's share of max |k|, from the rows this wave filled (the
  // tile has landed and is visible): lane l takes chunks 2 (l & 7) and
  // 2 (l & 7) + 1 of row 8 w + (l >> 3)
  auto take_kmax = [&](int tile, const u16* kt) {
    if (kmax && owns_tile(tile)) {
      const int r = 8 * wave_u + (lane >> 3);
      const int c0 = 2 * (lane & 7);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(kt + r * kD + 8 * ((c0 + u) ^ (r & 15)));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kabs = __builtin_elementwise_max(kabs, __builtin_bit_cast(u16x2, v[e] & 0x7FFF7FFFu));
      }
    }
  };
  // K as the B operand: column n of key block kb is key 2 n + kb of the tile,
  // so that a lane's two blocks hold two neighbouring keys and its importance
  // values go out as one 32-bit store.  K-step ks reads chunk 2 ks + hf of
  // row 2 n + kb, at byte kbase[kb] ^ 32 ks (the 8 rows that one 128-byte
  // read phase touches, 2 n + kb for 8 consecutive n, still fall on 8
  // different slots)
  uint32_t kbase[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r = 2 * n + kb;
    kbase[kb] = 256u * r + 16u * (hf ^ (r & 15));
  }
  auto k_operand = [&](const u16* kt, int kb, int ks) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(kt) +
                                                     (kbase[kb] ^ (32u * ks))));
  };

  // prologue: the first kIRing - 1 tiles; tile 0 must have landed
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  using Slot2 = std::integral_constant<int, 2>;
  using Slot3 = std::integral_constant<int, 3>;
  fill(0, Slot0{});
  fill(1, Slot1{});
  fill(2, Slot2{});
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) require_loaded(qop[mb][ks]);
  wait_vm_ring_start();
  __syncthreads();
  // a tile's MFMAs: S for this wave's 2 row blocks x 2 key blocks
  auto mfma_phase = [&](const u16* kt, f32x16 (&sacc)[MB][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) sacc[mb][kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kop = k_operand(kt, kb, ks);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) sacc[mb][kb] = mfma_32x32x16(qop[mb][ks], kop, sacc[mb][kb]);
      }
    }
    // the order of issue: kIAhead operand reads first, then one more after
    // every MFMA pair, so that each read is issued kIAhead - 1 pairs (about
    // 64 clocks each) before its MFMAs, which covers LDS latency under the
    // other waves' reads
#pragma unroll
    for (int i = 0; i < kIAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 16 - kIAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kIAhead, 0);
  };
  // a tile's epilogue: importance values from S, and their stores.  In S's
  // accumulators register 4 j + i of lane (n, hf) is row 8 j + 4 hf + i of
  // the block: token j, head 4 hf + i, key column n (key 2 n + kb)
  auto epilogue = [&](const f32x16 (&sacc)[MB][2], int64_t key0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      uint32_t yv[2][2];   // [kb][token pair: 0 = tokens hf, 1 = tokens 2 + hf]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // y per (token, key), in fixed-point steps plus 0.5: max over the 8
        // heads = 4 here x the lane 32 away.  One fma per head: the scale's
        // low part (below 1e-7 of s c2) is dropped; the selection allows for
        // it and re-ranks every key near its threshold in float64.  The max
        // starts at 0, the clamp's lower end, so what crosses lanes is a
        // non-negative float (or -0), whose bits order as signed integers
        uint32_t m[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) v = fmaxf(v, fmaf(sacc[mb][kb][4 * j + i], c2s, nl2r[mb][j][i]));
          m[j] = __float_as_uint(v);
        }
        // the swap trades the high half of its first operand for the low half
        // of its second: the low half then holds both head halves of token j,
        // the high half both of token j + 1
        const auto p01 = __builtin_amdgcn_permlane32_swap(m[0], m[1], false, false);
        const auto p23 = __builtin_amdgcn_permlane32_swap(m[2], m[3], false, false);
        // the clamp's upper end, 65535 (as float bits), then truncate: rounds
        // to nearest
        constexpr int kTop = 0x477FFF00;
        const int y01 = min(max(static_cast<int>(p01[0]), static_cast<int>(p01[1])), kTop);
        const int y23 = min(max(static_cast<int>(p23[0]), static_cast<int>(p23[1])), kTop);
        yv[kb][0] = static_cast<uint32_t>(__int_as_float(y01));
        yv[kb][1] = static_cast<uint32_t>(__int_as_float(y23));
      }
      // Every lane stores (a fixed count of stores per phase, so the tile
      // loads can be waited for alone): keys at or past first_t land in the
      // row's unread tail (key < Spad), and a block past the chunk's end
      // repeats the last token, value for value
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<uint32_t*>(yrow[mb][u] + key0) = yv[0][u] | (yv[1][u] << 16);
    }
  };
  // The tile loops, one per group, one barrier per tile.  Between barriers
  // it and it + 1 group A runs the MFMAs of tile it and then its epilogue,
  // group B its epilogue of tile it - 1 and then the MFMAs of tile it, so
  // that on every SIMD one wave's epilogue runs beside the other's MFMAs.
  // Tile i's buffer is free once tile i - kIRing's reads (both groups' MFMAs,
  // before barrier i - kIRing + 1) are over: both groups fill it right after
  // barrier i - 3.  Tile it + 1 is read after barrier it + 1, so every wave
  // waits for its loads of that tile before that barrier.  Per tile a wave
  // issues its 2 loads and then its epilogue's 4 stores, and vector memory
  // operations count down in issue order, so once the pattern is steady tile
  // it + 1's loads are done when at most 16 operations are outstanding: the
  // stores and the later tiles' loads stay in flight.  Fills past the last
  // tile repeat key p_last into buffers that nobody reads again.  Both loops
  // are unrolled by the ring's length, so that every buffer is named
  // statically.
  if (!group_b) {
    auto step = [&](int it, auto slot_tag) {
      constexpr int kS = decltype(slot_tag)::value;
      f32x16 sacc[MB][2];
      fill(it + kIRing - 1, std::integral_constant<int, kS + kIRing - 1>{});
      take_kmax(it, ring(slot_tag));
      mfma_phase(ring(slot_tag), sacc);
      epilogue(sacc, static_cast<int64_t>(it) * kPKeys);
      if (it >= 2) wait_vm_ring_steady(); else wait_vm_all();
      phase_barrier();
    };
    for (int it = 0; it < n_tiles; it += kIRing) {
      step(it, Slot0{});
      if (it + 1 >= n_tiles) break;
      step(it + 1, Slot1{});
      if (it + 2 >= n_tiles) break;
      step(it + 2, Slot2{});
      if (it + 3 >= n_tiles) break;
      step(it + 3, Slot3{});
    }
  } else {
    // group B's share of tile 3 (group A's comes with its first step); waited
    // for at once (once per work-group), so that no fill is pending where
    // the loop starts
    fill(kIRing - 1, Slot3{});
    wait_vm_all();
    auto step = [&](int it, auto slot_tag) {
      f32x16 sacc[MB][2];
      take_kmax(it, ring(slot_tag));
      mfma_phase(ring(slot_tag), sacc);
      if (it >= 3) wait_vm_ring_steady(); else wait_vm_all();
      phase_barrier();
      fill(it + kIRing, slot_tag);   // into the buffer this tile leaves
      epilogue(sacc, static_cast<int64_t>(it) * kPKeys);
    };
    for (int it = 0; it < n_tiles; it += kIRing) {
      step(it, Slot0{});
      if (it + 1 >= n_tiles) break;
      step(it + 1, Slot1{});
      if (it + 2 >= n_tiles) break;
      step(it + 2, Slot2{});
      if (it + 3 >= n_tiles) break;
      step(it + 3, Slot3{});
    }
  }
  wait_vm_all();   // no fill may land after the work-group's LDS is released
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

// Importance of a decode row's keys for the dense selection (short contexts):
// the same 16-bit fixed-point y as the prefill chunk's importance pass, for
// every key j < S of row (b, g),
//   y[row][j] = max_h(s2_h[j] - lse2_h), stored as round((y - ybase) 2^10)
//               clamped to 0..65535, ybase = the row's top log-weight minus 64,
// with the same float32 arithmetic (the MFMA's float32 sum of exact bf16
// products, one fma per head with the scale's high part), so that the
// selection's error bound holds unchanged.  grid: (ceil(S / kDKeys), R); a
// work-group of 4 waves takes kDKeys keys, a wave 16-key subtiles in turn:
// S^T = K . Q^T on the bf16 MFMA with the 8 heads padded to 16 (lane (col,
// grp) holds head col of keys 4 grp .. 4 grp + 3), the maximum over the heads
// across lanes col 0..7.  kmax[row][wg] = the largest |k| (bf16 bits) of the
// keys the work-group read.
constexpr int kDKeys = kDecImpKeys;
constexpr int kDThreads = 256;
__global__ __launch_bounds__(kDThreads) void decode_importance_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const double* __restrict__ lse2,
    const float* __restrict__ ytop_h, u16* __restrict__ y, uint32_t* __restrict__ kmax,
    int64_t S, int64_t Spad, float c2_hi, int64_t kvp) {
  __shared__ uint32_t s_kmax;
  const int r = blockIdx.y;
  const int wg = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  if (tid == 0) s_kmax = 0u;
  const u16* kr = k + static_cast<size_t>(r) * kvp * kD;
  // the B operand: head col (zero for the padding heads), dims 32 c + 8 grp
  bf16x8 qb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qb[c] = col < kG ? as_bf16x8(load_u32x4(q + (static_cast<size_t>(r) * kG + col) * kD + 32 * c + 8 * grp))
                     : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  float yt = -INFINITY;
  for (int h = 0; h < kG; ++h) yt = fmaxf(yt, ytop_h[static_cast<size_t>(r) * kG + h]);
  const float ybase = yt - kYRange;
  // 2^10 ybase is exact, and so is its sum with 0.5 (|ybase| < 2^12)
  const float yoff = 0.5f - ybase * static_cast<float>(1 << kYFixBits);
  const float nl2r = col < kG ? fmaf(-static_cast<float>(lse2[static_cast<size_t>(r) * kG + col]),
                                     static_cast<float>(1 << kYFixBits), yoff)
                              : -INFINITY;
  const float c2s = c2_hi * static_cast<float>(1 << kYFixBits);   // exact
  u16* yrow = y + static_cast<size_t>(r) * Spad;
  const int64_t k0 = static_cast<int64_t>(wg) * kDKeys;
  const int64_t k1 = min(S, k0 + kDKeys);
  u16x2 kabs{0, 0};
  __syncthreads();
  for (int64_t key0 = k0 + 16 * wave; key0 < k1; key0 += 16 * (kDThreads / 64)) {
    // the A operand: key key0 + col (rows past S repeat the last), dims 32 c + 8 grp
    const int64_t key = min(key0 + col, S - 1);
    u32x4 ka[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ka[c] = load_u32x4(kr + key * kD + 32 * c + 8 * grp);
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) sacc = mfma_16x16x32(as_bf16x8(ka[c]), qb[c], sacc);
    if (key0 + col < k1) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kabs = __builtin_elementwise_max(kabs, __builtin_bit_cast(u16x2, ka[c][e] & 0x7FFF7FFFu));
    }
    // y in fixed-point steps plus 0.5 for head col, then the maximum over the
    // 8 heads: lanes col ^ 1, ^ 2, then the other quad of the 8
    float yv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = fmaf(sacc[i], c2s, nl2r);
      m = fmaxf(m, dpp_f32<0xB1>(m));
      m = fmaxf(m, dpp_f32<0x4E>(m));
      m = fmaxf(m, dpp_f32<0x141>(m));
      yv[i] = m;
    }
    // lane (0, grp) stores keys 4 grp .. 4 grp + 3 (8 bytes; keys at or past S
    // land in the row's unread tail below Spad)
    if (col == 0) {
      uint32_t v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        // clamp to 0..65535, then truncate: rounds to nearest
        v4[i] = static_cast<uint32_t>(__builtin_amdgcn_fmed3f(yv[i], 0.f, 65535.f));
      *reinterpret_cast<uint2*>(yrow + key0 + 4 * grp) =
          uint2{v4[0] | (v4[1] << 16), v4[2] | (v4[3] << 16)};
    }
  }
  uint32_t m = max(static_cast<uint32_t>(kabs[0]), static_cast<uint32_t>(kabs[1]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
  if (lane == 0) atomicMax(&s_kmax, m);
  __syncthreads();
  if (tid == 0) kmax[static_cast<size_t>(r) * gridDim.x + wg] = s_kmax;
}

}  // namespace

hipError_t launch_full_prefill(const Plan& p, const u16* q, const u16* k, const u16* v, u16* out,
                               float* lse, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;  // scale * log2(e)
  const float c2_hi = static_cast<float>(c2);
  const float c2_lo = static_cast<float>(c2 - static_cast<double>(c2_hi));
  constexpr int QC = kAttnQC;
  const int n_tblk = (p.T + 16 * QC - 1) / (16 * QC);
  const int n_wg = p.B * p.Hkv * n_tblk;
  hipLaunchKernelGGL(full_prefill_kernel<QC>, dim3(n_wg), dim3(kPThreads), 0, st, q, k, v, out,
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

hipError_t launch_decode_importance(const Plan& p, const u16* q, const u16* k, void* ws,
                                    hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  hipLaunchKernelGGL(decode_importance_kernel, dim3(p.n_ib, p.R), dim3(kDThreads), 0, st, q, k,
                     reinterpret_cast<const double*>(w + p.off_lse2),
                     reinterpret_cast<const float*>(w + p.off_ytop),
                     reinterpret_cast<u16*>(w + p.off_ybuf),
                     reinterpret_cast<uint32_t*>(w + p.off_kmax), p.S, p.Spad,
                     static_cast<float>(c2), p.kvp);
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
