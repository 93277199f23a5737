// Internal declarations shared by the HIP sources of libhs2.so (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/hs2.h"

namespace hs2 {

constexpr int kD = 128;          // head dim (v1)
constexpr int kG = 8;            // query heads per KV head (v1)
constexpr int kNB = 2048;        // selection histogram bins (top 11 bits of a 32-bit key)
constexpr int kBinShift = 21;    // 32 - 11
constexpr int kPNB = 512;        // prefill-chunk histogram bins (1/8 octave; top 9 bits)
constexpr int kUncCap = 2048;    // near-threshold keys handled in LDS; more take the slow path
constexpr int kMaxSel = 4096;    // top_k + window limit (index list kept in LDS)
constexpr int kSparseChunk = 128;  // selected keys per sparse work-group (a decode slice)
constexpr float kYRange = 64.0f;   // log2 range below the row's top score that the bins span
constexpr int kYFixBits = 10;      // prefill importance: fixed point, 2^-10 log2 units per step
constexpr int kImportanceTok = 64;  // prefill importance pass: chunk tokens per work-group
constexpr int kDecImpKeys = 256;    // decode importance pass (dense selection): keys per work-group
// the plan's dense decode selection: when all of K (the rows' K caches, 256
// bytes per key row) is at most this much
constexpr int64_t kDenseDecodeBytes = int64_t{64} << 20;
constexpr int kMaxSplits = 1024;   // context splits per row (full layer, decode)
constexpr int kDefaultCUs = 256;   // compute units assumed when no device can be queried
// Refinement of the log-normaliser: a key is dominant for head h when its
// probability under h is at least 2^kDomLog2; such (key, head) terms are
// summed again from exact float64 logits.  A head has at most 2^8 keys of
// weight 2^-8 or more, so a prefill row has at most 8 * 2^8 dominant keys: the
// list capacity covers them with room for float32 rounding at the cut.
constexpr float kDomLog2 = -8.0f;
// Decode refines further down, to 2^kDomFloorLog2, as far as a per-row budget
// of subtiles allows (the heaviest first).
constexpr float kDomFloorLog2 = -14.0f;
constexpr int kDomCap = 2304;      // dominant keys listed per prefill row
// Decode: for each subtile of 16 keys, each of its four 4-key quads and each
// head, how far the quad's largest base-2 logit lies below the subtile's, in
// steps of 1/kQuadSteps octave rounded down (255: that far or farther), one
// byte each, 32 bytes per subtile ([quad][head]).
constexpr int kQuadSteps = 16;
// A prefill chunk's selection bands its stored importance allowing for a
// refinement of lse2 of up to this many octaves (the change is checked).
constexpr double kDl2Allow = 0x1p-12;

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef double f64x4 __attribute__((ext_vector_type(4)));

// Per-row selection bookkeeping (lives in the workspace; zeroed each call).
struct RowInfo {
  uint32_t cert_count;  // entries appended to the row's first list
  uint32_t unc_count;   // entries appended to the row's band list
  uint32_t up_count;    // entries above the band appended to the selection
  uint32_t pad;
};
// Per-(row, chunk) result of the decode refinement: each head's relative
// change of its softmax denominator, the dominant subtiles seen and the
// subtiles whose recomputed float32 maximum differed from the stored one.
struct RefinePart {
  double corr[8];
  uint32_t n_dom, n_bad, pad0, pad1;
};
// Per-row statistics of the refinement (HS2_WS_REFINE): dominant units (decode:
// subtiles, prefill: keys), float32 replica mismatches (decode), dominant keys
// beyond the list capacity (prefill), reserved.
struct RefineStat {
  uint32_t n_dom, n_bad, n_over, pad;
};
constexpr int kScoreRound = 256;   // subtiles scored per round of a work-group
constexpr int kMaxChunks = 4096;   // candidate chunks per row
constexpr int64_t kPrefillBandCap = 8192;  // near-threshold keys listed per prefill row

// Where each piece of the workspace sits, for one shape.
struct Plan {
  int64_t S, Spad;
  int64_t kvp;               // K/V row pitch in tokens (the cache's capacity per head)
  int bs;                    // block-level selection: block size (0 = token-level)
  int B, T, Hq, Hkv, R;      // R = B*T*Hkv rows
  int k, w, cap;             // cap = k + w (index list capacity per row)
  int n_layers;
  int n_cu;                  // compute units of the current device (work-group targets)
  double scale;
  // full attention (decode split kernel) and the merge of its splits
  int n_split, kps;
  size_t off_part_m, off_part_l, off_part_o, off_stmax, off_qdiff, off_lse2, off_ytop;
  bool quads;                // decode: the quads' distances are written and used
  bool dense_dec;            // decode: selection from every key's importance
  int n_ib;                  // importance work-groups per row (decode) / token blocks (prefill)
  // selection state shared by both selection paths
  size_t off_hist, off_info;
  // selection from given scores
  int sel_chunk, sel_nchunk;
  size_t off_ukey, off_cert, off_unc, off_unck;
  // fused selection from the subtile maxima
  int hs_chunk, hs_nchunk;   // subtiles per work-group: bound histogram
  int cc_chunk, cc_nchunk;   // subtiles per work-group: the candidate-subtile lists
  size_t off_clist, off_ccnt, off_lo;
  int sc_chunk, sc_nchunk;   // scoring: list entries per work-group region, work-groups per row
  size_t off_hist_c, off_cand_y, off_cand_idx, off_cand_cnt, off_band_idx, off_band_key;
  // refinement of lse2 over the dominant keys: decode per-(row, chunk) partial
  // sums (RefinePart); prefill per-row dominant-key lists; per-row statistics
  int ref_nwg;                // decode: refinement work-groups per row
  size_t off_ref_part, off_ref_stat, off_dom_list;
  size_t off_dsub, off_dsub_cnt;   // decode: dominant subtiles per (row, candidate chunk)
  size_t off_cut;            // decode: each row's refinement cut (float, log2 probability)
  size_t off_lse2r;          // the refined lse2 (float64 [R][8]) the selection ranks with
  // prefill chunk: per-row log2 importance of the older keys (16-bit fixed point), band capacity per row
  size_t off_ybuf;
  size_t off_kmax;           // prefill: largest |k| (bf16 bits) per (batch, KV head)
  int64_t band_cap;
  // sparse
  int sp_nch;
  size_t off_sp_m, off_sp_l, off_sp_o;
  size_t off_idx_bad;        // the gather's index check: uint32 [R][sp_nch]
  size_t off_swa;            // the window branch's outputs [L][R][G][D] float32
  size_t total;
};

// KV Bridging: hidden [M][dm] (M = B * n_tok tokens) times W [2 Hkv D][dm]
// into rows pos0 .. pos0 + n_tok - 1 of the caches k, v [B][Hkv][kvp][D].
struct BridgeArgs {
  const u16* hidden;
  const u16* w;
  u16* k;
  u16* v;
  int64_t kvp, pos0;
  int M, n_tok, dm, Hkv;
};

// Keep e as the calling thread's last HIP error (hs2_last_hip_error) and
// return HS2_ERR_HIP (or HS2_OK for hipSuccess).
int record_hip_error(hipError_t e);

// ---------------------------------------------------------------- launchers
// Each returns the hipError_t of its launches (hipGetLastError()).

// Full attention, decode (T == 1): split-context flash-decode writing per-split
// partial (m, l, O), per-subtile (16 keys) maxima of every head's logits and
// each quad's distance below them.
hipError_t launch_full_decode_split(const Plan& p, const u16* q, const u16* k, const u16* v,
                                    void* ws, hipStream_t st);
// Merge the splits: out (bf16), lse (nullable), lse2 (fp64, base 2) and each
// head's bound on log2 importance; also clears the rows' selection state.
hipError_t launch_full_combine(const Plan& p, u16* out, float* lse, void* ws, hipStream_t st);
// KV Bridging into the cache (no workspace).
hipError_t launch_kv_bridge(const BridgeArgs& a, hipStream_t st);
// Per-key importance [R][S] (float32), recomputed from q, k and lse2.
hipError_t launch_full_scores(const Plan& p, const u16* q, const u16* k, float* scores,
                              void* ws, hipStream_t st);
// Refinement of lse2 over the dominant keys (decode), after the subtile-bound
// histogram: partial sums per chunk, then the per-row update of lse2 and lse
// (nullable).
hipError_t launch_lse_refine(const Plan& p, const u16* q, const u16* k, void* ws, hipStream_t st);
// The refined lse2 (and lse, nullable) from the refinement's partial sums; the
// fused selection does the same inside its scoring kernel instead.
hipError_t launch_lse_finalize(const Plan& p, float* lse, void* ws, hipStream_t st);
// The first two kernels of the fused decode selection: the subtile-bound
// histogram, then the candidate subtiles (and the refinement's dominant ones).
hipError_t launch_subtile_hist(const Plan& p, void* ws, hipStream_t st);
hipError_t launch_subtile_cand(const Plan& p, void* ws, hipStream_t st);
// Selection from given float32 scores, compared exactly.
hipError_t launch_scores_select(const Plan& p, const float* scores, int32_t* idx,
                                int32_t* n_sel, void* ws, hipStream_t st);
// Selection of the fused step: candidate subtiles from the maxima, float32
// rescoring on MFMA, float64 re-ranking near the threshold.
hipError_t launch_fused_select(const Plan& p, const u16* q, const u16* k, int32_t* idx,
                               int32_t* n_sel, float* lse, void* ws, hipStream_t st);

// Full attention over a prefill chunk (T > 1): causal flash attention writing
// out, lse (nullable), lse2 and each head's bound on log2 importance.
hipError_t launch_full_prefill(const Plan& p, const u16* q, const u16* k, const u16* v, u16* out,
                               float* lse, void* ws, hipStream_t st);
// Prefill chunk importance for the selection: per-row fixed-point y, each KV
// head's largest |k| and each row's dominant keys, in the workspace.
hipError_t launch_prefill_importance(const Plan& p, const u16* q, const u16* k, void* ws,
                                     hipStream_t st);
// Dense importance [R][S] of a prefill chunk for the caller, from float64
// logits and an exactly recomputed normaliser (no workspace).
hipError_t launch_prefill_scores(const Plan& p, const u16* q, const u16* k, float* scores,
                                 hipStream_t st);
// Decode importance for the dense selection: every key's fixed-point y and
// each work-group's largest |k|, in the workspace (as the prefill pass writes).
hipError_t launch_decode_importance(const Plan& p, const u16* q, const u16* k, void* ws,
                                    hipStream_t st);
// Selection of a prefill chunk's rows, or of decode rows in the dense mode:
// one work-group per row.  It first refines lse2 over the row's dominant keys
// (and writes lse, when non-null, from it).
hipError_t launch_prefill_select(const Plan& p, const u16* q, const u16* k, int32_t* idx,
                                 int32_t* n_sel, float* lse, void* ws, hipStream_t st);

// Sparse layers (all n_layers fused: one gather of the selected K/V rows).
// With window_branch, the previous generation's layer: the selected older
// tokens plus a separate branch over each layer's local window cache (k_loc,
// v_loc; NULL when the cache has no rows).
hipError_t launch_sparse(const Plan& p, const u16* q, const u16* k, const u16* v,
                         const int32_t* idx, const int32_t* n_sel, u16* out, void* ws,
                         hipStream_t st, bool window_branch = false, const u16* k_loc = nullptr,
                         const u16* v_loc = nullptr);

// ---------------------------------------------------------------- device helpers
#ifdef __HIPCC__
__device__ __forceinline__ float bf16_bits_to_f32(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// float -> bfloat16, round to nearest even (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16 f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming load: the data is read once, so it is marked non-temporal.
__device__ __forceinline__ u32x4 load_u32x4_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Fixed-point position of a log2 importance y within [ybase, ybase + kYRange)
// as a 32-bit key (monotone in y, saturating at both ends); its top 11 bits
// are the selection histogram bin (1/32 octave).  Every producer and consumer
// of a histogram uses this one function.
__device__ __forceinline__ uint32_t key_from_log2(float y, float ybase) {
  const float z = (y - ybase) * 67108864.0f;  // 2^32 / kYRange
  if (!(z > 0.f)) return 0u;
  if (z >= 4294967040.0f) return 0xFFFFFFFFu;
  return static_cast<uint32_t>(z);
}
// Order-preserving maps from floats to unsigned integers (larger value -> larger key).
__device__ __forceinline__ uint32_t ordered_u32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t ordered_u64(double d) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(d));
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element (i & 3) of the 8-byte chunk addressed by lane
// 4*e + (i >> 2), for e = 0..3.  So if lane i of a group addresses row
// base_row + (i >> 2), column c0 + 4*(i & 3) of a row-major bf16 tile, lane i
// gets column c0 + i of rows base_row .. base_row + 3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16_b64(const u16* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(uint2, r);
}
// V^T operand (A of O^T = V^T P^T) for d-block nb from a row-major V tile in
// LDS with row pitch `pitch`: lane (grp, col) gets V[key(grp, e)][16*nb + col]
// for e = 0..7 with key(grp, e) = 16*(e >> 2) + 4*grp + (e & 3).
__device__ __forceinline__ bf16x8 lds_vt_operand(const u16* tile, int pitch, int nb, int col,
                                                 int grp) {
  const u16* p0 = tile + (4 * grp + (col >> 2)) * pitch + 16 * nb + 4 * (col & 3);
  const uint2 a = lds_read_tr16_b64(p0);
  const uint2 b = lds_read_tr16_b64(p0 + 16 * pitch);
  return as_bf16x8(u32x4{a.x, a.y, b.x, b.y});
}
// Cross-row steps on the gfx950 row swaps (VALU, no LDS round trip).  With
// both operands v, v_permlane16_swap leaves rows (0, 0, 2, 2) of v in the
// first result and rows (1, 1, 3, 3) in the second, and v_permlane32_swap
// leaves rows (0, 1, 0, 1) and (2, 3, 2, 3): combining the two results pairs
// lane l with l ^ 16, or with l ^ 32.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// v + v[l ^ 16], then + v[l ^ 32]: each step adds the same two values in
// every lane of a pair (addition is commutative), as a lane-xor butterfly does.
__device__ __forceinline__ float sum_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// DPP moves within rows of 16 lanes (every source lane valid for the
// controls used: quad_perm, row_ror, row mirrors).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long u = __double_as_longlong(v);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), kCtrl, 0xF, 0xF, true));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), kCtrl, 0xF, 0xF, true));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
// v + v[l ^ 32] then + v[l ^ 16] for a double (the butterfly's first two steps).
__device__ __forceinline__ double sum_rows_f64(double v) {
  auto join = [](uint32_t hi, uint32_t lo) {
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
  };
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const auto l32 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(u), static_cast<uint32_t>(u), false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(u >> 32), static_cast<uint32_t>(u >> 32), false, false);
  v = join(h32[0], l32[0]) + join(h32[1], l32[1]);
  const uint64_t w = static_cast<uint64_t>(__double_as_longlong(v));
  const auto l16 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(w), static_cast<uint32_t>(w), false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(w >> 32), static_cast<uint32_t>(w >> 32), false, false);
  return join(h16[0], l16[0]) + join(h16[1], l16[1]);
}
// The refinement's cut for a decode row, by one wave (the value in every lane):
// the lowest whole bin of the row's histogram of subtile bounds (kNB bins of
// kYRange / kNB octave from ybase) down to which at most `budget` subtiles
// lie, clamped to [kDomFloorLog2, kDomLog2], as a log2 probability.  The
// selection's candidate kernel (which lists the dominant subtiles) and the
// refinement (which tests their pairs) both call it on the same histogram.
__device__ __forceinline__ float refine_cut_wave(const uint32_t* hist_row, float ybase,
                                                 uint32_t budget) {
  const int lane = threadIdx.x & 63;
  constexpr float kBinW = kYRange / kNB;
  constexpr int kPer = kNB / 64;
  const int floor_bin = max(0, min(kNB, static_cast<int>(ceilf((kDomFloorLog2 - ybase) / kBinW))));
  const int cap_bin = max(0, min(kNB, static_cast<int>(ceilf((kDomLog2 - ybase) / kBinW))));
  // lane l holds bins kNB-1-kPer*l .. kNB-kPer-kPer*l (the top bins in lane 0)
  uint32_t lsum = 0;
  for (int i = 0; i < kPer; ++i) lsum += hist_row[kNB - 1 - kPer * lane - i];
  uint32_t incl = lsum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const uint64_t over = __ballot(incl > budget);
  int b_cut = 0;   // the lowest bin whose count from the top stays within the budget
  if (over) {
    // the owner lane's bins, top down, one per lane, and their running count
    const int owner = __builtin_ctzll(over);
    const uint32_t above = __shfl(incl - lsum, owner);
    const int top = kNB - 1 - kPer * owner;
    const uint32_t cb = lane < kPer ? hist_row[top - lane] : 0u;
    uint32_t run = cb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(run, off);
      if (lane >= off) run += o;
    }
    const uint64_t hit = __ballot(lane < kPer && above + run > budget);
    b_cut = top - __builtin_ctzll(hit) + 1;   // the owner's bins reach past the budget
  }
  const int bin = max(min(b_cut, cap_bin), floor_bin);
  return ybase + static_cast<float>(bin) * kBinW;
}
// Sum of head h's refinement partials of one row (n_parts of them), by one
// wave, in every lane: lane l adds partials l, l + 64, ... in order, then the
// fixed pairing of a lane-xor butterfly.
__device__ __forceinline__ double refine_head_sum(const RefinePart* __restrict__ pr, int n_parts,
                                                  int h) {
  const int lane = threadIdx.x & 63;
  double c = 0.0;
  for (int i = lane; i < n_parts; i += 64) c += pr[i].corr[h];
  c += dpp_f64<0xB1>(c);     // lane ^ 1
  c += dpp_f64<0x4E>(c);     // lane ^ 2
  c += dpp_f64<0x141>(c);    // the other quad of the 8
  c += dpp_f64<0x128>(c);    // lane ^ 8 within the row of 16
  return sum_rows_f64(c);    // ^ 32, then ^ 16
}
// The refinement's budget of subtiles per decode row: a twentieth of them, at least 64.
__host__ __device__ __forceinline__ uint32_t refine_budget(int64_t S) {
  const int64_t n = (S + 15) / 16 / 20;
  return static_cast<uint32_t>(n > 64 ? n : 64);
}

// Wait until this wave's outstanding LDS operations are done, and keep the
// compiler from moving memory accesses across this point.
__device__ __forceinline__ void lds_fence_wave() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
#endif

}  // namespace hs2
