// Sparse-attention layers that reuse the full layer's KV cache and index list
// (news page "两天两连更：小米提前亮出V3底牌", section "两级KV共享：让模型少跑一半",
// item KV Reuse; the window and the chosen older tokens share one cache and one
// softmax, section "Token级选择：精准定位大海里的那根针").
//
// Design (gfx950):
//  * One work-group serves one row (batch, query token, KV head) and a slice of
//    its index list.  The slice's indices go to LDS; the work-group gathers the
//    selected K and V rows (256 contiguous bytes each) into LDS once, in
//    sub-chunks of 32, 64 or 128 keys, and every layer of the launch reads them there:
//    the N layers cost one gather, not N.
//  * Wave c handles column tile c = two layers x 8 query heads (16 MFMA
//    columns): S^T = K_sel . Q^T and O^T = V_sel^T . P^T on MFMA 16x16x32 bf16,
//    online softmax in base 2 across the sub-chunks.
//  * Decode has few rows, so the index list is cut into slices of 128 keys
//    spread over work-groups, and a combine kernel merges the slices; a
//    prefill chunk has enough rows to give each row one work-group.

#include <algorithm>

#include "hs2_internal.h"

namespace hs2 {
namespace {

// Keys gathered into LDS at a time (SUB).  With one work-group per row (a
// prefill chunk) 32 keeps a work-group's LDS at 17 KB, so many work-groups per
// CU hide each other's gather latency (measured on the 4096-token chunk: 128
// keys 1.71 ms, 64 keys 1.26 ms, 32 keys 1.12 ms); a decode slice is one
// 128-key sub-chunk (at 1M context 9.1 us against 11.5 us for 4 x 32).
constexpr int kSubRows = 32;
constexpr int kSubSlice = kSparseChunk;
// slices beyond two 70 KB work-groups per CU (256 CUs) gather 64 keys at a time
// instead, so all of them are resident at once (32K context x 64 rows: 19.5
// against 15.3 us; with fewer slices the single 128-key sub-chunk is faster)
constexpr int kSubSliceHalf = kSparseChunk / 2;
constexpr int64_t kSliceWgOneRound = 512;
constexpr int kPitch = 136;   // u16 per LDS row (272 bytes)

template <int NCT, int kSub>
__global__ __launch_bounds__(NCT * 64) void sparse_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_sel, u16* __restrict__ out,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ part_o,
    int64_t S, int T, int Hkv, int L, int layer0, int cap, int nch, int keys_per_wg,
    float c2_hi, float c2_lo, size_t layer_stride, int64_t kvp, int w_drop,
    const float* __restrict__ swa_add, uint32_t* __restrict__ bad) {
  __shared__ __align__(16) u16 klds[kSub * kPitch];
  __shared__ __align__(16) u16 vlds[kSub * kPitch];
  __shared__ int32_t sidx[2 * kSub];   // (two buffers when the gather is pipelined)
  __shared__ uint32_t s_bad;

  const int r = blockIdx.y;
  const int ch = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int b = r / (T * Hkv);
  const int g = r % Hkv;
  const size_t kvrow = static_cast<size_t>(b) * Hkv + g;
  const u16* kr = k + kvrow * static_cast<size_t>(kvp) * kD;
  const u16* vr = v + kvrow * static_cast<size_t>(kvp) * kD;
  // a count beyond the list's capacity (a malformed list) reads no further than it
  int ns = min(max(n_sel[r], 0), cap);
  if (w_drop >= 0) {
    // the separate-window variant: the window's entries (the last ones of the
    // ascending list) are left to the window branch
    const int64_t P = S - T + (r / Hkv) % T;
    const int64_t nwin = P - max(static_cast<int64_t>(0), P - w_drop + 1) + 1;
    ns = static_cast<int>(max(static_cast<int64_t>(0), ns - nwin));
  }
  const int pos_begin = ch * keys_per_wg;
  const int pos_end = min(ns, pos_begin + keys_per_wg);
  // the index check: entries this work-group reads that lie outside [0, P]
  // (they are still clamped into the cache, never read out of bounds) are
  // counted, and the count is written to bad[r][ch] whatever it is
  const int64_t P_row = S - T + (r / Hkv) % T;
  if (tid == 0) s_bad = 0u;

  const int layer = layer0 + 2 * wave + (col >> 3);  // this lane's column
  const int head = col & 7;
  const bool col_ok = layer < L;
  bf16x8 qb[4];
  {
    const u16* qr = q + static_cast<size_t>(col_ok ? layer : 0) * layer_stride +
                    (static_cast<size_t>(r) * kG + head) * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qb[c] = col_ok ? as_bf16x8(load_u32x4(qr + 32 * c + 8 * grp))
                     : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  f32x4 o[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // a sub-chunk's attention from LDS (its n_here keys), all layers of the wave
  auto compute = [&](int n_here) {
      for (int kb = 0; kb < n_here; kb += 32) {
        f32x4 sacc[2];
  #pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
          const u16* krow = klds + (kb + 16 * mt + col) * kPitch + 8 * grp;
  #pragma unroll
          for (int c = 0; c < 4; ++c)
            sacc[mt] = mfma_16x16x32(as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 32 * c)),
                                     qb[c], sacc[mt]);
        }
        float sv[8];
  #pragma unroll
        for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = kb + 16 * mt + 4 * grp + i;
            const float a = sacc[mt][i];
            sv[mt * 4 + i] = kk < n_here ? fmaf(a, c2_hi, a * c2_lo) : -INFINITY;
          }
        float tm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        tm = max_xor32(max_xor16(tm));
        const float m_new = fmaxf(m_run, tm);
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        float p[8];
  #pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(sv[e] - m_new);
        l_run = l_run * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
        m_run = m_new;
        const bf16x8 pb = as_bf16x8(u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
  #pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          o[nb] *= alpha;
          o[nb] = mfma_16x16x32(lds_vt_operand(vlds + kb * kPitch, kPitch, nb, col, grp), pb, o[nb]);
        }
      }
  };
  // the sub-chunk's pieces: 16 bytes of one key's K and V rows per thread and
  // piece, (key, c16) = piece >> 4, piece & 15
  constexpr int kPieces = (kSub * 16 + NCT * 64 - 1) / (NCT * 64);
  constexpr int kBatch = kPieces < 8 ? kPieces : 8;
  // entries outside [0, S) (padding, or a malformed list) read row 0 / S-1
  // instead of faulting; padding is masked out of the softmax
  auto load_pieces = [&](const int32_t* sx, int u0, u32x4 (&kv_k)[kBatch], u32x4 (&kv_v)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      // (pieces past the sub-chunk, when the thread count does not divide
      // it, read piece 0 and are not stored)
      const int pc0 = tid + (u0 + u) * NCT * 64;
      const int pc = pc0 < kSub * 16 ? pc0 : 0;
      const int key = pc >> 4, c16 = pc & 15;
      const int j = sx[key];
      const size_t jj = j < 0 ? 0 : static_cast<size_t>(min(static_cast<int64_t>(j), S - 1));
      kv_k[u] = load_u32x4(kr + jj * kD + 8 * c16);
      kv_v[u] = load_u32x4(vr + jj * kD + 8 * c16);
    }
  };
  auto store_pieces = [&](int u0, const u32x4 (&kv_k)[kBatch], const u32x4 (&kv_v)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int pc = tid + (u0 + u) * NCT * 64;
      if (pc >= kSub * 16) continue;
      const int key = pc >> 4, c16 = pc & 15;
      *reinterpret_cast<u32x4*>(klds + key * kPitch + 8 * c16) = kv_k[u];
      *reinterpret_cast<u32x4*>(vlds + key * kPitch + 8 * c16) = kv_v[u];
    }
  };
  // entry i of the sub-chunk at list position sc: its index (-1 past the
  // slice), counted when outside [0, P]
  auto take_index = [&](int sc, int i, int32_t raw) -> int32_t {
    const bool in = sc + i < pos_end;
    if (in && (raw < 0 || raw > P_row)) atomicAdd(&s_bad, 1u);
    return in ? raw : -1;
  };
  // (loads of list entries are clamped into the list, used or not)
  auto index_at = [&](int pos) { return idx[static_cast<size_t>(r) * cap + min(pos, cap - 1)]; };
  if constexpr (kPieces <= kBatch && kPieces <= 4) {
    // One batch of loads holds a sub-chunk: the next sub-chunk's rows are
    // gathered into registers while this one is computed from LDS, and the
    // indices two sub-chunks ahead are loaded meanwhile.  The prefetches are
    // unconditional (past the slice they read list entry cap - 1 or key row
    // 0), so the compiler waits for each only where it is used.
    int32_t jn = -1;
    if (tid < kSub) sidx[tid] = take_index(pos_begin, tid, index_at(pos_begin + tid));
    __syncthreads();
    u32x4 kv_k[kBatch], kv_v[kBatch];
    load_pieces(sidx, 0, kv_k, kv_v);
    if (tid < kSub) jn = index_at(pos_begin + kSub + tid);
    int buf = 0;
    for (int sc = pos_begin; sc < pos_end; sc += kSub) {
      __syncthreads();  // the previous sub-chunk is consumed, and its index buffer free
      store_pieces(0, kv_k, kv_v);
      if (tid < kSub) sidx[kSub * (buf ^ 1) + tid] = take_index(sc + kSub, tid, jn);
      __syncthreads();
      load_pieces(sidx + kSub * (buf ^ 1), 0, kv_k, kv_v);
      if (tid < kSub) jn = index_at(sc + 2 * kSub + tid);
      compute(min(kSub, pos_end - sc));
      buf ^= 1;
    }
  } else {
    for (int sc = pos_begin; sc < pos_end; sc += kSub) {
      const int n_here = min(kSub, pos_end - sc);
      __syncthreads();  // the previous sub-chunk is consumed
      for (int i = tid; i < kSub; i += blockDim.x) sidx[i] = take_index(sc, i, index_at(sc + i));
      __syncthreads();
      // all loads of a batch first, then its LDS stores, so a 256-thread
      // work-group gathers the sub-chunk in one memory round trip
#pragma unroll
      for (int u0 = 0; u0 < kPieces; u0 += kBatch) {
        u32x4 kv_k[kBatch], kv_v[kBatch];
        load_pieces(sidx, u0, kv_k, kv_v);
        store_pieces(u0, kv_k, kv_v);
      }
      __syncthreads();
      compute(n_here);
    }
  }
  l_run = sum_rows(l_run);
  __syncthreads();   // (every count is in)
  if (tid == 0) bad[static_cast<size_t>(r) * nch + ch] = s_bad;
  if (!col_ok) return;
  if (nch == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    u16* orow = out + static_cast<size_t>(layer) * layer_stride + (static_cast<size_t>(r) * kG + head) * kD;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * nb + 4 * grp + i;
        // the window branch's output, [L][R][G][D] (grid.y = R)
        const float add =
            swa_add ? swa_add[((static_cast<size_t>(layer) * gridDim.y + r) * kG + head) * kD + d]
                    : 0.f;
        orow[d] = f32_to_bf16_rne(o[nb][i] * inv + add);
      }
  } else {
    const size_t pb = ((static_cast<size_t>(r) * nch + ch) * L + layer) * kG + head;
    if (grp == 0) {
      part_m[pb] = m_run;
      part_l[pb] = l_run;
    }
    float* po = part_o + pb * kD;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[16 * nb + 4 * grp + i] = o[nb][i];
  }
}

// The separate sliding-window branch of the previous generation's sparse layer
// (news page, section "Token级选择：精准定位大海里的那根针": the branch and its
// local cache are what HySparse2 drops).  grid (R, L), one wave: layer n's own
// local K/V rows of the window [P - w + 1, P] (the local cache holds positions
// S - Lc .. S - 1), softmax over them, normalised output per head in float32
// to swa_out [L][R][G][D], which the sparse kernel then adds to the selected
// branch's output.  An empty window gives zeros.
__global__ __launch_bounds__(64) void swa_branch_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k_loc, const u16* __restrict__ v_loc,
    float* __restrict__ swa_out, int64_t S, int B, int T, int Hkv, int w, int64_t Lc,
    float c2_hi, float c2_lo, size_t layer_stride) {
  __shared__ __align__(16) u16 klds[32 * kPitch];
  __shared__ __align__(16) u16 vlds[32 * kPitch];
  const int r = blockIdx.x, n = blockIdx.y;
  const int R = gridDim.x;
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int b = r / (T * Hkv), t = (r / Hkv) % T, g = r % Hkv;
  const int64_t P = S - T + t;
  const int64_t first = max(static_cast<int64_t>(0), P - w + 1);
  const int nk = static_cast<int>(P - first + 1);
  const size_t cache = ((static_cast<size_t>(n) * B + b) * Hkv + g) * static_cast<size_t>(Lc);
  const int64_t row0 = first - (S - Lc);
  // no window rows (the caches may then be NULL): the branch adds zeros
  const bool any = nk > 0 && k_loc != nullptr && v_loc != nullptr;
  const u16* kl = any ? k_loc + (cache + row0) * kD : nullptr;
  const u16* vl = any ? v_loc + (cache + row0) * kD : nullptr;
  bf16x8 qb[4];
  {
    const u16* qr = q + static_cast<size_t>(n) * layer_stride +
                    (static_cast<size_t>(r) * kG + (col & 7)) * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qb[c] = col < kG ? as_bf16x8(load_u32x4(qr + 32 * c + 8 * grp))
                       : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  f32x4 o[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  for (int kb = 0; any && kb < nk; kb += 32) {
    const int n_here = min(32, nk - kb);
    // 32 rows of K and V, 16 pieces of 16 bytes each: 8 pieces per lane (rows
    // past the window repeat its last row and are masked below)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pc = lane + 64 * u;
      const int key = pc >> 4, c16 = pc & 15;
      const size_t row = static_cast<size_t>(kb + min(key, n_here - 1));
      *reinterpret_cast<u32x4*>(klds + key * kPitch + 8 * c16) = load_u32x4(kl + row * kD + 8 * c16);
      *reinterpret_cast<u32x4*>(vlds + key * kPitch + 8 * c16) = load_u32x4(vl + row * kD + 8 * c16);
    }
    __syncthreads();
    f32x4 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const u16* krow = klds + (16 * mt + col) * kPitch + 8 * grp;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sacc[mt] = mfma_16x16x32(as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 32 * c)),
                                 qb[c], sacc[mt]);
    }
    float sv[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 16 * mt + 4 * grp + i;
        const float a = sacc[mt][i];
        sv[mt * 4 + i] = kk < n_here ? fmaf(a, c2_hi, a * c2_lo) : -INFINITY;
      }
    float tm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    tm = max_xor32(max_xor16(tm));
    const float m_new = fmaxf(m_run, tm);
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(sv[e] - m_new);
    l_run = l_run * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
    m_run = m_new;
    const bf16x8 pb = as_bf16x8(u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                      pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      o[nb] *= alpha;
      o[nb] = mfma_16x16x32(lds_vt_operand(vlds, kPitch, nb, col, grp), pb, o[nb]);
    }
    __syncthreads();   // the tile is consumed before the next one is staged
  }
  l_run = sum_rows(l_run);
  if (col >= kG) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* dst = swa_out + ((static_cast<size_t>(n) * R + r) * kG + col) * kD;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[16 * nb + 4 * grp + i] = o[nb][i] * inv;
}

// grid (R, L): merge the slices of one row and layer.  The slices' maxima and
// sums go through LDS first, so the O loads below are independent of each other.
__global__ __launch_bounds__(256) void sparse_combine_kernel(
    const float* __restrict__ part_m, const float* __restrict__ part_l,
    const float* __restrict__ part_o, u16* __restrict__ out, int L, int nch,
    size_t layer_stride, const float* __restrict__ swa_add) {
  extern __shared__ float fac[];   // [nch][kG]
  __shared__ float inv_l[kG];
  const int r = blockIdx.x;
  const int layer = blockIdx.y;
  const int tid = threadIdx.x;
  for (int i = tid; i < nch * kG; i += blockDim.x) {
    const int c = i / kG, h = i % kG;
    fac[i] = part_m[((static_cast<size_t>(r) * nch + c) * L + layer) * kG + h];
  }
  __syncthreads();
  if (tid < kG) {
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, fac[c * kG + tid]);
    float l = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float mc = fac[c * kG + tid];
      const float f = (mc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mc - M);
      l += f * part_l[((static_cast<size_t>(r) * nch + c) * L + layer) * kG + tid];
      fac[c * kG + tid] = f;
    }
    inv_l[tid] = l > 0.f ? 1.f / l : 0.f;
  }
  __syncthreads();
  // one output per thread: blockIdx.z picks a quarter of the 8 x 128 outputs
  const int i = blockIdx.z * 256 + tid;
  const int h = i >> 7;
  const float* po = part_o + ((static_cast<size_t>(r) * nch) * L + layer) * kG * kD + i;
  const size_t cstride = static_cast<size_t>(L) * kG * kD;
  float a0 = 0.f, a1 = 0.f;
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    a0 += fac[c * kG + h] * po[c * cstride];
    a1 += fac[(c + 1) * kG + h] * po[(c + 1) * cstride];
  }
  if (c < nch) a0 += fac[c * kG + h] * po[c * cstride];
  out[static_cast<size_t>(layer) * layer_stride + static_cast<size_t>(r) * kG * kD + i] =
      f32_to_bf16_rne((a0 + a1) * inv_l[h] +
                      (swa_add ? swa_add[(static_cast<size_t>(layer) * gridDim.x + r) * kG * kD + i]
                               : 0.f));
}

}  // namespace

hipError_t launch_sparse(const Plan& p, const u16* q, const u16* k, const u16* v,
                         const int32_t* idx, const int32_t* n_sel, u16* out, void* ws,
                         hipStream_t st, bool window_branch, const u16* k_loc,
                         const u16* v_loc) {
  const bool swa = window_branch;
  char* w = static_cast<char*>(ws);
  const double c2 = p.scale * 1.4426950408889634;
  const float c2_hi = static_cast<float>(c2);
  const float c2_lo = static_cast<float>(c2 - static_cast<double>(c2_hi));
  const size_t layer_stride = static_cast<size_t>(p.B) * p.T * p.Hq * kD;
  // sliced (few rows): kSparseChunk keys per work-group, as the plan's slice count assumes
  const int keys_per_wg = p.sp_nch == 1 ? ((p.cap + kSubRows - 1) / kSubRows) * kSubRows : kSparseChunk;
  float* pm = reinterpret_cast<float*>(w + p.off_sp_m);
  float* pl = reinterpret_cast<float*>(w + p.off_sp_l);
  float* po = reinterpret_cast<float*>(w + p.off_sp_o);
  float* swa_out = swa ? reinterpret_cast<float*>(w + p.off_swa) : nullptr;
  if (swa) {
    const int64_t Lc = std::min<int64_t>(p.S, static_cast<int64_t>(p.T) + p.w - 1);
    hipLaunchKernelGGL(swa_branch_kernel, dim3(p.R, p.n_layers), dim3(64), 0, st, q, k_loc,
                       v_loc, swa_out, p.S, p.B, p.T, p.Hkv, p.w, Lc, c2_hi, c2_lo,
                       layer_stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int layer0 = 0; layer0 < p.n_layers; layer0 += 8) {
    const int nl = min(8, p.n_layers - layer0);
    const int nct = (nl + 1) / 2;
    dim3 grid(p.sp_nch, p.R);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(nct * 64), 0, st, q, k, v, idx, n_sel, out, pm, pl, po,
                         p.S, p.T, p.Hkv, p.n_layers, layer0, p.cap, p.sp_nch, keys_per_wg, c2_hi,
                         c2_lo, layer_stride, p.kvp, swa ? p.w : -1, swa_out,
                         reinterpret_cast<uint32_t*>(w + p.off_idx_bad));
    };
    if (p.sp_nch == 1) {
      switch (nct) {
        case 1: go(sparse_kernel<1, kSubRows>); break;
        case 2: go(sparse_kernel<2, kSubRows>); break;
        case 3: go(sparse_kernel<3, kSubRows>); break;
        default: go(sparse_kernel<4, kSubRows>); break;
      }
    } else if (static_cast<int64_t>(p.R) * p.sp_nch > kSliceWgOneRound) {
      switch (nct) {
        case 1: go(sparse_kernel<1, kSubSliceHalf>); break;
        case 2: go(sparse_kernel<2, kSubSliceHalf>); break;
        case 3: go(sparse_kernel<3, kSubSliceHalf>); break;
        default: go(sparse_kernel<4, kSubSliceHalf>); break;
      }
    } else {
      switch (nct) {
        case 1: go(sparse_kernel<1, kSubSlice>); break;
        case 2: go(sparse_kernel<2, kSubSlice>); break;
        case 3: go(sparse_kernel<3, kSubSlice>); break;
        default: go(sparse_kernel<4, kSubSlice>); break;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.sp_nch > 1) {
    hipLaunchKernelGGL(sparse_combine_kernel, dim3(p.R, p.n_layers, 4), dim3(256),
                       static_cast<size_t>(p.sp_nch) * kG * sizeof(float), st, pm, pl, po,
                       out, p.n_layers, p.sp_nch, layer_stride, swa_out);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace hs2
