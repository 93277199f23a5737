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
//    work-group sweeps its split front to back.  Split partials (m, l, O) are
//    merged by full_combine_kernel.
//  * S^T = K . Q^T on MFMA 16x16x32 bf16: K rows are the A operand (16 keys per
//    MFMA, loaded straight from HBM with 16-byte loads), the group's queries
//    padded to 16 heads are the B operand.  Half of the MFMA columns are
//    padding; the kernel is bound by HBM bytes, not by MFMA issue.
//  * O^T = V^T . P^T on MFMA: P^T comes out of the S^T accumulators already in
//    the B-operand lane layout (head = lane % 16), so only V needs a transpose;
//    it goes through a per-wave LDS tile (272-byte row pitch) and comes back
//    transposed with two ds_read_b64_tr_b16 per MFMA operand.
//  * Online softmax in base 2 with the running max rounded up to an integer:
//    every rescale factor is an exact power of two, and the normaliser l is
//    accumulated in float64, so the only error left in log-sum-exp comes from
//    the float32 logits themselves.
//  * Every key's float32 base-2 logit (scale*log2(e)*<q_h,k_j>) of every head is
//    written once (32 bytes per key row next to its 512 bytes of K/V); the
//    selection turns them into importances once lse is known.
//  * The next tile's K/V loads are issued before the current tile is processed
//    (two register buffers), so each wave keeps 16 KB of HBM reads in flight.

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;       // keys per wave iteration
constexpr int kVPitch = 136;    // u16 per V row in LDS: 272 bytes

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
    for (int c = 0; c < 4; ++c) t.ka[mt][c] = as_bf16x8(load_u32x4(base + 32 * c));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t key = t0 + grp + 4 * i;
    key = key < key_last ? key : key_last;
    t.vv[i] = load_u32x4(vr + key * kD + 8 * col);
  }
}

__device__ __forceinline__ float max8(const float* x) {
  float a = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  float b = fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]));
  return fmaxf(a, b);
}

__device__ __forceinline__ void process_tile(const KVTile& t, SoftmaxState& st,
                                             const bf16x8 (&qb)[4], u16* __restrict__ vw,
                                             float* __restrict__ lg, int64_t t0,
                                             int64_t key_end, int col, int grp, float c2_hi,
                                             float c2_lo) {
  // ---- S^T = K Q^T for 32 keys
  f32x4 sacc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) sacc[mt] = mfma_16x16x32(t.ka[mt][c], qb[c], sacc[mt]);
  }
  // base-2 logits; the scale is applied as a two-term product so that its
  // float32 rounding does not bias every logit of the row the same way
  float sv[8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = t0 + 16 * mt + 4 * grp + i;
      const float a = sacc[mt][i];
      const float x = fmaf(a, c2_hi, a * c2_lo);
      sv[mt * 4 + i] = key < key_end ? x : -INFINITY;
    }
  if (col < kG) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int64_t key0 = t0 + 16 * mt + 4 * grp;
      if (key0 + 3 < key_end) {
        *reinterpret_cast<f32x4*>(lg + key0) =
            f32x4{sv[mt * 4], sv[mt * 4 + 1], sv[mt * 4 + 2], sv[mt * 4 + 3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + i < key_end) lg[key0 + i] = sv[mt * 4 + i];
      }
    }
  }
  // ---- online softmax (per head = per lane % 16)
  float tm = max8(sv);
  tm = fmaxf(tm, __shfl_xor(tm, 16));
  tm = fmaxf(tm, __shfl_xor(tm, 32));
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
  // ---- V tile to LDS (natural layout), then V^T operands by column reads
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

__global__ __launch_bounds__(kWaves * 64, 2) void full_decode_split_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    float* __restrict__ logits, float* __restrict__ part_m, double* __restrict__ part_l,
    float* __restrict__ part_o, int64_t S, int64_t Spad, int kps, int n_split, float c2_hi,
    float c2_lo) {
  // V tiles during the stream; reused for the cross-wave merge afterwards
  __shared__ __align__(16) unsigned char smem[kWaves * kTile * kVPitch * 2];
  __shared__ float sm_m[kWaves][kG];
  __shared__ double sm_l[kWaves][kG];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int r = blockIdx.y;
  const int s = blockIdx.x;
  const int64_t key_begin = static_cast<int64_t>(s) * kps;
  const int64_t key_end = min(S, key_begin + kps);
  const u16* qr = q + static_cast<size_t>(r) * kG * kD;
  const u16* kr = k + static_cast<size_t>(r) * S * kD;
  const u16* vr = v + static_cast<size_t>(r) * S * kD;
  float* lg = logits + (static_cast<size_t>(r) * kG + (col < kG ? col : 0)) * Spad;
  u16* vw = reinterpret_cast<u16*>(smem) + wave * kTile * kVPitch;

  bf16x8 qb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qb[c] = col < kG ? as_bf16x8(load_u32x4(qr + col * kD + 32 * c + 8 * grp))
                     : as_bf16x8(u32x4{0u, 0u, 0u, 0u});

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
      process_tile(ta, st, qb, vw, lg, t0, key_end, col, grp, c2_hi, c2_lo);
      if (!more) break;
      t0 = t1;
      t1 = t0 + stride;
      more = t1 < key_end;
      if (more) load_tile(ta, kr, vr, t1, key_last, col, grp);
      process_tile(tb, st, qb, vw, lg, t0, key_end, col, grp, c2_hi, c2_lo);
      if (!more) break;
      t0 = t1;
    }
  }
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);

  __syncthreads();  // all waves done with their V tiles
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

// One work-group per row: merge the split partials.
__global__ __launch_bounds__(256) void full_combine_kernel(
    const float* __restrict__ part_m, const double* __restrict__ part_l,
    const float* __restrict__ part_o, int n_split, u16* __restrict__ out,
    float* __restrict__ lse_out, double* __restrict__ lse2, float* __restrict__ ytop,
    uint32_t* __restrict__ hist, RowInfo* __restrict__ info) {
  extern __shared__ float fac[];  // [n_split][kG]
  __shared__ float sM[kG];
  __shared__ double sL[kG];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t rb = static_cast<size_t>(r) * n_split;
  {
    const int h = tid >> 5, j = tid & 31;  // 8 heads x 32 lanes
    float M = -INFINITY;
    for (int s = j; s < n_split; s += 32) M = fmaxf(M, part_m[(rb + s) * kG + h]);
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 32));
    double L = 0.0;
    for (int s = j; s < n_split; s += 32) {
      const float ms = part_m[(rb + s) * kG + h];
      if (ms != -INFINITY) L += part_l[(rb + s) * kG + h] * ldexp(1.0, static_cast<int>(ms - M));
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) L += __shfl_xor(L, off, 32);
    if (j == 0) {
      sM[h] = M;
      sL[h] = L;
    }
  }
  __syncthreads();
  for (int i = tid; i < n_split * kG; i += blockDim.x) {
    const int s = i / kG, h = i % kG;
    const float ms = part_m[(rb + s) * kG + h];
    fac[i] = (ms == -INFINITY) ? 0.f
                               : ldexpf(1.f, static_cast<int>(ms - sM[h])) /
                                     static_cast<float>(sL[h]);
  }
  __syncthreads();
  for (int i = tid; i < kG * kD; i += blockDim.x) {
    const int h = i >> 7;
    float acc = 0.f;
    for (int s = 0; s < n_split; ++s) acc += part_o[(rb + s) * kG * kD + i] * fac[s * kG + h];
    out[static_cast<size_t>(r) * kG * kD + i] = f32_to_bf16_rne(acc);
  }
  if (tid < kG) {
    const double l2 = static_cast<double>(sM[tid]) + log2(sL[tid]);
    lse2[static_cast<size_t>(r) * kG + tid] = l2;
    if (lse_out) lse_out[static_cast<size_t>(r) * kG + tid] = static_cast<float>(l2 * M_LN2);
  }
  if (tid == 0) {
    float yt = -INFINITY;
    for (int h = 0; h < kG; ++h)
      yt = fmaxf(yt, static_cast<float>(static_cast<double>(sM[h]) -
                                        (static_cast<double>(sM[h]) + log2(sL[h]))));
    ytop[r] = yt;
  }
  // fresh selection state for this row
  for (int i = tid; i < kNB; i += blockDim.x) hist[static_cast<size_t>(r) * kNB + i] = 0u;
  if (tid == 0) info[r] = RowInfo{0, 0, 0, 0, 0u, 0u, 0u, 0};
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
                     reinterpret_cast<float*>(w + p.off_logits),
                     reinterpret_cast<float*>(w + p.off_part_m),
                     reinterpret_cast<double*>(w + p.off_part_l),
                     reinterpret_cast<float*>(w + p.off_part_o), p.S, p.Spad, p.kps, p.n_split,
                     c2_hi, c2_lo);
  return hipGetLastError();
}

hipError_t launch_full_combine(const Plan& p, u16* out, float* lse, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const size_t shm = static_cast<size_t>(p.n_split) * kG * sizeof(float);
  hipLaunchKernelGGL(full_combine_kernel, dim3(p.R), dim3(256), shm, st,
                     reinterpret_cast<const float*>(w + p.off_part_m),
                     reinterpret_cast<const double*>(w + p.off_part_l),
                     reinterpret_cast<const float*>(w + p.off_part_o), p.n_split, out, lse,
                     reinterpret_cast<double*>(w + p.off_lse2),
                     reinterpret_cast<float*>(w + p.off_ytop),
                     reinterpret_cast<uint32_t*>(w + p.off_hist),
                     reinterpret_cast<RowInfo*>(w + p.off_info));
  return hipGetLastError();
}

}  // namespace hs2
