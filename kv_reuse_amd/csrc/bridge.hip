// KV Bridging: the Cross-Decoder's full-attention K and V rows computed from
// the Self-Decoder's hidden states (news page "两天两连更：小米提前亮出V3底牌",
// section "两级KV共享：让模型少跑一半", item KV Bridging), written straight into
// the cache the full layer and its sparse layers read.  One token at the end
// of the cache is the decode-time append.
//
// The operation is a bf16 contraction over the hidden size dm:
//   C[f][m] = sum_k W[f][k] * H[m][k]      (fp32 accumulation, bf16 RNE output)
// with token m = b * n + t and feature f = (kv, g, d) of W [2][Hkv][D][dm];
// C[f][m] goes to cache_kv[b][g][pos0 + t][d].  Both operands are contiguous
// along the reduction, so every MFMA operand is one 16-byte load per lane.
//
// Two kernels:
//  * many tokens (a prefill chunk or a whole prompt): 128 tokens x 128
//    features (one KV head's K or V) per work-group, 4 waves of 64 x 64, the
//    reduction staged through LDS 64 deep with one barrier per stage; the
//    work-groups of one token tile sit on one XCD so its L2 serves the tile's
//    hidden rows to all 2 Hkv feature tiles;
//  * a few tokens (decode-time append, up to 64): the weights are the only
//    real traffic, so each work-group takes 16 features x 16 tokens and its 16
//    waves split the reduction, with operands loaded directly from global
//    memory (no reuse to stage) and a fixed-order sum of the 16 partials.

#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kBM = 128;      // tokens per work-group (large kernel)
constexpr int kBN = 128;      // features per work-group: one head's K or V
constexpr int kBK = 64;       // reduction depth of one LDS stage
constexpr int kBPitch = 72;   // u16 per LDS row: 36 dwords, so the 16-byte reads
                              // of 8 or 16 consecutive rows cover every bank once
constexpr int kSmallWaves = 16;

__device__ __forceinline__ int xcd_group(int id, int n) {
  // hardware dispatch sends work-group id to XCD id % 8; renumber so that XCD x
  // processes the contiguous range [x * n/8, (x+1) * n/8)
  if (n % 8 != 0) return id;
  return (id & 7) * (n >> 3) + (id >> 3);
}

// Store four features (consecutive d) of token m, already in fp32.
__device__ __forceinline__ void store4(const BridgeArgs& a, int f, int m, f32x4 c) {
  const int b = m / a.n_tok, t = m - b * a.n_tok;
  const int hd = f / kD;                 // (kv, g) of the feature
  const int kv = hd / a.Hkv, g = hd - kv * a.Hkv;
  const int d = f - hd * kD;
  u16* dst = (kv == 0 ? a.k : a.v) +
             ((static_cast<size_t>(b) * a.Hkv + g) * a.kvp + a.pos0 + t) * kD + d;
  const uint2 pk{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
  *reinterpret_cast<uint2*>(dst) = pk;
}

// grid: 2 Hkv * ceil(M / 128) work-groups of 256 threads.
__global__ __launch_bounds__(256, 2) void bridge_gemm_kernel(BridgeArgs a) {
  __shared__ __align__(16) u16 wl[2][kBN * kBPitch];
  __shared__ __align__(16) u16 hl[2][kBM * kBPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n_ft = 2 * a.Hkv;
  const int lin = xcd_group(blockIdx.x, gridDim.x);
  const int ft = lin % n_ft;
  const int m0 = (lin / n_ft) * kBM;
  const int f0 = ft * kBN;
  const int wm = wave & 1, wn = wave >> 1;  // the wave's 64 tokens and 64 features

  // staging: thread tid moves 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 j
  const int lr = tid >> 3, lc = tid & 7;
  const u16* wsrc[4];
  const u16* hsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wsrc[j] = a.w + static_cast<size_t>(f0 + lr + 32 * j) * a.dm + 8 * lc;
    const int m = min(m0 + lr + 32 * j, a.M - 1);   // rows past the end repeat the last
    hsrc[j] = a.hidden + static_cast<size_t>(m) * a.dm + 8 * lc;
  }
  u32x4 wr[4], hr[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wr[j] = load_u32x4(wsrc[j] + kt * kBK);
      hr[j] = load_u32x4(hsrc[j] + kt * kBK);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4*>(&wl[buf][(lr + 32 * j) * kBPitch + 8 * lc]) = wr[j];
      *reinterpret_cast<u32x4*>(&hl[buf][(lr + 32 * j) * kBPitch + 8 * lc]) = hr[j];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.dm / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 wa[4], hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wa[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &wl[buf][(64 * wn + 16 * i + col) * kBPitch + 32 * ks + 8 * grp]));
        hb[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &hl[buf][(64 * wm + 16 * i + col) * kBPitch + 32 * ks + 8 * grp]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(wa[i], hb[j], acc[i][j]);
    }
    // the other buffer was last read before the previous barrier
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }
  // C[feature 4 grp + e][token col] of block (i, j)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 64 * wm + 16 * j + col;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) store4(a, f0 + 64 * wn + 16 * i + 4 * grp, m, acc[i][j]);
  }
}

// grid: (2 Hkv D / 16, ceil(M / 16)) work-groups of 16 waves.
__global__ __launch_bounds__(kSmallWaves * 64) void bridge_small_kernel(BridgeArgs a) {
  __shared__ f32x4 red[kSmallWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int f = 16 * blockIdx.x + col;                    // A row: a feature
  const int m = min(16 * static_cast<int>(blockIdx.y) + col, a.M - 1);   // B column: a token
  const u16* wp = a.w + static_cast<size_t>(f) * a.dm + 8 * grp;
  const u16* hp = a.hidden + static_cast<size_t>(m) * a.dm + 8 * grp;
  const int nks = a.dm / 32;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  // wave w takes reduction steps w, w + 16, ...; eight loads of each operand in
  // flight per round (one round at d_model = 4096)
  constexpr int kU = 8;
  for (int s0 = wave; s0 < nks; s0 += kU * kSmallWaves) {
    u32x4 wv[kU], hv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = s0 + u * kSmallWaves;
      if (s < nks) {
        wv[u] = load_u32x4(wp + 32 * s);
        hv[u] = load_u32x4(hp + 32 * s);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (s0 + u * kSmallWaves < nks) acc = mfma_16x16x32(as_bf16x8(wv[u]), as_bf16x8(hv[u]), acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 c = red[0][lane];
  for (int w = 1; w < kSmallWaves; ++w) c += red[w][lane];
  const int mo = 16 * blockIdx.y + col;
  if (mo < a.M) store4(a, 16 * blockIdx.x + 4 * grp, mo, c);
}

}  // namespace

hipError_t launch_kv_bridge(const BridgeArgs& a, hipStream_t st) {
  if (a.M <= 64) {
    dim3 grid(2 * a.Hkv * kD / 16, (a.M + 15) / 16);
    hipLaunchKernelGGL(bridge_small_kernel, grid, dim3(kSmallWaves * 64), 0, st, a);
  } else {
    const int n_wg = 2 * a.Hkv * ((a.M + kBM - 1) / kBM);
    hipLaunchKernelGGL(bridge_gemm_kernel, dim3(n_wg), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace hs2
